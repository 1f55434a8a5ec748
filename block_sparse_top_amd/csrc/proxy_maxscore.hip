// Stage 1 of MSA: proxy block max scores.
//
// The proxy pass of the MiniMax-AI/MSA README (section "Usage": dense pass,
// output_o off, output_maxscore on) and the max-pooling of proxy scores over
// 128-token KV blocks of the Flash-MSA article (paragraph comparing MSA with
// DSA): for each query row and proxy head, the largest scaled proxy logit in
// every causally visible 128-key block.
//
// Design (gfx950):
//  * one workgroup = 256 threads = 4 waves, one proxy head, one row tile of
//    up to 256 rows whose positions share a 256-aligned window; wave w owns
//    rows 64w .. 64w+63 as two 32-row MFMA column tiles;
//  * S^T = K Q^T on MFMA (bf16 32x32x16 or fp8 32x32x64): keys are the MFMA
//    rows, queries the columns, so each lane holds one query row and the
//    max over keys is an in-register reduction plus one lane swap;
//  * the tile's proxy Q stays in registers for the whole key loop; each K
//    block (one page of one head, 32 KB bf16 / 16 KB fp8) is loaded with
//    coalesced 16-byte loads into a double-buffered LDS tile; every A
//    fragment read from LDS feeds two MFMAs (the wave's two row tiles);
//  * only blocks up to the tile's last local block are visited; the two
//    boundary blocks apply the per-row causal mask; scales are applied after
//    the max (they are positive);
//  * workgroup order: workgroups of one proxy head are consecutive modulo
//    the head count, so with 8 proxy heads each XCD streams one head's K
//    through its own L2; long (late) tiles launch first.
#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

struct ProxyArgs {
  const uint8_t* pq;         // [T, P, 128] bf16 or fp8
  const uint8_t* pk;         // [N, Pk, 128, 128]
  const float* qs;           // [P]  (fp8)
  const float* ks;           // [Pk] (fp8)
  const int32_t* kv_indices;
  const int32_t* tiles;
  const int32_t* page_start;
  int32_t tile_lo, ntiles;
  int32_t P, Pk, nb_max;
  int64_t row_begin, row_end, row_count;
  float* out;                // [P, nb_max, row_count]
  float scale;
};

template <bool FP8>
struct ProxyTraits;

template <>
struct ProxyTraits<false> {
  static constexpr int kElem = 2;             // bytes per element
  static constexpr int kRowBytes = 256;       // one key row
  static constexpr int kLdsRow = 272;         // padded LDS row (bank spread)
  static constexpr int kSteps = 8;            // MFMA k-steps over d = 128
  typedef bf16x8 Frag;
};
template <>
struct ProxyTraits<true> {
  static constexpr int kElem = 1;
  static constexpr int kRowBytes = 128;
  static constexpr int kLdsRow = 144;
  static constexpr int kSteps = 2;
  typedef i32x8 Frag;
};

template <bool FP8>
__device__ __forceinline__ typename ProxyTraits<FP8>::Frag load_frag_global(const uint8_t* p) {
  if constexpr (FP8) {
    i32x4 a = *reinterpret_cast<const i32x4*>(p);
    i32x4 b = *reinterpret_cast<const i32x4*>(p + 16);
    i32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
  } else {
    return *reinterpret_cast<const bf16x8*>(p);
  }
}

template <bool FP8>
__device__ __forceinline__ typename ProxyTraits<FP8>::Frag load_frag_lds(const uint8_t* p) {
  if constexpr (FP8) {
    i32x4 a = lds_load16<i32x4>(p);
    i32x4 b = lds_load16<i32x4>(p + 16);
    i32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
  } else {
    return lds_load16<bf16x8>(p);
  }
}

template <bool FP8>
__device__ __forceinline__ f32x16 mma(const typename ProxyTraits<FP8>::Frag& a,
                                      const typename ProxyTraits<FP8>::Frag& b, const f32x16& c) {
  if constexpr (FP8) return mfma32x32x64_fp8(a, b, c);
  else return mfma32x32x16(a, b, c);
}

template <bool FP8>
__global__ __launch_bounds__(256) void proxy_maxscore_kernel(ProxyArgs a) {
  using Tr = ProxyTraits<FP8>;
  using Frag = typename Tr::Frag;
  constexpr int kBlockBytes = 128 * Tr::kRowBytes;        // one K block in global memory
  constexpr int kChunks = kBlockBytes / 16 / 256;         // 16-byte chunks per thread
  constexpr int kChunksPerRow = Tr::kRowBytes / 16;
  constexpr int kStepBytes = Tr::kRowBytes / Tr::kSteps;  // bytes of d per MFMA k-step
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][128 * Tr::kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = blockIdx.x % a.P;
  const int t = a.tile_lo + (a.ntiles - 1 - (int)(blockIdx.x / a.P));
  const int seq = a.tiles[4 * t + 0];
  const int row0 = a.tiles[4 * t + 1];
  const int nrows = a.tiles[4 * t + 2];
  const int pos0 = a.tiles[4 * t + 3];
  const int ph = (a.Pk == a.P) ? p : 0;
  const int32_t* pages = a.kv_indices + a.page_start[seq];
  const int b_last = (pos0 + nrows - 1) >> 7;
  const int b_full = (pos0 + 1) >> 7;  // blocks < b_full are visible to every row of the tile

  // Q fragments (B operand): lane -> query column lane%32 of row tile `sub`,
  // k-run (lane/32) of each k-step.
  Frag qf[2][Tr::kSteps];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int r = 64 * wave + 32 * sub + (lane & 31);
    const bool valid = r < nrows;
    const uint8_t* src = a.pq + ((int64_t)(row0 + (valid ? r : 0)) * a.P + p) * (128 * Tr::kElem);
#pragma unroll
    for (int s = 0; s < Tr::kSteps; ++s) {
      qf[sub][s] = load_frag_global<FP8>(src + s * kStepBytes + (lane >> 5) * (kStepBytes / 2));
      if (!valid) qf[sub][s] = Frag{};
    }
  }

  // Cooperative K block load: thread -> chunks tid + 256*i (coalesced).
  i32x4 stage[kChunks];
  auto gload = [&](int b) {
    const uint8_t* src = a.pk + ((int64_t)pages[b] * a.Pk + ph) * kBlockBytes;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) stage[i] = *reinterpret_cast<const i32x4*>(src + (int64_t)(tid + 256 * i) * 16);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      lds_store16<i32x4>(&lds[buf][(c / kChunksPerRow) * Tr::kLdsRow + (c % kChunksPerRow) * 16], stage[i]);
    }
  };

  float scale = a.scale;
  if constexpr (FP8) scale *= a.qs[p] * a.ks[ph];
  const bool wave_active = 64 * wave < nrows;
  const int my_row = 64 * wave + lane;          // row this lane writes
  const int64_t my_grow = row0 + my_row;
  const bool writes = my_row < nrows && my_grow >= a.row_begin && my_grow < a.row_end;
  float* outp = a.out + (int64_t)p * a.nb_max * a.row_count + (my_grow - a.row_begin);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int b = 0; b <= b_last; ++b) {
    const int buf = b & 1;
    if (b < b_last) gload(b + 1);
    if (wave_active) {
      float m[2] = {kNegInf, kNegInf};
      const bool masked = b >= b_full;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        const uint8_t* arow = &lds[buf][(32 * kt + (lane & 31)) * Tr::kLdsRow + (lane >> 5) * (kStepBytes / 2)];
#pragma unroll
        for (int s = 0; s < Tr::kSteps; ++s) {
          const Frag af = load_frag_lds<FP8>(arow + s * kStepBytes);
          acc[0] = mma<FP8>(af, qf[0][s], acc[0]);
          acc[1] = mma<FP8>(af, qf[1][s], acc[1]);
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          if (masked) {
            const int rpos = pos0 + 64 * wave + 32 * sub + (lane & 31);
            const int lim = rpos - (b * 128 + 32 * kt + 4 * (lane >> 5));  // key offset bound
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int koff = 8 * (i >> 2) + (i & 3);
              const float v = koff <= lim ? acc[sub][i] : kNegInf;
              m[sub] = fmaxf(m[sub], v);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) m[sub] = fmaxf(m[sub], acc[sub][i]);
          }
        }
      }
      m[0] = fmaxf(m[0], wave_xor32(m[0]));
      m[1] = fmaxf(m[1], wave_xor32(m[1]));
      if (writes) outp[(int64_t)b * a.row_count] = (lane < 32 ? m[0] : m[1]) * scale;
    }
    if (b < b_last) lstore(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_proxy_maxscore(const msa_plan_s* p, const DevMeta& m, const void* pq, const void* pk,
                                 const float* qs, const float* ks, const int32_t* kv_indices, int32_t tile_lo,
                                 int32_t tile_hi, int64_t row_begin, int64_t row_count, float* max_score,
                                 hipStream_t st) {
  if (tile_hi <= tile_lo) return hipSuccess;
  ProxyArgs a;
  a.pq = static_cast<const uint8_t*>(pq);
  a.pk = static_cast<const uint8_t*>(pk);
  a.qs = qs;
  a.ks = ks;
  a.kv_indices = kv_indices;
  a.tiles = m.tiles;
  a.page_start = m.page_start;
  a.tile_lo = tile_lo;
  a.ntiles = tile_hi - tile_lo;
  a.P = p->d.num_proxy_heads;
  a.Pk = p->d.num_proxy_kv_heads;
  a.nb_max = p->nb_max;
  a.row_begin = row_begin;
  a.row_end = row_begin + row_count;
  a.row_count = row_count;
  a.out = max_score;
  a.scale = p->d.proxy_sm_scale;
  const dim3 grid((unsigned)(a.ntiles * a.P)), block(256);
  if (p->d.proxy_dtype == MSA_FP8_E4M3) {
    { ProfScope ps_(p, "proxy_maxscore", st); hipLaunchKernelGGL(proxy_maxscore_kernel<true>, grid, block, 0, st, a); }
  } else {
    { ProfScope ps_(p, "proxy_maxscore", st); hipLaunchKernelGGL(proxy_maxscore_kernel<false>, grid, block, 0, st, a); }
  }
  return hipGetLastError();
}

}  // namespace msa
