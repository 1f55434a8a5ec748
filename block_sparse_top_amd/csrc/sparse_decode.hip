// Stage 3b of MSA: paged sparse decode (MiniMax-AI/MSA README, section
// "Stacks": paged FP8 decode of the sparse attention).  One new query token
// per sequence, already the last key of its sequence, attends to the keys of
// its group's selected 128-key blocks.
//
// Design (gfx950), HBM-bound (every selected K/V byte is read once):
//  * grid = (split, KV group, sequence), 8 waves per workgroup; the valid
//    selected blocks are listed once per workgroup (one ballot), and each
//    block is cut into four 32-key slices dealt round-robin to the waves, so
//    the waves stay balanced (17 blocks = 68 slices over 8 waves) and each
//    wave streams its slices independently, with the next slices' loads in
//    flight while the current one is computed (no workgroup barrier in the
//    loop).  Splits are only used when (sequence, group) pairs are too few to
//    fill the GPU; a small kernel then merges them by log-sum-exp;
//  * S^T = K Q^T on bf16 MFMA 16x16x32: the 32 keys are two 16-row tiles
//    whose rows are interleaved so that each lane ends up holding 8
//    consecutive keys of one head - exactly the B operand layout of the
//    following O^T = V^T P^T product;
//  * fp8 codes are widened to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8);
//    the per-head fp32 scales multiply the logits and the output;
//  * V reaches the A operand through a wave-private, double-buffered LDS
//    tile with transposing reads (ds_read_b64_tr_b8 for fp8,
//    ds_read_b64_tr_b16 for bf16); LDS operations of one wave execute in
//    order, so the wave needs no barrier between its write and its reads;
//  * online softmax per wave; the 8 waves merge through LDS at the end.
#include <mutex>

#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

struct DecodeArgs {
  const uint8_t* q;     // bf16 [S, Hq, 128]
  const uint8_t* kp;    // [N, Hkv, 128, 128] fp8 or bf16
  const uint8_t* vp;
  const float* ks;      // [Hkv] (fp8)
  const float* vs;
  const int32_t* kv_indices;
  const int32_t* sel;   // [S, Hkv, k]
  DevMeta m;
  uint16_t* out;        // bf16 [S, Hq, 128]
  float* lse;           // [S, Hq] or null
  float* part_o;        // [S, Hq, nsplit, 128]
  float* part_ml;       // [S, Hq, nsplit, 2] (lse, unused)
  int32_t Hq, Hkv, G, k, nsplit;
  float scale_log2;
};

template <bool FP8>
struct DecTraits;
template <>
struct DecTraits<true> {
  static constexpr int kRow = 128;      // bytes per key row
  static constexpr int kVRow = 144;     // LDS bytes per V row
  static constexpr int kKLoads = 2;     // 16-byte loads per lane per K tile
  static constexpr int kVLoads = 4;     // 16-byte loads per lane for the slice's V rows
};
template <>
struct DecTraits<false> {
  static constexpr int kRow = 256;
  static constexpr int kVRow = 272;
  static constexpr int kKLoads = 4;
  static constexpr int kVLoads = 8;
};

constexpr int kDecWaves = 8;

template <bool FP8>
struct SliceRegs {
  i32x4 k[2 * DecTraits<FP8>::kKLoads];
  i32x4 v[DecTraits<FP8>::kVLoads];
};

template <bool FP8>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecodeArgs a) {
  using Tr = DecTraits<FP8>;
  constexpr int kVTile = 32 * Tr::kVRow;
  constexpr int kRedBytes = kDecWaves * 16 * (129 + 2) * 4;
  constexpr int kVBytes = kDecWaves * 2 * kVTile;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kVBytes > kRedBytes ? kVBytes : kRedBytes];
  __shared__ int32_t blist[64];
  __shared__ int32_t plist[64];   // their pages, looked up once
  __shared__ int32_t s_nvalid;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q16 = lane >> 4, m16 = lane & 15;
  const int split = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;
  const int G = a.G;
  const int32_t kv_len = a.m.kv[seq];
  const int32_t pos = kv_len - 1;
  const int local = pos >> 7;
  const int32_t* selrow = a.sel + ((int64_t)seq * a.Hkv + g) * a.k;
  const int32_t* pages = a.kv_indices + a.m.page_start[seq];

  // valid selected blocks, in slot order (k <= 64: one wave), and their pages:
  // the slices' K/V loads then depend on no further global load
  if (wave == 0) {
    const int b = lane < a.k ? selrow[lane] : -1;
    const bool ok = b >= 0 && b <= local;
    const uint64_t mask = __ballot(ok);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (ok) {
      blist[before] = b;
      plist[before] = pages[b];
    }
    if (lane == 0) s_nvalid = __popcll(mask);
  }
  __syncthreads();
  const int nslices = 4 * s_nvalid;
  const int per = (nslices + a.nsplit - 1) / a.nsplit;
  const int s_lo = split * per, s_hi = min(nslices, s_lo + per);

  // Q (B operand of S^T): lane -> head m16, d-run 32*q16 .. +32, 8 per k-step
  bf16x8 qf[4];
  {
    const int hh = m16 < G ? m16 : 0;
    const uint8_t* qrow = a.q + ((int64_t)seq * a.Hq + g * G + hh) * 256 + q16 * 64;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(qrow + st * 16);
      if (m16 >= G) qf[st] = bf16x8{};
    }
  }
  const float kscale = FP8 ? a.ks[g] : 1.f;
  const float vscale = FP8 ? a.vs[g] : 1.f;
  const float c = a.scale_log2 * kscale;

  // global loads of one 32-key slice: this lane's two interleaved K rows and
  // half a V row (two lanes per V row)
  auto issue = [&](SliceRegs<FP8>& R, int sl) {
    const int key0 = 32 * (sl & 3);
    const int32_t page = plist[sl >> 2];
    const int64_t blk = ((int64_t)page * a.Hkv + g) * (128 * Tr::kRow);
    const uint8_t* kb = a.kp + blk + (int64_t)key0 * Tr::kRow;
    const uint8_t* vb = a.vp + blk + (int64_t)key0 * Tr::kRow;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // tile j row i=m16 holds key 8*(i/4) + 4*j + i%4 of the slice
      const int key = 8 * (m16 >> 2) + 4 * j + (m16 & 3);
      const uint8_t* src = kb + key * Tr::kRow + q16 * (Tr::kRow / 4);
#pragma unroll
      for (int x = 0; x < Tr::kKLoads; ++x) R.k[j * Tr::kKLoads + x] = *reinterpret_cast<const i32x4*>(src + 16 * x);
    }
    const uint8_t* vsrc = vb + (lane >> 1) * Tr::kRow + (lane & 1) * (Tr::kRow / 2);
#pragma unroll
    for (int x = 0; x < Tr::kVLoads; ++x) R.v[x] = *reinterpret_cast<const i32x4*>(vsrc + 16 * x);
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{};

  auto compute = [&](const SliceRegs<FP8>& R, int sl, uint8_t* vt) {
    const int b = blist[sl >> 2];
    const int key0 = 32 * (sl & 3);
    // V slice -> LDS; rows past kv_len are page padding (may hold NaN, and
    // P = 0 there but 0 * NaN is NaN)
    const bool vrow_ok = b * 128 + key0 + (lane >> 1) < kv_len;
#pragma unroll
    for (int x = 0; x < Tr::kVLoads; ++x)
      lds_store16<i32x4>(vt + (lane >> 1) * Tr::kVRow + (lane & 1) * (Tr::kRow / 2) + 16 * x,
                         vrow_ok ? R.v[x] : i32x4{});
    // S^T tiles
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 af;
        if constexpr (FP8) {
          const i32x4 w = R.k[j * Tr::kKLoads + st / 2];
          af = fp8x8_to_bf16x8((uint32_t)w[(st & 1) * 2], (uint32_t)w[(st & 1) * 2 + 1]);
        } else {
          af = __builtin_bit_cast(bf16x8, R.k[j * Tr::kKLoads + st]);
        }
        sacc[j] = mfma16x16x32(af, qf[st], sacc[j]);
      }
    }
    // lane holds keys key0 + 8*q16 + t, t = 4j + e; mask keys past the position
    const int lim = pos - (b * 128 + key0 + 8 * q16);
    float cm = kNegInf;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = (4 * j + e) <= lim ? sacc[j][e] : kNegInf;
        sacc[j][e] = sv;
        cm = fmaxf(cm, sv);
      }
    }
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = wave_max32(cm);
    const float m_new = fmaxf(m_run, cm);
    // a wave whose keys so far are all masked keeps m = -inf; use 0 as the
    // reference then so that no (-inf) - (-inf) appears
    const float m_ref = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_ref) * c);
    float psum = 0.f;
    float pv[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[4 * j + e] = fast_exp2((sacc[j][e] - m_ref) * c);
        psum += pv[4 * j + e];
      }
    }
    i32x4 pw;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x2 two = {(__bf16)pv[2 * t], (__bf16)pv[2 * t + 1]};
      pw[t] = __builtin_bit_cast(int, two);
    }
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[dt] *= alpha;
      bf16x8 vf;
      if constexpr (FP8) {
        // lane m16 of group q16 gets bytes V[8*q16 + e][16*dt + m16], e = 0..7
        const i32x2 w = lds_read_tr8(vt + (8 * q16 + (m16 >> 1)) * Tr::kVRow + 16 * dt + 8 * (m16 & 1));
        vf = fp8x8_to_bf16x8((uint32_t)w[0], (uint32_t)w[1]);
      } else {
        const s16x4 lo = lds_read_tr16(vt + (8 * q16 + (m16 >> 2)) * Tr::kVRow + (16 * dt + 4 * (m16 & 3)) * 2);
        const s16x4 hi = lds_read_tr16(vt + (8 * q16 + 4 + (m16 >> 2)) * Tr::kVRow + (16 * dt + 4 * (m16 & 3)) * 2);
        vf = join_tr16(lo, hi);
      }
      oacc[dt] = mfma16x16x32(vf, pf, oacc[dt]);
    }
  };

  // this wave's slices: s_lo + wave, + 8, ...; kBufs register buffers (the
  // next kBufs - 1 slices' loads in flight while one is computed), two LDS
  // tiles.  The loop runs whole rounds of kBufs steps, and every step issues
  // its loads: past the last slice they repeat it (in bounds, never
  // computed) and its compute is skipped by a wave-uniform branch.  The loads
  // in flight are then the same on every path, each buffer keeps its
  // registers, and the compiler's wait before each slice is exact.
  constexpr int kBufs = FP8 ? 3 : 2;   // bf16 slices take twice the registers
  uint8_t* vt0 = smem + (2 * wave) * kVTile;
  uint8_t* vt1 = vt0 + kVTile;
  SliceRegs<FP8> rb[kBufs];
  const int sl0 = s_lo + wave;
  const int nsteps = sl0 < s_hi ? (s_hi - sl0 + kDecWaves - 1) / kDecWaves : 0;
  if (nsteps > 0) {
    const int last = s_hi - 1;
    // in buffer order (the loop's waits count on rb[0]'s loads being the oldest)
#pragma unroll
    for (int i = 0; i < kBufs - 1; ++i) {
      issue(rb[i], min(sl0 + kDecWaves * i, last));
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int it = 0; it < nsteps; it += kBufs) {
#pragma unroll
      for (int i = 0; i < kBufs; ++i) {
        const int sl = sl0 + kDecWaves * (it + i);
        issue(rb[(i + kBufs - 1) % kBufs], min(sl + kDecWaves * (kBufs - 1), last));
        if (it + i < nsteps) compute(rb[i], sl, (i & 1) ? vt1 : vt0);
      }
    }
  }

  // waves -> LDS: running max, lane-group sums, O^T (lane holds d = 16dt + 4q16 + e of head m16)
  l_run += __shfl_xor(l_run, 16);
  l_run = wave_sum32(l_run);
  __syncthreads();  // every wave is done with its V tiles; reuse smem
  float* red = reinterpret_cast<float*>(smem);  // [wave][head][131]: o[128], m, l
  float* mine = red + (wave * 16 + m16) * 131;
  if (q16 == 0) {
    mine[128] = m_run;
    mine[129] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[16 * dt + 4 * q16 + e] = oacc[dt][e];
  __syncthreads();

  // combine the waves: thread -> (head, 4 consecutive d) for 16 heads x 128 d
  const int hh = tid >> 5;          // 16 heads
  const int d0 = (tid & 31) * 4;    // 32 x 4 = 128
  if (hh < G) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red[(w * 16 + hh) * 131 + 128]);
    float wsum = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* rw = red + (w * 16 + hh) * 131;
      const float f = rw[128] == kNegInf ? 0.f : fast_exp2((rw[128] - M) * c);
      wsum += f * rw[129];
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] += f * rw[d0 + x];
    }
    const int h = g * G + hh;
    const float lse_v = (wsum > 0.f) ? (M * c + fast_log2(wsum)) * kLn2 : kNegInf;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (a.nsplit == 1) {
      bf16x4 ob;
      const bf16x2 lo2 = {(__bf16)(o[0] * inv * vscale), (__bf16)(o[1] * inv * vscale)};
      const bf16x2 hi2 = {(__bf16)(o[2] * inv * vscale), (__bf16)(o[3] * inv * vscale)};
      const i32x2 pk = {__builtin_bit_cast(int, lo2), __builtin_bit_cast(int, hi2)};
      ob = __builtin_bit_cast(bf16x4, pk);
      *reinterpret_cast<bf16x4*>(a.out + ((int64_t)seq * a.Hq + h) * 128 + d0) = ob;
      if (a.lse && d0 == 0) a.lse[(int64_t)seq * a.Hq + h] = lse_v;
    } else {
      float* po = a.part_o + (((int64_t)seq * a.Hq + h) * a.nsplit + split) * 128 + d0;
#pragma unroll
      for (int x = 0; x < 4; ++x) po[x] = o[x] * inv * vscale;
      if (d0 == 0) a.part_ml[(((int64_t)seq * a.Hq + h) * a.nsplit + split) * 2] = lse_v;
    }
  }
}

// Merge decode splits: one wave per (sequence, head), lane -> 2 columns.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* part_o, const float* part_ml, uint16_t* out,
                                                           float* lse, int32_t S, int32_t Hq, int32_t nsplit) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)S * Hq) return;
  float M = kNegInf;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, part_ml[(idx * nsplit + sp) * 2]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float l = part_ml[(idx * nsplit + sp) * 2];
    if (l == kNegInf) continue;
    const float w = fast_exp2((l - M) * kLog2e);
    const f32x2 v = *reinterpret_cast<const f32x2*>(part_o + (idx * nsplit + sp) * 128 + 2 * lane);
    L += w;
    o0 += w * v[0];
    o1 += w * v[1];
  }
  bf16x2 o;
  o[0] = (__bf16)(o0 / L);
  o[1] = (__bf16)(o1 / L);
  *reinterpret_cast<bf16x2*>(out + idx * 128 + 2 * lane) = o;
  if (lse && lane == 0) lse[idx] = M + fast_log2(L) * kLn2;
}

// Scratch of msa_sparse_attn_decode_noalloc: the plan metadata and the split
// partials live here instead of in a caller workspace.  Each device holds its
// own copy (allocated with the code object, kept until the process ends);
// host code uses only the per-device address from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

hipError_t launch_decode(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                         const float* ks, const float* vs, const int32_t* kv_indices, const int32_t* sel,
                         void* out, float* lse, char* ws, hipStream_t st) {
  DecodeArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.kp = static_cast<const uint8_t*>(kp);
  a.vp = static_cast<const uint8_t*>(vp);
  a.ks = ks;
  a.vs = vs;
  a.kv_indices = kv_indices;
  a.sel = sel;
  a.m = m;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.part_o = reinterpret_cast<float*>(ws + p->lay.dec_o);
  a.part_ml = reinterpret_cast<float*>(ws + p->lay.dec_ml);
  a.Hq = p->d.num_qo_heads;
  a.Hkv = p->d.num_kv_heads;
  a.G = p->G;
  a.k = p->d.topk;
  a.nsplit = p->dec_splits;
  a.scale_log2 = p->d.sm_scale * kLog2e;
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)p->S), block(64 * kDecWaves);
  {
    ProfEvents pe(p, "decode");
    if (p->d.kv_dtype == MSA_FP8_E4M3)
      hipExtLaunchKernelGGL(decode_kernel<true>, grid, block, 0, st, pe.start, pe.stop, 0, a);
    else
      hipExtLaunchKernelGGL(decode_kernel<false>, grid, block, 0, st, pe.start, pe.stop, 0, a);
  }
  if (a.nsplit > 1) {
    const int64_t nw = (int64_t)p->S * a.Hq;
    ProfEvents pe(p, "decode_merge");
    hipExtLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, st, pe.start, pe.stop, 0,
                          a.part_o, a.part_ml, a.out, lse, p->S, a.Hq, a.nsplit);
  }
  return hipGetLastError();
}

}  // namespace msa
