// Stage 1 of MSA: proxy block max scores, and optionally the top-k block
// selection fused into the same pass.
//
// The proxy pass of the MiniMax-AI/MSA README (section "Usage": dense pass,
// output_o off, output_maxscore on) and the max-pooling of proxy scores over
// 128-token KV blocks of the Flash-MSA article (paragraph comparing MSA with
// DSA): for each query row and proxy head, the largest scaled proxy logit in
// every causally visible 128-key block.
//
// Design (gfx950):
//  * one workgroup = 512 threads = 8 waves, one proxy head, one row tile of
//    up to 512 rows whose positions share a 512-aligned window; wave w owns
//    rows 64w .. 64w+63 as two 32-row MFMA column tiles, so each K tile
//    staged in LDS feeds 512 rows;
//  * S^T = K Q^T on MFMA (bf16 32x32x16 or fp8 32x32x64): keys are the MFMA
//    rows, queries the columns, so each lane holds one query row and the
//    max over keys is an in-register reduction plus one lane swap;
//  * the tile's proxy Q stays in registers for the whole key loop; each K
//    block (one page of one head, 32 KB bf16 / 16 KB fp8) goes straight from
//    global memory into one of two LDS tiles (global_load_lds_dwordx4, no
//    registers) while the other is being read; every A fragment read from
//    LDS feeds two MFMAs (the wave's two row tiles);
//  * only blocks up to the tile's last local block are visited; the two
//    boundary blocks apply the per-row causal mask; scales are applied after
//    the max (they are positive);
//  * workgroup order: workgroups of one proxy head are consecutive modulo
//    the head count, so with 8 proxy heads each XCD streams one head's K
//    through its own L2; long (late) tiles launch first.
#include <type_traits>

#include "device_common.hpp"
#include "msa_internal.hpp"
#include "proxy_exact.hpp"

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
  float* out;                // [P, nb_max, row_count] (block max scores) or null
  int32_t* sel;              // [T, P, k] selections when fused with top-k, else null
  int32_t k;                 // slots per (row, group), local block included (fused path)
  float scale;
  // low-precision proxies, fused path: (row, group) pairs whose selection the
  // score error bound cannot certify, queued for exact re-scoring
  int32_t* rq;               // [row_count * P][kRqInts]
  int32_t* rq_count;         // entries queued (zeroed before the pass)
};

// Fused selection: each lane keeps its row's best kSelCap (score, block)
// pairs in descending score order.  Blocks arrive in ascending order and an
// equal score never displaces a listed one, so ties go to the lower block,
// exactly as in the separate top-k over the same fp32 scores.  The
// low-precision formats keep kSelCapLowp pairs: the extra ones hold the
// blocks just below the boundary, which the score error bound may leave
// undecided (see the epilogue).
constexpr int kSelCap = 16;
constexpr int kSelCapLowp = 24;

// A queued (row, group) pair: [0] row, [1] the row's first page-table entry
// (offset into kv_indices), [2] n_in | m << 8 | overflow << 16, [3 .. 15) the
// list's 24 block ids as 16-bit pairs (in list order: descending
// low-precision score), [15] local block | proxy head << 16.
constexpr int kRqInts = 16;

// MXFP4 K rows are 64 bytes of E2M1 codes; the block's 128 x 4 E8M0 scale
// bytes follow the codes (page record); an MXFP4 q row is 64 code bytes then
// its 4 scale bytes.

template <Fmt F>
struct ProxyTraits;

// K tiles live in LDS unpadded, with the 16-byte chunks of each row permuted
// (physical chunk = logical chunk ^ swz(row)) so that the 16 rows read by a
// fragment load hit 16 distinct bank groups.
template <>
struct ProxyTraits<Fmt::BF16> {
  static constexpr int kQRowBytes = 256;      // one proxy q row (one head)
  static constexpr int kKRowBytes = 256;      // one key row
  static constexpr int kKBlockBytes = 128 * 256;
  static constexpr int kSteps = 8;            // MFMA k-steps over d = 128
  __device__ static int swz(int row) { return row & 15; }
  typedef bf16x8 AFrag;
  typedef bf16x8 BFrag;
};
template <>
struct ProxyTraits<Fmt::FP8> {
  static constexpr int kQRowBytes = 128;
  static constexpr int kKRowBytes = 128;
  static constexpr int kKBlockBytes = 128 * 128;
  static constexpr int kSteps = 2;
  __device__ static int swz(int row) { return (row >> 1) & 7; }
  typedef i32x8 AFrag;
  typedef i32x8 BFrag;
};
template <>
struct ProxyTraits<Fmt::MX4K> {
  static constexpr int kQRowBytes = 128;
  static constexpr int kKRowBytes = 64;
  static constexpr int kKBlockBytes = 128 * 64 + 128 * 4;
  static constexpr int kSteps = 2;
  __device__ static int swz(int row) { return (row >> 2) & 3; }
  typedef i32x4 AFrag;
  typedef i32x8 BFrag;
};
template <>
struct ProxyTraits<Fmt::MX4QK> {
  static constexpr int kQRowBytes = 68;
  static constexpr int kKRowBytes = 64;
  static constexpr int kKBlockBytes = 128 * 64 + 128 * 4;
  static constexpr int kSteps = 2;
  __device__ static int swz(int row) { return (row >> 2) & 3; }
  typedef i32x4 AFrag;
  typedef i32x4 BFrag;
};

template <Fmt F>
constexpr bool kMxK = F == Fmt::MX4K || F == Fmt::MX4QK;

template <bool FP8>
__device__ __forceinline__ typename std::conditional<FP8, i32x8, bf16x8>::type load_frag_global(const uint8_t* p) {
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

// 16 bytes from a 4-byte aligned address (MXFP4 q rows are 68 bytes apart)
__device__ __forceinline__ i32x4 load16_a4(const uint8_t* p) {
  const int32_t* q = reinterpret_cast<const int32_t*>(p);
  return i32x4{q[0], q[1], q[2], q[3]};
}

// The B fragment (proxy q) of k-step st for lane half h, from a q row in
// global memory; for MXFP4 q also the lane's scale word (byte 2st + h is
// picked by op_sel 2st after the shift).  FP4 operands: lane half h holds
// one whole 32-dim MX block, 2st + h (codes 0-15 at k = 16h.., 16-31 at
// k = 32 + 16h..); the fp8 q of the (fp8 q, MXFP4 K) pair is gathered in
// that k order: dims 64st + 16h .. +15, then 64st + 32 + 16h .. +15.
template <Fmt F>
__device__ __forceinline__ typename ProxyTraits<F>::BFrag load_q_frag(const uint8_t* row, int st, int h) {
  using Tr = ProxyTraits<F>;
  if constexpr (F == Fmt::BF16 || F == Fmt::FP8) {
    constexpr int kStepBytes = Tr::kQRowBytes / Tr::kSteps;
    return load_frag_global<F == Fmt::FP8>(row + st * kStepBytes + h * (kStepBytes / 2));
  } else if constexpr (F == Fmt::MX4K) {
    const i32x4 x = *reinterpret_cast<const i32x4*>(row + 64 * st + 16 * h);
    const i32x4 y = *reinterpret_cast<const i32x4*>(row + 64 * st + 32 + 16 * h);
    return i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  } else {
    return load16_a4(row + 16 * (2 * st + h));
  }
}

// The A fragment (K) of key row `row`, k-step st, lane half h, from an LDS tile.
template <Fmt F>
__device__ __forceinline__ typename ProxyTraits<F>::AFrag load_k_frag(const uint8_t* tile, int row, int st, int h) {
  using Tr = ProxyTraits<F>;
  const uint8_t* base = tile + row * Tr::kKRowBytes;
  if constexpr (F == Fmt::BF16) {
    return lds_load16<bf16x8>(base + (((h + 2 * st) ^ Tr::swz(row)) << 4));
  } else if constexpr (F == Fmt::FP8) {
    const int c = 2 * h + 4 * st;
    i32x4 a = lds_load16<i32x4>(base + ((c ^ Tr::swz(row)) << 4));
    i32x4 b = lds_load16<i32x4>(base + (((c + 1) ^ Tr::swz(row)) << 4));
    return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    return lds_load16<i32x4>(base + (((2 * st + h) ^ Tr::swz(row)) << 4));
  }
}

// One k-step of S^T = K Q^T.  sa / sb: the lanes' E8M0 scale words (MXFP4
// operands), byte 2st picked by op_sel; fp8 operands take scale 2^0.
template <Fmt F>
__device__ __forceinline__ f32x16 mma(const typename ProxyTraits<F>::AFrag& a,
                                      const typename ProxyTraits<F>::BFrag& b, const f32x16& c, int st, int32_t sa,
                                      int32_t sb) {
  if constexpr (F == Fmt::BF16) {
    return mfma32x32x16(a, b, c);
  } else if constexpr (F == Fmt::FP8) {
    return mfma32x32x64_fp8(a, b, c);
  } else if constexpr (F == Fmt::MX4K) {
    const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    return st == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 0, sa, 0, 127)
                   : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 2, sa, 0, 127);
  } else {
    const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return st == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb)
                   : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 2, sa, 2, sb);
  }
}

// 4 waves of 64 rows: a workgroup covers half of a 512-row plan tile, so two
// workgroups (2 waves per SIMD each) share a CU and one's per-block barrier
// or K fetch overlaps the other's MFMAs
constexpr int kProxyWaves = 4;
constexpr int kProxySubs = 512 / (64 * kProxyWaves);

template <Fmt F, bool TOPK>
__global__ __launch_bounds__(64 * kProxyWaves, 2) void proxy_maxscore_kernel(ProxyArgs a) {
  using Tr = ProxyTraits<F>;
  using AFrag = typename Tr::AFrag;
  using BFrag = typename Tr::BFrag;
  constexpr int kBlockBytes = Tr::kKBlockBytes;           // one K block in global memory
  constexpr int kCodeBytes = 128 * Tr::kKRowBytes;        // its key rows (MXFP4: the scales follow)
  constexpr int kStageLoads = kCodeBytes / (F == Fmt::BF16 ? 2 : 1) / 1024 / kProxyWaves;  // 1 KB loads per wave per stage
  constexpr int kChunksPerRow = Tr::kKRowBytes / 16;
  constexpr int kRowsPerKB = 1024 / Tr::kKRowBytes;
  // K arrives in stages through a ring of four LDS tiles, each stage issued
  // three stages before it is used: half blocks (64 key rows) for bf16,
  // whole blocks for the smaller fp8 and MXFP4 blocks (an MXFP4 tile: the
  // codes, then the rows' scales).  Four distinct tile objects (not one array
  // indexed by a runtime buffer number): the loads in flight into three of
  // them are then provably disjoint from the reads of the fourth.
  constexpr int kParts = F == Fmt::BF16 ? 2 : 1;        // stages per block
  constexpr int kStageBytes = kBlockBytes / kParts;
  constexpr int kStageCodeBytes = kCodeBytes / kParts;
  constexpr int kStageRows = 128 / kParts;
  __shared__ __attribute__((aligned(1024))) uint8_t h0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t h1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t h2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t h3[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hsel = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave branches stay scalar
  const int p = blockIdx.x % a.P;
  const int qi = (int)(blockIdx.x / a.P);
  const int t = a.tile_lo + (a.ntiles - 1 - qi / kProxySubs);   // long tiles first
  const int part = kProxySubs - 1 - qi % kProxySubs;            // and their later rows first
  const int seq = a.tiles[4 * t + 0];
  const int row0 = a.tiles[4 * t + 1] + 64 * kProxyWaves * part;
  const int nrows = min(64 * kProxyWaves, a.tiles[4 * t + 2] - 64 * kProxyWaves * part);
  if (nrows <= 0) return;
  const int pos0 = a.tiles[4 * t + 3] + 64 * kProxyWaves * part;
  const int ph = (a.Pk == a.P) ? p : 0;
  const int32_t* pages = a.kv_indices + a.page_start[seq];
  const int b_last = (pos0 + nrows - 1) >> 7;
  const int b_full = (pos0 + 1) >> 7;  // blocks < b_full are visible to every row of the tile

  // Q fragments (B operand): lane -> query column lane%32 of row tile `sub`,
  // k-run (lane/32) of each k-step; MXFP4 q also a scale word per row.
  BFrag qf[2][Tr::kSteps];
  int32_t qsc[2] = {0x7f7f7f7f, 0x7f7f7f7f};
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int r = 64 * wave + 32 * sub + (lane & 31);
    const bool valid = r < nrows;
    const uint8_t* src = a.pq + ((int64_t)(row0 + (valid ? r : 0)) * a.P + p) * Tr::kQRowBytes;
#pragma unroll
    for (int s = 0; s < Tr::kSteps; ++s) {
      qf[sub][s] = load_q_frag<F>(src, s, hsel);
      if (!valid) qf[sub][s] = BFrag{};
    }
    if constexpr (F == Fmt::MX4QK) {
      if (valid) qsc[sub] = (int32_t)(*reinterpret_cast<const uint32_t*>(src + 64) >> (8 * hsel));
    }
  }

  // Stage `part` of a K block -> LDS without registers: each wave issues
  // kStageLoads direct 1 KB loads (global_load_lds_dwordx4: lane i fills
  // bytes 16i..16i+15 of the KB), fetching for each lane the global chunk its
  // swizzled slot holds (the swizzle depends on the row modulo 16, so tile
  // and block rows agree); an MXFP4 block's 512 scale bytes follow
  // unswizzled (the last wave).
  auto kload = [&](int32_t page, int part, uint8_t* tile) {
    const uint8_t* src = a.pk + ((int64_t)page * a.Pk + ph) * kBlockBytes;
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int kb = wave + kProxyWaves * i;             // which KB of the tile
      const int row = kStageRows * part + kb * kRowsPerKB + lane / kChunksPerRow;
      const int pc = lane % kChunksPerRow;               // physical chunk written by this lane
      const int lc = pc ^ Tr::swz(row);                  // logical chunk it must hold
      global_load_lds16(src + row * Tr::kKRowBytes + lc * 16, (MSA_LDS void*)(tile + kb * 1024));
    }
    if constexpr (kMxK<F>) {
      static_assert(kParts == 1, "MXFP4 K stages are whole blocks");
      if (wave == kProxyWaves - 1 && lane < 32)
        global_load_lds16(src + kCodeBytes + lane * 16, (MSA_LDS void*)(tile + kCodeBytes));
    }
  };

  float scale = a.scale;
  if constexpr (F == Fmt::FP8) scale *= a.qs[p] * a.ks[ph];
  if constexpr (F == Fmt::MX4K) scale *= a.qs[p];
  const bool wave_active = 64 * wave < nrows;
  const int my_row = 64 * wave + lane;          // row this lane writes
  const int64_t my_grow = row0 + my_row;
  const bool writes = my_row < nrows && my_grow >= a.row_begin && my_grow < a.row_end;
  float* outp = a.out + (int64_t)p * a.nb_max * a.row_count + (my_grow - a.row_begin);

  const int my_local = (pos0 + my_row) >> 7;   // this lane's row's local block
  constexpr bool LOWP = TOPK && F != Fmt::BF16;  // low-precision scores: selection certified or re-scored
  constexpr int kCap = LOWP ? kSelCapLowp : (TOPK ? kSelCap : 1);
  float tv[kCap];
  int ti[kCap];
#pragma unroll
  for (int j = 0; j < kCap; ++j) {
    tv[j] = kNegInf;
    ti[j] = -1;
  }
  // largest |q_d| of the lane's row (code units; MXFP4 q: its largest block
  // scale times 6) and, for MXFP4 K, the largest K scale code seen
  float qinf = 0.f;
  uint32_t kmaxe = 0;
  if constexpr (LOWP) {
    float pm[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if constexpr (F == Fmt::MX4QK) {
        pm[sub] = 6.0f * e8m0_value(max(qsc[sub] & 0xff, (qsc[sub] >> 16) & 0xff));
      } else {
        float m = 0.f;
#pragma unroll
        for (int st = 0; st < Tr::kSteps; ++st)
#pragma unroll
          for (int w = 0; w < (int)(sizeof(BFrag) / 4); ++w) m = fmaxf(m, e4m3_absmax4((uint32_t)qf[sub][st][w]));
        pm[sub] = m;
      }
      pm[sub] = wave_max32(pm[sub]);
    }
    qinf = lane < 32 ? pm[0] : pm[1];
  }

  // Fused selection: after each block, its score is inserted into the row's
  // list, sorted by descending score with equal scores in ascending block
  // order.  A new block has a larger id than every listed one, so inserting
  // score v is a slot-parallel update (slots rewritten from the last to the
  // first): slot j takes med3(old[j-1], v, old[j]) as its score, and keeps its
  // block if v <= old[j], takes the new block if old[j-1] >= v > old[j], else
  // the block of slot j-1 (strict compares: an equal listed score stays
  // ahead, so ties keep the lower block id).
  float pend_v = 0.f, cv = kNegInf;
  int pend_b = 0, ci = 0;
  bool pend_ok = false;
  auto ins_begin = [&]() {
    cv = pend_ok ? pend_v : kNegInf;  // -inf changes nothing
    ci = pend_b;
  };
  auto ins_steps = [&](int r) {  // slots kCap-1 - 4r down to kCap-4 - 4r
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = kCap - 1 - (4 * r + jj);
      const bool gj = cv > tv[j];
      const bool gp = j > 0 ? cv > tv[j > 0 ? j - 1 : 0] : false;
      const float up = j > 0 ? tv[j > 0 ? j - 1 : 0] : kPosInf;
      const int upi = j > 0 ? ti[j > 0 ? j - 1 : 0] : 0;
      // selects, not branches (every lane updates its own list)
      const int nv = __builtin_unpredictable(gp) ? upi : ci;
      ti[j] = __builtin_unpredictable(gj) ? nv : ti[j];
      tv[j] = __builtin_amdgcn_fmed3f(up, cv, tv[j]);
    }
  };

  // keys 64 hf .. 64 hf + 63 of block b (their key rows from `tile`, their
  // MXFP4 scale words from `scales`): m takes the max over them (rows `sub`
  // of the lane's two row tiles)
  auto half_max = [&](const uint8_t* tile, const uint8_t* scales, int b, int hf, float (&m)[2]) {
    {
      f32x16 acc[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = f32x16{};
      int32_t ksc[2] = {0, 0};
      if constexpr (kMxK<F>) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          ksc[j] = (int32_t)(lds_load16<uint32_t>(scales + 4 * (32 * j + (lane & 31))) >> (8 * hsel));
          // bytes 0 and 2 of the shifted word are the ones this lane's MFMAs
          // use.  Only blocks before the tile's last local block can compete
          // for any of its rows, and they are whole (a sequence's partial last
          // block, whose slots past kv_len may hold anything, never competes).
          if constexpr (LOWP)
            if (b < b_last) kmaxe = max(kmaxe, max((uint32_t)ksc[j] & 0xffu, ((uint32_t)ksc[j] >> 16) & 0xffu));
        }
      }
      AFrag fr[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) fr[0][j] = load_k_frag<F>(tile, 32 * j + (lane & 31), 0, hsel);
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) {
        if (st + 1 < Tr::kSteps) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            fr[(st + 1) & 1][j] = load_k_frag<F>(tile, 32 * j + (lane & 31), st + 1, hsel);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j][0] = mma<F>(fr[st & 1][j], qf[0][st], acc[j][0], st, ksc[j], qsc[0]);
          acc[j][1] = mma<F>(fr[st & 1][j], qf[1][st], acc[j][1], st, ksc[j], qsc[1]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep LDS fragment reads one k-step ahead at most
      }
      if (b >= b_full) {
        // boundary block: key (32kt + 8(i/4) + 4(lane/32) + i%4) is visible to
        // this lane's row iff its position does not exceed the row's
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int lim = pos0 + 64 * wave + 32 * sub + (lane & 31) - (b * 128 + 4 * (lane >> 5));
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; i += 2)
              m[sub] = max3f(m[sub], (32 * (2 * hf + j) + 8 * (i >> 2) + (i & 3)) <= lim ? acc[j][sub][i] : kNegInf,
                             (32 * (2 * hf + j) + 8 * (i >> 2) + (i & 3) + 1) <= lim ? acc[j][sub][i + 1] : kNegInf);
        }
      } else {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; i += 2) m[sub] = max3f(m[sub], acc[j][sub][i], acc[j][sub][i + 1]);
      }
    }
  };
  auto finish = [&](int b, float (&m)[2]) {
    m[0] = wave_max32(m[0]);
    m[1] = wave_max32(m[1]);
    const float v = (lane < 32 ? m[0] : m[1]) * scale;
    if constexpr (TOPK) {
      // blocks before the local one compete (the local block is forced);
      // inserted during the next block
      pend_v = v;
      pend_b = b;
      pend_ok = b < my_local;
      ins_begin();
      // a score not above the list's last entry changes nothing: skip the
      // insertion when that holds for every row of the wave (on long rows,
      // most blocks once the lists have filled)
      if (__builtin_amdgcn_ballot_w64(cv > tv[kCap - 1]) != 0) {
#pragma unroll
        for (int r = 0; r < kCap / 4; ++r) ins_steps(r);
      }
    } else {
      if (writes) outp[(int64_t)b * a.row_count] = v;
    }
  };

  // Page ids: lane i holds page (64*w + i) of window w; the next window is
  // loaded a whole window ahead, and the id of a block is picked with a
  // uniform-index lane read, so no page-table latency sits in the loop.
  int pw_cur = lane <= b_last ? pages[lane] : 0;
  int pw_next = 64 + lane <= b_last ? pages[64 + lane] : 0;
  int cur_w = 0;
  auto page_of = [&](int x) -> int32_t {
    return __builtin_amdgcn_readlane((x >> 6) == cur_w ? pw_cur : pw_next, x & 63);
  };
  auto advance = [&](int x) {  // x: the block about to be computed
    if ((x & 63) == 0 && (x >> 6) != cur_w) {
      pw_cur = pw_next;
      cur_w = x >> 6;
      const int nx = 64 * (cur_w + 1) + lane;
      pw_next = nx <= b_last ? pages[nx] : 0;
    }
  };

  // Stages s = 2 b + hf over the blocks' halves, loop unrolled by four over
  // the four tiles: stage s waits for its own half (the two later halves may
  // stay in flight), a barrier makes every wave's part of it visible and
  // frees stage s - 1's tile, into which the half of stage s + 3 is issued
  // before stage s computes.  Past the last stage the loads repeat it (in
  // bounds, never read), so every stage issues the same loads and the wait
  // count is exact; groups run unconditionally and the two stages of an odd
  // last block follow the loop (no branch inside the loop body that the
  // per-row selection state has to flow through).
  const int S = kParts * (b_last + 1);
  auto issue = [&](int s2, uint8_t* tile) {
    const int ss = min(s2, S - 1);
    kload(page_of(ss / kParts), ss % kParts, tile);
  };
  float m[2] = {kNegInf, kNegInf};
  // `part` is a constant at each call (stages s2 with s2 % kParts == part)
  auto stage = [&](int s2, int part, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    const int b = s2 / kParts;
    // this wave's part of stage s2 has landed; after the barrier every wave's
    // has, and every wave is done with stage s2 - 1's tile (its reads fed
    // that stage's products).  No workgroup fence: it would wait for every
    // load in flight, the ring included.
    wait_vmcnt<2 * kStageLoads>();
    lds_barrier();
    if (part == 0) advance(b);
    issue(s2 + 3, nxt);
    if (wave_active) {
      if (part == 0) m[0] = m[1] = kNegInf;
      if constexpr (kParts == 2) {
        half_max(cur, cur, b, part, m);
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) half_max(cur + 64 * hf * Tr::kKRowBytes, cur + kCodeBytes + 256 * hf, b, hf, m);
      }
      if (part == kParts - 1) finish(b, m);
    }
  };
  issue(0, h0);
  issue(1, h1);
  issue(2, h2);
  __syncthreads();  // the q fragments' loads above are long done; a plain barrier before the ring
  int s2 = 0;
  for (; s2 + 3 < S; s2 += 4) {
    stage(s2, 0, h0, h3);
    stage(s2 + 1, 1 % kParts, h1, h0);
    stage(s2 + 2, 0, h2, h1);
    stage(s2 + 3, 1 % kParts, h3, h2);
  }
  // the last S % 4 stages (S % 4 is 0 or 2 for half-block stages)
  if (s2 < S) stage(s2, 0, h0, h3);
  if (s2 + 1 < S) stage(s2 + 1, 1 % kParts, h1, h0);
  if (s2 + 2 < S) stage(s2 + 2, 0, h2, h1);
  wait_all_mem();  // the repeated loads past the last stage land before the workgroup ends

  if constexpr (TOPK) {
    // the R = min(k - 1, local) best earlier blocks and the local block, ascending, -1 padded
    const int R = min(a.k - 1, my_local);
    bool queued = false;
    if constexpr (LOWP) {
      // Low-precision scores f are within delta of the exact scores s.  With
      // theta = the R-th largest f: a listed block with f > theta + 2 delta
      // beats every block with f <= theta exactly, so it is in the exact top
      // R ("sure"); a block with f < theta - 2 delta is beaten by the R listed
      // blocks with f >= theta, so it is out.  When exactly R blocks have
      // f >= theta - 2 delta (and, if blocks were dropped from the list, the
      // last listed one is below that too), the list's top R is the exact top
      // R.  Otherwise the pair is queued: the blocks in the band are
      // re-scored exactly (all competing blocks if the band may run past the
      // list).
      uint32_t ke = kmaxe;
      if constexpr (kMxK<F>) {
        // largest K scale code over every block the workgroup visited (each
        // lane saw its rows' codes for every block)
        ke = max(ke, (uint32_t)__shfl_xor((int)ke, 32));
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) ke = max(ke, (uint32_t)__shfl_xor((int)ke, o));
      }
      const float kinf = kMxK<F> ? 6.0f * e8m0_value(ke) : 448.0f;
      // delta, rounded up a little against the fp32 products above
      const float delta = ScoreBound<F>::kCoef * 1.0001f * scale * qinf * kinf;
      const float theta = tv[R > 0 ? R - 1 : 0];
      int n_in = 0, m = 0;
#pragma unroll
      for (int j = 0; j < kCap; ++j) {
        // entries past the row's competing blocks were never filled
        n_in += (j < R && tv[j] > theta + 2.f * delta) ? 1 : 0;
        m += (j < my_local && tv[j] >= theta - 2.f * delta) ? 1 : 0;
      }
      const bool ovf = my_local > kCap && tv[kCap - 1] >= theta - 2.f * delta;
      const bool unc = writes && R > 0 && R < my_local && n_in < R && (m > R || ovf);
      const uint64_t mask = __ballot(unc);
      if (mask) {
        const int first = (int)__builtin_ctzll(mask);
        int base = 0;
        if (lane == first) base = atomicAdd(a.rq_count, __popcll(mask));
        base = __builtin_amdgcn_readlane(base, first);
        if (unc) {
          int32_t* e = a.rq + (int64_t)(base + lanes_below(mask)) * kRqInts;
          e[0] = (int32_t)my_grow;
          e[1] = a.page_start[seq];
          e[2] = n_in | (m << 8) | ((ovf ? 1 : 0) << 16);
#pragma unroll
          for (int j = 0; j < kCap; j += 2) e[3 + j / 2] = (ti[j] & 0xffff) | (ti[j + 1] << 16);
          e[15] = my_local | (p << 16);
        }
      }
      queued = unc;
    }
    if (writes && !queued) {
#pragma unroll
      for (int j = 0; j < kCap; ++j)
        if (j >= R) ti[j] = 0x7fffffff;
#pragma unroll
      for (int rnd = 0; rnd < kCap; ++rnd)  // odd-even transposition sort by block id
#pragma unroll
        for (int j = rnd & 1; j + 1 < kCap; j += 2) {
          const int x = ti[j], y = ti[j + 1];
          ti[j] = min(x, y);
          ti[j + 1] = max(x, y);
        }
      int32_t* dst = a.sel + ((int64_t)my_grow * a.P + p) * a.k;
#pragma unroll
      for (int j = 0; j <= kSelCap; ++j) {
        if (j >= a.k) break;
        const int v = j < R ? ti[j < kCap ? j : 0] : (j == R ? my_local : -1);
        dst[j] = v;
      }
    }
  }
}

// Exact re-scoring of the queued (row, group) pairs of the fused
// low-precision pass.  One wave per pair, looping over the queue: the band
// blocks of the pair's list (or, if the band may run past the list, every
// competing block not already sure) in ascending block order; each is scored
// exactly (exact_block_dotmax), the need = R - n_in best are kept with ties to
// the lower block, and the row is written like the fused pass writes it.  The
// entry carries everything the pair needs (no plan metadata is read); the
// band blocks' page ids are loaded lane-parallel before the first is scored.
template <Fmt F>
__global__ __launch_bounds__(256) void topk_refine_kernel(ProxyArgs a) {
  using Tr = ProxyTraits<F>;
  __shared__ int32_t cand_lds[4][kSelCapLowp];
  __shared__ int32_t cand_pg[4][kSelCapLowp];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int count = __builtin_amdgcn_readfirstlane(*a.rq_count);
  for (int e = blockIdx.x * 4 + wave; e < count; e += gridDim.x * 4) {
    const int32_t* ent = a.rq + (int64_t)e * kRqInts;
    const int ev = lane < kRqInts ? ent[lane] : 0;  // the entry, one int per lane
    const int r = __builtin_amdgcn_readlane(ev, 0);
    const int32_t* pages = a.kv_indices + __builtin_amdgcn_readlane(ev, 1);
    const int hdr = __builtin_amdgcn_readlane(ev, 2);
    const int lp = __builtin_amdgcn_readlane(ev, 15);
    const int n_in = hdr & 0xff, m = (hdr >> 8) & 0xff;
    const bool ovf = (hdr >> 16) & 1;
    const int local = lp & 0xffff, p = (int)((uint32_t)lp >> 16);
    const int R = min(a.k - 1, local);
    const int need = R - n_in;
    // list ids: lane j < 24 holds entry j
    const int lw = __shfl(ev, 3 + min(lane, kSelCapLowp - 1) / 2);
    const int lid = lane < kSelCapLowp ? (int)((uint32_t)lw >> (16 * (lane & 1))) & 0xffff : 0x7fffffff;
    const bool cand = !ovf && lane >= n_in && lane < m && lid < local;
    const int32_t cpg = cand ? pages[lid] : 0;
    const int ph = a.Pk == a.P ? p : 0;
    const uint8_t* qrow = a.pq + ((int64_t)r * a.P + p) * Tr::kQRowBytes;
    const ExactQ q = exact_load_q<F>(qrow);
    float sc = a.scale;
    if constexpr (F == Fmt::FP8) sc *= a.qs[p] * a.ks[ph];
    if constexpr (F == Fmt::MX4K) sc *= a.qs[p];
    // the uniform top-`need` list (every lane holds a copy)
    float bv[kSelCap];
    int bi[kSelCap];
#pragma unroll
    for (int j = 0; j < kSelCap; ++j) {
      bv[j] = kNegInf;
      bi[j] = 0x7fffffff;
    }
    auto consider = [&](int b, int32_t page) {
      const uint8_t* blk = a.pk + ((int64_t)page * a.Pk + ph) * Tr::kKBlockBytes;
      const float v = exact_block_dotmax<F>(q, blk, 128) * sc;
      // insert before the first strictly smaller listed score (ascending block
      // order: equal scores keep the lower block ahead)
#pragma unroll
      for (int j = kSelCap - 1; j >= 0; --j) {
        const bool gj = j < need && v > bv[j];
        const bool gp = j > 0 && v > bv[j > 0 ? j - 1 : 0];
        if (gj) {
          bv[j] = gp ? bv[j > 0 ? j - 1 : 0] : v;
          bi[j] = gp ? bi[j > 0 ? j - 1 : 0] : b;
        }
      }
    };
    if (!ovf) {
      // band entries n_in .. m-1, visited in ascending block order
      const uint64_t cm = __ballot(cand);
      int rank = 0;
      for (int j = n_in; j < m; ++j)
        rank += ((cm >> j) & 1) && __builtin_amdgcn_readlane(lid, j) < lid ? 1 : 0;
      if (cand) {
        cand_lds[wave][rank] = lid;
        cand_pg[wave][rank] = cpg;
      }
      wave_lds_sync();
      const int nc = __popcll(cm);
      for (int c = 0; c < nc; ++c)
        consider(__builtin_amdgcn_readfirstlane(cand_lds[wave][c]), __builtin_amdgcn_readfirstlane(cand_pg[wave][c]));
      wave_lds_sync();
    } else {
      // every competing block except the sure ones, page ids 64 at a time
      for (int b0 = 0; b0 < local; b0 += 64) {
        const int32_t pw = b0 + lane < local ? pages[b0 + lane] : 0;
        for (int b = b0; b < min(b0 + 64, local); ++b) {
          bool is_sure = false;
          for (int j = 0; j < n_in; ++j) is_sure |= __builtin_amdgcn_readlane(lid, j) == b;
          if (!is_sure) consider(b, __builtin_amdgcn_readlane(pw, b - b0));
        }
      }
    }
    // the row: sure ids (lanes < n_in) and the kept ones, ascending, then the
    // local block and -1 padding
    int mine = 0x7fffffff;
    if (lane < n_in) mine = lid;
#pragma unroll
    for (int j = 0; j < kSelCap; ++j)
      if (lane == n_in + j && j < need) mine = bi[j];
    int rank = 0;
    for (int j = 0; j < R; ++j) rank += __builtin_amdgcn_readlane(mine, j) < mine ? 1 : 0;
    int32_t* dst = a.sel + ((int64_t)r * a.P + p) * a.k;
    if (lane < R) dst[rank] = mine;
    if (lane == R) dst[R] = local;
    if (lane > R && lane < a.k) dst[lane] = -1;
  }
}

// One query row per sequence (the indexer pass of a decode step): the row
// tiles above would leave 511 of 512 rows idle, so this kernel streams each
// sequence's proxy-K blocks straight from global memory into MFMA A
// operands instead, and one MFMA serves every proxy head that shares the K
// head (keys are the MFMA rows, those heads its columns).  Grid: (block
// chunk, K head used, sequence); wave w of a workgroup takes the chunk's
// blocks w, w+4, ... (about one workgroup per CU, each wave streaming a long
// run of blocks, measured faster than more, shorter workgroups).  Output:
// block maxima in the max_score layout.
struct ProxyRowArgs {
  const uint8_t* pq;
  const uint8_t* pk;
  const float* qs;
  const float* ks;
  const int32_t* kv_indices;
  DevMeta m;
  int32_t P, Pk, nb_max, blocks_per_wg;
  int64_t row_begin, row_count;
  float* out;              // block maxima: out[head * o_h + block * o_b + row * o_r]
  int64_t o_h, o_b, o_r;   // [P, nb_max, row_count] for max_score, [row_count, P, nb_max] in the workspace
  int32_t* kmx;            // MXFP4 K, fused low-precision selection: largest scale code per block [row_count, Pk, nb_max]
  float scale;
};

constexpr int kRowWaves = 4;

template <Fmt F>
__global__ __launch_bounds__(64 * kRowWaves) void proxy_onerow_kernel(ProxyRowArgs a) {
  static_assert(F == Fmt::BF16 || F == Fmt::FP8, "MXFP4 K has its own kernel below");
  using Tr = ProxyTraits<F>;
  using Frag = typename Tr::AFrag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rl = blockIdx.z;              // row within the call's range
  const int seq = (int)(a.row_begin + rl);    // one row per sequence: row index = sequence index
  // blockIdx.y: the K head (P_k = P), or with one shared K head the group of
  // 32 proxy heads (MFMA columns) this workgroup serves
  const int kh = a.Pk == 1 ? 0 : (int)blockIdx.y;
  const int head0 = a.Pk == 1 ? 32 * (int)blockIdx.y : kh;
  const int32_t kv_len = a.m.kv[seq];
  const int nb = (kv_len + 127) >> 7;
  const int b0 = blockIdx.x * a.blocks_per_wg, b1 = min(nb, b0 + a.blocks_per_wg);
  if (b0 >= nb) return;
  const int ncols = a.Pk == 1 ? min(32, a.P - head0) : 1;  // query heads this K head serves here
  const int j = lane & 31, hsel = lane >> 5;
  const bool col_ok = j < ncols;
  const int head = head0 + (col_ok ? j : 0);
  // B operand: the served heads' proxy q rows (zero columns past ncols)
  Frag qf[Tr::kSteps];
  {
    const uint8_t* src = a.pq + ((int64_t)seq * a.P + head) * Tr::kQRowBytes;
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) {
      qf[st] = load_q_frag<F>(src, st, hsel);
      if (!col_ok) qf[st] = Frag{};
    }
  }
  float scale = a.scale;
  if constexpr (F == Fmt::FP8) scale *= a.qs[head] * a.ks[kh];
  const int32_t* pages = a.kv_indices + a.m.page_start[seq];
  // a key row in global memory has the q row's layout: same fragment loads
  auto load_tile = [&](Frag (&f)[Tr::kSteps], int32_t page, int t) {
    const uint8_t* src = a.pk + ((int64_t)page * a.Pk + kh) * Tr::kKBlockBytes + (32 * t + j) * Tr::kKRowBytes;
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) f[st] = load_q_frag<F>(src, st, hsel);
  };
  // Software pipeline over whole blocks: block b + 4's sixteen KB (fp8: 64
  // VGPRs per buffer) is in flight while block b is multiplied.
  int b = b0 + wave;
  if (b >= b1) return;
  Frag fa[4][Tr::kSteps], fb[4][Tr::kSteps];
#pragma unroll
  for (int t = 0; t < 4; ++t) load_tile(fa[t], pages[b], t);
  auto step = [&](Frag (&cur)[4][Tr::kSteps], Frag (&nxt)[4][Tr::kSteps], int b) {
    const int bn = min(b + kRowWaves, b1 - 1);  // past the chunk's end: reload its last block (unused)
    const int32_t pn = pages[bn];
#pragma unroll
    for (int t = 0; t < 4; ++t) load_tile(nxt[t], pn, t);
    float m = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) acc = mma<F>(cur[t][st], qf[st], acc, st, 0, 0);
      // C[i][j]: key 32t + 8(r/4) + 4 hsel + r%4 of register r; keys at or
      // past kv_len are page padding
      const int lim = kv_len - 1 - (b * 128 + 32 * t + 4 * hsel);
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = max3f(m, (8 * (r >> 2) + (r & 3)) <= lim ? acc[r] : kNegInf,
                  (8 * (r >> 2) + (r & 3) + 1) <= lim ? acc[r + 1] : kNegInf);
    }
    m = wave_max32(m);
    if (lane < ncols) a.out[head * a.o_h + b * a.o_b + rl * a.o_r] = m * scale;
  };
  for (; b + kRowWaves < b1; b += 2 * kRowWaves) {
    step(fa, fb, b);
    step(fb, fa, b + kRowWaves);
  }
  if (b < b1) step(fa, fb, b);
}

// MXFP4 proxy K, one query row per sequence.  A page record of one proxy-K
// head holds 128 key rows of E2M1 codes, then 128 rows of E8M0 scales (the
// MXFP4 record above).  The scaled f8f6f4 MFMA takes the codes as its FP4 A
// operand with each lane's own block scale, and the proxy q (fp8, or MXFP4
// with its own scales) as its B operand, so every product is exact; see
// load_q_frag for the lane layout.  Schedule as in the fp8/bf16 kernel
// above: whole blocks, the next one in flight.
struct MxTile {
  i32x4 c[2];  // MX blocks h and 2 + h of key j (k-steps 0 and 1)
  int32_t sc;  // the key's four scale bytes >> 8h
};

template <Fmt F>
__global__ __launch_bounds__(64 * kRowWaves) void proxy_onerow_mxfp4_kernel(ProxyRowArgs a) {
  static_assert(kMxK<F>, "MXFP4 K only");
  using Tr = ProxyTraits<F>;
  constexpr int kCodeBytes = 128 * Tr::kKRowBytes;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rl = blockIdx.z;
  const int seq = (int)(a.row_begin + rl);
  const int kh = a.Pk == 1 ? 0 : (int)blockIdx.y;
  const int head0 = a.Pk == 1 ? 32 * (int)blockIdx.y : kh;
  const int32_t kv_len = a.m.kv[seq];
  const int nb = (kv_len + 127) >> 7;
  const int b0 = blockIdx.x * a.blocks_per_wg, b1 = min(nb, b0 + a.blocks_per_wg);
  if (b0 >= nb) return;
  const int ncols = a.Pk == 1 ? min(32, a.P - head0) : 1;
  const int j = lane & 31, hsel = lane >> 5;
  const bool col_ok = j < ncols;
  const int head = head0 + (col_ok ? j : 0);
  typename Tr::BFrag qf[2];
  int32_t qsc = 0x7f7f7f7f;
  {
    const uint8_t* src = a.pq + ((int64_t)seq * a.P + head) * Tr::kQRowBytes;
#pragma unroll
    for (int st = 0; st < 2; ++st) qf[st] = col_ok ? load_q_frag<F>(src, st, hsel) : typename Tr::BFrag{};
    if constexpr (F == Fmt::MX4QK) {
      if (col_ok) qsc = (int32_t)(*reinterpret_cast<const uint32_t*>(src + 64) >> (8 * hsel));
    }
  }
  float scale = a.scale;
  if constexpr (F == Fmt::MX4K) scale *= a.qs[head];
  const int32_t* pages = a.kv_indices + a.m.page_start[seq];
  auto load_tile = [&](MxTile& f, int32_t page, int t) {
    const uint8_t* rec = a.pk + ((int64_t)page * a.Pk + kh) * Tr::kKBlockBytes;
    const int key = 32 * t + j;
    const uint8_t* cp = rec + key * Tr::kKRowBytes + hsel * 16;
    f.c[0] = *reinterpret_cast<const i32x4*>(cp);
    f.c[1] = *reinterpret_cast<const i32x4*>(cp + 32);
    f.sc = (int32_t)(*reinterpret_cast<const uint32_t*>(rec + kCodeBytes + key * 4) >> (8 * hsel));
  };
  int b = b0 + wave;
  if (b >= b1) return;
  MxTile fa[4], fb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) load_tile(fa[t], pages[b], t);
  auto step = [&](MxTile (&cur)[4], MxTile (&nxt)[4], int b) {
    const int bn = min(b + kRowWaves, b1 - 1);  // past the chunk's end: reload its last block (unused)
    const int32_t pn = pages[bn];
#pragma unroll
    for (int t = 0; t < 4; ++t) load_tile(nxt[t], pn, t);
    float m = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16 acc = f32x16{};
      acc = mma<F>(cur[t].c[0], qf[0], acc, 0, cur[t].sc, qsc);
      acc = mma<F>(cur[t].c[1], qf[1], acc, 1, cur[t].sc, qsc);
      const int lim = kv_len - 1 - (b * 128 + 32 * t + 4 * hsel);
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = max3f(m, (8 * (r >> 2) + (r & 3)) <= lim ? acc[r] : kNegInf,
                  (8 * (r >> 2) + (r & 3) + 1) <= lim ? acc[r + 1] : kNegInf);
    }
    m = wave_max32(m);
    if (lane < ncols) a.out[head * a.o_h + b * a.o_b + rl * a.o_r] = m * scale;
    if (a.kmx) {
      // the block's largest scale code (bounds its |k|); every key of the
      // block is in some lane's four tiles, bytes 0 and 2 of each shifted word
      uint32_t e = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) e = max(e, max((uint32_t)cur[t].sc & 0xffu, ((uint32_t)cur[t].sc >> 16) & 0xffu));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) e = max(e, (uint32_t)__shfl_xor((int)e, o));
      if (lane == 0) a.kmx[(rl * a.Pk + kh) * a.nb_max + b] = (int32_t)e;
    }
  };
  for (; b + kRowWaves < b1; b += 2 * kRowWaves) {
    step(fa, fb, b);
    step(fb, fa, b + kRowWaves);
  }
  if (b < b1) step(fa, fb, b);
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_proxy_maxscore(const msa_plan_s* p, const DevMeta& m, const void* pq, const void* pk,
                                 const float* qs, const float* ks, const int32_t* kv_indices, int32_t tile_lo,
                                 int32_t tile_hi, int64_t row_begin, int64_t row_count, float* max_score,
                                 int32_t* sel, const SelScratch& scr, hipStream_t st) {
  const bool lowp = p->d.proxy_dtype != MSA_BF16;
  if (p->one_row) {
    // indexer pass of a decode step: block maxima by the one-row kernel (into
    // the workspace when the selection is fused), then the top-k kernel
    ProxyRowArgs r;
    r.pq = static_cast<const uint8_t*>(pq);
    r.pk = static_cast<const uint8_t*>(pk);
    r.qs = qs;
    r.ks = ks;
    r.kv_indices = kv_indices;
    r.m = m;
    r.P = p->d.num_proxy_heads;
    r.Pk = p->d.num_proxy_kv_heads;
    r.nb_max = p->nb_max;
    r.row_begin = row_begin;
    r.row_count = row_count;
    r.out = sel ? scr.dms : max_score;
    // the wave-per-row selection reads its row's scores contiguously:
    // row-major in the workspace (low-precision one-row plans always qualify)
    const bool rm = sel && onerow_wave_topk(p);
    if (rm) {
      r.o_r = (int64_t)r.P * r.nb_max;
      r.o_h = r.nb_max;
      r.o_b = 1;
    } else {
      r.o_h = (int64_t)r.nb_max * row_count;
      r.o_b = row_count;
      r.o_r = 1;
    }
    r.kmx = sel && lowp ? scr.kmx : nullptr;
    r.scale = p->d.proxy_sm_scale;
    // grid.y: K heads, or with one shared K head groups of 32 proxy heads
    const int khs = r.Pk == 1 ? (r.P + 31) / 32 : r.P;
    // about one workgroup per CU over (sequence, K head, block chunk)
    const int64_t units = row_count * khs;
    const int64_t want = p->num_cu;
    r.blocks_per_wg = (int32_t)std::max<int64_t>(kRowWaves, (p->nb_max * units + want - 1) / want);
    const dim3 grid((unsigned)((p->nb_max + r.blocks_per_wg - 1) / r.blocks_per_wg), (unsigned)khs,
                    (unsigned)row_count);
    {
      ProfEvents pe(p, sel ? "proxy_topk" : "proxy_maxscore");
      const dim3 blk(64 * kRowWaves);
      switch (p->d.proxy_dtype) {
        case MSA_MXFP4_QK:
          hipExtLaunchKernelGGL(proxy_onerow_mxfp4_kernel<Fmt::MX4QK>, grid, blk, 0, st, pe.start, pe.stop, 0, r);
          break;
        case MSA_MXFP4:
          hipExtLaunchKernelGGL(proxy_onerow_mxfp4_kernel<Fmt::MX4K>, grid, blk, 0, st, pe.start, pe.stop, 0, r);
          break;
        case MSA_FP8_E4M3:
          hipExtLaunchKernelGGL(proxy_onerow_kernel<Fmt::FP8>, grid, blk, 0, st, pe.start, pe.stop, 0, r);
          break;
        default:
          hipExtLaunchKernelGGL(proxy_onerow_kernel<Fmt::BF16>, grid, blk, 0, st, pe.start, pe.stop, 0, r);
      }
    }
    if (sel && lowp)
      return launch_topk_exact(p, m, scr.dms, scr.kmx, pq, pk, qs, ks, kv_indices, row_begin, row_count, sel, st);
    if (sel) return launch_topk(p, m, scr.dms, rm, row_begin, row_count, sel, st);
    return hipGetLastError();
  }
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
  a.sel = sel;
  a.k = p->d.topk;
  a.scale = p->d.proxy_sm_scale;
  a.rq = scr.rq;
  a.rq_count = scr.rq_count;
  const bool refine = sel && lowp;
  if (refine) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, scr.rq_count, 1);
  const dim3 grid((unsigned)(a.ntiles * kProxySubs * a.P)), block(64 * kProxyWaves);
  {
    ProfEvents pe(p, sel ? "proxy_topk" : "proxy_maxscore");
    auto go = [&](auto kernel) { hipExtLaunchKernelGGL(kernel, grid, block, 0, st, pe.start, pe.stop, 0, a); };
    switch (p->d.proxy_dtype) {
      case MSA_MXFP4_QK: sel ? go(proxy_maxscore_kernel<Fmt::MX4QK, true>) : go(proxy_maxscore_kernel<Fmt::MX4QK, false>); break;
      case MSA_MXFP4: sel ? go(proxy_maxscore_kernel<Fmt::MX4K, true>) : go(proxy_maxscore_kernel<Fmt::MX4K, false>); break;
      case MSA_FP8_E4M3: sel ? go(proxy_maxscore_kernel<Fmt::FP8, true>) : go(proxy_maxscore_kernel<Fmt::FP8, false>); break;
      default: sel ? go(proxy_maxscore_kernel<Fmt::BF16, true>) : go(proxy_maxscore_kernel<Fmt::BF16, false>);
    }
  }
  if (refine) {
    // waves loop over the queued pairs; the queue length is read on the device
    ProfEvents pe(p, "topk_refine");
    const dim3 rg((unsigned)(3 * p->num_cu)), rb(256);  // three waves per SIMD fit its registers
    switch (p->d.proxy_dtype) {
      case MSA_MXFP4_QK: hipExtLaunchKernelGGL(topk_refine_kernel<Fmt::MX4QK>, rg, rb, 0, st, pe.start, pe.stop, 0, a); break;
      case MSA_MXFP4: hipExtLaunchKernelGGL(topk_refine_kernel<Fmt::MX4K>, rg, rb, 0, st, pe.start, pe.stop, 0, a); break;
      default: hipExtLaunchKernelGGL(topk_refine_kernel<Fmt::FP8>, rg, rb, 0, st, pe.start, pe.stop, 0, a);
    }
  }
  return hipGetLastError();
}

}  // namespace msa
