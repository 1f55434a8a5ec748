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
  float* out;                // [P, nb_max, row_count] (block max scores) or null
  int32_t* sel;              // [T, P, k] selections when fused with top-k, else null
  int32_t k;                 // slots per (row, group), local block included (fused path)
  float scale;
};

// Fused selection: each lane keeps its row's best kSelCap (score, block)
// pairs in descending score order.  Blocks arrive in ascending order and an
// equal score never displaces a listed one, so ties go to the lower block,
// exactly as in the separate top-k over the same fp32 scores.
constexpr int kSelCap = 16;

template <bool FP8>
struct ProxyTraits;

// K tiles live in LDS unpadded, with the 16-byte chunks of each row permuted
// (physical chunk = logical chunk ^ swz(row)) so that the 16 rows read by a
// fragment load hit 16 distinct bank groups.
template <>
struct ProxyTraits<false> {
  static constexpr int kElem = 2;             // bytes per element
  static constexpr int kRowBytes = 256;       // one key row
  static constexpr int kSteps = 8;            // MFMA k-steps over d = 128
  __device__ static int swz(int row) { return row & 15; }
  typedef bf16x8 Frag;
};
template <>
struct ProxyTraits<true> {
  static constexpr int kElem = 1;
  static constexpr int kRowBytes = 128;
  static constexpr int kSteps = 2;
  __device__ static int swz(int row) { return (row >> 1) & 7; }
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

// A fragment of key row `row`, logical 16-byte chunk `c` (and c+1 for fp8).
template <bool FP8>
__device__ __forceinline__ typename ProxyTraits<FP8>::Frag load_frag_lds(const uint8_t* tile, int row, int c) {
  using Tr = ProxyTraits<FP8>;
  const uint8_t* base = tile + row * Tr::kRowBytes;
  if constexpr (FP8) {
    i32x4 a = lds_load16<i32x4>(base + ((c ^ Tr::swz(row)) << 4));
    i32x4 b = lds_load16<i32x4>(base + (((c + 1) ^ Tr::swz(row)) << 4));
    i32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
  } else {
    return lds_load16<bf16x8>(base + ((c ^ Tr::swz(row)) << 4));
  }
}

template <bool FP8>
__device__ __forceinline__ f32x16 mma(const typename ProxyTraits<FP8>::Frag& a,
                                      const typename ProxyTraits<FP8>::Frag& b, const f32x16& c) {
  if constexpr (FP8) return mfma32x32x64_fp8(a, b, c);
  else return mfma32x32x16(a, b, c);
}

constexpr int kProxyWaves = 8;

template <bool FP8, bool TOPK>
__global__ __launch_bounds__(64 * kProxyWaves) void proxy_maxscore_kernel(ProxyArgs a) {
  using Tr = ProxyTraits<FP8>;
  using Frag = typename Tr::Frag;
  constexpr int kBlockBytes = 128 * Tr::kRowBytes;        // one K block in global memory
  constexpr int kLoads = kBlockBytes / 1024 / kProxyWaves;  // 1 KB direct-to-LDS loads per wave
  constexpr int kChunksPerRow = Tr::kRowBytes / 16;
  constexpr int kRowsPerKB = 1024 / Tr::kRowBytes;
  constexpr int kStepBytes = Tr::kRowBytes / Tr::kSteps;  // bytes of d per MFMA k-step
  // two distinct tile objects (not one array indexed by a runtime buffer
  // number): the loads in flight into one are then provably disjoint from
  // the reads of the other
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kBlockBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kBlockBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave branches stay scalar
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

  // K block -> LDS without registers: each wave issues kLoads direct 1 KB
  // loads (global_load_lds_dwordx4: lane i fills bytes 16i..16i+15 of the
  // KB), fetching for each lane the global chunk its swizzled slot holds.
  auto kload = [&](int32_t page, uint8_t* tile) {
    const uint8_t* src = a.pk + ((int64_t)page * a.Pk + ph) * kBlockBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int kb = wave + kProxyWaves * i;             // which KB of the tile
      const int row = kb * kRowsPerKB + lane / kChunksPerRow;
      const int pc = lane % kChunksPerRow;               // physical chunk written by this lane
      const int lc = pc ^ Tr::swz(row);                  // logical chunk it must hold
      global_load_lds16(src + row * Tr::kRowBytes + lc * 16, (MSA_LDS void*)(tile + kb * 1024));
    }
  };

  float scale = a.scale;
  if constexpr (FP8) scale *= a.qs[p] * a.ks[ph];
  const bool wave_active = 64 * wave < nrows;
  const int my_row = 64 * wave + lane;          // row this lane writes
  const int64_t my_grow = row0 + my_row;
  const bool writes = my_row < nrows && my_grow >= a.row_begin && my_grow < a.row_end;
  float* outp = a.out + (int64_t)p * a.nb_max * a.row_count + (my_grow - a.row_begin);

  const int my_local = (pos0 + my_row) >> 7;   // this lane's row's local block
  float tv[TOPK ? kSelCap : 1];
  int ti[TOPK ? kSelCap : 1];
#pragma unroll
  for (int j = 0; j < (TOPK ? kSelCap : 1); ++j) {
    tv[j] = kNegInf;
    ti[j] = -1;
  }
  const int chunk0 = ((lane >> 5) * (kStepBytes / 2)) >> 4;

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
  auto ins_steps = [&](int r) {  // slots 15 - 4r down to 12 - 4r
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = kSelCap - 1 - (4 * r + jj);
      const bool gj = cv > tv[j];
      const bool gp = j > 0 ? cv > tv[j > 0 ? j - 1 : 0] : false;
      const float up = j > 0 ? tv[j > 0 ? j - 1 : 0] : kPosInf;
      const int upi = j > 0 ? ti[j > 0 ? j - 1 : 0] : 0;
      ti[j] = gj ? (gp ? upi : ci) : ti[j];
      tv[j] = __builtin_amdgcn_fmed3f(up, cv, tv[j]);
    }
  };

  auto block_max = [&](const uint8_t* tile, int b, float (&m)[2]) {
    m[0] = m[1] = kNegInf;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 acc[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = f32x16{};
      Frag fr[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) fr[0][j] = load_frag_lds<FP8>(tile, 32 * (2 * hf + j) + (lane & 31), chunk0);
#pragma unroll
      for (int st = 0; st < Tr::kSteps; ++st) {
        if (st + 1 < Tr::kSteps) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            fr[(st + 1) & 1][j] = load_frag_lds<FP8>(tile, 32 * (2 * hf + j) + (lane & 31),
                                                     chunk0 + (((st + 1) * kStepBytes) >> 4));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j][0] = mma<FP8>(fr[st & 1][j], qf[0][st], acc[j][0]);
          acc[j][1] = mma<FP8>(fr[st & 1][j], qf[1][st], acc[j][1]);
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
    m[0] = fmaxf(m[0], wave_xor32(m[0]));
    m[1] = fmaxf(m[1], wave_xor32(m[1]));
    const float v = (lane < 32 ? m[0] : m[1]) * scale;
    if constexpr (TOPK) {
      // blocks before the local one compete (the local block is forced);
      // inserted during the next block
      pend_v = v;
      pend_b = b;
      pend_ok = b < my_local;
      ins_begin();
#pragma unroll
      for (int r = 0; r < kSelCap / 4; ++r) ins_steps(r);
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

  // block loop unrolled by two over the two tiles: block b computes from one
  // tile while block b+1 streams into the other; pairs run unconditionally
  // and an odd last block follows the loop (no branch inside the loop body
  // that the per-row selection state has to flow through)
  auto step = [&](int b, const uint8_t* tile, uint8_t* next_tile) __attribute__((always_inline)) {
    advance(b);
    if (b + 1 <= b_last) kload(page_of(b + 1), next_tile);
    float m[2];
    if (wave_active) {
      block_max(tile, b, m);
      finish(b, m);
    }
    wait_all_mem();
    __syncthreads();
  };
  kload(page_of(0), lds0);
  wait_all_mem();
  __syncthreads();
  int b = 0;
  for (; b + 1 <= b_last; b += 2) {
    step(b, lds0, lds1);
    step(b + 1, lds1, lds0);
  }
  if (b <= b_last) step(b, lds0, lds1);

  if constexpr (TOPK) {
    // the R = min(k - 1, local) best earlier blocks and the local block, ascending, -1 padded
    if (writes) {
      const int R = min(a.k - 1, my_local);
#pragma unroll
      for (int j = 0; j < kSelCap; ++j)
        if (j >= R) ti[j] = 0x7fffffff;
#pragma unroll
      for (int rnd = 0; rnd < kSelCap; ++rnd)  // odd-even transposition sort by block id
#pragma unroll
        for (int j = rnd & 1; j + 1 < kSelCap; j += 2) {
          const int x = ti[j], y = ti[j + 1];
          ti[j] = min(x, y);
          ti[j + 1] = max(x, y);
        }
      int32_t* dst = a.sel + ((int64_t)my_grow * a.P + p) * a.k;
#pragma unroll
      for (int j = 0; j <= kSelCap; ++j) {
        if (j >= a.k) break;
        const int v = j < R ? ti[j < kSelCap ? j : 0] : (j == R ? my_local : -1);
        dst[j] = v;
      }
    }
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
  float* out;  // [P, nb_max, row_count]
  float scale;
};

constexpr int kRowWaves = 4;

template <bool FP8>
__global__ __launch_bounds__(64 * kRowWaves) void proxy_onerow_kernel(ProxyRowArgs a) {
  using Tr = ProxyTraits<FP8>;
  using Frag = typename Tr::Frag;
  constexpr int kStepBytes = Tr::kRowBytes / Tr::kSteps;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rl = blockIdx.z;              // row within the call's range
  const int seq = (int)(a.row_begin + rl);    // one row per sequence: row index = sequence index
  const int kh = blockIdx.y;                  // K head
  const int32_t kv_len = a.m.kv[seq];
  const int nb = (kv_len + 127) >> 7;
  const int b0 = blockIdx.x * a.blocks_per_wg, b1 = min(nb, b0 + a.blocks_per_wg);
  if (b0 >= nb) return;
  const int ncols = a.Pk == 1 ? a.P : 1;      // query heads this K head serves
  const int j = lane & 31, hsel = lane >> 5;
  const bool col_ok = j < ncols;
  const int head = a.Pk == 1 ? (col_ok ? j : 0) : kh;
  // B operand: the served heads' proxy q rows (zero columns past ncols)
  Frag qf[Tr::kSteps];
  {
    const uint8_t* src = a.pq + ((int64_t)seq * a.P + head) * (128 * Tr::kElem) + hsel * (kStepBytes / 2);
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) {
      qf[st] = load_frag_global<FP8>(src + st * kStepBytes);
      if (!col_ok) qf[st] = Frag{};
    }
  }
  float scale = a.scale;
  if constexpr (FP8) scale *= a.qs[head] * a.ks[kh];
  const int32_t* pages = a.kv_indices + a.m.page_start[seq];
  auto load_tile = [&](Frag (&f)[Tr::kSteps], int32_t page, int t) {
    const uint8_t* src = a.pk + ((int64_t)page * a.Pk + kh) * (128 * Tr::kRowBytes) + (32 * t + j) * Tr::kRowBytes +
                         hsel * (kStepBytes / 2);
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) f[st] = load_frag_global<FP8>(src + st * kStepBytes);
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
      for (int st = 0; st < Tr::kSteps; ++st) acc = mma<FP8>(cur[t][st], qf[st], acc);
      // C[i][j]: key 32t + 8(r/4) + 4 hsel + r%4 of register r; keys at or
      // past kv_len are page padding
      const int lim = kv_len - 1 - (b * 128 + 32 * t + 4 * hsel);
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = max3f(m, (8 * (r >> 2) + (r & 3)) <= lim ? acc[r] : kNegInf,
                  (8 * (r >> 2) + (r & 3) + 1) <= lim ? acc[r + 1] : kNegInf);
    }
    m = fmaxf(m, wave_xor32(m));
    if (lane < ncols) a.out[((int64_t)head * a.nb_max + b) * a.row_count + rl] = m * scale;
  };
  for (; b + kRowWaves < b1; b += 2 * kRowWaves) {
    step(fa, fb, b);
    step(fb, fa, b + kRowWaves);
  }
  if (b < b1) step(fa, fb, b);
}

// MXFP4 proxy K, one query row per sequence.  A page record of one proxy-K
// head holds 128 key rows of E2M1 codes (64 B each, element 2i in the low
// nibble of byte i), then 128 rows of E8M0 scales (4 B each, byte c scaling
// dims 32c..32c+31).  The scaled f8f6f4 MFMA takes the codes as its FP4 A
// operand and the fp8 proxy q as its B operand (unit scale), so every product
// is exact.  FP4 A layout of v_mfma_scale_f32_32x32x64_f8f6f4 (probed): lane
// (row i, half h) holds 32 codes, codes 0-15 at k = 16h..16h+15 and codes
// 16-31 at k = 32+16h..47+16h, and its own scale byte (picked by op_sel)
// scales all 32.  So a lane takes one whole MX block: at k-step st, lane
// (key j, h) holds block 2st + h (the 16 code bytes at 32st + 16h of the key
// row) with that block's scale byte (the key's scale word shifted right by
// 8h, op_sel 2st), and the q fragment of lane (column, h') pairs with it:
// dims 64st + 16h' .. +15 then 64st + 32 + 16h' .. +15.  Schedule as in the
// fp8/bf16 kernel above: whole blocks, the next one in flight.
constexpr int kMxRowCodeBytes = 64;                          // 128 dims x 4 bits
constexpr int kMxRecordBytes = 128 * kMxRowCodeBytes + 128 * 4;

struct MxTile {
  i32x4 c[2];  // MX blocks h and 2 + h of key j (k-steps 0 and 1)
  int32_t sc;  // the key's four scale bytes >> 8h
};

template <int ST>
__device__ __forceinline__ f32x16 mma_fp4_fp8(const i32x4& a, const i32x8& b, int32_t sa, const f32x16& c) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  // format codes: A = 4 (E2M1), B = 0 (E4M3); A's scale is byte 2 ST of sa, B's 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 2 * ST, sa, 0, 127);
}

__global__ __launch_bounds__(64 * kRowWaves) void proxy_onerow_mxfp4_kernel(ProxyRowArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rl = blockIdx.z;
  const int seq = (int)(a.row_begin + rl);
  const int kh = blockIdx.y;
  const int32_t kv_len = a.m.kv[seq];
  const int nb = (kv_len + 127) >> 7;
  const int b0 = blockIdx.x * a.blocks_per_wg, b1 = min(nb, b0 + a.blocks_per_wg);
  if (b0 >= nb) return;
  const int ncols = a.Pk == 1 ? a.P : 1;
  const int j = lane & 31, hsel = lane >> 5;
  const bool col_ok = j < ncols;
  const int head = a.Pk == 1 ? (col_ok ? j : 0) : kh;
  i32x8 qf[2];
  {
    const uint8_t* src = a.pq + ((int64_t)seq * a.P + head) * 128 + hsel * 16;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const i32x4 x = *reinterpret_cast<const i32x4*>(src + 64 * st);
      const i32x4 y = *reinterpret_cast<const i32x4*>(src + 64 * st + 32);
      qf[st] = col_ok ? i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]} : i32x8{};
    }
  }
  const float scale = a.scale * a.qs[head];
  const int32_t* pages = a.kv_indices + a.m.page_start[seq];
  auto load_tile = [&](MxTile& f, int32_t page, int t) {
    const uint8_t* rec = a.pk + ((int64_t)page * a.Pk + kh) * kMxRecordBytes;
    const int key = 32 * t + j;
    const uint8_t* cp = rec + key * kMxRowCodeBytes + hsel * 16;
    f.c[0] = *reinterpret_cast<const i32x4*>(cp);
    f.c[1] = *reinterpret_cast<const i32x4*>(cp + 32);
    f.sc = (int32_t)(*reinterpret_cast<const uint32_t*>(rec + 128 * kMxRowCodeBytes + key * 4) >> (8 * hsel));
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
      acc = mma_fp4_fp8<0>(cur[t].c[0], qf[0], cur[t].sc, acc);
      acc = mma_fp4_fp8<1>(cur[t].c[1], qf[1], cur[t].sc, acc);
      const int lim = kv_len - 1 - (b * 128 + 32 * t + 4 * hsel);
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = max3f(m, (8 * (r >> 2) + (r & 3)) <= lim ? acc[r] : kNegInf,
                  (8 * (r >> 2) + (r & 3) + 1) <= lim ? acc[r + 1] : kNegInf);
    }
    m = fmaxf(m, wave_xor32(m));
    if (lane < ncols) a.out[((int64_t)head * a.nb_max + b) * a.row_count + rl] = m * scale;
  };
  for (; b + kRowWaves < b1; b += 2 * kRowWaves) {
    step(fa, fb, b);
    step(fb, fa, b + kRowWaves);
  }
  if (b < b1) step(fa, fb, b);
}

}  // namespace

hipError_t launch_proxy_maxscore(const msa_plan_s* p, const DevMeta& m, const void* pq, const void* pk,
                                 const float* qs, const float* ks, const int32_t* kv_indices, int32_t tile_lo,
                                 int32_t tile_hi, int64_t row_begin, int64_t row_count, float* max_score,
                                 int32_t* sel, float* scratch, hipStream_t st) {
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
    r.out = sel ? scratch : max_score;
    r.scale = p->d.proxy_sm_scale;
    const int khs = r.Pk == 1 ? 1 : r.P;
    // about one workgroup per CU over (sequence, K head, block chunk)
    const int64_t units = row_count * khs;
    const int64_t want = p->num_cu;
    r.blocks_per_wg = (int32_t)std::max<int64_t>(kRowWaves, (p->nb_max * units + want - 1) / want);
    const dim3 grid((unsigned)((p->nb_max + r.blocks_per_wg - 1) / r.blocks_per_wg), (unsigned)khs,
                    (unsigned)row_count);
    {
      ProfEvents pe(p, sel ? "proxy_topk" : "proxy_maxscore");
      if (p->d.proxy_dtype == MSA_MXFP4)
        hipExtLaunchKernelGGL(proxy_onerow_mxfp4_kernel, grid, dim3(64 * kRowWaves), 0, st, pe.start, pe.stop, 0, r);
      else if (p->d.proxy_dtype == MSA_FP8_E4M3)
        hipExtLaunchKernelGGL(proxy_onerow_kernel<true>, grid, dim3(64 * kRowWaves), 0, st, pe.start, pe.stop, 0, r);
      else
        hipExtLaunchKernelGGL(proxy_onerow_kernel<false>, grid, dim3(64 * kRowWaves), 0, st, pe.start, pe.stop, 0, r);
    }
    if (sel) return launch_topk(p, m, scratch, row_begin, row_count, sel, st);
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
  const dim3 grid((unsigned)(a.ntiles * a.P)), block(64 * kProxyWaves);
  const bool fp8 = p->d.proxy_dtype == MSA_FP8_E4M3;
  if (sel) {
    ProfEvents pe(p, "proxy_topk");
    if (fp8) hipExtLaunchKernelGGL((proxy_maxscore_kernel<true, true>), grid, block, 0, st, pe.start, pe.stop, 0, a);
    else hipExtLaunchKernelGGL((proxy_maxscore_kernel<false, true>), grid, block, 0, st, pe.start, pe.stop, 0, a);
  } else {
    ProfEvents pe(p, "proxy_maxscore");
    if (fp8) hipExtLaunchKernelGGL((proxy_maxscore_kernel<true, false>), grid, block, 0, st, pe.start, pe.stop, 0, a);
    else hipExtLaunchKernelGGL((proxy_maxscore_kernel<false, false>), grid, block, 0, st, pe.start, pe.stop, 0, a);
  }
  return hipGetLastError();
}

}  // namespace msa
