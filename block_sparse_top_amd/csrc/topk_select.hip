// Stage 2 of MSA: top-k block selection.
//
// `sparse_topk_select` of the MiniMax-AI/MSA README (section "Usage"): from
// the per-block max scores, keep `topk` KV blocks per (row, group), bounded
// by the row's visible blocks.  The local block is always kept (Flash-MSA
// article, paragraph on the forward kernels), so topk - 1 slots compete
// among the blocks before it; ties go to the lower block id; output ascending
// and -1 padded.  The README credits its indexer to a histogram step plus an
// insertion sort; the same two ideas appear here in a per-thread form.
//
// Design (gfx950), one thread per (row, group) (plans with one query row per
// sequence use the wave-per-row kernel further down):
//  * max_score is [P][nb_max][rows] (rows fastest), so at every block index
//    the 64 lanes of a wave read 64 consecutive floats: every load is one
//    coalesced 256-byte line;
//  * pass 1 folds the row into NG = 2*KS group maxima (block b -> group
//    b % NG).  The group maxima are distinct blocks, so their R-th largest
//    (R = topk-1 competing slots) is a lower bound tau of the row's R-th
//    largest score; found by a register insertion sort of the NG maxima;
//  * pass 2 compacts (score, id) of the blocks scoring >= tau (about 19 on
//    average for random scores, rarely above 34) into a per-thread LDS list,
//    in ascending block order;
//  * pass 3 runs a register insertion sort of those scores to find the exact
//    R-th value tau* and how many scores equal to it are taken, and pass 4
//    emits the chosen ids in ascending order (ties: lowest ids first).  If
//    the list overflows (heavy exact ties), passes 3-4 stream the row.
#include "device_common.hpp"
#include "msa_internal.hpp"
#include "proxy_exact.hpp"

namespace msa {
namespace {

constexpr int kTopkThreads = 128;
constexpr int kCap = 48;  // per-thread candidate list length

struct TopkArgs {
  const float* ms;          // [P, nb_max, row_count] (the wave kernels: ms[p * s_p + b * s_b + row * s_r])
  int32_t* sel;             // [T, Hkv, k]
  DevMeta m;
  int64_t row_begin, row_count;
  int64_t s_p, s_b, s_r;
  int32_t P, k;
};

// Insert v into the descending list top[0..KS).
template <int KS>
__device__ __forceinline__ void insert_desc(float (&top)[KS], float v) {
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const float hi = fmaxf(top[j], v);
    v = fminf(top[j], v);
    top[j] = hi;
  }
}

template <int KS>
__device__ __forceinline__ float pick(const float (&top)[KS], int i) {
  float r = top[0];
#pragma unroll
  for (int j = 1; j < KS; ++j) r = (j == i) ? top[j] : r;
  return r;
}

template <int KS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  constexpr int NG = 2 * KS;
  __shared__ float cval[kCap][kTopkThreads];
  __shared__ uint16_t cid[kCap][kTopkThreads];
  const int tid = threadIdx.x;
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * kTopkThreads + tid;
  if (i >= a.row_count) return;
  const int32_t r = (int32_t)(a.row_begin + i);
  const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
  const int32_t pos = a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s]);
  const int local = pos >> 7;
  const int k = a.k;
  const int R = min(k - 1, local);
  int32_t* out = a.sel + ((int64_t)r * a.P + p) * k;
  const float* col = a.ms + (int64_t)p * a.m.nb_max * a.row_count + i;
  const int64_t stride = a.row_count;

  if (R == local) {  // every visible block is selected
    for (int j = 0; j < k; ++j) out[j] = j <= local ? j : -1;
    return;
  }

  // pass 1: group maxima, then tau = R-th largest of them
  float gm[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) gm[j] = kNegInf;
  // loads use clamped addresses (always in bounds, issued back to back);
  // entries past the competing range are masked to -inf, never duplicated,
  // so that the group maxima stay maxima of disjoint sets
  for (int b0 = 0; b0 < local; b0 += NG) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int b = b0 + j;
      const float v = col[(int64_t)min(b, local - 1) * stride];
      gm[j] = fmaxf(gm[j], b < local ? v : kNegInf);
    }
  }
  float top[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) top[j] = kNegInf;
#pragma unroll
  for (int j = 0; j < NG; ++j) insert_desc<KS>(top, gm[j]);
  const float tau = pick<KS>(top, R - 1);

  // pass 2: compact candidates (score, id)
  int cnt = 0;
  for (int b0 = 0; b0 < local; b0 += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = col[(int64_t)min(b0 + j, local - 1) * stride];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (b0 + j < local && v[j] >= tau) {
        if (cnt < kCap) {
          cval[cnt][tid] = v[j];
          cid[cnt][tid] = (uint16_t)(b0 + j);
        }
        ++cnt;
      }
    }
  }
  const bool listed = cnt <= kCap;

  // pass 3: exact R-th value among the candidates
#pragma unroll
  for (int j = 0; j < KS; ++j) top[j] = kNegInf;
  if (listed) {
    for (int c = 0; c < cnt; ++c) insert_desc<KS>(top, cval[c][tid]);
  } else {
    for (int b = 0; b < local; ++b) {
      const float v = col[(int64_t)b * stride];
      if (v >= tau) insert_desc<KS>(top, v);
    }
  }
  const float tstar = pick<KS>(top, R - 1);
  int gt = 0;
#pragma unroll
  for (int j = 0; j < KS; ++j) gt += (j < R && top[j] > tstar) ? 1 : 0;
  int need_eq = R - gt;

  // pass 4: emit ascending ids
  int w = 0;
  const int n = listed ? cnt : local;
  for (int c = 0; c < n; ++c) {
    const float v = listed ? cval[c][tid] : col[(int64_t)c * stride];
    const int b = listed ? (int)cid[c][tid] : c;
    bool take = v > tstar;
    if (!take && v == tstar && need_eq > 0) {
      take = true;
      --need_eq;
    }
    if (take) out[w++] = b;
  }
  out[w++] = local;
  for (; w < k; ++w) out[w] = -1;
}


// Wave-uniform unsigned max: 16-lane row reductions by DPP (quad_perm xor 1,
// xor 2, then row_ror 4, 8), then the four row results read by readlane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x124>(v));
  v = max(v, dpp<0x128>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// The largest t such that at least n lanes have v >= t, i.e. the n-th largest
// v of the wave (n >= 1), built bit by bit from ballot counts.
__device__ __forceinline__ uint32_t wave_nth_largest(uint32_t v, int n) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    if (__popcll(__ballot(v >= c)) >= n) t = c;
  }
  return t;
}

// Plans with one query row per sequence (the indexer pass of a decode step:
// few rows, up to thousands of blocks each): one wave per (row, group), each
// lane holding VPL scores (block b at lane b % 64, register b / 64) as
// order-preserving unsigned keys (a larger score has a larger key, -0 counts
// as +0, key 0 marks a block outside the competing range).  With R =
// min(topk - 1, local) competing slots:
//  1. t = the R-th largest of the 64 lane maxima: at least R keys are >= t,
//     so every block of the top R has a key >= t;
//  2. if at most 64 keys are >= t, they are compacted (register by register,
//     lane by lane: ascending block id) to one per lane in LDS, tau = their
//     R-th largest key is found the same way, and the blocks with key > tau
//     plus the lowest-id ones with key == tau are written in lane order, so
//     ascending, followed by the local block and -1 padding;
//  3. otherwise (many equal scores) R rounds each take the wave's largest
//     key, find its lowest block by one ballot per register and retire it;
//     ids are then ordered by rank.
template <int VPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(TopkArgs a) {
  constexpr int kNone = 0x7fffffff;
  __shared__ uint32_t cand_key[4][64];
  __shared__ int32_t cand_id[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= a.row_count * a.P) return;
  const int64_t rl = pair / a.P;
  const int p = (int)(pair % a.P);
  const int32_t r = (int32_t)(a.row_begin + rl);  // = its sequence: one query row each
  const int local = __builtin_amdgcn_readfirstlane((a.m.kv[r] - 1) >> 7);
  const int R = min(a.k - 1, local);
  const float* col = a.ms + p * a.s_p + rl * a.s_r;
  uint32_t key[VPL];
  const int last = max(local - 1, 0);  // clamped loads: issued back to back, always in bounds
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int b = 64 * i + lane;
    const float x = col[min(b, last) * a.s_b];
    const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
    key[i] = b < local ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
  }
  int32_t* dst = a.sel + ((int64_t)r * a.P + p) * a.k;
  if (lane == 0) dst[R] = local;
  if (lane > R && lane < a.k) dst[lane] = -1;
  if (R == 0) return;

  uint32_t lm = key[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) lm = max(lm, key[i]);
  const uint32_t t = wave_nth_largest(lm, R);
  int total = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) total += __popcll(__ballot(key[i] >= t));

  if (total <= 64) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const bool c = key[i] >= t;
      const uint64_t m = __ballot(c);
      if (c) {
        const int pos = base + lanes_below(m);
        cand_key[wave][pos] = key[i];
        cand_id[wave][pos] = 64 * i + lane;
      }
      base += __popcll(m);
    }
    wave_lds_sync();
    const uint32_t ck = lane < total ? cand_key[wave][lane] : 0u;
    const int32_t cid = lane < total ? cand_id[wave][lane] : kNone;
    const uint32_t tau = wave_nth_largest(ck, R);
    const uint64_t gt = __ballot(ck > tau);
    uint64_t eq = __ballot(ck == tau && lane < total);
    uint64_t take = gt;
    for (int need = R - __popcll(gt); need > 0; --need) {  // the lowest-id ties
      const uint64_t low = eq & (~eq + 1);
      take |= low;
      eq ^= low;
    }
    if ((take >> lane) & 1) dst[lanes_below(take)] = cid;
    return;
  }

  int mine = kNone;  // lane j < R keeps round j's block
  for (int round = 0; round < R; ++round) {
    uint32_t km = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) km = max(km, key[i]);
    const uint32_t wm = wave_max_u32_uniform(km);
    int wb = kNone;
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i) {
      const uint64_t hit = __ballot(key[i] == wm);
      if (hit) wb = 64 * i + (int)__builtin_ctzll(hit);
    }
    if (lane == round) mine = wb;
    const bool own = lane == (wb & 63);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i == (wb >> 6) && own) key[i] = 0u;  // retire it
  }
  int rank = 0;
  for (int j = 0; j < R; ++j) rank += __builtin_amdgcn_readlane(mine, j) < mine ? 1 : 0;
  if (lane < R) dst[rank] = mine;
}

// Order-preserving key of a float (larger float, larger key; -0 as +0) and back.
__device__ __forceinline__ uint32_t f2key(float x) {
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct ExactRowArgs {
  const uint8_t* pq;
  const uint8_t* pk;
  const float* qs;
  const float* ks;
  const int32_t* kv_indices;
  const int32_t* kmx;  // MXFP4 K: largest scale code of each block [row_count, Pk, nb_max]
  int32_t Pk;
  float scale;
};

constexpr int kExWaves = 8;       // waves per (row, group): band blocks are re-scored in parallel
constexpr int kExBand = 2048;     // band scores held in LDS (one-row low-precision plans have <= 2048 blocks)

// The decode-step indexer's selection for the low-precision proxy formats
// (one query row per sequence, every block score of the row available in the
// workspace, row-major): one workgroup of kExWaves waves per (row, group);
// each wave reads the row (block b at lane b % 64, register b / 64, as
// order-preserving keys as in topk_wave_kernel) and takes the same branches.
//  * theta = the R-th largest score: the R-th largest lane maximum t0 is a
//    lower bound (R lanes hold a distinct score >= t0), the scores >= t0 are
//    compacted to one per lane when they fit, and theta is found bit by bit
//    from ballot counts over them (else over the whole row);
//  * delta = the format's score error bound for this row: blocks above
//    theta + 2 delta are in the exact top R, blocks below theta - 2 delta are
//    out; if exactly R blocks reach theta - 2 delta they are the answer;
//  * else the band blocks are scored exactly, band block c by wave c %
//    kExWaves (page ids loaded up front, lane-parallel), the scores
//    meet in LDS, and wave 0 keeps the best R - n_in in ascending block order
//    (a later block displaces a kept one only with a strictly larger score:
//    ties go to the lower block), the kept list distributed over the lanes.
template <int VPL, Fmt F>
__global__ __launch_bounds__(64 * kExWaves) void topk_wave_exact_kernel(TopkArgs a, ExactRowArgs x) {
  __shared__ int32_t sure_ids[64];
  __shared__ uint32_t top_keys[kExWaves][64];
  __shared__ float band_v[kExBand];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rl = blockIdx.x / a.P;
  const int p = (int)(blockIdx.x % a.P);
  const int32_t r = (int32_t)(a.row_begin + rl);  // = its sequence: one query row each
  const int local = __builtin_amdgcn_readfirstlane((a.m.kv[r] - 1) >> 7);
  const int R = min(a.k - 1, local);
  const int kh = x.Pk == a.P ? p : 0;
  int32_t* dst = a.sel + ((int64_t)r * a.P + p) * a.k;
  if (wave == 0) {
    if (lane == 0) dst[R] = local;
    if (lane > R && lane < a.k) dst[lane] = -1;
  }
  if (R == 0) return;
  if (R == local) {  // every competing block is selected
    if (wave == 0)
      for (int j = lane; j < R; j += 64) dst[j] = j;
    return;
  }
  // the row's scores (and scale codes) are loaded up to nb_max, all in
  // bounds, so the loads do not wait for the sequence length; the page ids of
  // the competing blocks are loaded next, while theta is found
  const float* row = a.ms + p * a.s_p + rl * a.s_r;  // s_b == 1
  const int nbm1 = a.m.nb_max - 1;
  uint32_t key[VPL];
  uint32_t kmaxe = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int b = 64 * i + lane;
    key[i] = f2key(row[min(b, nbm1)]);
    if constexpr (F != Fmt::FP8) {
      const uint32_t e = (uint32_t)x.kmx[(rl * x.Pk + kh) * a.m.nb_max + min(b, nbm1)];
      kmaxe = b < local ? max(kmaxe, e) : kmaxe;
    }
  }
  const int last = max(local - 1, 0);
  const int32_t* pages = x.kv_indices + a.m.page_start[r];
  int32_t pg[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    pg[i] = pages[min(64 * i + lane, last)];
    key[i] = 64 * i + lane < local ? key[i] : 0u;
  }
  // theta: the R-th largest key
  uint32_t lm = key[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) lm = max(lm, key[i]);
  const uint32_t t0 = wave_nth_largest(lm, R);
  int c0 = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) c0 += __popcll(__ballot(key[i] >= t0));
  uint32_t t = 0;
  if (c0 <= 64) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const bool c = key[i] >= t0;
      const uint64_t m = __ballot(c);
      if (c) top_keys[wave][base + lanes_below(m)] = key[i];
      base += __popcll(m);
    }
    wave_lds_sync();
    t = wave_nth_largest(lane < c0 ? top_keys[wave][lane] : 0u, R);
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) cnt += __popcll(__ballot(key[i] >= c));
      if (cnt >= R) t = c;
    }
  }
  const float theta = key2f(t);
  // delta: bound coefficient x scales x max|q| x max|k| (value units)
  const uint8_t* qrow = x.pq + ((int64_t)r * a.P + p) * (F == Fmt::MX4QK ? 68 : 128);
  float qinf;
  if constexpr (F == Fmt::MX4QK) {
    qinf = 6.0f * e8m0_value(max_byte4(*reinterpret_cast<const uint32_t*>(qrow + 64)));
  } else {
    const uint32_t w = lane < 32 ? *reinterpret_cast<const uint32_t*>(qrow + 4 * lane) : 0u;
    qinf = e4m3_absmax4(w);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) qinf = fmaxf(qinf, __shfl_xor(qinf, o));
  }
  float kinf = 448.0f;
  if constexpr (F != Fmt::FP8) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) kmaxe = max(kmaxe, (uint32_t)__shfl_xor((int)kmaxe, o));
    kinf = 6.0f * e8m0_value(kmaxe);
  }
  float sc = x.scale;
  if constexpr (F == Fmt::FP8) sc *= x.qs[p] * x.ks[kh];
  if constexpr (F == Fmt::MX4K) sc *= x.qs[p];
  const float delta = ScoreBound<F>::kCoef * 1.0001f * sc * qinf * kinf;
  const uint32_t lo = f2key(theta - 2.f * delta), hi = f2key(theta + 2.f * delta);
  int n_in = 0, nb = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    n_in += __popcll(__ballot(key[i] > hi));
    nb += __popcll(__ballot(key[i] >= lo && key[i] <= hi));
  }
  if (nb == R - n_in) {
    // certified: the R blocks reaching theta - 2 delta, ascending
    if (wave == 0) {
      int base = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const bool c = key[i] >= lo;
        const uint64_t m = __ballot(c);
        if (c) dst[base + lanes_below(m)] = 64 * i + lane;
        base += __popcll(m);
      }
    }
    return;
  }
  if (wave == 0) {
    // sure blocks, ascending, into LDS
    int base = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const bool c = key[i] > hi;
      const uint64_t m = __ballot(c);
      if (c) sure_ids[base + lanes_below(m)] = 64 * i + lane;
      base += __popcll(m);
    }
  }
  if (nb > wave) {
    // this wave's band blocks c = wave, wave + kExWaves, ...: exact scores
    const ExactQ q = exact_load_q<F>(qrow);
    int c = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      uint64_t m = __ballot(key[i] >= lo && key[i] <= hi);
      while (m) {
        const int l = (int)__builtin_ctzll(m);
        m &= m - 1;
        if (c % kExWaves == wave && c < kExBand) {
          const int32_t page = __builtin_amdgcn_readlane(pg[i], l);
          const uint8_t* blk = x.pk + ((int64_t)page * x.Pk + kh) * (F == Fmt::FP8 ? 128 * 128 : 128 * 68);
          const float v = exact_block_dotmax<F>(q, blk, 128) * sc;
          if (lane == 0) band_v[c] = v;
        }
        ++c;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int need = R - n_in;
  float kv_ = kNegInf;  // the kept list: slot `lane`
  int ki = 0x7fffffff;
  int c = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    uint64_t m = __ballot(key[i] >= lo && key[i] <= hi);
    while (m) {
      const int b = 64 * i + (int)__builtin_ctzll(m);
      m &= m - 1;
      const float v = band_v[min(c, kExBand - 1)];
      ++c;
      // insert before the first strictly smaller kept score
      const float up = __shfl_up(kv_, 1);
      const int upi = __shfl_up(ki, 1);
      const bool gj = lane < need && v > kv_;
      const bool gp = lane > 0 && v > up;
      if (gj) {
        kv_ = gp ? up : v;
        ki = gp ? upi : b;
      }
    }
  }
  // the row: sure ids and kept ids, ascending
  int mine = 0x7fffffff;
  if (lane < n_in) mine = sure_ids[lane];
  const int kept = __shfl(ki, max(lane - n_in, 0));
  if (lane >= n_in && lane < R) mine = kept;
  int rank = 0;
  for (int j = 0; j < R; ++j) rank += __builtin_amdgcn_readlane(mine, j) < mine ? 1 : 0;
  if (lane < R) dst[rank] = mine;
}

}  // namespace

hipError_t launch_topk_exact(const msa_plan_s* p, const DevMeta& m, const float* max_score, const int32_t* kmx,
                             const void* pq, const void* pk, const float* qs, const float* ks,
                             const int32_t* kv_indices, int64_t row_begin, int64_t row_count, int32_t* sel,
                             hipStream_t st) {
  TopkArgs a;
  a.ms = max_score;
  a.sel = sel;
  a.m = m;
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.P = p->d.num_proxy_heads;
  a.k = p->d.topk;
  ExactRowArgs x;
  x.pq = static_cast<const uint8_t*>(pq);
  x.pk = static_cast<const uint8_t*>(pk);
  x.qs = qs;
  x.ks = ks;
  x.kv_indices = kv_indices;
  x.kmx = kmx;
  x.Pk = p->d.num_proxy_kv_heads;
  x.scale = p->d.proxy_sm_scale;
  // row-major scores [row_count, P, nb_max]
  a.s_r = (int64_t)a.P * p->nb_max;
  a.s_p = p->nb_max;
  a.s_b = 1;
  const unsigned grid = (unsigned)(row_count * a.P);
  const int vpl = (p->nb_max + 63) / 64;
  ProfEvents pe(p, "topk_select");
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(64 * kExWaves), 0, st, pe.start, pe.stop, 0, a, x);
  };
#define MSA_EXACT_VPL(V)                                                               \
  switch (p->d.proxy_dtype) {                                                          \
    case MSA_FP8_E4M3: go(topk_wave_exact_kernel<V, Fmt::FP8>); break;                 \
    case MSA_MXFP4: go(topk_wave_exact_kernel<V, Fmt::MX4K>); break;                   \
    default: go(topk_wave_exact_kernel<V, Fmt::MX4QK>);                                \
  }
  if (vpl <= 4) { MSA_EXACT_VPL(4) }
  else if (vpl <= 8) { MSA_EXACT_VPL(8) }
  else if (vpl <= 16) { MSA_EXACT_VPL(16) }
  else { MSA_EXACT_VPL(32) }
#undef MSA_EXACT_VPL
  return hipGetLastError();
}

hipError_t launch_topk(const msa_plan_s* p, const DevMeta& m, const float* max_score, bool row_major,
                       int64_t row_begin, int64_t row_count, int32_t* sel, hipStream_t st) {
  TopkArgs a;
  a.ms = max_score;
  a.sel = sel;
  a.m = m;
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.P = p->d.num_proxy_heads;
  a.k = p->d.topk;
  if (row_major) {
    a.s_r = (int64_t)a.P * p->nb_max;
    a.s_p = p->nb_max;
    a.s_b = 1;
  } else {
    a.s_p = (int64_t)p->nb_max * row_count;
    a.s_b = row_count;
    a.s_r = 1;
  }
  if (onerow_wave_topk(p)) {
    // one wave per (row, group): these plans have few rows and long score rows
    const unsigned grid = (unsigned)((row_count * a.P + 3) / 4);
    const int vpl = (p->nb_max + 63) / 64;
    ProfEvents pe(p, "topk_select");
    if (vpl <= 4) hipExtLaunchKernelGGL(topk_wave_kernel<4>, dim3(grid), dim3(256), 0, st, pe.start, pe.stop, 0, a);
    else if (vpl <= 8) hipExtLaunchKernelGGL(topk_wave_kernel<8>, dim3(grid), dim3(256), 0, st, pe.start, pe.stop, 0, a);
    else if (vpl <= 16) hipExtLaunchKernelGGL(topk_wave_kernel<16>, dim3(grid), dim3(256), 0, st, pe.start, pe.stop, 0, a);
    else hipExtLaunchKernelGGL(topk_wave_kernel<32>, dim3(grid), dim3(256), 0, st, pe.start, pe.stop, 0, a);
    return hipGetLastError();
  }
  if (row_major) return hipErrorInvalidValue;  // the thread-per-row kernel reads max_score's layout
  const dim3 grid((unsigned)((row_count + kTopkThreads - 1) / kTopkThreads), (unsigned)a.P), block(kTopkThreads);
  const int need = a.k - 1;
  if (need <= 16) { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  else if (need <= 32) { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<32>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  else { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<64>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  return hipGetLastError();
}

}  // namespace msa
