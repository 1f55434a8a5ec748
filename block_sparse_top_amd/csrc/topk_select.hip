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

namespace msa {
namespace {

constexpr int kTopkThreads = 128;
constexpr int kCap = 48;  // per-thread candidate list length

struct TopkArgs {
  const float* ms;          // [P, nb_max, row_count]
  int32_t* sel;             // [T, Hkv, k]
  DevMeta m;
  int64_t row_begin, row_count;
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

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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
  const float* col = a.ms + (int64_t)p * a.m.nb_max * a.row_count + rl;
  uint32_t key[VPL];
  const int last = max(local - 1, 0);  // clamped loads: issued back to back, always in bounds
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int b = 64 * i + lane;
    const float x = col[(int64_t)min(b, last) * a.row_count];
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

}  // namespace

hipError_t launch_topk(const msa_plan_s* p, const DevMeta& m, const float* max_score, int64_t row_begin,
                       int64_t row_count, int32_t* sel, hipStream_t st) {
  TopkArgs a;
  a.ms = max_score;
  a.sel = sel;
  a.m = m;
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.P = p->d.num_proxy_heads;
  a.k = p->d.topk;
  if (p->one_row && p->nb_max <= 64 * 32 && a.k <= 64) {
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
  const dim3 grid((unsigned)((row_count + kTopkThreads - 1) / kTopkThreads), (unsigned)a.P), block(kTopkThreads);
  const int need = a.k - 1;
  if (need <= 16) { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  else if (need <= 32) { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<32>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  else { ProfEvents pe(p, "topk_select"); hipExtLaunchKernelGGL(topk_kernel<64>, grid, block, 0, st, pe.start, pe.stop, 0, a); }
  return hipGetLastError();
}

}  // namespace msa
