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
// Design (gfx950), one thread per (row, group):
//  * max_score is [P][nb_max][rows] (rows fastest), so at every block index
//    the 64 lanes of a wave read 64 consecutive floats: every load is one
//    coalesced 256-byte line;
//  * pass 1 folds the row into NG group maxima (block b -> group b % NG,
//    NG >= topk-1).  Their minimum tau is a lower bound of the (topk-1)-th
//    largest score, because the NG maxima are distinct blocks;
//  * pass 2 compacts the ids of blocks scoring >= tau (typically 30-60) into
//    a per-thread LDS list, in ascending block order;
//  * pass 3 runs a register insertion sort of those scores to find the exact
//    (topk-1)-th value tau* and how many scores equal to it are taken, and
//    pass 4 emits the chosen ids in ascending order (ties: lowest ids first).
//    If the list overflows (heavy ties), passes 3-4 stream the row instead.
#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int kTopkThreads = 256;
constexpr int kCap = 96;  // per-thread candidate list length

struct TopkArgs {
  const float* ms;          // [P, nb_max, row_count]
  int32_t* sel;             // [T, Hkv, k]
  DevMeta m;
  int64_t row_begin, row_count;
  int32_t P, k;
};

template <int NG>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint16_t cand[kCap][kTopkThreads];
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

  // pass 1: group maxima
  float gm[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) gm[j] = kNegInf;
  for (int b0 = 0; b0 < local; b0 += NG) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int b = b0 + j;
      if (b < local) gm[j] = fmaxf(gm[j], col[(int64_t)b * stride]);
    }
  }
  float tau = gm[0];
#pragma unroll
  for (int j = 1; j < NG; ++j) tau = fminf(tau, gm[j]);

  // pass 2: compact candidate ids
  int cnt = 0;
  for (int b = 0; b < local; ++b) {
    const float v = col[(int64_t)b * stride];
    if (v >= tau) {
      if (cnt < kCap) cand[cnt][tid] = (uint16_t)b;
      ++cnt;
    }
  }
  const bool listed = cnt <= kCap;
  const int n = listed ? cnt : local;

  // pass 3: insertion sort of the candidate scores (descending, NG slots)
  float top[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) top[j] = kNegInf;
  for (int c = 0; c < n; ++c) {
    const int b = listed ? (int)cand[c][tid] : c;
    float v = col[(int64_t)b * stride];
    if (!listed && v < tau) continue;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float hi = fmaxf(top[j], v);
      v = fminf(top[j], v);
      top[j] = hi;
    }
  }
  float tstar = top[0];
  int gt = 0;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    if (j == R - 1) tstar = top[j];
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) gt += (j < R && top[j] > tstar) ? 1 : 0;
  int need_eq = R - gt;

  // pass 4: emit ascending ids
  int w = 0;
  for (int c = 0; c < n; ++c) {
    const int b = listed ? (int)cand[c][tid] : c;
    const float v = col[(int64_t)b * stride];
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
  const dim3 grid((unsigned)((row_count + kTopkThreads - 1) / kTopkThreads), (unsigned)a.P), block(kTopkThreads);
  const int need = a.k - 1;
  if (need <= 16) hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, a);
  else if (need <= 32) hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(topk_kernel<64>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace msa
