// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "msa.h"

namespace msa {

// Device view of the plan's metadata (lives at the start of the workspace).
struct DevMeta {
  const int32_t* qo;          // [S]
  const int32_t* kv;          // [S]
  const int32_t* row_start;   // [S+1]
  const int32_t* page_start;  // [S+1]
  const int32_t* tiles;       // [ntiles][4] = seq, first row, rows, first position
  int32_t S, T, NB, nb_max;
};

// Optional event bracketing of one named internal kernel (msa_profile_kernel).
struct Profiler {
  std::string kernel;                                   // empty = off
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  std::vector<hipEvent_t> pool;
};

struct PlanLayout {
  size_t meta = 0, meta_bytes = 0;
  // prefill window scratch
  size_t counts = 0, cursor = 0, offsets = 0, items = 0, nitems = 0, gitems = 0, entries = 0, part_o = 0, bwd_d = 0;
  // per-(token, group, slot) partials of the proxy distillation term (plans
  // with one bf16 proxy head and proxy-K head per KV group), and the fused
  // key-side backward's even-chunk dK / dV partials (128 KB per (group, block))
  size_t kl_part = 0, kl_stash = 0;
  int64_t max_items = 0;
  // decode split scratch
  size_t dec_o = 0, dec_ml = 0;
  // block scores of the fused selection on one-query-row plans (and, MXFP4
  // K, each block's largest scale code)
  size_t dms = 0, kmx = 0;
  // low-precision proxies: queue of (row, group) pairs re-scored exactly
  size_t rq = 0, rq_count = 0;
  size_t total = 0;
};

}  // namespace msa

struct msa_plan_s {
  msa_plan_desc_t d;                 // copy; host pointers cleared
  std::vector<int32_t> qo, kv, nb, row_start, page_start;
  int32_t S = 0, T = 0, NB = 0, nb_max = 0, G = 0;
  int64_t max_rows = 0;              // rows per proxy/top-k call
  int64_t attn_window = 0;           // rows per prefill attention window
  std::vector<int32_t> tiles;        // proxy row tiles (seq, row0, nrows, pos0)
  int32_t ntiles = 0;
  std::vector<int32_t> meta;         // uploaded blob
  msa::PlanLayout lay;
  // prefill attention schedule
  int32_t tokens_per_chunk = 0;      // 128 / G query tokens per 128-row chunk
  int32_t entries_per_item = 0;      // tokens per work item
  // decode schedule
  int32_t dec_splits = 1;
  bool one_row = false;              // prefill plan whose every sequence has one query row
  bool xcd_pin = false;              // prefill attention: a KV group's work items stay on one XCD
  int32_t num_cu = 256;              // compute units of the device the plan was made on
  uint64_t uid = 0;                  // serial number (workspace records name plans by it)
  mutable msa::Profiler prof;
};

namespace msa {

DevMeta dev_meta(const msa_plan_s* p, const void* workspace);

// Start/stop events for one stage when the plan profiles `name` (both null
// otherwise).  They are handed to hipExtLaunchKernelGGL, which stamps them
// with the dispatch's own begin and end: `start` on a stage's first kernel,
// `stop` on its last.
struct ProfEvents {
  ProfEvents(const msa_plan_s* p, const char* name);
  hipEvent_t start = nullptr, stop = nullptr;
};

// Workspace areas of the fused selection (msa_proxy_topk_select).
struct SelScratch {
  float* dms = nullptr;        // one-query-row plans: block scores [P, nb_max, rows]
  int32_t* kmx = nullptr;      // one-query-row plans, MXFP4 K: largest scale code per block
  int32_t* rq = nullptr;       // low-precision proxies: queue of pairs to re-score exactly
  int32_t* rq_count = nullptr;
};

// Kernel launchers (defined in the .hip files).  They assume validated inputs.
hipError_t launch_proxy_maxscore(const msa_plan_s* p, const DevMeta& m, const void* pq, const void* pk,
                                 const float* qs, const float* ks, const int32_t* kv_indices, int32_t tile_lo,
                                 int32_t tile_hi, int64_t row_begin, int64_t row_count, float* max_score,
                                 int32_t* sel, const SelScratch& scr, hipStream_t st);
// Sparse prefill partial records: padding rows of a work item write to one
// of this many trash records (by workgroup) after the window's records.  The
// region holds, per record, the larger of the forward's record (4 planes of
// 32 bytes, one of 16 and 8 of {lse, step}: 152) and the backward's dQ partial record
// (5 planes and a 4-byte step: 164).
constexpr int64_t kTrashRecords = 256;
constexpr int64_t kPartRecordBytes = 168;
// One-query-row plans whose rows fit the wave-per-row top-k kernels (at most
// 32 registers of 64 block scores per lane, topk - 1 kept ids in the lanes).
inline bool onerow_wave_topk(const msa_plan_s* p) { return p->one_row && p->nb_max <= 64 * 32 && p->d.topk <= 64; }
// `row_major`: scores laid out [row_count, P, nb_max] (the workspace copy of
// a one-query-row plan's fused selection) instead of max_score's [P, nb_max,
// row_count].
hipError_t launch_topk(const msa_plan_s* p, const DevMeta& m, const float* max_score, bool row_major,
                       int64_t row_begin, int64_t row_count, int32_t* sel, hipStream_t st);
// Exact selection of one-query-row plans with low-precision proxies (band
// blocks re-scored from the proxy operands); scores and scale codes row-major.
hipError_t launch_topk_exact(const msa_plan_s* p, const DevMeta& m, const float* max_score, const int32_t* kmx,
                             const void* pq, const void* pk, const float* qs, const float* ks,
                             const int32_t* kv_indices, int64_t row_begin, int64_t row_count, int32_t* sel,
                             hipStream_t st);
hipError_t launch_prefill_window(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp,
                                 const void* vp, const float* ks, const float* vs, const int32_t* kv_indices,
                                 const int32_t* sel, void* out, float* lse, char* ws, int32_t w0, int32_t w1,
                                 hipStream_t st);
// Proxy distillation operands of the fused backward (bf16 proxy q [T, Hkv,
// 128] and proxy K pool, fp32 gradients); null in the main-only backward.
struct KlOperands {
  const void* pq;
  const void* pkp;
  float* dpq;      // [T, Hkv, 128]
  float* dpk;      // [N, Hkv, 128, 128]
  float* plse;     // [T, Hkv] proxy log-sum-exp (natural log), written
  float proxy_scale, grad_scale;
};
hipError_t launch_prefill_backward_window(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp,
                                          const void* vp, const int32_t* kv_indices, const int32_t* sel,
                                          const void* out, const float* lse, const void* dout, float* dq, float* dk,
                                          float* dv, const KlOperands* kl, char* ws, int32_t w0, int32_t w1,
                                          bool first_window, hipStream_t st);
// Dense causal attention (the warm-up mode): forward; the backward's dq (and
// the proxy term's dense p_main part into kl->dpq) and dk, dv (and into
// kl->dpk); D = <dout, out> for rows [w0, w1) into D[0 ..).
hipError_t launch_dense_forward(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                                const int32_t* kv_indices, void* out, float* lse, hipStream_t st);
hipError_t launch_dense_dq(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                           const int32_t* kv_indices, const float* lse, const float* D, const void* dout, float* dq,
                           const KlOperands* kl, hipStream_t st);
hipError_t launch_dense_dkv(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                            const int32_t* kv_indices, const float* lse, const float* D, const void* dout, float* dk,
                            float* dv, const KlOperands* kl, char* ws, hipStream_t st);
hipError_t launch_bwd_prep(const msa_plan_s* p, const void* out, const void* dout, float* D, int32_t w0, int32_t w1,
                           hipStream_t st);
// The dense proxy part of the distillation gradient, after every window of
// the fused backward has stored its sparse part in dpq and dpk.
hipError_t launch_proxy_kl_dense(const msa_plan_s* p, const DevMeta& m, const int32_t* kv_indices,
                                 const KlOperands& kl, hipStream_t st);
// The current device's static scratch of the allocation-free decode entry
// point (address from hipGetSymbolAddress, looked up once per device).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
hipError_t launch_decode(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                         const float* ks, const float* vs, const int32_t* kv_indices, const int32_t* sel,
                         void* out, float* lse, char* ws, hipStream_t st);

}  // namespace msa
