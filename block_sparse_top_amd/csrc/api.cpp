// Host side of the MSA C ABI: plan construction, argument validation,
// workspace layout and dispatch to the kernel launchers.  The plan follows
// the plan -> run split of the MiniMax-AI/MSA README (section "Usage": the
// plan is built from qo_lens / kv_lens, head counts, page size and topk).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "msa_internal.hpp"

namespace {

thread_local std::string g_last_error;

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status_t ok() {
  g_last_error.clear();
  return MSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

#define MSA_CHECK_PTR(p)                                                                        \
  do {                                                                                          \
    if ((p) == nullptr) return fail(MSA_ERR_INVALID_ARG, "%s: `%s` is NULL", __func__, #p);     \
    if (!aligned16(p)) return fail(MSA_ERR_INVALID_ARG, "%s: `%s` is not 16-byte aligned", __func__, #p); \
  } while (0)

#define MSA_CHECK_PTR_FN(fn, p)                                                                  \
  do {                                                                                           \
    if ((p) == nullptr) return fail(MSA_ERR_INVALID_ARG, "%s: `%s` is NULL", fn, #p);            \
    if (!aligned16(p)) return fail(MSA_ERR_INVALID_ARG, "%s: `%s` is not 16-byte aligned", fn, #p); \
  } while (0)

msa_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

// Which plan's metadata each workspace holds.  A call uploads the plan's
// metadata (one hipMemcpyAsync on its stream, ordered before its kernels)
// unless the record says that this workspace already holds exactly this
// plan's metadata, uploaded on the same stream.  Records are dropped when
// their plan is destroyed, when another plan's call may have written over
// their metadata (its workspace overlaps it), and by msa_workspace_reset.
// Plans are identified by a serial number, never by their address.
struct WsRecord {
  const char* meta_begin;
  const char* meta_end;
  const void* ws;
  uint64_t plan_uid;
  hipStream_t stream;
};
std::mutex g_ws_mu;
std::vector<WsRecord> g_ws;  // few entries: one per live workspace
std::atomic<uint64_t> g_plan_serial{1};

void forget_overlapping(const char* lo, const char* hi, uint64_t keep_uid, const void* keep_ws) {
  g_ws.erase(std::remove_if(g_ws.begin(), g_ws.end(),
                            [&](const WsRecord& r) {
                              if (r.plan_uid == keep_uid && r.ws == keep_ws) return false;
                              return r.meta_begin < hi && lo < r.meta_end;
                            }),
             g_ws.end());
}

msa_status_t upload_meta(msa_plan_s* p, void* ws, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  const char* base = static_cast<const char*>(ws);
  // this call's kernels may write anywhere in [ws, ws + total): other plans'
  // metadata there is no longer trusted
  forget_overlapping(base, base + p->lay.total, p->uid, ws);
  for (const WsRecord& r : g_ws)
    if (r.ws == ws && r.plan_uid == p->uid && r.stream == st) return MSA_OK;
  g_ws.erase(std::remove_if(g_ws.begin(), g_ws.end(), [&](const WsRecord& r) { return r.ws == ws; }), g_ws.end());
  hipError_t e = hipMemcpyAsync(static_cast<char*>(ws) + p->lay.meta, p->meta.data(),
                                p->meta.size() * sizeof(int32_t), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_status(e, "metadata upload");
  g_ws.push_back({base + p->lay.meta, base + p->lay.meta + p->lay.meta_bytes, ws, p->uid, st});
  return MSA_OK;
}

msa_status_t check_ws(const msa_plan_s* p, void* ws, size_t bytes) {
  if (ws == nullptr) return fail(MSA_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (bytes < p->lay.total)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %zu", bytes, p->lay.total);
  return MSA_OK;
}

// Per-head fp32 scales come with fp8 tensors only: fp8 (both), MXFP4 (its
// fp8 q); MXFP4 tensors carry their block scales in the data.
msa_status_t check_proxy_scales(const msa_plan_s* p, const float* qs, const float* ks, const char* fn) {
  const msa_dtype_t dt = p->d.proxy_dtype;
  const bool want_q = dt == MSA_FP8_E4M3 || dt == MSA_MXFP4, want_k = dt == MSA_FP8_E4M3;
  if (want_q != (qs != nullptr) || want_k != (ks != nullptr))
    return fail(MSA_ERR_INVALID_ARG, "%s: proxy_q_scale must be given iff proxy q is fp8 (fp8, MXFP4), proxy_k_scale "
                "iff proxy K is fp8", fn);
  return MSA_OK;
}

msa_status_t check_rows(const msa_plan_s* p, int64_t row_begin, int64_t row_count, const char* fn) {
  if (row_count <= 0 || row_begin < 0 || row_begin + row_count > p->T)
    return fail(MSA_ERR_INVALID_ARG, "%s: row range [%lld, %lld) is empty or outside [0, %d)", fn,
                (long long)row_begin, (long long)(row_begin + row_count), p->T);
  if (row_count > p->max_rows)
    return fail(MSA_ERR_INVALID_ARG, "%s: row_count %lld exceeds the plan's max_rows_per_call %lld", fn,
                (long long)row_count, (long long)p->max_rows);
  return MSA_OK;
}

}  // namespace

namespace msa {

DevMeta dev_meta(const msa_plan_s* p, const void* workspace) {
  const int32_t* base = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + p->lay.meta);
  DevMeta m;
  m.S = p->S;
  m.T = p->T;
  m.NB = p->NB;
  m.nb_max = p->nb_max;
  m.qo = base;
  m.kv = base + p->S;
  m.row_start = base + 2 * p->S;
  m.page_start = base + 3 * p->S + 1;
  m.tiles = base + 4 * p->S + 2;
  return m;
}

namespace {
hipEvent_t take_event(msa::Profiler& pr) {
  if (!pr.pool.empty()) {
    hipEvent_t e = pr.pool.back();
    pr.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
const char* const kKernelNames[] = {"proxy_maxscore", "topk_select", "proxy_topk", "topk_refine", "csr", "partial_attn",
                                    "merge",          "decode",      "decode_merge", "bwd_dq", "bwd_dq_sum",
                                    "bwd_dkv",        "kl_dq_sum",   "kl_dense_dq",  "kl_dense_dk",
                                    "dense_fwd",      "dense_dq",    "dense_dkv"};
}  // namespace

ProfEvents::ProfEvents(const msa_plan_s* p, const char* name) {
  if (p->prof.kernel.empty() || p->prof.kernel != name) return;
  start = take_event(p->prof);
  stop = take_event(p->prof);
  if (!start || !stop) {
    if (start) p->prof.pool.push_back(start);
    if (stop) p->prof.pool.push_back(stop);
    start = stop = nullptr;
    return;
  }
  p->prof.pending.emplace_back(start, stop);
}

}  // namespace msa

extern "C" {

msa_status_t msa_profile_kernel(msa_plan_t p, const char* kernel) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_profile_kernel: NULL plan");
  if (!kernel) {
    p->prof.kernel.clear();
    return ok();
  }
  for (const char* n : msa::kKernelNames)
    if (std::strcmp(n, kernel) == 0) {
      p->prof.kernel = kernel;
      return ok();
    }
  return fail(MSA_ERR_INVALID_ARG, "msa_profile_kernel: unknown kernel '%s'", kernel);
}

msa_status_t msa_profile_read(msa_plan_t p, double* total_ms, int64_t* launches) {
  if (!p || !total_ms || !launches) return fail(MSA_ERR_INVALID_ARG, "msa_profile_read: NULL argument");
  double tot = 0.0;
  msa_status_t st = MSA_OK;
  for (auto& pr : p->prof.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess && st == MSA_OK) st = hip_status(e, "msa_profile_read");
    tot += ms;
    p->prof.pool.push_back(pr.first);
    p->prof.pool.push_back(pr.second);
  }
  *launches = (int64_t)p->prof.pending.size();
  *total_ms = tot;
  p->prof.pending.clear();
  return st == MSA_OK ? ok() : st;
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

msa_status_t msa_workspace_reset(const void* workspace, size_t bytes) {
  if (!workspace) return fail(MSA_ERR_INVALID_ARG, "msa_workspace_reset: workspace is NULL");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  const char* lo = static_cast<const char*>(workspace);
  forget_overlapping(lo, lo + std::max<size_t>(bytes, 1), 0, nullptr);
  return ok();
}

msa_status_t msa_plan(const msa_plan_desc_t* desc, msa_plan_t* out, size_t* workspace_bytes) {
  if (!desc || !out || !workspace_bytes) return fail(MSA_ERR_INVALID_ARG, "msa_plan: NULL argument");
  *out = nullptr;
  const msa_plan_desc_t& d = *desc;
  if (d.batch < 1) return fail(MSA_ERR_INVALID_ARG, "msa_plan: batch must be >= 1 (got %d)", d.batch);
  if (d.mode != MSA_PREFILL && d.mode != MSA_DECODE) return fail(MSA_ERR_INVALID_ARG, "msa_plan: bad mode");
  if (!d.kv_lens_host) return fail(MSA_ERR_INVALID_ARG, "msa_plan: kv_lens_host is NULL");
  if (d.mode == MSA_PREFILL && !d.qo_lens_host) return fail(MSA_ERR_INVALID_ARG, "msa_plan: qo_lens_host is NULL");
  if (d.num_qo_heads < 1 || d.num_kv_heads < 1 || d.num_qo_heads % d.num_kv_heads)
    return fail(MSA_ERR_INVALID_ARG, "msa_plan: need num_qo_heads %% num_kv_heads == 0 (got %d, %d)",
                d.num_qo_heads, d.num_kv_heads);
  const int G = d.num_qo_heads / d.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_plan: GQA group size %d not in {1,2,4,8,16}", G);
  if (d.head_dim != 128) return fail(MSA_ERR_UNSUPPORTED, "msa_plan: head_dim %d != 128", d.head_dim);
  if (d.page_size != 128) return fail(MSA_ERR_UNSUPPORTED, "msa_plan: page_size %d != 128", d.page_size);
  if (d.topk < 1 || d.topk > 64) return fail(MSA_ERR_INVALID_ARG, "msa_plan: topk %d not in [1, 64]", d.topk);
  if (d.kv_dtype != MSA_BF16 && d.kv_dtype != MSA_FP8_E4M3 && d.kv_dtype != MSA_MXFP4)
    return fail(MSA_ERR_INVALID_ARG, "msa_plan: bad kv_dtype");
  if (d.mode == MSA_DECODE && d.kv_dtype == MSA_MXFP4)
    return fail(MSA_ERR_UNSUPPORTED, "msa_plan: MXFP4 K/V are built for prefill");
  if (!(d.sm_scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "msa_plan: sm_scale must be > 0");
  if (d.mode == MSA_PREFILL) {
    if (d.proxy_dtype != MSA_BF16 && d.proxy_dtype != MSA_FP8_E4M3 && d.proxy_dtype != MSA_MXFP4 &&
        d.proxy_dtype != MSA_MXFP4_QK)
      return fail(MSA_ERR_INVALID_ARG, "msa_plan: bad proxy_dtype");
    if (d.num_proxy_heads != d.num_kv_heads)
      return fail(MSA_ERR_UNSUPPORTED, "msa_plan: num_proxy_heads (%d) must equal num_kv_heads (%d)",
                  d.num_proxy_heads, d.num_kv_heads);
    if (d.num_proxy_kv_heads != 1 && d.num_proxy_kv_heads != d.num_proxy_heads)
      return fail(MSA_ERR_INVALID_ARG, "msa_plan: num_proxy_kv_heads must be 1 or num_proxy_heads");
    if (!(d.proxy_sm_scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "msa_plan: proxy_sm_scale must be > 0");
  }
  if (d.max_rows_per_call < 0) return fail(MSA_ERR_INVALID_ARG, "msa_plan: max_rows_per_call < 0");
  if (d.attn_window_rows < 0) return fail(MSA_ERR_INVALID_ARG, "msa_plan: attn_window_rows < 0");
  if (d.decode_splits < 0 || d.decode_splits > 64)
    return fail(MSA_ERR_INVALID_ARG, "msa_plan: decode_splits %d not in [0, 64]", d.decode_splits);

  msa_plan_s* p = new (std::nothrow) msa_plan_s();
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_plan: out of host memory");
  p->uid = g_plan_serial.fetch_add(1);
  p->d = d;
  p->d.qo_lens_host = nullptr;
  p->d.kv_lens_host = nullptr;
  p->S = d.batch;
  p->G = G;
  {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      p->num_cu = ncu;
  }
  int64_t T = 0, NB = 0;
  p->row_start.push_back(0);
  p->page_start.push_back(0);
  for (int s = 0; s < d.batch; ++s) {
    const int32_t kv = d.kv_lens_host[s];
    const int32_t qo = d.mode == MSA_DECODE ? 1 : d.qo_lens_host[s];
    if (d.mode == MSA_DECODE && d.qo_lens_host && d.qo_lens_host[s] != 1) {
      delete p;
      return fail(MSA_ERR_INVALID_ARG, "msa_plan: decode plans need qo_len == 1 (sequence %d has %d)", s,
                  d.qo_lens_host[s]);
    }
    if (qo < 1 || kv < qo) {
      delete p;
      return fail(MSA_ERR_INVALID_ARG, "msa_plan: sequence %d needs 1 <= qo_len <= kv_len (got %d, %d)", s, qo, kv);
    }
    const int32_t nb = (kv + 127) / 128;
    p->qo.push_back(qo);
    p->kv.push_back(kv);
    p->nb.push_back(nb);
    T += qo;
    NB += nb;
    p->nb_max = std::max(p->nb_max, nb);
    if (T > (int64_t)INT32_MAX / 64 || NB > (int64_t)INT32_MAX / 64) {
      delete p;
      return fail(MSA_ERR_UNSUPPORTED, "msa_plan: too many rows or pages");
    }
    p->row_start.push_back((int32_t)T);
    p->page_start.push_back((int32_t)NB);
  }
  // block ids are kept in 16 bits by the selection kernels' candidate lists
  if (p->nb_max > 65536) {
    const int32_t nbm = p->nb_max;
    delete p;
    return fail(MSA_ERR_UNSUPPORTED, "msa_plan: a sequence of %d blocks exceeds the limit of 65536 blocks (8388608 keys)",
                nbm);
  }
  p->T = (int32_t)T;
  p->NB = (int32_t)NB;
  p->max_rows = d.max_rows_per_call > 0 ? std::min<int64_t>(d.max_rows_per_call, T) : std::min<int64_t>(T, 32768);

  // Proxy row tiles: rows of one sequence whose positions fall in one
  // 512-aligned position window (at most 512 rows, one per lane of the proxy
  // kernel's 8 waves x 64 rows).
  for (int s = 0; s < p->S; ++s) {
    const int32_t first_pos = p->kv[s] - p->qo[s];
    int32_t i = 0;
    while (i < p->qo[s]) {
      const int32_t pos = first_pos + i;
      const int32_t end_pos = (pos / 512 + 1) * 512;
      const int32_t n = std::min(p->qo[s] - i, end_pos - pos);
      p->tiles.insert(p->tiles.end(), {s, p->row_start[s] + i, n, pos});
      i += n;
    }
  }
  p->ntiles = (int32_t)(p->tiles.size() / 4);

  // Metadata blob.
  p->meta.reserve(4 * p->S + 2 + p->tiles.size());
  p->meta.insert(p->meta.end(), p->qo.begin(), p->qo.end());
  p->meta.insert(p->meta.end(), p->kv.begin(), p->kv.end());
  p->meta.insert(p->meta.end(), p->row_start.begin(), p->row_start.end());
  p->meta.insert(p->meta.end(), p->page_start.begin(), p->page_start.end());
  p->meta.insert(p->meta.end(), p->tiles.begin(), p->tiles.end());

  // Workspace layout.
  msa::PlanLayout& L = p->lay;
  size_t off = 0;
  L.meta = off;
  L.meta_bytes = p->meta.size() * sizeof(int32_t);
  off = align_up(off + L.meta_bytes, 256);
  const int64_t Hkv = d.num_kv_heads, Hq = d.num_qo_heads, K = d.topk;
  if (d.mode == MSA_PREFILL) {
    p->tokens_per_chunk = 128 / G;
    // up to 16 chunks of 128 query rows per K/V load, at most 512 entries (LDS staging)
    p->entries_per_item = std::min(512, p->tokens_per_chunk * 16);
    // attention window: rows whose partials live at once.  Larger windows
    // give each (block, group) more rows per K/V load and fewer launches;
    // by default up to 32768 rows, capped at 16 GiB of partials.
    const int64_t per_row = Hq * K * (128 * 2 + 4);
    const int64_t auto_w = std::max<int64_t>(256, std::min<int64_t>(32768, ((int64_t)16 << 30) / per_row));
    p->attn_window = std::min<int64_t>(T, d.attn_window_rows > 0 ? d.attn_window_rows : auto_w);
    // each of the five planes of partial records (32 bytes a record) stays
    // under 2^32 bytes: the merge addresses a plane with a 32-bit offset
    p->attn_window = std::min<int64_t>(p->attn_window, (((int64_t)1 << 27) - msa::kTrashRecords) / (Hq * K));
    {
      const char* pin = std::getenv("MSA_XCD_PIN");
      p->xcd_pin = pin && pin[0] == '1';
    }
    const int64_t W = p->attn_window;
    const int64_t nkey = Hkv * NB;
    L.counts = off; off = align_up(off + nkey * 4, 256);
    L.cursor = off; off = align_up(off + nkey * 4, 256);
    L.offsets = off; off = align_up(off + (nkey + 1) * 4, 256);
    L.max_items = (W * Hkv * K + p->entries_per_item - 1) / p->entries_per_item + nkey;
    L.items = off; off = align_up(off + L.max_items * 16, 256);
    L.nitems = off; off = align_up(off + 16, 256);
    L.gitems = off; off = align_up(off + (Hkv + 1) * 4, 256);  // first work item of each KV group
    L.entries = off; off = align_up(off + W * Hkv * K * 4, 256);
    // the forward's partial records and the backward's dQ partial records
    // (block floating point, 152 and 164 bytes), each followed by
    // kTrashRecords records that take the stores of padding rows
    L.part_o = off;
    off = align_up(off + (W * Hq * K + msa::kTrashRecords) * msa::kPartRecordBytes, 256);
    L.bwd_d = off; off = align_up(off + W * Hq * 4, 256);  // the sparse backward's D = <dout, out> [W, Hq]
    // the fused backward's proxy distillation term needs one bf16 proxy head
    // and proxy-K head per KV group: its per-(token, group, slot) partials
    if (d.proxy_dtype == MSA_BF16 && d.num_proxy_heads == Hkv && d.num_proxy_kv_heads == Hkv) {
      L.kl_part = off;
      off = align_up(off + W * Hkv * K * 128 * 2, 256);
      L.kl_stash = off;
      off = align_up(off + nkey * 128 * 128 * 2 * 4, 256);
    }
    // one query row per sequence (a decode step's indexer pass): the proxy
    // pass uses the one-row kernel, and the fused selection keeps its block
    // scores here
    p->one_row = std::all_of(p->qo.begin(), p->qo.end(), [](int32_t q) { return q == 1; });
    const bool lowp = d.proxy_dtype != MSA_BF16;
    if (p->one_row) {
      L.dms = off;
      off = align_up(off + (int64_t)d.num_proxy_heads * p->nb_max * T * 4, 256);
      if (d.proxy_dtype == MSA_MXFP4 || d.proxy_dtype == MSA_MXFP4_QK) {
        L.kmx = off;
        off = align_up(off + (int64_t)d.num_proxy_kv_heads * p->nb_max * T * 4, 256);
      }
    } else if (lowp) {
      // every (row, group) pair may need exact re-scoring: 64 bytes each
      L.rq_count = off;
      off = align_up(off + 4, 256);
      L.rq = off;
      off = align_up(off + (int64_t)T * d.num_proxy_heads * 64, 256);
    }
  } else {
    // one workgroup per (sequence, group) when that fills the GPU; otherwise
    // split each pair's 32-key slices over up to 8 workgroups
    const int64_t pairs = (int64_t)p->S * Hkv;
    p->dec_splits = (int)std::max<int64_t>(1, std::min<int64_t>(8, (512 + pairs - 1) / pairs));
    if (pairs >= 192) p->dec_splits = 1;
    if (d.decode_splits > 0) p->dec_splits = d.decode_splits;
    L.dec_o = off; off = align_up(off + (size_t)p->S * Hq * p->dec_splits * 128 * 4, 256);
    L.dec_ml = off; off = align_up(off + (size_t)p->S * Hq * p->dec_splits * 2 * 4, 256);
  }
  L.total = off;
  *workspace_bytes = L.total;
  *out = p;
  return ok();
}

msa_status_t msa_plan_destroy(msa_plan_t plan) {
  if (plan) {
    {
      std::lock_guard<std::mutex> lk(g_ws_mu);
      g_ws.erase(std::remove_if(g_ws.begin(), g_ws.end(),
                                [&](const WsRecord& r) { return r.plan_uid == plan->uid; }),
                 g_ws.end());
    }
    for (auto& pr : plan->prof.pending) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
    for (hipEvent_t e : plan->prof.pool) (void)hipEventDestroy(e);
  }
  delete plan;
  return ok();
}

msa_status_t msa_plan_info(msa_plan_t p, int64_t* total_rows, int32_t* nb_max, int64_t* max_rows_per_call) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_plan_info: NULL plan");
  if (total_rows) *total_rows = p->T;
  if (nb_max) *nb_max = p->nb_max;
  if (max_rows_per_call) *max_rows_per_call = p->max_rows;
  return ok();
}

msa_status_t msa_proxy_block_maxscore(msa_plan_t p, const void* proxy_q, const void* proxy_k_pages,
                                      const float* proxy_q_scale, const float* proxy_k_scale,
                                      const int32_t* kv_indices, int64_t row_begin, int64_t row_count,
                                      float* max_score, void* workspace, size_t workspace_bytes,
                                      msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_proxy_block_maxscore: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_proxy_block_maxscore: decode plan");
  MSA_CHECK_PTR(proxy_q);
  MSA_CHECK_PTR(proxy_k_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(max_score);
  msa_status_t st = check_proxy_scales(p, proxy_q_scale, proxy_k_scale, __func__);
  if (st != MSA_OK) return st;
  if ((st = check_rows(p, row_begin, row_count, __func__)) != MSA_OK) return st;
  if ((st = check_ws(p, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  // tiles intersecting the row range
  int32_t lo = 0, hi = p->ntiles;
  while (lo < p->ntiles && p->tiles[4 * lo + 1] + p->tiles[4 * lo + 2] <= row_begin) ++lo;
  while (hi > lo && p->tiles[4 * (hi - 1) + 1] >= row_begin + row_count) --hi;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  return hip_status(msa::launch_proxy_maxscore(p, m, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale,
                                               kv_indices, lo, hi, row_begin, row_count, max_score, nullptr,
                                               msa::SelScratch{}, hs),
                    __func__);
}

msa_status_t msa_proxy_topk_select(msa_plan_t p, const void* proxy_q, const void* proxy_k_pages,
                                   const float* proxy_q_scale, const float* proxy_k_scale,
                                   const int32_t* kv_indices, int64_t row_begin, int64_t row_count,
                                   int32_t* kv_block_indexes, void* workspace, size_t workspace_bytes,
                                   msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_proxy_topk_select: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_proxy_topk_select: decode plan");
  if (p->d.topk > 17 && !p->one_row)
    return fail(MSA_ERR_UNSUPPORTED, "msa_proxy_topk_select: topk %d > 17; use msa_proxy_block_maxscore + msa_topk_select",
                p->d.topk);
  if (p->one_row && p->d.proxy_dtype != MSA_BF16 && p->nb_max > 2048)
    return fail(MSA_ERR_UNSUPPORTED,
                "msa_proxy_topk_select: one-query-row plans with a low-precision proxy select over at most 2048 "
                "blocks per sequence (got %d)", p->nb_max);
  MSA_CHECK_PTR(proxy_q);
  MSA_CHECK_PTR(proxy_k_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(kv_block_indexes);
  msa_status_t st = check_proxy_scales(p, proxy_q_scale, proxy_k_scale, __func__);
  if (st != MSA_OK) return st;
  if (row_count < 1 || row_begin < 0 || row_begin + row_count > p->T)
    return fail(MSA_ERR_INVALID_ARG, "msa_proxy_topk_select: rows [%lld, %lld) outside [0, %lld)", (long long)row_begin,
                (long long)(row_begin + row_count), (long long)p->T);
  if ((st = check_ws(p, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  int32_t lo = 0, hi = p->ntiles;
  while (lo < p->ntiles && p->tiles[4 * lo + 1] + p->tiles[4 * lo + 2] <= row_begin) ++lo;
  while (hi > lo && p->tiles[4 * (hi - 1) + 1] >= row_begin + row_count) --hi;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  char* ws = static_cast<char*>(workspace);
  msa::SelScratch scr;
  if (p->one_row) scr.dms = reinterpret_cast<float*>(ws + p->lay.dms);
  if (p->lay.kmx) scr.kmx = reinterpret_cast<int32_t*>(ws + p->lay.kmx);
  if (p->lay.rq) {
    scr.rq = reinterpret_cast<int32_t*>(ws + p->lay.rq);
    scr.rq_count = reinterpret_cast<int32_t*>(ws + p->lay.rq_count);
  }
  return hip_status(msa::launch_proxy_maxscore(p, m, proxy_q, proxy_k_pages, proxy_q_scale, proxy_k_scale,
                                               kv_indices, lo, hi, row_begin, row_count, nullptr, kv_block_indexes,
                                               scr, hs),
                    __func__);
}

msa_status_t msa_topk_select(msa_plan_t p, const float* max_score, int64_t row_begin, int64_t row_count,
                             int32_t* kv_block_indexes, void* workspace, size_t workspace_bytes,
                             msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_topk_select: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_topk_select: decode plan");
  MSA_CHECK_PTR(max_score);
  MSA_CHECK_PTR(kv_block_indexes);
  msa_status_t st = check_rows(p, row_begin, row_count, __func__);
  if (st != MSA_OK) return st;
  if ((st = check_ws(p, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  return hip_status(msa::launch_topk(p, m, max_score, false, row_begin, row_count, kv_block_indexes, hs), __func__);
}

static msa_status_t prefill_rows(const char* fn, msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                 const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                 const int32_t* kv_block_indexes, void* out, float* lse, int64_t row_begin,
                                 int64_t row_count, void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "%s: NULL plan", fn);
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "%s: decode plan", fn);
  MSA_CHECK_PTR(q);
  MSA_CHECK_PTR(k_pages);
  MSA_CHECK_PTR(v_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(kv_block_indexes);
  MSA_CHECK_PTR(out);
  if (lse && !aligned16(lse)) return fail(MSA_ERR_INVALID_ARG, "%s: lse not 16-byte aligned", fn);
  const bool fp8 = p->d.kv_dtype == MSA_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr))
    return fail(MSA_ERR_INVALID_ARG, "%s: k_scale and v_scale must be given iff K/V are fp8", fn);
  if (row_count < 1 || row_begin < 0 || row_begin + row_count > p->T)
    return fail(MSA_ERR_INVALID_ARG, "%s: rows [%lld, %lld) outside [0, %lld)", fn, (long long)row_begin,
                (long long)(row_begin + row_count), (long long)p->T);
  msa_status_t st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  const int64_t r1 = row_begin + row_count;
  for (int64_t w0 = row_begin; w0 < r1; w0 += p->attn_window) {
    const int32_t w1 = (int32_t)std::min<int64_t>(r1, w0 + p->attn_window);
    hipError_t e = msa::launch_prefill_window(p, m, q, k_pages, v_pages, k_scale, v_scale, kv_indices,
                                              kv_block_indexes, out, lse, static_cast<char*>(workspace), (int32_t)w0,
                                              w1, hs);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

msa_status_t msa_sparse_attn_prefill(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                     const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                     const int32_t* kv_block_indexes, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, msa_stream_t stream) {
  return prefill_rows(__func__, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out, lse, 0,
                      p ? p->T : 0, workspace, workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_prefill_rows(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                          const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                          const int32_t* kv_block_indexes, void* out, float* lse, int64_t row_begin,
                                          int64_t row_count, void* workspace, size_t workspace_bytes,
                                          msa_stream_t stream) {
  return prefill_rows(__func__, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out, lse,
                      row_begin, row_count, workspace, workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_prefill_backward(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                              const int32_t* kv_indices, const int32_t* kv_block_indexes,
                                              const void* out, const float* lse, const void* dout, float* dq,
                                              float* dk_pages, float* dv_pages, void* workspace, size_t workspace_bytes,
                                              msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attn_prefill_backward: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attn_prefill_backward: decode plan");
  if (p->d.kv_dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attn_prefill_backward: the backward is built for bf16 K/V");
  MSA_CHECK_PTR(q);
  MSA_CHECK_PTR(k_pages);
  MSA_CHECK_PTR(v_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(kv_block_indexes);
  MSA_CHECK_PTR(out);
  MSA_CHECK_PTR(lse);
  MSA_CHECK_PTR(dout);
  MSA_CHECK_PTR(dq);
  MSA_CHECK_PTR(dk_pages);
  MSA_CHECK_PTR(dv_pages);
  msa_status_t st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  for (int64_t w0 = 0; w0 < p->T; w0 += p->attn_window) {
    const int32_t w1 = (int32_t)std::min<int64_t>(p->T, w0 + p->attn_window);
    hipError_t e = msa::launch_prefill_backward_window(p, m, q, k_pages, v_pages, kv_indices, kv_block_indexes, out,
                                                       lse, dout, dq, dk_pages, dv_pages, nullptr,
                                                       static_cast<char*>(workspace), (int32_t)w0, w1, w0 == 0, hs);
    if (e != hipSuccess) return hip_status(e, __func__);
  }
  return ok();
}

msa_status_t msa_sparse_attn_prefill_backward_kl(msa_plan_t p, const void* q, const void* k_pages,
                                                 const void* v_pages, const int32_t* kv_indices,
                                                 const int32_t* kv_block_indexes, const void* out, const float* lse,
                                                 const void* dout, const void* proxy_q, const void* proxy_k_pages,
                                                 float kl_grad_scale, float* dq, float* dk_pages, float* dv_pages,
                                                 float* dproxy_q, float* dproxy_k_pages, float* proxy_lse,
                                                 void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attn_prefill_backward_kl: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attn_prefill_backward_kl: decode plan");
  if (p->d.kv_dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_attn_prefill_backward_kl: the backward is built for bf16 K/V");
  if (p->lay.kl_part == 0)
    return fail(MSA_ERR_UNSUPPORTED,
                "msa_sparse_attn_prefill_backward_kl: needs a bf16 proxy with one proxy head and one proxy-K head "
                "per KV group");
  if (!std::isfinite(kl_grad_scale))
    return fail(MSA_ERR_INVALID_ARG, "msa_sparse_attn_prefill_backward_kl: kl_grad_scale is not finite");
  MSA_CHECK_PTR(q);
  MSA_CHECK_PTR(k_pages);
  MSA_CHECK_PTR(v_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(kv_block_indexes);
  MSA_CHECK_PTR(out);
  MSA_CHECK_PTR(lse);
  MSA_CHECK_PTR(dout);
  MSA_CHECK_PTR(proxy_q);
  MSA_CHECK_PTR(proxy_k_pages);
  MSA_CHECK_PTR(dq);
  MSA_CHECK_PTR(dk_pages);
  MSA_CHECK_PTR(dv_pages);
  MSA_CHECK_PTR(dproxy_q);
  MSA_CHECK_PTR(dproxy_k_pages);
  MSA_CHECK_PTR(proxy_lse);
  msa_status_t st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  const msa::KlOperands kl{proxy_q, proxy_k_pages, dproxy_q, dproxy_k_pages, proxy_lse, p->d.proxy_sm_scale,
                           kl_grad_scale};
  for (int64_t w0 = 0; w0 < p->T; w0 += p->attn_window) {
    const int32_t w1 = (int32_t)std::min<int64_t>(p->T, w0 + p->attn_window);
    hipError_t e = msa::launch_prefill_backward_window(p, m, q, k_pages, v_pages, kv_indices, kv_block_indexes, out,
                                                       lse, dout, dq, dk_pages, dv_pages, &kl,
                                                       static_cast<char*>(workspace), (int32_t)w0, w1, w0 == 0, hs);
    if (e != hipSuccess) return hip_status(e, __func__);
  }
  return hip_status(msa::launch_proxy_kl_dense(p, m, kv_indices, kl, hs), __func__);
}

msa_status_t msa_dense_attn_prefill(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                    const int32_t* kv_indices, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_dense_attn_prefill: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_dense_attn_prefill: decode plan");
  if (p->d.kv_dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_dense_attn_prefill: the dense attention is built for bf16 K/V");
  MSA_CHECK_PTR(q);
  MSA_CHECK_PTR(k_pages);
  MSA_CHECK_PTR(v_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(out);
  MSA_CHECK_PTR(lse);
  msa_status_t st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  return hip_status(msa::launch_dense_forward(p, m, q, k_pages, v_pages, kv_indices, out, lse, hs), __func__);
}

msa_status_t msa_dense_attn_prefill_backward(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                             const int32_t* kv_indices, const void* out, const float* lse,
                                             const void* dout, const void* proxy_q, const void* proxy_k_pages,
                                             float kl_grad_scale, float* dq, float* dk_pages, float* dv_pages,
                                             float* dproxy_q, float* dproxy_k_pages, float* proxy_lse,
                                             void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "msa_dense_attn_prefill_backward: NULL plan");
  if (p->d.mode != MSA_PREFILL) return fail(MSA_ERR_UNSUPPORTED, "msa_dense_attn_prefill_backward: decode plan");
  if (p->d.kv_dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "msa_dense_attn_prefill_backward: the dense attention is built for bf16 K/V");
  MSA_CHECK_PTR(q);
  MSA_CHECK_PTR(k_pages);
  MSA_CHECK_PTR(v_pages);
  MSA_CHECK_PTR(kv_indices);
  MSA_CHECK_PTR(out);
  MSA_CHECK_PTR(lse);
  MSA_CHECK_PTR(dout);
  MSA_CHECK_PTR(dq);
  MSA_CHECK_PTR(dk_pages);
  MSA_CHECK_PTR(dv_pages);
  const bool with_kl = proxy_q != nullptr || proxy_k_pages != nullptr;
  if (with_kl) {
    if (p->d.proxy_dtype != MSA_BF16 || p->d.num_proxy_heads != p->d.num_kv_heads ||
        p->d.num_proxy_kv_heads != p->d.num_kv_heads)
      return fail(MSA_ERR_UNSUPPORTED,
                  "msa_dense_attn_prefill_backward: the proxy term needs a bf16 proxy with one proxy head and one "
                  "proxy-K head per KV group");
    if (!std::isfinite(kl_grad_scale))
      return fail(MSA_ERR_INVALID_ARG, "msa_dense_attn_prefill_backward: kl_grad_scale is not finite");
    MSA_CHECK_PTR(proxy_q);
    MSA_CHECK_PTR(proxy_k_pages);
    MSA_CHECK_PTR(dproxy_q);
    MSA_CHECK_PTR(dproxy_k_pages);
    MSA_CHECK_PTR(proxy_lse);
  }
  // D = <dout, out> for every row lives in the partial-output area
  if ((size_t)p->T * p->d.num_qo_heads * 4 > p->lay.bwd_d - p->lay.part_o)
    return fail(MSA_ERR_UNSUPPORTED,
                "msa_dense_attn_prefill_backward: the plan's attention window is too short for this many rows "
                "(its partial area holds D = <dout, out> of every row)");
  msa_status_t st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  float* D = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->lay.part_o);
  const msa::KlOperands kl{proxy_q, proxy_k_pages, dproxy_q, dproxy_k_pages, proxy_lse, p->d.proxy_sm_scale,
                           kl_grad_scale};
  const msa::KlOperands* klp = with_kl ? &kl : nullptr;
  hipError_t e = msa::launch_bwd_prep(p, out, dout, D, 0, p->T, hs);
  if (e == hipSuccess) e = msa::launch_dense_dq(p, m, q, k_pages, v_pages, kv_indices, lse, D, dout, dq, klp, hs);
  if (e == hipSuccess)
    e = msa::launch_dense_dkv(p, m, q, k_pages, v_pages, kv_indices, lse, D, dout, dk_pages, dv_pages, klp,
                              static_cast<char*>(workspace), hs);
  if (e == hipSuccess && with_kl) e = msa::launch_proxy_kl_dense(p, m, kv_indices, kl, hs);
  return hip_status(e, __func__);
}

static msa_status_t decode_args(const char* fn, msa_plan_t p, const void* q, const void* k_pages,
                                const void* v_pages, const float* k_scale, const float* v_scale,
                                const int32_t* kv_indices, const int32_t* kv_block_indexes, void* out, float* lse) {
  if (!p) return fail(MSA_ERR_INVALID_ARG, "%s: NULL plan", fn);
  if (p->d.mode != MSA_DECODE) return fail(MSA_ERR_UNSUPPORTED, "%s: prefill plan", fn);
  MSA_CHECK_PTR_FN(fn, q);
  MSA_CHECK_PTR_FN(fn, k_pages);
  MSA_CHECK_PTR_FN(fn, v_pages);
  MSA_CHECK_PTR_FN(fn, kv_indices);
  MSA_CHECK_PTR_FN(fn, kv_block_indexes);
  MSA_CHECK_PTR_FN(fn, out);
  if (lse && !aligned16(lse)) return fail(MSA_ERR_INVALID_ARG, "%s: lse not 16-byte aligned", fn);
  const bool fp8 = p->d.kv_dtype == MSA_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr))
    return fail(MSA_ERR_INVALID_ARG, "%s: scale pointers must be given iff K/V are fp8", fn);
  return MSA_OK;
}

static msa_status_t decode_common(const char* fn, msa_plan_t p, const void* q, const void* k_pages,
                                  const void* v_pages, const float* k_scale, const float* v_scale,
                                  const int32_t* kv_indices, const int32_t* kv_block_indexes, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, msa_stream_t stream);

msa_status_t msa_sparse_attn_decode(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                    const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                    const int32_t* kv_block_indexes, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, msa_stream_t stream) {
  return decode_common(__func__, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out, lse,
                       workspace, workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_decode_noalloc(msa_plan_t p, const void* q, const void* k_pages, const void* v_pages,
                                            const float* k_scale, const float* v_scale, const int32_t* kv_indices,
                                            const int32_t* kv_block_indexes, void* out, float* lse,
                                            msa_stream_t stream) {
  msa_status_t st = decode_args(__func__, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes,
                                out, lse);
  if (st != MSA_OK) return st;
  void* scr = nullptr;
  size_t scr_bytes = 0;
  hipError_t e = msa::noalloc_scratch(&scr, &scr_bytes);
  if (e != hipSuccess) return hip_status(e, "msa_sparse_attn_decode_noalloc: static scratch address");
  if (p->lay.total > scr_bytes)
    return fail(MSA_ERR_INVALID_ARG,
                "msa_sparse_attn_decode_noalloc: the plan needs %zu bytes of scratch, above the static scratch of "
                "%zu bytes; use msa_sparse_attn_decode with a workspace",
                p->lay.total, scr_bytes);
  return decode_common(__func__, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out, lse,
                       scr, scr_bytes, stream);
}

static msa_status_t decode_common(const char* fn, msa_plan_t p, const void* q, const void* k_pages,
                                  const void* v_pages, const float* k_scale, const float* v_scale,
                                  const int32_t* kv_indices, const int32_t* kv_block_indexes, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  msa_status_t st = decode_args(fn, p, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes, out, lse);
  if (st != MSA_OK) return st;
  st = check_ws(p, workspace, workspace_bytes);
  if (st != MSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = upload_meta(p, workspace, hs)) != MSA_OK) return st;
  const msa::DevMeta m = msa::dev_meta(p, workspace);
  return hip_status(msa::launch_decode(p, m, q, k_pages, v_pages, k_scale, v_scale, kv_indices, kv_block_indexes,
                                       out, lse, static_cast<char*>(workspace), hs),
                    fn);
}

}  // extern "C"
