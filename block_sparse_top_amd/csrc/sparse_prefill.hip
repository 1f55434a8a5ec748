// Stage 3a of MSA: block-sparse GQA prefill attention.
//
// Attention of each query row over only its group's selected 128-key blocks
// (MiniMax-AI/MSA README, section "Usage": attention with kv_block_indexes;
// README section "Stacks": block-sparse prefill with CSR metadata).  As the
// Flash-MSA article describes for its main attention (paragraph on the
// forward kernels), block-sparse attention is recast as variable-length
// dense attention: every selected (block, group) pair becomes one short
// "sequence" of 128 keys whose queries are the rows that selected it.
//
// Per window of rows [w0, w1) (bounded workspace):
//  1. csr_count / csr_scan / csr_fill: invert kv_block_indexes into, per
//     (group, block), the list of (row, slot) entries that selected it, and a
//     list of work items of at most `entries_per_item` rows each;
//  2. partial_attn: one workgroup per work item loads the block's K and V
//     (32 KB each) into LDS once, then for chunks of 128 query rows
//     (128/G tokens x G heads of the group) computes S^T = K Q^T and
//     O^T = V^T P^T on bf16 MFMA with the causal mask, and writes a
//     normalised partial output (bf16) and its log-sum-exp per
//     (row, head, slot);
//  3. merge: per (row, head) the slot partials are combined with their
//     log-sum-exp weights into the final output and lse.
#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int kKRow = 272;  // LDS bytes per K row (256 + 16: spreads 16-byte reads over banks)
constexpr int kVRow = 320;  // LDS bytes per V row (256 + 64: spreads transposed 8-byte reads)

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

struct CsrArgs {
  const int32_t* sel;  // [T, Hkv, k]
  DevMeta m;
  int32_t* counts;     // [Hkv * NB]
  int32_t* cursor;     // [Hkv * NB]
  const int32_t* offsets;
  int32_t* entries;
  int32_t w0, w1, Hkv, k;
};

// One thread per (row, group): visit the row's valid slots (0 <= b <= local).
template <bool FILL>
__global__ __launch_bounds__(256) void csr_pass_kernel(CsrArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nrows = a.w1 - a.w0;
  if (idx >= nrows * a.Hkv) return;
  const int32_t rl = (int32_t)(idx / a.Hkv);
  const int g = (int)(idx % a.Hkv);
  const int32_t r = a.w0 + rl;
  const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
  const int32_t pos = a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s]);
  const int local = pos >> 7;
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  const int32_t pb = a.m.page_start[s];
  for (int slot = 0; slot < a.k; ++slot) {
    const int b = row[slot];
    if (b < 0 || b > local) continue;
    const int key = g * a.m.NB + pb + b;
    if (!FILL) {
      atomicAdd(&a.counts[key], 1);
    } else {
      const int at = atomicAdd(&a.cursor[key], 1);
      a.entries[a.offsets[key] + at] = rl * a.k + slot;
    }
  }
}

// Single workgroup: exclusive scan of the counts into offsets, and the work
// item list (g, global block, first entry, end entry).
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(const int32_t* counts, int32_t* offsets, int4* items,
                                                                int32_t* nitems, int32_t n, int32_t NB, int32_t epi) {
  __shared__ int32_t s_e[kScanThreads], s_i[kScanThreads];
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int32_t se = 0, si = 0;
  for (int j = lo; j < hi; ++j) {
    se += counts[j];
    si += (counts[j] + epi - 1) / epi;
  }
  s_e[t] = se;
  s_i[t] = si;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
    int32_t ve = t >= off ? s_e[t - off] : 0, vi = t >= off ? s_i[t - off] : 0;
    __syncthreads();
    s_e[t] += ve;
    s_i[t] += vi;
    __syncthreads();
  }
  int32_t e = s_e[t] - se, it = s_i[t] - si;
  for (int j = lo; j < hi; ++j) {
    const int32_t c = counts[j];
    offsets[j] = e;
    for (int32_t x = 0; x < c; x += epi) items[it++] = make_int4(j / NB, j % NB, e + x, e + min(c, x + epi));
    e += c;
  }
  if (t == kScanThreads - 1) {
    offsets[n] = s_e[t];
    *nitems = s_i[t];
  }
}

struct PartialArgs {
  const uint8_t* q;      // bf16 [T, Hq, 128]
  const uint8_t* kp;     // bf16 [N, Hkv, 128, 128]
  const uint8_t* vp;
  const int32_t* kv_indices;
  const int32_t* entries;
  const int4* items;
  const int32_t* nitems;
  DevMeta m;
  uint16_t* part_o;      // [rows, Hq, k, 128] bf16
  float* part_lse;       // [rows, Hq, k]
  int32_t Hq, Hkv, G, k, w0;
  float scale_log2;      // sm_scale * log2(e)
};

__global__ __launch_bounds__(256, 2) void partial_attn_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[128 * kKRow];
  __shared__ __attribute__((aligned(16))) uint8_t vs[128 * kVRow];
  const int item = blockIdx.x;
  if (item >= *a.nitems) return;
  const int4 it = a.items[item];
  const int g = it.x, gb = it.y, e0 = it.z, e1 = it.w;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = upper_bound_i32(a.m.page_start, a.m.S + 1, gb) - 1;
  const int b = gb - a.m.page_start[s];
  const int32_t page = a.kv_indices[gb];
  const int32_t first_pos = a.m.kv[s] - a.m.qo[s];
  const int32_t rs = a.m.row_start[s];

  {  // K and V block -> LDS (coalesced 16-byte chunks)
    const uint8_t* kb = a.kp + ((int64_t)page * a.Hkv + g) * 32768;
    const uint8_t* vb = a.vp + ((int64_t)page * a.Hkv + g) * 32768;
    i32x4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      kr[i] = *reinterpret_cast<const i32x4*>(kb + c * 16);
      vr[i] = *reinterpret_cast<const i32x4*>(vb + c * 16);
    }
    const int kv_in_block = a.m.kv[s] - b * 128;  // V rows at or past this are page padding
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      lds_store16<i32x4>(&ks[(c >> 4) * kKRow + (c & 15) * 16], kr[i]);
      // padding may hold anything; P is 0 there but 0 * NaN is NaN
      lds_store16<i32x4>(&vs[(c >> 4) * kVRow + (c & 15) * 16], (c >> 4) < kv_in_block ? vr[i] : i32x4{});
    }
  }
  __syncthreads();

  const int G = a.G;
  const int MT = 128 / G;                      // tokens per 128-row chunk
  const int qr = 32 * wave + (lane & 31);      // this lane's query row within the chunk
  const int half = lane >> 5;
  const int q16 = lane >> 4, m16 = lane & 15;
  for (int c0 = e0; c0 < e1; c0 += MT) {
    const int e = c0 + qr / G;
    const bool valid = e < e1;
    const int ent = a.entries[valid ? e : e0];
    const int rl = ent / a.k, slot = ent % a.k;
    const int32_t r = a.w0 + rl;
    const int h = g * G + qr % G;
    const int32_t pos = first_pos + (r - rs);

    bf16x8 qf[8];
    const uint8_t* qrow = a.q + ((int64_t)r * a.Hq + h) * 256;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + st * 32 + half * 16);

    // S^T = K Q^T: 4 key tiles of 32
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 af = lds_load16<bf16x8>(&ks[(32 * kt + (lane & 31)) * kKRow + st * 32 + half * 16]);
        acc[kt] = mfma32x32x16(af, qf[st], acc[kt]);
      }
    }
    // causal mask (keys past the row's position), row max
    const int lim = pos - b * 128 - 4 * half;
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = 32 * kt + 8 * (i >> 2) + (i & 3);
        const float v = koff <= lim ? acc[kt][i] : kNegInf;
        acc[kt][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, wave_xor32(mx));
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2((acc[kt][i] - mx) * a.scale_log2);
        acc[kt][i] = pv;
        sum += pv;
      }
    }
    sum += wave_xor32(sum);

    // O^T = V^T P^T
    f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pf;
#pragma unroll
        for (int t = 0; t < 8; ++t) pf[t] = (__bf16)acc[kt][8 * u + t];
        const int key0 = 32 * kt + 16 * u + 4 * (q16 >> 1);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d0 = 32 * dt + 16 * (q16 & 1);
          const s16x4 lo = lds_read_tr16(&vs[(key0 + (m16 >> 2)) * kVRow + (d0 + 4 * (m16 & 3)) * 2]);
          const s16x4 hi = lds_read_tr16(&vs[(key0 + 8 + (m16 >> 2)) * kVRow + (d0 + 4 * (m16 & 3)) * 2]);
          const bf16x8 vf = join_tr16(lo, hi);
          oacc[dt] = mfma32x32x16(vf, pf, oacc[dt]);
        }
      }
    }
    if (valid) {
      const float inv = 1.f / sum;
      const int64_t pi = ((int64_t)rl * a.Hq + h) * a.k + slot;
      uint16_t* orow = a.part_o + pi * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          bf16x4 o;
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t] = (__bf16)(oacc[dt][4 * gq + t] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * gq + 4 * half) = o;
        }
      }
      if (half == 0) a.part_lse[pi] = (mx * a.scale_log2 + fast_log2(sum)) * kLn2;
    }
  }
}

struct MergeArgs {
  const int32_t* sel;
  DevMeta m;
  const uint16_t* part_o;
  const float* part_lse;
  uint16_t* out;   // bf16 [T, Hq, 128]
  float* lse;      // [T, Hq] or null
  int32_t Hq, Hkv, G, k, w0, w1;
};

// One wave per (row, head); lane l owns output columns 2l, 2l+1.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)(a.w1 - a.w0) * a.Hq) return;
  const int32_t rl = (int32_t)(idx / a.Hq);
  const int h = (int)(idx % a.Hq);
  const int g = h / a.G;
  const int32_t r = a.w0 + rl;
  const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
  const int local = (a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s])) >> 7;
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  const int64_t base = ((int64_t)rl * a.Hq + h) * a.k;
  float M = kNegInf;
  for (int slot = 0; slot < a.k; ++slot) {
    const int b = row[slot];
    if (b >= 0 && b <= local) M = fmaxf(M, a.part_lse[base + slot]);
  }
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int slot = 0; slot < a.k; ++slot) {
    const int b = row[slot];
    if (b < 0 || b > local) continue;
    const float w = fast_exp2((a.part_lse[base + slot] - M) * kLog2e);
    const uint32_t two = *reinterpret_cast<const uint32_t*>(a.part_o + (base + slot) * 128 + 2 * lane);
    L += w;
    o0 += w * __builtin_bit_cast(float, two << 16);
    o1 += w * __builtin_bit_cast(float, two & 0xffff0000u);
  }
  const float inv = 1.f / L;
  bf16x2 o;
  o[0] = (__bf16)(o0 * inv);
  o[1] = (__bf16)(o1 * inv);
  *reinterpret_cast<bf16x2*>(a.out + ((int64_t)r * a.Hq + h) * 128 + 2 * lane) = o;
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.Hq + h] = M + fast_log2(L) * kLn2;
}

}  // namespace

hipError_t launch_prefill_window(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp,
                                 const void* vp, const int32_t* kv_indices, const int32_t* sel, void* out,
                                 float* lse, char* ws, int32_t w0, int32_t w1, hipStream_t st) {
  const PlanLayout& L = p->lay;
  const int Hkv = p->d.num_kv_heads, Hq = p->d.num_qo_heads, k = p->d.topk;
  const int32_t nkey = Hkv * p->NB;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int4* items = reinterpret_cast<int4*>(ws + L.items);
  int32_t* nitems = reinterpret_cast<int32_t*>(ws + L.nitems);
  int32_t* entries = reinterpret_cast<int32_t*>(ws + L.entries);
  // counts and cursor are adjacent 256-aligned segments: clear both
  const int64_t nclear = (int64_t)(L.offsets - L.counts) / 4;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<int64_t>(1024, (nclear + 255) / 256)), dim3(256), 0, st,
                     counts, nclear, 0);
  CsrArgs c;
  c.sel = sel;
  c.m = m;
  c.counts = counts;
  c.cursor = cursor;
  c.offsets = offsets;
  c.entries = entries;
  c.w0 = w0;
  c.w1 = w1;
  c.Hkv = Hkv;
  c.k = k;
  const int64_t nthreads = (int64_t)(w1 - w0) * Hkv;
  const dim3 cgrid((unsigned)((nthreads + 255) / 256));
  hipLaunchKernelGGL(csr_pass_kernel<false>, cgrid, dim3(256), 0, st, c);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, counts, offsets, items, nitems, nkey,
                     p->NB, p->entries_per_item);
  hipLaunchKernelGGL(csr_pass_kernel<true>, cgrid, dim3(256), 0, st, c);

  PartialArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.kp = static_cast<const uint8_t*>(kp);
  a.vp = static_cast<const uint8_t*>(vp);
  a.kv_indices = kv_indices;
  a.entries = entries;
  a.items = items;
  a.nitems = nitems;
  a.m = m;
  a.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p->G;
  a.k = k;
  a.w0 = w0;
  a.scale_log2 = p->d.sm_scale * kLog2e;
  // upper bound on the number of work items of this window
  const int64_t max_items = ((int64_t)(w1 - w0) * Hkv * k + p->entries_per_item - 1) / p->entries_per_item + nkey;
  hipLaunchKernelGGL(partial_attn_kernel, dim3((unsigned)max_items), dim3(256), 0, st, a);

  MergeArgs mg;
  mg.sel = sel;
  mg.m = m;
  mg.part_o = a.part_o;
  mg.part_lse = a.part_lse;
  mg.out = static_cast<uint16_t*>(out);
  mg.lse = lse;
  mg.Hq = Hq;
  mg.Hkv = Hkv;
  mg.G = p->G;
  mg.k = k;
  mg.w0 = w0;
  mg.w1 = w1;
  const int64_t nwaves = (int64_t)(w1 - w0) * Hq;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((nwaves + 3) / 4)), dim3(256), 0, st, mg);
  return hipGetLastError();
}

}  // namespace msa
