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
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {


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
  int32_t with_local;  // 1: a row's own block is an entry too (the backward); 0: it is not (the forward)
};

// One thread per row of one group (grid.y = group); a row's valid slots are
// those with 0 <= b <= local (b < local without the row's own block).  With LDS_HIST the workgroup first histograms
// its 256 rows' blocks in LDS, so global memory sees one atomic per touched
// (group, block) bin per workgroup instead of one per entry.
constexpr int kMaxLdsBins = 16384;

// A row's slots, kSlotChunk at a time: the loads of a chunk are issued
// together, so a row waits for one memory latency per chunk rather than one
// per slot.  A row is 16-byte aligned when k is a multiple of 4 (sel is), and
// then loads as int4.  Slots past k read as -1 (not an entry).
constexpr int kSlotChunk = 16;
__device__ __forceinline__ void load_slots(const int32_t* row, int s0, int k, int32_t (&v)[kSlotChunk]) {
  if ((k & 3) == 0) {
#pragma unroll
    for (int j = 0; j < kSlotChunk; j += 4) {
      const i32x4 x = s0 + j < k ? *reinterpret_cast<const i32x4*>(row + s0 + j) : i32x4{-1, -1, -1, -1};
      v[j] = x[0];
      v[j + 1] = x[1];
      v[j + 2] = x[2];
      v[j + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSlotChunk; ++j) v[j] = s0 + j < k ? row[s0 + j] : -1;
  }
}

template <bool FILL, bool LDS_HIST>
__global__ __launch_bounds__(256) void csr_pass_kernel(CsrArgs a) {
  extern __shared__ int32_t hist[];
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int32_t nrows = a.w1 - a.w0;
  const int32_t rl = (int32_t)blockIdx.x * 256 + tid;
  const bool valid = rl < nrows;
  const int32_t r = a.w0 + (valid ? rl : 0);
  const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
  const int32_t pos = a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s]);
  // entries: blocks 0 <= b < bend; an invalid lane has none
  const int bend = valid ? (pos >> 7) + a.with_local : 0;
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  const int32_t pb = a.m.page_start[s];
  const int NB = a.m.NB;
  int32_t* counts = a.counts + (int64_t)g * NB;
  int32_t* cursor = a.cursor + (int64_t)g * NB;
  const int32_t* offsets = a.offsets + (int64_t)g * NB;
  int32_t v[kSlotChunk];
  if constexpr (!LDS_HIST) {
    if (!valid) return;
    for (int s0 = 0; s0 < a.k; s0 += kSlotChunk) {
      load_slots(row, s0, a.k, v);
#pragma unroll
      for (int j = 0; j < kSlotChunk; ++j) {
        const int b = v[j];
        if (b < 0 || b >= bend) continue;
        if (!FILL) atomicAdd(&counts[pb + b], 1);
        else a.entries[offsets[pb + b] + atomicAdd(&cursor[pb + b], 1)] = (rl << 6) | (s0 + j);
      }
    }
    return;
  } else {
    for (int i = tid; i < NB; i += 256) hist[i] = 0;
    __syncthreads();
    for (int s0 = 0; s0 < a.k; s0 += kSlotChunk) {
      load_slots(row, s0, a.k, v);
#pragma unroll
      for (int j = 0; j < kSlotChunk; ++j)
        if (v[j] >= 0 && v[j] < bend) atomicAdd(&hist[pb + v[j]], 1);
    }
    __syncthreads();
    for (int i = tid; i < NB; i += 256) {
      const int c = hist[i];
      if (c == 0) continue;
      if (!FILL) atomicAdd(&counts[i], c);
      else hist[i] = offsets[i] + atomicAdd(&cursor[i], c);  // this workgroup's range in bin i
    }
    if (!FILL) return;
    __syncthreads();
    for (int s0 = 0; s0 < a.k; s0 += kSlotChunk) {
      load_slots(row, s0, a.k, v);
#pragma unroll
      for (int j = 0; j < kSlotChunk; ++j)
        if (v[j] >= 0 && v[j] < bend) a.entries[atomicAdd(&hist[pb + v[j]], 1)] = (rl << 6) | (s0 + j);
    }
  }
}

// Single workgroup: exclusive scan of the counts into offsets, and the work
// item list (g, global block, first entry, end entry).
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(const int32_t* counts, int32_t* offsets, int4* items,
                                                                int32_t* nitems, int32_t* gitems, int32_t n, int32_t NB,
                                                                int32_t epi) {
  __shared__ int32_t s_e[kScanThreads], s_i[kScanThreads];
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  // a thread's counts are read 8 at a time (loads issued together)
  int32_t se = 0, si = 0;
  for (int j0 = lo; j0 < hi; j0 += 8) {
    int32_t c8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c8[u] = j0 + u < hi ? counts[j0 + u] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      se += c8[u];
      si += (c8[u] + epi - 1) / epi;
    }
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
  for (int j0 = lo; j0 < hi; j0 += 8) {
    int32_t c8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c8[u] = j0 + u < hi ? counts[j0 + u] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      if (j >= hi) break;
      const int32_t c = c8[u];
      offsets[j] = e;
      if (j % NB == 0) gitems[j / NB] = it;  // keys are group-major: a group's items are contiguous
      for (int32_t x = 0; x < c; x += epi) items[it++] = make_int4(j / NB, j % NB, e + x, e + min(c, x + epi));
      e += c;
    }
  }
  if (t == kScanThreads - 1) {
    offsets[n] = s_e[t];
    *nitems = s_i[t];
    gitems[n / NB] = s_i[t];
  }
}

// K/V page formats: bf16; fp8 e4m3 with one fp32 scale per KV head (the
// codes widen to bf16 exactly, the scales fold into the logit scale and the
// output); MXFP4 records (codes widen with their E8M0 block scale, exactly).
enum class KvFmt : int { BF16 = 0, FP8 = 1, MX4 = 2 };

// Forward partial records: the window's rows in tiles of 2^rec_shift = 128 / G
// rows (the rows of one merge workgroup), tile after tile; inside a tile of
// tr rows starting at row t0, slot-major: window row rl, slot `slot`, query
// head g * G + hh is record t0 k Hq + ((slot Hkv + g) tr + rl - t0) G + hh
// (the last tile of the rec_rows-row index may be shorter).  A token's G
// heads are adjacent (for G = 4 one 128-byte line per plane), and one slot
// of a tile's rows for one group is contiguous: the merge, which takes one
// slot of a block's consecutive rows at a time, reads 4 KB pieces of one
// tile's region.  Below 2^32: the plan caps the window.
__device__ __forceinline__ uint32_t fwd_rec(int slot, int g, int rl, int hh, int Hkv, int G, int k, int rec_rows,
                                            int rec_shift) {
  const uint32_t t0 = ((uint32_t)rl >> rec_shift) << rec_shift;
  const uint32_t tr = min(1u << rec_shift, (uint32_t)rec_rows - t0);
  return t0 * (uint32_t)k * (uint32_t)(Hkv * G) +
         (((uint32_t)slot * (uint32_t)Hkv + (uint32_t)g) * tr + ((uint32_t)rl - t0)) * (uint32_t)G + (uint32_t)hh;
}

struct PartialArgs {
  const uint8_t* q;      // bf16 [T, Hq, 128]
  const uint8_t* kp;     // [N, Hkv, 128, 128] bf16 / fp8, or [N, Hkv, 8704 B] MXFP4 records
  const uint8_t* vp;
  const float* ks;       // fp8: [Hkv] scales, else null
  const float* vs;
  const int32_t* kv_indices;
  const int32_t* entries;
  const int4* items;
  const int32_t* nitems;
  const int32_t* gitems;  // first item of each KV group, [Hkv + 1]
  int32_t xcd_pin;        // 1: workgroup i runs an item of the groups assigned to XCD i % 8
  DevMeta m;
  uint8_t* part_pk;      // partial records, block floating point (see store_rows_bfp9): planes of
  int64_t plane_stride;  //   32 bytes per record (fwd_rec order) + trash records, this far apart
  float2* part_st;       //   {log-sum-exp, step} per record, indexed as the records (then the trash entries)
  int64_t trash;         // index of the first of kTrashRecords trash records (rows * Hq * k)
  int32_t rec_rows, rec_shift;  // record index (fwd_rec): the plan's window rows, log2(128 / G)
  int32_t Hq, Hkv, G, k, w0;
  float scale_log2;      // sm_scale * log2(e)
};

constexpr int kMaxItemEntries = 512;   // entries_per_item = min(512, 16 chunks of 128 / G tokens)

// Eight K/V elements of key row `row`, dims 8 col .. 8 col + 7, as bf16
// (exact) from a page of format F.
template <KvFmt F>
__device__ __forceinline__ i32x4 load_kv8(const uint8_t* page, int row, int col) {
  if constexpr (F == KvFmt::BF16) {
    return *reinterpret_cast<const i32x4*>(page + row * 256 + col * 16);
  } else if constexpr (F == KvFmt::FP8) {
    const i32x2 c = *reinterpret_cast<const i32x2*>(page + row * 128 + col * 8);
    return __builtin_bit_cast(i32x4, fp8x8_to_bf16x8((uint32_t)c[0], (uint32_t)c[1]));
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(page + row * 64 + col * 4);
    const uint32_t e = (*reinterpret_cast<const uint32_t*>(page + 128 * 64 + row * 4) >> (8 * (col >> 2))) & 0xffu;
    const float sc = e ? __uint_as_float(e << 23) : 5.877471754111438e-39f;  // 2^(e - 127); e = 0: 2^-127
    return i32x4{__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0)),
                 __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1)),
                 __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2)),
                 __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3))};
  }
}

// The partial outputs of the sparse prefill in block floating point.  A
// record holds one (row, head, slot) partial O (128 values) as 10-bit signed
// integers n with O_d ~ step * n_d, step = 2^(E - 9) * 1024 / 1023 for the
// smallest E with max_d |O_d| < 2^E: |O_d| / step < 511.5, so |n_d| <= 511
// and the rounding error |O_d - step n_d| <= step / 2 < 2^-9 max_d |O_d| (a
// bf16 value carries up to 2^-8 of its own magnitude).  A record is 160 bytes
// against 256 in bf16: the partials are written once and read once, so this
// is 35% of the traffic of the partial attention's stores and of the merge.
// The lane holding dims d = 32 dt + 8 gq + 4 h + t (h: its MFMA lane half)
// for gq, t = 0..3 packs their 16 values, j = 4 gq + t, into one 160-bit
// group (field j at bits 10 j .. 10 j + 9, two's complement), five words;
// word w of group c = 4 h + dt is dword c of the record's 32 bytes in plane
// w.  The backward's dQ records are indexed (row * k + slot) * Hq + head and
// the forward's in fwd_rec order; in both the G heads of one (row, slot)
// entry are adjacent: for G >= 4 every store instruction of a plane writes
// whole 128-byte lines.  The step sits beside the log-sum-exp (float2).
constexpr float kBfpMagic = 12582912.0f;  // 1.5 * 2^23: x + magic keeps round(x) in the low mantissa bits

// Encodes a wave's 32 rows x 128 dims of output, held as four O^T MFMA tiles
// (oacc[dt]: C[dim][row], dims 32 dt ..; lane (row, h) holds dims 32 dt +
// 8 gq + 4 h + t in register 4 gq + t), scaled by `mul`, and stores the five
// plane words of each lane's group straight from the lanes (16 bytes per
// lane and plane) at record rec(row).  Returns the lane's row's step.
template <typename RecIndex>
__device__ __forceinline__ float store_rows_bfp10(const f32x16 (&oacc)[4], float mul, uint8_t* planes,
                                                  int64_t plane_stride, RecIndex rec, int lane) {
  const int jrow = lane & 31, half = lane >> 5;
  float amax = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; i += 2) amax = absmax3f(amax, oacc[dt][i], oacc[dt][i + 1]);
  amax = wave_max32(amax);
  // E = e - 126 for the biased exponent e of max|O|; rows below 2^-118 keep zeros
  const uint32_t e = __float_as_uint(amax * mul) >> 23;
  const bool live = e >= 9;
  const float f = live ? mul * __uint_as_float((262u - e) << 23) * (1023.f / 1024.f) : 0.f;   // 1 / step
  const float step = live ? __uint_as_float((e - 8u) << 23) * (1024.f / 1023.f) : 0.f;      // 2^(E - 9) * 1024 / 1023
  uint32_t wd[5][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    uint32_t n[16];  // low 10 bits: n in two's complement
#pragma unroll
    for (int j = 0; j < 16; ++j) n[j] = __float_as_uint(__builtin_fmaf(oacc[dt][j], f, kBfpMagic));
    // word w = group bits 32 w .. 32 w + 31: fields 3 w (from its bit 2 w) to
    // 3 w + 3 (up to its bit 9 - 2 w); each alignbit shifts the word being
    // built down and brings the next field in at the top
#pragma unroll
    for (int w = 0; w < 5; ++w) {
      const uint32_t x0 = n[3 * w] << 22;
      const uint32_t x1 = __builtin_amdgcn_alignbit(n[3 * w + 1], x0, 10);
      const uint32_t x2 = __builtin_amdgcn_alignbit(n[3 * w + 2], x1, 10);
      wd[w][dt] = __builtin_amdgcn_alignbit(n[3 * w + 3], x2, 2 + 2 * w);
    }
  }
  uint8_t* dst = planes + rec(jrow) * 32 + 16 * half;
#pragma unroll
  for (int w = 0; w < 5; ++w)
    __builtin_nontemporal_store(i32x4{(int)wd[w][0], (int)wd[w][1], (int)wd[w][2], (int)wd[w][3]},
                                reinterpret_cast<i32x4*>(dst + w * plane_stride));
  return step;
}

// The forward's partial records: 9-bit signed fields, n = round(O / step) in
// [-255, 255] with step = 2^(E-8) * 256/255 for the smallest E with max|O| <
// 2^E (|O| / step < 255).  The error, at most step / 2 < 2^-8 * max|O|, and
// the output's bf16 rounding stay inside the output tolerance even when one
// value row of size 4 carries a row's whole output (8-bit fields would not).
// Encoding is one FMA per value (adding 1.5 * 2^23 leaves n in the low
// bits).  A lane's 64 values (value j of group dt is value 16 dt + j) form
// one stream of 576 bits, value f at bits 9 f .. 9 f + 8, i.e. 18 words:
// words 0-15 in planes 0-3 (plane p: words 4 p .. 4 p + 3, 16 bytes per lane,
// 32 per record as the 10-bit form), words 16-17 in a fifth, half-width
// plane (8 bytes per lane, 16 per record) after them.  Returns the step.
constexpr int kFwdFullPlanes = 4;
// word Q of the stream: the fields that cover it, inserted at the top and
// shifted down (alignbit), the last one by the bits it has in the word
template <int Q>
__device__ __forceinline__ uint32_t bfp9_word(const uint32_t (&t)[64]) {
  constexpr int lo = 32 * Q, hi = lo + 32;
  constexpr int f0 = lo / 9, f1 = (hi - 1) / 9;
  uint32_t w = 0;
#pragma unroll
  for (int f = f0; f < f1; ++f) w = __builtin_amdgcn_alignbit(t[f], w, 9);
  return __builtin_amdgcn_alignbit(t[f1], w, hi - 9 * f1);
}
struct Rec9 {       // one record's planes as a lane of the merge holds them
  i32x4 p[4];       // words 0-15
  i32x2 x;          // words 16-17
};
template <typename RecIndex>
__device__ __forceinline__ float store_rows_bfp9(const f32x16 (&oacc)[4], float mul, uint8_t* planes,
                                                 int64_t plane_stride, RecIndex rec, int lane) {
  const int jrow = lane & 31, half = lane >> 5;
  float amax = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; i += 2) amax = absmax3f(amax, oacc[dt][i], oacc[dt][i + 1]);
  amax = wave_max32(amax);
  // E = e - 126 for the biased exponent e of max|O|; rows below 2^-119 keep zeros
  const uint32_t e = __float_as_uint(amax * mul) >> 23;
  const bool live = e >= 8;
  const float f = live ? mul * __uint_as_float((261u - e) << 23) * (255.f / 256.f) : 0.f;   // 1 / step
  const float step = live ? __uint_as_float((e - 7u) << 23) * (256.f / 255.f) : 0.f;       // 2^(E - 8) * 256 / 255
  uint32_t t[64];  // low 9 bits: n in two's complement
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) t[16 * dt + j] = __float_as_uint(__builtin_fmaf(oacc[dt][j], f, kBfpMagic));
  const int64_t r = rec(jrow);
  uint8_t* dst = planes + r * 32 + 16 * half;
  __builtin_nontemporal_store(i32x4{(int)bfp9_word<0>(t), (int)bfp9_word<1>(t), (int)bfp9_word<2>(t), (int)bfp9_word<3>(t)},
                              reinterpret_cast<i32x4*>(dst));
  __builtin_nontemporal_store(i32x4{(int)bfp9_word<4>(t), (int)bfp9_word<5>(t), (int)bfp9_word<6>(t), (int)bfp9_word<7>(t)},
                              reinterpret_cast<i32x4*>(dst + plane_stride));
  __builtin_nontemporal_store(i32x4{(int)bfp9_word<8>(t), (int)bfp9_word<9>(t), (int)bfp9_word<10>(t), (int)bfp9_word<11>(t)},
                              reinterpret_cast<i32x4*>(dst + 2 * plane_stride));
  __builtin_nontemporal_store(i32x4{(int)bfp9_word<12>(t), (int)bfp9_word<13>(t), (int)bfp9_word<14>(t), (int)bfp9_word<15>(t)},
                              reinterpret_cast<i32x4*>(dst + 3 * plane_stride));
  __builtin_nontemporal_store(i32x2{(int)bfp9_word<16>(t), (int)bfp9_word<17>(t)},
                              reinterpret_cast<i32x2*>(planes + kFwdFullPlanes * plane_stride + r * 16 + 8 * half));
  return step;
}

template <KvFmt F>
__global__ __launch_bounds__(256, 2) void partial_attn_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[128 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t vs[128 * 256];
  __shared__ int32_t ent_s[kMaxItemEntries];
  __shared__ int32_t rk_s[kMaxItemEntries];  // an entry's record, head 0 of the group (fwd_rec)
  int item = blockIdx.x;
  if (a.xcd_pin) {
    // workgroups are dealt to the 8 XCDs round-robin: XCD x = blockIdx % 8
    // runs the items of groups g = x (mod 8) (Hkv >= 8), or every (8 / Hkv)-th
    // item of group x % Hkv (Hkv < 8), so a group's gathered Q rows stay in
    // one XCD's L2
    const int x = (int)(blockIdx.x & 7), jj = (int)(blockIdx.x >> 3);
    item = -1;
    if (a.Hkv >= 8) {
      int rem = jj;
      for (int gg = x; gg < a.Hkv; gg += 8) {
        const int lo = a.gitems[gg], n = a.gitems[gg + 1] - lo;
        if (rem < n) {
          item = lo + rem;
          break;
        }
        rem -= n;
      }
    } else {
      const int per = 8 / a.Hkv, gg = x % a.Hkv;
      const int cand = a.gitems[gg] + jj * per + x / a.Hkv;
      if (cand < a.gitems[gg + 1]) item = cand;
    }
    if (item < 0) return;
  } else if (item >= *a.nitems) {
    return;
  }
  const int4 it = a.items[item];
  const int g = it.x, gb = it.y, e0 = it.z, e1 = it.w;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = upper_bound_i32(a.m.page_start, a.m.S + 1, gb) - 1;
  const int b = gb - a.m.page_start[s];
  const int32_t page = a.kv_indices[gb];
  const int32_t first_pos = a.m.kv[s] - a.m.qo[s];
  const int32_t rs = a.m.row_start[s];
  const int n_ent = e1 - e0;

  {  // K and V block -> LDS as bf16 (coalesced loads); this item's entries -> LDS
    constexpr int64_t kPageBytes = F == KvFmt::BF16 ? 32768 : F == KvFmt::FP8 ? 16384 : 128 * 64 + 128 * 4;
    const uint8_t* kb = a.kp + ((int64_t)page * a.Hkv + g) * kPageBytes;
    const uint8_t* vb = a.vp + ((int64_t)page * a.Hkv + g) * kPageBytes;
    i32x4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      kr[i] = load_kv8<F>(kb, c >> 4, c & 15);
      vr[i] = load_kv8<F>(vb, c >> 4, c & 15);
    }
    for (int i = tid; i < n_ent; i += 256) {
      const int32_t ent = a.entries[e0 + i];
      ent_s[i] = ent;
      rk_s[i] = (int32_t)fwd_rec(ent & 63, g, ent >> 6, 0, a.Hkv, a.G, a.k, a.rec_rows, a.rec_shift);
    }
    const int kv_in_block = a.m.kv[s] - b * 128;  // V rows at or past this are page padding
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      lds_store16<i32x4>(&ks[k_swz(c >> 4, c & 15)], kr[i]);
      // padding may hold anything; P is 0 there but 0 * NaN is NaN
      lds_store16<i32x4>(&vs[v_swz(c >> 4, c & 15)], (c >> 4) < kv_in_block ? vr[i] : i32x4{});
    }
  }
  __syncthreads();

  const int G = a.G;
  const int MT = 128 / G;                      // tokens per 128-row chunk
  const int qr = 32 * wave + (lane & 31);      // this lane's query row within a chunk
  const int half = lane >> 5;
  const int q16 = lane >> 4, m16 = lane & 15;
  const int hh = qr % G, tok = qr / G;
  const int h = g * G + hh;
  const int nchunks = (n_ent + MT - 1) / MT;
  // fp8 pages: logits and outputs carry the group's K and V scales
  const float scale_log2 = F == KvFmt::FP8 ? a.scale_log2 * a.ks[g] : a.scale_log2;
  const float v_scale = F == KvFmt::FP8 ? a.vs[g] : 1.f;
  // K row 32 kt + (lane & 31), column chunk 2 st + half: kbase[st] + 8192 kt
  int kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = (lane & 31) * 256 + (((2 * st + half) ^ (lane & 15)) << 4);
  // V row 32 kt + 16 u + 4 (q16 >> 1) + (m16 >> 2) (+ 8), bytes 64 dt + 32 (q16 & 1)
  // + 8 (m16 & 3): vbase[dt] + 256 (32 kt + 16 u) (+ 2048)
  int vbase[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vbase[dt] = (4 * (q16 >> 1) + (m16 >> 2)) * 256 +
                ((4 * (dt ^ (m16 >> 2)) + 2 * (q16 & 1) + ((m16 & 3) >> 1)) << 4) + 8 * (m16 & 1);

  // Q fragments (B operand) of a chunk's row for this lane: gathered rows
  auto load_q = [&](bf16x8 (&qf)[8], int chunk) {
    const int e = min(chunk * MT + tok, n_ent - 1);
    const int32_t r = a.w0 + (ent_s[e] >> 6);
    const uint8_t* qrow = a.q + ((int64_t)r * a.Hq + h) * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + st * 32);
  };

  // One 128-row chunk: S^T = K Q^T, causal mask, softmax, O^T = V^T P^T,
  // normalised bf16 partial and log-sum-exp out.
  auto process = [&](const bf16x8 (&qf)[8], int chunk) __attribute__((always_inline)) {
    const int e = chunk * MT + tok;
    const bool valid = e < n_ent;
    const int ent = ent_s[valid ? e : 0];
    const int rl = ent >> 6, slot = ent & 63;
    const int32_t pos = first_pos + (a.w0 + rl - rs);

    // S^T = K Q^T: 4 key tiles of 32
    // K fragments read one k-step ahead of the products that use them
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    bf16x8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) kf[0][kt] = lds_load16<bf16x8>(&ks[kbase[0] + 8192 * kt]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kf[(st + 1) & 1][kt] = lds_load16<bf16x8>(&ks[kbase[st + 1] + 8192 * kt]);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc[kt] = mfma32x32x16(kf[st & 1][kt], qf[st], acc[kt]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Row max on the raw scores with v_max3 (two scores per instruction),
    // then p = exp2(s * scale - max * scale) as one FMA and one exp2.  Only a
    // row's own (diagonal) block needs the causal mask: tiles whose every row
    // sees the whole block take the branch without it; the masked branch sets
    // hidden scores to -inf in place (exp2 then gives 0).
    const int lim = pos - b * 128 - 4 * half;  // last visible key offset, minus this lane's 4-key shift
    if (__builtin_amdgcn_ballot_w64(lim < 124) != 0) {  // 124 + 3: the last key offset a lane holds
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) acc[kt][i] = kNegInf;
    }
    float mraw = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mraw = max3f(mraw, acc[kt][i], acc[kt][i + 1]);
    mraw = wave_max32(mraw);
    const float mx = mraw * scale_log2;  // scaled row max (log2 domain)
    float sum = 0.f;
    bf16x8 pf[4][2];
    // P for key tile kt: p = exp2(s * scale - max), bf16 pairs, fp32 row sum
    auto make_p = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 pw;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p0 = fast_exp2(__builtin_fmaf(acc[kt][8 * u + 2 * t], scale_log2, -mx));
          const float p1 = fast_exp2(__builtin_fmaf(acc[kt][8 * u + 2 * t + 1], scale_log2, -mx));
          sum += p0 + p1;
          const bf16x2 two = {(__bf16)p0, (__bf16)p1};
          pw[t] = __builtin_bit_cast(int, two);
        }
        pf[kt][u] = __builtin_bit_cast(bf16x8, pw);
      }
    };

    // O^T = V^T P^T, software-pipelined: the exponentials of key tile kt + 1
    // are computed between the matrix products of tile kt, so that the vector
    // unit and the matrix core work at once inside the wave
    f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    make_p(0);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt + 1 < 4) make_p(kt + 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 lo = lds_read_tr16(&vs[vbase[dt] + 256 * (32 * kt + 16 * u)]);
          const s16x4 hi = lds_read_tr16(&vs[vbase[dt] + 256 * (32 * kt + 16 * u + 8)]);
          oacc[dt] = mfma32x32x16(join_tr16(lo, hi), pf[kt][u], oacc[dt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // bound the hoisting of transposed reads
    }
    sum = wave_sum32(sum);

    // Output: the normalised partials in block floating point, non-temporal
    // (the merge reads each of them once).  Padding rows write to one of
    // kTrashRecords records picked by the workgroup: with one shared record,
    // every workgroup's padding stores hit the same lines from every XCD,
    // which doubled the kernel's time on windows of many small work items.
    const int64_t trash = a.trash + (int64_t)(blockIdx.x & (kTrashRecords - 1));
    auto rec_index = [&](int wrow) -> int64_t {
      const int srow = 32 * wave + wrow;
      const int se = chunk * MT + srow / G;
      const int64_t rec = (int64_t)((uint32_t)rk_s[min(se, n_ent - 1)] + (uint32_t)(srow & (G - 1)));
      return se < n_ent ? rec : trash;
    };
    // sum >= 1 (the row max contributes exp2(0)): the hardware reciprocal's
    // 1-ulp error is far below the encoding's step
    const float step = store_rows_bfp9(oacc, v_scale * __builtin_amdgcn_rcpf(sum), a.part_pk, a.plane_stride,
                                      rec_index, lane);
    {  // both halves hold the row's max, sum and step and store the same value
      // indexed as the records: a token's G heads are adjacent, so one store
      // instruction writes G * 8 contiguous bytes per token (scattered 8-byte
      // pieces, one per line, had cost the kernel an eighth of its time)
      const int64_t pi = valid ? (int64_t)fwd_rec(slot, g, rl, hh, a.Hkv, G, a.k, a.rec_rows, a.rec_shift) : trash;
      a.part_st[pi] = float2{(mx + fast_log2(sum)) * kLn2, step};  // mx is already scaled
    }
  };

  // Two register buffers of gathered Q rows: the next chunk's loads are
  // issued before the current chunk's work, a whole chunk ahead of their use.
  // Every chunk issues the same loads (past the end they repeat the last
  // chunk) and the same stores (padding rows go to the trash slot), so the
  // compiler's wait counts stay exact and never wait for the prefetch.
  bf16x8 qa[8], qb[8];
  load_q(qa, 0);
  wait_vmem();  // nothing in flight on entering the loop
  for (int chunk = 0; chunk < nchunks; chunk += 2) {
    load_q(qb, min(chunk + 1, nchunks - 1));
    __builtin_amdgcn_sched_barrier(0);
    process(qa, chunk);
    __builtin_amdgcn_sched_barrier(0);
    if (chunk + 1 >= nchunks) break;
    load_q(qa, min(chunk + 2, nchunks - 1));
    __builtin_amdgcn_sched_barrier(0);
    process(qb, chunk + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The local block of every row inside the merge.  Each row's own
// (diagonal) block is computed here rather than as a slot of partial_attn:
// one workgroup per (KV group, block, 128 rows of the block's own query rows
// x G heads), whose Q rows are contiguous (no gather) and whose key tiles
// past a wave's last row are skipped.  The row's other slots' partial
// records (bfp) are summed first, against their own maximum log-sum-exp,
// while the block's K and V rows land in LDS; the local block comes last,
// its weight folded into its P, and its products add onto the slots' sum.
// A lane holds the dims of its row that store_rows_bfp10 packed from the
// same lane position, so a slot's record is one 16-byte load per plane.
struct LocalMergeArgs {
  const uint8_t* q;      // bf16 [T, Hq, 128]
  const uint8_t* kp;     // K / V pages (format F)
  const uint8_t* vp;
  const float* ks;       // fp8: [Hkv] scales, else null
  const float* vs;
  const int32_t* kv_indices;
  const int32_t* sel;    // [T, Hkv, k]
  DevMeta m;
  const uint8_t* part_pk;  // partial_attn's records and their {lse, step}
  int64_t plane_stride;
  const float2* part_st;
  int32_t rec_rows, rec_shift;  // record index (fwd_rec)
  uint16_t* out;         // bf16 [T, Hq, 128]
  float* lse;            // [T, Hq] or null
  int32_t Hq, Hkv, G, k, w0, w1;
  int32_t key0;          // first (block, group) key of the launch: block * Hkv
  float scale_log2;      // sm_scale * log2(e)
};

template <KvFmt F>
__global__ __launch_bounds__(256, 2) void local_merge_kernel(LocalMergeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[128 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t vs[128 * 256];
  constexpr int kBatch = 16;
  __shared__ float ws_s[kBatch * 256];           // slot weights, [slot][thread]: each lane its own
  const int G = a.G;
  // workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8):
  // XCD x takes the x-th eighth of the launch's (block, group) keys, so that
  // the G workgroups of a key share its K/V in one L2 and each XCD streams
  // a contiguous range of records, query rows and output rows
  const uint32_t nwg = gridDim.x, bid = blockIdx.x;
  const int wid = (int)(nwg % 8 == 0 ? (bid % 8) * (nwg / 8) + bid / 8 : bid);
  const int c = wid % G;                         // which 128 of the block's rows x G heads
  const int key = a.key0 + wid / G;
  const int gb = key / a.Hkv, g = key % a.Hkv;
  const int s = upper_bound_i32(a.m.page_start, a.m.S + 1, gb) - 1;
  const int b = gb - a.m.page_start[s];
  const int32_t first_pos = a.m.kv[s] - a.m.qo[s];
  const int32_t rs = a.m.row_start[s];
  // the block's keys b*128 + t that are query rows of this window
  const int32_t p_lo = max(max(b * 128, first_pos), first_pos + (a.w0 - rs));
  const int32_t p_hi = min(min(b * 128 + 128, a.m.kv[s]), first_pos + (a.w1 - rs));
  const int MT = 128 / G;                        // tokens per 128 rows
  const int32_t t0 = p_lo - b * 128 + c * MT;    // this workgroup's first token
  const int32_t t_hi = p_hi - b * 128;
  if (t0 >= t_hi) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t page = a.kv_indices[gb];
  // K and V of the block -> LDS as bf16 (as partial_attn): the 16-key passes
  // that the workgroup's last row sees
  {
    constexpr int64_t kPageBytes = F == KvFmt::BF16 ? 32768 : F == KvFmt::FP8 ? 16384 : 128 * 64 + 128 * 4;
    const uint8_t* kb = a.kp + ((int64_t)page * a.Hkv + g) * kPageBytes;
    const uint8_t* vb = a.vp + ((int64_t)page * a.Hkv + g) * kPageBytes;
    const int passes = 2 * ((min(t0 + MT, t_hi) - 1) / 32 + 1);
    const int kv_in_block = a.m.kv[s] - b * 128;  // rows at or past this are page padding
    if constexpr (F == KvFmt::BF16) {
      // straight from global memory (untracked direct loads, waited for
      // before the local block's products, after the merge): one wave
      // instruction fills 4 rows; lane l physical chunk l % 16 of row
      // 4 i + l / 16, i.e. fetches the logical chunk the swizzle puts there.
      // Page padding rows fetch the block's last key row instead (finite;
      // every query row's mask hides them).
      for (int i = wave; i < 4 * passes; i += 4) {
        const int krow = 4 * i + (lane >> 4), pc = lane & 15;
        const int srow = min(krow, kv_in_block - 1);
        global_load_lds16_untracked(kb + srow * 256 + ((pc ^ (krow & 15)) << 4), (MSA_LDS void*)(ks + 1024 * i));
        global_load_lds16_untracked(vb + srow * 256 + ((pc ^ ((krow & 3) << 2)) << 4), (MSA_LDS void*)(vs + 1024 * i));
      }
    } else {  // widened to bf16 on the way (through registers)
      i32x4 kr[8], vr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < passes) {
          const int cc = tid + 256 * i;
          kr[i] = load_kv8<F>(kb, cc >> 4, cc & 15);
          vr[i] = load_kv8<F>(vb, cc >> 4, cc & 15);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < passes) {
          const int cc = tid + 256 * i;
          lds_store16<i32x4>(&ks[k_swz(cc >> 4, cc & 15)], kr[i]);
          lds_store16<i32x4>(&vs[v_swz(cc >> 4, cc & 15)], (cc >> 4) < kv_in_block ? vr[i] : i32x4{});
        }
      }
    }
  }
  const int half = lane >> 5;
  const int qr = 32 * wave + (lane & 31);        // this lane's row within the 128
  const int hh = qr % G;
  const int32_t t = t0 + qr / G;
  const bool row_ok = t < t_hi;
  const int32_t tt = row_ok ? t : t_hi - 1;     // padding lanes repeat the last row (nothing stored)
  const int32_t r = rs + (b * 128 + tt - first_pos);
  const int h = g * G + hh;
  const float scale_log2 = F == KvFmt::FP8 ? a.scale_log2 * a.ks[g] : a.scale_log2;
  const float v_scale = F == KvFmt::FP8 ? a.vs[g] : 1.f;
  // Q fragments: requested now, used by the local block's products last
  bf16x8 qf[8];
  {
    const uint8_t* qrow = a.q + ((int64_t)r * a.Hq + h) * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + st * 32);
  }

  // The row's other slots first (blocks 0 <= blk < b; the local block is b),
  // against their own maximum Ms: oacc = sum_s w_s n_s step_s with
  // w_s = exp(lse_s - Ms), Ls = sum_s w_s.  Their {lse, step}, 16 slots per
  // batch of loads; each slot's weight goes to LDS ([slot][thread]) and the
  // records are added one slot after another, each loaded three slots ahead.
  // A slot that holds no record weighs 0: its stats may hold anything, NaN
  // too, and are not read into the result; its (unwritten) record is
  // integers, always finite, and adds exactly 0.
  const int32_t rl = r - a.w0;
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  // {lse, step} of slot j: indexed as the records, Hkv tr G records apart
  // (tr: the rows of the row's record tile)
  const uint32_t rec0 = fwd_rec(0, g, rl, hh, a.Hkv, G, a.k, a.rec_rows, a.rec_shift);
  const uint32_t rec_slot = fwd_rec(1, g, rl, hh, a.Hkv, G, a.k, a.rec_rows, a.rec_shift) - rec0;
  const float2* st_row = a.part_st + rec0;
  // with k a multiple of 4 (and the selection 16-byte aligned) the row of
  // block ids goes in 16-byte pieces
  const bool vec_blk = (a.k & 3) == 0 && (reinterpret_cast<uintptr_t>(a.sel) & 15) == 0;
  auto load_stats = [&](int s0, int (&blk)[kBatch], float2 (&ls)[kBatch]) {
    if (vec_blk) {
#pragma unroll
      for (int j = 0; j < kBatch; j += 4) {
        const i32x4 bv = *reinterpret_cast<const i32x4*>(row + min(s0 + j, a.k - 4));
        const bool in = s0 + j < a.k;  // then all four are
#pragma unroll
        for (int q = 0; q < 4; ++q) blk[j + q] = in ? bv[q] : -1;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) blk[j] = s0 + j < a.k ? row[min(s0 + j, a.k - 1)] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) ls[j] = st_row[(uint32_t)min(s0 + j, a.k - 1) * rec_slot];
  };
  // a plane holds under 2^32 bytes (the plan caps the window): one 32-bit
  // offset per slot serves the planes' uniform bases (the fifth, half-width
  // plane at half the offset)
  const uint8_t* const plane0 = a.part_pk;
  const uint8_t* const plane1 = plane0 + a.plane_stride;
  const uint8_t* const plane2 = plane1 + a.plane_stride;
  const uint8_t* const plane3 = plane2 + a.plane_stride;
  const uint8_t* const plane4 = plane3 + a.plane_stride;
  auto rec_load = [&](int slot, Rec9& w) {
    const uint32_t rec = rec0 + (uint32_t)slot * rec_slot;
    const uint32_t off = rec * 32u + 16u * half;
    w.p[0] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(plane0 + off));
    w.p[1] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(plane1 + off));
    w.p[2] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(plane2 + off));
    w.p[3] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(plane3 + off));
    w.x = __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(plane4 + (off >> 1)));
  };
  float Ms = kNegInf;
  int blk0[kBatch];
  float2 ls0[kBatch];
  load_stats(0, blk0, ls0);
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (blk0[j] >= 0 && blk0[j] < b) Ms = fmaxf(Ms, ls0[j].x);
  for (int s0 = kBatch; s0 < a.k; s0 += kBatch) {
    int blk[kBatch];
    float2 ls[kBatch];
    load_stats(s0, blk, ls);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (blk[j] >= 0 && blk[j] < b) Ms = fmaxf(Ms, ls[j].x);
  }
  float Ls = 0.f;
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  // value j of group dt: bits 9 f .. of the lane's 576-bit stream, f = 16 dt
  // + j (store_rows_bfp9); a signed bit-field extract, after one alignbit
  // for the values that straddle two words
  auto word = [&](const Rec9& w, int q) -> uint32_t { return q < 16 ? (uint32_t)w.p[q >> 2][q & 3] : (uint32_t)w.x[q - 16]; };
  auto field = [&](const Rec9& w, int dt, int j) -> float {
    const int bit = 9 * (16 * dt + j), q = bit >> 5, o = bit & 31;
    const uint32_t x0 = word(w, q);
    if (o <= 23) return (float)((int)(x0 << (23 - o)) >> 23);
    return (float)((int)(__builtin_amdgcn_alignbit(word(w, q + 1), x0, o) << 23) >> 23);
  };
  auto add_rec = [&](const Rec9& w, float ws) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[dt][j] = __builtin_fmaf(ws, field(w, dt, j), oacc[dt][j]);
  };
  auto put_weights = [&](const int (&blk)[kBatch], const float2 (&ls)[kBatch]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = blk[j] >= 0 && blk[j] < b;
      const float w = in ? fast_exp2((ls[j].x - Ms) * kLog2e) : 0.f;
      Ls += w;
      ws_s[j * 256 + tid] = in ? w * ls[j].y : 0.f;  // this lane's own slot weights
    }
  };
  Rec9 rb[4];  // records of four consecutive slots, slot j in rb[j % 4]
  rec_load(0, rb[0]);
  put_weights(blk0, ls0);
  for (int s0 = 0; s0 < a.k; s0 += kBatch) {
    if (s0 > 0) {
      int blk[kBatch];
      float2 ls[kBatch];
      load_stats(s0, blk, ls);
      put_weights(blk, ls);
      rec_load(s0, rb[0]);
    }
    // the batch's slots padded to a multiple of 4: a padding slot re-reads
    // slot k - 1's record and weighs 0 (put_weights), so every load of the
    // ring is unconditional and stays in flight across the loop
    const int n4 = (min(kBatch, a.k - s0) + 3) & ~3;  // the same in every lane
#pragma unroll
    for (int u = 1; u < 4; ++u) rec_load(min(s0 + u, a.k - 1), rb[u]);
    // (the scheduler would otherwise hoist later slots' decoding, and with it
    // their waits, above the earlier slots' adds)
    int j = 0;
    for (; j + 4 < n4; j += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        add_rec(rb[u], ws_s[(j + u) * 256 + tid]);
        rec_load(min(s0 + j + u + 4, a.k - 1), rb[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      add_rec(rb[u], ws_s[(j + u) * 256 + tid]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The local block, into the same accumulators.  Its K and V rows are in
  // LDS (each wave waits for its own direct loads, the barrier for
  // everyone's; for the register path the barrier orders the stores).
  if constexpr (F == KvFmt::BF16) wait_vmem();
  __syncthreads();
  const int q16 = lane >> 4, m16 = lane & 15;
  int kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = (lane & 31) * 256 + (((2 * st + half) ^ (lane & 15)) << 4);
  int vbase[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vbase[dt] = (4 * (q16 >> 1) + (m16 >> 2)) * 256 +
                ((4 * (dt ^ (m16 >> 2)) + 2 * (q16 & 1) + ((m16 & 3) >> 1)) << 4) + 8 * (m16 & 1);
  // key tiles holding a visible key of some row of the wave: its rows are
  // consecutive tokens, the last one sees keys 0 .. its t
  int tmax = tt;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) tmax = max(tmax, __shfl_xor(tmax, o));
  const int nkt = __builtin_amdgcn_readfirstlane(min(4, (tmax >> 5) + 1));  // the same in every lane
  const int lim = tt - 4 * half;                 // last visible key offset, minus the lane's 4-key shift

  // S^T = K Q^T on the live tiles; K fragments one k-step ahead
  f32x16 acc[4];
  {
    bf16x8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      if (kt < nkt) kf[0][kt] = lds_load16<bf16x8>(&ks[kbase[0] + 8192 * kt]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          if (kt < nkt) kf[(st + 1) & 1][kt] = lds_load16<bf16x8>(&ks[kbase[st + 1] + 8192 * kt]);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        if (kt < nkt) acc[kt] = mfma32x32x16(kf[st & 1][kt], qf[st], st == 0 ? f32x16{} : acc[kt]);
    }
  }
  // causal mask (hidden scores -inf), row max, p = exp2(s * scale - max) in place
  float mraw = kNegInf;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    if (kt < nkt) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) acc[kt][i] = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; i += 2) mraw = max3f(mraw, acc[kt][i], acc[kt][i + 1]);
    }
  mraw = wave_max32(mraw);
  const float mx = mraw * scale_log2;
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    if (kt < nkt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[kt][i] = fast_exp2(__builtin_fmaf(acc[kt][i], scale_log2, -mx));
        sum += acc[kt][i];
      }
    }
  sum = wave_sum32(sum);  // >= 1: the row max contributes exp2(0)
  // weights: the slots' exp(Ms - M), the local block's exp(lse_loc - M) / sum
  // (folded into its P before the bf16 rounding, with fp8's V scale)
  const float lse_loc = (mx + fast_log2(sum)) * kLn2;  // natural log
  const float M = fmaxf(Ms, lse_loc);
  const float alpha = fast_exp2((Ms - M) * kLog2e);    // 0 without a counted slot
  const float beta = fast_exp2((lse_loc - M) * kLog2e);
  const float L = Ls * alpha + beta;
  const float f_loc = v_scale * beta / sum;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
  // O^T += V^T P^T on the live tiles
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    if (kt < nkt) {
      bf16x8 pf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 pw;
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
          const bf16x2 two = {(__bf16)(acc[kt][8 * u + 2 * tq] * f_loc), (__bf16)(acc[kt][8 * u + 2 * tq + 1] * f_loc)};
          pw[tq] = __builtin_bit_cast(int, two);
        }
        pf[u] = __builtin_bit_cast(bf16x8, pw);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 lo = lds_read_tr16(&vs[vbase[dt] + 256 * (32 * kt + 16 * u)]);
          const s16x4 hi = lds_read_tr16(&vs[vbase[dt] + 256 * (32 * kt + 16 * u + 8)]);
          oacc[dt] = mfma32x32x16(join_tr16(lo, hi), pf[u], oacc[dt]);
        }
      }
    }
  }
  if (!row_ok) return;
  const float inv = 1.f / L;
  // lane (row, half): dims 32 dt + 8 gq + 4 half + tq in register 4 gq + tq
  uint16_t* orow = a.out + ((int64_t)r * a.Hq + h) * 128;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const bf16x2 t0v = {(__bf16)(oacc[dt][4 * gq] * inv), (__bf16)(oacc[dt][4 * gq + 1] * inv)};
      const bf16x2 t1v = {(__bf16)(oacc[dt][4 * gq + 2] * inv), (__bf16)(oacc[dt][4 * gq + 3] * inv)};
      *reinterpret_cast<i32x2*>(orow + 32 * dt + 8 * gq + 4 * half) =
          i32x2{__builtin_bit_cast(int, t0v), __builtin_bit_cast(int, t1v)};
    }
  if (a.lse && half == 0) a.lse[(int64_t)r * a.Hq + h] = M + fast_log2(L) * kLn2;
}

// Reading a record 8 lanes at a time: lane l takes dword l of each of the
// record's five planes, group l of store_rows_bfp10: dims 32 dt + 8 gq + 4 h
// + t for h = l / 4, dt = l % 4 and gq, t = 0..3.  Decoding: a field inside
// one word is a signed bit-field extract, the four that straddle two words
// first join them with one alignbit.
constexpr int kMergeLanes = 8;

struct BfpRec {
  uint32_t w[5];
};

__device__ __forceinline__ BfpRec load_bfp_rec(const uint8_t* planes, int64_t plane_stride, int64_t rec, int l) {
  BfpRec r;
  const uint8_t* src = planes + rec * 32 + 4 * l;
#pragma unroll
  for (int w = 0; w < 5; ++w) r.w[w] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src + w * plane_stride));
  return r;
}

// field j (0..15) of a group: n, from its bits 10 j .. 10 j + 9
__device__ __forceinline__ float bfp_field(const BfpRec& r, int j) {
  const int bit = 10 * j, q = bit >> 5, o = bit & 31;
  if (o <= 22) return (float)((int)(r.w[q] << (22 - o)) >> 22);
  return (float)((int)(__builtin_amdgcn_alignbit(r.w[q + 1], r.w[q], o) << 22) >> 22);
}


}  // namespace

namespace {

// Invert kv_block_indexes for rows [w0, w1) into per-(group, block) entry
// lists (counts, offsets, entries) and the capped work items.
// Canonical order within each (group, block) bin: ascending window row (a row
// enters a bin at most once).  The fill pass places entries in the order its
// atomics land; the forward does not care (one partial per entry), but the
// backward's dk/dv sum a bin's rows in entry order, and this order makes those
// gradients bit-reproducible.  Per bin: the rows go into an LDS bitmap over the
// window (their slots into a byte per row), a prefix of the words' popcounts
// ranks them, and each entry is written back at its rank.  Dynamic LDS:
// W / 8 bytes of bitmap, then W slot bytes.
constexpr int kOrderThreads = 256;
constexpr int kOrderMaxRows = 65536;    // windows up to this many rows are ordered
__global__ __launch_bounds__(kOrderThreads) void csr_order_kernel(const int32_t* offsets, int32_t* entries,
                                                                 int32_t W) {
  extern __shared__ uint32_t bits[];
  __shared__ int32_t wsum[kOrderThreads / 64];
  uint8_t* slot_of = reinterpret_cast<uint8_t*>(bits + (W + 31) / 32);
  const int32_t e0 = offsets[blockIdx.x], n = offsets[blockIdx.x + 1] - e0;
  if (n <= 1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (W + 31) / 32;
  for (int i = tid; i < nw; i += kOrderThreads) bits[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kOrderThreads) {
    const int32_t e = entries[e0 + i];
    atomicOr(&bits[(e >> 6) >> 5], 1u << ((e >> 6) & 31));
    slot_of[e >> 6] = (uint8_t)(e & 63);
  }
  __syncthreads();
  // thread t owns words [t * per, (t + 1) * per); exclusive prefix of their popcounts
  const int per = (nw + kOrderThreads - 1) / kOrderThreads;
  const int w_lo = min(nw, tid * per), w_hi = min(nw, w_lo + per);
  int cnt = 0;
  for (int w = w_lo; w < w_hi; ++w) cnt += __popc(bits[w]);
  int incl = cnt;   // inclusive scan within the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - cnt;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  for (int w = w_lo; w < w_hi; ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      const int32_t rl = 32 * w + b;
      entries[e0 + base++] = (rl << 6) | slot_of[rl];
    }
  }
}

void build_csr(const msa_plan_s* p, const DevMeta& m, const int32_t* sel, char* ws, int32_t w0, int32_t w1,
               hipStream_t st, bool sorted, bool with_local) {
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
  {
  ProfEvents pe(p, "csr");
  hipExtLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<int64_t>(1024, (nclear + 255) / 256)), dim3(256), 0,
                        st, pe.start, nullptr, 0, counts, nclear, 0);
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
  c.with_local = with_local ? 1 : 0;
  const dim3 cgrid((unsigned)((w1 - w0 + 255) / 256), (unsigned)Hkv);
  const bool lds_hist = p->NB <= kMaxLdsBins;
  const size_t hist_bytes = lds_hist ? (size_t)p->NB * 4 : 0;
  if (lds_hist) hipLaunchKernelGGL((csr_pass_kernel<false, true>), cgrid, dim3(256), hist_bytes, st, c);
  else hipLaunchKernelGGL((csr_pass_kernel<false, false>), cgrid, dim3(256), 0, st, c);
  int32_t* gitems = reinterpret_cast<int32_t*>(ws + L.gitems);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, counts, offsets, items, nitems, gitems, nkey,
                     p->NB, p->entries_per_item);
  const bool order = sorted && w1 - w0 <= kOrderMaxRows;   // longer windows keep the fill order
  hipEvent_t fill_stop = order ? nullptr : pe.stop;
  if (lds_hist) hipExtLaunchKernelGGL((csr_pass_kernel<true, true>), cgrid, dim3(256), hist_bytes, st, nullptr, fill_stop, 0, c);
  else hipExtLaunchKernelGGL((csr_pass_kernel<true, false>), cgrid, dim3(256), 0, st, nullptr, fill_stop, 0, c);
  if (order) {
    const int32_t W = w1 - w0;
    const size_t lds = (size_t)(W + 31) / 32 * 4 + (size_t)W;
    hipExtLaunchKernelGGL(csr_order_kernel, dim3((unsigned)nkey), dim3(kOrderThreads), lds, st, nullptr, pe.stop, 0,
                          offsets, entries, W);
  }
  }

}

}  // namespace

hipError_t launch_prefill_window(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp,
                                 const void* vp, const float* ks, const float* vs, const int32_t* kv_indices,
                                 const int32_t* sel, void* out, float* lse, char* ws, int32_t w0, int32_t w1,
                                 hipStream_t st) {
  const PlanLayout& L = p->lay;
  const int Hkv = p->d.num_kv_heads, Hq = p->d.num_qo_heads, k = p->d.topk;
  const int32_t nkey = Hkv * p->NB;
  const int32_t* entries = reinterpret_cast<const int32_t*>(ws + L.entries);
  const int4* items = reinterpret_cast<const int4*>(ws + L.items);
  const int32_t* nitems = reinterpret_cast<const int32_t*>(ws + L.nitems);
  // a row's own block is computed by local_merge_kernel, not as an entry
  build_csr(p, m, sel, ws, w0, w1, st, /*sorted=*/false, /*with_local=*/false);

  PartialArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.kp = static_cast<const uint8_t*>(kp);
  a.vp = static_cast<const uint8_t*>(vp);
  a.ks = ks;
  a.vs = vs;
  a.kv_indices = kv_indices;
  a.entries = entries;
  a.items = items;
  a.nitems = nitems;
  a.gitems = reinterpret_cast<const int32_t*>(ws + L.gitems);
  a.xcd_pin = p->xcd_pin && (Hkv % 8 == 0 || 8 % Hkv == 0);
  a.m = m;
  // the partial records' planes share the region the backward uses for its
  // dQ partials (168 bytes per record; the forward needs 152)
  a.trash = p->attn_window * Hq * k;
  a.rec_rows = (int32_t)p->attn_window;
  a.rec_shift = __builtin_ctz((unsigned)(128 / p->G));
  const int64_t nrec = a.trash + kTrashRecords;
  a.part_pk = reinterpret_cast<uint8_t*>(ws + L.part_o);
  a.plane_stride = nrec * 32;
  // after the four full planes, the half-width fifth (16 bytes per record)
  a.part_st = reinterpret_cast<float2*>(a.part_pk + kFwdFullPlanes * a.plane_stride + nrec * 16);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p->G;
  a.k = k;
  a.w0 = w0;
  a.scale_log2 = p->d.sm_scale * kLog2e;
  // upper bound on the number of work items of this window
  const int64_t max_items = ((int64_t)(w1 - w0) * Hkv * k + p->entries_per_item - 1) / p->entries_per_item + nkey;
  // pinned: 8 x a bound on one XCD's items (a group has at most W k / epi + NB)
  const int64_t group_items = ((int64_t)(w1 - w0) * k + p->entries_per_item - 1) / p->entries_per_item + p->NB;
  const int64_t grid_items = !a.xcd_pin ? max_items
                             : Hkv >= 8 ? 8 * (Hkv / 8) * group_items
                                        : 8 * ((group_items + 8 / Hkv - 1) / (8 / Hkv));
  {
    ProfEvents pe(p, "partial_attn");
    const dim3 grid((unsigned)grid_items), blk(256);
    if (p->d.kv_dtype == MSA_MXFP4)
      hipExtLaunchKernelGGL(partial_attn_kernel<KvFmt::MX4>, grid, blk, 0, st, pe.start, pe.stop, 0, a);
    else if (p->d.kv_dtype == MSA_FP8_E4M3)
      hipExtLaunchKernelGGL(partial_attn_kernel<KvFmt::FP8>, grid, blk, 0, st, pe.start, pe.stop, 0, a);
    else
      hipExtLaunchKernelGGL(partial_attn_kernel<KvFmt::BF16>, grid, blk, 0, st, pe.start, pe.stop, 0, a);
  }

  LocalMergeArgs mg;
  mg.q = a.q;
  mg.kp = a.kp;
  mg.vp = a.vp;
  mg.ks = ks;
  mg.vs = vs;
  mg.kv_indices = kv_indices;
  mg.sel = sel;
  mg.m = m;
  mg.part_pk = a.part_pk;
  mg.plane_stride = a.plane_stride;
  mg.part_st = a.part_st;
  mg.rec_rows = a.rec_rows;
  mg.rec_shift = a.rec_shift;
  mg.out = static_cast<uint16_t*>(out);
  mg.lse = lse;
  mg.Hq = Hq;
  mg.Hkv = Hkv;
  mg.G = p->G;
  mg.k = k;
  mg.w0 = w0;
  mg.w1 = w1;
  mg.scale_log2 = a.scale_log2;
  {
    // one workgroup per (block, group, 128 of the block's rows x G heads)
    // over the blocks that hold the window's rows: rows go sequence by
    // sequence and position by position, so those blocks are the global
    // blocks gb(w0) .. gb(w1 - 1)
    auto gb_of_row = [&](int32_t r) {
      const int sq = (int)(std::upper_bound(p->row_start.begin(), p->row_start.end(), r) - p->row_start.begin()) - 1;
      return p->page_start[sq] + (p->kv[sq] - p->qo[sq] + (r - p->row_start[sq])) / 128;
    };
    const int32_t gb_lo = gb_of_row(w0), gb_hi = gb_of_row(w1 - 1);
    mg.key0 = gb_lo * Hkv;
    ProfEvents pe(p, "merge");
    const dim3 grid((unsigned)((int64_t)(gb_hi - gb_lo + 1) * Hkv * p->G)), blk(256);
    if (p->d.kv_dtype == MSA_MXFP4)
      hipExtLaunchKernelGGL(local_merge_kernel<KvFmt::MX4>, grid, blk, 0, st, pe.start, pe.stop, 0, mg);
    else if (p->d.kv_dtype == MSA_FP8_E4M3)
      hipExtLaunchKernelGGL(local_merge_kernel<KvFmt::FP8>, grid, blk, 0, st, pe.start, pe.stop, 0, mg);
    else
      hipExtLaunchKernelGGL(local_merge_kernel<KvFmt::BF16>, grid, blk, 0, st, pe.start, pe.stop, 0, mg);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward: gradients of the attention above for training, over the same
// cached selection (the Flash-MSA article: block indexes are computed once in
// the forward pass and reused, so everything but the proxy pass stays linear
// in the cached blocks).  With P the softmax of a row over its keys, L its
// log-sum-exp (from the forward) and dO the upstream gradient:
//   D = <dO, O>;  dP = dO V^T;  dS = P (dP - D)
//   dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO
// in two kernels that reuse the forward's layouts:
//  * bwd_dq (row-centric, per work item): S^T = K Q^T, P^T = exp2(S^T
//    scale_log2 - L log2 e), dP^T = V dO^T, dS^T, then dQ^T = K^T dS^T with
//    K^T read transposed from LDS (the forward's V^T P^T step); a bf16 dQ
//    partial per (row, head, slot), summed over slots by bwd_dq_sum;
//  * bwd_dkv (key-centric, one workgroup per (group, block) over all its
//    rows): wave w owns keys 32w..32w+31; S = Q K^T and dP = dO V^T put the
//    keys on lanes, so P and dS are directly the A operands of
//    dV += P^T dO and dK += dS^T Q, whose dO and Q operands are read
//    transposed from LDS.
// S and dP are computed in both kernels (7 products instead of 5): each
// kernel then needs no layout exchange of P or dS between waves.
namespace {

struct PrepArgs {
  const uint16_t* out;    // bf16 [T, Hq, 128]
  const uint16_t* dout;
  float* D;               // [W, Hq]
  int32_t w0, w1, Hq;
};

// D = <dO, O> per (row, head): 16 lanes per pair, 8 columns each.
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepArgs a) {
  const int sub = threadIdx.x & 15;
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = idx < (int64_t)(a.w1 - a.w0) * a.Hq;   // shuffles need every lane
  const int64_t id = live ? idx : 0;
  const int64_t off = ((int64_t)a.w0 * a.Hq + id) * 128 + 8 * sub;
  const i32x4 o = *reinterpret_cast<const i32x4*>(a.out + off);
  const i32x4 g = *reinterpret_cast<const i32x4*>(a.dout + off);
  float acc = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    acc += __builtin_bit_cast(float, (uint32_t)o[x] << 16) * __builtin_bit_cast(float, (uint32_t)g[x] << 16);
    acc += __builtin_bit_cast(float, (uint32_t)o[x] & 0xffff0000u) * __builtin_bit_cast(float, (uint32_t)g[x] & 0xffff0000u);
  }
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) acc += __shfl_xor(acc, sh, 16);
  if (live && sub == 0) a.D[id] = acc;
}

struct BwdDqArgs {
  const uint8_t* q;       // bf16 [T, Hq, 128]
  const uint8_t* dout;
  const uint8_t* kp;      // bf16 [N, Hkv, 128, 128]
  const uint8_t* vp;
  const float* lse;       // [T, Hq], natural log
  const float* D;         // [W, Hq]
  const int32_t* kv_indices;
  const int32_t* entries;
  const int4* items;
  const int32_t* nitems;
  DevMeta m;
  uint8_t* part_pk;       // dQ partials, block floating point (store_rows_bfp10): five planes of
  int64_t plane_stride;   //   32 bytes per record [W, k, Hq] + trash records, this far apart
  float* part_step;       //   each record's step, indexed as the records (then the trash entries)
  int64_t trash;          // index of the first of kTrashRecords trash records
  int32_t Hq, Hkv, G, k, w0;
  float scale_log2, sm_scale;
  // proxy distillation term (KL kernels only): proxy K pool bf16 [N, Hkv,
  // 128, 128] and per-(token, group, slot) partials bf16 [W, Hkv, k, 128] of
  // (1/G) sum over the group's heads h of sum_j P_hj pk_j
  const uint8_t* pkp;
  uint16_t* klpart;
  float inv_g;
};

// K sits in LDS once (rt_swz): read directly as the S^T operand and with
// transposed reads (addresses ktlo / kthi below) as K^T; each 128-key block is
// taken in two 64-key halves, so that the plain variant fits two workgroups
// per CU (74 KB of LDS, 256 registers).
template <bool KL>
__global__ __launch_bounds__(256, KL ? 1 : 2) void bwd_dq_kernel(BwdDqArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[128 * 256];   // K, rt_swz: S^T operand and K^T reads
  __shared__ __attribute__((aligned(16))) uint8_t vs[128 * 256];   // V, rt_swz: dP^T operand
  __shared__ __attribute__((aligned(16))) uint8_t pkt[KL ? 128 * 256 : 16];   // proxy K, v_swz
  __shared__ int32_t ent_s[kMaxItemEntries];
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
  const int n_ent = e1 - e0;
  {  // K and V -> LDS; padding rows (past kv_len) zeroed: dS and P are 0 there but 0 * NaN is NaN
    const uint8_t* kb = a.kp + ((int64_t)page * a.Hkv + g) * 32768;
    const uint8_t* vb = a.vp + ((int64_t)page * a.Hkv + g) * 32768;
    i32x4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      kr[i] = *reinterpret_cast<const i32x4*>(kb + c * 16);
      vr[i] = *reinterpret_cast<const i32x4*>(vb + c * 16);
    }
    for (int i = tid; i < n_ent; i += 256) ent_s[i] = a.entries[e0 + i];
    const int kv_in_block = a.m.kv[s] - b * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const bool live_row = (c >> 4) < kv_in_block;
      lds_store16<i32x4>(&ks[rt_swz(c >> 4, c & 15)], live_row ? kr[i] : i32x4{});
      lds_store16<i32x4>(&vs[rt_swz(c >> 4, c & 15)], live_row ? vr[i] : i32x4{});
    }
    if constexpr (KL) {
      const uint8_t* pb = a.pkp + ((int64_t)page * a.Hkv + g) * 32768;
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const i32x4*>(pb + (tid + 256 * i) * 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = tid + 256 * i;
        lds_store16<i32x4>(&pkt[v_swz(c >> 4, c & 15)], (c >> 4) < kv_in_block ? kr[i] : i32x4{});
      }
    }
  }
  __syncthreads();

  const int G = a.G;
  const int MT = 128 / G;
  const int qr = 32 * wave + (lane & 31);
  const int half = lane >> 5;
  const int q16 = lane >> 4, m16 = lane & 15;
  const int hh = qr % G, tok = qr / G;
  const int h = g * G + hh;
  const int nchunks = (n_ent + MT - 1) / MT;
  int kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = rt_swz((lane & 31), 2 * st + half);
  int vbase[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vbase[dt] = (4 * (q16 >> 1) + (m16 >> 2)) * 256 +
                ((4 * (dt ^ (m16 >> 2)) + 2 * (q16 & 1) + ((m16 & 3) >> 1)) << 4) + 8 * (m16 & 1);
  // transposed reads of the rt_swz tile: lane (q16, m16) fetches dims
  // 32 dt + 16 (q16 & 1) + 4 (m16 & 3) .. +3 of key row r0 (lo) or r0 + 8
  // (hi), r0 = 4 (q16 >> 1) + m16 / 4 (+ the 16-row offsets of the reads)
  int ktlo[4], kthi[4];
  {
    const int r0 = 4 * (q16 >> 1) + (m16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int c = 4 * dt + 2 * (q16 & 1) + ((m16 & 3) >> 1);
      ktlo[dt] = rt_swz(r0, c) + 8 * (m16 & 1);
      kthi[dt] = rt_swz(r0 + 8, c) + 8 * (m16 & 1);
    }
  }

  // The row of a chunk: padding rows (past the item's entries) repeat a real
  // one; their output is discarded.  Each wave's rows come from global memory
  // straight into registers: the next chunk's q rows are loaded once this
  // chunk's S^T is issued, its dO rows once dP^T is, its lse and D early.
  auto entry_at = [&](int chunk) { return ent_s[min(chunk * MT + tok, max(n_ent - 1, 0))]; };
  auto q_ptr = [&](const uint8_t* base, int ent) {
    return base + ((int64_t)(a.w0 + (ent >> 6)) * a.Hq + h) * 256 + half * 16;
  };
  bf16x8 qf[8], df[8];
  float l2 = 0.f, dval = 0.f;
  int ent = 0;
  // (lse and D are issued first, so that they are the oldest loads in flight
  // wherever the loop waits for them)
  if (nchunks > 0) {
    ent = entry_at(0);
    l2 = a.lse[(int64_t)(a.w0 + (ent >> 6)) * a.Hq + h];
    dval = a.D[(int64_t)(ent >> 6) * a.Hq + h];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(q_ptr(a.q, ent) + st * 32);
      df[st] = *reinterpret_cast<const bf16x8*>(q_ptr(a.dout, ent) + st * 32);
    }
  }
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int32_t r = a.w0 + (ent >> 6);
    const int32_t pos = first_pos + (r - rs);
    const float l2c = l2 * kLog2e, dvc = dval;
    const int ent_next = entry_at(chunk + 1);
    l2 = a.lse[(int64_t)(a.w0 + (ent_next >> 6)) * a.Hq + h];
    dval = a.D[(int64_t)(ent_next >> 6) * a.Hq + h];
    const int lim = pos - b * 128 - 4 * half;
    f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    f32x16 kacc[KL ? 4 : 1];
#pragma unroll
    for (int dt = 0; dt < (KL ? 4 : 1); ++dt) kacc[dt] = f32x16{};
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {   // keys 64 kh .. 64 kh + 63
      // S^T = K Q^T, then P^T in place (hidden keys: -inf -> 0)
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = mfma32x32x16(lds_load16<bf16x8>(&ks[kbase[st] + 8192 * (2 * kh + t)]), qf[st], acc[t]);
      if (kh == 1) {
#pragma unroll
        for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(q_ptr(a.q, ent_next) + st * 32);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ex = fast_exp2(__builtin_fmaf(acc[t][i], a.scale_log2, -l2c));
          acc[t][i] = (32 * (2 * kh + t) + 8 * (i >> 2) + (i & 3)) <= lim ? ex : 0.f;
        }
      // dP^T = V dO^T
      f32x16 dacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          dacc[t] = mfma32x32x16(lds_load16<bf16x8>(&vs[kbase[st] + 8192 * (2 * kh + t)]), df[st], dacc[t]);
      if (kh == 1) {
#pragma unroll
        for (int st = 0; st < 8; ++st) df[st] = *reinterpret_cast<const bf16x8*>(q_ptr(a.dout, ent_next) + st * 32);
      }
      // dS^T = P^T (dP^T - D) as bf16 B operands (and P^T itself for the proxy term)
      bf16x8 sf[2][2], pfk[KL ? 2 : 1][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          i32x4 pw, qw;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int i0 = 8 * u + 2 * x;
            const bf16x2 two = {(__bf16)(acc[t][i0] * (dacc[t][i0] - dvc)),
                                (__bf16)(acc[t][i0 + 1] * (dacc[t][i0 + 1] - dvc))};
            pw[x] = __builtin_bit_cast(int, two);
            if constexpr (KL) {
              const bf16x2 pp = {(__bf16)acc[t][i0], (__bf16)acc[t][i0 + 1]};
              qw[x] = __builtin_bit_cast(int, pp);
            }
          }
          sf[t][u] = __builtin_bit_cast(bf16x8, pw);
          if constexpr (KL) pfk[t][u] = __builtin_bit_cast(bf16x8, qw);
        }
      // dQ^T += K^T dS^T (and pk^T P^T for the proxy term)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ro = 256 * 32 * (2 * kh + t);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const s16x4 lo = lds_read_tr16(&ks[ktlo[dt] + ro + 256 * 16 * u]);
            const s16x4 hi = lds_read_tr16(&ks[kthi[dt] + ro + 256 * 16 * u]);
            oacc[dt] = mfma32x32x16(join_tr16(lo, hi), sf[t][u], oacc[dt]);
            if constexpr (KL) {
              const s16x4 plo = lds_read_tr16(&pkt[vbase[dt] + ro + 256 * 16 * u]);
              const s16x4 phi = lds_read_tr16(&pkt[vbase[dt] + ro + 256 * (16 * u + 8)]);
              kacc[dt] = mfma32x32x16(join_tr16(plo, phi), pfk[t][u], kacc[dt]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the scaled partial in block floating point, straight from the lanes
    // (records (row * k + slot) * Hq + head: the G heads of an entry share
    // lines); padding rows go to one of kTrashRecords trash records
    {
      const int srow = 32 * wave + (lane & 31);
      const int se = chunk * MT + srow / G;
      const int64_t trash = a.trash + (int64_t)(blockIdx.x & (kTrashRecords - 1));
      const int sent = ent_s[min(se, n_ent - 1)];
      const int head = g * G + (srow & (G - 1));
      auto rec_index = [&](int) -> int64_t {  // the lane's own row
        return se < n_ent ? ((int64_t)(sent >> 6) * a.k + (sent & 63)) * a.Hq + head : trash;
      };
      const float step = store_rows_bfp10(oacc, a.sm_scale, a.part_pk, a.plane_stride, rec_index, lane);
      // both halves hold the row's step and store the same value, at the
      // record's index (a token's heads adjacent: one contiguous piece per
      // token and store instruction)
      a.part_step[rec_index(0)] = step;
    }
    if constexpr (KL) {
      // sum_j P_hj pk_j for this wave's rows (kacc: C[dim][row] = pk^T P^T),
      // summed over a token's G heads (adjacent lanes); one bf16 store per
      // (token, slot) from the token's first lane.
      // G is a power of two up to 16 and a token's heads sit in G aligned
      // lanes of a 16-lane row: xor 1 and xor 2 (quad permutations) leave
      // every lane its pair and then quad sum; once each quad holds one value,
      // the half-row mirror (lane i <- 7 - i within 8) adds the other quad of
      // the 8, and once each 8 holds one value, the row mirror (i <- 15 - i)
      // adds the other 8
      float kv[64];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) kv[16 * dt + i] = kacc[dt][i];
      if (G >= 2)
#pragma unroll
        for (int e = 0; e < 64; ++e) kv[e] += dpp_f32<0xB1>(kv[e]);
      if (G >= 4)
#pragma unroll
        for (int e = 0; e < 64; ++e) kv[e] += dpp_f32<0x4E>(kv[e]);
      if (G >= 8)
#pragma unroll
        for (int e = 0; e < 64; ++e) kv[e] += dpp_f32<0x141>(kv[e]);
      if (G >= 16)
#pragma unroll
        for (int e = 0; e < 64; ++e) kv[e] += dpp_f32<0x140>(kv[e]);
      if (hh == 0 && chunk * MT + tok < n_ent) {
        uint16_t* dst = a.klpart + (((int64_t)(ent >> 6) * a.Hkv + g) * a.k + (ent & 63)) * 128 + 4 * half;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float* k4 = &kv[16 * dt + 4 * r4];
            const bf16x2 lo2 = {(__bf16)(k4[0] * a.inv_g), (__bf16)(k4[1] * a.inv_g)};
            const bf16x2 hi2 = {(__bf16)(k4[2] * a.inv_g), (__bf16)(k4[3] * a.inv_g)};
            *reinterpret_cast<i32x2*>(dst + 32 * dt + 8 * r4) = i32x2{__builtin_bit_cast(int, lo2), __builtin_bit_cast(int, hi2)};
          }
      }
    }
    ent = ent_next;
  }
}

struct DqSumArgs {
  const int32_t* sel;
  DevMeta m;
  const uint16_t* part;
  float* dq;              // fp32 [T, Hq, 128]
  int32_t Hq, Hkv, G, k, w0, w1;
};

// dQ of a (row, head) = the sum of its valid slots' partials; 16 lanes per
// pair, 8 columns each.
__global__ __launch_bounds__(256) void bwd_dq_sum_kernel(DqSumArgs a) {
  const int sub = threadIdx.x & 15;
  const int64_t idx = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (idx >= (int64_t)(a.w1 - a.w0) * a.Hq) return;
  const int32_t rl = (int32_t)(idx / a.Hq);
  const int h = (int)(idx % a.Hq);
  const int g = h / a.G;
  const int32_t r = a.w0 + rl;
  const int64_t base = ((int64_t)rl * a.Hq + h) * a.k;
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // 16 slots at a time: the partials are loaded before the selection says
  // which of them count (slots past topk repeat the last one)
  for (int s0 = 0; s0 < a.k; s0 += 16) {
    i32x4 v[16];
    int bk[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(a.part + (base + min(s0 + j, a.k - 1)) * 128 + 8 * sub));
#pragma unroll
    for (int j = 0; j < 16; ++j) bk[j] = s0 + j < a.k ? row[s0 + j] : -1;
    const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
    const int local = (a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s])) >> 7;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (bk[j] < 0 || bk[j] > local) continue;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        o[2 * x] += __builtin_bit_cast(float, (uint32_t)v[j][x] << 16);
        o[2 * x + 1] += __builtin_bit_cast(float, (uint32_t)v[j][x] & 0xffff0000u);
      }
    }
  }
  float* dst = a.dq + ((int64_t)r * a.Hq + h) * 128 + 8 * sub;
  *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
}

// dq = the sum over a row's slots of its block-floating-point partials
// (bwd_dq): 8 lanes per (row, head), each reading its dword of the planes
// (load_bfp_rec), slots 8 at a time, the first 8 slots' records issued before
// anything else; lane l of the 8 reads slot l's block id (coalesced) and a
// slot counts when its block is at most the row's local block (bwd_dq wrote
// nothing for the others: their step is taken as 0).  topk <= 64.
struct DqBfpSumArgs {
  const int32_t* sel;
  DevMeta m;
  const uint8_t* part_pk;
  int64_t plane_stride;
  const float* part_step;
  float* dq;              // fp32 [T, Hq, 128]
  int32_t Hq, Hkv, G, k, w0, w1;
};
__global__ __launch_bounds__(256) void bwd_dq_sum_bfp_kernel(DqBfpSumArgs a) {
  constexpr int NL = kMergeLanes;
  const int l = threadIdx.x & (NL - 1);
  const int64_t idx = (int64_t)blockIdx.x * (256 / NL) + (threadIdx.x / NL);
  const bool live = idx < (int64_t)(a.w1 - a.w0) * a.Hq;   // shuffles need every lane
  const int64_t id = live ? idx : 0;
  const int32_t rl = (int32_t)(id / a.Hq);
  const int h = (int)(id % a.Hq);
  const int g = h / a.G;
  const int32_t r = a.w0 + rl;
  auto rec_of = [&](int slot) -> int64_t { return ((int64_t)rl * a.k + slot) * a.Hq + h; };
  BfpRec v[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) v[j] = load_bfp_rec(a.part_pk, a.plane_stride, rec_of(min(j, a.k - 1)), l);
  const int32_t* row = a.sel + ((int64_t)r * a.Hkv + g) * a.k;
  const int ngroups = (a.k + NL - 1) / NL;
  int b_g[8];
  float st_g[8];
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    const int slot = min(NL * gi + l, a.k - 1);
    const bool in = gi < ngroups && NL * gi + l < a.k;
    b_g[gi] = in ? row[slot] : -1;
    st_g[gi] = in ? a.part_step[rec_of(slot)] : 0.f;
  }
  const int s = upper_bound_i32(a.m.row_start, a.m.S + 1, r) - 1;
  const int local = (a.m.kv[s] - a.m.qo[s] + (r - a.m.row_start[s])) >> 7;
#pragma unroll
  for (int gi = 0; gi < 8; ++gi)
    if (!(b_g[gi] >= 0 && b_g[gi] <= local)) st_g[gi] = 0.f;  // never written: never read into the sum
  float o[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) o[x] = 0.f;
  for (int gi = 0; gi < ngroups; ++gi) {
    float stl = st_g[0];
#pragma unroll
    for (int q = 1; q < 8; ++q) stl = q == gi ? st_g[q] : stl;
    if (gi > 0) {
#pragma unroll
      for (int j = 0; j < NL; ++j) v[j] = load_bfp_rec(a.part_pk, a.plane_stride, rec_of(min(NL * gi + j, a.k - 1)), l);
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const float step = __shfl(stl, j, NL);
      if (step == 0.f) continue;
#pragma unroll
      for (int x = 0; x < 16; ++x) o[x] = __builtin_fmaf(step, bfp_field(v[j], x), o[x]);
    }
  }
  if (!live) return;
  const int hh = l >> 2, dt = l & 3;
  float* drow = a.dq + ((int64_t)r * a.Hq + h) * 128;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq)
    *reinterpret_cast<f32x4*>(drow + 32 * dt + 8 * gq + 4 * hh) = f32x4{o[4 * gq], o[4 * gq + 1], o[4 * gq + 2], o[4 * gq + 3]};
}

struct BwdKvArgs {
  const uint8_t* q;       // bf16 [T, Hq, 128]
  const uint8_t* dout;
  const uint8_t* kp;      // bf16 [N, Hkv, 128, 128]
  const uint8_t* vp;
  const float* lse;       // [T, Hq], natural log
  const float* D;         // [W, Hq]
  const int32_t* kv_indices;
  const int32_t* entries;
  const int32_t* offsets; // [Hkv * NB + 1]
  DevMeta m;
  float* dk;              // fp32 [N, Hkv, 128, 128]
  float* dv;
  int32_t Hq, Hkv, G, NB, w0, w1, accumulate;
  float scale_log2, sm_scale;
  // proxy distillation term (KL kernels only): proxy q bf16 [T, Hkv, 128];
  // dpk fp32 [N, Hkv, 128, 128] receives (1/G) sum over rows and heads of
  // P_hj pq[token]
  const uint8_t* pq;
  float* dpk;
  float inv_g;
  // KL kernels: the even chunks' dK / dV partials of each (group, block),
  // [key][wave][tile][register][lane] fp32 (see bwd_dkv_kernel)
  float* stash;
};


// Workgroup shape.  Without the proxy term: two groups of four waves take
// alternate chunks of the block's rows (each wave of a group owns 32 keys)
// and sum their dK / dV partials through LDS at the end; two waves per SIMD,
// at most 256 registers each, so the products accumulate in ordinary
// registers that the vector unit reads directly.  With it (a third set of
// 32x128 accumulators): one group, one wave per SIMD.
template <bool KL>
constexpr int bwd_dkv_groups() { return KL ? 1 : 2; }
template <bool KL>
constexpr int bwd_dkv_threads() { return 256 * bwd_dkv_groups<KL>(); }

// DENSE: every row of the window that sees the block (the warm-up mode's
// dense main attention), in row order, instead of the bin's CSR entries.
template <bool KL, bool DENSE = false>
__global__ __launch_bounds__(bwd_dkv_threads<KL>()) void bwd_dkv_kernel(BwdKvArgs a) {
  constexpr int kGroups = bwd_dkv_groups<KL>();
  constexpr int kTile = 32 * 256;  // a chunk's 32 rows of 128 bf16
  // K and V of the block (rt_swz; rows past kv_len zeroed), the B operands of
  // every chunk's S and dP products (with the proxy term, one wave per SIMD
  // has the registers to hold its keys' K and V rows instead).  Then per
  // group and buffer: the chunk's q rows, dO rows and (KL) proxy q rows (row
  // i: token i / G), rt_swz; two buffers, three for the second group (its
  // dV / dK products of a chunk run one iteration late, below).  The first
  // 128 KB hold the second group's partials for the final sum.
  constexpr int kKinds = KL ? 3 : 2;
  constexpr int kKvBytes = KL ? 0 : 2 * 128 * 256;
  constexpr int kGroupBytes = 2 * kKinds * kTile;   // the first group's
  constexpr int kBufs1 = 3;                          // the second group's buffers
  __shared__ __attribute__((aligned(16))) uint8_t smem[kKvBytes + kGroupBytes + (kGroups - 1) * kBufs1 * kKinds * kTile];
  __shared__ __attribute__((aligned(16))) float l2_s[kGroups][2][32];
  __shared__ __attribute__((aligned(16))) float d_s[kGroups][2][32];
  __shared__ __attribute__((aligned(16))) int32_t pos_s[kGroups][2][32];
  static_assert(KL || kKvBytes + kGroupBytes + kBufs1 * kKinds * kTile >= 4 * 8 * 16 * 64 * 4,
                "partials fit the tiles' space");
  uint8_t* const kv_k = smem;
  uint8_t* const kv_v = smem + (KL ? 0 : 128 * 256);
  // block-major order: the early, most selected blocks of every group start first
  const int gb = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int key = g * a.NB + gb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = kGroups == 1 ? 0 : tid >> 8;   // chunk group
  const int gtid = tid & 255, wave = gtid >> 6;  // wave within the group: keys 32 wave ..
  uint8_t* const gsm = smem + kKvBytes + grp * kGroupBytes;
  const int s = upper_bound_i32(a.m.page_start, a.m.S + 1, gb) - 1;
  const int b = gb - a.m.page_start[s];
  const int32_t page = a.kv_indices[gb];
  const int32_t first_pos = a.m.kv[s] - a.m.qo[s];
  const int32_t rs = a.m.row_start[s];
  int e0 = 0, n_ent = 0, dense_lo = 0;   // dense: window-relative first row
  if constexpr (DENSE) {
    const int32_t lo = max(max(0, b * 128 - first_pos), a.w0 - rs);
    const int32_t hi = min(a.m.qo[s], a.w1 - rs);
    n_ent = max(0, hi - lo);
    dense_lo = rs + lo - a.w0;
  } else {
    e0 = a.offsets[key];
    n_ent = a.offsets[key + 1] - e0;
  }
  const int G = a.G;
  const int MT = 32 / G;                       // tokens per 32-row chunk
  const int half = lane >> 5, j = lane & 31;
  bf16x8 bk_r[KL ? 8 : 1], bv_r[KL ? 8 : 1];
  if constexpr (KL) {
    // lane (j, half), step st: key 32 wave + j, dims 16 st + 8 half ..
    const int krow = 32 * wave + j;
    const bool live_row = krow < a.m.kv[s] - b * 128;
    const int64_t off = ((int64_t)page * a.Hkv + g) * 32768 + krow * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      bk_r[st] = live_row ? *reinterpret_cast<const bf16x8*>(a.kp + off + st * 32) : bf16x8{};
      bv_r[st] = live_row ? *reinterpret_cast<const bf16x8*>(a.vp + off + st * 32) : bf16x8{};
    }
  } else {  // K and V -> LDS (16-byte pieces; rows past kv_len zeroed)
    const int kv_rows = a.m.kv[s] - b * 128;
    const uint8_t* kb = a.kp + ((int64_t)page * a.Hkv + g) * 32768;
    const uint8_t* vb = a.vp + ((int64_t)page * a.Hkv + g) * 32768;
    constexpr int kRounds = 2048 / bwd_dkv_threads<KL>();
    i32x4 kr[kRounds], vr[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int c = tid + bwd_dkv_threads<KL>() * i;
      kr[i] = *reinterpret_cast<const i32x4*>(kb + c * 16);
      vr[i] = *reinterpret_cast<const i32x4*>(vb + c * 16);
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int c = tid + bwd_dkv_threads<KL>() * i;
      const bool live_row = (c >> 4) < kv_rows;
      lds_store16<i32x4>(&kv_k[rt_swz(c >> 4, c & 15)], live_row ? kr[i] : i32x4{});
      lds_store16<i32x4>(&kv_v[rt_swz(c >> 4, c & 15)], live_row ? vr[i] : i32x4{});
    }
  }
  const int q16 = lane >> 4, m16 = lane & 15;
  const int nchunks = (n_ent + MT - 1) / MT;
  const int keypos = b * 128 + 32 * wave + j;  // this lane's key position
  const int krow = 32 * wave + j;              // its K / V row
  // transposed reads: lane (q16, m16) fetches dims 32 dt + 16 (q16 & 1) +
  // 4 (m16 & 3) .. +3 of tile row r0 (lo) or r0 + 8 (hi), r0 = 4 (q16 >> 1) +
  // m16 / 4 (+ 16 u)
  int vlo[4], vhi[4];
  {
    const int r0 = 4 * (q16 >> 1) + (m16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int c = 4 * dt + 2 * (q16 & 1) + ((m16 & 3) >> 1);
      vlo[dt] = rt_swz(r0, c) + 8 * (m16 & 1);
      vhi[dt] = rt_swz(r0 + 8, c) + 8 * (m16 & 1);
    }
  }
  f32x16 dkacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x16 dvacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x16 pkacc[KL ? 4 : 1];
#pragma unroll
  for (int dt = 0; dt < (KL ? 4 : 1); ++dt) pkacc[dt] = f32x16{};
  // Gathered rows (row i of a chunk: token i / G, head i % G).  Two waves
  // per SIMD (no proxy term): straight from global memory to LDS
  // (global_load_lds_dwordx4), so that no register holds them: instruction
  // i of wave w of a group fills bytes 1024 (2 w + i) .. +1023 of the chunk's
  // tile, lane l its 16-byte slot, i.e. row ri_i = 8 w + 4 i + l / 16 at
  // physical chunk l % 16, so the lane fetches that row's logical chunk
  // (rt_swz); the next chunk is issued once every wave is past the barrier
  // that retires the buffer it overwrites.  One wave per SIMD (proxy term):
  // through registers, the next chunk's loads issued before the barrier (a
  // wave alone on its SIMD has nothing else to hide them behind), stored to
  // LDS at the start of the next chunk.  Threads below 32 of the group also
  // fetch row gtid's lse, D and position into registers; entry ids one chunk
  // earlier.  Past the last chunk a group runs a chunk whose rows are all
  // padding (position -1: no key visible).
  const int ri0 = 8 * wave + (lane >> 4), ri1 = ri0 + 4;
  const int lc0 = (lane & 15) ^ rt_swz_key(ri0), lc1 = (lane & 15) ^ rt_swz_key(ri1);
  // Chunk order.  Two groups: group grp takes chunks grp, grp + 2, ..., and
  // the final dK / dV is (even chunks' sum) + (odd chunks' sum).  One group
  // (KL): the even chunks in order, then the odd ones; the even chunks'
  // partials are parked in `stash` in between and added at the end, so that
  // the result is the same fp32 sum bit for bit (a group's padding chunk
  // adds exact zeros).
  const int n_even = (nchunks + 1) / 2;
  const int niter = kGroups == 2 ? n_even : nchunks;
  auto chunk_of = [&](int it) { return kGroups == 2 ? 2 * it + grp : it < n_even ? 2 * it : 2 * (it - n_even) + 1; };
  float* const stash = KL ? a.stash + (int64_t)(key * 4 + wave) * (8 * 16 * 64) + lane : nullptr;
  // entries and lse stay raw in registers until used
  auto entry_of = [&](int chunk, int ri) {
    const int e = min(chunk * MT + ri / G, n_ent - 1);
    if constexpr (DENSE) return (dense_lo + e) << 6;
    else return a.entries[e0 + e];
  };
  auto row_src = [&](const uint8_t* base, int32_t ent, int ri, int lc) {
    return base + ((int64_t)(a.w0 + (ent >> 6)) * a.Hq + g * G + ri % G) * 256 + lc * 16;
  };
  auto prow_src = [&](int32_t ent, int lc) {
    return a.pq + ((int64_t)(a.w0 + (ent >> 6)) * a.Hkv + g) * 256 + lc * 16;
  };
  // tiles of buffer `buf`: q, dO, (KL) proxy q
  const int nbufs = grp == 1 ? kBufs1 : 2;
  auto tile = [&](int kind, int buf) { return gsm + (nbufs * kind + buf) * kTile; };
  // (untracked by the compiler: it would wait for them before the current
  // chunk's first LDS read; the wait before the next barrier orders them)
  auto issue_rows = [&](int32_t ea, int32_t eb, int buf) {
    uint8_t* const w0b = tile(0, buf) + 2048 * wave;
    uint8_t* const w1b = tile(1, buf) + 2048 * wave;
    global_load_lds16_untracked(row_src(a.q, ea, ri0, lc0), (MSA_LDS void*)w0b);
    global_load_lds16_untracked(row_src(a.q, eb, ri1, lc1), (MSA_LDS void*)(w0b + 1024));
    global_load_lds16_untracked(row_src(a.dout, ea, ri0, lc0), (MSA_LDS void*)w1b);
    global_load_lds16_untracked(row_src(a.dout, eb, ri1, lc1), (MSA_LDS void*)(w1b + 1024));
    if constexpr (KL) {
      uint8_t* const w2b = tile(2, buf) + 2048 * wave;
      global_load_lds16_untracked(prow_src(ea, lc0), (MSA_LDS void*)w2b);
      global_load_lds16_untracked(prow_src(eb, lc1), (MSA_LDS void*)(w2b + 1024));
    }
  };
  i32x4 rr[KL ? 6 : 1];  // KL: the next chunk's q, dO and proxy q pieces of rows ri0, ri1
  auto load_rows = [&](int32_t ea, int32_t eb) {
    if constexpr (KL) {
      rr[0] = *reinterpret_cast<const i32x4*>(row_src(a.q, ea, ri0, lane & 15));
      rr[1] = *reinterpret_cast<const i32x4*>(row_src(a.q, eb, ri1, lane & 15));
      rr[2] = *reinterpret_cast<const i32x4*>(row_src(a.dout, ea, ri0, lane & 15));
      rr[3] = *reinterpret_cast<const i32x4*>(row_src(a.dout, eb, ri1, lane & 15));
      rr[4] = *reinterpret_cast<const i32x4*>(prow_src(ea, lane & 15));
      rr[5] = *reinterpret_cast<const i32x4*>(prow_src(eb, lane & 15));
    }
  };
  auto store_rows = [&](int buf) {
    if constexpr (KL) {
#pragma unroll
      for (int kind = 0; kind < 3; ++kind) {
        lds_store16<i32x4>(tile(kind, buf) + rt_swz(ri0, lane & 15), rr[2 * kind]);
        lds_store16<i32x4>(tile(kind, buf) + rt_swz(ri1, lane & 15), rr[2 * kind + 1]);
      }
    }
  };
  if (niter > 0) {
    int32_t ea = entry_of(chunk_of(0), ri0), eb = entry_of(chunk_of(0), ri1);
    int32_t es = gtid < 32 ? entry_of(chunk_of(0), gtid) : 0;
    if constexpr (KL) load_rows(ea, eb);
    else issue_rows(ea, eb, 0);
    float rlse = 0.f, rdd = 0.f;
    int32_t rpos = 0;
    if (gtid < 32) {
      const int h = g * G + gtid % G;
      rlse = a.lse[(int64_t)(a.w0 + (es >> 6)) * a.Hq + h];
      rdd = a.D[(int64_t)(es >> 6) * a.Hq + h];
      rpos = chunk_of(0) * MT + gtid / G < n_ent ? first_pos + (a.w0 + (es >> 6) - rs) : -1;  // padding rows see no key
    }
    ea = entry_of(chunk_of(1), ri0);
    eb = entry_of(chunk_of(1), ri1);
    es = gtid < 32 ? entry_of(chunk_of(1), gtid) : 0;
    // One chunk in phases.  head: the chunk's row values to LDS, the barrier
    // after which its rows are in LDS (and every wave is done with the buffer
    // the next chunk fills), the next chunk's loads; products: S, dP, then P
    // and dS as bf16 A operands; update: dV += P^T dO, dK += dS^T Q.  tb is
    // the chunk's tile buffer, the row values' buffer is it & 1.
    auto head = [&](int it, int tb, int tb_next) __attribute__((always_inline)) {
      const int rb = it & 1;
      store_rows(tb);
      if (gtid < 32) {
        l2_s[grp][rb][gtid] = rlse * kLog2e;
        d_s[grp][rb][gtid] = rdd;
        pos_s[grp][rb][gtid] = rpos;
      }
      const int cn = chunk_of(it + 1);
      if constexpr (KL) load_rows(ea, eb);
      // this chunk's rows are in LDS (each wave waits for its own direct
      // loads, the barrier for everyone's; K and V the first time); every
      // wave is done with the previous chunk, whose buffer the next one fills
      if constexpr (!KL) wait_vmem();
      lds_barrier();
      if constexpr (!KL) issue_rows(ea, eb, tb_next);
      if (gtid < 32) {
        const int h = g * G + gtid % G;
        rlse = a.lse[(int64_t)(a.w0 + (es >> 6)) * a.Hq + h];
        rdd = a.D[(int64_t)(es >> 6) * a.Hq + h];
        rpos = cn * MT + gtid / G < n_ent ? first_pos + (a.w0 + (es >> 6) - rs) : -1;
      }
      ea = entry_of(chunk_of(it + 2), ri0);
      eb = entry_of(chunk_of(it + 2), ri1);
      es = gtid < 32 ? entry_of(chunk_of(it + 2), gtid) : 0;
    };
    auto products = [&](int it, int tb, bf16x8 (&pf)[2], bf16x8 (&sf)[2]) __attribute__((always_inline)) {
      const int buf = it & 1;
      const uint8_t* const qb = tile(0, tb);
      const uint8_t* const db = tile(1, tb);
      // the rows' lse, D and positions as 4-row runs (register r of the
      // products below holds row 8(r/4) + 4 half + r%4): with the proxy term
      // (registers to spare, one wave per SIMD) read before the products,
      // whose latency then covers theirs, else read where used
      f32x4 l2v[4], dv4[4];
      i32x4 ps4[4];
      auto read_rows = [&](int t4) {
        l2v[t4] = *reinterpret_cast<const f32x4*>(&l2_s[grp][buf][8 * t4 + 4 * half]);
        dv4[t4] = *reinterpret_cast<const f32x4*>(&d_s[grp][buf][8 * t4 + 4 * half]);
        ps4[t4] = *reinterpret_cast<const i32x4*>(&pos_s[grp][buf][8 * t4 + 4 * half]);
      };
      if constexpr (KL) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) read_rows(t4);
      }
      // S = Q K^T and dP = dO V^T for this wave's 32 keys: C[row][key], key on lanes
      // fragments from LDS read one k-step ahead of their products
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      bf16x8 aq[2], ad[2], bkl[KL ? 1 : 2], bvl[KL ? 1 : 2];
      auto frags = [&](int st, int x) {
        aq[x] = lds_load16<bf16x8>(&qb[rt_swz(j, 2 * st + half)]);
        ad[x] = lds_load16<bf16x8>(&db[rt_swz(j, 2 * st + half)]);
        if constexpr (!KL) {
          bkl[x] = lds_load16<bf16x8>(&kv_k[rt_swz(krow, 2 * st + half)]);
          bvl[x] = lds_load16<bf16x8>(&kv_v[rt_swz(krow, 2 * st + half)]);
        }
      };
      frags(0, 0);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) frags(st + 1, (st + 1) & 1);
        if constexpr (KL) {
          sacc = mfma32x32x16(aq[st & 1], bk_r[st], sacc);
          pacc = mfma32x32x16(ad[st & 1], bv_r[st], pacc);
        } else {
          sacc = mfma32x32x16(aq[st & 1], bkl[st & 1], sacc);
          pacc = mfma32x32x16(ad[st & 1], bvl[st & 1], pacc);
        }
      }
      // P and dS as bf16 A operands
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 pw, sw;
        if constexpr (!KL) {
          read_rows(2 * u);
          read_rows(2 * u + 1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float pv[2], sv[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int rr = 8 * u + 2 * t + x;
            const float ex = fast_exp2(__builtin_fmaf(sacc[rr], a.scale_log2, -l2v[rr >> 2][rr & 3]));
            const float p = keypos <= ps4[rr >> 2][rr & 3] ? ex : 0.f;
            pv[x] = p;
            sv[x] = p * (pacc[rr] - dv4[rr >> 2][rr & 3]);
          }
          const bf16x2 p2 = {(__bf16)pv[0], (__bf16)pv[1]};
          const bf16x2 s2 = {(__bf16)sv[0], (__bf16)sv[1]};
          pw[t] = __builtin_bit_cast(int, p2);
          sw[t] = __builtin_bit_cast(int, s2);
        }
        pf[u] = __builtin_bit_cast(bf16x8, pw);
        sf[u] = __builtin_bit_cast(bf16x8, sw);
      }
    };
    auto update = [&](int tb, const bf16x8 (&pf)[2], const bf16x8 (&sf)[2]) __attribute__((always_inline)) {
      const uint8_t* const qb = tile(0, tb);
      const uint8_t* const db = tile(1, tb);
      const uint8_t* const pb = tile(2, tb);  // KL only
      // dV += P^T dO, dK += dS^T Q: dO and Q read transposed, rows in the same order
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 dlo = lds_read_tr16(&db[vlo[dt] + 256 * (16 * u)]);
          const s16x4 dhi = lds_read_tr16(&db[vhi[dt] + 256 * (16 * u)]);
          dvacc[dt] = mfma32x32x16(pf[u], join_tr16(dlo, dhi), dvacc[dt]);
          const s16x4 qlo = lds_read_tr16(&qb[vlo[dt] + 256 * (16 * u)]);
          const s16x4 qhi = lds_read_tr16(&qb[vhi[dt] + 256 * (16 * u)]);
          dkacc[dt] = mfma32x32x16(sf[u], join_tr16(qlo, qhi), dkacc[dt]);
          if constexpr (KL) {   // P^T times the rows' proxy q
            const s16x4 plo = lds_read_tr16(&pb[vlo[dt] + 256 * (16 * u)]);
            const s16x4 phi = lds_read_tr16(&pb[vhi[dt] + 256 * (16 * u)]);
            pkacc[dt] = mfma32x32x16(pf[u], join_tr16(plo, phi), pkacc[dt]);
          }
        }
      }
    };
    bool late = false;   // the second group: each chunk's update one iteration late
    if constexpr (kGroups == 2) late = grp == 1;
    if (!late) {
      auto step = [&](int it) __attribute__((always_inline)) {
        const int tb = it & 1;
        head(it, tb, tb ^ 1);
        bf16x8 pf[2], sf[2];
        products(it, tb, pf, sf);
        update(tb, pf, sf);
      };
      const int it_split = KL ? n_even : niter;
      for (int it = 0; it < it_split; ++it) step(it);
      if constexpr (KL) {
        if (n_even < nchunks) {  // the even chunks are done: park their dK / dV partials
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              stash[(dt * 16 + r) * 64] = dkacc[dt][r];
              stash[((4 + dt) * 16 + r) * 64] = dvacc[dt][r];
            }
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) dkacc[dt] = dvacc[dt] = f32x16{};
        }
        for (int it = it_split; it < niter; ++it) step(it);
      }
    } else if constexpr (kGroups == 2) {
      // Both groups pass the same barrier every chunk; with the same order of
      // phases the two waves of a SIMD (one per group) would run their
      // products and their vector work at the same time.  This group runs a
      // chunk's update after the next chunk's barrier, while the first group
      // runs its S and dP products, and its P / dS work while the first group
      // runs its update.  Three tile buffers: chunk it in it % 3 (the update
      // of chunk it - 1 reads its buffer while chunk it + 1's rows land).
      // The sums are the same, chunk by chunk in the same order.
      bf16x8 pf[2], sf[2];
      int tb = 0;
      for (int it = 0; it < niter; ++it) {
        const int tb_next = tb == kBufs1 - 1 ? 0 : tb + 1;
        head(it, tb, tb_next);
        if (it > 0) update(tb == 0 ? kBufs1 - 1 : tb - 1, pf, sf);
        products(it, tb, pf, sf);
        tb = tb_next;
      }
      update(tb == 0 ? kBufs1 - 1 : tb - 1, pf, sf);
    }
  }
  if constexpr (kGroups == 2) {
    // the second group's partials -> LDS (over the tiles), added by the first
    // group in a fixed order: [wave][tile: dK 0-3, dV 0-3][register][lane]
    float* const red = reinterpret_cast<float*>(smem);
    // the last chunk's loads of the next (padding) rows may still be in
    // flight into the tiles' space: every wave waits for its own, then the
    // barrier for everyone's
    wait_vmem();
    __syncthreads();  // every wave is done with the tiles
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[((wave * 8 + dt) * 16 + r) * 64 + lane] = dkacc[dt][r];
          red[((wave * 8 + 4 + dt) * 16 + r) * 64 + lane] = dvacc[dt][r];
        }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[dt][r] += red[((wave * 8 + dt) * 16 + r) * 64 + lane];
        dvacc[dt][r] += red[((wave * 8 + 4 + dt) * 16 + r) * 64 + lane];
      }
  }
  if constexpr (KL) {
    if (n_even < nchunks) {  // even chunks' partials + odd chunks' (this lane's own stores, read back)
      wait_vmem();
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dkacc[dt][r] = stash[(dt * 16 + r) * 64] + dkacc[dt][r];
          dvacc[dt][r] = stash[((4 + dt) * 16 + r) * 64] + dvacc[dt][r];
        }
    }
  }
  // C[key][d]: lane (d, half), register r -> key 32 wave + 8 (r/4) + 4 half + r%4
  const int64_t pbase = ((int64_t)page * a.Hkv + g) * 128;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 32 * wave + 8 * (r >> 2) + 4 * half + (r & 3);
      const int64_t o = (pbase + kk) * 128 + 32 * dt + j;
      const float vk = dkacc[dt][r] * a.sm_scale, vv = dvacc[dt][r];
      a.dk[o] = a.accumulate ? a.dk[o] + vk : vk;
      a.dv[o] = a.accumulate ? a.dv[o] + vv : vv;
      if constexpr (KL) {
        const float vp = pkacc[dt][r] * a.inv_g;
        a.dpk[o] = a.accumulate ? a.dpk[o] + vp : vp;
      }
    }
}

}  // namespace

hipError_t launch_dense_dkv(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                            const int32_t* kv_indices, const float* lse, const float* D, const void* dout, float* dk,
                            float* dv, const KlOperands* kl, char* ws, hipStream_t st) {
  BwdKvArgs kv{};
  kv.q = static_cast<const uint8_t*>(q);
  kv.dout = static_cast<const uint8_t*>(dout);
  kv.kp = static_cast<const uint8_t*>(kp);
  kv.vp = static_cast<const uint8_t*>(vp);
  kv.lse = lse;
  kv.D = D;
  kv.kv_indices = kv_indices;
  kv.m = m;
  kv.dk = dk;
  kv.dv = dv;
  kv.Hq = p->d.num_qo_heads;
  kv.Hkv = p->d.num_kv_heads;
  kv.G = p->G;
  kv.NB = p->NB;
  kv.w0 = 0;
  kv.w1 = p->T;
  kv.accumulate = 0;
  kv.scale_log2 = p->d.sm_scale * kLog2e;
  kv.sm_scale = p->d.sm_scale;
  kv.pq = kl ? static_cast<const uint8_t*>(kl->pq) : nullptr;
  kv.dpk = kl ? kl->dpk : nullptr;
  kv.inv_g = 1.f / (float)p->G;
  kv.stash = kl ? reinterpret_cast<float*>(ws + p->lay.kl_stash) : nullptr;
  const dim3 grid((unsigned)(p->d.num_kv_heads * p->NB));
  ProfEvents pe(p, "dense_dkv");
  if (kl)
    hipExtLaunchKernelGGL((bwd_dkv_kernel<true, true>), grid, dim3(bwd_dkv_threads<true>()), 0, st, pe.start,
                          pe.stop, 0, kv);
  else
    hipExtLaunchKernelGGL((bwd_dkv_kernel<false, true>), grid, dim3(bwd_dkv_threads<false>()), 0, st, pe.start,
                          pe.stop, 0, kv);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const msa_plan_s* p, const void* out, const void* dout, float* D, int32_t w0, int32_t w1,
                           hipStream_t st) {
  const int64_t npairs = (int64_t)(w1 - w0) * p->d.num_qo_heads;
  PrepArgs pa{static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), D, w0, w1, p->d.num_qo_heads};
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((npairs + 15) / 16)), dim3(256), 0, st, pa);
  return hipGetLastError();
}

hipError_t launch_prefill_backward_window(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp,
                                          const void* vp, const int32_t* kv_indices, const int32_t* sel,
                                          const void* out, const float* lse, const void* dout, float* dq, float* dk,
                                          float* dv, const KlOperands* kl, char* ws, int32_t w0, int32_t w1,
                                          bool first_window, hipStream_t st) {
  const PlanLayout& L = p->lay;
  const int Hkv = p->d.num_kv_heads, Hq = p->d.num_qo_heads, k = p->d.topk;
  const int32_t nkey = Hkv * p->NB;
  build_csr(p, m, sel, ws, w0, w1, st, /*sorted=*/true, /*with_local=*/true);
  float* D = reinterpret_cast<float*>(ws + L.bwd_d);
  const int64_t npairs = (int64_t)(w1 - w0) * Hq;
  {
    PrepArgs pa{static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), D, w0, w1, Hq};
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((npairs + 15) / 16)), dim3(256), 0, st, pa);
  }
  BwdDqArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.dout = static_cast<const uint8_t*>(dout);
  a.kp = static_cast<const uint8_t*>(kp);
  a.vp = static_cast<const uint8_t*>(vp);
  a.lse = lse;
  a.D = D;
  a.kv_indices = kv_indices;
  a.entries = reinterpret_cast<const int32_t*>(ws + L.entries);
  a.items = reinterpret_cast<const int4*>(ws + L.items);
  a.nitems = reinterpret_cast<const int32_t*>(ws + L.nitems);
  a.m = m;
  // the dQ partial records' planes and steps share the region the forward's
  // partial records use (160 + 4 bytes per record of its 168)
  a.trash = p->attn_window * Hq * k;
  const int64_t nrec = a.trash + kTrashRecords;
  a.part_pk = reinterpret_cast<uint8_t*>(ws + L.part_o);
  a.plane_stride = nrec * 32;
  a.part_step = reinterpret_cast<float*>(a.part_pk + 5 * a.plane_stride);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p->G;
  a.k = k;
  a.w0 = w0;
  a.scale_log2 = p->d.sm_scale * kLog2e;
  a.sm_scale = p->d.sm_scale;
  a.pkp = kl ? static_cast<const uint8_t*>(kl->pkp) : nullptr;
  a.klpart = kl ? reinterpret_cast<uint16_t*>(ws + L.kl_part) : nullptr;
  a.inv_g = 1.f / (float)p->G;
  const int64_t max_items = ((int64_t)(w1 - w0) * Hkv * k + p->entries_per_item - 1) / p->entries_per_item + nkey;
  {
    ProfEvents pe(p, "bwd_dq");
    if (kl)
      hipExtLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)max_items), dim3(256), 0, st, pe.start, pe.stop, 0, a);
    else
      hipExtLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)max_items), dim3(256), 0, st, pe.start, pe.stop, 0, a);
  }
  {
    DqBfpSumArgs ds{sel, m, a.part_pk, a.plane_stride, a.part_step, dq, Hq, Hkv, p->G, k, w0, w1};
    constexpr int kPairsPerBlock = 256 / kMergeLanes;
    ProfEvents pe(p, "bwd_dq_sum");
    hipExtLaunchKernelGGL(bwd_dq_sum_bfp_kernel, dim3((unsigned)((npairs + kPairsPerBlock - 1) / kPairsPerBlock)),
                          dim3(256), 0, st, pe.start, pe.stop, 0, ds);
  }
  if (kl) {   // the sparse proxy term of each (row, group): sum of its slots, into dpq
    DqSumArgs ds{sel, m, a.klpart, kl->dpq, Hkv, Hkv, 1, k, w0, w1};
    const int64_t n = (int64_t)(w1 - w0) * Hkv;
    ProfEvents pe(p, "kl_dq_sum");
    hipExtLaunchKernelGGL(bwd_dq_sum_kernel, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, st, pe.start, pe.stop,
                          0, ds);
  }
  BwdKvArgs kv;
  kv.q = a.q;
  kv.dout = a.dout;
  kv.kp = a.kp;
  kv.vp = a.vp;
  kv.lse = lse;
  kv.D = D;
  kv.kv_indices = kv_indices;
  kv.entries = a.entries;
  kv.offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  kv.m = m;
  kv.dk = dk;
  kv.dv = dv;
  kv.Hq = Hq;
  kv.Hkv = Hkv;
  kv.G = p->G;
  kv.NB = p->NB;
  kv.w0 = w0;
  kv.w1 = w1;
  kv.accumulate = first_window ? 0 : 1;
  kv.scale_log2 = a.scale_log2;
  kv.sm_scale = a.sm_scale;
  kv.pq = kl ? static_cast<const uint8_t*>(kl->pq) : nullptr;
  kv.dpk = kl ? kl->dpk : nullptr;
  kv.inv_g = a.inv_g;
  kv.stash = kl ? reinterpret_cast<float*>(ws + L.kl_stash) : nullptr;
  {
    ProfEvents pe(p, "bwd_dkv");
    if (kl)
      hipExtLaunchKernelGGL(bwd_dkv_kernel<true>, dim3((unsigned)nkey), dim3(bwd_dkv_threads<true>()), 0, st,
                            pe.start, pe.stop, 0, kv);
    else
      hipExtLaunchKernelGGL(bwd_dkv_kernel<false>, dim3((unsigned)nkey), dim3(bwd_dkv_threads<false>()), 0, st,
                            pe.start, pe.stop, 0, kv);
  }
  return hipGetLastError();
}

}  // namespace msa
