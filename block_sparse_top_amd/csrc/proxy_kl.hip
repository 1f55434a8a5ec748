// Dense part of the proxy distillation gradient (Flash-MSA article, backward
// paragraph: the gradient of KL(main || proxy) with respect to a proxy score
// is the proxy probability minus the main probability).
//
// For row r and KV group g (driven by proxy head g) over the row's visible
// keys j:  dz_j = grad_scale (p_proxy_j - p_main_j), with p_proxy the dense
// causal softmax of z_j = proxy_scale <pq[r, g], pk[j, g]> and p_main the
// group mean of the main attention over the cached selection.  The p_main
// part is sparse and comes from the fused main backward, which leaves
//   dpq[r, g] = (1/G) sum_h sum_j P_hj pk_j       and
//   dpk[j, g] = (1/G) sum_r sum_h P_hj pq[r, g]
// in the gradient buffers.  The two kernels here add the dense part:
//  1. kl_dense_dq: per 128-row quarter of a proxy row tile and proxy head, one
//     online-softmax sweep over the visible key blocks accumulates
//     sum_j p_proxy_j pk_j (dQ^T = K^T P^T on MFMA, rescaled as the row max
//     grows) and the row's proxy log-sum-exp; dpq = out_scale (dense - sparse).
//  2. kl_dense_dk: per (key block, proxy head), every row that sees the
//     block in 32-row chunks (rows prefetched into registers, LDS tiles
//     double-buffered): S = Q K^T, P from the row's log-sum-exp, dK += P^T Q;
//     dpk = out_scale (dense - sparse).
#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

struct KlDqArgs {
  const uint8_t* pq;      // bf16 [T, P, 128]
  const uint8_t* pk;      // bf16 [N, P, 128, 128]
  const int32_t* kv_indices;
  DevMeta m;
  float* plse;            // [T, P], natural log
  float* dpq;             // [T, P, 128]: sparse term on entry, gradient on exit
  int32_t P;
  float scale_log2, out_scale;
};

__global__ __launch_bounds__(256, 2) void kl_dense_dq_kernel(KlDqArgs a) {
  // one tile of each (64 KB): two workgroups share a CU, and one's block
  // loads overlap the other's MFMAs
  __shared__ __attribute__((aligned(16))) uint8_t ks[1][128 * 256];   // proxy K, k_swz: S^T operand
  __shared__ __attribute__((aligned(16))) uint8_t kt[1][128 * 256];   // proxy K, v_swz: transposed reads
  const int p = blockIdx.y;
  const int qi = (int)gridDim.x - 1 - (int)blockIdx.x;   // later quarters (more keys) start first
  const int t = qi >> 2, sub = qi & 3;
  const int s = a.m.tiles[4 * t];
  const int n = min(128, a.m.tiles[4 * t + 2] - 128 * sub);
  if (n <= 0) return;
  const int row0 = a.m.tiles[4 * t + 1] + 128 * sub;
  const int pos0 = a.m.tiles[4 * t + 3] + 128 * sub;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int q16 = lane >> 4, m16 = lane & 15;
  const int ri = min(32 * wave + j, n - 1);
  const bool live = 32 * wave + j < n;
  const int32_t r = row0 + ri, pos = pos0 + ri;
  const int nblk = ((pos0 + n - 1) >> 7) + 1;
  const int32_t* pages = a.kv_indices + a.m.page_start[s];
  const int kv_len = a.m.kv[s];
  bf16x8 qf[8];
  {
    const uint8_t* qrow = a.pq + ((int64_t)r * a.P + p) * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + st * 32);
  }
  int kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = j * 256 + (((2 * st + half) ^ (lane & 15)) << 4);
  int vbase[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vbase[dt] = (4 * (q16 >> 1) + (m16 >> 2)) * 256 +
                ((4 * (dt ^ (m16 >> 2)) + 2 * (q16 & 1) + ((m16 & 3) >> 1)) << 4) + 8 * (m16 & 1);
  i32x4 kr[8];
  auto load_blk = [&](int b) {
    const uint8_t* base = a.pk + ((int64_t)pages[b] * a.P + p) * 32768;
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const i32x4*>(base + (tid + 256 * i) * 16);
  };
  auto store_blk = [&](int b, int buf, bool both) {   // rows past kv_len zeroed
    const int kv_in_block = kv_len - 128 * b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const i32x4 v = (c >> 4) < kv_in_block ? kr[i] : i32x4{};
      lds_store16<i32x4>(&ks[buf][k_swz(c >> 4, c & 15)], v);
      if (both) lds_store16<i32x4>(&kt[buf][v_swz(c >> 4, c & 15)], v);
    }
  };
  // S^T = K Q^T for block b in buffer buf, scaled to the log2 domain, hidden keys -inf:
  // register i of tile kt_ holds key 32 kt_ + 8 (i / 4) + 4 half + i % 4
  auto scores = [&](int b, int buf, f32x16 (&acc)[4]) {
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_) acc[kt_] = f32x16{};
    bf16x8 kf[2][4];   // K fragments read one k-step ahead of their products
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_) kf[0][kt_] = lds_load16<bf16x8>(&ks[buf][kbase[0] + 8192 * kt_]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 1 < 8) {
#pragma unroll
        for (int kt_ = 0; kt_ < 4; ++kt_) kf[(st + 1) & 1][kt_] = lds_load16<bf16x8>(&ks[buf][kbase[st + 1] + 8192 * kt_]);
      }
#pragma unroll
      for (int kt_ = 0; kt_ < 4; ++kt_) acc[kt_] = mfma32x32x16(kf[st & 1][kt_], qf[st], acc[kt_]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int lim = pos - b * 128 - 4 * half;
    const bool all_visible = b * 128 + 127 <= pos0;
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = acc[kt_][i] * a.scale_log2;
        acc[kt_][i] = all_visible || (32 * kt_ + 8 * (i >> 2) + (i & 3)) <= lim ? x : -INFINITY;
      }
  };

  // One sweep, online softmax (a flash-attention forward with the proxy K as
  // both keys and values): per block the row max (both halves of the row's
  // keys: lane ^ 32), the accumulator rescaled when it grows, P = exp2(z - m)
  // and dQ^T += K^T P^T; the row's sum of P gives its log-sum-exp at the end.
  float mrun = -INFINITY, lrun = 0.f;   // lrun: this lane's half of the row
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int b = 0; b < nblk; ++b) {
    const int buf = 0;
    load_blk(b);
    __syncthreads();   // every wave is done with the previous block's tiles
    store_blk(b, buf, true);
    __syncthreads();
    f32x16 acc[4];
    scores(b, buf, acc);
    float bm = -INFINITY;
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_)
#pragma unroll
      for (int i = 0; i < 16; i += 2) bm = max3f(bm, acc[kt_][i], acc[kt_][i + 1]);
    bm = wave_max32(bm);
    const float mnew = fmaxf(mrun, bm);   // finite: key 0 of block 0 is visible to every row
    if (mnew > mrun) {
      const float alpha = fast_exp2(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      mrun = mnew;
    }
    bf16x8 pf[4][2];
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 pw;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int i0 = 8 * u + 2 * tt;
          const float p0 = fast_exp2(acc[kt_][i0] - mrun), p1 = fast_exp2(acc[kt_][i0 + 1] - mrun);
          lrun += p0 + p1;
          const bf16x2 two = {(__bf16)p0, (__bf16)p1};
          pw[tt] = __builtin_bit_cast(int, two);
        }
        pf[kt_][u] = __builtin_bit_cast(bf16x8, pw);
      }
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 lo4 = lds_read_tr16(&kt[buf][vbase[dt] + 256 * (32 * kt_ + 16 * u)]);
          const s16x4 hi4 = lds_read_tr16(&kt[buf][vbase[dt] + 256 * (32 * kt_ + 16 * u + 8)]);
          oacc[dt] = mfma32x32x16(join_tr16(lo4, hi4), pf[kt_][u], oacc[dt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float lt = wave_sum32(lrun);
  if (live && half == 0) a.plse[(int64_t)r * a.P + p] = (mrun + fast_log2(lt)) * kLn2;
  const float inv_l = 1.f / lt;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] *= inv_l;
  // C[dim][row]: register i of tile dt holds dim 32 dt + 8 (i / 4) + 4 half + i % 4
  if (live) {
    float* dst = a.dpq + ((int64_t)r * a.P + p) * 128 + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4* d4 = reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * r4);
        const f32x4 sp = *d4;
        *d4 = f32x4{a.out_scale * (oacc[dt][4 * r4] - sp[0]), a.out_scale * (oacc[dt][4 * r4 + 1] - sp[1]),
                    a.out_scale * (oacc[dt][4 * r4 + 2] - sp[2]), a.out_scale * (oacc[dt][4 * r4 + 3] - sp[3])};
      }
  }
}

struct KlDkArgs {
  const uint8_t* pq;      // bf16 [T, P, 128]
  const uint8_t* pk;      // bf16 [N, P, 128, 128]
  const int32_t* kv_indices;
  DevMeta m;
  const float* plse;      // [T, P], natural log
  float* dpk;             // [N, P, 128, 128]: sparse term on entry, gradient on exit
  int32_t P;
  float scale_log2, out_scale;
};

__global__ __launch_bounds__(256) void kl_dense_dk_kernel(KlDkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t qt[2][32 * 256];   // a chunk's 32 proxy q rows, rt_swz
  __shared__ __attribute__((aligned(16))) float l2_s[2][32];
  __shared__ __attribute__((aligned(16))) int32_t pos_s[2][32];
  // block-major order: early blocks, seen by the most rows, start first
  const int gb = blockIdx.x / a.P, p = blockIdx.x % a.P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = upper_bound_i32(a.m.page_start, a.m.S + 1, gb) - 1;
  const int b = gb - a.m.page_start[s];
  const int32_t page = a.kv_indices[gb];
  const int32_t first_pos = a.m.kv[s] - a.m.qo[s];
  const int32_t i0 = max(0, 128 * b - first_pos);          // first row that sees the block
  const int32_t nrows = a.m.qo[s] - i0;
  const int32_t r0 = a.m.row_start[s] + i0;
  const int half = lane >> 5, j = lane & 31;
  // this wave's 32 proxy K rows, the B operand of every chunk's S (rows past
  // kv_len zeroed)
  bf16x8 bk[8];
  {
    const int krow = 32 * wave + j;
    const bool live_row = krow < a.m.kv[s] - b * 128;
    const uint8_t* kb = a.pk + ((int64_t)page * a.P + p) * 32768 + krow * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) bk[st] = live_row ? *reinterpret_cast<const bf16x8*>(kb + st * 32) : bf16x8{};
  }
  const int q16 = lane >> 4, m16 = lane & 15;
  const int keypos = b * 128 + 32 * wave + j;
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
  const int nchunks = (nrows + 31) / 32;
  // gather slots: rows ri0 and ri0 + 16 of a chunk, 16-byte column cc; the
  // next chunk's rows are loaded while this one computes
  const int ri0 = tid >> 4, cc = tid & 15, ri1 = ri0 + 16;
  auto row_ptr = [&](int chunk, int ri) {
    const int i = min(chunk * 32 + ri, nrows - 1);
    return reinterpret_cast<const i32x4*>(a.pq + ((int64_t)(r0 + i) * a.P + p) * 256 + cc * 16);
  };
  if (nchunks > 0) {
    i32x4 rq0 = *row_ptr(0, ri0), rq1 = *row_ptr(0, ri1);
    float rlse = 0.f;
    if (tid < 32) rlse = a.plse[(int64_t)(r0 + min(tid, nrows - 1)) * a.P + p];
    for (int chunk = 0; chunk < nchunks; ++chunk) {
      const int buf = chunk & 1;
      lds_store16<i32x4>(&qt[buf][rt_swz(ri0, cc)], rq0);
      lds_store16<i32x4>(&qt[buf][rt_swz(ri1, cc)], rq1);
      if (tid < 32) {
        const int i = chunk * 32 + tid;
        l2_s[buf][tid] = rlse * kLog2e;
        pos_s[buf][tid] = i < nrows ? first_pos + i0 + i : -1;   // padding rows see no key
      }
      rq0 = *row_ptr(chunk + 1, ri0);
      rq1 = *row_ptr(chunk + 1, ri1);
      if (tid < 32) rlse = a.plse[(int64_t)(r0 + min((chunk + 1) * 32 + tid, nrows - 1)) * a.P + p];
      lds_barrier();
      const uint8_t* qb = qt[buf];
      // S = Q K^T for this wave's 32 keys: C[row][key], key on lanes
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 aq = lds_load16<bf16x8>(&qb[rt_swz(j, 2 * st + half)]);
        sacc = mfma32x32x16(aq, bk[st], sacc);
      }
      f32x4 l2v[4];
      i32x4 ps4[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        l2v[t4] = *reinterpret_cast<const f32x4*>(&l2_s[buf][8 * t4 + 4 * half]);
        ps4[t4] = *reinterpret_cast<const i32x4*>(&pos_s[buf][8 * t4 + 4 * half]);
      }
      // P (register r holds row 8 (r / 4) + 4 half + r % 4) as bf16 A operands
      bf16x8 pf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 pw;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          float pv[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int rr = 8 * u + 2 * tt + x;
            const float ex = fast_exp2(__builtin_fmaf(sacc[rr], a.scale_log2, -l2v[rr >> 2][rr & 3]));
            pv[x] = keypos <= ps4[rr >> 2][rr & 3] ? ex : 0.f;
          }
          const bf16x2 p2 = {(__bf16)pv[0], (__bf16)pv[1]};
          pw[tt] = __builtin_bit_cast(int, p2);
        }
        pf[u] = __builtin_bit_cast(bf16x8, pw);
      }
      // dK += P^T Q: the q rows read transposed
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 qlo = lds_read_tr16(&qb[vlo[dt] + 256 * (16 * u)]);
          const s16x4 qhi = lds_read_tr16(&qb[vhi[dt] + 256 * (16 * u)]);
          dkacc[dt] = mfma32x32x16(pf[u], join_tr16(qlo, qhi), dkacc[dt]);
        }
    }
  }
  // C[key][d]: lane (d, half), register r -> key 32 wave + 8 (r / 4) + 4 half + r % 4
  const int64_t pbase = ((int64_t)page * a.P + p) * 128;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 32 * wave + 8 * (r >> 2) + 4 * half + (r & 3);
      const int64_t o = (pbase + kk) * 128 + 32 * dt + j;
      a.dpk[o] = a.out_scale * (dkacc[dt][r] - a.dpk[o]);
    }
}

}  // namespace

hipError_t launch_proxy_kl_dense(const msa_plan_s* p, const DevMeta& m, const int32_t* kv_indices,
                                 const KlOperands& kl, hipStream_t st) {
  const int P = p->d.num_kv_heads;
  const float scale_log2 = kl.proxy_scale * kLog2e;
  const float out_scale = kl.proxy_scale * kl.grad_scale;
  {
    KlDqArgs a{static_cast<const uint8_t*>(kl.pq), static_cast<const uint8_t*>(kl.pkp), kv_indices, m, kl.plse,
               kl.dpq, P, scale_log2, out_scale};
    ProfEvents pe(p, "kl_dense_dq");
    hipExtLaunchKernelGGL(kl_dense_dq_kernel, dim3((unsigned)(4 * p->ntiles), (unsigned)P), dim3(256), 0, st,
                          pe.start, pe.stop, 0, a);
  }
  {
    KlDkArgs a{static_cast<const uint8_t*>(kl.pq), static_cast<const uint8_t*>(kl.pkp), kv_indices, m, kl.plse,
               kl.dpk, P, scale_log2, out_scale};
    ProfEvents pe(p, "kl_dense_dk");
    hipExtLaunchKernelGGL(kl_dense_dk_kernel, dim3((unsigned)(p->NB * P)), dim3(256), 0, st, pe.start, pe.stop, 0,
                          a);
  }
  return hipGetLastError();
}

}  // namespace msa
