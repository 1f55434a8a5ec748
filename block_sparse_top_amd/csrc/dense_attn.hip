// Dense causal GQA attention, the warm-up mode of the Flash-MSA article
// (backward paragraph: a warm-up in which the main attention runs densely,
// without block indexes, and the proxy learns only in the backward pass).
//
//  1. dense_fwd: per (group, run of 128 / G query tokens of one proxy row
//     tile), the G heads of those tokens (128 rows, 4 waves x 32) against
//     every visible 128-key block: S^T = K Q^T, online softmax (the row's max
//     over both lane halves, the accumulator rescaled as it grows), O^T +=
//     V^T P^T; out (bf16) and lse.  K and V of the next block are loaded into
//     registers while the current one is multiplied; LDS tiles are
//     double-buffered behind one barrier per block.
//  2. dense_dq: the same rows and blocks for the backward: S^T, P^T from the
//     forward's lse, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
//     With the proxy distillation term it also accumulates pk^T P^T and
//     stores (1/G) of its sum over each token's heads into dproxy_q (the
//     dense p_main part that the dense proxy kernel subtracts).
//  dk and dv come from the key-centric backward kernel in its dense form.
#include "device_common.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr float kLn2d = 0.6931471805599453f;

// Query rows of a workgroup: tokens [u * TW, (u + 1) * TW) of a proxy row
// tile (TW = 128 / G) for one group, row qr = 32 wave + j <-> token qr / G,
// head qr % G.
struct DenseRows {
  int s, row0, pos0, n_tok;   // sequence, first row and position of the run, live tokens
  int r, pos, h, hh, tok;     // this lane's row
  bool live;
};

__device__ __forceinline__ bool dense_rows(const DevMeta& m, int G, int g, int wave, int j, DenseRows& d) {
  const int TW = 128 / G, subs = 4 * G;
  const int qi = (int)gridDim.x - 1 - (int)blockIdx.x;   // later tiles (more keys) start first
  const int t = qi / subs, u = qi % subs;
  const int n = m.tiles[4 * t + 2] - u * TW;
  if (n <= 0) return false;
  d.s = m.tiles[4 * t];
  d.row0 = m.tiles[4 * t + 1] + u * TW;
  d.pos0 = m.tiles[4 * t + 3] + u * TW;
  d.n_tok = min(n, TW);
  const int qr = 32 * wave + j;
  d.hh = qr % G;
  d.tok = qr / G;
  d.live = d.tok < d.n_tok;
  const int tk = min(d.tok, d.n_tok - 1);
  d.r = d.row0 + tk;
  d.pos = d.pos0 + tk;
  d.h = g * G + d.hh;
  return true;
}

struct DenseFwdArgs {
  const uint8_t* q;       // bf16 [T, Hq, 128]
  const uint8_t* kp;      // bf16 [N, Hkv, 128, 128]
  const uint8_t* vp;
  const int32_t* kv_indices;
  DevMeta m;
  uint16_t* out;          // bf16 [T, Hq, 128]
  float* lse;             // [T, Hq], natural log
  int32_t Hq, Hkv, G;
  float scale_log2;
};

__global__ __launch_bounds__(256, 2) void dense_fwd_kernel(DenseFwdArgs a) {
  // one K and one V tile (64 KB): two workgroups share a CU, and one's block
  // loads overlap the other's MFMAs
  __shared__ __attribute__((aligned(16))) uint8_t ks[1][128 * 256];   // K, k_swz: S^T operand
  __shared__ __attribute__((aligned(16))) uint8_t vt[1][128 * 256];   // V, v_swz: transposed reads
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int q16 = lane >> 4, m16 = lane & 15;
  DenseRows d;
  if (!dense_rows(a.m, a.G, g, wave, j, d)) return;
  const int nblk = ((d.pos0 + d.n_tok - 1) >> 7) + 1;
  const int32_t* pages = a.kv_indices + a.m.page_start[d.s];
  const int kv_len = a.m.kv[d.s];
  bf16x8 qf[8];
  {
    const uint8_t* qrow = a.q + ((int64_t)d.r * a.Hq + d.h) * 256 + half * 16;
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
  i32x4 kr[8], vr[8];
  auto load_blk = [&](int b) {
    const int64_t off = ((int64_t)pages[b] * a.Hkv + g) * 32768;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kr[i] = *reinterpret_cast<const i32x4*>(a.kp + off + (tid + 256 * i) * 16);
      vr[i] = *reinterpret_cast<const i32x4*>(a.vp + off + (tid + 256 * i) * 16);
    }
  };
  auto store_blk = [&](int b, int buf) {   // rows past kv_len zeroed (0 * NaN is NaN)
    const int kv_in_block = kv_len - 128 * b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const bool live_row = (c >> 4) < kv_in_block;
      lds_store16<i32x4>(&ks[buf][k_swz(c >> 4, c & 15)], live_row ? kr[i] : i32x4{});
      lds_store16<i32x4>(&vt[buf][v_swz(c >> 4, c & 15)], live_row ? vr[i] : i32x4{});
    }
  };
  float mrun = -INFINITY, lrun = 0.f;
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int b = 0; b < nblk; ++b) {
    const int buf = 0;
    load_blk(b);
    __syncthreads();   // every wave is done with the previous block's tiles
    store_blk(b, buf);
    __syncthreads();
    // S^T = K Q^T: register i of tile kt_ holds key 32 kt_ + 8 (i / 4) + 4 half + i % 4
    // (K fragments read one k-step ahead of their products)
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    bf16x8 kf[2][4];
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
    const int lim = d.pos - b * 128 - 4 * half;
    const bool all_visible = b * 128 + 127 <= d.pos0;
    float bm = -INFINITY;
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = acc[kt_][i] * a.scale_log2;
        acc[kt_][i] = all_visible || (32 * kt_ + 8 * (i >> 2) + (i & 3)) <= lim ? x : -INFINITY;
      }
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_)
#pragma unroll
      for (int i = 0; i < 16; i += 2) bm = max3f(bm, acc[kt_][i], acc[kt_][i + 1]);
    bm = wave_max32(bm);
    const float mnew = fmaxf(mrun, bm);   // finite: key 0 is visible to every row
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
    auto make_p = [&](int kt_) __attribute__((always_inline)) {
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
    };
    // O^T += V^T P^T, with the exponentials of key tile kt_ + 1 computed
    // between the products of tile kt_
    make_p(0);
#pragma unroll
    for (int kt_ = 0; kt_ < 4; ++kt_) {
      if (kt_ + 1 < 4) make_p(kt_ + 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 lo4 = lds_read_tr16(&vt[buf][vbase[dt] + 256 * (32 * kt_ + 16 * u)]);
          const s16x4 hi4 = lds_read_tr16(&vt[buf][vbase[dt] + 256 * (32 * kt_ + 16 * u + 8)]);
          oacc[dt] = mfma32x32x16(join_tr16(lo4, hi4), pf[kt_][u], oacc[dt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float lt = wave_sum32(lrun);
  if (!d.live) return;
  if (half == 0) a.lse[(int64_t)d.r * a.Hq + d.h] = (mrun + fast_log2(lt)) * kLn2d;
  const float inv_l = 1.f / lt;
  // C[dim][row]: register i of tile dt holds dim 32 dt + 8 (i / 4) + 4 half + i % 4
  uint16_t* dst = a.out + ((int64_t)d.r * a.Hq + d.h) * 128 + 4 * half;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const bf16x2 lo2 = {(__bf16)(oacc[dt][4 * r4] * inv_l), (__bf16)(oacc[dt][4 * r4 + 1] * inv_l)};
      const bf16x2 hi2 = {(__bf16)(oacc[dt][4 * r4 + 2] * inv_l), (__bf16)(oacc[dt][4 * r4 + 3] * inv_l)};
      *reinterpret_cast<i32x2*>(dst + 32 * dt + 8 * r4) = i32x2{__builtin_bit_cast(int, lo2), __builtin_bit_cast(int, hi2)};
    }
}

struct DenseDqArgs {
  const uint8_t* q;       // bf16 [T, Hq, 128]
  const uint8_t* dout;
  const uint8_t* kp;      // bf16 [N, Hkv, 128, 128]
  const uint8_t* vp;
  const float* lse;       // [T, Hq], natural log
  const float* D;         // [T, Hq]
  const int32_t* kv_indices;
  DevMeta m;
  float* dq;              // fp32 [T, Hq, 128]
  int32_t Hq, Hkv, G;
  float scale_log2, sm_scale;
  // proxy distillation term: proxy K pool bf16 [N, Hkv, 128, 128]; dpq fp32
  // [T, Hkv, 128] receives (1/G) sum_h sum_j P_hj pk_j
  const uint8_t* pkp;
  float* dpq;
  float inv_g;
};

// K sits in LDS once (rt_swz), read directly for S^T and transposed for K^T;
// blocks are taken in two 64-key halves.  The plain variant loads each block
// straight into LDS and fits two workgroups per CU (64 KB, 256 registers),
// whose block loads overlap each other's MFMAs; with the proxy term (96 KB)
// one workgroup per CU prefetches the next block into registers instead.
template <bool KL>
__global__ __launch_bounds__(256, KL ? 1 : 2) void dense_dq_kernel(DenseDqArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[128 * 256];   // K, rt_swz: S^T operand and K^T reads
  __shared__ __attribute__((aligned(16))) uint8_t vs[128 * 256];   // V, rt_swz: dP^T operand
  __shared__ __attribute__((aligned(16))) uint8_t pkt[KL ? 128 * 256 : 16];   // proxy K, v_swz
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int q16 = lane >> 4, m16 = lane & 15;
  const int G = a.G;
  DenseRows d;
  if (!dense_rows(a.m, G, g, wave, j, d)) return;
  const int nblk = ((d.pos0 + d.n_tok - 1) >> 7) + 1;
  const int32_t* pages = a.kv_indices + a.m.page_start[d.s];
  const int kv_len = a.m.kv[d.s];
  bf16x8 qf[8], df[8];
  {
    const int64_t off = ((int64_t)d.r * a.Hq + d.h) * 256 + half * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(a.q + off + st * 32);
      df[st] = *reinterpret_cast<const bf16x8*>(a.dout + off + st * 32);
    }
  }
  const float l2 = a.lse[(int64_t)d.r * a.Hq + d.h] * kLog2e;
  const float dval = a.D[(int64_t)d.r * a.Hq + d.h];
  int kbase[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) kbase[st] = rt_swz(j, 2 * st + half);
  int vbase[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vbase[dt] = (4 * (q16 >> 1) + (m16 >> 2)) * 256 +
                ((4 * (dt ^ (m16 >> 2)) + 2 * (q16 & 1) + ((m16 & 3) >> 1)) << 4) + 8 * (m16 & 1);
  // transposed reads of the rt_swz tile: lane (q16, m16) fetches dims
  // 32 dt + 16 (q16 & 1) + 4 (m16 & 3) .. +3 of key row r0 (lo) or r0 + 8 (hi)
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
  i32x4 kr[8], vr[8], pr[KL ? 8 : 1];
  auto load_blk = [&](int b) {
    const int64_t off = ((int64_t)pages[b] * a.Hkv + g) * 32768;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kr[i] = *reinterpret_cast<const i32x4*>(a.kp + off + (tid + 256 * i) * 16);
      vr[i] = *reinterpret_cast<const i32x4*>(a.vp + off + (tid + 256 * i) * 16);
      if constexpr (KL) pr[i] = *reinterpret_cast<const i32x4*>(a.pkp + off + (tid + 256 * i) * 16);
    }
  };
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x16 kacc[KL ? 4 : 1];
#pragma unroll
  for (int dt = 0; dt < (KL ? 4 : 1); ++dt) kacc[dt] = f32x16{};
  if constexpr (KL) load_blk(0);
  for (int b = 0; b < nblk; ++b) {
    if constexpr (!KL) load_blk(b);
    __syncthreads();   // the previous block's tiles are no longer read
    {
      const int kv_in_block = kv_len - 128 * b;   // rows past kv_len zeroed
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = tid + 256 * i;
        const bool live_row = (c >> 4) < kv_in_block;
        lds_store16<i32x4>(&ks[rt_swz(c >> 4, c & 15)], live_row ? kr[i] : i32x4{});
        lds_store16<i32x4>(&vs[rt_swz(c >> 4, c & 15)], live_row ? vr[i] : i32x4{});
        if constexpr (KL) lds_store16<i32x4>(&pkt[v_swz(c >> 4, c & 15)], live_row ? pr[i] : i32x4{});
      }
    }
    if constexpr (KL) {
      if (b + 1 < nblk) load_blk(b + 1);
      lds_barrier();
    } else {
      __syncthreads();
    }
    const int lim = d.pos - b * 128 - 4 * half;
    const bool all_visible = b * 128 + 127 <= d.pos0;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {   // keys 64 kh .. 64 kh + 63
      // S^T = K Q^T, then P^T in place (hidden keys 0)
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = mfma32x32x16(lds_load16<bf16x8>(&ks[kbase[st] + 8192 * (2 * kh + t)]), qf[st], acc[t]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ex = fast_exp2(__builtin_fmaf(acc[t][i], a.scale_log2, -l2));
          acc[t][i] = all_visible || (32 * (2 * kh + t) + 8 * (i >> 2) + (i & 3)) <= lim ? ex : 0.f;
        }
      // dP^T = V dO^T
      f32x16 dacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          dacc[t] = mfma32x32x16(lds_load16<bf16x8>(&vs[kbase[st] + 8192 * (2 * kh + t)]), df[st], dacc[t]);
      // dS^T = P^T (dP^T - D) as bf16 B operands (and P^T itself for the proxy term)
      bf16x8 sf[2][2], pfk[KL ? 2 : 1][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          i32x4 pw, qw;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int i0 = 8 * u + 2 * tt;
            const bf16x2 two = {(__bf16)(acc[t][i0] * (dacc[t][i0] - dval)),
                                (__bf16)(acc[t][i0 + 1] * (dacc[t][i0 + 1] - dval))};
            pw[tt] = __builtin_bit_cast(int, two);
            if constexpr (KL) {
              const bf16x2 pp = {(__bf16)acc[t][i0], (__bf16)acc[t][i0 + 1]};
              qw[tt] = __builtin_bit_cast(int, pp);
            }
          }
          sf[t][u] = __builtin_bit_cast(bf16x8, pw);
          if constexpr (KL) pfk[t][u] = __builtin_bit_cast(bf16x8, qw);
        }
      // dQ^T += K^T dS^T (and pk^T P^T)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ro = 256 * 32 * (2 * kh + t);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const s16x4 lo4 = lds_read_tr16(&ks[ktlo[dt] + ro + 256 * 16 * u]);
            const s16x4 hi4 = lds_read_tr16(&ks[kthi[dt] + ro + 256 * 16 * u]);
            oacc[dt] = mfma32x32x16(join_tr16(lo4, hi4), sf[t][u], oacc[dt]);
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
  }
  if (d.live) {
    float* dst = a.dq + ((int64_t)d.r * a.Hq + d.h) * 128 + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * r4) =
            f32x4{oacc[dt][4 * r4] * a.sm_scale, oacc[dt][4 * r4 + 1] * a.sm_scale, oacc[dt][4 * r4 + 2] * a.sm_scale,
                  oacc[dt][4 * r4 + 3] * a.sm_scale};
  }
  if constexpr (KL) {
    // sum over the token's G heads (G aligned lanes of a 16-lane row): quad
    // xor 1 and xor 2, then the half-row and row mirrors once each quad / 8
    // holds one value; the token's first lane stores
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
    if (d.live && d.hh == 0) {
      float* dst = a.dpq + ((int64_t)d.r * a.Hkv + g) * 128 + 4 * half;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float* k4 = &kv[16 * dt + 4 * r4];
          *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * r4) =
              f32x4{k4[0] * a.inv_g, k4[1] * a.inv_g, k4[2] * a.inv_g, k4[3] * a.inv_g};
        }
    }
  }
}

}  // namespace

hipError_t launch_dense_forward(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                                const int32_t* kv_indices, void* out, float* lse, hipStream_t st) {
  DenseFwdArgs a{static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(kp), static_cast<const uint8_t*>(vp),
                 kv_indices, m, static_cast<uint16_t*>(out), lse, p->d.num_qo_heads, p->d.num_kv_heads, p->G,
                 p->d.sm_scale * kLog2e};
  ProfEvents pe(p, "dense_fwd");
  hipExtLaunchKernelGGL(dense_fwd_kernel, dim3((unsigned)(p->ntiles * 4 * p->G), (unsigned)p->d.num_kv_heads),
                        dim3(256), 0, st, pe.start, pe.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_dense_dq(const msa_plan_s* p, const DevMeta& m, const void* q, const void* kp, const void* vp,
                           const int32_t* kv_indices, const float* lse, const float* D, const void* dout, float* dq,
                           const KlOperands* kl, hipStream_t st) {
  DenseDqArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.dout = static_cast<const uint8_t*>(dout);
  a.kp = static_cast<const uint8_t*>(kp);
  a.vp = static_cast<const uint8_t*>(vp);
  a.lse = lse;
  a.D = D;
  a.kv_indices = kv_indices;
  a.m = m;
  a.dq = dq;
  a.Hq = p->d.num_qo_heads;
  a.Hkv = p->d.num_kv_heads;
  a.G = p->G;
  a.scale_log2 = p->d.sm_scale * kLog2e;
  a.sm_scale = p->d.sm_scale;
  a.pkp = kl ? static_cast<const uint8_t*>(kl->pkp) : nullptr;
  a.dpq = kl ? kl->dpq : nullptr;
  a.inv_g = 1.f / (float)p->G;
  const dim3 grid((unsigned)(p->ntiles * 4 * p->G), (unsigned)p->d.num_kv_heads);
  ProfEvents pe(p, "dense_dq");
  if (kl)
    hipExtLaunchKernelGGL(dense_dq_kernel<true>, grid, dim3(256), 0, st, pe.start, pe.stop, 0, a);
  else
    hipExtLaunchKernelGGL(dense_dq_kernel<false>, grid, dim3(256), 0, st, pe.start, pe.stop, 0, a);
  return hipGetLastError();
}

}  // namespace msa
