// Exact re-scoring of proxy blocks for the low-precision proxy formats.
//
// The matrix cores do not sum fp8 (and fp8 x FP4) products exactly: on
// gfx950 a product far below the largest one of its group loses low bits, so
// a block score from v_mfma_scale_f32_32x32x64_f8f6f4 can be off by up to
// about 2^-10.7 of max|q| * max|k| (scaled) -- measured over random and
// adversarial operands.  Selection must not depend on that: the block-score
// indexer of the Flash-MSA article (paragraph on the forward kernels) and the
// README's `sparse_topk_select` rank blocks by their proxy scores, so blocks
// whose low-precision scores lie within the error bound of the top-k boundary
// are scored again here, exactly: every product of two stored codes is exact
// in fp32, the 128 products of a key are summed in fp32 (relative error
// below 2^-18 of sum |products|), and the scales are applied once.
//
// One wave re-scores one block.  Lane l owns dims 32 (l >> 4) .. +31 (one
// MXFP4 scale block) and keys (l & 15) + 16 i, i = 0..7.
#pragma once

#include "device_common.hpp"

namespace msa {

// Proxy (q, K) formats: bf16 x bf16, fp8 x fp8, fp8 q x MXFP4 K, MXFP4 q x
// MXFP4 K.
enum class Fmt : int { BF16 = 0, FP8 = 1, MX4K = 2, MX4QK = 3 };

// Bound on |low-precision score - exact score| per unit of
// proxy_sm_scale * max|q_d| * max|k_jd| (value units).  Measured worst case:
// 2^-10.7 (fp8 x fp8), 2^-11.3 (fp8 x FP4), 2^-19.7 (FP4 x FP4) over eight
// operand distributions; the bounds below are 3.2x and 8x above them.
template <Fmt F>
struct ScoreBound {
  static constexpr float kCoef = F == Fmt::MX4QK ? 0x1p-17f : 0x1p-9f;
};

// E2M1 code (4 bits) -> value, exact: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives
// (the q row; key codes go through the hardware conversion, which gives the
// same values).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

// The largest |value| of the e4m3 codes packed in w (four bytes), as a code value.
__device__ __forceinline__ float e4m3_absmax4(uint32_t w) {
  const uint32_t a = w & 0x7f7f7f7fu;  // magnitude codes order like their values
  const uint32_t m = max(max(a & 0xffu, (a >> 8) & 0xffu), max((a >> 16) & 0xffu, a >> 24));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(m, 1.0f, false);
  return v[0];
}

// The largest byte of w.
__device__ __forceinline__ uint32_t max_byte4(uint32_t w) {
  return max(max(w & 0xffu, (w >> 8) & 0xffu), max((w >> 16) & 0xffu, w >> 24));
}

// 2^(e - 127) for an E8M0 scale code e (0..254), exact.
__device__ __forceinline__ float e8m0_value(uint32_t e) { return __builtin_ldexpf(1.0f, (int)e - 127); }

// The lane's q dims as code values (fp8: e4m3 code values, unscaled; MXFP4:
// E2M1 values) and, for MXFP4 q, its block's scale code.
struct ExactQ {
  float v[32];
  uint32_t e;
};

template <Fmt F>
__device__ __forceinline__ ExactQ exact_load_q(const uint8_t* row) {
  ExactQ q;
  const int dq = (threadIdx.x & 63) >> 4;
  if constexpr (F == Fmt::MX4QK) {
    // 64 code bytes (element 2i in the low nibble of byte i), then 4 scale bytes
    const uint8_t* c = row + 16 * dq;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = c[i];
      q.v[2 * i] = e2m1_value(b & 15u);
      q.v[2 * i + 1] = e2m1_value(b >> 4);
    }
    q.e = row[64 + dq];
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row + 32 * dq);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t x = w[i];
      const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, false);
      const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, true);
      q.v[4 * i] = a[0];
      q.v[4 * i + 1] = a[1];
      q.v[4 * i + 2] = b[0];
      q.v[4 * i + 3] = b[1];
    }
    q.e = 127;
  }
  return q;
}

// max over keys j < nkeys of sum_d q_d k_jd, in code units with the MXFP4
// block scales applied (the caller applies proxy_sm_scale and the fp8 head
// scales).  `blk`: the block's proxy-K page of one head (fp8: 128 rows of 128
// codes; MXFP4: the 8704-byte record).  Uniform result.
template <Fmt F>
__device__ __forceinline__ float exact_block_dotmax(const ExactQ& q, const uint8_t* blk, int nkeys) {
  const int lane = threadIdx.x & 63;
  const int dq = lane >> 4, kk = lane & 15;
  // every load of the block is issued before any arithmetic (one round trip)
  constexpr int kV = F == Fmt::FP8 ? 2 : 1;
  i32x4 x[8][kV];
  uint32_t ke[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = 16 * i + kk;
    if constexpr (F == Fmt::FP8) {
      const i32x4* src = reinterpret_cast<const i32x4*>(blk + key * 128 + 32 * dq);
      x[i][0] = src[0];
      x[i][kV - 1] = src[1];
      ke[i] = 127;
    } else {
      x[i][0] = *reinterpret_cast<const i32x4*>(blk + key * 64 + 16 * dq);
      ke[i] = blk[128 * 64 + key * 4 + dq];
    }
  }
  float best = kNegInf;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = 16 * i + kk;
    float acc = 0.f;
    if constexpr (F == Fmt::FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t c = (uint32_t)x[i][h][w];
          const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
          const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, true);
          const int d = 16 * h + 4 * w;
          acc = __builtin_fmaf(q.v[d], a[0], acc);
          acc = __builtin_fmaf(q.v[d + 1], a[1], acc);
          acc = __builtin_fmaf(q.v[d + 2], b[0], acc);
          acc = __builtin_fmaf(q.v[d + 3], b[1], acc);
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t c = (uint32_t)x[i][0][w];
        // byte n of the word: element 2n in the low nibble, 2n + 1 in the high one
        const f32x2 k0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
        const f32x2 k1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
        const f32x2 k2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
        const f32x2 k3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
        acc = __builtin_fmaf(q.v[8 * w], k0[0], acc);
        acc = __builtin_fmaf(q.v[8 * w + 1], k0[1], acc);
        acc = __builtin_fmaf(q.v[8 * w + 2], k1[0], acc);
        acc = __builtin_fmaf(q.v[8 * w + 3], k1[1], acc);
        acc = __builtin_fmaf(q.v[8 * w + 4], k2[0], acc);
        acc = __builtin_fmaf(q.v[8 * w + 5], k2[1], acc);
        acc = __builtin_fmaf(q.v[8 * w + 6], k3[0], acc);
        acc = __builtin_fmaf(q.v[8 * w + 7], k3[1], acc);
      }
      // the key's and (MXFP4 q) the row's block scales: exact powers of two
      acc = __builtin_ldexpf(acc, (int)ke[i] - 127 + (int)q.e - 127);
    }
    // the four dim blocks of a key sit in lanes kk, kk + 16, kk + 32, kk + 48
    acc += __shfl_xor(acc, 16);
    acc = wave_sum32(acc);
    best = key < nkeys ? fmaxf(best, acc) : best;
  }
  // max over the 16 key lanes of a row
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) best = fmaxf(best, __shfl_xor(best, o));
  return best;
}

}  // namespace msa
