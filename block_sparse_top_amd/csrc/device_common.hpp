// Device helpers shared by the MSA kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (checked on hardware):
//   v_mfma_f32_32x32x16_bf16: A[i][k] in lane (i + 32*(k/8)), element k%8;
//     B[k][j] in lane (j + 32*(k/8)), element k%8;
//     C[i][j] in lane (j + 32*((i/4)%2)), register 4*(i/8) + i%4.
//   v_mfma_f32_16x16x32_bf16: A[i][k] in lane (i + 16*(k/8)), element k%8;
//     B[k][j] in lane (j + 16*(k/8)), element k%8;
//     C[i][j] in lane (j + 16*(i/4)), register i%4.
//   v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales): as 32x32x16 with
//     32 consecutive k per lane half: A[i][k] in lane (i + 32*(k/32)), byte k%32.
//     With an E2M1 (FP4) A operand (4 registers) lane (i + 32h) instead holds
//     k = 16h..16h+15 as codes 0-15 and k = 32+16h..47+16h as codes 16-31
//     (code n in bits 4n..4n+3), and its own E8M0 scale byte (op_sel) scales
//     all 32 of them.
// Because a contraction is a sum over k, A and B may both use any one
// permutation of k; the kernels exploit that to load 16- or 32-byte runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kBlock = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_huge_valf();

#define MSA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp8 e4m3 x fp8 e4m3, block scales fixed at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Eight OCP e4m3 codes (two dwords) -> eight bf16, exactly (v_cvt_scalef32_pk_bf16_fp8
// with unit scale; the last argument picks bytes 0-1 or 2-3).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  const i32x4 r = {__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), __builtin_bit_cast(int, c),
                   __builtin_bit_cast(int, d)};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max(a, b, c) as one v_max3_f32.  Written as an instruction because the
// compiler otherwise quiets every operand it cannot prove canonical (one
// extra v_max per matrix-core result); the operands here are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(a, fmaxf(b, c));
#endif
}

// max(a, |b|, |c|) as one v_max3_f32 with absolute-value source modifiers
// (through max3f the compiler clears each sign bit with a v_and first).
__device__ __forceinline__ float absmax3f(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(a, fmaxf(fabsf(b), fabsf(c)));
#endif
}

// The values of v in lanes lane % 32 (.x) and 32 + lane % 32 (.y): the two
// half-waves swapped in registers by v_permlane32_swap, with no LDS round
// trip (a shuffle through ds_bpermute sits on the critical path of every
// cross-half reduction).
__device__ __forceinline__ f32x2 wave_halves32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// max(v, v of lane ^ 32) and v + v of lane ^ 32, the same in both lanes
__device__ __forceinline__ float wave_max32(float v) {
  const f32x2 h = wave_halves32(v);
  return max3f(h[0], h[1], h[1]);
}
__device__ __forceinline__ float wave_sum32(float v) {
  const f32x2 h = wave_halves32(v);
  return h[0] + h[1];
}

// Read 16 bytes from LDS.
template <typename T>
__device__ __forceinline__ T lds_load16(const void* p) {
  return *(const MSA_LDS T*)(p);
}
template <typename T>
__device__ __forceinline__ void lds_store16(void* p, const T& v) {
  *(MSA_LDS T*)(p) = v;
}

__device__ __forceinline__ void lds_store8(void* p, const i32x2& v) { *(MSA_LDS i32x2*)(p) = v; }

// Order one wave's LDS writes before its following LDS reads of other lanes'
// data (a wave executes in lockstep and its LDS operations complete in order;
// the fences keep the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// global_load_lds_dwordx4: each lane's 16 bytes at `g` land at LDS
// `l + 16 * lane` (l is wave-uniform; it goes through M0).  The body exists
// only in the device pass (the builtin has no host meaning).
__device__ __forceinline__ void global_load_lds16(const void* g, MSA_LDS void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}

// The same load issued from inline assembly, so that the compiler does not
// track it: it then puts no wait for it before the following LDS reads,
// which it cannot tell apart from the load's destination (and would make
// wait for the load right after its issue).  No register receives data; M0
// is set in the same block (one wait state before the load reads it).  The
// caller orders the load before every read of its destination itself: a
// vmcnt wait for it, then a barrier.
__device__ __forceinline__ void global_load_lds16_untracked(const void* g, MSA_LDS void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(g) : "memory", "m0");
#endif
}

// Wait for all outstanding vector memory operations only (loads and stores;
// on this architecture one counter covers both, in issue order).
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  // simm16: vmcnt bits [3:0] and [15:14] = 0, expcnt [6:4] = 7, lgkmcnt [11:8] = 15 (no wait)
  __builtin_amdgcn_s_waitcnt(0x0f70);
#endif
}

// Wait for every outstanding memory counter (vector memory, LDS, exports).
// Wait until at most N of this wave's vector memory operations are
// outstanding (N < 64; loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
#if defined(__HIP_DEVICE_COMPILE__)
  // simm16: vmcnt [3:0] and [15:14], expcnt [6:4] = 7 and lgkmcnt [11:8] = 15 (no wait on those)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
#endif
}

__device__ __forceinline__ void wait_all_mem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0);
#endif
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 4 bf16 read by lane 4*e + i/4, for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MSA_LDS s16x4*)(p));
}
// ds_read_b64_tr_b8: within each group of 16 lanes, lane i receives byte
// (i % 8) of the 8 bytes read by lane 2*e + i/8, for e = 0..7.
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MSA_LDS i32x2*)(p));
}

// Two transposed 4 x bf16 reads -> one 8 x bf16 MFMA operand (whole-vector
// casts: element-wise reassembly of these results has been miscompiled).
__device__ __forceinline__ bf16x8 join_tr16(const s16x4& lo, const s16x4& hi) {
  const i32x2 a = __builtin_bit_cast(i32x2, lo), b = __builtin_bit_cast(i32x2, hi);
  const i32x4 r = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  return __builtin_bit_cast(bf16x8, r);
}

// The value of another lane, chosen by the DPP control CTRL (quad
// permutations, row mirrors) within each 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  // every lane's source exists for these controls; the update form (old 0,
  // bound_ctrl) lets the compiler fold the move into the consuming add
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// K and V sit in LDS as unpadded 256-byte rows whose 16-byte chunks are
// XOR-swizzled by row.  K: chunk c of row r at c ^ (r & 15), so each 16 lanes
// of an MFMA operand read (16 rows, one column chunk) hit 16 distinct chunk
// positions.  V: chunk c at c ^ 4 (r & 3), so the 8 rows x 4 chunks of a
// transposed read cover every bank exactly twice.  The per-lane part of each
// read address is computed once (8 K bases, one per 32-byte column step; 4 V
// bases, one per 32-column tile) and the row offsets become immediates.
__device__ __forceinline__ int k_swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// Tiles read both row-wise (16 consecutive rows at one 16-byte chunk: the
// A operands) and transposed (ds_read_b64_tr_b16 over groups of 4 rows): the
// chunk is XORed with a bijection of the row's low 4 bits whose row & 3 part
// moves chunk bits 2-3, so each 16-lane phase of either pattern touches every
// bank once (k_swz: the transposed reads collide pairwise; v_swz: the
// row-wise reads collide 4 ways).
__device__ __forceinline__ int rt_swz_key(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int rt_swz(int row, int chunk) { return row * 256 + ((chunk ^ rt_swz_key(row)) << 4); }
__device__ __forceinline__ int v_swz(int row, int chunk) { return row * 256 + ((chunk ^ ((row & 3) << 2)) << 4); }

// A workgroup barrier that waits only for this wave's LDS traffic, so global
// loads issued before it (the next chunk's rows) stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Number of set bits of a wave mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int upper_bound_i32(const int32_t* a, int n, int32_t x) {
  // first index i in [0, n) with a[i] > x (a ascending)
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

}  // namespace msa
