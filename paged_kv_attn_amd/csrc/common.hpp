// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Operand layouts of the matrix-core instructions used here (wave64; lane l):
//   v_mfma_f32_32x32x16_bf16 / _fp8_fp8:  A[i][k] in lane (i + 32*(k/8)), slot k%8;
//       B[k][j] in lane (j + 32*(k/8)), slot k%8;
//       C[i][j] in lane (j + 32*((i/4)%2)), register 4*(i/8) + i%4.
//   v_mfma_f32_16x16x32_bf16:  A[i][k] in lane (i + 16*(k/8)), slot k%8;
//       B[k][j] in lane (j + 16*(k/8)), slot k%8;
//       C[i][j] in lane (j + 16*(i/4)), register i%4.
//   ds_read_b64_tr_b16 (per group of 16 lanes): lane L supplies an 8-byte LDS
//       address holding 4 16-bit values x_L[0..3]; lane l receives
//       { x_{4j + l/4}[l%4] : j = 0..3 }.
// These were checked on the hardware with in-bounds probes before use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// LDS byte pointer. Kernels that pass LDS addresses around (through lambdas,
// slot selects) keep them in this type: a generic pointer converted back to an
// LDS address costs a null check per use.
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

struct alignas(16) U128 { uint32_t x, y, z, w; };
struct alignas(8) U64 { uint32_t x, y; };

__device__ __forceinline__ bf16x8 as_bf16x8(const U128& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(const U64& a, const U64& b) {
  U128 u{a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 A and B and unit scales (E8M0 127):
// the full-rate fp8 product. Lane i + 32 h supplies 32 bytes, k = 32 h .. 32 h + 31,
// of A's row i and of B's column i (checked on the hardware with an in-bounds
// probe: A and B pair byte for byte); C as for the other 32x32 shapes.
__device__ __forceinline__ f32x16 mfma32x64_fp8(const U128& a0, const U128& a1, const U128& b0, const U128& b1,
                                               const f32x16& c) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma32_fp8(const U64& a, const U64& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b),
                                                    c, 0, 0, 0);
}

// 4 bf16 values of one LDS transpose read (see the layout note above).
// 16 bytes from LDS (ds_read_b128).
__device__ __forceinline__ U128 lds_load16(const lds_char* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)p;
  return __builtin_bit_cast(U128, v);
}

// 8 bytes from LDS (ds_read_b64).
__device__ __forceinline__ U64 lds_load8(const lds_char* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *(const __attribute__((address_space(3))) u32x2*)p;
  return __builtin_bit_cast(U64, v);
}
// 8 bytes to LDS (ds_write_b64).
__device__ __forceinline__ void lds_store8(lds_char* p, const U64& x) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  *(__attribute__((address_space(3))) u32x2*)p = __builtin_bit_cast(u32x2, x);
}
// 16 bytes to LDS (ds_write_b128).
__device__ __forceinline__ void lds_store16(lds_char* p, const U128& x) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  *(__attribute__((address_space(3))) u32x4*)p = __builtin_bit_cast(u32x4, x);
}

__device__ __forceinline__ U64 lds_read_tr16(const lds_char* lds_addr) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_addr);
  return __builtin_bit_cast(U64, v);
}
__device__ __forceinline__ U64 lds_read_tr16(const void* lds_addr) {
  auto p = (lds_s16x4*)(lds_addr);
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  return __builtin_bit_cast(U64, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Value from the lane 32 places away, combined with this lane's by max / sum.
// v_permlane32_swap swaps the upper half of its first operand with the lower
// half of its second; swapping x with itself hands each lane (r0, r1) =
// (x[l mod 32], x[l mod 32 + 32]), i.e. both halves' values in every lane.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even pack of two floats into bf16x2 (low half = a); one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Index of this thread's wave in the workgroup, as a scalar (wave-uniform)
// value so that everything derived from it stays in scalar registers and
// branches on it stay uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Raw buffer resource over [base, base + bytes): 128-bit loads at byte offsets
// at or beyond `bytes` return zeros (hardware range check), which zero-fills
// tile rows past a sequence's end without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds_wave_base + 16 l (one contiguous 1 KiB block per wave instruction); bytes
// outside the buffer's range arrive as zeros. Tracked by vmcnt.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, byte_off,
                                           0, 0, 0);
}

__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, lds_char* lds_wave_base, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, byte_off, 0, 0, 0);
}

// As buf_load16_lds, with the non-temporal cache policy: for data read once
// (streamed KV), so it does not displace reusable lines in L2.
__device__ __forceinline__ void buf_load16_lds_stream(__amdgpu_buffer_rsrc_t r, lds_char* lds_wave_base, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, byte_off, 0, 0, /*nt*/ 2);
}

// Wait until this wave's vector-memory loads (including loads into LDS) have
// completed: s_waitcnt vmcnt(0) with the LDS and export counters left free.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// ... until at most N of them are outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ U128 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return __builtin_bit_cast(U128, v);
}

// Four floats -> four OCP E4M3FN bytes (low byte = a), round to nearest even,
// saturated to +-448 first (so finite inputs never become NaN).
__device__ __forceinline__ uint32_t pack_fp8x4_sat(float a, float b, float c, float d) {
  const float m = 448.0f;
  a = __builtin_fminf(__builtin_fmaxf(a, -m), m);
  b = __builtin_fminf(__builtin_fmaxf(b, -m), m);
  c = __builtin_fminf(__builtin_fmaxf(c, -m), m);
  d = __builtin_fminf(__builtin_fmaxf(d, -m), m);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// 8 fp8 bytes -> 8 bf16 (exact: every E4M3FN value is a bf16 value), two
// values per v_cvt_scalef32_pk_bf16_fp8 with a unit scale (word_sel picks
// bytes 0-1 or 2-3 of the source; byte 2k lands in the low half).
__device__ __forceinline__ U128 fp8x8_to_bf16x8(U64 in) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)in.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)in.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)in.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)in.y, 1.0f, true);
  return U128{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
              __builtin_bit_cast(uint32_t, d)};
}

// K/V batch entry read by batch entry b: idx[b] with a cache batch index, else
// b; -1 (no keys) for an index outside [0, count).
__device__ __forceinline__ int kv_entry(const int32_t* idx, int count, int b) {
  if (!idx) return b;
  const int e = idx[b];
  return (e >= 0 && e < count) ? e : -1;
}

// tanh for the logit soft-cap, from exp: tanh(x) = sign(x) (1 - e) / (1 + e),
// e = exp(-2|x|). Relative error a few ulp of fp32 away from 0; near 0 the
// absolute error is ~1e-7, far below the bf16 rounding of P.
__device__ __forceinline__ float tanh_fast(float x) {
  float ax = fabsf(x);
  float e = fast_exp2(-2.0f * kLog2e * ax);
  float t = (1.0f - e) * fast_rcp(1.0f + e);
  return copysignf(t, x);
}

// Soft-capped logit cap * tanh(y), y = x * pre, in the kernels' log2 units
// (post = cap * log2 e), from the identity tanh(y) = 1 - 2 / (1 + e^(2y)):
// one exp, one reciprocal, an add and an FMA; k2 = 2 log2(e) * pre.
// y -> +inf: e^(2y) = inf, reciprocal 0, result post; y -> -inf: result -post.
// Absolute error ~ post * 2^-23 (the cancellation in 1 - 2r near y = 0).
__device__ __forceinline__ float softcap_logit(float x, float k2, float post) {
  const float r = fast_rcp(1.0f + fast_exp2(x * k2));
  return __builtin_fmaf(r, -2.0f * post, post);
}

}  // namespace attn
