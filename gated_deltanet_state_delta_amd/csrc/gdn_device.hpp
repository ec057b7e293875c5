// gdn_device.hpp -- device helpers shared by the libgdn kernels (gfx950 only).
//
// Scalar conversions, the fused gate, 16-byte global accesses, DPP row
// reductions and the 16x16 MFMA fragment helpers the prefill kernel is built
// from.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned short us4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

// ----------------------------------------------------------------- scalars --

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Input element -> fp32 (bf16 widening is exact).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// fp32 -> io element, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Four consecutive io elements -> f4 (8-byte load for bf16, 16-byte for fp32).
__device__ __forceinline__ f4 load4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 load4(const __bf16* p) {
  const bf4 v = *reinterpret_cast<const bf4*>(p);
  return f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// ------------------------------------------------------------------- gate --
// The "qwen" gate of the ONNX GatedDeltaNet card / the fused gate of the
// FlashInfer decode page: g = -exp(A_log) * softplus(a + dt_bias), softplus
// being the identity above 20.  Accurate libm forms: the gate is not hot.

__device__ __forceinline__ float softplus20(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

__device__ __forceinline__ float gate_log_decay(float A_log, float dt_bias, float a) {
  return -expf(A_log) * softplus20(a + dt_bias);
}

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// The same gates from the hardware exp2 / log2 / reciprocal (relative error
// about 1e-6), for the fused gate on a prefill prep wave's critical path.
// eA = exp(A_log) is computed once per head.
__device__ __forceinline__ float gate_log_decay_fast(float eA, float dt_bias, float a) {
  const float x = a + dt_bias;
  const float sp = x > 20.0f ? x
                             : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(x * 1.4426950408889634f)) *
                                   0.6931471805599453f;
  return -eA * sp;
}
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// ------------------------------------------------------- 16-byte accesses --
// Non-temporal loads/stores for data touched exactly once (state pools).

__device__ __forceinline__ f4 ld_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void st_nt(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}

// ---------------------------------------------------------- raw buffers --
// Buffer resources for row-structured streams: one 4-SGPR resource per base
// pointer, a per-lane byte offset that stays constant (voffset) and a
// wave-uniform row offset (soffset), so a load or store costs no VALU work.
// The range check is effectively off (records = 2^32 - 1); callers only use
// these for rows known to be in bounds.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
// A resource covering `bytes` bytes from `base` (accesses past them read
// zeros and touch no memory), its fields taken through readfirstlane so the
// compiler keeps it in SGPRs (a resource it cannot prove uniform makes it
// loop over the lanes' distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_n(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}
template <typename E> __device__ __forceinline__ E buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ __bf16 buf_load<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(__bf16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
template <> __device__ __forceinline__ float buf_load<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, __bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// DPP moves: lanes whose row is not in ROWMASK (or whose source lane lies
// outside the row for the shifts) receive `fill`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f(float fill, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i(int fill, int v) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROWMASK, 0xF, false);
}
// Inclusive wave-wide scans (sum, max) in lane order: shifts within 16-lane
// rows (row_shr 1, 2, 4, 8), then the row totals carried across rows
// (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3).
__device__ __forceinline__ float wave_scan_add(float v) {
  v += dpp_f<0x111, 0xF>(0.f, v);
  v += dpp_f<0x112, 0xF>(0.f, v);
  v += dpp_f<0x114, 0xF>(0.f, v);
  v += dpp_f<0x118, 0xF>(0.f, v);
  v += dpp_f<0x142, 0xA>(0.f, v);
  v += dpp_f<0x143, 0xC>(0.f, v);
  return v;
}
__device__ __forceinline__ int wave_scan_max(int v) {
  v = max(v, dpp_i<0x111, 0xF>(-1, v));
  v = max(v, dpp_i<0x112, 0xF>(-1, v));
  v = max(v, dpp_i<0x114, 0xF>(-1, v));
  v = max(v, dpp_i<0x118, 0xF>(-1, v));
  v = max(v, dpp_i<0x142, 0xA>(-1, v));
  v = max(v, dpp_i<0x143, 0xC>(-1, v));
  return v;
}

// ----------------------------------------------------- DPP row reductions --
// Sum over aligned groups of L lanes (L in {1, 2, 4, 8, 16}); every lane of
// the group ends with the group's sum.  quad_perm swaps for 2 and 4,
// row_half_mirror for 8, row_mirror for 16.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (L >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}

// ------------------------------------------------------------- barriers --
// Workgroup barrier for LDS hand-offs only: waits for this wave's own LDS
// operations (lgkmcnt 0) but not for its outstanding global loads, so loads
// issued before the barrier keep flying across it (the compiler still waits
// for them before their first use).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ MFMA tiles --
// All products are built from 16x16 output tiles.  A "K16 fragment" of an
// operand is what one lane holds for 16 contraction indices: lane l
// (x = l % 16, g = l / 16) holds the 4 values at contraction indices
// 4g .. 4g+3 for row/column x.  This is exactly how a 16x16 fp32 accumulator
// is spread (lane (col, g) holds rows 4g .. 4g+3), so an accumulator tile is
// directly a B fragment for the next product, with the tile's rows as the
// contraction index.  Because a product sums over the contraction index, any
// assignment of contraction indices to (lane group, register) gives the same
// result as long as A and B use the same one; the helpers below rely on that.

// acc += A(16 x 16) * B(16 x 16) for io element type bf16 (1 MFMA) ...
__device__ __forceinline__ f4 mma_k16(f4 acc, bf4 a, bf4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a),
                                                   __builtin_bit_cast(s4, b), acc, 0, 0, 0);
}
// ... and fp32 (4 MFMAs of K = 4; register s of every lane is one K step).
__device__ __forceinline__ f4 mma_k16(f4 acc, f4 a, f4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  return acc;
}

// acc += A(16 x 32) * B(32 x 16): two K16 fragments per operand.  bf16 uses
// one 16x16x32 MFMA (register halves = the two K16 blocks).
__device__ __forceinline__ f4 mma_k32(f4 acc, bf4 a0, bf4 a1, bf4 b0, bf4 b1) {
  const bf8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const bf8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f4 mma_k32(f4 acc, f4 a0, f4 a1, f4 b0, f4 b1) {
  return mma_k16(mma_k16(acc, a0, b0), a1, b1);
}

// Fragment type for an operand element type.
template <typename E> struct frag_of;
template <> struct frag_of<__bf16> { typedef bf4 type; };
template <> struct frag_of<float> { typedef f4 type; };

// Accumulator (fp32) -> operand fragment.
__device__ __forceinline__ void cvt_frag(f4 x, bf4& o) {
  o = bf4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
__device__ __forceinline__ void cvt_frag(f4 x, f4& o) { o = x; }

// Four consecutive operand elements from LDS.
__device__ __forceinline__ void lds_frag(const __bf16* p, bf4& o) {
  o = *reinterpret_cast<const bf4*>(p);
}
__device__ __forceinline__ void lds_frag(const float* p, f4& o) {
  o = *reinterpret_cast<const f4*>(p);
}

}  // namespace gdn
