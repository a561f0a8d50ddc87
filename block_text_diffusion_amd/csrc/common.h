// Device-side helpers shared by the canvas-denoise kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_FP4 = 3 };

// ---- bf16 -------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// fp32 -> bf16, round to nearest even (the hardware conversion)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two fp32 -> packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- E4M3FN (OCP) -> fp32, exact ----------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t s = (b & 0x80u) << 24;
  uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return __uint_as_float(__float_as_uint(v) | s);
}

// ---- Philox4x32-10 (Salmon et al., SC'11) -------------------------------
struct u4 { uint32_t x, y, z, w; };
__device__ __forceinline__ u4 philox(u4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    u4 n;
    n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
    n.y = (uint32_t)p1;
    n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
    n.w = (uint32_t)p0;
    c = n;
  }
  return c;
}

// uniform token id in [0, V) for (seed; pos, step, block, req), tag 0
__device__ __forceinline__ int32_t canvas_token(uint64_t seed, uint32_t pos, uint32_t step,
                                                uint32_t block, uint32_t req, uint32_t V) {
  u4 c = {pos, step, block, req};
  u4 r = philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (int32_t)(((uint64_t)r.x * V) >> 32);
}

// ---- LDS staging ----------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maxima).  Loads
// that copy global memory straight into LDS (global_load_lds) count in vmcnt.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---- wave reductions -----------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- per-row E4M3 activation quantisation ----------------------------------
// Four values already rounded to bf16 (as fp32), scaled by inv = 448 / amax of
// their row, clamped to +-448 and rounded to E4M3 (nearest even), packed low
// byte first.  Every producer of E4M3 activation rows uses this, so a row
// quantised by the standalone quantiser or by the kernel that writes it gets
// the same codes.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
  const float f0 = fminf(fmaxf(a * inv, -448.f), 448.f);
  const float f1 = fminf(fmaxf(b * inv, -448.f), 448.f);
  const float f2 = fminf(fmaxf(c * inv, -448.f), 448.f);
  const float f3 = fminf(fmaxf(d * inv, -448.f), 448.f);
  uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, p, true);
}
// the row's quantisation factor and stored scale from its max |value|
__device__ __forceinline__ float e4m3_inv(float amax) { return amax > 0.f ? 448.0f / amax : 1.0f; }
__device__ __forceinline__ float e4m3_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

}  // namespace cd
