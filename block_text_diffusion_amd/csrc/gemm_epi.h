// MFMA tile step and epilogues shared by the GEMM kernels.  A lane (or thread) holds four
// consecutive packed output columns n..n+3 of one row.
#pragma once
#include "common.h"
#include "kernels.h"

namespace cd {

template <int AT>
__device__ __forceinline__ void store4(void* base, int64_t idx, float v0, float v1, float v2, float v3) {
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(v0, v1, v2, v3);
  } else {
    uint2 p;
    p.x = pack_bf16(v0, v1);
    p.y = pack_bf16(v2, v3);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = p;
  }
}
template <int AT>
__device__ __forceinline__ void store2(void* base, int64_t idx, float v0, float v1) {
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(base) + idx) = make_float2(v0, v1);
  } else {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(base) + idx) =
        pack_bf16(v0, v1);
  }
}
template <int AT>
__device__ __forceinline__ void store1(void* base, int64_t idx, float v) {
  if constexpr (AT == DT_F32) reinterpret_cast<float*>(base)[idx] = v;
  else reinterpret_cast<uint16_t*>(base)[idx] = f2bf(v);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// fp8 weight fragment (16 E4M3 bytes) -> two bf16 operand fragments.  E4M3
// values are exact in bf16; the hardware conversion (scale 1) turns bytes
// 2q, 2q+1 of each 8-byte half into one packed bf16 pair.
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
}
__device__ __forceinline__ void widen_fp8(const u32x4& w, u32x4 (&wb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    wb[h][0] = fp8x2_lo(w[2 * h]);
    wb[h][1] = fp8x2_hi(w[2 * h]);
    wb[h][2] = fp8x2_lo(w[2 * h + 1]);
    wb[h][3] = fp8x2_hi(w[2 * h + 1]);
  }
}
// MXFP4 weight fragment -> two bf16 operand fragments.  w[0], w[1]: the
// lane's 8 code bytes (16 E2M1 values, even column in the low nibble), w[2]:
// its E8M0 scale byte.  The hardware conversion turns byte b of a word into
// the bf16 pair (low nibble, high nibble) times the scale, exactly.
__device__ __forceinline__ uint32_t fp4x2(uint32_t v, float s, int b) {
  switch (b) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3));
  }
}
__device__ __forceinline__ void widen_fp4(const u32x4& w, u32x4 (&wb)[2]) {
  const float s = __uint_as_float(w[2] << 23);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int b = 0; b < 4; ++b) wb[h][b] = fp4x2(w[h], s, b);
}
// one MXFP4 tile fragment: 8 code bytes at p, the scale byte at ps
__device__ __forceinline__ u32x4 load_fp4(const uint8_t* p, const uint8_t* ps) {
  const uint2 c = *reinterpret_cast<const uint2*>(p);
  u32x4 r;
  r[0] = c.x; r[1] = c.y; r[2] = *ps; r[3] = 0;
  return r;
}
// the 8 code bytes only (the scales come as one dword per four k-tiles)
__device__ __forceinline__ u32x4 load_fp4_codes(const uint8_t* p) {
  const uint2 c = *reinterpret_cast<const uint2*>(p);
  u32x4 r;
  r[0] = c.x; r[1] = c.y; r[2] = 0; r[3] = 0;
  return r;
}
__device__ __forceinline__ f32x4 mma_bf16(const u32x4& a, const u32x4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// one k-tile of MFMA work: acc += W_tile(16 x KF) * X_tile(16 x KF)^T
template <int WT>
__device__ __forceinline__ f32x4 mma_tile(const u32x4& w, const u32x4* x, f32x4 acc) {
  if constexpr (WT == DT_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w[j]), __uint_as_float(x[0][j]), acc, 0, 0, 0);
  } else if constexpr (WT == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                  __builtin_bit_cast(bf16x8, x[0]), acc, 0, 0, 0);
  } else {
    u32x4 wb[2];
    if constexpr (WT == DT_FP4) widen_fp4(w, wb);
    else widen_fp8(w, wb);
    acc = mma_bf16(wb[0], x[0], acc);
    acc = mma_bf16(wb[1], x[1], acc);
  }
  return acc;
}

// Store of four packed columns n..n+3 (multiple of 4) of one output row.
// sc: fp8 per-row weight scales of this group (or null).  ks: contraction
// split of an fp32 partial (EPI_F32 only).
template <int AT, int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs& a, const float* sc, int row, int n, const float* vin, int ks) {
  if (n >= a.N) return;
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = sc ? vin[q] * sc[n + q] : vin[q];
  if constexpr (EPI == EPI_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + ks * a.y_kstride + (int64_t)row * a.ldy + n) =
        make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (EPI == EPI_ROWS) {
    store4<AT>(a.Y, (int64_t)row * a.ldy + n, v[0], v[1], v[2], v[3]);
  } else if constexpr (EPI == EPI_RESID) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + (int64_t)row * a.ldy + n);
    float4 o = *p;
    o.x += v[0]; o.y += v[1]; o.z += v[2]; o.w += v[3];
    *p = o;
  } else if constexpr (EPI == EPI_QKV) {
    const int dh = a.dh, half = dh >> 1;
    const int req = row / a.rows_per_req;
    const int pos = a.pos0[req * a.pos0_stride] + (row - req * a.rows_per_req);
    const int qdim = a.Hq * dh, kdim = a.Hkv * dh;
    if (n < qdim + kdim) {
      // packed columns n..n+3 of a head are logical (i, i+half, i+1, i+1+half)
      const int head = (n < qdim) ? n / dh : (n - qdim) / dh;
      const int p = n % dh;
      const int i0 = p >> 1;
      float x0 = v[0], y0 = v[1], x1 = v[2], y1 = v[3];
      if (a.rope_cs) {
        const float* cs = a.rope_cs + ((int64_t)pos * half + i0) * 2;
        const float c0 = cs[0], s0 = cs[1], c1 = cs[2], s1 = cs[3];
        const float rx0 = x0 * c0 - y0 * s0, ry0 = y0 * c0 + x0 * s0;
        const float rx1 = x1 * c1 - y1 * s1, ry1 = y1 * c1 + x1 * s1;
        x0 = rx0; y0 = ry0; x1 = rx1; y1 = ry1;
      }
      if (n < qdim) {
        // queries leave scaled for a base-2 softmax (one rounding, as unscaled)
        const float qs = a.q_scale;
        const int64_t base = (int64_t)row * a.ldy + head * dh;
        store2<AT>(a.Y, base + i0, x0 * qs, x1 * qs);
        store2<AT>(a.Y, base + i0 + half, y0 * qs, y1 * qs);
      } else {
        const int64_t base = (int64_t)req * a.kv_req_stride + ((int64_t)head * a.max_ctx + pos) * dh;
        store2<AT>(a.kc, base + i0, x0, x1);
        store2<AT>(a.kc, base + i0 + half, y0, y1);
      }
    } else {
      const int c = n - qdim - kdim;
      const int head = c / dh, dd = c % dh;
      const int64_t base = (int64_t)req * a.kv_req_stride + ((int64_t)head * dh + dd) * a.max_ctx + pos;
#pragma unroll
      for (int q = 0; q < 4; ++q) store1<AT>(a.vc, base + (int64_t)q * a.max_ctx, v[q]);
    }
  }
}

// SwiGLU of a gate tile and its up tile: packed gate columns ng..ng+3 (in an
// even 16-column tile), up columns ng+16..ng+19; hidden column
// (ng / 32) * 16 + ng % 16.
template <int AT>
__device__ __forceinline__ void epi_swiglu(const GemmArgs& a, const float* sc, int row, int ng, const float* g,
                                           const float* u) {
  const int j = (ng >> 5) * 16 + (ng & 15);
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float gg = sc ? g[q] * sc[ng + q] : g[q];
    const float uu = sc ? u[q] * sc[ng + 16 + q] : u[q];
    v[q] = silu(gg) * uu;
  }
  store4<AT>(a.Y, (int64_t)row * a.ldy + j, v[0], v[1], v[2], v[3]);
}

}  // namespace cd
