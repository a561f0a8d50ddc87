// Synthetic weights and weight packing.
//
// Synthetic weights: element n of tensor tau is 0.02 * z with z a standard
// normal from Philox4x32-10 (counter (n/4 lo, n/4 hi, tau, 1 << 24), key =
// seed) through Box-Muller in fp64 -- words (r0, r1) feed elements 4q and
// 4q+1 (cosine, sine), (r2, r3) feed 4q+2 and 4q+3 -- rounded once from fp64
// to the storage format (fp32, bf16, or E4M3FN with a bf16 scale per output
// row equal to bf16(max|w_row| / 448), or MXFP4: E2M1 codes with one E8M0
// scale 2^e per 32 columns of a row, e = floor(log2(max|w_block|)) - 2 (the
// largest E2M1 power of two is 2^2; OCP Microscaling Formats v1.0), codes
// round(w / 2^e) to nearest even, saturating at +-6).  The kernel writes the packed MFMA
// layout directly; packed rows are permuted so that the rotary pairs (i,
// i+dh/2) of Q and K heads, and the gate/up rows of SwiGLU FFNs, land in the
// same lane (see the row maps below).
#include "common.h"
#include "kernels.h"

namespace cd {

enum { MODE_SYNTH = 0, MODE_PACK = 1, MODE_UNPACK = 2 };

// packed row p -> (source tensor, logical row), or sel = -1 for a zero row
__device__ __forceinline__ void row_source(const PackDesc& d, int p, int& sel, int& n) {
  sel = -1; n = 0;
  if (d.perm == PERM_NONE) {
    if (p < d.n_rows_src[0]) { sel = 0; n = p; }
  } else if (d.perm == PERM_QKV) {
    const int qd = d.Hq * d.dh, kd = d.Hkv * d.dh;
    int base;
    if (p < qd) { sel = 0; base = p; }
    else if (p < qd + kd) { sel = 1; base = p - qd; }
    else if (p < qd + 2 * kd) { sel = 2; n = p - qd - kd; return; }
    else return;
    const int head = base / d.dh, pp = base % d.dh;
    n = head * d.dh + (pp & 1) * (d.dh >> 1) + (pp >> 1);
  } else {  // PERM_GU: even 16-row tiles from gate, odd from up
    const int t = p >> 4;
    const int s = t & 1;
    const int r = (t >> 1) * 16 + (p & 15);
    if (r < d.n_rows_src[s]) { sel = s; n = r; }
  }
}

__device__ __forceinline__ int64_t packed_offset(const PackDesc& d, int p, int k) {
  const int es = esize(d.dt);
  if (d.rowmajor) return ((int64_t)p * d.K + k) * es;
  const int KF = 64 / es, KT = d.K / KF;
  const int tile_k = k / KF, kk = k % KF, q = KF / 4;
  const int lane = (p & 15) + 16 * (kk / q);
  return (((int64_t)(p >> 4) * KT + tile_k) * 64 + lane) * 16 + (kk % q) * es;
}

// fp64 -> value with `sig` significant bits, RNE, smallest quantum 2^minq
__device__ __forceinline__ double round_sig(double x, int sig, int minq) {
  int e;
  frexp(x, &e);
  int q = e - sig;
  if (q < minq) q = minq;
  return ldexp(rint(ldexp(x, -q)), q);
}
__device__ __forceinline__ double round_bf16_d(double x) { return round_sig(x, 8, -133); }
__device__ __forceinline__ double round_e4m3_d(double x) {
  double r = round_sig(x, 4, -9);
  return fmin(fmax(r, -448.0), 448.0);
}
__device__ __forceinline__ uint32_t e4m3_encode(double v) {  // v exactly E4M3
  uint32_t s = v < 0 ? 0x80u : 0u;
  double a = fabs(v);
  if (a < 0.015625) return s | (uint32_t)(a * 512.0);
  int e;
  double m = frexp(a, &e);            // a = m * 2^e, m in [0.5, 1)
  uint32_t ex = (uint32_t)(e - 1 + 7);
  uint32_t mant = (uint32_t)((m * 2.0 - 1.0) * 8.0);
  return s | (ex << 3) | mant;
}

// fp64 value already on the E2M1 grid -> 4-bit code (sign in bit 3; -0 -> 0)
__device__ __forceinline__ uint32_t e2m1_encode(double v) {
  const uint32_t s = v < 0 ? 8u : 0u;
  const double a = fabs(v);
  if (a == 0.0) return 0u;
  if (a == 0.5) return s | 1u;
  int e;
  const double m = frexp(a, &e);      // a = m * 2^e: biased exponent e, mantissa bit (2m - 1) * 2
  return s | ((uint32_t)e << 1) | (uint32_t)((m * 2.0 - 1.0) * 2.0);
}
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const float mag = (c & 6u) ? __uint_as_float(((((c >> 1) & 3u) + 126u) << 23) | ((c & 1u) << 22))
                             : 0.5f * (float)(c & 1u);
  return (c & 8u) ? -mag : mag;
}
// byte offsets of the 8-byte lane chunk holding columns k..k+15 (k % 16 == 0)
// of packed row p, and of the scale of the 32-column block holding column k
__device__ __forceinline__ int64_t fp4_chunk(int p, int k, int KT) {
  return ((((int64_t)(p >> 4) * KT + k / 64) * 64) + (p & 15) + 16 * ((k % 64) / 16)) * 8;
}
__device__ __forceinline__ int64_t fp4_scale(int p, int k, int KT) {
  const int kt = k / 64, KT4 = (KT + 3) / 4;
  return (((int64_t)(p >> 4) * KT4 + kt / 4) * 32 + (p & 15) * 2 + (k % 64) / 32) * 4 + kt % 4;
}

__device__ __forceinline__ void synth4(uint64_t seed, uint32_t tau, uint64_t q, double w[4]) {
  u4 c = {(uint32_t)q, (uint32_t)(q >> 32), tau, 1u << 24};
  u4 r = philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const double two32 = 2.3283064365386963e-10;  // 2^-32
  double u1a = ((double)r.x + 1.0) * two32, u2a = (double)r.y * two32;
  double u1b = ((double)r.z + 1.0) * two32, u2b = (double)r.w * two32;
  double ra = sqrt(-2.0 * log(u1a)), rb = sqrt(-2.0 * log(u1b));
  const double twopi = 2.0 * 3.141592653589793;
  double aa = twopi * u2a, ab = twopi * u2b;
  w[0] = 0.02 * (ra * cos(aa));
  w[1] = 0.02 * (ra * sin(aa));
  w[2] = 0.02 * (rb * cos(ab));
  w[3] = 0.02 * (rb * sin(ab));
}

__device__ __forceinline__ void put4(const PackDesc& d, uint8_t* dst, int p, int k, const double w[4], double scale) {
  int64_t off = packed_offset(d, p, k);
  if (d.dt == DT_F32) {
    float4 v = make_float4((float)w[0], (float)w[1], (float)w[2], (float)w[3]);
    *reinterpret_cast<float4*>(dst + off) = v;
  } else if (d.dt == DT_BF16) {
    uint16_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (uint16_t)(__float_as_uint((float)round_bf16_d(w[i])) >> 16);
    uint2 v;
    v.x = b[0] | ((uint32_t)b[1] << 16);
    v.y = b[2] | ((uint32_t)b[3] << 16);
    *reinterpret_cast<uint2*>(dst + off) = v;
  } else {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double qv = scale > 0 ? round_e4m3_d(w[i] / scale) : 0.0;
      v |= e4m3_encode(qv) << (8 * i);
    }
    *reinterpret_cast<uint32_t*>(dst + off) = v;
  }
}

// grid: x = packed row, y = group.  256 threads, 4 elements per thread-step.
template <int MODE>
__global__ __launch_bounds__(256) void k_pack(PackDesc d, int64_t dst_gstride, int64_t scale_gstride,
                                              int tau_gstride, uint64_t seed, const float* s0,
                                              const float* s1, const float* s2, float* o0, float* o1,
                                              float* o2) {
  const int p = blockIdx.x;
  const int g = blockIdx.y;
  uint8_t* dst = d.dst + (int64_t)g * dst_gstride;
  float* scale = d.scale ? d.scale + (int64_t)g * scale_gstride : nullptr;
  int sel, n;
  row_source(d, p, sel, n);
  if (d.only_sel >= 0 && sel != d.only_sel) return;
  const int K = d.K;
  const int nq = K / 4;

  if (d.dt == DT_FP4) {
    // one thread per 32-column block: scale, codes, two 8-byte lane chunks
    const int KT = K / 64;
    uint8_t* mx = dst + d.mx_off;
    const float* src = sel == 0 ? s0 : sel == 1 ? s1 : s2;
    float* out = sel == 0 ? o0 : sel == 1 ? o1 : o2;
    const uint32_t tau = sel >= 0 ? d.tau[sel] + (uint32_t)(g * tau_gstride) : 0;
    for (int b = threadIdx.x; b < K / 32; b += 256) {
      const int k0 = 32 * b;
      if (MODE == MODE_UNPACK) {
        if (sel < 0) return;
        const float sc = __uint_as_float((uint32_t)mx[fp4_scale(p, k0, KT)] << 23);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint2 c = *reinterpret_cast<const uint2*>(dst + fp4_chunk(p, k0 + 16 * h, KT));
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t word = i < 8 ? c.x : c.y;
            out[(int64_t)n * K + k0 + 16 * h + i] = e2m1_decode((word >> (4 * (i & 7))) & 15u) * sc;
          }
        }
        continue;
      }
      double w[32];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (sel < 0) {
          w[4 * j] = w[4 * j + 1] = w[4 * j + 2] = w[4 * j + 3] = 0.0;
        } else if (MODE == MODE_SYNTH) {
          synth4(seed, tau, ((uint64_t)n * K) / 4 + 8 * b + j, w + 4 * j);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(src + (int64_t)n * K + k0 + 4 * j);
          w[4 * j] = f.x; w[4 * j + 1] = f.y; w[4 * j + 2] = f.z; w[4 * j + 3] = f.w;
        }
      }
      double amax = 0.0;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(w[i]));
      int e = 0;
      if (amax > 0.0) {
        frexp(amax, &e);                  // amax in [2^(e-1), 2^e): floor(log2 amax) = e - 1
        e = min(max(e - 3, -126), 127);   // -126: the scale stays a normal fp32 number
      }
      mx[fp4_scale(p, k0, KT)] = (uint8_t)(e + 127);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 c = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const double q = fmin(fmax(round_sig(ldexp(w[16 * h + i], -e), 2, -1), -6.0), 6.0);
          const uint32_t code = e2m1_encode(q) << (4 * (i & 7));
          if (i < 8) c.x |= code; else c.y |= code;
        }
        *reinterpret_cast<uint2*>(dst + fp4_chunk(p, k0 + 16 * h, KT)) = c;
      }
    }
    return;
  }

  if (MODE == MODE_UNPACK) {
    if (sel < 0) return;
    float* out = sel == 0 ? o0 : sel == 1 ? o1 : o2;
    float sc = (d.dt == DT_FP8) ? scale[p] : 1.0f;
    for (int j = threadIdx.x; j < nq; j += 256) {
      const int k = 4 * j;
      int64_t off = packed_offset(d, p, k);
      float v[4];
      if (d.dt == DT_F32) {
        float4 f = *reinterpret_cast<const float4*>(dst + off);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      } else if (d.dt == DT_BF16) {
        uint2 b = *reinterpret_cast<const uint2*>(dst + off);
        v[0] = bf2f(b.x & 0xFFFF); v[1] = bf2f(b.x >> 16); v[2] = bf2f(b.y & 0xFFFF); v[3] = bf2f(b.y >> 16);
      } else {
        uint32_t b = *reinterpret_cast<const uint32_t*>(dst + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = e4m3_to_f32((b >> (8 * i)) & 0xFF) * sc;
      }
      *reinterpret_cast<float4*>(out + (int64_t)n * K + k) = make_float4(v[0], v[1], v[2], v[3]);
    }
    return;
  }

  const float* src = sel == 0 ? s0 : sel == 1 ? s1 : s2;
  const uint32_t tau = sel >= 0 ? d.tau[sel] + (uint32_t)(g * tau_gstride) : 0;
  auto values = [&](int j, double w[4]) {
    if (sel < 0) { w[0] = w[1] = w[2] = w[3] = 0.0; return; }
    if (MODE == MODE_SYNTH) {
      synth4(seed, tau, ((uint64_t)n * K) / 4 + j, w);
    } else {
      float4 f = *reinterpret_cast<const float4*>(src + (int64_t)n * K + 4 * j);
      w[0] = f.x; w[1] = f.y; w[2] = f.z; w[3] = f.w;
    }
  };

  double sc = 0.0;
  if (d.dt == DT_FP8) {
    double mxd = 0.0;
    for (int j = threadIdx.x; j < nq; j += 256) {
      double w[4];
      values(j, w);
#pragma unroll
      for (int i = 0; i < 4; ++i) mxd = fmax(mxd, fabs(w[i]));
    }
    // non-negative doubles order like their 64-bit patterns: reduce the
    // row maximum exactly with an integer max in LDS
    unsigned long long bits = (unsigned long long)__double_as_longlong(mxd);
    __shared__ unsigned long long shb;
    if (threadIdx.x == 0) shb = 0;
    __syncthreads();
    atomicMax(&shb, bits);
    __syncthreads();
    mxd = __longlong_as_double((long long)shb);
    sc = round_bf16_d(mxd / 448.0);
    if (threadIdx.x == 0) scale[p] = (float)sc;
  }
  for (int j = threadIdx.x; j < nq; j += 256) {
    double w[4];
    values(j, w);
    put4(d, dst, p, 4 * j, w, sc);
  }
}

static void launch_mode(int mode, const PackDesc& d, int n_groups, int64_t dst_gstride, int64_t scale_gstride,
                        int tau_gstride, uint64_t seed, const float* s0, const float* s1, const float* s2,
                        float* o0, float* o1, float* o2, hipStream_t s) {
  dim3 grid(d.Npad, n_groups);
  if (mode == MODE_SYNTH)
    hipLaunchKernelGGL(k_pack<MODE_SYNTH>, grid, dim3(256), 0, s, d, dst_gstride, scale_gstride, tau_gstride,
                       seed, s0, s1, s2, o0, o1, o2);
  else if (mode == MODE_PACK)
    hipLaunchKernelGGL(k_pack<MODE_PACK>, grid, dim3(256), 0, s, d, dst_gstride, scale_gstride, tau_gstride,
                       seed, s0, s1, s2, o0, o1, o2);
  else
    hipLaunchKernelGGL(k_pack<MODE_UNPACK>, grid, dim3(256), 0, s, d, dst_gstride, scale_gstride, tau_gstride,
                       seed, s0, s1, s2, o0, o1, o2);
}

void launch_synth(const PackDesc& d, int n_groups, int64_t dst_gstride, int64_t scale_gstride, int tau_gstride,
                  uint64_t seed, hipStream_t s) {
  launch_mode(MODE_SYNTH, d, n_groups, dst_gstride, scale_gstride, tau_gstride, seed, nullptr, nullptr, nullptr,
              nullptr, nullptr, nullptr, s);
}
void launch_pack(const PackDesc& d, const float* s0, const float* s1, const float* s2, hipStream_t s) {
  launch_mode(MODE_PACK, d, 1, 0, 0, 0, 0, s0, s1, s2, nullptr, nullptr, nullptr, s);
}
void launch_unpack(const PackDesc& d, float* o0, float* o1, float* o2, hipStream_t s) {
  launch_mode(MODE_UNPACK, d, 1, 0, 0, 0, 0, nullptr, nullptr, nullptr, o0, o1, o2, s);
}

}  // namespace cd
