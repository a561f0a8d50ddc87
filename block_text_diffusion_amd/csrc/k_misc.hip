// Small kernels of the step: embedding gather, RMSNorm (unit gain), rotary
// table, canvas start (uniform Philox token ids), request bookkeeping.
#include "common.h"
#include "kernels.h"

namespace cd {

// h[t] = E[ids[t]] (storage fp32 or bf16), residual stream kept in fp32
// ids outside [0, V) are clamped (the embedding table is never read out of range)
__global__ __launch_bounds__(256) void k_embed(int edt, const void* E, const int32_t* ids, int V, int d, float* h) {
  const int t = blockIdx.x;
  const int64_t row = min(max(ids[t], 0), V - 1);
  for (int c = threadIdx.x; c < d; c += 256) {
    float v = edt == DT_F32 ? reinterpret_cast<const float*>(E)[row * d + c]
                            : bf2f(reinterpret_cast<const uint16_t*>(E)[row * d + c]);
    h[(int64_t)t * d + c] = v;
  }
}
void launch_embed(int edt, const void* E, const int32_t* ids, int T, int V, int d, float* h, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(T), dim3(256), 0, s, edt, E, ids, V, d, h);
}

// u = h / sqrt(mean(h^2) + eps), one wave per row (four rows per workgroup).
// Rows of up to 4096 values stay in registers between the sum of squares and
// the scaling: every load of the row is issued before the first use, at
// clamped addresses so none of them is conditional.
template <int AT>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* h, int T, int d, float eps, void* u, uint8_t* q8,
                                                 float* s8) {
  constexpr int NV = 16;   // float4 per lane held in registers
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* x = h + (int64_t)t * d;
  auto put = [&](int c, float4 v, float inv) {
    if constexpr (AT == DT_F32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(u) + (int64_t)t * d + c) =
          make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    } else {
      uint2 p;
      p.x = pack_bf16(v.x * inv, v.y * inv);
      p.y = pack_bf16(v.z * inv, v.w * inv);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(u) + (int64_t)t * d + c) = p;
    }
  };
  float ss = 0.f;
  if (d <= 256 * NV) {
    float4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = *reinterpret_cast<const float4*>(x + min((lane + 64 * j) * 4, d - 4));
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((lane + 64 * j) * 4 < d) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    if constexpr (AT == DT_BF16) {
      if (q8) {
        // also the E4M3 row of the bf16 values with its scale (the input of
        // an fp8 GEMM), as the standalone quantiser would compute it
        uint2 p[NV];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          p[j].x = pack_bf16(v[j].x * inv, v[j].y * inv);
          p[j].y = pack_bf16(v[j].z * inv, v[j].w * inv);
          if ((lane + 64 * j) * 4 < d)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf2f(p[j].x & 0xFFFF)), fabsf(bf2f(p[j].x >> 16))),
                                     fmaxf(fabsf(bf2f(p[j].y & 0xFFFF)), fabsf(bf2f(p[j].y >> 16)))));
        }
        amax = wave_max(amax);
        const float qi = e4m3_inv(amax);
        if (lane == 0) s8[t] = e4m3_scale(amax);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int c = (lane + 64 * j) * 4;
          if (c >= d) continue;
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(u) + (int64_t)t * d + c) = p[j];
          *reinterpret_cast<uint32_t*>(q8 + (int64_t)t * d + c) =
              e4m3x4(bf2f(p[j].x & 0xFFFF), bf2f(p[j].x >> 16), bf2f(p[j].y & 0xFFFF), bf2f(p[j].y >> 16), qi);
        }
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((lane + 64 * j) * 4 < d) put((lane + 64 * j) * 4, v[j], inv);
  } else {
    for (int c = lane * 4; c < d; c += 256) {
      const float4 v = *reinterpret_cast<const float4*>(x + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 4; c < d; c += 256) put(c, *reinterpret_cast<const float4*>(x + c), inv);
  }
}
void launch_rmsnorm(int adt, const float* h, int T, int d, float eps, void* u, hipStream_t s, uint8_t* q8, float* s8) {
  const dim3 grid((T + 3) / 4);
  if (adt == DT_F32) hipLaunchKernelGGL(k_rmsnorm<DT_F32>, grid, dim3(256), 0, s, h, T, d, eps, u, nullptr, nullptr);
  else hipLaunchKernelGGL(k_rmsnorm<DT_BF16>, grid, dim3(256), 0, s, h, T, d, eps, u, d <= 4096 ? q8 : nullptr, s8);
}

// cs[pos][i] = (cos, sin)(pos * theta^(-2i/dh)), computed in fp64
__global__ void k_rope_table(float* cs, int max_ctx, int dh, double theta) {
  const int half = dh / 2;
  const int64_t n = (int64_t)max_ctx * half;
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(j / half), i = (int)(j % half);
    const double ang = (double)pos * pow(theta, -2.0 * i / dh);
    cs[2 * j] = (float)cos(ang);
    cs[2 * j + 1] = (float)sin(ang);
  }
}
void launch_rope_table(float* cs, int max_ctx, int dh, float theta, hipStream_t s) {
  hipLaunchKernelGGL(k_rope_table, dim3(1024), dim3(256), 0, s, cs, max_ctx, dh, (double)theta);
}

__global__ void k_init_canvas(int32_t* canvas, ReqDev* rq, int req, int C, int V, uint64_t seed, int block, int rid) {
  for (int i = threadIdx.x; i < C; i += blockDim.x)
    canvas[(int64_t)req * C + i] = canvas_token(seed, i, 0, block, rid, V);
  if (threadIdx.x == 0) {
    rq[req].t = 0;
    rq[req].block = block;
    rq[req].rid = rid;
    rq[req].seed = seed;
    rq[req].stopped = 0;
  }
}
void launch_init_canvas(int32_t* canvas, ReqDev* rq, int req, int C, int V, uint64_t seed, int block, int rid,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_init_canvas, dim3(1), dim3(256), 0, s, canvas, rq, req, C, V, seed, block, rid);
}

__global__ void k_advance(ReqDev* rq, int req, int dP) { rq[req].P += dP; }
void launch_advance(ReqDev* rq, int req, int dP, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3(1), dim3(1), 0, s, rq, req, dP);
}

__global__ void k_copy_i32(const int32_t* src, int32_t* dst, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = src[i];
}
void launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_i32, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
}
__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
void launch_zero_u32(void* p, int64_t n, hipStream_t s) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b > 0) hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)b), dim3(256), 0, s, reinterpret_cast<uint32_t*>(p), n);
}
__global__ void k_copy_f32(const float* src, float* dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
void launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)b), dim3(256), 0, s, src, dst, n);
}

}  // namespace cd
