// Canvas attention: softmax(Q K^T / sqrt(dh)) V over the committed KV cache
// plus the canvas itself, with no mask (every canvas token sees every other
// canvas token and the whole committed history); the same kernel with a
// causal mask serves the prompt prefill.
//
// Work item = (request, KV head, block of 128 query rows, key split).  The
// 128 query rows are the Hq/Hkv query heads that share one KV head times
// 128/(Hq/Hkv) tokens, so each K/V fragment feeds every head of its group
// (grouped-query reuse).  Each wave owns 32 query rows (two 16-row tiles):
//  * S^T = K Q^T on MFMA (A = key tile, B = query tile), so a lane holds 4
//    keys of one query and the P fragment of the next product is already in
//    its registers (no shuffle or LDS round trip between the two MFMAs);
//  * online softmax in base 2 with the 1/sqrt(dh) scale folded in; row max
//    and sum reduce across the 4 lane groups with two xor shuffles;
//  * O^T += V^T P^T on MFMA; V is cached transposed ([dh][ctx]) so its
//    fragments are contiguous in the key index.
// Each split writes an unnormalised partial (O, max, sum); a merge kernel
// combines the splits, which fills the chip at one request's 8 KV heads.
#include "common.h"
#include "kernels.h"

namespace cd {

template <int AT>
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t elem) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(base) + elem * (AT == DT_F32 ? 4 : 2));
}
template <int AT>
__device__ __forceinline__ uint2 ld8(const void* base, int64_t elem) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(base) + elem * (AT == DT_F32 ? 4 : 2));
}

template <int AT, int DH>
__global__ __launch_bounds__(256) void k_attn(const AttnArgs a) {
  constexpr int KF = (AT == DT_F32) ? 16 : 32;   // contraction elements per fragment
  constexpr int KQ = KF / 4;                     // per lane
  constexpr int NK = DH / KF;                    // fragments across dh
  constexpr int ND = DH / 16;                    // 16-wide d tiles of the output
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.Hq / a.Hkv;
  const int TB = 128 / G;                        // tokens per query block

  int bid = blockIdx.x;
  const int s = bid % a.n_split; bid /= a.n_split;
  const int qb = bid % a.q_blocks; bid /= a.q_blocks;
  const int g = bid % a.Hkv; bid /= a.Hkv;
  const int r = bid;
  if (r >= a.n_req) return;

  const int pos0 = a.pos0[r * a.pos0_stride];
  const int nrows = a.rows_per_req;
  const int nkeys = pos0 + nrows;
  const int hh = (wave * 32) / TB;               // head within group
  const int h = g * G + hh;
  const int tok0 = qb * TB + (wave * 32) % TB;   // first token of this wave

  const int kbeg = s * a.split_len;
  int kend = min(kbeg + a.split_len, nkeys);
  if (a.causal) kend = min(kend, pos0 + min(tok0 + 32, nrows));

  const int64_t ld = (int64_t)a.Hq * DH;
  const void* kc = reinterpret_cast<const uint8_t*>(a.kc) + (int64_t)r * a.kv_req_stride * (AT == DT_F32 ? 4 : 2);
  const void* vc = reinterpret_cast<const uint8_t*>(a.vc) + (int64_t)r * a.kv_req_stride * (AT == DT_F32 ? 4 : 2);
  const int64_t khead = (int64_t)g * a.max_ctx * DH;   // [Hkv][ctx][dh]
  const int64_t vhead = (int64_t)g * DH * a.max_ctx;   // [Hkv][dh][ctx]

  // query fragments, resident for the whole key loop
  u32x4 qf[2][NK];
  int qtok[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    int tok = tok0 + qt * 16 + (lane & 15);
    qtok[qt] = tok;
    int tc = min(tok, nrows - 1);
    int64_t row = (int64_t)r * nrows + tc;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[qt][kk] = ld16<AT>(a.Q, row * ld + h * DH + kk * KF + (lane >> 4) * KQ);
  }

  const float sl2 = 1.4426950408889634f / sqrtf((float)DH);
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 o[2][ND];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[qt][dt] = f32x4{0, 0, 0, 0};

  for (int key0 = kbeg; key0 < kend; key0 += 32) {
    // S^T tiles: [subtile st: keys key0+16st..][query tile qt]
    f32x4 sacc[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 kf[NK];
      const int64_t krow = khead + (int64_t)(key0 + st * 16 + (lane & 15)) * DH;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kf[kk] = ld16<AT>(kc, krow + kk * KF + (lane >> 4) * KQ);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          if constexpr (AT == DT_F32) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[kk][j]), __uint_as_float(qf[qt][kk][j]), acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kk]),
                                                          __builtin_bit_cast(bf16x8, qf[qt][kk]), acc, 0, 0, 0);
          }
        }
        sacc[st][qt] = acc;
      }
    }
    // mask, online softmax (base 2)
    float p[2][2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int qpos = pos0 + qtok[qt];
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kidx = key0 + st * 16 + (lane >> 4) * 4 + q;
          bool ok = kidx < kend && (!a.causal || kidx <= qpos);
          float v = ok ? sacc[st][qt][q] * sl2 : -INFINITY;
          p[qt][st][q] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m[qt], mt);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m[qt] - mn);
      float sum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e = (mn == -INFINITY) ? 0.f : exp2f(p[qt][st][q] - mn);
          p[qt][st][q] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      l[qt] = l[qt] * alpha + sum;
      m[qt] = mn;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        o[qt][dt][0] *= alpha; o[qt][dt][1] *= alpha; o[qt][dt][2] *= alpha; o[qt][dt][3] *= alpha;
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int64_t vrow = vhead + (int64_t)(dt * 16 + (lane & 15)) * a.max_ctx + key0 + (lane >> 4) * 4;
      if constexpr (AT == DT_F32) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          u32x4 vf = ld16<AT>(vc, vrow + st * 16);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vf[j]), p[qt][st][j], o[qt][dt], 0, 0, 0);
        }
      } else {
        uint2 v0 = ld8<AT>(vc, vrow), v1 = ld8<AT>(vc, vrow + 16);
        u32x4 vf = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          u32x4 pf;
          pf[0] = (uint32_t)f2bf(p[qt][0][0]) | ((uint32_t)f2bf(p[qt][0][1]) << 16);
          pf[1] = (uint32_t)f2bf(p[qt][0][2]) | ((uint32_t)f2bf(p[qt][0][3]) << 16);
          pf[2] = (uint32_t)f2bf(p[qt][1][0]) | ((uint32_t)f2bf(p[qt][1][1]) << 16);
          pf[3] = (uint32_t)f2bf(p[qt][1][2]) | ((uint32_t)f2bf(p[qt][1][3]) << 16);
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf),
                                                              __builtin_bit_cast(bf16x8, pf), o[qt][dt], 0, 0, 0);
        }
      }
    }
  }

  // partial results: O^T lane holds d = dt*16 + 4*(lane/16) + q of query lane%16
  const int64_t rows_total = (int64_t)a.n_req * nrows;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int tok = qtok[qt];
    if (tok >= nrows) continue;
    const int64_t row = (int64_t)r * nrows + tok;
    const int64_t base = (((int64_t)s * rows_total + row) * a.Hq + h);
    float* po = a.part_o + base * DH;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16 + (lane >> 4) * 4) =
          make_float4(o[qt][dt][0], o[qt][dt][1], o[qt][dt][2], o[qt][dt][3]);
    if ((lane >> 4) == 0) {
      a.part_ml[base * 2] = m[qt];
      a.part_ml[base * 2 + 1] = l[qt];
    }
  }
}

// combine key splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
template <int AT>
__global__ void k_attn_merge(const AttnArgs a, int dh) {
  const int64_t row = blockIdx.x;
  const int64_t rows_total = (int64_t)a.n_req * a.rows_per_req;
  const int idx = threadIdx.x * 4;
  if (idx >= a.Hq * dh) return;
  const int h = idx / dh, d = idx % dh;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[(((int64_t)s * rows_total + row) * a.Hq + h) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0, 0, 0, 0);
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t base = ((int64_t)s * rows_total + row) * a.Hq + h;
    const float ms = a.part_ml[base * 2];
    if (ms == -INFINITY) continue;
    const float w = exp2f(ms - M);
    L += w * a.part_ml[base * 2 + 1];
    float4 v = *reinterpret_cast<const float4*>(a.part_o + base * dh + d);
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  const float inv = 1.0f / L;
  const int64_t o = row * (int64_t)a.Hq * dh + idx;
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.O) + o) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 p;
    p.x = (uint32_t)f2bf(acc.x * inv) | ((uint32_t)f2bf(acc.y * inv) << 16);
    p.y = (uint32_t)f2bf(acc.z * inv) | ((uint32_t)f2bf(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.O) + o) = p;
  }
}

void launch_attention(int adt, const AttnArgs& a, hipStream_t s) {
  const int blocks = a.n_req * a.Hkv * a.q_blocks * a.n_split;
  if (adt == DT_F32) {
    if (a.dh == 64) hipLaunchKernelGGL((k_attn<DT_F32, 64>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn<DT_F32, 128>), dim3(blocks), dim3(256), 0, s, a);
  } else {
    if (a.dh == 64) hipLaunchKernelGGL((k_attn<DT_BF16, 64>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn<DT_BF16, 128>), dim3(blocks), dim3(256), 0, s, a);
  }
}

void launch_attn_merge(int adt, const AttnArgs& a, hipStream_t s) {
  const int rows = a.n_req * a.rows_per_req;
  const int threads = (a.Hq * a.dh / 4 + 63) / 64 * 64;
  if (adt == DT_F32) hipLaunchKernelGGL(k_attn_merge<DT_F32>, dim3(rows), dim3(threads), 0, s, a, a.dh);
  else hipLaunchKernelGGL(k_attn_merge<DT_BF16>, dim3(rows), dim3(threads), 0, s, a, a.dh);
}

}  // namespace cd
