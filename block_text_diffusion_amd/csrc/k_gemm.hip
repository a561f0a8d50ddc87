// Weight-streaming GEMM  Y[m][n] = sum_k X[m][k] * W[n][k]  on CDNA4 MFMA.
//
// The canvas step at batch 1 multiplies a few hundred (dense layers) or a few
// dozen (one routed expert) activation rows by large weight matrices, so it
// is bound by streaming the weights from HBM once.  Design:
//  * weights are pre-packed in MFMA operand order (see kernels.h), so each
//    wave fetches a 16 x KF tile as one contiguous 1 KB load straight into
//    registers (no LDS round trip for the streamed operand);
//  * a workgroup is 4 waves; each wave owns two 16-column weight tiles and
//    MT 16-row activation tiles, so every weight byte is read by exactly one
//    wave per row block; activation fragments (small, L2 resident) are loaded
//    per lane from row-major X, optionally through a row map (MoE gather);
//  * the k loop is software pipelined in stages of 4 tiles with two register
//    sets, keeping 8 KB of weight loads in flight per wave;
//  * the product is computed transposed (A = weight tile, B = activation
//    tile), so each lane ends with 4 consecutive output columns of one row
//    and the epilogues store 8-16 contiguous bytes per lane;
//  * dense launches remap block ids so that the row blocks of one weight
//    slice run on the same XCD and share its L2; grouped launches keep the
//    dispatcher's round-robin so the real tiles spread over all 8 XCDs.
// Epilogues: fp32 store (router / LM head logits), row store (expert
// outputs), fp32 residual add, SwiGLU of interleaved gate/up tiles, and
// QKV with rotary embedding scattering K/V into the cache.
#include "common.h"
#include "kernels.h"

namespace cd {

template <int AT>
__device__ __forceinline__ void store4(void* base, int64_t idx, float v0, float v1, float v2, float v3) {
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(v0, v1, v2, v3);
  } else {
    uint2 p;
    p.x = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
    p.y = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = p;
  }
}
template <int AT>
__device__ __forceinline__ void store2(void* base, int64_t idx, float v0, float v1) {
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(base) + idx) = make_float2(v0, v1);
  } else {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(base) + idx) =
        (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
  }
}
template <int AT>
__device__ __forceinline__ void store1(void* base, int64_t idx, float v) {
  if constexpr (AT == DT_F32) reinterpret_cast<float*>(base)[idx] = v;
  else reinterpret_cast<uint16_t*>(base)[idx] = f2bf(v);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

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
    // E4M3 has 4 significant bits, so its bf16 image is exact (top half of fp32)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 wb;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = w[2 * h + (q >> 1)];
        uint32_t b0 = (word >> (16 * (q & 1))) & 0xFFu;
        uint32_t b1 = (word >> (16 * (q & 1) + 8)) & 0xFFu;
        wb[q] = (__float_as_uint(e4m3_to_f32(b0)) >> 16) | (__float_as_uint(e4m3_to_f32(b1)) & 0xFFFF0000u);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb),
                                                    __builtin_bit_cast(bf16x8, x[h]), acc, 0, 0, 0);
    }
  }
  return acc;
}

template <int WT, int AT, int MT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs a) {
  constexpr int MROWS = 16 * MT;
  constexpr int U = 4;
  constexpr int XW = (WT == DT_FP8) ? 2 : 1;        // 16-byte activation loads per k-tile
  constexpr int XSTEP = (WT == DT_FP8) ? 128 : 64;  // activation bytes per k-tile
  constexpr int KF = 64 / (WT == DT_F32 ? 4 : WT == DT_BF16 ? 2 : 1);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Dense launches (chunk-major) remap block ids so the row blocks that share
  // a weight slice run on one XCD (the dispatcher deals workgroups to the 8
  // XCDs round-robin) and share its L2.  Grouped launches keep the natural
  // order: their real tiles come first and must spread over all XCDs.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  int logical = a.chunk_major ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
  const int ksplit = a.ksplit > 1 ? a.ksplit : 1;
  const int ks = logical % ksplit;
  logical /= ksplit;
  int tile, chunk;
  if (a.chunk_major) { chunk = logical / a.max_tiles; tile = logical - chunk * a.max_tiles; }
  else { tile = logical / a.n_chunks; chunk = logical - tile * a.n_chunks; }
  if (tile >= a.max_tiles || chunk >= a.n_chunks) return;

  int group, row0, rows;
  if (a.tiles) {
    if (tile >= *a.n_tiles) return;
    group = a.tiles[4 * tile];
    row0 = a.tiles[4 * tile + 1];
    rows = a.tiles[4 * tile + 2];
  } else {
    group = 0;
    row0 = tile * MROWS;
    rows = min(MROWS, a.M - row0);
    if (rows <= 0) return;
  }
  const int nt0 = chunk * 8 + wave * 2;
  if (nt0 >= a.Nt) return;

  const int KTall = a.K / KF;
  const int kt_beg = (int)((int64_t)KTall * ks / ksplit);
  const int KT = (int)((int64_t)KTall * (ks + 1) / ksplit) - kt_beg;   // k-tiles of this split
  const uint8_t* wp0 = a.W + (int64_t)group * a.w_gstride + ((int64_t)nt0 * KTall + kt_beg) * 1024 + lane * 16;
  const uint8_t* wp1 = wp0 + (int64_t)KTall * 1024;
  const int esa = (AT == DT_F32) ? 4 : 2;
  const uint8_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = mt * 16 + (lane & 15);
    int src = 0;
    if (r < rows) src = a.row_map ? a.row_map[row0 + r] : row0 + r;
    if (src < 0) src = 0;
    xp[mt] = reinterpret_cast<const uint8_t*>(a.X) + ((int64_t)src * a.ldx) * esa + (lane >> 4) * 16 * XW +
             (int64_t)kt_beg * XSTEP;
  }

  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) { acc[mt][0] = f32x4{0, 0, 0, 0}; acc[mt][1] = f32x4{0, 0, 0, 0}; }

  u32x4 wA[2][U], wB[2][U];
  u32x4 xA[MT][U][XW], xB[MT][U][XW];

  auto load = [&](u32x4 (&w)[2][U], u32x4 (&x)[MT][U][XW], int kt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[0][u] = *reinterpret_cast<const u32x4*>(wp0 + (int64_t)(kt + u) * 1024);
      w[1][u] = *reinterpret_cast<const u32x4*>(wp1 + (int64_t)(kt + u) * 1024);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < XW; ++h)
          x[mt][u][h] = *reinterpret_cast<const u32x4*>(xp[mt] + (int64_t)(kt + u) * XSTEP + h * 16);
  };
  auto compute = [&](const u32x4 (&w)[2][U], const u32x4 (&x)[MT][U][XW]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][0] = mma_tile<WT>(w[0][u], x[mt][u], acc[mt][0]);
        acc[mt][1] = mma_tile<WT>(w[1][u], x[mt][u], acc[mt][1]);
      }
  };

  // Two register stages; inside the loop every load is unconditional so the
  // compiler's wait counts keep the next stage's loads in flight while the
  // current stage's MFMAs run.
  // sched_barrier keeps the scheduler from sinking the prefetch loads next to
  // their uses, which would serialise the stages again.
  const int nfull = KT / U;
  if (nfull > 0) {
    load(wA, xA, 0);
    int b = 0;
    for (; b + 2 < nfull; b += 2) {
      load(wB, xB, (b + 1) * U);
      __builtin_amdgcn_sched_barrier(0);
      compute(wA, xA);
      __builtin_amdgcn_sched_barrier(0);
      load(wA, xA, (b + 2) * U);
      __builtin_amdgcn_sched_barrier(0);
      compute(wB, xB);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (b + 1 < nfull) {
      load(wB, xB, (b + 1) * U);
      __builtin_amdgcn_sched_barrier(0);
      compute(wA, xA);
      __builtin_amdgcn_sched_barrier(0);
      compute(wB, xB);
    } else {
      compute(wA, xA);
    }
  }
  for (int kt = nfull * U; kt < KT; ++kt) {
    u32x4 w0 = *reinterpret_cast<const u32x4*>(wp0 + (int64_t)kt * 1024);
    u32x4 w1 = *reinterpret_cast<const u32x4*>(wp1 + (int64_t)kt * 1024);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 xx[XW];
#pragma unroll
      for (int h = 0; h < XW; ++h) xx[h] = *reinterpret_cast<const u32x4*>(xp[mt] + (int64_t)kt * XSTEP + h * 16);
      acc[mt][0] = mma_tile<WT>(w0, xx, acc[mt][0]);
      acc[mt][1] = mma_tile<WT>(w1, xx, acc[mt][1]);
    }
  }

  // ---- epilogue: lane holds Y[row][n..n+3] of tile (mt, nw) ----
  const int nq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + (lane & 15);
    if (r >= rows) continue;
    const int row = row0 + r;
    if constexpr (EPI == EPI_SWIGLU) {
      const int j = (nt0 >> 1) * 16 + nq;   // hidden column
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float g = acc[mt][0][q], u = acc[mt][1][q];
        if (a.wscale) {
          const float* sc = a.wscale + (int64_t)group * a.s_gstride;
          g *= sc[nt0 * 16 + nq + q];
          u *= sc[(nt0 + 1) * 16 + nq + q];
        }
        v[q] = silu(g) * u;
      }
      store4<AT>(a.Y, (int64_t)row * a.ldy + j, v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int nw = 0; nw < 2; ++nw) {
        const int n = (nt0 + nw) * 16 + nq;
        if (n >= a.N) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[mt][nw][q];
        if (a.wscale) {
          const float* sc = a.wscale + (int64_t)group * a.s_gstride;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] *= sc[n + q];
        }
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
              float c0 = cs[0], s0 = cs[1], c1 = cs[2], s1 = cs[3];
              float rx0 = x0 * c0 - y0 * s0, ry0 = y0 * c0 + x0 * s0;
              float rx1 = x1 * c1 - y1 * s1, ry1 = y1 * c1 + x1 * s1;
              x0 = rx0; y0 = ry0; x1 = rx1; y1 = ry1;
            }
            if (n < qdim) {
              int64_t base = (int64_t)row * a.ldy + head * dh;
              store2<AT>(a.Y, base + i0, x0, x1);
              store2<AT>(a.Y, base + i0 + half, y0, y1);
            } else {
              int64_t base = (int64_t)req * a.kv_req_stride + ((int64_t)head * a.max_ctx + pos) * dh;
              store2<AT>(a.kc, base + i0, x0, x1);
              store2<AT>(a.kc, base + i0 + half, y0, y1);
            }
          } else {
            const int c = n - qdim - kdim;
            const int head = c / dh, dd = c % dh;
            int64_t base = (int64_t)req * a.kv_req_stride + ((int64_t)head * dh + dd) * a.max_ctx + pos;
#pragma unroll
            for (int q = 0; q < 4; ++q) store1<AT>(a.vc, base + (int64_t)q * a.max_ctx, v[q]);
          }
        }
      }
    }
  }
}

template <int WT, int AT, int MT, int EPI>
static void run(const GemmArgs& a, hipStream_t s) {
  int64_t blocks = (int64_t)a.max_tiles * a.n_chunks * (a.ksplit > 1 ? a.ksplit : 1);
  blocks = round_up(blocks, 8);
  hipLaunchKernelGGL((k_gemm<WT, AT, MT, EPI>), dim3((unsigned)blocks), dim3(256), 0, s, a);
}

template <int WT, int AT, int MT>
static void run_epi(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_F32: run<WT, AT, MT, EPI_F32>(a, s); break;
    case EPI_ROWS: run<WT, AT, MT, EPI_ROWS>(a, s); break;
    case EPI_RESID: run<WT, AT, MT, EPI_RESID>(a, s); break;
    case EPI_SWIGLU: run<WT, AT, MT, EPI_SWIGLU>(a, s); break;
    case EPI_QKV: run<WT, AT, MT, EPI_QKV>(a, s); break;
  }
}

template <int WT, int AT>
static void run_mt(int mt, int epi, const GemmArgs& a, hipStream_t s) {
  switch (mt) {
    case 1: run_epi<WT, AT, 1>(epi, a, s); break;
    case 2: run_epi<WT, AT, 2>(epi, a, s); break;
    case 4: run_epi<WT, AT, 4>(epi, a, s); break;
  }
}

void launch_gemm(int wdt, int adt, int mt, int epi, const GemmArgs& a, hipStream_t s) {
  if (wdt == DT_F32) run_mt<DT_F32, DT_F32>(mt, epi, a, s);
  else if (wdt == DT_BF16) run_mt<DT_BF16, DT_BF16>(mt, epi, a, s);
  else run_mt<DT_FP8, DT_BF16>(mt, epi, a, s);
}

}  // namespace cd
