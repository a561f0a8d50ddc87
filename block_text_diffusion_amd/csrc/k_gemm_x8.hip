// fp8 x fp8 GEMM on 128-row work items (the batched fp8 model's QKV, O and
// routed-expert projections; the MXFP4 model's routed experts with F4):
//   Y[m][n] = sx[m] * sw[n] * sum_k qx[m][k] qw[n][k]
// qw: E4M3 weights in the packed fragment tiles (per-row scale sw, applied
// by the epilogue like the register path's); qx: E4M3 activations with one
// fp32 scale sx per row, written by k_quant_fp8 just before the launch.
// The contraction runs on the 16x16x128 fp8 MFMA, twice the bf16 rate: a
// stage is two 64-column k-tiles, and one MFMA takes both k-tiles' bytes of
// a lane (32 per operand).  Weights and activations assign the same K
// columns to a lane's bytes (the weight tile and activation fragment layouts
// match), so the product is the dot product whatever order the hardware
// gives the 128 bytes.  Otherwise the structure of k_gemm_x: work item =
// 128 rows x 256 columns, eight waves (all 128 rows x two 16-column weight
// tiles each), activation fragments copied into LDS with global_load_lds,
// weights into registers, DIST stages in flight; two workgroups per CU.
//
// F4: MXFP4 weights (E2M1 codes, one E8M0 scale per 32 columns of a row) on
// the same MFMA with block scales: Y[m][n] = sx[m] * sum_k qx[m][k] *
// e2m1[n][k] * 2^(e[n][k/32] - 127).  With E2M1 in the weight operand, a
// lane's 32 codes are the 32 consecutive columns 128s + 32q.. (q = lane/16)
// of its row, one MX block, and its scale operand is that block's exponent;
// an E4M3 operand gives the lane's bytes 0-15 columns 128s + 16q.. and
// bytes 16-31 columns 128s + 64 + 16q.. (a bounded probe of one-hot
// operands on the GPU showed both), which is the activation fragment
// layout above, so the activations are staged unchanged.  The MXFP4 tile
// (16 rows x 64 columns, 8 code bytes per lane for columns 16c.. of the
// tile) gives a lane its 32 columns as two 8-byte chunks 128 bytes apart,
// and the scale dword of its (row, 32-column half) holds four k-tiles'
// exponents.
#include "common.h"
#include "gemm_epi.h"
#include "kernels.h"

namespace cd {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma_fp8(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                         f32x4 acc) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  // formats E4M3 / E4M3, no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}
// E2M1 weights (32 codes in the first four dwords) with their E8M0 block
// exponent in the low byte of ws, E4M3 activations at unit scale (127)
__device__ __forceinline__ f32x4 mma_fp4(const u32x4& w, uint32_t ws, const u32x4& b0, const u32x4& b1,
                                         f32x4 acc) {
  const i32x8 a = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 0, 0, (int)ws, 0, 127);
}

// Q8_ROWS rows x 256 columns per work item; every wave takes all Q8_MTW row
// tiles and two of the 16 weight tiles, so each weight byte is loaded once
// per workgroup (with two row halves of four tiles each, both halves loaded
// the same weights: 96 instead of 64 KB of global loads per CU and stage; the
// single row group reads twice the activation fragments from LDS and ran the
// 32-request passes 2.4% and the 4096-row prefills 3% faster).  A 256-row
// tile of the routing table (or a 256-row slab of a dense launch) is
// Q8_PIECES work items of Q8_ROWS rows.  128-row items (64 accumulator
// VGPRs, 128 VGPRs in all, 48 KB of LDS) let two workgroups share a CU, so
// one item's first loads and its epilogue overlap the other's MFMAs.  Same
// box against 256-row items (one workgroup per CU): 32-request fp8 pass
// 72.6 -> 68.6 ms (expert gate/up 16.8 -> 15.2, down 14.6 -> 12.5, QKV
// 4.93 -> 4.41 ms), MXFP4 pass 67.2 -> 64.9 ms, fp8-model 4096-token prefill
// 34.1 -> 31.5 ms; results bit-identical (each output keeps its MFMA
// sequence).  Keeping 256-row items for the MXFP4 down projection alone was
// slower (pass 67.5 vs 66.5 ms, down 12.7 vs 11.6 ms, same box).
constexpr int Q8_WAVES = 8, Q8_MTW = 8, Q8_NTW = 2, Q8_WN = 8;
constexpr int Q8_NBUF = 3, Q8_DIST = 2;
constexpr int Q8_ROWS = 16 * Q8_MTW, Q8_PIECES = 256 / Q8_ROWS;
static_assert(Q8_PIECES * Q8_ROWS == 256, "a 256-row tile splits into whole work items");

template <int EPI, bool F4>
__global__ __launch_bounds__(512, 256 / Q8_ROWS) void k_gemm_x8(const GemmArgs a) {
  constexpr int BLK = 2 * Q8_MTW;                 // activation fragments per stage: row tiles x 2 k-tiles
  constexpr int BPW = BLK / Q8_WAVES;             // each wave copies BPW
  // vector loads per wave per stage: fp8, two 16-byte halves per weight
  // tile; F4, two 8-byte code chunks and a scale dword
  constexpr int LPS = BPW + (F4 ? 3 : 2) * Q8_NTW;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[Q8_NBUF][BLK * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Q8_WN, wn = wave % Q8_WN;
  const int nchunks = (a.Nt + 15) / 16;
  // work items dealt to the 8 XCDs tile-major: a row tile's column chunks run
  // back to back on one XCD, so its (gathered) activation rows come into that
  // XCD's L2 once; the row tiles of one expert are adjacent as well, so its
  // weight chunks are shared there too (same-process A/B against chunk-major:
  // 70.9 -> 70.0 ms per 32-request MXFP4 pass, 77.6 -> 76.2 ms fp8)
  int chunk, tile;
  {
    const int nt = a.tiles ? *a.n_tiles * Q8_PIECES : (a.M + Q8_ROWS - 1) / Q8_ROWS;
    const int work = nt * nchunks;
    const int w8 = (work + 7) & ~7;
    const int bid = blockIdx.x;
    if (bid >= w8) return;
    const int logical = (bid & 7) * (w8 >> 3) + (bid >> 3);
    if (logical >= work) return;
    tile = logical / nchunks;
    chunk = logical - tile * nchunks;
  }
  int group = 0, row0, rows;
  if (a.tiles) {
    // piece `part` of table tile t: its rows part*Q8_ROWS.. (a tile with
    // fewer rows leaves its last pieces empty; the whole workgroup returns
    // before its first barrier)
    const int t = tile / Q8_PIECES, part = tile - t * Q8_PIECES;
    group = a.tiles[4 * t];
    row0 = a.tiles[4 * t + 1] + part * Q8_ROWS;
    rows = min(Q8_ROWS, a.tiles[4 * t + 2] - part * Q8_ROWS);
    if (rows <= 0) return;
  } else {
    row0 = tile * Q8_ROWS;
    rows = min(Q8_ROWS, a.M - row0);
  }
  const int KT = a.K / 64;                  // 64-column k-tiles
  const int nst = (KT + 1) / 2;             // stages of two k-tiles (the last may hold one)
  const int nt0 = chunk * 16 + wn * Q8_NTW;
  const bool row_live = wm * Q8_MTW * 16 < rows;
  const uint8_t* wbase = a.W + (int64_t)group * a.w_gstride;
  const uint8_t* wp[Q8_NTW];
  const uint8_t* mxp[Q8_NTW];
  const int qa = lane >> 4;
#pragma unroll
  for (int j = 0; j < Q8_NTW; ++j) {
    const int64_t t = min(nt0 + j, a.Nt - 1);
    if constexpr (F4) {
      wp[j] = wbase + t * KT * 512 + ((lane & 15) + 32 * (qa & 1)) * 8;
      mxp[j] = wbase + a.mx_off + t * ((KT + 3) / 4) * 128 + ((lane & 15) * 2 + (qa & 1)) * 4;
    } else {
      wp[j] = wbase + t * KT * 1024 + lane * 16;
      mxp[j] = nullptr;
    }
  }
  // fragment f = mt*2 + h: rows mt*16.. of k-tile 2s + h; rows past the
  // tile's end read its last row (finite), their results are dropped
  const uint8_t* xsrc[BPW];
  int xh[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int f = wave * BPW + i;
    const int mt = f >> 1;
    xh[i] = f & 1;
    const int r = min(mt * 16 + (lane & 15), rows - 1);
    int src = a.row_map ? a.row_map[row0 + r] : row0 + r;
    if (src < 0) src = 0;
    xsrc[i] = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)src * a.ldx + (lane >> 4) * 16;
  }

  f32x4 acc[Q8_MTW][Q8_NTW];
#pragma unroll
  for (int mt = 0; mt < Q8_MTW; ++mt)
#pragma unroll
    for (int j = 0; j < Q8_NTW; ++j) acc[mt][j] = f32x4{0, 0, 0, 0};
  u32x4 w[Q8_DIST][Q8_NTW][F4 ? 1 : 2];
  uint32_t wsd[Q8_DIST][Q8_NTW];   // F4: the scale dwords

  // k-tile indices past the end are clamped to the last one: every copy
  // stays in bounds (a missing second k-tile gets a copy of the last one,
  // whose weights the MFMA then takes as zero)
  auto issue = [&](int s) {
    uint8_t* dst = xs[s % Q8_NBUF] + wave * BPW * 1024;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int kt = min(2 * s + xh[i], KT - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xsrc[i] + (int64_t)kt * 64),
                                       (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
  };
  // F4: the lane's k-tile is 2s + q/2, clamped like the copies (the codes
  // of a k-tile past the end are zeroed by compute)
  auto issue_w = [&](u32x4 (&ww)[Q8_NTW][F4 ? 1 : 2], uint32_t (&sd)[Q8_NTW], int s) {
    if constexpr (F4) {
      const int ktc = min(2 * s + (qa >> 1), KT - 1);
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j) {
        const uint2 c0 = *reinterpret_cast<const uint2*>(wp[j] + (int64_t)ktc * 512);
        const uint2 c1 = *reinterpret_cast<const uint2*>(wp[j] + (int64_t)ktc * 512 + 128);
        ww[j][0] = u32x4{c0.x, c0.y, c1.x, c1.y};
        sd[j] = *reinterpret_cast<const uint32_t*>(mxp[j] + (int64_t)(ktc >> 2) * 128);
      }
    } else {
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ww[j][h] = *reinterpret_cast<const u32x4*>(wp[j] + (int64_t)min(2 * s + h, KT - 1) * 1024);
    }
  };
  // one stage: for each of the wave's 16 row tiles, the fragment pair (two
  // k-tiles) from LDS and two MFMAs; the LDS reads run one row tile ahead
  // of the MFMAs that use them.  SINGLE: the stage holds one k-tile (odd K
  // at the last stage); the weights' second half is zero there, so the
  // second fragment (a finite copy of the last k-tile) adds nothing.  F4:
  // the lanes whose k-tile is past the end (q/2 = 1 there) take zero codes;
  // each lane's exponent is byte (k-tile mod 4) of its scale dword.
  auto compute = [&](const u32x4 (&ww)[Q8_NTW][F4 ? 1 : 2], const uint32_t (&sd)[Q8_NTW], const uint8_t* buf,
                     bool single, int s) {
    u32x4 w1[Q8_NTW];
    uint32_t es[Q8_NTW];
    if constexpr (F4) {
      const bool zero = single && (qa >> 1);
      const int sh = 8 * (min(2 * s + (qa >> 1), KT - 1) & 3);
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j) {
        w1[j] = zero ? u32x4{0, 0, 0, 0} : ww[j][0];
        es[j] = sd[j] >> sh;
      }
    } else {
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j) {
        w1[j] = single ? u32x4{0, 0, 0, 0} : ww[j][1];
        es[j] = 0;
      }
    }
    const uint8_t* p0 = buf + ((wm * Q8_MTW) * 2 * 64 + lane) * 16;
    u32x4 xa[2], xb[2];
    auto rd = [&](u32x4 (&x)[2], int mt) {
      x[0] = *reinterpret_cast<const u32x4*>(p0 + mt * 2048);
      x[1] = *reinterpret_cast<const u32x4*>(p0 + mt * 2048 + 1024);
    };
    rd(xa, 0);
#pragma unroll
    for (int mt = 0; mt < Q8_MTW; mt += 2) {
      rd(xb, mt + 1);
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j)
        acc[mt][j] = F4 ? mma_fp4(w1[j], es[j], xa[0], xa[1], acc[mt][j])
                        : mma_fp8(ww[j][0], w1[j], xa[0], xa[1], acc[mt][j]);
      if (mt + 2 < Q8_MTW) rd(xa, mt + 2);
#pragma unroll
      for (int j = 0; j < Q8_NTW; ++j)
        acc[mt + 1][j] = F4 ? mma_fp4(w1[j], es[j], xb[0], xb[1], acc[mt + 1][j])
                            : mma_fp8(ww[j][0], w1[j], xb[0], xb[1], acc[mt + 1][j]);
    }
    // order: reads of tile 0, then (reads of tile mt+1, MFMAs of tile mt)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int mt = 0; mt + 1 < Q8_MTW; ++mt) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, Q8_NTW, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, Q8_NTW, 0);
  };

#pragma unroll
  for (int j = 0; j < Q8_DIST; ++j) {
    issue(j);
    issue_w(w[j], wsd[j], j);
  }
  for (int s0 = 0; s0 < nst; s0 += Q8_DIST) {
#pragma unroll
    for (int j = 0; j < Q8_DIST; ++j) {
      const int s = s0 + j;
      // stage s has landed for this wave; after the barrier for every wave,
      // and the buffer of stage s-1 (which stage s+DIST reuses) is free
      wait_vmcnt<(Q8_DIST - 1) * LPS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(s + Q8_DIST);
      __builtin_amdgcn_sched_barrier(0);
      if (s < nst && row_live) compute(w[j], wsd[j], xs[s % Q8_NBUF], 2 * s + 1 >= KT, s);
      __builtin_amdgcn_sched_barrier(0);
      issue_w(w[j], wsd[j], s + Q8_DIST);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();   // no LDS copy may still be in flight when the workgroup exits

  const int nq = (lane >> 4) * 4;
  const float* sc = a.wscale ? a.wscale + (int64_t)group * a.s_gstride : nullptr;
#pragma unroll
  for (int mt = 0; mt < Q8_MTW; ++mt) {
    const int r = (wm * Q8_MTW + mt) * 16 + (lane & 15);
    if (r >= rows) continue;
    const int row = row0 + r;
    int src = a.row_map ? a.row_map[row] : row;
    if (src < 0) src = 0;
    const float xsr = a.xscale[src];
#pragma unroll
    for (int j = 0; j < Q8_NTW; j += 2) {
      if (nt0 + j >= a.Nt) break;     // Nt is even: tiles come in valid pairs
      float v0[4], v1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { v0[q] = acc[mt][j][q] * xsr; v1[q] = acc[mt][j + 1][q] * xsr; }
      if constexpr (EPI == EPI_SWIGLU) {
        epi_swiglu<DT_BF16>(a, sc, row, (nt0 + j) * 16 + nq, v0, v1);
      } else {
        epi_store<DT_BF16, EPI>(a, sc, row, (nt0 + j) * 16 + nq, v0, 0);
        epi_store<DT_BF16, EPI>(a, sc, row, (nt0 + j + 1) * 16 + nq, v1, 0);
      }
    }
  }
}

template <int EPI, bool F4>
static void run_x8(const GemmArgs& a, hipStream_t s) {
  const int chunks = (a.Nt + 15) / 16;
  const int tiles = a.tiles ? a.max_tiles * Q8_PIECES : (a.M + Q8_ROWS - 1) / Q8_ROWS;
  const int blocks = (int)round_up((int64_t)tiles * chunks, 8);
  hipLaunchKernelGGL((k_gemm_x8<EPI, F4>), dim3(blocks), dim3(64 * Q8_WAVES), 0, s, a);
}

int launch_gemm_x8(int wdt, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.ksplit > 1 || !a.xscale || a.K % 64 || (wdt != DT_FP8 && wdt != DT_FP4)) return -5;
  if (wdt == DT_FP4) {
    // routed experts only
    switch (epi) {
      case EPI_SWIGLU: run_x8<EPI_SWIGLU, true>(a, s); break;
      case EPI_ROWS: run_x8<EPI_ROWS, true>(a, s); break;
      default: return -5;
    }
    return 0;
  }
  switch (epi) {
    case EPI_RESID: run_x8<EPI_RESID, false>(a, s); break;
    case EPI_SWIGLU: run_x8<EPI_SWIGLU, false>(a, s); break;
    case EPI_QKV: run_x8<EPI_QKV, false>(a, s); break;
    case EPI_ROWS: run_x8<EPI_ROWS, false>(a, s); break;
    default: return -5;
  }
  return 0;
}

// ---- per-row E4M3 quantisation of bf16 activations ------------------------------
// q[r][k] = e4m3(x[r][k] * 448 / amax_r) (nearest even, clamped to +-448),
// s[r] = amax_r / 448 (1 for an all-zero row), so x ~= s[r] * q[r][k].  One
// wave per row, the row held in registers (K <= 4096, a multiple of 64);
// rows at or past *n_dev (if given) are skipped.
__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t* x, int64_t ldx, int n, int K, uint8_t* q,
                                                   int64_t ldq, float* s, const int32_t* n_dev) {
  constexpr int NV = 8;   // 8-element chunks per lane: K <= 64 * 8 * 8
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n_dev) n = min(n, *n_dev);
  if (row >= n) return;
  const int nc = K / 8;
  const uint16_t* xr = x + (int64_t)row * ldx;
  uint4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = *reinterpret_cast<const uint4*>(xr + 8 * min(lane + 64 * i, nc - 1));
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i >= nc) break;
    const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      amax = fmaxf(amax, fmaxf(fabsf(bf2f(w4[t] & 0xFFFF)), fabsf(bf2f(w4[t] >> 16))));
  }
  amax = wave_max(amax);
  const float inv = e4m3_inv(amax);
  if (lane == 0) s[row] = e4m3_scale(amax);
  uint8_t* qr = q + (int64_t)row * ldq;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i >= nc) break;
    const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t o[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      o[t] = e4m3x4(bf2f(w4[2 * t] & 0xFFFF), bf2f(w4[2 * t] >> 16), bf2f(w4[2 * t + 1] & 0xFFFF),
                    bf2f(w4[2 * t + 1] >> 16), inv);
    *reinterpret_cast<uint2*>(qr + 8 * (lane + 64 * i)) = make_uint2(o[0], o[1]);
  }
}

int launch_quant_fp8(const void* x, int64_t ldx, int n, int K, uint8_t* q, int64_t ldq, float* s,
                     const int32_t* n_dev, hipStream_t st) {
  if (K % 64 || K > 64 * 8 * 8 || n < 1) return -5;
  hipLaunchKernelGGL(k_quant_fp8, dim3((n + 3) / 4), dim3(256), 0, st, reinterpret_cast<const uint16_t*>(x), ldx, n,
                     K, q, ldq, s, n_dev);
  return 0;
}

}  // namespace cd
