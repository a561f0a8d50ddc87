// GEMM on 256-row work items with the activations staged in LDS:
// Y[m][n] = sum_k X[m][k] * W[n][k].  A work item is a 256-row slab of a
// dense launch, or a 256-row tile of one expert (grouped launch), times a
// 256-column chunk, so every weight byte feeds 256 rows and every activation
// byte 256 columns (with fp8 weights the items are 128-row halves of these,
// see XRows).  Used for the LM head at the canvas batch and for every
// GEMM at more than 256 rows (batched canvases, prefill).
//  * per k-tile stage the workgroup copies the 16 activation fragments
//    (16 rows x KF columns each, 1 KB, already in MFMA operand order) from
//    global memory straight into LDS with global_load_lds_dwordx4 -- each
//    lane's 16 bytes land at the wave's LDS base + lane*16, which is exactly
//    the fragment layout -- so staging costs no VGPRs;
//  * bf16 and fp32 weights: the 16 weight fragments of the stage (256
//    columns) are copied into LDS the same way, so the two row halves that
//    use a weight tile share one global read of it; fp8 weights go straight
//    into registers (a grouped fp8 launch shares a weight chunk between few
//    row tiles, and there the extra LDS traffic cost more than it saved);
//  * eight waves, two per SIMD: waves 0-3 take rows 0-127 and waves 4-7 rows
//    128-255, each with four weight fragments and its eight activation
//    fragments of the stage read from LDS (one contiguous, conflict-free 1 KB
//    ds_read each);
//  * activations and weights are both prefetched DIST stages ahead, so the
//    one in-order vmcnt counter covers both streams with a single wait per
//    stage;
//  * fp8 weights are widened to bf16 once per stage for all row tiles;
//  * the contraction can also be split into fp32 partials (EPI_F32 with
//    ksplit > 1).
#include "common.h"
#include "gemm_epi.h"
#include "kernels.h"

namespace cd {

constexpr int XWAVES = 8; // two waves per SIMD: one's waits overlap the other's MFMAs
constexpr int XNTW = 4;   // weight tiles per wave: a workgroup covers 256 columns, so the
                          // activations are re-read from L2 once per 256 output columns

// Rows per work item.  bf16 / fp32 weights (staged in LDS, 128 KB per
// workgroup): 256 rows, 16 row tiles, eight per wave (waves 0-3 rows 0-127,
// waves 4-7 rows 128-255).  fp8 weights (in registers): 128 rows, four row
// tiles per wave, so the accumulators take 64 instead of 128 VGPRs and two
// workgroups share a CU, one's first loads and epilogue overlapping the
// other's MFMAs (the 32-request pass's output projection 6.65 -> 5.39 ms,
// same box; the bf16 instantiations ran slower that way: canvas LM head
// 0.44-0.46 -> 0.49 ms, 32-request LM head 12.5 -> 13.7 ms).  A 256-row tile
// of the routing table is then PIECES work items.
template <int WT>
struct XRows {
  static constexpr int MT = WT == DT_FP8 ? 8 : 16;   // 16-row tiles per work item
  static constexpr int MTW = MT / 2;                 // row tiles per wave
  static constexpr int PIECES = 16 / MT, PER_CU = 16 / MT;
};

template <int WT, int AT, int EPI>
__global__ __launch_bounds__(512, (XRows<WT>::PER_CU)) void k_gemm_x(const GemmArgs a) {
  constexpr int XMT = XRows<WT>::MT, XMTW = XRows<WT>::MTW, XPIECES = XRows<WT>::PIECES;
  constexpr int KF = 64 / (WT == DT_F32 ? 4 : WT == DT_BF16 ? 2 : 1);
  constexpr bool F4 = WT == DT_FP4;                   // MXFP4: 512-byte tiles + a scale byte per lane
  constexpr int TB = F4 ? 512 : 1024;                 // bytes per weight tile
  constexpr int XW = (WT >= DT_FP8) ? 2 : 1;          // 1 KB activation fragments per k-tile and row tile
  constexpr int XSTEP = (WT >= DT_FP8) ? 128 : 64;    // activation bytes per k-tile (per lane group)
  constexpr bool WLDS = WT < DT_FP8;                  // weights staged in LDS
  constexpr int NBUF = WLDS ? 4 : 2;
  constexpr int DIST = NBUF - 1;
  constexpr int BLK = XMT * XW;                       // activation fragments per stage
  constexpr int BPW = BLK / XWAVES;                   // activation fragments each wave copies
  constexpr int WFR = WLDS ? 4 * XNTW : 0;            // weight fragments per stage in LDS (256 columns)
  constexpr int WPW = WFR / XWAVES;                   // weight fragments each wave copies
  constexpr int NWP = WLDS ? WPW : XNTW;              // weight streams of this wave
  constexpr int LPS = BPW + NWP * (F4 ? 2 : 1);       // vector loads per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t xs[NBUF][(BLK + WFR) * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;         // row half, column pair
  const int ksplit = a.ksplit > 1 ? a.ksplit : 1;
  const int nchunks = (a.Nt + 4 * XNTW - 1) / (4 * XNTW);
  // Work item = (row tile of up to 256 rows, 256-column chunk, k split).
  // Items are dealt to the 8 XCDs in contiguous runs (the dispatcher deals
  // workgroups round-robin), chunk-major: the row tiles of one weight chunk
  // run back to back on one XCD and share that chunk through its L2.  A
  // dense fp32-output launch over many row slabs (the LM head of a batch of
  // canvases) takes super-tiles of 4 slabs x 8 chunks instead, so the 32
  // items an XCD runs at once read 8 weight chunks and 4 activation slabs
  // rather than one chunk and every slab: at 8192 rows that cuts the bytes
  // streamed from the last-level cache about 2.7x (LM head 12.1 -> 11.4 ms
  // per 32-request pass, same box); the 4096-row prefill's QKV ran 0.3 ms
  // slower that way and stays chunk-major.
  int ks, chunk, tile;
  {
    int nt;
    if (a.tiles) nt = *a.n_tiles * XPIECES;
    else nt = (a.M + XMT * 16 - 1) / (XMT * 16);
    const int work = nt * nchunks * ksplit;
    const int w8 = (work + 7) & ~7;
    const int bid = blockIdx.x;
    if (bid >= w8) return;
    int logical = (bid & 7) * (w8 >> 3) + (bid >> 3);
    if (logical >= work) return;
    ks = logical % ksplit;
    logical /= ksplit;
    if (EPI == EPI_F32 && !a.tiles && ksplit == 1 && nt >= 8 && nt % 4 == 0 && nchunks % 8 == 0) {
      const int i = logical & 31, st = logical >> 5, nsg = nt >> 2;
      const int cg = st / nsg, sg = st - cg * nsg;
      tile = sg * 4 + (i >> 3);
      chunk = cg * 8 + (i & 7);
    } else {
      chunk = logical / nt;
      tile = logical - chunk * nt;
    }
  }
  int group = 0, row0, rows;
  if (a.tiles) {
    // piece `part` of table tile t (a tile of fewer rows leaves its last
    // pieces empty: the workgroup returns before its first barrier)
    const int t = tile / XPIECES, part = tile - t * XPIECES;
    group = a.tiles[4 * t];
    row0 = a.tiles[4 * t + 1] + part * XMT * 16;
    rows = min(XMT * 16, a.tiles[4 * t + 2] - part * XMT * 16);
    if (rows <= 0) return;
  } else {
    row0 = tile * XMT * 16;
    rows = min(XMT * 16, a.M - row0);
  }
  const int KTall = a.K / KF;
  const int kt0 = (int)((int64_t)KTall * ks / ksplit);
  const int nst = (int)((int64_t)KTall * (ks + 1) / ksplit) - kt0;
  // tiles past Nt load a valid tile and store nothing; idle waves still
  // copy activations and meet the barriers
  const int nt0 = chunk * 4 * XNTW + wn * XNTW;
  const int esa = (AT == DT_F32) ? 4 : 2;

  // a wave whose 128 rows all lie past the tile's end skips the MFMAs (it
  // still copies activations and meets every barrier)
  const bool row_live = wm * XMTW * 16 < rows;
  const uint8_t* wbase = a.W + (int64_t)group * a.w_gstride;
  // LDS-staged weights: this wave copies fragments wave*WPW.. of the
  // chunk's 16 tiles; else it loads its own four tiles nt0.. into registers
  const uint8_t* wp[NWP];
  const uint8_t* mxp[NWP];
#pragma unroll
  for (int j = 0; j < NWP; ++j) {
    const int t = WLDS ? chunk * 4 * XNTW + wave * WPW + j : nt0 + j;
    wp[j] = wbase + ((int64_t)min(t, a.Nt - 1) * KTall + kt0) * TB + lane * (TB / 64);
    mxp[j] = wbase + a.mx_off + (int64_t)min(t, a.Nt - 1) * ((KTall + 3) / 4) * 128 +
             ((lane & 15) * 2 + (lane >> 5)) * 4;
  }
  // rows past the tile's end read its last row (finite); their results are dropped
  const uint8_t* xsrc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = wave * BPW + i;
    const int mt = b / XW, h = b % XW;
    const int r = min(mt * 16 + (lane & 15), rows - 1);
    int src = a.row_map ? a.row_map[row0 + r] : row0 + r;
    if (src < 0) src = 0;
    xsrc[i] = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)src * a.ldx * esa + (lane >> 4) * 16 * XW + h * 16 +
              (int64_t)kt0 * XSTEP;
  }

  f32x4 acc[XMTW][XNTW];
#pragma unroll
  for (int mt = 0; mt < XMTW; ++mt)
#pragma unroll
    for (int j = 0; j < XNTW; ++j) acc[mt][j] = f32x4{0, 0, 0, 0};
  u32x4 w[WLDS ? 1 : DIST][XNTW];   // register weight stages (fp8)

  // stage indices past the end are clamped to the last stage: the copies
  // stay in bounds and land in buffers no later stage reads
  auto issue = [&](int s) {
    const int sc = min(s, nst - 1);
    uint8_t* dst = xs[s % NBUF] + wave * BPW * 1024;
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xsrc[i] + (int64_t)sc * XSTEP),
                                       (lds_void*)(dst + i * 1024), 16, 0, 0);
    if constexpr (WLDS) {
      uint8_t* wdst = xs[s % NBUF] + (BLK + wave * WPW) * 1024;
#pragma unroll
      for (int j = 0; j < WPW; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(wp[j] + (int64_t)sc * 1024),
                                         (lds_void*)(wdst + j * 1024), 16, 0, 0);
    }
  };
  auto issue_w = [&](u32x4 (&ww)[XNTW], int s) {
    const int sc = min(s, nst - 1);
#pragma unroll
    for (int j = 0; j < XNTW; ++j) {
      if constexpr (F4) {
        const int kt = kt0 + sc;   // scale byte of k-tile kt in its group of four
        ww[j] = load_fp4(wp[j] + (int64_t)sc * TB, mxp[j] + (int64_t)(kt >> 2) * 128 + (kt & 3));
      }
      else ww[j] = *reinterpret_cast<const u32x4*>(wp[j] + (int64_t)sc * 1024);
    }
  };
  // all 16 row tiles are computed: rows past M hold copies of row M-1 (finite)
  // and their results are dropped, which keeps the loop free of branches
  // LDS fragment reads run one row tile ahead of the MFMAs that use them
  auto compute = [&](const u32x4 (&wr)[XNTW], const uint8_t* buf) {
    u32x4 ww[XNTW];
#pragma unroll
    for (int j = 0; j < XNTW; ++j) {
      if constexpr (WLDS) ww[j] = *reinterpret_cast<const u32x4*>(buf + ((BLK + wn * XNTW + j) * 64 + lane) * 16);
      else ww[j] = wr[j];
    }
    u32x4 xa[XW], xb[XW];
    auto rd = [&](u32x4 (&x)[XW], int mt) {
#pragma unroll
      for (int h = 0; h < XW; ++h)
        x[h] = *reinterpret_cast<const u32x4*>(buf + (((wm * XMTW + mt) * XW + h) * 64 + lane) * 16);
    };
    rd(xa, 0);
    if constexpr (WT >= DT_FP8) {
      // widen the fp8 / MXFP4 weight fragments once for all row tiles
      u32x4 wb[XNTW][2];
#pragma unroll
      for (int j = 0; j < XNTW; ++j) {
        if constexpr (F4) widen_fp4(ww[j], wb[j]);
        else widen_fp8(ww[j], wb[j]);
      }
#pragma unroll
      for (int mt = 0; mt < XMTW; mt += 2) {
        rd(xb, mt + 1);
#pragma unroll
        for (int j = 0; j < XNTW; ++j) {
          acc[mt][j] = mma_bf16(wb[j][0], xa[0], acc[mt][j]);
          acc[mt][j] = mma_bf16(wb[j][1], xa[1], acc[mt][j]);
        }
        if (mt + 2 < XMTW) rd(xa, mt + 2);
#pragma unroll
        for (int j = 0; j < XNTW; ++j) {
          acc[mt + 1][j] = mma_bf16(wb[j][0], xb[0], acc[mt + 1][j]);
          acc[mt + 1][j] = mma_bf16(wb[j][1], xb[1], acc[mt + 1][j]);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < XMTW; mt += 2) {
        rd(xb, mt + 1);
#pragma unroll
        for (int j = 0; j < XNTW; ++j) acc[mt][j] = mma_tile<WT>(ww[j], xa, acc[mt][j]);
        if (mt + 2 < XMTW) rd(xa, mt + 2);
#pragma unroll
        for (int j = 0; j < XNTW; ++j) acc[mt + 1][j] = mma_tile<WT>(ww[j], xb, acc[mt + 1][j]);
      }
    }
    // order: weight reads and reads of tile 0, then (reads of tile mt+1,
    // MFMAs of tile mt)
    constexpr int RD = XW;                                                     // DS reads per tile
    constexpr int MF = XNTW * (WT == DT_F32 ? 4 : (WT >= DT_FP8 ? 2 : 1));     // MFMAs per tile
    __builtin_amdgcn_sched_group_barrier(0x100, (WLDS ? XNTW : 0) + RD, 0);
#pragma unroll
    for (int mt = 0; mt + 1 < XMTW; ++mt) {
      __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
  };

#pragma unroll
  for (int j = 0; j < DIST; ++j) {
    issue(j);
    if constexpr (!WLDS) issue_w(w[j], j);
  }
  for (int s0 = 0; s0 < nst; s0 += DIST) {
#pragma unroll
    for (int j = 0; j < DIST; ++j) {
      const int s = s0 + j;
      // Stage s (activations and weights) has landed for this wave; after
      // the barrier also for every wave, and stage s-1's buffer is free.  A
      // plain s_barrier: __syncthreads' release fence would wait for every
      // outstanding load, draining the prefetch.
      wait_vmcnt<(DIST - 1) * LPS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(s + DIST);
      __builtin_amdgcn_sched_barrier(0);
      if (s < nst && row_live) compute(w[WLDS ? 0 : j], xs[s % NBUF]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!WLDS) {
        issue_w(w[j], s + DIST);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  wait_vmcnt<0>();   // no LDS copy may still be in flight when the workgroup exits

  const int nq = (lane >> 4) * 4;
  const float* sc = a.wscale ? a.wscale + (int64_t)group * a.s_gstride : nullptr;
#pragma unroll
  for (int mt = 0; mt < XMTW; ++mt) {
    const int r = (wm * XMTW + mt) * 16 + (lane & 15);
    if (r >= rows) continue;
    const int row = row0 + r;
#pragma unroll
    for (int j = 0; j < XNTW; j += 2) {
      if (nt0 + j >= a.Nt) break;     // Nt is even: tiles come in valid pairs
      float v0[4], v1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { v0[q] = acc[mt][j][q]; v1[q] = acc[mt][j + 1][q]; }
      if constexpr (EPI == EPI_SWIGLU) {
        epi_swiglu<AT>(a, sc, row, (nt0 + j) * 16 + nq, v0, v1);
      } else {
        epi_store<AT, EPI>(a, sc, row, (nt0 + j) * 16 + nq, v0, ks);
        epi_store<AT, EPI>(a, sc, row, (nt0 + j + 1) * 16 + nq, v1, ks);
      }
    }
  }
}

template <int WT, int AT, int EPI>
static void run_x(const GemmArgs& a, hipStream_t s) {
  // grid sized for the most work items (grouped: max_tiles times the pieces
  // of a tile; dense: the row slabs), rounded to the 8 XCDs; surplus
  // workgroups return at once
  const int chunks = (a.Nt + 4 * XNTW - 1) / (4 * XNTW);
  constexpr int XMT = XRows<WT>::MT;
  const int tiles = a.tiles ? a.max_tiles * XRows<WT>::PIECES : (a.M + XMT * 16 - 1) / (XMT * 16);
  const int blocks = (int)round_up((int64_t)tiles * chunks * (a.ksplit > 1 ? a.ksplit : 1), 8);
  hipLaunchKernelGGL((k_gemm_x<WT, AT, EPI>), dim3(blocks), dim3(64 * XWAVES), 0, s, a);
}

template <int WT, int AT>
static void run_x_epi(int epi, const GemmArgs& a, hipStream_t s) {
  if constexpr (WT == DT_FP4) {   // routed experts only
    if (epi == EPI_SWIGLU) run_x<WT, AT, EPI_SWIGLU>(a, s);
    else run_x<WT, AT, EPI_ROWS>(a, s);
  } else {
    switch (epi) {
      case EPI_F32: run_x<WT, AT, EPI_F32>(a, s); break;
      case EPI_RESID: run_x<WT, AT, EPI_RESID>(a, s); break;
      case EPI_SWIGLU: run_x<WT, AT, EPI_SWIGLU>(a, s); break;
      case EPI_QKV: run_x<WT, AT, EPI_QKV>(a, s); break;
      case EPI_ROWS: run_x<WT, AT, EPI_ROWS>(a, s); break;
    }
  }
}

int launch_gemm_x(int wdt, int adt, int epi, const GemmArgs& a, hipStream_t s) {
  if (wdt == DT_FP4 && a.ksplit > 1) return -5;   // MXFP4 scales are indexed from k-tile 0
  if (wdt == DT_F32) run_x_epi<DT_F32, DT_F32>(epi, a, s);
  else if (wdt == DT_BF16) run_x_epi<DT_BF16, DT_BF16>(epi, a, s);
  else if (wdt == DT_FP8) run_x_epi<DT_FP8, DT_BF16>(epi, a, s);
  else run_x_epi<DT_FP4, DT_BF16>(epi, a, s);
  return 0;
}

}  // namespace cd
