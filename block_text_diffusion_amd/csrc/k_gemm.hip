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
//    wave per row block;
//  * the activation fragments of a stage (rows of row-major X, optionally
//    through a row map for the MoE gather) are copied once per workgroup
//    straight into LDS (global_load_lds) and read there by all 4 waves,
//    instead of each wave fetching the same fragments from L2;
//  * the k loop is software pipelined in stages of 4 k-tiles, issued two
//    stages ahead (two weight register sets, three LDS buffers), keeping
//    8-16 KB of weight loads in flight per wave;
//  * the product is computed transposed (A = weight tile, B = activation
//    tile), so each lane ends with 4 consecutive output columns of one row
//    and the epilogues store 8-16 contiguous bytes per lane;
//  * dense launches remap block ids so that the row blocks of one weight
//    slice run on the same XCD and share its L2; grouped launches deal their
//    real tiles evenly to the 8 XCDs.
// Epilogues: fp32 store (router / LM head logits), row store (expert
// outputs), fp32 residual add, SwiGLU of interleaved gate/up tiles, and
// QKV with rotary embedding scattering K/V into the cache.
#include "common.h"
#include "gemm_epi.h"
#include "kernels.h"

namespace cd {

// NW waves per workgroup, NTW = 8/NW weight tiles per wave: a workgroup
// always covers 8 weight tiles (128 columns).  Four waves of two tiles suit
// launches with several workgroups per CU and the SwiGLU epilogue (gate and
// up tiles in one wave); eight waves of one tile put two waves on each SIMD
// when a dense launch has only about one workgroup per CU.
template <int WT, int AT, int MT, int EPI, int NW, int CT = 8>
__global__ __launch_bounds__(64 * NW) void k_gemm(const GemmArgs a) {
  constexpr int NTW = CT / NW;
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  static_assert(NTW >= 1 && NTW * NW == CT, "weight tiles per wave");
  static_assert(EPI != EPI_SWIGLU || NTW == 2, "SwiGLU needs gate and up tiles in one wave");
  constexpr int MROWS = 16 * MT;
  constexpr int U = 4;
  constexpr bool F4 = WT == DT_FP4;                 // MXFP4: 512-byte tiles + a scale byte per lane
  constexpr int TB = F4 ? 512 : 1024;               // bytes per weight tile
  constexpr int XW = (WT >= DT_FP8) ? 2 : 1;        // 16-byte activation loads per k-tile
  constexpr int XSTEP = (WT >= DT_FP8) ? 128 : 64;  // activation bytes per k-tile
  constexpr int KF = 64 / (WT == DT_F32 ? 4 : WT == DT_BF16 ? 2 : 1);
  constexpr int NFR = MT * U * XW;        // 1 KB activation fragments per stage
  constexpr int FPW = NFR / NW;           // fragments each wave copies
  constexpr int STG = NFR * 1024;
  constexpr int XBUF = 3;
  static_assert(!F4 || U == 4, "MXFP4 scales come as one dword per four k-tiles");
  constexpr int LPS = FPW + NTW * U + (F4 ? NTW : 0);   // vector loads per wave per stage
  static_assert(NFR % NW == 0, "stage fragments");
  __shared__ __attribute__((aligned(1024))) uint8_t xs[XBUF * STG];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Dense launches (chunk-major) remap block ids so the row blocks that share
  // a weight slice run on one XCD (the dispatcher deals workgroups to the 8
  // XCDs round-robin) and share its L2.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int ksplit = a.ksplit > 1 ? a.ksplit : 1;
  int ks, tile, chunk;
  if (a.tiles) {
    // Grouped: the grid is sized for the most tiles routing can produce; the
    // real work (n_tiles x chunks) is dealt evenly to the 8 XCDs in
    // contiguous runs, expert-major: each expert's items form one run, its
    // column chunks in order and, inside a chunk, its row tiles back to back.
    // A hot expert's second and later row tiles then re-read its weights from
    // that XCD's L2 instead of from HBM, and an expert's gathered activation
    // rows are re-read from L2 across its chunks.  Same-process A/B at the
    // canvas batch, logits bit-identical: bf16 gate/up 4.94 -> 4.87 and down
    // 2.75 -> 2.67 ms per pass against every chunk's tiles back to back
    // (chunk-major over all experts), MXFP4 experts about the same.  The tile
    // table gives each tile its index inside its expert and the expert's tile
    // count, which locate the expert's run.
    const int nt = *a.n_tiles;
    const int work = nt * a.n_chunks * ksplit;
    const int w8 = (work + 7) & ~7;
    if (bid >= w8) return;
    int logical = (bid & 7) * (w8 >> 3) + (bid >> 3);
    if (logical >= work) return;
    ks = logical % ksplit;
    logical /= ksplit;
    // the expert's run holds items [first tile x n_chunks, (first tile +
    // tile count) x n_chunks), so the tile of index logical / n_chunks is one
    // of its tiles
    const int t0 = logical / a.n_chunks;
    const int meta = a.tiles[4 * t0 + 3];
    const int ft = t0 - (meta & 0xFFFF), nte = meta >> 16;
    const int local = logical - ft * a.n_chunks;
    chunk = local / nte;
    tile = ft + local - chunk * nte;
  } else {
    int logical = a.chunk_major ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
    ks = logical % ksplit;
    logical /= ksplit;
    if (a.chunk_major) { chunk = logical / a.max_tiles; tile = logical - chunk * a.max_tiles; }
    else { tile = logical / a.n_chunks; chunk = logical - tile * a.n_chunks; }
  }
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
  // a wave past the last weight tile still copies its share of the
  // activations and meets every barrier; it computes on a valid tile and
  // stores nothing
  const int nt0 = chunk * CT + wave * NTW;
  const bool active = nt0 < a.Nt;
  const int ntc = active ? nt0 : 0;

  const int KTall = a.K / KF;
  const int kt_beg = (int)((int64_t)KTall * ks / ksplit);
  const int KT = (int)((int64_t)KTall * (ks + 1) / ksplit) - kt_beg;   // k-tiles of this split
  const int nst = (KT + U - 1) / U;                                      // stages of U k-tiles
  const uint8_t* wp0 = a.W + (int64_t)group * a.w_gstride + ((int64_t)ntc * KTall + kt_beg) * TB + lane * (TB / 64);
  // MXFP4 scales: one dword per lane per four k-tiles (the launcher refuses
  // an MXFP4 launch with a split contraction, so stages start at k-tile 4 * st)
  const int KT4 = (KTall + 3) / 4;
  const uint8_t* mxp0 = a.W + (int64_t)group * a.w_gstride + a.mx_off + (int64_t)ntc * KT4 * 128 +
                        ((lane & 15) * 2 + (lane >> 5)) * 4;
  const int esa = (AT == DT_F32) ? 4 : 2;
  // this wave's share of the activation fragments of a stage: fragment
  // f = (mt*U + u)*XW + h holds rows mt*16.. at k-tile u (half h for fp8)
  const uint8_t* xsrc[FPW];
  int xu[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = wave * FPW + i;
    const int h = f % XW, u = (f / XW) % U, mt = f / (XW * U);
    const int r = mt * 16 + (lane & 15);
    int src = 0;
    if (r < rows) src = a.row_map ? a.row_map[row0 + r] : row0 + r;
    if (src < 0) src = 0;
    xsrc[i] = reinterpret_cast<const uint8_t*>(a.X) + ((int64_t)src * a.ldx) * esa + (lane >> 4) * 16 * XW + h * 16 +
              (int64_t)kt_beg * XSTEP;
    xu[i] = u;
  }

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[mt][j] = f32x4{0, 0, 0, 0};

  u32x4 wA[NTW][U], wB[NTW][U];   // two register stages of the wave's weight tiles

  // loads of stage st (k-tiles st*U ..), clamped to the last k-tile: weights
  // into register set ww, activations straight into LDS buffer st%XBUF
  auto issue = [&](u32x4 (&ww)[NTW][U], int st) {
    const int kt = st * U;
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const int kk = min(kt + xu[i], KT - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xsrc[i] + (int64_t)kk * XSTEP),
                                       (lds_void*)(xs + (st % XBUF) * STG + (wave * FPW + i) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(kt + u, KT - 1);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        if constexpr (F4)
          ww[j][u] = load_fp4_codes(wp0 + ((int64_t)j * KTall + kk) * TB);
        else
          ww[j][u] = *reinterpret_cast<const u32x4*>(wp0 + ((int64_t)j * KTall + kk) * 1024);
      }
    }
    if constexpr (F4) {
      const int s4 = min(st, KT4 - 1);
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        ww[j][0][3] = *reinterpret_cast<const uint32_t*>(mxp0 + ((int64_t)j * KT4 + s4) * 128);
    }
  };
  auto compute = [&](const u32x4 (&ww)[NTW][U], int st) {
    const uint8_t* buf = xs + (st % XBUF) * STG + lane * 16;
    const int nu = min(U, KT - st * U);   // k-tiles of a short last stage
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < nu) {
        if constexpr (WT >= DT_FP8) {
          // widen the fp8 / MXFP4 weight fragments once for all row tiles
          u32x4 wb[NTW][2];
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            if constexpr (F4) {
              u32x4 t = ww[j][u];
              t[2] = (ww[j][0][3] >> (8 * u)) & 0xFFu;   // this k-tile's scale byte
              widen_fp4(t, wb[j]);
            } else {
              widen_fp8(ww[j][u], wb[j]);
            }
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const u32x4 x = *reinterpret_cast<const u32x4*>(buf + ((mt * U + u) * XW + h) * 1024);
#pragma unroll
              for (int j = 0; j < NTW; ++j) acc[mt][j] = mma_bf16(wb[j][h], x, acc[mt][j]);
            }
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            u32x4 x[XW];
#pragma unroll
            for (int h = 0; h < XW; ++h) x[h] = *reinterpret_cast<const u32x4*>(buf + ((mt * U + u) * XW + h) * 1024);
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[mt][j] = mma_tile<WT>(ww[j][u], x, acc[mt][j]);
          }
        }
      }
    }
  };
  // Stage st's loads are issued two stages ahead.  At the top of stage st the
  // wave waits until only stage st+1's loads are outstanding (loads complete
  // in order; at the last stage, until none are), then the barrier makes
  // every wave's activation copies of stage st visible; the copy into the
  // buffer of stage st+2 is issued only after that barrier, when every wave
  // is done with stage st-1, its last reader.  Inside the loop every stage
  // issues (the stages it issues exist), so the same loads are in flight on
  // every path and the compiler's own waits before the MFMAs stay at this
  // stage's loads instead of draining the prefetch; the last two or three
  // stages are peeled off.
  auto step = [&](u32x4 (&ww)[NTW][U], int st, bool more, bool next) {
    if (next) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute(ww, st);
    __builtin_amdgcn_sched_barrier(0);
    if (more) issue(ww, st + 2);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nst > 0) {
    issue(wA, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(wB, 1);   // with a single stage its k-tiles clamp to the last one (unused)
    __builtin_amdgcn_sched_barrier(0);
    int st = 0;
    for (; st + 3 < nst; st += 2) {
      step(wA, st, true, true);
      step(wB, st + 1, true, true);
    }
    const int left = nst - st;   // 1, 2 or 3 stages; st and st+1 already issued
    if (left == 3) {
      step(wA, st, true, true);
      step(wB, st + 1, false, true);
      step(wA, st + 2, false, false);
    } else if (left == 2) {
      step(wA, st, false, true);
      step(wB, st + 1, false, false);
    } else {
      step(wA, st, false, false);
    }
  }
  if (!active) return;

  // ---- epilogue: lane holds Y[row][n..n+3] of tile (mt, nw) ----
  const int nq = (lane >> 4) * 4;
  const float* sc = a.wscale ? a.wscale + (int64_t)group * a.s_gstride : nullptr;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + (lane & 15);
    if (r >= rows) continue;
    const int row = row0 + r;
    if constexpr (EPI == EPI_SWIGLU) {
      float g[4], u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { g[q] = acc[mt][0][q]; u[q] = acc[mt][1][q]; }
      epi_swiglu<AT>(a, sc, row, nt0 * 16 + nq, g, u);
    } else {
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[mt][j][q];
        epi_store<AT, EPI>(a, sc, row, (nt0 + j) * 16 + nq, v, ks);
      }
    }
  }
}

template <int WT, int AT, int MT, int EPI, int NW>
static void run(const GemmArgs& a, hipStream_t s) {
  int64_t blocks = (int64_t)a.max_tiles * a.n_chunks * (a.ksplit > 1 ? a.ksplit : 1);
  blocks = round_up(blocks, 8);
  hipLaunchKernelGGL((k_gemm<WT, AT, MT, EPI, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a);
}

// eight waves for dense launches of at least 32-row tiles, except SwiGLU
template <int WT, int AT, int MT, int EPI>
static void run_nw(const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI != EPI_SWIGLU && MT >= 2) {
    if (!a.tiles) { run<WT, AT, MT, EPI, 8>(a, s); return; }
  }
  run<WT, AT, MT, EPI, 4>(a, s);
}

template <int WT, int AT, int MT>
static void run_epi(int epi, const GemmArgs& a, hipStream_t s) {
  if constexpr (WT == DT_FP4) {   // routed experts only
    if (epi == EPI_SWIGLU) run_nw<WT, AT, MT, EPI_SWIGLU>(a, s);
    else run_nw<WT, AT, MT, EPI_ROWS>(a, s);
  } else {
    switch (epi) {
      case EPI_F32: run_nw<WT, AT, MT, EPI_F32>(a, s); break;
      case EPI_ROWS: run_nw<WT, AT, MT, EPI_ROWS>(a, s); break;
      case EPI_RESID: run_nw<WT, AT, MT, EPI_RESID>(a, s); break;
      case EPI_SWIGLU: run_nw<WT, AT, MT, EPI_SWIGLU>(a, s); break;
      case EPI_QKV: run_nw<WT, AT, MT, EPI_QKV>(a, s); break;
    }
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

int launch_gemm(int wdt, int adt, int mt, int epi, const GemmArgs& a, hipStream_t s) {
  if (wdt == DT_FP4 && a.ksplit > 1) return -5;   // MXFP4 scales are indexed from k-tile 0
  if (wdt == DT_F32) run_mt<DT_F32, DT_F32>(mt, epi, a, s);
  else if (wdt == DT_BF16) run_mt<DT_BF16, DT_BF16>(mt, epi, a, s);
  else if (wdt == DT_FP8) run_mt<DT_FP8, DT_BF16>(mt, epi, a, s);
  else run_mt<DT_FP4, DT_BF16>(mt, epi, a, s);
  return 0;
}

}  // namespace cd
