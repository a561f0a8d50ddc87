// MoE routing: top-k over router logits, the sort of the (token, slot)
// assignments by expert, the tile table of the grouped GEMM, and the
// gate-weighted combine back into the residual stream.
//
// Top-k: sixteen lanes (one DPP row) per token; k rounds of a row-wide argmax
// (ties to the lower expert id); gates = softmax over the k selected logits.
// Sort: an assignment's rank among the earlier assignments of its expert is
// found per wave (wave_match_rank) plus per-expert prefixes over the waves.  Small batches (up to 4096 assignments): one workgroup ranks,
// counts, scans the padded segments and places every assignment.  Larger
// batches: blocks of 512 assignments rank and count, a single workgroup turns
// the counts into per-block bases and expert segments padded to the GEMM row
// tile, and the placement adds segment base, block base and rank.  Either way
// the permuted order is (expert, token, slot) regardless of timing; every row
// of a segment is computed on its own and the combine reads a token's slots
// in choice order, so no result depends on the order inside a segment.
#include "common.h"
#include "kernels.h"

namespace cd {

constexpr int ROUTE_BLK = 512;

// Sixteen lanes (one DPP row) per token, four tokens per wave; lane j of the
// row ends up holding the j-th choice (k <= 16).  Lane l holds experts
// l, l+16, ...; each of the k rounds takes every lane's best expert not yet
// taken and reduces the row with four DPP exchanges (quad swaps, then the
// half-row and row mirrors), keeping the larger logit and on ties the lower
// expert id.  Non-finite logits cannot produce an invalid id: NaN ranks as
// -inf and every round picks the best expert not yet taken (ties and -inf to
// the lowest id), so the k ids are always distinct and inside [0, E).
template <int CTRL>
__device__ __forceinline__ void row_best(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bv), __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, 0xF, 0xF, false);
  const bool b = (ov > bv) | ((ov == bv) & (oi < bi));
  bv = b ? ov : bv;
  bi = b ? oi : bi;
}
template <int CTRL>
__device__ __forceinline__ void row_add(float& v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;

template <int NPL>   // experts per lane: E <= 16 * NPL
__global__ __launch_bounds__(256) void k_topk(RouteArgs a) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int t = (blockIdx.x * 256 + threadIdx.x) >> 4;
  if (t >= a.T) return;   // whole rows leave together
  // logit = sum of the router's split partials, added in split order.  The
  // partials come in chunks of four splits, every load of a chunk issued
  // before the first add and none of them conditional (split and expert
  // indices are clamped; the extra loads are not added), so they overlap.
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += 4) {
    float part[NPL][4];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = min(l16 + 16 * i, a.E - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sp = min(s0 + q, a.nsplit - 1);
        part[i][q] = a.logits[((int64_t)sp * a.T + t) * a.E + e];
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (s0 + q < a.nsplit) v[i] += part[i][q];
  }
  // candidate i of this lane: (logit, expert id); an expert past E or already
  // taken is (-inf, INT_MAX), which no available expert ties with or loses to.
  // A NaN logit ranks as -inf, so the k ids stay distinct experts in [0, E),
  // and it makes the row's gates NaN, so the fault reaches the logits and the
  // sampler's non-finite check instead of vanishing into finite gates.
  int eid[NPL];
  float poison = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l16 + 16 * i;
    const bool live = e < a.E;
    eid[i] = live ? e : 0x7FFFFFFF;
    poison = (live && v[i] != v[i]) ? __builtin_nanf("") : poison;
    v[i] = (live && v[i] == v[i]) ? v[i] : -INFINITY;
  }
  row_add<DPP_QUAD_XOR1>(poison);
  row_add<DPP_QUAD_XOR2>(poison);
  row_add<DPP_ROW_HALF_MIRROR>(poison);
  row_add<DPP_ROW_MIRROR>(poison);
  float my_v = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {   // branch-free: bitwise, not short-circuit, conditions
      const bool b = (v[i] > bv) | ((v[i] == bv) & (eid[i] < bi));
      bv = b ? v[i] : bv;
      bi = b ? eid[i] : bi;
    }
    row_best<DPP_QUAD_XOR1>(bv, bi);
    row_best<DPP_QUAD_XOR2>(bv, bi);
    row_best<DPP_ROW_HALF_MIRROR>(bv, bi);
    row_best<DPP_ROW_MIRROR>(bv, bi);
    my_v = (l16 == j) ? bv : my_v;
    my_id = (l16 == j) ? bi : my_id;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool hit = eid[i] == bi;
      v[i] = hit ? -INFINITY : v[i];
      eid[i] = hit ? 0x7FFFFFFF : eid[i];
    }
  }
  // gates: softmax over the k selected logits (the row's lane 0 holds the
  // largest); uniform if every selected logit is -inf
  const float mx = __shfl(my_v, lane & ~15, 64);
  float g = l16 < a.k ? (mx == -INFINITY ? 1.f : expf(my_v - mx)) : 0.f;
  float sum = g;
  row_add<DPP_QUAD_XOR1>(sum);
  row_add<DPP_QUAD_XOR2>(sum);
  row_add<DPP_ROW_HALF_MIRROR>(sum);
  row_add<DPP_ROW_MIRROR>(sum);
  if (l16 < a.k) {
    g = g / sum + poison;
    a.topk_id[(int64_t)t * a.k + l16] = my_id;
    a.topk_gate[(int64_t)t * a.k + l16] = g;
    if (a.trace_ids) a.trace_ids[(int64_t)t * a.k + l16] = my_id;
    if (a.trace_gates) a.trace_gates[(int64_t)t * a.k + l16] = g;
  }
}

// Small batches (at most 4096 assignments): count, scan, tile table and
// placement in one workgroup of 1024 threads.  The assignments are taken in
// chunks of 64 (one wave each); each chunk ranks and counts its assignments
// per expert in its own row of an LDS table, and a per-expert prefix over the
// chunks turns the counts into bases, so every segment lists its rows in
// assignment order (token, slot).
constexpr int ROUTE_ONE_MAX = 4096;
constexpr int ROUTE_CHUNKS = ROUTE_ONE_MAX / 64;

// Rank of this lane's assignment (expert e, -1: none) among the earlier
// assignments of its wave with the same expert, counted into the wave's own
// LDS row by one LDS atomic per lane.  The LDS resolves the lanes of one
// instruction that hit the same counter in lane order (as measured on gfx950;
// no result depends on it, only the order of rows inside a segment does).
__device__ __forceinline__ int wave_match_rank(int e, uint32_t* counts) {
  return e >= 0 ? (int)atomicAdd(&counts[e], 1u) : 0;
}

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}
__global__ __launch_bounds__(1024) void k_route_one(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t ccnt[ROUTE_CHUNKS * 256];   // [chunk][expert]
  __shared__ int32_t cnt[256], seg[256], tile0[256];
  __shared__ int32_t totals[2];
  constexpr int PT = ROUTE_ONE_MAX / 1024;   // assignments per thread
  const int n = a.T * a.k, E = a.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = (n + 63) / 64;
  int ex[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int i = q * 1024 + tid;
    const int e = i < n ? a.topk_id[i] : -1;
    ex[q] = (e >= 0 && e < E) ? e : -1;
  }
  for (int i = tid * 4; i < nchunk * E; i += 1024 * 4) *reinterpret_cast<uint4*>(ccnt + i) = make_uint4(0, 0, 0, 0);
  __syncthreads();
  // chunk q*16 + wave holds assignments (q*16 + wave)*64 .. +63
  int rk[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) rk[q] = wave_match_rank(ex[q], ccnt + (q * 16 + wave) * E);
  __syncthreads();
  if (tid < E) {
    // exclusive prefix over the chunks, 16 cells loaded before any is used
    int run = 0;
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = c0 + j < nchunk ? ccnt[(c0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c0 + j < nchunk) {
          ccnt[(c0 + j) * E + tid] = (uint32_t)run;
          run += v[j];
        }
    }
    cnt[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PT; ++q)
    if (ex[q] >= 0) rk[q] += ccnt[(q * 16 + wave) * E + ex[q]];
  if (tid < 64) {   // segment and tile offsets: wave-wide exclusive scans, 4 experts per lane
    int pad[4], nt[4], sp = 0, st = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      const int t = e < E ? cnt[e] : 0;
      pad[q] = (t + a.mrows - 1) / a.mrows * a.mrows;
      nt[q] = pad[q] / a.mrows;
      sp += pad[q];
      st += nt[q];
    }
    int ep = wave_excl_scan(sp, lane), et = wave_excl_scan(st, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) { seg[e] = ep; tile0[e] = et; }
      ep += pad[q];
      et += nt[q];
    }
    if (lane == 63) { totals[0] = ep; totals[1] = et; }
  }
  __syncthreads();
  if (tid == 0) { a.seg_off[E] = totals[0]; *a.n_tiles = totals[1]; }
  if (tid < E) {
    const int off = seg[tid], total = cnt[tid];
    a.seg_off[tid] = off;
    for (int i = 0; i * a.mrows < total; ++i) {
      int32_t* tl = a.tiles + 4 * (int64_t)(tile0[tid] + i);
      tl[0] = tid;
      tl[1] = off + i * a.mrows;
      tl[2] = min(a.mrows, total - i * a.mrows);
      // index inside the expert | the expert's tile count << 16 (the
      // row-tiled GEMM's expert-major order; it reads this only below 256 rows
      // per expert on average, where an expert has fewer than 16 E <= 4096 tiles)
      tl[3] = i | (((total + a.mrows - 1) / a.mrows) << 16);
    }
  }
  // padding rows of every segment (fewer than mrows each): wave w takes
  // experts w, w+16, ..., its lanes the rows
  for (int e = tid >> 6; e < E; e += 16) {
    const int total = cnt[e], pad = (total + a.mrows - 1) / a.mrows * a.mrows;
    for (int r = total + lane; r < pad; r += 64) a.row_map[seg[e] + r] = -1;
  }
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    if (ex[q] < 0) continue;
    const int i = q * 1024 + tid;
    const int slot = seg[ex[q]] + rk[q];
    a.slot[i] = slot;
    a.row_map[slot] = i / a.k;
  }
}

// one assignment per thread: its rank inside (block, expert) -- the rank
// inside its wave plus the per-expert prefix over the block's 8 waves, kept
// in slot[] until the placement -- and the block's count per expert
__global__ __launch_bounds__(ROUTE_BLK) void k_route_count(RouteArgs a) {
  constexpr int NWB = ROUTE_BLK / 64;
  __shared__ uint32_t wc[NWB * 256];   // [wave][expert]
  const int b = blockIdx.x, n = a.T * a.k, E = a.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = b * ROUTE_BLK + tid;
  for (int c = tid; c < NWB * E; c += ROUTE_BLK) wc[c] = 0;
  const int e0 = i < n ? a.topk_id[i] : -1;
  const int e = (e0 >= 0 && e0 < E) ? e0 : -1;   // ids outside [0, E) match no expert
  __syncthreads();
  int r = wave_match_rank(e, wc + wave * E);
  __syncthreads();
  if (tid < E) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NWB; ++w) {
      const int c = wc[w * E + tid];
      wc[w * E + tid] = (uint32_t)run;
      run += c;
    }
    a.blk_cnt[(int64_t)b * E + tid] = run;
  }
  __syncthreads();
  if (e >= 0) r += wc[wave * E + e];
  if (i < n) a.slot[i] = r;
}

// single workgroup: per-block bases, padded segments, tile table, pad rows
__global__ __launch_bounds__(256) void k_route_scan(RouteArgs a, int n_blk) {
  __shared__ int32_t tot[256], seg[256], tile0[256];
  __shared__ int32_t totals[2];
  const int tid = threadIdx.x, lane = tid & 63, E = a.E;
  if (tid < E) {
    // counts are loaded 16 blocks at a time so the loads overlap
    int total = 0;
    for (int b0 = 0; b0 < n_blk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < n_blk ? a.blk_cnt[(int64_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < n_blk) a.blk_cnt[(int64_t)(b0 + j) * E + tid] = total;   // exclusive base within the expert
        total += c[j];
      }
    }
    tot[tid] = total;
  }
  __syncthreads();
  if (tid < 64) {   // segment and tile offsets: wave-wide exclusive scans, 4 experts per lane
    int pad[4], nt[4], sp = 0, st = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      const int t = e < E ? tot[e] : 0;
      pad[q] = (t + a.mrows - 1) / a.mrows * a.mrows;
      nt[q] = pad[q] / a.mrows;
      sp += pad[q];
      st += nt[q];
    }
    int ep = wave_excl_scan(sp, lane), et = wave_excl_scan(st, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) { seg[e] = ep; tile0[e] = et; }
      ep += pad[q];
      et += nt[q];
    }
    if (lane == 63) { totals[0] = ep; totals[1] = et; }
  }
  __syncthreads();
  if (tid == 0) { a.seg_off[E] = totals[0]; *a.n_tiles = totals[1]; }
  if (tid < E) {
    const int off = seg[tid], total = tot[tid];
    a.seg_off[tid] = off;
    for (int i = 0; i * a.mrows < total; ++i) {
      int32_t* tl = a.tiles + 4 * (int64_t)(tile0[tid] + i);
      tl[0] = tid;
      tl[1] = off + i * a.mrows;
      tl[2] = min(a.mrows, total - i * a.mrows);
      // index inside the expert | the expert's tile count << 16 (the
      // row-tiled GEMM's expert-major order; it reads this only below 256 rows
      // per expert on average, where an expert has fewer than 16 E <= 4096 tiles)
      tl[3] = i | (((total + a.mrows - 1) / a.mrows) << 16);
    }
  }
  // padding rows of every segment (fewer than mrows each): wave w takes
  // experts w, w+4, ..., its lanes the rows
  for (int e = tid >> 6; e < E; e += 4) {
    const int total = tot[e], pad = (total + a.mrows - 1) / a.mrows * a.mrows;
    for (int r = total + lane; r < pad; r += 64) a.row_map[seg[e] + r] = -1;
  }
}

// one assignment per thread: slot = segment base + block base + rank
__global__ __launch_bounds__(ROUTE_BLK) void k_route_place(RouteArgs a) {
  const int b = blockIdx.x, n = a.T * a.k;
  const int i = b * ROUTE_BLK + threadIdx.x;
  if (i >= n) return;
  const int e = a.topk_id[i];
  if (e < 0 || e >= a.E) return;
  const int slot = a.seg_off[e] + a.blk_cnt[(int64_t)b * a.E + e] + a.slot[i];
  a.slot[i] = slot;
  a.row_map[slot] = i / a.k;
}

void launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.E <= 128) hipLaunchKernelGGL(k_topk<8>, dim3((a.T + 15) / 16), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_topk<16>, dim3((a.T + 15) / 16), dim3(256), 0, s, a);
  if (a.T * a.k <= ROUTE_ONE_MAX) {
    hipLaunchKernelGGL(k_route_one, dim3(1), dim3(1024), 0, s, a);
    return;
  }
  const int n_blk = (a.T * a.k + ROUTE_BLK - 1) / ROUTE_BLK;
  hipLaunchKernelGGL(k_route_count, dim3(n_blk), dim3(ROUTE_BLK), 0, s, a);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(256), 0, s, a, n_blk);
  hipLaunchKernelGGL(k_route_place, dim3(n_blk), dim3(ROUTE_BLK), 0, s, a);
}

// h[t] += sum_j gate[t][j] * Y[slot[t][j]] (j in order: deterministic), then
// + add[t] (the shared FFN's fp32 row) when given.  When u is given the
// workgroup also writes the RMSNorm (unit gain) of the new row into it, the
// input of the next layer or of the LM head.
//
// NI > 0: the row's NI column groups (1024 columns each, d <= 1024 NI) stay in
// registers.  After the gates and slots, every load of the row (h, the k
// expert rows in batches of 8, the shared row) is issued before the first
// use, and the norm is taken from the registers, so a token costs two memory
// round trips.  NI = 0 (d > 4096): one column group at a time.
template <int AT, int NI>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ Yp, const int32_t* __restrict__ slot,
                                                 const float* __restrict__ gate, const float* __restrict__ add,
                                                 int k, int d, float* __restrict__ h, void* __restrict__ u,
                                                 float eps, uint8_t* __restrict__ q8, float* __restrict__ s8) {
  __shared__ float red[4], red8[4];
  const int t = blockIdx.x;
  float g[16];
  int64_t yr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int jc = min(j, k - 1);
    g[j] = gate[(int64_t)t * k + jc];
    yr[j] = slot[(int64_t)t * k + jc];
  }
  auto row8 = [&](int64_t r, int c) -> float4 {
    if constexpr (AT == DT_F32) {
      return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(Yp) + r * d + c);
    } else {
      const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Yp) + r * d + c);
      return make_float4(bf2f(b.x & 0xFFFF), bf2f(b.x >> 16), bf2f(b.y & 0xFFFF), bf2f(b.y >> 16));
    }
  };
  auto put_u = [&](int c, const float4& v, float inv) {
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
  if constexpr (NI > 0) {
    float4 acc[NI], sh[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = min(threadIdx.x * 4 + 1024 * i, d - 4);   // past the row's end: a valid column, unused
      acc[i] = *reinterpret_cast<const float4*>(h + (int64_t)t * d + c);
      sh[i] = add ? *reinterpret_cast<const float4*>(add + (int64_t)t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += 8) {
      if (j0 >= k) break;
      float4 y[NI][8];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) y[i][q] = row8(yr[j0 + q], min(threadIdx.x * 4 + 1024 * i, d - 4));
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (j0 + q < k) {
            const float gq = g[j0 + q];
            acc[i].x += gq * y[i][q].x; acc[i].y += gq * y[i][q].y; acc[i].z += gq * y[i][q].z; acc[i].w += gq * y[i][q].w;
          }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      if (c >= d) continue;
      if (add) { acc[i].x += sh[i].x; acc[i].y += sh[i].y; acc[i].z += sh[i].z; acc[i].w += sh[i].w; }
      *reinterpret_cast<float4*>(h + (int64_t)t * d + c) = acc[i];
      ss += acc[i].x * acc[i].x + acc[i].y * acc[i].y + acc[i].z * acc[i].z + acc[i].w * acc[i].w;
    }
    if (!u) return;
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
    if constexpr (AT == DT_BF16) {
      if (q8) {
        // also the E4M3 row of the bf16 values with its scale (the input of
        // the next layer's fp8 QKV GEMM), as the standalone quantiser would
        uint2 p[NI];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          p[i].x = pack_bf16(acc[i].x * inv, acc[i].y * inv);
          p[i].y = pack_bf16(acc[i].z * inv, acc[i].w * inv);
          if (threadIdx.x * 4 + 1024 * i < d)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf2f(p[i].x & 0xFFFF)), fabsf(bf2f(p[i].x >> 16))),
                                     fmaxf(fabsf(bf2f(p[i].y & 0xFFFF)), fabsf(bf2f(p[i].y >> 16)))));
        }
        amax = wave_max(amax);
        if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red8[0], red8[1]), fmaxf(red8[2], red8[3]));
        const float qi = e4m3_inv(amax);
        if (threadIdx.x == 0) s8[t] = e4m3_scale(amax);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int c = threadIdx.x * 4 + 1024 * i;
          if (c >= d) continue;
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(u) + (int64_t)t * d + c) = p[i];
          *reinterpret_cast<uint32_t*>(q8 + (int64_t)t * d + c) =
              e4m3x4(bf2f(p[i].x & 0xFFFF), bf2f(p[i].x >> 16), bf2f(p[i].y & 0xFFFF), bf2f(p[i].y >> 16), qi);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = threadIdx.x * 4 + 1024 * i;
      if (c < d) put_u(c, acc[i], inv);
    }
  } else {
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
      float4 acc = *reinterpret_cast<const float4*>(h + (int64_t)t * d + c);
#pragma unroll
      for (int j0 = 0; j0 < 16; j0 += 8) {
        if (j0 >= k) break;
        float4 y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = row8(yr[j0 + q], c);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (j0 + q < k) {
            acc.x += g[j0 + q] * y[q].x; acc.y += g[j0 + q] * y[q].y; acc.z += g[j0 + q] * y[q].z; acc.w += g[j0 + q] * y[q].w;
          }
      }
      if (add) {
        const float4 v = *reinterpret_cast<const float4*>(add + (int64_t)t * d + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      *reinterpret_cast<float4*>(h + (int64_t)t * d + c) = acc;
      ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
    }
    if (!u) return;
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
    // each thread reads back the elements of h it wrote itself
    for (int c = threadIdx.x * 4; c < d; c += 1024) put_u(c, *reinterpret_cast<const float4*>(h + (int64_t)t * d + c), inv);
  }
}

template <int AT>
static void run_combine(const void* Yp, const int32_t* slot, const float* gate, const float* add, int T, int k, int d,
                        float* h, void* u, float eps, uint8_t* q8, float* s8, hipStream_t s) {
  const dim3 g(T), b(256);
  switch ((d + 1023) / 1024) {
    case 1: hipLaunchKernelGGL((k_combine<AT, 1>), g, b, 0, s, Yp, slot, gate, add, k, d, h, u, eps, q8, s8); break;
    case 2: hipLaunchKernelGGL((k_combine<AT, 2>), g, b, 0, s, Yp, slot, gate, add, k, d, h, u, eps, q8, s8); break;
    case 3: hipLaunchKernelGGL((k_combine<AT, 3>), g, b, 0, s, Yp, slot, gate, add, k, d, h, u, eps, q8, s8); break;
    case 4: hipLaunchKernelGGL((k_combine<AT, 4>), g, b, 0, s, Yp, slot, gate, add, k, d, h, u, eps, q8, s8); break;
    default:   // d > 4096: no E4M3 rows (the fp8 GEMMs take d <= 4096)
      hipLaunchKernelGGL((k_combine<AT, 0>), g, b, 0, s, Yp, slot, gate, add, k, d, h, u, eps, nullptr, nullptr);
      break;
  }
}

void launch_combine(int adt, const void* Yp, const int32_t* slot, const float* gate, const float* add, int T, int k,
                    int d, float* h, void* u, float eps, hipStream_t s, uint8_t* q8, float* s8) {
  if (adt == DT_F32) run_combine<DT_F32>(Yp, slot, gate, add, T, k, d, h, u, eps, nullptr, nullptr, s);
  else run_combine<DT_BF16>(Yp, slot, gate, add, T, k, d, h, u, eps, u ? q8 : nullptr, s8, s);
}

}  // namespace cd
