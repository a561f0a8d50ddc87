// MoE routing: top-k over router logits, deterministic counting sort of the
// (token, slot) assignments by expert, the tile table of the grouped GEMM,
// and the gate-weighted combine back into the residual stream.
//
// Top-k: one wave per token; k rounds of a wave-wide argmax (ties to the
// lower expert id); gates = softmax over the k selected logits.
// Sort: assignments (t, j) in order t*k + j are cut into blocks of 512; one
// thread per expert counts its assignments per block, a single workgroup
// turns the counts into per-block bases and expert segments padded to the
// GEMM row tile, and the same per-expert scan places every assignment.  The
// permuted order is therefore (expert, token, slot) regardless of timing.
#include "common.h"
#include "kernels.h"

namespace cd {

constexpr int ROUTE_BLK = 512;

// One wave per token; lane j ends up holding the j-th choice.  Non-finite
// logits cannot produce an invalid id: NaN ranks as -inf and every round
// picks the best expert not yet taken (ties and -inf to the lowest id), so
// the k ids are always distinct and inside [0, E).
__global__ __launch_bounds__(256) void k_topk(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  // logit = sum of the router's split partials, added in split order; all
  // partials of a lane are loaded before the first add so the loads overlap
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float x = -INFINITY;
    if (e < a.E) {
      float part[MAX_ROUTER_SPLIT];
#pragma unroll
      for (int s = 0; s < MAX_ROUTER_SPLIT; ++s)
        part[s] = s < a.nsplit ? a.logits[((int64_t)s * a.T + t) * a.E + e] : 0.f;
      x = 0.f;
#pragma unroll
      for (int s = 0; s < MAX_ROUTER_SPLIT; ++s)
        if (s < a.nsplit) x += part[s];
      if (x != x) x = -INFINITY;
    }
    v[i] = x;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < a.E && !(taken & (1u << i)) && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == j) { my_v = bv; my_id = bi; }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == bi) taken |= 1u << i;
  }
  // gates: softmax over the k selected logits (lane 0 holds the largest);
  // uniform if every selected logit is -inf
  const float mx = __shfl(my_v, 0, 64);
  float g = lane < a.k ? (mx == -INFINITY ? 1.f : expf(my_v - mx)) : 0.f;
  const float sum = wave_sum(g);
  if (lane < a.k) {
    g = g / sum;
    a.topk_id[(int64_t)t * a.k + lane] = my_id;
    a.topk_gate[(int64_t)t * a.k + lane] = g;
    if (a.trace_ids) a.trace_ids[(int64_t)t * a.k + lane] = my_id;
    if (a.trace_gates) a.trace_gates[(int64_t)t * a.k + lane] = g;
  }
}

// Small batches: count, scan, tile table and placement in one workgroup.
// Thread g owns the 16 consecutive assignments of group g; cnt[e][g] counts
// expert e in group g and becomes, after a per-expert prefix over groups, the
// rank base of that group inside expert e's segment.  Ranks therefore follow
// assignment order (token, slot).
constexpr int RG = 16;
constexpr int ROUTE_ONE_CNT = 24576;   // E * groups (uint16 LDS cells)

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x - v;
}

__global__ __launch_bounds__(256) void k_route_one(RouteArgs a) {
  __shared__ uint16_t cnt[ROUTE_ONE_CNT];
  __shared__ int32_t seg[256], tile0[256], tot[256];
  __shared__ int32_t totals[2];
  const int n = a.T * a.k, ng = (n + RG - 1) / RG, E = a.E;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < E * ng; i += 256) cnt[i] = 0;
  __syncthreads();
  int ex[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    const int i = tid * RG + j;
    const int e = (tid < ng && i < n) ? a.topk_id[i] : -1;
    ex[j] = (e >= 0 && e < E) ? e : -1;
  }
#pragma unroll
  for (int j = 0; j < RG; ++j)
    if (ex[j] >= 0) cnt[ex[j] * ng + tid] += 1;          // column tid is this thread's alone
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int c = 0; c < ng; ++c) {
      const int v = cnt[tid * ng + c];
      cnt[tid * ng + c] = (uint16_t)run;
      run += v;
    }
    tot[tid] = run;
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
    const int pad = (total + a.mrows - 1) / a.mrows * a.mrows;
    a.seg_off[tid] = off;
    for (int i = 0; i * a.mrows < total; ++i) {
      int32_t* tl = a.tiles + 4 * (int64_t)(tile0[tid] + i);
      tl[0] = tid;
      tl[1] = off + i * a.mrows;
      tl[2] = min(a.mrows, total - i * a.mrows);
      tl[3] = 0;
    }
    for (int r = off + total; r < off + pad; ++r) a.row_map[r] = -1;
  }
  if (tid < ng) {
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int e = ex[j];
      if (e < 0) continue;
      int r = 0;
#pragma unroll
      for (int jj = 0; jj < j; ++jj) r += (ex[jj] == e);
      const int slot = seg[e] + cnt[e * ng + tid] + r;
      const int i = tid * RG + j;
      a.slot[i] = slot;
      a.row_map[slot] = i / a.k;
    }
  }
}

__global__ __launch_bounds__(256) void k_route_count(RouteArgs a) {
  __shared__ int32_t ex[ROUTE_BLK];
  const int b = blockIdx.x;
  const int n = a.T * a.k;
  const int beg = b * ROUTE_BLK, cnt = min(ROUTE_BLK, n - beg);
  for (int i = threadIdx.x; i < cnt; i += 256) ex[i] = a.topk_id[beg + i];
  __syncthreads();
  const int e = threadIdx.x;   // ids outside [0, E) match no expert
  if (e >= a.E) return;
  int c = 0;
  for (int i = 0; i < cnt; ++i) c += (ex[i] == e);
  a.blk_cnt[(int64_t)b * a.E + e] = c;
}

// single workgroup: per-block bases, padded segments, tile table, pad rows
__global__ __launch_bounds__(256) void k_route_scan(RouteArgs a, int n_blk) {
  __shared__ int32_t padded[256], tcount[256];
  const int e = threadIdx.x;
  int total = 0;
  if (e < a.E) {
    // counts are loaded 16 blocks at a time so the loads overlap
    for (int b0 = 0; b0 < n_blk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < n_blk ? a.blk_cnt[(int64_t)(b0 + j) * a.E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < n_blk) a.blk_cnt[(int64_t)(b0 + j) * a.E + e] = total;   // exclusive base within the expert
        total += c[j];
      }
    }
  }
  const int pad = (total + a.mrows - 1) / a.mrows * a.mrows;
  padded[e] = e < a.E ? pad : 0;
  tcount[e] = e < a.E ? pad / a.mrows : 0;
  __syncthreads();
  if (e == 0) {
    int acc = 0, tacc = 0;
    for (int i = 0; i < a.E; ++i) {
      int p = padded[i], tc = tcount[i];
      padded[i] = acc; tcount[i] = tacc;
      acc += p; tacc += tc;
    }
    a.seg_off[a.E] = acc;
    *a.n_tiles = tacc;
  }
  __syncthreads();
  if (e >= a.E) return;
  const int off = padded[e];
  a.seg_off[e] = off;
  int t0 = tcount[e];
  for (int i = 0; i * a.mrows < total; ++i) {
    int32_t* tl = a.tiles + 4 * (int64_t)(t0 + i);
    tl[0] = e;
    tl[1] = off + i * a.mrows;
    tl[2] = min(a.mrows, total - i * a.mrows);
    tl[3] = 0;
  }
  for (int r = off + total; r < off + pad; ++r) a.row_map[r] = -1;
}

__global__ __launch_bounds__(256) void k_route_place(RouteArgs a) {
  __shared__ int32_t ex[ROUTE_BLK];
  const int b = blockIdx.x;
  const int n = a.T * a.k;
  const int beg = b * ROUTE_BLK, cnt = min(ROUTE_BLK, n - beg);
  for (int i = threadIdx.x; i < cnt; i += 256) ex[i] = a.topk_id[beg + i];
  __syncthreads();
  const int e = threadIdx.x;
  if (e >= a.E) return;
  int slot = a.seg_off[e] + a.blk_cnt[(int64_t)b * a.E + e];
  for (int i = 0; i < cnt; ++i) {
    if (ex[i] == e) {
      const int asg = beg + i;
      a.slot[asg] = slot;
      a.row_map[slot] = asg / a.k;
      ++slot;
    }
  }
}

void launch_route(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  const int ng = (a.T * a.k + RG - 1) / RG;
  if (ng <= 256 && ng * a.E <= ROUTE_ONE_CNT) {
    hipLaunchKernelGGL(k_route_one, dim3(1), dim3(256), 0, s, a);
    return;
  }
  const int n_blk = (a.T * a.k + ROUTE_BLK - 1) / ROUTE_BLK;
  hipLaunchKernelGGL(k_route_count, dim3(n_blk), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(256), 0, s, a, n_blk);
  hipLaunchKernelGGL(k_route_place, dim3(n_blk), dim3(256), 0, s, a);
}

// h[t] += sum_j gate[t][j] * Y[slot[t][j]]   (j in order: deterministic)
template <int AT>
__global__ __launch_bounds__(256) void k_combine(const void* Yp, const int32_t* slot, const float* gate, int k,
                                                 int d, float* h) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 acc = *reinterpret_cast<const float4*>(h + (int64_t)t * d + c);
    for (int j = 0; j < k; ++j) {
      const float g = gate[(int64_t)t * k + j];
      const int64_t row = slot[(int64_t)t * k + j];
      float y0, y1, y2, y3;
      if constexpr (AT == DT_F32) {
        float4 y = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(Yp) + row * d + c);
        y0 = y.x; y1 = y.y; y2 = y.z; y3 = y.w;
      } else {
        uint2 y = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Yp) + row * d + c);
        y0 = bf2f(y.x & 0xFFFF); y1 = bf2f(y.x >> 16); y2 = bf2f(y.y & 0xFFFF); y3 = bf2f(y.y >> 16);
      }
      acc.x += g * y0; acc.y += g * y1; acc.z += g * y2; acc.w += g * y3;
    }
    *reinterpret_cast<float4*>(h + (int64_t)t * d + c) = acc;
  }
}

void launch_combine(int adt, const void* Yp, const int32_t* slot, const float* gate, int T, int k, int d, float* h,
                    hipStream_t s) {
  if (adt == DT_F32) hipLaunchKernelGGL(k_combine<DT_F32>, dim3(T), dim3(256), 0, s, Yp, slot, gate, k, d, h);
  else hipLaunchKernelGGL(k_combine<DT_BF16>, dim3(T), dim3(256), 0, s, Yp, slot, gate, k, d, h);
}

}  // namespace cd
