// Fused vocabulary-wide sampler.
//
// Pass 1 (k_sample_part): the fp32 logits are read exactly once.  Each row
// is cut into chunks of at most 8192 logits, one 256-thread workgroup per
// (row, chunk), so a 256-row canvas launches 8192 workgroups; each thread
// streams 16-byte loads, four in flight, and keeps an online (max m, S = sum e^(z-m),
// U = sum e^(z-m)(z-m), index of the first max).  Partials merge across the
// wave with shuffles and across waves through LDS.
// Pass 2 (k_sample_final): one workgroup per request, one thread per canvas
// position, merges that row's chunk partials in fp64 and derives
// entropy H = ln S - U/S (nats), max prob 1/S and the argmax; locks when max
// prob > threshold (position takes the argmax), else re-noises with
// Philox(seed; position, pass, block, request); then the canvas mean entropy,
// argmax stability against the previous pass and the stop flag.
#include "common.h"
#include "kernels.h"
#include "../../include/cd.h"

namespace cd {

struct Acc { float m, S, U; int idx; };

__device__ __forceinline__ Acc merge(Acc a, Acc b) {
  if (b.m > a.m || (b.m == a.m && b.idx < a.idx)) { Acc t = a; a = b; b = t; }   // a holds the max
  if (b.m == -INFINITY) return a;
  const float d = b.m - a.m;          // <= 0
  const float f = __expf(d);
  Acc r;
  r.m = a.m;
  r.idx = a.idx;
  r.S = a.S + f * b.S;
  r.U = a.U + f * (b.U + d * b.S);
  return r;
}

__global__ __launch_bounds__(256) void k_sample_part(SampleArgs a) {
  __shared__ Acc sh[4];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int64_t base = (int64_t)row * a.V + (int64_t)chunk * a.chunk;
  const float4* z4 = reinterpret_cast<const float4*>(a.logits + base);
  const float L2E = 1.4426950408889634f;
  float m = -INFINITY, S = 0.f, U = 0.f;
  int idx = 0x7FFFFFFF;
  const int n4 = a.chunk / 4;
  // Four 16-byte loads per thread are issued before any is used (indices
  // clamped, so none is conditional; non-temporal: the logits are read once),
  // then taken in the order i, i+256, ... as a one-load loop would.
  constexpr int UNR = 4;
  typedef float f32v4 __attribute__((ext_vector_type(4)));
  const f32v4* zv = reinterpret_cast<const f32v4*>(z4);
  for (int i0 = threadIdx.x; i0 < n4; i0 += 256 * UNR) {
    f32v4 vv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) vv[u] = __builtin_nontemporal_load(zv + min(i0 + u * 256, n4 - 1));
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * 256;
      if (i >= n4) break;
      float z[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      float vm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      if (vm > m) {
        int j = 0;
        while (z[j] != vm) ++j;
        if (m != -INFINITY) {
          const float dd = m - vm;
          const float f = exp2f(dd * L2E);
          U = f * (U + dd * S);
          S = f * S;
        }
        m = vm;
        idx = chunk * a.chunk + 4 * i + j;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float dz = z[q] - m;
        const float e = exp2f(dz * L2E);
        S += e;
        U += e * dz;
      }
    }
  }
  // a NaN logit never passes the comparisons above; make it visible
  Acc acc = {m, S, U, idx};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Acc b;
    b.m = __shfl_xor(acc.m, o, 64);
    b.S = __shfl_xor(acc.S, o, 64);
    b.U = __shfl_xor(acc.U, o, 64);
    b.idx = __shfl_xor(acc.idx, o, 64);
    acc = merge(acc, b);
  }
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    Acc r = merge(merge(sh[0], sh[1]), merge(sh[2], sh[3]));
    a.part[(int64_t)row * a.n_chunks + chunk] = make_float4(r.m, r.S, r.U, __int_as_float(r.idx));
  }
}

__global__ __launch_bounds__(256) void k_sample_final(SampleArgs a) {
  __shared__ double shH[4];
  __shared__ int shL[4], shS[4], shX[4], shN[4];
  const int rr = blockIdx.x;            // request within the call
  int step, block, req;
  uint64_t seed;
  if (a.rq) {
    // a slot without an active canvas rides along in the pass: its rows were
    // computed, but none of its state changes; its record reads step 0
    const int ra = a.req0 + rr;
    if (!((a.active[ra >> 6] >> (ra & 63)) & 1)) {
      if (threadIdx.x == 0) {
        cd_step_info z = {};
        reinterpret_cast<cd_step_info*>(a.info)[rr] = z;
      }
      return;
    }
    step = a.rq[rr].t + 1; block = a.rq[rr].block; req = a.rq[rr].rid; seed = a.rq[rr].seed;
  } else {
    step = a.step; block = a.block; req = a.req0 + rr; seed = a.seed;
  }
  double Hsum = 0.0;
  int nlock = 0, stable = 1, xeq = 1, nonfin = 0;
  for (int i = threadIdx.x; i < a.C; i += 256) {
    const int64_t row = (int64_t)rr * a.C + i;
    // the row's chunk partials in groups of 8, each group loaded before use
    // (indices clamped: a repeated last chunk leaves the maximum unchanged and
    // is skipped in the sums), chunks taken in ascending order
    const float4* pr = a.part + row * a.n_chunks;
    const int nc = a.n_chunks;
    double M = -INFINITY;
    for (int c0 = 0; c0 < nc; c0 += 8) {
      float mx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mx[u] = pr[min(c0 + u, nc - 1)].x;
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmax(M, (double)mx[u]);
    }
    double S = 0.0, U = 0.0;
    int idx = 0x7FFFFFFF;
    for (int c0 = 0; c0 < nc; c0 += 8) {
      float4 pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = pr[min(c0 + u, nc - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float4 p = pv[u];
        if (c0 + u >= nc || p.x == -INFINITY) continue;
        const double d = (double)p.x - M;
        const double f = exp(d);
        S += f * (double)p.y;
        U += f * ((double)p.z + d * (double)p.y);
        if ((double)p.x == M) idx = min(idx, __float_as_int(p.w));
      }
    }
    const double H = log(S) - U / S;
    const double pm = 1.0 / S;
    const bool bad = !(S >= 1.0) || !isfinite(S) || !isfinite(U) || !isfinite(M);
    if (bad) { nonfin = 1; idx = 0; }
    const bool lk = !bad && (a.lock_rule ? H <= (double)a.ent_bound : pm > (double)a.lock_th);
    const int tok = lk ? idx : canvas_token(seed, i, step, block, req, a.V);
    if (a.prev_a && a.prev_a[row] != idx) stable = 0;
    if (a.canvas_in && a.canvas_in[row] != idx) xeq = 0;
    a.argmax[row] = idx;
    a.entropy[row] = H;
    a.pmax[row] = pm;
    a.lock[row] = lk ? 1 : 0;
    a.tokens[row] = tok;
    Hsum += H;
    nlock += lk;
  }
  // block reductions
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Hsum += __shfl_xor(Hsum, o, 64);
    nlock += __shfl_xor(nlock, o, 64);
    stable &= __shfl_xor(stable, o, 64);
    xeq &= __shfl_xor(xeq, o, 64);
    nonfin |= __shfl_xor(nonfin, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { shH[w] = Hsum; shL[w] = nlock; shS[w] = stable; shX[w] = xeq; shN[w] = nonfin; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double Hbar = (shH[0] + shH[1] + shH[2] + shH[3]) / a.C;
    const int st = a.prev_a ? (shS[0] & shS[1] & shS[2] & shS[3]) : 0;
    cd_step_info inf;
    inf.step = step;
    inf.n_locked = shL[0] + shL[1] + shL[2] + shL[3];
    inf.stable = (step >= 2) ? st : 0;
    inf.canvas_is_argmax = a.canvas_in ? (shX[0] & shX[1] & shX[2] & shX[3]) : 0;
    inf.nonfinite = shN[0] | shN[1] | shN[2] | shN[3];
    inf.mean_entropy = Hbar;
    inf.stop = (step >= a.max_steps) || (step >= 2 && inf.stable && Hbar < (double)a.stop_H);
    reinterpret_cast<cd_step_info*>(a.info)[rr] = inf;
    if (a.rq) a.rq[rr].t = step;
  }
}

void launch_sampler_part(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sample_part, dim3(a.n_chunks, a.rows), dim3(256), 0, s, a);
}
void launch_sampler_final(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sample_final, dim3(a.rows / a.C), dim3(256), 0, s, a);
}

}  // namespace cd
