// Fused vocabulary-wide sampler.
//
// Pass 1 (k_sample_part): the fp32 logits are read exactly once.  Each row
// is cut into chunks of (normally) at most 8192 logits, one 256-thread
// workgroup per (row, chunk), so a 256-row canvas launches 8192 workgroups;
// each thread loads its 32 logits of a chunk with eight 16-byte loads in
// flight and keeps (max m, S = sum e^(z-m), U = sum e^(z-m)(z-m), index of
// the first max).  Partials merge across the wave with shuffles and across
// waves through LDS.
// Pass 2 (k_sample_final): one workgroup per request, one thread per canvas
// position, merges that row's chunk partials in fp64 and derives
// entropy H = ln S - U/S (nats), max prob 1/S and the argmax; locks when max
// prob > threshold (position takes the argmax), else re-noises with
// Philox(seed; position, pass, block, request); then the canvas mean entropy,
// argmax stability against the previous pass and the stop flag.  A request
// whose stop has fired takes no further pass: a later pass leaves its state
// as it was and flags its record (after_stop).
#include <mutex>

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
  __shared__ float shM[4];
  __shared__ Acc sh[4];
  const int chunk = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int64_t base = (int64_t)row * a.V + (int64_t)chunk * a.chunk;
  typedef float f32v4 __attribute__((ext_vector_type(4)));
  const f32v4* zv = reinterpret_cast<const f32v4*>(a.logits + base);
  const float L2E = 1.4426950408889634f;
  const int n4 = a.chunk / 4;
  // A thread takes its float4s of the chunk in blocks of NL (an 8192-logit
  // chunk is one block): all NL 16-byte non-temporal loads are issued first
  // (indices clamped, so none is conditional; repeats are skipped), the
  // block's maximum is taken, and the exponentials are summed against the
  // running maximum, so no per-element branch rescales the sums (they are
  // rescaled once per block when the maximum grows).  The first argmax is
  // searched for only by the threads that hold the workgroup's maximum.
  constexpr int NL = 8, BLK = NL * 256;
  float m = -INFINITY, S = 0.f, U = 0.f;
  int mb = 0;   // first block of this thread that reached its maximum
  f32v4 v[NL];
  for (int b0 = 0; b0 < n4; b0 += BLK) {
#pragma unroll
    for (int u = 0; u < NL; ++u) v[u] = __builtin_nontemporal_load(zv + min(b0 + tid + u * 256, n4 - 1));
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NL; ++u)
      if (b0 + tid + u * 256 < n4) mx = fmaxf(mx, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    if (mx > m) {
      if (m != -INFINITY) {   // only when a chunk spans several blocks
        const float dd = m - mx;
        const float f = __builtin_amdgcn_exp2f(dd * L2E);
        U = f * (U + dd * S);
        S = f * S;
      }
      m = mx;
      mb = b0;
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      if (b0 + tid + u * 256 >= n4) continue;
      const float z[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // v_exp_f32 directly: an exponent below -126 may come out as 0
        // instead of a subnormal, a change of at most 2^-126 relative to S
        const float dz = z[q] - m;
        const float e = __builtin_amdgcn_exp2f(dz * L2E);
        S += e;
        U += e * dz;
      }
    }
  }
  // the workgroup's maximum (a NaN logit never wins a comparison; it shows
  // up as a NaN sum instead)
  float wm = m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, 64));
  if ((tid & 63) == 0) shM[tid >> 6] = wm;
  __syncthreads();
  wm = fmaxf(fmaxf(shM[0], shM[1]), fmaxf(shM[2], shM[3]));
  int idx = 0x7FFFFFFF;
  if (m == wm && m != -INFINITY) {
    // first element equal to the maximum in this thread's first block that
    // reached it (reloaded when a later block has replaced the registers)
    if (mb + BLK < n4) {
#pragma unroll
      for (int u = 0; u < NL; ++u) v[u] = zv[min(mb + tid + u * 256, n4 - 1)];
    }
#pragma unroll
    for (int u = NL - 1; u >= 0; --u) {
      const int i = mb + tid + u * 256;
      if (i >= n4) continue;
      if (v[u].w == m) idx = chunk * a.chunk + 4 * i + 3;
      if (v[u].z == m) idx = chunk * a.chunk + 4 * i + 2;
      if (v[u].y == m) idx = chunk * a.chunk + 4 * i + 1;
      if (v[u].x == m) idx = chunk * a.chunk + 4 * i;
    }
  }
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
  if ((tid & 63) == 0) sh[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
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
    if (a.rq[rr].stopped) {
      // a pass after the stop of this block is refused for this request: its
      // canvas, argmax and last record stay as they were (the pass did write
      // keys/values of its canvas rows past P, which a commit would have to
      // redo); the record is marked so the next synchronising call reports it
      if (threadIdx.x == 0) reinterpret_cast<cd_step_info*>(a.info)[rr].after_stop = 1;
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
    // the row's chunk partials, up to 32 loaded at once (indices clamped: a
    // repeated last chunk is skipped), merged in ascending chunk order into
    // fp64 sums; exp(m_c - M) <= 1 in fp32 (exactly 1 for the max chunk)
    const float4* pr = a.part + row * a.n_chunks;
    const int nc = a.n_chunks;
    constexpr int NB = 32;
    float M = -INFINITY;
    double S = 0.0, U = 0.0;
    int idx = 0x7FFFFFFF;
    for (int c0 = 0; c0 < nc; c0 += NB) {
      float4 pv[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) pv[u] = pr[min(c0 + u, nc - 1)];
      float Mb = -INFINITY;
#pragma unroll
      for (int u = 0; u < NB; ++u) Mb = fmaxf(Mb, pv[u].x);
      if (Mb > M) {   // a later batch holds a larger maximum: rescale the sums so far
        if (M != -INFINITY) {
          const double d = (double)M - (double)Mb;
          const double f = (double)__expf((float)d);
          U = f * (U + d * S);
          S = f * S;
        }
        M = Mb;
        idx = 0x7FFFFFFF;   // the first maximum lies in this batch or later
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float4 p = pv[u];
        if (c0 + u >= nc || p.x == -INFINITY) continue;
        const double d = (double)p.x - (double)M;
        const double f = p.x == M ? 1.0 : (double)__expf(p.x - M);
        S += f * (double)p.y;
        U += f * ((double)p.z + d * (double)p.y);
        if (p.x == M) idx = min(idx, __float_as_int(p.w));
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
    inf.after_stop = 0;
    reinterpret_cast<cd_step_info*>(a.info)[rr] = inf;
    if (a.rq) {
      a.rq[rr].t = step;
      a.rq[rr].stopped = inf.stop;
    }
  }
}

// Fixed partial buffer of the allocation-free sampler entry point: one per
// GPU, alive until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) float4 scratch[SAMPLER_SCRATCH_PARTIALS];

int sampler_scratch(float4** out) {
  static std::mutex mu;
  static float4* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -4;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -4;
    ptr[dev] = reinterpret_cast<float4*>(p);
  }
  *out = ptr[dev];
  return 0;
}

void launch_sampler_part(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sample_part, dim3(a.n_chunks, a.rows), dim3(256), 0, s, a);
}
void launch_sampler_final(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sample_final, dim3(a.rows / a.C), dim3(256), 0, s, a);
}

}  // namespace cd
