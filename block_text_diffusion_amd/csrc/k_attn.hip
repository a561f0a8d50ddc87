// Canvas attention: softmax(Q K^T / sqrt(dh)) V over the committed KV cache
// plus the canvas itself, with no mask (every canvas token sees every other
// canvas token and the whole committed history: the bidirectional denoising
// pass of the DiffusionGemma pages, canvas explainer step ③); the same kernel
// with a causal mask serves the prompt prefill (step ①).
//
// Work item = (request, KV head, block of 256 query rows, key split).  The
// 256 query rows are the Hq/Hkv query heads that share one KV head times
// 256/(Hq/Hkv) tokens, so every K/V byte feeds all heads of its group.  Each
// of the 8 waves owns 32 query rows (two 16-row tiles); waves w and w+4 share
// a SIMD, and the second half runs half a key block behind the first, so one
// wave's softmax (VALU, exp) overlaps the other's MFMAs.
//  * Keys go in blocks of 64.  The block's K tile and V^T tile are copied
//    from global memory straight into LDS (global_load_lds, 16 bytes a lane),
//    already cut into 1 KB MFMA operand fragments, shared by the 8 waves and
//    prefetched DIST blocks ahead, so the cache is read once per work item
//    and every LDS read is one conflict-free 1 KB wave access.
//  * S^T = K Q^T on MFMA (A = key fragment from LDS, B = query fragment held
//    in registers for the whole loop): a lane ends with keys of one query.
//    The 16 key rows of a K fragment are taken in the order that leaves each
//    lane holding 8 consecutive keys of a 32-key chunk, which is exactly the
//    P^T operand of the next product, so P never leaves registers.
//  * softmax in base 2 against a per-row reference that starts the score
//    accumulators and moves only when a score exceeds it by more than a
//    threshold, so most blocks need neither a cross-lane maximum nor a
//    rescale of O (lazy rescaling); masked keys start at -inf;
//  * O^T += V^T P^T on MFMA; V is cached transposed ([dh][ctx]) so its
//    fragments are contiguous in the key index; on the bf16 path the row sums
//    come from one more MFMA with an all-ones operand.
// With one key split the kernel normalises and writes O itself; otherwise
// each split writes an unnormalised partial (O in the activation type, its
// reference and row sum in fp32) and a merge kernel combines them in fp32.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace cd {

template <int AT>
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t elem) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(base) + elem * (AT == DT_F32 ? 4 : 2));
}

template <int AT, int DH>
struct AttnShape {
  static constexpr int ES = (AT == DT_F32) ? 4 : 2;
  static constexpr int KF = (AT == DT_F32) ? 16 : 32;   // contraction elements per fragment
  static constexpr int KQ = KF / 4;                     // per lane
  static constexpr int NK = DH / KF;                    // K fragments across dh
  static constexpr int ND = DH / 16;                    // 16-wide dh tiles
  static constexpr int VF = (AT == DT_F32) ? 4 : 2;     // V fragments per dh tile and key block
  static constexpr int NFK = 4 * NK, NFV = ND * VF, NF = NFK + NFV;
  static constexpr int NW = 8;                          // waves per workgroup
  static constexpr int QTW = 2;                         // 16-row query tiles per wave
  static constexpr int FPW = NF / NW;                   // fragments each wave copies
  static constexpr int STAGE = NF * 1024;
  static constexpr int NBUF = (STAGE * 4 <= 128 * 1024) ? 4 : 2;
  // staggered halves (below) need a buffer between the one being copied and
  // the one the late half still reads
  static constexpr bool PP = NBUF >= 4;
  static constexpr int DIST = PP ? NBUF - 2 : NBUF - 1;
  static_assert(NF % NW == 0 && NW * QTW * 16 == ATT_QR, "work split");
};

// key held by row i (0..15) of K fragment subtile st (0..3) of a 64-key block:
// subtiles 2c and 2c+1 interleave the 32 keys of chunk c in groups of four
__device__ __forceinline__ int att_key(int st, int i) {
  return 32 * (st >> 1) + 8 * (i >> 2) + 4 * (st & 1) + (i & 3);
}

template <int AT, int DH>
__global__ __launch_bounds__(512) void k_attn(const AttnArgs a) {
  using S = AttnShape<AT, DH>;
  constexpr int KF = S::KF, KQ = S::KQ, NK = S::NK, ND = S::ND, NFK = S::NFK, FPW = S::FPW, QTW = S::QTW;
  constexpr int WR = QTW * 16;                   // query rows per wave
  constexpr int NBUF = S::NBUF, DIST = S::DIST, STAGE = S::STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hkv;
  const int TB = ATT_QR / G;                     // tokens per query block

  // Work items go to the 8 XCDs (the dispatcher deals workgroups to them
  // round-robin) in contiguous runs, query block fastest, so the query blocks
  // that read one key range run back to back on one XCD and the second finds
  // the keys and values in that XCD's L2.  The grid is rounded up to a
  // multiple of 8; surplus workgroups return at once.
  const int work = a.n_req * a.Hkv * a.q_blocks * a.n_split;
  const int w8 = (work + 7) & ~7;
  int bid = (int)(blockIdx.x & 7) * (w8 >> 3) + (int)(blockIdx.x >> 3);
  if (bid >= work) return;
  const int qb = bid % a.q_blocks; bid /= a.q_blocks;
  const int s = bid % a.n_split; bid /= a.n_split;
  const int g = bid % a.Hkv; bid /= a.Hkv;
  const int r = bid;

  const int pos0 = a.pos0[r * a.pos0_stride];
  const int nrows = a.rows_per_req;
  const int nkeys = pos0 + nrows;
  const int hh = (wave * WR) / TB;               // head within group
  const int h = g * G + hh;
  const int tok0 = qb * TB + (wave * WR) % TB;   // first token of this wave

  const int kbeg = s * a.split_len;
  int kend = min(kbeg + a.split_len, nkeys);
  if (a.causal) kend = min(kend, pos0 + min((qb + 1) * TB, nrows));   // last token of the work item
  const int nblk = kend > kbeg ? (kend - kbeg + ATT_KB - 1) / ATT_KB : 0;

  const int ae = S::ES;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.kc) + ((int64_t)r * a.kv_req_stride + (int64_t)g * a.max_ctx * DH) * ae;
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.vc) + ((int64_t)r * a.kv_req_stride + (int64_t)g * DH * a.max_ctx) * ae;
  // last key a copy may start at: K rows up to kend-1; V^T groups of 4 (fp32)
  // or 8 (bf16) keys starting at or below kend-1 (the cache length is a
  // multiple of 64, so such a group stays inside the row)
  constexpr int VG = (AT == DT_F32) ? 4 : 8;
  const int klast = max(kend - 1, 0);
  const int vlast = (klast / VG) * VG;

  // copy of key block b (clamped to the last block) into its LDS buffer
  auto issue = [&](int b) {
    const int bc = min(b, nblk - 1);
    const int kb0 = kbeg + bc * ATT_KB;
    uint8_t* buf = lds + (b % NBUF) * STAGE;
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
      const int f = wave * FPW + i;
      const uint8_t* src;
      if (f < NFK) {
        const int st = f / NK, kk = f % NK;
        const int key = min(kb0 + att_key(st, lane & 15), klast);
        src = kc + ((int64_t)key * DH + kk * KF + (lane >> 4) * KQ) * ae;
      } else {
        const int fv = f - NFK;
        int dt, vk;
        if constexpr (AT == DT_F32) { dt = fv / 4; const int st = fv % 4; vk = kb0 + 32 * (st >> 1) + 8 * (lane >> 4) + 4 * (st & 1); }
        else { dt = fv / 2; const int c = fv % 2; vk = kb0 + 32 * c + 8 * (lane >> 4); }
        vk = min(vk, vlast);
        src = vc + ((int64_t)(dt * 16 + (lane & 15)) * a.max_ctx + vk) * ae;
      }
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_void*)(buf + f * 1024), 16, 0, 0);
    }
  };

  // query fragments, resident for the whole key loop
  const int64_t ld = (int64_t)a.Hq * DH;
  u32x4 qf[QTW][NK];
  int qpos[QTW];
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    const int tok = tok0 + qt * 16 + (lane & 15);
    qpos[qt] = pos0 + tok;
    const int tc = min(tok, nrows - 1);
    const int64_t row = (int64_t)r * nrows + tc;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qf[qt][kk] = ld16<AT>(a.Q, row * ld + h * DH + kk * KF + (lane >> 4) * KQ);
  }

  // The queries arrive multiplied by log2(e) / sqrt(dh) (the QKV epilogue
  // applies it before rounding), so a score s is already the base-2 exponent
  // of its softmax weight.
  // Lazy rescaling.  Scores are taken relative to a per-row reference mref
  // (equal in the four lanes that hold a query's keys), which enters as the
  // initial value of the score accumulators, so the MFMAs return s - mref.
  // The reference moves only when a score of the block exceeds it by more
  // than tau (every p = 2^(s - mref) stays below 2^tau), so a typical block
  // needs no cross-lane maximum and no rescale of O.  O and the row sum l
  // always share the reference, so the result is exact up to rounding for any
  // reference.
  const float tau = a.rescale_log2;
  float mref[QTW];      // -inf until the row has seen a visible key
  f32x4 o[QTW][ND];
  f32x4 lacc[QTW];      // bf16: row sums from an MFMA with a ones operand (all four equal);
                        // f32: this lane's partial sum in [0]
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    mref[qt] = -INFINITY;
    lacc[qt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[qt][dt] = f32x4{0, 0, 0, 0};
  }

  // The work on one key block comes in three phases: scores (MFMA), softmax
  // (VALU), and the O update (MFMA).
  f32x4 sacc[4][QTW];   // S^T[st][qt] - mref: keys of subtile st x query tile qt; then P^T
  u32x4 pf[QTW][2];     // P^T in bf16 (bf16 path)

  // Masked keys (past the end of the range, or after the query under the
  // causal mask) start at -inf, so they leave the MFMA as -inf and exp2 turns
  // them into 0.  Blocks whose keys are all visible to every row of the wave
  // take the unmasked variant.
  auto scores = [&](int b, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint8_t* buf = lds + (b % NBUF) * STAGE + lane * 16;
    const int kb0 = kbeg + b * ATT_KB;
    float base[QTW];
#pragma unroll
    for (int qt = 0; qt < QTW; ++qt) base[qt] = mref[qt] == -INFINITY ? 0.f : -mref[qt];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int qt = 0; qt < QTW; ++qt) {
        if constexpr (MASKED) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kidx = kb0 + 32 * (st >> 1) + 8 * (lane >> 4) + 4 * (st & 1) + q;
            const bool ok = kidx < kend && (!a.causal || kidx <= qpos[qt]);
            sacc[st][qt][q] = ok ? base[qt] : -INFINITY;
          }
        } else {
          sacc[st][qt] = f32x4{base[qt], base[qt], base[qt], base[qt]};
        }
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(buf + (st * NK + kk) * 1024);
#pragma unroll
        for (int qt = 0; qt < QTW; ++qt) {
          if constexpr (AT == DT_F32) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              sacc[st][qt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[j]), __uint_as_float(qf[qt][kk][j]),
                                                                  sacc[st][qt], 0, 0, 0);
          } else {
            sacc[st][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                                   __builtin_bit_cast(bf16x8, qf[qt][kk]), sacc[st][qt], 0, 0, 0);
          }
        }
      }
    }
  };

  // p = 2^(s - mref); lane holds keys kb0 + 32c + 8*(lane/16) + 4*half + q
  auto softmax = [&]() {
#pragma unroll
    for (int qt = 0; qt < QTW; ++qt) {
      float lm = sacc[0][qt][0];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) lm = fmaxf(lm, sacc[st][qt][q]);
      const bool first = mref[qt] == -INFINITY;
      if (__ballot(first || lm > tau)) {
        // move the reference: to the row maximum on a row's first visible
        // keys, else up by the excess of the row maximum over it (if any)
        float rm = fmaxf(lm, __shfl_xor(lm, 16, 64));
        rm = fmaxf(rm, __shfl_xor(rm, 32, 64));
        const float sh = first ? (rm == -INFINITY ? 0.f : rm) : fmaxf(rm, 0.f);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int q = 0; q < 4; ++q) sacc[st][qt][q] -= sh;
        const float alpha = first ? 1.0f : __builtin_amdgcn_exp2f(-sh);
        mref[qt] = first ? (rm == -INFINITY ? -INFINITY : rm) : mref[qt] + sh;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            o[qt][dt][0] *= alpha; o[qt][dt][1] *= alpha; o[qt][dt][2] *= alpha; o[qt][dt][3] *= alpha;
          }
          lacc[qt][0] *= alpha; lacc[qt][1] *= alpha; lacc[qt][2] *= alpha; lacc[qt][3] *= alpha;
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) sacc[st][qt][q] = __builtin_amdgcn_exp2f(sacc[st][qt][q]);   // -inf -> 0
      if constexpr (AT == DT_F32) {
        float sum = 0.f;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int q = 0; q < 4; ++q) sum += sacc[st][qt][q];
        lacc[qt][0] += sum;
      }
    }
    if constexpr (AT != DT_F32) {
#pragma unroll
      for (int qt = 0; qt < QTW; ++qt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pf[qt][c][0] = pack_bf16(sacc[2 * c][qt][0], sacc[2 * c][qt][1]);
          pf[qt][c][1] = pack_bf16(sacc[2 * c][qt][2], sacc[2 * c][qt][3]);
          pf[qt][c][2] = pack_bf16(sacc[2 * c + 1][qt][0], sacc[2 * c + 1][qt][1]);
          pf[qt][c][3] = pack_bf16(sacc[2 * c + 1][qt][2], sacc[2 * c + 1][qt][3]);
        }
    }
  };

  // O^T += V^T P^T; on the bf16 path also l += 1 P^T (the row sums of the
  // bf16 weights that multiply V)
  auto update = [&](int b) {
    const uint8_t* buf = lds + (b % NBUF) * STAGE + lane * 16;
    if constexpr (AT == DT_F32) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const u32x4 vf = *reinterpret_cast<const u32x4*>(buf + (NFK + dt * 4 + st) * 1024);
#pragma unroll
          for (int qt = 0; qt < QTW; ++qt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vf[j]), sacc[st][qt][j], o[qt][dt], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 vf = *reinterpret_cast<const u32x4*>(buf + (NFK + dt * 2 + c) * 1024);
#pragma unroll
          for (int qt = 0; qt < QTW; ++qt)
            o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf),
                                                                __builtin_bit_cast(bf16x8, pf[qt][c]), o[qt][dt], 0, 0, 0);
        }
      const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
      for (int qt = 0; qt < QTW; ++qt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones),
                                                             __builtin_bit_cast(bf16x8, pf[qt][c]), lacc[qt], 0, 0, 0);
    }
  };

  // scores and softmax of block b, masked only where needed
  // The MFMA phases run at a raised wave priority: when the other wave on
  // the SIMD is in its softmax, the MFMA pipe is fed first and the VALU work
  // fills the gaps.
  auto scores_softmax = [&](int b) {
    const int kb0 = kbeg + b * ATT_KB;
    const bool full = kb0 + ATT_KB <= kend && (!a.causal || kb0 + ATT_KB - 1 <= pos0 + tok0);
    __builtin_amdgcn_s_setprio(1);
    if (full) scores(b, std::integral_constant<bool, false>{});
    else scores(b, std::integral_constant<bool, true>{});
    __builtin_amdgcn_s_setprio(0);
    softmax();
  };
  auto update_p = [&](int b) {
    __builtin_amdgcn_s_setprio(1);
    update(b);
    __builtin_amdgcn_s_setprio(0);
  };

  // Block b has landed for this wave; after the barrier it has for every
  // wave, and no wave still reads the buffer that block b + DIST goes into.
  auto sync_issue = [&](int b) {
    wait_vmcnt<(DIST - 1) * FPW>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(b + DIST);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nblk > 0) {
#pragma unroll
    for (int j = 0; j < DIST; ++j) issue(j);
    if (!S::PP || wave < S::NW / 2) {
      for (int b = 0; b < nblk; ++b) {
        sync_issue(b);
        scores_softmax(b);
        update_p(b);
      }
    } else {
      // The second half of the waves runs half a block behind: it meets
      // barrier b after the softmax of block b-1 and updates O with that
      // block after the barrier.  Each SIMD holds one wave of each half, so
      // one wave's softmax runs under the other's MFMAs.  The copy issued at
      // barrier b overwrites block b-2's buffer, which the late waves left
      // before barrier b.
      sync_issue(0);
      scores_softmax(0);
      for (int b = 1; b < nblk; ++b) {
        sync_issue(b);
        update_p(b - 1);
        scores_softmax(b);
      }
      update_p(nblk - 1);
    }
  }
  // the row sum and the reference (base 2) for the merge
  float l[QTW], m[QTW];
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    float sum = lacc[qt][0];
    if constexpr (AT == DT_F32) {
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
    }
    l[qt] = sum;
    m[qt] = mref[qt];
  }
  wait_vmcnt<0>();   // no copy into LDS may be in flight when the workgroup exits

  // O^T lane holds d = dt*16 + 4*(lane/16) + q of query lane%16
  const int64_t rows_total = (int64_t)a.n_req * nrows;
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    const int tok = tok0 + qt * 16 + (lane & 15);
    if (tok >= nrows) continue;
    const int64_t row = (int64_t)r * nrows + tok;
    if (a.n_split == 1) {
      const float inv = 1.0f / l[qt];
      const int64_t ob = row * ld + (int64_t)h * DH + (lane >> 4) * 4;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const float v0 = o[qt][dt][0] * inv, v1 = o[qt][dt][1] * inv, v2 = o[qt][dt][2] * inv, v3 = o[qt][dt][3] * inv;
        if constexpr (AT == DT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.O) + ob + dt * 16) = make_float4(v0, v1, v2, v3);
        } else {
          uint2 pk;
          pk.x = pack_bf16(v0, v1);
          pk.y = pack_bf16(v2, v3);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.O) + ob + dt * 16) = pk;
        }
      }
      continue;
    }
    const int64_t base = (((int64_t)s * rows_total + row) * a.Hq + h);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int64_t e = base * DH + dt * 16 + (lane >> 4) * 4;
      if constexpr (AT == DT_F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.part_o) + e) =
            make_float4(o[qt][dt][0], o[qt][dt][1], o[qt][dt][2], o[qt][dt][3]);
      } else {   // the partials of the bf16 path are kept in bf16 as well
        uint2 pk;
        pk.x = pack_bf16(o[qt][dt][0], o[qt][dt][1]);
        pk.y = pack_bf16(o[qt][dt][2], o[qt][dt][3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.part_o) + e) = pk;
      }
    }
    if ((lane >> 4) == 0) {
      a.part_ml[base * 2] = m[qt];
      a.part_ml[base * 2 + 1] = l[qt];
    }
  }
}

// combine key splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (row, head, 4 dims); every split's partial is loaded before
// any is used, so the loads overlap instead of queueing one split at a time.
template <int AT>
__global__ __launch_bounds__(256) void k_attn_merge(const AttnArgs a, int dh) {
  constexpr int MS = ATT_MAX_SPLIT;
  const int64_t rows_total = (int64_t)a.n_req * a.rows_per_req;
  const int quads = a.Hq * dh / 4;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= rows_total * quads) return;
  const int64_t row = t / quads;
  const int idx = (int)(t % quads) * 4;
  const int h = idx / dh, d = idx % dh;
  float ms[MS], ls[MS];
  float4 os[MS];
  // no load is conditional: splits past n_split re-read the last one (their
  // values are then dropped), so all of them are in flight at once
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const int64_t base = ((int64_t)min(s, a.n_split - 1) * rows_total + row) * a.Hq + h;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + base * 2);
    float4 ov;
    if constexpr (AT == DT_F32) {
      ov = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.part_o) + base * dh + d);
    } else {
      const uint2 pk = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.part_o) + base * dh + d);
      ov = make_float4(bf2f(pk.x & 0xFFFF), bf2f(pk.x >> 16), bf2f(pk.y & 0xFFFF), bf2f(pk.y >> 16));
    }
    const bool live = s < a.n_split;
    ms[s] = live ? ml.x : -INFINITY;
    ls[s] = live ? ml.y : 0.f;
    os[s] = live ? ov : make_float4(0, 0, 0, 0);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) M = fmaxf(M, ms[s]);
  float L = 0.f;
  float4 acc = make_float4(0, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (ms[s] == -INFINITY) continue;
    const float w = exp2f(ms[s] - M);
    L += w * ls[s];
    acc.x += w * os[s].x; acc.y += w * os[s].y; acc.z += w * os[s].z; acc.w += w * os[s].w;
  }
  const float inv = 1.0f / L;
  const int64_t o = row * (int64_t)a.Hq * dh + idx;
  if constexpr (AT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.O) + o) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 p;
    p.x = pack_bf16(acc.x * inv, acc.y * inv);
    p.y = pack_bf16(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.O) + o) = p;
  }
}

void launch_attention(int adt, const AttnArgs& a, hipStream_t s) {
  const int blocks = (a.n_req * a.Hkv * a.q_blocks * a.n_split + 7) & ~7;
  if (adt == DT_F32) {
    if (a.dh == 64) hipLaunchKernelGGL((k_attn<DT_F32, 64>), dim3(blocks), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_attn<DT_F32, 128>), dim3(blocks), dim3(512), 0, s, a);
  } else {
    if (a.dh == 64) hipLaunchKernelGGL((k_attn<DT_BF16, 64>), dim3(blocks), dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_attn<DT_BF16, 128>), dim3(blocks), dim3(512), 0, s, a);
  }
}

void launch_attn_merge(int adt, const AttnArgs& a, hipStream_t s) {
  if (a.n_split <= 1) return;   // the attention kernel wrote O itself
  const int64_t threads = (int64_t)a.n_req * a.rows_per_req * (a.Hq * a.dh / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (adt == DT_F32) hipLaunchKernelGGL(k_attn_merge<DT_F32>, grid, dim3(256), 0, s, a, a.dh);
  else hipLaunchKernelGGL(k_attn_merge<DT_BF16>, grid, dim3(256), 0, s, a, a.dh);
}

}  // namespace cd
