// libcd host runtime: buffer plan, argument/state validation, and the
// orchestration of the canvas denoise step, block commit and generation loop
// on one HIP stream.  The library never allocates device memory: weights and
// state live in two caller buffers carved up by Plan.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/cd.h"
#include "kernels.h"

using namespace cd;

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t hip_status(const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CD_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return CD_OK;
}

constexpr int64_t ALIGN = 256;
constexpr int GROUPED_MT = 2;          // expert GEMM row tile = 32 rows (few rows per expert)
constexpr int BIG_TILE_ROWS = 256;     // expert row tile of the LDS-staged kernel (many rows per expert)

// Many rows per expert (batched canvases, prefill): 256-row expert tiles on
// the LDS-staged kernels, which reuse every weight byte for all rows of a
// work item (256, or 128 for fp8 weights and the fp8-activation kernel, whose
// work items are the two halves of a tile).
bool big_expert_tiles(int64_t assignments, int E) { return assignments >= (int64_t)BIG_TILE_ROWS * E; }
constexpr int MAX_SPLIT = ATT_MAX_SPLIT;   // attention key splits
constexpr int MAX_RSPLIT = MAX_ROUTER_SPLIT;         // router contraction splits

struct Carve {
  int64_t off = 0;
  int64_t take(int64_t bytes) {
    int64_t o = off;
    off = round_up(off + std::max<int64_t>(bytes, 1), ALIGN);
    return o;
  }
};

struct LayerOff {
  int64_t qkv, qkv_s, wo, wo_s, wr, gu, gu_s, dn, dn_s, sgu, sdn;
};

struct Plan {
  cd_config c;
  int wdt_attn, wdt_exp, wdt_other, adt;
  int ctx;                 // KV capacity rounded to 64
  int Tmax;                // rows of the largest forward
  int qkv_npad, wo_npad, wr_npad, gu_npad, dn_npad, sgu_npad, sdn_npad, lm_npad;
  int64_t gu_stride, dn_stride;        // bytes per expert
  int64_t gu_mx, dn_mx;                // MXFP4: offset of an expert's scales in its stride
  // weights
  int64_t embed, lm;
  std::vector<LayerOff> layer;
  int64_t weights_bytes;
  // state
  int64_t rq, canvas, argmax, lock, entropy, pmax, info, h, u, q, o, part_o, part_ml, rlog, topk_id,
      topk_gate, blk_cnt, seg_off, row_map, slot, tiles, n_tiles, aperm, yperm, sact, sout, logits, spart, rope,
      kcache, vcache, zero;
  // fp8 activations of the W8A8 path (fp8 attention weights and forwards of
  // more than 256 rows): E4M3 rows with one fp32 scale per row
  bool x8;
  int64_t xq, xqs, aq, aqs;
  int x8_ld;
  int64_t max_rows, max_tiles, n_blk_max, n_chunks;
  int64_t kv_req_stride, kv_layer_stride;   // elements
  int64_t state_bytes;
};

int32_t validate_config(const cd_config* c) {
  if (!c) return fail(CD_ERR_INVALID_ARG, "null config");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->n_experts < 1 || c->top_k < 1 || c->expert_hidden < 1 || c->shared_hidden < 0 || c->vocab < 1 ||
      c->canvas_len < 1 || c->max_steps < 1 || c->max_requests < 1 || c->max_ctx < 1 || c->max_prefill < 1)
    return fail(CD_ERR_INVALID_ARG, "config fields must be positive");
  if (c->weight_dtype < CD_F32 || c->weight_dtype > CD_MXFP4) return fail(CD_ERR_INVALID_ARG, "bad weight_dtype");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(CD_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads) return fail(CD_ERR_INVALID_ARG, "n_q_heads %% n_kv_heads != 0");
  if (c->n_q_heads / c->n_kv_heads > 4 || c->n_q_heads / c->n_kv_heads == 3)
    return fail(CD_ERR_UNSUPPORTED, "1, 2 or 4 query heads per KV head");
  if (c->d_model % 64 || c->expert_hidden % 64 || c->shared_hidden % 64 || (c->n_q_heads * c->head_dim) % 64)
    return fail(CD_ERR_UNSUPPORTED, "d_model, expert_hidden, shared_hidden, n_q_heads*head_dim must be multiples of 64");
  if (c->n_experts > 256 || c->top_k > 16 || c->top_k > c->n_experts)
    return fail(CD_ERR_UNSUPPORTED, "n_experts <= 256 and top_k <= min(16, n_experts) required");
  if (c->vocab % 128) return fail(CD_ERR_UNSUPPORTED, "vocab must be a multiple of 128");
  if (c->max_ctx < c->canvas_len + 1) return fail(CD_ERR_INVALID_ARG, "max_ctx must exceed canvas_len");
  if (c->max_requests > 256) return fail(CD_ERR_UNSUPPORTED, "max_requests <= 256");
  if (!(c->lock_threshold >= 0.f && c->lock_threshold <= 1.f) || !(c->stop_entropy >= 0.f) || !(c->rms_eps >= 0.f) ||
      !(c->rope_theta >= 0.f))
    return fail(CD_ERR_INVALID_ARG, "bad sampler/norm constants");
  if (!(c->attn_rescale_log2 >= 0.f && c->attn_rescale_log2 <= 64.f))
    return fail(CD_ERR_INVALID_ARG, "attn_rescale_log2 must lie in [0, 64]");
  if ((c->lock_rule != CD_LOCK_MAXPROB && c->lock_rule != CD_LOCK_ENTROPY) ||
      !(c->entropy_bound >= 0.f && c->entropy_bound < INFINITY))
    return fail(CD_ERR_INVALID_ARG, "bad lock rule or entropy bound");
  return CD_OK;
}

int sampler_chunks(int V) {
  int n = 1;
  while (V / n > 8192 && (V % (2 * n * 4)) == 0) n *= 2;   // chunks of at most 8192 logits
  return n;
}

// expert row tile of the register-path grouped GEMM, in 16-row tiles: 32
// rows; 16 for MXFP4, whose 4-bit weight bytes are no more than the
// activation bytes a tile stages, so padding rows cost as much as weights
int grouped_mt(const Plan& p) { return p.wdt_exp == CD_MXFP4 ? 1 : GROUPED_MT; }

Plan make_plan(const cd_config& c) {
  Plan p;
  p.c = c;
  // CD_FP8: attention and experts fp8; CD_MXFP4: attention fp8, experts
  // MXFP4; everything else bf16 in both
  const bool narrow = c.weight_dtype == CD_FP8 || c.weight_dtype == CD_MXFP4;
  p.wdt_attn = narrow ? CD_FP8 : c.weight_dtype;
  p.wdt_exp = c.weight_dtype;
  p.wdt_other = narrow ? CD_BF16 : c.weight_dtype;
  p.adt = c.weight_dtype == CD_F32 ? CD_F32 : CD_BF16;
  p.ctx = (int)round_up(c.max_ctx, 64);
  const int C = c.canvas_len, d = c.d_model, dh = c.head_dim, L = c.n_layers, E = c.n_experts;
  p.Tmax = std::max(c.max_requests * C, c.max_prefill);
  p.qkv_npad = (int)round_up((c.n_q_heads + 2 * c.n_kv_heads) * dh, 32);
  p.wo_npad = (int)round_up(d, 32);
  p.wr_npad = (int)round_up(E, 32);
  p.gu_npad = 2 * c.expert_hidden;
  p.dn_npad = (int)round_up(d, 32);
  p.sgu_npad = 2 * c.shared_hidden;
  p.sdn_npad = (int)round_up(d, 32);
  p.lm_npad = (int)round_up(c.vocab, 32);
  const bool f8 = p.wdt_attn == CD_FP8, f8e = p.wdt_exp == CD_FP8;
  // an expert's stride holds its packed tiles and, for MXFP4, their scales
  p.gu_stride = round_up(packed_total(p.gu_npad, d, p.wdt_exp), ALIGN);
  p.dn_stride = round_up(packed_total(p.dn_npad, c.expert_hidden, p.wdt_exp), ALIGN);
  p.gu_mx = packed_bytes(p.gu_npad, d, p.wdt_exp);
  p.dn_mx = packed_bytes(p.dn_npad, c.expert_hidden, p.wdt_exp);

  Carve w;
  p.embed = w.take((int64_t)c.vocab * d * esize(p.wdt_other));
  p.lm = w.take(packed_bytes(p.lm_npad, d, p.wdt_other));
  p.layer.resize(L);
  for (int l = 0; l < L; ++l) {
    LayerOff& o = p.layer[l];
    o.qkv = w.take(packed_bytes(p.qkv_npad, d, p.wdt_attn));
    o.qkv_s = f8 ? w.take(p.qkv_npad * 4) : -1;
    o.wo = w.take(packed_bytes(p.wo_npad, (int64_t)c.n_q_heads * dh, p.wdt_attn));
    o.wo_s = f8 ? w.take(p.wo_npad * 4) : -1;
    o.wr = w.take(packed_bytes(p.wr_npad, d, p.wdt_other));
    o.gu = w.take(p.gu_stride * E);
    o.gu_s = f8e ? w.take((int64_t)p.gu_npad * 4 * E) : -1;
    o.dn = w.take(p.dn_stride * E);
    o.dn_s = f8e ? w.take((int64_t)p.dn_npad * 4 * E) : -1;
    o.sgu = c.shared_hidden ? w.take(packed_bytes(p.sgu_npad, d, p.wdt_other)) : -1;
    o.sdn = c.shared_hidden ? w.take(packed_bytes(p.sdn_npad, c.shared_hidden, p.wdt_other)) : -1;
  }
  p.weights_bytes = w.off;

  const int R = c.max_requests, T = p.Tmax, k = c.top_k, ae = esize(p.adt);
  const int mrows = 16 * grouped_mt(p);
  // expert segments are padded to the row tile: size for the larger tile
  // when the largest forward can take it
  const int pad_rows = big_expert_tiles((int64_t)T * k, E) ? BIG_TILE_ROWS : mrows;
  p.max_rows = round_up((int64_t)T * k + (int64_t)E * pad_rows, 64);
  p.max_tiles = ((int64_t)T * k + mrows - 1) / mrows + E;
  p.n_blk_max = ((int64_t)T * k + 511) / 512;
  p.n_chunks = sampler_chunks(c.vocab);
  p.kv_layer_stride = (int64_t)c.n_kv_heads * p.ctx * dh;
  p.kv_req_stride = p.kv_layer_stride * L;

  Carve s;
  p.zero = s.take(256);
  p.rq = s.take(sizeof(ReqDev) * R);
  p.canvas = s.take(4LL * R * C);
  p.argmax = s.take(4LL * R * C);
  p.lock = s.take(1LL * R * C);
  p.entropy = s.take(8LL * R * C);
  p.pmax = s.take(8LL * R * C);
  p.info = s.take(sizeof(cd_step_info) * R);
  p.h = s.take(4LL * T * d);
  p.u = s.take((int64_t)ae * T * d);
  p.q = s.take((int64_t)ae * T * c.n_q_heads * dh);
  p.o = s.take((int64_t)ae * T * c.n_q_heads * dh);
  p.part_o = s.take(4LL * MAX_SPLIT * T * c.n_q_heads * dh);
  p.part_ml = s.take(8LL * MAX_SPLIT * T * c.n_q_heads);
  p.rlog = s.take(4LL * MAX_RSPLIT * T * E);
  p.topk_id = s.take(4LL * T * k);
  p.topk_gate = s.take(4LL * T * k);
  p.blk_cnt = s.take(4LL * p.n_blk_max * E);
  p.seg_off = s.take(4LL * (E + 1));
  p.row_map = s.take(4LL * p.max_rows);
  p.slot = s.take(4LL * T * k);
  p.tiles = s.take(16LL * p.max_tiles);
  p.n_tiles = s.take(4);
  p.aperm = s.take((int64_t)ae * p.max_rows * c.expert_hidden);
  p.yperm = s.take((int64_t)ae * p.max_rows * d);
  p.sact = s.take((int64_t)ae * T * std::max(c.shared_hidden, 1));
  p.sout = s.take(4LL * T * (c.shared_hidden ? d : 1));
  p.logits = s.take(4LL * R * C * c.vocab);
  p.spart = s.take(16LL * R * C * p.n_chunks);
  p.rope = s.take(8LL * p.ctx * (dh / 2));
  p.kcache = s.take((int64_t)ae * p.kv_req_stride * R);
  p.vcache = s.take((int64_t)ae * p.kv_req_stride * R);
  // W8A8 needs fp8 attention weights, a forward that takes the LDS-staged
  // kernel (more than 256 rows) and contraction widths the quantiser holds
  const int qd = c.n_q_heads * dh;
  p.x8 = p.wdt_attn == CD_FP8 && T > 256 && std::max(d, qd) <= 4096 && c.expert_hidden <= 4096 &&
         qd % 64 == 0;
  p.x8_ld = std::max(d, qd);
  p.xq = p.x8 ? s.take((int64_t)T * p.x8_ld) : -1;
  p.xqs = p.x8 ? s.take(4LL * T) : -1;
  p.aq = p.x8 ? s.take(p.max_rows * (int64_t)c.expert_hidden) : -1;
  p.aqs = p.x8 ? s.take(4LL * p.max_rows) : -1;
  p.state_bytes = s.off;
  return p;
}

struct HostReq {
  int P = 0, t = 0, block = 0;
  int rid = -1;   // Philox request index once set (a moved or served request keeps its own), else the slot
  bool active = false;
  uint64_t seed = 0;
};

}  // namespace

struct ProfRec {
  int cls;
  hipEvent_t a, b;
};

struct cd_ctx {
  Plan p;
  uint8_t* W;
  uint8_t* S;
  std::vector<HostReq> req;
  bool prof = false;
  std::vector<ProfRec> recs;          // recorded this window
  std::vector<hipEvent_t> pool;       // reusable events
  size_t pool_used = 0;
  float* trace_h = nullptr;
  float* trace_hmid = nullptr;
  int32_t* trace_ids = nullptr;
  float* trace_gates = nullptr;
  // a second stream (default priority) of the library's own: above 256 rows,
  // and in captured passes, the shared FFN runs there while the router,
  // routing and expert GEMMs run on the caller's stream; the two join before
  // the combine, inside the same call.  Created on first use; if that fails
  // the shared FFN runs on the caller's stream.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool side_tried = false;
  // first refusal of a kernel launcher during the current call (0 = none)
  int32_t launch_err = 0;
  // Denoise passes replayed as HIP graphs.  A pass's launches depend on the
  // host only through (first slot, number of slots, longest context, active
  // slots): every other argument is a fixed address in the two buffers or a
  // constant of the plan, and the per-request state is read on the device.
  // One captured graph therefore serves every pass with the same four values
  // (all the passes of a block).  Captured on a stream of the library's own,
  // launched on the caller's.
  struct PassGraph {
    int r0, n_req, nkeys;
    uint64_t act[4];
    hipGraphExec_t exec;
    uint64_t used;
  };
  bool graphs = true;
  bool capturing = false;   // a pass is being captured on cap
  hipStream_t cap = nullptr;
  std::vector<PassGraph> pass_graphs;
  uint64_t graph_clock = 0;
  template <class T> T* st(int64_t off) const { return reinterpret_cast<T*>(S + off); }
  template <class T> T* wt(int64_t off) const { return off < 0 ? nullptr : reinterpret_cast<T*>(W + off); }
};

namespace {

hipStream_t strm(void* s) { return reinterpret_cast<hipStream_t>(s); }

hipEvent_t pool_event(cd_ctx* c) {
  if (c->pool_used == c->pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->pool.push_back(e);
  }
  return c->pool[c->pool_used++];
}

bool ensure_side(cd_ctx* c) {
  if (!c->side_tried) {
    c->side_tried = true;
    if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess) c->side = nullptr;
    if (c->side && (hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
                    hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess)) {
      hipStreamDestroy(c->side);
      c->side = nullptr;
    }
    (void)hipGetLastError();
  }
  return c->side != nullptr;
}

// Records events around one launch when profiling is on.
struct Prof {
  cd_ctx* c;
  int cls;
  hipStream_t s;
  hipEvent_t b = nullptr;
  Prof(cd_ctx* c_, int cls_, hipStream_t s_) : c(c_), cls(cls_), s(s_) {
    if (c->prof) {
      hipEvent_t a = pool_event(c);
      b = pool_event(c);
      if (a && b) {
        hipEventRecord(a, s);
        c->recs.push_back({cls, a, b});
      } else {
        b = nullptr;
      }
    }
  }
  ~Prof() {
    if (b) hipEventRecord(b, s);
  }
};
#define PROF(cls) Prof prof_guard_##__LINE__(c, cls, s)

// ---- GEMM dispatch ---------------------------------------------------------------
struct GemmCall {
  int wdt, epi, mt;
  GemmArgs a;
};

GemmArgs gemm_base(const void* X, int64_t ldx, const uint8_t* W, const float* wscale, int K, int Npad, int N,
                   void* Y, int64_t ldy) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.X = X; a.ldx = ldx; a.W = W; a.wscale = wscale; a.K = K;
  a.Nt = Npad / 16; a.N = N; a.n_chunks = (a.Nt + 7) / 8;
  a.Y = Y; a.ldy = ldy;
  return a;
}

// contraction split of the router GEMM: enough k-splits that the launch has
// about 128 workgroups, at least 8 k-tiles each
int router_split(const cd_config& g, int T) {
  const int kt = g.d_model / (g.weight_dtype == CD_F32 ? 16 : 32);
  const int tiles = (T + 63) / 64;
  int sp = 1;
  while (sp < MAX_RSPLIT && tiles * sp * 2 <= 128 && kt / (sp * 2) >= 8) sp *= 2;
  return sp;
}

void note_launch(cd_ctx* c, int st) {
  if (st && !c->launch_err) c->launch_err = st;
}

// Dense GEMM.  The LM head (thousands of 128-column chunks) at up to 256
// rows takes the LDS-staged kernel: one workgroup per chunk holds all rows,
// so the activations are read once per chunk.  Every other layer takes the
// row-tiled kernel: at the canvas batch, 32-row tiles give each weight chunk
// 8 workgroups on one XCD (one HBM read, the rest from its L2) and fill the
// chip without splitting the contraction.  Larger batches take the
// LDS-staged kernel when there are enough (256-row slab, 256-column chunk)
// items to fill the chip; the expert-combining epilogue gathers 8 rows per
// output and keeps the many workgroups of the row-tiled kernel.
bool dense_lds_staged(int M, int64_t Nt, int ksplit) {
  const int64_t x_items = (int64_t)((M + 255) / 256) * ((Nt + 15) / 16);
  return ksplit <= 1 && ((M > 256 && x_items >= 256) || (Nt + 7) / 8 >= 512);
}
// Whether a dense launch (as gemm_dense decides) or a grouped expert launch (as
// gemm_grouped decides) runs W8A8 on E4M3 activation rows; the forward asks
// before the launch so that the kernel producing those rows also writes them
// in E4M3.
bool dense_takes_x8(const cd_ctx* c, int wdt, int epi, int64_t Nt, int M, int ksplit, bool w8a8) {
  return dense_lds_staged(M, Nt, ksplit) && w8a8 && wdt == CD_FP8 && c->p.x8 && epi != EPI_F32;
}
bool grouped_takes_x8(const cd_ctx* c, int wdt, int64_t rows) {
  return big_expert_tiles(rows, c->p.c.n_experts) && (wdt == CD_FP8 || wdt == CD_MXFP4) && c->p.x8;
}

// w8a8: the launch may quantise its activations to E4M3 (fp8 weights on the
// LDS-staged kernel).  The QKV projection takes it; the output projection
// keeps bf16 activations, since its output feeds the router directly and the
// activation rounding moved near-tie routing decisions too far.
// quantised: the activation rows are already in the E4M3 buffer (written by
// the kernel that produced them), so the W8A8 path skips its quantiser.
void gemm_dense(cd_ctx* c, int wdt, int epi, GemmArgs a, int M, hipStream_t s, bool w8a8 = false,
                bool quantised = false) {
  if (dense_lds_staged(M, a.Nt, a.ksplit)) {
    a.M = M;
    a.tiles = nullptr;
    if (dense_takes_x8(c, wdt, epi, a.Nt, M, a.ksplit, w8a8)) {
      // W8A8: the activation rows quantised to E4M3 with a scale per row
      uint8_t* xq = c->st<uint8_t>(c->p.xq);
      float* xqs = c->st<float>(c->p.xqs);
      if (!quantised) {
        PROF(CD_PROF_QUANT);
        note_launch(c, launch_quant_fp8(a.X, a.ldx, M, a.K, xq, a.K, xqs, nullptr, s));
      }
      a.X = xq; a.ldx = a.K; a.xscale = xqs;
      note_launch(c, launch_gemm_x8(wdt, epi, a, s));
      return;
    }
    note_launch(c, launch_gemm_x(wdt, c->p.adt, epi, a, s));
    return;
  }
  const int mt = M > 256 ? 4 : (M > 16 ? 2 : 1);
  a.M = M;
  a.max_tiles = (M + 16 * mt - 1) / (16 * mt);
  a.chunk_major = 1;
  a.tiles = nullptr;
  note_launch(c, launch_gemm(wdt, c->p.adt, mt, epi, a, s));
}

// rows: assignments of this forward (T * top_k); the grid is sized for the
// most tiles they can form, so idle workgroups stay few
// x_rows: rows of X (the tokens for gate/up, the permuted rows for down);
// x_rows_dev: their device count (down: the padded segments' end) or null
void gemm_grouped(cd_ctx* c, int wdt, int epi, GemmArgs a, int64_t rows, int x_rows, const int32_t* x_rows_dev,
                  hipStream_t s, bool quantised = false) {
  a.tiles = c->st<int32_t>(c->p.tiles);
  a.n_tiles = c->st<int32_t>(c->p.n_tiles);
  if (big_expert_tiles(rows, c->p.c.n_experts)) {
    a.max_tiles = (int)std::min<int64_t>(c->p.max_tiles, (rows + BIG_TILE_ROWS - 1) / BIG_TILE_ROWS +
                                                            std::min<int64_t>(rows, c->p.c.n_experts));
    if (grouped_takes_x8(c, wdt, rows)) {
      // W8A8 (see gemm_dense), or MXFP4 weights x E4M3 activations on the
      // block-scaled MFMA; the down projection's input has its own buffer
      const bool down = epi == EPI_ROWS;
      uint8_t* xq = c->st<uint8_t>(down ? c->p.aq : c->p.xq);
      float* xqs = c->st<float>(down ? c->p.aqs : c->p.xqs);
      if (!(quantised && !down)) {
        PROF(CD_PROF_QUANT);
        note_launch(c, launch_quant_fp8(a.X, a.ldx, x_rows, a.K, xq, a.K, xqs, x_rows_dev, s));
      }
      a.X = xq; a.ldx = a.K; a.xscale = xqs;
      note_launch(c, launch_gemm_x8(wdt, epi, a, s));
      return;
    }
    note_launch(c, launch_gemm_x(wdt, c->p.adt, epi, a, s));
    return;
  }
  const int mt = grouped_mt(c->p), mrows = 16 * mt;
  a.max_tiles = (int)std::min<int64_t>(c->p.max_tiles, (rows + mrows - 1) / mrows + std::min<int64_t>(rows, c->p.c.n_experts));
  a.chunk_major = 0;
  note_launch(c, launch_gemm(wdt, c->p.adt, mt, epi, a, s));
}

// ---- forward over rows of requests r0..r0+n_req-1 --------------------------------------
// ids: rows_per_req ids per request; positions P_r + i; causal: prefill mask.
void forward(cd_ctx* c, int r0, int n_req, int rows_per_req, const int32_t* ids, bool causal, bool head,
             bool trace, hipStream_t s) {
  const Plan& p = c->p;
  const cd_config& g = p.c;
  const int T = n_req * rows_per_req;
  const int d = g.d_model, dh = g.head_dim, E = g.n_experts, k = g.top_k;
  const int qd = g.n_q_heads * dh;
  const int adt = p.adt, ae = esize(adt);
  float* h = c->st<float>(p.h);
  void* u = c->st<void>(p.u);
  void* Q = c->st<void>(p.q);
  void* O = c->st<void>(p.o);
  ReqDev* rq = c->st<ReqDev>(p.rq) + r0;
  const int32_t* pos0 = &rq->P;
  const int pos_stride = (int)(sizeof(ReqDev) / 4);
  const float* rope = g.rope_theta > 0 ? c->st<float>(p.rope) : nullptr;

  int nkeys_max = 0;
  for (int r = r0; r < r0 + n_req; ++r) nkeys_max = std::max(nkeys_max, c->req[r].P + rows_per_req);
  const int G = g.n_q_heads / g.n_kv_heads;
  const int TB = ATT_QR / G;
  AttnArgs at;
  memset(&at, 0, sizeof at);
  at.Q = Q; at.O = O;
  at.kv_req_stride = p.kv_req_stride;
  at.max_ctx = p.ctx; at.Hq = g.n_q_heads; at.Hkv = g.n_kv_heads; at.dh = dh;
  at.rows_per_req = rows_per_req; at.n_req = n_req;
  at.pos0 = pos0; at.pos0_stride = pos_stride;
  at.causal = causal ? 1 : 0;
  at.rescale_log2 = g.attn_rescale_log2 > 0.f ? g.attn_rescale_log2 : 8.0f;
  at.q_blocks = (rows_per_req + TB - 1) / TB;
  // key splits: enough work items for one per CU, each split at least two
  // 64-key blocks
  const int base_wg = n_req * g.n_kv_heads * at.q_blocks;
  int ns = std::max(1, (256 + base_wg - 1) / base_wg);
  ns = std::min(ns, MAX_SPLIT);
  ns = std::min(ns, std::max(1, (nkeys_max + 2 * ATT_KB - 1) / (2 * ATT_KB)));
  at.split_len = (int)round_up((nkeys_max + ns - 1) / ns, ATT_KB);
  at.n_split = (nkeys_max + at.split_len - 1) / at.split_len;
  at.part_o = c->st<void>(p.part_o);
  at.part_ml = c->st<float>(p.part_ml);

  { PROF(CD_PROF_EMBED); launch_embed(p.wdt_other, c->W + p.embed, ids, T, g.vocab, d, h, s); }
  // When the QKV projection or the routed experts run W8A8, the kernel that
  // writes their input u (the RMSNorm, or the combine for the next layer)
  // also writes its E4M3 rows and scales into the activation buffer they read.
  const bool qkv8 = dense_takes_x8(c, p.wdt_attn, EPI_QKV, p.qkv_npad / 16, T, 1, true);
  const bool gu8 = grouped_takes_x8(c, p.wdt_exp, (int64_t)T * k);
  uint8_t* xq = p.x8 ? c->st<uint8_t>(p.xq) : nullptr;
  float* xqs = p.x8 ? c->st<float>(p.xqs) : nullptr;
  // u holds RMSNorm(h) once a combine has written it for the next consumer
  bool u_ready = false;
  for (int l = 0; l < g.n_layers; ++l) {
    const LayerOff& lw = p.layer[l];
    if (trace && c->trace_h) launch_copy_f32(h, c->trace_h + (int64_t)l * T * d, (int64_t)T * d, s);
    if (!u_ready) {
      PROF(CD_PROF_RMSNORM);
      launch_rmsnorm(adt, h, T, d, g.rms_eps, u, s, qkv8 ? xq : nullptr, xqs);
    }
    u_ready = false;
    // QKV + rotary, K/V scattered into the cache at positions P_r + i
    {
      GemmArgs a = gemm_base(u, d, c->W + lw.qkv, c->wt<float>(lw.qkv_s), d, p.qkv_npad,
                             (g.n_q_heads + 2 * g.n_kv_heads) * dh, Q, qd);
      uint8_t* kc = c->S + p.kcache + ((int64_t)r0 * p.kv_req_stride + l * p.kv_layer_stride) * ae;
      uint8_t* vc = c->S + p.vcache + ((int64_t)r0 * p.kv_req_stride + l * p.kv_layer_stride) * ae;
      a.kc = kc; a.vc = vc; a.kv_req_stride = p.kv_req_stride;
      a.max_ctx = p.ctx; a.Hq = g.n_q_heads; a.Hkv = g.n_kv_heads; a.dh = dh;
      a.rows_per_req = rows_per_req; a.pos0 = pos0; a.pos0_stride = pos_stride; a.rope_cs = rope;
      a.q_scale = (float)(1.4426950408889634 / std::sqrt((double)dh));   // log2(e) / sqrt(dh)
      { PROF(CD_PROF_QKV); gemm_dense(c, p.wdt_attn, EPI_QKV, a, T, s, true, qkv8); }
      at.kc = kc; at.vc = vc;
    }
    { PROF(CD_PROF_ATTN); launch_attention(adt, at, s); }
    { PROF(CD_PROF_ATTN_MERGE); launch_attn_merge(adt, at, s); }
    {
      GemmArgs a = gemm_base(O, qd, c->W + lw.wo, c->wt<float>(lw.wo_s), qd, p.wo_npad, d, h, d);
      PROF(CD_PROF_O_PROJ);
      gemm_dense(c, p.wdt_attn, EPI_RESID, a, T, s);
    }
    if (trace && c->trace_hmid) launch_copy_f32(h, c->trace_hmid + (int64_t)l * T * d, (int64_t)T * d, s);
    { PROF(CD_PROF_RMSNORM); launch_rmsnorm(adt, h, T, d, g.rms_eps, u, s, gu8 ? xq : nullptr, xqs); }
    // The shared FFN depends only on u, so its two projections can run on the
    // side stream (its fp32 output rows go to a buffer of their own) while
    // the router and the routing run here; the combine then adds the routed
    // experts and the shared FFN into the residual.  The branch joins before
    // the combine.  Above 256 rows the expert GEMMs it overlaps are bound by
    // their MFMAs.  At 256 rows and below it mostly fills the latency-bound
    // routing (the rest of it overlaps the start of the HBM-bound expert
    // GEMMs), which pays only inside a captured graph (edges instead of the
    // runtime's event waits), so a pass launched one by one runs the shared
    // FFN in line.
    const bool fork = g.shared_hidden && (T > 256 || c->capturing) && ensure_side(c);
    if (g.shared_hidden) {
      hipStream_t ss = fork ? c->side : s;
      if (fork) {
        hipEventRecord(c->ev_fork, s);
        hipStreamWaitEvent(c->side, c->ev_fork, 0);
      }
      GemmArgs a = gemm_base(u, d, c->W + lw.sgu, nullptr, d, p.sgu_npad, 2 * g.shared_hidden,
                             c->st<void>(p.sact), g.shared_hidden);
      { Prof pg(c, CD_PROF_SHARED_GU, ss); gemm_dense(c, p.wdt_other, EPI_SWIGLU, a, T, ss); }
      GemmArgs b = gemm_base(c->st<void>(p.sact), g.shared_hidden, c->W + lw.sdn, nullptr, g.shared_hidden,
                             p.sdn_npad, d, c->st<float>(p.sout), d);
      { Prof pd(c, CD_PROF_SHARED_DOWN, ss); gemm_dense(c, p.wdt_other, EPI_F32, b, T, ss); }
      if (fork) hipEventRecord(c->ev_join, c->side);
    }
    // router logits as fp32 partial sums over a split contraction (the
    // top-k kernel adds them in split order): the router weight is small, so
    // splitting K is what gives the launch enough waves
    const int rsplit = router_split(g, T);
    {
      GemmArgs a = gemm_base(u, d, c->W + lw.wr, nullptr, d, p.wr_npad, E, c->st<float>(p.rlog), E);
      a.ksplit = rsplit;
      a.y_kstride = (int64_t)T * E;
      PROF(CD_PROF_ROUTER);
      gemm_dense(c, p.wdt_other, EPI_F32, a, T, s);
    }
    RouteArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.logits = c->st<float>(p.rlog); ra.nsplit = rsplit; ra.T = T; ra.E = E; ra.k = k;
    ra.topk_id = c->st<int32_t>(p.topk_id); ra.topk_gate = c->st<float>(p.topk_gate);
    ra.blk_cnt = c->st<int32_t>(p.blk_cnt); ra.seg_off = c->st<int32_t>(p.seg_off);
    ra.row_map = c->st<int32_t>(p.row_map); ra.slot = c->st<int32_t>(p.slot);
    ra.tiles = c->st<int32_t>(p.tiles); ra.n_tiles = c->st<int32_t>(p.n_tiles);
    ra.mrows = big_expert_tiles((int64_t)T * k, E) ? BIG_TILE_ROWS : 16 * grouped_mt(p);
    ra.max_rows = (int)p.max_rows; ra.max_tiles = (int)p.max_tiles;
    if (trace && c->trace_ids) {
      ra.trace_ids = c->trace_ids + (int64_t)l * T * k;
      ra.trace_gates = c->trace_gates + (int64_t)l * T * k;
    }
    { PROF(CD_PROF_ROUTE); launch_route(ra, s); }
    {
      GemmArgs a = gemm_base(u, d, c->W + lw.gu, c->wt<float>(lw.gu_s), d, p.gu_npad, 2 * g.expert_hidden,
                             c->st<void>(p.aperm), g.expert_hidden);
      a.row_map = c->st<int32_t>(p.row_map);
      a.w_gstride = p.gu_stride; a.s_gstride = p.gu_npad; a.mx_off = p.gu_mx;
      PROF(CD_PROF_EXPERT_GU);
      gemm_grouped(c, p.wdt_exp, EPI_SWIGLU, a, (int64_t)T * k, T, nullptr, s, gu8);
    }
    {
      GemmArgs a = gemm_base(c->st<void>(p.aperm), g.expert_hidden, c->W + lw.dn, c->wt<float>(lw.dn_s),
                             g.expert_hidden, p.dn_npad, d, c->st<void>(p.yperm), d);
      a.w_gstride = p.dn_stride; a.s_gstride = p.dn_npad; a.mx_off = p.dn_mx;
      PROF(CD_PROF_EXPERT_DOWN);
      gemm_grouped(c, p.wdt_exp, EPI_ROWS, a, (int64_t)T * k, (int)p.max_rows, c->st<int32_t>(p.seg_off) + E, s);
    }
    // h += sum_j gate_j * y_j (choice order) + shared FFN row; the same kernel
    // writes u = RMSNorm(h) for the next layer or the LM head (every reader
    // of this layer's u ran before it on this stream or joined above)
    if (fork) hipStreamWaitEvent(s, c->ev_join, 0);
    {
      u_ready = l + 1 < g.n_layers || head;
      const bool q8 = qkv8 && l + 1 < g.n_layers;   // the next layer's QKV input in E4M3
      PROF(CD_PROF_COMBINE);
      launch_combine(adt, c->st<void>(p.yperm), c->st<int32_t>(p.slot), c->st<float>(p.topk_gate),
                     g.shared_hidden ? c->st<float>(p.sout) : nullptr, T, k, d, h, u_ready ? u : nullptr,
                     g.rms_eps, s, q8 ? xq : nullptr, xqs);
    }
  }
  if (head) {
    if (!u_ready) { PROF(CD_PROF_RMSNORM); launch_rmsnorm(adt, h, T, d, g.rms_eps, u, s); }
    float* logits = c->st<float>(p.logits) + (int64_t)r0 * g.canvas_len * g.vocab;
    GemmArgs a = gemm_base(u, d, c->W + p.lm, nullptr, d, p.lm_npad, g.vocab, logits, g.vocab);
    PROF(CD_PROF_LM_HEAD);
    gemm_dense(c, p.wdt_other, EPI_F32, a, T, s);
  }
}

void sample(cd_ctx* c, int r0, int n_req, hipStream_t s) {
  const Plan& p = c->p;
  const cd_config& g = p.c;
  const int C = g.canvas_len;
  SampleArgs a;
  memset(&a, 0, sizeof a);
  a.logits = c->st<float>(p.logits) + (int64_t)r0 * C * g.vocab;
  a.rows = n_req * C; a.V = g.vocab; a.C = C;
  a.n_chunks = (int)p.n_chunks; a.chunk = g.vocab / a.n_chunks;
  a.part = c->st<float4>(p.spart);
  a.prev_a = c->st<int32_t>(p.argmax) + (int64_t)r0 * C;
  a.tokens = c->st<int32_t>(p.canvas) + (int64_t)r0 * C;
  a.argmax = c->st<int32_t>(p.argmax) + (int64_t)r0 * C;
  a.lock = c->st<uint8_t>(p.lock) + (int64_t)r0 * C;
  a.entropy = c->st<double>(p.entropy) + (int64_t)r0 * C;
  a.pmax = c->st<double>(p.pmax) + (int64_t)r0 * C;
  a.info = c->st<cd_step_info>(p.info) + r0;
  a.canvas_in = c->st<int32_t>(p.canvas) + (int64_t)r0 * C;
  a.rq = c->st<ReqDev>(p.rq) + r0;
  a.req0 = r0;
  for (int r = r0; r < r0 + n_req; ++r)
    if (c->req[r].active) a.active[r >> 6] |= 1ull << (r & 63);
  a.max_steps = g.max_steps; a.lock_th = g.lock_threshold; a.stop_H = g.stop_entropy;
  a.lock_rule = g.lock_rule; a.ent_bound = g.entropy_bound;
  { PROF(CD_PROF_SAMPLER_PART); launch_sampler_part(a, s); }
  { PROF(CD_PROF_SAMPLER_FINAL); launch_sampler_final(a, s); }
}

int32_t check_ctx(cd_ctx* c) { return c ? CD_OK : fail(CD_ERR_INVALID_ARG, "null context"); }

// end of a call that launched a forward: a launcher refusal, else the HIP status
int32_t finish(cd_ctx* c, const char* where) {
  if (c->launch_err) {
    const int32_t st = c->launch_err;
    c->launch_err = 0;
    return fail(st, "%s: a GEMM launch was refused (MXFP4 weights with a split contraction)", where);
  }
  return hip_status(where);
}

// One pass over requests r0..r0+n_req-1.  Requests without an active canvas
// ride along: their rows go through the forward (whatever ids their canvas
// holds, keys/values written past their committed length), but the sampler
// leaves their state untouched.
void release_graphs(cd_ctx* c) {
  if (c->pass_graphs.empty()) return;
  hipDeviceSynchronize();   // a graph may still run on some stream
  for (auto& pg : c->pass_graphs) hipGraphExecDestroy(pg.exec);
  c->pass_graphs.clear();
}

constexpr size_t MAX_PASS_GRAPHS = 16;

// The pass as a graph: 0 when it was launched on s, 1 when it was not captured
// (graphs then stay off for this context and the caller runs the pass
// directly), or an error status.
int32_t step_graph(cd_ctx* c, int r0, int n_req, hipStream_t s) {
  const cd_config& g = c->p.c;
  int nkeys = 0;
  uint64_t act[4] = {0, 0, 0, 0};
  for (int r = r0; r < r0 + n_req; ++r) {
    nkeys = std::max(nkeys, c->req[r].P + g.canvas_len);
    if (c->req[r].active) act[r >> 6] |= 1ull << (r & 63);
  }
  cd_ctx::PassGraph* hit = nullptr;
  for (auto& pg : c->pass_graphs)
    if (pg.r0 == r0 && pg.n_req == n_req && pg.nkeys == nkeys && !memcmp(pg.act, act, sizeof act)) hit = &pg;
  if (!hit) {
    ensure_side(c);   // the shared FFN's stream and events exist before the capture
    if (!c->cap && hipStreamCreateWithFlags(&c->cap, hipStreamNonBlocking) != hipSuccess) {
      c->cap = nullptr;
      c->graphs = false;
      (void)hipGetLastError();
      return 1;
    }
    if (hipStreamBeginCapture(c->cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      c->graphs = false;
      (void)hipGetLastError();
      return 1;
    }
    c->capturing = true;
    forward(c, r0, n_req, g.canvas_len, c->st<int32_t>(c->p.canvas) + (int64_t)r0 * g.canvas_len, false, true,
            true, c->cap);
    sample(c, r0, n_req, c->cap);
    c->capturing = false;
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(c->cap, &graph);
    if (c->launch_err) {
      if (graph) hipGraphDestroy(graph);
      return finish(c, "denoise step");
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = (ec == hipSuccess && graph) ? hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) : ec;
    if (graph) hipGraphDestroy(graph);
    if (ei != hipSuccess || !exec) {
      c->graphs = false;
      (void)hipGetLastError();
      return 1;
    }
    if (c->pass_graphs.size() >= MAX_PASS_GRAPHS) {
      // drop the least recently used graph
      size_t lru = 0;
      for (size_t i = 1; i < c->pass_graphs.size(); ++i)
        if (c->pass_graphs[i].used < c->pass_graphs[lru].used) lru = i;
      hipDeviceSynchronize();
      hipGraphExecDestroy(c->pass_graphs[lru].exec);
      c->pass_graphs.erase(c->pass_graphs.begin() + lru);
    }
    cd_ctx::PassGraph pg;
    pg.r0 = r0; pg.n_req = n_req; pg.nkeys = nkeys;
    memcpy(pg.act, act, sizeof act);
    pg.exec = exec;
    pg.used = 0;
    c->pass_graphs.push_back(pg);
    hit = &c->pass_graphs.back();
  }
  hit->used = ++c->graph_clock;
  if (hipGraphLaunch(hit->exec, s) != hipSuccess) return hip_status("graph launch");
  return 0;
}

int32_t step_internal(cd_ctx* c, int r0, int n_req, hipStream_t s) {
  const cd_config& g = c->p.c;
  int n_active = 0;
  for (int r = r0; r < r0 + n_req; ++r) {
    const HostReq& q = c->req[r];
    if (!q.active) {
      if ((int64_t)q.P + g.canvas_len > g.max_ctx)
        return fail(CD_ERR_CAPACITY, "idle request %d has no room for a canvas (release it)", r);
      continue;
    }
    if (q.t >= g.max_steps) return fail(CD_ERR_BAD_STATE, "request %d reached the step cap", r);
    ++n_active;
  }
  if (!n_active) return fail(CD_ERR_BAD_STATE, "no request in 0..%d has an active canvas", r0 + n_req - 1);
  // per-launch profiling events and trace copies are taken eagerly
  int32_t st = 1;
  if (c->graphs && !c->prof && !c->trace_h && !c->trace_hmid && !c->trace_ids && !c->trace_gates)
    st = step_graph(c, r0, n_req, s);
  if (st > 1 || st < 0) return st;
  if (st == 1) {
    forward(c, r0, n_req, g.canvas_len, c->st<int32_t>(c->p.canvas) + (int64_t)r0 * g.canvas_len, false, true,
            true, s);
    sample(c, r0, n_req, s);
  }
  for (int r = r0; r < r0 + n_req; ++r)
    if (c->req[r].active) c->req[r].t++;
  return finish(c, "denoise step");
}

int32_t read_info(cd_ctx* c, int r, cd_step_info* out, hipStream_t s) {
  if (hipMemcpyAsync(out, c->st<cd_step_info>(c->p.info) + r, sizeof(cd_step_info), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return hip_status("step info copy");
  if (hipStreamSynchronize(s) != hipSuccess) return hip_status("stream sync");
  return CD_OK;
}

PackDesc desc_for(const cd_ctx* c, int kind, int layer, int expert, int& status) {
  const Plan& p = c->p;
  const cd_config& g = p.c;
  PackDesc d;
  memset(&d, 0, sizeof d);
  d.only_sel = -1;
  status = CD_OK;
  const int dh = g.head_dim, dm = g.d_model, E = g.n_experts;
  const bool layered = kind >= CD_W_Q;
  if (layered && (layer < 0 || layer >= g.n_layers)) { status = fail(CD_ERR_INVALID_ARG, "layer out of range"); return d; }
  const bool per_expert = kind == CD_W_GATE || kind == CD_W_UP || kind == CD_W_DOWN;
  if (per_expert && (expert < 0 || expert >= E)) { status = fail(CD_ERR_INVALID_ARG, "expert out of range"); return d; }
  if ((kind >= CD_W_SHARED_GATE) && !g.shared_hidden) { status = fail(CD_ERR_INVALID_ARG, "no shared FFN"); return d; }
  const LayerOff* lw = layered ? &p.layer[layer] : nullptr;
  uint8_t* W = c->W;
  switch (kind) {
    case CD_W_EMBED:
      d.dst = W + p.embed; d.dt = p.wdt_other; d.perm = PERM_NONE; d.Npad = g.vocab; d.K = dm; d.rowmajor = 1;
      d.n_rows_src[0] = g.vocab; break;
    case CD_W_LM:
      d.dst = W + p.lm; d.dt = p.wdt_other; d.perm = PERM_NONE; d.Npad = p.lm_npad; d.K = dm; d.n_rows_src[0] = g.vocab;
      break;
    case CD_W_Q: case CD_W_K: case CD_W_V:
      d.dst = W + lw->qkv; d.scale = c->wt<float>(lw->qkv_s); d.dt = p.wdt_attn; d.perm = PERM_QKV;
      d.Npad = p.qkv_npad; d.K = dm; d.Hq = g.n_q_heads; d.Hkv = g.n_kv_heads; d.dh = dh;
      d.only_sel = kind - CD_W_Q; break;
    case CD_W_O:
      d.dst = W + lw->wo; d.scale = c->wt<float>(lw->wo_s); d.dt = p.wdt_attn; d.perm = PERM_NONE;
      d.Npad = p.wo_npad; d.K = g.n_q_heads * dh; d.n_rows_src[0] = dm; break;
    case CD_W_ROUTER:
      d.dst = W + lw->wr; d.dt = p.wdt_other; d.perm = PERM_NONE; d.Npad = p.wr_npad; d.K = dm; d.n_rows_src[0] = E;
      break;
    case CD_W_GATE: case CD_W_UP:
      d.dst = W + lw->gu + p.gu_stride * expert;
      d.scale = lw->gu_s >= 0 ? c->wt<float>(lw->gu_s) + (int64_t)p.gu_npad * expert : nullptr;
      d.dt = p.wdt_exp; d.perm = PERM_GU; d.Npad = p.gu_npad; d.K = dm; d.mx_off = p.gu_mx;
      d.n_rows_src[0] = d.n_rows_src[1] = g.expert_hidden; d.only_sel = kind - CD_W_GATE; break;
    case CD_W_DOWN:
      d.dst = W + lw->dn + p.dn_stride * expert;
      d.scale = lw->dn_s >= 0 ? c->wt<float>(lw->dn_s) + (int64_t)p.dn_npad * expert : nullptr;
      d.dt = p.wdt_exp; d.perm = PERM_NONE; d.Npad = p.dn_npad; d.K = g.expert_hidden; d.n_rows_src[0] = dm;
      d.mx_off = p.dn_mx; break;
    case CD_W_SHARED_GATE: case CD_W_SHARED_UP:
      d.dst = W + lw->sgu; d.dt = p.wdt_other; d.perm = PERM_GU; d.Npad = p.sgu_npad; d.K = dm;
      d.n_rows_src[0] = d.n_rows_src[1] = g.shared_hidden; d.only_sel = kind - CD_W_SHARED_GATE; break;
    case CD_W_SHARED_DOWN:
      d.dst = W + lw->sdn; d.dt = p.wdt_other; d.perm = PERM_NONE; d.Npad = p.sdn_npad; d.K = g.shared_hidden;
      d.n_rows_src[0] = dm; break;
    default:
      status = fail(CD_ERR_INVALID_ARG, "unknown weight kind %d", kind);
  }
  return d;
}

}  // namespace

extern "C" {

int32_t cd_weights_bytes(const cd_config* cfg, size_t* bytes) {
  int32_t st = validate_config(cfg);
  if (st) return st;
  if (!bytes) return fail(CD_ERR_INVALID_ARG, "null bytes");
  *bytes = (size_t)make_plan(*cfg).weights_bytes;
  return CD_OK;
}

int32_t cd_state_bytes(const cd_config* cfg, size_t* bytes) {
  int32_t st = validate_config(cfg);
  if (st) return st;
  if (!bytes) return fail(CD_ERR_INVALID_ARG, "null bytes");
  *bytes = (size_t)make_plan(*cfg).state_bytes;
  return CD_OK;
}

int32_t cd_ctx_create(const cd_config* cfg, void* d_weights, void* d_state, cd_ctx** out) {
  int32_t st = validate_config(cfg);
  if (st) return st;
  if (!d_weights || !d_state || !out) return fail(CD_ERR_INVALID_ARG, "null buffer or output pointer");
  if ((reinterpret_cast<uintptr_t>(d_weights) | reinterpret_cast<uintptr_t>(d_state)) % ALIGN)
    return fail(CD_ERR_INVALID_ARG, "buffers must be 256-byte aligned");
  cd_ctx* c = new cd_ctx;
  c->p = make_plan(*cfg);
  c->W = reinterpret_cast<uint8_t*>(d_weights);
  c->S = reinterpret_cast<uint8_t*>(d_state);
  c->req.assign(cfg->max_requests, HostReq());
  *out = c;
  g_err.clear();
  return CD_OK;
}

int32_t cd_ctx_destroy(cd_ctx* ctx) {
  if (ctx) {
    release_graphs(ctx);
    if (ctx->cap) hipStreamDestroy(ctx->cap);
    if (ctx->side) {
      hipStreamSynchronize(ctx->side);
      hipStreamDestroy(ctx->side);
    }
    if (ctx->ev_fork) hipEventDestroy(ctx->ev_fork);
    if (ctx->ev_join) hipEventDestroy(ctx->ev_join);
    for (hipEvent_t e : ctx->pool) hipEventDestroy(e);
  }
  delete ctx;
  return CD_OK;
}

int32_t cd_reset(cd_ctx* c, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  hipStream_t s = strm(stream);
  if (hipMemsetAsync(c->S, 0, c->p.state_bytes, s) != hipSuccess) return hip_status("state clear");
  launch_rope_table(c->st<float>(c->p.rope), c->p.ctx, c->p.c.head_dim, c->p.c.rope_theta, s);
  for (auto& r : c->req) r = HostReq();
  return hip_status("reset");
}

int32_t cd_synth_weights(cd_ctx* c, uint64_t seed, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  hipStream_t s = strm(stream);
  const Plan& p = c->p;
  const cd_config& g = p.c;
  const uint32_t S = 8 + 3 * g.n_experts;
  int status;
  PackDesc d = desc_for(c, CD_W_EMBED, 0, 0, status);
  d.tau[0] = 0;
  launch_synth(d, 1, 0, 0, 0, seed, s);
  d = desc_for(c, CD_W_LM, 0, 0, status);
  d.tau[0] = 1;
  launch_synth(d, 1, 0, 0, 0, seed, s);
  for (int l = 0; l < g.n_layers; ++l) {
    const uint32_t b = 2 + l * S;
    d = desc_for(c, CD_W_Q, l, 0, status);
    d.only_sel = -1; d.tau[0] = b; d.tau[1] = b + 1; d.tau[2] = b + 2;
    launch_synth(d, 1, 0, 0, 0, seed, s);
    d = desc_for(c, CD_W_O, l, 0, status);
    d.tau[0] = b + 3;
    launch_synth(d, 1, 0, 0, 0, seed, s);
    d = desc_for(c, CD_W_ROUTER, l, 0, status);
    d.tau[0] = b + 4;
    launch_synth(d, 1, 0, 0, 0, seed, s);
    d = desc_for(c, CD_W_GATE, l, 0, status);
    d.only_sel = -1; d.tau[0] = b + 5; d.tau[1] = b + 6;
    launch_synth(d, g.n_experts, p.gu_stride, p.gu_npad, 3, seed, s);
    d = desc_for(c, CD_W_DOWN, l, 0, status);
    d.tau[0] = b + 7;
    launch_synth(d, g.n_experts, p.dn_stride, p.dn_npad, 3, seed, s);
    if (g.shared_hidden) {
      const uint32_t sb = b + 5 + 3 * g.n_experts;
      d = desc_for(c, CD_W_SHARED_GATE, l, 0, status);
      d.only_sel = -1; d.tau[0] = sb; d.tau[1] = sb + 1;
      launch_synth(d, 1, 0, 0, 0, seed, s);
      d = desc_for(c, CD_W_SHARED_DOWN, l, 0, status);
      d.tau[0] = sb + 2;
      launch_synth(d, 1, 0, 0, 0, seed, s);
    }
  }
  return hip_status("synth weights");
}

int32_t cd_set_weight(cd_ctx* c, int32_t kind, int32_t layer, int32_t expert, const float* d_logical, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  if (!d_logical) return fail(CD_ERR_INVALID_ARG, "null source");
  int status;
  PackDesc d = desc_for(c, kind, layer, expert, status);
  if (status) return status;
  const float* src[3] = {nullptr, nullptr, nullptr};
  src[d.only_sel < 0 ? 0 : d.only_sel] = d_logical;
  if (d.perm == PERM_QKV) {   // rows of each part: Hq*dh, Hkv*dh, Hkv*dh
    d.n_rows_src[0] = c->p.c.n_q_heads * c->p.c.head_dim;
    d.n_rows_src[1] = d.n_rows_src[2] = c->p.c.n_kv_heads * c->p.c.head_dim;
  }
  launch_pack(d, src[0], src[1], src[2], strm(stream));
  return hip_status("set weight");
}

int32_t cd_get_weight(cd_ctx* c, int32_t kind, int32_t layer, int32_t expert, float* d_logical, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  if (!d_logical) return fail(CD_ERR_INVALID_ARG, "null destination");
  int status;
  PackDesc d = desc_for(c, kind, layer, expert, status);
  if (status) return status;
  float* dst[3] = {nullptr, nullptr, nullptr};
  dst[d.only_sel < 0 ? 0 : d.only_sel] = d_logical;
  launch_unpack(d, dst[0], dst[1], dst[2], strm(stream));
  return hip_status("get weight");
}

int32_t cd_prefill(cd_ctx* c, int32_t req, const int32_t* d_ids, int32_t n, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const cd_config& g = c->p.c;
  if (req < 0 || req >= g.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  if (!d_ids || n < 1 || n > g.max_prefill) return fail(CD_ERR_INVALID_ARG, "prefill needs 1..max_prefill ids");
  HostReq& q = c->req[req];
  if (q.active) return fail(CD_ERR_BAD_STATE, "request %d has an active canvas", req);
  if ((int64_t)q.P + n + g.canvas_len > g.max_ctx) return fail(CD_ERR_CAPACITY, "KV cache too small for prefill");
  hipStream_t s = strm(stream);
  forward(c, req, 1, n, d_ids, true, false, true, s);
  launch_advance(c->st<ReqDev>(c->p.rq), req, n, s);
  q.P += n;
  return finish(c, "prefill");
}

// canvas start of slot req; rid keys its Philox stream (the slot itself for
// the public call, the queue index in the batched loop)
static int32_t init_canvas_internal(cd_ctx* c, int32_t req, uint64_t seed, int32_t block, int32_t rid,
                                    hipStream_t s) {
  const cd_config& g = c->p.c;
  HostReq& q = c->req[req];
  if (q.active) return fail(CD_ERR_BAD_STATE, "request %d already has an active canvas", req);
  if ((int64_t)q.P + g.canvas_len > g.max_ctx) return fail(CD_ERR_CAPACITY, "KV cache full");
  launch_init_canvas(c->st<int32_t>(c->p.canvas), c->st<ReqDev>(c->p.rq), req, g.canvas_len, g.vocab, seed, block,
                     rid, s);
  q.active = true; q.t = 0; q.block = block; q.seed = seed; q.rid = rid;
  return hip_status("init canvas");
}

// every per-slot row of request `from` (K/V region, canvas, last pass
// outputs, device state) copied to the free slot `to`; `from` is released
static int32_t move_internal(cd_ctx* c, int from, int to, hipStream_t s) {
  const Plan& p = c->p;
  const int64_t C = p.c.canvas_len, kvb = p.kv_req_stride * esize(p.adt);
  const int64_t span[][2] = {{p.kcache, kvb}, {p.vcache, kvb}, {p.canvas, 4 * C}, {p.argmax, 4 * C},
                             {p.lock, C},     {p.entropy, 8 * C}, {p.pmax, 8 * C}, {p.rq, (int64_t)sizeof(ReqDev)},
                             {p.info, (int64_t)sizeof(cd_step_info)}};
  for (const auto& x : span)
    if (hipMemcpyAsync(c->S + x[0] + to * x[1], c->S + x[0] + from * x[1], x[1], hipMemcpyDeviceToDevice, s) !=
        hipSuccess)
      return hip_status("slot move");
  if (c->req[from].P) launch_advance(c->st<ReqDev>(p.rq), from, -c->req[from].P, s);
  launch_zero_u32(c->st<cd_step_info>(p.info) + from, sizeof(cd_step_info) / 4, s);
  if (c->req[from].rid < 0) c->req[from].rid = from;
  c->req[to] = c->req[from];
  c->req[from] = HostReq();
  return hip_status("slot move");
}

int32_t cd_init_canvas(cd_ctx* c, int32_t req, uint64_t seed, int32_t block, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const cd_config& g = c->p.c;
  if (req < 0 || req >= g.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  if (block < 0) return fail(CD_ERR_INVALID_ARG, "negative block index");
  return init_canvas_internal(c, req, seed, block, c->req[req].rid >= 0 ? c->req[req].rid : req, strm(stream));
}

int32_t cd_release(cd_ctx* c, int32_t req, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  if (req < 0 || req >= c->p.c.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  HostReq& q = c->req[req];
  hipStream_t s = strm(stream);
  if (q.P) launch_advance(c->st<ReqDev>(c->p.rq), req, -q.P, s);
  // the slot's last step record goes with the request
  launch_zero_u32(c->st<cd_step_info>(c->p.info) + req, sizeof(cd_step_info) / 4, s);
  q = HostReq();
  return hip_status("release");
}

int32_t cd_move_request(cd_ctx* c, int32_t from, int32_t to, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const int R = c->p.c.max_requests;
  if (from < 0 || from >= R || to < 0 || to >= R || from == to)
    return fail(CD_ERR_INVALID_ARG, "bad slots %d -> %d", from, to);
  if (c->req[to].P || c->req[to].active) return fail(CD_ERR_BAD_STATE, "slot %d is not free", to);
  return move_internal(c, from, to, strm(stream));
}

int32_t cd_denoise_step(cd_ctx* c, int32_t n_req, cd_step_info* d_info, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  if (n_req < 1 || n_req > c->p.c.max_requests) return fail(CD_ERR_INVALID_ARG, "n_req out of range");
  if (!d_info) return fail(CD_ERR_INVALID_ARG, "null step info");
  hipStream_t s = strm(stream);
  if (int32_t st = step_internal(c, 0, n_req, s)) return st;
  if (hipMemcpyAsync(d_info, c->st<cd_step_info>(c->p.info), sizeof(cd_step_info) * n_req, hipMemcpyDeviceToDevice,
                     s) != hipSuccess)
    return hip_status("step info copy");
  return CD_OK;
}

int32_t cd_abort_canvas(cd_ctx* c, int32_t req) {
  if (int32_t st = check_ctx(c)) return st;
  if (req < 0 || req >= c->p.c.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  HostReq& q = c->req[req];
  if (!q.active) return fail(CD_ERR_BAD_STATE, "request %d has no active canvas", req);
  q.active = false;
  q.t = 0;
  return CD_OK;
}

int32_t cd_set_graphs(cd_ctx* c, int32_t enable) {
  if (int32_t st = check_ctx(c)) return st;
  if (!enable) release_graphs(c);
  c->graphs = enable != 0;
  return CD_OK;
}

int32_t cd_profile(cd_ctx* c, int32_t enable) {
  if (int32_t st = check_ctx(c)) return st;
  c->prof = enable != 0;
  if (c->prof) {
    c->recs.clear();
    c->pool_used = 0;
  }
  return CD_OK;
}

int32_t cd_profile_read(cd_ctx* c, double* ms, int32_t* launches, int32_t n_classes) {
  if (int32_t st = check_ctx(c)) return st;
  if (!ms || !launches || n_classes < 1 || n_classes > CD_PROF_CLASSES)
    return fail(CD_ERR_INVALID_ARG, "bad profile output arrays");
  for (int i = 0; i < n_classes; ++i) { ms[i] = 0.0; launches[i] = 0; }
  for (const ProfRec& r : c->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return hip_status("profile event sync");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return hip_status("profile elapsed");
    if (r.cls < n_classes) { ms[r.cls] += t; launches[r.cls] += 1; }
  }
  return CD_OK;
}

int32_t cd_read_step_info(cd_ctx* c, const cd_step_info* d_info, int32_t n_req, cd_step_info* h_info, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  if (!d_info || !h_info || n_req < 1) return fail(CD_ERR_INVALID_ARG, "bad step info arguments");
  hipStream_t s = strm(stream);
  if (hipMemcpyAsync(h_info, d_info, sizeof(cd_step_info) * n_req, hipMemcpyDeviceToHost, s) != hipSuccess)
    return hip_status("step info copy");
  if (hipStreamSynchronize(s) != hipSuccess) return hip_status("stream sync");
  for (int r = 0; r < n_req; ++r)
    if (h_info[r].after_stop)
      return fail(CD_ERR_BAD_STATE, "request %d was given a denoise pass after its stop (records copied)", r);
  return CD_OK;
}

int32_t cd_commit_block(cd_ctx* c, int32_t req, int32_t* d_out_ids, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const cd_config& g = c->p.c;
  if (req < 0 || req >= g.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  if (!d_out_ids) return fail(CD_ERR_INVALID_ARG, "null output ids");
  HostReq& q = c->req[req];
  if (!q.active || q.t < 1) return fail(CD_ERR_BAD_STATE, "request %d has no denoised canvas to commit", req);
  hipStream_t s = strm(stream);
  cd_step_info info;
  if (int32_t st = read_info(c, req, &info, s)) return st;
  if (info.after_stop)
    return fail(CD_ERR_BAD_STATE, "request %d was given a denoise pass after its stop; abort its canvas", req);
  int32_t* a = c->st<int32_t>(c->p.argmax) + (int64_t)req * g.canvas_len;
  if (!info.canvas_is_argmax) forward(c, req, 1, g.canvas_len, a, false, false, true, s);
  launch_copy_i32(a, d_out_ids, g.canvas_len, s);
  launch_advance(c->st<ReqDev>(c->p.rq), req, g.canvas_len, s);
  q.P += g.canvas_len;
  q.active = false;
  return finish(c, "commit");
}

int32_t cd_generate(cd_ctx* c, int32_t req, const int32_t* d_prefix, int32_t n_prefix, int32_t n_blocks,
                    uint64_t seed, int32_t* d_out_ids, int32_t* h_steps_per_block, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const cd_config& g = c->p.c;
  if (req < 0 || req >= g.max_requests) return fail(CD_ERR_INVALID_ARG, "request %d out of range", req);
  if (n_blocks < 1 || !d_out_ids || !h_steps_per_block || n_prefix < 0 || (n_prefix > 0 && !d_prefix))
    return fail(CD_ERR_INVALID_ARG, "bad generate arguments");
  HostReq& q = c->req[req];
  if (q.active) return fail(CD_ERR_BAD_STATE, "request %d has an active canvas", req);
  if ((int64_t)q.P + n_prefix + (int64_t)n_blocks * g.canvas_len > g.max_ctx)
    return fail(CD_ERR_CAPACITY, "KV cache too small for %d blocks", n_blocks);
  if (n_prefix > g.max_prefill) return fail(CD_ERR_INVALID_ARG, "prefix longer than max_prefill");
  hipStream_t s = strm(stream);
  if (n_prefix > 0)
    if (int32_t st = cd_prefill(c, req, d_prefix, n_prefix, stream)) return st;
  for (int b = 0; b < n_blocks; ++b) {
    if (int32_t st = cd_init_canvas(c, req, seed, b, stream)) return st;
    int steps = 0;
    for (;;) {
      if (int32_t st = step_internal(c, req, 1, s)) return st;
      cd_step_info info;
      if (int32_t st = read_info(c, req, &info, s)) return st;
      steps = info.step;
      if (info.nonfinite) return fail(CD_ERR_NUMERIC, "non-finite logits at block %d pass %d", b, steps);
      if (info.stop) break;
    }
    h_steps_per_block[b] = steps;
    if (int32_t st = cd_commit_block(c, req, d_out_ids + (int64_t)b * g.canvas_len, stream)) return st;
  }
  return hip_status("generate");
}

// the loop of cd_serve, on arguments it has validated
static int32_t serve_loop(cd_ctx* c, int32_t n_queue, const int32_t* d_prefix, const int64_t* h_prefix_off,
                          const int32_t* h_prefix_len, const int32_t* h_n_blocks, const uint64_t* h_seeds,
                          int32_t n_slots, int32_t* d_out, const int64_t* h_out_off, int32_t* h_steps, void* stream) {
  const int C = c->p.c.canvas_len;
  hipStream_t s = strm(stream);
  for (int r = 0; r < n_slots; ++r)
    if (int32_t st = cd_release(c, r, stream)) return st;
  std::vector<int64_t> steps_off(n_queue + 1, 0);
  for (int q = 0; q < n_queue; ++q) steps_off[q + 1] = steps_off[q] + h_n_blocks[q];
  std::vector<int> slot_q(n_slots, -1), slot_b(n_slots, 0);
  int next = 0;
  // a free slot takes the next queued request: cleared, prefilled, first canvas
  auto admit = [&](int r) -> int32_t {
    slot_q[r] = -1;
    if (int32_t st = cd_release(c, r, stream)) return st;
    if (next >= n_queue) return CD_OK;
    const int q = next++;
    if (int32_t st = cd_prefill(c, r, d_prefix + h_prefix_off[q], h_prefix_len[q], stream)) return st;
    if (int32_t st = init_canvas_internal(c, r, h_seeds[q], 0, q, s)) return st;
    slot_q[r] = q;
    slot_b[r] = 0;
    return CD_OK;
  };
  for (int r = 0; r < n_slots; ++r)
    if (int32_t st = admit(r)) return st;
  std::vector<cd_step_info> info(n_slots);
  for (;;) {
    int n_act = 0;   // busy slots past the last one are not computed
    for (int r = 0; r < n_slots; ++r)
      if (slot_q[r] >= 0) n_act = r + 1;
    if (!n_act) break;
    if (int32_t st = step_internal(c, 0, n_act, s)) return st;
    if (hipMemcpyAsync(info.data(), c->st<cd_step_info>(c->p.info), sizeof(cd_step_info) * n_act,
                       hipMemcpyDeviceToHost, s) != hipSuccess)
      return hip_status("step info copy");
    if (hipStreamSynchronize(s) != hipSuccess) return hip_status("stream sync");
    for (int r = 0; r < n_act; ++r) {
      const int q = slot_q[r];
      if (q < 0) continue;
      if (info[r].nonfinite) return fail(CD_ERR_NUMERIC, "non-finite logits for queued request %d", q);
      if (!info[r].stop) continue;
      const int b = slot_b[r];
      h_steps[steps_off[q] + b] = info[r].step;
      if (int32_t st = cd_commit_block(c, r, d_out + h_out_off[q] + (int64_t)b * C, stream)) return st;
      if (b + 1 < h_n_blocks[q]) {
        slot_b[r] = b + 1;
        if (int32_t st = init_canvas_internal(c, r, h_seeds[q], b + 1, q, s)) return st;
      } else if (int32_t st = admit(r)) {
        return st;
      }
    }
    // with the queue drained, idle slots would ride along below busy ones:
    // the highest busy request moves into the lowest idle slot
    for (;;) {
      int hi = -1, lo = -1;
      for (int r = n_slots - 1; r >= 0 && hi < 0; --r)
        if (slot_q[r] >= 0) hi = r;
      for (int r = 0; r < hi && lo < 0; ++r)
        if (slot_q[r] < 0) lo = r;
      if (lo < 0) break;
      if (int32_t st = move_internal(c, hi, lo, s)) return st;
      slot_q[lo] = slot_q[hi]; slot_b[lo] = slot_b[hi];
      slot_q[hi] = -1;
    }
  }
  return hip_status("serve");
}

int32_t cd_serve(cd_ctx* c, int32_t n_queue, const int32_t* d_prefix, const int64_t* h_prefix_off,
                 const int32_t* h_prefix_len, const int32_t* h_n_blocks, const uint64_t* h_seeds, int32_t n_slots,
                 int32_t* d_out, const int64_t* h_out_off, int32_t* h_steps, void* stream) {
  if (int32_t st = check_ctx(c)) return st;
  const cd_config& g = c->p.c;
  if (n_queue < 1 || n_slots < 1 || n_slots > g.max_requests || !d_prefix || !h_prefix_off || !h_prefix_len ||
      !h_n_blocks || !h_seeds || !d_out || !h_out_off || !h_steps)
    return fail(CD_ERR_INVALID_ARG, "bad serve arguments");
  for (int q = 0; q < n_queue; ++q) {
    if (h_prefix_len[q] < 1 || h_prefix_len[q] > g.max_prefill || h_n_blocks[q] < 1 || h_prefix_off[q] < 0 ||
        h_out_off[q] < 0)
      return fail(CD_ERR_INVALID_ARG, "bad prefix length, block count or offset for queued request %d", q);
    if ((int64_t)h_prefix_len[q] + (int64_t)h_n_blocks[q] * g.canvas_len > g.max_ctx)
      return fail(CD_ERR_CAPACITY, "queued request %d does not fit the KV cache", q);
  }
  for (int r = 0; r < n_slots; ++r)
    if (c->req[r].active) return fail(CD_ERR_BAD_STATE, "slot %d has an active canvas", r);
  const int32_t st = serve_loop(c, n_queue, d_prefix, h_prefix_off, h_prefix_len, h_n_blocks, h_seeds, n_slots,
                                d_out, h_out_off, h_steps, stream);
  if (st) {
    // a failed loop still releases its slots (the error message is kept)
    for (int r = 0; r < n_slots; ++r) {
      if (c->req[r].P) launch_advance(c->st<ReqDev>(c->p.rq), r, -c->req[r].P, strm(stream));
      c->req[r] = HostReq();
    }
  }
  return st;
}

int32_t cd_sample_workspace_bytes(int32_t rows, int32_t vocab, size_t* bytes) {
  if (rows < 1 || vocab < 128 || vocab % 128 || !bytes) return fail(CD_ERR_INVALID_ARG, "bad sampler shape");
  *bytes = (size_t)16 * rows * sampler_chunks(vocab);
  return CD_OK;
}

// argument checks shared by the two sampler entry points
static int32_t check_sample_args(const cd_config* cfg, const float* d_logits, int32_t rows, int32_t step,
                                 int32_t block, int32_t req0, const int32_t* d_tokens, const int32_t* d_argmax,
                                 const uint8_t* d_lock, const double* d_entropy, const double* d_pmax,
                                 const cd_step_info* d_info) {
  if (!cfg) return fail(CD_ERR_INVALID_ARG, "null config");
  if (cfg->vocab < 128 || cfg->vocab % 128 || cfg->canvas_len < 1)
    return fail(CD_ERR_UNSUPPORTED, "vocab must be a positive multiple of 128");
  if (rows < 1 || rows % cfg->canvas_len) return fail(CD_ERR_INVALID_ARG, "rows must be a multiple of canvas_len");
  if (!d_logits || !d_tokens || !d_argmax || !d_lock || !d_entropy || !d_pmax || !d_info)
    return fail(CD_ERR_INVALID_ARG, "null buffer");
  if (step < 1 || block < 0 || req0 < 0) return fail(CD_ERR_INVALID_ARG, "bad step/block/request");
  return CD_OK;
}

static int32_t sample_on(const cd_config* cfg, const float* d_logits, int32_t rows, const int32_t* d_prev_argmax,
                         uint64_t seed, int32_t step, int32_t block, int32_t req0, int32_t* d_tokens,
                         int32_t* d_argmax, uint8_t* d_lock, double* d_entropy, double* d_pmax,
                         cd_step_info* d_info, float4* part, void* stream) {
  SampleArgs a;
  memset(&a, 0, sizeof a);
  a.logits = d_logits; a.rows = rows; a.V = cfg->vocab; a.C = cfg->canvas_len;
  a.n_chunks = sampler_chunks(cfg->vocab); a.chunk = cfg->vocab / a.n_chunks;
  a.part = part;
  a.prev_a = d_prev_argmax; a.tokens = d_tokens; a.argmax = d_argmax; a.lock = d_lock;
  a.entropy = d_entropy; a.pmax = d_pmax; a.info = d_info; a.canvas_in = nullptr; a.rq = nullptr;
  a.seed = seed; a.step = step; a.block = block; a.req0 = req0;
  a.max_steps = cfg->max_steps; a.lock_th = cfg->lock_threshold; a.stop_H = cfg->stop_entropy;
  a.lock_rule = cfg->lock_rule; a.ent_bound = cfg->entropy_bound;
  launch_sampler_part(a, strm(stream));
  launch_sampler_final(a, strm(stream));
  return hip_status("sample step");
}

int32_t cd_sample_step(const cd_config* cfg, const float* d_logits, int32_t rows, const int32_t* d_prev_argmax,
                       uint64_t seed, int32_t step, int32_t block, int32_t req0, int32_t* d_tokens,
                       int32_t* d_argmax, uint8_t* d_lock, double* d_entropy, double* d_pmax,
                       cd_step_info* d_info, void* d_workspace, void* stream) {
  if (int32_t st = check_sample_args(cfg, d_logits, rows, step, block, req0, d_tokens, d_argmax, d_lock, d_entropy,
                                     d_pmax, d_info))
    return st;
  if (!d_workspace) return fail(CD_ERR_INVALID_ARG, "null workspace");
  return sample_on(cfg, d_logits, rows, d_prev_argmax, seed, step, block, req0, d_tokens, d_argmax, d_lock,
                   d_entropy, d_pmax, d_info, reinterpret_cast<float4*>(d_workspace), stream);
}

int32_t cd_sample_step_noalloc(const cd_config* cfg, const float* d_logits, int32_t rows,
                               const int32_t* d_prev_argmax, uint64_t seed, int32_t step, int32_t block,
                               int32_t req0, int32_t* d_tokens, int32_t* d_argmax, uint8_t* d_lock,
                               double* d_entropy, double* d_pmax, cd_step_info* d_info, void* stream) {
  if (int32_t st = check_sample_args(cfg, d_logits, rows, step, block, req0, d_tokens, d_argmax, d_lock, d_entropy,
                                     d_pmax, d_info))
    return st;
  const int64_t partials = (int64_t)rows * sampler_chunks(cfg->vocab);
  if (partials > SAMPLER_SCRATCH_PARTIALS)
    return fail(CD_ERR_CAPACITY, "rows x chunks = %lld partials exceed the fixed buffer's %d (at most %d rows at "
                "vocab %d)", (long long)partials, SAMPLER_SCRATCH_PARTIALS,
                SAMPLER_SCRATCH_PARTIALS / sampler_chunks(cfg->vocab), cfg->vocab);
  float4* part = nullptr;
  if (sampler_scratch(&part)) return fail(CD_ERR_HIP, "fixed sampler buffer: device address lookup failed");
  return sample_on(cfg, d_logits, rows, d_prev_argmax, seed, step, block, req0, d_tokens, d_argmax, d_lock,
                   d_entropy, d_pmax, d_info, part, stream);
}

int32_t cd_get_buffer(cd_ctx* c, int32_t which, void** d_ptr, size_t* bytes) {
  if (int32_t st = check_ctx(c)) return st;
  if (!d_ptr) return fail(CD_ERR_INVALID_ARG, "null output");
  const Plan& p = c->p;
  const cd_config& g = p.c;
  const int64_t RC = (int64_t)g.max_requests * g.canvas_len;
  const int ae = esize(p.adt);
  int64_t off, n;
  switch (which) {
    case CD_BUF_LOGITS: off = p.logits; n = 4 * RC * g.vocab; break;
    case CD_BUF_CANVAS: off = p.canvas; n = 4 * RC; break;
    case CD_BUF_ARGMAX: off = p.argmax; n = 4 * RC; break;
    case CD_BUF_ENTROPY: off = p.entropy; n = 8 * RC; break;
    case CD_BUF_PMAX: off = p.pmax; n = 8 * RC; break;
    case CD_BUF_LOCK: off = p.lock; n = RC; break;
    case CD_BUF_KCACHE: off = p.kcache; n = (int64_t)ae * p.kv_req_stride * g.max_requests; break;
    case CD_BUF_VCACHE: off = p.vcache; n = (int64_t)ae * p.kv_req_stride * g.max_requests; break;
    case CD_BUF_HIDDEN: off = p.h; n = 4LL * p.Tmax * g.d_model; break;
    default: return fail(CD_ERR_INVALID_ARG, "unknown buffer %d", which);
  }
  *d_ptr = c->S + off;
  if (bytes) *bytes = (size_t)n;
  return CD_OK;
}

int32_t cd_get_config(cd_ctx* c, cd_config* out) {
  if (int32_t st = check_ctx(c)) return st;
  if (!out) return fail(CD_ERR_INVALID_ARG, "null output");
  *out = c->p.c;
  return CD_OK;
}

int32_t cd_get_length(cd_ctx* c, int32_t req, int32_t* P) {
  if (int32_t st = check_ctx(c)) return st;
  if (req < 0 || req >= c->p.c.max_requests || !P) return fail(CD_ERR_INVALID_ARG, "bad request or output");
  *P = c->req[req].P;
  return CD_OK;
}

int32_t cd_set_trace(cd_ctx* c, float* d_h_layers, int32_t* d_topk_ids, float* d_topk_gates,
                     float* d_h_mid_layers) {
  if (int32_t st = check_ctx(c)) return st;
  c->trace_h = d_h_layers;
  c->trace_hmid = d_h_mid_layers;
  c->trace_ids = d_topk_ids;
  c->trace_gates = d_topk_gates;
  return CD_OK;
}

const char* cd_last_error(void) { return g_err.c_str(); }

}  // extern "C"
