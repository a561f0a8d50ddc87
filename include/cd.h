/*
 * cd.h — C ABI of libcd: the canvas denoise step of block text diffusion
 * (DiffusionGemma-style) on one AMD MI355X (gfx950).
 *
 * The method (see the DiffusionGemma pages: the 256-token canvas explainer,
 * section "256-token Canvas 怎麼從雜訊變成文字？" steps ① to ④; the
 * MarkTechPost article, sections "how text diffusion works" and
 * "architecture"; the Google launch blog, "how text diffusion works"):
 *   ① the prompt is encoded causally into a reusable KV cache;
 *   ② a canvas of 256 token ids is drawn uniformly from the vocabulary;
 *   ③ passes run a bidirectional forward over the canvas (reading the
 *      committed KV cache), lock confident positions, re-noise the rest, and
 *      stop once the canvas mean entropy is below 0.005 nats and the argmax is
 *      unchanged over two consecutive passes (at most 48 passes);
 *   ④ the converged block is committed to the KV cache and the next canvas
 *      is conditioned on it.
 *
 * Conventions
 *  - Memory: every device buffer passed in is owned by the caller.  The
 *    library allocates no device memory: weights and state live in two
 *    caller-allocated device buffers whose sizes cd_weights_bytes and
 *    cd_state_bytes report.  Pointers marked d_ are device pointers, h_ host.
 *  - Streams: every call enqueues on the caller's hipStream_t (passed as
 *    void*) and returns without waiting, except where stated (cd_commit_block,
 *    cd_generate and cd_read_step_info synchronise the stream).  A forward
 *    (prefill, denoise pass, commit) with a shared FFN also uses a second
 *    stream that the context owns (default priority): it forks from the
 *    caller's stream with an event and joins back into it within the same
 *    call, so work enqueued later on the caller's stream sees every result.
 *    A context is therefore used from one stream at a time.
 *  - Errors: every function returns CD_OK (0) or a negative code.  All
 *    arguments and the request state are checked before anything is
 *    enqueued, so a failing call changes nothing.  A kernel fault surfaces as
 *    CD_ERR_HIP from the next call that synchronises.  cd_last_error() gives a
 *    message for the calling thread's last failure.
 *  - Threads: a context is used from one host thread at a time.
 */
#ifndef CD_H_
#define CD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CD_OK = 0,
  CD_ERR_INVALID_ARG = -1,  /* bad pointer, size or shape */
  CD_ERR_BAD_STATE = -2,    /* call out of order for this request */
  CD_ERR_CAPACITY = -3,     /* KV cache or workspace too small */
  CD_ERR_HIP = -4,          /* HIP runtime error */
  CD_ERR_UNSUPPORTED = -5,  /* shape the kernels do not handle */
  CD_ERR_NUMERIC = -6       /* non-finite logits met by the sampler */
};

/* Weight storage formats.  CD_FP8 stores attention projections and routed
 * experts as OCP E4M3FN with one bf16 scale per output row and every other
 * tensor as bf16; activations are then bf16.  CD_MXFP4 stores the routed
 * experts as MXFP4 (OCP Microscaling Formats v1.0: E2M1 elements, one E8M0
 * scale 2^e per 32 contraction elements of a row, e = floor(log2(max|w|))
 * - 2, elements round(w / 2^e) to nearest even saturating at +-6), the
 * attention projections as E4M3FN like CD_FP8, and everything else bf16;
 * the pages list a 4-bit checkpoint (NVFP4, an NVIDIA format) beside BF16
 * and FP8, and MXFP4 is the 4-bit format gfx950 converts natively. */
enum { CD_F32 = 0, CD_BF16 = 1, CD_FP8 = 2, CD_MXFP4 = 3 };

/* Lock rule of the sampler.  CD_LOCK_MAXPROB: a position keeps its argmax
 * when its max probability exceeds lock_threshold (the canvas explainer
 * page, step ③: confident tokens stay, uncertain ones are re-noised).
 * CD_LOCK_ENTROPY: it keeps its argmax when its entropy is at most
 * entropy_bound nats (the explainer's A/B guide serves the model with an
 * entropy-bound sampler and bound 0.1, giving only the name and the bound;
 * read here as the same per-position keep/re-noise choice made on the
 * entropy instead of the max probability). */
enum { CD_LOCK_MAXPROB = 0, CD_LOCK_ENTROPY = 1 };

typedef struct cd_config {
  int32_t n_layers;       /* decoder layers */
  int32_t d_model;        /* hidden width, multiple of 64 */
  int32_t n_q_heads;      /* query heads */
  int32_t n_kv_heads;     /* key/value heads (grouped-query attention) */
  int32_t head_dim;       /* 64 or 128 */
  int32_t n_experts;      /* routed experts, <= 256 */
  int32_t top_k;          /* experts per token, <= 16 */
  int32_t expert_hidden;  /* SwiGLU hidden width of each expert, mult. of 64 */
  int32_t shared_hidden;  /* hidden width of the shared SwiGLU FFN, 0 = none */
  int32_t vocab;          /* vocabulary size, multiple of 128 */
  int32_t canvas_len;     /* tokens per canvas / block (the pages: 256) */
  int32_t max_steps;      /* pass cap per block (the pages: 48) */
  float lock_threshold;   /* lock a position when max prob > this (0.9) */
  float stop_entropy;     /* stop when mean canvas entropy < this (0.005) */
  float rms_eps;          /* RMSNorm epsilon */
  float rope_theta;       /* rotary base; 0 disables rotary embedding */
  int32_t weight_dtype;   /* CD_F32, CD_BF16, CD_FP8 or CD_MXFP4 */
  int32_t max_requests;   /* requests denoised together (<= 256) */
  int32_t max_ctx;        /* KV capacity per request, tokens */
  int32_t max_prefill;    /* largest single prefill call, tokens */
  float attn_rescale_log2; /* attention softmax: the running row reference moves only when a
                              score exceeds it by more than this many powers of two (the
                              result is exact up to rounding for any value); 0 selects 8 */
  int32_t lock_rule;      /* CD_LOCK_MAXPROB or CD_LOCK_ENTROPY */
  float entropy_bound;    /* CD_LOCK_ENTROPY: lock when entropy <= this, nats (0.1) */
} cd_config;

/* Per-request result of one denoise pass, written to device memory. */
typedef struct cd_step_info {
  int32_t step;             /* pass index t (1-based) within the block */
  int32_t stop;             /* 1 when the adaptive stop or the cap fired */
  int32_t n_locked;         /* positions locked by the lock rule this pass */
  int32_t stable;           /* argmax equal to the previous pass's everywhere */
  int32_t canvas_is_argmax; /* the canvas fed to this pass equals its argmax */
  int32_t nonfinite;        /* a logit was NaN or infinite */
  int32_t after_stop;       /* 1: a pass ran after this block's stop had fired; it was
                               refused for this request (the rest of the record is that
                               of the stopping pass) */
  double mean_entropy;      /* canvas mean entropy, nats */
} cd_step_info;

typedef struct cd_ctx cd_ctx;

/* Sizes of the caller-allocated device buffers for a configuration.
 * Returns CD_ERR_INVALID_ARG / CD_ERR_UNSUPPORTED for shapes outside the
 * documented limits. */
int32_t cd_weights_bytes(const cd_config* cfg, size_t* bytes);
int32_t cd_state_bytes(const cd_config* cfg, size_t* bytes);

/* Bind a context to caller buffers (d_weights: cd_weights_bytes bytes,
 * d_state: cd_state_bytes bytes, both 256-byte aligned).  The context keeps
 * the pointers; the caller keeps the buffers alive until cd_ctx_destroy.
 * Enqueues nothing; the state is cleared by cd_reset on a stream. */
int32_t cd_ctx_create(const cd_config* cfg, void* d_weights, void* d_state, cd_ctx** out);
int32_t cd_ctx_destroy(cd_ctx* ctx);

/* Clear all request state (KV lengths, canvases) on the stream. */
int32_t cd_reset(cd_ctx* ctx, void* stream);

/* Fill the weight buffer with synthetic N(0, 0.02^2) weights.  Element n of
 * the [out][in] row-major tensor with id tau is 0.02*z, z from Box-Muller in
 * fp64 over Philox4x32-10(key = seed; counter = (n/4 low, n/4 high, tau,
 * 1 << 24)): words (r0, r1) give elements 4q, 4q+1 as
 * sqrt(-2 ln((r0+1)/2^32)) * (cos, sin)(2 pi r1/2^32), words (r2, r3) give
 * 4q+2, 4q+3; the value is rounded once to the storage format.  Tensor ids:
 * embedding 0, LM head 1, and for layer l, base 2 + l*(8 + 3E): +0 Wq, +1 Wk,
 * +2 Wv, +3 Wo, +4 router, +5+3e / +6+3e / +7+3e expert e gate / up / down,
 * +5+3E / +6+3E / +7+3E shared gate / up / down. */
int32_t cd_synth_weights(cd_ctx* ctx, uint64_t seed, void* stream);

/* Tensor kinds for cd_set_weight / cd_get_weight (logical [out][in] layout). */
enum { CD_W_EMBED = 0, CD_W_LM = 1, CD_W_Q = 2, CD_W_K = 3, CD_W_V = 4, CD_W_O = 5,
       CD_W_ROUTER = 6, CD_W_GATE = 7, CD_W_UP = 8, CD_W_DOWN = 9,
       CD_W_SHARED_GATE = 10, CD_W_SHARED_UP = 11, CD_W_SHARED_DOWN = 12 };

/* Copy one tensor between a caller fp32 device buffer d_logical
 * ([out][in] row-major) and the library's internal layout.  set rounds to the
 * storage format (fp8 tensors get fresh per-row scales); get returns the
 * stored values.  layer / expert are ignored where they do not apply. */
int32_t cd_set_weight(cd_ctx* ctx, int32_t kind, int32_t layer, int32_t expert,
                      const float* d_logical, void* stream);
int32_t cd_get_weight(cd_ctx* ctx, int32_t kind, int32_t layer, int32_t expert,
                      float* d_logical, void* stream);

/* ① Causal prefill: forward of n prompt ids (d_ids, int32, device) of
 * request req at positions P..P+n-1 with causal attention, appending their
 * keys/values to the KV cache; P grows by n.  Allowed when no canvas is
 * active; n <= max_prefill; CD_ERR_CAPACITY if P + n + canvas_len > max_ctx. */
int32_t cd_prefill(cd_ctx* ctx, int32_t req, const int32_t* d_ids, int32_t n, void* stream);

/* ② Canvas start for request req, block index `block`: token i is
 * floor(r0 * V / 2^32) with (r0..r3) = Philox4x32-10(key = seed;
 * counter = (i, 0, block, id)).  id is the request's index: its slot req,
 * unless the request was moved here (cd_move_request), which keeps the
 * index it had.  Allowed when no canvas is active. */
int32_t cd_init_canvas(cd_ctx* ctx, int32_t req, uint64_t seed, int32_t block, void* stream);

/* ③ One denoise pass over request slots 0..n_req-1, at least one of them
 * with an active canvas.  A slot without one rides along: its rows are
 * computed (keys/values land past its committed length, which needs
 * P + canvas_len <= max_ctx, else CD_ERR_CAPACITY) but none of its state
 * changes and its record is all zero.  Each active canvas gets a
 * bidirectional forward (keys = committed cache + canvas),
 * LM head to fp32 logits, then the sampler: per position entropy (nats),
 * argmax (ties to the lowest id) and max prob; lock when max prob >
 * lock_threshold (CD_LOCK_ENTROPY: when entropy <= entropy_bound; the
 * position takes the argmax), else re-noise with
 * Philox(seed; i, t, block, id), id the request index of the canvas start;
 * stop when t >= 2, mean entropy < stop_entropy and the argmax equals the
 * previous pass's at every position, or when t == max_steps.  d_info
 * receives n_req cd_step_info records.  CD_ERR_BAD_STATE if no slot has a
 * canvas or an active one has reached max_steps.  The explainer's step ④
 * commits the block once its stop has fired: a pass over a request whose
 * stop already fired in this block is refused for that request on the
 * device (its canvas, argmax and last record stay as they were; keys/values
 * of its canvas rows past P are rewritten, as for a ride-along slot), its
 * record is flagged after_stop, and the next cd_read_step_info or
 * cd_commit_block for it returns CD_ERR_BAD_STATE (cd_abort_canvas then
 * drops the canvas). */
int32_t cd_denoise_step(cd_ctx* ctx, int32_t n_req, cd_step_info* d_info, void* stream);

/* Drop the active canvas of request req without committing it (the
 * request returns to the state after its last commit).  Host-side only. */
int32_t cd_abort_canvas(cd_ctx* ctx, int32_t req);

/* Free slot req for a new prompt: P = 0, no canvas (an active one is
 * dropped) and an all-zero step record.  The cache rows it held are simply
 * overwritten later. */
int32_t cd_release(cd_ctx* ctx, int32_t req, void* stream);

/* Move the request in slot `from` (any state, also mid-block) to the free
 * slot `to` (P == 0, no canvas): its K/V region, canvas, last pass outputs,
 * step record and step state are copied on the stream, and `from` is
 * released.  Its
 * Philox streams keep their request index, so the move changes no result.
 * A server uses it to keep busy slots at the front: a pass over slots
 * 0..n-1 then computes no idle slot.  CD_ERR_BAD_STATE if `to` is not free. */
int32_t cd_move_request(cd_ctx* ctx, int32_t from, int32_t to, void* stream);

/* Copy n_req step records from device to host and wait for the stream.
 * Returns CD_ERR_BAD_STATE (the records are still copied) when a record is
 * flagged after_stop. */
int32_t cd_read_step_info(cd_ctx* ctx, const cd_step_info* d_info, int32_t n_req,
                          cd_step_info* h_info, void* stream);

/* ④ Commit the block of request req: the committed ids are the argmax of
 * the last pass (written to d_out_ids, canvas_len int32).  Their keys/values
 * come from a canvas-mode pass over the committed ids at positions
 * P..P+C-1, unless the last pass's canvas already equalled its argmax (then
 * that pass's keys/values are the same and are kept).  The cache below P is
 * never written.  P grows by canvas_len.  Synchronises the stream once.
 * CD_ERR_BAD_STATE (nothing committed) if no pass ran since the canvas
 * start, or a pass ran after the stop (record flagged after_stop). */
int32_t cd_commit_block(cd_ctx* ctx, int32_t req, int32_t* d_out_ids, void* stream);

/* Whole loop for one request (the canvas explainer, steps ① to ④, with the
 * next canvas conditioned on the committed blocks as in the MarkTechPost
 * article's "architecture" section, block-autoregressive diffusion):
 * optional prefill of n_prefix ids, then
 * n_blocks blocks of init -> passes to the adaptive stop -> commit.
 * d_out_ids receives n_blocks*canvas_len ids; h_steps_per_block (host,
 * n_blocks entries) the passes each block took.  Synchronises every pass.
 * CD_ERR_NUMERIC if the sampler met non-finite logits. */
int32_t cd_generate(cd_ctx* ctx, int32_t req, const int32_t* d_prefix, int32_t n_prefix,
                    int32_t n_blocks, uint64_t seed, int32_t* d_out_ids,
                    int32_t* h_steps_per_block, void* stream);

/* Batched loop over a queue of n_queue requests on n_slots slots (the
 * retire/admit loop of a server; the explainer's A/B guide and official
 * benchmark serve the model at several request concurrencies, and its
 * steps ① to ④ are run per request, each with its own adaptive stop).  Request q: prompt d_prefix +
 * h_prefix_off[q] (device ids; host offsets), h_prefix_len[q] >= 1 ids,
 * h_n_blocks[q] blocks, seed h_seeds[q]; its Philox streams are keyed by
 * request index q (not by slot), so its output is that of cd_generate of
 * the same prompt and seed run as request q (up to the rounding order of a
 * batched pass: split counts depend on the batch).  Slots 0..n_slots-1 are released
 * first and take requests in queue order; each pass denoises every slot up
 * to the highest busy one (idle ones ride along); a block that stops is
 * committed to d_out + h_out_off[q] + b*canvas_len and its slot starts the
 * next block, or, after the last, takes the next queued request.  Once the
 * queue is empty, busy requests move down into idle slots (as
 * cd_move_request) so that the passes shrink with the work left.
 * h_steps (host) receives the passes per block, request after request
 * (sum of h_n_blocks entries).  Synchronises every pass; every slot is
 * released on return, also when the call fails (argument errors excepted:
 * they change nothing).  CD_ERR_NUMERIC on non-finite logits. */
int32_t cd_serve(cd_ctx* ctx, int32_t n_queue, const int32_t* d_prefix, const int64_t* h_prefix_off,
                 const int32_t* h_prefix_len, const int32_t* h_n_blocks, const uint64_t* h_seeds,
                 int32_t n_slots, int32_t* d_out, const int64_t* h_out_off, int32_t* h_steps,
                 void* stream);

/* Sampler alone on caller logits (the canvas explainer, step ③: per
 * position entropy, argmax and lock / re-noise, then the adaptive stop on
 * the canvas mean entropy and argmax stability; the MarkTechPost article,
 * "how text diffusion works": low-confidence tokens are re-noised and
 * predicted again).  Logits rows x vocab fp32, device, rows a
 * multiple of canvas_len, treated as rows/canvas_len requests at pass `step`
 * of block `block`, request indices req0, req0+1, ...  d_prev_argmax (rows
 * int32, may be NULL: then no stability) is the previous pass's argmax.
 * Outputs (device, rows entries each): d_tokens next canvas ids, d_argmax,
 * d_lock (uint8), d_entropy (f64), d_pmax (f64); d_info one record per
 * request.  d_workspace: cd_sample_workspace_bytes bytes. */
int32_t cd_sample_workspace_bytes(int32_t rows, int32_t vocab, size_t* bytes);
int32_t cd_sample_step(const cd_config* cfg, const float* d_logits, int32_t rows,
                       const int32_t* d_prev_argmax, uint64_t seed, int32_t step,
                       int32_t block, int32_t req0, int32_t* d_tokens, int32_t* d_argmax,
                       uint8_t* d_lock, double* d_entropy, double* d_pmax,
                       cd_step_info* d_info, void* d_workspace, void* stream);

/* cd_sample_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The chunk partials go to a fixed
 * buffer inside the library (one per GPU, 1 MiB, held until the process
 * ends): rows * chunks must not exceed 65536, chunks = the number of
 * 8192-logit pieces of a row (32 at vocab 262144, so at most 2048 rows);
 * larger calls return CD_ERR_CAPACITY with nothing enqueued.  The buffer is
 * fully written before it is read, so nothing needs clearing between calls;
 * calls that overlap in time on one GPU (other streams, other threads) share
 * the buffer and race.  No device memory is allocated or freed.  Arguments,
 * outputs and results are those of cd_sample_step. */
int32_t cd_sample_step_noalloc(const cd_config* cfg, const float* d_logits, int32_t rows,
                               const int32_t* d_prev_argmax, uint64_t seed, int32_t step, int32_t block,
                               int32_t req0, int32_t* d_tokens, int32_t* d_argmax, uint8_t* d_lock,
                               double* d_entropy, double* d_pmax, cd_step_info* d_info, void* stream);

/* Internal buffers exposed for inspection (device pointers into d_state). */
enum { CD_BUF_LOGITS = 0,   /* f32 [max_requests*C][vocab] last pass logits */
       CD_BUF_CANVAS = 1,   /* i32 [max_requests][C] current canvas */
       CD_BUF_ARGMAX = 2,   /* i32 [max_requests][C] last pass argmax */
       CD_BUF_ENTROPY = 3,  /* f64 [max_requests][C] last pass entropies */
       CD_BUF_PMAX = 4,     /* f64 [max_requests][C] last pass max probs */
       CD_BUF_LOCK = 5,     /* u8 [max_requests][C] last pass lock mask */
       CD_BUF_KCACHE = 6,   /* [max_requests][L][Hkv][max_ctx][dh] keys (act type) */
       CD_BUF_VCACHE = 7,   /* [max_requests][L][Hkv][dh][max_ctx] values (act type) */
       CD_BUF_HIDDEN = 8 }; /* f32 [tokens][d] residual stream after the last layer */
int32_t cd_get_buffer(cd_ctx* ctx, int32_t which, void** d_ptr, size_t* bytes);

/* The configuration a context was created with (host copy). */
int32_t cd_get_config(cd_ctx* ctx, cd_config* out);

/* Committed length P of a request (host mirror; no synchronisation). */
int32_t cd_get_length(cd_ctx* ctx, int32_t req, int32_t* P);

/* Optional parity trace: when set, every forward (prefill, denoise pass,
 * commit recompute) over T rows writes each layer's input residual rows
 * (f32 [L][T][d]), its routing (i32 ids / f32 gates [L][T][top_k]) and its
 * residual rows after the attention block, the input of the MoE block's
 * RMSNorm (f32 [L][T][d]), to these caller buffers, sized for the largest T
 * used.  NULL pointers switch a part off; cd_set_trace(ctx, NULL, NULL,
 * NULL, NULL) switches tracing off. */
int32_t cd_set_trace(cd_ctx* ctx, float* d_h_layers, int32_t* d_topk_ids, float* d_topk_gates,
                     float* d_h_mid_layers);

/* Graph replay of denoise passes (on by default).  The launches of one pass
 * depend on the host only through the first slot, the number of slots, the
 * longest context among them and which of them hold a canvas; the first pass
 * with a new combination of these is captured into a HIP graph on a stream of
 * the library's own and every later one replays it with one launch on the
 * caller's stream (at most 16 graphs are kept per context, least recently
 * used dropped first).  The results are the same as those of the launches
 * made one by one.  Passes run while profiling (cd_profile) or tracing
 * (cd_set_trace) is on, and passes of a context where a capture failed, are
 * launched one by one.  enable = 0 releases the context's graphs (waiting
 * for the device) and launches every later pass one by one.  Not thread-safe
 * per context, like every other call. */
int32_t cd_set_graphs(cd_ctx* ctx, int32_t enable);

/* Per-kernel timing with HIP events recorded on the call's stream around
 * every launch (enable = 1 starts a fresh window, 0 stops recording).
 * cd_profile_read waits for the recorded events and returns, per kernel
 * class, the summed milliseconds and the number of launches (arrays of
 * n_classes entries, at most CD_PROF_CLASSES). */
enum { CD_PROF_EMBED = 0, CD_PROF_RMSNORM, CD_PROF_QKV, CD_PROF_ATTN, CD_PROF_ATTN_MERGE, CD_PROF_O_PROJ,
       CD_PROF_ROUTER, CD_PROF_ROUTE, CD_PROF_EXPERT_GU, CD_PROF_EXPERT_DOWN, CD_PROF_COMBINE,
       CD_PROF_SHARED_GU, CD_PROF_SHARED_DOWN, CD_PROF_LM_HEAD, CD_PROF_SAMPLER_PART, CD_PROF_SAMPLER_FINAL,
       CD_PROF_OTHER, CD_PROF_QUANT, CD_PROF_CLASSES };
int32_t cd_profile(cd_ctx* ctx, int32_t enable);
int32_t cd_profile_read(cd_ctx* ctx, double* ms, int32_t* launches, int32_t n_classes);

/* Message for the calling thread's last error ("" if none). */
const char* cd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CD_H_ */
