// Kernel argument structs and host launchers (internal to libcd).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cd {

// ---------------------------------------------------------------------------
// Packed weight layout.  A weight W[N][K] (output rows x contraction) is
// stored as 16-row x KF-column fragment tiles of 1024 bytes: tile (nt, kt)
// at byte ((nt * (K/KF)) + kt) * 1024; lane l of a wave holds the 16 bytes of
// row nt*16 + l%16, columns kt*KF + (l/16)*(KF/4) + [0, KF/4).  KF = 64 / size
// of the element (fp32 16, bf16 32, fp8 64).  One 16-byte load per lane then
// fetches a whole tile as one contiguous 1 KB wave access, already in MFMA
// operand order.  N is padded to a multiple of 32 (zero rows).
//
// MXFP4 (dtype 3, routed experts only): E2M1 codes, two per byte (the even
// column in the low nibble), in 16-row x 64-column tiles of 512 bytes; lane l
// holds the 8 bytes of row nt*16 + l%16, columns kt*64 + (l/16)*16 + [0, 16).
// Each row has one E8M0 scale (2^(byte - 127)) per 32 columns; the scales
// follow the tiles in groups of four k-tiles: the scale of row r, column c
// (k-tile kt = c / 64) is byte ((nt * KT4 + kt / 4) * 32 + (r % 16) * 2 +
// (c % 64) / 32) * 4 + kt % 4 after them, KT4 = ceil(KT / 4), so one dword
// per lane (lane l: index (l % 16) * 2 + l / 32) holds its scales of four
// consecutive k-tiles.
// ---------------------------------------------------------------------------
__host__ __device__ inline int esize(int dt) { return dt == 0 ? 4 : dt == 1 ? 2 : 1; }
__host__ __device__ inline int kfrag(int dt) { return 64 / esize(dt); }
// bytes of the packed tiles (MXFP4: codes only; the scales follow at this offset)
__host__ __device__ inline int64_t packed_bytes(int64_t Npad, int64_t K, int dt) {
  return dt == 3 ? Npad * K / 2 : Npad * K * esize(dt);
}
// packed bytes including MXFP4 scales
__host__ __device__ inline int64_t packed_total(int64_t Npad, int64_t K, int dt) {
  return packed_bytes(Npad, K, dt) + (dt == 3 ? (Npad / 16) * ((K / 64 + 3) / 4) * 128 : 0);
}
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Row permutations applied when packing.
enum { PERM_NONE = 0, PERM_QKV = 1, PERM_GU = 2 };

enum { EPI_F32 = 0, EPI_ROWS = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_QKV = 4 };

struct GemmArgs {
  // activations: row-major [rows][ldx], element type = act dtype
  const void* X;
  int64_t ldx;
  const int32_t* row_map;  // tile row -> source row of X, or null (identity)
  // weights: packed tiles, one block of tiles per group
  const uint8_t* W;
  int64_t w_gstride;       // bytes between groups
  const float* wscale;     // fp8 per-row scales [group][Npad], or null
  int64_t s_gstride;
  int64_t mx_off;          // MXFP4: bytes from a group's tiles to its E8M0 scales
  int K, Nt, N, n_chunks;  // Nt = packed 16-row tiles; N = logical outputs
  // work tiles: grouped (device table) or dense (M rows)
  // [max_tiles][4]: group, row0, rows, and (index of the tile inside its
  // group) | (the group's tile count << 16); tiles are sorted by group
  const int32_t* tiles;
  const int32_t* n_tiles;  // device count for grouped launches
  int max_tiles;
  int M;
  int chunk_major;
  int ksplit;              // split of the contraction (EPI_F32 only); 0 or 1 = none
  int64_t y_kstride;       // elements between the fp32 partial outputs of the splits
  // epilogue
  void* Y;
  int64_t ldy;
  // EPI_QKV
  void* kc;
  void* vc;
  int64_t kv_req_stride;   // elements between requests (same layer)
  int max_ctx, Hq, Hkv, dh;
  int rows_per_req;
  const int32_t* pos0;     // per request: position of its row 0
  int pos0_stride;         // int32 stride between requests in pos0
  const float* rope_cs;    // [max_ctx][dh/2] (cos, sin) pairs, or null
  float q_scale;           // EPI_QKV: factor on the query outputs before their rounding
  const float* xscale;     // fp8 activations (launch_gemm_x8): scale of each source row of X
};

// Both launchers return 0, or CD_ERR_UNSUPPORTED (-5) for an MXFP4 launch with
// a split contraction (its scale dwords are indexed from k-tile 0).
int launch_gemm(int wdt, int adt, int mt, int epi, const GemmArgs& a, hipStream_t s);
// 256-row work items (128-row halves with fp8 weights), activations staged in
// LDS (a.ksplit > 1: EPI_F32 partials)
int launch_gemm_x(int wdt, int adt, int epi, const GemmArgs& a, hipStream_t s);
// fp8 (DT_FP8) or MXFP4 (DT_FP4, EPI_SWIGLU / EPI_ROWS) weights x fp8
// activations (E4M3 rows of X, one fp32 scale per row in a.xscale) on the
// 16x16x128 f8f6f4 MFMA, 128-row work items (two per 256-row tile or slab,
// two workgroups per CU); every epilogue but EPI_F32, no split contraction.
// 0 or CD_ERR_UNSUPPORTED.
int launch_gemm_x8(int wdt, int epi, const GemmArgs& a, hipStream_t s);
// q = E4M3 rows of bf16 x with one scale per row (amax / 448), for
// launch_gemm_x8; rows at or past *n_dev (if not null) are skipped.  K a
// multiple of 64, at most 4096.  0 or CD_ERR_UNSUPPORTED.
int launch_quant_fp8(const void* x, int64_t ldx, int n, int K, uint8_t* q, int64_t ldq, float* s,
                     const int32_t* n_dev, hipStream_t st);
// ---- weight synthesis / packing --------------------------------------------
struct PackDesc {
  uint8_t* dst;        // packed tiles (or row-major for embedding)
  float* scale;        // fp8 per-row scales or null
  int64_t mx_off;      // MXFP4: bytes from dst to the E8M0 scales
  int dt;              // storage dtype
  int perm;            // PERM_*
  int Npad, K;
  int rowmajor;        // 1: plain row-major [N][K] (embedding)
  int n_rows_src[3];   // logical rows of each source tensor
  int Hq, Hkv, dh;     // PERM_QKV
  uint32_t tau[3];     // tensor ids of the sources (synthesis)
  int only_sel;        // >= 0: touch only rows of that source (pack / unpack)
};
void launch_synth(const PackDesc& d, int n_groups, int64_t dst_gstride, int64_t scale_gstride,
                  int tau_gstride, uint64_t seed, hipStream_t s);
void launch_pack(const PackDesc& d, const float* src0, const float* src1, const float* src2,
                 hipStream_t s);
void launch_unpack(const PackDesc& d, float* out0, float* out1, float* out2, hipStream_t s);

// ---- attention ---------------------------------------------------------------
// attention work item: 256 query rows (heads of a KV group x tokens), keys in
// blocks of 64, at most 16 key splits
constexpr int ATT_QR = 256, ATT_KB = 64, ATT_MAX_SPLIT = 16;
struct AttnArgs {
  const void* Q;          // [rows][Hq*dh] act
  void* O;                // [rows][Hq*dh] act
  const void* kc;         // layer base of request 0: [Hkv][max_ctx][dh]
  const void* vc;         // layer base of request 0: [Hkv][dh][max_ctx]
  int64_t kv_req_stride;
  int max_ctx, Hq, Hkv, dh;
  int rows_per_req, n_req;
  const int32_t* pos0;    // per-request position of row 0 (= committed length)
  int pos0_stride;
  int causal;             // 0: keys [0, pos0+rows) all visible; 1: key <= query pos
  float rescale_log2;     // lazy softmax: the row reference moves when a score exceeds it by more (log2)
  int n_split, split_len; // key range split
  void* part_o;           // [n_split][rows_total][Hq][dh] unnormalised partial O: f32, or bf16
                          // when the activations are bf16
  float* part_ml;         // [n_split][rows_total][Hq][2] f32
  int q_blocks;           // query blocks of ATT_QR/(Hq/Hkv) tokens per request
};
void launch_attention(int adt, const AttnArgs& a, hipStream_t s);

// ---- MoE routing ----------------------------------------------------------------
constexpr int MAX_ROUTER_SPLIT = 16;   // contraction splits of the router GEMM
struct RouteArgs {
  const float* logits;   // [nsplit][T][E] router logit partials (summed in split order)
  int nsplit;
  int T, E, k;
  int32_t* topk_id;      // [T][k]
  float* topk_gate;      // [T][k]
  int32_t* blk_cnt;      // [n_blk][E]
  int32_t* seg_off;      // [E+1] padded segment offsets
  int32_t* row_map;      // [max_rows] token of each permuted row, -1 pad
  int32_t* slot;         // [T][k] permuted row of assignment (t, j)
  int32_t* tiles;        // [max_tiles][4], as GemmArgs::tiles
  int32_t* n_tiles;      // [1]
  int mrows;             // rows per GEMM tile
  int max_rows, max_tiles;
  int32_t* trace_ids;    // optional
  float* trace_gates;
};
void launch_route(const RouteArgs& a, hipStream_t s);

// ---- misc ---------------------------------------------------------------------------
void launch_embed(int edt, const void* E, const int32_t* ids, int T, int V, int d, float* h, hipStream_t s);
// u[t] = RMSNorm(h[t]) (unit gain) in the activation type; with bf16
// activations, d <= 4096 and q8 given, also the E4M3 rows of u (row stride d)
// and their scales s8, exactly as launch_quant_fp8 would make them from u
void launch_rmsnorm(int adt, const float* h, int T, int d, float eps, void* u, hipStream_t s, uint8_t* q8 = nullptr,
                    float* s8 = nullptr);
void launch_rope_table(float* cs, int max_ctx, int dh, float theta, hipStream_t s);
// h[t] += sum_j gate[t][j] * Yp[slot[t][j]] (choice order) + add[t] (fp32 row, or null);
// when u is not null also u[t] = RMSNorm(h[t]) (unit gain) in the activation type,
// and (bf16, d <= 4096, q8 given) its E4M3 rows and scales as launch_rmsnorm
void launch_combine(int adt, const void* Yp, const int32_t* slot, const float* gate, const float* add, int T, int k,
                    int d, float* h, void* u, float eps, hipStream_t s, uint8_t* q8 = nullptr, float* s8 = nullptr);
void launch_attn_merge(int adt, const AttnArgs& a, hipStream_t s);
void launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

// per-request device state
struct ReqDev {
  int32_t P;        // committed length
  int32_t t;        // passes done in the current block
  int32_t block;
  int32_t rid;      // request index that keys the Philox stream (the slot, unless a batched loop assigns one)
  uint64_t seed;
  int32_t stopped;  // the adaptive stop (or the cap) fired in the current block; cleared by the canvas start
  int32_t pad_;
};
// canvas of slot req for block `block`, its Philox stream keyed by rid
void launch_init_canvas(int32_t* canvas, ReqDev* rq, int req, int C, int V, uint64_t seed,
                        int block, int rid, hipStream_t s);
// P += dP for slot req
void launch_advance(ReqDev* rq, int req, int dP, hipStream_t s);
void launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t s);
// n 32-bit words at p set to zero (a fill kernel, not a memset node)
void launch_zero_u32(void* p, int64_t n, hipStream_t s);

// ---- sampler ------------------------------------------------------------------------
struct SampleArgs {
  const float* logits;   // [rows][V]
  int rows, V, C;
  int n_chunks, chunk;   // chunk = V / n_chunks floats
  float4* part;          // [rows][n_chunks] (m, S, U, idx as float bits)
  const int32_t* prev_a; // [rows] or null
  int32_t* tokens;       // [rows] next canvas
  int32_t* argmax;       // [rows]
  uint8_t* lock;         // [rows]
  double* entropy;       // [rows]
  double* pmax;          // [rows]
  void* info;            // cd_step_info per request
  const int32_t* canvas_in;  // canvas fed to this pass (for canvas_is_argmax), or null
  ReqDev* rq;            // per-request state of request req0 + i, or null
  uint64_t active[4];    // with rq: bit r set when request r has an active canvas (others are left untouched)
  uint64_t seed;         // used when rq is null
  int step, block, req0; // used when rq is null
  int max_steps;
  float lock_th, stop_H;
  int lock_rule;         // 0: max prob > lock_th; 1: entropy <= ent_bound
  float ent_bound;
};
void launch_sampler_part(const SampleArgs& a, hipStream_t s);
// Partials held by the library's own fixed device buffer (allocation-free
// sampler entry point): at most this many (row, chunk) partials, 16 bytes each.
constexpr int SAMPLER_SCRATCH_PARTIALS = 65536;
// That buffer's device address on the current device (looked up once per
// device with hipGetSymbolAddress); 0, or CD_ERR_HIP (-4) on failure.
int sampler_scratch(float4** out);
void launch_sampler_final(const SampleArgs& a, hipStream_t s);

}  // namespace cd
