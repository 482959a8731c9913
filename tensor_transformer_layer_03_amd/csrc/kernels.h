// Internal launchers of the gfx950 kernels (host-callable, enqueue only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl {

enum DType { DT_F32 = 0, DT_BF16 = 1 };
inline size_t dtype_size(int dt) { return dt == DT_BF16 ? 2 : 4; }

// ------------------------------------------------------------------ tracing
// Optional per-launch event timing (see tpl_trace_enable in tp_layer.h).
enum KernelId {
  K_GEMM_NT = 0, K_GEMM_NN, K_GEMM_TN, K_ATTN_FWD, K_ATTN_BWD_PRE, K_ATTN_BWD_DQ,
  K_ATTN_BWD_DKDV, K_LN_FWD, K_LN_BWD, K_LN_BWD_COLS, K_COLSUM, K_COLSUM_FINAL,
  K_PARTIAL_SUM, K_XENT_STATS, K_XENT_FINISH, K_XENT_DLOGITS, K_XENT_MERGE, K_EMB_FWD, K_EMB_SORT, K_EMB_BWD,
  K_ROWS_GATHER, K_ROWS_EXPAND, K_GEMM_PAIR, K_ATTN_BWD_PAIR,
  K_COUNT
};
const char* kernel_name(int id);
struct TraceScope {
  int slot;
  hipStream_t stream;
  TraceScope(int kernel_id, hipStream_t s, double work = 0.0);
  ~TraceScope();
};

// ------------------------------------------------------------------ GEMM
// C[M][N] = sum_k A(m,k) B(n,k) with an epilogue.
enum Epilogue {
  EPI_NONE = 0,       // C = acc
  EPI_BIAS = 1,       // C = acc + bias[n]
  EPI_BIAS_GELU = 2,  // u = acc + bias[n]; C = GeLU'(u); C2 = GeLU(u)
  EPI_DGELU = 3,      // C = acc * C2[m][n]  (C2 holds GeLU'(u) from EPI_BIAS_GELU, read-only)
  EPI_XENT = 4        // C = acc (logits); per-row (max, sum exp) of each tile column
};
struct GemmDesc {
  int dtype;          // storage type of A, B (and C unless c_f32)
  bool a_kmajor;      // A(m,k) at A[m*lda+k] (true) or A[k*lda+m] (false)
  bool b_kmajor;      // B(n,k) at B[n*ldb+k] (true) or B[k*ldb+n] (false)
  int epi;
  bool c_f32;         // C is fp32 (weight gradients) instead of the storage type
  int64_t M, N, K;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  void* C; int64_t ldc;
  void* C2; int64_t ldc2;
  const void* bias;
  // split-K workspace (or NULL: never split) and its capacity in floats; fp32
  // weight gradients need gemm_ws_floats, a bf16 dgrad with few tiles and a
  // long K uses whatever capacity is given (all splits as fp32 partials)
  float* ws;
  size_t ws_floats;
  // EPI_XENT only: targets [M] (global ids), v0 = first vocabulary id of the
  // columns, xpart = per-tile (max, sum exp) [tile column][M][2]
  const int32_t* targets; int64_t v0; float* xpart;
  // EPI_DGELU only (or NULL): column sums of the rounded output per block of
  // half a tile's rows, [gemm_colpart_chunks()][N], blocks in row order
  float* colpart;
};
hipError_t launch_gemm(const GemmDesc& d, hipStream_t s);
// A block's activation-gradient product dg (A K-major, B MN-major, storage
// type out, EPI_NONE or EPI_DGELU) and its weight-gradient product wg (both
// MN-major, fp32 out, ldc == N) in one launch on 256x256 tiles (or 128x128
// ones for an EPI_NONE dg: plan.tile), wg and an EPI_NONE dg possibly split
// over K inside it. gemm_pair_plan says whether
// that beats two launches (and fills *plan either way); the launch then needs
// gemm_pair_ws_floats of workspace: an EPI_DGELU dg's
// gemm_pair_colpart_chunks(dg.M) column partials (dg.colpart is ignored:
// they go to ws) or a split dg's fp32 slices first, then wg's split slices.
struct PairPlan { int dg_splits, dg_kchunk, wg_splits, wg_kchunk; int tile = 256; };   // tile: 256 or 128
bool gemm_pair_plan(const GemmDesc& dg, const GemmDesc& wg, PairPlan* plan);
int64_t gemm_pair_colpart_chunks(int64_t M);
size_t gemm_pair_ws_floats(const GemmDesc& dg, const GemmDesc& wg, const PairPlan& plan);
// Column-sum work that launch_gemm_pair runs inside the launch summing wg's
// split slices (a launch fewer), or in a launch of its own when there is no
// such sum: TAIL_COLSUM_FINAL: out[c] = sum of the nchunks partial rows
// ws[chunk][c] in chunk order; TAIL_COLSUM_PARTIALS: the per-32-row column
// partials of the bf16 [rows][cols] operand X (row stride ld) into ws
// ([ceil(rows/32)][cols], colsum_ws_floats). Its buffers must not overlap the
// pair's workspace.
enum { TAIL_NONE = 0, TAIL_COLSUM_FINAL = 1, TAIL_COLSUM_PARTIALS = 2 };
struct PairTail {
  int kind;
  const void* X;
  int64_t ld, rows, nchunks;
  int cols;
  float* ws;
  float* out;
};
hipError_t launch_gemm_pair(const GemmDesc& dg, const GemmDesc& wg, const PairPlan& plan, float* ws, hipStream_t s,
                            const PairTail* tail = nullptr);
// Floats of split-K workspace the product (M, N, K) with both operands MN-major
// and an fp32 output takes (0: it is not split).
size_t gemm_ws_floats(int dtype, int64_t M, int64_t N, int64_t K);
// Workspace floats a bf16 activation-gradient product (A K-major, B MN-major,
// M x N output, depth K) uses when it splits over K (0 when it does not).
size_t gemm_dgrad_ws_floats(int dtype, int64_t M, int64_t N, int64_t K);
// Row blocks of the column partials an EPI_DGELU product writes to colpart.
int64_t gemm_colpart_chunks(int dtype, int64_t M, int64_t N);
// Number of tile columns of the logits product with the fused statistics
// epilogue (0: this shape/dtype takes the unfused path), and the floats of
// per-tile statistics it needs at most.
int xent_gemm_tile_cols(int dtype, int64_t M, int64_t N);
// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();
size_t xent_part_floats(int64_t M, int64_t N);

// ------------------------------------------------------------------ attention
struct AttnDesc {
  int dtype, batch, heads, seq, head_dim, causal;
  const void* qkv; int64_t ld_qkv;  // [N][3*h_r]: Q heads | K heads | V heads
  void* ctx; int64_t ld_ctx;        // [N][h_r]
  float* lse;                       // [batch][heads][seq]
  // backward
  const void* dctx;                 // [N][h_r]
  void* dqkv;                       // [N][3*h_r]
  float* delta;                     // [batch][heads][seq]
};
hipError_t launch_attn_fwd(const AttnDesc& d, hipStream_t s);
hipError_t launch_attn_bwd(const AttnDesc& d, hipStream_t s);

// ------------------------------------------------------------------ row / column ops
hipError_t launch_layernorm_fwd(int dtype, const void* x, const void* g, const void* b, void* y,
                                float* mu, float* rstd, int64_t rows, int cols, float eps,
                                hipStream_t s);
// dx = dy + LN_bwd(dsum); column partials of (dsum*xhat, dsum, dy) into ws.
hipError_t launch_layernorm_bwd(int dtype, const void* dy, const void* dsum, const void* x,
                                const float* mu, const float* rstd, const void* g, void* dx,
                                float* d_g, float* d_b, float* d_bout, float* ws, int64_t rows,
                                int cols, hipStream_t s);
size_t layernorm_bwd_ws_floats(int64_t rows, int cols);
// out[c] = sum_r X[r][c] over rows (two deterministic stages, ws partials).
hipError_t launch_colsum(int dtype, const void* X, int64_t ld, int64_t rows, int cols, float* out,
                         float* ws, hipStream_t s);
size_t colsum_ws_floats(int64_t rows, int cols);
// out[c] = sum over chunks of ws[chunk][c] (fixed order).
hipError_t launch_colsum_final(const float* ws, int64_t nchunks, int cols, float* out, hipStream_t s);
hipError_t launch_partial_sum(int dtype, const void* const* parts, int n, const void* bias,
                              const void* residual, void* out, int64_t rows, int cols,
                              hipStream_t s);

// ------------------------------------------------------------------ cross-entropy
// stats[row] = fixed-order log-sum-exp merge of the T tile (max, sum exp) pairs
// of xpart [T][rows][2], and the target logit read from logits.
hipError_t launch_xent_merge(int dtype, const float* xpart, int tcols, int64_t rows, const void* logits, int vr,
                             const int32_t* targets, int64_t v0, float* stats, hipStream_t s);
hipError_t launch_xent_stats(int dtype, const void* logits, int64_t rows, int vr,
                             const int32_t* targets, int64_t v0, float* stats, hipStream_t s);
hipError_t launch_xent_finish(const float* const* all_stats, int t, int64_t rows,
                              const uint8_t* mask, float* lse, float* loss_rows, float* loss,
                              hipStream_t s);
hipError_t launch_xent_dlogits(int dtype, void* logits, int64_t rows, int vr,
                               const int32_t* targets, int64_t v0, const uint8_t* mask,
                               const float* lse, const float* loss, float dloss, hipStream_t s);

// ------------------------------------------------------------------ input embedding
// Workspace bytes of the backward (sort keys / values twice, segment starts).
size_t embedding_ws_bytes(int64_t rows, int vr);
// The allocation-free backward's workspace: a device array of
// kNoAllocScratchBytes per GPU; *ptr = its address on the current device
// (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);
// Row gather / expand of a masked loss's rows (row_bytes a multiple of 4):
// gather: dst[i] = src[rows[i]] (i < n; an index outside [0, n_src) gives zeros);
// expand: dst[r] = src[pos[r]] if 0 <= pos[r] < n_src, else zeros (r < n_dst).
hipError_t launch_rows_gather(const void* src, const int32_t* rows, int64_t n, int64_t n_src, int64_t row_bytes,
                              void* dst, hipStream_t s);
hipError_t launch_rows_expand(const void* src, const int32_t* pos, int64_t n_dst, int64_t n_src, int64_t row_bytes,
                              void* dst, hipStream_t s);
hipError_t launch_embedding_fwd(int dtype, const int32_t* tokens, const void* emb, void* out, int64_t rows, int cols,
                                int64_t v0, int vr, hipStream_t s);
hipError_t launch_embedding_bwd(int dtype, const int32_t* tokens, const void* d_out, float* d_emb, int64_t rows,
                                int cols, int64_t v0, int vr, void* ws, hipStream_t s);

}  // namespace tpl
