/*
 * tp_layer.h -- C ABI of the MI355X (gfx950) tensor-parallel transformer-layer
 * shard library (libtplayer.so).
 *
 * What it computes: one tensor-parallel rank's share of a Megatron-LM
 * transformer layer, forward and backward, and the vocabulary-parallel output
 * embedding fused with cross-entropy.
 *   - podcast page "Megatron-LM's parallelism" (xiaoyuzhoufm.com), Outline:
 *     intra-layer parallelism; MLP weights split by columns then rows;
 *     K/Q/V split by attention heads; two all-reduces per module, four per
 *     layer forward+backward; output embedding split along the vocabulary with
 *     the loss fused in; dropout/LayerNorm/residual duplicated per rank;
 *     LayerNorm/residual placement (pre-LN) for large models.
 *   - guide page "From Transformer splitting to communication optimisation"
 *     (rkmt.cn): section 3.1 (fc1 column-parallel so GeLU needs no exchange,
 *     fc2 row-parallel on fc1's local output), section 3.2 (QKV split by heads,
 *     output projection split by rows), section 3.3 (vocabulary-split output
 *     layer with the gather deferred into the cross-entropy).
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless marked "host".
 *   - Storage type is desc->dtype (fp32 or bf16); all accumulation is fp32.
 *     Weight/bias gradients, LayerNorm/softmax/xent statistics are fp32.
 *   - Activations are row-major [N][cols] with N = micro_batch*seq rows in
 *     batch-major order (row n = b*seq + s).
 *   - Weights use the nn.Linear layout W[out][in] (y = x W^T + b). Rank r owns
 *     heads [r*a_r, (r+1)*a_r), ffn columns [r*f_r, (r+1)*f_r) and vocabulary
 *     ids [r*V_r, (r+1)*V_r) (a_r = heads/tp, f_r = ffn/tp, V_r = vocab/tp,
 *     h_r = a_r*head_dim).
 *   - Ownership: the caller owns every buffer. The library never allocates or
 *     frees device memory, never keeps a pointer after a call returns and never
 *     synchronises: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream). Calls are reentrant; buffers passed to concurrent calls
 *     must not overlap. The profiling helpers tpl_trace_* are the one
 *     exception: while enabled they keep process-wide state (an event pool
 *     and its records), create HIP events, and tpl_trace_read synchronises
 *     on the recorded events; the computation calls never depend on them.
 *     Launch plans (tile shapes, splits over K, paired launches) are chosen
 *     on the host from the shapes and the device's compute-unit count and
 *     memoized per shape: the same call on the same device always launches
 *     the same kernels, so results are bitwise repeatable.
 *   - Errors: arguments are validated on the host before anything is
 *     launched; a failed check returns TPL_ERR_INVALID_ARG (bad value, null or
 *     misaligned pointer) or TPL_ERR_UNSUPPORTED (valid but not implemented,
 *     e.g. head_dim not in {64, 96, 128}) and writes nothing. A launch failure
 *     returns TPL_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation. Pointers must be 16-byte aligned.
 *   - Shape rules: hidden == heads*head_dim; tp divides heads, ffn and vocab;
 *     0 <= rank < tp; head_dim in {64, 96, 128}; hidden, ffn/tp and vocab/tp
 *     multiples of 8; seq >= 1, micro_batch >= 1; N*max(cols) < 2^31.
 */
#ifndef TP_LAYER_H_
#define TP_LAYER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TPL_OK = 0,
  TPL_ERR_INVALID_ARG = 1,
  TPL_ERR_UNSUPPORTED = 2,
  TPL_ERR_HIP = 3
} tpl_status;

typedef enum { TPL_F32 = 0, TPL_BF16 = 1 } tpl_dtype;
typedef enum { TPL_BLOCK_ATTN = 0, TPL_BLOCK_MLP = 1 } tpl_block;
typedef enum { TPL_BWD_SHARD = 0, TPL_BWD_REPLICATED = 1, TPL_BWD_SHARD_RECOMPUTE = 2 } tpl_bwd_phase;
typedef enum { TPL_XENT_LOCAL = 0, TPL_XENT_FINISH = 1 } tpl_xent_phase;

/* The problem statement of the pages: hidden size, heads, TP degree and rank,
 * sequence, micro-batch, vocabulary. */
typedef struct {
  int32_t hidden;       /* h = heads*head_dim */
  int32_t heads;        /* a (whole layer) */
  int32_t head_dim;     /* d in {64, 96, 128} */
  int32_t ffn;          /* f (whole layer), usually 4h */
  int32_t tp;           /* t, the tensor-parallel degree */
  int32_t rank;         /* this rank, 0 <= rank < t */
  int32_t seq;          /* s */
  int32_t micro_batch;  /* b */
  int32_t vocab;        /* V (whole vocabulary) */
  int32_t causal;       /* 1: key j visible to query i iff j <= i (GPT); 0: no mask (BERT) */
  int32_t dtype;        /* tpl_dtype: storage type of activations and weights */
  float ln_eps;         /* LayerNorm epsilon (1e-5 in every workload) */
} tpl_desc;

/* One block's parameters on this rank, storage dtype.
 *   ATTN: w_in = W_qkv [3*h_r][h], rows = [Q rows of the rank's heads; K rows; V rows],
 *         head-major with head_dim rows per head; b_in = b_qkv [3*h_r];
 *         w_out = W_o [h][h_r] (the columns of the rank's heads).
 *   MLP:  w_in = W_1 [f_r][h], b_in = b_1 [f_r]; w_out = W_2 [h][f_r].
 *   ln_g, ln_b: [h] (replicated). The row-parallel output bias is not here: it
 *   is added once, after the partial sum (shard_partial_sum's `bias`). */
typedef struct {
  const void* ln_g;
  const void* ln_b;
  const void* w_in;
  const void* b_in;
  const void* w_out;
} tpl_block_params;

/* fp32 gradients, overwritten (never accumulated).
 *   Written by TPL_BWD_SHARD: d_w_in, d_b_in, d_w_out (shapes of w_in, b_in, w_out).
 *   Written by TPL_BWD_REPLICATED: d_ln_g, d_ln_b, d_b_out ([h] each;
 *   d_b_out = sum over rows of dy, the gradient of the row-parallel bias). */
typedef struct {
  float* d_w_in;
  float* d_b_in;
  float* d_w_out;
  float* d_ln_g;
  float* d_ln_b;
  float* d_b_out;
} tpl_block_grads;

/* Size in bytes of the `saved` buffer that tp_layer_shard_fwd fills and
 * tp_layer_shard_bwd reads (activations kept for the backward pass plus the
 * backward's own scratch). Returns 0 if the descriptor is invalid. */
size_t tp_layer_saved_bytes(const tpl_desc* desc, tpl_block block);

/* Forward of one block on this rank (podcast page Outline; guide page 3.1/3.2).
 *   ATTN: y = LN1(x); qkv = y W_qkv^T + b_qkv; per head of this rank,
 *         O = softmax(Q K^T/sqrt(d) (+causal mask)) V; partial = ctx W_o^T.
 *   MLP:  z = LN2(x); u = z W_1^T + b_1; a = GeLU(u) (exact erf form);
 *         partial = a W_2^T.
 * x: [N][h] block input (replicated on every rank).
 * partial: [N][h] out, this rank's row-parallel partial sum, without the
 *          row-parallel bias or the residual (summed by shard_partial_sum).
 * saved: tp_layer_saved_bytes() bytes (required: it also holds the block's
 *        intermediates -- LN output, qkv / GeLU'(u), attention output / GeLU output,
 *        LN and softmax statistics -- and the backward's scratch). */
tpl_status tp_layer_shard_fwd(const tpl_desc* desc, tpl_block block, const void* x,
                              const tpl_block_params* params, void* partial, void* saved,
                              void* stream);

/* The all-reduce stand-in (podcast page Key concepts: all-reduce; Outline: two
 * per module): out = residual + bias + sum_{i<n} partials[i], accumulated in
 * fp32 in the order residual, bias, partials[0..n-1] and rounded once to the
 * storage type. partials: HOST array of n device pointers, each [rows][cols];
 * bias: [cols] or NULL; residual: [rows][cols] or NULL; out may alias residual
 * or partials[i]. 1 <= n <= 16; cols a multiple of 8. */
tpl_status shard_partial_sum(const tpl_desc* desc, const void* const* partials, int32_t n,
                             const void* bias, const void* residual, void* out, int64_t rows,
                             int32_t cols, void* stream);

/* Backward of one block on this rank, in two phases around the all-reduce of
 * the gradient w.r.t. the block's LayerNorm output. Defining passages:
 * podcast page "Megatron-LM's parallelism", Outline (two all-reduces per
 * module, four per layer forward+backward: in the backward each block's
 * input gradient is all-reduced once; LayerNorm, dropout and the residual
 * are duplicated on every rank, so their backward runs replicated after the
 * all-reduce); guide page "From Transformer splitting to communication
 * optimisation", section 3.1 (the MLP's column-parallel first layer and
 * row-parallel second layer, so GeLU's gradient is local to the rank's
 * columns) and section 3.2 (QKV split by heads, output projection split by
 * rows).
 *   TPL_BWD_SHARD: from dy ([N][h], gradient of the block output) and `saved`,
 *     writes d_ln_partial [N][h] (this rank's partial gradient w.r.t. the LN
 *     output) and grads->d_w_in, d_b_in, d_w_out.
 *       MLP: du = (dy W_2) * GeLU'(u); dW_2 = dy^T a; dW_1 = du^T z;
 *            db_1 = sum_n du; d_ln_partial = du W_1.
 *       ATTN: dctx = dy W_o; dW_o = dy^T ctx; flash-attention backward ->
 *             dqkv; dW_qkv = dqkv^T y; db_qkv = sum_n dqkv; d_ln_partial = dqkv W_qkv.
 *   TPL_BWD_REPLICATED: from dy, d_ln_sum (= sum over ranks of d_ln_partial),
 *     the block input x and `saved`, writes dx = dy + LN_bwd(d_ln_sum) [N][h]
 *     and grads->d_ln_g, d_ln_b, d_b_out.
 *   TPL_BWD_SHARD_RECOMPUTE: activation recomputation (overview page section
 *     3: checkpointing trades compute for memory). As TPL_BWD_SHARD, but the
 *     block's forward stash (LN output and statistics; ATTN: qkv, ctx, LSE;
 *     MLP: GeLU'(u) and GeLU(u)) is first recomputed from the block input x into
 *     `saved`, so `saved` need not hold this block's forward: one buffer of
 *     tp_layer_saved_bytes can serve every layer of a model. Results are
 *     identical to TPL_BWD_SHARD. A later TPL_BWD_REPLICATED call with the
 *     same `saved` uses the recomputed LN statistics.
 * Unused pointers for a phase may be NULL. For TPL_BWD_SHARD and
 * TPL_BWD_REPLICATED `saved` must come from tp_layer_shard_fwd (or a
 * recomputing call) with the same desc, block, x and params; its scratch part
 * is overwritten. */
tpl_status tp_layer_shard_bwd(const tpl_desc* desc, tpl_block block, tpl_bwd_phase phase,
                              const void* dy, const void* d_ln_sum, const void* x,
                              const tpl_block_params* params, void* saved, void* d_ln_partial,
                              void* dx, const tpl_block_grads* grads, void* stream);

/* Size in bytes of the `stats` buffer of vocab_parallel_xent_fwd for this
 * descriptor (0 if the descriptor is invalid). Its first N*3 floats are the
 * row statistics exchanged between ranks; the rest is scratch for the
 * per-tile statistics of the logits product (bf16). */
size_t vocab_parallel_xent_stats_bytes(const tpl_desc* desc);

/* Vocabulary-parallel cross-entropy forward (guide page 3.3; podcast page
 * Outline: output embedding split along the vocabulary, loss fused).
 *   TPL_XENT_LOCAL: logits = hidden E_r^T ([N][V_r], storage dtype, kept for
 *     the backward) and per-row statistics stats[n] = (m, se, tl):
 *     m = max_j logits[n][j], se = sum_j exp(logits[n][j] - m),
 *     tl = logits[n][targets[n] - rank*V_r] if the target is in this rank's
 *     range, else 0, over the stored (rounded) logits. The shard's softmax is
 *     never materialised: in bf16 the statistics are taken in the product's
 *     epilogue per 256- or 128-column tile and merged per row in a fixed
 *     order. `stats` must hold vocab_parallel_xent_stats_bytes(desc) bytes.
 *   TPL_XENT_FINISH: from the t ranks' stats (all_stats: HOST array of t device
 *     pointers, in rank order; only the first N*3 floats of each are read):
 *     M = max_r m_r, S = sum_r se_r exp(m_r - M),
 *     lse[n] = M + ln S, loss_rows[n] = mask[n] * (lse[n] - sum_r tl_r),
 *     loss[0] = sum_n loss_rows[n] / sum_n mask[n], loss[1] = sum_n mask[n].
 * hidden: [N][h]; emb: E_r [V_r][h]; targets: [N] int32 global ids in [0, V)
 * (an id outside [0, V) gives tl = 0 on every rank); loss_mask: [N] uint8 or
 * NULL (every row counts). Pointers a phase does not use may be NULL. */
tpl_status vocab_parallel_xent_fwd(const tpl_desc* desc, tpl_xent_phase phase,
                                   const void* hidden, const void* emb, const int32_t* targets,
                                   const uint8_t* loss_mask, void* logits, float* stats,
                                   const float* const* all_stats, float* lse, float* loss_rows,
                                   float* loss, void* stream);

/* Loss rows of a masked loss (podcast page, Outline: the large-BERT variant;
 * its masked-token loss is taken on a fraction of the positions). The loss
 * needs logits, dlogits, dH and dE only for those rows, so a caller that knows
 * them (the batch's mask gives their index list) gathers them, runs
 * vocab_parallel_xent_fwd/bwd on a descriptor of that many rows with
 * loss_mask NULL (the mean over the gathered rows is the masked mean), and
 * expands dH back to every row.
 *   tpl_rows_gather: dst row i = src row rows[i], i < n.
 *   tpl_rows_expand: dst row r = src row pos[r] if pos[r] >= 0, else zeros,
 *     r < n_dst (pos[r] = index of row r in the gathered list, or -1).
 * src: n_src rows of row_bytes bytes (a multiple of 4); an index outside
 * [0, n_src) reads nothing and gives a zero row. rows / pos: int32 device
 * arrays. Pointers 4-byte aligned; INVALID_ARG for negative sizes or a bad
 * row_bytes, before any launch. */
tpl_status tpl_rows_gather(const void* src, int64_t n_src, const int32_t* rows, int64_t n, int64_t row_bytes,
                           void* dst, void* stream);
tpl_status tpl_rows_expand(const void* src, int64_t n_src, const int32_t* pos, int64_t n_dst, int64_t row_bytes,
                           void* dst, void* stream);

/* Vocabulary-parallel input embedding (guide page 3.3: the input layer is
 * split along the vocabulary and the ranks' outputs summed by an all-reduce).
 *   fwd: x_partial [N][h] (storage dtype) row n = E_r[tokens[n] - rank*V_r] if
 *     the id lies in this rank's range [rank*V_r, (rank+1)*V_r), else zeros.
 *     shard_partial_sum over the ranks' partials (the all-reduce) gives the
 *     lookup E[tokens[n]].
 *   bwd: from d_out [N][h] (storage dtype; the gradient of the summed output,
 *     the same on every rank), d_emb_in [V_r][h] fp32 (overwritten) row v =
 *     sum of d_out[n] over the rows whose id is rank*V_r + v, added in
 *     ascending n (a stable sort of the ids, no float atomics: deterministic);
 *     rows no id points to are zero. No communication.
 * tokens: [N] int32 global ids (ids outside [0, V) contribute nothing);
 * emb_in: E_r [V_r][h] storage dtype; workspace: device scratch of
 * vocab_parallel_embedding_ws_bytes(desc) bytes, overwritten. */
size_t vocab_parallel_embedding_ws_bytes(const tpl_desc* desc);
tpl_status vocab_parallel_embedding_fwd(const tpl_desc* desc, const int32_t* tokens, const void* emb_in,
                                        void* x_partial, void* stream);
tpl_status vocab_parallel_embedding_bwd(const tpl_desc* desc, const int32_t* tokens, const void* d_out,
                                        float* d_emb_in, void* workspace, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward as vocab_parallel_embedding_bwd, with its workspace taken from a
 * device array of TPL_NOALLOC_SCRATCH_BYTES inside the library (one per GPU,
 * held until the process ends) instead of a workspace argument. It calls no
 * allocating routine. Limit: vocab_parallel_embedding_ws_bytes(desc) <=
 * TPL_NOALLOC_SCRATCH_BYTES (16 B per row plus 4 B per vocabulary row of the
 * rank, rounded up to 256 B), else TPL_ERR_UNSUPPORTED before any launch.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU (different streams, or several threads) race and must be serialised
 * by the caller. The first call on a device looks the array's address up
 * (TPL_ERR_HIP if that fails). Results are bitwise those of
 * vocab_parallel_embedding_bwd. */
#define TPL_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
tpl_status vocab_parallel_embedding_bwd_noalloc(const tpl_desc* desc, const int32_t* tokens, const void* d_out,
                                                float* d_emb_in, void* stream);

/* Vocabulary-parallel cross-entropy backward for this rank (guide page
 * "From Transformer splitting to communication optimisation", section 3.3:
 * the output layer split along the vocabulary with the gather deferred into
 * the cross-entropy, so each rank forms the gradient of its own logits from
 * the exchanged row statistics and needs one all-reduce of its hidden-state
 * gradient; podcast page, Outline: output embedding split along the
 * vocabulary, loss fused in).
 *   dlogits = g_n (exp(logits - lse_n) - [j == targets[n] - rank*V_r]) with
 *   g_n = dloss * mask[n] / loss[1], written IN PLACE over `logits`;
 *   d_hidden_partial = dlogits E_r ([N][h], storage dtype; summed over ranks
 *   by shard_partial_sum); d_emb = dlogits^T hidden ([V_r][h], fp32).
 * lse and loss are the FINISH outputs. */
tpl_status vocab_parallel_xent_bwd(const tpl_desc* desc, const void* hidden, const void* emb,
                                   const int32_t* targets, const uint8_t* loss_mask, void* logits,
                                   const float* lse, const float* loss, float dloss,
                                   void* d_hidden_partial, float* d_emb, void* stream);

/* Dense product used by every parallel linear layer, exposed for unit checks
 * and timing: C[M][N] = sum_k A(m,k) B(n,k) (+ bias[n]).
 *   a_kmajor = 1: A stored [M][lda] (A(m,k) = A[m*lda+k]); 0: stored [K][lda]
 *   (A(m,k) = A[k*lda+m]). b_kmajor likewise for B with n. A and B have the
 *   storage dtype; C is the storage dtype (c_f32 = 0) or fp32 (c_f32 = 1).
 *   bias: [N] storage dtype or NULL. */
tpl_status tpl_gemm(int32_t dtype, int32_t a_kmajor, int32_t b_kmajor, int64_t M, int64_t N,
                    int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    const void* bias, void* C, int64_t ldc, int32_t c_f32, void* stream);

/* Per-kernel timing for profiling (not needed for computation).
 * tpl_trace_enable(capacity) makes every later launch record a HIP event pair
 * on the stream it is launched on, up to `capacity` launches (0 disables and
 * drops the records); returns the capacity, or -1 if events could not be made.
 * tpl_trace_read copies up to max_n records to host arrays: a kernel-name
 * index (see tpl_trace_kernel_name), the elapsed milliseconds, and the
 * launch's algorithmic work (flops for the MFMA kernels -- GEMM 2*M*N*K,
 * attention over the visible query-key pairs only -- and bytes read+written
 * once for the memory-bound kernels). It synchronises the recorded events and
 * returns the number copied (-1 on a HIP error). Not thread-safe with
 * concurrent launches on other threads. */
int32_t tpl_trace_enable(int32_t capacity);
int32_t tpl_trace_read(int32_t* kernel_ids, float* ms, double* work, int32_t max_n);
const char* tpl_trace_kernel_name(int32_t kernel_id);

/* Human-readable status text. */
const char* tpl_status_string(tpl_status status);

#ifdef __cplusplus
}
#endif
#endif /* TP_LAYER_H_ */
