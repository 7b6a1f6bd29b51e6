/*
 * tpcol.h -- C ABI of the MI355X (gfx950) tensor-parallel shard library.
 *
 * The library computes ONE tensor-parallel shard's share of a transformer
 * block on one GPU: the column-parallel GEMM with a fused activation
 * epilogue, head-local attention, the row-parallel GEMM that yields a
 * partial sum, the sum of the N partials (standing in for the all-reduce),
 * and the MLP backward.  Shard i of N is the i-th contiguous block:
 *   column shard  W_i = W[:, i*w : (i+1)*w]   (output dimension split)
 *   row shard     W_i = W[i*w : (i+1)*w, :]   (input dimension split)
 * following "张量并行" (section 并行化矩阵乘法运算: column-linear and
 * row-linear sharding; section MLP 层的并行化: A column-split, B row-split)
 * and "Infra: Tensor Parallel" (Column-wise TP / Row-wise TP equations).
 *
 * Conventions shared by every call:
 *   - Matrices are row-major; ld* is the row stride in ELEMENTS (>= width).
 *   - Weights are [in x out] and used as X @ W (the pages' X W notation).
 *   - dtype TP_F32: every operand float32.  TP_BF16: inputs, weights and the
 *     activation outputs are bfloat16 (raw 16-bit patterns); accumulation is
 *     always float32; partial sums P and all gradients are float32.
 *   - Pointers are DEVICE pointers unless stated otherwise, must be 16-byte
 *     aligned, and ld * element size must be a multiple of 16 bytes.  The
 *     contiguous (last) dimension of every matrix must be a multiple of the
 *     16-byte vector (8 elements for bf16, 4 for fp32).  Token counts
 *     (M, b*s) may be anything >= 0; M == 0 is a no-op returning TP_OK
 *     (the backward then writes zero weight gradients), and the pointers
 *     of empty matrices may be NULL.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: they validate on the host, enqueue kernels and return.
 *     Kernel faults surface at the caller's next synchronisation.
 *   - The library never allocates device memory.  Scratch space comes from
 *     the caller's workspace (ws, ws_bytes); query its size with the
 *     matching *_workspace() function.  A workspace must not be used by two
 *     calls that can run at the same time.
 *   - Validation happens before any launch; on error nothing is enqueued,
 *     outputs are untouched and a detail string is kept for tp_last_error().
 *   - Operands must not alias outputs.
 */
#ifndef TPCOL_H
#define TPCOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_ARG = -1,        /* NULL required pointer, bad enum, bad count        */
    TP_ERR_SHAPE = -2,      /* non-positive size, ld < width, indivisible split  */
    TP_ERR_ALIGN = -3,      /* pointer / ld / width not 16-byte vectorisable     */
    TP_ERR_DTYPE = -4,      /* unsupported dtype for this call                   */
    TP_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required           */
    TP_ERR_HIP = -6         /* a HIP runtime call or kernel launch failed        */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum {
    TP_ACT_NONE = 0,        /* identity (e.g. the QKV projection)                */
    TP_ACT_GELU_ERF = 1,    /* exact GELU  z * Phi(z)                            */
    TP_ACT_SWIGLU = 2       /* SiLU(X Wg) * (X Wu): needs the second weight Wup  */
} tp_act;

/*
 * Column-parallel linear with fused activation:
 *     H_i = act(X @ W_i + bias_i)            (TP_ACT_NONE / TP_ACT_GELU_ERF)
 *     H_i = SiLU(X @ W_i) * (X @ Wup_i)      (TP_ACT_SWIGLU; bias must be NULL)
 * X is replicated on every shard (no communication before the layer);
 * W_i is the i-th column block.  The activation is column-separable, so it is
 * applied per shard ("张量并行", MLP 层的并行化: GELU([Y1,Y2]) =
 * [GELU(Y1), GELU(Y2)]; "Infra: Tensor Parallel", Column-wise TP).  The
 * pre-activation is never written to memory.
 *   X    [M x K]   ldx         dtype
 *   W    [K x Ni]  ldw         dtype   (W_gate for SwiGLU)
 *   Wup  [K x Ni]  ldwu        dtype   (SwiGLU only, else NULL)
 *   bias [Ni]                  dtype   (optional, NULL for none)
 *   H    [M x Ni]  ldh         dtype   (output)
 * M <= the GEMV threshold (16 by default) selects the weight-streaming decode
 * path, which needs tp_col_linear_gelu_workspace() bytes of ws (256-byte
 * aligned scratch for split-K partial sums; contents on entry do not
 * matter).  Larger M needs no workspace (ws may be NULL).
 */
int tp_col_linear_gelu(int dtype, int act, int64_t M, int64_t K, int64_t Ni,
                       const void *X, int64_t ldx,
                       const void *W, int64_t ldw,
                       const void *Wup, int64_t ldwu,
                       const void *bias,
                       void *H, int64_t ldh,
                       void *ws, size_t ws_bytes, void *stream);
size_t tp_col_linear_gelu_workspace(int dtype, int act, int64_t M, int64_t K, int64_t Ni);

/*
 * tp_col_linear_gelu for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results, with no workspace.  No call allocates.
 * The decode path (M <= the GEMV threshold) keeps its split-K partial sums
 * in a static device array of the library (2 MiB of fp32 partials, one copy
 * per GPU, held until the process ends) and runs the same two kernels as
 * tp_col_linear_gelu (the split-K pass, then the sum of the partials in
 * split order with bias and activation), so the results are identical.
 * Every decode shape fits that array (the split count is chosen so that the
 * partials never exceed 2 MiB).  Larger M uses the GEMM path, which needs no
 * scratch.  Calls that overlap on one GPU (different streams, or different
 * host threads without ordering) share the array and race; calls ordered
 * on one stream do not.
 */
int tp_col_linear_gelu_noalloc(int dtype, int act, int64_t M, int64_t K, int64_t Ni,
                               const void *X, int64_t ldx,
                               const void *W, int64_t ldw,
                               const void *Wup, int64_t ldwu,
                               const void *bias,
                               void *H, int64_t ldh, void *stream);

/*
 * Row-parallel linear, this shard's partial sum (no bias, no reduction):
 *     P_i = X_i @ W_i
 * X_i is this shard's slice of the input's last dimension (H_i or O_i), W_i
 * the i-th row block ("张量并行", 两个矩阵相乘: X A = sum_i X_i A_i;
 * "Infra: Tensor Parallel", Row-wise TP).  The row bias belongs after the
 * sum (tp_shard_sum), since adding it per shard would count it N times.
 *   Xi [M x Ki] ldx dtype ; Wi [Ki x N] ldw dtype ; P [M x N] ldp float32.
 * Workspace rules as for tp_col_linear_gelu (needed only for M <= threshold).
 */
int tp_row_linear_partial(int dtype, int64_t M, int64_t Ki, int64_t N,
                          const void *Xi, int64_t ldx,
                          const void *Wi, int64_t ldw,
                          float *P, int64_t ldp,
                          void *ws, size_t ws_bytes, void *stream);
size_t tp_row_linear_partial_workspace(int dtype, int64_t M, int64_t Ki, int64_t N);

/*
 * Decode linear on a pre-packed weight.  In the decode phase every request
 * adds one token, so a linear layer reads its whole weight once per token
 * for 2 * M flops per weight (parallelism overview post, Prefill-Decode
 * 分离 -> Decode 阶段 -> 线性层: memory-bound); the weight does not change
 * between tokens, so it can be stored once in the order the weight-streaming
 * kernel reads it.
 *
 * tp_decode_pack_weight: Wp = panels of 64 columns, each holding every row:
 *     Wp[(s * Kp + k) * 64 + c] = W[k][64 s + c]     (bf16)
 * for panels s < ceil(N / 64), rows k < Kp = K rounded up to a multiple of
 * 64, columns c < 64; entries past K or N are zero.  Wp must hold
 * tp_decode_packed_weight_bytes(K, N) bytes (16-byte aligned), and the call
 * writes all of them.  W [K x N] ldw bf16 is row-major as everywhere else.
 *
 * tp_decode_linear_packed: the decode path of tp_col_linear_gelu /
 * tp_row_linear_partial with W read from its panels:
 *     Y = act(X @ W + bias)   out_dtype TP_BF16, act TP_ACT_NONE / TP_ACT_GELU_ERF
 *     Y = X @ W (+ bias)      out_dtype TP_F32 (row-parallel partial), act NONE
 *   X  [M x K] ldx bf16, 1 <= M <= 16 (M == 0: no-op)
 *   Wp tp_decode_pack_weight's output for the same K, N (wp_bytes its size)
 *   Y  [M x N] ldy, bf16 or fp32 (out_dtype)
 *   ws tp_decode_linear_packed_workspace(M, K, N) bytes, 256-byte aligned
 *      (split-K partial sums; contents on entry do not matter)
 * Each workgroup's share of a panel is one contiguous run of memory (in the
 * row-major layout it is 128 bytes from each of its rows).  The sums are
 * taken in the same order as the row-major decode path, so for the same X,
 * W and bias both give identical results.  dtype is bf16 only; M > 16, fp32
 * output with an activation, or a Wp smaller than the panels need return an
 * error before any launch.
 */
size_t tp_decode_packed_weight_bytes(int64_t K, int64_t N);
int tp_decode_pack_weight(int dtype, int64_t K, int64_t N,
                          const void *W, int64_t ldw,
                          void *Wp, size_t wp_bytes, void *stream);
int tp_decode_linear_packed(int act, int out_dtype, int64_t M, int64_t K, int64_t N,
                            const void *X, int64_t ldx,
                            const void *Wp, size_t wp_bytes,
                            const void *bias,
                            void *Y, int64_t ldy,
                            void *ws, size_t ws_bytes, void *stream);
size_t tp_decode_linear_packed_workspace(int64_t M, int64_t K, int64_t N);

/*
 * Head-sharded self-attention block, this shard's partial output:
 *     [Q | K | V] = X @ Wqkv_i            (heads_local heads, each d wide)
 *     O_t = softmax(Q_t K_t^T / sqrt(d) [+ causal mask]) V_t   per head t
 *     P_i = [O_1 ... O_heads_local] @ Wo_i
 * The local heads feed the local row block of Wo directly: no gather of the
 * heads is needed ("Infra: Tensor Parallel", MHA: Wo row-wise, heads
 * column-wise; "张量并行", Multi-Head Attention 的并行化; parallelism overview
 * post, section 1 Tensor Parallelism).  Packing of Wqkv_i columns: Q heads,
 * then K heads, then V heads, head t at offset t*d inside each block
 * ("Megatron-LM 实战 04", TPAttention: qkv reshaped to (3, heads, d)).
 * Causal: key j is visible to query i iff j <= i (within one sequence).
 *   X    [b*s x h]                      ldx    dtype (token-major, batch-major)
 *   Wqkv [h x 3*heads_local*d]          ldwqkv dtype
 *   Wo   [heads_local*d x h]            ldwo   dtype
 *   P    [b*s x h]                      ldp    float32 (output)
 *   ws   tp_attn_heads_shard_workspace() bytes: QKV_i [b*s x 3*hl*d] then
 *        O_i [b*s x hl*d], both dtype row-major, readable after the call,
 *        then each query row's softmax statistic (fp32 [b][hl][s], log2 of
 *        sum_j exp2(S_ij log2(e)) for the scaled scores S), which
 *        tp_attn_shard_backward reads.
 * TP_BF16 with d == 128 runs the flash kernels; TP_F32, or any head dim
 * 1..256, runs general kernels (fp32 softmax and accumulation either way;
 * b*heads_local <= 65535 there).  d outside 1..256, or 3*heads_local*d above
 * 2^24, is TP_ERR_SHAPE; heads_local*d*element size must be a multiple of 16
 * bytes (TP_ERR_ALIGN).
 */
int tp_attn_heads_shard(int dtype, int64_t b, int64_t s, int64_t h,
                        int64_t heads_local, int64_t d, int causal,
                        const void *X, int64_t ldx,
                        const void *Wqkv, int64_t ldwqkv,
                        const void *Wo, int64_t ldwo,
                        float *P, int64_t ldp,
                        void *ws, size_t ws_bytes, void *stream);
size_t tp_attn_heads_shard_workspace(int dtype, int64_t b, int64_t s,
                                     int64_t heads_local, int64_t d);

/*
 * Grouped-query variant of tp_attn_heads_shard: the shard holds heads_local
 * query heads and kv_heads_local key/value heads; query head t (local) reads
 * key/value head t / (heads_local / kv_heads_local), i.e. consecutive groups
 * of query heads share one key/value head ("张量并行", 相关分析: GQA has
 * num_attention_heads >= num_kv_heads, and K/V heads must stay consistent
 * across shards).  With more shards than key/value heads, each shard holds
 * the one key/value head its query heads read, replicated on the shards of
 * the group.  kv_heads_local == heads_local is tp_attn_heads_shard.
 *   Wqkv [h x (heads_local + 2*kv_heads_local)*d]: Q heads, then K heads,
 *        then V heads, head u at offset u*d inside its block.
 *   ws   tp_attn_gqa_shard_workspace() bytes: QKV_i [b*s x (hl + 2*kvl)*d]
 *        then O_i [b*s x hl*d], dtype row-major, readable after the call,
 *        then the per-row softmax statistic as for tp_attn_heads_shard.
 * heads_local must be a multiple of kv_heads_local, and
 * (heads_local + 2*kv_heads_local)*d at most 2^24 (TP_ERR_SHAPE); otherwise
 * as tp_attn_heads_shard.
 */
int tp_attn_gqa_shard(int dtype, int64_t b, int64_t s, int64_t h,
                      int64_t heads_local, int64_t kv_heads_local, int64_t d, int causal,
                      const void *X, int64_t ldx,
                      const void *Wqkv, int64_t ldwqkv,
                      const void *Wo, int64_t ldwo,
                      float *P, int64_t ldp,
                      void *ws, size_t ws_bytes, void *stream);
size_t tp_attn_gqa_shard_workspace(int dtype, int64_t b, int64_t s, int64_t heads_local,
                                   int64_t kv_heads_local, int64_t d);

/*
 * Backward of the attention shard (multi-head: kv_heads_local ==
 * heads_local; grouped-query otherwise), given dY = dL/dY broadcast to every
 * shard.  A shard owns whole heads, so it differentiates them alone
 * ("张量并行", Multi-Head Attention 的并行化); the projections follow the
 * row- and column-wise backward equations of "Infra: Tensor Parallel":
 *   output projection (row-wise)  dWo_i = O_i^T dY,  dO_i = dY Wo_i^T
 *   per head (chain rule through the products and the row softmax)
 *                                 dV = P^T dO,  dS = P * (dO V^T - rowsum(dO*O)),
 *                                 dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
 *                                 (a kv head sums its query heads' dK, dV)
 *   QKV projection (column-wise)  dWqkv_i = X^T [dQ | dK | dV],
 *                                 dX_i = [dQ | dK | dV] Wqkv_i^T
 * dX_i is this shard's partial of dX = sum_i dX_i (f's backward all-reduce;
 * tp_shard_sum).
 *   X, Wqkv, Wo, dY: as in the forward call (dtype); dY [b*s x h] lddy.
 *   fwd_ws: the workspace of the forward call (tp_attn_heads_shard or
 *        tp_attn_gqa_shard) on the same inputs, as it left it: QKV_i, O_i
 *        and the row statistic are read, not recomputed.
 *   Outputs (float32, dense unless noted): dWqkv [h x (hl + 2*kvl)*d],
 *        dWo [hl*d x h], dXi [b*s x h] with row stride lddx.
 *   ws   tp_attn_shard_backward_workspace() bytes: dO_i (dtype), D (fp32),
 *        [dQ | dK | dV] (dtype, packed like QKV_i) and, for bf16 grouped-query
 *        shards with d == 128 whose kv heads alone would not fill the device,
 *        fp32 dK/dV partials of head subsets (added in a fixed order).
 * dtype and shape rules as for tp_attn_gqa_shard.  Both
 * workspaces 256-byte aligned.  Every sum runs in a fixed order: repeated
 * calls give identical bits.
 */
int tp_attn_shard_backward(int dtype, int64_t b, int64_t s, int64_t h,
                           int64_t heads_local, int64_t kv_heads_local, int64_t d, int causal,
                           const void *X, int64_t ldx,
                           const void *Wqkv, int64_t ldwqkv,
                           const void *Wo, int64_t ldwo,
                           const void *dY, int64_t lddy,
                           const void *fwd_ws, size_t fwd_ws_bytes,
                           float *dWqkv, float *dWo, float *dXi, int64_t lddx,
                           void *ws, size_t ws_bytes, void *stream);
size_t tp_attn_shard_backward_workspace(int dtype, int64_t b, int64_t s, int64_t heads_local,
                                        int64_t kv_heads_local, int64_t d);

/*
 * Sum of the N shard partials, added in shard order in float32, plus an
 * optional bias added once:
 *     Y = sum_{i<n} P_i (+ bias)
 * It stands in for the row-parallel layer's all-reduce (g's forward;
 * "张量并行", 行并行 and MLP 层的并行化) and for the column layer's backward
 * all-reduce of dX (f's backward) when all partials live in one GPU.
 *   partials  HOST array of n device pointers, each [M x N] float32, ldp
 *   bias      [N] float32 or NULL
 *   Y         [M x N] ldy, out_dtype (TP_F32 or TP_BF16, RNE rounding)
 * 1 <= n <= 64.  Y may alias partials[0] when out_dtype == TP_F32 and
 * ldy == ldp.
 */
int tp_shard_sum(int out_dtype, int64_t M, int64_t N, int n,
                 const float *const *partials, int64_t ldp,
                 const float *bias, void *Y, int64_t ldy, void *stream);

/*
 * Sequence-parallel end of a tensor-parallel block, for one rank: the
 * all-reduce of the row-parallel partials splits into a reduce-scatter and
 * an all-gather, and LayerNorm runs on the rank's reduce-scattered rows
 * (parallelism overview post, 5 Sequence Parallelism).  For the `rows` token
 * rows of this rank:
 *     Ysum = sum_{i<n} P_i (+ bias, once) (+ residual)
 *     Y    = gamma * (Ysum - mean) / sqrt(var + eps) + beta
 * with mean and population variance over the full hidden row of N values
 * ("张量并行", 相关分析: LayerNorm needs statistics of the complete hidden
 * dimension).  Partials are added in shard order, then the bias, then the
 * residual.  The caller passes each partial's pointer at the rank's first
 * row (rank r of n holds token rows r*T/n .. (r+1)*T/n - 1 in the
 * sequence-major token order); with Y pointing into one [T x N] buffer at
 * the same row, the n ranks' outputs form the all-gathered activation.
 *   partials  HOST array of n device pointers, each [rows x N] fp32, ldp
 *   bias      [N] fp32 or NULL;  residual [rows x N] fp32 (ldr) or NULL
 *   gamma, beta [N] fp32 (required);  eps >= 0
 *   Ysum      [rows x N] fp32 (ldys) or NULL: the pre-norm sum (the
 *             residual stream of the next block)
 *   Y         [rows x N] out_dtype (ldy)
 * N must be a multiple of 4 (fp32) / 8 (bf16 Y), 4 <= N <= 8192
 * (TP_ERR_SHAPE); 1 <= n <= 64.
 */
int tp_shard_reduce_scatter_layernorm(int out_dtype, int64_t rows, int64_t N, int n,
                                      const float *const *partials, int64_t ldp,
                                      const float *bias, const float *residual, int64_t ldr,
                                      const float *gamma, const float *beta, float eps,
                                      float *Ysum, int64_t ldys,
                                      void *Y, int64_t ldy, void *stream);

/*
 * Vocabulary-parallel cross-entropy ("张量并行", 损失计算层的并行化): the
 * logits [T x V] are split by vocabulary columns, shard i holding columns
 * vocab_start .. vocab_start + Vi - 1.  Instead of gathering the b*s*v
 * logits, each shard reduces its slice of every row (step 1), the shards'
 * row numbers are combined -- a b*s-sized all-reduce (step 2) -- giving the
 * softmax denominator, each shard sums the loss of the rows whose target
 * token it holds (step 3), and the n shard losses are summed -- an n-sized
 * all-reduce (step 4).  The row statistics carry the row max next to the
 * sum of exponentials, which keeps the same denominator within fp32 range.
 *
 * Step 1: stats [T x 2] fp32 = (max_j z[t][j], sum_j exp(z[t][j] - max))
 *         over the shard's Vi columns.  logits dtype TP_F32 / TP_BF16,
 *         row-major [T x Vi] with row stride ldz >= Vi elements; any width,
 *         stride and element-aligned address (16-byte vectors inside rows).
 *         A row whose values are all -inf yields (-inf, 0).
 */
int tp_vocab_ce_shard_stats(int dtype, int64_t T, int64_t Vi, const void *logits, int64_t ldz,
                            float *stats, void *stream);
/*
 * Step 2: lse[t] = M + log sum_i s_i[t] exp(m_i[t] - M), M = max_i m_i[t]
 *         (the row's log-sum-exp over the whole vocabulary), shards added in
 *         index order.  stats: HOST array of n device pointers ([T x 2]).
 */
int tp_vocab_ce_lse(int64_t T, int n, const float *const *stats, float *lse, void *stream);
/*
 * Step 3: shard_loss[0] = sum over rows t whose target lies in this shard's
 *         columns of (lse[t] - z[t][target[t] - vocab_start]) (fp32, rows
 *         added in a fixed order).  row_loss [T] (optional) receives each
 *         row's term, 0 for rows whose target is elsewhere.  targets: int32
 *         token ids [T]; ids outside every shard contribute nothing.
 */
int tp_vocab_ce_shard_loss(int dtype, int64_t T, int64_t Vi, int64_t vocab_start,
                           const void *logits, int64_t ldz, const int32_t *targets,
                           const float *lse, float *row_loss, float *shard_loss, void *stream);
/*
 * Step 4: total[0] = sum_i shard_losses[i][0] in shard order (the summed
 *         cross-entropy of the T rows).  shard_losses: HOST array of n
 *         device pointers to one float each.
 */
int tp_vocab_ce_total(int n, const float *const *shard_losses, float *total, void *stream);

/*
 * MLP shard backward given dY (broadcast to every shard):
 *   row layer    dW2_i = H_i^T dY,  dH_i = dY W2_i^T
 *   activation   dZ_i = dH_i * GELU'(Z_i)          (GELU; Z_i recomputed)
 *                dZu = dH * SiLU(Zg), dZg = dH * Zu * SiLU'(Zg)   (SwiGLU)
 *   column layer dW1_i = X^T dZ_i,  db1_i = sum over tokens of dZ_i,
 *                dX_i = dZ_i W1_i^T (SwiGLU: dZg Wg_i^T + dZu Wu_i^T)
 * ("Infra: Tensor Parallel", Column-wise and Row-wise TP backward equations;
 * "张量并行", 行并行 backward of g and MLP 层的并行化 backward of f.)
 * dX_i is this shard's partial of dX = sum_i dX_i; sum them with
 * tp_shard_sum (f's backward all-reduce).
 *   X  [M x K] ldx, W1 [K x Ni] ldw1 (W_gate for SwiGLU), Wup [K x Ni] ldwu
 *   (SwiGLU else NULL), b1 [Ni] (GELU only, optional), W2 [Ni x K] ldw2,
 *   dY [M x K] lddy: all dtype.
 *   Outputs (float32, dense): dW1 [K x Ni], dWup [K x Ni] (SwiGLU else NULL),
 *   dW2 [Ni x K], db1 [Ni] (optional; GELU only), dXi [M x K] ldd x.
 *   ws: tp_mlp_shard_backward_workspace() bytes; holds dH_i, H_i and dZ_i
 *   ([M x Ni] each, dtype; dZg and dZu for SwiGLU) and, without SwiGLU, a
 *   second dH-sized region and max(64, ceil(M / 128)) fp32 rows [. x Ni]
 *   of partial column sums for db1 (per 128-row tile of dZ when the
 *   recompute's epilogue forms them, else per row split of a column-sum
 *   pass).  After the recompute the dH region (GELU: with the
 *   region after it) holds fp32 K-range partials of the weight gradients.
 *   Every partial is added in a fixed order, so all outputs are
 *   deterministic.
 */
int tp_mlp_shard_backward(int dtype, int act, int64_t M, int64_t K, int64_t Ni,
                          const void *X, int64_t ldx,
                          const void *W1, int64_t ldw1,
                          const void *Wup, int64_t ldwu,
                          const void *b1,
                          const void *W2, int64_t ldw2,
                          const void *dY, int64_t lddy,
                          float *dW1, float *dWup, float *dW2, float *db1,
                          float *dXi, int64_t lddx,
                          void *ws, size_t ws_bytes, void *stream);
size_t tp_mlp_shard_backward_workspace(int dtype, int act, int64_t M, int64_t Ni);

/*
 * Host-only divisibility check of a tensor-parallel split (no GPU use):
 * ffn % n == 0, heads % n == 0 and h % heads == 0 ("Megatron-LM 实战 04",
 * TPAttention asserts and 常见问题; "Infra: Tensor Parallel", the head count
 * must be a multiple of the TP size).  heads == 0 skips the head checks.
 * Returns TP_OK or TP_ERR_SHAPE.
 */
int tp_check_split(int64_t h, int64_t ffn, int64_t heads, int64_t n);

/* Tuning/testing option: token count at or below which the linear calls take
 * the decode GEMV path (default 16, range 0..16; 0 disables the GEMV path).
 * Process-wide; returns the previous value, or TP_ERR_ARG if out of range.
 * The environment variable TPCOL_GEMV_MAX_M (an integer 0..16), read when the
 * library loads, sets the initial value. */
int tp_set_gemv_max_m(int max_m);

/* Static description of a status code.  Never NULL. */
const char *tp_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none). */
const char *tp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TPCOL_H */
