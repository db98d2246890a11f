/*
 * crisp.h -- C ABI of the CRISP sparse-attention prefill on MI355X (gfx950).
 *
 * The method is the one of the paper digest page "CRISP: Cliff-awaRe
 * Input-adaptive Sparse Prefilling with Structural-Mass-Motivated Routing"
 * (called "the digest" below): per attention head, a proxy softmax of the last
 * b = 128 queries against all keys (PatSearch, Algorithm 2) routes the head to
 * Vertical-Slash or Pooled-Estimation by its structural mass C_struct; VS heads
 * keep the 128-token key blocks above a sink-aware noise floor (VSIndex,
 * Algorithm 3), PE heads keep blocks by a gamma-cumsum over a pooled block map
 * (PEIndex, Algorithm 4); exact masked softmax attention then runs over the
 * selected blocks only (Algorithm 1, method-steps section step 4).
 *
 * The three method calls split Algorithm 1 at its intermediate results:
 *   crisp_route       -> (pattern, block reductions of the proxy A_hat)
 *   crisp_select      -> the index set S as a block CSR
 *   crisp_sparse_attn -> A(Q, K, V, S)
 * dense_attn computes exact causal attention over every block, the dense
 * baseline the digest's speedups are measured against.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout.  Q and the output O are [batch][h_q][n][d]; K and V are
 *   [batch][h_kv][n][d]; all contiguous, row-major, bf16 bit patterns for
 *   Q/K/V.  Query head h reads KV head h / (h_q / h_kv).
 * Memory.  Every buffer is a device pointer (hipMalloc'ed or a torch CUDA
 *   tensor), 16-byte aligned, owned and freed by the caller.  The library
 *   never allocates, frees or synchronises; every kernel is enqueued on
 *   `stream` (a hipStream_t; NULL = the default stream).  Outputs are complete
 *   once the stream reaches that point.
 * Errors.  Arguments are validated on the host before any HIP call, so a bad
 *   argument returns its status without touching the GPU.  A failed launch
 *   returns CRISP_ERR_HIP (crisp_last_error() gives the HIP message).  After a
 *   non-OK return the outputs are unspecified.  No C++ exception crosses the ABI.
 * Threads.  The library holds no global state except a thread-local error
 *   string; concurrent calls on different streams are safe when their buffers
 *   do not overlap.  Results are bitwise deterministic.
 * Empty input.  batch == 0 is valid and enqueues nothing.
 */
#ifndef CRISP_H_
#define CRISP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem shape.  n % 128 == 0 and 384 <= n <= 1048576 (at least three key
 * blocks, so that the noise floor's N_b - 2 is positive); d in {64, 128};
 * h_q % h_kv == 0; batch >= 0; batch*h_q <= 65535 and
 * batch*h_q*(n/128) < 2^24.  Otherwise CRISP_ERR_SHAPE. */
typedef struct {
  int32_t batch, n, h_q, h_kv, d;
} crisp_shape;

/* Method settings (digest, method-steps section and reproducibility notes).
 * block, last_q, w_sink, w_local: the block size B, the proxy size b and the
 *   anchor widths; only 128 is supported (CRISP_ERR_UNSUPPORTED otherwise).
 * k_min_tokens: minimum per-direction VS budget in tokens (1024 on the pages),
 *   a non-negative multiple of block (CRISP_ERR_PARAM otherwise).
 * tau: routing threshold, VS iff C_struct >= tau (0.2).  Finite.
 * alpha: noise-floor multiplier, keep p > alpha * mu (1.0 or 1.25).  >= 0.
 * gamma: PE coverage target, 0 < gamma <= 1 (0.95). */
typedef struct {
  int32_t block, last_q, w_sink, w_local, k_min_tokens;
  float tau, alpha, gamma;
} crisp_cfg;

enum crisp_status {
  CRISP_OK = 0,
  CRISP_ERR_NULL = -1,        /* a required pointer is NULL                 */
  CRISP_ERR_SHAPE = -2,       /* shape outside the supported range          */
  CRISP_ERR_PARAM = -3,       /* setting out of range                       */
  CRISP_ERR_UNSUPPORTED = -4, /* valid on the pages, not implemented here   */
  CRISP_ERR_WORKSPACE = -5,   /* ws_bytes smaller than the size query gives */
  CRISP_ERR_CAPACITY = -6,    /* col_capacity below crisp_max_blocks        */
  CRISP_ERR_HIP = -7,         /* a HIP launch failed                        */
  CRISP_ERR_ALIGN = -8,       /* a device pointer is not 16-byte aligned    */
  CRISP_ERR_SCRATCH = -9      /* shape needs more than the static scratch   */
};

enum crisp_out_dtype { CRISP_OUT_F32 = 0, CRISP_OUT_BF16 = 1 };

enum crisp_call {
  CRISP_CALL_ROUTE = 0, CRISP_CALL_SELECT = 1, CRISP_CALL_ATTN = 2, CRISP_CALL_DENSE = 3,
  CRISP_CALL_FLEX_ROUTE = 4, CRISP_CALL_FLEX_SELECT = 5
};

/* Device workspace in bytes that `call` needs for this shape (pure host
 * arithmetic, no HIP call).  Writes *bytes; returns a status.  The workspace
 * is scratch: its contents on entry do not matter and are clobbered. */
int crisp_workspace_bytes(const crisp_shape* shape, const crisp_cfg* cfg, int call, size_t* bytes);

/* Worst-case number of selected (query block, key block) tiles over all heads:
 * batch * h_q * N_b * (N_b + 1) / 2 (every causal tile).  The col_idx capacity
 * crisp_select requires.  Pure host arithmetic. */
int crisp_max_blocks(const crisp_shape* shape, int64_t* blocks);

/* PatSearch (digest: core-method section and the Algorithm 2 caption).
 * For every (batch, query head) with Q_hat = its last 128 query rows, the
 * causal proxy A_hat = Softmax(Q_hat K^T / sqrt(d)) is formed tile by tile
 * (never stored) and reduced to
 *   p_vert[kb]  = (1/b) sum_i sum_{j in key block kb} A_hat[i, j]
 *   p_slash[kb] = (1/b) sum over entries on diagonals t = j + b-1-i with
 *                 floor(t / 128) = kb,
 *   c_struct    = p_vert[0] + p_vert[N_b-1]  (mass on the first and last 128 keys),
 *   pattern     = 1 (Vertical-Slash) if c_struct >= tau else 0 (Pooled-Estimation).
 * q_bf16 [batch][h_q][n][d], k_bf16 [batch][h_kv][n][d] (read);
 * c_struct [batch*h_q] f32, pattern [batch*h_q] int8,
 * p_vert, p_slash [batch*h_q][N_b] f32 (written).  Reductions are fp32 in a
 * fixed order.  ws: crisp_workspace_bytes(CRISP_CALL_ROUTE) bytes. */
int crisp_route(const crisp_shape* shape, const crisp_cfg* cfg,
                const void* q_bf16, const void* k_bf16,
                float* c_struct, int8_t* pattern, float* p_vert, float* p_slash,
                void* ws, size_t ws_bytes, void* stream);

/* crisp_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels, arguments and outputs as crisp_route, with the workspace
 * replaced by a static device buffer of CRISP_ROUTE_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine); the
 * caller still passes the inputs and outputs.  Shapes whose routing workspace
 * (crisp_workspace_bytes(CRISP_CALL_ROUTE), about 1.6 KiB per query head and
 * key block) exceeds the buffer return CRISP_ERR_SCRATCH before any HIP call
 * (64 MiB covers, e.g., 32 query heads at up to 131072 tokens; 32 heads at
 * 524288 tokens need about 206 MiB).  Every call on a GPU shares that GPU's buffer:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  Nothing in the buffer needs clearing between
 * calls: each kernel writes all of the scratch it later reads.  Other errors
 * as crisp_route. */
#define CRISP_ROUTE_SCRATCH_BYTES (64u << 20)
int crisp_route_noalloc(const crisp_shape* shape, const crisp_cfg* cfg,
                        const void* q_bf16, const void* k_bf16,
                        float* c_struct, int8_t* pattern, float* p_vert, float* p_slash,
                        void* stream);

/* Index selection: VSIndex for pattern 1 heads, PEIndex for pattern 0 heads
 * (digest: method-steps section steps 2-3, Algorithm 3 and 4 captions, and the
 * prerequisite section on the cumulative-coverage threshold).
 * VS head, per direction d in {vert, slash}:
 *   mu = max(1 - p_d[0] - p_d[N_b-1], 0) / (N_b - 2); keep the blocks with
 *   p_d > alpha*mu, at least k_min_tokens/128 of them (top-k, ties to the lower
 *   index) and at most N_b; then add blocks 0 and N_b-1.  Vertical block kb
 *   selects key block kb; slash block k selects the block diagonal N_b-1-k.
 * PE head: mean-pooled Q and K blocks give the block-causal softmax map A_bar;
 *   x = A_bar / N_b over the cells kb <= qb is ordered descending (ties to the
 *   lower flat index qb*N_b + kb) and the shortest prefix with sum >= gamma is
 *   kept; every row also keeps its diagonal block.
 * Output: block CSR over rows r = (b*h_q + h)*N_b + qb: row_ptr
 *   [batch*h_q*N_b + 1] int64 (row_ptr[0] = 0; the total is left in device
 *   memory at row_ptr[last]), col_idx int32 key-block indices, ascending and
 *   distinct within each row, all <= qb.  col_capacity (entries of col_idx)
 *   must be >= crisp_max_blocks(shape), checked on the host.
 * sel_mask (optional, may be NULL): [batch*h_q][2][N_b] uint8, for VS heads
 *   1 where a vertical ([0][kb]) or slash ([1][k]) block is selected, all 0 for
 *   PE heads.
 * pattern, p_vert, p_slash are crisp_route's outputs (any values accepted).
 * ws: crisp_workspace_bytes(CRISP_CALL_SELECT) bytes. */
int crisp_select(const crisp_shape* shape, const crisp_cfg* cfg,
                 const void* q_bf16, const void* k_bf16,
                 const int8_t* pattern, const float* p_vert, const float* p_slash,
                 int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                 uint8_t* sel_mask, void* ws, size_t ws_bytes, void* stream);

/* Exact block-sparse attention A(Q, K, V, S) = Softmax(QK^T/sqrt(d) + M_S) V,
 * causal (digest: prerequisite section on prefill and sparse attention).
 * Query p in block qb attends to the keys j <= p of the key blocks listed in
 * CSR row (b*h_q + h)*N_b + qb.  row_ptr/col_idx as produced by crisp_select
 * (any CSR is accepted: row ranges are clamped to [0, col_capacity], entries
 * outside [0, qb] are skipped).  A query with no visible key gets output 0.
 * out: [batch][h_q][n][d], f32 (CRISP_OUT_F32) or bf16 (CRISP_OUT_BF16).
 * bf16 MFMA for QK^T and PV with fp32 accumulation; softmax in fp32 with P
 * rounded to bf16 for the PV product and the row sums taken over those same
 * rounded weights, so the choice of each row's softmax reference maximum m
 * cancels in the normalisation.  At d = 128, m is the maximum of the row's
 * first 64 keys whenever the Cauchy-Schwarz bound of every logit of the row
 * (|q| times the largest key norm of its KV head, over sqrt(d)) lies at most
 * 64 log2 units above it (weights then stay below 2^64); otherwise, and at
 * d = 64, m is raised whenever a 64-key stage's maximum exceeds it by more
 * than 2^8.
 * ws: crisp_workspace_bytes(CRISP_CALL_ATTN) bytes (work-queue counters, the
 * largest key norm of each KV head and a V^T copy of V; the call resets them,
 * so concurrent calls must not share one workspace). */
int crisp_sparse_attn(const crisp_shape* shape, const crisp_cfg* cfg,
                      const void* q_bf16, const void* k_bf16, const void* v_bf16,
                      const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                      void* out, int out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Dense exact causal attention (the result FlashAttention computes; digest,
 * prerequisite section on FlashAttention): crisp_sparse_attn with every key
 * block kb <= qb selected, same kernels and precision.
 * ws: crisp_workspace_bytes(CRISP_CALL_DENSE) bytes (as for
 * crisp_sparse_attn). */
int dense_attn(const crisp_shape* shape, const void* q_bf16, const void* k_bf16,
               const void* v_bf16, void* out, int out_dtype, void* ws, size_t ws_bytes,
               void* stream);

/* Variants of VSIndex on the same kernels (bits of `variant`):
 * CRISP_VARIANT_MEDIAN_FLOOR: mu = the median of the N_b - 2 non-anchor
 *   block scores instead of their mean (the digest's limitations and
 *   weakness notes, Table 9); the rest of the rule is unchanged.
 * CRISP_VARIANT_SLASH_BAND: a selected slash block covers the token offsets
 *   128 delta .. 128 delta + 127, which reach the tiles of block diagonals
 *   delta and delta + 1; both are selected (the default selects delta only).
 * CRISP_VARIANT_PE_PER_ROW: PE heads run the gamma-cumsum inside each query-
 *   block row of the pooled map (each row a distribution over kb <= qb: the
 *   row keeps its shortest descending prefix reaching gamma, ties to the lower
 *   block, plus its diagonal) instead of over the whole flattened map (the
 *   digest's PEIndex steps leave the flattening's extent open).
 * Everything else (arguments, workspace CRISP_CALL_SELECT, errors) is as for
 * crisp_select; unknown bits give CRISP_ERR_PARAM. */
enum crisp_variant { CRISP_VARIANT_MEDIAN_FLOOR = 1, CRISP_VARIANT_SLASH_BAND = 2, CRISP_VARIANT_PE_PER_ROW = 4 };
int crisp_select_variant(const crisp_shape* shape, const crisp_cfg* cfg, int variant, const void* q_bf16,
                         const void* k_bf16, const int8_t* pattern, const float* p_vert, const float* p_slash,
                         int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws,
                         size_t ws_bytes, void* stream);

/* The FlexPrefill baseline: the routing and VS budget rule that CRISP
 * replaces, on the same kernels (digest: prerequisite sections on
 * Jensen-Shannon divergence and on the cumulative-coverage threshold).
 *
 * flex_route: given p_vert from crisp_route (a_hat, the proxy's block-pooled
 * key distribution), forms a_bar[kb] = softmax over key blocks of
 * mean(last 128 query rows) . mean(K rows of block kb) / sqrt(d), and writes
 * jsd[bh] = D_JS(a_hat, a_bar) = 1/2 KL(a_hat||m) + 1/2 KL(a_bar||m),
 * m = (a_hat + a_bar)/2, natural log, and pattern[bh] = 1 (VS) iff
 * jsd >= tau_jsd, else 0 (PE).  The pages give no value for tau_jsd.
 * q, k as for crisp_route; p_vert [batch*h_q][N_b] fp32 (device, read);
 * jsd [batch*h_q] fp32 and pattern [batch*h_q] int8 (device, written).
 * ws: crisp_workspace_bytes(CRISP_CALL_FLEX_ROUTE) bytes (pooled keys).
 * Errors: as crisp_route; CRISP_ERR_PARAM for a negative or non-finite tau_jsd. */
int flex_route(const crisp_shape* shape, const crisp_cfg* cfg, float tau_jsd, const void* q_bf16,
               const void* k_bf16, const float* p_vert, float* jsd, int8_t* pattern, void* ws,
               size_t ws_bytes, void* stream);

/* flex_select: crisp_select with the per-direction VS rule replaced by the
 * gamma-cumsum budget (cfg->gamma): the shortest prefix of p_d sorted
 * descending (ties to the lower block) whose sum reaches gamma, its count
 * clipped to [k_min, N_b], then the anchor blocks 0 and N_b-1.  PE heads,
 * the CSR and every argument and error are as for crisp_select (cfg->alpha
 * is not used).  ws: crisp_workspace_bytes(CRISP_CALL_FLEX_SELECT) bytes. */
int flex_select(const crisp_shape* shape, const crisp_cfg* cfg, const void* q_bf16, const void* k_bf16,
                const int8_t* pattern, const float* p_vert, const float* p_slash, int64_t* row_ptr,
                int32_t* col_idx, int64_t col_capacity, uint8_t* sel_mask, void* ws, size_t ws_bytes,
                void* stream);

/* Sequence length below which the sparse path does not pay for itself.
 * Routing and selection cost a near-fixed 0.12-0.2 ms below 16K tokens and a
 * short causal map has few tiles to skip, so dense attention wins on short
 * inputs (the digest's limitations paragraph, item 7, reports the same, with
 * the crossover between 8K and 64K tokens on its GPU).  Measured on one
 * MI355X with Llama-shaped layers (32 query / 8 KV heads, d = 128, 75% VS
 * heads): dense / sparse layer time 0.88-0.98 at n = 6144 and 1.06-1.15 at
 * n = 7168 (four runs). */
#define CRISP_DENSE_BELOW_TOKENS 7168

/* Which path a prefill of this shape takes: *use_dense = 1 when
 * shape->n < CRISP_DENSE_BELOW_TOKENS (call dense_attn), else 0 (call
 * crisp_route, crisp_select and crisp_sparse_attn).  The shape is validated
 * as for the other calls.  Pure host logic; returns a status. */
int crisp_use_dense(const crisp_shape* shape, int32_t* use_dense);

/* ---- measurement: the sustained bf16 MFMA rate of this GPU ----
 * For callers that report a kernel against the MFMA roofline of the running
 * part (the benchmark).  Launches one workgroup of 512 threads per CU (two
 * waves per SIMD); each wave issues 32 v_mfma_f32_32x32x16_bf16 per iteration
 * on register operands loaded from `operands` (device, CRISP_PROBE_OPERAND_BYTES
 * bytes of bf16 values chosen by the caller: the sustained rate of a
 * power-limited part depends on the data).  Workgroup i writes one float to
 * sink[i % CRISP_PROBE_SINK_FLOATS] (device).  *flop (host) receives the work
 * of the launch (32768 FLOP per MFMA); the caller times the launch on
 * `stream`.  Errors: CRISP_ERR_NULL, CRISP_ERR_ALIGN (16-byte operands, 4-byte
 * sink), CRISP_ERR_PARAM (iters outside [1, 10^7]), CRISP_ERR_HIP. */
#define CRISP_PROBE_OPERAND_BYTES 65536
#define CRISP_PROBE_SINK_FLOATS 4096
int crisp_mfma_probe(const void* operands, float* sink, int iters, double* flop, void* stream);

/* Static description of a status code. */
const char* crisp_status_string(int status);

/* Detail of the last CRISP_ERR_HIP on the calling thread ("" if none). */
const char* crisp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CRISP_H_ */
