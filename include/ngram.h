/*
 * ngram.h — C ABI of libngram.so: the hashed n-gram embedding gather-sum on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  "Qwen Brought Back N-Grams. All 51 Billion Parameters of
 * Them.", section "N-grams, of all things": for each token the bigram and
 * trigram context is hashed into one learned table (20,000,000 rows x 2560),
 * 16 rows are gathered and summed into one 2560-wide vector, which is added to
 * the residual stream.  "Qwen3.8-Flash-Next: A 51B N-gram Embedding Table
 * with Heterogeneous Memory Prefetch", Key point 1: the sum is fused with the
 * 1-gram embedding through an elementwise gate, h = e_1gram(w_t) + W_g (.) e_N.
 *
 * The pages leave the hash open.  This library fixes it:
 *   c0 = w_t, c1 = w_{t-1}, c2 = w_{t-2}, each a 21-bit field; context before
 *   a sequence's first token is the caller's 2-token history, else NGRAM_PAD_ID;
 *   bigram key  K2 = c1 << 21 | c0, trigram key K3 = c2 << 42 | c1 << 21 | c0;
 *   row_k = splitmix64(K ^ seed_k) mod R, K = K2 for k = 0..7, K3 for 8..15,
 *   where splitmix64(x) is the first output of Steele, Lea and Flood's
 *   splitmix64 generator from state x, and the default seed_k is output k of
 *   that generator from state 0.
 * Arithmetic: acc = +0.0f; for k = 0..15: acc += (float)T[row_k][j] (bf16
 * table), acc = fmaf((float)q[row_k][j], scale[row_k], acc) (int8 table) or
 * acc += e2m1 * 2^(E-127) (MXFP4 table, the product exact);
 * h = fmaf(W_g[j], acc, e1[w_t][j]) (or + 0 without e1); y = residual + h (or h);
 * out = bf16 round-to-nearest-even of y (NaN -> 0x7FC0).  The order is fixed,
 * so results are reproducible bit for bit.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned (hipMalloc / torch).  The library
 *     allocates nothing in a compute call, keeps no state between calls, and
 *     only enqueues work on `stream` (NULL = the default stream): no sync.
 *   - Row-major layouts; bf16 values are passed as their uint16_t bit pattern.
 *   - Return value: NGRAM_OK or a negative ngram_status.  Arguments are
 *     checked on the host before anything is enqueued; on error nothing is
 *     launched.  ngram_last_error() gives a message (thread-local).
 *   - Token ids in [0, V) (and < NGRAM_PAD_ID), history ids in [0, NGRAM_PAD_ID]
 *     and row ids in [0, R) are preconditions checked on the device: a token
 *     that breaks one gets NaN outputs (bf16 0x7FC0 / fp32 0x7FC00000) and row
 *     ids -1, and no memory outside the arguments is ever read.
 *   - seq_offsets[S+1] (int32, device) must rise from 0 to n; sequence s
 *     holds tokens seq_offsets[s] .. seq_offsets[s+1]-1; empty sequences are
 *     allowed.
 */
#ifndef NGRAM_H
#define NGRAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NGRAM_K 16                 /* rows per token: 8 bigram + 8 trigram seeds */
#define NGRAM_PAD_ID 0x1FFFFF      /* 2^21 - 1, context before a sequence start */
#define NGRAM_MAX_ROWS 2147483647  /* R <= 2^31 - 1 (row ids are int32) */
#define NGRAM_MAX_D 65536          /* row width limit */

typedef struct ihipStream_t* ngram_stream_t;   /* the same type as hipStream_t */

typedef enum {
    NGRAM_OK = 0,
    NGRAM_EINVAL = -1,   /* null pointer, negative size, bad enum, d % 8 != 0 */
    NGRAM_EALIGN = -2,   /* a pointer is not aligned as documented */
    NGRAM_ERANGE = -3,   /* R, d or V outside the supported range */
    NGRAM_EHIP = -4,     /* the HIP runtime reported an error */
    NGRAM_ENOTSUP = -5   /* a combination the library does not support */
} ngram_status;

typedef enum { NGRAM_TABLE_BF16 = 0, NGRAM_TABLE_INT8_ROWSCALE = 1, NGRAM_TABLE_MXFP4 = 2 } ngram_dtype;
typedef enum { NGRAM_IN_DEVICE = 0, NGRAM_IN_HOST = 1 } ngram_location;

/* The hashed table: [R][d] row-major.  bf16: data 16-byte aligned.  int8:
 * data 8-byte aligned and row_scale[R] fp32 (4-byte aligned), value of
 * element j of row r = q[r][j] * row_scale[r].  MXFP4 (OCP Microscaling FP4;
 * "Qwen 3.8 Flash-Next Deep Dive…", section 1, sizes the table at FP4): each
 * row is d/2 + d/32 bytes, the E2M1 codes (element 2m in the low nibble of
 * byte m) then one E8M0 scale per 32 elements; value = e2m1 * 2^(E-127), NaN
 * for E = 255; d a multiple of 128, data 16-byte aligned, row_scale unused.  location NGRAM_IN_DEVICE: data
 * and row_scale in device memory.  NGRAM_IN_HOST: data is pinned host memory
 * mapped for the device (ngram_host_alloc, or hipHostMalloc); rows are read
 * over PCIe by the GPU (zero copy); row_scale stays in device memory. */
typedef struct {
    const void* data;
    const float* row_scale;
    int64_t R;
    int32_t d;
    int32_t dtype;      /* ngram_dtype */
    int32_t location;   /* ngram_location */
    int32_t reserved;
} ngram_table;

/* Launch-shape overrides, for tuning and for tests that cover several tile
 * shapes; the plain entry points use the library's own choice.  Results are
 * bit-identical for every value: only the speed changes.
 *   tokens_per_workgroup: tokens a gather workgroup hashes into LDS and then
 *     gathers (0: the library's choice, 1 for bf16 tables, 4 for int8 and
 *     MXFP4 tables, 1 on the gated path for every table type; at most 64);
 *   host_workgroups: the grid cap for a table in pinned host memory, whose
 *     workgroups then loop over the tiles (0: the library's choice, 8). */
typedef struct {
    int32_t tokens_per_workgroup;
    int32_t host_workgroups;
} ngram_launch;

const char* ngram_status_string(int status);
const char* ngram_last_error(void);
int ngram_version(void);

/* seeds[k], k = 0..15: outputs 0..15 of the splitmix64 generator from state 0. */
void ngram_default_seeds(uint64_t seeds[NGRAM_K]);

/* Context and hash: "N-grams, of all things" + the fixed hash
 * above.  tokens[n] int32, seq_offsets[S+1] int32, history[S][2] int32 (w_{t-2},
 * w_{t-1} before the sequence) or NULL for pad, seeds: HOST array of 16 or
 * NULL for the defaults.  Writes rows_out[n][16] int32 (device).
 * Errors: EINVAL (null / n < 0 / S < 1 with n > 0), ERANGE (R outside
 * [1, 2^31-1]). */
int ngram_hash(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
               const int32_t* history, const uint64_t* seeds, int64_t R, int32_t* rows_out,
               ngram_stream_t stream);

/* Gather and sum: "N-grams, of all things": eN_out[i][j] =
 * the fp32 sum over k = 0..15 in order of row rows[i][k] of T (dequantised
 * inside the sum for int8).  rows[n][16] int32 (device), eN_out[n][d] fp32
 * (device, 16-byte aligned).  T may live in device or pinned host memory.
 * Errors: EINVAL, EALIGN, ERANGE (see ngram_table). */
int ngram_embed_bag(const ngram_table* T, const int32_t* rows, int64_t n, float* eN_out,
                    ngram_stream_t stream);
/* The same sums rounded to bf16 (nearest, ties to even; NaN to 0x7FC0) into
 * out[n][d] (bf16 bits, device, 16-byte aligned): the input of
 * ngram_project.  Other arguments and rules as ngram_embed_bag. */
int ngram_embed_bag_bf16(const ngram_table* T, const int32_t* rows, int64_t n, uint16_t* out,
                         ngram_stream_t stream);
/* The same with launch-shape overrides (NULL: none); EINVAL for values out of
 * range. */
int ngram_embed_bag_ex(const ngram_table* T, const int32_t* rows, int64_t n, float* eN_out,
                       const ngram_launch* launch, ngram_stream_t stream);

/* Gate and residual: "Qwen3.8-Flash-Next: …", Key point 1, and the
 * residual add of "N-grams, of all things": out[i][j] = bf16(residual[i][j] +
 * fmaf(W_g[j], eN[i][j], e1[tokens[i]][j])).  eN[n][d] fp32, tokens[n] int32,
 * e1[V][d] bf16 or NULL, W_g[d] fp32, residual[n][d] bf16 or NULL, out[n][d]
 * bf16; out may equal residual (in-place update).  All device, eN / e1 / W_g /
 * residual / out 16-byte aligned.  Errors: EINVAL, EALIGN, ERANGE (V < 1). */
int ngram_gate_add(const float* eN, const int32_t* tokens, int64_t n, int32_t d,
                   const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                   uint16_t* out, ngram_stream_t stream);

/* The whole path in one kernel: context, hash, gather, fp32 sum,
 * gate, residual add and bf16 rounding.  Same arguments and rules as the
 * three calls above; the row lists live in LDS; rows_out[n][16] (device) is
 * written when non-NULL.  Results are bit-identical to ngram_hash +
 * ngram_embed_bag + ngram_gate_add. */
int ngram_forward(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                  const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                  const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                  uint16_t* out, int32_t* rows_out, ngram_stream_t stream);
int ngram_forward_ex(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                     const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                     const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                     uint16_t* out, int32_t* rows_out, const ngram_launch* launch, ngram_stream_t stream);

/* Normalised, input-gated variant of ngram_forward.  "Qwen 3.8 Flash-Next
 * Deep Dive…" draws a "Projection / Normalization" stage after the lookup and
 * "Qwen3.8-Flash-Next: …" (summary) fuses the n-gram and 1-gram vectors "via a
 * gating network"; neither is defined there.  Form taken, per token, from its
 * fp32 sum eN:
 *   r      = 1 / sqrt(S / d + eps),   S = sum over j of eN[j]^2;
 *   n[j]   = eN[j] r gamma[j];
 *   logit  = sum over j of (u[j] e1[j] + v[j] n[j]) + b;
 *   alpha  = 1 / (1 + exp(-logit));
 *   out[j] = bf16(residual[j] + e1[w_t][j] + alpha W_g[j] n[j]).
 * Everything after eN is evaluated in float64 and the output is rounded once
 * to bf16 from the float64 value (ties to even).  The sums have no stated
 * order, so r and the logit can differ from another float64 evaluation by a
 * few units in the last place (a relative error of order d 2^-53).
 * e1 [V][d] bf16 is required; gamma, u, v [d] fp32 (device, 16-byte aligned);
 * eps finite >= 0, b finite; d <= 8192 (ERANGE).  stats_out [n][2] float64
 * (device, 8-byte aligned, may be NULL) receives (r, logit) per token, NaN
 * for an invalid token.  Other arguments and rules as ngram_forward. */
int ngram_forward_gated(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                        const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                        const uint16_t* e1, int64_t V, const float* W_g, const float* gamma,
                        const float* u, const float* v, float b, float eps,
                        const uint16_t* residual, uint16_t* out, int32_t* rows_out,
                        double* stats_out, ngram_stream_t stream);
int ngram_forward_gated_ex(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                           const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                           const uint16_t* e1, int64_t V, const float* W_g, const float* gamma,
                           const float* u, const float* v, float b, float eps,
                           const uint16_t* residual, uint16_t* out, int32_t* rows_out,
                           double* stats_out, const ngram_launch* launch, ngram_stream_t stream);

/* The normalised, input-gated epilogue of ngram_forward_gated on given fp32
 * sums: eN[n][d] (device, 16-byte aligned) takes the place of the gathered
 * sums, tokens[n] (device int32) names each token's e1 row (an id outside
 * [0, V) gives NaN outputs and NaN stats).  Same formula, precision, rounding
 * and arguments as ngram_forward_gated; the sums over j run in the same order,
 * so ngram_embed_bag followed by this call gives bit for bit what
 * ngram_forward_gated gives.  With ngram_project in between it is the
 * projected path: lookup, projection, normalisation and gate. */
int ngram_norm_gate_add(const float* eN, const int32_t* tokens, int64_t n, int32_t d, const uint16_t* e1,
                        int64_t V, const float* W_g, const float* gamma, const float* u, const float* v, float b,
                        float eps, const uint16_t* residual, uint16_t* out, double* stats_out,
                        ngram_stream_t stream);

/* Projection: "Qwen 3.8 Flash-Next Deep Dive…", section 1, draws a
 * "Projection / Normalization" stage between the lookup and the trunk and
 * does not define it.  Form taken: a learned linear map of each token's sum
 * x (d_in columns) to d_out columns, with x and the weights P [d_out][d_in]
 * in bf16 (the model's storage type; ngram_embed_bag_bf16 gives x as the
 * fp32 sums rounded to bf16):
 *   y[i][o] = sum over j of P[o][j] * x[i][j].
 * Each product is exact and the sum is accumulated in fp32 by the matrix
 * cores in an order this library does not fix, so y can differ from another
 * fp32 evaluation by up to about d_in 2^-24 sum |terms|.  x[n][d_in] and
 * P (bf16 bits), y[n][d_out] fp32: device, row-major, 16-byte aligned; d_in a
 * multiple of 64 and d_out of 8 (EINVAL otherwise), both <= NGRAM_MAX_D
 * (ERANGE); n >= 0 (n = 0 launches nothing). */
int ngram_project(const uint16_t* x, int64_t n, int32_t d_in, const uint16_t* P, int32_t d_out, float* y,
                  ngram_stream_t stream);

/* Pinned-host-table path, "N-grams, of all things" / "Which is why the
 * offload matters more than the parameter count": the table shard sits in
 * pinned host memory and the selected rows are gathered by the GPU over PCIe
 * on a side stream, overlapped with compute on the main stream.
 *
 * ngram_host_alloc: pinned, device-mapped, 4 KiB-aligned host memory of
 * `bytes` bytes (hipHostMalloc); *host_ptr receives it; free with
 * ngram_host_free.  These two are the only calls that allocate. */
int ngram_host_alloc(int64_t bytes, void** host_ptr);
int ngram_host_free(void* host_ptr);

/* Stage the distinct rows a batch selects from a table in pinned host memory
 * in device memory: "Qwen Brought Back N-Grams…", section "Which is why the
 * offload matters more than the parameter count" (the selected rows of the
 * pinned-host shard gathered into a small BF16 GPU buffer on a dedicated
 * stream), and "Qwen3.8-Flash-Next: A 51B N-gram Embedding Table with
 * Heterogeneous Memory Prefetch", Key point 3 (a DMA pipeline over PCIe 5.0
 * that moves the rows while the GPU computes; T_DMA = K d S / BW).
 *   rows[n][16] int32 (device): the batch's row ids.
 *   stage_out [16 n][row] (device, 16-byte aligned, room for 16 n rows):
 *     stage row u = T_host row U_u, for the distinct valid row ids U_0,
 *     U_1, … (each once, in an unspecified order); stage_scale_out[u] (int8
 *     tables, device) its row scale, else may be NULL.
 *   remap_out[n][16] int32 (device): the stage row of rows[i][k], or -1 where
 *     rows[i][k] is outside [0, R).
 *   *n_staged_out (device int64): the number of distinct rows staged.
 * ngram_embed_bag on the stage (as a device table of 16 n rows) with
 * remap_out then gives exactly what ngram_embed_bag gives on T_host with rows.
 *   mode 0 (zero copy): a capped grid of GPU workgroups reads each distinct
 *     row over PCIe through the device mapping and writes it to the stage.
 *     Only enqueues work on `stream`.
 *   mode 1 (async copy): the GPU finds the distinct rows, the call reads
 *     their list back into `pinned` (it waits for `stream` up to that point),
 *     then enqueues one host-to-device copy per distinct row on `stream` (the
 *     DMA engines move the bytes, no compute unit is used) and returns.  Not
 *     capturable in a HIP graph.
 * workspace: device memory of ngram_gather_host_workspace_bytes(n, d) bytes,
 * 16-byte aligned; pinned (mode 1 only, else may be NULL): pinned host memory
 * (ngram_host_alloc) of ngram_gather_host_pinned_bytes(n) bytes, 16-byte
 * aligned.  Calls that can overlap need a workspace and a pinned buffer each.
 * Run it on a side stream and join with an event.  Errors: EINVAL, EALIGN,
 * ERANGE (n > 2^26), ENOTSUP when T_host is not in host memory, EHIP. */
int64_t ngram_gather_host_workspace_bytes(int64_t n, int32_t d);
int64_t ngram_gather_host_pinned_bytes(int64_t n);
int ngram_gather_host(const ngram_table* T_host, const int32_t* rows, int64_t n, void* workspace,
                      int64_t workspace_bytes, void* pinned, int64_t pinned_bytes, void* stage_out,
                      float* stage_scale_out, int32_t* remap_out, int64_t* n_staged_out, int32_t mode,
                      ngram_stream_t stream);

/* Row pool in front of a pinned-host table: a hot-row cache in HBM plus a
 * per-batch gather of the distinct missing rows.  "Qwen 3.8 Flash-Next Deep
 * Dive…", section 1, calls phrase frequency heavily Zipfian, so a small set of
 * rows carries much of the traffic; "Qwen Brought Back N-Grams…", section
 * "Which is why the offload matters more than the parameter count", reads the
 * rows of a pinned-host shard over PCIe, which bounds the host gather.  Every pool
 * row is an exact copy of a table row, so summing from the pool gives
 * bit-identical results to summing from the host table.
 *
 * data [pool_rows][d] in the table's dtype (device, 16-byte aligned);
 * row_scale [pool_rows] fp32 for int8 tables, else NULL; slot_of_row [R] int32
 * (device): the pool row that caches table row r, or -1.  Pool rows
 * [0, cached) hold cached rows; rows [cached, pool_rows) stage misses.  All
 * three buffers are caller-owned. */
typedef struct {
    void* data;
    float* row_scale;
    int32_t* slot_of_row;
    int64_t pool_rows;
    int64_t cached;
} ngram_row_pool;

/* Bytes of device workspace ngram_pool_gather needs for n tokens, and that
 * ngram_select_hot_rows needs (n = 0). */
int64_t ngram_pool_workspace_bytes(int64_t n);

/* Empty the cache: slot_of_row[r] = -1 for all r, P->cached = 0. */
int ngram_pool_reset(const ngram_table* T_host, ngram_row_pool* P, ngram_stream_t stream);

/* Cache table rows hot_rows[0..C) (device int32) in pool rows 0..C-1 (read
 * over PCIe) and point slot_of_row at them, after clearing it; duplicate or
 * out-of-range ids leave their pool row unused.  Sets P->cached = C.
 * Errors: EINVAL, ERANGE (C > pool_rows), ENOTSUP (T_host not in host memory). */
int ngram_pool_cache_rows(const ngram_table* T_host, ngram_row_pool* P, const int32_t* hot_rows,
                          int64_t C, ngram_stream_t stream);

/* Per batch: map rows[n][16] to pool rows.  A cached row maps to its slot;
 * each distinct uncached row is read over PCIe exactly once into pool row
 * cached + u (u = 0, 1, … in an unspecified order); an out-of-range row id
 * maps to -1.  Writes pool_rows_out[n][16] (device int32) and, if non-NULL,
 * *fetched_out (device int64) = the number of distinct rows read over PCIe.
 * ngram_embed_bag on the pool (as a device table of pool_rows rows) with
 * pool_rows_out then gives exactly ngram_embed_bag(T_host, rows).
 * Needs P->pool_rows >= P->cached + 16 * n (ERANGE) and a device workspace of
 * ngram_pool_workspace_bytes(n) bytes, 16-byte aligned (EINVAL). */
int ngram_pool_gather(const ngram_table* T_host, const ngram_row_pool* P, const int32_t* rows,
                      int64_t n, int32_t* pool_rows_out, int64_t* fetched_out, void* workspace,
                      int64_t workspace_bytes, ngram_stream_t stream);

/* counts[r] += number of (token, k) with rows[i][k] == r, for r in [0, R);
 * accumulate = 0 clears counts first.  counts [R] int32, device. */
int ngram_count_rows(const int32_t* rows, int64_t n, int64_t R, int32_t* counts, int32_t accumulate,
                     ngram_stream_t stream);

/* Choose up to C hot rows from counts[R]: every row whose count reaches the
 * smallest threshold that keeps the set within C (counts above 1023 count as
 * 1023; where even the top value holds more than C rows, C of them are taken
 * in an unspecified order).  Rows never counted are not chosen.  Writes
 * hot_rows_out[0..*selected) (device int32, C entries of room) and *selected
 * (HOST int64).  Synchronizes `stream` (it reads a 1024-bin histogram back),
 * so it belongs between batches, not in a captured graph.  Workspace:
 * ngram_pool_workspace_bytes(0) bytes of device memory. */
int ngram_select_hot_rows(const int32_t* counts, int64_t R, int64_t C, int32_t* hot_rows_out,
                          int64_t* selected, void* workspace, int64_t workspace_bytes,
                          ngram_stream_t stream);

/* Gradients of a learned table ("Qwen Brought Back N-Grams…", section
 * "N-grams, of all things": "a learned, hash-addressed embedding table").  The
 * pages define only the forward; these follow from it by the chain rule, with
 * the bf16 output rounding passed straight through.  dout = dL/dout, bf16
 * [n][d]; rows = the forward's row ids [n][16] (a token whose ids are -1 or
 * outside [0, R) contributes nothing).  Each sum runs in a fixed order, so
 * every result is reproducible bit for bit, with no floating-point atomics:
 * the ids are grouped by a stable radix sort that keeps positions ascending.
 * Workspace: ngram_grad_workspace_bytes(n, d) bytes of device memory,
 * 256-byte aligned; calls in order on one stream may share one workspace,
 * calls that can run at the same time (on different streams) need one each.
 * The table gradient is bound by HBM bandwidth, the e1 and gate gradients by
 * their in-order chains, so running ngram_grad_e1 and ngram_grad_gate on a
 * second stream beside ngram_grad_table hides most of them.  n <= 2^20
 * (ERANGE). */
int64_t ngram_grad_workspace_bytes(int64_t n, int32_t d);

/* Table gradient, sparse: for each distinct valid row id r in ascending order
 * u = 0, 1, …: grad_rows_out[u] = r and grad_out[u][j] = acc over positions
 * t = 16 i + k with rows[t] == r, ascending t, of acc = fmaf(W_g[j],
 * dout[i][j], acc) from +0.  *n_unique_out (device int64) = the number of
 * rows.  grad_rows_out holds 16 n int32, grad_out 16 n x d fp32 (16-byte
 * aligned); entries from *n_unique_out on are unspecified. */
int ngram_grad_table(const int32_t* rows, int64_t n, int32_t d, int64_t R, const float* W_g,
                     const uint16_t* dout, int32_t* grad_rows_out, float* grad_out,
                     int64_t* n_unique_out, void* workspace, int64_t workspace_bytes,
                     ngram_stream_t stream);

/* e1 gradient, sparse: for each distinct token v in [0, V) of a valid
 * position, ascending: grad_tokens_out[u] = v, grad_out[u][j] = acc over
 * tokens i with tokens[i] == v, ascending i, of acc = acc + dout[i][j] from
 * +0.  grad_tokens_out holds n int32, grad_out n x d fp32. */
int ngram_grad_e1(const int32_t* tokens, const int32_t* rows, int64_t n, int32_t d, int64_t V,
                  const uint16_t* dout, int32_t* grad_tokens_out, float* grad_out,
                  int64_t* n_unique_out, void* workspace, int64_t workspace_bytes,
                  ngram_stream_t stream);

/* Gate gradient: grad_Wg_out[j] = the sum over valid tokens i of
 * dout[i][j] eN[i][j], accumulated in float64 (every product is exact there)
 * and rounded once to fp32; the sum has no stated order, but the library's
 * is fixed, so the bits are reproducible.  eN [n][d] fp32 is the forward's
 * sum (ngram_embed_bag); grad_Wg_out [d] fp32. */
int ngram_grad_gate(const int32_t* rows, const uint16_t* dout, const float* eN, int64_t n, int32_t d,
                    float* grad_Wg_out, void* workspace, int64_t workspace_bytes,
                    ngram_stream_t stream);

/* The gate gradient with no workspace argument and no allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).  Same result, bit for bit,
 * as ngram_grad_gate.  Its float64 chunk partials (ceil(n / 128) x d of them)
 * live in a static device array of 16 MiB that the library holds on each GPU
 * it runs on until the process ends: ceil(n / 128) * d must not exceed
 * ngram_grad_gate_noalloc_max_elements() (2^21), else ERANGE and nothing is
 * launched.  Calls on one GPU share that array, so calls that can overlap on
 * one GPU (different streams, or other threads) race: serialise them.  The
 * calling thread's current device must be the stream's device.  Other
 * arguments, rules and errors as ngram_grad_gate. */
int64_t ngram_grad_gate_noalloc_max_elements(void);
int ngram_grad_gate_noalloc(const int32_t* rows, const uint16_t* dout, const float* eN, int64_t n, int32_t d,
                            float* grad_Wg_out, ngram_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NGRAM_H */
