/*
 * CPU oracle for the hashed n-gram embedding gather-sum.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library; it is written from the definitions below and nothing else.
 *
 * What is computed, and where it is stated:
 *   - "Qwen Brought Back N-Grams. All 51 Billion Parameters of Them.",
 *     section "N-grams, of all things": per token, the bigram and trigram
 *     context is hashed into one 20M-row table, 16 rows are gathered and
 *     summed into one 2560-wide vector, which is added to the residual stream.
 *   - "Qwen3.8-Flash-Next: A 51B N-gram Embedding Table with Heterogeneous
 *     Memory Prefetch", Key point 1, the fusion equation
 *     h0 = e_1gram(w_t) + W_g (elementwise) e_Ngram, and "a deterministic hash".
 *   - Key point 3 of the same page: the INT8 table size.
 *
 * The pages leave the hash, the packing, the seeds, the padding, the order of
 * the sum and the rounding open.  The readings taken (each one a plain
 * choice, not a claim about the pages):
 *   - hash: splitmix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom
 *     Number Generators", OOPSLA 2014; finaliser constants of Vigna's public
 *     domain splitmix64): splitmix64(x) is the generator's first output from
 *     state x, i.e. mix(x + gamma);
 *   - keys: 21-bit fields; bigram K2 = c1<<21 | c0, trigram
 *     K3 = c2<<42 | c1<<21 | c0, with c0 = w_t, c1 = w_{t-1}, c2 = w_{t-2};
 *   - rows: row_k = splitmix64(key_k XOR seed_k) mod R, key_k = K2 for
 *     k = 0..7 and K3 for k = 8..15; default seed_k = splitmix64(k * gamma);
 *   - context before a sequence's first token: the caller's 2-token history
 *     when given, else the pad id 2^21 - 1;
 *   - sum: fp32, starting from +0, k = 0..15 in order; int8 rows are
 *     dequantised inside the sum as acc = fmaf(q, scale_row, acc);
 *   - gate: h = fmaf(W_g[j], acc, e1[w_t][j]) (or + 0 without e1);
 *     y = residual + h (or h without residual); out = bf16 round-to-nearest-
 *     even of y, NaN to the canonical quiet NaN 0x7FC0.
 * Build with -ffp-contract=off: every fp32 operation above is one IEEE
 * operation, and fmaf is the C library's correctly rounded fused multiply-add.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_K 16
#define ORACLE_PAD 0x1FFFFF
#define ORACLE_GAMMA 0x9E3779B97F4A7C15ull

/* splitmix64: one output of the generator from state x (mod 2^64). */
uint64_t oracle_splitmix64(uint64_t x)
{
    uint64_t z = x + ORACLE_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Outputs 0..15 of the splitmix64 generator started from state 0. */
void oracle_default_seeds(uint64_t seeds[ORACLE_K])
{
    for (int k = 0; k < ORACLE_K; ++k)
        seeds[k] = oracle_splitmix64((uint64_t)k * ORACLE_GAMMA);
}

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round an fp32 value to the nearest bf16, ties to even. */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f))
        return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void oracle_bf16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

/*
 * The n-gram context of every token: ctx[i] = (c0, c1, c2) = (w_t, w_{t-1},
 * w_{t-2}).  Sequence s holds tokens seq_offsets[s] .. seq_offsets[s+1]-1.
 * Its extended stream is [h0, h1, tokens of s...] with (h0, h1) = history[s]
 * or (PAD, PAD); position p of s reads c1 = ext[p+1], c2 = ext[p].
 */
void oracle_context(const int32_t* tokens, int64_t n, const int32_t* seq_offsets,
                    int32_t S, const int32_t* history, int32_t* ctx)
{
    (void)n;
    for (int32_t s = 0; s < S; ++s) {
        int64_t start = seq_offsets[s], end = seq_offsets[s + 1];
        int64_t len = end - start;
        int32_t* ext = (int32_t*)malloc(sizeof(int32_t) * (size_t)(len + 2));
        ext[0] = history ? history[2 * s] : ORACLE_PAD;
        ext[1] = history ? history[2 * s + 1] : ORACLE_PAD;
        for (int64_t p = 0; p < len; ++p)
            ext[p + 2] = tokens[start + p];
        for (int64_t p = 0; p < len; ++p) {
            int64_t i = start + p;
            ctx[3 * i + 0] = ext[p + 2];
            ctx[3 * i + 1] = ext[p + 1];
            ctx[3 * i + 2] = ext[p];
        }
        free(ext);
    }
}

/* rows[i][k] = splitmix64(key_k XOR seeds[k]) mod R. */
void oracle_hash(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                 const int32_t* history, const uint64_t* seeds, int64_t R, int32_t* rows)
{
    int32_t* ctx = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)(n > 0 ? n : 1));
    oracle_context(tokens, n, seq_offsets, S, history, ctx);
    for (int64_t i = 0; i < n; ++i) {
        uint64_t c0 = (uint64_t)(uint32_t)ctx[3 * i + 0];
        uint64_t c1 = (uint64_t)(uint32_t)ctx[3 * i + 1];
        uint64_t c2 = (uint64_t)(uint32_t)ctx[3 * i + 2];
        uint64_t bigram = (c1 << 21) | c0;
        uint64_t trigram = (c2 << 42) | (c1 << 21) | c0;
        for (int k = 0; k < ORACLE_K; ++k) {
            uint64_t key = k < 8 ? bigram : trigram;
            uint64_t h = oracle_splitmix64(key ^ seeds[k]);
            rows[i * ORACLE_K + k] = (int32_t)(h % (uint64_t)R);
        }
    }
    free(ctx);
}

/* eN[i][j] = sum over k = 0..15, in order, of T[rows[i][k]][j] (fp32). */
void oracle_embed_bag_bf16(const uint16_t* T, int64_t R, int32_t d, const int32_t* rows,
                           int64_t n, float* eN)
{
    (void)R;
    for (int64_t i = 0; i < n; ++i)
        for (int32_t j = 0; j < d; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < ORACLE_K; ++k) {
                int64_t r = rows[i * ORACLE_K + k];
                acc = acc + oracle_bf16_to_f32(T[r * d + j]);
            }
            eN[i * d + j] = acc;
        }
}

/* INT8 rows with one fp32 scale per row, dequantised inside the sum. */
void oracle_embed_bag_int8(const int8_t* Q, const float* scale, int64_t R, int32_t d,
                           const int32_t* rows, int64_t n, float* eN)
{
    (void)R;
    for (int64_t i = 0; i < n; ++i)
        for (int32_t j = 0; j < d; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < ORACLE_K; ++k) {
                int64_t r = rows[i * ORACLE_K + k];
                acc = fmaf((float)Q[r * d + j], scale[r], acc);
            }
            eN[i * d + j] = acc;
        }
}

/*
 * 4-bit rows: "Qwen 3.8 Flash-Next Deep Dive…", section 1, sizes the table
 * at FP4.  Format taken: OCP Microscaling (MX) FP4, i.e. E2M1 element codes
 * with one E8M0 scale per 32 elements.  A row of d elements is d/2 + d/32
 * bytes: bytes 0 .. d/2-1 hold the codes, element 2m in the low nibble of
 * byte m and 2m+1 in the high nibble; bytes d/2 .. d/2+d/32-1 hold the scales,
 * scale g for elements 32g .. 32g+31.  Element value = e2m1(code) * 2^(E-127)
 * (exact in fp32), NaN when E = 255.  E2M1: sign bit 3, exponent bits 2-1
 * (bias 1), mantissa bit 0; exponent 0 is subnormal (0 or 0.5).
 */
float oracle_e2m1(int code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return sign ? -mag : mag;
}

float oracle_mxfp4_value(const uint8_t* row, int32_t d, int32_t j)
{
    uint8_t byte = row[j / 2];
    int code = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
    int E = row[d / 2 + j / 32];
    if (E == 255)
        return NAN;
    return ldexpf(oracle_e2m1(code), E - 127);
}

/* eN[i][j] = sum over k = 0..15, in order, of the MXFP4 value of row
 * rows[i][k] at j (fp32, from +0). */
void oracle_embed_bag_mxfp4(const uint8_t* T, int64_t R, int32_t d, const int32_t* rows,
                            int64_t n, float* eN)
{
    (void)R;
    const int64_t row_bytes = d / 2 + d / 32;
    for (int64_t i = 0; i < n; ++i)
        for (int32_t j = 0; j < d; ++j) {
            float acc = 0.0f;
            for (int k = 0; k < ORACLE_K; ++k) {
                int64_t r = rows[i * ORACLE_K + k];
                acc = acc + oracle_mxfp4_value(T + r * row_bytes, d, j);
            }
            eN[i * d + j] = acc;
        }
}

/*
 * out[i][j] = bf16(residual[i][j] + fmaf(W_g[j], eN[i][j], e1[e1_rows[i]][j])).
 * e1_rows[i] is the token w_t (the 1-gram id).  e1 and residual may be NULL.
 */
void oracle_gate_add(const float* eN, const int32_t* e1_rows, int64_t n, int32_t d,
                     const uint16_t* e1, const float* W_g, const uint16_t* residual,
                     uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        for (int32_t j = 0; j < d; ++j) {
            float base = e1 ? oracle_bf16_to_f32(e1[(int64_t)e1_rows[i] * d + j]) : 0.0f;
            float h = fmaf(W_g[j], eN[i * d + j], base);
            float y = residual ? oracle_bf16_to_f32(residual[i * d + j]) + h : h;
            out[i * d + j] = oracle_bf16_rne(y);
        }
}

/* The whole path for a bf16 (dtype 0), int8 (dtype 1) or MXFP4 (dtype 2)
 * table, one step after another: context and hash, then the sum, then gate
 * and residual.  An MXFP4 table is passed as its [R][d/2 + d/32] bytes. */
void oracle_forward(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                    const int32_t* history, const uint64_t* seeds, int32_t dtype,
                    const void* table, const float* scale, int64_t R, int32_t d,
                    const uint16_t* e1, const float* W_g, const uint16_t* residual,
                    uint16_t* out, int32_t* rows_out, float* eN_out)
{
    size_t nn = (size_t)(n > 0 ? n : 1);
    int32_t* rows = rows_out ? rows_out : (int32_t*)malloc(sizeof(int32_t) * ORACLE_K * nn);
    float* eN = eN_out ? eN_out : (float*)malloc(sizeof(float) * (size_t)d * nn);
    oracle_hash(tokens, n, seq_offsets, S, history, seeds, R, rows);
    if (dtype == 0)
        oracle_embed_bag_bf16((const uint16_t*)table, R, d, rows, n, eN);
    else if (dtype == 1)
        oracle_embed_bag_int8((const int8_t*)table, scale, R, d, rows, n, eN);
    else
        oracle_embed_bag_mxfp4((const uint8_t*)table, R, d, rows, n, eN);
    oracle_gate_add(eN, tokens, n, d, e1, W_g, residual, out);
    if (!rows_out)
        free(rows);
    if (!eN_out)
        free(eN);
}

/*
 * Gradients.  The pages define only the forward pass of a "learned" table
 * ("Qwen Brought Back N-Grams…", section "N-grams, of all things"); these
 * follow from it by the chain rule, with the bf16 output rounding passed
 * straight through.  g is dL/dout, bf16 [n][d].  A token whose row ids are
 * -1 (invalid input) contributes nothing.  The order of each sum is fixed:
 *   table:  dT[r][j]  = sum over positions t = 16 i + k with rows[t] == r, in
 *           ascending t, of acc = fmaf(W_g[j], g[i][j], acc), from +0;
 *   e1:     de1[v][j] = sum over tokens i with tokens[i] == v, ascending i,
 *           of acc = acc + g[i][j], from +0;
 *   gate:   dW_g[j]   = the sum over valid tokens i of g[i][j] * eN[i][j], a
 *           single sum with no stated order: evaluated here in float64 over
 *           ascending i (every product of a bf16 and an fp32 value is exact in
 *           float64) and rounded once to fp32; out64 (may be NULL) receives
 *           the float64 value before that rounding.
 * The residual's gradient is g itself.
 */
void oracle_grad_table_rows(const int32_t* rows, int64_t n, int32_t d, const float* W_g,
                            const uint16_t* g, const int32_t* query, int64_t nq, float* out)
{
    for (int64_t q = 0; q < nq; ++q) {
        float* acc = out + q * d;
        for (int32_t j = 0; j < d; ++j)
            acc[j] = 0.0f;
        for (int64_t t = 0; t < n * ORACLE_K; ++t) {
            if (rows[t] != query[q] || rows[t] < 0)
                continue;
            const int64_t i = t / ORACLE_K;
            for (int32_t j = 0; j < d; ++j)
                acc[j] = fmaf(W_g[j], oracle_bf16_to_f32(g[i * d + j]), acc[j]);
        }
    }
}

void oracle_grad_e1_tokens(const int32_t* tokens, const int32_t* rows, int64_t n, int32_t d,
                           const uint16_t* g, const int32_t* query, int64_t nq, float* out)
{
    for (int64_t q = 0; q < nq; ++q) {
        float* acc = out + q * d;
        for (int32_t j = 0; j < d; ++j)
            acc[j] = 0.0f;
        for (int64_t i = 0; i < n; ++i) {
            if (tokens[i] != query[q] || rows[i * ORACLE_K] < 0)
                continue;
            for (int32_t j = 0; j < d; ++j)
                acc[j] = acc[j] + oracle_bf16_to_f32(g[i * d + j]);
        }
    }
}

void oracle_grad_gate(const int32_t* rows, const uint16_t* g, const float* eN, int64_t n, int32_t d,
                      float* out, double* out64)
{
    for (int32_t j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            if (rows[i * ORACLE_K] < 0)
                continue;
            acc = acc + (double)oracle_bf16_to_f32(g[i * d + j]) * (double)eN[i * d + j];
        }
        if (out64)
            out64[j] = acc;
        out[j] = (float)acc;
    }
}

/*
 * Round a float64 value to the nearest bf16, ties to even; NaN to 0x7FC0.
 * In the binade [2^(e-1), 2^e) a bf16 value has 8 significant bits, so its
 * spacing is 2^(e-8) (never below the subnormal spacing 2^-133).  The two
 * bf16 neighbours of |x| and their midpoint are exact float64 values, so the
 * choice is made by exact comparisons.
 */
uint16_t oracle_bf16_rne_f64(double x)
{
    if (isnan(x))
        return 0x7FC0;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    if (isinf(a))
        return sign | 0x7F80;
    int e = 0;
    (void)frexp(a, &e);                          /* 2^(e-1) <= a < 2^e, or a == 0 */
    int qe = e - 8;
    if (qe < -133)
        qe = -133;
    const double m = floor(ldexp(a, -qe));       /* a = (m + f) * 2^qe, 0 <= f < 1 */
    const double lo = ldexp(m, qe);
    const double hi = ldexp(m + 1.0, qe);
    const double mid = ldexp(m + 0.5, qe);
    const int odd = fmod(m, 2.0) != 0.0;
    const double r = (a > mid || (a == mid && odd)) ? hi : lo;
    if (r >= 0x1p128)
        return sign | 0x7F80;                    /* beyond the largest bf16: infinity */
    const float f = (float)r;                    /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/*
 * Normalised, input-gated fusion.  "Qwen 3.8 Flash-Next Deep Dive…" draws a
 * "Projection / Normalization" stage between the table lookup and the trunk,
 * and the summary of "Qwen3.8-Flash-Next: …" fuses the n-gram vector with the
 * 1-gram embedding "via a gating network".  Neither page defines the two.
 * Form taken, per token, from its fp32 sum x = eN (d columns):
 *   S      = sum over j of x[j]^2;
 *   r      = 1 / sqrt(S / d + eps);
 *   n[j]   = x[j] * r * gamma[j];                          RMS normalisation
 *   logit  = sum over j of (u[j] e1[j] + v[j] n[j]) + b;
 *   alpha  = 1 / (1 + exp(-logit));                        sigmoid gate unit
 *   y[j]   = residual[j] + e1[j] + alpha W_g[j] n[j];
 *   out[j] = y[j] rounded once to bf16, ties to even.
 * The pages fix no precision for any of this, so it is evaluated here in
 * float64, each sum over ascending j, and rounded to bf16 only at the end.
 * stats_out (may be NULL) gets {r, logit} per token, y_out (may be NULL) y.
 */
void oracle_norm_gate_add(const float* eN, const int32_t* e1_rows, int64_t n, int32_t d,
                          const uint16_t* e1, const float* W_g, const float* gamma, const float* u,
                          const float* v, float b, float eps, const uint16_t* residual,
                          uint16_t* out, double* stats_out, double* y_out)
{
    double* nv = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
    for (int64_t i = 0; i < n; ++i) {
        const float* x = eN + i * d;
        const uint16_t* e1_token = e1 + (int64_t)e1_rows[i] * d;
        const uint16_t* res_token = residual ? residual + i * d : NULL;
        double S = 0.0;
        for (int32_t j = 0; j < d; ++j)
            S = S + (double)x[j] * (double)x[j];
        const double r = 1.0 / sqrt(S / (double)d + (double)eps);
        for (int32_t j = 0; j < d; ++j)
            nv[j] = (double)x[j] * r * (double)gamma[j];
        double Z = 0.0;
        for (int32_t j = 0; j < d; ++j)
            Z = Z + ((double)u[j] * (double)oracle_bf16_to_f32(e1_token[j]) + (double)v[j] * nv[j]);
        const double logit = Z + (double)b;
        const double alpha = 1.0 / (1.0 + exp(-logit));
        for (int32_t j = 0; j < d; ++j) {
            const double h = (double)oracle_bf16_to_f32(e1_token[j]) + alpha * (double)W_g[j] * nv[j];
            const double y = res_token ? (double)oracle_bf16_to_f32(res_token[j]) + h : h;
            out[i * d + j] = oracle_bf16_rne_f64(y);
            if (y_out)
                y_out[i * d + j] = y;
        }
        if (stats_out) {
            stats_out[2 * i] = r;
            stats_out[2 * i + 1] = logit;
        }
    }
    free(nv);
}

/*
 * Projection.  "Qwen 3.8 Flash-Next Deep Dive…" draws a "Projection /
 * Normalization" stage between the table lookup and the trunk and does not
 * define it.  Form taken: a learned linear map of each token's n-gram sum x
 * (d_in columns) to d_out columns, with the weights P [d_out][d_in] stored
 * as bf16 (the model's storage type) and x rounded to bf16 first, ties to
 * even (the pages fix no precision):
 *   y[i][o] = sum over j of P[o][j] * bf16(x[i][j]).
 * A product of two bf16 values has at most 16 significant bits, so each term
 * is exact in float64; the sum is taken over ascending j in float64.
 * abs_out (may be NULL) receives the sum of |terms| per output, the scale of
 * the error of any other order of the same sum.
 */
void oracle_project(const float* x, int64_t n, int32_t d_in, const uint16_t* P, int32_t d_out,
                    double* y_out, double* abs_out)
{
    double* xb = (double*)malloc(sizeof(double) * (size_t)(d_in > 0 ? d_in : 1));
    for (int64_t i = 0; i < n; ++i) {
        for (int32_t j = 0; j < d_in; ++j)
            xb[j] = (double)oracle_bf16_to_f32(oracle_bf16_rne(x[i * d_in + j]));
        for (int32_t o = 0; o < d_out; ++o) {
            double acc = 0.0, a = 0.0;
            for (int32_t j = 0; j < d_in; ++j) {
                const double t = (double)oracle_bf16_to_f32(P[(int64_t)o * d_in + j]) * xb[j];
                acc = acc + t;
                a = a + fabs(t);
            }
            y_out[i * d_out + o] = acc;
            if (abs_out)
                abs_out[i * d_out + o] = a;
        }
    }
    free(xb);
}
