// libngram.so: the hashed n-gram embedding gather-sum for MI355X (gfx950).
//
// Method: "Qwen Brought Back N-Grams. All 51 Billion Parameters of Them.",
// section "N-grams, of all things" (hash the bigram and trigram context of a
// token into one 20M x 2560 table, gather 16 rows, sum them, add the sum to
// the residual stream), and "Qwen3.8-Flash-Next: A 51B N-gram Embedding Table
// with Heterogeneous Memory Prefetch", Key point 1 (gate with the 1-gram
// embedding: h = e_1gram(w_t) + W_g (.) e_N).  The hash, seeds, padding,
// summation order and rounding are fixed in include/ngram.h.
//
// Layout of the work on CDNA4.  The path is a gather-reduce that moves about
// 97 KB of HBM per token for 0.5 flop per byte, so it is bound by HBM
// bandwidth; there is no contraction and no MFMA.  One workgroup owns a tile
// of tokens.  Its threads first hash the tile's (token, k) pairs, one pair per
// thread, into a row list in LDS.  Then each wavefront owns 512-column slices
// of the rows: every lane loads 16 bytes (8 bf16, or 8 int8) of each of the
// 16 rows, so one load instruction reads 1 KiB contiguous of one row.  The
// compiler keeps about ten of the 16 loads of a slice in flight before the
// first add at 76 VGPRs (six wavefronts per SIMD); forcing all 16 ahead
// costs 122 VGPRs and measured 2% slower.  The row ids
// are wave-uniform (read from LDS, moved to scalar registers), so each row
// address is a scalar base plus a per-lane offset.  The sum runs in fp32 in
// k order, the gate is one fused multiply-add, the residual one add, and the
// result is rounded to bf16 in registers and stored with one 16-byte store per
// lane: the residual is read once and written once.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ngram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kK = NGRAM_K;
constexpr uint32_t kPad = NGRAM_PAD_ID;
constexpr int kVec = 8;                 // table elements per lane per slice
constexpr int kSlice = 64 * kVec;       // columns per wavefront slice
constexpr uint32_t kNaNbf16 = 0x7FC0u;
constexpr uint32_t kNaNf32 = 0x7FC00000u;

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Seeds {
    uint64_t s[kK];
};

// splitmix64 (Steele, Lea and Flood, OOPSLA 2014; Vigna's finaliser
// constants): the generator's first output from state x.
__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------
// Context: (w_t, w_{t-1}, w_{t-2}) of token i, from its own sequence, else the
// sequence's history, else the pad id.  Memory-safe for any seq_offsets.
struct Ctx {
    uint32_t c0, c1, c2;
    bool ok;
};

// The ids of tokens i, i-1, i-2 (pad before the batch start).  They do not
// depend on the sequence, so they are loaded before the sequence lookup.
struct TokIds {
    uint32_t t0, t1, t2;
};

__device__ inline TokIds token_ids(const int32_t* __restrict__ tok, int64_t i) {
    TokIds q;
    q.t0 = static_cast<uint32_t>(tok[i]);
    q.t1 = i >= 1 ? static_cast<uint32_t>(tok[i - 1]) : kPad;
    q.t2 = i >= 2 ? static_cast<uint32_t>(tok[i - 2]) : kPad;
    return q;
}

// so / hist point to global memory or to their copies in LDS.
__device__ inline Ctx context_of(const TokIds& q, int64_t i, const int32_t* so, int S, const int32_t* hist,
                                 uint32_t c0_limit) {
    int lo = 0, hi = S - 1;     // the last sequence s with so[s] <= i
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(so[mid]) <= i) lo = mid; else hi = mid - 1;
    }
    const int64_t p = i - static_cast<int64_t>(so[lo]);
    const uint32_t h0 = hist ? static_cast<uint32_t>(hist[2 * lo]) : kPad;
    const uint32_t h1 = hist ? static_cast<uint32_t>(hist[2 * lo + 1]) : kPad;
    Ctx c;
    c.c0 = q.t0;
    c.c1 = p >= 1 ? q.t1 : h1;
    c.c2 = p >= 2 ? q.t2 : (p == 1 ? h1 : h0);
    c.ok = c.c0 < c0_limit && c.c1 <= kPad && c.c2 <= kPad;
    return c;
}

// Up to this many sequences, a workgroup copies seq_offsets (and the
// history) into LDS in one round of loads, overlapped with its token loads,
// and searches there: the global binary search is a chain of dependent loads
// at the start of every workgroup (measured on MI355X at the prefill shape:
// 521-523 us with 8 sequences against 484 us for the same tokens as one).
constexpr int kStageSeqs = 255;
constexpr int kSeqLds = (kStageSeqs + 1) + 2 * kStageSeqs;   // int32 words
// Staging costs a barrier: it pays in batches of many tokens, not in small
// decode steps (B = 2 and 4 measured 3% slower with it), and with one
// sequence there is no search to replace.
constexpr int64_t kStageMinTokens = 1024;

__host__ __device__ inline int32_t stage_for(int64_t n, int S) {
    return S >= 2 && S <= kStageSeqs && n >= kStageMinTokens ? 1 : 0;
}

__device__ inline void stage_seqs(const int32_t* __restrict__ so, const int32_t* __restrict__ hist, int S,
                                  int32_t* lseq) {
    for (int t = threadIdx.x; t <= S; t += blockDim.x) lseq[t] = so[t];
    if (hist)
        for (int t = threadIdx.x; t < 2 * S; t += blockDim.x) lseq[kStageSeqs + 1 + t] = hist[t];
}

__device__ inline int32_t hashed_row(const Ctx& c, int k, const Seeds& sd, uint64_t R) {
    const uint64_t c0 = c.c0, c1 = c.c1, c2 = c.c2;
    const uint64_t bigram = (c1 << 21) | c0;
    const uint64_t trigram = (c2 << 42) | (c1 << 21) | c0;
    const uint64_t key = k < 8 ? bigram : trigram;
    return static_cast<int32_t>(splitmix64(key ^ sd.s[k]) % R);
}

// ---------------------------------------------------------------------------
// Element helpers.
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return kNaNbf16;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// MXFP4 slice of one row: 4 bytes of E2M1 codes (8 elements) and their E8M0
// scale byte.  A row is d/2 code bytes then d/32 scale bytes.
struct Fp4Slice {
    uint32_t codes;
    uint32_t scale;
};

// A wave-uniform address, passed through readfirstlane so that it stays in
// scalar registers: a load from it plus a 32-bit lane offset is then one
// scalar-base vector-offset global load, with no 64-bit address per lane.
typedef const __attribute__((address_space(1))) uint8_t* gbytes;

__device__ inline gbytes uniform_ptr(const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<gbytes>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ inline gbytes uniform_row(const void* base, int32_t r, int64_t row_bytes) {
    const uint64_t u = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(base) + static_cast<int64_t>(r) * row_bytes);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<gbytes>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Eight table elements of one row slice, as raw bits.  `row` is the row's
// wave-uniform start; `off` the lane's byte offset of the 8 elements (`aux`
// the offset of an MXFP4 slice's scale byte).
template <int DT> struct Row8;

template <> struct Row8<NGRAM_TABLE_BF16> {
    using Raw = uint4;
    __device__ static int64_t row_bytes(int64_t d) { return 2 * d; }
    __device__ static uint32_t lane_off(int64_t j0) { return static_cast<uint32_t>(j0) * 2u; }
    __device__ static Raw load(gbytes row, uint32_t off, uint32_t aux) {
        (void)aux;
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(row + off);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
};
template <> struct Row8<NGRAM_TABLE_INT8_ROWSCALE> {
    using Raw = uint2;
    __device__ static int64_t row_bytes(int64_t d) { return d; }
    __device__ static uint32_t lane_off(int64_t j0) { return static_cast<uint32_t>(j0); }
    __device__ static Raw load(gbytes row, uint32_t off, uint32_t aux) {
        (void)aux;
        const u32x2 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(row + off);
        return make_uint2(v.x, v.y);
    }
};
// An MXFP4 row is d/2 code bytes then d/32 scale bytes: columns j0..j0+7
// are code bytes j0/2 .. j0/2+3 and share scale byte d/2 + j0/32.
template <> struct Row8<NGRAM_TABLE_MXFP4> {
    using Raw = Fp4Slice;
    __device__ static int64_t row_bytes(int64_t d) { return d / 2 + d / 32; }
    __device__ static uint32_t lane_off(int64_t j0) { return static_cast<uint32_t>(j0) >> 1; }
    __device__ static Raw load(gbytes row, uint32_t off, uint32_t aux) {
        Fp4Slice f;
        f.codes = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(row + off);
        f.scale = row[aux];
        return f;
    }
};

__device__ inline void store_out(uint16_t* o, const uint4& v) {
    u32x4 w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    *reinterpret_cast<u32x4*>(o) = w;
}

// 8 bf16 values at byte offset `off` of a row with a wave-uniform start.
__device__ inline uint4 load_row8(gbytes row, uint32_t off) {
    const u32x4 t = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(row + off);
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ inline void store_row8(gbytes row, uint32_t off, const uint4& v) {
    u32x4 t;
    t.x = v.x; t.y = v.y; t.z = v.z; t.w = v.w;
    *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(
        const_cast<__attribute__((address_space(1))) uint8_t*>(row + off)) = t;
}

typedef float v2f __attribute__((ext_vector_type(2)));

// acc += e2m1 * 2^(E-127) for the 8 elements; the hardware conversion takes
// the scale's exponent (exact for the power-of-two E8M0 scale, including the
// subnormal 2^-127, which ldexp gives exactly).  The largest E seen is kept
// in `emax`: E = 255 (NaN) is applied after the sum.
__device__ inline void add_fp4(float acc[8], const Fp4Slice& f, uint32_t& emax) {
    const uint32_t E = f.scale;
    emax = E > emax ? E : emax;
    const float s = __builtin_ldexpf(1.0f, static_cast<int>(E) - 127);
    const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.codes, s, 0);
    const v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.codes, s, 1);
    const v2f c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.codes, s, 2);
    const v2f e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.codes, s, 3);
    acc[0] = acc[0] + a.x; acc[1] = acc[1] + a.y;
    acc[2] = acc[2] + b.x; acc[3] = acc[3] + b.y;
    acc[4] = acc[4] + c.x; acc[5] = acc[5] + c.y;
    acc[6] = acc[6] + e.x; acc[7] = acc[7] + e.y;
}

__device__ inline void add_row(float acc[8], const uint4& v) {
    acc[0] = acc[0] + bf16lo(v.x); acc[1] = acc[1] + bf16hi(v.x);
    acc[2] = acc[2] + bf16lo(v.y); acc[3] = acc[3] + bf16hi(v.y);
    acc[4] = acc[4] + bf16lo(v.z); acc[5] = acc[5] + bf16hi(v.z);
    acc[6] = acc[6] + bf16lo(v.w); acc[7] = acc[7] + bf16hi(v.w);
}

__device__ inline float i8f(uint32_t w, int b) {
    return static_cast<float>(static_cast<int8_t>((w >> (8 * b)) & 0xFFu));
}

__device__ inline void fma_row(float acc[8], const uint2& v, float s) {
    acc[0] = __builtin_fmaf(i8f(v.x, 0), s, acc[0]);
    acc[1] = __builtin_fmaf(i8f(v.x, 1), s, acc[1]);
    acc[2] = __builtin_fmaf(i8f(v.x, 2), s, acc[2]);
    acc[3] = __builtin_fmaf(i8f(v.x, 3), s, acc[3]);
    acc[4] = __builtin_fmaf(i8f(v.y, 0), s, acc[4]);
    acc[5] = __builtin_fmaf(i8f(v.y, 1), s, acc[5]);
    acc[6] = __builtin_fmaf(i8f(v.y, 2), s, acc[6]);
    acc[7] = __builtin_fmaf(i8f(v.y, 3), s, acc[7]);
}

// The lane's 8 columns of the 16 rows r[0..15], all loads issued back to
// back ...
template <int DT>
__device__ inline void gather_load(typename Row8<DT>::Raw v[kK], const void* __restrict__ tab, const int32_t r[kK],
                                   int64_t d, int64_t j0) {
    uint32_t off = Row8<DT>::lane_off(j0);
    uint32_t aux = static_cast<uint32_t>(d >> 1) + (static_cast<uint32_t>(j0) >> 5);
    // Materialise the lane offsets here as 32-bit registers: each row load is
    // then the row's scalar base plus this offset, with no 64-bit address
    // computed per lane and row.
    if constexpr (DT == NGRAM_TABLE_MXFP4) __asm__ volatile("" : "+v"(off), "+v"(aux));
    else __asm__ volatile("" : "+v"(off));
    const int64_t rb = Row8<DT>::row_bytes(d);
#pragma unroll
    for (int k = 0; k < kK; ++k) v[k] = Row8<DT>::load(uniform_row(tab, r[k], rb), off, aux);
}

// ... and summed in fp32 in k order.
template <int DT>
__device__ inline void gather_reduce(float acc[8], const typename Row8<DT>::Raw v[kK],
                                     const float* __restrict__ scale, const int32_t r[kK]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    if constexpr (DT == NGRAM_TABLE_BF16) {
#pragma unroll
        for (int k = 0; k < kK; ++k) add_row(acc, v[k]);
    } else if constexpr (DT == NGRAM_TABLE_INT8_ROWSCALE) {
        float s[kK];
#pragma unroll
        for (int k = 0; k < kK; ++k) s[k] = scale[r[k]];
#pragma unroll
        for (int k = 0; k < kK; ++k) fma_row(acc, v[k], s[k]);
    } else {
        uint32_t emax = 0;
#pragma unroll
        for (int k = 0; k < kK; ++k) add_fp4(acc, v[k], emax);
        if (emax == 255u) {
            // a NaN term makes the in-order sum NaN
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __uint_as_float(kNaNf32);
        }
    }
}

// The fp32 sum over k = 0..15 of the lane's 8 columns of rows r[0..15].
template <int DT, bool WS = false>
__device__ inline void gather_sum(float acc[8], const void* __restrict__ tab,
                                  const float* __restrict__ scale, const int32_t r[kK],
                                  int64_t d, int64_t j0) {
    typename Row8<DT>::Raw v[kK];
    if constexpr (DT == NGRAM_TABLE_INT8_ROWSCALE && WS) {
        // WS: every lane of the wavefront is active (whole 512-column
        // slices).  The 16 row scales by one load ahead of the rows: lane
        // k < 16 takes row k's scale (the other lanes row 0's, unused), and
        // readlane hands each one to the whole wavefront once the load is
        // back (the rows' loads, issued after it, can still be in flight:
        // loads complete in issue order).  Sixteen per-row loads of one
        // broadcast word each otherwise share the load queue with the rows
        // (measured: int8 prefill shape 566-576 -> 554-559 us).
        int32_t rk = 0;
#pragma unroll
        for (int k = 0; k < kK; ++k) __asm__("v_writelane_b32 %0, %1, %2" : "+v"(rk) : "s"(r[k]), "n"(k));
        const float sv = scale[rk];
        __builtin_amdgcn_sched_barrier(0);
        gather_load<DT>(v, tab, r, d, j0);
        // all 16 row loads in flight before the first add (2 registers each)
        __builtin_amdgcn_sched_barrier(0);
        float sk[kK];
#pragma unroll
        for (int k = 0; k < kK; ++k) sk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), k));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < kK; ++k) fma_row(acc, v[k], sk[k]);
        return;
    }
    gather_load<DT>(v, tab, r, d, j0);
    // MXFP4 rows take 2 registers per row slice, so all 32 loads fit in
    // flight before the first add (measured 3% faster; for int8 the same
    // costs 101 VGPRs and 20%, for bf16 122 VGPRs and 2%)
    if constexpr (DT == NGRAM_TABLE_MXFP4) __builtin_amdgcn_sched_barrier(0);
    gather_reduce<DT>(acc, v, scale, r);
}

// out = bf16(res + fmaf(w, acc, e1)) for the lane's 8 columns.
// out = bf16(res + fmaf(w, acc, e1)) for the lane's 8 columns, from the
// lane's e1 and residual slices (each ignored when absent).
template <bool E1, bool RES>
__device__ inline uint4 gate8v(const float acc[8], const float w[8], const uint4& e, const uint4& rv) {
    float base[8];
    if constexpr (E1) {
        base[0] = bf16lo(e.x); base[1] = bf16hi(e.x); base[2] = bf16lo(e.y); base[3] = bf16hi(e.y);
        base[4] = bf16lo(e.z); base[5] = bf16hi(e.z); base[6] = bf16lo(e.w); base[7] = bf16hi(e.w);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) base[q] = 0.0f;
    }
    float y[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) y[q] = __builtin_fmaf(w[q], acc[q], base[q]);
    if constexpr (RES) {
        y[0] = bf16lo(rv.x) + y[0]; y[1] = bf16hi(rv.x) + y[1];
        y[2] = bf16lo(rv.y) + y[2]; y[3] = bf16hi(rv.y) + y[3];
        y[4] = bf16lo(rv.z) + y[4]; y[5] = bf16hi(rv.z) + y[5];
        y[6] = bf16lo(rv.w) + y[6]; y[7] = bf16hi(rv.w) + y[7];
    }
    uint4 o;
    o.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
    o.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
    o.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
    o.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
    return o;
}

// The same, loading the e1 and residual slices from their rows.
template <bool E1, bool RES>
__device__ inline uint4 gate8(const float acc[8], const float w[8], const uint16_t* __restrict__ e1row,
                              const uint16_t* __restrict__ resrow) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const uint4 e = E1 ? *reinterpret_cast<const uint4*>(e1row) : z;
    const uint4 rv = RES ? *reinterpret_cast<const uint4*>(resrow) : z;
    return gate8v<E1, RES>(acc, w, e, rv);
}

__device__ inline void load_w8(float w[8], const float* __restrict__ wg, int64_t j0) {
    const float4 a = *reinterpret_cast<const float4*>(wg + j0);
    const float4 b = *reinterpret_cast<const float4*>(wg + j0 + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// ---------------------------------------------------------------------------
// Fused kernel: context, hash, gather, sum, gate, residual, rounding.
struct FwdArgs {
    const int32_t* tok;
    const int32_t* so;
    const int32_t* hist;
    const void* tab;
    const float* scale;
    const uint16_t* e1;
    const float* wg;
    const uint16_t* res;
    uint16_t* out;
    int32_t* rows_out;
    int64_t n;
    uint64_t R;
    int32_t S;
    int32_t d;
    int32_t tpw;        // tokens per workgroup
    uint32_t c0_limit;  // token ids must be below this (V, capped at the pad id)
    int32_t stage;      // copy seq_offsets / history into LDS (see stage_for)
    Seeds sd;
};

// A tile's hash phase: one thread per (token, k) writes the row id into LDS
// (and rows_out), and w_t per token; -1 marks an invalid token.
__device__ inline void hash_tile(const FwdArgs& a, int64_t tile0, int32_t* lrows, int32_t* ltok, int32_t* lseq) {
    const int nt = a.tpw * kK;
    if (a.stage) {
        // the thread's first (token, k): its ids are loaded ahead of the staging
        TokIds first = {kPad, kPad, kPad};
        if (static_cast<int>(threadIdx.x) < nt && tile0 + (threadIdx.x >> 4) < a.n)
            first = token_ids(a.tok, tile0 + (threadIdx.x >> 4));
        stage_seqs(a.so, a.hist, a.S, lseq);
        __syncthreads();
        for (int t = threadIdx.x; t < nt; t += blockDim.x) {
            const int tl = t >> 4, k = t & (kK - 1);
            const int64_t i = tile0 + tl;
            int32_t row = -1, c0 = -1;
            if (i < a.n) {
                const TokIds q = t == static_cast<int>(threadIdx.x) ? first : token_ids(a.tok, i);
                const Ctx c = context_of(q, i, lseq, a.S, a.hist ? lseq + kStageSeqs + 1 : nullptr, a.c0_limit);
                if (c.ok) {
                    row = hashed_row(c, k, a.sd, a.R);
                    c0 = static_cast<int32_t>(c.c0);
                }
                if (a.rows_out) a.rows_out[i * kK + k] = row;
            }
            lrows[t] = row;
            if (k == 0) ltok[tl] = c0;
        }
    } else {
        for (int t = threadIdx.x; t < nt; t += blockDim.x) {
            const int tl = t >> 4, k = t & (kK - 1);
            const int64_t i = tile0 + tl;
            int32_t row = -1, c0 = -1;
            if (i < a.n) {
                const Ctx c = context_of(token_ids(a.tok, i), i, a.so, a.S, a.hist, a.c0_limit);
                if (c.ok) {
                    row = hashed_row(c, k, a.sd, a.R);
                    c0 = static_cast<int32_t>(c.c0);
                }
                if (a.rows_out) a.rows_out[i * kK + k] = row;
            }
            lrows[t] = row;
            if (k == 0) ltok[tl] = c0;
        }
    }
    __syncthreads();
}

// One tile: hash its tokens' rows into LDS, then each wavefront gathers,
// sums, gates and stores its slices of every token of the tile.
template <int DT, bool E1, bool RES, bool WS>
__device__ inline void fwd_tile(const FwdArgs& a, int64_t tile0, int32_t* lrows, int32_t* ltok) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int64_t d = a.d;
    const int nslices = (a.d + kSlice - 1) / kSlice;
    hash_tile(a, tile0, lrows, ltok, lrows + a.tpw * (kK + 1));

    const int64_t rem = a.n - tile0;
    const int tile_n = rem < a.tpw ? static_cast<int>(rem) : a.tpw;
    for (int sl = wave; sl < nslices; sl += nwaves) {
        const int64_t j0 = static_cast<int64_t>(sl) * kSlice + lane * kVec;
        if (j0 >= d) continue;
        float w[8];
        load_w8(w, a.wg, j0);
        // e1, residual and output rows are addressed as the row's uniform
        // start plus this 32-bit lane offset (no 64-bit address per lane held
        // across the loop: fewer registers, more wavefronts per SIMD)
        uint32_t off2 = static_cast<uint32_t>(j0) * 2u;
        __asm__ volatile("" : "+v"(off2));
        for (int tl = 0; tl < tile_n; ++tl) {
            const int64_t i = tile0 + tl;
            const gbytes orow = uniform_ptr(a.out + i * d);
            const int32_t c0 = __builtin_amdgcn_readfirstlane(ltok[tl]);
            if (c0 < 0) {
                uint32_t nn = kNaNbf16 | (kNaNbf16 << 16);
                __asm__ volatile("" : "+v"(nn));    // made here, not held in registers across the loop
                store_row8(orow, off2, make_uint4(nn, nn, nn, nn));
                continue;
            }
            int32_t r[kK];
#pragma unroll
            for (int k = 0; k < kK; ++k) r[k] = __builtin_amdgcn_readfirstlane(lrows[tl * kK + k]);
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            float acc[8];
            uint4 e = z, rv = z;
            if constexpr (DT == NGRAM_TABLE_MXFP4 && (E1 || RES)) {
                // the e1 and residual slices do not depend on the sum: issue
                // their loads ahead of the rows, so a token costs one memory
                // round trip (MXFP4 runs 4 tokens per wavefront in sequence;
                // bf16 and int8 measured no gain, nor did bf16 decode steps)
                if constexpr (E1) e = load_row8(uniform_row(a.e1, c0, 2 * d), off2);
                if constexpr (RES) rv = load_row8(uniform_ptr(a.res + i * d), off2);
                __builtin_amdgcn_sched_barrier(0);
                gather_sum<DT>(acc, a.tab, a.scale, r, d, j0);
            } else {
                gather_sum<DT, WS>(acc, a.tab, a.scale, r, d, j0);
                if constexpr (E1) e = load_row8(uniform_row(a.e1, c0, 2 * d), off2);
                if constexpr (RES) rv = load_row8(uniform_ptr(a.res + i * d), off2);
            }
            store_row8(orow, off2, gate8v<E1, RES>(acc, w, e, rv));
        }
    }
}

// ---------------------------------------------------------------------------
// Normalised, input-gated fusion ("Qwen 3.8 Flash-Next Deep Dive…": a
// "Projection / Normalization" stage after the lookup; "Qwen3.8-Flash-Next:
// …", summary: fusion "via a gating network"; the pages define neither, the
// form taken is), per token from its fp32 sum eN:
//   r = 1 / sqrt(S / d + eps),  S = sum over j of eN[j]^2,
//   n[j] = eN[j] r gamma[j],
//   logit = sum over j of (u[j] e1[j] + v[j] n[j]) + b,
//   alpha = 1 / (1 + exp(-logit)),
//   out[j] = bf16(residual[j] + e1[j] + alpha W_g[j] n[j]).
// All of it is evaluated in float64 (the squares and the u e1 products of
// fp32 and bf16 values are exact there) and rounded to bf16 once, from the
// float64 value.  The sums have no stated order; on CDNA4 a lane adds its 8
// columns, a 64-lane xor butterfly adds the wavefront's lanes, and the
// wavefronts' sums meet in LDS.
struct GatedArgs {
    FwdArgs f;
    const float* eN;    // MODE 3: the fp32 sums [n][d], read instead of gathered
    const float* gamma;
    const float* u;
    const float* v;
    double* stats;      // [n][2] = (r, logit), or null
    float b;
    float eps;
};

// x from another lane of the same 16-lane row, chosen by a DPP control word
// (both 32-bit halves moved with the same pattern).
template <int CTRL>
__device__ inline double dpp_f64(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xF, 0xF, false));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ inline double readlane_f64(double x, int lane) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), lane));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// The sum of x over the wavefront's 64 lanes, the same value in every lane.
// Within each 16-lane row, lanes exchange by DPP: neighbours (xor 1), pairs
// (xor 2), the two halves of 8 (half mirror), the two halves of 16 (mirror);
// each step adds two values whose sum is the same whichever lane forms it,
// so all 16 lanes of a row hold the same row sum.  The four row sums are then
// added in row order.
__device__ inline double wave_sum(double x) {
    x = x + dpp_f64<0xB1>(x);     // quad_perm [1,0,3,2]
    x = x + dpp_f64<0x4E>(x);     // quad_perm [2,3,0,1]
    x = x + dpp_f64<0x141>(x);    // row_half_mirror
    x = x + dpp_f64<0x140>(x);    // row_mirror
    return ((readlane_f64(x, 0) + readlane_f64(x, 16)) + readlane_f64(x, 32)) + readlane_f64(x, 48);
}

__device__ inline void load_f8(float w[8], const float* __restrict__ p, int64_t j0) {
    const float4 a = *reinterpret_cast<const float4*>(p + j0);
    const float4 b = *reinterpret_cast<const float4*>(p + j0 + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// float64 to bf16, rounded once to nearest, ties to even; NaN to 0x7FC0.
// Rounding to fp32 toward zero and setting the last bit when that dropped
// anything ("round to odd") keeps the information a second rounding needs:
// fp32 carries 16 more significant bits than bf16 over the same exponent
// range, so the fp32-to-bf16 rounding to nearest even that follows decides
// exactly as a direct rounding of x would.
__device__ inline uint32_t bf16_rne_f64(double x) {
    if (x != x) return kNaNbf16;
    const float t = __double2float_rz(x);
    uint32_t u = __float_as_uint(t);
    if (static_cast<double>(t) != x) u |= 1u;
    return bf16_rne(__uint_as_float(u));
}

// One tile: wavefront w owns columns 512w .. 512w+511 (one block; the launch
// has one wavefront per block).  Each token takes two workgroup barriers, one
// per sum over its columns; a token's validity is uniform over the workgroup,
// so every wavefront reaches the same barriers.  ONE: the tile is one token,
// so there is no token loop (a loop lets the compiler keep loop-invariant
// float64 constants of exp in registers through the gather).
template <int DT, bool RES, bool FULL, bool ONE, bool LOADED = false>
__device__ inline void gated_tile(const GatedArgs& g, int64_t tile0, int32_t* lrows, int32_t* ltok, double* lred) {
    constexpr bool EARLY = FULL && ONE;
    const FwdArgs& a = g.f;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int64_t d = a.d;
    const uint32_t jl = static_cast<uint32_t>(wave * kSlice + lane * kVec);   // the lane's first column
    const bool col = FULL || jl < static_cast<uint32_t>(d);  // FULL: d a multiple of 512, all lanes have columns
    if constexpr (!LOADED) hash_tile(a, tile0, lrows, ltok, lrows + a.tpw * (kK + 1));

    const int64_t rem = a.n - tile0;
    const int tile_n = ONE ? 1 : (rem < a.tpw ? static_cast<int>(rem) : a.tpw);
    for (int tl = 0; tl < tile_n; ++tl) {
        const int64_t i = tile0 + tl;
        int32_t c0;
        if constexpr (LOADED) {
            // the token's e1 row; an id outside [0, V) makes the token invalid
            const uint32_t t = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(a.tok[i]));
            c0 = t < a.c0_limit ? static_cast<int32_t>(t) : -1;
        } else {
            c0 = __builtin_amdgcn_readfirstlane(ltok[tl]);
        }
        if (c0 < 0) {
            if (col) {
                const uint32_t nn = kNaNbf16 | (kNaNbf16 << 16);
                *reinterpret_cast<uint4*>(a.out + i * d + jl) = make_uint4(nn, nn, nn, nn);
            }
            if (g.stats && threadIdx.x == 0) {
                g.stats[2 * i] = __longlong_as_double(0x7FF8000000000000ll);
                g.stats[2 * i + 1] = __longlong_as_double(0x7FF8000000000000ll);
            }
            continue;
        }
        double* red = lred + tl * 2 * nwaves;        // [2][nwaves], one slot set per token
        float acc[8];
        // the e1 slice is loaded with the rows, so it is there at the
        // second sum (measured: 3% faster; loading the residual slice early
        // too costs 13 registers and two wavefronts per SIMD, 4% slower)
        uint4 e1v = make_uint4(0u, 0u, 0u, 0u), rv = e1v;
        if (col) {
            e1v = load_row8(uniform_row(a.e1, c0, 2 * d), 2u * jl);
            if constexpr (LOADED) {
                const float4 x0 = *reinterpret_cast<const float4*>(g.eN + i * d + jl);
                const float4 x1 = *reinterpret_cast<const float4*>(g.eN + i * d + jl + 4);
                acc[0] = x0.x; acc[1] = x0.y; acc[2] = x0.z; acc[3] = x0.w;
                acc[4] = x1.x; acc[5] = x1.y; acc[6] = x1.z; acc[7] = x1.w;
            } else {
                int32_t r[kK];
#pragma unroll
                for (int k = 0; k < kK; ++k) r[k] = __builtin_amdgcn_readfirstlane(lrows[tl * kK + k]);
                __builtin_amdgcn_sched_barrier(0);
                gather_sum<DT, FULL>(acc, a.tab, a.scale, r, d, jl);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        }
        // Everything else the token needs (its residual slice, gamma, u, v
        // and W_g) is fetched here, once the sum is formed: the row slices'
        // registers are free by then, and the loads arrive during the two
        // block sums instead of adding two memory round trips after them.
        // (EARLY: with every lane holding columns and one token per
        // workgroup; otherwise the registers this takes make the compiler
        // spill, and the loads follow the sums that need them.)
        float gm[8], uu[8], vv[8], w8[8];
        if constexpr (EARLY) {
            // the residual slice last: loads complete in issue order, and
            // the first block sum waits only for gamma, u and v
            __builtin_amdgcn_sched_barrier(0);
            load_f8(gm, g.gamma, jl);
            load_f8(uu, g.u, jl);
            load_f8(vv, g.v, jl);
            load_w8(w8, a.wg, jl);
            if constexpr (RES) rv = load_row8(uniform_ptr(a.res + i * d), 2u * jl);
        }
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = s + static_cast<double>(acc[e]) * static_cast<double>(acc[e]);
        s = wave_sum(s);
        if (lane == 0) red[wave] = s;
        __syncthreads();
        double S = red[0];
        for (int w = 1; w < nwaves; ++w) S = S + red[w];
        const double rn = 1.0 / sqrt(S / static_cast<double>(d) + static_cast<double>(g.eps));

        // n = eN r gamma is formed again after the second barrier (the same
        // operations give the same bits), so the float64 n is not kept
        // across it.
        double z = 0.0;
        if (col) {
            if constexpr (!EARLY) {
                load_f8(gm, g.gamma, jl);
                load_f8(uu, g.u, jl);
                load_f8(vv, g.v, jl);
            }
            const float ev[8] = {bf16lo(e1v.x), bf16hi(e1v.x), bf16lo(e1v.y), bf16hi(e1v.y),
                                 bf16lo(e1v.z), bf16hi(e1v.z), bf16lo(e1v.w), bf16hi(e1v.w)};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double nv = static_cast<double>(acc[e]) * rn * static_cast<double>(gm[e]);
                z = z + (static_cast<double>(uu[e]) * static_cast<double>(ev[e]) + static_cast<double>(vv[e]) * nv);
            }
        }
        z = wave_sum(z);
        if (lane == 0) red[nwaves + wave] = z;
        __syncthreads();
        double Z = red[nwaves];
        for (int w = 1; w < nwaves; ++w) Z = Z + red[nwaves + w];
        const double logit = Z + static_cast<double>(g.b);
        const double alpha = 1.0 / (1.0 + exp(-logit));
        if (col) {
            const float ev[8] = {bf16lo(e1v.x), bf16hi(e1v.x), bf16lo(e1v.y), bf16hi(e1v.y),
                                 bf16lo(e1v.z), bf16hi(e1v.z), bf16lo(e1v.w), bf16hi(e1v.w)};
            if constexpr (!EARLY) {
                load_f8(gm, g.gamma, jl);
                load_w8(w8, a.wg, jl);
                if constexpr (RES) rv = load_row8(uniform_ptr(a.res + i * d), 2u * jl);
            }
            float rf[8];
            if constexpr (RES) {
                rf[0] = bf16lo(rv.x); rf[1] = bf16hi(rv.x); rf[2] = bf16lo(rv.y); rf[3] = bf16hi(rv.y);
                rf[4] = bf16lo(rv.z); rf[5] = bf16hi(rv.z); rf[6] = bf16lo(rv.w); rf[7] = bf16hi(rv.w);
            }
            uint32_t ob[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double nv = static_cast<double>(acc[e]) * rn * static_cast<double>(gm[e]);
                double y = static_cast<double>(ev[e]) + alpha * static_cast<double>(w8[e]) * nv;
                if constexpr (RES) y = static_cast<double>(rf[e]) + y;
                ob[e] = bf16_rne_f64(y);
            }
            uint4 ov;
            ov.x = ob[0] | (ob[1] << 16);
            ov.y = ob[2] | (ob[3] << 16);
            ov.z = ob[4] | (ob[5] << 16);
            ov.w = ob[6] | (ob[7] << 16);
            store_out(a.out + i * d + jl, ov);
        }
        if (g.stats && threadIdx.x == 0) {
            g.stats[2 * i] = rn;
            g.stats[2 * i + 1] = logit;
        }
    }
}

// MODE 0: one token per workgroup; 1: one tile of tpw tokens per workgroup;
// 2: a capped grid loops over the tiles (tables in host memory); 3: one
// token per workgroup whose fp32 sum is read from g.eN (no hash, no gather).
template <int DT, bool RES, bool FULL, int MODE>
__device__ inline void gated_body(const GatedArgs& g) {
    extern __shared__ int32_t lds[];
    // [tpw][2][nwaves] float64 sums first (8-byte aligned), then the row
    // lists [tpw][16], w_t [tpw] and the staged sequence table
    const int nwaves = blockDim.x >> 6;
    double* lred = reinterpret_cast<double*>(lds);
    int32_t* lrows = lds + 2 * (g.f.tpw * 2 * nwaves);
    int32_t* ltok = lrows + g.f.tpw * kK;
    if constexpr (MODE == 0) {
        gated_tile<DT, RES, FULL, true>(g, static_cast<int64_t>(blockIdx.x), lrows, ltok, lred);
    } else if constexpr (MODE == 3) {
        gated_tile<DT, RES, FULL, true, true>(g, static_cast<int64_t>(blockIdx.x), lrows, ltok, lred);
    } else if constexpr (MODE == 1) {
        gated_tile<DT, RES, FULL, false>(g, static_cast<int64_t>(blockIdx.x) * g.f.tpw, lrows, ltok, lred);
    } else {
        const int64_t ntiles = (g.f.n + g.f.tpw - 1) / g.f.tpw;
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            gated_tile<DT, RES, FULL, false>(g, tile * g.f.tpw, lrows, ltok, lred);
            __syncthreads();              // the next tile rewrites the LDS lists
        }
    }
}

// One token per workgroup (MODE 0 and 3) on whole 512-column blocks, held
// to at most 72 registers so that 7 wavefronts fit per SIMD: with the
// token's residual, gamma, u, v and W_g fetched as soon as its sum is
// formed, the compiler's own choice is 78 registers and 6 wavefronts.
template <int DT, bool RES, int MODE>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(7)))
ngram_gated_kernel(const GatedArgs g) {
    static_assert(MODE == 0 || MODE == 3, "one token per workgroup");
    gated_body<DT, RES, true, MODE>(g);
}

// Every other case: a ragged last block, tiles of several tokens (MODE 1)
// and the capped grid (MODE 2).
template <int DT, bool RES, bool FULL, int MODE>
__global__ void __launch_bounds__(1024) ngram_gated_any_kernel(const GatedArgs g) {
    gated_body<DT, RES, FULL, MODE>(g);
}

// PERSIST = false: one tile per workgroup (tables in HBM).  PERSIST = true:
// a capped grid loops over the tiles (tables in host memory, read over PCIe).
// WS: d is a multiple of 512 (every slice whole; int8 only).
template <int DT, bool E1, bool RES, bool PERSIST, bool WS>
__global__ void __launch_bounds__(1024) ngram_fwd_kernel(const FwdArgs a) {
    extern __shared__ int32_t lds[];
    int32_t* lrows = lds;                 // [tpw][16] row ids (-1: invalid token)
    int32_t* ltok = lds + a.tpw * kK;     // [tpw] w_t (-1: invalid token)
    if constexpr (!PERSIST) {
        fwd_tile<DT, E1, RES, WS>(a, static_cast<int64_t>(blockIdx.x) * a.tpw, lrows, ltok);
    } else {
        const int64_t ntiles = (a.n + a.tpw - 1) / a.tpw;
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            fwd_tile<DT, E1, RES, WS>(a, tile * a.tpw, lrows, ltok);
            __syncthreads();              // the next tile rewrites the LDS lists
        }
    }
}

// ---------------------------------------------------------------------------
// Unfused pieces: hash, gather-sum (fp32 out), gate-add.
struct HashArgs {
    const int32_t* tok;
    const int32_t* so;
    const int32_t* hist;
    int32_t* rows_out;
    int64_t n;
    uint64_t R;
    int32_t S;
    uint32_t c0_limit;
    int32_t stage;
    Seeds sd;
};

__global__ void __launch_bounds__(256) ngram_hash_kernel(const HashArgs a) {
    __shared__ int32_t lseq[kSeqLds];
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool live = t < a.n * kK;
    const int64_t i = t >> 4;
    const int k = static_cast<int>(t & (kK - 1));
    TokIds q = {kPad, kPad, kPad};
    if (live) q = token_ids(a.tok, i);
    const bool staged = a.stage != 0;
    if (staged) stage_seqs(a.so, a.hist, a.S, lseq);
    if (staged) __syncthreads();
    if (!live) return;
    const Ctx c = staged ? context_of(q, i, lseq, a.S, a.hist ? lseq + kStageSeqs + 1 : nullptr, a.c0_limit)
                         : context_of(q, i, a.so, a.S, a.hist, a.c0_limit);
    a.rows_out[t] = c.ok ? hashed_row(c, k, a.sd, a.R) : -1;
}

struct BagArgs {
    const void* tab;
    const float* scale;
    const int32_t* rows;
    float* eN;
    uint16_t* eN16;     // bf16 output instead of eN (the sums rounded to nearest, ties to even)
    int64_t n;
    int64_t R;
    int32_t d;
    int32_t tpw;
};

// OUT16: the sums rounded to bf16 (eN16), else fp32 (eN).  Output rows are
// addressed as the row's uniform start plus a 32-bit lane offset, as in the
// fused kernel (fewer registers, more wavefronts per SIMD).
template <int DT, bool OUT16, bool WS>
__device__ inline void bag_tile(const BagArgs& a, int64_t tile0, int32_t* lds) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int64_t d = a.d;
    const int nslices = (a.d + kSlice - 1) / kSlice;
    for (int t = threadIdx.x; t < a.tpw * kK; t += blockDim.x) {
        const int64_t i = tile0 + (t >> 4);
        int32_t r = -1;
        if (i < a.n) {
            r = a.rows[i * kK + (t & (kK - 1))];
            if (r < 0 || r >= a.R) r = -1;
        }
        lds[t] = r;
    }
    __syncthreads();
    const int64_t rem = a.n - tile0;
    const int tile_n = rem < a.tpw ? static_cast<int>(rem) : a.tpw;
    for (int sl = wave; sl < nslices; sl += nwaves) {
        const int64_t j0 = static_cast<int64_t>(sl) * kSlice + lane * kVec;
        if (j0 >= d) continue;
        uint32_t off = static_cast<uint32_t>(j0) * (OUT16 ? 2u : 4u);
        __asm__ volatile("" : "+v"(off));
        // fp32 output of a whole 512-column slice (uniform over the wavefront)
        const bool full = !OUT16 && (static_cast<int64_t>(sl) + 1) * kSlice <= d;
        float* stage = reinterpret_cast<float*>(lds + a.tpw * kK) + wave * kSlice;
        const uint32_t offa = (static_cast<uint32_t>(sl) * kSlice + lane * 4u) * 4u;
        for (int tl = 0; tl < tile_n; ++tl) {
            const int64_t i = tile0 + tl;
            int32_t r[kK];
            bool ok = true;
#pragma unroll
            for (int k = 0; k < kK; ++k) {
                r[k] = __builtin_amdgcn_readfirstlane(lds[tl * kK + k]);
                ok = ok && r[k] >= 0;
            }
            float acc[8];
            if (ok) {
                gather_sum<DT, WS>(acc, a.tab, a.scale, r, d, j0);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = __uint_as_float(kNaNf32);
            }
            if constexpr (OUT16) {
                uint4 w;
                w.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
                w.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
                w.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
                w.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
                store_row8(uniform_ptr(a.eN16 + i * d), off, w);
            } else {
                const gbytes orow = uniform_ptr(a.eN + i * d);
                if (full) {
                    // through the wavefront's 2 KiB of LDS, so that each of
                    // the two stores writes 1 KiB of consecutive addresses
                    // (lane l: columns 4l..4l+3, then 256+4l..256+4l+3)
                    // rather than 16 bytes per lane at a 32-byte stride
                    *reinterpret_cast<float4*>(stage + lane * 8) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    *reinterpret_cast<float4*>(stage + lane * 8 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
                    __builtin_amdgcn_wave_barrier();
                    const float4 p = *reinterpret_cast<const float4*>(stage + lane * 4);
                    const float4 q = *reinterpret_cast<const float4*>(stage + kSlice / 2 + lane * 4);
                    __builtin_amdgcn_wave_barrier();
                    store_row8(orow, offa, make_uint4(__float_as_uint(p.x), __float_as_uint(p.y),
                                                      __float_as_uint(p.z), __float_as_uint(p.w)));
                    store_row8(orow, offa + 2u * kSlice, make_uint4(__float_as_uint(q.x), __float_as_uint(q.y),
                                                                    __float_as_uint(q.z), __float_as_uint(q.w)));
                } else {
                    store_row8(orow, off, make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                     __float_as_uint(acc[2]), __float_as_uint(acc[3])));
                    store_row8(orow, off + 16u, make_uint4(__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                                                           __float_as_uint(acc[6]), __float_as_uint(acc[7])));
                }
            }
        }
    }
}

// WS: d is a multiple of 512 (every slice whole; int8 only).
template <int DT, bool PERSIST, bool OUT16, bool WS = false>
__global__ void __launch_bounds__(1024) ngram_bag_kernel(const BagArgs a) {
    extern __shared__ int32_t lds[];
    if constexpr (!PERSIST) {
        bag_tile<DT, OUT16, WS>(a, static_cast<int64_t>(blockIdx.x) * a.tpw, lds);
    } else {
        const int64_t ntiles = (a.n + a.tpw - 1) / a.tpw;
        for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
            bag_tile<DT, OUT16, WS>(a, tile * a.tpw, lds);
            __syncthreads();
        }
    }
}

struct GateArgs {
    const float* eN;
    const int32_t* tok;
    const uint16_t* e1;
    const float* wg;
    const uint16_t* res;
    uint16_t* out;
    int64_t n;
    int32_t d;
    uint32_t c0_limit;
};

template <bool E1, bool RES>
__global__ void __launch_bounds__(256) ngram_gate_kernel(const GateArgs a) {
    const int64_t dv = a.d / kVec;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (g >= a.n * dv) return;
    const int64_t i = g / dv;
    const int64_t j0 = (g - i * dv) * kVec;
    const int64_t d = a.d;
    uint16_t* o = a.out + i * d + j0;
    const uint32_t c0 = static_cast<uint32_t>(a.tok[i]);
    if (c0 >= a.c0_limit) {
        const uint32_t nn = kNaNbf16 | (kNaNbf16 << 16);
        *reinterpret_cast<uint4*>(o) = make_uint4(nn, nn, nn, nn);
        return;
    }
    const float4 x0 = reinterpret_cast<const float4*>(a.eN + i * d + j0)[0];
    const float4 x1 = reinterpret_cast<const float4*>(a.eN + i * d + j0)[1];
    const float acc[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float w[8];
    load_w8(w, a.wg, j0);
    const uint16_t* e1row = E1 ? a.e1 + static_cast<int64_t>(c0) * d + j0 : nullptr;
    const uint16_t* resrow = RES ? a.res + i * d + j0 : nullptr;
    *reinterpret_cast<uint4*>(o) = gate8<E1, RES>(acc, w, e1row, resrow);
}

// ---------------------------------------------------------------------------
// Projection: y[i][o] = sum over j of P[o][j] * x[i][j] for bf16 x and P
// ("Qwen 3.8 Flash-Next Deep Dive…", section 1: a "Projection /
// Normalization" stage after the lookup; the form is taken, the page does
// not define it).  A dense contraction, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation of exact bf16 products).
// A workgroup of 8 wavefronts owns a 256 x 256 tile of y (wavefront w: rows
// 128 (w >> 2), columns 64 (w & 3), as 4 x 2 MFMA tiles of 32 x 32) and walks
// K in steps of 64 through two LDS buffers.  Operands go from global memory
// straight into LDS (global_load_lds_dwordx4: lane L's 16 bytes land at the
// instruction's LDS base + 16 L), so they hold no registers on the way.  A
// step issues the next step's loads into the other buffer, then runs its four
// k-quarters: the 8 MFMAs of a quarter with the 6 fragment reads of the next
// quarter scheduled between them; a wavefront then waits for its own loads
// and the workgroup barrier closes the step, after which the step's last
// quarter of MFMAs runs beside the first reads of the next step.
// LDS rows are 64 bf16 (128 bytes, eight 16-byte chunks); chunk c of row r is
// stored at position c ^ ((r >> 1) & 7), so the 16 rows a 16-lane group of an
// operand read touches fall on 16 different 16-byte bank groups.  A load
// instruction fills 8 rows (1 KiB): lane L writes row L >> 3, position L & 7,
// so it fetches chunk (L & 7) ^ f(row) of that row.
// Tiles are ordered row-tile major and handed out XCD by XCD: workgroup b
// runs on XCD b mod 8, and the tiles of XCD x are a contiguous run of the
// order, so one row tile's x stays in that XCD's L2.  When a run is whole
// rows of tiles, the XCD walks it column by column instead, so its
// concurrent tiles share one P tile.
constexpr int kPM = 256, kPN = 256, kPK = 64, kPThreads = 512;
constexpr int kPTile = kPM * kPK * 2;                  // bytes of one operand tile of one step (x or P)
constexpr int kPStage = 2 * kPTile;                    // one LDS buffer: x tile then P tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct ProjArgs {
    const uint16_t* x;     // [n][K] bf16
    const uint16_t* P;     // [N][K] bf16
    float* y;              // [n][N] fp32
    int64_t n;
    int32_t K;
    int32_t N;
    int32_t ntiles_n;      // ceil(N / 256)
    int32_t ntiles;        // all tiles
};

__device__ inline uint32_t proj_pos(int row, int c) {
    return static_cast<uint32_t>(row) * (kPK * 2) + (static_cast<uint32_t>(c ^ ((row >> 1) & 7)) << 4);
}

// The step's 256-row x and P tiles into LDS buffer `buf`: 32 + 32
// instructions of 8 rows each, 4 + 4 per wavefront.  `xrow`, `prow`: the
// lane's source row pointers for its 4 row groups (rows past n or N are
// clamped to the last row: their results are never stored).
__device__ inline void proj_issue(uint8_t* buf, const uint16_t* const xrow[4], const uint16_t* const prow[4],
                                  const uint32_t chunk[4], int wave, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int g = 4 * wave + q;                       // row group: rows 8 g .. 8 g + 7
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(xrow[q] + k0 + 8 * chunk[q]),
            (__attribute__((address_space(3))) void*)(buf + g * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(prow[q] + k0 + 8 * chunk[q]),
            (__attribute__((address_space(3))) void*)(buf + kPTile + g * 1024), 16, 0, 0);
    }
}

// The wavefront's operand fragments of k-quarter kk from the LDS tiles xs and
// ps: lane L holds k = 16 kk + 8 (L >> 5) .. +7 of row L & 31 of each of its
// four 32-row x tiles and two 32-row P tiles.
__device__ __forceinline__ void proj_frags(bf16x8 fa[4], bf16x8 fb[2], const uint8_t* xs, const uint8_t* ps, int wm,
                                           int wn, int lane, int kk) {
    const int c = 2 * kk + (lane >> 5);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        fa[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xs + proj_pos(wm + 32 * s + (lane & 31), c)));
#pragma unroll
    for (int s = 0; s < 2; ++s)
        fb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ps + proj_pos(wn + 32 * s + (lane & 31), c)));
}

__device__ __forceinline__ void proj_mfma8(f32x16 acc[4][2], const bf16x8 fa[4], const bf16x8 fb[2]) {
#pragma unroll
    for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
            acc[sm][sn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sm], fb[sn], acc[sm][sn], 0, 0, 0);
}

// Scheduling of one quarter: MFMA, read, MFMA, read, ... (six reads between
// the eight MFMAs), so the LDS reads run while the matrix core is busy.
__device__ __forceinline__ void proj_interleave() {
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
}

__global__ void __launch_bounds__(kPThreads, 1) project_kernel(const ProjArgs a) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t plds[];   // [2][x 256 rows | P 256 rows] x 128 B
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // XCD-aware tile order: tiles of XCD b mod 8 form a contiguous run
    const int b = blockIdx.x, per = (a.ntiles + 7) / 8, xcd = b & 7, slot = b >> 3;
    const int full_xcds = a.ntiles - 8 * (per - 1);      // XCDs that get `per` tiles; the rest get per - 1
    if (slot >= (xcd < full_xcds ? per : per - 1)) return;
    const int base = xcd < full_xcds ? xcd * per : full_xcds * per + (xcd - full_xcds) * (per - 1);
    const int count = xcd < full_xcds ? per : per - 1;
    int mt, nt;
    if (base % a.ntiles_n == 0 && count % a.ntiles_n == 0) {
        // the run is whole rows of tiles: walk it column by column, so the
        // XCD's concurrent tiles read the same P tile (measured 4-5% faster
        // at 32768 x 2560 x 2560 than row by row)
        const int rows_x = count / a.ntiles_n;
        nt = slot / rows_x;
        mt = base / a.ntiles_n + (slot - nt * rows_x);
    } else {
        const int tile = base + slot;
        mt = tile / a.ntiles_n;
        nt = tile - mt * a.ntiles_n;
    }
    const int64_t m0 = static_cast<int64_t>(mt) * kPM;
    const int n0 = nt * kPN;
    const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
    // the lane's load sources: row 8 (4 wave + q) + (lane >> 3), chunk (lane & 7) ^ f(row)
    const uint16_t* xrow[4];
    const uint16_t* prow[4];
    uint32_t chunk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 8 * (4 * wave + q) + (lane >> 3);
        const int64_t xr = m0 + r < a.n ? m0 + r : a.n - 1;
        const int pr = n0 + r < a.N ? n0 + r : a.N - 1;
        xrow[q] = a.x + xr * a.K;
        prow[q] = a.P + static_cast<int64_t>(pr) * a.K;
        chunk[q] = static_cast<uint32_t>((lane & 7) ^ ((r >> 1) & 7));
    }
    const int KT = a.K / kPK;

    f32x16 acc[4][2];
#pragma unroll
    for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[sm][sn][e] = 0.0f;

    proj_issue(plds, xrow, prow, chunk, wave, 0);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Software pipeline over k-quarters (kk = 0..3 of a 64-wide step): the
    // 8 MFMAs of one quarter run while the 6 fragment reads of the next are
    // issued between them, and the last quarter of a step runs after the
    // step's barrier, beside the first reads of the next step.  ca/cb: the
    // fragments the next MFMAs use; na/nb: the ones being read.
    bf16x8 ca[4], cb[2], na[4], nb[2];
    proj_frags(ca, cb, plds, plds + kPTile, wm, wn, lane, 0);
    if (KT > 1) proj_issue(plds + kPStage, xrow, prow, chunk, wave, kPK);
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) {
        proj_frags(na, nb, plds, plds + kPTile, wm, wn, lane, kk);
        proj_mfma8(acc, ca, cb);
        proj_interleave();
#pragma unroll
        for (int s = 0; s < 4; ++s) ca[s] = na[s];
        cb[0] = nb[0]; cb[1] = nb[1];
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kt = 1; kt < KT; ++kt) {
        const uint8_t* xs = plds + (kt & 1) * kPStage;
        const uint8_t* ps = xs + kPTile;
        // the buffer of step kt - 1 was read out before the barrier
        if (kt + 1 < KT) proj_issue(plds + ((kt + 1) & 1) * kPStage, xrow, prow, chunk, wave, (kt + 1) * kPK);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            proj_frags(na, nb, xs, ps, wm, wn, lane, kk);
            proj_mfma8(acc, ca, cb);
            proj_interleave();
#pragma unroll
            for (int s = 0; s < 4; ++s) ca[s] = na[s];
            cb[0] = nb[0]; cb[1] = nb[1];
        }
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    proj_mfma8(acc, ca, cb);
    // Lane L holds rows 8 (e >> 2) + 4 (L >> 5) + (e & 3), column L & 31 of
    // each 32 x 32 tile.  The operand buffers are free (every read of them
    // finished before the last barrier), so each 32 x 32 tile goes through
    // this wavefront's 4 KiB of LDS and out as 16 bytes per lane: one store
    // instruction writes 8 rows of 128 consecutive bytes, where one 4-byte
    // value per lane took 4 times the instructions.  d_out % 8 == 0, so a
    // lane's 4 columns are all inside the row or all past it.
    float* st = reinterpret_cast<float*>(plds + wave * 4096);
    const int rq = lane >> 3, cq = 4 * (lane & 7);
#pragma unroll
    for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                st[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * 32 + (lane & 31)] = acc[sm][sn][e];
            __builtin_amdgcn_wave_barrier();
            const int col = n0 + wn + 32 * sn + cq;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(st + (8 * q + rq) * 32 + cq);
                const int64_t row = m0 + wm + 32 * sm + 8 * q + rq;
                if (row < a.n && col < a.N) *reinterpret_cast<float4*>(a.y + row * a.N + col) = v;
            }
            __builtin_amdgcn_wave_barrier();
        }
}

// Zero-copy staging of host-table rows: one wavefront per (token, k) row,
// 16-byte lanes (8- or 4-byte when the row size is not a multiple of 16), a
// whole row's loads issued before its stores; stage row t = i*16 + k.
struct StageArgs {
    const void* tab;
    const float* scale;
    const int32_t* rows;
    void* stage;
    float* stage_scale;
    int32_t* remap;
    int64_t nrows;      // n * 16
    int64_t R;
    int64_t row_bytes;
};

template <typename U>
__global__ void __launch_bounds__(1024) ngram_stage_kernel(const StageArgs a) {
    constexpr int kUnroll = 8;            // up to 8 x 64 lanes x 16 B of a row in flight
    const int lane = threadIdx.x & 63;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t nu = a.row_bytes / static_cast<int64_t>(sizeof(U));
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); t < a.nrows;
         t += waves) {
        const int32_t r = a.rows[t];
        const bool ok = r >= 0 && r < a.R;
        if (lane == 0) {
            a.remap[t] = ok ? static_cast<int32_t>(t) : -1;
            if (ok && a.stage_scale) a.stage_scale[t] = a.scale[r];
        }
        if (!ok) continue;
        const U* src = reinterpret_cast<const U*>(static_cast<const char*>(a.tab) + static_cast<int64_t>(r) * a.row_bytes);
        U* dst = reinterpret_cast<U*>(static_cast<char*>(a.stage) + t * a.row_bytes);
        for (int64_t q0 = 0; q0 < nu; q0 += 64 * kUnroll) {
            U buf[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q = q0 + u * 64 + lane;
                if (q < nu) buf[u] = src[q];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q = q0 + u * 64 + lane;
                if (q < nu) dst[q] = buf[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row pool: hot-row cache and per-batch dedup of misses for host tables.
template <typename U>
__device__ inline void copy_row(const U* __restrict__ src, U* __restrict__ dst, int64_t nu, int lane) {
    constexpr int kUnroll = 8;
    for (int64_t q0 = 0; q0 < nu; q0 += 64 * kUnroll) {
        U buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t q = q0 + u * 64 + lane;
            if (q < nu) buf[u] = src[q];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t q = q0 + u * 64 + lane;
            if (q < nu) dst[q] = buf[u];
        }
    }
}

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* p, int64_t count, int32_t v) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = v;
}

struct PoolArgs {
    const void* tab;           // host table (device-side address)
    const float* scale;        // host table's row scales (device) or null
    const int32_t* rows;       // [n*16]
    void* pool;                // [pool_rows][row_bytes]
    float* pool_scale;         // [pool_rows] or null
    const int32_t* slot_of_row;
    int32_t* pool_rows_out;    // [n*16]
    int32_t* keys;             // [H] hash set of missing row ids (-1: empty)
    int32_t* vals;             // [H] their staging index
    int32_t* miss;             // [n*16] distinct missing row ids, in staging order
    uint32_t* counter;         // number of distinct missing rows
    int64_t* fetched_out;
    int64_t nrows;             // n * 16
    int64_t R;
    int64_t cached;
    int64_t row_bytes;
    uint32_t mask;             // H - 1
    uint32_t shift;            // 32 - log2(H)
};

__device__ inline uint32_t set_home(int32_t r, uint32_t shift) {
    return (static_cast<uint32_t>(r) * 0x9E3779B1u) >> shift;
}

__global__ void __launch_bounds__(256) pool_insert_kernel(const PoolArgs a) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= a.nrows) return;
    const int32_t r = a.rows[t];
    if (r < 0 || r >= a.R || (a.slot_of_row && a.slot_of_row[r] >= 0)) return;
    uint32_t h = set_home(r, a.shift);
    for (uint32_t probe = 0; probe <= a.mask; ++probe) {
        const int32_t prev = atomicCAS(&a.keys[h], -1, r);
        if (prev == -1) {
            const uint32_t u = atomicAdd(a.counter, 1u);
            a.vals[h] = static_cast<int32_t>(u);
            a.miss[u] = r;
            return;
        }
        if (prev == r) return;
        h = (h + 1) & a.mask;
    }
}

__global__ void __launch_bounds__(256) pool_resolve_kernel(const PoolArgs a) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= a.nrows) return;
    const int32_t r = a.rows[t];
    int32_t out = -1;
    if (r >= 0 && r < a.R) {
        const int32_t s = a.slot_of_row ? a.slot_of_row[r] : -1;
        if (s >= 0) {
            out = s;
        } else {
            uint32_t h = set_home(r, a.shift);
            for (uint32_t probe = 0; probe <= a.mask; ++probe) {
                const int32_t k = a.keys[h];
                if (k == r) {
                    out = static_cast<int32_t>(a.cached + a.vals[h]);
                    break;
                }
                if (k == -1) break;
                h = (h + 1) & a.mask;
            }
        }
    }
    a.pool_rows_out[t] = out;
}

// Copy the distinct missing rows from the host table into the pool, one
// wavefront per row, on a capped persistent grid.
template <typename U>
__global__ void __launch_bounds__(1024) pool_fetch_kernel(const PoolArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t nmiss = static_cast<int64_t>(*a.counter);
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.fetched_out) *a.fetched_out = nmiss;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t nu = a.row_bytes / static_cast<int64_t>(sizeof(U));
    for (int64_t u = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); u < nmiss;
         u += waves) {
        const int32_t r = a.miss[u];
        const int64_t dst_row = a.cached + u;
        if (lane == 0 && a.pool_scale) a.pool_scale[dst_row] = a.scale[r];
        copy_row<U>(reinterpret_cast<const U*>(static_cast<const char*>(a.tab) + static_cast<int64_t>(r) * a.row_bytes),
                    reinterpret_cast<U*>(static_cast<char*>(a.pool) + dst_row * a.row_bytes), nu, lane);
    }
}

// The distinct-row count and, for int8 tables, the staged rows' scales, when
// the rows themselves are copied by the DMA engines (ngram_gather_host mode 1).
__global__ void __launch_bounds__(256) stage_meta_kernel(const PoolArgs a) {
    const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nmiss = static_cast<int64_t>(*a.counter);
    if (u == 0 && a.fetched_out) *a.fetched_out = nmiss;
    if (u < nmiss && a.pool_scale) a.pool_scale[u] = a.scale[a.miss[u]];
}

// Cache hot rows: wavefront per pool slot s, claiming slot_of_row[hot[s]].
template <typename U>
__global__ void __launch_bounds__(1024) pool_cache_kernel(const void* tab, const float* scale, const int32_t* hot,
                                                          int64_t C, int64_t R, void* pool, float* pool_scale,
                                                          int32_t* slot_of_row, int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t nu = row_bytes / static_cast<int64_t>(sizeof(U));
    for (int64_t s = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); s < C; s += waves) {
        const int32_t r = hot[s];
        if (r < 0 || r >= R) continue;
        int claimed = 0;
        if (lane == 0) claimed = atomicCAS(&slot_of_row[r], -1, static_cast<int32_t>(s)) == -1;
        claimed = __shfl(claimed, 0);
        if (!claimed) continue;
        if (lane == 0 && pool_scale) pool_scale[s] = scale[r];
        copy_row<U>(reinterpret_cast<const U*>(static_cast<const char*>(tab) + static_cast<int64_t>(r) * row_bytes),
                    reinterpret_cast<U*>(static_cast<char*>(pool) + s * row_bytes), nu, lane);
    }
}

__global__ void __launch_bounds__(256) count_rows_kernel(const int32_t* rows, int64_t nrows, int64_t R, int32_t* counts) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= nrows) return;
    const int32_t r = rows[t];
    if (r >= 0 && r < R) atomicAdd(&counts[r], 1);
}

constexpr int kHistBins = 1024;

__global__ void __launch_bounds__(256) count_hist_kernel(const int32_t* counts, int64_t R, int32_t* hist) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < R; r += stride) {
        const int32_t c = counts[r];
        if (c > 0) atomicAdd(&hist[c < kHistBins - 1 ? c : kHistBins - 1], 1);
    }
}

__global__ void __launch_bounds__(256) select_kernel(const int32_t* counts, int64_t R, int32_t tau, int64_t C,
                                                     int32_t* hot, uint32_t* sel) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < R; r += stride) {
        int32_t c = counts[r];
        if (c > kHistBins - 1) c = kHistBins - 1;
        if (c >= tau) {
            const uint32_t idx = atomicAdd(sel, 1u);
            if (idx < C) hot[idx] = static_cast<int32_t>(r);
        }
    }
}

// ---------------------------------------------------------------------------
// Gradients (the forward's chain rule, bf16 output rounding passed through):
// a stable LSD radix sort of (key, position) pairs groups equal row ids (or
// token ids) with their positions still ascending, then a segmented reduce
// sums each group in that fixed order.  No floating-point atomics, so every
// result is reproducible bit for bit.
constexpr int kSortItems = 4;                      // items per thread
constexpr int kSortThreads = 512;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortTile = kSortThreads * kSortItems;   // 2048 items per tile (256 tiles at prefill)
constexpr int kRadixBits = 9;
constexpr int kRadixBins = 1 << kRadixBits;            // 512
constexpr int kScanTile = 4096;                        // items per tile of the segment scan

// Where the first pass takes its items: the ids themselves (key = the id,
// or limit when it is out of range or its token is padding; value = the
// item's index), so no separate pass writes the initial keys.  The first
// pass's histogram kernel also clears the group and long-group counts.
struct SortSource {
    const int32_t* ids;            // NULL on later passes: read kin / vin
    const int32_t* valid_rows;     // NULL, or item t is valid only if valid_rows[t * stride] >= 0
    int stride;
    uint32_t limit;
    int64_t* n_unique;             // cleared by the first pass (NULL on later ones)
    uint32_t* nlong;
};

__device__ inline uint32_t sort_key(const SortSource& s, const uint32_t* __restrict__ kin, int64_t t) {
    if (!s.ids) return kin[t];
    const int32_t id = s.ids[t];
    bool ok = id >= 0 && static_cast<uint32_t>(id) < s.limit;
    if (s.valid_rows) ok = ok && s.valid_rows[t * s.stride] >= 0;
    return ok ? static_cast<uint32_t>(id) : s.limit;
}

// Per-tile digit counts: block_hist[digit][tile].
__global__ void __launch_bounds__(kSortThreads) radix_hist_kernel(SortSource src, const uint32_t* __restrict__ keys,
                                                                  int64_t N, int shift,
                                                                  uint32_t* __restrict__ block_hist, int64_t nblocks) {
    __shared__ uint32_t h[kRadixBins];
    if (src.n_unique && blockIdx.x == 0 && threadIdx.x == 0) {
        *src.n_unique = 0;
        *src.nlong = 0u;
    }
    for (int q = threadIdx.x; q < kRadixBins; q += kSortThreads) h[q] = 0;
    __syncthreads();
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kSortTile;
    for (int q = 0; q < kSortItems; ++q) {
        const int64_t idx = tile0 + q * kSortThreads + threadIdx.x;
        if (idx < N) atomicAdd(&h[(sort_key(src, keys, idx) >> shift) & (kRadixBins - 1)], 1u);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kRadixBins; q += kSortThreads)
        block_hist[static_cast<int64_t>(q) * nblocks + blockIdx.x] = h[q];
}

// Per digit d (one workgroup each, 256 threads): the exclusive scan of its
// tile counts block_hist[d][tile] over the tiles, in place, in chunks of 256
// tiles, and the digit's total in dtot[d].
__global__ void __launch_bounds__(256) digit_scan_kernel(uint32_t* __restrict__ block_hist, int64_t nblocks,
                                                         uint32_t* __restrict__ dtot) {
    __shared__ uint32_t wsum[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* h = block_hist + static_cast<int64_t>(blockIdx.x) * nblocks;
    uint32_t carry = 0;
    for (int64_t c0 = 0; c0 < nblocks; c0 += 256) {
        const int64_t t = c0 + threadIdx.x;
        const uint32_t v = t < nblocks ? h[t] : 0u;
        uint32_t x = v;                              // inclusive scan over the wavefront
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        uint32_t before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const uint32_t chunk = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        if (t < nblocks) h[t] = before + x - v;
        carry += chunk;
        __syncthreads();                             // wsum is rewritten by the next chunk
    }
    if (threadIdx.x == 0) dtot[blockIdx.x] = carry;
}

// Stable scatter of one 9-bit digit.  Tile order is (wavefront, round, lane):
// an item's rank among equal digits of its tile = equal digits in earlier
// wavefronts + in earlier rounds of its wavefront + in lower lanes of its
// round (lanes with an equal digit found by nine ballots).  An item of digit
// q goes to (the count of smaller digits: the exclusive scan of dtot, formed
// here) + (digit q in earlier tiles: offs[q][tile]) + its rank.  The tile is
// first reordered in LDS, so each store instruction writes runs of
// consecutive addresses rather than 64 scattered words.
__global__ void __launch_bounds__(kSortThreads) radix_scatter_kernel(SortSource src,
                                                                     const uint32_t* __restrict__ kin,
                                                                     const int32_t* __restrict__ vin, int64_t N,
                                                                     int shift, const uint32_t* __restrict__ offs,
                                                                     const uint32_t* __restrict__ dtot, int64_t nblocks,
                                                                     uint32_t* __restrict__ kout,
                                                                     int32_t* __restrict__ vout) {
    __shared__ uint32_t cnt[kSortWaves][kRadixBins];
    __shared__ uint32_t base[kRadixBins];
    __shared__ uint32_t tstart[kRadixBins];
    __shared__ uint32_t skey[kSortTile];
    __shared__ int32_t sval[kSortTile];
    __shared__ uint32_t wtot[kSortWaves];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int q = threadIdx.x; q < kSortWaves * kRadixBins; q += kSortThreads) (&cnt[0][0])[q] = 0;
    {
        // digit q = thread q (kSortThreads == kRadixBins): exclusive scan of the totals
        static_assert(kSortThreads == kRadixBins, "one thread per digit");
        const uint32_t tot = dtot[threadIdx.x];
        uint32_t x = tot;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wtot[w] = x;
        __syncthreads();
        uint32_t earlier = 0;
        for (int ww = 0; ww < w; ++ww) earlier += wtot[ww];
        base[threadIdx.x] = earlier + x - tot;
    }
    __syncthreads();
    const int64_t base0 = static_cast<int64_t>(blockIdx.x) * kSortTile + w * (64 * kSortItems);
    const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[kSortItems], local[kSortItems];
    int32_t val[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t idx = base0 + r * 64 + lane;
        const bool active = idx < N;
        key[r] = active ? sort_key(src, kin, idx) : 0u;
        val[r] = active ? (src.ids ? static_cast<int32_t>(idx) : vin[idx]) : 0;
        const uint32_t dg = (key[r] >> shift) & (kRadixBins - 1);
        uint64_t same = __ballot(active);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const bool bit = (dg >> b) & 1u;
            const uint64_t m = __ballot(active && bit);
            same &= bit ? m : ~m;
        }
        const uint32_t rank = static_cast<uint32_t>(__popcll(same & lower));
        uint32_t before = 0;
        if (active) before = cnt[w][dg];
        if (active && rank == 0) cnt[w][dg] = before + static_cast<uint32_t>(__popcll(same));
        local[r] = before + rank;
    }
    __syncthreads();
    {
        // digit dg = thread dg: cnt[w][dg] := equal digits in wavefronts
        // before w (exclusive prefix); tstart[dg] := the tile's items of
        // smaller digits; base[dg] := where the tile's run of dg starts in
        // the output
        const int dg = threadIdx.x;
        uint32_t acc = 0;
        for (int ww = 0; ww < kSortWaves; ++ww) {
            const uint32_t c = cnt[ww][dg];
            cnt[ww][dg] = acc;
            acc += c;
        }
        base[dg] += offs[static_cast<int64_t>(dg) * nblocks + blockIdx.x];
        uint32_t x = acc;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wtot[w] = x;             // its first use ended two barriers ago
        __syncthreads();
        uint32_t earlier = 0;
        for (int ww = 0; ww < w; ++ww) earlier += wtot[ww];
        tstart[dg] = earlier + x - acc;
    }
    __syncthreads();
    // the tile's items into LDS in output order (digit, then rank) ...
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t idx = base0 + r * 64 + lane;
        if (idx < N) {
            const uint32_t dg = (key[r] >> shift) & (kRadixBins - 1);
            const uint32_t slot = tstart[dg] + cnt[w][dg] + local[r];
            skey[slot] = key[r];
            sval[slot] = val[r];
        }
    }
    __syncthreads();
    // ... and out from there, consecutive threads taking consecutive slots, so
    // that the stores of one digit's run go to consecutive addresses
    const int64_t left = N - static_cast<int64_t>(blockIdx.x) * kSortTile;
    const int count = left < kSortTile ? static_cast<int>(left) : kSortTile;
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int slot = r * kSortThreads + threadIdx.x;
        if (slot < count) {
            const uint32_t k = skey[slot];
            const uint32_t dg = (k >> shift) & (kRadixBins - 1);
            const uint32_t pos = base[dg] + static_cast<uint32_t>(slot) - tstart[dg];
            kout[pos] = k;
            vout[pos] = sval[slot];
        }
    }
}

// Group numbering of the sorted keys, first half: per tile of kScanTile
// items, the exclusive scan of the group-start flags (a valid key that
// differs from its predecessor) into seg[], and the tile's count.
__global__ void __launch_bounds__(1024) seg_scan_kernel(const uint32_t* __restrict__ keys, int64_t N, uint32_t limit,
                                                        uint32_t* __restrict__ seg, uint32_t* __restrict__ tile_sums) {
    __shared__ uint32_t wsum[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * 4;
    uint32_t f[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t t = base + q;
        f[q] = 0u;
        if (t < N) {
            const uint32_t k = keys[t];
            f[q] = (k < limit && (t == 0 || keys[t - 1] != k)) ? 1u : 0u;
        }
        s += f[q];
    }
    uint32_t x = s;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t t = lane < 16 ? wsum[lane] : 0u;
        for (int off = 1; off < 16; off <<= 1) {
            const uint32_t y = __shfl_up(t, off);
            if (lane >= off) t += y;
        }
        if (lane < 16) wsum[lane] = t;
    }
    __syncthreads();
    uint32_t prefix = (wave > 0 ? wsum[wave - 1] : 0u) + x - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (base + q < N) seg[base + q] = prefix;
        prefix += f[q];
    }
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = wsum[15];
}

// Groups longer than this many items are walked by long_walk_kernel, with
// four times the rows in flight per wavefront (a
// Zipf-hot token's e1 gradient adds thousands of dL/dout rows, one after
// another per column): 512 items for the table's row groups, 64 for the e1
// gradient's token groups, whose Zipf head holds dozens of tokens with
// hundreds of items each (walked 16 rows at a time by seg_walk_kernel,
// they set its length).  The list of long groups has room for
// 16 n / kLongGroup + 1 entries, which covers both.
constexpr int kLongGroup = 512;
constexpr int kLongGroupE1 = 64;
static_assert(kLongGroupE1 * kK >= kLongGroup, "the e1 call's long groups must fit the list");

// Second half: seg[t] += the counts of the earlier tiles (each workgroup adds
// them up itself), then each group's first index, its id, the end sentinel
// and the group count; a group longer than long_min items (its last item t
// has the same key as item t - long_min, the keys being sorted) is also
// listed in longs[], in an unspecified order.
__global__ void __launch_bounds__(1024) seg_bounds_kernel(const uint32_t* __restrict__ keys, uint32_t* __restrict__ seg,
                                                          const uint32_t* __restrict__ tile_sums, int64_t N,
                                                          uint32_t limit, int32_t* __restrict__ seg_start,
                                                          int32_t* __restrict__ ids_out, int64_t* __restrict__ n_unique,
                                                          int32_t* __restrict__ longs, uint32_t* __restrict__ nlong,
                                                          int long_min) {
    __shared__ uint32_t red[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t part = 0;
    for (int64_t q = threadIdx.x; q < blockIdx.x; q += 1024) part += tile_sums[q];
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    uint32_t earlier = 0;
    for (int q = 0; q < 16; ++q) earlier += red[q];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t t = base + q;
        if (t >= N) break;
        const uint32_t sg = seg[t] + earlier;
        seg[t] = sg;
        const uint32_t k = keys[t];
        if (k >= limit) continue;
        const bool first = t == 0 || keys[t - 1] != k;
        if (first) {
            seg_start[sg] = static_cast<int32_t>(t);
            ids_out[sg] = static_cast<int32_t>(k);
        }
        if (t + 1 == N || keys[t + 1] >= limit) {
            const uint32_t U = sg + (first ? 1u : 0u);
            seg_start[U] = static_cast<int32_t>(t + 1);
            *n_unique = U;
        }
        const bool last = t + 1 == N || keys[t + 1] != k;
        if (last && t >= long_min && keys[t - long_min] == k)     // then not first: group sg - 1
            longs[atomicAdd(nlong, 1u)] = static_cast<int32_t>(sg - 1u);
    }
}

__global__ void __launch_bounds__(64) set_i64_kernel(int64_t* p, int64_t v) {
    if (threadIdx.x == 0) *p = v;
}

// Workgroup c owns the groups that start among sorted items [64 c, 64 c + 64)
// and walks their items in order (past the chunk's end for the last group),
// one wavefront per 512-column slice: acc = fmaf(W_g, g[i], acc) (table) or
// acc + g[i] (e1), i = position >> pos_shift; a group's sum is stored when
// the id changes.  The dL/dout rows of the next DEPTH items are loaded ahead
// (groups can be thousands of items long: a Zipf-hot token's e1 gradient).
constexpr int kWalkChunk = 128;

// 16 rows ahead: the deepest prefetch that stays in registers (no scratch).
constexpr int kWalkDepth = 16;

// Rows of items tb + first .. tb + first + B - 1 (lanes of pl hold the
// positions of items tb + 0 .. 63); an item past the end loads item tb's row,
// which is always valid, and is not added.
template <int B>
__device__ inline void walk_load(uint4 gv[B], int32_t pl, int first, int64_t tb, int64_t te,
                                 const uint16_t* __restrict__ g, int32_t d, int64_t ja, int64_t jb, int pos_shift) {
#pragma unroll
    for (int m = 0; m < B; ++m) {
        const int src = tb + first + m < te ? first + m : 0;
        const int64_t i = static_cast<int64_t>(__builtin_amdgcn_readlane(pl, src) >> pos_shift);
        const uint2 a = *reinterpret_cast<const uint2*>(g + i * d + ja);
        const uint2 b = *reinterpret_cast<const uint2*>(g + i * d + jb);
        gv[m] = make_uint4(a.x, a.y, b.x, b.y);
    }
}

// Add the bank's items in order; when the id changes, store the finished
// group's sum and start the next one.
template <bool WEIGHT, int B>
__device__ inline void walk_add(float acc[8], const float w[8], const uint4 gv[B], uint32_t kl, int first,
                                int64_t tb, int64_t te, uint32_t& prev, int64_t& uo, float* __restrict__ out,
                                int32_t d, int64_t ja, int64_t jb, bool ok_a, bool ok_b) {
    // (ok_a, ok_b: the lane's two column groups exist)
#pragma unroll
    for (int m = 0; m < B; ++m) {
        if (tb + first + m < te) {          // uniform predicate, so every index stays constant
            const uint32_t km = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kl), first + m));
            if (km != prev) {               // a new group: store the finished one
                float* o = out + uo * d;
                if (ok_a) *reinterpret_cast<float4*>(o + ja) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                if (ok_b) *reinterpret_cast<float4*>(o + jb) = make_float4(acc[4], acc[5], acc[6], acc[7]);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
                ++uo;
                prev = km;
            }
            const float x[8] = {bf16lo(gv[m].x), bf16hi(gv[m].x), bf16lo(gv[m].y), bf16hi(gv[m].y),
                                bf16lo(gv[m].z), bf16hi(gv[m].z), bf16lo(gv[m].w), bf16hi(gv[m].w)};
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = WEIGHT ? __builtin_fmaf(w[q], x[q], acc[q]) : acc[q] + x[q];
        }
    }
}

template <bool WEIGHT, bool FULL>
__global__ void __launch_bounds__(1024) seg_walk_kernel(const uint32_t* __restrict__ keys,
                                                        const uint32_t* __restrict__ seg,
                                                        const int32_t* __restrict__ seg_start,
                                                        const int64_t* __restrict__ n_unique,
                                                        const int32_t* __restrict__ sorted_pos, int pos_shift,
                                                        const uint16_t* __restrict__ g, const float* __restrict__ W,
                                                        int32_t d, float* __restrict__ out, int long_min) {
    const int64_t U = *n_unique;
    if (U == 0) return;
    const int64_t nvalid = seg_start[U];
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWalkChunk;
    if (t0 >= nvalid) return;
    // group of item t0 = seg[t0] + flag[t0] - 1; it starts here or earlier
    const uint32_t k0 = keys[t0];
    const bool starts = t0 == 0 || keys[t0 - 1] != k0;
    int64_t u = static_cast<int64_t>(seg[t0]) - (starts ? 0 : 1);
    if (!starts) ++u;                               // that group belongs to an earlier chunk
    if (u >= U || seg_start[u] >= t0 + kWalkChunk) return;
    // last group that starts inside the chunk
    const int64_t tl = (t0 + kWalkChunk < nvalid ? t0 + kWalkChunk : nvalid) - 1;
    const bool tl_starts = keys[tl - 1 >= 0 ? tl - 1 : 0] != keys[tl] || tl == 0;
    const int64_t u_last = static_cast<int64_t>(seg[tl]) - (tl_starts ? 0 : 1);
    const int64_t t_begin = seg_start[u];
    int64_t t_end = seg_start[u_last + 1];
    // a group longer than long_min items (only the last one can be) is
    // walked by long_walk_kernel instead
    if (t_end - seg_start[u_last] > long_min) {
        if (u_last == u) return;
        t_end = seg_start[u_last];
    }

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    const int nslices = (d + kSlice - 1) / kSlice;
    // The walk stays in uniform control flow: every lane loads its share of
    // the ids and positions that readlane then reads from any lane.  Lanes
    // past the row's end work on column 0 and do not store.
    for (int sl = wave; sl < nslices; sl += nwaves) {
        // lane l owns columns 4l..4l+3 and 256+4l..256+4l+3 of the slice, so
        // each of a group's two row stores writes 1 KiB of consecutive
        // addresses (d is a multiple of 8, so a 4-column group is whole)
        const int64_t j0a = static_cast<int64_t>(sl) * kSlice + lane * 4;
        const int64_t j0b = j0a + kSlice / 2;
        const bool ok_a = FULL || j0a < d, ok_b = FULL || j0b < d;
        // (FULL: d is a multiple of 512, every lane has both column groups,
        // and the second is the first plus 512 bytes in every row)
        const int64_t ja = FULL || ok_a ? j0a : 0, jb = FULL || ok_b ? j0b : 0;
        float w[8];
        if (WEIGHT) {
            const float4 wa = *reinterpret_cast<const float4*>(W + ja);
            const float4 wb = *reinterpret_cast<const float4*>(W + jb);
            w[0] = wa.x; w[1] = wa.y; w[2] = wa.z; w[3] = wa.w;
            w[4] = wb.x; w[5] = wb.y; w[6] = wb.z; w[7] = wb.w;
        }
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        int64_t uo = u;
        uint32_t prev = keys[t_begin];
        // ids and positions of 64 items per vector load, the next 64 loaded
        // while the current ones are walked; lane m of (kl, pl) is item tb + m
        uint32_t kl = t_begin + lane < t_end ? keys[t_begin + lane] : 0u;
        int32_t pl = t_begin + lane < t_end ? sorted_pos[t_begin + lane] : 0;
        for (int64_t tb = t_begin; tb < t_end; tb += 64) {
            const int64_t tn = tb + 64 + lane;
            const uint32_t kl_next = tn < t_end ? keys[tn] : 0u;
            const int32_t pl_next = tn < t_end ? sorted_pos[tn] : 0;
            for (int m0 = 0; m0 < 64 && tb + m0 < t_end; m0 += kWalkDepth) {
                uint4 gv[kWalkDepth];
                walk_load<kWalkDepth>(gv, pl, m0, tb, t_end, g, d, ja, FULL ? ja + kSlice / 2 : jb, pos_shift);
                walk_add<WEIGHT, kWalkDepth>(acc, w, gv, kl, m0, tb, t_end, prev, uo, out, d, ja, jb, ok_a, ok_b);
            }
            kl = kl_next;
            pl = pl_next;
        }
        float* o = out + uo * d;
        if (ok_a) *reinterpret_cast<float4*>(o + ja) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (ok_b) *reinterpret_cast<float4*>(o + jb) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// One long group per workgroup iteration, one wavefront per workgroup: lane c
// of workgroup (x, y) owns column 64 y + c and adds the group's items in
// position order, so each column's sum runs in the same order as in
// seg_walk_kernel.  A group's items are taken in units of 64, kLongUnits units
// in flight.  The dL/dout rows go straight into LDS (global_load_lds_dwordx4:
// lanes 8 j .. 8 j + 7 of an instruction fetch 16 bytes each of item j's 64
// columns, which land as one 128-byte row), so a wavefront keeps 256 rows in
// flight without holding them in registers; a chain of thousands of items then
// waits for memory once per 256 items rather than once per 64.  The items'
// positions take the same route, issued before the rows of the unit kLongUnits
// earlier: the load counter drains in issue order, so when a unit's rows have
// landed, so have the positions of the unit whose rows are issued next.
constexpr int kLongUnits = 4;      // units of 64 items in flight
constexpr int kLongOps = 9;        // loads per unit: 1 of 64 positions + 8 of 8 rows
static_assert((kLongUnits - 1) * kLongOps == 27, "the wait below counts the loads of kLongUnits - 1 units");

struct LongLds {
    uint8_t rows[kLongUnits][64 * 128];        // item j of a unit: its 64 columns at 128 j
    int32_t pos[2 * kLongUnits][64];
};

// Positions of unit x's items (past te: item tb0's, which is valid) into pos[slot].
__device__ inline void long_issue_pos(LongLds& L, int slot, const int32_t* __restrict__ sorted_pos, int64_t tb0,
                                      int64_t te, int64_t x, int lane) {
    const int64_t t = tb0 + 64 * x + lane;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(sorted_pos + (t < te ? t : tb0)),
                                     (__attribute__((address_space(3))) void*)(&L.pos[slot][0]), 4, 0, 0);
}

// Rows of the unit whose positions are in pos[pslot] into rows[slot]: load m
// fetches items 8 m .. 8 m + 7, lane l item 8 m + (l >> 3), columns lc .. lc + 7.
__device__ inline void long_issue_rows(LongLds& L, int slot, int pslot, const uint16_t* __restrict__ g, int32_t d,
                                       int64_t lc, int pos_shift, int lane) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int64_t i = static_cast<int64_t>(L.pos[pslot][8 * m + (lane >> 3)] >> pos_shift);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + i * d + lc),
                                         (__attribute__((address_space(3))) void*)(&L.rows[slot][1024 * m]), 16, 0, 0);
    }
}

template <bool WEIGHT>
__global__ void __launch_bounds__(64) long_walk_kernel(const int32_t* __restrict__ longs,
                                                       const uint32_t* __restrict__ nlong,
                                                       const int32_t* __restrict__ seg_start,
                                                       const int32_t* __restrict__ sorted_pos, int pos_shift,
                                                       const uint16_t* __restrict__ g, const float* __restrict__ W,
                                                       int32_t d, float* __restrict__ out) {
    __shared__ LongLds L;
    const int lane = threadIdx.x;
    const int64_t col = static_cast<int64_t>(blockIdx.y) * 64 + lane;
    const bool col_ok = col < d;
    // d % 8 == 0: the 8 columns a lane fetches are all inside the row or all
    // past it (then it fetches columns 0 .. 7, which no lane adds)
    const int64_t lcol = static_cast<int64_t>(blockIdx.y) * 64 + (lane & 7) * 8;
    const int64_t lc = lcol < d ? lcol : 0;
    const float w = WEIGHT ? W[col_ok ? col : 0] : 1.0f;
    const int64_t count = *nlong;
    for (int64_t q = blockIdx.x; q < count; q += gridDim.x) {
        const int64_t u = longs[q];
        const int64_t tb0 = seg_start[u], te = seg_start[u + 1];
        const int64_t nunits = (te - tb0 + 63) / 64;
        for (int x = 0; x < kLongUnits; ++x) long_issue_pos(L, x, sorted_pos, tb0, te, x, lane);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (int x = 0; x < kLongUnits; ++x) {
            long_issue_pos(L, x + kLongUnits, sorted_pos, tb0, te, x + kLongUnits, lane);
            long_issue_rows(L, x, x, g, d, lc, pos_shift, lane);
        }
        float acc = 0.0f;
        for (int64_t k = 0; k < nunits; ++k) {
            // unit k's rows have landed (the loads of the kLongUnits - 1 later
            // units may still be in flight), and with them every earlier load
            __asm__ volatile("s_waitcnt vmcnt(27)" ::: "memory");
            const int rs = static_cast<int>(k % kLongUnits);
            const int64_t left = te - tb0 - 64 * k;
            const int nk = left < 64 ? static_cast<int>(left) : 64;
            const uint16_t* r = reinterpret_cast<const uint16_t*>(&L.rows[rs][0]) + lane;
#pragma unroll 16
            for (int j = 0; j < nk; ++j) {
                const float x = __uint_as_float(static_cast<uint32_t>(r[64 * j]) << 16);
                acc = WEIGHT ? __builtin_fmaf(w, x, acc) : acc + x;
            }
            // slot rs is read out before it is refilled
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            long_issue_pos(L, static_cast<int>(k % (2 * kLongUnits)), sorted_pos, tb0, te, k + 2 * kLongUnits, lane);
            long_issue_rows(L, rs, static_cast<int>((k + kLongUnits) % (2 * kLongUnits)), g, d, lc, pos_shift, lane);
        }
        // no load may land once the slots serve the next group or the
        // workgroup has ended
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (col_ok) out[u * d + col] = acc;
    }
}

// dW_g[j] = the sum over valid tokens i of g[i][j] eN[i][j], accumulated in
// float64 (each product of a bf16 and an fp32 value is exact there) and
// rounded once to fp32.  The sum has no stated order; here: per chunk of
// kGateChunk tokens, each of a workgroup's 4 wavefronts sums a quarter of the
// chunk, the quarters are added in LDS, and the chunk partials are then added
// per column.  The order is fixed, so the bits are reproducible.
constexpr int kGateChunk = 128;
constexpr int kGateWaves = 4;
constexpr int kGateCols = 4;       // columns per lane: 256 per wavefront
constexpr int kGateUnroll = 8;     // tokens whose loads are issued together
constexpr int kGateGrid = 1024;    // workgroups at most: 4 of 4 wavefronts per compute unit

__global__ void __launch_bounds__(256) gate_grad_partial_kernel(const int32_t* __restrict__ rows,
                                                                const uint16_t* __restrict__ g,
                                                                const float* __restrict__ eN, int64_t n, int32_t d,
                                                                int64_t nchunks, int colblocks,
                                                                double* __restrict__ partials) {
    __shared__ double lp[kGateWaves][64 * kGateCols];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int kPerWave = kGateChunk / kGateWaves;
    // work item q = (chunk q / colblocks, 256-column block q % colblocks)
    for (int64_t q = blockIdx.x; q < nchunks * colblocks; q += gridDim.x) {
        const int64_t c = q / colblocks;
        const int64_t j0 = ((q % colblocks) * 64 + lane) * kGateCols;
        const bool col = j0 < d;       // d % 8 == 0, so the lane's 4 columns are all in range
        const int64_t i0 = c * kGateChunk + wave * kPerWave;
        const int64_t i1 = i0 + kPerWave < n ? i0 + kPerWave : n;
        double part[kGateCols] = {0.0, 0.0, 0.0, 0.0};
        if (col) {
            for (int64_t ib = i0; ib < i1; ib += kGateUnroll) {
                uint2 gv[kGateUnroll];
                float4 ev[kGateUnroll];
                bool ok[kGateUnroll];
#pragma unroll
                for (int u = 0; u < kGateUnroll; ++u) {
                    const int64_t i = ib + u < i1 ? ib + u : ib;
                    ok[u] = ib + u < i1 && rows[i * kK] >= 0;
                    gv[u] = *reinterpret_cast<const uint2*>(g + i * d + j0);
                    ev[u] = *reinterpret_cast<const float4*>(eN + i * d + j0);
                }
#pragma unroll
                for (int u = 0; u < kGateUnroll; ++u) {
                    if (!ok[u]) continue;
                    part[0] = part[0] + static_cast<double>(bf16lo(gv[u].x)) * static_cast<double>(ev[u].x);
                    part[1] = part[1] + static_cast<double>(bf16hi(gv[u].x)) * static_cast<double>(ev[u].y);
                    part[2] = part[2] + static_cast<double>(bf16lo(gv[u].y)) * static_cast<double>(ev[u].z);
                    part[3] = part[3] + static_cast<double>(bf16hi(gv[u].y)) * static_cast<double>(ev[u].w);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < kGateCols; ++e) lp[wave][lane * kGateCols + e] = part[e];
        __syncthreads();
        if (wave == 0 && col) {
#pragma unroll
            for (int e = 0; e < kGateCols; ++e) {
                double t = lp[0][lane * kGateCols + e];
                for (int w = 1; w < kGateWaves; ++w) t = t + lp[w][lane * kGateCols + e];
                partials[c * d + j0 + e] = t;
            }
        }
        __syncthreads();               // lp is rewritten by the next item
    }
}

// Per column: the chunk partials, 16 wavefronts each adding every 16th chunk,
// then the 16 sums in wavefront order, rounded once to fp32.
constexpr int kGateTotalWaves = 16;

__global__ void __launch_bounds__(1024) gate_grad_total_kernel(const double* __restrict__ partials, int64_t nchunks,
                                                               int32_t d, float* __restrict__ out) {
    __shared__ double red[kGateTotalWaves][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    double t = 0.0;
    if (j < d) {
#pragma unroll 8
        for (int64_t c = wave; c < nchunks; c += kGateTotalWaves) t = t + partials[c * d + j];
    }
    red[wave][lane] = t;
    __syncthreads();
    if (wave == 0 && j < d) {
        double s = red[0][lane];
        for (int w = 1; w < kGateTotalWaves; ++w) s = s + red[w][lane];
        out[j] = static_cast<float>(s);
    }
}

// ---------------------------------------------------------------------------
// Host side.
int hip_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NGRAM_EHIP, "%s: %s", what, hipGetErrorString(e));
    return NGRAM_OK;
}

int check_table(const ngram_table* T) {
    if (!T) return fail(NGRAM_EINVAL, "table is NULL");
    if (!T->data) return fail(NGRAM_EINVAL, "table data is NULL");
    if (T->R < 1 || T->R > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "R=%lld outside [1, 2^31-1]", (long long)T->R);
    if (T->d <= 0 || T->d % kVec != 0) return fail(NGRAM_EINVAL, "d=%d must be a positive multiple of 8", T->d);
    if (T->d > NGRAM_MAX_D) return fail(NGRAM_ERANGE, "d=%d above %d", T->d, NGRAM_MAX_D);
    if (T->dtype == NGRAM_TABLE_BF16) {
        if (!aligned(T->data, 16)) return fail(NGRAM_EALIGN, "bf16 table data not 16-byte aligned");
    } else if (T->dtype == NGRAM_TABLE_INT8_ROWSCALE) {
        if (!aligned(T->data, 8)) return fail(NGRAM_EALIGN, "int8 table data not 8-byte aligned");
        if (!T->row_scale) return fail(NGRAM_EINVAL, "int8 table needs row_scale");
        if (!aligned(T->row_scale, 4)) return fail(NGRAM_EALIGN, "row_scale not 4-byte aligned");
    } else if (T->dtype == NGRAM_TABLE_MXFP4) {
        if (T->d % 128 != 0) return fail(NGRAM_EINVAL, "MXFP4 rows need d %% 128 == 0 (d=%d)", T->d);
        if (!aligned(T->data, 16)) return fail(NGRAM_EALIGN, "MXFP4 table data not 16-byte aligned");
    } else {
        return fail(NGRAM_EINVAL, "unknown table dtype %d", T->dtype);
    }
    if (T->location != NGRAM_IN_DEVICE && T->location != NGRAM_IN_HOST)
        return fail(NGRAM_EINVAL, "unknown table location %d", T->location);
    return NGRAM_OK;
}

// The device-side address of the table data (host tables: the mapping).
int table_device_ptr(const ngram_table* T, const void** out) {
    if (T->location == NGRAM_IN_DEVICE) {
        *out = T->data;
        return NGRAM_OK;
    }
    void* dp = nullptr;
    const hipError_t e = hipHostGetDevicePointer(&dp, const_cast<void*>(T->data), 0);
    if (e != hipSuccess || !dp) {
        (void)hipGetLastError();
        return fail(NGRAM_EHIP, "host table is not pinned, device-mapped memory: %s", hipGetErrorString(e));
    }
    *out = dp;
    return NGRAM_OK;
}

int check_tokens(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S) {
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > INT32_MAX) return fail(NGRAM_ERANGE, "n=%lld above 2^31-1", (long long)n);
    if (n > 0 && !tokens) return fail(NGRAM_EINVAL, "tokens is NULL");
    if (n > 0 && !seq_offsets) return fail(NGRAM_EINVAL, "seq_offsets is NULL");
    if (n > 0 && S < 1) return fail(NGRAM_EINVAL, "S=%d must be >= 1 when n > 0", S);
    return NGRAM_OK;
}

Seeds make_seeds(const uint64_t* seeds) {
    Seeds s;
    for (int k = 0; k < kK; ++k) s.s[k] = seeds ? seeds[k] : splitmix64(static_cast<uint64_t>(k) * 0x9E3779B97F4A7C15ull);
    return s;
}

uint32_t c0_limit_for(const uint16_t* e1, int64_t V) {
    if (!e1) return kPad;
    return V < static_cast<int64_t>(kPad) ? static_cast<uint32_t>(V) : kPad;
}

// Launch shape of the slice kernels: one wavefront per 512-column slice (at
// most 16 per workgroup) and `tpw` tokens per workgroup.
struct Shape {
    int waves;
    int tpw;
    int64_t grid;
    bool persist;
};

// Tokens per workgroup: 1 for bf16 rows; 4 for int8 rows, whose half-size
// slices leave the per-workgroup hash phase and barrier a larger share of the
// time (measured on MI355X at 2560 columns: int8 5.3 TB/s at 1 token per
// workgroup, 6.6 TB/s at 4; bf16 best at 1).
Shape slice_shape(int64_t n, int32_t d, int32_t dtype, const ngram_launch* L) {
    const int nslices = (d + kSlice - 1) / kSlice;
    Shape s;
    s.waves = nslices < 16 ? nslices : 16;
    int tpw = L ? L->tokens_per_workgroup : 0;
    if (tpw <= 0) tpw = dtype == NGRAM_TABLE_BF16 ? 1 : 4;     // int8, MXFP4: 4
    if (tpw > 64) tpw = 64;
    s.tpw = tpw;
    s.grid = (n + tpw - 1) / tpw;
    s.persist = false;
    return s;
}

// A table in pinned host memory is read over PCIe, which a few workgroups
// saturate; a capped, persistent grid leaves the other compute units to the
// work it overlaps with on other streams.  Measured on MI355X (8192 tokens,
// 5M x 2560 bf16 host table, against a bf16 GEMM loop on another stream):
// 8 workgroups read at 58 GB/s and leave 4.3 ms of an 11.6 ms gather
// exposed; 64 leave 9.5 ms, 256 leave 12.5 ms.
constexpr int kHostWorkgroups = 8;

int host_workgroups(const ngram_launch* L) {
    return L && L->host_workgroups > 0 ? L->host_workgroups : kHostWorkgroups;
}

int64_t table_row_bytes(const ngram_table* T) {
    const int64_t d = T->d;
    if (T->dtype == NGRAM_TABLE_BF16) return 2 * d;
    if (T->dtype == NGRAM_TABLE_MXFP4) return d / 2 + d / 32;
    return d;
}

unsigned grid_for(int64_t count) {
    int64_t g = (count + 255) / 256;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return static_cast<unsigned>(g);
}

// Workspace of ngram_pool_gather: a hash set of 2^k >= 2 * 16 n slots (keys and
// staging indices), the list of distinct missing rows, a counter; the
// selection call reuses the front for a 1024-bin histogram and a counter.
struct PoolLayout {
    int64_t H, log2H, keys, vals, miss, counter, total;
};

PoolLayout pool_layout(int64_t n) {
    PoolLayout L;
    L.log2H = 6;
    while ((int64_t{1} << L.log2H) < 2 * kK * n) ++L.log2H;
    L.H = int64_t{1} << L.log2H;
    L.keys = 0;
    L.vals = 4 * L.H;
    L.miss = 8 * L.H;
    L.counter = ((8 * L.H + 4 * kK * n) + 15) & ~int64_t{15};
    L.total = L.counter + 16;
    const int64_t select_need = 4 * (kHistBins + 4);
    if (L.total < select_need) L.total = select_need;
    return L;
}

int check_pool(const ngram_table* T, const ngram_row_pool* P) {
    int rc = check_table(T);
    if (rc) return rc;
    if (T->location != NGRAM_IN_HOST) return fail(NGRAM_ENOTSUP, "the row pool fronts a host table");
    if (!P || !P->data || !P->slot_of_row) return fail(NGRAM_EINVAL, "pool, pool data or slot_of_row is NULL");
    if (!aligned(P->data, 16)) return fail(NGRAM_EALIGN, "pool data not 16-byte aligned");
    if (T->dtype == NGRAM_TABLE_INT8_ROWSCALE && !P->row_scale) return fail(NGRAM_EINVAL, "int8 pool needs row_scale");
    if (P->pool_rows < 0 || P->pool_rows > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "pool_rows out of range");
    return NGRAM_OK;
}

// Workspace of the gradient calls, for N = 16 n sort items (the table) and
// the gate's chunk partials.
struct GradLayout {
    int64_t N, nblocks, ntiles, keysA, valsA, keysB, valsB, segs, starts, hist, dtot, tiles, longs, parts, total;
};

GradLayout grad_layout(int64_t n, int32_t d) {
    auto up = [](int64_t x) { return (x + 255) & ~int64_t{255}; };
    GradLayout L;
    L.N = kK * n;
    L.nblocks = (L.N + kSortTile - 1) / kSortTile;
    L.ntiles = (L.N + kScanTile - 1) / kScanTile;
    int64_t o = 0;
    L.keysA = o; o = up(o + 4 * L.N);
    L.valsA = o; o = up(o + 4 * L.N);
    L.keysB = o; o = up(o + 4 * L.N);
    L.valsB = o; o = up(o + 4 * L.N);
    L.segs = o; o = up(o + 4 * L.N);
    L.starts = o; o = up(o + 4 * (L.N + 1));
    L.hist = o; o = up(o + 4 * kRadixBins * (L.nblocks > 0 ? L.nblocks : 1));
    L.dtot = o; o = up(o + 4 * kRadixBins);
    L.tiles = o; o = up(o + 4 * (L.ntiles > 0 ? L.ntiles : 1));
    L.longs = o; o = up(o + 16 + 4 * (L.N / kLongGroup + 1));
    L.parts = o; o = up(o + 8 * ((n + kGateChunk - 1) / kGateChunk) * static_cast<int64_t>(d > 0 ? d : 1));
    L.total = o;
    return L;
}

// Stable sort of N (key, value) pairs by key (keys <= limit), ping-ponging
// between the A and B buffers; returns the buffers that hold the result.
// Each 9-bit pass: per-tile digit counts, each digit's scan over the tiles
// (one workgroup per digit), the stable scatter.
void radix_sort(char* ws, const GradLayout& L, int64_t N, const SortSource& first, hipStream_t st,
                uint32_t** keys_out, int32_t** vals_out) {
    uint32_t* kA = reinterpret_cast<uint32_t*>(ws + L.keysA);
    int32_t* vA = reinterpret_cast<int32_t*>(ws + L.valsA);
    uint32_t* kB = reinterpret_cast<uint32_t*>(ws + L.keysB);
    int32_t* vB = reinterpret_cast<int32_t*>(ws + L.valsB);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* dtot = reinterpret_cast<uint32_t*>(ws + L.dtot);
    const int64_t nblocks = (N + kSortTile - 1) / kSortTile;
    int bits = 1;
    while (bits < 32 && (first.limit >> bits) != 0) ++bits;
    const int passes = (bits + kRadixBits - 1) / kRadixBits;
    for (int p = 0; p < passes; ++p) {
        const int shift = kRadixBits * p;
        const SortSource src = p == 0 ? first : SortSource{nullptr, nullptr, 0, first.limit, nullptr, nullptr};
        hipLaunchKernelGGL(radix_hist_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kSortThreads), 0, st, src,
                           kA, N, shift, hist, nblocks);
        hipLaunchKernelGGL(digit_scan_kernel, dim3(kRadixBins), dim3(256), 0, st, hist, nblocks, dtot);
        hipLaunchKernelGGL(radix_scatter_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kSortThreads), 0, st, src,
                           kA, vA, N, shift, hist, dtot, nblocks, kB, vB);
        uint32_t* tk = kA; kA = kB; kB = tk;
        int32_t* tv = vA; vA = vB; vB = tv;
    }
    *keys_out = kA;
    *vals_out = vA;
}

// Sort, find the groups of equal ids and reduce each group in position order
// (groups longer than long_min items in a launch of their own).
template <bool WEIGHT>
int grad_by_groups(const int32_t* ids, int64_t N, int stride, const int32_t* valid_rows, uint32_t limit, int pos_shift,
                   const uint16_t* g, const float* W, int32_t d, int32_t* ids_out, float* grad_out, int64_t* n_unique,
                   void* workspace, const GradLayout& L, int long_min, hipStream_t st) {
    char* ws = static_cast<char*>(workspace);
    if (N == 0) {
        hipLaunchKernelGGL(set_i64_kernel, dim3(1), dim3(64), 0, st, n_unique, int64_t{0});
        return hip_status("gradient launch");
    }
    uint32_t* nlong = reinterpret_cast<uint32_t*>(ws + L.longs);
    int32_t* longs = reinterpret_cast<int32_t*>(ws + L.longs + 16);
    uint32_t* keys = nullptr;
    int32_t* pos = nullptr;
    radix_sort(ws, L, N, SortSource{ids, valid_rows, stride, limit, n_unique, nlong}, st, &keys, &pos);
    uint32_t* segs = reinterpret_cast<uint32_t*>(ws + L.segs);
    int32_t* starts = reinterpret_cast<int32_t*>(ws + L.starts);
    uint32_t* tiles = reinterpret_cast<uint32_t*>(ws + L.tiles);
    const unsigned ntiles = static_cast<unsigned>((N + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(ntiles), dim3(1024), 0, st, keys, N, limit, segs, tiles);
    hipLaunchKernelGGL(seg_bounds_kernel, dim3(ntiles), dim3(1024), 0, st, keys, segs, tiles, N, limit, starts, ids_out,
                       n_unique, longs, nlong, long_min);
    const int nslices = (d + kSlice - 1) / kSlice;
    const int waves = nslices < 16 ? nslices : 16;
    const int64_t grid = (N + kWalkChunk - 1) / kWalkChunk;
    if (d % kSlice == 0)
        hipLaunchKernelGGL((seg_walk_kernel<WEIGHT, true>), dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0, st,
                           keys, segs, starts, n_unique, pos, pos_shift, g, W, d, grad_out, long_min);
    else
        hipLaunchKernelGGL((seg_walk_kernel<WEIGHT, false>), dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0, st,
                           keys, segs, starts, n_unique, pos, pos_shift, g, W, d, grad_out, long_min);
    hipLaunchKernelGGL((long_walk_kernel<WEIGHT>), dim3(64, static_cast<unsigned>((d + 63) / 64)), dim3(64), 0, st,
                       longs, nlong, starts, pos, pos_shift, g, W, d, grad_out);
    return hip_status("gradient launch");
}

void cap_for_host(Shape& sh, const ngram_table* T, const ngram_launch* L) {
    if (T->location == NGRAM_IN_HOST && sh.grid > host_workgroups(L)) {
        sh.grid = host_workgroups(L);
        sh.persist = true;
    }
}

int check_launch(const ngram_launch* L) {
    if (L && (L->tokens_per_workgroup < 0 || L->tokens_per_workgroup > 64 || L->host_workgroups < 0 ||
              L->host_workgroups > 65536))
        return fail(NGRAM_EINVAL, "launch: tokens_per_workgroup must be in [0, 64], host_workgroups in [0, 65536]");
    return NGRAM_OK;
}

template <int DT, bool E1, bool RES>
void launch_fwd(const FwdArgs& a, const Shape& sh, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(sh.grid));
    const dim3 block(64 * sh.waves);
    const size_t lds = static_cast<size_t>(sh.tpw) * (kK + 1) * sizeof(int32_t) +
                       (a.stage ? kSeqLds * sizeof(int32_t) : 0);
    if constexpr (DT == NGRAM_TABLE_INT8_ROWSCALE) {
        if (a.d % kSlice == 0) {
            if (sh.persist) hipLaunchKernelGGL((ngram_fwd_kernel<DT, E1, RES, true, true>), grid, block, lds, st, a);
            else hipLaunchKernelGGL((ngram_fwd_kernel<DT, E1, RES, false, true>), grid, block, lds, st, a);
            return;
        }
    }
    if (sh.persist) hipLaunchKernelGGL((ngram_fwd_kernel<DT, E1, RES, true, false>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((ngram_fwd_kernel<DT, E1, RES, false, false>), grid, block, lds, st, a);
}

template <int DT>
void launch_fwd_dt(const FwdArgs& a, const Shape& sh, hipStream_t st) {
    const bool e1 = a.e1 != nullptr, res = a.res != nullptr;
    if (e1 && res) launch_fwd<DT, true, true>(a, sh, st);
    else if (e1) launch_fwd<DT, true, false>(a, sh, st);
    else if (res) launch_fwd<DT, false, true>(a, sh, st);
    else launch_fwd<DT, false, false>(a, sh, st);
}

// The gated kernel: one wavefront per 512-column block (d <= 8192).
template <int DT, bool RES, int MODE>
void launch_gated_mode(const GatedArgs& g, dim3 grid, dim3 block, size_t lds, bool full, hipStream_t st) {
    if constexpr (MODE == 0 || MODE == 3) {
        if (full) hipLaunchKernelGGL((ngram_gated_kernel<DT, RES, MODE>), grid, block, lds, st, g);
        else hipLaunchKernelGGL((ngram_gated_any_kernel<DT, RES, false, MODE>), grid, block, lds, st, g);
    } else {
        if (full) hipLaunchKernelGGL((ngram_gated_any_kernel<DT, RES, true, MODE>), grid, block, lds, st, g);
        else hipLaunchKernelGGL((ngram_gated_any_kernel<DT, RES, false, MODE>), grid, block, lds, st, g);
    }
}

template <int DT>
void launch_gated_dt(const GatedArgs& g, const Shape& sh, hipStream_t st) {
    const int nb = (g.f.d + kSlice - 1) / kSlice;
    const dim3 grid(static_cast<unsigned>(sh.grid)), block(64 * nb);
    const size_t lds = static_cast<size_t>(sh.tpw) * ((kK + 1) * sizeof(int32_t) + 2 * nb * sizeof(double)) +
                       (g.f.stage ? kSeqLds * sizeof(int32_t) : 0);
    const bool res = g.f.res != nullptr, full = g.f.d % kSlice == 0;
    if (sh.persist) {
        if (res) launch_gated_mode<DT, true, 2>(g, grid, block, lds, false, st);
        else launch_gated_mode<DT, false, 2>(g, grid, block, lds, false, st);
    } else if (sh.tpw == 1) {
        if (res) launch_gated_mode<DT, true, 0>(g, grid, block, lds, full, st);
        else launch_gated_mode<DT, false, 0>(g, grid, block, lds, full, st);
    } else {
        if (res) launch_gated_mode<DT, true, 1>(g, grid, block, lds, full, st);
        else launch_gated_mode<DT, false, 1>(g, grid, block, lds, full, st);
    }
}


// The gate gradient's two launches, given the float64 partials buffer
// (nchunks x d doubles).
void launch_gate_grad(const int32_t* rows, const uint16_t* dout, const float* eN, int64_t n, int32_t d,
                      float* grad_Wg_out, double* parts, hipStream_t stream) {
    const int64_t nchunks = (n + kGateChunk - 1) / kGateChunk;
    if (nchunks > 0) {
        // at most kGateGrid workgroups, each taking an equal share of the
        // items, so the kernel leaves room on every compute unit for work
        // on other streams (the sort of the table gradient)
        const int colblocks = (d / kGateCols + 63) / 64;
        const int64_t items = nchunks * colblocks;
        const int64_t per = (items + kGateGrid - 1) / kGateGrid;
        const int64_t grid = (items + per - 1) / per;
        hipLaunchKernelGGL(gate_grad_partial_kernel, dim3(static_cast<unsigned>(grid)), dim3(64 * kGateWaves), 0,
                           stream, rows, dout, eN, n, d, nchunks, colblocks, parts);
    }
    hipLaunchKernelGGL(gate_grad_total_kernel, dim3(static_cast<unsigned>((d + 63) / 64)), dim3(64 * kGateTotalWaves),
                       0, stream, parts, nchunks, d, grad_Wg_out);
}

// Scratch of the allocation-free gate gradient: the float64 chunk partials
// live in this file-scope device array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands for the symbol): it passes the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr int64_t kNoAllocScratchBytes = int64_t{16} << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// each device, with that device current).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NGRAM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(NGRAM_ENOTSUP, "device %d above the supported %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(NGRAM_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NGRAM_OK;
}

// ngram_embed_bag and ngram_embed_bag_bf16: the sums to fp32 or to bf16.
template <bool OUT16>
void launch_bag(const BagArgs& a, int32_t dtype, bool persist, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
    if (dtype == NGRAM_TABLE_BF16) {
        if (persist) hipLaunchKernelGGL((ngram_bag_kernel<NGRAM_TABLE_BF16, true, OUT16>), grid, block, lds, st, a);
        else hipLaunchKernelGGL((ngram_bag_kernel<NGRAM_TABLE_BF16, false, OUT16>), grid, block, lds, st, a);
    } else if (dtype == NGRAM_TABLE_INT8_ROWSCALE) {
        constexpr int I8 = NGRAM_TABLE_INT8_ROWSCALE;
        if (a.d % kSlice == 0) {
            if (persist) hipLaunchKernelGGL((ngram_bag_kernel<I8, true, OUT16, true>), grid, block, lds, st, a);
            else hipLaunchKernelGGL((ngram_bag_kernel<I8, false, OUT16, true>), grid, block, lds, st, a);
        } else {
            if (persist) hipLaunchKernelGGL((ngram_bag_kernel<I8, true, OUT16>), grid, block, lds, st, a);
            else hipLaunchKernelGGL((ngram_bag_kernel<I8, false, OUT16>), grid, block, lds, st, a);
        }
    } else {
        if (persist) hipLaunchKernelGGL((ngram_bag_kernel<NGRAM_TABLE_MXFP4, true, OUT16>), grid, block, lds, st, a);
        else hipLaunchKernelGGL((ngram_bag_kernel<NGRAM_TABLE_MXFP4, false, OUT16>), grid, block, lds, st, a);
    }
}

int embed_bag_any(const ngram_table* T, const int32_t* rows, int64_t n, float* eN_out, uint16_t* eN16_out,
                  const ngram_launch* launch, ngram_stream_t stream) {
    int rc = check_table(T);
    if (rc) return rc;
    rc = check_launch(launch);
    if (rc) return rc;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > INT32_MAX) return fail(NGRAM_ERANGE, "n=%lld above 2^31-1", (long long)n);
    if (n > 0 && !rows) return fail(NGRAM_EINVAL, "rows is NULL");
    if (n > 0 && !aligned(eN_out ? static_cast<const void*>(eN_out) : eN16_out, 16))
        return fail(NGRAM_EALIGN, "output not 16-byte aligned");
    if (n == 0) return NGRAM_OK;
    const void* tab = nullptr;
    rc = table_device_ptr(T, &tab);
    if (rc) return rc;
    BagArgs a;
    a.tab = tab; a.scale = T->row_scale; a.rows = rows; a.eN = eN_out; a.eN16 = eN16_out;
    a.n = n; a.R = T->R; a.d = T->d;
    Shape sh = slice_shape(n, T->d, T->dtype, launch);
    cap_for_host(sh, T, launch);
    a.tpw = sh.tpw;
    const dim3 grid(static_cast<unsigned>(sh.grid)), block(64 * sh.waves);
    // the row lists [tpw][16], then (fp32 output) 2 KiB per wavefront
    const size_t lds = static_cast<size_t>(sh.tpw) * kK * sizeof(int32_t) +
                       (eN16_out ? 0 : static_cast<size_t>(sh.waves) * kSlice * sizeof(float));
    if (eN16_out) launch_bag<true>(a, T->dtype, sh.persist, grid, block, lds, stream);
    else launch_bag<false>(a, T->dtype, sh.persist, grid, block, lds, stream);
    return hip_status("ngram_embed_bag launch");
}

}  // namespace

// ===========================================================================
extern "C" {

const char* ngram_status_string(int status) {
    switch (status) {
        case NGRAM_OK: return "NGRAM_OK";
        case NGRAM_EINVAL: return "NGRAM_EINVAL: invalid argument";
        case NGRAM_EALIGN: return "NGRAM_EALIGN: misaligned pointer";
        case NGRAM_ERANGE: return "NGRAM_ERANGE: size out of range";
        case NGRAM_EHIP: return "NGRAM_EHIP: HIP runtime error";
        case NGRAM_ENOTSUP: return "NGRAM_ENOTSUP: not supported";
        default: return "unknown ngram status";
    }
}

const char* ngram_last_error(void) { return g_err; }

int ngram_version(void) { return 1; }

void ngram_default_seeds(uint64_t seeds[NGRAM_K]) {
    const Seeds s = make_seeds(nullptr);
    for (int k = 0; k < kK; ++k) seeds[k] = s.s[k];
}

int ngram_hash(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
               const int32_t* history, const uint64_t* seeds, int64_t R, int32_t* rows_out,
               ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_tokens(tokens, n, seq_offsets, S);
    if (rc) return rc;
    if (R < 1 || R > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "R=%lld outside [1, 2^31-1]", (long long)R);
    if (n > 0 && !rows_out) return fail(NGRAM_EINVAL, "rows_out is NULL");
    if (n == 0) return NGRAM_OK;
    HashArgs a;
    a.tok = tokens; a.so = seq_offsets; a.hist = history; a.rows_out = rows_out;
    a.n = n; a.R = static_cast<uint64_t>(R); a.S = S; a.c0_limit = kPad; a.stage = stage_for(n, S);
    a.sd = make_seeds(seeds);
    const int64_t total = n * kK;
    hipLaunchKernelGGL(ngram_hash_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                       stream, a);
    return hip_status("ngram_hash launch");
}

int ngram_embed_bag(const ngram_table* T, const int32_t* rows, int64_t n, float* eN_out,
                    ngram_stream_t stream) {
    return ngram_embed_bag_ex(T, rows, n, eN_out, nullptr, stream);
}

int ngram_embed_bag_ex(const ngram_table* T, const int32_t* rows, int64_t n, float* eN_out,
                       const ngram_launch* launch, ngram_stream_t stream) {
    g_err[0] = 0;
    if (n > 0 && !eN_out) return fail(NGRAM_EINVAL, "eN_out is NULL");
    return embed_bag_any(T, rows, n, eN_out, nullptr, launch, stream);
}

int ngram_embed_bag_bf16(const ngram_table* T, const int32_t* rows, int64_t n, uint16_t* out,
                         ngram_stream_t stream) {
    g_err[0] = 0;
    if (n > 0 && !out) return fail(NGRAM_EINVAL, "out is NULL");
    return embed_bag_any(T, rows, n, nullptr, out, nullptr, stream);
}


int ngram_gate_add(const float* eN, const int32_t* tokens, int64_t n, int32_t d,
                   const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                   uint16_t* out, ngram_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > INT32_MAX) return fail(NGRAM_ERANGE, "n=%lld above 2^31-1", (long long)n);
    if (d <= 0 || d % kVec != 0) return fail(NGRAM_EINVAL, "d=%d must be a positive multiple of 8", d);
    if (d > NGRAM_MAX_D) return fail(NGRAM_ERANGE, "d=%d above %d", d, NGRAM_MAX_D);
    if (!W_g) return fail(NGRAM_EINVAL, "W_g is NULL");
    if (e1 && V < 1) return fail(NGRAM_ERANGE, "V=%lld must be >= 1 with e1", (long long)V);
    if (n > 0 && (!eN || !tokens || !out)) return fail(NGRAM_EINVAL, "eN, tokens or out is NULL");
    if (!aligned(W_g, 16) || (e1 && !aligned(e1, 16)) || (residual && !aligned(residual, 16)) ||
        (n > 0 && (!aligned(eN, 16) || !aligned(out, 16))))
        return fail(NGRAM_EALIGN, "eN, e1, W_g, residual and out must be 16-byte aligned");
    if (n == 0) return NGRAM_OK;
    GateArgs a;
    a.eN = eN; a.tok = tokens; a.e1 = e1; a.wg = W_g; a.res = residual; a.out = out;
    a.n = n; a.d = d; a.c0_limit = c0_limit_for(e1, V);
    const int64_t total = n * (d / kVec);
    const dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
    if (e1 && residual) hipLaunchKernelGGL((ngram_gate_kernel<true, true>), grid, block, 0, stream, a);
    else if (e1) hipLaunchKernelGGL((ngram_gate_kernel<true, false>), grid, block, 0, stream, a);
    else if (residual) hipLaunchKernelGGL((ngram_gate_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((ngram_gate_kernel<false, false>), grid, block, 0, stream, a);
    return hip_status("ngram_gate_add launch");
}

int ngram_project(const uint16_t* x, int64_t n, int32_t d_in, const uint16_t* P, int32_t d_out, float* y,
                  ngram_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (d_in <= 0 || d_in % kPK != 0 || d_out <= 0 || d_out % kVec != 0)
        return fail(NGRAM_EINVAL, "d_in=%d must be a positive multiple of %d and d_out=%d of %d", d_in, kPK, d_out, kVec);
    if (d_in > NGRAM_MAX_D || d_out > NGRAM_MAX_D)
        return fail(NGRAM_ERANGE, "d_in=%d or d_out=%d above %d", d_in, d_out, NGRAM_MAX_D);
    if (!P) return fail(NGRAM_EINVAL, "P is NULL");
    if (n > 0 && (!x || !y)) return fail(NGRAM_EINVAL, "x or y is NULL");
    if (!aligned(P, 16) || (n > 0 && (!aligned(x, 16) || !aligned(y, 16))))
        return fail(NGRAM_EALIGN, "x, P and y must be 16-byte aligned");
    const int64_t mtiles = (n + kPM - 1) / kPM, ntiles = (d_out + kPN - 1) / kPN;
    if (mtiles * ntiles > INT32_MAX / 2) return fail(NGRAM_ERANGE, "n=%lld too large for one launch", (long long)n);
    if (n == 0) return NGRAM_OK;
    ProjArgs a;
    a.x = x; a.P = P; a.y = y; a.n = n; a.K = d_in; a.N = d_out; a.ntiles_n = static_cast<int32_t>(ntiles);
    a.ntiles = static_cast<int32_t>(mtiles * ntiles);
    // 8 * ceil(tiles / 8) workgroups: the XCD-aware order gives every XCD a
    // run of tiles, and the workgroups beyond a short run exit at once
    const int64_t grid = 8 * ((a.ntiles + 7) / 8);
    hipLaunchKernelGGL(project_kernel, dim3(static_cast<unsigned>(grid)), dim3(kPThreads), 2 * kPStage, stream, a);
    return hip_status("ngram_project launch");
}

int ngram_norm_gate_add(const float* eN, const int32_t* tokens, int64_t n, int32_t d, const uint16_t* e1,
                        int64_t V, const float* W_g, const float* gamma, const float* u, const float* v, float b,
                        float eps, const uint16_t* residual, uint16_t* out, double* stats_out,
                        ngram_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > INT32_MAX) return fail(NGRAM_ERANGE, "n=%lld above 2^31-1", (long long)n);
    if (d <= 0 || d % kVec != 0) return fail(NGRAM_EINVAL, "d=%d must be a positive multiple of 8", d);
    if (d > 16 * kSlice) return fail(NGRAM_ERANGE, "d=%d above %d for the gated path", d, 16 * kSlice);
    if (!W_g || !gamma || !u || !v || !e1) return fail(NGRAM_EINVAL, "W_g, gamma, u, v or e1 is NULL");
    if (V < 1) return fail(NGRAM_ERANGE, "V=%lld must be >= 1", (long long)V);
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(b))
        return fail(NGRAM_EINVAL, "eps must be finite and >= 0, b finite");
    if (n > 0 && (!eN || !tokens || !out)) return fail(NGRAM_EINVAL, "eN, tokens or out is NULL");
    if (!aligned(W_g, 16) || !aligned(gamma, 16) || !aligned(u, 16) || !aligned(v, 16) || !aligned(e1, 16) ||
        (residual && !aligned(residual, 16)) || (n > 0 && (!aligned(out, 16) || !aligned(eN, 16))) ||
        (stats_out && !aligned(stats_out, 8)))
        return fail(NGRAM_EALIGN, "eN, e1, W_g, gamma, u, v, residual and out must be 16-byte aligned, stats_out 8");
    if (n == 0) return NGRAM_OK;
    GatedArgs g{};
    FwdArgs& a = g.f;
    a.tok = tokens; a.e1 = e1; a.wg = W_g; a.res = residual; a.out = out;
    a.n = n; a.d = d; a.tpw = 1;
    a.c0_limit = c0_limit_for(e1, V);
    g.eN = eN; g.gamma = gamma; g.u = u; g.v = v; g.stats = stats_out; g.b = b; g.eps = eps;
    const int nb = (d + kSlice - 1) / kSlice;
    const dim3 grid(static_cast<unsigned>(n)), block(64 * nb);
    const size_t lds = 2 * nb * sizeof(double) + (kK + 1) * sizeof(int32_t);
    const bool full = d % kSlice == 0;
    if (residual) launch_gated_mode<NGRAM_TABLE_BF16, true, 3>(g, grid, block, lds, full, stream);
    else launch_gated_mode<NGRAM_TABLE_BF16, false, 3>(g, grid, block, lds, full, stream);
    return hip_status("ngram_norm_gate_add launch");
}

int ngram_forward(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                  const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                  const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                  uint16_t* out, int32_t* rows_out, ngram_stream_t stream) {
    return ngram_forward_ex(tokens, n, seq_offsets, S, history, seeds, T, e1, V, W_g, residual, out, rows_out,
                            nullptr, stream);
}

int ngram_forward_ex(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                     const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                     const uint16_t* e1, int64_t V, const float* W_g, const uint16_t* residual,
                     uint16_t* out, int32_t* rows_out, const ngram_launch* launch, ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_tokens(tokens, n, seq_offsets, S);
    if (rc) return rc;
    rc = check_launch(launch);
    if (rc) return rc;
    rc = check_table(T);
    if (rc) return rc;
    if (!W_g) return fail(NGRAM_EINVAL, "W_g is NULL");
    if (e1 && V < 1) return fail(NGRAM_ERANGE, "V=%lld must be >= 1 with e1", (long long)V);
    if (n > 0 && !out) return fail(NGRAM_EINVAL, "out is NULL");
    if (!aligned(W_g, 16) || (e1 && !aligned(e1, 16)) || (residual && !aligned(residual, 16)) ||
        (n > 0 && !aligned(out, 16)))
        return fail(NGRAM_EALIGN, "e1, W_g, residual and out must be 16-byte aligned");
    if (n == 0) return NGRAM_OK;
    const void* tab = nullptr;
    rc = table_device_ptr(T, &tab);
    if (rc) return rc;
    FwdArgs a;
    a.tok = tokens; a.so = seq_offsets; a.hist = history; a.tab = tab; a.scale = T->row_scale;
    a.e1 = e1; a.wg = W_g; a.res = residual; a.out = out; a.rows_out = rows_out;
    a.n = n; a.R = static_cast<uint64_t>(T->R); a.S = S; a.d = T->d;
    a.c0_limit = c0_limit_for(e1, V);
    a.stage = stage_for(n, S);
    a.sd = make_seeds(seeds);
    Shape sh = slice_shape(n, T->d, T->dtype, launch);
    cap_for_host(sh, T, launch);
    a.tpw = sh.tpw;
    if (T->dtype == NGRAM_TABLE_BF16) launch_fwd_dt<NGRAM_TABLE_BF16>(a, sh, stream);
    else if (T->dtype == NGRAM_TABLE_INT8_ROWSCALE) launch_fwd_dt<NGRAM_TABLE_INT8_ROWSCALE>(a, sh, stream);
    else launch_fwd_dt<NGRAM_TABLE_MXFP4>(a, sh, stream);
    return hip_status("ngram_forward launch");
}

int ngram_forward_gated(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                        const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                        const uint16_t* e1, int64_t V, const float* W_g, const float* gamma, const float* u,
                        const float* v, float b, float eps, const uint16_t* residual, uint16_t* out,
                        int32_t* rows_out, double* stats_out, ngram_stream_t stream) {
    return ngram_forward_gated_ex(tokens, n, seq_offsets, S, history, seeds, T, e1, V, W_g, gamma, u, v, b, eps,
                                  residual, out, rows_out, stats_out, nullptr, stream);
}

int ngram_forward_gated_ex(const int32_t* tokens, int64_t n, const int32_t* seq_offsets, int32_t S,
                           const int32_t* history, const uint64_t* seeds, const ngram_table* T,
                           const uint16_t* e1, int64_t V, const float* W_g, const float* gamma, const float* u,
                           const float* v, float b, float eps, const uint16_t* residual, uint16_t* out,
                           int32_t* rows_out, double* stats_out, const ngram_launch* launch,
                           ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_tokens(tokens, n, seq_offsets, S);
    if (rc) return rc;
    rc = check_launch(launch);
    if (rc) return rc;
    rc = check_table(T);
    if (rc) return rc;
    if (T->d > 16 * kSlice) return fail(NGRAM_ERANGE, "d=%d above %d for the gated path", T->d, 16 * kSlice);
    if (!W_g || !gamma || !u || !v || !e1) return fail(NGRAM_EINVAL, "W_g, gamma, u, v or e1 is NULL");
    if (V < 1) return fail(NGRAM_ERANGE, "V=%lld must be >= 1", (long long)V);
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(b))
        return fail(NGRAM_EINVAL, "eps must be finite and >= 0, b finite");
    if (n > 0 && !out) return fail(NGRAM_EINVAL, "out is NULL");
    if (!aligned(W_g, 16) || !aligned(gamma, 16) || !aligned(u, 16) || !aligned(v, 16) || !aligned(e1, 16) ||
        (residual && !aligned(residual, 16)) || (n > 0 && !aligned(out, 16)) || (stats_out && !aligned(stats_out, 8)))
        return fail(NGRAM_EALIGN, "e1, W_g, gamma, u, v, residual and out must be 16-byte aligned, stats_out 8");
    if (n == 0) return NGRAM_OK;
    const void* tab = nullptr;
    rc = table_device_ptr(T, &tab);
    if (rc) return rc;
    GatedArgs g;
    FwdArgs& a = g.f;
    a.tok = tokens; a.so = seq_offsets; a.hist = history; a.tab = tab; a.scale = T->row_scale;
    a.e1 = e1; a.wg = W_g; a.res = residual; a.out = out; a.rows_out = rows_out;
    a.n = n; a.R = static_cast<uint64_t>(T->R); a.S = S; a.d = T->d;
    a.c0_limit = c0_limit_for(e1, V);
    a.stage = stage_for(n, S);
    a.sd = make_seeds(seeds);
    g.eN = nullptr;
    g.gamma = gamma; g.u = u; g.v = v; g.stats = stats_out; g.b = b; g.eps = eps;
    // One token per workgroup for every table type (the kernel then has no
    // token loop, which keeps it at 69-78 VGPRs instead of 113-128).
    Shape sh = slice_shape(n, T->d, T->dtype, launch);
    if (!(launch && launch->tokens_per_workgroup > 0)) {
        sh.tpw = 1;
        sh.grid = n;
    }
    cap_for_host(sh, T, launch);
    a.tpw = sh.tpw;
    if (T->dtype == NGRAM_TABLE_BF16) launch_gated_dt<NGRAM_TABLE_BF16>(g, sh, stream);
    else if (T->dtype == NGRAM_TABLE_INT8_ROWSCALE) launch_gated_dt<NGRAM_TABLE_INT8_ROWSCALE>(g, sh, stream);
    else launch_gated_dt<NGRAM_TABLE_MXFP4>(g, sh, stream);
    return hip_status("ngram_forward_gated launch");
}

int ngram_host_alloc(int64_t bytes, void** host_ptr) {
    g_err[0] = 0;
    if (!host_ptr) return fail(NGRAM_EINVAL, "host_ptr is NULL");
    *host_ptr = nullptr;
    if (bytes <= 0) return fail(NGRAM_EINVAL, "bytes=%lld must be positive", (long long)bytes);
    void* p = nullptr;
    const hipError_t e = hipHostMalloc(&p, static_cast<size_t>(bytes), hipHostMallocMapped | hipHostMallocNonCoherent);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NGRAM_EHIP, "hipHostMalloc(%lld): %s", (long long)bytes, hipGetErrorString(e));
    }
    *host_ptr = p;
    return NGRAM_OK;
}

int ngram_host_free(void* host_ptr) {
    g_err[0] = 0;
    if (!host_ptr) return NGRAM_OK;
    const hipError_t e = hipHostFree(host_ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NGRAM_EHIP, "hipHostFree: %s", hipGetErrorString(e));
    }
    return NGRAM_OK;
}

int64_t ngram_gather_host_workspace_bytes(int64_t n, int32_t d) {
    if (n < 0 || d <= 0) return -1;
    return pool_layout(n).total;
}

int64_t ngram_gather_host_pinned_bytes(int64_t n) {
    if (n < 0) return -1;
    return 16 + 4 * kK * n;
}

int ngram_gather_host(const ngram_table* T_host, const int32_t* rows, int64_t n, void* workspace,
                      int64_t workspace_bytes, void* pinned, int64_t pinned_bytes, void* stage_out,
                      float* stage_scale_out, int32_t* remap_out, int64_t* n_staged_out, int32_t mode,
                      ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_table(T_host);
    if (rc) return rc;
    if (T_host->location != NGRAM_IN_HOST) return fail(NGRAM_ENOTSUP, "ngram_gather_host needs a host table");
    if (mode != 0 && mode != 1) return fail(NGRAM_EINVAL, "mode=%d must be 0 (zero copy) or 1 (async copy)", mode);
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > (1 << 26)) return fail(NGRAM_ERANGE, "n=%lld above 2^26", (long long)n);
    if (n > 0 && (!rows || !stage_out || !remap_out || !n_staged_out))
        return fail(NGRAM_EINVAL, "rows, stage_out, remap_out or n_staged_out is NULL");
    if (n > 0 && T_host->dtype == NGRAM_TABLE_INT8_ROWSCALE && !stage_scale_out)
        return fail(NGRAM_EINVAL, "int8 table needs stage_scale_out");
    if (n > 0 && !aligned(stage_out, 16)) return fail(NGRAM_EALIGN, "stage_out not 16-byte aligned");
    const PoolLayout L = pool_layout(n);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)
        return fail(NGRAM_EINVAL, "workspace needs %lld bytes, 16-byte aligned", (long long)L.total);
    const int64_t nrows = kK * n;
    const int64_t pinned_need = ngram_gather_host_pinned_bytes(n);
    if (mode == 1 && (!pinned || !aligned(pinned, 16) || pinned_bytes < pinned_need))
        return fail(NGRAM_EINVAL, "mode 1 needs %lld bytes of pinned host memory, 16-byte aligned",
                    (long long)pinned_need);
    if (n == 0) return NGRAM_OK;
    const void* tab = nullptr;
    rc = table_device_ptr(T_host, &tab);
    if (rc) return rc;
    char* ws = static_cast<char*>(workspace);
    PoolArgs a;
    a.tab = tab; a.scale = T_host->row_scale; a.rows = rows; a.pool = stage_out;
    a.pool_scale = T_host->dtype == NGRAM_TABLE_INT8_ROWSCALE ? stage_scale_out : nullptr;
    a.slot_of_row = nullptr; a.pool_rows_out = remap_out;
    a.keys = reinterpret_cast<int32_t*>(ws + L.keys);
    a.vals = reinterpret_cast<int32_t*>(ws + L.vals);
    a.miss = reinterpret_cast<int32_t*>(ws + L.miss);
    a.counter = reinterpret_cast<uint32_t*>(ws + L.counter);
    a.fetched_out = n_staged_out;
    a.nrows = nrows; a.R = T_host->R; a.cached = 0; a.row_bytes = table_row_bytes(T_host);
    a.mask = static_cast<uint32_t>(L.H - 1);
    a.shift = 32u - static_cast<uint32_t>(L.log2H);
    // distinct rows: keys := -1, counter := 0, insert, then resolve to staging indices
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(L.H)), dim3(256), 0, stream, a.keys, L.H, -1);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, stream, reinterpret_cast<int32_t*>(a.counter), 4, 0);
    const dim3 g(static_cast<unsigned>((nrows + 255) / 256)), b(256);
    hipLaunchKernelGGL(pool_insert_kernel, g, b, 0, stream, a);
    hipLaunchKernelGGL(pool_resolve_kernel, g, b, 0, stream, a);
    if (mode == 0) {
        int64_t blocks = (nrows + 15) / 16;
        if (blocks > kHostWorkgroups) blocks = kHostWorkgroups;
        if (a.row_bytes % 16 == 0) hipLaunchKernelGGL(pool_fetch_kernel<u32x4>, dim3(blocks), dim3(1024), 0, stream, a);
        else if (a.row_bytes % 8 == 0) hipLaunchKernelGGL(pool_fetch_kernel<u32x2>, dim3(blocks), dim3(1024), 0, stream, a);
        else hipLaunchKernelGGL(pool_fetch_kernel<uint32_t>, dim3(blocks), dim3(1024), 0, stream, a);
        return hip_status("ngram_gather_host launch");
    }
    // mode 1: read the distinct-row list back, then enqueue one host-to-device
    // copy per row on the stream (the DMA engines; no compute units)
    hipLaunchKernelGGL(stage_meta_kernel, g, b, 0, stream, a);
    rc = hip_status("ngram_gather_host launch");
    if (rc) return rc;
    char* hp = static_cast<char*>(pinned);
    uint32_t* h_count = reinterpret_cast<uint32_t*>(hp);
    int32_t* h_miss = reinterpret_cast<int32_t*>(hp + 16);
    hipError_t e = hipMemcpyAsync(h_count, a.counter, 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h_miss, a.miss, 4 * nrows, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NGRAM_EHIP, "reading the distinct-row list: %s", hipGetErrorString(e));
    }
    const int64_t U = *h_count;
    const char* host_tab = static_cast<const char*>(T_host->data);
    char* stage = static_cast<char*>(stage_out);
    for (int64_t u = 0; u < U; ++u) {
        e = hipMemcpyAsync(stage + u * a.row_bytes, host_tab + static_cast<int64_t>(h_miss[u]) * a.row_bytes,
                           static_cast<size_t>(a.row_bytes), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(NGRAM_EHIP, "copy of row %lld of %lld: %s", (long long)u, (long long)U, hipGetErrorString(e));
        }
    }
    return NGRAM_OK;
}

int64_t ngram_pool_workspace_bytes(int64_t n) {
    if (n < 0) return -1;
    return pool_layout(n).total;
}

int ngram_pool_reset(const ngram_table* T_host, ngram_row_pool* P, ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_table(T_host);
    if (rc) return rc;
    if (!P || !P->slot_of_row) return fail(NGRAM_EINVAL, "pool or slot_of_row is NULL");
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(T_host->R)), dim3(256), 0, stream, P->slot_of_row, T_host->R, -1);
    rc = hip_status("ngram_pool_reset launch");
    if (!rc) P->cached = 0;
    return rc;
}

int ngram_pool_cache_rows(const ngram_table* T_host, ngram_row_pool* P, const int32_t* hot_rows, int64_t C,
                          ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_pool(T_host, P);
    if (rc) return rc;
    if (C < 0 || C > P->pool_rows) return fail(NGRAM_ERANGE, "C=%lld outside [0, pool_rows]", (long long)C);
    if (C > 0 && !hot_rows) return fail(NGRAM_EINVAL, "hot_rows is NULL");
    const void* tab = nullptr;
    rc = table_device_ptr(T_host, &tab);
    if (rc) return rc;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(T_host->R)), dim3(256), 0, stream, P->slot_of_row, T_host->R, -1);
    if (C > 0) {
        const int64_t row_bytes = table_row_bytes(T_host);
        int64_t blocks = (C + 15) / 16;
        if (blocks > kHostWorkgroups) blocks = kHostWorkgroups;
        float* pscale = T_host->dtype == NGRAM_TABLE_INT8_ROWSCALE ? P->row_scale : nullptr;
        if (row_bytes % 16 == 0)
            hipLaunchKernelGGL(pool_cache_kernel<u32x4>, dim3(blocks), dim3(1024), 0, stream, tab, T_host->row_scale,
                               hot_rows, C, T_host->R, P->data, pscale, P->slot_of_row, row_bytes);
        else if (row_bytes % 8 == 0)
            hipLaunchKernelGGL(pool_cache_kernel<u32x2>, dim3(blocks), dim3(1024), 0, stream, tab, T_host->row_scale,
                               hot_rows, C, T_host->R, P->data, pscale, P->slot_of_row, row_bytes);
        else
            hipLaunchKernelGGL(pool_cache_kernel<uint32_t>, dim3(blocks), dim3(1024), 0, stream, tab,
                               T_host->row_scale, hot_rows, C, T_host->R, P->data, pscale, P->slot_of_row, row_bytes);
    }
    rc = hip_status("ngram_pool_cache_rows launch");
    if (!rc) P->cached = C;
    return rc;
}

int ngram_pool_gather(const ngram_table* T_host, const ngram_row_pool* P, const int32_t* rows, int64_t n,
                      int32_t* pool_rows_out, int64_t* fetched_out, void* workspace, int64_t workspace_bytes,
                      ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_pool(T_host, P);
    if (rc) return rc;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > (1 << 26)) return fail(NGRAM_ERANGE, "n=%lld above 2^26", (long long)n);
    if (P->cached < 0 || P->pool_rows < P->cached + kK * n)
        return fail(NGRAM_ERANGE, "pool_rows=%lld < cached %lld + 16 n", (long long)P->pool_rows, (long long)P->cached);
    if (n > 0 && (!rows || !pool_rows_out)) return fail(NGRAM_EINVAL, "rows or pool_rows_out is NULL");
    const PoolLayout L = pool_layout(n);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < L.total)
        return fail(NGRAM_EINVAL, "workspace needs %lld bytes, 16-byte aligned", (long long)L.total);
    if (n == 0) return NGRAM_OK;
    const void* tab = nullptr;
    rc = table_device_ptr(T_host, &tab);
    if (rc) return rc;
    char* ws = static_cast<char*>(workspace);
    PoolArgs a;
    a.tab = tab; a.scale = T_host->row_scale; a.rows = rows; a.pool = P->data;
    a.pool_scale = T_host->dtype == NGRAM_TABLE_INT8_ROWSCALE ? P->row_scale : nullptr;
    a.slot_of_row = P->slot_of_row; a.pool_rows_out = pool_rows_out;
    a.keys = reinterpret_cast<int32_t*>(ws + L.keys);
    a.vals = reinterpret_cast<int32_t*>(ws + L.vals);
    a.miss = reinterpret_cast<int32_t*>(ws + L.miss);
    a.counter = reinterpret_cast<uint32_t*>(ws + L.counter);
    a.fetched_out = fetched_out;
    a.nrows = n * kK; a.R = T_host->R; a.cached = P->cached; a.row_bytes = table_row_bytes(T_host);
    a.mask = static_cast<uint32_t>(L.H - 1);
    a.shift = 32u - static_cast<uint32_t>(L.log2H);
    // keys := -1 and counter := 0 with one fill (the counter word follows the keys' region)
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(L.H)), dim3(256), 0, stream, a.keys, L.H, -1);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, stream, reinterpret_cast<int32_t*>(a.counter), 4, 0);
    const dim3 g(static_cast<unsigned>((a.nrows + 255) / 256)), b(256);
    hipLaunchKernelGGL(pool_insert_kernel, g, b, 0, stream, a);
    hipLaunchKernelGGL(pool_resolve_kernel, g, b, 0, stream, a);
    int64_t blocks = (a.nrows + 15) / 16;
    if (blocks > kHostWorkgroups) blocks = kHostWorkgroups;
    if (a.row_bytes % 16 == 0) hipLaunchKernelGGL(pool_fetch_kernel<u32x4>, dim3(blocks), dim3(1024), 0, stream, a);
    else if (a.row_bytes % 8 == 0) hipLaunchKernelGGL(pool_fetch_kernel<u32x2>, dim3(blocks), dim3(1024), 0, stream, a);
    else hipLaunchKernelGGL(pool_fetch_kernel<uint32_t>, dim3(blocks), dim3(1024), 0, stream, a);
    return hip_status("ngram_pool_gather launch");
}

int ngram_count_rows(const int32_t* rows, int64_t n, int64_t R, int32_t* counts, int32_t accumulate,
                     ngram_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > INT32_MAX / kK) return fail(NGRAM_ERANGE, "n=%lld above (2^31-1)/16", (long long)n);
    if (R < 1 || R > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "R=%lld outside [1, 2^31-1]", (long long)R);
    if (!counts || (n > 0 && !rows)) return fail(NGRAM_EINVAL, "counts or rows is NULL");
    if (!accumulate) hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(R)), dim3(256), 0, stream, counts, R, 0);
    if (n > 0)
        hipLaunchKernelGGL(count_rows_kernel, dim3(static_cast<unsigned>((n * kK + 255) / 256)), dim3(256), 0, stream,
                           rows, n * kK, R, counts);
    return hip_status("ngram_count_rows launch");
}

int ngram_select_hot_rows(const int32_t* counts, int64_t R, int64_t C, int32_t* hot_rows_out, int64_t* selected,
                          void* workspace, int64_t workspace_bytes, ngram_stream_t stream) {
    g_err[0] = 0;
    if (R < 1 || R > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "R=%lld outside [1, 2^31-1]", (long long)R);
    if (C < 0 || C > INT32_MAX) return fail(NGRAM_ERANGE, "C=%lld outside [0, 2^31-1]", (long long)C);
    if (!counts || !selected || (C > 0 && !hot_rows_out)) return fail(NGRAM_EINVAL, "counts, hot_rows_out or selected is NULL");
    const int64_t need = pool_layout(0).total;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
        return fail(NGRAM_EINVAL, "workspace needs %lld bytes, 16-byte aligned", (long long)need);
    *selected = 0;
    if (C == 0) return NGRAM_OK;
    int32_t* hist = static_cast<int32_t*>(workspace);
    uint32_t* sel = reinterpret_cast<uint32_t*>(hist + kHistBins);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(4), dim3(256), 0, stream, hist, kHistBins + 4, 0);
    hipLaunchKernelGGL(count_hist_kernel, dim3(grid_for(R)), dim3(256), 0, stream, counts, R, hist);
    int rc = hip_status("ngram_select_hot_rows launch");
    if (rc) return rc;
    int32_t h[kHistBins];
    hipError_t e = hipMemcpyAsync(h, hist, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(NGRAM_EHIP, "reading the count histogram: %s", hipGetErrorString(e));
    // smallest threshold whose set {count >= tau} holds at most C rows
    int32_t tau = 1;
    int64_t cum = 0;
    for (int b = kHistBins - 1; b >= 1; --b) {
        if (cum + h[b] > C) {
            tau = b + 1;
            break;
        }
        cum += h[b];
    }
    if (tau > kHistBins - 1) tau = kHistBins - 1;    // the top value alone overflows C: take C of it
    hipLaunchKernelGGL(select_kernel, dim3(grid_for(R)), dim3(256), 0, stream, counts, R, tau, C, hot_rows_out, sel);
    rc = hip_status("ngram_select_hot_rows launch");
    if (rc) return rc;
    uint32_t got = 0;
    e = hipMemcpyAsync(&got, sel, sizeof(got), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(NGRAM_EHIP, "reading the selection count: %s", hipGetErrorString(e));
    *selected = got < static_cast<uint64_t>(C) ? static_cast<int64_t>(got) : C;
    return NGRAM_OK;
}

int64_t ngram_grad_workspace_bytes(int64_t n, int32_t d) {
    if (n < 0 || d <= 0) return -1;
    return grad_layout(n, d).total;
}

static int check_grad_common(int64_t n, int32_t d, const uint16_t* dout, void* workspace, int64_t workspace_bytes) {
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    // 32-bit item indices and counts throughout the sort and the walks; each
    // group-numbering workgroup adds the counts of all earlier tiles, so the
    // tested range 16 n <= 2^24 is also the accepted one
    if (n > (1 << 20)) return fail(NGRAM_ERANGE, "n=%lld above 2^20", (long long)n);
    if (d <= 0 || d % kVec != 0) return fail(NGRAM_EINVAL, "d=%d must be a positive multiple of 8", d);
    if (d > NGRAM_MAX_D) return fail(NGRAM_ERANGE, "d=%d above %d", d, NGRAM_MAX_D);
    if (n > 0 && (!dout || !aligned(dout, 16))) return fail(NGRAM_EINVAL, "dout is NULL or not 16-byte aligned");
    const int64_t need = grad_layout(n, d).total;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
        return fail(NGRAM_EINVAL, "workspace needs %lld bytes, 256-byte aligned", (long long)need);
    return NGRAM_OK;
}

int ngram_grad_table(const int32_t* rows, int64_t n, int32_t d, int64_t R, const float* W_g, const uint16_t* dout,
                     int32_t* grad_rows_out, float* grad_out, int64_t* n_unique_out, void* workspace,
                     int64_t workspace_bytes, ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_grad_common(n, d, dout, workspace, workspace_bytes);
    if (rc) return rc;
    if (R < 1 || R > NGRAM_MAX_ROWS) return fail(NGRAM_ERANGE, "R=%lld outside [1, 2^31-1]", (long long)R);
    if (!n_unique_out || !W_g || !aligned(W_g, 16)) return fail(NGRAM_EINVAL, "n_unique_out or W_g is NULL/misaligned");
    if (n > 0 && (!rows || !grad_rows_out || !grad_out || !aligned(grad_out, 16)))
        return fail(NGRAM_EINVAL, "rows, grad_rows_out or grad_out is NULL/misaligned");
    const GradLayout L = grad_layout(n, d);
    return grad_by_groups<true>(rows, kK * n, 0, nullptr, static_cast<uint32_t>(R), 4, dout, W_g, d, grad_rows_out,
                                grad_out, n_unique_out, workspace, L, kLongGroup, stream);
}

int ngram_grad_e1(const int32_t* tokens, const int32_t* rows, int64_t n, int32_t d, int64_t V, const uint16_t* dout,
                  int32_t* grad_tokens_out, float* grad_out, int64_t* n_unique_out, void* workspace,
                  int64_t workspace_bytes, ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_grad_common(n, d, dout, workspace, workspace_bytes);
    if (rc) return rc;
    if (V < 1 || V > static_cast<int64_t>(kPad)) return fail(NGRAM_ERANGE, "V=%lld outside [1, 2^21-1]", (long long)V);
    if (!n_unique_out) return fail(NGRAM_EINVAL, "n_unique_out is NULL");
    if (n > 0 && (!tokens || !rows || !grad_tokens_out || !grad_out || !aligned(grad_out, 16)))
        return fail(NGRAM_EINVAL, "tokens, rows, grad_tokens_out or grad_out is NULL/misaligned");
    const GradLayout L = grad_layout(n, d);
    return grad_by_groups<false>(tokens, n, kK, rows, static_cast<uint32_t>(V), 0, dout, nullptr, d, grad_tokens_out,
                                 grad_out, n_unique_out, workspace, L, kLongGroupE1, stream);
}

int ngram_grad_gate(const int32_t* rows, const uint16_t* dout, const float* eN, int64_t n, int32_t d,
                    float* grad_Wg_out, void* workspace, int64_t workspace_bytes, ngram_stream_t stream) {
    g_err[0] = 0;
    int rc = check_grad_common(n, d, dout, workspace, workspace_bytes);
    if (rc) return rc;
    if (!grad_Wg_out) return fail(NGRAM_EINVAL, "grad_Wg_out is NULL");
    if (n > 0 && (!rows || !eN || !aligned(eN, 16))) return fail(NGRAM_EINVAL, "rows or eN is NULL/misaligned");
    const GradLayout L = grad_layout(n, d);
    double* parts = reinterpret_cast<double*>(static_cast<char*>(workspace) + L.parts);
    launch_gate_grad(rows, dout, eN, n, d, grad_Wg_out, parts, stream);
    return hip_status("ngram_grad_gate launch");
}

int64_t ngram_grad_gate_noalloc_max_elements(void) { return kNoAllocScratchBytes / 8; }

int ngram_grad_gate_noalloc(const int32_t* rows, const uint16_t* dout, const float* eN, int64_t n, int32_t d,
                            float* grad_Wg_out, ngram_stream_t stream) {
    g_err[0] = 0;
    if (n < 0) return fail(NGRAM_EINVAL, "n=%lld is negative", (long long)n);
    if (n > (1 << 20)) return fail(NGRAM_ERANGE, "n=%lld above 2^20", (long long)n);
    if (d <= 0 || d % kVec != 0) return fail(NGRAM_EINVAL, "d=%d must be a positive multiple of 8", d);
    if (d > NGRAM_MAX_D) return fail(NGRAM_ERANGE, "d=%d above %d", d, NGRAM_MAX_D);
    if (!grad_Wg_out) return fail(NGRAM_EINVAL, "grad_Wg_out is NULL");
    if (n > 0 && (!rows || !dout || !aligned(dout, 16) || !eN || !aligned(eN, 16)))
        return fail(NGRAM_EINVAL, "rows, dout or eN is NULL or dout / eN not 16-byte aligned");
    const int64_t nchunks = (n + kGateChunk - 1) / kGateChunk;
    if (nchunks * static_cast<int64_t>(d) > kNoAllocScratchBytes / 8)
        return fail(NGRAM_ERANGE, "ceil(n/%d) * d = %lld partials exceed the %lld-double static scratch", kGateChunk,
                    (long long)(nchunks * d), (long long)(kNoAllocScratchBytes / 8));
    void* p = nullptr;
    int rc = scratch_address(&p);
    if (rc) return rc;
    launch_gate_grad(rows, dout, eN, n, d, grad_Wg_out, static_cast<double*>(p), stream);
    return hip_status("ngram_grad_gate_noalloc launch");
}

}  // extern "C"
