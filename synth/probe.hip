// Measurement probes for the benchmark (libprobe.so), not part of the n-gram
// path: a bare random-row gather that shows what the memory system delivers
// for a given row size and load width, with no arithmetic and no writes; and
// the same gather with a token's other streams beside it (a row of a
// token-indexed table, a residual row read and an output row written), the
// byte mix of the fused forward without its arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int LB> struct Word;
template <> struct Word<4> { using T = uint32_t; __device__ static uint32_t fold(T v) { return v; } };
template <> struct Word<8> { using T = uint2; __device__ static uint32_t fold(T v) { return v.x ^ v.y; } };
template <> struct Word<16> { using T = uint4; __device__ static uint32_t fold(T v) { return v.x ^ v.y ^ v.z ^ v.w; } };

// Token i (workgroup i) reads its 16 rows rows[16 i .. 16 i + 15] of
// row_bytes bytes each, LB bytes per lane: thread t covers byte offset t * LB
// of every row (the launch has row_bytes / LB threads, rounded up to whole
// wavefronts).  The 16 loads of a thread are issued before they are folded;
// the fold is written only if it equals `never`, so the traffic is the rows'
// bytes alone.
template <int LB>
__global__ void __launch_bounds__(1024) gather_probe_kernel(const uint8_t* __restrict__ tab, int64_t row_bytes,
                                                            const int32_t* __restrict__ rows, uint32_t never,
                                                            uint32_t* __restrict__ out) {
    using W = Word<LB>;
    const int64_t i = blockIdx.x;
    const int64_t off = static_cast<int64_t>(threadIdx.x) * LB;
    if (off >= row_bytes) return;
    typename W::T v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t r = __builtin_amdgcn_readfirstlane(rows[i * 16 + k]);
        v[k] = *reinterpret_cast<const typename W::T*>(tab + r * row_bytes + off);
    }
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) x ^= W::fold(v[k]);
    if (x == never) out[i] = x;
}

// The gather above plus, per token i, side_bytes each of row tokens[i] of
// `e1`, row i of `res` and row i of `out` (16 bytes per thread, threads
// 0 .. side_bytes / 16 - 1): out's row holds the XOR of what the thread read,
// so every byte of it is written.
template <int LB>
__global__ void __launch_bounds__(1024) gather_mix_probe_kernel(const uint8_t* __restrict__ tab, int64_t row_bytes,
                                                                const int32_t* __restrict__ rows,
                                                                const int32_t* __restrict__ tokens,
                                                                const uint8_t* __restrict__ e1,
                                                                const uint8_t* __restrict__ res, int64_t side_bytes,
                                                                uint8_t* __restrict__ out) {
    using W = Word<LB>;
    const int64_t i = blockIdx.x;
    const int64_t off = static_cast<int64_t>(threadIdx.x) * LB;
    const int64_t soff = static_cast<int64_t>(threadIdx.x) * 16;
    const bool side = soff < side_bytes;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (side) {
        const int64_t c = tokens[i];
        a = *reinterpret_cast<const uint4*>(e1 + c * side_bytes + soff);
        b = *reinterpret_cast<const uint4*>(res + i * side_bytes + soff);
    }
    uint32_t x = 0;
    if (off < row_bytes) {
        typename W::T v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t r = __builtin_amdgcn_readfirstlane(rows[i * 16 + k]);
            v[k] = *reinterpret_cast<const typename W::T*>(tab + r * row_bytes + off);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) x ^= W::fold(v[k]);
    }
    if (side)
        *reinterpret_cast<uint4*>(out + i * side_bytes + soff) = make_uint4(a.x ^ b.x ^ x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
}

}  // namespace

extern "C" int probe_gather(const void* tab, int64_t row_bytes, const int32_t* rows, int64_t n, int32_t lane_bytes,
                            uint32_t* out, hipStream_t stream) {
    if (!tab || !rows || !out || n <= 0 || row_bytes <= 0 || row_bytes % lane_bytes != 0) return -1;
    const int64_t threads = (row_bytes / lane_bytes + 63) / 64 * 64;
    if (threads > 1024) return -1;
    const dim3 grid(static_cast<unsigned>(n)), block(static_cast<unsigned>(threads));
    const uint8_t* t = static_cast<const uint8_t*>(tab);
    if (lane_bytes == 4) hipLaunchKernelGGL(gather_probe_kernel<4>, grid, block, 0, stream, t, row_bytes, rows, 0x9E3779B9u, out);
    else if (lane_bytes == 8) hipLaunchKernelGGL(gather_probe_kernel<8>, grid, block, 0, stream, t, row_bytes, rows, 0x9E3779B9u, out);
    else if (lane_bytes == 16) hipLaunchKernelGGL(gather_probe_kernel<16>, grid, block, 0, stream, t, row_bytes, rows, 0x9E3779B9u, out);
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int probe_gather_mix(const void* tab, int64_t row_bytes, const int32_t* rows, int64_t n,
                                int32_t lane_bytes, const int32_t* tokens, const void* e1, const void* res,
                                int64_t side_bytes, void* out, hipStream_t stream) {
    if (!tab || !rows || !tokens || !e1 || !res || !out || n <= 0 || row_bytes <= 0 || side_bytes <= 0 ||
        row_bytes % lane_bytes != 0 || side_bytes % 16 != 0)
        return -1;
    const int64_t a = row_bytes / lane_bytes, b = side_bytes / 16;
    const int64_t threads = ((a > b ? a : b) + 63) / 64 * 64;
    if (threads > 1024) return -1;
    const dim3 grid(static_cast<unsigned>(n)), block(static_cast<unsigned>(threads));
    const uint8_t* t = static_cast<const uint8_t*>(tab);
    const uint8_t* e = static_cast<const uint8_t*>(e1);
    const uint8_t* r = static_cast<const uint8_t*>(res);
    uint8_t* o = static_cast<uint8_t*>(out);
    if (lane_bytes == 4)
        hipLaunchKernelGGL(gather_mix_probe_kernel<4>, grid, block, 0, stream, t, row_bytes, rows, tokens, e, r, side_bytes, o);
    else if (lane_bytes == 8)
        hipLaunchKernelGGL(gather_mix_probe_kernel<8>, grid, block, 0, stream, t, row_bytes, rows, tokens, e, r, side_bytes, o);
    else if (lane_bytes == 16)
        hipLaunchKernelGGL(gather_mix_probe_kernel<16>, grid, block, 0, stream, t, row_bytes, rows, tokens, e, r, side_bytes, o);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
