// GPU fill kernels for the seeded synthetic inputs (libsynth.so).
//
// Same definitions as the numpy generator in synth/__init__.py: Philox4x32-10
// (Salmon, Moraes, Dror and Shaw, SC 2011) with counter (g_lo, g_hi, tag, 0),
// g = element / 4, key = seed; element e takes word e % 4; values are built
// by exact integer operations and exact power-of-two scalings.  No part of
// the n-gram method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
        const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
        const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
        const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n1 = lo1, n2 = hi0 ^ c[3] ^ k1, n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
}

enum Kind { BF16_NORMAL12 = 0, BF16_NORMAL6 = 1, BF16_WIDE = 2, F32_UNIT = 3, I8_NORMAL = 4, F32_SCALE = 5 };

template <int KIND>
__device__ inline void put(void* dst, int64_t idx, uint32_t x) {
    if constexpr (KIND == BF16_NORMAL12 || KIND == BF16_NORMAL6) {
        const int s = static_cast<int>((x & 127u) + ((x >> 7) & 127u) + ((x >> 14) & 127u) + ((x >> 21) & 127u)) - 254;
        const float f = static_cast<float>(s) * (KIND == BF16_NORMAL12 ? 0x1p-12f : 0x1p-6f);
        static_cast<uint16_t*>(dst)[idx] = static_cast<uint16_t>(__float_as_uint(f) >> 16);
    } else if constexpr (KIND == BF16_WIDE) {
        const uint32_t b = ((x & 1u) << 15) | ((100u + ((x >> 1) & 31u)) << 7) | ((x >> 6) & 127u);
        static_cast<uint16_t*>(dst)[idx] = static_cast<uint16_t>(b);
    } else if constexpr (KIND == F32_UNIT) {
        static_cast<float*>(dst)[idx] = static_cast<float>(x >> 8) * 0x1p-24f;
    } else if constexpr (KIND == I8_NORMAL) {
        const int s = static_cast<int>((x & 63u) + ((x >> 6) & 63u) + ((x >> 12) & 63u) + ((x >> 18) & 63u)) - 126;
        static_cast<int8_t*>(dst)[idx] = static_cast<int8_t>(s);
    } else {
        static_cast<float*>(dst)[idx] = static_cast<float>((1u << 23) + (x & 0x7FFFFFu)) * 0x1p-34f;
    }
}

// Thread t covers Philox block g = g0 + t (elements 4g .. 4g+3), writing the
// elements that fall in [offset, offset + numel) to dst[e - offset].
template <int KIND>
__global__ void __launch_bounds__(256) fill_kernel(void* dst, int64_t numel, int64_t offset,
                                                   uint64_t seed, uint32_t tag) {
    const int64_t g0 = offset >> 2;
    const int64_t gend = (offset + numel + 3) >> 2;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t g = g0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < gend; g += stride) {
        uint32_t c[4] = {static_cast<uint32_t>(g), static_cast<uint32_t>(static_cast<uint64_t>(g) >> 32), tag, 0u};
        philox4x32_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int64_t e = 4 * g + w;
            if (e >= offset && e < offset + numel) put<KIND>(dst, e - offset, c[w]);
        }
    }
}

// Bytes of 4-bit MXFP4 rows (row width d, d/2 + d/32 bytes per row): code
// bytes are the word's low byte, scale bytes an E8M0 exponent.
template <bool WIDE>
__global__ void __launch_bounds__(256) fill_mxfp4_kernel(uint8_t* dst, int64_t numel, int64_t offset, uint64_t seed,
                                                         uint32_t tag, int32_t d) {
    const int64_t rb = d / 2 + d / 32;
    const int64_t g0 = offset >> 2;
    const int64_t gend = (offset + numel + 3) >> 2;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t g = g0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < gend; g += stride) {
        uint32_t c[4] = {static_cast<uint32_t>(g), static_cast<uint32_t>(static_cast<uint64_t>(g) >> 32), tag, 0u};
        philox4x32_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int64_t e = 4 * g + w;
            if (e < offset || e >= offset + numel) continue;
            const int64_t b = e % rb;
            const uint32_t x = c[w];
            const uint32_t sc = WIDE ? 100u + ((x >> 8) & 31u) : 119u + (x & 3u);
            dst[e - offset] = static_cast<uint8_t>(b < d / 2 ? (x & 0xFFu) : sc);
        }
    }
}

}  // namespace

extern "C" int synth_fill_mxfp4(int kind, uint64_t seed, uint32_t tag, void* dst, int64_t numel, int64_t offset,
                                int32_t d, hipStream_t stream) {
    if (numel <= 0) return 0;
    if (!dst || offset < 0 || d <= 0 || d % 32 != 0) return -1;
    const int64_t blocks = ((offset + numel + 3) >> 2) - (offset >> 2);
    int64_t grid = (blocks + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (kind == 6)
        hipLaunchKernelGGL(fill_mxfp4_kernel<false>, dim3(grid), dim3(256), 0, stream, static_cast<uint8_t*>(dst), numel,
                           offset, seed, tag, d);
    else if (kind == 7)
        hipLaunchKernelGGL(fill_mxfp4_kernel<true>, dim3(grid), dim3(256), 0, stream, static_cast<uint8_t*>(dst), numel,
                           offset, seed, tag, d);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int synth_fill(int kind, uint64_t seed, uint32_t tag, void* dst, int64_t numel, int64_t offset,
                          hipStream_t stream) {
    if (numel <= 0) return 0;
    if (!dst || offset < 0) return -1;
    const int64_t blocks = ((offset + numel + 3) >> 2) - (offset >> 2);
    int64_t grid = (blocks + 255) / 256;
    if (grid > 65536) grid = 65536;
    const dim3 g(static_cast<unsigned>(grid)), b(256);
    switch (kind) {
        case BF16_NORMAL12: hipLaunchKernelGGL(fill_kernel<BF16_NORMAL12>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        case BF16_NORMAL6: hipLaunchKernelGGL(fill_kernel<BF16_NORMAL6>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        case BF16_WIDE: hipLaunchKernelGGL(fill_kernel<BF16_WIDE>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        case F32_UNIT: hipLaunchKernelGGL(fill_kernel<F32_UNIT>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        case I8_NORMAL: hipLaunchKernelGGL(fill_kernel<I8_NORMAL>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        case F32_SCALE: hipLaunchKernelGGL(fill_kernel<F32_SCALE>, g, b, 0, stream, dst, numel, offset, seed, tag); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
