// probe.hip -- plain kernels that measure what a kernel on this device can
// reach, beside the specification's figures.  Streaming: a read of a buffer
// folded into one register per lane, and a copy.  Each thread issues U
// independent 16-byte loads per round, lanes of a wavefront on consecutive
// 16-byte pieces; the grid strides over the buffer.  The rate depends on the
// bytes a CU keeps in flight (loads per thread times waves per CU), which the
// caller sets with U and the grid.  Matrix cores: back-to-back 32x32x16 bf16
// matrix instructions on register operands, four independent accumulator
// chains per wavefront, no memory traffic.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace tfla {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                         u32x4* __restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t b = t; b < n; b += U * stride) {
        u32x4 x[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t i = b + j * stride;
            x[j] = i < n ? src[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= x[j];
    }
    // a store the compiler cannot drop, that (almost) never happens
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu) sink[t & 255] = acc;
}

template <int U>
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (size_t b = t; b < n; b += U * stride) {
        u32x4 x[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t i = b + j * stride;
            if (i < n) x[j] = src[i];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t i = b + j * stride;
            if (i < n) dst[i] = x[j];
        }
    }
}

template <int U>
hipError_t probe_launch(int mode, const u32x4* src, u32x4* dst, size_t n, int blocks, hipStream_t s)
{
    if (mode == 0) probe_read_kernel<U><<<blocks, 256, 0, s>>>(src, n, dst);
    else probe_copy_kernel<U><<<blocks, 256, 0, s>>>(src, dst, n);
    return hipGetLastError();
}

// 4 chains x iters matrix instructions per wavefront (32768 flops each);
// the operands depend on the lane so that nothing folds, and the sums are
// stored only in a case that does not occur
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink)
{
    constexpr int CH = 4;
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = to_bf16(1.0f + 0.001f * (float)((threadIdx.x + e) & 7));
        b[e] = to_bf16(0.5f - 0.001f * (float)((threadIdx.x * 3 + e) & 7));
    }
    f32x16 acc[CH];
    for (int c = 0; c < CH; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = mma32(a, b, acc[c]);
    }
    float sum = 0.0f;
    for (int c = 0; c < CH; ++c)
        for (int r = 0; r < 16; ++r) sum += acc[c][r];
    if (sum == -1.0f) sink[threadIdx.x] = sum;
}

}  // namespace

hipError_t launch_mfma_probe(int iters, int blocks, float* sink, hipStream_t stream)
{
    probe_mfma_kernel<<<blocks, 256, 0, stream>>>(iters, sink);
    return hipGetLastError();
}

hipError_t launch_stream_probe(int mode, const void* src, void* dst, size_t bytes, int loads, int blocks,
                               hipStream_t stream)
{
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    const size_t n = bytes / 16;
    switch (loads) {
    case 1: return probe_launch<1>(mode, s, d, n, blocks, stream);
    case 2: return probe_launch<2>(mode, s, d, n, blocks, stream);
    case 4: return probe_launch<4>(mode, s, d, n, blocks, stream);
    case 8: return probe_launch<8>(mode, s, d, n, blocks, stream);
    case 16: return probe_launch<16>(mode, s, d, n, blocks, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tfla
