// Measurement kernels of the VBQ library (gfx950): what the packed GEMV is
// compared with, not part of its path.
//
//   stream_read  reads a buffer once with 16-byte loads and keeps nothing: the
//                HBM read rate a launch of that size can reach on this GPU
//                (its ramp and drain included), the practical ceiling of any
//                streaming kernel.
//   dense_gemv   y = W x for a dense fp16 W [n][k] row-major: the baseline the
//                VBQ paper (arXiv 2607.02893) compares decode against in §6
//                (Figure 5 and the Table 2 caption: the same weights
//                dequantized to dense FP16).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vbq_internal.h"

using vbq::fail;

namespace {

constexpr uint32_t kWave = 64;

// Every thread reads 16-byte chunks t, t + T, t + 2T, ... (T = all threads of
// the launch), four loads in flight per round; the XOR of what it read is
// stored only if it equals a value no buffer the benches pass produces, so
// the loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void stream_read(const uint4 *__restrict__ buf, uint64_t chunks,
                                                   uint32_t *__restrict__ sink) {
    const uint64_t T = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * T < chunks; i += 4 * T) {
        const uint4 a = buf[i], b = buf[i + T], c = buf[i + 2 * T], d = buf[i + 3 * T];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < chunks; i += T) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Dense fp16 GEMV: a wave owns kRows consecutive rows; lane l holds the
// activations of the 16-byte chunks l, l + 64, ... of a row in registers (up
// to kChunks of them; a row has k / 8 chunks) and reads the same chunks of
// each of its rows, so every full load instruction of the wave is 1 KiB
// contiguous. fp16 products, fp32 sums (v_dot2_f32_f16), then a shuffle row
// sum.
template <uint32_t kChunks, uint32_t kRows>
__global__ __launch_bounds__(256) void dense_gemv(const uint4 *__restrict__ w, const uint4 *__restrict__ x,
                                                  float *__restrict__ y, uint32_t n, uint32_t row_chunks) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const uint32_t r0 = wave * kRows;
    if (r0 >= n) return;
    uint4 xv[kChunks];
#pragma unroll
    for (uint32_t c = 0; c < kChunks; ++c)
        xv[c] = c * kWave + lane < row_chunks ? x[c * kWave + lane] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (uint32_t r = 0; r < kRows; ++r) {
        const uint32_t row = r0 + r < n ? r0 + r : n - 1;
        const uint4 *wr = w + static_cast<uint64_t>(row) * row_chunks;
        float acc = 0.f;
#pragma unroll
        for (uint32_t c = 0; c < kChunks; ++c) {
            if (c * kWave + lane >= row_chunks) break;
            const uint4 v = wr[c * kWave + lane];
            acc = dot2(v.x, xv[c].x, acc);
            acc = dot2(v.y, xv[c].y, acc);
            acc = dot2(v.z, xv[c].z, acc);
            acc = dot2(v.w, xv[c].w, acc);
        }
#pragma unroll
        for (uint32_t off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
        if (lane == 0 && r0 + r < n) y[r0 + r] = acc;
    }
}

constexpr uint32_t kDenseMaxChunks = 32;   // k up to 16384

// the instance holding exactly ceil(k / 512) chunks a lane
template <uint32_t kChunks>
void launch_dense(uint32_t chunks, const void *w, const void *x, float *y, uint32_t n, uint32_t k, hipStream_t s) {
    if constexpr (kChunks <= kDenseMaxChunks) {
        if (chunks != kChunks) return launch_dense<kChunks + 1>(chunks, w, x, y, n, k, s);
        constexpr uint32_t kRows = 2;
        const uint32_t waves = (n + kRows - 1) / kRows;
        const uint32_t blocks = (waves * kWave + 255) / 256;
        hipLaunchKernelGGL((dense_gemv<kChunks, kRows>), dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint4 *>(w), static_cast<const uint4 *>(x), y, n, k / 8);
    }
}

}  // namespace

extern "C" vbq_status vbq_probe_stream_read(const void *buf, uint64_t bytes, uint32_t *sink, uint32_t blocks,
                                            void *stream) {
    return vbq::guarded("vbq_probe_stream_read", [&]() -> vbq_status {
        vbq::clear_error();
        if (bytes == 0) return VBQ_OK;
        if (!buf || !sink) return fail(VBQ_ERR_NULL, "vbq_probe_stream_read: buf or sink is NULL");
        if (bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
            return fail(VBQ_ERR_ALIGN, "vbq_probe_stream_read: buf and bytes must be multiples of 16");
        if (blocks == 0 || blocks > (1u << 20))
            return fail(VBQ_ERR_SHAPE, "vbq_probe_stream_read: blocks=%u outside [1, 2^20]", blocks);
        (void)hipGetLastError();
        hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const uint4 *>(buf), bytes / 16, sink);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(VBQ_ERR_HIP, "vbq_probe_stream_read: launch failed: %s", hipGetErrorString(e));
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_probe_dense_gemv(const uint16_t *w, const uint16_t *x, float *y, uint32_t n, uint32_t k,
                                           void *stream) {
    return vbq::guarded("vbq_probe_dense_gemv", [&]() -> vbq_status {
        vbq::clear_error();
        if (n == 0) return VBQ_OK;
        if (!w || !x || !y) return fail(VBQ_ERR_NULL, "vbq_probe_dense_gemv: w, x or y is NULL");
        if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(x)) & 15u)
            return fail(VBQ_ERR_ALIGN, "vbq_probe_dense_gemv: w and x must be 16-byte aligned");
        if (k == 0 || k % 64 || k > 512 * kDenseMaxChunks)
            return fail(VBQ_ERR_SHAPE, "vbq_probe_dense_gemv: k=%u is not a multiple of 64 in [64, %u]", k,
                        512 * kDenseMaxChunks);
        (void)hipGetLastError();
        launch_dense<1>((k + 511) / 512, w, x, y, n, k, static_cast<hipStream_t>(stream));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(VBQ_ERR_HIP, "vbq_probe_dense_gemv: launch failed: %s", hipGetErrorString(e));
        return VBQ_OK;
    });
}
