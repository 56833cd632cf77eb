// Device half of the VBQ library (gfx950): argument checks, launches and kernels.
//
// VBQ paper (arXiv 2607.02893) §6, "Fused kernels over packed weights": each
// group's packed bytes are read once, expanded to integer codes in registers,
// combined with the group's fp16 scale and accumulated into y = W x; no dense
// weight matrix is ever written. Grid and scale: §3.1 Eq. (1).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vbq_internal.h"

using vbq::fail;

namespace {

constexpr uint32_t kWave = 64;

__device__ __forceinline__ float half_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// b-bit field -> integer code: b = 1 is a sign bit, b >= 2 two's complement.
__device__ __forceinline__ int decode_field(uint32_t f, uint32_t b) {
    if (b == 1) return f ? -1 : 1;
    const uint32_t sh = 32u - b;
    return static_cast<int>(f << sh) >> sh;
}

// width of flat group t
__device__ __forceinline__ uint32_t group_bits(const uint8_t *widths, uint64_t t) {
    return 1u << ((widths[t >> 2] >> (2 * (t & 3))) & 3u);
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// One wave per row; lane i decodes element i of each group in turn, so the
// width branch is uniform across the wave. The scale is folded into the code
// (s*q is exact in fp32: 11 x 7 significant bits) and the product with x is
// accumulated per lane in fp32, then summed across the wave.
__global__ __launch_bounds__(256) void gemv_rowwave(const uint8_t *__restrict__ widths,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint32_t *__restrict__ row_offsets,
                                                    const uint8_t *__restrict__ payload,
                                                    const uint16_t *__restrict__ x, float *__restrict__ y,
                                                    uint32_t n, uint32_t groups, uint32_t k, uint32_t m) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const uint32_t mm = blockIdx.y;
    if (r >= n || mm >= m) return;
    const uint16_t *xm = x + uint64_t(mm) * k;
    uint32_t off = row_offsets[r];
    float acc = 0.f;
    for (uint32_t j = 0; j < groups; ++j) {
        const uint64_t t = uint64_t(r) * groups + j;
        const uint32_t b = group_bits(widths, t);
        const float s = half_to_float(scales[t]);
        const uint32_t bit = b * lane;
        const uint32_t f = (payload[off + (bit >> 3)] >> (bit & 7)) & ((1u << b) - 1u);
        acc += (s * static_cast<float>(decode_field(f, b))) * half_to_float(xm[j * kWave + lane]);
        off += 8u * b;
    }
    acc = wave_sum(acc);
    if (lane == 0) y[uint64_t(mm) * n + r] = acc;
}

__global__ __launch_bounds__(256) void unpack_rowwave(const uint8_t *__restrict__ widths,
                                                      const uint32_t *__restrict__ row_offsets,
                                                      const uint8_t *__restrict__ payload, int8_t *__restrict__ codes,
                                                      uint32_t n, uint32_t groups) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (r >= n) return;
    uint32_t off = row_offsets[r];
    int8_t *dst = codes + uint64_t(r) * groups * kWave;
    for (uint32_t j = 0; j < groups; ++j) {
        const uint32_t b = group_bits(widths, uint64_t(r) * groups + j);
        const uint32_t bit = b * lane;
        const uint32_t f = (payload[off + (bit >> 3)] >> (bit & 7)) & ((1u << b) - 1u);
        dst[j * kWave + lane] = static_cast<int8_t>(decode_field(f, b));
        off += 8u * b;
    }
}

__global__ void fill_zero(float *__restrict__ y, uint64_t count) {
    const uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < count) y[i] = 0.f;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vbq_status check_matrix(const char *who, const vbq_matrix *w) {
    if (!w) return fail(VBQ_ERR_NULL, "%s: matrix view is NULL", who);
    if (w->abi_version != VBQ_ABI_VERSION)
        return fail(VBQ_ERR_ABI, "%s: abi_version %u, library %u", who, w->abi_version, VBQ_ABI_VERSION);
    if (w->k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "%s: k=%u is not a multiple of 64", who, w->k);
    if (w->k > VBQ_MAX_K) return fail(VBQ_ERR_SHAPE, "%s: k=%u exceeds %u", who, w->k, VBQ_MAX_K);
    if (w->n == 0) return VBQ_OK;
    if (!w->row_offsets) return fail(VBQ_ERR_NULL, "%s: row_offsets is NULL", who);
    if (w->k && (!w->widths || !w->scales || !w->payload))
        return fail(VBQ_ERR_NULL, "%s: widths, scales or payload is NULL", who);
    if (!aligned16(w->row_offsets) || (w->k && (!aligned16(w->widths) || !aligned16(w->scales) ||
                                                !aligned16(w->payload))))
        return fail(VBQ_ERR_ALIGN, "%s: a matrix array is not 16-byte aligned", who);
    return VBQ_OK;
}

vbq_status launched(const char *who) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VBQ_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return VBQ_OK;
}

vbq_status run_gemm(const char *who, const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y, void *stream) {
    vbq::clear_error();
    vbq_status st = check_matrix(who, w);
    if (st != VBQ_OK) return st;
    if (m == 0 || m > VBQ_MAX_BATCH) return fail(VBQ_ERR_SHAPE, "%s: m=%u outside [1, %u]", who, m, VBQ_MAX_BATCH);
    if (w->n == 0) return VBQ_OK;
    if (!y || (w->k && !x)) return fail(VBQ_ERR_NULL, "%s: x or y is NULL", who);
    if (!aligned16(y) || (w->k && !aligned16(x))) return fail(VBQ_ERR_ALIGN, "%s: x or y is not 16-byte aligned", who);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (w->k == 0) {
        const uint64_t count = uint64_t(m) * w->n;
        hipLaunchKernelGGL(fill_zero, dim3(uint32_t((count + 255) / 256)), dim3(256), 0, s, y, count);
        return launched(who);
    }
    const uint32_t groups = w->k / VBQ_GROUP;
    hipLaunchKernelGGL(gemv_rowwave, dim3((w->n + 3) / 4, m), dim3(256), 0, s, w->widths, w->scales, w->row_offsets,
                       w->payload, x, y, w->n, groups, w->k, m);
    return launched(who);
}

}  // namespace

extern "C" vbq_status vbq_gemv(const vbq_matrix *w, const uint16_t *x, float *y, void *stream) {
    return run_gemm("vbq_gemv", w, x, 1, y, stream);
}

extern "C" vbq_status vbq_gemm_smallbatch(const vbq_matrix *w, const uint16_t *x, uint32_t m, float *y,
                                          void *stream) {
    return run_gemm("vbq_gemm_smallbatch", w, x, m, y, stream);
}

extern "C" vbq_status vbq_unpack_codes(const vbq_matrix *w, int8_t *codes_out, void *stream) {
    vbq::clear_error();
    vbq_status st = check_matrix("vbq_unpack_codes", w);
    if (st != VBQ_OK) return st;
    if (w->n == 0 || w->k == 0) return VBQ_OK;
    if (!codes_out) return fail(VBQ_ERR_NULL, "vbq_unpack_codes: codes_out is NULL");
    if (!aligned16(codes_out)) return fail(VBQ_ERR_ALIGN, "vbq_unpack_codes: codes_out is not 16-byte aligned");
    (void)hipGetLastError();
    hipLaunchKernelGGL(unpack_rowwave, dim3((w->n + 3) / 4), dim3(256), 0, static_cast<hipStream_t>(stream),
                       w->widths, w->row_offsets, w->payload, codes_out, w->n, w->k / VBQ_GROUP);
    return launched("vbq_unpack_codes");
}
