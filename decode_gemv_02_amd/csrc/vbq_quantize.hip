// Per-group quantizer of the VBQ library (gfx950): fp32 weights -> the int8
// codes and binary16 scales that vbq_pack takes.
//
// VBQ paper (arXiv 2607.02893) §3.1 Eq. (1): a group of 64 weights at b >= 2
// bits has scale s = max|w| / (2^(b-1) - 1) and codes clip(round(w / s),
// -(2^(b-1) - 1), 2^(b-1) - 1); at 1 bit a weight keeps its sign and the scale
// is the group's mean magnitude. Where the pages leave a step open:
//   - max|w|, the b >= 2 scale and the ratios are fp32 with correctly rounded
//     division; the 1-bit magnitudes are summed in fp64 (exact for any
//     realistic spread of magnitudes, so the order of the sum does not show)
//     and divided by 64;
//   - the stored scale is that value rounded once to binary16 (nearest even;
//     the fp64 mean goes straight to binary16, with no fp32 step), saturated
//     at 65504, and the codes are computed with the stored scale;
//   - ties round away from zero; sign(0) = +1 (also -0.0); a stored scale of 0
//     gives codes 0 at b >= 2.
//
// Work decomposition: a team of 16 lanes holds one group, four weights a
// lane, so one wave reads four groups (1 KiB) per load; each team has one
// (small matrices) or four groups' loads in flight before it reduces the
// first. The group's largest
// magnitude or magnitude sum is reduced across its 16 lanes with
// butterflies, so every lane ends with the same value and the same scale.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <unordered_map>

#include "vbq_internal.h"

using vbq::fail;

namespace {

constexpr uint32_t kLanesPerGroup = 16;
constexpr uint32_t kBlock = 256;
constexpr uint32_t kTeams = kBlock / kLanesPerGroup;          // 16-lane teams per workgroup
// Groups a team keeps in flight: four for large matrices; one below kFewGroups groups, where the
// launch is short and a wider grid fills the chip sooner (4096x4096: 19.1 against 22.0 us).
constexpr uint64_t kFewGroups = 1u << 19;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// binary16 bits of a non-negative value, one rounding to nearest even, saturated at the largest finite half
template <typename T>
__device__ __forceinline__ uint16_t stored_scale(T s) {
    const _Float16 h = static_cast<_Float16>(s);
    const uint16_t bits = __builtin_bit_cast(uint16_t, h);
    return (bits & 0x7FFFu) >= 0x7C00u ? 0x7BFFu : bits;
}

__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (uint32_t d = 1; d < kLanesPerGroup; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, kLanesPerGroup));
    return v;
}

__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
    for (uint32_t d = 1; d < kLanesPerGroup; d <<= 1) v += __shfl_xor(v, d, kLanesPerGroup);
    return v;
}

// b >= 2: the code of w for stored scale s (binary16 value as fp32)
__device__ __forceinline__ uint32_t code_of(float w, float s, float qmax) {
    if (s == 0.f) return 0u;
    const float q = fminf(fmaxf(roundf(__fdiv_rn(w, s)), -qmax), qmax);   // roundf: ties away from zero
    return static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu;
}

// One lane's four weights of a group of width b: the packed int8 codes, and the group's scale in *s16
// (every lane of the team computes the same scale).
__device__ __forceinline__ uint32_t quantize_quad(float4 v, uint32_t b, uint16_t *s16) {
    const float m0 = fabsf(v.x), m1 = fabsf(v.y), m2 = fabsf(v.z), m3 = fabsf(v.w);
    if (b == 1) {
        const double sum = group_sum(((static_cast<double>(m0) + m1) + m2) + m3);
        *s16 = stored_scale(sum * (1.0 / 64.0));   // fp64 -> binary16 directly
        // sign(w) as an int8 code, +1 for w >= 0 (and -0.0)
        return (v.x < 0.f ? 0xFFu : 1u) | ((v.y < 0.f ? 0xFFu : 1u) << 8) | ((v.z < 0.f ? 0xFFu : 1u) << 16) |
               ((v.w < 0.f ? 0xFFu : 1u) << 24);
    }
    if (b == 2 || b == 4 || b == 8) {
        const float amax = group_max(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
        const float qmax = static_cast<float>((1u << (b - 1)) - 1u);
        *s16 = stored_scale(__fdiv_rn(amax, qmax));
        const float s = static_cast<float>(__builtin_bit_cast(_Float16, *s16));
        return code_of(v.x, s, qmax) | (code_of(v.y, s, qmax) << 8) | (code_of(v.z, s, qmax) << 16) |
               (code_of(v.w, s, qmax) << 24);
    }
    *s16 = 0;   // another width value leaves scale 0 and codes 0
    return 0u;
}

// Workgroup x covers groups [x * kGroupsPerBlock, (x + 1) * kGroupsPerBlock): pass j hands group
// x * kGroupsPerBlock + j * kTeams + team to a team, so each pass reads 4 KiB contiguous. All of a
// team's loads are issued before the first reduction.
template <uint32_t kGroupsPerTeam>
__global__ __launch_bounds__(kBlock) void quantize_groups(const float4 *__restrict__ w, const uint8_t *__restrict__ bits,
                                                         uint32_t *__restrict__ codes, uint16_t *__restrict__ scales,
                                                         uint64_t groups) {
    constexpr uint32_t kGroupsPerBlock = kTeams * kGroupsPerTeam;
    const uint32_t team = threadIdx.x / kLanesPerGroup, lane = threadIdx.x % kLanesPerGroup;
    const uint64_t first = static_cast<uint64_t>(blockIdx.x) * kGroupsPerBlock + team;
    float4 v[kGroupsPerTeam];
    uint32_t b[kGroupsPerTeam];
#pragma unroll
    for (uint32_t j = 0; j < kGroupsPerTeam; ++j) {
        const uint64_t g = first + j * kTeams;   // team-uniform, so whole teams take each branch
        if (g < groups) {
            // each weight is read once: a non-temporal load keeps the stream out of the caches
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(w) + g * kLanesPerGroup + lane);
            v[j] = make_float4(t.x, t.y, t.z, t.w);
            b[j] = bits[g];
        }
    }
#pragma unroll
    for (uint32_t j = 0; j < kGroupsPerTeam; ++j) {
        const uint64_t g = first + j * kTeams;
        if (g < groups) {
            uint16_t s16;
            codes[g * kLanesPerGroup + lane] = quantize_quad(v[j], b[j], &s16);
            if (lane == 0) scales[g] = s16;
        }
    }
}

// ---------------------------------------------------------------- soft quantizer (training side)
// VBQ §3.2 "Differentiable bit selection": per group, pi = softmax((logits + e) / tau) over the widths
// (1, 2, 4, 8) mixes the group's Eq. (1) reconstructions at the four widths, and the group's expected
// width is sum_k pi_k * B_k. At training time the scales stay fp32 (no binary16 rounding); scales, ratios
// and code decisions are fp32 as in the hard quantizer, the 1-bit mean is summed in fp64.
__device__ __forceinline__ float recon_code(float w, float s, float qmax) {
    if (s == 0.f) return 0.f;
    return fminf(fmaxf(roundf(__fdiv_rn(w, s)), -qmax), qmax);
}

__global__ __launch_bounds__(kBlock) void soft_quantize_groups(const float4 *__restrict__ w,
                                                              const float4 *__restrict__ logits,
                                                              const float4 *__restrict__ gumbel, float tau,
                                                              float4 *__restrict__ w_soft, float4 *__restrict__ pi,
                                                              float *__restrict__ group_bits, uint64_t groups) {
    const uint64_t t = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    const uint64_t g = t / kLanesPerGroup;   // whole 16-lane teams share a group: they leave together
    if (g >= groups) return;
    const float4 v = w[t];
    const float4 l = logits[g], e = gumbel[g];
    const float z0 = __fdiv_rn(l.x + e.x, tau), z1 = __fdiv_rn(l.y + e.y, tau);
    const float z2 = __fdiv_rn(l.z + e.z, tau), z3 = __fdiv_rn(l.w + e.w, tau);
    const float zm = fmaxf(fmaxf(z0, z1), fmaxf(z2, z3));
    const float p0 = expf(z0 - zm), p1 = expf(z1 - zm), p2 = expf(z2 - zm), p3 = expf(z3 - zm);
    const float ps = (p0 + p1) + (p2 + p3);
    const float4 pk = make_float4(__fdiv_rn(p0, ps), __fdiv_rn(p1, ps), __fdiv_rn(p2, ps), __fdiv_rn(p3, ps));
    const float m0 = fabsf(v.x), m1 = fabsf(v.y), m2 = fabsf(v.z), m3 = fabsf(v.w);
    const float s1 = static_cast<float>(group_sum(((static_cast<double>(m0) + m1) + m2) + m3) * (1.0 / 64.0));
    const float amax = group_max(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
    const float s2 = amax, s4 = __fdiv_rn(amax, 7.f), s8 = __fdiv_rn(amax, 127.f);
    const float c1 = pk.x * s1, c2 = pk.y * s2, c4 = pk.z * s4, c8 = pk.w * s8;
    auto mix = [&](float x) {
        const float q1 = x < 0.f ? -1.f : 1.f;
        return fmaf(c8, recon_code(x, s8, 127.f),
                    fmaf(c4, recon_code(x, s4, 7.f), fmaf(c2, recon_code(x, s2, 1.f), c1 * q1)));
    };
    w_soft[t] = make_float4(mix(v.x), mix(v.y), mix(v.z), mix(v.w));
    if ((t & (kLanesPerGroup - 1)) == 0) {
        pi[g] = pk;
        group_bits[g] = fmaf(8.f, pk.w, fmaf(4.f, pk.z, fmaf(2.f, pk.y, pk.x)));
    }
}

// Mean of group_bits[0, groups) in fp64, in a fixed order: workgroup b of the first kernel adds the
// contiguous chunk [b * chunk, (b + 1) * chunk) (strided per lane, then a tree), the second adds the
// partial sums (a tree over at most kParts values).
constexpr uint32_t kParts = 1024;

__global__ __launch_bounds__(256) void chunk_sums(const float *__restrict__ group_bits, uint64_t groups,
                                                  uint64_t chunk, double *__restrict__ part) {
    __shared__ double s[256];
    const uint64_t lo = static_cast<uint64_t>(blockIdx.x) * chunk;
    const uint64_t hi = lo + chunk < groups ? lo + chunk : groups;
    double acc = 0.0;
    for (uint64_t i = lo + threadIdx.x; i < hi; i += 256) acc += group_bits[i];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (uint32_t half = 128; half > 0; half >>= 1) {
        if (threadIdx.x < half) s[threadIdx.x] += s[threadIdx.x + half];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = s[0];
}

__global__ __launch_bounds__(kParts) void mean_of_parts(const double *__restrict__ part, uint32_t parts,
                                                        uint64_t groups, double *__restrict__ out) {
    __shared__ double s[kParts];
    s[threadIdx.x] = threadIdx.x < parts ? part[threadIdx.x] : 0.0;
    __syncthreads();
    for (uint32_t half = kParts / 2; half > 0; half >>= 1) {
        if (threadIdx.x < half) s[threadIdx.x] += s[threadIdx.x + half];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = groups ? s[0] / static_cast<double>(groups) : 0.0;
}

// kParts doubles of device scratch per (device, stream), allocated on first use (never while the
// stream is being captured) and held until the process ends
std::mutex g_parts_mu;
std::unordered_map<uint64_t, double *> g_parts;

vbq_status parts_for(hipStream_t stream, double **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VBQ_ERR_HIP, "vbq_soft_quantize: hipGetDevice failed");
    const uint64_t key = (static_cast<uint64_t>(dev) << 56) ^ reinterpret_cast<uintptr_t>(stream);
    std::lock_guard<std::mutex> lock(g_parts_mu);
    double *&p = g_parts[key];
    if (!p) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
            return fail(VBQ_ERR_HIP, "vbq_soft_quantize: could not query the stream's capture state");
        if (cs != hipStreamCaptureStatusNone)
            return fail(VBQ_ERR_HIP, "vbq_soft_quantize: first call on a stream that is being captured (the library "
                                     "does not allocate during capture; call once on this stream first)");
        if (hipMalloc(reinterpret_cast<void **>(&p), kParts * sizeof(double)) != hipSuccess) {
            p = nullptr;
            return fail(VBQ_ERR_HIP, "vbq_soft_quantize: scratch hipMalloc failed");
        }
    }
    *out = p;
    return VBQ_OK;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" vbq_status vbq_quantize(uint32_t n, uint32_t k, const float *w, const uint8_t *bits, int8_t *codes_out,
                                   uint16_t *scales_out, void *stream) {
    return vbq::guarded("vbq_quantize", [&]() -> vbq_status {
        vbq::clear_error();
        if (k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_quantize: k=%u is not a multiple of 64", k);
        if (n == 0 || k == 0) return VBQ_OK;
        if (!w || !bits || !codes_out || !scales_out) return fail(VBQ_ERR_NULL, "vbq_quantize: a pointer is NULL");
        if (!aligned(w, 16) || !aligned(codes_out, 4) || !aligned(scales_out, 2))
            return fail(VBQ_ERR_ALIGN, "vbq_quantize: w must be 16-byte, codes 4-byte and scales 2-byte aligned");
        const uint64_t groups = static_cast<uint64_t>(n) * (k / VBQ_GROUP);
        const bool few = groups < kFewGroups;
        const uint64_t per_block = static_cast<uint64_t>(kTeams) * (few ? 1u : 4u);
        const uint64_t blocks = (groups + per_block - 1) / per_block;
        if (blocks > 0x7FFFFFFFull) return fail(VBQ_ERR_SHAPE, "vbq_quantize: %llu groups exceed one launch",
                                                static_cast<unsigned long long>(groups));
        (void)hipGetLastError();
        const hipStream_t s = static_cast<hipStream_t>(stream);
        if (few)
            hipLaunchKernelGGL(quantize_groups<1>, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, s,
                               reinterpret_cast<const float4 *>(w), bits, reinterpret_cast<uint32_t *>(codes_out),
                               scales_out, groups);
        else
            hipLaunchKernelGGL(quantize_groups<4>, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, s,
                               reinterpret_cast<const float4 *>(w), bits, reinterpret_cast<uint32_t *>(codes_out),
                               scales_out, groups);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(VBQ_ERR_HIP, "vbq_quantize: launch failed: %s", hipGetErrorString(e));
        return VBQ_OK;
    });
}

extern "C" vbq_status vbq_soft_quantize(uint32_t n, uint32_t k, const float *w, const float *logits,
                                        const float *gumbel, float tau, float *w_soft, float *pi, float *group_bits,
                                        double *mean_bits, void *stream) {
    return vbq::guarded("vbq_soft_quantize", [&]() -> vbq_status {
        vbq::clear_error();
        if (k % VBQ_GROUP) return fail(VBQ_ERR_SHAPE, "vbq_soft_quantize: k=%u is not a multiple of 64", k);
        if (!(tau > 0.f) || tau > 3.0e38f) return fail(VBQ_ERR_SHAPE, "vbq_soft_quantize: tau must be positive and finite");
        if (!mean_bits) return fail(VBQ_ERR_NULL, "vbq_soft_quantize: mean_bits is NULL");
        if (!aligned(mean_bits, 8)) return fail(VBQ_ERR_ALIGN, "vbq_soft_quantize: mean_bits must be 8-byte aligned");
        const uint64_t groups = static_cast<uint64_t>(n) * (k / VBQ_GROUP);
        const uint64_t blocks = (groups * kLanesPerGroup + kBlock - 1) / kBlock;
        if (groups) {
            if (!w || !logits || !gumbel || !w_soft || !pi || !group_bits)
                return fail(VBQ_ERR_NULL, "vbq_soft_quantize: a pointer is NULL");
            if (!aligned(w, 16) || !aligned(w_soft, 16) || !aligned(logits, 16) || !aligned(gumbel, 16) ||
                !aligned(pi, 16) || !aligned(group_bits, 4))
                return fail(VBQ_ERR_ALIGN, "vbq_soft_quantize: w, w_soft, logits, gumbel and pi must be 16-byte aligned");
            if (blocks > 0x7FFFFFFFull)
                return fail(VBQ_ERR_SHAPE, "vbq_soft_quantize: %llu groups exceed one launch",
                            static_cast<unsigned long long>(groups));
        }
        const hipStream_t s = static_cast<hipStream_t>(stream);
        double *parts = nullptr;
        const vbq_status ps = parts_for(s, &parts);
        if (ps != VBQ_OK) return ps;
        (void)hipGetLastError();
        if (groups == 0) {   // no group: the mean is taken as 0
            hipLaunchKernelGGL(mean_of_parts, dim3(1), dim3(kParts), 0, s, static_cast<const double *>(parts), 0u,
                               uint64_t(0), mean_bits);
        } else {
            hipLaunchKernelGGL(soft_quantize_groups, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, s,
                               reinterpret_cast<const float4 *>(w), reinterpret_cast<const float4 *>(logits),
                               reinterpret_cast<const float4 *>(gumbel), tau, reinterpret_cast<float4 *>(w_soft),
                               reinterpret_cast<float4 *>(pi), group_bits, groups);
            const uint64_t chunk = (groups + kParts - 1) / kParts;
            const uint32_t nparts = static_cast<uint32_t>((groups + chunk - 1) / chunk);
            hipLaunchKernelGGL(chunk_sums, dim3(nparts), dim3(256), 0, s, static_cast<const float *>(group_bits), groups,
                               chunk, parts);
            hipLaunchKernelGGL(mean_of_parts, dim3(1), dim3(kParts), 0, s, static_cast<const double *>(parts), nparts,
                               groups, mean_bits);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(VBQ_ERR_HIP, "vbq_soft_quantize: launch failed: %s", hipGetErrorString(e));
        return VBQ_OK;
    });
}
