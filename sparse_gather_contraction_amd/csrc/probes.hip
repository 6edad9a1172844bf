// probes.hip — microbenchmarks of what the gfx950 device reaches on this machine, for the benchmark's
// "achievable" figures beside the published peaks (libdisco_probes.so; not part of the DISCO
// library).  Each probe is a plain kernel with a fixed, in-bounds access pattern:
//   * read stream: every element of a device buffer read once with 16-byte loads (grid-stride,
//     four loads in flight per lane), summed so the loads are kept; one float per workgroup out;
//   * copy: the same stream written to a second buffer (read + write bytes);
//   * fp32 FMA loop: eight independent v_fmac_f32 chains per lane (packed fp32 ops are disabled
//     in this build, as in the library);
//   * bf16 MFMA loop: four independent v_mfma_f32_32x32x16_bf16 accumulators per wave.
#include <hip/hip_runtime.h>
#include <cstdint>

extern "C" {
hipError_t disco_probe_read(const void *buf, size_t bytes, float *out, int blocks, void *stream);
hipError_t disco_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream);
hipError_t disco_probe_fma(int iters, float *out, int blocks, void *stream);
hipError_t disco_probe_mfma(int iters, float *out, int blocks, void *stream);
}

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const float4 *__restrict__ p, size_t n16, float *out)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const float4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        s.x += a.x + b.x + c.x + d.x;
        s.y += a.y + b.y + c.y + d.y;
        s.z += a.z + b.z + c.z + d.z;
        s.w += a.w + b.w + c.w + d.w;
    }
    for (; i < n16; i += stride) {
        const float4 a = p[i];
        s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
    }
    const float t = s.x + s.y + s.z + s.w;
    if (t == 12345.678f) out[blockIdx.x] = t;  // keeps the loads; never true for the probe's data
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                        size_t n16)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void fma_kernel(int iters, float *out)
{
    float a[8];
    const float m = 1.0f + 1e-7f * (float)(threadIdx.x & 7), c = 1e-7f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = (float)(threadIdx.x + k);
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += a[k];
    out[blockIdx.x * kThreads + threadIdx.x] = t;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float *out)
{
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(1.0f / (float)(1 + ((threadIdx.x + k) & 15)));
        b[k] = (__bf16)(1.0f / (float)(2 + ((threadIdx.x * 3 + k) & 15)));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += c0[k] + c1[k] + c2[k] + c3[k];
    out[blockIdx.x * kThreads + threadIdx.x] = t;
}

}  // namespace

// bytes must be a multiple of 16 and the buffers 16-byte aligned (the caller passes torch tensors
// of whole 16-byte units); out holds `blocks` floats (fma, mfma: blocks * 256).
hipError_t disco_probe_read(const void *buf, size_t bytes, float *out, int blocks, void *stream)
{
    if (bytes % 16 != 0 || (uintptr_t)buf % 16 != 0 || blocks <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const float4 *)buf,
                       bytes / 16, out);
    return hipGetLastError();
}

hipError_t disco_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream)
{
    if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0 || blocks <= 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, (const float4 *)src,
                       (float4 *)dst, bytes / 16);
    return hipGetLastError();
}

hipError_t disco_probe_fma(int iters, float *out, int blocks, void *stream)
{
    if (iters <= 0 || blocks <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError();
}

hipError_t disco_probe_mfma(int iters, float *out, int blocks, void *stream)
{
    if (iters <= 0 || blocks <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError();
}
