// probes.hip — microbenchmarks of what the gfx950 device reaches on this machine, for the benchmark's
// "achievable" figures beside the published peaks (libdisco_probes.so; not part of the DISCO
// library).  Each probe is a plain kernel with a fixed, in-bounds access pattern:
//   * read stream: every element of a device buffer read once with 16-byte loads (grid-stride,
//     four loads in flight per lane), summed so the loads are kept; one float per workgroup out;
//   * copy: the same stream written to a second buffer (read + write bytes);
//   * fp32 FMA loop: eight independent v_fmac_f32 chains per lane (packed fp32 ops are disabled
//     in this build, as in the library);
//   * bf16 MFMA loop: four independent v_mfma_f32_32x32x16_bf16 accumulators per wave;
//   * LDS read loop: 4-, 8- or 16-byte LDS reads per lane over a 64 KiB array, consecutive lanes
//     on consecutive words (no bank conflicts), eight waves per workgroup, one workgroup per CU;
//   * direct global -> LDS read stream: every 16-byte unit of a buffer loaded once with
//     buffer_load_dwordx4 ... lds into a per-wave LDS ring, at most `inflight` loads in flight per
//     wave (the path the library's stage loads take);
//   * direct global -> LDS row-piece stream: the buffer read as `rows` rows of equal length, each
//     workgroup step taking one `piece`-byte piece of every row at the workgroup's column tile (the
//     shape of a GEMM operand tile whose rows lie far apart), four waves, double-buffered steps;
//   * LDS-fed MFMA loop: per step two 16-byte reads and `nb32` 4-byte reads per lane feeding two
//     v_mfma_f32_32x32x16_bf16 (the operand traffic of a contraction block of the fused kernel:
//     one psi operand in 4-byte words, the x runs of two channels), loads issued one step ahead.
#include <hip/hip_runtime.h>
#include <cstdint>

extern "C" {
hipError_t disco_probe_read(const void *buf, size_t bytes, float *out, int blocks, void *stream);
hipError_t disco_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream);
hipError_t disco_probe_fma(int iters, float *out, int blocks, void *stream);
hipError_t disco_probe_mfma(int iters, float *out, int blocks, void *stream);
hipError_t disco_probe_lds(int iters, int width, float *out, int blocks, void *stream);
hipError_t disco_probe_lds_mfma(int iters, int nb32, float *out, int blocks, void *stream);
hipError_t disco_probe_lds_mfma_q(int iters, int p, int q, int depth, int threads, float *out, int blocks, void *stream);
hipError_t disco_probe_dma_read(const void *buf, size_t bytes, int inflight, int blocks, void *stream);
hipError_t disco_probe_dma_rows(const void *buf, size_t bytes, int rows, int piece, int blocks, void *stream);
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

constexpr int kLdsThreads = 512;
constexpr int kLdsBytes = 65536;

// Fills the array with lane-dependent words; every later read address is masked into it.
__device__ __forceinline__ void fill_lds(uint32_t *lds)
{
    for (int i = threadIdx.x; i < kLdsBytes / 4; i += kLdsThreads) lds[i] = 0x9e3779b9u * (uint32_t)(i + 1);
    __syncthreads();
}

template <int W>
__global__ __launch_bounds__(kLdsThreads) void lds_kernel(int iters, float *out)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    fill_lds(lds);
    const unsigned char *base = reinterpret_cast<const unsigned char *>(lds);
    const uint32_t lane_off = (uint32_t)(threadIdx.x & 63) * W + (uint32_t)(threadIdx.x >> 6) * 4096u;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t off = (lane_off + (uint32_t)(8 * it + u) * 64u * W) & (kLdsBytes - 1);
            if constexpr (W == 16) {
                const uint4 v = *reinterpret_cast<const uint4 *>(base + off);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            } else if constexpr (W == 8) {
                const uint2 v = *reinterpret_cast<const uint2 *>(base + off);
                acc ^= v.x ^ v.y;
            } else {
                acc ^= *reinterpret_cast<const uint32_t *>(base + off);
            }
        }
    }
    out[blockIdx.x * kLdsThreads + threadIdx.x] = (float)acc;
}

template <int NB32>
__global__ __launch_bounds__(kLdsThreads) void lds_mfma_kernel(int iters, float *out)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    fill_lds(lds);
    const unsigned char *base = reinterpret_cast<const unsigned char *>(lds);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // x runs: 16 bytes per lane, consecutive lanes 16 bytes apart; psi words: 4 bytes per lane,
    // consecutive lanes 4 bytes apart, NB32 words 256 bytes apart
    const uint32_t xo = (uint32_t)lane * 16u + (uint32_t)wave * 2048u, ao = 32768u + (uint32_t)lane * 4u + (uint32_t)wave * 1024u;
    f32x16 d0 = {}, d1 = {};
    auto ld = [&](int it, bf16x8 &b0, bf16x8 &b1, uint32_t (&a)[NB32]) {
        const uint32_t step = (uint32_t)(it & 7) * 1024u;
        b0 = *reinterpret_cast<const bf16x8 *>(base + ((xo + step) & 32767u));
        b1 = *reinterpret_cast<const bf16x8 *>(base + ((xo + step + 16384u) & 32767u));
#pragma unroll
        for (int i = 0; i < NB32; ++i)
            a[i] = *reinterpret_cast<const uint32_t *>(base + (32768u | ((ao + step + 256u * i) & 32767u)));
    };
    bf16x8 b0, b1, nb0, nb1;
    uint32_t a[NB32], na[NB32];
    ld(0, b0, b1, a);
    for (int it = 0; it < iters; ++it) {
        ld(it + 1, nb0, nb1, na);
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = NB32 > 4 ? __builtin_amdgcn_perm(a[(i + 1) % NB32], a[i], 0x05040302u) : a[i];
        const bf16x8 av = __builtin_bit_cast(bf16x8, w);
        d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, d1, 0, 0, 0);
        b0 = nb0;
        b1 = nb1;
#pragma unroll
        for (int i = 0; i < NB32; ++i) a[i] = na[i];
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += d0[k] + d1[k];
    out[blockIdx.x * kLdsThreads + threadIdx.x] = t;
}

// P psi operands (phase pairs) x Q x operands (channels): per step 4P four-byte psi reads and Q
// 16-byte x reads per lane feed P Q MFMAs; operands are loaded DEPTH steps ahead.  TH threads per
// workgroup.
template <int P, int Q, int DEPTH, int TH>
__global__ __launch_bounds__(TH) void lds_mfma_q_kernel(int iters, float *out)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    for (int i = threadIdx.x; i < kLdsBytes / 4; i += TH) lds[i] = 0x9e3779b9u * (uint32_t)(i + 1);
    __syncthreads();
    const unsigned char *base = reinterpret_cast<const unsigned char *>(lds);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t xo = (uint32_t)lane * 16u + (uint32_t)wave * 2048u, ao = (uint32_t)lane * 4u + (uint32_t)wave * 1024u;
    f32x16 d[P][Q];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int c = 0; c < Q; ++c) d[p][c] = f32x16{};
    bf16x8 b[DEPTH][Q];
    uint32_t a[DEPTH][P][4];
    auto ld = [&](int it, bf16x8 (&bb)[Q], uint32_t (&aa)[P][4]) {
        const uint32_t step = (uint32_t)(it & 7) * 1024u;
#pragma unroll
        for (int c = 0; c < Q; ++c) bb[c] = *reinterpret_cast<const bf16x8 *>(base + ((xo + step + 4096u * c) & 32767u));
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                aa[p][i] = *reinterpret_cast<const uint32_t *>(base + (32768u | ((ao + step + 256u * i + 4096u * p) & 32767u)));
    };
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) ld(j, b[j], a[j]);
    for (int it = 0; it < iters; it += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, a[j][p]);
#pragma unroll
                for (int c = 0; c < Q; ++c) d[p][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[j][c], d[p][c], 0, 0, 0);
            }
            ld(it + j + DEPTH, b[j], a[j]);
        }
    }
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int c = 0; c < Q; ++c)
#pragma unroll
            for (int k = 0; k < 16; ++k) t += d[p][c][k];
    out[blockIdx.x * TH + threadIdx.x] = t;
}

typedef void __attribute__((address_space(3))) *lds_ptr_t;

// Wave w of a workgroup streams 1 KiB units u = (blockIdx * waves + w) + k * (gridDim * waves) of the
// buffer into LDS slot k % RING of its own 16 KiB area; the wait before each load keeps at most
// INFL - 1 older loads in flight.  The buffer resource bounds every read (units past the end read 0).
template <int INFL>
__global__ __launch_bounds__(256) void dma_read_kernel(const void *buf, uint32_t bytes, uint32_t n_units)
{
    constexpr int RING = 16;
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * RING * 1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(buf), 0, (int)bytes, 0x00020000);
    const uint32_t stride = gridDim.x * 4u;
    uint32_t u = blockIdx.x * 4u + (uint32_t)wave;
    unsigned char *area = lds + wave * RING * 1024;
    for (int k = 0; u < n_units; ++k, u += stride) {
        if constexpr (INFL == 4) __builtin_amdgcn_s_waitcnt(0x0f73);  // vmcnt <= 3
        else if constexpr (INFL == 8) __builtin_amdgcn_s_waitcnt(0x0f77);  // vmcnt <= 7
        else __builtin_amdgcn_s_waitcnt(0x0f7f);  // vmcnt <= 15
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(area + 1024 * (k % RING)), 16, u * 1024u + 16u * (uint32_t)lane, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// Workgroup g walks column tiles g, g + gridDim, ... of a row-major buffer of `rows` rows of
// `row_bytes` bytes: per tile it loads the `piece` bytes at column tile * piece of every row into its
// LDS stage — the tile's pieces taken as one run of 16-byte lane units, 1 KiB per wave instruction,
// waves in turn (with 512-byte pieces a wave instruction covers two rows) — keeping at most 15 loads
// in flight per wave.  Every offset is below rows * row_bytes; LDS offsets wrap inside the stage.
__global__ __launch_bounds__(256) void dma_rows_kernel(const void *buf, uint32_t bytes, int rows, uint32_t row_bytes,
                                                       int piece, int n_tiles)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][32768];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(buf), 0, (int)bytes, 0x00020000);
    const int n_inst = rows * piece / 1024;
    int k = 0;
    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x, ++k) {
        unsigned char *stage = lds[k & 1];
        for (int u = wave; u < n_inst; u += 4) {
            __builtin_amdgcn_s_waitcnt(0x0f7f);  // vmcnt <= 15: bounded in flight
            const uint32_t b = 1024u * (uint32_t)u + 16u * (uint32_t)lane;  // byte in the tile's run of pieces
            const uint32_t r = b / (uint32_t)piece, w = b - r * (uint32_t)piece;
            const uint32_t off = r * row_bytes + (uint32_t)tile * (uint32_t)piece + w;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + ((1024 * u) & 32767)), 16, off, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
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

// width: 4, 8 or 16 bytes per lane per read; out holds blocks * 512 floats.  Each workgroup
// performs iters * 8 reads per lane.
hipError_t disco_probe_lds(int iters, int width, float *out, int blocks, void *stream)
{
    if (iters <= 0 || blocks <= 0) return hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
    if (width == 4) hipLaunchKernelGGL(lds_kernel<4>, dim3(blocks), dim3(kLdsThreads), 0, st, iters, out);
    else if (width == 8) hipLaunchKernelGGL(lds_kernel<8>, dim3(blocks), dim3(kLdsThreads), 0, st, iters, out);
    else if (width == 16) hipLaunchKernelGGL(lds_kernel<16>, dim3(blocks), dim3(kLdsThreads), 0, st, iters, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// nb32: 4 (aligned psi words) or 5 (realigned); two MFMAs per iteration per wave; out holds
// blocks * 512 floats.
hipError_t disco_probe_lds_mfma(int iters, int nb32, float *out, int blocks, void *stream)
{
    if (iters <= 0 || blocks <= 0) return hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
    if (nb32 == 4) hipLaunchKernelGGL(lds_mfma_kernel<4>, dim3(blocks), dim3(kLdsThreads), 0, st, iters, out);
    else if (nb32 == 5) hipLaunchKernelGGL(lds_mfma_kernel<5>, dim3(blocks), dim3(kLdsThreads), 0, st, iters, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// p psi operands x q channels per step (see the kernel), prefetch depth, threads 256 or 512; iters a
// multiple of depth; p q MFMAs per iteration per wave; out holds blocks * threads floats.
hipError_t disco_probe_lds_mfma_q(int iters, int p, int q, int depth, int threads, float *out, int blocks, void *stream)
{
    if (iters <= 0 || blocks <= 0 || depth <= 0 || iters % depth != 0) return hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
#define PROBE_Q(PP, QQ, DD, TT)                                                                                  \
    if (p == PP && q == QQ && depth == DD && threads == TT) {                                                    \
        hipLaunchKernelGGL((lds_mfma_q_kernel<PP, QQ, DD, TT>), dim3(blocks), dim3(TT), 0, st, iters, out);      \
        return hipGetLastError();                                                                                \
    }
    PROBE_Q(1, 2, 2, 512) PROBE_Q(1, 4, 2, 512) PROBE_Q(2, 2, 2, 512) PROBE_Q(2, 1, 2, 512)
    PROBE_Q(1, 4, 2, 256) PROBE_Q(2, 2, 2, 256) PROBE_Q(2, 4, 2, 256) PROBE_Q(4, 2, 2, 256) PROBE_Q(4, 4, 2, 256)
    PROBE_Q(2, 4, 1, 256) PROBE_Q(4, 1, 2, 256) PROBE_Q(4, 1, 2, 512)
#undef PROBE_Q
    return hipErrorInvalidValue;
}

// bytes: a multiple of 1024 below 2^32; inflight 4, 8 or 16; 256 threads per workgroup.
hipError_t disco_probe_dma_read(const void *buf, size_t bytes, int inflight, int blocks, void *stream)
{
    if (bytes % 1024 != 0 || bytes >= ((size_t)1 << 32) || blocks <= 0 || (uintptr_t)buf % 16 != 0) return hipErrorInvalidValue;
    const hipStream_t st = (hipStream_t)stream;
    const uint32_t n = (uint32_t)(bytes / 1024);
    if (inflight == 4) hipLaunchKernelGGL(dma_read_kernel<4>, dim3(blocks), dim3(256), 0, st, buf, (uint32_t)bytes, n);
    else if (inflight == 8) hipLaunchKernelGGL(dma_read_kernel<8>, dim3(blocks), dim3(256), 0, st, buf, (uint32_t)bytes, n);
    else if (inflight == 16) hipLaunchKernelGGL(dma_read_kernel<16>, dim3(blocks), dim3(256), 0, st, buf, (uint32_t)bytes, n);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// rows x (bytes / rows) buffer read in pieces of `piece` bytes (a multiple of 16 dividing the row
// length, rows * piece a multiple of 1024); bytes below 2^32.
hipError_t disco_probe_dma_rows(const void *buf, size_t bytes, int rows, int piece, int blocks, void *stream)
{
    if (rows <= 0 || piece <= 0 || piece % 16 != 0 || ((int64_t)rows * piece) % 1024 != 0 || bytes >= ((size_t)1 << 32) ||
        bytes % rows != 0 || blocks <= 0)
        return hipErrorInvalidValue;
    const size_t row_bytes = bytes / rows;
    if (row_bytes % piece != 0 || (uintptr_t)buf % 16 != 0) return hipErrorInvalidValue;
    const int n_tiles = (int)(row_bytes / piece);
    hipLaunchKernelGGL(dma_rows_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, buf, (uint32_t)bytes, rows,
                       (uint32_t)row_bytes, piece, n_tiles);
    return hipGetLastError();
}
