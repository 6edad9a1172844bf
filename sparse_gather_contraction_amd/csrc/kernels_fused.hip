// kernels_fused.hip — fused DISCO convolution for gfx950.
//
// y[b,o,ho,wo] = sum_{c,k} W[o,c,k] * out[b,c,k,ho,wo]  ("contraction + einsum",
// torch-harmonics "disco-kernel-dev" page, "Architecture snapshot").
//
// The (B,C,K,Ho,Wo) contraction is never written to device memory.  A block
// owns one (b, ho) latitude, a tile of kPx output longitudes and a block of
// kOBlk output channels.  It walks the input channels in chunks whose
// (c, k) rows fill kR reduction rows: the chunk is contracted on the vector
// ALUs (fp32, serial per element, the forward plan's segments), rounded to
// the data type (bf16 or fp16) into LDS as a [pixel][c*K + k] tile, and then
// multiplied on the matrix cores: v_mfma_f32_16x16x32_{bf16,f16} with W as the
// A operand (16 o x 32 rows) and the LDS tile as the B operand (32 rows x 16
// pixels), fp32 accumulation in registers across all chunks.  fp32 data keeps
// the chunk in fp32 and runs the einsum on v_mfma_f32_16x16x4_f32.
#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace disco {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kPx = 64;        // output longitudes per block
constexpr int kOBlk = 256;     // output channels per block (64 per wave)
constexpr int kR = 64;         // reduction rows (c*K + k) per chunk: two MFMA k-steps
constexpr int kLdsStride = kR + 8;  // 16-bit elements per pixel row in LDS (16-byte aligned rows)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-bit data types of the kernel: storage, raw bits, and the matching MFMA.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
    static __device__ __forceinline__ short bits(bf16_t v) { return (short)v; }
    static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Elem<f16_t> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ float to_f32(f16_t v) { return (float)v; }
    static __device__ __forceinline__ f16_t from_f32(float v) { return (f16_t)v; }
    static __device__ __forceinline__ short bits(f16_t v) { return __builtin_bit_cast(short, v); }
    static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <> struct Elem<float> {  // fp32 data (the contraction's loads and tile; the einsum has its own kernel)
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};

// NB entries of a segment from entry t, for NP channel planes at once: the NB * NP x loads go out
// together, then the multiply-adds in entry order; base = (j0 + t + wo) mod Wo on entry, advanced past
// the NB entries.
template <int NB, int NP, int G, typename T>
__device__ __forceinline__ void contract_batch(const T *const (&row)[NP], const float *__restrict__ v, int t, int &base,
                                               int Wo, int in_stride, const bool (&valid)[NP],
                                               float (&acc)[NP][kMaxGroup])
{
    float xv[NP][NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        int idx = base + u;
        while (idx >= Wo) idx -= Wo;
#pragma unroll
        for (int p = 0; p < NP; ++p) xv[p][u] = valid[p] ? Elem<T>::to_f32(row[p][(int64_t)in_stride * idx]) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float w = v[(t + u) * G + g];
#pragma unroll
            for (int p = 0; p < NP; ++p) acc[p][g] = fmaf(w, xv[p][u], acc[p][g]);
        }
    base += NB;
    while (base >= Wo) base -= Wo;
}

// One item of the forward plan for NP channel planes at longitude wo: acc[p][g] = row g of the item,
// summed over its segments' entries in order.
template <int NP, int G, typename T>
__device__ __forceinline__ void contract_item(const T *const (&plane)[NP], const Item &it,
                                              const Seg *__restrict__ segs, const float *__restrict__ vals, int Wo,
                                              int in_stride, int wo, const bool (&valid)[NP],
                                              float (&acc)[NP][kMaxGroup])
{
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[p][g] = 0.0f;
    for (int q = it.seg_begin; q < it.seg_end; ++q) {
        const Seg sg = segs[q];
        const float *v = vals + sg.val_off;
        const T *row[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) row[p] = plane[p] + sg.in_off;
        int base = sg.j0 + wo;  // (j0 + t + wo) mod Wo at t = 0
        while (base >= Wo) base -= Wo;
        int t = 0;
        for (; t + 8 <= sg.m; t += 8) contract_batch<8, NP, G, T>(row, v, t, base, Wo, in_stride, valid, acc);
        if (t + 4 <= sg.m) {
            contract_batch<4, NP, G, T>(row, v, t, base, Wo, in_stride, valid, acc);
            t += 4;
        }
        if (t + 2 <= sg.m) {
            contract_batch<2, NP, G, T>(row, v, t, base, Wo, in_stride, valid, acc);
            t += 2;
        }
        if (t < sg.m) contract_batch<1, NP, G, T>(row, v, t, base, Wo, in_stride, valid, acc);
    }
}

// The chunk's contraction (channels c0 .. c0 + ccn - 1) into the LDS tile [pixel][c K + k] (S: the
// tile's element type, STRIDE its row length): per pass over eight of the chunk's channels, thread
// (cl, px) handles channels cl and cl + 4 at longitude wo0 + px — two independent chains of loads in
// flight — and writes the tile type's rounding of each sum.
template <typename T, typename S, int STRIDE>
__device__ __forceinline__ void contract_chunk(const T *__restrict__ xb, S *__restrict__ tile,
                                               const Item *__restrict__ items, const Seg *__restrict__ segs,
                                               const float *__restrict__ vals, int it_begin, int it_end,
                                               int64_t plane_sz, int c0, int ccn, int CC, int K, int Wo, int HoWo,
                                               int in_stride, int wo0, int tid)
{
    static_assert(kThreads == 4 * kPx, "four channels of kPx pixels per thread row");
    constexpr int NP = 2;
    const int cl0 = tid / kPx, px = tid - cl0 * kPx;
    const int wo = wo0 + px;
    for (int cb = 0; cb < CC; cb += 4 * NP) {
        const T *plane[NP];
        bool valid[NP];
        int cl[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            cl[p] = cb + cl0 + 4 * p;
            valid[p] = cl[p] < ccn && wo < Wo;
            plane[p] = xb + (int64_t)(c0 + (cl[p] < ccn ? cl[p] : 0)) * plane_sz;
        }
        for (int ii = it_begin; ii < it_end; ++ii) {
            const Item it = items[ii];
            float a[NP][kMaxGroup];
            switch (it.G) {
            case 1: contract_item<NP, 1, T>(plane, it, segs, vals, Wo, in_stride, wo, valid, a); break;
            case 2: contract_item<NP, 2, T>(plane, it, segs, vals, Wo, in_stride, wo, valid, a); break;
            case 3: contract_item<NP, 3, T>(plane, it, segs, vals, Wo, in_stride, wo, valid, a); break;
            default: contract_item<NP, 4, T>(plane, it, segs, vals, Wo, in_stride, wo, valid, a); break;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (cl[p] < CC) {
                    for (int g = 0; g < it.G; ++g) {
                        const int k = it.out_off[g] / HoWo;
                        tile[px * STRIDE + cl[p] * K + k] = Elem<S>::from_f32(valid[p] ? a[p][g] : 0.0f);
                    }
                }
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fused_kernel(const T *__restrict__ x, const T *__restrict__ W,
                                                         T *__restrict__ y, const Item *__restrict__ items,
                                                         const int32_t *__restrict__ block_ptr,
                                                         const int32_t *__restrict__ ho_order,
                                                         const Seg *__restrict__ segs, const float *__restrict__ vals,
                                                         int B, int C, int Co, int K, int Ho, int Wo, int Hi, int Wi,
                                                         int in_stride, int n_pt, int n_ob)
{
    typedef typename Elem<T>::vec8 vec8;
    __shared__ __attribute__((aligned(16))) T tile[kPx * kLdsStride];

    int bid = blockIdx.x;
    const int pt = bid % n_pt;
    bid /= n_pt;
    const int ob = bid % n_ob;
    bid /= n_ob;
    const int b = bid % B;
    const int ho = ho_order[bid / B];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wo0 = pt * kPx;
    const int o_base = ob * kOBlk + wave * 64;
    const int CC = kR / K;  // channels per chunk (host guarantees K <= kR)
    const int64_t plane_sz = (int64_t)Hi * Wi;
    const int it_begin = block_ptr[ho], it_end = block_ptr[ho + 1];
    const int HoWo = Ho * Wo;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < C; c0 += CC) {
        const int ccn = min(CC, C - c0);
        __syncthreads();  // the previous chunk's MFMA reads of `tile` are done
        // ---- contraction of channels [c0, c0+ccn) into tile[px][cl*K + k] ----
        contract_chunk<T, T, kLdsStride>(x + (int64_t)b * C * plane_sz, tile, items, segs, vals, it_begin, it_end,
                                         plane_sz, c0, ccn, CC, K, Wo, HoWo, in_stride, wo0, tid);
        // rows past the chunk's (c, k) range are zero
        for (int e = tid; e < kPx * kR; e += kThreads) {
            const int px = e / kR, r = e - px * kR;
            if (r >= ccn * K) tile[px * kLdsStride + r] = Elem<T>::from_f32(0.0f);
        }
        __syncthreads();
        // ---- einsum on the matrix cores ----
        const int rvalid = ccn * K;
#pragma unroll
        for (int ks = 0; ks < kR / 32; ++ks) {
            const int rr0 = ks * 32 + 8 * (lane >> 4);
            vec8 bop[4];
#pragma unroll
            for (int p4 = 0; p4 < 4; ++p4) {
                const int px = p4 * 16 + (lane & 15);
                bop[p4] = *reinterpret_cast<const vec8 *>(&tile[px * kLdsStride + rr0]);
            }
#pragma unroll
            for (int ot = 0; ot < 4; ++ot) {
                const int o = o_base + ot * 16 + (lane & 15);
                i16x8 av;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int rr = rr0 + i;
                    av[i] = (o < Co && rr < rvalid) ? Elem<T>::bits(W[((int64_t)o * C + c0) * K + rr]) : (short)0;
                }
                const vec8 aop = __builtin_bit_cast(vec8, av);
#pragma unroll
                for (int p4 = 0; p4 < 4; ++p4)
                    acc[ot][p4] = Elem<T>::mfma(aop, bop[p4], acc[ot][p4]);
            }
        }
    }
    // ---- epilogue: D[row = o][col = pixel]; lane holds col lane&15, rows 4*(lane>>4)+a ----
#pragma unroll
    for (int ot = 0; ot < 4; ++ot)
#pragma unroll
        for (int p4 = 0; p4 < 4; ++p4)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int o = o_base + ot * 16 + 4 * (lane >> 4) + a;
                const int wo = wo0 + p4 * 16 + (lane & 15);
                if (o < Co && wo < Wo) y[(((int64_t)b * Co + o) * Ho + ho) * Wo + wo] = Elem<T>::from_f32(acc[ot][p4][a]);
            }
}

// fp32 data: the same block structure with an fp32 contraction tile and the einsum on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32: A = W, 16 output channels x 4 rows; B = the tile, 4 rows x
// 16 pixels), fp32 products and accumulation throughout.  W arrives packed in A-operand order
// (launch_pack_wa_f32): an A operand spans 16 output channels whose W rows lie C K floats apart, so
// loading it from W itself would touch 16 cache lines per 4-byte load.

// Packed W for fused_f32_kernel: for chunk t (channels c0 = t CC .. + CC - 1, CC = kR / K), 16-channel
// output tile o16, step quadruple kq and lane l, the float4 Wa[((t n_ot16 + o16) (kR / 16) + kq) 64 + l]
// holds, for j = 0..3, W[o][c0 K + rr] with o = 16 o16 + l % 16 and rr = 4 (4 kq + j) + l / 16 — the A
// operand of step 4 kq + j for that lane — and zero where o >= Co or rr reaches past the chunk's
// channels.
__global__ __launch_bounds__(256) void pack_wa_f32_kernel(const float *__restrict__ W, float *__restrict__ Wa, int Co,
                                                          int C, int K, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int j = (int)(i & 3), l = (int)((i >> 2) & 63), kq = (int)((i >> 8) % (kR / 16));
    const int64_t rest = (i >> 8) / (kR / 16);
    const int n_ot16 = (Co + 15) / 16;
    const int o16 = (int)(rest % n_ot16);
    const int t = (int)(rest / n_ot16);
    const int CC = kR / K, c0 = t * CC, ccn = min(CC, C - c0);
    const int o = 16 * o16 + (l & 15), rr = 4 * (4 * kq + j) + (l >> 4);
    Wa[i] = (o < Co && rr < ccn * K) ? W[((int64_t)o * C + c0) * K + rr] : 0.0f;
}
constexpr int kLdsStride32 = kR + 4;  // floats per pixel row (the 16 lanes of a row group hit distinct banks)

__global__ __launch_bounds__(kThreads) void fused_f32_kernel(const float *__restrict__ x, const float4 *__restrict__ Wa,
                                                             float *__restrict__ y, const Item *__restrict__ items,
                                                             const int32_t *__restrict__ block_ptr,
                                                             const int32_t *__restrict__ ho_order,
                                                             const Seg *__restrict__ segs,
                                                             const float *__restrict__ vals, int B, int C, int Co,
                                                             int K, int Ho, int Wo, int Hi, int Wi, int in_stride,
                                                             int n_pt, int n_ob)
{
    __shared__ __attribute__((aligned(16))) float tile[kPx * kLdsStride32];

    int bid = blockIdx.x;
    const int pt = bid % n_pt;
    bid /= n_pt;
    const int ob = bid % n_ob;
    bid /= n_ob;
    const int b = bid % B;
    const int ho = ho_order[bid / B];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wo0 = pt * kPx;
    const int o_base = ob * kOBlk + wave * 64;
    const int CC = kR / K;
    const int n_ot16 = (Co + 15) / 16;
    const int64_t plane_sz = (int64_t)Hi * Wi;
    const int it_begin = block_ptr[ho], it_end = block_ptr[ho + 1];
    const int HoWo = Ho * Wo;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < C; c0 += CC) {
        const int ccn = min(CC, C - c0);
        __syncthreads();  // the previous chunk's MFMA reads of `tile` are done
        contract_chunk<float, float, kLdsStride32>(x + (int64_t)b * C * plane_sz, tile, items, segs, vals, it_begin,
                                                   it_end, plane_sz, c0, ccn, CC, K, Wo, HoWo, in_stride, wo0, tid);
        for (int e = tid; e < kPx * kR; e += kThreads) {
            const int px = e / kR, r = e - px * kR;
            if (r >= ccn * K) tile[px * kLdsStride32 + r] = 0.0f;
        }
        __syncthreads();
        const int rl = lane >> 4;  // the lane's row within a 4-row step
        // A operands of the chunk's 16 steps: W packed by launch_pack_wa_f32, one 16-byte load per lane and
        // output-channel tile for four steps (zeros past Co and past the chunk's ccn K rows)
        const float4 *wq = Wa + (int64_t)(c0 / CC) * n_ot16 * (kR / 16) * 64 + lane;
#pragma unroll
        for (int kq = 0; kq < kR / 16; ++kq) {
            float4 aq[4];
#pragma unroll
            for (int ot = 0; ot < 4; ++ot) {
                const int o16 = (o_base >> 4) + ot;
                aq[ot] = o16 < n_ot16 ? wq[((int64_t)o16 * (kR / 16) + kq) * 64] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = (4 * kq + j) * 4 + rl;
                float bop[4];
#pragma unroll
                for (int p4 = 0; p4 < 4; ++p4) bop[p4] = tile[(p4 * 16 + (lane & 15)) * kLdsStride32 + rr];
#pragma unroll
                for (int ot = 0; ot < 4; ++ot) {
                    const float aop = j == 0 ? aq[ot].x : j == 1 ? aq[ot].y : j == 2 ? aq[ot].z : aq[ot].w;
#pragma unroll
                    for (int p4 = 0; p4 < 4; ++p4)
                        acc[ot][p4] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, bop[p4], acc[ot][p4], 0, 0, 0);
                }
            }
        }
    }
    // D[row = o][col = pixel]: lane holds col lane & 15, rows 4 (lane >> 4) + a
#pragma unroll
    for (int ot = 0; ot < 4; ++ot)
#pragma unroll
        for (int p4 = 0; p4 < 4; ++p4)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int o = o_base + ot * 16 + 4 * (lane >> 4) + a;
                const int wo = wo0 + p4 * 16 + (lane & 15);
                if (o < Co && wo < Wo) y[(((int64_t)b * Co + o) * Ho + ho) * Wo + wo] = acc[ot][p4][a];
            }
}

}  // namespace

hipError_t launch_fused(const FusedLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.Co == 0) return hipSuccess;
    const int n_pt = (a.Wo + kPx - 1) / kPx;
    const int n_ob = (a.Co + kOBlk - 1) / kOBlk;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_ob * n_pt;
    if (a.f32) {
        if (!a.Wa && a.C > 0) return hipErrorInvalidValue;  // the fp32 kernel takes W packed (launch_pack_wa_f32)
        hipLaunchKernelGGL(fused_f32_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, (const float *)a.x,
                           (const float4 *)a.Wa, (float *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals, a.B,
                           a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob);
    } else if (a.f16)
        hipLaunchKernelGGL(fused_kernel<f16_t>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, (const f16_t *)a.x,
                           (const f16_t *)a.W, (f16_t *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals, a.B,
                           a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob);
    else
        hipLaunchKernelGGL(fused_kernel<bf16_t>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, (const bf16_t *)a.x,
                           (const bf16_t *)a.W, (bf16_t *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals, a.B,
                           a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob);
    return hipGetLastError();
}

int64_t fused_wa_f32_floats(int Co, int C, int K)
{
    if (K < 1 || K > kR) return 0;
    const int64_t CC = kR / K, n_chunks = (C + CC - 1) / CC, n_ot16 = (Co + 15) / 16;
    return n_chunks * n_ot16 * (kR / 16) * 64 * 4;
}

hipError_t launch_pack_wa_f32(const float *W, float *Wa, int Co, int C, int K, hipStream_t stream)
{
    const int64_t total = fused_wa_f32_floats(Co, C, K);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_wa_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, W, Wa, Co, C, K,
                       total);
    return hipGetLastError();
}

int fused_max_k() { return kR; }

}  // namespace disco
