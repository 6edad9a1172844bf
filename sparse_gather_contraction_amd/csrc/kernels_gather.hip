// kernels_gather.hip — strided circular-correlation gather for gfx950.
//
// One kernel serves the forward CSR contraction and the atomic-free transpose
// (the backward gathers per input pixel over the row-inverted psi; see
// plan.hpp for how both map onto segments).  Per block: one work item (a
// group of G destination rows that share a segment list) for one (b, c)
// plane.  Segment headers and values are block-uniform and live in scalar
// registers (the index loads are amortised over all lanes, the role the
// channel tiling plays on the page's CUDA backward, section "BC_TILE
// optimization").  Lanes own destination positions j; each lane keeps G x T
// fp32 accumulators and sums its terms serially in segment order, so the
// result is deterministic and every destination element is written once.
#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace disco {

constexpr int kGatherThreads = 256;

template <int G, int T, typename TI, typename TO>
__device__ __forceinline__ void gather_item(const TI *__restrict__ src, TO *__restrict__ dst, const Item &it,
                                            const Seg *__restrict__ segs, const float *__restrict__ vals,
                                            int L, int in_stride)
{
    const int tid = threadIdx.x;
    for (int wb = 0; wb < L; wb += kGatherThreads * T) {
        float acc[G][T];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int u = 0; u < T; ++u) acc[g][u] = 0.0f;
        for (int q = it.seg_begin; q < it.seg_end; ++q) {
            const Seg sg = segs[q];
            const float *v = vals + sg.val_off;
            const TI *row = src + sg.in_off;
            for (int t = 0; t < sg.m; ++t) {
                int base = sg.j0 + t;
                if (base >= L) base -= L;
                float vv[G];
#pragma unroll
                for (int g = 0; g < G; ++g) vv[g] = v[t * G + g];
#pragma unroll
                for (int u = 0; u < T; ++u) {
                    const int j = wb + tid + kGatherThreads * u;
                    if (j < L) {
                        int idx = base + j;
                        if (idx >= L) idx -= L;
                        const float xv = load_elem(row, (int64_t)in_stride * idx);
#pragma unroll
                        for (int g = 0; g < G; ++g) acc[g][u] = fmaf(vv[g], xv, acc[g][u]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < T; ++u) {
            const int j = wb + tid + kGatherThreads * u;
            if (j < L) {
#pragma unroll
                for (int g = 0; g < G; ++g) store_elem(dst, (int64_t)it.out_off[g] + (int64_t)it.out_stride * j, acc[g][u]);
            }
        }
    }
}

template <int T, typename TI, typename TO>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(const TI *__restrict__ src, TO *__restrict__ dst,
                                                                const Item *__restrict__ items,
                                                                const int32_t *__restrict__ order,
                                                                const Seg *__restrict__ segs,
                                                                const float *__restrict__ vals, int BC,
                                                                int64_t src_plane, int64_t dst_plane, int L,
                                                                int in_stride)
{
    const int ii = blockIdx.x / BC;
    const int bc = blockIdx.x - ii * BC;
    const Item it = items[order[ii]];
    src += (int64_t)bc * src_plane;
    dst += (int64_t)bc * dst_plane;
    switch (it.G) {
    case 1: gather_item<1, T>(src, dst, it, segs, vals, L, in_stride); break;
    case 2: gather_item<2, T>(src, dst, it, segs, vals, L, in_stride); break;
    case 3: gather_item<3, T>(src, dst, it, segs, vals, L, in_stride); break;
    default: gather_item<4, T>(src, dst, it, segs, vals, L, in_stride); break;
    }
}

template <typename TI, typename TO>
static hipError_t launch_typed(const GatherLaunch &a, hipStream_t stream)
{
    const int per = (a.L + kGatherThreads - 1) / kGatherThreads;
    dim3 grid((unsigned)((int64_t)a.n_items * a.BC)), block(kGatherThreads);
    const TI *src = (const TI *)a.src;
    TO *dst = (TO *)a.dst;
#define DISCO_GATHER_LAUNCH(TT)                                                                          \
    hipLaunchKernelGGL((gather_kernel<TT, TI, TO>), grid, block, 0, stream, src, dst, a.items, a.order, \
                       a.segs, a.vals, a.BC, a.src_plane, a.dst_plane, a.L, a.in_stride)
    if (per <= 1) DISCO_GATHER_LAUNCH(1);
    else if (per == 2) DISCO_GATHER_LAUNCH(2);
    else if (per == 3) DISCO_GATHER_LAUNCH(3);
    else DISCO_GATHER_LAUNCH(4);
#undef DISCO_GATHER_LAUNCH
    return hipGetLastError();
}

hipError_t launch_gather(const GatherLaunch &a, hipStream_t stream)
{
    if (a.n_items == 0 || a.BC == 0) return hipSuccess;
    if (a.dtype == 1) return launch_typed<bf16_t, bf16_t>(a, stream);
    if (a.dtype == 2) return launch_typed<f16_t, f16_t>(a, stream);
    return launch_typed<float, float>(a, stream);
}

}  // namespace disco
