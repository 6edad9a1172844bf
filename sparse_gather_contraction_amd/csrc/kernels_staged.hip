// kernels_staged.hip — LDS-staged circular-correlation gather for gfx950.
//
// Same primitive as kernels_gather.hip (forward CSR contraction, and the
// backward as a gather over the row-inverted psi), organised so that every
// source value read from LDS feeds several FMAs:
//   * a block runs one task (NI items, G rows each) on NP planes; its source
//     rows (the latitude band of x, or the (k, ho) band of gout) are copied
//     to LDS in stages with 16-byte coalesced loads, each row followed by a
//     wrap halo so a circular index never needs a modulo inside a segment;
//   * a lane owns T consecutive output positions.  A segment of m <= 8
//     entries needs the m + T - 1 consecutive source values starting at the
//     lane's first position; they are read once into registers and used for
//     all m*T*G multiply-adds (longitude-shift reuse, and rows that share a
//     support reuse each value G times);
//   * segment headers and values are block-uniform (scalar loads), one
//     fully unrolled body per segment length.
// Every output element is accumulated by one lane, serially in segment
// order: results are deterministic and no atomics are used.
#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace disco {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float lds_to_f32(const float *p) { return *p; }
__device__ __forceinline__ float lds_to_f32(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float lds_to_f32(const f16_t *p) { return (float)*p; }

template <int G, int T, int S, int M, typename TI>
__device__ __forceinline__ void seg_body(const TI *p, const float *__restrict__ v, float (&acc)[G][T])
{
    float w[M + T - 1];
#pragma unroll
    for (int q = 0; q < M + T - 1; ++q) w[q] = lds_to_f32(p + S * q);
#pragma unroll
    for (int s = 0; s < M; ++s) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float vv = v[s * G + g];
#pragma unroll
            for (int t = 0; t < T; ++t) acc[g][t] = fmaf(vv, w[s + t], acc[g][t]);
        }
    }
}

template <int G, int T, int S, typename TI>
__device__ __forceinline__ void run_segments(const TI *lds_plane, const Seg *__restrict__ segs,
                                             const float *__restrict__ vals, int q0, int q1, int jl, int L,
                                             float (&acc)[G][T])
{
    for (int q = q0; q < q1; ++q) {
        const Seg sg = segs[q];
        int base = sg.j0 + jl;
        if (base >= L) base -= L;
        const TI *p = lds_plane + sg.in_off + S * base;
        const float *v = vals + sg.val_off;
        switch (sg.m) {
        case 1: seg_body<G, T, S, 1>(p, v, acc); break;
        case 2: seg_body<G, T, S, 2>(p, v, acc); break;
        case 3: seg_body<G, T, S, 3>(p, v, acc); break;
        case 4: seg_body<G, T, S, 4>(p, v, acc); break;
        case 5: seg_body<G, T, S, 5>(p, v, acc); break;
        case 6: seg_body<G, T, S, 6>(p, v, acc); break;
        case 7: seg_body<G, T, S, 7>(p, v, acc); break;
        default: seg_body<G, T, S, 8>(p, v, acc); break;
        }
    }
}

// Copy the stage's source rows of every plane of the block into LDS.
// Rows are split over the 4 waves; lanes copy 16-byte chunks (or single
// elements when the rows are not 16-byte aligned).
template <typename TI>
__device__ __forceinline__ void stage_rows(TI *lds, const TI *__restrict__ src, const int32_t *__restrict__ rows,
                                           int nrows, int NP, int plane0, int BC, int64_t src_plane, int row_len,
                                           int copy_len, int lrow, int stage_elems, bool vec)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    constexpr int CH = 16 / (int)sizeof(TI);
    for (int ps = 0; ps < NP; ++ps) {
        const int plane = plane0 + ps;
        if (plane >= BC) break;
        const TI *sp = src + (int64_t)plane * src_plane;
        TI *dp = lds + ps * stage_elems;
        for (int r = wave; r < nrows; r += 4) {
            const TI *srow = sp + (int64_t)rows[r] * row_len;
            TI *drow = dp + r * lrow;
            if (vec) {
                const int nch = copy_len / CH;
                for (int c = lane; c < nch; c += 64) {
                    int e = c * CH;
                    while (e >= row_len) e -= row_len;
                    *reinterpret_cast<uint4 *>(drow + c * CH) = *reinterpret_cast<const uint4 *>(srow + e);
                }
            } else {
                for (int c = lane; c < copy_len; c += 64) {
                    int e = c;
                    while (e >= row_len) e -= row_len;
                    drow[c] = srow[e];
                }
            }
        }
    }
}

template <int NI, int G, int T, int S, typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void staged_gather_kernel(
    const TI *__restrict__ src, TO *__restrict__ dst, const Task *__restrict__ tasks, const Stage *__restrict__ stages,
    const int32_t *__restrict__ stage_rows_g, const int32_t *__restrict__ stage_segptr, const Seg *__restrict__ segs,
    const float *__restrict__ vals, const Item *__restrict__ items, int BC, int n_pg, int64_t src_plane,
    int64_t dst_plane, int L, int row_len, int copy_len, int lrow, int wpp, int NP, int stage_elems, int vec)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    TI *lds = reinterpret_cast<TI *>(smem);

    const int ti = blockIdx.x / n_pg;
    const int pg = blockIdx.x - ti * n_pg;
    const Task task = tasks[ti];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int pslot = wave / wpp;
    const int plane = pg * NP + pslot;
    const bool plane_ok = plane < BC;
    const int jl = (wave - pslot * wpp) * 64 * T + lane * T;  // first output position of this lane
    const int jlc = jl < L ? jl : 0;                         // idle lanes read valid LDS, results dropped
    const TI *my_lds = lds + pslot * stage_elems;

    float acc[NI][G][T];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[i][g][t] = 0.0f;

    for (int st = task.stage_begin; st < task.stage_end; ++st) {
        const Stage sg = stages[st];
        __syncthreads();  // previous stage fully consumed
        stage_rows<TI>(lds, src, stage_rows_g + sg.row_begin, sg.row_end - sg.row_begin, NP, pg * NP, BC, src_plane,
                       row_len, copy_len, lrow, stage_elems, vec != 0);
        __syncthreads();
        if (plane_ok) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                run_segments<G, T, S, TI>(my_lds, segs, vals, stage_segptr[sg.segptr + i],
                                          stage_segptr[sg.segptr + i + 1], jlc, L, acc[i]);
        }
    }

    if (plane_ok && jl < L) {
        TO *dp = dst + (int64_t)plane * dst_plane;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const Item it = items[task.item_begin + i];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int j = jl + t;
                    if (j < L) store_elem(dp, (int64_t)it.out_off[g] + (int64_t)it.out_stride * j, acc[i][g][t]);
                }
        }
    }
}

template <int NI, int G, int T, int S, typename TI, typename TO>
hipError_t launch_one(const StagedLaunch &a, hipStream_t stream)
{
    const int n_pg = (a.BC + a.NP - 1) / a.NP;
    const int64_t nblk = (int64_t)a.n_tasks * n_pg;
    const size_t lds = (size_t)a.NP * a.stage_elems * sizeof(TI);
    hipLaunchKernelGGL((staged_gather_kernel<NI, G, T, S, TI, TO>), dim3((unsigned)nblk), dim3(kThreads), lds, stream,
                       (const TI *)a.src, (TO *)a.dst, a.tasks, a.stages, a.stage_rows, a.stage_segptr, a.segs, a.vals,
                       a.items, a.BC, n_pg, a.src_plane, a.dst_plane, a.L, a.row_len, a.copy_len, a.lrow, a.wpp, a.NP,
                       a.stage_elems, a.vec);
    return hipGetLastError();
}

template <int NI, int G, int T, typename TI, typename TO>
hipError_t dispatch_s(const StagedLaunch &a, hipStream_t stream)
{
    if (a.S == 1) return launch_one<NI, G, T, 1, TI, TO>(a, stream);
    return launch_one<NI, G, T, 2, TI, TO>(a, stream);
}

template <int NI, int G, typename TI, typename TO>
hipError_t dispatch_t(const StagedLaunch &a, hipStream_t stream)
{
    if (a.T == 3) return dispatch_s<NI, G, 3, TI, TO>(a, stream);
    return dispatch_s<NI, G, 6, TI, TO>(a, stream);
}

template <typename TI, typename TO>
hipError_t dispatch_typed(const StagedLaunch &a, hipStream_t stream)
{
    if (a.NI == 2) return dispatch_t<2, 1, TI, TO>(a, stream);
    switch (a.G) {
    case 1: return dispatch_t<1, 1, TI, TO>(a, stream);
    case 2: return dispatch_t<1, 2, TI, TO>(a, stream);
    case 3: return dispatch_t<1, 3, TI, TO>(a, stream);
    default: return dispatch_t<1, 4, TI, TO>(a, stream);
    }
}

}  // namespace

bool staged_supported(int NI, int G, int T, int S)
{
    const bool ni_g = (NI == 1 && G >= 1 && G <= 4) || (NI == 2 && G == 1);
    return ni_g && (T == 3 || T == 6) && (S == 1 || S == 2);
}

hipError_t launch_staged(const StagedLaunch &a, hipStream_t stream)
{
    if (a.n_tasks == 0 || a.BC == 0) return hipSuccess;
    if (a.dtype == 1) return dispatch_typed<bf16_t, bf16_t>(a, stream);
    if (a.dtype == 2) return dispatch_typed<f16_t, f16_t>(a, stream);
    return dispatch_typed<float, float>(a, stream);
}

}  // namespace disco
