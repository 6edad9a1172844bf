// kernels_tile.hip — register-tiled fp32 gather for gfx950 (forward CSR contraction, and the
// backward as a gather over the row-inverted psi; torch-harmonics "disco-kernel-dev" page,
// "Architecture snapshot" and "Backward direction — gather vs scatter").
//
// Workgroup = one task (every destination row of one output latitude, or of the longitude
// residues of one input row) x NPB channel planes, four waves.  A wave serves PW planes (PW = 2:
// each half-wave owns one plane); a lane owns kTileT consecutive positions of its plane and keeps
// NI x G x kTileT fp32 accumulators in registers for the whole task.  Tasks much heavier than the
// mean split their records over WS = 2 or 4 waves that share the same planes (then NPB =
// 4 PW / WS) and add their partial sums in wave order at the end.
//   * Per stage the task's source rows are copied to LDS (a forward input row split by
//     longitude residue, s = 2: even and odd columns, so a segment reads consecutive words; every
//     LDS row carries a wrap halo so no index needs a modulo inside a record), and so are the
//     stage's records (64 bytes: window offset, wrap threshold, entry count c, values [c][G]).
//   * Records are read as LDS broadcasts.  Per record a lane reads its c + kTileT - 1 window
//     values once and issues c x G x kTileT multiply-adds (longitude-shift reuse); records of an
//     item are grouped by c, one branch-free software-pipelined loop per c.
// Each output element is summed by one lane (or by WS lanes, added in a fixed order) in record
// order and written once: no atomics, the result is bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"
#include "plan_tile.hpp"

namespace disco {

namespace {

constexpr int kThreads = 256;
constexpr int T = kTileT;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One class of records (all with C entries) of one item: a branch-free loop, software-pipelined
// and unrolled by two so that two sets of registers (window, values, header) alternate without
// copies.  The step of record r issues the header read of record r + 2 step, the window reads and
// the value reads of record r + step, and only then the C x G x kTileT multiply-adds of record r,
// whose window and values arrived during the previous step: the LDS latency overlaps the
// arithmetic.  Records sit in LDS, so every read is an in-order LDS read and each wait leaves the
// newest reads in flight; prefetch indices are clamped to the last record, so every read is of a
// valid record.  The empty asm statements with a memory clobber keep each step's reads ahead of
// its multiply-adds.
//   lrec: the stage's records (index r - rb); lane: the lane's window base (bytes: plane buffer +
//   4 x first position); wrap: 4 L, taken off when the lane's first position reaches the record's
//   threshold.
template <int C, int G>
__device__ __forceinline__ void run_class(const TileRec *lrec, const char *lane, int jlc, int wrap, int r, int r1,
                                          int step, float (&acc)[G][T])
{
    r = uni(r);
    r1 = uni(r1);
    step = uni(step);
    if (r >= r1) return;
    constexpr int NW = C + T - 1, NV = C * G;
    const int last = r1 - 1;
    auto hdr = [&](int idx, int &a, int &w) {
        const int2 h = *reinterpret_cast<const int2 *>(&lrec[uni(idx)].a);
        a = h.x;
        w = h.y;
    };
    auto vals = [&](int idx, float (&v)[NV]) {
        const float4 *vp = reinterpret_cast<const float4 *>(&lrec[uni(idx)].v[0]);
#pragma unroll
        for (int q4 = 0; q4 < (NV + 3) / 4; ++q4) {
            const float4 f = vp[q4];
            if (4 * q4 + 0 < NV) v[4 * q4 + 0] = f.x;
            if (4 * q4 + 1 < NV) v[4 * q4 + 1] = f.y;
            if (4 * q4 + 2 < NV) v[4 * q4 + 2] = f.z;
            if (4 * q4 + 3 < NV) v[4 * q4 + 3] = f.w;
        }
    };
    auto window = [&](int a, int w, float (&win)[NW]) {
        const float *p = reinterpret_cast<const float *>(lane + a - (jlc >= w ? wrap : 0));
#pragma unroll
        for (int u = 0; u < NW; ++u) win[u] = p[u];
    };
    auto fma_all = [&](const float (&v)[NV], const float (&win)[NW]) {
#pragma unroll
        for (int e = 0; e < C; ++e)
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int t = 0; t < T; ++t) acc[g][t] = fmaf(v[e * G + g], win[e + t], acc[g][t]);
    };
    int aa, wa, ab, wb;
    float va[NV], vb[NV], xa[NW], xb[NW];
    hdr(r, aa, wa);
    vals(r, va);
    window(aa, wa, xa);
    hdr(min(r + step, last), ab, wb);
    for (;;) {
        // current: (va, xa); header of the next record in (ab, wb)
        hdr(min(r + 2 * step, last), aa, wa);
        window(ab, wb, xb);
        vals(min(r + step, last), vb);
        __asm__ volatile("" ::: "memory");
        fma_all(va, xa);
        r += step;
        if (r >= r1) break;
        // current: (vb, xb); header of the next record in (aa, wa)
        hdr(min(r + 2 * step, last), ab, wb);
        window(aa, wa, xa);
        vals(min(r + step, last), va);
        __asm__ volatile("" ::: "memory");
        fma_all(vb, xb);
        r += step;
        if (r >= r1) break;
    }
}

// Records of item i in one stage: one loop per entry count; wave `wsi` of the WS waves sharing the
// planes takes every WS-th record of each class.  ptr: the item's class bounds (global record
// indices); rb: the stage's first record (LDS index 0).
template <int G>
__device__ __forceinline__ void run_item(const TileRec *lrec, const char *lane, int jlc, int wrap,
                                         const int32_t *__restrict__ ptr, int rb, int wsi, int WS, float (&acc)[G][T])
{
    constexpr int CM = tile_piece_max(G);
    int p[kTileClasses + 1];
#pragma unroll
    for (int q = 0; q <= kTileClasses; ++q) p[q] = uni(ptr[q] - rb);
    run_class<1, G>(lrec, lane, jlc, wrap, p[0] + wsi, p[1], WS, acc);
    run_class<2, G>(lrec, lane, jlc, wrap, p[1] + wsi, p[2], WS, acc);
    run_class<3, G>(lrec, lane, jlc, wrap, p[2] + wsi, p[3], WS, acc);
    if constexpr (CM >= 4) run_class<4, G>(lrec, lane, jlc, wrap, p[3] + wsi, p[4], WS, acc);
    if constexpr (CM >= 5) run_class<5, G>(lrec, lane, jlc, wrap, p[4] + wsi, p[5], WS, acc);
    if constexpr (CM >= 6) run_class<6, G>(lrec, lane, jlc, wrap, p[5] + wsi, p[6], WS, acc);
    if constexpr (CM >= 7) run_class<7, G>(lrec, lane, jlc, wrap, p[6] + wsi, p[7], WS, acc);
    if constexpr (CM >= 8) run_class<8, G>(lrec, lane, jlc, wrap, p[7] + wsi, p[8], WS, acc);
}

// Copy records [rb, re) of the stage to LDS (16-byte units; the loads of a batch are issued
// together, their indices clamped to the range).
__device__ __forceinline__ void stage_recs(const TileLaunch &a, TileRec *lrec, int rb, int re, int tid)
{
    const float4 *src = reinterpret_cast<const float4 *>(a.recs + rb);
    float4 *dst = reinterpret_cast<float4 *>(lrec);
    const int n = 4 * (re - rb);
    for (int u0 = 0; u0 < n; u0 += 4 * 256) {
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[min(u0 + 256 * k + tid, n - 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int u = u0 + 256 * k + tid;
            if (u < n) dst[u] = v[k];
        }
    }
}

// Copy the stage's source rows of the workgroup's NPB planes into LDS (all four waves).  Vector
// path (rows 16-byte aligned, L >= kTileHalo): a (row, plane) pair is row_len / 4 units of 16
// bytes plus the halo units (the row's first kTileHalo positions again: 4 units, or 8 when a
// forward row splits into two residue rows); a wave takes two pairs at a time and issues all
// their loads before any LDS write, so the loads are in flight together.
__device__ __forceinline__ void stage_band(const TileLaunch &a, float *lds, const int32_t *__restrict__ rows,
                                           int nrows, int plane0, int NPB, int wave, int lane)
{
    const int stage_floats = a.rows_per_stage * a.deint * a.lrow;
    const int NRP = nrows * NPB;
    if (a.vec) {
        const int U = a.row_len >> 2;
        const int UH = U + (a.deint == 1 ? kTileHalo / 4 : kTileHalo / 2);
        for (int rp0 = wave; rp0 < NRP; rp0 += 8) {
            float4 v[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rp = rp0 + 4 * j;
                const int r = rp / NPB, ps = rp - r * NPB;
                const bool ok = rp < NRP && plane0 + ps < a.BC;
                const float *srow = a.src + (int64_t)(plane0 + ps) * a.src_plane +
                                    (int64_t)(ok ? rows[r] : 0) * a.row_len;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int u = lane + 64 * k;
                    const int ug = u < U ? u : u - U;
                    if (ok && u < UH) v[j][k] = *reinterpret_cast<const float4 *>(srow + 4 * ug);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rp = rp0 + 4 * j;
                const int r = rp / NPB, ps = rp - r * NPB;
                if (!(rp < NRP && plane0 + ps < a.BC)) continue;
                float *drow = lds + ps * stage_floats + r * a.deint * a.lrow;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int u = lane + 64 * k;
                    if (u >= UH) continue;
                    if (a.deint == 1) {
                        const int d = u < U ? 4 * u : a.L + 4 * (u - U);
                        *reinterpret_cast<float4 *>(drow + d) = v[j][k];
                    } else {
                        const int d = u < U ? 2 * u : a.L + 2 * (u - U);
                        *reinterpret_cast<float2 *>(drow + d) = make_float2(v[j][k].x, v[j][k].z);
                        *reinterpret_cast<float2 *>(drow + a.lrow + d) = make_float2(v[j][k].y, v[j][k].w);
                    }
                }
            }
        }
        return;
    }
    for (int rp = wave; rp < NRP; rp += 4) {
        const int r = rp / NPB, ps = rp - r * NPB;
        const int plane = plane0 + ps;
        if (plane >= a.BC) continue;
        const float *srow = a.src + (int64_t)plane * a.src_plane + (int64_t)rows[r] * a.row_len;
        float *drow = lds + ps * stage_floats + r * a.deint * a.lrow;
        for (int e = lane; e < a.row_len; e += 64) {
            const int rho = a.deint == 1 ? 0 : (e & 1);
            const int jj = a.deint == 1 ? e : (e >> 1);
            drow[rho * a.lrow + jj] = srow[e];
        }
        // wrap halo: positions L .. L + kTileHalo - 1 repeat positions 0 .. kTileHalo - 1 (mod L)
        for (int h = lane; h < a.deint * kTileHalo; h += 64) {
            const int rho = h / kTileHalo, pos = h % kTileHalo;
            int jj = pos;
            while (jj >= a.L) jj -= a.L;
            drow[rho * a.lrow + a.L + pos] = srow[rho + a.deint * jj];
        }
    }
}

template <int NI, int G, int PW>
__global__ __launch_bounds__(kThreads) void tile_gather_kernel(TileLaunch a)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    // workgroup -> (task, plane group, WS): tasks [0, n_ws4) split their records over 4 waves,
    // [n_ws4, n_ws2) over 2, the rest give each wave its own PW planes
    int bid = blockIdx.x, ti, pg, WS;
    {
        const int npg4 = (a.BC + PW - 1) / PW, npg2 = (a.BC + 2 * PW - 1) / (2 * PW);
        const int npg1 = (a.BC + 4 * PW - 1) / (4 * PW);
        const int nb4 = a.n_ws4 * npg4, nb2 = (a.n_ws2 - a.n_ws4) * npg2;
        if (bid < nb4) {
            WS = 4; ti = bid / npg4; pg = bid - ti * npg4;
        } else if (bid < nb4 + nb2) {
            bid -= nb4;
            WS = 2; ti = a.n_ws4 + bid / npg2; pg = bid - (ti - a.n_ws4) * npg2;
        } else {
            bid -= nb4 + nb2;
            WS = 1; ti = a.n_ws2 + bid / npg1; pg = bid - (ti - a.n_ws2) * npg1;
        }
    }
    ti = uni(ti);
    pg = uni(pg);
    WS = uni(WS);
    const int NPB = 4 * PW / WS;  // planes of this workgroup
    const Task task = a.tasks[ti];
    const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wsi = wave % WS;    // this wave's share of the records
    const int ps = (wave / WS) * PW + (PW == 2 ? (lane >> 5) : 0);
    const int ql = PW == 2 ? (lane & 31) : lane;
    const int plane0 = pg * NPB;
    const int plane = plane0 + ps;
    const int jl = ql * T;
    const int jlc = jl < a.L ? jl : 0;  // lanes past the row read valid LDS, results dropped
    const int stage_floats = a.rows_per_stage * a.deint * a.lrow;
    const float *my = lds + ps * stage_floats;

    float acc[NI][G][T];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[i][g][t] = 0.0f;

    TileRec *lrec = reinterpret_cast<TileRec *>(lds + 4 * PW * stage_floats);  // after the row area
    const char *lane_base = reinterpret_cast<const char *>(my + jlc);
    for (int st = task.stage_begin; st < task.stage_end; ++st) {
        const Stage sg = a.stages[uni(st)];
        const int32_t *rp = a.stage_recptr + sg.segptr;
        const int rb = uni(rp[0]), re = uni(rp[NI * kTileClasses]);
        __syncthreads();  // the previous stage is consumed
        stage_band(a, lds, a.stage_rows + sg.row_begin, sg.row_end - sg.row_begin, plane0, NPB, wave, lane);
        stage_recs(a, lrec, rb, re, threadIdx.x);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NI; ++i)
            run_item<G>(lrec, lane_base, jlc, 4 * a.L, rp + i * kTileClasses, rb, wsi, WS, acc[i]);
    }

    if (WS > 1) {
        // waves 1 .. WS-1 of each group hand their partial sums to wave 0 of the group through LDS,
        // which adds them in wave order
        constexpr int NA = NI * G * T;
        __syncthreads();  // every wave is done with the stage buffers
        float *red = lds + (size_t)(wave - 1) * 64 * NA;
        if (wsi != 0) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int t = 0; t < T; ++t) red[((i * G + g) * T + t) * 64 + lane] = acc[i][g][t];
        }
        __syncthreads();
        if (wsi != 0) return;
        for (int k = 1; k < WS; ++k) {
            const float *src = lds + (size_t)(wave + k - 1) * 64 * NA;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int t = 0; t < T; ++t) acc[i][g][t] += src[((i * G + g) * T + t) * 64 + lane];
        }
    }

    if (plane < a.BC) {
        float *dp = a.dst + (int64_t)plane * a.dst_plane;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const Item it = a.items[task.item_begin + i];
            if (it.out_off[0] < 0) continue;  // padding item
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int j = jl + t;
                    if (j < a.L) dp[(int64_t)it.out_off[g] + (int64_t)it.out_stride * j] = acc[i][g][t];
                }
        }
    }
}

template <int NI, int G>
hipError_t launch_pw(const TileLaunch &a, hipStream_t stream)
{
    const int64_t PW = a.PW;
    const int64_t nblk = (int64_t)a.n_ws4 * ((a.BC + PW - 1) / PW) +
                         (int64_t)(a.n_ws2 - a.n_ws4) * ((a.BC + 2 * PW - 1) / (2 * PW)) +
                         (int64_t)(a.n_tasks - a.n_ws2) * ((a.BC + 4 * PW - 1) / (4 * PW));
    const size_t stage = (size_t)4 * a.PW * a.rows_per_stage * a.deint * a.lrow * sizeof(float) +
                         (size_t)a.max_recs * sizeof(TileRec);
    const size_t red = a.n_ws2 > 0 ? (size_t)3 * 64 * NI * G * T * sizeof(float) : 0;
    const size_t lds = stage > red ? stage : red;
    if (a.PW == 2)
        hipLaunchKernelGGL((tile_gather_kernel<NI, G, 2>), dim3((unsigned)nblk), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((tile_gather_kernel<NI, G, 1>), dim3((unsigned)nblk), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

bool tile_supported(int NI, int G, int PW)
{
    if (PW != 1 && PW != 2) return false;
    if (G == 1) return NI == 1 || NI == 2 || NI == 4 || NI == 8;
    if (G == 2) return NI == 1 || NI == 2 || NI == 4;
    return (G == 3 || G == 4) && (NI == 1 || NI == 2);
}

hipError_t launch_tile(const TileLaunch &a, hipStream_t stream)
{
    if (a.n_tasks == 0 || a.BC == 0) return hipSuccess;
    switch (a.G) {
    case 1:
        if (a.NI == 1) return launch_pw<1, 1>(a, stream);
        if (a.NI == 2) return launch_pw<2, 1>(a, stream);
        if (a.NI == 4) return launch_pw<4, 1>(a, stream);
        return launch_pw<8, 1>(a, stream);
    case 2:
        if (a.NI == 1) return launch_pw<1, 2>(a, stream);
        if (a.NI == 2) return launch_pw<2, 2>(a, stream);
        return launch_pw<4, 2>(a, stream);
    case 3:
        if (a.NI == 1) return launch_pw<1, 3>(a, stream);
        return launch_pw<2, 3>(a, stream);
    default:
        if (a.NI == 1) return launch_pw<1, 4>(a, stream);
        return launch_pw<2, 4>(a, stream);
    }
}

}  // namespace disco
