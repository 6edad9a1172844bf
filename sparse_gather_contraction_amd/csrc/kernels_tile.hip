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
//     A stage's rows and records travel by direct global -> LDS loads, all issued before one wait
//     (its metadata is read first, into registers, so no global load waits behind them).
//   * Records are read as LDS broadcasts.  Per record a lane reads its c + kTileT - 1 window
//     values once and issues c x G x kTileT multiply-adds (longitude-shift reuse); records of an
//     item are grouped by c, one branch-free software-pipelined loop per c.
// Each output element is summed by one lane (or by WS lanes, added in a fixed order) in record
// order and written once: no atomics, the result is bitwise reproducible.
#include <cstddef>

#include "common.hpp"
#include "kernels.hpp"
#include "plan_tile.hpp"

namespace disco {

namespace {

constexpr int kThreads = 256;
constexpr int T = kTileT;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef void __attribute__((address_space(3))) *lptr_t;

// Raw buffer resource over `bytes` bytes at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Direct global -> LDS loads (buffer_load_dword / _dwordx4 ... lds): lane i of the instruction
// writes LDS base `l` + 4 i (dma4) or + 16 i (dma16); lanes outside the exec mask write nothing.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *l)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *l)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l, 16, voff, 0, 0, 0);
}

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
// planes takes every WS-th record of each class.  bounds (bounds_hi): lane q holds the stage's record
// bound q (q + 64) (global record index; item-major, then by entry count), `base` = i kTileClasses; rb:
// the stage's first record (LDS index 0).
template <int G>
__device__ __forceinline__ void run_item(const TileRec *lrec, const char *lane, int jlc, int wrap, int bounds,
                                         int bounds_hi, int base, int rb, int wsi, int WS, float (&acc)[G][T])
{
    constexpr int CM = tile_piece_max(G);
    int p[kTileClasses + 1];
#pragma unroll
    for (int q = 0; q <= kTileClasses; ++q) {
        const int idx = base + q;  // a constant once the item loop is unrolled
        p[q] = (idx < 64 ? __builtin_amdgcn_readlane(bounds, idx) : __builtin_amdgcn_readlane(bounds_hi, idx - 64)) - rb;
    }
    run_class<1, G>(lrec, lane, jlc, wrap, p[0] + wsi, p[1], WS, acc);
    run_class<2, G>(lrec, lane, jlc, wrap, p[1] + wsi, p[2], WS, acc);
    run_class<3, G>(lrec, lane, jlc, wrap, p[2] + wsi, p[3], WS, acc);
    if constexpr (CM >= 4) run_class<4, G>(lrec, lane, jlc, wrap, p[3] + wsi, p[4], WS, acc);
    if constexpr (CM >= 5) run_class<5, G>(lrec, lane, jlc, wrap, p[4] + wsi, p[5], WS, acc);
    if constexpr (CM >= 6) run_class<6, G>(lrec, lane, jlc, wrap, p[5] + wsi, p[6], WS, acc);
    if constexpr (CM >= 7) run_class<7, G>(lrec, lane, jlc, wrap, p[6] + wsi, p[7], WS, acc);
    if constexpr (CM >= 8) run_class<8, G>(lrec, lane, jlc, wrap, p[7] + wsi, p[8], WS, acc);
}

// Queue records [rb, re) of the stage into LDS (16-byte direct loads spread over the workgroup).
__device__ __forceinline__ void dma_recs(const TileLaunch &a, unsigned char *lrec, int rb, int re, int wave, int lane)
{
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.recs, (uint32_t)a.n_recs * (uint32_t)sizeof(TileRec));
    const int n = 4 * (re - rb);
    for (int u0 = 64 * wave; u0 < n; u0 += 256) {
        const int u = u0 + lane;
        if (u < n) dma16(rs, (uint32_t)sizeof(TileRec) * (uint32_t)rb + 16u * (uint32_t)u, lrec + 16 * u0);
    }
}

// Queue the stage's source rows of the workgroup's NPB planes into LDS by direct loads (source rows
// 16-byte aligned, L >= kTileHalo).  LDS row positions 0 .. L + kTileHalo - 1 of a plane's row: with
// deint = 1 position j holds row element j mod L (16-byte loads, one per four positions); with
// deint = 2 the two residue rows rho = 0, 1 hold elements 2 (j mod L) + rho (4-byte loads, lane j of
// an instruction writing position j, so the even/odd split costs no register traffic).  (Row, plane)
// pairs go round the four waves.  rows_v: lane r holds the stage's source row r.
__device__ __forceinline__ void dma_band(const TileLaunch &a, float *lds, int rows_v, int nrows, int plane0, int NPB,
                                         int wave, int lane)
{
    const int stage_floats = a.rows_per_stage * a.deint * a.lrow;
    const uint32_t plane_bytes = 4u * (uint32_t)a.src_plane;
    const int lg = __builtin_ctz((unsigned)NPB);  // NPB = 4 PW / WS is a power of two
    for (int rp = wave; rp < (nrows << lg); rp += 4) {  // (row, plane) pairs round the waves
        const int r = rp >> lg, ps = rp & (NPB - 1);
        if (plane0 + ps >= a.BC) continue;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.src + (int64_t)(plane0 + ps) * a.src_plane, plane_bytes);
        const uint32_t row0 = 4u * (uint32_t)(__builtin_amdgcn_readlane(rows_v, r) * a.row_len);
        float *drow = lds + ps * stage_floats + r * a.deint * a.lrow;
        if (a.deint == 1) {
            const int U = a.row_len >> 2, UH = U + kTileHalo / 4;
            for (int u0 = 0; u0 < UH; u0 += 64) {
                const int u = u0 + lane;
                const int ug = u < U ? u : u - U;
                if (u < UH) dma16(rs, row0 + 16u * (uint32_t)ug, drow + 4 * u0);
            }
        } else {
            const int npos = a.L + kTileHalo;
            for (int rho = 0; rho < 2; ++rho)
                for (int j0 = 0; j0 < npos; j0 += 64) {
                    const int j = j0 + lane;
                    const int jg = j < a.L ? j : j - a.L;
                    if (j < npos) dma4(rs, row0 + 4u * (uint32_t)(2 * jg + rho), drow + rho * a.lrow + j0);
                }
        }
    }
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

// Copy the stage's source rows of the workgroup's NPB planes into LDS with ordinary loads and
// stores (source rows not 16-byte aligned, or L < kTileHalo).
__device__ __forceinline__ void stage_band(const TileLaunch &a, float *lds, const int32_t *__restrict__ rows,
                                           int nrows, int plane0, int NPB, int wave, int lane)
{
    const int stage_floats = a.rows_per_stage * a.deint * a.lrow;
    const int NRP = nrows * NPB;
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

// Per-workgroup constants of the stage loop.
struct StageCtx {
    int plane0, NPB, wave, lane;
    int ps, jlc;      // the lane's plane within the workgroup, first position (clamped into the row)
    int wsi, WS;      // the wave's share of the records, waves sharing the planes
    int stage_floats; // floats of one plane's rows in a stage buffer
};

// A stage's metadata, one load per lane: lane q holds record bound q (bounds_hi: q + 64; there are
// NI kTileClasses + 1 <= 65), lane r < nrows source row r (a stage has at most kTileMaxStageRows <= 64
// rows).  It is read before the stage is queued, so no global load waits behind the direct loads.
struct StageMeta {
    int bounds_v, bounds_hi, rows_v;
    int rb, re, nrows;
    int row_begin;  // into stage_rows (the plain copy path reads them there)
};

// From the stage's descriptor fields (row range in stage_rows, record bounds at stage_recptr + segptr).
template <int NI>
__device__ __forceinline__ StageMeta load_meta(const TileLaunch &a, int row_begin, int row_end, int segptr, int lane)
{
    const int32_t *rp = a.stage_recptr + uni(segptr);
    StageMeta m;
    m.row_begin = uni(row_begin);
    m.nrows = uni(row_end) - m.row_begin;
    m.bounds_v = lane <= NI * kTileClasses ? rp[lane] : 0;
    m.bounds_hi = (NI * kTileClasses >= 64 && lane + 64 <= NI * kTileClasses) ? rp[lane + 64] : 0;
    m.rows_v = lane < m.nrows ? a.stage_rows[m.row_begin + lane] : 0;
    m.rb = __builtin_amdgcn_readlane(m.bounds_v, 0);
    m.re = NI * kTileClasses < 64 ? __builtin_amdgcn_readlane(m.bounds_v, NI * kTileClasses)
                                  : __builtin_amdgcn_readlane(m.bounds_hi, NI * kTileClasses - 64);
    return m;
}

// Queue a stage into the stage buffer: direct loads for 16-byte aligned source rows, else ordinary
// copies; either way the data is in place after the issuing threads' waits and the next barrier.
template <int PW>
__device__ __forceinline__ void queue_stage(const TileLaunch &a, const StageCtx &sc, const StageMeta &m, float *buf)
{
    float *lrec = buf + 4 * PW * sc.stage_floats;
    if (a.vec) {
        dma_band(a, buf, m.rows_v, m.nrows, sc.plane0, sc.NPB, sc.wave, sc.lane);
        dma_recs(a, reinterpret_cast<unsigned char *>(lrec), m.rb, m.re, sc.wave, sc.lane);
    } else {
        stage_band(a, buf, a.stage_rows + m.row_begin, m.nrows, sc.plane0, sc.NPB, sc.wave, sc.lane);
        stage_recs(a, reinterpret_cast<TileRec *>(lrec), m.rb, m.re, threadIdx.x);
    }
}

// Contract the records of a stage in LDS (metadata m): LDS and registers only.
template <int NI, int G, int PW>
__device__ __forceinline__ void compute_stage(const TileLaunch &a, const StageCtx &sc, const StageMeta &m,
                                              const float *cur, float (&acc)[NI][G][T])
{
    const TileRec *lrec = reinterpret_cast<const TileRec *>(cur + 4 * PW * sc.stage_floats);
    const char *lane_base = reinterpret_cast<const char *>(cur + sc.ps * sc.stage_floats + sc.jlc);
#pragma unroll
    for (int i = 0; i < NI; ++i)
        run_item<G>(lrec, lane_base, sc.jlc, 4 * a.L, m.bounds_v, m.bounds_hi, i * kTileClasses, m.rb, sc.wsi, sc.WS,
                    acc[i]);
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
    // the first stage's descriptor needs only the task number: read beside the task, so the first
    // stage's metadata loads wait for one round trip instead of two (task, then its descriptors)
    Stage f0 = {0, 0, 0, 0};
    if (a.n_stages > 0) f0 = a.task_first[ti];
    const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wsi = wave % WS;    // this wave's share of the records
    const int ps = (wave / WS) * PW + (PW == 2 ? (lane >> 5) : 0);
    const int ql = PW == 2 ? (lane & 31) : lane;
    const int plane0 = pg * NPB;
    const int plane = plane0 + ps;
    const int jl = ql * T;
    const int jlc = jl < a.L ? jl : 0;  // lanes past the row read valid LDS, results dropped
    const int stage_floats = a.rows_per_stage * a.deint * a.lrow;

    float acc[NI][G][T];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[i][g][t] = 0.0f;

    // stage buffer: [rows of the 4 PW planes][records]
    float *buf = lds;
    const StageCtx sc{plane0, NPB, wave, lane, ps, jlc, wsi, WS, stage_floats};
    // the task's items, read now so the epilogue waits on no load: lane q < 8 NI holds 32-bit word q of
    // items [item_begin, item_begin + NI) (out_stride is word 3, out_off[g] word 4 + g of an item)
    static_assert(sizeof(Item) == 32 && offsetof(Item, out_stride) == 12 && offsetof(Item, out_off) == 16,
                  "item layout");
    const int32_t *itw = reinterpret_cast<const int32_t *>(a.items + task.item_begin);
    const int items_v = lane < 8 * NI ? itw[lane] : 0;
    // The task's stage descriptors, read now (lane j: stage stage_begin + j), so that a stage's metadata
    // loads depend on no other load; each stage's metadata is read while the previous stage's loads are
    // in flight, so a stage costs one global round trip (its direct loads) before its contraction.
    const int sb = uni(task.stage_begin), se = uni(task.stage_end);
    const int4 sv = lane < se - sb ? reinterpret_cast<const int4 *>(a.stages + sb)[lane] : make_int4(0, 0, 0, 0);
    auto meta_of = [&](int st) {
        const int j = uni(st - sb);
        if (j < 64)
            return load_meta<NI>(a, __builtin_amdgcn_readlane(sv.x, j), __builtin_amdgcn_readlane(sv.y, j),
                                 __builtin_amdgcn_readlane(sv.z, j), lane);
        const Stage sg = a.stages[uni(st)];  // tasks of more than 64 stages
        return load_meta<NI>(a, sg.row_begin, sg.row_end, sg.segptr, lane);
    };
    static_assert(sizeof(Stage) == 16, "stage layout: row_begin, row_end, segptr, pad");
    StageMeta m = {};
    if (a.n_stages > 0) m = load_meta<NI>(a, f0.row_begin, f0.row_end, f0.segptr, lane);  // stage sb, if any
    for (int st = sb; st < se; ++st) {
        __syncthreads();  // the previous stage is consumed
        queue_stage<PW>(a, sc, m, buf);
        const StageMeta mn = st + 1 < se ? meta_of(st + 1) : m;
        __builtin_amdgcn_s_waitcnt(0);  // this thread's loads have landed
        __syncthreads();                // everyone's have
        compute_stage<NI, G, PW>(a, sc, m, buf, acc);
        m = mn;
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
            const int out_stride = __builtin_amdgcn_readlane(items_v, 8 * i + 3);
            if (__builtin_amdgcn_readlane(items_v, 8 * i + 4) < 0) continue;  // padding item
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int out_off = __builtin_amdgcn_readlane(items_v, 8 * i + 4 + g);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int j = jl + t;
                    if (j < a.L) dp[(int64_t)out_off + (int64_t)out_stride * j] = acc[i][g][t];
                }
            }
        }
    }
}

template <int NI, int G, int PW>
hipError_t launch_one(const TileLaunch &a, int64_t nblk, size_t lds, hipStream_t stream)
{
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&tile_gather_kernel<NI, G, PW>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tile_gather_kernel<NI, G, PW>), dim3((unsigned)nblk), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
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
    return a.PW == 2 ? launch_one<NI, G, 2>(a, nblk, lds, stream) : launch_one<NI, G, 1>(a, nblk, lds, stream);
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
