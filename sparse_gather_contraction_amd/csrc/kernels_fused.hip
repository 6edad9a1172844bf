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
// the chunk in fp32 and runs the einsum on v_mfma_f32_16x16x4_f32.  Both take W
// packed per call in their A-operand order, and their contraction reads x from
// per-latitude source windows staged in LDS for each chunk and the latitude's psi
// from an LDS copy made once per block (plan.hpp, FusedWindows).
#include <algorithm>
#include <climits>

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
// fp32: LDS for a chunk's source windows and for the latitude's psi (the kernel's registers allow two
// workgroups per CU, which up to 80 KiB of LDS per workgroup keeps); these budgets hold whole-ring
// windows of 360x720 grids, so no latitude falls back to per-entry global reads, which would leave a
// tail of polar workgroups longer than the rest of the launch
constexpr int kFusedWinBytes = 36 * 1024;
constexpr int kFusedPsiBytes = 24 * 1024;

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

typedef void __attribute__((address_space(3))) *lptr_t;

// Raw buffer resource over `bytes` bytes at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// The chunk's source windows (plan.hpp, FusedWindows) into LDS by direct global -> LDS loads, one load per
// staged position into a 4-byte slot (4-byte loads for fp32 data, 2-byte loads for 16-bit data, whose value
// is the slot's low half); (row, channel) pairs go round the four waves, lane l of an instruction writing
// position q0 + l.  win: [channel][wl slots]; xb: the batch's channel planes.
template <typename T>
__device__ __forceinline__ void stage_fwin(const T *__restrict__ xb, uint32_t *win, const FWin *__restrict__ rows,
                                           int r0, int r1, int wl, int64_t plane_sz, int c0, int ccn, int Wo,
                                           int in_stride, int wo0, int wave, int lane)
{
    constexpr int E = sizeof(T);
    const int nj = (r1 - r0) * ccn;
    for (int job = wave; job < nj; job += kThreads / 64) {
        const int r = r0 + job / ccn, cl = job - (job / ccn) * ccn;
        const FWin w = rows[r];
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(xb + (int64_t)(c0 + cl) * plane_sz, E * (uint32_t)plane_sz);
        for (int q0 = 0; q0 < w.len; q0 += 64) {
            const int q = q0 + lane;
            const int idx = (w.a + wo0 + q) % Wo;
            const uint32_t voff = E * (uint32_t)(w.in_off + in_stride * idx);
            lptr_t dst = (lptr_t)(win + cl * wl + w.base + q0);
            if (q < w.len) {
                if constexpr (E == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
                else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 2, voff, 0, 0, 0);
            }
        }
    }
}

// The value of a staged window slot (T: the data type).
template <typename T>
__device__ __forceinline__ float slot_val(uint32_t w)
{
    if constexpr (sizeof(T) == 4) return __uint_as_float(w);
    else return Elem<T>::to_f32(__builtin_bit_cast(T, (unsigned short)w));
}

// The chunk's contraction from the staged windows: as contract_chunk, but a segment's entry t at pixel px
// reads window position seg_off + t + px of its channel (no modulo, no global load).
template <int NB, int NP, int G, typename T>
__device__ __forceinline__ void contract_batch_win(const uint32_t *const (&lw)[NP], const float *__restrict__ v, int t,
                                                   int pos, float (&acc)[NP][kMaxGroup])
{
    float xv[NP][NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int p = 0; p < NP; ++p) xv[p][u] = slot_val<T>(lw[p][pos + u]);
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float w = v[(t + u) * G + g];
#pragma unroll
            for (int p = 0; p < NP; ++p) acc[p][g] = fmaf(w, xv[p][u], acc[p][g]);
        }
}

// segs, seg_off and vals hold the plan's segments from s_base and values from v_base (the whole plan, or
// the latitude's runs copied to LDS).
template <int NP, int G, typename T>
__device__ __forceinline__ void contract_item_win(const uint32_t *const (&lw)[NP], const Item &it,
                                                  const Seg *__restrict__ segs, const int32_t *__restrict__ seg_off,
                                                  const float *__restrict__ vals, int s_base, int v_base, int px,
                                                  float (&acc)[NP][kMaxGroup])
{
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[p][g] = 0.0f;
    for (int q = it.seg_begin - s_base; q < it.seg_end - s_base; ++q) {
        const Seg sg = segs[q];
        const float *v = vals + (sg.val_off - v_base);
        const int pos = seg_off[q] + px;
        int t = 0;
        for (; t + 8 <= sg.m; t += 8) contract_batch_win<8, NP, G, T>(lw, v, t, pos + t, acc);
        if (t + 4 <= sg.m) {
            contract_batch_win<4, NP, G, T>(lw, v, t, pos + t, acc);
            t += 4;
        }
        if (t + 2 <= sg.m) {
            contract_batch_win<2, NP, G, T>(lw, v, t, pos + t, acc);
            t += 2;
        }
        if (t < sg.m) contract_batch_win<1, NP, G, T>(lw, v, t, pos + t, acc);
    }
}

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

// contract_chunk from the chunk's staged windows (win: [channel][wl slots]); the same multiply-adds in the
// same order, so the same sums.
template <typename T, int STRIDE>
__device__ __forceinline__ void contract_chunk_win(const uint32_t *win, int wl, T *__restrict__ tile,
                                                   const Item *__restrict__ items, const Seg *__restrict__ segs,
                                                   const int32_t *__restrict__ seg_off, const float *__restrict__ vals,
                                                   int it_begin, int it_end, int s_base, int v_base, int ccn, int CC,
                                                   int K, int Wo, int HoWo, int wo0, int tid)
{
    constexpr int NP = 2;
    const int cl0 = tid / kPx, px = tid - cl0 * kPx;
    const int wo = wo0 + px;
    for (int cb = 0; cb < CC; cb += 4 * NP) {
        const uint32_t *lw[NP];
        bool valid[NP];
        int cl[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            cl[p] = cb + cl0 + 4 * p;
            valid[p] = cl[p] < ccn && wo < Wo;
            lw[p] = win + (cl[p] < ccn ? cl[p] : 0) * wl;  // channels past the chunk read staged data, dropped
        }
        for (int ii = it_begin; ii < it_end; ++ii) {
            const Item it = items[ii];
            float a[NP][kMaxGroup];
            switch (it.G) {
            case 1: contract_item_win<NP, 1, T>(lw, it, segs, seg_off, vals, s_base, v_base, px, a); break;
            case 2: contract_item_win<NP, 2, T>(lw, it, segs, seg_off, vals, s_base, v_base, px, a); break;
            case 3: contract_item_win<NP, 3, T>(lw, it, segs, seg_off, vals, s_base, v_base, px, a); break;
            default: contract_item_win<NP, 4, T>(lw, it, segs, seg_off, vals, s_base, v_base, px, a); break;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (cl[p] < CC) {
                    for (int g = 0; g < it.G; ++g) {
                        const int k = it.out_off[g] / HoWo;
                        tile[px * STRIDE + cl[p] * K + k] = Elem<T>::from_f32(valid[p] ? a[p][g] : 0.0f);
                    }
                }
            }
        }
    }
}

// The source windows and psi of one workgroup's latitude (plan.hpp, FusedWindows): windows when the
// launch has them (wcap > 0; else the tables are not passed) and the latitude's fit the LDS area (wcap
// slots per channel), else global reads; with windows, the latitude's items, segments, values and window
// offsets are copied to LDS once (psi_cap bytes after the windows) when they fit, so the chunks read no
// psi from memory.
struct WinTables {
    const FWin *rows;
    const int32_t *ho_ptr, *ho_len, *seg_off;
    const int4 *ho_psi;
    int wcap, psi_cap;
};

struct LatWin {
    bool use_win, use_psi;
    int wl, r0, r1;
    int n_it, s0, v0;
    const Item *l_items;
    const Seg *l_segs;
    const float *l_vals;
    const int32_t *l_off;
};

// The copies run on all threads; they are visible after the caller's next barrier.
__device__ __forceinline__ LatWin setup_lat(const WinTables &wt, uint32_t *win, int CC, int ho, int it_begin,
                                            int it_end, const Item *__restrict__ items, const Seg *__restrict__ segs,
                                            const float *__restrict__ vals, int tid)
{
    LatWin L;
    L.wl = wt.wcap > 0 ? wt.ho_len[ho] : 0;
    L.use_win = wt.wcap > 0 && L.wl <= wt.wcap;
    L.r0 = L.use_win ? wt.ho_ptr[ho] : 0;
    L.r1 = L.use_win ? wt.ho_ptr[ho + 1] : 0;
    const int4 pr = L.use_win && wt.psi_cap > 0 ? wt.ho_psi[ho] : make_int4(0, 0, 0, 0);  // s0, s1, v0, v1
    const int n_it = it_end - it_begin, n_sg = pr.y - pr.x, n_v = pr.w - pr.z;
    L.use_psi = L.use_win && wt.psi_cap > 0 && n_it * 32 + n_sg * 20 + n_v * 4 <= wt.psi_cap;
    L.n_it = n_it;
    L.s0 = pr.x;
    L.v0 = pr.z;
    unsigned char *lpsi = reinterpret_cast<unsigned char *>(win) + ((int64_t)CC * wt.wcap * 4 + 15) / 16 * 16;
    Item *l_items = reinterpret_cast<Item *>(lpsi);
    Seg *l_segs = reinterpret_cast<Seg *>(lpsi + n_it * 32);
    float *l_vals = reinterpret_cast<float *>(lpsi + n_it * 32 + n_sg * 16);
    int32_t *l_off = reinterpret_cast<int32_t *>(lpsi + n_it * 32 + n_sg * 16 + n_v * 4);
    if (L.use_psi) {
        const int32_t *src_it = reinterpret_cast<const int32_t *>(items + it_begin);
        const int32_t *src_sg = reinterpret_cast<const int32_t *>(segs + pr.x);
        for (int e = tid; e < 8 * n_it; e += kThreads) reinterpret_cast<int32_t *>(l_items)[e] = src_it[e];
        for (int e = tid; e < 4 * n_sg; e += kThreads) reinterpret_cast<int32_t *>(l_segs)[e] = src_sg[e];
        for (int e = tid; e < n_v; e += kThreads) l_vals[e] = vals[pr.z + e];
        for (int e = tid; e < n_sg; e += kThreads) l_off[e] = wt.seg_off[pr.x + e];
    }
    L.l_items = l_items;
    L.l_segs = l_segs;
    L.l_vals = l_vals;
    L.l_off = l_off;
    return L;
}

// One chunk's contraction into the tile: from staged windows (staged here: one wait and a barrier) and
// the LDS psi copy where the latitude has them, else from memory.  Caller: a barrier before (the previous
// chunk is done with the tile and the windows).
template <typename T, int STRIDE>
__device__ __forceinline__ void contract_any(const LatWin &L, const WinTables &wt, uint32_t *win, const T *xb,
                                             T *__restrict__ tile, const Item *__restrict__ items,
                                             const Seg *__restrict__ segs, const float *__restrict__ vals,
                                             int it_begin, int it_end, int64_t plane_sz, int c0, int ccn, int CC, int K,
                                             int Wo, int HoWo, int in_stride, int wo0, int tid, int wave, int lane)
{
    if (L.use_win) {
        stage_fwin<T>(xb, win, wt.rows, L.r0, L.r1, L.wl, plane_sz, c0, ccn, Wo, in_stride, wo0, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);  // this thread's window loads have landed
        __syncthreads();                // everyone's have
        if (L.use_psi)
            contract_chunk_win<T, STRIDE>(win, L.wl, tile, L.l_items, L.l_segs, L.l_off, L.l_vals, 0, L.n_it, L.s0,
                                          L.v0, ccn, CC, K, Wo, HoWo, wo0, tid);
        else
            contract_chunk_win<T, STRIDE>(win, L.wl, tile, items, segs, wt.seg_off, vals, it_begin, it_end, 0, 0, ccn,
                                          CC, K, Wo, HoWo, wo0, tid);
    } else {
        contract_chunk<T, T, STRIDE>(xb, tile, items, segs, vals, it_begin, it_end, plane_sz, c0, ccn, CC, K, Wo,
                                     HoWo, in_stride, wo0, tid);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fused_kernel(const T *__restrict__ x, const i16x8 *__restrict__ Wa,
                                                         T *__restrict__ y, const Item *__restrict__ items,
                                                         const int32_t *__restrict__ block_ptr,
                                                         const int32_t *__restrict__ ho_order,
                                                         const Seg *__restrict__ segs, const float *__restrict__ vals,
                                                         int B, int C, int Co, int K, int Ho, int Wo, int Hi, int Wi,
                                                         int in_stride, int n_pt, int n_ob, WinTables wt)
{
    typedef typename Elem<T>::vec8 vec8;
    __shared__ __attribute__((aligned(16))) T tile[kPx * kLdsStride];
    // dynamic LDS: [CC][wcap] 4-byte slots of source windows, then psi_cap bytes for the latitude's psi
    extern __shared__ __attribute__((aligned(16))) uint32_t win[];

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
    const int n_ot16 = (Co + 15) / 16;
    const int64_t plane_sz = (int64_t)Hi * Wi;
    const int it_begin = block_ptr[ho], it_end = block_ptr[ho + 1];
    const int HoWo = Ho * Wo;
    const T *xb = x + (int64_t)b * C * plane_sz;
    const LatWin L = setup_lat(wt, win, CC, ho, it_begin, it_end, items, segs, vals, tid);

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < C; c0 += CC) {
        const int ccn = min(CC, C - c0);
        __syncthreads();  // the previous chunk's MFMA reads of `tile` and window reads are done
        // ---- contraction of channels [c0, c0+ccn) into tile[px][cl*K + k] ----
        contract_any<T, kLdsStride>(L, wt, win, xb, tile, items, segs, vals, it_begin, it_end, plane_sz, c0, ccn, CC,
                                    K, Wo, HoWo, in_stride, wo0, tid, wave, lane);
        // rows past the chunk's (c, k) range are zero
        for (int e = tid; e < kPx * kR; e += kThreads) {
            const int px = e / kR, r = e - px * kR;
            if (r >= ccn * K) tile[px * kLdsStride + r] = Elem<T>::from_f32(0.0f);
        }
        __syncthreads();
        // ---- einsum on the matrix cores ----
        // A operands: W packed by launch_pack_wa16 in operand order, one 16-byte load per lane, output-channel
        // tile and k-step (zeros past Co and past the chunk's ccn K rows)
        const i16x8 *wq = Wa + (int64_t)(c0 / CC) * n_ot16 * (kR / 32) * 64 + lane;
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
                const int o16 = (o_base >> 4) + ot;
                const i16x8 av = o16 < n_ot16 ? wq[((int64_t)o16 * (kR / 32) + ks) * 64] : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
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

// Packed W for fused_kernel (16-bit data): for chunk t (channels c0 = t CC .. + CC - 1), 16-channel output
// tile o16, k-step ks (32 rows) and lane l, the eight 16-bit values at Wa[(((t n_ot16 + o16) (kR / 32) + ks)
// 64 + l) 8 + e] are W[o][c0 K + rr] with o = 16 o16 + l % 16 and rr = 32 ks + 8 (l / 16) + e — the A
// operand of that step for that lane — and zero where o >= Co or rr reaches past the chunk's channels.
__global__ __launch_bounds__(256) void pack_wa16_kernel(const uint16_t *__restrict__ W, uint16_t *__restrict__ Wa,
                                                        int Co, int C, int K, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int e = (int)(i & 7), l = (int)((i >> 3) & 63), ks = (int)((i >> 9) % (kR / 32));
    const int64_t rest = (i >> 9) / (kR / 32);
    const int n_ot16 = (Co + 15) / 16;
    const int o16 = (int)(rest % n_ot16);
    const int t = (int)(rest / n_ot16);
    const int CC = kR / K, c0 = t * CC, ccn = min(CC, C - c0);
    const int o = 16 * o16 + (l & 15), rr = 32 * ks + 8 * (l >> 4) + e;
    Wa[i] = (o < Co && rr < ccn * K) ? W[((int64_t)o * C + c0) * K + rr] : (uint16_t)0;
}

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
                                                             int n_pt, int n_ob, const FWin *__restrict__ fw_rows,
                                                             const int32_t *__restrict__ fw_ho_ptr,
                                                             const int32_t *__restrict__ fw_ho_len,
                                                             const int32_t *__restrict__ seg_off, int wcap,
                                                             const int4 *__restrict__ fw_ho_psi, int psi_cap)
{
    __shared__ __attribute__((aligned(16))) float tile[kPx * kLdsStride32];
    // dynamic LDS: [CC][wcap] 4-byte slots of source windows, then psi_cap bytes for the latitude's psi
    extern __shared__ __attribute__((aligned(16))) uint32_t win[];

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
    const float *xb = x + (int64_t)b * C * plane_sz;
    const WinTables wt{fw_rows, fw_ho_ptr, fw_ho_len, seg_off, fw_ho_psi, wcap, psi_cap};
    const LatWin L = setup_lat(wt, win, CC, ho, it_begin, it_end, items, segs, vals, tid);

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < C; c0 += CC) {
        const int ccn = min(CC, C - c0);
        __syncthreads();  // the previous chunk's MFMA reads of `tile` and window reads are done
        contract_any<float, kLdsStride32>(L, wt, win, xb, tile, items, segs, vals, it_begin, it_end, plane_sz, c0, ccn,
                                          CC, K, Wo, HoWo, in_stride, wo0, tid, wave, lane);
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
    // windows in LDS where the plan has them and a channel plane is below 2 GiB (32-bit load offsets)
    const bool win_ok = a.fw_rows && a.fw_ho_ptr && a.fw_ho_len && a.fw_seg_off && a.fw_cap > 0 &&
                        (int64_t)a.Hi * a.Wi <= INT32_MAX / 4;
    const int wcap = win_ok ? a.fw_cap : 0;
    const int psi_cap = wcap > 0 && a.fw_ho_psi ? std::min(a.fw_psi_bytes, kFusedPsiBytes) : 0;
    const size_t lds = ((size_t)(kR / a.K) * wcap * 4 + 15) / 16 * 16 + (size_t)psi_cap;  // 4-byte window slots
    const WinTables wt{a.fw_rows, a.fw_ho_ptr, a.fw_ho_len, a.fw_seg_off, reinterpret_cast<const int4 *>(a.fw_ho_psi),
                       wcap, psi_cap};
    if (a.f32) {
        if (!a.Wa && a.C > 0) return hipErrorInvalidValue;  // the fp32 kernel takes W packed (launch_pack_wa_f32)
        hipError_t e = allow_lds(reinterpret_cast<const void *>(&fused_f32_kernel), lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fused_f32_kernel, dim3((unsigned)nblk), dim3(kThreads), lds, stream, (const float *)a.x,
                           (const float4 *)a.Wa, (float *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals, a.B,
                           a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob, a.fw_rows, a.fw_ho_ptr,
                           a.fw_ho_len, a.fw_seg_off, wcap, reinterpret_cast<const int4 *>(a.fw_ho_psi), psi_cap);
    } else {
        if (!a.Wa16 && a.C > 0) return hipErrorInvalidValue;  // the kernel takes W packed (launch_pack_wa16)
        const i16x8 *wa = reinterpret_cast<const i16x8 *>(a.Wa16);
        const void *fn = a.f16 ? reinterpret_cast<const void *>(&fused_kernel<f16_t>)
                               : reinterpret_cast<const void *>(&fused_kernel<bf16_t>);
        hipError_t e = allow_lds(fn, lds);
        if (e != hipSuccess) return e;
        if (a.f16)
            hipLaunchKernelGGL(fused_kernel<f16_t>, dim3((unsigned)nblk), dim3(kThreads), lds, stream,
                               (const f16_t *)a.x, wa, (f16_t *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals,
                               a.B, a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob, wt);
        else
            hipLaunchKernelGGL(fused_kernel<bf16_t>, dim3((unsigned)nblk), dim3(kThreads), lds, stream,
                               (const bf16_t *)a.x, wa, (bf16_t *)a.y, a.items, a.block_ptr, a.ho_order, a.segs, a.vals,
                               a.B, a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.in_stride, n_pt, n_ob, wt);
    }
    return hipGetLastError();
}

int fused_win_cap_f32(int K, const int32_t *ho_len, int nho)
{
    // positions per channel of the largest latitude window set within kFusedWinBytes
    if (K < 1 || K > kR) return 0;
    const int64_t cc = kR / K;
    int cap = 0;
    for (int i = 0; i < nho; ++i)
        if ((int64_t)ho_len[i] * cc * (int64_t)sizeof(float) <= kFusedWinBytes) cap = std::max(cap, ho_len[i]);
    return cap;
}

int64_t fused_wa_f32_floats(int Co, int C, int K)
{
    if (K < 1 || K > kR) return 0;
    const int64_t CC = kR / K, n_chunks = (C + CC - 1) / CC, n_ot16 = (Co + 15) / 16;
    return n_chunks * n_ot16 * (kR / 16) * 64 * 4;
}

int64_t fused_wa16_elems(int Co, int C, int K)
{
    if (K < 1 || K > kR) return 0;
    const int64_t CC = kR / K, n_chunks = (C + CC - 1) / CC, n_ot16 = (Co + 15) / 16;
    return n_chunks * n_ot16 * (kR / 32) * 64 * 8;
}

hipError_t launch_pack_wa16(const void *W, void *Wa, int Co, int C, int K, hipStream_t stream)
{
    const int64_t total = fused_wa16_elems(Co, C, K);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_wa16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       (const uint16_t *)W, (uint16_t *)Wa, Co, C, K, total);
    return hipGetLastError();
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

int fused_tile_px() { return kPx; }

}  // namespace disco
