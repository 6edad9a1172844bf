// kernels_fused_mfma.hip — fused DISCO convolution on the gfx950 matrix cores.
//
// y[b,o,ho,wo] = sum_{c,k} W[o,c,k] * out[b,c,k,ho,wo], out = CSR contraction
// ("contraction + einsum", torch-harmonics "disco-kernel-dev" page,
// "Architecture snapshot"; the packed-psi idea follows its "kpacked layout"
// section, re-derived for MFMA).
//
// Workgroup = (b, ho, npx output longitudes, up to 256 output channels);
// wave w owns the 32 longitudes [px0 + 32w, px0 + 32w + 32) and all output
// channels.  Input channels are walked in chunks of kCh:
//  1. stage: the packed A blocks of the latitude's psi piece, the x windows
//     of the piece's source rows for the kCh channels, and the chunk's W
//     slice in MFMA A-operand order;
//  2. contraction: for each block, one v_mfma_f32_32x32x16_bf16 per channel,
//     A = [bf16(psi) ; bf16 residue] (32 x 16), B = 16 consecutive x values
//     per longitude (eight aligned 2-byte LDS reads per lane);
//  3. einsum, chained in registers: lane (h = lane/32) holds out[k] for
//     k in {4h..4h+3, 8+4h..8+4h+3} (sum of the two psi halves), which is
//     exactly the B operand of the next v_mfma_f32_32x32x16_bf16 when the
//     reduction rows of one channel are ordered that way; W is packed to the
//     same order.  fp32 accumulators for 256 output channels x 32 longitudes
//     stay in registers across all chunks.
// A latitude whose packed psi is one piece keeps it resident and
// double-buffers the x windows: the next chunk's windows stream into LDS by
// direct global->LDS loads while the current chunk is contracted.  Caps
// spanning whole rings (several pieces) stage synchronously per piece.
// No atomics; every output is written once.
#include "common.hpp"
#include "kernels.hpp"
#include "plan_fused.hpp"

namespace disco {

namespace {

constexpr int kCh = 4;          // input channels per chunk
constexpr int kMaxOt = 8;       // 32-row output-channel tiles per workgroup (256 channels)
constexpr int kNpx = 256;       // output longitudes per workgroup (8 waves)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Eight consecutive bf16 at a 2-byte aligned LDS address (element loads keep the alias
// information of the pointer they are based on).
__device__ __forceinline__ bf16x8 lds8(const bf16_t *p)
{
    const __bf16 *q = reinterpret_cast<const __bf16 *>(p);
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = q[i];
    return v;
}

__device__ __forceinline__ int mod_l(int g, int L)
{
    g %= L;
    return g < 0 ? g + L : g;
}

struct Ctx {
    const bf16_t *x, *W;
    const FRow *rows;
    const bf16_t *adata;
    const int32_t *block_xoff;
    bf16_t *w_area, *a_area;
    int32_t *o_area;
    int B, C, Co, K, L, Wi, s, n_ot, b, px0, o_base, tid, nthreads, wave, nwaves, lane, col, h, pxw;
    int64_t plane_sz;
};

// W slice of the chunk starting at channel c0, in A-operand order: entry (ot, cl, lane).
__device__ __forceinline__ void stage_w(const Ctx &c, int c0)
{
    for (int e = c.tid; e < c.n_ot * kCh * 64; e += c.nthreads) {
        const int ln = e & 63;
        const int t2 = e >> 6;
        const int cl = t2 % kCh, ot = t2 / kCh;
        const int o = c.o_base + ot * 32 + (ln & 31);
        const int hh = ln >> 5;
        const int ch = c0 + cl;
        uint2 lo4 = make_uint2(0u, 0u), hi4 = make_uint2(0u, 0u);
        if (c.K == 16) {
            if (o < c.Co && ch < c.C) {
                const bf16_t *wr = c.W + ((int64_t)o * c.C + ch) * 16;
                lo4 = *reinterpret_cast<const uint2 *>(wr + 4 * hh);
                hi4 = *reinterpret_cast<const uint2 *>(wr + 8 + 4 * hh);
            }
        } else {
            i16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = (i < 4) ? 4 * hh + i : 8 + 4 * hh + (i - 4);
                v[i] = (o < c.Co && ch < c.C && k < c.K) ? (short)c.W[((int64_t)o * c.C + ch) * c.K + k] : (short)0;
            }
            const uint4 u = __builtin_bit_cast(uint4, v);
            lo4 = make_uint2(u.x, u.y);
            hi4 = make_uint2(u.z, u.w);
        }
        *reinterpret_cast<uint4 *>(c.w_area + (int64_t)e * 8) = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
    }
}

// Packed A blocks and block offsets of a piece.
__device__ __forceinline__ void stage_a(const Ctx &c, const FPiece &pc, int nblk)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(c.adata + (int64_t)pc.blk_begin * 512);
    uint4 *dst = reinterpret_cast<uint4 *>(c.a_area);
    for (int e = c.tid; e < nblk * 64; e += c.nthreads) dst[e] = src[e];
    for (int e = c.tid; e < nblk; e += c.nthreads) c.o_area[e] = c.block_xoff[pc.blk_begin + e];
}

// x windows of one chunk, synchronous: rows over waves, positions over lanes; channels past C are zeros.
__device__ __forceinline__ void stage_windows(const Ctx &c, bf16_t *xbuf, const FPiece &pc, int xwin, int c0,
                                              bool vec)
{
    const int ccn = min(kCh, c.C - c0);
    const int nrows = pc.row_end - pc.row_begin;
    for (int cl = 0; cl < kCh; ++cl) {
        for (int r = c.wave; r < nrows; r += c.nwaves) {
            const FRow fr = c.rows[pc.row_begin + r];
            bf16_t *dst = xbuf + cl * xwin + fr.lds_off;
            if (cl >= ccn) {
                for (int e8 = c.lane; e8 < (fr.len >> 3); e8 += 64)
                    *reinterpret_cast<uint4 *>(dst + 8 * e8) = make_uint4(0u, 0u, 0u, 0u);
                continue;
            }
            const int hi = fr.sr / c.s, rho = fr.sr - hi * c.s;
            const bf16_t *xrow = c.x + ((int64_t)c.b * c.C + (c0 + cl)) * c.plane_sz + (int64_t)hi * c.Wi;
            const int g0 = mod_l(c.px0 + fr.start, c.L);
            if (vec) {
                // s == 1: 8-element chunks never straddle the row end (L and g0 are multiples of 8)
                for (int e8 = c.lane; e8 < (fr.len >> 3); e8 += 64) {
                    int pos = g0 + 8 * e8;
                    while (pos >= c.L) pos -= c.L;
                    *reinterpret_cast<uint4 *>(dst + 8 * e8) = *reinterpret_cast<const uint4 *>(xrow + pos);
                }
            } else {
                for (int e = c.lane; e < fr.len; e += 64) {
                    int pos = g0 + e;
                    while (pos >= c.L) pos -= c.L;
                    dst[e] = xrow[(int64_t)c.s * pos + rho];
                }
            }
        }
    }
}

// x windows of one chunk queued as direct global->LDS loads (global_load_lds_dwordx4: lane i of
// an instruction writes LDS base + 16*i).  s == 1 and 16-byte aligned rows only.  The caller
// waits (s_waitcnt + barrier) before the windows are read; channels past C get zero stores.
__device__ __forceinline__ void queue_windows(const Ctx &c, bf16_t *xbuf, const FPiece &pc, int xwin, int c0)
{
    const int ccn = min(kCh, c.C - c0);
    const int nrows = pc.row_end - pc.row_begin;
    for (int cl = 0; cl < kCh; ++cl) {
        for (int r = c.wave; r < nrows; r += c.nwaves) {
            const FRow fr = c.rows[pc.row_begin + r];
            bf16_t *dst = xbuf + cl * xwin + fr.lds_off;
            const int nch = fr.len >> 3;
            if (cl >= ccn) {
                for (int e8 = c.lane; e8 < nch; e8 += 64)
                    *reinterpret_cast<uint4 *>(dst + 8 * e8) = make_uint4(0u, 0u, 0u, 0u);
                continue;
            }
            const bf16_t *xrow = c.x + ((int64_t)c.b * c.C + (c0 + cl)) * c.plane_sz + (int64_t)fr.sr * c.Wi;
            const int g0 = mod_l(c.px0 + fr.start, c.L);
            for (int t = 0; t < nch; t += 64) {
                const int e8 = t + c.lane;
                if (e8 < nch) {
                    int pos = g0 + 8 * e8;
                    while (pos >= c.L) pos -= c.L;
                    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(xrow + pos),
                                                     (void __attribute__((address_space(3))) *)(dst + 8 * t), 16, 0,
                                                     0);
                }
            }
        }
    }
}

// Contraction of one piece on the matrix cores.  Operands of block i+1 are read while block
// i's MFMAs run; the body is straight-line (the last iteration re-reads the last block) so
// LDS waits stay partial.
__device__ __forceinline__ void contract(const Ctx &c, const bf16_t *x_area, int xwin, int nblk, f32x16 (&d)[kCh])
{
    if (nblk <= 0) return;
    const int32_t *boff = c.o_area;
    const int lane_x = c.pxw + c.col + 8 * c.h;
    const bf16_t *a_lane = c.a_area + c.lane * 8;
    int off_n = boff[0] + lane_x;
    int off_nn = boff[nblk > 1 ? 1 : 0];
    bf16x8 a_n = *reinterpret_cast<const bf16x8 *>(a_lane);
    bf16x8 bop[kCh];
#pragma unroll
    for (int cl = 0; cl < kCh; ++cl) bop[cl] = lds8(x_area + cl * xwin + off_n);
    for (int i = 0; i < nblk; ++i) {
        const bf16x8 a_c = a_n;
        const int ip = min(i + 1, nblk - 1);
        off_n = off_nn + lane_x;
        off_nn = boff[min(i + 2, nblk - 1)];
        a_n = *reinterpret_cast<const bf16x8 *>(a_lane + ip * 512);
#pragma unroll
        for (int cl = 0; cl < kCh; ++cl) {
            d[cl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, bop[cl], d[cl], 0, 0, 0);
            bop[cl] = lds8(x_area + cl * xwin + off_n);
        }
    }
}

// Einsum of a chunk into the y accumulators.
__device__ __forceinline__ void einsum(const Ctx &c, f32x16 (&d)[kCh], f32x16 (&yacc)[kMaxOt])
{
#pragma unroll
    for (int cl = 0; cl < kCh; ++cl) {
        bf16x8 bop;
#pragma unroll
        for (int a = 0; a < 8; ++a) bop[a] = (__bf16)(d[cl][a] + d[cl][a + 8]);
#pragma unroll
        for (int ot = 0; ot < kMaxOt; ++ot) {
            if (ot < c.n_ot) {
                const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(c.w_area + ((ot * kCh + cl) * 64 + c.lane) * 8);
                yacc[ot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bop, yacc[ot], 0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ void zero(f32x16 (&d)[kCh])
{
#pragma unroll
    for (int cl = 0; cl < kCh; ++cl)
#pragma unroll
        for (int a = 0; a < 16; ++a) d[cl][a] = 0.0f;
}

// One chunk of a double-buffered latitude: contract from `cur` while the next chunk's windows
// stream into `nxt`.  The two buffers are restrict parameters so that the compiler knows the
// queued direct loads do not alias the reads (it then keeps the LDS waits partial).
__device__ __forceinline__ void dbuf_step(const Ctx &c, const FPiece &pc, int xwin, int nblk, int c0,
                                          const bf16_t *__restrict__ cur, bf16_t *__restrict__ nxt,
                                          f32x16 (&yacc)[kMaxOt])
{
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads into `cur` have landed
    __syncthreads();                // everyone's have; the previous chunk is done with W and `nxt`
    stage_w(c, c0);
    __syncthreads();                // W slice visible (a full fence: nothing may be in flight yet)
    if (c0 + kCh < c.C) queue_windows(c, nxt, pc, xwin, c0 + kCh);  // lands while this chunk computes
    f32x16 d[kCh];
    zero(d);
    contract(c, cur, xwin, nblk, d);
    einsum(c, d, yacc);
}

__global__ __launch_bounds__(512) void fused_mfma_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ W, bf16_t *__restrict__ y,
    const FPiece *__restrict__ pieces, const FRow *__restrict__ rows, const int32_t *__restrict__ block_xoff,
    const bf16_t *__restrict__ adata, const int32_t *__restrict__ ho_piece, const int32_t *__restrict__ ho_order,
    int B, int C, int Co, int K, int Ho, int L, int Hi, int Wi, int s, int n_pxb, int n_ob, int n_ot, int max_blk,
    int vec)
{
    // LDS: [W slice: n_ot*kCh*512 bf16] [block offsets: max_blk int32 (16-B rounded)]
    //      [piece: blocks*512 bf16 | x windows: kCh*xwin bf16, twice for a double-buffered piece]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    Ctx c;
    c.w_area = reinterpret_cast<bf16_t *>(smem);
    c.o_area = reinterpret_cast<int32_t *>(c.w_area + n_ot * kCh * 512);
    c.a_area = reinterpret_cast<bf16_t *>(c.o_area + ((max_blk + 3) & ~3));

    int bid = blockIdx.x;
    const int pxb = bid % n_pxb;
    bid /= n_pxb;
    const int ob = bid % n_ob;
    bid /= n_ob;
    c.b = bid % B;
    const int ho = ho_order[bid / B];

    c.x = x; c.W = W; c.rows = rows; c.adata = adata; c.block_xoff = block_xoff;
    c.B = B; c.C = C; c.Co = Co; c.K = K; c.L = L; c.Wi = Wi; c.s = s; c.n_ot = n_ot;
    c.nthreads = blockDim.x;
    c.nwaves = c.nthreads >> 6;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);  // wave-uniform: row loops run on the scalar unit
    c.col = c.lane & 31;
    c.h = c.lane >> 5;
    c.px0 = pxb * kNpx;
    c.pxw = c.wave * 32;
    c.o_base = ob * (kMaxOt * 32);
    c.plane_sz = (int64_t)Hi * Wi;
    const int p_begin = ho_piece[ho], p_end = ho_piece[ho + 1];

    f32x16 yacc[kMaxOt];
#pragma unroll
    for (int ot = 0; ot < kMaxOt; ++ot)
#pragma unroll
        for (int a = 0; a < 16; ++a) yacc[ot][a] = 0.0f;

    const FPiece pc0 = pieces[p_begin];
    if (vec && pc0.dbuf) {
        // One piece: packed A resident, x windows double-buffered.
        const FPiece pc = pc0;
        const int nblk = pc.blk_end - pc.blk_begin;
        const int xwin = pc.xwin_elems;
        bf16_t *xs0 = c.a_area + nblk * 512;
        bf16_t *xs1 = xs0 + kCh * xwin;
        stage_a(c, pc, nblk);
        queue_windows(c, xs0, pc, xwin, 0);
        for (int c0 = 0; c0 < C; c0 += 2 * kCh) {
            dbuf_step(c, pc, xwin, nblk, c0, xs0, xs1, yacc);
            if (c0 + kCh < C) dbuf_step(c, pc, xwin, nblk, c0 + kCh, xs1, xs0, yacc);
        }
    } else {
        for (int c0 = 0; c0 < C; c0 += kCh) {
            f32x16 d[kCh];
            zero(d);
            for (int pi = p_begin; pi < p_end; ++pi) {
                const FPiece pc = pieces[pi];
                const int nblk = pc.blk_end - pc.blk_begin;
                const int xwin = pc.xwin_elems;
                bf16_t *x_area = c.a_area + nblk * 512;
                __syncthreads();  // previous piece's LDS (and the previous chunk's W slice) fully consumed
                if (pi == p_begin) stage_w(c, c0);
                if (c0 == 0 || p_end - p_begin > 1) stage_a(c, pc, nblk);
                stage_windows(c, x_area, pc, xwin, c0, vec != 0);
                __syncthreads();
                contract(c, x_area, xwin, nblk, d);
            }
            einsum(c, d, yacc);
        }
    }

    // ---- epilogue: yacc[ot] row = output channel, column = longitude ----
    const int wo = c.px0 + c.pxw + c.col;
    if (wo < L) {
#pragma unroll
        for (int ot = 0; ot < kMaxOt; ++ot) {
            if (ot < n_ot) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int o = c.o_base + ot * 32 + 8 * (a >> 2) + 4 * c.h + (a & 3);
                    if (o < Co) y[(((int64_t)c.b * Co + o) * Ho + ho) * L + wo] = f32_to_bf16(yacc[ot][a]);
                }
            }
        }
    }
}

}  // namespace

size_t fused_mfma_lds_bytes(int n_ot, int max_piece_elems, int max_blk)
{
    return (size_t)n_ot * kCh * 512 * 2 + (size_t)((max_blk + 3) & ~3) * 4 + (size_t)max_piece_elems * 2;
}

int fused_mfma_channels_per_chunk() { return kCh; }

int fused_mfma_npx() { return kNpx; }

size_t fused_mfma_reserved_bytes()
{
    // W slice at the largest output-channel tile count, plus the block offsets of a piece
    // (a piece holds at most 160 KiB / 1 KiB blocks)
    return (size_t)kMaxOt * kCh * 512 * 2 + 160 * 4 + 16;
}

hipError_t launch_fused_mfma(const FusedMfmaLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.Co == 0) return hipSuccess;
    const int n_pxb = (a.Wo + kNpx - 1) / kNpx;
    const int n_ob = (a.Co + kMaxOt * 32 - 1) / (kMaxOt * 32);
    const int n_ot = std::min(kMaxOt, (a.Co + 31) / 32);
    const size_t lds = fused_mfma_lds_bytes(n_ot, a.max_piece_elems, a.max_blk);
    hipError_t e = hipFuncSetAttribute((const void *)fused_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_ob * n_pxb;
    const int vec = (a.s == 1 && a.Wo % 8 == 0 && ((int64_t)a.Hi * a.Wi) % 8 == 0 && ((uintptr_t)a.x % 16) == 0) ? 1 : 0;
    hipLaunchKernelGGL(fused_mfma_kernel, dim3((unsigned)nblk), dim3(kNpx / 32 * 64), lds, stream,
                       (const bf16_t *)a.x, (const bf16_t *)a.W, (bf16_t *)a.y, a.pieces, a.rows, a.block_xoff,
                       (const bf16_t *)a.adata, a.ho_piece, a.ho_order, a.B, a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi,
                       a.s, n_pxb, n_ob, n_ot, a.max_blk, vec);
    return hipGetLastError();
}

}  // namespace disco
