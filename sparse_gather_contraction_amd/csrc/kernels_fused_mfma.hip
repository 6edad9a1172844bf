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
//  1. stage (per piece of the latitude's packed psi): the packed A blocks,
//     the x windows of the piece's source rows for the kCh channels, and, at
//     the first piece, the chunk's W slice in MFMA A-operand order;
//  2. contraction: for each block, one v_mfma_f32_32x32x16_bf16 per channel,
//     A = [bf16(psi) ; bf16 residue] (32 x 16), B = 16 consecutive x values
//     per longitude (one unaligned 16-byte LDS read per lane);
//  3. einsum, chained in registers: lane (h = lane/32) holds out[k] for
//     k in {4h..4h+3, 8+4h..8+4h+3} (sum of the two psi halves), which is
//     exactly the B operand of the next v_mfma_f32_32x32x16_bf16 when the
//     reduction rows of one channel are ordered that way; W is packed to the
//     same order.  fp32 accumulators for 256 output channels x 32 longitudes
//     stay in registers across all chunks.
// No atomics; every output is written once.
#include "common.hpp"
#include "kernels.hpp"
#include "plan_fused.hpp"

namespace disco {

namespace {

constexpr int kCh = 4;          // input channels per chunk
constexpr int kMaxOt = 8;       // 32-row output-channel tiles per workgroup (256 channels)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int mod_l(int g, int L)
{
    g %= L;
    return g < 0 ? g + L : g;
}

__global__ __launch_bounds__(512) void fused_mfma_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ W, bf16_t *__restrict__ y,
    const FPiece *__restrict__ pieces, const FRow *__restrict__ rows, const int32_t *__restrict__ block_xoff,
    const bf16_t *__restrict__ adata, const int32_t *__restrict__ ho_piece, const int32_t *__restrict__ ho_order,
    int B, int C, int Co, int K, int Ho, int L, int Hi, int Wi, int s, int npx, int n_pxb, int n_ob, int n_ot,
    int max_blk, int vec)
{
    // LDS: [W slice: n_ot*kCh*512 bf16] [block offsets: max_blk int32 (rounded to 16 B)]
    //      [piece: blocks*512 bf16 | kCh windows of xwin_elems bf16 each]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16_t *w_area = reinterpret_cast<bf16_t *>(smem);
    int32_t *o_area = reinterpret_cast<int32_t *>(w_area + n_ot * kCh * 512);
    bf16_t *a_area = reinterpret_cast<bf16_t *>(o_area + ((max_blk + 3) & ~3));

    int bid = blockIdx.x;
    const int pxb = bid % n_pxb;
    bid /= n_pxb;
    const int ob = bid % n_ob;
    bid /= n_ob;
    const int b = bid % B;
    const int ho = ho_order[bid / B];

    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, h = lane >> 5;
    const int px0 = pxb * npx;
    const int pxw = wave * 32;  // this wave's first longitude within the tile
    const int o_base = ob * (kMaxOt * 32);
    const int64_t plane_sz = (int64_t)Hi * Wi;
    const int p_begin = ho_piece[ho], p_end = ho_piece[ho + 1];

    f32x16 yacc[kMaxOt];
#pragma unroll
    for (int ot = 0; ot < kMaxOt; ++ot)
#pragma unroll
        for (int a = 0; a < 16; ++a) yacc[ot][a] = 0.0f;

    for (int c0 = 0; c0 < C; c0 += kCh) {
        const int ccn = min(kCh, C - c0);
        f32x16 d[kCh];
#pragma unroll
        for (int cl = 0; cl < kCh; ++cl)
#pragma unroll
            for (int a = 0; a < 16; ++a) d[cl][a] = 0.0f;

        for (int pi = p_begin; pi < p_end; ++pi) {
            const FPiece pc = pieces[pi];
            const int nblk = pc.blk_end - pc.blk_begin;
            const int xwin = pc.xwin_elems;
            bf16_t *x_area = a_area + nblk * 512;
            __syncthreads();  // previous piece's LDS (and the previous chunk's W slice) fully consumed
            // ---- W slice of this chunk, in A-operand order (first piece only) ----
            if (pi == p_begin) {
                for (int e = tid; e < n_ot * kCh * 64; e += nthreads) {
                    const int ln = e & 63;
                    const int t2 = e >> 6;
                    const int cl = t2 % kCh, ot = t2 / kCh;
                    const int o = o_base + ot * 32 + (ln & 31);
                    const int hh = ln >> 5;
                    const int c = c0 + cl;
                    uint2 lo4 = make_uint2(0u, 0u), hi4 = make_uint2(0u, 0u);
                    if (K == 16) {
                        if (o < Co && c < C) {
                            const bf16_t *wr = W + ((int64_t)o * C + c) * 16;
                            lo4 = *reinterpret_cast<const uint2 *>(wr + 4 * hh);
                            hi4 = *reinterpret_cast<const uint2 *>(wr + 8 + 4 * hh);
                        }
                    } else {
                        i16x8 v;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int k = (i < 4) ? 4 * hh + i : 8 + 4 * hh + (i - 4);
                            v[i] = (o < Co && c < C && k < K) ? (short)W[((int64_t)o * C + c) * K + k] : (short)0;
                        }
                        const uint4 u = __builtin_bit_cast(uint4, v);
                        lo4 = make_uint2(u.x, u.y);
                        hi4 = make_uint2(u.z, u.w);
                    }
                    *reinterpret_cast<uint4 *>(w_area + (int64_t)e * 8) = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
                }
            }
            // ---- packed A blocks of the piece (they do not depend on the channel: a latitude with a
            //      single piece keeps them from the first chunk on) ----
            if (c0 == 0 || p_end - p_begin > 1) {
                const uint4 *src = reinterpret_cast<const uint4 *>(adata + (int64_t)pc.blk_begin * 512);
                uint4 *dst = reinterpret_cast<uint4 *>(a_area);
                for (int e = tid; e < nblk * 64; e += nthreads) dst[e] = src[e];
                for (int e = tid; e < nblk; e += nthreads) o_area[e] = block_xoff[pc.blk_begin + e];
            }
            // ---- x windows: (channel, row) pairs over waves, positions over lanes ----
            {
                const int nrows = pc.row_end - pc.row_begin;
                for (int pr = wave; pr < kCh * nrows; pr += nwaves) {
                    const int cl = pr / nrows;
                    const FRow fr = rows[pc.row_begin + (pr - cl * nrows)];
                    bf16_t *dst = x_area + cl * xwin + fr.lds_off;
                    if (cl >= ccn) {  // channels past C contribute zeros
                        for (int e8 = lane; e8 < (fr.len >> 3); e8 += 64)
                            *reinterpret_cast<uint4 *>(dst + 8 * e8) = make_uint4(0u, 0u, 0u, 0u);
                        continue;
                    }
                    const int hi = fr.sr / s, rho = fr.sr - hi * s;
                    const bf16_t *xrow = x + ((int64_t)b * C + (c0 + cl)) * plane_sz + (int64_t)hi * Wi;
                    const int g0 = mod_l(px0 + fr.start, L);
                    if (vec) {
                        // s == 1: 8-element chunks never straddle the row end (L and g0 are multiples of 8)
                        for (int e8 = lane; e8 < (fr.len >> 3); e8 += 64) {
                            int pos = g0 + 8 * e8;
                            pos = pos >= L ? pos - L * (pos / L) : pos;
                            *reinterpret_cast<uint4 *>(dst + 8 * e8) = *reinterpret_cast<const uint4 *>(xrow + pos);
                        }
                    } else {
                        for (int e = lane; e < fr.len; e += 64) {
                            int pos = g0 + e;
                            pos = pos >= L ? pos - L * (pos / L) : pos;
                            dst[e] = xrow[(int64_t)s * pos + rho];
                        }
                    }
                }
            }
            __syncthreads();
            // ---- contraction on the matrix cores ----
            // operands of block i+1 are read from LDS while block i's MFMAs run; block
            // offsets are scalar-loaded two blocks ahead
            if (nblk > 0) {
                const int32_t *boff = o_area;
                const int lane_x = pxw + col + 8 * h;
                const bf16_t *a_lane = a_area + lane * 8;
                // the loop body is straight-line (the last iteration re-reads the last block) so that
                // LDS waits stay partial
                int off_n = boff[0] + lane_x;
                int off_nn = boff[nblk > 1 ? 1 : 0];
                bf16x8 a_n = *reinterpret_cast<const bf16x8 *>(a_lane);
                bf16x8 bop[kCh];
#pragma unroll
                for (int cl = 0; cl < kCh; ++cl) __builtin_memcpy(&bop[cl], x_area + cl * xwin + off_n, 16);
                for (int i = 0; i < nblk; ++i) {
                    const bf16x8 a_c = a_n;
                    const int ip = min(i + 1, nblk - 1);
                    off_n = off_nn + lane_x;
                    off_nn = boff[min(i + 2, nblk - 1)];
                    a_n = *reinterpret_cast<const bf16x8 *>(a_lane + ip * 512);
#pragma unroll
                    for (int cl = 0; cl < kCh; ++cl) {
                        d[cl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_c, bop[cl], d[cl], 0, 0, 0);
                        __builtin_memcpy(&bop[cl], x_area + cl * xwin + off_n, 16);
                    }
                }
            }
        }
        // ---- einsum: chunk channels -> y accumulators ----
#pragma unroll
        for (int cl = 0; cl < kCh; ++cl) {
            {
                i16x8 pk;
#pragma unroll
                for (int a = 0; a < 8; ++a) pk[a] = (short)f32_to_bf16(d[cl][a] + d[cl][a + 8]);
                const bf16x8 bop = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
                for (int ot = 0; ot < kMaxOt; ++ot) {
                    if (ot < n_ot) {
                        const bf16x8 aw =
                            *reinterpret_cast<const bf16x8 *>(w_area + ((ot * kCh + cl) * 64 + lane) * 8);
                        yacc[ot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bop, yacc[ot], 0, 0, 0);
                    }
                }
            }
        }
    }
    // ---- epilogue: yacc[ot] row = output channel, column = longitude ----
    const int wo = px0 + pxw + col;
    if (wo < L) {
#pragma unroll
        for (int ot = 0; ot < kMaxOt; ++ot) {
            if (ot < n_ot) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int o = o_base + ot * 32 + 8 * (a >> 2) + 4 * h + (a & 3);
                    if (o < Co) y[(((int64_t)b * Co + o) * Ho + ho) * L + wo] = f32_to_bf16(yacc[ot][a]);
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

hipError_t launch_fused_mfma(const FusedMfmaLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.Co == 0) return hipSuccess;
    const int n_pxb = (a.Wo + a.npx - 1) / a.npx;
    const int n_ob = (a.Co + kMaxOt * 32 - 1) / (kMaxOt * 32);
    const int n_ot = std::min(kMaxOt, (a.Co + 31) / 32);
    const size_t lds = fused_mfma_lds_bytes(n_ot, a.max_piece_elems, a.max_blk);
    hipError_t e = hipFuncSetAttribute((const void *)fused_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_ob * n_pxb;
    const int vec = (a.s == 1 && a.Wo % 8 == 0 && ((int64_t)a.Hi * a.Wi) % 8 == 0 && ((uintptr_t)a.x % 16) == 0) ? 1 : 0;
    hipLaunchKernelGGL(fused_mfma_kernel, dim3((unsigned)nblk), dim3(a.npx / 32 * 64), lds, stream,
                       (const bf16_t *)a.x, (const bf16_t *)a.W, (bf16_t *)a.y, a.pieces, a.rows, a.block_xoff,
                       (const bf16_t *)a.adata, a.ho_piece, a.ho_order, a.B, a.C, a.Co, a.K, a.Ho, a.Wo, a.Hi, a.Wi,
                       a.s, a.npx, n_pxb, n_ob, n_ot, a.max_blk, vec);
    return hipGetLastError();
}

}  // namespace disco
