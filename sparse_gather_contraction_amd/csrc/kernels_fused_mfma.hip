// kernels_fused_mfma.hip — fused DISCO convolution on the gfx950 matrix cores.
//
// y[b,o,ho,wo] = sum_{c,k} W[o,c,k] * out[b,c,k,ho,wo], out = CSR contraction
// ("contraction + einsum", torch-harmonics "disco-kernel-dev" page,
// "Architecture snapshot"; its tensor-core forward takes psi in the bf16
// compute type, "kpacked layout" section — here psi is packed per source row
// instead, re-derived for MFMA).
//
// Workgroup = (b, ho, 256 output longitudes, up to 256 output channels), eight
// waves.  Waves w and w + 4 share the phase pair q = 2(w % 4) + {0, 1}: the 64
// longitudes px0 + 8n + q, n < 32.  Input channels are walked in chunks of
// kCh = 4; within a chunk the latitude's psi pieces are streamed (a "step" is
// one piece of one chunk):
//  * contraction (wave half h2 = w / 4 takes channels 2 h2, 2 h2 + 1 of the
//    chunk): per block (16 offsets d0..d0+15 of one source row) and channel,
//    one v_mfma_f32_32x32x16_bf16 with
//      A = psi rows (k, q) for the wave's two phases, P[k, d0 + t - q]
//          (eight 2-byte LDS reads per lane; one A serves both channels),
//      B = x[px0 + 8n + d0 + t], which is phase independent and read as one
//          aligned 16-byte LDS run per lane;
//  * einsum (wave half h2 takes half of the output-channel tiles): the result
//    rows are ordered so that a lane holds the reduction slots 8h..8h+7 =
//    basis k of one longitude for each phase, i.e. exactly the B operand of
//    v_mfma_f32_32x32x16_bf16 against W (A operand: W[o, c, 8h..8h+7],
//    contiguous in memory).  The two waves of a pair swap their channels'
//    operands (bf16) through LDS.  fp32 accumulators for 128 output channels
//    x 64 longitudes stay in registers across all chunks.
// Stage buffers are double-buffered: the next step's block descriptors, psi
// and x windows stream into LDS by direct global->LDS loads while the
// current step is contracted; the chunk's W slice likewise.  No atomics;
// every output is written once.
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "plan_fused.hpp"

namespace disco {

namespace {

constexpr int kCh = 4;          // input channels per chunk
constexpr int kMaxOt = 8;       // 32-row output-channel tiles per workgroup (256 channels)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWBytes = kMaxOt * kCh * 1024;  // W slice of one chunk
constexpr int kXchBytes = kWaves * 4 * 1024;  // operand exchange (2 channels x 2 phases per wave)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef void __attribute__((address_space(3))) *lptr_t;

// Raw buffer resource over `bytes` bytes at `base` (reads past the end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Direct global -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i of the
// instruction writes LDS base `l` + 16 i.  The buffer form (rather than the global form) keeps
// the compiler's LDS wait counting exact for the LDS reads that overlap the transfer.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *l)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l, 16, voff, 0, 0, 0);
}

struct Ctx {
    const bf16_t *x, *W;
    __amdgpu_buffer_rsrc_t descs_rs, adata_rs, w_rs;
    const FRow *rows;
    int B, C, Co, K, L, Wi, s, n_ot, b, px0, o_base, tid, wave, lane;
    int64_t plane_sz;
    int64_t x_bstride;  // elements between batches of x (C planes when contiguous)
    bool vec_x, vec_w;
    int x_half;  // s = 2: this lane reads the odd half of the split window area
    bool vec_out;  // contraction-only mode: output rows are 16-byte aligned (L, strides multiples of 8)
    float scale;  // contraction result scale: 2^-e for fp16 psi, 1 for bf16
    // contraction-only mode: out[b, c, k, ho, wo] at out + b * out_bstride
    bf16_t *out;
    int64_t out_bstride;
    int Ho, ho;
    // fused op that also keeps its contraction: save[b, c, k, ho, wo] at save + b * save_bstride
    bf16_t *save;
    int64_t save_bstride;
    bool vec_save;  // save rows are 16-byte aligned
};

// ---- 16-bit operand types ----------------------------------------------------------------------
// F16 selects fp16 data and psi (psi stored as fp16 of psi * 2^e, the plan's exponent e putting the
// largest |psi| near 2^14; the contraction result is scaled back by 2^-e exactly in fp32), else
// bf16.  Operands travel as raw 16-bit patterns.

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(i16x8 a, i16x8 b, f32x16 c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// fp32 -> 16-bit pattern, round to nearest even; fp16 values are scaled first (exact, a power of 2)
template <bool F16>
__device__ __forceinline__ short to16(float v, float scale)
{
    if constexpr (F16)
        return __builtin_bit_cast(short, (_Float16)(v * scale));
    else
        return __builtin_bit_cast(short, (__bf16)v);
}

template <bool F16>
__device__ __forceinline__ i16x8 to_op8(const f32x16 &v, int base, float scale)
{
    i16x8 r;
#pragma unroll
    for (int a = 0; a < 8; ++a) r[a] = to16<F16>(v[base + a], scale);
    return r;
}

// ---- staging ---------------------------------------------------------------------------------

// Contiguous global -> LDS copy of n16 16-byte units starting at byte voff of buffer r, spread
// over the workgroup (lane i of a wave's instruction writes base + 16 i).
__device__ __forceinline__ void copy_units(const Ctx &c, __amdgpu_buffer_rsrc_t r, uint32_t voff, unsigned char *dst,
                                           int n16)
{
    for (int u0 = c.wave * 64; u0 < n16; u0 += kThreads) {
        const int u = u0 + c.lane;
        if (u < n16) dma16(r, voff + 16u * (uint32_t)u, dst + 16 * u0);
    }
}

// x windows of one piece for the chunk starting at channel c0: window of row r holds input
// columns s px0 + start + i (mod Wi) of input latitude hi.  Rows go round the waves; a wave
// handles all channels of its rows (row data is read once, no integer division).
// With s = 2 a channel's window area keeps its 16-byte units split by parity: unit u (counted
// from the area's start; rows start at even units) sits at unit (u % 2) * (win_elems / 16) + u / 2.
// A lane's x runs are units 2 n + {0, 1} past the block's first, so the 64 lanes of a read then
// touch consecutive units of one half instead of every other unit (no LDS bank conflicts).
__device__ __forceinline__ int split_unit(int u, int half) { return (u & 1) * half + (u >> 1); }

template <int NCH>
__device__ __forceinline__ void stage_windows(const Ctx &c, const FPiece &pc, int c0, bf16_t *win)
{
    const int nrows = pc.row_end - pc.row_begin;
    const int ccn = min(NCH, c.C - c0);
    const bf16_t *plane0 = c.x + (int64_t)c.b * c.x_bstride + (int64_t)c0 * c.plane_sz;
    const bool split = c.s == 2;
    const int half = pc.win_elems >> 4;  // units per half of a split area
    for (int r = c.wave; r < nrows; r += kWaves) {
        const FRow fr = c.rows[pc.row_begin + r];
        const int nch = fr.len >> 3;
        const int u_row = fr.win_off >> 3;  // the row's first unit (even when split)
        int g0 = c.s * c.px0 + fr.start;  // within a few Wi of [0, Wi)
        while (g0 < 0) g0 += c.Wi;
        while (g0 >= c.Wi) g0 -= c.Wi;
        if (c.vec_x) {
            // Wi and g0 are multiples of 8: 8-column runs never straddle the row end.  One buffer
            // resource spans the chunk's channel planes.
            const uint32_t plane_bytes = 2u * (uint32_t)c.plane_sz;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(plane0, plane_bytes * (uint32_t)ccn);
            const uint32_t row0 = 2u * (uint32_t)(fr.sr * c.Wi);
            // units of one parity (split) or all units go to consecutive LDS units, one per lane
            const int npar = split ? 2 : 1, nu = split ? nch >> 1 : nch;
            for (int par = 0; par < npar; ++par) {
                bf16_t *dst = win + 8 * (split ? par * half + (u_row >> 1) : u_row);
                for (int t = 0; t < nu; t += 64) {
                    const int i = t + c.lane;
                    const int e8 = split ? 2 * i + par : i;  // unit of the row
                    int pos = g0 + 8 * e8;
                    while (pos >= c.Wi) pos -= c.Wi;
                    const uint32_t voff = row0 + 2u * (uint32_t)pos;
                    if (i < nu) {
                        for (int cl = 0; cl < ccn; ++cl) dma16(rs, voff + plane_bytes * cl, dst + cl * pc.win_elems + 8 * t);
                    }
                }
            }
        } else {
            const bf16_t *xrow = plane0 + (int64_t)fr.sr * c.Wi;
            for (int e = c.lane; e < fr.len; e += 64) {
                int pos = g0 + e;
                while (pos >= c.Wi) pos -= c.Wi;
                const int idx = split ? 8 * split_unit(u_row + (e >> 3), half) + (e & 7) : fr.win_off + e;
                for (int cl = 0; cl < ccn; ++cl) win[cl * pc.win_elems + idx] = xrow[cl * c.plane_sz + pos];
            }
        }
        for (int cl = ccn; cl < NCH; ++cl)  // channels past C are zeros
            for (int e8 = c.lane; e8 < nch; e8 += 64) {
                const int u = split ? split_unit(u_row + e8, half) : u_row + e8;
                *reinterpret_cast<uint4 *>(win + cl * pc.win_elems + 8 * u) = make_uint4(0u, 0u, 0u, 0u);
            }
    }
}

// Block descriptors and psi of piece pc.
__device__ __forceinline__ void stage_psi(const Ctx &c, const FPiece &pc, unsigned char *buf)
{
    copy_units(c, c.descs_rs, 8u * (uint32_t)pc.desc_begin, buf, pc.desc_words / 4);
    copy_units(c, c.adata_rs, 2u * (uint32_t)pc.a_begin, buf + 4 * pc.desc_words, pc.a_elems / 8);
}

// One step's stage: block descriptors, psi and windows of piece pc for channels c0..c0+NCH-1.
template <int NCH>
__device__ __forceinline__ void stage_step(const Ctx &c, const FPiece &pc, int c0, unsigned char *buf)
{
    stage_psi(c, pc, buf);
    stage_windows<NCH>(c, pc, c0, reinterpret_cast<bf16_t *>(buf + 4 * pc.desc_words + 2 * pc.a_elems));
}

// W slice of the chunk starting at c0 in A-operand order: unit (ot, cl), lane l holds
// W[o_base + 32 ot + l % 32, c0 + cl, 8 (l / 32) .. + 7].
__device__ __forceinline__ void stage_w(const Ctx &c, int c0, unsigned char *wb)
{
    const int o = c.o_base + (c.lane & 31);
    const int hh = c.lane >> 5;
    for (int u = c.wave; u < c.n_ot * kCh; u += kWaves) {
        const int ot = u / kCh, cl = u - ot * kCh;
        const int oo = o + 32 * ot, ch = c0 + cl;
        unsigned char *dst = wb + 1024 * u;
        const bool ok = oo < c.Co && ch < c.C;
        if (c.vec_w) {
            if (ok) dma16(c.w_rs, 2u * (uint32_t)(((int64_t)oo * c.C + ch) * 16 + 8 * hh), dst);
            else *reinterpret_cast<uint4 *>(dst + 16 * c.lane) = make_uint4(0u, 0u, 0u, 0u);
        } else {
            i16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 8 * hh + i;
                v[i] = (ok && k < c.K) ? (short)c.W[((int64_t)oo * c.C + ch) * c.K + k] : (short)0;
            }
            *reinterpret_cast<i16x8 *>(dst + 16 * c.lane) = v;
        }
    }
}

// ---- compute ---------------------------------------------------------------------------------

// Operands of one block: five 4-byte words of psi (pairs of consecutive offsets of one basis
// function; realigned at the point of use, so that the wait for them falls just before the
// MFMA) and the two channels' x runs.
template <bool PERM>
struct Ops {
    unsigned a[PERM ? 5 : 4];
    i16x8 b0, b1;
};

// KR: basis rows of the psi layout; one offset pair of psi spans KR 4-byte words.  Without PERM the
// lane's eight psi values are four aligned words (lanes whose phase shift is odd read the piece's
// second psi copy, whose words hold the offset pairs that start one offset later, and with s even
// no shift is odd); with PERM the piece holds one copy and an odd shift reads five words and
// realigns them.
template <int KR, bool PERM>
__device__ __forceinline__ void load_ops(Ops<PERM> &o, const unsigned char *a_base, const unsigned char *x_base,
                                         int wel2, int a_off, int x_off)
{
    o.b0 = *reinterpret_cast<const i16x8 *>(x_base + x_off);
    o.b1 = *reinterpret_cast<const i16x8 *>(x_base + wel2 + x_off);
    const unsigned *p = reinterpret_cast<const unsigned *>(a_base + a_off);
#pragma unroll
    for (int i = 0; i < (PERM ? 5 : 4); ++i) o.a[i] = p[KR * i];
}

// sel (PERM only): 0x03020100 (even first offset: words as read) or 0x05040302 (odd: shifted by one)
template <bool F16, bool PERM>
__device__ __forceinline__ void mfma_ops(const Ops<PERM> &o, unsigned sel, f32x16 (&d)[2])
{
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = PERM ? __builtin_amdgcn_perm(o.a[i + 1], o.a[i], sel) : o.a[i];
    const i16x8 a = __builtin_bit_cast(i16x8, w);
    d[0] = mfma32<F16>(a, o.b0, d[0]);
    d[1] = mfma32<F16>(a, o.b1, d[1]);
}

// Contraction of one step for the wave's two channels.  Blocks go in pairs (P, Q): the operands
// of one block are read while the other block's MFMAs run, and the descriptors of a pair are
// read two pairs ahead.  Scheduling barriers keep that order (the compiler would otherwise
// move the reads next to their uses).
template <int KR, bool PERM, bool F16>
__device__ __forceinline__ void contract_pairs(const unsigned char *__restrict__ stage, const unsigned char *a_base,
                                               const unsigned char *x_base, int wel2, int npair, unsigned sel,
                                               f32x16 (&d)[2])
{
    const int4 *desc = reinterpret_cast<const int4 *>(stage);
    const int lastp = npair - 1;
    int4 dA = desc[0];
    int4 dB = desc[min(1, lastp)];
    Ops<PERM> P, Q;
    load_ops<KR>(P, a_base, x_base, wel2, dA.x, dA.y);
    for (int j = 0; j < npair; ++j) {
        const int4 dC = desc[min(j + 2, lastp)];
        load_ops<KR>(Q, a_base, x_base, wel2, dA.z, dA.w);
        __builtin_amdgcn_sched_barrier(0);
        mfma_ops<F16>(P, sel, d);
        __builtin_amdgcn_sched_barrier(0);
        load_ops<KR>(P, a_base, x_base, wel2, dB.x, dB.y);
        __builtin_amdgcn_sched_barrier(0);
        mfma_ops<F16>(Q, sel, d);
        __builtin_amdgcn_sched_barrier(0);
        dA = dB;
        dB = dC;
    }
}

// odd: the lane's phase shift is odd (second psi copy, or the realigning selector); x_half: the
// lane reads the odd half of a split window area (s = 2)
template <int KR, bool F16>
__device__ __forceinline__ void contract(const unsigned char *__restrict__ stage, const unsigned char *__restrict__ win,
                                         const FPiece &pc, int a_lane2, int x_lane2, int x_half, bool odd, int ch0,
                                         f32x16 (&d)[2])
{
    const int npair = pc.nblk >> 1;
    if (npair <= 0) return;
    const unsigned char *a_base = stage + 4 * pc.desc_words + a_lane2;
    const int wel2 = 2 * pc.win_elems;
    const unsigned char *x_base = win + ch0 * wel2 + x_lane2 + x_half * pc.win_elems;
    if (pc.realign)
        contract_pairs<KR, true, F16>(stage, a_base, x_base, wel2, npair, odd ? 0x05040302u : 0x03020100u, d);
    else
        contract_pairs<KR, false, F16>(stage, a_base + (odd ? pc.a_copy_bytes : 0), x_base, wel2, npair, 0u, d);
}

// Einsum of a chunk: swap operands with the partner wave through `xch`, then accumulate the
// wave's NOT/2 output-channel tiles for both phases.  Caller: barrier before (everyone done with
// `xch` as a stage buffer, W slice visible).
template <int NOTH, bool F16>
__device__ __forceinline__ void einsum(unsigned char *__restrict__ xch, const unsigned char *__restrict__ wb,
                                       int lane, int pp, int h2, float scale, f32x16 (&d)[2],
                                       f32x16 (&yacc)[2][NOTH])
{
    i16x8 own[2][2], oth[2][2];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            own[cl][ph] = to_op8<F16>(d[cl], 8 * ph, scale);
            *reinterpret_cast<i16x8 *>(xch + 1024 * (((pp * 2 + h2) * 2 + cl) * 2 + ph) + 16 * lane) = own[cl][ph];
        }
    __syncthreads();
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int ph = 0; ph < 2; ++ph)
            oth[cl][ph] =
                *reinterpret_cast<const i16x8 *>(xch + 1024 * (((pp * 2 + (1 - h2)) * 2 + cl) * 2 + ph) + 16 * lane);
#pragma unroll
    for (int j = 0; j < NOTH; ++j) {
        const int ot = h2 * NOTH + j;
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
            const i16x8 wo = *reinterpret_cast<const i16x8 *>(wb + 1024 * (ot * kCh + 2 * h2 + cl) + 16 * lane);
            const i16x8 wt = *reinterpret_cast<const i16x8 *>(wb + 1024 * (ot * kCh + 2 * (1 - h2) + cl) + 16 * lane);
            yacc[0][j] = mfma32<F16>(wo, own[cl][0], yacc[0][j]);
            yacc[1][j] = mfma32<F16>(wo, own[cl][1], yacc[1][j]);
            yacc[0][j] = mfma32<F16>(wt, oth[cl][0], yacc[0][j]);
            yacc[1][j] = mfma32<F16>(wt, oth[cl][1], yacc[1][j]);
        }
    }
}

__device__ __forceinline__ void zero(f32x16 (&d)[2])
{
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int a = 0; a < 16; ++a) d[cl][a] = 0.0f;
}

// One step: wait for its stage, queue the next step's stage (and the chunk's W slice at a
// chunk start), contract, and run the einsum at the chunk's last piece (the consumed stage
// buffer then carries the operand exchange).  The buffers are restrict parameters so that the
// compiler keeps the queued direct loads in flight across the LDS reads of the current stage.
// Contraction-only mode: the chunk's contraction result (channels kCh t + 2 h2 + cl) goes through
// an LDS tile [channel][basis][256 longitudes] (the 32 KiB the fused op keeps for its W slice), so
// that each output row leaves as 16-byte stores rather than 2-byte stores 16 bytes apart.  With the
// basis order the psi rows were read in, register a of lane (n, hh) holds basis k = 8 hh + a % 8 of
// phase 2 pp + a / 8; registers a and a + 8 are neighbouring longitudes and share one LDS word.
// The tile is reused at the next chunk only after that chunk's opening barrier.
template <bool F16>
__device__ __forceinline__ void store_contraction(const Ctx &c, const f32x16 (&d)[2], int t, int pp, int h2,
                                                  unsigned char *__restrict__ tile_bytes)
{
    const int r = c.lane & 31, hh = c.lane >> 5;
    uint32_t *tile32 = reinterpret_cast<uint32_t *>(tile_bytes);
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t lo = (uint16_t)to16<F16>(d[cl][j], c.scale), hi = (uint16_t)to16<F16>(d[cl][j + 8], c.scale);
            tile32[(((2 * h2 + cl) * 16 + 8 * hh + j) * 256 + 8 * r + 2 * pp) >> 1] = lo | (hi << 16);
        }
    __syncthreads();
    const bf16_t *tile = reinterpret_cast<const bf16_t *>(tile_bytes);
    const int64_t HoL = (int64_t)c.Ho * c.L;
    for (int u = c.tid; u < kCh * 16 * 32; u += kThreads) {
        const int seg = u & 31, row = u >> 5, k = row & 15, ch = kCh * t + (row >> 4);
        const int wo = c.px0 + 8 * seg;
        if (k >= c.K || ch >= c.C || wo >= c.L) continue;
        bf16_t *dst = c.out + (int64_t)c.b * c.out_bstride + ((int64_t)ch * c.K + k) * HoL + (int64_t)c.ho * c.L + wo;
        const bf16_t *src = tile + row * 256 + 8 * seg;
        if (c.vec_out && wo + 8 <= c.L) {
            *reinterpret_cast<i16x8 *>(dst) = *reinterpret_cast<const i16x8 *>(src);
        } else {
            for (int e = 0; e < 8 && wo + e < c.L; ++e) dst[e] = src[e];
        }
    }
}

// Fused op that keeps its contraction: chunk t's result (channels kCh t .. + 3), read back from the
// einsum's operand exchange — the fp32 accumulators rounded to the data type, exactly the values
// the einsum multiplied and the values the contraction-only mode writes — to save[b, c, k, ho, ...]
// as 16-byte row segments (by the first output-channel block only: the others hold the same values).
// Exchange unit (pp, h2, cl, ph), lane (r, hh) holds basis 8 hh .. + 7 of longitude px0 + 8 r + 2 pp + ph,
// channel kCh t + 2 h2 + cl.  Thread (chl, hh, r, kh) reads the four bases 8 hh + 4 kh .. + 3 of its
// eight units (one 8-byte read each; the 64 lanes of a wave read 512 contiguous bytes, free of bank
// conflicts) and writes the four rows' eight longitudes px0 + 8 r .. + 7.  Called after the einsum
// (every wave's operands are in the exchange); the exchange is overwritten only after the next
// step's opening barrier.
__device__ __forceinline__ void save_contraction(const Ctx &c, const unsigned char *__restrict__ xch, int t)
{
    static_assert(kThreads == kCh * 2 * 32 * 2, "one thread per (channel, basis half, column, basis quarter)");
    const int kh = c.tid & 1, r = (c.tid >> 1) & 31, hh = (c.tid >> 6) & 1, chl = c.tid >> 7;
    const int ch = kCh * t + chl, wo = c.px0 + 8 * r, k0 = 8 * hh + 4 * kh;
    if (ch >= c.C || wo >= c.L || k0 >= c.K) return;
    const int h2 = chl >> 1, cl = chl & 1;
    const unsigned char *src = xch + 1024 * (h2 * 2 + cl) * 2 + 16 * (r + 32 * hh) + 8 * kh;
    uint2 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)  // q = 2 pp + ph: unit ((pp * 2 + h2) * 2 + cl) * 2 + ph
        v[q] = *reinterpret_cast<const uint2 *>(src + 1024 * (8 * (q >> 1) + (q & 1)));
    const int64_t HoL = (int64_t)c.Ho * c.L;
    bf16_t *dst0 = c.save + (int64_t)c.b * c.save_bstride + ((int64_t)ch * c.K + k0) * HoL + (int64_t)c.ho * c.L + wo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (k0 + j >= c.K) break;
        uint32_t h[8];  // basis k0 + j of the eight longitudes
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t w = (j < 2) ? v[q].x : v[q].y;
            h[q] = (j & 1) ? (w >> 16) : (w & 0xffffu);
        }
        bf16_t *dst = dst0 + (int64_t)j * HoL;
        if (c.vec_save && wo + 8 <= c.L) {
            uint4 o;
            o.x = h[0] | (h[1] << 16);
            o.y = h[2] | (h[3] << 16);
            o.z = h[4] | (h[5] << 16);
            o.w = h[6] | (h[7] << 16);
            *reinterpret_cast<uint4 *>(dst) = o;
        } else {
            for (int e = 0; e < 8 && wo + e < c.L; ++e) dst[e] = (bf16_t)h[e];
        }
    }
}

// Zero rows of a contraction (B, C, K, Ho, L) at dst for this workgroup's latitude and span: a latitude
// without psi entries has no pieces, so no step writes its rows.
__device__ __forceinline__ void zero_contraction(const Ctx &c, bf16_t *dst, int64_t bstride, bool vec)
{
    const int64_t HoL = (int64_t)c.Ho * c.L;
    for (int u = c.tid; u < c.C * c.K * 32; u += kThreads) {
        const int seg = u & 31, row = u >> 5, k = row % c.K, ch = row / c.K;
        const int wo = c.px0 + 8 * seg;
        if (wo >= c.L) continue;
        bf16_t *p = dst + (int64_t)c.b * bstride + ((int64_t)ch * c.K + k) * HoL + (int64_t)c.ho * c.L + wo;
        if (vec && wo + 8 <= c.L) {
            *reinterpret_cast<uint4 *>(p) = make_uint4(0u, 0u, 0u, 0u);
        } else {
            for (int e = 0; e < 8 && wo + e < c.L; ++e) p[e] = 0;
        }
    }
}

// EIN: fused op (einsum into yacc); else contraction-only (the chunk's result is written out).
// SAVE (with EIN): the fused op also writes each chunk's contraction to c.save.
template <int NOTH, bool F16, bool EIN, bool SAVE = false>
__device__ __forceinline__ void run_step(const Ctx &c, const FPiece *__restrict__ pieces, int p_begin, int npieces,
                                         int nsteps, int st, int t, int p, unsigned char *__restrict__ cur,
                                         unsigned char *__restrict__ nxt, unsigned char *__restrict__ wb, int a_lane2,
                                         int x_lane2, bool odd, int pp, int h2, f32x16 (&d)[2], f32x16 (&yacc)[2][NOTH])
{
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads into `cur` (and W) have landed
    __syncthreads();                // everyone's have; the previous step is done with `nxt` and W
    if (EIN && p == 0 && t > 0) stage_w(c, kCh * t, wb);
    if (st + 1 < nsteps) {
        const int p1 = (p + 1 == npieces) ? 0 : p + 1;
        const int t1 = (p + 1 == npieces) ? t + 1 : t;
        stage_step<kCh>(c, pieces[p_begin + p1], kCh * t1, nxt);
    }
    if (p == 0) zero(d);
    const FPiece pc = pieces[p_begin + p];
    contract<16, F16>(cur, cur + 4 * pc.desc_words + 2 * pc.a_elems, pc, a_lane2, x_lane2, c.x_half, odd, 2 * h2, d);
    if (p + 1 == npieces) {
        if constexpr (EIN) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // W slice visible; `cur` free for the exchange
            einsum<NOTH, F16>(cur, wb, c.lane, pp, h2, c.scale, d, yacc);
            if constexpr (SAVE) {
                if (c.o_base == 0) save_contraction(c, cur, t);  // one output-channel block writes it
            }
        } else {
            store_contraction<F16>(c, d, t, pp, h2, wb);
        }
    }
}

// One chunk of a latitude whose psi stays resident: only the x windows stream (double-buffered).
template <int NOTH, bool F16, bool EIN, bool SAVE = false>
__device__ __forceinline__ void run_chunk_resident(const Ctx &c, const FPiece &pc, int nchunks, int t,
                                                   const unsigned char *__restrict__ stage,
                                                   unsigned char *__restrict__ cur, unsigned char *__restrict__ nxt,
                                                   unsigned char *__restrict__ wb, int a_lane2, int x_lane2,
                                                   bool odd, int pp, int h2, f32x16 (&d)[2],
                                                   f32x16 (&yacc)[2][NOTH])
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (EIN && t > 0) stage_w(c, kCh * t, wb);
    if (t + 1 < nchunks) stage_windows<kCh>(c, pc, kCh * (t + 1), reinterpret_cast<bf16_t *>(nxt));
    zero(d);
    contract<16, F16>(stage, cur, pc, a_lane2, x_lane2, c.x_half, odd, 2 * h2, d);
    if constexpr (EIN) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // W slice visible; `cur` free for the exchange
        einsum<NOTH, F16>(cur, wb, c.lane, pp, h2, c.scale, d, yacc);
        if constexpr (SAVE) {
            if (c.o_base == 0) save_contraction(c, cur, t);  // one output-channel block writes it
        }
    } else {
        store_contraction<F16>(c, d, t, pp, h2, wb);
    }
}

template <int NOT, bool F16, bool EIN, bool SAVE = false>
__global__ __launch_bounds__(kThreads) void fused_mfma_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ W, bf16_t *__restrict__ y,
    const FPiece *__restrict__ pieces, const FRow *__restrict__ rows, const int32_t *__restrict__ descs,
    const bf16_t *__restrict__ adata, const int32_t *__restrict__ ho_piece, const int32_t *__restrict__ ho_order,
    int B, int C, int Co, int K, int Ho, int L, int Hi, int Wi, int s, int n_pxb, int n_ob, int buf_bytes,
    uint32_t desc_bytes, uint32_t adata_bytes, int vec_x, int vec_w, int vec_out, float scale, int64_t x_bstride,
    int64_t out_bstride, bf16_t *__restrict__ save, int64_t save_bstride, int vec_save)
{
    // vec_w: W rows load as 16-byte runs; vec_out: output rows (y, or out in contraction-only mode) start 16-byte aligned
    constexpr int NOTH = NOT / 2;
    // LDS: [W slice: NOT * kCh KiB; contraction-only: the 32 KiB output tile] [stage buffer 0] [stage buffer 1]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *wb = smem;
    unsigned char *buf0 = smem + (EIN ? NOT * kCh * 1024 : kWBytes);
    unsigned char *buf1 = buf0 + buf_bytes;

    int bid = blockIdx.x;
    const int pxb = bid % n_pxb;
    bid /= n_pxb;
    const int ob = bid % n_ob;
    bid /= n_ob;
    Ctx c;
    c.b = bid % B;
    const int ho = ho_order[bid / B];
    c.x = x; c.W = W; c.rows = rows;
    c.descs_rs = make_rsrc(descs, desc_bytes);
    c.adata_rs = make_rsrc(adata, adata_bytes);
    c.w_rs = make_rsrc(W, vec_w ? (uint32_t)(2 * (int64_t)Co * C * 16) : 0u);
    c.B = B; c.C = C; c.Co = Co; c.K = K; c.L = L; c.Wi = Wi; c.s = s; c.n_ot = NOT;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.px0 = pxb * kFusedSpan;
    c.o_base = ob * (kMaxOt * 32);
    c.plane_sz = (int64_t)Hi * Wi;
    c.x_bstride = x_bstride;
    c.vec_x = vec_x != 0;
    c.vec_w = EIN && vec_w != 0;
    c.vec_out = vec_out != 0;
    c.scale = scale;
    c.out = y;
    c.out_bstride = out_bstride;
    c.Ho = Ho;
    c.ho = ho;
    c.save = save;
    c.save_bstride = save_bstride;
    c.vec_save = vec_save != 0;

    // lane constants: A row r = lane % 32 is (phase 2 pp + r / 16, MFMA row m = r % 16 -> basis k);
    // the basis order puts k = 8h + a in result register a of lane half h
    const int pp = c.wave & 3, h2 = c.wave >> 2;
    const int r = c.lane & 31, hh = c.lane >> 5;
    const int m = r & 15;
    const int kb = (m < 8) ? 8 * (m >> 2) + (m & 3) : 8 * ((m - 8) >> 2) + 4 + (m & 3);
    // psi words: offset pair (base + 8 hh - s q) / 2 rounded down, basis kb; an odd shift reads the
    // second copy, whose pair m starts at offset 2 m + 1
    const int q = 2 * pp + (r >> 4), sq = s * q;
    const int a_lane2 = 64 * (4 * hh - (sq + 1) / 2) + 4 * kb;  // bytes
    const bool odd = (sq & 1) != 0;  // reads the second psi copy
    // x runs: units s n + hh past the block's first (bytes); with s = 2 the area is split by parity
    const int x_lane2 = s == 2 ? 16 * r : 2 * (8 * s * r + 8 * hh);
    c.x_half = s == 2 ? hh : 0;

    f32x16 yacc[2][NOTH];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph)
#pragma unroll
        for (int j = 0; j < NOTH; ++j)
#pragma unroll
            for (int a = 0; a < 16; ++a) yacc[ph][j][a] = 0.0f;
    f32x16 d[2];
    zero(d);

    const int p_begin = ho_piece[ho];
    const int npieces = ho_piece[ho + 1] - p_begin;
    const int nchunks = (C + kCh - 1) / kCh;
    const int nsteps = npieces * nchunks;
    FPiece pc0;
    pc0.resident = 0;
    if (npieces == 1) pc0 = pieces[p_begin];
    if (npieces == 1 && pc0.resident) {
        // LDS after W: [descriptors + psi][window buffer 0][window buffer 1]
        unsigned char *stage = buf0;
        unsigned char *w0 = stage + 4 * pc0.desc_words + 2 * pc0.a_elems;
        unsigned char *w1 = w0 + pc0.resident;
        if (EIN) stage_w(c, 0, wb);
        stage_psi(c, pc0, stage);
        stage_windows<kCh>(c, pc0, 0, reinterpret_cast<bf16_t *>(w0));
        for (int t = 0; t < nchunks; t += 2) {
            run_chunk_resident<NOTH, F16, EIN, SAVE>(c, pc0, nchunks, t, stage, w0, w1, wb, a_lane2, x_lane2, odd, pp, h2, d,
                                               yacc);
            if (t + 1 < nchunks)
                run_chunk_resident<NOTH, F16, EIN, SAVE>(c, pc0, nchunks, t + 1, stage, w1, w0, wb, a_lane2, x_lane2, odd, pp, h2, d,
                                         yacc);
        }
    } else if (nsteps > 0) {
        if (EIN) stage_w(c, 0, wb);
        stage_step<kCh>(c, pieces[p_begin], 0, buf0);
        int t = 0, p = 0;
        for (int st = 0; st < nsteps; st += 2) {
            run_step<NOTH, F16, EIN, SAVE>(c, pieces, p_begin, npieces, nsteps, st, t, p, buf0, buf1, wb, a_lane2, x_lane2, odd, pp, h2, d,
                           yacc);
            if (++p == npieces) { p = 0; ++t; }
            if (st + 1 < nsteps) {
                run_step<NOTH, F16, EIN, SAVE>(c, pieces, p_begin, npieces, nsteps, st + 1, t, p, buf1, buf0, wb, a_lane2, x_lane2, odd, pp,
                               h2, d, yacc);
                if (++p == npieces) { p = 0; ++t; }
            }
        }
    } else {
        // no psi entries at this latitude: the contraction is zero (y gets zeros from the epilogue)
        if constexpr (!EIN) zero_contraction(c, c.out, c.out_bstride, c.vec_out);
        if constexpr (SAVE) {
            if (c.o_base == 0) zero_contraction(c, c.save, c.save_bstride, c.vec_save);
        }
    }

    // ---- epilogue: yacc[ph][j] row = output channel (h2 NOTH + j) 32 + 8 (a / 4) + 4 hh + a % 4, column
    // n = longitude px0 + 8n + 2 pp + ph.  Pass j writes the 64 channels of tile j of both wave halves
    // through a 32 KiB LDS tile [channel][256 longitudes] (stage buffer space, free once the last chunk
    // is done), so that output rows leave as 16-byte stores; the two phases of a register share a word.
    if constexpr (!EIN) return;
    uint32_t *tile32 = reinterpret_cast<uint32_t *>(buf0);
    const bf16_t *tile = reinterpret_cast<const bf16_t *>(buf0);
#pragma unroll
    for (int j = 0; j < NOTH; ++j) {
        __syncthreads();  // the last chunk (or the previous pass) is done with the tile's space
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int ol = 32 * h2 + 8 * (a >> 2) + 4 * hh + (a & 3);
            const uint32_t lo = (uint16_t)to16<F16>(yacc[0][j][a], 1.0f), hi = (uint16_t)to16<F16>(yacc[1][j][a], 1.0f);
            tile32[(ol * 256 + 8 * r + 2 * pp) >> 1] = lo | (hi << 16);
        }
        __syncthreads();
        for (int u = c.tid; u < 64 * 32; u += kThreads) {
            const int seg = u & 31, ol = u >> 5;
            const int o = c.o_base + ((ol >> 5) * NOTH + j) * 32 + (ol & 31), wo = c.px0 + 8 * seg;
            if (o >= Co || wo >= L) continue;
            bf16_t *dst = y + (((int64_t)c.b * Co + o) * Ho + ho) * L + wo;
            const bf16_t *src = tile + ol * 256 + 8 * seg;
            if (c.vec_out && wo + 8 <= L) {
                *reinterpret_cast<i16x8 *>(dst) = *reinterpret_cast<const i16x8 *>(src);
            } else {
                for (int e = 0; e < 8 && wo + e < L; ++e) dst[e] = src[e];
            }
        }
    }
}


// ---- forward contraction on the matrix cores -------------------------------------------------
//
// out[b,c,k,ho,wo] for bf16 inputs (the "kpacked" tensor-core forward of the torch-harmonics
// "disco-kernel-dev" page, re-derived with the same phase-split psi as the fused kernel).
// Workgroup = (b, ho, 256 output longitudes, FCH channels), eight waves: wave w takes phase group
// g = w % NG (PH = 32/KR phases per MFMA) and channel pair w / NG.  The latitude's pieces stream
// through two LDS stage buffers (two workgroups share a CU, so one computes while the other
// waits for its stage); every output element is written once, from its accumulator.

template <int KR, int FCH, bool F16>
__device__ __forceinline__ void fwd_step(const Ctx &c, const FPiece *__restrict__ pieces, int p_begin, int npieces,
                                         int p, int c0, unsigned char *__restrict__ cur,
                                         unsigned char *__restrict__ nxt, int a_lane2, int x_lane2, bool odd,
                                         int cp, f32x16 (&d)[2])
{
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads into `cur` have landed
    __syncthreads();                // everyone's have; the previous step is done with `nxt`
    if (p + 1 < npieces) stage_step<FCH>(c, pieces[p_begin + p + 1], c0, nxt);
    const FPiece pc = pieces[p_begin + p];
    contract<KR, F16>(cur, cur + 4 * pc.desc_words + 2 * pc.a_elems, pc, a_lane2, x_lane2, c.x_half, odd, 2 * cp, d);
}

template <int KR, bool F16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void fwd_mfma_kernel(
    const bf16_t *__restrict__ x, bf16_t *__restrict__ out, const FPiece *__restrict__ pieces,
    const FRow *__restrict__ rows, const int32_t *__restrict__ descs, const bf16_t *__restrict__ adata,
    const int32_t *__restrict__ ho_piece, const int32_t *__restrict__ ho_order, int B, int C, int K, int Ho, int L,
    int Hi, int Wi, int s, int n_pxb, int n_cb, int buf_bytes, uint32_t desc_bytes, uint32_t adata_bytes, int vec_x,
    OutMap om, float scale, int64_t x_bstride, int64_t out_bstride, int vec_out)
{
    // vec_out: output rows start 16-byte aligned (row length, plane and batch strides multiples of 8)
    constexpr int PH = 32 / KR, NG = 8 / PH, WPG = kWaves / NG, FCH = 2 * WPG;
    static_assert(FCH * KR * 256 * 2 == 32768, "the epilogue tile is 32 KiB");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *buf0 = smem;
    unsigned char *buf1 = smem + buf_bytes;

    int bid = blockIdx.x;
    const int pxb = bid % n_pxb;
    bid /= n_pxb;
    const int cb = bid % n_cb;
    bid /= n_cb;
    Ctx c;
    c.b = bid % B;
    const int ho = ho_order[bid / B];
    c.x = x; c.W = nullptr; c.rows = rows;
    c.descs_rs = make_rsrc(descs, desc_bytes);
    c.adata_rs = make_rsrc(adata, adata_bytes);
    c.w_rs = make_rsrc(nullptr, 0u);
    c.B = B; c.C = C; c.Co = 0; c.K = K; c.L = L; c.Wi = Wi; c.s = s; c.n_ot = 0;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.px0 = pxb * kFusedSpan;
    c.o_base = 0;
    c.plane_sz = (int64_t)Hi * Wi;
    c.x_bstride = x_bstride;
    c.vec_x = vec_x != 0;
    c.vec_w = false;
    c.vec_out = false;
    c.scale = scale;

    // lane constants: A row r = lane % 32 is (phase PH g + r / KR, basis k = r % KR)
    const int g = c.wave % NG, cp = c.wave / NG;
    const int r = c.lane & 31, hh = c.lane >> 5;
    const int q = PH * g + r / KR, sq = s * q;
    const int a_lane2 = 4 * KR * (4 * hh - (sq + 1) / 2) + 4 * (r % KR);  // bytes
    const bool odd = (sq & 1) != 0;  // reads the second psi copy
    // x runs: units s n + hh past the block's first (bytes); with s = 2 the area is split by parity
    const int x_lane2 = s == 2 ? 16 * r : 2 * (8 * s * r + 8 * hh);
    c.x_half = s == 2 ? hh : 0;

    f32x16 d[2];
    zero(d);
    const int p_begin = ho_piece[ho];
    const int npieces = ho_piece[ho + 1] - p_begin;
    const int c0 = cb * FCH;
    if (npieces > 0) {
        stage_step<FCH>(c, pieces[p_begin], c0, buf0);
        for (int p = 0; p < npieces; p += 2) {
            fwd_step<KR, FCH, F16>(c, pieces, p_begin, npieces, p, c0, buf0, buf1, a_lane2, x_lane2, odd, cp, d);
            if (p + 1 < npieces)
                fwd_step<KR, FCH, F16>(c, pieces, p_begin, npieces, p + 1, c0, buf1, buf0, a_lane2, x_lane2, odd, cp, d);
        }
    }

    // ---- epilogue: register a of lane (n = r, hh) is row 8 (a / 4) + 4 hh + a % 4 = (phase, k) ----
    // The block's result goes through an LDS tile so that output rows leave as 16-byte stores.  Forward
    // layout: tile [channel][k][256 longitudes], row (c, k) is out[b, c, k, ho, px0 ...].  Gradient
    // layout: the KR rows of group ho are input rows hi = (ho KR + k) / s with residue (ho KR + k) % s
    // at longitude s wo + residue, so the tile is [channel][KR / s][s 256] and row (c, j) is
    // gx[b, c, ho KR / s + j, s px0 ...]; this needs KR % s == 0, else the 2-byte stores below.
    const int sr = om.inverse ? om.s : 1;
    if (sr > 0 && KR % sr == 0) {
        __syncthreads();  // every wave is done with the stage buffers
        bf16_t *tile = reinterpret_cast<bf16_t *>(smem);
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int row = 8 * (a >> 2) + 4 * hh + (a & 3);
                const int k = row % KR, wl = 8 * r + PH * g + row / KR;
                tile[((2 * cp + cl) * KR + k - k % sr) * 256 + sr * wl + k % sr] = (bf16_t)to16<F16>(d[cl][a], scale);
            }
        __syncthreads();
        const int row_len = om.inverse ? om.wi : L;  // elements of an output row
        const int seg_per_row = 32 * sr, rows_per_ch = KR / sr;
        for (int u = c.tid; u < FCH * KR * 32; u += kThreads) {
            const int ch_l = u / (KR * 32), v = u - ch_l * (KR * 32);
            const int j = v / seg_per_row, seg = v - j * seg_per_row;
            const int cc = c0 + ch_l;
            const int pos = sr * c.px0 + 8 * seg;  // first element of the segment within its output row
            if (cc >= C || pos >= row_len) continue;
            int64_t row_off;
            if (om.inverse) {
                const int rr = ho * KR + j * sr;  // first of the sr rows that share input row rr / sr
                if (rr >= om.rows) continue;
                row_off = (int64_t)(rr / sr) * om.wi;
            } else {
                if (j >= K) continue;
                row_off = ((int64_t)j * Ho + ho) * L;
            }
            bf16_t *dst = out + (int64_t)c.b * out_bstride + (int64_t)cc * om.plane + row_off + pos;
            const bf16_t *src = tile + (ch_l * rows_per_ch + j) * (256 * sr) + 8 * seg;
            if (vec_out && pos + 8 <= row_len) {
                *reinterpret_cast<i16x8 *>(dst) = *reinterpret_cast<const i16x8 *>(src);
            } else {
                for (int e = 0; e < 8 && pos + e < row_len; ++e) dst[e] = src[e];
            }
        }
        return;
    }
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const int cc = c0 + 2 * cp + cl;
        if (cc >= C) continue;
        bf16_t *plane = out + (int64_t)c.b * out_bstride + (int64_t)cc * om.plane;
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int row = 8 * (a >> 2) + 4 * hh + (a & 3);
            const int k = row % KR, wo = c.px0 + 8 * r + PH * g + row / KR;
            if (k >= K || wo >= L) continue;
            if (om.inverse) {
                // row ho * KR + k is input row hi = row / s, residue row % s of the gradient
                const int rr = ho * KR + k;
                if (rr < om.rows) {
                    const int hi = rr / om.s;
                    plane[(int64_t)hi * om.wi + (rr - hi * om.s) + (int64_t)om.s * wo] = (bf16_t)to16<F16>(d[cl][a], scale);
                }
            } else {
                plane[((int64_t)k * Ho + ho) * L + wo] = (bf16_t)to16<F16>(d[cl][a], scale);
            }
        }
    }
}

}  // namespace

int fused_mfma_channels_per_chunk() { return kCh; }

int fwd_mfma_channels(int kr) { return kr == 8 ? 8 : 4; }

// Allow kernel `fn` `lds` bytes of dynamic LDS on the current device.  The request is checked on the
// host against the device's per-workgroup LDS (an oversized request returns hipErrorInvalidValue and
// nothing is launched), and hipFuncSetAttribute runs only when a kernel needs more than it was last
// given on that device (once per kernel and device in steady state).  DISCO_TEST_LDS_EXTRA (a test
// knob) adds bytes to every request, so tests can make a launch exceed the device and see the refusal.
hipError_t allow_lds(const void *fn, size_t lds)
{
    if (const char *x = getenv("DISCO_TEST_LDS_EXTRA")) lds += (size_t)std::max(0L, atol(x));
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::vector<int> dev_max(64, -1);
    static std::vector<std::pair<std::pair<const void *, int>, size_t>> granted;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (dev_max[dev] < 0) {
        int v = 0;
        if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return e;
        dev_max[dev] = v;
    }
    if (lds > (size_t)dev_max[dev]) return hipErrorInvalidValue;
    for (auto &g : granted)
        if (g.first.first == fn && g.first.second == dev) {
            if (lds <= g.second) return hipSuccess;
            if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
                return e;
            g.second = lds;
            return hipSuccess;
        }
    if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess) return e;
    granted.push_back({{fn, dev}, lds});
    return hipSuccess;
}

hipError_t launch_fwd_mfma(const FwdMfmaLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.C == 0) return hipSuccess;
    const int fch = fwd_mfma_channels(a.kr);
    const int n_pxb = (a.Wo + kFusedSpan - 1) / kFusedSpan;
    const int n_cb = (a.C + fch - 1) / fch;
    const int buf_bytes = (a.max_piece_bytes + 15) & ~15;
    const size_t lds = std::max<size_t>(2 * (size_t)buf_bytes, 32768);  // stage buffers; the epilogue's tile
    const void *fn = a.kr == 8 ? (a.f16 ? (const void *)fwd_mfma_kernel<8, true> : (const void *)fwd_mfma_kernel<8, false>)
                               : (a.f16 ? (const void *)fwd_mfma_kernel<16, true> : (const void *)fwd_mfma_kernel<16, false>);
    hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_cb * n_pxb;
    const int64_t x_bs = a.x_bstride > 0 ? a.x_bstride : (int64_t)a.C * a.Hi * a.Wi;
    const int64_t out_bs = a.out_bstride > 0 ? a.out_bstride : (int64_t)a.C * a.om.plane;
    const bool planes16 = ((int64_t)a.Hi * a.Wi) % 8 == 0 && a.Wi % 8 == 0 && ((uintptr_t)a.x % 16) == 0 &&
                          (int64_t)a.Hi * a.Wi * 2 * fch < ((int64_t)1 << 31);
    const int vec_x = planes16 && (x_bs % 8) == 0 ? 1 : 0;
    const int64_t row_len = a.om.inverse ? a.om.wi : a.Wo;
    const int vec_out = (row_len % 8 == 0 && a.om.plane % 8 == 0 && out_bs % 8 == 0 && ((uintptr_t)a.out % 16) == 0) ? 1 : 0;
#define DISCO_FWD_LAUNCH(KR, F16)                                                                                   \
    hipLaunchKernelGGL((fwd_mfma_kernel<KR, F16>), dim3((unsigned)nblk), dim3(kThreads), lds, stream,             \
                       (const bf16_t *)a.x, (bf16_t *)a.out, a.pieces, a.rows, a.descs, (const bf16_t *)a.adata,       \
                       a.ho_piece, a.ho_order, a.B, a.C, a.K, a.Ho, a.Wo, a.Hi, a.Wi, a.s, n_pxb, n_cb, buf_bytes,    \
                       a.desc_bytes, a.adata_bytes, vec_x, a.om, a.scale, x_bs, out_bs, vec_out)
    if (a.kr == 8) {
        if (a.f16) DISCO_FWD_LAUNCH(8, true);
        else DISCO_FWD_LAUNCH(8, false);
    } else {
        if (a.f16) DISCO_FWD_LAUNCH(16, true);
        else DISCO_FWD_LAUNCH(16, false);
    }
#undef DISCO_FWD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_fused_contract(const FusedContractLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.C == 0) return hipSuccess;
    const int n_pxb = (a.Wo + kFusedSpan - 1) / kFusedSpan;
    const int buf_bytes = std::max((a.max_piece_bytes + 15) & ~15, kXchBytes);
    const size_t lds = fused_mfma_lds_bytes(kMaxOt, a.max_piece_bytes, a.max_resident_bytes);  // 32 KiB output tile
    const void *fn = a.f16 ? (const void *)fused_mfma_kernel<2, true, false> : (const void *)fused_mfma_kernel<2, false, false>;
    hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_pxb;
    const int64_t x_bs = a.x_bstride > 0 ? a.x_bstride : (int64_t)a.C * a.Hi * a.Wi;
    const int64_t out_bs = a.out_bstride > 0 ? a.out_bstride : (int64_t)a.C * a.K * a.Ho * a.Wo;
    const bool planes16 = ((int64_t)a.Hi * a.Wi) % 8 == 0 && a.Wi % 8 == 0 && ((uintptr_t)a.x % 16) == 0 &&
                          x_bs % 8 == 0 && (int64_t)a.Hi * a.Wi * 2 * kCh < ((int64_t)1 << 31);
    const int vec_x = planes16 ? 1 : 0;
    const int vec_out = (a.Wo % 8 == 0 && out_bs % 8 == 0 && ((uintptr_t)a.out % 16) == 0) ? 1 : 0;
#define DISCO_CONTRACT_LAUNCH(F16)                                                                               \
    hipLaunchKernelGGL((fused_mfma_kernel<2, F16, false>), dim3((unsigned)nblk), dim3(kThreads), lds, stream,      \
                       (const bf16_t *)a.x, (const bf16_t *)nullptr, (bf16_t *)a.out, a.pieces, a.rows, a.descs,      \
                       (const bf16_t *)a.adata, a.ho_piece, a.ho_order, a.B, a.C, 0, a.K, a.Ho, a.Wo, a.Hi, a.Wi,     \
                       a.s, n_pxb, 1, buf_bytes, a.desc_bytes, a.adata_bytes, vec_x, 0, vec_out, a.scale, x_bs, out_bs,  \
                       (bf16_t *)nullptr, (int64_t)0, 0)
    if (a.f16) DISCO_CONTRACT_LAUNCH(true);
    else DISCO_CONTRACT_LAUNCH(false);
#undef DISCO_CONTRACT_LAUNCH
    return hipGetLastError();
}

int fused_mfma_exchange_bytes() { return kXchBytes; }

size_t fused_mfma_reserved_bytes() { return (size_t)kWBytes; }

size_t fused_mfma_lds_bytes(int n_ot, int max_piece_bytes, int max_resident_bytes)
{
    const size_t buf = std::max<size_t>(((size_t)max_piece_bytes + 15) & ~(size_t)15, (size_t)kXchBytes);
    return (size_t)n_ot * kCh * 1024 + std::max<size_t>(2 * buf, (size_t)max_resident_bytes);
}

namespace {

// Wp[(o C + c) 16 + k] = W[(o C + c) K + k] for k < K, else 0: W in the 16-element rows the fused
// kernel's direct W-slice loads read (one thread per output element).
__global__ __launch_bounds__(256) void pack_w16_kernel(const bf16_t *__restrict__ W, bf16_t *__restrict__ Wp,
                                                       int64_t rows, int K)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * 16) return;
    const int64_t r = i >> 4;
    const int k = (int)(i & 15);
    Wp[i] = k < K ? W[r * K + k] : (bf16_t)0;
}

}  // namespace

hipError_t launch_pack_w16(const void *W, void *Wp, int Co, int C, int K, hipStream_t stream)
{
    const int64_t rows = (int64_t)Co * C;
    if (rows == 0) return hipSuccess;
    if (K < 1 || K > 16) return hipErrorInvalidValue;
    const int64_t n = rows * 16;
    hipLaunchKernelGGL(pack_w16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, (const bf16_t *)W,
                       (bf16_t *)Wp, rows, K);
    return hipGetLastError();
}

hipError_t launch_fused_mfma(const FusedMfmaLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.Co == 0) return hipSuccess;
    const int n_pxb = (a.Wo + kFusedSpan - 1) / kFusedSpan;
    const int n_ob = (a.Co + kMaxOt * 32 - 1) / (kMaxOt * 32);
    const int n_ot1 = std::min(kMaxOt, (a.Co + 31) / 32);
    const int n_ot = n_ot1 <= 2 ? 2 : n_ot1 <= 4 ? 4 : 8;  // tiles past Co hold zero W
    const int buf_bytes = std::max((a.max_piece_bytes + 15) & ~15, kXchBytes);
    const size_t lds = fused_mfma_lds_bytes(n_ot, a.max_piece_bytes, a.max_resident_bytes);
    const bool sv = a.save != nullptr;
#define DISCO_FUSED_FN(N, F16) (sv ? (const void *)fused_mfma_kernel<N, F16, true, true> : (const void *)fused_mfma_kernel<N, F16, true, false>)
    const void *fn = a.f16 ? (n_ot == 2 ? DISCO_FUSED_FN(2, true) : n_ot == 4 ? DISCO_FUSED_FN(4, true) : DISCO_FUSED_FN(8, true))
                           : (n_ot == 2 ? DISCO_FUSED_FN(2, false) : n_ot == 4 ? DISCO_FUSED_FN(4, false) : DISCO_FUSED_FN(8, false));
#undef DISCO_FUSED_FN
    hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * a.Ho * n_ob * n_pxb;
    // direct loads need 16-byte aligned runs and buffer offsets below 2^31
    const bool planes16 = ((int64_t)a.Hi * a.Wi) % 8 == 0 && a.Wi % 8 == 0 && ((uintptr_t)a.x % 16) == 0 &&
                          (int64_t)a.Hi * a.Wi * 2 * kCh < ((int64_t)1 << 31);
    const int vec_x = planes16 ? 1 : 0;
    // W rows of 16 elements (K = 16, or W packed by launch_pack_w16): the slice arrives by direct loads
    const int vec_w = ((a.K == 16 || a.w16) && ((uintptr_t)a.W % 16) == 0 && (int64_t)a.Co * a.C * 32 < ((int64_t)1 << 31)) ? 1 : 0;
    const int vec_y = (a.Wo % 8 == 0 && ((uintptr_t)a.y % 16) == 0) ? 1 : 0;
    const int64_t x_bs = (int64_t)a.C * a.Hi * a.Wi;
    const int64_t save_bs = (int64_t)a.C * a.K * a.Ho * a.Wo;  // save is (B, C, K, Ho, Wo), contiguous
    const int vec_save = (sv && a.Wo % 8 == 0 && ((uintptr_t)a.save % 16) == 0) ? 1 : 0;
#define DISCO_FUSED_LAUNCH(N, F16)                                                                               \
    if (sv)                                                                                                      \
        hipLaunchKernelGGL((fused_mfma_kernel<N, F16, true, true>), dim3((unsigned)nblk), dim3(kThreads), lds,     \
                           stream, (const bf16_t *)a.x, (const bf16_t *)a.W, (bf16_t *)a.y, a.pieces, a.rows,         \
                           a.descs, (const bf16_t *)a.adata, a.ho_piece, a.ho_order, a.B, a.C, a.Co, a.K, a.Ho, a.Wo, \
                           a.Hi, a.Wi, a.s, n_pxb, n_ob, buf_bytes, a.desc_bytes, a.adata_bytes, vec_x, vec_w, vec_y, \
                           a.scale, x_bs, (int64_t)0, (bf16_t *)a.save, save_bs, vec_save);                          \
    else                                                                                                         \
        hipLaunchKernelGGL((fused_mfma_kernel<N, F16, true, false>), dim3((unsigned)nblk), dim3(kThreads), lds,    \
                           stream, (const bf16_t *)a.x, (const bf16_t *)a.W, (bf16_t *)a.y, a.pieces, a.rows,         \
                           a.descs, (const bf16_t *)a.adata, a.ho_piece, a.ho_order, a.B, a.C, a.Co, a.K, a.Ho, a.Wo, \
                           a.Hi, a.Wi, a.s, n_pxb, n_ob, buf_bytes, a.desc_bytes, a.adata_bytes, vec_x, vec_w, vec_y, \
                           a.scale, x_bs, (int64_t)0, (bf16_t *)nullptr, (int64_t)0, 0)
    if (a.f16) {
        switch (n_ot) {
        case 2: DISCO_FUSED_LAUNCH(2, true); break;
        case 4: DISCO_FUSED_LAUNCH(4, true); break;
        default: DISCO_FUSED_LAUNCH(8, true); break;
        }
    } else {
        switch (n_ot) {
        case 2: DISCO_FUSED_LAUNCH(2, false); break;
        case 4: DISCO_FUSED_LAUNCH(4, false); break;
        default: DISCO_FUSED_LAUNCH(8, false); break;
        }
    }
#undef DISCO_FUSED_LAUNCH
    return hipGetLastError();
}

// ---- the einsum alone ------------------------------------------------------------------------
//
// y[b, o, p] = sum_{c,k} W[o, c, k] * t[b, c, k, p] over flattened output positions p = ho Wo + wo
// ("contraction + einsum" of the torch-harmonics "disco-kernel-dev" page, "Architecture snapshot",
// with the contraction already in device memory): the fused kernel's einsum tile fed from memory.
// Workgroup = (b, 256 positions, up to 256 output channels), eight waves; wave w takes positions
// p0 + 64 (w % 4) + 2n + ph (n < 32, ph = 0, 1: the two MFMA column sets) and output-channel tiles
// h2 NOTH .. + NOTH - 1 (h2 = w / 4), fp32 accumulators in registers for all channels.  A step
// covers kEch input channels: the W slice (A operand order, as in the fused kernel) and the t tile
// [channel][basis][256 positions] come in by direct global->LDS loads, the t tiles through a ring of
// three stages issued two steps ahead (the t stream is the op's bound, and its rate follows the bytes
// in flight) and the W slices through a ring of two issued one step ahead.  A lane's B operand (basis
// 8 hh .. 8 hh + 7 at one position) is assembled from eight 4-byte LDS words, each holding the two
// neighbouring positions of both column sets.  The 16-byte units of a tile row are XOR-swizzled by
// 8 on rows whose basis index has bit 3 set, so the two lane halves (basis 0..7 and 8..15) read
// disjoint bank halves.  At 256 channels and K = 16 the tile reads t once from HBM (the W slices
// come from L2), and the op is bound by that stream: 256 flops per byte of t, below the ratio of
// the bf16 matrix-core peak to the HBM bandwidth.  Four channels per step with two stages measured
// faster than two channels per step with three to five stages (fewer barriers per MFMA).

namespace {

constexpr int kEch = 4;                                  // input channels per step
constexpr int kTring = 3;                                // t tile stages (issued two steps ahead)
constexpr int kWring = 2;                                // W slice stages (issued one step ahead)
constexpr int kTileBytes = kEch * 16 * kFusedSpan * 2;   // 32 KiB
constexpr int kTileLoads = kTileBytes / 16 / kThreads;   // direct loads per thread per tile

// W slice of the step starting at channel c0, unit (ot, cl) = W[o_base + 32 ot + l % 32, c0 + cl,
// 8 (l / 32) .. + 7] for lane l.  With vec_w every unit is one direct load (rows past Co or C
// read zeros), so with NOT = 8 (16 units over 8 waves) each thread issues exactly two.
__device__ __forceinline__ void stage_w_ein(const Ctx &c, int c0, unsigned char *wb)
{
    const int o = c.o_base + (c.lane & 31);
    const int hh = c.lane >> 5;
    for (int u = c.wave; u < c.n_ot * kEch; u += kWaves) {
        const int ot = u / kEch, cl = u - ot * kEch;
        const int oo = o + 32 * ot, ch = c0 + cl;
        unsigned char *dst = wb + 1024 * u;
        const bool ok = oo < c.Co && ch < c.C;
        if (c.vec_w) {
            // rows past Co or C read zeros through the buffer bounds (one load per unit either way)
            const uint32_t voff = ok ? 2u * (uint32_t)(((int64_t)oo * c.C + ch) * 16 + 8 * hh) : 0x80000000u;
            dma16(c.w_rs, voff, dst);
        } else {
            i16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 8 * hh + i;
                v[i] = (ok && k < c.K) ? (short)c.W[((int64_t)oo * c.C + ch) * c.K + k] : (short)0;
            }
            *reinterpret_cast<i16x8 *>(dst + 16 * c.lane) = v;
        }
    }
}

__device__ __forceinline__ void stage_tile(const Ctx &c, const bf16_t *t, int64_t HW, int64_t p0, int c0, bool vec,
                                           unsigned char *tile)
{
    const int ccn = min(kEch, c.C - c0);
    const bf16_t *base = t + ((int64_t)c.b * c.C + c0) * c.K * HW;
    constexpr int kUnits = kTileBytes / 16;  // 32 rows of 32 units
    if (vec) {
        // one resource over the step's valid channels (fewer than 2^31 bytes: checked by the launcher)
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(2 * (int64_t)max(ccn, 0) * c.K * HW));
#pragma unroll
        for (int i = 0; i < kTileLoads; ++i) {
            const int slot = i * kThreads + c.tid;
            const int R = slot >> 5, u = (slot & 31) ^ (8 * ((R >> 3) & 1));
            const int cl = R >> 4, k = R & 15;
            const int64_t p = p0 + 8 * u;
            const bool ok = k < c.K && cl < ccn && p < HW;
            const uint32_t voff = ok ? (uint32_t)(2 * ((int64_t)(cl * c.K + k) * HW + p)) : 0x80000000u;
            dma16(rs, voff, tile + 16 * (i * kThreads + 64 * c.wave));
        }
    } else {
        for (int slot = c.tid; slot < kUnits; slot += kThreads) {
            const int R = slot >> 5, u = (slot & 31) ^ (8 * ((R >> 3) & 1));
            const int cl = R >> 4, k = R & 15;
            const int64_t p = p0 + 8 * u;
            i16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (k < c.K && cl < ccn && p + e < HW) ? (short)base[(int64_t)(cl * c.K + k) * HW + p + e] : (short)0;
            *reinterpret_cast<i16x8 *>(tile + 16 * slot) = v;
        }
    }
}

// One step: B operands of the kEch channels from the tile, MFMAs against the W slice.  The LDS
// reads of channel ch + 1 (eight words of t, NOTH W operands) are issued before the MFMAs of
// channel ch, so their latency hides behind those MFMAs; scheduling barriers keep that order.
template <int NOTH, bool F16>
__device__ __forceinline__ void einsum_chunk(const unsigned char *__restrict__ tile, const unsigned char *__restrict__ wb,
                                             int lane, int pp, int h2, f32x16 (&yacc)[2][NOTH])
{
    const int r = lane & 31, hh = lane >> 5;
    const unsigned *t32 = reinterpret_cast<const unsigned *>(tile);
    // word of a row with basis bit 3 = hh holding positions 64 pp + 2 r and + 1
    const unsigned *tl = t32 + 8 * hh * 128 + 4 * ((8 * pp + (r >> 2)) ^ (8 * hh)) + (r & 3);
    // A operand of tile ot = h2 NOTH + j and channel ch at wl + 1024 (j kEch + ch)
    const unsigned char *wl = wb + 1024 * (h2 * NOTH * kEch) + 16 * lane;
    unsigned w[2][8];
    i16x8 a[2][NOTH];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[0][i] = tl[i * 128];
#pragma unroll
    for (int j = 0; j < NOTH; ++j) a[0][j] = *reinterpret_cast<const i16x8 *>(wl + 1024 * (j * kEch));
#pragma unroll
    for (int ch = 0; ch < kEch; ++ch) {
        const int sl = ch & 1;
        if (ch + 1 < kEch) {
#pragma unroll
            for (int i = 0; i < 8; ++i) w[sl ^ 1][i] = tl[((ch + 1) * 16 + i) * 128];
#pragma unroll
            for (int j = 0; j < NOTH; ++j) a[sl ^ 1][j] = *reinterpret_cast<const i16x8 *>(wl + 1024 * (j * kEch + ch + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        unsigned e0[4], e1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e0[q] = __builtin_amdgcn_perm(w[sl][2 * q + 1], w[sl][2 * q], 0x05040100u);  // low halves: even positions
            e1[q] = __builtin_amdgcn_perm(w[sl][2 * q + 1], w[sl][2 * q], 0x07060302u);  // high halves: odd positions
        }
        const i16x8 b0 = __builtin_bit_cast(i16x8, e0), b1 = __builtin_bit_cast(i16x8, e1);
#pragma unroll
        for (int j = 0; j < NOTH; ++j) {
            yacc[0][j] = mfma32<F16>(a[sl][j], b0, yacc[0][j]);
            yacc[1][j] = mfma32<F16>(a[sl][j], b1, yacc[1][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Wait until at most N of this thread's direct loads are in flight and its LDS writes are done.
template <int N>
__device__ __forceinline__ void wait_loads()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // vmcnt N, expcnt 7 (no wait), lgkmcnt 0
}

template <int NOT, bool F16>
__global__ __launch_bounds__(kThreads) void einsum_mfma_kernel(const bf16_t *__restrict__ t, const bf16_t *__restrict__ W,
                                                               bf16_t *__restrict__ y, int B, int C, int Co, int K,
                                                               int64_t HW, int n_pt, int n_ob, int vec_t, int vec_w,
                                                               int vec_y)
{
    constexpr int NOTH = NOT / 2;
    constexpr int kW = NOT * kEch * 1024;
    // LDS: [W slice ring: kWring x kW][t tile ring: kTring x kTileBytes]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int bid = blockIdx.x;
    const int pt = bid % n_pt;
    bid /= n_pt;
    const int ob = bid % n_ob;
    Ctx c;
    c.b = bid / n_ob;
    c.W = W;
    c.w_rs = make_rsrc(W, vec_w ? (uint32_t)(2 * (int64_t)Co * C * 16) : 0u);
    c.B = B; c.C = C; c.Co = Co; c.K = K; c.n_ot = NOT;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.o_base = ob * (kMaxOt * 32);
    c.vec_w = vec_w != 0;
    const int64_t p0 = (int64_t)pt * kFusedSpan;
    const bool vec = vec_t != 0;
    const int pp = c.wave & 3, h2 = c.wave >> 2;
    const int r = c.lane & 31, hh = c.lane >> 5;

    f32x16 yacc[2][NOTH];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph)
#pragma unroll
        for (int j = 0; j < NOTH; ++j)
#pragma unroll
            for (int a = 0; a < 16; ++a) yacc[ph][j][a] = 0.0f;

    // Step st's stage: W slice st (issued during step st - 1, or before the loop) and t tile st (issued
    // during step st - 2).  Issue order is W slice st + 1, then t tile st + 2, so when step st begins
    // only t tile st + 1 was issued after everything it needs; with direct loads for both operands and
    // NOT = 8 a thread issues exactly kTileLoads loads per t tile, so "at most kTileLoads in flight"
    // means step st's operands have landed.  Otherwise wait for everything.
    const bool ring = vec && c.vec_w && NOT == 8;
    const int nsteps = (C + kEch - 1) / kEch;
    unsigned char *const wring = smem;
    unsigned char *const tring = smem + kWring * kW;
    auto issue_w = [&](int st) { stage_w_ein(c, kEch * st, wring + (st % kWring) * kW); };
    auto issue_t = [&](int st) { stage_tile(c, t, HW, p0, kEch * st, vec, tring + (st % kTring) * kTileBytes); };
    if (nsteps > 0) {
        issue_w(0);
        issue_t(0);
    }
    if (nsteps > 1) issue_t(1);
    for (int st = 0; st < nsteps; ++st) {
        // A bare barrier: __syncthreads() would add a workgroup release fence, and the compiler makes
        // such a fence wait for every direct load into LDS still in flight (the later steps' too).
        // The compiler-level fences keep LDS accesses on their side of the barrier.
        if (ring && st + 1 < nsteps) wait_loads<kTileLoads>();  // t tile st + 1 may stay in flight
        else __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // everyone's loads have landed; every wave is done with step st - 1
        asm volatile("" ::: "memory");
        if (st + 1 < nsteps) issue_w(st + 1);  // into step st - 1's W slot
        if (st + 2 < nsteps) issue_t(st + 2);  // into step st - 1's t slot
        einsum_chunk<NOTH, F16>(tring + (st % kTring) * kTileBytes, wring + (st % kWring) * kW, c.lane, pp, h2, yacc);
    }
    __builtin_amdgcn_s_waitcnt(0);  // nothing in flight before the ring's space is reused

    // epilogue: yacc[ph][j] row = output channel (h2 NOTH + j) 32 + 8 (a / 4) + 4 hh + a % 4, column
    // = position p0 + 64 pp + 2 r + ph.  Pass j writes 64 channels through a 32 KiB LDS tile
    // [channel][256 positions] (the ring's first 32 KiB) so that rows leave as 16-byte stores.
    uint32_t *tile32 = reinterpret_cast<uint32_t *>(smem);
    const bf16_t *tile = reinterpret_cast<const bf16_t *>(smem);
#pragma unroll
    for (int j = 0; j < NOTH; ++j) {
        __syncthreads();  // the last step (or the previous pass) is done with the tile's space
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int ol = 32 * h2 + 8 * (a >> 2) + 4 * hh + (a & 3);
            const uint32_t lo = (uint16_t)to16<F16>(yacc[0][j][a], 1.0f), hi = (uint16_t)to16<F16>(yacc[1][j][a], 1.0f);
            tile32[ol * 128 + 32 * pp + r] = lo | (hi << 16);
        }
        __syncthreads();
        for (int u = c.tid; u < 64 * 32; u += kThreads) {
            const int seg = u & 31, ol = u >> 5;
            const int o = c.o_base + ((ol >> 5) * NOTH + j) * 32 + (ol & 31);
            const int64_t p = p0 + 8 * seg;
            if (o >= Co || p >= HW) continue;
            bf16_t *dst = y + ((int64_t)c.b * Co + o) * HW + p;
            const bf16_t *src = tile + ol * 256 + 8 * seg;
            if (vec_y && p + 8 <= HW) {
                *reinterpret_cast<i16x8 *>(dst) = *reinterpret_cast<const i16x8 *>(src);
            } else {
                for (int e = 0; e < 8 && p + e < HW; ++e) dst[e] = src[e];
            }
        }
    }
}

}  // namespace

hipError_t launch_einsum_mfma(const EinsumLaunch &a, hipStream_t stream)
{
    if (a.B == 0 || a.Co == 0 || a.HW == 0) return hipSuccess;
    const int n_pt = (int)((a.HW + kFusedSpan - 1) / kFusedSpan);
    const int n_ob = (a.Co + kMaxOt * 32 - 1) / (kMaxOt * 32);
    const int n_ot1 = std::min(kMaxOt, (a.Co + 31) / 32);
    const int n_ot = n_ot1 <= 2 ? 2 : n_ot1 <= 4 ? 4 : 8;  // tiles past Co hold zero W
    const size_t lds = (size_t)kWring * n_ot * kEch * 1024 + (size_t)kTring * kTileBytes;  // 160 KiB at 256 channels
    const void *fn = a.f16 ? (n_ot == 2   ? (const void *)einsum_mfma_kernel<2, true>
                              : n_ot == 4 ? (const void *)einsum_mfma_kernel<4, true>
                                          : (const void *)einsum_mfma_kernel<8, true>)
                           : (n_ot == 2   ? (const void *)einsum_mfma_kernel<2, false>
                              : n_ot == 4 ? (const void *)einsum_mfma_kernel<4, false>
                                          : (const void *)einsum_mfma_kernel<8, false>);
    hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int64_t nblk = (int64_t)a.B * n_ob * n_pt;
    // direct loads: 16-byte aligned runs, and one chunk's channels addressable with 32-bit offsets
    const int vec_t = (a.HW % 8 == 0 && ((uintptr_t)a.t % 16) == 0 &&
                       (int64_t)2 * kEch * a.K * a.HW < ((int64_t)1 << 31)) ? 1 : 0;
    // W rows of 16 elements (K = 16, or W packed by launch_pack_w16): the slice arrives by direct loads
    const int vec_w = ((a.K == 16 || a.w16) && ((uintptr_t)a.W % 16) == 0 && (int64_t)a.Co * a.C * 32 < ((int64_t)1 << 31)) ? 1 : 0;
    const int vec_y = (a.HW % 8 == 0 && ((uintptr_t)a.y % 16) == 0) ? 1 : 0;
#define DISCO_EINSUM_LAUNCH(N, F16)                                                                              \
    hipLaunchKernelGGL((einsum_mfma_kernel<N, F16>), dim3((unsigned)nblk), dim3(kThreads), lds, stream,           \
                       (const bf16_t *)a.t, (const bf16_t *)a.W, (bf16_t *)a.y, a.B, a.C, a.Co, a.K, a.HW, n_pt,     \
                       n_ob, vec_t, vec_w, vec_y)
    if (a.f16) {
        switch (n_ot) {
        case 2: DISCO_EINSUM_LAUNCH(2, true); break;
        case 4: DISCO_EINSUM_LAUNCH(4, true); break;
        default: DISCO_EINSUM_LAUNCH(8, true); break;
        }
    } else {
        switch (n_ot) {
        case 2: DISCO_EINSUM_LAUNCH(2, false); break;
        case 4: DISCO_EINSUM_LAUNCH(4, false); break;
        default: DISCO_EINSUM_LAUNCH(8, false); break;
        }
    }
#undef DISCO_EINSUM_LAUNCH
    return hipGetLastError();
}

}  // namespace disco
