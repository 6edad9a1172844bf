// plan_fused.hpp — phase-split psi plan for the matrix-core contraction (fused conv and forward).
//
// Output longitudes are handled in spans of 256 = 8 phases x 32 columns:
// column n of phase q is longitude px0 + 8n + q.  With s = Wi/Wo and psi values
// P[k, t] of one output latitude ho and one input latitude hi at signed
// input-column offsets t,
//
//   out[k, px0 + 8n + q] = sum_t P[k, t] * x[hi, s (px0 + 8n + q) + t]
//                        = sum_blocks sum_{u<16} P[k, t0 + u - s q] * x[hi, s px0 + 8 s n + t0 + u]
//
// where the blocks start at offsets t0 that are multiples of 8 and step by 16
// (the first at floor8(min t), enough of them that t0 + 16 - 7 s passes max t).
// The x operand of a block, x[hi, s px0 + 8 s n + t0 + u], does not depend on
// the phase and is read as aligned 16-byte runs; the phase only shifts psi.
// One v_mfma_f32_32x32x16_bf16 per (block, channel, phase group) computes kr
// basis rows for 32/kr phases at once (kr = 16: two phases, kr = 8: four).
//
// Per input latitude the plan stores psi densely as bf16 (round to nearest
// even) by e = t - (first block start - 8 s) and basis k, pairs of e
// interleaved ([e/2][k][e%2], so one 4-byte word holds two consecutive
// offsets); when s is odd a lane whose phase shift is odd either reads a second
// copy that holds the pairs (2m+1, 2m+2), four aligned words, or reads five words
// of the one copy and realigns them (the plan picks per latitude, PhasePlanParams::
// psi_copies); per block a descriptor (byte offsets of its psi rows and of its
// window run in the piece stage); per row the window of input columns
// s px0 + first + i, i < len = span of its blocks + 256 s + 8 (mod Wi; + 16 when
// s = 2, where the kernels keep a channel's window area split by the parity of its
// 16-byte units, unit u at unit (u % 2) (area / 16) + u / 2, and the descriptor's
// window offset counts bytes into one half).  Blocks are contracted in pairs: a
// piece with an odd block count gets a zero block.
//
// Rows are cut into sub-rows and grouped into pieces; a piece's descriptors,
// psi and windows (for one chunk of channels) fit one of two LDS stage
// buffers.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace disco {

constexpr int kFusedKMax = 16;   // basis functions the packed layout holds
constexpr int kBlkJ = 16;        // offsets per block (MFMA reduction depth)
constexpr int kFusedSpan = 256;  // output longitudes per workgroup (8 phases x 32 columns)

struct FRow {          // one sub-row of a piece
    int32_t sr;        // source row = input latitude hi
    int32_t start;     // signed input-column offset of the window's first position (window = s px0 + start + i)
    int32_t len;       // window length in positions (multiple of 8; of 16 when s = 2)
    int32_t win_off;   // element offset of this window inside one channel's window area
};

struct FPiece {
    int32_t desc_begin;  // first block descriptor (pairs of int32)
    int32_t nblk;        // blocks of the piece (even)
    int32_t desc_words;  // int32 words staged for the descriptors (2 * nblk, a multiple of 4)
    int32_t a_begin;     // first bf16 of the piece's psi in adata (multiple of 8)
    int32_t a_elems;     // bf16 count of the piece's psi (multiple of 8)
    int32_t row_begin, row_end;
    int32_t win_elems;   // window elements per channel (multiple of 8; of 16 when s = 2)
    int32_t resident;    // > 0: the latitude's only piece, whose descriptors and psi stay in LDS for all
                         // chunks while the windows are double-buffered; the value is the window buffer
                         // size in bytes (at least the operand exchange)
    int32_t a_copy_bytes;  // > 0: byte offset of the second psi copy (pairs starting one offset later)
    int32_t realign;       // one psi copy and odd shifts: lanes read five words and realign them
    int32_t pad;
};

struct FusedPlan {
    bool ok = false;
    int32_t ch = 4;                     // channels per chunk
    int32_t kr = 16;                    // basis rows per phase in one MFMA (16 or 8)
    int32_t s = 1;                      // Wi / Wo
    int32_t max_piece_bytes = 0;        // largest streamed piece stage (descriptors + psi + ch windows)
    int32_t max_resident_bytes = 0;     // largest resident layout (descriptors + psi + 2 window buffers)
    int32_t max_win = 0;                // largest window area per channel
    std::vector<int32_t> ho_piece;      // [Ho + 1]: pieces of latitude ho
    std::vector<int32_t> ho_order;      // latitudes, heaviest first
    std::vector<FPiece> pieces;
    std::vector<FRow> rows;
    std::vector<int32_t> descs;         // per block: byte offsets (psi rows, window run) in the piece stage
    std::vector<uint16_t> adata;        // bf16 psi, [e][16] per sub-row
    std::vector<uint16_t> adata16;      // the same layout as fp16 of psi * 2^psi16_exp
    int32_t psi16_exp = 0;              // puts the largest |psi| in [2^14, 2^15)
    int64_t mfma_blocks = 0;            // total blocks over all latitudes
};

struct PhasePlanParams {
    int kr = 16;            // basis rows per phase in one MFMA: 16 or 8 (K <= kr)
    int ch = 4;             // channels per stage
    int piece_budget = 0;   // LDS bytes of one piece stage
    int xch_bytes = 0;      // smallest window buffer of a resident latitude
    bool allow_resident = true;
    // s odd: 1 = one psi copy (realigned reads), 2 = two copies, 3 = two copies where the latitude
    // is resident with them, else one
    int psi_copies = 3;
};

// Build the plan; a piece stage takes at most `piece_budget` bytes of LDS for
// `ch` channels; a latitude of one piece is resident when its descriptors,
// psi and two window buffers of at least `xch_bytes` each fit 2 * piece_budget.
// ok = false if the shape is outside the packed kernels (K > kr, s > 2, Wo or
// Wi not a multiple of 8).
void build_phase_plan(const CSRView &c, const PhasePlanParams &prm, FusedPlan &out);

// The backward as a forward over the row-inverted psi.  gx[b,c,hi,rho + s j] =
// sum over entries (k, ho; hi, wi) with wi = rho (mod s) of val * gout[b,c,k,ho,(j - (wi - rho)/s) mod Wo],
// i.e. output row r = hi s + rho reads gout row k Ho + ho at column (j + delta) mod Wo with
// delta = -(wi - rho)/s.  The inverse CSR groups g output rows per "latitude": row index
// (r % g) * Ho' + r / g, Ho' = ceil(Hi s / g); source "latitudes" are the K Ho gout rows (length Wo,
// stride 1), so the phase-split plan of this CSR drives the forward kernel.
struct InverseCSR {
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> col_hi, col_wi;
    std::vector<float> val;
    CSRView view;
};
void build_inverse_csr(const CSRView &c, int g, InverseCSR &out);

// The per-basis transpose of psi when Wi = Wo (s = 1): row (k, hi) holds an entry (ho, (Wo - wi) mod Wo)
// of value val for every entry (k, ho; hi, wi) of psi.  As a psi from the (Ho, Wo) grid to the (Hi, Wo)
// grid it gives z[k, hi, j] = sum over those entries of val * g[ho, (j - wi) mod Wo], the adjoint of the
// forward's basis-k contraction, so the fused convolution over it computes the fused op's input gradient.
struct TransposedCSR {
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> col_hi, col_wi;
    std::vector<float> val;
    CSRView view;
};
void build_transposed_csr(const CSRView &c, TransposedCSR &out);  // requires c.Wi == c.Wo

// Bytes of one piece stage in LDS.
inline int64_t fused_piece_bytes(int64_t desc_words, int64_t a_elems, int64_t ch, int64_t win_elems)
{
    return 4 * desc_words + 2 * a_elems + 2 * ch * win_elems;
}

}  // namespace disco
