// plan_fused.hpp — packed-psi plan for the matrix-core fused convolution.
//
// The contraction of one output latitude ho is rewritten as dense products:
// for every source row sr (input latitude hi and longitude residue rho, so
// row sr holds x[hi, rho + s*j] for j in [0, Wo)) the K psi rows at ho are
// laid out densely over the union of their column positions, as signed
// offsets d from output longitude 0, in blocks of 16 consecutive offsets
// (zeros where a row has no entry):
//
//   out[k, wo] = sum_sr sum_blocks sum_{t<16} P[k, d_blk + t] * xrow_sr[(wo + d_blk + t) mod Wo]
//
// One block is the A operand of one v_mfma_f32_32x32x16_bf16: rows 0..15
// hold bf16(P) for k = 0..15, rows 16..31 the bf16 rounding residue
// P - bf16(P), so the sum of the two halves of the result carries psi to
// about 16 significant bits.  The B operand is 16 consecutive source values
// per output longitude (a Hankel slice of the row), read from an LDS window.
//
// Blocks are grouped into pieces whose source-row windows and packed blocks
// fit the LDS budget; a latitude whose rows are whole rings (the caps at the
// poles) gets several pieces.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace disco {

constexpr int kFusedKMax = 16;   // psi rows per latitude the packed layout holds
constexpr int kBlkJ = 16;        // offsets per block (MFMA reduction depth)

struct FRow {          // one source row of a piece
    int32_t sr;        // source row = hi * s + rho
    int32_t start;     // signed offset of the first window position (window = px0 + start + e)
    int32_t len;       // window length in positions (multiple of 8)
    int32_t lds_off;   // element offset of this row's window inside one channel's window area
};

struct FBlock {        // one packed 32x16 A operand
    int32_t row;       // index into the piece's rows (absolute index in rows[])
    int32_t rel;       // offset of the block's first position from the row window start
};
// The kernel reads, per block, only xoff = rows[row].lds_off + rel (element offset of
// the block's first window position within one channel's window area).

struct FPiece {
    int32_t blk_begin, blk_end;   // blocks (also index the packed A data, 512 bf16 each)
    int32_t row_begin, row_end;   // rows
    int32_t xwin_elems;           // window elements per channel (sum of row lens)
    int32_t dbuf;                 // 1: the latitude's only piece, with room for two window buffers
                                  //    (a latitude of one piece with dbuf = 0 keeps its blocks resident)
    int32_t pad[2];
};

struct FusedPlan {
    bool ok = false;
    int32_t npx = 0;              // output longitudes per workgroup
    int32_t ch = 4;               // channels per chunk
    int32_t max_xwin = 0;         // max window elements per channel over all pieces
    int32_t max_blk = 0;          // max blocks per piece
    int32_t max_piece_elems = 0;  // max over pieces of 512 * blocks + (1 + dbuf) * ch * window elements
    std::vector<int32_t> ho_piece;      // [Ho + 1]: pieces of latitude ho
    std::vector<int32_t> ho_order;      // latitudes, heaviest first
    std::vector<FPiece> pieces;
    std::vector<FRow> rows;
    std::vector<FBlock> blocks;
    std::vector<int32_t> block_xoff;    // per block: rows[row].lds_off + rel
    std::vector<uint16_t> adata;        // packed A operands, 512 bf16 per block in lane order
    int64_t mfma_blocks = 0;            // total blocks over all latitudes
};

// Build from the forward plan.  `npx` output longitudes per workgroup, `ch`
// channels per chunk; a piece's packed blocks plus its windows for `ch`
// channels take at most `a_budget` bytes of LDS.  A latitude that fits in one
// piece with two window buffers is one double-buffered piece; otherwise it is
// split into pieces with one buffer.  ok = false if the shape is
// outside the packed kernel (K > 16, s > 2, Wo not a multiple of 8).
void build_fused_plan(const CSRView &c, const GatherPlan &fwd, int npx, int ch, int a_budget, FusedPlan &out);

}  // namespace disco
