// plan.hpp — host-side work plans for the DISCO gather kernels.
//
// Both directions of the CSR contraction (torch-harmonics "disco-kernel-dev"
// page, "Architecture snapshot"; the backward as a gather per input pixel,
// section "Backward direction — gather vs scatter") are reduced to one
// primitive, a strided circular correlation over rows of length L = Wo:
//
//   dst[row_g][j * out_stride] = sum_{segments} sum_{t < m} val[t][g] *
//                                src[in_off + in_stride * ((j0 + t + j) mod L)]
//
// Forward:  s = Wi/Wo.  Input column wi = s*jj + rho, so
//           x[hi, (wi + s*wo) mod Wi] = x[hi*Wi + rho + s*((jj + wo) mod Wo)]:
//           in_off = hi*Wi + rho, in_stride = s, and a run of consecutive jj of
//           one (hi, rho) is one segment.  Rows k of one output latitude with
//           the same column set share the segment and carry G values each.
// Backward: gx[hi, rho + s*j] = sum over entries (k, ho, wi') with
//           wi' = rho + s*jj' of val * gout[k, ho, (j - jj') mod Wo]:
//           in_off = (k*Ho + ho)*Wo, in_stride = 1, shift u = (-jj') mod Wo,
//           out_off = hi*Wi + rho, out_stride = s.  This is the row-inverted
//           psi: every gx element is owned by exactly one item, no atomics.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace disco {

constexpr int kMaxGroup = 4;     // rows sharing one segment list
constexpr int kMaxSegLen = 64;   // longer runs are split

struct Seg {          // 16 bytes
    int32_t in_off;   // offset of the source row within a plane
    int32_t j0;       // shift of the first entry, in [0, L)
    int32_t m;        // number of entries (1..kMaxSegLen)
    int32_t val_off;  // index of the first value; values are [m][G]
};

struct Item {                   // 32 bytes
    int32_t seg_begin, seg_end; // segment range
    int32_t G;                  // rows written by this item (1..kMaxGroup)
    int32_t out_stride;         // element stride along j of the destination rows
    int32_t out_off[kMaxGroup]; // destination row offsets within a plane
};

struct GatherPlan {
    std::vector<Seg> segs;
    std::vector<float> vals;
    std::vector<Item> items;        // grouped by output row block (ho for fwd, hi for bwd)
    std::vector<int32_t> order;     // item indices, heaviest first (launch order)
    std::vector<int32_t> block_ptr; // items of block b: [block_ptr[b], block_ptr[b+1])
    int64_t nnz_updates_per_col = 0;  // sum over items of (entries * G) = nnz
    int32_t L = 0;                  // circular length (Wo)
    int32_t in_stride = 1;
};

struct CSRView {
    int32_t K, Ho, Wo, Hi, Wi;
    int64_t nnz;
    const int64_t *row_ptr;
    const int32_t *col_hi;
    const int32_t *col_wi;
    const float *val;
};

// ---------------------------------------------------------------------------
// Staged plan: the same segments, regrouped for the LDS-staged gather kernel.
//
// A task is the work of one block for one group of planes: NI items (the
// forward: one row group of one latitude; the backward: the s residue items
// of one input row).  Its source rows are copied to LDS in stages of at most
// `rows_per_stage` rows; each staged row holds row_len elements followed by a
// wrap halo (a copy of its first `halo` elements), `lrow` elements in all.
// Segments are cut to at most kStagedSegLen entries and carry LDS offsets:
// lds_off = slot * lrow + rho (rho = longitude residue of the forward).
constexpr int kStagedSegLen = 8;
constexpr int kStagedHaloPos = 16;   // halo, in positions (covers kStagedSegLen + T - 1 for T <= 9)

struct Task {
    int32_t stage_begin, stage_end;  // into stages
    int32_t item_begin;              // items [item_begin, item_begin + NI)
    int32_t work;                    // entries * G summed over its items (for ordering)
};

struct Stage {
    int32_t row_begin, row_end;      // into stage_rows (source row indices within a plane)
    int32_t segptr;                  // stage_segptr[segptr + i] .. [segptr + i + 1]: segments of item i
    int32_t pad;
};

struct StagedPlan {
    bool ok = false;                 // false: shape not covered, use the plain gather
    int32_t NI = 1, G = 1, T = 3, S = 1;     // items per task, rows per item, positions per lane, source stride
    int32_t wpp = 4, NP = 1;         // waves per plane, planes per block (4 waves per block)
    int32_t L = 0, row_len = 0, lrow = 0, halo = 0, rows_per_stage = 0;
    std::vector<Seg> segs;
    std::vector<float> vals;
    std::vector<Item> items;
    std::vector<Task> tasks;         // heaviest first
    std::vector<Stage> stages;
    std::vector<int32_t> stage_rows;
    std::vector<int32_t> stage_segptr;
};

// Regroup `p` (built by build_forward_plan / build_backward_plan) for the
// staged kernel.  `backward` selects the row-inverted source layout (source
// rows of length Wo, one task per input row covering all s residues);
// `elem_bytes` is the source element size; `lds_budget` the bytes of LDS one
// block may use.  Returns plans with ok = false when the shape is outside
// what the staged kernel covers.
void build_staged_plan(const CSRView &c, const GatherPlan &p, bool backward, int elem_bytes, int lds_budget,
                       StagedPlan &out);

// Returns "" on success, else a message; `code` receives a disco_status value.
std::string validate_csr(const CSRView &c, int *code);

void build_forward_plan(const CSRView &c, GatherPlan &p);
void build_backward_plan(const CSRView &c, GatherPlan &p);

// ---------------------------------------------------------------------------
// Source windows of the vector-ALU fused kernels (kernels_fused.hip): per output latitude (block b of
// the forward plan), its distinct source rows, each with the shortest circular arc of shifts
// [a, a + span) that its segments read.  A workgroup of `px` output longitudes from wo0 stages, per
// channel, positions (a + wo0 + q) mod L, q < span + px - 1, of every such row back to back; segment q
// of the plan then reads entry t at longitude wo0 + p from staged position seg_off[q] + t + p.
struct FWin {           // 16 bytes
    int32_t in_off;     // source row within a plane (in_stride apart positions)
    int32_t a;          // first shift of the arc, in [0, L)
    int32_t len;        // staged positions: span + px - 1
    int32_t base;       // first staged position of the row within the latitude's area
};

struct FusedWindows {
    std::vector<int32_t> ho_ptr;   // [blocks + 1]: rows of block b
    std::vector<FWin> rows;
    std::vector<int32_t> ho_len;   // [blocks]: staged positions per channel (sum of the rows' len)
    std::vector<int32_t> seg_off;  // [segments]: base of its row + ((j0 - a) mod L)
    int32_t max_len = 0;           // largest ho_len
    // the latitude's psi as one contiguous run of the plan: segments [s0, s1), values [v0, v1) (its items
    // are [block_ptr[b], block_ptr[b + 1])); psi_ok false when some latitude's runs are not contiguous
    std::vector<int32_t> ho_psi;   // [blocks][4]: s0, s1, v0, v1
    bool psi_ok = true;
};

void build_fused_windows(const GatherPlan &p, int32_t px, FusedWindows &out);

}  // namespace disco
