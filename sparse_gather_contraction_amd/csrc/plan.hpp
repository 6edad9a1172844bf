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

// Returns "" on success, else a message; `code` receives a disco_status value.
std::string validate_csr(const CSRView &c, int *code);

void build_forward_plan(const CSRView &c, GatherPlan &p);
void build_backward_plan(const CSRView &c, GatherPlan &p);

}  // namespace disco
