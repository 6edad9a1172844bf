// kernels.hpp — launch descriptors of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "plan.hpp"
#include "plan_fused.hpp"
#include "plan_tile.hpp"

namespace disco {

// element types of the data: 0 = fp32, 1 = bf16, 2 = fp16
struct GatherLaunch {
    const void *src;
    void *dst;
    int32_t dtype;
    const Item *items;     // device
    const int32_t *order;  // device, heaviest item first
    const Seg *segs;       // device
    const float *vals;     // device
    int32_t n_items;
    int32_t BC;            // number of (b, c) planes
    int64_t src_plane, dst_plane;
    int32_t L, in_stride;
};

hipError_t launch_gather(const GatherLaunch &a, hipStream_t stream);

struct StagedLaunch {
    const void *src;
    void *dst;
    int32_t dtype;
    const Task *tasks;            // device, heaviest first
    const Stage *stages;
    const int32_t *stage_rows;
    const int32_t *stage_segptr;
    const Seg *segs;
    const float *vals;
    const Item *items;
    int32_t n_tasks, BC;
    int64_t src_plane, dst_plane;
    int32_t L, row_len, copy_len, lrow, wpp, NP, stage_elems, vec;
    int32_t NI, G, T, S;
};

// Register-tiled fp32 gather (kernels_tile.hip) over a TilePlan.
struct TileLaunch {
    const float *src;
    float *dst;
    const Task *tasks;          // device, heaviest first
    const Stage *stages;
    const Stage *task_first;    // per task: its first stage's descriptor (TilePlan::task_first)
    const int32_t *stage_rows;
    const int32_t *stage_recptr;
    const TileRec *recs;
    const Item *items;
    int32_t n_stages;           // stages in all (0: task_first is not read)
    int32_t n_tasks, BC;        // tasks, planes
    int32_t n_ws4, n_ws2;       // task classes by wave split (see TilePlan)
    int64_t src_plane, dst_plane;
    int32_t L, row_len, lrow, deint, rows_per_stage, NI, G, PW;
    int32_t max_recs;           // records of the largest stage (LDS after the rows)
    int32_t n_recs;             // records in all
    int32_t vec;                // source rows are 16-byte aligned (row_len and plane a multiple of 4), L >= halo,
                                // plane below 2 GiB: stages stream in by direct global -> LDS loads
};
// Allow kernel `fn` `lds` bytes of dynamic LDS on the current device: checked on the host against the
// device's per-workgroup LDS (hipErrorInvalidValue, nothing launched, when it does not fit), the
// function attribute raised only when a kernel needs more than it was last given on that device.
hipError_t allow_lds(const void *fn, size_t lds);

bool tile_supported(int NI, int G, int PW);
hipError_t launch_tile(const TileLaunch &a, hipStream_t stream);

// true when the staged kernel has an instantiation for these parameters
bool staged_supported(int NI, int G, int T, int S);
hipError_t launch_staged(const StagedLaunch &a, hipStream_t stream);

struct FusedLaunch {
    const void *x;          // (B, C, Hi, Wi) bf16, fp16 or fp32
    const void *W;          // (Co, C, K)
    void *y;                // (B, Co, Ho, Wo)
    bool f16;               // fp16 data (else bf16)
    bool f32 = false;       // fp32 data: fp32 contraction tile and fp32 matrix-core einsum
    const Item *items;      // forward plan items, grouped by ho
    const int32_t *block_ptr;  // [Ho + 1]
    const int32_t *ho_order;   // [Ho], heaviest latitude first
    const Seg *segs;
    const float *vals;
    int32_t B, C, Co, K, Ho, Wo, Hi, Wi, in_stride;
    const float *Wa = nullptr;  // fp32 data: W packed by launch_pack_wa_f32 (required)
    const void *Wa16 = nullptr; // 16-bit data: W packed by launch_pack_wa16 (required)
    // fp32 data: the forward plan's source windows (plan.hpp, FusedWindows; null: global reads) and the
    // positions per channel the kernel's LDS area holds (fused_win_cap_f32)
    const FWin *fw_rows = nullptr;
    const int32_t *fw_ho_ptr = nullptr, *fw_ho_len = nullptr, *fw_seg_off = nullptr;
    int32_t fw_cap = 0;
    const int32_t *fw_ho_psi = nullptr;  // [Ho][4]: the latitude's segment and value runs (null: not contiguous)
    int32_t fw_psi_bytes = 0;            // largest latitude's psi in LDS (items, segments, values, offsets)
};

hipError_t launch_fused(const FusedLaunch &a, hipStream_t stream);
// fp32 fused kernel: positions per channel of its LDS window area for this plan (latitudes with more
// read their sources from global memory)
int fused_win_cap_f32(int K, const int32_t *ho_len, int nho);
// fp32 fused kernel: floats of W packed in its A-operand order (0 when K is outside 1 .. 64), and the packing
int64_t fused_wa_f32_floats(int Co, int C, int K);
// 16-bit fused kernel: elements of W packed in its A-operand order (0 when K is outside 1 .. 64), and the packing
int64_t fused_wa16_elems(int Co, int C, int K);
hipError_t launch_pack_wa16(const void *W, void *Wa, int Co, int C, int K, hipStream_t stream);
hipError_t launch_pack_wa_f32(const float *W, float *Wa, int Co, int C, int K, hipStream_t stream);

struct FusedMfmaLaunch {
    const void *x, *W;
    void *y;
    const FPiece *pieces;
    const FRow *rows;
    const int32_t *descs;
    const uint16_t *adata;
    const int32_t *ho_piece, *ho_order;
    int32_t B, C, Co, K, Ho, Wo, Hi, Wi, s, max_piece_bytes, max_resident_bytes;
    uint32_t desc_bytes, adata_bytes;  // sizes of the descriptor and psi arrays
    bool f16;     // fp16 data and psi (adata then holds fp16 psi * 2^e)
    float scale;  // 2^-e for fp16, 1 for bf16
    void *save = nullptr;  // non-null: also write the contraction (B, C, K, Ho, Wo), data type, contiguous
    bool w16 = false;      // W holds rows of 16 elements (launch_pack_w16 output), not of K
};

hipError_t launch_fused_mfma(const FusedMfmaLaunch &a, hipStream_t stream);

// W (Co, C, K) with K <= 16 into rows of 16 elements (zeros past K), the layout the fused kernel's
// direct W-slice loads read; Wp holds Co * C * 16 16-bit elements.
hipError_t launch_pack_w16(const void *W, void *Wp, int Co, int C, int K, hipStream_t stream);

// The fused kernel's contraction alone, out[b, c, k, ho, wo] (K <= 16), over the fused op's plan:
// each block walks all channels with the latitude's psi resident where it fits.
struct FusedContractLaunch {
    const void *x;
    void *out;
    const FPiece *pieces;
    const FRow *rows;
    const int32_t *descs;
    const uint16_t *adata;
    const int32_t *ho_piece, *ho_order;
    int32_t B, C, K, Ho, Wo, Hi, Wi, s, max_piece_bytes, max_resident_bytes;
    uint32_t desc_bytes, adata_bytes;
    bool f16;
    float scale;
    int64_t x_bstride = 0, out_bstride = 0;  // elements between batches (0: contiguous)
};
hipError_t launch_fused_contract(const FusedContractLaunch &a, hipStream_t stream);

// The einsum alone, y[b, o, p] = sum_{c,k} W[o, c, k] * t[b, c, k, p] (p = ho Wo + wo, K <= 16),
// on the fused kernel's matrix-core einsum tile with t staged from device memory.
struct EinsumLaunch {
    const void *t, *W;
    void *y;
    int32_t B, C, Co, K;
    int64_t HW;
    bool f16;
    bool w16 = false;  // W holds rows of 16 elements (launch_pack_w16 output), not of K
};
hipError_t launch_einsum_mfma(const EinsumLaunch &a, hipStream_t stream);
size_t fused_mfma_lds_bytes(int n_ot, int max_piece_bytes, int max_resident_bytes);
int fused_mfma_channels_per_chunk();
int fused_mfma_exchange_bytes();     // LDS bytes of the einsum operand exchange

// Where the forward kernel writes: out (B, C, K, Ho, Wo), or, for the backward run as a forward
// over the inverse CSR, gx (B, C, Hi, Wi) with row ho * kr + k = hi * s + rho at columns rho + s * j.
struct OutMap {
    int64_t plane;   // elements per (b, c) plane of the output
    int32_t inverse; // 0: forward layout; 1: gradient layout
    int32_t rows;    // inverse: Hi * s
    int32_t wi;      // inverse: Wi
    int32_t s;       // inverse: Wi / Wo
};

struct FwdMfmaLaunch {
    const void *x;
    void *out;
    const FPiece *pieces;
    const FRow *rows;
    const int32_t *descs;
    const uint16_t *adata;
    const int32_t *ho_piece, *ho_order;
    int32_t B, C, K, Ho, Wo, Hi, Wi, s, kr, max_piece_bytes;  // geometry of the source/psi (the inverse CSR's for the backward)
    uint32_t desc_bytes, adata_bytes;
    OutMap om;
    bool f16;     // fp16 data and psi (adata then holds fp16 psi * 2^e)
    float scale;  // 2^-e for fp16, 1 for bf16
    int64_t x_bstride = 0, out_bstride = 0;  // elements between batches (0: C contiguous planes)
};

hipError_t launch_fwd_mfma(const FwdMfmaLaunch &a, hipStream_t stream);
int fwd_mfma_channels(int kr);       // channels per forward workgroup for a psi group of kr rows
size_t fused_mfma_reserved_bytes();  // LDS bytes besides the two piece stage buffers
int fused_max_k();  // largest K the fused kernel accepts
int fused_tile_px();  // output longitudes per workgroup of the vector-ALU fused kernels

// C[m][n] = sum_k A[m][k] B[n][k] on bf16 (or fp16) matrix cores (operands contiguous along k; k
// ranges and Kd multiples of 8; operand buffers below 2 GiB).  out_f32: fp32 partials [split][M][N],
// one per k range of k_per_split (a multiple of 32); else 16-bit C with row stride ldc
// (k_per_split = 0: one range).
struct GemmNtLaunch {
    const void *A;
    int64_t lda;
    int32_t M;
    uint32_t a_bytes;
    const void *B;
    int64_t ldb;
    int32_t N;
    uint32_t b_bytes;
    int32_t Kd, k_per_split;
    bool out_f32;
    void *C;
    int64_t ldc;
    bool f16 = false;  // fp16 operands and output (else bf16)
};
hipError_t launch_gemm_nt(const GemmNtLaunch &g, hipStream_t stream);
// dst (Cn x R) = src (R x Cn)^T, 16-bit elements (bf16 or fp16: the bits are moved).
hipError_t launch_transpose_bf16(const void *src, void *dst, int R, int Cn, hipStream_t stream);
// W (Co, C, K) with K <= 16 into W' (C, Co, 16): W'[c, o, k] = W[o, c, k], zeros past K (16-bit elements).
hipError_t launch_permute_w16(const void *W, void *Wt, int Co, int C, int K, hipStream_t stream);
// dW[o][col0 + m] = 16-bit(sum_{z < Z} P[z][o][m]) (fp16 when f16, else bf16), summed in increasing z.
hipError_t launch_reduce_partials(const float *P, int Z, int Co, int Mc, void *dW, int64_t ldw, int col0, bool f16,
                                  hipStream_t stream);

}  // namespace disco
