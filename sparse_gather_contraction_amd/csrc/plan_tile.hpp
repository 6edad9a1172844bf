// plan_tile.hpp — host plan of the register-tiled fp32 gather (kernels_tile.hip).
//
// Same primitive as plan.hpp (the forward CSR contraction, and the backward as a
// gather over the row-inverted psi), regrouped so that one workgroup
// accumulates every destination row of one output latitude (forward) or of one
// input row's longitude residues (backward) at once:
//   * a task = NI items of G rows each (NI * G <= kTileMaxRows accumulator rows
//     per lane position), all reading one band of source rows;
//   * the band is staged to LDS in stages of at most rows_per_stage source
//     rows; a forward source row (input latitude hi, Wi columns) is split by
//     longitude residue rho = wi mod s into s LDS rows of Wo positions, so
//     that every segment reads consecutive LDS words;
//   * each segment of the gather plan becomes records of at most
//     tile_piece_max(G) entries, 64 bytes each: window offset, wrap
//     threshold, entry count and the values [c][G]; a stage's records are
//     contiguous and travel to LDS with its rows; within a stage the
//     records of an item are grouped by entry count, so the kernel runs one
//     branch-free, software-pipelined loop per count;
//   * tasks much heavier than the mean (the polar latitudes) split their
//     records over 2 or 4 waves that share the same planes and add their
//     partial sums in a fixed order.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace disco {

constexpr int kTileT = 6;          // consecutive positions per lane
constexpr int kTileHalo = 16;      // wrap halo per LDS row, positions (>= largest piece + kTileT - 1)
constexpr int kTileMaxRows = 8;    // accumulator rows per task (NI * G): 48 accumulators per lane
constexpr int kTileMaxL = 384;     // longest destination row the kernel covers (64 lanes x kTileT)
constexpr int kTileRecVals = 12;   // value slots per record
constexpr int kTileClasses = 8;    // records are grouped by entry count c = 1 .. 8
constexpr int kTileMaxStageRows = 64;  // source rows per stage (one per lane of the kernel's row list)

// entries per record for G rows sharing the segment
constexpr int tile_piece_max(int G) { return G == 1 ? 8 : (G == 2 ? 6 : (G == 3 ? 4 : 3)); }

struct TileRec {                 // 64 bytes
    int32_t a;                   // byte offset of the window start, 4 (lds_off + j0): lds_off = float offset
                                 // of the LDS row within a plane's stage buffer, j0 = first shift in [0, L)
    int32_t w;                   // L - j0: lanes whose first position is >= w wrap (read 4 L bytes lower)
    int32_t c;                   // entries (1 .. tile_piece_max(G))
    int32_t j0;
    float v[kTileRecVals];       // values [c][G]
};

struct TilePlan {
    bool ok = false;             // false: shape not covered (the staged or plain gather runs)
    int32_t NI = 1, G = 1;       // items per task, rows per item
    int32_t PW = 2;              // planes per wave: 2 when L <= 192 (32 lanes per plane), else 1
    int32_t NP = 8;              // planes staged per workgroup (4 PW; 4 PW / WS with a record split)
    int32_t deint = 1;           // LDS rows per staged source row (s for the forward, 1 for the backward)
    int32_t L = 0;               // destination positions per row (Wo)
    int32_t row_len = 0;         // elements of a source row in a plane (Wi forward, Wo backward)
    int32_t lrow = 0;            // floats per LDS row (L + halo, a multiple of 4)
    int32_t rows_per_stage = 0;  // source rows per stage
    int32_t max_recs = 0;        // most records of one stage (the stage's records are copied to LDS too)
    // Heavy tasks split their records over the workgroup's waves (WS = 4 or 2 waves share the same
    // planes and sum their partial accumulators in wave order at the end); tasks are ordered by
    // work, so tasks [0, n_ws4) take WS = 4, [n_ws4, n_ws2) WS = 2, the rest WS = 1.
    int32_t n_ws4 = 0, n_ws2 = 0;
    std::vector<Task> tasks;     // heaviest first
    std::vector<Stage> stages;   // Stage::segptr indexes stage_recptr
    // per task (task order): its first stage's descriptor (stages[0] for a task without stages), so
    // that a workgroup can read it knowing only its task number, beside the task itself
    std::vector<Stage> task_first;
    std::vector<int32_t> stage_rows;    // source row index within a plane (hi, or k Ho + ho)
    // per stage NI * kTileClasses + 1 bounds into recs: item-major, then by entry count c = 1..8
    std::vector<int32_t> stage_recptr;
    std::vector<TileRec> recs;
    std::vector<Item> items;     // NI per task; out_off[0] < 0 marks padding
};

// Wave-split classes of a launch over BC planes: the plan's (n_ws4, n_ws2), except that with fewer
// planes than a workgroup of one-wave tasks holds (4 PW) and tasks of kTileSplitMinRecs records or
// more on average, the tasks split their records over more waves, so that no wave is left without a
// plane: every task over 4 waves (PW planes per workgroup) when BC <= 2 PW, else at least over 2
// (2 PW planes) when BC < 4 PW.  Smaller tasks keep the plan's classes: for them the partial sums'
// pass through LDS costs more than the split saves.
constexpr int kTileSplitMinRecs = 32;
void tile_wave_split(int32_t n_tasks, int64_t n_recs, int32_t PW, int32_t plan_ws4, int32_t plan_ws2, int64_t BC,
                     int32_t &n_ws4, int32_t &n_ws2);

// `p` from build_forward_plan (backward = false) or build_backward_plan (backward = true);
// `lds_budget` = bytes of LDS one workgroup may use.
void build_tile_plan(const CSRView &c, const GatherPlan &p, bool backward, int lds_budget, TilePlan &out);

}  // namespace disco
