// plan_check.cpp — host-only checker of the device work plans (built with g++ and the address
// and undefined-behaviour sanitizers by the CPU test suite; it never touches a GPU).
//
// For one CSR read from a file it builds every plan disco_psi_create builds and checks
//   * that every index a kernel derives from a plan stays inside the buffer it addresses
//     (segments, records and stages of the plain, staged and tiled gathers, LDS reads and
//     writes, output offsets; descriptors, psi words and window runs of the phase-split
//     matrix-core plans), and
//   * that the plans reproduce the contraction: each kernel's loop structure is replayed on
//     the CPU in fp64 and compared with the CSR definition (for the matrix-core plans: every
//     lane's operands of every v_mfma_f32_32x32x16 block, summed as the instruction does, with
//     psi rounded to bf16 as the plan stores it), every destination element of the gathers is
//     written by exactly one item, and the row-inverted CSR of the matrix-core backward
//     reproduces the backward.
// Usage: plan_check <csr file>; exit status 0 when every check passes.
// File layout (little endian): int32 K, Ho, Wo, Hi, Wi; int64 nnz; int64 row_ptr[K Ho + 1];
// int32 col_hi[nnz]; int32 col_wi[nnz]; float val[nnz].
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "plan.hpp"
#include "plan_fused.hpp"
#include "plan_tile.hpp"

using namespace disco;

namespace {

int g_fail = 0;

void report(const std::string &what)
{
    if (g_fail < 20) fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++g_fail;
}

// the message is built only when the check fails (checks run in the replay's inner loops)
#define check(ok, what)            \
    do {                           \
        if (!(ok)) report(what);   \
    } while (0)

// CSR definition in fp64: out[k, ho, wo] for one plane
std::vector<double> ref_fwd(const CSRView &c, const std::vector<double> &x)
{
    const int s = c.Wi / c.Wo;
    std::vector<double> out((size_t)c.K * c.Ho * c.Wo, 0.0);
    for (int64_t r = 0; r < (int64_t)c.K * c.Ho; ++r)
        for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e)
            for (int wo = 0; wo < c.Wo; ++wo)
                out[r * c.Wo + wo] += (double)c.val[e] * x[(size_t)c.col_hi[e] * c.Wi + (c.col_wi[e] + s * wo) % c.Wi];
    return out;
}

std::vector<double> ref_bwd(const CSRView &c, const std::vector<double> &g)
{
    const int s = c.Wi / c.Wo;
    std::vector<double> gx((size_t)c.Hi * c.Wi, 0.0);
    for (int64_t r = 0; r < (int64_t)c.K * c.Ho; ++r)
        for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e)
            for (int wo = 0; wo < c.Wo; ++wo)
                gx[(size_t)c.col_hi[e] * c.Wi + (c.col_wi[e] + s * wo) % c.Wi] += (double)c.val[e] * g[r * c.Wo + wo];
    return gx;
}

void compare(const std::vector<double> &got, const std::vector<double> &want, const std::vector<int> &writes,
             const char *what)
{
    double err = 0.0, scale = 0.0;
    for (size_t i = 0; i < want.size(); ++i) scale = std::max(scale, std::fabs(want[i]));
    int64_t bad_writes = 0;
    for (size_t i = 0; i < want.size(); ++i) {
        err = std::max(err, std::fabs(got[i] - want[i]));
        if (writes[i] != 1) ++bad_writes;
    }
    check(err <= 1e-9 * std::max(scale, 1.0), std::string(what) + ": replay differs from the CSR definition");
    check(bad_writes == 0, std::string(what) + ": " + std::to_string(bad_writes) +
                               " destination elements not written exactly once");
}

// ---- plain gather (kernels_gather.hip) -------------------------------------------------------
void check_gather(const CSRView &c, const GatherPlan &p, bool backward, const std::vector<double> &src,
                  const std::vector<double> &want)
{
    const char *what = backward ? "gather plan (backward)" : "gather plan (forward)";
    const int64_t src_plane = backward ? (int64_t)c.K * c.Ho * c.Wo : (int64_t)c.Hi * c.Wi;
    const int64_t dst_plane = backward ? (int64_t)c.Hi * c.Wi : (int64_t)c.K * c.Ho * c.Wo;
    std::vector<double> got(dst_plane, 0.0);
    std::vector<int> writes(dst_plane, 0);
    check(p.order.size() == p.items.size(), std::string(what) + ": order size");
    for (size_t i = 0; i < p.items.size(); ++i) {
        const Item &it = p.items[i];
        check(it.G >= 1 && it.G <= kMaxGroup, std::string(what) + ": item G");
        check(it.seg_begin >= 0 && it.seg_begin <= it.seg_end && it.seg_end <= (int32_t)p.segs.size(),
              std::string(what) + ": item segment range");
        std::vector<double> acc((size_t)it.G * p.L, 0.0);
        for (int32_t q = it.seg_begin; q < it.seg_end && q < (int32_t)p.segs.size(); ++q) {
            const Seg &sg = p.segs[q];
            check(sg.m >= 1 && sg.m <= kMaxSegLen && sg.j0 >= 0 && sg.j0 < p.L, std::string(what) + ": segment fields");
            check(sg.val_off >= 0 && (int64_t)sg.val_off + (int64_t)sg.m * it.G <= (int64_t)p.vals.size(),
                  std::string(what) + ": segment values out of range");
            for (int32_t t = 0; t < sg.m; ++t) {
                int base = sg.j0 + t;
                if (base >= p.L) base -= p.L;
                for (int j = 0; j < p.L; ++j) {
                    int idx = base + j;
                    if (idx >= p.L) idx -= p.L;
                    const int64_t a = (int64_t)sg.in_off + (int64_t)p.in_stride * idx;
                    check(a >= 0 && a < src_plane, std::string(what) + ": source read out of the plane");
                    if (a < 0 || a >= src_plane) return;
                    for (int g = 0; g < it.G; ++g)
                        acc[(size_t)g * p.L + j] += (double)p.vals[sg.val_off + t * it.G + g] * src[a];
                }
            }
        }
        for (int g = 0; g < it.G; ++g)
            for (int j = 0; j < p.L; ++j) {
                const int64_t o = (int64_t)it.out_off[g] + (int64_t)it.out_stride * j;
                check(o >= 0 && o < dst_plane, std::string(what) + ": store out of the plane");
                if (o < 0 || o >= dst_plane) return;
                got[o] = acc[(size_t)g * p.L + j];
                writes[o]++;
            }
    }
    compare(got, want, writes, what);
}

// ---- source windows of the vector-ALU fused kernels (plan.hpp, FusedWindows) -----------------------
// Replays the fused kernels' contraction from staged windows: for every latitude and tile of px
// output longitudes, the window image as the staging writes it, then every entry's read at
// seg_off + t + (wo - wo0), which must stay inside its own row's staged positions.
void check_windows(const CSRView &c, const GatherPlan &p, const FusedWindows &w, int px, const std::vector<double> &x,
                   const std::vector<double> &want)
{
    const std::string what = "fused windows";
    const int32_t L = p.L, nb = (int32_t)p.block_ptr.size() - 1;
    check(w.ho_ptr.size() == (size_t)nb + 1 && w.ho_len.size() == (size_t)nb && w.seg_off.size() == p.segs.size(),
          what + ": table sizes");
    if (w.ho_ptr.size() != (size_t)nb + 1 || w.ho_len.size() != (size_t)nb || w.seg_off.size() != p.segs.size()) return;
    const int64_t src_plane = (int64_t)c.Hi * c.Wi, dst_plane = (int64_t)c.K * c.Ho * c.Wo;
    std::vector<double> got(dst_plane, 0.0);
    std::vector<int> writes(dst_plane, 0);
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t r0 = w.ho_ptr[b], r1 = w.ho_ptr[b + 1];
        check(0 <= r0 && r0 <= r1 && r1 <= (int32_t)w.rows.size(), what + ": row range");
        if (!(0 <= r0 && r0 <= r1 && r1 <= (int32_t)w.rows.size())) return;
        int32_t base = 0;
        for (int32_t r = r0; r < r1; ++r) {
            const FWin &fr = w.rows[r];
            check(fr.base == base && fr.len >= px && fr.a >= 0 && fr.a < L, what + ": row fields");
            check(fr.in_off >= 0 && (int64_t)fr.in_off + (int64_t)p.in_stride * (L - 1) < src_plane,
                  what + ": row out of the plane");
            if ((int64_t)fr.in_off + (int64_t)p.in_stride * (L - 1) >= src_plane || fr.in_off < 0) return;
            base += fr.len;
        }
        check(base == w.ho_len[b], what + ": latitude length");
        for (int32_t wo0 = 0; wo0 < L; wo0 += px) {
            std::vector<double> img((size_t)std::max(base, 0), NAN);
            for (int32_t r = r0; r < r1; ++r) {
                const FWin &fr = w.rows[r];
                for (int32_t q = 0; q < fr.len; ++q)
                    img[(size_t)fr.base + q] = x[(size_t)fr.in_off + (size_t)p.in_stride * ((fr.a + wo0 + q) % L)];
            }
            for (int32_t i = p.block_ptr[b]; i < p.block_ptr[b + 1]; ++i) {
                const Item &it = p.items[i];
                for (int32_t j = wo0; j < std::min(L, wo0 + px); ++j) {
                    double acc[kMaxGroup] = {0.0, 0.0, 0.0, 0.0};
                    for (int32_t q = it.seg_begin; q < it.seg_end; ++q) {
                        const Seg &sg = p.segs[q];
                        int32_t rr = -1;  // the segment's row
                        for (int32_t r = r0; r < r1; ++r)
                            if (w.rows[r].in_off == sg.in_off) rr = r;
                        check(rr >= 0, what + ": segment without a row");
                        if (rr < 0) return;
                        const FWin &fr = w.rows[rr];
                        for (int32_t t = 0; t < sg.m; ++t) {
                            const int64_t pos = (int64_t)w.seg_off[q] + t + (j - wo0);
                            check(pos >= fr.base && pos < (int64_t)fr.base + fr.len, what + ": read outside its row");
                            if (pos < fr.base || pos >= (int64_t)fr.base + fr.len) return;
                            for (int g = 0; g < it.G; ++g) acc[g] += (double)p.vals[sg.val_off + t * it.G + g] * img[pos];
                        }
                    }
                    for (int g = 0; g < it.G; ++g) {
                        const int64_t o = (int64_t)it.out_off[g] + (int64_t)it.out_stride * j;
                        check(o >= 0 && o < dst_plane, what + ": store out of the plane");
                        if (o < 0 || o >= dst_plane) return;
                        got[o] = acc[g];
                        writes[o]++;
                    }
                }
            }
        }
    }
    compare(got, want, writes, what.c_str());
}

// ---- LDS-staged gather (kernels_staged.hip) ----------------------------------------------------
void check_staged(const CSRView &c, const StagedPlan &sp, bool backward, int elem_bytes, int lds_budget,
                  const std::vector<double> &src, const std::vector<double> &want)
{
    if (!sp.ok) return;
    const std::string what = std::string("staged plan (") + (backward ? "backward" : "forward") + ", " +
                             std::to_string(elem_bytes) + "-byte elements)";
    const int64_t dst_plane = backward ? (int64_t)c.Hi * c.Wi : (int64_t)c.K * c.Ho * c.Wo;
    const int64_t nsrc_rows = backward ? (int64_t)c.K * c.Ho : c.Hi;
    check((int64_t)sp.NP * sp.rows_per_stage * sp.lrow * elem_bytes <= lds_budget, what + ": stage exceeds its LDS");
    check(sp.lrow >= sp.row_len + sp.halo, what + ": LDS row shorter than row + halo");
    if (sp.lrow < sp.row_len + sp.halo) return;  // the replay below would write past its rows
    std::vector<double> got(dst_plane, 0.0);
    std::vector<int> writes(dst_plane, 0);
    const int T = sp.T, S_ = sp.S;
    const int lanes = 64 * sp.wpp;
    for (const Task &task : sp.tasks) {
        check(task.item_begin >= 0 && task.item_begin + sp.NI <= (int32_t)sp.items.size(), what + ": task items");
        check(task.stage_begin >= 0 && task.stage_begin <= task.stage_end && task.stage_end <= (int32_t)sp.stages.size(),
              what + ": task stages");
        std::vector<double> acc((size_t)sp.NI * sp.G * sp.L, 0.0);
        for (int32_t st = task.stage_begin; st < task.stage_end; ++st) {
            const Stage &sg = sp.stages[st];
            const int nrows = sg.row_end - sg.row_begin;
            check(nrows >= 1 && nrows <= sp.rows_per_stage, what + ": rows per stage");
            // LDS image of the stage: row r holds source positions (e mod row_len) for e < row_len + halo
            std::vector<double> lds((size_t)sp.rows_per_stage * sp.lrow, NAN);
            for (int r = 0; r < nrows; ++r) {
                const int32_t row = sp.stage_rows[sg.row_begin + r];
                check(row >= 0 && row < nsrc_rows, what + ": stage row out of the plane");
                for (int e = 0; e < sp.row_len + sp.halo; ++e) lds[(size_t)r * sp.lrow + e] = src[(size_t)row * sp.row_len + e % sp.row_len];
            }
            for (int i = 0; i < sp.NI; ++i) {
                const int32_t q0 = sp.stage_segptr[sg.segptr + i], q1 = sp.stage_segptr[sg.segptr + i + 1];
                check(q0 >= 0 && q0 <= q1 && q1 <= (int32_t)sp.segs.size(), what + ": stage segment range");
                for (int32_t q = q0; q < q1; ++q) {
                    const Seg &s = sp.segs[q];
                    check(s.m >= 1 && s.m <= kStagedSegLen, what + ": segment length");
                    check((int64_t)s.val_off + (int64_t)s.m * sp.G <= (int64_t)sp.vals.size(), what + ": segment values");
                    for (int lane = 0; lane < lanes; ++lane) {
                        const int jl = lane * T;
                        if (jl >= sp.L) continue;
                        int base = s.j0 + jl;
                        if (base >= sp.L) base -= sp.L;
                        for (int u = 0; u < s.m + T - 1; ++u) {
                            const int64_t a = s.in_off + (int64_t)S_ * (base + u);
                            check(a >= 0 && a < (int64_t)nrows * sp.lrow, what + ": LDS read outside the staged rows");
                            if (a < 0 || a >= (int64_t)nrows * sp.lrow) return;
                            check(!std::isnan(lds[a]), what + ": LDS read of an unstaged word");
                        }
                        for (int t = 0; t < T && jl + t < sp.L; ++t)
                            for (int e = 0; e < s.m; ++e)
                                for (int g = 0; g < sp.G; ++g)
                                    acc[((size_t)i * sp.G + g) * sp.L + jl + t] +=
                                        (double)sp.vals[s.val_off + e * sp.G + g] * lds[s.in_off + S_ * (base + e + t)];
                    }
                }
            }
        }
        for (int i = 0; i < sp.NI; ++i) {
            const Item &it = sp.items[task.item_begin + i];
            for (int g = 0; g < sp.G; ++g)
                for (int j = 0; j < sp.L; ++j) {
                    const int64_t o = (int64_t)it.out_off[g] + (int64_t)it.out_stride * j;
                    check(o >= 0 && o < dst_plane, what + ": store out of the plane");
                    if (o < 0 || o >= dst_plane) return;
                    got[o] = acc[((size_t)i * sp.G + g) * sp.L + j];
                    writes[o]++;
                }
        }
    }
    compare(got, want, writes, what.c_str());
}

// ---- register-tiled fp32 gather (kernels_tile.hip) ---------------------------------------------
void check_tile(const CSRView &c, const TilePlan &tp, bool backward, int lds_budget, const std::vector<double> &src,
                const std::vector<double> &want)
{
    if (!tp.ok) return;
    const std::string what = std::string("tiled plan (") + (backward ? "backward" : "forward") + ")";
    const int64_t dst_plane = backward ? (int64_t)c.Hi * c.Wi : (int64_t)c.K * c.Ho * c.Wo;
    const int64_t nsrc_rows = backward ? (int64_t)c.K * c.Ho : c.Hi;
    const int T = kTileT;
    const int stage_floats = tp.rows_per_stage * tp.deint * tp.lrow;
    check((int64_t)tp.NP * stage_floats * 4 + (int64_t)sizeof(TileRec) * tp.max_recs <= lds_budget,
          what + ": stage rows and records exceed the LDS");
    check(tp.lrow % 4 == 0 && tp.lrow >= tp.L + kTileHalo, what + ": LDS row layout");
    if (tp.lrow < tp.L + kTileHalo || tp.deint < 1) return;  // the replay below would write past its rows
    check(tp.deint * tp.L == tp.row_len, what + ": residue rows do not tile the source row");
    check(tp.NP == 4 * tp.PW && (tp.PW == 1 || tp.PW == 2) && (64 / tp.PW) * T >= tp.L, what + ": lane layout");
    check(0 <= tp.n_ws4 && tp.n_ws4 <= tp.n_ws2 && tp.n_ws2 <= (int32_t)tp.tasks.size(), what + ": wave-split classes");
    check(tp.NI * tp.G <= kTileMaxRows, what + ": more accumulator rows than the kernel holds");
    // any launch may split its tasks over waves (few planes: tile_wave_split), so the sums' area must fit
    check(3LL * 64 * tp.NI * tp.G * T * 4 <= lds_budget, what + ": wave-split sums exceed the LDS");
    std::vector<double> got(dst_plane, 0.0);
    std::vector<int> writes(dst_plane, 0);
    const int lanes = 64 / tp.PW;  // lanes of one plane
    const int cmax = tile_piece_max(tp.G);
    check(tp.task_first.size() == tp.tasks.size(), what + ": one first-stage descriptor per task");
    for (size_t ti = 0; ti < tp.tasks.size(); ++ti) {
        // the kernel reads task_first[ti] and that stage's metadata before it knows the task's stages
        const Task &t = tp.tasks[ti];
        const Stage &f = tp.task_first[ti];
        if (tp.stages.empty()) continue;  // not read then
        const Stage &want = t.stage_begin < t.stage_end && t.stage_begin >= 0 && t.stage_begin < (int32_t)tp.stages.size()
                                ? tp.stages[t.stage_begin] : tp.stages[0];
        check(f.row_begin == want.row_begin && f.row_end == want.row_end && f.segptr == want.segptr,
              what + ": first-stage descriptor of a task");
    }
    for (const Task &task : tp.tasks) {
        check(task.item_begin >= 0 && task.item_begin + tp.NI <= (int32_t)tp.items.size(), what + ": task items");
        check(task.stage_begin >= 0 && task.stage_begin <= task.stage_end && task.stage_end <= (int32_t)tp.stages.size(),
              what + ": task stages");
        std::vector<double> acc((size_t)tp.NI * tp.G * tp.L, 0.0);
        for (int32_t st = task.stage_begin; st < task.stage_end; ++st) {
            const Stage &sg = tp.stages[st];
            const int nrows = sg.row_end - sg.row_begin;
            check(nrows >= 1 && nrows <= tp.rows_per_stage && nrows <= kTileMaxStageRows, what + ": rows per stage");
            check(tp.stage_recptr[sg.segptr + tp.NI * kTileClasses] - tp.stage_recptr[sg.segptr] <= tp.max_recs,
                  what + ": stage holds more records than its LDS area");
            // LDS image as the staging loop writes it: residue rho of staged row r at (r deint + rho) lrow,
            // positions [0, L) and the halo [L, L + kTileHalo)
            std::vector<double> lds((size_t)stage_floats, NAN);
            for (int r = 0; r < nrows; ++r) {
                const int32_t row = tp.stage_rows[sg.row_begin + r];
                check(row >= 0 && row < nsrc_rows, what + ": stage row out of the plane");
                if (row < 0 || row >= nsrc_rows) return;
                for (int e = 0; e < tp.row_len; ++e) {
                    const int rho = e % tp.deint, jj = e / tp.deint;
                    lds[(size_t)(r * tp.deint + rho) * tp.lrow + jj] = src[(size_t)row * tp.row_len + e];
                }
                for (int h = 0; h < tp.deint * kTileHalo; ++h) {
                    const int rho = h / kTileHalo, pos = h % kTileHalo;
                    lds[(size_t)(r * tp.deint + rho) * tp.lrow + tp.L + pos] =
                        src[(size_t)row * tp.row_len + rho + tp.deint * (pos % tp.L)];
                }
            }
            for (int i = 0; i < tp.NI; ++i) {
                for (int cl = 0; cl < kTileClasses; ++cl) {
                const int32_t r0 = tp.stage_recptr[sg.segptr + i * kTileClasses + cl];
                const int32_t r1 = tp.stage_recptr[sg.segptr + i * kTileClasses + cl + 1];
                check(r0 >= 0 && r0 <= r1 && r1 <= (int32_t)tp.recs.size(), what + ": stage record range");
                for (int32_t q = r0; q < r1; ++q) {
                    const TileRec &rec = tp.recs[q];
                    const int rc = rec.c;
                    check(rc == cl + 1, what + ": record in the wrong entry-count class");
                    check(rc >= 1 && rc <= cmax && rc * tp.G <= kTileRecVals, what + ": record entry count");
                    check(rec.j0 >= 0 && rec.j0 < tp.L && rec.w == tp.L - rec.j0, what + ": record shift");
                    const int lds_off = rec.a / 4 - rec.j0;  // float offset of the record's LDS row
                    check(rec.a % 4 == 0 && lds_off >= 0 && lds_off % tp.lrow == 0 && lds_off / tp.lrow < nrows * tp.deint,
                          what + ": record LDS row");
                    for (int lane = 0; lane < lanes; ++lane) {
                        const int jl = lane * T;
                        const int jlc = jl < tp.L ? jl : 0;
                        // the kernel's address: 4 jlc + a, less 4 L when jlc >= w
                        const int64_t byte = 4LL * jlc + rec.a - (jlc >= rec.w ? 4LL * tp.L : 0);
                        const int64_t base = byte / 4 - lds_off;  // position within the row
                        check(byte % 4 == 0 && base >= 0 && base < tp.L, what + ": window start outside its row");
                        if (base < 0 || base >= tp.L) return;
                        for (int u = 0; u < rc + T - 1; ++u) {
                            const int64_t a = (int64_t)lds_off + base + u;
                            const bool in_row = base + u < tp.lrow;
                            check(in_row && a < stage_floats, what + ": LDS read past its row");
                            if (!in_row || a >= stage_floats) return;
                            check(!std::isnan(lds[a]), what + ": LDS read of an unstaged word");
                        }
                        if (jl >= tp.L) continue;
                        check(base == (rec.j0 + jl) % tp.L, what + ": window start is not (j0 + j) mod L");
                        for (int t = 0; t < T && jl + t < tp.L; ++t)
                            for (int e = 0; e < rc; ++e)
                                for (int g = 0; g < tp.G; ++g)
                                    acc[((size_t)i * tp.G + g) * tp.L + jl + t] +=
                                        (double)rec.v[e * tp.G + g] * lds[lds_off + base + e + t];
                    }
                }
                }
            }
        }
        for (int i = 0; i < tp.NI; ++i) {
            const Item &it = tp.items[task.item_begin + i];
            if (it.out_off[0] < 0) continue;
            for (int g = 0; g < tp.G; ++g)
                for (int j = 0; j < tp.L; ++j) {
                    const int64_t o = (int64_t)it.out_off[g] + (int64_t)it.out_stride * j;
                    check(o >= 0 && o < dst_plane, what + ": store out of the plane");
                    if (o < 0 || o >= dst_plane) return;
                    got[o] = acc[((size_t)i * tp.G + g) * tp.L + j];
                    writes[o]++;
                }
        }
    }
    compare(got, want, writes, what.c_str());
}

// The tiled kernel's workgroup -> (task, planes, record share) decode, replayed for BC planes:
// every (task, plane) pair must be served by exactly WS waves with distinct shares.
void check_tile_grid(const TilePlan &tp, int BC)
{
    if (!tp.ok) return;
    const std::string what = "tiled grid (" + std::to_string(BC) + " planes)";
    const int PW = tp.PW, nt = (int)tp.tasks.size();
    int32_t n_ws4 = 0, n_ws2 = 0;  // the classes the launch uses for BC planes
    tile_wave_split(nt, (int64_t)tp.recs.size(), PW, tp.n_ws4, tp.n_ws2, BC, n_ws4, n_ws2);
    check(0 <= n_ws4 && n_ws4 <= n_ws2 && n_ws2 <= nt, what + ": wave-split classes");
    const int npg4 = (BC + PW - 1) / PW, npg2 = (BC + 2 * PW - 1) / (2 * PW), npg1 = (BC + 4 * PW - 1) / (4 * PW);
    const int64_t nblk = (int64_t)n_ws4 * npg4 + (int64_t)(n_ws2 - n_ws4) * npg2 + (int64_t)(nt - n_ws2) * npg1;
    std::vector<int> seen((size_t)nt * BC, 0);
    for (int64_t b = 0; b < nblk; ++b) {
        int bid = (int)b, ti, pg, WS;
        const int nb4 = n_ws4 * npg4, nb2 = (n_ws2 - n_ws4) * npg2;
        if (bid < nb4) {
            WS = 4; ti = bid / npg4; pg = bid - ti * npg4;
        } else if (bid < nb4 + nb2) {
            bid -= nb4;
            WS = 2; ti = n_ws4 + bid / npg2; pg = bid - (ti - n_ws4) * npg2;
        } else {
            bid -= nb4 + nb2;
            WS = 1; ti = n_ws2 + bid / npg1; pg = bid - (ti - n_ws2) * npg1;
        }
        check(ti >= 0 && ti < nt, what + ": task index out of range");
        if (ti < 0 || ti >= nt) return;
        const int NPB = 4 * PW / WS;
        check(NPB <= tp.NP, what + ": more planes in a workgroup than its LDS holds");
        for (int wave = 0; wave < 4; ++wave)
            for (int half = 0; half < PW; ++half) {
                const int wsi = wave % WS;
                const int ps = (wave / WS) * PW + half;
                check(ps < NPB, what + ": plane slot outside the workgroup's planes");
                const int plane = pg * NPB + ps;
                if (plane < BC) seen[(size_t)ti * BC + plane] |= 1 << wsi;
            }
    }
    for (int ti = 0; ti < nt; ++ti) {
        const int WS = ti < n_ws4 ? 4 : (ti < n_ws2 ? 2 : 1);
        for (int pl = 0; pl < BC; ++pl)
            check(seen[(size_t)ti * BC + pl] == (1 << WS) - 1, what + ": a (task, plane) is not served by each share once");
    }
}



// ---- phase-split plans of the matrix-core kernels (kernels_fused_mfma.hip) -------------------

float bf16_value(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// round to nearest even, written here from the bf16 format (8 exponent bits, 7 fraction bits)
float round_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return f;  // NaN stays NaN
    const uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7fffu + lsb) & 0xffff0000u;
    float r;
    std::memcpy(&r, &u, 4);
    return r;
}

// CSR definition at one output element with bf16 psi: sum over row (k, ho) of psi * src[hi, (wi + s wo) mod Wi]
double ref_at(const CSRView &c, const std::vector<double> &src, int k, int ho, int wo)
{
    const int s = c.Wi / c.Wo;
    const int64_t r = (int64_t)k * c.Ho + ho;
    double acc = 0.0;
    for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e)
        acc += (double)round_bf16(c.val[e]) * src[(size_t)c.col_hi[e] * c.Wi + (c.col_wi[e] + (int64_t)s * wo) % c.Wi];
    return acc;
}

struct PhaseBudget {
    int kr, ch;
    int64_t piece_budget;  // bytes of one streamed stage
    bool resident;         // resident latitudes allowed
    int xch_bytes;         // smallest window buffer of a resident latitude
};

// Replays the matrix-core contraction of plan p over CSR c (source plane src = c.Hi rows of c.Wi):
// for every latitude and the checked longitude spans, the piece stages are built as the kernels
// build them (descriptors and psi copied from the plan, window rows from the source plane, the
// rest of the window area left as NaN), every lane of every block reads its psi words (four, or
// five realigned) and its x runs with the kernels' lane offsets (A row r of phase group g:
// phase q, basis k; B column n), and the 16-offset products are summed in fp64.  Rows k >= K and
// longitudes past Wo are computed and must stay finite; the others must match the definition.
void check_phase(const CSRView &c, const FusedPlan &p, const PhaseBudget &bu, const std::vector<double> &src,
                 const std::string &what)
{
    if (!p.ok) return;
    const int s = c.Wi / c.Wo, kr = bu.kr;
    check(p.s == s && p.kr == kr && p.ch == bu.ch, what + ": plan parameters");
    check((int)p.ho_piece.size() == c.Ho + 1 && p.ho_piece[0] == 0 && p.ho_piece.back() == (int32_t)p.pieces.size(),
          what + ": latitude piece table");
    if ((int)p.ho_piece.size() != c.Ho + 1) return;
    std::vector<int> seen(c.Ho, 0);
    check((int)p.ho_order.size() == c.Ho, what + ": latitude order size");
    for (int32_t h : p.ho_order) {
        check(h >= 0 && h < c.Ho, what + ": latitude order entry");
        if (h >= 0 && h < c.Ho) ++seen[h];
    }
    for (int h = 0; h < c.Ho; ++h) check(seen[h] == 1, what + ": latitude order is not a permutation");
    check(p.adata.size() == p.adata16.size(), what + ": fp16 psi size");
    // structure of every piece
    for (size_t i = 0; i < p.pieces.size(); ++i) {
        const FPiece &pc = p.pieces[i];
        const std::string pw = what + ": piece " + std::to_string(i);
        check(pc.nblk >= 0 && pc.nblk % 2 == 0 && pc.desc_words == 2 * pc.nblk && pc.desc_words % 4 == 0,
              pw + " block count / descriptor words");
        check(pc.desc_begin >= 0 && 2 * ((int64_t)pc.desc_begin + pc.nblk) <= (int64_t)p.descs.size() &&
                  (2 * (int64_t)pc.desc_begin) % 4 == 0,
              pw + " descriptors outside the table or not 16-byte aligned");
        check(pc.a_begin >= 0 && pc.a_begin % 8 == 0 && pc.a_elems >= 0 && pc.a_elems % 8 == 0 &&
                  (int64_t)pc.a_begin + pc.a_elems <= (int64_t)p.adata.size(),
              pw + " psi range outside the table or not 16-byte units");
        check(pc.row_begin >= 0 && pc.row_begin <= pc.row_end && pc.row_end <= (int32_t)p.rows.size(), pw + " rows");
        check(pc.win_elems >= 0 && pc.win_elems % 8 == 0 && pc.win_elems <= p.max_win, pw + " window area");
        check(pc.a_copy_bytes == 0 || (pc.a_copy_bytes == pc.a_elems && pc.a_elems % 16 == 0), pw + " second psi copy");
        check(!(pc.a_copy_bytes > 0 && pc.realign), pw + " two copies and realigned reads");
        if (pc.row_begin < 0 || pc.row_end > (int32_t)p.rows.size() || pc.row_begin > pc.row_end) continue;
        int64_t covered = 0;
        for (int32_t j = pc.row_begin; j < pc.row_end; ++j) {
            const FRow &fr = p.rows[j];
            check(fr.sr >= 0 && fr.sr < c.Hi, pw + " source row outside the plane");
            check(fr.len > 0 && fr.len % (s == 2 ? 16 : 8) == 0 && fr.start % 8 == 0 && fr.win_off == covered,
                  pw + " window rows not contiguous 8-element runs (16 when s = 2)");
            covered += fr.len;
        }
        check(covered == pc.win_elems, pw + " window rows do not fill the window area");
        const int64_t stage = 4 * (int64_t)pc.desc_words + 2 * (int64_t)pc.a_elems;
        if (pc.resident > 0) {
            check(bu.resident, pw + " resident piece in a streamed plan");
            check(p.ho_piece.size() > 1, pw + " resident");
            check(pc.resident % 16 == 0 && pc.resident >= 2 * (int64_t)bu.ch * pc.win_elems && pc.resident >= bu.xch_bytes,
                  pw + " resident window buffer too small");
            check(stage + 2 * (int64_t)pc.resident <= p.max_resident_bytes &&
                      p.max_resident_bytes <= 2 * bu.piece_budget,
                  pw + " resident layout exceeds its LDS");
        } else {
            check(fused_piece_bytes(pc.desc_words, pc.a_elems, bu.ch, pc.win_elems) <= p.max_piece_bytes &&
                      p.max_piece_bytes <= bu.piece_budget,
                  pw + " stage exceeds its LDS");
        }
    }
    for (int h = 0; h < c.Ho; ++h) {
        const int n = p.ho_piece[h + 1] - p.ho_piece[h];
        check(n >= 0, what + ": latitude pieces");
        for (int i = p.ho_piece[h]; i < p.ho_piece[h + 1]; ++i)
            check(p.pieces[i].resident == 0 || n == 1, what + ": a resident latitude has one piece");
    }
    if (g_fail) return;

    // the replay
    const int PH = 32 / kr;  // phases per MFMA
    const int n_spans = (c.Wo + kFusedSpan - 1) / kFusedSpan;
    // columns: both ends of a span (the window's first and last runs) and a few inside; every span
    // of a narrow grid, else the first and the last (ragged) one
    std::vector<int> spans, cols = {0, 1, 2, 15, 16, 30, 31};
    if (c.Wo <= 2 * kFusedSpan) {
        for (int i = 0; i < n_spans; ++i) spans.push_back(i);
    } else {
        spans = {0, n_spans - 1};
    }
    double scale = 0.0, err = 0.0;
    std::vector<double> win, acc;
    for (int ho = 0; ho < c.Ho; ++ho) {
        for (int sp : spans) {
            const int px0 = sp * kFusedSpan;
            acc.assign((size_t)8 * kr * cols.size(), 0.0);
            for (int pi = p.ho_piece[ho]; pi < p.ho_piece[ho + 1]; ++pi) {
                const FPiece &pc = p.pieces[pi];
                // a channel's window area as the kernels stage it: element e of the area at e, or with
                // s = 2 split by unit parity, unit u at unit (u % 2) (win_elems / 16) + u / 2
                const int half = pc.win_elems / 16;
                auto phys = [&](int64_t e) {
                    if (s != 2) return e;
                    const int64_t u = e / 8;
                    return 8 * ((u % 2) * half + u / 2) + e % 8;
                };
                win.assign(pc.win_elems, NAN);
                for (int32_t j = pc.row_begin; j < pc.row_end; ++j) {
                    const FRow &fr = p.rows[j];
                    for (int i = 0; i < fr.len; ++i) {
                        int64_t col = ((int64_t)s * px0 + fr.start + i) % c.Wi;
                        if (col < 0) col += c.Wi;
                        const int64_t e = phys((int64_t)fr.win_off + i);
                        check(e >= 0 && e < pc.win_elems, what + ": staged window element outside the area");
                        if (e < 0 || e >= pc.win_elems) return;
                        win[e] = src[(size_t)fr.sr * c.Wi + col];
                    }
                }
                const int64_t psi_bytes = 2 * (int64_t)pc.a_elems;
                for (int blk = 0; blk < pc.nblk; ++blk) {
                    const int32_t ax = p.descs[2 * ((size_t)pc.desc_begin + blk)];
                    const int32_t xo = p.descs[2 * ((size_t)pc.desc_begin + blk) + 1];
                    check(ax % 4 == 0 && xo % 16 == 0, what + ": block descriptor alignment");
                    check(s != 2 || pc.win_elems % 16 == 0, what + ": split window area of odd unit count");
                    for (int q = 0; q < 8; ++q) {
                        const int sq = s * q;
                        const bool odd = (sq & 1) != 0;
                        for (int k = 0; k < kr; ++k) {
                            for (int hh = 0; hh < 2; ++hh) {
                                // psi: the lane's words (A row = phase q, basis k; K half hh)
                                const int64_t lane = 4 * (int64_t)kr * (4 * hh - (sq + 1) / 2) + 4 * k + ax +
                                                     (odd && !pc.realign ? pc.a_copy_bytes : 0);
                                const int nw = pc.realign ? 5 : 4;
                                float h10[10];
                                bool in = true;
                                for (int w = 0; w < nw; ++w) {
                                    const int64_t b = lane + 4 * (int64_t)kr * w;
                                    in = in && b >= 0 && b + 4 <= psi_bytes;
                                    if (b < 0 || b + 4 > psi_bytes) continue;
                                    h10[2 * w] = bf16_value(p.adata[pc.a_begin + b / 2]);
                                    h10[2 * w + 1] = bf16_value(p.adata[pc.a_begin + b / 2 + 1]);
                                }
                                check(in, what + ": psi word read outside the piece's psi");
                                if (!in) return;
                                const int sh = (pc.realign && odd) ? 1 : 0;
                                for (size_t ci = 0; ci < cols.size(); ++ci) {
                                    const int n = cols[ci];
                                    // B column n, K half hh: the kernels' lane byte offset (x_lane2, and
                                    // with s = 2 the odd half for hh = 1) plus the descriptor's
                                    const int64_t xb = s == 2 ? xo + 16 * (int64_t)n + (int64_t)hh * pc.win_elems
                                                              : xo + 2 * (8 * (int64_t)s * n + 8 * hh);
                                    check(xb % 16 == 0, what + ": x run not 16-byte aligned");
                                    const int64_t ex = xb / 2;
                                    check(ex >= 0 && ex + 8 <= pc.win_elems, what + ": x run outside the window area");
                                    if (ex < 0 || ex + 8 > pc.win_elems) return;
                                    double sum = 0.0;
                                    for (int i = 0; i < 8; ++i) {
                                        const double a = h10[sh + i];
                                        if (a != 0.0) sum += a * win[ex + i];
                                    }
                                    acc[((size_t)q * kr + k) * cols.size() + ci] += sum;
                                }
                            }
                        }
                    }
                }
            }
            for (int q = 0; q < 8; ++q)
                for (int k = 0; k < kr; ++k)
                    for (size_t ci = 0; ci < cols.size(); ++ci) {
                        const double got = acc[((size_t)q * kr + k) * cols.size() + ci];
                        const int wo = px0 + 8 * cols[ci] + q;
                        if (k >= c.K || wo >= c.Wo) {
                            check(std::isfinite(got), what + ": row past K or longitude past Wo reads unstaged LDS");
                            continue;
                        }
                        const double want = ref_at(c, src, k, ho, wo);
                        scale = std::max(scale, std::fabs(want));
                        if (!(std::fabs(got - want) <= err)) err = std::isnan(got) ? INFINITY : std::fabs(got - want);
                    }
        }
    }
    check(err <= 1e-9 * std::max(scale, 1.0),
          what + ": replay differs from the CSR definition (max error " + std::to_string(err) + ")");
    (void)PH;
}

// The row-inverted CSR of the matrix-core backward: its forward over gout rows, row r = ho' g + k'
// (= hi s + rho), column wo', must equal the backward gx[hi, rho + s wo'].
void check_inverse(const CSRView &c, const InverseCSR &inv, int g, const std::vector<double> &gsrc,
                   const std::vector<double> &want_b)
{
    const int s = c.Wi / c.Wo;
    const CSRView &v = inv.view;
    check(v.K == g && v.Ho == (c.Hi * s + g - 1) / g && v.Wo == c.Wo && v.Hi == c.K * c.Ho && v.Wi == c.Wo &&
              v.nnz == c.nnz,
          "inverse CSR shape");
    int code = 0;
    const std::string msg = validate_csr(v, &code);
    check(code == 0, "inverse CSR rejected: " + msg);
    if (code != 0) return;
    double err = 0.0, scale = 0.0;
    for (int ho = 0; ho < v.Ho; ++ho)
        for (int k = 0; k < g; ++k) {
            const int64_t r = (int64_t)ho * g + k;
            const int64_t R = (int64_t)k * v.Ho + ho;
            if (r >= (int64_t)c.Hi * s) {
                check(v.row_ptr[R] == v.row_ptr[R + 1], "inverse CSR: a row past the gradient holds entries");
                continue;
            }
            const int hi = (int)(r / s), rho = (int)(r % s);
            for (int wo = 0; wo < c.Wo; ++wo) {
                double acc = 0.0;
                for (int64_t e = v.row_ptr[R]; e < v.row_ptr[R + 1]; ++e)
                    acc += (double)v.val[e] * gsrc[(size_t)v.col_hi[e] * v.Wi + (v.col_wi[e] + wo) % v.Wi];
                const double want = want_b[(size_t)hi * c.Wi + rho + (int64_t)s * wo];
                scale = std::max(scale, std::fabs(want));
                err = std::max(err, std::fabs(acc - want));
            }
        }
    check(err <= 1e-9 * std::max(scale, 1.0), "inverse CSR: its forward differs from the backward");
}

// The per-basis transpose (Wi = Wo): its forward over gradient plane k must equal the backward of
// basis k alone (the gradient with every other basis plane zero).
void check_transposed(const CSRView &c, const TransposedCSR &tr, const std::vector<double> &g)
{
    const CSRView &v = tr.view;
    check(v.K == c.K && v.Ho == c.Hi && v.Wo == c.Wo && v.Hi == c.Ho && v.Wi == c.Wo && v.nnz == c.nnz,
          "transposed CSR shape");
    int code = 0;
    const std::string msg = validate_csr(v, &code);
    check(code == 0, "transposed CSR rejected: " + msg);
    if (code != 0) return;
    const size_t plane = (size_t)c.Ho * c.Wo;
    double err = 0.0, scale = 0.0;
    for (int k = 0; k < c.K; ++k) {
        std::vector<double> gk(g.size(), 0.0);
        std::copy(g.begin() + k * plane, g.begin() + (k + 1) * plane, gk.begin() + k * plane);
        const std::vector<double> want = ref_bwd(c, gk);
        for (int hi = 0; hi < c.Hi; ++hi) {
            const int64_t R = (int64_t)k * v.Ho + hi;
            for (int j = 0; j < c.Wo; ++j) {
                double acc = 0.0;
                for (int64_t e = v.row_ptr[R]; e < v.row_ptr[R + 1]; ++e)
                    acc += (double)v.val[e] * g[k * plane + (size_t)v.col_hi[e] * v.Wi + (v.col_wi[e] + j) % v.Wi];
                const double w = want[(size_t)hi * c.Wi + j];
                scale = std::max(scale, std::fabs(w));
                err = std::max(err, std::fabs(acc - w));
            }
        }
    }
    check(err <= 1e-9 * std::max(scale, 1.0), "transposed CSR: its forward differs from the per-basis backward");
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s <csr file>\n", argv[0]);
        return 2;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 2;
    }
    int32_t hdr[5];
    int64_t nnz = 0;
    if (fread(hdr, 4, 5, f) != 5 || fread(&nnz, 8, 1, f) != 1 || nnz < 0) {
        fprintf(stderr, "bad header\n");
        return 2;
    }
    const int64_t R = (int64_t)hdr[0] * hdr[1];
    std::vector<int64_t> row_ptr(R + 1);
    std::vector<int32_t> col_hi(nnz), col_wi(nnz);
    std::vector<float> val(nnz);
    if (fread(row_ptr.data(), 8, R + 1, f) != (size_t)(R + 1) || fread(col_hi.data(), 4, nnz, f) != (size_t)nnz ||
        fread(col_wi.data(), 4, nnz, f) != (size_t)nnz || fread(val.data(), 4, nnz, f) != (size_t)nnz) {
        fprintf(stderr, "short file\n");
        return 2;
    }
    fclose(f);
    CSRView c{hdr[0], hdr[1], hdr[2], hdr[3], hdr[4], nnz, row_ptr.data(), col_hi.data(), col_wi.data(), val.data()};
    int code = 0;
    const std::string msg = validate_csr(c, &code);
    if (code != 0) {
        fprintf(stderr, "CSR rejected: %s\n", msg.c_str());
        return 3;
    }

    std::mt19937_64 rng(12345);
    std::normal_distribution<double> nd;
    std::vector<double> x((size_t)c.Hi * c.Wi), g((size_t)c.K * c.Ho * c.Wo);
    for (auto &v : x) v = (double)(float)nd(rng);
    for (auto &v : g) v = (double)(float)nd(rng);
    const std::vector<double> want_f = ref_fwd(c, x), want_b = ref_bwd(c, g);

    GatherPlan fp, bp;
    build_forward_plan(c, fp);
    build_backward_plan(c, bp);
    check_gather(c, fp, false, x, want_f);
    check_gather(c, bp, true, g, want_b);
    FusedWindows fw;
    build_fused_windows(fp, 64, fw);  // the vector-ALU fused kernels' 64-longitude tiles
    check_windows(c, fp, fw, 64, x, want_f);
    // the library's budgets (disco_api.hip): 40 KiB per staged or tiled workgroup
    const int budget = 40 * 1024;
    for (int esz : {4, 2}) {
        StagedPlan sf, sb;
        build_staged_plan(c, fp, false, esz, budget, sf);
        build_staged_plan(c, bp, true, esz, budget, sb);
        check_staged(c, sf, false, esz, budget, x, want_f);
        check_staged(c, sb, true, esz, budget, g, want_b);
    }
    TilePlan tf, tb;
    build_tile_plan(c, fp, false, budget, tf);
    build_tile_plan(c, bp, true, budget, tb);
    check_tile(c, tf, false, budget, x, want_f);
    check_tile(c, tb, true, budget, g, want_b);
    for (int BC : {1, 2, 3, 5, 8, 13, 128}) {
        check_tile_grid(tf, BC);
        check_tile_grid(tb, BC);
    }
    // matrix-core plans with the library's parameters (disco_api.hip, kernels_fused_mfma.hip): fused
    // conv (basis rows 16, four channels per chunk, two 64 KiB stages beside the 32 KiB W slice,
    // resident latitudes with 32 KiB operand exchange), forward (basis rows 8 or 16, 8 or 4 channels,
    // 40 KiB stages), backward (8 gradient rows per group over the row-inverted CSR)
    FusedPlan fup, fwp, bwp;
    {
        PhaseBudget bf{16, 4, ((160 * 1024 - 32 * 1024) / 2) & ~15, true, 32 * 1024};
        PhasePlanParams prm;
        prm.kr = bf.kr; prm.ch = bf.ch; prm.piece_budget = (int)bf.piece_budget; prm.xch_bytes = bf.xch_bytes;
        build_phase_plan(c, prm, fup);
        check_phase(c, fup, bf, x, "fused matrix-core plan");
        const int fkr = c.K <= 8 ? 8 : 16;
        PhaseBudget bw{fkr, fkr == 8 ? 8 : 4, 40 * 1024, false, 0};
        PhasePlanParams fprm;
        fprm.kr = bw.kr; fprm.ch = bw.ch; fprm.piece_budget = (int)bw.piece_budget; fprm.xch_bytes = 0;
        fprm.allow_resident = false;
        build_phase_plan(c, fprm, fwp);
        check_phase(c, fwp, bw, x, "forward matrix-core plan");
        const int g8 = 8;
        InverseCSR inv;
        build_inverse_csr(c, g8, inv);
        check_inverse(c, inv, g8, g, want_b);
        PhaseBudget bb{8, 8, 40 * 1024, false, 0};
        PhasePlanParams bprm = fprm;
        bprm.kr = 8; bprm.ch = 8;
        build_phase_plan(inv.view, bprm, bwp);
        check_phase(inv.view, bwp, bb, g, "backward matrix-core plan (row-inverted CSR)");
        if (fup.ok && c.Wi == c.Wo) {
            // the fused backward's gx: the fused plan of the per-basis transpose, replayed over gradient plane 0
            TransposedCSR tr;
            build_transposed_csr(c, tr);
            check_transposed(c, tr, g);
            FusedPlan fut;
            build_phase_plan(tr.view, prm, fut);
            check(fut.ok, "fused plan of the per-basis transpose not built");
            const std::vector<double> g0(g.begin(), g.begin() + (size_t)c.Ho * c.Wo);
            if (fut.ok) check_phase(tr.view, fut, bf, g0, "fused matrix-core plan of the per-basis transpose");
        }
    }

    printf("plan_check: K=%d Ho=%d Wo=%d Hi=%d Wi=%d nnz=%lld tiled fwd %s (NI=%d G=%d, %zu tasks, %d/%d split) "
           "bwd %s (NI=%d, %zu tasks, %d/%d split); matrix-core fused %s (%zu pieces), fwd %s (%zu), bwd %s (%zu)\n",
           c.K, c.Ho, c.Wo, c.Hi, c.Wi, (long long)c.nnz, tf.ok ? "on" : "off", tf.NI, tf.G, tf.tasks.size(), tf.n_ws4,
           tf.n_ws2, tb.ok ? "on" : "off", tb.NI, tb.tasks.size(), tb.n_ws4, tb.n_ws2, fup.ok ? "on" : "off",
           fup.pieces.size(), fwp.ok ? "on" : "off", fwp.pieces.size(), bwp.ok ? "on" : "off", bwp.pieces.size());
    if (g_fail) {
        fprintf(stderr, "plan_check: %d check(s) failed\n", g_fail);
        return 1;
    }
    return 0;
}
