// plan_tile.cpp — builds the register-tiled fp32 gather plan (see plan_tile.hpp).
#include "plan_tile.hpp"

#include <algorithm>
#include <climits>

namespace disco {

namespace {

// (NI, G) pairs the kernel is instantiated for
bool ni_supported(int NI, int G)
{
    if (G == 1) return NI == 1 || NI == 2 || NI == 4 || NI == 8;
    if (G == 2) return NI == 1 || NI == 2 || NI == 4;
    return (G == 3 || G == 4) && (NI == 1 || NI == 2);
}

}  // namespace

void build_tile_plan(const CSRView &c, const GatherPlan &p, bool backward, int lds_budget, TilePlan &out)
{
    out = TilePlan();
    const int32_t s = c.Wi / c.Wo;
    const int32_t L = p.L;
    if (L <= 0 || L > kTileMaxL) return;
    if (!backward && s > 2) return;
    out.L = L;
    out.deint = backward ? 1 : s;
    out.row_len = backward ? c.Wo : c.Wi;
    out.PW = (L <= 32 * kTileT) ? 2 : 1;
    out.NP = 4 * out.PW;
    out.lrow = (L + kTileHalo + 3) / 4 * 4;
    const int64_t row_bytes = (int64_t)out.NP * out.deint * out.lrow * 4;
    int32_t rps = (int32_t)std::min<int64_t>(kTileMaxStageRows, lds_budget / row_bytes);
    if (rps < 1) return;

    // rows per item: keep G when every item agrees, else split every item into single rows
    int32_t G = p.items.empty() ? 1 : p.items[0].G;
    for (const Item &it : p.items)
        if (it.G != G) G = -1;
    const bool split = G < 0;
    if (split) G = 1;
    out.G = G;

    struct XItem { int32_t src, g; };  // source item, its row g (or -1: all rows)
    const int32_t nblocks = (int32_t)p.block_ptr.size() - 1;
    std::vector<std::vector<XItem>> per_block(nblocks);
    int32_t n_max = 0;
    for (int32_t b = 0; b < nblocks; ++b) {
        for (int32_t i = p.block_ptr[b]; i < p.block_ptr[b + 1]; ++i) {
            if (split)
                for (int32_t g = 0; g < p.items[i].G; ++g) per_block[b].push_back({i, g});
            else
                per_block[b].push_back({i, -1});
        }
        n_max = std::max<int32_t>(n_max, (int32_t)per_block[b].size());
    }
    const int32_t cap = kTileMaxRows / G;
    int32_t NI = 0;
    for (int32_t n = 1; n <= cap; ++n)
        if (ni_supported(n, G) && (NI == 0 || NI < n_max)) NI = n;
    if (NI == 0) return;
    out.NI = NI;
    const int32_t cmax = tile_piece_max(G);

    std::vector<Task> tasks;
    // stages of rps source rows; fewer rows when the largest stage's records do not fit beside them
    for (;; --rps) {
    if (rps < 1) { out = TilePlan(); return; }
    out.rows_per_stage = rps;
    out.items.clear(); out.stages.clear(); out.stage_rows.clear(); out.stage_recptr.clear(); out.recs.clear();
    tasks.clear();
    for (int32_t b = 0; b < nblocks; ++b) {
        const auto &xs = per_block[b];
        for (size_t t0 = 0; t0 < xs.size(); t0 += NI) {
            Task task;
            task.item_begin = (int32_t)out.items.size();
            task.stage_begin = (int32_t)out.stages.size();
            int64_t work = 0;
            std::vector<int32_t> rows;
            for (int32_t i = 0; i < NI; ++i) {
                Item it;
                if (t0 + i < xs.size()) {
                    const XItem &xi = xs[t0 + i];
                    const Item &src = p.items[xi.src];
                    it = src;
                    if (xi.g >= 0) {
                        it.G = 1;
                        it.out_off[0] = src.out_off[xi.g];
                        for (int32_t g = 1; g < kMaxGroup; ++g) it.out_off[g] = 0;
                    }
                    for (int32_t q = src.seg_begin; q < src.seg_end; ++q) rows.push_back(p.segs[q].in_off / out.row_len);
                } else {
                    it = Item();
                    it.seg_begin = it.seg_end = 0;
                    it.G = G;
                    it.out_stride = 0;
                    for (int32_t g = 0; g < kMaxGroup; ++g) it.out_off[g] = -1;
                }
                out.items.push_back(it);
            }
            std::sort(rows.begin(), rows.end());
            rows.erase(std::unique(rows.begin(), rows.end()), rows.end());
            for (size_t r0 = 0; r0 < rows.size(); r0 += out.rows_per_stage) {
                const size_t r1 = std::min(rows.size(), r0 + (size_t)out.rows_per_stage);
                Stage st;
                st.row_begin = (int32_t)out.stage_rows.size();
                for (size_t r = r0; r < r1; ++r) out.stage_rows.push_back(rows[r]);
                st.row_end = (int32_t)out.stage_rows.size();
                st.segptr = (int32_t)out.stage_recptr.size();
                st.pad = 0;
                for (int32_t i = 0; i < NI; ++i) {
                    std::vector<TileRec> by_c[kTileClasses];
                    if (t0 + i < xs.size()) {
                        const XItem &xi = xs[t0 + i];
                        const Item &src = p.items[xi.src];
                        for (int32_t q = src.seg_begin; q < src.seg_end; ++q) {
                            const Seg &sg = p.segs[q];
                            const int32_t row = sg.in_off / out.row_len;
                            const int32_t rho = sg.in_off - row * out.row_len;
                            if (row < rows[r0] || row > rows[r1 - 1]) continue;
                            const int32_t slot = (int32_t)(std::lower_bound(rows.begin() + r0, rows.begin() + r1, row) -
                                                           (rows.begin() + r0));
                            for (int32_t off = 0; off < sg.m; off += cmax) {
                                TileRec rec = {};
                                rec.j0 = (sg.j0 + off) % L;
                                rec.a = 4 * ((slot * out.deint + rho) * out.lrow + rec.j0);
                                rec.w = L - rec.j0;
                                const int32_t c = std::min(cmax, sg.m - off);
                                rec.c = c;
                                for (int32_t e = 0; e < c; ++e) {
                                    if (xi.g >= 0) {
                                        rec.v[e] = p.vals[sg.val_off + (off + e) * src.G + xi.g];
                                    } else {
                                        for (int32_t g = 0; g < G; ++g)
                                            rec.v[e * G + g] = p.vals[sg.val_off + (off + e) * src.G + g];
                                    }
                                }
                                work += (int64_t)c * G;
                                by_c[c - 1].push_back(rec);
                            }
                        }
                    }
                    for (int32_t cl = 0; cl < kTileClasses; ++cl) {
                        out.stage_recptr.push_back((int32_t)out.recs.size());
                        out.recs.insert(out.recs.end(), by_c[cl].begin(), by_c[cl].end());
                    }
                }
                out.stage_recptr.push_back((int32_t)out.recs.size());
                out.stages.push_back(st);
            }
            task.stage_end = (int32_t)out.stages.size();
            task.work = (int32_t)std::min<int64_t>(work, INT32_MAX);
            tasks.push_back(task);
        }
    }
    int32_t max_recs = 0;
    for (const Stage &st : out.stages)
        max_recs = std::max(max_recs, out.stage_recptr[st.segptr + NI * kTileClasses] - out.stage_recptr[st.segptr]);
    out.max_recs = max_recs;
    if (row_bytes * rps + (int64_t)sizeof(TileRec) * max_recs <= lds_budget) break;
    }
    std::stable_sort(tasks.begin(), tasks.end(), [](const Task &a, const Task &b) { return a.work > b.work; });
    // record split: a task more than twice the mean work spreads over 2 waves, more than four times
    // over 4, so that no single wave carries a polar latitude alone
    int64_t total = 0;
    for (const Task &t : tasks) total += t.work;
    const double mean = tasks.empty() ? 0.0 : (double)total / (double)tasks.size();
    out.n_ws4 = out.n_ws2 = 0;
    for (const Task &t : tasks) {
        if (t.work > 4.0 * mean) ++out.n_ws4;
        if (t.work > 2.0 * mean) ++out.n_ws2;
    }
    out.tasks = std::move(tasks);
    out.task_first.clear();
    for (const Task &t : out.tasks)
        out.task_first.push_back(t.stage_begin < t.stage_end ? out.stages[t.stage_begin]
                                                             : (out.stages.empty() ? Stage{0, 0, 0, 0} : out.stages[0]));
    out.ok = true;
}

void tile_wave_split(int32_t n_tasks, int64_t n_recs, int32_t PW, int32_t plan_ws4, int32_t plan_ws2, int64_t BC,
                     int32_t &n_ws4, int32_t &n_ws2)
{
    n_ws4 = plan_ws4;
    n_ws2 = plan_ws2;
    if (n_recs < (int64_t)kTileSplitMinRecs * n_tasks) return;
    if (BC <= 2 * (int64_t)PW) {
        n_ws4 = n_ws2 = n_tasks;
    } else if (BC < 4 * (int64_t)PW) {
        n_ws2 = n_tasks;
    }
}

}  // namespace disco
