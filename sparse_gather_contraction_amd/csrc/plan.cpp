// plan.cpp — builds the forward and row-inverted (backward) gather plans.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <climits>
#include <cstdint>
#include <numeric>

namespace disco {

namespace {

enum { kOk = 0, kInvalid = 1, kShape = 2, kPsi = 4 };

struct Run {
    int32_t in_off;
    int32_t j0;
    int32_t m;
    int64_t first;  // index of the first entry in the caller's entry list
};

// Turn a list of (row key, position) entries, sorted by (key, pos) and unique,
// into runs of consecutive positions on a circle of length L.  A run that
// ends at L-1 and a run of the same key that starts at 0 are merged (the run
// then wraps).  Runs are split to at most kMaxSegLen entries.
// `key[i]` is the source-row offset, `pos[i]` the position in [0, L).
// `perm` receives entry indices in run order (so values can be gathered).
void make_runs(const std::vector<int32_t> &key, const std::vector<int32_t> &pos, int32_t L,
               std::vector<Run> &runs, std::vector<int64_t> &perm)
{
    runs.clear();
    perm.clear();
    const int64_t n = (int64_t)key.size();
    int64_t i = 0;
    while (i < n) {
        // all entries of one key
        int64_t kb = i;
        while (i < n && key[i] == key[kb]) ++i;
        int64_t ke = i;
        // maximal runs of consecutive positions within [kb, ke)
        std::vector<std::pair<int64_t, int64_t>> r;  // [begin, end) in entry index
        int64_t a = kb;
        for (int64_t j = kb + 1; j <= ke; ++j) {
            if (j == ke || pos[j] != pos[j - 1] + 1) {
                r.push_back({a, j});
                a = j;
            }
        }
        // wrap merge: last run ends at L-1, first run starts at 0, and they differ
        bool wrap = r.size() > 1 && pos[r.front().first] == 0 && pos[r.back().second - 1] == L - 1;
        std::vector<std::vector<int64_t>> merged;
        for (size_t q = 0; q < r.size(); ++q) {
            if (wrap && q == 0) continue;  // appended after the last run
            std::vector<int64_t> idx;
            for (int64_t j = r[q].first; j < r[q].second; ++j) idx.push_back(j);
            if (wrap && q + 1 == r.size())
                for (int64_t j = r.front().first; j < r.front().second; ++j) idx.push_back(j);
            merged.push_back(std::move(idx));
        }
        for (auto &idx : merged) {
            for (size_t s = 0; s < idx.size(); s += kMaxSegLen) {
                size_t e = std::min(idx.size(), s + (size_t)kMaxSegLen);
                Run run;
                run.in_off = key[idx[s]];
                run.j0 = pos[idx[s]];
                run.m = (int32_t)(e - s);
                run.first = (int64_t)perm.size();
                for (size_t t = s; t < e; ++t) perm.push_back(idx[t]);
                runs.push_back(run);
            }
        }
    }
}

void finish_order(GatherPlan &p)
{
    std::vector<int64_t> work(p.items.size());
    for (size_t i = 0; i < p.items.size(); ++i) {
        int64_t n = 0;
        for (int32_t s = p.items[i].seg_begin; s < p.items[i].seg_end; ++s) n += p.segs[s].m;
        work[i] = n * p.items[i].G + 1;
    }
    p.order.resize(p.items.size());
    std::iota(p.order.begin(), p.order.end(), 0);
    std::stable_sort(p.order.begin(), p.order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });
}

}  // namespace

std::string validate_csr(const CSRView &c, int *code)
{
    char buf[256];
    *code = kShape;
    if (c.K <= 0 || c.Ho <= 0 || c.Wo <= 0 || c.Hi <= 0 || c.Wi <= 0) return "K, Ho, Wo, Hi and Wi must all be positive";
    if (c.Wi % c.Wo != 0) {
        snprintf(buf, sizeof buf, "Wi (%d) must be an integer multiple of Wo (%d)", c.Wi, c.Wo);
        return buf;
    }
    if ((int64_t)c.K * c.Ho * c.Wo >= (int64_t)1 << 31 || (int64_t)c.Hi * c.Wi >= (int64_t)1 << 31)
        return "a (K, Ho, Wo) or (Hi, Wi) plane exceeds 2^31 elements";
    *code = kInvalid;
    if (!c.row_ptr) return "row_ptr is NULL";
    if (c.nnz > 0 && (!c.col_hi || !c.col_wi || !c.val)) return "col_hi, col_wi or val is NULL";
    *code = kPsi;
    if (c.nnz < 0 || c.nnz >= ((int64_t)1 << 31)) return "nnz must be in [0, 2^31)";
    const int64_t R = (int64_t)c.K * c.Ho;
    if (c.row_ptr[0] != 0) return "row_ptr[0] must be 0";
    for (int64_t r = 0; r < R; ++r)
        if (c.row_ptr[r + 1] < c.row_ptr[r]) {
            snprintf(buf, sizeof buf, "row_ptr decreases at row %lld", (long long)r);
            return buf;
        }
    if (c.row_ptr[R] != c.nnz) return "row_ptr[K*Ho] must equal nnz";
    for (int64_t e = 0; e < c.nnz; ++e) {
        if (c.col_hi[e] < 0 || c.col_hi[e] >= c.Hi || c.col_wi[e] < 0 || c.col_wi[e] >= c.Wi) {
            snprintf(buf, sizeof buf, "entry %lld has column (%d, %d) outside [0,%d)x[0,%d)", (long long)e,
                     c.col_hi[e], c.col_wi[e], c.Hi, c.Wi);
            return buf;
        }
    }
    // duplicate (hi, wi) within a row
    std::vector<int64_t> keys;
    for (int64_t r = 0; r < R; ++r) {
        keys.clear();
        for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) keys.push_back((int64_t)c.col_hi[e] * c.Wi + c.col_wi[e]);
        std::sort(keys.begin(), keys.end());
        if (std::adjacent_find(keys.begin(), keys.end()) != keys.end()) {
            snprintf(buf, sizeof buf, "row %lld holds a duplicate column", (long long)r);
            return buf;
        }
    }
    *code = kOk;
    return "";
}

void build_forward_plan(const CSRView &c, GatherPlan &p)
{
    const int32_t s = c.Wi / c.Wo;
    p = GatherPlan();
    p.L = c.Wo;
    p.in_stride = s;
    p.block_ptr.push_back(0);
    std::vector<int64_t> perm;
    std::vector<Run> runs;
    for (int32_t ho = 0; ho < c.Ho; ++ho) {
        // sorted entry lists of the K rows at this latitude
        std::vector<std::vector<int64_t>> ent(c.K);  // entry indices sorted by column
        for (int32_t k = 0; k < c.K; ++k) {
            const int64_t r = (int64_t)k * c.Ho + ho;
            auto &v = ent[k];
            for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) v.push_back(e);
            std::sort(v.begin(), v.end(), [&](int64_t a, int64_t b) {
                // order by (hi, rho, jj): source row first, then position
                int64_t ka = ((int64_t)c.col_hi[a] * s + c.col_wi[a] % s) * c.Wo + c.col_wi[a] / s;
                int64_t kb = ((int64_t)c.col_hi[b] * s + c.col_wi[b] % s) * c.Wo + c.col_wi[b] / s;
                return ka < kb;
            });
        }
        auto same_support = [&](int32_t a, int32_t b) {
            if (ent[a].size() != ent[b].size()) return false;
            for (size_t i = 0; i < ent[a].size(); ++i)
                if (c.col_hi[ent[a][i]] != c.col_hi[ent[b][i]] || c.col_wi[ent[a][i]] != c.col_wi[ent[b][i]]) return false;
            return true;
        };
        // groups of rows with identical column sets, in order of first appearance
        std::vector<std::vector<int32_t>> groups;
        for (int32_t k = 0; k < c.K; ++k) {
            bool placed = false;
            for (auto &g : groups)
                if (same_support(g[0], k)) { g.push_back(k); placed = true; break; }
            if (!placed) groups.push_back({k});
        }
        for (auto &grp : groups) {
            for (size_t g0 = 0; g0 < grp.size(); g0 += kMaxGroup) {
                const int32_t G = (int32_t)std::min<size_t>(kMaxGroup, grp.size() - g0);
                const auto &base = ent[grp[g0]];
                std::vector<int32_t> key(base.size()), pos(base.size());
                for (size_t i = 0; i < base.size(); ++i) {
                    const int64_t e = base[i];
                    key[i] = c.col_hi[e] * c.Wi + c.col_wi[e] % s;
                    pos[i] = c.col_wi[e] / s;
                }
                make_runs(key, pos, c.Wo, runs, perm);
                Item it;
                it.seg_begin = (int32_t)p.segs.size();
                for (const Run &rn : runs) {
                    Seg sg;
                    sg.in_off = rn.in_off;
                    sg.j0 = rn.j0;
                    sg.m = rn.m;
                    sg.val_off = (int32_t)p.vals.size();
                    for (int32_t t = 0; t < rn.m; ++t) {
                        const int64_t i = perm[rn.first + t];
                        for (int32_t g = 0; g < G; ++g) p.vals.push_back(c.val[ent[grp[g0 + g]][i]]);
                    }
                    p.segs.push_back(sg);
                }
                it.seg_end = (int32_t)p.segs.size();
                it.G = G;
                it.out_stride = 1;
                for (int32_t g = 0; g < kMaxGroup; ++g)
                    it.out_off[g] = g < G ? (grp[g0 + g] * c.Ho + ho) * c.Wo : 0;
                p.nnz_updates_per_col += (int64_t)base.size() * G;
                p.items.push_back(it);
            }
        }
        p.block_ptr.push_back((int32_t)p.items.size());
    }
    finish_order(p);
}

void build_backward_plan(const CSRView &c, GatherPlan &p)
{
    const int32_t s = c.Wi / c.Wo;
    p = GatherPlan();
    p.L = c.Wo;
    p.in_stride = 1;
    p.block_ptr.push_back(0);
    // bucket entries by (hi, rho)
    const int64_t nb = (int64_t)c.Hi * s;
    std::vector<int64_t> cnt(nb + 1, 0);
    std::vector<int32_t> kho(c.nnz);
    {
        int32_t r = 0;
        for (int64_t e = 0; e < c.nnz; ++e) {
            while (c.row_ptr[r + 1] <= e) ++r;
            kho[e] = r;  // r = k*Ho + ho
            cnt[(int64_t)c.col_hi[e] * s + c.col_wi[e] % s + 1]++;
        }
    }
    for (int64_t b = 0; b < nb; ++b) cnt[b + 1] += cnt[b];
    std::vector<int64_t> bucket(c.nnz);
    {
        std::vector<int64_t> fill(cnt.begin(), cnt.end() - 1);
        for (int64_t e = 0; e < c.nnz; ++e) bucket[fill[(int64_t)c.col_hi[e] * s + c.col_wi[e] % s]++] = e;
    }
    auto shift = [&](int64_t e) { return (c.Wo - c.col_wi[e] / s) % c.Wo; };  // u = (-jj') mod Wo
    std::vector<int64_t> perm;
    std::vector<Run> runs;
    for (int32_t hi = 0; hi < c.Hi; ++hi) {
        for (int32_t rho = 0; rho < s; ++rho) {
            const int64_t b = (int64_t)hi * s + rho;
            std::vector<int64_t> es(bucket.begin() + cnt[b], bucket.begin() + cnt[b + 1]);
            std::sort(es.begin(), es.end(), [&](int64_t a, int64_t b2) {
                if (kho[a] != kho[b2]) return kho[a] < kho[b2];
                return shift(a) < shift(b2);
            });
            std::vector<int32_t> key(es.size()), pos(es.size());
            for (size_t i = 0; i < es.size(); ++i) {
                key[i] = kho[es[i]] * c.Wo;
                pos[i] = (int32_t)shift(es[i]);
            }
            make_runs(key, pos, c.Wo, runs, perm);
            Item it;
            it.seg_begin = (int32_t)p.segs.size();
            for (const Run &rn : runs) {
                Seg sg;
                sg.in_off = rn.in_off;
                sg.j0 = rn.j0;
                sg.m = rn.m;
                sg.val_off = (int32_t)p.vals.size();
                for (int32_t t = 0; t < rn.m; ++t) p.vals.push_back(c.val[es[perm[rn.first + t]]]);
                p.segs.push_back(sg);
            }
            it.seg_end = (int32_t)p.segs.size();
            it.G = 1;
            it.out_stride = s;
            it.out_off[0] = hi * c.Wi + rho;
            for (int32_t g = 1; g < kMaxGroup; ++g) it.out_off[g] = 0;
            p.nnz_updates_per_col += (int64_t)es.size();
            p.items.push_back(it);
        }
        p.block_ptr.push_back((int32_t)p.items.size());
    }
    finish_order(p);
}

void build_staged_plan(const CSRView &c, const GatherPlan &p, bool backward, int elem_bytes, int lds_budget,
                       StagedPlan &out)
{
    out = StagedPlan();
    const int32_t s = c.Wi / c.Wo;
    const int32_t L = p.L;
    out.L = L;
    out.S = backward ? 1 : s;
    if (out.S > 2) return;
    if (L <= 192) { out.T = 3; out.wpp = 1; }
    else if (L <= 384) { out.T = 3; out.wpp = 2; }
    else if (L <= 768) { out.T = 3; out.wpp = 4; }
    else if (L <= 1536) { out.T = 6; out.wpp = 4; }
    else return;
    out.NP = 4 / out.wpp;
    out.row_len = backward ? c.Wo : c.Wi;
    out.halo = out.S * kStagedHaloPos;
    int32_t lrow = out.row_len + out.halo;
    const int32_t align = 16 / elem_bytes;
    lrow = (lrow + align - 1) / align * align;
    out.lrow = lrow;
    out.rows_per_stage = (lds_budget / out.NP) / (lrow * elem_bytes);
    if (out.rows_per_stage < 1) return;

    // Rows sharing a segment list: keep G when every item agrees, else split to single rows.
    int32_t G = p.items.empty() ? 1 : p.items[0].G;
    for (const Item &it : p.items)
        if (it.G != G) G = -1;
    const bool split_rows = (G < 0);
    if (split_rows) G = 1;
    out.G = G;
    out.NI = (backward && s <= 2) ? s : 1;

    // expanded items: (source item, row g within it or -1 for all)
    struct XItem { int32_t src; int32_t g; };
    std::vector<XItem> xitems;
    for (int32_t i = 0; i < (int32_t)p.items.size(); ++i) {
        if (split_rows)
            for (int32_t g = 0; g < p.items[i].G; ++g) xitems.push_back({i, g});
        else
            xitems.push_back({i, -1});
    }
    // tasks: NI consecutive expanded items (the backward plan lists the s residues of one input row in order)
    const int32_t NI = out.NI;
    if ((int32_t)xitems.size() % NI != 0) { out = StagedPlan(); return; }
    std::vector<Task> tasks;
    for (size_t t0 = 0; t0 < xitems.size(); t0 += NI) {
        Task task;
        task.item_begin = (int32_t)out.items.size();
        task.stage_begin = (int32_t)out.stages.size();
        int64_t work = 0;
        // items
        for (int32_t i = 0; i < NI; ++i) {
            const XItem &xi = xitems[t0 + i];
            const Item &src = p.items[xi.src];
            Item it = src;
            if (xi.g >= 0) {
                it.G = 1;
                it.out_off[0] = src.out_off[xi.g];
                for (int32_t g = 1; g < kMaxGroup; ++g) it.out_off[g] = 0;
            }
            out.items.push_back(it);
        }
        // distinct source rows of the task
        std::vector<int32_t> rows;
        for (int32_t i = 0; i < NI; ++i) {
            const Item &src = p.items[xitems[t0 + i].src];
            for (int32_t q = src.seg_begin; q < src.seg_end; ++q)
                rows.push_back(p.segs[q].in_off / out.row_len);
        }
        std::sort(rows.begin(), rows.end());
        rows.erase(std::unique(rows.begin(), rows.end()), rows.end());
        for (size_t r0 = 0; r0 < rows.size(); r0 += out.rows_per_stage) {
            const size_t r1 = std::min(rows.size(), r0 + (size_t)out.rows_per_stage);
            Stage st;
            st.row_begin = (int32_t)out.stage_rows.size();
            for (size_t r = r0; r < r1; ++r) out.stage_rows.push_back(rows[r]);
            st.row_end = (int32_t)out.stage_rows.size();
            st.segptr = (int32_t)out.stage_segptr.size();
            st.pad = 0;
            for (int32_t i = 0; i < NI; ++i) {
                out.stage_segptr.push_back((int32_t)out.segs.size());
                const XItem &xi = xitems[t0 + i];
                const Item &src = p.items[xi.src];
                for (int32_t q = src.seg_begin; q < src.seg_end; ++q) {
                    const Seg &sg = p.segs[q];
                    const int32_t row = sg.in_off / out.row_len;
                    if (row < rows[r0] || row > rows[r1 - 1]) continue;
                    const int32_t slot = (int32_t)(std::lower_bound(rows.begin() + r0, rows.begin() + r1, row) -
                                                   (rows.begin() + r0));
                    const int32_t rho = sg.in_off - row * out.row_len;
                    for (int32_t off = 0; off < sg.m; off += kStagedSegLen) {
                        Seg ns;
                        ns.in_off = slot * lrow + rho;
                        ns.j0 = (sg.j0 + off) % L;
                        ns.m = std::min(kStagedSegLen, sg.m - off);
                        ns.val_off = (int32_t)out.vals.size();
                        for (int32_t t = 0; t < ns.m; ++t) {
                            if (xi.g >= 0)
                                out.vals.push_back(p.vals[sg.val_off + (off + t) * src.G + xi.g]);
                            else
                                for (int32_t g = 0; g < src.G; ++g) out.vals.push_back(p.vals[sg.val_off + (off + t) * src.G + g]);
                        }
                        work += (int64_t)ns.m * G;
                        out.segs.push_back(ns);
                    }
                }
            }
            out.stage_segptr.push_back((int32_t)out.segs.size());
            out.stages.push_back(st);
        }
        task.stage_end = (int32_t)out.stages.size();
        task.work = (int32_t)std::min<int64_t>(work, INT32_MAX);
        tasks.push_back(task);
    }
    std::stable_sort(tasks.begin(), tasks.end(), [](const Task &a, const Task &b) { return a.work > b.work; });
    out.tasks = std::move(tasks);
    out.ok = true;
}

void build_fused_windows(const GatherPlan &p, int32_t px, FusedWindows &out)
{
    out = FusedWindows();
    const int32_t L = p.L;
    const int32_t nb = p.block_ptr.empty() ? 0 : (int32_t)p.block_ptr.size() - 1;
    out.ho_ptr.assign(1, 0);
    out.ho_len.assign(nb, 0);
    out.seg_off.assign(p.segs.size(), 0);
    for (int32_t b = 0; b < nb; ++b) {
        // segments of the block by source row
        std::vector<std::pair<int32_t, int32_t>> by_row;  // (in_off, segment)
        for (int32_t i = p.block_ptr[b]; i < p.block_ptr[b + 1]; ++i)
            for (int32_t q = p.items[i].seg_begin; q < p.items[i].seg_end; ++q) by_row.push_back({p.segs[q].in_off, q});
        std::sort(by_row.begin(), by_row.end());
        int32_t base = 0;
        for (size_t r0 = 0; r0 < by_row.size();) {
            size_t r1 = r0;
            while (r1 < by_row.size() && by_row[r1].first == by_row[r0].first) ++r1;
            // shortest arc: start at one segment's first shift, cover every segment's shifts (mod L)
            int32_t best_a = 0, best_span = INT32_MAX;
            for (size_t u = r0; u < r1; ++u) {
                const int32_t a = p.segs[by_row[u].second].j0;
                int32_t span = 0;
                for (size_t v = r0; v < r1; ++v) {
                    const Seg &sg = p.segs[by_row[v].second];
                    span = std::max(span, (sg.j0 - a + L) % L + sg.m);
                }
                if (span < best_span) {
                    best_span = span;
                    best_a = a;
                }
            }
            FWin w;
            w.in_off = by_row[r0].first;
            w.a = best_a;
            w.len = best_span + px - 1;
            w.base = base;
            for (size_t v = r0; v < r1; ++v) {
                const int32_t q = by_row[v].second;
                out.seg_off[q] = base + (p.segs[q].j0 - best_a + L) % L;
            }
            out.rows.push_back(w);
            base += w.len;
            r0 = r1;
        }
        out.ho_len[b] = base;
        out.max_len = std::max(out.max_len, base);
        out.ho_ptr.push_back((int32_t)out.rows.size());
        // the latitude's segments and values as contiguous runs (the plan appends them item by item)
        int32_t s0 = INT32_MAX, s1 = 0, v0 = INT32_MAX, v1 = 0;
        int64_t ns = 0, nv = 0;
        for (int32_t i = p.block_ptr[b]; i < p.block_ptr[b + 1]; ++i) {
            const Item &it = p.items[i];
            s0 = std::min(s0, it.seg_begin);
            s1 = std::max(s1, it.seg_end);
            ns += it.seg_end - it.seg_begin;
            for (int32_t q = it.seg_begin; q < it.seg_end; ++q) {
                v0 = std::min(v0, p.segs[q].val_off);
                v1 = std::max(v1, p.segs[q].val_off + p.segs[q].m * it.G);
                nv += (int64_t)p.segs[q].m * it.G;
            }
        }
        if (ns == 0) s0 = s1 = v0 = v1 = 0;
        if (ns != s1 - s0 || nv != (int64_t)v1 - v0) out.psi_ok = false;
        out.ho_psi.insert(out.ho_psi.end(), {s0, s1, v0, v1});
    }
}

}  // namespace disco
