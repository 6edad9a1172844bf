// plan_fused.cpp — packs psi into dense 16-offset blocks per (latitude, source row).
#include "plan_fused.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>

namespace disco {

namespace {

uint16_t bf16_rne(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

int32_t floor8(int32_t v) { return (v >= 0) ? (v / 8) * 8 : -(((-v) + 7) / 8) * 8; }
int32_t round_up8(int32_t v) { return (v + 7) / 8 * 8; }

}  // namespace

void build_fused_plan(const CSRView &c, const GatherPlan & /*fwd*/, int npx, int ch, int lds_budget, FusedPlan &out)
{
    out = FusedPlan();
    const int32_t s = c.Wi / c.Wo;
    const int32_t L = c.Wo;
    if (c.K > kFusedKMax || s > 2 || L % 8 != 0 || npx % 32 != 0) return;
    out.npx = npx;
    out.ch = ch;
    out.ho_piece.push_back(0);
    std::vector<int64_t> work(c.Ho, 0);

    for (int32_t ho = 0; ho < c.Ho; ++ho) {
        // dense psi per source row: sr -> (d -> P[k])
        std::map<int32_t, std::map<int32_t, std::vector<float>>> rowsP;
        for (int32_t k = 0; k < c.K; ++k) {
            const int64_t r = (int64_t)k * c.Ho + ho;
            for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) {
                const int32_t sr = c.col_hi[e] * s + c.col_wi[e] % s;
                const int32_t j = c.col_wi[e] / s;
                const int32_t d = (j <= L / 2) ? j : j - L;
                auto &v = rowsP[sr][d];
                if (v.empty()) v.assign(kFusedKMax, 0.0f);
                v[k] = c.val[e];
            }
        }
        struct SubRow { int32_t sr, astart, len; std::vector<int32_t> dblk; };
        std::vector<SubRow> subs;
        // split each source row into blocks of 16 offsets (skipping empty ones), then into
        // sub-rows small enough for one piece
        for (auto &kv : rowsP) {
            const int32_t sr = kv.first;
            const auto &m = kv.second;
            const int32_t dmin = m.begin()->first, dmax = m.rbegin()->first;
            std::vector<int32_t> dblk;
            for (int32_t d0 = dmin; d0 <= dmax; d0 += kBlkJ) {
                auto it = m.lower_bound(d0);
                if (it != m.end() && it->first < d0 + kBlkJ) dblk.push_back(d0);
            }
            // a sub-row must fit the budget with one channel-chunk of windows
            size_t q = 0;
            while (q < dblk.size()) {
                size_t q1 = q + 1;
                auto cost = [&](size_t a, size_t b) {
                    const int32_t astart = floor8(dblk[a]);
                    const int32_t len = round_up8(dblk[b - 1] + kBlkJ - astart + npx);
                    return (int64_t)ch * len * 2 + (int64_t)(b - a) * 1024;
                };
                while (q1 < dblk.size() && cost(q, q1 + 1) <= lds_budget) ++q1;
                SubRow sub;
                sub.sr = sr;
                sub.astart = floor8(dblk[q]);
                sub.len = round_up8(dblk[q1 - 1] + kBlkJ - sub.astart + npx);
                sub.dblk.assign(dblk.begin() + q, dblk.begin() + q1);
                subs.push_back(std::move(sub));
                q = q1;
            }
        }
        // pack sub-rows into pieces
        size_t i = 0;
        while (i < subs.size()) {
            FPiece pc;
            pc.blk_begin = (int32_t)out.blocks.size();
            pc.row_begin = (int32_t)out.rows.size();
            int32_t xwin = 0, nblk = 0;
            while (i < subs.size()) {
                const SubRow &sb = subs[i];
                const int64_t cost = (int64_t)ch * (xwin + sb.len) * 2 + (int64_t)(nblk + sb.dblk.size()) * 1024;
                if (nblk > 0 && cost > lds_budget) break;
                FRow fr;
                fr.sr = sb.sr;
                fr.start = sb.astart;
                fr.len = sb.len;
                fr.lds_off = xwin;
                const int32_t row_index = (int32_t)out.rows.size();
                out.rows.push_back(fr);
                const auto &m = rowsP[sb.sr];
                for (int32_t d0 : sb.dblk) {
                    FBlock b;
                    b.row = row_index;
                    b.rel = d0 - sb.astart;
                    out.blocks.push_back(b);
                    out.block_xoff.push_back(fr.lds_off + b.rel);
                    // A operand in lane order: lane l -> row r = l % 32 (k = r % 16, hi/lo part = r / 16),
                    // offsets 8 * (l / 32) + t, t < 8
                    for (int32_t l = 0; l < 64; ++l) {
                        const int32_t r = l % 32, k = r % 16, part = r / 16, h = l / 32;
                        for (int32_t t = 0; t < 8; ++t) {
                            const int32_t d = d0 + 8 * h + t;
                            float v = 0.0f;
                            auto it = m.find(d);
                            if (it != m.end() && k < c.K) v = it->second[k];
                            const uint16_t hi = bf16_rne(v);
                            out.adata.push_back(part == 0 ? hi : bf16_rne(v - bf16_val(hi)));
                        }
                    }
                }
                xwin += sb.len;
                nblk += (int32_t)sb.dblk.size();
                ++i;
            }
            pc.blk_end = (int32_t)out.blocks.size();
            pc.row_end = (int32_t)out.rows.size();
            pc.xwin_elems = xwin;
            pc.pad[0] = pc.pad[1] = pc.pad[2] = 0;
            out.max_xwin = std::max(out.max_xwin, xwin);
            out.max_blk = std::max(out.max_blk, nblk);
            out.max_piece_elems = std::max(out.max_piece_elems, nblk * 512 + ch * xwin);
            work[ho] += nblk;
            out.pieces.push_back(pc);
        }
        out.mfma_blocks += work[ho];
        out.ho_piece.push_back((int32_t)out.pieces.size());
    }
    out.ho_order.resize(c.Ho);
    for (int32_t h = 0; h < c.Ho; ++h) out.ho_order[h] = h;
    std::stable_sort(out.ho_order.begin(), out.ho_order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });
    out.ok = true;
}

}  // namespace disco
