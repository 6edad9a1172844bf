// plan_fused.cpp — packs psi into dense 16-offset blocks per (latitude, source row).
#include "plan_fused.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <cstdint>
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

void build_fused_plan(const CSRView &c, const GatherPlan & /*fwd*/, int npx, int ch, int a_budget, FusedPlan &out)
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
        // blocks of one sub-row: A operand in lane order, lane l -> row r = l % 32 (k = r % 16,
        // hi/lo part = r / 16), offsets 8 * (l / 32) + t, t < 8
        auto append_blocks = [&](int32_t sr, int32_t astart, int32_t lds_off, int32_t row_index,
                                 const std::vector<int32_t> &dblk) {
            const auto &m = rowsP[sr];
            for (int32_t d0 : dblk) {
                FBlock b;
                b.row = row_index;
                b.rel = d0 - astart;
                out.blocks.push_back(b);
                out.block_xoff.push_back(lds_off + b.rel);
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
        };
        // split each source row into blocks of 16 offsets (skipping empty ones), then into
        // sub-rows within both piece limits
        std::vector<SubRow> subs;
        for (auto &kv : rowsP) {
            const int32_t sr = kv.first;
            const auto &m = kv.second;
            const int32_t dmin = m.begin()->first, dmax = m.rbegin()->first;
            std::vector<int32_t> dblk;
            for (int32_t d0 = dmin; d0 <= dmax; d0 += kBlkJ) {
                auto it = m.lower_bound(d0);
                if (it != m.end() && it->first < d0 + kBlkJ) dblk.push_back(d0);
            }
            auto len_of = [&](size_t a, size_t b) {
                const int32_t astart = floor8(dblk[a]);
                return round_up8(dblk[b - 1] + kBlkJ - astart + npx);
            };
            size_t q = 0;
            while (q < dblk.size()) {
                size_t q1 = q + 1;
                while (q1 < dblk.size() &&
                       (int64_t)ch * len_of(q, q1 + 1) * 2 + (int64_t)(q1 + 1 - q) * 1024 <= a_budget)
                    ++q1;
                SubRow sub;
                sub.sr = sr;
                sub.astart = floor8(dblk[q]);
                sub.len = len_of(q, q1);
                sub.dblk.assign(dblk.begin() + q, dblk.begin() + q1);
                subs.push_back(std::move(sub));
                q = q1;
            }
        }
        // One piece with two window buffers when the whole latitude fits; otherwise pieces with one
        // buffer (a latitude of one such piece keeps its packed blocks resident, windows staged
        // synchronously; several pieces restage everything per channel chunk).
        int64_t tot_len = 0, tot_blk = 0;
        for (const SubRow &sb : subs) {
            tot_len += sb.len;
            tot_blk += (int64_t)sb.dblk.size();
        }
        const bool one_dbuf = 2 * (int64_t)ch * tot_len * 2 + tot_blk * 1024 <= a_budget;
        auto emit = [&](size_t s0, size_t s1, int32_t dbuf) {
            FPiece pc;
            pc.blk_begin = (int32_t)out.blocks.size();
            pc.row_begin = (int32_t)out.rows.size();
            int32_t xwin = 0, nblk = 0;
            for (size_t j = s0; j < s1; ++j) {
                const SubRow &sb = subs[j];
                FRow fr;
                fr.sr = sb.sr;
                fr.start = sb.astart;
                fr.len = sb.len;
                fr.lds_off = xwin;
                const int32_t row_index = (int32_t)out.rows.size();
                out.rows.push_back(fr);
                append_blocks(sb.sr, sb.astart, fr.lds_off, row_index, sb.dblk);
                xwin += sb.len;
                nblk += (int32_t)sb.dblk.size();
            }
            pc.blk_end = (int32_t)out.blocks.size();
            pc.row_end = (int32_t)out.rows.size();
            pc.xwin_elems = xwin;
            pc.dbuf = dbuf;
            pc.pad[0] = pc.pad[1] = 0;
            out.max_xwin = std::max(out.max_xwin, xwin);
            out.max_blk = std::max(out.max_blk, nblk);
            out.max_piece_elems = std::max(out.max_piece_elems, nblk * 512 + (1 + dbuf) * ch * xwin);
            work[ho] += nblk;
            out.pieces.push_back(pc);
        };
        if (one_dbuf) {
            emit(0, subs.size(), 1);
        } else {
            std::vector<size_t> cuts{0};
            int64_t xwin = 0, nblk = 0;
            for (size_t j = 0; j < subs.size(); ++j) {
                const int64_t cost = (int64_t)ch * (xwin + subs[j].len) * 2 + (nblk + (int64_t)subs[j].dblk.size()) * 1024;
                if (j > cuts.back() && cost > a_budget) {
                    cuts.push_back(j);
                    xwin = nblk = 0;
                }
                xwin += subs[j].len;
                nblk += (int64_t)subs[j].dblk.size();
            }
            cuts.push_back(subs.size());
            for (size_t q = 0; q + 1 < cuts.size(); ++q) emit(cuts[q], cuts[q + 1], 0);
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
