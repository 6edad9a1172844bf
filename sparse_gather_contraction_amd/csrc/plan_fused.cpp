// plan_fused.cpp — phase-split psi plan: blocks, sub-rows and pieces per output latitude.
#include "plan_fused.hpp"

#include <algorithm>
#include <cmath>
#include <cstdint>
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

// fp32 -> fp16 bits, round to nearest even (subnormals and overflow to infinity included); the
// rounding is done in double, where every step is exact.
uint16_t f16_rne(float f)
{
    const double v = (double)f;
    const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
    const double a = std::fabs(v);
    if (std::isnan(v)) return (uint16_t)(sign | 0x7e00u);
    if (a < std::ldexp(1.0, -14)) {  // subnormal range: multiples of 2^-24
        const double q = std::nearbyint(a * std::ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)q);  // q = 1024 is the smallest normal
    }
    int e = 0;
    const double m = std::frexp(a, &e);  // a = m 2^e, m in [0.5, 1)
    double q = std::nearbyint(m * 2048.0);  // 11 significant bits
    if (q == 2048.0) { q = 1024.0; ++e; }
    const int ef = e - 1 + 15;  // biased exponent of 1.f x 2^(e-1)
    if (ef >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(ef << 10) | (uint16_t)(q - 1024.0));
}

int32_t floor8(int32_t v) { return (v >= 0) ? (v / 8) * 8 : -(((-v) + 7) / 8) * 8; }

struct SubRow {
    int32_t hi;                // input latitude (the source row)
    std::vector<int32_t> t0;   // kept block starts, ascending (multiples of 8, step 16)
    int32_t first() const { return t0.front(); }
};

}  // namespace

void build_phase_plan(const CSRView &c, const PhasePlanParams &prm, FusedPlan &out)
{
    out = FusedPlan();
    const int32_t s = c.Wi / c.Wo;
    const int32_t kr = prm.kr, ch = prm.ch;
    if (c.K > kr || (kr != 8 && kr != 16) || s < 1 || s > 2 || c.Wo % 8 != 0 || c.Wi % 8 != 0) return;
    out.ch = ch;
    out.kr = kr;
    out.s = s;
    out.ho_piece.push_back(0);
    {
        float vmax = 0.0f;
        for (int64_t e = 0; e < c.nnz; ++e) vmax = std::max(vmax, std::fabs(c.val[e]));
        int ex = 0;
        if (vmax > 0.0f && std::isfinite(vmax)) std::frexp((double)vmax, &ex);  // vmax in [2^(ex-1), 2^ex)
        out.psi16_exp = vmax > 0.0f ? 15 - ex : 0;
    }
    const double psi16_scale = std::ldexp(1.0, out.psi16_exp);
    std::vector<int64_t> work(c.Ho, 0);
    const int32_t smax = 7 * s;                            // largest phase shift of psi
    // psi e-rows of a sub-row (even): a lane reads four words (two copies) or five (one copy, the
    // fifth realigns an odd shift) from pair (base + 8 hh - s q) / 2
    int32_t tail = 16;
    auto ra_of = [&](const SubRow &sb) { return sb.t0.back() - sb.first() + 8 * s + tail; };
    // window positions; with s = 2 rows are whole pairs of 8-element units (the kernels split the area
    // by unit parity, and a row then starts at an even unit)
    auto len_of = [&](const SubRow &sb) { return sb.t0.back() - sb.first() + 256 * s + (s == 2 ? 16 : 8); };
    auto cost_of = [&](int64_t nblk, int64_t a_elems, int64_t win) {
        return fused_piece_bytes(2 * nblk, a_elems, ch, win);
    };
    // resident layout of a whole latitude (rows uncut): descriptors, psi and two window buffers
    auto resident_bytes = [&](const std::vector<SubRow> &whole, int32_t copies) {
        int64_t nb = 0, ae = 0, we = 0;
        for (const SubRow &sb : whole) {
            nb += (int64_t)sb.t0.size();
            ae += (int64_t)copies * kr * ra_of(sb);
            we += len_of(sb);
        }
        if (nb & 1) { ++nb; ae += (int64_t)copies * kr * (8 * s + tail); }
        const int64_t wbuf = std::max<int64_t>(2 * (int64_t)ch * we, prm.xch_bytes);
        return 4 * 2 * nb + 2 * ae + 2 * wbuf;
    };

    for (int32_t ho = 0; ho < c.Ho; ++ho) {
        // dense psi per input latitude: hi -> (t -> P[k]), t = signed input-column offset
        std::map<int32_t, std::map<int32_t, std::vector<float>>> rowsP;
        for (int32_t k = 0; k < c.K; ++k) {
            const int64_t r = (int64_t)k * c.Ho + ho;
            for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) {
                const int32_t wi = c.col_wi[e];
                const int32_t t = (wi <= c.Wi / 2) ? wi : wi - c.Wi;
                auto &v = rowsP[c.col_hi[e]][t];
                if (v.empty()) v.assign(kr, 0.0f);
                v[k] = c.val[e];
            }
        }
        // blocks per source row (skipping blocks that see no entry at any phase)
        std::vector<SubRow> whole;
        for (auto &kv : rowsP) {
            const auto &m = kv.second;
            const int32_t tmin = m.begin()->first, tmax = m.rbegin()->first;
            const int32_t T0 = floor8(tmin);
            SubRow sr;
            sr.hi = kv.first;
            for (int32_t t0 = T0; t0 == T0 || t0 - 1 - smax < tmax; t0 += kBlkJ) {
                auto it = m.lower_bound(t0 - smax);
                if (it != m.end() && it->first <= t0 + kBlkJ - 1) sr.t0.push_back(t0);
            }
            if (!sr.t0.empty()) whole.push_back(sr);
        }
        // psi copies: odd phase shifts (s odd) read a second copy whose offset pairs start one offset
        // later, or realign five words of the one copy.  Resident when the whole latitude (rows uncut)
        // keeps its descriptors and psi in LDS next to two window buffers; otherwise rows are cut into
        // sub-rows that fit a streamed stage.
        int32_t copies = 1;
        bool resident = false;
        const int64_t res_budget = 2 * (int64_t)prm.piece_budget;
        if ((s & 1) && prm.psi_copies == 2) {
            copies = 2;
        } else if ((s & 1) && prm.psi_copies == 3 && prm.allow_resident && !whole.empty()) {
            tail = 16;
            if (resident_bytes(whole, 2) <= res_budget) copies = 2;
        }
        const bool realign = (s & 1) && copies == 1;
        tail = realign ? 18 : 16;
        if (prm.allow_resident && !whole.empty()) resident = resident_bytes(whole, copies) <= res_budget;
        std::vector<SubRow> subs;
        if (resident) {
            subs = whole;
        } else {
            for (const SubRow &sr : whole) {
                SubRow cur;
                cur.hi = sr.hi;
                for (int32_t t0 : sr.t0) {
                    SubRow trial = cur;
                    trial.t0.push_back(t0);
                    // room for the zero block a piece with an odd block count gets, so that a piece of
                    // one sub-row (never cut further) stays within the budget
                    if (!cur.t0.empty() && cost_of((int64_t)trial.t0.size() + 1,
                                                   (int64_t)copies * kr * (ra_of(trial) + 8 * s + tail),
                                                   len_of(trial)) > prm.piece_budget) {
                        subs.push_back(cur);
                        cur.t0.clear();
                    }
                    cur.t0.push_back(t0);
                }
                if (!cur.t0.empty()) subs.push_back(cur);
            }
        }
        // group sub-rows into pieces
        size_t q = 0;
        while (q < subs.size()) {
            size_t q1 = q;
            int64_t nb = 0, ae = 0, we = 0;
            while (q1 < subs.size()) {
                const int64_t nb2 = nb + (int64_t)subs[q1].t0.size();
                const int64_t ae2 = ae + (int64_t)copies * kr * ra_of(subs[q1]);
                const int64_t we2 = we + len_of(subs[q1]);
                if (!resident && q1 > q && cost_of(nb2 + 1, ae2 + (int64_t)copies * kr * (8 * s + tail), we2) > prm.piece_budget)
                    break;
                nb = nb2; ae = ae2; we = we2;
                ++q1;
            }
            const bool pad = (nb & 1) != 0;  // blocks are contracted in pairs: pad with a zero block
            FPiece pc;
            pc.desc_begin = (int32_t)(out.descs.size() / 2);
            pc.nblk = (int32_t)(nb + (pad ? 1 : 0));
            pc.desc_words = 2 * pc.nblk;
            pc.a_begin = (int32_t)out.adata.size();
            pc.a_elems = (int32_t)(ae + (pad ? copies * kr * (8 * s + tail) : 0));
            pc.row_begin = (int32_t)out.rows.size();
            pc.win_elems = (int32_t)we;
            int32_t a_row_e = 0, win_off = 0;
            std::vector<uint16_t> copy1;  // second psi copy of the piece (s odd)
            std::vector<uint16_t> copy1_16;
            auto put_pairs = [&](std::vector<uint16_t> &dst, std::vector<uint16_t> &dst16,
                                 const std::map<int32_t, std::vector<float>> &m, int32_t e_base, int32_t ra,
                                 int32_t shift) {
                // [e pair][k][2]: word m holds offsets e_base + shift + 2m and + 1 (relative to first - 8 s)
                for (int32_t e2 = 0; e2 < ra; e2 += 2) {
                    auto it0 = m.find(e_base + shift + e2), it1 = m.find(e_base + shift + e2 + 1);
                    for (int32_t k = 0; k < kr; ++k) {
                        const float v0 = (it0 != m.end() && k < c.K) ? it0->second[k] : 0.0f;
                        const float v1 = (it1 != m.end() && k < c.K) ? it1->second[k] : 0.0f;
                        dst.push_back(bf16_rne(v0));
                        dst.push_back(bf16_rne(v1));
                        dst16.push_back(f16_rne((float)(v0 * psi16_scale)));
                        dst16.push_back(f16_rne((float)(v1 * psi16_scale)));
                    }
                }
            };
            for (size_t j = q; j < q1; ++j) {
                const SubRow &sb = subs[j];
                const int32_t first = sb.first(), ra = ra_of(sb);
                const auto &m = rowsP[sb.hi];
                FRow fr;
                fr.sr = sb.hi;
                fr.start = first;
                fr.len = len_of(sb);
                fr.win_off = win_off;
                out.rows.push_back(fr);
                for (int32_t t0 : sb.t0) {
                    out.descs.push_back(2 * kr * (a_row_e + (t0 - first) + 8 * s));
                    // window run: bytes into a channel's area; with s = 2 bytes into one parity half
                    // (unit u of the area at 16 (u / 2): the run's first unit is even)
                    out.descs.push_back((s == 2 ? 1 : 2) * (win_off + (t0 - first)));
                }
                put_pairs(out.adata, out.adata16, m, first - 8 * s, ra, 0);
                if (copies == 2) put_pairs(copy1, copy1_16, m, first - 8 * s, ra, 1);
                a_row_e += ra;
                win_off += fr.len;
            }
            if (pad) {  // zero psi rows; the window offset reads the piece's first window
                out.descs.push_back(2 * kr * (a_row_e + 8 * s));
                out.descs.push_back(0);
                out.adata.insert(out.adata.end(), (size_t)kr * (8 * s + tail), (uint16_t)0);
                out.adata16.insert(out.adata16.end(), (size_t)kr * (8 * s + tail), (uint16_t)0);
                if (copies == 2) {
                    copy1.insert(copy1.end(), (size_t)kr * (8 * s + tail), (uint16_t)0);
                    copy1_16.insert(copy1_16.end(), (size_t)kr * (8 * s + tail), (uint16_t)0);
                }
            }
            out.adata.insert(out.adata.end(), copy1.begin(), copy1.end());
            out.adata16.insert(out.adata16.end(), copy1_16.begin(), copy1_16.end());
            pc.row_end = (int32_t)out.rows.size();
            pc.resident = 0;
            pc.a_copy_bytes = copies == 2 ? pc.a_elems : 0;  // byte offset of the second copy = half the psi bytes
            pc.realign = realign ? 1 : 0;
            pc.pad = 0;
            const int64_t stage_bytes = 4 * (int64_t)pc.desc_words + 2 * (int64_t)pc.a_elems;
            const int64_t wbuf = std::max<int64_t>(2 * (int64_t)ch * pc.win_elems, prm.xch_bytes);
            if (resident) {
                pc.resident = (int32_t)wbuf;
                out.max_resident_bytes = std::max<int32_t>(out.max_resident_bytes, (int32_t)(stage_bytes + 2 * wbuf));
            } else {
                out.max_piece_bytes = std::max<int32_t>(
                    out.max_piece_bytes, (int32_t)fused_piece_bytes(pc.desc_words, pc.a_elems, ch, pc.win_elems));
            }
            out.pieces.push_back(pc);
            out.max_win = std::max(out.max_win, pc.win_elems);
            work[ho] += pc.nblk + 8;  // per-piece stage overhead counted as a few blocks
            out.mfma_blocks += pc.nblk;
            q = q1;
        }
        out.ho_piece.push_back((int32_t)out.pieces.size());
    }
    if (out.adata.size() * 2 >= ((size_t)1 << 31) || out.descs.size() * 4 >= ((size_t)1 << 31)) {
        out = FusedPlan();  // beyond 32-bit buffer offsets
        return;
    }
    out.ho_order.resize(c.Ho);
    for (int32_t h = 0; h < c.Ho; ++h) out.ho_order[h] = h;
    std::stable_sort(out.ho_order.begin(), out.ho_order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });
    out.ok = true;
}

void build_inverse_csr(const CSRView &c, int g, InverseCSR &out)
{
    const int32_t s = c.Wi / c.Wo;
    const int32_t rows = c.Hi * s;
    const int32_t groups = (rows + g - 1) / g;
    const int64_t nrow = (int64_t)g * groups;
    out.row_ptr.assign(nrow + 1, 0);
    auto target = [&](int64_t e) {
        const int32_t wi = c.col_wi[e], rho = wi % s, r = c.col_hi[e] * s + rho;
        return (int64_t)(r % g) * groups + r / g;
    };
    for (int64_t e = 0; e < c.nnz; ++e) ++out.row_ptr[target(e) + 1];
    for (int64_t r = 0; r < nrow; ++r) out.row_ptr[r + 1] += out.row_ptr[r];
    out.col_hi.resize(c.nnz);
    out.col_wi.resize(c.nnz);
    out.val.resize(c.nnz);
    std::vector<int64_t> fill(out.row_ptr.begin(), out.row_ptr.end() - 1);
    for (int32_t k = 0; k < c.K; ++k)
        for (int32_t ho = 0; ho < c.Ho; ++ho) {
            const int64_t r = (int64_t)k * c.Ho + ho;
            for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) {
                const int32_t wi = c.col_wi[e], rho = wi % s;
                const int64_t dst = fill[target(e)]++;
                out.col_hi[dst] = k * c.Ho + ho;
                out.col_wi[dst] = (c.Wo - (wi - rho) / s) % c.Wo;
                out.val[dst] = c.val[e];
            }
        }
    out.view = CSRView();
    out.view.K = g;
    out.view.Ho = groups;
    out.view.Wo = c.Wo;
    out.view.Hi = c.K * c.Ho;
    out.view.Wi = c.Wo;
    out.view.nnz = c.nnz;
    out.view.row_ptr = out.row_ptr.data();
    out.view.col_hi = out.col_hi.data();
    out.view.col_wi = out.col_wi.data();
    out.view.val = out.val.data();
}

void build_transposed_csr(const CSRView &c, TransposedCSR &out)
{
    const int64_t nrow = (int64_t)c.K * c.Hi;
    out.row_ptr.assign(nrow + 1, 0);
    for (int32_t k = 0; k < c.K; ++k)
        for (int64_t e = c.row_ptr[(int64_t)k * c.Ho]; e < c.row_ptr[(int64_t)(k + 1) * c.Ho]; ++e)
            ++out.row_ptr[(int64_t)k * c.Hi + c.col_hi[e] + 1];
    for (int64_t r = 0; r < nrow; ++r) out.row_ptr[r + 1] += out.row_ptr[r];
    out.col_hi.resize(c.nnz);
    out.col_wi.resize(c.nnz);
    out.val.resize(c.nnz);
    std::vector<int64_t> fill(out.row_ptr.begin(), out.row_ptr.end() - 1);
    for (int32_t k = 0; k < c.K; ++k)
        for (int32_t ho = 0; ho < c.Ho; ++ho) {
            const int64_t r = (int64_t)k * c.Ho + ho;
            for (int64_t e = c.row_ptr[r]; e < c.row_ptr[r + 1]; ++e) {
                const int64_t dst = fill[(int64_t)k * c.Hi + c.col_hi[e]]++;
                out.col_hi[dst] = ho;
                out.col_wi[dst] = (c.Wo - c.col_wi[e]) % c.Wo;
                out.val[dst] = c.val[e];
            }
        }
    out.view = CSRView();
    out.view.K = c.K;
    out.view.Ho = c.Hi;
    out.view.Wo = c.Wo;
    out.view.Hi = c.Ho;
    out.view.Wi = c.Wo;
    out.view.nnz = c.nnz;
    out.view.row_ptr = out.row_ptr.data();
    out.view.col_hi = out.col_hi.data();
    out.view.col_wi = out.col_wi.data();
    out.view.val = out.val.data();
}

}  // namespace disco
