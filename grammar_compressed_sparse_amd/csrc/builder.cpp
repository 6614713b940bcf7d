// Host builder: CSRV encoding -> RePair per tile -> merge -> levels ->
// pass-through completion -> level-bucketed layout.
//
// Page: "Right Multiplication on Grammar-Compressed Matrices: A Streaming,
// Memory-Bounded GPU Engine" (arXiv 2607.24971v1).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <sched.h>
#include <thread>

#include "grammar.hpp"

namespace gcs {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }
const char* last_error() { return g_err.c_str(); }

int resolve_threads(int requested)
{
    if (requested > 0) return requested;
    if (const char* e = std::getenv("OMP_NUM_THREADS")) {
        int v = std::atoi(e);
        if (v > 0) return v;
    }
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    unsigned h = std::thread::hardware_concurrency();
    return h ? (int)h : 1;
}

template <class F>
static void parallel_for(int64_t n, int threads, F&& f)
{
    threads = (int)std::min<int64_t>(threads, std::max<int64_t>(n, 1));
    if (threads <= 1) {
        for (int64_t i = 0; i < n; ++i) f(i);
        return;
    }
    std::atomic<int64_t> next{0};
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t)
        pool.emplace_back([&] {
            for (int64_t i; (i = next.fetch_add(1)) < n;) f(i);
        });
    for (auto& th : pool) th.join();
}

static double ms_since(std::chrono::steady_clock::time_point t0)
{
    return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// Phase timing of the builder on stderr when GCS_BUILD_TRACE is set.
struct PhaseTrace {
    bool on = std::getenv("GCS_BUILD_TRACE") != nullptr;
    std::chrono::steady_clock::time_point t = std::chrono::steady_clock::now();
    void mark(const char* what)
    {
        if (on) std::fprintf(stderr, "[gcs build] %-28s %9.1f ms\n", what, ms_since(t));
        t = std::chrono::steady_clock::now();
    }
};

// ---------------------------------------------------------------------------
// levels, completion, layout
// ---------------------------------------------------------------------------

// Levels by Eq. (3.1): lvl(terminal) = 0, lvl(N -> AB) = 1 + max(lvl A, lvl B).
// P(v) (plast) = the highest level among v's rule parents; C references do not
// count (a root is emitted at its own level and never carried upward,
// section 4.3).  Completion (section 4.2, Figure 3.1) gives v one shared chain
// of pass-through copies at levels lvl(v)+1 .. P(v)-1, so each completed
// level holds exactly the values alive across it.
//
// Layout of level k (section 4.3: levels contiguous, buffers alternate):
//   [ binary nodes (rules of level k) | pass-through nodes ]
// each segment ordered by the first column of the node's expansion, then by
// rule id.  A rule's expansion is a run of consecutive columns and its left
// child starts at the same column, so consecutive parents read children that
// sit close together in the level below: the gathers of a wavefront touch few
// cache lines.  (The pages keep nodes in RePair index order for the same
// purpose.)  Each pass-through node stores the arena offset of its source;
// the pass-through nodes of level k are the carried binary nodes of level k-1
// merged with the continuing pass-through nodes of level k-1, two lists that
// are already sorted by first column.
gcs_status finish_layout(Grammar& g, int threads)
{
    auto t0 = std::chrono::steady_clock::now();
    PhaseTrace tr;
    const int64_t alpha = g.alpha(), R = g.nrules();
    if (alpha + R >= (int64_t)INT32_MAX) {
        set_error("grammar exceeds the 32-bit symbol space");
        return GCS_ERANGE;
    }
    g.lvl.assign((size_t)R, 0);
    g.plast.assign((size_t)R, 0);
    std::vector<int32_t> fc((size_t)R, 0);  // first column of the expansion
    // Eq. 3.1 in blocks of consecutive rules none of which references a rule
    // of its own block (the rules of one RePair round form such a block), so
    // a block's rules are independent
    {
        std::vector<int64_t> bstart{0};
        for (int64_t i = 0, s = 0; i < R; ++i) {
            const int64_t hi = std::max<int64_t>(g.ra[i], g.rb[i]) - alpha;  // < 0: two terminals
            if (hi >= s) bstart.push_back(s = i);
        }
        bstart.push_back(R);
        auto one = [&](int64_t i) {
            const int32_t a = g.ra[i], b = g.rb[i];
            const int32_t la = a < alpha ? 0 : g.lvl[a - alpha], lb = b < alpha ? 0 : g.lvl[b - alpha];
            g.lvl[i] = 1 + std::max(la, lb);
            fc[i] = a < alpha ? g.tcol[a] : fc[a - alpha];
        };
        for (size_t x = 0; x + 1 < bstart.size(); ++x) {
            const int64_t b0 = bstart[x], b1 = bstart[x + 1];
            if (b1 - b0 < 65536) {
                for (int64_t i = b0; i < b1; ++i) one(i);
            } else {
                const int64_t nch = (b1 - b0 + 16383) / 16384;
                parallel_for(nch, threads, [&](int64_t c) {
                    for (int64_t i = b0 + c * 16384; i < std::min(b1, b0 + (c + 1) * 16384); ++i) one(i);
                });
            }
        }
    }
    // P(v): highest level of a rule parent
    const int64_t nch_r = std::max<int64_t>(1, (R + 65535) / 65536);
    std::vector<int32_t> lmax_ch((size_t)nch_r, 0);
    parallel_for(nch_r, threads, [&](int64_t c) {
        auto amax = [](int32_t* p, int32_t v) {
            int32_t cur = __atomic_load_n(p, __ATOMIC_RELAXED);
            while (cur < v && !__atomic_compare_exchange_n(p, &cur, v, true, __ATOMIC_RELAXED, __ATOMIC_RELAXED)) {
            }
        };
        int32_t m = 0;
        for (int64_t i = c * 65536; i < std::min(R, (c + 1) * 65536); ++i) {
            const int32_t l = g.lvl[i];
            m = std::max(m, l);
            if (g.ra[i] >= alpha) amax(&g.plast[g.ra[i] - alpha], l);
            if (g.rb[i] >= alpha) amax(&g.plast[g.rb[i] - alpha], l);
        }
        lmax_ch[c] = m;
    });
    int32_t L = 0;
    for (int32_t m : lmax_ch) L = std::max(L, m);
    g.L = L;
    tr.mark("levels (Eq. 3.1)");

    // rules ordered by (first column, id), then by (level, first column, id):
    // stable parallel counting sorts (16-bit digits of the column, then the level)
    const int T = std::max(1, threads);
    auto stable_sort_by = [&](const std::vector<int32_t>& in, std::vector<int32_t>& out, int64_t nbuckets,
                              auto&& key) {
        const int64_t nt = std::min<int64_t>(T, std::max<int64_t>(1, (int64_t)in.size() / 65536));
        std::vector<int64_t> off((size_t)(nt * nbuckets), 0);
        const int64_t n = (int64_t)in.size();
        parallel_for(nt, threads, [&](int64_t t) {
            int64_t* h = &off[(size_t)(t * nbuckets)];
            for (int64_t p = n * t / nt; p < n * (t + 1) / nt; ++p) h[key(in[p])]++;
        });
        int64_t run = 0;
        for (int64_t d = 0; d < nbuckets; ++d)
            for (int64_t t = 0; t < nt; ++t) {
                const int64_t c = off[(size_t)(t * nbuckets + d)];
                off[(size_t)(t * nbuckets + d)] = run;
                run += c;
            }
        out.resize(in.size());
        parallel_for(nt, threads, [&](int64_t t) {
            int64_t* h = &off[(size_t)(t * nbuckets)];
            for (int64_t p = n * t / nt; p < n * (t + 1) / nt; ++p) out[h[key(in[p])]++] = in[p];
        });
    };
    std::vector<int32_t> byfc((size_t)R), tmp;
    std::iota(byfc.begin(), byfc.end(), 0);
    int32_t fcmax = 0;
    for (int64_t i = 0; i < R; ++i) fcmax = std::max(fcmax, fc[i]);
    stable_sort_by(byfc, tmp, 65536, [&](int32_t v) { return fc[v] & 0xFFFF; });
    if (fcmax >= 65536) {
        stable_sort_by(tmp, byfc, 65536, [&](int32_t v) { return (uint32_t)fc[v] >> 16; });
    } else {
        byfc.swap(tmp);
    }
    std::vector<int32_t> order;
    stable_sort_by(byfc, order, (int64_t)L + 1, [&](int32_t v) { return g.lvl[v]; });
    std::vector<int64_t> cnt_lvl((size_t)L + 2, 0);
    for (int64_t i = 0; i < R; ++i) cnt_lvl[g.lvl[i]]++;
    std::vector<int64_t> lvl_start((size_t)L + 2, 0);
    for (int k = 1; k <= L + 1; ++k) lvl_start[k] = lvl_start[k - 1] + cnt_lvl[k - 1];
    std::vector<int32_t> pos((size_t)R, 0);  // position within own level
    parallel_for(nch_r, threads, [&](int64_t c) {
        for (int64_t p = c * 65536; p < std::min(R, (c + 1) * 65536); ++p)
            pos[order[p]] = (int32_t)(p - lvl_start[g.lvl[order[p]]]);
    });
    tr.mark("order levels by column");

    // pass-through lists: v is carried at levels lvl(v)+1 .. P(v)-1
    // (section 4.2), each level's list ordered by (first column, id); ptpos
    // holds v's position in the list of each level it is carried at
    g.lv.assign((size_t)L + 1, Level{});
    std::vector<int64_t> ptidx((size_t)R + 1, 0);  // first entry of v in ptpos
    {
        std::vector<int64_t> part((size_t)nch_r + 1, 0);
        parallel_for(nch_r, threads, [&](int64_t c) {
            int64_t s = 0;
            for (int64_t v = c * 65536; v < std::min(R, (c + 1) * 65536); ++v)
                s += std::max(0, g.plast[v] - g.lvl[v] - 1);
            part[c + 1] = s;
        });
        for (int64_t c = 0; c < nch_r; ++c) part[c + 1] += part[c];
        parallel_for(nch_r, threads, [&](int64_t c) {
            int64_t s = part[c];
            for (int64_t v = c * 65536; v < std::min(R, (c + 1) * 65536); ++v) {
                ptidx[v] = s;
                s += std::max(0, g.plast[v] - g.lvl[v] - 1);
            }
        });
        ptidx[R] = part[nch_r];
    }
    g.pt_total = ptidx[R];
    std::vector<int32_t> ptflat((size_t)g.pt_total), ptpos((size_t)g.pt_total);
    std::vector<int64_t> pt_off((size_t)L + 2, 0);
    {
        const int64_t nt = std::min<int64_t>(T, std::max<int64_t>(1, R / 65536));
        const int64_t nl = (int64_t)L + 1;
        std::vector<int64_t> cnt((size_t)(nt * nl), 0);
        parallel_for(nt, threads, [&](int64_t t) {
            int64_t* h = &cnt[(size_t)(t * nl)];
            for (int64_t p = R * t / nt; p < R * (t + 1) / nt; ++p) {
                const int32_t v = byfc[p];
                for (int k = g.lvl[v] + 1; k < g.plast[v]; ++k) h[k]++;
            }
        });
        std::vector<int64_t> npt((size_t)nl, 0);
        for (int64_t k = 0; k < nl; ++k)
            for (int64_t t = 0; t < nt; ++t) npt[k] += cnt[(size_t)(t * nl + k)];
        for (int64_t k = 0; k < nl; ++k) pt_off[k + 1] = pt_off[k] + npt[k];
        for (int64_t k = 0; k < nl; ++k) {
            int64_t run = pt_off[k];
            for (int64_t t = 0; t < nt; ++t) {
                const int64_t c = cnt[(size_t)(t * nl + k)];
                cnt[(size_t)(t * nl + k)] = run;
                run += c;
            }
        }
        parallel_for(nt, threads, [&](int64_t t) {
            int64_t* h = &cnt[(size_t)(t * nl)];
            for (int64_t p = R * t / nt; p < R * (t + 1) / nt; ++p) {
                const int32_t v = byfc[p];
                for (int k = g.lvl[v] + 1; k < g.plast[v]; ++k) {
                    const int64_t e = h[k]++;
                    ptflat[e] = v;
                    ptpos[ptidx[v] + (k - g.lvl[v] - 1)] = (int32_t)(e - pt_off[k]);
                }
            }
        });
    }
    g.wmax = 0;
    for (int k = 1; k <= L; ++k) g.wmax = std::max<int64_t>(g.wmax, cnt_lvl[k] + (pt_off[k + 1] - pt_off[k]));
    std::vector<int32_t>().swap(byfc);
    std::vector<int32_t>().swap(tmp);
    tr.mark("pass-through lists");
    auto align64 = [](int64_t v) { return (v + 63) & ~int64_t(63); };
    g.buf_a = align64(alpha);
    g.buf_b = g.buf_a + align64(g.wmax);
    g.arena = L > 0 ? g.buf_b + align64(g.wmax) : alpha;
    if (g.arena >= (int64_t)INT32_MAX) {
        set_error("value arena exceeds 2^31-1 elements");
        return GCS_ERANGE;
    }
    int64_t co = 0;
    for (int k = 1; k <= L; ++k) {
        g.lv[k].nb = cnt_lvl[k];
        g.lv[k].npt = pt_off[k + 1] - pt_off[k];
        g.lv[k].base = (k & 1) ? g.buf_a : g.buf_b;
        g.lv[k].child_off = co;
        g.lv[k].pt_off = pt_off[k];
        co += cnt_lvl[k];
    }
    // the arena offset of nonterminal w as read from level j (w alive at
    // level j: its own level or a carried copy)
    auto slot = [&](int32_t w, int j) -> int32_t {
        const Level& P = g.lv[j];
        if (g.lvl[w] == j) return (int32_t)(P.base + pos[w]);
        return (int32_t)(P.base + P.nb + ptpos[ptidx[w] + (j - g.lvl[w] - 1)]);
    };
    // Within a run of equal first column, binary nodes are ordered by the
    // arena offset of their right child and pass-through nodes by that of
    // their source, level by level upwards (so the level below is final).
    // Left children share the parent's first column, so they stay as close
    // as before; a wavefront's right children, which start where the left
    // child's expansion ends, come from fewer cache lines.
    {
        auto refine = [&](int32_t* list, int64_t n, auto&& key) {
            const int64_t nch = std::max<int64_t>(1, n / 65536);
            parallel_for(nch, threads, [&](int64_t c) {
                // this chunk's runs: those that start inside [n c / nch, n (c+1) / nch)
                auto run_start = [&](int64_t i) {
                    while (i < n && i > 0 && fc[list[i - 1]] == fc[list[i]]) ++i;
                    return i;
                };
                const int64_t s = run_start(n * c / nch), e = run_start(n * (c + 1) / nch);
                std::vector<std::pair<int64_t, int32_t>> buf;
                for (int64_t i = s; i < e;) {
                    int64_t j = i + 1;
                    while (j < e && fc[list[j]] == fc[list[i]]) ++j;
                    if (j - i > 1) {
                        buf.clear();
                        for (int64_t t = i; t < j; ++t) buf.emplace_back(key(list[t]), list[t]);
                        std::stable_sort(buf.begin(), buf.end(),
                                         [](const auto& p, const auto& q) { return p.first < q.first; });
                        for (int64_t t = i; t < j; ++t) list[t] = buf[(size_t)(t - i)].second;
                    }
                    i = j;
                }
            });
        };
        for (int k = 1; k <= L; ++k) {
            int32_t* b = order.data() + lvl_start[k];
            refine(b, cnt_lvl[k], [&](int32_t v) -> int64_t {
                const int32_t r = g.rb[v];
                return r < alpha ? r : slot(r - (int32_t)alpha, k - 1);
            });
            parallel_for(std::max<int64_t>(1, (cnt_lvl[k] + 65535) / 65536), threads, [&](int64_t c) {
                for (int64_t p = c * 65536; p < std::min(cnt_lvl[k], (c + 1) * 65536); ++p) pos[b[p]] = (int32_t)p;
            });
            const int64_t np = pt_off[k + 1] - pt_off[k];
            int32_t* pl = ptflat.data() + pt_off[k];
            refine(pl, np, [&](int32_t v) -> int64_t { return slot(v, k - 1); });
            parallel_for(std::max<int64_t>(1, (np + 65535) / 65536), threads, [&](int64_t c) {
                for (int64_t p = c * 65536; p < std::min(np, (c + 1) * 65536); ++p) {
                    const int32_t v = pl[p];
                    ptpos[ptidx[v] + (k - g.lvl[v] - 1)] = (int32_t)p;
                }
            });
        }
    }
    tr.mark("order within first-column runs");

    // column slices: weighted quantiles of the first column, every rule
    // weighted by the level slots it occupies (itself plus its chain)
    {
        const int64_t mcols = std::max<int64_t>(g.n_cols, 1);
        std::vector<double> w((size_t)mcols + 1, 0.0);
        double tot = 0;
        for (int64_t i = 0; i < R; ++i) {
            double wi = 1.0 + std::max(0, g.plast[i] - g.lvl[i] - 1);
            w[fc[i]] += wi;
            tot += wi;
        }
        for (int64_t t = 0; t < alpha; ++t) {  // bare terminals and the terminal array
            w[g.tcol[t]] += 1.0;
            tot += 1.0;
        }
        g.col_cut[0] = 0;
        double run = 0;
        int x = 1;
        for (int64_t c = 0; c < mcols && x < kSlices; ++c) {
            run += w[c];
            while (x < kSlices && run >= tot * x / kSlices) g.col_cut[x++] = (int32_t)(c + 1);
        }
        for (; x < kSlices; ++x) g.col_cut[x] = (int32_t)mcols;
        g.col_cut[kSlices] = INT32_MAX;
    }
    auto slice_of = [&](int32_t col) -> int {
        return (int)(std::upper_bound(g.col_cut + 1, g.col_cut + kSlices, col) - (g.col_cut + 1));
    };
    for (int k = 1; k <= L; ++k) {
        Level& l = g.lv[k];
        auto b = order.begin() + lvl_start[k];
        auto pb = ptflat.begin() + pt_off[k];
        for (int x = 0; x <= kSlices; ++x) {
            const int32_t cut = g.col_cut[x];
            l.bsl[x] = x == kSlices ? l.nb : std::partition_point(b, b + l.nb, [&](int32_t v) { return fc[v] < cut; }) - b;
            l.psl[x] = x == kSlices ? l.npt
                                    : std::partition_point(pb, pb + l.npt, [&](int32_t v) { return fc[v] < cut; }) - pb;
        }
    }
    for (int x = 0; x <= kSlices; ++x) {
        g.lv[0].bsl[x] = g.lv[0].psl[x] = 0;
    }

    tr.mark("column slices");
    // children and pass-through sources (slot above)
    g.child.resize((size_t)2 * R);
    g.ptsrc.resize((size_t)g.pt_total);
    parallel_for(nch_r, threads, [&](int64_t c) {
        for (int64_t v = c * 65536; v < std::min(R, (c + 1) * 65536); ++v) {
            const int k = g.lvl[v];
            const int32_t a = g.ra[v], b = g.rb[v];
            const int64_t at = 2 * (g.lv[k].child_off + pos[v]);
            g.child[at] = a < alpha ? a : slot(a - (int32_t)alpha, k - 1);
            g.child[at + 1] = b < alpha ? b : slot(b - (int32_t)alpha, k - 1);
        }
    });
    const int64_t nch_p = std::max<int64_t>(1, (g.pt_total + 65535) / 65536);
    parallel_for(nch_p, threads, [&](int64_t c) {
        const int64_t e0 = c * 65536, e1 = std::min(g.pt_total, (c + 1) * 65536);
        int k = (int)(std::upper_bound(pt_off.begin(), pt_off.end(), e0) - pt_off.begin()) - 1;
        for (int64_t e = e0; e < e1; ++e) {
            while (e >= pt_off[k + 1]) ++k;
            g.ptsrc[e] = slot(ptflat[e], k - 1);
        }
    });

    // emission groups: C-occurrences at their symbol's level (section 4.3: a
    // root is emitted the moment its level is computed), grouped by (level,
    // slice of the symbol's first column, row), rows ascending, C order within
    // a group
    tr.mark("children and sources");
    const int64_t n = g.n_rows;
    const int NB = (L + 1) * kSlices;
    // per symbol: its emission bucket (level * kSlices + slice) and the arena
    // offset of its value, so a C entry costs one lookup
    struct SymInfo {
        int32_t bucket, off;
    };
    std::vector<SymInfo> sym((size_t)(alpha + R));
    parallel_for((alpha + R + 65535) / 65536, threads, [&](int64_t b) {
        for (int64_t s = b * 65536; s < std::min(alpha + R, (b + 1) * 65536); ++s) {
            if (s < alpha) {
                sym[s] = {slice_of(g.tcol[s]), (int32_t)s};
            } else {
                const int64_t v = s - alpha;
                const int l = g.lvl[v];
                sym[s] = {l * kSlices + slice_of(fc[v]), (int32_t)(g.lv[l].base + pos[v])};
            }
        }
    });
    tr.mark("emission: symbol table");
    // row blocks processed in parallel: per block and bucket, count entries
    // and groups (a row opens a group in every bucket it touches), then fill
    // at offsets from a (bucket, block) prefix sum, so groups stay ordered by
    // (level, slice, row)
    const int64_t nblk = std::max<int64_t>(1, std::min<int64_t>((n + 4095) / 4096, 64 * (int64_t)threads));
    auto blk_rows = [&](int64_t b) { return std::make_pair(n * b / nblk, n * (b + 1) / nblk); };
    std::vector<int64_t> cnt_e((size_t)nblk * NB, 0), cnt_g((size_t)nblk * NB, 0);
    parallel_for(nblk, threads, [&](int64_t b) {
        int64_t* ce = &cnt_e[(size_t)b * NB];
        int64_t* cg = &cnt_g[(size_t)b * NB];
        std::vector<int32_t> seen_row((size_t)NB, -1);
        auto [r0, r1] = blk_rows(b);
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t e = g.c_off[r]; e < g.c_off[r + 1]; ++e) {
                const int bk = sym[g.c_sym[e]].bucket;
                ce[bk]++;
                if (seen_row[bk] != (int32_t)r) {
                    seen_row[bk] = (int32_t)r;
                    cg[bk]++;
                }
            }
    });
    tr.mark("emission: count");
    const int64_t C = (int64_t)g.c_sym.size();
    int64_t G = 0;
    for (int64_t v : cnt_g) G += v;
    if (C >= (int64_t)INT32_MAX || G >= (int64_t)INT32_MAX) {
        set_error("C exceeds the 32-bit index space");
        return GCS_ERANGE;
    }
    g.erow.assign((size_t)G, 0);
    g.eoff.assign((size_t)G + 1, 0);
    g.epos.assign((size_t)C, 0);
    if (tr.on) std::fprintf(stderr, "[gcs build] C = %lld, groups = %lld, blocks = %lld, buckets = %d\n", (long long)C,
                            (long long)G, (long long)nblk, NB);
    tr.mark("emission: allocate");
    // offsets: bucket-major, block-minor
    std::vector<int64_t> off_e((size_t)nblk * NB), off_g((size_t)nblk * NB);
    {
        int64_t go = 0, eo = 0;
        for (int l = 0; l <= L; ++l) {
            g.lv[l].grp_off = go;
            for (int x = 0; x < kSlices; ++x) {
                const int bk = l * kSlices + x;
                g.lv[l].gsl[x] = go - g.lv[l].grp_off;
                for (int64_t b = 0; b < nblk; ++b) {
                    off_g[(size_t)b * NB + bk] = go;
                    off_e[(size_t)b * NB + bk] = eo;
                    go += cnt_g[(size_t)b * NB + bk];
                    eo += cnt_e[(size_t)b * NB + bk];
                }
            }
            g.lv[l].gsl[kSlices] = go - g.lv[l].grp_off;
            g.lv[l].ngrp = go - g.lv[l].grp_off;
        }
    }
    tr.mark("emission: offsets");
    parallel_for(nblk, threads, [&](int64_t b) {
        int64_t* gf = &off_g[(size_t)b * NB];
        int64_t* ef = &off_e[(size_t)b * NB];
        std::vector<int32_t> seen_row((size_t)NB, -1);
        auto [r0, r1] = blk_rows(b);
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t e = g.c_off[r]; e < g.c_off[r + 1]; ++e) {
                const SymInfo si = sym[g.c_sym[e]];
                const int bk = si.bucket;
                if (seen_row[bk] != (int32_t)r) {
                    seen_row[bk] = (int32_t)r;
                    g.erow[gf[bk]] = (int32_t)r;
                    g.eoff[gf[bk]] = (int32_t)ef[bk];
                    gf[bk]++;
                }
                g.epos[ef[bk]++] = si.off;
            }
    });
    g.eoff[G] = (int32_t)C;
    tr.mark("emission groups");
    g.t_layer = ms_since(t0);
    return GCS_OK;
}

// ---------------------------------------------------------------------------
// CSRV + RePair
// ---------------------------------------------------------------------------

int32_t Csrv::vindex(int64_t k) const
{
    if (kind == GCS_VAL_ONES) return 0;
    if (kind == GCS_VAL_I8) return i8_index[(int)((const int8_t*)m->val)[k] + 128];
    const double x = ((const double*)m->val)[k];
    if (x == 0.0) return -1;
    return (int32_t)(std::lower_bound(V->begin(), V->end(), x) - V->begin());
}

int32_t Csrv::term_id(int64_t k) const
{
    const int32_t vi = vindex(k);
    if (vi < 0) return -1;
    const int32_t j = m->col[k];
    if (small_v) return (int32_t)(cbase[j] + __builtin_popcountll(cmask[j] & ((1ULL << vi) - 1)));
    return (int32_t)(std::lower_bound(tkeys.begin(), tkeys.end(), (int64_t)j * nV + vi) - tkeys.begin());
}

// Input checks, V and the terminal alphabet (CSRV, section 2, Eq. 2.2): the
// distinct <l, j> in use, compacted and ordered by (column, value index).
gcs_status csrv_encode(const gcs_csr_view* m, int threads, Grammar& g, Csrv& enc)
{
    if (!m || m->n_rows < 0 || m->n_cols < 0 || (m->n_rows > 0 && !m->row_ptr)) {
        set_error("invalid matrix view");
        return GCS_EINVAL;
    }
    if (m->val_kind < GCS_VAL_ONES || m->val_kind > GCS_VAL_F64 || (m->val_kind != GCS_VAL_ONES && !m->val &&
                                                                     m->n_rows > 0 && m->row_ptr[m->n_rows] > 0)) {
        set_error("invalid value kind or missing values");
        return GCS_EINVAL;
    }
    if (m->n_rows >= (int64_t)INT32_MAX || m->n_cols >= (int64_t)INT32_MAX) {
        set_error("matrix dimensions exceed 2^31-1");
        return GCS_ERANGE;
    }
    const int64_t n = m->n_rows, mc = m->n_cols;
    const int64_t nnz_stored = n > 0 ? m->row_ptr[n] : 0;
    if (n > 0 && m->row_ptr[0] != 0) {
        set_error("row_ptr[0] must be 0");
        return GCS_EINVAL;
    }
    if (nnz_stored > 0 && !m->col) {
        set_error("missing column array");
        return GCS_EINVAL;
    }
    g.n_rows = n;
    g.n_cols = mc;
    enc.m = m;
    enc.kind = m->val_kind;
    enc.V = &g.V;

    // validate rows in parallel
    std::atomic<int> bad{0};
    const int64_t vblk = 4096;
    parallel_for((n + vblk - 1) / vblk, threads, [&](int64_t b) {
        for (int64_t r = b * vblk; r < std::min(n, (b + 1) * vblk); ++r) {
            int64_t s = m->row_ptr[r], e = m->row_ptr[r + 1];
            if (e < s || e > nnz_stored) {
                bad = 1;
                return;
            }
            for (int64_t k = s; k < e; ++k) {
                int32_t c = m->col[k];
                if (c < 0 || c >= mc || (k > s && c <= m->col[k - 1])) {
                    bad = 2;
                    return;
                }
                if (m->val_kind == GCS_VAL_F64 && !std::isfinite(((const double*)m->val)[k])) {
                    bad = 3;
                    return;
                }
            }
        }
    });
    if (bad) {
        set_error(bad == 1 ? "row_ptr not monotone" : bad == 2 ? "columns must be strictly increasing and < n_cols"
                                                                : "non-finite matrix value");
        return GCS_EINVAL;
    }

    // V: distinct nonzero values, ascending (CSRV, section 2)
    const int kind = m->val_kind;
    for (int c = 0; c < 256; ++c) enc.i8_index[c] = -1;
    const int64_t nblk_v = std::max<int64_t>(1, std::min<int64_t>(threads, nnz_stored / 65536));
    if (kind == GCS_VAL_ONES) {
        if (nnz_stored > 0) g.V = {1.0};
    } else if (kind == GCS_VAL_I8) {
        std::vector<std::vector<char>> seen((size_t)nblk_v, std::vector<char>(256, 0));
        const int8_t* v = (const int8_t*)m->val;
        parallel_for(nblk_v, threads, [&](int64_t b) {
            for (int64_t k = nnz_stored * b / nblk_v; k < nnz_stored * (b + 1) / nblk_v; ++k) seen[b][(int)v[k] + 128] = 1;
        });
        for (int c = 0; c < 256; ++c) {
            bool any = false;
            for (auto& sb : seen) any = any || sb[c];
            if (any && c != 128) {
                enc.i8_index[c] = (int32_t)g.V.size();
                g.V.push_back((double)(c - 128));
            }
        }
        if (seen.size() && std::any_of(seen.begin(), seen.end(), [](const std::vector<char>& sb) { return sb[128] != 0; }))
            enc.has_zeros = true;
    } else {
        const double* v = (const double*)m->val;
        std::vector<double> vals;
        vals.reserve((size_t)nnz_stored);
        for (int64_t k = 0; k < nnz_stored; ++k) {
            if (v[k] != 0.0) vals.push_back(v[k]);
            else enc.has_zeros = true;
        }
        std::sort(vals.begin(), vals.end());
        vals.erase(std::unique(vals.begin(), vals.end()), vals.end());
        g.V = vals;
    }
    const int64_t nV = (int64_t)g.V.size();
    enc.nV = nV;

    // terminal compaction: distinct <l, j> in use, sorted by (j, l)
    enc.small_v = nV <= 64;
    if (enc.small_v) {
        enc.cmask.assign((size_t)mc, 0);
        const int64_t nblk = std::min<int64_t>(threads, std::max<int64_t>(1, n / 1024));
        std::vector<std::vector<uint64_t>> part((size_t)nblk);
        parallel_for(nblk, threads, [&](int64_t b) {
            std::vector<uint64_t>& pm = part[b];
            pm.assign((size_t)mc, 0);
            int64_t r0 = n * b / nblk, r1 = n * (b + 1) / nblk;
            for (int64_t k = (n ? m->row_ptr[r0] : 0); k < (n ? m->row_ptr[r1] : 0); ++k) {
                int32_t vi = enc.vindex(k);
                if (vi >= 0) pm[m->col[k]] |= 1ULL << vi;
            }
        });
        for (auto& pm : part)
            for (int64_t j = 0; j < mc; ++j) enc.cmask[j] |= pm[j];
        enc.cbase.assign((size_t)mc + 1, 0);
        for (int64_t j = 0; j < mc; ++j) enc.cbase[j + 1] = enc.cbase[j] + __builtin_popcountll(enc.cmask[j]);
        const int64_t alpha = enc.cbase[mc];
        if (alpha >= (int64_t)INT32_MAX) {
            set_error("too many distinct terminals");
            return GCS_ERANGE;
        }
        g.tcol.resize((size_t)alpha);
        g.tval.resize((size_t)alpha);
        for (int64_t j = 0; j < mc; ++j) {
            int64_t t = enc.cbase[j];
            for (uint64_t mk = enc.cmask[j]; mk; mk &= mk - 1) {
                g.tcol[t] = (int32_t)j;
                g.tval[t] = __builtin_ctzll(mk);
                ++t;
            }
        }
    } else {
        enc.tkeys.reserve((size_t)nnz_stored);
        for (int64_t r = 0; r < n; ++r)
            for (int64_t k = m->row_ptr[r]; k < m->row_ptr[r + 1]; ++k) {
                int32_t vi = enc.vindex(k);
                if (vi >= 0) enc.tkeys.push_back((int64_t)m->col[k] * nV + vi);
            }
        std::sort(enc.tkeys.begin(), enc.tkeys.end());
        enc.tkeys.erase(std::unique(enc.tkeys.begin(), enc.tkeys.end()), enc.tkeys.end());
        g.tcol.resize(enc.tkeys.size());
        g.tval.resize(enc.tkeys.size());
        for (size_t t = 0; t < enc.tkeys.size(); ++t) {
            g.tcol[t] = (int32_t)(enc.tkeys[t] / nV);
            g.tval[t] = (int32_t)(enc.tkeys[t] % nV);
        }
    }
    if (g.alpha() >= (int64_t)INT32_MAX) {
        set_error("too many distinct terminals");
        return GCS_ERANGE;
    }
    return GCS_OK;
}

// Tiles of a (row chunk x column chunk) partition, RePaired apart, as one
// grammar: rule ids = tile rule base + local index; row r of C = its tiles'
// sequences in column-chunk order.  where[r] = position of row r in the
// tiles' row order.
static gcs_status merge_tiles(Grammar& g, std::vector<RePairResult>& res, int64_t ncc, int64_t rc,
                              const std::vector<int32_t>& where, int threads)
{
    const int64_t ntiles = (int64_t)res.size(), n = g.n_rows, alpha = g.alpha();
    const int64_t vblk = 4096;
    std::vector<int64_t> rbase((size_t)ntiles + 1, 0);
    for (int64_t t = 0; t < ntiles; ++t) rbase[t + 1] = rbase[t] + (int64_t)res[t].rule_a.size();
    const int64_t R = rbase[ntiles];
    if (alpha + R >= (int64_t)INT32_MAX) {
        set_error("grammar exceeds the 32-bit symbol space");
        return GCS_ERANGE;
    }
    try {
        g.ra.resize((size_t)R);
        g.rb.resize((size_t)R);
        parallel_for(ntiles, threads, [&](int64_t t) {
            const int32_t shift = (int32_t)rbase[t];
            auto remap = [&](int32_t s) { return s < alpha ? s : s + shift; };
            for (size_t i = 0; i < res[t].rule_a.size(); ++i) {
                g.ra[rbase[t] + i] = remap(res[t].rule_a[i]);
                g.rb[rbase[t] + i] = remap(res[t].rule_b[i]);
            }
        });
        // C: row r = concatenation over column chunks of its tile sequences
        g.c_off.assign((size_t)n + 1, 0);
        std::vector<std::vector<int64_t>> tile_row_start((size_t)ntiles);
        for (int64_t t = 0; t < ntiles; ++t) {
            auto& s = tile_row_start[t];
            s.resize(res[t].row_len.size() + 1, 0);
            for (size_t i = 0; i < res[t].row_len.size(); ++i) s[i + 1] = s[i] + res[t].row_len[i];
        }
        for (int64_t r = 0; r < n; ++r) {
            int64_t rb = where[r] / rc, ri = where[r] - rb * rc, len = 0;
            for (int64_t cb = 0; cb < ncc; ++cb) len += res[rb * ncc + cb].row_len[ri];
            g.c_off[r + 1] = g.c_off[r] + len;
        }
        g.c_sym.resize((size_t)g.c_off[n]);
        parallel_for((n + vblk - 1) / vblk, threads, [&](int64_t b) {
            for (int64_t r = b * vblk; r < std::min(n, (b + 1) * vblk); ++r) {
                int64_t rb = where[r] / rc, ri = where[r] - rb * rc, o = g.c_off[r];
                for (int64_t cb = 0; cb < ncc; ++cb) {
                    const int64_t t = rb * ncc + cb;
                    const int32_t shift = (int32_t)rbase[t];
                    for (int64_t e = tile_row_start[t][ri]; e < tile_row_start[t][ri + 1]; ++e) {
                        int32_t s = res[t].seq[e];
                        g.c_sym[o++] = s < alpha ? s : s + shift;
                    }
                }
            }
        });
    } catch (const std::bad_alloc&) {
        set_error("out of host memory merging tiles");
        return GCS_ENOMEM;
    }
    return GCS_OK;
}

static gcs_status build_from_csr(const gcs_csr_view* m, const gcs_build_opts* opts, Grammar& g)
{
    auto t0 = std::chrono::steady_clock::now();
    const int threads = resolve_threads(opts ? opts->n_threads : 0);
    if (opts && (opts->repair < GCS_REPAIR_EXACT || opts->repair > GCS_REPAIR_ROUNDS || opts->reserved != 0)) {
        set_error("unknown RePair mode or nonzero reserved option");
        return GCS_EINVAL;
    }
    const bool rounds_mode = opts && opts->repair == GCS_REPAIR_ROUNDS;
    Csrv enc;
    if (gcs_status st = csrv_encode(m, threads, g, enc)) return st;
    const int64_t n = m->n_rows, mc = m->n_cols;
    const int64_t alpha = g.alpha();
    const int64_t vblk = 4096;
    auto term_id = [&](int64_t k) -> int32_t { return enc.term_id(k); };
    g.t_csrv = ms_since(t0);

    // tiles
    auto t1 = std::chrono::steady_clock::now();
    const int64_t cc = (opts && opts->col_chunk > 0) ? opts->col_chunk : std::max<int64_t>(mc, 1);
    const int64_t rc = (opts && opts->row_chunk > 0) ? opts->row_chunk : std::max<int64_t>(n, 1);
    const int64_t ncc = std::max<int64_t>(1, (mc + cc - 1) / cc), nrc = std::max<int64_t>(1, (n + rc - 1) / rc);
    const int64_t ntiles = ncc * nrc;
    g.n_tiles = ntiles;
    // row order of the row tiles: natural, or grouped by similarity (rows
    // ordered by two MinHash values of their column sets, so rows sharing
    // many columns -- and hence pairs -- tend to land in the same tile)
    std::vector<int32_t> perm((size_t)n), where((size_t)n);
    for (int64_t r = 0; r < n; ++r) perm[r] = (int32_t)r;
    if (opts && opts->row_order == GCS_ROWS_SIMILAR && nrc > 1) {
        std::vector<uint64_t> h1((size_t)n), h2((size_t)n);
        auto mix = [](uint64_t z) {
            z += 0x9E3779B97F4A7C15ULL;
            z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
            z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
            return z ^ (z >> 31);
        };
        parallel_for((n + vblk - 1) / vblk, threads, [&](int64_t b) {
            for (int64_t r = b * vblk; r < std::min(n, (b + 1) * vblk); ++r) {
                uint64_t a = UINT64_MAX, c = UINT64_MAX;
                for (int64_t k = m->row_ptr[r]; k < m->row_ptr[r + 1]; ++k) {
                    a = std::min(a, mix((uint64_t)m->col[k] * 2 + 1));
                    c = std::min(c, mix((uint64_t)m->col[k] * 2 + 2));
                }
                h1[r] = a;
                h2[r] = c;
            }
        });
        std::sort(perm.begin(), perm.end(), [&](int32_t u, int32_t v) {
            if (h1[u] != h1[v]) return h1[u] < h1[v];
            if (h2[u] != h2[v]) return h2[u] < h2[v];
            return u < v;
        });
    }
    for (int64_t i = 0; i < n; ++i) where[perm[i]] = (int32_t)i;
    std::vector<RePairResult> res((size_t)ntiles);
    std::atomic<int> fail{0};
    std::atomic<int64_t> nnz_total{0};
    // tiles are independent; run the larger ones first
    parallel_for(ntiles, threads, [&](int64_t t) {
        if (fail) return;
        const int64_t rb = t / ncc, cb = t % ncc;
        const int64_t r0 = rb * rc, r1 = std::min(n, r0 + rc);
        const int32_t c0 = (int32_t)(cb * cc), c1 = (int32_t)std::min<int64_t>(mc, (cb + 1) * cc);
        std::vector<int64_t> off;
        std::vector<int32_t> seq;
        try {
            off.reserve((size_t)(r1 - r0 + 1));
            off.push_back(0);
            for (int64_t i = r0; i < r1; ++i) {
                const int64_t r = perm[i];
                const int32_t* cb_ = m->col + m->row_ptr[r];
                const int32_t* ce_ = m->col + m->row_ptr[r + 1];
                const int32_t* s = (ncc == 1) ? cb_ : std::lower_bound(cb_, ce_, c0);
                const int32_t* e = (ncc == 1) ? ce_ : std::lower_bound(s, ce_, c1);
                for (const int32_t* p = s; p < e; ++p) {
                    int32_t tid = term_id(p - m->col);
                    if (tid >= 0) seq.push_back(tid);
                }
                off.push_back((int64_t)seq.size());
            }
        } catch (const std::bad_alloc&) {
            fail = 1;
            return;
        }
        if ((int64_t)seq.size() >= (int64_t)INT32_MAX) {
            fail = 2;
            return;
        }
        nnz_total += (int64_t)seq.size();
        const bool ok = rounds_mode ? repair_rounds_tile(seq, off, (int32_t)alpha, res[t])
                                    : repair_tile(seq, off, (int32_t)alpha, res[t]);
        if (!ok) fail = 1;
    });
    if (fail) {
        set_error(fail == 2 ? "a RePair tile exceeds 2^31-1 symbols (use col_chunk/row_chunk)"
                            : "out of host memory in RePair");
        return fail == 2 ? GCS_ERANGE : GCS_ENOMEM;
    }
    g.nnz = nnz_total;

    if (gcs_status st = merge_tiles(g, res, ncc, rc, where, threads)) return st;
    g.t_repair = ms_since(t1);
    return finish_layout(g, threads);
}

// The host builder fed by a row source, tile by tile (the CSR of a whole
// matrix never exists in this process).  Pass 1 fetches every tile once for
// V and the terminal alphabet (per-column masks of value indices: first-seen
// ids, renumbered once V is sorted); pass 2 fetches the tiles again in waves
// of `threads`, encodes them and runs RePair on the wave in parallel.  The
// result equals build_from_csr on the assembled matrix with the same options.
static gcs_status build_from_source(gcs_row_source src, void* ctx, int64_t n, int64_t mc, int32_t val_kind,
                                    const gcs_build_opts* opts, Grammar& g)
{
    auto t0 = std::chrono::steady_clock::now();
    if (!src || n < 0 || mc < 0 || (val_kind != GCS_VAL_ONES && val_kind != GCS_VAL_F64)) {
        set_error("invalid row source, shape or value kind (GCS_VAL_ONES or GCS_VAL_F64)");
        return GCS_EINVAL;
    }
    if (n >= (int64_t)INT32_MAX || mc >= (int64_t)INT32_MAX) {
        set_error("matrix dimensions exceed 2^31-1");
        return GCS_ERANGE;
    }
    if (opts && (opts->repair < GCS_REPAIR_EXACT || opts->repair > GCS_REPAIR_ROUNDS || opts->reserved != 0 ||
                 opts->row_order != GCS_ROWS_NATURAL)) {
        set_error("unknown RePair mode, nonzero reserved option, or a row order other than natural");
        return GCS_EINVAL;
    }
    const int threads = resolve_threads(opts ? opts->n_threads : 0);
    const bool rounds_mode = opts && opts->repair == GCS_REPAIR_ROUNDS;
    const bool ones = val_kind == GCS_VAL_ONES;
    g.n_rows = n;
    g.n_cols = mc;
    const int64_t cc = (opts && opts->col_chunk > 0) ? opts->col_chunk : std::max<int64_t>(mc, 1);
    const int64_t rc = (opts && opts->row_chunk > 0) ? opts->row_chunk : std::max<int64_t>(n, 1);
    const int64_t ncc = std::max<int64_t>(1, (mc + cc - 1) / cc), nrc = std::max<int64_t>(1, (n + rc - 1) / rc);
    const int64_t ntiles = ncc * nrc;
    g.n_tiles = ntiles;
    struct Tile {
        std::vector<int64_t> rp;
        std::vector<int32_t> col;
        std::vector<double> val;
    };
    // one tile from the source, checked like a CSR input
    auto fetch = [&](int64_t t, Tile& T) -> gcs_status {
        const int64_t r0 = (t / ncc) * rc, nr = std::min(n, r0 + rc) - r0;
        const int64_t c0 = (t % ncc) * cc, nc = std::min(mc, c0 + cc) - c0;
        const int64_t cnt = src(ctx, r0, nr, c0, nc, nullptr, nullptr, nullptr, 0);
        if (cnt < 0) {
            set_error("the row source reported a failure");
            return GCS_EINVAL;
        }
        if (cnt >= (int64_t)INT32_MAX) {
            set_error("a tile exceeds 2^31-1 nonzeros (use col_chunk/row_chunk)");
            return GCS_ERANGE;
        }
        T.rp.assign((size_t)nr + 1, 0);
        T.col.resize((size_t)cnt);
        T.val.resize(ones ? 0 : (size_t)cnt);
        const int64_t got = src(ctx, r0, nr, c0, nc, T.rp.data(), cnt ? T.col.data() : nullptr,
                                ones || !cnt ? nullptr : T.val.data(), cnt);
        if (got != cnt || T.rp[0] != 0 || T.rp[nr] != cnt) {
            set_error("the row source returned a different count than it reported, or row_ptr[0] != 0");
            return GCS_EINVAL;
        }
        for (int64_t r = 0; r < nr; ++r) {
            if (T.rp[r + 1] < T.rp[r]) {
                set_error("row_ptr not monotone in a tile from the row source");
                return GCS_EINVAL;
            }
            for (int64_t k = T.rp[r]; k < T.rp[r + 1]; ++k) {
                const int32_t c = T.col[k];
                if (c < c0 || c >= c0 + nc || (k > T.rp[r] && c <= T.col[k - 1])) {
                    set_error("columns of a source tile must be strictly increasing and inside the tile");
                    return GCS_EINVAL;
                }
                if (!ones && !std::isfinite(T.val[k])) {
                    set_error("non-finite matrix value");
                    return GCS_EINVAL;
                }
            }
        }
        return GCS_OK;
    };
    // pass 1: V (distinct nonzero values) and, while |V| <= 64, per-column
    // masks of first-seen value ids; otherwise the distinct (column, value)
    std::vector<double> seen;         // first-seen order
    std::vector<uint64_t> cm((size_t)mc, 0);
    std::vector<std::pair<int32_t, double>> keys;  // general case
    bool small = true;
    int64_t nnz = 0;
    for (int64_t t = 0; t < ntiles; ++t) {
        Tile T;
        if (gcs_status st = fetch(t, T)) return st;
        for (size_t k = 0; k < T.col.size(); ++k) {
            const double v = ones ? 1.0 : T.val[k];
            if (v == 0.0) continue;
            ++nnz;
            if (small) {
                size_t id = std::find(seen.begin(), seen.end(), v) - seen.begin();
                if (id == seen.size()) {
                    if (seen.size() == 64) {
                        // more than 64 values: keep (column, value) keys instead
                        small = false;
                        for (int64_t j = 0; j < mc; ++j)
                            for (uint64_t mk = cm[j]; mk; mk &= mk - 1) keys.push_back({(int32_t)j, seen[__builtin_ctzll(mk)]});
                        std::vector<uint64_t>().swap(cm);
                    } else {
                        seen.push_back(v);
                    }
                }
                if (small) {
                    cm[T.col[k]] |= 1ULL << id;
                    continue;
                }
            }
            keys.push_back({T.col[k], v});
        }
        if (!small && keys.size() > 1u << 24) {  // keep the key list compact
            std::sort(keys.begin(), keys.end());
            keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
        }
    }
    if (small) {
        g.V = seen;
    } else {
        std::sort(keys.begin(), keys.end());
        keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
        for (const auto& kv : keys) g.V.push_back(kv.second);
    }
    std::sort(g.V.begin(), g.V.end());
    g.V.erase(std::unique(g.V.begin(), g.V.end()), g.V.end());
    auto vidx = [&](double v) { return (int32_t)(std::lower_bound(g.V.begin(), g.V.end(), v) - g.V.begin()); };
    std::vector<int64_t> cbase;
    if (small) {
        int32_t perm[64];
        for (size_t i = 0; i < seen.size(); ++i) perm[i] = vidx(seen[i]);
        cbase.assign((size_t)mc + 1, 0);
        for (int64_t j = 0; j < mc; ++j) {
            uint64_t m2 = 0;
            for (uint64_t mk = cm[j]; mk; mk &= mk - 1) m2 |= 1ULL << perm[__builtin_ctzll(mk)];
            cm[j] = m2;
            cbase[j + 1] = cbase[j] + __builtin_popcountll(m2);
        }
        if (cbase[mc] >= (int64_t)INT32_MAX) {
            set_error("too many distinct terminals");
            return GCS_ERANGE;
        }
        g.tcol.resize((size_t)cbase[mc]);
        g.tval.resize((size_t)cbase[mc]);
        for (int64_t j = 0; j < mc; ++j) {
            int64_t t = cbase[j];
            for (uint64_t mk = cm[j]; mk; mk &= mk - 1, ++t) {
                g.tcol[t] = (int32_t)j;
                g.tval[t] = __builtin_ctzll(mk);
            }
        }
    } else {
        std::sort(keys.begin(), keys.end());
        keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
        if ((int64_t)keys.size() >= (int64_t)INT32_MAX) {
            set_error("too many distinct terminals");
            return GCS_ERANGE;
        }
        g.tcol.resize(keys.size());
        g.tval.resize(keys.size());
        for (size_t t = 0; t < keys.size(); ++t) {
            g.tcol[t] = keys[t].first;
            g.tval[t] = vidx(keys[t].second);
        }
    }
    const int64_t alpha = g.alpha();
    auto term_id = [&](int32_t j, double v) -> int32_t {
        const int32_t vi = vidx(v);
        if (small) return (int32_t)(cbase[j] + __builtin_popcountll(cm[j] & ((1ULL << vi) - 1)));
        return (int32_t)(std::lower_bound(keys.begin(), keys.end(), std::make_pair(j, v)) - keys.begin());
    };
    g.t_csrv = ms_since(t0);
    // pass 2: waves of tiles, RePair in parallel
    auto t1 = std::chrono::steady_clock::now();
    std::vector<RePairResult> res((size_t)ntiles);
    const int64_t wave = std::max(1, threads);
    std::atomic<int> fail{0};
    for (int64_t w0 = 0; w0 < ntiles; w0 += wave) {
        const int64_t w1 = std::min(ntiles, w0 + wave);
        std::vector<Tile> tiles((size_t)(w1 - w0));
        for (int64_t t = w0; t < w1; ++t)
            if (gcs_status st = fetch(t, tiles[t - w0])) return st;
        parallel_for(w1 - w0, threads, [&](int64_t i) {
            Tile& T = tiles[i];
            std::vector<int32_t> seq;
            std::vector<int64_t> off;
            try {
                seq.reserve(T.col.size());
                off.reserve(T.rp.size());
                off.push_back(0);
                for (size_t r = 0; r + 1 < T.rp.size(); ++r) {
                    for (int64_t k = T.rp[r]; k < T.rp[r + 1]; ++k) {
                        const double v = ones ? 1.0 : T.val[k];
                        if (v != 0.0) seq.push_back(term_id(T.col[k], v));
                    }
                    off.push_back((int64_t)seq.size());
                }
                std::vector<int32_t>().swap(T.col);
                std::vector<double>().swap(T.val);
                const bool ok = rounds_mode ? repair_rounds_tile(seq, off, (int32_t)alpha, res[w0 + i])
                                            : repair_tile(seq, off, (int32_t)alpha, res[w0 + i]);
                if (!ok) fail = 1;
            } catch (const std::bad_alloc&) {
                fail = 1;
            }
        });
        if (fail) {
            set_error("out of host memory in RePair");
            return GCS_ENOMEM;
        }
    }
    g.nnz = nnz;
    std::vector<int32_t> where((size_t)n);
    for (int64_t r = 0; r < n; ++r) where[r] = (int32_t)r;
    if (gcs_status st = merge_tiles(g, res, ncc, rc, where, threads)) return st;
    g.t_repair = ms_since(t1);
    return finish_layout(g, threads);
}

}  // namespace gcs

// ---------------------------------------------------------------------------
// C ABI: host builder and inspection
// ---------------------------------------------------------------------------

using gcs::Grammar;

extern "C" const char* gcs_last_error(void) { return gcs::last_error(); }

extern "C" gcs_status gcs_build_grammar(const gcs_csr_view* m, const gcs_build_opts* opts, gcs_grammar** out)
{
    if (!out) {
        gcs::set_error("null output pointer");
        return GCS_EINVAL;
    }
    *out = nullptr;
    try {
        auto* h = new gcs_grammar();
        gcs_status st = gcs::build_from_csr(m, opts, h->g);
        if (st != GCS_OK) {
            delete h;
            return st;
        }
        *out = h;
        return GCS_OK;
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of host memory");
        return GCS_ENOMEM;
    }
}

extern "C" gcs_status gcs_build_grammar_rows(gcs_row_source src, void* ctx, int64_t n_rows, int64_t n_cols,
                                             int32_t val_kind, const gcs_build_opts* opts, gcs_grammar** out)
{
    if (!out) {
        gcs::set_error("null output pointer");
        return GCS_EINVAL;
    }
    *out = nullptr;
    try {
        auto* h = new gcs_grammar();
        gcs_status st = gcs::build_from_source(src, ctx, n_rows, n_cols, val_kind, opts, h->g);
        if (st != GCS_OK) {
            delete h;
            return st;
        }
        *out = h;
        return GCS_OK;
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of host memory");
        return GCS_ENOMEM;
    }
}

extern "C" gcs_status gcs_edge_spans(const gcs_grammar* h, int64_t* hist, int64_t cap, int64_t* max_span)
{
    if (!h || cap < 0 || (cap > 0 && !hist)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    const int64_t alpha = g.alpha(), R = g.nrules();
    std::vector<int64_t> cnt((size_t)g.L + 1, 0);
    for (int64_t i = 0; i < R; ++i)
        for (int32_t c : {g.ra[i], g.rb[i]}) cnt[g.lvl[i] - (c < alpha ? 0 : g.lvl[c - alpha])]++;
    int64_t mx = 0;
    for (int64_t d = 0; d <= g.L; ++d)
        if (cnt[d]) mx = d;
    for (int64_t d = 0; d < cap; ++d) hist[d] = d <= g.L ? cnt[d] : 0;
    if (max_span) *max_span = mx;
    return GCS_OK;
}

extern "C" gcs_status gcs_expand_row(const gcs_grammar* h, int64_t r, int32_t* sym, int64_t cap, int64_t* len)
{
    if (!h || !len || cap < 0 || (cap > 0 && !sym)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    if (r < 0 || r >= g.n_rows) {
        gcs::set_error("row out of range");
        return GCS_EINVAL;
    }
    const int64_t alpha = g.alpha();
    int64_t n = 0;
    std::vector<int32_t> stack;
    for (int64_t e = g.c_off[r + 1] - 1; e >= g.c_off[r]; --e) stack.push_back(g.c_sym[e]);
    while (!stack.empty()) {  // leftmost symbol on top
        const int32_t s = stack.back();
        stack.pop_back();
        if (s < alpha) {
            if (n < cap) sym[n] = s;
            ++n;
        } else {
            stack.push_back(g.rb[s - alpha]);
            stack.push_back(g.ra[s - alpha]);
        }
    }
    *len = n;
    if (n > cap) {
        gcs::set_error("the expanded row is longer than cap");
        return GCS_ERANGE;
    }
    return GCS_OK;
}

extern "C" gcs_status gcs_grammar_from_rules(int64_t n_rows, int64_t n_cols, const double* values, int64_t n_values,
                                             const int32_t* term_col, const int32_t* term_val, int64_t n_terms,
                                             const int32_t* rule_a, const int32_t* rule_b, int64_t n_rules,
                                             const int64_t* c_off, const int32_t* c_sym, gcs_grammar** out)
{
    if (!out || n_rows < 0 || n_cols < 0 || n_values < 0 || n_terms < 0 || n_rules < 0 ||
        (n_values && !values) || (n_terms && (!term_col || !term_val)) || (n_rules && (!rule_a || !rule_b)) ||
        !c_off) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    *out = nullptr;
    if (n_terms + n_rules >= (int64_t)INT32_MAX || n_rows >= (int64_t)INT32_MAX) {
        gcs::set_error("grammar exceeds the 32-bit symbol space");
        return GCS_ERANGE;
    }
    for (int64_t t = 0; t < n_terms; ++t)
        if (term_col[t] < 0 || term_col[t] >= n_cols || term_val[t] < 0 || term_val[t] >= n_values) {
            gcs::set_error("terminal out of range");
            return GCS_EINVAL;
        }
    for (int64_t i = 0; i < n_rules; ++i)
        if (rule_a[i] < 0 || rule_b[i] < 0 || rule_a[i] >= n_terms + i || rule_b[i] >= n_terms + i) {
            gcs::set_error("rule symbol out of range or not in topological order");
            return GCS_EINVAL;
        }
    if (c_off[0] != 0) {
        gcs::set_error("c_off[0] must be 0");
        return GCS_EINVAL;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        if (c_off[r + 1] < c_off[r]) {
            gcs::set_error("c_off not monotone");
            return GCS_EINVAL;
        }
    const int64_t C = c_off[n_rows];
    if (C && !c_sym) {
        gcs::set_error("missing c_sym");
        return GCS_EINVAL;
    }
    for (int64_t e = 0; e < C; ++e)
        if (c_sym[e] < 0 || c_sym[e] >= n_terms + n_rules) {
            gcs::set_error("C symbol out of range");
            return GCS_EINVAL;
        }
    try {
        auto* h = new gcs_grammar();
        Grammar& g = h->g;
        g.n_rows = n_rows;
        g.n_cols = n_cols;
        g.V.assign(values, values + n_values);
        g.tcol.assign(term_col, term_col + n_terms);
        g.tval.assign(term_val, term_val + n_terms);
        g.ra.assign(rule_a, rule_a + n_rules);
        g.rb.assign(rule_b, rule_b + n_rules);
        g.c_off.assign(c_off, c_off + n_rows + 1);
        g.c_sym.assign(c_sym, c_sym + C);
        // nnz = total expansion length
        std::vector<int64_t> len((size_t)n_rules);
        for (int64_t i = 0; i < n_rules; ++i)
            len[i] = (rule_a[i] < n_terms ? 1 : len[rule_a[i] - n_terms]) +
                     (rule_b[i] < n_terms ? 1 : len[rule_b[i] - n_terms]);
        for (int64_t e = 0; e < C; ++e) g.nnz += c_sym[e] < n_terms ? 1 : len[c_sym[e] - n_terms];
        gcs_status st = gcs::finish_layout(g, gcs::resolve_threads(0));
        if (st != GCS_OK) {
            delete h;
            return st;
        }
        *out = h;
        return GCS_OK;
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of host memory");
        return GCS_ENOMEM;
    }
}

extern "C" gcs_status gcs_merge_grammars(const gcs_grammar* const* parts, int32_t n_parts, int32_t n_threads,
                                         gcs_grammar** out)
{
    if (!out || n_parts < 1 || !parts) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    *out = nullptr;
    for (int32_t p = 0; p < n_parts; ++p)
        if (!parts[p]) {
            gcs::set_error("null grammar among the parts");
            return GCS_EINVAL;
        }
    const Grammar& g0 = parts[0]->g;
    int64_t alpha = 0, R = 0, C = 0;
    int32_t last_col = -1;
    for (int32_t p = 0; p < n_parts; ++p) {
        const Grammar& gp = parts[p]->g;
        if (gp.n_rows != g0.n_rows || gp.n_cols != g0.n_cols) {
            gcs::set_error("parts differ in shape");
            return GCS_EINVAL;
        }
        if (!gp.tcol.empty()) {
            if (gp.tcol.front() <= last_col) {
                gcs::set_error("parts must cover disjoint, increasing column ranges");
                return GCS_EINVAL;
            }
            last_col = gp.tcol.back();
        }
        alpha += gp.alpha();
        R += gp.nrules();
        C += (int64_t)gp.c_sym.size();
    }
    if (alpha + R >= (int64_t)INT32_MAX) {
        gcs::set_error("merged grammar exceeds the 32-bit symbol space");
        return GCS_ERANGE;
    }
    try {
        auto* h = new gcs_grammar();
        Grammar& g = h->g;
        g.n_rows = g0.n_rows;
        g.n_cols = g0.n_cols;
        g.n_tiles = 0;
        // values: the sorted union of the parts' values
        for (int32_t p = 0; p < n_parts; ++p) g.V.insert(g.V.end(), parts[p]->g.V.begin(), parts[p]->g.V.end());
        std::sort(g.V.begin(), g.V.end());
        g.V.erase(std::unique(g.V.begin(), g.V.end()), g.V.end());
        g.tcol.reserve((size_t)alpha);
        g.tval.reserve((size_t)alpha);
        g.ra.reserve((size_t)R);
        g.rb.reserve((size_t)R);
        // symbol s of part p: terminal s < alpha_p -> t_off + s; rule s - alpha_p -> alpha + r_off + (s - alpha_p)
        std::vector<int64_t> t_off(n_parts), r_off(n_parts);
        int64_t to = 0, ro = 0;
        for (int32_t p = 0; p < n_parts; ++p) {
            const Grammar& gp = parts[p]->g;
            t_off[p] = to;
            r_off[p] = ro;
            to += gp.alpha();
            ro += gp.nrules();
            g.nnz += gp.nnz;
            g.n_tiles += gp.n_tiles;
            g.t_csrv += gp.t_csrv;
            g.t_repair += gp.t_repair;
        }
        auto sym = [&](int32_t p, int32_t s) -> int32_t {
            const int64_t ap = parts[p]->g.alpha();
            return (int32_t)(s < ap ? t_off[p] + s : alpha + r_off[p] + (s - ap));
        };
        for (int32_t p = 0; p < n_parts; ++p) {
            const Grammar& gp = parts[p]->g;
            for (int64_t t = 0; t < gp.alpha(); ++t) {
                g.tcol.push_back(gp.tcol[t]);
                const double v = gp.V[gp.tval[t]];
                g.tval.push_back((int32_t)(std::lower_bound(g.V.begin(), g.V.end(), v) - g.V.begin()));
            }
            for (int64_t i = 0; i < gp.nrules(); ++i) {
                g.ra.push_back(sym(p, gp.ra[i]));
                g.rb.push_back(sym(p, gp.rb[i]));
            }
        }
        // C: each row's sequences of the parts, in part (column) order
        g.c_off.assign((size_t)g.n_rows + 1, 0);
        g.c_sym.resize((size_t)C);
        int64_t o = 0;
        for (int64_t r = 0; r < g.n_rows; ++r) {
            g.c_off[r] = o;
            for (int32_t p = 0; p < n_parts; ++p) {
                const Grammar& gp = parts[p]->g;
                for (int64_t e = gp.c_off[r]; e < gp.c_off[r + 1]; ++e) g.c_sym[o++] = sym(p, gp.c_sym[e]);
            }
        }
        g.c_off[g.n_rows] = o;
        gcs_status st = gcs::finish_layout(g, gcs::resolve_threads(n_threads));
        if (st != GCS_OK) {
            delete h;
            return st;
        }
        *out = h;
        return GCS_OK;
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of host memory");
        return GCS_ENOMEM;
    }
}

extern "C" gcs_status gcs_grammar_stats(const gcs_grammar* h, gcs_stats* out)
{
    if (!h || !out) {
        gcs::set_error("null argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    out->n_rows = g.n_rows;
    out->n_cols = g.n_cols;
    out->nnz = g.nnz;
    out->n_values = (int64_t)g.V.size();
    out->n_terminals = g.alpha();
    out->n_rules = g.nrules();
    out->n_passthrough = g.pt_total;
    out->depth = g.L;
    out->max_width = g.wmax;
    out->c_len = (int64_t)g.c_sym.size();
    out->n_tiles = g.n_tiles;
    out->n_emit_groups = (int64_t)g.erow.size();
    out->t_csrv_ms = g.t_csrv;
    out->t_repair_ms = g.t_repair;
    out->t_layer_ms = g.t_layer;
    return GCS_OK;
}

extern "C" gcs_status gcs_level_widths(const gcs_grammar* h, int64_t* w, int64_t cap)
{
    if (!h || (cap > 0 && !w)) {
        gcs::set_error("null argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    for (int64_t k = 0; k <= g.L && k < cap; ++k) w[k] = k == 0 ? g.alpha() : g.lv[k].nb + g.lv[k].npt;
    return GCS_OK;
}

extern "C" gcs_status gcs_export_grammar(const gcs_grammar* h, double* values, int32_t* term_col, int32_t* term_val,
                                         int32_t* rule_a, int32_t* rule_b, int32_t* rule_level, int32_t* rule_plast,
                                         int64_t* c_off, int32_t* c_sym)
{
    if (!h) {
        gcs::set_error("null grammar");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    auto cp = [](auto* dst, const auto& v) {
        if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
    };
    cp(values, g.V);
    cp(term_col, g.tcol);
    cp(term_val, g.tval);
    cp(rule_a, g.ra);
    cp(rule_b, g.rb);
    cp(rule_level, g.lvl);
    cp(rule_plast, g.plast);
    cp(c_off, g.c_off);
    cp(c_sym, g.c_sym);
    return GCS_OK;
}

extern "C" gcs_status gcs_layout_counts(const gcs_grammar* h, int64_t* c)
{
    if (!h || !c) {
        gcs::set_error("null argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    c[0] = g.L + 1;
    c[1] = (int64_t)g.child.size() / 2;
    c[2] = (int64_t)g.ptsrc.size();
    c[3] = (int64_t)g.erow.size();
    c[4] = (int64_t)g.epos.size();
    c[5] = g.arena;
    c[6] = g.buf_a;
    c[7] = g.buf_b;
    return GCS_OK;
}

extern "C" gcs_status gcs_export_layout(const gcs_grammar* h, int64_t* level_meta, int32_t* child, int32_t* ptsrc,
                                        int32_t* erow, int32_t* eoff, int32_t* epos)
{
    if (!h) {
        gcs::set_error("null grammar");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    if (level_meta)
        for (int k = 0; k <= g.L; ++k) {
            const gcs::Level& l = g.lv[k];
            int64_t* o = level_meta + 8 * k;
            o[0] = l.nb;
            o[1] = l.npt;
            o[2] = l.child_off;
            o[3] = l.pt_off;
            o[4] = 0;
            o[5] = l.base;
            o[6] = l.grp_off;
            o[7] = l.ngrp;
        }
    auto cp = [](auto* dst, const auto& v) {
        if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
    };
    cp(child, g.child);
    cp(ptsrc, g.ptsrc);
    cp(erow, g.erow);
    cp(eoff, g.eoff);
    cp(epos, g.epos);
    return GCS_OK;
}

extern "C" gcs_status gcs_export_slices(const gcs_grammar* h, int64_t* out, int32_t* col_cut)
{
    if (!h) {
        gcs::set_error("null grammar");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    constexpr int S = gcs::kSlices + 1;
    if (out)
        for (int k = 0; k <= g.L; ++k)
            for (int x = 0; x < S; ++x) {
                out[(int64_t)k * 3 * S + x] = g.lv[k].bsl[x];
                out[(int64_t)k * 3 * S + S + x] = g.lv[k].psl[x];
                out[(int64_t)k * 3 * S + 2 * S + x] = g.lv[k].gsl[x];
            }
    if (col_cut) std::memcpy(col_cut, g.col_cut, sizeof(g.col_cut));
    return GCS_OK;
}

extern "C" void gcs_free_grammar(gcs_grammar* h) { delete h; }
