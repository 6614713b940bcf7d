// Host side of the device engine for y = M x on MI355X: the device handle,
// upload of the grammar image (and the narrow levels' LDS image), the launch
// sequence of a sweep, the batched and BFS drivers and the C ABI of gcs.h.
// The kernels are in kernels.hpp.
//
// Device memory (all owned by the caller):
//   grammar image  child pairs | pass-through sources | emission groups
//                  (erow, eoff, epos) | emission chunks | terminal
//                  descriptors | V | launch table | narrow levels' LDS image
//   workspace      counters (256 B) | value arena [T (alpha) | buffer A |
//                  buffer B] | slice accumulators
//   batch workspace (batched sweeps only, per call)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <utility>
#include <vector>

#include "grammar.hpp"
#include "kernels.hpp"
#include "staging.hpp"

// ------------------------------------------------------------ device handle

struct gcs_device {
    gcs_policy policy;
    int device;
    int64_t n_rows, n_cols, alpha, L;
    int64_t arena_len = 0;  // values in the arena (terminals and both level buffers)
    std::vector<gcs::Level> lv;
    std::vector<int32_t> team_log2;  // per level: lanes per emission group
    const int2* child;
    const int32_t* ptsrc;
    const int32_t *erow, *eoff, *epos, *tcol, *tval;
    const void* V;
    void* arena;
    void* acc;  // kSlices x n_rows row accumulators
    unsigned long long* counters;  // [0], [1]: BFS counts
    unsigned* barrier;             // tail grid barrier counter
    int* err;                      // set by the tail kernel if its barrier timed out
    std::vector<gcs::LevelArgs> largs;  // launch k = 1..L+1 at index k-1
    const int32_t* chunk = nullptr;     // stream emission chunks of every level (grammar image)
    bool l0_on = false;                 // level 0's emission groups cut by sub-slice
    int64_t grp_skip = 0;               // groups not uploaded at the start of erow / eoff (level 0's when cut)
    int32_t l0_sub = 1;                 // into this many sub-slices per slice
    bool win_on = false;                // Boolean level-0 emission by window_emit_kernel (words, no groups)
    int64_t win_words = 0;
    gcs::WinArgs win{};
    int32_t win_grid = 0;
    size_t win_lds = 0;
    const int32_t *l0row = nullptr, *l0off = nullptr;  // its groups then (rows, root offsets)
    std::vector<int64_t> chunk_off;     // per level: first entry of its chunks
    std::vector<std::array<int32_t, gcs::kSlices + 1>> chunk_sl;  // per level: chunks of each slice
    int64_t tail_k0 = 1, tail_nent = 0;  // levels tail_k0..L and the last emission run in the tail kernel
    int64_t tail_multi = 0;              // of which the first tail_multi run on the whole tail grid
    int32_t tail_wgs = 0;
    bool tail_coop = false;              // the tail as a cooperative launch (GCS_TAIL_COOP=1 at upload)
    unsigned spin_limit = 1u << 25;      // polls before a tail barrier gives up (GCS_TAIL_SPIN_LIMIT at upload)
    int64_t grid_max = 0;  // cap on workgroups of a wide level launch (multiple of kSlices)
    const gcs::LevelArgs* tail_table = nullptr;
    gcs::FlatArgs flat{};      // the narrowest tail launches, run in LDS by one workgroup
    size_t flat_lds = 0;       // dynamic LDS bytes of the tail launch
    size_t flat_budget = 0;    // LDS budget of that phase on this device (the same for every handle)
    bool flat_attr = false;    // the tail kernel's dynamic LDS limit has been raised to flat_budget
    int64_t* pinned;
    // profiling
    std::vector<hipEvent_t> events;
    int64_t prof_max = 0, prof_used = 0;
    bool profiling = false;
    int32_t prof_mode = GCS_PROFILE_LAUNCHES;
};

namespace gcs {
namespace {

size_t elem_bytes(gcs_policy p)
{
    switch (p) {
    case GCS_PLUS_F64: return 8;
    case GCS_PLUS_F32: return 4;
    case GCS_PLUS_F32_ACC_F64: return 8;
    case GCS_BOOL_OR: return 1;
    case GCS_PLUS_I64: return 8;
    case GCS_MIN_PLUS_F32: return 4;
    case GCS_MIN_PLUS_F64: return 8;
    }
    return 0;
}
// the policy's emission goes straight into y (no slice accumulators)
bool direct_emit(gcs_policy p)
{
    switch (p) {
    case GCS_PLUS_F64: return kDirectEmit<PolPlusF64>;
    case GCS_PLUS_F32: return kDirectEmit<PolPlusF32>;
    case GCS_PLUS_F32_ACC_F64: return kDirectEmit<PolPlusF32AccF64>;
    case GCS_BOOL_OR: return kDirectEmit<PolBoolOr>;
    case GCS_PLUS_I64: return kDirectEmit<PolPlusI64>;
    case GCS_MIN_PLUS_F32: return kDirectEmit<PolMinPlusF32>;
    case GCS_MIN_PLUS_F64: return kDirectEmit<PolMinPlusF64>;
    }
    return false;
}
size_t x_bytes(gcs_policy p) { return p == GCS_PLUS_F32 || p == GCS_PLUS_F32_ACC_F64 ? 4 : elem_bytes(p); }
size_t y_bytes(gcs_policy p) { return elem_bytes(p); }
size_t v_bytes(gcs_policy p) { return elem_bytes(p); }

inline size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct Image {
    size_t child, ptsrc, erow, eoff, epos, chunk, l0row, l0off, wchunk, wword, tcol, tval, V, table, flat, total;
};

// roots emitted at level k (the same whether or not level 0's groups are cut)
inline int64_t level_roots(const Grammar& g, int64_t k)
{
    const Level& l = g.lv[k];
    return l.ngrp > 0 ? g.eoff[l.grp_off + l.ngrp] - g.eoff[l.grp_off] : 0;
}

// ------------------------------------------------ level-0 emission by sub-slice
//
// The emission of level 0 gathers bare terminals: for a large terminal array
// each slice's share of T (alpha * value bytes / 8) exceeds the 4 MB L2 of
// its XCD, and a slice's groups, taken in row order, gather from all of it.
// For the direct policies (whose emission may write a row more than once)
// the upload cuts every level-0 group further by column sub-slice, S equal
// parts of the slice's terminal range, and orders a slice's new groups by
// (sub-slice, row): the workgroups of an XCD then gather from one window of
// about kLevel0Window bytes at a time.  The permuted roots take the place of
// level 0's roots in the uploaded root list; the new rows and offsets are
// their own image section (the grammar's own level-0 groups stay unused).
// Measured on MI355X, tropical fp32 on the 5e7-node copy graph (25 MB of T
// per slice): the launch emitting level 0 takes 14.0 ms uncut, 6.95 / 6.68 /
// 6.50 ms cut into 8 / 13 / 24 sub-slices when few x[j] are finite, and
// 9.8 / 10.1 / 11.0 ms into 4 / 8 / 10 when all are (every group then ends
// in an atomic, and more sub-slices mean more groups); a 3 MB window is the
// compromise.
constexpr double kLevel0Window = 3.0 * 1024 * 1024;
constexpr double kWinTarget = 26.0 * 1024;  // Boolean LDS window target (window_emit_kernel)
constexpr int32_t kLevel0MaxSplit = 64;

// first terminal of each column slice (terminals are sorted by column)
std::array<int64_t, kSlices + 1> slice_terms(const Grammar& g)
{
    std::array<int64_t, kSlices + 1> t0{};
    for (int x = 0; x <= kSlices; ++x)
        t0[x] = x == kSlices ? g.alpha()
                             : std::lower_bound(g.tcol.begin(), g.tcol.end(), g.col_cut[x]) - g.tcol.begin();
    return t0;
}

inline int32_t sub_of(int64_t t, int x, const std::array<int64_t, kSlices + 1>& t0, int32_t S)
{
    const int64_t n = t0[x + 1] - t0[x];
    const int64_t sub = n > 0 ? (t - t0[x]) * S / n : 0;
    return (int32_t)std::max<int64_t>(0, std::min<int64_t>(S - 1, sub));
}

// How level 0's emission is organized on upload (direct policies only).
// By default as a word stream (window_emit_kernel): cut into S sub-slices
// per slice so that every sub-slice's terminals fit one LDS window of
// kWinBytes (Boolean terminals are bits, so S is small: 47 for the 5e7
// terminals of the copy graph, whose fp32 values take 646).  Where no S up to
// kLevel0MaxWindowSplit fits, or with GCS_LEVEL0_WINDOW=0, the level kernel
// emits level 0's groups, cut into S sub-slices when a slice's share of T
// exceeds kLevel0Window.  GCS_LEVEL0_SPLIT=S forces a count (0: no cut).
struct Level0Plan {
    bool cut = false;     // level 0's groups are cut by sub-slice
    int32_t S = 1;        // sub-slices per slice
    bool window = false;  // level-0 emission as words from LDS windows
};

constexpr int32_t kLevel0MaxWindowSplit = 4096;

Level0Plan level0_plan(const Grammar& g, gcs_policy p)
{
    Level0Plan pl;
    if (!direct_emit(p) || g.lv.empty() || g.lv[0].ngrp == 0) return pl;
    const char* ew = std::getenv("GCS_LEVEL0_WINDOW");
    const bool allow = !(ew && std::atoi(ew) == 0);
    // the largest slice's share of T (slices are weighted quantiles of the
    // first column, so their terminal counts differ)
    const bool bits = p == GCS_BOOL_OR;
    const int64_t eb = (int64_t)elem_bytes(p);
    const auto t0 = slice_terms(g);
    int64_t widest = 0;
    for (int x = 0; x < kSlices; ++x) widest = std::max(widest, t0[x + 1] - t0[x]);
    const double per_slice = (double)widest * (bits ? 0.125 : (double)eb);
    // a window holds a chunk's terminals, which lie in one sub-slice of at
    // most ceil(widest / S) terminals, plus the 16-byte alignment of both ends
    auto fits = [&](int64_t S) {
        const int64_t span = (widest + S - 1) / S;
        return (bits ? (span + 7) / 8 : span * eb) + 32 <= kWinBytes;
    };
    if (const char* e = std::getenv("GCS_LEVEL0_SPLIT")) {
        pl.S = std::max(0, std::min(kLevel0MaxSplit, std::atoi(e)));
        pl.cut = pl.S >= 1;
        pl.S = std::max(1, pl.S);
        pl.window = allow && pl.cut && fits(pl.S);
        return pl;
    }
    if (allow) {
        // Boolean: windows of about kWinTarget bytes (smaller windows
        // measured faster with the earlier, group-based window kernel on the
        // copy graph: its level 0 in 2.24 ms at 59 KB, 2.10 ms at 39 KB,
        // 2.02 ms at 26 KB); values: the fewest sub-slices that fit
        const double target = bits ? kWinTarget : (double)(kWinBytes - 64);
        const int64_t S = std::max<int64_t>(1, (int64_t)std::ceil(per_slice / target));
        if (S <= kLevel0MaxWindowSplit && fits(S)) {
            pl.S = (int32_t)S;
            pl.cut = pl.window = true;
            return pl;
        }
    }
    pl.S = (int32_t)std::max(1.0, std::min((double)kLevel0MaxSplit, std::ceil(per_slice / kLevel0Window)));
    pl.cut = pl.S > 1;
    return pl;
}

// For each slice x, calls fn(x) on a thread of its own.
template <class Fn>
void per_slice(Fn fn)
{
    std::vector<std::thread> th;
    for (int x = 0; x < kSlices; ++x) th.emplace_back(fn, x);
    for (auto& t : th) t.join();
}

// Level-0 groups after the cut (one per run of equal sub-slice inside a
// group), and how many skip words the word stream would need without chunk
// boundaries (an upper bound: a chunk restarts its rows): a gap of d rows
// between consecutive roots of one sub-slice takes (d - 1) / kWordMaxDelta.
struct Level0Counts {
    int64_t groups = 0, skips = 0;
};

Level0Counts level0_counts(const Grammar& g, int32_t S)
{
    const Level& l = g.lv[0];
    const auto t0 = slice_terms(g);
    std::array<int64_t, kSlices> n{}, sk{};
    per_slice([&](int x) {
        int64_t c = 0, k = 0;
        std::vector<int32_t> last((size_t)S, -1);
        for (int64_t gi = l.gsl[x]; gi < l.gsl[x + 1]; ++gi) {
            const int32_t r = g.erow[l.grp_off + gi];
            int32_t prev = -1;
            for (int64_t e = g.eoff[l.grp_off + gi]; e < g.eoff[l.grp_off + gi + 1]; ++e) {
                const int32_t s = sub_of(g.epos[e], x, t0, S);
                if (s != prev) {
                    ++c;
                    if (last[s] >= 0 && r > last[s]) k += (r - last[s] - 1) / kWordMaxDelta;
                    last[s] = r;
                }
                prev = s;
            }
        }
        n[x] = c;
        sk[x] = k;
    });
    Level0Counts out;
    for (int x = 0; x < kSlices; ++x) {
        out.groups += n[x];
        out.skips += sk[x];
    }
    return out;
}

struct Level0Split {
    bool on = false;
    int32_t S = 1;
    std::vector<int32_t> row, off;  // per new group: its row; root offsets (ngrp + 1 entries)
    std::vector<int32_t> pos;       // level 0's roots in the new order (root list positions [0, pos.size()))
    int64_t gsl[kSlices + 1] = {};  // new groups of each slice
    std::vector<int64_t> sgs;       // first new group of (slice x, sub-slice s) at x * S + s; kSlices * S + 1 entries
};

// The cut itself: per slice, runs counted per sub-slice, then placed
// sub-slice major, each sub-slice's runs in the grammar's group (row) order.
void level0_split(const Grammar& g, int32_t S, Level0Split& out)
{
    const Level& l = g.lv[0];
    const auto t0 = slice_terms(g);
    const int64_t r0 = g.eoff[l.grp_off], r1 = g.eoff[l.grp_off + l.ngrp];
    out.on = true;
    out.S = S;
    out.sgs.assign((size_t)kSlices * S + 1, 0);
    std::array<std::vector<int64_t>, kSlices> ng, nr;
    per_slice([&](int x) {
        ng[x].assign(S, 0);
        nr[x].assign(S, 0);
        for (int64_t gi = l.gsl[x]; gi < l.gsl[x + 1]; ++gi) {
            int32_t prev = -1;
            for (int64_t e = g.eoff[l.grp_off + gi]; e < g.eoff[l.grp_off + gi + 1]; ++e) {
                const int32_t s = sub_of(g.epos[e], x, t0, S);
                ng[x][s] += s != prev;
                nr[x][s] += 1;
                prev = s;
            }
        }
    });
    std::array<int64_t, kSlices + 1> gbase{};
    for (int x = 0; x < kSlices; ++x) {
        int64_t c = 0;
        for (int64_t v : ng[x]) c += v;
        gbase[x + 1] = gbase[x] + c;
    }
    for (int x = 0; x <= kSlices; ++x) out.gsl[x] = gbase[x];
    out.row.assign((size_t)gbase[kSlices], 0);
    out.off.assign((size_t)gbase[kSlices] + 1, 0);
    out.pos.assign((size_t)(r1 - r0), 0);
    out.off[gbase[kSlices]] = (int32_t)r1;
    out.sgs[(size_t)kSlices * S] = gbase[kSlices];
    per_slice([&](int x) {
        std::vector<int64_t> gs(S), rs(S);
        int64_t gacc = gbase[x], racc = g.eoff[l.grp_off + l.gsl[x]];
        for (int32_t s = 0; s < S; ++s) {
            gs[s] = gacc;
            rs[s] = racc;
            out.sgs[(size_t)x * S + s] = gacc;
            gacc += ng[x][s];
            racc += nr[x][s];
        }
        for (int64_t gi = l.gsl[x]; gi < l.gsl[x + 1]; ++gi) {
            const int64_t e0 = g.eoff[l.grp_off + gi], e1 = g.eoff[l.grp_off + gi + 1];
            int64_t e = e0;
            while (e < e1) {
                const int32_t s = sub_of(g.epos[e], x, t0, S);
                const int64_t gn = gs[s]++;
                out.row[gn] = g.erow[l.grp_off + gi];
                out.off[gn] = (int32_t)rs[s];
                do {
                    out.pos[rs[s]++ - r0] = g.epos[e++];
                } while (e < e1 && sub_of(g.epos[e], x, t0, S) == s);
            }
        }
    });
}

// The word stream of a Boolean level 0 after its cut (see
// window_emit_kernel): per slice and sub-slice, the roots in the cut's
// (row) order, in chunks of at most window_chunk_entries roots, each chunk
// with the 16-byte aligned range of T bytes its roots' bits lie in and the
// row of its first root.  About an 8192th of the roots per chunk: many
// chunks per workgroup slot of the device (balance), each still loading its
// window once.  Two int4 per chunk.
int64_t window_chunk_entries(int64_t roots)
{
    const int64_t ce = std::max<int64_t>((int64_t)kWinBlock * kWinWords, roots / 8192);
    return (ce + kWinWords - 1) / kWinWords * kWinWords;
}
size_t window_chunk_bound(int64_t roots, int32_t S)
{
    return (size_t)(roots / window_chunk_entries(roots) + (int64_t)kSlices * S + 1);
}
// the roots, the skip words (bounded by level0_counts) and every chunk's
// padding
size_t window_word_bound(int64_t roots, int32_t S, int64_t skips)
{
    return (size_t)(roots + skips + (int64_t)kWinWords * (int64_t)window_chunk_bound(roots, S));
}

// eb: bytes per terminal value, 0 for bits.  False (with the error set) if
// a window exceeds kWinBytes or rows decrease inside a sub-slice.
bool build_window_words(const Level0Split& l0, int64_t n_rows, int64_t eb, std::vector<uint32_t>& words,
                        std::vector<int4>& wch)
{
    const int32_t S = l0.S;
    const int64_t ce = window_chunk_entries((int64_t)l0.pos.size());
    std::array<std::vector<uint32_t>, kSlices> pw;
    std::array<std::vector<int4>, kSlices> pc;
    std::array<int, kSlices> ok{};
    per_slice([&](int x) {  // each slice on a thread of its own
        std::vector<uint32_t>& W = pw[x];
        std::vector<int4>& Ch = pc[x];
        ok[x] = 1;
        for (int32_t s = 0; s < S && ok[x]; ++s) {
            const int64_t g0 = l0.sgs[(size_t)x * S + s], g1 = l0.sgs[(size_t)x * S + s + 1];
            if (g0 == g1) continue;
            int64_t gi = g0;
            const int64_t r_end = l0.off[g1];
            for (int64_t e = l0.off[g0]; e < r_end && ok[x];) {
                const int64_t ee = std::min<int64_t>(r_end, e + ce);
                int64_t tmin = INT64_MAX, tmax = -1;
                for (int64_t q = e; q < ee; ++q) {
                    tmin = std::min<int64_t>(tmin, l0.pos[q]);
                    tmax = std::max<int64_t>(tmax, l0.pos[q]);
                }
                const int64_t b0 = eb ? (tmin * eb) & ~int64_t(15) : (tmin >> 3) & ~int64_t(15);
                const int64_t b1 = eb ? ((tmax + 1) * eb + 15) & ~int64_t(15) : ((tmax >> 3) + 16) & ~int64_t(15);
                const int64_t term0 = eb ? b0 / eb : b0 * 8;  // the window's first terminal
                if (b1 - b0 > kWinBytes || term0 > INT32_MAX) {
                    ok[x] = 0;
                    break;
                }
                while (l0.off[gi + 1] <= e) ++gi;
                const int32_t row0 = l0.row[gi];
                const size_t w0 = W.size();
                int32_t prev = row0;
                for (int64_t q = e; q < ee; ++q) {
                    while (l0.off[gi + 1] <= q) ++gi;
                    const int32_t r = l0.row[gi];
                    if (r < prev || r >= n_rows) {
                        ok[x] = -1;
                        break;
                    }
                    int64_t d = r - prev;
                    for (; d > kWordMaxDelta; d -= kWordMaxDelta)
                        W.push_back(((uint32_t)kWordMaxDelta << kWordPosBits) | kWordSkip);
                    W.push_back(((uint32_t)d << kWordPosBits) | (uint32_t)(l0.pos[q] - term0));
                    prev = r;
                }
                while (W.size() % kWinWords) W.push_back(kWordSkip);
                Ch.push_back(make_int4((int32_t)w0, (int32_t)W.size(), (int32_t)b0, (int32_t)b1));
                Ch.push_back(make_int4(row0, (int32_t)term0, 0, 0));
                e = ee;
            }
        }
    });
    words.clear();
    wch.clear();
    for (int x = 0; x < kSlices; ++x) {
        if (ok[x] != 1) {
            set_error(ok[x] == 0 ? "internal error: a level-0 window exceeds the LDS budget"
                                 : "level-0 emission rows are not in ascending order within a slice");
            return false;
        }
        if (words.size() + pw[x].size() >= (size_t)INT32_MAX) {
            set_error("level-0 word stream exceeds the 32-bit index space");
            return false;
        }
        const int32_t base = (int32_t)words.size();
        words.insert(words.end(), pw[x].begin(), pw[x].end());
        for (size_t i = 0; i < pc[x].size(); i += 2) {
            int4 c = pc[x][i];
            c.x += base;
            c.y += base;
            wch.push_back(c);
            wch.push_back(pc[x][i + 1]);
        }
    }
    return true;
}

// Stream emission chunks (see stream_block): per level and slice, runs of
// consecutive groups with at most kStreamCap roots (a longer group alone)
// and at most kStreamCap groups; an entry is the level-relative index of a
// chunk's first group.  Every chunk but a slice's last was closed either by
// the group limit or because it and the next chunk hold more than kStreamCap
// roots together, which bounds the count by chunk_bound.
size_t chunk_bound(const Grammar& g, int64_t g0_split)
{
    // g0_split: level 0's group count after a sub-slice cut (the larger count bounds both)
    const size_t G = g.erow.size() - (size_t)g.lv[0].ngrp + (size_t)std::max<int64_t>(g0_split, g.lv[0].ngrp);
    const size_t C = g.epos.size(), K = kStreamCap;
    return (G + K - 1) / K + 2 * ((C + K - 1) / K) + (size_t)kSlices * (g.L + 1) + 1;
}

// none0: level 0 has no groups on the device (its Boolean words instead)
void build_chunks(const Grammar& g, const Level0Split* l0, bool none0, std::vector<int32_t>& chunk,
                  std::vector<int64_t>& off, std::vector<std::array<int32_t, kSlices + 1>>& sl)
{
    chunk.clear();
    off.assign((size_t)g.L + 1, 0);
    sl.assign((size_t)g.L + 1, {});
    for (int64_t k = 0; k <= g.L; ++k) {
        const Level& l = g.lv[k];
        // level 0 after a sub-slice cut: its own groups and root offsets
        const bool cut = k == 0 && l0 && l0->on;
        const int32_t* eo = cut ? l0->off.data() : g.eoff.data() + l.grp_off;
        const int64_t* gsl = cut ? l0->gsl : l.gsl;
        off[k] = (int64_t)chunk.size();
        if (k == 0 && none0) continue;
        for (int x = 0; x < kSlices; ++x) {
            sl[k][x] = (int32_t)((int64_t)chunk.size() - off[k]);
            int64_t gi = gsl[x];
            while (gi < gsl[x + 1]) {
                chunk.push_back((int32_t)gi);
                int64_t roots = 0, cnt = 0;
                while (gi < gsl[x + 1] && cnt < kStreamCap) {
                    const int64_t len = eo[gi + 1] - eo[gi];
                    if (cnt > 0 && roots + len > kStreamCap) break;
                    roots += len;
                    ++cnt;
                    ++gi;
                }
            }
        }
        sl[k][kSlices] = (int32_t)((int64_t)chunk.size() - off[k]);
    }
}

inline size_t al16(size_t v) { return (v + 15) & ~size_t(15); }

// Upper bound on the narrow launches' image (32-bit words, all of it loaded
// into LDS): at most kFlatLdsMax bytes, and no more than a table entry and a
// group offset per launch, every staged slot (at most the terminals and the
// arena), three fold words per emission group and the grammar's own indices
// as 16-bit slots.
size_t flat_section_words(const Grammar& g)
{
    const size_t G = g.erow.size(), C = g.epos.size();
    const size_t bound = (size_t)kFlatEntryWords * (g.L + 2) + G + g.L + 2 + (size_t)g.arena + 3 * G + 1 +
                         (g.child.size() + g.ptsrc.size() + 1) / 2 + (C + 1) / 2 + 8;
    return std::min(kFlatLdsMax / 4, bound);
}

Image image_layout(const Grammar& g, gcs_policy p)
{
    const Level0Plan pl = level0_plan(g, p);
    const Level0Counts lc = pl.cut ? level0_counts(g, pl.S) : Level0Counts{};
    const int64_t g0 = lc.groups;
    // level 0's roots; with windows the device holds their words instead of
    // their groups and root positions, and the root list starts at level 1's
    const int64_t r0 = g.lv.empty() || g.lv[0].ngrp == 0 ? 0 : g.eoff[g.lv[0].grp_off + g.lv[0].ngrp];
    const size_t rskip = pl.window ? (size_t)r0 : 0;
    Image m{};
    size_t o = 0;
    m.child = o;
    o = al256(o + g.child.size() * 4);
    m.ptsrc = o;
    o = al256(o + g.ptsrc.size() * 4);
    // when level 0's groups are cut, the grammar's own level-0 groups are not
    // uploaded: the sections start at level 1's first group
    const size_t skip = pl.cut ? (size_t)g.lv[0].ngrp : 0;
    m.erow = o;
    o = al256(o + (g.erow.size() - skip) * 4);
    m.eoff = o;
    o = al256(o + (g.eoff.size() - skip) * 4);
    m.epos = o;
    o = al256(o + (g.epos.size() - rskip) * 4);
    m.chunk = o;
    o = al256(o + chunk_bound(g, g0) * 4);
    const bool groups0 = pl.cut && !pl.window;  // level 0's cut groups on the device
    m.l0row = o;
    o = al256(o + (groups0 ? (size_t)g0 * 4 : 0));
    m.l0off = o;
    o = al256(o + (groups0 ? (size_t)(g0 + 1) * 4 : 0));
    m.wchunk = o;
    o = al256(o + (pl.window ? 2 * window_chunk_bound(r0, pl.S) * sizeof(int4) : 0));
    m.wword = o;
    o = al256(o + (pl.window ? window_word_bound(r0, pl.S, lc.skips) * 4 : 0));
    m.tcol = o;
    o = al256(o + g.tcol.size() * 4);
    m.tval = o;
    o = al256(o + g.tval.size() * 4);
    m.V = o;
    o = al256(o + g.V.size() * v_bytes(p));
    m.table = o;
    o = al256(o + (size_t)(g.L + 1) * sizeof(LevelArgs));
    m.flat = o;
    o = al256(o + 4 * flat_section_words(g));
    m.total = o;
    return m;
}

size_t arena_bytes(const Grammar& g, gcs_policy p) { return al256((size_t)g.arena * elem_bytes(p)); }
size_t acc_bytes(const Grammar& g, gcs_policy p) { return al256((size_t)kSlices * g.n_rows * elem_bytes(p)); }
size_t workspace_bytes(const Grammar& g, gcs_policy p) { return arena_bytes(g, p) + acc_bytes(g, p) + 256; }

bool valid_policy(int p) { return p >= GCS_PLUS_F64 && p <= GCS_MIN_PLUS_F64; }

// batch workspace: [arena x B | kSlices x n_rows x B accumulators]
size_t batch_arena_bytes(int64_t arena, gcs_policy p, int64_t B) { return al256((size_t)(arena * B) * elem_bytes(p)); }
// rows of the batch arena: all of it, or without the terminal array when the
// leaves are evaluated in the sweep
int64_t batch_arena_rows(const gcs_device* d, int32_t flags)
{
    return (flags & GCS_BATCH_LEAVES_IN_SWEEP) ? d->arena_len - d->alpha : d->arena_len;
}
size_t batch_workspace_bytes(int64_t arena_rows, int64_t n_rows, gcs_policy p, int64_t B)
{
    return batch_arena_bytes(arena_rows, p, B) + al256((size_t)(kSlices * n_rows * B) * elem_bytes(p));
}

// The narrow launches' image, built at upload: tail entry j is launch
// k = tail_k0 + j (level k when k <= L, and the emission of level k-1).
struct FlatImage {
    int64_t first = 0;              // tail entry of the first narrow launch
    std::vector<int32_t> words;     // the image (loaded whole into LDS)
    FlatArgs args{};                // idx is set at upload
    size_t lds_bytes = 0;
};

// Picks the longest suffix of tail entries that fits: every entry's work
// (nodes plus emission lanes) at most flat_max, all slots and sums below 2^16,
// the LDS part within budget.  Then rewrites every reference as a slot.
// Returns false (with the error set) only if a reference breaks the layering.
bool build_flat(const Grammar& g, const gcs_device* d, size_t elem, size_t budget, int64_t flat_max, bool direct,
                FlatImage& fi)
{
    const int64_t nent = d->tail_nent, k0 = d->tail_k0, alpha = g.alpha();
    auto width = [&](int64_t k) -> int64_t { return k >= 1 && k <= g.L ? g.lv[k].nb + g.lv[k].npt : 0; };
    auto for_refs = [&](int64_t j, auto&& fn) {  // children, pass-through sources, roots, in that order
        const int64_t k = k0 + j;
        if (k <= g.L) {
            const Level& l = g.lv[k];
            for (int64_t t = 0; t < 2 * l.nb; ++t) fn(g.child[2 * l.child_off + t]);
            for (int64_t t = 0; t < l.npt; ++t) fn(g.ptsrc[l.pt_off + t]);
        }
        const Level& pl = g.lv[k - 1];
        for (int64_t e = g.eoff[pl.grp_off]; e < g.eoff[pl.grp_off + pl.ngrp]; ++e) fn(g.epos[e]);
    };
    // selection, from the last entry backwards
    fi.first = nent;
    {
        std::vector<int32_t> terms;
        int64_t produced = 0, sums = 0, nrefs = 0, nroots = 0, ngoff = 0;
        for (int64_t j = nent - 1; j >= 0; --j) {
            const int64_t k = k0 + j;
            const Level& pl = g.lv[k - 1];
            if (width(k) + ((int64_t)pl.ngrp << d->team_log2[k - 1]) > flat_max) break;
            std::vector<int32_t> prev;
            for_refs(j, [&](int32_t c) { (c < alpha ? terms : prev).push_back(c); });
            std::sort(terms.begin(), terms.end());
            terms.erase(std::unique(terms.begin(), terms.end()), terms.end());
            std::sort(prev.begin(), prev.end());
            prev.erase(std::unique(prev.begin(), prev.end()), prev.end());
            produced += width(k);
            sums += pl.ngrp;
            nrefs += k <= g.L ? 2 * g.lv[k].nb + g.lv[k].npt : 0;
            nroots += g.eoff[pl.grp_off + pl.ngrp] - g.eoff[pl.grp_off];
            ngoff += pl.ngrp + 1;
            const int64_t staged = (int64_t)terms.size() + (int64_t)prev.size(), slots = staged + produced;
            // folds: at most one per emission sum (accumulator index, offset,
            // 16-bit list entry and the accumulator value itself)
            const int64_t words = (kFlatEntryWords * (nent - j) + ngoff + staged + 2 * sums + 1 + (nrefs + 1) / 2 +
                                   (nroots + 1) / 2 + (sums + 1) / 2 + 3) / 4 * 4;
            const size_t bytes = al16(4 * (size_t)words) + al16((size_t)slots * elem) + 2 * al16((size_t)sums * elem);
            if (slots > 65535 || sums > 65535 || bytes > budget) break;
            fi.first = j;
        }
    }
    const int64_t f0 = fi.first, n_ent = nent - f0;
    if (n_ent == 0) return true;
    // stage slots: the terminals referenced, then the first narrow launch's
    // references to the level the grid computed, each in increasing order
    std::vector<int32_t> terms, prevs;
    for (int64_t j = f0; j < nent; ++j)
        for_refs(j, [&](int32_t c) {
            if (c < alpha) terms.push_back(c);
            else if (j == f0) prevs.push_back(c);
        });
    for (auto* v : {&terms, &prevs}) {
        std::sort(v->begin(), v->end());
        v->erase(std::unique(v->begin(), v->end()), v->end());
    }
    const int64_t n_stage = (int64_t)(terms.size() + prevs.size());
    std::vector<int64_t> sb((size_t)g.L + 2, 0);  // first slot of level k's nodes
    int64_t slot = n_stage;
    for (int64_t j = f0; j < nent; ++j) {
        sb[k0 + j] = slot;
        slot += width(k0 + j);
    }
    const int64_t n_slots = slot;
    bool ok = true;
    auto map = [&](int32_t c, int64_t j) -> uint16_t {
        int64_t r;
        if (c < alpha) {
            r = std::lower_bound(terms.begin(), terms.end(), c) - terms.begin();
        } else if (j == f0) {
            r = (int64_t)terms.size() + (std::lower_bound(prevs.begin(), prevs.end(), c) - prevs.begin());
        } else {
            const int64_t kb = k0 + j - 1, off = (int64_t)c - g.lv[kb].base;
            if (off < 0 || off >= width(kb)) ok = false;
            r = sb[kb] + off;
        }
        if (r < 0 || r >= n_slots) {
            ok = false;
            r = 0;
        }
        return (uint16_t)r;
    };
    std::vector<int32_t> ent, goff;
    std::vector<uint16_t> refs, roots;
    std::vector<std::pair<int32_t, int32_t>> folds;  // (accumulator, sum slot) in level order
    int32_t sums = 0;
    for (int64_t j = f0; j < nent; ++j) {
        const int64_t k = k0 + j;
        const Level& pl = g.lv[k - 1];
        const int64_t nb = k <= g.L ? g.lv[k].nb : 0, npt = k <= g.L ? g.lv[k].npt : 0;
        const int32_t e[kFlatEntryWords] = {(int32_t)nb, (int32_t)npt, (int32_t)pl.ngrp, d->team_log2[k - 1],
                                            (int32_t)(k <= g.L ? sb[k] : 0), (int32_t)refs.size(),
                                            (int32_t)goff.size(), sums};
        ent.insert(ent.end(), e, e + kFlatEntryWords);
        if (k <= g.L) {
            const Level& l = g.lv[k];
            for (int64_t t = 0; t < 2 * l.nb; ++t) refs.push_back(map(g.child[2 * l.child_off + t], j));
            for (int64_t t = 0; t < l.npt; ++t) refs.push_back(map(g.ptsrc[l.pt_off + t], j));
        }
        goff.push_back((int32_t)roots.size());
        int x = 0;
        for (int64_t gi = 0; gi < pl.ngrp; ++gi) {
            while (x < kSlices - 1 && gi >= pl.gsl[x + 1]) ++x;
            const int64_t G = pl.grp_off + gi;
            for (int32_t e2 = g.eoff[G]; e2 < g.eoff[G + 1]; ++e2) roots.push_back(map(g.epos[e2], j));
            goff.push_back((int32_t)roots.size());
            // fold key: the row's slice accumulator, or the row of y itself
            // for a direct (idempotent) emission
            folds.push_back({(int32_t)(direct ? g.erow[G] : x * g.n_rows + g.erow[G]), sums + (int32_t)gi});
        }
        sums += (int32_t)pl.ngrp;
    }
    if (!ok) {
        set_error("internal layout check failed: a narrow level reads outside the level below");
        return false;
    }
    std::stable_sort(folds.begin(), folds.end(),
                     [](const std::pair<int32_t, int32_t>& a, const std::pair<int32_t, int32_t>& b) {
                         return a.first < b.first;
                     });
    std::vector<int32_t> facc, foff{0};
    std::vector<uint16_t> flist;
    for (size_t i = 0; i < folds.size(); ++i) {
        if (i == 0 || folds[i].first != folds[i - 1].first) {
            if (i) foff.push_back((int32_t)flist.size());
            facc.push_back(folds[i].first);
        }
        flist.push_back((uint16_t)folds[i].second);
    }
    if (!folds.empty()) foff.push_back((int32_t)flist.size());
    FlatArgs& fa = fi.args;
    std::vector<int32_t>& w = fi.words;
    auto put = [&](const std::vector<int32_t>& v) {
        const int32_t at = (int32_t)w.size();
        w.insert(w.end(), v.begin(), v.end());
        return at;
    };
    auto put16 = [&](const std::vector<uint16_t>& v) {
        const int32_t at = (int32_t)w.size();
        w.resize(w.size() + (v.size() + 1) / 2, 0);
        if (!v.empty()) std::memcpy(w.data() + at, v.data(), v.size() * 2);
        return at;
    };
    std::vector<int32_t> stage(terms);
    stage.insert(stage.end(), prevs.begin(), prevs.end());
    w = ent;
    fa.goff_word = put(goff);
    fa.stage_word = put(stage);
    fa.facc_word = put(facc);
    fa.foff_word = put(foff);
    fa.refs_word = put16(refs);
    fa.roots_word = put16(roots);
    fa.flist_word = put16(flist);
    w.resize((w.size() + 3) / 4 * 4, 0);
    fa.idx_words = (int32_t)w.size();
    fa.n_ent = (int32_t)n_ent;
    fa.n_stage = (int32_t)n_stage;
    fa.n_terms = (int32_t)terms.size();
    fa.alpha = (int32_t)alpha;
    fa.n_fold = (int32_t)facc.size();
    fa.vals_off = (int32_t)al16(4 * w.size());
    fa.gsum_off = (int32_t)(fa.vals_off + al16((size_t)n_slots * elem));
    fa.accv_off = (int32_t)(fa.gsum_off + al16((size_t)sums * elem));
    fi.lds_bytes = fa.accv_off + al16((size_t)fa.n_fold * elem);
    if (fi.lds_bytes > budget || w.size() > flat_section_words(g)) {
        set_error("internal layout check failed: the narrow levels' image exceeds its bound");
        return false;
    }
    return true;
}

// Every index a kernel dereferences must stay inside its buffer: children,
// pass-through sources and emission positions inside the arena, emission rows
// inside y, terminal descriptors inside x and V.  Checked once per upload.
bool layout_in_bounds(const Grammar& g)
{
    const int64_t arena = g.arena, alpha = g.alpha();
    // sizes inside the 32-bit index space and the level table complete
    if ((int64_t)g.lv.size() != (int64_t)g.L + 1 || alpha > arena || g.epos.size() >= (size_t)INT32_MAX ||
        g.erow.size() >= (size_t)INT32_MAX || g.child.size() >= (size_t)INT32_MAX ||
        g.ptsrc.size() >= (size_t)INT32_MAX || g.eoff.size() != g.erow.size() + 1)
        return false;
    // each level's emission groups follow the previous level's, ending at the last group
    int64_t go = 0;
    for (int k = 0; k <= g.L; ++k) {
        if (g.lv[k].grp_off != go || g.lv[k].ngrp < 0) return false;
        go += g.lv[k].ngrp;
    }
    if (go != (int64_t)g.erow.size()) return false;
    for (int32_t c : g.child)
        if (c < 0 || c >= arena) return false;
    for (int32_t c : g.ptsrc)
        if (c < 0 || c >= arena) return false;
    int64_t co = 0, po = 0;
    for (int k = 0; k <= g.L; ++k) {
        const Level& l = g.lv[k];
        for (int x = 0; x < kSlices; ++x)
            if (l.gsl[x] > l.gsl[x + 1] || (k > 0 && (l.bsl[x] > l.bsl[x + 1] || l.psl[x] > l.psl[x + 1])))
                return false;
        if (l.gsl[0] != 0 || l.gsl[kSlices] != l.ngrp) return false;
        if (k > 0 && (l.bsl[0] != 0 || l.bsl[kSlices] != l.nb || l.psl[0] != 0 || l.psl[kSlices] != l.npt))
            return false;
    }
    if (g.n_rows * kSlices >= (int64_t)INT32_MAX) return false;
    for (int k = 1; k <= g.L; ++k) {
        const Level& l = g.lv[k];
        // level buffers start past the terminals rounded up to 64 (room for
        // the Boolean sweep's packed terminal words)
        if (l.base < ((alpha + 63) & ~int64_t(63)) || l.base + l.nb + l.npt > arena) return false;
        if (l.child_off != co || l.pt_off != po) return false;
        co += l.nb;
        po += l.npt;
    }
    if (2 * co != (int64_t)g.child.size() || po != (int64_t)g.ptsrc.size()) return false;
    // every emission group holds at least one root (the kernels clamp a
    // lane's root index to its group's last root)
    for (size_t i = 0; i + 1 < g.eoff.size(); ++i)
        if (g.eoff[i] < 0 || g.eoff[i] >= g.eoff[i + 1]) return false;
    if (!g.eoff.empty() && g.eoff.back() != (int32_t)g.epos.size()) return false;
    for (int32_t e : g.epos)
        if (e < 0 || e >= arena) return false;
    for (int32_t r : g.erow)
        if (r < 0 || r >= g.n_rows) return false;
    for (int64_t t = 0; t < alpha; ++t)
        if (g.tcol[t] < 0 || g.tcol[t] >= g.n_cols || g.tval[t] < 0 || g.tval[t] >= (int64_t)g.V.size())
            return false;
    return arena <= (int64_t)INT32_MAX;
}

gcs_status check_values(const Grammar& g, gcs_policy p)
{
    if (p == GCS_PLUS_I64)
        for (double v : g.V)
            if (v != (double)(int64_t)v) {
                set_error("GCS_PLUS_I64 needs integral matrix values");
                return GCS_EINVAL;
            }
    return GCS_OK;
}

gcs_status hip_fail(hipError_t e, const char* what)
{
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return GCS_EHIP;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int want)
    {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != want && hipSetDevice(want) != hipSuccess) ok = false;
    }
    ~DeviceGuard()
    {
        int cur;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

inline int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

inline int64_t vblocks(const LevelArgs& a) { return (int64_t)kSlices * (a.pb_bin + a.pb_pt + a.pb_emit); }

// Launch arguments of level launch k = 1..L+1 (level k, or none for k = L+1,
// with the emission of level k-1), device pointers included.
LevelArgs make_args(const gcs_device* d, int64_t k)
{
    LevelArgs a{};
    int64_t mb = 0, mp = 0, mg = 0;
    if (k <= d->L) {
        const Level& l = d->lv[k];
        a.child = d->child + l.child_off;
        a.ptsrc = d->ptsrc + l.pt_off;
        a.nb = (int32_t)l.nb;
        a.cur = (int32_t)l.base;
        a.prev = (int32_t)d->lv[k - 1].base;
        for (int x = 0; x <= kSlices; ++x) {
            a.bsl[x] = (int32_t)l.bsl[x];
            a.psl[x] = (int32_t)l.psl[x];
        }
        for (int x = 0; x < kSlices; ++x) {
            mb = std::max<int64_t>(mb, l.bsl[x + 1] - l.bsl[x]);
            mp = std::max<int64_t>(mp, l.psl[x + 1] - l.psl[x]);
        }
    }
    const Level& e = d->lv[k - 1];
    if (k == 1 && d->l0_on) {  // level 0's groups cut by sub-slice
        a.erow = d->l0row;
        a.eoff = d->l0off;
    } else if (k == 1 && d->win_on) {  // no level-0 groups on the device (never read)
        a.erow = d->erow;
        a.eoff = d->eoff;
    } else {  // the uploaded sections begin at group grp_skip
        a.erow = d->erow + (e.grp_off - d->grp_skip);
        a.eoff = d->eoff + (e.grp_off - d->grp_skip);
    }
    a.epos = d->epos;
    a.chunk = d->chunk + d->chunk_off[k - 1];
    for (int x = 0; x <= kSlices; ++x) a.csl[x] = d->chunk_sl[k - 1][x];
    a.n_rows = (int32_t)d->n_rows;
    a.alpha = (int32_t)d->alpha;
    if (k > d->L) a.prev = (int32_t)e.base;
    a.team_log2 = d->team_log2[k - 1];
    for (int x = 0; x <= kSlices; ++x) a.gsl[x] = (int32_t)e.gsl[x];
    for (int x = 0; x < kSlices; ++x) mg = std::max<int64_t>(mg, e.gsl[x + 1] - e.gsl[x]);
    a.pb_bin = ceil_div(mb, kBlock * kBinItems);
    a.pb_pt = ceil_div(mp, kBlock * kBinItems);
    a.pb_emit = ceil_div(mg << a.team_log2, kBlock);
    return a;
}

// Stream emission can replace a team of one or two lanes (stream_block folds
// in their order).  By default it does where the groups are that short and
// the level has enough chunks to fill the device: on MI355X it took the
// launch emitting the copy graph's 1.7e8 groups of bare terminals from 6.62
// to 5.47 ms, but slowed levels of a few dozen chunks (too few workgroups,
// each with a longer chain of dependent steps) from 7.5 to 9.8 us.
constexpr int64_t kStreamMinChunks = 2048;
bool stream_capable(const gcs_device* d, int64_t k) { return d->team_log2[k] <= 1; }
bool prefer_stream(const gcs_device* d, const Grammar& g, int64_t k)
{
    const int64_t ngrp = d->lv[k].ngrp;  // the device's view (level 0 possibly cut)
    if (ngrp == 0 || !stream_capable(d, k)) return false;
    return level_roots(g, k) <= 8 * ngrp && d->chunk_sl[k][kSlices] >= kStreamMinChunks;
}

bool has_tail(const gcs_device* d)
{
    if (d->n_rows > 0) return true;
    for (int64_t k = d->tail_k0; k <= d->L + 1; ++k)
        if (vblocks(d->largs[k - 1]) > 0) return true;
    return false;
}
// the leaf launch also resets the tail's barrier counter
bool has_leaf(const gcs_device* d) { return d->alpha > 0 || d->n_rows > 0 || has_tail(d); }

// launches of one sweep
int64_t count_launches(const gcs_device* d)
{
    int64_t c = has_leaf(d) ? 1 : 0;
    for (int64_t k = 1; k < d->tail_k0; ++k) c += vblocks(d->largs[k - 1]) > 0;
    c += d->win_on ? 1 : 0;
    return c + (has_tail(d) ? 1 : 0);
}

template <class P>
gcs_status run_sweep(gcs_device* d, const void* xv, void* yv, hipStream_t s, hipEvent_t* ev = nullptr,
                     int32_t accumulate = 0, bool span = false)
{
    using A = typename P::A;
    auto* arena = (A*)d->arena;
    auto* y = (typename P::Y*)yv;
    // direct emission writes y itself (cleared by the leaf launch unless
    // accumulating); otherwise the slice accumulators, reduced into y at the end
    auto* acc = kDirectEmit<P> ? (A*)yv : (A*)d->acc;
    // profiling: events[2i] before launch i, events[2i+1] right after it; or
    // (span) events[0] before the first wide level launch, events[1] after the last
    int64_t li = 0;
    auto mark = [&]() {
        if (ev && !span) (void)hipEventRecord(ev[li++], s);
    };
    const int32_t n_acc = kDirectEmit<P> ? (accumulate ? 0 : (int32_t)d->n_rows) : (int32_t)(kSlices * d->n_rows);
    if (has_leaf(d)) {
        mark();
        const int64_t items = std::max<int64_t>(d->alpha, n_acc);
        if (items >= kLeafMultiMin)
            leaf_kernel<P, kLeafItems><<<ceil_div(items, kBlock * kLeafItems), kBlock, 0, s>>>(
                d->tcol, d->tval, (const typename P::W*)d->V, (const typename P::X*)xv, arena, (int32_t)d->alpha,
                acc, n_acc, d->barrier);
        else
            leaf_kernel<P, 1><<<std::max(1, ceil_div(items, kBlock)), kBlock, 0, s>>>(
                d->tcol, d->tval, (const typename P::W*)d->V, (const typename P::X*)xv, arena, (int32_t)d->alpha,
                acc, n_acc, d->barrier);
        mark();
    }
    if (ev && span) (void)hipEventRecord(ev[0], s);
    for (int64_t k = 1; k < d->tail_k0; ++k) {
        const LevelArgs& a = d->largs[k - 1];
        const int64_t grid = std::min<int64_t>(vblocks(a), d->grid_max);
        if (grid > 0) {
            mark();
            level_kernel<P><<<(int32_t)grid, kBlock, 0, s>>>(a, arena, acc);
            mark();
        }
        if constexpr (kDirectEmit<P>) {
            if (k == 1 && d->win_on) {  // level 0's emission: words, terminals from LDS windows of T
                mark();
                window_emit_kernel<P><<<d->win_grid, kWinBlock, d->win_lds, s>>>(d->win, arena, y);
                mark();
            }
        }
    }
    if (ev && span) (void)hipEventRecord(ev[1], s);
    if (has_tail(d)) {
        mark();
        const LevelArgs* table = d->tail_table;
        int32_t n_multi = (int32_t)d->tail_multi, n_rows = (int32_t)d->n_rows;
        FlatArgs flat = d->flat;
        unsigned* bar = d->barrier;
        int* errp = d->err;
        // the limit is a property of the kernel, shared by every handle: all
        // of them raise it to the same device budget (never lower it)
        if (d->flat_lds > 65536 && !d->flat_attr) {
            hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&tail_kernel<P>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)d->flat_budget);
            if (ea != hipSuccess) return hip_fail(ea, "hipFuncSetAttribute (tail LDS)");
            d->flat_attr = true;
        }
        int32_t n_grid = d->tail_wgs;
        unsigned spin = d->spin_limit;
        void* args[] = {&table, &n_multi, &n_grid, &flat, &arena, &acc, &y, &n_rows, &accumulate, &bar, &errp, &spin};
        const unsigned wgs = (unsigned)d->tail_wgs + (flat.n_ent > 0 ? 1u : 0u);
        // an ordinary launch by default: the grid (at most one workgroup per
        // CU) has the device to itself behind the sweep's earlier launches,
        // and the barrier's bounded wait flags the sweep if it ever is not
        // all resident; a cooperative launch (tail_coop) has the runtime
        // certify residency, for devices shared with long-running kernels,
        // and costs ~11 us more launch latency per sweep on MI355X
        hipError_t e;
        if (!d->tail_coop) {
            tail_kernel<P><<<dim3(wgs), dim3(kTailBlock), d->flat_lds, s>>>(table, n_multi, n_grid, flat, arena, acc, y,
                                                                           n_rows, accumulate, bar, errp, spin);
            e = hipGetLastError();
        } else {
            e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&tail_kernel<P>), dim3(wgs), dim3(kTailBlock),
                                           args, d->flat_lds, s);
        }
        if (e != hipSuccess) return hip_fail(e, "tail launch");
        mark();
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_fail(err, "sweep launch");
    return GCS_OK;
}

template <class P, bool LEAVES>
void launch_level_batch(int VW, int64_t grid, const BatchArgs& ba, typename P::A* arena, typename P::A* acc,
                        hipStream_t s)
{
    switch (VW) {
    case 1: level_batch_kernel<P, 1, LEAVES><<<(int32_t)grid, kBlock, 0, s>>>(ba, arena, acc); break;
    case 2: level_batch_kernel<P, 2, LEAVES><<<(int32_t)grid, kBlock, 0, s>>>(ba, arena, acc); break;
    case 4: level_batch_kernel<P, 4, LEAVES><<<(int32_t)grid, kBlock, 0, s>>>(ba, arena, acc); break;
    case 8: level_batch_kernel<P, 8, LEAVES><<<(int32_t)grid, kBlock, 0, s>>>(ba, arena, acc); break;
    default: level_batch_kernel<P, 16, LEAVES><<<(int32_t)grid, kBlock, 0, s>>>(ba, arena, acc); break;
    }
}

// Y = M X for B vectors: leaf, one launch per level k = 1..L+1 (level k and
// the emission of level k-1), slice reduction into Y.
template <class P>
gcs_status run_sweep_batch(gcs_device* d, const void* xv, void* yv, int32_t B, void* ws, int32_t flags,
                           hipStream_t s)
{
    using A = typename P::A;
    const bool leaves = (flags & GCS_BATCH_LEAVES_IN_SWEEP) != 0;
    const int32_t accumulate = (flags & GCS_BATCH_ACCUMULATE) ? 1 : 0;
    auto* arena = (A*)ws;
    // direct policies emit into Y itself (cleared here unless accumulating)
    auto* acc = kDirectEmit<P> ? (A*)yv
                               : (A*)((unsigned char*)ws + batch_arena_bytes(batch_arena_rows(d, flags), d->policy, B));
    // widest access of at most 16 bytes that divides the row
    int VW = 1;
    while (VW * 2 * (int)sizeof(A) <= 16 && B % (VW * 2) == 0) VW *= 2;
    int vb_log2 = 0;
    while ((1 << vb_log2) < B / VW) ++vb_log2;
    const int32_t per = kBlock >> vb_log2;
    const int64_t n_acc = kDirectEmit<P> ? (accumulate ? 0 : d->n_rows * B) : (int64_t)kSlices * d->n_rows * B;
    // the terminal array (unless the leaves are evaluated in the sweep) and
    // the accumulator clear
    const int64_t t_rows = leaves ? 0 : d->alpha;
    const int64_t leaf_items = std::max<int64_t>(t_rows * B, n_acc);
    const int64_t grid_leaf = std::min<int64_t>(std::max<int64_t>(1, (leaf_items + kBlock - 1) / kBlock), 1 << 16);
    leaf_batch_kernel<P><<<(int32_t)grid_leaf, kBlock, 0, s>>>(d->tcol, d->tval, (const typename P::W*)d->V,
                                                                (const typename P::X*)xv, arena, t_rows, B, acc,
                                                                n_acc);
    for (int64_t k = 1; k <= d->L + 1; ++k) {
        BatchArgs ba{};
        ba.a = d->largs[k - 1];
        ba.B = B;
        ba.vb_log2 = vb_log2;
        ba.leaf_alpha = leaves ? (int32_t)d->alpha : 0;
        ba.tbase = leaves ? (int32_t)d->alpha : 0;
        ba.tcol = d->tcol;
        ba.tval = d->tval;
        ba.V = d->V;
        ba.X = xv;
        int64_t mb = 0, mp = 0, mg = 0;
        for (int x = 0; x < kSlices; ++x) {
            mb = std::max<int64_t>(mb, ba.a.bsl[x + 1] - ba.a.bsl[x]);
            mp = std::max<int64_t>(mp, ba.a.psl[x + 1] - ba.a.psl[x]);
            mg = std::max<int64_t>(mg, ba.a.gsl[x + 1] - ba.a.gsl[x]);
        }
        ba.pb_bin = ceil_div(mb, per * kBinItems);
        ba.pb_pt = ceil_div(mp, per * kBinItems);
        ba.pb_emit = ceil_div(mg, per);
        const int64_t grid = (int64_t)kSlices * (ba.pb_bin + ba.pb_pt + ba.pb_emit);
        if (grid > 0) {
            if (leaves) launch_level_batch<P, true>(VW, grid, ba, arena, acc, s);
            else launch_level_batch<P, false>(VW, grid, ba, arena, acc, s);
        }
        if constexpr (kDirectEmit<P>) {
            if (k == 1 && d->win_on) {  // level 0's emission from its words, vector by vector
                if (leaves) window_batch_kernel<P, true><<<d->win_grid, kWinBlock, 0, s>>>(d->win, ba, arena, acc);
                else window_batch_kernel<P, false><<<d->win_grid, kWinBlock, 0, s>>>(d->win, ba, arena, acc);
            }
        }
    }
    const int64_t n = d->n_rows * B;
    if (n > 0 && !kDirectEmit<P>) {
        const int64_t grid = std::min<int64_t>((n + kBlock - 1) / kBlock, 1 << 16);
        reduce_batch_kernel<P><<<(int32_t)grid, kBlock, 0, s>>>(acc, (typename P::Y*)yv, n, accumulate);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_fail(err, "batched sweep launch");
    return GCS_OK;
}

}  // namespace
}  // namespace gcs

using gcs::Grammar;

extern "C" gcs_status gcs_level0_words(const gcs_grammar* h, gcs_policy p, uint32_t* words, int64_t words_cap,
                                      int32_t* chunks, int64_t chunks_cap, int64_t* n_words, int64_t* n_chunks,
                                      int32_t* n_sub)
{
    if (!h || !n_words || !n_chunks || !gcs::valid_policy(p) || words_cap < 0 || chunks_cap < 0) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    gcs_status st = gcs::check_values(g, p);
    if (st != GCS_OK) return st;
    *n_words = *n_chunks = 0;
    const gcs::Level0Plan pl = gcs::level0_plan(g, p);
    if (n_sub) *n_sub = pl.window ? pl.S : 0;
    if (!pl.window) return GCS_OK;
    gcs::Level0Split l0;
    gcs::level0_split(g, pl.S, l0);
    std::vector<uint32_t> w;
    std::vector<int4> c;
    if (!gcs::build_window_words(l0, g.n_rows, p == GCS_BOOL_OR ? 0 : (int64_t)gcs::elem_bytes(p), w, c))
        return GCS_ESTATE;
    *n_words = (int64_t)w.size();
    *n_chunks = (int64_t)(c.size() / 2);
    if (words) {
        if (words_cap < *n_words) {
            gcs::set_error("words capacity too small");
            return GCS_ERANGE;
        }
        std::memcpy(words, w.data(), w.size() * 4);
    }
    if (chunks) {
        if (chunks_cap < 8 * *n_chunks) {
            gcs::set_error("chunks capacity too small");
            return GCS_ERANGE;
        }
        std::memcpy(chunks, c.data(), c.size() * sizeof(int4));
    }
    return GCS_OK;
}

extern "C" gcs_status gcs_device_layout(const gcs_grammar* h, gcs_policy p, gcs_dev_sizes* out)
{
    if (!h || !out || !gcs::valid_policy(p)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    gcs_status st = gcs::check_values(g, p);
    if (st != GCS_OK) return st;
    out->grammar_bytes = gcs::image_layout(g, p).total;
    out->workspace_bytes = gcs::workspace_bytes(g, p);
    out->x_len = g.n_cols;
    out->y_len = g.n_rows;
    out->x_elem_bytes = (int32_t)gcs::x_bytes(p);
    out->y_elem_bytes = (int32_t)gcs::y_bytes(p);
    return GCS_OK;
}

// ------------------------------------------------------------ fixed scratch
// The batch workspace of gcs_sweep_right_batch_scratch: one array per GPU in
// the library's device code, for callers that cannot allocate.  Host code
// never passes the array's name to a kernel: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
hipError_t g_scratch_err[kScratchDevices] = {};
bool g_scratch_done[kScratchDevices] = {};

// resolves the scratch address of device `dev`, which must be current
void scratch_setup(int dev)
{
    if (dev < 0 || dev >= kScratchDevices) return;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_done[dev]) return;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
    g_scratch_err[dev] = e;
    g_scratch_done[dev] = true;
}
}  // namespace

extern "C" gcs_status gcs_upload(const gcs_grammar* h, gcs_policy p, void* grammar_dev, size_t grammar_bytes,
                                 void* workspace_dev, size_t workspace_bytes, void* stream, gcs_device** out)
{
    if (!h || !out || !gcs::valid_policy(p) || !grammar_dev || !workspace_dev) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    *out = nullptr;
    const Grammar& g = h->g;
    gcs_status st = gcs::check_values(g, p);
    if (st != GCS_OK) return st;
    if (!gcs::layout_in_bounds(g)) {
        gcs::set_error("internal layout check failed: an index falls outside its buffer");
        return GCS_ESTATE;
    }
    const gcs::Image im = gcs::image_layout(g, p);
    if (grammar_bytes < im.total || workspace_bytes < gcs::workspace_bytes(g, p)) {
        gcs::set_error("device buffers smaller than gcs_device_layout reports");
        return GCS_EINVAL;
    }
    if (((uintptr_t)grammar_dev & 255) || ((uintptr_t)workspace_dev & 255)) {
        gcs::set_error("device buffers must be 256-byte aligned");
        return GCS_EINVAL;
    }
    hipStream_t s = (hipStream_t)stream;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return gcs::hip_fail(e, "hipGetDevice");
    scratch_setup(dev);  // device set-up: the fixed scratch of this GPU

    // policy-typed V
    std::vector<unsigned char> vbuf(g.V.size() * gcs::v_bytes(p));
    for (size_t i = 0; i < g.V.size(); ++i) {
        unsigned char* o = vbuf.data() + i * gcs::v_bytes(p);
        switch (p) {
        case GCS_PLUS_F64:
        case GCS_PLUS_F32_ACC_F64:
        case GCS_MIN_PLUS_F64: {
            double v = g.V[i];
            std::memcpy(o, &v, 8);
            break;
        }
        case GCS_PLUS_F32:
        case GCS_MIN_PLUS_F32: {
            float v = (float)g.V[i];
            std::memcpy(o, &v, 4);
            break;
        }
        case GCS_BOOL_OR: *o = 1; break;
        case GCS_PLUS_I64: {
            int64_t v = (int64_t)g.V[i];
            std::memcpy(o, &v, 8);
            break;
        }
        }
    }
    // level 0's emission cut by column sub-slice (direct policies, large T;
    // Boolean: LDS windows)
    gcs::Level0Split l0;
    const gcs::Level0Plan l0_plan = gcs::level0_plan(g, p);
    if (l0_plan.cut) gcs::level0_split(g, l0_plan.S, l0);
    const int64_t r0 = g.lv[0].ngrp > 0 ? g.eoff[g.lv[0].grp_off + g.lv[0].ngrp] : 0;  // level 0's roots: [0, r0)
    const bool win_on = l0_plan.window;  // Boolean level 0 as words (window_emit_kernel)
    if (l0.on && ((int64_t)l0.pos.size() != r0 || g.lv[0].grp_off != 0 ||
                  (!win_on && im.l0off - im.l0row < l0.row.size() * 4))) {
        gcs::set_error("internal error: level-0 sub-slice cut does not match the image");
        return GCS_ESTATE;
    }
    std::vector<uint32_t> words;
    std::vector<int4> wch;
    if (win_on) {
        if (!gcs::build_window_words(l0, g.n_rows, p == GCS_BOOL_OR ? 0 : (int64_t)gcs::elem_bytes(p), words, wch))
            return GCS_ESTATE;
        if (wch.size() * sizeof(int4) > im.wword - im.wchunk || words.size() * 4 > im.tcol - im.wword) {
            gcs::set_error("internal error: more window chunks or words than the image holds");
            return GCS_ESTATE;
        }
    }
    const size_t skip0 = l0.on ? (size_t)g.lv[0].ngrp : 0;  // the grammar's level-0 groups, not uploaded when cut
    // with windows the root list on the device starts at level 1's roots:
    // the uploaded group offsets are rebased by level 0's root count
    const size_t rskip = win_on ? (size_t)r0 : 0;
    std::vector<int32_t> eoff_rebased;
    if (win_on) {
        eoff_rebased.assign(g.eoff.begin() + (ptrdiff_t)skip0, g.eoff.end());
        for (int32_t& v : eoff_rebased) v -= (int32_t)r0;
    }
    std::vector<int32_t> chunk;
    std::vector<int64_t> chunk_off;
    std::vector<std::array<int32_t, gcs::kSlices + 1>> chunk_sl;
    gcs::build_chunks(g, &l0, win_on, chunk, chunk_off, chunk_sl);
    if (chunk.size() > gcs::chunk_bound(g, l0.on ? (int64_t)l0.row.size() : 0)) {
        gcs::set_error("internal error: more emission chunks than the image holds");
        return GCS_ESTATE;
    }
    auto* base = (unsigned char*)grammar_dev;
    struct Sec {
        size_t off;
        const void* src;
        size_t bytes;
    } secs[] = {
        {im.child, g.child.data(), g.child.size() * 4}, {im.ptsrc, g.ptsrc.data(), g.ptsrc.size() * 4},
        {im.erow, g.erow.data() + skip0, (g.erow.size() - skip0) * 4},
        {im.eoff, win_on ? eoff_rebased.data() : g.eoff.data() + skip0, (g.eoff.size() - skip0) * 4},
        // the root list, level 0's part in the sub-slice order when cut (and
        // left out with windows)
        {im.epos, l0.on ? l0.pos.data() : g.epos.data(), (size_t)(r0 - (int64_t)rskip) * 4},
        {im.epos + (size_t)(r0 - (int64_t)rskip) * 4, g.epos.data() + r0, (g.epos.size() - (size_t)r0) * 4},
        {im.chunk, chunk.data(), chunk.size() * 4},
        {im.l0row, l0.row.data(), win_on ? 0 : l0.row.size() * 4},
        {im.l0off, l0.off.data(), win_on ? 0 : l0.off.size() * 4},
        {im.wchunk, wch.data(), wch.size() * sizeof(int4)},
        {im.wword, words.data(), words.size() * 4},
        {im.tcol, g.tcol.data(), g.tcol.size() * 4},
        {im.tval, g.tval.data(), g.tval.size() * 4},    {im.V, vbuf.data(), vbuf.size()},
    };
    {
        gcs::PinnedStage stage;
        e = stage.init();
        if (e != hipSuccess) return gcs::hip_fail(e, "hipHostMalloc (upload staging)");
        for (const Sec& c : secs) {
            if (!c.bytes) continue;
            e = stage.h2d(base + c.off, c.src, c.bytes, s);
            if (e != hipSuccess) return gcs::hip_fail(e, "hipMemcpyAsync (upload)");
        }
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipStreamSynchronize (upload)");
    }

    auto* d = new gcs_device();
    d->policy = p;
    d->device = dev;
    d->n_rows = g.n_rows;
    d->n_cols = g.n_cols;
    d->alpha = g.alpha();
    d->L = g.L;
    d->arena_len = g.arena;
    d->lv = g.lv;
    if (l0.on) {  // the device's view of level 0: the cut groups, or none with windows
        d->lv[0].ngrp = win_on ? 0 : (int64_t)l0.row.size();
        for (int x = 0; x <= gcs::kSlices; ++x) d->lv[0].gsl[x] = win_on ? 0 : l0.gsl[x];
        d->l0_sub = l0.S;
        if (!win_on) {
            d->l0_on = true;
            d->l0row = (const int32_t*)(base + im.l0row);
            d->l0off = (const int32_t*)(base + im.l0off);
        }
    }
    if (win_on) {
        d->win_on = true;
        d->win.chunk = (const int4*)(base + im.wchunk);
        d->win.word = (const uint32_t*)(base + im.wword);
        d->win.n_chunks = (int32_t)(wch.size() / 2);
        d->win_grid = d->win.n_chunks;
        d->win_words = (int64_t)words.size();
        int32_t mb = 0;
        for (size_t i = 0; i < wch.size(); i += 2) mb = std::max(mb, wch[i].w - wch[i].z);
        d->win_lds = (size_t)std::max(mb, 16);
    }
    // emission team per level: about GCS_EMIT_PER_LANE (default 4) roots per
    // lane, at most one wave
    const char* pl_env = std::getenv("GCS_EMIT_PER_LANE");
    const double per_lane = pl_env ? std::max(0.5, std::atof(pl_env)) : 4.0;
    d->team_log2.assign(g.lv.size(), 0);
    for (size_t k = 0; k < g.lv.size(); ++k) {
        const gcs::Level& l = d->lv[k];
        if (l.ngrp == 0) continue;
        const int64_t roots = gcs::level_roots(g, (int64_t)k);
        const double mean = (double)roots / (double)l.ngrp;
        int t = 0;
        while (t < 6 && (double)(1 << t) * per_lane < mean && (l.ngrp << (t + 1)) < (int64_t)INT32_MAX - gcs::kBlock) ++t;
        d->team_log2[k] = t;
    }
    d->child = (const int2*)(base + im.child);
    d->ptsrc = (const int32_t*)(base + im.ptsrc);
    // group g of the grammar at erow + (g - grp_skip): when level 0 is cut,
    // the sections begin at level 1's first group
    d->erow = (const int32_t*)(base + im.erow);
    d->eoff = (const int32_t*)(base + im.eoff);
    d->grp_skip = (int64_t)skip0;
    d->epos = (const int32_t*)(base + im.epos);
    d->chunk = (const int32_t*)(base + im.chunk);
    d->chunk_off = std::move(chunk_off);
    d->chunk_sl = std::move(chunk_sl);
    d->tcol = (const int32_t*)(base + im.tcol);
    d->tval = (const int32_t*)(base + im.tval);
    d->V = base + im.V;
    // [counters (256 B) | arena | accumulators]: the counters come first so
    // that uploads sharing one workspace share them at the same address
    d->counters = (unsigned long long*)workspace_dev;
    d->arena = (unsigned char*)workspace_dev + 256;
    d->acc = (unsigned char*)workspace_dev + 256 + gcs::arena_bytes(g, p);
    d->barrier = (unsigned*)(d->counters + 2);
    d->err = (int*)(d->counters + 3);
    // launch arguments of every level; the narrow levels at the top go to the
    // persistent tail kernel: from the first level k0 after which no launch
    // needs more than tail_vb virtual blocks per tail workgroup
    int dev_cu = 0;
    (void)hipDeviceGetAttribute(&dev_cu, hipDeviceAttributeMultiprocessorCount, dev);
    auto env_int = [](const char* name, int dflt) {
        const char* v = std::getenv(name);
        return v ? std::atoi(v) : dflt;
    };
    // the tail kernel as a cooperative launch only on request
    d->tail_coop = env_int("GCS_TAIL_COOP", 0) != 0;
    // polls before a tail barrier gives up and marks the sweep failed: about
    // a second by default; a small value forces the failure path (tests)
    d->spin_limit = (unsigned)std::max(0, env_int("GCS_TAIL_SPIN_LIMIT", 1 << 25));
    int coop = 0;
    (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (d->tail_coop && !coop) {
        delete d;
        gcs::set_error("GCS_TAIL_COOP=1: the device does not support cooperative launches");
        return GCS_EHIP;
    }
    // 8 workgroups (one per XCD), one virtual block per 256-lane quarter and
    // level: measured best on MI355X with the ordinary tail launch (fewest
    // arrivals per barrier round; the wider levels this leaves out run as
    // launches): 0.0645 ms per sweep on the 512 x 4096 genotype against 0.071 /
    // 0.075 / 0.081 ms with 16 / 32 / 64, the bench matrix 0.450 ms either way
    // (at most one fewer than the compute units: the narrow levels' workgroup
    // joins the grid, and each of these workgroups needs a CU)
    d->tail_wgs = std::max(gcs::kSlices, (std::min(env_int("GCS_TAIL_WGS", 8), std::max(dev_cu - 1, gcs::kSlices)) /
                                          gcs::kSlices) * gcs::kSlices);
    const int64_t tail_vb = std::max(1, env_int("GCS_TAIL_VB", 1));
    // wide launches: one virtual block per workgroup unless GCS_GRID_MAX caps
    // the grid (then workgroups stride over the blocks)
    d->grid_max = std::max(gcs::kSlices, env_int("GCS_GRID_MAX", INT32_MAX) / gcs::kSlices * gcs::kSlices);
    d->largs.resize((size_t)g.L + 1);
    for (int64_t k = 1; k <= g.L + 1; ++k) d->largs[k - 1] = gcs::make_args(d, k);
    d->tail_k0 = g.L + 1;
    const int64_t quarters = gcs::kTailBlock / gcs::kBlock;
    while (d->tail_k0 > 1 && gcs::vblocks(d->largs[d->tail_k0 - 2]) <= tail_vb * quarters * d->tail_wgs) --d->tail_k0;
    // level 0's cut groups are emitted by a wide launch only (the narrow
    // levels' LDS image is built from the grammar's own groups)
    if (d->l0_on || d->win_on) d->tail_k0 = std::max<int64_t>(d->tail_k0, 2);
    d->tail_nent = g.L + 2 - d->tail_k0;
    // emission mode of each wide launch: chunks where the groups are short
    // and uneven, teams elsewhere (GCS_EMIT_STREAM = 0 keeps teams, 1 takes
    // chunks wherever the team has at most two lanes; the bits are the same)
    {
        const int forced = env_int("GCS_EMIT_STREAM", -1);
        for (int64_t k = 1; k < d->tail_k0; ++k) {
            gcs::LevelArgs& a = d->largs[k - 1];
            const bool st = forced >= 0 ? forced != 0 && gcs::stream_capable(d, k - 1) : gcs::prefer_stream(d, g, k - 1);
            if (!st) continue;
            a.stream = 1;
            int32_t mc = 0;
            for (int x = 0; x < gcs::kSlices; ++x) mc = std::max(mc, a.csl[x + 1] - a.csl[x]);
            a.pb_emit = mc;
        }
        if (d->win_on) {  // launch 1's emission runs in window_emit_kernel
            d->largs[0].stream = 0;
            d->largs[0].pb_emit = 0;
        }
        if (std::getenv("GCS_UPLOAD_TRACE")) {
            int n_stream = 0;
            for (int64_t k = 1; k < d->tail_k0; ++k) n_stream += d->largs[k - 1].stream != 0;
            std::fprintf(stderr, "[gcs upload] stream emission in %d of %lld wide launches\n", n_stream,
                         (long long)d->tail_k0 - 1);
            std::fprintf(stderr,
                         "[gcs upload] level-0 emission in %d sub-slices per slice (%lld groups, %lld before); "
                         "LDS windows %d (%d chunks, %lld words, %zu bytes)\n",
                         d->l0_on || d->win_on ? d->l0_sub : 0, (long long)d->lv[0].ngrp, (long long)g.lv[0].ngrp,
                         (int)d->win_on, d->win_on ? d->win.n_chunks : 0, (long long)d->win_words, d->win_lds);
        }
    }
    // the narrowest entries at the end run on workgroup 0 alone, in LDS: as
    // many as fit its budget, each with at most GCS_TAIL_FLAT work items
    {
        int max_lds = 0;
        (void)hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        const size_t budget = std::min(gcs::kFlatLdsMax, (size_t)std::max(0, max_lds - 2048));
        d->flat_budget = budget;
        gcs::FlatImage fi;
        if (!gcs::build_flat(g, d, gcs::elem_bytes(p), budget, env_int("GCS_TAIL_FLAT", 4096), gcs::direct_emit(p), fi)) {
            delete d;
            return GCS_ESTATE;
        }
        d->tail_multi = fi.first;
        d->flat = fi.args;
        d->flat_lds = fi.args.n_ent > 0 ? fi.lds_bytes : 0;
        d->flat.idx = (const int32_t*)(base + im.flat);
        if (std::getenv("GCS_UPLOAD_TRACE"))
            std::fprintf(stderr,
                         "[gcs upload] levels %lld: wide launches 1..%lld, tail grid %d workgroups over %lld "
                         "launches, narrow launches %d in LDS (%zu bytes: %d image words, %d staged of which %d "
                         "terminals, %d folds)\n",
                         (long long)g.L, (long long)d->tail_k0 - 1, d->tail_wgs, (long long)d->tail_multi,
                         fi.args.n_ent, d->flat_lds, fi.args.idx_words, fi.args.n_stage, fi.args.n_terms,
                         fi.args.n_fold);
        if (!fi.words.empty()) {
            e = hipMemcpyAsync(base + im.flat, fi.words.data(), fi.words.size() * 4, hipMemcpyHostToDevice, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            if (e != hipSuccess) {
                delete d;
                return gcs::hip_fail(e, "hipMemcpyAsync (narrow levels)");
            }
        }
    }
    d->tail_table = (const gcs::LevelArgs*)(base + im.table) + (d->tail_k0 - 1);
    e = hipMemcpyAsync(base + im.table, d->largs.data(), d->largs.size() * sizeof(gcs::LevelArgs),
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete d;
        return gcs::hip_fail(e, "hipMemcpyAsync (launch table)");
    }
    e = hipMemsetAsync(d->counters, 0, 256, s);  // BFS counts, barrier, error flag
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete d;
        return gcs::hip_fail(e, "hipMemsetAsync (counters)");
    }
    d->pinned = nullptr;
    e = hipHostMalloc((void**)&d->pinned, 64, hipHostMallocDefault);
    if (e != hipSuccess) {
        delete d;
        return gcs::hip_fail(e, "hipHostMalloc");
    }
    *out = d;
    return GCS_OK;
}

static gcs_status sweep_dispatch(gcs_device* d, const void* x_dev, void* y_dev, void* stream, hipEvent_t* ev,
                                 int32_t accumulate = 0, bool span = false)
{
    if (!d || (d->n_cols > 0 && !x_dev) || (d->n_rows > 0 && !y_dev)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    if (!guard.ok) {
        gcs::set_error("cannot select the upload's device");
        return GCS_EHIP;
    }
    hipStream_t s = (hipStream_t)stream;
    switch (d->policy) {
    case GCS_PLUS_F64: return gcs::run_sweep<gcs::PolPlusF64>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_PLUS_F32: return gcs::run_sweep<gcs::PolPlusF32>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_PLUS_F32_ACC_F64: return gcs::run_sweep<gcs::PolPlusF32AccF64>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_BOOL_OR: return gcs::run_sweep<gcs::PolBoolOr>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_PLUS_I64: return gcs::run_sweep<gcs::PolPlusI64>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_MIN_PLUS_F32: return gcs::run_sweep<gcs::PolMinPlusF32>(d, x_dev, y_dev, s, ev, accumulate, span);
    case GCS_MIN_PLUS_F64: return gcs::run_sweep<gcs::PolMinPlusF64>(d, x_dev, y_dev, s, ev, accumulate, span);
    }
    gcs::set_error("corrupt device handle");
    return GCS_ESTATE;
}

extern "C" gcs_status gcs_sweep_right(gcs_device* d, const void* x_dev, void* y_dev, void* stream)
{
    return sweep_dispatch(d, x_dev, y_dev, stream, nullptr);
}

extern "C" gcs_status gcs_sweep_right_acc(gcs_device* d, const void* x_dev, void* y_dev, void* stream)
{
    return sweep_dispatch(d, x_dev, y_dev, stream, nullptr, 1);
}

static bool batch_flags_ok(int32_t flags)
{
    return (flags & ~(GCS_BATCH_ACCUMULATE | GCS_BATCH_LEAVES_IN_SWEEP)) == 0;
}

extern "C" gcs_status gcs_batch_workspace_bytes(const gcs_device* d, int32_t nvec, int32_t flags, size_t* bytes)
{
    if (!d || !bytes || nvec < 1 || nvec > gcs::kMaxBatch || !batch_flags_ok(flags)) {
        gcs::set_error("invalid argument (nvec must be in 1..64, flags known)");
        return GCS_EINVAL;
    }
    *bytes = gcs::batch_workspace_bytes(gcs::batch_arena_rows(d, flags), d->n_rows, d->policy, nvec);
    return GCS_OK;
}

static gcs_status batch_dispatch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec, void* workspace_dev,
                                 int32_t flags, hipStream_t s);

extern "C" gcs_status gcs_sweep_right_batch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec,
                                            void* workspace_dev, size_t workspace_bytes, int32_t flags,
                                            void* stream)
{
    if (!d || nvec < 1 || nvec > gcs::kMaxBatch || !batch_flags_ok(flags) || (d->n_cols > 0 && !x_dev) ||
        (d->n_rows > 0 && !y_dev) || !workspace_dev) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    if ((uintptr_t)workspace_dev & 255) {
        gcs::set_error("the batch workspace must be 256-byte aligned");
        return GCS_EINVAL;
    }
    if (workspace_bytes < gcs::batch_workspace_bytes(gcs::batch_arena_rows(d, flags), d->n_rows, d->policy, nvec)) {
        gcs::set_error("batch workspace smaller than gcs_batch_workspace_bytes reports");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    if (!guard.ok) {
        gcs::set_error("cannot select the upload's device");
        return GCS_EHIP;
    }
    return batch_dispatch(d, x_dev, y_dev, nvec, workspace_dev, flags, (hipStream_t)stream);
}

static gcs_status batch_dispatch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec, void* workspace_dev,
                                 int32_t flags, hipStream_t s)
{
    switch (d->policy) {
    case GCS_PLUS_F64: return gcs::run_sweep_batch<gcs::PolPlusF64>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_PLUS_F32: return gcs::run_sweep_batch<gcs::PolPlusF32>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_PLUS_F32_ACC_F64:
        return gcs::run_sweep_batch<gcs::PolPlusF32AccF64>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_BOOL_OR: return gcs::run_sweep_batch<gcs::PolBoolOr>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_PLUS_I64: return gcs::run_sweep_batch<gcs::PolPlusI64>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_MIN_PLUS_F32:
        return gcs::run_sweep_batch<gcs::PolMinPlusF32>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    case GCS_MIN_PLUS_F64:
        return gcs::run_sweep_batch<gcs::PolMinPlusF64>(d, x_dev, y_dev, nvec, workspace_dev, flags, s);
    }
    gcs::set_error("invalid policy");
    return GCS_EINVAL;
}

extern "C" gcs_status gcs_sweep_right_batch_scratch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec,
                                                    int32_t flags, void* stream)
{
    if (!d || nvec < 1 || nvec > gcs::kMaxBatch || !batch_flags_ok(flags) || (d->n_cols > 0 && !x_dev) ||
        (d->n_rows > 0 && !y_dev)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const size_t need = gcs::batch_workspace_bytes(gcs::batch_arena_rows(d, flags), d->n_rows, d->policy, nvec);
    if (need > kScratchBytes) {
        gcs::set_error("this batched sweep needs " + std::to_string(need) + " bytes of workspace; the fixed scratch "
                       "array holds " + std::to_string(kScratchBytes) + " (use gcs_sweep_right_batch with a "
                       "caller-provided workspace, or fewer vectors)");
        return GCS_ERANGE;
    }
    gcs::DeviceGuard guard(d->device);
    if (!guard.ok) {
        gcs::set_error("cannot select the upload's device");
        return GCS_EHIP;
    }
    scratch_setup(d->device);  // done at upload already; no-op then
    void* ws = nullptr;
    hipError_t se = hipSuccess;
    if (d->device >= 0 && d->device < kScratchDevices) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        ws = g_scratch_ptr[d->device];
        se = g_scratch_err[d->device];
    }
    if (!ws) {
        gcs::set_error(std::string("no scratch address for this device: ") +
                       (se != hipSuccess ? hipGetErrorString(se) : "device index out of range"));
        return GCS_EHIP;
    }
    return batch_dispatch(d, x_dev, y_dev, nvec, ws, flags, (hipStream_t)stream);
}

extern "C" int64_t gcs_sweep_launches(const gcs_device* d) { return d ? gcs::count_launches(d) : 0; }

static void release_events(gcs_device* d)
{
    for (hipEvent_t e : d->events) (void)hipEventDestroy(e);
    d->events.clear();
    d->profiling = false;
    d->prof_max = d->prof_used = 0;
}

// events per profiled sweep and timings per sweep
static int64_t prof_pairs(const gcs_device* d)
{
    return d->prof_mode == GCS_PROFILE_LEVEL_SPAN ? 1 : gcs::count_launches(d);
}

extern "C" gcs_status gcs_profile_begin(gcs_device* d, int64_t max_sweeps, int32_t mode)
{
    if (!d || max_sweeps <= 0 || (mode != GCS_PROFILE_LAUNCHES && mode != GCS_PROFILE_LEVEL_SPAN)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    release_events(d);
    d->prof_mode = mode;
    const int64_t per = 2 * prof_pairs(d);
    d->events.resize((size_t)(per * max_sweeps));
    for (auto& e : d->events) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            e = nullptr;
            d->events.erase(std::remove(d->events.begin(), d->events.end(), nullptr), d->events.end());
            release_events(d);
            return gcs::hip_fail(err, "hipEventCreate");
        }
    }
    d->prof_max = max_sweeps;
    d->prof_used = 0;
    d->profiling = true;
    return GCS_OK;
}

extern "C" gcs_status gcs_sweep_right_profiled(gcs_device* d, const void* x_dev, void* y_dev, void* stream)
{
    if (!d || !d->profiling) {
        gcs::set_error("gcs_profile_begin was not called");
        return GCS_ESTATE;
    }
    if (d->prof_used == d->prof_max) {
        gcs::set_error("more sweeps than gcs_profile_begin reserved");
        return GCS_ERANGE;
    }
    const int64_t per = 2 * prof_pairs(d);
    gcs_status st = sweep_dispatch(d, x_dev, y_dev, stream, d->events.data() + per * d->prof_used, 0,
                                   d->prof_mode == GCS_PROFILE_LEVEL_SPAN);
    if (st == GCS_OK) d->prof_used++;
    return st;
}

extern "C" gcs_status gcs_sweep_right_acc_profiled(gcs_device* d, const void* x_dev, void* y_dev, void* stream)
{
    if (!d || !d->profiling) {
        gcs::set_error("gcs_profile_begin was not called");
        return GCS_ESTATE;
    }
    if (d->prof_used == d->prof_max) {
        gcs::set_error("more sweeps than gcs_profile_begin reserved");
        return GCS_ERANGE;
    }
    const int64_t per = 2 * prof_pairs(d);
    gcs_status st = sweep_dispatch(d, x_dev, y_dev, stream, d->events.data() + per * d->prof_used, 1,
                                   d->prof_mode == GCS_PROFILE_LEVEL_SPAN);
    if (st == GCS_OK) d->prof_used++;
    return st;
}

extern "C" gcs_status gcs_profile_end(gcs_device* d, float* launch_ms, int64_t cap, int64_t* sweeps,
                                      int64_t* launches)
{
    if (!d || !d->profiling || !sweeps || !launches) {
        gcs::set_error("gcs_profile_begin was not called");
        return GCS_ESTATE;
    }
    gcs::DeviceGuard guard(d->device);
    const int64_t nl = prof_pairs(d), per = 2 * nl;
    *sweeps = d->prof_used;
    *launches = nl;
    if (cap < d->prof_used * nl || (cap > 0 && !launch_ms)) {
        release_events(d);
        gcs::set_error("launch_ms too small");
        return GCS_ERANGE;
    }
    for (int64_t s = 0; s < d->prof_used; ++s) {
        hipError_t err = hipEventSynchronize(d->events[per * s + per - 1]);
        if (err != hipSuccess) {
            release_events(d);
            return gcs::hip_fail(err, "hipEventSynchronize");
        }
        for (int64_t i = 0; i < nl; ++i) {
            float ms = 0;
            err = hipEventElapsedTime(&ms, d->events[per * s + 2 * i], d->events[per * s + 2 * i + 1]);
            if (err != hipSuccess) {
                release_events(d);
                return gcs::hip_fail(err, "hipEventElapsedTime");
            }
            launch_ms[s * nl + i] = ms;
        }
    }
    release_events(d);
    return GCS_OK;
}

extern "C" gcs_status gcs_bfs(gcs_device* d, const int64_t* sources_dev, int64_t n_sources, uint8_t* frontier_dev,
                              uint8_t* visited_dev, uint8_t* y_dev, int64_t* new_counts, int64_t cap,
                              int64_t* passes, void* stream)
{
    if (!d || !passes || n_sources < 0 || (n_sources > 0 && !sources_dev) || cap < 0 || (cap > 0 && !new_counts)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    if (d->policy != GCS_BOOL_OR || d->n_rows != d->n_cols) {
        gcs::set_error("gcs_bfs needs a square matrix uploaded with GCS_BOOL_OR");
        return GCS_ESTATE;
    }
    const int64_t n = d->n_rows;
    if (n > 0 && (!frontier_dev || !visited_dev || !y_dev)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    if (!guard.ok) {
        gcs::set_error("cannot select the upload's device");
        return GCS_EHIP;
    }
    hipStream_t s = (hipStream_t)stream;
    const int grid = (int)std::min<int64_t>(std::max<int64_t>((n + gcs::kBlock - 1) / gcs::kBlock, 1), 4096);
    gcs::bfs_clear_kernel<<<grid, gcs::kBlock, 0, s>>>(frontier_dev, visited_dev, n, d->counters);
    if (n_sources > 0)
        gcs::bfs_seed_kernel<<<(int)std::min<int64_t>((n_sources + gcs::kBlock - 1) / gcs::kBlock, 1024), gcs::kBlock,
                               0, s>>>(sources_dev, n_sources, frontier_dev, visited_dev, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return gcs::hip_fail(e, "bfs init launch");
    int64_t t = 0;
    for (;;) {
        if (t == cap) {
            gcs::set_error("BFS needs more passes than the counts array holds");
            *passes = t;
            return GCS_ERANGE;
        }
        gcs_status st = gcs::run_sweep<gcs::PolBoolOr>(d, frontier_dev, y_dev, s);
        if (st != GCS_OK) return st;
        const int slot = (int)(t & 1);
        gcs::bfs_update_kernel<<<grid, gcs::kBlock, 0, s>>>(y_dev, frontier_dev, visited_dev, n, d->counters, slot);
        e = hipGetLastError();
        if (e != hipSuccess) return gcs::hip_fail(e, "bfs update launch");
        // the pass's count and the failure flag (counters[3]) in one read
        e = hipMemcpyAsync(d->pinned, d->counters, 32, hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipMemcpyAsync (bfs count)");
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipStreamSynchronize (bfs)");
        int failed = 0;
        std::memcpy(&failed, d->pinned + 3, sizeof(int));
        if (failed) {
            (void)hipMemsetAsync(d->err, 0, sizeof(int), s);  // reported here, not again by gcs_device_check
            (void)hipStreamSynchronize(s);
            gcs::set_error("BFS pass " + std::to_string(t + 1) + ": its tail kernel timed out at a grid barrier; "
                           "the visited set is invalid");
            *passes = t;
            return GCS_ESTATE;
        }
        const int64_t c = d->pinned[slot];
        new_counts[t++] = c;
        if (c == 0) break;
    }
    *passes = t;
    return GCS_OK;
}

extern "C" gcs_status gcs_device_check(gcs_device* d, void* stream)
{
    if (!d) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(d->pinned, d->err, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return gcs::hip_fail(e, "gcs_device_check");
    int flag;
    std::memcpy(&flag, d->pinned, sizeof(int));
    if (flag) {
        e = hipMemsetAsync(d->err, 0, sizeof(int), s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        gcs::set_error("a sweep's tail kernel timed out at its grid barrier; its results are invalid");
        return GCS_ESTATE;
    }
    return GCS_OK;
}

extern "C" void gcs_free_device(gcs_device* d)
{
    if (!d) return;
    release_events(d);
    if (d->pinned) (void)hipHostFree(d->pinned);
    delete d;
}

// ------------------------------------------------------------ column groups swept together

struct gcs_group {
    gcs_policy policy;
    int device;
    int64_t n_rows, n_cols;
    std::vector<gcs_device*> devs;
    int64_t n_launch = 0;                 // level launches: the largest L + 1 of the groups
    std::vector<int64_t> ent_off;         // launch k (1-based) uses entries [ent_off[k-1], ent_off[k])
    std::vector<int64_t> vblocks;         // virtual blocks of launch k at index k-1
    int64_t leaf_blocks = 0, n_leaf = 0;  // leaf table: n_leaf entries (groups with terminals or rows)
    const gcs::GroupEntry* ents = nullptr;
    const gcs::LeafEntry* leaf = nullptr;
    void* const* accs = nullptr;
    // profiling: one pair of events around the level launches of each sweep
    std::vector<hipEvent_t> events;
    int64_t prof_max = 0, prof_used = 0;
    bool profiling = false;
};

namespace {

bool group_policy_ok(gcs_policy p)
{
    return p == GCS_PLUS_F64 || p == GCS_PLUS_F32 || p == GCS_PLUS_F32_ACC_F64 || p == GCS_PLUS_I64;
}

// entries of every launch, the leaf table and the accumulator pointers
struct GroupPlan {
    std::vector<gcs::GroupEntry> ents;
    std::vector<int64_t> ent_off, vblocks;
    std::vector<gcs::LeafEntry> leaf;
    std::vector<void*> accs;
    int64_t n_launch = 0, leaf_blocks = 0;
    size_t off_leaf = 0, off_accs = 0, total = 0;
};

gcs_status group_plan(gcs_device* const* devs, int32_t n, GroupPlan& pl)
{
    if (!devs || n < 1) {
        gcs::set_error("invalid argument: no device handles");
        return GCS_EINVAL;
    }
    for (int32_t i = 0; i < n; ++i) {
        const gcs_device* d = devs[i];
        if (!d) {
            gcs::set_error("invalid argument: null device handle");
            return GCS_EINVAL;
        }
        if (!group_policy_ok(d->policy) || d->policy != devs[0]->policy || d->n_rows != devs[0]->n_rows ||
            d->n_cols != devs[0]->n_cols || d->device != devs[0]->device) {
            gcs::set_error("group sweeps take uploads of one matrix shape, one device and one plus-times policy "
                           "(fp64, fp32, fp32->fp64, int64)");
            return GCS_EINVAL;
        }
    }
    // each group needs its own arena and accumulators: workspaces must not overlap
    const size_t eb = gcs::elem_bytes(devs[0]->policy);
    std::vector<std::pair<uintptr_t, uintptr_t>> ws;
    for (int32_t i = 0; i < n; ++i) {
        const gcs_device* d = devs[i];
        const uintptr_t b = (uintptr_t)d->counters;
        const uintptr_t e = (uintptr_t)d->acc + (size_t)gcs::kSlices * d->n_rows * eb;
        ws.push_back({b, e});
    }
    std::sort(ws.begin(), ws.end());
    for (size_t i = 1; i < ws.size(); ++i)
        if (ws[i].first < ws[i - 1].second) {
            gcs::set_error("group sweeps need a separate workspace per upload (these overlap)");
            return GCS_EINVAL;
        }
    for (int32_t i = 0; i < n; ++i) pl.n_launch = std::max<int64_t>(pl.n_launch, devs[i]->L + 1);
    pl.ent_off.assign((size_t)pl.n_launch + 1, 0);
    pl.vblocks.assign((size_t)pl.n_launch, 0);
    for (int64_t k = 1; k <= pl.n_launch; ++k) {
        int64_t vb = 0;
        for (int32_t i = 0; i < n; ++i) {
            gcs_device* d = devs[i];
            if (k > d->L + 1) continue;
            const gcs::LevelArgs& a = d->largs[k - 1];
            const int64_t nb = gcs::vblocks(a);
            if (nb == 0) continue;
            gcs::GroupEntry e{};
            e.a = a;
            e.arena = d->arena;
            e.acc = d->acc;
            e.block0 = (int32_t)vb;
            pl.ents.push_back(e);
            vb += nb;
        }
        if (vb >= (int64_t)INT32_MAX) {
            gcs::set_error("a group launch exceeds 2^31 workgroups");
            return GCS_ERANGE;
        }
        pl.vblocks[k - 1] = vb;
        pl.ent_off[k] = (int64_t)pl.ents.size();
    }
    const int64_t per = (int64_t)gcs::kBlock * gcs::kGroupLeafItems;
    for (int32_t i = 0; i < n; ++i) {
        gcs_device* d = devs[i];
        const int64_t n_acc = (int64_t)gcs::kSlices * d->n_rows;
        const int64_t items = std::max<int64_t>(d->alpha, n_acc);
        gcs::LeafEntry e{};
        e.tcol = d->tcol;
        e.tval = d->tval;
        e.V = d->V;
        e.T = d->arena;
        e.acc = d->acc;
        e.alpha = (int32_t)d->alpha;
        e.n_acc = (int32_t)n_acc;
        e.block0 = (int32_t)pl.leaf_blocks;
        if (items == 0) continue;
        pl.leaf.push_back(e);
        pl.leaf_blocks += (items + per - 1) / per;
    }
    for (int32_t i = 0; i < n; ++i) pl.accs.push_back(devs[i]->acc);
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    pl.off_leaf = al(pl.ents.size() * sizeof(gcs::GroupEntry));
    pl.off_accs = pl.off_leaf + al(pl.leaf.size() * sizeof(gcs::LeafEntry));
    pl.total = pl.off_accs + al(pl.accs.size() * sizeof(void*));
    return GCS_OK;
}

void release_group_events(gcs_group* g)
{
    for (hipEvent_t e : g->events) (void)hipEventDestroy(e);
    g->events.clear();
    g->profiling = false;
    g->prof_max = g->prof_used = 0;
}

template <class P>
gcs_status run_group(gcs_group* g, const void* xv, void* yv, int32_t accumulate, hipStream_t s, hipEvent_t* ev)
{
    using namespace gcs;
    const int32_t n_leaf = (int32_t)g->n_leaf;
    if (g->leaf_blocks > 0)
        leaf_group_kernel<P><<<(unsigned)g->leaf_blocks, kBlock, 0, s>>>(g->leaf, n_leaf,
                                                                         (const typename P::X*)xv);
    if (ev) (void)hipEventRecord(ev[0], s);
    for (int64_t k = 1; k <= g->n_launch; ++k) {
        const int64_t e0 = g->ent_off[k - 1], e1 = g->ent_off[k];
        if (e1 == e0) continue;
        level_group_kernel<P><<<(unsigned)g->vblocks[k - 1], kBlock, 0, s>>>(g->ents + e0, (int32_t)(e1 - e0));
    }
    if (ev) (void)hipEventRecord(ev[1], s);
    if (g->n_rows > 0) {
        const int64_t grid = std::min<int64_t>((g->n_rows + kBlock - 1) / kBlock, 1 << 16);
        reduce_group_kernel<P><<<(unsigned)grid, kBlock, 0, s>>>(g->accs, (int32_t)g->devs.size(),
                                                                 (typename P::Y*)yv, (int32_t)g->n_rows, accumulate);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "group sweep launch");
    return GCS_OK;
}

}  // namespace

extern "C" gcs_status gcs_group_layout(gcs_device* const* devs, int32_t n, size_t* table_bytes)
{
    if (!table_bytes) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    GroupPlan pl;
    if (gcs_status st = group_plan(devs, n, pl)) return st;
    *table_bytes = pl.total;
    return GCS_OK;
}

extern "C" gcs_status gcs_group_create(gcs_device* const* devs, int32_t n, void* table_dev, size_t table_bytes,
                                       void* stream, gcs_group** out)
{
    if (!out || !table_dev) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    *out = nullptr;
    try {
        GroupPlan pl;
        if (gcs_status st = group_plan(devs, n, pl)) return st;
        if (table_bytes < pl.total || ((uintptr_t)table_dev & 255)) {
            gcs::set_error("group table smaller than gcs_group_layout reports, or not 256-byte aligned");
            return GCS_EINVAL;
        }
        gcs::DeviceGuard guard(devs[0]->device);
        if (!guard.ok) {
            gcs::set_error("cannot select the uploads' device");
            return GCS_EHIP;
        }
        hipStream_t s = (hipStream_t)stream;
        std::vector<unsigned char> img(pl.total, 0);
        if (!pl.ents.empty()) std::memcpy(img.data(), pl.ents.data(), pl.ents.size() * sizeof(gcs::GroupEntry));
        if (!pl.leaf.empty())
            std::memcpy(img.data() + pl.off_leaf, pl.leaf.data(), pl.leaf.size() * sizeof(gcs::LeafEntry));
        std::memcpy(img.data() + pl.off_accs, pl.accs.data(), pl.accs.size() * sizeof(void*));
        hipError_t e = hipMemcpyAsync(table_dev, img.data(), pl.total, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipMemcpyAsync (group table)");
        auto* g = new gcs_group();
        g->policy = devs[0]->policy;
        g->device = devs[0]->device;
        g->n_rows = devs[0]->n_rows;
        g->n_cols = devs[0]->n_cols;
        g->devs.assign(devs, devs + n);
        g->n_launch = pl.n_launch;
        g->ent_off = pl.ent_off;
        g->vblocks = pl.vblocks;
        g->leaf_blocks = pl.leaf_blocks;
        g->n_leaf = (int64_t)pl.leaf.size();
        auto* base = (unsigned char*)table_dev;
        g->ents = (const gcs::GroupEntry*)base;
        g->leaf = (const gcs::LeafEntry*)(base + pl.off_leaf);
        g->accs = (void* const*)(base + pl.off_accs);
        *out = g;
        return GCS_OK;
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of host memory");
        return GCS_ENOMEM;
    }
}

static gcs_status group_dispatch(gcs_group* g, const void* x_dev, void* y_dev, int32_t accumulate, void* stream,
                                 hipEvent_t* ev)
{
    if (!g || (g->n_cols > 0 && !x_dev) || (g->n_rows > 0 && !y_dev) || (accumulate & ~1)) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(g->device);
    if (!guard.ok) {
        gcs::set_error("cannot select the uploads' device");
        return GCS_EHIP;
    }
    hipStream_t s = (hipStream_t)stream;
    switch (g->policy) {
    case GCS_PLUS_F64: return run_group<gcs::PolPlusF64>(g, x_dev, y_dev, accumulate, s, ev);
    case GCS_PLUS_F32: return run_group<gcs::PolPlusF32>(g, x_dev, y_dev, accumulate, s, ev);
    case GCS_PLUS_F32_ACC_F64: return run_group<gcs::PolPlusF32AccF64>(g, x_dev, y_dev, accumulate, s, ev);
    case GCS_PLUS_I64: return run_group<gcs::PolPlusI64>(g, x_dev, y_dev, accumulate, s, ev);
    default: break;
    }
    gcs::set_error("corrupt group handle");
    return GCS_ESTATE;
}

extern "C" gcs_status gcs_group_sweep_right(gcs_group* g, const void* x_dev, void* y_dev, int32_t accumulate,
                                            void* stream)
{
    return group_dispatch(g, x_dev, y_dev, accumulate, stream, nullptr);
}

extern "C" int64_t gcs_group_launches(const gcs_group* g)
{
    if (!g) return 0;
    int64_t n = (g->leaf_blocks > 0 ? 1 : 0) + (g->n_rows > 0 ? 1 : 0);
    for (int64_t k = 1; k <= g->n_launch; ++k) n += g->ent_off[k] > g->ent_off[k - 1] ? 1 : 0;
    return n;
}

extern "C" gcs_status gcs_group_profile_begin(gcs_group* g, int64_t max_sweeps)
{
    if (!g || max_sweeps < 1) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(g->device);
    release_group_events(g);
    g->events.resize((size_t)(2 * max_sweeps));
    for (auto& e : g->events) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) {
            g->events.clear();
            return gcs::hip_fail(err, "hipEventCreate");
        }
    }
    g->prof_max = max_sweeps;
    g->prof_used = 0;
    g->profiling = true;
    return GCS_OK;
}

extern "C" gcs_status gcs_group_sweep_right_profiled(gcs_group* g, const void* x_dev, void* y_dev,
                                                     int32_t accumulate, void* stream)
{
    if (!g || !g->profiling) {
        gcs::set_error("gcs_group_profile_begin was not called");
        return GCS_ESTATE;
    }
    if (g->prof_used == g->prof_max) {
        gcs::set_error("more sweeps than gcs_group_profile_begin reserved");
        return GCS_ERANGE;
    }
    gcs_status st = group_dispatch(g, x_dev, y_dev, accumulate, stream, g->events.data() + 2 * g->prof_used);
    if (st == GCS_OK) g->prof_used++;
    return st;
}

extern "C" gcs_status gcs_group_profile_end(gcs_group* g, float* level_ms, int64_t cap, int64_t* sweeps)
{
    if (!g || !g->profiling || !sweeps) {
        gcs::set_error("gcs_group_profile_begin was not called");
        return GCS_ESTATE;
    }
    gcs::DeviceGuard guard(g->device);
    if (cap < g->prof_used || (g->prof_used > 0 && !level_ms)) {
        gcs::set_error("level_ms holds fewer entries than profiled sweeps");
        return GCS_ERANGE;
    }
    for (int64_t i = 0; i < g->prof_used; ++i) {
        hipError_t e = hipEventSynchronize(g->events[2 * i + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&level_ms[i], g->events[2 * i], g->events[2 * i + 1]);
        if (e != hipSuccess) {
            release_group_events(g);
            return gcs::hip_fail(e, "group profile events");
        }
    }
    *sweeps = g->prof_used;
    release_group_events(g);
    return GCS_OK;
}

extern "C" void gcs_group_free(gcs_group* g)
{
    if (!g) return;
    {
        gcs::DeviceGuard guard(g->device);
        release_group_events(g);
    }
    delete g;
}
