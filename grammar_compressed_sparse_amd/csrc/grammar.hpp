// Host-side grammar: CSRV encoding, RePair, levels, pass-through completion and
// the level-bucketed layout that the device sweep consumes.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "gcs.h"

namespace gcs {

void set_error(const std::string& msg);
int resolve_threads(int requested);

// RePair on one tile: rows of terminal symbols, concatenated in `seq` with row
// offsets `row_off` (nrows + 1).  New nonterminals are numbered nt_base + i in
// creation order (so rule i only references symbols < nt_base + i).  On return
// rule_a/rule_b hold the rules and `seq`/`row_len` the final row sequences
// (rows concatenated).  Returns false on allocation failure.
struct RePairResult {
    std::vector<int32_t> rule_a, rule_b;
    std::vector<int32_t> seq;
    std::vector<int64_t> row_len;
};
bool repair_tile(const std::vector<int32_t>& seq_in, const std::vector<int64_t>& row_off, int32_t nt_base,
                 RePairResult& out);
// The same contract, round-based (rounds.hpp): many non-overlapping pairs per
// pass; the host form of the device builder.
bool repair_rounds_tile(const std::vector<int32_t>& seq_in, const std::vector<int64_t>& row_off, int32_t nt_base,
                        RePairResult& out);

// Column slices: every level is cut into kSlices contiguous pieces by global
// first-column thresholds, one piece per XCD of the device.
constexpr int kSlices = 8;

struct Level {
    int64_t nb;        // binary nodes (rules whose level is k)
    int64_t npt;       // pass-through nodes
    int64_t child_off; // first child pair of this level
    int64_t pt_off;    // first pass-through source of this level
    int64_t reserved;
    int64_t base;      // arena offset of this level's values (level 0: terminal array)
    int64_t grp_off;   // first emission group of this level
    int64_t ngrp;
    // slice x covers binary nodes [bsl[x], bsl[x+1]), pass-through nodes
    // [psl[x], psl[x+1]) and emission groups grp_off + [gsl[x], gsl[x+1])
    int64_t bsl[kSlices + 1], psl[kSlices + 1], gsl[kSlices + 1];
};

struct Grammar {
    int64_t n_rows = 0, n_cols = 0, nnz = 0, n_tiles = 1;
    std::vector<double> V;                 // distinct nonzero values, ascending
    std::vector<int32_t> tcol, tval;       // terminal t = <tval+1, tcol+1>, sorted by (col, val)
    std::vector<int32_t> ra, rb;           // rules; symbol < alpha = terminal, else alpha + rule
    std::vector<int64_t> c_off;            // n_rows + 1
    std::vector<int32_t> c_sym;
    // levels (Eq. 3.1) and completion (section 4.2)
    std::vector<int32_t> lvl, plast;       // per rule
    int32_t L = 0;
    // layout (section 4.3)
    std::vector<Level> lv;                 // 0..L
    std::vector<int32_t> child;            // 2 per binary node
    std::vector<int32_t> ptsrc;            // arena offset of each pass-through node's source
    std::vector<int32_t> erow, eoff, epos; // emission groups, ordered by (level, slice, row)
    int32_t col_cut[kSlices + 1] = {};     // slice x = first columns [col_cut[x], col_cut[x+1])
    int64_t wmax = 0, pt_total = 0, buf_a = 0, buf_b = 0, arena = 0;
    double t_csrv = 0, t_repair = 0, t_layer = 0;

    int64_t alpha() const { return (int64_t)tcol.size(); }
    int64_t nrules() const { return (int64_t)ra.size(); }
};

// Levels, pass-through completion and layout from (tcol/tval, ra/rb, C).
gcs_status finish_layout(Grammar& g, int threads);

// CSRV encoding of a CSR input (section 2, 'CSRV'): the checks, V and the
// compacted terminal alphabet; term_id(k) is the terminal of nonzero k (-1 for
// a stored zero, which is dropped).
struct Csrv {
    const gcs_csr_view* m = nullptr;
    int kind = 0;
    int32_t i8_index[256];             // int8 value + 128 -> index into V (-1: zero)
    bool small_v = true;               // |V| <= 64: per-column bit masks
    bool has_zeros = false;            // some stored entry is zero
    std::vector<int64_t> cbase;        // small_v: first terminal of each column (n_cols + 1)
    std::vector<uint64_t> cmask;       // small_v: value indices present in each column
    std::vector<int64_t> tkeys;        // otherwise: sorted keys col * |V| + value index
    const std::vector<double>* V = nullptr;
    int64_t nV = 0;
    int32_t vindex(int64_t k) const;
    int32_t term_id(int64_t k) const;
};
gcs_status csrv_encode(const gcs_csr_view* m, int threads, Grammar& g, Csrv& enc);

}  // namespace gcs

struct gcs_grammar {
    gcs::Grammar g;
};
