"""Test aids (not the oracle): CSRV strings, grammar expansion, the CPU
W-array sweep over the grammar, and a host emulator of the uploaded layout.

Page: "Right Multiplication on Grammar-Compressed Matrices" (arXiv
2607.24971v1).  These helpers localise bugs (builder vs layout vs kernels);
parity of products is always judged against ``oracle``.
"""
from __future__ import annotations

import threading

import numpy as np

# pytest's capture manager, set by conftest at configure time, so that the
# progress lines of long GPU tests reach the terminal while the test runs
CAPTURE = None
_PROGRESS_LOCK = threading.Lock()


def progress(msg):
    """Print a progress line at once, past pytest's output capture: a test
    that prints nothing for minutes is indistinguishable from a hung one.
    Worker threads may call it (one at a time: capture is process-wide)."""
    with _PROGRESS_LOCK:
        if CAPTURE is not None:
            with CAPTURE.global_and_fixture_disabled():
                print(msg, flush=True)
        else:
            print(msg, flush=True)


def csr_from_dense(M):
    rp, cl, vl = [0], [], []
    for row in M:
        for j, a in enumerate(row):
            if a != 0:
                cl.append(j)
                vl.append(a)
        rp.append(len(cl))
    return np.array(rp, np.int64), np.array(cl, np.int32), np.array(vl, np.float64)


def terminal_ids(ex):
    """(col, value index) -> terminal id, from an exported grammar."""
    return {(int(c), int(v)): t for t, (c, v) in enumerate(zip(ex["term_col"], ex["term_val"]))}


def csrv_rows(row_ptr, col, val, ex):
    """The CSRV string of section 2 (Eq. 2.2), one terminal list per row, with
    terminals as the grammar's ids (<l, j> compacted)."""
    V = list(ex["values"])
    vindex = {v: i for i, v in enumerate(V)}
    tid = terminal_ids(ex)
    rows = []
    for r in range(len(row_ptr) - 1):
        seq = []
        for k in range(row_ptr[r], row_ptr[r + 1]):
            v = 1.0 if val is None else float(val[k])
            if v != 0.0:
                seq.append(tid[(int(col[k]), vindex[v])])
        rows.append(seq)
    return rows


def expansions(ex):
    """Expansion of every rule to its terminal string (iterative, topological)."""
    a = len(ex["term_col"])
    exp = []
    for A, B in zip(ex["rule_a"], ex["rule_b"]):
        ea = [int(A)] if A < a else exp[A - a]
        eb = [int(B)] if B < a else exp[B - a]
        exp.append(ea + eb)
    return exp


def expand_rows(ex):
    a = len(ex["term_col"])
    exp = expansions(ex)
    out = []
    co, cs = ex["c_off"], ex["c_sym"]
    for r in range(len(co) - 1):
        seq = []
        for s in cs[co[r]:co[r + 1]]:
            seq.extend([int(s)] if s < a else exp[s - a])
        out.append(seq)
    return out


def levels_eq31(ex):
    """Eq. (3.1) recomputed: lvl(terminal) = 0, lvl(N->AB) = 1 + max."""
    a = len(ex["term_col"])
    lv = []
    for A, B in zip(ex["rule_a"], ex["rule_b"]):
        la = 0 if A < a else lv[A - a]
        lb = 0 if B < a else lv[B - a]
        lv.append(1 + max(la, lb))
    return np.array(lv, np.int64)


def live_widths(ex):
    """w_k = |live(k)| from the uncompleted grammar: nodes of level k plus the
    nodes of lower levels that a nonterminal parent above level k still needs
    (live(k) = {v: lvl v = k} U {v: lvl v < k <= P(v) - 1})."""
    a = len(ex["term_col"])
    lv = levels_eq31(ex)
    R = len(lv)
    P = np.zeros(R, np.int64)
    for i, (A, B) in enumerate(zip(ex["rule_a"], ex["rule_b"])):
        for c in (A, B):
            if c >= a:
                P[c - a] = max(P[c - a], lv[i])
    L = int(lv.max()) if R else 0
    w = np.zeros(L + 1, np.int64)
    for v in range(R):
        w[lv[v]] += 1
        for k in range(lv[v] + 1, P[v]):
            w[k] += 1
    return w, lv, P


def w_array_sweep(ex, x, op="plus"):
    """The mm-repair CPU right product (section 2, Lemma 2.1/2.2): W[i] =
    cv(A_i) + cv(B_i) in index order, y[r] = combination of its C symbols."""
    a = len(ex["term_col"])
    V = ex["values"]
    if op == "plus":
        T = [V[v] * x[c] for c, v in zip(ex["term_col"], ex["term_val"])]
        comb, zero = (lambda p, q: p + q), 0.0
    else:
        T = [bool(x[c]) for c in ex["term_col"]]
        comb, zero = (lambda p, q: p or q), False
    W = []
    for A, B in zip(ex["rule_a"], ex["rule_b"]):
        W.append(comb(T[A] if A < a else W[A - a], T[B] if B < a else W[B - a]))
    co, cs = ex["c_off"], ex["c_sym"]
    y = []
    for r in range(len(co) - 1):
        acc = zero
        for s in cs[co[r]:co[r + 1]]:
            acc = comb(acc, T[s] if s < a else W[s - a])
        y.append(acc)
    return y


def emulate_layout(lay, ex, x, op="plus", dtype=np.float64, poison=True):
    """Executes the exported device layout on the host exactly as the kernels
    do: leaf, then per level binary nodes, pass-through ranges and emission of
    the previous level.  With ``poison`` the buffer of level k-2 is filled
    with NaN (or a sentinel) before level k writes it, so any read that is not
    from level k-1 or the terminal array corrupts the result."""
    a = len(ex["term_col"])
    arena = np.zeros(max(lay["arena"], 1), dtype)
    V = np.asarray(ex["values"])
    tc, tv = ex["term_col"], ex["term_val"]
    if op == "plus":
        arena[:a] = (V[tv] * np.asarray(x, np.float64)[tc]).astype(dtype)
        comb = np.add
        bad = np.nan if np.issubdtype(dtype, np.floating) else -(1 << 60)
    else:
        arena[:a] = (np.asarray(x)[tc] != 0).astype(dtype)
        comb = np.bitwise_or
        bad = 0x80
    n = len(ex["c_off"]) - 1
    S = lay["slices"].shape[2] - 1
    acc = np.zeros((S, n), dtype)  # per-slice row accumulators
    meta = lay["level_meta"]
    L = meta.shape[0] - 1

    def emit(level):
        nb_, npt_, co_, ro_, nr_, base_, g0, ng = meta[level]
        gsl = lay["slices"][level, 2]
        assert gsl[0] == 0 and gsl[S] == ng
        for x in range(S):
            for g in range(g0 + gsl[x], g0 + gsl[x + 1]):
                e0, e1 = lay["eoff"][g], lay["eoff"][g + 1]
                s = arena[lay["epos"][e0]]
                for e in range(e0 + 1, e1):
                    s = comb(s, arena[lay["epos"][e]])
                acc[x, lay["erow"][g]] = comb(acc[x, lay["erow"][g]], s)

    for k in range(1, L + 2):
        if k <= L:
            nb, npt, co, ro, nr, base, _, _ = meta[k]
            if poison:
                width = lay["buf_b"] - lay["buf_a"]
                arena[base:base + width] = bad
            ch = lay["child"][co:co + nb]
            vals = comb(arena[ch[:, 0]], arena[ch[:, 1]])
            ptv = arena[lay["ptsrc"][ro:ro + npt]]
            emit(k - 1)  # reads level k-1 before level k overwrites nothing of it
            arena[base:base + nb] = vals
            arena[base + nb:base + nb + npt] = ptv
        else:
            emit(k - 1)
    y = acc[0].copy()
    for x in range(1, S):
        y = comb(y, acc[x])
    return y


def we_grammar_arrays(we):
    """The worked example's (C, R, V) of Eq. (2.3)-(2.4) as gcs_grammar_from_rules
    arrays: terminals are numbered in order of first appearance in R."""
    terms = []
    idx = {}
    for A, B in we["R"]["rules"]:
        for s in (A, B):
            if "t" in s:
                key = tuple(s["t"])
                if key not in idx:
                    idx[key] = len(terms)
                    terms.append(key)
    alpha = len(terms)

    def enc(s):
        return idx[tuple(s["t"])] if "t" in s else alpha + s["N"] - 1

    ra = [enc(A) for A, B in we["R"]["rules"]]
    rb = [enc(B) for A, B in we["R"]["rules"]]
    roots = we["C"]["row_roots"]
    c_off = list(range(len(roots) + 1))
    c_sym = [alpha + r - 1 for r in roots]
    term_col = [j - 1 for (l, j) in terms]
    term_val = [l - 1 for (l, j) in terms]
    return dict(n_rows=len(roots), n_cols=7, values=we["V"]["values"], term_col=term_col, term_val=term_val,
                rule_a=ra, rule_b=rb, c_off=c_off, c_sym=c_sym)
