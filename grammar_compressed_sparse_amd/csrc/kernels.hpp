// Device code of the sweep for gfx950 (CDNA4): policies, launch arguments and
// kernels.  Host code (upload, launch sequence, C ABI) is in sweep.hip.
//
// Page: "Right Multiplication on Grammar-Compressed Matrices: A Streaming,
// Memory-Bounded GPU Engine" (arXiv 2607.24971v1), section 4.3 (streaming,
// double-buffered sweep; Listing 1), section 5 (leaf / combine / emit
// policies), section 4.4 "Batched evaluation (SpMM)".
//
// A sweep: leaf_kernel (terminal array T, clears the row accumulators),
// level_kernel once per wide level k (binary nodes and pass-through copies of
// level k, emission of level k-1 into per-slice row accumulators, by teams
// or by chunks of short groups), then one cooperative tail_kernel for the
// narrow top levels, the last emission and the reduction of the slice
// accumulators into y.  Child, source and root indices are absolute arena
// offsets ([T | buffer A | buffer B], level parity applied), so one read,
// fetch(arena, c), serves a terminal and a node of the level below alike
// (the Boolean policy keeps terminals as bits).  Every part of a level is cut
// into kSlices column slices and workgroup b serves slice b % kSlices, which
// keeps a slice on one XCD and its gathers in that XCD's L2.  Emission is
// deterministic (each (level, slice, row) group is combined in a fixed
// order); the Boolean and tropical policies emit straight into y instead.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "grammar.hpp"

namespace gcs {

// ---------------------------------------------------------------- policies
// poison(): what y holds after a sweep whose tail grid barrier timed out (a
// value no correct sweep produces: NaN, 0xFF for a Boolean, INT64_MIN)

struct PolPlusF64 {
    using X = double;  // x element
    using A = double;  // arena (T and level buffers)
    using Y = double;  // y element
    using W = double;  // V element on the device
    __device__ static A leaf(W v, X x) { return v * x; }
    __device__ static A comb(A a, A b) { return a + b; }
    __device__ static Y emit(Y y, A s) { return y + s; }
    __device__ static Y yzero() { return 0.0; }
    __device__ static A ident() { return 0.0; }
    __device__ static Y poison() { return __builtin_nan(""); }
};
struct PolPlusF32 {
    using X = float;
    using A = float;
    using Y = float;
    using W = float;
    __device__ static A leaf(W v, X x) { return v * x; }
    __device__ static A comb(A a, A b) { return a + b; }
    __device__ static Y emit(Y y, A s) { return y + s; }
    __device__ static Y yzero() { return 0.0f; }
    __device__ static A ident() { return 0.0f; }
    __device__ static Y poison() { return __builtin_nanf(""); }
};
struct PolPlusF32AccF64 {
    using X = float;
    using A = double;
    using Y = double;
    using W = double;
    __device__ static A leaf(W v, X x) { return v * (double)x; }
    __device__ static A comb(A a, A b) { return a + b; }
    __device__ static Y emit(Y y, A s) { return y + s; }
    __device__ static Y yzero() { return 0.0; }
    __device__ static A ident() { return 0.0; }
    __device__ static Y poison() { return __builtin_nan(""); }
};
struct PolBoolOr {
    using X = uint8_t;
    using A = uint8_t;
    using Y = uint8_t;
    using W = uint8_t;
    __device__ static A leaf(W, X x) { return x != 0; }
    __device__ static A comb(A a, A b) { return a | b; }
    __device__ static Y emit(Y y, A s) { return y | s; }
    __device__ static Y yzero() { return 0; }
    __device__ static A ident() { return 0; }
    __device__ static Y poison() { return 0xFF; }
};
struct PolPlusI64 {
    using X = int64_t;
    using A = int64_t;
    using Y = int64_t;
    using W = int64_t;
    __device__ static A leaf(W v, X x) { return v * x; }
    __device__ static A comb(A a, A b) { return a + b; }
    __device__ static Y emit(Y y, A s) { return y + s; }
    __device__ static Y yzero() { return 0; }
    __device__ static A ident() { return 0; }
    __device__ static Y poison() { return INT64_MIN; }
};

// tropical (min, +): leaf = matrix value + x[j], combine = min, identity
// +infinity (section 5); exact, since min never rounds and every sum is
// formed once, in the leaf
struct PolMinPlusF32 {
    using X = float;
    using A = float;
    using Y = float;
    using W = float;
    __device__ static A leaf(W v, X x) { return v + x; }
    __device__ static A comb(A a, A b) { return b < a ? b : a; }
    __device__ static Y emit(Y y, A s) { return s < y ? s : y; }
    __device__ static Y yzero() { return __builtin_huge_valf(); }
    __device__ static A ident() { return __builtin_huge_valf(); }
    __device__ static Y poison() { return __builtin_nanf(""); }
};
struct PolMinPlusF64 {
    using X = double;
    using A = double;
    using Y = double;
    using W = double;
    __device__ static A leaf(W v, X x) { return v + x; }
    __device__ static A comb(A a, A b) { return b < a ? b : a; }
    __device__ static Y emit(Y y, A s) { return s < y ? s : y; }
    __device__ static Y yzero() { return __builtin_huge_val(); }
    __device__ static A ident() { return __builtin_huge_val(); }
    __device__ static Y poison() { return __builtin_nan(""); }
};

// Policies whose emission goes straight into y because the combination is
// idempotent and exact, so its result does not depend on the order of the
// writers: OR (a lane whose partial OR is 1 stores 1; racing writers write
// the same byte) and min (an atomic minimum).  Their sweep has no slice
// accumulators and no final reduction.  direct(p, v) folds a lane's partial
// v into *p; the identity is a no-op.
template <class P>
constexpr bool kDirectEmit = false;
template <>
constexpr bool kDirectEmit<PolBoolOr> = true;
template <>
constexpr bool kDirectEmit<PolMinPlusF32> = true;
template <>
constexpr bool kDirectEmit<PolMinPlusF64> = true;

__device__ __forceinline__ void direct(uint8_t* p, uint8_t v)
{
    if (v) *p = 1;
}
// IEEE order of non-negative floats is the order of their bits as signed
// integers, and of negative floats the reverse order of their bits as
// unsigned integers, so min is an integer min or an unsigned max.  A value
// no smaller than what y holds changes nothing and skips the atomic (y only
// decreases, so a stale read can only let an atomic through).
__device__ __forceinline__ void direct(float* p, float v)
{
    if (!(v < __builtin_huge_valf())) return;
    if (!(v < __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) return;
    if (v >= 0.0f) atomicMin((int*)p, __float_as_int(v));
    else atomicMax((unsigned int*)p, __float_as_uint(v));
}
__device__ __forceinline__ void direct(double* p, double v)
{
    if (!(v < __builtin_huge_val())) return;
    if (!(v < __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) return;
    if (v >= 0.0) atomicMin((long long*)p, __double_as_longlong(v));
    else atomicMax((unsigned long long*)p, (unsigned long long)__double_as_longlong(v));
}

// The Boolean sweep keeps its terminals one bit each: terminal c is bit c % 8
// of byte c / 8 of T (the leaf launch packs 64 of them per wave with a
// ballot).  The terminal array is most of what a Boolean sweep gathers from;
// packed, it is an eighth of the size and an XCD's share of it stays in that
// XCD's L2.  Level values stay one byte each (0 or 1), and the packed words,
// ceil(alpha / 64) * 8 bytes, end before the level buffers, which start at
// alpha rounded up to a multiple of 64.
template <class P>
constexpr bool kBitTerms = false;
template <>
constexpr bool kBitTerms<PolBoolOr> = true;

// the value of arena reference c (terminals below alpha)
template <class P>
__device__ __forceinline__ typename P::A fetch(const typename P::A* __restrict__ arena, int32_t c, int32_t alpha)
{
    if constexpr (kBitTerms<P>) {
        const bool t = c < alpha;
        return (typename P::A)((arena[t ? c >> 3 : c] >> (t ? c & 7 : 0)) & 1);
    } else {
        return arena[c];
    }
}

// lane exchange inside a wave for every arena type
__device__ inline double xchg(double v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline float xchg(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline int64_t xchg(int64_t v, int m) { return __shfl_xor((long long)v, m, 64); }
__device__ inline uint8_t xchg(uint8_t v, int m) { return (uint8_t)__shfl_xor((int)v, m, 64); }

// An empty asm statement that takes v as an input: v must be computed before
// this point on every lane, which keeps the compiler from sinking a lane's
// independent loads into the masked store that consumes them (one load in
// flight at a time instead of all of them).  Emits no instruction.
template <class T>
__device__ __forceinline__ void issue_before(const T& v)
{
    if constexpr (sizeof(T) == 8) {
        asm volatile("" ::"v"(v));
    } else {
        asm volatile("" ::"v"((int32_t)v));
    }
}

// ---------------------------------------------------------------- kernels

constexpr int kBlock = 256;
// terminals (and accumulators) per lane of a large leaf launch; a small one
// keeps one per lane so that its grid still covers the device
constexpr int kLeafItems = 4;
constexpr int64_t kLeafMultiMin = (int64_t)kLeafItems * kBlock * 2048;
constexpr int kBinItems = 4;  // binary nodes per lane (independent gathers in flight)
constexpr int kEmitItems = 2;  // roots per emission lane loaded before the first combine
constexpr int kTailBlock = 1024;  // lanes per workgroup of the persistent tail
constexpr size_t kFlatLdsMax = 160 * 1024;  // LDS cap of the tail's single-workgroup phase
constexpr int kFlatEntryWords = 8;  // per narrow launch in that phase's table
constexpr int kStageItems = 8;  // loads per lane in flight while that phase stages its values
constexpr int kFlagOffset = 32;  // tail barrier: release flag, in 4-byte words past the arrival counter
constexpr int kStreamItems = 4;  // roots per lane and round of a stream emission block
constexpr int kStreamCap = kBlock * kStreamItems;  // roots per round, and the most groups of a stream chunk

template <class P, int kLeafItems>
__global__ __launch_bounds__(kBlock) void leaf_kernel(const int32_t* __restrict__ tcol,
                                                      const int32_t* __restrict__ tval,
                                                      const typename P::W* __restrict__ V,
                                                      const typename P::X* __restrict__ x,
                                                      typename P::A* __restrict__ T, int32_t alpha,
                                                      typename P::A* __restrict__ acc, int32_t n_acc,
                                                      unsigned* __restrict__ barrier)
{
    // kLeafItems terminals per lane, i = base + u * kBlock + lane, all loads
    // issued before the first value is formed (indices past alpha are clamped
    // to alpha - 1 and their values discarded)
    const int32_t base = blockIdx.x * (kBlock * kLeafItems) + threadIdx.x;
    if (alpha > 0) {
        int32_t c[kLeafItems];
#pragma unroll
        for (int u = 0; u < kLeafItems; ++u) c[u] = min(base + u * kBlock, alpha - 1);
        int32_t col[kLeafItems], val[kLeafItems];
#pragma unroll
        for (int u = 0; u < kLeafItems; ++u) {
            col[u] = tcol[c[u]];
            val[u] = tval[c[u]];
        }
        typename P::A t[kLeafItems];
#pragma unroll
        for (int u = 0; u < kLeafItems; ++u) t[u] = P::leaf(V[val[u]], x[col[u]]);
#pragma unroll
        for (int u = 0; u < kLeafItems; ++u) {
            const int32_t i = base + u * kBlock;
            if constexpr (kBitTerms<P>) {
                // every lane of the wave takes part in the ballot; lane l gives
                // bit l of the word of terminals i0 .. i0 + 63 (i0 = i - l)
                const uint64_t w = __ballot(i < alpha && t[u]);
                if ((threadIdx.x & 63) == 0 && i < alpha) ((uint64_t*)T)[i >> 6] = w;
            } else {
                if (i < alpha) T[i] = t[u];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kLeafItems; ++u) {
        const int32_t i = base + u * kBlock;
        if (i < n_acc) acc[i] = P::ident();
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {  // the tail kernel's grid barrier counts rounds from 0 in every sweep
        barrier[0] = 0;
        barrier[kFlagOffset] = 0;
        barrier[kFlagOffset + 1] = 0;  // and this sweep has not failed yet
    }
}

// Per-launch arguments.  Every part of the grid (binary nodes, pass-through
// nodes, emission groups) is cut into kSlices column slices; a part holds
// kSlices * blocks-per-slice workgroups and workgroup b of a part serves slice
// b % kSlices.  Workgroups are dealt to the XCDs round-robin, so all of a
// slice's work lands on one XCD and its gathers stay inside that XCD's L2.
struct LevelArgs {
    const int2* child;     // this level's binary nodes
    const int32_t* ptsrc;  // this level's pass-through sources
    const int32_t* erow;   // emission groups of the previous level
    const int32_t* eoff;
    const int32_t* epos;
    const int32_t* chunk;  // stream emission: first group of each chunk of the previous level
    int32_t cur, nb;       // arena offset of this level's buffer; binary node count
    int32_t prev, alpha;   // arena offset of the level below; terminals (arena offsets below alpha)
    int32_t n_rows;        // stride of the per-slice row accumulators
    int32_t team_log2;     // lanes per emission group = 1 << team_log2 (<= 64)
    int32_t pb_bin, pb_pt, pb_emit;  // workgroups per slice in each part
    int32_t bsl[kSlices + 1], psl[kSlices + 1], gsl[kSlices + 1];
    int32_t stream;              // emission by chunks (stream_block) instead of teams
    int32_t csl[kSlices + 1];    // chunks of each slice (indices into chunk)
};

static_assert(sizeof(LevelArgs) % 4 == 0, "LevelArgs is copied as 32-bit words");

// One emission lane: combines the roots e0, e0 + team, ... below e1 of its
// group in that order, kEmitItems independent loads per round (indices past
// e1 are clamped to e1 - 1, the group's last root, and discarded).  A lane of
// an invalid team, or one with no root, returns the identity.
template <class P, class Idx, class Val>
__device__ __forceinline__ typename P::A emit_rounds(const Idx* __restrict__ epos, int32_t e0, int32_t e1,
                                                     int32_t team, bool valid, Val val)
{
    using A = typename P::A;
    A s = P::ident();
    int32_t e = e0;
    do {
        int32_t p[kEmitItems];
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) p[u] = epos[min(e + u * team, e1 - 1)];
        A v[kEmitItems];
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) v[u] = val(p[u]);
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) issue_before(v[u]);
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u)
            if (valid && e + u * team < e1) s = P::comb(s, v[u]);
        e += kEmitItems * team;
    } while (valid && e < e1);
    return s;
}

// The fixed xor butterfly over a team of adjacent lanes (every lane of the
// team ends with the same combination, in the same order on every run).
template <class P>
__device__ __forceinline__ typename P::A team_combine(typename P::A s, int32_t team)
{
    for (int32_t o = team >> 1; o > 0; o >>= 1) s = P::comb(s, xchg(s, o));
    return s;
}

// One workgroup's share of a level launch: virtual block b of the grid.
// Every load of a part is issued unconditionally (indices past the end of
// the part are clamped to its last element, which exists because a block
// with no element returns first), so a lane keeps all of its independent
// gathers in flight at once; only the stores and the combines are masked.
template <class P>
__device__ __forceinline__ void level_block(const LevelArgs& a, int32_t b, int32_t tid,
                                            typename P::A* __restrict__ arena, typename P::A* __restrict__ acc)
{
    using A = typename P::A;
    const int32_t part_bin = a.pb_bin * kSlices, part_pt = a.pb_pt * kSlices;
    if (b < part_bin) {
        const int32_t x = b % kSlices, i = b / kSlices, end = a.bsl[x + 1];
        const int32_t first = a.bsl[x] + i * (kBlock * kBinItems);
        if (first >= end) return;
        const int32_t t0 = first + tid;
        int2 c[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) c[u] = a.child[min(t0 + u * kBlock, end - 1)];
        A v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = P::comb(fetch<P>(arena, c[u].x, a.alpha), fetch<P>(arena, c[u].y, a.alpha));
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) issue_before(v[u]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            if (t < end) arena[a.cur + t] = v[u];
        }
        return;
    }
    b -= part_bin;
    if (b < part_pt) {
        const int32_t x = b % kSlices, i = b / kSlices, end = a.psl[x + 1];
        const int32_t first = a.psl[x] + i * (kBlock * kBinItems);
        if (first >= end) return;
        const int32_t t0 = first + tid;
        int32_t src[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) src[u] = a.ptsrc[min(t0 + u * kBlock, end - 1)];
        A v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = fetch<P>(arena, src[u], a.alpha);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) issue_before(v[u]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            if (t < end) arena[a.cur + a.nb + t] = v[u];
        }
        return;
    }
    b -= part_pt;
    // emission: a team of 2^team_log2 adjacent lanes per (slice, row) group;
    // lane sub of a team takes the group's roots sub, sub + team, ... in that
    // order, kEmitItems of them per round as independent loads; a fixed xor
    // butterfly combines the team (deterministic), and the team's first lane
    // updates the slice's accumulator of the row (each (slice, row) has one
    // group per level and levels are ordered launches, so a plain
    // read-modify-write suffices).  Teams past the slice's last group read
    // that group and discard it.
    const int32_t x = b % kSlices, i = b / kSlices;
    const int32_t gend = a.gsl[x + 1];
    const int32_t gfirst = a.gsl[x] + ((i * kBlock) >> a.team_log2);
    if (gfirst >= gend) return;
    const int32_t gl = i * kBlock + tid;
    const int32_t team = 1 << a.team_log2;
    const int32_t graw = a.gsl[x] + (gl >> a.team_log2), sub = gl & (team - 1);
    const bool valid = graw < gend;
    const int32_t g = valid ? graw : gend - 1;
    if constexpr (kDirectEmit<P>) {
        // acc is y itself: the team's first lane folds the team's combination
        // into the row (one store or atomic per group, not one per lane)
        const A part = emit_rounds<P>(a.epos, a.eoff[g] + sub, a.eoff[g + 1], team, valid,
                                      [&](int32_t c) { return fetch<P>(arena, c, a.alpha); });
        const A s = team_combine<P>(part, team);
        if (valid && sub == 0) direct(acc + a.erow[g], s);
        return;
    }
    // the accumulator is read beside the roots (its address needs only the
    // group's row), not after the team has combined them
    A* r = acc + (int64_t)x * a.n_rows + a.erow[g];
    const A old = *r;
    const int32_t e1 = a.eoff[g + 1];
    const A s0 =
        emit_rounds<P>(a.epos, a.eoff[g] + sub, e1, team, valid, [&](int32_t c) { return fetch<P>(arena, c, a.alpha); });
    issue_before(old);
    const A s = team_combine<P>(s0, team);
    if (valid && sub == 0) *r = P::comb(old, s);
}

// Stream emission, for levels whose groups are short and uneven (a team per
// group leaves most lanes of a wave idle while its longest group finishes).
// The host cuts each slice's groups into chunks of consecutive groups with at
// most kStreamCap roots and kStreamCap groups (a longer group is a chunk of
// its own).  A block takes one chunk and works in rounds of kStreamCap roots:
// each lane loads kStreamItems of the round's roots (consecutive lanes read
// consecutive roots) and puts their values in LDS; then lane j folds the part
// of the chunk's groups j, j + kBlock, ... that falls in the round, left to
// right, and keeps its partials for the next round.  Used only where the
// level's team has one or two lanes, and folded in that team's order: roots
// 0, 1, 2, ... for one lane; for two, roots 0, 2, 4, ... and 1, 3, 5, ...
// apart, then the two partials combined as the team's butterfly does.  So
// the bits do not depend on the mode, and the accumulator still takes one
// read-modify-write per (slice, row) and level.
template <class P>
__device__ __forceinline__ void stream_block(const LevelArgs& a, int32_t b, int32_t tid,
                                             typename P::A* __restrict__ arena, typename P::A* __restrict__ acc)
{
    using A = typename P::A;
    constexpr int Q = kStreamCap / kBlock;  // groups per lane, at most
    __shared__ A win[kStreamCap];
    const int32_t x = b % kSlices, ci = a.csl[x] + b / kSlices;
    if (ci >= a.csl[x + 1]) return;  // the same for the whole block
    const int32_t g0 = a.chunk[ci], g1 = ci + 1 < a.csl[x + 1] ? a.chunk[ci + 1] : a.gsl[x + 1];
    const int32_t r0 = a.eoff[g0], r1 = a.eoff[g1];
    const int32_t odd = a.team_log2;  // 1: a two-lane team's order (roots at odd places apart)
    int32_t lo[Q], hi[Q], row[Q];
    A s0[Q], s1[Q], old[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int32_t g = g0 + tid + q * kBlock, gg = min(g, g1 - 1);
        lo[q] = a.eoff[gg];
        hi[q] = g < g1 ? a.eoff[gg + 1] : lo[q];
        row[q] = a.erow[gg];
        s0[q] = P::ident();
        s1[q] = P::ident();
    }
    if constexpr (!kDirectEmit<P>) {
#pragma unroll
        for (int q = 0; q < Q; ++q) old[q] = acc[(int64_t)x * a.n_rows + row[q]];
    }
    for (int32_t rb = r0; rb < r1; rb += kStreamCap) {
        const int32_t n = min(kStreamCap, r1 - rb);
        int32_t p[kStreamItems];
#pragma unroll
        for (int u = 0; u < kStreamItems; ++u) p[u] = a.epos[rb + min(tid + u * kBlock, n - 1)];
        A v[kStreamItems];
#pragma unroll
        for (int u = 0; u < kStreamItems; ++u) v[u] = fetch<P>(arena, p[u], a.alpha);
#pragma unroll
        for (int u = 0; u < kStreamItems; ++u) win[tid + u * kBlock] = v[u];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int32_t e1 = min(hi[q], rb + n);
            for (int32_t e = max(lo[q], rb); e < e1; ++e) {
                const A v = win[e - rb];
                if ((e - lo[q]) & odd) s1[q] = P::comb(s1[q], v);
                else s0[q] = P::comb(s0[q], v);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (g0 + tid + q * kBlock >= g1) continue;
        const A sum = odd ? P::comb(s0[q], s1[q]) : s0[q];
        if constexpr (kDirectEmit<P>) {
            direct(acc + row[q], sum);
        } else {
            acc[(int64_t)x * a.n_rows + row[q]] = P::comb(old[q], sum);
        }
    }
}

// Level-0 emission of the direct policies (Boolean, tropical) from LDS.
// Level 0's roots are bare terminals, and a direct emission updates y[row]
// in place (a store of 1 where a bit is set; an atomic min), so level 0
// needs no groups: the upload lists its (row, terminal) pairs per column
// sub-slice in row order, cut into chunks whose terminals lie in a window of
// at most kWinBytes of T, and packs every pair into one 32-bit word:
//   bits [0, 19): the terminal's offset from the window's first terminal
//                 (Boolean terminals are bits, the others values)
//                 (kWordSkip: no terminal, the word only advances the row);
//   bits [19, 32): the row's increase over the previous word's row (the
//                 chunk's first row for its first word), at most
//                 kWordMaxDelta; a longer gap is bridged by skip words.
// A chunk's words start at a multiple of kWinWords and are padded to one
// with zero-increase skip words.  A workgroup of kWinBlock lanes copies its
// chunk's window into LDS once (16-byte loads), then takes kWinWords
// consecutive words per lane per round: a prefix sum of the increases
// (in the lane, then over the workgroup) gives each word's row, and the bit
// comes from LDS; a lane combines its consecutive words of one row before
// it updates y.  A root then costs 4 streamed bytes and no L2 request of
// its own.  Workgroup b takes chunk b: a chunk touches HBM only to stream
// its words and load its window once, so it gains nothing from its slice's
// XCD, and the slices' level-0 work differs.
constexpr int kWinBlock = 1024;
constexpr int kWinWords = 8;              // words per lane and round (two 16-byte loads)
constexpr int32_t kWinBytes = 60 * 1024;  // LDS window: bytes of packed terminals, a multiple of 16
constexpr int kWordPosBits = 19;
constexpr uint32_t kWordSkip = (1u << kWordPosBits) - 1;
constexpr int32_t kWordMaxDelta = (1 << (32 - kWordPosBits)) - 1;
static_assert((uint32_t)kWinBytes * 8 <= kWordSkip, "every bit of a window has an offset below kWordSkip");

struct WinArgs {
    // per chunk two int4: {first word, end word, window [b0, b1) in bytes of
    // T (multiples of 16)} and {row of the first word, the window's first
    // terminal, 0, 0}
    const int4* chunk;
    const uint32_t* word;
    int32_t n_chunks;
};

// Exclusive prefix sum over the workgroup's lanes (v >= 0); *total gets the
// sum of all.  Every lane calls it; wsum holds one slot per wave.
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_sum(int32_t v, int32_t* wsum, int32_t* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int32_t t = wsum[w];
        before += w < wave ? t : 0;
        all += t;
    }
    __syncthreads();  // wsum is rewritten by the next call
    *total = all;
    return before + inc - v;
}

// One round of a chunk: this lane's kWinWords words from word i0 (skip words
// past e1) and each word's row; *row_base advances past the round.  Called
// by every lane of the workgroup.
__device__ __forceinline__ void window_round(const uint32_t* __restrict__ words, int32_t i0, int32_t e1,
                                             int32_t* row_base, int32_t* wsum, uint32_t (&wd)[kWinWords],
                                             int32_t (&row)[kWinWords])
{
    if (i0 < e1) {
        const uint4 u0 = ((const uint4*)(words + i0))[0], u1 = ((const uint4*)(words + i0))[1];
        wd[0] = u0.x, wd[1] = u0.y, wd[2] = u0.z, wd[3] = u0.w;
        wd[4] = u1.x, wd[5] = u1.y, wd[6] = u1.z, wd[7] = u1.w;
    } else {
#pragma unroll
        for (int i = 0; i < kWinWords; ++i) wd[i] = kWordSkip;
    }
    int32_t inc = 0;
#pragma unroll
    for (int i = 0; i < kWinWords; ++i) {
        inc += (int32_t)(wd[i] >> kWordPosBits);
        row[i] = inc;
    }
    int32_t total;
    const int32_t before = block_exclusive_sum<kWinBlock>(inc, wsum, &total) + *row_base;
#pragma unroll
    for (int i = 0; i < kWinWords; ++i) row[i] += before;
    *row_base += total;
}

template <class P>
__global__ __launch_bounds__(kWinBlock) void window_emit_kernel(WinArgs w, const typename P::A* __restrict__ T,
                                                                typename P::Y* __restrict__ y)
{
    static_assert(kDirectEmit<P>, "window emission updates y in place");
    using A = typename P::A;
    extern __shared__ __align__(16) unsigned char win[];
    __shared__ int32_t wsum[kWinBlock / 64];
    const int4 c0 = w.chunk[2 * blockIdx.x], c1 = w.chunk[2 * blockIdx.x + 1];
    const int4* src = (const int4*)((const unsigned char*)T + c0.z);
    int4* dst = (int4*)win;
    for (int32_t i = threadIdx.x; i < (c0.w - c0.z) / 16; i += kWinBlock) dst[i] = src[i];
    __syncthreads();
    int32_t row_base = c1.x;
    for (int32_t base = c0.x; base < c0.y; base += kWinBlock * kWinWords) {
        uint32_t wd[kWinWords];
        int32_t row[kWinWords];
        window_round(w.word, base + (int32_t)threadIdx.x * kWinWords, c0.y, &row_base, wsum, wd, row);
        A v[kWinWords];
#pragma unroll
        for (int i = 0; i < kWinWords; ++i) {
            const uint32_t t = wd[i] & kWordSkip;
            if (t == kWordSkip) v[i] = P::ident();
            else if constexpr (kBitTerms<P>) v[i] = (win[t >> 3] >> (t & 7)) & 1u;
            else v[i] = ((const A*)win)[t];
        }
        // runs of one row (rows never decrease inside a chunk): one update
        // each; an identity update touches nothing (skip words' rows)
        A s = v[0];
#pragma unroll
        for (int i = 1; i < kWinWords; ++i) {
            if (row[i] != row[i - 1]) {
                direct(&y[row[i - 1]], s);
                s = v[i];
            } else {
                s = P::comb(s, v[i]);
            }
        }
        direct(&y[row[kWinWords - 1]], s);
    }
}

// One wide level.  By default the grid has one workgroup per virtual block
// (measured faster on MI355X than a grid capped near the resident count);
// with a cap, each workgroup strides over the level's virtual blocks.  The
// stride (gridDim.x) is a multiple of kSlices, so a workgroup keeps serving
// the same slice on the same XCD.  The emission part runs by teams
// (level_block) or, where the host chose it, by chunks (stream_block); a
// virtual block is the same for all lanes of a workgroup, so the chunk path's
// workgroup barriers are reached by every lane.
template <class P>
__global__ __launch_bounds__(kBlock) void level_kernel(LevelArgs a, typename P::A* __restrict__ arena,
                                                       typename P::A* __restrict__ acc)
{
    const int32_t nvb = kSlices * (a.pb_bin + a.pb_pt + a.pb_emit), nodes = kSlices * (a.pb_bin + a.pb_pt);
    for (int32_t vb = blockIdx.x; vb < nvb; vb += gridDim.x) {
        if (a.stream && vb >= nodes) stream_block<P>(a, vb - nodes, threadIdx.x, arena, acc);
        else level_block<P>(a, vb, threadIdx.x, arena, acc);
    }
}

// Grid-wide barrier for the co-resident tail grid.  bar[0] counts arrivals
// in this sweep; bar[kFlagOffset] (another cache line) holds the last round
// released and bar[kFlagOffset + 1] whether this sweep has failed (both
// cleared by the sweep's leaf launch).  Every wave first waits for its own
// stores to complete; one lane per workgroup then arrives with a
// device-scope release increment, the last arriver of the round publishes
// the round number with a release store, and the others poll that flag with
// relaxed device-scope loads (pollers never touch the line the arrivals
// update) and acquire once it is released.  The wait is bounded: after
// spin_limit polls (about a second by default; 0 = never wait, which fails
// every workgroup but the last arriver, for tests) the workgroup gives up
// and returns false, and the caller marks the sweep failed; a sweep already
// marked failed waits no more, so the grid always drains, and the next
// sweep starts with a clean mark.
__device__ __forceinline__ bool grid_barrier(unsigned* bar, unsigned round, unsigned spin_limit)
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
    __syncthreads();
    __shared__ int ok;
    if (threadIdx.x == 0) {
        ok = 1;
        unsigned* flag = bar + kFlagOffset;
        const unsigned prev = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1 == round * gridDim.x) {
            __hip_atomic_store(flag, round, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else if (spin_limit == 0) {
            ok = 0;  // never wait: the failure path on purpose (tests)
        } else if (__hip_atomic_load(flag + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            unsigned spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < round) {
                if (++spins == spin_limit) {
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    return ok != 0;
}

// The narrowest launches, run by one extra workgroup of kTailBlock lanes with
// workgroup barriers only and everything they touch held in LDS.  The host
// rewrites each of their value references (a child, a pass-through source, a
// root) as a slot of one LDS value array: slots [0, n_stage) are staged from
// the arena (the n_terms terminal values first, then values of the level the
// grid computed last), and every narrow level owns the slots its nodes are
// written to.  Emission sums go to LDS slots (gsum); at the end each touched
// row accumulator takes its sums in level order (fold lists): the same
// operations in the same order as one read-modify-write per level.
struct FlatArgs {
    const int32_t* idx;  // the LDS image, idx_words 32-bit words (a multiple of four)
    int32_t idx_words, n_ent, n_stage, n_terms, n_fold;
    int32_t alpha;  // terminals: arena references below alpha
    // word offsets in the image: entry table at 0, then these arrays
    int32_t goff_word, stage_word, facc_word, foff_word, refs_word, roots_word, flist_word;
    int32_t vals_off, gsum_off, accv_off;  // byte offsets of the value, sum and accumulator arrays in LDS
};

// for (i = tid; i < n; i += kTailBlock) op(i), four independent iterations at
// a time: op(i0..i3, live1..live3) must only load when live is false (i is
// then clamped to n - 1) and store when it is true
template <class Op>
__device__ __forceinline__ void block_rounds(int32_t n, int32_t tid, Op op)
{
    for (int32_t i0 = tid; i0 < n; i0 += 4 * kTailBlock) op(i0, min(i0 + kTailBlock, n - 1), min(i0 + 2 * kTailBlock, n - 1),
                                                              min(i0 + 3 * kTailBlock, n - 1), i0 + kTailBlock < n,
                                                              i0 + 2 * kTailBlock < n, i0 + 3 * kTailBlock < n);
}

// vals[i] = the value of arena reference stage[i], for i in [lo, hi)
template <class P>
__device__ __forceinline__ void stage_values(const int32_t* stage, const typename P::A* __restrict__ arena,
                                             typename P::A* vals, int32_t lo, int32_t hi, int32_t alpha, int32_t tid)
{
    using A = typename P::A;
    block_rounds(hi - lo, tid, [&](int32_t i0, int32_t i1, int32_t i2, int32_t i3, bool l1, bool l2, bool l3) {
        const A v0 = fetch<P>(arena, stage[lo + i0], alpha), v1 = fetch<P>(arena, stage[lo + i1], alpha);
        const A v2 = fetch<P>(arena, stage[lo + i2], alpha), v3 = fetch<P>(arena, stage[lo + i3], alpha);
        issue_before(v0);
        issue_before(v1);
        issue_before(v2);
        issue_before(v3);
        vals[lo + i0] = v0;
        if (l1) vals[lo + i1] = v1;
        if (l2) vals[lo + i2] = v2;
        if (l3) vals[lo + i3] = v3;
    });
}

// Before the grid levels finish: the image into LDS and the terminal values
// (complete since the leaf launch).
template <class P>
__device__ __noinline__ void flat_prefetch(const FlatArgs f, const typename P::A* __restrict__ arena)
{
    using A = typename P::A;
    extern __shared__ __align__(16) unsigned char flat_lds[];
    const int32_t tid = threadIdx.x;
    int32_t* iw = (int32_t*)flat_lds;
    const int4* src = (const int4*)f.idx;
    int4* dst = (int4*)iw;
    block_rounds(f.idx_words / 4, tid, [&](int32_t i0, int32_t i1, int32_t i2, int32_t i3, bool l1, bool l2, bool l3) {
        const int4 v0 = src[i0], v1 = src[i1], v2 = src[i2], v3 = src[i3];
        dst[i0] = v0;
        if (l1) dst[i1] = v1;
        if (l2) dst[i2] = v2;
        if (l3) dst[i3] = v3;
    });
    // the stage indices straight from the image in global memory (the LDS
    // copy is not yet visible to other lanes)
    stage_values<P>(f.idx + f.stage_word, arena, (A*)(flat_lds + f.vals_off), 0, f.n_terms, f.alpha, tid);
    __syncthreads();
}

// After the grid levels: their values, the accumulators to fold, the narrow
// levels, the folds.
template <class P>
__device__ __noinline__ void flat_phase(const FlatArgs f, const typename P::A* __restrict__ arena,
                                        typename P::A* __restrict__ acc)
{
    using A = typename P::A;
    extern __shared__ __align__(16) unsigned char flat_lds[];
    const int32_t tid = threadIdx.x;
    const int32_t* iw = (const int32_t*)flat_lds;
    A* vals = (A*)(flat_lds + f.vals_off);
    A* gsum = (A*)(flat_lds + f.gsum_off);
    A* accv = (A*)(flat_lds + f.accv_off);
    const int32_t* facc = iw + f.facc_word;
    // one gather round for the grid's last level and the accumulators to
    // fold: item i < n_prev stages slot n_terms + i, the rest accumulators
    {
        const int32_t* stage = iw + f.stage_word;
        const int32_t n_prev = f.n_stage - f.n_terms, n = n_prev + (kDirectEmit<P> ? 0 : f.n_fold);
        for (int32_t i0 = tid; i0 < n; i0 += kStageItems * kTailBlock) {
            A v[kStageItems];
#pragma unroll
            for (int u = 0; u < kStageItems; ++u) {
                const int32_t i = min(i0 + u * kTailBlock, n - 1);
                v[u] = i < n_prev ? arena[stage[f.n_terms + i]] : acc[facc[i - n_prev]];
            }
#pragma unroll
            for (int u = 0; u < kStageItems; ++u) issue_before(v[u]);
#pragma unroll
            for (int u = 0; u < kStageItems; ++u) {
                const int32_t i = i0 + u * kTailBlock;
                if (i < n) {
                    if (i < n_prev) vals[f.n_terms + i] = v[u];
                    else accv[i - n_prev] = v[u];
                }
            }
        }
    }
    __syncthreads();
    const uint16_t* refs = (const uint16_t*)(iw + f.refs_word);
    const uint16_t* roots = (const uint16_t*)(iw + f.roots_word);
    const int32_t* goff = iw + f.goff_word;
    auto val = [&](int32_t c) -> A { return vals[c]; };
    for (int32_t j = 0; j < f.n_ent; ++j) {
        const int32_t* e = iw + j * kFlatEntryWords;
        const int32_t nb = e[0], npt = e[1], ng = e[2], tl = e[3], out = e[4], r0 = e[5], g0 = e[6], s0 = e[7];
        // this level's nodes (slots out ..) from the level below; the emission
        // of the level below reads other slots, so no barrier in between
        for (int32_t t = tid; t < nb; t += kTailBlock)
            vals[out + t] = P::comb(vals[refs[r0 + 2 * t]], vals[refs[r0 + 2 * t + 1]]);
        for (int32_t t = tid; t < npt; t += kTailBlock) vals[out + nb + t] = vals[refs[r0 + 2 * nb + t]];
        const int32_t team = 1 << tl;
        for (int32_t gl0 = 0; gl0 < (ng << tl); gl0 += kTailBlock) {
            const int32_t gl = gl0 + tid;
            const int32_t graw = gl >> tl, sub = gl & (team - 1);
            const bool valid = graw < ng;
            const int32_t gg = valid ? graw : ng - 1;
            const A part = emit_rounds<P>(roots, goff[g0 + gg] + sub, goff[g0 + gg + 1], team, valid, val);
            const A sum = team_combine<P>(part, team);
            if (valid && sub == 0) gsum[s0 + graw] = sum;
        }
        __syncthreads();
    }
    const int32_t* foff = iw + f.foff_word;
    const uint16_t* flist = (const uint16_t*)(iw + f.flist_word);
    for (int32_t i = tid; i < f.n_fold; i += kTailBlock) {
        if constexpr (kDirectEmit<P>) {
            // fold i is a row of y: fold its sums into it
            A a = P::ident();
            for (int32_t k = foff[i]; k < foff[i + 1]; ++k) a = P::comb(a, gsum[flist[k]]);
            direct(acc + facc[i], a);
        } else {
            A a = accv[i];
            for (int32_t k = foff[i]; k < foff[i + 1]; ++k) a = P::comb(a, gsum[flist[k]]);
            acc[facc[i]] = a;
        }
    }
}

// Levels k0..L (each with the emission of the level below), the emission of
// level L and the final slice reduction, in one cooperative launch of
// workgroups with kTailBlock lanes.  Entries [0, n_multi) run on the first
// n_grid workgroups (a multiple of kSlices): the four 256-lane quarters of a
// workgroup take virtual blocks blockIdx.x + (quarter + 4j) * n_grid, all of
// the same slice, so a workgroup stays on its slice's XCD; grid barriers
// separate the entries.  The f.n_ent narrowest levels run on one more
// workgroup (blockIdx.x == n_grid), in LDS, which loads its image while the
// others work and only joins their barriers; the others wait for it at the
// next grid barrier.  Then every workgroup reduces
// y[r] = acc[0][r] (+) ... (+) acc[7][r].
template <class P>
__global__ __launch_bounds__(kTailBlock) void tail_kernel(const LevelArgs* __restrict__ table, int32_t n_multi,
                                                          int32_t n_grid, FlatArgs f,
                                                          typename P::A* __restrict__ arena,
                                                          typename P::A* __restrict__ acc,
                                                          typename P::Y* __restrict__ y, int32_t n_rows,
                                                          int32_t accumulate, unsigned* __restrict__ bar,
                                                          int* __restrict__ err, unsigned spin_limit)
{
    // a timed-out barrier marks this sweep failed (bar[kFlagOffset + 1]) and
    // raises the sticky flag gcs_device_check reports
    auto fail = [&]() {
        __hip_atomic_store(bar + kFlagOffset + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    constexpr int Q = kTailBlock / kBlock;
    const int32_t q = threadIdx.x / kBlock, ltid = threadIdx.x % kBlock;
    const bool flat_wg = f.n_ent > 0 && (int32_t)blockIdx.x == n_grid;
    if (flat_wg) flat_prefetch<P>(f, arena);
    unsigned round = 0;
    for (int32_t li = 0; li < n_multi; ++li) {
        if (!flat_wg) {
            const LevelArgs& a = table[li];
            const int32_t nvb = kSlices * (a.pb_bin + a.pb_pt + a.pb_emit);
            for (int32_t vb = blockIdx.x + q * n_grid; vb < nvb; vb += Q * n_grid)
                level_block<P>(a, vb, ltid, arena, acc);
        }
        if (!grid_barrier(bar, ++round, spin_limit) && threadIdx.x == 0) fail();
    }
    if (f.n_ent > 0) {
        if (flat_wg) flat_phase<P>(f, arena, acc);
        if (!grid_barrier(bar, ++round, spin_limit) && threadIdx.x == 0) fail();
    }
    if constexpr (!kDirectEmit<P>) {
        for (int32_t r = blockIdx.x * kTailBlock + threadIdx.x; r < n_rows; r += gridDim.x * kTailBlock) {
            typename P::A s = acc[r];
#pragma unroll
            for (int x = 1; x < kSlices; ++x) s = P::comb(s, acc[(int64_t)x * n_rows + r]);
            y[r] = P::emit(accumulate ? y[r] : P::yzero(), s);
        }
    }
    // a failed sweep leaves no plausible y: every workgroup that sees the
    // mark overwrites all of y after its own writes
    if (__hip_atomic_load(bar + kFlagOffset + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        __syncthreads();
        for (int32_t r = threadIdx.x; r < n_rows; r += kTailBlock) y[r] = P::poison();
    }
}

// ---------------------------------------------------------------- column groups swept together

// Several uploaded grammars of one matrix (disjoint column groups, section
// 4.4) swept as one: launch k runs level k (with the emission of level k-1)
// of every group that has it.  A group's entry holds its launch arguments,
// its own arena and accumulators, and the first virtual block of its share of
// the launch; shares are multiples of kSlices, so a virtual block keeps its
// slice's XCD.  Narrow levels of many groups together fill the chip, so no
// persistent tail is needed.
struct GroupEntry {
    LevelArgs a;
    void* arena;
    void* acc;
    int32_t block0, pad;
};
struct LeafEntry {
    const int32_t *tcol, *tval;
    const void* V;
    void *T, *acc;
    int32_t alpha, n_acc, block0, pad;
};
constexpr int kGroupLeafItems = 4;

template <class E>
__device__ __forceinline__ int32_t find_entry(const E* __restrict__ ents, int32_t n, int32_t vb)
{
    int32_t lo = 0, hi = n - 1;  // the last entry with block0 <= vb
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (ents[mid].block0 <= vb) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <class P>
__global__ __launch_bounds__(kBlock) void leaf_group_kernel(const LeafEntry* __restrict__ ents, int32_t n_ent,
                                                            const typename P::X* __restrict__ x)
{
    const LeafEntry& e = ents[find_entry(ents, n_ent, (int32_t)blockIdx.x)];
    auto* T = (typename P::A*)e.T;
    auto* acc = (typename P::A*)e.acc;
    const auto* V = (const typename P::W*)e.V;
    const int32_t base = ((int32_t)blockIdx.x - e.block0) * (kBlock * kGroupLeafItems) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kGroupLeafItems; ++u) {
        const int32_t i = base + u * kBlock;
        if (i < e.alpha) T[i] = P::leaf(V[e.tval[i]], x[e.tcol[i]]);
        if (i < e.n_acc) acc[i] = P::ident();
    }
}

template <class P>
__global__ __launch_bounds__(kBlock) void level_group_kernel(const GroupEntry* __restrict__ ents, int32_t n_ent)
{
    const GroupEntry& e = ents[find_entry(ents, n_ent, (int32_t)blockIdx.x)];
    const LevelArgs& a = e.a;
    const int32_t b = (int32_t)blockIdx.x - e.block0, nodes = kSlices * (a.pb_bin + a.pb_pt);
    auto* arena = (typename P::A*)e.arena;
    auto* acc = (typename P::A*)e.acc;
    if (a.stream && b >= nodes) stream_block<P>(a, b - nodes, threadIdx.x, arena, acc);
    else level_block<P>(a, b, threadIdx.x, arena, acc);
}

// y[r] = y0 (+) s_0 (+) s_1 ... with s_g the combination of group g's eight
// slice accumulators of row r in slice order: the additions, in the same
// order, of a sweep of group 0 followed by accumulating sweeps of the others
template <class P>
__global__ __launch_bounds__(kBlock) void reduce_group_kernel(void* const* __restrict__ accs, int32_t n_grp,
                                                              typename P::Y* __restrict__ y, int32_t n_rows,
                                                              int32_t accumulate)
{
    for (int32_t r = blockIdx.x * kBlock + threadIdx.x; r < n_rows; r += gridDim.x * kBlock) {
        typename P::Y v = accumulate ? y[r] : P::yzero();
        for (int32_t gi = 0; gi < n_grp; ++gi) {
            const auto* acc = (const typename P::A*)accs[gi];
            typename P::A s = acc[r];
#pragma unroll
            for (int x = 1; x < kSlices; ++x) s = P::comb(s, acc[(int64_t)x * n_rows + r]);
            v = P::emit(v, s);
        }
        y[r] = v;
    }
}

// ---------------------------------------------------------------- batched right product

// Y = M X for B vectors at once (X: m x B and Y: n x B, row-major).  Every
// value becomes a row of B values (terminal array, arena and accumulators
// scaled by B), a node's B values adjacent, so the lanes of a node gather
// consecutive addresses: at B = 32 in fp32 one cache line serves a whole
// node.  Lanes come in groups of VB = 2^vb_log2 >= B (lane b of a group
// takes vector b; lanes b >= B compute vector B-1 again and store nothing);
// a 256-lane block takes 256 / VB nodes, or emission groups, at a time.
// Same grammar, slices and emission groups as the single-vector sweep; every
// level is its own launch.
constexpr int kMaxBatch = 64;
constexpr int kBatchEmitItems = 4;  // roots per emission lane loaded before the first combine

struct BatchArgs {
    LevelArgs a;                     // the level's launch arguments (pointers, counts, slices)
    int32_t B, vb_log2;              // vectors; lanes per node = 1 << vb_log2
    int32_t pb_bin, pb_pt, pb_emit;  // workgroups per slice in each part at this width
    // leaves evaluated in the sweep: a reference c < leaf_alpha is computed as
    // V[tval[c]] (x) X[tcol[c]] instead of read; arena rows start at node tbase
    int32_t leaf_alpha, tbase;
    const int32_t *tcol, *tval;
    const void *V, *X;
};

template <class P>
__global__ __launch_bounds__(kBlock) void leaf_batch_kernel(const int32_t* __restrict__ tcol,
                                                            const int32_t* __restrict__ tval,
                                                            const typename P::W* __restrict__ V,
                                                            const typename P::X* __restrict__ X,
                                                            typename P::A* __restrict__ T, int64_t alpha, int32_t B,
                                                            typename P::A* __restrict__ acc, int64_t n_acc)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < alpha * B; i += stride) {
        const int64_t p = i / B, b = i - p * B;
        T[i] = P::leaf(V[tval[p]], X[(int64_t)tcol[p] * B + b]);
    }
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n_acc; i += stride) acc[i] = P::ident();
}

// VW adjacent values of a node's row, loaded and stored as one access of
// VW * sizeof(A) <= 16 bytes (the row and the lane's offset in it are
// multiples of that size)
template <class A, int VW>
struct alignas(sizeof(A) * VW) Row {
    A v[VW];
};

template <class P, int VW>
__device__ __forceinline__ Row<typename P::A, VW> comb_row(const Row<typename P::A, VW>& a,
                                                           const Row<typename P::A, VW>& b)
{
    Row<typename P::A, VW> r;
#pragma unroll
    for (int i = 0; i < VW; ++i) r.v[i] = P::comb(a.v[i], b.v[i]);
    return r;
}

template <class T>
__device__ __forceinline__ void issue_before_row(const T& r)
{
    static_assert(sizeof(T) % 4 == 0 || sizeof(T) < 4, "row size");
    if constexpr (sizeof(T) >= 4) {
        const int32_t* w = (const int32_t*)&r;
#pragma unroll
        for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"v"(w[i]));
    } else {
        issue_before(r.v[0]);
    }
}

// One level of the batched sweep; each lane takes VW consecutive vectors of
// a node (vb_log2 counts lanes per node: 2^vb_log2 >= B / VW).
template <class P, int VW, bool LEAVES>
__global__ __launch_bounds__(kBlock) void level_batch_kernel(BatchArgs ba, typename P::A* __restrict__ arena_a,
                                                             typename P::A* __restrict__ acc_a)
{
    using A = typename P::A;
    using R = Row<A, VW>;
    R* __restrict__ arena = (R*)arena_a;
    R* __restrict__ acc = (R*)acc_a;
    const LevelArgs& a = ba.a;
    const int64_t W = ba.B / VW;  // Row elements per node
    const int32_t tid = threadIdx.x, per = kBlock >> ba.vb_log2, slot = tid >> ba.vb_log2;
    const int32_t lane_w = tid & ((1 << ba.vb_log2) - 1);
    const bool live = lane_w < W;
    const int64_t vw = min((int64_t)lane_w, W - 1);  // the row element this lane gathers
    // the row element of reference c: a stored value, or a leaf computed in
    // place (same arithmetic as the leaf kernel)
    auto row_of = [&](int32_t c) -> R {
        if (!LEAVES || c >= ba.leaf_alpha) return arena[(int64_t)(c - ba.tbase) * W + vw];
        using XR = Row<typename P::X, VW>;
        const typename P::W v = ((const typename P::W*)ba.V)[ba.tval[c]];
        const XR xr = ((const XR*)ba.X)[(int64_t)ba.tcol[c] * W + vw];
        R r;
#pragma unroll
        for (int k = 0; k < VW; ++k) r.v[k] = P::leaf(v, xr.v[k]);
        return r;
    };
    int32_t b = blockIdx.x;
    const int32_t part_bin = ba.pb_bin * kSlices, part_pt = ba.pb_pt * kSlices;
    if (b < part_bin) {
        const int32_t x = b % kSlices, i = b / kSlices, end = a.bsl[x + 1];
        const int32_t first = a.bsl[x] + i * (per * kBinItems);
        if (first >= end) return;
        const int32_t t0 = first + slot;
        int2 c[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) c[u] = a.child[min(t0 + u * per, end - 1)];
        R v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = comb_row<P, VW>(row_of(c[u].x), row_of(c[u].y));
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) issue_before_row(v[u]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * per;
            if (t < end && live) arena[(int64_t)(a.cur + t - ba.tbase) * W + vw] = v[u];
        }
        return;
    }
    b -= part_bin;
    if (b < part_pt) {
        const int32_t x = b % kSlices, i = b / kSlices, end = a.psl[x + 1];
        const int32_t first = a.psl[x] + i * (per * kBinItems);
        if (first >= end) return;
        const int32_t t0 = first + slot;
        int32_t src[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) src[u] = a.ptsrc[min(t0 + u * per, end - 1)];
        R v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = row_of(src[u]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) issue_before_row(v[u]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * per;
            if (t < end && live) arena[(int64_t)(a.cur + a.nb + t - ba.tbase) * W + vw] = v[u];
        }
        return;
    }
    b -= part_pt;
    // emission: the lanes of a group each combine the group's roots in C
    // order for their vectors, then update the slice accumulator of the row
    const int32_t x = b % kSlices, i = b / kSlices, gend = a.gsl[x + 1];
    const int32_t gfirst = a.gsl[x] + i * per;
    if (gfirst >= gend) return;
    const int32_t graw = gfirst + slot;
    const bool valid = graw < gend;
    const int32_t g = valid ? graw : gend - 1;
    // direct policies: acc is Y itself (no slices)
    R* r = acc + ((kDirectEmit<P> ? 0 : (int64_t)x * a.n_rows) + a.erow[g]) * W + vw;
    R old;
    if constexpr (!kDirectEmit<P>) old = *r;
    const int32_t e0 = a.eoff[g], e1 = a.eoff[g + 1];
    R s;
#pragma unroll
    for (int k = 0; k < VW; ++k) s.v[k] = P::ident();
    int32_t e = e0;
    do {
        int32_t p[kBatchEmitItems];
#pragma unroll
        for (int u = 0; u < kBatchEmitItems; ++u) p[u] = a.epos[min(e + u, e1 - 1)];
        R v[kBatchEmitItems];
#pragma unroll
        for (int u = 0; u < kBatchEmitItems; ++u) v[u] = row_of(p[u]);
#pragma unroll
        for (int u = 0; u < kBatchEmitItems; ++u) issue_before_row(v[u]);
#pragma unroll
        for (int u = 0; u < kBatchEmitItems; ++u)
            if (e + u < e1) s = comb_row<P, VW>(s, v[u]);
        e += kBatchEmitItems;
    } while (valid && e < e1);
    if constexpr (kDirectEmit<P>) {
        if (valid && live)
#pragma unroll
            for (int k = 0; k < VW; ++k) direct(&r->v[k], s.v[k]);
    } else {
        issue_before_row(old);
        if (valid && live) *r = comb_row<P, VW>(old, s);
    }
}

// Level-0 emission of the batched sweep of a direct policy from the same
// chunks and words as window_emit_kernel: every round's (row, terminal)
// pairs are staged in LDS, then teams of the least power of two >= B lanes
// take one pair at a time, lane b reading vector b of the terminal's row of
// T (or computing it, with the leaves in the sweep) and updating Y's row in
// place.  (One vector per lane: the level launches' lanes may take
// several, ba.vb_log2 counts those.)
template <class P, bool LEAVES>
__global__ __launch_bounds__(kWinBlock) void window_batch_kernel(WinArgs w, BatchArgs ba,
                                                                 const typename P::A* __restrict__ T,
                                                                 typename P::A* __restrict__ Y)
{
    static_assert(kDirectEmit<P>, "window emission updates Y in place");
    __shared__ int32_t wsum[kWinBlock / 64];
    __shared__ int2 pair[kWinBlock * kWinWords / 2];
    const int4 c0 = w.chunk[2 * blockIdx.x], c1 = w.chunk[2 * blockIdx.x + 1];
    const int32_t B = ba.B;
    int32_t lg = 0;
    while ((1 << lg) < B) ++lg;
    const int32_t per = kWinBlock >> lg, team = threadIdx.x >> lg, b = threadIdx.x & ((1 << lg) - 1);
    const int64_t tb = c1.y;  // the window's first terminal
    int32_t row_base = c1.x;
    for (int32_t base = c0.x; base < c0.y; base += kWinBlock * kWinWords) {
        uint32_t wd[kWinWords];
        int32_t row[kWinWords];
        window_round(w.word, base + (int32_t)threadIdx.x * kWinWords, c0.y, &row_base, wsum, wd, row);
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // the round's pairs in two halves of LDS
#pragma unroll
            for (int i = 0; i < kWinWords / 2; ++i) {
                const uint32_t t = wd[h * (kWinWords / 2) + i] & kWordSkip;
                pair[threadIdx.x * (kWinWords / 2) + i] =
                    make_int2(t == kWordSkip ? -1 : row[h * (kWinWords / 2) + i], (int32_t)(tb + t));
            }
            __syncthreads();
            if (b < B)
                for (int32_t j = team; j < kWinBlock * kWinWords / 2; j += per) {
                    const int2 q = pair[j];
                    if (q.x < 0) continue;
                    const typename P::A v =
                        LEAVES ? P::leaf(((const typename P::W*)ba.V)[ba.tval[q.y]],
                                         ((const typename P::X*)ba.X)[(int64_t)ba.tcol[q.y] * B + b])
                               : T[(int64_t)q.y * B + b];
                    direct(&Y[(int64_t)q.x * B + b], v);
                }
            __syncthreads();
        }
    }
}

template <class P>
__global__ __launch_bounds__(kBlock) void reduce_batch_kernel(const typename P::A* __restrict__ acc,
                                                              typename P::Y* __restrict__ Y, int64_t n, int32_t accumulate)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        typename P::A s = acc[i];
#pragma unroll
        for (int x = 1; x < kSlices; ++x) s = P::comb(s, acc[(int64_t)x * n + i]);
        Y[i] = P::emit(accumulate ? Y[i] : P::yzero(), s);
    }
}

__global__ __launch_bounds__(kBlock) void bfs_clear_kernel(uint8_t* __restrict__ f, uint8_t* __restrict__ vis,
                                                           int64_t n, unsigned long long* __restrict__ cnt)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        f[i] = 0;
        vis[i] = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x < 2) cnt[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kBlock) void bfs_seed_kernel(const int64_t* __restrict__ src, int64_t ns,
                                                          uint8_t* __restrict__ f, uint8_t* __restrict__ vis,
                                                          int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < ns; i += (int64_t)gridDim.x * kBlock) {
        const int64_t v = src[i];
        if (v >= 0 && v < n) {  // out-of-range sources are ignored (the binding rejects them first)
            f[v] = 1;
            vis[v] = 1;
        }
    }
}

// f = y AND NOT visited; visited |= f; cnt[slot] += |f|; cnt[slot ^ 1] = 0.
__global__ __launch_bounds__(kBlock) void bfs_update_kernel(const uint8_t* __restrict__ y, uint8_t* __restrict__ f,
                                                            uint8_t* __restrict__ vis, int64_t n,
                                                            unsigned long long* __restrict__ cnt, int slot)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    unsigned long long mine = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const uint8_t nf = (y[i] != 0) & (vis[i] == 0);
        f[i] = nf;
        vis[i] |= nf;
        mine += nf;
    }
    // wave sum, then one atomic per wave
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_down(mine, o, 64);
    if ((threadIdx.x & 63) == 0 && mine) atomicAdd(&cnt[slot], mine);
    if (blockIdx.x == 0 && threadIdx.x == 0) cnt[slot ^ 1] = 0;
}

}  // namespace gcs
