// Device engine for y = M x on a properly layered grammar, gfx950 (CDNA4).
//
// Page: "Right Multiplication on Grammar-Compressed Matrices: A Streaming,
// Memory-Bounded GPU Engine" (arXiv 2607.24971v1), section 4.3 (streaming,
// double-buffered sweep; Listing 1), section 5 (leaf / combine / emit
// policies).
//
// Device memory (all owned by the caller):
//   grammar image  child pairs | pass-through sources | emission groups
//                  (erow, eoff, epos) | terminal descriptors | V
//   workspace      value arena [T (alpha) | buffer A | buffer B] | counters
// Level k's values live in A (k odd) or B (k even); every child index is an
// absolute arena offset with that parity already applied, so a node reads
// arena[child] whether the child is a terminal (persistent T) or a node of
// level k-1, without tags or branches.
//
// One sweep = 1 + (L + 1) launches on the caller's stream:
//   leaf:        T[p] = V[l_p] (x) x[j_p], and y = identity
//   level k:     binary nodes  cur[t] = arena[left] (+) arena[right]
//                pass-throughs cur[nb + t] = arena[src[t]]
//                emission of level k-1: y[row] = y[row] (+) sum of its roots
//   final:       emission of level L
// Emission of a level runs in the launch after the level is computed, while
// its buffer is still intact (it is overwritten two levels later).  Each
// (row, level) group is one lane that folds its roots in C order and then
// updates y[row] with a plain read-modify-write: a row has at most one group
// per level and the levels are ordered launches, so no atomics are needed and
// the result is deterministic for every policy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "grammar.hpp"

namespace gcs {

// ---------------------------------------------------------------- policies

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
// unsigned integers, so min is an integer min or an unsigned max
__device__ __forceinline__ void direct(float* p, float v)
{
    if (!(v < __builtin_huge_valf())) return;
    if (v >= 0.0f) atomicMin((int*)p, __float_as_int(v));
    else atomicMax((unsigned int*)p, __float_as_uint(v));
}
__device__ __forceinline__ void direct(double* p, double v)
{
    if (!(v < __builtin_huge_val())) return;
    if (v >= 0.0) atomicMin((long long*)p, __double_as_longlong(v));
    else atomicMax((unsigned long long*)p, (unsigned long long)__double_as_longlong(v));
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
constexpr int kBinItems = 4;  // binary nodes per lane (independent gathers in flight)
constexpr int kEmitItems = 4;  // roots per emission lane loaded before the first combine
constexpr int kTailBlock = 1024;  // lanes per workgroup of the persistent tail
constexpr size_t kFlatLdsMax = 160 * 1024;  // LDS cap of the tail's single-workgroup phase
constexpr int kFlatEntryWords = 8;  // per narrow launch in that phase's table
constexpr int kStageItems = 8;  // loads per lane in flight while that phase stages its values
constexpr int kFlagOffset = 32;  // tail barrier: release flag, in 4-byte words past the arrival counter

template <class P>
__global__ __launch_bounds__(kBlock) void leaf_kernel(const int32_t* __restrict__ tcol,
                                                      const int32_t* __restrict__ tval,
                                                      const typename P::W* __restrict__ V,
                                                      const typename P::X* __restrict__ x,
                                                      typename P::A* __restrict__ T, int32_t alpha,
                                                      typename P::A* __restrict__ acc, int32_t n_acc,
                                                      unsigned* __restrict__ barrier)
{
    const int32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < alpha) T[i] = P::leaf(V[tval[i]], x[tcol[i]]);
    if (i < n_acc) acc[i] = P::ident();
    if (i == 0) {  // the tail kernel's grid barrier counts rounds from 0 in every sweep
        barrier[0] = 0;
        barrier[kFlagOffset] = 0;
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
    int32_t cur, nb;       // arena offset of this level's buffer; binary node count
    int32_t prev, alpha;   // arena offset of the level below; terminals (arena offsets below alpha)
    int32_t n_rows;        // stride of the per-slice row accumulators
    int32_t team_log2;     // lanes per emission group = 1 << team_log2 (<= 64)
    int32_t pb_bin, pb_pt, pb_emit;  // workgroups per slice in each part
    int32_t bsl[kSlices + 1], psl[kSlices + 1], gsl[kSlices + 1];
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
        for (int u = 0; u < kBinItems; ++u) v[u] = P::comb(arena[c[u].x], arena[c[u].y]);
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
        for (int u = 0; u < kBinItems; ++u) v[u] = arena[src[u]];
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
        // acc is y itself: store 1 where this lane's roots OR to 1
        const A part = emit_rounds<P>(a.epos, a.eoff[g] + sub, a.eoff[g + 1], team, valid,
                                      [&](int32_t c) { return arena[c]; });
        if (valid) direct(acc + a.erow[g], part);
        return;
    }
    // the accumulator is read beside the roots (its address needs only the
    // group's row), not after the team has combined them
    A* r = acc + (int64_t)x * a.n_rows + a.erow[g];
    const A old = *r;
    const int32_t e1 = a.eoff[g + 1];
    const A s0 = emit_rounds<P>(a.epos, a.eoff[g] + sub, e1, team, valid, [&](int32_t c) { return arena[c]; });
    issue_before(old);
    const A s = team_combine<P>(s0, team);
    if (valid && sub == 0) *r = P::comb(old, s);
}

// One wide level.  By default the grid has one workgroup per virtual block
// (measured faster on MI355X than a grid capped near the resident count);
// with a cap, each workgroup strides over the level's virtual blocks.  The
// stride (gridDim.x) is a multiple of kSlices, so a workgroup keeps serving
// the same slice on the same XCD.
template <class P>
__global__ __launch_bounds__(kBlock) void level_kernel(LevelArgs a, typename P::A* __restrict__ arena,
                                                       typename P::A* __restrict__ acc)
{
    const int32_t nvb = kSlices * (a.pb_bin + a.pb_pt + a.pb_emit);
    for (int32_t vb = blockIdx.x; vb < nvb; vb += gridDim.x) level_block<P>(a, vb, threadIdx.x, arena, acc);
}

// Grid-wide barrier for the co-resident tail grid.  bar[0] counts arrivals
// in this sweep; bar[kFlagOffset] (another cache line) holds the last round
// released.  Every wave first waits for its own stores to complete; one lane
// per workgroup then arrives with a device-scope release increment, the last
// arriver of the round publishes the round number with a release store, and
// the others poll that flag with relaxed device-scope loads (pollers never
// touch the line the arrivals update) and acquire once it is released.  The
// wait is bounded: after about a second of polling the workgroup gives up and
// returns false (the caller flags the sweep as failed), so the grid always
// drains.
__device__ __forceinline__ bool grid_barrier(unsigned* bar, unsigned round, const int* err)
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
        } else if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            unsigned spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < round) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins == (1u << 25)) {
                    ok = 0;
                    break;
                }
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

// vals[i] = arena[stage[i]] for i in [lo, hi)
template <class A>
__device__ __forceinline__ void stage_values(const int32_t* stage, const A* __restrict__ arena, A* vals, int32_t lo,
                                             int32_t hi, int32_t tid)
{
    block_rounds(hi - lo, tid, [&](int32_t i0, int32_t i1, int32_t i2, int32_t i3, bool l1, bool l2, bool l3) {
        const A v0 = arena[stage[lo + i0]], v1 = arena[stage[lo + i1]];
        const A v2 = arena[stage[lo + i2]], v3 = arena[stage[lo + i3]];
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
    stage_values<A>(f.idx + f.stage_word, arena, (A*)(flat_lds + f.vals_off), 0, f.n_terms, tid);
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
                                                          int* __restrict__ err)
{
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
        if (!grid_barrier(bar, ++round, err) && threadIdx.x == 0)
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (f.n_ent > 0) {
        if (flat_wg) flat_phase<P>(f, arena, acc);
        if (!grid_barrier(bar, ++round, err) && threadIdx.x == 0)
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (!kDirectEmit<P>) {
        for (int32_t r = blockIdx.x * kTailBlock + threadIdx.x; r < n_rows; r += gridDim.x * kTailBlock) {
            typename P::A s = acc[r];
#pragma unroll
            for (int x = 1; x < kSlices; ++x) s = P::comb(s, acc[(int64_t)x * n_rows + r]);
            y[r] = P::emit(accumulate ? y[r] : P::yzero(), s);
        }
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
    auto fetch = [&](int32_t c) -> R {
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
        for (int u = 0; u < kBinItems; ++u) v[u] = comb_row<P, VW>(fetch(c[u].x), fetch(c[u].y));
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
        for (int u = 0; u < kBinItems; ++u) v[u] = fetch(src[u]);
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
        int32_t p[kEmitItems];
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) p[u] = a.epos[min(e + u, e1 - 1)];
        R v[kEmitItems];
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) v[u] = fetch(p[u]);
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u) issue_before_row(v[u]);
#pragma unroll
        for (int u = 0; u < kEmitItems; ++u)
            if (e + u < e1) s = comb_row<P, VW>(s, v[u]);
        e += kEmitItems;
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
    int64_t tail_k0 = 1, tail_nent = 0;  // levels tail_k0..L and the last emission run in the tail kernel
    int64_t tail_multi = 0;              // of which the first tail_multi run on the whole tail grid
    int32_t tail_wgs = 0;
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
size_t x_bytes(gcs_policy p) { return p == GCS_PLUS_F32 || p == GCS_PLUS_F32_ACC_F64 ? 4 : elem_bytes(p); }
size_t y_bytes(gcs_policy p) { return elem_bytes(p); }
size_t v_bytes(gcs_policy p) { return elem_bytes(p); }

inline size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct Image {
    size_t child, ptsrc, erow, eoff, epos, tcol, tval, V, table, flat, total;
};

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
    Image m{};
    size_t o = 0;
    m.child = o;
    o = al256(o + g.child.size() * 4);
    m.ptsrc = o;
    o = al256(o + g.ptsrc.size() * 4);
    m.erow = o;
    o = al256(o + g.erow.size() * 4);
    m.eoff = o;
    o = al256(o + g.eoff.size() * 4);
    m.epos = o;
    o = al256(o + g.epos.size() * 4);
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
        if (l.base < 0 || l.base + l.nb + l.npt > arena) return false;
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
    a.erow = d->erow + e.grp_off;
    a.eoff = d->eoff + e.grp_off;
    a.epos = d->epos;
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
        leaf_kernel<P><<<std::max(1, ceil_div(std::max<int64_t>(d->alpha, n_acc), kBlock)), kBlock, 0, s>>>(
            d->tcol, d->tval, (const typename P::W*)d->V, (const typename P::X*)xv, arena, (int32_t)d->alpha, acc,
            n_acc, d->barrier);
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
        void* args[] = {&table, &n_multi, &n_grid, &flat, &arena, &acc, &y, &n_rows, &accumulate, &bar, &errp};
        const unsigned wgs = (unsigned)d->tail_wgs + (flat.n_ent > 0 ? 1u : 0u);
        hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&tail_kernel<P>), dim3(wgs),
                                                  dim3(kTailBlock), args, d->flat_lds, s);
        if (e != hipSuccess) return hip_fail(e, "tail launch (cooperative)");
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
        if (grid <= 0) continue;
        if (leaves) launch_level_batch<P, true>(VW, grid, ba, arena, acc, s);
        else launch_level_batch<P, false>(VW, grid, ba, arena, acc, s);
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
    auto* base = (unsigned char*)grammar_dev;
    struct Sec {
        size_t off;
        const void* src;
        size_t bytes;
    } secs[] = {
        {im.child, g.child.data(), g.child.size() * 4}, {im.ptsrc, g.ptsrc.data(), g.ptsrc.size() * 4},
        {im.erow, g.erow.data(), g.erow.size() * 4},    {im.eoff, g.eoff.data(), g.eoff.size() * 4},
        {im.epos, g.epos.data(), g.epos.size() * 4},    {im.tcol, g.tcol.data(), g.tcol.size() * 4},
        {im.tval, g.tval.data(), g.tval.size() * 4},    {im.V, vbuf.data(), vbuf.size()},
    };
    for (const Sec& c : secs) {
        if (!c.bytes) continue;
        e = hipMemcpyAsync(base + c.off, c.src, c.bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipMemcpyAsync (upload)");
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return gcs::hip_fail(e, "hipStreamSynchronize (upload)");

    auto* d = new gcs_device();
    d->policy = p;
    d->device = dev;
    d->n_rows = g.n_rows;
    d->n_cols = g.n_cols;
    d->alpha = g.alpha();
    d->L = g.L;
    d->arena_len = g.arena;
    d->lv = g.lv;
    // emission team per level: about GCS_EMIT_PER_LANE (default 4) roots per
    // lane, at most one wave
    const char* pl_env = std::getenv("GCS_EMIT_PER_LANE");
    const double per_lane = pl_env ? std::max(0.5, std::atof(pl_env)) : 4.0;
    d->team_log2.assign(g.lv.size(), 0);
    for (size_t k = 0; k < g.lv.size(); ++k) {
        const gcs::Level& l = g.lv[k];
        if (l.ngrp == 0) continue;
        const int64_t roots = g.eoff[l.grp_off + l.ngrp] - g.eoff[l.grp_off];
        const double mean = (double)roots / (double)l.ngrp;
        int t = 0;
        while (t < 6 && (double)(1 << t) * per_lane < mean && (l.ngrp << (t + 1)) < (int64_t)INT32_MAX - gcs::kBlock) ++t;
        d->team_log2[k] = t;
    }
    d->child = (const int2*)(base + im.child);
    d->ptsrc = (const int32_t*)(base + im.ptsrc);
    d->erow = (const int32_t*)(base + im.erow);
    d->eoff = (const int32_t*)(base + im.eoff);
    d->epos = (const int32_t*)(base + im.epos);
    d->tcol = (const int32_t*)(base + im.tcol);
    d->tval = (const int32_t*)(base + im.tval);
    d->V = base + im.V;
    d->arena = workspace_dev;
    d->acc = (unsigned char*)workspace_dev + gcs::arena_bytes(g, p);
    d->counters = (unsigned long long*)((unsigned char*)workspace_dev + gcs::arena_bytes(g, p) + gcs::acc_bytes(g, p));
    d->barrier = (unsigned*)(d->counters + 2);
    d->err = (int*)(d->counters + 3);
    // launch arguments of every level; the narrow levels at the top go to the
    // persistent tail kernel: from the first level k0 after which no launch
    // needs more than tail_vb virtual blocks per tail workgroup
    int dev_cu = 0;
    (void)hipDeviceGetAttribute(&dev_cu, hipDeviceAttributeMultiprocessorCount, dev);
    int coop = 0;
    (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (!coop) {
        delete d;
        gcs::set_error("the device does not support cooperative launches");
        return GCS_EHIP;
    }
    auto env_int = [](const char* name, int dflt) {
        const char* v = std::getenv(name);
        return v ? std::atoi(v) : dflt;
    };
    // 16 workgroups (2 per XCD), one virtual block per 256-lane quarter and
    // level: measured best on MI355X for the tail (fewer arrivals per barrier
    // round; the wider levels this leaves out run faster as launches)
    // (at most one fewer than the compute units: the narrow levels' workgroup
    // joins the cooperative grid, and each of these workgroups needs a CU)
    d->tail_wgs = std::max(gcs::kSlices, (std::min(env_int("GCS_TAIL_WGS", 16), std::max(dev_cu - 1, gcs::kSlices)) /
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
    d->tail_nent = g.L + 2 - d->tail_k0;
    // the narrowest entries at the end run on workgroup 0 alone, in LDS: as
    // many as fit its budget, each with at most GCS_TAIL_FLAT work items
    {
        int max_lds = 0;
        (void)hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        const size_t budget = std::min(gcs::kFlatLdsMax, (size_t)std::max(0, max_lds - 2048));
        d->flat_budget = budget;
        gcs::FlatImage fi;
        const bool direct = p == GCS_BOOL_OR || p == GCS_MIN_PLUS_F32 || p == GCS_MIN_PLUS_F64;
        if (!gcs::build_flat(g, d, gcs::elem_bytes(p), budget, env_int("GCS_TAIL_FLAT", 4096), direct, fi)) {
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
    hipStream_t s = (hipStream_t)stream;
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
        e = hipMemcpyAsync(d->pinned, d->counters + slot, 8, hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipMemcpyAsync (bfs count)");
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return gcs::hip_fail(e, "hipStreamSynchronize (bfs)");
        const int64_t c = d->pinned[0];
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
