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
#include <cstdlib>
#include <cstring>
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

// lane exchange inside a wave for every arena type
__device__ inline double xchg(double v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline float xchg(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ inline int64_t xchg(int64_t v, int m) { return __shfl_xor((long long)v, m, 64); }
__device__ inline uint8_t xchg(uint8_t v, int m) { return (uint8_t)__shfl_xor((int)v, m, 64); }

// ---------------------------------------------------------------- kernels

constexpr int kBlock = 256;
constexpr int kBinItems = 4;  // binary nodes per lane (independent gathers in flight)

template <class P>
__global__ __launch_bounds__(kBlock) void leaf_kernel(const int32_t* __restrict__ tcol,
                                                      const int32_t* __restrict__ tval,
                                                      const typename P::W* __restrict__ V,
                                                      const typename P::X* __restrict__ x,
                                                      typename P::A* __restrict__ T, int32_t alpha,
                                                      typename P::Y* __restrict__ y, int32_t n_rows)
{
    const int32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < alpha) T[i] = P::leaf(V[tval[i]], x[tcol[i]]);
    if (i < n_rows) y[i] = P::yzero();
}

struct LevelArgs {
    const int2* child;     // this level's binary nodes
    const int32_t* ptsrc;  // this level's pass-through sources
    const int32_t* erow;   // emission groups of the previous level
    const int32_t* eoff;
    const int32_t* epos;
    int32_t nb, npt, xcd_remap, ngrp;
    int32_t cur;           // arena offset of this level's buffer
    int32_t blk_bin, blk_pt;
    int32_t team_log2;     // lanes per emission group = 1 << team_log2 (<= 64)
};

template <class P>
__global__ __launch_bounds__(kBlock) void level_kernel(LevelArgs a, typename P::A* __restrict__ arena,
                                                       typename P::Y* __restrict__ y)
{
    using A = typename P::A;
    int32_t b = blockIdx.x;
    if (a.xcd_remap) {
        // workgroups are dealt to the 8 XCDs round-robin; renumber them so
        // that each XCD (and its L2) works on one contiguous share of the
        // level, whose children sit together in the level below
        const int32_t G = gridDim.x, x = b & 7, i = b >> 3, q = G >> 3, r = G & 7;
        b = x * q + (x < r ? x : r) + i;
    }
    if (b < a.blk_bin) {
        const int32_t t0 = b * (kBlock * kBinItems) + threadIdx.x;
        int2 c[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            c[u] = t < a.nb ? a.child[t] : make_int2(0, 0);
        }
        A v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = P::comb(arena[c[u].x], arena[c[u].y]);
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            if (t < a.nb) arena[a.cur + t] = v[u];
        }
    } else if (b < a.blk_bin + a.blk_pt) {
        const int32_t t0 = (b - a.blk_bin) * (kBlock * kBinItems) + threadIdx.x;
        int32_t src[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            src[u] = t < a.npt ? a.ptsrc[t] : 0;
        }
        A v[kBinItems];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) v[u] = arena[src[u]];
#pragma unroll
        for (int u = 0; u < kBinItems; ++u) {
            const int32_t t = t0 + u * kBlock;
            if (t < a.npt) arena[a.cur + a.nb + t] = v[u];
        }
    } else {
        // a team of 2^team_log2 adjacent lanes per (row, level) group: lanes
        // stride over the group's roots, then a fixed xor butterfly combines
        // the team (deterministic), and the team's first lane updates y[row]
        const int32_t gl = (b - a.blk_bin - a.blk_pt) * kBlock + threadIdx.x;
        const int32_t team = 1 << a.team_log2;
        const int32_t g = gl >> a.team_log2, sub = gl & (team - 1);
        A s = P::ident();
        if (g < a.ngrp) {
            const int32_t e1 = a.eoff[g + 1];
            for (int32_t e = a.eoff[g] + sub; e < e1; e += team) s = P::comb(s, arena[a.epos[e]]);
        }
        for (int32_t o = team >> 1; o > 0; o >>= 1) s = P::comb(s, xchg(s, o));
        if (g < a.ngrp && sub == 0) {
            const int32_t row = a.erow[g];
            y[row] = P::emit(y[row], s);
        }
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
    std::vector<gcs::Level> lv;
    std::vector<int32_t> team_log2;  // per level: lanes per emission group
    int32_t xcd_remap;
    const int2* child;
    const int32_t* ptsrc;
    const int32_t *erow, *eoff, *epos, *tcol, *tval;
    const void* V;
    void* arena;
    unsigned long long* counters;
    int64_t* pinned;
    // profiling
    std::vector<hipEvent_t> events;
    int64_t prof_max = 0, prof_used = 0;
    bool profiling = false;
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
    }
    return 0;
}
size_t x_bytes(gcs_policy p) { return p == GCS_PLUS_F32 || p == GCS_PLUS_F32_ACC_F64 ? 4 : elem_bytes(p); }
size_t y_bytes(gcs_policy p) { return elem_bytes(p); }
size_t v_bytes(gcs_policy p) { return elem_bytes(p); }

inline size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct Image {
    size_t child, ptsrc, erow, eoff, epos, tcol, tval, V, total;
};

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
    m.total = o > 0 ? o : 256;
    return m;
}

size_t workspace_bytes(const Grammar& g, gcs_policy p) { return al256((size_t)g.arena * elem_bytes(p)) + 256; }

bool valid_policy(int p) { return p >= GCS_PLUS_F64 && p <= GCS_PLUS_I64; }

// Every index a kernel dereferences must stay inside its buffer: children,
// pass-through sources and emission positions inside the arena, emission rows
// inside y, terminal descriptors inside x and V.  Checked once per upload.
bool layout_in_bounds(const Grammar& g)
{
    const int64_t arena = g.arena, alpha = g.alpha();
    for (int32_t c : g.child)
        if (c < 0 || c >= arena) return false;
    for (int32_t c : g.ptsrc)
        if (c < 0 || c >= arena) return false;
    int64_t co = 0, po = 0;
    for (int k = 1; k <= g.L; ++k) {
        const Level& l = g.lv[k];
        if (l.base < 0 || l.base + l.nb + l.npt > arena) return false;
        if (l.child_off != co || l.pt_off != po) return false;
        co += l.nb;
        po += l.npt;
    }
    if (2 * co != (int64_t)g.child.size() || po != (int64_t)g.ptsrc.size()) return false;
    for (size_t i = 0; i + 1 < g.eoff.size(); ++i)
        if (g.eoff[i] < 0 || g.eoff[i] > g.eoff[i + 1]) return false;
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

// launches of one sweep with work in them
int64_t count_launches(const gcs_device* d)
{
    int64_t c = std::max<int64_t>(d->alpha, d->n_rows) > 0 ? 1 : 0;
    for (int64_t k = 1; k <= d->L + 1; ++k) {
        const int64_t w = (k <= d->L ? d->lv[k].nb + d->lv[k].npt : 0) + d->lv[k - 1].ngrp;
        c += w > 0;
    }
    return c;
}

template <class P>
gcs_status run_sweep(gcs_device* d, const void* xv, void* yv, hipStream_t s, hipEvent_t* ev = nullptr)
{
    using A = typename P::A;
    auto* arena = (A*)d->arena;
    auto* y = (typename P::Y*)yv;
    int64_t li = 0;
    auto mark = [&]() {
        if (ev) (void)hipEventRecord(ev[li++], s);
    };
    const int32_t leaf_n = (int32_t)std::max<int64_t>(d->alpha, d->n_rows);
    if (leaf_n > 0) mark();
    if (leaf_n > 0)
        leaf_kernel<P><<<(leaf_n + kBlock - 1) / kBlock, kBlock, 0, s>>>(
            d->tcol, d->tval, (const typename P::W*)d->V, (const typename P::X*)xv, arena, (int32_t)d->alpha, y,
            (int32_t)d->n_rows);
    for (int64_t k = 1; k <= d->L + 1; ++k) {
        LevelArgs a{};
        if (k <= d->L) {
            const Level& l = d->lv[k];
            a.child = d->child + l.child_off;
            a.ptsrc = d->ptsrc + l.pt_off;
            a.nb = (int32_t)l.nb;
            a.npt = (int32_t)l.npt;
            a.cur = (int32_t)l.base;
        }
        const Level& e = d->lv[k - 1];
        a.erow = d->erow + e.grp_off;
        a.eoff = d->eoff + e.grp_off;
        a.epos = d->epos;
        a.ngrp = (int32_t)e.ngrp;
        a.blk_bin = (a.nb + kBlock * kBinItems - 1) / (kBlock * kBinItems);
        a.blk_pt = (a.npt + kBlock * kBinItems - 1) / (kBlock * kBinItems);
        a.xcd_remap = d->xcd_remap;
        a.team_log2 = d->team_log2[k - 1];
        const int32_t blk_emit = (int32_t)(((int64_t)a.ngrp << a.team_log2) + kBlock - 1) / kBlock;
        const int32_t grid = a.blk_bin + a.blk_pt + blk_emit;
        if (grid > 0) {
            mark();
            level_kernel<P><<<grid, kBlock, 0, s>>>(a, arena, y);
        }
    }
    mark();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_fail(err, "sweep launch");
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
        case GCS_PLUS_F32_ACC_F64: {
            double v = g.V[i];
            std::memcpy(o, &v, 8);
            break;
        }
        case GCS_PLUS_F32: {
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
    d->lv = g.lv;
    {
        const char* e = std::getenv("GCS_XCD_REMAP");
        d->xcd_remap = e ? std::atoi(e) != 0 : 1;
    }
    // emission team per level: about four roots per lane, at most one wave
    d->team_log2.assign(g.lv.size(), 0);
    for (size_t k = 0; k < g.lv.size(); ++k) {
        const gcs::Level& l = g.lv[k];
        if (l.ngrp == 0) continue;
        const int64_t roots = g.eoff[l.grp_off + l.ngrp] - g.eoff[l.grp_off];
        const double per_lane = 4.0, mean = (double)roots / (double)l.ngrp;
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
    d->counters = (unsigned long long*)((unsigned char*)workspace_dev + gcs::al256((size_t)g.arena *
                                                                                  gcs::elem_bytes(p)));
    d->pinned = nullptr;
    e = hipHostMalloc((void**)&d->pinned, 64, hipHostMallocDefault);
    if (e != hipSuccess) {
        delete d;
        return gcs::hip_fail(e, "hipHostMalloc");
    }
    *out = d;
    return GCS_OK;
}

static gcs_status sweep_dispatch(gcs_device* d, const void* x_dev, void* y_dev, void* stream, hipEvent_t* ev)
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
    case GCS_PLUS_F64: return gcs::run_sweep<gcs::PolPlusF64>(d, x_dev, y_dev, s, ev);
    case GCS_PLUS_F32: return gcs::run_sweep<gcs::PolPlusF32>(d, x_dev, y_dev, s, ev);
    case GCS_PLUS_F32_ACC_F64: return gcs::run_sweep<gcs::PolPlusF32AccF64>(d, x_dev, y_dev, s, ev);
    case GCS_BOOL_OR: return gcs::run_sweep<gcs::PolBoolOr>(d, x_dev, y_dev, s, ev);
    case GCS_PLUS_I64: return gcs::run_sweep<gcs::PolPlusI64>(d, x_dev, y_dev, s, ev);
    }
    gcs::set_error("corrupt device handle");
    return GCS_ESTATE;
}

extern "C" gcs_status gcs_sweep_right(gcs_device* d, const void* x_dev, void* y_dev, void* stream)
{
    return sweep_dispatch(d, x_dev, y_dev, stream, nullptr);
}

extern "C" int64_t gcs_sweep_launches(const gcs_device* d) { return d ? gcs::count_launches(d) : 0; }

static void release_events(gcs_device* d)
{
    for (hipEvent_t e : d->events) (void)hipEventDestroy(e);
    d->events.clear();
    d->profiling = false;
    d->prof_max = d->prof_used = 0;
}

extern "C" gcs_status gcs_profile_begin(gcs_device* d, int64_t max_sweeps)
{
    if (!d || max_sweeps <= 0) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    gcs::DeviceGuard guard(d->device);
    release_events(d);
    const int64_t per = gcs::count_launches(d) + 1;
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
    const int64_t per = gcs::count_launches(d) + 1;
    gcs_status st = sweep_dispatch(d, x_dev, y_dev, stream, d->events.data() + per * d->prof_used);
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
    const int64_t nl = gcs::count_launches(d), per = nl + 1;
    *sweeps = d->prof_used;
    *launches = nl;
    if (cap < d->prof_used * nl || (cap > 0 && !launch_ms)) {
        release_events(d);
        gcs::set_error("launch_ms too small");
        return GCS_ERANGE;
    }
    for (int64_t s = 0; s < d->prof_used; ++s) {
        hipError_t err = hipEventSynchronize(d->events[per * s + nl]);
        if (err != hipSuccess) {
            release_events(d);
            return gcs::hip_fail(err, "hipEventSynchronize");
        }
        for (int64_t i = 0; i < nl; ++i) {
            float ms = 0;
            err = hipEventElapsedTime(&ms, d->events[per * s + i], d->events[per * s + i + 1]);
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

extern "C" void gcs_free_device(gcs_device* d)
{
    if (!d) return;
    release_events(d);
    if (d->pinned) (void)hipHostFree(d->pinned);
    delete d;
}
