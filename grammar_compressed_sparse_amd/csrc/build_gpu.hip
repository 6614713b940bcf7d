// Device builder: the CSRV string and round-based RePair (rounds.hpp) on the
// GPU; levels, pass-through completion and layout stay on the host
// (finish_layout).  Page: "Right Multiplication on Grammar-Compressed
// Matrices: A Streaming, Memory-Bounded GPU Engine", section 2 ('CSRV',
// 'Grammar') and section 4.1.
//
// The sequence lives on the device as 32-bit words (symbol | row-end mark in
// bit 31).  One round is eight launches:
//   clear     the pair table (a prefix of the workspace table sized for the
//             round) and the round's counters
//   count     every position with a right neighbour in its row inserts its
//             pair into an open-addressing table (64-bit keys, CAS insert,
//             linear probing) and adds 1 to its count; per-block maxima and
//             insert counts give the largest count and the distinct pairs
//   -- the host reads those 24 bytes: table too full -> retry with a larger
//      prefix; largest count < 2 -> done
//   cand      per position: its pair's count if it reaches the threshold
//   win       per position: outranks both overlapping candidates? then add
//             one win to its pair and keep the smallest winning position
//   mark      replaced = won and the pair won at least twice; new rule = the
//             pair's first winning position; kept = the left neighbour was not
//             replaced; per-block counts
//   scan      exclusive prefix sums of the block counts (one workgroup)
//   assign    rule ids in position order, rules written out
//   rewrite   kept positions compacted into the other sequence buffer
//   -- the host reads the totals
// The ranked kernels give every block 4096 consecutive positions and rank
// inside it with wave ballots, so every number depends only on the input:
// the result is the host round-based RePair's, bit for bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "grammar.hpp"
#include "rounds.hpp"
#include "staging.hpp"

namespace gcs {
namespace gb {

using namespace rounds;

constexpr int kThreads = 256;
constexpr int kIters = 16;
constexpr int64_t kChunk = (int64_t)kThreads * kIters;  // positions per block of the ranked kernels
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
constexpr unsigned long long kEmpty = ~0ULL;
constexpr int kMaxProbe = 256;
constexpr int kScanThreads = 1024;

struct Ctrl {
    uint32_t fmax;       // largest pair count of the round
    uint32_t overflow;   // a probe sequence exceeded kMaxProbe
    uint32_t total_new;  // rules made by the round
    uint32_t total_keep; // sequence length after the round
    unsigned long long distinct;  // distinct pairs inserted
    unsigned long long pad[5];
};

// ------------------------------------------------------------ kernels

__device__ inline uint32_t wave_max(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ inline uint32_t wave_sum(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
    return v;
}

// terminal id of every nonzero: cbase[j] + the value indices of column j below
// its own (CSRV's <l, j>, compacted); code[k] is the value index (int8
// values through the table code_of, or the code itself for pre-coded input)
__global__ __launch_bounds__(kThreads) void k_terms(const int32_t* __restrict__ col, const int8_t* __restrict__ val,
                                                    int ones, const uint64_t* __restrict__ cmask,
                                                    const int32_t* __restrict__ cbase,
                                                    const int32_t* __restrict__ code_of, uint32_t* __restrict__ seq,
                                                    int64_t nnz)
{
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * kThreads) {
        const int32_t j = col[k];
        const int32_t vi = ones ? 0 : code_of[(int)val[k] + 128];
        seq[k] = (uint32_t)(cbase[j] + __popcll(cmask[j] & ((1ULL << vi) - 1ULL)));
    }
}

__global__ __launch_bounds__(kThreads) void k_rowend(const int64_t* __restrict__ rp, int64_t n_rows,
                                                     uint32_t* __restrict__ seq)
{
    for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < n_rows; r += (int64_t)gridDim.x * kThreads)
        if (rp[r + 1] > rp[r]) seq[rp[r + 1] - 1] |= kEnd;
}

__global__ __launch_bounds__(kThreads) void k_clear(unsigned long long* __restrict__ key, uint32_t* __restrict__ cnt,
                                                    uint32_t* __restrict__ wins, uint32_t* __restrict__ first,
                                                    int64_t T, Ctrl* ctrl)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctrl->fmax = 0;
        ctrl->overflow = 0;
        ctrl->distinct = 0;
    }
    for (int64_t h = (int64_t)blockIdx.x * kThreads + threadIdx.x; h < T; h += (int64_t)gridDim.x * kThreads) {
        key[h] = kEmpty;
        cnt[h] = 0;
        wins[h] = 0;
        first[h] = 0xFFFFFFFFu;
    }
}

__global__ __launch_bounds__(kThreads) void k_count(const uint32_t* __restrict__ seq, int64_t n,
                                                    uint32_t* __restrict__ slot, unsigned long long* key,
                                                    uint32_t* cnt, uint64_t mask, Ctrl* ctrl)
{
    __shared__ uint32_t s_max[kThreads / 64], s_ins[kThreads / 64], s_ovf[kThreads / 64];
    uint32_t lmax = 0, lins = 0, lovf = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        const uint32_t w = seq[i];
        uint32_t s = kNoSlot;
        if (!(w & kEnd)) {
            const unsigned long long k = pair_key(w & kSym, seq[i + 1] & kSym);
            uint64_t h = (uint64_t)pair_hash(k) & mask;
            bool found = false;
            for (int p = 0; p <= kMaxProbe; ++p) {
                unsigned long long cur = __hip_atomic_load(&key[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (cur == kEmpty) {
                    cur = atomicCAS(&key[h], kEmpty, k);
                    if (cur == kEmpty) {
                        ++lins;
                        found = true;
                        break;
                    }
                }
                if (cur == k) {
                    found = true;
                    break;
                }
                h = (h + 1) & mask;
            }
            if (found) {
                lmax = max(lmax, atomicAdd(&cnt[h], 1u) + 1u);
                s = (uint32_t)h;
            } else {
                lovf = 1;
            }
        }
        slot[i] = s;
    }
    lmax = wave_max(lmax);
    lins = wave_sum(lins);
    lovf = wave_max(lovf);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_max[wv] = lmax;
        s_ins[wv] = lins;
        s_ovf[wv] = lovf;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = 0, c = 0, o = 0;
        for (int x = 0; x < kThreads / 64; ++x) {
            m = max(m, s_max[x]);
            c += s_ins[x];
            o |= s_ovf[x];
        }
        if (m) atomicMax(&ctrl->fmax, m);
        if (c) atomicAdd(&ctrl->distinct, (unsigned long long)c);
        if (o) atomicOr(&ctrl->overflow, 1u);
    }
}

__global__ __launch_bounds__(kThreads) void k_cand(const uint32_t* __restrict__ slot, const uint32_t* __restrict__ cnt,
                                                   uint32_t tau, uint32_t* __restrict__ cpos, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        const uint32_t s = slot[i];
        const uint32_t c = s != kNoSlot ? cnt[s] : 0u;
        cpos[i] = c >= tau ? c : 0u;
    }
}

__global__ __launch_bounds__(kThreads) void k_win(const uint32_t* __restrict__ seq, const uint32_t* __restrict__ slot,
                                                  const uint32_t* __restrict__ cpos, uint32_t* wins, uint32_t* first,
                                                  uint8_t* __restrict__ flag, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        uint8_t won = 0;
        const uint32_t c = cpos[i];
        if (c) {  // a candidate has a right neighbour in its row: i + 1 < n
            const uint32_t a = seq[i] & kSym, b = seq[i + 1] & kSym;
            const uint64_t k = pair_key(a, b);
            const uint64_t r = rank(c, k);
            bool w = true;
            if (i > 0) {
                const uint32_t cl = cpos[i - 1];
                if (cl) {
                    const uint64_t kl = pair_key(seq[i - 1] & kSym, a);
                    w = outranks(r, k, rank(cl, kl), kl);
                }
            }
            if (w) {
                const uint32_t cr = cpos[i + 1];
                if (cr) {  // then i + 1 has a right neighbour too
                    const uint64_t kr = pair_key(b, seq[i + 2] & kSym);
                    w = outranks(r, k, rank(cr, kr), kr);
                }
            }
            if (w) {
                const uint32_t s = slot[i];
                atomicAdd(&wins[s], 1u);
                atomicMin(&first[s], (uint32_t)i);
                won = 1;
            }
        }
        flag[i] = won;
    }
}

// mk bits: 1 replaced, 2 first occurrence of a new rule, 4 kept
__device__ inline bool replaced(const uint8_t* flag, const uint32_t* slot, const uint32_t* wins, int64_t i)
{
    return flag[i] && wins[slot[i]] >= 2u;
}

__device__ inline void block_totals(uint32_t a, uint32_t b, uint32_t* out_a, uint32_t* out_b)
{
    __shared__ uint32_t s_a[kThreads / 64], s_b[kThreads / 64];
    a = wave_sum(a);
    b = wave_sum(b);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_a[wv] = a;
        s_b[wv] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t ta = 0, tb = 0;
        for (int x = 0; x < kThreads / 64; ++x) {
            ta += s_a[x];
            tb += s_b[x];
        }
        *out_a = ta;
        *out_b = tb;
    }
}

__global__ __launch_bounds__(kThreads) void k_mark(const uint8_t* __restrict__ flag, const uint32_t* __restrict__ slot,
                                                   const uint32_t* __restrict__ wins,
                                                   const uint32_t* __restrict__ first, uint8_t* __restrict__ mk,
                                                   uint32_t* __restrict__ blk_new, uint32_t* __restrict__ blk_keep,
                                                   int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    uint32_t nnew = 0, nkeep = 0;
    for (int it = 0; it < kIters; ++it) {
        const int64_t i = base + (int64_t)it * kThreads + threadIdx.x;
        if (i >= n) break;
        const bool rep = replaced(flag, slot, wins, i);
        const bool nw = rep && first[slot[i]] == (uint32_t)i;
        const bool keep = !(i > 0 && replaced(flag, slot, wins, i - 1));
        mk[i] = (uint8_t)((rep ? 1 : 0) | (nw ? 2 : 0) | (keep ? 4 : 0));
        nnew += nw;
        nkeep += keep;
    }
    block_totals(nnew, nkeep, &blk_new[blockIdx.x], &blk_keep[blockIdx.x]);
}

// exclusive scans of the per-block counts, one workgroup
__global__ __launch_bounds__(kScanThreads) void k_scan(const uint32_t* __restrict__ blk_new,
                                                       const uint32_t* __restrict__ blk_keep,
                                                       uint32_t* __restrict__ off_new, uint32_t* __restrict__ off_keep,
                                                       int64_t nblk, Ctrl* ctrl)
{
    __shared__ uint32_t s_a[kScanThreads], s_b[kScanThreads];
    const int64_t per = (nblk + kScanThreads - 1) / kScanThreads;
    const int64_t b0 = (int64_t)threadIdx.x * per, b1 = min(nblk, b0 + per);
    uint32_t a = 0, b = 0;
    for (int64_t x = b0; x < b1; ++x) {
        a += blk_new[x];
        b += blk_keep[x];
    }
    s_a[threadIdx.x] = a;
    s_b[threadIdx.x] = b;
    __syncthreads();
    for (int o = 1; o < kScanThreads; o <<= 1) {  // inclusive Hillis-Steele scan
        uint32_t va = threadIdx.x >= (unsigned)o ? s_a[threadIdx.x - o] : 0u;
        uint32_t vb = threadIdx.x >= (unsigned)o ? s_b[threadIdx.x - o] : 0u;
        __syncthreads();
        s_a[threadIdx.x] += va;
        s_b[threadIdx.x] += vb;
        __syncthreads();
    }
    uint32_t ra = s_a[threadIdx.x] - a, rb = s_b[threadIdx.x] - b;
    for (int64_t x = b0; x < b1; ++x) {
        off_new[x] = ra;
        off_keep[x] = rb;
        ra += blk_new[x];
        rb += blk_keep[x];
    }
    if (threadIdx.x == kScanThreads - 1) {
        ctrl->total_new = s_a[kScanThreads - 1];
        ctrl->total_keep = s_b[kScanThreads - 1];
    }
}

// rank of a predicate among the positions of this block in position order;
// returns the rank of the calling lane (valid where pred holds) and advances
// `running` by the iteration's total
__device__ inline uint32_t block_rank(bool pred, uint32_t& running, uint32_t* s_w)
{
    const unsigned long long bal = __ballot(pred);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t lrank = (uint32_t)__popcll(bal & ((1ULL << lane) - 1ULL));
    if (lane == 0) s_w[wv] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int x = 0; x < kThreads / 64; ++x) {
        if (x < wv) before += s_w[x];
        total += s_w[x];
    }
    __syncthreads();
    const uint32_t r = running + before + lrank;
    running += total;
    return r;
}

__global__ __launch_bounds__(kThreads) void k_assign(const uint32_t* __restrict__ seq,
                                                     const uint32_t* __restrict__ slot, const uint8_t* __restrict__ mk,
                                                     const uint32_t* __restrict__ off_new, uint32_t* __restrict__ ids,
                                                     uint32_t* __restrict__ rules, uint32_t nt_next, int64_t n)
{
    __shared__ uint32_t s_w[kThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    uint32_t running = off_new[blockIdx.x];
    for (int it = 0; it < kIters; ++it) {
        if (base + (int64_t)it * kThreads >= n) break;  // uniform over the block
        const int64_t i = base + (int64_t)it * kThreads + threadIdx.x;
        const bool nw = i < n && (mk[i] & 2);
        const uint32_t r = block_rank(nw, running, s_w);
        if (nw) {
            ids[slot[i]] = nt_next + r;
            rules[2 * (int64_t)r] = seq[i] & kSym;
            rules[2 * (int64_t)r + 1] = seq[i + 1] & kSym;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_rewrite(const uint32_t* __restrict__ seq,
                                                      const uint32_t* __restrict__ slot,
                                                      const uint8_t* __restrict__ mk,
                                                      const uint32_t* __restrict__ off_keep,
                                                      const uint32_t* __restrict__ ids, uint32_t* __restrict__ out,
                                                      int64_t n)
{
    __shared__ uint32_t s_w[kThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    uint32_t running = off_keep[blockIdx.x];
    for (int it = 0; it < kIters; ++it) {
        if (base + (int64_t)it * kThreads >= n) break;  // uniform over the block
        const int64_t i = base + (int64_t)it * kThreads + threadIdx.x;
        const uint8_t m = i < n ? mk[i] : (uint8_t)0;
        const uint32_t dst = block_rank((m & 4) != 0, running, s_w);
        if (m & 4) out[dst] = (m & 1) ? (ids[slot[i]] | (seq[i + 1] & kEnd)) : seq[i];
    }
}

// ------------------------------------------------------------ host side

inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
    size_t seq_a, seq_b, slot, cpos, flag, mk, blk_new, blk_keep, off_new, off_keep, rules, key, cnt, wins, first,
        ids, rowptr, cmask, cbase, code_of, ctrl, total;
};

int64_t default_table(int64_t nnz)
{
    int64_t t = 1024;
    while (t < 2 * nnz) t <<= 1;
    return t;
}

WsLayout ws_layout(int64_t n_rows, int64_t n_cols, int64_t nnz, int64_t T)
{
    WsLayout w{};
    const int64_t nblk = std::max<int64_t>(1, (nnz + kChunk - 1) / kChunk);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += up256(std::max<size_t>(bytes, 1));
        return at;
    };
    const size_t N = (size_t)std::max<int64_t>(nnz, 1);
    w.seq_a = take(4 * N);
    w.seq_b = take(4 * N);
    w.slot = take(4 * N);  // the uploaded column indices before the first round
    w.cpos = take(4 * N);
    w.flag = take(N);      // the uploaded int8 values before the first round
    w.mk = take(N);
    w.blk_new = take(4 * (size_t)nblk);
    w.blk_keep = take(4 * (size_t)nblk);
    w.off_new = take(4 * (size_t)nblk);
    w.off_keep = take(4 * (size_t)nblk);
    w.rules = take(8 * (N / 2 + 1));
    w.key = take(8 * (size_t)T);
    w.cnt = take(4 * (size_t)T);
    w.wins = take(4 * (size_t)T);
    w.first = take(4 * (size_t)T);
    w.ids = take(4 * (size_t)T);
    w.rowptr = take(8 * (size_t)(n_rows + 1));
    w.cmask = take(8 * (size_t)std::max<int64_t>(n_cols, 1));
    w.cbase = take(4 * (size_t)std::max<int64_t>(n_cols, 1));
    w.code_of = take(4 * 256);
    w.ctrl = take(sizeof(Ctrl));
    w.total = o;
    return w;
}

bool valid_table(int64_t T) { return T >= 1024 && T <= (1LL << 32) && (T & (T - 1)) == 0; }

gcs_status fail_hip(hipError_t e, const char* what)
{
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return GCS_EHIP;
}

double ms_since(std::chrono::steady_clock::time_point t0)
{
    return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

inline int grid_for(int64_t n)
{
    return (int)std::max<int64_t>(1, std::min<int64_t>((n + kThreads - 1) / kThreads, 65536));
}

gcs_status build(const gcs_csr_view* m, const gcs_build_opts* opts, int64_t table_entries, void* ws_dev,
                 size_t ws_bytes, hipStream_t st, Grammar& g)
{
    auto t0 = std::chrono::steady_clock::now();
    const bool trace = std::getenv("GCS_BUILD_TRACE") != nullptr;
    if (opts && (opts->col_chunk != 0 || opts->row_chunk != 0 || opts->row_order != GCS_ROWS_NATURAL ||
                 opts->repair != GCS_REPAIR_ROUNDS || opts->reserved != 0)) {
        set_error("the device builder runs round-based RePair on one tile: col_chunk = row_chunk = 0, natural row "
                  "order, repair = GCS_REPAIR_ROUNDS");
        return GCS_EINVAL;
    }
    const int threads = resolve_threads(opts ? opts->n_threads : 0);
    Csrv enc;
    if (gcs_status s = csrv_encode(m, threads, g, enc)) return s;
    if (!enc.small_v) {
        set_error("the device builder takes at most 64 distinct values (gcs_build_grammar takes any)");
        return GCS_EINVAL;
    }
    const int64_t n = m->n_rows, mc = m->n_cols;
    // stored zeros are dropped: compact a host copy first (rare)
    std::vector<int64_t> rp_f;
    std::vector<int32_t> col_f;
    std::vector<int8_t> code_f;
    const int64_t* rp = m->row_ptr;
    const int32_t* col = m->col;
    const int8_t* val8 = m->val_kind == GCS_VAL_I8 ? (const int8_t*)m->val : nullptr;
    int32_t code_of[256];
    for (int c = 0; c < 256; ++c) code_of[c] = enc.i8_index[c] < 0 ? 0 : enc.i8_index[c];
    const bool ones = m->val_kind == GCS_VAL_ONES;
    if (enc.has_zeros || m->val_kind == GCS_VAL_F64) {
        // value indices as int8 codes, zeros removed
        rp_f.assign((size_t)n + 1, 0);
        for (int64_t r = 0; r < n; ++r) {
            for (int64_t k = rp[r]; k < rp[r + 1]; ++k) {
                const int32_t vi = enc.vindex(k);
                if (vi < 0) continue;
                col_f.push_back(col[k]);
                code_f.push_back((int8_t)vi);
            }
            rp_f[r + 1] = (int64_t)col_f.size();
        }
        rp = rp_f.data();
        col = col_f.data();
        val8 = code_f.data();
        for (int c = 0; c < 256; ++c) code_of[c] = (c >= 128 && c < 128 + 64) ? c - 128 : 0;
    }
    const int64_t nnz = n > 0 ? rp[n] : 0;
    if (nnz >= (int64_t)INT32_MAX) {
        set_error("the device builder takes fewer than 2^31 - 1 nonzeros per call (build column groups)");
        return GCS_ERANGE;
    }
    const int64_t T = table_entries > 0 ? table_entries : default_table(nnz);
    if (!valid_table(T)) {
        set_error("table_entries must be 0 or a power of two in [2^10, 2^32]");
        return GCS_EINVAL;
    }
    const WsLayout W = ws_layout(n, mc, nnz, T);
    if (!ws_dev || ws_bytes < W.total || ((uintptr_t)ws_dev & 255)) {
        set_error("build workspace missing, misaligned or smaller than gcs_build_workspace_bytes");
        return GCS_EINVAL;
    }
    char* base = (char*)ws_dev;
    uint32_t* seq[2] = {(uint32_t*)(base + W.seq_a), (uint32_t*)(base + W.seq_b)};
    uint32_t* slot = (uint32_t*)(base + W.slot);
    uint32_t* cpos = (uint32_t*)(base + W.cpos);
    uint8_t* flag = (uint8_t*)(base + W.flag);
    uint8_t* mk = (uint8_t*)(base + W.mk);
    uint32_t* blk_new = (uint32_t*)(base + W.blk_new);
    uint32_t* blk_keep = (uint32_t*)(base + W.blk_keep);
    uint32_t* off_new = (uint32_t*)(base + W.off_new);
    uint32_t* off_keep = (uint32_t*)(base + W.off_keep);
    uint32_t* rules = (uint32_t*)(base + W.rules);
    unsigned long long* key = (unsigned long long*)(base + W.key);
    uint32_t* cnt = (uint32_t*)(base + W.cnt);
    uint32_t* wins = (uint32_t*)(base + W.wins);
    uint32_t* first = (uint32_t*)(base + W.first);
    uint32_t* ids = (uint32_t*)(base + W.ids);
    int64_t* d_rp = (int64_t*)(base + W.rowptr);
    uint64_t* d_cmask = (uint64_t*)(base + W.cmask);
    int32_t* d_cbase = (int32_t*)(base + W.cbase);
    int32_t* d_code = (int32_t*)(base + W.code_of);
    Ctrl* ctrl = (Ctrl*)(base + W.ctrl);

    const int64_t alpha = g.alpha();
    hipError_t e = hipSuccess;
    // CSRV on the device: columns, values, per-column masks and bases
    {
        std::vector<int32_t> cb((size_t)std::max<int64_t>(mc, 1), 0);
        for (int64_t j = 0; j < mc; ++j) cb[j] = (int32_t)enc.cbase[j];
        gcs::PinnedStage stage;  // the large host arrays go through pinned buffers
        e = stage.init();
        if (e == hipSuccess && nnz > 0) {
            e = stage.h2d(slot, col, 4 * (size_t)nnz, st);
            if (e == hipSuccess && !ones) e = stage.h2d(flag, val8, (size_t)nnz, st);
        }
        if (e == hipSuccess && n > 0) e = stage.h2d(d_rp, rp, 8 * (size_t)(n + 1), st);
        if (e == hipSuccess && mc > 0)
            e = hipMemcpyAsync(d_cmask, enc.cmask.data(), 8 * (size_t)mc, hipMemcpyHostToDevice, st);
        if (e == hipSuccess && mc > 0) e = hipMemcpyAsync(d_cbase, cb.data(), 4 * (size_t)mc, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipMemcpyAsync(d_code, code_of, sizeof(code_of), hipMemcpyHostToDevice, st);
        if (e == hipSuccess && nnz > 0) {
            k_terms<<<grid_for(nnz), kThreads, 0, st>>>((const int32_t*)slot, (const int8_t*)flag, ones ? 1 : 0,
                                                        d_cmask, d_cbase, d_code, seq[0], nnz);
            k_rowend<<<grid_for(n), kThreads, 0, st>>>(d_rp, n, seq[0]);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host arrays may go after this
        if (e != hipSuccess) return fail_hip(e, "device builder: CSRV upload");
    }
    g.t_csrv = ms_since(t0);
    auto t1 = std::chrono::steady_clock::now();

    int64_t len = nnz, R = 0, cur = 0, rounds = 0;
    int64_t Tr = std::min<int64_t>(T, std::max<int64_t>(1 << 16, default_table(nnz / 16)));
    Ctrl hc{};
    while (len > 1) {
        if (alpha + R + len / 2 >= (int64_t)kSym) {
            set_error("grammar exceeds the 31-bit symbol space of the device builder");
            return GCS_ERANGE;
        }
        k_clear<<<grid_for(Tr), kThreads, 0, st>>>(key, cnt, wins, first, Tr, ctrl);
        k_count<<<grid_for(len), kThreads, 0, st>>>(seq[cur], len, slot, key, cnt, (uint64_t)(Tr - 1), ctrl);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipMemcpyAsync(&hc, ctrl, sizeof(Ctrl), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return fail_hip(e, "device builder: pair count");
        // a probe ran past its limit (the count is incomplete), or the table
        // is more than 3/4 full (long probes): count again in a larger prefix
        if (hc.overflow || 4 * (int64_t)hc.distinct > 3 * Tr) {
            if (Tr >= T) {
                if (!hc.overflow) goto counted;  // complete, only slow
                set_error("device builder: the pair table is too small for this input (raise table_entries)");
                return GCS_ENOMEM;
            }
            Tr = std::min<int64_t>(T, Tr * 8);
            continue;
        }
    counted:
        if (hc.fmax < 2) break;
        const uint32_t tau = threshold(hc.fmax);
        const int64_t nblk = (len + kChunk - 1) / kChunk;
        k_cand<<<grid_for(len), kThreads, 0, st>>>(slot, cnt, tau, cpos, len);
        k_win<<<grid_for(len), kThreads, 0, st>>>(seq[cur], slot, cpos, wins, first, flag, len);
        k_mark<<<(unsigned)nblk, kThreads, 0, st>>>(flag, slot, wins, first, mk, blk_new, blk_keep, len);
        k_scan<<<1, kScanThreads, 0, st>>>(blk_new, blk_keep, off_new, off_keep, nblk, ctrl);
        k_assign<<<(unsigned)nblk, kThreads, 0, st>>>(seq[cur], slot, mk, off_new, ids, rules + 2 * R,
                                                       (uint32_t)(alpha + R), len);
        k_rewrite<<<(unsigned)nblk, kThreads, 0, st>>>(seq[cur], slot, mk, off_keep, ids, seq[cur ^ 1], len);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipMemcpyAsync(&hc, ctrl, sizeof(Ctrl), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return fail_hip(e, "device builder: round");
        const int64_t reps = len - (int64_t)hc.total_keep;
        if (trace)
            std::fprintf(stderr, "[gcs gpu build] round %lld: len %lld, distinct %llu (table %lld), max %u, tau %u, "
                                 "rules %u, replaced %lld\n",
                         (long long)rounds, (long long)len, hc.distinct, (long long)Tr, hc.fmax, tau, hc.total_new,
                         (long long)reps);
        R += hc.total_new;
        len = hc.total_keep;
        cur ^= 1;
        ++rounds;
        // next table: at most two new pairs per replacement
        Tr = std::min<int64_t>(T, std::max<int64_t>(1 << 16, default_table((int64_t)hc.distinct + 2 * reps)));
    }
    // results back to the host
    std::vector<uint32_t> hr((size_t)(2 * R)), hs((size_t)len);
    if (R > 0) e = hipMemcpyAsync(hr.data(), rules, 8 * (size_t)R, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess && len > 0) e = hipMemcpyAsync(hs.data(), seq[cur], 4 * (size_t)len, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(e, "device builder: copy back");
    g.ra.resize((size_t)R);
    g.rb.resize((size_t)R);
    for (int64_t i = 0; i < R; ++i) {
        g.ra[i] = (int32_t)hr[2 * i];
        g.rb[i] = (int32_t)hr[2 * i + 1];
    }
    g.c_off.assign((size_t)n + 1, 0);
    g.c_sym.resize((size_t)len);
    int64_t p = 0;
    for (int64_t r = 0; r < n; ++r) {
        if (rp[r + 1] > rp[r]) {
            while (p < len && !(hs[p] & kEnd)) g.c_sym[p] = (int32_t)hs[p], ++p;
            if (p >= len) {
                set_error("device builder: row structure lost (internal error)");
                return GCS_ESTATE;
            }
            g.c_sym[p] = (int32_t)(hs[p] & kSym);
            ++p;
        }
        g.c_off[r + 1] = p;
    }
    if (p != len) {
        set_error("device builder: row structure lost (internal error)");
        return GCS_ESTATE;
    }
    g.nnz = nnz;
    g.n_tiles = 1;
    g.t_repair = ms_since(t1);
    if (trace)
        std::fprintf(stderr, "[gcs gpu build] %lld rounds, |R| = %lld, |C| = %lld, CSRV %.1f ms, RePair %.1f ms\n",
                     (long long)rounds, (long long)R, (long long)len, g.t_csrv, g.t_repair);
    return finish_layout(g, threads);
}

}  // namespace gb
}  // namespace gcs

extern "C" gcs_status gcs_build_workspace_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz, int64_t table_entries,
                                                size_t* bytes)
{
    if (!bytes || n_rows < 0 || n_cols < 0 || nnz < 0) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const int64_t T = table_entries > 0 ? table_entries : gcs::gb::default_table(nnz);
    if (!gcs::gb::valid_table(T)) {
        gcs::set_error("table_entries must be 0 or a power of two in [2^10, 2^32]");
        return GCS_EINVAL;
    }
    *bytes = gcs::gb::ws_layout(n_rows, n_cols, nnz, T).total;
    return GCS_OK;
}

extern "C" gcs_status gcs_build_grammar_gpu(const gcs_csr_view* m, const gcs_build_opts* opts, int64_t table_entries,
                                            void* workspace_dev, size_t workspace_bytes, void* stream,
                                            gcs_grammar** out)
{
    if (!out) {
        gcs::set_error("null output pointer");
        return GCS_EINVAL;
    }
    *out = nullptr;
    try {
        auto* h = new gcs_grammar();
        gcs_status st = gcs::gb::build(m, opts, table_entries, workspace_dev, workspace_bytes, (hipStream_t)stream,
                                       h->g);
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
