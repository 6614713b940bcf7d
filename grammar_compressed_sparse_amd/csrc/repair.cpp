// RePair (Larsson & Moffat, "Off-line dictionary-based compression", Proc. IEEE
// 2000), restricted to pairs inside one row as the mm-repair scheme requires
// (page "Right Multiplication on Grammar-Compressed Matrices", section 2
// 'Grammar' and section 4.1): repeatedly replace the most frequent pair of
// adjacent symbols by a new nonterminal until no pair occurs twice.
//
// Data structures, all O(n) words:
//   - the sequence as doubly linked live positions per row (nxt/prv), so a
//     replacement deletes the right symbol in O(1);
//   - for every tracked pair a record {frequency, occurrence list} reached by
//     a chained hash on the pair key; occurrence lists are doubly linked
//     through the left position of each occurrence (onx/opv);
//   - an exact bucket queue indexed by frequency.  Within a row every column
//     occurs at most once, so a pair occurs at most once per row and its
//     frequency never exceeds the number of rows.
//
// Facts that keep the bookkeeping small (all follow from distinct columns
// within a row): no pair (a, a) exists, so occurrences never overlap; a pair
// is created only in the step that creates the newer of its two symbols, so
// a pair whose count drops below 2 is dropped for good, and the pairs created
// in one step are counted in two small per-step maps keyed by the neighbour
// symbol.  Ties among equally frequent pairs are broken by the bucket order
// (most recently queued first), which is deterministic.
#include <algorithm>
#include <cstring>

#include "grammar.hpp"

namespace gcs {
namespace {

struct Rec {
    uint64_t key;
    int32_t freq;
    int32_t head;  // first occurrence (left position)
    int32_t qprev, qnext;
    int32_t hnext;
    int32_t in_hash;
};

inline uint64_t pair_key(int32_t a, int32_t b) { return ((uint64_t)(uint32_t)a << 32) | (uint32_t)b; }

// 64-bit finalizer of MurmurHash3 (fmix64, public domain)
inline uint64_t hmix(uint64_t k)
{
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdULL;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ULL;
    k ^= k >> 33;
    return k;
}

// Open-addressing map int32 -> record index, cleared in O(1) by a stamp.
struct StepMap {
    std::vector<int32_t> key, val;
    std::vector<uint32_t> stamp;
    std::vector<int32_t> used;
    uint32_t cur = 0;
    uint64_t mask = 0;

    void reset(size_t expect)
    {
        size_t cap = 16;
        while (cap < 2 * expect) cap <<= 1;
        if (cap > key.size()) {
            key.assign(cap, 0);
            val.assign(cap, 0);
            stamp.assign(cap, 0);
            cur = 0;
        }
        mask = key.size() - 1;
        if (++cur == 0) {
            std::fill(stamp.begin(), stamp.end(), 0);
            cur = 1;
        }
        used.clear();
    }
    // returns a reference to the value slot; *fresh set if the key was absent
    int32_t& get(int32_t k, bool* fresh)
    {
        uint64_t h = hmix((uint64_t)(uint32_t)k) & mask;
        while (stamp[h] == cur && key[h] != k) h = (h + 1) & mask;
        *fresh = stamp[h] != cur;
        if (*fresh) {
            stamp[h] = cur;
            key[h] = k;
            used.push_back((int32_t)h);
        }
        return val[h];
    }
};

class Engine {
  public:
    std::vector<int32_t> sym, nxt, prv, onx, opv;
    std::vector<Rec> rec;
    std::vector<int32_t> free_rec;
    std::vector<int32_t> htab;
    uint64_t hmask = 0;
    int64_t live = 0;
    std::vector<int32_t> bucket;
    StepMap left_new, right_new;

    int32_t new_rec(uint64_t key)
    {
        int32_t r;
        if (!free_rec.empty()) {
            r = free_rec.back();
            free_rec.pop_back();
        } else {
            r = (int32_t)rec.size();
            rec.push_back(Rec{});
        }
        Rec& x = rec[r];
        x.key = key;
        x.freq = 0;
        x.head = -1;
        x.qprev = x.qnext = -1;
        x.hnext = -1;
        x.in_hash = 0;
        return r;
    }

    void grow_hash()
    {
        size_t cap = htab.size() * 2;
        htab.assign(cap, -1);
        hmask = cap - 1;
        for (int32_t r = 0; r < (int32_t)rec.size(); ++r) {
            if (!rec[r].in_hash) continue;
            uint64_t h = hmix(rec[r].key) & hmask;
            rec[r].hnext = htab[h];
            htab[h] = r;
        }
    }

    void hash_insert(int32_t r)
    {
        if ((uint64_t)live + 1 > htab.size()) grow_hash();
        uint64_t h = hmix(rec[r].key) & hmask;
        rec[r].hnext = htab[h];
        htab[h] = r;
        rec[r].in_hash = 1;
        ++live;
    }

    int32_t find(uint64_t key) const
    {
        for (int32_t r = htab[hmix(key) & hmask]; r != -1; r = rec[r].hnext)
            if (rec[r].key == key) return r;
        return -1;
    }

    void hash_erase(int32_t r)
    {
        uint64_t h = hmix(rec[r].key) & hmask;
        int32_t* p = &htab[h];
        while (*p != r) p = &rec[*p].hnext;
        *p = rec[r].hnext;
        rec[r].in_hash = 0;
        --live;
    }

    void release(int32_t r) { free_rec.push_back(r); }

    void pq_push(int32_t r)
    {
        int32_t f = rec[r].freq;
        rec[r].qprev = -1;
        rec[r].qnext = bucket[f];
        if (bucket[f] != -1) rec[bucket[f]].qprev = r;
        bucket[f] = r;
    }

    void pq_remove(int32_t r)
    {
        Rec& x = rec[r];
        if (x.qprev != -1) rec[x.qprev].qnext = x.qnext;
        else bucket[x.freq] = x.qnext;
        if (x.qnext != -1) rec[x.qnext].qprev = x.qprev;
    }

    void occ_link(int32_t r, int32_t pos)
    {
        int32_t h = rec[r].head;
        onx[pos] = h;
        opv[pos] = -1;
        if (h != -1) opv[h] = pos;
        rec[r].head = pos;
    }

    void occ_unlink(int32_t r, int32_t pos)
    {
        if (opv[pos] != -1) onx[opv[pos]] = onx[pos];
        else rec[r].head = onx[pos];
        if (onx[pos] != -1) opv[onx[pos]] = opv[pos];
    }

    // The pair starting at live position pos disappears.
    void decrement(int32_t pos)
    {
        int32_t r = find(pair_key(sym[pos], sym[nxt[pos]]));
        if (r == -1) return;  // untracked (its count fell below 2 earlier)
        occ_unlink(r, pos);
        pq_remove(r);
        if (--rec[r].freq >= 2) {
            pq_push(r);
        } else {
            hash_erase(r);
            release(r);
        }
    }
};

}  // namespace

bool repair_tile(const std::vector<int32_t>& seq_in, const std::vector<int64_t>& row_off, int32_t nt_base,
                 RePairResult& out)
{
    try {
        const int64_t n = (int64_t)seq_in.size();
        const int64_t nrows = (int64_t)row_off.size() - 1;
        out.rule_a.clear();
        out.rule_b.clear();
        out.row_len.assign((size_t)nrows, 0);
        Engine E;
        E.sym = seq_in;
        E.nxt.resize((size_t)n);
        E.prv.resize((size_t)n);
        E.onx.resize((size_t)n);
        E.opv.resize((size_t)n);
        size_t cap = 1024;
        while (cap < (size_t)(n / 2 + 1)) cap <<= 1;
        E.htab.assign(cap, -1);
        E.hmask = cap - 1;
        E.rec.reserve((size_t)std::min<int64_t>(n / 2 + 16, 1 << 26));

        // initial pairs
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t b = row_off[r], e = row_off[r + 1];
            for (int64_t i = b; i < e; ++i) {
                E.prv[i] = i > b ? (int32_t)(i - 1) : -1;
                E.nxt[i] = i + 1 < e ? (int32_t)(i + 1) : -1;
            }
            for (int64_t i = b; i + 1 < e; ++i) {
                uint64_t k = pair_key(E.sym[i], E.sym[i + 1]);
                int32_t x = E.find(k);
                if (x == -1) {
                    x = E.new_rec(k);
                    E.hash_insert(x);
                }
                E.rec[x].freq++;
                E.occ_link(x, (int32_t)i);
            }
        }
        int32_t maxf = 1;
        for (const Rec& x : E.rec) maxf = std::max(maxf, x.freq);
        E.bucket.assign((size_t)maxf + 1, -1);
        for (int32_t x = 0; x < (int32_t)E.rec.size(); ++x) {
            if (E.rec[x].freq >= 2) {
                E.pq_push(x);
            } else {
                E.hash_erase(x);
                E.release(x);
            }
        }

        std::vector<int32_t> fresh_recs;
        int32_t next_sym = nt_base;
        for (int32_t f = maxf; f >= 2;) {
            int32_t r = E.bucket[f];
            if (r == -1) {
                --f;
                continue;
            }
            const int32_t A = (int32_t)(E.rec[r].key >> 32), B = (int32_t)(uint32_t)E.rec[r].key;
            const int32_t N = next_sym++;
            out.rule_a.push_back(A);
            out.rule_b.push_back(B);
            E.pq_remove(r);
            E.hash_erase(r);
            E.left_new.reset((size_t)f);
            E.right_new.reset((size_t)f);
            fresh_recs.clear();
            for (int32_t i = E.rec[r].head; i != -1;) {
                const int32_t next_occ = E.onx[i];
                const int32_t j = E.nxt[i], p = E.prv[i], q = E.nxt[j];
                if (p != -1) E.decrement(p);
                if (q != -1) E.decrement(j);
                E.sym[i] = N;
                E.nxt[i] = q;
                if (q != -1) E.prv[q] = i;
                bool fresh;
                if (p != -1) {
                    int32_t& slot = E.left_new.get(E.sym[p], &fresh);
                    if (fresh) {
                        slot = E.new_rec(pair_key(E.sym[p], N));
                        fresh_recs.push_back(slot);
                    }
                    E.rec[slot].freq++;
                    E.occ_link(slot, p);
                }
                if (q != -1) {
                    int32_t& slot = E.right_new.get(E.sym[q], &fresh);
                    if (fresh) {
                        slot = E.new_rec(pair_key(N, E.sym[q]));
                        fresh_recs.push_back(slot);
                    }
                    E.rec[slot].freq++;
                    E.occ_link(slot, i);
                }
                i = next_occ;
            }
            E.release(r);
            for (int32_t x : fresh_recs) {
                if (E.rec[x].freq >= 2) {
                    E.hash_insert(x);
                    E.pq_push(x);
                } else {
                    E.release(x);
                }
            }
            if (next_sym == INT32_MAX) return false;
        }

        // final sequences
        out.seq.clear();
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t b = row_off[r], e = row_off[r + 1];
            if (b == e) continue;
            int64_t c = 0;
            for (int32_t i = (int32_t)b; i != -1; i = E.nxt[i]) {
                out.seq.push_back(E.sym[i]);
                ++c;
            }
            out.row_len[(size_t)r] = c;
        }
        return true;
    } catch (const std::bad_alloc&) {
        return false;
    }
}

}  // namespace gcs
