// Round-based RePair on the host (the pass structure is described in
// rounds.hpp).  One tile per call, like repair_tile; it is the host form of
// the device builder in build_gpu.hip and follows the same steps in the same
// order, so both give the same rules, numbered alike, and the same final
// sequence.
#include <algorithm>
#include <cstring>

#include "grammar.hpp"
#include "rounds.hpp"

namespace gcs {
namespace {

using namespace rounds;

struct PairTable {
    std::vector<uint64_t> key;
    std::vector<uint32_t> cnt, wins, first, id;
    uint64_t mask = 0;

    void reset(int64_t pairs)
    {
        size_t cap = 16;
        while (cap < (size_t)(2 * pairs)) cap <<= 1;
        key.assign(cap, ~0ULL);
        cnt.assign(cap, 0);
        wins.assign(cap, 0);
        first.assign(cap, UINT32_MAX);
        id.resize(cap);
        mask = cap - 1;
    }
    uint32_t insert(uint64_t k)
    {
        uint64_t h = (uint64_t)pair_hash(k) & mask;
        while (key[h] != k) {
            if (key[h] == ~0ULL) {
                key[h] = k;
                break;
            }
            h = (h + 1) & mask;
        }
        return (uint32_t)h;
    }
};

}  // namespace

bool repair_rounds_tile(const std::vector<int32_t>& seq_in, const std::vector<int64_t>& row_off, int32_t nt_base,
                        RePairResult& out)
{
    try {
        const int64_t nrows = (int64_t)row_off.size() - 1;
        int64_t n = (int64_t)seq_in.size();
        out.rule_a.clear();
        out.rule_b.clear();
        out.row_len.assign((size_t)nrows, 0);
        if (n >= (int64_t)UINT32_MAX) return false;
        std::vector<uint32_t> S((size_t)n), S2;
        for (int64_t r = 0; r < nrows; ++r)
            for (int64_t k = row_off[r]; k < row_off[r + 1]; ++k)
                S[k] = (uint32_t)seq_in[k] | (k + 1 == row_off[r + 1] ? kEnd : 0u);
        std::vector<int64_t> slot((size_t)n);
        std::vector<uint32_t> cpos((size_t)n);
        std::vector<uint8_t> flag((size_t)n);
        PairTable T;
        int64_t next = nt_base;
        for (;;) {
            // 1. counts
            T.reset(n);
            uint32_t fmax = 0;
            for (int64_t i = 0; i < n; ++i) {
                if (S[i] & kEnd) {
                    slot[i] = -1;
                    continue;
                }
                const uint32_t h = T.insert(pair_key(S[i] & kSym, S[i + 1] & kSym));
                fmax = std::max(fmax, ++T.cnt[h]);
                slot[i] = h;
            }
            if (fmax < 2) break;
            // 2. candidates
            const uint32_t tau = threshold(fmax);
            for (int64_t i = 0; i < n; ++i) {
                const uint32_t c = slot[i] >= 0 ? T.cnt[slot[i]] : 0;
                cpos[i] = c >= tau ? c : 0;
            }
            // 3. winners
            for (int64_t i = 0; i < n; ++i) {
                flag[i] = 0;
                if (!cpos[i]) continue;
                const uint64_t k = pair_key(S[i] & kSym, S[i + 1] & kSym);
                const uint64_t r = rank(cpos[i], k);
                if (i > 0 && cpos[i - 1]) {
                    const uint64_t kl = pair_key(S[i - 1] & kSym, S[i] & kSym);
                    if (!outranks(r, k, rank(cpos[i - 1], kl), kl)) continue;
                }
                if (cpos[i + 1]) {  // S[i] is not a row end, so i + 1 < n
                    const uint64_t kr = pair_key(S[i + 1] & kSym, S[i + 2] & kSym);
                    if (!outranks(r, k, rank(cpos[i + 1], kr), kr)) continue;
                }
                flag[i] = 1;
                T.wins[slot[i]]++;
                T.first[slot[i]] = std::min(T.first[slot[i]], (uint32_t)i);
            }
            // 4. rules, numbered by first winning occurrence
            for (int64_t i = 0; i < n; ++i) {
                if (!flag[i] || T.wins[slot[i]] < 2) continue;
                flag[i] = 3;
                if (T.first[slot[i]] == (uint32_t)i) {
                    if (next >= (int64_t)kSym) return false;
                    T.id[slot[i]] = (uint32_t)next++;
                    out.rule_a.push_back((int32_t)(S[i] & kSym));
                    out.rule_b.push_back((int32_t)(S[i + 1] & kSym));
                }
            }
            // 5. rewrite: a replaced occurrence keeps its left position and
            // takes the row-end mark of the deleted right symbol
            S2.resize((size_t)n);
            int64_t o = 0;
            for (int64_t i = 0; i < n; ++i) {
                if (i > 0 && flag[i - 1] == 3) continue;
                S2[o++] = flag[i] == 3 ? (T.id[slot[i]] | (S[i + 1] & kEnd)) : S[i];
            }
            S2.resize((size_t)o);
            S.swap(S2);
            n = o;
        }
        out.seq.resize((size_t)n);
        int64_t i = 0;
        for (int64_t r = 0; r < nrows; ++r) {
            if (row_off[r + 1] == row_off[r]) continue;
            const int64_t b = i;
            while (!(S[i] & kEnd)) out.seq[i] = (int32_t)S[i], ++i;
            out.seq[i] = (int32_t)(S[i] & kSym);
            ++i;
            out.row_len[(size_t)r] = i - b;
        }
        return true;
    } catch (const std::bad_alloc&) {
        return false;
    }
}

}  // namespace gcs
