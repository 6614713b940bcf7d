// Round-based RePair: the definitions that the host builder (repair_rounds.cpp)
// and the device builder (build_gpu.hip) must share so that both produce the
// same grammar, bit for bit.
//
// RePair (page "Right Multiplication on Grammar-Compressed Matrices", section 2
// 'Grammar' and section 4.1) replaces a most frequent pair of adjacent symbols
// by a new nonterminal until no pair occurs twice, never pairing across two
// rows.  The round-based form replaces many pairs per pass over the sequence:
//
//   1. count every pair (a, b) of adjacent symbols of one row; f = the largest
//      count; stop when f < 2;
//   2. an occurrence is a candidate when its pair's count is at least
//      threshold(f) = max(2, ceil(f / kBand));
//   3. an occurrence wins when it outranks the candidate occurrences that
//      overlap it (the one starting one position earlier and the one starting
//      one position later): rank = (count, pair_hash, key), larger wins, so
//      the more frequent pair keeps a contested symbol;
//   4. a pair with at least two winning occurrences becomes a rule; rules of a
//      round are numbered in the order of their first winning occurrence;
//      every winning occurrence of such a pair is replaced (the left symbol
//      takes the rule, the right one is deleted).  Winners of pairs that won
//      only once stay as they are.
//
// A round never replaces two overlapping occurrences, each new rule is used at
// least twice, and the pair with the largest rank always wins everywhere, so
// every round makes at least one rule.  The stop rule is RePair's: the final
// sequence holds no pair twice.  With kBand = 1 a round takes only pairs of
// the largest count; a larger band trades closeness to the one-pair-at-a-time
// order for fewer passes.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define GCS_RHD __host__ __device__
#else
#define GCS_RHD
#endif

namespace gcs {
namespace rounds {

// bit 31 of a sequence word marks the last symbol of its row; symbols are < 2^31
constexpr uint32_t kEnd = 0x80000000u;
constexpr uint32_t kSym = 0x7FFFFFFFu;
// a round takes the pairs whose count is at least 1/kBand of the largest
constexpr uint32_t kBand = 10;

GCS_RHD inline uint64_t pair_key(uint32_t a, uint32_t b) { return ((uint64_t)a << 32) | (uint64_t)b; }

// 64-bit finalizer of MurmurHash3 (fmix64, public domain), upper half
GCS_RHD inline uint32_t pair_hash(uint64_t k)
{
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdULL;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ULL;
    k ^= k >> 33;
    return (uint32_t)(k >> 32);
}

GCS_RHD inline uint32_t threshold(uint32_t fmax)
{
    uint32_t t = (fmax + kBand - 1) / kBand;
    return t < 2 ? 2 : t;
}

// rank of a candidate occurrence; 0 = not a candidate
GCS_RHD inline uint64_t rank(uint32_t count, uint64_t key)
{
    return ((uint64_t)count << 32) | (uint64_t)pair_hash(key);
}

// strict order between two overlapping occurrences (their keys differ: a row
// never holds a symbol twice, so (a, b) and (b, c) are different pairs)
GCS_RHD inline bool outranks(uint64_t ra, uint64_t ka, uint64_t rb, uint64_t kb)
{
    return ra != rb ? ra > rb : ka > kb;
}

}  // namespace rounds
}  // namespace gcs
