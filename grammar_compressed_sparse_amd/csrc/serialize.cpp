// Serialized layered grammar: compress once, reuse across runs.  The pages
// report a serialized grammar's on-disk size beside the device footprint
// (section 5, Table 5.1) and treat construction as a one-time offline cost
// amortised over many products (section 7, item 2); this is that file here,
// our own format.  One little-endian binary file:
//
//   "GCSGRAM1", u32 version, u32 byte-order mark 0x01020304, u32 kSlices,
//   u32 reserved, then the scalars (n_rows, n_cols, nnz, n_tiles, L,
//   col_cut[kSlices + 1], wmax, pt_total, buf_a, buf_b, arena, build times),
//   then every array as (u64 element count, raw elements) in a fixed order,
//   then a u64 checksum of everything before it.
//
// Loading checks the header, every count against the others, and the
// checksum; the device upload checks every index against its buffer again.
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "grammar.hpp"

namespace gcs {
namespace {

constexpr char kMagic[8] = {'G', 'C', 'S', 'G', 'R', 'A', 'M', '1'};
constexpr uint32_t kVersion = 1, kByteOrder = 0x01020304u;
constexpr int kLevelWords = 8 + 3 * (kSlices + 1);  // int64 fields of Level

// 64-bit running checksum over 8-byte words (multiply-xorshift mixing of each
// word into the state; a trailing partial word is zero-padded)
struct Checksum {
    uint64_t h = 0x9E3779B97F4A7C15ull;
    uint64_t carry = 0;
    int nc = 0;
    void word(uint64_t w)
    {
        h ^= w + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
        h *= 0xBF58476D1CE4E5B9ull;
        h ^= h >> 31;
    }
    void bytes(const void* p, size_t n)
    {
        const unsigned char* b = (const unsigned char*)p;
        while (n && nc) {  // finish a pending partial word
            carry |= (uint64_t)*b++ << (8 * nc);
            --n;
            if (++nc == 8) {
                word(carry);
                carry = 0;
                nc = 0;
            }
        }
        for (; n >= 8; n -= 8, b += 8) {
            uint64_t w;
            std::memcpy(&w, b, 8);
            word(w);
        }
        while (n--) carry |= (uint64_t)*b++ << (8 * nc++);
    }
    uint64_t value() const
    {
        Checksum c = *this;
        if (c.nc) c.word(c.carry);
        return c.h;
    }
};

struct FileCloser {
    void operator()(FILE* f) const
    {
        if (f) std::fclose(f);
    }
};

class Writer {
public:
    explicit Writer(FILE* f) : f_(f) {}
    bool raw(const void* p, size_t n)
    {
        sum_.bytes(p, n);
        return n == 0 || std::fwrite(p, 1, n, f_) == n;
    }
    template <class T>
    bool pod(const T& v) { return raw(&v, sizeof(T)); }
    template <class T>
    bool array(const std::vector<T>& v)
    {
        const uint64_t n = v.size();
        return pod(n) && raw(v.data(), n * sizeof(T));
    }
    bool finish()
    {
        const uint64_t c = sum_.value();
        return std::fwrite(&c, 1, 8, f_) == 8;
    }

private:
    FILE* f_;
    Checksum sum_;
};

class Reader {
public:
    explicit Reader(FILE* f) : f_(f) {}
    bool raw(void* p, size_t n)
    {
        if (n && std::fread(p, 1, n, f_) != n) return false;
        sum_.bytes(p, n);
        return true;
    }
    template <class T>
    bool pod(T& v) { return raw(&v, sizeof(T)); }
    // an array of at most `max` elements (a bound from sizes read before it)
    template <class T>
    bool array(std::vector<T>& v, uint64_t max)
    {
        uint64_t n = 0;
        if (!pod(n) || n > max) return false;
        v.resize(n);
        return raw(v.data(), n * sizeof(T));
    }
    bool finish()
    {
        const uint64_t expect = sum_.value();
        uint64_t c = 0;
        if (std::fread(&c, 1, 8, f_) != 8 || c != expect) return false;
        char extra;
        return std::fread(&extra, 1, 1, f_) == 0;  // nothing after the checksum
    }

private:
    FILE* f_;
    Checksum sum_;
};

}  // namespace
}  // namespace gcs

using gcs::Grammar;

static gcs_status save_grammar(const gcs_grammar* h, const char* path)
{
    if (!h || !path) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    const Grammar& g = h->g;
    std::unique_ptr<FILE, gcs::FileCloser> f(std::fopen(path, "wb"));
    if (!f) {
        gcs::set_error(std::string("cannot open for writing: ") + path);
        return GCS_EINVAL;
    }
    gcs::Writer w(f.get());
    const uint32_t head[4] = {gcs::kVersion, gcs::kByteOrder, (uint32_t)gcs::kSlices, 0};
    bool ok = w.raw(gcs::kMagic, 8) && w.raw(head, sizeof(head));
    const int64_t sc[] = {g.n_rows, g.n_cols, g.nnz, g.n_tiles, g.L, g.wmax, g.pt_total, g.buf_a, g.buf_b, g.arena};
    ok = ok && w.raw(sc, sizeof(sc)) && w.raw(g.col_cut, sizeof(g.col_cut));
    const double times[3] = {g.t_csrv, g.t_repair, g.t_layer};
    ok = ok && w.raw(times, sizeof(times));
    std::vector<int64_t> lvw;
    lvw.reserve(g.lv.size() * gcs::kLevelWords);
    for (const gcs::Level& l : g.lv) {
        const int64_t head8[8] = {l.nb, l.npt, l.child_off, l.pt_off, l.reserved, l.base, l.grp_off, l.ngrp};
        lvw.insert(lvw.end(), head8, head8 + 8);
        lvw.insert(lvw.end(), l.bsl, l.bsl + gcs::kSlices + 1);
        lvw.insert(lvw.end(), l.psl, l.psl + gcs::kSlices + 1);
        lvw.insert(lvw.end(), l.gsl, l.gsl + gcs::kSlices + 1);
    }
    ok = ok && w.array(g.V) && w.array(g.tcol) && w.array(g.tval) && w.array(g.ra) && w.array(g.rb) &&
         w.array(g.c_off) && w.array(g.c_sym) && w.array(g.lvl) && w.array(g.plast) && w.array(lvw) &&
         w.array(g.child) && w.array(g.ptsrc) && w.array(g.erow) && w.array(g.eoff) && w.array(g.epos) &&
         w.finish();
    if (!ok || std::fflush(f.get()) != 0) {
        gcs::set_error(std::string("write failed: ") + path);
        return GCS_EINVAL;
    }
    return GCS_OK;
}

static gcs_status load_grammar(const char* path, gcs_grammar** out)
{
    if (!path || !out) {
        gcs::set_error("invalid argument");
        return GCS_EINVAL;
    }
    *out = nullptr;
    std::unique_ptr<FILE, gcs::FileCloser> f(std::fopen(path, "rb"));
    if (!f) {
        gcs::set_error(std::string("cannot open: ") + path);
        return GCS_EINVAL;
    }
    auto fail = [&](const char* why) {
        gcs::set_error(std::string(why) + ": " + path);
        return GCS_EINVAL;
    };
    gcs::Reader r(f.get());
    char magic[8];
    uint32_t head[4];
    if (!r.raw(magic, 8) || std::memcmp(magic, gcs::kMagic, 8) != 0) return fail("not a serialized grammar");
    if (!r.raw(head, sizeof(head)) || head[0] != gcs::kVersion || head[1] != gcs::kByteOrder ||
        head[2] != (uint32_t)gcs::kSlices)
        return fail("unsupported grammar file version, byte order or slice count");
    std::unique_ptr<gcs_grammar> h(new (std::nothrow) gcs_grammar());
    if (!h) {
        gcs::set_error("out of memory");
        return GCS_ENOMEM;
    }
    Grammar& g = h->g;
    int64_t sc[10];
    double times[3];
    if (!r.raw(sc, sizeof(sc)) || !r.raw(g.col_cut, sizeof(g.col_cut)) || !r.raw(times, sizeof(times)))
        return fail("truncated grammar file");
    g.n_rows = sc[0];
    g.n_cols = sc[1];
    g.nnz = sc[2];
    g.n_tiles = sc[3];
    const int64_t L = sc[4];
    g.wmax = sc[5];
    g.pt_total = sc[6];
    g.buf_a = sc[7];
    g.buf_b = sc[8];
    g.arena = sc[9];
    g.t_csrv = times[0];
    g.t_repair = times[1];
    g.t_layer = times[2];
    if (g.n_rows < 0 || g.n_cols < 0 || g.nnz < 0 || L < 0 || L >= INT32_MAX || g.arena < 0 ||
        g.n_cols > INT32_MAX)
        return fail("corrupt grammar file (sizes)");
    g.L = (int32_t)L;
    // every count is bounded by sizes read before it (an implausibly large
    // count fails here instead of allocating)
    const uint64_t big = (uint64_t)1 << 40;
    std::vector<int64_t> lvw;
    bool ok = r.array(g.V, (uint64_t)g.nnz + 1) && r.array(g.tcol, (uint64_t)g.arena) && r.array(g.tval, g.tcol.size()) &&
              r.array(g.ra, big) && r.array(g.rb, g.ra.size()) && r.array(g.c_off, (uint64_t)g.n_rows + 1) &&
              r.array(g.c_sym, big) && r.array(g.lvl, g.ra.size()) && r.array(g.plast, g.ra.size()) &&
              r.array(lvw, (uint64_t)(L + 1) * gcs::kLevelWords) && r.array(g.child, 2 * g.ra.size()) &&
              r.array(g.ptsrc, big) && r.array(g.erow, big) && r.array(g.eoff, g.erow.size() + 1) &&
              r.array(g.epos, g.c_sym.size());
    if (!ok) return fail("truncated or corrupt grammar file");
    if (!r.finish()) return fail("grammar file checksum mismatch");
    // consistency of the counts (the upload checks every index)
    if (g.tval.size() != g.tcol.size() || g.rb.size() != g.ra.size() || g.c_off.size() != (size_t)g.n_rows + 1 ||
        g.lvl.size() != g.ra.size() || g.plast.size() != g.ra.size() ||
        lvw.size() != (size_t)(L + 1) * gcs::kLevelWords || g.child.size() != 2 * g.ra.size() ||
        g.eoff.size() != g.erow.size() + 1 || g.epos.size() != g.c_sym.size() ||
        (g.n_rows > 0 && (g.c_off[0] != 0 || g.c_off[g.n_rows] != (int64_t)g.c_sym.size())) ||
        (!g.eoff.empty() && (g.eoff.front() != 0 || g.eoff.back() != (int32_t)g.epos.size())))
        return fail("inconsistent grammar file");
    g.lv.resize((size_t)L + 1);
    for (int64_t k = 0; k <= L; ++k) {
        const int64_t* p = lvw.data() + k * gcs::kLevelWords;
        gcs::Level& l = g.lv[k];
        l.nb = p[0];
        l.npt = p[1];
        l.child_off = p[2];
        l.pt_off = p[3];
        l.reserved = p[4];
        l.base = p[5];
        l.grp_off = p[6];
        l.ngrp = p[7];
        std::memcpy(l.bsl, p + 8, sizeof(l.bsl));
        std::memcpy(l.psl, p + 8 + gcs::kSlices + 1, sizeof(l.psl));
        std::memcpy(l.gsl, p + 8 + 2 * (gcs::kSlices + 1), sizeof(l.gsl));
    }
    *out = h.release();
    return GCS_OK;
}

// no exception crosses the C ABI: allocation failures become GCS_ENOMEM
extern "C" gcs_status gcs_save_grammar(const gcs_grammar* h, const char* path)
{
    try {
        return save_grammar(h, path);
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of memory");
        return GCS_ENOMEM;
    }
}

extern "C" gcs_status gcs_load_grammar(const char* path, gcs_grammar** out)
{
    try {
        return load_grammar(path, out);
    } catch (const std::bad_alloc&) {
        gcs::set_error("out of memory");
        return GCS_ENOMEM;
    }
}
