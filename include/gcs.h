/*
 * gcs.h -- C ABI of the grammar-compressed right product y = M x on MI355X.
 *
 * Method: "Right Multiplication on Grammar-Compressed Matrices: A Streaming,
 * Memory-Bounded GPU Engine" (arXiv 2607.24971v1).  The matrix is encoded
 * as a CSRV string (section 2, Eq. 2.2), compressed by RePair into
 * (C, R, V) (section 2, Eq. 2.3-2.4; section 4.1), completed with
 * pass-through nodes into a properly layered grammar (Definition 3.2,
 * section 4.2) and evaluated by a bottom-up, level-synchronous sweep over two
 * alternating value buffers (Lemma 3.3, section 4.3, Listing 1), with the
 * leaf / combine / emit operations chosen by a policy (section 5).
 *
 * Conventions
 *   - Every call returns a gcs_status (0 = GCS_OK, < 0 = error) unless it is
 *     declared void; nothing throws across the ABI.  gcs_last_error() returns
 *     a thread-local message describing the most recent failure.
 *   - Host arrays passed in are borrowed for the duration of the call only.
 *   - Host grammars (gcs_grammar) are owned by the library until
 *     gcs_free_grammar.
 *   - ALL DEVICE MEMORY IS OWNED BY THE CALLER.  gcs_device_layout reports
 *     the byte sizes; the caller allocates (e.g. torch.empty(..., 'cuda')),
 *     passes the pointers to gcs_upload and keeps them alive until
 *     gcs_free_device.  The library never allocates device memory.  It does
 *     allocate one small pinned host word per device handle (BFS counter).
 *   - Streams are hipStream_t passed as void*; NULL is the null stream.  All
 *     device work is enqueued asynchronously on the given stream; kernel
 *     faults surface at the caller's next synchronisation.
 */
#ifndef GCS_H
#define GCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GCS_OK = 0,
    GCS_EINVAL = -1, /* malformed argument or input matrix                      */
    GCS_ENOMEM = -2, /* host allocation failed                                   */
    GCS_EHIP = -3,   /* a HIP runtime call failed (message holds the HIP error)  */
    GCS_ERANGE = -4, /* a size exceeds the 32-bit index space of the layout      */
    GCS_ESTATE = -5  /* call not valid in the object's state (e.g. wrong policy) */
} gcs_status;

/* Leaf / combine / emit policy (section 5: any monoid homomorphism by swapping
 * a small leaf/combine/emit policy).  Element types of x and y:
 *   GCS_PLUS_F64          x double,  y double;  T and buffers double
 *   GCS_PLUS_F32          x float,   y float;   T and buffers float
 *   GCS_PLUS_F32_ACC_F64  x float,   y double;  T and buffers double
 *   GCS_BOOL_OR           x uint8 0/1, y uint8 0/1; leaf = x[j], combine = OR
 *   GCS_PLUS_I64          x int64,   y int64; matrix values must be integers
 *   GCS_MIN_PLUS_F32      x float,   y float;  tropical: leaf = M[r][j] + x[j],
 *                         combine = min, +infinity for a row with no entry
 *                         (one Bellman-Ford relaxation per pass)
 *   GCS_MIN_PLUS_F64      as GCS_MIN_PLUS_F32 in double  */
typedef enum {
    GCS_PLUS_F64 = 0,
    GCS_PLUS_F32 = 1,
    GCS_PLUS_F32_ACC_F64 = 2,
    GCS_BOOL_OR = 3,
    GCS_PLUS_I64 = 4,
    GCS_MIN_PLUS_F32 = 5,
    GCS_MIN_PLUS_F64 = 6
} gcs_policy;

/* Value array of a CSR input. */
typedef enum {
    GCS_VAL_ONES = 0, /* every stored entry is 1 (val ignored, may be NULL) */
    GCS_VAL_I8 = 1,   /* int8_t val[nnz]                                    */
    GCS_VAL_F64 = 2   /* double val[nnz]                                    */
} gcs_val_kind;

/* A sparse matrix in CSR form (host memory, borrowed).  Columns of each row
 * must be strictly increasing and < n_cols; row_ptr[0] == 0 and row_ptr is
 * non-decreasing.  Stored zeros are dropped; non-finite values are rejected. */
typedef struct {
    int64_t n_rows;
    int64_t n_cols;
    const int64_t* row_ptr; /* n_rows + 1 */
    const int32_t* col;     /* row_ptr[n_rows] */
    int32_t val_kind;       /* gcs_val_kind */
    int32_t reserved;
    const void* val;
} gcs_csr_view;

/* Row order for row tiles. */
typedef enum {
    GCS_ROWS_NATURAL = 0, /* row tiles are consecutive rows                                    */
    GCS_ROWS_SIMILAR = 1  /* rows ordered by two MinHash values of their column sets first,    */
                          /* so rows that share many columns tend to share a tile              */
} gcs_row_order;

/* Builder options.  RePair runs independently on each tile of a
 * (row chunk x column chunk) partition; tiles run in parallel.  Column chunks
 * lose no rule sharing (terminals carry their column, so rules never span
 * two column ranges); they only cut pairs that straddle a chunk border.  Row
 * chunks lose the sharing between rows of different tiles; the pages' prior
 * work partitions by row blocks (section 1).  y is always in the input's row
 * order. */
/* RePair variant.  Both replace frequent pairs of adjacent symbols of one row
 * by new nonterminals until no pair occurs twice (section 2 'Grammar',
 * section 4.1); several grammars are correct, and the sweep accepts any.
 *   GCS_REPAIR_EXACT   one most frequent pair at a time (Larsson and Moffat's
 *                      linked-list form; ties: the most recently queued pair)
 *   GCS_REPAIR_ROUNDS  round-based: each pass over the sequence replaces every
 *                      non-overlapping occurrence of the pairs whose count is
 *                      at least a tenth of the largest (the more frequent pair
 *                      keeps a contested symbol), and makes a rule of each
 *                      pair replaced at least twice.  Shallower grammars with
 *                      far fewer pass-through nodes; the form the device
 *                      builder (gcs_build_grammar_gpu) runs, with identical
 *                      output. */
typedef enum { GCS_REPAIR_EXACT = 0, GCS_REPAIR_ROUNDS = 1 } gcs_repair_mode;

typedef struct {
    int32_t n_threads; /* 0 = OMP_NUM_THREADS if set, else the CPUs of the affinity mask */
    int32_t col_chunk; /* columns per tile; 0 = all columns                               */
    int32_t row_chunk; /* rows per tile; 0 = all rows                                     */
    int32_t row_order; /* gcs_row_order: which rows share a row tile                      */
    int32_t repair;    /* gcs_repair_mode                                                 */
    int32_t reserved;  /* must be 0                                                       */
} gcs_build_opts;

/* Structural figures of a built grammar (section 4.4, Table 4.1 columns). */
typedef struct {
    int64_t n_rows, n_cols, nnz;
    int64_t n_values;      /* |V|: distinct nonzero values                      */
    int64_t n_terminals;   /* alpha: distinct <l, j> terminals in use           */
    int64_t n_rules;       /* |R|                                                */
    int64_t n_passthrough; /* +pt: pass-through nodes added by completion       */
    int64_t depth;         /* L                                                  */
    int64_t max_width;     /* w*: widest completed level (= streaming buffer)   */
    int64_t c_len;         /* |C|: symbols of the final sequence                */
    int64_t n_tiles;       /* RePair tiles                                       */
    int64_t n_emit_groups; /* (level, slice, row) emission groups               */
    double t_csrv_ms;      /* CSRV encoding                                      */
    double t_repair_ms;    /* RePair (all tiles, wall time)                      */
    double t_layer_ms;     /* levels + completion + bucketing + layout ("+pt")  */
} gcs_stats;

typedef struct gcs_grammar gcs_grammar;
typedef struct gcs_device gcs_device;

/* ---- host builder ---------------------------------------------------- */

/* CSRV encoding (section 2, 'CSRV', Eq. 2.2), RePair never pairing across
 * rows (section 2 'Grammar', section 4.1), levels (Eq. 3.1), pass-through
 * completion (section 4.2) and the level-bucketed layout (section 4.3).
 * opts may be NULL (defaults).  *out receives a new grammar on GCS_OK. */
gcs_status gcs_build_grammar(const gcs_csr_view* m, const gcs_build_opts* opts, gcs_grammar** out);

/* A row source: the matrix handed over block by block, so that a matrix too
 * large for host memory never has to exist whole (section 2, 'CSRV': S is
 * built row by row).  Called with row_ptr == NULL it returns the number of
 * stored entries of rows [row0, row0 + nrows) in columns [col0, col0 + ncols);
 * called with arrays (row_ptr: nrows + 1 entries, col and val: cap entries;
 * val is NULL for GCS_VAL_ONES) it fills that block as CSR -- row_ptr
 * relative to the block (row_ptr[0] = 0), absolute column indices, strictly
 * increasing per row -- and returns the count again.  A negative return
 * aborts the build (GCS_EINVAL).  Called from the building thread only. */
typedef int64_t (*gcs_row_source)(void* ctx, int64_t row0, int64_t nrows, int64_t col0, int64_t ncols,
                                  int64_t* row_ptr, int32_t* col, double* val, int64_t cap);

/* gcs_build_grammar on a matrix pulled from a row source, one tile (row
 * chunk x column chunk of opts; whole matrix by default) at a time: one
 * pass over the tiles for V and the terminal alphabet, a second that
 * encodes and runs RePair on n_threads tiles at a time, so host memory holds
 * about n_threads tiles plus the grammar.  val_kind: GCS_VAL_ONES or
 * GCS_VAL_F64 (int8 values are handed over as doubles).  The grammar equals
 * gcs_build_grammar's on the assembled CSR with the same options; the row
 * order must be GCS_ROWS_NATURAL.  Errors as gcs_build_grammar, plus
 * GCS_EINVAL for a source that fails, changes its count between the two
 * calls, or returns columns outside the requested block. */
gcs_status gcs_build_grammar_rows(gcs_row_source src, void* ctx, int64_t n_rows, int64_t n_cols, int32_t val_kind,
                                  const gcs_build_opts* opts, gcs_grammar** out);

/* Row r as the grammar encodes it: C[r] expanded through R (Lemma 2.2: the
 * roots of row r expand to its CSRV row), i.e. the terminals of row r's
 * nonzeros in column order (term_col / term_val of gcs_export_grammar give
 * their column and value index).  Writes min(cap, *len) terminal ids to sym
 * and the full length to *len.  GCS_ERANGE if cap < *len, GCS_EINVAL for r
 * outside [0, n_rows).  A test and inspection hook. */
gcs_status gcs_expand_row(const gcs_grammar* g, int64_t r, int32_t* sym, int64_t cap, int64_t* len);

/* A grammar given explicitly (e.g. Eq. 2.3-2.4 of the pages' worked
 * example), then levelled, completed and laid out as above.
 *   values[n_values]        V, distinct nonzero values
 *   term_col/term_val[n_terms]  terminal t = <term_val[t]+1, term_col[t]+1>
 *                           (0-based value index and column), distinct pairs
 *   rule_a/rule_b[n_rules]  rule i: N_i -> rule_a[i] rule_b[i]; a symbol s <
 *                           n_terms is terminal s, s >= n_terms is rule
 *                           s - n_terms, which must be < i (topological order)
 *   c_off[n_rows+1], c_sym[c_off[n_rows]]  row r's sequence in C.
 * Rejected (GCS_EINVAL) if any index is out of range or the order is not
 * topological. */
gcs_status gcs_grammar_from_rules(int64_t n_rows, int64_t n_cols, const double* values, int64_t n_values,
                                  const int32_t* term_col, const int32_t* term_val, int64_t n_terms,
                                  const int32_t* rule_a, const int32_t* rule_b, int64_t n_rules,
                                  const int64_t* c_off, const int32_t* c_sym, gcs_grammar** out);

/* One grammar from grammars of disjoint column groups of the same matrix
 * (section 4.4 builds one grammar per column chunk; a matrix too large to
 * build whole is built chunk by chunk and merged).  parts[0..n_parts) must
 * have equal n_rows and n_cols and cover increasing, disjoint column ranges
 * (part p's terminal columns all below part p+1's).  The merged grammar has
 * the union of the values, the parts' terminals and rules in part order
 * (symbols renumbered), each row's sequence the concatenation of the parts'
 * sequences of that row, and is levelled, completed and laid out afresh
 * with n_threads host threads (0: as gcs_build_grammar).  Its products
 * equal the sum (or OR, or min) of the parts' products.  The parts are not
 * modified; the caller frees them and *out (gcs_free_grammar).
 * GCS_EINVAL on a shape mismatch or overlapping/unordered columns,
 * GCS_ERANGE beyond the 32-bit symbol space, GCS_ENOMEM. */
gcs_status gcs_merge_grammars(const gcs_grammar* const* parts, int32_t n_parts, int32_t n_threads,
                              gcs_grammar** out);

gcs_status gcs_grammar_stats(const gcs_grammar* g, gcs_stats* out);

/* Completed widths w_k, k = 0..L (w_0 = alpha, the terminal array).  Writes
 * min(cap, L+1) entries. */
gcs_status gcs_level_widths(const gcs_grammar* g, int64_t* w, int64_t cap);

/* Distribution of edge spans (section 4.1: RePair's level-skipping edges,
 * reported beside the depth L; section 4.2: completion's cost follows it):
 * hist[d] = number of edges rule -> child with lvl(rule) - lvl(child) = d,
 * both children of every rule, a terminal child at level 0; d = 1..L
 * (hist[0] = 0).  Writes cap entries (zeros past L); *max_span (may be
 * NULL) gets the largest span present. */
gcs_status gcs_edge_spans(const gcs_grammar* g, int64_t* hist, int64_t cap, int64_t* max_span);

/* Copies of the grammar (test and inspection hooks).  Each pointer may be
 * NULL to skip that array; sizes follow gcs_grammar_stats.
 *   values[|V|]; term_col/term_val[alpha]; rule_a/rule_b/rule_level/
 *   rule_plast[|R|] (plast = highest level of a rule parent, 0 if none);
 *   c_off[n_rows+1], c_sym[|C|].  Symbols as in gcs_grammar_from_rules. */
gcs_status gcs_export_grammar(const gcs_grammar* g, double* values, int32_t* term_col, int32_t* term_val,
                              int32_t* rule_a, int32_t* rule_b, int32_t* rule_level, int32_t* rule_plast,
                              int64_t* c_off, int32_t* c_sym);

/* The layered layout exactly as uploaded (for host-side emulation).
 * Arena = [T (alpha) | buffer A | buffer B]; odd levels live in A, even in
 * B.  Level k occupies [base, base + nb + npt): its nb binary nodes, then its
 * npt pass-through nodes.  Per level k (0..L): level_meta[8*k + ...] =
 *   {nb, npt, child_off, pt_off, 0, base, grp_off, n_grp};
 * child[2*i], child[2*i+1]: arena offsets of binary node i's children;
 * ptsrc[i]: arena offset of pass-through node i's source;
 * emit groups g: erow[g], epos[eoff[g] .. eoff[g+1]) (arena offsets).
 * Counts come from gcs_layout_counts. */
gcs_status gcs_layout_counts(const gcs_grammar* g, int64_t* counts8);
/* counts8 = {n_levels (L+1), n_child_pairs, n_passthrough, n_groups, n_epos, arena_elems, buf_a, buf_b} */
gcs_status gcs_export_layout(const gcs_grammar* g, int64_t* level_meta, int32_t* child, int32_t* ptsrc,
                             int32_t* erow, int32_t* eoff, int32_t* epos);

/* Column slices of the layout: every level is cut into 8 contiguous pieces by
 * first-column thresholds col_cut[0..8] (slice x = first columns in
 * [col_cut[x], col_cut[x+1])), one piece per XCD.  out[(k*3 + 0)*9 + x] =
 * first binary node of slice x at level k (x = 8: end), [(k*3+1)*9 + x] the
 * same for pass-through nodes, [(k*3+2)*9 + x] for emission groups (relative
 * to the level's first group).  Either pointer may be NULL. */
gcs_status gcs_export_slices(const gcs_grammar* g, int64_t* out, int32_t* col_cut);

/* Level 0's word stream as gcs_upload lays it out for a direct policy
 * (Boolean, tropical), computed on the host with no device call (for
 * host-side checks).  Level 0's roots are the bare terminals of C (section
 * 2, 'Grammar'); Listing 1 (section 4.3) loops over levels 1..L, and this
 * library emits level 0 right after the leaf kernel.  The upload lists
 * them per column slice and column sub-slice in row order, one 32-bit word
 * each: bits [0, 19) the terminal's offset from the chunk's first terminal
 * (0x7FFFF: no terminal, the word only advances the row), bits [19, 32) the
 * row's increase over the previous word's row (the chunk's first row for
 * its first word).  chunks[8*i .. 8*i+8) = {first word, end word, first
 * byte and end byte of the chunk's window in the device terminal array
 * (Boolean terminals are bits, bit c % 8 of byte c / 8), first row, first
 * terminal of the window, 0, 0}.  Either array may be NULL (then only the
 * counts are returned); *n_sub gets the sub-slices per slice (may be NULL).
 * All counts are 0 when the policy's upload emits level 0 otherwise: a
 * non-direct policy, GCS_LEVEL0_WINDOW=0, or a slice too wide for an LDS
 * window.  GCS_ERANGE if words_cap < *n_words or chunks_cap < 8 * *n_chunks;
 * GCS_ESTATE if the grammar's level-0 rows are out of order. */
gcs_status gcs_level0_words(const gcs_grammar* g, gcs_policy p, uint32_t* words, int64_t words_cap, int32_t* chunks,
                            int64_t chunks_cap, int64_t* n_words, int64_t* n_chunks, int32_t* n_sub);

void gcs_free_grammar(gcs_grammar* g);

/* ---- device builder ---------------------------------------------------- */

/* Bytes of the device workspace gcs_build_grammar_gpu needs for a CSR of
 * n_rows x n_cols with nnz stored entries and a pair table of table_entries
 * slots (0: the smallest power of two >= 2 nnz, always enough; a power of two
 * in [2^10, 2^32] otherwise).  About 22 bytes per nonzero plus 24 per table
 * slot.  GCS_EINVAL for negative sizes or a bad table size. */
gcs_status gcs_build_workspace_bytes(int64_t n_rows, int64_t n_cols, int64_t nnz, int64_t table_entries,
                                     size_t* bytes);

/* gcs_build_grammar with the CSRV string and RePair computed on the device
 * (section 2 'CSRV' and 'Grammar', section 4.1), in the round-based form
 * (GCS_REPAIR_ROUNDS; the result is bit for bit the grammar gcs_build_grammar
 * makes with opts.repair = GCS_REPAIR_ROUNDS and one tile); levels,
 * completion and layout run on the host as there.  m is host memory; opts may
 * be NULL, otherwise it must ask for one tile (col_chunk = row_chunk = 0,
 * natural row order) and GCS_REPAIR_ROUNDS; n_threads sets the host threads.
 * At most 64 distinct values and fewer than 2^31 - 1 nonzeros (larger
 * matrices: one call per column group).  workspace_dev: caller-owned device
 * memory of gcs_build_workspace_bytes(n_rows, n_cols, nnz, table_entries)
 * bytes, 256-byte aligned, free again when the call returns; the call runs on
 * `stream` and synchronises it several times (twice per RePair round); the
 * CSR arrays go through two 16 MiB pinned host buffers that the call
 * allocates and frees.  *out receives a new host grammar on GCS_OK.  GCS_EINVAL (bad input or
 * options, small or misaligned workspace), GCS_ERANGE (beyond the 31-bit
 * symbol space), GCS_ENOMEM (host memory, or the pair table is too small
 * for the input: pass a larger table_entries), GCS_EHIP. */
gcs_status gcs_build_grammar_gpu(const gcs_csr_view* m, const gcs_build_opts* opts, int64_t table_entries,
                                 void* workspace_dev, size_t workspace_bytes, void* stream, gcs_grammar** out);

/* ---- device ----------------------------------------------------------- */

typedef struct {
    size_t grammar_bytes;   /* read-only grammar image (child indices, pass-through sources, emit lists, emission
                               chunk table, terminals, V, launch table, narrow levels' LDS image) */
    size_t workspace_bytes; /* value arena [T | A | B], 8 x n_rows row accumulators, 256-byte counters  */
    int64_t x_len;          /* elements of x (= n_cols)                                                 */
    int64_t y_len;          /* elements of y (= n_rows)                                                 */
    int32_t x_elem_bytes;
    int32_t y_elem_bytes;
} gcs_dev_sizes;

/* Serialized grammar (section 5, Table 5.1 reports its size; section 7,
 * item 2: construction is a one-time offline cost): gcs_save_grammar writes
 * everything the upload and the inspection calls need to `path` (one binary
 * file, little-endian, ending in a checksum); gcs_load_grammar reads it back
 * into a new grammar owned by the caller (free with gcs_free_grammar) that
 * behaves exactly like the one saved.  GCS_EINVAL if the file cannot be
 * opened or written, is not a grammar file, comes from an incompatible
 * version, is truncated, fails its checksum or has inconsistent sizes
 * (gcs_last_error says which); GCS_ENOMEM if memory runs out. */
gcs_status gcs_save_grammar(const gcs_grammar* g, const char* path);
gcs_status gcs_load_grammar(const char* path, gcs_grammar** out);

/* Sizes for a policy.  GCS_EINVAL for GCS_PLUS_I64 when V has non-integral
 * values; GCS_ERANGE if the arena exceeds 2^31 - 1 elements. */
gcs_status gcs_device_layout(const gcs_grammar* g, gcs_policy p, gcs_dev_sizes* out);

/* One-time host-to-device copy (the host/device boundary) of the grammar
 * image into grammar_dev (>= grammar_bytes, 256-byte aligned) on `stream`;
 * workspace_dev (>= workspace_bytes, 256-byte aligned) holds 256 bytes of
 * counters, the value arena and the row accumulators.  Both stay owned by the
 * caller.  Several uploads may share one workspace (at least the largest of
 * their sizes) when every sweep on any of them is ordered after the others
 * (one stream): a sweep writes every arena value before reading it, and the
 * uploads then share the counters, the failure flag of gcs_device_check
 * included.  The grammar object may be freed after this
 * call returns.  The call synchronises `stream`: the copy is complete when it
 * returns.  The image goes through two 16 MiB pinned host buffers that the
 * call allocates and frees (GCS_EHIP if they cannot be had). */
gcs_status gcs_upload(const gcs_grammar* g, gcs_policy p, void* grammar_dev, size_t grammar_bytes,
                      void* workspace_dev, size_t workspace_bytes, void* stream, gcs_device** out);

/* y = M x under the uploaded policy: evaluate the terminal array (and clear
 * the row accumulators), then for k = 1..L evaluate level k and emit the
 * roots of level k-1, then emit level L (section 4.3, Listing 1), and finally
 * y[r] = the combination of row r's 8 slice accumulators.  The Boolean and
 * tropical policies emit straight into y instead (OR and min do not depend on
 * the order of the writers): y is cleared first and there are no
 * accumulators.  x_dev holds x_len elements, y_dev y_len elements, both
 * device memory of the policy's types; x is not modified.  Asynchronous on
 * `stream`.  Calls on one device handle share its workspace, so they must be
 * ordered (same stream or synchronised). */
gcs_status gcs_sweep_right(gcs_device* d, const void* x_dev, void* y_dev, void* stream);

/* y (+)= M x: as gcs_sweep_right, but row r's result is combined into the
 * existing y[r] (added; OR for the Boolean policy, min for the tropical ones)
 * instead of replacing it.
 * Lets a matrix too large for one grammar be swept as independent column
 * groups (each group its own grammar and upload, rules never spanning
 * columns of two groups), accumulating into one y. */
gcs_status gcs_sweep_right_acc(gcs_device* d, const void* x_dev, void* y_dev, void* stream);

/* Batched right product Y = M X (section 4.4, "Batched evaluation (SpMM)";
 * appendix A): nvec vectors (1..64) in one sweep over the uploaded grammar.
 * X is x_len x nvec and Y is y_len x nvec, both row-major device arrays of the
 * policy's x and y types (X[j * nvec + b] is entry j of vector b).  Every
 * value of the sweep becomes a row of nvec values, so the level buffers, the
 * slice accumulators and (unless leaves are evaluated in the sweep) the
 * terminal array live in a separate, caller-owned batch workspace of at least
 * gcs_batch_workspace_bytes(d, nvec, flags) bytes, 256-byte aligned:
 * (alpha + 2 w*) * nvec values, or 2 w* * nvec with
 * GCS_BATCH_LEAVES_IN_SWEEP, plus 8 * y_len * nvec accumulators.
 * Flags:
 *   GCS_BATCH_ACCUMULATE       Y (+)= M X instead of Y = M X
 *   GCS_BATCH_LEAVES_IN_SWEEP  no terminal array: a reference to terminal
 *                              <l, j> computes V[l] (x) X[j] where it is read
 *                              (section 7 item 3 names the Theta(alpha B)
 *                              terminal array as the cost this removes);
 *                              same results, bit for bit
 * Column b of Y equals gcs_sweep_right on column b of X up to the order of
 * floating-point additions within a row's emission (bit-exact for the
 * Boolean, int64 and tropical policies).  Asynchronous on `stream`; calls
 * sharing one workspace must be ordered.
 * GCS_EINVAL for a null handle or buffer, nvec outside 1..64, unknown flags,
 * or a workspace that is misaligned or too small. */
enum { GCS_BATCH_ACCUMULATE = 1, GCS_BATCH_LEAVES_IN_SWEEP = 2 };
gcs_status gcs_batch_workspace_bytes(const gcs_device* d, int32_t nvec, int32_t flags, size_t* bytes);
gcs_status gcs_sweep_right_batch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec, void* workspace_dev,
                                 size_t workspace_bytes, int32_t flags, void* stream);

/* gcs_sweep_right_batch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, bit for bit, with the batch
 * workspace taken from a fixed array of 64 MiB (67,108,864 bytes) in the
 * library's device code instead of a workspace argument.  Each GPU holds its
 * own copy of the array from the first gcs_upload on it until the process
 * ends.  Allocates nothing (no hipMalloc, hipFree or allocating routine).
 * GCS_ERANGE, with the size in the message, when gcs_batch_workspace_bytes(d,
 * nvec, flags) exceeds 64 MiB; other errors as gcs_sweep_right_batch.
 * Every call on a GPU shares that GPU's array and keeps the previous call's
 * contents there; a call writes every part it reads (terminal rows, level
 * buffers, accumulators cleared by its first launch) before reading it.
 * Calls that overlap on one GPU (concurrent streams or threads, any handle)
 * race on the array: order them. */
gcs_status gcs_sweep_right_batch_scratch(gcs_device* d, const void* x_dev, void* y_dev, int32_t nvec, int32_t flags,
                                         void* stream);

/* BFS fixpoint with the Boolean policy on a square matrix (section 5: one
 * Boolean pass is one frontier expansion; the fixpoint repeats it):
 *   f = visited = sources; repeat { y = M f; f = y AND NOT visited;
 *   visited |= f } until f is empty.
 * sources_dev: int64 device array of n_sources node ids (< n); frontier_dev,
 * visited_dev, y_dev: n-byte device arrays.  new_counts (host, cap entries)
 * receives |f| after each pass (the last pass gives 0); *passes the number
 * of passes.  Synchronises `stream` once per pass to read the count.
 * GCS_ESTATE if not uploaded with GCS_BOOL_OR or not square, or at the first
 * pass whose persistent tail kernel gave up at a grid barrier (read with that
 * pass's count; the device flag is cleared, *passes counts the failed pass,
 * and frontier and visited are not to be used); GCS_ERANGE if the fixpoint
 * needs more than cap passes. */
gcs_status gcs_bfs(gcs_device* d, const int64_t* sources_dev, int64_t n_sources, uint8_t* frontier_dev,
                   uint8_t* visited_dev, uint8_t* y_dev, int64_t* new_counts, int64_t cap, int64_t* passes,
                   void* stream);

/* ---- column groups swept together ---------------------------------------- */

/* Uploads of the column groups of one matrix (section 4.4: built per column
 * chunk; each group's rules reference only its own terminals, so the product
 * is the sum of the groups' products) swept as one: launch k evaluates level
 * k, with the emission of level k-1, of every group that has it, so narrow
 * levels of many groups fill the device together and need no persistent
 * tail; a last launch folds every group's slice accumulators into y.
 * y = y0 + sum_g M_g x with exactly the additions, in the same order, of
 * gcs_sweep_right on group 0 followed by gcs_sweep_right_acc on the others
 * (bit for bit).  Plus-times policies only (fp64, fp32, fp32->fp64, int64);
 * all uploads on one device with one policy and shape, each with its own
 * workspace (GCS_EINVAL if workspaces overlap).  The handles must outlive
 * the group.
 *   gcs_group_layout: bytes of the device launch table (caller-owned memory).
 *   gcs_group_create: copies the table into table_dev (256-byte aligned,
 *     synchronises `stream`).
 *   gcs_group_sweep_right: y = M x (accumulate = 0) or y += M x (1),
 *     asynchronous on `stream`; sweeps of a group, and of its member
 *     handles, must be ordered.
 *   gcs_group_profile_begin / _sweep_right_profiled / _profile_end: events
 *     right before the first and after the last level launch of each sweep;
 *     level_ms[s] = that span of sweep s.
 *   gcs_group_launches: launches per sweep. */
typedef struct gcs_group gcs_group;
gcs_status gcs_group_layout(gcs_device* const* devs, int32_t n, size_t* table_bytes);
gcs_status gcs_group_create(gcs_device* const* devs, int32_t n, void* table_dev, size_t table_bytes, void* stream,
                            gcs_group** out);
gcs_status gcs_group_sweep_right(gcs_group* g, const void* x_dev, void* y_dev, int32_t accumulate, void* stream);
gcs_status gcs_group_profile_begin(gcs_group* g, int64_t max_sweeps);
gcs_status gcs_group_sweep_right_profiled(gcs_group* g, const void* x_dev, void* y_dev, int32_t accumulate,
                                          void* stream);
gcs_status gcs_group_profile_end(gcs_group* g, float* level_ms, int64_t cap, int64_t* sweeps);
int64_t gcs_group_launches(const gcs_group* g);
void gcs_group_free(gcs_group* g);

/* ---- profiling --------------------------------------------------------- */

/* Kernel launches of one sweep: 1 (terminal array, clear accumulators), one
 * per wide level k (level k with the emission of level k-1), and 1 persistent
 * launch for the narrow levels, the emission of level L and the reduction of
 * the slice accumulators into y. */
int64_t gcs_sweep_launches(const gcs_device* d);

/* What a profiled sweep times. */
typedef enum {
    GCS_PROFILE_LAUNCHES = 0,   /* every launch: an event right before and right after each */
    GCS_PROFILE_LEVEL_SPAN = 1  /* the wide level launches together: one event right before the
                                   first and one right after the last (two events per sweep) */
} gcs_profile_mode;

/* Timing of sweeps with HIP events on the sweep's own stream, for
 * benchmarking.  gcs_profile_begin reserves events for up to max_sweeps
 * sweeps in the given mode; each gcs_sweep_right_profiled is gcs_sweep_right
 * with those events recorded; gcs_profile_end synchronises the events and
 * writes launch_ms[s * launches + i] = time between the i-th pair of events of
 * sweep s (launches = gcs_sweep_launches for GCS_PROFILE_LAUNCHES, 1 for
 * GCS_PROFILE_LEVEL_SPAN: 0 ms when the sweep has no wide level launch), then
 * releases the events.
 * GCS_EINVAL for an unknown mode; GCS_ERANGE if more than max_sweeps sweeps
 * were profiled or cap is too small; GCS_ESTATE without gcs_profile_begin. */
gcs_status gcs_profile_begin(gcs_device* d, int64_t max_sweeps, int32_t mode);
gcs_status gcs_sweep_right_profiled(gcs_device* d, const void* x_dev, void* y_dev, void* stream);
/* gcs_sweep_right_acc with the same events (a matrix swept as column groups). */
gcs_status gcs_sweep_right_acc_profiled(gcs_device* d, const void* x_dev, void* y_dev, void* stream);
gcs_status gcs_profile_end(gcs_device* d, float* launch_ms, int64_t cap, int64_t* sweeps, int64_t* launches);

/* Synchronises `stream` and reports whether any sweep since the last check
 * failed on the device: the persistent kernel that evaluates the narrow top
 * levels (at most one workgroup per compute unit, launched as an ordinary
 * kernel behind the sweep's earlier launches; GCS_TAIL_COOP=1 in the
 * environment at gcs_upload makes it a cooperative launch, for devices shared with
 * long-running kernels) waits at a grid-wide barrier with a bounded wait
 * (about a second), and flags the sweep instead of hanging if its
 * workgroups were not all resident.  A flagged sweep leaves y poisoned (NaN
 * for floating-point policies, 0xFF bytes for Boolean, INT64_MIN for int64),
 * and the flag marks only that sweep: later sweeps wait at their barriers as
 * usual.  GCS_ESTATE (and the flag cleared) if a sweep since the last check
 * was flagged, GCS_OK otherwise. */
gcs_status gcs_device_check(gcs_device* d, void* stream);

void gcs_free_device(gcs_device* d);

const char* gcs_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GCS_H */
