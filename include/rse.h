/*
 * rse.h -- C ABI of the MI355X (gfx950) sparse-embedding training hot path.
 *
 * The library implements one training step of dynamic sparse embeddings as
 * four calls:
 *
 *   idmap_find_or_insert     feature ID -> row offset, inserting new IDs
 *   blocks_grow              add a chunk of rows to the embedding blocks
 *   embedding_bag_fwd        pooled gather (sum or mean) over CSR bags
 *   embedding_bag_bwd_update merge duplicate-row gradients (sort + segmented
 *                            reduction, no floating-point atomics) and apply
 *                            a row-wise SGD / Adagrad / Adam update to the
 *                            rows seen in the batch only
 *
 * Where the operations come from (web pages; title and section):
 *  - "RecIS：阿里开源推荐系统统一训练框架" (pomoai.com), "Embedding Engine":
 *    a dynamic two-level table -- an IDMap from feature ID to memory offset
 *    over EmbeddingBlocks, contiguous chunked blocks that hold parameters and
 *    optimizer state and grow without reallocating; same-attribute tables may
 *    be merged into one.  "代码架构": a fused sparse-gradient update kernel
 *    with fewer atomics and vectorised memory access for the lookup.
 *  - "阿里 RecIS：搜广推训练的背景与难点" (muyuuuu.github.io): IDs are
 *    arbitrary and sparse over a huge range (a dense or modulo-indexed table
 *    either wastes memory or makes distinct IDs share a row); a lookup reads
 *    only the indexed row and backward updates only that row.
 *  - "DLRM模型的核心价值与工业落地挑战" (mokono.cn), section 2.1: EmbeddingBag
 *    sum pooling over variable-length inputs with sparse gradients.
 *  - "DLRM — Meta 把工业推荐模型拆成 4 个标准积木" (estelledc.github.io),
 *    "踩过的坑" item 4: a sparse optimizer that updates only the rows seen.
 *
 * Conventions for every call:
 *  - Every function returns an int status: RSE_OK (0) or a negative
 *    RSE_ERR_* code; rse_status_str() names it.  No C++ exception crosses
 *    the ABI.
 *  - Pointers named d_* are device (HBM) pointers owned by the caller; the
 *    library never allocates or frees device memory and writes only into
 *    buffers it is given.  Other pointers are host pointers.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls enqueue work on it and return without synchronising, except the
 *    query calls documented as synchronising.  All calls that touch one
 *    map or one blocks object must be ordered on one stream (or the caller
 *    synchronises between streams).
 *  - Host-detectable errors (null pointer, negative size, workspace too
 *    small, unsupported dim or dtype, too many tables) return at once and
 *    enqueue nothing.  Conditions only the device can see (map full, not
 *    enough free rows, malformed offsets) leave a sticky status in the
 *    object (read with rse_idmap_status / rse_blocks_status) and commit
 *    nothing from that call.
 *  - Layouts: ids, row offsets and CSR offsets are int64.  A batch holds
 *    n_tables * batch bags, table-major: bag j = t * batch + b spans
 *    ids[bag_offsets[j] .. bag_offsets[j+1]).  Pooled outputs and upstream
 *    gradients are fp32 [batch, n_tables, dim], sample-major.
 */
#ifndef RSE_H
#define RSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status --- */
enum {
    RSE_OK = 0,
    RSE_ERR_INVALID_ARG = -1,     /* null pointer, negative size, bad enum */
    RSE_ERR_UNSUPPORTED = -2,     /* dim / dtype / optimizer not built */
    RSE_ERR_WORKSPACE = -3,       /* workspace smaller than *_workspace_size */
    RSE_ERR_IDMAP_FULL = -4,      /* a table's keys would exceed max_load */
    RSE_ERR_NEED_GROW = -5,       /* not enough free rows: call blocks_grow */
    RSE_ERR_CHUNK_TOO_SMALL = -6, /* chunk smaller than rows_per_chunk rows */
    RSE_ERR_MAX_CHUNKS = -7,      /* chunk table full */
    RSE_ERR_HIP = -8,             /* a HIP runtime call failed */
    RSE_ERR_BAD_INPUT = -9,       /* device saw malformed offsets or ids */
    RSE_ERR_TOO_MANY_ROWS = -10   /* more than RSE_MAX_ROWS rows */
};

#define RSE_MAX_TABLES 1024
#define RSE_MAX_MERGED_TABLES 128           /* table id must fit in 7 bits */
#define RSE_MAX_ROWS 4294967294LL            /* row offsets fit in 32 bits */
#define RSE_MAX_BWD_IDS 1073741823LL         /* lookups per backward call (2^30 - 1) */

enum { RSE_F32 = 0, RSE_BF16 = 1 };               /* weight storage type */
enum { RSE_SGD = 0, RSE_ADAGRAD = 1, RSE_ADAM = 2 };
enum { RSE_SUM = 0, RSE_MEAN = 1 };

/* Name of a status code (static string). */
const char* rse_status_str(int status);

/* Library version, as major * 10000 + minor * 100 + patch. */
int rse_version(void);

/* Opaque host-side handles.  Each refers to caller device memory that must
 * outlive it. */
typedef struct rse_idmap rse_idmap;
typedef struct rse_blocks rse_blocks;

/* --------------------------------------------------- EmbeddingBlocks --- */
/*
 * EmbeddingBlocks ("RecIS", "Embedding Engine"): rows of weights plus
 * optimizer state in chunks of 2^rows_per_chunk_log2 rows.  Row r lives in
 * chunk r >> rows_per_chunk_log2 at index r & (2^rows_per_chunk_log2 - 1);
 * a row never moves once written, and adding a chunk leaves existing rows
 * in place.
 *
 * Row layout (row_bytes, a multiple of 16): weights [dim] in the storage type,
 * then fp32 state: Adagrad acc[dim]; Adam m[dim] then v[dim]; SGD none.
 *
 * A new row is initialised from its key: column c of a row with key k in
 * map table t is q * 2^-27 (fp32, q = (h >> 40) - 2^23) or q * 2^-11 (bf16,
 * q = (h >> 56) - 128), where h is the SplitMix64 output function applied to
 * (k XOR ((seed + t) * 0x9E3779B97F4A7C15)) + (c + 1) * 0x9E3779B97F4A7C15,
 * all mod 2^64; state starts at 0.  (t is 0 for a merged map.)
 */

/* Bytes of one row (host only; no GPU needed). */
int rse_blocks_row_bytes(int32_t dim, int32_t w_dtype, int32_t optim, int64_t* row_bytes_out);

/* Device bytes the caller must provide for the blocks' metadata (row counter,
 * status, chunk pointer table). */
int rse_blocks_meta_size(int32_t max_chunks, size_t* bytes_out);

/* Create a blocks object over caller memory d_meta (meta_bytes >=
 * rse_blocks_meta_size).  Supported dims: 4, 8, ..., 256 (powers of two) for
 * fp32 and 8, ..., 256 for bf16.  rows_per_chunk_log2 in [4, 32].  Clears
 * the metadata on `stream`. */
int rse_blocks_create(rse_blocks** out, void* d_meta, size_t meta_bytes, int32_t dim,
                      int32_t w_dtype, int32_t optim, int32_t rows_per_chunk_log2,
                      int32_t max_chunks, uint64_t init_seed, void* stream);
int rse_blocks_destroy(rse_blocks* blocks);

/* Register one more chunk (caller device memory, 256-byte aligned, at least
 * 2^rows_per_chunk_log2 * row_bytes bytes).  Existing rows do not move.
 * Errors: RSE_ERR_CHUNK_TOO_SMALL, RSE_ERR_MAX_CHUNKS, RSE_ERR_TOO_MANY_ROWS,
 * RSE_ERR_INVALID_ARG (null or misaligned). */
int blocks_grow(rse_blocks* blocks, void* d_chunk, size_t chunk_bytes, void* stream);

/* Host-known capacity (no synchronisation). */
int rse_blocks_capacity(const rse_blocks* blocks, int64_t* rows_capacity_out,
                        int64_t* rows_per_chunk_out, int32_t* n_chunks_out);

/* Rows in use and sticky status (synchronises `stream`). */
int rse_blocks_status(rse_blocks* blocks, int64_t* rows_used_out, int32_t* status_out,
                      void* stream);

/* Copy rows d_offs[0..n) out: weights widened to fp32 into d_w_out [n, dim],
 * optimizer state into d_state_out [n, k * dim] (k = 0, 1, 2 for SGD,
 * Adagrad, Adam; may be NULL).  Offsets must be < rows used. */
int rse_blocks_read_rows(const rse_blocks* blocks, const int64_t* d_offs, int64_t n,
                         float* d_w_out, float* d_state_out, void* stream);

/*
 * Restoring saved rows ("RecIS：阿里开源推荐系统统一训练框架", "Saver": the
 * sparse parameters and their optimizer state are exported and imported).
 * rse_blocks_write_rows is the inverse of rse_blocks_read_rows: row
 * d_offs[i] receives weights d_w[i, :] (fp32; bf16 storage rounds to nearest
 * even, which is exact for values read from bf16 rows) and state
 * d_state[i, :] (k * dim floats, NULL for SGD).  Offsets outside the
 * capacity set the sticky status RSE_ERR_BAD_INPUT and are skipped.  The row
 * counter is not changed; rse_blocks_set_rows_used sets it (0 <= rows_used
 * <= capacity, else RSE_ERR_INVALID_ARG), so that keys inserted later get
 * the rows after the restored ones.
 */
int rse_blocks_write_rows(rse_blocks* blocks, const int64_t* d_offs, int64_t n, const float* d_w,
                          const float* d_state, void* stream);
int rse_blocks_set_rows_used(rse_blocks* blocks, int64_t rows_used, void* stream);

/* ------------------------------------------------------------- IDMap --- */
/*
 * IDMap ("RecIS", "Embedding Engine"): an open-addressing hash map from a
 * 64-bit feature ID to a row offset.  Each table has its own region of
 * 16-byte slots {key, value}, probed in buckets of 8 slots (one 128-byte
 * line) from the bucket chosen by a 64-bit mix of the key; inserts are
 * lock-free (64-bit compare-and-swap).  Every int64 is a legal key: the
 * value used to mark an empty slot is kept in a per-table side slot.
 *
 * merged = 1 ("RecIS": merging same-attribute tables): one region for all
 * logical tables, keyed by (t << 56) | id; ids must lie in [0, 2^56) and
 * there may be at most RSE_MAX_MERGED_TABLES logical tables.
 */

/* Device bytes for a map with n_tables regions (slots_per_table: host array,
 * each rounded up to a multiple of 8 slots). */
int rse_idmap_mem_size(int32_t n_tables, const int64_t* slots_per_table, size_t* bytes_out);

/* Create a map over caller memory d_mem and clear it on `stream`.
 * max_load in (0, 0.95]: a table refuses inserts beyond max_load * slots.
 * For merged = 1, n_tables must be 1 (one region). */
int rse_idmap_create(rse_idmap** out, void* d_mem, size_t mem_bytes, int32_t n_tables,
                     const int64_t* slots_per_table, double max_load, int32_t merged,
                     uint64_t hash_seed, void* stream);
int rse_idmap_destroy(rse_idmap* map);

/* Workspace bytes for one idmap_find_or_insert over n_ids lookups. */
int rse_idmap_workspace_size(int64_t n_ids, size_t* bytes_out);

/*
 * Map every lookup to its row offset, inserting missing keys if
 * insert_missing != 0.
 *
 * Table t's lookups are d_ids[d_bounds[t*stride] .. d_bounds[(t+1)*stride])
 * for t in [0, n_tables); with d_bounds = the bag offsets and stride = batch
 * this is the table-major bag layout.  d_bounds[0] must be 0 and
 * d_bounds[n_tables*stride] must equal n_ids.
 *
 * New keys receive consecutive offsets from the blocks' row counter in order
 * of first sight (lookup index order); their rows are initialised (see
 * EmbeddingBlocks) and the row counter advances by the number of new keys,
 * written to *d_n_new_out (device int64).  A missing key without insert
 * gives offset -1, which pooling and backward skip.
 *
 * If the new keys would exceed a table's max_load (RSE_ERR_IDMAP_FULL) or
 * the free rows (RSE_ERR_NEED_GROW), nothing is inserted, missing keys get
 * -1, *d_n_new_out is 0 and the map's sticky status is set; the caller may
 * grow and repeat the call with identical results.
 *
 * d_ws: rse_idmap_workspace_size(n_ids) bytes of device scratch.
 */
int idmap_find_or_insert(rse_idmap* map, rse_blocks* blocks, const int64_t* d_ids,
                         int64_t n_ids, const int64_t* d_bounds, int64_t stride,
                         int32_t n_tables, int32_t insert_missing, int64_t* d_row_off_out,
                         int64_t* d_n_new_out, void* d_ws, size_t ws_bytes, void* stream);

/*
 * idmap_find_or_insert without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results, errors and
 * stream semantics as idmap_find_or_insert; the scratch is a static array of
 * the library on each GPU (about 52 MiB, allocated when the library's code
 * is loaded on that GPU and held until the process ends), so the call
 * allocates nothing.  It uses the scratch of the current device (hipGetDevice);
 * `stream` must belong to that device.
 *
 * Limit: n_ids <= RSE_NOALLOC_MAX_IDS, else RSE_ERR_WORKSPACE with nothing
 * enqueued.  All calls on one GPU share its scratch: two calls that may run
 * at the same time on that GPU (different streams, or different host threads)
 * race and give wrong results; order them on one stream.
 */
#define RSE_NOALLOC_MAX_IDS 2097152LL
int idmap_find_or_insert_noalloc(rse_idmap* map, rse_blocks* blocks, const int64_t* d_ids,
                                 int64_t n_ids, const int64_t* d_bounds, int64_t stride,
                                 int32_t n_tables, int32_t insert_missing,
                                 int64_t* d_row_off_out, int64_t* d_n_new_out, void* stream);

/* Sticky status and per-table key counts (host array of the map's n_tables,
 * may be NULL).  Synchronises `stream`. */
int rse_idmap_status(rse_idmap* map, int32_t* status_out, int64_t* n_keys_out, void* stream);

/* Reset the sticky status of a map or blocks object to RSE_OK. */
int rse_idmap_clear_status(rse_idmap* map, void* stream);
int rse_blocks_clear_status(rse_blocks* blocks, void* stream);

/* Copy the live entries (any order) into d_keys_out / d_table_out /
 * d_off_out, at most `capacity` of them; the number of live entries is
 * written to *d_count_out.  In merged mode keys are (t << 56) | id and the
 * table index is 0. */
int rse_idmap_export(rse_idmap* map, int64_t* d_keys_out, int32_t* d_table_out,
                     int64_t* d_off_out, int64_t capacity, int64_t* d_count_out, void* stream);

/*
 * Insert saved entries (the inverse of rse_idmap_export, "RecIS", "Saver"):
 * key d_keys[i] of table d_tables[i] (0 for a merged map, whose keys are
 * already (t << 56) | id) maps to row d_offs[i].  The keys must not be in
 * the map yet.  A table index or offset out of range, or a duplicate key,
 * sets the sticky status RSE_ERR_BAD_INPUT; entries that would take a
 * table past its max_load set RSE_ERR_IDMAP_FULL and nothing is inserted.
 * After a duplicate the map's contents are unspecified (recreate it).
 * The blocks' rows are not touched: restore them with rse_blocks_write_rows.
 */
int rse_idmap_import(rse_idmap* map, const int64_t* d_keys, const int32_t* d_tables, const int64_t* d_offs,
                     int64_t n, void* stream);

/* ----------------------------------- admission, eviction, resize ----- */
/*
 * The hook on the hash table for feature admission and eviction ("RecIS：
 * 阿里开源推荐系统统一训练框架", "代码架构").  The pages name the hook but
 * give no policy; the policies here are definitions:
 *
 * Age.  rse_idmap_set_stamps attaches one uint32 stamp per row (caller
 * memory, n_stamps >= the blocks' capacity at every find call, else that
 * call returns RSE_ERR_INVALID_ARG; the caller zeroes it).  While attached,
 * every lookup of idmap_find_or_insert that resolves to a row writes the
 * map's clock (rse_idmap_set_clock, host-side, no launch) into the row's
 * stamp.  NULL / 0 detaches.  A call that fails may already have stamped
 * the rows it found.
 *
 * Admission.  rse_idmap_set_admission attaches a count-min sketch of
 * `depth` (1..8) rows of `width` uint32 counters (caller memory, depth *
 * width entries; the call zeroes it on `stream`) and a threshold.  With
 * insert_missing, every lookup of a key absent from the map when the call
 * starts adds 1 to the key's counter in each row (counter j of key k in
 * region r: fmix64(k ^ r * 0x9E3779B97F4A7C15 ^ salt_j) reduced to
 * [0, width) by a 64x64 multiply-high, salt_j the (j+1)-th SplitMix64
 * output of `seed`); then an absent key is inserted iff the minimum of its
 * counters is >= threshold, else its lookups get -1.  All lookups of a key
 * in a call get the same answer.  Counters never decay (they wrap after
 * 2^32 counts).  threshold <= 1 turns admission off (d_sketch may be NULL).
 * A call that fails (capacity) takes its counts back; a call with a bad id
 * counts nothing.
 *
 * Eviction and resize.  rse_idmap_rehash clears `dst` (a map with the same
 * number of tables and the same merged flag as `src`, in memory that does
 * not overlap it; any size) and copies every key of `src` into it with the
 * same offset, except, when `src` has stamps attached, keys whose row's
 * stamp is below min_clock (those are evicted).  With min_clock 0 or no
 * stamps it is a plain resize.  If a table's kept keys exceed dst's
 * max_load, dst's sticky status becomes RSE_ERR_IDMAP_FULL, dst stays empty
 * and nothing else changes.  Otherwise, if the blocks have a free list
 * (rse_blocks_set_free_list, capacity >= the blocks' capacity, else
 * RSE_ERR_INVALID_ARG), it is rebuilt: every row below rows_used that no
 * kept key references, ascending; idmap_find_or_insert then gives new keys
 * (ranked by first sight) the listed rows in order before it takes rows
 * past rows_used, and initialises them like new rows.  Without a free list
 * evicted rows are not reused.  `src` is not modified; dst takes over
 * src's stamps, clock and admission settings (host side).  Workspace: at
 * least rse_idmap_rehash_workspace_size bytes (a bit per row of the blocks'
 * capacity and per slot of src); stream-ordered, no synchronisation.  A
 * row offset in `src` at or beyond the blocks' capacity fails the call with
 * RSE_ERR_BAD_INPUT in dst's status.
 */
int rse_idmap_set_stamps(rse_idmap* map, uint32_t* d_stamps, int64_t n_stamps);
int rse_idmap_set_clock(rse_idmap* map, uint32_t clock);
int rse_idmap_set_admission(rse_idmap* map, uint32_t* d_sketch, int32_t depth, int64_t width,
                            uint32_t threshold, uint64_t seed, void* stream);
int rse_idmap_rehash_workspace_size(const rse_idmap* src, const rse_blocks* blocks, size_t* bytes_out);
int rse_idmap_rehash(rse_idmap* dst, rse_idmap* src, rse_blocks* blocks, uint32_t min_clock, void* d_ws,
                     size_t ws_bytes, void* stream);

/* Attach a free list of rows (caller memory, `capacity` uint32 entries;
 * NULL / 0 detaches).  Either way the list is emptied (on `stream`); a later
 * rse_idmap_rehash fills it. */
int rse_blocks_set_free_list(rse_blocks* blocks, uint32_t* d_free, int64_t capacity, void* stream);
/* Entries of the free list handed out so far and entries left (those are
 * d_free[head .. head + count)).  Synchronises `stream`. */
int rse_blocks_free_status(rse_blocks* blocks, int64_t* head_out, int64_t* count_out, void* stream);

/* ------------------------------------------- fused feature transforms -- */
/*
 * Raw feature values -> int64 ids for every table in one launch ("RecIS：
 * 阿里开源推荐系统统一训练框架", "Feature Engine": Hash, Mod and Bucketize,
 * small operations merged into one GPU kernel launch).  The pages name the
 * operations only; definitions:
 *
 * Lookup i of table t (bounds[t*stride] <= i < bounds[(t+1)*stride], the
 * ids' table-major layout) holds one 64-bit raw value; table t's program
 * says whether that is an int64 (RSE_FT_INT64) or the bits of a float64
 * (RSE_FT_FLOAT64) and applies up to RSE_FT_MAX_OPS operations in order:
 *   RSE_FT_HASH, arg = seed (bits): XXH64 (xxHash64 of the value's 8
 *     little-endian bytes with that seed); the digest read as int64;
 *   RSE_FT_MOD, arg = m > 0: floor modulo of the value as a signed int64,
 *     a result in [0, m);
 *   RSE_FT_BUCKETIZE, arg = index of the table's first boundary in the
 *     boundary array, n_boundaries = their number (ascending, no NaN):
 *     the number of boundaries <= x for the float64 x (NaN: all of them);
 *   RSE_FT_IDENTITY: nothing.
 * An integer program may use Hash and Mod; a float program must start with
 * Bucketize or Hash; the value after the last operation is the id.
 *
 * rse_features_create validates the programs and boundaries on the host
 * (RSE_ERR_INVALID_ARG if any breaks these rules) and copies them into
 * caller device memory of rse_features_mem_size bytes (256-byte aligned);
 * it synchronises `stream`.  feature_transform writes ids[0..n) (it may
 * write in place over the raw array); malformed bounds (bounds[0] != 0,
 * bounds[n_tables*stride] != n, a decreasing pair) set the sticky status
 * RSE_ERR_BAD_INPUT (rse_features_status, synchronising) and write nothing.
 */
#define RSE_FT_MAX_OPS 4
enum { RSE_FT_INT64 = 0, RSE_FT_FLOAT64 = 1 };
enum { RSE_FT_IDENTITY = 0, RSE_FT_HASH = 1, RSE_FT_MOD = 2, RSE_FT_BUCKETIZE = 3 };
typedef struct rse_feature_op {
    int32_t kind;
    int32_t n_boundaries;   /* RSE_FT_BUCKETIZE */
    int64_t arg;
} rse_feature_op;
typedef struct rse_feature_program {
    int32_t input;          /* RSE_FT_INT64 | RSE_FT_FLOAT64 */
    int32_t n_ops;
    rse_feature_op ops[RSE_FT_MAX_OPS];
} rse_feature_program;
typedef struct rse_features rse_features;

int rse_features_mem_size(int32_t n_tables, int64_t n_boundaries, size_t* bytes_out);
int rse_features_create(rse_features** out, void* d_mem, size_t mem_bytes, const rse_feature_program* programs,
                        int32_t n_tables, const double* boundaries, int64_t n_boundaries, void* stream);
int rse_features_destroy(rse_features* features);
int feature_transform(const rse_features* features, const int64_t* d_raw, int64_t n, const int64_t* d_bounds,
                      int64_t stride, int64_t* d_ids_out, void* stream);
int rse_features_status(rse_features* features, int32_t* status_out, void* stream);

/* ------------------------------------------------- pooled forward ----- */
/*
 * out[b, t, :] = sum over the rows of bag j = t*batch + b ("DLRM ... 2.1":
 * EmbeddingBag sum), divided by the bag length for RSE_MEAN.  Rows are
 * accumulated in fp64 in bag order and rounded once to fp32; an empty bag
 * gives 0; offset -1 contributes nothing.  bag_offsets[0] must be 0 and
 * bag_offsets[n_tables*batch] must equal n_ids.  Malformed offsets (those
 * endpoints, a decreasing pair, an offset outside [0, n_ids]) and rows at or
 * beyond the blocks' capacity set the blocks' sticky status to
 * RSE_ERR_BAD_INPUT; the bags they concern are skipped (their output is not
 * written) or the row is left out of the sum, and nothing is read out of
 * bounds.
 */
int embedding_bag_fwd(const rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                      const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                      int32_t pooling, float* d_out, void* stream);

/* ------------------------------------------ sparse backward + update -- */
typedef struct rse_optim {
    int32_t kind;   /* RSE_SGD | RSE_ADAGRAD | RSE_ADAM */
    int32_t reserved;
    double lr;
    double eps;     /* Adagrad, Adam */
    double beta1;   /* Adam */
    double beta2;   /* Adam */
    int64_t step;   /* Adam: 1-based global step of this update */
} rse_optim;

/* Workspace bytes for one embedding_bag_bwd_update. */
int rse_bwd_workspace_size(int64_t n_ids, int32_t n_tables, int64_t batch, int32_t dim,
                           size_t* bytes_out);

/*
 * Sparse backward and row-wise update ("RecIS", "代码架构": fused sparse
 * gradient update; "DLRM", "踩过的坑" 4: sparse optimizer).
 *
 * Lookup i of bag j = t*batch + b contributes g_i = grad[b, t, :] (divided
 * by the bag length for RSE_MEAN) to row d_row_off[i].  The (row, bag)
 * pairs are radix-sorted by row (stable), so each touched row's g is the
 * fp64 sum of its contributions in lookup order (segments longer than 64
 * are summed in pieces of 64 lookups, 32 for fp32 rows of dim 16 or less,
 * and the pieces added in a fixed order); no
 * floating-point atomics are used and the result is run-to-run identical.
 * Then, once per touched row, in fp64 and rounded once to the storage type:
 *   SGD:     w -= lr * g
 *   Adagrad: a = fp32(a + g*g);  w -= lr * (g / (sqrt(a) + eps))
 *   Adam:    m = fp32(b1 m + (1-b1) g);  v = fp32(b2 v + (1-b2) g g);
 *            w -= lr * ((m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps))
 * (Adam is the lazy form of Kingma & Ba 2015, Algorithm 1).  The square
 * roots and the quotients by (sqrt(.) + eps) are computed to about 1e-14
 * relative (fp32 estimates refined by one Newton step in fp64), the mean
 * pooling share as g * (1 / len), the bias corrections as products with
 * precomputed reciprocals.  bf16 weights round to nearest even.  Rows not in the batch are not read or written.
 * The number of distinct touched rows is written to *d_n_unique_out.
 * n_ids may not exceed RSE_MAX_BWD_IDS.  The device sort waits on results of
 * other workgroups with a bounded spin; should a wait time out, nothing is
 * updated, *d_n_unique_out stays 0 and the blocks' sticky status becomes
 * RSE_ERR_HIP.
 */
int embedding_bag_bwd_update(rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                             const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                             int32_t pooling, const float* d_grad, const rse_optim* opt,
                             int64_t* d_n_unique_out, void* d_ws, size_t ws_bytes,
                             void* stream);

/*
 * embedding_bag_bwd_update in two halves, so that the half that does not need
 * the gradient can run while the forward does (same passages as above).
 *
 * embedding_bag_bwd_prepare validates the bag offsets and row offsets,
 * sorts the lookups by row into d_ws and indexes the runs of equal rows
 * (one-lookup, short and long segments); it reads only d_row_off and
 * d_bag_offsets, so it may run on another stream concurrently with
 * embedding_bag_fwd of the same batch (the caller orders it after the
 * find-or-insert that wrote d_row_off).  *plan_out (host memory, caller
 * owned) receives what the apply needs: the key width and the key used for
 * lookups without a row, both fixed from the blocks' capacity at this call,
 * so a blocks_grow between the halves is harmless.
 *
 * embedding_bag_bwd_apply reduces the gradient over the sorted lookups and
 * updates the rows; it must be ordered after the prepare that wrote d_ws and
 * plan (on one stream, or with an event), with the same d_ws, n_tables,
 * batch and d_bag_offsets contents.  A plan may be applied more than once
 * (each apply updates the rows again).  d_ws must not be reused by another
 * prepare until the apply has run.  Bad input found by the prepare (sticky
 * status RSE_ERR_BAD_INPUT) makes the apply update nothing and write 0 to
 * *d_n_unique_out.  Returns RSE_ERR_INVALID_ARG if plan does not match the
 * call (n_tables * batch, the blocks' dim).
 */
typedef struct rse_bwd_plan {
    int64_t n_ids;         /* lookups sorted */
    int64_t n_bags;        /* n_tables * batch */
    uint32_t invalid;      /* sort key of lookups without a row: 2^key_bits - 1 */
    int32_t key_bits;      /* bits of the row keys sorted on */
    int32_t sorted_in_alt; /* which half of the workspace holds the sorted pairs */
    int32_t dim;           /* the blocks' dim */
} rse_bwd_plan;

int embedding_bag_bwd_prepare(rse_blocks* blocks, const int64_t* d_row_off, int64_t n_ids,
                              const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                              void* d_ws, size_t ws_bytes, rse_bwd_plan* plan_out, void* stream);

int embedding_bag_bwd_apply(rse_blocks* blocks, const rse_bwd_plan* plan,
                            const int64_t* d_bag_offsets, int32_t n_tables, int64_t batch,
                            int32_t pooling, const float* d_grad, const rse_optim* opt,
                            int64_t* d_n_unique_out, void* d_ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------- DLRM dot interaction -- */
/*
 * "DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "核心思想" item 3 and "案例 3":
 * the dense vector (bottom-MLP output) and the N pooled embeddings of each
 * sample are stacked, every pair of them is dotted, the strict upper
 * triangle is kept and concatenated after the dense vector
 * ([4,3,4] pooled -> [4,6] -> [4,10] for batch 4, d 4, N = 3).
 *
 * With F = n_tables + 1 vectors per sample, x_0 = d_dense[b, :] and
 * x_{t+1} = d_pooled[b, t, :] (the layout embedding_bag_fwd writes), and the
 * P = F (F - 1) / 2 pairs i < j in row-major order (0,1), (0,2), ...,
 * (0,F-1), (1,2), ...:
 *   dlrm_interaction_fwd: d_out [batch, dim + P] fp32:
 *     out[b, 0:dim] = x_0,  out[b, dim + p(i,j)] = x_i . x_j
 *   dlrm_interaction_bwd: from d_dout [batch, dim + P], with g_ij = g_ji =
 *     dout[b, dim + p(i,j)] and dx_i = sum_{j != i} g_ij x_j:
 *     d_ddense [batch, dim] = dout[b, 0:dim] + dx_0,
 *     d_dpooled [batch, n_tables, dim] = dx_{t+1}  (the upstream gradient
 *     embedding_bag_bwd_update takes).
 * Precision: with n_tables + 1 <= 32 and dim in {32, 64, 128} the
 * matrix cores compute the dot products in fp32 over blocks of at most 64
 * elements, the blocks added in fp64 (|error| <= 65 * 2^-24 * sum_k
 * |x_ik x_jk|), and the gradients in fp32 (|error| <= 33 * 2^-24 *
 * sum_j |g_ij x_jk|, plus one rounding for the dense gradient); other
 * shapes accumulate in fp64 (products of fp32 values are exact) and round
 * once.  All pointers are device pointers; the inputs are not modified.
 * RSE_ERR_UNSUPPORTED if one sample's vectors and pair matrix,
 * (n_tables + 1) * (dim + 1 + n_tables + 1) floats, exceed 64 KiB.
 */
int dlrm_interaction_fwd(const float* d_dense, const float* d_pooled, int64_t batch, int32_t n_tables,
                         int32_t dim, float* d_out, void* stream);
int dlrm_interaction_bwd(const float* d_dense, const float* d_pooled, const float* d_dout, int64_t batch,
                         int32_t n_tables, int32_t dim, float* d_ddense, float* d_dpooled, void* stream);

/* ------------------------------------------------------- kernel trace -- */
/*
 * Per-kernel timing with HIP events, for measurement: while a trace is
 * active the library records an event pair on the launch stream around every
 * launch of the chosen kernel (process-wide, up to 4096 launches).  Host
 * code only; recording adds two stream markers per traced launch.
 */
enum {
    RSE_K_PROBE = 1,       /* IDMap probe / insert-claim kernel */
    RSE_K_FWD = 2,         /* pooled forward kernel */
    RSE_K_SORT_SCATTER = 3, /* radix-sort scatter (one per digit pass) */
    RSE_K_SEG_UPDATE = 4,  /* segmented reduction + fused optimizer */
    RSE_K_COMBINE = 5,     /* long-segment combine */
    RSE_K_INTERACT = 6     /* DLRM dot interaction forward */
};

/* Start tracing `kernel` (one RSE_K_* id); clears earlier records. */
int rse_trace_start(int32_t kernel);

/* Stop tracing; synchronises the recorded events and returns the number of
 * traced launches and their summed duration in milliseconds. */
int rse_trace_stop(int64_t* n_launches_out, double* total_ms_out);

#ifdef __cplusplus
}
#endif
#endif /* RSE_H */
