/*
 * mi355emb -- one training step of a GPU-resident sparse embedding layer on MI355X (gfx950).
 *
 * The step the library runs, and where each part is described:
 *   - A unified, insert-free hash table.  Keys are int64 with the raw id in the low 48 bits and the
 *     field (table) id in the high 16 bits, so all fields share one table and one kernel serves the
 *     lookup and one the update (Tencent PCG GPU training talk, "compute optimisation", unified
 *     hash table paragraph).  The table is prepared off-GPU and copied to HBM in one piece per PASS;
 *     there is no insert (same talk, flash paragraph of "optimisations of each stage").  Optionally
 *     split in two tables by key parity ("Multiple Hash") with per-field row widths ("dynamic
 *     embedding") (same talk, space optimisation).
 *   - Forward: probe every key of a CSR batch and sum-pool each bag, as EmbeddingBag(mode='sum')
 *     over flat ids and offsets (JD ads article, section 4.2.1).
 *   - Backward: deduplicate the touched rows, reduce each row's gradient over its occurrences, and
 *     apply element-wise sparse Adagrad to those rows only; untouched rows and state stay as they
 *     are (JD ads article, section 3.2.1), with fp16 rows, an fp32 master copy for the update and
 *     fp32 optimizer state (JD ads article, sections 3.2.3 and 5.2).
 *
 * Conventions for every function:
 *   - Return value: 0 (EMB_OK) or a negative emb_status.  Nothing throws.  emb_last_error() gives a
 *     thread-local message for the last failure on the calling thread.
 *   - "d_" pointers are device pointers (HBM), owned by the caller; the hot-path entry points never
 *     allocate device memory.  Host pointers passed to a function are only read during the call.
 *   - Device buffers read or written with vector accesses (d_out, d_rowref, d_grad, d_ws) must be
 *     16-byte aligned (EMB_EINVAL otherwise); torch allocations are.
 *   - Device work is enqueued on the caller's stream (a hipStream_t passed as void*, NULL = the null
 *     stream) and is asynchronous unless a function says it synchronises.
 *   - A table object is not thread-safe; distinct tables are independent.
 *   - Batch validation: with the environment variable EMB_VALIDATE=1, every call that takes a
 *     batch (lookup_pool_fwd, lookup_probe, pool_fwd, sparse_adagrad_bwd, sparse_ftrl_bwd,
 *     sparse_bwd_dedup) first checks it on the device -- offsets[0] == 0, offsets never
 *     decrease, offsets[n_bags] == nnz, and for the calls that take rowrefs, each rowref is
 *     EMB_ROWREF_MISS or names a whole row of its bag's field inside the table -- and returns
 *     EMB_EINVAL naming the failed check.  The check costs O(nnz) device work, allocates 256
 *     bytes of device memory once per table and synchronises the stream.  Without it the kernels
 *     clamp offsets into [0, nnz] and treat rowrefs at or above the table's rowref space as
 *     misses, so malformed input gives wrong results but no access outside the caller's buffers
 *     and the table's arena.
 */
#ifndef MI355EMB_H
#define MI355EMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct EmbTable EmbTable; /* opaque; created and destroyed by the library */
typedef void* emb_stream_t;       /* a hipStream_t */

typedef enum { EMB_F32 = 0, EMB_F16 = 1 } emb_dtype;

typedef enum {
  EMB_OK = 0,
  EMB_EINVAL = -1,     /* bad argument: null pointer, bad size, bad descriptor field */
  EMB_EDUPKEY = -2,    /* the prebuilt key set holds a key twice */
  EMB_ESENTINEL = -3,  /* a prebuilt key equals the EMPTY marker (all 64 bits set) */
  EMB_ERANGE = -4,     /* a field id >= n_fields, or a size beyond a documented limit */
  EMB_ENOSPACE = -5,   /* arena or workspace smaller than required */
  EMB_ESTATE = -6,     /* call out of order, e.g. lookup before pass_flash */
  EMB_EHIP = -7,       /* a HIP runtime call failed; the HIP error text is in emb_last_error() */
  EMB_ENOMEM = -8      /* host allocation failed */
} emb_status;

/* Marker stored in rowref for an occurrence that found no row. */
#define EMB_ROWREF_MISS 0xFFFFFFFFu

/* Table flags. */
#define EMB_FLAG_PINNED_STAGING 1 /* keep the host image in pinned memory (needs a GPU at create) */
/* The forward probes buckets either one lane per key or eight lanes per bucket (wave-cooperative);
 * by default it picks the cooperative form for bucket arrays of 2 GiB and more, where the per-lane
 * form's address translations thrash.  These flags force one form (both give the same results). */
#define EMB_FLAG_PROBE_COOP 2
#define EMB_FLAG_PROBE_LANE 4
/* Keep a device bitmap with one bit per rowref unit, set by sparse_adagrad_bwd for every row it
 * updates and cleared by each pass_flash, so that pass_writeback_touched can copy back only the
 * rows a PASS changed.  Costs rowref_space / 8 bytes of arena and one atomic per updated row. */
#define EMB_FLAG_TRACK_TOUCHED 8
/* Keep the FTRL-Proximal linear state z (fp32 per row element, zero at create) beside the
 * accumulator, so that sparse_ftrl_bwd can update the table.  The state travels with the rows in
 * pass_flash, both write-backs and table_carry_state. */
#define EMB_FLAG_FTRL 16

typedef struct {
  int32_t n_fields;          /* F, 1..65535; field id 0xFFFF is reserved for the EMPTY marker */
  const int32_t* field_dim;  /* F row widths, each a multiple of 8 in [8, 256] */
  int32_t row_dtype;         /* EMB_F32 or EMB_F16 */
  int32_t has_master;        /* 1: keep an fp32 master copy beside fp16 rows (EMB_F16 only) */
  int32_t n_tables;          /* 1: one unified table; 2: two tables, a key lives in table (key & 1) */
  double load_factor;        /* in (0, 1]; each table gets ceil(N_t / load_factor) home slots */
  float acc_init;            /* Adagrad accumulator start value when no accumulator is supplied */
  int32_t flags;             /* EMB_FLAG_* */
} EmbTableDesc;

typedef struct {
  uint64_t arena_bytes;      /* device bytes pass_flash needs */
  uint64_t key_bytes;        /* of which the probed key buckets */
  uint64_t state_bytes;      /* of which rows + accumulator + master */
  uint64_t n_keys;
  uint64_t total_elems;      /* row elements over all keys */
  uint32_t rowref_space;     /* rowref values run over [0, rowref_space) */
  uint32_t granule;          /* row elements per rowref unit */
  uint64_t n_home[2];        /* home slots per table */
  uint64_t n_keys_t[2];      /* keys per table */
  uint64_t n_buckets[2];     /* 128-byte buckets per table */
  double mean_displacement;  /* mean of (slot - home) over all keys */
  uint64_t max_displacement;
  uint32_t unique_by_width;  /* 1: sparse_adagrad_bwd lists unique rows grouped by row width */
} EmbTableInfo;

/*
 * Build the table from a prebuilt key set (the PASS's deduplicated keys) and each key's row and
 * optimizer state.  Host only: no device work.
 *   keys   : n_keys int64 keys, any order.  Must be distinct (EMB_EDUPKEY), never all-ones
 *            (EMB_ESENTINEL), with field id (key >> 48) < n_fields (EMB_ERANGE).
 *   rows   : row data packed in key order; key i contributes field_dim[field(key i)] elements of
 *            row_dtype.  NULL: rows start at zero, or at fp16(master) when master is given.
 *   acc    : fp32, same packing as rows.  NULL: every element starts at desc->acc_init.
 *   master : fp32, same packing (fp16 tables with has_master only).  NULL: master = fp32(row).
 * Layout (ordered linear probing in 128-byte buckets of 15 keys; rows stored in slot order) is a
 * pure function of the key set.  The inputs are copied; the caller may free them on return.
 * Size limits (EMB_ERANGE): each table at most 2^32 - 16 buckets, both tables' bucket arrays
 * together below 2^32 buckets (512 GiB), and the rowref space below 2^32 units.
 */
int table_create_from_prebuilt(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys,
                               const void* rows, const float* acc, const float* master,
                               EmbTable** out);

/*
 * table_create_from_prebuilt(desc, keys, n_keys, NULL, NULL, NULL) with the layout computed on the
 * GPU: the keys go over to d_ws, are radix-sorted there by (table, home slot) with equal homes
 * ordered by key, placed by a prefix-max scan (slot_i = max(home_i, slot_{i-1} + 1) is
 * i + max_{j<=i}(home_j - j)), and their rowrefs come from a prefix sum of row units; the key
 * buckets and the rowref order come back to the host.  The table, its image and every later
 * result are identical to the host build's (the pages prepare each PASS's table off the GPU:
 * Tencent PCG GPU training talk, flash paragraph; this moves the sort, the longest part of that
 * preparation at 800M keys, onto the GPU).  Rows start at zero and accumulators at acc_init: fill
 * them with table_fill_state before the first pass_flash.
 *   d_ws, ws_bytes : device workspace, 256-byte aligned, at least table_build_workspace_bytes()
 *                    (EMB_ENOSPACE); free again when the call returns.  The arena the table will
 *                    be flashed into may serve, since nothing is flashed yet.
 * Synchronises `stream`.  Errors as for table_create_from_prebuilt; n_keys must be below 2^31
 * (EMB_ERANGE); EMB_EHIP on a failed device call.
 */
int table_build_workspace_bytes(const EmbTableDesc* desc, int64_t n_keys, size_t* bytes);
int table_create_on_device(const EmbTableDesc* desc, const int64_t* keys, int64_t n_keys,
                           void* d_ws, size_t ws_bytes, emb_stream_t stream, EmbTable** out);

/* Sizes and builder statistics of a table (host only). */
int table_info(const EmbTable* t, EmbTableInfo* info);

/* Device bytes pass_flash needs in its arena (host only). */
int table_device_bytes(const EmbTable* t, size_t* bytes);

/*
 * Copy the whole prebuilt table (key buckets, rows, accumulator, master, field metadata) into the
 * caller's device arena in one bulk host-to-device copy, enqueued on `stream`.  The arena must be
 * 256-byte aligned and at least table_device_bytes() long (EMB_ENOSPACE).  The arena stays bound
 * to the table until the next pass_flash or table_destroy; rowrefs from an earlier flash are
 * invalid afterwards.  A pinned host image (EMB_FLAG_PINNED_STAGING) goes over in one DMA and the
 * call returns once it is enqueued.  A pageable image goes through two 256 MiB pinned bounce
 * buffers owned by the table (allocated at the first such copy; a plain copy when that fails):
 * the host copies one chunk while the DMA of the previous one runs, so the call returns only once
 * the last chunk is enqueued.
 */
int pass_flash(EmbTable* t, void* d_arena, size_t arena_bytes, emb_stream_t stream);

/*
 * Forward: one launch probes every key and sum-pools every bag.
 *   d_keys    : nnz int64 keys of the CSR batch.
 *   d_offsets : n_bags + 1 int32 offsets, offsets[0] = 0, non-decreasing, offsets[n_bags] = nnz.
 *               Bag j belongs to sample j / F and field j % F (sample-major); n_bags % F == 0.
 *   d_out     : [n_bags / F, sum_f field_dim[f]] of out_dtype, row-major; field f of sample b is
 *               written at columns [sum_{f'<f} field_dim[f'], + field_dim[f]).  Every element is
 *               written (an empty bag gives zeros).  Sums are taken in fp32 and rounded once.
 *   d_rowref  : nnz uint32, the row each occurrence resolved to (EMB_ROWREF_MISS when the key is
 *               absent, is the EMPTY marker, or has a field id other than its bag's field).  This is
 *               the state sparse_adagrad_bwd consumes; it is valid until the next pass_flash.
 *   d_slot    : nullable; nnz int64 logical slot of each occurrence in its table (-1 on a miss).
 *   d_n_miss  : nullable; one int64 to which the number of missed occurrences is added.
 * A miss adds nothing to its bag.  Errors: EMB_ESTATE before pass_flash; EMB_EINVAL on null
 * required pointers, n_bags % F != 0, nnz < 0 or n_bags/nnz >= 2^31.
 */
int lookup_pool_fwd(EmbTable* t, const int64_t* d_keys, const int32_t* d_offsets, int64_t n_bags,
                    int64_t nnz, void* d_out, int32_t out_dtype, uint32_t* d_rowref,
                    int64_t* d_slot, int64_t* d_n_miss, emb_stream_t stream);

/*
 * Probe statistics (collision monitoring: the JD ads article, section 4.3, advises watching hash
 * collisions by sampling the traffic).  While d_stats is set, every lookup_pool_fwd and
 * lookup_probe of the table adds to four int64 counters on the device, in the same launch:
 *   d_stats[0] += scans run (occurrences whose key is not the EMPTY marker and whose field is
 *                 their bag's field; every other occurrence misses without a scan),
 *   d_stats[1] += scans that read more than the key's home bucket (128 bytes, 15 slots; the home
 *                 slot h lies in bucket h / 15 and a scan stops at the key or at an empty slot),
 *   d_stats[2] += buckets read by all scans,
 *   d_stats[3]  = max(d_stats[3], the most buckets one scan read).
 * A scan's buckets are those from its home bucket to the one where it stops; the wave-cooperative
 * probe also loads the following bucket early for keys homed near their bucket's end, and such a
 * load is not counted when the home bucket ends the scan.
 * The caller zeroes the counters and reads them when it likes; d_stats = NULL stops the counting.
 * Host only (no device work); d_stats must be 8-byte aligned (EMB_EINVAL).
 */
int table_probe_stats(EmbTable* t, int64_t* d_stats);

/* Device workspace bytes sparse_adagrad_bwd and sparse_ftrl_bwd need for a batch of this shape
 * (host only). */
int bwd_workspace_bytes(const EmbTable* t, int64_t n_bags, int64_t nnz, size_t* bytes);

/*
 * Backward + update: deduplicate the rows named by d_rowref, sum each row's upstream-gradient
 * slices over its occurrences (a key repeated inside a bag counts every time), and apply sparse
 * Adagrad to each touched element:
 *     acc += g*g;   delta = lr * g / (sqrt(acc) + eps)   (the new acc)
 *     fp32 rows: w -= delta;  fp16 rows with master: master -= delta, row = fp16(master);
 *     fp16 rows without master: row = fp16(fp32(row) - delta).
 * Rows, accumulators and masters that no occurrence names are not touched.
 *   d_rowref, d_offsets, n_bags, nnz : as produced for / by lookup_pool_fwd on this flash.  The
 *                rowrefs must be the forward's for these same offsets: a rowref at or above the
 *                table's rowref space counts as a miss, but on a mixed-width table a rowref
 *                inside the space that names a narrower row than its bag's field updates
 *                elements of other rows (the arrays are padded, so nothing outside the table's
 *                state changes).  EMB_VALIDATE=1 rejects such rowrefs.
 *   d_grad     : upstream gradient, same shape and layout as the forward output, grad_dtype.
 *   d_ws       : workspace of at least bwd_workspace_bytes(n_bags, nnz) (EMB_ENOSPACE); its
 *                contents need no initialisation.
 *   d_unique   : nullable; receives the U distinct touched rowrefs in ascending order, which is
 *                ascending (table, slot) order.  On a mixed-width table whose info reports
 *                unique_by_width, the list is grouped by row width first (narrowest first,
 *                rows of 16-byte-slice counts 1, 2, 4, ... as one group each) and ascending
 *                within each group: the backward sorts by (width, rowref) so that each update
 *                piece sees one width.  Needs room for min(nnz, rows) entries.
 *   d_count    : nullable (only with d_unique); occurrence count of each unique rowref.
 *   d_n_unique : nullable; receives U (int64).
 * The gradient reduction and the update run in a fixed order, so results are reproducible run to
 * run.  Errors as for lookup_pool_fwd.
 */
int sparse_adagrad_bwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                       int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                       float lr, float eps, void* d_ws, size_t ws_bytes, uint32_t* d_unique,
                       int32_t* d_count, int64_t* d_n_unique, emb_stream_t stream);

/*
 * sparse_adagrad_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, allocation-free training loops, harnesses that forbid
 * hipMalloc).  The workspace is a static device array inside the library, 64 MiB per device,
 * held by every device the library runs on until the process ends; its address is looked up
 * once per device.  The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine, also with EMB_VALIDATE=1 (its flag word lives at the array's end).
 *   Limit: batches whose bwd_workspace_bytes exceed 64 MiB - 256 bytes get EMB_ENOSPACE before
 *          any device work (about 3M occurrences of rows up to 64 elements wide).
 *   Sharing: every call on one device uses that device's one array, and each call leaves its
 *          contents behind (the call itself needs none of them cleared).  Calls that overlap on
 *          one device -- on two streams, from two threads, or on two tables -- race; order
 *          them on one stream or with events.
 * Arguments, outputs and other errors as for sparse_adagrad_bwd; results are bit-identical to
 * it for the same inputs.
 */
int sparse_adagrad_bwd_noalloc(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                               int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                               float lr, float eps, uint32_t* d_unique, int32_t* d_count,
                               int64_t* d_n_unique, emb_stream_t stream);

/*
 * The same backward with the FTRL update in place of Adagrad, on tables created with
 * EMB_FLAG_FTRL (EMB_ESTATE otherwise).  The JD ads article's sparse-optimizer section names FTRL
 * as the Adagrad variant used for sparse features; the update is per-coordinate FTRL-Proximal
 * (McMahan et al., "Ad Click Prediction: a View from the Trenches", KDD 2013, Algorithm 1), with
 * the table's accumulator as the squared-gradient sum n, its linear state z, and w the stored
 * weight (the fp32 master when the table keeps one, else the row).  Per touched element, with g
 * the summed gradient:
 *     n' = n + g*g;   sigma = (sqrt(n') - sqrt(n)) / alpha;   z' = z + g - sigma * w;
 *     w' = 0 when |z'| <= l1, else -(z' - sign(z') * l1) / ((beta + sqrt(n')) / alpha + l2);
 * w' is stored like the Adagrad result (fp32 row; fp32 master and fp16 row = fp16(master); fp16
 * row).  A touched row whose z and g are zero gets weight 0.  alpha must be > 0 and beta, l1, l2
 * finite and >= 0 (EMB_EINVAL).  Other arguments, outputs and errors as for sparse_adagrad_bwd.
 */
int sparse_ftrl_bwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                    int64_t n_bags, int64_t nnz, const void* d_grad, int32_t grad_dtype,
                    float alpha, float beta, float l1, float l2, void* d_ws, size_t ws_bytes,
                    uint32_t* d_unique, int32_t* d_count, int64_t* d_n_unique,
                    emb_stream_t stream);

/*
 * The two halves of each call above, for callers that overlap them on two streams.  The
 * deduplication of the backward depends only on the rowrefs the probe produced, not on the
 * gradient (the Tencent PCG talk, "optimisations of each stage", deduplicates a batch's keys
 * before the update), so it can run on a second stream while the forward pools, or while dense
 * layers compute, and the update then needs only the gradient.  Each half runs the same kernels
 * as the fused call, so results are bit-identical to it.
 *
 * lookup_probe: the forward's probe alone.  Writes d_rowref (and d_slot, d_n_miss when given)
 *   exactly as lookup_pool_fwd does and pools nothing.  Arguments and errors as for
 *   lookup_pool_fwd.
 * pool_fwd: the forward's pooling alone, of the rowrefs lookup_probe wrote for the same batch
 *   (d_rowref, d_offsets, n_bags, nnz as given to it, on the same flash).  Writes d_out exactly
 *   as lookup_pool_fwd does; a rowref at or above the table's rowref space adds nothing, like
 *   EMB_ROWREF_MISS.  Arguments and errors as for lookup_pool_fwd.
 * sparse_bwd_dedup: the backward's deduplication alone: sorts the batch's (rowref, bag) pairs
 *   into d_ws (at least bwd_workspace_bytes(n_bags, nnz) bytes, EMB_ENOSPACE otherwise); a rowref
 *   at or above the table's rowref space is a miss, as in every backward.  It
 *   enables one sparse_adagrad_apply or sparse_ftrl_apply call with the same d_ws, n_bags and nnz;
 *   the workspace must not be used by anything else in between.  Arguments and errors otherwise as
 *   for sparse_adagrad_bwd.
 * sparse_adagrad_apply / sparse_ftrl_apply: the reduction and update of sparse_adagrad_bwd /
 *   sparse_ftrl_bwd from a workspace sparse_bwd_dedup prepared; order them after it on the
 *   device (same stream, or an event).  EMB_ESTATE when the last backward call on this table was
 *   not a sparse_bwd_dedup of this d_ws, n_bags and nnz, or a pass_flash or
 *   pass_writeback_touched came in between.
 *   Arguments, outputs and other errors as for the fused calls.
 */
int lookup_probe(EmbTable* t, const int64_t* d_keys, const int32_t* d_offsets, int64_t n_bags,
                 int64_t nnz, uint32_t* d_rowref, int64_t* d_slot, int64_t* d_n_miss,
                 emb_stream_t stream);
int pool_fwd(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets, int64_t n_bags,
             int64_t nnz, void* d_out, int32_t out_dtype, emb_stream_t stream);
int sparse_bwd_dedup(EmbTable* t, const uint32_t* d_rowref, const int32_t* d_offsets,
                     int64_t n_bags, int64_t nnz, void* d_ws, size_t ws_bytes,
                     emb_stream_t stream);
int sparse_adagrad_apply(EmbTable* t, int64_t n_bags, int64_t nnz, const void* d_grad,
                         int32_t grad_dtype, float lr, float eps, void* d_ws, size_t ws_bytes,
                         uint32_t* d_unique, int32_t* d_count, int64_t* d_n_unique,
                         emb_stream_t stream);
int sparse_ftrl_apply(EmbTable* t, int64_t n_bags, int64_t nnz, const void* d_grad,
                      int32_t grad_dtype, float alpha, float beta, float l1, float l2, void* d_ws,
                      size_t ws_bytes, uint32_t* d_unique, int32_t* d_count,
                      int64_t* d_n_unique, emb_stream_t stream);

/*
 * Copy rows, accumulators and masters from the device arena back into the table's host image
 * (the end-of-PASS write-back).  Synchronises `stream`.  A pageable image is filled through the
 * same bounce buffers as pass_flash (the DMA of one chunk overlaps the host copy of the other).
 */
int pass_writeback(EmbTable* t, emb_stream_t stream);

/*
 * Smallest workspace pass_writeback_touched accepts (host only).  A larger one moves the rows in
 * fewer, larger pieces; a few hundred MiB reaches the copy engine's rate.  EMB_ESTATE on a table
 * created without EMB_FLAG_TRACK_TOUCHED.
 */
int writeback_workspace_bytes(const EmbTable* t, size_t* min_bytes);

/*
 * End-of-PASS write-back of only the rows sparse_adagrad_bwd updated since pass_flash (or since
 * the last pass_writeback_touched) -- the incremental form of pass_writeback, for tables created
 * with EMB_FLAG_TRACK_TOUCHED (Tencent PCG GPU training talk: the PASS's embedding rows and
 * optimizer state are prepared off the GPU and flashed whole; the updated ones must come back
 * before the next PASS is built).  On the device the touched rows' units (rows, accumulators,
 * masters, unit index) are compacted into d_ws in pieces; each piece is copied to pinned host
 * memory and scattered into the host image while the next piece is compacted and copied.  The
 * bitmap words it reads are cleared, so a second call moves only rows updated in between.
 * Rows the call writes are also marked dirty for table_dirty_keys.
 *   d_ws, ws_bytes : device workspace, 256-byte aligned, at least writeback_workspace_bytes()
 *                    (EMB_ENOSPACE); not used by the table after the call returns.
 *   n_units_out    : nullable; receives the number of rowref units copied (rows x their units).
 * Synchronises `stream`.  EMB_ESTATE before pass_flash or without EMB_FLAG_TRACK_TOUCHED.
 */
int pass_writeback_touched(EmbTable* t, void* d_ws, size_t ws_bytes, int64_t* n_units_out,
                           emb_stream_t stream);

/*
 * Incremental export: the keys whose rows pass_writeback_touched has written into the host image
 * since the last call with clear != 0 (the pages' hourly incremental model beside the daily full
 * one, Tencent PCG GPU training talk, export paragraph; table_export then reads their state).
 * Keys come in rowref order.  keys_out may be NULL to count only; otherwise it holds cap entries
 * and EMB_ENOSPACE is returned (nothing cleared, *n_out set) when more are dirty.  Host only.
 */
int table_dirty_keys(EmbTable* t, int64_t* keys_out, int64_t cap, int64_t* n_out, int clear);

/*
 * Next-PASS rebuild: for every key of `dst` also present in `src`, copy its row, accumulator and
 * master from src's host image into dst's (the state as of src's last write-back); keys new in
 * dst keep what they were created or filled with.  The two tables must agree on field count,
 * field dims, row dtype and master (EMB_EINVAL otherwise).  Host only, threaded; it takes effect
 * at dst's next pass_flash.  n_carried (nullable) receives the number of keys copied.
 */
int table_carry_state(EmbTable* dst, const EmbTable* src, int64_t* n_carried);

/*
 * Read the host image by key: for each of the n keys, write its row (row_dtype, packed with the
 * width of the key's field), accumulator and master (each pointer nullable) -- the state as of the
 * last pass_writeback, or as built when none happened.  A key not in the table gives EMB_EINVAL.
 */
int table_export(const EmbTable* t, const int64_t* keys, int64_t n, void* rows, float* acc,
                 float* master);

/*
 * Write rows and state into the host image for keys [first, first + n) of the key list given to
 * table_create_from_prebuilt, in that list's order: rows (row_dtype), acc and master (fp32) are
 * packed like the create arrays, each key with the width of its field.  Lets a caller stream a
 * PASS's state into the image in pieces (create with rows, acc and master NULL, then fill) instead
 * of holding it twice (Tencent PCG GPU training talk, flash paragraph: the whole table is prepared
 * off the GPU and then copied in one piece).
 *   rows NULL with master given (fp16 table): rows become the fp16 round-to-nearest of master.
 *   master NULL on a table with a master copy: master becomes f32(row) when rows are given.
 *   acc NULL: the accumulator is left as it is (acc_init after create).
 * Host only; it takes effect at the next pass_flash, and must not run while a pass_flash or
 * pass_writeback copy of this table is in flight.  A range outside the key list, or master on a
 * table without one, gives EMB_EINVAL.
 */
int table_fill_state(EmbTable* t, int64_t first, int64_t n, const void* rows, const float* acc,
                     const float* master);

/*
 * FTRL linear state in the host image (tables with EMB_FLAG_FTRL, EMB_EINVAL otherwise), packed
 * like the create arrays: fill writes z for keys [first, first + n) of the create-time key list
 * (it takes effect at the next pass_flash); export reads z of n keys as of the last write-back.
 */
int table_fill_linear(EmbTable* t, int64_t first, int64_t n, const float* z);
int table_export_linear(const EmbTable* t, const int64_t* keys, int64_t n, float* z);

/* Host-side lookup of n keys: rowref (EMB_ROWREF_MISS if absent) and logical slot (-1). */
int table_key_rowref(const EmbTable* t, const int64_t* keys, int64_t n, uint32_t* rowref,
                     int64_t* slot);

/* Key of each rowref (host).  An invalid rowref gives EMB_EINVAL. */
int table_rowref_keys(const EmbTable* t, const uint32_t* rowrefs, int64_t n, int64_t* keys_out);

/*
 * Kernel timing.  With timing on, each kernel launch of this table (or only those named `only`,
 * when it is not NULL) is bracketed by HIP events on the stream it runs on.  emb_timing_read
 * synchronises those events and reports, per kernel name, the number of launches and the summed
 * milliseconds since the last read, then resets.
 *   names  : buffer of name_cap bytes receiving '\n'-separated kernel names.
 *   counts, ms : arrays of cap entries.  *n_out receives the number of kernel names.
 */
int emb_timing_enable(EmbTable* t, int enable, const char* only);
int emb_timing_read(EmbTable* t, char* names, size_t name_cap, int64_t* counts, double* ms,
                    int32_t cap, int32_t* n_out);

void table_destroy(EmbTable* t);
const char* emb_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MI355EMB_H */
