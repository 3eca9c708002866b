/*
 * chunkattn.h -- C ABI of the MI355X (gfx950) ChunkAttention decode step.
 *
 * The library keeps the KV cache of a batch of sequences as fixed-size chunks
 * in a prefix tree, so a prefix shared by several sequences is stored once
 * (prefix-aware KV cache: paperlayer.ai summary of arXiv 2402.15220v4,
 * section 3.1 and Figure 1; explainer 0h-n0.github.io/posts/paper-2402-15220,
 * "Prefix-Aware KV Cache").  One decode step (one query token per live
 * sequence, summary section 2.2) runs as a two-phase partition (summary,
 * section 3.2 and Figure 2): a chunk-first phase over chunks shared by two or
 * more sequences, a sequence-first phase over each sequence's private chunks,
 * and a log-sum-exp merge of the partial results (explainer, output
 * combination formula).  The result equals softmax(q K^T / sqrt(d)) V over
 * each sequence's stored tokens, up to rounding.
 *
 * Conventions
 *  - Every call returns an int status: CA_OK (0) or a negative CA_E_* code.
 *    ca_last_error() then holds a message; it stays valid until the next call
 *    on the same context.  No C++ exception crosses this boundary.
 *  - Device pointers are raw HIP device addresses; the library never allocates
 *    device memory and never frees caller memory.  Streams are hipStream_t
 *    passed as void* (NULL = the null stream).  Device work is enqueued on
 *    the caller's stream only and is asynchronous: errors inside kernels
 *    surface through the stream.  Host-side tables are built on the calling
 *    thread.
 *  - Chunk-table uploads copy from pinned host staging: the caller's
 *    (ca_attach_staging), or, if the caller lends none, pinned memory the
 *    library allocates at the first upload (three buffers of at least 1 MiB
 *    each, and of twice the table; a larger table reallocates one) and frees
 *    in ca_destroy.  That is the library's only allocation.
 *  - CA_E_HIP from a call that only reads the tree (ca_attend,
 *    ca_attend_phase, ca_prepare) leaves the context usable; the next step
 *    uploads the table again.  ca_insert enqueues its copies before it
 *    changes the tree, so after CA_E_HIP the tree is as it was.  After
 *    appends (ca_append, ca_append_batch, ca_decode_step) have changed the
 *    tree, a failure to enqueue their K/V writes leaves tokens in the tree
 *    that the pool does not hold: every later call that changes the tree or
 *    runs device work then returns CA_E_STATE (destroy the context).
 *  - A context is not thread-safe.  Calls that enqueue device work on
 *    different streams must be ordered by the caller.
 *  - Calls that change the tree (ca_insert, ca_append, ca_append_batch,
 *    ca_decode_step) return CA_E_STATE, changing nothing, when a device pool
 *    is attached and `stream` is capturing a HIP graph: a replay would repeat
 *    their device writes but not the host's tree update.  Capture ca_attend.
 *  - Element types: K, V, Q and the output are IEEE binary16 (fp16); the
 *    kernels accumulate in fp32.  Token ids are int32.
 *  - head_dim 128; chunk_size 64 (the chunk size of the summary's Table 3,
 *    the tuned setting), 128 (a chunk is two 64-key tiles, and the kernels
 *    read only the tiles that hold tokens) or 32 (two chunks share a 64-key
 *    tile, each read as one half); any head count >= 1.
 */
#ifndef CHUNKATTN_H
#define CHUNKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CA_OK = 0,
  CA_E_INVALID_ARG = -1,  /* bad pointer, size or shape */
  CA_E_UNSUPPORTED = -2,  /* head_dim / chunk_size / flag not supported */
  CA_E_NO_CAPACITY = -3,  /* not enough free chunk slots in the pool */
  CA_E_DUP_SEQ = -4,      /* seq_id already live */
  CA_E_UNKNOWN_SEQ = -5,  /* seq_id not live */
  CA_E_EMPTY = -6,        /* attend with no live sequence */
  CA_E_WORKSPACE = -7,    /* workspace missing or smaller than ca_workspace_bytes */
  CA_E_HIP = -8,          /* a HIP runtime call failed; message has its text */
  CA_E_NO_POOL = -9,      /* device work requested on a context without a pool */
  CA_E_STATE = -10,       /* call not allowed in the current state */
  CA_E_INTERNAL = -11
};

/* ca_create_ex flags. */
enum {
  /* Never match an existing prefix: every sequence gets its own chunks, so
   * every chunk is private and a step runs the sequence-first phase over each
   * sequence's whole block list.  This is the unshared paged layout used as
   * the comparator (PagedAttention-style block tables; summary section 4.1). */
  CA_CREATE_UNSHARED = 1,
  /* Keep the prefix tree (a shared prefix is stored once) but run no
   * chunk-first phase: every sequence streams its whole path, shared chunks
   * included, in the sequence-first phase, so a shared chunk is read once per
   * sequence that holds it.  This is the "physically shared KV without
   * two-phase partition" baseline (PagedAttn*, summary section 4.1 and
   * Table 3), used as the second comparator. */
  CA_CREATE_NO_CHUNK_FIRST = 2
};

/* ca_set_option keys. */
enum {
  CA_OPT_CF_CHUNKS_PER_TASK = 1, /* chunk refs of one shared run per chunk-first task (1..64), or
                                    0 (default): chosen per plan, 4, 8, 16, 32 or 64 (8 to 64
                                    with 32-token chunks), so that a chunk-first wave's chain of
                                    dependent tile loads stays well inside the step's streaming
                                    time (ca_stats reports the choice).  A ref is a 64-key tile
                                    (a chunk of 128 is two), or half a tile with chunks of 32. */
  CA_OPT_SF_CHUNKS_PER_TASK = 2, /* private chunk refs per sequence-first task (1..256), or 0
                                    (default): chosen per plan, the largest of 16, 8 and 4 that
                                    still gives the step about 2.5 rounds of blocks over the
                                    chip's resident block slots, 4 rounds when chunk-first
                                    blocks share the launch (there 3 instead of 4 where it
                                    makes more tasks and no one-chunk remainder; ca_stats
                                    reports the choice) */
  CA_OPT_FUSED_MERGE = 3,        /* 0: a step is a partials launch and a merge launch.
                                    1: one launch whose grid ends with merge blocks; each waits
                                    until the partials of its (sequence, head) are written (all
                                    by blocks earlier in the grid) and merges them.
                                    2 (default): one launch when the step merges at least 3072
                                    (sequence, head) pairs, else two (measured crossover on
                                    MI355X).  All give the same bits; ca_stats reports the
                                    choice for the current tree. */
  CA_OPT_MERGE_POLL_LIMIT = 4,   /* one-launch step: how many times a merge wave checks that
                                    its partials have arrived before it gives up and writes
                                    NaN for its (sequence, head); 0 (default): the library's
                                    own bound (about 0.1 s, never reached in practice).  For
                                    exercising that failure path. */
  CA_OPT_FAIL_DEVICE_OPS = 5,    /* for tests of failure handling: the next `value` device
                                    operations of the context (table uploads, kernel
                                    launches) fail with CA_E_HIP before anything is
                                    enqueued; 0 (default) turns it off.  Does not touch the
                                    chunk table. */
  CA_OPT_PREBUILD_PLAN = 6,      /* 1 (default): when ca_decode_step, or ca_append_batch over
                                    every live sequence in ascending id order, has enqueued its
                                    work and the next such append will change the table's shape
                                    (a last chunk is full or shared, or a chunk of 128 opens
                                    its second tile), the call also builds the table of that
                                    tree before it returns, while the GPU runs the work just
                                    enqueued (the summary's section 3.3: context generation
                                    on the CPU overlapped with the GPU); that next append then
                                    takes it instead of rebuilding.  ca_decode_step also
                                    copies that table into the workspace after its own step
                                    (a call in between that needs the current table uploads
                                    it again), with each sequence's last chunk at its fill
                                    before the next token: the next decode step then stores
                                    the tokens of the chunks it opens itself (row-major
                                    chunks, CA_OPT_ROW_APPENDS) and uploads nothing.
                                    0: every table is built and uploaded in the call that
                                    needs it. */
  CA_OPT_ROW_APPENDS = 7,        /* 1 (default): chunks that appends create keep their keys
                                    row-major in their slot (one K row and one V row per
                                    token and head: a decoded token is two contiguous 256-byte
                                    writes per head), and the sequence-first phase reads them
                                    by rows; an insert that makes such a chunk shared, or
                                    splits it, first rewrites it in the tile layout.  0:
                                    chunks made from now on use the tile layout (one token's
                                    K and V then land in pieces of two dozen lines). */
  CA_OPT_FAIL_AFTER_DEVICE_OPS = 8 /* for tests of failure handling: this many device
                                    operations of the context succeed before the failures
                                    of CA_OPT_FAIL_DEVICE_OPS begin (default 0). */
};

/* ca_attend_phase phases.  A step is CA_PHASE_PARTIALS (one launch holding
 * the chunk-first and the sequence-first work) followed by CA_PHASE_MERGE.
 * CA_PHASE_CHUNK_FIRST and CA_PHASE_SEQUENCE_FIRST launch only one side of
 * the partials launch, to time the two phases apart; run both (either order)
 * in place of CA_PHASE_PARTIALS. */
enum {
  CA_PHASE_CHUNK_FIRST = 1,
  CA_PHASE_SEQUENCE_FIRST = 2,
  CA_PHASE_MERGE = 3,
  CA_PHASE_PARTIALS = 4
};

typedef struct ca_ctx ca_ctx;

typedef struct ca_stats_t {
  int64_t live_sequences;
  int64_t chunks;            /* tree nodes = occupied slots */
  int64_t shared_chunks;     /* chunks referenced by >= 2 sequences */
  int64_t unique_tokens;     /* tokens stored once (sum of chunk fills) */
  int64_t attended_tokens;   /* sum over live sequences of their length */
  int64_t capacity_slots;
  int64_t free_slots;
  int64_t table_rebuilds;    /* host rebuilds of the chunk table */
  double last_rebuild_ms;    /* host time of the last rebuild */
  int64_t cf_tasks;          /* chunk-first tasks (runs of shared chunks) */
  int64_t cf_units;          /* chunk-first work units (task x 32-row block) */
  int64_t sf_tasks;          /* sequence-first tasks */
  int64_t partials;          /* partial results per head */
  int64_t cf_chunk_reads;    /* chunk tiles read per head by the chunk-first phase */
  int64_t sf_chunk_reads;    /* chunk tiles read per head by the sequence-first phase */
  int64_t unique_kv_bytes;   /* unique_tokens * 4 * heads * head_dim */
  int64_t attended_kv_bytes; /* attended_tokens * 4 * heads * head_dim */
  int64_t shared_tokens;     /* tokens held in chunks with >= 2 references */
  int64_t private_tokens;    /* tokens held in chunks with one reference */
  int64_t fill_refreshes;    /* plan updates that only refreshed chunk fills */
  int64_t table_uploads;     /* host-to-device copies of the chunk table */
  int64_t patched_appends;   /* appends whose fill counts went into the device
                                table in place (stored by the write launch or by
                                the decode step's own blocks), with no upload */
  int64_t cf_chunks_per_task; /* chunk-first group of the current plan */
  int64_t one_launch_step;    /* 1 if ca_attend runs the step as one launch */
  int64_t sf_chunks_per_task; /* sequence-first group of the current plan */
  int64_t prebuilt_plans;     /* tables built ahead, by the call before the one that needed them */
  int64_t row_chunks;         /* chunks stored row-major (made by appends, never shared) */
} ca_stats_t;

/* Bytes of one chunk slot: K and V of every head in fp16, 4 * heads *
 * chunk_size * head_dim, and of one head more when heads is a power of two
 * from 16 up (4 * (heads + 1) * chunk_size * head_dim): the pool's 64-key
 * tiles are then not a power of two apart (at 32 heads a tile would be
 * exactly 1 MiB), which streams faster on MI355X where decoding has spread a
 * batch's chunks over tiles allocated a power of two apart.  Returns 0 for
 * non-positive arguments. */
size_t ca_slot_bytes(int heads, int head_dim, int chunk_size);

/* Create a context.  heads >= 1; head_dim must be 128 and chunk_size 1..64 or
 * 128 (else CA_E_UNSUPPORTED); a device pool (ca_attach_pool) further needs
 * chunk_size 32, 64 or 128, other sizes serve host-only contexts (tree and
 * tables).  Scale is 1/sqrt(head_dim) computed in fp32.
 * *out receives the context; the caller owns it and frees it with
 * ca_destroy. */
int ca_create(int heads, int head_dim, int chunk_size, ca_ctx** out);
int ca_create_ex(int heads, int head_dim, int chunk_size, int flags, ca_ctx** out);
void ca_destroy(ca_ctx* ctx);

/* Lend the context a device pool of capacity_slots slots, each
 * ca_slot_bytes() long, 256-byte aligned.  Layout inside the pool: 64-key
 * tiles, tile-major (ca_slot_bytes(heads, 128, 64) bytes apart), then head,
 * then K tile and V tile of 64 x 128 fp16 each (tile element order is private
 * to the library; the extra head's room at the end of a tile is never
 * touched); a slot of 64 tokens is one tile, of 128 two, and two slots of 32
 * share one.  With chunk_size 32 the
 * slots are used in pairs: an odd last slot is left out of the capacity.
 * dev may be NULL: the context then manages the tree and tables on the host
 * only and every call that needs the device returns CA_E_NO_POOL.  A device
 * pool needs chunk_size 32, 64 or 128 (CA_E_UNSUPPORTED otherwise).  Allowed
 * only while no sequence is live (CA_E_STATE otherwise).  The caller keeps
 * the memory alive and owns it. */
int ca_attach_pool(ca_ctx* ctx, void* dev, int64_t capacity_slots);

/* Device workspace needed by ca_attend for the current tree: the chunk table
 * and the partial results.  Changes after insert/append/remove. */
int ca_workspace_bytes(ca_ctx* ctx, size_t* out);

/* Lend a device workspace (256-byte aligned).  The caller owns it; it must
 * stay alive while enqueued steps use it, and the library keeps the chunk
 * table there from one call to the next: the caller does not write into it
 * while it is attached.  Attaching another buffer (or NULL) makes the next
 * step upload the table again, also if the first buffer is attached again
 * later. */
int ca_attach_workspace(ca_ctx* ctx, void* dev, size_t bytes);

/* Pinned host staging for chunk-table uploads (the plan is cached and copied
 * to the device only after the tree changed shape: summary section 3.3):
 * ca_staging_bytes gives the size the current tree needs (three parts, each
 * one table, so an upload never waits for the last two).  ca_attach_staging
 * lends `bytes` of pinned host memory (hipHostMalloc, or a pinned torch
 * tensor), 256-byte aligned; the caller owns it and keeps it alive until it
 * attaches another or destroys the context.  It first waits for copies still
 * reading earlier staging, so that memory may be freed once it returns.
 * host NULL: back to library-owned staging.  A step whose table must be
 * uploaded and does not fit the attached staging returns CA_E_WORKSPACE.
 * The first pinned host-to-device copy of more than 16 KiB in a process
 * costs about 6 ms in the HIP runtime on MI355X, once; a caller whose decode
 * loop must not meet it makes such a copy at start-up (the Python binding
 * does when it allocates a pool). */
int ca_staging_bytes(ca_ctx* ctx, size_t* out);
int ca_attach_staging(ca_ctx* ctx, void* host, size_t bytes);

/* Tuning knobs (CA_OPT_*).  Takes effect at the next table rebuild. */
int ca_set_option(ca_ctx* ctx, int option, int value);

/* Add a sequence (prefix detection at arrival: summary section 3.1; explainer
 * "dynamic prefix detection").  tokens: n >= 1 host int32 ids.  k_dev, v_dev:
 * fp16 [n][heads][head_dim] device tensors holding the keys/values of the
 * whole sequence; only the rows after the longest stored prefix are copied,
 * stream-ordered on `stream`, so the caller keeps them alive until the stream
 * passes this call.  A divergence inside a stored chunk splits that chunk.
 * *n_matched (may be NULL) receives the number of leading tokens already
 * stored.  Errors: CA_E_DUP_SEQ, CA_E_INVALID_ARG (n < 1, NULL pointers),
 * CA_E_NO_CAPACITY, CA_E_HIP (the copy could not be enqueued).  A failed call
 * changes nothing: the copies are enqueued before the tree changes.  One
 * exception is internal: chunks stored row-major (CA_OPT_ROW_APPENDS) that
 * the insert shares or splits are first rewritten as tiles in a launch of
 * their own; if that launch went out and a later one fails, they stay tiles
 * (same tokens, same K/V, the same results). */
int ca_insert(ca_ctx* ctx, int64_t seq_id, const int32_t* tokens, int32_t n,
              const void* k_dev, const void* v_dev, void* stream, int32_t* n_matched);

/* Append n >= 1 decoded tokens to a live sequence (summary section 3.1:
 * decoding appends to leaf chunks or grows new chunks).  Writes into the
 * sequence's last chunk only if that chunk is private and not full, else
 * grows new private chunks.  k_dev, v_dev: fp16 [n][heads][head_dim].
 * An append that lands wholly in place keeps the table's shape, as in
 * ca_append_batch (fill counts stored on the device by the write launch).
 * Errors: CA_E_UNKNOWN_SEQ, CA_E_INVALID_ARG, CA_E_NO_CAPACITY (nothing
 * changes); CA_E_HIP (the tree changed but the K/V could not be written: the
 * context is unusable, see the conventions above). */
int ca_append(ca_ctx* ctx, int64_t seq_id, const int32_t* tokens, int32_t n,
              const void* k_dev, const void* v_dev, void* stream);

/* One decode token for each of n >= 1 live sequences: token tokens[j] with
 * K/V row j of k_dev, v_dev (fp16 [n][heads][head_dim]) goes to seq_ids[j].
 * Same placement rules as ca_append; all KV writes go out in batched
 * launches.  When every append lands in place (a private, non-full last
 * chunk), the cached chunk table keeps its shape (it is rebuilt when a chunk
 * fills up or a sequence joins or leaves: summary section 3.3); if the table
 * is then already on the device, the write launch also stores the new fill
 * counts into the workspace copy, so the next step uploads nothing.  Those
 * stores are ordered on `stream` like the K/V writes: enqueue appends and
 * steps of one context on one stream (or order them with events).
 * Errors: CA_E_UNKNOWN_SEQ, CA_E_INVALID_ARG (an id repeated in the batch),
 * CA_E_NO_CAPACITY; all are detected before anything changes.  CA_E_HIP: as
 * for ca_append. */
int ca_append_batch(ca_ctx* ctx, int32_t n, const int64_t* seq_ids, const int32_t* tokens,
                    const void* k_dev, const void* v_dev, void* stream);

/* Remove a finished sequence: every chunk on its path loses one reference and
 * chunks left without references return their slots (explainer, "dynamic
 * prefix detection").  Pure host bookkeeping; steps already enqueued still
 * see the old data, but slots freed here may be overwritten by the next
 * insert/append, so order those after the enqueued steps.
 * Error: CA_E_UNKNOWN_SEQ. */
int ca_remove(ca_ctx* ctx, int64_t seq_id);

/* One decode step.  q_dev: fp16 [n_live][heads][head_dim]; out_dev: fp16
 * [n_live][heads][head_dim]; row r belongs to the r-th live sequence in
 * ascending seq_id order (ca_list_sequences).  Uploads the chunk table if the
 * tree changed since the last upload, then enqueues the step on `stream`: a
 * partials launch (chunk-first and sequence-first blocks in one grid) and a
 * merge launch, or one launch whose last blocks merge (CA_OPT_FUSED_MERGE;
 * by default one launch from 3072 (sequence, head) pairs up).
 * The merge folds the partials in a
 * fixed order, so the result does not depend on block timing.  Steps of one
 * context must not overlap (they share the workspace and its arrival
 * counters).  No host synchronisation.
 * HIP graphs: a step whose table is already on the device (a step or
 * ca_prepare ran since the tree last changed shape) enqueues kernel launches
 * only, and can be captured; the graph replays the step with the pointers
 * and the tree shape of the capture (appends that only grow chunks in place
 * keep it valid: they store the fill counts on the device).  A step that
 * would upload the table while its stream is capturing returns CA_E_STATE.
 * Errors: CA_E_EMPTY, CA_E_WORKSPACE, CA_E_NO_POOL, CA_E_HIP, CA_E_STATE. */
int ca_attend(ca_ctx* ctx, const void* q_dev, void* out_dev, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, serving
 * loops or harnesses that forbid allocation): ca_attend with the step's
 * workspace (chunk table, arrival counters, partial results) in a static
 * device array of the library instead of the caller's workspace.  The array
 * holds 16 MiB (CA_NOALLOC_SCRATCH_BYTES); a step whose ca_workspace_bytes is
 * larger returns CA_E_WORKSPACE.  There is one array per device, in the
 * library's code object, held until the process ends; the current device
 * (hipGetDevice) is the one used, and must hold the pool, q, out and the
 * stream.  Its address is looked up (hipGetSymbolAddress) at the first call
 * on each device.  The call allocates nothing: when the table must be
 * uploaded it copies from staging the caller attached (ca_attach_staging;
 * CA_E_STATE without), and the arrival counters start at zero with each
 * upload.  Every context on a device shares that device's array: a context
 * whose table another context has replaced there uploads it again, so calls
 * of different contexts can alternate, but calls that overlap on one device
 * (different streams or threads, without ordering) race.  Same arguments,
 * results and other errors as ca_attend. */
#define CA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int ca_attend_noalloc(ca_ctx* ctx, const void* q_dev, void* out_dev, void* stream);

/* One decode step of the whole batch (summary section 3.1: decoding appends
 * to leaf chunks; section 2.2: one query token per sequence): token tokens[r]
 * with K/V row r of k_dev, v_dev (fp16 [n_live][heads][head_dim]) is appended
 * to the r-th live sequence in ascending seq_id order, then every sequence
 * attends with row r of q_dev; out_dev as for ca_attend.  The result, the
 * tree and the stored K/V are those of ca_append_batch over all live
 * sequences followed by ca_attend.  When every token grows its sequence's
 * private last chunk in place (63 of every 64 steps of a batch that decodes
 * in lockstep), no separate write launch runs: the block of the step that
 * reads that chunk writes the token into the pool, uses it, and stores the
 * grown fill count into the device table; otherwise the writes go out first,
 * as in ca_append_batch.  The caller keeps k_dev and v_dev alive until the
 * stream passes the step.  Errors: those of ca_append_batch, and
 * CA_E_INVALID_ARG for a NULL q_dev or out_dev, leave everything unchanged;
 * CA_E_WORKSPACE (a step that grew new chunks can need a larger workspace)
 * and CA_E_UNSUPPORTED (a step beyond the kernels' index range) come after
 * the tokens were stored: attach a workspace of ca_workspace_bytes and finish
 * with ca_attend.  CA_E_HIP from the step's launch also comes after the
 * tokens were stored (by a write launch in its place); if they cannot be
 * stored either, the context is unusable (see the conventions above). */
int ca_decode_step(ca_ctx* ctx, const int32_t* tokens, const void* k_dev, const void* v_dev,
                   const void* q_dev, void* out_dev, void* stream);

/* The same step split into its launches, for measuring each kernel: call
 * ca_prepare once (uploads the table if needed), then ca_attend_phase with
 * CA_PHASE_PARTIALS (or CA_PHASE_CHUNK_FIRST and CA_PHASE_SEQUENCE_FIRST)
 * and then CA_PHASE_MERGE, on one stream.  Same arguments and errors as
 * ca_attend, plus CA_E_INVALID_ARG for an unknown phase. */
int ca_prepare(ca_ctx* ctx, void* stream);
int ca_attend_phase(ca_ctx* ctx, int phase, const void* q_dev, void* out_dev, void* stream);

/* Live sequence ids in ascending order (the row order of q and out).  Writes
 * min(count, cap) ids and returns the count (>= 0) or an error code. */
int ca_list_sequences(ca_ctx* ctx, int64_t* ids, int cap);

/* The chunk table in DFS pre-order: 7 int32 per row (node_id, parent_row,
 * token_start, n_tokens, seq_begin, seq_end, slot), parent_row -1 under the
 * root, [seq_begin, seq_end) the node's contiguous range in the DFS order of
 * sequences, which is written to dfs_seq_order.  Sizes go to *n_rows and
 * *n_seqs; nothing is written if a capacity is too small (CA_E_INVALID_ARG).
 * Pointers may be NULL with capacity 0 to query sizes. */
int ca_export_table(ca_ctx* ctx, int32_t* rows, int cap_rows, int64_t* dfs_seq_order,
                    int cap_seqs, int* n_rows, int* n_seqs);

/* The device table of the current plan as it is uploaded (records, chunk
 * refs, row and partial lists, zeroed arrival counters; its layout is
 * private to the library): *bytes receives its size; buf may be NULL with
 * cap 0 to query it.  For bit-exact comparison of plans in tests.
 * CA_E_INVALID_ARG if cap is too small (nothing written). */
int ca_export_plan(ca_ctx* ctx, void* buf, size_t cap, size_t* bytes);

int ca_stats(ca_ctx* ctx, ca_stats_t* out);
const char* ca_last_error(ca_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKATTN_H */
