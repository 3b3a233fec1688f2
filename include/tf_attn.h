/*
 * tf_attn.h -- C ABI of the shared-round attention library (MI355X, gfx950).
 *
 * One launch serves the query rows of many concurrent streams.  A segment
 * table in device memory names, for each stream, where its K/V cache lives,
 * which packed query rows are its own and how many keys it has; the stream's
 * K/V sits in pages of a shared pool, in a wrapping ring, or in one
 * contiguous buffer.  tf_attn_rows writes split-K partials (or the output
 * directly when there is one split), tf_attn_merge combines the partials with
 * an online-softmax merge, and tf_argmax picks each row's first largest
 * logit and flags rows that hold a nonfinite one.
 *
 * Sources (the pages this library is built from):
 *  - TensorFold PR #1503, "lfm2_moe CUDA: attention pages from the shared KV
 *    pool, and the prompt cache": a per-stream table (where the stream's
 *    cache is, which packed rows are its own, how many keys it holds) that
 *    lets one launch per layer serve every stream
 *    (the shared-rounds commit); reads through a slot's page table and the
 *    refusal of rows past a slot's pages (the pool-leasing commit); the GPU
 *    argmax with its tie and nonfinite rules (the lfm2_argmax commit).
 *  - TensorFold PR #1653, "spark25 CUDA: the full layers' caches in pages of
 *    the core pool ...": paged decode part/merge kernels, prompt rows read
 *    through the slot's page-table row in pages of whole 32-key tiles, with
 *    the page id looked up once per chunk instead of once per key.
 *  - TensorFold PR #1562, "Qwen3.6 MTP drafter on CUDA: draft a shared
 *    round's streams together": one rows kernel for all streams, each packed
 *    row finding its ring and slot count through a table, bit-equal to a
 *    launch per stream;
 *    ring slots folded in groups with the next group in flight; the tree
 *    attention kernel beside it, checked to give the same drafts as chains.
 *  - TensorFold PR #1394, "lfm2: a cheaper DSpark hold": the drafter's block
 *    attention, the target's kernels with a FULL flag under which every row
 *    of a block sees the block's whole key range.
 *
 * Conventions
 *  - All tensors are bf16 (stored as 16-bit patterns), accumulation is fp32,
 *    outputs are rounded to bf16 with round-to-nearest-even.
 *  - Ownership: the caller allocates every buffer (device memory unless
 *    marked "host").  The library allocates nothing, keeps no state between
 *    calls, never synchronises the stream and launches only on the stream it
 *    is given.  Calls are thread-safe.
 *  - Errors: scalar arguments are checked on the host before anything is
 *    launched; a bad call returns a negative TF_E_* code and launches
 *    nothing.  Segment contents live in device memory and are checked by the
 *    kernels: an invalid segment sets bits in the optional device error word
 *    (TF_ERR_*), and its rows are written as NaN when its row range and
 *    partial range are themselves valid (otherwise nothing is written for
 *    it).  tf_check_segments runs the same checks on a host copy.
 *  - NaN rule: keys outside a row's visible range are never used.  If any
 *    visible score of a (row, head) is NaN or +-Inf, every output element of
 *    that (row, head) is NaN.  Otherwise an output element whose value is not
 *    finite is written as NaN (0x7FC0).
 */
#ifndef TF_ATTN_H
#define TF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* How a segment's K/V is stored (one kind per launch). */
typedef enum tf_kv_kind {
    TF_KV_CONTIG = 0, /* per stream: k, v -> [n_kv_heads][capacity][head_dim]               */
    TF_KV_PAGED = 1,  /* shared pool: k, v -> [pool_pages][n_kv_heads][page_size][head_dim]; */
                      /* logical key j is row j % page_size of pool page pages[j / page_size] */
    TF_KV_RING = 2    /* per stream: k, v -> [n_kv_heads][capacity][head_dim], capacity = ring */
                      /* slots; logical key j is in slot (first + j) mod capacity            */
} tf_kv_kind;

/* Which keys a row sees (one mask per launch).  Row r of an n-row segment: */
typedef enum tf_mask {
    TF_MASK_CAUSAL = 0, /* keys [0, key_count - n + r + 1): up to and including its own     */
    TF_MASK_FULL = 1,   /* keys [0, key_count): a non-causal block (PR #1394, FULL flag)      */
    TF_MASK_TREE = 2    /* keys [0, key_count - n), its own key key_count - n + r, and key
                           key_count - n + j for every bit j set in tree[row_offset + r];
                           needs n <= 64 (PR #1562, tree attention)                         */
} tf_mask;

/* Return codes. */
enum {
    TF_OK = 0,
    TF_E_INVALID = -1,     /* null pointer, negative count, n_q_heads % n_kv_heads != 0, ...     */
    TF_E_UNSUPPORTED = -2, /* head_dim not 64/128/256, page_size not a power of two in
                              [32, 1024], split_keys not a multiple of 32                        */
    TF_E_PAST_PAGES = -3,  /* a segment holds more keys than its pages / ring / buffer (host check) */
    TF_E_WORKSPACE = -4,   /* partials or argmax workspace missing or too small                  */
    TF_E_LAUNCH = -5       /* the HIP runtime refused the launch                                 */
};

/* Bits the kernels OR into the optional device error word. */
enum {
    TF_ERR_PAST_PAGES = 1, /* key_count > capacity (x page_size for PAGED)                       */
    TF_ERR_BAD_PAGE = 2,   /* a page id outside [0, pool_pages)                                  */
    TF_ERR_BAD_ROWS = 4,   /* n_rows < 1, n_rows > key_count, rows outside [0, total_rows), or
                              n_rows > 64 under TF_MASK_TREE                                   */
    TF_ERR_BAD_RING = 8,   /* ring first outside [0, capacity)                                   */
    TF_ERR_PARTIALS = 16,  /* the segment's partial records fall outside the workspace           */
    TF_ERR_BAD_LAYER = 32, /* tf_state_*: a layer's pointer is null or not 16-byte aligned       */
    TF_ERR_HINTS = 64,     /* n_rows > max_rows or key_count > max_keys: the launch's grid does not
                              cover the segment; the rows it covers are written as NaN, the rest
                              of the segment's rows and splits are not written                   */
    TF_ERR_STORAGE = 128   /* CONTIG / RING: one kv head's run of the buffer, capacity * head_dim
                              * 2 bytes, is 4 GiB or more (beyond the kernels' 32-bit offsets)  */
};

/*
 * One stream's span of a shared launch.  The table (an array of these)
 * lives in device memory.  48 bytes, 8-byte aligned.
 *
 * Row r (0-based) of an n-row segment is packed query row row_offset + r.
 * The segment's new rows are its newest keys: row r's own key is logical key
 * key_count - n_rows + r.  Which keys it sees is the launch's tf_mask
 * (causal count: [0, key_count - n_rows + r + 1)).
 */
typedef struct tf_segment {
    const void *k;          /* bf16 K storage (see tf_kv_kind)                                 */
    const void *v;          /* bf16 V storage, same layout as k                                */
    const int32_t *pages;   /* PAGED: logical page -> pool page id; NULL otherwise             */
    int32_t capacity;       /* PAGED: entries of pages[]; RING: slots; CONTIG: keys allocated  */
    int32_t first;          /* RING: slot that holds logical key 0; 0 otherwise                */
    int32_t row_offset;     /* first packed query row of this segment                          */
    int32_t n_rows;         /* 1 <= n_rows <= key_count                                        */
    int32_t key_count;      /* keys of the stream, the segment's new rows included             */
    int32_t partial_offset; /* first partial record of this segment (see tf_plan_partials)     */
} tf_segment;

/*
 * Arguments of tf_attn_rows / tf_attn_merge.  Host memory; the pointers in
 * it are device pointers.
 *
 * Partial records: record index
 *     partial_offset + (r * n_q_heads + h) * n_splits + t,
 * with n_splits = ceil(key_count / split_keys) of the record's segment,
 * holds split t (the keys in [t * split_keys, (t + 1) * split_keys) that
 * row r sees) of row r, query head h.  A record is head_dim + 4 floats:
 *     [0] m  : reference for the split's scaled scores (natural-log units):
 *              one of them, at most 8 ln 2 below their max (so no weight
 *              exceeds 2^8); -inf if the split is empty, NaN if it saw a
 *              nonfinite score;
 *     [1] l  : sum over the split of exp(score - m);
 *     [2..3] : unused;
 *     [4..]  : o[head_dim] = sum over the split of exp(score - m) * v.
 * Any m gives the same softmax: m + ln(l) (the split's log-sum-exp) and o / l
 * are what a record fixes.
 */
typedef struct tf_attn_args {
    int32_t kind;             /* tf_kv_kind                                                  */
    int32_t n_segments;       /* >= 0                                                        */
    int32_t total_rows;       /* packed query rows of q and out                              */
    int32_t max_rows;         /* >= every segment's n_rows (grid sizing only)                */
    int32_t max_keys;         /* >= every segment's key_count (grid sizing only)             */
    int32_t min_rows;         /* <= every segment's n_rows, or 0 if unknown (kernel choice
                                 only: lets a launch whose segments all have many query
                                 vectors skip the decode kernel)                             */
    int32_t n_q_heads;        /* Hq                                                          */
    int32_t n_kv_heads;       /* Hkv; query head h reads kv head h / (Hq / Hkv)              */
    int32_t head_dim;         /* 64, 128 or 256                                              */
    int32_t page_size;        /* PAGED: keys per page (power of two, 32..1024); else ignored */
    int32_t pool_pages;       /* PAGED: pages in the pool (page ids are checked against it)  */
    int32_t split_keys;       /* keys per partial (multiple of 32), or 0 = one split: then
                                 tf_attn_rows writes out directly and needs no partials      */
    float scale;              /* score = scale * (q . k), finite and > 0, normally 1/sqrt(D) */
    int32_t mask;             /* tf_mask                                                     */
    const tf_segment *segs;   /* device: n_segments entries                                  */
    const uint64_t *tree;     /* TF_MASK_TREE: device, one ancestor mask per packed row (bit j
                                 = the segment's row j is on the row's path to its root);
                                 ignored otherwise                                           */
    const void *q;            /* device bf16 [total_rows][n_q_heads][head_dim]               */
    void *out;                /* device bf16 [total_rows][n_q_heads][head_dim]               */
    float *partials;          /* device fp32 records (split_keys > 0)                        */
    size_t partials_bytes;    /* size of partials                                            */
    int32_t *err;             /* device int32 error word (TF_ERR_* bits ORed in), or NULL    */
} tf_attn_args;

/*
 * tf_attn_rows: attention of every segment's rows over its own keys
 * (TensorFold PR #1503, the shared-rounds commit: one launch per layer serves
 * every stream's rows from the segment table, partials held apart per
 * stream; PR #1653, the paged decode part kernel and the paged prompt rows
 * read through the page table with the page id looked up once per tile;
 * PR #1562, one rows kernel for all streams of a round, bit-equal to a
 * launch per stream, ring slots read with the next group in flight).
 * With split_keys > 0 writes one partial record per (row, head, split) of
 * every segment; with split_keys == 0 writes out.  Each (row, head)'s
 * result depends only on its own segment: a batched launch is bit-equal to
 * one launch per segment, and to the same keys stored as pages, a ring or a
 * contiguous buffer.  Returns TF_OK or a TF_E_* code (nothing launched).
 */
int tf_attn_rows(const tf_attn_args *a, hipStream_t stream);

/*
 * tf_attn_merge: combine each (row, head)'s partial records into out:
 *     M = max m_t, L = sum l_t e^(m_t - M), out = sum o_t e^(m_t - M) / L,
 * the o sum taken in split order t = 0, 1, ... and L by a fixed reduction
 * tree over t; a NaN record makes the output NaN.
 * Needs split_keys > 0 and the partials tf_attn_rows wrote with the same
 * arguments (TensorFold PR #1653: the paged decode merge, with nonfinite
 * heads kept off the fast path).
 */
int tf_attn_merge(const tf_attn_args *a, hipStream_t stream);

/*
 * tf_attn_static: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same as tf_attn_rows followed, when split_keys > 0, by tf_attn_merge,
 * except that the split partials live in a device array the library owns
 * (TF_STATIC_PARTIALS_BYTES bytes on each device it runs on, held until the
 * process ends) instead of a caller workspace.  a->partials must be NULL
 * (TF_E_INVALID otherwise); a->partials_bytes is the size tf_plan_partials
 * returned for the table and must be at most TF_STATIC_PARTIALS_BYTES
 * (TF_E_WORKSPACE otherwise).  The call allocates nothing.  Every call on a
 * device shares that device's array, which keeps the last call's records:
 * calls that overlap on one GPU (other streams, other threads) race.  Same
 * return codes and device error bits as tf_attn_rows / tf_attn_merge;
 * TF_E_LAUNCH also if the array's address cannot be obtained.
 */
#define TF_STATIC_PARTIALS_BYTES ((size_t)16 << 20)
int tf_attn_static(const tf_attn_args *a, hipStream_t stream);

/*
 * tf_argmax: for each row of bf16 logits (row i starts at logits + i *
 * row_stride elements; the first `vocab` are read) writes ids[i], the lowest
 * id among the largest values, and flags[i] = 1 if any of the row's logits is
 * NaN or +-Inf (else 0).  NaN ranks as -inf for the id, +0.0 equals -0.0
 * (TensorFold PR #1503, the lfm2_argmax commit and the router note).  One
 * launch.  workspace: device memory of at least tf_argmax_workspace_bytes(
 * n_rows, vocab) bytes (16 per row, 8-byte aligned) that holds zeros before
 * its first use; every call leaves it all zero again, so one zeroed
 * allocation serves every later call.  Calls that share a workspace must not
 * overlap.  Returns TF_E_INVALID for null pointers, vocab < 1, row_stride <
 * vocab; TF_E_WORKSPACE if the workspace is too small; TF_E_UNSUPPORTED for a
 * vocabulary of more than 65535 * 16384 logits.
 */
int tf_argmax(const void *logits, int32_t n_rows, int32_t vocab, int64_t row_stride,
              int32_t *ids, uint8_t *flags, void *workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * KV append (TensorFold PR #1653, the kernel that puts a chunk's K/V rows
 * into the core pool's pages; PR #1562, the drafter's ring rows written at
 * the ring's head with the wrap).
 *
 * tf_kv_put writes every segment's new keys and values into its storage.
 * The new keys of a segment are its last n_rows logical keys,
 * [key_count - n_rows, key_count) -- the keys tf_attn_rows gives the
 * segment's rows (each row sees itself) -- so a round is: update the table,
 * tf_kv_put, tf_attn_rows.  Row r of the segment comes from packed row
 * row_offset + r of k_new / v_new, bf16 [total_rows][n_kv_heads][head_dim]
 * (laid out like q).  Logical key j goes to
 *     PAGED:  page pages[j / page_size], offset j % page_size;
 *     RING:   slot (first + j) mod capacity;
 *     CONTIG: row j;
 * in the segment's k / v storage (which must be writable; layout as in
 * tf_kv_kind).  No other storage byte is written.  Segments must not
 * write the same storage row.  Per-segment problems set TF_ERR_* bits in
 * *err and skip that segment (BAD_ROWS, PAST_PAGES, BAD_RING) or that
 * row (BAD_PAGE); nothing is written out of bounds.  Returns TF_OK,
 * TF_E_INVALID or TF_E_UNSUPPORTED (nothing launched).
 */
typedef struct tf_put_args {
    int32_t kind;             /* tf_kv_kind                                                  */
    int32_t n_segments;       /* >= 0                                                        */
    int32_t total_rows;       /* packed rows of k_new and v_new                              */
    int32_t max_rows;         /* >= every segment's n_rows (grid sizing only)                */
    int32_t n_kv_heads;       /* Hkv                                                         */
    int32_t head_dim;         /* 64, 128 or 256                                              */
    int32_t page_size;        /* PAGED: keys per page (power of two, 32..1024)               */
    int32_t pool_pages;       /* PAGED: pages in the pool                                    */
    const tf_segment *segs;   /* device: n_segments entries (partial_offset unused)          */
    const void *k_new;        /* device bf16 [total_rows][n_kv_heads][head_dim]              */
    const void *v_new;        /* device bf16, same layout                                    */
    int32_t *err;             /* device int32 error word, or NULL                            */
} tf_put_args;

int tf_kv_put(const tf_put_args *a, hipStream_t stream);

/*
 * Kept state copy (TensorFold PR #1503, the prompt-cache commit of the
 * lfm2_moe pool: a kept state holds the K and V rows of positions [0, at)
 * for every attention layer, moved as runs of whole pages plus the last page's
 * leading rows, and is restored into the pages of the stream that resumes
 * it).
 *
 * tf_state_save copies positions [0, at) of every layer's K and V from the
 * stream's pool pages into the layer's state buffers; tf_state_restore copies
 * them back into another page list (the new stream's pages).  Pool pages are
 * [pool_pages][n_kv_heads][page_size][head_dim] bf16 (the PAGED layout of
 * tf_kv_kind); a state buffer has the same shape with the stream's logical
 * pages in order, [ceil(at / page_size)][n_kv_heads][page_size][head_dim]:
 * state page i holds the rows of logical page i, so whole pages copy as
 * units and the last page copies only its first at - (pages - 1) * page_size
 * rows.  Rows at or past `at` are never written: not in the state (save),
 * not in the pool (restore).  Page ids outside [0, pool_pages) set
 * TF_ERR_BAD_PAGE and that page is skipped; a null or misaligned layer
 * pointer sets TF_ERR_BAD_LAYER and that layer is skipped.  One launch
 * covers every layer.  Returns TF_OK, TF_E_INVALID, TF_E_UNSUPPORTED or
 * TF_E_PAST_PAGES (at > n_pages * page_size), nothing launched on an error.
 */
typedef struct tf_state_layer {
    void *pool_k;             /* device bf16 pool of the layer's keys                        */
    void *pool_v;             /* device bf16 pool of the layer's values                      */
    void *state_k;            /* device bf16 state buffer of the layer's keys                */
    void *state_v;            /* device bf16 state buffer of the layer's values              */
} tf_state_layer;

typedef struct tf_state_args {
    int32_t n_layers;         /* >= 0                                                        */
    int32_t n_kv_heads;       /* >= 1                                                        */
    int32_t head_dim;         /* 64, 128 or 256                                              */
    int32_t page_size;        /* positions per page (power of two, 32..1024)                 */
    int32_t pool_pages;       /* pages in each pool (page ids are checked against it)        */
    int32_t at;               /* positions [0, at) are copied; >= 0                          */
    int32_t n_pages;          /* entries of pages[]                                          */
    const int32_t *pages;     /* device: the stream's logical page -> pool page id           */
    const tf_state_layer *layers; /* device: n_layers entries, pointers 16-byte aligned      */
    int32_t *err;             /* device int32 error word, or NULL                            */
} tf_state_args;

int tf_state_save(const tf_state_args *a, hipStream_t stream);
int tf_state_restore(const tf_state_args *a, hipStream_t stream);

/* Workspace bytes tf_argmax needs for n_rows rows of vocab logits (zeroed once by the caller). */
size_t tf_argmax_workspace_bytes(int32_t n_rows, int32_t vocab);

/*
 * tf_plan_partials (host): assign each segment's partial_offset in the
 * host table (segments laid out in order) and return the workspace size in
 * bytes for split_keys > 0 (TensorFold PR #1503, the shared-rounds commit:
 * the caller owns the scratch the partials live in, one range per stream).  Reads n_rows and key_count of each host
 * segment.  Returns TF_E_INVALID on bad counts, TF_E_UNSUPPORTED on a bad
 * split_keys or head_dim.
 */
int tf_plan_partials(tf_segment *host_segs, int32_t n_segments, int32_t n_q_heads,
                     int32_t head_dim, int32_t split_keys, size_t *partials_bytes);

/*
 * tf_check_segments (host): the kernels' per-segment checks on a host copy
 * of the table, plus the ones only the host can do (rows of different
 * segments must not overlap; the pages pointer of a PAGED segment must be
 * non-null).  max_rows / max_keys must bound the table (the kernels flag a
 * segment past them with TF_ERR_HINTS).  Returns TF_OK, TF_E_PAST_PAGES (a
 * segment holds more keys than its storage), TF_E_WORKSPACE (partial records
 * outside the workspace), TF_E_UNSUPPORTED (a CONTIG / RING kv-head run of 4
 * GiB or more, TF_ERR_STORAGE on the device) or TF_E_INVALID.  Page ids live
 * in device memory and are checked by the kernels only.  The checks follow
 * TensorFold PR #1503 (the pool-leasing commit: a slot's rows are refused past
 * its pages) and the table fields of its shared-rounds commit.
 */
int tf_check_segments(const tf_attn_args *a, const tf_segment *host_segs);

/* Static description of a return code. */
const char *tf_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TF_ATTN_H */
