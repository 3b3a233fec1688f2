// C ABI entry points (include/tf_attn.h): host-side checks, partial planning
// and kernel dispatch.  Nothing here allocates or synchronises.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <vector>

#include "device.hpp"
#include "tf_attn.h"

namespace tfa {
hipError_t launch_rows_valu(const RowsParams &p, int head_dim, int kind, hipStream_t st);
hipError_t launch_rows_mfma(const RowsParams &p, int head_dim, int kind, int max_q, hipStream_t st);
int mfma_query_tile(int head_dim, int64_t max_q);
hipError_t launch_merge(const RowsParams &p, int head_dim, int max_rows, hipStream_t st);
hipError_t launch_argmax(const uint16_t *logits, int n_rows, int vocab, int64_t row_stride,
                         int32_t *ids, uint8_t *flags, void *workspace, hipStream_t st);
int argmax_chunk_count(int vocab);
size_t argmax_slot_bytes();
}  // namespace tfa

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t record_bytes(int head_dim) { return (int64_t)(head_dim + 4) * (int64_t)sizeof(float); }

int n_splits_of(int key_count, int split_keys)
{
    return split_keys > 0 ? (key_count + split_keys - 1) / split_keys : 1;
}

// Checks shared by tf_attn_rows, tf_attn_merge and tf_check_segments.
int check_args(const tf_attn_args *a, bool need_partials)
{
    if (a == nullptr)
        return TF_E_INVALID;
    if (a->kind != TF_KV_CONTIG && a->kind != TF_KV_PAGED && a->kind != TF_KV_RING)
        return TF_E_INVALID;
    if (a->n_segments < 0 || a->total_rows < 0 || a->max_rows < 0 || a->max_keys < 0 ||
        a->min_rows < 0 || a->min_rows > a->max_rows)
        return TF_E_INVALID;
    if (a->n_q_heads < 1 || a->n_kv_heads < 1 || a->n_q_heads % a->n_kv_heads != 0)
        return TF_E_INVALID;
    if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
        return TF_E_UNSUPPORTED;
    if (a->kind == TF_KV_PAGED) {
        const int ps = a->page_size;
        if (ps < 32 || ps > 1024 || (ps & (ps - 1)) != 0)
            return TF_E_UNSUPPORTED;
        if (a->pool_pages < 1)
            return TF_E_INVALID;
    }
    if (a->split_keys < 0 || a->split_keys % 32 != 0)
        return TF_E_UNSUPPORTED;
    if (!(a->scale > 0.0f && a->scale < 3.0e38f))   // also refuses NaN and +inf
        return TF_E_INVALID;
    if (a->mask != TF_MASK_CAUSAL && a->mask != TF_MASK_FULL && a->mask != TF_MASK_TREE)
        return TF_E_INVALID;
    if (a->n_segments == 0)
        return TF_OK;
    if (a->max_rows < 1 || a->max_keys < a->max_rows)
        return TF_E_INVALID;
    if (a->segs == nullptr || a->q == nullptr || a->out == nullptr)
        return TF_E_INVALID;
    if (!aligned16(a->q) || !aligned16(a->out))
        return TF_E_INVALID;
    if (a->mask == TF_MASK_TREE &&
        (a->tree == nullptr || (reinterpret_cast<uintptr_t>(a->tree) & 7u) != 0 || a->max_rows > 64))
        return TF_E_INVALID;
    const int64_t splits = n_splits_of(a->max_keys, a->split_keys);
    if ((int64_t)a->n_segments * splits > 0x7FFFFFFF || (int64_t)a->n_segments * a->max_rows > 0x7FFFFFFF)
        return TF_E_INVALID;
    if (need_partials || a->split_keys > 0) {
        if (a->split_keys == 0)
            return TF_E_INVALID;   // merge needs split partials
        if (a->partials == nullptr || (int64_t)a->partials_bytes < record_bytes(a->head_dim))
            return TF_E_WORKSPACE;
        if (!aligned16(a->partials))
            return TF_E_INVALID;
    }
    return TF_OK;
}

// Whether the product of the (non-negative) factors stays at or below limit,
// without overflowing on the way.
bool product_fits(std::initializer_list<int64_t> factors, int64_t limit)
{
    int64_t x = 1;
    for (const int64_t f : factors) {
        if (f == 0)
            return true;
        if (f < 0 || x > limit / f)
            return false;
        x *= f;
    }
    return true;
}

tfa::RowsParams make_params(const tf_attn_args *a)
{
    tfa::RowsParams p;
    p.segs = a->segs;
    p.q = static_cast<const uint16_t *>(a->q);
    p.out = static_cast<uint16_t *>(a->out);
    p.partials = a->partials;
    p.max_records = a->split_keys > 0 ? (int64_t)a->partials_bytes / record_bytes(a->head_dim) : 0;
    p.err = a->err;
    p.n_segments = a->n_segments;
    p.total_rows = a->total_rows;
    p.hq = a->n_q_heads;
    p.hkv = a->n_kv_heads;
    p.group = a->n_q_heads / a->n_kv_heads;
    p.page_size = a->kind == TF_KV_PAGED ? a->page_size : 1;
    p.page_shift = 0;
    while ((1 << p.page_shift) < p.page_size)
        ++p.page_shift;
    p.pool_pages = a->kind == TF_KV_PAGED ? a->pool_pages : 0;
    p.split_keys = a->split_keys;
    p.n_split_max = n_splits_of(a->max_keys, a->split_keys);
    p.max_rows = a->max_rows;
    p.max_keys = a->max_keys;
    p.c_log2 = (float)((double)a->scale * 1.4426950408889634073599);
    p.mfma_min_q = tfa::kMfmaMinQ;
    p.mask = a->mask;
    p.tree = a->mask == TF_MASK_TREE ? a->tree : nullptr;
    return p;
}

}  // namespace

extern "C" {

const char *tf_strerror(int code)
{
    switch (code) {
    case TF_OK:
        return "ok";
    case TF_E_INVALID:
        return "invalid argument";
    case TF_E_UNSUPPORTED:
        return "unsupported shape (head_dim, page_size or split_keys)";
    case TF_E_PAST_PAGES:
        return "a segment holds more keys than its pages, ring or buffer";
    case TF_E_WORKSPACE:
        return "workspace missing or too small";
    case TF_E_LAUNCH:
        return "kernel launch failed";
    default:
        return "unknown error";
    }
}

int tf_plan_partials(tf_segment *host_segs, int32_t n_segments, int32_t n_q_heads,
                     int32_t head_dim, int32_t split_keys, size_t *partials_bytes)
{
    if (partials_bytes == nullptr || n_segments < 0 || n_q_heads < 1 ||
        (n_segments > 0 && host_segs == nullptr))
        return TF_E_INVALID;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return TF_E_UNSUPPORTED;
    if (split_keys <= 0 || split_keys % 32 != 0)
        return TF_E_UNSUPPORTED;
    int64_t at = 0;
    for (int i = 0; i < n_segments; ++i) {
        tf_segment &s = host_segs[i];
        if (s.n_rows < 1 || s.key_count < s.n_rows)
            return TF_E_INVALID;
        if (at > 0x7FFFFFFF)
            return TF_E_INVALID;
        s.partial_offset = (int32_t)at;
        at += (int64_t)s.n_rows * n_q_heads * n_splits_of(s.key_count, split_keys);
    }
    if (at > 0x7FFFFFFF)
        return TF_E_INVALID;
    *partials_bytes = (size_t)(at * record_bytes(head_dim));
    return TF_OK;
}

int tf_check_segments(const tf_attn_args *a, const tf_segment *host_segs)
{
    int rc = check_args(a, false);
    if (rc != TF_OK)
        return rc;
    if (a->n_segments > 0 && host_segs == nullptr)
        return TF_E_INVALID;
    const int64_t max_records =
        a->split_keys > 0 ? (int64_t)a->partials_bytes / record_bytes(a->head_dim) : 0;
    std::vector<std::pair<int64_t, int64_t>> spans;
    spans.reserve((size_t)a->n_segments);
    int past = 0, workspace = 0, storage = 0;
    for (int i = 0; i < a->n_segments; ++i) {
        const tf_segment &s = host_segs[i];
        if (s.k == nullptr || s.v == nullptr || !aligned16(s.k) || !aligned16(s.v))
            return TF_E_INVALID;
        if (s.n_rows < 1 || s.n_rows > s.key_count || s.n_rows > a->max_rows || s.n_rows < a->min_rows ||
            s.key_count > a->max_keys)
            return TF_E_INVALID;
        if (s.row_offset < 0 || (int64_t)s.row_offset + s.n_rows > a->total_rows)
            return TF_E_INVALID;
        if (a->kind == TF_KV_PAGED) {
            if (s.pages == nullptr || s.capacity < 0)
                return TF_E_INVALID;
            if ((int64_t)s.key_count > (int64_t)s.capacity * a->page_size)
                past = 1;
        } else {
            if (s.capacity < 0)
                return TF_E_INVALID;
            if (s.key_count > s.capacity)
                past = 1;
            if (a->kind == TF_KV_RING && (s.first < 0 || s.first >= s.capacity))
                return TF_E_INVALID;
            if (a->kind == TF_KV_CONTIG && s.first != 0)
                return TF_E_INVALID;
            // one kv head's run must stay within the kernels' 32-bit offsets
            if ((int64_t)s.capacity * a->head_dim * 2 > 0xFFFFFFFFll)
                storage = 1;
        }
        if (a->split_keys > 0) {
            const int64_t need = (int64_t)s.n_rows * a->n_q_heads * n_splits_of(s.key_count, a->split_keys);
            if (s.partial_offset < 0 || (int64_t)s.partial_offset + need > max_records)
                workspace = 1;
        }
        spans.emplace_back((int64_t)s.row_offset, (int64_t)s.row_offset + s.n_rows);
    }
    std::sort(spans.begin(), spans.end());
    for (size_t i = 1; i < spans.size(); ++i)
        if (spans[i].first < spans[i - 1].second)
            return TF_E_INVALID;   // two segments write the same output rows
    if (storage)
        return TF_E_UNSUPPORTED;
    if (past)
        return TF_E_PAST_PAGES;
    if (workspace)
        return TF_E_WORKSPACE;
    return TF_OK;
}

int tf_attn_rows(const tf_attn_args *a, hipStream_t stream)
{
    const int rc = check_args(a, false);
    if (rc != TF_OK)
        return rc;
    if (a->n_segments == 0)
        return TF_OK;
    tfa::RowsParams p = make_params(a);
    // one block per (split, segment, kv head), in a one-dimensional grid
    if (!product_fits({p.n_split_max, p.n_segments, p.hkv}, (int64_t)INT32_MAX / 256))
        return TF_E_UNSUPPORTED;
    // Segments with at most kMfmaMinQ query vectors per kv head (decode,
    // short verify) run on the VALU kernel, the others on the MFMA kernel;
    // the choice depends on the segment alone.
    const int64_t nq_max = (int64_t)a->max_rows * p.group;
    const int qb = tfa::mfma_query_tile(a->head_dim, nq_max);
    const int64_t n_qt = (nq_max + qb - 1) / qb;
    if (nq_max > p.mfma_min_q &&
        !product_fits({n_qt, p.n_split_max, p.n_segments, p.hkv}, (int64_t)INT32_MAX / 512))
        return TF_E_UNSUPPORTED;
    if (a->min_rows > 0 && (int64_t)a->min_rows * p.group > p.mfma_min_q) {
        // every segment has many query vectors: no decode launch, and the
        // matrix-core kernel takes all segments (so none is dropped even if
        // the hint were wrong)
        p.mfma_min_q = 0;
    } else if (tfa::launch_rows_valu(p, a->head_dim, a->kind, stream) != hipSuccess) {
        return TF_E_LAUNCH;
    }
    if (nq_max > p.mfma_min_q) {
        if (tfa::launch_rows_mfma(p, a->head_dim, a->kind, (int)nq_max, stream) != hipSuccess)
            return TF_E_LAUNCH;
    }
    return TF_OK;
}

int tf_attn_merge(const tf_attn_args *a, hipStream_t stream)
{
    const int rc = check_args(a, true);
    if (rc != TF_OK)
        return rc;
    if (a->n_segments == 0)
        return TF_OK;
    const tfa::RowsParams p = make_params(a);
    if (tfa::launch_merge(p, a->head_dim, a->max_rows, stream) != hipSuccess)
        return TF_E_LAUNCH;
    return TF_OK;
}

size_t tf_argmax_workspace_bytes(int32_t n_rows, int32_t vocab)
{
    if (n_rows <= 0 || vocab <= 0)
        return 0;
    return (size_t)n_rows * tfa::argmax_slot_bytes();
}

int tf_argmax(const void *logits, int32_t n_rows, int32_t vocab, int64_t row_stride, int32_t *ids,
              uint8_t *flags, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (n_rows < 0 || vocab < 1 || row_stride < vocab)
        return TF_E_INVALID;
    if (n_rows == 0)
        return TF_OK;
    if (logits == nullptr || ids == nullptr || flags == nullptr)
        return TF_E_INVALID;
    if ((reinterpret_cast<uintptr_t>(logits) & 1u) != 0)
        return TF_E_INVALID;
    if (workspace == nullptr || workspace_bytes < tf_argmax_workspace_bytes(n_rows, vocab) ||
        (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
        return TF_E_WORKSPACE;
    if ((int64_t)n_rows * tfa::argmax_chunk_count(vocab) > 0x7FFFFFFF)
        return TF_E_INVALID;
    if (tfa::argmax_chunk_count(vocab) > 0xFFFF)
        return TF_E_UNSUPPORTED;   // a row's chunk count must fit the counter's 16 bits
    if (tfa::launch_argmax(static_cast<const uint16_t *>(logits), n_rows, vocab, row_stride, ids, flags,
                           workspace, stream) != hipSuccess)
        return TF_E_LAUNCH;
    return TF_OK;
}

}  // extern "C"
