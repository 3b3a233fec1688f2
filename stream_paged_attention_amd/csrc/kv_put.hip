// tf_kv_put: write each segment's new K/V rows into its pages, ring or
// buffer (TensorFold PR #1653, putting a chunk's rows into the core pool's
// pages; PR #1562, the ring rows written at the head, wrapping).
//
// One workgroup per (segment, new row).  A row is Hkv runs of head_dim bf16
// in the packed source (token-major, like q) and one run per kv head in the
// storage (head-major pages [page][Hkv][P][D], rings and buffers
// [Hkv][slots][D]), so every 16-byte unit moves with coalesced loads and
// stores; K and V are copied by the same threads.  The destination of
// logical key j is computed once per workgroup.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kPutThreads = 256;

struct PutParams {
    const tf_segment *segs;
    const uint16_t *k_new;
    const uint16_t *v_new;
    int32_t *err;
    int n_segments;
    int total_rows;
    int hkv;
    int page_size;
    int page_shift;
    int pool_pages;
};

template <int D, int KIND>
__global__ __launch_bounds__(kPutThreads) void kv_put_kernel(PutParams p, int max_rows)
{
    const int seg_i = blockIdx.x / max_rows;
    const int r = blockIdx.x % max_rows;
    const tf_segment &sd = p.segs[seg_i];
    const int n_rows = sd.n_rows, kc = sd.key_count, row_offset = sd.row_offset;
    const int capacity = sd.capacity, first = sd.first;
    const bool head = threadIdx.x == 0 && r == 0;
    if (r >= max(n_rows, 1))
        return;
    if (n_rows < 1 || n_rows > kc || row_offset < 0 || (int64_t)row_offset + n_rows > p.total_rows) {
        if (head)
            report(p.err, TF_ERR_BAD_ROWS);
        return;
    }
    int bad = n_rows > max_rows ? TF_ERR_HINTS : 0;   // rows past the grid: skip the segment
    if constexpr (KIND == TF_KV_PAGED) {
        if (sd.pages == nullptr || capacity < 0 || (int64_t)kc > ((int64_t)capacity << p.page_shift))
            bad |= TF_ERR_PAST_PAGES;
    } else {
        if (kc > capacity)
            bad |= TF_ERR_PAST_PAGES;
    }
    if constexpr (KIND == TF_KV_RING) {
        if (first < 0 || first >= capacity)
            bad |= TF_ERR_BAD_RING;
    }
    if (bad) {
        if (head)
            report(p.err, bad);
        return;
    }
    const int j = kc - n_rows + r;   // logical key of new row r
    // destination: element offset of (kv head 0, dim 0) of key j and the
    // stride between kv heads
    int64_t dst0, head_stride;
    if constexpr (KIND == TF_KV_PAGED) {
        const int page = load_global<int32_t>(sd.pages + (j >> p.page_shift));
        if ((unsigned)page >= (unsigned)p.pool_pages) {
            if (threadIdx.x == 0)
                report(p.err, TF_ERR_BAD_PAGE);
            return;
        }
        head_stride = (int64_t)p.page_size * D;
        dst0 = (int64_t)page * p.hkv * head_stride + (int64_t)(j & (p.page_size - 1)) * D;
    } else {
        int slot = j;
        if constexpr (KIND == TF_KV_RING) {
            slot = first + j;
            slot -= (slot >= capacity) ? capacity : 0;
        }
        head_stride = (int64_t)capacity * D;
        dst0 = (int64_t)slot * D;
    }
    uint16_t *kd = const_cast<uint16_t *>(static_cast<const uint16_t *>(sd.k));
    uint16_t *vd = const_cast<uint16_t *>(static_cast<const uint16_t *>(sd.v));
    const int64_t src0 = (int64_t)(row_offset + r) * p.hkv * D;
    constexpr int UPH = D / 8;   // 16-byte units per kv head
    const int units = p.hkv * UPH;
    for (int u = threadIdx.x; u < units; u += kPutThreads) {
        const int h = u / UPH;
        const int c = u % UPH;
        const int64_t s = src0 + (int64_t)h * D + c * 8;
        const int64_t d = dst0 + (int64_t)h * head_stride + c * 8;
        const u32x4_t kx = load_global<u32x4_t>(p.k_new + s);
        const u32x4_t vx = load_global<u32x4_t>(p.v_new + s);
        *reinterpret_cast<u32x4_t *>(kd + d) = kx;
        *reinterpret_cast<u32x4_t *>(vd + d) = vx;
    }
}

template <int D>
hipError_t launch_put_d(const PutParams &p, int kind, int max_rows, hipStream_t st)
{
    const dim3 grid((unsigned)(p.n_segments * max_rows));
    switch (kind) {
    case TF_KV_CONTIG:
        hipLaunchKernelGGL((kv_put_kernel<D, TF_KV_CONTIG>), grid, dim3(kPutThreads), 0, st, p, max_rows);
        break;
    case TF_KV_PAGED:
        hipLaunchKernelGGL((kv_put_kernel<D, TF_KV_PAGED>), grid, dim3(kPutThreads), 0, st, p, max_rows);
        break;
    default:
        hipLaunchKernelGGL((kv_put_kernel<D, TF_KV_RING>), grid, dim3(kPutThreads), 0, st, p, max_rows);
        break;
    }
    return hipGetLastError();
}

bool aligned16p(const void *x) { return ((uintptr_t)x & 15u) == 0; }

}  // namespace

}  // namespace tfa

extern "C" int tf_kv_put(const tf_put_args *a, hipStream_t stream)
{
    if (a == nullptr)
        return TF_E_INVALID;
    if (a->kind != TF_KV_CONTIG && a->kind != TF_KV_PAGED && a->kind != TF_KV_RING)
        return TF_E_INVALID;
    if (a->n_segments < 0 || a->total_rows < 0 || a->max_rows < 0 || a->n_kv_heads < 1)
        return TF_E_INVALID;
    if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
        return TF_E_UNSUPPORTED;
    tfa::PutParams p{};
    p.page_size = 1;
    if (a->kind == TF_KV_PAGED) {
        const int ps = a->page_size;
        if (ps < 32 || ps > 1024 || (ps & (ps - 1)) != 0)
            return TF_E_UNSUPPORTED;
        if (a->pool_pages < 1)
            return TF_E_INVALID;
        p.page_size = ps;
        while ((1 << p.page_shift) < ps)
            ++p.page_shift;
        p.pool_pages = a->pool_pages;
    }
    if (a->n_segments == 0)
        return TF_OK;
    if (a->max_rows < 1 || (int64_t)a->n_segments * a->max_rows > 0x7FFFFFFF)
        return TF_E_INVALID;
    if (a->segs == nullptr || a->k_new == nullptr || a->v_new == nullptr)
        return TF_E_INVALID;
    if (!tfa::aligned16p(a->k_new) || !tfa::aligned16p(a->v_new))
        return TF_E_INVALID;
    p.segs = a->segs;
    p.k_new = static_cast<const uint16_t *>(a->k_new);
    p.v_new = static_cast<const uint16_t *>(a->v_new);
    p.err = a->err;
    p.n_segments = a->n_segments;
    p.total_rows = a->total_rows;
    p.hkv = a->n_kv_heads;
    hipError_t e;
    switch (a->head_dim) {
    case 64:
        e = tfa::launch_put_d<64>(p, a->kind, a->max_rows, stream);
        break;
    case 128:
        e = tfa::launch_put_d<128>(p, a->kind, a->max_rows, stream);
        break;
    default:
        e = tfa::launch_put_d<256>(p, a->kind, a->max_rows, stream);
        break;
    }
    return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}
