// tf_state_save / tf_state_restore: copy the K and V rows of a stream's
// positions [0, at) between its pool pages and a kept state (TensorFold
// PR #1503, the prompt-cache commit: whole pages copied as units, then the
// last page's rows; the state restored into the resuming stream's pages).
//
// One workgroup per (layer, K or V, logical page, 16 KB chunk of the page).
// A page is n_kv_heads x page_size x head_dim bf16, contiguous in both the
// pool and the state (head-major pages), so a chunk is one contiguous run in
// each: every thread moves four 16-byte units, all loads issued before any
// store.  The page id is read once per workgroup.  In the last page only rows
// below `at` move.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kUnitsPerThread = 4;
constexpr int kChunkUnits = kCopyThreads * kUnitsPerThread;   // 16 KB per workgroup

struct StateParams {
    const int32_t *pages;
    const tf_state_layer *layers;
    int32_t *err;
    int hkv;
    int page_size;
    int pool_pages;
    int at;
    int n_state_pages;       // ceil(at / page_size)
    int rows_last;           // rows of the last state page: at - (n_state_pages - 1) * page_size
    int64_t page_units;      // 16-byte units per page: hkv * page_size * D * 2 / 16
    int n_chunks;            // chunks per page
};

template <int D, bool SAVE>
__global__ __launch_bounds__(kCopyThreads) void state_copy_kernel(StateParams p)
{
    // work item order: chunk fastest, then page, K/V, layer slowest
    int rest = blockIdx.x;
    const int chunk = rest % p.n_chunks;
    rest /= p.n_chunks;
    const int page = rest % p.n_state_pages;
    rest /= p.n_state_pages;
    const int kv = rest & 1;
    const int layer = rest >> 1;

    const tf_state_layer &L = p.layers[layer];
    // a layer with any null or misaligned pointer is skipped whole
    const uintptr_t ptrs[4] = {reinterpret_cast<uintptr_t>(L.pool_k), reinterpret_cast<uintptr_t>(L.pool_v),
                               reinterpret_cast<uintptr_t>(L.state_k), reinterpret_cast<uintptr_t>(L.state_v)};
    bool layer_ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        layer_ok = layer_ok && ptrs[i] != 0 && (ptrs[i] & 15u) == 0;
    if (!layer_ok) {
        if (threadIdx.x == 0 && page == 0 && chunk == 0 && kv == 0)
            report(p.err, TF_ERR_BAD_LAYER);
        return;
    }
    const char *pool_c = reinterpret_cast<const char *>(kv ? ptrs[1] : ptrs[0]);
    const char *state_c = reinterpret_cast<const char *>(kv ? ptrs[3] : ptrs[2]);
    const int pid = load_global<int32_t>(p.pages + page);
    if ((unsigned)pid >= (unsigned)p.pool_pages) {
        if (threadIdx.x == 0 && chunk == 0)
            report(p.err, TF_ERR_BAD_PAGE);
        return;
    }
    // units of one (kv head, row): D * 2 / 16; in the last page a unit moves
    // only if its row is below at
    constexpr int kRowUnits = D * 2 / 16;
    const bool last = page == p.n_state_pages - 1;
    const int64_t pool0 = (int64_t)pid * p.page_units;
    const int64_t state0 = (int64_t)page * p.page_units;
    const char *src = SAVE ? pool_c : state_c;
    char *dst = const_cast<char *>(SAVE ? state_c : pool_c);
    const int64_t src0 = SAVE ? pool0 : state0;
    const int64_t dst0 = SAVE ? state0 : pool0;

    u32x4_t x[kUnitsPerThread];
    bool move[kUnitsPerThread];
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
        const int64_t u = (int64_t)chunk * kChunkUnits + i * kCopyThreads + threadIdx.x;
        const int row = (int)((u / kRowUnits) % p.page_size);
        move[i] = u < p.page_units && (!last || row < p.rows_last);
        if (move[i])
            x[i] = load_stream<u32x4_t>(src + (src0 + u) * 16);
    }
#pragma unroll
    for (int i = 0; i < kUnitsPerThread; ++i) {
        const int64_t u = (int64_t)chunk * kChunkUnits + i * kCopyThreads + threadIdx.x;
        if (move[i])
            __builtin_nontemporal_store(x[i], reinterpret_cast<__attribute__((address_space(1))) u32x4_t *>(
                                                  reinterpret_cast<uintptr_t>(dst + (dst0 + u) * 16)));
    }
}

template <bool SAVE>
int state_copy(const tf_state_args *a, hipStream_t st)
{
    if (a == nullptr || a->n_layers < 0 || a->n_kv_heads < 1 || a->at < 0 || a->n_pages < 0)
        return TF_E_INVALID;
    if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
        return TF_E_UNSUPPORTED;
    const int ps = a->page_size;
    if (ps < 32 || ps > 1024 || (ps & (ps - 1)) != 0)
        return TF_E_UNSUPPORTED;
    if (a->pool_pages < 1)
        return TF_E_INVALID;
    if ((int64_t)a->at > (int64_t)a->n_pages * ps)
        return TF_E_PAST_PAGES;
    if (a->at == 0 || a->n_layers == 0)
        return TF_OK;
    if (a->pages == nullptr || a->layers == nullptr)
        return TF_E_INVALID;
    StateParams p;
    p.pages = a->pages;
    p.layers = a->layers;
    p.err = a->err;
    p.hkv = a->n_kv_heads;
    p.page_size = ps;
    p.pool_pages = a->pool_pages;
    p.at = a->at;
    p.n_state_pages = (a->at + ps - 1) / ps;
    p.rows_last = a->at - (p.n_state_pages - 1) * ps;
    p.page_units = (int64_t)a->n_kv_heads * ps * a->head_dim * 2 / 16;
    const int64_t chunks = (p.page_units + kChunkUnits - 1) / kChunkUnits;
    const int64_t grid = chunks * p.n_state_pages * 2 * a->n_layers;
    if (chunks > INT32_MAX || grid > INT32_MAX)
        return TF_E_UNSUPPORTED;
    p.n_chunks = (int)chunks;
    const dim3 g((unsigned)grid);
    switch (a->head_dim) {
    case 64:
        hipLaunchKernelGGL((state_copy_kernel<64, SAVE>), g, dim3(kCopyThreads), 0, st, p);
        break;
    case 128:
        hipLaunchKernelGGL((state_copy_kernel<128, SAVE>), g, dim3(kCopyThreads), 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((state_copy_kernel<256, SAVE>), g, dim3(kCopyThreads), 0, st, p);
        break;
    }
    return hipGetLastError() == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

}  // namespace

}  // namespace tfa

extern "C" int tf_state_save(const tf_state_args *a, hipStream_t stream)
{
    return tfa::state_copy<true>(a, stream);
}

extern "C" int tf_state_restore(const tf_state_args *a, hipStream_t stream)
{
    return tfa::state_copy<false>(a, stream);
}
