// tf_attn_merge: combine each (row, head)'s split partials into bf16 output
// (TensorFold PR #1503, the shared-window merge body; PR #1653, the paged
// decode merge with nonfinite heads kept off its fast path).
//
// One wave per (segment, row, query head), running merge_one (merge.hpp).
// Everything depends only on the record's own segment, so a batched launch
// equals one launch per segment.
#include "merge.hpp"

namespace tfa {

namespace {

constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(RowsParams p, int max_rows)
{
    const int seg_i = blockIdx.x / max_rows;
    const int r = blockIdx.x % max_rows;
    const int h = blockIdx.y * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= p.hq)
        return;
    const tf_segment &sd = p.segs[seg_i];
    // every field is read here, before the error word may be written: that
    // store could alias the table, and a field read after it is fetched again
    const int n_rows = sd.n_rows, kc = sd.key_count, row_offset = sd.row_offset;
    const int partial_offset = sd.partial_offset;
    if (r >= n_rows)
        return;
    if (n_rows < 1 || n_rows > kc || row_offset < 0 || (int64_t)row_offset + n_rows > p.total_rows ||
        (p.mask == TF_MASK_TREE && n_rows > 64))
        return;   // reported by tf_attn_rows; no row can be addressed safely
    const int n_splits = (kc + p.split_keys - 1) / p.split_keys;
    const int64_t first = (int64_t)partial_offset + ((int64_t)r * p.hq + h) * n_splits;
    // past the hints the rows kernels did not write every record: NaN
    const bool hints_ok = n_rows <= max_rows && kc <= p.max_keys;
    if (!hints_ok && r == 0 && h == 0 && lane == 0)
        report(p.err, TF_ERR_HINTS);
    const bool parts_ok = hints_ok && partial_offset >= 0 &&
                          (int64_t)partial_offset + (int64_t)n_rows * p.hq * n_splits <= p.max_records;
    uint16_t *dst = p.out + ((size_t)(row_offset + r) * p.hq + h) * D;
    merge_one<D>(p.partials + (parts_ok ? first : 0) * (D + 4), n_splits, parts_ok, dst, lane);
}

}  // namespace

// grid = (n_segments * max_rows, ceil(Hq / 4)); one wave per (row, head).
hipError_t launch_merge(const RowsParams &p, int head_dim, int max_rows, hipStream_t st)
{
    const dim3 grid((unsigned)(p.n_segments * max_rows), (unsigned)((p.hq + kWaves - 1) / kWaves));
    switch (head_dim) {
    case 64:
        hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(64 * kWaves), 0, st, p, max_rows);
        break;
    case 128:
        hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(64 * kWaves), 0, st, p, max_rows);
        break;
    default:
        hipLaunchKernelGGL((merge_kernel<256>), grid, dim3(64 * kWaves), 0, st, p, max_rows);
        break;
    }
    return hipGetLastError();
}

}  // namespace tfa
