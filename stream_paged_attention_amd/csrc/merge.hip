// tf_attn_merge: combine each (row, head)'s split partials into bf16 output
// (TensorFold PR #1503, the shared-window merge body; PR #1653, the paged
// decode merge with nonfinite heads kept off its fast path).
//
// One wave per (segment, row, query head); lane i owns D/64 consecutive
// dimensions, so every record's o[] is read with one coalesced wave load.
// Splits are folded in order t = 0, 1, ... (fixed order: bit-reproducible and
// independent of the other segments of the launch).
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(RowsParams p, int max_rows)
{
    constexpr int DL = D / 64;   // dims per lane
    const int seg_i = blockIdx.x / max_rows;
    const int r = blockIdx.x % max_rows;
    const int h = blockIdx.y * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= p.hq)
        return;
    const tf_segment &sd = p.segs[seg_i];
    const int n_rows = sd.n_rows, kc = sd.key_count, row_offset = sd.row_offset;
    if (r >= n_rows)
        return;
    if (n_rows < 1 || n_rows > kc || row_offset < 0 || (int64_t)row_offset + n_rows > p.total_rows)
        return;   // reported by tf_attn_rows; no row can be addressed safely
    const int n_splits = (kc + p.split_keys - 1) / p.split_keys;
    const int64_t first = (int64_t)sd.partial_offset + ((int64_t)r * p.hq + h) * n_splits;
    uint16_t *dst = p.out + ((size_t)(row_offset + r) * p.hq + h) * D + lane * DL;
    float acc[DL];
    const bool parts_ok = sd.partial_offset >= 0 &&
                          (int64_t)sd.partial_offset + (int64_t)n_rows * p.hq * n_splits <= p.max_records;
    bool nan_out = !parts_ok;
    if (parts_ok) {
        const float *rec = p.partials + first * (D + 4);
        float big = -INFINITY;
        for (int t = 0; t < n_splits; ++t) {
            const float mt = rec[(int64_t)t * (D + 4)];
            nan_out = nan_out || __builtin_isnan(mt);
            big = fmaxf(big, mt);
        }
        nan_out = nan_out || big == -INFINITY;
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < DL; ++i)
            acc[i] = 0.0f;
        for (int t = 0; t < n_splits; ++t) {
            const float *rt = rec + (int64_t)t * (D + 4);
            const float mt = rt[0];
            if (mt == -INFINITY)
                continue;   // empty split
            const float w = exp2_fast((mt - big) * kLog2e);
            lsum += rt[1] * w;
            const float *ot = rt + 4 + lane * DL;
            if constexpr (DL == 1) {
                acc[0] += ot[0] * w;
            } else if constexpr (DL == 2) {
                const float2 x = *reinterpret_cast<const float2 *>(ot);
                acc[0] += x.x * w;
                acc[1] += x.y * w;
            } else {
                const float4 x = *reinterpret_cast<const float4 *>(ot);
                acc[0] += x.x * w;
                acc[1] += x.y * w;
                acc[2] += x.z * w;
                acc[3] += x.w * w;
            }
        }
#pragma unroll
        for (int i = 0; i < DL; ++i)
            acc[i] = acc[i] / lsum;
    }
    uint16_t b[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i)
        b[i] = nan_out ? kBf16NaN : bf16_out(acc[i]);
    if constexpr (DL == 1) {
        dst[0] = b[0];
    } else if constexpr (DL == 2) {
        *reinterpret_cast<uint32_t *>(dst) = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
    } else {
        *reinterpret_cast<uint2 *>(dst) =
            make_uint2((uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16));
    }
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
