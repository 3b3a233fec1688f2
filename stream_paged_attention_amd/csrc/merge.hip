// tf_attn_merge: combine each (row, head)'s split partials into bf16 output
// (TensorFold PR #1503, the shared-window merge body; PR #1653, the paged
// decode merge with nonfinite heads kept off its fast path).
//
// One wave per (segment, row, query head).  The split maxima and sums are
// read lane-parallel (lane t holds split t) and reduced with a fixed xor
// butterfly, which gives every lane the same bits; then each lane, owning
// D/64 consecutive dimensions, folds the splits' o[] in split order with
// several loads in flight.  Everything depends only on the record's own
// segment, so a batched launch equals one launch per segment.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(RowsParams p, int max_rows)
{
    constexpr int DL = D / 64;   // dims per lane
    constexpr int RS = D + 4;    // record stride (floats)
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
    const bool parts_ok = sd.partial_offset >= 0 &&
                          (int64_t)sd.partial_offset + (int64_t)n_rows * p.hq * n_splits <= p.max_records;
    float acc[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i)
        acc[i] = 0.0f;
    bool nan_out = !parts_ok;
    if (parts_ok) {
        const float *rec = p.partials + first * RS;
        // max over splits and NaN check, lane-parallel
        float big = -INFINITY;
        bool bad = false;
        for (int t = lane; t < n_splits; t += 64) {
            const float mt = rec[(int64_t)t * RS];
            bad = bad || __builtin_isnan(mt);
            big = fmaxf(big, mt);
        }
        big = wave_max(big);
        nan_out = __builtin_amdgcn_ballot_w64(bad) != 0 || big == -INFINITY;
        // L = sum_t l_t e^(m_t - M)
        float lsum = 0.0f;
        for (int t = lane; t < n_splits; t += 64) {
            const float mt = rec[(int64_t)t * RS];
            if (mt != -INFINITY)
                lsum += rec[(int64_t)t * RS + 1] * exp2_fast((mt - big) * kLog2e);
        }
        lsum = wave_sum(lsum);
        // O = sum_t o_t e^(m_t - M), splits in order
#pragma unroll 4
        for (int t = 0; t < n_splits; ++t) {
            const float *rt = rec + (int64_t)t * RS;
            const float mt = rt[0];
            const float w = (mt == -INFINITY) ? 0.0f : exp2_fast((mt - big) * kLog2e);
            const float *ot = rt + 4 + lane * DL;
            if constexpr (DL == 1) {
                acc[0] = fmaf(ot[0], w, acc[0]);
            } else if constexpr (DL == 2) {
                const float2 x = *reinterpret_cast<const float2 *>(ot);
                acc[0] = fmaf(x.x, w, acc[0]);
                acc[1] = fmaf(x.y, w, acc[1]);
            } else {
                const float4 x = *reinterpret_cast<const float4 *>(ot);
                acc[0] = fmaf(x.x, w, acc[0]);
                acc[1] = fmaf(x.y, w, acc[1]);
                acc[2] = fmaf(x.z, w, acc[2]);
                acc[3] = fmaf(x.w, w, acc[3]);
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
