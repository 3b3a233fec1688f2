// The merge of one (row, head)'s split records by one wave (merge_kernel,
// tf_attn_merge; TensorFold PR #1503, the shared-window merge body; PR
// #1653, the paged decode merge).
//
//     M = max_t m_t,  L = sum_t l_t e^(m_t - M),  out = sum_t o_t e^(m_t - M) / L
//
// Lane t reads split t's (m, l); M and L reduce over lanes by a fixed xor
// butterfly (the same bits in every lane); each lane owns D/64 dimensions
// and sums the splits' o in split order.  Every load is issued before any
// result is used (one memory round trip per 16 splits).  A NaN record (or
// an empty (row, head)) gives NaN.
#pragma once

#include "device.hpp"

namespace tfa {

constexpr int kMergeChunk = 16;   // splits whose o loads are in flight together

__device__ __forceinline__ float merge_wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float merge_wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

// Load the lane's DL floats of o from a record (16-, 8- or 4-byte aligned).
template <int DL>
__device__ __forceinline__ void load_o(const float *src, float (&dst)[DL])
{
    if constexpr (DL == 4) {
        const float4 x = *reinterpret_cast<const float4 *>(src);
        dst[0] = x.x;
        dst[1] = x.y;
        dst[2] = x.z;
        dst[3] = x.w;
    } else if constexpr (DL == 2) {
        const float2 x = *reinterpret_cast<const float2 *>(src);
        dst[0] = x.x;
        dst[1] = x.y;
    } else {
        dst[0] = src[0];
    }
}

// Merge the n_splits records starting at `rec` (record stride D + 4 floats)
// into dst[0 .. D) (bf16).  parts_ok false: write NaN.
template <int D>
__device__ __forceinline__ void merge_one(const float *rec, int n_splits, bool parts_ok, uint16_t *dst, int lane)
{
    constexpr int DL = D / 64;   // dims per lane
    constexpr int RS = D + 4;    // record stride (floats)
    float acc[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i)
        acc[i] = 0.0f;
    bool nan_out = !parts_ok;
    if (parts_ok) {
        // lane t holds split t's (m, l), read together; splits past 64 are
        // read in a loop
        float ml = -INFINITY, ll = 0.0f;
        if (lane < n_splits) {
            const float2 x = *reinterpret_cast<const float2 *>(rec + (int64_t)lane * RS);
            ml = x.x;
            ll = x.y;
        }
        // the first chunk of o is in flight while the maxima reduce
        float of[kMergeChunk][DL];
        const int c0 = min(n_splits, kMergeChunk);
#pragma unroll
        for (int u = 0; u < kMergeChunk; ++u)
            if (u < c0)
                load_o<DL>(rec + (int64_t)u * RS + 4 + lane * DL, of[u]);
        bool bad = __builtin_isnan(ml);
        float big = ml;
        for (int t = lane + 64; t < n_splits; t += 64) {
            const float mt = rec[(int64_t)t * RS];
            bad = bad || __builtin_isnan(mt);
            big = fmaxf(big, mt);
        }
        big = merge_wave_max(big);
        nan_out = __builtin_amdgcn_ballot_w64(bad) != 0 || big == -INFINITY;
        // weight of split t, computed by lane t (splits past 64 directly)
        const float wl = (ml == -INFINITY) ? 0.0f : exp2_fast((ml - big) * kLog2e);
        float lsum = ll * wl;
        for (int t = lane + 64; t < n_splits; t += 64) {
            const float mt = rec[(int64_t)t * RS];
            if (mt != -INFINITY)
                lsum += rec[(int64_t)t * RS + 1] * exp2_fast((mt - big) * kLog2e);
        }
        lsum = merge_wave_sum(lsum);
        for (int t0 = 0; t0 < n_splits; t0 += kMergeChunk) {
            const int cn = min(n_splits - t0, kMergeChunk);
            if (t0 > 0) {
#pragma unroll
                for (int u = 0; u < kMergeChunk; ++u)
                    if (u < cn)
                        load_o<DL>(rec + (int64_t)(t0 + u) * RS + 4 + lane * DL, of[u]);
            }
#pragma unroll
            for (int u = 0; u < kMergeChunk; ++u) {
                if (u < cn) {
                    const int t = t0 + u;
                    float w;
                    if (t < 64) {
                        w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), t));
                    } else {
                        const float mt = rec[(int64_t)t * RS];
                        w = (mt == -INFINITY) ? 0.0f : exp2_fast((mt - big) * kLog2e);
                    }
#pragma unroll
                    for (int i = 0; i < DL; ++i)
                        acc[i] = fmaf(of[u][i], w, acc[i]);
                }
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
    uint16_t *d = dst + lane * DL;
    if constexpr (DL == 1) {
        d[0] = b[0];
    } else if constexpr (DL == 2) {
        *reinterpret_cast<uint32_t *>(d) = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
    } else {
        *reinterpret_cast<uint2 *>(d) =
            make_uint2((uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16));
    }
}

}  // namespace tfa
