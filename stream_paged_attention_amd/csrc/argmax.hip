// tf_argmax: greedy pick of each row's first largest logit, with a flag on
// rows that hold a NaN or +-Inf (TensorFold PR #1503, the lfm2_argmax commit:
// equal maxima resolve to the smaller id and a nonfinite row is flagged; the
// router note: a NaN counts as -inf).
//
// Every logit becomes an order-preserving key: its bf16 value mapped to an
// unsigned 16-bit rank (NaN taken as -inf, -0.0 as +0.0) above the complement
// of its id, so the largest key is the largest value at the lowest id.  The
// max of keys is order-independent, so the pick does not depend on how the
// row is cut up.  Phase 1: one workgroup per (row, 8192-logit chunk) reduces
// its chunk to a key and a flag.  Phase 2: one wave per row reduces the
// chunks.  A row of one chunk (vocabularies up to 8192) is finished by
// phase 1, which then writes the id and flag itself: one launch.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kChunk = 8192;
constexpr int kThreads = 256;
constexpr int kPerThread = kChunk / kThreads;   // 32 logits, 4 groups of 8

__device__ __forceinline__ uint32_t rank16(uint32_t b, uint32_t &nonfinite)
{
    nonfinite |= ((b & 0x7F80u) == 0x7F80u) ? 1u : 0u;
    if ((b & 0x7FFFu) > 0x7F80u)
        b = 0xFF80u;   // NaN ranks as -inf
    if (b == 0x8000u)
        b = 0u;        // -0.0 equals +0.0
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__global__ __launch_bounds__(kThreads) void argmax_chunks(const uint16_t *logits, int vocab,
                                                          int64_t row_stride, int n_chunks,
                                                          int vec_ok, uint64_t *keys,
                                                          uint32_t *flags, int32_t *row_ids,
                                                          uint8_t *row_flags)
{
    const int chunk = blockIdx.x % n_chunks;
    const int row = blockIdx.x / n_chunks;
    const int c0 = chunk * kChunk;
    const uint16_t *x = logits + (int64_t)row * row_stride;
    uint32_t best = 0;   // every real key is > 0 (rank >= 0x007F)
    uint32_t nonfinite = 0;
#pragma unroll
    for (int it = 0; it < kPerThread / 8; ++it) {
        const int local = it * (kThreads * 8) + threadIdx.x * 8;   // first of 8 logits
        const int i0 = c0 + local;
        if (vec_ok && i0 + 8 <= vocab) {
            const uint4 w = *reinterpret_cast<const uint4 *>(x + i0);
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t b = (e & 1) ? (u[e >> 1] >> 16) : (u[e >> 1] & 0xFFFFu);
                const uint32_t key = (rank16(b, nonfinite) << 16) | (0xFFFFu - (uint32_t)(local + e));
                best = max(best, key);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (i0 + e < vocab) {
                    const uint32_t key = (rank16(x[i0 + e], nonfinite) << 16) |
                                         (0xFFFFu - (uint32_t)(local + e));
                    best = max(best, key);
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        best = max(best, (uint32_t)__shfl_xor((int)best, off));
        nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off);
    }
    __shared__ uint32_t sb[kThreads / 64], sf[kThreads / 64];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sb[wave] = best;
        sf[wave] = nonfinite;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            best = max(best, sb[w]);
            nonfinite |= sf[w];
        }
        const uint32_t id = (uint32_t)c0 + (0xFFFFu - (best & 0xFFFFu));
        if (n_chunks == 1) {
            row_ids[row] = (int32_t)id;
            row_flags[row] = nonfinite ? 1 : 0;
            return;
        }
        const uint64_t key = ((uint64_t)(best >> 16) << 32) | (uint64_t)(0xFFFFFFFFu - id);
        keys[(int64_t)row * n_chunks + chunk] = key;
        flags[(int64_t)row * n_chunks + chunk] = nonfinite;
    }
}

__global__ __launch_bounds__(kThreads) void argmax_rows(int n_rows, int n_chunks,
                                                        const uint64_t *keys,
                                                        const uint32_t *cflags, int32_t *ids,
                                                        uint8_t *flags)
{
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n_rows)
        return;
    uint64_t best = 0;
    uint32_t nonfinite = 0;
    for (int c = lane; c < n_chunks; c += 64) {
        const uint64_t k = keys[(int64_t)row * n_chunks + c];
        best = k > best ? k : best;
        nonfinite |= cflags[(int64_t)row * n_chunks + c];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, off);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
        nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off);
    }
    if (lane == 0) {
        ids[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
        flags[row] = nonfinite ? 1 : 0;
    }
}

}  // namespace

int argmax_chunk_count(int vocab) { return (vocab + kChunk - 1) / kChunk; }

hipError_t launch_argmax(const uint16_t *logits, int n_rows, int vocab, int64_t row_stride,
                         int32_t *ids, uint8_t *flags, void *workspace, hipStream_t st)
{
    const int n_chunks = argmax_chunk_count(vocab);
    uint64_t *keys = static_cast<uint64_t *>(workspace);
    uint32_t *cflags = reinterpret_cast<uint32_t *>(keys + (int64_t)n_rows * n_chunks);
    const int vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0 && (row_stride & 7) == 0) ? 1 : 0;
    hipLaunchKernelGGL(argmax_chunks, dim3((unsigned)(n_chunks * n_rows)), dim3(kThreads), 0, st,
                       logits, vocab, row_stride, n_chunks, vec_ok, keys, cflags, ids, flags);
    if (n_chunks == 1)
        return hipGetLastError();
    hipLaunchKernelGGL(argmax_rows, dim3((unsigned)((n_rows + 3) / 4)), dim3(kThreads), 0, st, n_rows,
                       n_chunks, keys, cflags, ids, flags);
    return hipGetLastError();
}

}  // namespace tfa
