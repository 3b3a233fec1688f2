// tf_argmax: greedy pick of each row's first largest logit, with a flag on
// rows that hold a NaN or +-Inf (TensorFold PR #1503, the lfm2_argmax commit:
// equal maxima resolve to the smaller id and a nonfinite row is flagged; the
// router note: a NaN counts as -inf).
//
// Every logit becomes an order-preserving key: its bf16 value mapped to an
// unsigned 16-bit rank (NaN taken as -inf, -0.0 as +0.0) above the complement
// of its id, so the largest key is the largest value at the lowest id.  The
// max of keys is order-independent, so the pick does not depend on how the
// row is cut up.  One launch: one workgroup per (row, 16384-logit chunk)
// reduces its chunk to a key and a flag.  A row of one chunk is finished
// there.  Otherwise each chunk folds its key into the row's 64-bit slot of
// the workspace with an atomic max, then counts itself (and its flag) into
// the row's counter word; the chunk that completes the count reads the final
// key back with an exchange that re-zeroes the slot, writes the id and flag,
// and zeroes the counter: the workspace is left as it was found, all zero.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kChunk = 16384;   // 8 chunks a row at 128 000 logits
constexpr int kThreads = 1024;
constexpr int kPerThread = kChunk / kThreads;   // 16 logits, 2 groups of 8

__device__ __forceinline__ uint32_t rank16(uint32_t b, uint32_t &nonfinite)
{
    nonfinite |= ((b & 0x7F80u) == 0x7F80u) ? 1u : 0u;
    if ((b & 0x7FFFu) > 0x7F80u)
        b = 0xFF80u;   // NaN ranks as -inf
    if (b == 0x8000u)
        b = 0u;        // -0.0 equals +0.0
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// A row's workspace slot: the largest chunk key so far and the count of
// chunks done (low 16 bits) plus the count of chunks holding a nonfinite
// logit (high 16 bits).  All zero between calls.
struct RowSlot {
    uint64_t key;
    uint32_t count;
    uint32_t pad;
};

__global__ __launch_bounds__(kThreads) void argmax_chunks(const uint16_t *logits, int vocab,
                                                          int64_t row_stride, int n_chunks,
                                                          int vec_ok, RowSlot *slots,
                                                          int32_t *row_ids, uint8_t *row_flags)
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
        RowSlot *slot = slots + row;
        __hip_atomic_fetch_max(&slot->key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the max is performed (acknowledged) before this chunk is counted,
        // so the chunk that sees the full count reads every chunk's key
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const uint32_t add = 1u + (nonfinite ? 0x10000u : 0u);
        const uint32_t old = __hip_atomic_fetch_add(&slot->count, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((old & 0xFFFFu) == (uint32_t)(n_chunks - 1)) {
            const uint64_t fin = __hip_atomic_exchange(&slot->key, (uint64_t)0, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&slot->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            row_ids[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(fin & 0xFFFFFFFFu));
            row_flags[row] = ((old >> 16) + (nonfinite ? 1u : 0u)) != 0 ? 1 : 0;
        }
    }
}

}  // namespace

int argmax_chunk_count(int vocab) { return (vocab + kChunk - 1) / kChunk; }

size_t argmax_slot_bytes() { return sizeof(RowSlot); }

hipError_t launch_argmax(const uint16_t *logits, int n_rows, int vocab, int64_t row_stride,
                         int32_t *ids, uint8_t *flags, void *workspace, hipStream_t st)
{
    const int n_chunks = argmax_chunk_count(vocab);
    const int vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0 && (row_stride & 7) == 0) ? 1 : 0;
    hipLaunchKernelGGL(argmax_chunks, dim3((unsigned)(n_chunks * n_rows)), dim3(kThreads), 0, st,
                       logits, vocab, row_stride, n_chunks, vec_ok, static_cast<RowSlot *>(workspace), ids,
                       flags);
    return hipGetLastError();
}

}  // namespace tfa
