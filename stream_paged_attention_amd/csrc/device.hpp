// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tf_attn.h"

namespace tfa {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr uint16_t kBf16NaN = 0x7FC0;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Parameters of one rows launch (passed by value to the kernels).
struct RowsParams {
    const tf_segment *segs;
    const uint16_t *q;
    uint16_t *out;
    float *partials;
    int64_t max_records;   // records the partials workspace holds
    int32_t *err;
    int n_segments;
    int total_rows;
    int hq;
    int hkv;
    int group;             // hq / hkv
    int page_size;
    int page_shift;        // log2(page_size)
    int pool_pages;
    int split_keys;        // 0 = one split per (row, head), written straight to out
    int n_split_max;       // grid extent per segment
    int max_rows;          // the launch's hints: the grid covers n_rows <= max_rows and
    int max_keys;          // key_count <= max_keys (a segment past them is an error)
    float c_log2;          // scale * log2(e): scores are kept in base-2 units
    int mfma_min_q;        // segments with more query vectors per kv head than this
                           // (n_rows * group) take the matrix-core kernel
    int mask;              // tf_mask
    const uint64_t *tree;  // TF_MASK_TREE: ancestor mask per packed row
};

// Which keys row r of an n-row segment over kc keys sees (tf_mask), as
// a limit and a tree test: key j counts when row_sees<MASK>(j, ...).
// lim is one past the row's last seen key, cut at the split end k_end.
// The mask is a template argument (one kernel instance each).  Under
// TF_MASK_TREE tb = kc - n is the
// first new key and anc holds the row's ancestors and itself; otherwise tb
// is INT32_MAX and every key below lim counts.  Every key below
// min(lim, tb) counts (unmasked tiles).
struct RowVis {
    int lim;
    int tb;
    uint64_t anc;
};

template <int MASK>
__device__ __forceinline__ RowVis row_vis(const RowsParams &p, int kc, int n, int r, int row_offset,
                                          int k_end)
{
    RowVis v;
    v.tb = INT32_MAX;
    v.anc = 0;
    if constexpr (MASK == TF_MASK_TREE) {
        v.tb = kc - n;
        v.anc = p.tree[row_offset + r] | (1ull << r);
        v.lim = min(v.tb + (64 - __clzll((long long)v.anc)), k_end);
    } else if constexpr (MASK == TF_MASK_FULL) {
        v.lim = k_end;
    } else {
        v.lim = min(kc - n + r + 1, k_end);
    }
    return v;
}

template <int MASK>
__device__ __forceinline__ bool row_sees(int key, int lim, int tb, uint64_t anc)
{
    if constexpr (MASK == TF_MASK_TREE)
        return key < lim && (key < tb || ((anc >> ((key - tb) & 63)) & 1ull) != 0);
    else
        return key < lim;
}

// Query vectors per kv head above which a segment is served by the MFMA
// kernel (prompt chunks, long verify rounds); at or below, by the VALU kernel.
constexpr int kMfmaMinQ = 4;

// Loads through the global address space.  Pointers that come out of the
// segment table are generic; read through them directly the compiler emits
// flat loads, which count against both the vector-memory and the LDS/scalar
// wait counters and make it wait for every load in flight (including
// prefetched ones) before the first use of any.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T load_global(const void *p)
{
    return *reinterpret_cast<const __attribute__((address_space(1))) T *>(
        reinterpret_cast<uintptr_t>(p));
}

// Streaming load (non-temporal hint): K/V rows are read once per launch.
template <typename T>
__device__ __forceinline__ T load_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) T *>(
        reinterpret_cast<uintptr_t>(p)));
}

// v_dot2_f32_bf16: a.x*b.x + a.y*b.y + c with fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two floats to a packed bf16 pair (low half a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2_t v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Exact widening of the low / high bf16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN -> canonical NaN.
__device__ __forceinline__ uint16_t bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return kBf16NaN;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Output rule: a nonfinite value is written as NaN.
__device__ __forceinline__ uint16_t bf16_out(float x)
{
    return __builtin_isfinite(x) ? bf16_rne(x) : kBf16NaN;
}

// max / min as one v_med3_f32 (median of x, y and +-inf).  fmaxf / fminf
// compile to v_max / v_min plus a canonicalising v_max x, x on each input,
// three instructions; here NaN behaviour is irrelevant (a NaN score is
// caught through the softmax sum).
__device__ __forceinline__ float max2(float x, float y) { return __builtin_amdgcn_fmed3f(x, y, INFINITY); }
__device__ __forceinline__ float min2(float x, float y) { return __builtin_amdgcn_fmed3f(x, y, -INFINITY); }

// Cross-row lane exchanges (gfx950): v_permlane16_swap / v_permlane32_swap
// on two copies of x give, summed (or maxed), x combined with the lane 16
// (resp. 32) apart, in every lane.
__device__ __forceinline__ void swap16(float x, float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    a = __int_as_float(r[0]);
    b = __int_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    a = __int_as_float(r[0]);
    b = __int_as_float(r[1]);
}

// v_exp_f32 (2^x).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutation inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Lane rotation by 8 inside a 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float ror8(float x) { return dpp<0x128>(x); }

// Sum over the 16 lanes of a DPP row; every lane of the row receives it.
// quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// Online-softmax state merge (base-2 units): (m, l, o) <- (m, l, o) (+) (mb, lb, ob).
// An empty state is (-inf, 0, 0); two empties stay empty.
__device__ __forceinline__ void merge_scales(float m, float mb, float &mn, float &fa, float &fb)
{
    mn = fmaxf(m, mb);
    const float ms = (mn == -INFINITY) ? 0.0f : mn;
    fa = exp2_fast(m - ms);
    fb = exp2_fast(mb - ms);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which waits for every load and store the wave has in
// flight (a full HBM round trip for the stores just issued).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest kv-head run of a CONTIG / RING buffer, in bytes, that the kernels'
// 32-bit offsets address.
constexpr int64_t kMaxHeadRunBytes = 0xFFFFFFFFll;

// Per-segment checks shared by the rows kernels: the launch's hints and the
// storage kinds' limits.  Returns TF_ERR_* bits (0 = fine).
template <int KIND>
__device__ __forceinline__ int segment_errors(const RowsParams &p, const tf_segment &sd, int head_dim)
{
    int e = 0;
    if (sd.n_rows > p.max_rows || sd.key_count > p.max_keys)
        e |= TF_ERR_HINTS;
    if constexpr (KIND == TF_KV_PAGED) {
        if (sd.pages == nullptr || sd.capacity < 0 ||
            (int64_t)sd.key_count > ((int64_t)sd.capacity << p.page_shift))
            e |= TF_ERR_PAST_PAGES;
    } else {
        if (sd.key_count > sd.capacity)
            e |= TF_ERR_PAST_PAGES;
        if ((int64_t)sd.capacity * head_dim * 2 > kMaxHeadRunBytes)
            e |= TF_ERR_STORAGE;
    }
    if constexpr (KIND == TF_KV_RING) {
        if (sd.first < 0 || sd.first >= sd.capacity)
            e |= TF_ERR_BAD_RING;
    }
    return e;
}

__device__ __forceinline__ void report(int32_t *err, int bits)
{
    if (err != nullptr && bits != 0)
        atomicOr(err, bits);
}

}  // namespace tfa
