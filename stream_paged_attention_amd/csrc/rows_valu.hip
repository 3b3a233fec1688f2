// tf_attn_rows, VALU path: decode and verify rows over paged, ring or
// contiguous K/V (gfx950, wave64).
//
// Work item = one workgroup = (segment, kv head g, split t).  It serves every
// query vector of the segment that reads kv head g: its n_rows rows times
// the group's Hq/Hkv query heads (TensorFold PR #1503: one launch serves all
// streams' rows from the segment table; PR #1562: each row's ring, slots and
// segment come from the table).
//
// Inside a work item the split's keys are cut into tiles of TK keys (one
// tile never crosses a page: pages hold whole tiles, PR #1653).  Wave w
// takes tiles w, w+4, w+8, ...  A wave step covers 4 keys: lanes 16*kg ..
// 16*kg+15 hold key kg, each lane D/16 of its dimensions, loaded straight
// from HBM with 8- or 16-byte loads so that one wave load instruction reads
// 4 whole consecutive key rows (1 KB at D = 128).  The next tile's loads are
// issued before the current tile is folded (the ring's slot groups in flight
// one ahead, PR #1562).  The page id of every tile a wave will read is
// fetched once, one lane per tile, and taken out with readlane (the per-chunk
// page lookup hoisted out of the key loop, PR #1653).
//
// Scores: v_dot2_f32_bf16 on packed bf16 pairs, then a 16-lane DPP row sum.
// Each 16-lane key group keeps its own online-softmax state (max, sum, o)
// per query vector; at the end the four key groups of a wave are merged with
// lane shuffles and the four waves through LDS, always in the same order, so
// the bits of a (row, head) depend only on its own segment.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Tile shape.  Each lane holds 64 bytes of a tile's K (and 64 of its V):
// a wave's K tile is 4 KB (16 keys at D = 128, 8 at D = 256, 32 at D = 64),
// half that when a pass serves 8 query vectors, so that two K/V tiles in
// flight, the scores and the accumulators stay in registers.
template <int D, int QT>
struct Geo {
    static constexpr int W = D / 32;                  // packed bf16 pairs per lane per key
    static constexpr int DPL = D / 16;                // dims per lane
    static constexpr int NS_BASE = 512 / D;           // wave steps (4 keys each) at 64 B / lane
    static constexpr int NS = (QT <= 4 || NS_BASE == 1) ? NS_BASE : NS_BASE / 2;
    static constexpr int TK = 4 * NS;                 // keys per tile
};

// Dimension held by lane sub-index sl in pair w, half hh (K, V, q and o agree).
template <int D>
__device__ __forceinline__ int lane_dim(int sl, int w, int hh)
{
    if constexpr (D == 64)
        return sl * 4 + 2 * w + hh;
    else if constexpr (D == 128)
        return sl * 8 + 2 * w + hh;
    else
        return (w >> 2) * 128 + sl * 8 + 2 * (w & 3) + hh;
}

template <int D>
__device__ __forceinline__ void load_row(uint32_t (&r)[D / 32], const uint16_t *row, int sl)
{
    if constexpr (D == 64) {
        const uint2 x = *reinterpret_cast<const uint2 *>(row + sl * 4);
        r[0] = x.x;
        r[1] = x.y;
    } else if constexpr (D == 128) {
        const uint4 x = *reinterpret_cast<const uint4 *>(row + sl * 8);
        r[0] = x.x;
        r[1] = x.y;
        r[2] = x.z;
        r[3] = x.w;
    } else {
        const uint4 x = *reinterpret_cast<const uint4 *>(row + sl * 8);
        const uint4 y = *reinterpret_cast<const uint4 *>(row + 128 + sl * 8);
        r[0] = x.x;
        r[1] = x.y;
        r[2] = x.z;
        r[3] = x.w;
        r[4] = y.x;
        r[5] = y.y;
        r[6] = y.z;
        r[7] = y.w;
    }
}

// Store the lane's D/16 fp32 values (in lane_dim order) at dst[lane_dim(..)].
template <int D>
__device__ __forceinline__ void store_f32(float *dst, const float (&o)[D / 16], int sl)
{
    if constexpr (D == 64) {
        *reinterpret_cast<float4 *>(dst + sl * 4) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
        for (int c = 0; c < D / 128; ++c) {
            float *p = dst + c * 128 + sl * 8;
            *reinterpret_cast<float4 *>(p) = make_float4(o[8 * c], o[8 * c + 1], o[8 * c + 2], o[8 * c + 3]);
            *reinterpret_cast<float4 *>(p + 4) =
                make_float4(o[8 * c + 4], o[8 * c + 5], o[8 * c + 6], o[8 * c + 7]);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_bf16(uint16_t *dst, const float (&x)[D / 16], int sl)
{
    uint32_t w[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
        w[i] = (uint32_t)bf16_out(x[2 * i]) | ((uint32_t)bf16_out(x[2 * i + 1]) << 16);
    if constexpr (D == 64) {
        *reinterpret_cast<uint2 *>(dst + sl * 4) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
        for (int c = 0; c < D / 128; ++c)
            *reinterpret_cast<uint4 *>(dst + c * 128 + sl * 8) =
                make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    }
}

struct Seg {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *pages;
    int capacity, first, row_offset, n_rows, key_count, partial_offset;
};

// Element offset of this lane's key row for wave step j of a tile.  PAGED:
// the tile lies inside one page, so every row of it is in bounds.  CONTIG
// and RING: keys past the last one are clamped to it (in bounds; the fold
// ignores them).  RING: slot = first + key, wrapped by one compare-and-
// subtract (first < slots and key < key_count <= slots).
template <int D, int KIND>
struct Addr {
    size_t base;   // PAGED: offset of key (tile_k0 + kg); CONTIG: kv head's row 0
    size_t head;   // RING: offset of the kv head's slot 0
    int first;     // CONTIG / RING: key (tile_k0 + kg)
    int last;      // CONTIG / RING: last valid key
    int ring0;     // RING: slot of logical key 0
    int cap;

    __device__ __forceinline__ size_t at(int j) const
    {
        if constexpr (KIND == TF_KV_PAGED) {
            return base + (size_t)(4 * j) * D;
        } else if constexpr (KIND == TF_KV_CONTIG) {
            return base + (size_t)min(first + 4 * j, last) * D;
        } else {
            int slot = ring0 + min(first + 4 * j, last);
            slot -= (slot >= cap) ? cap : 0;
            return head + (size_t)slot * D;
        }
    }
};

// Fold one K/V tile into the key group's online-softmax state.  key0 is the
// lane's first key; with MASKED, key key0 + 4j counts for query vector v only
// below lim[v] (causal limit and split end) and then contributes exactly
// nothing, not even a NaN from its value.  chk[v] turns NaN as soon as a
// counted score is NaN or +-Inf (x * 0 is NaN exactly for those).
template <int D, int QT, bool MASKED>
__device__ __forceinline__ void fold_tile(const uint32_t (&kb)[Geo<D, QT>::NS][Geo<D, QT>::W],
                                          const uint32_t (&vb)[Geo<D, QT>::NS][Geo<D, QT>::W],
                                          const uint32_t (&qr)[QT][Geo<D, QT>::W], float c_log2,
                                          float (&m)[QT], float (&l)[QT],
                                          float (&o)[QT][Geo<D, QT>::DPL], float (&chk)[QT],
                                          int key0, const int (&lim)[QT])
{
    constexpr int NS = Geo<D, QT>::NS, W = Geo<D, QT>::W, DPL = Geo<D, QT>::DPL;
    float s[QT][NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            float a = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w)
                a = dot2_bf16(qr[v][w], kb[j][w], a);
            s[v][j] = row16_sum(a) * c_log2;
        }
    }
#pragma unroll
    for (int v = 0; v < QT; ++v) {
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            float x = s[v][j];
            if constexpr (MASKED) {
                const bool vis = key0 + 4 * j < lim[v];
                chk[v] = fmaf(vis ? x : 0.0f, 0.0f, chk[v]);
                x = vis ? x : -INFINITY;
                s[v][j] = x;
            } else {
                chk[v] = fmaf(x, 0.0f, chk[v]);
            }
            mt = fmaxf(mt, x);
        }
        const float mn = fmaxf(m[v], mt);
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        const float alpha = exp2_fast(m[v] - ms);
        m[v] = mn;
        l[v] *= alpha;
#pragma unroll
        for (int d = 0; d < DPL; ++d)
            o[v][d] *= alpha;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const float p = exp2_fast(s[v][j] - ms);
            l[v] += p;
            s[v][j] = p;
        }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float vf[DPL];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            vf[2 * w] = bf16_lo(vb[j][w]);
            vf[2 * w + 1] = bf16_hi(vb[j][w]);
        }
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            if constexpr (MASKED) {
                if (key0 + 4 * j < lim[v]) {
#pragma unroll
                    for (int d = 0; d < DPL; ++d)
                        o[v][d] = fmaf(s[v][j], vf[d], o[v][d]);
                }
            } else {
#pragma unroll
                for (int d = 0; d < DPL; ++d)
                    o[v][d] = fmaf(s[v][j], vf[d], o[v][d]);
            }
        }
    }
}

template <int D, int KIND, int QT>
__global__ __launch_bounds__(kThreads) void rows_valu_kernel(RowsParams p)
{
    constexpr int W = Geo<D, QT>::W, DPL = Geo<D, QT>::DPL, TK = Geo<D, QT>::TK, NS = Geo<D, QT>::NS;
    __shared__ float xw[kWaves][QT][D + 4];

    const int seg_i = blockIdx.x / p.n_split_max;
    const int t = blockIdx.x % p.n_split_max;
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kg = lane >> 4;
    const int sl = lane & 15;

    const tf_segment &sd = p.segs[seg_i];
    Seg s;
    s.k = static_cast<const uint16_t *>(sd.k);
    s.v = static_cast<const uint16_t *>(sd.v);
    s.pages = sd.pages;
    s.capacity = sd.capacity;
    s.first = sd.first;
    s.row_offset = sd.row_offset;
    s.n_rows = sd.n_rows;
    s.key_count = sd.key_count;
    s.partial_offset = sd.partial_offset;

    // ---- per-segment checks (identical in every work item of the segment)
    int errbits = 0;
    const bool rows_ok = s.n_rows >= 1 && s.n_rows <= s.key_count && s.row_offset >= 0 &&
                         (int64_t)s.row_offset + s.n_rows <= p.total_rows;
    if (!rows_ok) {
        // no row of this segment can be addressed safely: report and write nothing
        if (threadIdx.x == 0 && g == 0 && t == 0)
            report(p.err, TF_ERR_BAD_ROWS);
        return;
    }
    if constexpr (KIND == TF_KV_PAGED) {
        if (s.pages == nullptr || s.capacity < 0 ||
            (int64_t)s.key_count > ((int64_t)s.capacity << p.page_shift))
            errbits |= TF_ERR_PAST_PAGES;
    } else {
        if (s.key_count > s.capacity)
            errbits |= TF_ERR_PAST_PAGES;
    }
    if constexpr (KIND == TF_KV_RING) {
        if (s.first < 0 || s.first >= s.capacity)
            errbits |= TF_ERR_BAD_RING;
    }
    const int kc = s.key_count > 0 ? s.key_count : 1;
    const int n_splits = p.split_keys > 0 ? (kc + p.split_keys - 1) / p.split_keys : 1;
    if (t >= n_splits)
        return;   // block-uniform: this grid cell has no split of this segment
    bool parts_ok = true;
    if (p.split_keys > 0) {
        const int64_t need = (int64_t)s.n_rows * p.hq * n_splits;
        parts_ok = s.partial_offset >= 0 && (int64_t)s.partial_offset + need <= p.max_records;
        if (!parts_ok)
            errbits |= TF_ERR_PARTIALS;
    }

    const int group = p.group;
    const int nq = s.n_rows * group;
    const int k0 = p.split_keys > 0 ? t * p.split_keys : 0;
    const int k_end = p.split_keys > 0 ? min(k0 + p.split_keys, s.key_count) : s.key_count;
    const int n_tiles = errbits ? 0 : (k_end - k0 + TK - 1) / TK;
    const int my_tiles = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;

    for (int qt0 = 0; qt0 < nq; qt0 += QT) {
        // ---- query vectors of this tile: v -> (row r, head h)
        uint32_t qr[QT][W];
        int lim[QT];
        float m[QT], l[QT], o[QT][DPL];
        float chk[QT];   // NaN once a counted score was not finite
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            const int qv = qt0 + v;
            const int r = qv / group;
            const int h = g * group + qv % group;
            m[v] = -INFINITY;
            l[v] = 0.0f;
            chk[v] = 0.0f;
#pragma unroll
            for (int d = 0; d < DPL; ++d)
                o[v][d] = 0.0f;
            if (qv < nq) {
                load_row<D>(qr[v], p.q + ((size_t)(s.row_offset + r) * p.hq + h) * D, sl);
                lim[v] = min(s.key_count - s.n_rows + r + 1, k_end);
            } else {
#pragma unroll
                for (int w = 0; w < W; ++w)
                    qr[v][w] = 0u;
                lim[v] = 0;
            }
        }
        int lim_min = lim[0];
#pragma unroll
        for (int v = 1; v < QT; ++v)
            if (qt0 + v < nq)
                lim_min = min(lim_min, lim[v]);

        // ---- key tiles of this wave, double-buffered
        bool page_bad = false;
        int pid = 0;
        auto tile_key0 = [&](int i) { return k0 + (wave + kWaves * i) * TK; };
        auto setup = [&](int i) {
            Addr<D, KIND> a;
            const int key = tile_key0(i) + kg;
            a.cap = s.capacity;
            if constexpr (KIND == TF_KV_PAGED) {
                if ((i & 63) == 0) {
                    const int ti = i + lane;
                    pid = ti < my_tiles ? s.pages[tile_key0(ti) >> p.page_shift] : 0;
                }
                int page = __builtin_amdgcn_readlane(pid, i & 63);
                if ((unsigned)page >= (unsigned)p.pool_pages) {
                    page_bad = true;
                    page = 0;
                }
                a.base = (((size_t)page * p.hkv + g) * p.page_size + (key & (p.page_size - 1))) * D;
            } else if constexpr (KIND == TF_KV_CONTIG) {
                a.base = (size_t)g * s.capacity * D;
                a.first = key;
                a.last = s.key_count - 1;
            } else {
                a.head = (size_t)g * s.capacity * D;
                a.first = key;
                a.last = s.key_count - 1;
                a.ring0 = s.first;
            }
            return a;
        };
        // Loads are unconditional: a key at or past k_end is read from an
        // in-bounds address (its own page for PAGED, the last key for
        // CONTIG/RING) and then excluded by the masked fold, which never
        // lets such a key's score or value reach the state.
        auto load_tile = [&](uint32_t (&kb)[NS][W], uint32_t (&vb)[NS][W], int i) {
            const Addr<D, KIND> a = setup(i);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const size_t off = a.at(j);
                load_row<D>(kb[j], s.k + off, sl);
                load_row<D>(vb[j], s.v + off, sl);
            }
        };
        // Full tiles (every key visible to every query vector of the pass)
        // come first in key order; the masked tail (split end, causal rows)
        // is folded by a separate loop so that the fast loop carries no
        // per-key masks.
        const int n_full = max(0, min(n_tiles, (lim_min - k0) / TK));
        const int my_full = n_full > wave ? (n_full - wave + kWaves - 1) / kWaves : 0;
        for (int i = 0; i < my_full; ++i) {
            uint32_t kb[NS][W], vb[NS][W];
            load_tile(kb, vb, i);
            fold_tile<D, QT, false>(kb, vb, qr, p.c_log2, m, l, o, chk, tile_key0(i) + kg, lim);
        }
        for (int i = my_full; i < my_tiles; ++i) {
            uint32_t kb[NS][W], vb[NS][W];
            load_tile(kb, vb, i);
            fold_tile<D, QT, true>(kb, vb, qr, p.c_log2, m, l, o, chk, tile_key0(i) + kg, lim);
        }
        if (page_bad) {
            if (lane == 0)
                report(p.err, TF_ERR_BAD_PAGE);
#pragma unroll
            for (int v = 0; v < QT; ++v)
                chk[v] = NAN;
        }

        // ---- merge the four key groups of the wave (lanes l, l^16, l^32, l^48)
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
            for (int v = 0; v < QT; ++v) {
                const float mb = __shfl_xor(m[v], off);
                const float lb = __shfl_xor(l[v], off);
                const float cb = __shfl_xor(chk[v], off);
                float mn, fa, fb;
                merge_scales(m[v], mb, mn, fa, fb);
                m[v] = mn;
                l[v] = l[v] * fa + lb * fb;
                chk[v] += cb;
#pragma unroll
                for (int d = 0; d < DPL; ++d) {
                    const float ob = __shfl_xor(o[v][d], off);
                    o[v][d] = o[v][d] * fa + ob * fb;
                }
            }
        }

        // ---- every wave parks its state in LDS; then all threads finalise
        // (query vector, dimension pairs), merging the waves in wave order
        if (lane < 16) {
#pragma unroll
            for (int v = 0; v < QT; ++v) {
                float *rec = xw[wave][v];
                if (lane == 0) {
                    rec[0] = m[v];
                    rec[1] = l[v];
                    rec[2] = chk[v];
                }
                store_f32<D>(rec + 4, o[v], sl);
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < QT * (D / 2); e += kThreads) {
            const int v = e / (D / 2);
            const int d = 2 * (e % (D / 2));
            const int qv = qt0 + v;
            if (qv >= nq)
                break;   // e only grows with v
            float mm = xw[0][v][0], ll = xw[0][v][1], cc = xw[0][v][2];
            float o0 = xw[0][v][4 + d], o1 = xw[0][v][5 + d];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                float mn, fa, fb;
                merge_scales(mm, xw[w][v][0], mn, fa, fb);
                mm = mn;
                ll = ll * fa + xw[w][v][1] * fb;
                cc += xw[w][v][2];
                o0 = o0 * fa + xw[w][v][4 + d] * fb;
                o1 = o1 * fa + xw[w][v][5 + d] * fb;
            }
            const int r = qv / group;
            const int h = g * group + qv % group;
            const bool nan_out = __builtin_isnan(cc) || errbits != 0;
            if (p.split_keys > 0) {
                if (!parts_ok)
                    continue;
                const int64_t recno = s.partial_offset + ((int64_t)r * p.hq + h) * n_splits + t;
                float *rec = p.partials + recno * (D + 4);
                if (d == 0)
                    *reinterpret_cast<float4 *>(rec) =
                        make_float4(nan_out ? NAN : mm * kLn2, nan_out ? NAN : ll, 0.0f, 0.0f);
                *reinterpret_cast<float2 *>(rec + 4 + d) =
                    make_float2(nan_out ? NAN : o0, nan_out ? NAN : o1);
            } else {
                const uint32_t b0 = nan_out ? kBf16NaN : bf16_out(o0 / ll);
                const uint32_t b1 = nan_out ? kBf16NaN : bf16_out(o1 / ll);
                *reinterpret_cast<uint32_t *>(p.out + ((size_t)(s.row_offset + r) * p.hq + h) * D + d) =
                    b0 | (b1 << 16);
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0 && g == 0 && t == 0)
        report(p.err, errbits);
}

// Query vectors per pass: 4, or 8 when a segment can have more than 4 (not
// at D = 256, where 8 would not fit in registers).  Each query vector's
// arithmetic is the same whatever the pass width.
template <int D, int KIND>
hipError_t launch_qt(const RowsParams &p, int qt, dim3 grid, hipStream_t st)
{
    if constexpr (D == 256) {
        hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 4>), grid, dim3(kThreads), 0, st, p);
    } else {
        if (qt <= 4)
            hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 4>), grid, dim3(kThreads), 0, st, p);
        else
            hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 8>), grid, dim3(kThreads), 0, st, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_kind(const RowsParams &p, int kind, int qt, dim3 grid, hipStream_t st)
{
    switch (kind) {
    case TF_KV_CONTIG:
        return launch_qt<D, TF_KV_CONTIG>(p, qt, grid, st);
    case TF_KV_PAGED:
        return launch_qt<D, TF_KV_PAGED>(p, qt, grid, st);
    default:
        return launch_qt<D, TF_KV_RING>(p, qt, grid, st);
    }
}

}  // namespace

// Launch the VALU rows kernel; grid = (n_segments * n_split_max, n_kv_heads).
hipError_t launch_rows_valu(const RowsParams &p, int head_dim, int kind, int qt, hipStream_t st)
{
    const dim3 grid((unsigned)(p.n_segments * p.n_split_max), (unsigned)p.hkv);
    switch (head_dim) {
    case 64:
        return launch_kind<64>(p, kind, qt, grid, st);
    case 128:
        return launch_kind<128>(p, kind, qt, grid, st);
    default:
        return launch_kind<256>(p, kind, qt, grid, st);
    }
}

}  // namespace tfa
