// tf_attn_rows, VALU path: decode and verify rows over paged, ring or
// contiguous K/V (gfx950, wave64).
//
// Work item = one workgroup = (segment, kv head g, split t).  It serves every
// query vector of the segment that reads kv head g: its n_rows rows times
// the group's Hq/Hkv query heads (TensorFold PR #1503: one launch serves all
// streams' rows from the segment table; PR #1562: a packed row finds its
// ring and slot count through the table).
//
// Inside a work item the split's keys are cut into tiles of TK keys (a tile
// never crosses a page: pages hold whole tiles, PR #1653).  Wave w takes
// tiles w, w+4, w+8, ...  A wave step covers 64/LPK keys: the LPK lanes of a
// key group hold one key, D/LPK of its dimensions each, loaded straight from
// HBM with 16-byte loads so that one wave load instruction reads whole
// 128-byte lines of consecutive keys.  The next tile's loads are issued
// before the current tile is folded (the ring's slot groups in flight one
// ahead, PR #1562).  The page id of every tile a wave will read is fetched
// once, one lane per tile, and taken out with readlane (PR #1653 likewise
// looks a page id up once per chunk, not once per key).
//
// Scores: v_dot2_f32_bf16 on packed bf16 pairs, then a DPP sum over the key
// group.  Online softmax per query vector with a wave-wide reference m (raw
// score units): weights are 2^((s - m) c), c = scale * log2(e), summed into
// l and, times v, into o per key group.  The reference is raised only when a
// score exceeds it by more than 8 / c (so weights stay <= 2^8), decided for
// the whole wave at once and set to the wave's max, so most tiles need no
// rescale and every key group of a wave shares m: at the end their l and o
// are plain sums (DPP and lane-swap exchanges), the waves are merged through
// LDS in wave order, and the bits of a (row, head) depend only on its own
// segment.  Each lane also keeps the smallest counted score, to see a -inf.
#include "device.hpp"

namespace tfa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 8.0f;   // log2 of the largest weight a stale reference may give

// Shape of one pass: LPK lanes per key, DPL dims per lane, NS wave steps of
// KPS keys per tile, CH tiles in flight per wave.  8 lanes per key where the
// accumulators fit (3 DPP steps per 8 keys: D 64 and 128), 16 at D 256.
template <int D, int QT>
struct Geo {
    static constexpr int LPK = D == 256 ? 16 : 8;
    static constexpr int KPS = 64 / LPK;              // keys per wave step
    static constexpr int DPL = D / LPK;               // dims per lane
    static constexpr int W = DPL / 2;                 // packed bf16 pairs per lane per key
    static constexpr int NS = (DPL <= 8) ? 2 : 1;     // wave steps per tile
    static constexpr int TK = NS * KPS;               // keys per tile
    // Key pairs (8 lanes a key: D 64 and 128): the key groups 2i and 2i+1 of
    // a 16-lane row hold adjacent keys; each lane of the pair loads the same
    // half of both keys' values and accumulates that half of the output over
    // both keys with one v_dot2_f32_bf16 per dim pair, the weights rounded
    // to bf16 (fp32 sums).  The output accumulators halve, which pays for
    // more tiles in flight.
    static constexpr bool PAIR = LPK == 8;
    static constexpr int OPL = PAIR ? DPL / 2 : DPL;  // output dims accumulated per lane
    static constexpr int WV = PAIR ? W / 2 : W;       // value registers per key and step
    static constexpr int CH = PAIR ? 3 : 2;           // tiles in flight per wave
    // Partial sums parked in LDS per wave and query vector: one per 16-lane
    // row (R = 4), or per row pair / per wave (R = 2, 1) where 4 would not
    // fit in 32 KB per workgroup.
    static constexpr int R4_BYTES = kWaves * QT * 4 * D * 4;
    static constexpr int R = R4_BYTES <= 32768 ? 4 : (R4_BYTES / 2 <= 32768 ? 2 : 1);
    static_assert(DPL == 4 || DPL % 8 == 0, "lane slice must be 8 bytes or whole 16-byte chunks");
    static_assert(!PAIR || (R == 4 && OPL % 4 == 0), "pair mode keeps one output row per 16 lanes");
};

// Dimension of element e (0 .. DPL-1) of lane sub-index sl: 16-byte chunk c
// covers dims c*8*LPK + sl*8 .. +8, so a chunk's load reads 8*LPK contiguous
// dims (one or more whole 128-byte lines) across the key group.
template <int D, int QT>
__device__ __forceinline__ int lane_dim(int sl, int e)
{
    using G = Geo<D, QT>;
    if constexpr (G::DPL == 4)
        return sl * 4 + e;
    else
        return (e >> 3) * (8 * G::LPK) + sl * 8 + (e & 7);
}

// Dimension of output element i (0 .. OPL-1) of a lane in the pair mode:
// the even lane of a pair keeps the first half of its slice (16-byte chunk
// 0 at D 128, the first 8 bytes at D 64), the odd lane the second half.
template <int D, int QT>
__device__ __forceinline__ int pair_dim(int sl, int odd, int i)
{
    using G = Geo<D, QT>;
    if constexpr (G::DPL == 8)
        return sl * 8 + odd * 4 + i;
    else
        return odd * (8 * G::LPK) + sl * 8 + i;
}

// Byte offset, within a key row, of the half slice a pair-mode lane keeps.
template <int D, int QT>
__device__ __forceinline__ uint32_t pair_lane_bytes(int sl, int odd)
{
    using G = Geo<D, QT>;
    if constexpr (G::DPL == 8)
        return (uint32_t)(sl * 16 + odd * 8);
    else
        return (uint32_t)(odd * 16 * G::LPK + sl * 16);
}

// Load the kept half slice (WV registers) of one value row.
template <int D, int QT>
__device__ __forceinline__ void load_half(uint32_t *r, const char *base, uint32_t off)
{
    using G = Geo<D, QT>;
    if constexpr (G::WV == 2) {
        const u32x2_t x = load_stream<u32x2_t>(base + off);
        r[0] = x.x;
        r[1] = x.y;
    } else {
        static_assert(G::WV == 4, "a half slice is 8 or 16 bytes");
        const u32x4_t x = load_stream<u32x4_t>(base + off);
        r[0] = x.x;
        r[1] = x.y;
        r[2] = x.z;
        r[3] = x.w;
    }
}

// Load the lane's slice of one key row: base is uniform across the wave
// (SGPR pair), off a 32-bit byte offset, so the loads use the global
// SGPR-base form with immediate offsets for the chunks.
template <int D, int QT, bool STREAM = false>
__device__ __forceinline__ void load_row(uint32_t *r, const char *base, uint32_t off)
{
    using G = Geo<D, QT>;
    if constexpr (G::DPL == 4) {
        const u32x2_t x = STREAM ? load_stream<u32x2_t>(base + off) : load_global<u32x2_t>(base + off);
        r[0] = x.x;
        r[1] = x.y;
    } else {
#pragma unroll
        for (int c = 0; c < G::DPL / 8; ++c) {
            const char *a = base + off + c * 16 * G::LPK;
            const u32x4_t x = STREAM ? load_stream<u32x4_t>(a) : load_global<u32x4_t>(a);
            r[4 * c] = x.x;
            r[4 * c + 1] = x.y;
            r[4 * c + 2] = x.z;
            r[4 * c + 3] = x.w;
        }
    }
}

template <int D, int QT>
__device__ __forceinline__ void store_f32(float *dst, const float *o, int sl)
{
    using G = Geo<D, QT>;
    if constexpr (G::DPL == 4) {
        *reinterpret_cast<float4 *>(dst + sl * 4) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
        for (int c = 0; c < G::DPL / 8; ++c) {
            float *p = dst + c * 8 * G::LPK + sl * 8;
            *reinterpret_cast<float4 *>(p) = make_float4(o[8 * c], o[8 * c + 1], o[8 * c + 2], o[8 * c + 3]);
            *reinterpret_cast<float4 *>(p + 4) =
                make_float4(o[8 * c + 4], o[8 * c + 5], o[8 * c + 6], o[8 * c + 7]);
        }
    }
}

// acc + a.lo * b.lo + a.hi * b.hi in the three-address form (VOP3), so that
// a long-lived accumulator need not share its register with the result
// (the two-address v_dot2c form made the compiler copy the accumulators)
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc)
{
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(acc));
    return r;
}

template <int D, int QT>
__device__ __forceinline__ void store_pair_f32(float *dst, const float *o, int sl, int odd)
{
    using G = Geo<D, QT>;
    float *p = dst + pair_dim<D, QT>(sl, odd, 0);
#pragma unroll
    for (int i = 0; i < G::OPL; i += 4)
        *reinterpret_cast<float4 *>(p + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
}

// Sum over the LPK lanes of a key group (DPP: quad swaps, half-row mirror,
// row mirror); every lane of the group receives the sum.
template <int LPK>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    if constexpr (LPK == 16)
        x += dpp<0x140>(x);
    return x;
}

struct Seg {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *pages;
    int capacity, first, row_offset, n_rows, key_count, partial_offset;
};

// Where wave step j of a tile reads this lane's key row: a uniform base
// (the kv head's run inside the tile's page, or the head's row 0 / slot 0)
// plus a 32-bit byte offset.  PAGED: the tile lies inside one page, so every
// row is in bounds.  CONTIG and RING: keys past the last one are clamped to
// it (in bounds; the masked fold ignores them).  RING: slot = first + key,
// wrapped by one compare-and-subtract (first < slots, key < key_count <= slots).
template <int D, int QT, int KIND>
struct Addr {
    const char *kbase;
    const char *vbase;
    uint32_t off0;   // PAGED: byte offset of the lane's first row and slice
    int first;       // CONTIG / RING: the lane's first key
    int last;        // CONTIG / RING: last valid key
    int ring0;       // RING: slot of logical key 0
    int cap;
    uint32_t lane_b; // byte offset of the lane's slice within a row
    int delta;       // pair mode: the partner key is this lane's key + delta (+-1)
    uint32_t lane_v; // pair mode: byte offset of the kept half slice within a row

    // row of the lane's key (dk = 0) or its partner's (dk = delta) at wave
    // step j, plus the byte offset b within the row
    __device__ __forceinline__ uint32_t row_at(int j, int dk, uint32_t b) const
    {
        constexpr int KPS = Geo<D, QT>::KPS;
        constexpr uint32_t ROW = D * 2;
        if constexpr (KIND == TF_KV_PAGED) {
            // pairs (2i, 2i+1) never straddle a page
            return off0 + (uint32_t)(KPS * j + dk) * ROW + b;
        } else if constexpr (KIND == TF_KV_CONTIG) {
            return (uint32_t)min(first + dk + KPS * j, last) * ROW + b;
        } else {
            int slot = ring0 + min(first + dk + KPS * j, last);
            slot -= (slot >= cap) ? cap : 0;
            return (uint32_t)slot * ROW + b;
        }
    }
    __device__ __forceinline__ uint32_t at(int j) const { return row_at(j, 0, lane_b); }
};

__device__ __forceinline__ float uniform(float x)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Per-query-vector online-softmax state.  m, mc and thr are the same in
// every lane of the wave; lo, l and o belong to the lane's key group.
template <int D, int QT>
struct State {
    float m[QT];    // reference max (raw score units), -inf before the first score
    float mc[QT];   // m * c, or 0 while m is -inf
    float thr[QT];  // m + 8 / c: a score above it raises the reference
    float lo[QT];   // min of the counted scores (-inf flags a -inf score)
    float l[QT];
    float o[QT][Geo<D, QT>::OPL];
};

// max / min as a single v_max_f32 / v_min_f32: the compiler's versions for
// values of unknown origin add a canonicalising v_max on each input
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmin(float a, float b)
{
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Combine a value over the key groups of the wave (lanes LPK apart), result
// in every lane.
template <int LPK>
__device__ __forceinline__ float groups_max(float x)
{
    float a, b;
    if constexpr (LPK == 8)
        x = vmax(x, ror8(x));
    swap16(x, a, b);
    x = vmax(a, b);
    swap32(x, a, b);
    return vmax(a, b);
}

// Fold one K/V tile.  key0 is the lane's first key.  With MASKED, key
// key0 + KPS*j counts for query vector v only below lim[v] (mask limit and
// split end) and, under a tree mask, when it is the row's or an ancestor's
// (row_sees); a key that does not
// count adds exactly nothing, not even a NaN from its value.
template <int D, int QT, bool MASKED, int MASK>
__device__ __forceinline__ void fold_tile(const uint32_t (&kb)[Geo<D, QT>::NS][Geo<D, QT>::W],
                                          const uint32_t (&vb)[Geo<D, QT>::NS][Geo<D, QT>::W],
                                          const uint32_t (&qr)[QT][Geo<D, QT>::W], float c,
                                          float lazy, State<D, QT> &st, int key0, int delta,
                                          const int (&lim)[QT], int tb, const uint64_t (&anc)[QT])
{
    using G = Geo<D, QT>;
    constexpr int NS = G::NS, W = G::W, DPL = G::DPL, KPS = G::KPS, OPL = G::OPL;
    float s[QT][NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            // first product in the three-operand form with an inline 0
            // (the two-operand form would need a register zeroed first)
            float a;
            asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(a) : "v"(qr[v][0]), "v"(kb[j][0]));
#pragma unroll
            for (int w = 1; w < W; ++w)
                a = dot2_bf16(qr[v][w], kb[j][w], a);
            s[v][j] = group_sum<G::LPK>(a);
        }
    }
    // need: lanes holding a score above its reference's threshold, as a
    // wave mask (each compare writes a lane mask; ORing them is scalar work)
    uint64_t need = 0;
#pragma unroll
    for (int v = 0; v < QT; ++v) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            // the smallest counted score: a -inf score gives p = 0, so it
            // has to be recorded apart (NaN rule)
            if constexpr (MASKED) {
                const int key = key0 + KPS * j;
                const bool vis = row_sees<MASK>(key, lim[v], tb, anc[v]);
                st.lo[v] = vmin(st.lo[v], vis ? s[v][j] : INFINITY);
                s[v][j] = vis ? s[v][j] : -INFINITY;
            } else {
                st.lo[v] = vmin(st.lo[v], s[v][j]);
            }
            need |= __builtin_amdgcn_ballot_w64(s[v][j] > st.thr[v]);
        }
    }
    // raise the reference to the wave's max when some score passed it
    if (need != 0) {
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            float t = s[v][0];
#pragma unroll
            for (int j = 1; j < NS; ++j)
                t = vmax(t, s[v][j]);
            const float tm = uniform(groups_max<G::LPK>(t));
            // only a query vector whose own max passed its reference moves;
            // one that saw nothing (all masked) keeps m = -inf and mc = 0
            const bool up = tm > st.m[v];
            const float alpha = up ? exp2_fast((st.m[v] - tm) * c) : 1.0f;
            // m, m*c and the threshold are wave-uniform: kept in scalar
            // registers (readfirstlane), they cost no vector registers
            st.m[v] = uniform(up ? tm : st.m[v]);
            st.mc[v] = uniform(up ? tm * c : st.mc[v]);
            st.thr[v] = uniform(up ? tm + lazy : st.thr[v]);
            st.l[v] *= alpha;
#pragma unroll
            for (int d = 0; d < OPL; ++d)
                st.o[v][d] *= alpha;
        }
    }
#pragma unroll
    for (int v = 0; v < QT; ++v) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const float p = exp2_fast(fmaf(s[v][j], c, -st.mc[v]));
            st.l[v] += p;
            s[v][j] = p;
        }
    }
    if constexpr (G::PAIR) {
        // value product over the key pair: vb[j][0 .. WV) holds the kept
        // half of this lane's key, vb[j][WV .. W) the same dims of the
        // partner's key; v_perm builds (own, partner) pairs per dim and one
        // v_dot2_f32_bf16 adds both keys' terms with bf16 weights
        constexpr int WV = G::WV;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            uint32_t pa[WV], pb[WV];
#pragma unroll
            for (int w = 0; w < WV; ++w) {
                pa[w] = __builtin_amdgcn_perm(vb[j][WV + w], vb[j][w], 0x05040100u);
                pb[w] = __builtin_amdgcn_perm(vb[j][WV + w], vb[j][w], 0x07060302u);
            }
#pragma unroll
            for (int v = 0; v < QT; ++v) {
                // the partner key's weight (row_ror:8 reads a lane of the
                // same row in every lane, so no old value is needed)
                const float pp = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s[v][j]), 0x128, 0xF, 0xF, true));
                const uint32_t pk = pack_bf16(s[v][j], pp);
                if constexpr (MASKED) {
                    // a key this query vector may not see has weight 0; its
                    // value half is cleared too, so a NaN there cannot leak
                    const int key = key0 + KPS * j;
                    const uint32_t keep =
                        (row_sees<MASK>(key, lim[v], tb, anc[v]) ? 0x0000FFFFu : 0u) |
                        (row_sees<MASK>(key + delta, lim[v], tb, anc[v]) ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int w = 0; w < WV; ++w) {
                        st.o[v][2 * w] = dot2_acc(pk, pa[w] & keep, st.o[v][2 * w]);
                        st.o[v][2 * w + 1] = dot2_acc(pk, pb[w] & keep, st.o[v][2 * w + 1]);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < WV; ++w) {
                        st.o[v][2 * w] = dot2_acc(pk, pa[w], st.o[v][2 * w]);
                        st.o[v][2 * w + 1] = dot2_acc(pk, pb[w], st.o[v][2 * w + 1]);
                    }
                }
            }
        }
    } else {
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
                // a key this query vector may not see has p = 0; its value is
                // replaced by 0 too, so a NaN there cannot leak in
                const int key = key0 + KPS * j;
                const bool vis = row_sees<MASK>(key, lim[v], tb, anc[v]);
#pragma unroll
                for (int d = 0; d < DPL; ++d)
                    st.o[v][d] = fmaf(s[v][j], vis ? vf[d] : 0.0f, st.o[v][d]);
            } else {
#pragma unroll
                for (int d = 0; d < DPL; ++d)
                    st.o[v][d] = fmaf(s[v][j], vf[d], st.o[v][d]);
            }
        }
    }
    }
}

template <int D, int KIND, int QT, int MASK>
__global__ __launch_bounds__(kThreads) void rows_valu_kernel(RowsParams p)
{
    using G = Geo<D, QT>;
    constexpr int W = G::W, DPL = G::DPL, TK = G::TK, NS = G::NS, LPK = G::LPK, CH = G::CH;
    constexpr int R = G::R;
    // per wave, query vector and row group: o[D]; l and the smallest score;
    // per wave and query vector: the reference m
    __shared__ float xo[kWaves][QT][R][D];
    __shared__ float xl[kWaves][QT][R][2];
    __shared__ float xm[kWaves][QT];

    // Work items in dispatch order: kv head fastest, then segment, split
    // slowest.  Consecutive blocks go to different XCDs (round robin), so
    // every XCD gets an even share of each split band; cells past a
    // segment's last split come late and exit at once.
    const int g = blockIdx.x % p.hkv;
    const int seg_i = (blockIdx.x / p.hkv) % p.n_segments;
    const int t = blockIdx.x / (p.hkv * p.n_segments);
    const int lane = threadIdx.x & 63;
    // wave index as a scalar: everything derived from it (tile lists, loop
    // bounds) stays in scalar registers and the loops branch on scalars
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = lane / LPK;
    const int sl = lane % LPK;
    // pair mode: key groups 2i and 2i+1 are partners
    const int odd = kg & 1;
    const int delta = odd ? -1 : 1;
    const uint32_t lane_v = G::PAIR ? pair_lane_bytes<D, QT>(sl, odd) : 0u;

    // the whole row in scalar registers here, in one memory round trip (a
    // copy, so the checks below read registers): left to the compiler, each
    // field was fetched at its first use, one wait after another
    const tf_segment sd = p.segs[seg_i];
    asm volatile("" ::"s"(sd.k), "s"(sd.v), "s"(sd.pages), "s"(sd.capacity), "s"(sd.first), "s"(sd.row_offset),
                 "s"(sd.n_rows), "s"(sd.key_count), "s"(sd.partial_offset));
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

    // segments with many query vectors per kv head go to rows_mfma_kernel
    if (s.n_rows * p.group > p.mfma_min_q)
        return;

    // ---- per-segment checks (identical in every work item of the segment)
    const bool rows_ok = s.n_rows >= 1 && s.n_rows <= s.key_count && s.row_offset >= 0 &&
                         (int64_t)s.row_offset + s.n_rows <= p.total_rows &&
                         (MASK != TF_MASK_TREE || s.n_rows <= 64);
    if (!rows_ok) {
        // no row of this segment can be addressed safely: report and write nothing
        if (threadIdx.x == 0 && g == 0 && t == 0)
            report(p.err, TF_ERR_BAD_ROWS);
        return;
    }
    // hints, storage bounds, ring start; any of them: no key is read and the
    // segment's rows are written as NaN
    int errbits = segment_errors<KIND>(p, sd, D);
    const int n_splits = p.split_keys > 0 ? (s.key_count + p.split_keys - 1) / p.split_keys : 1;
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
    // the scale lives in a VGPR: the exponent's fma then reads only m * c
    // from a scalar register (one scalar operand per VALU instruction)
    float c;
    asm("v_mov_b32 %0, %1" : "=v"(c) : "s"(p.c_log2));
    const float lazy = kLazy / p.c_log2;

    for (int qt0 = 0; qt0 < nq; qt0 += QT) {
        // ---- query vectors of this pass: v -> (row r, head h)
        uint32_t qr[QT][W];
        int lim[QT];
        uint64_t anc[QT];
        int tb = INT32_MAX;   // the segment's first new key under a tree mask
        State<D, QT> st;
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            const int qv = qt0 + v;
            const int r = qv / group;
            const int h = g * group + qv % group;
            st.m[v] = -INFINITY;
            st.mc[v] = 0.0f;
            st.thr[v] = -INFINITY;
            st.lo[v] = INFINITY;
            st.l[v] = 0.0f;
#pragma unroll
            for (int d = 0; d < DPL; ++d)
                st.o[v][d] = 0.0f;
            if (qv < nq) {
                load_row<D, QT>(qr[v], reinterpret_cast<const char *>(p.q) +
                                           ((size_t)(s.row_offset + r) * p.hq + h) * (D * 2),
                                (uint32_t)(sl * (G::DPL == 4 ? 8 : 16)));
                const RowVis rv = row_vis<MASK>(p, s.key_count, s.n_rows, r, s.row_offset, k_end);
                lim[v] = rv.lim;
                anc[v] = rv.anc;
                tb = rv.tb;
            } else {
#pragma unroll
                for (int w = 0; w < W; ++w)
                    qr[v][w] = 0u;
                lim[v] = 0;
                anc[v] = 0;
            }
        }
        // keys below lim_min count for every query vector of the pass
        int lim_min = min(lim[0], tb);
#pragma unroll
        for (int v = 1; v < QT; ++v)
            if (qt0 + v < nq)
                lim_min = min(lim_min, lim[v]);

        // ---- this wave's key tiles
        bool page_bad = false;
        int pid = 0;
        auto tile_key0 = [&](int i) { return k0 + (wave + kWaves * i) * TK; };
        // page ids of this wave's tiles i0 .. i0+63, one lane per tile
        auto load_pids = [&](int i0) {
            if constexpr (KIND == TF_KV_PAGED) {
                const int ti = i0 + lane;
                pid = ti < my_tiles ? load_global<int32_t>(s.pages + (tile_key0(ti) >> p.page_shift)) : 0;
            }
        };
        const uint32_t lane_b = (uint32_t)sl * (G::DPL == 4 ? 8u : 16u);
        auto setup = [&](int i) {
            Addr<D, QT, KIND> a;
            const int key = tile_key0(i) + kg;
            a.cap = s.capacity;
            a.lane_b = lane_b;
            a.delta = delta;
            a.lane_v = lane_v;
            if constexpr (KIND == TF_KV_PAGED) {
                int page = __builtin_amdgcn_readlane(pid, i & 63);
                if ((unsigned)page >= (unsigned)p.pool_pages) {
                    page_bad = true;
                    page = 0;
                }
                const size_t run = ((size_t)page * p.hkv + g) * p.page_size * (D * 2);
                a.kbase = reinterpret_cast<const char *>(s.k) + run;
                a.vbase = reinterpret_cast<const char *>(s.v) + run;
                a.off0 = (uint32_t)(key & (p.page_size - 1)) * (D * 2);
            } else {
                const size_t head = (size_t)g * s.capacity * (D * 2);
                a.kbase = reinterpret_cast<const char *>(s.k) + head;
                a.vbase = reinterpret_cast<const char *>(s.v) + head;
                a.first = key;
                a.last = s.key_count - 1;
                a.ring0 = s.first;
            }
            return a;
        };
        // Loads are unconditional: a key at or past k_end is read from an
        // in-bounds address (its own page for PAGED, the last key for
        // CONTIG/RING) and then excluded by the masked fold.
        auto load_tile = [&](uint32_t (&kb)[NS][W], uint32_t (&vb)[NS][W], int i) {
            const Addr<D, QT, KIND> a = setup(i);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint32_t off = a.at(j);
                load_row<D, QT, true>(kb[j], a.kbase, off);
            }
            if constexpr (G::PAIR) {
                // the kept half of this key's value row, then the same half
                // of the partner key's row
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    load_half<D, QT>(&vb[j][0], a.vbase, a.row_at(j, 0, a.lane_v));
                    load_half<D, QT>(&vb[j][G::WV], a.vbase, a.row_at(j, a.delta, a.lane_v));
                }
            } else {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const uint32_t off = a.at(j);
                    load_row<D, QT, true>(vb[j], a.vbase, off);
                }
            }
            // keep the issue order tile by tile (K, then V): the waits before
            // each fold count loads in issue order
            __builtin_amdgcn_sched_barrier(0);
        };
        // Full tiles (every key visible to every query vector of the pass)
        // come first in key order and run through a rolling pipeline: CH
        // tiles are in flight, and as soon as tile i is folded its registers
        // take the loads of tile i + CH.  Loads past the last full tile
        // repeat it (an L2 hit, never waited for: the barriers below order
        // LDS only) so that every wait before a fold is an exact count in
        // issue order.  The masked tail (split end, causal rows, a tree's block) is folded
        // one tile at a time by its own loop.
        const int n_full = max(0, min(n_tiles, (lim_min - k0) / TK));
        const int my_full = n_full > wave ? (n_full - wave + kWaves - 1) / kWaves : 0;
        for (int b0 = 0; b0 < my_full; b0 += 64) {
            // page ids for this batch first, so no load other than K/V is in
            // flight inside the pipeline (a wait for one would drain it)
            load_pids(b0);
            const int b1 = min(my_full, b0 + 64);
            uint32_t kb[CH][NS][W], vb[CH][NS][W];
#pragma unroll
            for (int u = 0; u < CH; ++u)
                load_tile(kb[u], vb[u], min(b0 + u, b1 - 1));
            // whole groups of CH tiles: no guard inside the hot loop (a
            // guarded fold made the compiler keep two copies of the state)
            int i0 = b0;
            for (; i0 + CH <= b1; i0 += CH) {
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    const int i = i0 + u;
                    fold_tile<D, QT, false, MASK>(kb[u], vb[u], qr, c, lazy, st, tile_key0(i) + kg, delta,
                                                  lim, tb, anc);
                    load_tile(kb[u], vb[u], min(i + CH, b1 - 1));
                }
            }
            // the last b1 - i0 < CH tiles are in kb[0 ..]
#pragma unroll
            for (int u = 0; u < CH - 1; ++u)
                if (i0 + u < b1)
                    fold_tile<D, QT, false, MASK>(kb[u], vb[u], qr, c, lazy, st, tile_key0(i0 + u) + kg, delta,
                                                  lim, tb, anc);
        }
        for (int i = my_full; i < my_tiles; ++i) {
            if (i == my_full || (i & 63) == 0)
                load_pids(i & ~63);
            uint32_t kb[NS][W], vb[NS][W];
            load_tile(kb, vb, i);
            fold_tile<D, QT, true, MASK>(kb, vb, qr, c, lazy, st, tile_key0(i) + kg, delta, lim, tb, anc);
        }
        if (page_bad) {
            if (lane == 0)
                report(p.err, TF_ERR_BAD_PAGE);
#pragma unroll
            for (int v = 0; v < QT; ++v)
                st.l[v] = NAN;
        }

        // ---- the key groups of a wave share m, so their l and o add up.  A
        // DPP step folds the two key groups of each 16-lane row (LPK 8),
        // lane swaps fold rows where fewer than 4 row sums are kept; the
        // lanes of one copy park their sums in LDS, then all threads finish
        // (query vector, dimension pair) elements: rows and waves summed in
        // a fixed order, each wave scaled to the largest reference.
        auto fold = [&](float x, bool mn) {
            float a, b;
            if constexpr (LPK == 8)
                x = mn ? vmin(x, ror8(x)) : x + ror8(x);
            if constexpr (R <= 2) {
                swap16(x, a, b);
                x = mn ? vmin(a, b) : a + b;
            }
            if constexpr (R == 1) {
                swap32(x, a, b);
                x = mn ? vmin(a, b) : a + b;
            }
            return x;
        };
        const bool writer = (LPK == 16 || (lane & 8) == 0) && (R == 4 || (lane & 16) == 0) &&
                            (R >= 2 || (lane & 32) == 0);
        const int rg = R == 4 ? (lane >> 4) : (R == 2 ? (lane >> 5) : 0);
#pragma unroll
        for (int v = 0; v < QT; ++v) {
            const float lv = fold(st.l[v], false);
            const float lov = fold(st.lo[v], true);
            if constexpr (G::PAIR) {
                // each 16-lane row already holds its key pair's whole output,
                // half a slice per lane
                store_pair_f32<D, QT>(xo[wave][v][rg], st.o[v], sl, odd);
                if (writer && sl == 0) {
                    xl[wave][v][rg][0] = lv;
                    xl[wave][v][rg][1] = lov;
                }
            } else {
#pragma unroll
                for (int d = 0; d < DPL; ++d)
                    st.o[v][d] = fold(st.o[v][d], false);
                if (writer) {
                    store_f32<D, QT>(xo[wave][v][rg], st.o[v], sl);
                    if (sl == 0) {
                        xl[wave][v][rg][0] = lv;
                        xl[wave][v][rg][1] = lov;
                    }
                }
            }
            if (lane == 0)
                xm[wave][v] = st.m[v];
        }
        lds_barrier();
        for (int e = threadIdx.x; e < QT * (D / 2); e += kThreads) {
            const int v = e / (D / 2);
            const int d = 2 * (e % (D / 2));
            const int qv = qt0 + v;
            if (qv >= nq)
                break;   // e only grows with v
            float mm = xm[0][v];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                mm = max2(mm, xm[w][v]);
            const float ms = (mm == -INFINITY) ? 0.0f : mm;
            float ll = 0.0f, lw = INFINITY, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = exp2_fast((xm[w][v] - ms) * c);
                float lr = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    lr += xl[w][v][q][0];
                    lw = min2(lw, xl[w][v][q][1]);
                    const float2 x = *reinterpret_cast<const float2 *>(&xo[w][v][q][d]);
                    a0 += x.x;
                    a1 += x.y;
                }
                ll = fmaf(lr, f, ll);
                o0 = fmaf(a0, f, o0);
                o1 = fmaf(a1, f, o1);
            }
            const int r = qv / group;
            const int h = g * group + qv % group;
            const bool nan_out = __builtin_isnan(ll) || lw == -INFINITY || errbits != 0;
            if (p.split_keys > 0) {
                if (!parts_ok)
                    continue;
                const int64_t recno = s.partial_offset + ((int64_t)r * p.hq + h) * n_splits + t;
                float *rec = p.partials + recno * (D + 4);
                if (d == 0)
                    *reinterpret_cast<float4 *>(rec) =
                        make_float4(nan_out ? NAN : mm * (c * kLn2), nan_out ? NAN : ll, 0.0f, 0.0f);
                *reinterpret_cast<float2 *>(rec + 4 + d) =
                    make_float2(nan_out ? NAN : o0, nan_out ? NAN : o1);
            } else {
                const uint32_t b0 = nan_out ? kBf16NaN : bf16_out(o0 / ll);
                const uint32_t b1 = nan_out ? kBf16NaN : bf16_out(o1 / ll);
                *reinterpret_cast<uint32_t *>(p.out + ((size_t)(s.row_offset + r) * p.hq + h) * D + d) =
                    b0 | (b1 << 16);
            }
        }
        lds_barrier();   // xo, xl and xm are rewritten by the next pass
    }
    if (threadIdx.x == 0 && g == 0 && t == 0)
        report(p.err, errbits);
}

// One pass of 4 query vectors: this kernel serves the segments with at most
// kMfmaMinQ (= 4) query vectors per kv head; the rest take rows_mfma_kernel.
static_assert(kMfmaMinQ <= 4, "the decode kernel is launched for 4 query vectors a pass");

template <int D, int KIND>
hipError_t launch_qt(const RowsParams &p, dim3 grid, hipStream_t st)
{
    if (p.mask == TF_MASK_TREE)
        hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 4, TF_MASK_TREE>), grid, dim3(kThreads), 0, st, p);
    else if (p.mask == TF_MASK_FULL)
        hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 4, TF_MASK_FULL>), grid, dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((rows_valu_kernel<D, KIND, 4, TF_MASK_CAUSAL>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_kind(const RowsParams &p, int kind, dim3 grid, hipStream_t st)
{
    switch (kind) {
    case TF_KV_CONTIG:
        return launch_qt<D, TF_KV_CONTIG>(p, grid, st);
    case TF_KV_PAGED:
        return launch_qt<D, TF_KV_PAGED>(p, grid, st);
    default:
        return launch_qt<D, TF_KV_RING>(p, grid, st);
    }
}

}  // namespace

// Launch the VALU rows kernel; one block per (split, segment, kv head).
hipError_t launch_rows_valu(const RowsParams &p, int head_dim, int kind, hipStream_t st)
{
    const dim3 grid((unsigned)(p.n_segments * p.n_split_max * p.hkv));
    switch (head_dim) {
    case 64:
        return launch_kind<64>(p, kind, grid, st);
    case 128:
        return launch_kind<128>(p, kind, grid, st);
    default:
        return launch_kind<256>(p, kind, grid, st);
    }
}

}  // namespace tfa
