// tf_attn_rows, matrix-core path: segments with many query vectors per kv
// head (prompt chunks, long verify rounds), with bf16 MFMA for the score and
// value products (TensorFold PR #1503, the paged prompt kernels with the
// dense tiles on the tensor cores; PR #1653, the head-dim-256 paged prompt
// kernels with the page id hoisted per tile).
//
// Work item = one workgroup = (segment, kv head g, split t, query tile).  A
// query tile is QB query vectors (row-major over the segment's rows, the
// group's query heads fastest); each of the NW waves owns NQB blocks of 16.
// A tile with fewer blocks than waves (verify and drafter rounds) gives each
// block several waves, which split its output dims.  Which workgroup serves
// which item is set by grid_cell (grid_cell.hpp), so that the shader
// engines get even shares of the keys.
//
// Per 32-key tile, all from LDS, each wave computes
//     S^T = K Q^T          (v_mfma_f32_16x16x32_bf16, A = K rows, B = Q^T)
// so that a lane holds the scores of one query vector (lane % 16) for four
// keys of each 16-key block, then the online softmax for its query vector,
// and
//     O^T += V^T P^T       (A = V^T from ds_read_tr16_b64, B = P^T in bf16)
// where P^T is exactly the S^T register layout: no lane exchange between
// the two products.  P is rounded to bf16 (fp32 sums); a product against a
// block of ones accumulates l = sum p from the same rounded weights next to
// O.
//
// K/V tiles are staged through LDS by direct global->LDS loads (16 bytes a
// lane, 1 KB a wave instruction), double buffered: the next tile's loads are
// in flight while the current one is multiplied.  Within a key row the
// 16-byte units are XOR-swizzled by the key index so that the 16 lanes
// reading one unit column hit distinct banks.  NBUF tile buffers: NBUF - 1
// tiles in flight while one is multiplied, one barrier per tile.
//
// Two shapes at head dim 256.  Prompt chunks: 8 waves (128 query vectors) a
// workgroup with four tile buffers (128 KB of LDS), one workgroup a CU, so
// each staged tile serves 128 vectors.  Launches whose segments all have at
// most 64 query vectors per kv head (verify rounds): 4 waves a workgroup
// with two tile buffers (64 KB) and registers held to two waves a SIMD, so
// that two workgroups share a CU and run out of step; with one 8-wave
// workgroup a CU those launches ran their work items in two to three rounds
// of barrier-locked waves.
//
// Masking (causal rows, a tree's block, split end, keys past the count)
// happens on the scores.  A masked key's value must add exactly nothing, but 0 * NaN = NaN
// on the matrix core: in tiles that mask anything, nonfinite value elements
// are replaced by 0 before the product, and an indicator product records
// which (dimension, query vector) outputs saw a nonfinite value among their
// visible keys; those are written as NaN (the NaN rule for values).
#include "device.hpp"
#include "grid_cell.hpp"

namespace tfa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kKT = 32;                // keys per tile
constexpr float kMLazy = 8.0f;         // log2 of the largest weight a stale reference may give

// SMALL: the head-dim-256 shape for launches of at most 64 query vectors
// per kv head (it changes nothing below 256)
template <int D, bool SMALL = false>
struct MGeo {
    static constexpr int NW = D == 256 && !SMALL ? 8 : 4;   // waves per workgroup
    static constexpr int KS = D / 32;                 // 32-dim steps of the score product
    static constexpr int DB = D / 16;                 // 16-dim blocks of the output
    static constexpr int UPR = D / 8;                 // 16-byte units per key row
    static constexpr int NQB = 1;                     // 16-vector blocks per wave
    static constexpr int QB = NW * 16 * NQB;          // query vectors per workgroup
    static constexpr int TILE = kKT * D * 2;          // bytes of one K (or V) tile
    static constexpr int LOADS = TILE / 1024 / NW;    // 1 KB wave loads per wave per tile (K or V)
    // LDS tile buffers (K and V): NBUF - 1 tiles in flight while one is
    // multiplied; 128 KB of LDS at D 256 (one workgroup of 8 waves a CU),
    // 64 KB for the small D 256 shape and D 64 (two workgroups of 4 waves),
    // 48 KB used at D 128 (two workgroups a CU, see NBUF_LDS: the ring
    // drafter 25.7 -> 24.9 us against four buffers, 28.9 us with five, six
    // buffers (one workgroup a CU) 40 us)
    static constexpr int NBUF = D == 256 ? (SMALL ? 2 : 4) : (D == 128 ? 3 : 8);
    static constexpr int PD = NBUF - 1;               // prefetch distance in tiles
    // LDS allocated: at D 128 four buffers' worth, of which three are used, so
    // that two workgroups share a CU.  Three a CU (which the registers allow
    // once they drop to 168) ran the ring drafter at 30.5 us against 26.5.
    static constexpr int NBUF_LDS = D == 128 ? 4 : NBUF;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == TILE, "tile must split into 1 KB wave loads");
};

template <int N>
struct IntC {
    static constexpr int value = N;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// Byte offset of 16-byte unit `c` of key row `key` in an LDS tile.
template <int D>
__device__ __forceinline__ uint32_t unit_off(int key, int c)
{
    using G = MGeo<D>;
    return (uint32_t)(key * G::UPR + (c ^ (key & (G::UPR - 1)))) * 16u;
}

// Workgroup barrier with no fence.  The LDS tiles are written by direct
// global->LDS loads; each wave establishes their completion itself with an
// explicit vmcnt wait before the barrier (a fence would also wait for the
// tiles still in flight).  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void tile_barrier()
{
    asm volatile("s_barrier" ::: "memory");
}

// One direct global->LDS load: 16 bytes per lane from `src` into LDS at
// lds_base + 16 * lane (lds_base is wave-uniform, in M0).  Issued from asm
// so that the compiler does not count it against the LDS reads of the tile
// being multiplied (it would wait for every tile in flight before each);
// the kernel waits for these loads explicitly.  No register is written.
// M0 is written here and nowhere else in this file's kernels (the compiler
// sets it only for LDS-DMA builtins, which are not used): tests check the
// generated code for any other M0 access.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n), n = 0 .. 63 (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `newer` tiles of L loads each are still in flight
// (newer = 0 .. MAXN, uniform).
template <int L, int MAXN>
__device__ __forceinline__ void wait_tiles(int newer)
{
    if constexpr (MAXN <= 0) {
        wait_vm<0>();
    } else {
        if (newer >= MAXN)
            wait_vm<L * MAXN>();
        else
            wait_tiles<L, MAXN - 1>(newer);
    }
}

template <int D, int KIND, int MASK, bool SMALL>
__global__ __launch_bounds__((64 * MGeo<D, SMALL>::NW))
__attribute__((amdgpu_waves_per_eu(SMALL ? 2 : 1))) void rows_mfma_kernel(RowsParams p)
{
    using G = MGeo<D, SMALL>;
    constexpr int KS = G::KS, DB = G::DB, NQB = G::NQB, QB = G::QB, LOADS = G::LOADS, NW = G::NW;
    constexpr int NBUF = G::NBUF, PD = G::PD;
    __shared__ __attribute__((aligned(1024))) char kv_lds[G::NBUF_LDS][2][G::TILE];   // [buffer][K, V]

    // ---- work item (grid_cell)
    const Cell cell = grid_cell(blockIdx.x, p.hkv, p.n_segments, p.n_split_max);
    const int g = cell.g;
    const int seg_i = cell.seg;
    const int t = cell.t;
    const int qt = cell.qt;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lg = lane >> 4;     // lane group (0..3)
    const int lc = lane & 15;     // lane column

    // the whole row in scalar registers here, in one memory round trip (a
    // copy, so the checks below read registers): left to the compiler, each
    // field was fetched at its first use, one wait after another
    const tf_segment sd = p.segs[seg_i];
    asm volatile("" ::"s"(sd.k), "s"(sd.v), "s"(sd.pages), "s"(sd.capacity), "s"(sd.first), "s"(sd.row_offset),
                 "s"(sd.n_rows), "s"(sd.key_count), "s"(sd.partial_offset));
    const char *kbase = static_cast<const char *>(sd.k);
    const char *vbase = static_cast<const char *>(sd.v);
    const int32_t *pages = sd.pages;
    const int capacity = sd.capacity, first = sd.first, row_offset = sd.row_offset;
    const int n_rows = sd.n_rows, kc = sd.key_count, partial_offset = sd.partial_offset;

    const int group = p.group;
    const int nq = n_rows * group;
    // rows_valu_kernel serves the segments with few query vectors
    if (nq <= p.mfma_min_q)
        return;
    const bool rows_ok = n_rows >= 1 && n_rows <= kc && row_offset >= 0 &&
                         (int64_t)row_offset + n_rows <= p.total_rows &&
                         (MASK != TF_MASK_TREE || n_rows <= 64);
    if (!rows_ok) {
        if (threadIdx.x == 0 && g == 0 && t == 0 && qt == 0)
            report(p.err, TF_ERR_BAD_ROWS);
        return;
    }
    if (qt * QB >= nq)
        return;
    int errbits = segment_errors<KIND>(p, sd, D);
    const int n_splits = p.split_keys > 0 ? (kc + p.split_keys - 1) / p.split_keys : 1;
    if (t >= n_splits)
        return;
    bool parts_ok = true;
    if (p.split_keys > 0) {
        const int64_t need = (int64_t)n_rows * p.hq * n_splits;
        parts_ok = partial_offset >= 0 && (int64_t)partial_offset + need <= p.max_records;
        if (!parts_ok)
            errbits |= TF_ERR_PARTIALS;
    }
    const int k0 = p.split_keys > 0 ? t * p.split_keys : 0;
    const int k_end = p.split_keys > 0 ? min(k0 + p.split_keys, kc) : kc;
    const float c = p.c_log2;
    const float lazy = kMLazy / c;

    // ---- which query vectors and output dims this wave computes.  A tile
    // with fewer 16-vector blocks than waves gives each block kw waves (a
    // power of two): they compute the same scores and weights, and each
    // accumulates 1 / kw of the output dims.  Every (vector, dim) output goes
    // through the same operations whatever kw is; the other waves of the
    // workgroup only stop idling.  kw is uniform over the workgroup and
    // selects one of the compiled loop bodies below.
    static_assert(NQB == 1, "the dim split assumes one 16-vector block per wave");
    constexpr int KW_MAX = NW < DB / 2 ? NW : DB / 2;
    const int nvb = min(NW, (nq - qt * QB + 15) / 16);   // blocks holding a vector
    int kw = KW_MAX;
    while (kw > 1 && NW / kw < nvb)
        kw >>= 1;
    const int nb = NW / kw;       // blocks served at once
    const int dg = wave / nb;     // dim group, 0 .. kw - 1
    // block wave % nb; a block at or past nvb holds no vector (the wave idles)
    const int qv0 = qt * QB + (wave % nb) * 16;
    int lim[NQB];
    uint64_t anc[NQB];
    int tb = INT32_MAX;   // the segment's first new key under a tree mask
    bool qvalid[NQB];
    int lim_min = INT32_MAX, lim_max = k0;
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
        const int qv = qv0 + b * 16 + lc;
        qvalid[b] = qv < nq;
        const int r = qv / group;
        const RowVis rv = row_vis<MASK>(p, kc, n_rows, qvalid[b] ? r : 0, row_offset, k_end);
        lim[b] = qvalid[b] ? rv.lim : 0;
        anc[b] = rv.anc;
        tb = rv.tb;
    }
    // wave-wide visible range: tiles below lim_min are unmasked for every
    // query vector of the wave, tiles at or past lim_max are invisible
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
        int lo_b = qvalid[b] ? min(lim[b], tb) : INT32_MAX;
        int hi_b = qvalid[b] ? lim[b] : k0;
        // reduce over the 64 lanes (the 4 lane groups hold the same values)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            lo_b = min(lo_b, __shfl_xor(lo_b, off));
            hi_b = max(hi_b, __shfl_xor(hi_b, off));
        }
        lim_min = min(lim_min, __builtin_amdgcn_readfirstlane(lo_b));
        lim_max = max(lim_max, __builtin_amdgcn_readfirstlane(hi_b));
    }
    // workgroup-wide number of tiles: every wave loads its share of every
    // tile the workgroup needs
    __shared__ int wg_hi[NW];
    if (lane == 0)
        wg_hi[wave] = lim_max;
    lds_barrier();
    int blk_hi = k0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        blk_hi = max(blk_hi, wg_hi[w]);
    const int n_tiles = errbits ? 0 : (blk_hi - k0 + kKT - 1) / kKT;
    const bool wave_live = lim_max > k0;   // this wave has a visible key in the split

    // ---- Q^T fragments (B operand): vector lc of block b, dims 32s + 8 lg .. + 8
    u32x4_t qf[NQB][KS];
#pragma unroll
    for (int b = 0; b < NQB; ++b) {
        const int qv = qv0 + b * 16 + lc;
        const int r = qv / group;
        const int h = g * group + qv % group;
        const char *qrow = reinterpret_cast<const char *>(p.q) +
                           ((size_t)(row_offset + (qvalid[b] ? r : 0)) * p.hq + h) * (D * 2);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[b][s] = qvalid[b] ? load_global<u32x4_t>(qrow + (s * 32 + lg * 8) * 2) : u32x4_t{0, 0, 0, 0};
        }
    }

    // ---- K/V tile loads: wave `wave` fills 1 KB chunks wave*LOADS .. +LOADS
    // of each tile; lane `lane` of chunk ch fills unit U = ch*64 + lane
    bool page_bad = false;
    int pid = 0;
    auto load_pids = [&](int i0) {
        if constexpr (KIND == TF_KV_PAGED) {
            const int ti = i0 + lane;
            pid = ti < n_tiles ? load_global<int32_t>(pages + ((k0 + ti * kKT) >> p.page_shift)) : 0;
        }
    };
    auto issue = [&](int i, int buf) {
        const int kt = k0 + i * kKT;
        const char *kb_ = kbase;
        const char *vb_ = vbase;
        size_t run = 0;
        if constexpr (KIND == TF_KV_PAGED) {
            int page = __builtin_amdgcn_readlane(pid, i & 63);
            if ((unsigned)page >= (unsigned)p.pool_pages) {
                page_bad = true;
                page = 0;
            }
            run = (((size_t)page * p.hkv + g) * p.page_size + (kt & (p.page_size - 1))) * (D * 2);
        } else {
            run = (size_t)g * capacity * (D * 2);
        }
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int ch = wave * LOADS + u;
            const int U = ch * 64 + lane;
            const int key = U / G::UPR;
            const int cu = (U % G::UPR) ^ (key & (G::UPR - 1));
            size_t off;
            if constexpr (KIND == TF_KV_PAGED) {
                off = run + (size_t)key * (D * 2) + cu * 16;
            } else {
                // clamp keys past the count to the last key (in bounds; masked)
                int j = min(kt + key, kc - 1);
                if constexpr (KIND == TF_KV_RING) {
                    j += first;
                    j -= (j >= capacity) ? capacity : 0;
                }
                off = run + (size_t)j * (D * 2) + cu * 16;
            }
            // LDS byte addresses of the two destination chunks
            const uint32_t lk = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)(
                &kv_lds[buf][0][ch * 1024]));
            const uint32_t lv = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)(
                &kv_lds[buf][1][ch * 1024]));
            dma16(kb_ + off, __builtin_amdgcn_readfirstlane(lk));
            dma16(vb_ + off, __builtin_amdgcn_readfirstlane(lv));
        }
    };

    // ---- the tile loop and the write, for kw = KW waves a block
    auto body = [&](auto kw_c) {
        constexpr int KW = decltype(kw_c)::value;
        constexpr int DBG = DB / KW;   // dim blocks of this wave
        const int db0 = dg * DBG;
        // ---- state per block of 16 query vectors (per lane: its vector)
        float m[NQB], mc[NQB], thr[NQB], lo[NQB];
        f32x4_t o[NQB][DBG];   // o[b][j]: dim block db0 + j
        f32x4_t lsum[NQB];   // ones-block product: every element is l of the lane's vector
        uint32_t nanmask[NQB][(DBG * 4 + 31) / 32];
#pragma unroll
        for (int b = 0; b < NQB; ++b) {
            m[b] = -INFINITY;
            mc[b] = 0.0f;
            thr[b] = -INFINITY;
            lo[b] = INFINITY;
            lsum[b] = f32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int d = 0; d < DBG; ++d)
                o[b][d] = f32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int w = 0; w < (DBG * 4 + 31) / 32; ++w)
                nanmask[b][w] = 0;
        }
        const uint32_t one2 = 0x3F803F80u;   // two bf16 ones
        const bf16x8_t ones = as_bf16x8(u32x4_t{one2, one2, one2, one2});

        // Q fragments and the first page ids complete before the pipeline
        // starts: a register load still pending inside the loop would make every
        // iteration wait for all loads (the tile loads issued from asm included)
        if (n_tiles > 0)
            load_pids(0);
        wait_vm<0>();
#pragma unroll
        for (int u = 0; u < PD; ++u)
            if (u < n_tiles)
                issue(u, u);
        for (int i = 0; i < n_tiles; ++i) {
            const int buf = i % NBUF;
            const int kt = k0 + i * kKT;
            // tiles i .. i + PD - 1 are in flight (those that exist); wait for
            // the oldest.  The LDS reads of tile i - 1 are complete (their
            // products consumed them) before this wave reaches the barrier.
            const int newer = min(PD - 1, n_tiles - 1 - i);
            wait_tiles<2 * LOADS, PD - 1>(newer);
            // after the barrier: every wave's loads of tile i have landed and
            // every wave is done with tile i - 1, whose buffer takes tile i + PD
            tile_barrier();
            if (i + PD < n_tiles) {
                if (((i + PD) & 63) == 0) {
                    // next batch of page ids (every 64 tiles): drains the tiles in flight
                    load_pids(i + PD);
                    wait_vm<0>();
                }
                issue(i + PD, (i + PD) % NBUF);
            }
            if (!wave_live || kt >= lim_max)
                continue;    // nothing visible to this wave in the tile
            const char *kt_lds = kv_lds[buf][0];
            const char *vt_lds = kv_lds[buf][1];
            const bool full = kt + kKT <= lim_min;

            // -- scores S^T: 2 key blocks x NQB vector blocks
            // (even and odd dim steps accumulate apart: four independent
            // product chains per vector block keep the matrix pipe busy)
            f32x4_t s[NQB][2], s2[NQB][2];
#pragma unroll
            for (int b = 0; b < NQB; ++b)
                s[b][0] = s[b][1] = s2[b][0] = s2[b][1] = f32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ks += 2) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const u32x4_t kf = *reinterpret_cast<const u32x4_t *>(
                            kt_lds + unit_off<D>(kb * 16 + lc, (ks + h) * 4 + lg));
#pragma unroll
                        for (int b = 0; b < NQB; ++b) {
                            f32x4_t &acc = h ? s2[b][kb] : s[b][kb];
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[b][ks + h]),
                                                                         acc, 0, 0, 0);
                        }
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < NQB; ++b) {
                s[b][0] += s2[b][0];
                s[b][1] += s2[b][1];
            }

            // -- online softmax per vector; P^T fragments in bf16
            u32x4_t pf[NQB];   // P^T rounded to bf16
            uint64_t need = 0;
            float tmax[NQB];
#pragma unroll
            for (int b = 0; b < NQB; ++b) {
                float mx = -INFINITY;
                // one branch a tile (per element it costs ~6 % of the kernel)
                if (full) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            lo[b] = min2(lo[b], s[b][kb][e]);
                            mx = max2(mx, s[b][kb][e]);
                        }
                } else {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = s[b][kb][e];
                            const int key = kt + kb * 16 + lg * 4 + e;
                            const bool vis = row_sees<MASK>(key, lim[b], tb, anc[b]);
                            lo[b] = min2(lo[b], vis ? x : INFINITY);
                            x = vis ? x : -INFINITY;
                            s[b][kb][e] = x;
                            mx = max2(mx, x);
                        }
                }
                tmax[b] = mx;   // the lane's own maximum; reduced below
            }
            // the weights from the current reference, rounded to bf16 (fp32
            // sums: the value product and l take the same rounded weights).
            // They are computed while the row maxima reduce across lanes; the
            // rare step whose maximum moves the reference computes them again.
            auto weights = [&]() {
#pragma unroll
                for (int b = 0; b < NQB; ++b) {
                    float pe[8];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pe[kb * 4 + e] = exp2_fast(fmaf(s[b][kb][e], c, -mc[b]));
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        pf[b][w] = pack_bf16(pe[2 * w], pe[2 * w + 1]);
                }
            };
            weights();
#pragma unroll
            for (int b = 0; b < NQB; ++b) {
                float mx = tmax[b], a, bb;
                swap16(mx, a, bb);
                mx = max2(a, bb);
                swap32(mx, a, bb);
                mx = max2(a, bb);
                tmax[b] = mx;
                need |= __builtin_amdgcn_ballot_w64(mx > thr[b]);
            }
            if (need != 0) {
#pragma unroll
                for (int b = 0; b < NQB; ++b) {
                    const bool up = tmax[b] > m[b];
                    const float alpha = up ? exp2_fast((m[b] - tmax[b]) * c) : 1.0f;
                    m[b] = up ? tmax[b] : m[b];
                    mc[b] = up ? tmax[b] * c : mc[b];
                    thr[b] = up ? tmax[b] + lazy : thr[b];
                    lsum[b] *= alpha;
#pragma unroll
                    for (int d = 0; d < DBG; ++d)
                        o[b][d] *= alpha;
                }
                weights();
            }
#pragma unroll
            for (int b = 0; b < NQB; ++b)
                lsum[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, as_bf16x8(pf[b]), lsum[b], 0, 0, 0);

            // -- values: O^T += V^T P^T per 16-dim block.  V^T fragment of lane
            // (lg, lc): dims 16 db + lc, keys 4 lg .. + 4 and 16 + 4 lg .. + 4,
            // by two transposed reads of 4 x 16 blocks
            auto vread = [&](int db) {
                // the 16 lanes of group lg read the 4 x 16 block of keys
                // 4 lg .. + 4 (resp. 16 + 4 lg ..), dims 16 db .. + 16: lane
                // i of the group reads key 4 lg + i / 4, dims 16 db + 4 (i % 4) .. + 4
                const int key0 = lg * 4 + (lc >> 2);
                const int dim = db * 16 + (lc & 3) * 4;
                const uint32_t o0 = unit_off<D>(key0, dim >> 3) + (dim & 7) * 2;
                const uint32_t o1 = unit_off<D>(key0 + 16, dim >> 3) + (dim & 7) * 2;
                const i16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vt_lds + o0));
                const i16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vt_lds + o1));
                return u32x4_t{(uint32_t)(uint16_t)h0[0] | ((uint32_t)(uint16_t)h0[1] << 16),
                               (uint32_t)(uint16_t)h0[2] | ((uint32_t)(uint16_t)h0[3] << 16),
                               (uint32_t)(uint16_t)h1[0] | ((uint32_t)(uint16_t)h1[1] << 16),
                               (uint32_t)(uint16_t)h1[2] | ((uint32_t)(uint16_t)h1[3] << 16)};
            };
            // the products of two dim blocks (independent chains)
            auto pv2 = [&](int db, const u32x4_t &v0, const u32x4_t &v1) {
#pragma unroll
                for (int b = 0; b < NQB; ++b) {
                    o[b][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(v0), as_bf16x8(pf[b]), o[b][db], 0, 0, 0);
                    o[b][db + 1] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(v1), as_bf16x8(pf[b]), o[b][db + 1], 0, 0, 0);
                }
            };
            // masked tile: nonfinite values become 0 (exponent all ones -> zero)
            // and an indicator product records which (dim, vector) outputs saw
            // one among their visible keys
            uint64_t bad = 0;
            auto vclean = [&](u32x4_t vf, int db) {
                u32x4_t ind;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t x = vf[w];
                    const bool nlo = (x & 0x7F80u) == 0x7F80u;
                    const bool nhi = (x & 0x7F800000u) == 0x7F800000u;
                    vf[w] = (nlo ? 0u : (x & 0xFFFFu)) | (nhi ? 0u : (x & 0xFFFF0000u));
                    ind[w] = (nlo ? 0x3F80u : 0u) | (nhi ? 0x3F800000u : 0u);
                    bad |= __builtin_amdgcn_ballot_w64(nlo || nhi);
                }
                if (bad != 0) {
                    // count of visible nonfinite values per (dim, vector)
#pragma unroll
                    for (int b = 0; b < NQB; ++b) {
                        u32x4_t visf;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const int ka = kt + (w >> 1) * 16 + lg * 4 + (w & 1) * 2;
                            const bool v0 = row_sees<MASK>(ka, lim[b], tb, anc[b]);
                            const bool v1 = row_sees<MASK>(ka + 1, lim[b], tb, anc[b]);
                            visf[w] = (v0 ? 0x3F80u : 0u) | (v1 ? 0x3F800000u : 0u);
                        }
                        const f32x4_t cnt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(ind), as_bf16x8(visf), f32x4_t{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int bit = db * 4 + e;
                            if (cnt[e] > 0.0f)
                                nanmask[b][bit >> 5] |= 1u << (bit & 31);
                        }
                    }
                }
                return vf;
            };
            // The fragments of the next group of dim blocks are read while this
            // group's products run (a double buffer of VG fragments; the
            // scheduling barriers keep the compiler from reading further ahead
            // than the registers allow), so no product waits on its own read.
            // (local dim block j is dim block db0 + j)
            constexpr int VG = D == 256 ? 2 : (DBG < 4 ? DBG : 4);
            u32x4_t cur[VG], nxt[VG];
#pragma unroll
            for (int j = 0; j < VG; ++j)
                cur[j] = vread(db0 + j);
            // the value products run at raised wave priority, so that the
            // SIMD's arbiter favours the wave in this phase over one in its
            // softmax (about 1 % faster on all three MFMA workloads)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int g0 = 0; g0 < DBG; g0 += VG) {
                if (g0 + VG < DBG) {
#pragma unroll
                    for (int j = 0; j < VG; ++j)
                        nxt[j] = vread(db0 + g0 + VG + j);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < VG; j += 2) {
                    u32x4_t v0 = cur[j], v1 = cur[j + 1];
                    if (!full) {
                        v0 = vclean(v0, g0 + j);
                        v1 = vclean(v1, g0 + j + 1);
                    }
                    pv2(g0 + j, v0, v1);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (g0 + VG < DBG) {
#pragma unroll
                    for (int j = 0; j < VG; ++j)
                        cur[j] = nxt[j];
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (page_bad) {
            report(p.err, TF_ERR_BAD_PAGE);
#pragma unroll
            for (int b = 0; b < NQB; ++b)
                lsum[b] = f32x4_t{NAN, NAN, NAN, NAN};
        }

        // ---- write: lane (lg, lc) holds dims 16 (db0 + db) + 4 lg .. + 4 of vector lc
#pragma unroll
        for (int b = 0; b < NQB; ++b) {
            float a, bb;
            swap16(lo[b], a, bb);
            float lw = min2(a, bb);
            swap32(lw, a, bb);
            lw = min2(a, bb);
            if (!qvalid[b])
                continue;
            const int qv = qv0 + b * 16 + lc;
            const int r = qv / group;
            const int h = g * group + qv % group;
            const float ll = lsum[b][0];
            const bool nan_out = __builtin_isnan(ll) || lw == -INFINITY || errbits != 0;
            if (p.split_keys > 0) {
                if (!parts_ok)
                    continue;
                const int64_t recno = partial_offset + ((int64_t)r * p.hq + h) * n_splits + t;
                float *rec = p.partials + recno * (D + 4);
                if (lg == 0 && dg == 0)
                    *reinterpret_cast<float4 *>(rec) =
                        make_float4(nan_out ? NAN : m[b] * (c * kLn2), nan_out ? NAN : ll, 0.0f, 0.0f);
#pragma unroll
                for (int db = 0; db < DBG; ++db) {
                    float4 v;
                    float *vp = &v.x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int bit = db * 4 + e;
                        const bool nb = (nanmask[b][bit >> 5] >> (bit & 31)) & 1u;
                        vp[e] = (nan_out || nb) ? NAN : o[b][db][e];
                    }
                    *reinterpret_cast<float4 *>(rec + 4 + (db0 + db) * 16 + lg * 4) = v;
                }
            } else {
                uint16_t *dst = p.out + ((size_t)(row_offset + r) * p.hq + h) * D;
#pragma unroll
                for (int db = 0; db < DBG; ++db) {
                    uint16_t hb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int bit = db * 4 + e;
                        const bool nb = (nanmask[b][bit >> 5] >> (bit & 31)) & 1u;
                        hb[e] = (nan_out || nb) ? kBf16NaN : bf16_out(o[b][db][e] / ll);
                    }
                    *reinterpret_cast<uint2 *>(dst + (db0 + db) * 16 + lg * 4) =
                        make_uint2((uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16));
                }
            }
        }
    };
    if (kw == 1)
        body(IntC<1>{});
    else if (kw == 2)
        body(IntC<2 <= KW_MAX ? 2 : 1>{});
    else if (kw == 4)
        body(IntC<4 <= KW_MAX ? 4 : 1>{});
    else
        body(IntC<8 <= KW_MAX ? 8 : 1>{});
    if (threadIdx.x == 0 && g == 0 && t == 0 && qt == 0)
        report(p.err, errbits);
}

template <int D, int MASK, bool SMALL>
void launch_kind_m(const RowsParams &p, int kind, int n_qt, hipStream_t st)
{
    const dim3 grid((unsigned)(n_qt * p.n_split_max * p.n_segments * p.hkv));
    const dim3 block(64 * MGeo<D, SMALL>::NW);
    switch (kind) {
    case TF_KV_CONTIG:
        hipLaunchKernelGGL((rows_mfma_kernel<D, TF_KV_CONTIG, MASK, SMALL>), grid, block, 0, st, p);
        break;
    case TF_KV_PAGED:
        hipLaunchKernelGGL((rows_mfma_kernel<D, TF_KV_PAGED, MASK, SMALL>), grid, block, 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((rows_mfma_kernel<D, TF_KV_RING, MASK, SMALL>), grid, block, 0, st, p);
        break;
    }
}

template <int D, bool SMALL = false>
hipError_t launch_mask_m(const RowsParams &p, int kind, int n_qt, hipStream_t st)
{
    if (p.mask == TF_MASK_TREE)
        launch_kind_m<D, TF_MASK_TREE, SMALL>(p, kind, n_qt, st);
    else if (p.mask == TF_MASK_FULL)
        launch_kind_m<D, TF_MASK_FULL, SMALL>(p, kind, n_qt, st);
    else
        launch_kind_m<D, TF_MASK_CAUSAL, SMALL>(p, kind, n_qt, st);
    return hipGetLastError();
}

// The head-dim-256 launch takes the small shape when no segment has more
// query vectors per kv head than its tile.
bool small_shape(int head_dim, int64_t max_q)
{
    return head_dim == 256 && max_q <= MGeo<256, true>::QB;
}

}  // namespace

// Query vectors per MFMA workgroup for head dim D in a launch whose segments
// have at most max_q query vectors per kv head.
int mfma_query_tile(int head_dim, int64_t max_q)
{
    if (small_shape(head_dim, max_q))
        return MGeo<256, true>::QB;
    return head_dim == 256 ? MGeo<256>::QB : (head_dim == 128 ? MGeo<128>::QB : MGeo<64>::QB);
}

// Launch the MFMA rows kernel for the segments with more than p.mfma_min_q
// query vectors per kv head (max_q bounds them all); one block per (query
// tile, split, segment, kv head).
hipError_t launch_rows_mfma(const RowsParams &p, int head_dim, int kind, int max_q, hipStream_t st)
{
    const int qb = mfma_query_tile(head_dim, max_q);
    const int n_qt = (max_q + qb - 1) / qb;
    switch (head_dim) {
    case 64:
        return launch_mask_m<64>(p, kind, n_qt, st);
    case 128:
        return launch_mask_m<128>(p, kind, n_qt, st);
    default:
        if (small_shape(head_dim, max_q))
            return launch_mask_m<256, true>(p, kind, n_qt, st);
        return launch_mask_m<256>(p, kind, n_qt, st);
    }
}

}  // namespace tfa
