/*
 * Float64 CPU oracle for shared-round attention and greedy argmax.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the bench's
 * CPU-baseline leg are the only code that loads this library.  The HIP
 * library under stream_paged_attention_amd/ never includes, links or calls
 * it, and the two share no source: no header, helper, table or constant.
 *
 * What it computes, and the passages it follows:
 *
 *  - Softmax attention of every packed query row over its own stream's keys,
 *    with grouped KV heads: TensorFold PR #1503 ("lfm2_moe CUDA: attention
 *    pages from the shared KV pool, and the prompt cache"), the commit that
 *    runs every stream's rows from one segment table and checks them against
 *    a float64 attention; TensorFold PR #1562 ("Qwen3.6 MTP drafter on CUDA:
 *    draft a shared round's streams together"), its Gate section (FP64 check
 *    at the served shapes).
 *  - Which keys a row sees (TensorFold PR #1394, "lfm2: a cheaper DSpark
 *    hold", the DSpark drafter commit contrasting the FULL block flag with
 *    the target's causal count; PR #1562, the Qwen3.6 MTP drafter's tree
 *    attention beside its chains).  Row r of an n-row segment with
 *    key_count kc sees, by the launch's mask:
 *      causal: keys [0, kc - n + r + 1) (up to and including its own key);
 *      full:   keys [0, kc) (every row of the block sees the whole range);
 *      tree:   the context keys [0, kc - n), its own key kc - n + r, and the
 *              key kc - n + j of every row j whose bit is set in the row's
 *              64-bit ancestor mask (n <= 64).
 *  - Split-K partials and their merge (PR #1503, the shared-window chunk and
 *    merge bodies; PR #1653, "spark25 CUDA: the full layers' caches in pages
 *    of the core pool", the paged decode part/merge kernels).
 *  - Greedy argmax: the first (lowest-id) largest logit of each row, and a
 *    flag on any row holding a nonfinite logit (PR #1503, the lfm2_argmax
 *    commit and its contract entry: ties go to the lower id).  A NaN ranks
 *    as -inf when choosing the id (PR #1503, the router note in lfm2_moe.cu).
 *
 * Readings where the pages are silent:
 *  - GQA: query head h reads kv head h / (Hq / Hkv) (contiguous groups).
 *  - NaN rule: if any *visible* score of a (row, head) is NaN or +-Inf, all
 *    of that (row, head)'s outputs are NaN; otherwise an output element whose
 *    value is not finite is reported as NaN.  Keys outside the visible range
 *    are never read.
 *  - Empty split (the row sees none of the keys it covers): m = -inf,
 *    l = 0, o = 0, and the merge skips it.
 *
 * Inputs are bf16 bit patterns (uint16).  K and V are each stream's logical
 * rows [key][kv_head][dim], concatenated over streams; the oracle never sees
 * pages or rings.  Every product and sum is in double, in index order.
 *
 * Parity status: the attention value is pinned (torch's float64
 * scaled_dot_product_attention, closed forms, split/merge and causal
 * identities); the argmax is pinned (numpy argmax on finite rows, special
 * cases).  See tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

enum { MASK_CAUSAL = 0, MASK_FULL = 1, MASK_TREE = 2 };

/* One (row, head) task: where its query is and which keys it may see. */
typedef struct {
    int64_t qrow;      /* packed row index */
    int head;          /* query head */
    int seg;           /* segment */
    int row;           /* row within its segment */
    int n_rows;        /* rows of its segment */
    int key_count;     /* keys of its stream */
    int mask;          /* MASK_* */
    uint64_t anc;      /* tree: bit j = the segment's row j is an ancestor */
} task_t;

/* Whether the task's row sees key j of its stream (the masks above). */
static int sees(const task_t *t, int j)
{
    const int first_new = t->key_count - t->n_rows;   /* key of the segment's row 0 */
    if (j < 0 || j >= t->key_count)
        return 0;
    switch (t->mask) {
    case MASK_FULL:
        return 1;
    case MASK_TREE:
        if (j < first_new || j == first_new + t->row)
            return 1;
        return (int)((t->anc >> (j - first_new)) & 1u);
    default:
        return j <= first_new + t->row;
    }
}

static task_t *make_tasks(int n_seg, const int32_t *n_rows, const int32_t *key_count,
                          const int32_t *row_offset, int hq, int mask, const uint64_t *tree,
                          int64_t *n_tasks)
{
    int64_t total = 0;
    for (int s = 0; s < n_seg; ++s)
        total += (int64_t)n_rows[s] * hq;
    task_t *t = (task_t *)malloc(sizeof(task_t) * (size_t)(total > 0 ? total : 1));
    int64_t at = 0;
    for (int s = 0; s < n_seg; ++s)
        for (int r = 0; r < n_rows[s]; ++r)
            for (int h = 0; h < hq; ++h) {
                t[at].qrow = (int64_t)row_offset[s] + r;
                t[at].head = h;
                t[at].seg = s;
                t[at].row = r;
                t[at].n_rows = n_rows[s];
                t[at].key_count = key_count[s];
                t[at].mask = mask;
                t[at].anc = mask == MASK_TREE ? tree[row_offset[s] + r] : 0;
                ++at;
            }
    *n_tasks = total;
    return t;
}

static int threads_used(int n_threads)
{
#ifdef _OPENMP
    return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/* Scores of one query against the keys j in [j0, j1) its task sees, in
 * double (s[j - j0]; entries of unseen keys are left alone).  Returns 1 if
 * a seen score is not finite; *n_seen counts the seen keys. */
static int scores_into(const task_t *t, const uint16_t *q, const uint16_t *k, int hkv, int d,
                       int g, int j0, int j1, double scale, double *qd, double *s, int *n_seen)
{
    int nonfinite = 0;
    *n_seen = 0;
    for (int x = 0; x < d; ++x)
        qd[x] = bf16_value(q[x]);
    for (int j = j0; j < j1; ++j) {
        if (!sees(t, j))
            continue;
        const uint16_t *kr = k + ((int64_t)j * hkv + g) * d;
        double acc = 0.0;
        for (int x = 0; x < d; ++x)
            acc += qd[x] * bf16_value(kr[x]);
        acc *= scale;
        s[j - j0] = acc;
        ++*n_seen;
        if (!isfinite(acc))
            nonfinite = 1;
    }
    return nonfinite;
}

/*
 * oracle_attn: the unsplit definition.
 *   out[row][h][:] = sum_j softmax_j(scale * q.k_j) v_j over visible j.
 * Returns the number of threads used.
 */
int oracle_attn(int n_seg, const int32_t *n_rows, const int32_t *key_count,
                const int32_t *row_offset, const int64_t *key_base,
                int hq, int hkv, int d, double scale,
                const uint16_t *q, const uint16_t *k_all, const uint16_t *v_all,
                int mask, const uint64_t *tree, double *out, int n_threads)
{
    int64_t nt = 0;
    task_t *tasks = make_tasks(n_seg, n_rows, key_count, row_offset, hq, mask, tree, &nt);
    int maxkc = 1;
    for (int s = 0; s < n_seg; ++s)
        if (key_count[s] > maxkc)
            maxkc = key_count[s];
    const int group = hq / hkv;
    const int used = threads_used(n_threads);

#pragma omp parallel num_threads(used)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)maxkc);
        double *qd = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nt; ++i) {
            const task_t *t = &tasks[i];
            const int g = t->head / group;
            const uint16_t *qv = q + (t->qrow * hq + t->head) * d;
            const uint16_t *ks = k_all + key_base[t->seg] * hkv * d;
            const uint16_t *vs = v_all + key_base[t->seg] * hkv * d;
            double *o = out + (t->qrow * hq + t->head) * d;
            int n_seen = 0;
            if (scores_into(t, qv, ks, hkv, d, g, 0, t->key_count, scale, qd, s, &n_seen) ||
                n_seen == 0) {
                for (int x = 0; x < d; ++x)
                    o[x] = NAN;
                continue;
            }
            double m = -INFINITY;
            for (int j = 0; j < t->key_count; ++j)
                if (sees(t, j) && s[j] > m)
                    m = s[j];
            double l = 0.0;
            for (int x = 0; x < d; ++x)
                acc[x] = 0.0;
            for (int j = 0; j < t->key_count; ++j) {
                if (!sees(t, j))
                    continue;
                const double p = exp(s[j] - m);
                const uint16_t *vr = vs + ((int64_t)j * hkv + g) * d;
                l += p;
                for (int x = 0; x < d; ++x)
                    acc[x] += p * bf16_value(vr[x]);
            }
            for (int x = 0; x < d; ++x) {
                const double y = acc[x] / l;
                o[x] = isfinite(y) ? y : NAN;
            }
        }
        free(s);
        free(qd);
        free(acc);
    }
    free(tasks);
    return used;
}

/*
 * oracle_attn_partials: split-K pieces.  Split t of a row covers the keys
 * it sees in [t*split, (t+1)*split).  For each (row, head, split):
 *   m = max score, l = sum exp(score - m), o = sum exp(score - m) v.
 * Layout: m, l [total_rows][hq][n_split]; o [total_rows][hq][n_split][d].
 * A split holding a nonfinite visible score is all NaN; an empty split is
 * (m, l, o) = (-inf, 0, 0).
 */
int oracle_attn_partials(int n_seg, const int32_t *n_rows, const int32_t *key_count,
                         const int32_t *row_offset, const int64_t *key_base,
                         int hq, int hkv, int d, double scale,
                         const uint16_t *q, const uint16_t *k_all, const uint16_t *v_all,
                         int mask, const uint64_t *tree, int split, int n_split,
                         double *pm, double *pl, double *po, int n_threads)
{
    int64_t nt = 0;
    task_t *tasks = make_tasks(n_seg, n_rows, key_count, row_offset, hq, mask, tree, &nt);
    const int group = hq / hkv;
    const int used = threads_used(n_threads);

#pragma omp parallel num_threads(used)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)split);
        double *qd = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nt; ++i) {
            const task_t *t = &tasks[i];
            const int g = t->head / group;
            const uint16_t *qv = q + (t->qrow * hq + t->head) * d;
            const uint16_t *ks = k_all + key_base[t->seg] * hkv * d;
            const uint16_t *vs = v_all + key_base[t->seg] * hkv * d;
            for (int sp = 0; sp < n_split; ++sp) {
                const int64_t rec = (t->qrow * hq + t->head) * n_split + sp;
                double *o = po + rec * d;
                const int j0 = sp * split;
                const int j1 = j0 + split;
                int n_seen = 0;
                const int bad = scores_into(t, qv, ks, hkv, d, g, j0, j1, scale, qd, s, &n_seen);
                if (n_seen == 0) {
                    pm[rec] = -INFINITY;
                    pl[rec] = 0.0;
                    for (int x = 0; x < d; ++x)
                        o[x] = 0.0;
                    continue;
                }
                if (bad) {
                    pm[rec] = NAN;
                    pl[rec] = NAN;
                    for (int x = 0; x < d; ++x)
                        o[x] = NAN;
                    continue;
                }
                double m = -INFINITY;
                for (int j = j0; j < j1; ++j)
                    if (sees(t, j) && s[j - j0] > m)
                        m = s[j - j0];
                double l = 0.0;
                for (int x = 0; x < d; ++x)
                    o[x] = 0.0;
                for (int j = j0; j < j1; ++j) {
                    if (!sees(t, j))
                        continue;
                    const double p = exp(s[j - j0] - m);
                    const uint16_t *vr = vs + ((int64_t)j * hkv + g) * d;
                    l += p;
                    for (int x = 0; x < d; ++x)
                        o[x] += p * bf16_value(vr[x]);
                }
                pm[rec] = m;
                pl[rec] = l;
            }
        }
        free(s);
        free(qd);
    }
    free(tasks);
    return used;
}

/*
 * oracle_merge: combine the partials of every (row, head).
 *   M = max m_t over non-empty splits, L = sum l_t e^(m_t - M),
 *   out = (sum o_t e^(m_t - M)) / L.  Any NaN split makes the output NaN.
 */
void oracle_merge(int64_t n_rowheads, int n_split, int d,
                  const double *pm, const double *pl, const double *po, double *out)
{
    for (int64_t i = 0; i < n_rowheads; ++i) {
        const double *m = pm + i * n_split;
        const double *l = pl + i * n_split;
        double *o = out + i * d;
        int bad = 0;
        double big = -INFINITY;
        for (int t = 0; t < n_split; ++t) {
            if (isnan(m[t]))
                bad = 1;
            else if (m[t] > big)
                big = m[t];
        }
        if (bad || big == -INFINITY) {
            for (int x = 0; x < d; ++x)
                o[x] = NAN;
            continue;
        }
        double lsum = 0.0;
        for (int x = 0; x < d; ++x)
            o[x] = 0.0;
        for (int t = 0; t < n_split; ++t) {
            if (m[t] == -INFINITY)
                continue;
            const double w = exp(m[t] - big);
            lsum += l[t] * w;
            const double *ot = po + (i * n_split + t) * d;
            for (int x = 0; x < d; ++x)
                o[x] += ot[x] * w;
        }
        for (int x = 0; x < d; ++x) {
            const double y = o[x] / lsum;
            o[x] = isfinite(y) ? y : NAN;
        }
    }
}

/*
 * oracle_argmax: sequential scan of each row in id order.  The best id is
 * replaced only by a strictly larger value, so ties keep the lower id; NaN
 * compares as -inf; -0.0 and +0.0 are equal.  flag = 1 if any logit of the
 * row is NaN or +-Inf.
 */
void oracle_argmax(const uint16_t *logits, int n_rows, int vocab, int64_t row_stride,
                   int32_t *ids, uint8_t *flags)
{
    for (int r = 0; r < n_rows; ++r) {
        const uint16_t *row = logits + (int64_t)r * row_stride;
        int best = 0;
        double best_key = -INFINITY;
        int flag = 0;
        for (int i = 0; i < vocab; ++i) {
            const double x = bf16_value(row[i]);
            if (!isfinite(x))
                flag = 1;
            const double key = isnan(x) ? -INFINITY : x;
            if (i == 0 || key > best_key) {
                best = i;
                best_key = key;
            }
        }
        ids[r] = best;
        flags[r] = (uint8_t)flag;
    }
}
