/*
 * CPU oracle for S2O causal-prefill attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  The product path never calls it; it shares no source, header,
 * table or helper with the HIP library.  It is plain, slow and written to be
 * checked against the pages by eye.
 *
 * Sources (all about "S2O: Early Stopping for Sparse Attention via Online
 * Permutation", Zhang et al., arXiv 2602.22575):
 *   [ABS]  the authors' abstract, as reproduced on the pith.science page
 *          ("read the original abstract").
 *   [GIST] the gist.science technical summary (French), section "Méthodologie :
 *          S2O": "1. Permutation en ligne via Chargement Guidé par Index"
 *          (Classement par Segment, KV_perm, Chargement Planifié par
 *          Coordonnées), "2. Règle d'Arrêt Anticipé", "3. Implémentation du
 *          Noyau" (Passage 1, Passage 2).
 *   [LENS] the arxivlens summary (Methodology and Limitations facets).
 *
 * What is computed, per (batch b, query head h, query tile t of BM rows):
 *   geometry   segments of S tokens; tile t starts at row t*BM; its segment
 *              starts at a_t = floor(t*BM/S)*S; its history is keys [0, a_t).
 *              [GIST] "Classement par Segment".
 *   pool       qbar[k] = (sum over the tile's BM rows, ascending, in fp32) * 2^-log2(BM)
 *              -- the tile's representative query.  The pages leave the
 *              representative unspecified ([GIST] KV_perm); the mean of the
 *              tile's rows is the reading taken here.
 *   score      s[j] = fp32 dot(qbar, K[b, h/G, j]) for j < a_t, accumulated
 *              with one fmaf per dimension in ascending order (the canonical
 *              order, part of the definition so that any faithful evaluation
 *              gives the same bits).  Only causal-prefix keys are scored
 *              ([GIST] KV_perm).
 *   segment lists (optional granularity): one list per (b, h, segment), shared
 *              by the segment's tiles, scored against the segment's
 *              representative query ([GIST] KV_perm speaks of a
 *              representative query of the segment): the mean of the
 *              segment's tile queries, an fp32 sum over its tiles in
 *              ascending order times fl(1/number of tiles).
 *   shared lists (optional, with either granularity): one list per KV head
 *              instead of per query head, used by the G query heads of the
 *              group (a GQA form of KV_perm's shared index map); its
 *              representative is the mean of the G heads' representatives, an
 *              fp32 sum over the heads in ascending order from 0, times
 *              fl(1/G).
 *   block lists (optional granularity): entries are blocks of BN consecutive
 *              history keys instead of single keys.  Block c is scored with
 *              its mean key (fp32 sum of its BN rows in ascending order, then
 *              the exact power-of-two scaling), with the same fma chain; pass
 *              2 chunk c is then the BN keys of the c-th listed block.  This is
 *              the block-granularity counterpart the pages compare against
 *              ([ABS] and [GIST] contrast token-level ordering with block-level
 *              sparse attention).
 *   query permutation (optional, Q_perm): inside each segment the query rows
 *              are ordered by a coarse importance score against a shared
 *              guide vector ([GIST] Classement par Segment, Q_perm: queries
 *              reordered within a segment to favour those likely to produce
 *              salient horizontal bands).  The guide is the segment's mean key
 *              (fp32 sum of its key rows in ascending order, times fl(1/rows));
 *              a row's score is the same fma chain as above; rows are sorted by
 *              score descending, ties to the lower row.  Query tile t of the
 *              segment is then rows order[(t - first tile)*BM ...] of that
 *              order; its representative is the fp32 sum of those rows in that
 *              order times 1/BM; pass 1 runs each row over its own causal
 *              window [a_t, i] (key tiles up to the tile's last row); outputs
 *              go back to the rows' own positions.
 *   order      the list: history keys (or blocks) sorted by score descending,
 *              ties to the lower index ([GIST] KV_perm: indices form a global
 *              logical map).
 *   pass 1     for each row i, online softmax over keys [a_t, i] in BN-wide key
 *              tiles in ascending order ([GIST] Passage 1: dense causal window
 *              inside the current segment, initialising (m, l, acc)).
 *   pass 2     for chunk c = 0, 1, ... of BN consecutive list entries: the same
 *              online update with no mask (every history key precedes every
 *              row), then the chunk's marginal mass gain
 *              delta_i = sum_{j in chunk} exp(x_ij - m_i) and the ratio
 *              g_i = delta_i / l_i (l_i after adding the chunk).  Stop after
 *              chunk c when max_i g_i < tau ([GIST] "2. Règle d'Arrêt
 *              Anticipé": stop once the marginal gain falls below a threshold
 *              relative to the accumulated score; [ABS]: proceed from high to
 *              low importance and skip the remaining blocks; [GIST] Passage 2).
 *              The chunk that triggers the stop is kept; the comparison is
 *              strict, so tau = 0 never stops.
 *   output     O_i = acc_i / l_i; executed tiles = pass-1 key tiles + executed
 *              pass-2 chunks.
 *
 * Precision: the estimator (pool, score) is fp32 in the canonical order above;
 * the attention itself is evaluated in fp64.  bf16 inputs are widened exactly.
 * Build with -ffp-contract=off so that no multiply-add is fused except the
 * explicit fmaf calls.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t B, Hq, Hkv, N, d;
    int32_t dtype; /* 0: fp32 values, 1: bf16 bit patterns (uint16) */
    int32_t seg_len, tile_m, tile_n;
    double scale;
    int32_t per_segment; /* 0: one list per query tile; 1: one list per segment */
    int32_t block_lists; /* 0: entries are keys; 1: entries are blocks of tile_n keys */
    int32_t qperm;       /* 1: query rows permuted within each segment (Q_perm) */
    int32_t share_gqa;   /* 1: one list per (b, KV head, tile or segment), shared by the
                            G query heads of the group (not with qperm) */
} oracle_problem;

/* ---- element access ------------------------------------------------------ */

static float widen(const void *base, int32_t dtype, int64_t i) {
    if (dtype == 0) return ((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static int64_t q_index(const oracle_problem *p, int b, int h, int64_t row, int k) {
    return (((int64_t)b * p->Hq + h) * p->N + row) * p->d + k;
}

static int64_t kv_index(const oracle_problem *p, int b, int g, int64_t row, int k) {
    return (((int64_t)b * p->Hkv + g) * p->N + row) * p->d + k;
}

/* ---- geometry ([GIST] Classement par Segment) ----------------------------- */

int32_t oracle_num_tiles(const oracle_problem *p) { return p->N / p->tile_m; }

int64_t oracle_seg_start(const oracle_problem *p, int t) {
    int64_t first_row = (int64_t)t * p->tile_m;
    return (first_row / p->seg_len) * p->seg_len;
}

/* number of BN-wide key tiles in pass 1: keys [a_t, (t+1)*BM) */
int32_t oracle_pass1_tiles(const oracle_problem *p, int t) {
    int64_t a = oracle_seg_start(p, t);
    int64_t end = (int64_t)(t + 1) * p->tile_m;
    return (int32_t)((end - a + p->tile_n - 1) / p->tile_n);
}

/* Offsets of the lists.  Per-tile lists are ordered by (b, h, t); per-segment
 * lists by (b, h, segment) and tile t uses the list of its segment.  Computed
 * by walking the lists and adding their history lengths; lists of segment 0
 * are empty. */
static int32_t num_segments(const oracle_problem *p) { return (p->N + p->seg_len - 1) / p->seg_len; }

/* keys covered by one list entry */
static int64_t entry_keys(const oracle_problem *p) { return p->block_lists ? p->tile_n : 1; }

/* entries of the list tile t uses: its history length in keys or in blocks */
int64_t oracle_list_len(const oracle_problem *p, int t) { return oracle_seg_start(p, t) / entry_keys(p); }

static int64_t per_head_entries(const oracle_problem *p) {
    int64_t total = 0;
    if (p->per_segment) {
        for (int s = 0; s < num_segments(p); ++s) total += (int64_t)s * p->seg_len / entry_keys(p);
    } else {
        for (int u = 0; u < oracle_num_tiles(p); ++u) total += oracle_list_len(p, u);
    }
    return total;
}

/* heads that own lists, and the list head of query head h */
static int32_t list_heads(const oracle_problem *p) { return p->share_gqa ? p->Hkv : p->Hq; }
static int32_t list_head(const oracle_problem *p, int h) { return p->share_gqa ? h / (p->Hq / p->Hkv) : h; }

int64_t oracle_list_offset(const oracle_problem *p, int b, int h, int t) {
    int64_t off = ((int64_t)b * list_heads(p) + list_head(p, h)) * per_head_entries(p);
    if (p->per_segment) {
        int seg = (int)(oracle_seg_start(p, t) / p->seg_len);
        for (int s = 0; s < seg; ++s) off += (int64_t)s * p->seg_len / entry_keys(p);
    } else {
        for (int u = 0; u < t; ++u) off += oracle_list_len(p, u);
    }
    return off;
}

int64_t oracle_list_entries(const oracle_problem *p) {
    int64_t n = (int64_t)p->B * list_heads(p) * per_head_entries(p);
    if (p->qperm) n += (int64_t)p->B * p->Hq * p->N; /* the query orders, after every key list */
    return n;
}

/* Q_perm: offset of the query order of segment s of (b, h): after all key
 * lists, one run of N entries per (b, h), segment by segment; entries are
 * row numbers relative to the segment start. */
int64_t oracle_query_list_offset(const oracle_problem *p, int b, int h, int s) {
    return (int64_t)p->B * list_heads(p) * per_head_entries(p) + ((int64_t)b * p->Hq + h) * p->N +
           (int64_t)s * p->seg_len;
}

static int64_t seg_rows(const oracle_problem *p, int s) {
    int64_t a = (int64_t)s * p->seg_len, e = a + p->seg_len;
    return (e > p->N ? p->N : e) - a;
}

/* ---- estimator: pool and score ------------------------------------------- */

/* ---- query permutation (Q_perm) ------------------------------------------ */

/* Guide of segment s for KV head g: the segment's mean key. */
void oracle_guide(const oracle_problem *p, const void *K, int b, int g, int s, float *guide) {
    int64_t a = (int64_t)s * p->seg_len, n = seg_rows(p, s);
    float inv = 1.0f / (float)n;
    for (int k = 0; k < p->d; ++k) {
        float sum = 0.0f;
        for (int64_t j = 0; j < n; ++j) sum = sum + widen(K, p->dtype, kv_index(p, b, g, a + j, k));
        guide[k] = sum * inv;
    }
}

/* Importance scores of the query rows of segment s of head h (fma chain
 * against the guide, ascending k), in row order. */
void oracle_query_scores(const oracle_problem *p, const void *Q, const void *K, int b, int h, int s,
                         float *out) {
    int g = h / (p->Hq / p->Hkv);
    int64_t a = (int64_t)s * p->seg_len, n = seg_rows(p, s);
    float *guide = (float *)malloc(sizeof(float) * p->d);
    oracle_guide(p, K, b, g, s, guide);
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int k = 0; k < p->d; ++k) acc = fmaf(widen(Q, p->dtype, q_index(p, b, h, a + i, k)), guide[k], acc);
        out[i] = acc;
    }
    free(guide);
}

void oracle_order(const float *scores, int64_t n, int32_t *list);

/* Rows of tile t (absolute row numbers), in tile order. */
void oracle_tile_rows(const oracle_problem *p, const void *Q, const void *K, int b, int h, int t,
                      int64_t *rows) {
    int64_t row0 = (int64_t)t * p->tile_m;
    if (!p->qperm) {
        for (int r = 0; r < p->tile_m; ++r) rows[r] = row0 + r;
        return;
    }
    int s = (int)(oracle_seg_start(p, t) / p->seg_len);
    int64_t a = (int64_t)s * p->seg_len, n = seg_rows(p, s);
    float *sc = (float *)malloc(sizeof(float) * n);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * n);
    oracle_query_scores(p, Q, K, b, h, s, sc);
    oracle_order(sc, n, order);
    for (int r = 0; r < p->tile_m; ++r) rows[r] = a + order[row0 - a + r];
    free(order);
    free(sc);
}

/* Representative query of tile t: the mean of its BM rows (fp32 sum over the
 * rows in tile order, then an exact power-of-two scaling; BM must be a power
 * of two). */
void oracle_pool(const oracle_problem *p, const void *Q, const void *K, int b, int h, int t, float *qbar) {
    float inv = 1.0f / (float)p->tile_m; /* exact for powers of two */
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * p->tile_m);
    oracle_tile_rows(p, Q, K, b, h, t, rows);
    for (int k = 0; k < p->d; ++k) {
        float sum = 0.0f;
        for (int r = 0; r < p->tile_m; ++r) sum = sum + widen(Q, p->dtype, q_index(p, b, h, rows[r], k));
        qbar[k] = sum * inv;
    }
    free(rows);
}

/* Representative query of the list tile t uses: the tile's mean, or (segment
 * lists) the mean of the segment's tile means: fp32 sum over the segment's
 * tiles in ascending order, then one multiplication by fl(1/number of tiles). */
static void rep_query_head(const oracle_problem *p, const void *Q, const void *K, int b, int h, int t,
                           float *qbar) {
    if (!p->per_segment) {
        oracle_pool(p, Q, K, b, h, t, qbar);
        return;
    }
    int P = p->seg_len / p->tile_m;
    int first = (int)(oracle_seg_start(p, t) / p->tile_m);
    int last = first + P;
    if (last > oracle_num_tiles(p)) last = oracle_num_tiles(p);
    float *tq = (float *)malloc(sizeof(float) * p->d);
    for (int k = 0; k < p->d; ++k) qbar[k] = 0.0f;
    for (int u = first; u < last; ++u) {
        oracle_pool(p, Q, K, b, h, u, tq);
        for (int k = 0; k < p->d; ++k) qbar[k] = qbar[k] + tq[k];
    }
    float inv = 1.0f / (float)(last - first);
    for (int k = 0; k < p->d; ++k) qbar[k] = qbar[k] * inv;
    free(tq);
}

/* Shared lists: the mean of the group's G per-head representatives (fp32 sum
 * over the heads in ascending order from 0, then one multiplication by
 * fl(1/G)); otherwise the head's own representative. */
void oracle_rep_query(const oracle_problem *p, const void *Q, const void *K, int b, int h, int t, float *qbar) {
    if (!p->share_gqa) {
        rep_query_head(p, Q, K, b, h, t, qbar);
        return;
    }
    int G = p->Hq / p->Hkv, h0 = (h / G) * G;
    float *hq = (float *)malloc(sizeof(float) * p->d);
    for (int k = 0; k < p->d; ++k) qbar[k] = 0.0f;
    for (int j = 0; j < G; ++j) {
        rep_query_head(p, Q, K, b, h0 + j, t, hq);
        for (int k = 0; k < p->d; ++k) qbar[k] = qbar[k] + hq[k];
    }
    float inv = 1.0f / (float)G;
    for (int k = 0; k < p->d; ++k) qbar[k] = qbar[k] * inv;
    free(hq);
}

/* Mean key of block c (keys c*BN .. c*BN+BN-1) of KV head g: fp32 sum of the
 * BN rows in ascending order, then the exact power-of-two scaling (BN must be
 * a power of two). */
void oracle_pool_block(const oracle_problem *p, const void *K, int b, int g, int64_t c, float *kbar) {
    float inv = 1.0f / (float)p->tile_n;
    for (int k = 0; k < p->d; ++k) {
        float sum = 0.0f;
        for (int r = 0; r < p->tile_n; ++r)
            sum = sum + widen(K, p->dtype, kv_index(p, b, g, c * p->tile_n + r, k));
        kbar[k] = sum * inv;
    }
}

/* Scores of the entries of the list tile t uses: s[j] = fmaf chain over
 * k = 0..d-1 of qbar[k] times key j (or the mean key of block j). */
void oracle_score_tile(const oracle_problem *p, const void *Q, const void *K, int b, int h,
                       int t, float *scores) {
    int g = h / (p->Hq / p->Hkv);
    int64_t n = oracle_list_len(p, t);
    float *qbar = (float *)malloc(sizeof(float) * p->d);
    float *kbar = (float *)malloc(sizeof(float) * p->d);
    oracle_rep_query(p, Q, K, b, h, t, qbar);
    for (int64_t j = 0; j < n; ++j) {
        if (p->block_lists)
            oracle_pool_block(p, K, b, g, j, kbar);
        else
            for (int k = 0; k < p->d; ++k) kbar[k] = widen(K, p->dtype, kv_index(p, b, g, j, k));
        float acc = 0.0f;
        for (int k = 0; k < p->d; ++k) acc = fmaf(qbar[k], kbar[k], acc);
        scores[j] = acc;
    }
    free(kbar);
    free(qbar);
}

/* ---- order: history keys by score descending, ties to the lower index ---- */

typedef struct {
    float s;
    int32_t j;
} scored_key;

static int by_score_desc_then_index(const void *x, const void *y) {
    const scored_key *a = (const scored_key *)x, *c = (const scored_key *)y;
    if (a->s > c->s) return -1;
    if (a->s < c->s) return 1; /* -0.0 and +0.0 compare equal: a tie */
    return (a->j > c->j) - (a->j < c->j);
}

void oracle_order(const float *scores, int64_t n, int32_t *list) {
    scored_key *tmp = (scored_key *)malloc(sizeof(scored_key) * (n > 0 ? n : 1));
    for (int64_t j = 0; j < n; ++j) {
        tmp[j].s = scores[j];
        tmp[j].j = (int32_t)j;
    }
    qsort(tmp, (size_t)n, sizeof(scored_key), by_score_desc_then_index);
    for (int64_t j = 0; j < n; ++j) list[j] = tmp[j].j;
    free(tmp);
}

/* ---- attention: pass 1 + pass 2 with early stop -------------------------- */

typedef struct {
    double m, l;
    double *acc;
} row_state;

/* logit x_ij = scale * dot(Q_i, K_j) in double */
static double logit(const oracle_problem *p, const void *Q, const void *K, int b, int h, int g,
                    int64_t i, int64_t j) {
    double dot = 0.0;
    for (int k = 0; k < p->d; ++k)
        dot += (double)widen(Q, p->dtype, q_index(p, b, h, i, k)) *
               (double)widen(K, p->dtype, kv_index(p, b, g, j, k));
    return p->scale * dot;
}

/* Online-softmax update of one row with a set of keys; returns the set's mass
 * sum_j exp(x_ij - m_new) measured against the updated running max. */
static double absorb(const oracle_problem *p, const void *Q, const void *K, const void *V,
                     int b, int h, int g, int64_t i, const int64_t *keys, int nkeys,
                     row_state *st, double *x) {
    double m_new = st->m;
    for (int e = 0; e < nkeys; ++e) {
        x[e] = logit(p, Q, K, b, h, g, i, keys[e]);
        if (x[e] > m_new) m_new = x[e];
    }
    double rescale = exp(st->m - m_new); /* exp(-inf) = 0 on the first update */
    double mass = 0.0;
    st->l *= rescale;
    for (int k = 0; k < p->d; ++k) st->acc[k] *= rescale;
    for (int e = 0; e < nkeys; ++e) {
        double w = exp(x[e] - m_new);
        mass += w;
        for (int k = 0; k < p->d; ++k) st->acc[k] += w * (double)widen(V, p->dtype, kv_index(p, b, g, keys[e], k));
    }
    st->l += mass;
    st->m = m_new;
    return mass;
}

/*
 * One query tile.  `list` holds the tile's a_t history indices in visiting
 * order (block lists: its a_t / BN block indices; chunk c is block list[c]).  tau >= 0.  force_n > 0 executes exactly min(force_n, C_t) pass-2
 * chunks regardless of tau (used to re-check a tile at a given chunk count).
 * Outputs: out[BM*d] in double, *n_exec = pass-1 tiles + executed chunks,
 * gstar[c] = max_i g_i of chunk c for the executed chunks (may be NULL).
 * Returns the number of executed pass-2 chunks.
 */
int32_t oracle_attn_tile(const oracle_problem *p, const void *Q, const void *K, const void *V,
                         int b, int h, int t, const int32_t *list, double tau, int32_t force_n,
                         double *out, int32_t *n_exec, double *gstar) {
    int BM = p->tile_m, BN = p->tile_n, d = p->d;
    int g = h / (p->Hq / p->Hkv);
    int64_t a = oracle_seg_start(p, t);
    int32_t chunks = (int32_t)(a / BN);
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * BM);
    oracle_tile_rows(p, Q, K, b, h, t, rows);
    int64_t last = rows[0];
    for (int r = 1; r < BM; ++r)
        if (rows[r] > last) last = rows[r];
    row_state *st = (row_state *)malloc(sizeof(row_state) * BM);
    double *accs = (double *)calloc((size_t)BM * d, sizeof(double));
    double *x = (double *)malloc(sizeof(double) * BN);
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * BN);
    for (int r = 0; r < BM; ++r) {
        st[r].m = -INFINITY;
        st[r].l = 0.0;
        st[r].acc = accs + (size_t)r * d;
    }

    /* pass 1: contiguous key tiles of the current segment up to the tile's last
     * row, each row under its own causal mask */
    int32_t p1 = (int32_t)((last + 1 - a + BN - 1) / BN);
    for (int32_t c = 0; c < p1; ++c) {
        int64_t k0 = a + (int64_t)c * BN;
        for (int r = 0; r < BM; ++r) {
            int64_t i = rows[r];
            int n = 0;
            for (int e = 0; e < BN; ++e)
                if (k0 + e <= i) keys[n++] = k0 + e;
            if (n > 0) absorb(p, Q, K, V, b, h, g, i, keys, n, &st[r], x);
        }
    }

    /* pass 2: list chunks in order, early stop on the marginal gain */
    int32_t executed = 0;
    int32_t limit = (force_n > 0 && force_n < chunks) ? force_n : chunks;
    for (int32_t c = 0; c < limit; ++c) {
        for (int e = 0; e < BN; ++e)
            keys[e] = p->block_lists ? (int64_t)list[c] * BN + e : list[(int64_t)c * BN + e];
        double worst = 0.0; /* max over rows of g_i */
        for (int r = 0; r < BM; ++r) {
            double mass = absorb(p, Q, K, V, b, h, g, rows[r], keys, BN, &st[r], x);
            double gain = mass / st[r].l;
            if (gain > worst) worst = gain;
        }
        if (gstar) gstar[c] = worst;
        executed = c + 1;
        if (force_n <= 0 && worst < tau) break;
    }

    for (int r = 0; r < BM; ++r)
        for (int k = 0; k < d; ++k) out[(size_t)r * d + k] = st[r].acc[k] / st[r].l;
    *n_exec = p1 + executed;
    free(rows);
    free(keys);
    free(x);
    free(accs);
    free(st);
    return executed;
}

/* Dense causal softmax attention for rows [i0, i1) of (b, h), in double. */
void oracle_dense_rows(const oracle_problem *p, const void *Q, const void *K, const void *V,
                       int b, int h, int64_t i0, int64_t i1, double *out) {
    int g = h / (p->Hq / p->Hkv);
    double *x = (double *)malloc(sizeof(double) * p->N);
    for (int64_t i = i0; i < i1; ++i) {
        double mx = -INFINITY, den = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
            x[j] = logit(p, Q, K, b, h, g, i, j);
            if (x[j] > mx) mx = x[j];
        }
        double *o = out + (size_t)(i - i0) * p->d;
        for (int k = 0; k < p->d; ++k) o[k] = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
            double w = exp(x[j] - mx);
            den += w;
            for (int k = 0; k < p->d; ++k) o[k] += w * (double)widen(V, p->dtype, kv_index(p, b, g, j, k));
        }
        for (int k = 0; k < p->d; ++k) o[k] /= den;
    }
    free(x);
}

/* ---- whole problems and tile samples (OpenMP over tiles) ----------------- */

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The tile that owns list number u of a head: the tile itself (tile lists) or
 * the first tile of segment u (segment lists). */
static int list_owner(const oracle_problem *p, int u) {
    return p->per_segment ? u * (p->seg_len / p->tile_m) : u;
}

static int lists_per_head(const oracle_problem *p) {
    return p->per_segment ? num_segments(p) : oracle_num_tiles(p);
}

/* scores of every list, in the list layout */
void oracle_scores_all(const oracle_problem *p, const void *Q, const void *K, float *scores) {
    int32_t U = lists_per_head(p), LH = list_heads(p), G = p->Hq / LH;
    int64_t units = (int64_t)p->B * LH * U;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        int b = (int)(u / ((int64_t)LH * U)), h = (int)((u / U) % LH) * G; /* first head using the list */
        int t = list_owner(p, (int)(u % U));
        if (oracle_list_len(p, t) > 0)
            oracle_score_tile(p, Q, K, b, h, t, scores + oracle_list_offset(p, b, h, t));
    }
    if (!p->qperm) return;
    int32_t nseg = num_segments(p);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < (int64_t)p->B * p->Hq * nseg; ++u) {
        int b = (int)(u / ((int64_t)p->Hq * nseg)), h = (int)((u / nseg) % p->Hq), s = (int)(u % nseg);
        oracle_query_scores(p, Q, K, b, h, s, scores + oracle_query_list_offset(p, b, h, s));
    }
}

/* every list from the scores */
void oracle_lists_all(const oracle_problem *p, const float *scores, int32_t *lists) {
    int32_t U = lists_per_head(p), LH = list_heads(p), G = p->Hq / LH;
    int64_t units = (int64_t)p->B * LH * U;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        int b = (int)(u / ((int64_t)LH * U)), h = (int)((u / U) % LH) * G; /* first head using the list */
        int t = list_owner(p, (int)(u % U));
        int64_t off = oracle_list_offset(p, b, h, t);
        oracle_order(scores + off, oracle_list_len(p, t), lists + off);
    }
    if (!p->qperm) return;
    int32_t nseg = num_segments(p);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < (int64_t)p->B * p->Hq * nseg; ++u) {
        int b = (int)(u / ((int64_t)p->Hq * nseg)), h = (int)((u / nseg) % p->Hq), s = (int)(u % nseg);
        int64_t off = oracle_query_list_offset(p, b, h, s);
        oracle_order(scores + off, seg_rows(p, s), lists + off);
    }
}

/*
 * A set of tiles, each given as (b, h, t) in tiles[3*n..3*n+2].  For each:
 * scores, list, pass 1 and pass 2.  `lists_in` (may be NULL) supplies the full
 * list buffer in the (b, h, t) layout; when NULL the tile's list is computed
 * here.  Outputs per tile n: out[n*BM*d ...] (double), n_exec[n], chunks[n];
 * gstar (may be NULL) has room for max_chunks entries per tile; list_out (may
 * be NULL) receives each tile's list at offset n*max_list.
 * force_n (may be NULL) gives a per-tile forced chunk count (0 = use tau).
 */
void oracle_attn_tiles(const oracle_problem *p, const void *Q, const void *K, const void *V,
                       const int32_t *tiles, int64_t n_tiles, const int32_t *lists_in,
                       double tau, const int32_t *force_n, double *out, int32_t *n_exec,
                       int32_t *chunks, double *gstar, int64_t max_chunks, int32_t *list_out,
                       int64_t max_list) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_tiles; ++n) {
        int b = tiles[3 * n], h = tiles[3 * n + 1], t = tiles[3 * n + 2];
        int64_t a = oracle_list_len(p, t);
        int32_t *list;
        int32_t *owned = NULL;
        if (lists_in) {
            list = (int32_t *)lists_in + oracle_list_offset(p, b, h, t);
        } else {
            float *s = (float *)malloc(sizeof(float) * (a > 0 ? a : 1));
            owned = (int32_t *)malloc(sizeof(int32_t) * (a > 0 ? a : 1));
            if (a > 0) oracle_score_tile(p, Q, K, b, h, t, s);
            oracle_order(s, a, owned);
            free(s);
            list = owned;
        }
        if (list_out)
            for (int64_t j = 0; j < a; ++j) list_out[n * max_list + j] = list[j];
        chunks[n] = oracle_attn_tile(p, Q, K, V, b, h, t, list, tau, force_n ? force_n[n] : 0,
                                     out + (size_t)n * p->tile_m * p->d, &n_exec[n],
                                     gstar ? gstar + n * max_chunks : NULL);
        free(owned);
    }
}

/* dense rows for a set of (b, h, i0, i1) requests, out packed in order */
void oracle_dense_requests(const oracle_problem *p, const void *Q, const void *K, const void *V,
                           const int64_t *req, int64_t n_req, const int64_t *out_off, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_req; ++n)
        oracle_dense_rows(p, Q, K, V, (int)req[4 * n], (int)req[4 * n + 1], req[4 * n + 2],
                          req[4 * n + 3], out + out_off[n]);
}
