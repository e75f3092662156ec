/*
 * s2o.h -- C ABI of the MI355X (gfx950) S2O causal-prefill attention library.
 *
 * The method ("S2O: Early Stopping for Sparse Attention via Online
 * Permutation", Zhang et al., arXiv 2602.22575) keeps K/V in their original
 * order in HBM and visits history keys through small index lists ordered by an
 * importance estimate, stopping once a chunk's marginal softmax mass is small.
 * Sources cited below:
 *   [ABS]  the authors' abstract (pith.science page, "read the original abstract")
 *   [GIST] the gist.science technical summary, sections "Classement par
 *          Segment", "Chargement Planifié par Coordonnées", "2. Règle d'Arrêt
 *          Anticipé", "3. Implémentation du Noyau" (Passage 1 / Passage 2)
 *   [LENS] the arxivlens summary (Methodology, Limitations: tuning parameters are
 *          segment length, early-stopping threshold and scheduling parameters)
 *
 * Conventions for every call
 *   - Q is [B, Hq, N, d], K and V are [B, Hkv, N, d], O is [B, Hq, N, d]; all
 *     contiguous, row-major, d innermost, in the dtype named by the problem.
 *     Query head h reads KV head h / (Hq / Hkv).
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and is re-entrant.
 *     Inputs are read-only; outputs are fully overwritten; inputs must not
 *     alias outputs (not checked).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on that stream: arguments are validated on
 *     the host before anything is enqueued, and a failed validation enqueues
 *     nothing.  Faults during execution surface at the caller's next
 *     synchronisation, as usual in HIP.  No exception crosses the ABI.
 *   - Inputs must be finite; behaviour with NaN or Inf inputs is undefined.
 *
 * Geometry (per query head; [GIST] Classement par Segment)
 *   BM = tile_m query rows per tile, BN = tile_n keys per key tile / list chunk,
 *   T = N / BM tiles, S = seg_len.  Tile t covers rows [t*BM, (t+1)*BM); its
 *   segment starts at a_t = floor(t*BM / S) * S; its history is keys [0, a_t).
 *
 * List layout (scores and idx)
 *   Per-tile lists: one per (b, h, t), concatenated in (b, h, t) row-major
 *   order; tile t's list has a_t entries (segment-0 lists are empty).  With
 *   P = S / BM, s = floor(t / P) and L = one head's total,
 *     off(b, h, t) = (b*Hq + h)*L + S*(P*s*(s-1)/2 + (t - s*P)*s).
 *   Per-segment lists: one per (b, h, s), list s has s*S entries,
 *     off(b, h, s) = (b*Hq + h)*L + S*s*(s-1)/2, and tile t uses list floor(t/P).
 *   Block lists: the same layouts with every length and history term divided
 *     by tile_n; idx values are block numbers in [0, a_t / tile_n).
 *   Shared lists (S2O_SHARE_GQA): (b*Hkv + h/G) in place of (b*Hq + h), so the
 *     G = Hq / Hkv query heads of a KV head use one list.
 *   Entries are int64-addressed; idx values are key positions in [0, a_t).
 */
#ifndef S2O_H
#define S2O_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    S2O_OK = 0,
    S2O_ERR_INVALID_ARG = -1, /* null pointer, bad size or divisibility, bad tau */
    S2O_ERR_UNSUPPORTED = -2, /* valid request with no compiled kernel, causal = 0 for s2o_*,
                                 or sizes past the kernels' index ranges (e.g. N*d*2 >= 2^31) */
    S2O_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_bytes query */
    S2O_ERR_HIP = -4          /* a HIP launch failed */
} s2o_status;

typedef enum { S2O_F32 = 0, S2O_BF16 = 1 } s2o_dtype;

typedef struct {
    int32_t batch;    /* B  > 0 */
    int32_t heads_q;  /* Hq > 0 */
    int32_t heads_kv; /* Hkv > 0, divides Hq */
    int32_t seq_len;  /* N  > 0, multiple of tile_m */
    int32_t head_dim; /* d in {64, 128} */
    int32_t dtype;    /* s2o_dtype of Q, K, V and O */
    int32_t causal;   /* 1: causal mask.  The s2o_* calls require 1 (the method is
                         defined for causal prefill, [GIST] Classement par Segment) */
    int32_t seg_len;  /* S > 0, multiple of tile_m; N need not be a multiple of S */
    int32_t tile_m;   /* BM: 64 or 128 */
    int32_t tile_n;   /* BN: 64 */
    float scale;      /* softmax scale (1/sqrt(d) for standard attention): finite and > 0,
                         else S2O_ERR_INVALID_ARG */
    int32_t list_granularity; /* one of the S2O_LISTS_* values below, optionally ORed with
                                 S2O_QUERY_PERMUTATION or S2O_SHARE_GQA */
} s2o_problem;

/* Which query a list is ranked against ([GIST] KV_perm), and what an entry is.
 *   S2O_LISTS_PER_TILE: one list per (b, h, query tile), ranked against the
 *     tile's mean query;
 *   S2O_LISTS_PER_SEGMENT: one list per (b, h, segment), shared by the
 *     segment's tiles and ranked against the segment's representative query =
 *     fp32 sum of its tile means in ascending tile order times fl(1/tiles).
 *   ..._BLOCKS: the same lists with blocks of tile_n consecutive keys as
 *     entries (the block-granularity counterpart the pages compare S2O with,
 *     [ABS]): block c is scored with its mean key (fp32 sum of its rows in
 *     ascending order, times 1/tile_n), every list is 1/tile_n as long, and
 *     pass-2 chunk c is the tile_n keys of the c-th listed block. */
enum {
    S2O_LISTS_PER_TILE = 0,
    S2O_LISTS_PER_SEGMENT = 1,
    S2O_LISTS_PER_TILE_BLOCKS = 2,
    S2O_LISTS_PER_SEGMENT_BLOCKS = 3
};

/* Flag to OR into list_granularity: query permutation ([GIST] Classement par
 * Segment, Q_perm).  Inside each segment the query rows are ordered by their
 * score against a shared guide vector, here the segment's mean key (fp32 sum
 * of its key rows in ascending order, times fl(1/rows)); a row's score is the
 * fp32 fma chain over k of Q[row, k] * guide[k]; rows are sorted by score
 * descending, ties to the lower row.  Query tile t of a segment holds the rows
 * at positions t*BM .. t*BM+BM-1 of that order (positions count from the
 * segment start like rows); its representative query is the fp32 sum of those
 * rows in that order times 1/BM.  In attention each row keeps its own causal
 * window (pass 1 covers key tiles up to the tile's last row) and its output
 * goes to its own row.  The order of segment s of (b, h) is stored after all
 * key lists: at (total key-list entries) + (b*Hq + h)*N + s*S, as row numbers
 * relative to the segment start; the matching scores sit at the same offsets.
 * bf16 problems with seg_len <= 8192 only (else S2O_ERR_UNSUPPORTED). */
enum { S2O_QUERY_PERMUTATION = 4 };

/* Flag to OR into list_granularity: shared lists (the GQA form of [GIST]
 * KV_perm's shared index map).  One list per (b, KV head, tile or segment)
 * instead of per query head, read by the G query heads of the group; it is
 * ranked against the mean of the G heads' representatives (fp32 sum over the
 * heads in ascending order from 0, times fl(1/G)).  Lists are laid out as
 * above with (b*Hkv + h/G) in place of (b*Hq + h), so there are B*Hkv*L
 * entries.  Not with S2O_QUERY_PERMUTATION (S2O_ERR_UNSUPPORTED). */
enum { S2O_SHARE_GQA = 8 };

/* Validates a problem (sizes, divisibility, supported tiles).  Returns S2O_OK,
 * S2O_ERR_INVALID_ARG or S2O_ERR_UNSUPPORTED.  Pure host function. */
s2o_status s2o_check_problem(const s2o_problem *p);

/* Total list entries over all lists (per tile: B*Hq*sum_t a_t; per segment:
 * B*Hq*sum_s s*S; Hkv in place of Hq with S2O_SHARE_GQA; divided by tile_n
 * for block lists; plus B*Hq*N query-order entries with
 * S2O_QUERY_PERMUTATION).  -1 if the problem is invalid.  Pure
 * host function. */
int64_t s2o_list_entries(const s2o_problem *p);

/* Offset of the list tile t of (b, h) uses, in the layout above; -1 if out of
 * range or the problem is invalid.  Pure host function. */
int64_t s2o_list_offset(const s2o_problem *p, int32_t b, int32_t h, int32_t t);

/* Bytes of device workspace s2o_score needs (the pooled query of every tile
 * and, for per-segment lists, of every segment; for block lists also the mean
 * key of every block; all fp32).  0 if the problem is invalid. */
size_t s2o_score_workspace_bytes(const s2o_problem *p);

/* Importance estimator ([GIST] KV_perm: history keys are scored against a
 * representative query; only causal-prefix keys count).  For every list with
 * history: qbar = the tile's mean query (fp32 sum over its BM rows in ascending
 * order, then an exact scaling by 1/BM) or, for per-segment lists, the
 * segment's representative described above (with S2O_SHARE_GQA, the mean of
 * the group's G such representatives); then
 *   scores[off + j] = fp32 fma chain over k = 0..d-1 of qbar[k] * K[b, h/G, j, k],
 * accumulated from 0 in ascending k, for j in [0, history length).  This order
 * is part of the definition, so results are bit-reproducible.
 *   Q, K: device, problem dtype.  scores: device fp32 [s2o_list_entries].
 *   workspace: device, >= s2o_score_workspace_bytes, 256-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (causal = 0), WORKSPACE, HIP. */
s2o_status s2o_score(const s2o_problem *p, const void *Q, const void *K, float *scores,
                     void *workspace, size_t workspace_bytes, void *stream);

/* s2o_score without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as s2o_score, bit for
 * bit; the workspace is a static device array of
 * S2O_SCORE_NOALLOC_MAX_WORKSPACE bytes that every GPU the library runs on
 * holds until the process ends (its address is looked up on the first call on
 * each device).  The call allocates nothing.  Calls on one GPU share that
 * array, so calls that overlap on one GPU (other streams, other host threads)
 * race: serialise them.  Problems whose s2o_score_workspace_bytes exceeds the
 * maximum return S2O_ERR_WORKSPACE before anything is enqueued (64 MiB holds
 * every list form of one 128K-token Llama-3.1-8B-shaped layer).
 * Errors: as s2o_score, plus WORKSPACE for a problem above the maximum and HIP
 * when the array's device address cannot be obtained. */
#define S2O_SCORE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
s2o_status s2o_score_noalloc(const s2o_problem *p, const void *Q, const void *K, float *scores,
                             void *stream);

/* Bytes of device workspace s2o_build_index needs.  0 if the problem is invalid. */
size_t s2o_build_index_workspace_bytes(const s2o_problem *p);

/* Index build ([GIST] KV_perm: the resulting indices form a global logical map
 * that puts likely vertical and slash stripes first).  For every list, idx
 * receives the positions [0, history length) sorted by score descending, ties
 * broken by the lower position; -0.0 and +0.0 tie.  A segmented sort: one
 * bucketing pass between bounds sampled from each list's scores (scores
 * outside them join the end buckets), then each range of buckets is ranked
 * exactly by (score, position) inside value sub-buckets (crowded or oversized
 * ranges by radix passes instead).  The result is deterministic: the order
 * inside a bucket is arbitrary, the final ranking is not.
 *   scores: device fp32 [s2o_list_entries] (from s2o_score), 16-byte aligned.
 *   idx: device int32 [s2o_list_entries], 16-byte aligned.
 *   workspace: device, >= s2o_build_index_workspace_bytes, 256-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (causal = 0), WORKSPACE, HIP. */
s2o_status s2o_build_index(const s2o_problem *p, const float *scores, int32_t *idx,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Gathered attention with early stop ([GIST] 3. Implémentation du Noyau;
 * [GIST] 2. Règle d'Arrêt Anticipé; [ABS]).  Per tile t and row i:
 *   pass 1: online softmax over keys [a_t, i] (dense causal window inside the
 *           segment), initialising (m, l, acc);
 *   pass 2: for chunks c = 0, 1, ... of BN consecutive entries of the list the
 *           tile uses, gather those K/V rows, update (m, l, acc), and take the chunk
 *           mass delta_i = sum exp(x_ij - m_i) against the updated max; stop
 *           after chunk c when delta_i < tau * l_i (l after the chunk) for every
 *           row of the tile.  The stopping chunk is kept; tau = 0 never stops.
 *   O_i = acc_i / l_i in the problem dtype.  exec_tiles[b, h, t] = pass-1 key
 *   tiles + executed chunks (int32 [B, Hq, N/BM]; may be NULL).
 * QK^T and PV run on bf16 MFMA with an fp32 softmax for bf16 problems (P is
 * rounded to bf16 for PV; l and delta use fp32 P), and on fp32 MFMA for fp32
 * problems.
 *   idx: device int32 lists from s2o_build_index (or any lists in the layout
 *        above whose entries are in [0, a_t), and with S2O_QUERY_PERMUTATION
 *        query orders that are permutations of each segment's rows).
 *   tau: >= 0 and not NaN.
 * Errors: INVALID_ARG, UNSUPPORTED (causal = 0), HIP. */
s2o_status s2o_attn_fwd(const s2o_problem *p, const void *Q, const void *K, const void *V,
                        const int32_t *idx, float tau, void *O, int32_t *exec_tiles,
                        void *stream);

/* Dense softmax attention (the FlashAttention baseline the pages compare
 * against, [GIST] Résultats Expérimentaux), causal or not per p->causal, with
 * the same tiles and numerics as s2o_attn_fwd.  seg_len is ignored.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
s2o_status dense_attn_fwd(const s2o_problem *p, const void *Q, const void *K, const void *V,
                          void *O, void *stream);

/* Static description of a status code. */
const char *s2o_status_string(s2o_status s);

#ifdef __cplusplus
}
#endif

#endif /* S2O_H */
