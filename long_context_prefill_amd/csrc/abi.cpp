// C ABI entry points: host-side validation, geometry and dispatch.  The
// contract of every function is documented in include/s2o.h.
#include <math.h>

#include "s2o.h"
#include "s2o_internal.h"

namespace {

using s2o::Geometry;

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The problem scoring and sorting see: shared lists as one query head per KV
// head, block lists as a problem whose keys are blocks.
Geometry list_geometry(const Geometry &g) {
    const Geometry r = s2o::group_geometry(g);
    return g.blocks ? s2o::block_geometry(r) : r;
}

// Fills g from p, or returns the reason it cannot.
s2o_status make_geometry(const s2o_problem *p, Geometry &g) {
    if (!p) return S2O_ERR_INVALID_ARG;
    if (p->batch <= 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->seq_len <= 0 ||
        p->head_dim <= 0 || p->seg_len <= 0 || p->tile_m <= 0 || p->tile_n <= 0)
        return S2O_ERR_INVALID_ARG;
    if (p->dtype != S2O_F32 && p->dtype != S2O_BF16) return S2O_ERR_INVALID_ARG;
    if (p->causal != 0 && p->causal != 1) return S2O_ERR_INVALID_ARG;
    // the kernels mask with -inf before scaling and take row maxima on raw
    // logits, which needs a positive scale
    if (!isfinite(p->scale) || !(p->scale > 0.0f)) return S2O_ERR_INVALID_ARG;
    if (p->heads_q % p->heads_kv != 0) return S2O_ERR_INVALID_ARG;
    if (p->tile_m % p->tile_n != 0 || p->seq_len % p->tile_m != 0 || p->seg_len % p->tile_m != 0)
        return S2O_ERR_INVALID_ARG;
    if (!pow2(p->tile_m)) return S2O_ERR_INVALID_ARG;  // the pooled mean scales by 1/BM exactly
    // compiled kernels
    if (p->head_dim != 64 && p->head_dim != 128) return S2O_ERR_UNSUPPORTED;
    if (p->tile_m != 64 && p->tile_m != 128) return S2O_ERR_UNSUPPORTED;
    if (p->tile_n != s2o::kTileN) return S2O_ERR_UNSUPPORTED;
    if (p->list_granularity < 0 || p->list_granularity > 15) return S2O_ERR_INVALID_ARG;
    if ((p->list_granularity & S2O_QUERY_PERMUTATION) &&
        (p->dtype != S2O_BF16 || p->seg_len > s2o::kQuerySortCap))
        return S2O_ERR_UNSUPPORTED;
    if ((p->list_granularity & S2O_QUERY_PERMUTATION) && (p->list_granularity & S2O_SHARE_GQA))
        return S2O_ERR_UNSUPPORTED;

    g.B = p->batch;
    g.Hq = p->heads_q;
    g.Hkv = p->heads_kv;
    g.G = p->heads_q / p->heads_kv;
    g.N = p->seq_len;
    g.d = p->head_dim;
    g.S = p->seg_len;
    g.BM = p->tile_m;
    g.BN = p->tile_n;
    g.T = p->seq_len / p->tile_m;
    g.P = p->seg_len / p->tile_m;
    g.causal = p->causal;
    g.dtype = p->dtype;
    g.scale = p->scale;
    g.per_seg = p->list_granularity & 1;
    g.blocks = (p->list_granularity >> 1) & 1;
    g.qperm = (p->list_granularity >> 2) & 1;
    g.share = (p->list_granularity >> 3) & 1;
    g.nseg = (g.N + g.S - 1) / g.S;
    g.inv_P = 1.0f / (float)g.P;
    g.inv_P_last = 1.0f / (float)(g.T - (g.nseg - 1) * g.P);
    // L: history entries of one head's lists, walking the segments
    int64_t L = 0;
    for (int64_t s = 0; s < g.nseg; ++s) {
        int64_t tiles = (int64_t)g.P;
        int64_t first = s * g.P;
        if (first + tiles > g.T) tiles = g.T - first;
        L += (g.per_seg ? 1 : tiles) * s * g.S;
    }
    if (g.blocks) L /= g.BN;  // every history is a multiple of S, and S of BN
    g.list_per_head = L;
    g.list_entries = L * g.B * (g.share ? g.Hkv : g.Hq);
    g.query_entries = g.qperm ? (int64_t)g.B * g.Hq * g.N : 0;
    // index ranges the kernels assume (the attention kernel addresses one KV
    // head's K or V, and a tile's list, with 32-bit byte offsets)
    if ((int64_t)g.N * g.d * 2 >= (1ll << 31)) return S2O_ERR_UNSUPPORTED;
    const int64_t units = (int64_t)g.B * g.Hkv * g.T;
    if ((int64_t)g.B * g.Hq * g.T >= (1ll << 31) || ((units + 7) / 8) * 8 * g.G >= (1ll << 31))
        return S2O_ERR_UNSUPPORTED;
    const int64_t nseg = (g.N + g.S - 1) / g.S;
    if ((int64_t)g.B * g.Hkv * nseg > 65535) return S2O_ERR_UNSUPPORTED;
    const Geometry lg = list_geometry(g);
    int64_t e = lg.S & (-lg.S);
    if (e > 4096) e = 4096;
    if (lg.list_entries / e >= (1ll << 31)) return S2O_ERR_UNSUPPORTED;
    if (!s2o::sort_supported(lg)) return S2O_ERR_UNSUPPORTED;
    return S2O_OK;
}

s2o_status launch_status(hipError_t e) { return e == hipSuccess ? S2O_OK : S2O_ERR_HIP; }

bool workspace_ok(void *ws, size_t have, size_t need) {
    if (need == 0) return true;
    if (!ws || have < need) return false;
    return (reinterpret_cast<uintptr_t>(ws) & 255u) == 0;
}

}  // namespace

extern "C" {

s2o_status s2o_check_problem(const s2o_problem *p) {
    Geometry g;
    return make_geometry(p, g);
}

int64_t s2o_list_entries(const s2o_problem *p) {
    Geometry g;
    if (make_geometry(p, g) != S2O_OK) return -1;
    return g.list_entries + g.query_entries;
}

int64_t s2o_list_offset(const s2o_problem *p, int32_t b, int32_t h, int32_t t) {
    Geometry g;
    if (make_geometry(p, g) != S2O_OK) return -1;
    if (b < 0 || b >= g.B || h < 0 || h >= g.Hq || t < 0 || t >= g.T) return -1;
    return s2o::list_offset(g, b, h, t);
}

namespace {
size_t tile_query_bytes(const Geometry &g) { return ((size_t)g.B * g.Hq * g.T * g.d * sizeof(float) + 255) & ~(size_t)255; }
size_t segment_query_bytes(const Geometry &g) {
    return g.per_seg ? (((size_t)g.B * g.Hq * g.nseg * g.d * sizeof(float) + 255) & ~(size_t)255) : 0;
}
size_t block_key_bytes(const Geometry &g) {
    return g.blocks ? (((size_t)g.B * g.Hkv * (g.N / g.BN) * g.d * sizeof(float) + 255) & ~(size_t)255) : 0;
}
size_t group_query_bytes(const Geometry &g) {
    return g.share ? (((size_t)g.B * g.Hkv * (g.per_seg ? g.nseg : g.T) * g.d * sizeof(float) + 255) & ~(size_t)255)
                   : 0;
}
size_t guide_bytes(const Geometry &g) {
    return g.qperm ? (((size_t)g.B * g.Hkv * g.nseg * g.d * sizeof(float) + 255) & ~(size_t)255) : 0;
}
size_t query_order_bytes(const Geometry &g) {
    return g.qperm ? (((size_t)g.query_entries * sizeof(int32_t) + 255) & ~(size_t)255) : 0;
}
}

size_t s2o_score_workspace_bytes(const s2o_problem *p) {
    Geometry g;
    if (make_geometry(p, g) != S2O_OK) return 0;
    return tile_query_bytes(g) + segment_query_bytes(g) + block_key_bytes(g) + guide_bytes(g) +
           query_order_bytes(g) + group_query_bytes(g);
}

s2o_status s2o_score(const s2o_problem *p, const void *Q, const void *K, float *scores,
                     void *workspace, size_t workspace_bytes, void *stream) {
    Geometry g;
    s2o_status st = make_geometry(p, g);
    if (st != S2O_OK) return st;
    if (!g.causal) return S2O_ERR_UNSUPPORTED;
    if (!Q || !K || !aligned16(Q) || !aligned16(K)) return S2O_ERR_INVALID_ARG;
    if (g.list_entries + g.query_entries > 0 && (!scores || !aligned16(scores))) return S2O_ERR_INVALID_ARG;
    if (!workspace_ok(workspace, workspace_bytes, s2o_score_workspace_bytes(p))) return S2O_ERR_WORKSPACE;
    if (g.list_entries + g.query_entries == 0) return S2O_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = reinterpret_cast<char *>(workspace);
    float *qbar = reinterpret_cast<float *>(ws);
    float *qseg = g.per_seg ? reinterpret_cast<float *>(ws + tile_query_bytes(g)) : nullptr;
    char *after = ws + tile_query_bytes(g) + segment_query_bytes(g);
    float *kbar = reinterpret_cast<float *>(after);
    float *guides = reinterpret_cast<float *>(after + block_key_bytes(g));
    int32_t *qorder = reinterpret_cast<int32_t *>(after + block_key_bytes(g) + guide_bytes(g));
    float *qgrp = reinterpret_cast<float *>(after + block_key_bytes(g) + guide_bytes(g) + query_order_bytes(g));
    hipError_t e;
    if (g.qperm) {  // Q_perm: query scores (after the key lists) and the query order
        e = s2o::launch_query_scores(g, Q, K, guides, scores + g.list_entries, s);
        if (e != hipSuccess) return S2O_ERR_HIP;
        e = s2o::launch_query_sort(g, scores + g.list_entries, qorder, s);
        if (e != hipSuccess) return S2O_ERR_HIP;
    }
    if (g.list_entries == 0) return S2O_OK;
    e = s2o::launch_pool(g, Q, g.qperm ? qorder : nullptr, qbar, qseg, s);
    if (e != hipSuccess) return S2O_ERR_HIP;
    const float *rep = g.per_seg ? qseg : qbar;
    if (g.share) {  // shared lists: one representative per KV head
        e = s2o::launch_group_mean(g, rep, g.per_seg ? g.nseg : g.T, qgrp, s);
        if (e != hipSuccess) return S2O_ERR_HIP;
        rep = qgrp;
    }
    const Geometry sg = s2o::group_geometry(g);
    if (!g.blocks) return launch_status(s2o::launch_score(sg, rep, K, scores, s));
    // block lists: score the blocks' mean keys as the keys of the block geometry
    e = s2o::launch_pool_blocks(g, K, kbar, s);
    if (e != hipSuccess) return S2O_ERR_HIP;
    return launch_status(s2o::launch_score(s2o::block_geometry(sg), rep, kbar, scores, s));
}

size_t s2o_build_index_workspace_bytes(const s2o_problem *p) {
    Geometry g;
    if (make_geometry(p, g) != S2O_OK) return 0;
    return s2o::sort_workspace_bytes(list_geometry(g));
}

s2o_status s2o_build_index(const s2o_problem *p, const float *scores, int32_t *idx,
                           void *workspace, size_t workspace_bytes, void *stream) {
    Geometry g;
    s2o_status st = make_geometry(p, g);
    if (st != S2O_OK) return st;
    if (!g.causal) return S2O_ERR_UNSUPPORTED;
    if (g.list_entries + g.query_entries > 0 && (!scores || !idx || !aligned16(scores) || !aligned16(idx)))
        return S2O_ERR_INVALID_ARG;
    const Geometry lg = list_geometry(g);
    if (!workspace_ok(workspace, workspace_bytes, s2o::sort_workspace_bytes(lg))) return S2O_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (g.list_entries > 0) {
        hipError_t e = s2o::launch_sort(lg, scores, idx, workspace, s);
        if (e != hipSuccess) return S2O_ERR_HIP;
    }
    if (g.qperm)  // the query order, after the key lists
        return launch_status(s2o::launch_query_sort(g, scores + g.list_entries, idx + g.list_entries, s));
    return S2O_OK;
}

s2o_status s2o_attn_fwd(const s2o_problem *p, const void *Q, const void *K, const void *V,
                        const int32_t *idx, float tau, void *O, int32_t *exec_tiles, void *stream) {
    Geometry g;
    s2o_status st = make_geometry(p, g);
    if (st != S2O_OK) return st;
    if (!g.causal) return S2O_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O || !aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return S2O_ERR_INVALID_ARG;
    if (g.list_entries + g.query_entries > 0 && !idx) return S2O_ERR_INVALID_ARG;
    if (isnan(tau) || tau < 0.0f) return S2O_ERR_INVALID_ARG;
    return launch_status(s2o::launch_attention(g, Q, K, V, idx, g.qperm ? idx + g.list_entries : nullptr, tau, O,
                                               exec_tiles, true, reinterpret_cast<hipStream_t>(stream)));
}

s2o_status dense_attn_fwd(const s2o_problem *p, const void *Q, const void *K, const void *V,
                          void *O, void *stream) {
    Geometry g;
    s2o_problem q = p ? *p : s2o_problem{};
    if (p) {
        q.seg_len = p->seq_len;  // one segment: the dense schedule has no lists
        q.list_granularity = S2O_LISTS_PER_TILE;
    }
    s2o_status st = make_geometry(p ? &q : nullptr, g);
    if (st != S2O_OK) return st;
    if (!Q || !K || !V || !O || !aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return S2O_ERR_INVALID_ARG;
    return launch_status(s2o::launch_attention(g, Q, K, V, nullptr, nullptr, 0.0f, O, nullptr, false,
                                               reinterpret_cast<hipStream_t>(stream)));
}

const char *s2o_status_string(s2o_status s) {
    switch (s) {
        case S2O_OK: return "ok";
        case S2O_ERR_INVALID_ARG: return "invalid argument";
        case S2O_ERR_UNSUPPORTED: return "unsupported configuration";
        case S2O_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case S2O_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

}  // extern "C"
