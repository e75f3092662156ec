// Internal declarations shared by the host dispatch (abi.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s2o {

// Keys per key tile / list chunk; the only value the kernels are built for.
constexpr int kTileN = 64;

// Problem geometry after validation (all derived values precomputed).
struct Geometry {
    int32_t B, Hq, Hkv, G, N, d, S, BM, BN, T, P;  // P = S / BM tiles per segment
    int32_t causal;
    int32_t dtype;           // 0 fp32, 1 bf16
    int32_t per_seg;         // lists per segment (1) or per query tile (0)
    int32_t blocks;          // list entries are blocks of BN keys (1) or keys (0)
    int32_t qperm;           // query rows ordered within segments (Q_perm)
    int32_t share;           // one list per KV head, read by its G query heads
    int32_t nseg;            // segments, the last one possibly partial
    float inv_P, inv_P_last; // fl(1/tiles) of a full and of the last segment
    int64_t list_per_head;   // L: list entries of one (b, h), or of one (b, KV head) when shared
    int64_t list_entries;    // B * Hq * L (key lists), B * Hkv * L when shared
    int64_t query_entries;   // B * Hq * N with Q_perm (the query orders, after the key lists), else 0
    float scale;
};

// Offset of the list tile t of (b, h) uses:
//   per tile:    (b*Hq+h)*L + S*(P*s*(s-1)/2 + (t - s*P)*s), s = t / P
//   per segment: (b*Hq+h)*L + S*s*(s-1)/2
// with block entries every list is 1/BN as long (S is a multiple of BN), so the
// history term is divided by BN; shared lists put (b*Hkv + h/G) in place of
// (b*Hq + h).
__host__ __device__ inline int64_t list_offset(const Geometry &g, int b, int h, int t) {
    int64_t s = t / g.P;
    int64_t within = g.per_seg ? (int64_t)g.S * (s * (s - 1) / 2)
                               : (int64_t)g.S * (g.P * s * (s - 1) / 2 + (t - s * g.P) * s);
    if (g.blocks) within /= g.BN;
    const int64_t owner = g.share ? (int64_t)b * g.Hkv + h / g.G : (int64_t)b * g.Hq + h;
    return owner * g.list_per_head + within;
}

// Lists of one (b, h) and the tile owning list u (its first user).
__host__ __device__ inline int lists_per_head(const Geometry &g) { return g.per_seg ? g.nseg : g.T; }
__host__ __device__ inline int list_owner(const Geometry &g, int u) { return g.per_seg ? u * g.P : u; }

__host__ __device__ inline int64_t seg_start(const Geometry &g, int t) {
    return ((int64_t)t * g.BM / g.S) * g.S;
}

// Shared lists as a problem of their own: one query head per KV head (the
// group's mean representative), so scoring and sorting run unchanged.
inline Geometry group_geometry(const Geometry &g) {
    Geometry r = g;
    if (g.share) {
        r.Hq = g.Hkv;
        r.G = 1;
        r.share = 0;
    }
    return r;
}

// Block lists as a key problem of their own: each block becomes one "key" (its
// mean row, fp32), so N, S and BM shrink by BN and the lists keep their layout.
// Scoring and sorting run unchanged on this geometry.
inline Geometry block_geometry(const Geometry &g) {
    Geometry b = g;
    b.N = g.N / g.BN;
    b.S = g.S / g.BN;
    b.BM = g.BM / g.BN;
    b.BN = 1;
    b.blocks = 0;
    b.dtype = 0;
    return b;
}

// Kernel launchers (return hipSuccess or the launch error).
hipError_t launch_attention(const Geometry &g, const void *Q, const void *K, const void *V,
                            const int32_t *idx, const int32_t *qorder, float tau, void *O,
                            int32_t *exec_tiles, bool s2o, hipStream_t stream);

hipError_t launch_pool(const Geometry &g, const void *Q, const int32_t *qorder, float *qbar, float *qseg,
                       hipStream_t stream);
// shared lists: the group means of rows representatives [B, Hq, rows, d] -> [B, Hkv, rows, d]
hipError_t launch_group_mean(const Geometry &g, const float *rep, int rows, float *grp, hipStream_t stream);
// Q_perm: segment guides (mean keys), query scores, and the per-segment query order
hipError_t launch_query_scores(const Geometry &g, const void *Q, const void *K, float *guides, float *qscores,
                               hipStream_t stream);
hipError_t launch_query_sort(const Geometry &g, const float *qscores, int32_t *qorder, hipStream_t stream);
constexpr int kQuerySortCap = 8192;  // longest segment the query sort holds in LDS
hipError_t launch_pool_blocks(const Geometry &g, const void *K, float *kbar, hipStream_t stream);
hipError_t launch_score(const Geometry &g, const float *qrep, const void *K, float *scores,
                        hipStream_t stream);

size_t sort_workspace_bytes(const Geometry &g);
bool sort_supported(const Geometry &g);  // false: lists too long for blocks this small
hipError_t launch_sort(const Geometry &g, const float *scores, int32_t *idx, void *ws,
                       hipStream_t stream);

}  // namespace s2o
