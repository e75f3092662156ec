// Importance estimator for gfx950: mean-pooled query per tile, fp32 key scores.
//
// "S2O: Early Stopping for Sparse Attention via Online Permutation",
// gist.science technical summary, "Classement par Segment" (KV_perm): history
// keys are scored against a representative query; a causal mask keeps only
// prefix keys.  The representative is the mean of the tile's query rows.
//
// Scores are defined bit-exactly: qbar[k] = (fp32 sum of the BM rows in
// ascending order) * (1/BM) (per-segment lists: fp32 sum of the segment's tile
// means in ascending order times fl(1/tiles)), then s[j] = fma chain over
// k = 0..d-1 starting from 0 (2*d flops per (tile, key) pair).
//
// The chains run on the matrix cores: the fp32 MFMA with one product per
// output (32x32x1, two blocks) rounds once per step, exactly like fmaf, so
// issuing it for k = 0, 1, ..., d-1 gives every chain of the definition bit
// for bit.  One workgroup per (b, KV head, segment s >= 1, block of 256
// history keys); each lane keeps one key row in fp32 registers as its operand
// and the pooled queries (row-major [B, Hq, tiles, d]) are staged in LDS.
#include "s2o_internal.h"

namespace s2o {
namespace {

template <typename T>
__device__ inline float widen(T x);
template <>
__device__ inline float widen<float>(float x) { return x; }
template <>
__device__ inline float widen<__bf16>(__bf16 x) {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, x) << 16);
}

// qorder (Q_perm, else null): the rows of tile t are seg_start + qorder[bh*N +
// t*BM + r], r = 0..BM-1, summed in that order.
template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ Q, const int32_t *__restrict__ qorder,
                                                   float *__restrict__ qbar, Geometry g, int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int k = (int)(gid % g.d);
    const int64_t tile = gid / g.d;  // (b*Hq + h)*T + t
    const int t = (int)(tile % g.T);
    const int64_t bh = tile / g.T;
    const T *src = Q + bh * g.N * g.d + k;
    const int64_t row0 = (int64_t)t * g.BM, a = seg_start(g, t);
    // one sequential chain over the rows; the loads run POOL_BATCH rows ahead
    constexpr int POOL_BATCH = 32;
    float sum = 0.0f;
    const int32_t *ord = qorder ? qorder + bh * g.N + row0 : nullptr;
    auto row_of = [&](int r) -> int64_t { return ord ? a + ord[r] : row0 + r; };
    int r = 0;
    for (; r + POOL_BATCH <= g.BM; r += POOL_BATCH) {
        float v[POOL_BATCH];
#pragma unroll
        for (int u = 0; u < POOL_BATCH; ++u) v[u] = widen<T>(src[row_of(r + u) * g.d]);
#pragma unroll
        for (int u = 0; u < POOL_BATCH; ++u) sum = sum + v[u];
    }
    for (; r < g.BM; ++r) sum = sum + widen<T>(src[row_of(r) * g.d]);
    qbar[tile * g.d + k] = sum * (1.0f / (float)g.BM);  // exact: BM = 2^n
}

// Segment representatives (per-segment lists): mean of the segment's tile
// means, an fp32 sum over its tiles in ascending order times fl(1/tiles).
__global__ __launch_bounds__(256) void segpool_kernel(const float *__restrict__ qbar,
                                                      float *__restrict__ qseg, Geometry g,
                                                      int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int k = (int)(gid % g.d);
    const int64_t unit = gid / g.d;  // (b*Hq + h)*nseg + s
    const int s = (int)(unit % g.nseg);
    const int64_t bh = unit / g.nseg;
    const int first = s * g.P;
    const int last = min(g.T, first + g.P);
    float sum = 0.0f;
    for (int t = first; t < last; ++t) sum = sum + qbar[(bh * g.T + t) * g.d + k];
    qseg[gid] = sum * (s == g.nseg - 1 ? g.inv_P_last : g.inv_P);
}

// Shared lists: the mean of the G per-head representatives of a group, an
// fp32 sum over the heads in ascending order from 0 times fl(1/G).  One thread
// per (b, KV head, row, k); rep is [B, Hq, rows, d], grp is [B, Hkv, rows, d].
__global__ __launch_bounds__(256) void group_mean_kernel(const float *__restrict__ rep,
                                                         float *__restrict__ grp, Geometry g, int rows,
                                                         float inv_g, int64_t total) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int64_t per_head = (int64_t)rows * g.d;
    const int64_t bk = gid / per_head, in_head = gid % per_head;  // bk = b*Hkv + kvh
    const int64_t b = bk / g.Hkv, kvh = bk % g.Hkv;
    const float *src = rep + ((b * g.Hq + kvh * g.G) * per_head) + in_head;
    float sum = 0.0f;
    for (int j = 0; j < g.G; ++j) sum = sum + src[j * per_head];
    grp[gid] = sum * inv_g;
}

// Block lists: the mean key of every block of BN keys, fp32 sum of its rows in
// ascending order times 1/BN (exact: BN is a power of two), stored
// [B, Hkv, N/BN, d] in the natural layout so the score kernel reads it as keys.
template <typename T>
__global__ __launch_bounds__(256) void pool_blocks_kernel(const T *__restrict__ K, float *__restrict__ kbar,
                                                          Geometry g, int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int k = (int)(gid % g.d);
    const int64_t blk = gid / g.d;  // (b*Hkv + kvh)*(N/BN) + c
    const T *src = K + blk * g.BN * g.d + k;
    constexpr int BLK_BATCH = 32;  // one sequential chain; loads run a batch ahead
    float sum = 0.0f;
    int r = 0;
    for (; r + BLK_BATCH <= g.BN; r += BLK_BATCH) {
        float v[BLK_BATCH];
#pragma unroll
        for (int u = 0; u < BLK_BATCH; ++u) v[u] = widen<T>(src[(int64_t)(r + u) * g.d]);
#pragma unroll
        for (int u = 0; u < BLK_BATCH; ++u) sum = sum + v[u];
    }
    for (; r < g.BN; ++r) sum = sum + widen<T>(src[(int64_t)r * g.d]);
    kbar[gid] = sum * (1.0f / (float)g.BN);
}

// ---- Q_perm ----------------------------------------------------------------
// Guide of segment s for KV head kvh: the segment's mean key, fp32 sum of its
// rows in ascending order times fl(1/rows).  One thread per (b, kvh, s, k).
template <typename T>
__global__ __launch_bounds__(256) void guide_kernel(const T *__restrict__ K, float *__restrict__ guides,
                                                    Geometry g, int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int k = (int)(gid % g.d);
    const int64_t unit = gid / g.d;  // (b*Hkv + kvh)*nseg + s
    const int s = (int)(unit % g.nseg);
    const int64_t bg = unit / g.nseg;
    const int64_t a = (int64_t)s * g.S;
    const int64_t n = ((a + g.S) < g.N ? (a + g.S) : (int64_t)g.N) - a;
    const T *src = K + (bg * g.N + a) * g.d + k;
    // the sum stays one sequential chain over the rows; only the loads run
    // ahead, GUIDE_BATCH rows at a time (one thread per element leaves few
    // threads, so each must keep many loads in flight)
    constexpr int GUIDE_BATCH = 32;
    float sum = 0.0f;
    int64_t j = 0;
    for (; j + GUIDE_BATCH <= n; j += GUIDE_BATCH) {
        float v[GUIDE_BATCH];
#pragma unroll
        for (int u = 0; u < GUIDE_BATCH; ++u) v[u] = widen<T>(src[(j + u) * g.d]);
#pragma unroll
        for (int u = 0; u < GUIDE_BATCH; ++u) sum = sum + v[u];
    }
    for (; j < n; ++j) sum = sum + widen<T>(src[j * g.d]);
    guides[gid] = sum * (1.0f / (float)n);
}

// Importance score of every query row: fma chain over k of Q[row, k] times the
// guide of its segment, ascending k.  One thread per (b, h, row); written at
// the row's own position of the query-order region.
template <typename T>
__global__ __launch_bounds__(256) void query_score_kernel(const T *__restrict__ Q, const float *__restrict__ guides,
                                                          float *__restrict__ qscores, Geometry g, int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int64_t bh = gid / g.N;
    const int row = (int)(gid % g.N);
    const int b = (int)(bh / g.Hq), h = (int)(bh % g.Hq);
    const float *gd = guides + (((int64_t)b * g.Hkv + h / g.G) * g.nseg + row / g.S) * g.d;
    const T *q = Q + gid * g.d;
    // the row in 16-byte pieces; the fma chain is still ascending k
    constexpr int PER = 16 / (int)sizeof(T);
    float acc = 0.0f;
    for (int k0 = 0; k0 < g.d; k0 += PER) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(q + k0);
        const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
        for (int u = 0; u < PER; ++u) acc = __builtin_fmaf(widen<T>(e[u]), gd[k0 + u], acc);
    }
    qscores[gid] = acc;
}

// Query order of one segment of one (b, h): its rows sorted by score
// descending, ties to the lower row.  One workgroup sorts the segment in LDS
// with a bitonic network on (order-preserving key, row): the pair is unique, so
// the network's instability does not matter.  The segment is padded to a power
// of two with entries that sort after every real one.
constexpr int QSORT_THREADS = 1024;
__device__ inline uint32_t score_key(float f) {  // ascending key = descending score; -0 == +0
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}
__global__ __launch_bounds__(QSORT_THREADS) void query_sort_kernel(const float *__restrict__ qscores,
                                                                   int32_t *__restrict__ qorder, Geometry g) {
    __shared__ uint32_t key[kQuerySortCap];
    __shared__ int32_t row[kQuerySortCap];
    const int s = blockIdx.x % g.nseg;
    const int64_t bh = blockIdx.x / g.nseg;
    const int64_t a = (int64_t)s * g.S;
    const int n = (int)(((a + g.S) < g.N ? (a + g.S) : (int64_t)g.N) - a);
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    const float *src = qscores + bh * g.N + a;
    for (int i = threadIdx.x; i < n2; i += QSORT_THREADS) {
        key[i] = i < n ? score_key(src[i]) : 0xFFFFFFFFu;  // real keys stay below 0xFF800000
        row[i] = i;
    }
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n2; i += QSORT_THREADS) {
                const int l = i ^ j;
                if (l > i) {
                    const uint32_t ki = key[i], kl = key[l];
                    const int32_t ri = row[i], rl = row[l];
                    const bool gt = ki > kl || (ki == kl && ri > rl);
                    if (gt == ((i & k) == 0)) {  // ascending where bit k of i is clear
                        key[i] = kl;
                        key[l] = ki;
                        row[i] = rl;
                        row[l] = ri;
                    }
                }
            }
            __syncthreads();
        }
    }
    int32_t *dst = qorder + bh * g.N + a;
    for (int i = threadIdx.x; i < n; i += QSORT_THREADS) dst[i] = row[i];
}

// Scores on the matrix cores.  v_mfma_f32_32x32x1_2b_f32 adds one product per
// output per instruction with a single rounding, i.e. it is fmaf elementwise, so
// a chain of them over k = 0..d-1 reproduces the fma chain of the definition
// bit for bit while doing two 32x32 outer products per instruction: block b
// takes its 32 rows from A lanes [32b, 32b+32) and its 32 columns from B lanes
// [32b, 32b+32).  Here the rows are 32 (query head, tile) pairs (the same pairs
// in both blocks) and the columns are keys: every lane holds its own key row
// in fp32 registers as its B operand, so a wave scores 64 keys against NG
// groups of 32 pairs per pass.  The pooled queries of a pass are staged in LDS
// (row-major, padded by 4 floats against bank conflicts).
// Segments with few pairs (per-segment lists have one pair per query head)
// use v_mfma_f32_4x4x1_16b_f32 instead (SHAPE 4), which rounds the same way:
// its 16 blocks take their 4 rows from A lanes 4b..4b+3 and column j from B
// lane j, so with lane l holding the pooled query of pair l%4 as A one
// instruction scores 4 pairs against the wave's 64 keys, and output register r
// of lane l is pair r against the lane's own key.
constexpr int MS_KEYS = 256;  // keys per workgroup: 4 waves x 64

template <typename T, int D, int SHAPE, int NG>
__global__ __launch_bounds__(MS_KEYS, 2) void score_mfma_kernel(const float *__restrict__ qbar,
                                                               const T *__restrict__ K,
                                                               float *__restrict__ scores, Geometry g,
                                                               int nseg) {
    static_assert(SHAPE == 32 || SHAPE == 4, "32x32x1 or 4x4x1 blocks");
    typedef float f32x32 __attribute__((ext_vector_type(32)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int ROWS = SHAPE * NG, PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[ROWS * PITCH];
    __shared__ __attribute__((aligned(16))) int64_t srow[ROWS];  // list start of each staged pair, or -1
    const int s = blockIdx.y % nseg;
    const int bg = blockIdx.y / nseg;
    const int hist = s * g.S;
    if (s == 0 || (int)blockIdx.x * MS_KEYS >= hist) return;  // uniform
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = bg / g.Hkv, kvh = bg % g.Hkv;
    const int t_first = s * g.P;
    const int ntiles = g.per_seg ? 1 : min(g.T, (s + 1) * g.P) - t_first;
    const int npairs = ntiles * g.G;
    const int j0 = blockIdx.x * MS_KEYS + wave * 64;  // this wave's keys
    const bool wave_live = j0 < hist;                 // uniform per wave
    const int j = j0 + lane;

    float kr[D];
    {
        const T *row = K + ((int64_t)bg * g.N + (j < hist ? j : 0)) * D;
#pragma unroll
        for (int k = 0; k < D; k += 8) {
            uint4 raw = *reinterpret_cast<const uint4 *>(row + k);  // 8 bf16 or 4 fp32
            if constexpr (sizeof(T) == 2) {
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kr[k + 2 * e] = __uint_as_float(w[e] << 16);
                    kr[k + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            } else {
                uint4 raw2 = *reinterpret_cast<const uint4 *>(row + k + 4);
                kr[k] = __uint_as_float(raw.x);
                kr[k + 1] = __uint_as_float(raw.y);
                kr[k + 2] = __uint_as_float(raw.z);
                kr[k + 3] = __uint_as_float(raw.w);
                kr[k + 4] = __uint_as_float(raw2.x);
                kr[k + 5] = __uint_as_float(raw2.y);
                kr[k + 6] = __uint_as_float(raw2.z);
                kr[k + 7] = __uint_as_float(raw2.w);
            }
        }
    }

    // Pair pp -> (query head kvh*G + hq, tile t_first + ti), hq = pp / ntiles by a
    // multiply-high with ceil(2^32 / ntiles) (exact while pp * ntiles < 2^32,
    // else a plain division), and the pair's pooled query and list position in
    // closed form (the tiles of one head are consecutive in both layouts; the
    // list of tile t_first + ti starts ti * S * s after the segment's first list).
    const uint32_t magic = ntiles > 1 ? (uint32_t)((0x100000000ull + ntiles - 1) / (uint64_t)ntiles) : 0u;
    const bool by_magic = (int64_t)npairs * ntiles < 0x100000000ll;
    auto split = [&](int pp, int &hq, int &ti) {
        hq = ntiles == 1 ? pp : by_magic ? (int)__umulhi((uint32_t)pp, magic) : pp / ntiles;
        ti = pp - hq * ntiles;
    };
    const int qrows = g.per_seg ? g.nseg : g.T;  // pooled queries per head
    const float *qhead0 = qbar + (((int64_t)b * g.Hq + kvh * g.G) * qrows + (g.per_seg ? s : t_first)) * D;
    const int64_t L = g.list_per_head;
    const int64_t seg_first = g.per_seg ? (int64_t)g.S * (s * (s - 1) / 2)
                                        : (int64_t)g.S * ((int64_t)g.P * s * (s - 1) / 2);
    float *shead0 = scores + ((int64_t)b * g.Hq + kvh * g.G) * L + seg_first;
    const int64_t tile_step = g.per_seg ? 0 : (int64_t)g.S * s;

    for (int p0 = 0; p0 < npairs; p0 += ROWS) {
        // stage the pooled queries of pairs p0 .. p0+ROWS-1 (zeros past the last)
        constexpr int C4 = D / 4;
        for (int i = tid; i < ROWS * C4; i += MS_KEYS) {
            const int r = i / C4, c4 = i % C4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p0 + r < npairs) {
                int hq, ti;
                split(p0 + r, hq, ti);
                v = *reinterpret_cast<const float4 *>(qhead0 + ((int64_t)hq * qrows + ti) * D + 4 * c4);
            }
            *reinterpret_cast<float4 *>(&qs[r * PITCH + 4 * c4]) = v;
        }
        for (int r = tid; r < ROWS; r += MS_KEYS) {
            int64_t o = -1;
            if (p0 + r < npairs) {
                int hq, ti;
                split(p0 + r, hq, ti);
                o = hq * L + ti * tile_step;
            }
            srow[r] = o;
        }
        __syncthreads();
        if (SHAPE == 4 && wave_live) {
            f32x4 acc[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D; kk += 4) {
                float4 a[NG];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi)
                    a[gi] = *reinterpret_cast<const float4 *>(&qs[(4 * gi + (lane & 3)) * PITCH + kk]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
                        acc[gi] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[gi][u], kr[kk + u], acc[gi], 0, 0, 0);
            }
            // acc[gi][r] = score of staged pair 4 gi + r against key j0 + lane
            const int key = j0 + lane;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t o = srow[4 * gi + r];
                    if (o >= 0 && key < hist) shead0[o + key] = acc[gi][r];
                }
        }
        if (SHAPE == 32 && wave_live) {
            f32x32 acc[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int r = 0; r < 32; ++r) acc[gi][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D; kk += 4) {
                float4 a[NG];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi)
                    a[gi] = *reinterpret_cast<const float4 *>(&qs[(32 * gi + (lane & 31)) * PITCH + kk]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
                        acc[gi] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[gi][u], kr[kk + u], acc[gi], 0, 0, 0);
            }
            // acc[gi][16*blk + 4*q + e] = score of staged pair 32 gi + 8 q + 4 (lane/32) + e
            // against key j0 + 32 blk + lane%32; a pair's list start comes from srow
            const bool full = p0 + ROWS <= npairs && j0 + 64 <= hist;  // uniform per wave
            const int kl = j0 + (lane & 31);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int64_t ro[4];
                    const int rb = 32 * gi + 8 * q + 4 * (lane >> 5);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ro[e] = srow[rb + e];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int blk = 0; blk < 2; ++blk) {
                            const int key = kl + 32 * blk;
                            if (full || (ro[e] >= 0 && key < hist)) shead0[ro[e] + key] = acc[gi][16 * blk + 4 * q + e];
                        }
                }
            }
        }
        __syncthreads();  // the next pass restages qs
    }
}

// pairs: (query head, tile) pairs of a segment
template <typename T, int D>
void launch_score_mfma(int pairs, dim3 grid, const float *qbar, const void *K, float *scores,
                       const Geometry &g, int nseg, hipStream_t stream) {
    const T *k = reinterpret_cast<const T *>(K);
    if (pairs <= 4)
        hipLaunchKernelGGL((score_mfma_kernel<T, D, 4, 1>), grid, dim3(MS_KEYS), 0, stream, qbar, k, scores, g, nseg);
    else if (pairs <= 16)
        hipLaunchKernelGGL((score_mfma_kernel<T, D, 4, 4>), grid, dim3(MS_KEYS), 0, stream, qbar, k, scores, g, nseg);
    else if (pairs <= 32)
        hipLaunchKernelGGL((score_mfma_kernel<T, D, 32, 1>), grid, dim3(MS_KEYS), 0, stream, qbar, k, scores, g, nseg);
    else
        hipLaunchKernelGGL((score_mfma_kernel<T, D, 32, 2>), grid, dim3(MS_KEYS), 0, stream, qbar, k, scores, g, nseg);
}

}  // namespace

hipError_t launch_pool(const Geometry &g, const void *Q, const int32_t *qorder, float *qbar, float *qseg,
                       hipStream_t stream) {
    int64_t total = (int64_t)g.B * g.Hq * g.T * g.d;
    unsigned blocks = (unsigned)((total + 255) / 256);
    if (g.dtype == 1)
        hipLaunchKernelGGL(pool_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const __bf16 *>(Q), qorder, qbar, g, total);
    else
        hipLaunchKernelGGL(pool_kernel<float>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const float *>(Q), qorder, qbar, g, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !g.per_seg) return e;
    int64_t stotal = (int64_t)g.B * g.Hq * g.nseg * g.d;
    hipLaunchKernelGGL(segpool_kernel, dim3((unsigned)((stotal + 255) / 256)), dim3(256), 0, stream,
                       qbar, qseg, g, stotal);
    return hipGetLastError();
}

hipError_t launch_query_scores(const Geometry &g, const void *Q, const void *K, float *guides, float *qscores,
                               hipStream_t stream) {
    const int64_t gtotal = (int64_t)g.B * g.Hkv * g.nseg * g.d;
    const int64_t qtotal = (int64_t)g.B * g.Hq * g.N;
    if (g.dtype == 1) {
        hipLaunchKernelGGL(guide_kernel<__bf16>, dim3((unsigned)((gtotal + 255) / 256)), dim3(256), 0, stream,
                           reinterpret_cast<const __bf16 *>(K), guides, g, gtotal);
        hipLaunchKernelGGL(query_score_kernel<__bf16>, dim3((unsigned)((qtotal + 255) / 256)), dim3(256), 0,
                           stream, reinterpret_cast<const __bf16 *>(Q), guides, qscores, g, qtotal);
    } else {
        hipLaunchKernelGGL(guide_kernel<float>, dim3((unsigned)((gtotal + 255) / 256)), dim3(256), 0, stream,
                           reinterpret_cast<const float *>(K), guides, g, gtotal);
        hipLaunchKernelGGL(query_score_kernel<float>, dim3((unsigned)((qtotal + 255) / 256)), dim3(256), 0,
                           stream, reinterpret_cast<const float *>(Q), guides, qscores, g, qtotal);
    }
    return hipGetLastError();
}

hipError_t launch_query_sort(const Geometry &g, const float *qscores, int32_t *qorder, hipStream_t stream) {
    hipLaunchKernelGGL(query_sort_kernel, dim3((unsigned)((int64_t)g.B * g.Hq * g.nseg)), dim3(QSORT_THREADS), 0,
                       stream, qscores, qorder, g);
    return hipGetLastError();
}

hipError_t launch_group_mean(const Geometry &g, const float *rep, int rows, float *grp, hipStream_t stream) {
    const int64_t total = (int64_t)g.B * g.Hkv * rows * g.d;
    const float inv_g = 1.0f / (float)g.G;  // fl(1/G), rounded on the host
    hipLaunchKernelGGL(group_mean_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, rep, grp,
                       g, rows, inv_g, total);
    return hipGetLastError();
}

hipError_t launch_pool_blocks(const Geometry &g, const void *K, float *kbar, hipStream_t stream) {
    const int64_t total = (int64_t)g.B * g.Hkv * (g.N / g.BN) * g.d;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (g.dtype == 1)
        hipLaunchKernelGGL(pool_blocks_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const __bf16 *>(K), kbar, g, total);
    else
        hipLaunchKernelGGL(pool_blocks_kernel<float>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const float *>(K), kbar, g, total);
    return hipGetLastError();
}

hipError_t launch_score(const Geometry &g, const float *qbar, const void *K, float *scores,
                        hipStream_t stream) {
    const int nseg = (g.N + g.S - 1) / g.S;
    if (nseg < 2) return hipSuccess;  // no tile has history
    const int64_t max_hist = (int64_t)(nseg - 1) * g.S;
    dim3 grid((unsigned)((max_hist + MS_KEYS - 1) / MS_KEYS), (unsigned)(g.B * g.Hkv * nseg));
    const int pairs = (g.per_seg ? 1 : g.P) * g.G;  // most pairs of a segment
    if (g.dtype == 1) {
        if (g.d == 128) launch_score_mfma<__bf16, 128>(pairs, grid, qbar, K, scores, g, nseg, stream);
        else launch_score_mfma<__bf16, 64>(pairs, grid, qbar, K, scores, g, nseg, stream);
    } else {
        if (g.d == 128) launch_score_mfma<float, 128>(pairs, grid, qbar, K, scores, g, nseg, stream);
        else launch_score_mfma<float, 64>(pairs, grid, qbar, K, scores, g, nseg, stream);
    }
    return hipGetLastError();
}

}  // namespace s2o
