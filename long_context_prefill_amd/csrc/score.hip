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
// k = 0..d-1 starting from 0.  The work is plain fp32 ALU (2*d flops per (tile, key) pair); the
// fixed accumulation order rules out matrix cores.
//
// Layout of the score kernel: one workgroup per (b, KV head, segment s >= 1,
// block of 256 history keys).  Each thread holds one key row in fp32
// registers and runs it against every (query head of the group, tile of the
// segment) pair, four pairs at a time.  A pair's pooled query is spread over
// the 16 lanes of each row (D/16 registers per lane) and broadcast element by
// element with DPP row_newbcast as the fma's first operand; the next four
// pairs load while the current four compute.  Each chain is still evaluated in
// ascending k.
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
    // stored lane-major: element k of a pooled query at (k % 16) * (d / 16) + k / 16,
    // so a lane reads its d/16 elements (16c + lane, c = 0..) as one contiguous run
    qbar[tile * g.d + (k & 15) * (g.d >> 4) + (k >> 4)] = sum * (1.0f / (float)g.BM);  // exact: BM = 2^n
}

// Segment representatives (per-segment lists): mean of the segment's tile
// means, an fp32 sum over its tiles in ascending order times fl(1/tiles).
// Elementwise, so it works in the lane-major layout unchanged.
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

constexpr int SCORE_KEYS = 256;   // keys per workgroup (one per thread)
constexpr int SCORE_ILP = 4;      // pairs evaluated together (independent fma chains)

// acc[p] = fma(qbar_p[16c + n], kr[16c + n], acc[p]) for n = 0..15 in ascending
// order, for the four pairs p.  Lane i of every 16-lane row holds
// qbar_p[16c + i] in q_p; DPP row_newbcast:n hands lane n's value to its whole
// row, so every fma takes its pooled-query element straight from another
// lane's register at full rate.  The four chains are interleaved, which keeps
// three instructions between dependent ones (DPP needs two wait states after a
// VALU write of an operand); the leading s_nop covers writes made just before.
#define S2O_DPP_FMA(n, K)                                                                    \
    "v_fmac_f32_dpp %0, %4, " K " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n\t"        \
    "v_fmac_f32_dpp %1, %5, " K " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n\t"        \
    "v_fmac_f32_dpp %2, %6, " K " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n\t"        \
    "v_fmac_f32_dpp %3, %7, " K " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n\t"

__device__ __forceinline__ void fma16x4(float &a0, float &a1, float &a2, float &a3, float q0, float q1,
                                        float q2, float q3, const float *k) {
    asm volatile("s_nop 1\n\t"
                 S2O_DPP_FMA(0, "%8") S2O_DPP_FMA(1, "%9") S2O_DPP_FMA(2, "%10") S2O_DPP_FMA(3, "%11")
                 S2O_DPP_FMA(4, "%12") S2O_DPP_FMA(5, "%13") S2O_DPP_FMA(6, "%14") S2O_DPP_FMA(7, "%15")
                 S2O_DPP_FMA(8, "%16") S2O_DPP_FMA(9, "%17") S2O_DPP_FMA(10, "%18") S2O_DPP_FMA(11, "%19")
                 S2O_DPP_FMA(12, "%20") S2O_DPP_FMA(13, "%21") S2O_DPP_FMA(14, "%22") S2O_DPP_FMA(15, "%23")
                 : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)
                 : "v"(q0), "v"(q1), "v"(q2), "v"(q3), "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]),
                   "v"(k[5]), "v"(k[6]), "v"(k[7]), "v"(k[8]), "v"(k[9]), "v"(k[10]), "v"(k[11]), "v"(k[12]),
                   "v"(k[13]), "v"(k[14]), "v"(k[15])
                 : "memory");  // keeps the next group's loads issued ahead of the block
}
#undef S2O_DPP_FMA

template <typename T, int D>
__global__ __launch_bounds__(SCORE_KEYS, 2) void score_kernel(const float *__restrict__ qbar,
                                                              const T *__restrict__ K,
                                                              float *__restrict__ scores,
                                                              Geometry g, int nseg) {
    constexpr int NQ = D / 16;                   // 16-element chunks of a pooled query
    const int s = blockIdx.y % nseg;             // segment of the query tiles
    const int bg = blockIdx.y / nseg;            // b * Hkv + kv head
    const int hist = s * g.S;                    // history length of the segment's tiles
    const int j0 = blockIdx.x * SCORE_KEYS;
    if (s == 0 || j0 >= hist) return;
    const int b = bg / g.Hkv, kvh = bg % g.Hkv;
    const int t_first = s * g.P;
    // per-tile lists: one pair per (query head, tile of the segment); per-segment
    // lists: one pair per query head, ranked against the segment representative
    const int ntiles = g.per_seg ? 1 : min(g.T, (s + 1) * g.P) - t_first;
    const int npairs = ntiles * g.G;             // pair p -> (query head kvh*G + p / ntiles, tile)
    const int j = j0 + (int)threadIdx.x;
    const bool live = j < hist;
    const int col = threadIdx.x & 15;            // this lane's element of each 16-chunk

    float kr[D];
    {
        const T *row = K + ((int64_t)bg * g.N + (live ? j : 0)) * D;
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
    // else a plain division), and
    // the pair's pooled query and list position in closed form (the tiles of
    // one head are consecutive in both layouts; the list of tile t_first + ti
    // starts ti * S * s after the segment's first list).
    const uint32_t magic = ntiles > 1 ? (uint32_t)((0x100000000ull + ntiles - 1) / (uint64_t)ntiles) : 0u;
    const bool by_magic = (int64_t)npairs * ntiles < 0x100000000ll;
    const int qrows = g.per_seg ? g.nseg : g.T;  // pooled queries per head
    const float *qhead0 = qbar + (((int64_t)b * g.Hq + kvh * g.G) * qrows + (g.per_seg ? s : t_first)) * D;
    const int64_t L = g.list_per_head;
    const int64_t seg_first = g.per_seg ? (int64_t)g.S * (s * (s - 1) / 2)
                                        : (int64_t)g.S * ((int64_t)g.P * s * (s - 1) / 2);
    float *shead0 = scores + ((int64_t)b * g.Hq + kvh * g.G) * L + seg_first + j;
    const int64_t tile_step = g.per_seg ? 0 : (int64_t)g.S * s;
    auto split = [&](int pp, int &hq, int &ti) {
        hq = ntiles == 1 ? pp : by_magic ? (int)__umulhi((uint32_t)pp, magic) : pp / ntiles;
        ti = pp - hq * ntiles;
    };
    // q[i][c] = pooled query of pair p0 + i, element 16c + col (every row alike),
    // read as NQ contiguous floats of the lane-major layout
    auto load_group = [&](float (&q)[SCORE_ILP][NQ], int p0) {
#pragma unroll
        for (int i = 0; i < SCORE_ILP; ++i) {
            int hq, ti;
            split(min(p0 + i, npairs - 1), hq, ti);
            const float *src = qhead0 + ((int64_t)hq * qrows + ti) * D + col * NQ;
#pragma unroll
            for (int c = 0; c < NQ; c += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(src + c);
                q[i][c] = v.x;
                q[i][c + 1] = v.y;
                q[i][c + 2] = v.z;
                q[i][c + 3] = v.w;
            }
        }
    };
    auto store_group = [&](const float (&acc)[SCORE_ILP], int p0) {
#pragma unroll
        for (int i = 0; i < SCORE_ILP; ++i) {
            if (live && p0 + i < npairs) {
                int hq, ti;
                split(p0 + i, hq, ti);
                shead0[hq * L + ti * tile_step] = acc[i];
            }
        }
    };
    // Runs the four chains of pairs p0..p0+3 on q.  The previous group's scores
    // and the next group's loads go out after the first 16 steps, so that when
    // the next group starts, every memory operation it waits for (loads and
    // stores share one counter) was issued a whole group earlier.
    auto run_group = [&](const float (&q)[SCORE_ILP][NQ], int p0, float (&qnext)[SCORE_ILP][NQ],
                         float (&acc)[SCORE_ILP]) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        fma16x4(a0, a1, a2, a3, q[0][0], q[1][0], q[2][0], q[3][0], kr);
        if (p0 > 0) store_group(acc, p0 - SCORE_ILP);
        if (p0 + SCORE_ILP < npairs) load_group(qnext, p0 + SCORE_ILP);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 1; c < NQ; ++c)
            fma16x4(a0, a1, a2, a3, q[0][c], q[1][c], q[2][c], q[3][c], kr + 16 * c);
        acc[0] = a0;
        acc[1] = a1;
        acc[2] = a2;
        acc[3] = a3;
    };

    float qa[SCORE_ILP][NQ], qb[SCORE_ILP][NQ], acc[SCORE_ILP];
    load_group(qa, 0);
    int p0 = 0;
    for (;;) {
        run_group(qa, p0, qb, acc);
        if (p0 + SCORE_ILP >= npairs) break;
        p0 += SCORE_ILP;
        run_group(qb, p0, qa, acc);
        if (p0 + SCORE_ILP >= npairs) break;
        p0 += SCORE_ILP;
    }
    store_group(acc, p0);
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
    dim3 grid((unsigned)((max_hist + SCORE_KEYS - 1) / SCORE_KEYS), (unsigned)(g.B * g.Hkv * nseg));
    if (g.dtype == 1) {
        if (g.d == 128)
            hipLaunchKernelGGL((score_kernel<__bf16, 128>), grid, dim3(SCORE_KEYS), 0, stream, qbar,
                               reinterpret_cast<const __bf16 *>(K), scores, g, nseg);
        else
            hipLaunchKernelGGL((score_kernel<__bf16, 64>), grid, dim3(SCORE_KEYS), 0, stream, qbar,
                               reinterpret_cast<const __bf16 *>(K), scores, g, nseg);
    } else {
        if (g.d == 128)
            hipLaunchKernelGGL((score_kernel<float, 128>), grid, dim3(SCORE_KEYS), 0, stream, qbar,
                               reinterpret_cast<const float *>(K), scores, g, nseg);
        else
            hipLaunchKernelGGL((score_kernel<float, 64>), grid, dim3(SCORE_KEYS), 0, stream, qbar,
                               reinterpret_cast<const float *>(K), scores, g, nseg);
    }
    return hipGetLastError();
}

}  // namespace s2o
