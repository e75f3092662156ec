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
// segment) pair.  A pair's pooled query is the same for the whole wave, so it
// is read through the scalar cache and fed to the fmas as SGPR operands (no
// VGPRs, which keeps three waves per SIMD).  Two pairs are kept in flight for
// instruction-level parallelism; each chain is still evaluated in ascending k.
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

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ Q, float *__restrict__ qbar,
                                                   Geometry g, int64_t total) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int k = (int)(gid % g.d);
    const int64_t tile = gid / g.d;  // (b*Hq + h)*T + t
    const int t = (int)(tile % g.T);
    const int64_t bh = tile / g.T;
    const T *src = Q + (bh * g.N + (int64_t)t * g.BM) * g.d + k;
    float sum = 0.0f;
    for (int r = 0; r < g.BM; ++r) sum = sum + widen<T>(src[(int64_t)r * g.d]);
    qbar[gid] = sum * (1.0f / (float)g.BM);  // exact: BM is a power of two
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

constexpr int SCORE_KEYS = 256;   // keys per workgroup (one per thread)
constexpr int SCORE_ILP = 2;      // pairs evaluated together (independent fma chains)

template <typename T, int D>
__global__ __launch_bounds__(SCORE_KEYS, 2) void score_kernel(const float *__restrict__ qbar,
                                                              const T *__restrict__ K,
                                                              float *__restrict__ scores,
                                                              Geometry g, int nseg) {
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

    // pooled queries are wave-uniform: read them through the scalar cache so the
    // fma chains take them as SGPR operands
    for (int p0 = 0; p0 < npairs; p0 += SCORE_ILP) {
        const float *qp[SCORE_ILP];
#pragma unroll
        for (int i = 0; i < SCORE_ILP; ++i) {
            const int pp = min(p0 + i, npairs - 1);
            const int hq = pp / ntiles;
            const int t = t_first + pp - hq * ntiles;
            qp[i] = g.per_seg ? qbar + (((int64_t)b * g.Hq + kvh * g.G + hq) * g.nseg + s) * D
                              : qbar + (((int64_t)b * g.Hq + kvh * g.G + hq) * g.T + t) * D;
        }
        float acc[SCORE_ILP];
#pragma unroll
        for (int i = 0; i < SCORE_ILP; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) {
#pragma unroll
            for (int i = 0; i < SCORE_ILP; ++i) acc[i] = __builtin_fmaf(qp[i][k], kr[k], acc[i]);
        }
#pragma unroll
        for (int i = 0; i < SCORE_ILP; ++i) {
            const int pp = p0 + i;
            if (live && pp < npairs) {
                const int hq = pp / ntiles;
                const int t = t_first + pp - hq * ntiles;
                scores[list_offset(g, b, kvh * g.G + hq, t) + j] = acc[i];
            }
        }
    }
}

}  // namespace

hipError_t launch_pool(const Geometry &g, const void *Q, float *qbar, float *qseg, hipStream_t stream) {
    int64_t total = (int64_t)g.B * g.Hq * g.T * g.d;
    unsigned blocks = (unsigned)((total + 255) / 256);
    if (g.dtype == 1)
        hipLaunchKernelGGL(pool_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const __bf16 *>(Q), qbar, g, total);
    else
        hipLaunchKernelGGL(pool_kernel<float>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const float *>(Q), qbar, g, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !g.per_seg) return e;
    int64_t stotal = (int64_t)g.B * g.Hq * g.nseg * g.d;
    hipLaunchKernelGGL(segpool_kernel, dim3((unsigned)((stotal + 255) / 256)), dim3(256), 0, stream,
                       qbar, qseg, g, stotal);
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
