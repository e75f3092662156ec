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
    int64_t list_per_head;   // L: list entries of one (b, h)
    int64_t list_entries;    // B * Hq * L
    float scale;
};

// off(b,h,t) = (b*Hq+h)*L + S*(P*s*(s-1)/2 + (t - s*P)*s), s = t / P
__host__ __device__ inline int64_t list_offset(const Geometry &g, int b, int h, int t) {
    int64_t s = t / g.P;
    return ((int64_t)b * g.Hq + h) * g.list_per_head +
           (int64_t)g.S * (g.P * s * (s - 1) / 2 + (t - s * g.P) * s);
}

__host__ __device__ inline int64_t seg_start(const Geometry &g, int t) {
    return ((int64_t)t * g.BM / g.S) * g.S;
}

// Kernel launchers (return hipSuccess or the launch error).
hipError_t launch_attention(const Geometry &g, const void *Q, const void *K, const void *V,
                            const int32_t *idx, float tau, void *O, int32_t *exec_tiles,
                            bool s2o, hipStream_t stream);

hipError_t launch_pool(const Geometry &g, const void *Q, float *qbar, hipStream_t stream);
hipError_t launch_score(const Geometry &g, const float *qbar, const void *K, float *scores,
                        hipStream_t stream);

size_t sort_workspace_bytes(const Geometry &g);
hipError_t launch_sort(const Geometry &g, const float *scores, int32_t *idx, void *ws,
                       hipStream_t stream);

}  // namespace s2o
