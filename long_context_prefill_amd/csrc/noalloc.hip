// s2o_score for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// workspace s2o_score takes from its caller lives here in a static device
// array instead.  Contract in include/s2o.h.
#include <mutex>

#include "s2o.h"
#include "s2o_internal.h"

// Each GPU the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address: it is a host-side stand-in;
// scratch_address() looks up the device copy.
static __device__ __align__(256) unsigned char scratch[S2O_SCORE_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];  // per device: the address of its copy of `scratch`

// The current device's copy of `scratch`, looked up on the first call on that
// device (with the device current) and kept for later calls.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" s2o_status s2o_score_noalloc(const s2o_problem *p, const void *Q, const void *K, float *scores,
                                        void *stream) {
    const s2o_status st = s2o_check_problem(p);
    if (st != S2O_OK) return st;
    if (s2o_score_workspace_bytes(p) > S2O_SCORE_NOALLOC_MAX_WORKSPACE) return S2O_ERR_WORKSPACE;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return S2O_ERR_HIP;
    return s2o_score(p, Q, K, scores, ws, S2O_SCORE_NOALLOC_MAX_WORKSPACE, stream);
}
