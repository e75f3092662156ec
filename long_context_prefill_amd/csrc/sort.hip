// Segmented stable LSD radix sort for the per-tile index lists, gfx950.
//
// "S2O: Early Stopping for Sparse Attention via Online Permutation",
// gist.science technical summary, "Classement par Segment" (KV_perm): the
// history keys of each tile are ordered by their score; the indices form the
// logical map the attention kernel follows.  Order: score descending, ties to
// the lower position (LSD radix passes are stable and start from ascending
// positions).  -0.0 is folded onto +0.0 so the two tie.
//
// Every list is a multiple of the segment length S long and starts at a
// multiple of S, so the concatenated lists split into equal blocks of E
// elements (E = largest power of two dividing S, at most 4096) that never
// straddle two lists.  Four 8-bit passes, each:
//   hist    per block: digit histogram (wave-level multisplit, LDS counters)
//   scan    per list: for every digit, where each block's run starts
//   scatter per block: stable rank of every element within its digit, staged
//           sorted in LDS, then written out in order (runs are contiguous)
// Pass 0 reads the scores directly (key transform on the fly, positions
// implicit); pass 3 writes only the positions, into idx.
#include "s2o_internal.h"

namespace s2o {
namespace {

constexpr int RADIX = 256;
constexpr int SORT_THREADS = 256;
constexpr int MAX_BLOCK = 4096;

// fp32 -> uint32 whose ascending order is descending score order
__device__ inline uint32_t desc_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;  // -0.0 ties with +0.0
    uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}

__device__ inline uint64_t lanemask_lt() {
    return (1ull << (threadIdx.x & 63)) - 1ull;
}

// Lanes of the wave holding the same 8-bit digit as this lane.
__device__ inline uint64_t match_digit(uint32_t digit) {
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        uint64_t bal = __ballot((digit >> bit) & 1u);
        peers &= ((digit >> bit) & 1u) ? bal : ~bal;
    }
    return peers;
}

// Block geometry: E elements, NWV waves, ROUNDS rounds of 64 per wave.  Wave
// w owns elements [w*E/NWV, (w+1)*E/NWV); round r, lane l holds element
// w*E/NWV + 64*r + l, so block order == (wave, round, lane) order.
template <int E>
struct BlockCfg {
    static constexpr int NWV = E >= 256 ? 4 : E / 64;
    static constexpr int ROUNDS = E / (64 * NWV);
    static_assert(E % 64 == 0 && ROUNDS >= 1, "block size");
};

template <int E, bool FIRST>
__global__ __launch_bounds__(SORT_THREADS) void hist_kernel(const void *__restrict__ keys_in,
                                                            int32_t *__restrict__ hist, int shift) {
    using BC = BlockCfg<E>;
    __shared__ int cnt[4][RADIX];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 4 * RADIX; i += SORT_THREADS) (&cnt[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * E;
    if (wave < BC::NWV) {
        for (int r = 0; r < BC::ROUNDS; ++r) {
            int64_t e = base + (int64_t)wave * (E / BC::NWV) + 64 * r + lane;
            uint32_t key = FIRST ? desc_key(reinterpret_cast<const float *>(keys_in)[e])
                                 : reinterpret_cast<const uint32_t *>(keys_in)[e];
            uint32_t digit = (key >> shift) & 0xFFu;
            uint64_t peers = match_digit(digit);
            if ((peers & lanemask_lt()) == 0) cnt[wave][digit] += __popcll(peers);
        }
    }
    __syncthreads();
    for (int v = tid; v < RADIX; v += SORT_THREADS)
        hist[(int64_t)blockIdx.x * RADIX + v] = cnt[0][v] + cnt[1][v] + cnt[2][v] + cnt[3][v];
}

// One workgroup per list.  Turns the block histograms of the list
// into the start of each block's digit run, relative to the block's first
// element: hist[bb][v] = (list_off + sum_{v'<v} total[v'] + sum_{bb'<bb} hist[bb'][v]) - bb*E.
// The first pass also records each block's offset inside its list.
__global__ __launch_bounds__(RADIX) void scan_kernel(int32_t *__restrict__ hist,
                                                     int32_t *__restrict__ blk_pos, Geometry g,
                                                     int E, int first) {
    __shared__ int tot[RADIX];
    const int U = lists_per_head(g);
    const int t = list_owner(g, blockIdx.x % U);
    const int64_t bh = blockIdx.x / U;
    const int64_t len = seg_start(g, t);
    if (len == 0) return;
    const int b = (int)(bh / g.Hq), h = (int)(bh % g.Hq);
    const int64_t off = list_offset(g, b, h, t);
    const int64_t b0 = off / E, nb = len / E;
    const int v = threadIdx.x;
    int run = 0;
    for (int64_t bb = b0; bb < b0 + nb; ++bb) {
        int c = hist[bb * RADIX + v];
        hist[bb * RADIX + v] = run;
        run += c;
    }
    tot[v] = run;
    __syncthreads();
    // exclusive scan over digits (Hillis-Steele on 256 entries)
    for (int d = 1; d < RADIX; d <<= 1) {
        int x = v >= d ? tot[v - d] : 0;
        __syncthreads();
        tot[v] += x;
        __syncthreads();
    }
    const int digit_base = tot[v] - run;  // exclusive
    for (int64_t bb = b0; bb < b0 + nb; ++bb)
        hist[bb * RADIX + v] += (int)(digit_base + off - bb * E);
    if (first && v == 0)
        for (int64_t bb = b0; bb < b0 + nb; ++bb) blk_pos[bb] = (int32_t)(bb * E - off);
}

template <int E, bool FIRST, bool LAST>
__global__ __launch_bounds__(SORT_THREADS) void scatter_kernel(
    const void *__restrict__ keys_in, const int32_t *__restrict__ vals_in,
    uint32_t *__restrict__ keys_out, int32_t *__restrict__ vals_out,
    const int32_t *__restrict__ hist, const int32_t *__restrict__ blk_pos, int shift) {
    using BC = BlockCfg<E>;
    __shared__ int cnt[4][RADIX];       // per-wave digit counters, then wave offsets
    __shared__ int dstart[RADIX];       // first sorted position of each digit in the block
    __shared__ int dglob[RADIX];        // global run start of each digit (relative)
    __shared__ uint32_t skey[E];
    __shared__ int32_t sval[E];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 4 * RADIX; i += SORT_THREADS) (&cnt[0][0])[i] = 0;
    const int64_t base = (int64_t)blockIdx.x * E;
    for (int v = tid; v < RADIX; v += SORT_THREADS) dglob[v] = hist[(int64_t)blockIdx.x * RADIX + v];
    __syncthreads();

    uint32_t key[BC::ROUNDS];
    int32_t val[BC::ROUNDS];
    int rank[BC::ROUNDS];
    if (wave < BC::NWV) {
        const int32_t pos0 = FIRST ? blk_pos[blockIdx.x] : 0;
#pragma unroll
        for (int r = 0; r < BC::ROUNDS; ++r) {
            const int local = wave * (E / BC::NWV) + 64 * r + lane;
            const int64_t e = base + local;
            if (FIRST) {
                key[r] = desc_key(reinterpret_cast<const float *>(keys_in)[e]);
                val[r] = pos0 + local;
            } else {
                key[r] = reinterpret_cast<const uint32_t *>(keys_in)[e];
                val[r] = vals_in[e];
            }
            const uint32_t digit = (key[r] >> shift) & 0xFFu;
            const uint64_t peers = match_digit(digit);
            const int before = cnt[wave][digit];  // read by all peers before the leader updates
            rank[r] = before + __popcll(peers & lanemask_lt());
            if ((peers & lanemask_lt()) == 0) cnt[wave][digit] = before + __popcll(peers);
        }
    }
    __syncthreads();
    // per digit: exclusive offsets of the waves, and the digit's start in the block
    for (int v = tid; v < RADIX; v += SORT_THREADS) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            int c = cnt[w][v];
            cnt[w][v] = s;
            s += c;
        }
        dstart[v] = s;  // total for now
    }
    __syncthreads();
    if (tid < 64) {  // exclusive scan of the 256 digit totals by one wave
        int a0 = dstart[4 * tid], a1 = dstart[4 * tid + 1], a2 = dstart[4 * tid + 2], a3 = dstart[4 * tid + 3];
        int sum = a0 + a1 + a2 + a3, incl = sum;
        for (int d = 1; d < 64; d <<= 1) {
            int x = __shfl_up(incl, d);
            if (lane >= d) incl += x;
        }
        int ex = incl - sum;
        dstart[4 * tid] = ex;
        dstart[4 * tid + 1] = ex + a0;
        dstart[4 * tid + 2] = ex + a0 + a1;
        dstart[4 * tid + 3] = ex + a0 + a1 + a2;
    }
    __syncthreads();
    if (wave < BC::NWV) {
#pragma unroll
        for (int r = 0; r < BC::ROUNDS; ++r) {
            const uint32_t digit = (key[r] >> shift) & 0xFFu;
            const int p = dstart[digit] + cnt[wave][digit] + rank[r];
            skey[p] = key[r];
            sval[p] = val[r];
        }
    }
    __syncthreads();
    for (int i = tid; i < E; i += SORT_THREADS) {
        const uint32_t k = skey[i];
        const uint32_t digit = (k >> shift) & 0xFFu;
        const int64_t dst = base + dglob[digit] + (i - dstart[digit]);
        if (!LAST) keys_out[dst] = k;
        vals_out[dst] = sval[i];
    }
}

int block_elems(const Geometry &g) {
    int e = g.S & (-g.S);  // largest power of two dividing S
    return e > MAX_BLOCK ? MAX_BLOCK : e;
}

struct SortWs {
    uint32_t *keys_a, *keys_b;
    int32_t *vals_a;
    int32_t *hist, *blk_pos;
    size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SortWs carve(const Geometry &g, void *base) {
    const int64_t n = g.list_entries;
    const int64_t nblocks = n / block_elems(g);
    SortWs w;
    size_t off = 0;
    char *p = reinterpret_cast<char *>(base);
    w.keys_a = reinterpret_cast<uint32_t *>(p + off);
    off += align256(n * 4);
    w.keys_b = reinterpret_cast<uint32_t *>(p + off);
    off += align256(n * 4);
    w.vals_a = reinterpret_cast<int32_t *>(p + off);
    off += align256(n * 4);
    w.hist = reinterpret_cast<int32_t *>(p + off);
    off += align256((size_t)nblocks * RADIX * 4);
    w.blk_pos = reinterpret_cast<int32_t *>(p + off);
    off += align256((size_t)nblocks * 4);
    w.bytes = off;
    return w;
}

template <int E>
hipError_t run_sort(const Geometry &g, const float *scores, int32_t *idx, const SortWs &w,
                    hipStream_t stream) {
    const int64_t nblocks = g.list_entries / E;
    const unsigned lists = (unsigned)((int64_t)g.B * g.Hq * lists_per_head(g));
    // pass p: input keys/vals -> output keys/vals
    //   0: scores           -> keys_a, vals_a
    //   1: keys_a, vals_a   -> keys_b, idx      (idx doubles as scratch)
    //   2: keys_b, idx      -> keys_a, vals_a
    //   3: keys_a, vals_a   -> idx (positions only)
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 8 * pass;
        const void *kin = pass == 0 ? (const void *)scores : pass == 2 ? (const void *)w.keys_b
                                                                       : (const void *)w.keys_a;
        const int32_t *vin = pass == 1 ? w.vals_a : pass == 2 ? idx : w.vals_a;
        uint32_t *kout = pass == 1 ? w.keys_b : w.keys_a;
        int32_t *vout = pass == 1 || pass == 3 ? idx : w.vals_a;
        if (pass == 0)
            hipLaunchKernelGGL((hist_kernel<E, true>), dim3((unsigned)nblocks), dim3(SORT_THREADS), 0,
                               stream, kin, w.hist, shift);
        else
            hipLaunchKernelGGL((hist_kernel<E, false>), dim3((unsigned)nblocks), dim3(SORT_THREADS), 0,
                               stream, kin, w.hist, shift);
        hipLaunchKernelGGL(scan_kernel, dim3(lists), dim3(RADIX), 0, stream, w.hist, w.blk_pos, g, E,
                           pass == 0 ? 1 : 0);
        if (pass == 0)
            hipLaunchKernelGGL((scatter_kernel<E, true, false>), dim3((unsigned)nblocks),
                               dim3(SORT_THREADS), 0, stream, kin, vin, kout, vout, w.hist, w.blk_pos,
                               shift);
        else if (pass == 3)
            hipLaunchKernelGGL((scatter_kernel<E, false, true>), dim3((unsigned)nblocks),
                               dim3(SORT_THREADS), 0, stream, kin, vin, kout, vout, w.hist, w.blk_pos,
                               shift);
        else
            hipLaunchKernelGGL((scatter_kernel<E, false, false>), dim3((unsigned)nblocks),
                               dim3(SORT_THREADS), 0, stream, kin, vin, kout, vout, w.hist, w.blk_pos,
                               shift);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t sort_workspace_bytes(const Geometry &g) { return carve(g, nullptr).bytes; }

hipError_t launch_sort(const Geometry &g, const float *scores, int32_t *idx, void *ws,
                       hipStream_t stream) {
    if (g.list_entries == 0) return hipSuccess;
    SortWs w = carve(g, ws);
    switch (block_elems(g)) {
        case 4096: return run_sort<4096>(g, scores, idx, w, stream);
        case 2048: return run_sort<2048>(g, scores, idx, w, stream);
        case 1024: return run_sort<1024>(g, scores, idx, w, stream);
        case 512: return run_sort<512>(g, scores, idx, w, stream);
        case 256: return run_sort<256>(g, scores, idx, w, stream);
        case 128: return run_sort<128>(g, scores, idx, w, stream);
        default: return run_sort<64>(g, scores, idx, w, stream);
    }
}

}  // namespace s2o
