// Segmented sort of the index lists by (score descending, position), gfx950.
//
// "S2O: Early Stopping for Sparse Attention via Online Permutation",
// gist.science technical summary, "Classement par Segment" (KV_perm): the
// history keys of each list are ordered by their score; the indices form the
// logical map the attention kernel follows.  Order: score descending, ties to
// the lower position.  -0.0 is folded onto +0.0 so the two tie.
//
// Every list is a multiple of the segment length S long and starts at a
// multiple of S, so the concatenated lists split into equal blocks of E
// entries (E = largest power of two dividing S, at most 4096) that never
// straddle two lists.  Two data passes instead of four LSD passes:
//
//   1. bucket pass (one MSD step).  Each list's scores are split into
//      256 buckets of equal width between the minimum and maximum of a sample
//      of the list (every 16th run of 64 scores), highest values first; scores
//      outside the sampled range join the end buckets.  The bucket function is
//      monotone in the score (clamping keeps it so), so every bucket holds a
//      contiguous range of the final order, and equal scores share a bucket;
//      the sample only affects how evenly the buckets fill.  plan (per list:
//      sample bounds) -> hist (per block, LDS atomics) -> scan (per list) ->
//      scatter (per block: a slot in its digit's run for every entry from LDS
//      atomics on the block's digit counters, staged in LDS, written as
//      contiguous bucket runs of (key, position) pairs; each XCD takes a
//      contiguous share of the blocks, so the partial cache lines where
//      neighbouring blocks' runs meet are merged in one L2).  The order
//      inside a bucket is arbitrary; the steps below do not rely on it.
//   2. range sort.  Each workgroup owns the buckets that start inside its
//      chunk of C output positions, i.e. a contiguous range of the list, and
//      orders it without radix passes: NSB sub-buckets of equal score width
//      over the range (LDS atomics count them, a scan places them), then each
//      entry's rank inside its sub-bucket is counted by comparing (key,
//      position) with the few entries sharing it.  A range whose sub-buckets
//      are too full (clustered or repeated scores) or that exceeds the stage
//      (RANGE_CAP entries, sized for five workgroups per CU) is queued.  A
//      second kernel ranks queued ranges of up to CAP entries by sub-buckets
//      in a larger stage; what remains (crowded sub-buckets, or above CAP)
//      goes to a second queue, sorted by stable 8-bit LSD passes over the
//      bytes of the position, then of the key, that vary inside the range
//      (both relative to the range's lowest value): in LDS when the range
//      fits, else through global scratch, chunk by chunk in order.  Exact, and
//      ordered by (key, position) like the rest.
// When no list is longer than the LDS capacity (block lists, short sequences)
// one workgroup sorts each whole list in LDS and no workspace is used.
#include "s2o_internal.h"

#include <math.h>

namespace s2o {
namespace {

constexpr int NB = 256;        // buckets of pass 1 = radix of the LSD passes
constexpr int THREADS = 256;
constexpr int NWAVES = THREADS / 64;
constexpr int MAX_BLOCK = 4096;  // entries per pass-1 block
constexpr int MAX_CHUNK = 2048;  // output positions owned by a range-sort workgroup
constexpr int CAP = 4096;        // entries a range-sort workgroup holds in LDS
constexpr int CAP_ROUNDS = CAP / THREADS;
constexpr int RANGE_CAP = 3072;  // entries a range-sort workgroup stages (5 workgroups per CU)
constexpr int QUEUED_GRID = 1024;    // workgroups ranking the queued ranges
constexpr int OVERFLOW_GRID = 1024;  // workgroups draining the overflow queue
constexpr int NSB = 1536;        // value-linear sub-buckets of a range (LDS: 4 ranges per CU)
constexpr int SUB_LIMIT = 32;    // largest sub-bucket ranked by direct comparison
static_assert(NSB % (4 * THREADS) == 0 || NSB % THREADS == 0, "sub-bucket scan: whole counters per thread");
static_assert(NSB + 1 >= NWAVES * NB, "the LSD fallback reuses the sub-bucket counters");
static_assert(THREADS == NB, "the in-LDS passes give each thread one digit");
static_assert(NWAVES * NB == 4 * THREADS, "counter clear: four per thread");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> uint32 whose ascending order is descending score order
__device__ inline uint32_t desc_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;  // -0.0 ties with +0.0
    uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}

__device__ inline uint64_t lanemask_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Lanes of the wave holding the same 8-bit digit as this lane: per bit, the
// ballot of lanes with the bit set, complemented where this lane's bit is
// clear (xnor with the bit spread over a word), ANDed over the bits.
__device__ inline uint64_t match_digit(uint32_t digit) {
    uint32_t lo = ~0u, hi = ~0u;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const uint32_t m = (uint32_t)((int32_t)(digit << (31 - bit)) >> 31);  // 0 or ~0
        const uint64_t bal = __ballot(m != 0u);
        lo &= ~((uint32_t)bal ^ m);
        hi &= ~((uint32_t)(bal >> 32) ^ m);
    }
    return ((uint64_t)hi << 32) | lo;
}

// Exclusive scan of 256 ints in LDS, in place, by the first wave; the totals'
// sum is returned to that wave.  Callers synchronise around it.
__device__ inline void scan256(int *v) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        int a0 = v[4 * lane], a1 = v[4 * lane + 1], a2 = v[4 * lane + 2], a3 = v[4 * lane + 3];
        int sum = a0 + a1 + a2 + a3, incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            int x = __shfl_up(incl, d);
            if (lane >= d) incl += x;
        }
        int ex = incl - sum;
        v[4 * lane] = ex;
        v[4 * lane + 1] = ex + a0;
        v[4 * lane + 2] = ex + a0 + a1;
        v[4 * lane + 3] = ex + a0 + a1 + a2;
    }
}

// A list: global list id -> its offset and length in the concatenated layout.
struct ListRef {
    int64_t off, len;
};
__device__ inline ListRef list_ref(const Geometry &g, int lid) {
    const int U = lists_per_head(g);
    const int bh = lid / U, t = list_owner(g, lid % U);
    return {list_offset(g, bh / g.Hq, bh % g.Hq, t), seg_start(g, t)};
}

// Bucket function of pass 1: NB buckets of equal width over [lo, hi], the
// highest scores in digit 0, values outside [lo, hi] clamped to the end
// buckets.  Non-increasing in x, so buckets never interleave.
struct Buckets {
    float lo, sc;  // sc = 0: a single bucket
};
__device__ inline uint32_t bucket_digit(float x, Buckets r) {
    if (!(r.sc > 0.f)) return NB - 1;
    const float f = fminf(fmaxf((x - r.lo) * r.sc, 0.f), (float)(NB - 1));
    return (uint32_t)(NB - 1 - (int)f);
}

// Scores a list's bounds are sampled from: every SAMPLE_STRIDE-th run of
// SAMPLE_RUN consecutive scores (a run is 256 bytes).
constexpr int SAMPLE_RUN = 64;
constexpr int SAMPLE_STRIDE = 16;

// One workgroup per list: records which list every block belongs to, the
// list's bucket parameters from the sampled minimum and maximum, and empties
// the overflow queues.
__global__ __launch_bounds__(THREADS) void plan_kernel(const float *__restrict__ scores,
                                                       int32_t *__restrict__ blk_list, Buckets *__restrict__ list_bk,
                                                       int32_t *__restrict__ queue_len, Geometry g, int E) {
    __shared__ float red[2][NWAVES];
    if (blockIdx.x == 0 && threadIdx.x < 2) queue_len[threadIdx.x] = 0;  // both queues
    const ListRef L = list_ref(g, blockIdx.x);
    const int64_t b0 = L.off / E, nb = L.len / E;
    for (int64_t i = threadIdx.x; i < nb; i += THREADS) blk_list[b0 + i] = (int32_t)blockIdx.x;
    if (L.len == 0) return;
    // every length is a multiple of SAMPLE_RUN; sampled runs 0, STRIDE, 2*STRIDE, ...
    const int64_t runs = (L.len / SAMPLE_RUN + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
    constexpr int PIECES = SAMPLE_RUN / 4;  // float4 pieces per run
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t i = threadIdx.x; i < runs * PIECES; i += THREADS) {
        const int64_t pos = (i / PIECES) * SAMPLE_STRIDE * SAMPLE_RUN + (i % PIECES) * 4;
        const float4 x = *reinterpret_cast<const float4 *>(scores + L.off + pos);
        lo = fminf(fminf(lo, x.x), fminf(x.y, fminf(x.z, x.w)));
        hi = fmaxf(fmaxf(hi, x.x), fmaxf(x.y, fmaxf(x.z, x.w)));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, o));
        hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < NWAVES; ++w) {
            lo = fminf(lo, red[0][w]);
            hi = fmaxf(hi, red[1][w]);
        }
        const float d = hi - lo;
        float sc = d > 0.f ? (float)NB / d : 0.f;
        if (!(sc < INFINITY)) sc = 0.f;  // d overflowed or is denormal-small
        list_bk[blockIdx.x] = {lo, sc};
    }
}

// Per block: bucket histogram (order-free, so LDS atomics).
__global__ __launch_bounds__(THREADS) void hist_kernel(const float *__restrict__ scores,
                                                       const int32_t *__restrict__ blk_list,
                                                       const Buckets *__restrict__ list_bk,
                                                       int32_t *__restrict__ hist, int E) {
    __shared__ int cnt[NWAVES][NB];
    for (int i = threadIdx.x; i < NWAVES * NB; i += THREADS) (&cnt[0][0])[i] = 0;
    const Buckets bk = list_bk[blk_list[blockIdx.x]];
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const float *s = scores + (int64_t)blockIdx.x * E;
    constexpr int PER = MAX_BLOCK / (4 * THREADS);
    float4 xs[PER];  // every load of the thread is issued before the first is used
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int i = 4 * threadIdx.x + it * 4 * THREADS;
        if (i < E) xs[it] = *reinterpret_cast<const float4 *>(s + i);
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        if (4 * threadIdx.x + it * 4 * THREADS >= E) break;
        const float4 x = xs[it];
        atomicAdd(&cnt[wave][bucket_digit(x.x, bk)], 1);
        atomicAdd(&cnt[wave][bucket_digit(x.y, bk)], 1);
        atomicAdd(&cnt[wave][bucket_digit(x.z, bk)], 1);
        atomicAdd(&cnt[wave][bucket_digit(x.w, bk)], 1);
    }
    __syncthreads();
    for (int v = threadIdx.x; v < NB; v += THREADS) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) c += cnt[w][v];
        hist[(int64_t)blockIdx.x * NB + v] = c;
    }
}

// One workgroup (NB threads) per list.  Turns the block histograms into the
// start of each block's bucket run relative to the block's first entry,
//   hist[bb][v] = off + base[v] + sum_{bb' < bb} count[bb'][v] - bb*E,
// and records the list's bucket starts base[0..NB) and its length.
__global__ __launch_bounds__(NB) void scan_kernel(int32_t *__restrict__ hist, int32_t *__restrict__ bstart,
                                                  Geometry g, int E) {
    __shared__ int tot[NB];
    const ListRef L = list_ref(g, blockIdx.x);
    if (L.len == 0) return;
    const int64_t b0 = L.off / E, nb = L.len / E;
    const int v = threadIdx.x;
    // the blocks' counts are read SCAN_BATCH at a time, all loads before the first use
    constexpr int SCAN_BATCH = 8;
    int run = 0;
    for (int64_t bb = b0; bb < b0 + nb; bb += SCAN_BATCH) {
        int c[SCAN_BATCH];
#pragma unroll
        for (int u = 0; u < SCAN_BATCH; ++u) c[u] = bb + u < b0 + nb ? hist[(bb + u) * NB + v] : 0;
#pragma unroll
        for (int u = 0; u < SCAN_BATCH; ++u) {
            if (bb + u < b0 + nb) hist[(bb + u) * NB + v] = run;
            run += c[u];
        }
    }
    tot[v] = run;
    __syncthreads();
    scan256(tot);
    __syncthreads();
    const int base = tot[v];
    for (int64_t bb = b0; bb < b0 + nb; bb += SCAN_BATCH) {
        int c[SCAN_BATCH];
#pragma unroll
        for (int u = 0; u < SCAN_BATCH; ++u) c[u] = bb + u < b0 + nb ? hist[(bb + u) * NB + v] : 0;
#pragma unroll
        for (int u = 0; u < SCAN_BATCH; ++u)
            if (bb + u < b0 + nb) hist[(bb + u) * NB + v] = c[u] + (int)(base + L.off - (bb + u) * E);
    }
    int32_t *bs = bstart + (int64_t)blockIdx.x * (NB + 1);
    bs[v] = base;
    if (v == 0) bs[NB] = (int32_t)L.len;
}

// Per block: scatter into bucket runs of (key, position) pairs.  LDS atomics on
// one set of digit counters hand each entry a slot in its digit's run, in no
// particular order (the range sort orders every range by (key, position)
// itself); the entries are staged in LDS by digit and written as runs.
template <int E>
__global__ __launch_bounds__(THREADS) void scatter_kernel(const float *__restrict__ scores,
                                                          const int32_t *__restrict__ blk_list,
                                                          const Buckets *__restrict__ list_bk,
                                                          const int32_t *__restrict__ hist,
                                                          u32x2 *__restrict__ pairs, Geometry g, int64_t nblocks) {
    constexpr int NWV = E >= 256 ? NWAVES : E / 64;  // waves holding entries
    constexpr int ROUNDS = E / (64 * NWV);           // wave w owns [w*E/NWV, (w+1)*E/NWV)
    __shared__ int cnt[NB];          // digit counts, then each digit's first staged position
    __shared__ int dglob[NB];        // run start of each digit relative to the block, minus its staged start
    __shared__ u32x2 stage[E];       // (key, position) sorted by digit
    __shared__ uint8_t sdig[E];
    // XCD-aware order: block ids are dispatched round-robin over the 8 XCDs;
    // XCD x takes the contiguous blocks [x*per, (x+1)*per), so the blocks of a
    // list, whose bucket runs abut, write through the same L2
    const int64_t per = gridDim.x / 8;
    const int64_t blk = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
    if (blk >= nblocks) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int v = tid; v < NB; v += THREADS) {
        cnt[v] = 0;
        dglob[v] = hist[blk * NB + v];
    }
    const Buckets bk = list_bk[blk_list[blk]];
    __syncthreads();
    const int64_t base = blk * E;
    const int32_t pos0 = (int32_t)(base - list_ref(g, blk_list[blk]).off);

    float x[ROUNDS];
    uint32_t dig[ROUNDS];
    int rank[ROUNDS];
    if (wave < NWV) {
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) x[r] = scores[base + wave * (E / NWV) + 64 * r + lane];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            dig[r] = bucket_digit(x[r], bk);
            rank[r] = atomicAdd(&cnt[dig[r]], 1);  // a slot in the digit's run, in no particular order
        }
    }
    __syncthreads();
    scan256(cnt);
    __syncthreads();
    for (int v = tid; v < NB; v += THREADS) dglob[v] -= cnt[v];
    if (wave < NWV) {
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const int p = cnt[dig[r]] + rank[r];
            u32x2 pr;
            pr.x = desc_key(x[r]);
            pr.y = (uint32_t)(pos0 + wave * (E / NWV) + 64 * r + lane);
            stage[p] = pr;
            sdig[p] = (uint8_t)dig[r];
        }
    }
    __syncthreads();
    for (int i = tid; i < E; i += THREADS) pairs[base + dglob[sdig[i]] + i] = stage[i];
}

// Stable rank of one chunk (striped: entry w*rounds*64 + r*64 + lane) by the
// digit (rel >> shift) & 0xFF, over the first `rounds` of the R register
// rounds.  On return cnt[w][d] holds the offset of wave w's run inside digit
// d's run of the chunk and dtot[d] the chunk's count of d; an entry's position
// inside its digit run is cnt[w][d] + rank[r].
template <int R>
__device__ __forceinline__ void rank_chunk(const uint32_t (&rel)[R], int (&rank)[R], int rounds, int shift,
                                  int (*cnt)[NB], int *dtot) {
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int i = tid; i < NWAVES * NB; i += THREADS) (&cnt[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < rounds) {
            const uint32_t d = (rel[r] >> shift) & 0xFFu;
            const uint64_t peers = match_digit(d);
            const int before = cnt[wave][d];
            rank[r] = before + __popcll(peers & lanemask_lt());
            if ((peers & lanemask_lt()) == 0) cnt[wave][d] = before + __popcll(peers);
        }
        __builtin_amdgcn_sched_barrier(0);  // one round at a time: bounds register use
    }
    __syncthreads();
    for (int v = tid; v < NB; v += THREADS) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const int c = cnt[w][v];
            cnt[w][v] = s;
            s += c;
        }
        dtot[v] = s;
    }
    __syncthreads();
}

// Block-wide reductions (every thread gets the result).
__device__ inline uint32_t block_min(uint32_t x, uint32_t *sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    uint32_t r = sh[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) r = min(r, sh[w]);
    return r;
}
__device__ inline uint32_t block_or(uint32_t x, uint32_t *sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    uint32_t r = sh[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) r |= sh[w];
    return r;
}

// Sorts the m <= R*THREADS entries of one range in LDS and writes their
// positions: stable 8-bit LSD passes on the key relative to the range minimum,
// only over the bytes that vary.  With BY_POS the passes on the key are
// preceded by passes on the position relative to the range's lowest one, so
// the result is ordered by (key, position) whatever the input order; without
// it the input must list equal keys by ascending position.  Padding entries
// (all ones in both) stay last.  load(i) gives entry i as (key, position).
template <int R, bool BY_POS, typename Load>
__device__ __forceinline__ void sort_in_lds(Load load, int32_t *__restrict__ out, int m, u32x2 *stage,
                                            int (*cnt)[NB], uint32_t *red) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wbase = wave * R * 64 + lane;
    uint32_t rel[R];
    uint32_t prel[R];  // position relative to the lowest one
    int rank[R];
    uint32_t kmin = 0xFFFFFFFFu, pmin = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = wbase + 64 * r;
        u32x2 pr;
        pr.x = 0xFFFFFFFFu;
        pr.y = 0xFFFFFFFFu;
        if (i < m) pr = load(i);
        rel[r] = pr.x;
        prel[r] = pr.y;
        kmin = min(kmin, pr.x);
        pmin = min(pmin, pr.y);
    }
    kmin = block_min(kmin, red);
    if (BY_POS) pmin = block_min(pmin, red);
    uint32_t span = 0, pspan = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool real = wbase + 64 * r < m;
        rel[r] = real ? rel[r] - kmin : 0xFFFFFFFFu;
        span |= real ? rel[r] : 0u;
        if (BY_POS) {
            prel[r] = real ? prel[r] - pmin : 0xFFFFFFFFu;
            pspan |= real ? prel[r] : 0u;
        }
    }
    span = block_or(span, red);
    if (BY_POS) pspan = block_or(pspan, red);
    for (int pass = BY_POS ? 0 : 4; pass < 8; ++pass) {
        const bool on_pos = pass < 4;  // position bytes first, then key bytes
        const int shift = 8 * (pass & 3);
        if ((((on_pos ? pspan : span) >> shift) & 0xFFu) == 0) continue;  // digit constant in the range
        // per-wave digit counters: zero, count with stable in-wave ranks
        *reinterpret_cast<int4 *>(&cnt[0][0] + 4 * threadIdx.x) = int4{0, 0, 0, 0};
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t d = ((on_pos ? prel[r] : rel[r]) >> shift) & 0xFFu;
            const uint64_t peers = match_digit(d);
            const int before = cnt[wave][d];
            rank[r] = before + __popcll(peers & lanemask_lt());
            if ((peers & lanemask_lt()) == 0) cnt[wave][d] = before + __popcll(peers);
            __builtin_amdgcn_sched_barrier(0);  // one round at a time: bounds register use
        }
        __syncthreads();
        // thread v = digit v: wave offsets inside the digit, then the digit's
        // start (block-wide exclusive scan: in-wave shuffles, then wave totals)
        {
            const int v = threadIdx.x;
            int tot = 0;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) {
                const int c = cnt[w][v];
                cnt[w][v] = tot;
                tot += c;
            }
            int incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int x = __shfl_up(incl, o);
                if (lane >= o) incl += x;
            }
            if (lane == 63) red[wave] = (uint32_t)incl;
            __syncthreads();
            int base = 0;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) base += w < wave ? (int)red[w] : 0;
            const int start = base + incl - tot;  // first staged position of digit v
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) cnt[w][v] += start;
        }
        __syncthreads();
        // stage (key, position) pairs sorted by the digit: one read, one 8-byte write
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t d = ((on_pos ? prel[r] : rel[r]) >> shift) & 0xFFu;
            u32x2 pr;
            pr.x = rel[r];
            pr.y = prel[r];
            stage[cnt[wave][d] + rank[r]] = pr;
        }
        __syncthreads();
        // (the next pass writes the stage only after its own barriers)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x2 pr = stage[wbase + 64 * r];
            rel[r] = pr.x;
            prel[r] = pr.y;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (wbase + 64 * r < m) out[wbase + 64 * r] = (int32_t)(prel[r] + (BY_POS ? pmin : 0u));
}

// Inverse of desc_key: the score a key stands for (-0.0 comes back as +0.0).
__device__ inline float key_score(uint32_t key) {
    const uint32_t asc = ~key;
    return __uint_as_float((asc & 0x80000000u) ? (asc & 0x7FFFFFFFu) : ~asc);
}

// Sorts the m <= R*THREADS entries of one range and writes their positions,
// without radix passes: every entry goes to one of NSB sub-buckets of equal
// score width between the range's extremes (highest scores first; the map is
// monotone in the key, so sub-buckets hold contiguous runs of the order),
// counted with LDS atomics and placed by an exclusive scan; an entry's final
// rank is its sub-bucket's start plus the number of entries of its sub-bucket
// that precede it in (key, position) order.  The result is the unique sorted
// order, whatever order the atomics hand out slots in.  Returns false, having
// written nothing, when some sub-bucket holds more than SUB_LIMIT entries
// (clustered or repeated scores); the caller then sorts the range otherwise.
template <int R>
__device__ __forceinline__ bool rank_in_sub_buckets(const u32x2 *__restrict__ in, int32_t *__restrict__ out,
                                                    int m, uint64_t *stage, int *sbc, int *red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wbase = wave * R * 64 + lane;
    // Entries as (key << 32 | position): one 64-bit comparison orders them.
    // Padding entries (index >= m) take the same steps without branches: they
    // count into sbc[NSB], land in the stage's tail [m, R*THREADS) and write nothing.
    uint64_t e[R];
    int dig[R], slot[R];
    uint32_t kmin = 0xFFFFFFFFu, nkmax = 0xFFFFFFFFu;  // nkmax = ~(largest key)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = wbase + 64 * r;
        const bool real = i < m;
        const u32x2 v = in[real ? i : m - 1];  // in bounds for every lane, no branch
        const uint32_t key = real ? v.x : 0xFFFFFFFFu;
        e[r] = ((uint64_t)key << 32) | (real ? v.y : 0u);
        kmin = min(kmin, key);
        nkmax = min(nkmax, real ? ~v.x : 0xFFFFFFFFu);
    }
    for (int i = tid; i <= NSB; i += THREADS) sbc[i] = 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        nkmax = min(nkmax, (uint32_t)__shfl_xor((int)nkmax, o));
    }
    if (lane == 0) {
        red[wave] = (int)kmin;
        red[NWAVES + wave] = (int)nkmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
        kmin = min(kmin, (uint32_t)red[w]);
        nkmax = min(nkmax, (uint32_t)red[NWAVES + w]);
    }
    // sub-bucket of a score: floor((top - x) * NSB / (top - bottom)), clamped;
    // a single sub-bucket when the width is zero, not finite or too small to divide by
    const float top = key_score(kmin), width = top - key_score(~nkmax);
    const float scale = (float)NSB / width;
    const bool spread = width > 0.f && width < INFINITY && scale < INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int d = spread ? min((int)((top - key_score((uint32_t)(e[r] >> 32))) * scale), NSB - 1) : 0;
        dig[r] = wbase + 64 * r < m ? d : NSB;
        slot[r] = atomicAdd(&sbc[dig[r]], 1);
    }
    __syncthreads();
    // exclusive scan of the counts in place (sbc[NSB] = m), and the largest count
    {
        constexpr int PER = NSB / THREADS;
        int c[PER];
        int tot = 0, cmax = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            c[k] = sbc[tid * PER + k];
            tot += c[k];
            cmax = max(cmax, c[k]);
        }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int x = __shfl_up(incl, o);
            if (lane >= o) incl += x;
            cmax = max(cmax, __shfl_xor(cmax, o));
        }
        if (lane == 63) red[2 * NWAVES + wave] = incl;
        if (lane == 0) red[3 * NWAVES + wave] = cmax;
        __syncthreads();
        int base = 0;
        cmax = 0;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            base += w < wave ? red[2 * NWAVES + w] : 0;
            cmax = max(cmax, red[3 * NWAVES + w]);
        }
        if (cmax > SUB_LIMIT) return false;  // the same on every thread
        int run = base + incl - tot;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            sbc[tid * PER + k] = run;
            run += c[k];
        }
        if (tid == THREADS - 1) sbc[NSB] = run;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) stage[sbc[dig[r]] + slot[r]] = e[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int d = dig[r];
        const int b0 = sbc[d], b1 = d < NSB ? sbc[d + 1] : b0;
        int rank = b0;
        if (b1 - b0 > 1) {
            for (int j = b0; j < b1; ++j) rank += stage[j] < e[r] ? 1 : 0;
        }
        if (d < NSB) out[rank] = (int32_t)(uint32_t)e[r];
    }
    return true;
}

// A range queued for overflow_kernel.
struct Overflow {
    int32_t lid, rs, m;
};

// One workgroup per chunk of C output positions of a list: sorts the buckets
// that start inside the chunk (see the file comment) and writes positions.
// A range larger than RANGE_CAP, or with a sub-bucket fuller than SUB_LIMIT,
// is queued for overflow_kernel instead.
template <int C>
__global__ __launch_bounds__(THREADS, 4) void range_sort_kernel(const u32x2 *__restrict__ pairs,
                                                                int32_t *__restrict__ idx,
                                                                const int32_t *__restrict__ blk_list,
                                                                const int32_t *__restrict__ bstart,
                                                                Overflow *__restrict__ queue,
                                                                int32_t *__restrict__ queue_len,
                                                                Geometry g, int E) {
    __shared__ uint64_t stage[RANGE_CAP];
    __shared__ int sbc[NSB + 1];
    __shared__ int sred[4 * NWAVES];
    const int tid = threadIdx.x;
    const int64_t e0 = (int64_t)blockIdx.x * C;
    const int lid = blk_list[e0 / E];
    const ListRef L = list_ref(g, lid);
    const int32_t g0 = (int32_t)(e0 - L.off);
    const int32_t *bs = bstart + (int64_t)lid * (NB + 1);
    // buckets starting in [g0, g0 + C) are [lo_b, hi_b); bs[NB] = len >= g0 + C
    const int lo_b = __syncthreads_count(bs[tid] < g0);
    const int hi_b = __syncthreads_count(bs[tid] < g0 + C);
    const int32_t rs = bs[lo_b], m = bs[hi_b] - rs;
    if (m == 0) return;
    if (m > RANGE_CAP) {
        if (tid == 0) queue[atomicAdd(queue_len, 1)] = {lid, rs, m};
        return;
    }
    const u32x2 *in = pairs + L.off + rs;
    int32_t *out = idx + L.off + rs;
    switch ((m + THREADS - 1) / THREADS) {  // one instantiation per round count
#define S2O_SORT_CASE(R)                                                   \
    case R:                                                                \
        if (!rank_in_sub_buckets<R>(in, out, m, stage, sbc, sred) && tid == 0) \
            queue[atomicAdd(queue_len, 1)] = {lid, rs, m};                     \
        break;
        S2O_SORT_CASE(1) S2O_SORT_CASE(2) S2O_SORT_CASE(3) S2O_SORT_CASE(4)
        S2O_SORT_CASE(5) S2O_SORT_CASE(6) S2O_SORT_CASE(7) S2O_SORT_CASE(8)
        S2O_SORT_CASE(9) S2O_SORT_CASE(10) S2O_SORT_CASE(11) S2O_SORT_CASE(12)
#undef S2O_SORT_CASE
        default: break;
    }
}

// Short lists (every list at most CAP entries, e.g. block lists): one
// workgroup sorts a whole list in LDS straight from the scores.
__global__ __launch_bounds__(THREADS, 4) void list_sort_kernel(const float *__restrict__ scores,
                                                               int32_t *__restrict__ idx, Geometry g) {
    __shared__ u32x2 stage[CAP];
    __shared__ int cnt[NWAVES][NB];
    __shared__ uint32_t red[NWAVES];
    const ListRef L = list_ref(g, blockIdx.x);
    const int m = (int)L.len;
    if (m == 0) return;
    const float *s = scores + L.off;
    int32_t *out = idx + L.off;
    auto load = [s](int i) {
        u32x2 pr;
        pr.x = desc_key(s[i]);
        pr.y = (uint32_t)i;
        return pr;
    };
    switch ((m + THREADS - 1) / THREADS) {
#define S2O_SORT_CASE(R) \
    case R: sort_in_lds<R, false>(load, out, m, stage, cnt, red); break;
        S2O_SORT_CASE(1) S2O_SORT_CASE(2) S2O_SORT_CASE(3) S2O_SORT_CASE(4)
        S2O_SORT_CASE(5) S2O_SORT_CASE(6) S2O_SORT_CASE(7) S2O_SORT_CASE(8)
        S2O_SORT_CASE(9) S2O_SORT_CASE(10) S2O_SORT_CASE(11) S2O_SORT_CASE(12)
        S2O_SORT_CASE(13) S2O_SORT_CASE(14) S2O_SORT_CASE(15) S2O_SORT_CASE(16)
#undef S2O_SORT_CASE
        default: break;
    }
}

// Queued ranges of up to CAP entries, ranked by sub-buckets in a CAP-entry
// stage (range_sort_kernel's stage is smaller); each workgroup takes queued
// ranges in turn.  Ranges above CAP, and those whose sub-buckets are crowded,
// go on to the second queue.
__global__ __launch_bounds__(THREADS, 4) void queued_range_kernel(const u32x2 *__restrict__ pairs,
                                                                  int32_t *__restrict__ idx,
                                                                  const Overflow *__restrict__ queue,
                                                                  const int32_t *__restrict__ queue_len,
                                                                  Overflow *__restrict__ queue2,
                                                                  int32_t *__restrict__ queue2_len,
                                                                  Geometry g) {
    __shared__ uint64_t stage[CAP];
    __shared__ int sbc[NSB + 1];
    __shared__ int sred[4 * NWAVES];
    const int tid = threadIdx.x;
    const int nq = *queue_len;
    for (int q = blockIdx.x; q < nq; q += gridDim.x) {
        const Overflow ov = queue[q];
        const int64_t base = list_ref(g, ov.lid).off + ov.rs;
        const int m = ov.m;
        bool done = false;
        switch ((m + THREADS - 1) / THREADS) {
#define S2O_SORT_CASE(R) \
    case R: done = rank_in_sub_buckets<R>(pairs + base, idx + base, m, stage, sbc, sred); break;
            S2O_SORT_CASE(1) S2O_SORT_CASE(2) S2O_SORT_CASE(3) S2O_SORT_CASE(4)
            S2O_SORT_CASE(5) S2O_SORT_CASE(6) S2O_SORT_CASE(7) S2O_SORT_CASE(8)
            S2O_SORT_CASE(9) S2O_SORT_CASE(10) S2O_SORT_CASE(11) S2O_SORT_CASE(12)
            S2O_SORT_CASE(13) S2O_SORT_CASE(14) S2O_SORT_CASE(15) S2O_SORT_CASE(16)
#undef S2O_SORT_CASE
            default: break;  // above CAP
        }
        if (!done && tid == 0) queue2[atomicAdd(queue2_len, 1)] = ov;
        __syncthreads();  // the next range reuses the LDS
    }
}

// Ranges left over by queued_range_kernel (crowded sub-buckets, or above CAP):
// each workgroup takes them in turn; one that fits in LDS is sorted there
// with stable LSD passes, a larger one with stable LSD passes through global
// scratch, CAP entries at a time in order.  The scratch copy of a range sits
// at the range's own offset (slot_len = 0: scratch as long as the lists), or
// in the workgroup's slot of slot_len entries (slot_len >= the longest list).
__global__ __launch_bounds__(THREADS) void overflow_kernel(u32x2 *__restrict__ pairs,
                                                           u32x2 *__restrict__ scratch,
                                                           int32_t *__restrict__ idx,
                                                           const Overflow *__restrict__ queue,
                                                           const int32_t *__restrict__ queue_len,
                                                           Geometry g, int64_t slot_len) {
    __shared__ u32x2 stage[CAP];
    __shared__ int cnt[NWAVES][NB];
    __shared__ int dtot[NB];
    __shared__ int run[NB];
    __shared__ uint32_t red[NWAVES];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nq = *queue_len;
    uint32_t rel[CAP_ROUNDS], key[CAP_ROUNDS];
    int32_t pos[CAP_ROUNDS];
    int rank[CAP_ROUNDS];
    for (int q = blockIdx.x; q < nq; q += gridDim.x) {
        const Overflow ov = queue[q];
        const int64_t base = list_ref(g, ov.lid).off + ov.rs;
        const int m = ov.m;
        if (m <= CAP) {  // fits in LDS
            const u32x2 *in = pairs + base;
            auto load = [in](int i) { return in[i]; };
            switch ((m + THREADS - 1) / THREADS) {
#define S2O_SORT_CASE(R) \
    case R: sort_in_lds<R, true>(load, idx + base, m, stage, cnt, red); break;
                S2O_SORT_CASE(1) S2O_SORT_CASE(2) S2O_SORT_CASE(3) S2O_SORT_CASE(4)
                S2O_SORT_CASE(5) S2O_SORT_CASE(6) S2O_SORT_CASE(7) S2O_SORT_CASE(8)
                S2O_SORT_CASE(9) S2O_SORT_CASE(10) S2O_SORT_CASE(11) S2O_SORT_CASE(12)
                S2O_SORT_CASE(13) S2O_SORT_CASE(14) S2O_SORT_CASE(15) S2O_SORT_CASE(16)
#undef S2O_SORT_CASE
                default: break;
            }
            __syncthreads();  // the next range reuses the LDS
            continue;
        }
        u32x2 *src = pairs + base;
        u32x2 *dst = scratch + (slot_len > 0 ? (int64_t)blockIdx.x * slot_len : base);
        uint32_t kmin = 0xFFFFFFFFu, pmin = 0xFFFFFFFFu;
        for (int i = tid; i < m; i += THREADS) {
            kmin = min(kmin, src[i].x);
            pmin = min(pmin, src[i].y);
        }
        kmin = block_min(kmin, red);
        pmin = block_min(pmin, red);
        uint32_t span = 0, pspan = 0;
        for (int i = tid; i < m; i += THREADS) {
            span |= src[i].x - kmin;
            pspan |= src[i].y - pmin;
        }
        span = block_or(span, red);
        pspan = block_or(pspan, red);
        // position bytes first, then key bytes: ordered by (key, position)
        for (int pass = 0; pass < 8; ++pass) {
            const bool on_pos = pass < 4;
            const int shift = 8 * (pass & 3);
            if ((((on_pos ? pspan : span) >> shift) & 0xFFu) == 0) continue;
            auto value = [&](u32x2 pr) { return on_pos ? pr.y - pmin : pr.x - kmin; };
            for (int v = tid; v < NB; v += THREADS) run[v] = 0;
            __syncthreads();
            for (int i = tid; i < m; i += THREADS) atomicAdd(&run[(value(src[i]) >> shift) & 0xFFu], 1);
            __syncthreads();
            scan256(run);
            __syncthreads();
            for (int c0 = 0; c0 < m; c0 += CAP) {
                const int cm = min(CAP, m - c0);
                const int rounds = (cm + THREADS - 1) / THREADS;
                const int wbase = wave * rounds * 64 + lane;
#pragma unroll
                for (int r = 0; r < CAP_ROUNDS; ++r) {
                    if (r < rounds) {
                        const int i = wbase + 64 * r;
                        if (i < cm) {
                            const u32x2 pr = src[c0 + i];
                            rel[r] = value(pr);
                            key[r] = pr.x;
                            pos[r] = (int32_t)pr.y;
                        } else {
                            rel[r] = 0xFFFFFFFFu;
                            key[r] = 0;
                            pos[r] = 0;
                        }
                    }
                }
                rank_chunk<CAP_ROUNDS>(rel, rank, rounds, shift, cnt, dtot);
#pragma unroll
                for (int r = 0; r < CAP_ROUNDS; ++r) {
                    if (r < rounds && wbase + 64 * r < cm) {
                        const uint32_t d = (rel[r] >> shift) & 0xFFu;
                        u32x2 pr;
                        pr.x = key[r];
                        pr.y = (uint32_t)pos[r];
                        dst[run[d] + cnt[wave][d] + rank[r]] = pr;
                    }
                }
                __syncthreads();
                // padding entries (all ones, digit 0xFF in every pass) rank after
                // every real entry of digit 0xFF and are neither written nor counted
                for (int v = tid; v < NB; v += THREADS) run[v] += dtot[v] - (v == 0xFF ? rounds * THREADS - cm : 0);
                __syncthreads();
            }
            u32x2 *t = src;
            src = dst;
            dst = t;
        }
        for (int i = tid; i < m; i += THREADS) idx[base + i] = (int32_t)src[i].y;
        __syncthreads();  // the next range reuses the LDS
    }
}

int block_elems(const Geometry &g) {
    int e = g.S & (-g.S);  // largest power of two dividing S
    return e > MAX_BLOCK ? MAX_BLOCK : e;
}

// Longest list: the last segment's history.
int64_t max_list_len(const Geometry &g) { return (int64_t)(g.nseg - 1) * g.S; }
bool short_lists(const Geometry &g) { return max_list_len(g) <= CAP; }

int range_chunk(const Geometry &g) {
    const int e = block_elems(g);
    return e < MAX_CHUNK ? e : MAX_CHUNK;
}

struct SortWs {
    u32x2 *pairs, *scratch;
    int64_t slot_len;  // 0: scratch mirrors pairs; else one slot of this many entries per overflow workgroup
    int32_t *hist, *blk_list, *bstart, *queue_len;
    Buckets *list_bk;
    Overflow *queue, *queue2;
    size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SortWs carve(const Geometry &g, void *base) {
    const int64_t n = g.list_entries;
    const int64_t nblocks = n / block_elems(g);
    const int64_t lists = (int64_t)g.B * g.Hq * lists_per_head(g);
    SortWs w;
    size_t off = 0;
    char *p = reinterpret_cast<char *>(base);
    w.pairs = reinterpret_cast<u32x2 *>(p + off);
    off += align256(n * 8);
    // the overflow kernel's scratch: a copy of the lists, or one slot per
    // workgroup as long as the longest list, whichever is smaller
    const int64_t slots = (int64_t)OVERFLOW_GRID * max_list_len(g);
    w.slot_len = slots < n ? max_list_len(g) : 0;
    w.scratch = reinterpret_cast<u32x2 *>(p + off);
    off += align256((size_t)(w.slot_len > 0 ? slots : n) * 8);
    w.hist = reinterpret_cast<int32_t *>(p + off);
    off += align256((size_t)nblocks * NB * 4);
    w.blk_list = reinterpret_cast<int32_t *>(p + off);
    off += align256((size_t)nblocks * 4);
    w.list_bk = reinterpret_cast<Buckets *>(p + off);
    off += align256((size_t)lists * sizeof(Buckets));
    w.bstart = reinterpret_cast<int32_t *>(p + off);
    off += align256((size_t)lists * (NB + 1) * 4);
    w.queue = reinterpret_cast<Overflow *>(p + off);  // at most one entry per chunk
    off += align256((size_t)(n / range_chunk(g)) * sizeof(Overflow));
    w.queue2 = reinterpret_cast<Overflow *>(p + off);  // a subset of the first queue
    off += align256((size_t)(n / range_chunk(g)) * sizeof(Overflow));
    w.queue_len = reinterpret_cast<int32_t *>(p + off);  // [0]: first queue, [1]: second
    off += 256;
    w.bytes = off;
    return w;
}

template <int E>
hipError_t run_sort(const Geometry &g, const float *scores, int32_t *idx, const SortWs &w,
                    hipStream_t stream) {
    constexpr int C = E < MAX_CHUNK ? E : MAX_CHUNK;  // = range_chunk(g)
    const int64_t nblocks = g.list_entries / E;
    const unsigned lists = (unsigned)((int64_t)g.B * g.Hq * lists_per_head(g));
    hipLaunchKernelGGL(plan_kernel, dim3(lists), dim3(THREADS), 0, stream, scores, w.blk_list, w.list_bk,
                       w.queue_len, g, E);
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nblocks), dim3(THREADS), 0, stream, scores, w.blk_list,
                       w.list_bk, w.hist, E);
    hipLaunchKernelGGL(scan_kernel, dim3(lists), dim3(NB), 0, stream, w.hist, w.bstart, g, E);
    hipLaunchKernelGGL(scatter_kernel<E>, dim3((unsigned)(((nblocks + 7) / 8) * 8)), dim3(THREADS), 0, stream, scores,
                       w.blk_list, w.list_bk, w.hist, w.pairs, g, nblocks);
    hipLaunchKernelGGL(range_sort_kernel<C>, dim3((unsigned)(g.list_entries / C)), dim3(THREADS), 0, stream,
                       w.pairs, idx, w.blk_list, w.bstart, w.queue, w.queue_len, g, E);
    hipLaunchKernelGGL(queued_range_kernel, dim3(QUEUED_GRID), dim3(THREADS), 0, stream, w.pairs, idx, w.queue,
                       w.queue_len, w.queue2, w.queue_len + 1, g);
    hipLaunchKernelGGL(overflow_kernel, dim3(OVERFLOW_GRID), dim3(THREADS), 0, stream, w.pairs, w.scratch, idx,
                       w.queue2, w.queue_len + 1, g, w.slot_len);
    return hipGetLastError();
}

}  // namespace

size_t sort_workspace_bytes(const Geometry &g) { return short_lists(g) ? 0 : carve(g, nullptr).bytes; }

bool sort_supported(const Geometry &g) { return short_lists(g) || block_elems(g) >= 64; }

hipError_t launch_sort(const Geometry &g, const float *scores, int32_t *idx, void *ws,
                       hipStream_t stream) {
    if (g.list_entries == 0) return hipSuccess;
    if (short_lists(g)) {
        const unsigned lists = (unsigned)((int64_t)g.B * g.Hq * lists_per_head(g));
        hipLaunchKernelGGL(list_sort_kernel, dim3(lists), dim3(THREADS), 0, stream, scores, idx, g);
        return hipGetLastError();
    }
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
