// Gathered FlashAttention-style forward for gfx950, dense and S2O schedules.
//
// Method: "S2O: Early Stopping for Sparse Attention via Online Permutation"
// (gist.science technical summary, "3. Implémentation du Noyau": pass 1 is a
// dense causal window inside the current segment that initialises the online
// softmax state (m, l, acc); pass 2 resumes that state and walks the history
// keys in the order of the tile's index list, gathering K/V rows by index
// ("Chargement Planifié par Coordonnées"), and stops early on the marginal
// gain ("2. Règle d'Arrêt Anticipé").  The two passes are fused here: one
// workgroup runs both for its query tile, keeping (m, l, acc) in registers.
//
// Mapping to CDNA4:
//   * one workgroup per (b, query head, query tile of BM = 32*NW rows); each
//     wave owns 32 query rows;
//   * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 (fp32 problems:
//     v_mfma_f32_32x32x2_f32) so that in the 32x32 accumulator layout every
//     lane holds 16 keys of ONE query row: row statistics need one exchange
//     with the partner lane (lane ^ 32) instead of a cross-lane tree;
//   * the same layout makes the probabilities directly usable as the B
//     operand of O^T = V^T P^T, so P never leaves registers;
//   * bf16 (attn_kernel_bf16): K/V chunks of 64 keys go straight from HBM to
//     LDS (buffer loads with the LDS bit, 16 bytes of a gathered row per
//     lane, two stages each, K one chunk ahead of V); V stays row-major in
//     LDS and the PV operand is read with the transposing ds_read_b64_tr_b16;
//     the softmax reference is fixed after a tile's first chunk, with a
//     running-max restart when a chunk's mass overflows the check;
//   * fp32 (attn_kernel_f32): rows are staged through registers into
//     row-major LDS tiles, with the lazy running max throughout;
//   * the stop decision is uniform per workgroup: each wave ballots whether
//     any of its rows still gains >= tau, the waves exchange one flag each
//     through LDS at the barrier that already separates the LDS buffers;
//   * work order is heaviest-first (late tiles first) and the G query heads
//     sharing one KV head are placed on the same XCD so they share its L2.
#include "s2o_internal.h"

#include <mutex>
#include <type_traits>

namespace s2o {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct AttnParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    const int32_t *idx;
    const int32_t *qorder;  // Q_perm: row order of every segment (null: rows in place)
    int32_t *exec;
    Geometry g;
    float scale_log2;  // softmax scale * log2(e)
    float tau;
};

// Block -> (b, h, t).  Units (kv head, t, b) are ordered KV-head-major and,
// within a KV head, t-descending (heaviest tiles first), so that at any time
// the whole chip gathers from one KV head's K/V (67 MB at 128K), which stays in
// the Infinity Cache.  The G query heads of a unit get block ids congruent
// mod 8, i.e. the same XCD, where they share its L2.
struct Work {
    int b, h, t;
};

__device__ inline bool map_block(const Geometry &g, Work &w) {
    int bid = blockIdx.x;
    int x = bid & 7, r = bid >> 3;
    int hq = r % g.G;
    int u = 8 * (r / g.G) + x;
    int units = g.B * g.Hkv * g.T;
    if (u >= units) return false;
    int per_g = g.T * g.B;
    int kvh = u / per_g;
    int rem = u % per_g;
    w.t = g.T - 1 - rem / g.B;
    w.b = rem % g.B;
    w.h = kvh * g.G + hq;
    return true;
}

// Lanes l and l^32 hold the two halves of one query row.  v_permlane32_swap
// applied to (x, x) leaves x of lane l and of lane l^32 in the two results (in
// the same order in both lanes), so max/sum of the pair are bit-identical in
// the two lanes.
__device__ inline float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float max16(const f32x16 &v) {
    float m = v[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, v[r]);
    return m;
}

// Causal mask on a diagonal chunk.  Register r of block blk holds key
// key0 + 32*blk + 8*(r/4) + 4*half + r%4 for this lane's query row.
// Key kk is masked when kk > row, i.e. when its compile-time part
// 8*(r/4) + r%4 (+32) exceeds the lane's row - key0 - 4*half.
__device__ inline void mask_chunk(f32x16 &s0, f32x16 &s1, int key0, int row, int half) {
    const int lim = row - key0 - 4 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        s0[r] = kr > lim ? -INFINITY : s0[r];
        s1[r] = kr + 32 > lim ? -INFINITY : s1[r];
    }
}

// The running max m is only moved when a chunk's max exceeds it by more than
// kMaxSlack (log2 units): probabilities then stay below 2^kMaxSlack, and since
// l, delta and acc all use the same m the result (acc / l, delta / l) is
// unchanged while most chunks skip the rescale.
constexpr float kMaxSlack = 8.0f;
// Headroom (log2 units) between chunk 0's row max and the fixed reference of
// the bf16 kernel's first attempt: later logits may exceed that max by up to
// kFastHeadroom + 58 before a chunk's mass reaches the 2^64 check; logits more
// than 126 - kFastHeadroom below it underflow, negligible against the row's
// chunk-0 mass (>= 2^-kFastHeadroom).
constexpr float kFastHeadroom = 60.0f;

template <int NACC>
__device__ inline void rescale(f32x16 (&acc)[NACC], float alpha) {
    // skip when no row of the wave moved its max
    if (__ballot(alpha != 1.0f) == 0) return;
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
}

// fp32 kernel (attn_kernel_f32): fp32 MFMA (v_mfma_f32_32x32x2_f32), K and V
// rows staged through registers into row-major LDS tiles (rows padded so the
// operand reads are conflict-free), the same two-stage pipeline and stop
// decision as the bf16 kernel, and the lazy running max throughout.
template <int D, int NW>
struct FCfg {
    static constexpr int BM = 32 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int BN = kTileN;
    static constexpr int KSTR = D + 2;                      // K row stride (floats)
    static constexpr int VSTR = D + 8;                      // V row stride (floats)
    static constexpr int KBUF = BN * KSTR;
    static constexpr int VBUF = BN * VSTR;
    static constexpr int BUF = KBUF + VBUF;                 // floats per stage
    static constexpr size_t LDS_BYTES = 2 * BUF * sizeof(float);
    static constexpr int KCG = D / 4;                       // 16-byte pieces per row
    static constexpr int PIECES = BN * KCG / NT;            // pieces per thread per tile
    static_assert(PIECES >= 1, "tile too small for the thread count");
};

template <int D, int NW, bool S2O>
__global__ __launch_bounds__(64 * NW, 1) void attn_kernel_f32(AttnParams a) {
    using C = FCfg<D, NW>;
    constexpr int BM = C::BM, NT = C::NT, BN = C::BN;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    float *lds = reinterpret_cast<float *>(smem_raw);
    __shared__ int flags[2][NW];

    const Geometry &g = a.g;
    Work wk;
    if (!map_block(g, wk)) return;
    const int b = wk.b, h = wk.h, t = wk.t;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, half = lane >> 5;
    const int row0 = t * BM;
    const int my_row = row0 + 32 * wave + li;

    // schedule: pass-1 chunks are contiguous key tiles starting at base1; pass-2
    // chunks are consecutive BN-entry slices of the tile's list
    const int seg_a = S2O ? (int)seg_start(g, t) : 0;
    const int base1 = seg_a;
    const int n1 = g.causal ? (row0 + BM - base1) / BN : g.N / BN;
    const int n2 = S2O ? seg_a / BN : 0;
    const int total = n1 + n2;
    const int32_t *list = S2O ? a.idx + list_offset(g, b, h, t) : nullptr;

    const int kvh = h / g.G;
    const float *Qp = reinterpret_cast<const float *>(a.q) + ((int64_t)(b * g.Hq + h) * g.N) * D;
    const float *Kp = reinterpret_cast<const float *>(a.k) + ((int64_t)(b * g.Hkv + kvh) * g.N) * D;
    const float *Vp = reinterpret_cast<const float *>(a.v) + ((int64_t)(b * g.Hkv + kvh) * g.N) * D;

    auto chunk_row = [&](int k, int p) -> int {
        if (k < n1) return base1 + k * BN + p;
        return g.blocks ? list[k - n1] * BN + p : list[(k - n1) * BN + p];
    };

    // per-thread staging: piece i of a tile is row (i*NT + tid) / KCG, column
    // group (i*NT + tid) % KCG, for K and V alike
    int prow[C::PIECES], pcg[C::PIECES], rows[C::PIECES];
#pragma unroll
    for (int i = 0; i < C::PIECES; ++i) {
        prow[i] = (i * NT + tid) / C::KCG;
        pcg[i] = (i * NT + tid) % C::KCG;
    }
    u32x4 kreg[C::PIECES], vreg[C::PIECES];
    auto fetch_rows = [&](int k) {
#pragma unroll
        for (int i = 0; i < C::PIECES; ++i) rows[i] = chunk_row(k, prow[i]);
    };
    auto issue_loads = [&]() {
#pragma unroll
        for (int i = 0; i < C::PIECES; ++i) {
            kreg[i] = *reinterpret_cast<const u32x4 *>(Kp + (int64_t)rows[i] * D + pcg[i] * 4);
            vreg[i] = *reinterpret_cast<const u32x4 *>(Vp + (int64_t)rows[i] * D + pcg[i] * 4);
        }
    };
    auto store_lds = [&](int buf) {
        float *Kl = lds + buf * C::BUF;
        float *Vl = Kl + C::KBUF;
#pragma unroll
        for (int i = 0; i < C::PIECES; ++i) {
            float *dst = Kl + prow[i] * C::KSTR + pcg[i] * 4;  // K rows are only 8-byte aligned
            reinterpret_cast<u32x2 *>(dst)[0] = kreg[i].xy;
            reinterpret_cast<u32x2 *>(dst)[1] = kreg[i].zw;
            *reinterpret_cast<u32x4 *>(Vl + prow[i] * C::VSTR + pcg[i] * 4) = vreg[i];
        }
    };

    // Q operand in registers (B operand of S^T = K Q^T)
    float qf[D / 2];
#pragma unroll
    for (int s = 0; s < D / 2; ++s) qf[s] = Qp[(int64_t)my_row * D + 2 * s + half];

    constexpr int NACC = D / 32;
    f32x16 acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = a.scale_log2;

    // S^T of the chunk in stage `buf`: s0/s1 = keys 0..31 / 32..63 of the chunk
    // against this lane's query row
    auto qk = [&](int buf, f32x16 &s0, f32x16 &s1) {
        const float *Kl = lds + buf * C::BUF;
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 2; ++s) {
            float ka = Kl[li * C::KSTR + 2 * s + half];
            float kb = Kl[(32 + li) * C::KSTR + 2 * s + half];
            s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf[s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kb, qf[s], s1, 0, 0, 0);
        }
    };
    // O^T += V^T P^T with the probabilities of the chunk in stage `buf`; register r
    // of block 0 / 1 is key 8*(r/4) + 4*half + r%4 (+32) of the chunk
    auto pv = [&](int buf, const f32x16 &p0, const f32x16 &p1) {
        const float *Vl = lds + buf * C::BUF + C::KBUF;
#pragma unroll
        for (int cb = 0; cb < NACC; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int j = 8 * (r >> 2) + 4 * half + (r & 3);
                float v0 = Vl[j * C::VSTR + 32 * cb + li];
                float v1 = Vl[(32 + j) * C::VSTR + 32 * cb + li];
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v0, p0[r], acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v1, p1[r], acc[cb], 0, 0, 0);
            }
        }
    };

    // Software pipeline.  During iteration k the LDS stages hold chunks k and
    // k+1 and the registers receive chunk k+2; S_{k+1} = K_{k+1} Q^T is computed
    // before the softmax of chunk k, then PV(k) accumulates.  After a stop the
    // speculative S_{k+1} is dropped.
    fetch_rows(0);
    issue_loads();
    store_lds(0);
    if (total > 1) {
        fetch_rows(1);
        issue_loads();
        store_lds(1);
    }
    if (total > 2) fetch_rows(2);
    __syncthreads();
    f32x16 s0, s1;
    qk(0, s0, s1);

    int executed2 = 0;
    for (int k = 0; k < total; ++k) {
        const int buf = k & 1;
        const bool has2 = k + 2 < total;
        if (has2) {
            issue_loads();
            if (k + 3 < total) fetch_rows(k + 3);
        }
        const bool is_p2 = S2O && k >= n1;
        const int key0 = is_p2 ? 0 : base1 + k * BN;
        if (!is_p2 && g.causal && key0 + BN - 1 > row0 + 32 * wave) mask_chunk(s0, s1, key0, my_row, half);

        // row max of chunk k and the (lazy) new running max
        const float mx = pair_max(fmaxf(max16(s0), max16(s1))) * c;
        const float m_new = mx > m + kMaxSlack ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;

        f32x16 sn0, sn1;
        qk(buf ^ 1, sn0, sn1);  // stale stage when k+1 == total; unused then
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -m_new));
            s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -m_new));
        }
        rescale(acc, alpha);
        pv(buf, s0, s1);
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += s0[r] + s1[r];
        const float delta = pair_sum(sum);
        l = l * alpha + delta;
        const bool wave_cont = is_p2 && __ballot(!(delta < a.tau * l)) != 0;

        __syncthreads();  // every wave is done with stage `buf` (K_k was read last iteration)
        if (has2) store_lds(buf);
        if (is_p2 && lane == 0) flags[buf][wave] = wave_cont ? 1 : 0;
        __syncthreads();
        if (is_p2) {
            executed2 = k - n1 + 1;
            int any = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) any |= flags[buf][w];
            if (!any) break;
        }
        s0 = sn0;
        s1 = sn1;
    }

    // epilogue: O = acc / l; lane holds O[my_row][32cb + 8q + 4half + 0..3]
    const float inv = 1.0f / l;
    float *Op = reinterpret_cast<float *>(a.o) + ((int64_t)(b * g.Hq + h) * g.N + my_row) * D;
#pragma unroll
    for (int cb = 0; cb < NACC; ++cb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 o4 = make_float4(acc[cb][4 * q] * inv, acc[cb][4 * q + 1] * inv,
                                    acc[cb][4 * q + 2] * inv, acc[cb][4 * q + 3] * inv);
            *reinterpret_cast<float4 *>(Op + 32 * cb + 8 * q + 4 * half) = o4;
        }
    }
    if (a.exec && tid == 0) a.exec[((int64_t)b * g.Hq + h) * g.T + t] = n1 + executed2;
}

// ---------------------------------------------------------------------------
// bf16 kernel: K/V tiles move global -> LDS directly (global_load_lds_dwordx4,
// one 16-byte row piece per lane, row-gathered through the chunk's indices),
// so no VGPRs stage them and no VALU touches them on the way.  A tile is 64
// rows of D bf16, row-major, its 16-byte pieces XOR-swizzled per row so that
// the MFMA operand reads are free of bank conflicts:
//   K: piece c of row r lives in slot c ^ kswz(r); the QK^T A operand is one
//      16-byte read per lane;
//   V: piece c of key j lives in slot c ^ vswz(j); the PV A operand (V^T) is
//      read with ds_read_b64_tr_b16, which hands each lane four keys of one
//      column: within a group of 16 lanes, lane i supplies the 8-byte read of
//      (key e = i/4, columns 4*(i%4)..+3) and lane j receives column j of the
//      four keys.
// K runs one chunk ahead of V (QK^T of chunk k+1 overlaps the softmax of chunk
// k), with two LDS stages each: iteration k issues K_{k+2} and V_{k+1} into
// the stages freed by the previous iteration, and waits for them only at its
// end, so every load has a whole iteration to land; one barrier per iteration.
template <int D, int NW, bool S2O>
struct BCfg {
    static constexpr int BM = 32 * NW;
    static constexpr int NT = 64 * NW;
    static constexpr int BN = kTileN;
    static constexpr int CPR = D / 8;                  // 16-byte pieces per row
    static constexpr int ROWB = D * 2;                 // bytes per row
    static constexpr int TILEB = BN * ROWB;            // bytes per K or V tile
    static constexpr int INSTR = BN * CPR / 64 / NW;   // piece loads per lane per tile
    static constexpr size_t LDS_BYTES = 4 * TILEB;     // K stage 0/1, V stage 0/1
    static_assert(INSTR >= 1, "tile too small for the thread count");
};

template <int D>
__device__ inline int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int vswz(int j) { return D == 128 ? ((j & 3) << 2) : (((j >> 1) & 1) << 2); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D, int NW, bool S2O>
__global__ __launch_bounds__(64 * NW, 2) void attn_kernel_bf16(AttnParams a) {
    using C = BCfg<D, NW, S2O>;
    constexpr int BM = C::BM, BN = C::BN;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    unsigned char *lds = smem_raw;
    __shared__ int flags[2][NW];
    __shared__ int row_max[NW];
    __shared__ int acc_bad[NW];

    const Geometry &g = a.g;
    Work wk;
    if (!map_block(g, wk)) return;
    const int b = wk.b, h = wk.h, t = wk.t;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 31, half = lane >> 5;
    const int row0 = t * BM;
    const int seg_a = S2O ? (int)seg_start(g, t) : 0;
    const int base1 = seg_a;

    // Rows of this lane and the causal extent of the tile.  In place: the rows
    // row0 + 32*wave + li.  With Q_perm the tile holds the rows at positions
    // row0 .. row0+BM-1 of its segment's order; pass 1 then runs to the tile's
    // last row and the diagonal mask applies from the wave's first row.
    int my_row = row0 + 32 * wave + li;
    int wave_first = row0 + 32 * wave, tile_last = row0 + BM - 1;
    if (S2O && a.qorder) {
        my_row = seg_a + a.qorder[((int64_t)b * g.Hq + h) * g.N + row0 + 32 * wave + li];
        int lo = my_row, hi = my_row;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
            lo = min(lo, __shfl_xor(lo, o));
            hi = max(hi, __shfl_xor(hi, o));
        }
        wave_first = lo;
        if (lane == 0) row_max[wave] = hi;
        __syncthreads();
        tile_last = row_max[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) tile_last = max(tile_last, row_max[w]);
    }
    const int n1 = g.causal ? (tile_last + 1 - base1 + BN - 1) / BN : g.N / BN;
    const int n2 = S2O ? seg_a / BN : 0;
    const int total = n1 + n2;
    const int32_t *list = S2O ? a.idx + list_offset(g, b, h, t) : nullptr;
    // this tile's list as a buffer resource: 32-bit offsets per entry load
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)list, (short)0, S2O ? (int)((g.blocks ? seg_a / BN : seg_a) * 4) : 0, 0x00020000);

    const int kvh = h / g.G;
    const __bf16 *Qp = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)(b * g.Hq + h) * g.N) * D;
    const __bf16 *Kp = reinterpret_cast<const __bf16 *>(a.k) + ((int64_t)(b * g.Hkv + kvh) * g.N) * D;
    const __bf16 *Vp = reinterpret_cast<const __bf16 *>(a.v) + ((int64_t)(b * g.Hkv + kvh) * g.N) * D;

    // slot q = (wave*INSTR + i)*64 + lane of a tile: row q / CPR, slot q % CPR
    auto slot_row = [&](int i) { return ((wave * C::INSTR + i) * 64 + lane) / C::CPR; };
    auto slot_col = [&](int i) { return ((wave * C::INSTR + i) * 64 + lane) % C::CPR; };
    int krows[C::INSTR], vrows[C::INSTR];
    // Key rows this lane moves for chunk k: consecutive keys in pass 1; the
    // chunk's list entries in pass 2 (for block lists, the BN keys of one
    // listed block).  The branch is uniform across the workgroup.
    auto fetch_rows = [&](int k, int (&rows)[C::INSTR]) {
        if (!S2O || k < n1) {
#pragma unroll
            for (int i = 0; i < C::INSTR; ++i) rows[i] = base1 + k * BN + slot_row(i);
        } else if (g.blocks) {
            const int first = list[k - n1] * BN;
#pragma unroll
            for (int i = 0; i < C::INSTR; ++i) rows[i] = first + slot_row(i);
        } else {
            const int first = (k - n1) * BN;
#pragma unroll
            for (int i = 0; i < C::INSTR; ++i)
                rows[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(lrs, (unsigned)((first + slot_row(i)) * 4), 0, 0);
        }
    };
    // K and V of this KV head as buffer resources: 32-bit byte offsets per lane,
    // the LDS destination from a scalar base (the wave index made uniform), and
    // reads past the head's rows return zeros instead of touching other memory
    const int head_bytes = g.N * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kp, (short)0, head_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vp, (short)0, head_bytes, 0x00020000);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto issue_k = [&](int stage, const int (&rows)[C::INSTR]) {
#pragma unroll
        for (int i = 0; i < C::INSTR; ++i) {
            const int r = slot_row(i);
            const int c = slot_col(i) ^ kswz<D>(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krs, (lds_void *)(lds + stage * C::TILEB + (wave_s * C::INSTR + i) * 1024), 16,
                (unsigned)(rows[i] * C::ROWB + c * 16), 0, 0, 0);
        }
    };
    auto issue_v = [&](int stage, const int (&rows)[C::INSTR]) {
#pragma unroll
        for (int i = 0; i < C::INSTR; ++i) {
            const int r = slot_row(i);
            const int c = slot_col(i) ^ vswz<D>(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (lds_void *)(lds + (2 + stage) * C::TILEB + (wave_s * C::INSTR + i) * 1024), 16,
                (unsigned)(rows[i] * C::ROWB + c * 16), 0, 0, 0);
        }
    };

    // Q operand in registers (B operand of S^T = K Q^T)
    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = *reinterpret_cast<const bf16x8 *>(Qp + (int64_t)my_row * D + 16 * s + 8 * half);

    constexpr int NACC = D / 32;
    f32x16 acc[NACC];
    float m, l;
    const float c = a.scale_log2;

    // Per-lane LDS byte offsets of the operand reads.  With the stage a
    // compile-time constant (the loop below is unrolled by two), every read is
    // one of these bases plus an immediate offset, so no VALU computes addresses.
    //   K (A operand of S^T): step st reads 16-byte piece 2*st + half of rows li
    //   and 32 + li; both rows share the swizzle (kswz only looks at r & 15 or
    //   bits 1..3), so the second read is the first plus 32 rows.
    //   V (A operand of O^T, ds_read_b64_tr_b16): for step s and column block cb
    //   the lane reads key 16s + 4 v_h + v_e at column 32cb + 16 v_cg + 4 v_rq,
    //   and the same column of the key 8 further on; the swizzle depends on the
    //   key only through bits 0..1, which s and the +8 leave alone.
    constexpr int STEPS = D / 16;
    int koff[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) koff[st] = li * C::ROWB + (((2 * st + half) ^ kswz<D>(li)) << 4);
    const int gi = lane >> 4, i16 = lane & 15;
    const int v_h = gi >> 1, v_cg = gi & 1, v_e = i16 >> 2, v_rq = i16 & 3;
    int voff[NACC];
#pragma unroll
    for (int cb = 0; cb < NACC; ++cb) {
        const int key1 = 4 * v_h + v_e, col = 32 * cb + 16 * v_cg + 4 * v_rq;
        voff[cb] = key1 * C::ROWB + (((col >> 3) ^ vswz<D>(key1)) << 4) + (col & 7) * 2;
    }

    // S^T of the K tile in `stage` (s0: keys 0..31, s1: keys 32..63), with the
    // exponentials of the previous chunk's probabilities p0/p1 interleaved
    auto qk = [&](auto stage_c, f32x16 &s0, f32x16 &s1, f32x16 &p0, f32x16 &p1, float m_new, bool exps) {
        constexpr int stage = decltype(stage_c)::value;
        const unsigned char *Kt = lds + stage * C::TILEB;
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
        constexpr int EPS = 16 / STEPS;
        bf16x8 ka[2], kb[2];
        ka[0] = *reinterpret_cast<const bf16x8 *>(Kt + koff[0]);
        kb[0] = *reinterpret_cast<const bf16x8 *>(Kt + koff[0] + 32 * C::ROWB);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (st + 1 < STEPS) {
                ka[(st + 1) & 1] = *reinterpret_cast<const bf16x8 *>(Kt + koff[st + 1]);
                kb[(st + 1) & 1] = *reinterpret_cast<const bf16x8 *>(Kt + koff[st + 1] + 32 * C::ROWB);
            }
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1], qf[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[st & 1], qf[st], s1, 0, 0, 0);
            if (exps) {
#pragma unroll
                for (int e = 0; e < EPS; ++e) {
                    const int r = st * EPS + e;
                    p0[r] = __builtin_amdgcn_exp2f(fmaf(p0[r], c, -m_new));
                    p1[r] = __builtin_amdgcn_exp2f(fmaf(p1[r], c, -m_new));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Running max.  First attempt (track = false): the row max is taken on
    // chunk 0 only and the reference m is fixed kFastHeadroom above it, so a
    // chunk costs no max, no rescale test and no rescale; every chunk's mass
    // is checked against 2^64 instead (at most kFastHeadroom + 58 log2 units
    // above chunk 0's max; inf and NaN fail the check too), which keeps l far
    // from overflow, and the accumulators are checked for finiteness at the
    // end.  A failed check restarts the tile with the lazy running max
    // (track = true).  acc / l and delta / l do not depend on m, so
    // both attempts compute the same quantities.
    int executed2 = 0;
    // one attempt over the tile; returns true when it overflowed
    auto attempt = [&](auto track_c) -> bool {
    constexpr bool track = decltype(track_c)::value;
    bool overflow = false;
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    m = -INFINITY;
    l = 0.f;
    executed2 = 0;

    // prologue: K_0, V_0, K_1 into their stages; S_0
    fetch_rows(0, krows);
    issue_k(0, krows);
    issue_v(0, krows);
    if (total > 1) {
        fetch_rows(1, krows);
        issue_k(1, krows);
    }
    if (total > 2) fetch_rows(2, krows);
    if (total > 1) fetch_rows(1, vrows);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa0, sa1, sb0, sb1;
    qk(std::integral_constant<int, 0>{}, sa0, sa1, sb0, sb1, 0.f, false);
    __syncthreads();  // every wave has read K stage 0 before it is refilled

    // One chunk k whose K/V sit in stage kst; s holds S_k, sn receives S_{k+1}.
    // Returns false when the tile stops (or the schedule ends, or the first
    // attempt overflows) after chunk k.
    auto iteration = [&](auto kst_c, int k, f32x16 &s0, f32x16 &s1, f32x16 &sn0, f32x16 &sn1) -> bool {
        constexpr int kst = decltype(kst_c)::value;
        if (k + 2 < total) issue_k(kst, krows);            // K_{k+2} -> stage of K_k
        if (k + 1 < total) issue_v(kst ^ 1, vrows);        // V_{k+1} -> stage of V_{k-1}
        // V_{k+2} moves the rows K_{k+2} just used: keep them instead of reloading
#pragma unroll
        for (int i = 0; i < C::INSTR; ++i) vrows[i] = krows[i];
        if (k + 3 < total) fetch_rows(k + 3, krows);

        // Wave priority (two workgroups per CU, so two waves per SIMD): the
        // gather issue above and the end-of-chunk wait and barrier run at 0,
        // the softmax bookkeeping and the QK^T phase at 1, the PV phase and
        // the stop ballot at 2, so a wave in its PV phase issues ahead of one
        // computing exponentials.  Only the issue order changes.
        __builtin_amdgcn_s_setprio(1);
        const bool is_p2 = S2O && k >= n1;
        const int key0 = is_p2 ? 0 : base1 + k * BN;
        if (!is_p2 && g.causal && key0 + BN - 1 > wave_first) mask_chunk(s0, s1, key0, my_row, half);
        float alpha = 1.f;
        if (track || k == 0) {  // uniform
            const float mx = pair_max(fmaxf(max16(s0), max16(s1))) * c;
            const float m_new = !track ? mx + kFastHeadroom : mx > m + kMaxSlack ? mx : m;
            alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on chunk 0 (m = -inf)
            m = m_new;
            // (before the matrix-core phase: its branch would otherwise split
            // the exponentials from the products they are meant to overlap)
            if (k > 0) rescale(acc, alpha);
        }
        // phase 1: S_{k+1} on the matrix cores with the exponentials of chunk k
        // (stale stage when k+1 == total; the result is unused then)
        qk(std::integral_constant<int, kst ^ 1>{}, sn0, sn1, s0, s1, m, true);

        __builtin_amdgcn_s_setprio(2);
        // phase 2: O^T += V^T P^T for chunk k with the row sum
        float sum;
        {
            const unsigned char *Vt = lds + (2 + kst) * C::TILEB;
            bf16x8 pb[4];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pb[0][e] = (__bf16)s0[e];
                pb[1][e] = (__bf16)s0[8 + e];
                pb[2][e] = (__bf16)s1[e];
                pb[3][e] = (__bf16)s1[8 + e];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int cb = 0; cb < NACC; ++cb) {
                    const unsigned char *va1 = Vt + voff[cb] + 16 * s * C::ROWB;
                    v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)(va1));
                    v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)(va1 + 8 * C::ROWB));
                    bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], acc[cb], 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pair = s0[4 * s + e] + s1[4 * s + e];
                    sum = (s == 0 && e == 0) ? pair : sum + pair;  // no leading + 0
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const float delta = pair_sum(sum);
        l = l * alpha + delta;
        const bool wave_cont = is_p2 && __ballot(!(delta < a.tau * l)) != 0;
        const bool wave_ovf = !track && __ballot(!(delta < 0x1p64f)) != 0;

        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's K_{k+2} / V_{k+1} pieces and indices landed
        if (lane == 0) flags[kst][wave] = (wave_cont ? 1 : 0) | (wave_ovf ? 2 : 0);
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any |= flags[kst][w];
        if (any & 2) {
            overflow = true;
            return false;
        }
        if (is_p2) {
            executed2 = k - n1 + 1;
            if (!(any & 1)) return false;
        }
        return k + 1 < total;
    };
    for (int k = 0;; k += 2) {
        if (!iteration(std::integral_constant<int, 0>{}, k, sa0, sa1, sb0, sb1)) break;
        if (!iteration(std::integral_constant<int, 1>{}, k + 1, sb0, sb1, sa0, sa1)) break;
    }
    if (!track && !overflow) {
        // The mass check bounds every probability by 2^64, but p * V can still
        // overflow acc when |V| is large; an accumulator that is not finite
        // restarts the tile with the running max (probabilities <= 2^kMaxSlack).
        bool bad = false;
#pragma unroll
        for (int i = 0; i < NACC; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) bad |= !(fabsf(acc[i][r]) < INFINITY);
        const bool wave_bad = __ballot(bad) != 0;
        if (lane == 0) acc_bad[wave] = wave_bad ? 1 : 0;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) overflow |= acc_bad[w] != 0;
    }
    return overflow;
    };
    if (attempt(std::false_type{})) attempt(std::true_type{});

    const float inv = 1.0f / l;
    __bf16 *Op = reinterpret_cast<__bf16 *>(a.o) + ((int64_t)(b * g.Hq + h) * g.N + my_row) * D;
#pragma unroll
    for (int cb = 0; cb < NACC; ++cb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[cb][4 * q + e] * inv));
            *reinterpret_cast<u32x2 *>(Op + 32 * cb + 8 * q + 4 * half) = u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
        }
    }
    if (a.exec && tid == 0) a.exec[((int64_t)b * g.Hq + h) * g.T + t] = n1 + executed2;
}

// Raises a kernel's dynamic LDS limit once per process (the first launch of
// each instantiation); later launches read the stored result.
template <typename Kernel>
hipError_t lds_limit_once(Kernel kernel, size_t bytes) {
    static std::once_flag once;
    static hipError_t result = hipSuccess;
    std::call_once(once, [&] {
        result = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    });
    return result;
}

// Grid: B*Hkv*T units rounded up to a multiple of 8 (one per XCD), times G heads.
inline unsigned attention_grid(const Geometry &g) {
    const int64_t units = (int64_t)g.B * g.Hkv * g.T;
    return (unsigned)(((units + 7) / 8) * 8 * g.G);
}

template <int D, int NW, bool S2O>
hipError_t launch_bf16(const AttnParams &p, hipStream_t stream) {
    using C = BCfg<D, NW, S2O>;
    hipError_t e = lds_limit_once(&attn_kernel_bf16<D, NW, S2O>, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_kernel_bf16<D, NW, S2O>), dim3(attention_grid(p.g)), dim3(C::NT), C::LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

template <int D, int NW, bool S2O>
hipError_t launch_f32(const AttnParams &p, hipStream_t stream) {
    using C = FCfg<D, NW>;
    hipError_t e = lds_limit_once(&attn_kernel_f32<D, NW, S2O>, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_kernel_f32<D, NW, S2O>), dim3(attention_grid(p.g)), dim3(C::NT), C::LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_f32_schedule(const AttnParams &p, bool s2o, hipStream_t s) {
    return s2o ? launch_f32<D, NW, true>(p, s) : launch_f32<D, NW, false>(p, s);
}

}  // namespace

hipError_t launch_attention(const Geometry &g, const void *Q, const void *K, const void *V,
                            const int32_t *idx, const int32_t *qorder, float tau, void *O,
                            int32_t *exec_tiles, bool s2o, hipStream_t stream) {
    AttnParams p;
    p.q = Q;
    p.k = K;
    p.v = V;
    p.o = O;
    p.idx = idx;
    p.qorder = qorder;
    p.exec = exec_tiles;
    p.g = g;
    p.scale_log2 = g.scale * 1.4426950408889634f;
    p.tau = tau;
    if (g.dtype == 1) {
        if (g.d == 128)
            return g.BM == 128 ? (s2o ? launch_bf16<128, 4, true>(p, stream) : launch_bf16<128, 4, false>(p, stream))
                               : (s2o ? launch_bf16<128, 2, true>(p, stream) : launch_bf16<128, 2, false>(p, stream));
        return g.BM == 128 ? (s2o ? launch_bf16<64, 4, true>(p, stream) : launch_bf16<64, 4, false>(p, stream))
                           : (s2o ? launch_bf16<64, 2, true>(p, stream) : launch_bf16<64, 2, false>(p, stream));
    }
    if (g.d == 128)
        return g.BM == 128 ? launch_f32_schedule<128, 4>(p, s2o, stream) : launch_f32_schedule<128, 2>(p, s2o, stream);
    return g.BM == 128 ? launch_f32_schedule<64, 4>(p, s2o, stream) : launch_f32_schedule<64, 2>(p, s2o, stream);
}

}  // namespace s2o
