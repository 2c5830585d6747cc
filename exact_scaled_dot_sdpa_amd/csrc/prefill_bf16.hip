// prefill_bf16.hip -- fused attention forward for bf16 inputs on gfx950.
//
// One kernel computes O = softmax(scale * Q K^T [+ causal mask]) V and the
// per-row log-sum-exp without ever writing the score matrix to device memory
// ("Transformer 架构的数学与计算深度解析", sec. 6: tiles stay on chip; sec. 6.3 and
// "从注意力到 IO 感知执行" sec. 8, eqs. (1)-(2): the running max / denominator /
// un-normalised accumulator recurrence).
//
// gfx950 mapping
//   * A workgroup has NW waves of 32 query rows each, all of one (batch, K/V
//     head), and streams that head's K/V in tiles of BN = 64 keys.  The waves
//     cover HP query heads of the K/V head's group at 32 NW / HP query
//     positions.  Three forms:
//       - NW = 4, HP = 1: 128 rows of one head, two workgroups per CU (the
//         general case);
//       - NW = 8, HP = 1: 256 rows of one head, one workgroup per CU, still two
//         waves per SIMD, when every row sees a similar number of keys
//         (non-causal, or a causal chunk at least as far from the start as it
//         is long): each K/V tile staged in LDS serves twice as many rows;
//       - NW = 8, HP = 8 (or 4): 32 (or 64) query positions of 8 (or 4) heads,
//         for causal GQA layers whose rows sit at very different depths.  Each
//         tile again serves 256 rows, and since the waves share their query
//         positions they share the causal key range, so the triangular work
//         stays as finely balanced as with 32-row tiles.
//     The wide forms are used when the grid still holds two workgroups per
//     CU.  Each row's arithmetic is the same in every form.
//   * Key split, for causal grids of fewer 128-row workgroups than CUs (one
//     short layer): there the rows nearest the end of K set the time, since a
//     wave walks every visible key of its rows.  An 8-wave workgroup then
//     holds SK key groups of NW / SK waves over the same rows (4 x 2 waves
//     and 64 rows for d = 64, 2 x 4 waves and 128 rows for d = 128); group g
//     walks the g-th of SK equal runs of the row tile's key tiles through its
//     own LDS buffers, and at the end the groups' (O^T, reference, l) are
//     merged through LDS by one more step of the online-softmax recurrence.
//     Only the order of the sums differs from the other forms.
//   * K and V tiles go from HBM straight into LDS with global_load_lds_dwordx4
//     (no staging registers, no VALU work), double-buffered so the next tile
//     lands while the current one is computed; one barrier per tile.  Both
//     tiles stay row-major in LDS with the 16-byte chunks of each row XOR-
//     swizzled by a function of the row, which keeps the LDS reads below free
//     of bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (ds_read_b128 from LDS) is the A operand,
//     Q^T (held in registers for the whole kernel) the B operand.  In the fp32
//     result every lane holds ONE query row (lane % 32) and 16 keys per 32-key
//     block, the other 16 keys sitting in lane ^ 32: row max and row sum are
//     in-lane reductions plus (rarely) one exchange with lane ^ 32.
//   * P^T, converted to bf16 in registers (v_cvt_pk_bf16_f32), is directly the
//     B operand of O^T = V^T P^T (again 32x32x16).  Its A operand, V^T, is read
//     from the row-major V tile with ds_read_b64_tr_b16: a 16-lane group reads
//     a 4-key x 16-column block and each lane receives 4 keys of one column,
//     exactly the operand layout.  No transposed copy is ever stored.
//   * Softmax in base 2: p = exp2(s * scale * log2 e - m), one FMA + v_exp_f32.
//     The subtracted reference m is a past running max of the row; it is
//     raised (and O^T, l rescaled) only when a tile's probabilities would
//     exceed 2^24, which leaves u / l unchanged ("从注意力到 IO 感知执行",
//     sec. 8: the subtracted value only changes the representation) and
//     removes the per-tile row max and rescale from the common path.
//   * Causal: tiles beyond the last visible key of the workgroup are never
//     loaded; only tiles that straddle the diagonal (or the end of K) take the
//     masked code path.  Bottom-right alignment: row i sees j <= i + Nk - Nq.
//   * GQA: query head h reads K/V head h / (Hq / Hkv).  Work items are
//     ordered (batch, KV head) outermost, then query tile (heaviest causal
//     tile first), then the G / HP head blocks of the group, and spread over
//     the 8 XCDs in contiguous chunks, so the query heads sharing a K/V head
//     run on one XCD at the same time and read that head's K/V through one
//     L2.  Causal layers with one query head per K/V head have nothing to
//     share that way; there the blocks go out in dispatch order with the
//     query tiles of all heads heaviest first, so that the workgroups that
//     start late or share a CU are the light ones (9-22 % faster on such
//     layers of 1024-4096 rows).
#include "kernels.h"

#include <math.h>

#include <atomic>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BN = 64;   // keys per tile
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
// A tile whose 32 probabilities (per lane) sum above 2^24 triggers the
// rescale of the reference; below it every p <= 2^24, far from fp32 / bf16
// range limits, and fp32 keeps its relative precision.
constexpr float RESCALE_SUM = 16777216.f;

template <int D, int NW>
struct Cfg {
    static constexpr int BM = 32 * NW;              // query rows per workgroup
    static constexpr int NTHR = 64 * NW;            // threads per workgroup
    static constexpr int CH = D / 8;                // 16-byte chunks per row
    static constexpr int KS = D / 16;               // k-steps of the score MFMA
    static constexpr int CB = D / 32;               // 32-column blocks of O^T
    static constexpr int RPW = 64 / CH;             // rows one wave-wide 16-byte load covers
    static constexpr int ROUNDS = BN / (NW * RPW);  // such loads per wave per tile
    static constexpr int TILE = BN * D;             // elements of one K or V tile
    static_assert(ROUNDS * NW * RPW == BN, "tile split");
};

// XOR swizzles of the 16-byte chunk index within a row.
//   K rows are read 16 rows x one chunk at a time (ds_read_b128): 16
//   consecutive rows must land on 16 different 16-byte bank slots.
//   V rows are read 4 rows x 4 adjacent chunks at a time (transposing
//   loads of two 16-lane groups): 4 consecutive rows must land on disjoint
//   groups of 4 bank slots.
template <int D> __device__ __forceinline__ int swz_k(int row);
template <> __device__ __forceinline__ int swz_k<128>(int row) { return row & 15; }
template <> __device__ __forceinline__ int swz_k<64>(int row) { return (row >> 1) & 7; }
template <int D> __device__ __forceinline__ int swz_v(int row);
template <> __device__ __forceinline__ int swz_v<128>(int row) { return (row & 3) << 2; }
template <> __device__ __forceinline__ int swz_v<64>(int row) { return (row & 2) << 1; }

__device__ __forceinline__ float wave_xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

// Round-to-nearest-even pair conversion fp32 -> packed bf16 (lo in bits 0..15),
// a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int D, bool CAUSAL, int NW, int HP, int SK>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_bf16_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
    float sl2, int n_qtiles, int total)
{
    constexpr int NWG = NW / SK;          // waves per key group
    using C = Cfg<D, NWG>;
    constexpr int BMP = 32 * (NWG / HP);  // query positions per workgroup
    // double-buffered K and V tiles, row-major, chunk-swizzled; key group g
    // uses elements [g TILE, (g + 1) TILE) of each
    __shared__ __attribute__((aligned(1024))) __bf16 sK0[SK * C::TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sK1[SK * C::TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sV0[SK * C::TILE];
    __shared__ __attribute__((aligned(1024))) __bf16 sV1[SK * C::TILE];

    // ---- work item: XCD-contiguous remap of the linear block id ----------
    // Causal layers without grouped heads (and the key-split form) take the
    // blocks in dispatch order instead, query tiles heaviest first across
    // every head: the workgroups that start late, or share a CU, are then the
    // light ones.  Their heads share no K/V, which is what the XCD-contiguous
    // order keeps in one L2 for a GQA group.
    const int L = blockIdx.x;
    const int xcd = L & 7, local = L >> 3;
    const int per = total >> 3, rem = total & 7;
    const int G = Hq / Hkv;
    const bool flat = SK > 1 || (CAUSAL && G == 1);
    const int w = flat ? L : xcd * per + (xcd < rem ? xcd : rem) + local;
    const int nhb = G / HP;
    int gqb, tq_ord, hk, b;
    if (flat) {
        const int per_tile = total / n_qtiles;  // (batch, K/V head, head block) items per query tile
        tq_ord = w / per_tile;
        int t = w - tq_ord * per_tile;
        gqb = t % nhb;
        t /= nhb;
        hk = t % Hkv;
        b = t / Hkv;
    } else {
        gqb = w % nhb;
        int t = w / nhb;
        tq_ord = t % n_qtiles;
        t /= n_qtiles;
        hk = t % Hkv;
        b = t / Hkv;
    }
    const int tq = CAUSAL ? (n_qtiles - 1 - tq_ord) : tq_ord;
    const int q0 = tq * BMP;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(wave);
    const int grp = SK > 1 ? wave_all / NWG : 0;       // key group
    const int wave_u = SK > 1 ? wave_all % NWG : wave_all;  // wave within the group
    const int h = hk * G + gqb * HP + wave_u % HP;  // this wave's query head
    const int prow = q0 + (wave_u / HP) * 32;       // this wave's first query row
    const int n = lane & 31, g = lane >> 5;
    const int off = Nk - Nq;  // bottom-right causal offset

    const __bf16 *Qh = Q + ((size_t)(b * Hq + h) * Nq) * D;
    const __bf16 *Kh = K + ((size_t)(b * Hkv + hk) * Nk) * D;
    const __bf16 *Vh = V + ((size_t)(b * Hkv + hk) * Nk) * D;

    // ---- Q^T operands, resident for the whole kernel ---------------------
    const int qi = prow + n;  // this lane's query row
    bf16x8 qf[C::KS];
    if (qi < Nq) {
        const bf16x8 *src = reinterpret_cast<const bf16x8 *>(Qh + (size_t)qi * D + 8 * g);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = bf16x8{};
    }
    // The softmax below works on raw scores with a positive factor sl2: a
    // negative scale is applied by negating Q (exact in bf16), and a zero
    // scale becomes 1e-30, for which exp2 of every visible score is exactly
    // 1 (all weights equal, as with scale 0) while masked scores stay -inf.
    if (sl2 < 0.f) {
        sl2 = -sl2;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            u32x4 x = __builtin_bit_cast(u32x4, qf[s]);
            x ^= 0x80008000u;
            qf[s] = __builtin_bit_cast(bf16x8, x);
        }
    }
    sl2 = sl2 < 1e-30f ? 1e-30f : sl2;

    // ---- key range --------------------------------------------------------
    int kv_end = Nk;
    if (CAUSAL) {
        const int last_row = (q0 + BMP < Nq ? q0 + BMP : Nq);  // exclusive
        const int e = last_row + off;                        // keys < e are visible to some row
        kv_end = e < Nk ? e : Nk;
    }
    const int ntiles = (kv_end + BN - 1) / BN;
    // key group grp walks tiles [tb, tb + cnt); all groups step through nit
    // iterations together (a group with fewer tiles idles in the last one)
    int tb = 0, cnt = ntiles, nit = ntiles;
    if constexpr (SK > 1) {
        tb = ntiles * grp / SK;
        cnt = ntiles * (grp + 1) / SK - tb;
        nit = (ntiles + SK - 1) / SK;
    }

    // per-lane limit of visible keys (inclusive)
    const int lim = CAUSAL ? ((qi + off) < (Nk - 1) ? (qi + off) : (Nk - 1)) : (Nk - 1);
    const int wave_first_row = prow;

    // ---- HBM -> LDS tile loads -------------------------------------------
    // One wave-wide buffer_load_dwordx4 ... lds fills RPW consecutive rows
    // (1 KB): lane l lands at byte 16*l, i.e. row l / CH, chunk slot l % CH,
    // and fetches the chunk the swizzle puts in that slot.  Wave w fills rows
    // (NW r + w) * RPW .. + RPW - 1 in round r.  The buffer
    // descriptor of each tile starts at the tile's first row and ends at the
    // last row of K/V, so rows past the end read as zeros (hardware range
    // check); no per-lane address arithmetic is left in the loop.
    // The chunk swizzles of a loaded row do not depend on the round, so one
    // lane offset per tensor serves every round; rounds step by a scalar
    // offset (which the range check includes: out-of-range lanes write 0).
    const int wave_s = wave_u;
    const int ld_row = (SK > 1 ? wave_u : wave) * C::RPW + lane / C::CH, ld_slot = lane % C::CH;
    const int ld_voff_k = (ld_row * D + ((ld_slot ^ swz_k<D>(ld_row)) * 8)) * 2;
    const int ld_voff_v = (ld_row * D + ((ld_slot ^ swz_v<D>(ld_row)) * 8)) * 2;
    constexpr int ROUND_BYTES = NWG * C::RPW * D * 2;
    auto dma_rows = [&](const __bf16 *base, int j0, __bf16 *dst, int voff) {
        const int rows_left = Nk - j0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(base + (size_t)j0 * D), (short)0, (rows_left < BN ? rows_left : BN) * D * 2, 0x00020000);
#pragma unroll
        for (int r = 0; r < C::ROUNDS; ++r) {
            __bf16 *d = dst + (r * NWG + wave_s) * C::RPW * D;  // wave-uniform LDS destination
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)d, 16, voff, r * ROUND_BYTES, 0, 0);
        }
    };

    // ---- running state ----------------------------------------------------
    // m_ref: the reference subtracted before exp2, in units of
    // t = s * scale * log2(e): a past running max of the row, raised (with O^T
    // and l rescaled) only when a tile's probabilities would outgrow it.
    f32x16 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
    float m_ref = -INFINITY;
    float l_run = 0.f;  // this lane's share of the denominator

    // lane constants of the transposing V reads: a 16-lane group reads keys
    // [key0, key0 + 4) x columns [col0, col0 + 16); this lane's 8 bytes are key
    // key0 + tr_key, columns col0 + tr_col .. + 3.
    const int tr_grp = lane >> 4, tr_j = lane & 15;
    const int tr_key = 4 * (tr_grp >> 1) + (tr_j >> 2);
    const int tr_col = 16 * (tr_grp & 1) + 4 * (tr_j & 3);

    // Lane offsets (elements) of the LDS operand reads, fixed for the whole
    // kernel; everything else in a read address is a compile-time constant.
    //   K: row n (+32 for the second key half; the swizzle of row n + 32 is
    //      that of row n), chunk (2s + g) ^ swz.
    int k_off[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) k_off[s] = n * D + (((2 * s + g) ^ swz_k<D>(n)) * 8);
    //   V (transposing reads): key tr_key (+ 8*half + 16*hh + 32*kt, which
    //      keeps key & 3), column block cb -> chunk ((cb ^ (swz >> 2)) << 2)
    //      | (tr_col >> 3) when D = 128; the D = 64 swizzle is handled alike.
    int v_off[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
        const int col = cb * 32 + tr_col;
        v_off[cb] = tr_key * D + (((col >> 3) ^ swz_v<D>(tr_key)) * 8) + (col & 7);
    }

    // K operand of score MFMA number i (i = 0..2*KS-1) of a tile; MFMAs
    // alternate between the two 32-key halves (kt = i & 1, k-step i >> 1) so
    // that consecutive MFMAs accumulate into different registers.
    auto kfrag = [&](const __bf16 *sk, int i) {
        const int kt = i & 1, s = i >> 1;
        return *reinterpret_cast<const bf16x8 *>(sk + kt * 32 * D + k_off[s]);
    };
    // V^T operand of PV MFMA (cb, kt, hh) from two transposing LDS reads:
    // operand element i of lane (c, g) is key 16*hh + 32*kt + 4*g + i for
    // i < 4 and + 8 + 4*g + (i - 4) for i >= 4, matching the keys of P^T.
    auto vfrag = [&](const __bf16 *sv, int cb, int kt, int hh) {
        i16x4 part[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const __bf16 *p = sv + (kt * 32 + 16 * hh + 8 * half) * D + v_off[cb];
            part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // Plain S^T = K Q^T of one tile (prologue only).
    auto qk = [&](const __bf16 *sk, f32x16 (&st)[2]) {
        st[0] = f32x16{};
        st[1] = f32x16{};
#pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i)
            st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(sk, i), qf[i >> 1], st[i & 1], 0, 0, 0);
    };

    // Software pipeline over key tiles j = 0 .. ntiles-1.  K and V have their
    // own double-buffer rings; tile j's K sits in sK[j & 1], its V in
    // sV[j & 1].  Iteration j feeds the MFMA units the scores of tile j+1
    // while the vector ALUs turn the scores of tile j into P (the two streams
    // are interleaved instruction by instruction below), then multiplies P by
    // V of tile j.  Loads run ahead: iteration j starts K[j+2] and V[j+1]
    // into the buffers iteration j-1 finished with.
    // j counts the group's own tiles; its tile j is key tile tb + j
    const int goff = SK > 1 ? grp * C::TILE : 0;
    auto kbuf = [&](int j) { return ((j & 1) ? sK1 : sK0) + goff; };
    auto vbuf = [&](int j) { return ((j & 1) ? sV1 : sV0) + goff; };
    auto dma_k = [&](int j) { dma_rows(Kh, (tb + j) * BN, kbuf(j), ld_voff_k); };
    auto dma_v = [&](int j) { dma_rows(Vh, (tb + j) * BN, vbuf(j), ld_voff_v); };

    // One pipeline iteration; cur holds S^T of tile j, nxt receives tile j+1.
    // Returns false when this wave is done (its rows see no later key).
    auto iteration = [&](const int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        const int j0 = (tb + j) * BN;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K[j+1] and V[j] have landed
        __syncthreads();                                   // ... for every wave; K[j], V[j-1] are free
        if constexpr (SK > 1) {
            if (j >= cnt) return;  // this group's tiles are done
        }
        if (j + 2 < cnt) dma_k(j + 2);
        if (j + 1 < cnt) dma_v(j + 1);
        // waves whose rows see none of tile j skip it (and every later tile)
        if (CAUSAL && j0 > wave_first_row + 31 + off) return;

        // mask (diagonal and end-of-K tiles only): raw score -> -inf
        const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > wave_first_row + off);
        if (need_mask) {
            const int rel = lim - j0 - 4 * g;  // key offset limit inside the tile for this lane
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = kt * 32 + 8 * (r >> 2) + (r & 3);
                    if (kk > rel) cur[kt][r] = -INFINITY;
                }
            }
        }
        // Scores of tile j+1 on the MFMA units, interleaved with P^T of tile j
        // on the vector ALUs (bf16, round to nearest even; the denominator
        // sums the unrounded fp32 values so LSE carries no bf16 rounding).
        // P uses the current reference m_ref, a past running max; only when
        // some p would exceed 2^24 (the tile's exp sum tells) is the reference
        // raised to the running max, O^T and l rescaled and P recomputed.  The
        // first tile always takes that path.  Masked scores are -inf (p = 0).
        // The last iteration computes a discarded product of a stale buffer.
        const __bf16 *skn = kbuf(j + 1);
        constexpr int NQK = 2 * C::KS;       // score MFMAs per tile (8 or 16)
        constexpr int PAIRS_PER = 16 / NQK;  // softmax pairs per score MFMA
        constexpr int KAHEAD = 4;            // K operands in flight
        u32x4 pb[2][2];
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
        const bool fresh = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
        const float m_use = fresh ? 0.f : m_ref;
        bf16x8 kq[NQK];
#pragma unroll
        for (int i = 0; i < KAHEAD; ++i) kq[i] = kfrag(skn, i);
        nxt[0] = f32x16{};
        nxt[1] = f32x16{};
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            if (i + KAHEAD < NQK) kq[i + KAHEAD] = kfrag(skn, i + KAHEAD);
            nxt[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[i], qf[i >> 1], nxt[i & 1], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < PAIRS_PER; ++q) {
                const int pi = i * PAIRS_PER + q;  // pair index 0..15
                const int kt = pi >> 3, hh = (pi >> 2) & 1, ii = pi & 3;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii], sl2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii + 1], sl2, -m_use));
                pb[kt][hh][ii] = pack_bf16(p0, p1);
                ps[ii] += p0 + p1;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        if (fresh || __builtin_amdgcn_ballot_w64(!(psum <= RESCALE_SUM)) != 0) {  // rare
            float mr = cur[0][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = (kt == 0 ? 1 : 0); r < 16; ++r) mr = fmaxf(mr, cur[kt][r]);
            }
            const float mloc = mr * sl2;
            const float mp = fmaxf(mloc, wave_xor32(mloc));
            const float m_new = fmaxf(m_ref, mp);
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
            m_ref = m_new;
            const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
            psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii], sl2, -mu));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii + 1], sl2, -mu));
                        pb[kt][hh][ii] = pack_bf16(p0, p1);
                        psum += p0 + p1;
                    }
                }
            }
        }
        l_run += psum;

        // O^T += V^T P^T for tile j; cb innermost so consecutive MFMAs are
        // independent; operands read two MFMAs ahead
        const __bf16 *svc = vbuf(j);
        constexpr int NPV = 4 * C::CB;   // PV MFMAs per tile (8 or 16)
        constexpr int VAHEAD = 4;        // V operands in flight
        bf16x8 vq[NPV];
#pragma unroll
        for (int i = 0; i < VAHEAD; ++i) vq[i] = vfrag(svc, i % C::CB, (i / C::CB) >> 1, (i / C::CB) & 1);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int cb = i % C::CB, kh = i / C::CB, kt = kh >> 1, hh = kh & 1;
            if (i + VAHEAD < NPV) {
                const int i2 = i + VAHEAD;
                const int kh2 = i2 / C::CB;
                vq[i2] = vfrag(svc, i2 % C::CB, kh2 >> 1, kh2 & 1);
            }
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[i], __builtin_bit_cast(bf16x8, pb[kt][hh]), acc[cb],
                                                              0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    f32x16 stA[2], stB[2];
    if (nit > 0) {
        if (cnt > 0) {
            dma_k(0);
            dma_v(0);
            if (cnt > 1) dma_k(1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (cnt > 0) qk(kbuf(0), stA);
    }
    for (int j = 0; j < nit; j += 2) {
        iteration(j, stA, stB);
        if (j + 1 < nit) iteration(j + 1, stB, stA);
    }

    // ---- key groups: merge the partial states through LDS -----------------
    // Group g > 0 leaves (O^T, m_ref, l) of each lane in LDS; group 0 folds
    // them in: with m = max(m_0, m_g), O^T and l of each side are scaled by
    // 2^(m_side - m) and added (one more step of the online-softmax
    // recurrence, applied to two key ranges).  Lanes keep their layout, so
    // the merge is element-wise.
    __bf16 *stage_sk = nullptr;  // key-split form: LDS this wave may reuse for its output rows
    if constexpr (SK > 1) {
        constexpr int NE = 16 * C::CB + 2;             // floats per lane
        constexpr int ARR_F = SK * C::TILE / 2;         // floats per LDS array
        constexpr int BPA = ARR_F / (NE * 64);          // per-wave blocks per array
        static_assert(BPA * 4 >= (SK - 1) * NWG, "merge staging space");
        auto blk = [&](int bi) -> float * {
            const int ai = bi / BPA;
            float *base = ai == 0 ? (float *)sK0 : ai == 1 ? (float *)sK1 : ai == 2 ? (float *)sV0 : (float *)sV1;
            return base + (bi % BPA) * NE * 64 + lane;
        };
        __syncthreads();  // every group is done with its tiles
        if (grp > 0) {
            float *st = blk((grp - 1) * NWG + wave_u);
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[(16 * cb + r) * 64] = acc[cb][r];
            }
            st[16 * C::CB * 64] = m_ref;
            st[(16 * C::CB + 1) * 64] = l_run;
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll 1
        for (int g2 = 1; g2 < SK; ++g2) {
            const float *st = blk((g2 - 1) * NWG + wave_u);
            const float mg = st[16 * C::CB * 64], lg = st[(16 * C::CB + 1) * 64];
            const float mn = fmaxf(m_ref, mg);
            const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mn);
            const float ag = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - mn);
            l_run = l_run * a0 + lg * ag;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][r] = acc[cb][r] * a0 + st[(16 * cb + r) * 64] * ag;
            }
            m_ref = mn;
        }
        // only this wave reads its own staging blocks, so once its merge is
        // done the first of them can hold its output rows
        static_assert(NE * 64 * 4 >= 32 * D * 2, "a staging block holds 32 output rows");
        stage_sk = reinterpret_cast<__bf16 *>(blk(wave_u) - lane);
    }

    // ---- epilogue: O = u / l, LSE = ln(sum exp(s)) -----------------------
    const float l_tot = l_run + wave_xor32(l_run);
    {
        // Each lane holds 4-column pieces of its row, which would go out as
        // 8-byte stores scattered over 32 rows.  Instead the wave writes its
        // 32 rows to LDS (row-major, 16-byte chunks XOR-swizzled by row so the
        // writes spread over the banks) and stores them back as whole rows:
        // every wave-wide store covers 64 / CHK consecutive rows, 1 KB
        // contiguous.  The K/V tiles are free once every wave has passed the
        // barrier; wave w uses half w & 1 of buffer w / 2 (32 rows x D each).
        // The key-split form reuses the wave's own merge staging block.
        constexpr int CHK = D / 8;  // 16-byte chunks per row
        static_assert(NW <= 8 && 64 * D <= C::TILE, "four tile buffers hold 32 rows per wave");
        __bf16 *stg;
        if constexpr (SK > 1) {
            stg = stage_sk;
        } else {
            __syncthreads();
            stg = (wave_all < 2 ? sK0 : wave_all < 4 ? sK1 : wave_all < 6 ? sV0 : sV1) + (wave_all & 1) * 32 * D;
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int chunk = cb * 4 + rr;  // columns 8 chunk .. + 7; this lane's half is 4 g .. + 3
                const uint32_t lo = pack_bf16(acc[cb][4 * rr + 0] * inv, acc[cb][4 * rr + 1] * inv);
                const uint32_t hi = pack_bf16(acc[cb][4 * rr + 2] * inv, acc[cb][4 * rr + 3] * inv);
                *reinterpret_cast<u32x2 *>(stg + n * D + ((chunk ^ (n & (CHK - 1))) * 8) + 4 * g) = u32x2{lo, hi};
            }
        }
        // a wave's LDS accesses complete in order, so its reads below see its writes
        __bf16 *obase = O + ((size_t)(b * Hq + h) * Nq + prow) * D;
        constexpr int RPI = 64 / CHK;  // rows per wave-wide store
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int row = i * RPI + lane / CHK, chunk = lane % CHK;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + row * D + ((chunk ^ (row & (CHK - 1))) * 8));
            if (prow + row < Nq) *reinterpret_cast<u32x4 *>(obase + (size_t)row * D + chunk * 8) = val;
        }
        if (qi < Nq && LSE && g == 0)
            LSE[(size_t)(b * Hq + h) * Nq + qi] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * LN2 : -INFINITY;
    }
}

template <int D, bool CAUSAL, int NW, int HP, int SK = 1>
hipError_t launch_nw(const FwdArgs &a, hipStream_t stream) {
    constexpr int BMP = 32 * (NW / SK / HP);
    const float sl2 = a.scale * LOG2E;
    const int n_qtiles = (a.Nq + BMP - 1) / BMP;
    const long long total = (long long)a.B * (a.Hq / HP) * n_qtiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, NW, HP, SK>), dim3((unsigned)total), dim3(64 * NW), 0, stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (__bf16 *)a.o,
                       a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, sl2, n_qtiles, (int)total);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    int cus = 0;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const long long two_per_cu = 2LL * cus;
    // causal grid of fewer 128-row workgroups than CUs: the deepest rows
    // set the time, so their keys are split over the key groups of one
    // 8-wave workgroup (64 rows x 4 groups for d = 64, 128 rows x 2 groups
    // for d = 128, which needs twice the LDS per group)
    if (CAUSAL && (long long)a.B * a.Hq * ((a.Nq + 127) / 128) < cus) {
        if constexpr (D == 64) return launch_nw<D, CAUSAL, 8, 1, 4>(a, stream);
        else return launch_nw<D, CAUSAL, 8, 1, 2>(a, stream);
    }
    // 8-wave workgroups of 256 rows of one head when the rows see similar
    // numbers of keys and the grid still holds at least two of them per CU
    const bool even_rows = !CAUSAL || (long long)a.Nk - a.Nq >= a.Nq;
    if (even_rows) {
        const long long wide = (long long)a.B * a.Hq * ((a.Nq + 255) / 256);
        if (wide >= two_per_cu) return launch_nw<D, CAUSAL, 8, 1>(a, stream);
    }
    if constexpr (CAUSAL) {
        // rows at different depths: 8-wave workgroups over the same 32 (64)
        // query positions of 8 (4) heads that share a K/V head
        const int G = a.Hq / a.Hkv;
        if (!even_rows && G % 8 == 0 && (long long)a.B * (a.Hq / 8) * ((a.Nq + 31) / 32) >= two_per_cu)
            return launch_nw<D, CAUSAL, 8, 8>(a, stream);
        if (!even_rows && G % 4 == 0 && (long long)a.B * (a.Hq / 4) * ((a.Nq + 63) / 64) >= two_per_cu)
            return launch_nw<D, CAUSAL, 8, 4>(a, stream);
    }
    return launch_nw<D, CAUSAL, 4, 1>(a, stream);
}

}  // namespace

// Compute units of the current device, queried once per device.
hipError_t device_cu_count(int *out) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus = cus > 0 ? cus : 1;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    *out = cus;
    return hipSuccess;
}

hipError_t launch_prefill_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
