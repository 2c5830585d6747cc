// bwd_bf16.hip -- attention backward pass for bf16 inputs on gfx950.
//
// Given q, k, v, the forward output o, its log-sum-exp lse and the upstream
// gradient do, computes dq, dk, dv of O = softmax(scale * Q K^T [+ mask]) V
// by recomputing the weights tile by tile from lse instead of storing them
// ("Transformer 深度进阶：从矩阵视角到 FlashAttention 工程优化", the
// FlashAttention section: recomputation trades a few FLOPs for memory
// traffic; "Transformer 架构的数学与计算深度解析" sec. 3.3: training needs the
// gradients through the N x N weights).  The gradients are those of the
// definition, by the chain rule (the pages print none):
//
//   p_ij  = exp(scale * q_i.k_j - lse_i)          (the weights, recomputed)
//   D_i   = do_i . o_i  (= sum_j p_ij dp_ij)
//   dp_ij = do_i . v_j
//   ds_ij = p_ij (dp_ij - D_i)
//   dv_j  = sum_i p_ij do_i,  dk_j = scale sum_i ds_ij q_i,  dq_i = scale sum_j ds_ij k_j
//
// Three kernels, no atomics, deterministic:
//   * bwd_pre_kernel: D_i and lse_i * log2(e) for every row (HBM-bound,
//     reads o and do once).
//   * bwd_dq_kernel: each wave owns 32 query rows, and a workgroup's waves
//     all read one K/V head: 4 waves over 128 rows of one query head, or, on
//     causal layers whose rows sit at very different depths, 8 waves over the
//     same 32 (64) query positions of 8 (4) heads of the group, as in the
//     forward.  Q^T and dO^T stay in registers as MFMA B operands while
//     K/V tiles of 64 keys stream through LDS (DMA, double-buffered).  Per
//     32-key half of a tile: S^T = K Q^T and dP^T = V dO^T
//     (v_mfma_f32_32x32x16_bf16), P^T and dS^T on the vector ALUs, then
//     dQ^T += K^T dS^T, where dS^T (bf16) is used straight from the
//     accumulator layout as the B operand and K^T is read from the row-major
//     K tile with ds_read_b64_tr_b16.  Two waves per SIMD (two 4-wave
//     workgroups or one 8-wave workgroup per CU), so one wave's exp / VALU
//     work hides behind another's MFMAs.
//   * bwd_dkdv_kernel: a workgroup of 8 waves owns 128 keys of one K/V head;
//     its K and V rows stay resident in LDS while Q / dO tiles of 64 rows of every
//     query head of the GQA group stream through LDS, so dK and dV are summed
//     over the group in registers (K and V sit in LDS for the whole kernel
//     to leave room for that).  Two waves share each 32-key slice, one
//     per 32-row half of a tile (two waves per SIMD again), and add their
//     partial sums through LDS at the end.  Per half tile: S = Q K^T,
//     dP = dO V^T, P and dS, then dV^T += dO^T P and dK^T += Q^T dS with
//     dO^T, Q^T read transposed from LDS.
// Tiles that are read both row-wise (16 rows x one 16-byte chunk) and
// transposed (4 rows x 4 chunks per 32 lanes) use one XOR swizzle of the
// chunk index that keeps both patterns free of LDS bank conflicts.
// Causal: bottom-right alignment (row i sees keys j <= i + Nk - Nq); tiles no
// row of a wave can see are skipped, and only tiles crossing the diagonal or
// the ends of Q / K take the masked path.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int NTHR = 256;
constexpr int BN = 64;    // dq kernel: keys per tile
constexpr int BKN = 128;  // dkdv kernel: keys per workgroup
constexpr int BQ = 64;    // dkdv kernel: query rows per tile
constexpr int KNW = 8;    // dkdv kernel: waves per workgroup
constexpr float LOG2E = 1.44269504088896340736f;

template <int D>
struct Cfg {
    static constexpr int CH = D / 8;     // 16-byte chunks per row
    static constexpr int KS = D / 16;    // k-steps of a contraction over d
    static constexpr int CB = D / 32;    // 32-column blocks of a [D x 32] result
    static constexpr int RPW = 64 / CH;  // rows one wave-wide 16-byte DMA covers
};

// Chunk swizzles.  swz_rows: tiles read only row-wise -- 16 consecutive rows,
// one chunk each, hit 16 different bank slots.  swz_rt: tiles read row-wise
// AND transposed -- additionally, rows 4a..4a+3 read as 4 adjacent chunks
// (aligned to 4) by 32 lanes hit disjoint groups of 4 slots.
template <int D> __device__ __forceinline__ int swz_rows(int row);
template <> __device__ __forceinline__ int swz_rows<128>(int row) { return row & 15; }
template <> __device__ __forceinline__ int swz_rows<64>(int row) { return (row >> 1) & 7; }
template <int D> __device__ __forceinline__ int swz_rt(int row);
template <> __device__ __forceinline__ int swz_rt<128>(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
template <> __device__ __forceinline__ int swz_rt<64>(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ROWS rows of D bf16 from base[row0 ..] into an LDS tile, row-major with
// the chunk swizzle folded into voff (the lane's byte offset; see the
// kernels).  One wave-wide buffer_load_dwordx4 ... lds fills RPW rows; wave w
// of NW fills rows (NW r + w) * RPW .. in round r.  The descriptor ends at the last
// row of the tensor, so rows past it land as zeros.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(const __bf16 *base, int row0, int nrows, __bf16 *dst, int voff,
                                         int wave_s) {
    using C = Cfg<D>;
    constexpr int ROUNDS = ROWS / (NW * C::RPW);
    constexpr int ROUND_BYTES = NW * C::RPW * D * 2;
    static_assert(ROUNDS * NW * C::RPW == ROWS, "tile split");
    const int left = nrows - row0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(base + (size_t)row0 * D), (short)0, (left < ROWS ? left : ROWS) * D * 2, 0x00020000);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        __bf16 *d = dst + (r * NW + wave_s) * C::RPW * D;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)d, 16, voff, r * ROUND_BYTES, 0, 0);
    }
}

// 64 fp32 values base[row0 ..] into LDS (one dword per lane; past nrows: 0).
__device__ __forceinline__ void dma_row_vals(const float *base, int row0, int nrows, float *dst, int lane) {
    const int left = nrows - row0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(base + row0), (short)0, (left < 64 ? left : 64) * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 4, lane * 4, 0, 0, 0);
}

// Lane constants of the transposing reads (ds_read_b64_tr_b16): a 16-lane
// group reads rows [r0, r0 + 4) x columns [c0, c0 + 16); this lane supplies
// row tr_row, columns tr_col .. + 3, and receives 4 rows of one column.
struct TrLane {
    int row, col;
    __device__ TrLane(int lane) {
        const int grp = lane >> 4, j = lane & 15;
        row = 4 * (grp >> 1) + (j >> 2);
        col = 16 * (grp & 1) + 4 * (j & 3);
    }
};

// Element offsets of the transposing reads of an swz_rt tile: column block
// cb, row base 8 * m (m = 0 .. 7); the swizzle of row tr_row + 8m depends on
// m only through m & 1.
template <int D>
struct TrOffsets {
    int off[2][D / 32];
    __device__ TrOffsets(const TrLane &t) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const int row = t.row + 8 * par;
                const int col = cb * 32 + t.col;
                off[par][cb] = t.row * D + (((col >> 3) ^ swz_rt<D>(row)) * 8) + (col & 7);
            }
        }
    }
};

// A operand [32 columns of the tile (m) x 16 rows (k)] of a transposed
// product: k element i of lane (c, g) is tile row rb + 4g + i for i < 4 and
// rb + 8 + 4g + (i - 4) for i >= 4 (rb = 16 * step), the row order of the
// B operands built from an accumulator (see pack_b).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *tile, const TrOffsets<D> &o, int cb, int step) {
    i16x4 part[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const __bf16 *p = tile + (16 * step + 8 * half) * D + o.off[half][cb];
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand (16 k x 32 n) from the fp32 accumulator x of a 32 x 32 result
// whose rows become k: rows 16 * hh .. + 15, in the order tr_frag reads.
__device__ __forceinline__ bf16x8 pack_b(const f32x16 &x, int hh) {
    u32x4 u;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) u[ii] = pack_bf16(x[8 * hh + 2 * ii], x[8 * hh + 2 * ii + 1]);
    return __builtin_bit_cast(bf16x8, u);
}

// XCD-contiguous remap of the linear block id: the 8 XCDs each take a
// contiguous range of work items, so items that share data share an L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
    const int xcd = L & 7, local = L >> 3;
    const int per = total >> 3, rem = total & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// ---------------------------------------------------------------------------
// D_i = do_i . o_i and lse_i * log2(e) for every row (fp32).
template <int D>
__global__ __launch_bounds__(NTHR) void bwd_pre_kernel(const __bf16 *__restrict__ O,
                                                       const __bf16 *__restrict__ dO, const float *__restrict__ LSE,
                                                       float *__restrict__ Dv, float *__restrict__ L2,
                                                       long long rows) {
    constexpr int LPR = D / 8;  // lanes per row
    const long long t = (long long)blockIdx.x * NTHR + threadIdx.x;
    const long long row = t / LPR;
    const int part = (int)(t % LPR);
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(O + (size_t)row * D + part * 8);
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(dO + (size_t)row * D + part * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows && part == 0) {
        Dv[row] = acc;
        L2[row] = LSE[row] * LOG2E;
    }
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int NW, int HP>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_dq_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ L2, const float *__restrict__ Dv,
    __bf16 *__restrict__ dQ, int Hq, int Hkv, int Nq, int Nk, float sl2, float scale, int n_qtiles, int total)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) __bf16 sK0[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sK1[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV0[BN * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV1[BN * D];

    // work item: (batch, KV head) outermost, then query tile (heaviest causal
    // tile first), then the blocks of HP query heads of the group; the NW
    // waves cover HP heads at BMP query positions
    constexpr int BMP = 32 * (NW / HP);
    // (causal layers with one query head per K/V head: blocks in dispatch
    // order, query tiles heaviest first across all heads, as in the forward)
    const int G = Hq / Hkv;
    const bool flat = CAUSAL && G == 1;
    const int w = flat ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
    const int nhb = G / HP;
    int gqb, tq_ord, hk, b;
    if (flat) {
        const int per_tile = total / n_qtiles;
        tq_ord = w / per_tile;
        const int t = w - tq_ord * per_tile;  // nhb == 1
        gqb = 0;
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
    const int q0 = (CAUSAL ? (n_qtiles - 1 - tq_ord) : tq_ord) * BMP;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, g = lane >> 5;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int h = hk * G + gqb * HP + wave_s % HP;  // this wave's query head
    const int prow = q0 + (wave_s / HP) * 32;       // this wave's first query row
    const int off = Nk - Nq;

    const size_t qrow0 = (size_t)(b * Hq + h) * Nq;
    const __bf16 *Kh = K + (size_t)(b * Hkv + hk) * Nk * D;
    const __bf16 *Vh = V + (size_t)(b * Hkv + hk) * Nk * D;

    // Q^T and dO^T operands of this lane's query row, resident
    const int qi = prow + n;
    bf16x8 qf[C::KS], df[C::KS];
    float lse2 = 0.f, dd = 0.f;
    if (qi < Nq) {
        const bf16x8 *sq = reinterpret_cast<const bf16x8 *>(Q + (qrow0 + qi) * D + 8 * g);
        const bf16x8 *sd = reinterpret_cast<const bf16x8 *>(dO + (qrow0 + qi) * D + 8 * g);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            qf[s] = sq[2 * s];
            df[s] = sd[2 * s];
        }
        lse2 = L2[qrow0 + qi];
        dd = Dv[qrow0 + qi];
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            qf[s] = bf16x8{};
            df[s] = bf16x8{};
        }
    }

    int kv_end = Nk;
    if (CAUSAL) {
        const int last_row = q0 + BMP < Nq ? q0 + BMP : Nq;
        kv_end = last_row + off < Nk ? last_row + off : Nk;
    }
    const int ntiles = (kv_end + BN - 1) / BN;
    const int lim = CAUSAL ? (qi + off < Nk - 1 ? qi + off : Nk - 1) : Nk - 1;  // last visible key
    const int wave_first_row = prow;

    // DMA lane offsets: K is read row-wise and transposed, V row-wise only
    const int ld_row = wave * C::RPW + lane / C::CH, ld_slot = lane % C::CH;
    const int voff_k = (ld_row * D + ((ld_slot ^ swz_rt<D>(ld_row)) * 8)) * 2;
    const int voff_v = (ld_row * D + ((ld_slot ^ swz_rows<D>(ld_row)) * 8)) * 2;
    // row-read offsets: row n (+32 for the second key half), chunk 2s + g
    int k_off[C::KS], v_off[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
        k_off[s] = n * D + (((2 * s + g) ^ swz_rt<D>(n)) * 8);
        v_off[s] = n * D + (((2 * s + g) ^ swz_rows<D>(n)) * 8);
    }
    const TrLane trl(lane);
    const TrOffsets<D> kt_off(trl);

    f32x16 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};

    auto load = [&](int j, __bf16 *k_dst, __bf16 *v_dst) {
        dma_tile<D, BN, NW>(Kh, j * BN, Nk, k_dst, voff_k, wave_s);
        dma_tile<D, BN, NW>(Vh, j * BN, Nk, v_dst, voff_v, wave_s);
    };

    if (ntiles > 0) load(0, sK0, sV0);
    // Tile j reads one stage and refills the other with tile j+1.  The loop
    // below names the stage arrays explicitly (even tiles stage 0, odd tiles
    // stage 1): with a run-time choice the compiler cannot tell the stages
    // apart and waits for the just-issued refill before the tile's reads.
    auto tile = [&](int j, const __bf16 *sk, const __bf16 *sv, __bf16 *nk, __bf16 *nv) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (j + 1 < ntiles) load(j + 1, nk, nv);
        const int j0 = j * BN;
        if (CAUSAL && j0 > wave_first_row + 31 + off) return;  // no row of this wave sees tile j

        // one 32-key half at a time: S^T = K Q^T, dP^T = V dO^T, then P^T and
        // dS^T = P^T (dP^T - D) for this lane's row (lane (n, g) holds keys
        // j0 + 32 kt + 8 (r / 4) + 4 g + r % 4), then dQ^T += K^T dS^T
        const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > wave_first_row + off);
        const int rel = lim - j0 - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x16 st = f32x16{}, dp = f32x16{};
            // the two chains alternate, their operands read AH k-steps ahead
            // (so every MFMA finds its operands in registers: with the
            // chains one after the other the compiler kept a single K
            // operand in flight and each score MFMA waited for its read)
            constexpr int AH = 2;
            bf16x8 kq[C::KS], vq[C::KS];
            auto rk = [&](int s_) { return *reinterpret_cast<const bf16x8 *>(sk + kt * 32 * D + k_off[s_]); };
            auto rv = [&](int s_) { return *reinterpret_cast<const bf16x8 *>(sv + kt * 32 * D + v_off[s_]); };
#pragma unroll
            for (int s = 0; s < AH; ++s) {
                kq[s] = rk(s);
                vq[s] = rv(s);
            }
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                if (s + AH < C::KS) {
                    kq[s + AH] = rk(s + AH);
                    vq[s + AH] = rv(s + AH);
                }
                st = mfma(kq[s], qf[s], st);
                dp = mfma(vq[s], df[s], dp);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(st[r], sl2, -lse2));
                if (need_mask && kt * 32 + 8 * (r >> 2) + (r & 3) > rel) p = 0.f;
                st[r] = p * (dp[r] - dd);
            }
            {
                constexpr int NT = 2 * C::CB, TA = 3;  // K^T operands read TA MFMAs ahead
                bf16x8 tq[NT];
#pragma unroll
                for (int i = 0; i < TA; ++i) tq[i] = tr_frag<D>(sk, kt_off, i % C::CB, 2 * kt + i / C::CB);
                const bf16x8 bs0 = pack_b(st, 0), bs1 = pack_b(st, 1);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    if (i + TA < NT) tq[i + TA] = tr_frag<D>(sk, kt_off, (i + TA) % C::CB, 2 * kt + (i + TA) / C::CB);
                    const int cb = i % C::CB, hh = i / C::CB;
                    acc[cb] = mfma(tq[i], hh ? bs1 : bs0, acc[cb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    for (int j = 0; j < ntiles; j += 2) {
        tile(j, sK0, sV0, sK1, sV1);
        if (j + 1 < ntiles) tile(j + 1, sK1, sV1, sK0, sV0);
    }

    // dQ = scale * acc; lane (n, g) holds columns cb*32 + 8 rr + 4 g + 0..3.
    // The wave writes its 32 rows to LDS (16-byte chunks XOR-swizzled by row)
    // and stores them back as whole rows, 1 KB per wave-wide store, instead
    // of 8-byte pieces over 32 rows.  The K/V tiles are free once every wave
    // has passed the barrier; wave w uses half w & 1 of buffer w / 2.
    {
        constexpr int CHK = D / 8;  // 16-byte chunks per row
        static_assert(NW <= 8 && 64 * D <= BN * D, "four tile buffers hold 32 rows per wave");
        __syncthreads();
        __bf16 *stg = (wave_s < 2 ? sK0 : wave_s < 4 ? sK1 : wave_s < 6 ? sV0 : sV1) + (wave_s & 1) * 32 * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int chunk = cb * 4 + rr;
                const uint32_t lo = pack_bf16(acc[cb][4 * rr + 0] * scale, acc[cb][4 * rr + 1] * scale);
                const uint32_t hi = pack_bf16(acc[cb][4 * rr + 2] * scale, acc[cb][4 * rr + 3] * scale);
                *reinterpret_cast<u32x2 *>(stg + n * D + ((chunk ^ (n & (CHK - 1))) * 8) + 4 * g) = u32x2{lo, hi};
            }
        }
        // a wave's LDS accesses complete in order, so its reads below see its writes
        __bf16 *obase = dQ + (qrow0 + prow) * D;
        constexpr int RPI = 64 / CHK;  // rows per wave-wide store
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int row = i * RPI + lane / CHK, chunk = lane % CHK;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + row * D + ((chunk ^ (row & (CHK - 1))) * 8));
            if (prow + row < Nq) *reinterpret_cast<u32x4 *>(obase + (size_t)row * D + chunk * 8) = val;
        }
    }
}

// ---------------------------------------------------------------------------
// 8 waves: wave w owns keys k0 + 32 (w % 4) .. + 31 and the query rows
// 32 (w / 4) .. + 31 of every tile, so two waves (one per SIMD pair slot)
// accumulate partial dK / dV of the same keys; the partials are summed
// through LDS at the end.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(KNW * 64) void bwd_dkdv_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ L2, const float *__restrict__ Dv,
    __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, int Hq, int Hkv, int Nq, int Nk, float sl2, float scale,
    int n_ktiles, int total)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) __bf16 sQ0[BQ * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sQ1[BQ * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sD0[BQ * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sD1[BQ * D];
    __shared__ __attribute__((aligned(256))) float sL0[BQ];
    __shared__ __attribute__((aligned(256))) float sL1[BQ];
    __shared__ __attribute__((aligned(256))) float sE0[BQ];
    __shared__ __attribute__((aligned(256))) float sE1[BQ];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[BKN * D];  // the workgroup's V rows
    __shared__ __attribute__((aligned(1024))) __bf16 sK[BKN * D];  // the workgroup's K rows

    // work item: (batch, KV head) outermost, then key tile (heaviest causal
    // tile, the first, first)
    // (causal layers with one query head per K/V head: blocks in dispatch
    // order, key tiles heaviest first across all heads)
    const int G = Hq / Hkv;
    const bool flat = CAUSAL && G == 1;
    const int w = flat ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
    const int per_tile = total / n_ktiles;
    const int tk = flat ? w / per_tile : w % n_ktiles;
    const int bh = flat ? w - tk * per_tile : w / n_ktiles;
    const int hk = bh % Hkv, b = bh / Hkv;
    const int k0 = tk * BKN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, g = lane >> 5;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int kw = wave & 3, qh = wave >> 2;  // key slice, query half
    const int off = Nk - Nq;
    const int wk0 = k0 + kw * 32;  // this wave's first key
    const int kj = wk0 + n;        // this lane's key

    // K and V rows in LDS for the whole kernel (registers are the limit at
    // two waves per SIMD)
    const size_t krow0 = (size_t)(b * Hkv + hk) * Nk;

    // query tiles that see some key of the workgroup: rows >= k0 - off
    const int n_qt = (Nq + BQ - 1) / BQ;
    int t_start = 0;
    if (CAUSAL) {
        const int first = k0 - off;
        t_start = first > 0 ? first / BQ : 0;
        if (t_start > n_qt) t_start = n_qt;
    }
    const int nt = n_qt - t_start;
    const int steps = G * nt;

    const int ld_row = wave * C::RPW + lane / C::CH, ld_slot = lane % C::CH;
    const int voff = (ld_row * D + ((ld_slot ^ swz_rt<D>(ld_row)) * 8)) * 2;
    const int voff_v = (ld_row * D + ((ld_slot ^ swz_rows<D>(ld_row)) * 8)) * 2;
    // row reads of this wave's 32 query rows (row 32 qh + n) and of its keys'
    // V rows (row 32 kw + n), chunk 2s + g
    const int rq_base = (qh * 32 + n) * D, rv_base = (kw * 32 + n) * D;
    const int x_rt = g ^ swz_rt<D>(n), x_rows = g ^ swz_rows<D>(n);
    const TrLane trl(lane);
    const TrOffsets<D> t_off(trl);

    f32x16 acck[C::CB], accv[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
        acck[cb] = f32x16{};
        accv[cb] = f32x16{};
    }

    auto qbuf = [&](int u) { return (u & 1) ? sQ1 : sQ0; };
    auto dbuf = [&](int u) { return (u & 1) ? sD1 : sD0; };
    auto lbuf = [&](int u) { return (u & 1) ? sL1 : sL0; };
    auto ebuf = [&](int u) { return (u & 1) ? sE1 : sE0; };
    // Step u covers query tile n_qt - 1 - u / G of query head u % G: every
    // workgroup walks the tiles from the last one down with the heads
    // innermost, so the workgroups of one K/V head, which run together on one
    // XCD, read the same Q / dO tiles at about the same time, through L2
    // (7x less HBM traffic on a 64-head GQA layer at N = 8192 than walking
    // each workgroup's own range from its first tile).
    auto load = [&](int u) {
        const int gq = u % G, qt = n_qt - 1 - u / G;
        const size_t qrow0 = (size_t)(b * Hq + hk * G + gq) * Nq;
        dma_tile<D, BQ, KNW>(Q + qrow0 * D, qt * BQ, Nq, qbuf(u), voff, wave_s);
        dma_tile<D, BQ, KNW>(dO + qrow0 * D, qt * BQ, Nq, dbuf(u), voff, wave_s);
        if (wave_s == 0) {
            dma_row_vals(L2 + qrow0, qt * BQ, Nq, lbuf(u), lane);
            dma_row_vals(Dv + qrow0, qt * BQ, Nq, ebuf(u), lane);
        }
    };

    if (steps > 0) {
        dma_tile<D, BKN, KNW>(V + krow0 * D, k0, Nk, sV, voff_v, wave_s);
        dma_tile<D, BKN, KNW>(K + krow0 * D, k0, Nk, sK, voff_v, wave_s);
        load(0);
    }
    for (int u = 0; u < steps; ++u) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (u + 1 < steps) load(u + 1);
        const int qb = (n_qt - 1 - u / G) * BQ + qh * 32;  // this wave's first query row
        if (qb >= Nq || (CAUSAL && qb + 31 + off < wk0)) continue;  // none of its rows sees these keys
        const __bf16 *sq = qbuf(u), *sd = dbuf(u);
        const float *sl = lbuf(u) + qh * 32, *se = ebuf(u) + qh * 32;

        // S = Q K^T and dP = dO V^T for 32 rows x 32 keys
        // the two chains alternate, their four operands read two k-steps
        // ahead (one chain after the other, each MFMA waited for its own
        // two reads)
        f32x16 sc = f32x16{}, dp = f32x16{};
        {
            constexpr int AH = 2;
            bf16x8 qa[C::KS], ka[C::KS], da[C::KS], va[C::KS];
            auto rd = [&](int s_) {
                qa[s_] = *reinterpret_cast<const bf16x8 *>(sq + rq_base + (((2 * s_) ^ x_rt) * 8));
                ka[s_] = *reinterpret_cast<const bf16x8 *>(sK + rv_base + (((2 * s_) ^ x_rows) * 8));
                da[s_] = *reinterpret_cast<const bf16x8 *>(sd + rq_base + (((2 * s_) ^ x_rt) * 8));
                va[s_] = *reinterpret_cast<const bf16x8 *>(sV + rv_base + (((2 * s_) ^ x_rows) * 8));
            };
#pragma unroll
            for (int s = 0; s < AH; ++s) rd(s);
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                if (s + AH < C::KS) rd(s + AH);
                sc = mfma(qa[s], ka[s], sc);
                dp = mfma(da[s], va[s], dp);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // P and dS: lane (n, g) holds key kj and rows qb + 8 rr + 4 g + i
        const bool need_mask = (qb + 32 > Nq) || (wk0 + 32 > Nk) || (CAUSAL && wk0 + 31 > qb + off);
        u32x4 bp[2];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sl + 8 * rr + 4 * g);
            const f32x4 e4 = *reinterpret_cast<const f32x4 *>(se + 8 * rr + 4 * g);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rr + i;
                p[i] = __builtin_amdgcn_exp2f(fmaf(sc[r], sl2, -l4[i]));
                if (need_mask) {
                    const int qrow = qb + 8 * rr + 4 * g + i;
                    if (qrow >= Nq || kj >= Nk || (CAUSAL && kj > qrow + off)) p[i] = 0.f;
                }
                sc[r] = p[i] * (dp[r] - e4[i]);
            }
            bp[rr >> 1][2 * (rr & 1)] = pack_bf16(p[0], p[1]);
            bp[rr >> 1][2 * (rr & 1) + 1] = pack_bf16(p[2], p[3]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over this wave's 32 rows
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 bpv = __builtin_bit_cast(bf16x8, bp[hh]);
            const bf16x8 bs = pack_b(sc, hh);
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                accv[cb] = mfma(tr_frag<D>(sd, t_off, cb, 2 * qh + hh), bpv, accv[cb]);
                acck[cb] = mfma(tr_frag<D>(sq, t_off, cb, 2 * qh + hh), bs, acck[cb]);
            }
        }
    }

    // sum the two query halves' partials through LDS (the tile buffers are
    // free once every wave has passed the barrier): wave kw + 4 stores, wave
    // kw adds; element i of lane l at red[i * 64 + l]
    float *red = reinterpret_cast<float *>(kw == 0 ? sQ0 : kw == 1 ? sQ1 : kw == 2 ? sD0 : sD1);
    static_assert(C::CB * 16 * 64 * 4 <= BQ * D * 2, "reduction fits a tile buffer");
    __syncthreads();
    if (qh == 1) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(cb * 16 + r) * 64 + lane] = acck[cb][r];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acck[cb][r] += red[(cb * 16 + r) * 64 + lane];
    }
    __syncthreads();
    if (qh == 1) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(cb * 16 + r) * 64 + lane] = accv[cb][r];
    }
    __syncthreads();
    if (qh == 0 && kj < Nk) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) accv[cb][r] += red[(cb * 16 + r) * 64 + lane];
        __bf16 *rk = dK + (krow0 + kj) * D;
        __bf16 *rv = dV + (krow0 + kj) * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int c = cb * 32 + 8 * rr + 4 * g;
                *reinterpret_cast<u32x2 *>(rk + c) =
                    u32x2{pack_bf16(acck[cb][4 * rr + 0] * scale, acck[cb][4 * rr + 1] * scale),
                          pack_bf16(acck[cb][4 * rr + 2] * scale, acck[cb][4 * rr + 3] * scale)};
                *reinterpret_cast<u32x2 *>(rv + c) =
                    u32x2{pack_bf16(accv[cb][4 * rr + 0], accv[cb][4 * rr + 1]),
                          pack_bf16(accv[cb][4 * rr + 2], accv[cb][4 * rr + 3])};
            }
        }
    }
}

template <int D, bool CAUSAL, int NW, int HP>
hipError_t launch_dq_form(const BwdArgs &a, float sl2, long long rows, hipStream_t stream) {
    constexpr int BMP = 32 * (NW / HP);
    const int n_qtiles = (a.Nq + BMP - 1) / BMP;
    const long long total = (long long)a.B * (a.Hq / HP) * n_qtiles;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, NW, HP>), dim3((unsigned)total), dim3(64 * NW), 0, stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                       (const __bf16 *)a.dout, (const float *)(a.ws_d + rows), (const float *)a.ws_d,
                       (__bf16 *)a.dq, a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.scale, n_qtiles, (int)total);
    return hipGetLastError();
}

// The dq kernel's workgroup forms follow the forward's: for causal layers
// whose rows sit at very different depths, 8 waves over the same query
// positions of 8 (or 4) heads that share a K/V head, so that each K/V tile
// staged in LDS serves 256 rows; otherwise 4 waves over 128 rows of one head.
template <int D, bool CAUSAL>
hipError_t launch_dq(const BwdArgs &a, float sl2, long long rows, hipStream_t stream) {
    if constexpr (CAUSAL) {
        int cus = 0;
        const hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        const bool even_rows = (long long)a.Nk - a.Nq >= a.Nq;
        const int G = a.Hq / a.Hkv;
        if (!even_rows && G % 8 == 0 && (long long)a.B * (a.Hq / 8) * ((a.Nq + 31) / 32) >= 2LL * cus)
            return launch_dq_form<D, CAUSAL, 8, 8>(a, sl2, rows, stream);
        if (!even_rows && G % 4 == 0 && (long long)a.B * (a.Hq / 4) * ((a.Nq + 63) / 64) >= 2LL * cus)
            return launch_dq_form<D, CAUSAL, 8, 4>(a, sl2, rows, stream);
    }
    return launch_dq_form<D, CAUSAL, 4, 1>(a, sl2, rows, stream);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs &a, hipStream_t stream) {
    const float sl2 = a.scale * LOG2E;
    const long long rows = (long long)a.B * a.Hq * a.Nq;
    if (rows > 0) {
        const long long threads = rows * (D / 8);
        const long long blocks = (threads + NTHR - 1) / NTHR;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)blocks), dim3(NTHR), 0, stream,
                           (const __bf16 *)a.o, (const __bf16 *)a.dout, a.lse, a.ws_d, a.ws_d + rows, rows);
        const hipError_t e = launch_dq<D, CAUSAL>(a, sl2, rows, stream);
        if (e != hipSuccess) return e;
    }
    const int n_ktiles = (a.Nk + BKN - 1) / BKN;
    const long long total_k = (long long)a.B * a.Hkv * n_ktiles;
    if (total_k > 0) {
        if (total_k > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)total_k), dim3(KNW * 64), 0, stream,
                           (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                           (const __bf16 *)a.dout, (const float *)(a.ws_d + rows), (const float *)a.ws_d,
                           (__bf16 *)a.dk, (__bf16 *)a.dv,
                           a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.scale, n_ktiles, (int)total_k);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
