// prefill_fp8.hip -- fused attention forward for fp8 (OCP e4m3) q, k, v on
// gfx950, bf16 output.
//
// The same computation as the bf16 kernel (one fused pass, online softmax,
// the score matrix never leaves the chip: "Transformer 架构的数学与计算深度
// 解析" sec. 6, "从注意力到 IO 感知执行" sec. 8 eqs. (1)-(2)), with inputs
// stored as fp8 as FlashAttention-3 does on Hopper (pwwt.cn engineering
// blog, sec. 4.4).  The same blog (sec. 7.2) warns that fp8 is sensitive to
// quantisation: scores that lose precision before the softmax shift the
// attention distribution.  This kernel therefore quantises nothing itself:
//   * S^T = K Q^T runs on v_mfma_f32_32x32x64_f8f6f4.  The products of two
//     e4m3 values are exact, but the instruction's internal sum keeps fewer
//     bits than fp32: on gfx950 the 64-term dot products carry an absolute
//     error of up to about 2^-16 of the largest result (measured), against
//     2^-24 for the bf16 kernel's fp32 sums.  At scale 1/sqrt(d) that moves a
//     scaled score by ~1e-4, well inside the bf16 tolerances; the error grows
//     with |scale * score|, which is the sensitivity the blog warns about.
//   * P^T stays bf16 (as in the bf16 kernel) and O^T = V^T P^T runs on the
//     bf16 MFMA.  V stays fp8 in LDS: each operand is read with the 8-bit
//     transposing load (ds_read_b64_tr_b8, 8 keys of one column per lane)
//     and widened exactly in registers (every e4m3 value is a bf16 value;
//     v_cvt_scalef32_pk_bf16_fp8, 4 per operand).  A first design converted
//     each V tile once into a bf16 LDS tile; its LDS reads and writes cost
//     about 14 % of the kernel, and widening per operand, inside the P V
//     MFMA stream where the vector ALUs are otherwise idle, is 2.6 % faster
//     than that design overall.
// The caller folds the dequantisation factors of q and k into `scale`; the
// factor of v multiplies the output (`v_scale`, applied in fp32 before the
// final rounding).
//
// gfx950 mapping (as the bf16 kernel unless stated):
//   * 4 waves x 32 query rows, BN = 64 keys per tile, two workgroups per CU.
//   * Q^T (fp8, 32 bytes per lane per 64-wide k-step) stays in registers.
//   * K tiles: fp8 rows of d bytes, HBM -> LDS by DMA two tiles ahead; the
//     16-byte chunks are XOR-swizzled by the row so that the operand reads
//     (32 rows x one chunk) are conflict-free.
//   * V tiles: fp8 rows, HBM -> LDS by DMA one tile ahead, their 32-byte
//     bands XOR-swizzled by the row so that the transposing reads (16 rows x
//     one band) are conflict-free.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHR = 256;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float RESCALE_SUM = 16777216.f;  // see the bf16 kernel
constexpr int E8M0_ONE = 127;              // unit block scale of the f8f6f4 MFMA

template <int D>
struct Cfg {
    static constexpr int CH8 = D / 16;            // 16-byte chunks of an fp8 row
    static constexpr int KS8 = D / 64;            // k-steps of the fp8 score MFMA
    static constexpr int CB = D / 32;             // 32-column blocks of O^T
    static constexpr int RPW8 = 64 / CH8;         // fp8 rows one wave-wide DMA covers
    static constexpr int ROUNDS8 = BN / (4 * RPW8);
    static constexpr int TILE8 = BN * D;          // bytes of an fp8 tile
    static_assert(ROUNDS8 * 4 * RPW8 == BN, "tile split");
};

// Chunk swizzle of an fp8 K row (d bytes): 16 consecutive rows reading one
// chunk hit 16 different 16-byte bank slots (rows of 128 B pair up in a
// 256-byte bank line at d = 128, rows of 64 B group by four at d = 64).
template <int D> __device__ __forceinline__ int swz8(int row);
template <> __device__ __forceinline__ int swz8<128>(int row) { return (row >> 1) & 7; }
template <> __device__ __forceinline__ int swz8<64>(int row) { return (row >> 2) & 3; }
// Chunk swizzle of the fp8 V tile: XOR on bits 1-2 of the 16-byte chunk index
// (the 32-byte band), so that a transposing read of 16 consecutive rows x one
// 32-byte band touches every bank once per 256 bytes (rows of 128 B: bits 1-2
// of the row; rows of 64 B: bit 2).
template <int D> __device__ __forceinline__ int swzw(int row);
template <> __device__ __forceinline__ int swzw<128>(int row) { return ((row >> 1) & 3) << 1; }
template <> __device__ __forceinline__ int swzw<64>(int row) { return ((row >> 2) & 1) << 1; }

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0, E8M0_ONE);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHR, 2) void prefill_fp8_kernel(
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float sl2, float v_scale,
    int n_qtiles, int total)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[C::TILE8];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[C::TILE8];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[C::TILE8];  // fp8 V tiles
    __shared__ __attribute__((aligned(1024))) uint8_t sW1[C::TILE8];

    // ---- work item (same order and XCD remap as the bf16 kernel) ----------
    const int L = blockIdx.x;
    const int xcd = L & 7, local = L >> 3;
    const int per = total >> 3, rem = total & 7;
    const int w = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int G = Hq / Hkv;
    const int gq = w % G;
    int t = w / G;
    const int tq_ord = t % n_qtiles;
    t /= n_qtiles;
    const int hk = t % Hkv;
    const int b = t / Hkv;
    const int h = hk * G + gq;
    const int tq = CAUSAL ? (n_qtiles - 1 - tq_ord) : tq_ord;
    const int q0 = tq * BM;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, g = lane >> 5;
    const int off = Nk - Nq;

    const uint8_t *Qh = Q + ((size_t)(b * Hq + h) * Nq) * D;
    const uint8_t *Kh = K + ((size_t)(b * Hkv + hk) * Nk) * D;
    const uint8_t *Vh = V + ((size_t)(b * Hkv + hk) * Nk) * D;

    // ---- Q^T operands: lane (n, g) holds d = 64 s + 32 g .. + 31 of row qi
    const int qi = q0 + wave * 32 + n;
    i32x8 qf[C::KS8];
    if (qi < Nq) {
        const i32x8 *src = reinterpret_cast<const i32x8 *>(Qh + (size_t)qi * D + 32 * g);
#pragma unroll
        for (int s = 0; s < C::KS8; ++s) qf[s] = src[2 * s];
    } else {
#pragma unroll
        for (int s = 0; s < C::KS8; ++s) qf[s] = i32x8{};
    }
    // positive factor only (see the bf16 kernel): a negative scale negates Q
    // (the e4m3 sign bit), zero becomes 1e-30
    if (sl2 < 0.f) {
        sl2 = -sl2;
#pragma unroll
        for (int s = 0; s < C::KS8; ++s) qf[s] ^= (int)0x80808080;
    }
    sl2 = sl2 < 1e-30f ? 1e-30f : sl2;

    int kv_end = Nk;
    if (CAUSAL) {
        const int last_row = (q0 + BM < Nq ? q0 + BM : Nq);
        const int e = last_row + off;
        kv_end = e < Nk ? e : Nk;
    }
    const int ntiles = (kv_end + BN - 1) / BN;
    const int lim = CAUSAL ? ((qi + off) < (Nk - 1) ? (qi + off) : (Nk - 1)) : (Nk - 1);
    const int wave_first_row = q0 + wave * 32;

    // ---- DMA lane offsets ----------------------------------------------------
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int ld_row = wave * C::RPW8 + lane / C::CH8, ld_slot = lane % C::CH8;
    const int voff_k = ld_row * D + ((ld_slot ^ swz8<D>(ld_row)) * 16);
    const int voff_w = ld_row * D + ((ld_slot ^ swzw<D>(ld_row)) * 16);
    // BN fp8 rows base[row0 ..] into an LDS tile; rows past Nk read as 0
    // (the descriptor ends at the last row)
    // (the round stride is a named constant: this host compiler drops the
    // kernel's host stub when the DMA builtin's soffset is written out as a
    // product of template-dependent members inside the lambda)
    constexpr int ROUND8 = 4 * C::RPW8 * D;
    auto dma_rows8 = [&](const uint8_t *base, int row0, uint8_t *dst, int voff) {
        const int left = Nk - row0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(base + (size_t)row0 * D), (short)0, (left < BN ? left : BN) * D, 0x00020000);
#pragma unroll
        for (int r = 0; r < C::ROUNDS8; ++r) {
            uint8_t *d = dst + (r * 4 + wave_s) * C::RPW8 * D;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)d, 16, voff, r * ROUND8, 0, 0);
        }
    };

    // ---- running state -----------------------------------------------------
    f32x16 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
    float m_ref = -INFINITY;
    float l_run = 0.f;

    // K operand: row n (+32 for the second key half, same swizzle), bytes
    // 64 s + 32 g .. + 31 = chunks 4 s + 2 g and 4 s + 2 g + 1
    int k_off[C::KS8][2];
#pragma unroll
    for (int s = 0; s < C::KS8; ++s)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) k_off[s][hf] = n * D + (((4 * s + 2 * g + hf) ^ swz8<D>(n)) * 16);
    // V^T operand by ds_read_b64_tr_b8: in each 16-lane group G, output lane
    // 16 G + 8 h + c receives byte c of the 8-byte reads of lanes 16 G + h,
    // + 2, ..., + 14.  Lane a therefore reads the row holding the key that
    // k-slot e = (a % 16) / 2 of output lanes 16 G + 8 h + .. needs (the key
    // order of P^T: 4 g + {0..3, 8..11}, g = G / 2) at columns
    // 32 cb + 16 (G % 2) + 8 h .. + 7.
    int v_off[C::CB];
    {
        const int G = lane >> 4, i = lane & 15, e = i >> 1, hb = i & 1;
        const int rl = 4 * (G >> 1) + (e < 4 ? e : e + 4);  // key within the 16-key step
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
            v_off[cb] = rl * D + (((2 * cb + (G & 1)) ^ swzw<D>(rl)) * 16) + 8 * hb;
    }

    auto kfrag = [&](const uint8_t *sk, int kt, int s) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(sk + kt * 32 * D + k_off[s][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(sk + kt * 32 * D + k_off[s][1]);
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // 8 fp8 values of one V column, widened exactly to bf16 in registers
    auto vfrag = [&](const uint8_t *sw, int cb, int kt, int hh) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(sw + (kt * 32 + 16 * hh) * D + v_off[cb]));
        u32x4 y;
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
            y[2 * wd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[wd], 1.0f, false));
            y[2 * wd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)x[wd], 1.0f, true));
        }
        return __builtin_bit_cast(bf16x8, y);
    };
    auto qk = [&](const uint8_t *sk, f32x16 (&st)[2]) {
        st[0] = f32x16{};
        st[1] = f32x16{};
#pragma unroll
        for (int s = 0; s < C::KS8; ++s)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) st[kt] = mfma8(kfrag(sk, kt, s), qf[s], st[kt]);
    };

    // Rings: K[j] in sK[j & 1] (DMA'd two tiles ahead), fp8 V[j] in sW[j & 1]
    // (one tile ahead).  Iteration j starts K[j+2] and V[j+1], computes the
    // scores of tile j+1 with the softmax of tile j, then P V of tile j.
    auto kbuf = [&](int j) { return (j & 1) ? sK1 : sK0; };
    auto wbuf = [&](int j) { return (j & 1) ? sW1 : sW0; };
    auto dma_k = [&](int j) { dma_rows8(Kh, j * BN, kbuf(j), voff_k); };
    auto dma_w = [&](int j) { dma_rows8(Vh, j * BN, wbuf(j), voff_w); };

    auto iteration = [&](const int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        const int j0 = j * BN;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K[j+1], V[j] have landed
        __syncthreads();                                   // ... for every wave; K[j], V[j-1] are free
        if (j + 2 < ntiles) dma_k(j + 2);
        if (j + 1 < ntiles) dma_w(j + 1);
        if (CAUSAL && j0 > wave_first_row + 31 + off) return;

        const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > wave_first_row + off);
        if (need_mask) {
            const int rel = lim - j0 - 4 * g;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = kt * 32 + 8 * (r >> 2) + (r & 3);
                    if (kk > rel) cur[kt][r] = -INFINITY;
                }
            }
        }
        // scores of tile j+1 (2 * KS8 fp8 MFMAs) interleaved with P of tile j
        const uint8_t *skn = kbuf(j + 1);
        constexpr int NQK = 2 * C::KS8;
        constexpr int PAIRS_PER = 16 / NQK;
        u32x4 pb[2][2];
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
        const bool fresh = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
        const float m_use = fresh ? 0.f : m_ref;
        nxt[0] = f32x16{};
        nxt[1] = f32x16{};
        i32x8 kq = kfrag(skn, 0, 0);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int s = i >> 1, kt = i & 1;
            const i32x8 cur_k = kq;
            if (i + 1 < NQK) kq = kfrag(skn, (i + 1) & 1, (i + 1) >> 1);
            nxt[kt] = mfma8(cur_k, qf[s], nxt[kt]);
#pragma unroll
            for (int q = 0; q < PAIRS_PER; ++q) {
                const int pi = i * PAIRS_PER + q;
                const int pkt = pi >> 3, hh = (pi >> 2) & 1, ii = pi & 3;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[pkt][8 * hh + 2 * ii], sl2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[pkt][8 * hh + 2 * ii + 1], sl2, -m_use));
                pb[pkt][hh][ii] = pack_bf16(p0, p1);
                ps[ii] += p0 + p1;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        if (fresh || __builtin_amdgcn_ballot_w64(!(psum <= RESCALE_SUM)) != 0) {
            float mr = cur[0][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = (kt == 0 ? 1 : 0); r < 16; ++r) mr = fmaxf(mr, cur[kt][r]);
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
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii], sl2, -mu));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(cur[kt][8 * hh + 2 * ii + 1], sl2, -mu));
                        pb[kt][hh][ii] = pack_bf16(p0, p1);
                        psum += p0 + p1;
                    }
        }
        l_run += psum;

        // O^T += V^T P^T for tile j (fp8 V tile, widened per operand)
        const uint8_t *svc = wbuf(j);
        constexpr int NPV = 4 * C::CB;
        constexpr int VAHEAD = 4;
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
    if (ntiles > 0) {
        dma_k(0);
        dma_w(0);
        if (ntiles > 1) dma_k(1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        qk(sK0, stA);
    }
    for (int j = 0; j < ntiles; j += 2) {
        iteration(j, stA, stB);
        if (j + 1 < ntiles) iteration(j + 1, stB, stA);
    }

    // ---- epilogue ------------------------------------------------------------
    // O goes out as whole rows: the wave writes its 32 bf16 rows to LDS
    // (16-byte chunks XOR-swizzled by row), then stores them back with 1 KB
    // wave-wide stores of consecutive rows, instead of 8-byte pieces over 32
    // rows.  Once every wave has passed the barrier the fp8 tiles are free;
    // wave w uses buffer w (32 rows x D bf16 = one tile's bytes).
    const float l_tot = l_run + wave_xor32(l_run);
    {
        constexpr int CHK = D / 8;  // 16-byte chunks per row
        static_assert(NTHR == 256 && 32 * D * 2 <= C::TILE8, "one fp8 tile buffer holds a wave's 32 rows");
        __syncthreads();
        __bf16 *stg = reinterpret_cast<__bf16 *>(wave_s == 0 ? sK0 : wave_s == 1 ? sK1 : wave_s == 2 ? sW0 : sW1);
        const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
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
        const int row0 = q0 + wave * 32;
        __bf16 *obase = O + ((size_t)(b * Hq + h) * Nq + row0) * D;
        constexpr int RPI = 64 / CHK;  // rows per wave-wide store
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int row = i * RPI + lane / CHK, chunk = lane % CHK;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + row * D + ((chunk ^ (row & (CHK - 1))) * 8));
            if (row0 + row < Nq) *reinterpret_cast<u32x4 *>(obase + (size_t)row * D + chunk * 8) = val;
        }
    }
    if (qi < Nq && LSE && g == 0)
        LSE[(size_t)(b * Hq + h) * Nq + qi] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * LN2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8FwdArgs &a, hipStream_t stream) {
    const float sl2 = a.scale * LOG2E;
    const int n_qtiles = (a.Nq + BM - 1) / BM;
    const long long total = (long long)a.B * a.Hq * n_qtiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_fp8_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(NTHR), 0, stream,
                       (const uint8_t *)a.q, (const uint8_t *)a.k, (const uint8_t *)a.v, (__bf16 *)a.o, a.lse,
                       a.Hq, a.Hkv, a.Nq, a.Nk, sl2, a.v_scale, n_qtiles, (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp8(const Fp8FwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
