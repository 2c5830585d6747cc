// prefill_bf16.hip -- fused attention forward for bf16 inputs on gfx950.
//
// One kernel computes O = softmax(scale * Q K^T [+ causal mask]) V and the
// per-row log-sum-exp without ever writing the score matrix to device memory
// ("Transformer 架构的数学与计算深度解析", sec. 6: tiles stay on chip; sec. 6.3 and
// "从注意力到 IO 感知执行" sec. 8, eqs. (1)-(2): the running max / denominator /
// un-normalised accumulator recurrence).
//
// gfx950 mapping
//   * A workgroup owns BM = 128 query rows of one (batch, query head); each of
//     its 4 waves owns 32 rows.  K/V are streamed in tiles of BN = 64 keys.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q^T (held in
//     registers for the whole kernel) the B operand.  In the fp32 result every
//     lane holds ONE query row (lane % 32) and 16 keys per 32-key block, the
//     other 16 keys sitting in lane ^ 32.  Row max and row sum are therefore
//     in-lane reductions plus a single exchange with lane ^ 32.
//   * P^T, converted to bf16 in registers, is directly the B operand of
//     O^T = V^T P^T (again 32x32x16), whose A operand V^T is read from LDS
//     where the V tile is stored transposed with the keys of each 16-key
//     group permuted (bits 2 and 3 of the key index swapped), so that each
//     lane's 8 keys are one contiguous 16-byte LDS read.  No LDS round trip
//     for P, no cross-lane shuffles for the rescale of O^T (one query per
//     lane).
//   * Softmax in base 2: t = s * (scale * log2 e); exp2 is v_exp_f32.
//   * Causal: tiles beyond the last visible key of the workgroup are never
//     loaded; only tiles that straddle the diagonal (or the end of K) apply
//     the element mask.  Bottom-right alignment: row i sees j <= i + Nk - Nq.
//   * GQA: query head h reads K/V head h / (Hq / Hkv).  Work items are
//     ordered (batch, KV head) outermost, then query tile (heaviest causal
//     tile first), then the G query heads of the group, and spread over the
//     8 XCDs in contiguous chunks, so the query heads sharing a K/V head run
//     on one XCD at the same time and read that head's K/V through one L2.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NTHR = 256;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

template <int D>
struct Cfg {
    static constexpr int KST = D + 8;    // LDS row stride of K, elements (16 B pad)
    static constexpr int VST = BN + 8;   // LDS row stride of V^T, elements (16 B pad)
    static constexpr int KS = D / 16;    // k-steps of the score MFMA
    static constexpr int CB = D / 32;    // 32-column blocks of O^T
    static constexpr int CH = D / 8;     // 16-byte chunks per row
    static constexpr int KLD = BN * CH / NTHR;  // 16-byte K loads per thread
    static constexpr int KPT = D / 32;   // keys per thread when staging V
    static constexpr int VA = BN / KPT;  // key groups per tile when staging V
    static_assert(KLD * NTHR == BN * CH, "K tile split");
    static_assert(VA * CH == NTHR, "V tile split");
};

// Position of key j (0..BN-1) inside a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int vperm(int j) {
    return (j & ~12) | ((j >> 1) & 4) | ((j << 1) & 8);
}

__device__ __forceinline__ float wave_xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

// Round-to-nearest-even pair conversion fp32 -> packed bf16 (lo in bits 0..15),
// a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHR, 2) void prefill_bf16_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
    float sl2, int n_qtiles, int total)
{
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) __bf16 sK[BN * C::KST];
    __shared__ __attribute__((aligned(16))) __bf16 sV[D * C::VST];

    // ---- work item: XCD-contiguous remap of the linear block id ----------
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
    const int off = Nk - Nq;  // bottom-right causal offset

    const __bf16 *Qh = Q + ((size_t)(b * Hq + h) * Nq) * D;
    const __bf16 *Kh = K + ((size_t)(b * Hkv + hk) * Nk) * D;
    const __bf16 *Vh = V + ((size_t)(b * Hkv + hk) * Nk) * D;

    // ---- Q^T operands, resident for the whole kernel ---------------------
    const int qi = q0 + wave * 32 + n;  // this lane's query row
    bf16x8 qf[C::KS];
    if (qi < Nq) {
        const bf16x8 *src = reinterpret_cast<const bf16x8 *>(Qh + (size_t)qi * D + 8 * g);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = bf16x8{};
    }

    // ---- key range --------------------------------------------------------
    int kv_end = Nk;
    if (CAUSAL) {
        const int last_row = (q0 + BM < Nq ? q0 + BM : Nq);  // exclusive
        const int e = last_row + off;                        // keys < e are visible to some row
        kv_end = e < Nk ? e : Nk;
    }
    const int ntiles = (kv_end + BN - 1) / BN;

    // per-lane limit of visible keys (inclusive)
    const int lim = CAUSAL ? ((qi + off) < (Nk - 1) ? (qi + off) : (Nk - 1)) : (Nk - 1);
    const int wave_last_row = q0 + wave * 32 + 31;

    // ---- staging registers ------------------------------------------------
    u32x4 kreg[C::KLD];
    u32x4 vreg[C::KPT];
    const int va = tid % C::VA, vc = tid / C::VA;  // V staging: key group, column chunk

    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < C::KLD; ++i) {
            const int idx = tid + i * NTHR;
            const int row = idx / C::CH, ch = idx % C::CH;
            const int key = j0 + row;
            kreg[i] = key < Nk ? *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + ch * 8) : u32x4{};
        }
#pragma unroll
        for (int r = 0; r < C::KPT; ++r) {
            const int key = j0 + va * C::KPT + r;
            vreg[r] = key < Nk ? *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + vc * 8) : u32x4{};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::KLD; ++i) {
            const int idx = tid + i * NTHR;
            const int row = idx / C::CH, ch = idx % C::CH;
            *reinterpret_cast<u32x4 *>(sK + row * C::KST + ch * 8) = kreg[i];
        }
        const int pos = vperm(va * C::KPT);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = vc * 8 + e;
            const int dw = e >> 1;
            __bf16 *dst = sV + c * C::VST + pos;
            if (C::KPT == 4) {
                uint32_t x0, x1;
                if (e & 1) {
                    x0 = (vreg[0][dw] >> 16) | (vreg[1][dw] & 0xffff0000u);
                    x1 = (vreg[2][dw] >> 16) | (vreg[3][dw] & 0xffff0000u);
                } else {
                    x0 = (vreg[0][dw] & 0xffffu) | (vreg[1][dw] << 16);
                    x1 = (vreg[2][dw] & 0xffffu) | (vreg[3][dw] << 16);
                }
                *reinterpret_cast<u32x2 *>(dst) = u32x2{x0, x1};
            } else {
                uint32_t x0;
                if (e & 1) x0 = (vreg[0][dw] >> 16) | (vreg[1][dw] & 0xffff0000u);
                else x0 = (vreg[0][dw] & 0xffffu) | (vreg[1][dw] << 16);
                *reinterpret_cast<uint32_t *>(dst) = x0;
            }
        }
    };

    // ---- running state ----------------------------------------------------
    f32x16 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
    float m_run = -INFINITY;  // running max of t = s * scale * log2(e)
    float l_run = 0.f;        // this lane's share of the denominator

    if (ntiles > 0) load_tile(0);

    for (int it = 0; it < ntiles; ++it) {
        const int j0 = it * BN;
        __syncthreads();  // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (it + 1 < ntiles) load_tile(j0 + BN);

        if (CAUSAL && j0 > wave_last_row + off) continue;  // no row of this wave sees the tile

        // S^T = K Q^T for two 32-key blocks
        f32x16 st[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            st[kt] = f32x16{};
            const __bf16 *kp = sK + (kt * 32 + n) * C::KST + 8 * g;
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kp + 16 * s);
                st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[kt], 0, 0, 0);
            }
        }

        // scale (base 2) and mask
        const bool need_mask = (j0 + BN > Nk) || (CAUSAL && j0 + BN - 1 > q0 + wave * 32 + off);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = st[kt][r] * sl2;
                if (need_mask) {
                    const int key = j0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key > lim) x = -INFINITY;
                }
                st[kt][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        // P^T in bf16 (round to nearest even) for the MFMA; the denominator
        // sums the unrounded fp32 values, so LSE carries no bf16 rounding.
        u32x4 pb[2][2];
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(st[kt][8 * hh + 2 * i] - m_use);
                    const float p1 = __builtin_amdgcn_exp2f(st[kt][8 * hh + 2 * i + 1] - m_use);
                    const uint32_t pk = pack_bf16(p0, p1);
                    pb[kt][hh][i] = pk;
                    psum += p0 + p1;
                }
            }
        }
        l_run = l_run * alpha + psum;

#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const __bf16 *vp = sV + (cb * 32 + n) * C::VST + 8 * g;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vp + kt * 32 + 16 * hh);
                    const bf16x8 bb = __builtin_bit_cast(bf16x8, pb[kt][hh]);
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[cb], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: O = u / l, LSE = ln(sum exp(s)) -----------------------
    const float l_tot = l_run + wave_xor32(l_run);
    if (qi < Nq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        __bf16 *orow = O + ((size_t)(b * Hq + h) * Nq + qi) * D;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int c = cb * 32 + 8 * rr + 4 * g;
                const uint32_t lo = pack_bf16(acc[cb][4 * rr + 0] * inv, acc[cb][4 * rr + 1] * inv);
                const uint32_t hi = pack_bf16(acc[cb][4 * rr + 2] * inv, acc[cb][4 * rr + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + c) = u32x2{lo, hi};
            }
        }
        if (LSE && g == 0)
            LSE[(size_t)(b * Hq + h) * Nq + qi] =
                l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.Nq + BM - 1) / BM;
    const long long total = (long long)a.B * a.Hq * n_qtiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float sl2 = a.scale * LOG2E;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(NTHR), 0, stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (__bf16 *)a.o,
                       a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, sl2, n_qtiles, (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
