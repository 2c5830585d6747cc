// prefill_f32.hip -- fused attention forward for fp32 inputs on gfx950.
//
// The fp32 path exists for full-precision checks (max-abs error 1e-5 against
// an fp64 reference), so it keeps every product and sum in fp32 on the vector
// ALUs and uses the accurate expf / logf, with no reduced-precision matrix
// instruction anywhere.  It is the same blockwise online-softmax recurrence as
// the bf16 kernel ("Transformer 架构的数学与计算深度解析", sec. 6.3; "从注意力到
// IO 感知执行", sec. 8, eqs. (1)-(2)), applied to tiles of 64 keys.
//
// Mapping.  A workgroup of four waves owns QT = 4 * RW query rows of one
// (batch, head); each wave owns RW of them.  The workgroup stages each tile of
// 64 K and V rows in LDS (the next tile's loads are in flight while the
// current one is computed), and inside a wave the 64 lanes split the work two
// ways:
//   * scores: lane j holds key j of the tile and forms its dot product with
//     each of the wave's query rows (query rows are LDS broadcasts, the K row
//     a conflict-free 16-byte read from a row stride padded by 4 floats);
//     the tile maximum is a cross-lane reduction, and each lane keeps its own
//     partial denominator, summed across lanes once at the end;
//   * P V: lane c holds D / 64 consecutive output columns and runs over the
//     64 keys of the tile, with the probabilities read back from LDS as
//     broadcasts and the V row read contiguously.
// Every lane therefore does O(64 + D) work per tile and row instead of
// O(64 * D), and a small problem spreads over many waves: with RW = 1 a
// 128-row head already occupies 128 waves.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

constexpr int WAVES = 4;  // waves per workgroup
constexpr int TK = 64;    // keys per tile (one per lane in the score step)

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s, 64);
    return x;
}

template <int D, int RW, bool CAUSAL>
__global__ __launch_bounds__(64 * WAVES) void prefill_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float scale,
    int n_qtiles)
{
    constexpr int QT = WAVES * RW;  // query rows per workgroup
    constexpr int KS = D + 4;       // padded K row stride (floats)
    constexpr int NC = D / 64;      // output columns per lane
    constexpr int F4 = TK * D / 4;  // float4s per K (or V) tile
    constexpr int LPT = F4 / (64 * WAVES);  // float4 loads per thread per tile and tensor
    static_assert(F4 % (64 * WAVES) == 0, "tile loads");
    __shared__ __attribute__((aligned(16))) float sK[TK * KS];
    __shared__ __attribute__((aligned(16))) float sV[TK * D];
    __shared__ __attribute__((aligned(16))) float sQ[QT * D];
    __shared__ __attribute__((aligned(16))) float sP[WAVES][RW][TK];

    const int tq = blockIdx.x % n_qtiles;
    const int bh = blockIdx.x / n_qtiles;
    const int h = bh % Hq, b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int off = Nk - Nq;  // bottom-right alignment of the causal mask

    const float *Qh = Q + (size_t)(b * Hq + h) * Nq * D;
    const float *Kh = K + (size_t)(b * Hkv + hk) * Nk * D;
    const float *Vh = V + (size_t)(b * Hkv + hk) * Nk * D;

    // query tile (zeros beyond Nq; those rows are computed but never stored)
    for (int i = tid; i < QT * D / 4; i += 64 * WAVES) {
        const int row = tq * QT + i / (D / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < Nq) x = reinterpret_cast<const float4 *>(Qh)[(size_t)tq * QT * D / 4 + i];
        reinterpret_cast<float4 *>(sQ)[i] = x;
    }

    int kv_end = Nk;
    if (CAUSAL) {
        const int last = tq * QT + QT < Nq ? tq * QT + QT : Nq;  // one past the workgroup's last row
        kv_end = last + off < Nk ? last + off : Nk;
        if (kv_end < 0) kv_end = 0;
    }

    float4 kr[LPT], vr[LPT];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 64 * WAVES * i;
            const int key = j0 + idx / (D / 4);
            kr[i] = vr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (key < Nk) {
                kr[i] = reinterpret_cast<const float4 *>(Kh)[(size_t)j0 * D / 4 + idx];
                vr[i] = reinterpret_cast<const float4 *>(Vh)[(size_t)j0 * D / 4 + idx];
            }
        }
    };

    float o[RW][NC], m[RW], lp[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        m[r] = -INFINITY;
        lp[r] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) o[r][c] = 0.f;
    }

    if (kv_end > 0) fetch(0);
    for (int j0 = 0; j0 < kv_end; j0 += TK) {
        __syncthreads();  // the previous tile's readers are done
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + 64 * WAVES * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            *reinterpret_cast<float4 *>(sK + row * KS + 4 * c4) = kr[i];
            reinterpret_cast<float4 *>(sV)[idx] = vr[i];
        }
        __syncthreads();
        if (j0 + TK < kv_end) fetch(j0 + TK);

        // scores: lane = key
        float acc[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[r] = 0.f;
#pragma unroll 4
        for (int c4 = 0; c4 < D / 4; ++c4) {
            const float4 kv = *reinterpret_cast<const float4 *>(sK + lane * KS + 4 * c4);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float4 qv = *reinterpret_cast<const float4 *>(sQ + (wave * RW + r) * D + 4 * c4);
                acc[r] = fmaf(qv.x, kv.x, acc[r]);
                acc[r] = fmaf(qv.y, kv.y, acc[r]);
                acc[r] = fmaf(qv.z, kv.z, acc[r]);
                acc[r] = fmaf(qv.w, kv.w, acc[r]);
            }
        }
        const int key = j0 + lane;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int row = tq * QT + wave * RW + r;
            const bool vis = key < Nk && (!CAUSAL || key <= row + off);
            const float s = vis ? acc[r] * scale : -INFINITY;
            const float mnew = fmaxf(m[r], wave_max(s));
            float p = 0.f, alpha = 1.f;
            if (mnew != -INFINITY) {  // otherwise nothing is visible yet for this row
                alpha = expf(m[r] - mnew);  // m = -inf gives 0
                p = expf(s - mnew);
            }
            lp[r] = lp[r] * alpha + p;
#pragma unroll
            for (int c = 0; c < NC; ++c) o[r][c] *= alpha;
            m[r] = mnew;
            sP[wave][r][lane] = p;
        }
        // P V: lane = output columns; sP is written and read by this wave only
        // and LDS operations of one wave complete in order
#pragma unroll 2
        for (int j = 0; j < TK; j += 4) {
            float vv[4][NC];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (NC == 2) {
                    const float2 x = *reinterpret_cast<const float2 *>(sV + (j + t) * D + 2 * lane);
                    vv[t][0] = x.x;
                    vv[t][1] = x.y;
                } else {
                    vv[t][0] = sV[(j + t) * D + lane];
                }
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float4 pv = *reinterpret_cast<const float4 *>(&sP[wave][r][j]);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    o[r][c] = fmaf(pv.x, vv[0][c], o[r][c]);
                    o[r][c] = fmaf(pv.y, vv[1][c], o[r][c]);
                    o[r][c] = fmaf(pv.z, vv[2][c], o[r][c]);
                    o[r][c] = fmaf(pv.w, vv[3][c], o[r][c]);
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = tq * QT + wave * RW + r;
        const float l = wave_sum(lp[r]);
        if (row >= Nq) continue;
        float *dst = O + ((size_t)(b * Hq + h) * Nq + row) * D;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if constexpr (NC == 2) {
            *reinterpret_cast<float2 *>(dst + 2 * lane) = make_float2(o[r][0] * inv, o[r][1] * inv);
        } else {
            dst[lane] = o[r][0] * inv;
        }
        if (LSE && lane == 0) LSE[(size_t)(b * Hq + h) * Nq + row] = l > 0.f ? m[r] + logf(l) : -INFINITY;
    }
}

template <int D, int RW, bool CAUSAL>
hipError_t launch_rw(const FwdArgs &a, hipStream_t stream) {
    constexpr int QT = WAVES * RW;
    const int n_qtiles = (a.Nq + QT - 1) / QT;
    const long long total = (long long)a.B * a.Hq * n_qtiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D, RW, CAUSAL>), dim3((unsigned)total), dim3(64 * WAVES), 0, stream,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (float *)a.o, a.lse,
                       a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, n_qtiles);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    // four rows per wave share each K / V read; a grid that would leave the
    // chip's 1024 SIMDs mostly idle takes one row per wave instead
    const long long waves4 = (long long)a.B * a.Hq * ((a.Nq + 15) / 16) * WAVES;
    return waves4 >= 1024 ? launch_rw<D, 4, CAUSAL>(a, stream) : launch_rw<D, 1, CAUSAL>(a, stream);
}

}  // namespace

hipError_t launch_prefill_f32(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
