// prefill_f32.hip -- fused attention forward for fp32 inputs on gfx950.
//
// The fp32 path exists for full-precision checks (max-abs error 1e-5 against
// an fp64 reference), so it keeps every product and sum in fp32 on the vector
// ALUs and uses the accurate expf / logf, with no reduced-precision matrix
// instruction anywhere.  It is the same blockwise online-softmax recurrence as
// the bf16 kernel ("Transformer 架构的数学与计算深度解析", sec. 6.3; "从注意力到
// IO 感知执行", sec. 8, eqs. (1)-(2)): K/V tiles of 32 keys are staged in LDS
// and every lane carries one query row's running max m, denominator l and
// un-normalised accumulator u, dividing once at the end.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

constexpr int ROWS = 64;  // query rows per workgroup (one per lane)
constexpr int TN = 32;    // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(ROWS) void prefill_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk, float scale,
    int n_qtiles)
{
    __shared__ __attribute__((aligned(16))) float sK[TN * D];
    __shared__ __attribute__((aligned(16))) float sV[TN * D];

    const int tq = blockIdx.x % n_qtiles;
    const int bh = blockIdx.x / n_qtiles;
    const int h = bh % Hq, b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    const int lane = threadIdx.x;
    const int qi = tq * ROWS + lane;
    const int off = Nk - Nq;

    const float *Kh = K + (size_t)(b * Hkv + hk) * Nk * D;
    const float *Vh = V + (size_t)(b * Hkv + hk) * Nk * D;

    float q[D], u[D];
    if (qi < Nq) {
        const float4 *src = reinterpret_cast<const float4 *>(Q + ((size_t)(b * Hq + h) * Nq + qi) * D);
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            const float4 x = src[c];
            q[4 * c] = x.x; q[4 * c + 1] = x.y; q[4 * c + 2] = x.z; q[4 * c + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < D; ++c) q[c] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < D; ++c) u[c] = 0.f;
    float m = -INFINITY, l = 0.f;

    int kv_end = Nk;
    if (CAUSAL) {
        const int last_row = (tq * ROWS + ROWS < Nq) ? tq * ROWS + ROWS : Nq;
        kv_end = last_row + off < Nk ? last_row + off : Nk;
    }
    const int lim = CAUSAL ? qi + off : Nk - 1;  // last visible key of this row

    for (int j0 = 0; j0 < kv_end; j0 += TN) {
        __syncthreads();
        // stage K and V tiles (zeros beyond Nk)
        for (int idx = lane; idx < TN * D / 4; idx += ROWS) {
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int key = j0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < Nk) {
                kx = reinterpret_cast<const float4 *>(Kh + (size_t)key * D)[c4];
                vx = reinterpret_cast<const float4 *>(Vh + (size_t)key * D)[c4];
            }
            reinterpret_cast<float4 *>(sK)[idx] = kx;
            reinterpret_cast<float4 *>(sV)[idx] = vx;
        }
        __syncthreads();

        float s[TN];
        float mblk = -INFINITY;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) acc = fmaf(q[c], sK[j * D + c], acc);
            const int key = j0 + j;
            const bool vis = key < Nk && key <= lim;
            s[j] = vis ? acc * scale : -INFINITY;
            mblk = fmaxf(mblk, s[j]);
        }
        const float mnew = fmaxf(m, mblk);
        if (mnew != -INFINITY) {  // otherwise nothing is visible yet for this row
            const float alpha = expf(m - mnew);  // m = -inf gives 0
            l *= alpha;
#pragma unroll
            for (int c = 0; c < D; ++c) u[c] *= alpha;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float p = expf(s[j] - mnew);
                l += p;
#pragma unroll
                for (int c = 0; c < D; ++c) u[c] = fmaf(p, sV[j * D + c], u[c]);
            }
            m = mnew;
        }
    }

    if (qi < Nq) {
        float *dst = O + ((size_t)(b * Hq + h) * Nq + qi) * D;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c)
            reinterpret_cast<float4 *>(dst)[c] =
                make_float4(u[4 * c] * inv, u[4 * c + 1] * inv, u[4 * c + 2] * inv, u[4 * c + 3] * inv);
        if (LSE) LSE[(size_t)(b * Hq + h) * Nq + qi] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.Nq + ROWS - 1) / ROWS;
    const long long total = (long long)a.B * a.Hq * n_qtiles;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(ROWS), 0, stream,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (float *)a.o, a.lse,
                       a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const FwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
