// bwd_f32.hip -- gradients of the attention forward for fp32 inputs.
//
// Full-precision companion of the bf16 backward (the same recomputation from
// the saved log-sum-exp, "从注意力到 IO 感知执行", evaluation protocol: compare
// gradients with a higher-precision reference; "Transformer 架构的数学与计算
// 深度解析" sec. 3.3: training needs the gradients through the weights).  For
// row i of a query head and key j of its K/V head, with s = scale:
//   p_ij  = exp(s q_i . k_j - lse_i)          (0 where the causal mask hides j)
//   dp_ij = do_i . v_j,   D_i = do_i . o_i,   ds_ij = p_ij (dp_ij - D_i)
//   dq_i = s sum_j ds_ij k_j,   dk_j = s sum_i ds_ij q_i,   dv_j = sum_i p_ij do_i
// where dk and dv sum over the rows of every query head of the GQA group.
// Every product and sum is fp32 on the vector ALUs with the accurate expf, as
// in the fp32 forward; no reduced-precision matrix instruction is used.
//
// Three kernels:
//   * bwd_f32_pre_kernel: D_i for every row (one 64-lane group per row).
//   * bwd_f32_dq_kernel: 4 waves x RW query rows of one head share each
//     64-key K/V tile in LDS.  For the scores lane j holds key j (K and V
//     rows padded by 4 floats, so its 16-byte reads are conflict-free) and
//     forms s and dp with each of the wave's rows (LDS broadcasts); ds goes to
//     LDS and lane c then accumulates dq for D / 64 columns over the tile's
//     keys, as the fp32 forward's P V step does.
//   * bwd_f32_dkdv_kernel: 4 waves x RK keys of one K/V head; 64-row tiles of
//     Q and dO (every query head of the group in turn) stream through LDS.
//     Lane i holds row i of the tile for p and ds, then lane c accumulates dk
//     and dv for D / 64 columns over the tile's rows.
// Causal: bottom-right alignment (row i sees keys j <= i + Nk - Nq); tiles no
// row (key) of the workgroup can see are skipped.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

constexpr int WAVES = 4;
constexpr int NTHR = 64 * WAVES;
constexpr int TILE = 64;  // keys per K/V tile (dq), rows per Q/dO tile (dk, dv)

template <int D>
__global__ __launch_bounds__(NTHR) void bwd_f32_pre_kernel(const float *__restrict__ O, const float *__restrict__ dO,
                                                           float *__restrict__ Dv, long long rows) {
    const long long row = (long long)blockIdx.x * WAVES + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    float acc = 0.f;
    if (row < rows) {
#pragma unroll
        for (int c = lane; c < D; c += 64) acc = fmaf(O[(size_t)row * D + c], dO[(size_t)row * D + c], acc);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows && lane == 0) Dv[row] = acc;
}

// 16-byte dot product of two D-float rows in LDS.
template <int D>
__device__ __forceinline__ float dot_row(const float *a, const float *b) {
    float acc = 0.f;
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
        const float4 x = *reinterpret_cast<const float4 *>(a + 4 * c4);
        const float4 y = *reinterpret_cast<const float4 *>(b + 4 * c4);
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
    }
    return acc;
}

// Loads `rows` consecutive D-float rows from src (rows >= nvalid read as
// zeros) into registers, float4 by float4, NTHR threads.
template <int D, int ROWS>
struct TileRegs {
    static constexpr int F4 = ROWS * D / 4;
    static constexpr int LPT = (F4 + NTHR - 1) / NTHR;
    float4 r[LPT];
    __device__ __forceinline__ void fetch(const float *src, int nvalid, int tid) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + NTHR * i;
            r[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (idx < F4 && idx / (D / 4) < nvalid) r[i] = reinterpret_cast<const float4 *>(src)[idx];
        }
    }
    // into LDS rows of stride S floats
    template <int S>
    __device__ __forceinline__ void store(float *dst, int tid) const {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int idx = tid + NTHR * i;
            if (idx < F4) *reinterpret_cast<float4 *>(dst + (idx / (D / 4)) * S + 4 * (idx % (D / 4))) = r[i];
        }
    }
};

template <int D, int RW, bool CAUSAL>
__global__ __launch_bounds__(NTHR) void bwd_f32_dq_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dv, float *__restrict__ dQ,
    int Hq, int Hkv, int Nq, int Nk, float scale, int n_qtiles)
{
    constexpr int QT = WAVES * RW;  // query rows per workgroup
    constexpr int KS = D + 4;       // padded K / V row stride (floats)
    constexpr int NC = D / 64;      // dq columns per lane
    __shared__ __attribute__((aligned(16))) float sK[TILE * KS];
    __shared__ __attribute__((aligned(16))) float sV[TILE * KS];
    __shared__ __attribute__((aligned(16))) float sQ[QT * D];
    __shared__ __attribute__((aligned(16))) float sdO[QT * D];
    __shared__ __attribute__((aligned(16))) float sDS[WAVES][RW][TILE];

    const int tq = blockIdx.x % n_qtiles;
    const int bh = blockIdx.x / n_qtiles;
    const int h = bh % Hq, b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int off = Nk - Nq;
    const int row0 = tq * QT;
    const size_t qbase = (size_t)(b * Hq + h) * Nq;
    const float *Kh = K + (size_t)(b * Hkv + hk) * Nk * D;
    const float *Vh = V + (size_t)(b * Hkv + hk) * Nk * D;

    {
        TileRegs<D, QT> tq_r, tdo_r;
        const int nv = Nq - row0;
        tq_r.fetch(Q + (qbase + row0) * D, nv, tid);
        tdo_r.fetch(dO + (qbase + row0) * D, nv, tid);
        tq_r.template store<D>(sQ, tid);
        tdo_r.template store<D>(sdO, tid);
    }
    float lse[RW], dd[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = row0 + wave * RW + r;
        lse[r] = row < Nq ? LSE[qbase + row] : 0.f;
        dd[r] = row < Nq ? Dv[qbase + row] : 0.f;
    }

    int kv_end = Nk;
    if (CAUSAL) {
        const int last = row0 + QT < Nq ? row0 + QT : Nq;  // one past the workgroup's last row
        kv_end = last + off < Nk ? last + off : Nk;
    }

    float acc[RW][NC];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[r][c] = 0.f;

    TileRegs<D, TILE> kr, vr;
    if (kv_end > 0) {
        kr.fetch(Kh, Nk, tid);
        vr.fetch(Vh, Nk, tid);
    }
    for (int j0 = 0; j0 < kv_end; j0 += TILE) {
        __syncthreads();  // the previous tile's readers are done
        kr.template store<KS>(sK, tid);
        vr.template store<KS>(sV, tid);
        __syncthreads();
        if (j0 + TILE < kv_end) {
            kr.fetch(Kh + (size_t)(j0 + TILE) * D, Nk - j0 - TILE, tid);
            vr.fetch(Vh + (size_t)(j0 + TILE) * D, Nk - j0 - TILE, tid);
        }
        // ds for key j0 + lane and each of the wave's rows
        const int key = j0 + lane;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int row = row0 + wave * RW + r;
            const float s = dot_row<D>(sQ + (wave * RW + r) * D, sK + lane * KS);
            const float dp = dot_row<D>(sdO + (wave * RW + r) * D, sV + lane * KS);
            const bool vis = row < Nq && key < Nk && (!CAUSAL || key <= row + off);
            const float p = vis ? expf(fmaf(s, scale, -lse[r])) : 0.f;
            sDS[wave][r][lane] = p * (dp - dd[r]);
        }
        // dq += ds K: lane = columns; sDS is written and read by this wave
        // only, and one wave's LDS operations complete in order
#pragma unroll 4
        for (int j = 0; j < TILE; ++j) {
            float kv[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) kv[c] = sK[j * KS + NC * lane + c];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float ds = sDS[wave][r][j];
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[r][c] = fmaf(ds, kv[c], acc[r][c]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = row0 + wave * RW + r;
        if (row >= Nq) continue;
        float *dst = dQ + (qbase + row) * D + NC * lane;
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[c] = acc[r][c] * scale;
    }
}

template <int D, int RK, bool CAUSAL>
__global__ __launch_bounds__(NTHR) void bwd_f32_dkdv_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dv, float *__restrict__ dK,
    float *__restrict__ dV, int Hq, int Hkv, int Nq, int Nk, float scale, int n_ktiles)
{
    constexpr int KT = WAVES * RK;  // keys per workgroup
    constexpr int QS = D + 4;       // padded Q / dO row stride (floats)
    constexpr int NC = D / 64;      // dk / dv columns per lane
    __shared__ __attribute__((aligned(16))) float sK[KT * D];
    __shared__ __attribute__((aligned(16))) float sV[KT * D];
    __shared__ __attribute__((aligned(16))) float sQ[TILE * QS];
    __shared__ __attribute__((aligned(16))) float sdO[TILE * QS];
    __shared__ float sL[TILE], sD[TILE];
    __shared__ __attribute__((aligned(16))) float sP[WAVES][RK][TILE];
    __shared__ __attribute__((aligned(16))) float sDS[WAVES][RK][TILE];

    const int tk = blockIdx.x % n_ktiles;
    const int bhk = blockIdx.x / n_ktiles;
    const int hk = bhk % Hkv, b = bhk / Hkv;
    const int G = Hq / Hkv;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int off = Nk - Nq;
    const int key0 = tk * KT;
    const size_t kbase = (size_t)(b * Hkv + hk) * Nk;

    {
        TileRegs<D, KT> tk_r, tv_r;
        tk_r.fetch(K + (kbase + key0) * D, Nk - key0, tid);
        tv_r.fetch(V + (kbase + key0) * D, Nk - key0, tid);
        tk_r.template store<D>(sK, tid);
        tv_r.template store<D>(sV, tid);
    }

    // first row that sees any of the workgroup's keys (causal: j <= i + off)
    int i_begin = 0;
    if (CAUSAL) {
        i_begin = key0 - off;
        i_begin = i_begin < 0 ? 0 : i_begin;
        i_begin = i_begin / TILE * TILE;
    }

    float dk[RK][NC], dv[RK][NC];
#pragma unroll
    for (int r = 0; r < RK; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) dk[r][c] = dv[r][c] = 0.f;

    TileRegs<D, TILE> qr, dor;
    for (int g = 0; g < G; ++g) {
        const size_t qbase = (size_t)(b * Hq + hk * G + g) * Nq;
        for (int i0 = i_begin; i0 < Nq; i0 += TILE) {
            qr.fetch(Q + (qbase + i0) * D, Nq - i0, tid);
            dor.fetch(dO + (qbase + i0) * D, Nq - i0, tid);
            __syncthreads();  // the previous tile's readers are done
            qr.template store<QS>(sQ, tid);
            dor.template store<QS>(sdO, tid);
            if (tid < TILE) {
                const int row = i0 + tid;
                sL[tid] = row < Nq ? LSE[qbase + row] : 0.f;
                sD[tid] = row < Nq ? Dv[qbase + row] : 0.f;
            }
            __syncthreads();
            // p and ds for row i0 + lane and each of the wave's keys
            const int row = i0 + lane;
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                const int kl = wave * RK + r, key = key0 + kl;
                const float s = dot_row<D>(sQ + lane * QS, sK + kl * D);
                const float dp = dot_row<D>(sdO + lane * QS, sV + kl * D);
                const bool vis = row < Nq && key < Nk && (!CAUSAL || key <= row + off);
                const float p = vis ? expf(fmaf(s, scale, -sL[lane])) : 0.f;
                sP[wave][r][lane] = p;
                sDS[wave][r][lane] = p * (dp - sD[lane]);
            }
            // dv += p^T dO, dk += ds^T Q: lane = columns (this wave's sP /
            // sDS only; one wave's LDS operations complete in order)
#pragma unroll 4
            for (int i = 0; i < TILE; ++i) {
                float qv[NC], dov[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    qv[c] = sQ[i * QS + NC * lane + c];
                    dov[c] = sdO[i * QS + NC * lane + c];
                }
#pragma unroll
                for (int r = 0; r < RK; ++r) {
                    const float p = sP[wave][r][i], ds = sDS[wave][r][i];
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        dv[r][c] = fmaf(p, dov[c], dv[r][c]);
                        dk[r][c] = fmaf(ds, qv[c], dk[r][c]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RK; ++r) {
        const int key = key0 + wave * RK + r;
        if (key >= Nk) continue;
        float *dkr = dK + (kbase + key) * D + NC * lane;
        float *dvr = dV + (kbase + key) * D + NC * lane;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            dkr[c] = dk[r][c] * scale;
            dvr[c] = dv[r][c];
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs &a, hipStream_t stream) {
    constexpr int RW = 4, RK = 4;
    const long long rows = (long long)a.B * a.Hq * a.Nq;
    float *Dv = a.ws_d;
    hipLaunchKernelGGL((bwd_f32_pre_kernel<D>), dim3((unsigned)((rows + WAVES - 1) / WAVES)), dim3(NTHR), 0, stream,
                       (const float *)a.o, (const float *)a.dout, Dv, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_qtiles = (a.Nq + WAVES * RW - 1) / (WAVES * RW);
    const long long gq = (long long)a.B * a.Hq * n_qtiles;
    const int n_ktiles = (a.Nk + WAVES * RK - 1) / (WAVES * RK);
    const long long gk = (long long)a.B * a.Hkv * n_ktiles;
    if (gq > 0x7fffffffLL || gk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, RW, CAUSAL>), dim3((unsigned)gq), dim3(NTHR), 0, stream,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (const float *)a.dout, a.lse, Dv,
                       (float *)a.dq, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, n_qtiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, RK, CAUSAL>), dim3((unsigned)gk), dim3(NTHR), 0, stream,
                       (const float *)a.q, (const float *)a.k, (const float *)a.v, (const float *)a.dout, a.lse, Dv,
                       (float *)a.dk, (float *)a.dv, a.Hq, a.Hkv, a.Nq, a.Nk, a.scale, n_ktiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace attn
