// decode_bf16.hip -- one-token decode against a bf16 KV cache (split-KV).
//
// Each query of the new token attends to the first seq_lens[b] cached rows of
// its K/V head ("Transformer 笔记：注意力机制为什么会变成系统问题", KV-cache
// section).  The work is HBM-bound (about 4 FLOP per cache byte), so the
// kernels are built around streaming the valid cache rows exactly once:
//
//   split kernel  grid (split, KV head, sequence).  A workgroup streams its
//                 split's K and V rows with 16-byte loads (a row of d bf16 is
//                 d/8 lanes), serves all G = Hq/Hkv query heads of the group
//                 from each row it loads, and keeps for every head the running
//                 reference m, denominator l and un-normalised accumulator of
//                 the online softmax ("从注意力到 IO 感知执行", sec. 8, eqs.
//                 (1)-(2)).  The reference is raised only when a score exceeds
//                 it by more than 2^8 (in base 2), which leaves u / l exact
//                 (the same sec. 8 notes that the subtracted value only changes
//                 the representation) and skips almost every rescale.  Lanes
//                 handling different keys merge their states at the end of the
//                 split; the split's normalised partial output and its
//                 log-sum-exp go to the workspace.
//   merge kernel  grid (sequence * query head): lse = ln sum_s exp(lse_s),
//                 o = sum_s exp(lse_s - lse) o_s, which is one more step of the
//                 same recurrence applied to whole splits.
//
// Cache rows at or beyond seq_lens[b] are never loaded.
#include "kernels.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHR = 256;
constexpr int NWAVE = 4;
constexpr int UNROLL = 4;        // key rows per lane per step
constexpr float RESCALE_TH = 8.f;  // raise the reference when a score exceeds it by 2^8
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
    const int xi = __builtin_bit_cast(int, x);
    int r;
    switch (ctrl_sel) {
        case 0: r = __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xf, 0xf, false); break;   // quad xor 1
        case 1: r = __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xf, 0xf, false); break;   // quad xor 2
        case 2: r = __builtin_amdgcn_mov_dpp(xi, 0x141, 0xf, 0xf, false); break;  // mirror within 8
        default: r = __builtin_amdgcn_mov_dpp(xi, 0x140, 0xf, 0xf, false); break; // mirror within 16
    }
    return __builtin_bit_cast(float, r);
}

// Sum over the CH lanes that hold one cache row (CH = 8 or 16, aligned groups).
template <int CH>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_f(x, 0);
    x += dpp_f(x, 1);
    x += dpp_f(x, 2);
    if (CH == 16) x += dpp_f(x, 3);
    return x;
}

// Dot product of 8 bf16 pairs (packed two per dword), fp32 accumulation.
// The dwords are copied to scalars before the bit cast: a bit cast applied
// directly to a subscripted ext_vector element is miscompiled by this clang
// (every subscript reads element 0).
__device__ __forceinline__ float dot8(u32x4 q, u32x4 k) {
    const uint32_t qa[4] = {q.x, q.y, q.z, q.w}, ka[4] = {k.x, k.y, k.z, k.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t qq = qa[i], kk = ka[i];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qq), __builtin_bit_cast(bf16x2, kk), s, false);
    }
    return s;
}

template <int D, int G>
__global__ __launch_bounds__(NTHR) void decode_split_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ Kc, const __bf16 *__restrict__ Vc,
    const int32_t *__restrict__ seq_lens, float *__restrict__ ws_o, float *__restrict__ ws_lse, int Hq,
    int Hkv, int Lmax, int kps, int n_splits, float sl2)
{
    constexpr int CH = D / 8;    // lanes per cache row
    constexpr int KW = 64 / CH;  // rows per wave-wide load
    __shared__ float s_acc[NWAVE][G][D];
    __shared__ float s_m[NWAVE][G];
    __shared__ float s_l[NWAVE][G];

    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int k_begin = split * kps;
    if (k_begin >= L) return;  // empty split: the merge kernel never reads it
    const int k_end = (k_begin + kps < L) ? k_begin + kps : L;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = lane / CH, ch = lane % CH;

    const size_t head_row0 = (size_t)(b * Hkv + hk) * Lmax;
    const __bf16 *Kh = Kc + head_row0 * D + ch * 8;
    const __bf16 *Vh = Vc + head_row0 * D + ch * 8;

    u32x4 qv[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
        qv[hh] = *reinterpret_cast<const u32x4 *>(Q + ((size_t)(b * Hq + hk * G + hh)) * D + ch * 8);

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }

    constexpr int WSTEP = UNROLL * KW;     // rows per wave per step
    constexpr int BSTEP = NWAVE * WSTEP;   // rows per workgroup per step
    for (int base = k_begin + wave * WSTEP; base < k_end; base += BSTEP) {
        u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int key = base + u * KW + sub;
            if (key < k_end) {
                kr[u] = *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D);
                vr[u] = *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D);
            } else {
                kr[u] = u32x4{};
                vr[u] = u32x4{};
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const bool valid = base + u * KW + sub < k_end;
            float vf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[2 * i] = __builtin_bit_cast(float, vr[u][i] << 16);
                vf[2 * i + 1] = __builtin_bit_cast(float, vr[u][i] & 0xffff0000u);
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float dsum = row_sum<CH>(dot8(qv[hh], kr[u]));
                const float sc = valid ? dsum * sl2 : -INFINITY;
                if (sc > m[hh] + RESCALE_TH) {  // raise the reference (rare)
                    const float alpha = __builtin_amdgcn_exp2f(m[hh] - sc);
                    l[hh] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
                    m[hh] = sc;
                }
                const float p = valid ? __builtin_amdgcn_exp2f(sc - m[hh]) : 0.f;
                l[hh] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p, vf[e], acc[hh][e]);
            }
        }
    }

    // merge the KW lane groups of this wave (they hold different rows)
#pragma unroll
    for (int x = CH; x < 64; x <<= 1) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float mp = __shfl_xor(m[hh], x, 64);
            const float lp = __shfl_xor(l[hh], x, 64);
            const float M = fmaxf(m[hh], mp);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            const float f = __builtin_amdgcn_exp2f(m[hh] - Mu);
            const float fp = __builtin_amdgcn_exp2f(mp - Mu);
            l[hh] = l[hh] * f + lp * fp;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ap = __shfl_xor(acc[hh][e], x, 64);
                acc[hh][e] = acc[hh][e] * f + ap * fp;
            }
            m[hh] = M;
        }
    }
    if (sub == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][hh][ch * 8 + e] = acc[hh][e];
            if (ch == 0) {
                s_m[wave][hh] = m[hh];
                s_l[wave][hh] = l[hh];
            }
        }
    }
    __syncthreads();

    // merge the waves and write this split's partial result
    for (int idx = tid; idx < G * D; idx += NTHR) {
        const int hh = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, s_m[w][hh]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][hh] - Mu);
            lt += s_l[w][hh] * f;
            ot += s_acc[w][hh][c] * f;
        }
        const size_t row = (size_t)(b * Hq + hk * G + hh) * n_splits + split;
        ws_o[row * D + c] = ot / lt;  // lt > 0: the split holds at least one valid row
        if (c == 0) ws_lse[row] = (Mu + __log2f(lt)) * LN2;
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse, const int32_t *__restrict__ seq_lens,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int Hq, int Lmax, int kps, int n_splits)
{
    const int bh = blockIdx.x;
    const int b = bh / Hq;
    const int c = threadIdx.x;
    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int ns = (L + kps - 1) / kps;
    const float *lse_s = ws_lse + (size_t)bh * n_splits;
    const float *o_s = ws_o + (size_t)bh * n_splits * D;
    float lse = -INFINITY, o = 0.f;
    if (ns > 0) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, lse_s[s]);
        float S = 0.f;
        for (int s = 0; s < ns; ++s) S += expf(lse_s[s] - M);
        lse = M + logf(S);
        for (int s = 0; s < ns; ++s) o = fmaf(expf(lse_s[s] - lse), o_s[(size_t)s * D + c], o);
    }
    O[(size_t)bh * D + c] = (__bf16)o;
    if (LSE && c == 0) LSE[bh] = lse;
}

template <int D, int G>
hipError_t launch_g(const DecodeArgs &a, hipStream_t stream) {
    const float sl2 = a.scale * LOG2E;
    hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(a.n_splits, a.Hkv, a.B), dim3(NTHR), 0, stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k_cache, (const __bf16 *)a.v_cache, a.seq_lens,
                       a.ws_o, a.ws_lse, a.Hq, a.Hkv, a.Lmax, a.keys_per_split, a.n_splits, sl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, stream, a.ws_o, a.ws_lse,
                       a.seq_lens, (__bf16 *)a.o, a.lse, a.Hq, a.Lmax, a.keys_per_split, a.n_splits);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_g<D, 1>(a, stream);
        case 2: return launch_g<D, 2>(a, stream);
        case 4: return launch_g<D, 4>(a, stream);
        case 8: return launch_g<D, 8>(a, stream);
        case 16: return launch_g<D, 16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.d == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace attn
