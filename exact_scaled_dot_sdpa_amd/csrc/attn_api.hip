// attn_api.hip -- the C ABI declared in include/attn.h: argument validation
// (before any HIP runtime call), workspace sizing and kernel dispatch.
#include "attn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace {

constexpr int DEFAULT_KEYS_PER_SPLIT = 256;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool supported_d(int d) { return d == 64 || d == 128; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

int effective_kps(int keys_per_split) {
    return keys_per_split == 0 ? DEFAULT_KEYS_PER_SPLIT : keys_per_split;
}

bool valid_kps(int kps) { return kps >= 64 && kps <= 65536 && kps % 64 == 0; }

long long n_splits_for(int max_seq_len, int kps) {
    const long long s = ((long long)max_seq_len + kps - 1) / kps;
    return s < 1 ? 1 : s;
}

// fp32 partial outputs [B,Hq,S,d], then (256-byte aligned) partial LSEs [B,Hq,S]
void workspace_layout(int B, int Hq, int d, long long S, size_t *o_bytes, size_t *total) {
    const size_t rows = (size_t)B * Hq * (size_t)S;
    size_t ob = rows * (size_t)d * sizeof(float);
    ob = (ob + 255) & ~(size_t)255;
    *o_bytes = ob;
    *total = ob + rows * sizeof(float);
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, float scale, int causal, int dtype, hipStream_t stream)
{
    if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || Nq == 0) return ATTN_OK;  // nothing to compute
    if (!q || !o) return ATTN_ERR_INVALID_ARG;
    if (Nk > 0 && (!k || !v)) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
        return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    // every index stays in 32-bit row counts: B*H*N rows, d columns
    if ((long long)B * Hq * Nq > 0x7fffffffLL || (long long)B * Hkv * Nk > 0x7fffffffLL)
        return ATTN_ERR_UNSUPPORTED;

    attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0};
    const hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, stream)
                                            : attn::launch_prefill_f32(a, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_seq_len, int d, int keys_per_split)
{
    const int kps = effective_kps(keys_per_split);
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 0 || !supported_d(d) || !valid_kps(kps))
        return 0;
    size_t ob, total;
    workspace_layout(B, Hq, d, n_splits_for(max_seq_len, kps), &ob, &total);
    return total;
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *o,
                float *lse, int B, int Hq, int Hkv, int max_seq_len, int d, float scale, int keys_per_split,
                int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    const int kps = effective_kps(keys_per_split);
    if (!valid_kps(kps)) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d) || dtype != ATTN_BF16 || !supported_group(Hq / Hkv)) return ATTN_ERR_UNSUPPORTED;
    if (B == 0) return ATTN_OK;
    if (!q || !o || !seq_lens || (max_seq_len > 0 && (!k_cache || !v_cache))) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(seq_lens, 4) || (k_cache && !aligned(k_cache, 16)) ||
        (v_cache && !aligned(v_cache, 16)))
        return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    const long long S = n_splits_for(max_seq_len, kps);
    if (S > 65535 || Hkv > 65535 || B > 65535) return ATTN_ERR_UNSUPPORTED;  // grid y/z limits
    if ((long long)B * Hkv * max_seq_len > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
    size_t ob, need;
    workspace_layout(B, Hq, d, S, &ob, &need);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;

    attn::DecodeArgs a{q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, max_seq_len, d, scale, kps, (int)S,
                       (float *)workspace, (float *)((char *)workspace + ob)};
    const hipError_t e = attn::launch_decode_bf16(a, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char *attn_status_str(int status)
{
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
        case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
        default: return "ATTN_ERR_UNKNOWN";
    }
}

}  // extern "C"
