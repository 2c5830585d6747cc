// kernels.h -- internal launch interface between the C-ABI layer (attn_api.hip)
// and the device kernels.  Not installed, not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Shapes already validated by the caller.
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, Nq, Nk, d;
    float scale;
    int causal;
};

struct DecodeArgs {
    const void *q, *k_cache, *v_cache;
    const int32_t *seq_lens;
    void *o;
    float *lse;
    int B, Hq, Hkv, Lmax, d;
    float scale;
    int keys_per_split;
    int n_splits;
    float *ws_o;    // [B, Hq, n_splits, d] fp32
    float *ws_lse;  // [B, Hq, n_splits] fp32
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16(const FwdArgs &a, hipStream_t stream);
hipError_t launch_prefill_f32(const FwdArgs &a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);

}  // namespace attn
