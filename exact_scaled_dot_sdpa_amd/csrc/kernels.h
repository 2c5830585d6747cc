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
    int nhb;        // blocks of up to 16 query heads per K/V head: ceil(G / 16)
    int n_wg;       // workgroups of the split kernel; 0 = the default (two per CU; paged: occupancy)
    int max_wg;     // workgroups the workspace has partial-result slots for
    float *ws_o;    // [B*Hkv*nhb + max_wg - 1 slots, min(G, 16) heads, d] fp32
    float *ws_lse;  // [slots, min(G, 16)] fp32
    int32_t *ws_rec;  // [max_wg, 4] per range: the shared segment whose last piece it holds (or -1),
                      // that segment's first range, the batch's key count (low, high 32 bits)
    // paged cache (block_table != nullptr): k_cache / v_cache are a pool
    // [num_blocks, Hkv, block_size, d], Lmax = max_blocks * block_size
    const int32_t *block_table;  // [B, max_blocks]
    int block_size, max_blocks, num_blocks;
    int f32;  // q, the caches and o are fp32 (else bf16)
};

struct Fp8FwdArgs {
    const void *q, *k, *v;  // OCP e4m3 (E4M3FN) bytes
    void *o;                // bf16
    float *lse;
    int B, Hq, Hkv, Nq, Nk, d;
    float scale, v_scale;
    int causal;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *ws_d;  // [2, B*Hq*Nq] fp32: do_i . o_i, then lse_i * log2(e), per row (fp32: the first half only)
    int B, Hq, Hkv, Nq, Nk, d;
    float scale;
    int causal;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_prefill_bf16(const FwdArgs &a, hipStream_t stream);
hipError_t launch_prefill_f32(const FwdArgs &a, hipStream_t stream);
hipError_t launch_prefill_fp8(const Fp8FwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs &a, hipStream_t stream);

// Compute units of the current device (queried once per device, cached).
hipError_t device_cu_count(int *out);

// Size of the decode kernels' file-scope device scratch array, which serves
// callers that cannot allocate (attn_decode_noalloc).
constexpr size_t DECODE_SCRATCH_BYTES = size_t(32) << 20;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress and kept).
hipError_t decode_scratch(void **out);

}  // namespace attn
