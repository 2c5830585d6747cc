// attn_api.hip -- the C ABI declared in include/attn.h: argument validation
// (before any HIP runtime call), workspace sizing and kernel dispatch.
#include "attn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

static_assert(attn::DECODE_SCRATCH_BYTES == ATTN_DECODE_NOALLOC_MAX_BYTES,
              "the header states the scratch array's size");

namespace {

// Upper bound on the workgroups of the decode split kernel; the default
// (keys_per_split == 0) uses two per CU for a contiguous cache and as many as
// the device holds at once for a paged one, at most this.
constexpr int DECODE_MAX_WG = 2048;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool supported_d(int d) { return d == 64 || d == 128; }

struct DecodePlan {
    int nhb;     // blocks of up to 16 query heads per K/V head
    int gb;      // heads per partial-result slot: min(G, 16)
    int n_wg;    // split-kernel workgroups (0 = device default)
    int max_wg;  // workgroups the workspace is sized for
    long long slots;
};

// Sizes are valid and non-negative here.
DecodePlan decode_plan(int B, int Hq, int Hkv, int max_seq_len, int keys_per_split) {
    DecodePlan p;
    const int G = Hq / Hkv;
    p.nhb = (G + 15) / 16;
    p.gb = G < 16 ? G : 16;
    if (keys_per_split > 0) {
        const long long keys = (long long)B * Hkv * p.nhb * max_seq_len;
        long long n = (keys + keys_per_split - 1) / keys_per_split;
        n = n < 1 ? 1 : (n > DECODE_MAX_WG ? DECODE_MAX_WG : n);
        p.n_wg = (int)n;
        p.max_wg = (int)n;
    } else {
        p.n_wg = 0;
        p.max_wg = DECODE_MAX_WG;
    }
    p.slots = (long long)B * Hkv * p.nhb + p.max_wg - 1;
    return p;
}

// fp32 partial outputs [slots, gb, d], then (256-byte aligned) partial LSEs
// [slots, gb], then (256-byte aligned) int32 per-range records [max_wg, 4]
void workspace_layout(const DecodePlan &p, int d, size_t *o_bytes, size_t *rec_off, size_t *total) {
    const size_t rows = (size_t)p.slots * p.gb;
    size_t ob = rows * (size_t)d * sizeof(float);
    ob = (ob + 255) & ~(size_t)255;
    *o_bytes = ob;
    const size_t ro = (ob + rows * sizeof(float) + 255) & ~(size_t)255;
    *rec_off = ro;
    *total = ro + (size_t)p.max_wg * 4 * sizeof(int32_t);
}

// Every size is at least 1 and query heads form whole groups.
bool fwd_sizes_ok(int B, int Hq, int Hkv, int Nq, int Nk) {
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && Nq >= 1 && Nk >= 1;
}

bool decode_sizes_ok(int B, int Hq, int Hkv, int max_seq_len) {
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && max_seq_len >= 1;
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, float scale, int causal, attn_dtype_t dtype, hipStream_t stream)
{
    if (!fwd_sizes_ok(B, Hq, Hkv, Nq, Nk)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    // every index stays in 32-bit row counts: B*H*N rows, d columns
    if ((long long)B * Hq * Nq > 0x7fffffffLL || (long long)B * Hkv * Nk > 0x7fffffffLL)
        return ATTN_ERR_UNSUPPORTED;

    attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0};
    const hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, stream)
                                            : attn::launch_prefill_f32(a, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, float v_scale, int causal, hipStream_t stream)
{
    if (!fwd_sizes_ok(B, Hq, Hkv, Nq, Nk)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale) || !isfinite(v_scale)) return ATTN_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * Nq > 0x7fffffffLL || (long long)B * Hkv * Nk > 0x7fffffffLL)
        return ATTN_ERR_UNSUPPORTED;
    attn::Fp8FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, v_scale, causal ? 1 : 0};
    return attn::launch_prefill_fp8(a, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq)
{
    if (B < 1 || Hq < 1 || Nq < 1) return 0;
    return (size_t)B * Hq * Nq * 2 * sizeof(float);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
             attn_dtype_t dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!fwd_sizes_ok(B, Hq, Hkv, Nq, Nk)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * Hq * Nq > 0x7fffffffLL || (long long)B * Hkv * Nk > 0x7fffffffLL)
        return ATTN_ERR_UNSUPPORTED;
    // every tensor the kernels touch must be present and aligned (q and do
    // are also read for dk / dv, k and v also for dq)
    const void *p16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : p16)
        if (!p || !aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
    if (!lse || !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;

    attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, (float *)workspace, B, Hq, Hkv, Nq, Nk, d, scale,
                    causal ? 1 : 0};
    const hipError_t e = dtype == ATTN_F32 ? attn::launch_bwd_f32(a, stream) : attn::launch_bwd_bf16(a, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_decode_split_workspace_bytes(int B, int Hq, int Hkv, int max_seq_len, int d, int keys_per_split)
{
    if (!decode_sizes_ok(B, Hq, Hkv, max_seq_len) || !supported_d(d) || keys_per_split < 0) return 0;
    size_t ob, ro, total;
    workspace_layout(decode_plan(B, Hq, Hkv, max_seq_len, keys_per_split), d, &ob, &ro, &total);
    return total;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_seq_len, int d)
{
    return attn_decode_split_workspace_bytes(B, Hq, Hkv, max_seq_len, d, 0);
}

}  // extern "C"

namespace {

// Shared body of the decode entry points; the paged cache passes
// block_table != nullptr and Lmax = max_blocks * block_size.  use_scratch:
// the partial results go to the library's device scratch array (workspace
// arguments ignored), after every check and only if they fit in it.
int decode_call(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *o, float *lse,
                int B, int Hq, int Hkv, int Lmax, int d, float scale, int keys_per_split, attn_dtype_t dtype,
                void *workspace, size_t workspace_bytes, hipStream_t stream, const int32_t *block_table,
                int block_size, int max_blocks, int num_blocks, bool use_scratch = false)
{
    if (!decode_sizes_ok(B, Hq, Hkv, Lmax)) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (keys_per_split < 0) return ATTN_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
    if (!q || !o || !seq_lens || !k_cache || !v_cache) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(seq_lens, 4) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16))
        return ATTN_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    const DecodePlan p = decode_plan(B, Hq, Hkv, Lmax, keys_per_split);
    // cache rows, segment counts and the kernels' sums of 64 sequence
    // lengths stay in 32-bit arithmetic
    const long long rows = block_table ? (long long)num_blocks * Hkv * block_size : (long long)B * Hkv * Lmax;
    const long long page_keys = (long long)(B < 64 ? B : 64) * Lmax;
    if (rows > 0x7fffffffLL || page_keys > 0x7fffffffLL || (long long)B * Hq > 0x7fffffffLL ||
        p.slots > 0x7fffffffLL)
        return ATTN_ERR_UNSUPPORTED;
    size_t ob, ro, need;
    workspace_layout(p, d, &ob, &ro, &need);
    if (use_scratch) {
        if (need > attn::DECODE_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
        if (attn::decode_scratch(&workspace) != hipSuccess) return ATTN_ERR_LAUNCH;
        workspace_bytes = attn::DECODE_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_ERR_WORKSPACE;

    attn::DecodeArgs a{q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, Lmax, d, scale,
                       p.nhb, p.n_wg, p.max_wg, (float *)workspace, (float *)((char *)workspace + ob),
                       (int32_t *)((char *)workspace + ro), block_table, block_size, max_blocks, num_blocks,
                       dtype == ATTN_F32 ? 1 : 0};
    const hipError_t e = attn::launch_decode(a, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *o,
                float *lse, int B, int Hq, int Hkv, int max_seq_len, int d, float scale, attn_dtype_t dtype,
                void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return decode_call(q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, max_seq_len, d, scale, 0, dtype,
                       workspace, workspace_bytes, stream, nullptr, 0, 0, 0);
}

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *o,
                        float *lse, int B, int Hq, int Hkv, int max_seq_len, int d, float scale, attn_dtype_t dtype,
                        hipStream_t stream)
{
    return decode_call(q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, max_seq_len, d, scale, 0, dtype, nullptr,
                       0, stream, nullptr, 0, 0, 0, true);
}

int attn_decode_split(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *o,
                      float *lse, int B, int Hq, int Hkv, int max_seq_len, int d, float scale, int keys_per_split,
                      attn_dtype_t dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return decode_call(q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, max_seq_len, d, scale, keys_per_split,
                       dtype, workspace, workspace_bytes, stream, nullptr, 0, 0, 0);
}

int attn_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                      const int32_t *seq_lens, void *o, float *lse, int B, int Hq, int Hkv, int num_blocks,
                      int block_size, int max_blocks_per_seq, int d, float scale, int keys_per_split,
                      attn_dtype_t dtype, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1) return ATTN_ERR_INVALID_ARG;
    const long long lmax = (long long)max_blocks_per_seq * block_size;
    if (lmax > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
    if (!block_table || !aligned(block_table, 4)) return ATTN_ERR_INVALID_ARG;
    return decode_call(q, k_pages, v_pages, seq_lens, o, lse, B, Hq, Hkv, (int)lmax, d, scale, keys_per_split,
                       dtype, workspace, workspace_bytes, stream, block_table, block_size, max_blocks_per_seq,
                       num_blocks);
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
