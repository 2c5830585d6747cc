/*
 * attn.h -- C ABI of libattn.so: exact scaled dot-product attention on MI355X
 * (gfx950), computed as one fused tiled kernel per call that never writes the
 * score matrix to device memory.
 *
 * The operation (pages cited by title and section):
 *   "Transformer 架构的数学与计算深度解析：注意力机制的详尽研究报告", sec. 2.2-2.4:
 *     S = scale * Q K^T, A = row softmax(S), O = A V (rows of A sum to one);
 *     sec. 4.1: the causal mask removes future keys (weight exactly zero);
 *     sec. 6.3: the online-softmax recurrence that lets the kernel stream K/V
 *     tiles while keeping only a running max, a denominator and an
 *     accumulator per query row.
 *   "从注意力到 IO 感知执行" (auturnal.com review), sec. 8, eqs. (1)-(2): the
 *     same recurrence with the un-normalised accumulator u and o = u / l.
 *   pwwt.cn engineering blog on Transformer algorithm evolution, sec. 2.3:
 *     grouped-query attention, where consecutive query heads share a K/V head.
 *   "Transformer 笔记：注意力机制为什么会变成系统问题" (imreese.github.io),
 *     KV-cache section: a decode step's single query reads the cached K/V.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing.  Its global state is a per-device cache of two
 *     device properties (compute-unit count, decode occupancy), written once
 *     on first use with the value the runtime reports, which never changes a
 *     result, and the fixed device array of attn_decode_noalloc (see there).
 *     Calls on different streams or threads may run concurrently, except
 *     attn_decode_noalloc calls on one device.
 *   - Tensors are contiguous, row-major, head dim innermost, 16-byte aligned
 *     (lse and seq_lens: 4-byte aligned).
 *   - Calls are asynchronous on `stream` (NULL = the null stream) and return
 *     after the launch is enqueued.
 *   - Arguments are validated before any HIP runtime call; an invalid call
 *     returns a non-zero status and enqueues nothing.  No C++ exception
 *     crosses this interface.
 *   - Every size (batch, heads, sequence lengths) must be >= 1.
 *   - LSE is the natural-log log-sum-exp of each row's visible scaled scores,
 *     fp32; a decode row that sees no key (seq_lens[b] == 0) has O = 0 and
 *     LSE = -inf.
 */
#ifndef EXACT_SDPA_ATTN_H
#define EXACT_SDPA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle type, declared as hip_runtime_api.h declares it.
 * Skipped when that header came first: C99 forbids repeating a typedef (C11
 * and C++ accept it, so there either include order works; in C99 include
 * hip_runtime_api.h first, or this header alone). */
#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t *hipStream_t;
#endif

/* Element type of q, k, v, o (and of the caches for decode). */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Status codes (every entry point returns one of these as an int). */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, non-finite scale */
    ATTN_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. d not 64/128) */
    ATTN_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
    ATTN_ERR_LAUNCH = 4       /* the HIP runtime reported an error at launch */
} attn_status_t;

/*
 * attn_fwd -- prefill / self- or cross-attention forward, MHA or GQA:
 * O = softmax(scale * Q K^T [+ causal mask]) V row by row ("Transformer 架构的
 * 数学与计算深度解析", sec. 2.2-2.4 for the operation, sec. 4.1 for the causal
 * mask; computed with the online recurrence of its sec. 6.3 and of "从注意力到
 * IO 感知执行", sec. 8, eqs. (1)-(2), never storing the score matrix).
 *
 *   q   [B, Hq,  Nq, d]   dtype          (read)
 *   k   [B, Hkv, Nk, d]   dtype          (read)
 *   v   [B, Hkv, Nk, d]   dtype          (read)
 *   o   [B, Hq,  Nq, d]   dtype          (written; bf16 is rounded to nearest even)
 *   lse [B, Hq,  Nq]      fp32 or NULL   (written when non-NULL)
 *
 * Query head h uses K/V head h / (Hq / Hkv) (contiguous groups).
 * scale multiplies q.k before masking and the softmax (1/sqrt(d) in the
 * usual case; any finite value is accepted).  The kernels form q.k and
 * scale * log2(e) * q.k in fp32, so the results hold while those stay finite
 * (|scale * q.k| below about 2.3e38); beyond that rows may read NaN.
 * causal != 0 masks key j for query row i when j > i + (Nk - Nq): the query
 * block is aligned with the END of the key sequence, so the last query row
 * sees every key (chunked prefill and decode agree with full causal prefill).
 * causal requires Nq <= Nk.
 *
 * Sizes: B, Hq, Hkv, Nq, Nk >= 1, Hq % Hkv == 0, d in {64, 128}, and
 * B * Hq * Nq, B * Hkv * Nk < 2^31 (ATTN_ERR_UNSUPPORTED beyond).  Every row
 * sees at least one key (causal: row i sees keys 0 .. i + Nk - Nq).  dtype is
 * ATTN_F32 or ATTN_BF16; accumulation is fp32 in both cases.
 *
 * Returns ATTN_OK, or ATTN_ERR_INVALID_ARG / ATTN_ERR_UNSUPPORTED (nothing
 * launched), or ATTN_ERR_LAUNCH.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_fwd_fp8 -- attn_fwd for q, k, v stored as fp8 (OCP e4m3, E4M3FN: 1
 * sign, 4 exponent, 3 mantissa bits, bias 7, no infinities), output bf16.
 *
 * FlashAttention-3 uses fp8 on Hopper (pwwt.cn engineering blog on
 * Transformer algorithm evolution, sec. 4.4); the same blog (sec. 7.2) warns
 * that fp8 is sensitive to quantisation, because scores that lose precision
 * before the softmax shift the attention distribution.  This call quantises
 * nothing beyond its inputs: the weights enter P V in bf16 as in attn_fwd and
 * V is widened to bf16 exactly.  The scores come from the fp8 matrix
 * instruction, whose products are exact but whose internal sums keep about
 * 16 significant bits (an absolute error up to ~2^-16 of the largest
 * 64-term dot product, measured on gfx950) instead of fp32's 24.  At
 * scale = 1/sqrt(d) the results meet attn_fwd's bf16 tolerances; the score
 * error grows with |scale * q.k|.
 *
 *   q [B, Hq, Nq, d], k / v [B, Hkv, Nk, d]   e4m3 bytes (read)
 *   o [B, Hq, Nq, d] bf16 (written), lse [B, Hq, Nq] fp32 or NULL
 *
 * O = v_scale * softmax(scale * Q K^T [+ causal mask]) V, where Q, K, V are
 * the stored e4m3 values: a caller holding fp8 tensors with dequantisation
 * factors sq, sk, sv passes scale = softmax_scale * sq * sk and v_scale = sv.
 * lse is that of the scaled scores.  Sizes, head mapping, causal alignment,
 * returns and errors as attn_fwd (v_scale must be finite).
 */
int attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                 float v_scale, int causal, hipStream_t stream);

/*
 * attn_bwd_workspace_bytes -- bytes of device workspace attn_bwd needs:
 * two fp32 per query row (B * Hq * Nq * 8).  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/*
 * attn_bwd -- backward pass of attn_fwd: the gradients of
 * O = softmax(scale * Q K^T [+ causal mask]) V with respect to q, k and v for
 * an upstream gradient dout of o.
 *
 * The pages say that training needs these gradients ("Transformer 架构的数学与
 * 计算深度解析", sec. 3.3) and that FlashAttention recomputes the weights
 * instead of storing them ("Transformer 深度进阶：从矩阵视角到 FlashAttention
 * 工程优化", the FlashAttention section); they print no formula.  The call
 * returns the chain-rule derivative of the definition: with
 * p_ij = exp(scale q_i.k_j - lse_i), D_i = dout_i . o_i, dp_ij = dout_i . v_j
 * and ds_ij = p_ij (dp_ij - D_i):
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dout_i,
 * sums over visible pairs only; for GQA, dk and dv of a K/V head sum over
 * every query head of its group.
 *
 *   q, o, dout [B, Hq, Nq, d]   dtype (read): o and lse are attn_fwd's outputs
 *   k, v       [B, Hkv, Nk, d]  dtype (read)     for the same q, k, v, scale,
 *   lse        [B, Hq, Nq] fp32       (read)     causal
 *   dq         [B, Hq, Nq, d]   dtype (written)
 *   dk, dv     [B, Hkv, Nk, d]  dtype (written)
 *   workspace  >= attn_bwd_workspace_bytes(B, Hq, Nq) bytes of caller-owned
 *              device memory, 16-byte aligned; contents on entry do not
 *              matter; calls that overlap in time must not share it.
 *
 * Sizes, head mapping, scale and causal alignment as attn_fwd.  With
 * dtype == ATTN_BF16, products take bf16 operands (the weights and ds
 * rounded to nearest even) with fp32 accumulation, and the gradients are
 * rounded to bf16; with ATTN_F32 every product and sum is fp32 (for
 * full-precision gradient checks).  The result is deterministic (no
 * atomics).
 *
 * Returns ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_WORKSPACE (nothing launched in these three cases) or
 * ATTN_ERR_LAUNCH.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o,
             const void *dout, const float *lse, void *dq, void *dk, void *dv,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, attn_dtype_t dtype, void *workspace,
             size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode needs
 * for these sizes: fp32 partial results of the split (see attn_decode),
 *   partial outputs [S, min(G, 16), d], then (from the next 256-byte
 *   boundary) partial LSEs [S, min(G, 16)], then (from the next 256-byte
 *   boundary) one record of four int32 per split workgroup [W, 4], which
 *   tells the merge which shared block ends in that workgroup's range,
 * with G = Hq / Hkv, W = 2048 and S = B * Hkv * ceil(G / 16) + W - 1 slots.
 * Returns 0 for sizes attn_decode would reject.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_seq_len,
                                   int d);

/*
 * attn_decode -- one decode step per sequence against a KV cache.
 *
 *   q        [B, Hq, d]                 dtype (read): the new token's queries
 *   k_cache  [B, Hkv, max_seq_len, d]   dtype (read)
 *   v_cache  [B, Hkv, max_seq_len, d]   dtype (read)
 *   seq_lens [B] int32, device          (read): rows 0..seq_lens[b]-1 of
 *            sequence b are valid; values are clamped to [0, max_seq_len].
 *            Rows at or beyond seq_lens[b] are never read.
 *   o        [B, Hq, d]                 dtype (written)
 *   lse      [B, Hq] fp32 or NULL       (written when non-NULL)
 *   workspace / workspace_bytes: caller-owned device scratch of at least
 *            attn_decode_workspace_bytes(...) bytes, 16-byte aligned; its
 *            contents on entry do not matter.  Two calls that overlap in time
 *            must not share one workspace.
 *
 * Query head h of sequence b attends, without a mask, to the first
 * seq_lens[b] rows of K/V head h / (Hq / Hkv) ("Transformer 笔记：注意力机制为
 * 什么会变成系统问题", KV-cache section: the new token's query reads the
 * cached keys and values); this equals the last row of causal attn_fwd over
 * those rows.  The cache is not appended to.  The valid keys of all
 * (sequence, K/V head, block of 16 query heads) are laid end to end and cut
 * into equal ranges, one per workgroup, two per compute unit (fewer if the
 * device holds fewer at once; attn_decode_paged: as many as it holds);
 * the partial results of blocks that several ranges share are merged through
 * their log-sum-exps ("从注意力到 IO 感知执行", sec. 8, eqs. (1)-(2), applied
 * to whole ranges).  A sequence with seq_lens[b] == 0 gets O = 0 and
 * LSE = -inf.  dtype is ATTN_BF16 (the weights enter P V rounded to bf16)
 * or ATTN_F32 (fp32 products and weights throughout); accumulation is fp32
 * in both cases.  Any Hq / Hkv is supported.
 *
 * Sizes: B, Hq, Hkv, max_seq_len >= 1, Hq % Hkv == 0, d in {64, 128},
 * B * Hkv * max_seq_len < 2^31.
 * Returns ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_WORKSPACE (nothing launched in these three cases) or
 * ATTN_ERR_LAUNCH.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *seq_lens, void *o, float *lse, int B, int Hq,
                int Hkv, int max_seq_len, int d, float scale,
                attn_dtype_t dtype, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * attn_decode_split_workspace_bytes / attn_decode_split -- attn_decode with
 * an explicit split: keys_per_split > 0 asks for ranges of about that many
 * keys of the max_seq_len-sized cache, i.e. W = ceil(B * Hkv * ceil(G / 16) *
 * max_seq_len / keys_per_split) workgroups clamped to [1, 2048];
 * keys_per_split == 0 is the default of attn_decode (two workgroups per
 * compute unit) or attn_decode_paged (as many as the device holds at once).
 * The workspace then has S = B * Hkv * ceil(G / 16) + W - 1 slots and W
 * records (W = 2048 for keys_per_split == 0), laid out as for attn_decode.  Everything else is
 * attn_decode's.  The result is the same up to the order of floating-point
 * sums (split invariance).
 */
size_t attn_decode_split_workspace_bytes(int B, int Hq, int Hkv,
                                         int max_seq_len, int d,
                                         int keys_per_split);
int attn_decode_split(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *seq_lens, void *o, float *lse, int B,
                      int Hq, int Hkv, int max_seq_len, int d, float scale,
                      int keys_per_split, attn_dtype_t dtype, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, result and errors are attn_decode's, with no
 * workspace: the split's partial results go to a device array inside the
 * library, ATTN_DECODE_NOALLOC_MAX_BYTES (32 MiB) on each device the library
 * runs on, held until the process ends.  Sizes whose
 * attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, d) exceeds it return
 * ATTN_ERR_WORKSPACE (nothing launched).  The call allocates nothing; its
 * first call on a device looks the array's address up (hipGetSymbolAddress)
 * and keeps it.  Every call on one device shares that array: two calls that
 * overlap in time on one device (different streams or threads) race and give
 * undefined results; calls ordered on one stream are safe.  Nothing in the
 * array needs to start at zero.
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *seq_lens, void *o,
                        float *lse, int B, int Hq, int Hkv, int max_seq_len,
                        int d, float scale, attn_dtype_t dtype,
                        hipStream_t stream);

/*
 * attn_decode_paged -- attn_decode against a paged KV cache: each sequence's
 * cached rows live in fixed-size blocks anywhere in a pool, found through a
 * block table ("Transformer 笔记：注意力机制为什么会变成系统问题", the
 * FlashAttention / PagedAttention section; the pwwt.cn engineering blog,
 * sec. 3.3).
 *
 *   k_pages, v_pages [num_blocks, Hkv, block_size, d]  dtype (read): the pool
 *   block_table      [B, max_blocks_per_seq] int32, device (read): logical
 *            block j of sequence b is pool block block_table[b][j]; entries
 *            outside [0, num_blocks) are clamped into it (no fault, no error).
 *            Only row b of the table is read for sequence b, and only the
 *            entries of its valid blocks are used.
 *   seq_lens [B] int32, device: clamped to [0, max_blocks_per_seq *
 *            block_size]; rows at or beyond seq_lens[b] are never read
 *   q, o, lse, scale, dtype, stream: as for attn_decode.
 *   keys_per_split: as for attn_decode_split (0 = the default split).
 *   workspace: as for attn_decode, sized by attn_decode_split_workspace_bytes(
 *            B, Hq, Hkv, max_blocks_per_seq * block_size, d, keys_per_split).
 *
 * Blocks may be shared between sequences (shared prefixes).  block_size is
 * any positive value; a multiple of 32 keeps every 32-key chunk whole.
 * Sizes: num_blocks, block_size, max_blocks_per_seq >= 1,
 * max_blocks_per_seq * block_size < 2^31, num_blocks * Hkv * block_size < 2^31,
 * min(B, 64) * max_blocks_per_seq * block_size < 2^31; otherwise as for
 * attn_decode.
 */
int attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                      const int32_t *block_table, const int32_t *seq_lens,
                      void *o, float *lse, int B, int Hq, int Hkv,
                      int num_blocks, int block_size, int max_blocks_per_seq,
                      int d, float scale, int keys_per_split,
                      attn_dtype_t dtype, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_SDPA_ATTN_H */
