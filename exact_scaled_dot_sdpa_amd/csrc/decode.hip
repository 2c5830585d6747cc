// decode.hip -- one-token decode against a bf16 or fp32 KV cache.
//
// Each query of the new token attends to the first seq_lens[b] cached rows of
// its K/V head ("Transformer 笔记：注意力机制为什么会变成系统问题", KV-cache
// section).  The work is HBM-bound (about 4 FLOP per cache byte for four query
// heads per K/V head), so the design streams every valid cache row exactly
// once, keeps enough of them in flight to cover the memory latency, and keeps
// the per-byte instruction count low enough that the vector ALUs never become
// the limit.
//
// Work partition.  A (sequence b, K/V head hk, block hb of up to 16 query heads
// of the group) is one "segment" of seq_lens[b] keys; the segments are laid
// end to end (b outer, then hk, then hb) into one list of T keys, which is cut
// into n_wg equal ranges, one per single-wave workgroup.  With n_wg a whole
// multiple of the CU count that the chip holds at once (by default two per CU
// for a contiguous cache, three -- the occupancy limit -- for a paged one),
// every workgroup streams the same number of bytes whatever the length mix
// of the batch, and every CU the same number of workgroups.  A range that
// covers a whole segment writes its output rows directly.  A range that
// covers part of a segment writes a partial result (normalised output and
// log-sum-exp of its keys) to the workspace; a second kernel merges the
// partials of each shared segment, which is one more step of the
// online-softmax recurrence ("从注意力到 IO 感知执行", sec. 8, eqs. (1)-(2))
// applied to whole ranges.  Every workgroup computes the segment prefix sums
// itself from seq_lens (a 64-lane scan per 64 sequences); no planning kernel
// runs first.
//
// gfx950 mapping inside a workgroup (one wave):
//   * The range is walked in chunks of 32 keys (fewer at the end of a segment
//     or range).  The K and V rows of a chunk, and the query rows of its
//     segment, go from HBM straight into LDS with buffer_load ... lds (1 KB per
//     instruction); a ring of NST stages keeps NST-1 chunks in flight while one
//     is computed.  Each stage is its own LDS array, which lets the compiler
//     see that a stage's reads wait only for that stage's loads (with one
//     array it waits for every load in flight before each read).  The buffer descriptor of each load ends at the last valid
//     row, so rows at or beyond seq_lens[b] are never read: the hardware range
//     check returns zeros for them.
//   * Scores S = K Q^T on v_mfma_f32_16x16x32_bf16: the 16 keys of a half-chunk
//     are the M dimension and the (up to 16) query heads the N dimension, so
//     each lane ends up with 4 scores of one head; no cross-lane reduction is
//     needed for the dot products.
//   * Softmax in base 2 with a lazily raised reference, as in the prefill
//     kernel: the first chunk of a range sets the reference to its maximum;
//     later chunks only check that their probabilities stay below 2^24 and
//     rescale in the rare case they do not.
//   * P^T (bf16, in registers, exactly the B-operand layout) times V^T: the
//     A operand is read from the row-major V chunk with ds_read_b64_tr_b16,
//     so no transposed copy is stored.  O^T accumulates in 8 (d = 128) or 4
//     (d = 64) 16x16 fp32 tiles.
//   * LDS rows are XOR-swizzled per 16-byte chunk so that both operand reads
//     are free of bank conflicts.
//
// fp32 caches (full-precision checks) take the same walk, ring and merge with
// fp32 products throughout: the scores and P V run on
// v_mfma_f32_16x16x4_f32, whose 16 x 16 result has the layout of the bf16
// kernel's (lane: 4 keys of one head), so the softmax code is shared.  For the
// scores each lane reads 4 consecutive d-values of its key (A) and of its head
// (B) with one ds_read_b128 and feeds them to 4 MFMAs (the d-order of a dot
// product is free).  P stays fp32 (no bf16 rounding anywhere); the V^T
// operand of key 16 t + 4 g + i is read row-wise, 4 columns per lane and
// ds_read_b128, and the 16 x 16 output blocks cover the columns in the order
// that this read gives (block 4 h + e, row m <-> column 64 h + 4 m + e).
#include "kernels.h"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace attn {
namespace {

constexpr int CACHE_NT = 2;  // buffer-load cache-policy bit: non-temporal (streamed once)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int CK = 32;  // keys per chunk
#ifndef ATTN_DECODE_STAGES
#define ATTN_DECODE_STAGES 3
#endif
constexpr int DECODE_STAGES = ATTN_DECODE_STAGES;  // LDS ring depth (chunks)
static_assert(DECODE_STAGES >= 2 && DECODE_STAGES <= 4, "pipeline depth");
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
// A chunk whose (per lane, 8) probabilities sum above 2^24 raises the
// reference; below it every p <= 2^24 and fp32 keeps its relative precision.
constexpr float RESCALE_SUM = 16777216.f;

// ET: element type of q, the caches and o (__bf16 or float).
template <typename ET, int D>
struct DC {
    static constexpr bool F32 = sizeof(ET) == 4;
    static constexpr int ROWB = D * (int)sizeof(ET);  // bytes per row
    static constexpr int CH = ROWB / 16;             // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;              // rows per 1 KB load instruction
    static constexpr int KI = CK / RPI;              // load instructions per K (or V) chunk
    static constexpr int PER = 16 / RPI;             // instructions after which the swizzle repeats
    static constexpr int KS = D / 32;                // k-steps of the bf16 score MFMA
    static constexpr int CB = D / 16;                // 16-column blocks of O^T
    static constexpr int CHUNK_BYTES = CK * ROWB;    // one K or V chunk
};

// Stage layout in LDS: K chunk, V chunk, query rows of the chunk's segment.
template <typename ET, int D, int QR>
struct Stage {
    using C = DC<ET, D>;
    static constexpr int QROWS = (QR + C::RPI - 1) / C::RPI * C::RPI;
    static constexpr int QI = QROWS / C::RPI;  // load instructions for the query rows
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = C::CHUNK_BYTES;
    static constexpr int Q_OFF = 2 * C::CHUNK_BYTES;
    static constexpr int BYTES = Q_OFF + QROWS * C::ROWB;
    static constexpr int NI = 2 * C::KI + QI;  // load instructions per chunk
    static_assert(BYTES % 1024 == 0, "stage alignment");
    static_assert((QROWS & (QROWS - 1)) == 0 && QROWS <= 16, "query rows: power of two up to 16");
};

// XOR swizzles of the 16-byte chunk index within a row (see the operand reads
// for the access patterns they serve).  fp32 rows (16 or 32 chunks): 16
// consecutive rows read at one chunk index land on 16 different 16-byte bank
// slots, and so do the 16 lanes that read chunks 0..15 (+16 h) of one row.
template <typename ET, int D> __device__ __forceinline__ int swz_k(int row) {
    if constexpr (sizeof(ET) == 4) return row & 15;
    else if constexpr (D == 128) return row & 15;
    else return (row >> 1) & 7;
}
template <typename ET, int D> __device__ __forceinline__ int swz_v(int row) {
    if constexpr (sizeof(ET) == 4) return row & 15;
    else if constexpr (D == 128) return (row & 7) << 1;
    else return ((row >> 1) & 3) << 1;
}

__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Sum of x over the wave (every lane gets it).
__device__ __forceinline__ int wave_total(int x, int lane) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x, lane), 63);
}

// Lengths of the 8 pages of 64 sequences from p8 (lane i: sequence
// p8 + 64 k + i in Lg[k]; 0 past the batch), all loads issued before any is
// used, so the 8 pages cost one memory round trip.
__device__ __forceinline__ void load_pages8(int (&Lg)[8], const int32_t *__restrict__ seq_lens, int p8, int B,
                                            int Lmax, int lane) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const long long idx = (long long)p8 + 64 * k + lane;
        Lg[k] = idx < B ? seq_lens[idx] : 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) Lg[k] = clamp_len(Lg[k], Lmax);
}

// Round-to-nearest-even pair conversion fp32 -> packed bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// First key position of workgroup w's range: floor(w * T / n_wg).
__device__ __forceinline__ long long range_start(long long w, long long T, int n_wg) { return w * T / n_wg; }

// Loads of one chunk into a stage: K and V rows (kv_bytes of them are in
// range, the rest of the chunk reads as zeros) and the query rows of the
// segment (q_bytes in range).  voff_*: per-lane byte offsets within a 1 KB
// load, one per swizzle phase.
template <typename ET, int D, int QR>
__device__ __forceinline__ void dma_chunk(char *dst, const ET *k, const ET *v, const ET *q, int kv_bytes, int q_bytes,
                                          const int (&voff_k)[DC<ET, D>::PER],
                                          const int (&voff_v)[DC<ET, D>::PER]) {
    using C = DC<ET, D>;
    using S = Stage<ET, D, QR>;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)k, (short)0, kv_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)v, (short)0, kv_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)q, (short)0, q_bytes, 0x00020000);
    // Every cache row is read exactly once: the K/V loads carry the
    // non-temporal hint (aux bit 1, `nt`), so the stream does not displace
    // other data in L2 / MALL (decode alone 40 -> 35.7 us on the 16-sequence
    // workload, and 48 -> 40 us right after a prefill that left its output
    // dirty in the caches).
#pragma unroll
    for (int i = 0; i < C::KI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(dst + S::K_OFF + i * 1024), 16, voff_k[i % C::PER],
                                                 i * 1024, 0, CACHE_NT);
#pragma unroll
    for (int i = 0; i < C::KI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dst + S::V_OFF + i * 1024), 16, voff_v[i % C::PER],
                                                 i * 1024, 0, CACHE_NT);
#pragma unroll
    for (int i = 0; i < S::QI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(dst + S::Q_OFF + i * 1024), 16, voff_k[i % C::PER],
                                                 i * 1024, 0, 0);
}

// Merge of one segment's partial results (one wave): lse = ln sum_w
// exp(lse_w), o = sum_w exp(lse_w - lse) o_w over the workgroups w0..w1 with
// a non-empty range, i.e. one more step of the online-softmax recurrence
// applied to whole key ranges.  Writes the gblk output rows from head0.
template <typename OT, int D>
__device__ void merge_segment(const float *ws_o, const float *ws_lse, OT *O, float *LSE, int seg, int w0, int w1,
                              size_t head0, int gblk, int GB, long long T, int n_wg, int lane) {
    constexpr int C4 = D / 4;  // float4 groups per output row
    constexpr int RO = 2;      // outputs (float4) per lane per round
    constexpr int PB = 6;      // pieces whose loads are in flight together
    const int nout = gblk * C4;
    for (int base = 0; base < nout; base += 64 * RO) {
        int h[RO], c4[RO];
        bool act[RO];
        float M[RO], sum[RO];
        f32x4 o[RO];
#pragma unroll
        for (int r = 0; r < RO; ++r) {
            const int idx = base + 64 * r + lane;
            act[r] = idx < nout;
            h[r] = act[r] ? idx / C4 : 0;
            c4[r] = act[r] ? idx - h[r] * C4 : 0;
            M[r] = -INFINITY;
            sum[r] = 0.f;
            o[r] = f32x4{};
        }
        for (int wb = w0; wb <= w1; wb += PB) {
            float l[PB][RO];
            f32x4 ov[PB][RO];
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                const int wg = wb + j;
                const bool ok = wg <= w1 && (T >= n_wg || range_start(wg, T, n_wg) < range_start(wg + 1, T, n_wg));
#pragma unroll
                for (int r = 0; r < RO; ++r) {
                    l[j][r] = -INFINITY;
                    ov[j][r] = f32x4{};
                }
                if (ok) {  // uniform
                    const size_t slot = (size_t)seg + wg;
#pragma unroll
                    for (int r = 0; r < RO; ++r) {
                        l[j][r] = ws_lse[slot * GB + h[r]];
                        ov[j][r] = *reinterpret_cast<const f32x4 *>(ws_o + (slot * GB + h[r]) * D + 4 * c4[r]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < PB; ++j) {
#pragma unroll
                for (int r = 0; r < RO; ++r) {
                    if (l[j][r] == -INFINITY) continue;  // absent piece (a present one has a finite lse)
                    if (l[j][r] > M[r]) {
                        const float sc = __expf(M[r] - l[j][r]);
                        sum[r] *= sc;
                        o[r] *= sc;
                        M[r] = l[j][r];
                    }
                    const float e = __expf(l[j][r] - M[r]);
                    sum[r] += e;
                    o[r] += e * ov[j][r];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RO; ++r) {
            if (!act[r]) continue;
            const f32x4 res = o[r] * (1.f / sum[r]);
            if constexpr (sizeof(OT) == 4)
                *reinterpret_cast<f32x4 *>(O + (head0 + h[r]) * D + 4 * c4[r]) = res;
            else
                *reinterpret_cast<bf16x4 *>(O + (head0 + h[r]) * D + 4 * c4[r]) = __builtin_convertvector(res, bf16x4);
            if (LSE && c4[r] == 0) LSE[head0 + h[r]] = M[r] + __logf(sum[r]);
        }
    }
}

// block_table != nullptr (paged cache): Kc / Vc are a pool
// [num_blocks, Hkv, bs, d] and row j of sequence b lives in block
// block_table[b * max_blocks + j / bs] (entries clamped to the pool), row
// j % bs; otherwise Kc / Vc are [B, Hkv, Lmax, d].
template <typename ET, int D, int QR, int NST>
__global__ __launch_bounds__(64) void decode_chunk_kernel(
    const ET *__restrict__ Q, const ET *__restrict__ Kc, const ET *__restrict__ Vc, const int32_t *__restrict__ seq_lens,
    ET *__restrict__ O, float *__restrict__ LSE, float *__restrict__ ws_o, float *__restrict__ ws_lse,
    int32_t *__restrict__ ws_rec, int B, int Hq, int Hkv, int Lmax, int nhb, int n_wg, float sl2,
    const int32_t *__restrict__ block_table, int bs, int max_blocks, int num_blocks)
{
    using C = DC<ET, D>;
    using S = Stage<ET, D, QR>;
    // one LDS array per stage: the compiler then knows which in-flight
    // LDS-DMA a stage's reads depend on instead of waiting for all of them
    __shared__ __attribute__((aligned(1024))) char lds0[S::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[S::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds2[NST > 2 ? S::BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char lds3[NST > 3 ? S::BYTES : 16];
    auto stage = [&](int st) { return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : lds3; };

    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    const int G = Hq / Hkv;
    const int GB = G < 16 ? G : 16;  // heads per partial-result slot
    const int nsub = Hkv * nhb;      // segments per sequence

    // ---- this workgroup's key range [a0, a1) -----------------------------
    // The first page of 64 sequence lengths serves both the total and the
    // search, so a batch of up to 64 sequences costs one memory round trip.
    // Larger batches load the other pages eight at a time (one round trip
    // per 512 sequences), for the total and again, up to the page that holds
    // the range's first key, for the search.  A page's sum fits in 32 bits
    // (the boundary bounds 64 * max_seq_len); the batch's sum is 64-bit.
    int pageL = lane < B ? clamp_len(seq_lens[lane], Lmax) : 0;
    int incl = wave_incl_scan(pageL, lane);
    long long T = __builtin_amdgcn_readlane(incl, 63);
    for (int p8 = 64; p8 < B; p8 += 512) {
        int Lg[8];
        load_pages8(Lg, seq_lens, p8, B, Lmax, lane);
#pragma unroll
        for (int k = 0; k < 8; ++k) T += wave_total(Lg[k], lane);
    }
    T *= nsub;
    // this range's record for the merge kernel: no shared segment ends in it
    // (rewritten below by the range that holds a shared segment's last piece)
    if (lane == 0) *reinterpret_cast<i32x4 *>(ws_rec + 4 * w) = i32x4{-1, 0, 0, 0};
    // sequences with no visible key (seq_len 0) get O = 0 and LSE = -inf from
    // workgroup b mod n_wg (no range ever reaches them); lane i checks
    // sequence w + i n_wg, so one pass covers 64 of this workgroup's
    for (long long base = w; base < B; base += 64LL * n_wg) {
        const long long bz = base + (long long)lane * n_wg;
        const int from_page = __shfl(pageL, (int)(bz & 63), 64);
        int L = 1;
        if (bz < B) L = bz < 64 ? from_page : clamp_len(seq_lens[bz], Lmax);
        unsigned long long zero = __builtin_amdgcn_ballot_w64(L == 0);
        while (zero) {
            const long long bzz = base + (long long)__builtin_ctzll(zero) * n_wg;
            zero &= zero - 1;
            char *dst = reinterpret_cast<char *>(O + (size_t)bzz * Hq * D);
            for (int i = lane; i < Hq * C::ROWB / 16; i += 64) *reinterpret_cast<u32x4 *>(dst + 16 * i) = u32x4{};
            if (LSE)
                for (int i = lane; i < Hq; i += 64) LSE[(size_t)bzz * Hq + i] = -INFINITY;
        }
    }
    const long long a0 = range_start(w, T, n_wg), a1 = range_start(w + 1, T, n_wg);
    if (a0 >= a1) return;

    // locate a0: sequence b (page pb, lane f), segment sub, key; bstart is the
    // position of sequence b's first key in the batch list
    int pb = 0, f = 0;
    long long bstart = 0;
    {
        unsigned long long hit = __builtin_amdgcn_ballot_w64((long long)incl * nsub > a0);
        if (!hit) {
            bstart = (long long)__builtin_amdgcn_readlane(incl, 63) * nsub;
            bool found = false;
            for (int p8 = 64; p8 < B && !found; p8 += 512) {
                int Lg[8];
                load_pages8(Lg, seq_lens, p8, B, Lmax, lane);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (!found) {  // uniform
                        const long long tot = (long long)wave_total(Lg[k], lane) * nsub;
                        if (bstart + tot > a0) {
                            found = true;
                            pb = p8 + 64 * k;
                            pageL = Lg[k];
                        } else {
                            bstart += tot;
                        }
                    }
                }
            }
            // a0 < T, so some page holds it; lengths that changed between the
            // two reads (a caller's race) end the walk instead of running on
            if (!found) return;
            incl = wave_incl_scan(pageL, lane);
            hit = __builtin_amdgcn_ballot_w64(bstart + (long long)incl * nsub > a0);
            if (!hit) return;
        }
        f = __builtin_ctzll(hit);
        bstart += (long long)(__builtin_amdgcn_readlane(incl, f) - __builtin_amdgcn_readlane(pageL, f)) * nsub;
    }
    int b = pb + f;
    int Lb = __builtin_amdgcn_readlane(pageL, f);
    int sub, key;
    {
        const long long off = a0 - bstart;
        sub = (int)(off / Lb);
        key = (int)(off - (long long)sub * Lb);
    }
    long long pos = a0;
    bool piece_start = true;

    // ---- scale: positive factor sl2 (negative scale: negate Q) ------------
    const bool neg = sl2 < 0.f;
    sl2 = neg ? -sl2 : sl2;
    sl2 = sl2 < 1e-30f ? 1e-30f : sl2;

    // ---- DMA lane offsets (bytes within one 1 KB load) --------------------
    const int ld_q = lane / C::CH, ld_p = lane % C::CH;
    int voff_k[C::PER], voff_v[C::PER];
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
        const int R = i * C::RPI + ld_q;
        voff_k[i] = ld_q * C::ROWB + ((ld_p ^ swz_k<ET, D>(R)) * 16);
        voff_v[i] = ld_q * C::ROWB + ((ld_p ^ swz_v<ET, D>(R)) * 16);
    }

    // per-stage chunk records (wave-uniform): segment, key count, heads,
    // first / last chunk of this range's piece of the segment, the first and
    // last workgroup whose range touches the segment, first output row
    int m_seg[NST], m_cnt[NST], m_gblk[NST], m_w0[NST], m_w1[NST], m_head0[NST];
    bool m_first[NST], m_last[NST];
    int cur_w0 = 0, cur_w1 = 0;  // of the segment the cursor is in

    // paged cache: a page of 64 block-table entries of sequence bt_b, one per
    // lane, reloaded when the cursor leaves it
    int bt_b = -1, bt_base = 0, bt_page = 0;
    auto phys_block = [&](int lb) {
        if (b != bt_b || lb < bt_base || lb >= bt_base + 64) {
            bt_b = b;
            bt_base = lb & ~63;
            const int idx = bt_base + lane;
            bt_page = idx < max_blocks ? block_table[(size_t)b * max_blocks + idx] : 0;
        }
        const int p = __builtin_amdgcn_readlane(bt_page, lb - bt_base);
        return p < 0 ? 0 : (p > num_blocks - 1 ? num_blocks - 1 : p);
    };

    // Issue the loads of the next chunk of the range into stage st and
    // advance the cursor; false (nothing issued) once the range is done.
    auto issue = [&](const int st) {
        if (pos >= a1) return false;
        const long long left = a1 - pos;
        int cnt = Lb - key;
        cnt = cnt < CK ? cnt : CK;
        cnt = left < cnt ? (int)left : cnt;
        if (cnt <= 0) {  // cannot happen for a consistent walk; ends it rather than spin
            pos = a1;
            return false;
        }
        const int hk = sub / nhb, hb = sub - hk * nhb;
        const int gblk = G - 16 * hb < 16 ? G - 16 * hb : 16;
        if (piece_start) {
            const long long S0 = bstart + (long long)sub * Lb, S1 = S0 + Lb;
            cur_w0 = (int)(((S0 + 1) * n_wg - 1) / T);
            cur_w1 = (int)((S1 * n_wg - 1) / T);
        }
        size_t row0;
        if (block_table) {  // paged: a chunk never crosses a block
            const int lb = key / bs, off = key - lb * bs;
            cnt = cnt < bs - off ? cnt : bs - off;
            row0 = ((size_t)phys_block(lb) * Hkv + hk) * bs + off;
        } else {
            row0 = (size_t)(b * Hkv + hk) * Lmax + key;
        }
        dma_chunk<ET, D, QR>(stage(st), Kc + row0 * D, Vc + row0 * D, Q + ((size_t)b * Hq + hk * G + 16 * hb) * D,
                            cnt * C::ROWB, gblk * C::ROWB, voff_k, voff_v);
        m_seg[st] = b * nsub + sub;
        m_cnt[st] = cnt;
        m_gblk[st] = gblk;
        m_w0[st] = cur_w0;
        m_w1[st] = cur_w1;
        m_head0[st] = b * Hq + hk * G + 16 * hb;
        m_first[st] = piece_start;
        m_last[st] = (key + cnt == Lb) || (pos + cnt == a1);
        // advance
        piece_start = false;
        key += cnt;
        pos += cnt;
        if (key == Lb && pos < a1) {
            key = 0;
            piece_start = true;
            if (++sub == nsub) {
                sub = 0;
                do {  // next non-empty sequence (one exists: pos < a1)
                    bstart += (long long)Lb * nsub;
                    ++b;
                    if (++f == 64) {
                        f = 0;
                        pb += 64;
                        pageL = pb + lane < B ? clamp_len(seq_lens[pb + lane], Lmax) : 0;
                    }
                    Lb = __builtin_amdgcn_readlane(pageL, f);
                } while (Lb == 0 && b + 1 < B);
            }
        }
        return true;
    };

    // ---- operand read offsets (bytes), fixed for the kernel --------------
    const int n = lane & 15, g = lane >> 4;
    const int qn = n & (S::QROWS - 1);  // Q slot row read by this lane (lanes past QROWS get zeros)
    // bf16.  K (A operand, m = key n of a 16-key half) and Q (B operand, n =
    // head): row n, chunk 4 kk + g; a half-chunk t adds 16 rows (same
    // swizzle).  V (transposing reads): a 16-lane group g reads keys 4g ..
    // 4g+3 (+16 for the second half) x 16 columns of block cb; this lane's 8
    // bytes are key 4g + (n >> 2), columns 16 cb + 4 (n & 3) .. + 3.
    // fp32.  K and Q: row n (qn), chunk 4 kk + g for kk < D / 16, d-values
    // 16 kk + 4 g .. + 3 feeding 4 MFMAs; a half-chunk adds 16 rows.  V: key
    // 16 t + 4 g + i, chunk n + 16 h (columns 64 h + 4 n .. + 3).
    constexpr int NKO = C::F32 ? D / 16 : C::KS;  // K / Q operand reads per 16-key half
    constexpr int NVO = C::F32 ? 4 * (D / 64) : C::CB;
    int k_off[NKO], q_off[NKO], v_off[NVO];
#pragma unroll
    for (int kk = 0; kk < NKO; ++kk) {
        k_off[kk] = n * C::ROWB + (((4 * kk + g) ^ swz_k<ET, D>(n)) * 16);
        q_off[kk] = qn * C::ROWB + (((4 * kk + g) ^ swz_k<ET, D>(qn)) * 16);
    }
    if constexpr (C::F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i;  // + 16 t, same swizzle
#pragma unroll
            for (int h = 0; h < D / 64; ++h)
                v_off[i * (D / 64) + h] = row * C::ROWB + (((n + 16 * h) ^ swz_v<ET, D>(row)) * 16);
        }
    } else {
        const int row = 4 * g + (n >> 2);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const int col = 16 * cb + 4 * (n & 3);
            v_off[cb] = row * C::ROWB + ((((col >> 3) ^ swz_v<ET, D>(row))) * 16) + (col & 7) * 2;
        }
    }

    // ---- running state of the current piece ------------------------------
    f32x4 acc[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x4{};
    float m_ref = 0.f, l_run = 0.f;

    // Operands of one chunk, all read from LDS before the first MFMA:
    // Q / K (bf16x8 or 4 fp32 d-values per read) and V^T (bf16: transposing
    // reads; fp32: 4 columns of key 16 t + 4 g + i, index (t, i, h)).
    using Op = typename std::conditional<C::F32, f32x4, bf16x8>::type;
    constexpr int NV = C::F32 ? 8 * (D / 64) : C::CB;
    auto read_ops = [&](const char *src, Op (&qo)[NKO], Op (&ko)[2][NKO], Op (&vo)[NV]) {
#pragma unroll
        for (int kk = 0; kk < NKO; ++kk) {
            u32x4 qx = *reinterpret_cast<const u32x4 *>(src + S::Q_OFF + q_off[kk]);
            if (neg) qx ^= C::F32 ? 0x80000000u : 0x80008000u;
            if (S::QROWS < 16 && n >= S::QROWS) qx = u32x4{};  // heads beyond the stored rows
            qo[kk] = __builtin_bit_cast(Op, qx);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < NKO; ++kk)
                ko[t][kk] = *reinterpret_cast<const Op *>(src + S::K_OFF + t * 16 * C::ROWB + k_off[kk]);
        if constexpr (C::F32) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < NVO; ++j)
                    vo[t * NVO + j] = *reinterpret_cast<const f32x4 *>(src + S::V_OFF + t * 16 * C::ROWB + v_off[j]);
        } else {
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                i16x4 part[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(src + S::V_OFF + h * 16 * C::ROWB + v_off[cb]));
                vo[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
    };

    // Scores of a chunk: x[4 t + r] = q_n . k_(16 t + 4 g + r) (raw, unscaled).
    auto scores = [&](const Op (&qo)[NKO], const Op (&ko)[2][NKO], float (&x)[8]) {
        f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int kk = 0; kk < NKO; ++kk)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if constexpr (C::F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ko[t][kk][e], qo[kk][e], s[t], 0, 0, 0);
                } else {
                    s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ko[t][kk], qo[kk], s[t], 0, 0, 0);
                }
            }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * t + r] = s[t][r];
    };

    // O^T += V^T P^T for a chunk; p[4 t + r] belongs to key 16 t + 4 g + r.
    auto pv = [&](const Op (&vo)[NV], const float (&p)[8]) {
        if constexpr (C::F32) {
            // block 4 h + e, row m <-> column 64 h + 4 m + e
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int h = 0; h < D / 64; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[4 * h + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                vo[t * NVO + i * (D / 64) + h][e], p[4 * t + i], acc[4 * h + e], 0, 0, 0);
        } else {
            const u32x4 pw = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                              pack_bf16(p[6], p[7])};
            const bf16x8 pbv = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo[cb], pbv, acc[cb], 0, 0, 0);
        }
    };

    // Stores this lane's share of output row `row` (d floats, or d elements
    // of the cache type) scaled by inv: head n's columns as the O^T blocks
    // hold them.
    auto store_row = [&](auto *row, float inv) {
        using E = typename std::remove_pointer<decltype(row)>::type;
        if constexpr (C::F32) {
            // block 4 h + e, element i <-> column 64 h + 16 g + 4 i + e
#pragma unroll
            for (int h = 0; h < D / 64; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 v = {acc[4 * h][i] * inv, acc[4 * h + 1][i] * inv, acc[4 * h + 2][i] * inv,
                                     acc[4 * h + 3][i] * inv};
                    *reinterpret_cast<f32x4 *>(row + 64 * h + 16 * g + 4 * i) = v;
                }
        } else {
            // block cb, element i <-> column 16 cb + 4 g + i
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                if constexpr (sizeof(E) == 4)
                    *reinterpret_cast<f32x4 *>(row + 16 * cb + 4 * g) = acc[cb] * inv;
                else
                    *reinterpret_cast<bf16x4 *>(row + 16 * cb + 4 * g) = __builtin_convertvector(acc[cb] * inv, bf16x4);
            }
        }
    };

    auto compute = [&](const int st) {
        const int cnt = m_cnt[st];
        Op qo[NKO], ko[2][NKO], vo[NV];
        read_ops(stage(st), qo, ko, vo);
        // scores: lane holds head n, keys 16 t + 4 g + r
        float x[8];
        scores(qo, ko, x);
        if (cnt < CK) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (16 * (i >> 2) + 4 * g + (i & 3) >= cnt) x[i] = -INFINITY;
        }
        auto head_max = [&]() {
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            return mx * sl2;  // finite: key 0 of the chunk is valid
        };
        if (m_first[st]) {
            m_ref = head_max();
            l_run = 0.f;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x4{};
        }
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], sl2, -m_ref));
            psum += p[i];
        }
        if (__builtin_amdgcn_ballot_w64(!(psum <= RESCALE_SUM)) != 0) {
            // raise the reference to the running max (rare)
            const float m_new = fmaxf(m_ref, head_max());
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
            m_ref = m_new;
            psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], sl2, -m_ref));
                psum += p[i];
            }
        }
        l_run += psum;
        pv(vo, p);

        if (m_last[st]) {
            // end of this range's piece of the segment
            float lt = l_run + __shfl_xor(l_run, 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            const int gblk = m_gblk[st], seg = m_seg[st];
            const float inv = 1.f / lt;
            const float lse_piece = (m_ref + __log2f(lt)) * LN2;
            if (m_w0[st] == m_w1[st]) {
                // the whole segment lies in this range: the final result
                if (n < gblk) {
                    store_row(O + ((size_t)m_head0[st] + n) * D, inv);
                    if (LSE && g == 0) LSE[m_head0[st] + n] = lse_piece;
                }
            } else {
                // normalised partial output and log-sum-exp to slot
                // (segment + workgroup), merged by the merge kernel
                const size_t slot = (size_t)seg + w;
                if (n < gblk) {
                    store_row(ws_o + (slot * GB + n) * D, inv);
                    if (g == 0) ws_lse[slot * GB + n] = lse_piece;
                }
                // the segment's last piece: record it for the merge kernel
                if (m_w1[st] == w && lane == 0)
                    *reinterpret_cast<i32x4 *>(ws_rec + 4 * w) =
                        i32x4{seg, m_w0[st], (int)(unsigned)(unsigned long long)T, (int)((unsigned long long)T >> 32)};
            }
        }
    };

    // ---- the pipeline ------------------------------------------------------
    int issued = 0, done = 0;
#pragma unroll
    for (int u = 0; u < NST - 1; ++u)
        if (issue(u)) ++issued;
    // one pipeline step on stage u (a constant after inlining); false once
    // every issued chunk has been computed
    auto step = [&](const int u) {
        if (done == issued) return false;
        // chunk `done` sits in stage u; `after` chunks were issued after it
        const int after = issued - done - 1;
        if (after >= NST - 2) {
            wait_vmcnt<(NST - 2) * S::NI>();
        } else if (NST > 3 && after == 1) {
            wait_vmcnt<S::NI>();
        } else {
            wait_vmcnt<0>();
        }
        // the stage refilled next was consumed by the previous chunk
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (issue((u + NST - 1) % NST)) ++issued;
        compute(u);
        ++done;
        return true;
    };
    for (;;) {
        if (!step(0)) break;
        if (!step(1)) break;
        if constexpr (NST > 2) {
            if (!step(2)) break;
        }
        if constexpr (NST > 3) {
            if (!step(3)) break;
        }
    }
}

// Merges the partial results of the segments that several ranges share
// (segments inside one range were written directly by the split kernel,
// empty sequences too).  Workgroup w (one wave) takes the segment whose last
// piece lies in range w, as the split kernel recorded it: the segment, its
// first range and the batch's key count, so no sequence lengths are read.
template <typename ET, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse, const int32_t *__restrict__ ws_rec,
    ET *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int nhb, int n_wg)
{
    const int w = blockIdx.x, lane = threadIdx.x;
    const i32x4 r = *reinterpret_cast<const i32x4 *>(ws_rec + 4 * w);
    const int seg = r[0];
    if (seg < 0) return;
    const long long T = (long long)(((unsigned long long)(unsigned)r[3] << 32) | (unsigned)r[2]);
    const int G = Hq / Hkv;
    const int GB = G < 16 ? G : 16;
    const int nsub = Hkv * nhb;
    const int b = seg / nsub, sub = seg - b * nsub;
    const int hk = sub / nhb, hb = sub - hk * nhb;
    const int gblk = G - 16 * hb < 16 ? G - 16 * hb : 16;
    merge_segment<ET, D>(ws_o, ws_lse, O, LSE, seg, r[1], w, (size_t)b * Hq + hk * G + 16 * hb, gblk, GB, T, n_wg,
                         lane);
}

template <typename ET, int D, int QR, int NST>
hipError_t launch_cfg(const DecodeArgs &a, hipStream_t stream) {
    int n_wg = a.n_wg;
    if (n_wg <= 0) {
        // As many single-wave workgroups as the chip holds at once for a
        // paged cache, and at most two per CU for a contiguous one (the CU
        // count and occupancy are queried once per device; concurrent first
        // calls store the same values).  Timed interleaved on the decode
        // workload: contiguous, two per CU beat three (the occupancy limit)
        // by 1.5-2 %; paged, three per CU beat two by 4-5 % at block sizes
        // 64-256 and by 21 % at 16, its extra waves hiding the block-table
        // lookups; counts that are not a multiple of the CU count were slower.
        static std::atomic<int> cached_cus[64], cached_per_cu[64];
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        int cus = cached_cus[dev].load(std::memory_order_relaxed);
        int per_cu = cached_per_cu[dev].load(std::memory_order_relaxed);
        if (cus == 0 || per_cu == 0) {
            hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return e;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_chunk_kernel<ET, D, QR, NST>, 64, 0);
            if (e != hipSuccess) return e;
            cus = cus > 0 ? cus : 1;
            per_cu = per_cu > 0 ? per_cu : 1;
            cached_cus[dev].store(cus, std::memory_order_relaxed);
            cached_per_cu[dev].store(per_cu, std::memory_order_relaxed);
        }
        n_wg = cus * (a.block_table || per_cu < 2 ? per_cu : 2);
    }
    if (n_wg > a.max_wg) n_wg = a.max_wg;
    const float sl2 = a.scale * LOG2E;
    hipLaunchKernelGGL((decode_chunk_kernel<ET, D, QR, NST>), dim3(n_wg), dim3(64), 0, stream, (const ET *)a.q,
                       (const ET *)a.k_cache, (const ET *)a.v_cache, a.seq_lens, (ET *)a.o, a.lse, a.ws_o, a.ws_lse,
                       a.ws_rec, a.B, a.Hq, a.Hkv, a.Lmax, a.nhb, n_wg, sl2, a.block_table, a.block_size,
                       a.max_blocks, a.num_blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<ET, D>), dim3(n_wg), dim3(64), 0, stream, a.ws_o, a.ws_lse, a.ws_rec,
                       (ET *)a.o, a.lse, a.Hq, a.Hkv, a.nhb, n_wg);
    return hipGetLastError();
}

template <typename ET, int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream) {
    // fp32 stages are twice the size: a ring of two keeps two workgroups per
    // CU in LDS
    constexpr int NST = sizeof(ET) == 4 ? 2 : DECODE_STAGES;
    const int G = a.Hq / a.Hkv;
    return G <= 4 ? launch_cfg<ET, D, 4, NST>(a, stream) : launch_cfg<ET, D, 16, NST>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (a.f32) return a.d == 128 ? launch_d<float, 128>(a, stream) : launch_d<float, 64>(a, stream);
    return a.d == 128 ? launch_d<__bf16, 128>(a, stream) : launch_d<__bf16, 64>(a, stream);
}

}  // namespace attn
