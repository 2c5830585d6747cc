/* A C program built against include/attn.h alone and linked to libattn.so:
 * shows that the header is valid C (and, built as C++, that its extern "C"
 * block gives unmangled names), that every prototype has the type written
 * below, and that calls which touch no device memory behave as documented.
 * It makes no call that reaches the HIP runtime. Prints "ok" and returns 0
 * on success, else names the failed check and returns 1. */
#include "attn.h"

#include <stdio.h>
#include <string.h>

/* Each entry point assigned to a pointer of its documented type: a changed
 * prototype fails to compile (the build uses -Werror). */
static int (*const p_fwd)(const void *, const void *, const void *, void *, float *, int, int, int, int, int, int,
                          float, int, attn_dtype_t, hipStream_t) = attn_fwd;
static int (*const p_fwd_fp8)(const void *, const void *, const void *, void *, float *, int, int, int, int, int,
                              int, float, float, int, hipStream_t) = attn_fwd_fp8;
static size_t (*const p_bwd_ws)(int, int, int) = attn_bwd_workspace_bytes;
static int (*const p_bwd)(const void *, const void *, const void *, const void *, const void *, const float *, void *,
                          void *, void *, int, int, int, int, int, int, float, int, attn_dtype_t, void *, size_t,
                          hipStream_t) = attn_bwd;
static size_t (*const p_dec_ws)(int, int, int, int, int) = attn_decode_workspace_bytes;
static int (*const p_dec)(const void *, const void *, const void *, const int32_t *, void *, float *, int, int, int,
                          int, int, float, attn_dtype_t, void *, size_t, hipStream_t) = attn_decode;
static size_t (*const p_split_ws)(int, int, int, int, int, int) = attn_decode_split_workspace_bytes;
static int (*const p_split)(const void *, const void *, const void *, const int32_t *, void *, float *, int, int, int,
                            int, int, float, int, attn_dtype_t, void *, size_t, hipStream_t) = attn_decode_split;
static int (*const p_noalloc)(const void *, const void *, const void *, const int32_t *, void *, float *, int, int,
                              int, int, int, float, attn_dtype_t, hipStream_t) = attn_decode_noalloc;
static int (*const p_paged)(const void *, const void *, const void *, const int32_t *, const int32_t *, void *,
                            float *, int, int, int, int, int, int, int, float, int, attn_dtype_t, void *, size_t,
                            hipStream_t) = attn_decode_paged;
static const char *(*const p_str)(int) = attn_status_str;

static int failed = 0;

static void check(int ok, const char *what) {
    if (!ok) {
        printf("FAILED: %s\n", what);
        failed = 1;
    }
}

int main(void) {
    const int codes[] = {ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_LAUNCH};
    const char *names[] = {"ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE",
                           "ATTN_ERR_LAUNCH"};
    int i;
    for (i = 0; i < 5; ++i) {
        check(codes[i] == i, "status codes are 0..4");
        check(strcmp(p_str(codes[i]), names[i]) == 0, "attn_status_str names each status");
    }
    check(p_str(-7) != NULL && p_str(99) != NULL, "attn_status_str never returns NULL");
    check(ATTN_F32 == 0 && ATTN_BF16 == 1, "dtype codes");
    check(ATTN_DECODE_NOALLOC_MAX_BYTES == ((size_t)32 << 20), "no-alloc scratch limit");

    /* sizes: nonzero for a valid shape, zero for one the entry point refuses */
    check(p_dec_ws(16, 32, 8, 4096, 128) > 0, "decode workspace for the decode workload");
    check(p_dec_ws(16, 30, 8, 4096, 128) == 0, "decode workspace 0 when Hq is not a multiple of Hkv");
    check(p_split_ws(16, 32, 8, 4096, 128, 0) == p_dec_ws(16, 32, 8, 4096, 128),
          "keys_per_split 0 is the default split");
    check(p_bwd_ws(2, 8, 100) >= (size_t)2 * 8 * 100 * sizeof(float), "backward workspace holds D");

    /* argument checks that run before any HIP call (null tensor pointers) */
    check(p_fwd(NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 8, 64, 0.125f, 0, ATTN_BF16, NULL) == ATTN_ERR_INVALID_ARG,
          "attn_fwd rejects null pointers");
    check(p_fwd_fp8(NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 8, 128, 0.1f, 1.0f, 0, NULL) == ATTN_ERR_INVALID_ARG,
          "attn_fwd_fp8 rejects null pointers");
    check(p_bwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 8, 64, 0.125f, 0, ATTN_BF16, NULL,
                0, NULL) == ATTN_ERR_INVALID_ARG,
          "attn_bwd rejects null pointers");
    check(p_dec(NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 64, 0.125f, ATTN_BF16, NULL, 0, NULL) ==
              ATTN_ERR_INVALID_ARG,
          "attn_decode rejects null pointers");
    check(p_split(NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 64, 0.125f, 4, ATTN_BF16, NULL, 0, NULL) ==
              ATTN_ERR_INVALID_ARG,
          "attn_decode_split rejects null pointers");
    check(p_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 64, 0.125f, ATTN_BF16, NULL) ==
              ATTN_ERR_INVALID_ARG,
          "attn_decode_noalloc rejects null pointers");
    check(p_paged(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 4, 16, 2, 64, 0.125f, 0, ATTN_BF16, NULL, 0,
                  NULL) == ATTN_ERR_INVALID_ARG,
          "attn_decode_paged rejects null pointers");

    if (!failed) printf("ok\n");
    return failed;
}
