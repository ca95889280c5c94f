/* A C99 caller of libflowcache: the header compiles as C, the library links,
 * and the host-side checks answer without a GPU (no call here queues work). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flowcache.h"

static int fails = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL line %d: %s\n", __LINE__, #cond);            \
            ++fails;                                                  \
        }                                                             \
    } while (0)

int main(void) {
    CHECK(strcmp(fc_status_string(FC_OK), "ok") == 0);
    CHECK(strcmp(fc_status_string((fc_status)99), "unknown status") == 0);

    fc_kv_params p;
    memset(&p, 0, sizeof p);
    p.H = 24; p.d = 128; p.L_q = 3600; p.L_k = 18000; p.B_budget = 7200;
    p.lambda = 0.5f; p.pool_window = 7; p.softmax_scale = 0.0f; p.dtype = FC_BF16;
    const size_t need = fc_kv_compress_workspace_bytes(&p);
    CHECK(need > 0 && need % 256 == 0);
    void* dummy = (void*)(uintptr_t)4096;
    CHECK(fc_kv_compress(&p, NULL, dummy, dummy, dummy, dummy, (int32_t*)dummy, NULL, NULL, NULL, dummy, need,
                         NULL) == FC_ERR_INVALID_ARG);
    CHECK(fc_kv_compress(&p, dummy, dummy, dummy, dummy, dummy, (int32_t*)dummy, NULL, NULL, NULL, dummy,
                         need - 1, NULL) == FC_ERR_WORKSPACE);
    p.d = 96;
    CHECK(fc_kv_compress_workspace_bytes(&p) == 0);

    fc_l1_params l1 = {16, 5, 0.01f, FC_BF16};
    int64_t off[17];
    for (int i = 0; i <= 16; ++i) off[i] = (int64_t)i * 7372800;
    CHECK(fc_chunk_rel_l1_workspace_bytes(&l1, off) > 0);
    CHECK(fc_chunk_rel_l1_decide(&l1, off, dummy, dummy, NULL, dummy, (uint8_t*)dummy, NULL, dummy, 1 << 20,
                                 NULL) == FC_ERR_INVALID_ARG);

    fc_cache_params c = {24, 128, 7200, 3600, 0.5f, 7, 0.0f, FC_BF16};
    CHECK(fc_cache_commit_workspace_bytes(&c, 3600) > 0);
    int32_t L_clean = 7201;
    int32_t swapped = -1;
    CHECK(fc_cache_commit(&c, &L_clean, dummy, dummy, 10, 0, dummy, 3600, dummy, dummy, NULL, dummy, dummy, NULL,
                          &swapped, NULL, 0, NULL) == FC_ERR_INVALID_ARG);
    CHECK(swapped == -1);

    printf("%s\n", fails ? "C ABI checks failed" : "C ABI checks ok");
    return fails != 0;
}
