/*
 * abi_sanitize_run.c -- drives the host side of the C ABI (argument checks,
 * workspace sizing and chunking, the host contract check) with clang's
 * AddressSanitizer and UndefinedBehaviorSanitizer on the library's host code.
 * No call here reaches a kernel launch: every problem is either rejected or
 * only sized.  tests/test_oracle_sanitizers.py builds and runs it; exit 0 on
 * success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "msa.h"

#define CHECK(c, msg)                                    \
    do {                                                 \
        if (!(c)) {                                      \
            fprintf(stderr, "abi_sanitize_run: %s\n", msg); \
            return 1;                                    \
        }                                                \
    } while (0)

static msa_problem_t problem(int32_t nseq, int32_t tq, int32_t tk, int32_t mq, int32_t mk, int32_t H, int32_t h,
                             int32_t B, int32_t k) {
    static const int32_t fake[1] = {0};
    msa_problem_t p;
    memset(&p, 0, sizeof p);
    p.num_seqs = nseq;
    p.total_q = tq;
    p.total_k = tk;
    p.cu_seqlens_q = fake;   /* never dereferenced on the host */
    p.cu_seqlens_k = fake;
    p.max_seqlen_q = mq;
    p.max_seqlen_k = mk;
    p.num_heads = H;
    p.num_kv_heads = h;
    p.head_dim = 128;
    p.index_dim = 64;
    p.block_size = B;
    p.top_k = k;
    return p;
}

int main(void) {
    const void *F = (const void *)0x1000;   /* a fake device pointer: validation fails before any use */
    /* workspace sizes over a range of shapes, chunked and not */
    const int32_t lens[] = {1, 63, 64, 1000, 32768, 131072, 1 << 20};
    for (unsigned i = 0; i < sizeof lens / sizeof lens[0]; ++i)
        for (int op = 0; op <= 6; ++op) {
            msa_problem_t p = problem(1, lens[i], lens[i], lens[i], lens[i], 64, 8, 64, 1024);
            size_t n = msa_workspace_size(op, &p);
            if (op <= 5 && op != MSA_OP_SPARSE_ATTN_DECODE) CHECK(n != (size_t)-1, "size of a valid problem");
            (void)msa_workspace_wait_word(op, &p);
        }
    setenv("MSA_DEBUG_WORKSPACE_CAP", "100000", 1);
    msa_problem_t big = problem(1, 32768, 32768, 32768, 32768, 32, 8, 64, 32);
    CHECK(msa_workspace_size(MSA_OP_INDEX_TOPK, &big) <= 100000, "index chunks under a lowered cap");
    setenv("MSA_DEBUG_WORKSPACE_CAP", "not a number", 1);
    CHECK(msa_workspace_size(MSA_OP_INDEX_TOPK, &big) == (size_t)32768 * 8 * 512 * 4, "bad override ignored");
    unsetenv("MSA_DEBUG_WORKSPACE_CAP");
    /* rejected calls */
    msa_problem_t bad = problem(0, 4, 4, 4, 4, 8, 2, 64, 4);
    CHECK(msa_index_topk(&bad, F, F, (int32_t *)F, NULL, 0, NULL) == MSA_ERROR_INVALID_VALUE, "num_seqs 0");
    CHECK(msa_index_topk(NULL, F, F, (int32_t *)F, NULL, 0, NULL) == MSA_ERROR_INVALID_VALUE, "null problem");
    msa_problem_t p = problem(1, 128, 128, 128, 128, 8, 2, 64, 4);
    CHECK(msa_index_topk(&p, F, F, (int32_t *)F, NULL, 0, NULL) == MSA_ERROR_WORKSPACE, "missing workspace");
    CHECK(msa_sparse_attn_prefill(&p, NULL, F, F, F, 0.1f, (msa_bf16_t *)F, NULL, NULL, 0, NULL) ==
              MSA_ERROR_INVALID_VALUE, "null q");
    CHECK(msa_sparse_attn_decode(&p, F, F, F, F, 0.1f, (msa_bf16_t *)F, NULL, NULL, 0, NULL) ==
              MSA_ERROR_INVALID_VALUE, "decode shape");
    CHECK(msa_sparse_attn_decode_noalloc(&p, F, F, F, F, 0.1f, (msa_bf16_t *)F, NULL, NULL) ==
              MSA_ERROR_INVALID_VALUE, "no-alloc decode shape");
    CHECK(msa_sparse_attn_prefill_backward(&p, F, F, F, F, 0.1f, F, NULL, F, (msa_bf16_t *)F, (msa_bf16_t *)F,
                                           (msa_bf16_t *)F, NULL, 0, NULL) == MSA_ERROR_INVALID_VALUE, "null lse");
    msa_select_options_t opt = {3, 2};
    CHECK(msa_index_topk_ex(&p, &opt, NULL, F, F, (int32_t *)F, NULL, 0, NULL) == MSA_ERROR_INVALID_VALUE,
          "too many forced blocks");
    CHECK(msa_kv_append_paged(-1, 8, 128, 64, 16, F, F, F, F, (msa_bf16_t *)F, (msa_bf16_t *)F, (msa_bf16_t *)F,
                              NULL) == MSA_ERROR_INVALID_VALUE, "negative token count");
    CHECK(msa_status_string((msa_status_t)99) != NULL, "status string");
    /* the host contract check on host arrays */
    const int32_t cq[4] = {0, 3, 3, 5}, ck[4] = {0, 130, 135, 137};
    msa_problem_t hp = problem(3, 5, 137, 3, 130, 4, 2, 64, 2);
    int32_t ids[5 * 2 * 2];
    for (int i = 0; i < 20; ++i) ids[i] = (i % 2) ? -1 : 0;
    CHECK(msa_validate_host(&hp, cq, ck, ids) == MSA_SUCCESS, "valid contract");
    ids[0] = 5;
    CHECK(msa_validate_host(&hp, cq, ck, ids) == MSA_ERROR_INVALID_VALUE, "ineligible id");
    ids[0] = 0;
    ids[1] = 0;
    CHECK(msa_validate_host(&hp, cq, ck, ids) == MSA_ERROR_INVALID_VALUE, "duplicate id");
    const int32_t ck_other[4] = {0, 130, 131, 137};   /* other key lengths, still >= the query lengths */
    CHECK(msa_validate_host(&hp, cq, ck_other, NULL) == MSA_SUCCESS, "lengths within the maxima");
    const int32_t ck_short[4] = {0, 2, 131, 137};     /* 2 keys for 3 queries */
    CHECK(msa_validate_host(&hp, cq, ck_short, NULL) == MSA_ERROR_INVALID_VALUE, "len_k < len_q");
    const int32_t cq_bad[4] = {0, 4, 3, 5};
    CHECK(msa_validate_host(&hp, cq_bad, ck, NULL) == MSA_ERROR_INVALID_VALUE, "decreasing offsets");
    CHECK(msa_validate_host(NULL, cq, ck, NULL) == MSA_ERROR_INVALID_VALUE, "null problem");
    puts("abi_sanitize_run: ok");
    return 0;
}
