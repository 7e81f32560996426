// Drives the library's host logic through the C ABI with the runtime
// stand-ins of runtime_stub.hip (no GPU): static and paged caches, fp32 and
// fp16 models, every forward entry point.  Built with AddressSanitizer; the
// stand-in launchers check that every KV-cache address a kernel would touch
// lies in the cache allocation and that paged positions have a block.
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "../../include/llm.h"

extern "C" int hipMalloc(void **ptr, size_t size);
extern "C" int hipFree(void *ptr);

static int failures = 0;
#define EXPECT(x, want)                                                                       \
    do {                                                                                      \
        int r_ = (x);                                                                         \
        if (r_ != (want)) {                                                                   \
            printf("line %d: %s -> %d, expected %d (%s)\n", __LINE__, #x, r_, (want),        \
                   h ? llm_last_error(h) : "");                                               \
            failures++;                                                                       \
        }                                                                                     \
    } while (0)

static llm_params model(int dtype, int maxB, int S)
{
    llm_params p{};
    p.n_layers = 2;
    p.dim = dtype == LLM_F16 ? 512 : 64;
    p.n_heads = 4;
    p.n_kv_heads = 2;
    p.vocab_size = dtype == LLM_F16 ? 1024 : 256;
    p.multiple_of = dtype == LLM_F16 ? 64 : 32;
    p.norm_eps = 1e-5f;
    p.rope_theta = 10000.f;
    p.max_batch_size = maxB;
    p.max_seq_len = S;
    p.dtype = dtype;
    return p;
}

static void uniform_run(llm_t *h, int B, std::vector<int> chunks, int steps)
{
    std::vector<int> tok(B * 4096, 1);
    int pos = 0;
    for (int c : chunks) {
        EXPECT(llm_prefill_at(h, pos, tok.data(), B, c), LLM_OK);
        pos += c;
    }
    for (int p = pos; p < pos + steps; p++) {
        EXPECT(llm_set_tokens(h, p, tok.data(), nullptr), LLM_OK);
        EXPECT(llm_decode(h, p), LLM_OK);
    }
}

static void rows_run(llm_t *h, std::vector<int> lens, int steps)
{
    int M = 0;
    for (int l : lens) M += l;
    std::vector<int> tok(M, 1), t(lens.size(), 2);
    EXPECT(llm_prefill_varlen(h, tok.data(), lens.data(), (int)lens.size()), LLM_OK);
    for (int k = 0; k < steps; k++) {
        EXPECT(llm_set_tokens_rows(h, t.data(), nullptr), LLM_OK);
        EXPECT(llm_decode_rows(h), LLM_OK);
    }
}

int hostcheck_resid_norms();  // in the runtime stand-ins

int main()
{
    llm_t *h = nullptr;
    for (int paged = 0; paged < 2; paged++) {
        llm_paging pg{32, 2 * 3, 0.f};
        llm_params p = model(LLM_F32, 2, 96);
        EXPECT(paged ? llm_create_paged(&p, &pg, 99, nullptr, &h) : llm_create(&p, 99, nullptr, &h), LLM_OK);
        uniform_run(h, 2, {20}, 40);
        rows_run(h, {3, 40}, 30);
        uniform_run(h, 1, {5, 7}, 3);
        llm_destroy(h);
        h = nullptr;
    }
    for (int paged = 0; paged < 2; paged++) {
        llm_paging pg{64, 3 * 4, 0.f};
        llm_params p = model(LLM_F16, 3, 256);
        EXPECT(paged ? llm_create_paged(&p, &pg, 99, nullptr, &h) : llm_create(&p, 99, nullptr, &h), LLM_OK);
        uniform_run(h, 3, {40, 30}, 20);
        rows_run(h, {5, 70, 130}, 10);
        uniform_run(h, 2, {1}, 100);
        uniform_run(h, 1, {10}, 60);  // one row: the fused decode layer
        rows_run(h, {7}, 20);
        llm_destroy(h);
        h = nullptr;
    }
    {
        // a pool from the budget; exhaustion and release
        llm_paging pg{64, 0, 0.7f};
        llm_params p = model(LLM_F16, 3, 256);
        EXPECT(llm_create_paged(&p, &pg, 99, nullptr, &h), LLM_OK);
        if (llm_kv_num_blocks(h) != 12) { printf("budget pool: %d blocks\n", llm_kv_num_blocks(h)); failures++; }
        llm_destroy(h);
        llm_paging small{64, 4, 0.f};
        EXPECT(llm_create_paged(&p, &small, 99, nullptr, &h), LLM_OK);
        std::vector<int> tok(3 * 256, 1);
        EXPECT(llm_prefill(h, tok.data(), 3, 100), LLM_ENOMEM);  // 6 blocks needed
        EXPECT(llm_prefill(h, tok.data(), 2, 100), LLM_OK);
        EXPECT(llm_kv_set_block_table(h, 1, nullptr, 0), LLM_OK);
        EXPECT(llm_set_tokens(h, 100, tok.data(), nullptr), LLM_OK);
        EXPECT(llm_decode(h, 100), LLM_ESTATE);                 // row 1's cache released
        llm_destroy(h);
        h = nullptr;
    }
    {
        // scrambled tables, single-kernel entry points, timing hooks
        llm_paging pg{32, 3 * 8, 0.f};
        llm_params p = model(LLM_F16, 3, 256);
        EXPECT(llm_create_paged(&p, &pg, 99, nullptr, &h), LLM_OK);
        std::vector<int> perm(24);
        for (int i = 0; i < 24; i++) perm[i] = (i * 7 + 3) % 24;
        for (int r = 0; r < 3; r++) EXPECT(llm_kv_set_block_table(h, r, perm.data() + 8 * r, 8), LLM_OK);
        uniform_run(h, 3, {40, 30}, 20);
        float ms[9], us[6];
        EXPECT(llm_profile_decode(h, 89, 2, ms), LLM_OK);
        EXPECT(llm_profile_projections(h, 2, us), LLM_OK);
        void *dtok = nullptr, *k = nullptr, *v = nullptr, *q = nullptr, *o = nullptr;
        hipMalloc(&dtok, 3 * 256 * 4);
        EXPECT(llm_profile_prefill(h, (const int *)dtok, 3, 200, 1, ms), LLM_OK);
        const size_t kvb = (size_t)3 * 256 * 2 * 128 * 2, qb = (size_t)3 * 256 * 4 * 128 * 2;
        hipMalloc(&k, kvb);
        hipMalloc(&v, kvb);
        hipMalloc(&q, qb);
        hipMalloc(&o, qb);
        EXPECT(llm_op_kv_write(h, 1, k, v, 3, 256, 0), LLM_OK);
        EXPECT(llm_op_attention(h, 1, q, 3, 1, 255, o), LLM_OK);
        EXPECT(llm_op_attention(h, 1, q, 3, 256, 0, o), LLM_OK);
        for (void *x : {dtok, k, v, q, o}) hipFree(x);
        llm_destroy(h);
        h = nullptr;
    }
    // the decodes of 2..3 rows took the hand-over of split-K partials
    if (hostcheck_resid_norms() == 0) { printf("no normalisation added handed-over partials\n"); failures++; }
    printf(failures ? "FAILED %d\n" : "done\n", failures);
    return failures ? 1 : 0;
}
