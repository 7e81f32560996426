// A plain C++ program that runs a workload's prefill and decode steps through
// the library's C ABI, for hardware-counter runs (rocprofv3 --pmc) of the
// kernels in the launch configurations the benchmark times, in a process
// that loads nothing but the library.
//
//   profile_driver WORKLOAD [layers] [decode_steps]
//
// WORKLOAD: llama2-7b-bs1 (batch 1, 8-token prompt), llama2-13b-bs8 (batch 8,
// 1024-token prompts) or llama2-70b-gqa-bs32 (batch 32, 2048-token prompts).  `layers` overrides the depth (the per-layer
// kernels are the same at any depth).  Tokens are seeded and uniform over the
// vocabulary; decode steps are greedy.  Prints one line per phase with its
// wall time.
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/llm.h"

namespace {

uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

int fail(llm_t *h, const char *what, int rc)
{
    std::fprintf(stderr, "%s failed (%d): %s\n", what, rc, llm_last_error(h));
    return 1;
}

double now()
{
    return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc < 2) {
        std::fprintf(stderr, "usage: %s llama2-7b-bs1|llama2-13b-bs8|llama2-70b-gqa-bs32 [layers] [decode_steps]\n",
                     argv[0]);
        return 2;
    }
    llm_params p{};
    int B = 0, T = 0;
    uint64_t seed = 0;
    if (!std::strcmp(argv[1], "llama2-7b-bs1")) {
        p = llm_params{32, 4096, 32, 32, 32000, 256, 0.f, 1e-5f, 10000.f, 1, 2048, LLM_F16};
        B = 1, T = 8, seed = 1002;
    } else if (!std::strcmp(argv[1], "llama2-13b-bs8")) {
        p = llm_params{40, 5120, 40, 40, 32000, 256, 0.f, 1e-5f, 10000.f, 8, 2048, LLM_F16};
        B = 8, T = 1024, seed = 1004;
    } else if (!std::strcmp(argv[1], "llama2-70b-gqa-bs32")) {
        p = llm_params{80, 8192, 64, 8, 32000, 4096, 1.3f, 1e-5f, 10000.f, 32, 4096, LLM_F16};
        B = 32, T = 2048, seed = 1005;
    } else {
        std::fprintf(stderr, "unknown workload %s\n", argv[1]);
        return 2;
    }
    if (argc > 2) p.n_layers = std::atoi(argv[2]);
    const int steps = argc > 3 ? std::atoi(argv[3]) : 16;
    if (p.n_layers < 1 || steps < 0 || T + steps > p.max_seq_len) return 2;

    llm_t *h = nullptr;
    double t0 = now();
    int rc = llm_create(&p, seed, nullptr, &h);
    if (rc) return fail(h, "llm_create", rc);
    std::printf("create %.3f s (%d layers)\n", now() - t0, p.n_layers);
    std::vector<int32_t> tok((size_t)B * T);
    for (size_t i = 0; i < tok.size(); i++) tok[i] = (int32_t)((mix(seed * 7919 + i) >> 32) % (uint64_t)p.vocab_size);
    t0 = now();
    if ((rc = llm_prefill(h, tok.data(), B, T))) return fail(h, "llm_prefill", rc);
    if ((rc = llm_sample(h, 0.f, 1.f, nullptr, nullptr))) return fail(h, "llm_sample", rc);
    if ((rc = llm_sync(h))) return fail(h, "llm_sync", rc);
    std::printf("prefill %d x %d: %.3f s\n", B, T, now() - t0);
    t0 = now();
    for (int s = 0; s < steps; s++) {
        if ((rc = llm_decode(h, T + s))) return fail(h, "llm_decode", rc);
        if ((rc = llm_sample(h, 0.f, 1.f, nullptr, nullptr))) return fail(h, "llm_sample", rc);
    }
    if ((rc = llm_sync(h))) return fail(h, "llm_sync", rc);
    std::printf("decode %d steps: %.3f ms per step\n", steps, steps ? (now() - t0) * 1e3 / steps : 0.0);
    llm_destroy(h);
    std::printf("done\n");
    return 0;
}
