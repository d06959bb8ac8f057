// host_check.cpp -- exercises libdgc's host-side planning and argument
// checks (no GPU calls) for many layouts, for a build with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code.  Built and run by
// tests/test_host_sanitized.py.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "dgc.h"

#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            std::abort();                                                    \
        }                                                                    \
    } while (0)

int main() {
    std::mt19937_64 rng(7);
    size_t bytes = 0;
    // layouts from empty to thousands of tensors
    for (int round = 0; round < 300; ++round) {
        int T = 1 + int(rng() % (round < 250 ? 200 : 5000));
        std::vector<int64_t> sizes(T), kmax(T);
        for (int t = 0; t < T; ++t) {
            int64_t choice = int64_t(rng() % 6);
            sizes[t] = choice == 0 ? 0
                     : choice == 1 ? int64_t(rng() % 70000)
                     : choice == 2 ? 65536 + int64_t(rng() % 3)
                     : choice == 3 ? int64_t(rng() % 5000000)
                     : choice == 4 ? 1
                                   : int64_t(rng() % 400000);
            kmax[t] = sizes[t] ? int64_t(rng() % (sizes[t] + 1)) : 0;
        }
        CHECK(dgc_workspace_bytes(T, sizes.data(), kmax.data(), &bytes) == DGC_OK);
        CHECK(bytes > 0);
        // init with a too-small workspace is refused before any GPU call
        dgc_state* st = reinterpret_cast<dgc_state*>(0x1);
        CHECK(dgc_init_state(&st, T, sizes.data(), kmax.data(), 0.9f,
                             reinterpret_cast<float*>(256), reinterpret_cast<float*>(256),
                             reinterpret_cast<void*>(4096), bytes - 1, nullptr) ==
              DGC_ECAPACITY);
        CHECK(st == nullptr);
    }
    // invalid layouts
    int64_t big[1] = {int64_t(1) << 32}, one[1] = {1}, neg[1] = {-1};
    CHECK(dgc_workspace_bytes(1, big, one, &bytes) == DGC_EINVAL);
    CHECK(dgc_workspace_bytes(1, one, neg, &bytes) == DGC_EINVAL);
    CHECK(dgc_workspace_bytes(0, one, one, &bytes) == DGC_EINVAL);
    CHECK(dgc_workspace_bytes(1, nullptr, one, &bytes) == DGC_EINVAL);
    CHECK(dgc_workspace_bytes(1, one, one, nullptr) == DGC_EINVAL);
    CHECK(dgc_compress_binlocal(nullptr, nullptr, one, one, 0.0, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr) == DGC_EINVAL);
    CHECK(dgc_encode_counts(nullptr, one, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr) == DGC_EINVAL);
    CHECK(dgc_compress_sampled(nullptr, nullptr, one, one, 0.0, nullptr, nullptr, nullptr,
                               nullptr, nullptr, nullptr, nullptr) == DGC_EINVAL);
    for (int code = -6; code <= 1; ++code) CHECK(dgc_error_string(code) != nullptr);
    dgc_destroy_state(nullptr);
    std::printf("host check: ok\n");
    return 0;
}
