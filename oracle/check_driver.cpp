// check_driver.cpp -- runs every oracle function over random and edge-case
// inputs so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
// (host code only) can check the oracle's memory accesses.  Test
// infrastructure; built and run by tests/test_oracle_sanitized.py.
//
// Self-checks (abort on failure): exactly k entries selected, ascending
// indices, sent + residual == accumulated v, u and v zero where sent,
// decode(encode(x)) reproduces the sent values; for the bin-local selector,
// min(salient, cap) entries delivered, ascending, non-zero, masked.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int orc_clip_scale(const float* g, int64_t n, double clip, double* norm, float* scale);
void orc_momentum(const float* g, int64_t n, float scale, float m, float* u, float* v);
int64_t orc_select_mask(float* u, float* v, int64_t n, int64_t k, uint32_t* idx,
                        float* val);
int64_t orc_encode(const uint32_t* idx, const float* val, int64_t k, uint16_t* runs,
                   float* vals, int64_t cap);
int orc_decode_accumulate(const uint16_t* runs, const float* vals, int64_t E,
                          float* dense, int64_t n);
int64_t orc_k_for_density(int64_t n, int64_t num, int64_t den);
int orc_step(int32_t T, const int64_t* sizes, const int64_t* k, const float* g, float* u,
             float* v, float m, double clip, uint32_t* idx, float* val, double* norm,
             float* scale);
int64_t orc_binlocal_select_mask(float* u, float* v, int64_t n, int64_t L, int64_t cap,
                                 uint32_t* idx, float* val, int64_t* total);
int orc_binlocal_step(int32_t T, const int64_t* sizes, const int64_t* L, const int64_t* cap,
                      const float* g, float* u, float* v, float m, double clip,
                      uint32_t* idx, float* val, int64_t* count, int64_t* total,
                      double* norm, float* scale);
int64_t orc_sampled_select_mask(float* u, float* v, int64_t n, int64_t k, int64_t cap,
                                int32_t t, uint32_t* idx, float* val, int64_t* total,
                                uint32_t* theta);
int orc_sampled_step(int32_t T, const int64_t* sizes, const int64_t* k, const int64_t* cap,
                     const float* g, float* u, float* v, float m, double clip,
                     uint32_t* idx, float* val, int64_t* count, int64_t* total,
                     uint32_t* theta, double* norm, float* scale);
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            std::abort();                                               \
        }                                                               \
    } while (0)

static uint32_t bits(float x) {
    uint32_t b;
    std::memcpy(&b, &x, 4);
    return b;
}

int main() {
    std::mt19937_64 rng(12345);
    const int64_t sizes_pool[] = {0, 1, 2, 3, 17, 1000, 65535, 65536, 65537, 140001};
    for (int round = 0; round < 40; ++round) {
        int T = 1 + int(rng() % 5);
        std::vector<int64_t> sizes(T), k(T);
        int64_t n = 0, K = 0;
        for (int t = 0; t < T; ++t) {
            sizes[t] = sizes_pool[rng() % 10];
            int64_t choice = rng() % 4;
            k[t] = sizes[t] == 0 ? 0
                 : choice == 0 ? 0
                 : choice == 1 ? sizes[t]
                 : choice == 2 ? orc_k_for_density(sizes[t], 1, 1000)
                               : int64_t(rng() % (sizes[t] + 1));
            n += sizes[t];
            K += k[t];
        }
        std::vector<float> g(n), u(n), v(n);
        std::normal_distribution<float> nd(0.f, 1e-2f);
        for (int64_t i = 0; i < n; ++i) {
            g[i] = (rng() % 10 == 0) ? 0.f : nd(rng);
            if (rng() % 50 == 0) g[i] = 1e-42f;  // denormal
            u[i] = nd(rng) * 0.1f;
            v[i] = nd(rng) * 0.1f;
        }
        std::vector<float> v_pre(v), u_pre(u);
        double norm;
        float s;
        orc_clip_scale(g.data(), n, 0.5, &norm, &s);
        orc_momentum(g.data(), n, s, 0.9f, u_pre.data(), v_pre.data());
        std::vector<uint32_t> idx(K + 1);
        std::vector<float> val(K + 1);
        double norm2;
        float s2;
        CHECK(orc_step(T, sizes.data(), k.data(), g.data(), u.data(), v.data(), 0.9f, 0.5,
                       idx.data(), val.data(), &norm2, &s2) == 0);
        CHECK(norm2 == norm && s2 == s);
        int64_t off = 0, koff = 0;
        for (int t = 0; t < T; ++t) {
            std::vector<float> sent(sizes[t] > 0 ? sizes[t] : 1, 0.f);
            for (int64_t j = 0; j < k[t]; ++j) {
                uint32_t i = idx[koff + j];
                CHECK(int64_t(i) < sizes[t]);
                if (j) CHECK(idx[koff + j - 1] < i);
                CHECK(bits(val[koff + j]) == bits(v_pre[off + i]));
                CHECK(bits(u[off + i]) == 0 && bits(v[off + i]) == 0);
                sent[i] = val[koff + j];
            }
            for (int64_t i = 0; i < sizes[t]; ++i) {
                float back = sent[i] + v[off + i];
                CHECK(bits(back) == bits(v_pre[off + i] + 0.0f));
            }
            int64_t cap = k[t] + sizes[t] / 65536 + 1;
            std::vector<uint16_t> runs(cap);
            std::vector<float> vals(cap);
            int64_t E = orc_encode(idx.data() + koff, val.data() + koff, k[t], runs.data(),
                                   vals.data(), cap);
            CHECK(E >= k[t]);
            std::vector<float> dense(sizes[t] > 0 ? sizes[t] : 1, 0.f);
            CHECK(orc_decode_accumulate(runs.data(), vals.data(), E, dense.data(), sizes[t]) == 0);
            for (int64_t i = 0; i < sizes[t]; ++i) CHECK(dense[i] == sent[i]);
            off += sizes[t];
            koff += k[t];
        }
    }
    // bin-local selector: bins of random length, capacities from none to all
    for (int round = 0; round < 30; ++round) {
        int T = 1 + int(rng() % 4);
        std::vector<int64_t> sizes(T), L(T), cap(T), count(T), total(T);
        int64_t n = 0, C = 0;
        for (int t = 0; t < T; ++t) {
            sizes[t] = sizes_pool[rng() % 10];
            L[t] = 1 + int64_t(rng() % 1100);
            cap[t] = (rng() % 3 == 0) ? sizes[t] : int64_t(rng() % (sizes[t] / 8 + 2));
            n += sizes[t];
            C += cap[t];
        }
        std::vector<float> g(n), u(n), v(n);
        std::normal_distribution<float> nd(0.f, 1e-2f);
        for (int64_t i = 0; i < n; ++i) {
            g[i] = (rng() % 10 == 0) ? 0.f : nd(rng);
            u[i] = nd(rng) * 0.1f;
            v[i] = (rng() % 7 == 0) ? 0.f : nd(rng) * 0.1f;
        }
        std::vector<float> u_pre(u), v_pre(v);
        double norm;
        float s;
        orc_clip_scale(g.data(), n, 0.5, &norm, &s);
        orc_momentum(g.data(), n, s, 0.9f, u_pre.data(), v_pre.data());
        std::vector<uint32_t> idx(C + 1);
        std::vector<float> val(C + 1);
        CHECK(orc_binlocal_step(T, sizes.data(), L.data(), cap.data(), g.data(), u.data(),
                                v.data(), 0.9f, 0.5, idx.data(), val.data(), count.data(),
                                total.data(), &norm, &s) == 0);
        int64_t off = 0, coff = 0;
        for (int t = 0; t < T; ++t) {
            CHECK(count[t] == std::min(total[t], cap[t]));
            for (int64_t j = 0; j < count[t]; ++j) {
                uint32_t i = idx[coff + j];
                CHECK(int64_t(i) < sizes[t]);
                if (j) CHECK(idx[coff + j - 1] < i);
                CHECK(bits(val[coff + j]) == bits(v_pre[off + i]));
                CHECK(bits(val[coff + j]) & 0x7FFFFFFFu);
                CHECK(bits(u[off + i]) == 0 && bits(v[off + i]) == 0);
            }
            off += sizes[t];
            coff += cap[t];
        }
    }
    {
        float z[3] = {0.f, 0.f, 0.f};
        uint32_t i3[3];
        float v3[3];
        int64_t tot;
        CHECK(orc_binlocal_select_mask(z, z, 3, 0, 3, i3, v3, &tot) == -1);
        CHECK(orc_binlocal_select_mask(z, z, 3, 1, -1, i3, v3, &tot) == -1);
        CHECK(orc_binlocal_select_mask(z, z, 3, 2, 3, i3, v3, &tot) == 0 && tot == 0);
    }
    // sampled-threshold selector: whole-tensor and line samples, any k and cap
    for (int round = 0; round < 30; ++round) {
        int T = 1 + int(rng() % 4);
        std::vector<int64_t> sizes(T), k(T), cap(T), count(T), total(T);
        std::vector<uint32_t> theta(T);
        int64_t n = 0, C = 0;
        for (int t = 0; t < T; ++t) {
            sizes[t] = sizes_pool[rng() % 10];
            k[t] = sizes[t] ? int64_t(rng() % (sizes[t] + 1)) : 0;
            cap[t] = (rng() % 2) ? sizes[t] : int64_t(rng() % (sizes[t] / 4 + 2));
            n += sizes[t];
            C += cap[t];
        }
        std::vector<float> g(n), u(n), v(n);
        std::normal_distribution<float> nd(0.f, 1e-2f);
        for (int64_t i = 0; i < n; ++i) {
            g[i] = (rng() % 10 == 0) ? 0.f : nd(rng);
            u[i] = nd(rng) * 0.1f;
            v[i] = nd(rng) * 0.1f;
        }
        std::vector<uint32_t> idx(C + 1);
        std::vector<float> val(C + 1);
        double norm;
        float s;
        CHECK(orc_sampled_step(T, sizes.data(), k.data(), cap.data(), g.data(), u.data(),
                               v.data(), 0.9f, 0.5, idx.data(), val.data(), count.data(),
                               total.data(), theta.data(), &norm, &s) == 0);
        int64_t coff = 0;
        for (int t = 0; t < T; ++t) {
            CHECK(count[t] == std::min(total[t], cap[t]));
            CHECK(k[t] > 0 || (total[t] == 0 && theta[t] == 0xFFFFFFFFu));
            for (int64_t j = 1; j < count[t]; ++j) CHECK(idx[coff + j - 1] < idx[coff + j]);
            for (int64_t j = 0; j < count[t]; ++j)
                CHECK((bits(val[coff + j]) & 0x7FFFFFFFu) >= theta[t]);
            coff += cap[t];
        }
    }
    // a corrupt stream is refused without touching memory past the end
    std::vector<uint16_t> runs = {3, 4, 60000};
    std::vector<float> vals = {1.f, 1.f, 1.f};
    std::vector<float> dense(10, 0.f);
    CHECK(orc_decode_accumulate(runs.data(), vals.data(), 3, dense.data(), 10) == -1);
    // capacity and order errors
    uint32_t bad_idx[2] = {5, 5};
    float bad_val[2] = {1.f, 1.f};
    uint16_t r2[4];
    float v2[4];
    CHECK(orc_encode(bad_idx, bad_val, 2, r2, v2, 4) == -2);
    uint32_t far_idx[1] = {200000};
    CHECK(orc_encode(far_idx, bad_val, 1, r2, v2, 2) == -1);
    std::printf("oracle check driver: ok\n");
    return 0;
}
