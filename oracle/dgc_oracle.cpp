/*
 * dgc_oracle.cpp -- plain CPU oracle for the per-learner DGC compressor.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * arrays handed to both by the seeded input generators.
 *
 * Source of the method: the review page "[Paper Review] Deep Gradient
 * Compression: Reducing the Communication Bandwidth for Distributed Training"
 * (nubint.ai), section "Proposed method" (sparsification with local
 * accumulation, 32-bit value / 16-bit zero-run encoding, momentum
 * correction, local gradient clipping, momentum factor masking, warm-up),
 * and its Abstract (99.9% of the exchange is redundant; synchronous SGD
 * gradient exchange).  The page prints no formulas; the readings used here
 * are:
 *   clip:     S = sum g_i^2 in binary64; norm = sqrt(S); if clip > 0 and
 *             norm > clip then s = (float)(clip / norm) else s = 1;
 *             g'_i = fl32(g_i * s)
 *   momentum: u_i = fl32(fl32(m * u_i) + g'_i);  v_i = fl32(v_i + u_i)
 *   select:   key_i = bits(v_i) & 0x7FFFFFFF; the k entries that come first
 *             under (key descending, index ascending)
 *   mask:     u_i = v_i = +0.0f for every selected i, the rest untouched
 *   encode:   per selected j ascending, gap G = j - prev - 1; floor(G/65536)
 *             filler entries (65535, +0.0f) then (G mod 65536, v_j)
 *   decode:   pos = -1; per entry pos += run + 1; dense[pos] += value
 *
 * Arithmetic: binary32 with round-to-nearest-even, no FMA contraction
 * (built with -ffp-contract=off, no fast-math), denormals kept.
 *
 * Sum order of S: the definition fixes none.  Here S is summed in fixed
 * 65536-element blocks (each block left to right in binary64, then the
 * block sums left to right), so the result does not depend on the thread
 * count.  Every other loop is element-wise or per tensor and so has no
 * order to fix.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>
#include <utility>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

const int64_t kNormBlock = 65536;

inline uint32_t f32_bits(float x) {
    uint32_t b;
    std::memcpy(&b, &x, 4);
    return b;
}

inline uint32_t magnitude_key(float x) { return f32_bits(x) & 0x7FFFFFFFu; }

}  // namespace

extern "C" {

/* Number of OpenMP threads the oracle will use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads for later calls (no effect without
 * OpenMP).  Results do not depend on it. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Local gradient clipping (DGC review, "Proposed method": clipping bounds the
 * gradient locally, on each learner).  One norm over the learner's whole
 * gradient.
 * Returns 0; writes the binary64 norm and the binary32 scale.
 */
int orc_clip_scale(const float* g, int64_t n, double clip, double* norm_out,
                   float* scale_out) {
    int64_t nblocks = (n + kNormBlock - 1) / kNormBlock;
    std::vector<double> part((size_t)std::max<int64_t>(nblocks, 1), 0.0);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * kNormBlock, hi = std::min(n, lo + kNormBlock);
        double acc = 0.0;
        for (int64_t i = lo; i < hi; ++i) {
            double x = (double)g[i];
            acc += x * x;
        }
        part[(size_t)b] = acc;
    }
    double S = 0.0;
    for (int64_t b = 0; b < nblocks; ++b) S += part[(size_t)b];
    double norm = std::sqrt(S);
    float s = 1.0f;
    if (clip > 0.0 && norm > clip) s = (float)(clip / norm);
    *norm_out = norm;
    *scale_out = s;
    return 0;
}

/*
 * Momentum correction with local accumulation (DGC review, "Proposed
 * method": momentum correction; small gradients accumulate locally).
 * u <- m*u + g*s ; v <- v + u, each product and sum rounded to binary32.
 */
void orc_momentum(const float* g, int64_t n, float scale, float m, float* u,
                  float* v) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float gs = g[i] * scale;
        float mu = m * u[i];
        float un = mu + gs;
        u[i] = un;
        v[i] = v[i] + un;
    }
}

/*
 * Exact top-k of |v| for one tensor, then momentum factor masking (DGC
 * review, "Proposed method": only the entries of largest magnitude leave the
 * learner; momentum factor masking; the AdaComp page's "Citations in the
 * corpus" rank entries by absolute value).
 *
 * T = the k-th largest key (std::nth_element); every key > T is taken, and
 * of the keys == T the first r = k - #{key > T} in index order.  Writes the
 * k local indices ascending and the signed values of v before masking, then
 * sets u and v to +0.0f at those indices.  Returns the number written (k),
 * or -1 if k is outside [0, n].
 */
int64_t orc_select_mask(float* u, float* v, int64_t n, int64_t k,
                        uint32_t* idx, float* val) {
    if (k < 0 || k > n) return -1;
    if (k == 0) return 0;
    std::vector<uint32_t> keys((size_t)n);
    for (int64_t i = 0; i < n; ++i) keys[(size_t)i] = magnitude_key(v[i]);
    std::vector<uint32_t> work(keys);
    std::nth_element(work.begin(), work.begin() + (k - 1), work.end(),
                     [](uint32_t a, uint32_t b) { return a > b; });
    uint32_t T = work[(size_t)(k - 1)];
    int64_t above = 0;
    for (int64_t i = 0; i < n; ++i) above += keys[(size_t)i] > T;
    int64_t ties_left = k - above;
    int64_t out = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t key = keys[(size_t)i];
        bool take = key > T;
        if (!take && key == T && ties_left > 0) {
            take = true;
            --ties_left;
        }
        if (take) {
            idx[out] = (uint32_t)i;
            val[out] = v[i];
            ++out;
        }
    }
    for (int64_t j = 0; j < out; ++j) {
        u[idx[j]] = 0.0f;
        v[idx[j]] = 0.0f;
    }
    return out;
}

/*
 * Bin-local selection of one tensor, then momentum factor masking.
 *
 * Source: the AdaComp page ("AdaComp : Adaptive Residual Gradient Compression
 * for Data-Parallel Distributed Training"), Abstract (residues are selected
 * locally and the compression rate follows local activity) and "Citations in
 * the corpus" (the Hitchhiker's Guide entry: each layer's residual vector is
 * cut into bins of one fixed size, and the largest absolute value in a bin is
 * that bin's threshold for salient entries).
 *
 * The pages do not say what is compared with a bin's threshold.  Comparing
 * the residual itself would send exactly each bin's maximum, one entry per
 * bin, a fixed rate; the abstract's rate follows local activity.  Reading
 * taken: the residual is v after this step's accumulation; entry i of bin b
 * is salient when v_i is non-zero and v_i looked ahead by this step's update
 * once more, fl32(v_i + u_i), reaches the bin's largest |v|:
 *   bins      b = [b*L, min((b+1)*L, n)), restarting at each tensor
 *   threshold theta_b = max over the bin of key(v_j)
 *   salient   key(v_i) > 0  and  key(fl32(v_i + u_i)) >= theta_b
 * with key(x) = bits(x) & 0x7FFFFFFF (|x| ordered as an unsigned integer).
 * Salient entries are delivered in index order, at most cap of them; the
 * delivered ones are masked (u = v = +0.0f) and the rest stay in the
 * residual untouched.
 *
 * Writes the delivered local indices (ascending) and the signed values of v
 * before masking, and the number of salient entries (delivered or not) into
 * *total.  Returns the number delivered, or -1 if L < 1 or cap < 0.
 */
int64_t orc_binlocal_select_mask(float* u, float* v, int64_t n, int64_t L,
                                 int64_t cap, uint32_t* idx, float* val,
                                 int64_t* total) {
    if (L < 1 || cap < 0) return -1;
    int64_t sal = 0, out = 0;
    for (int64_t lo = 0; lo < n; lo += L) {
        int64_t hi = std::min(n, lo + L);
        uint32_t theta = 0;
        for (int64_t i = lo; i < hi; ++i) theta = std::max(theta, magnitude_key(v[i]));
        for (int64_t i = lo; i < hi; ++i) {
            float ahead = v[i] + u[i];
            if (magnitude_key(v[i]) == 0 || magnitude_key(ahead) < theta) continue;
            ++sal;
            if (out < cap) {
                idx[out] = (uint32_t)i;
                val[out] = v[i];
                ++out;
            }
        }
    }
    for (int64_t j = 0; j < out; ++j) {
        u[idx[j]] = 0.0f;
        v[idx[j]] = 0.0f;
    }
    *total = sal;
    return out;
}

/*
 * MurmurHash3's 32-bit finalizer (fmix32), from its published definition
 * (Austin Appleby, public domain): the counter-based generator that places
 * the sampled lines below.
 */
static uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

extern "C" uint32_t orc_fmix32(uint32_t h) { return fmix32(h); }

/*
 * The sampled threshold theta of one tensor (the first level of the sampled
 * and hierarchical selectors below): the J-th largest key of the sampled
 * lines, J = ceil(S*k/n), S the number of sampled elements; the lines are
 * placed as described for orc_sampled_select_mask.  Needs 1 <= k <= n.
 */
static uint32_t sampled_threshold(const float* v, int64_t n, int64_t k, int32_t t) {
    const int64_t lines = (n + 31) / 32;
    const int64_t ls = n <= 65536 ? lines
                                  : std::min<int64_t>(lines, std::max<int64_t>(512, lines / 256));
    const int64_t stride = lines / ls;
    std::vector<uint32_t> sample;
    for (int64_t j = 0; j < ls; ++j) {
        const uint32_t r = fmix32((uint32_t)j * 0x9E3779B9u ^ (uint32_t)t * 0x7F4A7C15u);
        const int64_t line = j * stride + (int64_t)(r % (uint64_t)stride);
        for (int64_t e = line * 32; e < std::min(n, line * 32 + 32); ++e)
            sample.push_back(magnitude_key(v[e]));
    }
    const int64_t S = (int64_t)sample.size();
    const int64_t J = (S * k + n - 1) / n;
    std::nth_element(sample.begin(), sample.begin() + (J - 1), sample.end(),
                     [](uint32_t a, uint32_t b) { return a > b; });
    return sample[(size_t)(J - 1)];
}

/*
 * Sampled-threshold selection of one tensor (tensor index t in its layout),
 * then momentum factor masking.
 *
 * Source: the DGC review, "Research questions" (RQ4: hierarchical
 * thresholding as a runtime strategy for scalable selection) and "Proposed
 * method" (only large entries are sent).  The page gives no algorithm; the
 * reading taken is the plainest sampled threshold:
 *   sample   the tensor's 32-element lines: all of them if n <= 65536, else
 *            ls = min(lines, max(512, lines / 256)) lines, line j (0 <= j <
 *            ls) being j*stride + fmix32(j*0x9E3779B9 ^ t*0x7F4A7C15) mod
 *            stride, stride = lines / ls (32-bit wrapping products); the
 *            sample is the keys of every element of those lines inside the
 *            tensor, S of them
 *   threshold  theta = the J-th largest sampled key, J = ceil(S*k/n): the
 *            sample's estimate of the k-th largest key
 *   sent     key(v_i) >= theta and v_i != 0, in index order, at most cap of
 *            them delivered and masked (u = v = +0.0f); the rest untouched
 * with key(x) = bits(x) & 0x7FFFFFFF.  k = 0 sends nothing.
 *
 * Writes the delivered indices / values (v before masking), the number of
 * entries at or above the threshold into *total and the threshold into
 * *theta (0xFFFFFFFF for k = 0).  Returns the number delivered, or -1 for a
 * k outside [0, n] or a negative cap.
 */
int64_t orc_sampled_select_mask(float* u, float* v, int64_t n, int64_t k,
                                int64_t cap, int32_t t, uint32_t* idx,
                                float* val, int64_t* total, uint32_t* theta) {
    if (k < 0 || k > n || cap < 0) return -1;
    *total = 0;
    *theta = 0xFFFFFFFFu;
    if (k == 0) return 0;
    const uint32_t th = sampled_threshold(v, n, k, t);
    *theta = th;
    int64_t sent = 0, out = 0;
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t key = magnitude_key(v[i]);
        if (key == 0 || key < th) continue;
        ++sent;
        if (out < cap) {
            idx[out] = (uint32_t)i;
            val[out] = v[i];
            ++out;
        }
    }
    for (int64_t j = 0; j < out; ++j) {
        u[idx[j]] = 0.0f;
        v[idx[j]] = 0.0f;
    }
    *total = sent;
    return out;
}

/*
 * Hierarchical thresholding of one tensor (tensor index t in its layout):
 * the sampled threshold as the first level, an exact select among what
 * passes it as the second, then momentum factor masking.
 *
 * Source: the DGC review, "Research questions" (RQ4 names hierarchical
 * thresholding as a runtime strategy for scalable selection) and "Proposed
 * method" (only large entries are sent).  The page names the strategy only;
 * the reading taken puts two levels on the sampled threshold:
 *   level 1  theta from the sample (sampled_threshold); the survivors are
 *            the non-zero entries with key(v_i) >= theta
 *   level 2  more than k survivors: the k of them that come first under
 *            (key descending, index ascending), the DGC rule; at most k
 *            survivors: all of them
 *   sent     in index order; u = v = +0.0f there, the rest untouched
 * so the count is min(k, survivors), never more than k.  k = 0 sends
 * nothing.
 *
 * Writes the sent indices / values (v before masking, at most k of them),
 * the survivor count into *total and theta into *theta (0xFFFFFFFF for
 * k = 0).  Returns the number sent, or -1 for a k outside [0, n].
 */
int64_t orc_hier_select_mask(float* u, float* v, int64_t n, int64_t k, int32_t t,
                             uint32_t* idx, float* val, int64_t* total,
                             uint32_t* theta) {
    if (k < 0 || k > n) return -1;
    *total = 0;
    *theta = 0xFFFFFFFFu;
    if (k == 0) return 0;
    const uint32_t th = sampled_threshold(v, n, k, t);
    *theta = th;
    // level 1: (key, index) of every survivor
    std::vector<std::pair<uint32_t, uint32_t>> surv;
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t key = magnitude_key(v[i]);
        if (key != 0 && key >= th) surv.push_back({key, (uint32_t)i});
    }
    *total = (int64_t)surv.size();
    // level 2: the first k under (key descending, index ascending)
    if ((int64_t)surv.size() > k) {
        std::sort(surv.begin(), surv.end(),
                  [](const std::pair<uint32_t, uint32_t>& a,
                     const std::pair<uint32_t, uint32_t>& b) {
                      return a.first != b.first ? a.first > b.first : a.second < b.second;
                  });
        surv.resize((size_t)k);
    }
    std::vector<uint32_t> sel;
    for (const auto& s : surv) sel.push_back(s.second);
    std::sort(sel.begin(), sel.end());
    const int64_t out = (int64_t)sel.size();
    for (int64_t j = 0; j < out; ++j) {
        idx[j] = sel[(size_t)j];
        val[j] = v[sel[(size_t)j]];
    }
    for (int64_t j = 0; j < out; ++j) {
        u[idx[j]] = 0.0f;
        v[idx[j]] = 0.0f;
    }
    return out;
}

/*
 * Zero-run encoding of one tensor's sparse gradient (DGC review, "Proposed
 * method": each sent value takes 32 bits and is preceded by the 16-bit
 * length of the zero run before it).  A gap longer than a 16-bit run can say
 * is split by filler entries (65535, +0.0f), each of which stands for 65535
 * zeros plus one slot holding zero.
 * Returns the entry count E, or -1 if cap entries are not enough, or -2 if
 * the indices are not strictly ascending.
 */
int64_t orc_encode(const uint32_t* idx, const float* val, int64_t k,
                   uint16_t* runs, float* vals, int64_t cap) {
    int64_t prev = -1, e = 0;
    for (int64_t j = 0; j < k; ++j) {
        int64_t cur = (int64_t)idx[j];
        if (cur <= prev) return -2;
        int64_t gap = cur - prev - 1;
        while (gap > 65535) {
            if (e >= cap) return -1;
            runs[e] = 65535;
            vals[e] = 0.0f;
            ++e;
            gap -= 65536;
        }
        if (e >= cap) return -1;
        runs[e] = (uint16_t)gap;
        vals[e] = val[j];
        ++e;
        prev = cur;
    }
    return e;
}

/*
 * Decode one tensor's stream and add it into dense (the aggregation of the
 * learners' sparse gradients in synchronous SGD, DGC review Abstract).
 * Returns 0, or -1 if the stream walks past the end of the tensor (dense is
 * then left with the entries before the bad one added).
 */
int orc_decode_accumulate(const uint16_t* runs, const float* vals, int64_t E,
                          float* dense, int64_t n) {
    int64_t pos = -1;
    for (int64_t e = 0; e < E; ++e) {
        pos += (int64_t)runs[e] + 1;
        if (pos >= n) return -1;
        dense[pos] = dense[pos] + vals[e];
    }
    return 0;
}

/*
 * Warm-up sparsity schedule (DGC review, "Proposed method": sparsity rises
 * gradually).  k = ceil(n * num / den) in integer arithmetic, density num/den.
 */
int64_t orc_k_for_density(int64_t n, int64_t num, int64_t den) {
    if (n <= 0 || num <= 0 || den <= 0) return 0;
    return (n * num + den - 1) / den;
}

/*
 * One learner step over T tensors laid end to end: clip over the whole
 * gradient, momentum correction, then per tensor select + mask.  idx/val
 * receive each tensor's k entries back to back (tensor order).  Returns 0,
 * or -1 on a bad k.
 */
int orc_step(int32_t T, const int64_t* sizes, const int64_t* k, const float* g,
             float* u, float* v, float m, double clip, uint32_t* idx,
             float* val, double* norm_out, float* scale_out) {
    int64_t n = 0;
    for (int32_t t = 0; t < T; ++t) n += sizes[t];
    orc_clip_scale(g, n, clip, norm_out, scale_out);
    orc_momentum(g, n, *scale_out, m, u, v);
    std::vector<int64_t> off((size_t)T + 1, 0), koff((size_t)T + 1, 0);
    for (int32_t t = 0; t < T; ++t) {
        if (k[t] < 0 || k[t] > sizes[t]) return -1;
        off[(size_t)t + 1] = off[(size_t)t] + sizes[t];
        koff[(size_t)t + 1] = koff[(size_t)t] + k[t];
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t t = 0; t < T; ++t) {
        int64_t got = orc_select_mask(u + off[(size_t)t], v + off[(size_t)t],
                                      sizes[t], k[t], idx + koff[(size_t)t],
                                      val + koff[(size_t)t]);
        if (got != k[t]) bad = 1;
    }
    return bad ? -1 : 0;
}

/*
 * One learner step with the bin-local selector: clip and momentum as in
 * orc_step, then per tensor orc_binlocal_select_mask with bin length L[t]
 * and capacity cap[t].  Tensor t's delivered entries go to idx/val at offset
 * cap[0] + ... + cap[t-1]; count[t] = number delivered, total[t] = number
 * salient.  Returns 0, or -1 on a bad L or cap.
 */
int orc_binlocal_step(int32_t T, const int64_t* sizes, const int64_t* L,
                      const int64_t* cap, const float* g, float* u, float* v,
                      float m, double clip, uint32_t* idx, float* val,
                      int64_t* count, int64_t* total, double* norm_out,
                      float* scale_out) {
    int64_t n = 0;
    for (int32_t t = 0; t < T; ++t) n += sizes[t];
    orc_clip_scale(g, n, clip, norm_out, scale_out);
    orc_momentum(g, n, *scale_out, m, u, v);
    std::vector<int64_t> off((size_t)T + 1, 0), coff((size_t)T + 1, 0);
    for (int32_t t = 0; t < T; ++t) {
        if (L[t] < 1 || cap[t] < 0) return -1;
        off[(size_t)t + 1] = off[(size_t)t] + sizes[t];
        coff[(size_t)t + 1] = coff[(size_t)t] + cap[t];
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        count[t] = orc_binlocal_select_mask(
            u + off[(size_t)t], v + off[(size_t)t], sizes[t], L[t], cap[t],
            idx + coff[(size_t)t], val + coff[(size_t)t], total + t);
    }
    return 0;
}

/*
 * One learner step with the sampled-threshold selector: clip and momentum as
 * in orc_step, then per tensor orc_sampled_select_mask with target k[t] and
 * capacity cap[t] (outputs at offset cap[0] + ... + cap[t-1]); count[t]
 * delivered, total[t] at or above the threshold, theta[t] the threshold.
 * Returns 0, or -1 on a bad k or cap.
 */
int orc_sampled_step(int32_t T, const int64_t* sizes, const int64_t* k,
                     const int64_t* cap, const float* g, float* u, float* v,
                     float m, double clip, uint32_t* idx, float* val,
                     int64_t* count, int64_t* total, uint32_t* theta,
                     double* norm_out, float* scale_out) {
    int64_t n = 0;
    for (int32_t t = 0; t < T; ++t) n += sizes[t];
    std::vector<int64_t> off((size_t)T + 1, 0), coff((size_t)T + 1, 0);
    for (int32_t t = 0; t < T; ++t) {
        if (k[t] < 0 || k[t] > sizes[t] || cap[t] < 0) return -1;
        off[(size_t)t + 1] = off[(size_t)t] + sizes[t];
        coff[(size_t)t + 1] = coff[(size_t)t] + cap[t];
    }
    orc_clip_scale(g, n, clip, norm_out, scale_out);
    orc_momentum(g, n, *scale_out, m, u, v);
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        count[t] = orc_sampled_select_mask(
            u + off[(size_t)t], v + off[(size_t)t], sizes[t], k[t], cap[t], t,
            idx + coff[(size_t)t], val + coff[(size_t)t], total + t, theta + t);
    }
    return 0;
}

/*
 * One learner step with the hierarchical selector: clip and momentum as in
 * orc_step, then per tensor orc_hier_select_mask with target k[t].  Tensor
 * t's sent entries go to idx/val at offset k[0] + ... + k[t-1]; count[t] =
 * number sent (min(k[t], total[t])), total[t] = survivors of the first
 * level, theta[t] the threshold.  Returns 0, or -1 on a bad k.
 */
int orc_hier_step(int32_t T, const int64_t* sizes, const int64_t* k, const float* g,
                  float* u, float* v, float m, double clip, uint32_t* idx, float* val,
                  int64_t* count, int64_t* total, uint32_t* theta, double* norm_out,
                  float* scale_out) {
    int64_t n = 0;
    for (int32_t t = 0; t < T; ++t) n += sizes[t];
    std::vector<int64_t> off((size_t)T + 1, 0), koff((size_t)T + 1, 0);
    for (int32_t t = 0; t < T; ++t) {
        if (k[t] < 0 || k[t] > sizes[t]) return -1;
        off[(size_t)t + 1] = off[(size_t)t] + sizes[t];
        koff[(size_t)t + 1] = koff[(size_t)t] + k[t];
    }
    orc_clip_scale(g, n, clip, norm_out, scale_out);
    orc_momentum(g, n, *scale_out, m, u, v);
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t t = 0; t < T; ++t) {
        count[t] = orc_hier_select_mask(
            u + off[(size_t)t], v + off[(size_t)t], sizes[t], k[t], t,
            idx + koff[(size_t)t], val + koff[(size_t)t], total + t, theta + t);
    }
    return 0;
}

/*
 * Commutative, shared-index compression (the ScaleComp abstract on the
 * taxoreview.com page: the learners' gradient distributions are alike, which
 * allows a commutative compressor whose communication cost does not grow
 * with the number of learners and which an all-reduce can carry).  The page
 * gives no mechanism; the reading taken here is the plainest one:
 *   - every learner of a step sends its v at one shared index set S per
 *     tensor; keeping the same indices on every learner is what makes the
 *     compressor commute with the sum over learners (selection at fixed
 *     indices is linear);
 *   - S is one learner's exact top-k (the DGC rule, ties toward the lower
 *     index), that learner being the step's leader, t mod W;
 *   - each learner masks u and v at S (momentum factor masking at the
 *     shared set) and keeps the rest as its residual.
 * This function is what a learner other than the leader does with S:
 * writes val[j] = v[idx[j]] (signed, before masking) for j < k, then sets
 * u and v to +0.0f at those indices.  idx must be strictly ascending and
 * below n.  Returns k, or -1 if k < 0 or the indices are not so.
 */
int64_t orc_shared_gather_mask(float* u, float* v, int64_t n, const uint32_t* idx,
                               int64_t k, float* val) {
    if (k < 0) return -1;
    int64_t prev = -1;
    for (int64_t j = 0; j < k; ++j) {
        int64_t i = (int64_t)idx[j];
        if (i <= prev || i >= n) return -1;
        prev = i;
    }
    for (int64_t j = 0; j < k; ++j) val[j] = v[idx[j]];
    for (int64_t j = 0; j < k; ++j) {
        u[idx[j]] = 0.0f;
        v[idx[j]] = 0.0f;
    }
    return k;
}

/*
 * One step of a learner that is not the leader: clip and momentum as in
 * orc_step, then per tensor orc_shared_gather_mask with the shared local
 * indices idx[koff_t .. koff_t + k[t]) (koff_t = k[0] + ... + k[t-1], the
 * layout orc_step writes).  val receives the values at the same offsets.
 * Returns 0, or -1 on a bad k or bad indices.
 */
int orc_shared_step(int32_t T, const int64_t* sizes, const int64_t* k,
                    const uint32_t* idx, const float* g, float* u, float* v,
                    float m, double clip, float* val, double* norm_out,
                    float* scale_out) {
    int64_t n = 0;
    std::vector<int64_t> off((size_t)T + 1, 0), koff((size_t)T + 1, 0);
    for (int32_t t = 0; t < T; ++t) {
        if (k[t] < 0 || k[t] > sizes[t]) return -1;
        off[(size_t)t + 1] = off[(size_t)t] + sizes[t];
        koff[(size_t)t + 1] = koff[(size_t)t] + k[t];
        n += sizes[t];
    }
    orc_clip_scale(g, n, clip, norm_out, scale_out);
    orc_momentum(g, n, *scale_out, m, u, v);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t t = 0; t < T; ++t) {
        int64_t got = orc_shared_gather_mask(u + off[(size_t)t], v + off[(size_t)t],
                                             sizes[t], idx + koff[(size_t)t], k[t],
                                             val + koff[(size_t)t]);
        if (got != k[t]) bad = 1;
    }
    return bad ? -1 : 0;
}

/*
 * The aggregate of shared-index compression: the element-wise sum of the W
 * learners' value vectors (each K long, the same index set), in learner
 * order from +0.0: out[j] = fl(...fl(fl(+0 + vals[0][j]) + vals[1][j])...
 * + vals[W-1][j]).  This is the reduction an all-reduce of K floats carries;
 * its size does not depend on W.
 */
void orc_shared_sum(int32_t W, const float* const* vals, int64_t K, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; ++j) {
        float s = 0.0f;
        for (int32_t w = 0; w < W; ++w) s = s + vals[w][j];
        out[j] = s;
    }
}

}  /* extern "C" */
