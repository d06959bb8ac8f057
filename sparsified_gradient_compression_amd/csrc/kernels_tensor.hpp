// kernels_tensor.hpp -- the exact top-k step in one workgroup per tensor,
// for layouts whose tensors all hold at most 2^22 elements.
//
// Method: DGC review page (nubint.ai), "Proposed method" -- only the largest
// |v| entries leave a learner; the rest accumulates; momentum factor
// masking.  Selection is exact top-k per tensor, ties to the lower index.
//
// The spread passes of kernels_compress.hpp take about twenty dependent
// launches per step, each ~4.7 us even with almost nothing to do.  Here the
// same step is four launches:
//   norm_partial   binary64 sum of g^2 (with clipping)
//   window_tensor  one 1024-thread workgroup per tensor: the clip scale from
//                  the norm partials (the same reduction as k_norm_final),
//                  then both levels of the sample window, each a pass over
//                  the sampled lines: every line of a tensor of up to 16384
//                  elements, else max(512, lines / 256) hashed lines as in
//                  kernels_compress.hpp (so small tensors get a window too)
//   fused          the element-wise pass (unchanged)
//   finish_tensor  one 1024-thread workgroup per tensor: the pieces' counts
//                  (source choice), the runs gathered into the ordered
//                  candidate list with the keys kept in LDS, the k-th
//                  largest key over those keys, and the index-ordered emit
// Decisions, results and the per-tensor record are the spread passes'.
#pragma once

#include "dgc_device.hpp"
#include "kernels_compress.hpp"

namespace dgc {

// Layouts whose tensors all hold at most this many elements take the
// per-tensor kernels: a tensor samples min(lines, max(512, lines / 256))
// of its 32-element lines, at most 512 (4 rounds of 128 lines for one
// workgroup), and has at most 4096 pieces (at most 4 per thread).  Larger
// tensors have lists too long for one workgroup to walk quickly (one CU
// against the spread passes' whole chip).
constexpr int64_t kTensorPathMaxN = int64_t(1) << 22;
constexpr int kWtLinesPerRound = kTsThreads / kLineLanes;  // 8 lanes per line
constexpr int kWtRounds = int(kMinSampleLines / kWtLinesPerRound);  // 4
static_assert((kTensorPathMaxN / kLine) / 256 <= kMinSampleLines,
              "a per-tensor window samples at most kMinSampleLines lines");
// Candidate-list items held in LDS by finish_tensor (longer lists go to
// the ordered list in memory instead).
constexpr int kFinItems = 10240;
// Consecutive pieces per thread in finish_tensor (4096 pieces = 2^22
// elements over 1024 threads).
constexpr int kFinPieces = int((kTensorPathMaxN / kPiece + kTsThreads - 1) / kTsThreads);
constexpr int kFinEmitUnroll = 4;  // 64-item rounds loaded together per wave
// Lists in LDS of at most this many items select by counting (fin_direct).
constexpr int kFinDirect = 128;
// Keys per thread per pass of the selection rounds, and 64-item rounds per
// batch of the wave gather (code unrolled this many times is fetched cold at
// every launch, and most tensors are short).
constexpr int kFinUnroll = 4;
constexpr int kFinBatch = 4;

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Inclusive max over the wave with the DPP moves of wave_inclusive_scan; a
// lane a move cannot reach gets 0, the identity here.
#define DGC_DPP(x, ctrl, rows) \
    uint32_t(__builtin_amdgcn_update_dpp(0, int(x), (ctrl), (rows), 0xF, true))
__device__ __forceinline__ uint32_t wave_inclusive_max(uint32_t x) {
    x = max(x, DGC_DPP(x, 0x111, 0xF));
    x = max(x, DGC_DPP(x, 0x112, 0xF));
    x = max(x, DGC_DPP(x, 0x114, 0xF));
    x = max(x, DGC_DPP(x, 0x118, 0xF));
    x = max(x, DGC_DPP(x, 0x142, 0xA));
    x = max(x, DGC_DPP(x, 0x143, 0xC));
    return x;
}
#undef DGC_DPP
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
    return uint32_t(__builtin_amdgcn_readlane(int(x), lane));
}

// Exclusive scan over the block; `row` (kTsWaves words) is not reused.
__device__ __forceinline__ uint32_t fin_block_scan(uint32_t x, uint32_t* row, uint32_t& total) {
    const int lane = lane_id();
    const int wid = int(threadIdx.x) >> 6;
    const uint32_t inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) row[wid] = inc;
    __syncthreads();
    uint32_t wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w) {
        const uint32_t s = row[w];
        if (w < wid) wpre += s;
        tot += s;
    }
    total = tot;
    return wpre + inc - x;
}

// S = the binary64 sum of the norm partials in k_norm_final's order: its
// 256 threads are this block's first four waves, each summing a strided
// share, then a butterfly per wave and the four wave sums in order.  The
// same operations in the same order give the same bits.
__device__ __forceinline__ double norm_sum_fixed(const double* __restrict__ partial,
                                                 int64_t nb, double* dl) {
    const int tid = int(threadIdx.x);
    if (tid < kBlock) {
        double a = 0.0;
        for (int64_t i = tid; i < nb; i += kBlock) a += partial[i];
#pragma unroll
        for (int d = kWave / 2; d >= 1; d >>= 1) a += __shfl_xor(a, d, kWave);
        if (lane_id() == 0) dl[tid >> 6] = a;
    }
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) s += dl[w];
    return s;
}

// One 1024-thread workgroup per tensor (grid = T).  Block 0 also writes the
// call's scalars (norm and scale).  Sets lo_key (the candidate threshold),
// wbin, wabove and wj of the tensor's record; lo_key = kNoKey means no
// candidates (k = 0, or the forced dense path).  The window: j =
// ceil(mu + 4 sqrt(mu) + 6) with mu = S k / n_t for S sampled keys; lo is
// the lower edge of the 21-bit bin that holds the j-th largest sampled key,
// or 0 when j > S.  The sample's loads go out before the norm partials', so
// the two waits overlap; its at most 16 keys per thread stay in registers
// for both levels.
__global__ __launch_bounds__(kTsThreads) void k_window_tensor(
    const float* __restrict__ g, const float* __restrict__ u, const float* __restrict__ v,
    DevLayout L, DevK K, const int64_t* __restrict__ wlines,
    const double* __restrict__ partial, int64_t nb,
    double clip, int clip_on, Scalars* __restrict__ sc, double* __restrict__ out_norm,
    float* __restrict__ out_scale, TensorState* __restrict__ ts, float m, int force_dense) {
    __shared__ uint32_t h[kBins0];
    __shared__ uint32_t h1[1024];
    __shared__ uint32_t rows[2 * kTsWaves];  // one scan row per level
    __shared__ uint32_t pick[2];
    __shared__ double dl[kWavesPerBlock];
    const int t = blockIdx.x;
    const int tid = int(threadIdx.x);
    const int64_t k = K.k[t];
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    const int64_t ls = wlines[t];  // at most kWtRounds * kWtLinesPerRound
    const bool active = k > 0 && !force_dense && ls > 0 && nt > 0;  // uniform
    // zero on entry (a barrier follows before any use)
    for (int b = tid; b < kBins0; b += kTsThreads) h[b] = 0;
    for (int b = tid; b < 1024; b += kTsThreads) h1[b] = 0;
    if (tid == 0) pick[0] = kNoKey;
    // Sampled line j (j < ls) starts at line j * stride + mix32(j * 0x9E3779B9
    // ^ t * 0x7F4A7C15) mod stride; stride = 1 samples every line.  Lane gl of
    // the 8-lane group grp takes elements 4 gl .. 4 gl + 3 of lines grp,
    // grp + 128, grp + 256, grp + 384.
    const int64_t lines = (nt + kLine - 1) / kLine;
    const int64_t stride = active ? lines / ls : 1;
    const int grp = tid / kLineLanes, gl = tid % kLineLanes;
    float gg[kWtRounds][4], uu[kWtRounds][4], vv[kWtRounds][4];
    bool ok[kWtRounds][4];
#pragma unroll
    for (int r = 0; r < kWtRounds; ++r) {
        const int64_t j = int64_t(r) * kWtLinesPerRound + grp;
        const bool line = active && j < ls;
        // stride < 2^32 (a tensor has fewer than 2^32 elements)
        const uint32_t hs = mix32(uint32_t(j) * 0x9E3779B9u ^ uint32_t(t) * 0x7F4A7C15u);
        const int64_t e = line ? (j * stride + int64_t(hs % uint32_t(stride))) * kLine + 4 * gl
                               : int64_t(0);
        const float *pg = g + o + e, *pu = u + o + e, *pv = v + o + e;
        if (line && e + 4 <= nt &&
            ((reinterpret_cast<uintptr_t>(pg) | reinterpret_cast<uintptr_t>(pu) |
              reinterpret_cast<uintptr_t>(pv)) & 15) == 0) {
            const float4 a = *reinterpret_cast<const float4*>(pg);
            const float4 bb = *reinterpret_cast<const float4*>(pu);
            const float4 c = *reinterpret_cast<const float4*>(pv);
            gg[r][0] = a.x; gg[r][1] = a.y; gg[r][2] = a.z; gg[r][3] = a.w;
            uu[r][0] = bb.x; uu[r][1] = bb.y; uu[r][2] = bb.z; uu[r][3] = bb.w;
            vv[r][0] = c.x; vv[r][1] = c.y; vv[r][2] = c.z; vv[r][3] = c.w;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) ok[r][c4] = true;
        } else {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                ok[r][c4] = line && e + c4 < nt;
                gg[r][c4] = ok[r][c4] ? pg[c4] : 0.0f;
                uu[r][c4] = ok[r][c4] ? pu[c4] : 0.0f;
                vv[r][c4] = ok[r][c4] ? pv[c4] : 0.0f;
            }
        }
    }
    // the scale
    float s = 1.0f;
    if (clip_on) {  // uniform
        const double S = norm_sum_fixed(partial, nb, dl);
        const double norm = sqrt(S);
        if (clip > 0.0 && norm > clip) s = float(clip / norm);
        if (t == 0 && tid == 0) {
            sc->norm = norm;
            sc->scale = s;
            if (out_norm) *out_norm = norm;
            if (out_scale) *out_scale = s;
        }
    } else {
        if (t == 0 && tid == 0) {
            sc->norm = -1.0;
            sc->scale = 1.0f;
            if (out_norm) *out_norm = -1.0;
            if (out_scale) *out_scale = 1.0f;
        }
        __syncthreads();  // h, h1 and pick cleared
    }
    if (tid == 0) {
        ts[t].lo_key = kNoKey;
        ts[t].wbin = kNoKey;
        ts[t].wabove = 0;
        ts[t].wj = 0;
        ts[t].floor = 0;  // exact top-k
    }
    if (!active) return;  // uniform
    uint32_t key[kWtRounds][4];
#pragma unroll
    for (int r = 0; r < kWtRounds; ++r)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            momentum_update(gg[r][c4], s, m, uu[r][c4], vv[r][c4]);
            key[r][c4] = ok[r][c4] ? mag_key(vv[r][c4]) : kNoKey;
        }
    // level 0: the top 11 bits
#pragma unroll
    for (int r = 0; r < kWtRounds; ++r)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            if (key[r][c4] != kNoKey) atomicAdd(&h[key[r][c4] >> 20], 1u);
    __syncthreads();
    // thread tid owns bins 2047 - 2 tid and 2046 - 2 tid (descending)
    const uint32_t c0 = h[kBins0 - 1 - 2 * tid], c1 = h[kBins0 - 2 - 2 * tid];
    uint32_t total;
    const uint32_t above = fin_block_scan(c0 + c1, rows, total);
    const double mu = double(total) * double(k) / double(nt);
    const double jd = ceil(mu + 4.0 * sqrt(mu) + 6.0);
    if (jd > double(total)) {  // uniform: (nearly) everything is a candidate
        if (tid == 0) ts[t].lo_key = 0;
        return;
    }
    const uint32_t j = uint32_t(jd);
    if (above < j && j <= above + c0) {
        pick[0] = uint32_t(kBins0 - 1 - 2 * tid);
        pick[1] = above;
    } else if (above + c0 < j && j <= above + c0 + c1) {
        pick[0] = uint32_t(kBins0 - 2 - 2 * tid);
        pick[1] = above + c0;
    }
    __syncthreads();
    const uint32_t wbin = pick[0], wabove = pick[1];
    if (wbin == kNoKey) return;  // uniform; cannot happen when j <= total
    // level 1: the next 10 bits of the keys in bin wbin
#pragma unroll
    for (int r = 0; r < kWtRounds; ++r)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            if (key[r][c4] != kNoKey && (key[r][c4] >> 20) == wbin)
                atomicAdd(&h1[(key[r][c4] >> 10) & 1023u], 1u);
    __syncthreads();
    const uint32_t c2 = h1[1023 - tid];
    uint32_t tot1;
    const uint32_t ab1 = fin_block_scan(c2, rows + kTsWaves, tot1);
    const uint32_t jr = j - wabove;
    if (ab1 < jr && jr <= ab1 + c2) {
        ts[t].lo_key = (wbin << 20) | (uint32_t(1023 - tid) << 10);
        ts[t].wbin = wbin;
        ts[t].wabove = wabove;
        ts[t].wj = j;
    }
}

// The selection rounds of finish_tensor share one histogram h (2048
// bins), zero on entry: each round reads its bins and zeroes them again,
// three barriers apart from the next round's increments.  Each round has
// its own scan row (kTsWaves words) and pick (2 words, kNoKey in pick[0]
// on entry), so nothing needs a barrier before reuse: a round costs three
// barriers (counts done; wave sums posted; pick posted).


// After the counts are in h[0, bins): the bin, counted from the top, that
// holds the krem-th largest, into pick; the bins are zeroed again.
template <int bins>
__device__ __forceinline__ void fin_pick(uint32_t* h, uint32_t krem, uint32_t* row,
                                         uint32_t* pick) {
    constexpr int per = (bins + kTsThreads - 1) / kTsThreads;
    const int tid = int(threadIdx.x);
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        const int b = bins - 1 - (tid * per + q);
        c[q] = b >= 0 ? h[b] : 0u;
        if (b >= 0) h[b] = 0;
        mine += c[q];
    }
    uint32_t total;
    uint32_t run = fin_block_scan(mine, row, total);
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (run < krem && krem <= run + c[q]) {
            pick[0] = uint32_t(bins - 1 - (tid * per + q));
            pick[1] = krem - run;
        }
        run += c[q];
    }
    __syncthreads();
}

// Digit D of the radix select over key_at(0 .. len-1): histogram of the
// keys that match the prefix (wave-aggregated increments for the top
// digit), then the bin holding the krem-th largest; extends the prefix and
// reduces krem.  Returns false (uniformly) if no bin holds it.
template <int D, typename KeyAt>
__device__ __forceinline__ bool fin_digit(const KeyAt& key_at, int64_t len, uint32_t& prefix,
                                          uint32_t& krem, uint32_t* h, uint32_t* row,
                                          uint32_t* pick) {
    constexpr int shift = Digit<D>::shift, bits = Digit<D>::bits;
    constexpr int bins = 1 << bits;
    constexpr uint32_t dmask = uint32_t(bins) - 1u;
    const int tid = int(threadIdx.x);
    for (int64_t i0 = 0; i0 < len; i0 += int64_t(kTsThreads) * kFinUnroll) {
        uint32_t key[kFinUnroll];
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            const int64_t i = i0 + int64_t(q) * kTsThreads + tid;
            key[q] = i < len ? key_at(i) : kNoKey;
        }
        // the candidates' top digit crowds into a few bins: aggregate per
        // wave; the lower digits spread out, one atomic per key
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            if (D == 0) {
                hist_inc(h, key[q] >> shift, key[q] != kNoKey);
            } else if (key[q] != kNoKey && (key[q] >> (shift + bits)) == prefix) {
                atomicAdd(&h[(key[q] >> shift) & dmask], 1u);
            }
        }
    }
    __syncthreads();
    fin_pick<bins>(h, krem, row, pick);
    const uint32_t b = pick[0], kr = pick[1];
    if (b == kNoKey) return false;
    prefix = (prefix << bits) | b;
    krem = kr;
    return true;
}

// The top 21 bits of the krem-th largest key among keys_at(0 .. len-1),
// all of them at least lo21 << 10, from one histogram of (key >> 10) - lo21
// (bin 2047 collects everything 2047 bins or more above lo21, counted in
// registers: most keys of a long list land there).  Sets prefix to those
// 21 bits and reduces krem; returns false (uniformly) when the krem-th key
// lies in the open top bin, or a key is below lo21 << 10, so that the
// caller takes the plain digits.
template <typename KeyAt>
__device__ __forceinline__ bool fin_prefix21(const KeyAt& key_at, int64_t len, uint32_t lo21,
                                             uint32_t& prefix, uint32_t& krem, uint32_t* h,
                                             uint32_t* row, uint32_t* pick) {
    constexpr int bins = kHistBins;  // 2048
    const int tid = int(threadIdx.x);
    int below = 0;
    uint32_t open = 0;
    for (int64_t i0 = 0; i0 < len; i0 += int64_t(kTsThreads) * kFinUnroll) {
        uint32_t key[kFinUnroll];
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            const int64_t i = i0 + int64_t(q) * kTsThreads + tid;
            key[q] = i < len ? key_at(i) : kNoKey;
        }
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            const bool in = key[q] != kNoKey;
            const uint32_t p21 = key[q] >> 10;
            below |= in && p21 < lo21;
            const uint32_t d = p21 - lo21;
            if (in && p21 >= lo21) {
                if (d < uint32_t(bins - 1)) atomicAdd(&h[d], 1u);
                else ++open;
            }
        }
    }
    open = lane_value(wave_inclusive_scan(open), kWave - 1);
    if (lane_id() == 0 && open) atomicAdd(&h[bins - 1], open);
    below = __syncthreads_or(below);
    fin_pick<bins>(h, krem, row, pick);
    const uint32_t b = pick[0], kr = pick[1];
    if (below || b == kNoKey || b == uint32_t(bins - 1)) return false;
    prefix = lo21 + b;
    krem = kr;
    return true;
}

// The krem-th largest of the keys key_at(0 .. len-1), len <= kTsThreads,
// by counting: thread i compares its key with every other (broadcast LDS
// reads); the key with g keys above it and e equal, g < krem <= g + e, is
// the k-th largest.  Sets prefix to that key and krem to krem - g (the keys
// equal to it that are taken); returns false (uniformly) if none is.
template <typename KeyAt>
__device__ __forceinline__ bool fin_direct(const KeyAt& key_at, int64_t len, uint32_t& prefix,
                                           uint32_t& krem, uint32_t* pick) {
    const int tid = int(threadIdx.x);
    if (tid < len) {
        const uint32_t key = key_at(tid);
        uint32_t g = 0, e = 0;
        for (int64_t j = 0; j < len; ++j) {
            const uint32_t kj = key_at(j);
            g += kj > key;
            e += kj == key;
        }
        if (g < krem && krem <= g + e) {  // every such thread holds the same key
            pick[0] = key;
            pick[1] = krem - g;
        }
    }
    __syncthreads();
    if (pick[0] == kNoKey) return false;
    prefix = pick[0];
    krem = pick[1];
    return true;
}

// After fin_prefix21: the keys whose top 21 bits are the prefix (one bin
// of 1024 key values) copied into lst (wave-aggregated positions from the
// counter *cnt, zero on entry), then the krem-th largest of them by
// counting.  Returns 1 with prefix the k-th largest key T and krem the keys
// equal to it that are taken; 0 if none is; -1 (uniformly) when more than
// kTsThreads keys share the bin, so that the caller takes digit 2.
template <typename KeyAt>
__device__ __forceinline__ int fin_low10(const KeyAt& key_at, int64_t len, uint32_t& prefix,
                                         uint32_t& krem, uint32_t* lst, uint32_t* cnt,
                                         uint32_t* pick) {
    const int tid = int(threadIdx.x);
    const uint32_t p21 = prefix;
    for (int64_t i0 = 0; i0 < len; i0 += int64_t(kTsThreads) * kFinUnroll) {
        uint32_t key[kFinUnroll];
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            const int64_t i = i0 + int64_t(q) * kTsThreads + tid;
            key[q] = i < len ? key_at(i) : kNoKey;
        }
#pragma unroll
        for (int q = 0; q < kFinUnroll; ++q) {
            const bool in = key[q] != kNoKey && (key[q] >> 10) == p21;
            const uint64_t bm = __ballot(in);
            if (bm) {  // uniform
                uint32_t base = 0;
                if (lane_id() == 0) base = atomicAdd(cnt, uint32_t(__popcll(bm)));
                base = lane_value(base, 0);
                const uint32_t pos = base + uint32_t(__popcll(bm & lanemask_lt()));
                if (in && pos < uint32_t(kTsThreads)) lst[pos] = key[q];
            }
        }
    }
    __syncthreads();
    const uint32_t m = *cnt;
    if (m > uint32_t(kTsThreads)) return -1;
    return fin_direct([&](int64_t j) -> uint32_t { return lst[j]; }, int64_t(m), prefix, krem,
                      pick) ? 1 : 0;
}

// Orders this wave's LDS accesses before its later ones (lanes exchange
// data through LDS with no block barrier).
__device__ __forceinline__ void fin_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Exclusive scan over the 1024-thread block with the block total, and
// whether any thread's flag is set, in one exchange.  `lds` holds
// 2 kTsWaves values.
__device__ __forceinline__ uint32_t ts_block_scan_any(uint32_t x, int flag, uint32_t* lds,
                                                      uint32_t& total, int& any) {
    const int lane = lane_id();
    const int wid = int(threadIdx.x) >> 6;
    const uint32_t inc = wave_inclusive_scan(x);
    const bool wf = __ballot(flag != 0) != 0;
    if (lane == kWave - 1) {
        lds[wid] = inc;
        lds[kTsWaves + wid] = wf ? 1u : 0u;
    }
    __syncthreads();
    uint32_t wpre = 0, tot = 0, f = 0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w) {
        const uint32_t s = lds[w];
        if (w < wid) wpre += s;
        tot += s;
        f |= lds[kTsWaves + w];
    }
    __syncthreads();
    total = tot;
    any = int(f);
    return wpre + inc - x;
}

// One 1024-thread workgroup per tensor (grid = T), after k_fused.
//   1. the tensor's pieces (at most 4096, up to four consecutive ones per
//      thread, counts kept in registers; one block scan gives the total and
//      every piece's offset): candidate total and overflow -> the source
//      (the candidate list when
//      no piece overflowed and there are k to capacity of them, else the
//      whole tensor), as k_group_scan decides it
//   2. list: the pieces' runs copied in piece order into LDS (index, v,
//      saved u; each wave copies the runs of its own threads' pieces, and
//      finds an item's piece from start-of-run marks; lists longer than
//      kFinItems go to the ordered list in memory instead, each item
//      finding its piece by binary search); whole tensor: the slotted
//      candidates' u and v put back (the fused pass masked them)
//   3. T and r: lists of at most kFinDirect items in LDS by counting;
//      else the top 21 bits from one histogram above the window edge, then
//      the last 10 by counting among the keys that share them (digit 2
//      when more than 1024 do); else the three radix digits
//   4. the emit of k_select_tensor: sent items to the outputs in index
//      order; on the list, the items not sent get u and v back; on the whole
//      tensor, u = v = +0 at the sent ones
// and the tensor's record (total, overflow, mode, len, T, r).
__global__ __launch_bounds__(kTsThreads) void k_finish_tensor(
    DevLayout L, DevK K, TensorState* __restrict__ ts, const CandSlot* __restrict__ slots,
    const uint32_t* __restrict__ run_cnt, float* __restrict__ u, float* __restrict__ v,
    uint32_t* __restrict__ olist_i, float* __restrict__ olist_v,
    float* __restrict__ olist_u, uint32_t* __restrict__ out_idx,
    float* __restrict__ out_val, int64_t* __restrict__ out_count,
    Scalars* __restrict__ sc) {
    __shared__ uint32_t sidx[kFinItems];
    __shared__ float sv[kFinItems];
    // the saved u as bits; before that, the start-of-run marks of the gather
    __shared__ uint32_t su[kFinItems];
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t pre[kFinPieces * kTsThreads];
    __shared__ uint32_t lds[2 * kTsWaves];
    __shared__ uint32_t wcnt[2 * kTsWaves];
    __shared__ uint32_t rows[4 * kTsWaves];  // the selection rounds' scan rows
    __shared__ uint32_t pick[10];            // and picks
    __shared__ uint32_t lcnt;                // fin_low10's counter
    const int t = blockIdx.x;
    const int tid = int(threadIdx.x);
    // zero on entry to the selection rounds (barriers follow)
    for (int b = tid; b < kHistBins; b += kTsThreads) h[b] = 0;
    if (tid < 10) pick[tid] = kNoKey;
    if (tid == 0) lcnt = 0;
    const int64_t k = K.k[t];
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    const int64_t p0 = L.pbase[t], np = L.pbase[t + 1] - p0;
    const uint32_t pcap = uint32_t(L.pcap[t]);
    const int64_t cap = L.obase[t + 1] - L.obase[t];
    const uint32_t lo_key = ts[t].lo_key;  // the window's lower edge
    const uint32_t fl = ts[t].floor;       // 0, or the hierarchical floor
    if (np > int64_t(kFinPieces) * kTsThreads) {  // uniform; the host keeps such layouts off
        if (tid == 0) latch_error(sc, kErrInternal);
        return;
    }
    // 1. candidates and overflow: thread tid owns the consecutive pieces
    // [q0, q1) (at most kFinPieces, spread evenly over the threads), so one
    // block scan gives the total and each piece's offset in the list
    const int64_t q0 = int64_t(tid) * np / kTsThreads;
    const int64_t q1 = int64_t(tid + 1) * np / kTsThreads;
    uint32_t cnt[kFinPieces];
    uint32_t mine = 0;
    int over = 0;
#pragma unroll
    for (int c = 0; c < kFinPieces; ++c) {
        const int64_t q = q0 + c;
        uint32_t x = (k > 0 && q < q1) ? run_cnt[p0 + q] : 0u;
        if (x > pcap) {  // overflowed: no slots, nothing masked
            over = 1;
            x = 0;
        }
        cnt[c] = x;
        mine += x;
    }
    uint32_t C;
    const uint32_t base = ts_block_scan_any(mine, over, lds, C, over);
    const uint32_t mode = select_mode(k, C, over, uint64_t(cap), lo_key, fl);
    // the hierarchical selector's whole survivor list of at most k: all sent
    const bool all = mode == kModeList && send_all(k, C, fl);
    const int64_t len = mode == kModeList ? int64_t(C) : nt;
    if (tid == 0) {
        ts[t].total = C;
        ts[t].overflow = uint32_t(over);
        ts[t].mode = mode;
        ts[t].len = uint32_t(len);
        ts[t].prefix = 0;
        ts[t].krem = all ? 0u : uint32_t(k > 0 ? k : 0);
        ts[t].done21 = all ? kDoneAll : 0u;
    }
    if (mode == kModeSkip) {  // uniform
        if (out_count && tid == 0) out_count[t] = 0;
        return;
    }
    const bool list = mode == kModeList;
    const bool in_lds = list && len <= kFinItems;
    // 2. gather, into LDS (the list when it fits), else into the ordered
    // list in memory or back into u and v
    bool gbad = false;
    if (C > 0) {  // uniform
        const CandSlot* src0 = slots + L.slbase[t];
        const int64_t d0 = L.obase[t];
        uint32_t run = base;
#pragma unroll
        for (int c = 0; c < kFinPieces; ++c) {
            if (q0 + c < q1) pre[q0 + c] = run;
            run += cnt[c];
        }
        const int lane = lane_id();
        if (in_lds) {  // uniform
            // The wave's own pieces hold the list's items [wb, we), and the
            // first of them starts a run.  Mark each run's start with its
            // piece + 1 (every other item 0): the running max of the marks
            // is then the piece of each item.  Marks, offsets and items are
            // the wave's own: no block barrier.
            // (every index below is also checked against the buffers, so
            // that no count can move an access out of them)
            const uint32_t wb = lane_value(base, 0);
            const uint32_t we = min(lane_value(base + mine, kWave - 1), uint32_t(kFinItems));
            for (uint32_t i = wb + uint32_t(lane); i < we; i += kWave) su[i] = 0u;
            fin_wave_sync();
            run = base;
#pragma unroll
            for (int c = 0; c < kFinPieces; ++c) {
                if (cnt[c] && run < we) su[run] = uint32_t(q0 + c) + 1u;
                run += cnt[c];
            }
            fin_wave_sync();
            uint32_t carry = 0;  // the piece + 1 of the item before a round
            for (uint32_t i0 = wb; i0 < we; i0 += uint32_t(kWave * kFinBatch)) {
                // the rounds' running maxima independently, then the carries
                uint32_t pc[kFinBatch];
#pragma unroll
                for (int b = 0; b < kFinBatch; ++b) {
                    const uint32_t i = i0 + uint32_t(b * kWave + lane);
                    pc[b] = wave_inclusive_max(i < we ? su[i] : 0u);
                }
#pragma unroll
                for (int b = 0; b < kFinBatch; ++b) {
                    const uint32_t last = lane_value(pc[b], kWave - 1);
                    pc[b] = max(pc[b], carry);  // >= 1 below we
                    carry = max(carry, last);
                }
                CandSlot it[kFinBatch];
                bool got[kFinBatch];
#pragma unroll
                for (int b = 0; b < kFinBatch; ++b) {
                    const uint32_t i = i0 + uint32_t(b * kWave + lane);
                    const uint32_t j = pc[b] - 1u;
                    got[b] = false;
                    if (i < we && j < uint32_t(np)) {
                        const uint32_t off = i - pre[j];
                        got[b] = off < pcap;
                        if (got[b]) it[b] = src0[int64_t(j) * pcap + off];
                    }
                    if (i < we && !got[b]) gbad = true;
                }
                // su[i] (a mark) is read only by the lane that writes it here
#pragma unroll
                for (int b = 0; b < kFinBatch; ++b) {
                    const uint32_t i = i0 + uint32_t(b * kWave + lane);
                    if (got[b]) {
                        sidx[i] = it[b].idx;
                        sv[i] = it[b].v;
                        su[i] = __float_as_uint(it[b].u);
                    }
                }
            }
        } else {
            // Consecutive threads on consecutive items (coalesced), each
            // finding its piece by binary search over the offsets
            // (kGatherBatch searches in lockstep), kGatherBatch slot loads
            // in flight per thread.
            __syncthreads();
            const int npi = int(np);
            for (uint32_t i0 = 0; i0 < C; i0 += kGatherBatch * kTsThreads) {
                CandSlot it[kGatherBatch];
                uint32_t is[kGatherBatch];
                int js[kGatherBatch];
#pragma unroll
                for (int b = 0; b < kGatherBatch; ++b)
                    is[b] = i0 + uint32_t(b) * kTsThreads + uint32_t(tid);
                piece_of(pre, npi, is, js);  // the last piece j with pre[j] <= i
                bool got[kGatherBatch];
#pragma unroll
                for (int b = 0; b < kGatherBatch; ++b) {
                    const uint32_t off = is[b] - pre[js[b]];
                    got[b] = is[b] < C && off < pcap;
                    if (got[b]) it[b] = src0[int64_t(js[b]) * pcap + off];
                    if (is[b] < C && !got[b]) gbad = true;
                }
#pragma unroll
                for (int b = 0; b < kGatherBatch; ++b) {
                    const uint32_t i = is[b];
                    if (!got[b]) continue;
                    if (list) {
                        olist_i[d0 + i] = it[b].idx;
                        olist_v[d0 + i] = it[b].v;
                        olist_u[d0 + i] = it[b].u;
                    } else if (int64_t(it[b].idx) < nt) {
                        v[o + it[b].idx] = it[b].v;
                        u[o + it[b].idx] = it[b].u;
                    }
                }
            }
        }
    }
    if (__syncthreads_or(gbad)) {  // uniform: counts that do not add up
        if (tid == 0) latch_error(sc, kErrInternal);
        return;
    }
    // Phases 3 and 4 are compiled twice, for the list in LDS and for items
    // in memory, so that every read goes to its own memory (a pointer that
    // could be either becomes a generic load waited for one at a time).
    auto finish = [&](auto lds_tag) {
        constexpr bool kLds = decltype(lds_tag)::value;
        // 3. T and r
        const float* srcv = list ? olist_v + L.obase[t] : v + o;
        auto val_at = [&](int64_t i) -> float {
            if constexpr (kLds) return sv[i]; else return srcv[i];
        };
        auto key_at = [&](int64_t i) -> uint32_t { return floor_key(mag_key(val_at(i)), fl); };
        // On the list, every key is at least the window's lower edge lo: the top
        // 21 bits of T come from one histogram of (key >> 10) - (lo >> 10) when
        // they lie within 2046 bins of lo's, else from the first two digits.
        uint32_t prefix = 0, krem = 0;
        if (!all) {  // uniform
            krem = uint32_t(k);
            bool ok;
            if (kLds && len <= kFinDirect) {  // uniform: a short list
                ok = fin_direct(key_at, len, prefix, krem, pick);
            } else {
                ok = list && lo_key != kNoKey &&
                     fin_prefix21(key_at, len, lo_key >> 10, prefix, krem, h, rows, pick);
                int low = -1;  // the last 10 bits: by counting within the prefix's bin
                if (ok) {  // uniform; pre is free after the gather
                    low = fin_low10(key_at, len, prefix, krem, pre, &lcnt, pick + 8);
                    ok = low != 0;
                } else {
                    prefix = 0;
                    krem = uint32_t(k);
                    ok = fin_digit<0>(key_at, len, prefix, krem, h, rows + kTsWaves, pick + 2);
                    ok = ok && fin_digit<1>(key_at, len, prefix, krem, h, rows + 2 * kTsWaves,
                                            pick + 4);
                }
                if (low < 0)  // uniform
                    ok = ok && fin_digit<2>(key_at, len, prefix, krem, h, rows + 3 * kTsWaves,
                                            pick + 6);
            }
            if (!ok) {  // uniform
                if (tid == 0) latch_error(sc, kErrInternal);
                return;
            }
            krem = last_rank<2>(prefix, krem, fl);
        }
        if (tid == 0) {
            ts[t].prefix = prefix;
            ts[t].krem = krem;
        }
        // 4. emit in index order: wave w owns items [c0, c1), a run of whole
        // 64-item rounds; a count pass gives every wave its output offsets
        const uint32_t T = prefix, r = krem;
        const bool dense = !list;
        const int lane = lane_id(), w = tid >> 6;
        const int64_t rounds = (len + kWave - 1) / kWave;
        const int64_t rpw = (rounds + kTsWaves - 1) / kTsWaves;
        const int64_t c0 = min(len, int64_t(w) * rpw * kWave);
        const int64_t c1 = min(len, int64_t(w + 1) * rpw * kWave);
        constexpr int64_t kStep = int64_t(kWave) * kFinEmitUnroll;
        uint32_t ng = 0, ne = 0;
        for (int64_t b0 = c0; b0 < c1; b0 += kStep) {
            uint32_t kk[kFinEmitUnroll];
    #pragma unroll
            for (int q = 0; q < kFinEmitUnroll; ++q) {
                const int64_t i = b0 + int64_t(q) * kWave + lane;
                kk[q] = i < c1 ? key_at(i) : kNoKey;
            }
    #pragma unroll
            for (int q = 0; q < kFinEmitUnroll; ++q) {
                ng += uint32_t(__popcll(__ballot(kk[q] != kNoKey && kk[q] > T)));
                ne += uint32_t(__popcll(__ballot(kk[q] == T)));
            }
        }
        if (lane == 0) {
            wcnt[w] = ng;
            wcnt[kTsWaves + w] = ne;
        }
        __syncthreads();
        uint32_t gb = 0, eb = 0;
        for (int j = 0; j < w; ++j) {
            gb += wcnt[j];
            eb += wcnt[kTsWaves + j];
        }
        if (out_count && tid == 0) out_count[t] = sent_count(wcnt, r);
        float* vt_ = v + o;
        const uint32_t* oli = olist_i + L.obase[t];
        const float* olu = olist_u + L.obase[t];
        uint32_t* oi = out_idx + K.koff[t];
        float* ov = out_val + K.koff[t];
        const uint64_t lt = lanemask_lt();
        bool bad = false;
        for (int64_t b0 = c0; b0 < c1; b0 += kStep) {
            float val[kFinEmitUnroll], usv[kFinEmitUnroll];
            uint32_t lidx[kFinEmitUnroll];
            bool in[kFinEmitUnroll];
    #pragma unroll
            for (int q = 0; q < kFinEmitUnroll; ++q) {
                const int64_t i = b0 + int64_t(q) * kWave + lane;
                in[q] = i < c1;
                val[q] = in[q] ? val_at(i) : 0.0f;
                lidx[q] = uint32_t(i);
                usv[q] = 0.0f;
                if (!dense && in[q]) {  // the list's index and saved u
                    if constexpr (kLds) {
                        lidx[q] = sidx[i];
                        usv[q] = __uint_as_float(su[i]);
                    } else {
                        lidx[q] = oli[i];
                        usv[q] = olu[i];
                    }
                }
            }
    #pragma unroll
            for (int q = 0; q < kFinEmitUnroll; ++q) {
                const uint32_t key = floor_key(mag_key(val[q]), fl);
                const bool gt = in[q] && key > T, eq = in[q] && key == T;
                const uint64_t bg = __ballot(gt), be = __ballot(eq);
                const uint32_t g1 = gb + uint32_t(__popcll(bg & lt));
                const uint32_t e1 = eb + uint32_t(__popcll(be & lt));
                bool send = false;
                uint32_t slot = 0;
                if (gt) { send = true; slot = g1 + min(e1, r); }
                else if (eq && e1 < r) { send = true; slot = g1 + e1; }
                if (send) {
                    // never write outside the outputs, whatever the counts say
                    if (int64_t(slot) >= k || int64_t(lidx[q]) >= nt) {
                        bad = true;
                    } else {
                        oi[slot] = lidx[q];
                        ov[slot] = val[q];
                        if (dense) {
                            u[o + lidx[q]] = 0.0f;
                            vt_[lidx[q]] = 0.0f;
                        }
                    }
                } else if (in[q] && !dense) {
                    if (int64_t(lidx[q]) >= nt) {
                        bad = true;
                    } else {
                        u[o + lidx[q]] = usv[q];
                        vt_[lidx[q]] = val[q];
                    }
                }
                gb += uint32_t(__popcll(bg));
                eb += uint32_t(__popcll(be));
            }
        }
        if (bad) latch_error(sc, kErrInternal);
    };
    if (in_lds) finish(BoolTag<true>{});  // uniform
    else finish(BoolTag<false>{});
}

}  // namespace dgc
