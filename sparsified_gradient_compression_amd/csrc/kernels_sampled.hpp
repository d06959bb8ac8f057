// kernels_sampled.hpp -- the sampled threshold of the approximate selector.
//
// Source: the DGC review page (nubint.ai), "Research questions" (RQ4:
// hierarchical thresholding as a runtime strategy for scalable selection)
// and "Proposed method" (only large entries are sent).  The page gives no
// algorithm; the rule here: per tensor t, a sample of whole 32-element
// lines -- every line when n_t <= 65536, else ls = min(lines, max(512,
// lines / 256)) lines, line j at j*stride + fmix32(j*0x9E3779B9 ^
// t*0x7F4A7C15) mod stride (the line placement of the exact path's window)
// -- gives S keys of v after this step's update; the threshold theta_t is
// the J-th largest of them, J = ceil(S * k_t / n_t), found exactly by three
// histogram levels over the sample (11, 10 and 10 bits of the key).  The
// element-wise pass then sends every non-zero entry with key >= theta_t
// (kernels_binlocal.hpp, threshold mode).
#pragma once

#include "dgc_device.hpp"
#include "kernels_compress.hpp"

namespace dgc {

constexpr uint32_t kModeSampled = 3;  // TensorState::mode of this selector

// Sample layout: lines sampled per tensor and blocks of kLinesPerSampleBlock
// of them (device pointers into the workspace).
struct DevSample {
    const int64_t* slines;  // [T] sampled lines (every line for small tensors)
    const int64_t* sbase;   // [T+1] first sample block of each tensor
    const uint32_t* smap;   // [sample blocks] tensor of each block
};

// Level 0: histogram of key >> 20; level 1: of (key >> 10) & 1023 among keys
// whose top 11 bits are the level-0 bin; level 2: of key & 1023 among keys
// whose top 21 bits are the level-1 prefix.  The keys are those of v after
// this step's update, computed from g, u, v at the sampled lines.
template <int LEVEL>
__global__ __launch_bounds__(kBlock) void k_sm_hist(
    const float* __restrict__ g, const float* __restrict__ u,
    const float* __restrict__ v, DevLayout L, DevSample A,
    const Scalars* __restrict__ sc, int clip_on, const TensorState* __restrict__ ts,
    float m, uint32_t* __restrict__ shist) {
    constexpr int bins = LEVEL == 0 ? kBins0 : 1024;
    __shared__ uint32_t h[bins];
    for (int b = threadIdx.x; b < bins; b += kBlock) h[b] = 0;
    __syncthreads();
    const int64_t sb = blockIdx.x;
    const int t = int(A.smap[sb]);
    const uint32_t sel = LEVEL == 0 ? 0u : LEVEL == 1 ? ts[t].wbin : ts[t].wabove;
    if (LEVEL > 0 && ts[t].wbin == kNoKey) return;  // uniform: no threshold needed
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    const int64_t lines = (nt + kLine - 1) / kLine;
    const int64_t ls = A.slines[t];
    const int64_t stride = lines / ls;
    const int64_t j0 = (sb - A.sbase[t]) * kLinesPerSampleBlock;
    const int64_t j1 = min(ls, j0 + kLinesPerSampleBlock);
    const float s = clip_on ? sc->scale : 1.0f;
    uint32_t key[kLinesPerGroup][4];
    bool ok[kLinesPerGroup][4];
    sample_line_keys(g, u, v, o, nt, t, stride, j0, j1, s, m, key, ok);
#pragma unroll
    for (int q = 0; q < kLinesPerGroup; ++q)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            if (!ok[q][c4]) continue;
            const uint32_t kk = key[q][c4];
            if (LEVEL == 0) atomicAdd(&h[kk >> 20], 1u);
            else if (LEVEL == 1 && (kk >> 20) == sel) atomicAdd(&h[(kk >> 10) & 1023u], 1u);
            else if (LEVEL == 2 && (kk >> 10) == sel) atomicAdd(&h[kk & 1023u], 1u);
        }
    __syncthreads();
    uint32_t* row = shist + int64_t(t) * kHistBins;
    for (int b = threadIdx.x; b < bins; b += kBlock)
        if (h[b]) atomicAdd(&row[b], h[b]);
}

// One block per tensor: find the bin holding the rank still sought, from
// the top, and narrow the search; the last level yields theta.  Level 0
// sets the rank J = ceil(S * k / n) from the sample size S (every sampled
// key lands in the level-0 histogram).  Clears the histogram row.
//   ts.wbin   level-0 bin (kNoKey: nothing to send, k = 0 or no sample)
//   ts.wabove level-1 prefix (top 21 bits)
//   ts.wj     rank still sought inside the current bin
//   ts.lo_key = ts.prefix = theta; ts.total = S; ts.krem = J
// For the hierarchical selector (hier 1) the last level sets instead
//   ts.floor = ts.lo_key = max(theta, 1)
// so that the element-wise pass takes the first level's survivors (non-zero,
// key >= theta) as candidates; with hier 2 (no candidates wanted: the
// forced whole-tensor path) lo_key stays kNoKey.  Until then floor is
// kNoKey (nothing survives), or 0 for the sampled selector (hier 0).
template <int LEVEL>
__global__ __launch_bounds__(kBlock) void k_sm_pick(
    DevLayout L, const int64_t* __restrict__ ktgt, uint32_t* __restrict__ shist,
    TensorState* __restrict__ ts, int hier) {
    constexpr int bins = LEVEL == 0 ? kBins0 : 1024;
    constexpr int per = bins / kBlock;
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t nt = L.o[t + 1] - L.o[t];
    uint32_t* row = shist + int64_t(t) * kHistBins;
    const uint32_t wbin = ts[t].wbin, wabove = ts[t].wabove, want = ts[t].wj;
    if (LEVEL > 0 && wbin == kNoKey) return;  // uniform
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        c[q] = row[bins - 1 - (threadIdx.x * per + q)];
        mine += c[q];
    }
    uint32_t total;
    const uint32_t above = block_exclusive_scan(mine, lds, total);  // has barriers
#pragma unroll
    for (int q = 0; q < per; ++q) row[bins - 1 - (threadIdx.x * per + q)] = 0;
    uint32_t rank;
    if (LEVEL == 0) {
        if (threadIdx.x == 0) {
            ts[t].mode = kModeSampled;
            ts[t].lo_key = kNoKey;
            ts[t].prefix = kNoKey;
            ts[t].wbin = kNoKey;
            ts[t].total = total;
            ts[t].krem = 0;
            ts[t].overflow = 0;
            ts[t].floor = hier ? kNoKey : 0u;
        }
        __syncthreads();
        const int64_t k = ktgt[t];
        if (k <= 0 || total == 0) return;
        const int64_t J = (int64_t(total) * k + nt - 1) / nt;
        rank = uint32_t(J);
        if (threadIdx.x == 0) ts[t].krem = rank;
    } else {
        rank = want;
    }
    uint32_t run = above;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (run < rank && rank <= run + c[q]) {
            const uint32_t b = uint32_t(bins - 1 - (threadIdx.x * per + q));
            if (LEVEL == 0) {
                ts[t].wbin = b;
            } else if (LEVEL == 1) {
                ts[t].wabove = (wbin << 10) | b;
            } else {
                const uint32_t theta = (wabove << 10) | b;
                if (hier) {
                    const uint32_t fl = theta > 0u ? theta : 1u;
                    ts[t].floor = fl;
                    ts[t].lo_key = hier == 1 ? fl : kNoKey;
                } else {
                    ts[t].lo_key = theta;
                }
                ts[t].prefix = theta;
            }
            ts[t].wj = rank - run;
        }
        run += c[q];
    }
}

}  // namespace dgc
