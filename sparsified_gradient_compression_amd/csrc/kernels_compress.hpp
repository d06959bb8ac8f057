// kernels_compress.hpp -- the compression step on gfx950.
//
// Method: DGC review page (nubint.ai), "Proposed method": local gradient
// clipping, momentum correction with local accumulation, sending only the
// largest |v| entries, momentum factor masking.  Selection is exact top-k
// per tensor with ties to the lower index.
//
// Pass structure for one step (all on the caller's stream, no host sync):
//   norm_partial/norm_final  binary64 sum of g^2 (only with clipping)
//                            (kernel boundaries order the passes: a
//                            device-scope fence per workgroup costs more on
//                            this chip than the extra launches)
//   sample/window            per tensor, keys of the would-be v on sampled
//                            32-element lines -> a candidate threshold lo
//   fused                    u, v update (20 B/elem); keys >= lo are
//                            written, index-ordered, into the fixed 12-byte
//                            slots {index, v, u} of their 1024-element piece
//                            (no atomics) and stored as u = v = +0 when the
//                            piece's run fits
//   group_sum/scan, gather   per tensor: choose the source (candidates when
//                            none overflowed and there are at least k, else
//                            the whole tensor); concatenate the pieces' runs
//                            into one index-ordered candidate list, or put
//                            the masked candidates back for the whole tensor
//   then either, spread over the chip:
//     hist<D>/resolve<D>     three radix digits (11,10,10 bits) -> the k-th
//                            largest key T and the tie quota r
//     emit_count/scan/write  index-ordered output of {key > T} plus the
//                            first r ties; the list's other candidates get
//                            their u, v back (whole tensor: u = v = +0 at
//                            the sent entries)
//   or, for short sources, the same in one workgroup per tensor:
//     select_tensor
#pragma once

#include "dgc_device.hpp"
#include "kernel_fused.hpp"

namespace dgc {

// ---------------------------------------------------------------- prep

// Zero `n` 32-bit words (a fill kernel: safe inside captured graphs).
__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* __restrict__ p,
                                                     int64_t n, uint32_t val) {
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * kBlock)
        p[i] = val;
}

// The per-call k tables of a layout of at most kKArgTensors tensors, from k
// passed by value: block t writes k[t], koff[t] = k[0] + ... + k[t-1],
// ktbase[t] (tiles of kTile entries before tensor t) and tensor t's entries
// of the tile map; the last block also writes the totals at index T.
constexpr int kKArgTensors = 480;
struct KArgs {
    int32_t T;
    int64_t k[kKArgTensors];
};
__global__ __launch_bounds__(kBlock) void k_ktables(KArgs a, int64_t* __restrict__ kk,
                                                    int64_t* __restrict__ koff,
                                                    int64_t* __restrict__ ktbase,
                                                    uint32_t* __restrict__ kmap) {
    const int t = blockIdx.x;
    int64_t off = 0, tb = 0;
    for (int i = 0; i < t; ++i) {  // a few hundred scalar adds at most
        off += a.k[i];
        tb += (a.k[i] + kTile - 1) / kTile;
    }
    const int64_t tiles = (a.k[t] + kTile - 1) / kTile;
    if (threadIdx.x == 0) {
        kk[t] = a.k[t];
        koff[t] = off;
        ktbase[t] = tb;
        if (t == a.T - 1) {
            koff[a.T] = off + a.k[t];
            ktbase[a.T] = tb + tiles;
        }
    }
    for (int64_t i = threadIdx.x; i < tiles; i += kBlock) kmap[tb + i] = uint32_t(t);
}

// Scalar outputs when nothing else writes them (an empty layout with
// clipping off).
__global__ void k_set_scalars(Scalars* __restrict__ sc, double* __restrict__ out_norm,
                              float* __restrict__ out_scale) {
    if (threadIdx.x == 0) {
        sc->norm = -1.0;
        sc->scale = 1.0f;
        if (out_norm) *out_norm = -1.0;
        if (out_scale) *out_scale = 1.0f;
    }
}

// ---------------------------------------------------------------- norm

// Block b sums g^2 over [b*chunk, min(n, (b+1)*chunk)) in binary64
// (chunk a multiple of 4): thread-strided float4 loads, one accumulator per float4 lane
// slot, then a fixed-order block reduction.  The squares of binary32 values
// are exact in binary64, so only the additions round.
__global__ __launch_bounds__(kBlock) void k_norm_partial(
    const float* __restrict__ g, int64_t n, int64_t chunk, double* __restrict__ partial) {
    __shared__ double lds[kWavesPerBlock];
    const int64_t lo = int64_t(blockIdx.x) * chunk;
    const int64_t hi = min(n, lo + chunk);
    const int64_t vlo = lo >> 2, vhi = hi >> 2;  // whole float4 units
    const float4* g4 = reinterpret_cast<const float4*>(g);
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int64_t i = vlo + threadIdx.x;
    for (; i + 3 * kBlock < vhi; i += 4 * kBlock) {
        float4 x0 = ld_stream(g + 4 * i), x1 = ld_stream(g + 4 * (i + kBlock)),
               x2 = ld_stream(g + 4 * (i + 2 * kBlock)),
               x3 = ld_stream(g + 4 * (i + 3 * kBlock));
        a0 += double(x0.x) * double(x0.x); a1 += double(x0.y) * double(x0.y);
        a2 += double(x0.z) * double(x0.z); a3 += double(x0.w) * double(x0.w);
        a0 += double(x1.x) * double(x1.x); a1 += double(x1.y) * double(x1.y);
        a2 += double(x1.z) * double(x1.z); a3 += double(x1.w) * double(x1.w);
        a0 += double(x2.x) * double(x2.x); a1 += double(x2.y) * double(x2.y);
        a2 += double(x2.z) * double(x2.z); a3 += double(x2.w) * double(x2.w);
        a0 += double(x3.x) * double(x3.x); a1 += double(x3.y) * double(x3.y);
        a2 += double(x3.z) * double(x3.z); a3 += double(x3.w) * double(x3.w);
    }
    for (; i < vhi; i += kBlock) {
        float4 x = g4[i];
        a0 += double(x.x) * double(x.x); a1 += double(x.y) * double(x.y);
        a2 += double(x.z) * double(x.z); a3 += double(x.w) * double(x.w);
    }
    // tail elements beyond the last whole float4 (only the last block)
    for (int64_t e = (vhi << 2) + threadIdx.x; e < hi; e += kBlock)
        a0 += double(g[e]) * double(g[e]);
    double s = block_sum_fixed((a0 + a1) + (a2 + a3), lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// One block: S = fixed-order sum of the partials; norm = sqrt(S);
// s = (float)(clip / norm) if norm > clip else 1 (all in binary64, one
// rounding to binary32 at the end).
__global__ __launch_bounds__(kBlock) void k_norm_final(
    const double* __restrict__ partial, int64_t nb, double clip,
    Scalars* __restrict__ sc, double* __restrict__ out_norm,
    float* __restrict__ out_scale) {
    __shared__ double lds[kWavesPerBlock];
    double a = 0.0;
    for (int64_t i = threadIdx.x; i < nb; i += kBlock) a += partial[i];
    double S = block_sum_fixed(a, lds);
    if (threadIdx.x == 0) {
        double norm = sqrt(S);
        float s = 1.0f;
        if (clip > 0.0 && norm > clip) s = float(clip / norm);
        sc->norm = norm;
        sc->scale = s;
        if (out_norm) *out_norm = norm;
        if (out_scale) *out_scale = s;
    }
}

// ---------------------------------------------------------------- sample

// Keys of the would-be v on sampled lines.  Block b belongs to one tensor
// (smap); it visits kLinesPerSampleBlock of the tensor's sampled lines, one
// 8-lane group per line (16 bytes of each of g, u, v per lane).  Sampled line j lies at a hashed offset inside
// the j-th of slines equal strides, so sampling does not alias with the
// tensor's row structure.  Level 0 histograms the top 11 key bits; level 1
// revisits the same lines and histograms the next 10 bits of the keys whose
// top 11 bits equal the bin chosen by level 0.
// A block's sampled lines are shared out to its 8-lane groups: group grp
// takes lines j0 + grp + kSampleGroups q (q < kLinesPerGroup) of [j0, j1);
// sampled line j of a tensor with `stride` lines per sampled line lies at
// j * stride + mix32(j * 0x9E3779B9 ^ t * 0x7F4A7C15) mod stride.  The keys
// of the would-be v there: every load is issued before the first update,
// so a group waits for memory once, not once per line.  ok[q][c] is false
// past j1 or past the tensor's end.
constexpr int kLineLanes = int(kLine / 4);  // 16 bytes per lane and array
constexpr int kSampleGroups = kBlock / kLineLanes;
constexpr int kLinesPerGroup = int(kLinesPerSampleBlock / kSampleGroups);
__device__ __forceinline__ void sample_line_keys(
    const float* __restrict__ g, const float* __restrict__ u, const float* __restrict__ v,
    int64_t o, int64_t nt, int t, int64_t stride, int64_t j0, int64_t j1, float s, float m,
    uint32_t (&key)[kLinesPerGroup][4], bool (&ok)[kLinesPerGroup][4]) {
    const int grp = int(threadIdx.x) / kLineLanes, gl = int(threadIdx.x) % kLineLanes;
    float gg[kLinesPerGroup][4], uu[kLinesPerGroup][4], vv[kLinesPerGroup][4];
#pragma unroll
    for (int q = 0; q < kLinesPerGroup; ++q) {
        const int64_t j = j0 + grp + int64_t(q) * kSampleGroups;
        const uint32_t r = mix32(uint32_t(j) * 0x9E3779B9u ^ uint32_t(t) * 0x7F4A7C15u);
        const int64_t e = (j * stride + int64_t(r % uint64_t(stride))) * kLine + 4 * gl;
        const bool line = j < j1;
        const float *pg = g + o + e, *pu = u + o + e, *pv = v + o + e;
        if (line && e + 4 <= nt &&
            ((reinterpret_cast<uintptr_t>(pg) | reinterpret_cast<uintptr_t>(pu) |
              reinterpret_cast<uintptr_t>(pv)) & 15) == 0) {
            const float4 a = *reinterpret_cast<const float4*>(pg);
            const float4 b = *reinterpret_cast<const float4*>(pu);
            const float4 c = *reinterpret_cast<const float4*>(pv);
            gg[q][0] = a.x; gg[q][1] = a.y; gg[q][2] = a.z; gg[q][3] = a.w;
            uu[q][0] = b.x; uu[q][1] = b.y; uu[q][2] = b.z; uu[q][3] = b.w;
            vv[q][0] = c.x; vv[q][1] = c.y; vv[q][2] = c.z; vv[q][3] = c.w;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) ok[q][c4] = true;
        } else {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                ok[q][c4] = line && e + c4 < nt;
                gg[q][c4] = ok[q][c4] ? pg[c4] : 0.0f;
                uu[q][c4] = ok[q][c4] ? pu[c4] : 0.0f;
                vv[q][c4] = ok[q][c4] ? pv[c4] : 0.0f;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kLinesPerGroup; ++q)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            momentum_update(gg[q][c4], s, m, uu[q][c4], vv[q][c4]);
            key[q][c4] = mag_key(vv[q][c4]);
        }
}

template <int LEVEL>
__global__ __launch_bounds__(kBlock) void k_sample(
    const float* __restrict__ g, const float* __restrict__ u,
    const float* __restrict__ v, DevLayout L, const Scalars* __restrict__ sc,
    int clip_on, const TensorState* __restrict__ ts, float m,
    uint32_t* __restrict__ shist) {
    __shared__ uint32_t h[kBins0];
    for (int b = threadIdx.x; b < kBins0; b += kBlock) h[b] = 0;
    __syncthreads();
    const int64_t sb = blockIdx.x;
    const int t = int(L.smap[sb]);
    const uint32_t wbin = LEVEL == 1 ? ts[t].wbin : 0u;
    if (LEVEL == 1 && wbin == kNoKey) return;  // uniform: window already set
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    const int64_t lines = (nt + kLine - 1) / kLine;
    const int64_t ls = L.slines[t];
    const int64_t stride = lines / ls;
    const int64_t j0 = (sb - L.sbase[t]) * kLinesPerSampleBlock;
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
            else if ((kk >> 20) == wbin) atomicAdd(&h[(kk >> 10) & 1023u], 1u);
        }
    __syncthreads();
    uint32_t* row = shist + int64_t(t) * kHistBins;
    for (int b = threadIdx.x; b < kBins0; b += kBlock)
        if (h[b]) atomicAdd(&row[b], h[b]);
}

// One block per tensor: place the candidate threshold lo just below the
// j-th largest sampled key, j = ceil(mu + 4 sqrt(mu) + 6) where mu = S*k/n
// is how many of the S samples the true top k should hold.  Level 0 finds
// the top-11-bit bin holding the j-th key (wbin) and how many samples lie
// above it (wabove); level 1 finds the 10-bit sub-bin inside it, and lo is
// that sub-bin's lower edge.  Small tensors (no sampled lines) and k = 0
// get no candidates.  Clears the histogram row for the next use.
template <int LEVEL>
__global__ __launch_bounds__(kBlock) void k_window(
    DevLayout L, DevK K, uint32_t* __restrict__ shist,
    TensorState* __restrict__ ts, int force_dense) {
    constexpr int bins = LEVEL == 0 ? kBins0 : 1024;
    constexpr int per = bins / kBlock;
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t nt = L.o[t + 1] - L.o[t];
    const int64_t k = K.k[t];
    uint32_t* row = shist + int64_t(t) * kHistBins;
    if (LEVEL == 1 && ts[t].wbin == kNoKey) return;  // decided at level 0
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        c[q] = row[bins - 1 - (threadIdx.x * per + q)];
        mine += c[q];
    }
    uint32_t total;
    uint32_t above = block_exclusive_scan(mine, lds, total);
#pragma unroll
    for (int q = 0; q < per; ++q) row[bins - 1 - (threadIdx.x * per + q)] = 0;
    if (LEVEL == 0) {
        // Defaults first (no candidates, no second level), then at most one
        // thread overwrites them.  No candidates sends a tensor with k > 0
        // to the dense path: small tensors, the forced dense path, or a
        // window that found no bin.
        if (threadIdx.x == 0) {
            ts[t].lo_key = kNoKey;
            ts[t].wbin = kNoKey;
            ts[t].floor = 0;  // exact top-k
        }
        __syncthreads();
        if (k <= 0 || force_dense || L.slines[t] == 0) return;
        const double mu = double(total) * double(k) / double(nt);
        const double jd = ceil(mu + 4.0 * sqrt(mu) + 6.0);
        if (jd > double(total)) {  // (nearly) everything: take all elements
            if (threadIdx.x == 0) ts[t].lo_key = 0;
            return;
        }
        const uint32_t j = uint32_t(jd);
        uint32_t run = above;
#pragma unroll
        for (int q = 0; q < per; ++q) {
            if (run < j && j <= run + c[q]) {
                ts[t].wbin = uint32_t(kBins0 - 1 - (threadIdx.x * per + q));
                ts[t].wabove = run;
                ts[t].wj = j;
            }
            run += c[q];
        }
    } else {
        __syncthreads();  // every thread has read wbin before it may change
        const uint32_t jr = ts[t].wj - ts[t].wabove;  // rank inside wbin
        const uint32_t wbin = ts[t].wbin;
        uint32_t run = above;
#pragma unroll
        for (int q = 0; q < per; ++q) {
            if (run < jr && jr <= run + c[q]) {
                uint32_t b2 = uint32_t(bins - 1 - (threadIdx.x * per + q));
                ts[t].lo_key = (wbin << 20) | (b2 << 10);
            }
            run += c[q];
        }
    }
}

// ---------------------------------------------------------------- source

// Piece groups: group g of tensor t holds pieces pbase[t] + 256 (g - gbase[t])
// onward (at most 256, never past the tensor).

// One block per group: the group's candidate count, with bit 31 set when a
// piece overflowed its slots.
__global__ __launch_bounds__(kBlock) void k_group_sum(
    DevLayout L, const uint32_t* __restrict__ run_cnt, uint32_t* __restrict__ gsum) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const int64_t g = blockIdx.x;
    const int t = int(L.gmap[g]);
    const int64_t p0 = L.pbase[t] + (g - L.gbase[t]) * kGroup;
    const int64_t p1 = min(p0 + kGroup, L.pbase[t + 1]);
    const int64_t p = p0 + int64_t(threadIdx.x);
    const uint32_t c = (p >= p0 && p < p1) ? run_cnt[p] : 0u;
    const int over = __syncthreads_or(c > uint32_t(L.pcap[t]));
    uint32_t tot;
    block_exclusive_scan(c, lds, tot);
    if (threadIdx.x == 0) gsum[g] = tot | (over ? 0x80000000u : 0u);
}

// The selection source of a tensor with C candidates (over: a piece ran
// out of slots; cap: the list's capacity).  Exact top-k (floor 0): the
// list when it is whole and holds k to cap items, else the whole tensor.
// Hierarchical selector (floor > 0): the candidates are the first level's
// survivors when the window edge is the floor; a whole list of at most k
// of them is sent as it is (send_all), a longer one is selected from, and
// otherwise the whole tensor is selected from under floor_key.
__device__ __forceinline__ uint32_t select_mode(int64_t k, uint32_t C, int over, uint64_t cap,
                                                uint32_t lo_key, uint32_t floor) {
    if (k <= 0) return kModeSkip;
    if (over || uint64_t(C) > cap) return kModeDense;
    if (floor != 0 && lo_key == floor) return kModeList;
    return int64_t(C) < k ? kModeDense : kModeList;
}

__device__ __forceinline__ bool send_all(int64_t k, uint32_t C, uint32_t floor) {
    return floor != 0 && int64_t(C) <= k;
}

// One block per tensor: scan its groups' counts (their offsets in the
// ordered list), then choose the selection source: the candidate list when
// no piece overflowed and there are at least k candidates, else the whole
// tensor.  Also counts the source's kTile-item tiles for the active-tile map.
__global__ __launch_bounds__(kBlock) void k_group_scan(
    DevLayout L, DevK K, TensorState* __restrict__ ts,
    const uint32_t* __restrict__ gsum, uint32_t* __restrict__ goff,
    uint32_t* __restrict__ atiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t nt = L.o[t + 1] - L.o[t];
    const int64_t k = K.k[t];
    uint32_t carry = 0;
    int over = 0;
    if (k > 0) {  // uniform
        // at most 16384 groups (n < 2^32): direct rounds, no LDS stage
        const int64_t g0 = L.gbase[t], ng = L.gbase[t + 1] - g0;
        for (int64_t base = 0; base < ng; base += kScanRound) {
            uint32_t x[kScanPer];
            scan_load_round<false>(gsum + g0, base, ng, nullptr, x);
            uint32_t local = 0;
#pragma unroll
            for (int q = 0; q < kScanPer; ++q) {
                over |= (x[q] >> 31) != 0;
                x[q] &= 0x7FFFFFFFu;
                local += x[q];
            }
            uint32_t tot;
            uint32_t run = carry + block_exclusive_scan(local, lds, tot);
            uint32_t r[kScanPer];
#pragma unroll
            for (int q = 0; q < kScanPer; ++q) {
                r[q] = run;
                run += x[q];
            }
            scan_store_round<false>(goff + g0, base, ng, nullptr, r);
            carry += tot;
        }
    }
    over = __syncthreads_or(over);
    const uint64_t cap = uint64_t(L.obase[t + 1] - L.obase[t]);
    const uint32_t mode = select_mode(k, carry, over, cap, ts[t].lo_key, ts[t].floor);
    // the hierarchical selector's complete survivor list of at most k: all
    // of it is sent (T = 0, r = 0, no digit pass)
    const bool all = mode == kModeList && send_all(k, carry, ts[t].floor);
    const int64_t len = mode == kModeList ? int64_t(carry) : nt;
    if (threadIdx.x == 0) {
        ts[t].total = carry;
        ts[t].overflow = uint32_t(over);
        ts[t].mode = mode;
        ts[t].len = uint32_t(len);
        ts[t].prefix = 0;
        ts[t].krem = all ? 0u : uint32_t(k > 0 ? k : 0);
        ts[t].done21 = all ? kDoneAll : 0u;
        atiles[t] = mode == kModeSkip ? 0u : uint32_t((len + kTile - 1) >> kTileShift);
    }
}

// Histogram increment with wave aggregation: twice, the bin of the lowest
// pending lane takes every lane of the wave that shares it with one LDS
// atomic (ballot + popcount); the lanes left add one each.  Keys that crowd
// into a few bins (the top digit of a candidate list) then cost a few
// atomics per wave instead of 64 on one address.  Every lane of the wave
// must call it.
__device__ __forceinline__ void hist_inc(uint32_t* h, uint32_t bin, bool valid) {
    uint64_t todo = __ballot(valid);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (!todo) break;  // uniform
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const uint32_t b = __shfl(bin, leader, kWave);
        const uint64_t same = __ballot(valid && bin == b) & todo;
        if (lane_id() == leader) atomicAdd(&h[b], uint32_t(__popcll(same)));
        todo &= ~same;
    }
    if ((todo >> lane_id()) & 1u) atomicAdd(&h[bin], 1u);
}

// For each of B items q[b]: the last j in [0, n) with pre[j] <= q[b] (pre
// non-decreasing, pre[0] = 0), i.e. the piece that holds item q[b] when
// pre[j] is the number of items before piece j.  Branchless halving of the
// range [j, j + len), the same steps for every item, so the B searches go
// in lockstep with their LDS reads in flight together (a search per item in
// turn waits on one read at a time).  Every read is in [0, n).
template <int B>
__device__ __forceinline__ void piece_of(const uint32_t* pre, int n, const uint32_t (&q)[B],
                                         int (&j)[B]) {
#pragma unroll
    for (int b = 0; b < B; ++b) j[b] = 0;
    for (int len = n; len > 1;) {  // uniform
        const int half = len >> 1;
#pragma unroll
        for (int b = 0; b < B; ++b) j[b] = pre[j[b] + half] <= q[b] ? j[b] + half : j[b];
        len -= half;
    }
}

// One block per group.  The fused pass masked the candidates of every piece
// whose run fit its slots (u = v = +0 there; each slot holds the index, v
// and u).  For a tensor on the list path, concatenate the group's piece
// runs, with their saved u, into the tensor's index-ordered candidate list
// (three arrays: local index, v, u).
// For any other tensor, put the slotted u and v back, so the dense path
// reads the true values.  Threads walk the group's items, several loads in
// flight each, and find each item's piece by binary search over the
// in-group prefix of the run lengths; accesses are coalesced.  With `hist`
// set (the spread passes follow), the list's keys are also counted by their
// top 21 bits above the window edge into the tensor's histogram row, for
// k_resolve21.
// With `runs` set (the host sets it at high k, where pieces hold long runs)
// a wave copies whole runs instead: the group's pieces are split over
// `split` workgroups (grid = groups x split), each wave takes every fourth
// of its workgroup's pieces and copies the piece's run, 64 items a round,
// kGatherRunUnroll rounds in flight: no search, 32-bit offsets, and the
// list's open top histogram bin (most of a dense list) counted in registers.
// At 25% density the per-item search made the gather issue ~112 vector
// instructions per item, which bounded it, not its bytes.
constexpr int kGatherBatch = 8;      // slot loads in flight per thread
constexpr int kGatherSplit = 4;      // workgroups per group with `runs`
constexpr int kGatherRunUnroll = 4;  // 64-item rounds in flight per wave
constexpr int64_t kGatherRunDensity = 8;  // runs when sum k >= n / 8

__global__ __launch_bounds__(kBlock) void k_gather(
    DevLayout L, const TensorState* __restrict__ ts,
    const CandSlot* __restrict__ slots,
    const uint32_t* __restrict__ run_cnt, const uint32_t* __restrict__ goff,
    uint32_t* __restrict__ olist_i, float* __restrict__ olist_v,
    float* __restrict__ olist_u, float* __restrict__ u, float* __restrict__ v,
    uint32_t* __restrict__ hist, int split, int runs) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t pre[kGroup + 1];
    __shared__ uint32_t h21[kHistBins];
    const int64_t g = blockIdx.x / split;
    const uint32_t part = blockIdx.x % split;
    const int t = int(L.gmap[g]);
    const bool list = ts[t].mode == kModeList;  // uniform
    // the list's top-21-bit histogram, unless nothing is left to select
    const bool hist21 = list && hist && ts[t].done21 == 0;
    const uint32_t lo21 = ts[t].lo_key >> 10;
    for (int b = threadIdx.x; b < kHistBins; b += kBlock) h21[b] = 0;
    const int64_t p0 = L.pbase[t] + (g - L.gbase[t]) * kGroup;
    const int64_t np = min(kGroup, L.pbase[t + 1] - p0);  // signed: >= 1 here
    if (np <= 0) return;  // uniform; cannot happen with a valid group map
    const int tid = int(threadIdx.x);
    const int64_t pcap = L.pcap[t];
    uint32_t c = tid < np ? run_cnt[p0 + tid] : 0u;
    if (c > uint32_t(pcap)) c = 0;  // overflowed: no slots, nothing masked
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(c, lds, tot);
    pre[threadIdx.x] = ex;
    if (threadIdx.x == 0) pre[kGroup] = tot;
    __syncthreads();
    if (tot == 0) return;  // uniform
    const CandSlot* src0 = slots + L.slbase[t] + (p0 - L.pbase[t]) * pcap;
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    // the list path guarantees this; it is checked so that no write can
    // leave the tensor's list whatever the counts say
    if (list && int64_t(goff[g]) + tot > L.obase[t + 1] - L.obase[t]) return;
    const int64_t d0 = list ? L.obase[t] + goff[g] : 0;
    // the group's item `pos`, read from its slot
    auto put = [&](const CandSlot& it, uint32_t pos) {
        if (list) {
            olist_i[d0 + pos] = it.idx;
            olist_v[d0 + pos] = it.v;
            olist_u[d0 + pos] = it.u;
        } else if (int64_t(it.idx) < nt) {
            v[o + it.idx] = it.v;
            u[o + it.idx] = it.u;
        }
    };
    if (runs) {  // uniform
        // this workgroup's pieces [ja, jb); wave w takes ja + w, ja + w + 4, ...
        const int ja = int(np * part / split), jb = int(np * (part + 1) / split);
        const int lane = lane_id();
        uint32_t open = 0;  // items in the open top bin
        for (int j = ja + (tid >> 6); j < jb; j += kWavesPerBlock) {
            const uint32_t pos0 = pre[j], cnt = pre[j + 1] - pos0;
            const CandSlot* sp = src0 + int64_t(j) * pcap;
            for (uint32_t i0 = 0; i0 < cnt; i0 += kWave * kGatherRunUnroll) {
                CandSlot it[kGatherRunUnroll];
#pragma unroll
                for (int r = 0; r < kGatherRunUnroll; ++r) {
                    const uint32_t i = i0 + uint32_t(r * kWave + lane);
                    if (i < cnt) it[r] = sp[i];
                }
#pragma unroll
                for (int r = 0; r < kGatherRunUnroll; ++r) {
                    const uint32_t i = i0 + uint32_t(r * kWave + lane);
                    if (i >= cnt) continue;
                    put(it[r], pos0 + i);
                    if (hist21) {  // uniform
                        const uint32_t d = (mag_key(it[r].v) >> 10) - lo21;
                        if (d < uint32_t(kHistBins - 1)) atomicAdd(&h21[d], 1u);
                        else ++open;
                    }
                }
            }
        }
        if (hist21) {  // uniform: add the workgroup's counts to the tensor's row
            for (int d = kWave / 2; d >= 1; d >>= 1) open += __shfl_xor(open, d, kWave);
            if (lane == 0 && open) atomicAdd(&h21[kHistBins - 1], open);
            __syncthreads();
            uint32_t* row = hist + int64_t(t) * kHistBins;
            for (int b = threadIdx.x; b < kHistBins; b += kBlock)
                if (h21[b]) atomicAdd(&row[b], h21[b]);
        }
        return;
    }
    // This workgroup's share of the group's items: [qa, qb).
    const uint32_t qa = uint32_t(uint64_t(tot) * part / uint32_t(split));
    const uint32_t qb = uint32_t(uint64_t(tot) * (part + 1) / uint32_t(split));
    if (qa >= qb) return;  // uniform
    // Threads take the items q = q0 + u kBlock + tid, kGatherBatch at a
    // time: each finds its piece by binary search over the piece prefixes
    // (largest j < np with pre[j] <= q), the batch's slot loads go out
    // together, then its stores.  Consecutive threads read consecutive
    // slots of one run and write consecutive list entries.
    for (uint32_t q0 = qa; q0 < qb; q0 += kGatherBatch * kBlock) {
        CandSlot it[kGatherBatch];
        uint32_t qs[kGatherBatch];
        int js[kGatherBatch];
#pragma unroll
        for (int b = 0; b < kGatherBatch; ++b) qs[b] = q0 + uint32_t(b) * kBlock + threadIdx.x;
        piece_of(pre, int(np), qs, js);
#pragma unroll
        for (int b = 0; b < kGatherBatch; ++b) {
            if (qs[b] < qb) it[b] = src0[int64_t(js[b]) * pcap + (qs[b] - pre[js[b]])];
        }
#pragma unroll
        for (int b = 0; b < kGatherBatch; ++b) {
            const uint32_t q = q0 + uint32_t(b) * kBlock + threadIdx.x;
            if (q < qb) put(it[b], q);
            // the list's keys by their top 21 bits above the window edge
            // (every candidate is at least lo); bin 2047 takes the rest
            if (hist21) {  // uniform
                const uint32_t d = (mag_key(it[b].v) >> 10) - lo21;
                hist_inc(h21, d < uint32_t(kHistBins - 1) ? d : uint32_t(kHistBins - 1),
                         q < qb);
            }
        }
    }
    if (hist21) {  // uniform: add the group's counts to the tensor's row
        __syncthreads();
        uint32_t* row = hist + int64_t(t) * kHistBins;
        for (int b = threadIdx.x; b < kHistBins; b += kBlock)
            if (h21[b]) atomicAdd(&row[b], h21[b]);
    }
}

// One block per tensor, after k_gather: on the list path, the bin of the
// gather's histogram that holds the krem-th largest key gives the top 21
// bits of T (lo21 + bin) unless it is the open top bin; then prefix and
// krem are set and done21 marks the tensor, so the first two digit passes
// skip it.  Clears the row.
__global__ __launch_bounds__(kBlock) void k_resolve21(TensorState* __restrict__ ts,
                                                      uint32_t* __restrict__ hist) {
    constexpr int per = kHistBins / kBlock;
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t pick[2];
    const int t = blockIdx.x;
    if (ts[t].done21 == kDoneAll) return;  // uniform: sent whole, row untouched
    if (ts[t].mode != kModeList) {  // uniform
        if (threadIdx.x == 0) ts[t].done21 = 0;
        return;
    }
    uint32_t* row = hist + int64_t(t) * kHistBins;
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        c[q] = row[kHistBins - 1 - (threadIdx.x * per + q)];
        mine += c[q];
    }
    if (threadIdx.x == 0) pick[0] = kNoKey;
    uint32_t total;
    uint32_t run = block_exclusive_scan(mine, lds, total);
#pragma unroll
    for (int q = 0; q < per; ++q) row[kHistBins - 1 - (threadIdx.x * per + q)] = 0;
    const uint32_t krem = ts[t].krem;
    const uint32_t lo21 = ts[t].lo_key >> 10;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (run < krem && krem <= run + c[q]) {
            pick[0] = uint32_t(kHistBins - 1 - (threadIdx.x * per + q));
            pick[1] = krem - run;
        }
        run += c[q];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t b = pick[0];
        if (b == kNoKey || b == uint32_t(kHistBins - 1)) {
            ts[t].done21 = 0;
        } else {
            ts[t].prefix = lo21 + b;
            ts[t].krem = pick[1];
            ts[t].done21 = kDone21;
        }
    }
}

// One block: exclusive scan of the active tile counts -> aoff[T+1].
__global__ __launch_bounds__(kBlock) void k_active_scan(
    int T, const uint32_t* __restrict__ atiles, uint32_t* __restrict__ aoff) {
    __shared__ uint32_t lds[kWavesPerBlock];
    uint32_t carry = 0;
    for (int base = 0; base < T; base += kBlock) {
        int t = base + threadIdx.x;
        uint32_t c = t < T ? atiles[t] : 0;
        uint32_t tot;
        uint32_t ex = block_exclusive_scan(c, lds, tot);
        if (t < T) aoff[t] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) aoff[T] = carry;
}

// One block per tensor: amap[a] = t for the tensor's active tiles.
__global__ __launch_bounds__(kBlock) void k_active_map(
    const uint32_t* __restrict__ atiles, const uint32_t* __restrict__ aoff,
    uint32_t* __restrict__ amap) {
    const int t = blockIdx.x;
    const uint32_t a0 = aoff[t], n = atiles[t];
    for (uint32_t j = threadIdx.x; j < n; j += kBlock) amap[a0 + j] = uint32_t(t);
}

// ---------------------------------------------------------------- select

// The values of tensor t's selection source: v itself on the dense path,
// else the candidate list's values (item i of the list is local index
// olist_i[obase + i]; item i of the dense source is index i).
__device__ __forceinline__ const float* source_values(uint32_t mode, const float* v,
                                                      const float* olist_v,
                                                      const DevLayout& L, int t) {
    return mode == kModeDense ? v + L.o[t] : olist_v + L.obase[t];
}

// Items ib .. ib + kPerThread - 1 of a selection source (0 past len): one
// 16-byte load when they are all there and 16-byte aligned (candidate lists
// start 16-byte aligned; a tensor's v does when its offset is a multiple of
// 4).
template <typename T>
__device__ __forceinline__ void load_items(const T* __restrict__ src, int64_t ib, int64_t len,
                                           T (&x)[kPerThread]) {
    static_assert(kPerThread == 4 && sizeof(T) == 4, "one 16-byte load per thread");
    if (ib + kPerThread <= len &&
        (reinterpret_cast<uintptr_t>(src + ib) & 15) == 0) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        const T4 y = *reinterpret_cast<const T4*>(src + ib);
        x[0] = y.x;
        x[1] = y.y;
        x[2] = y.z;
        x[3] = y.w;
    } else {
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) x[q] = ib + q < len ? src[ib + q] : T(0);
    }
}

template <int D>
struct Digit;
template <> struct Digit<0> { static constexpr int shift = 20, bits = 11; };
template <> struct Digit<1> { static constexpr int shift = 10, bits = 10; };
template <> struct Digit<2> { static constexpr int shift = 0, bits = 10; };

__device__ __forceinline__ void flush_hist(uint32_t* h, uint32_t* row) {
    __syncthreads();
    for (int b = threadIdx.x; b < kHistBins; b += kBlock) {
        uint32_t c = h[b];
        if (c) { atomicAdd(&row[b], c); h[b] = 0; }
    }
    __syncthreads();
}

// Active tiles: a in [0, aoff[T]) is tile (a - aoff[t]) of tensor
// t = amap[a]; the tile covers source items [kTile j, kTile (j + 1)) of the
// tensor's source (candidate list or whole tensor), clipped to len.  A
// workgroup's tiles only grow, so the walks keep the current tensor's state
// and load it again only past that tensor's last active tile (one round of
// dependent loads per tile instead of three).

// Histogram of digit D over the keys that match the prefix found so far.
// Workgroups stride over the active tiles.
template <int D>
__global__ __launch_bounds__(kBlock) void k_hist(
    DevLayout L, const TensorState* __restrict__ ts,
    const float* __restrict__ v, const float* __restrict__ olist_v,
    const uint32_t* __restrict__ amap, const uint32_t* __restrict__ aoff,
    uint32_t* __restrict__ hist) {
    constexpr int shift = Digit<D>::shift, bits = Digit<D>::bits;
    constexpr uint32_t dmask = (1u << bits) - 1;
    __shared__ uint32_t h[kHistBins];
    for (int b = threadIdx.x; b < kHistBins; b += kBlock) h[b] = 0;
    __syncthreads();
    const uint32_t A = aoff[L.T];
    int cur_t = -1;
    // current tensor: active tiles [ab, ae)
    uint32_t ab = 0, ae = 0, prefix = 0, fl = 0;
    int64_t len = 0;
    const float* src = v;
    for (uint32_t a = blockIdx.x; a < A; a += gridDim.x) {
        if (a >= ae) {  // uniform: the next tensor
            const int t = int(amap[a]);
            const uint32_t mode = ts[t].mode;
            len = ts[t].len;
            prefix = ts[t].prefix;
            fl = ts[t].floor;
            ab = aoff[t];
            ae = aoff[t + 1];
            src = source_values(mode, v, olist_v, L, t);
            if (cur_t >= 0) flush_hist(h, hist + int64_t(cur_t) * kHistBins);
            cur_t = t;
            // uniform: resolved from the gather (D < 2), or nothing to select
            if (ts[t].done21 > (D < 2 ? 0u : kDone21)) {
                // this workgroup's next tile at or past the tensor's end (the
                // loop's step adds the last stride)
                a += ((ae - a + gridDim.x - 1) / gridDim.x - 1) * gridDim.x;
                continue;
            }
        }
        // a thread's kPerThread consecutive items (a histogram does not
        // depend on the order): one 16-byte load when the source allows
        const int64_t ib = int64_t(a - ab) * kTile + int64_t(threadIdx.x) * kPerThread;
        float x[kPerThread];
        load_items(src, ib, len, x);
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            if (ib + q >= len) break;
            const uint32_t key = floor_key(mag_key(x[q]), fl);
            if (D == 0 || (key >> (shift + bits)) == prefix)
                atomicAdd(&h[(key >> shift) & dmask], 1u);
        }
    }
    if (cur_t >= 0) flush_hist(h, hist + int64_t(cur_t) * kHistBins);
}

// r once the last digit is placed: under the hierarchical selector's floor
// T = 0 means fewer than k survivors, which are then all sent (the keys at
// 0 are not survivors), so r = 0.
template <int D>
__device__ __forceinline__ uint32_t last_rank(uint32_t T, uint32_t r, uint32_t floor) {
    return (D == 2 && T == 0 && floor != 0) ? 0u : r;
}

// One block per tensor: find the bin of digit D holding the krem-th largest
// matching key; extend the prefix and reduce krem.  Clears the histogram.
// After D = 2, prefix is the k-th largest key T and krem is the number of
// keys equal to T to take (r).
template <int D>
__global__ __launch_bounds__(kBlock) void k_resolve(
    TensorState* __restrict__ ts, uint32_t* __restrict__ hist,
    Scalars* __restrict__ sc) {
    constexpr int bins = 1 << Digit<D>::bits;
    constexpr int per = bins / kBlock;
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ int found;
    const int t = blockIdx.x;
    if (ts[t].mode == kModeSkip) return;
    // the gather's histogram resolved it (D < 2), or nothing to select
    if (ts[t].done21 > (D < 2 ? 0u : kDone21)) return;
    uint32_t* row = hist + int64_t(t) * kHistBins;
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        c[q] = row[bins - 1 - (threadIdx.x * per + q)];
        mine += c[q];
    }
    if (threadIdx.x == 0) found = 0;
    uint32_t total;
    uint32_t above = block_exclusive_scan(mine, lds, total);
#pragma unroll
    for (int q = 0; q < per; ++q) row[bins - 1 - (threadIdx.x * per + q)] = 0;
    const uint32_t krem = ts[t].krem;
    const uint32_t prefix = ts[t].prefix;
    const uint32_t fl = ts[t].floor;
    __syncthreads();  // every thread has read prefix/krem before the update
    uint32_t run = above;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (run < krem && krem <= run + c[q]) {
            uint32_t b = uint32_t(bins - 1 - (threadIdx.x * per + q));
            const uint32_t np = (prefix << Digit<D>::bits) | b;
            ts[t].prefix = np;
            ts[t].krem = last_rank<D>(np, krem - run, fl);
            found = 1;
        }
        run += c[q];
    }
    __syncthreads();
    if (threadIdx.x == 0 && !found) latch_error(sc, kErrInternal);
}

// ---------------------------------------------------------------- emit

// Tiles are visited in kPerThread rounds of 256 consecutive items (item
// i0 + 256 q + tid), so every load and store of a round is coalesced.

// Per active tile: packed (#key > T) << 16 | #key == T.
__global__ __launch_bounds__(kBlock) void k_emit_count(
    DevLayout L, const TensorState* __restrict__ ts,
    const float* __restrict__ v, const float* __restrict__ olist_v,
    const uint32_t* __restrict__ amap, const uint32_t* __restrict__ aoff,
    uint32_t* __restrict__ tile_cnt) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const uint32_t A = aoff[L.T];
    uint32_t ab = 0, ae = 0, T = 0, fl = 0;  // current tensor: active tiles [ab, ae)
    int64_t len = 0;
    const float* src = v;
    for (uint32_t a = blockIdx.x; a < A; a += gridDim.x) {
        if (a >= ae) {  // uniform: the next tensor
            const int t = int(amap[a]);
            const uint32_t mode = ts[t].mode;
            len = ts[t].len;
            T = ts[t].prefix;
            fl = ts[t].floor;
            ab = aoff[t];
            ae = aoff[t + 1];
            src = source_values(mode, v, olist_v, L, t);
        }
        // a thread's kPerThread consecutive items (the tile's counts do not
        // depend on the order)
        const int64_t ib = int64_t(a - ab) * kTile + int64_t(threadIdx.x) * kPerThread;
        float x[kPerThread];
        load_items(src, ib, len, x);
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            if (ib + q < len) {
                const uint32_t key = floor_key(mag_key(x[q]), fl);
                cnt += (key > T) ? (1u << 16) : (key == T ? 1u : 0u);
            }
        }
        uint32_t tot;
        block_exclusive_scan(cnt, lds, tot);
        if (threadIdx.x == 0) tile_cnt[a] = tot;
    }
}

// One block per tensor: exclusive scan of its tiles' (>T, ==T) counts.
// With out_count set, also the tensor's sent count, #key > T + min(#key ==
// T, r) (k_t for exact top-k).
template <bool kStaged>
__global__ __launch_bounds__(kBlock) void k_emit_scan(
    const uint32_t* __restrict__ aoff, const uint32_t* __restrict__ tile_cnt,
    uint32_t* __restrict__ off_gt, uint32_t* __restrict__ off_eq,
    const TensorState* __restrict__ ts, int64_t* __restrict__ out_count) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t stage[kStaged ? kScanStage : 1];
    const int t = blockIdx.x;
    const uint32_t a0 = aoff[t];
    const int64_t na = int64_t(aoff[t + 1]) - a0;
    uint32_t cg = 0, ce = 0;
    for (int64_t base = 0; base < na; base += kScanRound) {
        uint32_t x[kScanPer];
        scan_load_round<kStaged>(tile_cnt + a0, base, na, stage, x);
        uint32_t lg = 0, le = 0;
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) {
            lg += x[q] >> 16;
            le += x[q] & 0xFFFFu;
        }
        uint32_t tg, te;
        uint32_t rg = cg + block_exclusive_scan(lg, lds, tg);
        uint32_t re = ce + block_exclusive_scan(le, lds, te);
        uint32_t r[kScanPer];
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) {
            r[q] = rg;
            rg += x[q] >> 16;
        }
        scan_store_round<kStaged>(off_gt + a0, base, na, stage, r);
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) {
            r[q] = re;
            re += x[q] & 0xFFFFu;
        }
        scan_store_round<kStaged>(off_eq + a0, base, na, stage, r);
        cg += tg;
        ce += te;
    }
    if (out_count && threadIdx.x == 0)
        out_count[t] = ts[t].mode == kModeSkip ? 0 : int64_t(cg) + min(ce, ts[t].krem);
}

// Where rank e of a tile's sent items sits in the LDS stage: bits 5-6 of e
// swizzle bits 0-1.  A thread stages its 4 consecutive items, so the lanes
// of one store are 4 ranks apart and, unswizzled, lanes l, l + 8, l + 16
// and l + 24 hit one bank; swizzled they do not, and the coalesced reads
// (consecutive ranks) stay a permutation of each 32-rank row.  A bijection
// on [0, kTile).
__device__ __forceinline__ uint32_t stage_at(uint32_t e) { return e ^ ((e >> 5) & 3u); }

// Per active tile: write the selected items in index order.  An item with
// key > T, or key == T while fewer than r ties precede it, is sent; its
// output slot is (#sent before it) = gt_before + min(eq_before, r).  On the
// dense path the sent items' u and v are masked here; on the list path the
// fused pass has masked every candidate already, and the candidates not
// sent get their u and v back.
__global__ __launch_bounds__(kBlock) void k_emit_write(
    DevLayout L, DevK K, const TensorState* __restrict__ ts,
    float* __restrict__ u, float* __restrict__ v,
    const uint32_t* __restrict__ olist_i, const float* __restrict__ olist_v,
    const float* __restrict__ olist_u, const uint32_t* __restrict__ amap,
    const uint32_t* __restrict__ aoff,
    const uint32_t* __restrict__ off_gt, const uint32_t* __restrict__ off_eq,
    uint32_t* __restrict__ out_idx,
    float* __restrict__ out_val, Scalars* __restrict__ sc) {
    __shared__ uint32_t lds2[kWavesPerBlock];
    __shared__ uint32_t s_idx[kTile];
    __shared__ float s_val[kTile];
    const uint32_t A = aoff[L.T];
    // current tensor: active tiles [ab, ae)
    uint32_t ab = 0, ae = 0, T = 0, r = 0, fl = 0;
    int64_t len = 0, o = 0, kt = 0, nt = 0;
    bool dense = false;
    float* vt_ = v;
    const float* src = v;
    const uint32_t* oli = olist_i;
    const float* olu = olist_u;
    uint32_t* oi = out_idx;
    float* ov = out_val;
    // A thread takes 4 consecutive items of a tile (vector loads; on the
    // list path the saved u comes too, the items not sent need it).  The
    // next tile of the same tensor is loaded before this one is worked on
    // (its loads then wait behind this tile's scan and stores, not in
    // front of the next one's).
    auto load_tile = [&](uint32_t at, uint32_t& cg, uint32_t& ce, float (&val)[kPerThread],
                         uint32_t (&lidx)[kPerThread], float (&usv)[kPerThread]) {
        cg = off_gt[at];
        ce = off_eq[at];
        const int64_t ib = int64_t(at - ab) * kTile + int64_t(threadIdx.x) * kPerThread;
        load_items(src, ib, len, val);
        if (dense) {
#pragma unroll
            for (int q = 0; q < kPerThread; ++q) {
                lidx[q] = uint32_t(ib + q);
                usv[q] = 0.0f;
            }
        } else {
            load_items(oli, ib, len, lidx);
            load_items(olu, ib, len, usv);
        }
    };
    bool have = false;  // the tile's loads were issued by the previous iteration
    uint32_t ncg = 0, nce = 0, nlidx[kPerThread];
    float nval[kPerThread], nusv[kPerThread];
    for (uint32_t a = blockIdx.x; a < A; a += gridDim.x) {
        if (a >= ae) {  // uniform: the next tensor
            const int t = int(amap[a]);
            const uint32_t mode = ts[t].mode;
            len = ts[t].len;
            T = ts[t].prefix;
            r = ts[t].krem;
            fl = ts[t].floor;
            o = L.o[t];
            nt = L.o[t + 1] - o;
            vt_ = v + o;
            dense = mode == kModeDense;
            src = source_values(mode, v, olist_v, L, t);
            oli = olist_i + L.obase[t];
            olu = olist_u + L.obase[t];
            oi = out_idx + K.koff[t];
            ov = out_val + K.koff[t];
            kt = K.k[t];
            ab = aoff[t];
            ae = aoff[t + 1];
            have = false;
        }
        // One block scan of the packed (#key > T, #key == T) counts gives
        // each item its place in index order; the sent items are staged in
        // LDS by their rank among the tile's sent items and stored coalesced.
        uint32_t cg, ce;
        float val[kPerThread], usv[kPerThread];
        uint32_t lidx[kPerThread];
        if (have) {  // uniform
            cg = ncg;
            ce = nce;
#pragma unroll
            for (int q = 0; q < kPerThread; ++q) {
                val[q] = nval[q];
                lidx[q] = nlidx[q];
                usv[q] = nusv[q];
            }
        } else {
            load_tile(a, cg, ce, val, lidx, usv);
        }
        const uint32_t an = a + gridDim.x;
        have = an < ae;  // uniform
        if (have) load_tile(an, ncg, nce, nval, nlidx, nusv);
        const int64_t ib = int64_t(a - ab) * kTile + int64_t(threadIdx.x) * kPerThread;
        bool bad = false;
        bool gt[kPerThread], eq[kPerThread];
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const bool ok = ib + q < len;
            const uint32_t key = floor_key(mag_key(val[q]), fl);
            gt[q] = ok && key > T;
            eq[q] = ok && key == T;
            c += (gt[q] ? (1u << 16) : 0u) + (eq[q] ? 1u : 0u);
        }
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan(c, lds2, tot);
        // items sent before the tile, and by the end of it
        const uint32_t sent0 = cg + min(ce, r);
        const uint32_t sent1 = cg + (tot >> 16) + min(ce + (tot & 0xFFFFu), r);
        uint32_t gb = cg + (pre >> 16), eb = ce + (pre & 0xFFFFu);
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            bool send = false;
            uint32_t slot = 0;
            if (gt[q]) { send = true; slot = gb + min(eb, r); }
            else if (eq[q] && eb < r) { send = true; slot = gb + eb; }
            gb += gt[q];
            eb += eq[q];
            if (send) {
                // never write outside the outputs, whatever the counts say
                if (int64_t(slot) >= kt || int64_t(lidx[q]) >= nt || slot - sent0 >= kTile) {
                    bad = true;
                } else {
                    s_idx[stage_at(slot - sent0)] = lidx[q];
                    s_val[stage_at(slot - sent0)] = val[q];
                    if (dense) {
                        u[o + lidx[q]] = 0.0f;
                        vt_[lidx[q]] = 0.0f;
                    }
                }
            } else if (ib + q < len && !dense) {
                if (int64_t(lidx[q]) >= nt) {
                    bad = true;
                } else {
                    u[o + lidx[q]] = usv[q];
                    vt_[lidx[q]] = val[q];
                }
            }
        }
        __syncthreads();
        const uint32_t ns = min(sent1 - sent0, uint32_t(kTile));
        for (uint32_t e = threadIdx.x; e < ns; e += kBlock) {
            if (int64_t(sent0 + e) < kt) {
                oi[sent0 + e] = s_idx[stage_at(e)];
                ov[sent0 + e] = s_val[stage_at(e)];
            }
        }
        __syncthreads();  // before the next tile overwrites the stage
        if (bad) latch_error(sc, kErrInternal);
    }
}

// ---------------------------------------------------------------- per tensor

// The same select and emit for one tensor in one 1024-thread workgroup,
// after the spread path's gather (DGC_OPT_SELECT_GRID 1 on layouts that the
// per-tensor kernels of kernels_tensor.hpp do not take): the three digit
// histograms live in LDS and are resolved in place, and the emit splits the
// source into 16 index-ordered wave chunks whose counts give each wave its
// output offsets.  One launch replaces the eleven of the spread passes
// (active tiles, three histogram and resolve pairs, count, scan, write).
// One workgroup sweeps ~3.7 G items/s, so long sources go faster as spread
// passes.  Results and the per-tensor record (prefix = T, krem = r) are the
// same as the spread passes'.
constexpr int kTsThreads = 1024;
constexpr int kTsWaves = kTsThreads / kWave;
constexpr int kTsHistUnroll = 8;  // keys loaded together per thread
constexpr int kTsEmitUnroll = 4;  // 64-item rounds loaded together per wave

// The tensor's sent count from the emit's per-wave counts (wcnt[w]: keys
// > T of wave w, wcnt[kTsWaves + w]: keys == T): #key > T + min(#key == T,
// r).
__device__ __forceinline__ int64_t sent_count(const uint32_t* wcnt, uint32_t r) {
    uint32_t g = 0, e = 0;
    for (int j = 0; j < kTsWaves; ++j) {
        g += wcnt[j];
        e += wcnt[kTsWaves + j];
    }
    return int64_t(g) + min(e, r);
}

// Exclusive scan across the 1024-thread workgroup; `lds` holds kTsWaves
// values.  Every thread must call it.
__device__ __forceinline__ uint32_t ts_block_scan(uint32_t x, uint32_t* lds, uint32_t& total) {
    const int lane = lane_id();
    const int wid = int(threadIdx.x) >> 6;
    const uint32_t inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) lds[wid] = inc;
    __syncthreads();
    uint32_t wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w) {
        const uint32_t s = lds[w];
        if (w < wid) wpre += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return wpre + inc - x;
}

// Digit D of the radix select over src[0, len): histogram of the keys that
// match the prefix, then the bin holding the krem-th largest; extends the
// prefix and reduces krem.  Returns false (uniformly) if no bin holds it.
template <int D>
__device__ __forceinline__ bool ts_digit(const float* __restrict__ src, int64_t len,
                                         uint32_t fl, uint32_t& prefix, uint32_t& krem,
                                         uint32_t* h, uint32_t* lds, uint32_t* pick) {
    constexpr int shift = Digit<D>::shift, bits = Digit<D>::bits;
    constexpr int bins = 1 << bits;
    constexpr uint32_t dmask = uint32_t(bins) - 1u;
    constexpr int per = (bins + kTsThreads - 1) / kTsThreads;
    const int tid = int(threadIdx.x);
    for (int b = tid; b < bins; b += kTsThreads) h[b] = 0;
    if (tid == 0) pick[0] = kNoKey;
    __syncthreads();
    for (int64_t i0 = 0; i0 < len; i0 += int64_t(kTsThreads) * kTsHistUnroll) {
        uint32_t key[kTsHistUnroll];
#pragma unroll
        for (int q = 0; q < kTsHistUnroll; ++q) {
            const int64_t i = i0 + int64_t(q) * kTsThreads + tid;
            key[q] = i < len ? floor_key(mag_key(src[i]), fl) : kNoKey;
        }
#pragma unroll
        for (int q = 0; q < kTsHistUnroll; ++q)
            if (key[q] != kNoKey && (D == 0 || (key[q] >> (shift + bits)) == prefix))
                atomicAdd(&h[(key[q] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread j owns bins bins-1-j*per ... bins-per-j*per (descending)
    uint32_t c[per];
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        const int b = bins - 1 - (tid * per + q);
        c[q] = b >= 0 ? h[b] : 0u;
        mine += c[q];
    }
    uint32_t total;
    uint32_t run = ts_block_scan(mine, lds, total);
#pragma unroll
    for (int q = 0; q < per; ++q) {
        if (run < krem && krem <= run + c[q]) {
            pick[0] = uint32_t(bins - 1 - (tid * per + q));
            pick[1] = krem - run;
        }
        run += c[q];
    }
    __syncthreads();
    const uint32_t b = pick[0], kr = pick[1];
    __syncthreads();  // every thread has read pick before the next digit
    if (b == kNoKey) return false;
    prefix = (prefix << bits) | b;
    krem = last_rank<D>(prefix, kr, fl);
    return true;
}

// One workgroup per tensor (grid = T).  Runs after k_group_scan and
// k_gather, like the spread passes it replaces.
__global__ __launch_bounds__(kTsThreads) void k_select_tensor(
    DevLayout L, DevK K, TensorState* __restrict__ ts,
    float* __restrict__ u, float* __restrict__ v,
    const uint32_t* __restrict__ olist_i, const float* __restrict__ olist_v,
    const float* __restrict__ olist_u, uint32_t* __restrict__ out_idx,
    float* __restrict__ out_val, int64_t* __restrict__ out_count,
    Scalars* __restrict__ sc) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t lds[kTsWaves];
    __shared__ uint32_t wcnt[2 * kTsWaves];
    __shared__ uint32_t pick[2];
    const int t = blockIdx.x;
    const uint32_t mode = ts[t].mode;
    if (mode == kModeSkip) {  // uniform
        if (out_count && threadIdx.x == 0) out_count[t] = 0;
        return;
    }
    const int64_t len = ts[t].len;
    const float* src = source_values(mode, v, olist_v, L, t);
    const uint32_t fl = ts[t].floor;
    uint32_t prefix = ts[t].prefix, krem = ts[t].krem;
    bool ok = true;
    if (ts[t].done21 != kDoneAll) {  // uniform
        ok = ts_digit<0>(src, len, fl, prefix, krem, h, lds, pick);
        ok = ok && ts_digit<1>(src, len, fl, prefix, krem, h, lds, pick);
        ok = ok && ts_digit<2>(src, len, fl, prefix, krem, h, lds, pick);
    }
    if (!ok) {  // uniform
        if (threadIdx.x == 0) latch_error(sc, kErrInternal);
        return;
    }
    if (threadIdx.x == 0) {
        ts[t].prefix = prefix;
        ts[t].krem = krem;
    }
    // Emit in index order.  Wave w owns items [c0, c1), a run of whole
    // 64-item rounds; a count pass gives every wave its offsets.
    const uint32_t T = prefix, r = krem;
    const bool dense = mode == kModeDense;
    const int lane = lane_id(), w = int(threadIdx.x) >> 6;
    const int64_t rounds = (len + kWave - 1) / kWave;
    const int64_t rpw = (rounds + kTsWaves - 1) / kTsWaves;
    const int64_t c0 = min(len, int64_t(w) * rpw * kWave);
    const int64_t c1 = min(len, int64_t(w + 1) * rpw * kWave);
    constexpr int64_t kStep = int64_t(kWave) * kTsEmitUnroll;
    uint32_t ng = 0, ne = 0;
    for (int64_t b0 = c0; b0 < c1; b0 += kStep) {
        uint32_t key[kTsEmitUnroll];
#pragma unroll
        for (int q = 0; q < kTsEmitUnroll; ++q) {
            const int64_t i = b0 + int64_t(q) * kWave + lane;
            key[q] = i < c1 ? floor_key(mag_key(src[i]), fl) : kNoKey;
        }
#pragma unroll
        for (int q = 0; q < kTsEmitUnroll; ++q) {
            ng += uint32_t(__popcll(__ballot(key[q] != kNoKey && key[q] > T)));
            ne += uint32_t(__popcll(__ballot(key[q] == T)));
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
    if (out_count && threadIdx.x == 0) out_count[t] = sent_count(wcnt, r);
    const int64_t o = L.o[t];
    const int64_t nt = L.o[t + 1] - o;
    float* vt_ = v + o;
    const uint32_t* oli = olist_i + L.obase[t];
    const float* olu = olist_u + L.obase[t];
    uint32_t* oi = out_idx + K.koff[t];
    float* ov = out_val + K.koff[t];
    const int64_t kt = K.k[t];
    const uint64_t lt = lanemask_lt();
    bool bad = false;
    for (int64_t b0 = c0; b0 < c1; b0 += kStep) {
        float val[kTsEmitUnroll], usv[kTsEmitUnroll];
        uint32_t lidx[kTsEmitUnroll];
        bool in[kTsEmitUnroll];
#pragma unroll
        for (int q = 0; q < kTsEmitUnroll; ++q) {
            const int64_t i = b0 + int64_t(q) * kWave + lane;
            in[q] = i < c1;
            val[q] = in[q] ? src[i] : 0.0f;
            lidx[q] = uint32_t(i);
            usv[q] = 0.0f;
            if (!dense && in[q]) {  // the list's index and saved u
                lidx[q] = oli[i];
                usv[q] = olu[i];
            }
        }
#pragma unroll
        for (int q = 0; q < kTsEmitUnroll; ++q) {
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
                if (int64_t(slot) >= kt || int64_t(lidx[q]) >= nt) {
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
}

}  // namespace dgc
