// kernels_codec.hpp -- zero-run encoding and decode + sum on gfx950.
//
// Format: DGC review page (nubint.ai), "Proposed method": sparse gradients
// leave as 32-bit values, each preceded by the 16-bit length of the zero run
// before it.  Per tensor, for the sent indices j in ascending order with gap
// G = j - prev - 1: floor(G/65536) fillers (65535, +0.0f), then
// (G mod 65536, value).  Runs and values are separate arrays (u16 and f32)
// at each tensor's capacity offset.
//
// Both directions are two-level scans over kTile-item tiles: count per tile,
// scan per tensor, then write.  The decoder adds each learner's stream with
// a plain read-modify-write: positions inside one stream are strictly
// increasing, so no two items of one launch touch the same element, and
// learners are added one launch after another in learner order.
#pragma once

#include "dgc_device.hpp"

namespace dgc {

// ---------------------------------------------------------------- encode

// Tiles of kTile entries are visited in kPerThread rounds of 256 consecutive
// entries (entry i0 + 256 q + tid), so loads and stores are coalesced.

// Fillers needed by entry i of a tensor's sorted index list (0 for an entry
// whose index is not above the previous one or not inside the tensor, which
// is flagged).
__device__ __forceinline__ uint32_t fillers_of(const uint32_t* id, int64_t i,
                                               int64_t nt, bool& bad,
                                               int64_t& gap) {
    const int64_t cur = id[i];
    const int64_t prev = i ? int64_t(id[i - 1]) : -1;
    if (cur <= prev || cur >= nt) { bad = true; gap = -1; return 0; }
    gap = cur - prev - 1;
    return uint32_t(gap >> 16);
}

// Entries of tensor t to encode: k_t, or, when the counts live on the
// device (a data-dependent selector), that count if it lies in [0, k_t] and
// else none (k_enc_scan flags it).
__device__ __forceinline__ int64_t enc_len(const DevK& K, const int64_t* kdev, int t) {
    const int64_t k = K.k[t];
    if (!kdev) return k;
    const int64_t c = kdev[t];
    return (c < 0 || c > k) ? 0 : c;
}

// Per k-tile: number of fillers its entries need.
__global__ __launch_bounds__(kBlock) void k_enc_count(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ idx, uint32_t* __restrict__ tile_f,
    Scalars* __restrict__ sc, int64_t n_ktiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_ktiles; vt += gridDim.x) {
        const int t = int(K.kmap[vt]);
        const int64_t kt = enc_len(K, kdev, t);
        const int64_t nt = L.o[t + 1] - L.o[t];
        const uint32_t* id = idx + K.koff[t];
        const int64_t i0 = (vt - K.ktbase[t]) * kTile;
        uint32_t f = 0;
        bool bad = false;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = i0 + q * kBlock + threadIdx.x;
            if (i < kt) {
                int64_t gap;
                f += fillers_of(id, i, nt, bad, gap);
            }
        }
        if (bad) latch_error(sc, kErrCorrupt);
        uint32_t tot;
        block_exclusive_scan(f, lds, tot);
        if (threadIdx.x == 0) tile_f[vt] = tot;
    }
}

// One block per tensor: scan the filler counts; E_t = k_t + fillers.
__global__ __launch_bounds__(kBlock) void k_enc_scan(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ tile_f, uint32_t* __restrict__ tile_foff,
    int64_t* __restrict__ entries, Scalars* __restrict__ sc) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t kb = K.ktbase[t], ntile = K.ktbase[t + 1] - kb;
    const uint32_t carry = block_scan_range<uint32_t>(tile_f + kb, tile_foff + kb, ntile, 0u, lds);
    if (threadIdx.x == 0) {
        if (kdev && (kdev[t] < 0 || kdev[t] > K.k[t])) latch_error(sc, kErrCorrupt);
        entries[t] = enc_len(K, kdev, t) + int64_t(carry);
    }
}

// Entry i lands at slot i + (fillers of entries <= i); its own fillers fill
// the slots just before it.
__global__ __launch_bounds__(kBlock) void k_enc_write(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ idx, const float* __restrict__ val,
    const uint32_t* __restrict__ tile_foff, uint16_t* __restrict__ runs,
    float* __restrict__ vals, int64_t n_ktiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_ktiles; vt += gridDim.x) {
        const int t = int(K.kmap[vt]);
        const int64_t kt = enc_len(K, kdev, t);
        const int64_t nt = L.o[t + 1] - L.o[t];
        const uint32_t* id = idx + K.koff[t];
        const float* vl = val + K.koff[t];
        const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
        const int64_t i0 = (vt - K.ktbase[t]) * kTile;
        uint32_t carry = tile_foff[vt];
        for (int q = 0; q < kPerThread; ++q) {
            if (i0 + q * kBlock >= kt) break;  // uniform
            const int64_t i = i0 + q * kBlock + threadIdx.x;
            bool bad = false;
            int64_t gap = -1;
            const uint32_t nf = i < kt ? fillers_of(id, i, nt, bad, gap) : 0u;
            uint32_t pre = 0, tot = 0;
            if (__syncthreads_or(nf != 0))  // fillers are rare: skip the scan
                pre = block_exclusive_scan(nf, lds, tot);
            if (i < kt && gap >= 0) {
                int64_t pos = i + int64_t(carry) + pre;
                for (uint32_t z = 0; z < nf; ++z, ++pos)
                    if (pos < cap) { runs[eb + pos] = 65535; vals[eb + pos] = 0.0f; }
                if (pos < cap) {
                    runs[eb + pos] = uint16_t(gap & 0xFFFF);
                    vals[eb + pos] = vl[i];
                }
            }
            carry += tot;
        }
    }
}

// ---------------------------------------------------------------- decode

__device__ __forceinline__ int64_t stream_len(const int64_t* entries, int t,
                                              int64_t cap) {
    int64_t e = entries[t];
    return (e < 0 || e > cap) ? 0 : e;
}

// Per capacity tile of one learner's stream: sum of (run + 1).  Flags an
// entry count outside [0, capacity].
__global__ __launch_bounds__(kBlock) void k_dec_count(
    DevLayout L, const uint16_t* __restrict__ runs,
    const int64_t* __restrict__ entries, uint32_t* __restrict__ tile_s,
    Scalars* __restrict__ sc, int64_t n_etiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_etiles; vt += gridDim.x) {
        const int t = int(L.emap[vt]);
        const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
        const int64_t j = vt - L.etbase[t];
        if (j == 0 && threadIdx.x == 0) {
            int64_t e = entries[t];
            if (e < 0 || e > cap) latch_error(sc, kErrCorrupt);
        }
        const int64_t E = stream_len(entries, t, cap);
        const int64_t i0 = j * kTile;
        uint32_t s = 0;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = i0 + q * kBlock + threadIdx.x;
            if (i < E) s += uint32_t(runs[eb + i]) + 1u;
        }
        uint32_t tot;
        block_exclusive_scan(s, lds, tot);
        if (threadIdx.x == 0) tile_s[vt] = tot;
    }
}

// One block per tensor: 64-bit exclusive scan of the tile sums.
__global__ __launch_bounds__(kBlock) void k_dec_scan(
    DevLayout L, const uint32_t* __restrict__ tile_s,
    uint64_t* __restrict__ tile_p) {
    __shared__ uint64_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t tb = L.etbase[t], ntile = L.etbase[t + 1] - tb;
    block_scan_range<uint64_t>(tile_s + tb, tile_p + tb, ntile, uint64_t(0), lds);
}

// dense[o_t + pos] += value for every entry of one learner's stream, where
// pos = (sum of run + 1 over the entries up to this one) - 1.  Entries whose
// position reaches the tensor's end add nothing and flag the stream as
// corrupt (positions only grow, so every later entry is past the end too).
__global__ __launch_bounds__(kBlock) void k_dec_write(
    DevLayout L, const uint16_t* __restrict__ runs,
    const float* __restrict__ vals, const int64_t* __restrict__ entries,
    const uint64_t* __restrict__ tile_p, float* __restrict__ dense,
    Scalars* __restrict__ sc, int64_t n_etiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_etiles; vt += gridDim.x) {
        const int t = int(L.emap[vt]);
        const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
        const int64_t o = L.o[t], nt = L.o[t + 1] - o;
        const int64_t E = stream_len(entries, t, cap);
        const int64_t i0 = (vt - L.etbase[t]) * kTile;
        uint64_t carry = tile_p[vt];
        bool bad = false;
        for (int q = 0; q < kPerThread; ++q) {
            if (i0 + q * kBlock >= E) break;  // uniform
            const int64_t i = i0 + q * kBlock + threadIdx.x;
            const uint32_t w = i < E ? uint32_t(runs[eb + i]) + 1u : 0u;
            uint32_t tot;
            const uint32_t ex = block_exclusive_scan(w, lds, tot);
            if (i < E) {
                const int64_t pos = int64_t(carry) + ex + w - 1;
                if (pos >= nt) bad = true;
                else dense[o + pos] = __fadd_rn(dense[o + pos], vals[eb + i]);
            }
            carry += tot;
        }
        if (bad) latch_error(sc, kErrCorrupt);
    }
}

}  // namespace dgc
