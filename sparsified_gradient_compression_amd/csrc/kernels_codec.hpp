// kernels_codec.hpp -- zero-run encoding and decode + sum on gfx950.
//
// Format: DGC review page (nubint.ai), "Proposed method": sparse gradients
// leave as 32-bit values, each preceded by the 16-bit length of the zero run
// before it.  Per tensor, for the sent indices j in ascending order with gap
// G = j - prev - 1: floor(G/65536) fillers (65535, +0.0f), then
// (G mod 65536, value).  Runs and values are separate arrays (u16 and f32)
// at each tensor's capacity offset.
//
// Both directions are two-level scans over 4096-item tiles: count per tile,
// scan per tensor, then write.  The decoder adds each learner's stream with
// a plain read-modify-write: positions inside one stream are strictly
// increasing, so no two items of one launch touch the same element, and
// learners are added one launch after another in learner order.
#pragma once

#include "dgc_device.hpp"

namespace dgc {

// ---------------------------------------------------------------- encode

// Per k-tile: number of fillers its items need.  Flags indices that are not
// strictly ascending or not inside the tensor.
__global__ __launch_bounds__(kBlock) void k_enc_count(
    DevLayout L, DevK K, const uint32_t* __restrict__ idx,
    uint32_t* __restrict__ tile_f, Scalars* __restrict__ sc, int64_t n_ktiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_ktiles; vt += gridDim.x) {
        const int t = int(K.kmap[vt]);
        const int64_t kt = K.k[t];
        const int64_t nt = L.o[t + 1] - L.o[t];
        const uint32_t* id = idx + K.koff[t];
        const int64_t s0 = (vt - K.ktbase[t]) * kTile + int64_t(threadIdx.x) * kPerThread;
        uint32_t f = 0;
        bool bad = false;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
            if (i >= kt) break;
            int64_t cur = id[i];
            int64_t prev = i ? int64_t(id[i - 1]) : -1;
            if (cur <= prev || cur >= nt) { bad = true; continue; }
            f += uint32_t((cur - prev - 1) >> 16);
        }
        if (bad) latch_error(sc, kErrCorrupt);
        uint32_t tot;
        block_exclusive_scan(f, lds, tot);
        if (threadIdx.x == 0) tile_f[vt] = tot;
    }
}

// One block per tensor: scan the filler counts; E_t = k_t + fillers.
__global__ __launch_bounds__(kBlock) void k_enc_scan(
    DevLayout L, DevK K, const uint32_t* __restrict__ tile_f,
    uint32_t* __restrict__ tile_foff, int64_t* __restrict__ entries) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t kb = K.ktbase[t], ntile = K.ktbase[t + 1] - kb;
    uint32_t carry = 0;
    for (int64_t base = 0; base < ntile; base += kBlock) {
        int64_t j = base + threadIdx.x;
        uint32_t x = j < ntile ? tile_f[kb + j] : 0;
        uint32_t tot;
        uint32_t ex = block_exclusive_scan(x, lds, tot);
        if (j < ntile) tile_foff[kb + j] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) entries[t] = K.k[t] + int64_t(carry);
}

__global__ __launch_bounds__(kBlock) void k_enc_write(
    DevLayout L, DevK K, const uint32_t* __restrict__ idx,
    const float* __restrict__ val, const uint32_t* __restrict__ tile_foff,
    uint16_t* __restrict__ runs, float* __restrict__ vals, int64_t n_ktiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    for (int64_t vt = blockIdx.x; vt < n_ktiles; vt += gridDim.x) {
        const int t = int(K.kmap[vt]);
        const int64_t kt = K.k[t];
        const int64_t nt = L.o[t + 1] - L.o[t];
        const uint32_t* id = idx + K.koff[t];
        const float* vl = val + K.koff[t];
        const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
        const int64_t s0 = (vt - K.ktbase[t]) * kTile + int64_t(threadIdx.x) * kPerThread;
        uint32_t f = 0;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
            if (i >= kt) break;
            int64_t cur = id[i];
            int64_t prev = i ? int64_t(id[i - 1]) : -1;
            if (cur <= prev || cur >= nt) continue;
            f += uint32_t((cur - prev - 1) >> 16);
        }
        uint32_t tot;
        uint32_t fb = tile_foff[vt] + block_exclusive_scan(f, lds, tot);
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
            if (i >= kt) break;
            int64_t cur = id[i];
            int64_t prev = i ? int64_t(id[i - 1]) : -1;
            if (cur <= prev || cur >= nt) continue;
            int64_t gap = cur - prev - 1;
            uint32_t nf = uint32_t(gap >> 16);
            int64_t pos = i + int64_t(fb);
            for (uint32_t z = 0; z < nf; ++z, ++pos)
                if (pos < cap) { runs[eb + pos] = 65535; vals[eb + pos] = 0.0f; }
            if (pos < cap) {
                runs[eb + pos] = uint16_t(gap & 0xFFFF);
                vals[eb + pos] = vl[i];
            }
            fb += nf;
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
        const int64_t s0 = j * kTile + int64_t(threadIdx.x) * kPerThread;
        uint32_t s = 0;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
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
    uint64_t carry = 0;
    for (int64_t base = 0; base < ntile; base += kBlock) {
        int64_t j = base + threadIdx.x;
        uint64_t x = j < ntile ? tile_s[tb + j] : 0;
        uint64_t tot;
        uint64_t ex = block_exclusive_scan(x, lds, tot);
        if (j < ntile) tile_p[tb + j] = carry + ex;
        carry += tot;
    }
}

// dense[o_t + pos] += value for every entry of one learner's stream.
// Entries whose position reaches the tensor's end add nothing and flag the
// stream as corrupt (positions only grow, so every later entry is past the
// end too).
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
        const int64_t j = vt - L.etbase[t];
        const int64_t s0 = j * kTile + int64_t(threadIdx.x) * kPerThread;
        uint32_t s = 0;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
            if (i < E) s += uint32_t(runs[eb + i]) + 1u;
        }
        uint32_t tot;
        uint32_t ex = block_exclusive_scan(s, lds, tot);
        int64_t pos = int64_t(tile_p[vt]) + ex - 1;
        bool bad = false;
        for (int q = 0; q < kPerThread; ++q) {
            int64_t i = s0 + q;
            if (i >= E) break;
            pos += int64_t(runs[eb + i]) + 1;
            if (pos >= nt) { bad = true; break; }
            dense[o + pos] = __fadd_rn(dense[o + pos], vals[eb + i]);
        }
        if (bad) latch_error(sc, kErrCorrupt);
    }
}

}  // namespace dgc
