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

// Each tensor's stream capacity is a multiple of kStreamAlign entries, so
// a thread's kPerThread consecutive entries (a multiple of kPerThread from
// the stream start) sit at 8-byte aligned runs and 16-byte aligned values
// whenever the arrays themselves are 16-byte aligned: one load or store
// each instead of four.
constexpr int64_t kStreamAlign = 8;
static_assert(kStreamAlign % kPerThread == 0 && kPerThread == 4, "vector stream access");

__device__ __forceinline__ bool aligned_as(const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Tiles of kTile entries are visited in kPerThread rounds of 256 consecutive
// entries (entry i0 + 256 q + tid), so loads and stores are coalesced.

// Fillers needed by an entry at index cur after one at prev (-1 before the
// first): 0 for an index not above the previous one or not inside the
// tensor, which is flagged.
__device__ __forceinline__ uint32_t fillers_after(int64_t prev, int64_t cur, int64_t nt,
                                                  bool& bad, int64_t& gap) {
    if (cur <= prev || cur >= nt) { bad = true; gap = -1; return 0; }
    gap = cur - prev - 1;
    return uint32_t(gap >> 16);
}

// The same for entry i of a tensor's sorted index list.
__device__ __forceinline__ uint32_t fillers_of(const uint32_t* id, int64_t i,
                                               int64_t nt, bool& bad,
                                               int64_t& gap) {
    return fillers_after(i ? int64_t(id[i - 1]) : -1, int64_t(id[i]), nt, bad, gap);
}

// Walks over per-tensor tiles: workgroup b takes the run of consecutive
// tiles [c0, c1), the n tiles cut into gridDim.x runs.  A workgroup's tiles
// then mostly share a tensor, so the walks below keep the current tensor's
// metadata and load it again only when a tile lies past that tensor's last
// tile: most tiles wait for one round of loads instead of three (with
// tiles dealt out grid-stride, a stride above a tensor's tile count put
// every tile in a new tensor).  Once a tile lies past its tensor's
// entries so do the tensor's later tiles, so a walk skips straight to the
// next tensor.
__device__ __forceinline__ void tile_run(int64_t n, int64_t& c0, int64_t& c1) {
    const int64_t per = (n + int64_t(gridDim.x) - 1) / int64_t(gridDim.x);
    c0 = min(n, int64_t(blockIdx.x) * per);
    c1 = min(n, c0 + per);
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

// Per k-tile: number of fillers its entries need.  A filler needs a gap of
// at least 65536, and the gaps of a tile's entries add up to (its last
// index) - (the index before its first) - (its entries): a tile spanning
// less than that needs none, which two loads show (DGC's 0.1% spans ~1M
// positions per tile and takes the entry-by-entry count; denser streams
// mostly do not).  A workgroup tests its next kEncTest tiles at once, one
// thread each (a dense stream's tiles then cost one round of loads per
// kEncTest tiles instead of one each), and counts entry by entry only the
// tiles the test does not settle.  Index order is checked by the write.
constexpr int kEncTest = 16;

// The automatic choice takes one workgroup per tensor (k_enc_tensor) when
// no tensor holds more than this many tiles of entries.
constexpr int64_t kEncTensorTiles = 8;

__global__ __launch_bounds__(kBlock) void k_enc_count(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ idx, uint32_t* __restrict__ tile_f,
    Scalars* __restrict__ sc, int64_t n_ktiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t full[kEncTest];  // tests (thread numbers) left unsettled
    __shared__ uint32_t nfull;
    const int64_t G = gridDim.x;
    for (int64_t vt0 = blockIdx.x; vt0 < n_ktiles; vt0 += G * kEncTest) {
        if (threadIdx.x == 0) nfull = 0;
        __syncthreads();
        if (threadIdx.x < uint32_t(kEncTest)) {
            const int64_t vt = vt0 + int64_t(threadIdx.x) * G;
            if (vt < n_ktiles) {
                const int t = int(K.kmap[vt]);
                const int64_t kt = enc_len(K, kdev, t);
                const int64_t i0 = (vt - K.ktbase[t]) * kTile;
                if (i0 < kt) {  // else nothing here: the scan stops before this tile
                    const uint32_t* id = idx + K.koff[t];
                    const int64_t i1 = min(kt, i0 + kTile);
                    const int64_t before = i0 ? int64_t(id[i0 - 1]) : -1;
                    if (int64_t(id[i1 - 1]) - before - (i1 - i0) < 65536)
                        tile_f[vt] = 0;
                    else
                        full[atomicAdd(&nfull, 1u)] = threadIdx.x;
                }
            }
        }
        __syncthreads();
        const uint32_t nf = nfull;
        for (uint32_t q = 0; q < nf; ++q) {  // uniform
            const int64_t vt = vt0 + int64_t(full[q]) * G;
            const int t = int(K.kmap[vt]);
            const int64_t kt = enc_len(K, kdev, t);
            const int64_t nt = L.o[t + 1] - L.o[t];
            const uint32_t* id = idx + K.koff[t];
            const int64_t i0 = (vt - K.ktbase[t]) * kTile;
            uint32_t f = 0;
            bool bad = false;
            for (int c = 0; c < kPerThread; ++c) {
                const int64_t i = i0 + c * kBlock + threadIdx.x;
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
        __syncthreads();  // every thread has read full[] before the next round resets it
    }
}

// One block per tensor: scan the filler counts; E_t = k_t + fillers.
template <bool kStaged>
__global__ __launch_bounds__(kBlock) void k_enc_scan(
    DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ tile_f, uint32_t* __restrict__ tile_foff,
    int64_t* __restrict__ entries, Scalars* __restrict__ sc) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t stage[kStaged ? kScanStage : 1];
    const int t = blockIdx.x;
    const int64_t kt = enc_len(K, kdev, t);
    // only the tiles that hold entries (k_enc_count skips the rest)
    const int64_t kb = K.ktbase[t], ntile = (kt + kTile - 1) / kTile;
    const uint32_t carry = block_scan_range<uint32_t, kStaged>(tile_f + kb, tile_foff + kb, ntile,
                                                              0u, lds, stage);
    if (threadIdx.x == 0) {
        if (kdev && (kdev[t] < 0 || kdev[t] > K.k[t])) latch_error(sc, kErrCorrupt);
        entries[t] = kt + int64_t(carry);
    }
}

// LDS of one encode workgroup: the block scan's wave totals and the stage
// that writes a tile with fillers back in strided order.
struct EncStage {
    uint32_t lds[kWavesPerBlock];
    uint32_t sslot[kTile];
    uint16_t sgap[kTile];
    float sval[kTile];
};

// One tile of a tensor's sorted list: entries [i0, min(kt, i0 + kTile)) of
// id / vl (nt elements), with `carry` fillers before the tile.  Entry i
// lands at slot i + carry + (fillers of the tile's entries up to and
// including i) of runs / vals (the tensor's cap slots); its own fillers
// fill the slots just before it.  An index not above the previous one or
// outside the tensor latches DGC_ECORRUPT and is not written.  vin / vout:
// id and vl are 16-byte aligned; runs 8-byte and vals 16-byte aligned.
// Every thread of the block calls it; it returns the tile's fillers, the
// same in every thread.
__device__ __forceinline__ uint32_t enc_tile(
    const uint32_t* __restrict__ id, const float* __restrict__ vl, int64_t i0, int64_t kt,
    int64_t nt, int64_t carry, uint16_t* __restrict__ runs, float* __restrict__ vals,
    int64_t cap, bool vin, bool vout, Scalars* __restrict__ sc, EncStage& S) {
    // Each thread takes kPerThread consecutive entries: one load round
    // and at most one block scan (only when the tile has fillers) give
    // every entry its slot.  Without fillers up to the tile's end the
    // thread's entries land in kPerThread consecutive aligned slots and
    // are stored as vectors; otherwise they are written back in the
    // strided order through LDS, so a wave's stores stay contiguous.
    const int64_t ib = i0 + int64_t(threadIdx.x) * kPerThread;
    uint32_t nfv[kPerThread];
    int64_t gapv[kPerThread];
    float xv[kPerThread];
    uint32_t F = 0;
    bool bad = false;
    if (vin && ib + kPerThread <= kt) {
        const uint4 x = *reinterpret_cast<const uint4*>(id + ib);
        const float4 y = *reinterpret_cast<const float4*>(vl + ib);
        const int64_t cur[kPerThread] = {x.x, x.y, x.z, x.w};
        xv[0] = y.x;
        xv[1] = y.y;
        xv[2] = y.z;
        xv[3] = y.w;
        int64_t prev = ib ? int64_t(id[ib - 1]) : -1;
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            nfv[c] = fillers_after(prev, cur[c], nt, bad, gapv[c]);
            prev = cur[c];
            F += nfv[c];
        }
    } else {
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const int64_t i = ib + c;
            gapv[c] = -1;
            nfv[c] = i < kt ? fillers_of(id, i, nt, bad, gapv[c]) : 0u;
            xv[c] = i < kt ? vl[i] : 0.0f;
            F += nfv[c];
        }
    }
    if (bad) latch_error(sc, kErrCorrupt);
    uint32_t pre = 0, tot = 0;
    const bool anyF = __syncthreads_or(F != 0);
    if (anyF)  // fillers are rare: skip the scan
        pre = block_exclusive_scan(F, S.lds, tot);
    else if (vout && (carry & (kPerThread - 1)) == 0) {  // uniform
        // entry i lands at slot i + carry
        const int64_t pos = ib + carry;
        if (ib + kPerThread <= kt && pos + kPerThread <= cap && gapv[0] >= 0 &&
            gapv[1] >= 0 && gapv[2] >= 0 && gapv[3] >= 0) {
            const uint2 r = make_uint2(
                uint32_t(gapv[0] & 0xFFFF) | (uint32_t(gapv[1] & 0xFFFF) << 16),
                uint32_t(gapv[2] & 0xFFFF) | (uint32_t(gapv[3] & 0xFFFF) << 16));
            *reinterpret_cast<uint2*>(runs + pos) = r;
            *reinterpret_cast<float4*>(vals + pos) = make_float4(xv[0], xv[1], xv[2], xv[3]);
        } else {
#pragma unroll
            for (int c = 0; c < kPerThread; ++c)
                if (ib + c < kt && gapv[c] >= 0 && pos + c < cap) {
                    runs[pos + c] = uint16_t(gapv[c] & 0xFFFF);
                    vals[pos + c] = xv[c];
                }
        }
        return 0;  // no LDS touched since the barrier above
    }
    // entry i lands at slot i + carry + (fillers of entries <= i); its own
    // fillers fill the slots just before it.  sslot: slot - i0 - carry
    // (below 1024 * 65537), or kNoKey for no entry.
    uint32_t fb = pre;
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
        const int64_t i = ib + c;
        fb += nfv[c];
        const int e = int(threadIdx.x) * kPerThread + c;
        const bool ok = i < kt && gapv[c] >= 0;
        S.sslot[e] = ok ? uint32_t(e) + fb : kNoKey;
        S.sgap[e] = uint16_t(gapv[c] & 0xFFFF);
        S.sval[e] = xv[c];
        if (ok && nfv[c]) {
            int64_t pos = i + carry + fb - nfv[c];
            for (uint32_t z = 0; z < nfv[c]; ++z, ++pos)
                if (pos < cap) { runs[pos] = 65535; vals[pos] = 0.0f; }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int e = q * kBlock + int(threadIdx.x);
        if (i0 + e >= kt) break;
        if (S.sslot[e] == kNoKey) continue;
        const int64_t pos = i0 + carry + S.sslot[e];
        if (pos < cap) {
            runs[pos] = S.sgap[e];
            vals[pos] = S.sval[e];
        }
    }
    __syncthreads();  // before the next tile overwrites the stage
    return tot;
}

// The write pass over all tiles of all tensors, each at the filler offset
// k_enc_scan gave it.
__global__ __launch_bounds__(kBlock) void k_enc_write(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ idx, const float* __restrict__ val,
    const uint32_t* __restrict__ tile_foff, uint16_t* __restrict__ runs,
    float* __restrict__ vals, Scalars* __restrict__ sc, int64_t n_ktiles) {
    __shared__ EncStage S;
    int64_t tb = 0, te = 0, kt = 0, nt = 0, eb = 0, cap = 0;  // current tensor
    const uint32_t* id = idx;
    const float* vl = val;
    bool vin = false, vout = false;  // 16-byte loads of idx, val; stores of runs, vals
    int64_t c0, c1;
    tile_run(n_ktiles, c0, c1);
    for (int64_t vt = c0; vt < c1;) {
        if (vt >= te) {  // uniform: the next tensor
            const int t = int(K.kmap[vt]);
            kt = enc_len(K, kdev, t);
            nt = L.o[t + 1] - L.o[t];
            id = idx + K.koff[t];
            vl = val + K.koff[t];
            eb = L.ebase[t];
            cap = L.ebase[t + 1] - eb;
            tb = K.ktbase[t];
            te = K.ktbase[t + 1];
            vin = aligned_as(id, 16) && aligned_as(vl, 16);
            vout = aligned_as(runs + eb, 8) && aligned_as(vals + eb, 16);
        }
        const int64_t i0 = (vt - tb) * kTile;
        if (i0 >= kt) {  // uniform: nothing here or later in this tensor
            vt = te;
            continue;
        }
        enc_tile(id, vl, i0, kt, nt, int64_t(tile_foff[vt]), runs + eb, vals + eb, cap, vin,
                 vout, sc, S);
        ++vt;
    }
}

// The count, scan and write in one launch, one workgroup per tensor: its
// tiles in order, each one's fillers carried into the next.  Each of the
// three tiled passes is a launch of a few microseconds however little it
// does, so layouts whose tensors hold few tiles each take this one.
__global__ __launch_bounds__(kBlock) void k_enc_tensor(
    DevLayout L, DevK K, const int64_t* __restrict__ kdev,
    const uint32_t* __restrict__ idx, const float* __restrict__ val,
    uint16_t* __restrict__ runs, float* __restrict__ vals,
    int64_t* __restrict__ entries, Scalars* __restrict__ sc) {
    __shared__ EncStage S;
    const int t = blockIdx.x;
    const int64_t kt = enc_len(K, kdev, t);
    const int64_t nt = L.o[t + 1] - L.o[t];
    const uint32_t* id = idx + K.koff[t];
    const float* vl = val + K.koff[t];
    const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
    const bool vin = aligned_as(id, 16) && aligned_as(vl, 16);
    const bool vout = aligned_as(runs + eb, 8) && aligned_as(vals + eb, 16);
    int64_t carry = 0;
    for (int64_t i0 = 0; i0 < kt; i0 += kTile)
        carry += enc_tile(id, vl, i0, kt, nt, carry, runs + eb, vals + eb, cap, vin, vout, sc,
                          S);
    if (threadIdx.x == 0) {
        if (kdev && (kdev[t] < 0 || kdev[t] > K.k[t])) latch_error(sc, kErrCorrupt);
        entries[t] = kt + carry;
    }
}

// ---------------------------------------------------------------- decode


// (run + 1) of the thread's entries ib .. ib + 3 (0 past E).
__device__ __forceinline__ void load_run_weights(const uint16_t* __restrict__ r, int64_t ib,
                                                 int64_t E, bool vec, uint32_t (&w)[4]) {
    if (vec && ib + 4 <= E) {
        const uint2 x = *reinterpret_cast<const uint2*>(r + ib);
        w[0] = (x.x & 0xFFFFu) + 1u;
        w[1] = (x.x >> 16) + 1u;
        w[2] = (x.y & 0xFFFFu) + 1u;
        w[3] = (x.y >> 16) + 1u;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = ib + c < E ? uint32_t(r[ib + c]) + 1u : 0u;
    }
}

__device__ __forceinline__ int64_t stream_len(const int64_t* entries, int t,
                                              int64_t cap) {
    int64_t e = entries[t];
    return (e < 0 || e > cap) ? 0 : e;
}

// Values of the thread's entries ib .. ib + 3 (0 past E).
__device__ __forceinline__ void load_vals4(const float* __restrict__ v, int64_t ib, int64_t E,
                                           bool vec, float (&x)[4]) {
    if (vec && ib + 4 <= E) {
        const float4 y = *reinterpret_cast<const float4*>(v + ib);
        x[0] = y.x;
        x[1] = y.y;
        x[2] = y.z;
        x[3] = y.w;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = ib + c < E ? v[ib + c] : 0.0f;
    }
}

// A thread's 4 entries from ib as loaded: run words and values by one 8- and
// one 16-byte load from min(ib, cap - 4).  A tensor's stream capacity cap
// is a multiple of kStreamAlign entries, so the address always lies inside
// it and the loads need no branch; the words are decoded (masked past E)
// only where they are used, so loads issued for the next tile stay in
// flight until then.  Needs the runs 8-byte and the values 16-byte aligned
// and cap >= 4.
struct RawEntries {
    uint2 r;
    float4 v;
};

__device__ __forceinline__ void load_raw(const uint16_t* __restrict__ r,
                                         const float* __restrict__ v, int64_t ib, int64_t cap,
                                         RawEntries& x) {
    const int64_t ic = min(ib, cap - 4);
    x.r = *reinterpret_cast<const uint2*>(r + ic);
    x.v = *reinterpret_cast<const float4*>(v + ic);
}

// (run + 1) of the loaded entries ib .. ib + 3 (0 past E), and their values.
__device__ __forceinline__ void raw_entries(const RawEntries& x, int64_t ib, int64_t E,
                                            uint32_t (&w)[4], float (&val)[4]) {
    w[0] = (x.r.x & 0xFFFFu) + 1u;
    w[1] = (x.r.x >> 16) + 1u;
    w[2] = (x.r.y & 0xFFFFu) + 1u;
    w[3] = (x.r.y >> 16) + 1u;
    val[0] = x.v.x;
    val[1] = x.v.y;
    val[2] = x.v.z;
    val[3] = x.v.w;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (ib + c >= E) w[c] = 0u;
}

// Adds one tile of a stream, entries [i0, min(E, i0 + kTile)), into a
// tensor's part of the dense sum (nt elements).  The thread holds the
// (run + 1) weights wv and values xv of entries i0 + 4 tid .. + 3 and their
// exclusive weight prefix ex within the tile; carry = the weights of the
// stream's entries before the tile.  The adds go back to entry
// i0 + 256 q + tid through LDS, so that a wave's adds stay close together
// when the stream is dense.  Returns whether an entry of this thread lies
// at or past the tensor's end (it adds nothing).  Every thread calls it; it
// ends with a barrier.
__device__ __forceinline__ bool dec_add_tile(int64_t i0, int64_t E, int64_t carry, uint32_t ex,
                                             const uint32_t (&wv)[4], const float (&xv)[4],
                                             float* __restrict__ dense_t, int64_t nt,
                                             uint32_t* trel, float* tval) {
    // positions relative to the tile's start (< 1024 * 65536)
    uint32_t rel = ex;
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
        rel += wv[c];
        const int e = int(threadIdx.x) * kPerThread + c;
        trel[e] = rel - 1u;
        tval[e] = xv[c];
    }
    __syncthreads();
    bool bad = false;
    int64_t at[kPerThread];  // position of each add, -1 for none
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int e = q * kBlock + int(threadIdx.x);
        at[q] = -1;
        if (i0 + e < E) {
            const int64_t pos = carry + trel[e];
            if (pos >= nt) bad = true;
            else at[q] = pos;
        }
    }
    // The four dense loads go out together (a lane without an add reads
    // element 0, which a tensor with entries in range has), so a tile waits
    // for one round trip, not four.
    if (nt > 0) {  // uniform
        float d[kPerThread];
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) d[q] = dense_t[at[q] < 0 ? 0 : at[q]];
#pragma unroll
        for (int q = 0; q < kPerThread; ++q)
            if (at[q] >= 0) dense_t[at[q]] = __fadd_rn(d[q], tval[q * kBlock + int(threadIdx.x)]);
    }
    __syncthreads();  // before the next tile overwrites trel
    return bad;
}

// Merged decode.  A tensor whose learners' streams together hold at least
// n_t / 16 entries touches most cache lines of its part of the dense sum
// once per learner when each stream is added on its own.  For such a tensor
// each learner's pass only records, per kDecBlock-element block of the
// tensor, the first entry at or past the block start and that entry's
// position; one merge pass then loads each block on chip, adds the learners'
// entries in learner order (a barrier between learners, so every element
// still sees fl(fl(d + x_0) + x_1) ...) and stores the block once.
constexpr int64_t kDecBlock = 4096;
constexpr int kDecBatch = 8;  // learners merged per pass
constexpr int64_t kXcds = 8;  // XCDs of an MI355X (block order of the merge pass)
// Accumulating, a tensor is merged when its streams together hold at least
// n_t / kDecMergeAcc entries (the merged pass reads and writes every block).
// A fresh sum merges every tensor (the merged pass only writes, and the
// scattered path would have to zero the tensor first), unless the tensors
// that could hold n_t / kDecMergeFresh entries are a small part of the
// layout: then the host zeroes the sum and every tensor is scattered.
constexpr int64_t kDecMergeAcc = 16, kDecMergeFresh = 256;
// Scattered batches take one workgroup per tensor (k_dec_tensor) when no
// tensor's streams can hold more than this many tiles together.
constexpr int64_t kDecTensorTiles = 8;
// Value bytes of a batch's streams (at capacity) up to which the bounds
// passes also load the values: a quarter of MI355X's 256 MB last-level
// cache.
constexpr int64_t kDecWarmBytes = int64_t(64) << 20;
constexpr uint32_t kDecScatter = 0, kDecMerge = 1;
constexpr uint32_t kBselMerged = 0x80000000u;

// Dense-block tables: tensor t has cdiv(n_t, kDecBlock) blocks; its bounds
// are bounds[w * DB + dbase[t] + j] for j in [0, blocks_t] (the last one a
// sentinel past the tensor's end).
struct DevDec {
    const int64_t* dbase;   // [T+1] first bound of each tensor (blocks_t + 1 each)
    const int64_t* bbase;   // [T+1] first dense block of each tensor (blocks_t each)
    const uint32_t* bmap;   // [NBLK] tensor of each dense block
    uint32_t* bsel;         // [NBLK] this batch: tensor | kBselMerged if merged
    uint32_t* dmode;        // [T] kDecScatter / kDecMerge for the current batch
    uint2* bounds;          // [kDecBatch * DB] {first entry index, its position}
    int64_t DB;
};

// The streams of one batch of learners (by value).
struct DecBatch {
    const uint16_t* runs[kDecBatch];
    const float* vals[kDecBatch];
    const int64_t* entries[kDecBatch];
    int W;
};

// One thread per dense block: the mode of the block's tensor for this
// batch (merged or scattered; force: 0 automatic, 1 always scattered, 2
// always merged).  The thread of a tensor's first block writes dmode[t] for
// the write passes; every thread writes bsel[blk] for the merge pass, which
// then finds its block's tensor in a line this pass has just written (the
// block map itself would be a miss to HBM at the head of every merge
// workgroup's chain: 1.06 against 0.93 ms for a fresh 2^30-element sum).
__global__ __launch_bounds__(kBlock) void k_dec_mode(DevLayout L, DecBatch S, DevDec Dd,
                                                     int force, int64_t n_blocks) {
    const int64_t blk = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (blk >= n_blocks) return;
    const int t = int(Dd.bmap[blk]);
    const int64_t nt = L.o[t + 1] - L.o[t];
    const int64_t cap = L.ebase[t + 1] - L.ebase[t];
    int64_t sum = 0;
    for (int w = 0; w < S.W; ++w) sum += stream_len(S.entries[w], t, cap);
    uint32_t mode = (kDecMergeAcc * sum >= nt) ? kDecMerge : kDecScatter;
    if (force == 1) mode = kDecScatter;
    if (force == 2) mode = kDecMerge;
    if (blk == Dd.bbase[t]) Dd.dmode[t] = mode;
    Dd.bsel[blk] = uint32_t(t) | (mode == kDecMerge ? kBselMerged : 0u);
}

// Per capacity tile of one learner's stream: sum of (run + 1).  Flags an
// entry count outside [0, capacity].
__global__ __launch_bounds__(kBlock) void k_dec_count(
    DevLayout L, const uint16_t* __restrict__ runs,
    const int64_t* __restrict__ entries, uint32_t* __restrict__ tile_s,
    Scalars* __restrict__ sc, int64_t n_etiles) {
    __shared__ uint32_t lds[kWavesPerBlock];
    int64_t tb = 0, te = 0, eb = 0, E = 0;  // current tensor: tiles [tb, te)
    int64_t c0, c1;
    tile_run(n_etiles, c0, c1);
    for (int64_t vt = c0; vt < c1;) {
        if (vt >= te) {  // uniform: the next tensor
            const int t = int(L.emap[vt]);
            eb = L.ebase[t];
            const int64_t cap = L.ebase[t + 1] - eb;
            tb = L.etbase[t];
            te = L.etbase[t + 1];
            const int64_t e = entries[t];
            if (vt == tb && threadIdx.x == 0 && (e < 0 || e > cap))
                latch_error(sc, kErrCorrupt);
            E = (e < 0 || e > cap) ? 0 : e;
        }
        const int64_t i0 = (vt - tb) * kTile;
        if (i0 >= E) {  // uniform: nothing here or later in this tensor
            vt = te;
            continue;
        }
        // thread-consecutive entries, as in k_dec_write
        const int64_t ib = i0 + int64_t(threadIdx.x) * kPerThread;
        uint32_t w[kPerThread];
        load_run_weights(runs + eb, ib, E, aligned_as(runs + eb, 8), w);
        const uint32_t s = w[0] + w[1] + w[2] + w[3];
        uint32_t tot;
        block_exclusive_scan(s, lds, tot);
        if (threadIdx.x == 0) tile_s[vt] = tot;
        ++vt;
    }
}

// One block per tensor: 64-bit exclusive scan of the sums of the tiles
// that hold entries (k_dec_count skips the rest).
template <bool kStaged>
__global__ __launch_bounds__(kBlock) void k_dec_scan(
    DevLayout L, const int64_t* __restrict__ entries, const uint32_t* __restrict__ tile_s,
    uint64_t* __restrict__ tile_p) {
    __shared__ uint64_t lds[kWavesPerBlock];
    __shared__ uint32_t stage[kStaged ? kScanStage : 1];
    const int t = blockIdx.x;
    const int64_t tb = L.etbase[t], cap = L.ebase[t + 1] - L.ebase[t];
    const int64_t ntile = (stream_len(entries, t, cap) + kTile - 1) / kTile;
    block_scan_range<uint64_t, kStaged>(tile_s + tb, tile_p + tb, ntile, uint64_t(0), lds,
                                        stage);
}

// dense[o_t + pos] += value for every entry of one learner's stream, where
// pos = (sum of run + 1 over the entries up to this one) - 1.  Entries whose
// position reaches the tensor's end add nothing and flag the stream as
// corrupt (positions only grow, so every later entry is past the end too).
// For a tensor in merged mode (merge_on and dmode[t] == kDecMerge) the
// entries are not added here: each records, for every dense block whose
// first entry it is (previous position < block start <= its position), its
// index and position in the learner's bound row (slot); the last entry also
// fills the blocks after it with {E, 0}.
__global__ __launch_bounds__(kBlock) void k_dec_write(
    DevLayout L, const uint16_t* __restrict__ runs,
    const float* __restrict__ vals, const int64_t* __restrict__ entries,
    const uint64_t* __restrict__ tile_p, float* __restrict__ dense,
    Scalars* __restrict__ sc, int64_t n_etiles, int merge_on, DevDec Dd, int slot,
    int warm) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t trel[kTile];
    __shared__ float tval[kTile];
    // current tensor: tiles [tb, te)
    int64_t tb = 0, te = 0, eb = 0, o = 0, nt = 0, E = 0, nb = 0;
    bool merged = false;
    uint2* bnd = nullptr;
    int64_t c0, c1;
    tile_run(n_etiles, c0, c1);
    for (int64_t vt = c0; vt < c1;) {
        if (vt >= te) {  // uniform: the next tensor
            const int t = int(L.emap[vt]);
            eb = L.ebase[t];
            const int64_t cap = L.ebase[t + 1] - eb;
            o = L.o[t];
            nt = L.o[t + 1] - o;
            E = stream_len(entries, t, cap);
            tb = L.etbase[t];
            te = L.etbase[t + 1];
            merged = merge_on && Dd.dmode[t] == kDecMerge;
            nb = (nt + kDecBlock - 1) / kDecBlock;  // sentinel index
            bnd = merged ? Dd.bounds + int64_t(slot) * Dd.DB + Dd.dbase[t] : nullptr;
        }
        const int64_t i0 = (vt - tb) * kTile;
        if (i0 >= E) {  // uniform: nothing here or later in this tensor
            vt = te;
            continue;
        }
        // Each thread takes kPerThread consecutive entries of the tile: one
        // load round and one block scan per tile give every entry its
        // position (the thread's running sum after the scan).
        bool bad = false;
        const int64_t ib = i0 + int64_t(threadIdx.x) * kPerThread;
        uint32_t wv[kPerThread];
        float xv[kPerThread] = {0.0f, 0.0f, 0.0f, 0.0f};
        load_run_weights(runs + eb, ib, E, aligned_as(runs + eb, 8), wv);
        // With warm set the values are loaded on the merged path too, where
        // they are not added here: the merge pass reads them next and then
        // finds them in cache instead of waiting on HBM at the end of its
        // chain of loads (fresh 2^30-element sum of 4 sparse learners: 0.93
        // -> 0.81 ms).  The host sets it only when the batch's values fit
        // well inside the last-level cache; larger ones would only be read
        // twice.
        if (!merged || warm) {  // uniform
            load_vals4(vals + eb, ib, E, aligned_as(vals + eb, 16), xv);
            if (merged)  // keep the loads: their values are not used on this path
                asm volatile("" ::"v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]));
        }
        const uint32_t s = wv[0] + wv[1] + wv[2] + wv[3];
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(s, lds, tot);
        const int64_t carry = int64_t(tile_p[vt]);
        if (!merged) {  // uniform
            if (dec_add_tile(i0, E, carry, ex, wv, xv, dense + o, nt, trel, tval))
                latch_error(sc, kErrCorrupt);
            ++vt;
            continue;
        }
        int64_t run = carry + ex;  // entries' (run + 1) before this one
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const int64_t i = ib + c;
            if (i >= E) break;
            run += wv[c];
            const int64_t pos = run - 1;
            if (pos >= nt) bad = true;
            {
                const int64_t prev = pos - int64_t(wv[c]);  // -1 for the first entry
                const int64_t b0 = prev < 0 ? 0 : prev / kDecBlock + 1;
                const int64_t b1 = min(pos / kDecBlock, nb);
                for (int64_t b = b0; b <= b1; ++b)
                    bnd[b] = make_uint2(uint32_t(i), uint32_t(min(pos, nt)));
                if (i == E - 1)
                    for (int64_t b = max(b0, b1 + 1); b <= nb; ++b)
                        bnd[b] = make_uint2(uint32_t(E), 0u);
            }
        }
        if (bad) latch_error(sc, kErrCorrupt);
        ++vt;
    }
}

// The scattered decode of a batch of learners in one launch, one workgroup
// per tensor: the learners in order (each tile ends with a barrier, so an
// element sees fl(fl(d + x_0) + x_1) ...), each stream's tiles in order with
// the position carried from tile to tile; an entry count outside
// [0, capacity] or a position past the tensor's end is flagged as in the
// tiled passes.  Each of k_dec_count, k_dec_scan and k_dec_write is a
// launch of a few microseconds however little it does, so layouts whose
// streams hold few tiles per tensor take this one.
__global__ __launch_bounds__(kBlock) void k_dec_tensor(DevLayout L, DecBatch S,
                                                       float* __restrict__ dense,
                                                       Scalars* __restrict__ sc) {
    __shared__ uint32_t lds[kWavesPerBlock];
    __shared__ uint32_t trel[kTile];
    __shared__ float tval[kTile];
    const int t = blockIdx.x;
    const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    bool bad = false;
    for (int w = 0; w < S.W; ++w) {
        const int64_t e = S.entries[w][t];
        bad |= e < 0 || e > cap;
        const int64_t E = (e < 0 || e > cap) ? 0 : e;
        const uint16_t* r = S.runs[w] + eb;
        const float* v = S.vals[w] + eb;
        const bool rvec = aligned_as(r, 8), vvec = aligned_as(v, 16);
        // With aligned streams the next tile's entries are loaded before
        // this tile's adds read their dense lines: the two return together,
        // so each tile after the first waits for one round trip, not two.
        const bool pre = rvec && vvec && E > 0;  // uniform
        int64_t carry = 0;
        // scan and add one tile whose entries the thread holds
        auto add = [&](int64_t i0, const uint32_t (&wv)[kPerThread],
                       const float (&xv)[kPerThread]) {
            uint32_t tot;
            const uint32_t ex = block_exclusive_scan(wv[0] + wv[1] + wv[2] + wv[3], lds, tot);
            bad |= dec_add_tile(i0, E, carry, ex, wv, xv, dense + o, nt, trel, tval);
            carry += tot;
        };
        if (pre) {
            // separate loops: a branch inside one would merge the next
            // tile's registers there and wait for its loads
            RawEntries cur;
            load_raw(r, v, int64_t(threadIdx.x) * kPerThread, cap, cur);
            for (int64_t i0 = 0; i0 < E; i0 += kTile) {
                const int64_t ib = i0 + int64_t(threadIdx.x) * kPerThread;
                // issued on every iteration (the last one repeats this
                // tile's address), so that this tile's words are one load
                // round behind it and their wait need not drain it
                RawEntries nxt;
                load_raw(r, v, i0 + kTile < E ? ib + kTile : ib, cap, nxt);
                __builtin_amdgcn_sched_barrier(0);
                uint32_t wv[kPerThread];
                float xv[kPerThread];
                raw_entries(cur, ib, E, wv, xv);
                add(i0, wv, xv);
                cur = nxt;
            }
        } else {
            for (int64_t i0 = 0; i0 < E; i0 += kTile) {
                const int64_t ib = i0 + int64_t(threadIdx.x) * kPerThread;
                uint32_t wv[kPerThread];
                float xv[kPerThread];
                load_run_weights(r, ib, E, rvec, wv);
                load_vals4(v, ib, E, vvec, xv);
                add(i0, wv, xv);
            }
        }
    }
    if (bad) latch_error(sc, kErrCorrupt);
}

typedef float dec_f4 __attribute__((ext_vector_type(4)));

// A fresh sum whose tensors are all scattered: dense[0, n) = +0.0 first.
// 16-byte stores from the first 16-byte boundary on, kDecBlock / 4 of them
// per workgroup; workgroup 0 also writes the head and the tail.  Plain
// stores, one workgroup per 16 KB: on MI355X that fills at about 6 TB/s,
// against 5 TB/s for a resident grid-stride loop and a few percent less
// with nontemporal stores.
__global__ __launch_bounds__(kBlock) void k_dec_fill(float* __restrict__ dense, int64_t n) {
    const int64_t head =
        min(n, int64_t((16 - (reinterpret_cast<uintptr_t>(dense) & 15)) & 15) / 4);
    const int64_t nv = (n - head) / 4;
    float4* v = reinterpret_cast<float4*>(dense + head);
    const uint32_t tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < int(kDecBlock / kBlock) / 4; ++q) {
        const int64_t i = int64_t(blockIdx.x) * (kDecBlock / 4) + q * kBlock + tid;
        if (i < nv) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (blockIdx.x == 0) {
        const int64_t tail = head + 4 * nv;
        if (tid < head) dense[tid] = 0.0f;
        if (tid < n - tail) dense[tail + tid] = 0.0f;
    }
}

// Merge pass: one workgroup per dense block of a merged tensor.  The block
// is loaded into LDS, each learner's entries inside it are added in learner
// order, and the block is stored once.  Positions are rebuilt from the
// recorded first position and the runs.  Blocks no learner touches are left
// alone.  With fresh set the block starts at +0.0 instead of being loaded (a
// new sum: fl(+0 + x_0) ...), and a block no learner touches is stored as
// zeros.
//
// The workgroup's loads are issued in three dependent rounds: the block's
// tensor; everything that depends on the tensor alone (layout, mode, entry
// counts, every learner's bounds); then every learner's first kBlock entries
// together with the block.  When no learner has more than kWave entries in
// the block, wave 0 holds them all after that round and adds them learner
// by learner: within one wave the LDS updates of learner w complete before
// those of learner w + 1, so no barrier separates the learners.
//
// Workgroup g runs on XCD g mod kXcds (MI355X dispatches workgroups to its
// eight XCDs round robin), and each XCD walks one contiguous range of
// blocks: neighbouring blocks share the cache lines of the block map, the
// bounds and the entries, and those lines then stay in one XCD's L2.  Whole
// aligned blocks are stored with nontemporal 16-byte stores: on MI355X that
// took a fresh 2^30-element sum from 1.28 to 0.99 ms against plain stores
// (a pure fill is the other way round, see k_dec_fill).
__global__ __launch_bounds__(kBlock) void k_dec_merge(
    DevLayout L, DecBatch S, DevDec Dd, float* __restrict__ dense, int64_t n_blocks,
    int fresh) {
    __shared__ __attribute__((aligned(16))) float tile[kDecBlock];
    __shared__ uint32_t lds[kWavesPerBlock];
    const int64_t per = (n_blocks + kXcds - 1) / kXcds;  // grid: kXcds * per
    const int64_t blk = int64_t(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (blk >= n_blocks) return;
    const uint32_t tid = threadIdx.x;
    // first loads: the block's tensor and mode (written by k_dec_mode)
    const uint32_t bs = Dd.bsel[blk];
    if (!(bs & kBselMerged)) return;  // uniform
    const int t = int(bs & ~kBselMerged);
    // second loads: all of them depend on t only
    const int64_t o = L.o[t], nt = L.o[t + 1] - o;
    const int64_t eb = L.ebase[t], cap = L.ebase[t + 1] - eb;
    const int64_t j = blk - Dd.bbase[t];
    const int64_t gb = Dd.dbase[t] + j;
    int64_t ent[kDecBatch];
    uint2 ba[kDecBatch], bb[kDecBatch];
#pragma unroll
    for (int w = 0; w < kDecBatch; ++w) {
        ent[w] = 0;
        ba[w] = bb[w] = make_uint2(0u, 0u);
        if (w < S.W) {  // uniform
            ent[w] = S.entries[w][t];
            const uint2* bnd = Dd.bounds + int64_t(w) * Dd.DB + gb;
            ba[w] = bnd[0];
            bb[w] = bnd[1];
        }
    }
    const int64_t lo_pos = j * kDecBlock;
    const int64_t len = min(kDecBlock, nt - lo_pos);
    uint32_t lo[kDecBatch], hi[kDecBatch], p0[kDecBatch];
    bool any = false, small = true;
#pragma unroll
    for (int w = 0; w < kDecBatch; ++w) {
        lo[w] = hi[w] = p0[w] = 0;
        if (w < S.W && ent[w] > 0 && ent[w] <= cap) {  // bounds hold this stream
            lo[w] = ba[w].x;
            p0[w] = ba[w].y;
            hi[w] = max(ba[w].x, bb[w].x);
            any = any || hi[w] > lo[w];
            small = small && hi[w] - lo[w] <= uint32_t(kWave);
        }
    }
    if (!any && !fresh) return;  // uniform
    // third loads: every learner's first kBlock entries, and the block
    uint32_t r0[kDecBatch];
    float x0[kDecBatch];
#pragma unroll
    for (int w = 0; w < kDecBatch; ++w) {
        const uint32_t i = lo[w] + tid;
        r0[w] = 0;
        x0[w] = 0.0f;
        if (i < hi[w]) {
            r0[w] = S.runs[w][eb + i];
            x0[w] = S.vals[w][eb + i];
        }
    }
    float* d = dense + o + lo_pos;
    const bool vec = len == kDecBlock && aligned_as(d, 16);  // uniform
    constexpr int kQ = int(kDecBlock / kBlock);       // values per thread
    float reg[kQ];
    if (vec) {
        // thread tid holds elements 4 (q kBlock + tid) + c, q < kQ / 4
#pragma unroll
        for (int q = 0; q < kQ / 4; ++q) {
            const int64_t e = 4 * (int64_t(q) * kBlock + tid);
            float4 x = fresh ? make_float4(0.f, 0.f, 0.f, 0.f)
                             : *reinterpret_cast<const float4*>(d + e);
            reg[4 * q] = x.x;
            reg[4 * q + 1] = x.y;
            reg[4 * q + 2] = x.z;
            reg[4 * q + 3] = x.w;
        }
#pragma unroll
        for (int q = 0; q < kQ / 4; ++q)
            *reinterpret_cast<float4*>(tile + 4 * (q * kBlock + tid)) =
                make_float4(reg[4 * q], reg[4 * q + 1], reg[4 * q + 2], reg[4 * q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int64_t e = int64_t(q) * kBlock + tid;
            reg[q] = (e < len && !fresh) ? d[e] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q) tile[q * kBlock + tid] = reg[q];
    }
    __syncthreads();
    if (small) {  // uniform: wave 0 holds every entry of the block
        if (tid < uint32_t(kWave)) {
#pragma unroll
            for (int w = 0; w < kDecBatch; ++w) {
                if (hi[w] <= lo[w]) continue;  // uniform
                const bool in = tid < hi[w] - lo[w];
                const uint32_t wt = (in && tid > 0) ? r0[w] + 1u : 0u;
                const int64_t at = int64_t(p0[w]) + wave_inclusive_scan(wt) - lo_pos;
                if (in && at >= 0 && at < len) tile[at] = __fadd_rn(tile[at], x0[w]);
            }
        }
    } else {
#pragma unroll
        for (int w = 0; w < kDecBatch; ++w) {
            if (hi[w] <= lo[w]) continue;  // uniform
            const uint16_t* rr = S.runs[w] + eb;
            const float* vv = S.vals[w] + eb;
            int64_t carry = int64_t(p0[w]);
            for (uint32_t base = lo[w]; base < hi[w]; base += kBlock) {
                const uint32_t i = base + tid;
                uint32_t run = r0[w];
                float x = x0[w];
                if (base != lo[w] && i < hi[w]) {
                    run = rr[i];
                    x = vv[i];
                }
                const uint32_t wt = (i < hi[w] && i > lo[w]) ? run + 1u : 0u;
                uint32_t tot;
                const uint32_t ex = block_exclusive_scan(wt, lds, tot);
                if (i < hi[w]) {
                    const int64_t at = carry + ex + wt - lo_pos;
                    if (at >= 0 && at < len) tile[at] = __fadd_rn(tile[at], x);
                }
                carry += tot;
            }
            __syncthreads();
        }
    }
    __syncthreads();
    if (vec) {
#pragma unroll
        for (int q = 0; q < kQ / 4; ++q) {
            const int64_t e = 4 * (int64_t(q) * kBlock + tid);
            const float4 x = *reinterpret_cast<const float4*>(tile + e);
            const dec_f4 y = {x.x, x.y, x.z, x.w};
            __builtin_nontemporal_store(y, reinterpret_cast<dec_f4*>(d + e));
        }
    } else {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int64_t e = int64_t(q) * kBlock + tid;
            if (e < len) d[e] = tile[e];
        }
    }
}

}  // namespace dgc
