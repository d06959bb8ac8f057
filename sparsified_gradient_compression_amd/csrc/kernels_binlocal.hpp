// kernels_binlocal.hpp -- the bin-local selector on gfx950, and the
// element-wise pass and placement it shares with the sampled threshold
// (kernels_sampled.hpp).
//
// Source: the AdaComp page ("AdaComp : Adaptive Residual Gradient Compression
// for Data-Parallel Distributed Training"), Abstract (residues are selected
// locally; the rate follows local activity) and "Citations in the corpus"
// (each layer's residual vector is cut into fixed-size bins; a bin's largest
// absolute value is its threshold).  What meets the threshold is not stated;
// the rule here: in bin b of L entries (restarting at each tensor),
//   theta_b = max key(v_j),  entry i is salient iff key(v_i) != 0 and
//   key(fl32(v_i + u_i)) >= theta_b,
// with v and u after this step's momentum correction and accumulation, and
// key(x) = bits(x) & 0x7FFFFFFF.  Clip, momentum and masking are DGC's.  At
// most cap_t salient entries are delivered per tensor, first in index order;
// only delivered entries are masked.
//
// Pieces here are a whole number of bins (L * floor(1024 / L) elements), so
// every threshold is known inside the wave that owns the piece:
//   k_bl_fused   momentum update, per-bin maxima in the wave's LDS, salient
//                flags, ranks by ballot; the piece's entries {index, v, u}
//                go to its own slots and u, v are masked in registers.  A
//                piece with more entries than slots keeps u, v unmasked.
//   k_bl_group   per 1024-piece group: exclusive prefix of piece counts.
//   k_bl_tscan   per tensor: group offsets, delivered and salient counts.
//   k_bl_gather  64 pieces per wave: slots -> (idx, val) at their final
//                positions; entries past the tensor's capacity get their u
//                and v back from the slot (as if never masked); a piece that
//                overflowed its slots is re-derived from u and v (same
//                arithmetic, same flags) and its delivered entries masked.
#pragma once

#include "dgc_device.hpp"
#include "kernel_fused.hpp"

namespace dgc {

constexpr int64_t kBlGroup = 1024;  // pieces per prefix group
constexpr int64_t kMaxBin = kPiece;  // largest bin length

// Selection rule of the pass: per-bin maxima (bin-local, AdaComp), or one
// threshold per tensor taken from TensorState::lo_key (the sampled
// threshold of kernels_sampled.hpp): key >= theta and key != 0.
constexpr int kSelBins = 0;
constexpr int kSelThresh = 1;

// Bin-local tables (device pointers into the workspace), passed by value.
struct DevBins {
    const int64_t* plen;   // [T] piece length, a whole number of bins
    const int64_t* magic;  // [T] ceil(2^32 / L) (0 when L = 1)
    const int64_t* pbase;  // [T+1] first piece of each tensor
    const int64_t* gbase;  // [T+1] first prefix group of each tensor
    const int64_t* pcap;   // [T] slots per piece
    const int64_t* slbase; // [T] first slot of each tensor (12-byte slots)
    const int64_t* rbins;  // [T] rounds per bin when L is 256, 512 or 1024, else 0
    PieceDesc* pdesc;      // [pieces]
    uint32_t* cnt;         // [pieces] salient entries of each piece
    uint32_t* pre;         // [pieces] exclusive prefix inside its group
    uint32_t* gsum;        // [groups] salient entries of each group
    uint32_t* goff;        // [groups] exclusive prefix inside its tensor
};

// Bin of the element e elements after a piece start (e < 1024): e / L by a
// multiply-high, exact for e < 2^22 / L.
__device__ __forceinline__ uint32_t bl_bin(uint32_t e, uint32_t magic) {
    return magic ? __umulhi(e, magic) : e;
}

// LDS written by some lanes of a wave and read by others, with no other
// wave involved: a wave's LDS operations complete in order, so a compiler
// fence at wavefront scope suffices.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Offset from the piece start of a lane's element (i, c): float4 units
// (64 lanes x 4) when the start is 16-byte aligned, else 64 consecutive
// elements per (i, c).  Both orders rank in index order below.
template <bool kAligned>
__device__ __forceinline__ uint32_t bl_off(int i, int c, int lane) {
    return kAligned ? uint32_t(((i * kWave + lane) << 2) + c)
                    : uint32_t((i * 4 + c) * kWave + lane);
}

// Salient flags of one piece of len elements.  vn / un hold v and u after
// the update (anything for elements past len).  th is this wave's 1024-entry
// LDS row.  rb > 0 (aligned pieces of bins of 256, 512 or 1024 elements):
// every bin is rb whole rounds of the float4 layout, so the bin maxima are
// wave reductions of the rounds and no LDS is used.
template <bool kAligned>
__device__ __forceinline__ void bl_flags(const float (&vn)[kRounds][4],
                                         const float (&un)[kRounds][4],
                                         uint32_t len, uint32_t magic, uint32_t rb,
                                         uint32_t* th, bool (&f)[kRounds][4]) {
    const int lane = lane_id();
    if (kAligned && rb) {  // uniform
        uint32_t rmax[kRounds];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            uint32_t m = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (bl_off<true>(i, c, lane) < len) m = max(m, mag_key(vn[i][c]));
#pragma unroll
            for (int d = kWave / 2; d >= 1; d >>= 1)
                m = max(m, uint32_t(__shfl_xor(int(m), d, kWave)));
            rmax[i] = m;
        }
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            const int b0 = i / int(rb) * int(rb);
            uint32_t theta = 0;
#pragma unroll
            for (int j = 0; j < kRounds; ++j)
                if (j >= b0 && j < b0 + int(rb)) theta = max(theta, rmax[j]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = mag_key(vn[i][c]);
                const uint32_t ahead = mag_key(__fadd_rn(vn[i][c], un[i][c]));
                f[i][c] = bl_off<true>(i, c, lane) < len && key != 0u && ahead >= theta;
            }
        }
        return;
    }
    uint4* th4 = reinterpret_cast<uint4*>(th);
    wave_lds_sync();  // after any reads of the row for a previous piece
#pragma unroll
    for (int q = 0; q < int(kPiece / (4 * kWave)); ++q)
        th4[q * kWave + lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
    // per-bin maxima: runs of one bin inside a lane's four elements are
    // folded first; a round that lies in one bin is folded across the wave
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        if (kAligned) {
            const uint32_t r0 = uint32_t(i * kWave * 4);
            const bool one_bin = bl_bin(r0, magic) == bl_bin(r0 + kWave * 4 - 1, magic);
            uint32_t rb = bl_bin(bl_off<true>(i, 0, lane), magic);
            uint32_t rk = bl_off<true>(i, 0, lane) < len ? mag_key(vn[i][0]) : 0u;
#pragma unroll
            for (int c = 1; c < 4; ++c) {
                const uint32_t e = bl_off<true>(i, c, lane);
                const uint32_t b = bl_bin(e, magic);
                const uint32_t k = e < len ? mag_key(vn[i][c]) : 0u;
                if (b != rb) {
                    if (rk) atomicMax(&th[rb], rk);
                    rb = b;
                    rk = k;
                } else {
                    rk = max(rk, k);
                }
            }
            if (one_bin) {
#pragma unroll
                for (int d = kWave / 2; d >= 1; d >>= 1)
                    rk = max(rk, uint32_t(__shfl_xor(int(rk), d, kWave)));
                if (lane == 0 && rk) atomicMax(&th[rb], rk);
            } else if (rk) {
                atomicMax(&th[rb], rk);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t e = bl_off<false>(i, c, lane);
                const uint32_t k = e < len ? mag_key(vn[i][c]) : 0u;
                if (k) atomicMax(&th[bl_bin(e, magic)], k);
            }
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t e = bl_off<kAligned>(i, c, lane);
            const uint32_t key = mag_key(vn[i][c]);
            const uint32_t ahead = mag_key(__fadd_rn(vn[i][c], un[i][c]));
            f[i][c] = e < len && key != 0u && ahead >= th[bl_bin(e, magic)];
        }
}

template <bool kAligned, int kSel>
__device__ __forceinline__ void sel_flags(const float (&vn)[kRounds][4],
                                          const float (&un)[kRounds][4],
                                          uint32_t len, uint32_t magic, uint32_t rb,
                                          uint32_t theta, uint32_t* th,
                                          bool (&f)[kRounds][4]) {
    if constexpr (kSel == kSelBins) {
        bl_flags<kAligned>(vn, un, len, magic, rb, th, f);
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int i = 0; i < kRounds; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = mag_key(vn[i][c]);
                f[i][c] = bl_off<kAligned>(i, c, lane) < len && key != 0u && key >= theta;
            }
    }
}

// Ranks of the flagged elements in index order, and their number.
template <bool kAligned>
__device__ __forceinline__ uint32_t bl_ranks(const bool (&f)[kRounds][4],
                                             uint32_t (&rank)[kRounds][4]) {
    const uint64_t lt = lanemask_lt();
    uint32_t total = 0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        uint64_t b[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = __ballot(f[i][c]);
        if (kAligned) {
            uint32_t before = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) before += __popcll(b[c] & lt);
            uint32_t own = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rank[i][c] = total + before + own;
                own += f[i][c];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) total += __popcll(b[c]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rank[i][c] = total + __popcll(b[c] & lt);
                total += __popcll(b[c]);
            }
        }
    }
    return total;
}

template <bool kAligned, int kSel>
__device__ __forceinline__ void bl_fused_piece(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    int64_t e0, uint32_t len, int t, const DevLayout& L, const DevBins& B,
    const TensorState* __restrict__ ts, float s, float m, uint32_t pcap_limit,
    CandSlot* __restrict__ slots, int64_t p, uint32_t* th) {
    const int lane = lane_id();
    const int64_t e1 = e0 + len;
    float un[kRounds][4], vn[kRounds][4];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        float gg[4] = {0, 0, 0, 0}, uu[4] = {0, 0, 0, 0}, vv[4] = {0, 0, 0, 0};
        if (kAligned) {
            const int64_t el = e0 + bl_off<true>(i, 0, lane);
            if (el + 4 <= e1) {
                const float4 a = ld_stream(g + el), b = ld_stream(u + el),
                             c = ld_stream(v + el);
                gg[0] = a.x; gg[1] = a.y; gg[2] = a.z; gg[3] = a.w;
                uu[0] = b.x; uu[1] = b.y; uu[2] = b.z; uu[3] = b.w;
                vv[0] = c.x; vv[1] = c.y; vv[2] = c.z; vv[3] = c.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (el + c < e1) { gg[c] = g[el + c]; uu[c] = u[el + c]; vv[c] = v[el + c]; }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t el = e0 + bl_off<false>(i, c, lane);
                if (el < e1) { gg[c] = g[el]; uu[c] = u[el]; vv[c] = v[el]; }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            momentum_update(gg[c], s, m, uu[c], vv[c]);
            un[i][c] = uu[c];
            vn[i][c] = vv[c];
        }
    }
    const uint32_t magic = uint32_t(B.magic[t]);
    const uint32_t rb = kSel == kSelBins ? uint32_t(B.rbins[t]) : 0u;
    const uint32_t theta = kSel == kSelThresh ? ts[t].lo_key : 0u;
    const int64_t o = L.o[t];
    const uint32_t pcap = min(uint32_t(B.pcap[t]), pcap_limit);
    bool f[kRounds][4];
    uint32_t rank[kRounds][4];
    sel_flags<kAligned, kSel>(vn, un, len, magic, rb, theta, th, f);
    const uint32_t total = bl_ranks<kAligned>(f, rank);
    // the slots keep u and v as they were, so masking here can be undone
    const bool early = total <= pcap;
    if (lane == 0) B.cnt[p] = total;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        float uu[4], vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool z = early && f[i][c];
            uu[c] = z ? 0.0f : un[i][c];
            vv[c] = z ? 0.0f : vn[i][c];
        }
        if (kAligned) {
            const int64_t el = e0 + bl_off<true>(i, 0, lane);
            if (el + 4 <= e1) {
                st_stream(u + el, uu[0], uu[1], uu[2], uu[3]);
                st_stream(v + el, vv[0], vv[1], vv[2], vv[3]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (el + c < e1) { u[el + c] = uu[c]; v[el + c] = vv[c]; }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t el = e0 + bl_off<false>(i, c, lane);
                if (el < e1) { u[el] = uu[c]; v[el] = vv[c]; }
            }
        }
    }
    if (total && early) {
        CandSlot* sl = slots + B.slbase[t] + (p - B.pbase[t]) * int64_t(pcap);
#pragma unroll
        for (int i = 0; i < kRounds; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (f[i][c])
                    sl[rank[i][c]] = CandSlot{uint32_t(e0 - o) + bl_off<kAligned>(i, c, lane),
                                              vn[i][c], un[i][c]};
    }
}

// LDS rows of the per-bin maxima (none for the threshold rule).
template <int kSel>
struct SelLds {
    static constexpr int kRows = kSel == kSelBins ? kWavesPerBlock : 1;
    static constexpr int kLen = kSel == kSelBins ? int(kMaxBin) : 4;
};

// Element-wise pass, one wave per piece.  With clipping off block 0 also
// writes the call's scalar outputs (norm -1, scale 1).  pcap_limit = 0
// sends every piece through the re-derivation in k_bl_gather (a test hook).
template <int kSel>
__global__ __launch_bounds__(kBlock) void k_bl_fused(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    DevLayout L, DevBins B, const TensorState* __restrict__ ts,
    Scalars* __restrict__ sc, int clip_on, float m,
    uint32_t pcap_limit, CandSlot* __restrict__ slots, int64_t n_pieces,
    double* __restrict__ out_norm, float* __restrict__ out_scale) {
    __shared__ __align__(16) uint32_t th[SelLds<kSel>::kRows][SelLds<kSel>::kLen];
    const float s = clip_on ? sc->scale : 1.0f;
    if (!clip_on && blockIdx.x == 0 && threadIdx.x == 0) {
        sc->norm = -1.0;
        sc->scale = 1.0f;
        if (out_norm) *out_norm = -1.0;
        if (out_scale) *out_scale = 1.0f;
    }
    const int64_t p = (int64_t(blockIdx.x) * kBlock + threadIdx.x) >> 6;
    if (p >= n_pieces) return;  // no block-wide barrier follows
    const PieceDesc d = B.pdesc[p];
    const int t = wave_uniform(int(d.tensor));
    uint32_t* row = th[kSel == kSelBins ? (threadIdx.x >> 6) : 0];
    if ((d.start & 3) == 0)
        bl_fused_piece<true, kSel>(g, u, v, d.start, d.len, t, L, B, ts, s, m, pcap_limit,
                                   slots, p, row);
    else
        bl_fused_piece<false, kSel>(g, u, v, d.start, d.len, t, L, B, ts, s, m, pcap_limit,
                                    slots, p, row);
}

// Piece descriptors for the current bin lengths, one thread per piece.
__global__ __launch_bounds__(kBlock) void k_bl_pdesc(DevLayout L, DevBins B,
                                                     int64_t n_pieces) {
    const int64_t p = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (p >= n_pieces) return;
    const int t = find_seg(B.pbase, L.T, p);
    const int64_t pl = B.plen[t];
    const int64_t off = (p - B.pbase[t]) * pl;
    const int64_t nt = L.o[t + 1] - L.o[t];
    PieceDesc d;
    d.start = L.o[t] + off;
    d.tensor = uint32_t(t);
    d.len = uint32_t(min(pl, nt - off));
    B.pdesc[p] = d;
}

// One wave per group of kBlGroup pieces of one tensor: exclusive prefix of
// the piece counts inside the group, and the group's total.
__global__ __launch_bounds__(kBlock) void k_bl_group(DevLayout L, DevBins B,
                                                     int64_t n_groups) {
    const int64_t gi = (int64_t(blockIdx.x) * kBlock + threadIdx.x) >> 6;
    if (gi >= n_groups) return;
    const int lane = lane_id();
    const int t = find_seg(B.gbase, L.T, gi);
    const int64_t p0 = B.pbase[t] + (gi - B.gbase[t]) * kBlGroup;
    const int64_t p1 = min(B.pbase[t + 1], p0 + kBlGroup);
    constexpr int kPer = int(kBlGroup / kWave);
    uint32_t c[kPer];
    uint32_t local = 0;
    const int64_t q0 = p0 + int64_t(lane) * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        c[j] = q0 + j < p1 ? B.cnt[q0 + j] : 0u;
        local += c[j];
    }
    const uint32_t inc = wave_inclusive_scan(local);
    uint32_t run = inc - local;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (q0 + j < p1) B.pre[q0 + j] = run;
        run += c[j];
    }
    if (lane == kWave - 1) B.gsum[gi] = inc;
}

// One block per tensor: group offsets, then count = min(total, cap) and
// total (salient entries, delivered or not).
__global__ __launch_bounds__(kBlock) void k_bl_tscan(DevK K, DevBins B,
                                                     int64_t* __restrict__ out_count,
                                                     int64_t* __restrict__ out_total) {
    __shared__ uint32_t lds[kWavesPerBlock];
    const int t = blockIdx.x;
    const int64_t gb = B.gbase[t], ng = B.gbase[t + 1] - gb;
    // a tensor has at most ceil(n / 513 / 1024) groups: short scans
    const uint32_t total = block_scan_range<uint32_t, false>(B.gsum + gb, B.goff + gb, ng, 0u,
                                                             lds, nullptr);
    if (threadIdx.x == 0) {
        out_count[t] = min(int64_t(total), K.k[t]);
        if (out_total) out_total[t] = int64_t(total);
    }
}

// Re-derive one overflowed piece from u and v (as k_bl_fused left them:
// unmasked) and deliver its entries from position pos0 on.
template <bool kAligned, int kSel>
__device__ __forceinline__ void bl_redo_piece(
    float* __restrict__ u, float* __restrict__ v, int64_t e0, uint32_t len,
    uint32_t magic, uint32_t rb, uint32_t theta, int64_t o, int64_t pos0, int64_t nd,
    int64_t obase, uint32_t* __restrict__ out_idx, float* __restrict__ out_val,
    uint32_t* th) {
    const int lane = lane_id();
    const int64_t e1 = e0 + len;
    float un[kRounds][4], vn[kRounds][4];
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t el = e0 + bl_off<kAligned>(i, c, lane);
            un[i][c] = el < e1 ? u[el] : 0.0f;
            vn[i][c] = el < e1 ? v[el] : 0.0f;
        }
    bool f[kRounds][4];
    uint32_t rank[kRounds][4];
    sel_flags<kAligned, kSel>(vn, un, len, magic, rb, theta, th, f);
    (void)bl_ranks<kAligned>(f, rank);
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (f[i][c] && int64_t(rank[i][c]) < nd) {
                const uint32_t e = bl_off<kAligned>(i, c, lane);
                const int64_t at = obase + pos0 + rank[i][c];
                out_idx[at] = uint32_t(e0 - o) + e;
                out_val[at] = vn[i][c];
                u[e0 + e] = 0.0f;
                v[e0 + e] = 0.0f;
            }
}

// Final placement, kWave pieces per wave.  Lane j first reads the fields of
// piece q0 + j; then the wave copies the entries of all slot pieces as one
// flat list (kUnroll entries per lane per round, so their loads overlap),
// finding each entry's piece by a binary search over the lanes' prefix
// sums; then it re-derives the overflowed pieces one after another.
// Tensor t's output starts at koff[t]; piece p's entries at
// goff[group of p] + pre[p] within it.
constexpr int kGatherUnroll = 4;

template <int kSel>
__global__ __launch_bounds__(kBlock) void k_bl_gather(
    float* __restrict__ u, float* __restrict__ v, DevLayout L, DevK K, DevBins B,
    const TensorState* __restrict__ ts, uint32_t pcap_limit,
    const CandSlot* __restrict__ slots, int64_t n_pieces,
    uint32_t* __restrict__ out_idx, float* __restrict__ out_val) {
    __shared__ __align__(16) uint32_t th[SelLds<kSel>::kRows][SelLds<kSel>::kLen];
    const int lane = lane_id();
    const int64_t q0 = ((int64_t(blockIdx.x) * kBlock + threadIdx.x) >> 6) * kWave;
    if (q0 >= n_pieces) return;  // no block-wide barrier follows
    const int64_t p = q0 + lane;
    const uint32_t count = p < n_pieces ? B.cnt[p] : 0u;
    // per-piece fields (lane = piece)
    int64_t sbase = 0, obase = 0, o = 0;
    uint32_t nd = 0, work = 0;
    bool redo = false;
    if (count) {
        const int t = int(B.pdesc[p].tensor);
        const int64_t jp = p - B.pbase[t];
        const int64_t pos0 = int64_t(B.goff[B.gbase[t] + jp / kBlGroup]) + B.pre[p];
        const int64_t cap = K.k[t];
        const uint32_t pcap = min(uint32_t(B.pcap[t]), pcap_limit);
        nd = uint32_t(max(int64_t(0), min(int64_t(count), cap - pos0)));
        obase = K.koff[t] + pos0;
        o = L.o[t];
        if (count <= pcap) {
            sbase = B.slbase[t] + jp * int64_t(pcap);
            work = count;
        } else {
            redo = nd > 0;
        }
    }
    // slot pieces: deliver the first nd entries, give the rest their u, v back
    const uint32_t inc = wave_inclusive_scan(work);
    const uint32_t excl = inc - work;
    const uint32_t all = uint32_t(__shfl(int(inc), kWave - 1, kWave));
    for (uint32_t base = 0; base < all; base += kWave * kGatherUnroll) {
        CandSlot x[kGatherUnroll];
        uint32_t r[kGatherUnroll];
        int src[kGatherUnroll];
#pragma unroll
        for (int q = 0; q < kGatherUnroll; ++q) {
            const uint32_t e = base + q * kWave + lane;
            // largest lane j with excl[j] <= e (a lane with work > 0)
            int j = 0;
#pragma unroll
            for (int step = kWave / 2; step >= 1; step >>= 1) {
                const uint32_t pv = uint32_t(__shfl(int(excl), j + step, kWave));
                if (pv <= e) j += step;
            }
            src[q] = j;
            r[q] = e - uint32_t(__shfl(int(excl), j, kWave));
            const int64_t sb = __shfl(sbase, j, kWave);
            if (e < all) x[q] = slots[sb + r[q]];
        }
#pragma unroll
        for (int q = 0; q < kGatherUnroll; ++q) {
            const uint32_t e = base + q * kWave + lane;
            const int j = src[q];
            const uint32_t ndj = uint32_t(__shfl(int(nd), j, kWave));
            const int64_t ob = __shfl(obase, j, kWave);
            const int64_t oj = __shfl(o, j, kWave);
            if (e >= all) continue;
            if (r[q] < ndj) {
                out_idx[ob + r[q]] = x[q].idx;
                out_val[ob + r[q]] = x[q].v;
            } else {
                v[oj + x[q].idx] = x[q].v;
                u[oj + x[q].idx] = x[q].u;
            }
        }
    }
    // overflowed pieces
    uint64_t todo = __ballot(redo);
    uint32_t* row = th[kSel == kSelBins ? (threadIdx.x >> 6) : 0];
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        const PieceDesc d = B.pdesc[q0 + j];
        const int t = wave_uniform(int(d.tensor));
        const int64_t ob = __shfl(obase, j, kWave);
        const int64_t ndj = int64_t(uint32_t(__shfl(int(nd), j, kWave)));
        const int64_t oj = L.o[t];
        const uint32_t theta = kSel == kSelThresh ? ts[t].lo_key : 0u;
        const uint32_t rb = kSel == kSelBins ? uint32_t(B.rbins[t]) : 0u;
        if ((d.start & 3) == 0)
            bl_redo_piece<true, kSel>(u, v, d.start, d.len, uint32_t(B.magic[t]), rb, theta,
                                      oj, 0, ndj, ob, out_idx, out_val, row);
        else
            bl_redo_piece<false, kSel>(u, v, d.start, d.len, uint32_t(B.magic[t]), rb, theta,
                                       oj, 0, ndj, ob, out_idx, out_val, row);
    }
}

}  // namespace dgc
