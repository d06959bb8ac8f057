// kernels_shared.hpp -- shared-index (commutative) compression on gfx950.
//
// Method: the ScaleComp abstract (taxoreview.com page) asks for a compressor
// that commutes with the sum over learners, so that an all-reduce can carry
// the aggregate and its cost does not grow with the number of learners.
// Reading: every learner of a step sends its v at one shared index set per
// tensor -- the leader's exact top-k, taken by dgc_compress -- and masks u
// and v there (DGC review, "Proposed method": momentum factor masking).  The
// aggregate is the learner-order binary32 sum of the value vectors.
//
// Passes of dgc_compress_shared (after the clip norm):
//   sh_poff    per 1024-element piece: where its tensor's shared entries
//              reach the piece (binary search over the ascending indices)
//   sh_fused   the element-wise pass (20 B/elem, as k_fused): u, v update;
//              the piece's shared offsets set bits of a per-wave LDS bitmap;
//              flagged entries get their rank by ballot + popcount, go to
//              out_val in index order and are stored as u = v = +0
// and of dgc_shared_sum:
//   sh_sum     per entry: the learners' values added in learner order from
//              +0.0; the sum written out and, for a fresh dense sum,
//              scattered at the shared index (after a zero fill)
#pragma once

#include "dgc_device.hpp"
#include "kernel_fused.hpp"

namespace dgc {

// One thread per piece: the first of the tensor's shared entries whose
// local index is at or past the piece's start (0 .. k_t), i.e. the start of
// the piece's run of shared entries.  Only the tensor's k_t entries are
// read, whatever they hold.
__global__ __launch_bounds__(kBlock) void k_sh_poff(
    DevLayout L, DevK K, const uint32_t* __restrict__ idx,
    uint32_t* __restrict__ poff, int64_t n_pieces) {
    const int64_t p = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (p >= n_pieces) return;
    const PieceDesc d = L.pdesc[p];
    const int t = int(d.tensor);
    const int64_t a = d.start - L.o[t];
    const uint32_t* id = idx + K.koff[t];
    int64_t lo = 0, hi = K.k[t];
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (int64_t(id[mid]) < a) lo = mid + 1; else hi = mid;
    }
    poff[p] = uint32_t(lo);
}

// The piece [e0, e1) of tensor t (local start a = e0 - o_t): g, u, v loaded
// and updated as in fused_piece; its shared entries [j0, j1) of the tensor
// set bits in the wave's 32-word LDS bitmap `bm` (bit e - e0 for element
// e); each flagged element takes its rank in index order, its v goes to
// out_val[koff_t + j0 + rank], and it is stored as u = v = +0.  A run whose
// indices leave the piece, repeat or are not ascending latches
// DGC_ECORRUPT (with the per-piece runs covering the tensor's entries in
// order, a set that passes every piece's check is ascending and inside its
// tensor); every write stays inside the piece's elements and its [j0, j1)
// output slots.
template <bool kAligned>
__device__ __forceinline__ void shared_piece(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    int64_t e0, int64_t e1, int t, int64_t p, const DevLayout& L, const DevK& K,
    float s, float m, const uint32_t* __restrict__ idx,
    const uint32_t* __restrict__ poff, float* __restrict__ out_val,
    Scalars* __restrict__ sc, uint32_t* bm) {
    const int lane = lane_id();
    float un[kRounds][4], vn[kRounds][4];
    bool full[kRounds];
    const int64_t ubase = e0 >> 2;
    if (kAligned) {
        float4 gv[kRounds], uv[kRounds], vv[kRounds];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            const int64_t el = (ubase + i * kWave + lane) << 2;
            full[i] = el + 4 <= e1;
            if (full[i]) {
                gv[i] = ld_stream(g + el);
                uv[i] = ld_stream(u + el);
                vv[i] = ld_stream(v + el);
            } else {
                float tg[4] = {0, 0, 0, 0}, tu[4] = {0, 0, 0, 0}, tv[4] = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (el + c < e1) { tg[c] = g[el + c]; tu[c] = u[el + c]; tv[c] = v[el + c]; }
                gv[i] = make_float4(tg[0], tg[1], tg[2], tg[3]);
                uv[i] = make_float4(tu[0], tu[1], tu[2], tu[3]);
                vv[i] = make_float4(tv[0], tv[1], tv[2], tv[3]);
            }
        }
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            float gg[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
            float uu[4] = {uv[i].x, uv[i].y, uv[i].z, uv[i].w};
            float vv4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                momentum_update(gg[c], s, m, uu[c], vv4[c]);
                un[i][c] = uu[c];
                vn[i][c] = vv4[c];
            }
        }
    } else {
        // element (i, c) of a lane is e0 + (i*4 + c)*64 + lane
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            full[i] = false;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t el = e0 + int64_t(i * 4 + c) * kWave + lane;
                const bool ok = el < e1;
                float gg = ok ? g[el] : 0.f, uu = ok ? u[el] : 0.f, vv = ok ? v[el] : 0.f;
                momentum_update(gg, s, m, uu, vv);
                un[i][c] = uu;
                vn[i][c] = vv;
            }
        }
    }
    // the piece's shared entries (read while the loads are in flight)
    const int64_t o = L.o[t];
    const int64_t a = e0 - o, len = e1 - e0;
    const int64_t kt = K.k[t];
    const int64_t kb = K.koff[t];
    const int64_t j0 = poff[p];
    const int64_t j1 = p + 1 < L.pbase[t + 1] ? int64_t(poff[p + 1]) : kt;
    bool bad = j1 < j0 || j1 - j0 > len || j1 > kt;  // uniform
    for (int w = lane; w < int(kPiece / 32); w += kWave) bm[w] = 0u;
    __builtin_amdgcn_wave_barrier();
    if (!bad) {
        // each entry inside the piece and above the one before it: with the
        // runs of all pieces covering [0, k_t) in order (poff[first] = 0,
        // non-decreasing), that makes the whole list ascending and in range
        for (int64_t j = j0 + lane; j < j1; j += kWave) {
            const int64_t cur = idx[kb + j];
            const int64_t prev = j > j0 ? int64_t(idx[kb + j - 1]) : a - 1;
            const int64_t off = cur - a;
            if (off >= 0 && off < len && cur > prev) atomicOr(&bm[off >> 5], 1u << (off & 31));
            else bad = true;
        }
    }
    // a wave's LDS operations complete in order: the reads below see every
    // bit set above
    __builtin_amdgcn_wave_barrier();
    bool f[kRounds][4];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        if (kAligned) {
            // offset (i*64 + lane)*4 + c: word i*8 + lane/8, bits 4*(lane%8) + c
            const uint32_t w = bm[i * 8 + (lane >> 3)] >> ((lane & 7) * 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) f[i][c] = (w >> c) & 1u;
        } else {
            // offset (i*4 + c)*64 + lane: word (i*4 + c)*2 + lane/32, bit lane%32
#pragma unroll
            for (int c = 0; c < 4; ++c)
                f[i][c] = (bm[(i * 4 + c) * 2 + (lane >> 5)] >> (lane & 31)) & 1u;
        }
    }
    // ranks in index order (as fused_piece)
    uint32_t rank[kRounds][4];
    uint32_t total = 0;
    const uint64_t lt = lanemask_lt();
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
    // repeated indices set fewer bits than the run holds
    if (!bad && int64_t(total) != j1 - j0) bad = true;
    // masked stores
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        float su[4], sv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            su[c] = f[i][c] ? 0.0f : un[i][c];
            sv[c] = f[i][c] ? 0.0f : vn[i][c];
        }
        if (kAligned) {
            const int64_t el = (ubase + i * kWave + lane) << 2;
            if (full[i]) {
                st_stream(u + el, su[0], su[1], su[2], su[3]);
                st_stream(v + el, sv[0], sv[1], sv[2], sv[3]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (el + c < e1) { u[el + c] = su[c]; v[el + c] = sv[c]; }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t el = e0 + int64_t(i * 4 + c) * kWave + lane;
                if (el < e1) { u[el] = su[c]; v[el] = sv[c]; }
            }
        }
    }
    // the values, in index order (rank < total <= j1 - j0 when bits were set)
    float* ov = out_val + kb + j0;
#pragma unroll
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (f[i][c]) ov[rank[i][c]] = vn[i][c];
    if (__ballot(bad) && lane == 0) latch_error(sc, kErrCorrupt);
}

// The element-wise pass of dgc_compress_shared: one wave per piece.  With
// clipping off the scale is 1 and block 0 writes the call's scalar outputs.
__global__ __launch_bounds__(kBlock) void k_sh_fused(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    DevLayout L, DevK K, Scalars* __restrict__ sc, int clip_on, float m,
    const uint32_t* __restrict__ idx, const uint32_t* __restrict__ poff,
    float* __restrict__ out_val, int64_t n_pieces, double* __restrict__ out_norm,
    float* __restrict__ out_scale) {
    __shared__ uint32_t bitmap[kWavesPerBlock][kPiece / 32];
    const float s = clip_on ? sc->scale : 1.0f;
    if (!clip_on && blockIdx.x == 0 && threadIdx.x == 0) {
        sc->norm = -1.0;
        sc->scale = 1.0f;
        if (out_norm) *out_norm = -1.0;
        if (out_scale) *out_scale = 1.0f;
    }
    uint32_t* bm = bitmap[threadIdx.x >> 6];
    const int64_t w0 = (int64_t(blockIdx.x) * kBlock + threadIdx.x) >> 6;
    const int64_t nw = (int64_t(gridDim.x) * kBlock) >> 6;
    for (int64_t p = w0; p < n_pieces; p += nw) {
        const PieceDesc d = L.pdesc[p];
        const int t = wave_uniform(int(d.tensor));
        const int64_t e0 = d.start;
        const int64_t e1 = e0 + d.len;
        if ((e0 & 3) == 0)
            shared_piece<true>(g, u, v, e0, e1, t, p, L, K, s, m, idx, poff, out_val, sc, bm);
        else
            shared_piece<false>(g, u, v, e0, e1, t, p, L, K, s, m, idx, poff, out_val, sc, bm);
    }
}

// ---------------------------------------------------------------- sum

constexpr int kShBatch = 16;  // learners added per pass

// One pass's learners (by value).
struct ShBatch {
    const float* vals[kShBatch];
    int W;
};

// Per entry j of the shared set: s = (first ? +0.0 : out_sum[j]) + the
// batch's values in learner order; out_sum[j] = s, and with `dense` set,
// dense[o_t + idx[j]] = s (an index outside its tensor latches
// DGC_ECORRUPT and is not written).  Workgroups stride over the k tiles; a
// tile's tensor comes from a binary search over the per-tensor tile bases
// (only L.T, L.o and K's k, koff and ktbase are read).
__global__ __launch_bounds__(kBlock) void k_sh_sum(
    DevLayout L, DevK K, ShBatch B, int first, const uint32_t* __restrict__ idx,
    float* __restrict__ out_sum, float* __restrict__ dense,
    Scalars* __restrict__ sc, int64_t n_ktiles) {
    for (int64_t vt = blockIdx.x; vt < n_ktiles; vt += gridDim.x) {
        const int t = find_seg(K.ktbase, L.T, vt);
        const int64_t kt = K.k[t], kb = K.koff[t];
        const int64_t i0 = (vt - K.ktbase[t]) * kTile;
        const int64_t o = L.o[t], nt = L.o[t + 1] - o;
        bool bad = false;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const int64_t i = i0 + int64_t(q) * kBlock + threadIdx.x;
            if (i >= kt) continue;
            const int64_t j = kb + i;
            float x[kShBatch];
#pragma unroll
            for (int w = 0; w < kShBatch; ++w)
                if (w < B.W) x[w] = B.vals[w][j];
            float s = first ? 0.0f : out_sum[j];
#pragma unroll
            for (int w = 0; w < kShBatch; ++w)
                if (w < B.W) s = __fadd_rn(s, x[w]);
            out_sum[j] = s;
            if (dense) {
                const int64_t ix = idx[j];
                if (ix < nt) dense[o + ix] = s;
                else bad = true;
            }
        }
        if (bad) latch_error(sc, kErrCorrupt);
    }
}

}  // namespace dgc
