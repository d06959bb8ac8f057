// kernel_fused.hpp -- the element-wise pass of the compression step on
// gfx950: clipping scale, momentum correction with local accumulation
// (DGC review page (nubint.ai), "Proposed method"), and the candidate
// output that feeds the exact top-k.  This is the kernel that moves
// 20 B per gradient element; everything else of a step is small.
#pragma once

#include "dgc_device.hpp"

namespace dgc {

typedef float f4v __attribute__((ext_vector_type(4)));

// Streaming float4 access that bypasses cache residency (each element of
// g, u, v is touched once per step).
__device__ __forceinline__ float4 ld_stream(const float* p) {
    f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_stream(float* p, float a, float b, float c, float d) {
    f4v x = {a, b, c, d};
    __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(p));
}

// ---------------------------------------------------------------- fused

// Element-wise momentum correction + accumulation, and candidate output.
// A wave owns one piece (<= 1024 elements, one tensor).  It loads g, u, v
// as float4 (64 lanes x 4 units) and updates u and v in registers; each
// candidate (key >= lo) gets its rank in index order by ballot + popcount
// (no atomics, so the layout is the same every run).  When the piece's
// candidates fit its pcap slots, they are masked optimistically: u and v
// are stored as +0 there, and each candidate's slot keeps what the zeros
// replaced (index, v, u).  The selection later puts back
// the candidates it does not send, so the scattered masking writes shrink
// to the few candidates outside the top k.  A piece with more candidates
// than slots stores u and v unmasked and writes no slots; its count above
// pcap sends the tensor to the dense path.  The loads depend only on the
// piece descriptor; the tensor's metadata is read while they are in flight.
template <bool kAligned>
__device__ __forceinline__ void fused_piece(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    int64_t e0, int64_t e1, int t, const DevLayout& L,
    const TensorState* __restrict__ ts, float s, float m,
    CandSlot* __restrict__ slots, uint32_t* __restrict__ run_cnt, int64_t p) {
    const int lane = lane_id();
    float un[kRounds][4], vn[kRounds][4];
    bool f[kRounds][4];
    bool full[kRounds];
    uint32_t lo;
    int64_t o, pcap;
    if (kAligned) {
        // e0 is a multiple of 4: 64 * kRounds float4 units cover the piece.
        const int64_t ubase = e0 >> 2;
        float4 gv[kRounds], uv[kRounds], vv[kRounds];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            int64_t el = (ubase + i * kWave + lane) << 2;
            full[i] = el + 4 <= e1;
            if (full[i]) {
                gv[i] = ld_stream(g + el);
                uv[i] = ld_stream(u + el);
                vv[i] = ld_stream(v + el);
            } else {
                float tg[4] = {0, 0, 0, 0}, tu[4] = {0, 0, 0, 0},
                      tv[4] = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (el + c < e1) { tg[c] = g[el + c]; tu[c] = u[el + c]; tv[c] = v[el + c]; }
                gv[i] = make_float4(tg[0], tg[1], tg[2], tg[3]);
                uv[i] = make_float4(tu[0], tu[1], tu[2], tu[3]);
                vv[i] = make_float4(tv[0], tv[1], tv[2], tv[3]);
            }
        }
        lo = ts[t].lo_key;
        o = L.o[t];
        pcap = L.pcap[t];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            int64_t el = (ubase + i * kWave + lane) << 2;
            float gg[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
            float uu[4] = {uv[i].x, uv[i].y, uv[i].z, uv[i].w};
            float vv4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                momentum_update(gg[c], s, m, uu[c], vv4[c]);
                un[i][c] = uu[c];
                vn[i][c] = vv4[c];
                f[i][c] = (el + c < e1) && mag_key(vv4[c]) >= lo;
            }
        }
    } else {
        // Unaligned piece start: 4 * kRounds scalar rounds of 64 consecutive
        // elements.
        // Element (i, c) of a lane is e0 + (i*4 + c)*64 + lane; ranks below
        // follow (i, c, lane) order, which is index order here.
        lo = ts[t].lo_key;
        o = L.o[t];
        pcap = L.pcap[t];
#pragma unroll
        for (int i = 0; i < kRounds; ++i) {
            full[i] = false;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                int64_t el = e0 + int64_t(i * 4 + c) * kWave + lane;
                bool ok = el < e1;
                float gg = ok ? g[el] : 0.f, uu = ok ? u[el] : 0.f,
                      vv = ok ? v[el] : 0.f;
                momentum_update(gg, s, m, uu, vv);
                un[i][c] = uu;
                vn[i][c] = vv;
                f[i][c] = ok && mag_key(vv) >= lo;
            }
        }
    }
    // Ranks in index order.
    uint32_t rank[kRounds][4];
    uint32_t total = 0;
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        uint64_t b[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = __ballot(f[i][c]);
        if (kAligned) {
            // order within round i: (lane, c)
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
            // order within round i: (c, lane)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rank[i][c] = total + __popcll(b[c] & lt);
                total += __popcll(b[c]);
            }
        }
    }
    // Masked stores: a candidate is stored as +0 when the piece's run fits.
    const bool fits = total <= uint32_t(pcap);  // wave-uniform
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
        float su[4], sv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool z = fits && f[i][c];
            su[c] = z ? 0.0f : un[i][c];
            sv[c] = z ? 0.0f : vn[i][c];
        }
        if (kAligned) {
            int64_t el = ((e0 >> 2) + i * kWave + lane) << 2;
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
                int64_t el = e0 + int64_t(i * 4 + c) * kWave + lane;
                if (el < e1) { u[el] = su[c]; v[el] = sv[c]; }
            }
        }
    }
    // The piece's run goes to its own pcap slots; a count above pcap marks
    // the overflow (the tensor then takes the dense path).
    if (lane == 0) run_cnt[p] = total;
    if (total && fits) {
        CandSlot* sl = slots + L.slbase[t] + (p - L.pbase[t]) * pcap;
        const int64_t unit0 = e0 >> 2;
#pragma unroll
        for (int i = 0; i < kRounds; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (f[i][c]) {
                    int64_t el = kAligned ? (((unit0 + i * kWave + lane) << 2) + c)
                                          : (e0 + int64_t(i * 4 + c) * kWave + lane);
                    CandSlot cs;
                    cs.idx = uint32_t(el - o);
                    cs.v = vn[i][c];
                    cs.u = un[i][c];
                    sl[rank[i][c]] = cs;
                }
    }
}

// With clipping off the scale is 1 and block 0 also writes the call's
// scalar outputs (norm -1, scale 1).
__global__ __launch_bounds__(kBlock) void k_fused(
    const float* __restrict__ g, float* __restrict__ u, float* __restrict__ v,
    DevLayout L, const TensorState* __restrict__ ts, Scalars* __restrict__ sc,
    int clip_on, float m, CandSlot* __restrict__ slots, uint32_t* __restrict__ run_cnt,
    int64_t n_pieces, double* __restrict__ out_norm, float* __restrict__ out_scale) {
    const float s = clip_on ? sc->scale : 1.0f;
    if (!clip_on && blockIdx.x == 0 && threadIdx.x == 0) {
        sc->norm = -1.0;
        sc->scale = 1.0f;
        if (out_norm) *out_norm = -1.0;
        if (out_scale) *out_scale = 1.0f;
    }
    const int64_t w0 = (int64_t(blockIdx.x) * kBlock + threadIdx.x) >> 6;
    const int64_t nw = (int64_t(gridDim.x) * kBlock) >> 6;
    for (int64_t p = w0; p < n_pieces; p += nw) {
        const PieceDesc d = L.pdesc[p];
        const int t = wave_uniform(int(d.tensor));
        const int64_t e0 = d.start;
        const int64_t e1 = e0 + d.len;
        if ((e0 & 3) == 0)
            fused_piece<true>(g, u, v, e0, e1, t, L, ts, s, m, slots, run_cnt, p);
        else
            fused_piece<false>(g, u, v, e0, e1, t, L, ts, s, m, slots, run_cnt, p);
    }
}

}  // namespace dgc
