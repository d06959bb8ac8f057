// dgc_device.hpp -- constants, device-visible layout structs and wave/block
// helpers shared by the libdgc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgc {

// ---------------------------------------------------------------- sizes

constexpr int kWave = 64;
constexpr int kBlock = 256;                 // threads per workgroup (4 waves)
constexpr int kWavesPerBlock = kBlock / kWave;

// Element-wise pass: one wave owns one "piece" of kPiece consecutive
// elements of one tensor (64 lanes x kRounds float4).  Candidates of a
// piece are written as one index-ordered run.
#ifndef DGC_PIECE_SHIFT
#define DGC_PIECE_SHIFT 10
#endif
constexpr int kPieceShift = DGC_PIECE_SHIFT;
constexpr int64_t kPiece = int64_t(1) << kPieceShift;
constexpr int kRounds = int(kPiece / (4 * 64));
static_assert(kRounds >= 1 && kRounds <= 8, "piece of 256..2048 elements");
// Pieces are scanned in groups of 256 (one workgroup per group).
constexpr int64_t kGroup = 256;

// Generic tiles for histogram / emit / encode / decode passes: 1024 items
// per workgroup visit (4 per thread).  Candidate lists are short (a few
// tens of thousands per tensor), so small tiles keep many workgroups busy.
#ifndef DGC_TILE_SHIFT
#define DGC_TILE_SHIFT 10
#endif
constexpr int kTileShift = DGC_TILE_SHIFT;
constexpr int64_t kTile = int64_t(1) << kTileShift;
constexpr int kPerThread = int(kTile / kBlock);

// Radix select on the 31-bit magnitude key: digits of 11, 10, 10 bits.
constexpr int kBins0 = 2048;
constexpr int kHistBins = 2048;  // histogram row per tensor (largest digit)

// Sample window: 32-element lines; tensors above kSmallN elements sample
// max(kMinSampleLines, lines/256) lines; smaller tensors skip the window and
// take the dense exact path (a few passes over at most 256 KiB).
constexpr int64_t kLine = 32;
constexpr int64_t kSmallN = 65536;
constexpr int64_t kMinSampleLines = 512;
constexpr int64_t kLinesPerSampleBlock = 64;

// Binary64 norm: one workgroup per chunk of 2^12 .. 2^18 elements (a power
// of two, the largest that still gives 256 workgroups), fixed order.
constexpr int64_t kNormChunkMin = int64_t(1) << 12;
constexpr int64_t kNormChunk = int64_t(1) << 18;

// Per-tensor selection modes (decided after the element-wise pass).
constexpr uint32_t kModeSkip = 0;   // k = 0
constexpr uint32_t kModeList = 1;   // select among the gathered candidates
constexpr uint32_t kModeDense = 2;  // exact select over the whole tensor

constexpr uint32_t kNoKey = 0xFFFFFFFFu;  // above every 31-bit key

// Device-side error latch values (negated DGC_* codes).
constexpr uint32_t kErrCorrupt = 4;
constexpr uint32_t kErrInternal = 3;

// ---------------------------------------------------------------- structs

// Per-tensor selection state, one per tensor in the workspace.
struct TensorState {
    uint32_t lo_key;    // candidate threshold from the sample window
    uint32_t total;     // candidates found by the element-wise pass
    uint32_t mode;      // kMode*
    uint32_t len;       // items of the select source (list length or n_t)
    uint32_t prefix;    // radix-select prefix; the threshold key T at the end
    uint32_t krem;      // k still to place within the prefix; r at the end
    uint32_t overflow;  // some piece found more candidates than its slots
    uint32_t wbin;      // sample window: chosen top-11-bit bin (or kNoKey)
    uint32_t wabove;    // sample window: samples above wbin
    uint32_t wj;        // sample window: rank j of the targeted sample
    uint32_t done21;    // kDone21: the top 21 bits of T were found from the
                        // gather's histogram (the first two digit passes
                        // skip it); kDoneAll: T and r are final (no digit
                        // pass)
    uint32_t floor;     // hierarchical selector: the survivors' least key,
                        // max(theta, 1); keys below it count as 0 in the
                        // select.  0 for exact top-k
    uint32_t pad[2];
};

// TensorState::done21
constexpr uint32_t kDone21 = 1;
constexpr uint32_t kDoneAll = 2;

// Per-call scalars.
struct Scalars {
    double norm;
    float scale;
    uint32_t status;  // latched kErr* (0 = fine)
    uint32_t pad[12];
};

// One 1024-element piece of the element-wise pass: global start, tensor,
// length (16 bytes, one load).
struct PieceDesc {
    int64_t start;
    uint32_t tensor;
    uint32_t len;
};

// A candidate of the exact path's element-wise pass: local index, v, and
// the u that the candidate's masking replaced (12 bytes, one piece's slots
// contiguous).
struct CandSlot {
    uint32_t idx;
    float v;
    float u;
};
static_assert(sizeof(CandSlot) == 12, "12-byte candidate slots");

// Layout tables (device pointers into the workspace), passed by value.
struct DevLayout {
    int32_t T;
    const int64_t* o;       // [T+1] element offsets
    const int64_t* pbase;   // [T+1] first piece of each tensor
    const int64_t* tbase;   // [T+1] first select/emit tile (ceil(n_t/kTile))
    const int64_t* obase;   // [T+1] ordered candidate list offsets (capacity)
    const int64_t* slbase;  // [T+1] candidate slot offsets (pieces x pcap)
    const int64_t* pcap;    // [T] candidate slots per piece
    const int64_t* sbase;   // [T+1] first sample block
    const int64_t* slines;  // [T] sampled lines (0 = no sampling)
    const int64_t* ebase;   // [T+1] encoded stream capacity offsets
    const int64_t* etbase;  // [T+1] tiles over encoded capacity
    const PieceDesc* pdesc; // [pieces] start, tensor and length of each piece
    const int64_t* gbase;   // [T+1] first piece group of each tensor
    const uint32_t* gmap;   // [groups] tensor of each piece group
    const uint32_t* smap;   // [sample blocks] tensor of each sample block
    const uint32_t* emap;   // [capacity tiles] tensor of each tile
};

// Per-call k tables.
struct DevK {
    const int64_t* k;       // [T]
    const int64_t* koff;    // [T+1] output offsets
    const int64_t* ktbase;  // [T+1] tiles over k (ceil(k_t/kTile))
    const uint32_t* kmap;   // [k tiles] tensor of each tile
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t mag_key(float x) {
    return __float_as_uint(x) & 0x7FFFFFFFu;
}

// The key the select ranks under the hierarchical selector's floor: keys
// below it (not survivors of the first level) count as 0.  The identity for
// floor 0.
__device__ __forceinline__ uint32_t floor_key(uint32_t key, uint32_t floor) {
    return key >= floor ? key : 0u;
}

// u <- fl(fl(m*u) + fl(g*s)); v <- fl(v + u).  Each operation rounds once
// (explicit _rn intrinsics: never contracted into an FMA).
__device__ __forceinline__ void momentum_update(float g, float s, float m,
                                                float& u, float& v) {
    float gs = __fmul_rn(g, s);
    float mu = __fmul_rn(m, u);
    u = __fadd_rn(mu, gs);
    v = __fadd_rn(v, u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

__device__ __forceinline__ int wave_uniform(int x) {
    return __builtin_amdgcn_readfirstlane(x);
}

// Largest t in [0, T) with base[t] <= x (base is non-decreasing, base[T] is
// the total, x < base[T]).  Empty segments are skipped.
__device__ __forceinline__ int find_seg(const int64_t* __restrict__ base,
                                        int T, int64_t x) {
    int lo = 0, hi = T;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (base[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Inclusive scan within a wave.  32-bit integers: DPP moves (row_shr 1, 2,
// 4, 8 within each 16-lane row, then row_bcast 15 and 31 across rows), six
// ALU steps; a lane a move cannot reach gets 0.  Wider types: Hillis-Steele
// with shuffles (each routed through the LDS crossbar).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
    if constexpr (sizeof(T) == 4) {
#define DGC_DPP_ADD(ctrl, rows) \
    x += T(__builtin_amdgcn_update_dpp(0, int(x), (ctrl), (rows), 0xF, true))
        DGC_DPP_ADD(0x111, 0xF);  // row_shr:1
        DGC_DPP_ADD(0x112, 0xF);  // row_shr:2
        DGC_DPP_ADD(0x114, 0xF);  // row_shr:4
        DGC_DPP_ADD(0x118, 0xF);  // row_shr:8
        DGC_DPP_ADD(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
        DGC_DPP_ADD(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef DGC_DPP_ADD
        return x;
    } else {
        const int lane = lane_id();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            T y = __shfl_up(x, d, kWave);
            if (lane >= d) x += y;
        }
        return x;
    }
}

// Exclusive scan across the 256-thread block.  `lds` holds kWavesPerBlock
// values.  Every thread must call it.  Returns the exclusive prefix; `total`
// receives the block sum.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T x, T* lds, T& total) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    T inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) lds[wid] = inc;
    __syncthreads();
    T wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        T s = lds[w];
        if (w < wid) wpre += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return wpre + inc - x;
}

// Long per-tensor scans run in one block, kScanRound values per round.  A
// thread owns kScanPer consecutive values of a round (their sum feeds one
// block-wide scan), but global loads and stores are lane-consecutive: all
// kScanPer loads of a round are issued at once into registers, then
// transposed through an LDS stage (index e + e/32, free of bank
// conflicts).  Read directly, a thread's consecutive values put every lane
// of a load on its own cache line, and the round costs one line request
// per value.  Direct reads remain cheaper for a round of at most
// kScanDirect values, and kernels whose scans are all short are built
// without the stage (kStaged = false: 34 KB less LDS and fewer registers),
// which the host picks when no tensor can need more than kScanStagedMin
// values.
constexpr int kScanPer = 32;
constexpr int64_t kScanDirect = 2048;
constexpr int64_t kScanStagedMin = 16384;
constexpr int kScanRound = kBlock * kScanPer;
constexpr int kScanStage = kScanRound + kScanRound / 32;
__device__ __forceinline__ int scan_pad(int e) { return e + (e >> 5); }

// Values [base, base + kScanRound) of in[0, count) (0 past count), each
// thread's kScanPer consecutive ones in x.
template <bool kStaged>
__device__ __forceinline__ void scan_load_round(const uint32_t* __restrict__ in, int64_t base,
                                                int64_t count, uint32_t* stage,
                                                uint32_t (&x)[kScanPer]) {
    const int tid = int(threadIdx.x);
    if (!kStaged || count - base <= kScanDirect) {  // uniform
        const int64_t i0 = base + int64_t(tid) * kScanPer;
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) x[q] = i0 + q < count ? in[i0 + q] : 0u;
        return;
    }
    uint32_t c[kScanPer];
#pragma unroll
    for (int q = 0; q < kScanPer; ++q) {
        const int64_t i = base + int64_t(q) * kBlock + tid;
        c[q] = i < count ? in[i] : 0u;
    }
#pragma unroll
    for (int q = 0; q < kScanPer; ++q) stage[scan_pad(q * kBlock + tid)] = c[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kScanPer; ++q) x[q] = stage[scan_pad(tid * kScanPer + q)];
    __syncthreads();
}

// Store each thread's kScanPer consecutive results r of the round at
// `base` into out[0, count), lane-consecutive, through the stage (32-bit
// halves for 64-bit results).
template <bool kStaged, typename TO>
__device__ __forceinline__ void scan_store_round(TO* __restrict__ out, int64_t base,
                                                 int64_t count, uint32_t* stage,
                                                 const TO (&r)[kScanPer]) {
    const int tid = int(threadIdx.x);
    if (!kStaged || count - base <= kScanDirect) {  // uniform
        const int64_t i0 = base + int64_t(tid) * kScanPer;
#pragma unroll
        for (int q = 0; q < kScanPer; ++q)
            if (i0 + q < count) out[i0 + q] = r[q];
        return;
    }
    constexpr int kHalves = sizeof(TO) / 4;
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
#pragma unroll
        for (int q = 0; q < kScanPer; ++q)
            stage[scan_pad(tid * kScanPer + q)] = uint32_t(uint64_t(r[q]) >> (32 * hv));
        __syncthreads();
        uint32_t c[kScanPer];
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) c[q] = stage[scan_pad(q * kBlock + tid)];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) {
            const int64_t i = base + int64_t(q) * kBlock + tid;
            if (i >= count) continue;
            if (kHalves == 1) {
                out[i] = TO(c[q]);
            } else {
                uint32_t* w = reinterpret_cast<uint32_t*>(out + i);
                w[hv] = c[q];  // little-endian halves of a 64-bit result
            }
        }
    }
}

// Exclusive scan of in[0, count) into out[0, count), starting at `carry`,
// by one block.  `lds` holds kWavesPerBlock values, `stage` kScanStage
// (unused unless kStaged).  Returns carry + total.  Every thread must call
// it.
template <typename TO, bool kStaged>
__device__ __forceinline__ TO block_scan_range(const uint32_t* __restrict__ in,
                                               TO* __restrict__ out, int64_t count,
                                               TO carry, TO* lds, uint32_t* stage) {
    for (int64_t base = 0; base < count; base += kScanRound) {
        uint32_t x[kScanPer];
        scan_load_round<kStaged>(in, base, count, stage, x);
        TO local = 0;
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) local += TO(x[q]);
        TO tot;
        TO run = carry + block_exclusive_scan(local, lds, tot);
        TO r[kScanPer];
#pragma unroll
        for (int q = 0; q < kScanPer; ++q) {
            r[q] = run;
            run += TO(x[q]);
        }
        scan_store_round<kStaged>(out, base, count, stage, r);
        carry += tot;
    }
    return carry;
}

// Exclusive prefix, in thread order, of two 0/1 flags across the block, from
// wave ballots; also their block totals.  `lds2` holds 2 * kWavesPerBlock
// values.  Every thread must call it.
__device__ __forceinline__ void block_flag_prefix2(bool a, bool b, uint32_t* lds2,
                                                   uint32_t& pa, uint32_t& pb,
                                                   uint32_t& ta, uint32_t& tb) {
    const int wid = threadIdx.x >> 6;
    const uint64_t lt = lanemask_lt();
    const uint64_t ba = __ballot(a), bb = __ballot(b);
    if (lane_id() == 0) {
        lds2[wid] = uint32_t(__popcll(ba));
        lds2[kWavesPerBlock + wid] = uint32_t(__popcll(bb));
    }
    __syncthreads();
    uint32_t wa = 0, wb = 0;
    ta = 0;
    tb = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        uint32_t x = lds2[w], y = lds2[kWavesPerBlock + w];
        if (w < wid) { wa += x; wb += y; }
        ta += x;
        tb += y;
    }
    __syncthreads();
    pa = wa + uint32_t(__popcll(ba & lt));
    pb = wb + uint32_t(__popcll(bb & lt));
}

// Sum across the block in a fixed order (deterministic for floating point).
__device__ __forceinline__ double block_sum_fixed(double x, double* lds) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) x += __shfl_xor(x, d, kWave);
    if (lane == 0) lds[wid] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += lds[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ void latch_error(Scalars* sc, uint32_t code) {
    atomicMax(&sc->status, code);
}

// 32-bit integer mix (the finaliser of MurmurHash3) for sample offsets.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

}  // namespace dgc
