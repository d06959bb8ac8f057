// dgc_api.hip -- host side of libdgc: argument checks, workspace layout and
// the launch sequence of each entry point.  See include/dgc.h for the
// contract of every function.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "dgc.h"
#include "dgc_device.hpp"
#include "kernels_binlocal.hpp"
#include "kernels_codec.hpp"
#include "kernels_compress.hpp"
#include "kernels_sampled.hpp"
#include "kernels_shared.hpp"
#include "kernels_tensor.hpp"

using namespace dgc;

namespace {

constexpr size_t kAlign = 256;

// Workgroups per compute unit of the encode / decode tile walks.
#ifndef DGC_CODEC_BLOCKS_PER_CU
#define DGC_CODEC_BLOCKS_PER_CU 32
#endif
constexpr int64_t kCodecBlocksPerCU = DGC_CODEC_BLOCKS_PER_CU;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Host-side layout of one state and the carving of its workspace.
struct Plan {
    int32_t T = 0;
    std::vector<int64_t> sizes, kmax;
    // tables uploaded at init (int64): o, pbase, tbase, obase, sbase,
    // slines, ebase, etbase, slbase, pcap -- each T+1 long (padded)
    std::vector<int64_t> o, pbase, tbase, obase, sbase, slines, ebase, etbase,
        slbase, pcap, gbase;
    std::vector<PieceDesc> pdesc;
    std::vector<uint32_t> smap, emap, gmap, bmap;
    // sampled threshold: lines sampled per tensor (every line of a small
    // tensor), their sample blocks, and the tensor of each block
    std::vector<int64_t> aslines, asbase;
    // per-tensor window of the per-tensor path: lines sampled per tensor
    // (every line up to kMinSampleLines of them, else as slines)
    std::vector<int64_t> wlines;
    std::vector<uint32_t> asmap;
    int64_t AS = 0;
    // merged decode: bounds per tensor (dense blocks + 1) and dense blocks
    std::vector<int64_t> dbase, bbase;
    int64_t DB = 0, NBLK = 0;
    int64_t n = 0, P = 0, G = 0, TT = 0, A = 0, SL = 0, S = 0, E = 0, ET = 0, NB = 0;
    int64_t norm_chunk = 0;
    // every tensor holds at most kTensorPathMaxN elements: dgc_compress takes
    // the per-tensor window and finish kernels, and small tensors get the
    // sample window (all of their lines) and candidate slots too
    bool tensor_path = true;
    // per-tensor scans that can exceed kScanStagedMin values take the
    // LDS-staged kernels: tiles over n (emit), capacity tiles (decode)
    bool staged_tiles = false, staged_etiles = false;
    int64_t et_max = 0;  // most capacity tiles of one tensor
    // bin-local selector: most pieces and prefix groups any bin length gives
    int64_t BP = 0, BG = 0;
    int64_t tiles = 0;  // entries of each per-tile array
    // workspace byte offsets
    size_t off_tab = 0, off_pdesc = 0, off_smap = 0, off_emap = 0, off_k = 0,
           off_kmap = 0, off_ts = 0, off_sc = 0, off_hist = 0, off_shist = 0,
           off_runc = 0, off_gmap = 0, off_gsum = 0, off_goff = 0, off_atiles = 0, off_aoff = 0,
           off_scratch = 0,
           off_amap = 0, off_slots = 0, off_olist = 0, off_olistv = 0, off_olistu = 0,
           off_ta = 0, off_tb = 0, off_tc = 0, off_t64 = 0, off_part = 0,
           off_bltab = 0, off_blpdesc = 0, off_blcnt = 0, off_blpre = 0, off_blgsum = 0,
           off_blgoff = 0, off_astab = 0, off_asmap = 0, off_ktgt = 0, off_dtab = 0,
           off_dmode = 0, off_bounds = 0, off_bmap = 0, off_bsel = 0, total = 0;
};

// Candidate slots per 1024-element piece: about six times the pieces' share
// of k_max plus 24 -- the sample window aims at 1.5-2.5 k candidates, so a
// piece overflows (sending its tensor to the dense path) only with a
// negligible probability for unstructured data.  Small tensors get none
// unless their whole tensor is sampled (the per-tensor path); otherwise
// they take the dense path.
int64_t piece_cap(int64_t n, int64_t kmax, bool small_slots) {
    if (n == 0 || (n <= kSmallN && !small_slots)) return 0;
    return std::min<int64_t>(kPiece, cdiv(6 * kPiece * kmax, n) + 24);
}

// Capacity of a tensor's ordered candidate list, a multiple of 4 items so
// that every tensor's list starts 16-byte aligned.
int64_t list_cap(int64_t n, int64_t kmax, int64_t slots, bool small_slots) {
    if (n <= kSmallN && !small_slots) return 0;
    return cdiv(std::min<int64_t>(std::min<int64_t>(n, slots), 8 * kmax + 16384), 4) * 4;
}

// Bin-local pieces are L * floor(1024 / L) elements, never fewer than 513
// (1 <= L <= 1024), so a tensor has at most ceil(n / 513) of them.
constexpr int64_t kBlMinPiece = kMaxBin / 2 + 1;

int64_t sample_lines(int64_t n) {
    if (n <= kSmallN) return 0;
    int64_t lines = cdiv(n, kLine);
    return std::min<int64_t>(lines, std::max<int64_t>(kMinSampleLines, lines / 256));
}

int make_plan(int32_t T, const int64_t* sizes, const int64_t* kmax, Plan& p) {
    if (T <= 0 || !sizes || !kmax) return DGC_EINVAL;
    p.T = T;
    p.sizes.assign(sizes, sizes + T);
    p.kmax.assign(kmax, kmax + T);
    p.o.assign(T + 1, 0);
    p.pbase.assign(T + 1, 0);
    p.tbase.assign(T + 1, 0);
    p.obase.assign(T + 1, 0);
    p.slbase.assign(T + 1, 0);
    p.pcap.assign(T + 1, 0);
    p.gbase.assign(T + 1, 0);
    p.sbase.assign(T + 1, 0);
    p.slines.assign(T + 1, 0);
    p.ebase.assign(T + 1, 0);
    p.etbase.assign(T + 1, 0);
    p.aslines.assign(T + 1, 0);
    p.asbase.assign(T + 1, 0);
    p.wlines.assign(T + 1, 0);
    p.dbase.assign(T + 1, 0);
    p.bbase.assign(T + 1, 0);
    for (int32_t t = 0; t < T; ++t)
        if (sizes[t] > kTensorPathMaxN) p.tensor_path = false;
    for (int32_t t = 0; t < T; ++t) {
        int64_t n = sizes[t], km = kmax[t];
        if (n < 0 || n >= (int64_t(1) << 32) || km < 0 || km > n) return DGC_EINVAL;
        p.o[t + 1] = p.o[t] + n;
        const int64_t np_ = cdiv(n, kPiece);
        p.pbase[t + 1] = p.pbase[t] + np_;
        p.gbase[t + 1] = p.gbase[t] + cdiv(np_, kGroup);
        p.tbase[t + 1] = p.tbase[t] + cdiv(n, kTile);
        p.pcap[t] = piece_cap(n, km, p.tensor_path);
        p.slbase[t + 1] = p.slbase[t] + np_ * p.pcap[t];
        p.obase[t + 1] = p.obase[t] + list_cap(n, km, np_ * p.pcap[t], p.tensor_path);
        p.slines[t] = sample_lines(n);
        p.sbase[t + 1] = p.sbase[t] + cdiv(p.slines[t], kLinesPerSampleBlock);
        // a multiple of kStreamAlign entries per tensor, so that every
        // tensor's stream starts 16-byte aligned in the run and value arrays
        const int64_t ecap = cdiv(km + n / 65536, kStreamAlign) * kStreamAlign;
        p.ebase[t + 1] = p.ebase[t] + ecap;
        p.etbase[t + 1] = p.etbase[t] + cdiv(ecap, kTile);
        p.aslines[t] = n <= kSmallN ? cdiv(n, kLine) : p.slines[t];
        p.wlines[t] = std::min<int64_t>(cdiv(n, kLine),
                                        std::max<int64_t>(kMinSampleLines, cdiv(n, kLine) / 256));
        p.asbase[t + 1] = p.asbase[t] + cdiv(p.aslines[t], kLinesPerSampleBlock);
        p.bbase[t + 1] = p.bbase[t] + cdiv(n, kDecBlock);
        p.dbase[t + 1] = p.dbase[t] + cdiv(n, kDecBlock) + 1;
        p.BP += cdiv(n, kBlMinPiece);
        p.BG += cdiv(cdiv(n, kBlMinPiece), kBlGroup);
    }
    p.n = p.o[T];
    for (int32_t t = 0; t < T; ++t) {
        p.staged_tiles |= p.tbase[t + 1] - p.tbase[t] > kScanStagedMin;
        p.staged_etiles |= p.etbase[t + 1] - p.etbase[t] > kScanStagedMin;
        p.et_max = std::max(p.et_max, p.etbase[t + 1] - p.etbase[t]);
    }
    p.P = p.pbase[T];
    p.G = p.gbase[T];
    p.TT = p.tbase[T];
    p.A = p.obase[T];
    p.SL = p.slbase[T];
    p.S = p.sbase[T];
    p.E = p.ebase[T];
    p.ET = p.etbase[T];
    // norm chunks: the largest power of two in [2^12, 2^18] that still gives
    // 256 workgroups (one per CU), so a small gradient still spreads over the
    // chip (ResNet-50's 25.6M elements: 390 workgroups of 2^16, not 98)
    p.norm_chunk = kNormChunk;
    while (p.norm_chunk > kNormChunkMin && p.n / p.norm_chunk < 256) p.norm_chunk >>= 1;
    p.NB = cdiv(p.n, p.norm_chunk);
    p.AS = p.asbase[T];
    p.DB = p.dbase[T];
    p.NBLK = p.bbase[T];
    if (p.P >= (int64_t(1) << 32) || p.TT >= (int64_t(1) << 32)) return DGC_EINVAL;
    // tiles over k never exceed tiles over n, so TT also bounds encode tiles
    p.tiles = std::max<int64_t>(std::max<int64_t>(p.TT, p.ET), 1);
    p.pdesc.resize(size_t(p.P));
    p.smap.resize(size_t(p.S));
    p.emap.resize(size_t(p.ET));
    p.gmap.resize(size_t(p.G));
    for (int32_t t = 0; t < T; ++t) {
        for (int64_t i = p.pbase[t]; i < p.pbase[t + 1]; ++i) {
            PieceDesc& d = p.pdesc[size_t(i)];
            d.start = p.o[t] + (i - p.pbase[t]) * kPiece;
            d.tensor = uint32_t(t);
            d.len = uint32_t(std::min<int64_t>(kPiece, p.o[t + 1] - d.start));
        }
        for (int64_t i = p.sbase[t]; i < p.sbase[t + 1]; ++i) p.smap[size_t(i)] = uint32_t(t);
        for (int64_t i = p.etbase[t]; i < p.etbase[t + 1]; ++i) p.emap[size_t(i)] = uint32_t(t);
        for (int64_t i = p.gbase[t]; i < p.gbase[t + 1]; ++i) p.gmap[size_t(i)] = uint32_t(t);
    }
    p.asmap.resize(size_t(p.AS));
    for (int32_t t = 0; t < T; ++t)
        for (int64_t i = p.asbase[t]; i < p.asbase[t + 1]; ++i) p.asmap[size_t(i)] = uint32_t(t);
    p.bmap.resize(size_t(p.NBLK));
    for (int32_t t = 0; t < T; ++t)
        for (int64_t i = p.bbase[t]; i < p.bbase[t + 1]; ++i) p.bmap[size_t(i)] = uint32_t(t);
    // carve
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + std::max<size_t>(bytes, 1));
        return at;
    };
    const size_t T1 = size_t(T) + 1;
    p.off_tab = take(11 * T1 * sizeof(int64_t));
    p.off_pdesc = take(size_t(p.P) * sizeof(PieceDesc));
    p.off_smap = take(size_t(p.S) * 4);
    p.off_emap = take(size_t(p.ET) * 4);
    p.off_gmap = take(size_t(p.G) * 4);
    p.off_k = take((3 * T1) * sizeof(int64_t));
    p.off_kmap = take(size_t(p.TT) * 4);
    p.off_bltab = take(7 * T1 * sizeof(int64_t));
    p.off_astab = take(3 * T1 * sizeof(int64_t));
    p.off_asmap = take(size_t(p.AS) * 4);
    p.off_ktgt = take(T1 * sizeof(int64_t));
    p.off_dtab = take(2 * T1 * sizeof(int64_t));
    p.off_bmap = take(size_t(p.NBLK) * 4);
    // Everything above is written from the host (layout tables at init, k
    // tables per call); everything from here on is device scratch, zeroed
    // at init.
    p.off_scratch = off;
    p.off_ts = take(size_t(T) * sizeof(TensorState));
    p.off_sc = take(sizeof(Scalars));
    p.off_hist = take(size_t(T) * kHistBins * 4);
    p.off_shist = take(size_t(T) * kHistBins * 4);
    p.off_runc = take(size_t(p.P) * 4);
    p.off_gsum = take(size_t(p.G) * 4);
    p.off_goff = take(size_t(p.G) * 4);
    p.off_atiles = take(size_t(T) * 4);
    p.off_aoff = take(T1 * 4);
    p.off_amap = take(size_t(p.TT) * 4);
    p.off_slots = take(size_t(p.SL) * sizeof(CandSlot));
    p.off_olist = take(size_t(p.A) * 4);
    p.off_olistv = take(size_t(p.A) * 4);
    p.off_olistu = take(size_t(p.A) * 4);
    p.off_ta = take(size_t(p.tiles) * 4);
    p.off_tb = take(size_t(p.tiles) * 4);
    p.off_tc = take(size_t(p.tiles) * 4);
    p.off_t64 = take(size_t(p.tiles) * 8);
    p.off_part = take(size_t(std::max<int64_t>(p.NB, 1)) * 8);
    p.off_blpdesc = take(size_t(p.BP) * sizeof(PieceDesc));
    p.off_blcnt = take(size_t(p.BP) * 4);
    p.off_blpre = take(size_t(p.BP) * 4);
    p.off_blgsum = take(size_t(p.BG) * 4);
    p.off_blgoff = take(size_t(p.BG) * 4);
    p.off_dmode = take(size_t(T) * 4);
    p.off_bounds = take(size_t(kDecBatch) * size_t(p.DB) * sizeof(uint2));
    p.off_bsel = take(size_t(p.NBLK) * 4);
    p.total = off;
    return DGC_OK;
}

// ---------------------------------------------------------------- static scratch

// dgc_shared_sum_static keeps its per-call tables and its status latch in
// this file-scope device array instead of a workspace: kStaticMaxTensors
// tensors at most.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses the array's name as an address:
// the address on each device comes from hipGetSymbolAddress.
constexpr int32_t kStaticMaxTensors = 16384;
constexpr size_t kStaticTable = (size_t(kStaticMaxTensors + 1) * 8 + kAlign - 1) / kAlign * kAlign;
// Scalars (status latch), then sizes, k, o, koff, ktbase
constexpr size_t kStaticScratchBytes = kAlign + 5 * kStaticTable;
static_assert(sizeof(Scalars) <= kAlign, "scalars fit their slot");

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kStaticMaxDevices = 64;
struct StaticScratch {
    std::once_flag once;
    int rc = DGC_EHIP;
    char* ptr = nullptr;  // device address of `scratch` on this device
    int num_cus = 0;
};
StaticScratch g_static[kStaticMaxDevices];

// The device address of `scratch` on device `dev` (current), found once.
int static_scratch(int dev, char** ptr, int* num_cus) {
    if (dev < 0 || dev >= kStaticMaxDevices) return DGC_EINVAL;
    StaticScratch& S = g_static[dev];
    std::call_once(S.once, [&S, dev]() {
        void* p = nullptr;
        int cus = 0;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess)
            return;
        S.ptr = static_cast<char*>(p);
        S.num_cus = cus;
        S.rc = DGC_OK;
    });
    if (S.rc != DGC_OK) return S.rc;
    *ptr = S.ptr;
    *num_cus = S.num_cus;
    return DGC_OK;
}

// One block: the layout and k tables of a static call from the copied
// sizes and k (exclusive prefix sums), and the status latch cleared.
__global__ __launch_bounds__(kBlock) void k_static_tables(
    int32_t T, const int64_t* __restrict__ sz, const int64_t* __restrict__ kk,
    int64_t* __restrict__ o, int64_t* __restrict__ koff, int64_t* __restrict__ ktbase,
    Scalars* __restrict__ sc) {
    __shared__ int64_t lds[kWavesPerBlock];
    int64_t co = 0, ck = 0, ct = 0;
    for (int32_t base = 0; base < T; base += kBlock) {
        const int32_t t = base + int32_t(threadIdx.x);
        const int64_t n = t < T ? sz[t] : 0, k = t < T ? kk[t] : 0;
        const int64_t tiles = (k + kTile - 1) / kTile;
        int64_t to, tk, tt;
        const int64_t eo = block_exclusive_scan(n, lds, to);
        const int64_t ek = block_exclusive_scan(k, lds, tk);
        const int64_t et = block_exclusive_scan(tiles, lds, tt);
        if (t < T) {
            o[t] = co + eo;
            koff[t] = ck + ek;
            ktbase[t] = ct + et;
        }
        co += to;
        ck += tk;
        ct += tt;
    }
    if (threadIdx.x == 0) {
        o[T] = co;
        koff[T] = ck;
        ktbase[T] = ct;
        sc->status = 0;
    }
}

// The call's status for the caller: DGC_OK, or DGC_ECORRUPT when an index
// left its tensor.
__global__ void k_static_status(const Scalars* __restrict__ sc, int32_t* __restrict__ status) {
    if (threadIdx.x == 0)
        *status = sc->status == kErrCorrupt ? DGC_ECORRUPT : (sc->status ? DGC_EHIP : DGC_OK);
}

}  // namespace

// A ring of HIP event pairs bracketing one kind of work on the caller's
// stream.  A slot is read back (host wait) before it is reused.
struct Timer {
    static constexpr int kRing = 64;
    hipEvent_t start[kRing] = {};
    hipEvent_t stop[kRing] = {};
    bool busy[kRing] = {};
    bool created = false;
    int next = 0;
    int open = -1;
    double acc_ms = 0.0;
    int64_t count = 0;
};

struct dgc_state {
    Plan plan;
    int timing = 0;  // DGC_OPT_KERNEL_TIMING: 0 off, 1 every timer, 2 the element-wise pass
    Timer timers[4];
    float m = 0.9f;
    float* u = nullptr;
    float* v = nullptr;
    char* ws = nullptr;
    int num_cus = 256;
    int select_path = 0;
    int fused_blocks = 0;  // 0: automatic
    hipEvent_t fused_event = nullptr;  // recorded after the element-wise pass
    hipStream_t last_stream = nullptr;
    std::vector<int64_t> k_last;  // k of the last upload
    std::vector<int64_t> k_tables;  // k, koff, ktbase (host copy)
    std::vector<uint32_t> kmap_host;
    bool k_valid = false;
    int64_t KT = 0;  // tiles over k of the last upload
    int64_t kt_max = 0;  // most tiles over k of one tensor (last upload)
    std::vector<int64_t> bins_last;  // bin lengths of the last upload
    std::vector<int64_t> bl_tables;  // plen, magic, pbase, gbase, pcap, slbase, rbins (host)
    bool bins_valid = false;
    std::vector<int64_t> ktgt_last;  // target k of the last sampled call
    bool ktgt_valid = false;
    std::vector<int64_t> bins_full;  // one 1024-element bin per piece
    DevSample A{};
    const int64_t* wlines = nullptr;  // [T] lines the per-tensor window samples
    DevDec Dd{};
    int decode_path = 0;  // 0 automatic, 1 scattered, 2 merged, 3 scattered per tensor
    int encode_path = 0;  // 0 automatic, 1 a workgroup per tensor, 2 tiled passes
    int select_grid = 0;  // 0 automatic, 1 a workgroup per tensor, 2 spread passes
    bool staged_k = false;  // some tensor has more than kScanStagedMin k tiles
    int64_t BP = 0, BG = 0;  // bin-local pieces and groups of the last upload
    DevBins B{};
    // device views
    DevLayout L{};
    DevK K{};
    TensorState* ts = nullptr;
    Scalars* sc = nullptr;
    uint32_t *hist = nullptr, *shist = nullptr,
             *run_cnt = nullptr, *gsum = nullptr, *goff = nullptr, *atiles = nullptr,
             *aoff = nullptr, *amap = nullptr, *ta = nullptr, *tb = nullptr,
             *tc = nullptr;
    // 12-byte candidate slots {index, v, u}, shared by all three selectors
    CandSlot* slots = nullptr;
    // the ordered candidate list: local index, v and saved u per item
    uint32_t* olist_i = nullptr;
    float *olist_v = nullptr, *olist_u = nullptr;
    uint64_t* t64 = nullptr;
    double* partial = nullptr;
};

namespace {

int timer_collect(Timer& tm, int slot) {
    if (!tm.busy[slot]) return DGC_OK;
    if (hipEventSynchronize(tm.stop[slot]) != hipSuccess) return DGC_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, tm.start[slot], tm.stop[slot]) != hipSuccess)
        return DGC_EHIP;
    tm.acc_ms += ms;
    tm.count += 1;
    tm.busy[slot] = false;
    return DGC_OK;
}

bool timer_on(const dgc_state* st, int which) {
    return st->timing == 1 || (st->timing == 2 && which == DGC_TIMER_FUSED) ||
           (st->timing == 3 && which != DGC_TIMER_FUSED);
}

int timer_begin(dgc_state* st, int which, hipStream_t s) {
    if (!timer_on(st, which)) return DGC_OK;
    Timer& tm = st->timers[which];
    if (!tm.created) {
        for (int i = 0; i < Timer::kRing; ++i)
            if (hipEventCreate(&tm.start[i]) != hipSuccess ||
                hipEventCreate(&tm.stop[i]) != hipSuccess)
                return DGC_EHIP;
        tm.created = true;
    }
    int slot = tm.next;
    if (timer_collect(tm, slot) != DGC_OK) return DGC_EHIP;
    if (hipEventRecord(tm.start[slot], s) != hipSuccess) return DGC_EHIP;
    tm.open = slot;
    return DGC_OK;
}

int timer_end(dgc_state* st, int which, hipStream_t s) {
    if (!timer_on(st, which)) return DGC_OK;
    Timer& tm = st->timers[which];
    if (tm.open < 0) return DGC_OK;
    if (hipEventRecord(tm.stop[tm.open], s) != hipSuccess) return DGC_EHIP;
    tm.busy[tm.open] = true;
    tm.next = (tm.open + 1) % Timer::kRing;
    tm.open = -1;
    return DGC_OK;
}

void timers_destroy(dgc_state* st) {
    for (Timer& tm : st->timers) {
        if (!tm.created) continue;
        for (int i = 0; i < Timer::kRing; ++i) {
            (void)hipEventDestroy(tm.start[i]);
            (void)hipEventDestroy(tm.stop[i]);
        }
        tm.created = false;
    }
}

#define DGC_TRY(expr)                      \
    do {                                   \
        int rc_ = (expr);                  \
        if (rc_ != DGC_OK) return rc_;     \
    } while (0)

#define DGC_LAUNCH_CHECK()                                   \
    do {                                                     \
        if (hipGetLastError() != hipSuccess) return DGC_EHIP; \
    } while (0)

bool aligned(const void* p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

int grid_for(int64_t work, int64_t cap) {
    return int(std::max<int64_t>(1, std::min<int64_t>(work, cap)));
}

// Upload k, its output offsets and its tile map when they change.  Up to
// kKArgTensors tensors, k travels in the launch's arguments and one small
// kernel writes every table on the device (nothing waits on the host);
// larger layouts copy host-built tables (pageable copies, staged by the
// runtime before the call returns).
int upload_k(dgc_state* st, const int64_t* k, hipStream_t s) {
    const Plan& p = st->plan;
    const int32_t T = p.T;
    if (st->k_valid && std::memcmp(st->k_last.data(), k, size_t(T) * 8) == 0)
        return DGC_OK;
    st->k_last.assign(k, k + T);
    // tile counts on the host too: they size the later launches
    int64_t KT = 0;
    st->staged_k = false;
    st->kt_max = 0;
    for (int32_t t = 0; t < T; ++t) {
        const int64_t tiles = cdiv(k[t], kTile);
        st->staged_k |= tiles > kScanStagedMin;
        st->kt_max = std::max(st->kt_max, tiles);
        KT += tiles;
    }
    st->KT = KT;
    int64_t* dk = reinterpret_cast<int64_t*>(st->ws + p.off_k);
    if (T <= kKArgTensors) {
        KArgs a{};
        a.T = T;
        for (int32_t t = 0; t < T; ++t) a.k[t] = k[t];
        k_ktables<<<T, kBlock, 0, s>>>(a, dk, dk + (T + 1), dk + 2 * (T + 1),
                                       reinterpret_cast<uint32_t*>(st->ws + p.off_kmap));
        if (hipGetLastError() != hipSuccess) return DGC_EHIP;
        st->k_valid = true;
        return DGC_OK;
    }
    std::vector<int64_t>& tb = st->k_tables;
    tb.assign(3 * (size_t(T) + 1), 0);
    int64_t* kk = tb.data();
    int64_t* koff = kk + (T + 1);
    int64_t* ktb = koff + (T + 1);
    for (int32_t t = 0; t < T; ++t) {
        kk[t] = k[t];
        koff[t + 1] = koff[t] + k[t];
        ktb[t + 1] = ktb[t] + cdiv(k[t], kTile);
    }
    st->kmap_host.resize(size_t(std::max<int64_t>(st->KT, 1)));
    for (int32_t t = 0; t < T; ++t)
        for (int64_t i = ktb[t]; i < ktb[t + 1]; ++i) st->kmap_host[size_t(i)] = uint32_t(t);
    // Pageable-source copies are staged by the runtime before returning,
    // so the host vectors may change on the next call.
    if (hipMemcpyAsync(dk, tb.data(), tb.size() * 8, hipMemcpyHostToDevice, s) != hipSuccess)
        return DGC_EHIP;
    if (st->KT > 0 &&
        hipMemcpyAsync(st->ws + p.off_kmap, st->kmap_host.data(),
                       size_t(st->KT) * 4, hipMemcpyHostToDevice, s) != hipSuccess)
        return DGC_EHIP;
    st->k_valid = true;
    return DGC_OK;
}

int check_k(const dgc_state* st, const int64_t* k) {
    if (!k) return DGC_EINVAL;
    for (int32_t t = 0; t < st->plan.T; ++t)
        if (k[t] < 0 || k[t] > st->plan.kmax[size_t(t)]) return DGC_EINVAL;
    return DGC_OK;
}

int check_bins(const dgc_state* st, const int64_t* bin_len) {
    if (!bin_len) return DGC_EINVAL;
    for (int32_t t = 0; t < st->plan.T; ++t)
        if (bin_len[t] < 1 || bin_len[t] > kMaxBin) return DGC_EINVAL;
    return DGC_OK;
}

// Upload the bin-local tables for these bin lengths when they change, and
// rebuild the piece descriptors on the device.
int upload_bins(dgc_state* st, const int64_t* bin_len, hipStream_t s) {
    const Plan& p = st->plan;
    const int32_t T = p.T;
    DGC_TRY(check_bins(st, bin_len));
    if (st->bins_valid && std::memcmp(st->bins_last.data(), bin_len, size_t(T) * 8) == 0)
        return DGC_OK;
    const size_t T1 = size_t(T) + 1;
    std::vector<int64_t>& tb = st->bl_tables;
    tb.assign(7 * T1, 0);
    int64_t* plen = tb.data();
    int64_t* magic = plen + T1;
    int64_t* pbase = magic + T1;
    int64_t* gbase = pbase + T1;
    int64_t* pcap = gbase + T1;
    int64_t* slb = pcap + T1;
    int64_t* rbins = slb + T1;
    for (int32_t t = 0; t < T; ++t) {
        const int64_t Lb = bin_len[t], n = p.sizes[size_t(t)];
        plen[t] = Lb * (kMaxBin / Lb);
        magic[t] = Lb == 1 ? 0 : ((int64_t(1) << 32) + Lb - 1) / Lb;
        // bins of whole 256-element rounds of a 1024-element piece
        rbins[t] = (Lb == 256 || Lb == 512 || Lb == 1024) ? Lb / 256 : 0;
        // the multiply-high bin index must equal e / L on every offset
        for (int64_t e = 0; e < plen[t]; ++e)
            if (Lb > 1 && int64_t((uint64_t(e) * uint64_t(magic[t])) >> 32) != e / Lb)
                return DGC_EINVAL;
        const int64_t np_ = cdiv(n, plen[t]);
        pbase[t + 1] = pbase[t] + np_;
        gbase[t + 1] = gbase[t] + cdiv(np_, kBlGroup);
        // the tensor's candidate slots, shared out among its pieces
        slb[t] = p.slbase[size_t(t)];
        const int64_t region = p.slbase[size_t(t) + 1] - slb[t];
        pcap[t] = np_ ? std::min<int64_t>(plen[t], region / np_) : 0;
    }
    if (pbase[T] > p.BP || gbase[T] > p.BG) return DGC_EINVAL;
    if (hipMemcpyAsync(st->ws + p.off_bltab, tb.data(), tb.size() * 8,
                       hipMemcpyHostToDevice, s) != hipSuccess)
        return DGC_EHIP;
    st->BP = pbase[T];
    st->BG = gbase[T];
    if (st->BP > 0) {
        k_bl_pdesc<<<grid_for(cdiv(st->BP, kBlock), cdiv(st->BP, kBlock)), kBlock, 0, s>>>(
            st->L, st->B, st->BP);
        if (hipGetLastError() != hipSuccess) return DGC_EHIP;
    }
    st->bins_last.assign(bin_len, bin_len + T);
    st->bins_valid = true;
    return DGC_OK;
}

int encode_impl(dgc_state* st, const int64_t* k, const int64_t* kdev,
                const uint32_t* idx, const float* val, uint16_t* runs, float* vals,
                int64_t* entries, hipStream_t stream) {
    const Plan& p = st->plan;
    int rc = check_k(st, k);
    if (rc != DGC_OK) return rc;
    int64_t K = 0;
    for (int32_t t = 0; t < p.T; ++t) K += k[t];
    if (!entries || !aligned(entries, 8)) return DGC_EINVAL;
    if (K > 0 && (!idx || !val || !runs || !vals || !aligned(idx, 4) ||
                  !aligned(val, 4) || !aligned(runs, 2) || !aligned(vals, 4)))
        return DGC_EINVAL;
    rc = upload_k(st, k, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const int T = p.T;
    const int64_t pg = int64_t(st->num_cus) * kCodecBlocksPerCU;
    DGC_TRY(timer_begin(st, DGC_TIMER_ENCODE, stream));
    if (st->encode_path == 1 || (st->encode_path == 0 && st->kt_max <= kEncTensorTiles)) {
        k_enc_tensor<<<T, kBlock, 0, stream>>>(st->L, st->K, kdev, idx, val, runs, vals,
                                               entries, st->sc);
        DGC_LAUNCH_CHECK();
        DGC_TRY(timer_end(st, DGC_TIMER_ENCODE, stream));
        return DGC_OK;
    }
    if (st->KT > 0)
        k_enc_count<<<grid_for(st->KT, pg), kBlock, 0, stream>>>(st->L, st->K, kdev, idx,
                                                                 st->ta, st->sc, st->KT);
    if (st->staged_k)
        k_enc_scan<true><<<T, kBlock, 0, stream>>>(st->K, kdev, st->ta, st->tb, entries,
                                                   st->sc);
    else
        k_enc_scan<false><<<T, kBlock, 0, stream>>>(st->K, kdev, st->ta, st->tb,
                                                    entries, st->sc);
    if (st->KT > 0)
        k_enc_write<<<grid_for(st->KT, pg), kBlock, 0, stream>>>(
            st->L, st->K, kdev, idx, val, st->tb, runs, vals, st->sc, st->KT);
    DGC_LAUNCH_CHECK();
    DGC_TRY(timer_end(st, DGC_TIMER_ENCODE, stream));
    return DGC_OK;
}

}  // namespace

extern "C" {

int64_t dgc_k_for_density(int64_t n, int64_t num, int64_t den) {
    if (n < 0 || den < 1 || num < 0 || num > den) return DGC_EINVAL;
    const __int128 p = __int128(n) * num;
    return int64_t((p + den - 1) / den);  // <= n because num <= den
}

int dgc_workspace_bytes(int32_t n_tensors, const int64_t* sizes,
                        const int64_t* k_max, size_t* bytes) {
    if (!bytes) return DGC_EINVAL;
    Plan p;
    int rc = make_plan(n_tensors, sizes, k_max, p);
    if (rc != DGC_OK) return rc;
    *bytes = p.total;
    return DGC_OK;
}

int dgc_init_state(dgc_state** out, int32_t n_tensors, const int64_t* sizes,
                   const int64_t* k_max, float momentum, float* u, float* v,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    if (!out) return DGC_EINVAL;
    *out = nullptr;
    dgc_state* st = new (std::nothrow) dgc_state;
    if (!st) return DGC_EINVAL;
    int rc = make_plan(n_tensors, sizes, k_max, st->plan);
    const Plan& p = st->plan;
    if (rc == DGC_OK && (!workspace || !aligned(workspace, kAlign))) rc = DGC_EINVAL;
    if (rc == DGC_OK && p.n > 0 && (!u || !v || !aligned(u, 16) || !aligned(v, 16)))
        rc = DGC_EINVAL;
    if (rc == DGC_OK && workspace_bytes < p.total) rc = DGC_ECAPACITY;
    if (!std::isfinite(momentum)) rc = DGC_EINVAL;
    if (rc != DGC_OK) {
        delete st;
        return rc;
    }
    st->m = momentum;
    st->u = u;
    st->v = v;
    st->ws = static_cast<char*>(workspace);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&st->num_cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess) {
        delete st;
        return DGC_EHIP;
    }
    char* ws = st->ws;
    const int32_t T = p.T;
    const size_t T1 = size_t(T) + 1;
    // layout tables
    std::vector<int64_t> tab(11 * T1, 0);
    const std::vector<int64_t>* src[11] = {&p.o,      &p.pbase,  &p.tbase, &p.obase,
                                           &p.sbase,  &p.slines, &p.ebase, &p.etbase,
                                           &p.slbase, &p.pcap,   &p.gbase};
    for (int i = 0; i < 11; ++i)
        std::copy(src[i]->begin(), src[i]->end(), tab.begin() + i * T1);
    int64_t* dtab = reinterpret_cast<int64_t*>(ws + p.off_tab);
    st->L.T = T;
    st->L.o = dtab;
    st->L.pbase = dtab + T1;
    st->L.tbase = dtab + 2 * T1;
    st->L.obase = dtab + 3 * T1;
    st->L.sbase = dtab + 4 * T1;
    st->L.slines = dtab + 5 * T1;
    st->L.ebase = dtab + 6 * T1;
    st->L.etbase = dtab + 7 * T1;
    st->L.slbase = dtab + 8 * T1;
    st->L.pcap = dtab + 9 * T1;
    st->L.gbase = dtab + 10 * T1;
    st->L.gmap = reinterpret_cast<uint32_t*>(ws + p.off_gmap);
    st->L.pdesc = reinterpret_cast<PieceDesc*>(ws + p.off_pdesc);
    st->L.smap = reinterpret_cast<uint32_t*>(ws + p.off_smap);
    st->L.emap = reinterpret_cast<uint32_t*>(ws + p.off_emap);
    int64_t* dk = reinterpret_cast<int64_t*>(ws + p.off_k);
    st->K.k = dk;
    st->K.koff = dk + T1;
    st->K.ktbase = dk + 2 * T1;
    st->K.kmap = reinterpret_cast<uint32_t*>(ws + p.off_kmap);
    st->ts = reinterpret_cast<TensorState*>(ws + p.off_ts);
    st->sc = reinterpret_cast<Scalars*>(ws + p.off_sc);
    st->hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
    st->shist = reinterpret_cast<uint32_t*>(ws + p.off_shist);
    st->run_cnt = reinterpret_cast<uint32_t*>(ws + p.off_runc);
    st->gsum = reinterpret_cast<uint32_t*>(ws + p.off_gsum);
    st->goff = reinterpret_cast<uint32_t*>(ws + p.off_goff);
    st->atiles = reinterpret_cast<uint32_t*>(ws + p.off_atiles);
    st->aoff = reinterpret_cast<uint32_t*>(ws + p.off_aoff);
    st->amap = reinterpret_cast<uint32_t*>(ws + p.off_amap);
    st->slots = reinterpret_cast<CandSlot*>(ws + p.off_slots);
    st->olist_i = reinterpret_cast<uint32_t*>(ws + p.off_olist);
    st->olist_v = reinterpret_cast<float*>(ws + p.off_olistv);
    st->olist_u = reinterpret_cast<float*>(ws + p.off_olistu);
    st->ta = reinterpret_cast<uint32_t*>(ws + p.off_ta);
    st->tb = reinterpret_cast<uint32_t*>(ws + p.off_tb);
    st->tc = reinterpret_cast<uint32_t*>(ws + p.off_tc);
    st->t64 = reinterpret_cast<uint64_t*>(ws + p.off_t64);
    st->partial = reinterpret_cast<double*>(ws + p.off_part);
    int64_t* bt = reinterpret_cast<int64_t*>(ws + p.off_bltab);
    st->B.plen = bt;
    st->B.magic = bt + T1;
    st->B.pbase = bt + 2 * T1;
    st->B.gbase = bt + 3 * T1;
    st->B.pcap = bt + 4 * T1;
    st->B.slbase = bt + 5 * T1;
    st->B.rbins = bt + 6 * T1;
    int64_t* at = reinterpret_cast<int64_t*>(ws + p.off_astab);
    st->A.slines = at;
    st->A.sbase = at + T1;
    st->wlines = at + 2 * T1;
    st->A.smap = reinterpret_cast<uint32_t*>(ws + p.off_asmap);
    st->bins_full.assign(size_t(T), kMaxBin);
    int64_t* dt = reinterpret_cast<int64_t*>(ws + p.off_dtab);
    st->Dd.dbase = dt;
    st->Dd.bbase = dt + T1;
    st->Dd.bmap = reinterpret_cast<uint32_t*>(ws + p.off_bmap);
    st->Dd.bsel = reinterpret_cast<uint32_t*>(ws + p.off_bsel);
    st->Dd.dmode = reinterpret_cast<uint32_t*>(ws + p.off_dmode);
    st->Dd.bounds = reinterpret_cast<uint2*>(ws + p.off_bounds);
    st->Dd.DB = p.DB;
    st->B.pdesc = reinterpret_cast<PieceDesc*>(ws + p.off_blpdesc);
    st->B.cnt = reinterpret_cast<uint32_t*>(ws + p.off_blcnt);
    st->B.pre = reinterpret_cast<uint32_t*>(ws + p.off_blpre);
    st->B.gsum = reinterpret_cast<uint32_t*>(ws + p.off_blgsum);
    st->B.goff = reinterpret_cast<uint32_t*>(ws + p.off_blgoff);

    // the uploaded tables must not lie in the scratch zeroed below
    if (p.off_pdesc >= p.off_scratch || p.off_smap >= p.off_scratch ||
        p.off_emap >= p.off_scratch || p.off_gmap >= p.off_scratch ||
        p.off_k >= p.off_scratch || p.off_kmap >= p.off_scratch ||
        p.off_tab >= p.off_scratch || p.off_bltab >= p.off_scratch ||
        p.off_astab >= p.off_scratch || p.off_asmap >= p.off_scratch ||
        p.off_ktgt >= p.off_scratch || p.off_dtab >= p.off_scratch ||
        p.off_bmap >= p.off_scratch) {
        delete st;
        return DGC_EINVAL;
    }
    bool ok = true;
    ok = ok && hipMemcpyAsync(dtab, tab.data(), tab.size() * 8,
                              hipMemcpyHostToDevice, stream) == hipSuccess;
    if (p.P) ok = ok && hipMemcpyAsync(ws + p.off_pdesc, p.pdesc.data(),
                                       size_t(p.P) * sizeof(PieceDesc),
                                       hipMemcpyHostToDevice, stream) == hipSuccess;
    if (p.S) ok = ok && hipMemcpyAsync(ws + p.off_smap, p.smap.data(), size_t(p.S) * 4,
                                       hipMemcpyHostToDevice, stream) == hipSuccess;
    if (p.ET) ok = ok && hipMemcpyAsync(ws + p.off_emap, p.emap.data(), size_t(p.ET) * 4,
                                        hipMemcpyHostToDevice, stream) == hipSuccess;
    if (p.G) ok = ok && hipMemcpyAsync(ws + p.off_gmap, p.gmap.data(), size_t(p.G) * 4,
                                       hipMemcpyHostToDevice, stream) == hipSuccess;
    if (p.NBLK) ok = ok && hipMemcpyAsync(ws + p.off_bmap, p.bmap.data(), size_t(p.NBLK) * 4,
                                          hipMemcpyHostToDevice, stream) == hipSuccess;
    std::vector<int64_t> atab(3 * T1, 0);
    std::copy(p.aslines.begin(), p.aslines.end(), atab.begin());
    std::copy(p.asbase.begin(), p.asbase.end(), atab.begin() + T1);
    std::copy(p.wlines.begin(), p.wlines.end(), atab.begin() + 2 * T1);
    ok = ok && hipMemcpyAsync(at, atab.data(), atab.size() * 8, hipMemcpyHostToDevice,
                              stream) == hipSuccess;
    if (p.AS) ok = ok && hipMemcpyAsync(ws + p.off_asmap, p.asmap.data(), size_t(p.AS) * 4,
                                        hipMemcpyHostToDevice, stream) == hipSuccess;
    std::vector<int64_t> dec_tab(2 * T1, 0);
    std::copy(p.dbase.begin(), p.dbase.end(), dec_tab.begin());
    std::copy(p.bbase.begin(), p.bbase.end(), dec_tab.begin() + T1);
    ok = ok && hipMemcpyAsync(dt, dec_tab.data(), dec_tab.size() * 8, hipMemcpyHostToDevice,
                              stream) == hipSuccess;
    // zero the scratch after the tables (histograms must start at zero) and
    // the state vectors u and v
    if (ok) {
        size_t zero_from = p.off_scratch;
        int64_t words = int64_t((p.total - zero_from) / 4);
        k_fill_u32<<<grid_for(cdiv(words, kBlock), 4096), kBlock, 0, stream>>>(
            reinterpret_cast<uint32_t*>(ws + zero_from), words, 0u);
        if (p.n) {
            k_fill_u32<<<grid_for(cdiv(p.n, kBlock), 8192), kBlock, 0, stream>>>(
                reinterpret_cast<uint32_t*>(u), p.n, 0u);
            k_fill_u32<<<grid_for(cdiv(p.n, kBlock), 8192), kBlock, 0, stream>>>(
                reinterpret_cast<uint32_t*>(v), p.n, 0u);
        }
        ok = hipGetLastError() == hipSuccess;
    }
    ok = ok && hipStreamSynchronize(stream) == hipSuccess;
    if (!ok) {
        delete st;
        return DGC_EHIP;
    }
    st->last_stream = stream;
    *out = st;
    return DGC_OK;
}

// The select and emit after the element-wise pass on the spread path:
// candidate totals and sources, the gather, then either one workgroup per
// tensor (every selection source short) or passes spread over the chip.
// With out_count set, each tensor's sent count is written too (zeros when
// every k is 0).
static int enqueue_select(dgc_state* st, int64_t K, uint32_t* out_idx, float* out_val,
                   int64_t* out_count, hipStream_t stream) {
    const Plan& p = st->plan;
    const int T = p.T;
    const int pg = st->num_cus * 8;  // persistent grids
    if (p.G > 0)
        k_group_sum<<<int(p.G), kBlock, 0, stream>>>(st->L, st->run_cnt, st->gsum);
    k_group_scan<<<T, kBlock, 0, stream>>>(st->L, st->K, st->ts, st->gsum, st->goff,
                                           st->atiles);
    // the select and emit: one workgroup per tensor when asked for, else
    // passes spread over the chip
    const bool per_tensor = st->select_grid == 1;
    // for the spread passes the gather also histograms the lists' top 21
    // bits, which k_resolve21 turns into T's top 21 bits where it can
    // at an average density of 1/8 or more the pieces hold long runs: the
    // gather copies them run by run, several workgroups per group
    const int runs = K * kGatherRunDensity >= p.n ? 1 : 0;
    const int split = runs ? kGatherSplit : 1;
    if (p.G > 0)
        k_gather<<<int(p.G * split), kBlock, 0, stream>>>(
            st->L, st->ts, st->slots, st->run_cnt, st->goff, st->olist_i, st->olist_v,
            st->olist_u, st->u, st->v, per_tensor ? nullptr : st->hist, split, runs);
    if (K > 0 && per_tensor) {
        k_select_tensor<<<T, kTsThreads, 0, stream>>>(
            st->L, st->K, st->ts, st->u, st->v, st->olist_i, st->olist_v, st->olist_u,
            out_idx, out_val, out_count, st->sc);
        DGC_LAUNCH_CHECK();
    } else if (K > 0) {
        k_resolve21<<<T, kBlock, 0, stream>>>(st->ts, st->hist);
        k_active_scan<<<1, kBlock, 0, stream>>>(T, st->atiles, st->aoff);
        k_active_map<<<T, kBlock, 0, stream>>>(st->atiles, st->aoff, st->amap);
        DGC_LAUNCH_CHECK();
        const int hg = grid_for(p.TT, pg);
        k_hist<0><<<hg, kBlock, 0, stream>>>(st->L, st->ts, st->v, st->olist_v, st->amap,
                                             st->aoff, st->hist);
        k_resolve<0><<<T, kBlock, 0, stream>>>(st->ts, st->hist, st->sc);
        k_hist<1><<<hg, kBlock, 0, stream>>>(st->L, st->ts, st->v, st->olist_v, st->amap,
                                             st->aoff, st->hist);
        k_resolve<1><<<T, kBlock, 0, stream>>>(st->ts, st->hist, st->sc);
        k_hist<2><<<hg, kBlock, 0, stream>>>(st->L, st->ts, st->v, st->olist_v, st->amap,
                                             st->aoff, st->hist);
        k_resolve<2><<<T, kBlock, 0, stream>>>(st->ts, st->hist, st->sc);
        DGC_LAUNCH_CHECK();
        k_emit_count<<<hg, kBlock, 0, stream>>>(st->L, st->ts, st->v, st->olist_v,
                                                st->amap, st->aoff, st->ta);
        if (p.staged_tiles)
            k_emit_scan<true><<<T, kBlock, 0, stream>>>(st->aoff, st->ta, st->tb, st->tc,
                                                        st->ts, out_count);
        else
            k_emit_scan<false><<<T, kBlock, 0, stream>>>(st->aoff, st->ta, st->tb, st->tc,
                                                         st->ts, out_count);
        k_emit_write<<<hg, kBlock, 0, stream>>>(st->L, st->K, st->ts, st->u, st->v,
                                                st->olist_i, st->olist_v, st->olist_u, st->amap,
                                                st->aoff, st->tb, st->tc, out_idx,
                                                out_val, st->sc);
        DGC_LAUNCH_CHECK();
    }
    if (K == 0 && out_count)
        k_fill_u32<<<grid_for(cdiv(2 * int64_t(T), kBlock), 64), kBlock, 0, stream>>>(
            reinterpret_cast<uint32_t*>(out_count), 2 * int64_t(T), 0u);
    DGC_LAUNCH_CHECK();
    return DGC_OK;
}

int dgc_compress(dgc_state* st, const float* g, const int64_t* k, double clip,
                 uint32_t* out_idx, float* out_val, double* out_norm,
                 float* out_scale, hipStream_t stream) {
    if (!st) return DGC_EINVAL;
    const Plan& p = st->plan;
    int rc = check_k(st, k);
    if (rc != DGC_OK) return rc;
    int64_t K = 0;
    for (int32_t t = 0; t < p.T; ++t) K += k[t];
    if (p.n > 0 && (!g || !aligned(g, 16))) return DGC_EINVAL;
    if (K > 0 && (!out_idx || !out_val || !aligned(out_idx, 4) || !aligned(out_val, 4)))
        return DGC_EINVAL;
    if (std::isnan(clip)) return DGC_EINVAL;
    rc = upload_k(st, k, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const int T = p.T;
    const bool clip_on = clip > 0.0;

    DGC_TRY(timer_begin(st, DGC_TIMER_COMPRESS, stream));
    const int force_dense = st->select_path == 1;
    if (p.tensor_path && st->select_grid != 2) {
        // per-tensor kernels: norm partials, window, element-wise pass, finish
        if (clip_on)
            k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                       st->partial);
        k_window_tensor<<<T, kTsThreads, 0, stream>>>(
            g, st->u, st->v, st->L, st->K, st->wlines, st->partial, p.NB, clip, int(clip_on),
            st->sc, out_norm, out_scale, st->ts, st->m, force_dense);
        DGC_LAUNCH_CHECK();
        if (p.P > 0) {
            int64_t fb = st->fused_blocks > 0 ? st->fused_blocks : cdiv(p.P, kWavesPerBlock);
            DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
            k_fused<<<grid_for(cdiv(p.P, kWavesPerBlock), fb), kBlock, 0, stream>>>(
                g, st->u, st->v, st->L, st->ts, st->sc, clip_on, st->m, st->slots,
                st->run_cnt, p.P, out_norm, out_scale);
            DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
        }
        if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
            return DGC_EHIP;
        k_finish_tensor<<<T, kTsThreads, 0, stream>>>(
            st->L, st->K, st->ts, st->slots, st->run_cnt, st->u, st->v, st->olist_i,
            st->olist_v, st->olist_u, out_idx, out_val, nullptr, st->sc);
        DGC_LAUNCH_CHECK();
        DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
        return DGC_OK;
    }
    if (clip_on) {
        k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                   st->partial);
        k_norm_final<<<1, kBlock, 0, stream>>>(st->partial, p.NB, clip, st->sc,
                                               out_norm, out_scale);
    } else if (p.P == 0) {
        k_set_scalars<<<1, 64, 0, stream>>>(st->sc, out_norm, out_scale);
    }
    DGC_LAUNCH_CHECK();
    if (p.S > 0 && !force_dense)
        k_sample<0><<<int(p.S), kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->sc,
                                                     clip_on, st->ts, st->m, st->shist);
    k_window<0><<<T, kBlock, 0, stream>>>(st->L, st->K, st->shist, st->ts, force_dense);
    if (p.S > 0 && !force_dense) {
        k_sample<1><<<int(p.S), kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->sc,
                                                     clip_on, st->ts, st->m, st->shist);
        k_window<1><<<T, kBlock, 0, stream>>>(st->L, st->K, st->shist, st->ts,
                                              force_dense);
    }
    DGC_LAUNCH_CHECK();
    if (p.P > 0) {
        // one piece per wave unless a grid cap is set (then waves loop)
        int64_t fb = st->fused_blocks > 0 ? st->fused_blocks : cdiv(p.P, kWavesPerBlock);
        DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
        k_fused<<<grid_for(cdiv(p.P, kWavesPerBlock), fb), kBlock, 0, stream>>>(
            g, st->u, st->v, st->L, st->ts, st->sc, clip_on, st->m, st->slots,
            st->run_cnt, p.P, out_norm, out_scale);
        DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
    }
    if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
        return DGC_EHIP;
    DGC_TRY(enqueue_select(st, K, out_idx, out_val, nullptr, stream));
    DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
    return DGC_OK;
}

int dgc_compress_binlocal(dgc_state* st, const float* g, const int64_t* bin_len,
                          const int64_t* cap, double clip, uint32_t* out_idx,
                          float* out_val, int64_t* out_count, int64_t* out_total,
                          double* out_norm, float* out_scale, hipStream_t stream) {
    if (!st) return DGC_EINVAL;
    const Plan& p = st->plan;
    int rc = check_k(st, cap);
    if (rc != DGC_OK) return rc;
    DGC_TRY(check_bins(st, bin_len));
    int64_t C = 0;
    for (int32_t t = 0; t < p.T; ++t) C += cap[t];
    if (p.n > 0 && (!g || !aligned(g, 16))) return DGC_EINVAL;
    if (C > 0 && (!out_idx || !out_val || !aligned(out_idx, 4) || !aligned(out_val, 4)))
        return DGC_EINVAL;
    if (!out_count || !aligned(out_count, 8)) return DGC_EINVAL;
    if (out_total && !aligned(out_total, 8)) return DGC_EINVAL;
    if (std::isnan(clip)) return DGC_EINVAL;
    rc = upload_k(st, cap, stream);
    if (rc != DGC_OK) return rc;
    rc = upload_bins(st, bin_len, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const int T = p.T;
    const bool clip_on = clip > 0.0;
    const uint32_t pcap_limit = st->select_path == 1 ? 0u : 0xFFFFFFFFu;

    DGC_TRY(timer_begin(st, DGC_TIMER_COMPRESS, stream));
    if (clip_on) {
        k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                   st->partial);
        k_norm_final<<<1, kBlock, 0, stream>>>(st->partial, p.NB, clip, st->sc,
                                               out_norm, out_scale);
    } else if (st->BP == 0) {
        k_set_scalars<<<1, 64, 0, stream>>>(st->sc, out_norm, out_scale);
    }
    DGC_LAUNCH_CHECK();
    const int64_t wb = cdiv(st->BP, kWavesPerBlock);  // one piece per wave
    if (st->BP > 0) {
        DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
        k_bl_fused<kSelBins><<<grid_for(wb, wb), kBlock, 0, stream>>>(
            g, st->u, st->v, st->L, st->B, st->ts, st->sc, clip_on, st->m, pcap_limit,
            st->slots, st->BP, out_norm, out_scale);
        DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
    }
    if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
        return DGC_EHIP;
    if (st->BG > 0) {
        const int64_t gb = cdiv(st->BG, kWavesPerBlock);
        k_bl_group<<<grid_for(gb, gb), kBlock, 0, stream>>>(st->L, st->B, st->BG);
    }
    k_bl_tscan<<<T, kBlock, 0, stream>>>(st->K, st->B, out_count, out_total);
    // also with every cap 0: entries masked in the element-wise pass that
    // are not delivered get their u and v back here
    if (st->BP > 0) {
        const int64_t gb = cdiv(st->BP, int64_t(kBlock));  // kWave pieces per wave
        k_bl_gather<kSelBins><<<grid_for(gb, gb), kBlock, 0, stream>>>(
            st->u, st->v, st->L, st->K, st->B, st->ts, pcap_limit,
            st->slots, st->BP, out_idx, out_val);
    }
    DGC_LAUNCH_CHECK();
    DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
    return DGC_OK;
}

int dgc_compress_sampled(dgc_state* st, const float* g, const int64_t* k,
                         const int64_t* cap, double clip, uint32_t* out_idx,
                         float* out_val, int64_t* out_count, int64_t* out_total,
                         double* out_norm, float* out_scale, hipStream_t stream) {
    if (!st || !k) return DGC_EINVAL;
    const Plan& p = st->plan;
    const int T = p.T;
    for (int32_t t = 0; t < T; ++t)
        if (k[t] < 0 || k[t] > p.sizes[size_t(t)]) return DGC_EINVAL;
    int rc = check_k(st, cap);
    if (rc != DGC_OK) return rc;
    int64_t C = 0;
    for (int32_t t = 0; t < T; ++t) C += cap[t];
    if (p.n > 0 && (!g || !aligned(g, 16))) return DGC_EINVAL;
    if (C > 0 && (!out_idx || !out_val || !aligned(out_idx, 4) || !aligned(out_val, 4)))
        return DGC_EINVAL;
    if (!out_count || !aligned(out_count, 8)) return DGC_EINVAL;
    if (out_total && !aligned(out_total, 8)) return DGC_EINVAL;
    if (std::isnan(clip)) return DGC_EINVAL;
    if (!st->ktgt_valid || std::memcmp(st->ktgt_last.data(), k, size_t(T) * 8) != 0) {
        st->ktgt_last.assign(k, k + T);
        if (hipMemcpyAsync(st->ws + p.off_ktgt, st->ktgt_last.data(), size_t(T) * 8,
                           hipMemcpyHostToDevice, stream) != hipSuccess)
            return DGC_EHIP;
        st->ktgt_valid = true;
    }
    rc = upload_k(st, cap, stream);
    if (rc != DGC_OK) return rc;
    rc = upload_bins(st, st->bins_full.data(), stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const bool clip_on = clip > 0.0;
    const uint32_t pcap_limit = st->select_path == 1 ? 0u : 0xFFFFFFFFu;
    const int64_t* ktgt = reinterpret_cast<const int64_t*>(st->ws + p.off_ktgt);

    DGC_TRY(timer_begin(st, DGC_TIMER_COMPRESS, stream));
    if (clip_on) {
        k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                   st->partial);
        k_norm_final<<<1, kBlock, 0, stream>>>(st->partial, p.NB, clip, st->sc,
                                               out_norm, out_scale);
    } else if (st->BP == 0) {
        k_set_scalars<<<1, 64, 0, stream>>>(st->sc, out_norm, out_scale);
    }
    // the threshold: three histogram levels over the sample
    const int AS = int(p.AS);
    if (AS > 0)
        k_sm_hist<0><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<0><<<T, kBlock, 0, stream>>>(st->L, ktgt, st->shist, st->ts, 0);
    if (AS > 0)
        k_sm_hist<1><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<1><<<T, kBlock, 0, stream>>>(st->L, ktgt, st->shist, st->ts, 0);
    if (AS > 0)
        k_sm_hist<2><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<2><<<T, kBlock, 0, stream>>>(st->L, ktgt, st->shist, st->ts, 0);
    DGC_LAUNCH_CHECK();
    const int64_t wb = cdiv(st->BP, kWavesPerBlock);  // one piece per wave
    if (st->BP > 0) {
        DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
        k_bl_fused<kSelThresh><<<grid_for(wb, wb), kBlock, 0, stream>>>(
            g, st->u, st->v, st->L, st->B, st->ts, st->sc, clip_on, st->m, pcap_limit,
            st->slots, st->BP, out_norm, out_scale);
        DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
    }
    if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
        return DGC_EHIP;
    if (st->BG > 0) {
        const int64_t gb = cdiv(st->BG, kWavesPerBlock);
        k_bl_group<<<grid_for(gb, gb), kBlock, 0, stream>>>(st->L, st->B, st->BG);
    }
    k_bl_tscan<<<T, kBlock, 0, stream>>>(st->K, st->B, out_count, out_total);
    if (st->BP > 0) {
        const int64_t gb = cdiv(st->BP, int64_t(kBlock));
        k_bl_gather<kSelThresh><<<grid_for(gb, gb), kBlock, 0, stream>>>(
            st->u, st->v, st->L, st->K, st->B, st->ts, pcap_limit,
            st->slots, st->BP, out_idx, out_val);
    }
    DGC_LAUNCH_CHECK();
    DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
    return DGC_OK;
}

int dgc_compress_hier(dgc_state* st, const float* g, const int64_t* k, double clip,
                      uint32_t* out_idx, float* out_val, int64_t* out_count,
                      double* out_norm, float* out_scale, hipStream_t stream) {
    if (!st) return DGC_EINVAL;
    const Plan& p = st->plan;
    int rc = check_k(st, k);
    if (rc != DGC_OK) return rc;
    int64_t K = 0;
    for (int32_t t = 0; t < p.T; ++t) K += k[t];
    if (p.n > 0 && (!g || !aligned(g, 16))) return DGC_EINVAL;
    if (K > 0 && (!out_idx || !out_val || !aligned(out_idx, 4) || !aligned(out_val, 4)))
        return DGC_EINVAL;
    if (!out_count || !aligned(out_count, 8)) return DGC_EINVAL;
    if (std::isnan(clip)) return DGC_EINVAL;
    rc = upload_k(st, k, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const int T = p.T;
    const bool clip_on = clip > 0.0;
    // 2: the forced whole-tensor path (no candidates, the floor still set)
    const int hier = st->select_path == 1 ? 2 : 1;

    DGC_TRY(timer_begin(st, DGC_TIMER_COMPRESS, stream));
    if (clip_on) {
        k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                   st->partial);
        k_norm_final<<<1, kBlock, 0, stream>>>(st->partial, p.NB, clip, st->sc,
                                               out_norm, out_scale);
    } else if (p.P == 0) {
        k_set_scalars<<<1, 64, 0, stream>>>(st->sc, out_norm, out_scale);
    }
    // level 1: the sampled threshold, three histogram levels over the sample
    const int AS = int(p.AS);
    if (AS > 0)
        k_sm_hist<0><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<0><<<T, kBlock, 0, stream>>>(st->L, st->K.k, st->shist, st->ts, hier);
    if (AS > 0)
        k_sm_hist<1><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<1><<<T, kBlock, 0, stream>>>(st->L, st->K.k, st->shist, st->ts, hier);
    if (AS > 0)
        k_sm_hist<2><<<AS, kBlock, 0, stream>>>(g, st->u, st->v, st->L, st->A, st->sc,
                                                clip_on, st->ts, st->m, st->shist);
    k_sm_pick<2><<<T, kBlock, 0, stream>>>(st->L, st->K.k, st->shist, st->ts, hier);
    DGC_LAUNCH_CHECK();
    // the element-wise pass: the survivors are the candidates
    if (p.P > 0) {
        int64_t fb = st->fused_blocks > 0 ? st->fused_blocks : cdiv(p.P, kWavesPerBlock);
        DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
        k_fused<<<grid_for(cdiv(p.P, kWavesPerBlock), fb), kBlock, 0, stream>>>(
            g, st->u, st->v, st->L, st->ts, st->sc, clip_on, st->m, st->slots,
            st->run_cnt, p.P, out_norm, out_scale);
        DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
    }
    if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
        return DGC_EHIP;
    // level 2: the exact select of k among them, or all of at most k
    if (p.tensor_path && st->select_grid != 2) {
        k_finish_tensor<<<T, kTsThreads, 0, stream>>>(
            st->L, st->K, st->ts, st->slots, st->run_cnt, st->u, st->v, st->olist_i,
            st->olist_v, st->olist_u, out_idx, out_val, out_count, st->sc);
        DGC_LAUNCH_CHECK();
    } else {
        DGC_TRY(enqueue_select(st, K, out_idx, out_val, out_count, stream));
    }
    DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
    return DGC_OK;
}

int dgc_compress_shared(dgc_state* st, const float* g, const int64_t* k,
                        const uint32_t* shared_idx, double clip, float* out_val,
                        double* out_norm, float* out_scale, hipStream_t stream) {
    if (!st) return DGC_EINVAL;
    const Plan& p = st->plan;
    int rc = check_k(st, k);
    if (rc != DGC_OK) return rc;
    int64_t K = 0;
    for (int32_t t = 0; t < p.T; ++t) K += k[t];
    if (p.n > 0 && (!g || !aligned(g, 16))) return DGC_EINVAL;
    if (K > 0 && (!shared_idx || !out_val || !aligned(shared_idx, 4) || !aligned(out_val, 4)))
        return DGC_EINVAL;
    if (std::isnan(clip)) return DGC_EINVAL;
    rc = upload_k(st, k, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    const bool clip_on = clip > 0.0;
    DGC_TRY(timer_begin(st, DGC_TIMER_COMPRESS, stream));
    if (clip_on) {
        k_norm_partial<<<grid_for(p.NB, p.NB), kBlock, 0, stream>>>(g, p.n, p.norm_chunk,
                                                                   st->partial);
        k_norm_final<<<1, kBlock, 0, stream>>>(st->partial, p.NB, clip, st->sc,
                                               out_norm, out_scale);
    } else if (p.P == 0) {
        k_set_scalars<<<1, 64, 0, stream>>>(st->sc, out_norm, out_scale);
    }
    DGC_LAUNCH_CHECK();
    if (p.P > 0) {
        // the pieces' shared runs go where dgc_compress keeps its candidate
        // counts (one 32-bit word per piece)
        k_sh_poff<<<grid_for(cdiv(p.P, kBlock), cdiv(p.P, kBlock)), kBlock, 0, stream>>>(
            st->L, st->K, shared_idx, st->run_cnt, p.P);
        DGC_TRY(timer_begin(st, DGC_TIMER_FUSED, stream));
        k_sh_fused<<<grid_for(cdiv(p.P, kWavesPerBlock), cdiv(p.P, kWavesPerBlock)), kBlock, 0,
                     stream>>>(g, st->u, st->v, st->L, st->K, st->sc, clip_on, st->m,
                               shared_idx, st->run_cnt, out_val, p.P, out_norm, out_scale);
        DGC_TRY(timer_end(st, DGC_TIMER_FUSED, stream));
    }
    DGC_LAUNCH_CHECK();
    if (st->fused_event && hipEventRecord(st->fused_event, stream) != hipSuccess)
        return DGC_EHIP;
    DGC_TRY(timer_end(st, DGC_TIMER_COMPRESS, stream));
    return DGC_OK;
}

int dgc_shared_sum(const dgc_state* cst, int32_t n_learners, const float* const* vals,
                   const int64_t* k, const uint32_t* shared_idx, float* out_sum,
                   float* dense, hipStream_t stream) {
    dgc_state* st = const_cast<dgc_state*>(cst);
    if (!st || n_learners < 0) return DGC_EINVAL;
    const Plan& p = st->plan;
    int rc = check_k(st, k);
    if (rc != DGC_OK) return rc;
    int64_t K = 0;
    for (int32_t t = 0; t < p.T; ++t) K += k[t];
    if (K > 0 && (!out_sum || !aligned(out_sum, 4))) return DGC_EINVAL;
    if (K > 0 && n_learners > 0 && !vals) return DGC_EINVAL;
    for (int32_t w = 0; K > 0 && w < n_learners; ++w)
        if (!vals[w] || !aligned(vals[w], 4)) return DGC_EINVAL;
    if (dense && !aligned(dense, 4)) return DGC_EINVAL;
    if (dense && K > 0 && (!shared_idx || !aligned(shared_idx, 4))) return DGC_EINVAL;
    rc = upload_k(st, k, stream);
    if (rc != DGC_OK) return rc;
    st->last_stream = stream;
    DGC_TRY(timer_begin(st, DGC_TIMER_DECODE, stream));
    if (dense && p.n > 0)
        k_dec_fill<<<int(cdiv(p.n, kDecBlock)), kBlock, 0, stream>>>(dense, p.n);
    if (K > 0) {
        const int pg = grid_for(st->KT, int64_t(st->num_cus) * kCodecBlocksPerCU);
        int32_t w0 = 0;
        do {
            ShBatch B{};
            B.W = std::min<int32_t>(kShBatch, n_learners - w0);
            for (int w = 0; w < B.W; ++w) B.vals[w] = vals[w0 + w];
            const bool last = w0 + B.W >= n_learners;
            k_sh_sum<<<pg, kBlock, 0, stream>>>(st->L, st->K, B, int(w0 == 0), shared_idx,
                                                out_sum, last ? dense : nullptr, st->sc,
                                                st->KT);
            w0 += B.W;
        } while (w0 < n_learners);
    }
    DGC_LAUNCH_CHECK();
    DGC_TRY(timer_end(st, DGC_TIMER_DECODE, stream));
    return DGC_OK;
}

int dgc_shared_sum_static(int32_t n_tensors, const int64_t* sizes, int32_t n_learners,
                          const float* const* vals, const int64_t* k,
                          const uint32_t* shared_idx, float* out_sum, float* dense,
                          int32_t* status, hipStream_t stream) {
    if (n_tensors <= 0 || !sizes || !k || n_learners < 0) return DGC_EINVAL;
    if (n_tensors > kStaticMaxTensors) return DGC_ECAPACITY;
    const int32_t T = n_tensors;
    int64_t n = 0, K = 0, KT = 0;
    for (int32_t t = 0; t < T; ++t) {
        if (sizes[t] < 0 || sizes[t] >= (int64_t(1) << 32) || k[t] < 0 || k[t] > sizes[t])
            return DGC_EINVAL;
        n += sizes[t];
        K += k[t];
        KT += cdiv(k[t], kTile);
    }
    if (K > 0 && (!out_sum || !aligned(out_sum, 4))) return DGC_EINVAL;
    if (K > 0 && n_learners > 0 && !vals) return DGC_EINVAL;
    for (int32_t w = 0; K > 0 && w < n_learners; ++w)
        if (!vals[w] || !aligned(vals[w], 4)) return DGC_EINVAL;
    if (dense && !aligned(dense, 4)) return DGC_EINVAL;
    if (dense && K > 0 && (!shared_idx || !aligned(shared_idx, 4))) return DGC_EINVAL;
    if (status && !aligned(status, 4)) return DGC_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DGC_EHIP;
    char* base = nullptr;
    int num_cus = 0;
    DGC_TRY(static_scratch(dev, &base, &num_cus));
    Scalars* sc = reinterpret_cast<Scalars*>(base);
    int64_t* sz = reinterpret_cast<int64_t*>(base + kAlign);
    int64_t* kk = reinterpret_cast<int64_t*>(base + kAlign + kStaticTable);
    int64_t* o = reinterpret_cast<int64_t*>(base + kAlign + 2 * kStaticTable);
    int64_t* koff = reinterpret_cast<int64_t*>(base + kAlign + 3 * kStaticTable);
    int64_t* ktbase = reinterpret_cast<int64_t*>(base + kAlign + 4 * kStaticTable);
    // pageable sources are staged by the runtime before the calls return
    if (hipMemcpyAsync(sz, sizes, size_t(T) * 8, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(kk, k, size_t(T) * 8, hipMemcpyHostToDevice, stream) != hipSuccess)
        return DGC_EHIP;
    k_static_tables<<<1, kBlock, 0, stream>>>(T, sz, kk, o, koff, ktbase, sc);
    DevLayout L{};
    L.T = T;
    L.o = o;
    DevK Kd{};
    Kd.k = kk;
    Kd.koff = koff;
    Kd.ktbase = ktbase;
    if (dense && n > 0)
        k_dec_fill<<<int(cdiv(n, kDecBlock)), kBlock, 0, stream>>>(dense, n);
    if (K > 0) {
        const int pg = grid_for(KT, int64_t(num_cus) * kCodecBlocksPerCU);
        int32_t w0 = 0;
        do {
            ShBatch B{};
            B.W = std::min<int32_t>(kShBatch, n_learners - w0);
            for (int w = 0; w < B.W; ++w) B.vals[w] = vals[w0 + w];
            const bool last = w0 + B.W >= n_learners;
            k_sh_sum<<<pg, kBlock, 0, stream>>>(L, Kd, B, int(w0 == 0), shared_idx, out_sum,
                                                last ? dense : nullptr, sc, KT);
            w0 += B.W;
        } while (w0 < n_learners);
    }
    if (status) k_static_status<<<1, 64, 0, stream>>>(sc, status);
    DGC_LAUNCH_CHECK();
    return DGC_OK;
}

int dgc_stream_capacity(const dgc_state* st, int64_t* cap_offsets) {
    if (!st || !cap_offsets) return DGC_EINVAL;
    std::copy(st->plan.ebase.begin(), st->plan.ebase.end(), cap_offsets);
    return DGC_OK;
}

int dgc_encode(const dgc_state* cst, const int64_t* k, const uint32_t* idx,
               const float* val, uint16_t* runs, float* vals, int64_t* entries,
               hipStream_t stream) {
    dgc_state* st = const_cast<dgc_state*>(cst);
    if (!st) return DGC_EINVAL;
    return encode_impl(st, k, nullptr, idx, val, runs, vals, entries, stream);
}

int dgc_encode_counts(const dgc_state* cst, const int64_t* cap, const int64_t* count,
                      const uint32_t* idx, const float* val, uint16_t* runs,
                      float* vals, int64_t* entries, hipStream_t stream) {
    dgc_state* st = const_cast<dgc_state*>(cst);
    if (!st || !count || !aligned(count, 8)) return DGC_EINVAL;
    return encode_impl(st, cap, count, idx, val, runs, vals, entries, stream);
}

// Shared by dgc_decode_accumulate (dense += the streams) and dgc_decode_sum
// (fresh: dense = the streams, from +0.0).  A fresh sum takes the merged
// path for every tensor of the first batch of learners, so each dense block
// is written once and never read; later batches add as usual.
static int decode_impl(dgc_state* st, int32_t n_learners, const uint16_t* const* runs,
                       const float* const* vals, const int64_t* const* entries,
                       float* dense, bool fresh, hipStream_t stream) {
    if (!st || n_learners < 0) return DGC_EINVAL;
    if (n_learners == 0 && !fresh) return DGC_OK;
    const Plan& p = st->plan;
    if (n_learners > 0 && (!runs || !vals || !entries)) return DGC_EINVAL;
    if (p.n > 0 && (!dense || !aligned(dense, 4))) return DGC_EINVAL;
    for (int32_t w = 0; w < n_learners; ++w) {
        if (!entries[w] || !aligned(entries[w], 8)) return DGC_EINVAL;
        if (p.E > 0 && (!runs[w] || !vals[w] || !aligned(runs[w], 2) ||
                        !aligned(vals[w], 4)))
            return DGC_EINVAL;
    }
    st->last_stream = stream;
    if (n_learners == 0 || p.ET == 0) {
        if (!fresh || p.n == 0) return DGC_OK;
        // no entries at all: a fresh sum is all +0.0
        DGC_TRY(timer_begin(st, DGC_TIMER_DECODE, stream));
        k_fill_u32<<<grid_for(cdiv(p.n, kBlock), 8192), kBlock, 0, stream>>>(
            reinterpret_cast<uint32_t*>(dense), p.n, 0u);
        DGC_LAUNCH_CHECK();
        DGC_TRY(timer_end(st, DGC_TIMER_DECODE, stream));
        return DGC_OK;
    }
    const int T = p.T;
    // grid-stride over capacity tiles; a workgroup that reaches a tile past
    // its stream's end skips to the next tensor
    const int pg = grid_for(p.ET, int64_t(st->num_cus) * kCodecBlocksPerCU);
    DGC_TRY(timer_begin(st, DGC_TIMER_DECODE, stream));
    // learners in batches of kDecBatch; each batch's merged tensors are
    // added by one merge pass before the next batch starts
    for (int32_t b0 = 0; b0 < n_learners; b0 += kDecBatch) {
        const int nbw = std::min<int32_t>(kDecBatch, n_learners - b0);
        const bool fresh_batch = fresh && b0 == 0;
        // A fresh sum zeroes dense at once and scatters every tensor when the
        // tensors that could reach n_t / kDecMergeFresh entries with full
        // streams hold less than 1/8 of the elements; otherwise it merges
        // every tensor (each block written once, never read).
        bool fill_all = fresh_batch && st->decode_path != 2;
        if (fill_all && st->decode_path == 0) {
            int64_t n_merge = 0;
            for (int32_t t = 0; t < T; ++t) {
                const int64_t nt = p.sizes[size_t(t)];
                const int64_t cap = p.ebase[size_t(t) + 1] - p.ebase[size_t(t)];
                if (nt > 0 && kDecMergeFresh * int64_t(nbw) * cap >= nt) n_merge += nt;
            }
            fill_all = 8 * n_merge < p.n;
        }
        // can any tensor reach the merge threshold with full streams?
        bool merge_on = (st->decode_path == 2 || (fresh_batch && !fill_all)) && p.NBLK > 0;
        // one learner reads and writes its lines once either way
        if (st->decode_path == 0 && nbw >= 2)
            for (int32_t t = 0; t < T && !merge_on; ++t) {
                const int64_t nt = p.sizes[size_t(t)];
                const int64_t cap = p.ebase[size_t(t) + 1] - p.ebase[size_t(t)];
                merge_on = nt > 0 && kDecMergeAcc * int64_t(nbw) * cap >= nt;
            }
        // the bounds passes also load the values (for the merge to find in
        // cache) when the batch's value capacity is at most kDecWarmBytes
        const bool warm = merge_on && int64_t(nbw) * p.E * 4 <= kDecWarmBytes;
        DecBatch S{};
        S.W = nbw;
        for (int w = 0; w < nbw; ++w) {
            S.runs[w] = runs[b0 + w];
            S.vals[w] = vals[b0 + w];
            S.entries[w] = entries[b0 + w];
        }
        // A fresh batch that merges merges every tensor, each block starting
        // at +0.0; one that zero-filled dense first is an accumulate batch
        // from there on (each tensor merged only where its streams are
        // dense enough).
        const bool merge_fresh = fresh_batch && !fill_all;
        // scattered, the batch's streams added by one workgroup per tensor:
        // when forced, or when no tensor's streams can hold more than
        // kDecTensorTiles tiles together
        const bool per_tensor =
            !merge_on && (st->decode_path == 3 ||
                          (st->decode_path == 0 && nbw * p.et_max <= kDecTensorTiles));
        if (per_tensor) {
            if (fill_all && p.n > 0)
                k_dec_fill<<<int(cdiv(p.n, kDecBlock)), kBlock, 0, stream>>>(dense, p.n);
            k_dec_tensor<<<T, kBlock, 0, stream>>>(st->L, S, dense, st->sc);
            DGC_LAUNCH_CHECK();
            continue;
        }
        if (merge_on)
            k_dec_mode<<<int(cdiv(p.NBLK, kBlock)), kBlock, 0, stream>>>(
                st->L, S, st->Dd, merge_fresh ? 2 : st->decode_path, p.NBLK);
        if (fill_all && p.n > 0)
            k_dec_fill<<<int(cdiv(p.n, kDecBlock)), kBlock, 0, stream>>>(dense, p.n);
        for (int w = 0; w < nbw; ++w) {
            k_dec_count<<<pg, kBlock, 0, stream>>>(st->L, S.runs[w], S.entries[w], st->ta,
                                                   st->sc, p.ET);
            if (p.staged_etiles)
                k_dec_scan<true><<<T, kBlock, 0, stream>>>(st->L, S.entries[w], st->ta, st->t64);
            else
                k_dec_scan<false><<<T, kBlock, 0, stream>>>(st->L, S.entries[w], st->ta, st->t64);
            k_dec_write<<<pg, kBlock, 0, stream>>>(st->L, S.runs[w], S.vals[w], S.entries[w],
                                                   st->t64, dense, st->sc, p.ET,
                                                   int(merge_on), st->Dd, w, int(warm));
            DGC_LAUNCH_CHECK();
        }
        if (merge_on)
            k_dec_merge<<<int(kXcds * cdiv(p.NBLK, kXcds)), kBlock, 0, stream>>>(
                st->L, S, st->Dd, dense, p.NBLK, int(merge_fresh));
        DGC_LAUNCH_CHECK();
    }
    DGC_TRY(timer_end(st, DGC_TIMER_DECODE, stream));
    return DGC_OK;
}

int dgc_decode_accumulate(const dgc_state* cst, int32_t n_learners,
                          const uint16_t* const* runs, const float* const* vals,
                          const int64_t* const* entries, float* dense,
                          hipStream_t stream) {
    return decode_impl(const_cast<dgc_state*>(cst), n_learners, runs, vals, entries, dense,
                       false, stream);
}

int dgc_decode_sum(const dgc_state* cst, int32_t n_learners, const uint16_t* const* runs,
                   const float* const* vals, const int64_t* const* entries, float* dense,
                   hipStream_t stream) {
    return decode_impl(const_cast<dgc_state*>(cst), n_learners, runs, vals, entries, dense,
                       true, stream);
}

int dgc_get_status(dgc_state* st) {
    if (!st) return DGC_EINVAL;
    if (hipStreamSynchronize(st->last_stream) != hipSuccess) return DGC_EHIP;
    uint32_t status = 0;
    if (hipMemcpy(&status, &st->sc->status, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return DGC_EHIP;
    if (status) {
        uint32_t zero = 0;
        if (hipMemcpy(&st->sc->status, &zero, 4, hipMemcpyHostToDevice) != hipSuccess)
            return DGC_EHIP;
    }
    if (status == kErrCorrupt) return DGC_ECORRUPT;
    if (status) return DGC_EHIP;
    return DGC_OK;
}

int dgc_get_path_counts(dgc_state* st, int64_t* n_window, int64_t* n_dense) {
    if (!st) return DGC_EINVAL;
    if (hipStreamSynchronize(st->last_stream) != hipSuccess) return DGC_EHIP;
    std::vector<TensorState> h(size_t(st->plan.T));
    if (hipMemcpy(h.data(), st->ts, h.size() * sizeof(TensorState),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return DGC_EHIP;
    int64_t nw = 0, nd = 0;
    for (const TensorState& s : h) {
        nw += s.mode == kModeList;
        nd += s.mode == kModeDense;
    }
    if (n_window) *n_window = nw;
    if (n_dense) *n_dense = nd;
    return DGC_OK;
}

int dgc_get_select_info(dgc_state* st, int64_t* info) {
    if (!st || !info) return DGC_EINVAL;
    if (hipStreamSynchronize(st->last_stream) != hipSuccess) return DGC_EHIP;
    std::vector<TensorState> h(size_t(st->plan.T));
    if (hipMemcpy(h.data(), st->ts, h.size() * sizeof(TensorState),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return DGC_EHIP;
    for (size_t t = 0; t < h.size(); ++t) {
        int64_t* r = info + 6 * t;
        r[0] = h[t].mode;
        r[1] = h[t].lo_key;
        r[2] = h[t].total;
        r[3] = h[t].overflow;
        r[4] = h[t].prefix;
        r[5] = h[t].krem;
    }
    return DGC_OK;
}

int dgc_set_fused_event(dgc_state* st, hipEvent_t ev) {
    if (!st) return DGC_EINVAL;
    st->fused_event = ev;
    return DGC_OK;
}

int dgc_set_option(dgc_state* st, int32_t option, int64_t value) {
    if (!st) return DGC_EINVAL;
    if (option == DGC_OPT_ENCODE_PATH) {
        if (value < 0 || value > 2) return DGC_EINVAL;
        st->encode_path = int(value);
        return DGC_OK;
    }
    if (option == DGC_OPT_DECODE_PATH) {
        if (value < 0 || value > 3) return DGC_EINVAL;
        st->decode_path = int(value);
        return DGC_OK;
    }
    if (option == DGC_OPT_SELECT_PATH) {
        if (value != 0 && value != 1) return DGC_EINVAL;
        st->select_path = int(value);
        return DGC_OK;
    }
    if (option == DGC_OPT_SELECT_GRID) {
        if (value < 0 || value > 2) return DGC_EINVAL;
        st->select_grid = int(value);
        return DGC_OK;
    }
    if (option == DGC_OPT_KERNEL_TIMING) {
        if (value < 0 || value > 3) return DGC_EINVAL;
        st->timing = int(value);
        return DGC_OK;
    }
    return DGC_EINVAL;
}

int dgc_get_kernel_time(dgc_state* st, int32_t timer, double* total_ms,
                        int64_t* count) {
    if (!st || timer < 0 || timer > 3) return DGC_EINVAL;
    Timer& tm = st->timers[timer];
    for (int i = 0; i < Timer::kRing; ++i)
        if (timer_collect(tm, i) != DGC_OK) return DGC_EHIP;
    if (total_ms) *total_ms = tm.acc_ms;
    if (count) *count = tm.count;
    tm.acc_ms = 0.0;
    tm.count = 0;
    return DGC_OK;
}

void dgc_destroy_state(dgc_state* st) {
    if (!st) return;
    timers_destroy(st);
    delete st;
}

const char* dgc_error_string(int code) {
    switch (code) {
        case DGC_OK: return "ok";
        case DGC_EINVAL: return "invalid argument";
        case DGC_ECAPACITY: return "workspace or buffer too small";
        case DGC_EHIP: return "HIP runtime error";
        case DGC_ECORRUPT: return "corrupt stream";
        default: return "unknown error";
    }
}

}  // extern "C"
