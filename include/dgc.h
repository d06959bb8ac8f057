/*
 * dgc.h -- C ABI of libdgc, the per-learner sparsifying gradient compressor
 * of Deep Gradient Compression (DGC) on AMD Instinct MI355X (gfx950).
 *
 * The method is described on the review page "[Paper Review] Deep Gradient
 * Compression: Reducing the Communication Bandwidth for Distributed
 * Training" (nubint.ai), section "Proposed method": send only the large
 * entries and keep the rest in a local accumulator; send each value in 32
 * bits after the 16-bit length of the zero run before it; momentum
 * correction; local
 * gradient clipping; momentum factor masking; warm-up to a rising sparsity.
 * Its Abstract places this in synchronous data-parallel SGD, where the
 * learners' sparse gradients are summed.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensors of one learner's gradient lie end to end in one flat
 *   binary32 array ("layout"): tensor t has n_t elements at offset
 *   o_t = n_0 + ... + n_{t-1}.  Indices in outputs are local to their tensor
 *   (uint32), so every n_t must be below 2^32.
 * - Pointers named "device" are HIP device memory owned by the caller;
 *   "host" pointers are ordinary host memory read during the call only.
 *   The library never allocates device memory; it mallocs only the small
 *   host-side dgc_state, freed by dgc_destroy_state.
 * - Calls enqueue work on the given stream and return without waiting for
 *   it (except dgc_get_status, dgc_get_path_counts and dgc_init_state, which
 *   synchronise).  Results are valid once the stream reaches that point.
 * - A dgc_state belongs to one learner (its u, v and workspace).  Calls on
 *   one state must not run concurrently on two streams.
 * - Return codes: DGC_OK (0) or a negative DGC_E* code.  Argument errors are
 *   detected on the host before anything is enqueued.  Errors found by the
 *   kernels (a corrupt stream) are latched in the workspace and reported by
 *   dgc_get_status.
 * - Arithmetic is IEEE binary32 with round-to-nearest-even, no FMA
 *   contraction and denormals kept, so results are reproducible bit for
 *   bit; the only binary64 value is the clipping norm.
 */
#ifndef DGC_H_
#define DGC_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DGC_OK 0
#define DGC_EINVAL (-1)    /* bad argument: null pointer, size, k, alignment */
#define DGC_ECAPACITY (-2) /* workspace or output buffer too small */
#define DGC_EHIP (-3)      /* a HIP runtime call or kernel launch failed */
#define DGC_ECORRUPT (-4)  /* a decoded stream ran past its tensor's end */

/* Largest bin length of dgc_compress_binlocal. */
#define DGC_MAX_BIN 1024

/* Options for dgc_set_option. */
#define DGC_OPT_SELECT_PATH 1   /* value 0: automatic (default); 1: always the
                                   dense exact path (no sample window); for
                                   dgc_compress_binlocal and
                                   dgc_compress_sampled, every piece's entries
                                   re-derived in the placement pass (no
                                   slots) -- the same results, slower */
#define DGC_OPT_KERNEL_TIMING 2 /* value 1: bracket the work of each call with
                                   HIP events on the call's stream (read with
                                   dgc_get_kernel_time); 2: only the
                                   element-wise pass (DGC_TIMER_FUSED, two
                                   events per compress call); 3: each call,
                                   but not its element-wise pass (an event
                                   record between two kernels delays the
                                   second by a few microseconds, so mode 1's
                                   DGC_TIMER_COMPRESS includes that
                                   overhead and mode 3's does not); 0: off
                                   (default) */
#define DGC_OPT_DECODE_PATH 3   /* dgc_decode_accumulate, per tensor: 0
                                   automatic (default: merged when the
                                   learners' streams hold at least n_t / 16
                                   entries together, else each stream added
                                   on its own -- by one workgroup per tensor,
                                   for up to 8 learners in one launch, when
                                   no tensor's streams can hold more than
                                   8192 entries together at capacity, else
                                   by passes spread over 1024-entry tiles);
                                   1 always on its own, spread; 2 always
                                   merged; 3 always on its own, a workgroup
                                   per tensor -- the same results, only the
                                   speed differs */
#define DGC_OPT_SELECT_GRID 4   /* dgc_compress and dgc_compress_hier, the
                                   exact select and emit: 0 automatic
                                   (default: when every tensor has at most
                                   2^22 elements, one 1024-thread workgroup
                                   per tensor for the window and for the
                                   gather, select and emit; else passes
                                   spread over all workgroups); 1 the same
                                   per-tensor kernels, and on layouts with a
                                   larger tensor one workgroup per tensor
                                   for the select and emit after the spread
                                   gather (slow for long sources); 2 always
                                   the spread passes -- the same results,
                                   only the speed differs */

#define DGC_OPT_ENCODE_PATH 5   /* dgc_encode and dgc_encode_counts: 0
                                   automatic (default: when no tensor sends
                                   more than 8192 entries, one workgroup per
                                   tensor counts, scans and writes its stream
                                   in one launch; else three passes spread
                                   over 1024-entry tiles); 1 always the
                                   workgroup per tensor; 2 always the tiled
                                   passes -- the same results, only the
                                   speed differs */

/* Timers for dgc_get_kernel_time. */
#define DGC_TIMER_FUSED 0     /* the element-wise pass of dgc_compress,
                                 dgc_compress_binlocal, dgc_compress_sampled or
                                 dgc_compress_shared */
#define DGC_TIMER_COMPRESS 1  /* all of one of those calls */
#define DGC_TIMER_ENCODE 2    /* all of dgc_encode / dgc_encode_counts */
#define DGC_TIMER_DECODE 3    /* all of dgc_decode_accumulate, dgc_decode_sum
                                 or dgc_shared_sum */

typedef struct dgc_state dgc_state;

/*
 * Warm-up schedule (DGC review, "Proposed method": warm-up starts at a low
 * sparsity and raises it step by step): the number of entries a tensor of
 * n elements sends at density num / den,
 *   k = ceil(n * num / den),
 * computed in exact integer arithmetic (128-bit product).  The density is
 * a fraction, never a binary floating-point number: ceil(350e6 * (1 -
 * 0.999)) in binary64 is 350001, not 350000.
 *   n          element count, n >= 0
 *   num, den   density numerator and denominator, 0 <= num <= den, den >= 1
 * Returns k (0 <= k <= n), or DGC_EINVAL (negative) for arguments outside
 * those ranges.  Pure host arithmetic: no state, no GPU, thread-safe.
 */
int64_t dgc_k_for_density(int64_t n, int64_t num, int64_t den);

/*
 * Workspace size for a layout.
 *   n_tensors  number of tensors T >= 1
 *   sizes      host int64[T], element counts n_t, 0 <= n_t < 2^32
 *   k_max      host int64[T], the largest k_t that dgc_compress, or the
 *              largest cap[t] that dgc_compress_binlocal / dgc_compress_sampled,
 *              will be given for tensor t (0 <= k_max[t] <= n_t); it sizes the
 *              candidate buffers and the encoded stream capacity.  The
 *              bin-local and sampled passes share the candidate slots out
 *              among their pieces: a k_max well below the entries a piece
 *              sends makes that piece take the slower re-derivation (same
 *              results)
 *   bytes      out: bytes of device workspace dgc_init_state needs
 * Returns DGC_OK or DGC_EINVAL.
 */
int dgc_workspace_bytes(int32_t n_tensors, const int64_t* sizes,
                        const int64_t* k_max, size_t* bytes);

/*
 * Create the state of one learner.
 *   st         out: new state (free with dgc_destroy_state)
 *   momentum   momentum constant m of the momentum correction (e.g. 0.9f)
 *   u, v       device float[n]: momentum buffer u and accumulated gradient
 *              v, n = sum of sizes, 16-byte aligned; zeroed here on stream
 *   workspace  device memory of at least dgc_workspace_bytes bytes,
 *              256-byte aligned, owned by the caller for the state's life
 *   stream     stream for the zeroing and the copy of layout tables; the
 *              call waits for it before returning
 * The state keeps the pointers; the caller keeps the memory alive.
 * Returns DGC_OK, DGC_EINVAL, DGC_ECAPACITY (workspace too small) or
 * DGC_EHIP.
 */
int dgc_init_state(dgc_state** st, int32_t n_tensors, const int64_t* sizes,
                   const int64_t* k_max, float momentum, float* u, float* v,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * One compression step of the learner (DGC review, "Proposed method":
 * local gradient clipping, momentum correction, sparsification with local
 * accumulation, momentum factor masking):
 *   1. if clip > 0: S = sum g_i^2 over the whole gradient (binary64),
 *      norm = sqrt(S), s = (float)(clip / norm) if norm > clip else 1;
 *      if clip <= 0: s = 1 and no norm is computed
 *   2. u_i = fl(fl(m * u_i) + fl(g_i * s));  v_i = fl(v_i + u_i)
 *   3. per tensor: the k_t entries first under (|v_i| descending, index
 *      ascending), with |v_i| compared as the bit pattern of v_i with the
 *      sign cleared (so +0 == -0; NaN payloads rank above infinity)
 *   4. those entries are written out and u_i = v_i = +0.0f at them; every
 *      other u_i, v_i keeps its value (the residual)
 * Arguments:
 *   g          device const float[n], 16-byte aligned: this step's gradient
 *   k          host int64[T], 0 <= k[t] <= k_max[t]  (warm-up: any k per step)
 *   clip       clipping threshold; <= 0 turns clipping off
 *   out_idx    device uint32[sum k], 4-byte aligned: tensor t's k_t local
 *              indices, ascending, at offset K_t = k_0 + ... + k_{t-1}
 *   out_val    device float[sum k]: the matching values of v (signed, taken
 *              before masking), same offsets
 *   out_norm   device double[1]: the norm, or -1.0 when clipping is off
 *   out_scale  device float[1]: the scale s applied to g
 * Exact for every k and input; the path taken (sample window or dense
 * histogram) changes only the speed.  Returns DGC_OK, DGC_EINVAL or
 * DGC_EHIP.
 */
int dgc_compress(dgc_state* st, const float* g, const int64_t* k, double clip,
                 uint32_t* out_idx, float* out_val, double* out_norm,
                 float* out_scale, hipStream_t stream);

/*
 * One compression step with the bin-local selector of AdaComp (the page
 * "AdaComp : Adaptive Residual Gradient Compression for Data-Parallel
 * Distributed Training": Abstract -- residues are selected locally and the
 * rate follows local activity; "Citations in the corpus" -- each layer's
 * residual vector is cut into fixed-size bins and a bin's largest absolute
 * value is its threshold).  Steps 1, 2 and 4 are dgc_compress's; step 3
 * becomes:
 *   3'. tensor t is cut into bins of bin_len[t] entries from its start (the
 *       last bin may be shorter); theta_b = max |v_j| over bin b; entry i
 *       is salient iff v_i != 0 and |fl(v_i + u_i)| >= theta_b, i.e. v
 *       looked ahead by this step's update u once more reaches the bin's
 *       largest |v| (magnitudes compared as sign-cleared bit patterns)
 * The first cap[t] salient entries of tensor t in index order are written
 * out and masked (u_i = v_i = +0.0f); salient entries beyond cap[t] stay in
 * the residual untouched.
 * Arguments:
 *   g          device const float[n], 16-byte aligned
 *   bin_len    host int64[T], 1 <= bin_len[t] <= DGC_MAX_BIN
 *   cap        host int64[T], 0 <= cap[t] <= k_max[t]: most entries to
 *              deliver for tensor t; cap[t] = n_t never truncates
 *   clip       as for dgc_compress
 *   out_idx    device uint32[sum cap]: tensor t's delivered local indices,
 *              ascending, at offset C_t = cap[0] + ... + cap[t-1]; slots
 *              past out_count[t] are left as they were
 *   out_val    device float[sum cap]: the matching values of v before
 *              masking, same offsets
 *   out_count  device int64[T], 8-byte aligned: out, entries delivered
 *              (min(salient, cap[t]))
 *   out_total  device int64[T] or NULL: out, salient entries per tensor
 *   out_norm, out_scale  as for dgc_compress
 * Exact and deterministic; the path (slots or re-derivation) changes only
 * the speed.  Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_compress_binlocal(dgc_state* st, const float* g, const int64_t* bin_len,
                          const int64_t* cap, double clip, uint32_t* out_idx,
                          float* out_val, int64_t* out_count, int64_t* out_total,
                          double* out_norm, float* out_scale, hipStream_t stream);

/*
 * One compression step with an approximate, sampled threshold in place of
 * exact top-k (DGC review, "Research questions": hierarchical thresholding
 * as a runtime strategy for scalable selection).  Steps 1, 2 and 4 are
 * dgc_compress's; step 3 becomes:
 *   3''. per tensor t, a sample of whole 32-element lines of v: every line
 *        when n_t <= 65536, else ls = min(lines, max(512, lines / 256))
 *        lines, line j (0 <= j < ls) at j*stride + fmix32(j*0x9E3779B9 ^
 *        t*0x7F4A7C15) mod stride with stride = lines / ls (32-bit wrapping
 *        products; fmix32 is MurmurHash3's finalizer); S sampled entries;
 *        theta_t = the J-th largest sampled |v|, J = ceil(S * k[t] / n_t);
 *        every entry with v_i != 0 and |v_i| >= theta_t is sent
 * so about k[t] entries leave, not exactly k[t].  The first cap[t] of them
 * in index order are written out and masked; the rest stay in the residual.
 * k[t] = 0 sends nothing.  One pass over g, u, v: no exact-select re-read.
 * Arguments:
 *   k          host int64[T], 0 <= k[t] <= n_t: the target count
 *   cap        host int64[T], 0 <= cap[t] <= k_max[t]: most entries to
 *              deliver; outputs at offset C_t = cap[0] + ... + cap[t-1]
 *   g, clip, out_idx, out_val, out_count, out_total, out_norm, out_scale
 *              as for dgc_compress_binlocal (out_total: entries at or above
 *              the threshold, delivered or not)
 * dgc_get_select_info then reports path 3, theta in [1] and [4], S in [2]
 * and J in [5].  Deterministic; encode with dgc_encode_counts.  Returns
 * DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_compress_sampled(dgc_state* st, const float* g, const int64_t* k,
                         const int64_t* cap, double clip, uint32_t* out_idx,
                         float* out_val, int64_t* out_count, int64_t* out_total,
                         double* out_norm, float* out_scale, hipStream_t stream);

/*
 * One learner step with hierarchical thresholding (DGC review, "Research
 * questions": RQ4 names hierarchical thresholding as a runtime strategy for
 * scalable selection; "Proposed method": only large entries are sent).  The
 * page names the strategy only; the reading taken stacks two levels:
 *   level 1  dgc_compress_sampled's threshold theta_t from the sampled
 *            lines (the ceil(S k_t / n_t)-th largest sampled key); the
 *            survivors are the non-zero entries with |v| key >= theta_t
 *   level 2  more than k_t survivors: the k_t of them first under (key
 *            descending, index ascending), the rule of dgc_compress; at
 *            most k_t: all of them
 * so a tensor sends E_t = min(k_t, survivors) entries, never more than k_t,
 * and exactly dgc_compress's selection whenever at least k_t survive.
 * Steps 1, 2 and 4 are dgc_compress's (clip, momentum, masking of the sent
 * entries).  The survivors are the element-wise pass's candidates; the
 * exact select then runs on them (or on the whole tensor under the floor
 * max(theta_t, 1) when a piece's candidates overflow its slots).
 * Arguments:
 *   g, k, clip, out_norm, out_scale  as for dgc_compress (k host int64[T],
 *              0 <= k[t] <= k_max[t])
 *   out_idx    device uint32[sum k], 4-byte aligned: tensor t's sent local
 *              indices, ascending, at offset K_t = k[0] + ... + k[t-1]; the
 *              first out_count[t] slots are written, the rest untouched
 *   out_val    device float[sum k], 4-byte aligned: their values (signed,
 *              before masking), same slots
 *   out_count  device int64[T], 8-byte aligned: E_t
 * With DGC_OPT_SELECT_PATH 1 the survivors are not kept as candidates and
 * the select always runs on the whole tensor (the same results, slower).
 * dgc_get_select_info then reports as for dgc_compress ([1] is
 * max(theta_t, 1), or 0xFFFFFFFF on the forced whole-tensor path; [2] the
 * survivors; a whole list of at most k_t has T = 0 and r = 0).
 * Deterministic; encode with dgc_encode_counts (cap = k).  Returns DGC_OK,
 * DGC_EINVAL (also for a k above k_max) or DGC_EHIP.
 */
int dgc_compress_hier(dgc_state* st, const float* g, const int64_t* k, double clip,
                      uint32_t* out_idx, float* out_val, int64_t* out_count,
                      double* out_norm, float* out_scale, hipStream_t stream);

/*
 * One step of a learner that sends at a shared index set: commutative
 * compression (the ScaleComp abstract on the taxoreview.com page: the
 * learners' gradient distributions are alike, which allows a compressor
 * that commutes with the sum over learners, whose communication cost does
 * not grow with their number and which an all-reduce can carry).  Reading:
 * each step one learner, the leader (step mod W), selects with
 * dgc_compress; every other learner calls this with the leader's out_idx,
 * so all learners send their v at the same indices, and dgc_shared_sum
 * adds their value vectors.  Steps 1, 2 and 4 are dgc_compress's; step 3
 * becomes:
 *   3s. out_val[j] = v[shared_idx[j]] for tensor t's k[t] shared local
 *       indices (at offset K_t = k[0] + ... + k[t-1]); u and v are masked
 *       (+0.0f) there
 * Arguments:
 *   g          device const float[n], 16-byte aligned
 *   k          host int64[T], 0 <= k[t] <= k_max[t]: the shared set's size
 *   shared_idx device const uint32[sum k], 4-byte aligned: per tensor k[t]
 *              strictly ascending local indices below n_t (dgc_compress's
 *              out_idx has this layout)
 *   clip       as for dgc_compress
 *   out_val    device float[sum k], 4-byte aligned: the values of v at the
 *              shared indices (signed, before masking), same offsets
 *   out_norm, out_scale  as for dgc_compress
 * A shared_idx that is not ascending or leaves its tensor latches
 * DGC_ECORRUPT (dgc_get_status); the affected values are then unspecified,
 * but nothing is written outside out_val, u and v.  Deterministic.
 * Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_compress_shared(dgc_state* st, const float* g, const int64_t* k,
                        const uint32_t* shared_idx, double clip, float* out_val,
                        double* out_norm, float* out_scale, hipStream_t stream);

/*
 * The aggregate of shared-index compression (ScaleComp abstract, as for
 * dgc_compress_shared): the element-wise sum of the learners' value vectors
 * in learner order from +0.0,
 *   out_sum[j] = fl(...fl(fl(+0 + vals[0][j]) + vals[1][j])... + vals[W-1][j]),
 * K = sum k floats whatever the number of learners (what an all-reduce
 * carries), and optionally the fresh dense sum: out_sum scattered at the
 * shared indices, +0.0 everywhere else -- the same bits as encoding every
 * learner's (shared_idx, values) and dgc_decode_sum of those streams.
 *   vals       host array of n_learners device pointers, each float[sum k]
 *              laid out as dgc_compress_shared's out_val (the leader's is
 *              dgc_compress's out_val)
 *   k          host int64[T], as given to the compress calls
 *   shared_idx device const uint32[sum k]: the shared indices (read only
 *              when dense is set)
 *   out_sum    device float[sum k], 4-byte aligned: out, the learner-order
 *              sums (required when sum k > 0)
 *   dense      device float[n], 4-byte aligned, or NULL: out, every element
 *              written
 * n_learners = 0 gives +0.0 sums.  An index outside its tensor latches
 * DGC_ECORRUPT and is not written.  Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_shared_sum(const dgc_state* st, int32_t n_learners, const float* const* vals,
                   const int64_t* k, const uint32_t* shared_idx, float* out_sum,
                   float* dense, hipStream_t stream);

/*
 * dgc_shared_sum without a state or workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): it allocates nothing, on the
 * device or the host.  Its per-call tables (the layout's offsets, the k
 * tables) and its status latch live in a static device array of 640 KiB
 * that the library holds on each GPU it runs on until the process ends;
 * its address on a device is looked up once, on the first call there.
 *   n_tensors  1 <= T <= 16384 (more returns DGC_ECAPACITY, before anything
 *              is enqueued)
 *   sizes      host int64[T], 0 <= n_t < 2^32: the layout (n = sum)
 *   k          host int64[T], 0 <= k[t] <= n_t
 *   n_learners, vals, shared_idx, out_sum, dense  as for dgc_shared_sum
 *   status     device int32[1], 4-byte aligned, or NULL: out, DGC_OK, or
 *              DGC_ECORRUPT when an index left its tensor (that entry is
 *              not written to dense)
 * The results are dgc_shared_sum's, bit for bit.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams,
 * other threads) race; calls in one stream's order do not.  The host
 * arrays may be reused as soon as the call returns.  Returns DGC_OK,
 * DGC_EINVAL, DGC_ECAPACITY or DGC_EHIP.
 */
int dgc_shared_sum_static(int32_t n_tensors, const int64_t* sizes, int32_t n_learners,
                          const float* const* vals, const int64_t* k,
                          const uint32_t* shared_idx, float* out_sum, float* dense,
                          int32_t* status, hipStream_t stream);

/*
 * Capacity layout of encoded streams: cap_offsets[t] (host int64[T+1]) is
 * the first entry slot of tensor t; tensor t may use up to
 * cap_offsets[t+1] - cap_offsets[t] entries: k_max[t] + floor(n_t / 65536),
 * enough for any selection of at most k_max[t] indices, rounded up to a
 * multiple of 8 (every tensor's stream then starts 16-byte aligned).
 */
int dgc_stream_capacity(const dgc_state* st, int64_t* cap_offsets);

/*
 * Zero-run encoding (DGC review, "Proposed method": 32-bit values, each
 * after a 16-bit zero-run length).  Per tensor, per selected index j in
 * ascending order with gap G = j - prev - 1 (prev = -1 at the start):
 * floor(G / 65536) filler entries (run 65535, value +0.0f), then the entry
 * (G mod 65536, value).  Zeros after the last selected index are not
 * encoded.  Each entry counts as 6 bytes (16-bit run + 32-bit value).
 *   k          host int64[T], as given to dgc_compress
 *   idx, val   device: dgc_compress's outputs for those k
 *   runs       device uint16[cap_offsets[T]]: runs, tensor t's at
 *              cap_offsets[t] (structure of arrays, little endian)
 *   vals       device float[cap_offsets[T]]: values, same slots
 *   entries    device int64[T]: out, entry count E_t per tensor
 * idx must be strictly ascending within each tensor (as dgc_compress
 * writes it).  Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_encode(const dgc_state* st, const int64_t* k, const uint32_t* idx,
               const float* val, uint16_t* runs, float* vals, int64_t* entries,
               hipStream_t stream);

/*
 * dgc_encode for a selection whose sizes are on the device (the output of
 * dgc_compress_binlocal): tensor t's entries are at offset
 * cap[0] + ... + cap[t-1] of idx / val, and count[t] of them are encoded.
 *   cap        host int64[T], as given to dgc_compress_binlocal
 *   count      device const int64[T], 8-byte aligned: entries per tensor;
 *              a count outside [0, cap[t]] encodes nothing for that tensor
 *              and latches DGC_ECORRUPT for dgc_get_status
 *   idx, val, runs, vals, entries  as for dgc_encode
 * Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_encode_counts(const dgc_state* st, const int64_t* cap,
                      const int64_t* count, const uint32_t* idx,
                      const float* val, uint16_t* runs, float* vals,
                      int64_t* entries, hipStream_t stream);

/*
 * Decode several learners' streams and add them into one dense sum (the
 * gradient exchange of synchronous SGD, DGC review Abstract):
 * for w = 0 .. n_learners-1 in order, per tensor, pos = -1 and for each
 * entry pos += run + 1; dense[o_t + pos] = fl(dense[o_t + pos] + value).
 * Fillers are added too (+0.0f).  The sum is not averaged.  Where the
 * streams are dense (DGC_OPT_DECODE_PATH) the learners' entries are added
 * block by block in one pass per 8 learners, still in learner order.
 *   runs, vals, entries  host arrays of n_learners device pointers, each
 *                        stream laid out as dgc_encode writes it for this
 *                        state's layout
 *   dense      device float[n]: accumulated in place (zero it first for a
 *              fresh sum)
 * A stream whose positions pass its tensor's end, or whose E_t is negative
 * or above capacity, adds nothing past that point and latches
 * DGC_ECORRUPT for dgc_get_status.  No float atomics are used: the result
 * is the same bits every run.  Returns DGC_OK, DGC_EINVAL or DGC_EHIP.
 */
int dgc_decode_accumulate(const dgc_state* st, int32_t n_learners,
                          const uint16_t* const* runs,
                          const float* const* vals,
                          const int64_t* const* entries, float* dense,
                          hipStream_t stream);

/*
 * A fresh dense sum of several learners' streams (the aggregate one step of
 * synchronous SGD applies, DGC review Abstract): the same result as zeroing
 * dense to +0.0 and calling dgc_decode_accumulate, bit for bit, without the
 * separate zeroing.  Every element of dense[n] is written, whatever it held
 * before.  For the first 8 learners either every tensor takes the
 * block-by-block path (each dense block written once, read never) or, when
 * the layout's streams cannot be dense enough for that to pay, dense is
 * zeroed and each stream added on its own; later learners are added as
 * dgc_decode_accumulate adds them.  DGC_OPT_DECODE_PATH 1 forces the second
 * way, 2 the first.  n_learners == 0 gives all +0.0.  Arguments, ownership
 * and errors as for dgc_decode_accumulate.
 */
int dgc_decode_sum(const dgc_state* st, int32_t n_learners,
                   const uint16_t* const* runs, const float* const* vals,
                   const int64_t* const* entries, float* dense,
                   hipStream_t stream);

/*
 * Wait for the state's last stream and return the latched device-side
 * error (DGC_OK or DGC_ECORRUPT: a corrupt stream in decoding, unsorted
 * input to an encoder, or a bad device count), clearing it.  Returns DGC_EHIP if the
 * wait fails.
 */
int dgc_get_status(dgc_state* st);

/*
 * How the last dgc_compress selected: per tensor it used either the sample
 * window (candidates gathered during the element-wise pass) or the dense
 * exact path.  Waits for the stream.  Either count may be NULL.
 */
int dgc_get_path_counts(dgc_state* st, int64_t* n_window, int64_t* n_dense);

/*
 * Per-tensor record of the last dgc_compress, dgc_compress_sampled or
 * dgc_compress_hier (waits for the stream):
 * info (host int64[6 * n_tensors]) receives for each tensor
 *   [0] path: 0 = k was 0, 1 = sample window, 2 = dense exact path,
 *       3 = the sampled threshold of dgc_compress_sampled (then [1] and [4]
 *       hold the threshold, [2] the sample size and [5] the rank J; the
 *       other fields below describe dgc_compress)
 *   [1] candidate threshold key of the sample window (0xFFFFFFFF = none)
 *   [2] candidates the element-wise pass found
 *   [3] 1 if a piece found more candidates than its slots hold
 *   [4] the k-th largest magnitude key T (bits of |v| with sign cleared)
 *   [5] how many entries equal to T were sent (r)
 */
int dgc_get_select_info(dgc_state* st, int64_t* info);

/*
 * Pipelining hook: record `ev` on the call's stream right after each
 * dgc_compress of this state has enqueued its element-wise pass (the one
 * that streams g, u and v).  A caller running several learners can make the
 * next learner's stream wait on it, so that learner's bandwidth-heavy
 * passes start while this one finishes its short selection kernels, and no
 * two element-wise passes overlap.  NULL turns it off.  The event stays
 * the caller's.  Returns DGC_OK or DGC_EINVAL.
 */
int dgc_set_fused_event(dgc_state* st, hipEvent_t ev);

/* Set an option (DGC_OPT_*).  Returns DGC_OK or DGC_EINVAL. */
int dgc_set_option(dgc_state* st, int32_t option, int64_t value);

/*
 * With DGC_OPT_KERNEL_TIMING on: total milliseconds and number of the
 * intervals of `timer` (DGC_TIMER_*) recorded since the last read, measured
 * between HIP events on the stream each call ran on.  Waits for those
 * events; resets the timer.  Either output may be NULL.
 */
int dgc_get_kernel_time(dgc_state* st, int32_t timer, double* total_ms,
                        int64_t* count);

/* Free the host-side state.  Device memory stays the caller's. */
void dgc_destroy_state(dgc_state* st);

/* Static text for a return code. */
const char* dgc_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* DGC_H_ */
