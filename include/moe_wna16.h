/*
 * moe_wna16.h -- C ABI of the routed weight-only-quantized (WNA16) MoE layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (PR "Incubate DeepSeek V4 WNA16 runtime on SM86", "What this
 * branch adds" items 1-3 and 9; model card
 * "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed"):
 *
 *   for every token t and each of its top-k slots j, with e = topk_ids[t][j]:
 *     h   = W13_e x_t                    fused gate (rows 0..I-1) and up (rows I..2I-1)
 *     a   = SwiGLU_{alpha,beta,clamp}(h[0:I], h[I:2I])
 *     out_t += topk_w[t][j] * (W2_e a)
 *   out is returned in BF16; the sum is carried in FP32.
 *
 *   W[n][k] = q[n][k] * s[n][k / group]: symmetric signed b-bit codes (b = 2 or
 *   4, no zero point) packed into 32-bit words and one FP16 scale per group of
 *   K elements.  Each projection has its own bit width and group size
 *   ("Validation completed": projection-specific group sizes).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller (except
 *     the *_out / plan arguments documented as host pointers).  The library
 *     allocates no memory and keeps no state between calls; calls on
 *     different streams may run concurrently.
 *   - Work is enqueued asynchronously on `stream`; no entry point
 *     synchronises the host.  The enqueued work is kernels only (no memset
 *     or copy nodes), so the calls can be captured into a HIP graph and
 *     replayed.
 *   - Workspace state: the first MOE_WNA16_SYNC_BYTES bytes of a forward
 *     workspace hold counters that the single-launch decode plan
 *     (moe_wna16_plan_t.single_launch) uses to order its workgroups.  They
 *     must be zero before a workspace's first forward call (allocate it
 *     zeroed, or clear them once); every call leaves them zero, except a
 *     call whose status word meta[2] (moe_wna16_workspace_layout) reports
 *     waits that gave up: clear them again before reusing that workspace.
 *     Nothing else carries over between calls.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     non-zero status means nothing was launched and no buffer was touched.
 *   - Device-side values (expert ids) are not validated on the host: an id
 *     outside [0, E) contributes nothing and is counted in the workspace.
 *
 * Packed formats (the pages fix the pieces; the order of fields and the sign
 * encoding are this library's stated reading):
 *   - Codes: row-major [rows][K * bits / 32] int32 words; the code for K index
 *     j*(32/bits)+i is bits [i*bits, (i+1)*bits) of word j, stored as
 *     q + 2^(bits-1) (so q lies in [-2^(bits-1), 2^(bits-1)-1]).
 *   - Scales: row-major [rows][K / group] IEEE binary16.
 *   - w13: rows = 2I, K = H; rows [0, I) gate (w1), rows [I, 2I) up (w3).
 *   - w2:  rows = H,  K = I.
 *   - SwiGLU: g' = min(g, clamp), u' = min(max(u, -clamp), clamp),
 *             a = g' * sigmoid(alpha * g') * (u' + beta); clamp = +INFINITY
 *             disables clamping.
 */
#ifndef MOE_WNA16_H
#define MOE_WNA16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Leading bytes of a forward workspace that must be zero before its first use. */
#define MOE_WNA16_SYNC_BYTES 32768

typedef enum {
    MOE_WNA16_OK = 0,
    MOE_WNA16_EINVAL = -1,      /* bad shape, null pointer, NaN parameter   */
    MOE_WNA16_EUNSUPPORTED = -2,/* bits / group / shape outside the kernels */
    MOE_WNA16_EALIGN = -3,      /* pointer not aligned as required          */
    MOE_WNA16_EWORKSPACE = -4,  /* workspace smaller than workspace_size    */
    MOE_WNA16_EARCH = -5,       /* current device is not gfx950             */
    MOE_WNA16_EHIP = -6,        /* a HIP runtime call or launch failed      */
    MOE_WNA16_ESCRATCH = -7     /* moe_wna16_forward_noalloc: the call needs */
                                /* more than the library's 32 MiB scratch    */
} moe_wna16_status;

/* Quantization of one projection: bits in {2, 4}; group in {32, 64, 128}. */
typedef struct {
    int32_t bits;
    int32_t group;
} moe_wna16_qparams;

/* Tiling chosen for a call (a pure function of the shapes; see moe_wna16_plan). */
typedef struct {
    int32_t block_m;        /* rows of (token, slot) pairs per tile: 4 or 64        */
    int32_t max_tiles;      /* tile capacity the grid is sized for                  */
    int32_t w13_variant;    /* 2: decode-shaped (4-row tiles, weight streaming),    */
                            /* 1: prefill-shaped (64-row MFMA tiles)                */
    int32_t w2_variant;     /* same encoding for the down projection               */
    int32_t gemms_one_launch; /* 1: both decode-shaped GEMMs run in one launch      */
                              /*    (same bits and group on both projections)      */
    int32_t convert_in_w2;  /* 1: the BF16 rounding runs inside the decode w2       */
                            /*    launch (decode shapes with T*H <= 2^18)          */
    int32_t single_launch;  /* 1: the whole layer (routing, reorder, both GEMMs,    */
                            /*    rounding) is one launch: gemms_one_launch and     */
                            /*    convert_in_w2 with T*topk <= 64, max_tiles <= 128 */
                            /*    and H <= 16384                                    */
    int32_t w13_ksplit;     /* single launch: K slices per gate/up (tile, column    */
                            /*    block), each its own workgroup (1, 2 or 4; more   */
                            /*    when few tiles would leave the GPU idle)          */
} moe_wna16_plan_t;

/*
 * Bytes of device workspace moe_wna16_forward needs for these sizes (any
 * bits / group).  *bytes_out is a HOST pointer.  Returns EINVAL on bad sizes.
 */
int moe_wna16_workspace_size(int T, int H, int I, int E, int topk, size_t *bytes_out);

/*
 * Tiling moe_wna16_forward will use for these arguments.  *plan_out is a
 * HOST pointer.  Returns the same status forward would return from its
 * shape / parameter checks (no device query).
 */
int moe_wna16_plan(int T, int H, int I, int E, int topk, moe_wna16_qparams q13,
                   moe_wna16_qparams q2, moe_wna16_plan_t *plan_out);

/*
 * The routed layer (see the top of this file).
 *
 *   x           [T, H] bf16, row-major                          16-byte aligned
 *   topk_ids    [T, topk] int32, expert ids                      4-byte aligned
 *   topk_w      [T, topk] float32 routing weights, used as given 4-byte aligned
 *   w13_packed  [E, 2I, H*b13/32] int32                         16-byte aligned
 *   w13_scales  [E, 2I, H/g13] fp16                              2-byte aligned
 *   w2_packed   [E, H, I*b2/32] int32                           16-byte aligned
 *   w2_scales   [E, H, I/g2] fp16                                2-byte aligned
 *   out         [T, H] bf16, written (never read)               16-byte aligned
 *   workspace   >= moe_wna16_workspace_size bytes               256-byte aligned
 *
 * Shapes: T >= 0 (T = 0 returns OK with no launch), 1 <= E <= 1024,
 * 1 <= topk <= 64, H and I multiples of 128, each group dividing its K.
 * Size limit (EUNSUPPORTED): T*H*2, (T*topk + 64*min(E, T*topk) + 64)*I*2 and
 * 2*I*H must each stay below 2^32 (the kernels use 32-bit byte offsets).
 * alpha, beta must be finite; clamp must be > 0 (or +INFINITY), not NaN.
 * The output is the FP32 sum rounded to BF16 (nearest even).  Summation
 * order across a token's experts is unspecified (FP32 atomics).
 */
int moe_wna16_forward(const void *x, const int32_t *topk_ids, const float *topk_w,
                      const int32_t *w13_packed, const uint16_t *w13_scales,
                      const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H, int I,
                      int E, int topk, moe_wna16_qparams q13, moe_wna16_qparams q2, float alpha,
                      float beta, float clamp, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * moe_wna16_forward with per-step timing; it launches the same kernels as
 * moe_wna16_forward.  `events` is a HOST array of 8 caller-created
 * hipEvent_t; for the four steps of the layer (in order: routing and
 * activation reorder -- with the prefill-shaped plan also the split of the
 * tile kernels' items over the XCDs, a launch of its own --, w13 + SwiGLU,
 * w2 + scatter-add, BF16 rounding) step i
 * records events[2i] when its launch starts and events[2i+1] when it ends,
 * from the dispatch packets themselves (no extra packets on the stream).
 * Steps that share a launch (see moe_wna16_plan_t: gemms_one_launch,
 * convert_in_w2): the launch records the first step's start event and the
 * last step's stop event, and the events in between are not recorded; so
 * with gemms_one_launch, events[2] and events[5] bracket the one w13 + w2
 * launch, with convert_in_w2, events[6] and events[7] stay unrecorded
 * (the rounding is inside the w2 launch), and with single_launch only
 * events[0] and events[5] are recorded, around the one launch.  Same checks and status codes as
 * moe_wna16_forward, plus EINVAL for a NULL `events`.
 */
int moe_wna16_forward_profiled(const void *x, const int32_t *topk_ids, const float *topk_w,
                               const int32_t *w13_packed, const uint16_t *w13_scales,
                               const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H,
                               int I, int E, int topk, moe_wna16_qparams q13,
                               moe_wna16_qparams q2, float alpha, float beta, float clamp,
                               void *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t *events);

/*
 * Expert-sorted tile layout of the T*topk (token, slot) pairs, pair index
 * p = t*topk + j: the grouping of an indexed MoE's routed pairs by expert
 * that the PR's BF16 "indexed MoE" path runs on ("What this branch adds"
 * item 3), on its own.  The layout is this library's (the pages do not
 * print one).  Bit-exact and deterministic:
 *   expert_offsets[E+1]  exclusive prefix sum of each expert's pair count
 *                        rounded up to a multiple of block_m
 *   sorted_ids[]         slot expert_offsets[e] + r holds the r-th smallest p
 *                        routed to e (stable); padding slots hold T*topk.
 *                        Capacity: (T*topk/block_m + min(E, T*topk)) * block_m.
 *   tile_expert[]        expert of each block_m-slot tile; capacity
 *                        T*topk/block_m + min(E, T*topk)
 *   inv_perm[T*topk]     slot of pair p, or -1 for an id outside [0, E)
 *   num_tiles[1]         expert_offsets[E] / block_m
 *   bad_ids[1]           number of ids outside [0, E)
 * Entries past num_tiles*block_m (sorted_ids) and num_tiles (tile_expert) are
 * left untouched.  block_m in [1, 1024]; E <= 1024; int32 buffers 4-byte
 * aligned.  T = 0 writes expert_offsets = 0 and num_tiles = bad_ids = 0.
 */
int moe_wna16_align(const int32_t *topk_ids, int T, int topk, int E, int block_m,
                    int32_t *sorted_ids, int32_t *tile_expert, int32_t *expert_offsets,
                    int32_t *inv_perm, int32_t *num_tiles, int32_t *bad_ids,
                    hipStream_t stream);

/*
 * Byte offset, inside the workspace of a moe_wna16_forward call with these
 * sizes, of the FP32 accumulator [T, H] (row-major float) that holds the
 * routed sum before its rounding to BF16.  It is valid once the call has
 * completed and is overwritten by the next call on the same workspace; it
 * lets a caller inspect the unrounded result.  *offset_out is a HOST pointer.
 * Same size checks and status codes as moe_wna16_workspace_size.
 */
int moe_wna16_workspace_f32_offset(int T, int H, int I, int E, int topk, size_t *offset_out);

/*
 * Where a moe_wna16_forward call with these sizes keeps, inside its
 * workspace, the results of its own expert sort and its status words (byte
 * offsets from the start of the workspace).  The contents are valid once the
 * call has completed and are overwritten by the next call on the same
 * workspace; they let a caller check the sort the layer actually ran (the
 * expert-sorted tile layout the PR's BF16 "indexed MoE" path needs, "What
 * this branch adds" item 3) and whether the call completed normally.
 *
 *   meta            int32 words:
 *                   [0] num_tiles of the layer's sort (expert_offsets[E] / block_m)
 *                   [1] ids outside [0, E)
 *                   [2] fused decode waits that gave up: 0 after a normal call.  In
 *                       the one-launch decode plan (moe_wna16_plan_t.gemms_one_launch)
 *                       each down-projection workgroup waits, with a bounded spin, for
 *                       the gate/up workgroups of its tile, and in the single-launch
 *                       plan each gate/up workgroup also waits for the routing
 *                       workgroups; a non-zero count means a wait ended at its bound,
 *                       that call's output is unreliable and the workspace's first
 *                       MOE_WNA16_SYNC_BYTES bytes must be cleared before its next use
 *                   [3..7] reserved, [8..25] the prefill tile kernels' split of their
 *                       (tile, column block) items over the 8 XCDs (gate/up then down:
 *                       8 range starts and the item count each); bytes [256,
 *                       MOE_WNA16_SYNC_BYTES) hold the single-launch counters
 *   expert_offsets  int32 [E + 1]     \
 *   sorted_ids      int32 [num_tiles * block_m]   the tile layout of
 *   tile_expert     int32 [num_tiles]             moe_wna16_align, with the
 *   inv_perm        int32 [T * topk]  /           plan's block_m
 *   out_f32         float [T, H]      the routed sum before its BF16 rounding
 *   total           = moe_wna16_workspace_size
 *
 * *layout_out is a HOST pointer.  Same size checks and status codes as
 * moe_wna16_workspace_size.
 */
typedef struct {
    size_t meta;
    size_t expert_offsets;
    size_t sorted_ids;
    size_t tile_expert;
    size_t inv_perm;
    size_t out_f32;
    size_t total;
} moe_wna16_workspace_layout_t;

int moe_wna16_workspace_layout(int T, int H, int I, int E, int topk,
                               moe_wna16_workspace_layout_t *layout_out);

/*
 * Quantizer: float weights -> the packed codes and scales the layer reads
 * (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "How it was created"
 * steps 2-5).  For every row and every group of `q.group` consecutive K
 * elements, with amax the group's largest |w|:
 *   s0  = amax / ((2^b - 1) / 2)                            (FP32)
 *   s_c = fp16_rne(min(s0 * (1 - c / (2C)), 65504)),  c = 0 .. C-1
 *   q   = clamp(rne(w / s_c), -2^(b-1), 2^(b-1) - 1)         (FP32 division; 0 if s_c = 0)
 *   err_c = sum over the group of imp[k] * (w - s_c * q)^2   (FP64)
 * and the smallest err_c wins (ties to the smaller c); C = n_candidates, so
 * C = 1 is plain round-to-nearest with the absmax scale.
 *
 *   w           [rows, K] bf16, row-major                       16-byte aligned
 *   imp         [K] float32 importance per input channel (>= 0), or NULL for
 *               all ones (the unweighted search)                 4-byte aligned
 *   codes_out   [rows, K*b/32] int32 in the packed format above  4-byte aligned
 *   scales_out  [rows, K/group] fp16                             2-byte aligned
 *   err_sums_out [4] float64, overwritten: sum (w - w')^2, sum w^2,
 *               sum imp (w - w')^2, sum imp w^2 over the matrix, w' the
 *               dequantized weight (summation order unspecified) 8-byte aligned
 *
 * rows >= 0 (rows = 0 writes zero sums), K > 0 a multiple of the group;
 * 1 <= n_candidates <= 64 (offsets are 64-bit: no limit on rows * K).  Non-finite weights are not
 * checked (their groups' codes are unspecified).  An imp containing NaN or
 * negative values gives unspecified scale choices.
 */
int moe_wna16_quantize(const void *w, const float *imp, int rows, int K, moe_wna16_qparams q,
                       int n_candidates, int32_t *codes_out, uint16_t *scales_out,
                       double *err_sums_out, hipStream_t stream);

/*
 * Prepared codes: a one-time reorder of one projection's packed codes into the
 * order the decode-shaped kernels stream (a one-time setup step and an
 * interface variant of the packed format of model card
 * "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed").  A pure
 * permutation of the 32-bit words:
 *
 *   a load unit is U = 512 / bits consecutive K elements of one row (16
 *   words); a block is 16 rows x one unit (256 words); blocks are stored
 *   [expert][row / 16][unit].  Inside a block, for rows r = 0..15 and lane
 *   groups g = 0..3, slot (g * 16 + r) holds words 4 (g*16+r) .. +3: for each
 *   quantization group of the unit in turn, the words of row r that hold the
 *   codes at in-group K offsets [g * group / 4, (g + 1) * group / 4).  For
 *   2-bit codes with group 32 (half a word per lane group and group), lane
 *   groups 2h and 2h+1 share one slot: slot (h * 16 + r) holds words
 *   8 (h*16+r) .. +7, word 2 gq + h of the unit for its groups gq = 0..7.
 *
 *   packed        [E, rows, K*bits/32] int32, the packed format   4-byte aligned
 *   prepared_out  [E, rows, K*bits/32] int32, written; must not
 *                 overlap `packed` (EINVAL)                      16-byte aligned
 *
 * rows % 16 == 0 and K % (512 / bits) == 0 (else EUNSUPPORTED); K a multiple
 * of the group.  E * rows = 0 returns OK with no launch.  For a layer: w13 is
 * prepared with rows = 2I, K = H; w2 with rows = H, K = I.
 */
int moe_wna16_prepare(const int32_t *packed, int E, int rows, int K, moe_wna16_qparams q,
                      int32_t *prepared_out, hipStream_t stream);

/*
 * moe_wna16_forward with both projections' codes in the prepared order
 * (scales unchanged).  Only decode-shaped calls (moe_wna16_plan reports
 * w13_variant = w2_variant = 2: T * topk <= 4E and K in whole load units):
 * other shapes return EUNSUPPORTED before any launch, and need the packed
 * codes.  `events` is NULL, or 8 events recorded as by
 * moe_wna16_forward_profiled.  Otherwise the same checks, status codes and
 * result as moe_wna16_forward.
 */
int moe_wna16_forward_prepared(const void *x, const int32_t *topk_ids, const float *topk_w,
                               const int32_t *w13_prepared, const uint16_t *w13_scales,
                               const int32_t *w2_prepared, const uint16_t *w2_scales, int T, int H,
                               int I, int E, int topk, moe_wna16_qparams q13,
                               moe_wna16_qparams q2, float alpha, float beta, float clamp,
                               void *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t *events);

/*
 * moe_wna16_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace.  Instead it uses a scratch array inside
 * the library: 32 MiB of device memory per GPU, held from the first call on
 * that GPU until the process ends.  It allocates nothing itself (no hipMalloc,
 * no allocating library call); its first call on a device looks the array's
 * address up once.
 *
 * Same arguments (codes in the packed order), checks, status codes and result
 * as moe_wna16_forward without its workspace arguments, except:
 *   - The workspace this call needs, laid out for the plan's tile size
 *     (moe_wna16_plan_t.block_m), must fit the 32 MiB; otherwise it returns
 *     MOE_WNA16_ESCRATCH before any launch.  Every decode-shaped call
 *     (block_m 4) with T <= 512 at H = 4096, I = 2048, E = 256 fits;
 *     prefill-shaped calls at those sizes do not (their 64-row tiles pad
 *     every expert's act rows) and need moe_wna16_forward.
 *   - Every call on one GPU uses that GPU's one array.  Calls ordered on one
 *     stream are fine (each clears what must start at zero); calls that
 *     overlap on one GPU -- on different streams, or from several host
 *     threads without ordering -- race on it and give undefined results.
 *   - The array keeps the last call's contents; nothing in it is meant to be
 *     read by the caller.
 */
int moe_wna16_forward_noalloc(const void *x, const int32_t *topk_ids, const float *topk_w,
                              const int32_t *w13_packed, const uint16_t *w13_scales,
                              const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H,
                              int I, int E, int topk, moe_wna16_qparams q13,
                              moe_wna16_qparams q2, float alpha, float beta, float clamp,
                              void *out, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *moe_wna16_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_WNA16_H */
