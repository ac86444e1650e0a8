// Host side of the C ABI declared in include/moe_wna16.h: argument checks,
// workspace layout, tiling plan and the launch sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "launch.hpp"
#include "moe_wna16.h"

namespace {

using wna16::LayerDims;
using wna16::Workspace;

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 64;
constexpr int kMaxBlockM = 64;       // largest tile the forward may choose
constexpr int kMinGroup = 32;        // sizing bound for the per-group bias arrays
constexpr size_t kRegionAlign = 256;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_qparams(moe_wna16_qparams q)
{
    return (q.bits == 2 || q.bits == 4) && (q.group == 32 || q.group == 64 || q.group == 128);
}

// Basic size checks shared by workspace sizing and forward.
int check_sizes(int T, int H, int I, int E, int topk)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0)
        return MOE_WNA16_EINVAL;
    if (E > kMaxExperts || topk > kMaxTopk)
        return MOE_WNA16_EUNSUPPORTED;
    if (H % 128 != 0 || I % 128 != 0)
        return MOE_WNA16_EUNSUPPORTED;
    // every index the kernels form stays within int32
    const long long P = (long long)T * topk;
    const long long slots = P + (long long)kMaxBlockM * (E < P ? E : P);
    if ((long long)T * H >= (1LL << 31) || slots * I >= (1LL << 31) || P >= (1LL << 30))
        return MOE_WNA16_EUNSUPPORTED;
    return MOE_WNA16_OK;
}

struct Layout {
    size_t meta, offsets, sorted, tiles, inv, xperm, xbias, act, actbias, outf32, ccounts, done,
        tdone, hsum, total;
};

// Workspace pieces for tiles of at most `bm` rows (the sort's padded slots
// and the act rows they index are bounded by P + bm * min(E, P)).
Layout layout_for(int T, int H, int I, int E, int topk, int bm)
{
    const size_t P = (size_t)T * topk;
    const size_t minEP = (size_t)E < P ? (size_t)E : P;
    const size_t max_tiles = P / 4 + minEP + 1;   // smallest block_m (4) bound
    const size_t max_slots = P + (size_t)bm * minEP;
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + bytes, kRegionAlign);
        return at;
    };
    // status words, the XCD split, then the single-launch decode's counters
    static_assert((8 + 2 * wna16::kSplitEntries) * sizeof(int32_t) <= wna16::kSyncPrepDone,
                  "status words");
    L.meta = take(wna16::kSyncBytes);
    L.offsets = take((size_t)(E + 1) * sizeof(int32_t));
    L.sorted = take(max_slots * sizeof(int32_t));
    L.tiles = take(max_tiles * sizeof(int32_t));
    L.inv = take((P ? P : 1) * sizeof(int32_t));
    L.xperm = take((size_t)T * H * sizeof(uint16_t));
    L.xbias = take((size_t)T * (H / kMinGroup) * sizeof(float));
    L.act = take(max_slots * (size_t)I * sizeof(uint16_t));
    // (twice: the single-launch decode stores each group's term in two halves)
    L.actbias = take(2 * max_slots * (size_t)(I / kMinGroup) * sizeof(float));
    L.outf32 = take((size_t)T * H * sizeof(float));
    L.ccounts = take((size_t)wna16::align_chunks((long long)P) * (E + 1) * sizeof(int32_t));
    L.done = take((size_t)H);   // one counter per 64 output columns, 64 bytes apart
    L.tdone = take(max_tiles * 64);   // one counter per tile, 64 bytes apart
    // single-launch decode (at most 64 pairs): the split w13 items' FP32
    // pre-activation sums, 2I per 4-row tile row (at most P + 3 min(E, P) rows)
    L.hsum = take(P <= (size_t)wna16::kSingleLaunchPairs ? (P + 3 * minEP) * 2 * (size_t)I * 4 : 0);
    L.total = o;
    return L;
}

// The caller-provided workspace covers every block_m <= 64 (any bits / group).
Layout layout_of(int T, int H, int I, int E, int topk)
{
    return layout_for(T, H, I, E, topk, kMaxBlockM);
}

// Tiling: a pure function of the shapes.
//   variant 2 (decode-shaped): 4-row tiles, whole-K activation rows in LDS,
//     barrier-free weight streaming; used while experts average <= 4 rows and
//     the LDS image fits 64 KB.
//   variant 1 (prefill-shaped): 64-row tiles of 16x16x32 MFMAs; empty 16-row
//     slices of a tile are skipped, so lightly used experts in a skewed batch
//     cost little extra.
void make_plan(int T, int H, int I, int E, int topk, moe_wna16_qparams q13,
               moe_wna16_qparams q2, moe_wna16_plan_t *plan)
{
    const long long P = (long long)T * topk;
    // the decode-shaped kernels walk K in whole load units of 512 / bits
    // elements (256 for 2-bit, 128 for 4-bit codes)
    const bool decode = P <= 4LL * E && wna16::decode_lds_bytes(H, q13.group) <= 65536 &&
                        wna16::decode_lds_bytes(I, q2.group) <= 65536 &&
                        H % (512 / q13.bits) == 0 && I % (512 / q2.bits) == 0;
    const int bm = decode ? wna16::kDecodeRows : 64;
    plan->block_m = bm;
    // tiles = sum over the used experts of ceil(count / bm) <= (P + (bm - 1) * used) / bm
    plan->max_tiles = (int)((P + (long long)(bm - 1) * (E < P ? E : P)) / bm);
    plan->w13_variant = decode ? 2 : 1;
    plan->w2_variant = decode ? 2 : 1;
    plan->gemms_one_launch =
        decode && wna16::decode_one_launch(q13.bits, q13.group, q2.bits, q2.group, H, I) ? 1 : 0;
    plan->convert_in_w2 = decode && (size_t)T * H <= wna16::kFusedConvertMax ? 1 : 0;
    plan->single_launch = plan->gemms_one_launch && plan->convert_in_w2 &&
                                  P <= wna16::kSingleLaunchPairs &&
                                  plan->max_tiles <= wna16::kSyncTiles &&
                                  H / 128 <= wna16::kSyncBlocks
                              ? 1
                              : 0;
    plan->w13_ksplit = plan->single_launch
                           ? wna16::decode_layer_ksplit(q13.bits, q13.group, H, I, plan->max_tiles)
                           : 1;
}

// The prefill-shaped kernels address activations, their bias terms and one
// expert's codes and scales with 32-bit byte offsets.
bool offsets_fit(int T, int H, int I, int E, int topk)
{
    const unsigned long long lim = 1ull << 32;
    const unsigned long long P = (unsigned long long)T * topk;
    const unsigned long long slots = P + 64ull * (unsigned long long)(E < (long long)P ? E : P) + 64;
    return (unsigned long long)T * H * 2 < lim && slots * I * 2 < lim &&
           2ull * I * H < lim;   // one expert's w13 codes at 4 bits, and its scales
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_WNA16_EHIP;
    if (dev < 0 || dev >= 64)
        return MOE_WNA16_EARCH;
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return MOE_WNA16_EHIP;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? MOE_WNA16_OK : MOE_WNA16_EARCH;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_WNA16_OK : MOE_WNA16_EHIP; }

// The workspace of moe_wna16_forward_noalloc: one array per device, held
// until the process ends, shared by every such call on that device (the
// route kernel clears what must start at zero on every call).  In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the
// device address that hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> g_scratch[64];

// Device address of the current device's scratch array (the device was
// checked by check_device, so its index is below 64).
int scratch_of_current_device(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_WNA16_EHIP;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_WNA16_EHIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return MOE_WNA16_OK;
}

}  // namespace

extern "C" {

const char *moe_wna16_status_string(int status)
{
    switch (status) {
    case MOE_WNA16_OK: return "ok";
    case MOE_WNA16_EINVAL: return "invalid argument (shape, null pointer or NaN parameter)";
    case MOE_WNA16_EUNSUPPORTED:
        return "unsupported configuration (bits must be 2 or 4, group 32/64/128 dividing K, "
               "H and I multiples of 128, E <= 1024, topk <= 64)";
    case MOE_WNA16_EALIGN: return "misaligned pointer";
    case MOE_WNA16_EWORKSPACE: return "workspace too small";
    case MOE_WNA16_EARCH: return "current device is not gfx950 (MI355X)";
    case MOE_WNA16_EHIP: return "HIP runtime error";
    case MOE_WNA16_ESCRATCH:
        return "call needs more workspace than moe_wna16_forward_noalloc's 32 MiB scratch "
               "(use moe_wna16_forward with a workspace)";
    default: return "unknown status";
    }
}

int moe_wna16_workspace_size(int T, int H, int I, int E, int topk, size_t *bytes_out)
{
    if (!bytes_out)
        return MOE_WNA16_EINVAL;
    const int st = check_sizes(T, H, I, E, topk);
    if (st != MOE_WNA16_OK)
        return st;
    *bytes_out = layout_of(T, H, I, E, topk).total;
    return MOE_WNA16_OK;
}

int moe_wna16_workspace_f32_offset(int T, int H, int I, int E, int topk, size_t *offset_out)
{
    if (!offset_out)
        return MOE_WNA16_EINVAL;
    const int st = check_sizes(T, H, I, E, topk);
    if (st != MOE_WNA16_OK)
        return st;
    *offset_out = layout_of(T, H, I, E, topk).outf32;
    return MOE_WNA16_OK;
}

int moe_wna16_workspace_layout(int T, int H, int I, int E, int topk,
                               moe_wna16_workspace_layout_t *layout_out)
{
    if (!layout_out)
        return MOE_WNA16_EINVAL;
    const int st = check_sizes(T, H, I, E, topk);
    if (st != MOE_WNA16_OK)
        return st;
    const Layout L = layout_of(T, H, I, E, topk);
    layout_out->meta = L.meta;
    layout_out->expert_offsets = L.offsets;
    layout_out->sorted_ids = L.sorted;
    layout_out->tile_expert = L.tiles;
    layout_out->inv_perm = L.inv;
    layout_out->out_f32 = L.outf32;
    layout_out->total = L.total;
    return MOE_WNA16_OK;
}

int moe_wna16_plan(int T, int H, int I, int E, int topk, moe_wna16_qparams q13,
                   moe_wna16_qparams q2, moe_wna16_plan_t *plan_out)
{
    if (!plan_out)
        return MOE_WNA16_EINVAL;
    int st = check_sizes(T, H, I, E, topk);
    if (st != MOE_WNA16_OK)
        return st;
    if (!valid_qparams(q13) || !valid_qparams(q2) || H % q13.group || I % q2.group)
        return MOE_WNA16_EUNSUPPORTED;
    make_plan(T, H, I, E, topk, q13, q2, plan_out);
    return MOE_WNA16_OK;
}

// noalloc: the workspace is the library's own per-device scratch array
// (workspace and workspace_bytes are ignored), laid out for the plan's tile
// size; calls that need more than the array return ESCRATCH.
static int forward_impl(const void *x, const int32_t *topk_ids, const float *topk_w,
                      const int32_t *w13_packed, const uint16_t *w13_scales,
                      const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H, int I,
                      int E, int topk, moe_wna16_qparams q13, moe_wna16_qparams q2, float alpha,
                      float beta, float clamp, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream,
                      const hipEvent_t *events, bool prepared, bool noalloc = false)
{
    int st = check_sizes(T, H, I, E, topk);
    if (st != MOE_WNA16_OK)
        return st;
    if (!std::isfinite(alpha) || !std::isfinite(beta) || std::isnan(clamp) || !(clamp > 0.f))
        return MOE_WNA16_EINVAL;
    if (!valid_qparams(q13) || !valid_qparams(q2) || H % q13.group || I % q2.group)
        return MOE_WNA16_EUNSUPPORTED;
    if (!offsets_fit(T, H, I, E, topk))
        return MOE_WNA16_EUNSUPPORTED;
    if (T == 0)
        return MOE_WNA16_OK;
    if (!x || !topk_ids || !topk_w || !w13_packed || !w13_scales || !w2_packed || !w2_scales ||
        !out || (!workspace && !noalloc))
        return MOE_WNA16_EINVAL;
    if (!aligned(x, 16) || !aligned(w13_packed, 16) || !aligned(w2_packed, 16) ||
        !aligned(out, 16) || (!noalloc && !aligned(workspace, kRegionAlign)) ||
        !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(w13_scales, 2) ||
        !aligned(w2_scales, 2))
        return MOE_WNA16_EALIGN;
    moe_wna16_plan_t plan;
    make_plan(T, H, I, E, topk, q13, q2, &plan);
    if (prepared && (plan.w13_variant != 2 || plan.w2_variant != 2))
        return MOE_WNA16_EUNSUPPORTED;   // prepared codes feed the decode-shaped kernels only
    const Layout L = noalloc ? layout_for(T, H, I, E, topk, plan.block_m)
                             : layout_of(T, H, I, E, topk);
    if (noalloc && L.total > kScratchBytes)
        return MOE_WNA16_ESCRATCH;
    if (!noalloc && workspace_bytes < L.total)
        return MOE_WNA16_EWORKSPACE;
    st = check_device();
    if (st != MOE_WNA16_OK)
        return st;
    if (noalloc && (st = scratch_of_current_device(&workspace)) != MOE_WNA16_OK)
        return st;
    LayerDims d{};
    d.T = T;
    d.H = H;
    d.I = I;
    d.E = E;
    d.topk = topk;
    d.bits13 = q13.bits;
    d.g13 = q13.group;
    d.bits2 = q2.bits;
    d.g2 = q2.group;
    d.block_m = plan.block_m;
    d.max_tiles = plan.max_tiles;
    d.variant13 = plan.w13_variant;
    d.variant2 = plan.w2_variant;
    d.alpha = alpha;
    d.beta = beta;
    d.clamp = clamp;
    d.prepared = prepared ? 1 : 0;

    char *base = static_cast<char *>(workspace);
    Workspace ws{};
    ws.meta = reinterpret_cast<int32_t *>(base + L.meta);
    ws.expert_offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    ws.sorted_ids = reinterpret_cast<int32_t *>(base + L.sorted);
    ws.tile_expert = reinterpret_cast<int32_t *>(base + L.tiles);
    ws.inv_perm = reinterpret_cast<int32_t *>(base + L.inv);
    ws.x_perm = reinterpret_cast<uint16_t *>(base + L.xperm);
    ws.x_bias = reinterpret_cast<float *>(base + L.xbias);
    ws.act = reinterpret_cast<uint16_t *>(base + L.act);
    ws.act_bias = reinterpret_cast<float *>(base + L.actbias);
    ws.out_f32 = reinterpret_cast<float *>(base + L.outf32);
    ws.chunk_counts = reinterpret_cast<int32_t *>(base + L.ccounts);
    ws.done = reinterpret_cast<int32_t *>(base + L.done);
    ws.tile_done = reinterpret_cast<int32_t *>(base + L.tdone);
    ws.hsum = (long long)T * topk <= wna16::kSingleLaunchPairs
                  ? reinterpret_cast<float *>(base + L.hsum)
                  : nullptr;
    ws.xcd_first = ws.meta + 8;
    ws.prep_done = reinterpret_cast<int32_t *>(base + L.meta + wna16::kSyncPrepDone);
    ws.blocks_done = reinterpret_cast<int32_t *>(base + L.meta + wna16::kSyncBlocksDone);
    ws.sync_tiles = reinterpret_cast<int32_t *>(base + L.meta + wna16::kSyncTilesAt);
    ws.sync_done = reinterpret_cast<int32_t *>(base + L.meta + wna16::kSyncDoneAt);
    ws.sync_split = reinterpret_cast<int32_t *>(base + L.meta + wna16::kSyncSplitAt);

    wna16::KernelEvents ev[4];
    if (events)
        for (int i = 0; i < 4; ++i)
            ev[i] = wna16::KernelEvents{events[2 * i], events[2 * i + 1]};
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    uint16_t *outb = static_cast<uint16_t *>(out);
    // Small decode batches: the whole layer is one launch, which carries the
    // routing step's start event and the down projection's stop event.
    if (plan.single_launch)
        return hip_status(wna16::launch_decode_layer(
            xb, topk_ids, w13_packed, w13_scales, w2_packed, w2_scales, topk_w, d, ws, stream,
            wna16::KernelEvents{ev[0].start, ev[2].stop}, outb));
    // Tile-kernel plans split the items over the XCDs right after the sort:
    // the split launch belongs to the routing step and carries its stop event.
    const bool split = plan.w13_variant == 1 || plan.w2_variant == 1;
    const wna16::KernelEvents route_ev{ev[0].start, split ? nullptr : ev[0].stop};
    if ((st = hip_status(wna16::launch_route(xb, topk_ids, d, ws, stream, route_ev))) !=
        MOE_WNA16_OK)
        return st;
    if (split && (st = hip_status(wna16::launch_split(
                      d, ws, stream, wna16::KernelEvents{nullptr, ev[0].stop}))) != MOE_WNA16_OK)
        return st;
    // Small outputs: the last decode w2 workgroup of each column block rounds
    // that block to BF16, which saves the convert launch.  Decode shapes whose
    // projections share a format run both GEMMs in one launch.  The profiled
    // entry launches the same kernels; a shared launch carries the first
    // step's start event and the last step's stop event, and the events in
    // between are not recorded.
    const bool fuse = plan.convert_in_w2 != 0;
    if (plan.gemms_one_launch) {
        if ((st = hip_status(wna16::launch_decode(
                 w13_packed, w13_scales, w2_packed, w2_scales, topk_w, d, ws, stream,
                 wna16::KernelEvents{ev[1].start, ev[2].stop}, fuse ? outb : nullptr))) !=
            MOE_WNA16_OK)
            return st;
    } else {
        if ((st = hip_status(wna16::launch_w13(w13_packed, w13_scales, d, ws, stream, ev[1]))) !=
            MOE_WNA16_OK)
            return st;
        if ((st = hip_status(wna16::launch_w2(w2_packed, w2_scales, topk_w, d, ws, stream,
                                              ev[2], fuse ? outb : nullptr))) != MOE_WNA16_OK)
            return st;
    }
    if (fuse)
        return MOE_WNA16_OK;
    return hip_status(wna16::launch_convert(ws.out_f32, outb, (size_t)T * H, stream, ev[3]));
}

int moe_wna16_forward(const void *x, const int32_t *topk_ids, const float *topk_w,
                      const int32_t *w13_packed, const uint16_t *w13_scales,
                      const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H, int I,
                      int E, int topk, moe_wna16_qparams q13, moe_wna16_qparams q2, float alpha,
                      float beta, float clamp, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream)
{
    return forward_impl(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H,
                        I, E, topk, q13, q2, alpha, beta, clamp, out, workspace, workspace_bytes,
                        stream, nullptr, false);
}

int moe_wna16_forward_profiled(const void *x, const int32_t *topk_ids, const float *topk_w,
                               const int32_t *w13_packed, const uint16_t *w13_scales,
                               const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H,
                               int I, int E, int topk, moe_wna16_qparams q13,
                               moe_wna16_qparams q2, float alpha, float beta, float clamp,
                               void *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t *events)
{
    if (!events)
        return MOE_WNA16_EINVAL;
    return forward_impl(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H,
                        I, E, topk, q13, q2, alpha, beta, clamp, out, workspace, workspace_bytes,
                        stream, events, false);
}

int moe_wna16_forward_prepared(const void *x, const int32_t *topk_ids, const float *topk_w,
                               const int32_t *w13_prepared, const uint16_t *w13_scales,
                               const int32_t *w2_prepared, const uint16_t *w2_scales, int T, int H,
                               int I, int E, int topk, moe_wna16_qparams q13,
                               moe_wna16_qparams q2, float alpha, float beta, float clamp,
                               void *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t *events)
{
    return forward_impl(x, topk_ids, topk_w, w13_prepared, w13_scales, w2_prepared, w2_scales, T,
                        H, I, E, topk, q13, q2, alpha, beta, clamp, out, workspace,
                        workspace_bytes, stream, events, true);
}

int moe_wna16_forward_noalloc(const void *x, const int32_t *topk_ids, const float *topk_w,
                              const int32_t *w13_packed, const uint16_t *w13_scales,
                              const int32_t *w2_packed, const uint16_t *w2_scales, int T, int H,
                              int I, int E, int topk, moe_wna16_qparams q13,
                              moe_wna16_qparams q2, float alpha, float beta, float clamp,
                              void *out, hipStream_t stream)
{
    return forward_impl(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H,
                        I, E, topk, q13, q2, alpha, beta, clamp, out, nullptr, 0, stream,
                        nullptr, false, true);
}

int moe_wna16_prepare(const int32_t *packed, int E, int rows, int K, moe_wna16_qparams q,
                      int32_t *prepared_out, hipStream_t stream)
{
    if (E < 0 || rows < 0 || K <= 0)
        return MOE_WNA16_EINVAL;
    if (!valid_qparams(q) || K % q.group || K % (512 / q.bits) || rows % 16)
        return MOE_WNA16_EUNSUPPORTED;
    const size_t bytes = (size_t)E * rows * (K / 32 * q.bits) * 4;
    if (bytes == 0)
        return MOE_WNA16_OK;
    if (!packed || !prepared_out)
        return MOE_WNA16_EINVAL;
    const uintptr_t a = reinterpret_cast<uintptr_t>(packed),
                    b = reinterpret_cast<uintptr_t>(prepared_out);
    if (a < b + bytes && b < a + bytes)
        return MOE_WNA16_EINVAL;   // the reorder cannot run in place
    if (!aligned(packed, 4) || !aligned(prepared_out, 16))
        return MOE_WNA16_EALIGN;
    const int st = check_device();
    if (st != MOE_WNA16_OK)
        return st;
    return hip_status(wna16::launch_prepare(reinterpret_cast<const uint32_t *>(packed), E, rows,
                                            K, q.bits, q.group,
                                            reinterpret_cast<uint32_t *>(prepared_out), stream));
}

int moe_wna16_align(const int32_t *topk_ids, int T, int topk, int E, int block_m,
                    int32_t *sorted_ids, int32_t *tile_expert, int32_t *expert_offsets,
                    int32_t *inv_perm, int32_t *num_tiles, int32_t *bad_ids, hipStream_t stream)
{
    if (T < 0 || topk <= 0 || E <= 0 || block_m <= 0)
        return MOE_WNA16_EINVAL;
    if (E > kMaxExperts || block_m > 1024 || (long long)T * topk >= (1LL << 30))
        return MOE_WNA16_EUNSUPPORTED;
    if ((T > 0 && (!topk_ids || !inv_perm || !sorted_ids || !tile_expert)) || !expert_offsets ||
        !num_tiles || !bad_ids)
        return MOE_WNA16_EINVAL;
    if (!aligned(topk_ids, 4) || !aligned(sorted_ids, 4) || !aligned(tile_expert, 4) ||
        !aligned(expert_offsets, 4) || !aligned(inv_perm, 4) || !aligned(num_tiles, 4) ||
        !aligned(bad_ids, 4))
        return MOE_WNA16_EALIGN;
    const int st = check_device();
    if (st != MOE_WNA16_OK)
        return st;
    return hip_status(wna16::launch_align(topk_ids, T, topk, E, block_m, sorted_ids, tile_expert,
                                          expert_offsets, inv_perm, num_tiles, bad_ids, stream));
}

int moe_wna16_quantize(const void *w, const float *imp, int rows, int K, moe_wna16_qparams q,
                       int n_candidates, int32_t *codes_out, uint16_t *scales_out,
                       double *err_sums_out, hipStream_t stream)
{
    if (rows < 0 || K <= 0 || n_candidates < 1 || n_candidates > 64)
        return MOE_WNA16_EINVAL;
    if (!valid_qparams(q) || K % q.group)
        return MOE_WNA16_EUNSUPPORTED;
    if ((rows > 0 && (!w || !codes_out || !scales_out)) || !err_sums_out)
        return MOE_WNA16_EINVAL;
    if (!aligned(w, 16) || !aligned(imp, 4) || !aligned(codes_out, 4) ||
        !aligned(scales_out, 2) || !aligned(err_sums_out, 8))
        return MOE_WNA16_EALIGN;   // weights are read 16 bytes at a time
    const int st = check_device();
    if (st != MOE_WNA16_OK)
        return st;
    return hip_status(wna16::launch_quantize(
        static_cast<const uint16_t *>(w), imp, rows, K, q.bits, q.group, n_candidates,
        reinterpret_cast<uint32_t *>(codes_out), scales_out, err_sums_out, stream));
}

}  // extern "C"
