// Internal launchers of the gfx950 kernels (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace wna16 {

// Device workspace regions of one forward call.
struct Workspace {
    int32_t *meta;            // [0] num_tiles, [1] bad ids, [2] fused decode waits that gave up
    int32_t *expert_offsets;  // [E + 1]
    int32_t *sorted_ids;      // [max_slots]
    int32_t *tile_expert;     // [max_tiles]
    int32_t *inv_perm;        // [P]
    uint16_t *x_perm;         // [T, H] bf16, fragment order per w13 group
    float *x_bias;            // [T, H / g13] minus each group's bias term (chain start)
    uint16_t *act;            // [max_slots, I] bf16, fragment order per w2 group
    float *act_bias;          // [max_slots, I / g2] minus each group's bias term
    float *out_f32;           // [T, H]
    int32_t *chunk_counts;    // [align chunks][E + 1]: per-chunk expert counts, then invalid ids
    int32_t *done;            // [H / 64][16]: decode w2 workgroups finished per column block
    int32_t *tile_done;       // [max_tiles][16]: fused decode, w13 workgroups finished per tile
    int32_t *xcd_first;       // [2][kSplitEntries]: tile kernel item range per XCD, w13 then w2
    // Single-launch decode: counters in the fixed region at the start of the
    // workspace, zero between calls (the call's last workgroup resets them).
    int32_t *prep_done;       // prep workgroups finished
    int32_t *blocks_done;     // down-projection column blocks finished
    int32_t *sync_tiles;      // [kSyncTiles][16]: gate/up workgroups finished per tile
    int32_t *sync_done;       // [kSyncBlocks][16]: down workgroups finished per column block
    int32_t *sync_split;      // [kSyncSplits]: split w13 slices finished per (tile, column block)
    float *hsum;              // [tile rows][2I] split w13 partial sums (null: no room, no split)
};

// Fixed region at the start of every workspace (byte offsets): the status
// words, then the single-launch decode counters, each on its own 64 bytes.
constexpr size_t kSyncBytes = 32768;
constexpr size_t kSyncPrepDone = 256, kSyncBlocksDone = 320, kSyncTilesAt = 1024;
constexpr int kSyncTiles = 128, kSyncBlocks = 128;
constexpr size_t kSyncDoneAt = kSyncTilesAt + (size_t)kSyncTiles * 64;
constexpr size_t kSyncSplitAt = kSyncDoneAt + (size_t)kSyncBlocks * 64;
constexpr int kSyncSplits = 2048;
static_assert(kSyncSplitAt + (size_t)kSyncSplits * 4 <= kSyncBytes, "sync region");

// Entries per GEMM of the tile kernel's XCD split: 8 range starts and the total.
constexpr int kSplitEntries = 9;

// Pairs per workgroup of the expert sort.
// Pairs per sort workgroup: a multiple of 1024 (one placement step), the
// smallest that keeps the sort at most kMaxSortBlocks workgroups (each one
// reads the counts of every chunk).
constexpr int kAlignStep = 1024;
constexpr int kMaxSortBlocks = 16;
inline int align_chunk(long long P)
{
    const long long per = (P + kMaxSortBlocks - 1) / kMaxSortBlocks;
    const long long c = (per + kAlignStep - 1) / kAlignStep * kAlignStep;
    return (int)(c < kAlignStep ? kAlignStep : c);
}
inline int align_chunks(long long P)
{
    const long long c = align_chunk(P);
    return P <= c ? 1 : (int)((P + c - 1) / c);
}

// Optional start/stop events recorded by the kernel dispatch itself
// (hipExtLaunchKernelGGL); null events record nothing.
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

struct LayerDims {
    int T, H, I, E, topk;
    int bits13, g13, bits2, g2;
    int block_m, max_tiles, variant13, variant2;
    float alpha, beta, clamp;
    int prepared;   // codes in the prepared block order (decode-shaped plans only)
};

// Expert-sorted tiles + activation reorder/bias + zeroed accumulator.
hipError_t launch_route(const uint16_t *x, const int32_t *topk_ids, const LayerDims &d,
                        const Workspace &ws, hipStream_t stream, const KernelEvents &ev);
// Tile-kernel plans (block_m 64): split each GEMM's items over the XCDs by
// cost, after the route launch (writes ws.xcd_first).
hipError_t launch_split(const LayerDims &d, const Workspace &ws, hipStream_t stream,
                        const KernelEvents &ev);
// Fused gate/up WNA16 GEMM with the SwiGLU epilogue.
hipError_t launch_w13(const int32_t *w13, const uint16_t *s13, const LayerDims &d,
                      const Workspace &ws, hipStream_t stream, const KernelEvents &ev);
// Down WNA16 GEMM with the routing-weighted FP32 scatter-add epilogue.  With
// a non-null out_bf16 (decode-shaped w2 and T*H <= kFusedConvertMax only) the
// last workgroup to finish also writes the BF16 output.
hipError_t launch_w2(const int32_t *w2, const uint16_t *s2, const float *topk_w,
                     const LayerDims &d, const Workspace &ws, hipStream_t stream,
                     const KernelEvents &ev, uint16_t *out_bf16 = nullptr);
// Both decode-shaped GEMMs in one launch (same bits and group on both
// projections); hipErrorNotSupported, before any launch, when the shapes do
// not allow it.  out_bf16 as for launch_w2.
hipError_t launch_decode(const int32_t *w13, const uint16_t *s13, const int32_t *w2,
                         const uint16_t *s2, const float *topk_w, const LayerDims &d,
                         const Workspace &ws, hipStream_t stream, const KernelEvents &ev,
                         uint16_t *out_bf16);
// Whether decode-shaped w13 and w2 of these formats and sizes run as one launch.
bool decode_one_launch(int bits13, int g13, int bits2, int g2, int H, int I);
// The whole decode-shaped layer in one launch (routing, activation reorder,
// zeroing, both GEMMs and the rounding): workgroups [0, n_pre) do the
// routing's work, the rest are the shared-launch GEMM items.  Needs the
// one-launch GEMMs, the fused rounding, at most 64 pairs, max_tiles <=
// kSyncTiles and H / 128 <= kSyncBlocks.
hipError_t launch_decode_layer(const uint16_t *x, const int32_t *topk_ids, const int32_t *w13,
                               const uint16_t *s13, const int32_t *w2, const uint16_t *s2,
                               const float *topk_w, const LayerDims &d, const Workspace &ws,
                               hipStream_t stream, const KernelEvents &ev, uint16_t *out_bf16);
// Pairs up to which the single-launch decode's tile lookup works (one wave).
constexpr int kSingleLaunchPairs = 64;
// K slices per w13 (tile, column block) in the single launch (1, 2 or 4).
int decode_layer_ksplit(int bits, int gs, int H, int I, int max_tiles);
// Largest T*H whose BF16 rounding the decode w2 kernel does itself (the last
// workgroup of each column block rounds that block).
constexpr size_t kFusedConvertMax = 1 << 18;
// Prepared block order of one projection's codes (prepare.hip): packed
// [E][rows][K*bits/32] -> blocks [E][rows/16][K/(512/bits)] of 256 words.
hipError_t launch_prepare(const uint32_t *packed, int E, int rows, int K, int bits, int group,
                          uint32_t *prepared, hipStream_t stream);
// Quantizer (quantize.hip): W [rows][K] BF16 -> codes, FP16 scales and the
// four reconstruction error sums.
hipError_t launch_quantize(const uint16_t *w, const float *imp, int rows, int K, int bits,
                           int group, int ncand, uint32_t *codes, uint16_t *scales,
                           double *sums, hipStream_t stream);
// FP32 accumulator -> BF16 output (round to nearest even).
hipError_t launch_convert(const float *src, uint16_t *dst, size_t n, hipStream_t stream,
                          const KernelEvents &ev);
// Dynamic LDS bytes of the decode-shaped GEMM for reduction length K, group gs.
size_t decode_lds_bytes(int K, int gs);
// Rows per tile of the decode-shaped GEMM.
constexpr int kDecodeRows = 4;
// Stand-alone tile layout (the moe_wna16_align entry point).
hipError_t launch_align(const int32_t *topk_ids, int T, int topk, int E, int block_m,
                        int32_t *sorted_ids, int32_t *tile_expert, int32_t *expert_offsets,
                        int32_t *inv_perm, int32_t *num_tiles, int32_t *bad_ids,
                        hipStream_t stream);

}  // namespace wna16
