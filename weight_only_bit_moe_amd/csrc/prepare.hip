// One-time reorder of packed codes into the prepared block order that the
// decode-shaped kernels stream (layout.hpp: prep_src_dword, prep_block_dword).
// It is a pure permutation of 32-bit words: blocks of 16 rows x one load unit
// (512 / bits K elements, 16 words per row) are stored [expert][row / 16][unit]
// and, inside a block, every lane's words sit together in the order the lane
// consumes them, so one 16-byte load per lane and unit replaces the strided
// loads and the cross-lane regrouping of the checkpoint layout, and a wave's
// load covers 1 KB of contiguous memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "layout.hpp"

namespace wna16 {

namespace {

constexpr int kPrepThreads = 256;

// One thread per output word; a grid-stride loop covers any size.
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(
    const uint32_t *__restrict__ packed, uint32_t *__restrict__ out, size_t total, int kw,
    int nunits, int bits, int gs)
{
    const bool split = bits == 2 && gs == 32;
    const size_t stride = (size_t)gridDim.x * kPrepThreads;
    for (size_t o = (size_t)blockIdx.x * kPrepThreads + threadIdx.x; o < total; o += stride) {
        const size_t block = o / kPrepBlockDwords;
        const int w = (int)(o % kPrepBlockDwords);
        const int u = (int)(block % (size_t)nunits);
        const size_t rblock = block / (size_t)nunits;      // expert * rows / 16 + row / 16
        int c, g, t;
        if (split) {
            const int slot = w / 8;                        // h * 16 + c
            t = w % 8;
            c = slot % 16;
            g = 2 * (slot / 16);
        } else {
            const int lane = w / 4;                        // g * 16 + c
            t = w % 4;
            c = lane % 16;
            g = lane / 16;
        }
        const size_t row = rblock * 16 + (size_t)c;
        out[o] = packed[row * (size_t)kw + (size_t)u * 16 + prep_src_dword(bits, gs, g, t)];
    }
}

}  // namespace

hipError_t launch_prepare(const uint32_t *packed, int E, int rows, int K, int bits, int group,
                          uint32_t *prepared, hipStream_t stream)
{
    const int kw = K * bits / 32;
    const int nunits = K / (512 / bits);
    const size_t total = (size_t)E * rows * kw;
    if (total == 0)
        return hipSuccess;
    size_t blocks = (total + kPrepThreads - 1) / kPrepThreads;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream,
                       packed, prepared, total, kw, nunits, bits, group);
    return hipGetLastError();
}

}  // namespace wna16
