// gfx950 (CDNA4) kernels of the routed WNA16 MoE layer.
//
// Data flow of one forward call (all on the caller's stream):
//   route    block 0: stable counting sort of the (token, slot) pairs into
//            expert-contiguous tiles of block_m rows; other blocks: copy x into
//            MFMA fragment order with a per-group bias term, and zero the FP32
//            accumulator.
//   w13      per (tile, column block): decode-shaped 4-row tiles stream packed
//            codes straight from HBM into registers; prefill-shaped 64-row
//            tiles copy every operand into an LDS ring.  Both unpack codes to
//            biased BF16, run 16x16x32 BF16 MFMA chains per K group, scale each
//            group's partial product once in FP32, and end in a
//            SwiGLU(alpha, beta, clamp) epilogue -> BF16 act in fragment order
//            plus its per-group bias term.
//   w2       per (tile, column block): same GEMM over act; the epilogue adds
//            routing_weight * y into out_f32 with FP32 atomics.
//   convert  out_f32 -> BF16 (round to nearest even).
//
// Weight format (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What
// changed"): signed b-bit codes, field i of word j = K index j*(32/b)+i,
// stored as q + 2^(b-1); FP16 scale per K group.  The MFMA never sees q
// directly: a field u becomes the BF16 number 128 + u with one shift, mask and
// OR per two codes (0x4300 is BF16 128.0 and has seven zero mantissa bits).
// Per row and group the operand is then q + c with c = 128 + 2^(b-1), so
//   sum_k x_k q_k = sum_k x_k (q_k + c) - c * sum_k x_k,
// and the MFMA chain of each group starts from -c * sum_k x_k (precomputed per
// activation row and group) instead of zero.  Products are exact in FP32 and
// the group result is multiplied by its FP16 scale once.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "layout.hpp"

namespace wna16 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;


constexpr int kMaxExperts = 1024;
constexpr int kAlignThreads = 1024;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}

__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// BF16 value `h` divided by 2^e (exact unless it underflows).
__device__ __forceinline__ uint32_t bf16_scaled(uint32_t h, int e)
{
    return e == 0 ? h : f32_to_bf16(bf16_to_f32(h) * __builtin_ldexpf(1.0f, -e));
}

// ---------------------------------------------------------------------------
// Stable expert sort of the pairs, on one or more workgroups of 1024 threads.
//
// Workgroup w places the pairs [w*chunk, (w+1)*chunk).  Every
// workgroup first counts all pairs per expert (the padded exclusive scan of
// those counts gives the expert offsets) and, separately, the pairs before
// its own range; its pairs of expert e then start at offset[e] + (pairs of e
// before the range).  Inside the range, pairs are taken 1024 at a time in
// index order: a pair's rank among equal experts = (equal experts in earlier
// waves of the step) + (equal experts in earlier lanes of its wave).  The
// lane part comes from 11 ballots (one per bit of the expert id), the wave
// part from a per-wave, per-expert count table in LDS.  The result equals a
// stable counting sort whatever the number of workgroups.
// ---------------------------------------------------------------------------
struct AlignShared {
    int cnt[kMaxExperts];
    int pre[kMaxExperts];
    int off[kMaxExperts + 1];
    int run[kMaxExperts];
    int wsum[kAlignThreads / 64];
    int bad;
    uint8_t wcnt[kAlignThreads / 64][kMaxExperts];
};

// Lanes of the wave holding the same 11-bit key as this lane.
__device__ __forceinline__ uint64_t match_key(int key)
{
    uint64_t m = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) {
        const uint64_t bb = __ballot((key >> bit) & 1);
        m &= ((key >> bit) & 1) ? bb : ~bb;
    }
    return m;
}

__device__ void align_block(AlignShared &sh, const int32_t *__restrict__ ids, int P, int E,
                            int bm, int32_t *__restrict__ sorted_ids,
                            int32_t *__restrict__ tile_expert, int32_t *__restrict__ offsets,
                            int32_t *__restrict__ inv_perm, int32_t *__restrict__ num_tiles,
                            int32_t *__restrict__ bad_ids, int blk, int nblk, int chunk,
                            const int32_t *__restrict__ chunk_counts = nullptr)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = kAlignThreads / 64;
    const int begin = blk * chunk;
    const int end = min(P, begin + chunk);
    for (int e = tid; e < kMaxExperts; e += kAlignThreads) {
        sh.cnt[e] = 0;
        sh.pre[e] = 0;
        for (int w = 0; w < NW; ++w)
            sh.wcnt[w][e] = 0;
    }
    if (tid == 0)
        sh.bad = 0;
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (chunk_counts != nullptr) {
        // counts of all pairs and of the pairs before this range, from the
        // per-chunk counts
        for (int e = tid; e <= E; e += kAlignThreads) {
            int all = 0, before = 0;
            for (int b = 0; b < nblk; ++b) {
                const int c = chunk_counts[(size_t)b * (E + 1) + e];
                all += c;
                before += b < blk ? c : 0;
            }
            if (e < E) {
                sh.cnt[e] = all;
                sh.pre[e] = before;
            } else {
                sh.bad = all;
            }
        }
    }
    // counts of all pairs and of the pairs before this workgroup's range;
    // one atomic per distinct expert of each wave
    for (int base = 0; chunk_counts == nullptr && base < P; base += kAlignThreads) {
        const int p = base + tid;
        const int e = p < P ? ids[p] : -1;
        const bool ok = p < P && e >= 0 && e < E;
        const uint64_t m = match_key(ok ? e : kMaxExperts);
        if (ok && (m & below) == 0) {
            const int c = __popcll(m);
            atomicAdd(&sh.cnt[e], c);
            if (base < begin)   // ranges start on multiples of kAlignThreads
                atomicAdd(&sh.pre[e], c);
        }
        if (!ok && p < P)
            atomicAdd(&sh.bad, 1);
    }
    __syncthreads();

    // exclusive scan of the padded counts (one expert per thread)
    const int padded = tid < E ? (sh.cnt[tid] + bm - 1) / bm * bm : 0;
    int incl = padded;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += y;
    }
    if (lane == 63)
        sh.wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < NW; ++w) {
            const int v = sh.wsum[w];
            sh.wsum[w] = acc;
            acc += v;
        }
        sh.off[E] = acc;
    }
    __syncthreads();
    if (tid < E) {
        sh.off[tid] = sh.wsum[wave] + incl - padded;
        sh.run[tid] = sh.off[tid] + sh.pre[tid];
    }
    __syncthreads();
    const int total = sh.off[E];
    if (blk == 0) {
        for (int e = tid; e <= E; e += kAlignThreads)
            offsets[e] = sh.off[e];
        if (tid == 0) {
            *num_tiles = total / bm;
            *bad_ids = sh.bad;
        }
    }
    // tile experts and padding slots: this workgroup's share of the slots
    const int share = (total + nblk - 1) / nblk;
    for (int s = blk * share + tid; s < min(total, (blk + 1) * share); s += kAlignThreads) {
        int lo = 0, hi = E - 1;  // last e with off[e] <= s
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.off[mid] <= s)
                lo = mid;
            else
                hi = mid - 1;
        }
        if (s % bm == 0)
            tile_expert[s / bm] = lo;
        if (s - sh.off[lo] >= sh.cnt[lo])
            sorted_ids[s] = P;
    }
    // stable placement of this workgroup's pairs
    for (int base = begin; base < end; base += kAlignThreads) {
        const int p = base + tid;
        const int e = p < end ? ids[p] : -1;
        const bool ok = p < end && e >= 0 && e < E;
        const uint64_t m = match_key(ok ? e : kMaxExperts);  // invalid lanes share one key
        const int rank = __popcll(m & below);
        const bool leader = (m & below) == 0;
        const int cw = __popcll(m);
        if (ok && leader)
            sh.wcnt[wave][e] = (uint8_t)cw;
        __syncthreads();
        if (ok) {
            int before = 0;
            for (int w = 0; w < wave; ++w)
                before += sh.wcnt[w][e];
            const int slot = sh.run[e] + before + rank;
            sorted_ids[slot] = p;
            inv_perm[p] = slot;
        } else if (p < end) {
            inv_perm[p] = -1;
        }
        __syncthreads();
        if (ok && leader) {
            atomicAdd(&sh.run[e], cw);  // leaders of several waves may share an expert
            sh.wcnt[wave][e] = 0;
        }
        __syncthreads();
    }
}

// Up to this many pairs, the first wave of the sort workgroup sorts them on
// its own (align_wave) and the other waves leave at once.
constexpr int kWaveSortPairs = 64;

// Orders LDS accesses of different lanes of one wave (a wave's LDS
// instructions complete in issue order; this keeps the compiler from moving
// them across and waits for the outstanding ones).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// The stable expert sort of P <= 64 pairs by one wave (lane p holds pair p),
// with the same results as align_block.  A pair's rank among the pairs of its
// expert is the number of earlier lanes holding the same id (the ballot match
// of align_block); the first of them (the leader) records the expert's padded
// count in LDS and later writes the expert's tiles and padding slots.  The
// expert offsets are a wave-level exclusive scan over per-lane runs of
// ceil(E / 64) consecutive experts.  No workgroup barrier is needed.
__device__ void align_wave(int *__restrict__ sh_cnt, int *__restrict__ sh_off,
                           const int32_t *__restrict__ ids, int P, int E, int bm,
                           int32_t *__restrict__ sorted_ids, int32_t *__restrict__ tile_expert,
                           int32_t *__restrict__ offsets, int32_t *__restrict__ inv_perm,
                           int32_t *__restrict__ num_tiles, int32_t *__restrict__ bad_ids)
{
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int e = lane < P ? ids[lane] : -1;
    const bool ok = lane < P && e >= 0 && e < E;
    const uint64_t m = match_key(ok ? e : kMaxExperts);   // invalid lanes share one key
    const int rank = __popcll(m & below);
    const bool leader = ok && (m & below) == 0;
    const int cnt = __popcll(m);
    const int padded = (cnt + bm - 1) / bm * bm;
    const int nbad = __popcll(__ballot(lane < P && !ok));

    for (int i = lane; i < E; i += 64)
        sh_cnt[i] = 0;
    wave_lds_sync();
    if (leader)
        sh_cnt[e] = padded;
    wave_lds_sync();
    const int per = (E + 63) / 64;
    const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
    int run = 0;
    for (int i = e0; i < e1; ++i)
        run += sh_cnt[i];
    int incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += y;
    }
    int acc = incl - run;
    for (int i = e0; i < e1; ++i) {
        const int c = sh_cnt[i];
        sh_off[i] = acc;
        offsets[i] = acc;
        acc += c;
    }
    const int total = __shfl(incl, 63, 64);
    if (lane == 0) {
        offsets[E] = total;
        *num_tiles = total / bm;
        *bad_ids = nbad;
    }
    wave_lds_sync();
    if (ok) {
        const int base = sh_off[e];
        sorted_ids[base + rank] = lane;
        inv_perm[lane] = base + rank;
        if (leader) {
            for (int s = base + cnt; s < base + padded; ++s)
                sorted_ids[s] = P;
            for (int t = base / bm; t < (base + padded) / bm; ++t)
                tile_expert[t] = e;
        }
    } else if (lane < P) {
        inv_perm[lane] = -1;
    }
}

// The tile layout align_wave writes, for one tile only, computed by one wave
// from the ids (P <= 64, lane p holds pair p): the tile count, the expert of
// tile b (-1 past the last tile) and its kDecodeRows pair indices (P for
// padding slots).  Every lane returns the same values.  Tiles list the
// experts in ascending order, each expert's pairs in ascending pair order,
// padded to multiples of 4 rows, so a pair's slot is (valid pairs with a
// smaller id) + (padding of the smaller ids' experts) + (its rank among its
// own id's pairs).  One pass over the 11 bits of the keys, most significant
// first, with a ballot per bit, gives every lane the mask of lanes with a
// smaller key and the mask of lanes with its own key; the padding of each
// expert (0..3 rows) is counted with two more ballots over the experts' first
// lanes.
__device__ __forceinline__ void wave_tile_lookup(const int32_t *__restrict__ ids, int P, int E,
                                                 int b, int &ntiles, int &expert,
                                                 int (&pair)[kDecodeRows])
{
    static_assert(kDecodeRows == 4, "padding counted in two bits");
    static_assert(kMaxExperts == 1024, "keys of 11 bits");
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int id = lane < P ? ids[lane] : -1;
    const bool ok = lane < P && id >= 0 && id < E;
    const int key = ok ? id : kMaxExperts;   // invalid lanes share the largest key
    uint64_t less = 0, same = ~0ull;
#pragma unroll
    for (int bit = 10; bit >= 0; --bit) {
        const bool mine = (key >> bit) & 1;
        const uint64_t ones = __ballot(mine);
        if (mine)
            less |= same & ~ones;   // same prefix so far, 0 where this lane has 1
        same &= mine ? ones : ~ones;
    }
    const uint64_t valid = __ballot(ok);
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    const bool leader = ok && rank == 0;
    const int pad = leader ? (kDecodeRows - cnt % kDecodeRows) % kDecodeRows : 0;
    const uint64_t pad1 = __ballot(pad & 1), pad2 = __ballot(pad & 2);
    const int off = __popcll(less & valid) + __popcll(less & pad1) + 2 * __popcll(less & pad2);
    ntiles = (__popcll(valid) + __popcll(pad1) + 2 * __popcll(pad2)) / kDecodeRows;
    const int s0 = b * kDecodeRows;
    const uint64_t own = __ballot(leader && off <= s0 && s0 < off + cnt + pad);
    expert = -1;
#pragma unroll
    for (int r = 0; r < kDecodeRows; ++r)
        pair[r] = P;
    if (own != 0) {
        const int L = __ffsll((unsigned long long)own) - 1;
        expert = __builtin_amdgcn_readlane(key, L);
        const int first = s0 - __builtin_amdgcn_readlane(off, L);   // rank of the tile's slot 0
#pragma unroll
        for (int r = 0; r < kDecodeRows; ++r) {
            const uint64_t hit = __ballot(key == expert && rank == first + r);
            pair[r] = hit != 0 ? __ffsll((unsigned long long)hit) - 1 : P;
        }
    }
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t *__restrict__ ids, int P, int E, int bm, int32_t *__restrict__ sorted_ids,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ offsets,
    int32_t *__restrict__ inv_perm, int32_t *__restrict__ num_tiles,
    int32_t *__restrict__ bad_ids, int chunk)
{
    __shared__ AlignShared sh;
    if (P <= kWaveSortPairs) {
        if (threadIdx.x < 64)
            align_wave(sh.cnt, sh.off, ids, P, E, bm, sorted_ids, tile_expert, offsets, inv_perm,
                       num_tiles, bad_ids);
        return;
    }
    align_block(sh, ids, P, E, bm, sorted_ids, tile_expert, offsets, inv_perm, num_tiles,
                bad_ids, blockIdx.x, gridDim.x, chunk);
}

// From this many sort workgroups on, the route kernel's sort takes its
// counts from align_count_kernel instead of recounting every pair.
constexpr int kCountedSortBlocks = 8;

// Workgroups the sort of P pairs runs on.
inline int align_blocks(int P) { return align_chunks(P); }

// Per-chunk expert counts (and invalid ids, in entry E) for the multi-
// workgroup sort inside the route kernel.
__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t *__restrict__ ids, int P, int E, int chunk, int32_t *__restrict__ counts)
{
    __shared__ int hist[kMaxExperts + 1];
    for (int e = threadIdx.x; e <= E; e += kAlignThreads)
        hist[e] = 0;
    __syncthreads();
    const int begin = blockIdx.x * chunk, end = min(P, begin + chunk);
    for (int p = begin + threadIdx.x; p < end; p += kAlignThreads) {
        const int e = ids[p];
        atomicAdd(&hist[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += kAlignThreads)
        counts[(size_t)blockIdx.x * (E + 1) + e] = hist[e];
}

// Device-coherent 4-byte store: the value is read by workgroups of the same
// launch on other XCDs.
__device__ __forceinline__ void store_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The 8 consecutive fragment positions [8q, 8q + 8) of one group, from the
// raw BF16 words `w` that frag_chunk_load fetched: position 8q + v holds the
// group element that word half (v >> 1) + 4 (v & 1) carries (see frag_src),
// divided by 2^frag_shift; `sum` gets their sum weighted by frag_bias_weight,
// in the same order as prep_x.
template <int BITS, int GS>
__device__ __forceinline__ u32x4_t frag_chunk(const u32x4_t w, int q, float &sum)
{
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int p0 = q * 8 + 2 * h;   // p0 and p0 + 1 share shift and weight
        const uint32_t lo0 = (w[h >> 1] >> (16 * (h & 1))) & 0xffffu;
        const uint32_t hi0 = (w[2 + (h >> 1)] >> (16 * (h & 1))) & 0xffffu;
        const uint32_t lo = bf16_scaled(lo0, frag_shift(BITS, GS, p0));
        const uint32_t hi = bf16_scaled(hi0, frag_shift(BITS, GS, p0));
        sum += bf16_to_f32(lo) * (float)frag_bias_weight(BITS, GS, p0);
        sum += bf16_to_f32(hi) * (float)frag_bias_weight(BITS, GS, p0);
        o[h] = lo | (hi << 16);
    }
    return o;
}

// Raw words for frag_chunk: the group elements that positions [8q, 8q + 8)
// hold, from the group's first element `grp` (16-byte aligned).  4-bit codes:
// 8 consecutive elements from g * gs / 4 + 8 s; 2-bit codes: 4 consecutive
// elements and the 4 that follow 8 later.
template <int BITS, int GS>
__device__ __forceinline__ u32x4_t frag_chunk_load(const uint16_t *grp, int q)
{
    const int pos = q * 8, st = pos >> 5, g = (pos >> 3) & 3;
    if constexpr (BITS == 4) {
        return *reinterpret_cast<const u32x4_t *>(grp + g * (GS / 4) + 8 * st);
    } else {
        const int base = GS == 32 ? 16 * (g >> 1) + 4 * (g & 1)
                                  : g * (GS / 4) + 16 * (st >> 1) + 4 * (st & 1);
        const u32x2_t a = *reinterpret_cast<const u32x2_t *>(grp + base);
        const u32x2_t b = *reinterpret_cast<const u32x2_t *>(grp + base + 8);
        return u32x4_t{a[0], a[1], b[0], b[1]};
    }
}

// x in MFMA fragment order with minus its per-group bias term, for thread
// `gid` of T * H / 8: GS / 8 consecutive threads per (token, group), 8
// fragment positions each (one 16-byte store); the group's bias term is
// summed across them with shuffles, so the threads of a group must run
// together (whole groups per wave: GS / 8 divides 64).
template <int BITS, int GS>
__device__ __forceinline__ void prep_x(const uint16_t *__restrict__ x, const Workspace &ws, int T,
                                       int H, int gid)
{
    constexpr int PL = GS / 8;
    const int ngroups = H / GS;
    const bool on = gid < T * ngroups * PL;
    const int q = gid % PL, tg = gid / PL;
    const int t = on ? tg / ngroups : 0, G = on ? tg % ngroups : 0;
    const u32x4_t raw = on ? frag_chunk_load<BITS, GS>(x + (size_t)t * H + (size_t)G * GS, q)
                           : u32x4_t{0u, 0u, 0u, 0u};
    float sum = 0.f;  // sum of (stored activation) * (its bias weight)
    const u32x4_t o = frag_chunk<BITS, GS>(raw, q, sum);
#pragma unroll
    for (int m = 1; m < PL; m <<= 1)
        sum += __shfl_xor(sum, m, 64);
    if (on) {
        u32x4_t *dst = reinterpret_cast<u32x4_t *>(ws.x_perm + (size_t)t * H + (size_t)G * GS) + q;
        float *bias = ws.x_bias + (size_t)t * ngroups + G;
        *dst = o;
        if (q == 0)
            *bias = -sum;   // stored negated: the chain start
    }
}

// ---------------------------------------------------------------------------
// Route kernel: blocks [0, nalign) sort the pairs; blocks [nalign, nalign +
// nprep) reorder x into fragment order and compute minus c * (group sum) per
// (token, w13 group); the remaining blocks zero the FP32 accumulator.
// ---------------------------------------------------------------------------
template <int BITS, int GS>
__global__ __launch_bounds__(kAlignThreads) void route_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ ids, int T, int H, int topk,
    int E, int bm, int nalign, int chunk, int nprep, size_t act_bias_n, int tdone_n, Workspace ws)
{
    __shared__ AlignShared sh;
    const int blk = blockIdx.x;
    if (blk < nalign) {
        if (T * topk <= kWaveSortPairs) {
            if (threadIdx.x < 64)
                align_wave(sh.cnt, sh.off, ids, T * topk, E, bm, ws.sorted_ids, ws.tile_expert,
                           ws.expert_offsets, ws.inv_perm, ws.meta, ws.meta + 1);
            return;
        }
        align_block(sh, ids, T * topk, E, bm, ws.sorted_ids, ws.tile_expert, ws.expert_offsets,
                    ws.inv_perm, ws.meta, ws.meta + 1, blk, nalign, chunk,
                    nalign >= kCountedSortBlocks ? ws.chunk_counts : nullptr);
        return;
    }
    if (blk < nalign + nprep) {
        prep_x<BITS, GS>(x, ws, T, H, (blk - nalign) * kAlignThreads + threadIdx.x);
        return;
    }
    // zero the accumulator and the act bias terms (the decode epilogue adds into them)
    const size_t n4 = (size_t)T * H / 4;
    const size_t nzero_threads = (size_t)(gridDim.x - nalign - nprep) * kAlignThreads;
    const size_t first = (size_t)(blk - nalign - nprep) * kAlignThreads + threadIdx.x;
    f32x4_t *o = reinterpret_cast<f32x4_t *>(ws.out_f32);
    for (size_t i = first; i < n4; i += nzero_threads)
        o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (size_t i = first; i < act_bias_n; i += nzero_threads)
        ws.act_bias[i] = 0.f;
    for (size_t i = first; i < (size_t)H / 4; i += nzero_threads)
        ws.done[i] = 0;
    for (size_t i = first; i < (size_t)tdone_n; i += nzero_threads)
        ws.tile_done[i] = 0;
    if (first == 0)
        ws.meta[2] = 0;   // fused decode waits that gave up (counted by this call)
}

// ---------------------------------------------------------------------------
// Pieces shared by the grouped WNA16 GEMM kernels.
//
// Lane l of an MFMA works on column c = l % 16 of a 16-column subtile and is
// in lane group g = l / 16.  Per K group it needs gs/4 codes of its weight
// row: the contiguous codes [g*gs/4, (g+1)*gs/4) of that group (a 2-bit
// 32-group: half of dword g/2), i.e. NDW dwords that one 16/8/4-byte load
// brings straight into registers.
// ---------------------------------------------------------------------------
struct GemmArgs {
    const uint16_t *a;        // W13: x_perm [T][K]; W2: act [slots][K]
    const float *a_bias;      // negated bias terms; W13: x_bias [T][K/gs]; W2: act_bias [slots][K/gs]
    const uint32_t *codes;    // [E][rows][K*bits/32], or the prepared block order (prepared = 1)
    const uint16_t *scales;   // [E][rows][K/gs]
    const int32_t *sorted_ids;
    const int32_t *tile_expert;
    const int32_t *num_tiles;
    const float *topk_w;      // W2 epilogue
    uint16_t *act_out;        // W13 epilogue
    float *act_bias_out;      // W13 epilogue
    float *out_f32;           // W2 epilogue
    uint16_t *out_bf16;       // W2 decode epilogue: non-null -> the last workgroup converts
    int32_t *done;            // W2 decode: finished workgroups per column block, 16 ints apart
    int32_t *tile_done;       // fused decode: w13 workgroups finished per tile, 16 ints apart
    int tile_target;          // fused decode w2: w13 workgroups per tile
    int32_t *status;          // fused decode w2: count of waits that gave up (meta word 2)
    // single-launch decode
    const int32_t *ids;       // routing ids: each workgroup looks its tile up
    int E;
    int nblk_self;            // workgroups of this GEMM per tile
    int n_pre;                // prep workgroups
    int32_t *prep_done;       // prep workgroups finished
    int32_t *blocks_done;     // down-projection column blocks finished
    int ksplit;               // w13: K slices per (tile, column block), each its own workgroup
    float *hsum;              // w13 with ksplit > 1: [tile rows][2N] FP32 pre-activations
    int32_t *split_done;      // w13 with ksplit > 1: slices finished per (tile, column block)
    int K;                    // reduction length (H for w13, I for w2)
    int N;                    // output columns (I gate columns for w13, H for w2)
    int P, topk;
    int bits_next, gs_next;   // W13 epilogue: format of the w2 operand
    float alpha, beta, clamp;
    int prepared;             // codes in the prepared block order (decode-shaped kernels only)
    const int32_t *xcd_first; // tile kernel: [9] first item of each XCD's range, then the total
};

template <int BITS, int GS>
struct CodeTraits {
    static constexpr int NDW = (GS * BITS / 128) > 0 ? GS * BITS / 128 : 1;
    static constexpr int S = GS / 32;  // MFMA steps per group
    // first dword of lane group g's codes inside group G
    static __device__ __forceinline__ int dword_off(int G, int g)
    {
        return (G * GS + g * (GS / 4)) * BITS / 32;
    }
};

// Constants of the code unpack held in registers the compiler cannot fold
// (produced once by a volatile move), so that (x & mask) | magic is selected
// as one v_and_or_b32: a VOP3 instruction cannot encode two literals.  The
// unpack itself stays ordinary code, so the compiler's hazard rules (e.g. a
// VALU write to an in-flight MFMA's accumulator input) still apply to it.
struct UnpackConsts {
    uint32_t magic;   // SGPR: BF16 128.0 in both halves
    uint32_t m3, mc, m30, mf;  // VGPRs: 0x00030003, 0x000C000C, 0x00300030, 0x000F000F
};

__device__ __forceinline__ UnpackConsts unpack_consts()
{
    UnpackConsts k;
    asm volatile("s_mov_b32 %0, 0x43004300" : "=s"(k.magic));
    asm volatile("v_mov_b32 %0, 0x00030003" : "=v"(k.m3));
    asm volatile("v_mov_b32 %0, 0x000c000c" : "=v"(k.mc));
    asm volatile("v_mov_b32 %0, 0x00300030" : "=v"(k.m30));
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.mf));
    return k;
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic)
{
    return (x & mask) | magic;
}

// Biased BF16 fragment of MFMA step s: 4-bit fields give 128 + u; 2-bit
// fields give 128 + m*u with the m of frag_shift (see layout.hpp).
template <int BITS, int GS, int NDW>
__device__ __forceinline__ bf16x8_t unpack(const uint32_t (&cw)[NDW], int s, int g,
                                           const UnpackConsts &k)
{
    u32x4_t r;
    if constexpr (BITS == 4) {
        const uint32_t d = cw[s];
        r[0] = and_or(d, k.mf, k.magic);
#pragma unroll
        for (int i = 1; i < 4; ++i)
            r[i] = and_or(d >> (4 * i), k.mf, k.magic);
    } else {
        const uint32_t d = (GS == 32) ? cw[0] : cw[s >> 1];
        const int h = (GS == 32) ? (g & 1) : (s & 1);
        if (h == 0) {  // field pairs 0, 1, 2 (word) and 3 (word >> 6)
            r[0] = and_or(d, k.m3, k.magic);
            r[1] = and_or(d, k.mc, k.magic);
            r[2] = and_or(d, k.m30, k.magic);
            r[3] = and_or(d >> 6, k.m3, k.magic);
        } else {       // field pairs 4, 5 (word >> 6) and 6, 7 (word >> 12)
            const uint32_t d6 = d >> 6, d12 = d >> 12;
            r[0] = and_or(d6, k.mc, k.magic);
            r[1] = and_or(d6, k.m30, k.magic);
            r[2] = and_or(d12, k.m3, k.magic);
            r[3] = and_or(d12, k.mc, k.magic);
        }
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

// FP32 -> BF16 (round to nearest even) of 4 consecutive values.
__device__ __forceinline__ u32x2_t to_bf16x4(const f32x4_t v)
{
    u32x2_t o;
    o[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    o[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    return o;
}

// The sigmoid's reciprocal is the hardware approximation (v_rcp_f32, about
// 1 ulp) instead of an IEEE division, whose fix-up sequence cost 4-5 % of the
// prefill gate/up launch; the result still feeds a BF16 rounding.
__device__ __forceinline__ float swiglu(float g, float u, float alpha, float beta, float clamp)
{
    const float gc = fminf(g, clamp);
    const float uc = fminf(fmaxf(u, -clamp), clamp);
    return gc * __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * gc)) * (uc + beta);
}

// ---------------------------------------------------------------------------
// Prefill-shaped grouped WNA16 GEMM ("tile" kernel).
//
// Workgroup = 8 waves on one tile of up to 64 (token, slot) rows of one
// expert and 512 weight rows (w13: 256 gate rows and the 256 matching up
// rows; w2: 512 output columns).  The waves split the weight rows (64 each,
// four 16-column subtiles), so every wave multiplies all of the tile's row
// subtiles: each unpacked code fragment feeds up to 4 MFMAs.  Row subtiles
// beyond the tile's real rows are skipped, so a 5-row expert costs one
// subtile, not four.
//
// K runs in chunks of 128.  Every operand of a chunk -- activation rows
// (already in fragment order), codes, scales and the rows' bias terms -- is
// copied from memory straight into LDS (global_load_lds, no registers) in
// the order the MFMA lanes read it, so each read is one ds_read.  The copies
// run up to STAGES - 1 chunks ahead (1 to 3) through a ring of LDS stages
// with explicit vmcnt waits, spread in small batches over the chunk's work.
//
// Work per chunk and wave: read the chunk's codes and unpack them to BF16
// fragments (VALU), then run the chains of every active row subtile and fold
// each group's chain into the FP32 accumulators with its scale (MFMA, with
// the fold and the next subtile's LDS reads under the MFMAs).  Both waves of
// a SIMD do the same; one barrier per chunk keeps the ring consistent.
//
// Workgroup ids are spread over the 8 XCDs round-robin by the hardware; the
// kernel gives each XCD a contiguous run of (tile, column block) items,
// tile-major, so one XCD's L2 serves both the column blocks of a tile
// (activation reuse) and consecutive tiles of one expert (weight reuse).  The
// runs are cut by estimated cost, not by count (split_kernel).
// ---------------------------------------------------------------------------
// LDS address (byte offset in the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}

// Copies from global memory straight into LDS (gfx950 global_load_lds):
// lane l's `bytes` bytes at base + voff land at LDS address lds + l * 16
// (16-byte copies) or lds + l * 4 (4- and 2-byte copies: every lane writes a
// whole dword slot; a 2-byte value sits in the slot's low half).
// `base` and `lds` are wave-uniform.  Written as inline asm so that the
// compiler does not track them: it would otherwise make every later LDS read
// wait for all copies in flight, which defeats the multi-stage ring.  The
// caller waits for them with vmcnt.  (M0 is set here; nothing else in these
// kernels keeps a value in M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(const void *base_in, uint32_t voff, uint32_t lds_in)
{
    // both are wave-uniform by construction; make that explicit for the
    // scalar-register operands
    // (readfirstlane returns int: cast to uint32_t before widening, or a low
    // half with bit 31 set would be sign-extended into the high half)
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_in);
    const uint64_t b64 = reinterpret_cast<uintptr_t>(base_in);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b64 >> 32));
    const void *base = reinterpret_cast<const void *>(((uint64_t)hi << 32) | (uint64_t)lo);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
                     "s"(lds)
                     : "memory", "m0");
    else if constexpr (BYTES == 4)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base),
                     "s"(lds)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(base),
                     "s"(lds)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

template <int BITS, int GS, bool W13>
struct Tile {
    static constexpr int BM = 64, MT = 4, NT = 4, NW = 8, NTHREADS = NW * 64;
    static constexpr int BN = NW * NT * 16;          // weight rows per workgroup (512)
    static constexpr int OUTC = W13 ? BN / 2 : BN;   // output columns per workgroup
    static constexpr int KC = 128;                   // K per chunk
    static constexpr int KS = KC / 32;               // MFMA steps per chunk
    static constexpr int GPC = KC / GS;              // groups per chunk
    static constexpr int S = GS / 32;                // MFMA steps per group
    static constexpr int NDW = CodeTraits<BITS, GS>::NDW;
    static constexpr int RB = KC * BITS / 8;         // code bytes of one row per chunk
    static constexpr int PIECES = RB / 16;           // 16-byte pieces per row and chunk
    static constexpr int ACT_STRIDE = OUTC + 8;      // W13 epilogue tile, bf16 elements
    static constexpr int kXcds = 8;

    // LDS: a ring of STAGES stages, each holding one chunk:
    //   A      [subtile][step][lane] 16-byte MFMA fragments              16 KB
    //   codes  [wave][subtile row][RB bytes], 16-byte pieces swizzled    NW*64*RB
    //   scales [wave][group][lane] dword slots, FP16 in the low half,
    //          lane = column * 4 + subtile                                NW*GPC*256
    //   bias   [group][row] FP32 (the chain start: minus the bias term)  GPC*256
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = MT * KS * 64 * 16;
    static constexpr int B_WAVE = 64 * RB;
    static constexpr int SC_OFF = B_OFF + NW * B_WAVE;
    static constexpr int SC_WAVE = GPC * 64 * 4;
    static constexpr int BI_OFF = SC_OFF + NW * SC_WAVE;
    static constexpr int STAGE = BI_OFF + GPC * 64 * 4;
    static constexpr int kLdsBudget = 160 * 1024 - 2048;   // the rest holds the row table
    static constexpr int STAGES = kLdsBudget / STAGE >= 4 ? 4 : kLdsBudget / STAGE;
    static_assert(STAGES >= 2, "two chunks must fit in LDS");
    static constexpr int LDS_BYTES = STAGES * STAGE;

    struct EpiW13 {
        uint16_t act[BM * ACT_STRIDE];
        float part[BM * (OUTC / 8)];
    };
    static_assert(sizeof(EpiW13) <= LDS_BYTES, "epilogue tile overlays the ring");
    struct Rows {
        int pair[BM];
        int src[BM];
        int real;
        size_t orow[BM];   // staged w2 epilogue: the output row's offset (token * N)
        float w[BM];       // staged w2 epilogue: the routing weight
    };
    // The w2 epilogue stages each wave's 64 x 64 result through LDS when the
    // ring can hold all eight (rows padded to 68 floats against bank
    // conflicts): then every atomic instruction adds 64 consecutive floats of
    // one output row, two full cache lines, instead of 16 floats of each of
    // 4 rows.  The FP32 atomics are performed per line, so this halves their
    // count (prefill w2 launches 7-8 % shorter).  Group-32 formats, whose
    // rings are smaller, keep the direct form.
    static constexpr int EPI_STRIDE = 68;
    static constexpr bool STAGED_EPI = LDS_BYTES >= NW * 64 * EPI_STRIDE * 4;

    // 16-byte piece position inside a row's chunk of codes: XOR-swizzled so
    // that the 8 (or 16) lanes of one LDS access phase hit distinct banks.
    static __host__ __device__ constexpr int swz(int row) { return PIECES == 4 ? (row >> 1) & 3 : (row >> 2) & 1; }

    // Per-lane copy sources: 32-bit byte offsets from workgroup-uniform
    // bases.  Padding rows and idle waves point at valid rows.
    struct Ctx {
        const uint16_t *a;
        const uint32_t *codes;      // this expert's codes
        const uint16_t *scales;     // this expert's scales
        const float *bias;          // bias terms of the A rows
        uint32_t aoff[2];           // A pieces this lane copies: row and K offset (bytes)
        uint32_t coff[4];           // code rows this lane copies (byte offsets)
        uint32_t soff;              // scale row this lane copies (byte offset)
        uint32_t boff;              // bias row this lane copies (byte offset)
        uint32_t ring;              // LDS address of the ring
        int b, nb, col0, tid, lane, wave, g;
        bool wave_on;
    };

    static __device__ __forceinline__ void workgroup_barrier()
    {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    template <int N>
    static __device__ __forceinline__ void wait_vm()
    {
        static_assert(N >= 0 && N < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    }

    // Copies each wave issues per chunk: A pieces (16 slots shared by 8
    // waves; slots of inactive subtiles get harmless copies so every wave
    // issues the same number), its code pieces, its scales (one 2-byte copy
    // per group) and one bias copy.
    template <int MTA>
    static constexpr int a_copies() { return MTA <= 2 ? 1 : 2; }
    template <int MTA>
    static constexpr int copies() { return a_copies<MTA>() + PIECES + GPC + 1; }

    // Copy item `idx` of chunk kc into `stage` (A pieces, then code pieces,
    // then scales, then bias terms).  Callers pass a compile-time index
    // (unrolled loops), so the branches fold away.
    template <int MTA>
    static __device__ __forceinline__ void copy_item(int idx, int stage, const Ctx &cx, int kc)
    {
        constexpr int NA = a_copies<MTA>();
        const uint32_t st = cx.ring + stage * STAGE;
        if (idx < NA) {
            const int slot = cx.wave + NW * idx;   // [subtile][step]
            copy_to_lds<16>(cx.a, cx.aoff[idx] + (uint32_t)kc * (KC * 2),
                            st + A_OFF + slot * 64 * 16);
        } else if (idx < NA + PIECES) {
            const int k = idx - NA;
            copy_to_lds<16>(cx.codes, cx.coff[k] + (uint32_t)kc * RB,
                            st + B_OFF + cx.wave * B_WAVE + k * 64 * 16);
        } else if (idx < NA + PIECES + GPC) {
            const int G = idx - NA - PIECES;
            copy_to_lds<2>(cx.scales, cx.soff + (uint32_t)(kc * GPC + G) * 2u,
                           st + SC_OFF + (cx.wave * GPC + G) * 256);
        } else {
            // every wave copies the bias terms of group wave % GPC (waves
            // with the same group write identical values)
            const int G = cx.wave % GPC;
            copy_to_lds<4>(cx.bias, cx.boff + (uint32_t)(kc * GPC + G) * 4u,
                           st + BI_OFF + G * 256);
        }
    }
    // Copies of one chunk still to be issued: the chunk's stage and the
    // chunk whose data goes there (past the last chunk, a repeat of the last
    // chunk into a stage nobody reads any more, which keeps the number of
    // copies per phase constant).
    struct Pending {
        int stage, kc;
    };
    template <int MTA>
    static __device__ __forceinline__ void copy_items(int first, int last, const Ctx &cx,
                                                      const Pending &pc)
    {
#pragma unroll
        for (int t = first; t < last; ++t)
            copy_item<MTA>(t, pc.stage, cx, pc.kc);
    }

    // VALU half: the chunk's codes of this wave's rows, unpacked into the
    // B fragments of all KS steps; copy items [C0, C1) of `pc` are spread
    // over it.  Ends by reading the first row subtile's activation
    // fragments and bias terms for the MFMA half.
    template <int MTA, int C0, int C1>
    static __device__ __forceinline__ void unpack_chunk(const unsigned char *lds, int stage,
                                                        const Ctx &cx, bf16x8_t (&bf)[NT][KS],
                                                        const UnpackConsts &magic,
                                                        const Pending &pc, bf16x8_t (&af)[KS],
                                                        f32x4_t (&nb)[GPC])
    {
        const int g = cx.g, c = cx.lane & 15;
        const unsigned char *st = lds + stage * STAGE;
        const unsigned char *bw = st + B_OFF + cx.wave * B_WAVE;
        // all code reads first (the copies below are ordered asm statements
        // the compiler does not move reads across), then the unpack
        uint32_t q[NT][GPC][NDW];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int row = j * 16 + c;
#pragma unroll
            for (int G = 0; G < GPC; ++G) {
                const int off = CodeTraits<BITS, GS>::dword_off(G, g) * 4;   // inside the row's chunk
                const unsigned char *src =
                    bw + row * RB + (((off >> 4) ^ swz(row)) << 4) + (off & 15);
                if constexpr (NDW == 4) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src);
                    q[j][G][0] = v[0];
                    q[j][G][1] = v[1];
                    q[j][G][2] = v[2];
                    q[j][G][3] = v[3];
                } else if constexpr (NDW == 2) {
                    const u32x2_t v = *reinterpret_cast<const u32x2_t *>(src);
                    q[j][G][0] = v[0];
                    q[j][G][1] = v[1];
                } else {
                    q[j][G][0] = *reinterpret_cast<const uint32_t *>(src);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
#pragma unroll
            for (int G = 0; G < GPC; ++G)
#pragma unroll
                for (int s = 0; s < S; ++s)
                    bf[j][G * S + s] = unpack<BITS, GS, NDW>(q[j][G], s, g, magic);
            copy_items<MTA>(C0 + j * (C1 - C0) / NT, C0 + (j + 1) * (C1 - C0) / NT, cx, pc);
        }
        load_subtile(st, cx, 0, af, nb);
    }

    // Activation fragments and (for groups of 64 or more) bias terms of row
    // subtile i.
    static constexpr bool PRE_BIAS = GPC <= 2;
    static __device__ __forceinline__ void load_subtile(const unsigned char *st, const Ctx &cx,
                                                        int i, bf16x8_t (&af)[KS],
                                                        f32x4_t (&nb)[GPC])
    {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            af[s] = *reinterpret_cast<const bf16x8_t *>(st + A_OFF +
                                                       ((i * KS + s) * 64 + cx.lane) * 16);
        if constexpr (PRE_BIAS) {
#pragma unroll
            for (int G = 0; G < GPC; ++G)
                nb[G] = *reinterpret_cast<const f32x4_t *>(
                    st + BI_OFF + (G * 64 + i * 16 + 4 * cx.g) * 4);
        }
    }

    // MFMA half: for each active row subtile and group, one chain per column
    // subtile starting from minus the bias term, folded into the
    // accumulators with the group's scale.  The next subtile's operands are
    // read while the current one's MFMAs run, the last fold of a subtile runs
    // under the next subtile's MFMAs, and copy items [C0, C1) of `pc` are
    // spread over the subtiles.  af / nb hold subtile 0's operands on entry.
    template <int MTA, int C0, int C1>
    static __device__ __forceinline__ void mfma_chunk(const unsigned char *lds, int stage,
                                                      const Ctx &cx, const bf16x8_t (&bf)[NT][KS],
                                                      f32x4_t (&acc)[MTA][NT], const Pending &pc,
                                                      bf16x8_t (&af)[KS], f32x4_t (&nb)[GPC])
    {
        const int g = cx.g, c = cx.lane & 15;
        const unsigned char *st = lds + stage * STAGE;
        // the chunk's scales, read once for all row subtiles
        u32x4_t sc[GPC];
#pragma unroll
        for (int G = 0; G < GPC; ++G)
            sc[G] = *reinterpret_cast<const u32x4_t *>(
                st + SC_OFF + ((cx.wave * GPC + G) * 64 + c * 4) * 4);
        auto scales = [&](int G) { return sc[G]; };
        f32x4_t pend[NT];   // last chain of the previous subtile, not yet folded
#pragma unroll
        for (int i = 0; i < MTA; ++i) {
            bf16x8_t an[KS];
            f32x4_t nbn[GPC];
            if (i + 1 < MTA)
                load_subtile(st, cx, i + 1, an, nbn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int G = 0; G < GPC; ++G) {
                if constexpr (!PRE_BIAS)
                    nb[G] = *reinterpret_cast<const f32x4_t *>(
                        st + BI_OFF + (G * 64 + i * 16 + 4 * g) * 4);
                f32x4_t accg[NT];
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            af[G * S + s], bf[j][G * S + s], s == 0 ? nb[G] : accg[j], 0, 0, 0);
                if (G == 0 && i > 0)
                    fold(acc[i - 1], pend, scales(GPC - 1));
                if (G + 1 < GPC) {
                    fold(acc[i], accg, scales(G));
                } else {
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        pend[j] = accg[j];
                }
            }
            copy_items<MTA>(C0 + i * (C1 - C0) / MTA, C0 + (i + 1) * (C1 - C0) / MTA, cx, pc);
            if (i + 1 < MTA) {
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    af[s] = an[s];
                if constexpr (PRE_BIAS) {
#pragma unroll
                    for (int G = 0; G < GPC; ++G)
                        nb[G] = nbn[G];
                }
            }
        }
        fold(acc[MTA - 1], pend, scales(GPC - 1));
    }

    // acc[j] += scale[j] * part[j]; scale j is the FP16 value in the low half
    // of sv[j]
    static __device__ __forceinline__ void fold(f32x4_t (&acc)[NT], const f32x4_t (&part)[NT],
                                                const u32x4_t &sv)
    {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float sc = f16_to_f32((uint16_t)(sv[j] & 0xffffu));
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[j][v] = fmaf(sc, part[j][v], acc[j][v]);
        }
    }

    static __device__ void run(const GemmArgs &args)
    {
        __shared__ __align__(16) unsigned char lds[LDS_BYTES];
        __shared__ Rows rows;
        Ctx cx;
        cx.tid = threadIdx.x;
        cx.lane = cx.tid & 63;
        cx.wave = __builtin_amdgcn_readfirstlane(cx.tid >> 6);
        cx.g = cx.lane >> 4;
        const int tid = cx.tid, lane = cx.lane;

        // (tile, column block) item of this workgroup: the jx-th of its XCD's
        // contiguous range (split_kernel balances the ranges' MFMA work)
        const int nblk = (args.N + OUTC - 1) / OUTC;
        const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
        const int item = args.xcd_first[xcd] + jx;
        if (item >= args.xcd_first[xcd + 1])
            return;
        cx.b = item / nblk;
        cx.nb = item % nblk;
        const int b = cx.b;
        const int e = args.tile_expert[b];

        if (tid < 64) {
            const int p = args.sorted_ids[b * BM + tid];
            const bool real = p < args.P;
            const int src0 = W13 ? args.sorted_ids[b * BM] / args.topk : b * BM;
            rows.pair[tid] = p;
            // padding rows copy row 0's data: their results are never stored
            rows.src[tid] = real ? (W13 ? p / args.topk : b * BM + tid) : src0;
            const uint64_t m = __ballot(real);
            if (tid == 0)
                rows.real = __popcll(m);
        }
        __syncthreads();
        const int K = args.K, ngroups = K / GS;
        cx.a = args.a;
        // A pieces: slot = wave + 8k -> subtile slot / 4, step slot % 4
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int slot = cx.wave + NW * k;
            cx.aoff[k] = (uint32_t)rows.src[(slot >> 2) * 16 + (lane & 15)] * (uint32_t)K * 2u +
                         (uint32_t)((slot & 3) * 32 + (lane >> 4) * 8) * 2u;
        }
        cx.bias = args.a_bias;
        cx.boff = (uint32_t)rows.src[lane] * (uint32_t)ngroups * 4u;
        cx.ring = lds_address(lds);

        // weight rows of this wave; a wave past the last column stays idle but
        // keeps copying (valid rows) and taking part in the barriers
        const int nrows = W13 ? 2 * args.N : args.N;
        cx.col0 = cx.nb * OUTC + cx.wave * (W13 ? NT / 2 : NT) * 16;
        cx.wave_on = cx.col0 < args.N;
        const uint32_t kw = (uint32_t)(K * BITS / 32);
        cx.codes = args.codes + (size_t)e * nrows * kw;
        cx.scales = args.scales + (size_t)e * nrows * ngroups;
        // weight row of (subtile j, column cc) of this wave
        auto wrow = [&](int j, int cc) -> uint32_t {
            if (!cx.wave_on)
                return 0u;
            if constexpr (W13)
                return (uint32_t)(cx.col0 + (j % (NT / 2)) * 16 + cc + (j >= NT / 2 ? args.N : 0));
            else
                return (uint32_t)(cx.col0 + j * 16 + cc);
        };
        // code copy k of this lane: 16-byte slot lane of rows [k*64/PIECES, ...)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int slot = k * 64 + lane;                      // in [row][position]
            const int row = slot / PIECES, pos = slot % PIECES;  // wave-local row j*16 + c
            const int piece = pos ^ swz(row);
            const uint32_t n = row < 64 ? wrow(row >> 4, row & 15) : 0u;
            cx.coff[k] = n * kw * 4u + (uint32_t)piece * 16u;
        }
        // scale copies: lane = column * 4 + subtile
        cx.soff = wrow(lane & 3, lane >> 2) * (uint32_t)ngroups * 2u;

        switch ((rows.real + 15) >> 4) {
        case 1: body<1>(lds, rows, args, cx); break;
        case 2: body<2>(lds, rows, args, cx); break;
        case 3: body<3>(lds, rows, args, cx); break;
        default: body<4>(lds, rows, args, cx); break;
        }
    }

    // The K loop and epilogue for a tile with MTA active 16-row subtiles.
    //
    // Chunk k lives in stage k % STAGES.  One barrier per chunk: after the
    // barrier that opens chunk k every wave is done with chunk k - 1, so the
    // copies of chunk k - 1 + STAGES go into its stage while chunk k is
    // unpacked and multiplied (spread over that work).  Before the next
    // barrier each wave waits for its copies of chunk k + 1; the copies
    // issued after those are always STAGES - 2 chunks' worth.
    template <int MTA>
    static __device__ void body(unsigned char *lds, Rows &rows, const GemmArgs &args,
                                const Ctx &cx)
    {
        f32x4_t acc[MTA][NT];
#pragma unroll
        for (int i = 0; i < MTA; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const UnpackConsts magic = unpack_consts();
        const int nchunks = args.K / KC;
        constexpr int L = copies<MTA>();
        constexpr int V = L / 2;   // items issued during the unpack; the rest during the MFMAs
        static_assert(STAGES * L < 64, "copies in flight exceed the wait counter");
        auto last = [&](int c) { return c < nchunks ? c : nchunks - 1; };

#pragma unroll
        for (int p = 0; p < STAGES - 1; ++p)
            copy_items<MTA>(0, L, cx, Pending{p, last(p)});
        wait_vm<(STAGES - 2) * L>();   // chunk 0

        for (int k = 0; k < nchunks; ++k) {
            bf16x8_t bf[NT][KS], af[KS];
            f32x4_t nb[GPC];
            const Pending pc{(k + STAGES - 1) % STAGES, last(k + STAGES - 1)};
            workgroup_barrier();
            unpack_chunk<MTA, 0, V>(lds, k % STAGES, cx, bf, magic, pc, af, nb);
            mfma_chunk<MTA, V, L>(lds, k % STAGES, cx, bf, acc, pc, af, nb);
            wait_vm<(STAGES - 2) * L>();   // chunk k + 1
        }
        wait_vm<0>();   // repeats of the last chunk may still be in flight
        __syncthreads();   // every wave is done with the ring

        const int rows_real = rows.real;
        if constexpr (W13) {
            epilogue_w13<MTA>(reinterpret_cast<EpiW13 *>(lds), args, acc, cx, rows_real);
        } else if constexpr (STAGED_EPI) {
            // routing-weighted scatter-add into the FP32 accumulator through
            // the LDS tile (the ring is free: every wave is past the barrier
            // above); each row's output offset and weight are computed once
            if (cx.tid < rows_real) {
                const int p = rows.pair[cx.tid];
                rows.orow[cx.tid] = (size_t)(p / args.topk) * args.N;
                rows.w[cx.tid] = args.topk_w[p];
            }
            float *tile = reinterpret_cast<float *>(lds) + cx.wave * 64 * EPI_STRIDE;
            if (cx.wave_on) {
                const int g = cx.g, c = cx.lane & 15;
#pragma unroll
                for (int i = 0; i < MTA; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            tile[(16 * i + 4 * g + v) * EPI_STRIDE + 16 * j + c] = acc[i][j][v];
            }
            __syncthreads();
            if (!cx.wave_on)
                return;
            float *out = args.out_f32 + cx.col0 + cx.lane;   // the wave's 64 columns
#pragma unroll 4
            for (int r = 0; r < rows_real; ++r)
                unsafeAtomicAdd(out + rows.orow[r], rows.w[r] * tile[r * EPI_STRIDE + cx.lane]);
        } else {
            if (!cx.wave_on)
                return;
            const int g = cx.g;
            // routing-weighted scatter-add into the FP32 accumulator
#pragma unroll
            for (int i = 0; i < MTA; ++i) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * i + 4 * g + v;
                    if (r >= rows_real)
                        continue;
                    const int p = rows.pair[r];
                    const float w = args.topk_w[p];
                    float *orow =
                        args.out_f32 + (size_t)(p / args.topk) * args.N + cx.col0 + (cx.lane & 15);
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        unsafeAtomicAdd(orow + j * 16, w * acc[i][j][v]);
                }
            }
        }
    }

    // SwiGLU on matching gate/up columns; BF16 act rows written in the w2
    // fragment order (scaled per frag_shift), with the per-group bias term of
    // each (row, w2 group): the workgroup covers whole w2 groups (gs2 <= 128).
    template <int MTA>
    static __device__ __forceinline__ void epilogue_w13(EpiW13 *epi, const GemmArgs &args,
                                                        const f32x4_t (&acc)[MTA][NT],
                                                        const Ctx &cx, int rows_real)
    {
        constexpr int NG = NT / 2;
        const int c = cx.lane & 15, g = cx.g;
        if (cx.wave_on) {
#pragma unroll
            for (int i = 0; i < MTA; ++i)
#pragma unroll
                for (int j = 0; j < NG; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float a = swiglu(acc[i][j][v], acc[i][NG + j][v], args.alpha,
                                               args.beta, args.clamp);
                        epi->act[(16 * i + 4 * g + v) * ACT_STRIDE + cx.wave * NG * 16 + j * 16 +
                                 c] = f32_to_bf16(a);
                    }
        }
        __syncthreads();
        switch (args.bits_next * 1000 + args.gs_next) {
        case 2032: act_out<2, 32>(epi, args, cx, rows_real); break;
        case 2064: act_out<2, 64>(epi, args, cx, rows_real); break;
        case 2128: act_out<2, 128>(epi, args, cx, rows_real); break;
        case 4032: act_out<4, 32>(epi, args, cx, rows_real); break;
        case 4064: act_out<4, 64>(epi, args, cx, rows_real); break;
        default: act_out<4, 128>(epi, args, cx, rows_real); break;
        }
    }

    template <int B2, int G2>
    static __device__ __forceinline__ void act_out(EpiW13 *epi, const GemmArgs &args,
                                                   const Ctx &cx, int rows_real)
    {
        const int tid = cx.tid;
        const int ncols = min(OUTC, args.N - cx.nb * OUTC);
        const int pieces = ncols / 8;
        for (int q = tid; q < rows_real * pieces; q += NTHREADS) {
            const int r = q / pieces, c8 = q % pieces;
            const int gl = (c8 * 8) / G2, q8 = ((c8 * 8) % G2) / 8;
            // the group's elements for positions [8 q8, 8 q8 + 8), from the
            // row's LDS copy (16-byte aligned groups)
            const u32x4_t raw = frag_chunk_load<B2, G2>(epi->act + r * ACT_STRIDE + gl * G2, q8);
            float sum = 0.f;
            const u32x4_t o = frag_chunk<B2, G2>(raw, q8, sum);
            *reinterpret_cast<u32x4_t *>(args.act_out + (size_t)(cx.b * BM + r) * args.N +
                                         cx.nb * OUTC + c8 * 8) = o;
            epi->part[r * (OUTC / 8) + c8] = sum;
        }
        __syncthreads();
        constexpr int per = G2 / 8;
        const int gpb = ncols / G2;  // w2 groups in this workgroup
        const int ngroups2 = args.N / G2;
        for (int q = tid; q < rows_real * gpb; q += NTHREADS) {
            const int r = q / gpb, gl = q % gpb;
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < per; ++k)
                sum += epi->part[r * (OUTC / 8) + gl * per + k];
            args.act_bias_out[(size_t)(cx.b * BM + r) * ngroups2 + cx.nb * (OUTC / G2) + gl] = -sum;
        }
    }
};

template <int BITS, int GS, bool W13>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void tile_kernel(
    const GemmArgs args)
{
    Tile<BITS, GS, W13>::run(args);
}

// ---------------------------------------------------------------------------
// Decode-shaped grouped WNA16 GEMM ("stream" kernel).
//
// Tiles hold at most 4 (token, slot) rows, so the weight stream dominates
// everything: each weight byte is used by <= 4 rows.  The whole K extent of
// the tile's activation rows and the scales of the workgroup's weight rows go
// to LDS once; after a single barrier every wave streams its own weight rows
// with a rolling register pipeline (D load units of 16 rows x 64 bytes per
// subtile in flight, no barrier until the epilogue).
//
// One load unit = dwords [16u, 16u+16) of a row: 256 codes (2-bit) or 128
// (4-bit), i.e. U/gs whole groups.  Lane group g loads 16 contiguous bytes of
// its row; v_permlane16/32_swap then regroup the dwords so that every lane
// holds, for each group of the unit, the dwords its MFMA fragments need
// (dwords [g*n, g*n + n) of the group with n = gs*bits/128).
// ---------------------------------------------------------------------------
// ONE: the single-launch decode layer (FUSED too): the tile comes from the
// routing ids; w13 stages x straight from the input rows in fragment order
// (args.a is x) and stores each act group's bias term in halves (no zeroing
// needed); w2 adds into the FP32 sum once this launch's prep workgroups have
// zeroed it; the workgroup that finishes last resets every counter.  With
// args.ksplit > 1 a w13 (tile, column block) runs as that many workgroups,
// each over one K slice: they add their partial pre-activations into
// args.hsum (zeroed by the prep) and the last one of them runs the epilogue.
template <int BITS, int GS, int NB, int D, bool W13, bool FUSED = false, bool PREP = false,
          bool ONE = false>
struct Stream {
    static constexpr int R = 4;                      // rows per tile
    static constexpr int NW = 4;                     // waves per workgroup
    static constexpr int NTHREADS = NW * 64;
    static constexpr int UK = 16 * 32 / BITS;        // K per load unit
    static constexpr int GPU = UK / GS;              // groups per unit
    static constexpr int S = GS / 32;                // MFMA steps per group
    static constexpr bool SPLIT = (BITS == 2 && GS == 32);  // half a dword per lane and group
    static constexpr int UDW = SPLIT ? 8 : 4;        // dwords a lane holds per unit and subtile
    static constexpr int COLS = W13 ? NB / 2 * 16 : NB * 16;  // output columns per wave
    static constexpr int BN = NW * COLS;             // output columns per workgroup

    // dynamic LDS: A rows, their group bias terms, the workgroup's scales
    static __host__ __device__ size_t lds_bytes(int K)
    {
        return (size_t)(R + 1) * (K + 8) * 2 + (size_t)R * (K / GS) * 4 +
               (size_t)NW * NB * 16 * (K / GS) * 2;
    }

    static __device__ __forceinline__ void load_unit(uint32_t (&dst)[NB][UDW],
                                                     const uint32_t *const *brow, int u, int g)
    {
        if constexpr (PREP) {
            // prepared blocks: this lane's words of unit u sit together, in
            // register order (brow already points at the lane's slot)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint32_t *p = brow[j] + (size_t)u * kPrepBlockDwords;
#pragma unroll
                for (int h = 0; h < UDW / 4; ++h) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p + 4 * h);
                    dst[j][4 * h + 0] = v[0];
                    dst[j][4 * h + 1] = v[1];
                    dst[j][4 * h + 2] = v[2];
                    dst[j][4 * h + 3] = v[3];
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const uint32_t *p = brow[j] + u * 16;
            if constexpr (SPLIT) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    dst[j][q] = p[2 * q + (g >> 1)];
            } else {
                int off;
                if constexpr (GPU == 2)
                    off = 8 * (g & 1) + 4 * (g >> 1);
                else
                    off = 4 * g;
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p + off);
                dst[j][0] = v[0];
                dst[j][1] = v[1];
                dst[j][2] = v[2];
                dst[j][3] = v[3];
            }
        }
    }

    // Regroup the loaded dwords across lane groups (see above).
    static __device__ __forceinline__ void regroup(uint32_t (&r)[UDW])
    {
        if constexpr (PREP) {
            // prepared blocks already hold the registers in this order
        } else if constexpr (!SPLIT && GPU == 2) {
            const auto a = __builtin_amdgcn_permlane16_swap(r[0], r[2], false, false);
            const auto b = __builtin_amdgcn_permlane16_swap(r[1], r[3], false, false);
            r[0] = a[0];
            r[2] = a[1];
            r[1] = b[0];
            r[3] = b[1];
        } else if constexpr (!SPLIT && GPU == 4) {  // 4x4 transpose over lane groups
            const auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
            const auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
            const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
            const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
            r[0] = c[0];
            r[1] = c[1];
            r[2] = d[0];
            r[3] = d[1];
        }
    }

    static __device__ __forceinline__ void take_unit(uint32_t (&r)[NB][UDW],
                                                     const uint32_t (&qd)[NB][UDW])
    {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int t = 0; t < UDW; ++t)
                r[j][t] = qd[j][t];
            regroup(r[j]);
        }
    }

    // MFMAs of one load unit: for each of its groups, the biased-code products
    // start from -c * (row group sum) and are scaled once by the group scale.
    // All LDS reads of the unit are issued first so their latency overlaps.
    static __device__ __forceinline__ void compute_unit(const uint32_t (&r)[NB][UDW], int u,
                                                        const uint16_t *sA, const float *sBias,
                                                        const uint16_t *sSw, int lds_stride,
                                                        int ngroups, int c, int g,
                                                        const UnpackConsts &magic,
                                                        f32x4_t (&acc)[NB])
    {
        bf16x8_t af[GPU][S];
        float negb[GPU];
        float sc[GPU][NB];
        // tile row r is MFMA row 4r, so result lane group g holds row g in
        // element 0; the other MFMA rows read the zero row
        const uint16_t *arow = sA + ((c & 3) == 0 ? (c >> 2) : R) * lds_stride;
#pragma unroll
        for (int gq = 0; gq < GPU; ++gq) {
            const int G = u * GPU + gq;
#pragma unroll
            for (int s = 0; s < S; ++s)
                af[gq][s] = *reinterpret_cast<const bf16x8_t *>(arow + G * GS + (s * 4 + g) * 8);
            negb[gq] = sBias[G * R + g];   // row g's chain start
#pragma unroll
            for (int j = 0; j < NB; ++j)
                sc[gq][j] = f16_to_f32(sSw[(j * 16 + c) * ngroups + G]);
        }
#pragma unroll
        for (int gq = 0; gq < GPU; ++gq) {
            f32x4_t accg[NB];
#pragma unroll
            for (int s = 0; s < S; ++s) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    uint32_t cw[4];
                    if constexpr (SPLIT) {
                        cw[0] = r[j][gq];
                    } else if constexpr (GPU == 1) {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            cw[t] = r[j][t];
                    } else if constexpr (GPU == 2) {
                        cw[0] = r[j][2 * gq];
                        cw[1] = r[j][2 * gq + 1];
                    } else {
                        cw[0] = r[j][gq];
                    }
                    constexpr int NDW = CodeTraits<BITS, GS>::NDW;
                    const bf16x8_t bf = unpack<BITS, GS, NDW>(
                        reinterpret_cast<const uint32_t(&)[NDW]>(cw), s, g, magic);
                    accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[gq][s], bf, s == 0 ? f32x4_t{negb[gq], 0.f, 0.f, 0.f} : accg[j],
                        0, 0, 0);
                }
            }
            // only element 0 holds a tile row
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j][0] = fmaf(sc[gq][j], accg[j][0], acc[j][0]);
        }
    }

    // Negated bias term (stored negated) of LDS item i = [group][row]: the
    // start of each MFMA chain (0 for padding rows).
    static constexpr int NBIAS_PRE = 2;
    static __device__ __forceinline__ float bias_item(const GemmArgs &args, int s0, int s1, int s2,
                                                      int s3, int i, int ngroups)
    {
        static_assert(R == 4, "four tile rows");
        const int G = i / R, r = i % R;
        const int sr = r == 0 ? s0 : r == 1 ? s1 : r == 2 ? s2 : s3;
        const float *bp = args.a_bias + (size_t)(sr >= 0 ? sr : 0) * ngroups + G;
        float bv;
        if constexpr (ONE && !W13) {   // the two halves the w13 items stored
            const float *bq = args.a_bias + ((size_t)(sr >= 0 ? sr : 0) * ngroups + G) * 2;
            bv = __hip_atomic_load(bq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                 __hip_atomic_load(bq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if constexpr (FUSED && !W13) {   // written by this launch's w13 items
            bv = __hip_atomic_load(bp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            bv = *bp;
        }
        return sr >= 0 ? bv : 0.f;
    }

    // 16 bytes of an activation row; device-coherent loads in the fused w2,
    // whose act rows were written by other workgroups of the same launch
    static __device__ __forceinline__ u32x4_t load_a(const uint16_t *p)
    {
        if constexpr (FUSED && !W13) {
            const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
            const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
        } else {
            return *reinterpret_cast<const u32x4_t *>(p);
        }
    }

    static __device__ void run(const GemmArgs &args, int b, int nb, int ks = 0)
    {
        extern __shared__ __align__(16) unsigned char smem[];
        int ntiles, e;
        int pair[R];
        if constexpr (ONE) {
            // the same tile layout as the route kernel's sort, from the ids
            wave_tile_lookup(args.ids, args.P, args.E, b, ntiles, e, pair);
        } else {
            // the tile count, the tile's expert and its rows load together
            // (one round trip; b < max_tiles keeps the last two in bounds,
            // their values are unused past the last tile)
            ntiles = *args.num_tiles;
            e = args.tile_expert[b];
#pragma unroll
            for (int r = 0; r < R; ++r)
                pair[r] = args.sorted_ids[b * R + r];
        }
        if (b >= ntiles) {
            // no tile at all (every id invalid): the output is the zeroed sum
            // (the single launch's prep writes it)
            if constexpr (!W13 && !ONE)
                if (args.out_bf16 && ntiles == 0 && b == 0)
                    convert_block(args, nb);
            return;
        }
        // this workgroup's K slice (the whole row unless a w13 item is split)
        const int nsplit = (ONE && W13) ? args.ksplit : 1;
        const int K = args.K / nsplit;                 // slice length
        const int kofs = ks * K;                       // slice start
        const int ngroups = K / GS;                    // groups of the slice (LDS layout)
        const int ngroups_row = args.K / GS;           // groups of a whole row (HBM strides)
        const int lds_stride = K + 8;
        // LDS: R activation rows + a zero row; the rows' negated bias terms as
        // [group][row]; the workgroup's scales
        uint16_t *sA = reinterpret_cast<uint16_t *>(smem);
        float *sBias = reinterpret_cast<float *>(smem + (size_t)(R + 1) * lds_stride * 2);
        uint16_t *sS = reinterpret_cast<uint16_t *>(smem + (size_t)(R + 1) * lds_stride * 2 +
                                                    (size_t)R * ngroups * 4);
        __shared__ float s_part[R][NW * (W13 ? NB / 2 : 1)];

        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int c = lane & 15, g = lane >> 4;
        // rows of the tile (padding rows have pair index P)
        int src[R];
        int rows_real = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool real = pair[r] < args.P;
            src[r] = real ? (W13 ? pair[r] / args.topk : b * R + r) : -1;
            rows_real += real ? 1 : 0;
        }

        // this lane's weight rows
        const int nrows = W13 ? 2 * args.N : args.N;
        const int kw = args.K * BITS / 32;
        const int nunits_row = args.K / UK;   // K % UK == 0: the plan sends other K to tile_kernel
        const int nunits = K / UK;            // units of the slice
        const int ubase = ks * nunits;        // its first unit
        const uint32_t *brow[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int n;
            if constexpr (W13)
                n = nb * BN + wave * COLS + (j % (NB / 2)) * 16 + c + (j >= NB / 2 ? args.N : 0);
            else
                n = nb * BN + wave * COLS + j * 16 + c;
            if constexpr (PREP)   // block (row / 16, first unit of the slice), this lane's slot
                brow[j] = args.codes +
                          (((size_t)e * (nrows / 16) + n / 16) * nunits_row + ubase) * kPrepBlockDwords +
                          prep_block_dword(BITS, GS, g, c, 0);
            else
                brow[j] = args.codes + ((size_t)e * nrows + n) * kw + (size_t)ubase * 16;
        }

        // ONE w2 (and split w13): whether the prep has zeroed the FP32 sums
        // this workgroup adds into, loaded early (its latency hides behind
        // the weight stream or the wait for the tile's w13 items)
        int prep_seen = 0;
        if constexpr (ONE)
            if (tid == 0 && (!W13 || nsplit > 1))
                prep_seen = __hip_atomic_load(args.prep_done, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);

        // The weight stream starts first: its HBM latency overlaps the staging.
        uint32_t q[D][NB][UDW];
#pragma unroll
        for (int d = 0; d < D; ++d)
            load_unit(q[d], brow, d, g);

        if constexpr (FUSED && !W13) {
            // the tile's act rows and bias terms come from this launch's w13
            // items: wait (bounded) until all of them are done
            if (tid == 0) {
                int32_t *cnt = args.tile_done + b * 16;
                bool ready = false;
                for (int it = 0; it < (1 << 22) && !ready; ++it) {
                    const int v =
                        __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ready = v >= args.tile_target;
                    if (!ready)
                        __builtin_amdgcn_s_sleep(2);
                }
                if constexpr (ONE) {
                    // the FP32 sum this workgroup adds into must be zeroed
                    bool zeroed = prep_seen >= args.n_pre;
                    for (int it = 0; it < (1 << 22) && !zeroed; ++it) {
                        __builtin_amdgcn_s_sleep(2);
                        zeroed = __hip_atomic_load(args.prep_done, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) >= args.n_pre;
                    }
                    ready = ready && zeroed;
                }
                // a wait that reached its bound is counted where the host can
                // read it: the act rows staged below may then be incomplete
                if (!ready)
                    __hip_atomic_fetch_add(args.status, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }

        // Activation rows (zero for padding rows), their bias terms and this
        // workgroup's scales go to LDS.  Each pass issues all of its loads
        // before its first LDS store, so the latencies overlap; the first bias
        // items load together with the first pass.  XDIRECT (single-launch
        // w13): the rows are x itself, put in fragment order here, and the
        // group bias terms are summed here (GS / 8 consecutive lanes hold one
        // group's chunks).
        constexpr bool XDIRECT = ONE && W13;
        float bpre[NBIAS_PRE];
#pragma unroll
        for (int k = 0; k < NBIAS_PRE; ++k) {
            const int i = tid + k * NTHREADS;
            bpre[k] = !XDIRECT && i < R * ngroups
                          ? bias_item(args, src[0], src[1], src[2], src[3], i, ngroups)
                          : 0.f;
        }
        {
            const int k8n = K / 8;
            const int srows = NW * NB * 16;
            const bool svec = ngroups % 8 == 0 && ngroups_row % 8 == 0 &&
                              reinterpret_cast<uintptr_t>(args.scales) % 16 == 0;
            const int sper = ngroups / 8;                  // 16-byte scale pieces per row
            const int spieces = svec ? srows * sper : 0;
            // chunks per thread and pass (one with XDIRECT: fewer live registers)
            constexpr int TP = XDIRECT ? 1 : 2;
            for (int k0 = 0; k0 < k8n || k0 < spieces; k0 += TP * NTHREADS) {
                u32x4_t v[TP][R], vs[TP];
#pragma unroll
                for (int t = 0; t < TP; ++t) {
                    const int k8 = k0 + t * NTHREADS + tid;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        v[t][r] = u32x4_t{0u, 0u, 0u, 0u};
                        if (src[r] >= 0 && k8 < k8n) {
                            if constexpr (XDIRECT)
                                v[t][r] = frag_chunk_load<BITS, GS>(
                                    args.a + (size_t)src[r] * args.K + kofs +
                                        (size_t)(k8 / (GS / 8)) * GS,
                                    k8 % (GS / 8));
                            else
                                v[t][r] = load_a(args.a + (size_t)src[r] * args.K + kofs +
                                                 (size_t)k8 * 8);
                        }
                    }
                    vs[t] = u32x4_t{0u, 0u, 0u, 0u};
                    if (k8 < spieces) {
                        const int rr = k8 / sper, kk = k8 % sper;
                        const int w = rr / (NB * 16), j = (rr / 16) % NB, cc = rr % 16;
                        int n;
                        if constexpr (W13)
                            n = nb * BN + w * COLS + (j % (NB / 2)) * 16 + cc +
                                (j >= NB / 2 ? args.N : 0);
                        else
                            n = nb * BN + w * COLS + j * 16 + cc;
                        vs[t] = *reinterpret_cast<const u32x4_t *>(
                            args.scales + ((size_t)e * nrows + n) * ngroups_row + kofs / GS +
                            kk * 8);
                    }
                }
#pragma unroll
                for (int t = 0; t < TP; ++t) {
                    const int k8 = k0 + t * NTHREADS + tid;
                    if constexpr (XDIRECT) {
                        // k8 < k8n is the same for the GS / 8 lanes of a group
                        constexpr int PL = GS / 8;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float sum = 0.f;
                            v[t][r] = frag_chunk<BITS, GS>(v[t][r], k8 % PL, sum);
#pragma unroll
                            for (int m = 1; m < PL; m <<= 1)
                                sum += __shfl_xor(sum, m, 64);
                            if (k8 < k8n && k8 % PL == 0)   // stored negated: the chain start
                                sBias[(k8 / PL) * R + r] = src[r] >= 0 ? -sum : 0.f;
                        }
                    }
                    if (k8 < k8n) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            reinterpret_cast<u32x4_t *>(sA + r * lds_stride)[k8] = v[t][r];
                        reinterpret_cast<u32x4_t *>(sA + R * lds_stride)[k8] =
                            u32x4_t{0u, 0u, 0u, 0u};
                    }
                    if (k8 < spieces)
                        *reinterpret_cast<u32x4_t *>(sS + (k8 / sper) * ngroups + (k8 % sper) * 8) =
                            vs[t];
                }
            }
            if constexpr (!XDIRECT) {
                for (int i = tid; i < R * ngroups; i += NTHREADS) {
                    if (i < NBIAS_PRE * NTHREADS)
                        continue;   // staged from the batch loaded above
                    sBias[i] = bias_item(args, src[0], src[1], src[2], src[3], i, ngroups);
                }
#pragma unroll
                for (int k = 0; k < NBIAS_PRE; ++k)
                    if (tid + k * NTHREADS < R * ngroups)
                        sBias[tid + k * NTHREADS] = bpre[k];
            }
            if (!svec) {   // scales without 16-byte alignment: one half at a time
                for (int i = tid; i < srows * ngroups; i += NTHREADS) {
                    const int rr = i / ngroups, G = i % ngroups;
                    const int w = rr / (NB * 16), j = (rr / 16) % NB, cc = rr % 16;
                    int n;
                    if constexpr (W13)
                        n = nb * BN + w * COLS + (j % (NB / 2)) * 16 + cc +
                            (j >= NB / 2 ? args.N : 0);
                    else
                        n = nb * BN + w * COLS + j * 16 + cc;
                    sS[i] = args.scales[((size_t)e * nrows + n) * ngroups_row + kofs / GS + G];
                }
            }
        }
        __syncthreads();

        const UnpackConsts magic = unpack_consts();
        f32x4_t acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const uint16_t *sSw = sS + (size_t)wave * NB * 16 * ngroups;

        // nunits is a multiple of D (checked by the host): the steady state
        // reloads every slot as soon as its unit is consumed, the last round
        // only drains.
        int u0 = 0;
        for (; u0 + D < nunits; u0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    regroup(q[d][j]);
                compute_unit(q[d], u0 + d, sA, sBias, sSw, lds_stride, ngroups, c, g, magic, acc);
                load_unit(q[d], brow, u0 + d + D, g);
                // keep the reload here: moving it later would drain the pipeline
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                regroup(q[d][j]);
            compute_unit(q[d], u0 + d, sA, sBias, sSw, lds_stride, ngroups, c, g, magic, acc);
        }

        // tile row g of every subtile lives in lane group g, element 0
        static_assert(R == 4, "one tile row per lane group");
        if constexpr (ONE && W13) {
            if (nsplit > 1) {
                // The sums this slice adds into must have been zeroed by the
                // prep (bounded wait; a give-up is counted).
                __shared__ int s_last_split;
                if (tid == 0) {
                    bool zeroed = prep_seen >= args.n_pre;
                    for (int it = 0; it < (1 << 22) && !zeroed; ++it) {
                        __builtin_amdgcn_s_sleep(2);
                        zeroed = __hip_atomic_load(args.prep_done, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) >= args.n_pre;
                    }
                    if (!zeroed)
                        __hip_atomic_fetch_add(args.status, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                // this slice's partial pre-activations (gate and up columns)
                float *hrow = args.hsum + (size_t)(b * R + g) * 2 * args.N;
                if (g < rows_real) {
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        unsafeAtomicAdd(hrow + nb * BN + wave * COLS + (j % (NB / 2)) * 16 + c +
                                            (j >= NB / 2 ? args.N : 0),
                                        acc[j][0]);
                }
                // the last slice of (tile, column block) to finish runs the
                // epilogue on the complete sums and clears the slice counter
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's atomics are done
                __syncthreads();
                if (tid == 0) {
                    int32_t *cnt = args.split_done + b * args.nblk_self + nb;
                    s_last_split = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
                    if (s_last_split)
                        __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                if (!s_last_split)
                    return;
                if (g < rows_real) {
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[j][0] = __hip_atomic_load(
                            hrow + nb * BN + wave * COLS + (j % (NB / 2)) * 16 + c +
                                (j >= NB / 2 ? args.N : 0),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if constexpr (W13) {
            constexpr int NG = NB / 2;
            const int gs2 = args.gs_next, bits2 = args.bits_next;
            const int ngroups2 = args.N / gs2;
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const int n = nb * BN + wave * COLS + j * 16 + c;  // gate column
                const int G2 = n / gs2;
                const int pin = frag_dst(bits2, gs2, n % gs2);
                const int pos = G2 * gs2 + pin;
                const int esh = frag_shift(bits2, gs2, pin);
                const float wgt = (float)frag_bias_weight(bits2, gs2, pin);
                float a = 0.f;
                if (g < rows_real) {
                    a = swiglu(acc[j][0], acc[NG + j][0], args.alpha, args.beta, args.clamp);
                    const uint32_t st = bf16_scaled(f32_to_bf16(a), esh);
                    uint16_t *dst = args.act_out + (size_t)(b * R + g) * args.N + pos;
                    if constexpr (FUSED)   // read by w2 workgroups of this launch
                        __hip_atomic_store(dst, (uint16_t)st, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *dst = (uint16_t)st;
                    a = bf16_to_f32(st) * wgt;
                }
                // sum of the 16 columns of this subtile (the lanes of group g)
#pragma unroll
                for (int m = 1; m < 16; m <<= 1)
                    a += __shfl_xor(a, m, 64);
                if (c == 0)
                    s_part[g][wave * NG + j] = a;
            }
            __syncthreads();
            // one partial sum per (row, w2 group) inside this workgroup; a group
            // wider than the workgroup gets two commutative contributions
            const int per = gs2 >= 16 ? gs2 / 16 : 1;              // subtiles per group
            const int nsub = NW * NG;                              // subtiles in the WG
            const int gspan = nsub < per ? nsub : per;
            for (int i = tid; i < rows_real * (nsub / gspan); i += NTHREADS) {
                const int v = i / (nsub / gspan), k = i % (nsub / gspan);
                float sum = 0.f;
                for (int t = 0; t < gspan; ++t)
                    sum += s_part[v][k * gspan + t];
                const int G2 = (nb * BN + k * gspan * 16) / gs2;
                if constexpr (ONE) {
                    // a group is at most two workgroups wide: each stores its half,
                    // a group inside one workgroup stores a zero second half
                    float *dst = args.act_bias_out + ((size_t)(b * R + v) * ngroups2 + G2) * 2;
                    store_coherent(dst + (gs2 > BN ? nb % 2 : 0), -sum);
                    if (gs2 <= BN)
                        store_coherent(dst + 1, 0.f);
                } else {
                    unsafeAtomicAdd(args.act_bias_out + (size_t)(b * R + v) * ngroups2 + G2,
                                    -sum);
                }
            }
            if constexpr (FUSED) {
                // act and its bias terms are performed (device scope): count
                // this workgroup done for its tile
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_fetch_add(args.tile_done + b * 16, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            if (g < rows_real) {
                const int p = g == 0 ? pair[0] : g == 1 ? pair[1] : g == 2 ? pair[2] : pair[3];
                const float w = args.topk_w[p];
                float *orow = args.out_f32 + (size_t)(p / args.topk) * args.N;
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    unsafeAtomicAdd(orow + nb * BN + wave * COLS + j * 16 + c, w * acc[j][0]);
            }
            if (args.out_bf16)
                arrive(args, ntiles, nb);
        }
    }

    // Small outputs: every workgroup counts itself done in its column block
    // once its atomics have been performed (each wave waits for them); the
    // last one of the block rounds the block's columns of every token,
    // reading them with device-coherent loads, and clears the block's
    // counter.  No cache flush is needed: the accumulator only ever changes
    // through device-scope atomics.  In the single launch the last block to
    // finish comes after every other workgroup has passed its waits: it
    // clears the prep and per-tile counters for the next call.
    static __device__ void arrive(const GemmArgs &args, int active, int nb)
    {
        __shared__ int last, fin;
        const int tid = threadIdx.x;
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's atomics are done
        __syncthreads();
        if (tid == 0)
            last = __hip_atomic_fetch_add(args.done + nb * 16, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == active - 1;
        __syncthreads();
        if (!last)
            return;
        if constexpr (ONE)
            if (tid == 0)
                fin = __hip_atomic_fetch_add(args.blocks_done, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == args.nblk_self - 1;
        convert_block(args, nb);
        if (tid == 0)
            __hip_atomic_store(args.done + nb * 16, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (ONE) {
            __syncthreads();
            if (fin) {
                for (int i = tid; i < active; i += NTHREADS)
                    __hip_atomic_store(args.tile_done + i * 16, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (tid == 0) {
                    __hip_atomic_store(args.prep_done, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(args.blocks_done, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    static __device__ void convert_block(const GemmArgs &args, int nb)
    {
        constexpr int Q = BN / 4;   // float4 per token row in the block
        const int n4 = (args.P / args.topk) * Q;
        for (int i0 = threadIdx.x; i0 < n4; i0 += 4 * NTHREADS) {
            f32x4_t v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * NTHREADS;
                const size_t e = (size_t)(i / Q) * args.N + nb * BN + (i % Q) * 4;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v[k][t] = i < n4 ? __hip_atomic_load(args.out_f32 + e + t, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                     : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * NTHREADS;
                const size_t e = (size_t)(i / Q) * args.N + nb * BN + (i % Q) * 4;
                if (i < n4)
                    *reinterpret_cast<u32x2_t *>(args.out_bf16 + e) = to_bf16x4(v[k]);
            }
        }
    }
};

template <int BITS, int GS, int NB, int D, bool W13, bool PREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void stream_kernel(
    const GemmArgs args)
{
    Stream<BITS, GS, NB, D, W13, false, PREP>::run(args, blockIdx.x, blockIdx.y);
}

// Both decode-shaped GEMMs in one launch: workgroups [0, n13) are the w13
// (tile, column block) items, tile-major, the rest the w2 items.  Workgroups
// are dispatched in id order, so every w13 item has been dispatched before
// any w2 item waits for its tile's w13 items; a w2 item streams its first
// weights while it waits.
template <int B13, int G13, int D13, int B2, int G2, int D2, bool PREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_kernel(
    const GemmArgs a13, const GemmArgs a2, int max_tiles, int nblk13, int nblk2)
{
    const int id = blockIdx.x, n13 = max_tiles * nblk13;
    if (id < n13)
        Stream<B13, G13, 2, D13, true, true, PREP>::run(a13, id / nblk13, id % nblk13);
    else
        Stream<B2, G2, 2, D2, false, true, PREP>::run(a2, (id - n13) / nblk2,
                                                      (id - n13) % nblk2);
}

// The single-launch decode's first n_pre workgroups (256 threads each):
// they zero the FP32 sum (and, with split w13 items, the partial
// pre-activation sums) with device-coherent stores and count themselves
// done (the items add into those sums only after that); then the first one's
// first wave sorts the pairs into the workspace (results the host may read;
// the GEMM items look their tiles up from the ids).  With no tile at all no
// GEMM item runs: the last prep workgroup writes the zero output and clears
// the counter itself.
__device__ void decode_prep(const GemmArgs &a13, const GemmArgs &a2, const Workspace &ws, int T,
                            int H, int max_tiles, int wg)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last, s_ntiles;
    const int tid = threadIdx.x;
    const int nthr = a13.n_pre * 256, gid = wg * 256 + tid;
    uint64_t *o = reinterpret_cast<uint64_t *>(ws.out_f32);
    for (int i = gid; i < T * H / 2; i += nthr)
        __hip_atomic_store(o + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a13.ksplit > 1) {
        uint64_t *h = reinterpret_cast<uint64_t *>(a13.hsum);
        const int nh = max_tiles * kDecodeRows * a13.N;   // 2N floats per tile row
        for (int i = gid; i < nh; i += nthr)
            __hip_atomic_store(h + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's stores are performed
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(a13.prep_done, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == a13.n_pre - 1;
    if (wg == 0 && tid < 64) {
        if (tid == 0)   // waits that gave up: counted afresh by every call
            __hip_atomic_store(a2.status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int *cnt = reinterpret_cast<int *>(smem);
        align_wave(cnt, cnt + a13.E, a13.ids, a13.P, a13.E, kDecodeRows, ws.sorted_ids,
                   ws.tile_expert, ws.expert_offsets, ws.inv_perm, ws.meta, ws.meta + 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    if (tid < 64) {
        int nt, e, pair[kDecodeRows];
        wave_tile_lookup(a13.ids, a13.P, a13.E, 0, nt, e, pair);
        if (tid == 0)
            s_ntiles = nt;
    }
    __syncthreads();
    if (s_ntiles != 0)
        return;
    for (int i = tid; i < T * H; i += 256)
        a2.out_bf16[i] = 0;
    if (tid == 0)
        __hip_atomic_store(a13.prep_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The whole decode-shaped layer in one launch: workgroups [0, n_pre) are the
// prep (decode_prep), then the w13 (tile, column block, K slice) items,
// tile-major, then the w2 items.  Workgroups are dispatched in id order, so every item a
// workgroup waits for has been dispatched before it.
template <int BITS, int GS, int D13, int D2, bool PREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void decode_layer_kernel(
    const GemmArgs a13, const GemmArgs a2, const Workspace ws, int T, int H, int max_tiles,
    int nblk13, int nblk2)
{
    const int per13 = nblk13 * a13.ksplit;   // w13 items per tile
    const int id = (int)blockIdx.x - a13.n_pre, n13 = max_tiles * per13;
    if (id < 0)
        decode_prep(a13, a2, ws, T, H, max_tiles, (int)blockIdx.x);
    else if (id < n13)
        Stream<BITS, GS, 2, D13, true, true, PREP, true>::run(
            a13, id / per13, (id % per13) / a13.ksplit, (id % per13) % a13.ksplit);
    else
        Stream<BITS, GS, 2, D2, false, true, PREP, true>::run(a2, (id - n13) / nblk2,
                                                              (id - n13) % nblk2);
}

__global__ void convert_kernel(const float *__restrict__ src, uint16_t *__restrict__ dst,
                               size_t n4)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4)
        return;
    reinterpret_cast<u32x2_t *>(dst)[i] = to_bf16x4(reinterpret_cast<const f32x4_t *>(src)[i]);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_align(const int32_t *topk_ids, int T, int topk, int E, int block_m,
                        int32_t *sorted_ids, int32_t *tile_expert, int32_t *expert_offsets,
                        int32_t *inv_perm, int32_t *num_tiles, int32_t *bad_ids,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(align_kernel, dim3(align_blocks(T * topk)), dim3(kAlignThreads), 0, stream,
                       topk_ids,
                       T * topk, E, block_m, sorted_ids, tile_expert, expert_offsets, inv_perm,
                       num_tiles, bad_ids, align_chunk(T * topk));
    return hipGetLastError();
}

template <int BITS, int GS>
static hipError_t route_t(const uint16_t *x, const int32_t *ids, const LayerDims &d,
                          const Workspace &ws, hipStream_t stream, const KernelEvents &ev)
{
    const long nthreads_prep = (long)d.T * (d.H / 8);   // 8 fragment positions per thread
    const int nprep = (int)((nthreads_prep + kAlignThreads - 1) / kAlignThreads);
    const long n4 = (long)d.T * d.H / 4;
    long nzero = (n4 + 4L * kAlignThreads - 1) / (4L * kAlignThreads);
    if (nzero < 1)
        nzero = 1;
    if (nzero > 1024)
        nzero = 1024;
    const int nalign = align_blocks(d.T * d.topk);
    const int chunk = align_chunk(d.T * d.topk);
    // With many sort workgroups, each one recounting every pair costs more
    // than one extra launch: count per chunk first, the sort sums the counts.
    const bool counted = nalign >= kCountedSortBlocks;
    hipEvent_t route_start = ev.start;
    if (counted) {
        hipExtLaunchKernelGGL(align_count_kernel, dim3(nalign), dim3(kAlignThreads), 0, stream,
                              ev.start, nullptr, 0, ids, d.T * d.topk, d.E, chunk,
                              ws.chunk_counts);
        route_start = nullptr;
    }
    hipExtLaunchKernelGGL((route_kernel<BITS, GS>), dim3(nalign + nprep + (int)nzero),
                          dim3(kAlignThreads), 0, stream, route_start, ev.stop, 0, x, ids, d.T, d.H,
                          d.topk, d.E, d.block_m, nalign, chunk, nprep,
                          // only the decode-shaped w13 adds into act_bias
                          d.variant13 == 2 ? (size_t)d.max_tiles * d.block_m * (d.I / d.g2) : 0,
                          d.max_tiles * 16, ws);
    return hipGetLastError();
}

hipError_t launch_route(const uint16_t *x, const int32_t *topk_ids, const LayerDims &d,
                        const Workspace &ws, hipStream_t stream, const KernelEvents &ev)
{
    const int key = d.bits13 * 1000 + d.g13;
    switch (key) {
    case 2032: return route_t<2, 32>(x, topk_ids, d, ws, stream, ev);
    case 2064: return route_t<2, 64>(x, topk_ids, d, ws, stream, ev);
    case 2128: return route_t<2, 128>(x, topk_ids, d, ws, stream, ev);
    case 4032: return route_t<4, 32>(x, topk_ids, d, ws, stream, ev);
    case 4064: return route_t<4, 64>(x, topk_ids, d, ws, stream, ev);
    case 4128: return route_t<4, 128>(x, topk_ids, d, ws, stream, ev);
    default: return hipErrorInvalidValue;
    }
}

// Workgroup slots per XCD of a tile-kernel launch: room for a split of up to
// max_tiles tiles whose longest range is 1.5 times the even share plus a tile.
static int tile_xcd_cap(int max_tiles, int N, bool w13)
{
    const int outc = w13 ? Tile<2, 128, true>::OUTC : Tile<2, 128, false>::OUTC;
    const long nblk = (N + outc - 1) / outc;
    const long per = ((long)max_tiles * nblk + 7) / 8;
    return (int)(per + per / 2 + nblk);
}

// Relative cost of one tile-kernel item: a fixed part (its expert's codes are
// copied and unpacked whatever the row count) plus the MFMA chains of its
// active 16-row slices, weighted 3 : 1 (measured best among 1 : 2, 2 : 1,
// 3 : 1 and 5 : 1 on 2048- and 8192-token Zipf-routed batches).  Padding
// slots sit at the end of a tile and hold P.
__device__ __forceinline__ int split_tile_cost(const int32_t *sorted_ids, int b, int P)
{
    int n = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        n += sorted_ids[b * 64 + 16 * s] < P ? 1 : 0;
    return 3 + n;
}

// Cost-balanced split of the tile kernel's (tile, column block) items over
// the 8 XCDs.  Each XCD keeps a contiguous, tile-major range (the L2 reuse of
// activations and expert codes stays), and range x starts at the first item
// whose preceding cost reaches x/8 of the total.  Every range is then capped
// at `cap` items, the workgroup slots the launch gives each XCD; since
// 8 * cap >= the item count, the capped ranges still cover every item once.
// One workgroup; writes first[9] for w13, then first[9] for w2.
__global__ __launch_bounds__(1024) void split_kernel(const int32_t *__restrict__ sorted_ids,
                                                     const int32_t *__restrict__ meta, int P,
                                                     int nblk13, int cap13, int nblk2, int cap2,
                                                     int32_t *__restrict__ first)
{
    __shared__ int wsum[16];
    __shared__ int rec_b[8], rec_num[8], rec_den[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntiles = meta[0];
    // the costs of this thread's first kCached tiles stay in registers for
    // the second pass
    constexpr int kCached = 4;
    int cost[kCached];
    int part = 0;
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
        const int b = tid + 1024 * i;
        cost[i] = b < ntiles ? split_tile_cost(sorted_ids, b, P) : 0;
        part += cost[i];
    }
    for (int b = tid + 1024 * kCached; b < ntiles; b += 1024)
        part += split_tile_cost(sorted_ids, b, P);
    for (int m = 32; m; m >>= 1)
        part += __shfl_xor(part, m, 64);
    if (lane == 0)
        wsum[wave] = part;
    __syncthreads();
    long long C = 0;
    for (int w = 0; w < 16; ++w)
        C += wsum[w];
    __syncthreads();
    // boundary x lies in the tile b with 8*S_b < x*C <= 8*(S_b + cost_b),
    // S_b = cost of the tiles before b (each x has exactly one such tile)
    long long carry = 0;
    for (int base = 0, i = 0; base < ntiles; base += 1024, ++i) {
        const int b = base + tid;
        int c = 0;
#pragma unroll
        for (int j = 0; j < kCached; ++j)
            c = i == j ? cost[j] : c;
        if (i >= kCached)
            c = b < ntiles ? split_tile_cost(sorted_ids, b, P) : 0;
        int incl = c;
        for (int m = 1; m < 64; m <<= 1) {
            const int v = __shfl_up(incl, m, 64);
            if (lane >= m)
                incl += v;
        }
        if (lane == 63)
            wsum[wave] = incl;
        __syncthreads();
        int before = 0, chunk = 0;
        for (int w = 0; w < 16; ++w) {
            before += w < wave ? wsum[w] : 0;
            chunk += wsum[w];
        }
        const long long S = carry + before + incl - c;
        if (b < ntiles)
            for (int x = 1; x < 8; ++x) {
                const long long t = (long long)x * C;
                if (8 * S < t && t <= 8 * (S + c)) {
                    rec_b[x] = b;
                    rec_num[x] = (int)(t - 8 * S);
                    rec_den[x] = 8 * c;
                }
            }
        carry += chunk;
        __syncthreads();
    }
    if (tid < 2) {
        const int nblk = tid == 0 ? nblk13 : nblk2, cap = tid == 0 ? cap13 : cap2;
        int B[9];
        B[0] = 0;
        B[8] = ntiles * nblk;
        for (int x = 1; x < 8; ++x)   // the tile's items up to the cost target
            B[x] = ntiles == 0 ? 0
                               : rec_b[x] * nblk + (nblk * rec_num[x] + rec_den[x] - 1) / rec_den[x];
        for (int x = 1; x < 8; ++x)   // ranges in order and inside the item count
            B[x] = max(B[x - 1], min(B[x], B[8]));
        for (int x = 1; x < 8; ++x)
            B[x] = min(B[x], B[x - 1] + cap);
        for (int x = 7; x >= 1; --x)
            B[x] = max(B[x], B[x + 1] - cap);
        for (int x = 0; x < 9; ++x)
            first[tid * kSplitEntries + x] = B[x];
    }
}

hipError_t launch_split(const LayerDims &d, const Workspace &ws, hipStream_t stream,
                        const KernelEvents &ev)
{
    if (d.block_m != Tile<2, 128, true>::BM)
        return hipErrorInvalidValue;
    const int o13 = Tile<2, 128, true>::OUTC, o2 = Tile<2, 128, false>::OUTC;
    hipExtLaunchKernelGGL(split_kernel, dim3(1), dim3(1024), 0, stream, ev.start, ev.stop, 0,
                          ws.sorted_ids, ws.meta, d.T * d.topk, (d.I + o13 - 1) / o13,
                          tile_xcd_cap(d.max_tiles, d.I, true), (d.H + o2 - 1) / o2,
                          tile_xcd_cap(d.max_tiles, d.H, false), ws.xcd_first);
    return hipGetLastError();
}

// Load units in flight per wave of the decode-shaped kernel: as many as fit
// without spilling.
template <int BITS, int GS, bool W13>
static constexpr int stream_depth()
{
    using S1 = Stream<BITS, GS, 2, 1, W13>;
    return S1::SPLIT ? 1 : S1::GPU == 4 ? 2 : (BITS == 4 && GS == 128) ? 8 : 4;
}

template <int BITS, int GS, int NB, int D, bool W13>
static void launch_stream(const GemmArgs &a, dim3 grid, hipStream_t stream,
                          const KernelEvents &ev)
{
    using K_ = Stream<BITS, GS, NB, D, W13>;
    if (a.prepared)
        hipExtLaunchKernelGGL((stream_kernel<BITS, GS, NB, D, W13, true>), grid,
                              dim3(K_::NTHREADS), (uint32_t)K_::lds_bytes(a.K), stream, ev.start,
                              ev.stop, 0, a);
    else
        hipExtLaunchKernelGGL((stream_kernel<BITS, GS, NB, D, W13, false>), grid,
                              dim3(K_::NTHREADS), (uint32_t)K_::lds_bytes(a.K), stream, ev.start,
                              ev.stop, 0, a);
}

// Tile shapes.  Variant 2 (few rows per expert, HBM-bound): the stream kernel
// on 4-row tiles.  Variant 1 (many rows per expert, MFMA-bound): the tile
// kernel on 64-row tiles.
template <int BITS, int GS, bool W13>
static hipError_t gemm_dispatch(const GemmArgs &a, int variant, int max_tiles, hipStream_t stream,
                                const KernelEvents &ev)
{
    if (variant == 2) {
        constexpr int NB = 2;
        constexpr int D = stream_depth<BITS, GS, W13>();
        using K_ = Stream<BITS, GS, NB, D, W13>;
        const dim3 grid(max_tiles, a.N / K_::BN);
        if ((a.K / K_::UK) % D == 0)
            launch_stream<BITS, GS, NB, D, W13>(a, grid, stream, ev);
        else
            launch_stream<BITS, GS, NB, 1, W13>(a, grid, stream, ev);
    } else {
        if (a.prepared)   // the tile kernel reads the checkpoint layout only
            return hipErrorNotSupported;
        using K_ = Tile<BITS, GS, W13>;
        if (!a.xcd_first)
            return hipErrorInvalidValue;
        const long grid = (long)K_::kXcds * tile_xcd_cap(max_tiles, a.N, W13);
        hipExtLaunchKernelGGL((tile_kernel<BITS, GS, W13>), dim3((unsigned)grid),
                              dim3(K_::NTHREADS), 0, stream, ev.start, ev.stop, 0, a);
    }
    return hipGetLastError();
}

template <bool W13>
static hipError_t gemm_select(const GemmArgs &a, int bits, int gs, int variant, int max_tiles,
                              hipStream_t stream, const KernelEvents &ev)
{
    switch (bits * 1000 + gs) {
    case 2032: return gemm_dispatch<2, 32, W13>(a, variant, max_tiles, stream, ev);
    case 2064: return gemm_dispatch<2, 64, W13>(a, variant, max_tiles, stream, ev);
    case 2128: return gemm_dispatch<2, 128, W13>(a, variant, max_tiles, stream, ev);
    case 4032: return gemm_dispatch<4, 32, W13>(a, variant, max_tiles, stream, ev);
    case 4064: return gemm_dispatch<4, 64, W13>(a, variant, max_tiles, stream, ev);
    case 4128: return gemm_dispatch<4, 128, W13>(a, variant, max_tiles, stream, ev);
    default: return hipErrorInvalidValue;
    }
}

static GemmArgs w13_args(const int32_t *w13, const uint16_t *s13, const LayerDims &d,
                         const Workspace &ws)
{
    GemmArgs a{};
    a.a = ws.x_perm;
    a.a_bias = ws.x_bias;
    a.codes = reinterpret_cast<const uint32_t *>(w13);
    a.scales = s13;
    a.sorted_ids = ws.sorted_ids;
    a.tile_expert = ws.tile_expert;
    a.num_tiles = ws.meta;
    a.act_out = ws.act;
    a.act_bias_out = ws.act_bias;
    a.K = d.H;
    a.N = d.I;
    a.P = d.T * d.topk;
    a.topk = d.topk;
    a.bits_next = d.bits2;
    a.gs_next = d.g2;
    a.alpha = d.alpha;
    a.beta = d.beta;
    a.clamp = d.clamp;
    a.tile_done = ws.tile_done;
    a.prepared = d.prepared;
    a.xcd_first = ws.xcd_first;
    a.ksplit = 1;
    return a;
}

hipError_t launch_w13(const int32_t *w13, const uint16_t *s13, const LayerDims &d,
                      const Workspace &ws, hipStream_t stream, const KernelEvents &ev)
{
    return gemm_select<true>(w13_args(w13, s13, d, ws), d.bits13, d.g13, d.variant13,
                             d.max_tiles, stream, ev);
}

static GemmArgs w2_args(const int32_t *w2, const uint16_t *s2, const float *topk_w,
                        const LayerDims &d, const Workspace &ws, uint16_t *out_bf16)
{
    GemmArgs a{};
    a.a = ws.act;
    a.a_bias = ws.act_bias;
    a.codes = reinterpret_cast<const uint32_t *>(w2);
    a.scales = s2;
    a.sorted_ids = ws.sorted_ids;
    a.tile_expert = ws.tile_expert;
    a.num_tiles = ws.meta;
    a.topk_w = topk_w;
    a.out_f32 = ws.out_f32;
    a.out_bf16 = out_bf16;
    a.done = ws.done;
    a.K = d.I;
    a.N = d.H;
    a.P = d.T * d.topk;
    a.topk = d.topk;
    a.tile_done = ws.tile_done;
    a.status = ws.meta + 2;
    a.prepared = d.prepared;
    a.xcd_first = ws.xcd_first + kSplitEntries;
    return a;
}

hipError_t launch_w2(const int32_t *w2, const uint16_t *s2, const float *topk_w,
                     const LayerDims &d, const Workspace &ws, hipStream_t stream,
                     const KernelEvents &ev, uint16_t *out_bf16)
{
    return gemm_select<false>(w2_args(w2, s2, topk_w, d, ws, out_bf16), d.bits2, d.g2,
                              d.variant2, d.max_tiles, stream, ev);
}

// The shared decode launches' w2 prefetch depth: the stand-alone w2's, or
// half of it when I holds too few load units (0: neither divides them).
template <int BITS, int GS>
static int decode_depth2(int I)
{
    constexpr int D2 = stream_depth<BITS, GS, false>();
    const int nunits = I / Stream<BITS, GS, 2, 1, false>::UK;
    if (nunits % D2 == 0)
        return D2;
    if (D2 > 1 && nunits % (D2 / 2) == 0)
        return D2 / 2;
    return 0;
}

template <int BITS, int GS, int D2>
static hipError_t decode_dispatch_d(const GemmArgs &a13, GemmArgs a2, int max_tiles,
                                    hipStream_t stream, const KernelEvents &ev)
{
    constexpr int D13 = stream_depth<BITS, GS, true>();
    using S13 = Stream<BITS, GS, 2, D13, true, true>;
    using S2 = Stream<BITS, GS, 2, D2, false, true>;
    const int nblk13 = a13.N / S13::BN, nblk2 = a2.N / S2::BN;
    a2.tile_target = nblk13;
    const size_t l13 = S13::lds_bytes(a13.K), l2 = S2::lds_bytes(a2.K);
    const dim3 grid((unsigned)(max_tiles * (nblk13 + nblk2)));
    const uint32_t lds = (uint32_t)(l13 > l2 ? l13 : l2);
    if (a13.prepared)
        hipExtLaunchKernelGGL((decode_kernel<BITS, GS, D13, BITS, GS, D2, true>), grid,
                              dim3(S13::NTHREADS), lds, stream, ev.start, ev.stop, 0, a13, a2,
                              max_tiles, nblk13, nblk2);
    else
        hipExtLaunchKernelGGL((decode_kernel<BITS, GS, D13, BITS, GS, D2, false>), grid,
                              dim3(S13::NTHREADS), lds, stream, ev.start, ev.stop, 0, a13, a2,
                              max_tiles, nblk13, nblk2);
    return hipGetLastError();
}

template <int BITS, int GS>
static hipError_t decode_dispatch(const GemmArgs &a13, const GemmArgs &a2, int max_tiles,
                                  hipStream_t stream, const KernelEvents &ev)
{
    constexpr int D2 = stream_depth<BITS, GS, false>();
    const int d2 = decode_depth2<BITS, GS>(a2.K);
    if (d2 == D2)
        return decode_dispatch_d<BITS, GS, D2>(a13, a2, max_tiles, stream, ev);
    if constexpr (D2 > 1)
        if (d2 == D2 / 2)
            return decode_dispatch_d<BITS, GS, D2 / 2>(a13, a2, max_tiles, stream, ev);
    return hipErrorNotSupported;
}

template <int BITS, int GS>
static bool decode_fits(int H, int I)
{
    constexpr int D13 = stream_depth<BITS, GS, true>();
    return (H / Stream<BITS, GS, 2, D13, true, true>::UK) % D13 == 0 &&
           decode_depth2<BITS, GS>(I) != 0;
}

bool decode_one_launch(int bits13, int g13, int bits2, int g2, int H, int I)
{
    if (bits13 != bits2 || g13 != g2)
        return false;
    switch (bits13 * 1000 + g13) {   // 2-bit g32: both bodies do not fit one kernel's registers
    case 2064: return decode_fits<2, 64>(H, I);
    case 2128: return decode_fits<2, 128>(H, I);
    case 4032: return decode_fits<4, 32>(H, I);
    case 4064: return decode_fits<4, 64>(H, I);
    case 4128: return decode_fits<4, 128>(H, I);
    default: return false;
    }
}

hipError_t launch_decode(const int32_t *w13, const uint16_t *s13, const int32_t *w2,
                         const uint16_t *s2, const float *topk_w, const LayerDims &d,
                         const Workspace &ws, hipStream_t stream, const KernelEvents &ev,
                         uint16_t *out_bf16)
{
    if (d.variant13 != 2 || d.variant2 != 2 ||
        !decode_one_launch(d.bits13, d.g13, d.bits2, d.g2, d.H, d.I))
        return hipErrorNotSupported;
    const GemmArgs a13 = w13_args(w13, s13, d, ws);
    const GemmArgs a2 = w2_args(w2, s2, topk_w, d, ws, out_bf16);
    switch (d.bits13 * 1000 + d.g13) {
    case 2064: return decode_dispatch<2, 64>(a13, a2, d.max_tiles, stream, ev);
    case 2128: return decode_dispatch<2, 128>(a13, a2, d.max_tiles, stream, ev);
    case 4032: return decode_dispatch<4, 32>(a13, a2, d.max_tiles, stream, ev);
    case 4064: return decode_dispatch<4, 64>(a13, a2, d.max_tiles, stream, ev);
    case 4128: return decode_dispatch<4, 128>(a13, a2, d.max_tiles, stream, ev);
    default: return hipErrorNotSupported;
    }
}

// K slices per w13 (tile, column block) in the single launch: split (2 or 4)
// while the w13 items would fill fewer than 3 workgroups per CU and every
// slice keeps whole rounds of the prefetch depth.
constexpr int kSplitMaxItems = 768;
template <int BITS, int GS>
static int decode_ksplit(int H, int max_tiles, int nblk13)
{
    constexpr int D13 = stream_depth<BITS, GS, true>();
    const int nunits = H / Stream<BITS, GS, 2, D13, true, true>::UK;
    int S = 1;
    while (S < 4 && (long)max_tiles * nblk13 * (2 * S) <= kSplitMaxItems &&
           nunits % (2 * S * D13) == 0 && max_tiles * nblk13 <= kSyncSplits)
        S *= 2;
    return S;
}

template <int BITS, int GS, int D2>
static hipError_t decode_layer_dispatch_d(const uint16_t *x, const int32_t *ids, GemmArgs a13,
                                          GemmArgs a2, const LayerDims &d, const Workspace &ws,
                                          hipStream_t stream, const KernelEvents &ev)
{
    constexpr int D13 = stream_depth<BITS, GS, true>();
    using S13 = Stream<BITS, GS, 2, D13, true, true, false, true>;
    using S2 = Stream<BITS, GS, 2, D2, false, true, false, true>;
    const int nblk13 = a13.N / S13::BN, nblk2 = a2.N / S2::BN;
    const int ksplit = ws.hsum ? decode_ksplit<BITS, GS>(d.H, d.max_tiles, nblk13) : 1;
    if (ksplit != decode_layer_ksplit(BITS, GS, d.H, d.I, d.max_tiles))
        return hipErrorInvalidValue;   // the plan reports the same split
    // zeroing: 4 stores of the FP32 sum per thread, and at most 8 of the
    // split sums
    const long prep_threads = (long)d.T * d.H / 8;
    const long hsum_threads = ksplit > 1 ? ((long)d.max_tiles * kDecodeRows * d.I + 7) / 8 : 0;
    const long nthr = prep_threads > hsum_threads ? prep_threads : hsum_threads;
    const int n_pre = (int)((nthr + 255) / 256);
    if (d.T * d.topk > kSingleLaunchPairs || d.max_tiles > kSyncTiles || nblk2 > kSyncBlocks ||
        d.block_m != kDecodeRows || n_pre < 1)
        return hipErrorInvalidValue;
    for (GemmArgs *a : {&a13, &a2}) {
        a->ids = ids;
        a->E = d.E;
        a->n_pre = n_pre;
        a->prep_done = ws.prep_done;
        a->blocks_done = ws.blocks_done;
        a->tile_done = ws.sync_tiles;
        a->status = ws.meta + 2;
        a->ksplit = 1;
    }
    a13.a = x;   // staged straight from the input rows
    a13.ksplit = ksplit;
    a13.hsum = ws.hsum;
    a13.split_done = ws.sync_split;
    a13.nblk_self = nblk13;
    a2.nblk_self = nblk2;
    a2.tile_target = nblk13;
    a2.done = ws.sync_done;
    size_t lds = S13::lds_bytes(a13.K / ksplit);
    if (S2::lds_bytes(a2.K) > lds)
        lds = S2::lds_bytes(a2.K);
    if ((size_t)2 * d.E * sizeof(int) > lds)   // the sort's per-expert counts and offsets
        lds = (size_t)2 * d.E * sizeof(int);
    const dim3 grid((unsigned)(n_pre + d.max_tiles * (nblk13 * ksplit + nblk2)));
    if (a13.prepared)
        hipExtLaunchKernelGGL((decode_layer_kernel<BITS, GS, D13, D2, true>), grid, dim3(256),
                              (uint32_t)lds, stream, ev.start, ev.stop, 0, a13, a2, ws, d.T,
                              d.H, d.max_tiles, nblk13, nblk2);
    else
        hipExtLaunchKernelGGL((decode_layer_kernel<BITS, GS, D13, D2, false>), grid, dim3(256),
                              (uint32_t)lds, stream, ev.start, ev.stop, 0, a13, a2, ws, d.T,
                              d.H, d.max_tiles, nblk13, nblk2);
    return hipGetLastError();
}

template <int BITS, int GS>
static hipError_t decode_layer_dispatch(const uint16_t *x, const int32_t *ids,
                                        const GemmArgs &a13, const GemmArgs &a2,
                                        const LayerDims &d, const Workspace &ws,
                                        hipStream_t stream, const KernelEvents &ev)
{
    constexpr int D2 = stream_depth<BITS, GS, false>();
    const int d2 = decode_depth2<BITS, GS>(a2.K);
    if (d2 == D2)
        return decode_layer_dispatch_d<BITS, GS, D2>(x, ids, a13, a2, d, ws, stream, ev);
    if constexpr (D2 > 1)
        if (d2 == D2 / 2)
            return decode_layer_dispatch_d<BITS, GS, D2 / 2>(x, ids, a13, a2, d, ws, stream, ev);
    return hipErrorNotSupported;
}

int decode_layer_ksplit(int bits, int gs, int H, int I, int max_tiles)
{
    const int nblk13 = I / 64;   // w13 items cover 64 act columns
    switch (bits * 1000 + gs) {
    case 2064: return decode_ksplit<2, 64>(H, max_tiles, nblk13);
    case 2128: return decode_ksplit<2, 128>(H, max_tiles, nblk13);
    case 4032: return decode_ksplit<4, 32>(H, max_tiles, nblk13);
    case 4064: return decode_ksplit<4, 64>(H, max_tiles, nblk13);
    case 4128: return decode_ksplit<4, 128>(H, max_tiles, nblk13);
    default: return 1;
    }
}

hipError_t launch_decode_layer(const uint16_t *x, const int32_t *topk_ids, const int32_t *w13,
                               const uint16_t *s13, const int32_t *w2, const uint16_t *s2,
                               const float *topk_w, const LayerDims &d, const Workspace &ws,
                               hipStream_t stream, const KernelEvents &ev, uint16_t *out_bf16)
{
    if (d.variant13 != 2 || d.variant2 != 2 || !out_bf16 ||
        !decode_one_launch(d.bits13, d.g13, d.bits2, d.g2, d.H, d.I))
        return hipErrorNotSupported;
    const GemmArgs a13 = w13_args(w13, s13, d, ws);
    const GemmArgs a2 = w2_args(w2, s2, topk_w, d, ws, out_bf16);
    switch (d.bits13 * 1000 + d.g13) {
    case 2064: return decode_layer_dispatch<2, 64>(x, topk_ids, a13, a2, d, ws, stream, ev);
    case 2128: return decode_layer_dispatch<2, 128>(x, topk_ids, a13, a2, d, ws, stream, ev);
    case 4032: return decode_layer_dispatch<4, 32>(x, topk_ids, a13, a2, d, ws, stream, ev);
    case 4064: return decode_layer_dispatch<4, 64>(x, topk_ids, a13, a2, d, ws, stream, ev);
    case 4128: return decode_layer_dispatch<4, 128>(x, topk_ids, a13, a2, d, ws, stream, ev);
    default: return hipErrorNotSupported;
    }
}

size_t decode_lds_bytes(int K, int gs)
{
    // the layout of Stream::lds_bytes, which depends on the group size only
    switch (gs) {
    case 32: return Stream<4, 32, 2, 1, true>::lds_bytes(K);
    case 64: return Stream<4, 64, 2, 1, true>::lds_bytes(K);
    default: return Stream<4, 128, 2, 1, true>::lds_bytes(K);
    }
}

hipError_t launch_convert(const float *src, uint16_t *dst, size_t n, hipStream_t stream,
                          const KernelEvents &ev)
{
    const size_t n4 = n / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256);
    hipExtLaunchKernelGGL(convert_kernel, dim3(blocks), dim3(256), 0, stream, ev.start, ev.stop,
                          0, src, dst, n4);
    return hipGetLastError();
}

}  // namespace wna16
