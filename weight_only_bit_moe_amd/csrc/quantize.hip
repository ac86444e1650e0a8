// gfx950 kernels of the quantizer: BF16 weights -> the packed codes and FP16
// group scales the layer reads (model card
// "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "How it was created" steps 2-5:
// symmetric b-bit weights per K group, a scale search weighted by an
// activation importance vector, signed codes packed into 32-bit words, and
// weighted and unweighted reconstruction error).
//
// Work split.  A wave owns a strip of 64 * 16 consecutive K columns and walks
// rows; each lane holds 16 consecutive weights (two 16-byte loads), so a group
// of GS weights spans GS / 16 lanes and the importance of the lane's columns
// stays in registers for every row.  Per row and group:
//   amax  by a butterfly over the group's lanes (DPP, no LDS);
//   s0 = amax / ((2^b - 1) / 2) (FP32 division);
//   for each candidate c: s_c = fp16_rne(min(s0 * f_c, 65504)),
//     f_c = 1 - c / (2C); error sum_k imp_k (w_k - s_c q_k)^2 in FP64, formed
//     as sum_k (sqrt(imp_k) d_k)^2 with one fma per weight (only the last-bit
//     rounding differs from imp * d * d, so only near-ties can rank apart);
//   the smallest error wins, ties to the smaller c;
//   the winner's codes q = clamp(rne(w / s)) by FP32 division, packed with the
//   least-significant field first as u = q + 2^(b-1): a lane's 16 codes fill
//   one word (2-bit) or two (4-bit).
//
// The search takes w * rcp(s) instead of w / s.  Only the error of each
// candidate is needed there, and it comes out the same: w is BF16 (8-bit
// significand) and s FP16 (11-bit), so whenever w / s is not exactly a
// half-integer it lies at least 2^-12 away from one (for |w / s| < 16), far
// more than the 2^-22 relative error of w * rcp(s); so rounding picks the
// same integer, except at exact half-integers, where both neighbours leave
// the same |w - s q| = s / 2.  Larger quotients clamp either way.  The error
// term w - s q is formed by one FP64 fma, exactly as (w - s*q) in FP64 since
// s*q is exact there.
//
// Butterflies: each step adds (or maxes) a lane's value with its partner's
// under XOR masks 1, 2, 7, 15 (DPP quad permutes and row mirrors); since the
// operation is commutative every lane of a group ends with the same bits, so
// all lanes take the same decision.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "launch.hpp"

namespace wna16 {

namespace {

constexpr int kQThreads = 256;
constexpr int kQEpl = 16;                 // weights per lane
constexpr int kQStrip = 64 * kQEpl;       // K columns per wave
constexpr int kQTargetWaves = 8192;       // 8 waves per SIMD over 256 CUs

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp(double v)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)b, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Reduction over aligned groups of L lanes (L in 1, 2, 4, 8, 16).
template <int L>
__device__ __forceinline__ float seg_max(float v)
{
    if constexpr (L >= 2) v = fmaxf(v, dpp<0xB1>(v));    // xor 1
    if constexpr (L >= 4) v = fmaxf(v, dpp<0x4E>(v));    // xor 2
    if constexpr (L >= 8) v = fmaxf(v, dpp<0x141>(v));   // xor 7 (half-row mirror)
    if constexpr (L >= 16) v = fmaxf(v, dpp<0x140>(v));  // xor 15 (row mirror)
    return v;
}

template <int L>
__device__ __forceinline__ double seg_sum(double v)
{
    if constexpr (L >= 2) v += dpp<0xB1>(v);
    if constexpr (L >= 4) v += dpp<0x4E>(v);
    if constexpr (L >= 8) v += dpp<0x141>(v);
    if constexpr (L >= 16) v += dpp<0x140>(v);
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__global__ void zero_sums(double *sums)
{
    if (threadIdx.x < 4)
        sums[threadIdx.x] = 0.0;
}

template <int BITS, int GS, bool IMP>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(
    const uint4 *__restrict__ w, const float *__restrict__ imp, int rows, int K, int ncand,
    int nstrips, int wps, uint32_t *__restrict__ codes, uint16_t *__restrict__ scales,
    double *__restrict__ sums)
{
#pragma clang fp contract(off)
    constexpr int L = GS / kQEpl;                // lanes per group
    constexpr float half_span = (float)((1 << BITS) - 1) / 2.0f;
    constexpr float qlo = -(float)(1 << (BITS - 1)), qhi = (float)((1 << (BITS - 1)) - 1);
    __shared__ float ftab[64];
    __shared__ double part[kQThreads / 64][4];
    if ((int)threadIdx.x < ncand)
        ftab[threadIdx.x] = 1.0f - (float)threadIdx.x / (float)(2 * ncand);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wid = blockIdx.x * (kQThreads / 64) + wave;
    const int strip = wid % nstrips;
    long long r = wid < nstrips * wps ? wid / nstrips : rows;
    const int k0 = strip * kQStrip + lane * kQEpl;
    const bool on = k0 < K;
    const size_t row_vecs = (size_t)K / 8;
    const int kw = K * BITS / 32, ng = K / GS;

    double im[kQEpl], rim[kQEpl];   // importance and its square root (FP64)
#pragma unroll
    for (int i = 0; i < kQEpl; ++i) {
        im[i] = (IMP && on) ? (double)imp[k0 + i] : 1.0;
        rim[i] = __builtin_sqrt(im[i]);
    }
    double a_err = 0.0, a_w2 = 0.0, a_ierr = 0.0, a_iw2 = 0.0;

    uint4 va = make_uint4(0, 0, 0, 0), vb = va;
    if (on && r < rows) {
        va = w[(size_t)r * row_vecs + k0 / 8];
        vb = w[(size_t)r * row_vecs + k0 / 8 + 1];
    }
    for (; r < rows; r += wps) {
        float x[kQEpl];
        const uint32_t words[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[2 * j] = __uint_as_float(words[j] << 16);
            x[2 * j + 1] = __uint_as_float(words[j] & 0xffff0000u);
        }
        if (on && r + wps < rows) {          // next row's weights in flight meanwhile
            va = w[(size_t)(r + wps) * row_vecs + k0 / 8];
            vb = w[(size_t)(r + wps) * row_vecs + k0 / 8 + 1];
        }
        float am = 0.0f;
        double wd[kQEpl];
#pragma unroll
        for (int i = 0; i < kQEpl; ++i) {
            am = fmaxf(am, fabsf(x[i]));
            wd[i] = (double)x[i];
        }
        am = seg_max<L>(am);
        const float s0 = am / half_span;

        double best = 0.0;
        float sbest = 0.0f;
        uint16_t hbest = 0;
        for (int c = 0; c < ncand; ++c) {
            const __half h = __float2half_rn(fminf(s0 * ftab[c], 65504.0f));
            const float s = __half2float(h);
            if (ncand == 1) {
                sbest = s;
                hbest = __half_as_ushort(h);
                break;
            }
            const float rs = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
            const double ns = -(double)s;
            double e = 0.0;
#pragma unroll
            for (int i = 0; i < kQEpl; ++i) {
                const float q = __builtin_amdgcn_fmed3f(rintf(x[i] * rs), qlo, qhi);
                const double d = __builtin_fma(ns, (double)q, wd[i]);
                // the search compares candidates: (sqrt(imp) d)^2 summed with
                // one fma, two FP64 operations instead of three
                const double t = IMP ? rim[i] * d : d;
                e = __builtin_fma(t, t, e);
            }
            e = seg_sum<L>(e);
            if (c == 0 || e < best) {
                best = e;
                sbest = s;
                hbest = __half_as_ushort(h);
            }
        }

        // the winner's codes (FP32 division, round half to even, clamp)
        uint32_t packed[2] = {0u, 0u};
        const double nsb = -(double)sbest;
#pragma unroll
        for (int i = 0; i < kQEpl; ++i) {
            const float q = sbest == 0.0f ? 0.0f : fminf(fmaxf(rintf(x[i] / sbest), qlo), qhi);
            const uint32_t u = (uint32_t)((int)q + (1 << (BITS - 1)));
            packed[(i * BITS) / 32] |= u << ((i * BITS) % 32);
            const double d = __builtin_fma(nsb, (double)q, wd[i]);
            a_err += d * d;
            a_w2 += wd[i] * wd[i];
            if (IMP) {
                a_ierr += (im[i] * d) * d;
                a_iw2 += (im[i] * wd[i]) * wd[i];
            }
        }
        if (on) {
            uint32_t *cw = codes + (size_t)r * kw + k0 * BITS / 32;
            cw[0] = packed[0];
            if (BITS == 4)
                cw[1] = packed[1];
            if (lane % L == 0)
                scales[(size_t)r * ng + k0 / GS] = hbest;
        }
    }
    if (!IMP) {
        a_ierr = a_err;
        a_iw2 = a_w2;
    }
    a_err = wave_sum(a_err);
    a_w2 = wave_sum(a_w2);
    a_ierr = wave_sum(a_ierr);
    a_iw2 = wave_sum(a_iw2);
    if (lane == 0) {
        part[wave][0] = a_err;
        part[wave][1] = a_w2;
        part[wave][2] = a_ierr;
        part[wave][3] = a_iw2;
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        double t = 0.0;
        for (int v = 0; v < kQThreads / 64; ++v)
            t += part[v][threadIdx.x];
        atomicAdd(sums + threadIdx.x, t);
    }
}

template <int BITS, int GS>
hipError_t launch_q(const uint16_t *w, const float *imp, int rows, int K, int ncand,
                    uint32_t *codes, uint16_t *scales, double *sums, hipStream_t stream)
{
    const int nstrips = (K + kQStrip - 1) / kQStrip;
    int wps = (kQTargetWaves + nstrips - 1) / nstrips;
    if (wps > rows)
        wps = rows;
    const long long waves = (long long)nstrips * wps;
    const unsigned blocks = (unsigned)((waves + kQThreads / 64 - 1) / (kQThreads / 64));
    const uint4 *wv = reinterpret_cast<const uint4 *>(w);
    if (imp)
        hipLaunchKernelGGL((quantize_kernel<BITS, GS, true>), dim3(blocks), dim3(kQThreads), 0,
                           stream, wv, imp, rows, K, ncand, nstrips, wps, codes, scales, sums);
    else
        hipLaunchKernelGGL((quantize_kernel<BITS, GS, false>), dim3(blocks), dim3(kQThreads), 0,
                           stream, wv, imp, rows, K, ncand, nstrips, wps, codes, scales, sums);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const uint16_t *w, const float *imp, int rows, int K, int bits,
                           int group, int ncand, uint32_t *codes, uint16_t *scales,
                           double *sums, hipStream_t stream)
{
    hipLaunchKernelGGL(zero_sums, dim3(1), dim3(64), 0, stream, sums);
    if (rows == 0)
        return hipGetLastError();
    switch (bits * 1000 + group) {
    case 2032: return launch_q<2, 32>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    case 2064: return launch_q<2, 64>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    case 2128: return launch_q<2, 128>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    case 4032: return launch_q<4, 32>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    case 4064: return launch_q<4, 64>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    case 4128: return launch_q<4, 128>(w, imp, rows, K, ncand, codes, scales, sums, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace wna16
