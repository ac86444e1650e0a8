// Host-side checks run under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by weight_only_bit_moe_amd.build.build_sanitized; no GPU needed).
//
// 1. Every C-ABI entry point declared in include/moe_wna16.h is called with
//    bad arguments (null pointers, bad shapes, unsupported formats,
//    misalignment, short workspaces, oversized no-alloc calls) and must
//    return the documented status before touching the device; the size,
//    layout and plan queries run over a range of shapes and must agree.
// 2. The oracle's C functions (test infrastructure) run on small seeded
//    inputs, including ragged shapes and invalid expert ids, with light
//    consistency checks, so that every buffer they index is exercised.
// Exit status 0 and the last line "host checks passed" mean no sanitizer
// report and no failed expectation.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "moe_wna16.h"

extern "C" {
int oracle_moe_forward_tokens(const uint16_t *x, const int32_t *ids, const float *topk_w,
                              const uint32_t *w13, const uint16_t *s13, const uint32_t *w2,
                              const uint16_t *s2, int T, int H, int I, int E, int topk,
                              int bits13, int group13, int bits2, int group2, double alpha,
                              double beta, double clamp, const int32_t *tokens, int ntok,
                              double *out, int nthreads);
int oracle_align(const int32_t *ids, int T, int topk, int E, int block_m, int32_t *sorted_ids,
                 int32_t *tile_expert, int32_t *expert_offsets, int32_t *inv_perm,
                 int32_t *num_tiles, int32_t *bad_ids);
int oracle_quantize(const uint16_t *w, const float *imp, int rows, int K, int bits, int group,
                    int ncand, uint32_t *codes, uint16_t *scales, int32_t *choice, double *sums);
int oracle_prepare(const uint32_t *packed, int E, int rows, int K, int bits, int group,
                   uint32_t *out);
uint16_t oracle_f64_to_f16_rne(double v);
double oracle_f16_to_f64(uint16_t h);
}

static int failures = 0;
#define EXPECT(cond, ...)                                                    \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__);      \
            std::fprintf(stderr, __VA_ARGS__);                               \
            std::fprintf(stderr, "\n");                                      \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

// An aligned, never dereferenced address: every call below returns before
// any device access.
static void *fake(uintptr_t off = 0) { return reinterpret_cast<void *>((uintptr_t)1 << 20 | off); }

static void check_abi()
{
    const moe_wna16_qparams q2{2, 128}, q4{4, 128}, qbad{3, 128}, gbad{2, 96};
    const float inf = INFINITY;
    size_t ws = 0;
    // size, offset, layout and plan queries
    const int shapes[][5] = {{0, 256, 128, 8, 2},      {4, 4096, 2048, 256, 6},
                             {64, 4096, 2048, 256, 6}, {2048, 4096, 2048, 256, 6},
                             {8192, 4096, 2048, 256, 8}, {7169, 128, 128, 256, 1},
                             {1, 128, 128, 1, 1},      {16, 256, 128, 1024, 64}};
    for (const auto &s : shapes) {
        size_t total = 0, f32 = 0;
        moe_wna16_workspace_layout_t lay{};
        moe_wna16_plan_t plan{};
        EXPECT(moe_wna16_workspace_size(s[0], s[1], s[2], s[3], s[4], &total) == MOE_WNA16_OK,
               "workspace_size");
        EXPECT(moe_wna16_workspace_f32_offset(s[0], s[1], s[2], s[3], s[4], &f32) ==
                   MOE_WNA16_OK, "f32 offset");
        EXPECT(moe_wna16_workspace_layout(s[0], s[1], s[2], s[3], s[4], &lay) == MOE_WNA16_OK,
               "layout");
        EXPECT(lay.total == total && lay.out_f32 == f32, "layout agrees with size and offset");
        EXPECT(lay.out_f32 + (size_t)s[0] * s[1] * 4 <= total, "accumulator inside workspace");
        EXPECT(moe_wna16_plan(s[0], s[1], s[2], s[3], s[4], q2, q4, &plan) == MOE_WNA16_OK,
               "plan");
        EXPECT(plan.block_m == 4 || plan.block_m == 64, "block_m");
    }
    EXPECT(moe_wna16_workspace_size(4, 100, 2048, 256, 6, &ws) == MOE_WNA16_EUNSUPPORTED, "H%128");
    EXPECT(moe_wna16_workspace_size(-1, 256, 128, 8, 2, &ws) == MOE_WNA16_EINVAL, "T<0");
    EXPECT(moe_wna16_workspace_size(4, 256, 128, 2000, 2, &ws) == MOE_WNA16_EUNSUPPORTED, "E");
    EXPECT(moe_wna16_workspace_size(4, 256, 128, 8, 65, &ws) == MOE_WNA16_EUNSUPPORTED, "topk");
    EXPECT(moe_wna16_workspace_size(4, 256, 128, 8, 2, nullptr) == MOE_WNA16_EINVAL, "null out");
    EXPECT(moe_wna16_workspace_layout(4, 256, 128, 8, 2, nullptr) == MOE_WNA16_EINVAL, "null");
    EXPECT(moe_wna16_plan(4, 256, 128, 8, 2, qbad, q2, nullptr) == MOE_WNA16_EINVAL, "null plan");
    moe_wna16_plan_t plan{};
    EXPECT(moe_wna16_plan(4, 256, 128, 8, 2, qbad, q2, &plan) == MOE_WNA16_EUNSUPPORTED, "bits");
    EXPECT(moe_wna16_plan(4, 384, 128, 8, 2, gbad, q2, &plan) == MOE_WNA16_EUNSUPPORTED, "group");

    // forward and its variants: argument checks before any device access
    void *p = fake();
    const int T = 4, H = 4096, I = 2048, E = 256, k = 6;
    moe_wna16_workspace_size(T, H, I, E, k, &ws);
    auto fwd = [&](const void *x, int t, moe_wna16_qparams a, moe_wna16_qparams b, float alpha,
                   float clamp, void *w, size_t wbytes) {
        return moe_wna16_forward(x, (int32_t *)p, (float *)p, (int32_t *)p, (uint16_t *)p,
                                 (int32_t *)p, (uint16_t *)p, t, H, I, E, k, a, b, alpha, 0.f,
                                 clamp, p, w, wbytes, nullptr);
    };
    EXPECT(fwd(nullptr, T, q2, q2, 1.f, inf, p, ws) == MOE_WNA16_EINVAL, "null x");
    EXPECT(fwd(p, T, q2, q2, NAN, inf, p, ws) == MOE_WNA16_EINVAL, "NaN alpha");
    EXPECT(fwd(p, T, q2, q2, 1.f, NAN, p, ws) == MOE_WNA16_EINVAL, "NaN clamp");
    EXPECT(fwd(p, T, q2, q2, 1.f, -1.f, p, ws) == MOE_WNA16_EINVAL, "clamp <= 0");
    EXPECT(fwd(p, T, qbad, q2, 1.f, inf, p, ws) == MOE_WNA16_EUNSUPPORTED, "bits");
    EXPECT(fwd(fake(2), T, q2, q2, 1.f, inf, p, ws) == MOE_WNA16_EALIGN, "x alignment");
    EXPECT(fwd(p, T, q2, q2, 1.f, inf, fake(16), ws) == MOE_WNA16_EALIGN, "workspace alignment");
    EXPECT(fwd(p, T, q2, q2, 1.f, inf, p, ws - 1) == MOE_WNA16_EWORKSPACE, "short workspace");
    EXPECT(fwd(p, 0, q2, q2, 1.f, inf, nullptr, 0) == MOE_WNA16_OK, "T = 0");
    EXPECT(fwd(p, T, q2, q2, 1.f, inf, nullptr, ws) == MOE_WNA16_EINVAL, "null workspace");
    EXPECT(moe_wna16_forward_profiled(p, (int32_t *)p, (float *)p, (int32_t *)p, (uint16_t *)p,
                                      (int32_t *)p, (uint16_t *)p, T, H, I, E, k, q2, q2, 1.f,
                                      0.f, inf, p, p, ws, nullptr, nullptr) == MOE_WNA16_EINVAL,
           "profiled without events");
    hipEvent_t ev[8] = {};
    EXPECT(moe_wna16_forward_prepared(p, (int32_t *)p, (float *)p, (int32_t *)p, (uint16_t *)p,
                                      (int32_t *)p, (uint16_t *)p, 2048, H, I, E, k, q2, q2, 1.f,
                                      0.f, inf, p, p, (size_t)1 << 40, nullptr, ev) ==
               MOE_WNA16_EUNSUPPORTED, "prepared codes on a prefill shape");
    EXPECT(moe_wna16_forward_noalloc(p, (int32_t *)p, (float *)p, (int32_t *)p, (uint16_t *)p,
                                     (int32_t *)p, (uint16_t *)p, 2048, H, I, E, k, q2, q2, 1.f,
                                     0.f, inf, p, nullptr) == MOE_WNA16_ESCRATCH,
           "no-alloc beyond its scratch");
    EXPECT(moe_wna16_forward_noalloc(nullptr, (int32_t *)p, (float *)p, (int32_t *)p,
                                     (uint16_t *)p, (int32_t *)p, (uint16_t *)p, T, H, I, E, k,
                                     q2, q2, 1.f, 0.f, inf, p, nullptr) == MOE_WNA16_EINVAL,
           "no-alloc null x");
    // align, prepare, quantize
    int32_t *ip = (int32_t *)p;
    EXPECT(moe_wna16_align(ip, -1, 2, 8, 16, ip, ip, ip, ip, ip, ip, nullptr) == MOE_WNA16_EINVAL,
           "align T");
    EXPECT(moe_wna16_align(ip, 4, 2, 2000, 16, ip, ip, ip, ip, ip, ip, nullptr) ==
               MOE_WNA16_EUNSUPPORTED, "align E");
    EXPECT(moe_wna16_align(ip, 4, 2, 8, 16, ip, ip, nullptr, ip, ip, ip, nullptr) ==
               MOE_WNA16_EINVAL, "align null offsets");
    EXPECT(moe_wna16_align((int32_t *)fake(2), 4, 2, 8, 16, ip, ip, ip, ip, ip, ip, nullptr) ==
               MOE_WNA16_EALIGN, "align alignment");
    EXPECT(moe_wna16_prepare(ip, 2, 24, 512, q2, ip, nullptr) == MOE_WNA16_EUNSUPPORTED,
           "prepare rows % 16");
    EXPECT(moe_wna16_prepare(ip, 2, 16, 512, q2, ip, nullptr) == MOE_WNA16_EINVAL,
           "prepare in place");
    EXPECT(moe_wna16_prepare(ip, 0, 16, 512, q2, nullptr, nullptr) == MOE_WNA16_OK,
           "prepare nothing");
    EXPECT(moe_wna16_quantize(p, nullptr, 4, 256, q2, 0, ip, (uint16_t *)p, (double *)p,
                              nullptr) == MOE_WNA16_EINVAL, "quantize candidates");
    EXPECT(moe_wna16_quantize(fake(8), nullptr, 4, 256, q2, 4, ip, (uint16_t *)p, (double *)p,
                              nullptr) == MOE_WNA16_EALIGN, "quantize alignment");
    for (int st = -7; st <= 0; ++st)
        EXPECT(std::strcmp(moe_wna16_status_string(st), "unknown status") != 0, "status %d", st);
    EXPECT(moe_wna16_status_string(42) != nullptr, "status string never null");
}

static void check_oracle()
{
    std::mt19937 rng(7);
    auto u32 = [&]() { return (uint32_t)rng(); };
    // the routed layer on a few small, ragged shapes, invalid ids included
    const int shapes[][9] = {// T, H, I, E, k, b13, g13, b2, g2
                             {5, 256, 128, 4, 2, 4, 128, 4, 128},
                             {7, 384, 256, 6, 3, 2, 64, 4, 32},
                             {3, 128, 128, 1, 1, 2, 32, 2, 128},
                             {0, 128, 128, 2, 1, 4, 64, 4, 64}};
    for (const auto &s : shapes) {
        const int T = s[0], H = s[1], I = s[2], E = s[3], k = s[4];
        const int b13 = s[5], g13 = s[6], b2 = s[7], g2 = s[8];
        std::vector<uint16_t> x((size_t)T * H);
        for (auto &v : x)
            v = (uint16_t)(0x3c00u + (u32() & 0x3ffu)) ^ (uint16_t)((u32() & 1u) << 15);
        std::vector<int32_t> ids((size_t)T * k);
        for (auto &v : ids)
            v = (int32_t)(u32() % (unsigned)(E + 2)) - 1;   // -1 and E are invalid
        std::vector<float> w((size_t)T * k, 0.25f);
        std::vector<uint32_t> w13((size_t)E * 2 * I * H * b13 / 32), w2((size_t)E * H * I * b2 / 32);
        for (auto &v : w13) v = u32();
        for (auto &v : w2) v = u32();
        std::vector<uint16_t> s13((size_t)E * 2 * I * (H / g13), 0x2000),
            s2((size_t)E * H * (I / g2), 0x2000);
        std::vector<int32_t> toks(T);
        for (int t = 0; t < T; ++t)
            toks[t] = T - 1 - t;
        std::vector<double> out((size_t)T * H + 1);
        EXPECT(oracle_moe_forward_tokens(x.data(), ids.data(), w.data(), w13.data(), s13.data(),
                                         w2.data(), s2.data(), T, H, I, E, k, b13, g13, b2, g2,
                                         1.702, 1.0, 7.0, toks.data(), T, out.data(), 2) == 0,
               "oracle forward");
        for (int t = 0; t < T * H; ++t)
            EXPECT(std::isfinite(out[t]), "finite output");
        EXPECT(oracle_moe_forward_tokens(x.data(), ids.data(), w.data(), w13.data(), s13.data(),
                                         w2.data(), s2.data(), T, H, I, E, k, 3, g13, b2, g2,
                                         1.0, 0.0, INFINITY, toks.data(), T, out.data(), 1) == -1,
               "oracle rejects bits");
    }
    // the expert sort: every valid pair exactly once, padding slots hold P
    for (int bm : {1, 4, 16, 64}) {
        const int T = 37, k = 3, E = 9, P = T * k;
        std::vector<int32_t> ids(P);
        for (auto &v : ids)
            v = (int32_t)(u32() % 11u) - 1;
        const int cap = P / bm + std::min(E, P) + 1;
        std::vector<int32_t> sorted((size_t)cap * bm, -7), tiles(cap, -7), offs(E + 1), inv(P);
        int32_t nt = 0, bad = 0;
        EXPECT(oracle_align(ids.data(), T, k, E, bm, sorted.data(), tiles.data(), offs.data(),
                            inv.data(), &nt, &bad) == 0, "oracle align");
        std::vector<int> seen(P, 0);
        for (int s = 0; s < nt * bm; ++s) {
            const int p = sorted[s];
            EXPECT(p >= 0 && p <= P, "slot content");
            if (p < P) {
                ++seen[p];
                EXPECT(inv[p] == s, "inverse permutation");
            }
        }
        int nbad = 0;
        for (int p = 0; p < P; ++p) {
            const bool ok = ids[p] >= 0 && ids[p] < E;
            nbad += ok ? 0 : 1;
            EXPECT(seen[p] == (ok ? 1 : 0), "pair placed once");
        }
        EXPECT(nbad == bad, "invalid id count");
    }
    // the quantizer and the prepared order
    for (int bits : {2, 4})
        for (int group : {32, 64, 128}) {
            const int rows = 5, K = 256;
            std::vector<uint16_t> wq((size_t)rows * K);
            for (auto &v : wq)
                v = (uint16_t)(0x3c00u + (u32() & 0x7ffu)) ^ (uint16_t)((u32() & 1u) << 15);
            std::vector<float> imp(K, 1.5f);
            std::vector<uint32_t> codes((size_t)rows * K * bits / 32);
            std::vector<uint16_t> scales((size_t)rows * K / group);
            std::vector<int32_t> choice((size_t)rows * K / group);
            double sums[4];
            EXPECT(oracle_quantize(wq.data(), imp.data(), rows, K, bits, group, 8, codes.data(),
                                   scales.data(), choice.data(), sums) == 0, "oracle quantize");
            EXPECT(sums[0] >= 0 && sums[1] > 0, "error sums");
            const int E = 2, prow = 32, PK = 1024;
            std::vector<uint32_t> packed((size_t)E * prow * PK * bits / 32), prep(packed.size());
            for (auto &v : packed) v = u32();
            if (group <= 512 / bits) {
                EXPECT(oracle_prepare(packed.data(), E, prow, PK, bits, group, prep.data()) == 0,
                       "oracle prepare");
                uint64_t a = 0, b = 0;
                for (size_t i = 0; i < packed.size(); ++i) {
                    a += packed[i];
                    b += prep[i];
                }
                EXPECT(a == b, "prepare permutes words");
            }
        }
    for (double v : {0.0, 1e-8, 6.1e-5, 0.333, 1.0, 2049.0, 65504.0})
        EXPECT(oracle_f16_to_f64(oracle_f64_to_f16_rne(v)) == (double)(float)oracle_f16_to_f64(
                   oracle_f64_to_f16_rne(v)), "fp16 round trip");
}

int main()
{
    check_abi();
    check_oracle();
    if (failures) {
        std::fprintf(stderr, "%d host check(s) failed\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
