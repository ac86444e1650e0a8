/*
 * CPU oracle for the routed weight-only-quantized (WNA16) MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * Plain, slow and meant to be read against the pages.  Every value is carried
 * in IEEE double; every sum runs in ascending index order.
 *
 * What it computes (the pages give the pieces, not a formula):
 *   - Expert weights are symmetric signed b-bit codes (b = 2 or 4) packed into
 *     32-bit words, with one FP16 scale per K group and no zero point
 *     (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed" and
 *     "How it was created" step 4).  W[n][k] = q[n][k] * s[n][k / group].
 *   - Each routed expert is a gated MLP: a fused gate/up projection (w13) and
 *     a down projection (w2), each with its own bit width and group size
 *     (PR "Incubate DeepSeek V4 WNA16 runtime on SM86", "What this branch
 *     adds" item 2, "Validation completed" on projection-specific groups).
 *   - Activations are BF16 and every token carries top-k expert indices
 *     (same PR, item 3, "BF16 indexed MoE").
 *   - The gate/up pair goes through SwiGLU with alpha, beta and clamp
 *     (same PR, item 9).
 *   - out[t] = sum_j w[t][j] * W2_e * SwiGLU(W13_e x_t), e = ids[t][j].
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes of this repository):
 *   R1 words are row-major [rows][K*b/32]: row n holds the K-contiguous codes
 *      of output channel n.
 *   R2 least-significant field first: K index j*(32/b)+i sits in bits
 *      [i*b, (i+1)*b) of word j.
 *   R3 offset binary: stored field u = q + 2^(b-1).
 *   R5 scales are [rows][K/group]; a group runs along K only.
 *   R6 g' = min(g, c), u' = clamp(u, -c, c), act = g' * sigmoid(alpha g') * (u' + beta);
 *      c = +inf means no clamp.
 *   R7 w13 rows [0, I) are the gate (w1), rows [I, 2I) the up projection (w3).
 *   R8 the routing weight multiplies the expert output; weights are used as
 *      given (no renormalisation).  Ids outside [0, E) contribute nothing.
 *   R12 alignment contract of the expert-sorted tiles (see oracle_align).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> double.  Field layout: 1 sign, 5 exponent (bias 15),
 * 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^(1-15-10) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double.  Field layout: 1 sign, 8 exponent (bias 127),
 * 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);             /* subnormal: m * 2^(1-127-7) */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);  /* (1 + m/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* Signed code at K index k of one packed row (readings R2, R3). */
int oracle_code(const uint32_t *row_words, int k, int bits)
{
    int per_word = 32 / bits;
    uint32_t word = row_words[k / per_word];
    int field = k % per_word;
    uint32_t u = (word >> (field * bits)) & ((1u << bits) - 1u);
    return (int)u - (1 << (bits - 1));
}

/* Dequantized weight W[n][k] = q * s (reading R5). */
double oracle_weight(const uint32_t *words, const uint16_t *scales, int K, int bits,
                     int group, int n, int k)
{
    const uint32_t *row = words + (size_t)n * (size_t)(K * bits / 32);
    double s = oracle_f16_to_f64(scales[(size_t)n * (size_t)(K / group) + (size_t)(k / group)]);
    return (double)oracle_code(row, k, bits) * s;
}

/* y[n] = sum_k W[n][k] * v[k] for n in [0, rows), ascending k. */
void oracle_qmatvec(const uint32_t *words, const uint16_t *scales, int rows, int K, int bits,
                    int group, const double *v, double *y)
{
    for (int n = 0; n < rows; ++n) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += oracle_weight(words, scales, K, bits, group, n, k) * v[k];
        y[n] = acc;
    }
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* SwiGLU with alpha, beta and clamp (reading R6). */
double oracle_swiglu(double g, double u, double alpha, double beta, double clamp)
{
    double gc = g < clamp ? g : clamp;
    double uc = u < -clamp ? -clamp : (u > clamp ? clamp : u);
    return gc * sigmoid(alpha * gc) * (uc + beta);
}

/* One expert on one token: y = W2_e * SwiGLU(W13_e x).  x has H entries, y has
 * H entries.  Work space: h (2I) and act (I). */
void oracle_expert(const uint32_t *w13, const uint16_t *s13, const uint32_t *w2,
                   const uint16_t *s2, int H, int I, int bits13, int group13, int bits2,
                   int group2, double alpha, double beta, double clamp, const double *x,
                   double *h, double *act, double *y)
{
    oracle_qmatvec(w13, s13, 2 * I, H, bits13, group13, x, h);
    for (int i = 0; i < I; ++i)
        act[i] = oracle_swiglu(h[i], h[I + i], alpha, beta, clamp);
    oracle_qmatvec(w2, s2, H, I, bits2, group2, act, y);
}

/*
 * Routed layer for the tokens listed in `tokens` (ntok of them); row r of
 * `out` ([ntok][H]) is the result for token tokens[r].  Passing every token in
 * order gives the whole layer.  Per-(token, slot) expert outputs are computed
 * independently (in parallel when OpenMP is on, `nthreads` <= 0 meaning its
 * default) and then summed per token in slot order j = 0..k-1.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_moe_forward_tokens(const uint16_t *x, const int32_t *ids, const float *topk_w,
                              const uint32_t *w13, const uint16_t *s13, const uint32_t *w2,
                              const uint16_t *s2, int T, int H, int I, int E, int topk,
                              int bits13, int group13, int bits2, int group2, double alpha,
                              double beta, double clamp, const int32_t *tokens, int ntok,
                              double *out, int nthreads)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0 || ntok < 0)
        return -1;
    if ((bits13 != 2 && bits13 != 4) || (bits2 != 2 && bits2 != 4))
        return -1;
    if (group13 <= 0 || group2 <= 0 || H % group13 || I % group2)
        return -1;
    if ((H * bits13) % 32 || (I * bits2) % 32)
        return -1;
    for (int r = 0; r < ntok; ++r)
        if (tokens[r] < 0 || tokens[r] >= T)
            return -1;

    const size_t w13_expert = (size_t)2 * I * (size_t)(H * bits13 / 32);
    const size_t s13_expert = (size_t)2 * I * (size_t)(H / group13);
    const size_t w2_expert = (size_t)H * (size_t)(I * bits2 / 32);
    const size_t s2_expert = (size_t)H * (size_t)(I / group2);
    const long npairs = (long)ntok * topk;

    double *ybuf = (double *)calloc((size_t)(npairs > 0 ? npairs : 1) * (size_t)H, sizeof(double));
    int *used = (int *)calloc((size_t)(npairs > 0 ? npairs : 1), sizeof(int));
    if (!ybuf || !used) {
        free(ybuf);
        free(used);
        return -1;
    }
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *h = (double *)malloc(sizeof(double) * (size_t)2 * I);
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
        if (!xv || !h || !act) {
            bad = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long pr = 0; pr < npairs; ++pr) {
                int t = tokens[pr / topk];
                int j = (int)(pr % topk);
                int e = ids[(size_t)t * topk + j];
                if (e < 0 || e >= E)
                    continue;                    /* R8: contributes nothing */
                for (int k = 0; k < H; ++k)
                    xv[k] = oracle_bf16_to_f64(x[(size_t)t * H + k]);
                oracle_expert(w13 + (size_t)e * w13_expert, s13 + (size_t)e * s13_expert,
                              w2 + (size_t)e * w2_expert, s2 + (size_t)e * s2_expert, H, I,
                              bits13, group13, bits2, group2, alpha, beta, clamp, xv, h, act,
                              ybuf + (size_t)pr * H);
                used[pr] = 1;
            }
        }
        free(xv);
        free(h);
        free(act);
    }
    if (!bad) {
        for (int r = 0; r < ntok; ++r) {
            double *o = out + (size_t)r * H;
            for (int n = 0; n < H; ++n)
                o[n] = 0.0;
            int t = tokens[r];
            for (int j = 0; j < topk; ++j) {
                long pr = (long)r * topk + j;
                if (!used[pr])
                    continue;
                double w = (double)topk_w[(size_t)t * topk + j];
                const double *y = ybuf + (size_t)pr * H;
                for (int n = 0; n < H; ++n)
                    o[n] += w * y[n];
            }
        }
    }
    free(ybuf);
    free(used);
    return bad ? -1 : 0;
}

/*
 * Expert-sorted tile layout of the (token, slot) pairs (reading R12).
 *
 * Pair p = t*topk + j has expert ids[p].  counts[e] = number of pairs with
 * expert e.  expert_offsets (E+1 entries) is the exclusive prefix sum of
 * counts rounded up to a multiple of block_m; its last entry is the padded
 * total.  sorted_ids[expert_offsets[e] + r] is the r-th smallest pair index
 * with expert e (a stable counting sort); the padding slots of each expert
 * hold P = T*topk.  tile_expert[b] = e for every tile b of block_m slots in
 * e's range; num_tiles = padded total / block_m.  inv_perm[p] is the slot of
 * pair p, or -1 when ids[p] lies outside [0, E) (such pairs are skipped and
 * counted in *bad_ids).  Buffers must hold the padded total (sorted_ids), the
 * tile count (tile_expert) and P (inv_perm) entries.  Returns 0 or -1.
 */
int oracle_align(const int32_t *ids, int T, int topk, int E, int block_m, int32_t *sorted_ids,
                 int32_t *tile_expert, int32_t *expert_offsets, int32_t *inv_perm,
                 int32_t *num_tiles, int32_t *bad_ids)
{
    if (T < 0 || topk <= 0 || E <= 0 || block_m <= 0)
        return -1;
    const long P = (long)T * topk;
    long *counts = (long *)calloc((size_t)E, sizeof(long));
    long *fill = (long *)calloc((size_t)E, sizeof(long));
    if (!counts || !fill) {
        free(counts);
        free(fill);
        return -1;
    }
    long bad = 0;
    for (long p = 0; p < P; ++p) {
        int e = ids[p];
        if (e < 0 || e >= E)
            ++bad;
        else
            ++counts[e];
    }
    long off = 0;
    for (int e = 0; e < E; ++e) {
        expert_offsets[e] = (int32_t)off;
        long padded = (counts[e] + block_m - 1) / block_m * block_m;
        for (long s = off; s < off + padded; ++s)
            sorted_ids[s] = (int32_t)P;
        for (long b = off / block_m; b < (off + padded) / block_m; ++b)
            tile_expert[b] = e;
        off += padded;
    }
    expert_offsets[E] = (int32_t)off;
    for (long p = 0; p < P; ++p) {
        int e = ids[p];
        if (e < 0 || e >= E) {
            inv_perm[p] = -1;
            continue;
        }
        long slot = expert_offsets[e] + fill[e]++;
        sorted_ids[slot] = (int32_t)p;
        inv_perm[p] = (int32_t)slot;
    }
    *num_tiles = (int32_t)(off / block_m);
    *bad_ids = (int32_t)bad;
    free(counts);
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Quantizer: from float weights to the codes and scales the layer reads
 * (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "How it was created"
 * steps 2-5: symmetric b-bit weights per K group, a scale search weighted by
 * an activation importance matrix, signed codes packed into 32-bit words, and
 * weighted and unweighted reconstruction error; "imatrix-weighted RTN").
 *
 * Readings (the card names the steps, not the arithmetic):
 *   Q1 the input is W [rows][K] in BF16 and an importance imp[K] >= 0 per
 *      input channel (NULL: every channel 1, i.e. plain unweighted RTN).
 *   Q2 base scale of a group: s0 = amax / ((2^b - 1) / 2) in FP32, amax the
 *      largest |w| of the group (the group's range onto the code span).
 *   Q3 candidates c = 0..C-1: s_c = fp16_rne(min(s0 * (1 - c / (2C)), 65504)),
 *      each factor and product in FP32 (C = 1: s0 only).
 *   Q4 codes for a scale s: q = clamp(rne(w / s), -2^(b-1), 2^(b-1) - 1) with
 *      w / s an FP32 division; s = 0 gives q = 0.
 *   Q5 err_c = sum_k imp_k (w_k - s_c q_k)^2 in double, ascending k; the
 *      smallest err_c wins, ties to the smaller c.
 *   Q6 error sums over the matrix (double): (w - w')^2, w^2, imp (w - w')^2,
 *      imp w^2, with w' = s q the reconstruction.
 * Codes are stored by R2/R3 (u = q + 2^(b-1), least-significant field first).
 * ------------------------------------------------------------------------- */

/* IEEE binary16 bits of the round-to-nearest-even of a finite v >= 0 that
 * is at most 65504 (the largest finite half). */
uint16_t oracle_f64_to_f16_rne(double v)
{
    if (v == 0.0)
        return 0;
    int e;
    frexp(v, &e);                       /* v = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;                     /* floor(log2 v) */
    if (ex < -14)
        ex = -14;                       /* subnormal range: quantum 2^-24 */
    double quantum = ldexp(1.0, ex - 10);
    double r = rint(v / quantum) * quantum;   /* rint: nearest, ties to even */
    if (r == 0.0)
        return 0;
    frexp(r, &e);
    ex = e - 1;
    if (ex < -14)                       /* subnormal: r = m * 2^-24 */
        return (uint16_t)(r / ldexp(1.0, -24));
    uint16_t frac = (uint16_t)(r / ldexp(1.0, ex - 10) - 1024.0);
    return (uint16_t)(((ex + 15) << 10) | frac);
}

/* Q4: the code of w for the FP16 scale s (both exact in float). */
static int quant_code(float w, float s, int bits)
{
    const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
    if (s == 0.0f)
        return 0;
    float r = rintf(w / s);
    if (r < (float)lo)
        return lo;
    if (r > (float)hi)
        return hi;
    return (int)r;
}

/*
 * Quantize W [rows][K] (BF16 bits) with groups of `group` along K.
 * Writes codes [rows][K*bits/32], scales [rows][K/group] (FP16 bits),
 * choice[rows][K/group] (the winning candidate c) and sums[4] (Q6).
 * Returns 0, or -1 on bad arguments.
 */
int oracle_quantize(const uint16_t *w, const float *imp, int rows, int K, int bits, int group,
                    int ncand, uint32_t *codes, uint16_t *scales, int32_t *choice,
                    double *sums)
{
    if (rows < 0 || K <= 0 || (bits != 2 && bits != 4) || group <= 0 || K % group ||
        (K * bits) % 32 || ncand < 1)
        return -1;
    const int ngroups = K / group, kw = K * bits / 32, per_word = 32 / bits;
    const float half_span = (float)((1 << bits) - 1) / 2.0f;
    double s_err = 0.0, s_w2 = 0.0, s_ierr = 0.0, s_iw2 = 0.0;
    int *q = (int *)malloc(sizeof(int) * (size_t)group);
    int *qbest = (int *)malloc(sizeof(int) * (size_t)group);
    if (!q || !qbest) {
        free(q);
        free(qbest);
        return -1;
    }
    for (int n = 0; n < rows; ++n) {
        uint32_t *row_words = codes + (size_t)n * kw;
        memset(row_words, 0, sizeof(uint32_t) * (size_t)kw);
        for (int G = 0; G < ngroups; ++G) {
            const uint16_t *wg = w + (size_t)n * K + (size_t)G * group;
            float amax = 0.0f;
            for (int i = 0; i < group; ++i) {
                float a = (float)fabs(oracle_bf16_to_f64(wg[i]));
                if (a > amax)
                    amax = a;
            }
            const float s0 = amax / half_span;                          /* Q2 */
            double best = 0.0;
            int cbest = -1;
            uint16_t hbest = 0;
            for (int c = 0; c < ncand; ++c) {
                const float f = 1.0f - (float)c / (float)(2 * ncand);    /* Q3 */
                float sc = s0 * f;
                if (sc > 65504.0f)
                    sc = 65504.0f;
                const uint16_t h = oracle_f64_to_f16_rne((double)sc);
                const double s = oracle_f16_to_f64(h);
                double err = 0.0;
                for (int i = 0; i < group; ++i) {
                    const double wv = oracle_bf16_to_f64(wg[i]);
                    q[i] = quant_code((float)wv, (float)s, bits);        /* Q4 */
                    const double d = wv - s * (double)q[i];
                    err += (imp ? (double)imp[G * group + i] : 1.0) * d * d;   /* Q5 */
                }
                if (cbest < 0 || err < best) {
                    best = err;
                    cbest = c;
                    hbest = h;
                    memcpy(qbest, q, sizeof(int) * (size_t)group);
                }
            }
            scales[(size_t)n * ngroups + G] = hbest;
            if (choice)
                choice[(size_t)n * ngroups + G] = cbest;
            const double s = oracle_f16_to_f64(hbest);
            for (int i = 0; i < group; ++i) {
                const int k = G * group + i;
                const uint32_t u = (uint32_t)(qbest[i] + (1 << (bits - 1)));   /* R3 */
                row_words[k / per_word] |= u << ((k % per_word) * bits);      /* R2 */
                const double wv = oracle_bf16_to_f64(wg[i]);
                const double d = wv - s * (double)qbest[i];
                const double im = imp ? (double)imp[k] : 1.0;
                s_err += d * d;                                              /* Q6 */
                s_w2 += wv * wv;
                s_ierr += im * d * d;
                s_iw2 += im * wv * wv;
            }
        }
    }
    sums[0] = s_err;
    sums[1] = s_w2;
    sums[2] = s_ierr;
    sums[3] = s_iw2;
    free(q);
    free(qbest);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Prepared code order: a one-time reorder of one projection's packed codes
 * (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed": signed
 * codes packed into INT32 words, R1-R3) into blocks that the decode-shaped
 * GPU kernels read with one 16-byte load per lane.  The pages describe no
 * such layout; it is this library's, stated in include/moe_wna16.h, and is a
 * pure permutation of words.  Written here from that statement in terms of K
 * offsets: a load unit is 512/bits K elements of a row, a block 16 rows x one
 * unit, blocks ordered [expert][row/16][unit]; slot (g*16 + r) of a block
 * lists, group by group, the words of row r holding the codes at in-group K
 * offsets [g*group/4, (g+1)*group/4).  2-bit codes with group 32: lane groups
 * 2h and 2h+1 share slot (h*16 + r), which lists for groups 0..7 the word
 * holding in-group offsets [16h, 16h+16).
 * ------------------------------------------------------------------------- */
int oracle_prepare(const uint32_t *packed, int E, int rows, int K, int bits, int group,
                   uint32_t *out)
{
    if (E < 0 || rows < 0 || rows % 16 || K <= 0 || (bits != 2 && bits != 4) || group <= 0 ||
        K % group || K % (512 / bits) || group % 32 || group > 512 / bits)
        return -1;
    const int unit = 512 / bits, nunits = K / unit, kw = K * bits / 32;
    const int per_word = 32 / bits;                 /* codes per word */
    const int gpu = unit / group;                   /* groups per unit */
    for (int e = 0; e < E; ++e)
        for (int rb = 0; rb < rows / 16; ++rb)
            for (int u = 0; u < nunits; ++u) {
                uint32_t *blk = out + (((size_t)e * (rows / 16) + rb) * nunits + u) * 256;
                for (int r = 0; r < 16; ++r) {
                    const uint32_t *row = packed + ((size_t)e * rows + rb * 16 + r) * kw;
                    if (bits == 2 && group == 32) {
                        for (int h = 0; h < 2; ++h)
                            for (int gq = 0; gq < 8; ++gq) {
                                const int k = u * unit + gq * 32 + 16 * h;
                                blk[(h * 16 + r) * 8 + gq] = row[k / per_word];
                            }
                        continue;
                    }
                    for (int g = 0; g < 4; ++g) {
                        int t = 0;
                        for (int gq = 0; gq < gpu; ++gq)
                            for (int k = g * group / 4; k < (g + 1) * group / 4; k += per_word)
                                blk[(g * 16 + r) * 4 + t++] =
                                    row[(u * unit + gq * group + k) / per_word];
                    }
                }
            }
    return 0;
}
