// Fragment order of the K dimension used by the WNA16 GEMM kernels.
//
// The GEMMs feed 16x16x32 BF16 MFMAs.  For one MFMA step every lane holds 8
// consecutive K elements of its fragment; lane l (0..63) belongs to lane group
// g = l / 16.  The packed weight codes are turned into BF16 two at a time with
// one shift, one mask and one OR (see unpack in kernels.hip): a 4-bit word
// yields the field pairs (i, i+4) and a 2-bit word the pairs (i, i+8).  Those
// pairs are adjacent in the MFMA fragment, so the activation operand must list
// its K elements in the same order.  Activations are therefore stored, inside
// each quantization group of `gs` elements, at position
//
//     pos = (s * 4 + g) * 8 + v      (MFMA step s, lane group g, element v)
//
// holding in-group K offset frag_src(bits, gs, pos).  Every MFMA step stays
// inside one group, so a group's partial product can be scaled once.
#pragma once

#if defined(__HIPCC__)
#define WNA16_HD __host__ __device__ __forceinline__
#else
#define WNA16_HD inline
#endif

namespace wna16 {

// In-group K offset stored at fragment position `pos` (0 <= pos < gs).
WNA16_HD int frag_src(int bits, int gs, int pos)
{
    const int s = pos >> 5, g = (pos >> 3) & 3, v = pos & 7;
    if (bits == 4)  // lane group g owns the gs/4 codes starting at g*gs/4; step s is its dword s
        return g * (gs >> 2) + 8 * s + (v >> 1) + 4 * (v & 1);
    if (gs == 32)   // 2-bit, one step per group: lane groups 2h, 2h+1 share dword h
        return 16 * (g >> 1) + 4 * (g & 1) + (v >> 1) + 8 * (v & 1);
    // 2-bit: step s reads half (s & 1) of dword (s >> 1) of the lane group's codes
    return g * (gs >> 2) + 16 * (s >> 1) + 4 * (s & 1) + (v >> 1) + 8 * (v & 1);
}

// Inverse of frag_src: fragment position of in-group K offset `off`.
WNA16_HD int frag_dst(int bits, int gs, int off)
{
    int g, s, v;
    if (bits == 4) {
        const int q = gs >> 2, r = off % q, r8 = r & 7;
        g = off / q;
        s = r >> 3;
        v = 2 * (r8 & 3) + (r8 >> 2);
    } else if (gs == 32) {
        const int r16 = off & 15, r8 = r16 & 7;
        g = 2 * (off >> 4) + (r8 >> 2);
        s = 0;
        v = 2 * (r8 & 3) + (r16 >> 3);
    } else {
        const int q = gs >> 2, r = off % q, r16 = r & 15, r8 = r16 & 7;
        g = off / q;
        s = 2 * (r >> 4) + (r8 >> 2);
        v = 2 * (r8 & 3) + (r16 >> 3);
    }
    return (s * 4 + g) * 8 + v;
}

// 2-bit fields are turned into BF16 without first shifting them down: the
// fields of one 32-bit word are read at bit offsets 0, 2 and 4 of the word
// shifted right by 0, 6 or 12, giving the BF16 number 128 + m*u with
// m = 1, 4 or 16.  The activation at that fragment position is stored divided
// by m (an exact power-of-two scaling), so the product is x*(128/m + u).
// frag_shift returns log2(m) for fragment position pos (0 for 4-bit codes).
WNA16_HD int frag_shift(int bits, int gs, int pos)
{
    if (bits == 4)
        return 0;
    const int s = pos >> 5, g = (pos >> 3) & 3, v = pos & 7;
    const int h = (gs == 32) ? (g & 1) : (s & 1);  // half of the word (fields 4h..4h+3)
    const int i = 4 * h + (v >> 1);                // field pair (i, i + 8)
    return 2 * (i % 3);
}

// With a = x/m and the operand 128 + m*u = 128 + m*(q + 2^(bits-1)):
//   x*q = a*(128 + m*u) - a*(128 + m*2^(bits-1)).
// frag_bias_weight is that last factor, so the sum of x*q over a group is the
// MFMA result minus (sum over the group of a * frag_bias_weight).
WNA16_HD int frag_bias_weight(int bits, int gs, int pos)
{
    return 128 + ((1 << (bits - 1)) << frag_shift(bits, gs, pos));
}

// Prepared code layout (written once by moe_wna16_prepare, read by the
// decode-shaped kernels).  A load unit is UK = 512 / bits consecutive K
// elements of one row (16 dwords: 1, 2, 4 or 8 quantization groups).  The
// codes of 16 rows x one unit form a block; blocks are stored
// [expert][row / 16][unit].  Inside a block, lane l = 16 g + c (row c of the
// 16, lane group g) finds at dwords l * 4 .. l * 4 + 3 the code words its MFMA
// fragments read, in register order: for each group of the unit in turn, the
// words holding lane group g's codes of that group (in-group K offsets
// [g * gs / 4, (g + 1) * gs / 4), see frag_src).  2-bit codes with gs = 32
// hold only 8 codes per lane group and group, half a word; lane groups 2h and
// 2h + 1 share word h of each group, so that block stores 32 lanes x 8 words,
// lane h * 16 + c at dwords (h * 16 + c) * 8 .. + 7, one word per group.
constexpr int kPrepBlockDwords = 256;

// Dword of the row's unit (0..15) that register t of lane group g holds.
WNA16_HD int prep_src_dword(int bits, int gs, int g, int t)
{
    if (bits == 2 && gs == 32)           // t = group (0..7), g / 2 = half
        return 2 * t + (g >> 1);
    const int per = gs * bits / 128;     // words per lane group and group: 4, 2 or 1
    const int words = gs * bits / 32;    // words per group
    return (t / per) * words + g * per + t % per;
}

// Dword offset, inside a block, of register t of lane (g, c).
WNA16_HD int prep_block_dword(int bits, int gs, int g, int c, int t)
{
    if (bits == 2 && gs == 32)
        return ((g >> 1) * 16 + c) * 8 + t;
    return (g * 16 + c) * 4 + t;
}

}  // namespace wna16
