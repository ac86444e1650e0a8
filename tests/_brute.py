"""Brute-force dense reference for the oracle's own pins (tiny inputs only).

Written independently of oracle/moe_oracle.c: vectorised numpy, every expert
evaluated for every token, with routing weight 0 for the experts a token did
not select.  Used only to check the oracle.
"""
import numpy as np


def unpack(words: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Signed codes [..., K] of packed rows [..., K*bits/32]: field i of word j
    holds K index j*(32/bits)+i, stored as q + 2^(bits-1)."""
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint64)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    fields = (w[..., :, None] >> shifts) & np.uint64((1 << bits) - 1)
    u = fields.reshape(*w.shape[:-1], w.shape[-1] * per)[..., :K]
    return u.astype(np.int64) - (1 << (bits - 1))


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of `unpack` along the last axis (K must be a multiple of 32/bits)."""
    per = 32 // bits
    q = np.asarray(codes, dtype=np.int64)
    u = (q + (1 << (bits - 1))).astype(np.uint64)
    assert u.min(initial=0) >= 0 and u.max(initial=0) < (1 << bits)
    u = u.reshape(*q.shape[:-1], q.shape[-1] // per, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return np.bitwise_or.reduce(u << shifts, axis=-1).astype(np.uint32)


def dequant(words, scales, K, bits, group):
    q = unpack(words, K, bits).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=-1)
    return q * s


def bf16_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def swiglu(g, u, alpha, beta, clamp):
    gc = np.minimum(g, clamp)
    uc = np.clip(u, -clamp, clamp)
    return gc / (1.0 + np.exp(-alpha * gc)) * (uc + beta)


def dense_forward(layer) -> np.ndarray:
    sp = layer.spec
    T, H, I, E, k = sp.T, sp.H, sp.I, sp.E, sp.topk
    W13 = dequant(layer.w13, layer.s13, H, sp.bits13, sp.group13)   # [E, 2I, H]
    W2 = dequant(layer.w2, layer.s2, I, sp.bits2, sp.group2)         # [E, H, I]
    x = bf16_to_f64(layer.x)                                         # [T, H]
    coef = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            e = int(layer.topk_ids[t, j])
            if 0 <= e < E:
                coef[t, e] += float(layer.topk_w[t, j])
    h = np.einsum("enk,tk->ten", W13, x)                             # [T, E, 2I]
    act = swiglu(h[..., :I], h[..., I:], sp.alpha, sp.beta, sp.clamp)
    y = np.einsum("eni,tei->ten", W2, act)                           # [T, E, H]
    return np.einsum("te,ten->tn", coef, y)
