"""Python access to the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports
this module, and this module imports nothing from the product package.

Every function returns float64 numpy arrays; see moe_oracle.c for what each
step computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: ISO C99 (no floating-point contraction),
    -O2, OpenMP over independent (token, slot) pairs."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = d
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = d
        lib.oracle_code.argtypes = [P, i, i]
        lib.oracle_code.restype = i
        lib.oracle_weight.argtypes = [P, P, i, i, i, i, i]
        lib.oracle_weight.restype = d
        lib.oracle_qmatvec.argtypes = [P, P, i, i, i, i, P, P]
        lib.oracle_qmatvec.restype = None
        lib.oracle_swiglu.argtypes = [d, d, d, d, d]
        lib.oracle_swiglu.restype = d
        lib.oracle_expert.argtypes = [P, P, P, P, i, i, i, i, i, i, d, d, d, P, P, P, P]
        lib.oracle_expert.restype = None
        lib.oracle_moe_forward_tokens.argtypes = [P, P, P, P, P, P, P] + [i] * 9 + [d, d, d, P,
                                                                                  i, P, i]
        lib.oracle_moe_forward_tokens.restype = i
        lib.oracle_align.argtypes = [P, i, i, i, i, P, P, P, P, P, P]
        lib.oracle_align.restype = i
        lib.oracle_f64_to_f16_rne.argtypes = [d]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_quantize.argtypes = [P, P, i, i, i, i, i, P, P, P, P]
        lib.oracle_quantize.restype = i
        lib.oracle_prepare.argtypes = [P, i, i, i, i, i, P]
        lib.oracle_prepare.restype = i
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f16_to_f64(h: int) -> float:
    return _load().oracle_f16_to_f64(int(h))


def bf16_to_f64(b: int) -> float:
    return _load().oracle_bf16_to_f64(int(b))


def codes(row_words: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Signed codes of one packed row, K of them."""
    w = _c(row_words, np.uint32)
    lib = _load()
    return np.array([lib.oracle_code(_ptr(w), k, bits) for k in range(K)], dtype=np.int64)


def weight(words, scales, K, bits, group, n, k) -> float:
    w = _c(words, np.uint32)
    s = _c(scales, np.float16).view(np.uint16)
    return _load().oracle_weight(_ptr(w), _ptr(s), K, bits, group, n, k)


def qmatvec(words, scales, rows, K, bits, group, v) -> np.ndarray:
    """y = W v with W[n][k] = q * s, for one packed matrix [rows][K*bits/32]."""
    w = _c(words, np.uint32)
    s = _c(scales, np.float16).view(np.uint16)
    v = _c(v, np.float64)
    y = np.empty(rows, np.float64)
    _load().oracle_qmatvec(_ptr(w), _ptr(s), rows, K, bits, group, _ptr(v), _ptr(y))
    return y


def swiglu(g: float, u: float, alpha: float = 1.0, beta: float = 0.0,
           clamp: float = float("inf")) -> float:
    return _load().oracle_swiglu(float(g), float(u), float(alpha), float(beta), float(clamp))


def expert(w13, s13, w2, s2, H, I, bits13, group13, bits2, group2, alpha, beta, clamp, x):
    """One expert on one float64 input vector; returns (h, act, y)."""
    w13 = _c(w13, np.uint32)
    s13 = _c(s13, np.float16).view(np.uint16)
    w2 = _c(w2, np.uint32)
    s2 = _c(s2, np.float16).view(np.uint16)
    x = _c(x, np.float64)
    h = np.empty(2 * I, np.float64)
    act = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    _load().oracle_expert(_ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), H, I, bits13, group13,
                          bits2, group2, float(alpha), float(beta), float(clamp), _ptr(x),
                          _ptr(h), _ptr(act), _ptr(y))
    return h, act, y


def forward(x, topk_ids, topk_w, w13, s13, w2, s2, *, H, I, E, bits13, group13, bits2, group2,
            alpha=1.0, beta=0.0, clamp=float("inf"), tokens: Optional[Sequence[int]] = None,
            nthreads: int = 0) -> np.ndarray:
    """Routed layer output in float64, for all tokens or the listed ones."""
    x = _c(x, np.uint16)
    T = x.shape[0]
    ids = _c(topk_ids, np.int32)
    k = ids.shape[1] if ids.ndim == 2 else 1
    tw = _c(topk_w, np.float32)
    w13 = _c(w13, np.uint32)
    s13 = _c(s13, np.float16).view(np.uint16)
    w2 = _c(w2, np.uint32)
    s2 = _c(s2, np.float16).view(np.uint16)
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    out = np.empty((len(tok), H), np.float64)
    rc = _load().oracle_moe_forward_tokens(
        _ptr(x), _ptr(ids), _ptr(tw), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), T, H, I, E, k,
        bits13, group13, bits2, group2, float(alpha), float(beta), float(clamp), _ptr(tok),
        len(tok), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_moe_forward_tokens rejected its arguments")
    return out


def forward_layer(layer, tokens=None, nthreads: int = 0) -> np.ndarray:
    """`forward` on a `weight_only_bit_moe_amd.inputs.Layer`-shaped object."""
    sp = layer.spec
    return forward(layer.x, layer.topk_ids, layer.topk_w, layer.w13, layer.s13, layer.w2,
                   layer.s2, H=sp.H, I=sp.I, E=sp.E, bits13=sp.bits13, group13=sp.group13,
                   bits2=sp.bits2, group2=sp.group2, alpha=sp.alpha, beta=sp.beta,
                   clamp=sp.clamp, tokens=tokens, nthreads=nthreads)


def align(topk_ids, E: int, block_m: int):
    """Expert-sorted tile layout (see oracle_align).  Returns a dict of arrays;
    `sorted_ids` and `tile_expert` are cut to the padded total / tile count."""
    ids = _c(topk_ids, np.int32)
    T = ids.shape[0]
    k = ids.shape[1] if ids.ndim == 2 else 1
    P = T * k
    cap_tiles = P // block_m + min(E, P) + 1
    sorted_ids = np.full(cap_tiles * block_m, -7, np.int32)
    tile_expert = np.full(cap_tiles, -7, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    inv_perm = np.zeros(max(P, 1), np.int32)
    nt = np.zeros(1, np.int32)
    bad = np.zeros(1, np.int32)
    rc = _load().oracle_align(_ptr(ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(tile_expert),
                              _ptr(offsets), _ptr(inv_perm), _ptr(nt), _ptr(bad))
    if rc != 0:
        raise ValueError("oracle_align rejected its arguments")
    n = int(nt[0])
    return dict(sorted_ids=sorted_ids[: n * block_m].copy(), tile_expert=tile_expert[:n].copy(),
                expert_offsets=offsets, inv_perm=inv_perm[:P].copy(), num_tiles=n,
                bad_ids=int(bad[0]))


def f64_to_f16_rne(v: float) -> int:
    """IEEE binary16 bits of round-to-nearest-even(v), 0 <= v <= 65504."""
    return int(_load().oracle_f64_to_f16_rne(float(v)))


def quantize(w_bf16, bits: int, group: int, ncand: int = 1, imp=None):
    """Symmetric b-bit quantization of W [rows][K] given as BF16 bit patterns
    (uint16), with the importance-weighted scale search of oracle_quantize.
    Returns dict(codes [rows][K*bits/32] uint32, scales [rows][K/group] uint16
    FP16 bits, choice [rows][K/group] int32, sums [4] float64)."""
    w = _c(w_bf16, np.uint16)
    rows, K = w.shape
    codes = np.zeros((rows, K * bits // 32), np.uint32)
    scales = np.zeros((rows, K // group), np.uint16)
    choice = np.zeros((rows, K // group), np.int32)
    sums = np.zeros(4, np.float64)
    impa = None if imp is None else _c(imp, np.float32)
    rc = _load().oracle_quantize(_ptr(w), None if impa is None else _ptr(impa), rows, K, bits,
                                 group, ncand, _ptr(codes), _ptr(scales), _ptr(choice),
                                 _ptr(sums))
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments")
    return dict(codes=codes, scales=scales, choice=choice, sums=sums)


def prepare(packed, bits: int, group: int):
    """Prepared block order of codes [E, rows, K*bits/32] (uint32 or int32
    words), as oracle_prepare; returns uint32 of the same shape."""
    w = _c(np.asarray(packed).view(np.uint32), np.uint32)
    E, rows, kw = w.shape
    out = np.zeros_like(w)
    rc = _load().oracle_prepare(_ptr(w), E, rows, kw * 32 // bits, bits, group, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_prepare rejected its arguments")
    return out
