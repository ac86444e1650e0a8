"""ctypes binding of libmoe_wna16.so (include/moe_wna16.h).

Argument marshalling only: every step of the layer runs in the library's
gfx950 kernels.  Torch supplies device memory and the current stream.  If the
library has not been built, every call raises; nothing falls back to another
implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_wna16.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EARCH, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7

#: every symbol include/moe_wna16.h declares
EXPORTED = ("moe_wna16_workspace_size", "moe_wna16_workspace_f32_offset",
            "moe_wna16_workspace_layout", "moe_wna16_plan",
            "moe_wna16_forward", "moe_wna16_forward_profiled", "moe_wna16_align",
            "moe_wna16_quantize", "moe_wna16_prepare", "moe_wna16_forward_prepared",
            "moe_wna16_forward_noalloc", "moe_wna16_status_string")


class QParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("max_tiles", ctypes.c_int32),
                ("w13_variant", ctypes.c_int32), ("w2_variant", ctypes.c_int32),
                ("gemms_one_launch", ctypes.c_int32), ("convert_in_w2", ctypes.c_int32),
                ("single_launch", ctypes.c_int32), ("w13_ksplit", ctypes.c_int32)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("meta", "expert_offsets", "sorted_ids",
                                                "tile_expert", "inv_perm", "out_f32", "total")]


class MoeWna16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {moe_wna16_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m weight_only_bit_moe_amd.build` "
            "(the layer has no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    P, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_wna16_workspace_size.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
    lib.moe_wna16_workspace_size.restype = i
    lib.moe_wna16_workspace_f32_offset.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
    lib.moe_wna16_workspace_f32_offset.restype = i
    lib.moe_wna16_workspace_layout.argtypes = [i, i, i, i, i, ctypes.POINTER(WorkspaceLayout)]
    lib.moe_wna16_workspace_layout.restype = i
    lib.moe_wna16_plan.argtypes = [i, i, i, i, i, QParams, QParams, ctypes.POINTER(Plan)]
    lib.moe_wna16_plan.restype = i
    lib.moe_wna16_forward.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, QParams, QParams,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P, sz, P]
    lib.moe_wna16_forward.restype = i
    lib.moe_wna16_forward_profiled.argtypes = lib.moe_wna16_forward.argtypes + [P]
    lib.moe_wna16_forward_profiled.restype = i
    lib.moe_wna16_align.argtypes = [P, i, i, i, i, P, P, P, P, P, P, P]
    lib.moe_wna16_align.restype = i
    lib.moe_wna16_quantize.argtypes = [P, P, i, i, QParams, i, P, P, P, P]
    lib.moe_wna16_quantize.restype = i
    lib.moe_wna16_prepare.argtypes = [P, i, i, i, QParams, P, P]
    lib.moe_wna16_prepare.restype = i
    lib.moe_wna16_forward_prepared.argtypes = lib.moe_wna16_forward.argtypes + [P]
    lib.moe_wna16_forward_prepared.restype = i
    lib.moe_wna16_forward_noalloc.argtypes = lib.moe_wna16_forward.argtypes[:18] + [P]
    lib.moe_wna16_forward_noalloc.restype = i
    lib.moe_wna16_status_string.argtypes = [i]
    lib.moe_wna16_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---- the C entry points, same names and argument order ---------------------

def moe_wna16_status_string(status: int) -> str:
    return load_library().moe_wna16_status_string(int(status)).decode()


def moe_wna16_workspace_size(T: int, H: int, I: int, E: int, topk: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().moe_wna16_workspace_size(T, H, I, E, topk, ctypes.byref(out))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_workspace_size")
    return out.value


def moe_wna16_workspace_f32_offset(T: int, H: int, I: int, E: int, topk: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().moe_wna16_workspace_f32_offset(T, H, I, E, topk, ctypes.byref(out))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_workspace_f32_offset")
    return out.value


def moe_wna16_workspace_layout(T: int, H: int, I: int, E: int, topk: int) -> dict:
    """Byte offsets of the sort results, status words and FP32 sum inside a
    forward's workspace (dict with the struct's field names)."""
    lay = WorkspaceLayout()
    st = load_library().moe_wna16_workspace_layout(T, H, I, E, topk, ctypes.byref(lay))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_workspace_layout")
    return {n: getattr(lay, n) for n, _ in WorkspaceLayout._fields_}


def workspace_meta(workspace, T, H, I, E, topk):
    """The 26 int32 status words of a completed forward (see the header):
    [0] tiles, [1] ids outside [0, E), [2] fused decode waits that gave up,
    [8..25] the prefill tile kernels' XCD split."""
    torch = _torch()
    off = moe_wna16_workspace_layout(T, H, I, E, topk)["meta"]
    return workspace[off: off + 26 * 4].view(torch.int32)


def workspace_sort(workspace, T, H, I, E, topk, block_m):
    """The expert sort a completed forward ran, read from its workspace: a dict
    like align() returns, cut to the tile count (host numpy arrays)."""
    torch = _torch()
    lay = moe_wna16_workspace_layout(T, H, I, E, topk)
    meta = workspace_meta(workspace, T, H, I, E, topk).cpu().numpy()
    n = int(meta[0])
    P = T * topk

    def ints(name, count):
        off = lay[name]
        return workspace[off: off + count * 4].view(torch.int32).cpu().numpy()

    return dict(sorted_ids=ints("sorted_ids", n * block_m), tile_expert=ints("tile_expert", n),
                expert_offsets=ints("expert_offsets", E + 1), inv_perm=ints("inv_perm", P),
                num_tiles=n, bad_ids=int(meta[1]))


def workspace_f32_sum(workspace, T, H, I, E, topk):
    """View of the FP32 sum (before BF16 rounding) inside a forward's workspace."""
    torch = _torch()
    off = moe_wna16_workspace_f32_offset(T, H, I, E, topk)
    return workspace[off: off + T * H * 4].view(torch.float32).view(T, H)


def moe_wna16_plan(T, H, I, E, topk, q13: Tuple[int, int], q2: Tuple[int, int]) -> dict:
    plan = Plan()
    st = load_library().moe_wna16_plan(T, H, I, E, topk, QParams(*q13), QParams(*q2),
                                       ctypes.byref(plan))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_plan")
    return dict(block_m=plan.block_m, max_tiles=plan.max_tiles, w13_variant=plan.w13_variant,
                w2_variant=plan.w2_variant, gemms_one_launch=plan.gemms_one_launch,
                convert_in_w2=plan.convert_in_w2, single_launch=plan.single_launch,
                w13_ksplit=plan.w13_ksplit)


def moe_wna16_forward(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H,
                      I, E, topk, q13, q2, alpha, beta, clamp, out, workspace, workspace_bytes,
                      stream) -> int:
    """Raw entry point on integer device addresses; returns the status."""
    return load_library().moe_wna16_forward(
        x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H, I, E, topk,
        QParams(*q13), QParams(*q2), alpha, beta, clamp, out, workspace, workspace_bytes, stream)


def moe_wna16_forward_profiled(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed,
                               w2_scales, T, H, I, E, topk, q13, q2, alpha, beta, clamp, out,
                               workspace, workspace_bytes, stream, events) -> int:
    """Raw entry point; `events` is a ctypes array of 8 hipEvent_t handles."""
    return load_library().moe_wna16_forward_profiled(
        x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H, I, E, topk,
        QParams(*q13), QParams(*q2), alpha, beta, clamp, out, workspace, workspace_bytes, stream,
        events)


def moe_wna16_forward_prepared(x, topk_ids, topk_w, w13_prepared, w13_scales, w2_prepared,
                               w2_scales, T, H, I, E, topk, q13, q2, alpha, beta, clamp, out,
                               workspace, workspace_bytes, stream, events=None) -> int:
    """Raw entry point; codes in the prepared order; `events` None or 8 hipEvent_t."""
    return load_library().moe_wna16_forward_prepared(
        x, topk_ids, topk_w, w13_prepared, w13_scales, w2_prepared, w2_scales, T, H, I, E, topk,
        QParams(*q13), QParams(*q2), alpha, beta, clamp, out, workspace, workspace_bytes, stream,
        events)


def moe_wna16_forward_noalloc(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed,
                              w2_scales, T, H, I, E, topk, q13, q2, alpha, beta, clamp, out,
                              stream) -> int:
    """Raw entry point without a workspace (the library's per-GPU scratch);
    returns the status."""
    return load_library().moe_wna16_forward_noalloc(
        x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, T, H, I, E, topk,
        QParams(*q13), QParams(*q2), alpha, beta, clamp, out, stream)


def moe_wna16_prepare(packed, E, rows, K, q, prepared_out, stream) -> int:
    """Raw entry point on integer device addresses; returns the status."""
    return load_library().moe_wna16_prepare(packed, E, rows, K, QParams(*q), prepared_out, stream)


def moe_wna16_align(topk_ids, T, topk, E, block_m, sorted_ids, tile_expert, expert_offsets,
                    inv_perm, num_tiles, bad_ids, stream) -> int:
    """Raw entry point on integer device addresses; returns the status."""
    return load_library().moe_wna16_align(topk_ids, T, topk, E, block_m, sorted_ids, tile_expert,
                                          expert_offsets, inv_perm, num_tiles, bad_ids, stream)


def moe_wna16_quantize(w, imp, rows, K, q: Tuple[int, int], n_candidates, codes_out,
                       scales_out, err_sums_out, stream) -> int:
    """Raw entry point on integer device addresses; returns the status."""
    return load_library().moe_wna16_quantize(w, imp, rows, K, QParams(*q), n_candidates,
                                             codes_out, scales_out, err_sums_out, stream)


# ---- torch conveniences (allocation + marshalling) --------------------------

def _torch():
    import torch
    return torch


def _check(t, name, dtypes, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


SYNC_BYTES = 32768   # MOE_WNA16_SYNC_BYTES: leading workspace bytes that start at zero


def workspace_for(T, H, I, E, topk, device):
    """A forward workspace for these sizes, zeroed (the single-launch decode's
    counters at its start must be zero before the first call; every call
    leaves them zero)."""
    torch = _torch()
    n = moe_wna16_workspace_size(T, H, I, E, topk)
    return torch.zeros(max(n, SYNC_BYTES), dtype=torch.uint8, device=device)


def forward(x, topk_ids, topk_w, w13_packed, w13_scales, w2_packed, w2_scales, *,
            bits=(4, 4), group=(128, 128), alpha: float = 1.0, beta: float = 0.0,
            clamp: Optional[float] = None, out=None, workspace=None, prepared: bool = False):
    """Routed WNA16 MoE layer on torch tensors (see include/moe_wna16.h).

    x [T, H] bf16; topk_ids [T, k] int32; topk_w [T, k] float32;
    w13_packed [E, 2I, H*b13/32] int32 (or uint32 bits); w13_scales [E, 2I, H/g13] fp16;
    w2_packed [E, H, I*b2/32] int32; w2_scales [E, H, I/g2] fp16.
    `bits` and `group` are (w13, w2) pairs.  With prepared=True the two code
    tensors hold the output of prepare() (same shapes) and the call must be
    decode-shaped.  Returns out [T, H] bf16.
    """
    torch = _torch()
    dev = x.device
    _check(x, "x", (torch.bfloat16,), dev)
    _check(topk_ids, "topk_ids", (torch.int32,), dev)
    _check(topk_w, "topk_w", (torch.float32,), dev)
    _check(w13_packed, "w13_packed", (torch.int32, torch.uint32), dev)
    _check(w13_scales, "w13_scales", (torch.float16,), dev)
    _check(w2_packed, "w2_packed", (torch.int32, torch.uint32), dev)
    _check(w2_scales, "w2_scales", (torch.float16,), dev)
    T, H = x.shape
    E, twoI = w13_packed.shape[0], w13_packed.shape[1]
    I = twoI // 2
    topk = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    b13, b2 = bits
    g13, g2 = group
    if tuple(w13_packed.shape) != (E, 2 * I, H * b13 // 32):
        raise ValueError(f"w13_packed shape {tuple(w13_packed.shape)} != {(E, 2 * I, H * b13 // 32)}")
    if tuple(w13_scales.shape) != (E, 2 * I, H // g13):
        raise ValueError(f"w13_scales shape {tuple(w13_scales.shape)} != {(E, 2 * I, H // g13)}")
    if tuple(w2_packed.shape) != (E, H, I * b2 // 32):
        raise ValueError(f"w2_packed shape {tuple(w2_packed.shape)} != {(E, H, I * b2 // 32)}")
    if tuple(w2_scales.shape) != (E, H, I // g2):
        raise ValueError(f"w2_scales shape {tuple(w2_scales.shape)} != {(E, H, I // g2)}")
    if tuple(topk_w.shape) != tuple(topk_ids.shape) or topk_ids.shape[0] != T:
        raise ValueError("topk_ids / topk_w must both be [T, k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", (torch.bfloat16,), dev)
    if workspace is None:
        workspace = workspace_for(T, H, I, E, topk, dev)
    _check(workspace, "workspace", (torch.uint8,), dev)
    c = math.inf if clamp is None else float(clamp)
    args = (x.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), w13_packed.data_ptr(),
            w13_scales.data_ptr(), w2_packed.data_ptr(), w2_scales.data_ptr(), T, H, I, E, topk,
            (b13, g13), (b2, g2), float(alpha), float(beta), c, out.data_ptr(),
            workspace.data_ptr(), workspace.numel(), _stream(dev))
    if prepared:
        st, name = moe_wna16_forward_prepared(*args), "moe_wna16_forward_prepared"
    else:
        st, name = moe_wna16_forward(*args), "moe_wna16_forward"
    if st != OK:
        raise MoeWna16Error(st, name)
    return out


def prepare(packed, bits: int, group: int):
    """Prepared block order of one projection's codes [E, rows, K*bits/32]
    (int32 or uint32, on the GPU): a new int32 tensor of the same shape."""
    torch = _torch()
    dev = packed.device
    _check(packed, "packed", (torch.int32, torch.uint32), dev)
    if packed.dim() != 3:
        raise ValueError("packed must be [E, rows, K*bits/32]")
    E, rows, kw = packed.shape
    K = kw * 32 // bits
    out = torch.empty((E, rows, kw), dtype=torch.int32, device=dev)
    st = moe_wna16_prepare(packed.data_ptr(), E, rows, K, (bits, group), out.data_ptr(),
                           _stream(dev))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_prepare")
    return out


def align(topk_ids, E: int, block_m: int):
    """Expert-sorted tile layout on the GPU; returns a dict of int32 tensors
    (sorted_ids / tile_expert at full capacity; cut them with num_tiles)."""
    torch = _torch()
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", (torch.int32,), dev)
    T = topk_ids.shape[0]
    topk = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    P = T * topk
    cap_tiles = P // block_m + min(E, P)
    z = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    r = dict(sorted_ids=z(cap_tiles * block_m), tile_expert=z(cap_tiles),
             expert_offsets=z(E + 1), inv_perm=z(P), num_tiles=z(1), bad_ids=z(1))
    st = moe_wna16_align(topk_ids.data_ptr(), T, topk, E, block_m, r["sorted_ids"].data_ptr(),
                         r["tile_expert"].data_ptr(), r["expert_offsets"].data_ptr(),
                         r["inv_perm"].data_ptr(), r["num_tiles"].data_ptr(),
                         r["bad_ids"].data_ptr(), _stream(dev))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_align")
    return r


def quantize(w, bits: int, group: int, n_candidates: int = 1, imp=None):
    """Quantize W [rows, K] (bf16, on the GPU) on the GPU.  Returns dict(codes
    int32 [rows, K*bits/32], scales fp16 [rows, K/group], sums float64 [4]:
    sum (w-w')^2, sum w^2, sum imp (w-w')^2, sum imp w^2)."""
    torch = _torch()
    dev = w.device
    _check(w, "w", (torch.bfloat16,), dev)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, K]")
    rows, K = w.shape
    if imp is not None:
        _check(imp, "imp", (torch.float32,), dev)
        if imp.shape != (K,):
            raise ValueError(f"imp must have shape ({K},)")
    codes = torch.empty((rows, K * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((rows, K // group), dtype=torch.float16, device=dev)
    sums = torch.empty(4, dtype=torch.float64, device=dev)
    st = moe_wna16_quantize(w.data_ptr() if rows else None,
                            None if imp is None else imp.data_ptr(), rows, K, (bits, group),
                            n_candidates, codes.data_ptr() if rows else None,
                            scales.data_ptr() if rows else None, sums.data_ptr(), _stream(dev))
    if st != OK:
        raise MoeWna16Error(st, "moe_wna16_quantize")
    return dict(codes=codes, scales=scales, sums=sums)
