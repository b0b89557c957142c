"""CPU oracle for block-sparse, head-masked self-attention — TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``head_masked_attention_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, float64, OpenMP over rows and
heads); this module only builds it with gcc and marshals numpy arrays.  Each
wrapper names the passage of the reference pages its C function follows.
Inputs are the exact values the GPU sees, upcast to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Token kinds, in the oracle's own numbering.
KINDS = {"text": 0, "conditioning": 1, "audio": 2, "other": 3,
         "image": 4, "video": 5, "padding": 6}
SPARSE, PINNED, DROPPED = 0, 1, 2

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           SRC, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    p = ctypes.c_void_p
    lib.orc_block_classes.argtypes = [ctypes.c_int, p, p, i64, i32, p]
    lib.orc_block_classes.restype = ctypes.c_int
    lib.orc_budget.argtypes = [i64, dbl, ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.orc_budget.restype = None
    lib.orc_select.argtypes = [p, p, i64, i64, i64, i64, i64, i32, p, dbl, i32, p, p]
    lib.orc_select.restype = ctypes.c_int
    lib.orc_radial.argtypes = [i64, i32, p, dbl, i32, p]
    lib.orc_radial.restype = ctypes.c_int
    lib.orc_attention_rows.argtypes = [p, p, p, i64, i64, i64, i64, i64, i32, p, i64, i64, p,
                                       dbl, i64, p, p, p, p, p]
    lib.orc_attention_rows.restype = ctypes.c_int
    lib.orc_head_mask.argtypes = [p, i64, dbl, i64, p]
    lib.orc_head_mask.restype = ctypes.c_int
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = dbl
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_decode_array.argtypes = [p, i64, p]
    lib.orc_e4m3_decode_array.restype = None
    lib.orc_quantize_e4m3.argtypes = [p, i64, i64, i64, i64, p, p]
    lib.orc_quantize_e4m3.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):            # a torch tensor: exact upcast on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def classes(segments, N: int, block: int) -> np.ndarray:
    """Block classes (SD.Next layout paragraph).  segments: [(kind, length)]."""
    kinds = np.array([KINDS[k] for k, _ in segments], dtype=np.int32)
    lens = np.array([n for _, n in segments], dtype=np.int64)
    out = np.empty(N // block, dtype=np.uint8)
    rc = _load().orc_block_classes(len(segments), _ptr(kinds), _ptr(lens), N, block, _ptr(out))
    if rc != 0:
        raise ValueError("segment lengths do not sum to N")
    return out


def budget(n_cand: int, b: float):
    """(k, is_dense) for a budget over n_cand candidates (SD.Next selector paragraph)."""
    k = ctypes.c_int64()
    d = ctypes.c_int32()
    _load().orc_budget(n_cand, float(b), ctypes.byref(k), ctypes.byref(d))
    return int(k.value), bool(d.value)


def select(q, k, block: int, segments, b: float, window_tokens: int = 0):
    """Content-aware selection (SD.Next selector + layout paragraphs).

    q [B,H,N,D], k [B,Hkv,N,D] -> (mask uint8 [B,H,NB,NB], near_tie uint8 [B,H,NB]).
    """
    q = _f64(q)
    k = _f64(k)
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    cls = classes(segments, N, block)
    NB = N // block
    mask = np.zeros((B, H, NB, NB), dtype=np.uint8)
    tie = np.zeros((B, H, NB), dtype=np.uint8)
    rc = _load().orc_select(_ptr(q), _ptr(k), B, H, Hkv, N, D, block, _ptr(cls), float(b),
                            int(window_tokens), _ptr(mask), _ptr(tie))
    if rc != 0:
        raise ValueError("bad select arguments")
    return mask, tie


def radial(N: int, block: int, segments, density: float, window_tokens: int = 0) -> np.ndarray:
    """Radial band control (SD.Next radial-control paragraph) -> uint8 [NB, NB]."""
    cls = classes(segments, N, block)
    NB = N // block
    mask = np.zeros((NB, NB), dtype=np.uint8)
    _load().orc_radial(NB, block, _ptr(cls), float(density), int(window_tokens), _ptr(mask))
    return mask


def attention(q, k, v, block: int, mask, head_mask=None, scale: float | None = None,
              rows=None, key_mask=None) -> np.ndarray:
    """Attention under an explicit -inf block mask (SD.Next flex-consumer paragraph).

    q [B,H,N,D]; k, v [B,Hkv,N,D]; mask uint8 [mB,mH,NB,NB] (mB in {1,B}, mH in
    {1,H}) or [NB,NB] (shared).  head_mask uint8 [H] or None.  rows: None for
    every row (returns [B,H,N,D]) or an int array [R,3] of (b, h, t) triples
    (returns [R,D]).  key_mask: None or uint8 [B,N] (or [N], shared by the
    batch): keys where it is 0 are -inf too (SD.Next sparse-stage paragraph,
    token mask composed with the block mask).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    if m.ndim == 2:
        m = m[None, None]
    mB, mH = m.shape[0], m.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    hm = None if head_mask is None else np.ascontiguousarray(head_mask, dtype=np.uint8)
    if rows is None:
        bb, hh, tt = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
        rows_arr = np.stack([bb.ravel(), hh.ravel(), tt.ravel()], axis=1)
    else:
        rows_arr = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    rb = np.ascontiguousarray(rows_arr[:, 0], dtype=np.int64)
    rh = np.ascontiguousarray(rows_arr[:, 1], dtype=np.int64)
    rt = np.ascontiguousarray(rows_arr[:, 2], dtype=np.int64)
    R = rows_arr.shape[0]
    km = None
    if key_mask is not None:
        km = np.ascontiguousarray(np.broadcast_to(np.asarray(key_mask, dtype=np.uint8), (B, N)))
    out = np.zeros((R, D), dtype=np.float64)
    rc = _load().orc_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, N, D, block, _ptr(m),
                                    mB, mH, None if hm is None else _ptr(hm), float(scale), R,
                                    _ptr(rb), _ptr(rh), _ptr(rt), _ptr(out),
                                    None if km is None else _ptr(km))
    if rc != 0:
        raise ValueError("bad attention arguments")
    if rows is None:
        return out.reshape(B, H, N, D)
    return out


def head_mask(importance, sparsity: float = 0.5, min_active: int = 4) -> np.ndarray:
    """Per-layer head mask (haagenti_sparse AttentionMask/MaskBuilder rule) -> uint8 [H]."""
    imp = np.ascontiguousarray(importance, dtype=np.float64)
    out = np.zeros(imp.shape[0], dtype=np.uint8)
    _load().orc_head_mask(_ptr(imp), imp.shape[0], float(sparsity), int(min_active), _ptr(out))
    return out


# ---- 8-bit float E4M3 (quantized consumer) --------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (uint8 array) as float64; NaN for the NaN codes."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code of a float32 value, ties to the even code."""
    return int(_load().orc_e4m3_encode(float(np.float32(x))))


def quantize_e4m3(x):
    """Per-(b, head) quantisation of x [B,H,N,D] -> (codes uint8 [B,H,N,D], scale float32 [B,H])."""
    x = _f64(x)
    B, H, N, D = x.shape
    codes = np.empty((B, H, N, D), dtype=np.uint8)
    scale = np.empty((B, H), dtype=np.float32)
    _load().orc_quantize_e4m3(_ptr(x), B, H, N, D, _ptr(codes), _ptr(scale))
    return codes, scale


def dequantize_e4m3(codes, scale) -> np.ndarray:
    """codes [B,H,N,D] times their (b, head) scale, in float64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, :, None, None]
