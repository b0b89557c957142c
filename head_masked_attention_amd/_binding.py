"""ctypes binding of libbsattn (argument marshalling only).

Every function has the name of the C entry point it calls (``select`` calls
``bsattn_select`` and so on).  PyTorch supplies device memory and the stream;
all arithmetic runs in the library's HIP kernels.  There is no fallback: if
libbsattn.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsattn.so")

# haagenti_sparse lib.rs: fraction of heads skipped, and the floor on active heads.
DEFAULT_SPARSITY = 0.5
MIN_ACTIVE_HEADS = 4

BF16, F32, FP8_E4M3 = 0, 1, 2
SEG_KINDS = {"text": 0, "conditioning": 1, "audio": 2, "other": 3,
             "image": 4, "video": 5, "padding": 6}
MAX_SEGMENTS = 32
STATUS_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_DTYPE", 3: "ERR_SHAPE", 4: "ERR_STRIDE",
                5: "ERR_LAYOUT", 6: "ERR_BUDGET", 7: "ERR_WORKSPACE", 8: "ERR_HIP",
                9: "ERR_UNSUPPORTED"}


class BsattnError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("D", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class _Segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("length", ctypes.c_int64)]


class _Layout(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("segments", ctypes.POINTER(_Segment)), ("window_tokens", ctypes.c_int32)]


class _BlockMask(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("nqb", ctypes.c_int32),
                ("nkb", ctypes.c_int32), ("mask", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("index", ctypes.c_void_p), ("is_dense", ctypes.c_int32), ("k", ctypes.c_int32)]


EXPORTS = ["bsattn_status_string", "bsattn_layout_classes", "bsattn_budget_k",
           "bsattn_select_workspace_bytes", "bsattn_select", "bsattn_radial", "bsattn_forward",
           "bsattn_forward_masked", "bsattn_quantize_fp8", "bsattn_forward_fp8", "bsattn_forward_fp8_masked",
           "bsattn_head_mask", "bsattn_mask_density", "bsattn_select_forward",
           "bsattn_stage_create", "bsattn_stage_decide", "bsattn_stage_destroy",
           "bsattn_stage_outcome_string", "bsattn_select_no_alloc", "bsattn_select_heads"]

class _StageConfig(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("min_length", ctypes.c_int64), ("n_steps", ctypes.c_int32),
                ("budget_first", ctypes.c_double), ("budget_later", ctypes.c_double),
                ("switch_step", ctypes.c_int32), ("exclude", ctypes.c_char_p),
                ("backend_block_mask", ctypes.c_int32), ("backend_masked_block", ctypes.c_int32)]


class _StageCall(ctypes.Structure):
    _fields_ = [("architecture", ctypes.c_char_p), ("pipeline", ctypes.c_char_p), ("denoiser", ctypes.c_char_p),
                ("self_attention", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("has_token_mask", ctypes.c_int32), ("causal", ctypes.c_int32), ("step", ctypes.c_int32),
                ("has_layout", ctypes.c_int32)]


class _StageDecision(ctypes.Structure):
    _fields_ = [("outcome", ctypes.c_int32), ("note", ctypes.c_int32), ("budget", ctypes.c_double),
                ("use_key_mask", ctypes.c_int32), ("first_report", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbsattn.so (raises if it is missing: no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with head_masked_attention_amd.build.build()")
    # torch ships its own HIP runtime under the same soname: load it first so
    # libbsattn binds to that one and torch's streams are valid in our calls
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.bsattn_status_string.argtypes = [ctypes.c_int]
    lib.bsattn_status_string.restype = ctypes.c_char_p
    lib.bsattn_layout_classes.argtypes = [ctypes.POINTER(_Layout), i64, P, ctypes.POINTER(i32)]
    lib.bsattn_budget_k.argtypes = [i32, dbl, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.bsattn_select_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i64]
    lib.bsattn_select_workspace_bytes.restype = ctypes.c_size_t
    lib.bsattn_select.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                  ctypes.POINTER(_Layout), dbl, ctypes.POINTER(_BlockMask), P,
                                  ctypes.c_size_t, P]
    lib.bsattn_select_heads.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                        ctypes.POINTER(_Layout), dbl, P, ctypes.POINTER(_BlockMask), P,
                                        ctypes.c_size_t, P]
    lib.bsattn_radial.argtypes = [ctypes.POINTER(_Layout), dbl, ctypes.POINTER(_BlockMask), P]
    lib.bsattn_select_no_alloc.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                           ctypes.POINTER(_Layout), dbl, ctypes.POINTER(_BlockMask), P]
    lib.bsattn_select_forward.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                          ctypes.POINTER(_Layout), dbl, P, ctypes.c_float, ctypes.POINTER(_Tensor),
                                          ctypes.POINTER(_BlockMask), P, ctypes.c_size_t, P]
    lib.bsattn_forward.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                   ctypes.POINTER(_Tensor), ctypes.POINTER(_BlockMask), P,
                                   ctypes.c_float, ctypes.POINTER(_Tensor), P]
    lib.bsattn_forward_masked.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                          ctypes.POINTER(_Tensor), ctypes.POINTER(_BlockMask), P, P, i64,
                                          ctypes.c_float, ctypes.POINTER(_Tensor), P]
    lib.bsattn_quantize_fp8.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), P, P, ctypes.c_size_t, P]
    lib.bsattn_forward_fp8.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                       P, P, P, ctypes.POINTER(_BlockMask), P, ctypes.c_float,
                                       ctypes.POINTER(_Tensor), P]
    lib.bsattn_forward_fp8_masked.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
                                              ctypes.POINTER(_Tensor), P, P, P, ctypes.POINTER(_BlockMask), P,
                                              P, i64, ctypes.c_float, ctypes.POINTER(_Tensor), P]
    lib.bsattn_head_mask.argtypes = [P, i32, dbl, i32, P]
    lib.bsattn_mask_density.argtypes = [ctypes.POINTER(_BlockMask), P, ctypes.POINTER(dbl)]
    lib.bsattn_stage_create.argtypes = [ctypes.POINTER(_StageConfig), ctypes.POINTER(P)]
    lib.bsattn_stage_decide.argtypes = [P, ctypes.POINTER(_StageCall), ctypes.POINTER(_StageDecision)]
    lib.bsattn_stage_destroy.argtypes = [P]
    lib.bsattn_stage_outcome_string.argtypes = [i32]
    for name in EXPORTS[1:]:
        if name not in ("bsattn_select_workspace_bytes", "bsattn_stage_destroy", "bsattn_stage_outcome_string"):
            getattr(lib, name).restype = ctypes.c_int
    lib.bsattn_stage_destroy.restype = None
    lib.bsattn_stage_outcome_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().bsattn_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise BsattnError(status, where, status_string(status))


@dataclass
class Layout:
    """Token layout of a packed sequence: ordered (kind, length) segments."""
    block: int = 64
    segments: list = field(default_factory=list)
    window_tokens: int = 0

    def _c(self):
        n = len(self.segments)
        arr = (_Segment * max(n, 1))()
        for i, (kind, length) in enumerate(self.segments):
            arr[i].kind = SEG_KINDS[kind] if isinstance(kind, str) else int(kind)
            arr[i].length = int(length)
        lay = _Layout(self.block, n, ctypes.cast(arr, ctypes.POINTER(_Segment)), self.window_tokens)
        return lay, arr   # keep arr alive with lay


@dataclass
class BlockMask:
    """Block mask in CSR-like form; torch tensors on the device."""
    mask: object      # uint8 [B,H,nqb,nkb]
    count: object     # int32 [B,H,nqb]
    index: object     # int32 [B,H,nqb,nkb], first count entries valid
    is_dense: bool = False
    k: int = 0

    def _c(self):
        B, H, nqb, nkb = self.mask.shape
        return _BlockMask(B, H, nqb, nkb, self.mask.data_ptr(), self.count.data_ptr(),
                          self.index.data_ptr(), int(self.is_dense), int(self.k))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):    # E4M3 codes
        return FP8_E4M3
    raise BsattnError(2, "tensor", f"unsupported dtype {t.dtype}")


def _tensor(t) -> _Tensor:
    if t.dim() != 4:
        raise BsattnError(3, "tensor", "expected a [B,H,N,D] tensor")
    B, H, N, D = t.shape
    sb, sh, sn, sd = t.stride()
    if sd != 1 and D > 1:
        raise BsattnError(4, "tensor", "the D axis must be contiguous")
    return _Tensor(t.data_ptr(), _dtype_code(t), B, H, N, D, sb, sh, sn)


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for allocating a call's temporaries and outputs.

    The caching allocator hands a freed block back out only to work on the
    stream it was allocated on.  Buffers that the library's kernels read or
    write on `stream` are therefore allocated on `stream` itself: a temporary
    (workspace, an internal block mask) dropped on return cannot be reused by
    other work until the kernels queued before it on that stream are done.
    """
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def empty_block_mask(B: int, H: int, nb: int, device) -> BlockMask:
    import torch
    return BlockMask(torch.empty((B, H, nb, nb), dtype=torch.uint8, device=device),
                     torch.empty((B, H, nb), dtype=torch.int32, device=device),
                     torch.empty((B, H, nb, nb), dtype=torch.int32, device=device))


def select_workspace_bytes(B, H, Hkv, N, block, D) -> int:
    return int(load_library().bsattn_select_workspace_bytes(B, H, Hkv, N, block, D))


def select(q, k, layout: Layout, budget: float, *, out: BlockMask | None = None,
           workspace=None, stream=None) -> BlockMask:
    """bsattn_select: content-aware block selection (no host sync)."""
    import torch
    lib = load_library()
    B, H, N, D = q.shape
    nb = N // layout.block
    need = select_workspace_bytes(B, H, k.shape[1], N, layout.block, D)
    with _on(stream):
        if out is None:
            out = empty_block_mask(B, H, nb, q.device)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    tq, tk = _tensor(q), _tensor(k)
    lay, _keep = layout._c()
    bm = out._c()
    st = lib.bsattn_select(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(lay), float(budget),
                           ctypes.byref(bm), workspace.data_ptr(), workspace.numel(),
                           _stream(q.device, stream))
    _check(st, "bsattn_select")
    out.is_dense, out.k = bool(bm.is_dense), int(bm.k)
    return out


def select_heads(q, k, layout: Layout, budget: float, head_mask, *, out: BlockMask | None = None,
                 workspace=None, stream=None) -> BlockMask:
    """bsattn_select_heads: bsattn_select under a head mask (uint8 device
    tensor [H], or None for every head); rows of masked heads come back
    empty and their sums are never pooled."""
    import torch
    lib = load_library()
    B, H, N, D = q.shape
    nb = N // layout.block
    hm = None
    if head_mask is not None:
        if head_mask.dtype != torch.uint8 or not head_mask.is_cuda:
            raise BsattnError(2, "bsattn_select_heads", "head_mask must be a uint8 device tensor")
        if head_mask.numel() != H or not head_mask.is_contiguous():
            raise BsattnError(3, "bsattn_select_heads", "head_mask must hold one byte per query head")
        hm = head_mask.data_ptr()
    need = select_workspace_bytes(B, H, k.shape[1], N, layout.block, D)
    with _on(stream):
        if out is None:
            out = empty_block_mask(B, H, nb, q.device)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    tq, tk = _tensor(q), _tensor(k)
    lay, _keep = layout._c()
    bm = out._c()
    st = lib.bsattn_select_heads(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(lay), float(budget), hm,
                                 ctypes.byref(bm), workspace.data_ptr(), workspace.numel(),
                                 _stream(q.device, stream))
    _check(st, "bsattn_select_heads")
    out.is_dense, out.k = bool(bm.is_dense), int(bm.k)
    return out


def select_no_alloc(q, k, layout: Layout, budget: float, *, out: BlockMask, stream=None) -> BlockMask:
    """bsattn_select_no_alloc: bsattn_select with the library's static
    per-GPU scratch in place of a workspace; `out` is required, so the call
    allocates nothing.  Calls overlapping on one GPU share the scratch."""
    lib = load_library()
    tq, tk = _tensor(q), _tensor(k)
    lay, _keep = layout._c()
    bm = out._c()
    st = lib.bsattn_select_no_alloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(lay), float(budget),
                                    ctypes.byref(bm), _stream(q.device, stream))
    _check(st, "bsattn_select_no_alloc")
    out.is_dense, out.k = bool(bm.is_dense), int(bm.k)
    return out


def select_forward(q, k, v, layout: Layout, budget: float, head_mask=None, scale: float = 0.0, *,
                   out=None, block_mask: BlockMask | None = None, workspace=None, stream=None):
    """bsattn_select_forward: selection and attention in one call (the result
    of select followed by forward).  Returns (out, block_mask)."""
    import torch
    lib = load_library()
    B, H, N, D = q.shape
    nb = N // layout.block
    need = select_workspace_bytes(B, H, k.shape[1], N, layout.block, D)
    with _on(stream):
        if block_mask is None:
            block_mask = empty_block_mask(B, H, nb, q.device)
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    hm_ptr = None
    if head_mask is not None:
        if head_mask.dtype != torch.uint8 or not head_mask.is_cuda or head_mask.numel() != H:
            raise BsattnError(3, "bsattn_select_forward", "head_mask must be a uint8 device tensor of H entries")
        hm_ptr = head_mask.data_ptr()
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    lay, _keep = layout._c()
    bm = block_mask._c()
    st = lib.bsattn_select_forward(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(lay),
                                   float(budget), hm_ptr, float(scale), ctypes.byref(to), ctypes.byref(bm),
                                   workspace.data_ptr(), workspace.numel(), _stream(q.device, stream))
    _check(st, "bsattn_select_forward")
    block_mask.is_dense, block_mask.k = bool(bm.is_dense), int(bm.k)
    return out, block_mask


def radial(layout: Layout, N: int, density: float, *, B: int = 1, H: int = 1, device=None,
           out: BlockMask | None = None, stream=None) -> BlockMask:
    """bsattn_radial: layout-only band control at the selector's density."""
    import torch
    lib = load_library()
    nb = N // layout.block
    if out is None:
        with _on(stream):
            out = empty_block_mask(B, H, nb, device if device is not None else torch.device("cuda"))
    lay, _keep = layout._c()
    bm = out._c()
    st = lib.bsattn_radial(ctypes.byref(lay), float(density), ctypes.byref(bm),
                           _stream(out.mask.device, stream))
    _check(st, "bsattn_radial")
    out.is_dense, out.k = bool(bm.is_dense), int(bm.k)
    return out


def forward(q, k, v, block_mask: BlockMask | None = None, head_mask=None, scale: float = 0.0,
            *, out=None, stream=None, key_mask=None):
    """bsattn_forward: attention over the kept blocks; masked heads give zeros.

    key_mask: optional uint8 device tensor [B, N] (or [N], shared by the
    batch); keys where it is 0 are masked in every row (bsattn_forward_masked).
    """
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    bm = None if block_mask is None else block_mask._c()
    hm = None
    if head_mask is not None:
        if head_mask.dtype != torch.uint8 or not head_mask.is_cuda:
            raise BsattnError(2, "bsattn_forward", "head_mask must be a uint8 device tensor")
        if head_mask.numel() != q.shape[1] or not head_mask.is_contiguous():
            raise BsattnError(3, "bsattn_forward", "head_mask must hold one byte per query head")
        hm = head_mask.data_ptr()
    if key_mask is None:
        st = lib.bsattn_forward(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                None if bm is None else ctypes.byref(bm), hm, float(scale),
                                ctypes.byref(to), _stream(q.device, stream))
        _check(st, "bsattn_forward")
        return out
    km, km_sb = _key_mask_arg(key_mask, q, "bsattn_forward_masked")
    st = lib.bsattn_forward_masked(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                   None if bm is None else ctypes.byref(bm), hm, km, km_sb, float(scale),
                                   ctypes.byref(to), _stream(q.device, stream))
    _check(st, "bsattn_forward_masked")
    return out


def quantize_fp8(x, *, out=None, scale=None, workspace=None, stream=None):
    """bsattn_quantize_fp8: bf16 [B,H,N,D] -> (E4M3 codes uint8 [B,H,N,D], scale float32 [B,H])."""
    import torch
    lib = load_library()
    B, H = x.shape[0], x.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if scale is None:
            scale = torch.empty((B, H), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(B * H, dtype=torch.int32, device=x.device)
    tx, to = _tensor(x), _tensor(out)
    st = lib.bsattn_quantize_fp8(ctypes.byref(tx), ctypes.byref(to), scale.data_ptr(), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(x.device, stream))
    _check(st, "bsattn_quantize_fp8")
    return out, scale


def _key_mask_arg(key_mask, q, where):
    """(pointer, batch stride) of an optional uint8 device key mask [B, N] or [N]."""
    import torch
    if key_mask.dtype != torch.uint8 or not key_mask.is_cuda:
        raise BsattnError(2, where, "key_mask must be a uint8 device tensor")
    if key_mask.shape[-1] != q.shape[2] or key_mask.stride(-1) != 1 or key_mask.dim() not in (1, 2):
        raise BsattnError(3, where, "key_mask must be [B, N] or [N] with unit key stride")
    if key_mask.dim() == 2 and key_mask.shape[0] != q.shape[0]:
        raise BsattnError(3, where, "key_mask batch must match q")
    km_sb = 0 if key_mask.dim() == 1 or key_mask.shape[0] == 1 else key_mask.stride(0)
    return key_mask.data_ptr(), int(km_sb)


def forward_fp8(q8, k8, v8, q_scale, k_scale, v_scale, block_mask: BlockMask | None = None, head_mask=None,
                scale: float = 0.0, *, out=None, stream=None, key_mask=None):
    """bsattn_forward_fp8: attention on E4M3 inputs with per-(b, head) scales; bf16 output.

    key_mask: optional uint8 device tensor [B, N] (or [N]); keys where it is 0
    are masked in every row (bsattn_forward_fp8_masked).
    """
    import torch
    lib = load_library()
    where = "bsattn_forward_fp8" if key_mask is None else "bsattn_forward_fp8_masked"
    if out is None:
        with _on(stream):
            out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    for name, sc, heads in (("q_scale", q_scale, q8.shape[1]), ("k_scale", k_scale, k8.shape[1]),
                            ("v_scale", v_scale, v8.shape[1])):
        if sc.dtype != torch.float32 or not sc.is_cuda or not sc.is_contiguous() or sc.numel() != q8.shape[0] * heads:
            raise BsattnError(3, where, f"{name} must be a contiguous float32 device [B, heads]")
    hm = None
    if head_mask is not None:
        if head_mask.dtype != torch.uint8 or not head_mask.is_cuda or head_mask.numel() != q8.shape[1]:
            raise BsattnError(3, where, "head_mask must hold one byte per query head")
        hm = head_mask.data_ptr()
    tq, tk, tv, to = _tensor(q8), _tensor(k8), _tensor(v8), _tensor(out)
    bm = None if block_mask is None else block_mask._c()
    if key_mask is None:
        st = lib.bsattn_forward_fp8(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), q_scale.data_ptr(),
                                    k_scale.data_ptr(), v_scale.data_ptr(), None if bm is None else ctypes.byref(bm),
                                    hm, float(scale), ctypes.byref(to), _stream(q8.device, stream))
    else:
        km, km_sb = _key_mask_arg(key_mask, q8, where)
        st = lib.bsattn_forward_fp8_masked(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), q_scale.data_ptr(),
                                           k_scale.data_ptr(), v_scale.data_ptr(),
                                           None if bm is None else ctypes.byref(bm), hm, km, km_sb, float(scale),
                                           ctypes.byref(to), _stream(q8.device, stream))
    _check(st, where)
    return out


def head_mask(importance, sparsity: float = DEFAULT_SPARSITY,
              min_active: int = MIN_ACTIVE_HEADS) -> np.ndarray:
    """bsattn_head_mask (host): keep the most important heads of one layer."""
    imp = np.ascontiguousarray(importance, dtype=np.float64)
    out = np.zeros(imp.shape[0], dtype=np.uint8)
    st = load_library().bsattn_head_mask(imp.ctypes.data_as(ctypes.c_void_p), imp.shape[0],
                                         float(sparsity), int(min_active),
                                         out.ctypes.data_as(ctypes.c_void_p))
    _check(st, "bsattn_head_mask")
    return out


def mask_density(block_mask: BlockMask, stream=None) -> float:
    """bsattn_mask_density: kept fraction of tiles (synchronises; off the hot path)."""
    bm = block_mask._c()
    d = ctypes.c_double()
    st = load_library().bsattn_mask_density(ctypes.byref(bm),
                                            _stream(block_mask.count.device, stream),
                                            ctypes.byref(d))
    _check(st, "bsattn_mask_density")
    return float(d.value)


def layout_classes(layout: Layout, N: int):
    """bsattn_layout_classes (host): per-block classes and the candidate count."""
    lay, _keep = layout._c()
    nb = N // layout.block
    cls = np.zeros(max(nb, 1), dtype=np.uint8)
    n = ctypes.c_int32()
    st = load_library().bsattn_layout_classes(ctypes.byref(lay), N,
                                              cls.ctypes.data_as(ctypes.c_void_p),
                                              ctypes.byref(n))
    _check(st, "bsattn_layout_classes")
    return cls[:nb], int(n.value)


def budget_k(n_cand: int, budget: float):
    """bsattn_budget_k (host): (k, is_dense)."""
    k = ctypes.c_int32()
    d = ctypes.c_int32()
    st = load_library().bsattn_budget_k(n_cand, float(budget), ctypes.byref(k), ctypes.byref(d))
    _check(st, "bsattn_budget_k")
    return int(k.value), bool(d.value)


# ---- host stage policy -------------------------------------------------------

STAGE_SPARSE, DECLINE_DISABLED, DECLINE_NO_BACKEND, DECLINE_EXCLUDED, DECLINE_NOT_SELF, \
    DECLINE_SHORT, DECLINE_CAUSAL, DECLINE_TOKEN_MASK = range(8)
NOTE_NONE, NOTE_NO_LAYOUT = 0, 1
DEFAULT_MIN_LENGTH = 8192


class Stage:
    """bsattn_stage_*: the sparse stage's per-call decision (host only).

    schedule: one budget, or (budget_first, budget_later, switch_step) for a
    per-step schedule with two values over n_steps steps.
    """

    def __init__(self, *, enabled=True, min_length=DEFAULT_MIN_LENGTH, n_steps=1, schedule=0.3,
                 exclude="", backend_block_mask=True, backend_masked_block=True):
        if isinstance(schedule, (tuple, list)):
            first, later, switch = schedule
        else:
            first, later, switch = float(schedule), float(schedule), int(n_steps)
        self._exclude = (exclude or "").encode()
        cfg = _StageConfig(int(bool(enabled)), int(min_length), int(n_steps), float(first), float(later),
                           int(switch), self._exclude, int(bool(backend_block_mask)),
                           int(bool(backend_masked_block)))
        self._lib = load_library()
        self._h = ctypes.c_void_p()
        _check(self._lib.bsattn_stage_create(ctypes.byref(cfg), ctypes.byref(self._h)), "bsattn_stage_create")

    def decide(self, q_len, kv_len=None, *, step=0, self_attention=True, has_token_mask=False,
               causal=False, has_layout=True, architecture=None, pipeline=None, denoiser=None) -> dict:
        enc = lambda x: None if x is None else str(x).encode()
        call = _StageCall(enc(architecture), enc(pipeline), enc(denoiser), int(bool(self_attention)),
                          int(q_len), int(q_len if kv_len is None else kv_len), int(bool(has_token_mask)),
                          int(bool(causal)), int(step), int(bool(has_layout)))
        d = _StageDecision()
        _check(self._lib.bsattn_stage_decide(self._h, ctypes.byref(call), ctypes.byref(d)), "bsattn_stage_decide")
        return {"outcome": d.outcome, "note": d.note, "budget": d.budget, "use_key_mask": bool(d.use_key_mask),
                "first_report": bool(d.first_report),
                "reason": self._lib.bsattn_stage_outcome_string(d.outcome).decode()}

    def close(self):
        if self._h:
            self._lib.bsattn_stage_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sparse_attention(q, k, v, stage: Stage, layout: Layout | None = None, *, step: int = 0, head_mask=None,
                     key_mask=None, causal: bool = False, self_attention: bool = True, architecture=None,
                     pipeline=None, denoiser=None, out=None, block_mask: BlockMask | None = None, stream=None):
    """One attention call through the sparse stage (orchestration only).

    Asks the stage whether to serve the call; if it does, runs bsattn_select at
    the step's budget (bsattn_select_heads under a head mask: the masked heads'
    rows of the selection come back empty) and bsattn_forward
    (bsattn_forward_masked when the call carries a token key mask).  A declined self-attention call of a supported
    shape is computed dense by the same kernel (every block kept); a causal
    or cross-attention call returns None for the caller's own attention.
    block_mask: optional caller buffer that receives a served call's
    selection (otherwise a temporary).  Returns (out or None, decision).
    """
    has_layout = layout is not None and len(layout.segments) > 0
    d = stage.decide(q.shape[2], k.shape[2], step=step, self_attention=self_attention,
                     has_token_mask=key_mask is not None, causal=causal, has_layout=has_layout,
                     architecture=architecture, pipeline=pipeline, denoiser=denoiser)
    if d["outcome"] == STAGE_SPARSE:
        lay = layout if layout is not None else Layout(64, [])
        bm = select_heads(q, k, lay, d["budget"], head_mask, out=block_mask, stream=stream)
        out = forward(q, k, v, bm, head_mask, out=out, stream=stream,
                      key_mask=key_mask if d["use_key_mask"] else None)
        return out, d
    if d["outcome"] in (DECLINE_CAUSAL, DECLINE_NOT_SELF) or q.shape[2] % 64 != 0:
        return None, d
    return forward(q, k, v, None, head_mask, out=out, stream=stream, key_mask=key_mask), d
