"""Thin Python binding over libfa.so, the gfx950 exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind
the C ABI declared in include/fa.h. PyTorch supplies device memory and the stream.
There is no CPU or PyTorch fallback: if libfa.so is missing, or a tensor is not on the
GPU, the call raises.

Raw entry points with the C names (``fa_forward``, ``fa_forward_splitkv``, ``fa_backward``,
``fa_forward_ex``, ``fa_backward_ex``, ``fa_status_string``, ...)
take torch tensors in the documented layouts and return nothing (they raise
``FAError`` on a non-zero status). ``attention_forward`` / ``attention_backward`` allocate
the outputs with torch and call them; ``flash_attention`` (contiguous (B, H, N, d)),
``flash_attn_func`` ((B, N, H, d) tensors or views with contiguous rows) and
``flash_attn_varlen_func`` (packed (total, H, d) with ``cu_seqlens``) wrap them for autograd
(the forward saves Q, K, V, O and LSE only -- "Triton 05: Flash Attention", section
"torch.autograd.Function 래핑").
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_FP16 = 0
FA_BF16 = 1
FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3

EXPORTED_SYMBOLS = ("fa_forward", "fa_forward_pingpong", "fa_forward_splitkv", "fa_forward_splitkv_workspace_bytes", "fa_backward",
                    "fa_backward_preprocess", "fa_backward_dkv", "fa_backward_dq", "fa_backward_dq_delta", "fa_forward_ex", "fa_backward_ex",
                    "fa_forward_splitkv_ex", "fa_forward_splitkv_ex_workspace_bytes", "fa_backward_noalloc",
                    "fa_backward_noalloc_max_rows", "fa_status_string")


class FAStrides(ctypes.Structure):
    """fa_strides: element strides (batch, head, row) of one operand; the head dim is contiguous."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


class FAProblem(ctypes.Structure):
    """fa_problem: shape, optional device cu_seqlens (variable lengths), mask, scale, dtype, and
    the key side's length bound / offsets / row count when they differ from the queries'."""
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
                ("cu_seqlens", ctypes.c_void_p), ("total", ctypes.c_int), ("causal", ctypes.c_int),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("N_k", ctypes.c_int),
                ("cu_seqlens_k", ctypes.c_void_p), ("total_k", ctypes.c_int)]

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def load_library() -> ctypes.CDLL:
    """Load libfa.so once. Raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_27_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_pingpong.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_forward_pingpong.restype = i
    lib.fa_forward_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
    lib.fa_forward_splitkv.restype = i
    lib.fa_forward_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_forward_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.fa_backward_preprocess.restype = i
    lib.fa_backward_dkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_backward_dkv.restype = i
    lib.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_backward_dq.restype = i
    lib.fa_backward_dq_delta.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_backward_dq_delta.restype = i
    S, P = FAStrides, ctypes.POINTER(FAProblem)
    lib.fa_forward_ex.argtypes = [P, vp, S, vp, S, vp, S, vp, S, vp, vp]
    lib.fa_forward_ex.restype = i
    lib.fa_backward_ex.argtypes = [P, vp, S, vp, S, vp, S, vp, S, vp, S, vp, vp, S, vp, S, vp, S, vp, vp]
    lib.fa_backward_ex.restype = i
    lib.fa_forward_splitkv_ex.argtypes = [P, vp, S, vp, S, vp, S, vp, S, vp, i, vp, ctypes.c_size_t, vp]
    lib.fa_forward_splitkv_ex.restype = i
    lib.fa_forward_splitkv_ex_workspace_bytes.argtypes = [P, i]
    lib.fa_forward_splitkv_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_noalloc_max_rows.argtypes = []
    lib.fa_backward_noalloc_max_rows.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


# ------------------------------------------------------------------------- marshalling

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: fp16 or bf16 only")


def _check_bhnd(name, t, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (B, H, N, d)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ValueError(f"the stream is on {stream.device}, the operands on {device}: all must share one GPU")
    return ctypes.c_void_p(stream.cuda_stream)


def _one_device(device, **tensors):
    """Every given tensor (None skipped) must live on `device`: a kernel reads and writes all
    its operands from one GPU."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the operands on {device}: all must share one GPU")


def _invoke(entry, device, *args):
    """Call a C entry point with `device` current (the library's launch-shape choices query
    the current device; the kernels run on the stream's)."""
    import torch
    with torch.cuda.device(device):
        return getattr(load_library(), entry)(*args)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def fa_forward(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """Forward: q, k, v, o (B,H,N,d) fp16/bf16; lse (B,H,N) float32 or None."""
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, q.shape, q.dtype)
    if lse is not None:
        _check_bhnd("lse", lse, (B, H, N), torch.float32)
    _one_device(q.device, k=k, v=v, o=o, lse=lse)
    st = _invoke("fa_forward", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                 float(scale), _dtype_code(q), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_forward")


def fa_forward_pingpong(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """fa_forward with the two-group ping-pong schedule (bit-identical outputs; arguments as fa_forward)."""
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, q.shape, q.dtype)
    if lse is not None:
        _check_bhnd("lse", lse, (B, H, N), torch.float32)
    _one_device(q.device, k=k, v=v, o=o, lse=lse)
    st = _invoke("fa_forward_pingpong", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                 int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_forward_pingpong")


def fa_forward_splitkv_workspace_bytes(B: int, H: int, N: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_forward_splitkv_workspace_bytes(B, H, N, d, num_splits))


def fa_forward_splitkv(q, k, v, o, lse, causal: bool, scale: float, num_splits: int, workspace=None,
                       stream=None) -> None:
    """Split-KV forward (same o / lse contract as fa_forward). `workspace` is a float32 GPU tensor
    of at least fa_forward_splitkv_workspace_bytes(...) bytes; None allocates one with torch."""
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, q.shape, q.dtype)
    if lse is not None:
        _check_bhnd("lse", lse, (B, H, N), torch.float32)
    need = fa_forward_splitkv_workspace_bytes(B, H, N, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q.device)
    if not workspace.is_cuda or workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 GPU tensor")
    _one_device(q.device, k=k, v=v, o=o, lse=lse, workspace=workspace)
    st = _invoke("fa_forward_splitkv", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                 int(bool(causal)), float(scale), _dtype_code(q), int(num_splits), _ptr(workspace),
                 workspace.numel() * 4, _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_forward_splitkv")


def fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, causal: bool, scale: float, stream=None) -> None:
    """Backward: all (B,H,N,d) tensors fp16/bf16; lse, delta (B,H,N) float32."""
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, q.shape, q.dtype)
    for name, t in (("lse", lse), ("delta", delta)):
        _check_bhnd(name, t, (B, H, N), torch.float32)
    _one_device(q.device, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    st = _invoke("fa_backward", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                 _ptr(dv), _ptr(delta), B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q),
                 _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward")


def fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal: bool, scale: float, stream=None) -> None:
    """fa_backward without the delta workspace: the library keeps it in a device array of
    fa_backward_noalloc_max_rows() rows per GPU, so the call allocates nothing. Calls that
    overlap in time on one GPU share that array and must not run concurrently."""
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    _one_device(q.device, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
    st = _invoke("fa_backward_noalloc", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                 _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q),
                 _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_noalloc")


def fa_backward_noalloc_max_rows() -> int:
    """Most B*H*N rows fa_backward_noalloc accepts (the size of its device array)."""
    return int(load_library().fa_backward_noalloc_max_rows())


def fa_backward_preprocess(o, do, delta, stream=None) -> None:
    """Backward stage 1: delta = rowsum(dO * O)."""
    import torch
    _check_bhnd("o", o)
    B, H, N, d = o.shape
    _check_bhnd("do", do, o.shape, o.dtype)
    _check_bhnd("delta", delta, (B, H, N), torch.float32)
    _one_device(o.device, do=do, delta=delta)
    st = _invoke("fa_backward_preprocess", o.device, _ptr(o), _ptr(do), _ptr(delta), B, H, N, d, _dtype_code(o),
                 _stream_handle(stream, o.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_preprocess")


def _check_stage(q, k, v, do, lse, delta, outs):
    import torch
    _check_bhnd("q", q)
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("do", do)) + tuple(outs):
        _check_bhnd(name, t, q.shape, q.dtype)
    for name, t in (("lse", lse), ("delta", delta)):
        _check_bhnd(name, t, (B, H, N), torch.float32)
    return B, H, N, d


def fa_backward_dkv(q, k, v, do, lse, delta, dk, dv, causal: bool, scale: float, stream=None) -> None:
    """Backward stage 2: dK, dV (K/V tile pinned per workgroup)."""
    B, H, N, d = _check_stage(q, k, v, do, lse, delta, (("dk", dk), ("dv", dv)))
    _one_device(q.device, k=k, v=v, do=do, lse=lse, delta=delta, dk=dk, dv=dv)
    st = _invoke("fa_backward_dkv", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dk),
                 _ptr(dv), B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q),
                 _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_dkv")


def fa_backward_dq(q, k, v, do, lse, delta, dq, causal: bool, scale: float, stream=None) -> None:
    """Backward stage 3: dQ (Q tile pinned per workgroup)."""
    B, H, N, d = _check_stage(q, k, v, do, lse, delta, (("dq", dq),))
    _one_device(q.device, k=k, v=v, do=do, lse=lse, delta=delta, dq=dq)
    st = _invoke("fa_backward_dq", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dq),
                 B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_dq")


def fa_backward_dq_delta(q, k, v, o, do, lse, dq, delta, causal: bool, scale: float, stream=None) -> None:
    """Backward stages 1 and 3 in one launch: dQ, with D computed from o and dO and written to delta."""
    B, H, N, d = _check_stage(q, k, v, do, lse, delta, (("dq", dq), ("o", o)))
    _one_device(q.device, k=k, v=v, o=o, do=do, lse=lse, delta=delta, dq=dq)
    st = _invoke("fa_backward_dq_delta", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                 _ptr(dq), _ptr(delta), B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q),
                 _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_dq_delta")


def attention_forward(q, k, v, causal: bool, scale: float | None = None, stream=None):
    """Allocate O and LSE with torch and run fa_forward. Returns (o, lse)."""
    import torch
    if scale is None:
        scale = q.shape[-1] ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_forward(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def attention_backward(q, k, v, o, do, lse, causal: bool, scale: float | None = None, stream=None):
    """Allocate dQ, dK, dV and the delta workspace with torch and run fa_backward."""
    import torch
    if scale is None:
        scale = q.shape[-1] ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_backward(q, k, v, o, do, lse, dq, dk, dv, delta, causal, scale, stream)
    return dq, dk, dv, delta


_AUTOGRAD = None


def _autograd_function():
    global _AUTOGRAD
    if _AUTOGRAD is not None:
        return _AUTOGRAD
    import torch

    class FlashAttentionFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            o, lse = attention_forward(q, k, v, causal, scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale = causal, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, _ = attention_backward(q, k, v, o, do.contiguous(), lse, ctx.causal, ctx.scale)
            return dq, dk, dv, None, None

    _AUTOGRAD = FlashAttentionFunction
    return FlashAttentionFunction


def flash_attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Differentiable exact attention on (B, H, N, d) GPU tensors."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _autograd_function().apply(q, k, v, causal, scale)


# ------------------------------------------------- strided operands and variable lengths

LAYOUTS = ("bhnd", "bnhd")


def _ex_operand(name, t, shape, dtype, layout, varlen):
    """fa_strides of a GPU tensor in `layout` ((B,H,N,d), (B,N,H,d), or (total,H,d) packed)."""
    if t is None:
        return FAStrides(0, 0, 0)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    st = t.stride()
    if st[-1] != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")
    if varlen:
        return FAStrides(0, st[1], st[0])
    if layout == "bhnd":
        return FAStrides(st[0], st[1], st[2])
    return FAStrides(st[0], st[2], st[1])


def _check_offsets(name, cu):
    import torch
    if not cu.is_cuda or cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor of B+1 offsets")


def _ex_problem(q, k, layout, cu_seqlens, max_seqlen, causal, scale, cu_seqlens_k=None, max_seqlen_k=None):
    """(problem, query-side shape, key-side shape, statistics shape, varlen) of a strided /
    variable-length call. The key side (k, v, dk, dv) may have another row count than q."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {LAYOUTS}")
    if k is None or k.dim() != q.dim():
        raise ValueError("k must have as many dimensions as q")
    if cu_seqlens is not None:
        if q.dim() != 3:
            raise ValueError("with cu_seqlens, q is (total, H, d)")
        _check_offsets("cu_seqlens", cu_seqlens)
        if max_seqlen is None:
            raise ValueError("max_seqlen (the longest sequence) is required with cu_seqlens")
        T, H, d = q.shape
        B = cu_seqlens.numel() - 1
        if cu_seqlens_k is not None:
            _check_offsets("cu_seqlens_k", cu_seqlens_k)
            if cu_seqlens_k.numel() != B + 1:
                raise ValueError("cu_seqlens_k must hold as many offsets as cu_seqlens")
            if max_seqlen_k is None:
                raise ValueError("max_seqlen_k is required with cu_seqlens_k")
            Tk, cuk, nk = k.shape[0], ctypes.c_void_p(cu_seqlens_k.data_ptr()), int(max_seqlen_k)
        else:
            if max_seqlen_k is not None:
                raise ValueError("max_seqlen_k needs cu_seqlens_k")
            Tk, cuk, nk = T, None, 0
        prob = FAProblem(B, H, int(max_seqlen), d, ctypes.c_void_p(cu_seqlens.data_ptr()), T, int(bool(causal)),
                         float(scale), _dtype_code(q), nk, cuk, Tk if cu_seqlens_k is not None else 0)
        return prob, (T, H, d), (Tk, H, d), (H, T), True
    if cu_seqlens_k is not None or max_seqlen_k is not None:
        raise ValueError("cu_seqlens_k / max_seqlen_k need cu_seqlens")
    if q.dim() != 4:
        raise ValueError("q is (B, H, N, d) or (B, N, H, d)")
    if layout == "bhnd":
        B, H, N, d = q.shape
        Nk = k.shape[2]
        kshape = (B, H, Nk, d)
    else:
        B, N, H, d = q.shape
        Nk = k.shape[1]
        kshape = (B, Nk, H, d)
    prob = FAProblem(B, H, N, d, None, 0, int(bool(causal)), float(scale), _dtype_code(q), Nk, None, 0)
    return prob, tuple(q.shape), kshape, (B, H, N), False


def fa_forward_ex(q, k, v, o, lse, causal: bool, scale: float, layout: str = "bnhd", cu_seqlens=None,
                  max_seqlen=None, stream=None, cu_seqlens_k=None, max_seqlen_k=None) -> None:
    """Forward on strided operands: (B,H,N,d) or (B,N,H,d) views whose head dim is contiguous,
    or, with cu_seqlens (int32, B+1 offsets on the GPU), packed (total, H, d) sequences; lse is
    (B, H, N) or, with cu_seqlens, (H, total) float32, or None. k and v may hold another
    number of rows than q (N_k keys; packed: cu_seqlens_k / max_seqlen_k); the causal mask
    then aligns the queries with the last keys."""
    import torch
    prob, qshape, kshape, sshape, varlen = _ex_problem(q, k, layout, cu_seqlens, max_seqlen, causal, scale,
                                                       cu_seqlens_k, max_seqlen_k)
    ops = [_ex_operand(n, t, sh, q.dtype, layout, varlen)
           for n, t, sh in (("q", q, qshape), ("k", k, kshape), ("v", v, kshape), ("o", o, qshape))]
    if lse is not None:
        _check_bhnd("lse", lse, sshape, torch.float32)
    _one_device(q.device, k=k, v=v, o=o, lse=lse, cu_seqlens=cu_seqlens, cu_seqlens_k=cu_seqlens_k)
    st = _invoke("fa_forward_ex", q.device, ctypes.byref(prob), _ptr(q), ops[0], _ptr(k), ops[1], _ptr(v), ops[2],
                 _ptr(o), ops[3], _ptr(lse), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_forward_ex")


def fa_forward_splitkv_ex_workspace_bytes(q, k, num_splits: int, layout: str = "bnhd", cu_seqlens=None,
                                          max_seqlen=None, cu_seqlens_k=None, max_seqlen_k=None) -> int:
    """Workspace bytes fa_forward_splitkv_ex needs for these operands (0 for invalid ones)."""
    prob = _ex_problem(q, k, layout, cu_seqlens, max_seqlen, False, 1.0, cu_seqlens_k, max_seqlen_k)[0]
    return int(load_library().fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(prob), int(num_splits)))


def fa_forward_splitkv_ex(q, k, v, o, lse, causal: bool, scale: float, num_splits: int, workspace=None,
                          layout: str = "bnhd", cu_seqlens=None, max_seqlen=None, stream=None, cu_seqlens_k=None,
                          max_seqlen_k=None) -> None:
    """fa_forward_ex with every Q tile's keys cut into num_splits ranges (decode: one query
    against a long key cache); workspace is a float32 GPU tensor of at least
    fa_forward_splitkv_ex_workspace_bytes bytes (allocated here when None). About 256
    workgroups in all did best on MI355X: num_splits ~ 256 / (B * H * ceil(N / 128))."""
    import torch
    prob, qshape, kshape, sshape, varlen = _ex_problem(q, k, layout, cu_seqlens, max_seqlen, causal, scale,
                                                       cu_seqlens_k, max_seqlen_k)
    ops = [_ex_operand(n, t, sh, q.dtype, layout, varlen)
           for n, t, sh in (("q", q, qshape), ("k", k, kshape), ("v", v, kshape), ("o", o, qshape))]
    if lse is not None:
        _check_bhnd("lse", lse, sshape, torch.float32)
    lib = load_library()
    need = int(lib.fa_forward_splitkv_ex_workspace_bytes(ctypes.byref(prob), int(num_splits)))
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=q.device)
    if not workspace.is_cuda or workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 GPU tensor")
    _one_device(q.device, k=k, v=v, o=o, lse=lse, workspace=workspace, cu_seqlens=cu_seqlens,
                cu_seqlens_k=cu_seqlens_k)
    st = _invoke("fa_forward_splitkv_ex", q.device, ctypes.byref(prob), _ptr(q), ops[0], _ptr(k), ops[1], _ptr(v),
                 ops[2], _ptr(o), ops[3], _ptr(lse), int(num_splits), _ptr(workspace), workspace.numel() * 4,
                 _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_forward_splitkv_ex")


def fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, causal: bool, scale: float, layout: str = "bnhd",
                   cu_seqlens=None, max_seqlen=None, stream=None, cu_seqlens_k=None, max_seqlen_k=None) -> None:
    """Backward on strided operands / packed sequences (same layouts and key-side rules as
    fa_forward_ex); delta is a float32 workspace shaped like lse."""
    import torch
    prob, qshape, kshape, sshape, varlen = _ex_problem(q, k, layout, cu_seqlens, max_seqlen, causal, scale,
                                                       cu_seqlens_k, max_seqlen_k)
    names = (("q", q, qshape), ("k", k, kshape), ("v", v, kshape), ("o", o, qshape), ("do", do, qshape),
             ("dq", dq, qshape), ("dk", dk, kshape), ("dv", dv, kshape))
    ops = [_ex_operand(n, t, sh, q.dtype, layout, varlen) for n, t, sh in names]
    for name, t in (("lse", lse), ("delta", delta)):
        _check_bhnd(name, t, sshape, torch.float32)
    _one_device(q.device, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta, cu_seqlens=cu_seqlens,
                cu_seqlens_k=cu_seqlens_k)
    st = _invoke("fa_backward_ex", q.device, ctypes.byref(prob), _ptr(q), ops[0], _ptr(k), ops[1], _ptr(v), ops[2],
                 _ptr(o), ops[3], _ptr(do), ops[4], _ptr(lse), _ptr(dq), ops[5], _ptr(dk), ops[6], _ptr(dv), ops[7],
                 _ptr(delta), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FAError(st, "fa_backward_ex")


def _row_major(t):
    return t if t.stride(-1) == 1 else t.contiguous()


_AUTOGRAD_EX = None


def _autograd_function_ex():
    global _AUTOGRAD_EX
    if _AUTOGRAD_EX is not None:
        return _AUTOGRAD_EX
    import torch

    class FlashAttentionExFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, cu_seqlens, max_seqlen, cu_seqlens_k, max_seqlen_k):
            q, k, v = _row_major(q), _row_major(k), _row_major(v)
            o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
            if cu_seqlens is None:
                B, N, H, _ = q.shape
                lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
            else:
                lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
            fa_forward_ex(q, k, v, o, lse, causal, scale, "bnhd", cu_seqlens, max_seqlen, None, cu_seqlens_k,
                          max_seqlen_k)
            ctx.save_for_backward(q, k, v, o, lse, cu_seqlens, cu_seqlens_k)
            ctx.causal, ctx.scale, ctx.max_seqlen, ctx.max_seqlen_k = causal, scale, max_seqlen, max_seqlen_k
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse, cu_seqlens, cu_seqlens_k = ctx.saved_tensors
            do = _row_major(do)
            dq, dk, dv = (torch.empty(t.shape, dtype=t.dtype, device=t.device) for t in (q, k, v))
            delta = torch.empty_like(lse)
            fa_backward_ex(q, k, v, o, do, lse, dq, dk, dv, delta, ctx.causal, ctx.scale, "bnhd", cu_seqlens,
                           ctx.max_seqlen, None, cu_seqlens_k, ctx.max_seqlen_k)
            return dq, dk, dv, None, None, None, None, None, None

    _AUTOGRAD_EX = FlashAttentionExFunction
    return FlashAttentionExFunction


def flash_attn_func(q, k, v, causal: bool = False, scale: float | None = None):
    """Differentiable exact attention on (B, N, H, d) GPU tensors (any strides with a
    contiguous head dim, e.g. slices of a packed (B, N, 3, H, d) tensor); k and v may hold
    N_k != N rows (the causal mask then aligns the queries with the last keys)."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _autograd_function_ex().apply(q, k, v, causal, scale, None, None, None, None)


def flash_attn_varlen_func(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
                           cu_seqlens_k=None, max_seqlen_k: int | None = None):
    """Differentiable exact attention over packed variable-length sequences: q, k, v are
    (total, H, d) GPU tensors, sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1] - 1
    (int32 GPU tensor of B+1 offsets), max_seqlen bounds every length. Each sequence attends
    only to itself ("FlashAttentionを1から", section "現場ではこう使う"). With cu_seqlens_k /
    max_seqlen_k the key rows of sequence b are k[cu_seqlens_k[b] : cu_seqlens_k[b+1]]."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    mk = None if max_seqlen_k is None else int(max_seqlen_k)
    return _autograd_function_ex().apply(q, k, v, causal, scale, cu_seqlens, int(max_seqlen), cu_seqlens_k, mk)
