"""Python binding of libfa.so (the MI355X fused attention library).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/fa.h``.  PyTorch supplies device memory and
the stream; this module turns tensors into pointers and sizes, calls the C entry
point of the same name, and raises on a non-OK status.  If ``libfa.so`` has not
been built the calls raise -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# FA_LIB_PATH selects another build of the same library (the sanitizer build of the CPU
# tests); by default the one built in-tree.
LIB_PATH = os.environ.get("FA_LIB_PATH") or os.path.join(_PKG, "libfa.so")
# The LDS-poison debug build (see build.py), loaded by its own tests through load_variant().
POISON_LIB_PATH = os.path.join(_PKG, "libfa_poison.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_ALIGN",
    5: "FA_ERR_SCALE", 6: "FA_ERR_DEVICE", 7: "FA_ERR_LAUNCH", 8: "FA_ERR_WORKSPACE", 9: "FA_ERR_SCRATCH",
    10: "FA_ERR_TILE",
}

# Bytes of the static device scratch behind fa_fwd_splitkv_qk_noalloc (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_causal", "fa_fwd_plan", "fa_fwd_splitkv_workspace_bytes", "fa_fwd_splitkv_splits",
           "fa_fwd_splitkv", "fa_fwd_splitkv_qk_workspace_bytes", "fa_fwd_splitkv_qk_splits", "fa_fwd_splitkv_qk",
           "fa_fwd_splitkv_qk_noalloc", "fa_fp8_padded_len", "fa_fp8_scale_blocks", "fa_quantize_fp8", "fa_fwd_fp8",
           "fa_fwd_fp8_causal", "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_causal", "fa_status_str", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class Plan(ctypes.Structure):
    _fields_ = [
        ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("waves", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("grid", ctypes.c_int64),
        ("kv_splits", ctypes.c_int32), ("wave_kv_splits", ctypes.c_int32), ("tail_kv_splits", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once; raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = load_variant(path)
    return _lib


def load_variant(path: str) -> ctypes.CDLL:
    """Load a build of the library at ``path`` with its argument types set (a debug build
    beside the in-tree one); the module's functions keep using ``load()``."""
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build() or "
                                f"python -m online_softmax_attention_fa_amd.build")
    lib = ctypes.CDLL(path)
    P, I64, F, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    fwd_args = [P, P, P, P, P, I64, I64, I64, I64, F, I, P]
    for name in ("fa_fwd", "fa_fwd_causal"):
        getattr(lib, name).argtypes = fwd_args
        getattr(lib, name).restype = I
    lib.fa_fwd_plan.argtypes = [I64, I64, I64, I64, I, I, ctypes.POINTER(Plan)]
    lib.fa_fwd_plan.restype = I
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [I64, I64, I64, I64, I, ctypes.c_int32]
    lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_splits.argtypes = [I64, I64, I64, I64, I]
    lib.fa_fwd_splitkv_splits.restype = ctypes.c_int32
    lib.fa_fwd_splitkv.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, I64, I64, I64, I64, F, I, ctypes.c_int32, P]
    lib.fa_fwd_splitkv.restype = I
    lib.fa_fwd_splitkv_qk_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I, ctypes.c_int32]
    lib.fa_fwd_splitkv_qk_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_qk_splits.argtypes = [I64, I64, I64, I64, I64, I]
    lib.fa_fwd_splitkv_qk_splits.restype = ctypes.c_int32
    lib.fa_fwd_splitkv_qk.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, I64, I64, I64, I64, I64, F, I,
                                      ctypes.c_int32, P]
    lib.fa_fwd_splitkv_qk.restype = I
    lib.fa_fwd_splitkv_qk_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I, ctypes.c_int32, P]
    lib.fa_fwd_splitkv_qk_noalloc.restype = I
    lib.fa_fp8_padded_len.argtypes = [I64]
    lib.fa_fp8_padded_len.restype = I64
    lib.fa_fp8_scale_blocks.argtypes = [I64]
    lib.fa_fp8_scale_blocks.restype = I64
    lib.fa_quantize_fp8.argtypes = [P, P, P, I64, I64, I64, I64, I, ctypes.c_int32, P]
    lib.fa_quantize_fp8.restype = I
    for name in ("fa_fwd_fp8", "fa_fwd_fp8_causal"):
        getattr(lib, name).argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, F, I, P]
        getattr(lib, name).restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    bwd_args = [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, I64, I64, I64, I64, F, I, P]
    for name in ("fa_bwd", "fa_bwd_causal"):
        getattr(lib, name).argtypes = bwd_args
        getattr(lib, name).restype = I
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = I
    return lib


def status_str(status: int) -> str:
    try:
        return load().fa_status_str(status).decode()
    except FileNotFoundError:
        return STATUS.get(status, f"status {status}")


def _check(status: int, where: str):
    if status != 0:
        raise FaError(status, where)


def dtype_code(torch_dtype) -> int:
    import torch

    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if torch_dtype not in codes:
        raise TypeError(f"unsupported dtype {torch_dtype}")
    return codes[torch_dtype]


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_device(t, name, device):
    """Every pointer handed to the library must be device memory on the call's GPU: a host
    pointer would reach the kernels as an unmapped address."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device} (got {t.device})")


def _check_tensor(t, name, device, shape, dtype):
    """Caller-supplied buffer: shape, dtype, contiguity and device, before any C call."""
    _on_device(t, name, device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {dtype} {tuple(shape)}; got {t.dtype} {tuple(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _workspace(workspace, need, device):
    """The caller's workspace (any dtype, contiguous, on the call's device), or a new one."""
    import torch

    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _on_device(workspace, "workspace", device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_qkv(q, k, v):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        _on_device(t, name, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v must share one dtype")


def fa_fwd(q, k, v, o=None, lse=None, scale=None, stream=None, causal=False):
    """O, LSE = attention(q, k, v) through ``fa_fwd`` (or ``fa_fwd_causal``).

    q, k, v: contiguous device tensors [B, H, N, d] (fp32 / fp16 / bf16).
    o, lse: optional preallocated outputs ([B,H,N,d] input dtype, [B,H,N] fp32).
    scale: defaults to 1/sqrt(d).  Returns (o, lse).
    """
    import torch

    lib = load()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor(o, "o", q.device, q.shape, q.dtype)
    _check_tensor(lse, "lse", q.device, (B, H, N), torch.float32)
    fn = lib.fa_fwd_causal if causal else lib.fa_fwd
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                B, H, N, d, float(scale), dtype_code(q.dtype), _stream_handle(stream))
    _check(st, "fa_fwd_causal" if causal else "fa_fwd")
    return o, lse


def fa_fwd_causal(q, k, v, o=None, lse=None, scale=None, stream=None):
    return fa_fwd(q, k, v, o=o, lse=lse, scale=scale, stream=stream, causal=True)


def fa_fwd_splitkv_workspace_bytes(B, H, N, d, dtype, splits=0) -> int:
    """Bytes of device workspace ``fa_fwd_splitkv`` needs for ``splits`` key ranges."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fa_fwd_splitkv_workspace_bytes(B, H, N, d, code, splits))


def fa_fwd_splitkv_splits(B, H, N, d, dtype) -> int:
    """The split count ``fa_fwd_splitkv`` picks for ``splits=0``."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fa_fwd_splitkv_splits(B, H, N, d, code))


def fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, dtype, splits=0) -> int:
    """Workspace bytes of ``fa_fwd_splitkv_qk`` (Nq query rows, Nk keys per head)."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, code, splits))


def fa_fwd_splitkv_qk_splits(B, H, Nq, Nk, d, dtype) -> int:
    """The split count ``fa_fwd_splitkv_qk`` picks for ``splits=0``."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fa_fwd_splitkv_qk_splits(B, H, Nq, Nk, d, code))


def fa_fwd_splitkv(q, k, v, o=None, lse=None, splits=0, workspace=None, scale=None, stream=None):
    """O, LSE = attention(q, k, v) with the key range cut into ``splits`` parts that are
    computed separately and merged by their LSE.  q [B, H, Nq, d]; k, v [B, H, Nk, d]:
    ``fa_fwd_splitkv`` when Nq = Nk, ``fa_fwd_splitkv_qk`` otherwise.  Returns (o, lse)."""
    import torch

    lib = load()
    if q.dim() != 4 or k.dim() != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"k must be [B, H, Nk, d] with q's B, H, d: q {tuple(q.shape)} k {tuple(k.shape)}")
    if k.shape[2] != q.shape[2]:
        return _splitkv_qk(lib, q, k, v, o, lse, splits, workspace, scale, stream)
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(o, "o", q.device, q.shape, q.dtype)
    _check_tensor(lse, "lse", q.device, (B, H, N), torch.float32)
    code = dtype_code(q.dtype)
    need = int(lib.fa_fwd_splitkv_workspace_bytes(B, H, N, d, code, splits))
    workspace = _workspace(workspace, need, q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                workspace.data_ptr(), _nbytes(workspace), B, H, N, d, float(scale), code,
                                int(splits), _stream_handle(stream))
    _check(st, "fa_fwd_splitkv")
    return o, lse


def fa_fp8_padded_len(N) -> int:
    """Key length of the transposed V codes: N rounded up to the fp8 forward's key tile."""
    return int(load().fa_fp8_padded_len(N))


def fa_fp8_scale_blocks(N) -> int:
    """Scale blocks (of 64 rows) per (batch, head)."""
    return int(load().fa_fp8_scale_blocks(N))


def fa_quantize_fp8(x, transpose=False, x8=None, scales=None, stream=None):
    """Block-scaled E4M3 codes of x [B, H, N, d] (bf16 / fp16) through ``fa_quantize_fp8``.

    Returns (codes, scales): codes uint8 [B, H, N, d], or [B, H, d, Np] when ``transpose``;
    scales fp32 [B, H, ceil(N / 64)]."""
    import torch

    lib = load()
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor [B, H, N, d]")
    B, H, N, d = x.shape
    shape = (B, H, d, fa_fp8_padded_len(N)) if transpose else (B, H, N, d)
    x8 = torch.empty(shape, dtype=torch.uint8, device=x.device) if x8 is None else x8
    scales = torch.empty((B, H, fa_fp8_scale_blocks(N)), dtype=torch.float32, device=x.device) if scales is None else scales
    _check_tensor(x8, "x8", x.device, shape, torch.uint8)
    _check_tensor(scales, "scales", x.device, (B, H, fa_fp8_scale_blocks(N)), torch.float32)
    with torch.cuda.device(x.device):
        st = lib.fa_quantize_fp8(x.data_ptr(), x8.data_ptr(), scales.data_ptr(), B, H, N, d,
                                 dtype_code(x.dtype), 1 if transpose else 0, _stream_handle(stream))
    _check(st, "fa_quantize_fp8")
    return x8, scales


def fa_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, o=None, lse=None, scale=None, out_dtype=None, stream=None,
               causal=False):
    """O, LSE of attention on block-scaled E4M3 inputs through ``fa_fwd_fp8`` (or
    ``fa_fwd_fp8_causal`` when ``causal``).

    q8, k8: uint8 [B, H, N, d]; vt8: uint8 [B, H, d, Np]; scales fp32 [B, H, nb].
    O has ``out_dtype`` (default bfloat16).  Returns (o, lse)."""
    import torch

    lib = load()
    name = "fa_fwd_fp8_causal" if causal else "fa_fwd_fp8"
    B, H, N, d = q8.shape
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    nb = fa_fp8_scale_blocks(N)
    if k8.shape != q8.shape or tuple(vt8.shape) != (B, H, d, fa_fp8_padded_len(N)):
        raise ValueError("k8 must match q8; vt8 must be [B, H, d, Np]")
    if not q8.is_cuda:
        raise ValueError("codes must be contiguous uint8 device tensors")
    dev = q8.device
    for arg, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        _check_tensor(t, arg, dev, t.shape, torch.uint8)
    for arg, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(t, arg, dev, (B, H, nb), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=dev) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor(o, "o", dev, (B, H, N, d), out_dtype)
    _check_tensor(lse, "lse", dev, (B, H, N), torch.float32)
    with torch.cuda.device(q8.device):
        st = getattr(lib, name)(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), q_scale.data_ptr(),
                                k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                                float(scale), dtype_code(out_dtype), _stream_handle(stream))
    _check(st, name)
    return o, lse


def _splitkv_qk(lib, q, k, v, o, lse, splits, workspace, scale, stream):
    import torch

    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o, lse = _qk_common(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = dtype_code(q.dtype)
    need = int(lib.fa_fwd_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, code, splits))
    workspace = _workspace(workspace, need, q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv_qk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   workspace.data_ptr(), _nbytes(workspace), B, H, Nq, Nk, d, float(scale), code,
                                   int(splits), _stream_handle(stream))
    _check(st, "fa_fwd_splitkv_qk")
    return o, lse


def _qk_common(q, k, v, o, lse):
    """Checks of a call with Nq query rows and Nk keys per head; returns (o, lse), allocated
    when not given."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"k must be [B, H, Nk, d] with q's B, H, d: q {tuple(q.shape)} k {tuple(k.shape)}")
    B, H, Nq, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous device tensor of q's dtype")
        _on_device(t, name, q.device)
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(o, "o", q.device, q.shape, q.dtype)
    _check_tensor(lse, "lse", q.device, (B, H, Nq), torch.float32)
    return o, lse


def fa_fwd_splitkv_noalloc(q, k, v, o=None, lse=None, splits=0, scale=None, stream=None):
    """``fa_fwd_splitkv_qk_noalloc``: the split-KV forward with its partials in the library's
    static device scratch (no workspace argument, no allocation inside the call).  q
    [B, H, Nq, d]; k, v [B, H, Nk, d].  o and lse are allocated here only when not given;
    pass them for an allocation-free call.  Returns (o, lse)."""
    import torch

    lib = load()
    o, lse = _qk_common(q, k, v, o, lse)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv_qk_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                           B, H, Nq, Nk, d, float(scale), dtype_code(q.dtype), int(splits),
                                           _stream_handle(stream))
    _check(st, "fa_fwd_splitkv_qk_noalloc")
    return o, lse


def fa_bwd_workspace_bytes(B, H, N, d, dtype) -> int:
    """Bytes of device workspace ``fa_bwd`` needs (0 for an invalid or empty shape)."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fa_bwd_workspace_bytes(B, H, N, d, code))


def fa_bwd(q, k, v, o, lse, do, dq=None, dk=None, dv=None, workspace=None, scale=None,
           stream=None, causal=False):
    """dQ, dK, dV of attention through ``fa_bwd`` (or ``fa_bwd_causal``).

    q, k, v, o, do: contiguous device tensors [B, H, N, d] (fp16 / bf16); lse: fp32
    [B, H, N] from the forward with the same scale and masking.  dq, dk, dv: optional
    preallocated outputs; workspace: optional uint8 device tensor of at least
    ``fa_bwd_workspace_bytes`` bytes.  Returns (dq, dk, dv).
    """
    import torch

    lib = load()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    for name, t in (("o", o), ("do", do)):
        _check_tensor(t, name, q.device, q.shape, q.dtype)
    _check_tensor(lse, "lse", q.device, (B, H, N), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(t, name, q.device, q.shape, q.dtype)
    code = dtype_code(q.dtype)
    need = int(lib.fa_bwd_workspace_bytes(B, H, N, d, code))
    workspace = _workspace(workspace, need, q.device)
    fn = lib.fa_bwd_causal if causal else lib.fa_bwd
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), _nbytes(workspace),
                B, H, N, d, float(scale), code, _stream_handle(stream))
    _check(st, "fa_bwd_causal" if causal else "fa_bwd")
    return dq, dk, dv


def fa_bwd_causal(q, k, v, o, lse, do, **kw):
    return fa_bwd(q, k, v, o, lse, do, causal=True, **kw)


def fa_fwd_plan(B, H, N, d, dtype, causal=False) -> dict:
    """The launch plan the library's chooser picks (pure host computation)."""
    lib = load()
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    plan = Plan()
    _check(lib.fa_fwd_plan(B, H, N, d, code, int(bool(causal)), ctypes.byref(plan)), "fa_fwd_plan")
    return plan.as_dict()


def fa_version() -> int:
    return load().fa_version()
