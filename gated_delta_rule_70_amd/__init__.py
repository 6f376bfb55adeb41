"""Channelwise gated delta rule on AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over ``libgdr.so`` (C ABI declared in ``include/gdr.h``).  It only
marshals arguments: PyTorch supplies device memory and the current HIP stream, and every
step of the computation runs in the library's HIP kernels.  There is no CPU fallback:
if the library is missing, the calls raise.

    import torch, gated_delta_rule_70_amd as gdr
    o, ht = gdr.chunk_prefill(q, k, v, g, beta, h0=None, chunk=64)   # prefill, any T >= 1
    o = gdr.decode_step(q1, k1, v1, g1, beta1, state)                  # T == 1, state in place
    o, ht = gdr.fused_recurrent(q, k, v, g, beta, h0=state)          # short calls, T tokens

Layouts (dense, row-major, on the GPU): q, k ``[B,T,HK,dk]`` and v ``[B,T,HV,dv]`` in
bf16 or fp32; g ``[B,T,HV,dk]`` and beta ``[B,T,HV]`` in fp32; states ``[B,HV,dk,dv]``
fp32; o ``[B,T,HV,dv]`` fp32, or bf16 with ``out_dtype=torch.bfloat16`` (or a bf16 ``o``
passed in): every entry point then stores each fp32 output rounded to nearest even.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["decode_step", "fused_recurrent", "chunk_prefill", "chunk_prefill_noalloc", "forward",
           "tree_verify", "chunk_prefill_varlen", "fused_recurrent_varlen", "workspace_bytes_varlen",
           "NOALLOC_SCRATCH_BYTES", "VARLEN_MAX_SEQS",
           "workspace_bytes", "GdrError", "lib", "Dims", "LIB_PATH", "ABI_VERSION",
           "RECURRENT_MAX_T", "TREE_MAX_T", "O_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")
ABI_VERSION = 8
NOALLOC_SCRATCH_BYTES = 64 << 20  # gdr_chunk_prefill_noalloc: the library's per-device scratch
RECURRENT_MAX_T = 8  # gdr_forward: calls of at most this many tokens take the fused recurrence
TREE_MAX_T = 64      # gdr_tree_verify: most nodes per tree
BF16, F32 = 0, 1
G_BF16 = 0x1  # gdr_dims.flags: g stored as bf16
K_L2NORM = 0x2  # keys given raw; the kernels normalise each key row (fused prologue)
G_SOFTPLUS = 0x4  # g given as gate logits a; the kernels use -softplus(a)
G_PER_KEY_HEAD = 0x8  # g is [B,T,HK,dk]: one gate per key head, shared by its value heads
PREP_SPLIT = 0x10  # prefill prep: one workgroup per key head (gram once per GQA group)
PREP_FUSED = 0x20  # prefill prep: one workgroup per value head
O_BF16 = 0x40  # o stored as bf16 (each fp32 output rounded to nearest even)
PREP_SPLIT_MAX_GROUP = 8  # largest HV / HK the split prep serves
VARLEN_MAX_SEQS = 4096  # most sequences in one packed variable-length call


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("HK", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gdr status {status}: {msg}")
        self.status = status


_lib = None
_VP = ctypes.c_void_p


def lib():
    """Load libgdr.so (after torch, so both share one HIP runtime) and bind its symbols."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gated_delta_rule_70_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.gdr_abi_version.restype = ctypes.c_int
    L.gdr_abi_version.argtypes = []
    L.gdr_status_str.restype = ctypes.c_char_p
    L.gdr_status_str.argtypes = [ctypes.c_int]
    L.gdr_decode_step.restype = ctypes.c_int
    L.gdr_decode_step.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9
    L.gdr_fused_recurrent.restype = ctypes.c_int
    L.gdr_fused_recurrent.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9
    L.gdr_tree_verify.restype = ctypes.c_int
    L.gdr_tree_verify.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9
    L.gdr_forward.restype = ctypes.c_int
    L.gdr_forward.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9 + [ctypes.c_size_t, _VP]
    L.gdr_chunk_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.gdr_chunk_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.gdr_chunk_prefill.restype = ctypes.c_int
    L.gdr_chunk_prefill.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9 + [ctypes.c_size_t, _VP]
    L.gdr_chunk_prefill_noalloc.restype = ctypes.c_int
    L.gdr_chunk_prefill_noalloc.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 9
    for name in ("gdr_chunk_prep", "gdr_chunk_carry"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = L.gdr_chunk_prefill.argtypes
    L.gdr_chunk_prefill_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.gdr_chunk_prefill_varlen_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.gdr_chunk_prefill_varlen.restype = ctypes.c_int
    L.gdr_chunk_prefill_varlen.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 10 + [ctypes.c_size_t, _VP]
    L.gdr_fused_recurrent_varlen.restype = ctypes.c_int
    L.gdr_fused_recurrent_varlen.argtypes = [ctypes.POINTER(Dims)] + [_VP] * 10
    if L.gdr_abi_version() != ABI_VERSION:
        raise RuntimeError("libgdr.so ABI version mismatch; rebuild it")
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise GdrError(status, lib().gdr_status_str(status).decode())


def _qkv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else _VP(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _out(o, shape, device, out_dtype):
    """The output tensor: ``o`` if given, else a new one of ``out_dtype``.  Either way fp32
    or bf16 (bf16: every entry point stores each fp32 output rounded to nearest even)."""
    if o is None:
        o = torch.empty(shape, device=device, dtype=out_dtype)
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o must be float32 or bfloat16, got {o.dtype}")
    _need(o, "o")
    return o


def _dims(q, v, chunk, g=None, k_l2norm=False, g_softplus=False, prep="auto") -> Dims:
    """gdr_dims for the call.  The gate layout follows g's shape: [B,T,HK,dk] with HK != HV
    is a gate per key head (so is HK == HV with the split prep forced, where the two layouts
    coincide).  ``prep`` ("auto", "fused", "split") picks the prefill's prep form."""
    B, T, HK, dk = q.shape
    HV, dv = v.shape[2], v.shape[3]
    if prep not in ("auto", "fused", "split"):
        raise ValueError(f"prep must be 'auto', 'fused' or 'split', got {prep!r}")
    flags = G_BF16 if g is not None and g.dtype == torch.bfloat16 else 0
    flags |= (K_L2NORM if k_l2norm else 0) | (G_SOFTPLUS if g_softplus else 0)
    if g is not None and g.shape[2] == HK and (HK != HV or prep == "split"):
        flags |= G_PER_KEY_HEAD
    flags |= {"auto": 0, "fused": PREP_FUSED, "split": PREP_SPLIT}[prep]
    return Dims(B, T, HK, HV, dk, dv, int(chunk), _qkv_dtype(q), flags)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _VP(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _shape_of(t) -> tuple:
    return tuple(t.shape)


def _check_shapes(q, k, v, g, beta, h0=None, o=None, ht=None, parent=None):
    """Every tensor's shape against the dims taken from q and v, on the host, before any
    pointer reaches the library (the C ABI sees no allocation sizes, so a short tensor
    would otherwise be read or written past its end).  Returns (B, T, HK, HV, dk, dv)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B,T,HK,dk], got shape {_shape_of(q)}")
    B, T, HK, dk = _shape_of(q)
    if _shape_of(k) != (B, T, HK, dk):
        raise ValueError(f"k must have q's shape {(B, T, HK, dk)}, got {_shape_of(k)}")
    if v.dim() != 4 or _shape_of(v)[:2] != (B, T):
        raise ValueError(f"v must be [B,T,HV,dv] with B,T = {(B, T)}, got {_shape_of(v)}")
    HV, dv = _shape_of(v)[2], _shape_of(v)[3]
    if HK < 1 or HV % HK:
        raise ValueError(f"value heads ({HV}) must be a multiple of key heads ({HK})")
    # g per value head, or per key head (shared by the key head's value heads)
    g_shape = (B, T, HK, dk) if g is not None and _shape_of(g) == (B, T, HK, dk) else (B, T, HV, dk)
    want = {"g": (g, g_shape), "beta": (beta, (B, T, HV)),
            "h0": (h0, (B, HV, dk, dv)), "o": (o, (B, T, HV, dv)), "ht": (ht, (B, HV, dk, dv)),
            "parent": (parent, (B, T))}
    for name, (t, shape) in want.items():
        if t is not None and _shape_of(t) != shape:
            what = f"{list(shape)} or {[B, T, HK, dk]}" if name == "g" else f"{list(shape)}"
            raise ValueError(f"{name} must be {what}, got {list(_shape_of(t))}")
    return B, T, HK, HV, dk, dv


def _check_inputs(q, k, v, g, beta):
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dt)
    # g is fp32, or bf16 with bf16 q/k/v (the library's I/O-lean input format)
    _need(g, "g", torch.bfloat16 if (g.dtype == torch.bfloat16 and dt == torch.bfloat16) else torch.float32)
    _need(beta, "beta", torch.float32)


def workspace_bytes(B, T, HK, HV, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    d = Dims(B, T, HK, HV, dk, dv, chunk, BF16 if dtype == torch.bfloat16 else F32)
    return int(lib().gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)))


def decode_step(q, k, v, g, beta, state, o=None, out_state=None, stream=None, k_l2norm=False,
                g_softplus=False, out_dtype=torch.float32):
    """One decode step (T == 1).  Updates ``state`` in place unless ``out_state`` is given.

    ``state`` may be None (zero initial state; then ``out_state`` receives the new state if
    given).  Returns ``o`` ``[B,1,HV,dv]`` (fp32, or ``out_dtype``).
    """
    ht = state if out_state is None else out_state
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=state, o=o, ht=ht)
    _check_inputs(q, k, v, g, beta)
    if state is not None:
        _need(state, "state", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    if ht is not None:
        _need(ht, "out_state", torch.float32)
    d = _dims(q, v, 0, g, k_l2norm, g_softplus)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    _check(lib().gdr_decode_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state), _ptr(o), _ptr(ht), _stream(stream)))
    return o


def chunk_prefill(q, k, v, g, beta, h0=None, chunk: int = 64, o=None, ht=None,
                  workspace=None, want_state: bool = True, stream=None, stage: str = "both",
                  k_l2norm=False, g_softplus=False, prep: str = "auto", out_dtype=torch.float32):
    """Chunkwise WY/UT prefill over all T tokens.  Returns ``(o, ht)`` (``ht`` None if not wanted).

    ``workspace`` (optional) is a uint8 GPU tensor of at least ``workspace_bytes(...)``
    bytes; one is allocated if omitted.  ``ht`` may be ``h0`` itself (in-place carry).
    ``stage`` selects "both" (gdr_chunk_prefill), "prep" (gdr_chunk_prep) or "carry"
    (gdr_chunk_carry, which needs a workspace filled by "prep" for the same inputs).
    g is ``[B,T,HV,dk]``, or ``[B,T,HK,dk]`` for a gate shared per key head; ``prep``
    ("auto", "fused", "split") then picks the form of the chunk-parallel stage.
    """
    entry = {"both": "gdr_chunk_prefill", "prep": "gdr_chunk_prep", "carry": "gdr_chunk_carry"}[stage]
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=h0, o=o, ht=ht)
    _check_inputs(q, k, v, g, beta)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(B, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q, v, chunk, g, k_l2norm, g_softplus, prep)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    need = int(lib().gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8)
    _check(getattr(lib(), entry)(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return o, ht


def chunk_prefill_noalloc(q, k, v, g, beta, h0=None, chunk: int = 64, o=None, ht=None,
                          want_state: bool = True, stream=None, k_l2norm=False, g_softplus=False,
                          prep: str = "auto", out_dtype=torch.float32):
    """gdr_chunk_prefill_noalloc: the chunked prefill with the library's own per-device
    scratch as workspace (no device allocation inside the call; pass ``o`` and ``ht`` to
    allocate nothing here either).  Returns ``(o, ht)``.  Calls needing more than
    ``NOALLOC_SCRATCH_BYTES`` of workspace raise GdrError (status GDR_ERR_SCRATCH)."""
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=h0, o=o, ht=ht)
    _check_inputs(q, k, v, g, beta)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(B, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q, v, chunk, g, k_l2norm, g_softplus, prep)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    _check(lib().gdr_chunk_prefill_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _stream(stream)))
    return o, ht


def fused_recurrent(q, k, v, g, beta, h0=None, o=None, ht=None, want_state: bool = True,
                    stream=None, k_l2norm=False, g_softplus=False, out_dtype=torch.float32):
    """The token recurrence over all T tokens in one launch (gdr_fused_recurrent): the state
    stays on chip for the whole call.  Returns ``(o, ht)``; ``ht`` may be ``h0`` itself
    (in-place), and is None if not wanted."""
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=h0, o=o, ht=ht)
    _check_inputs(q, k, v, g, beta)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(B, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q, v, 0, g, k_l2norm, g_softplus)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    _check(lib().gdr_fused_recurrent(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _stream(stream)))
    return o, ht


def forward(q, k, v, g, beta, h0=None, chunk: int = 64, o=None, ht=None, workspace=None,
            want_state: bool = True, stream=None, k_l2norm=False, g_softplus=False, prep: str = "auto",
            out_dtype=torch.float32):
    """Routed call (gdr_forward): the fused recurrence for T <= RECURRENT_MAX_T, the chunked
    prefill otherwise.  Returns ``(o, ht)``."""
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=h0, o=o, ht=ht)
    _check_inputs(q, k, v, g, beta)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(B, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q, v, chunk, g, k_l2norm, g_softplus, prep)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    if T > RECURRENT_MAX_T and workspace is None:
        need = int(lib().gdr_chunk_prefill_workspace_bytes(ctypes.byref(d)))
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check(lib().gdr_forward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(h0), _ptr(o), _ptr(ht), _ptr(workspace),
                             ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                             _stream(stream)))
    return o, ht


def workspace_bytes_varlen(N, T, HK, HV, dk, dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Workspace of a packed prefill of N sequences in T rows (any split of the rows)."""
    d = Dims(N, T, HK, HV, dk, dv, chunk, BF16 if dtype == torch.bfloat16 else F32)
    return int(lib().gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d)))


def _packed(q, k, v, g, beta, cu_seqlens, h0, o, ht):
    """Shapes of a packed batch: token tensors [T, H, d] (or with a leading 1), cu_seqlens
    [N+1] int32, states [N, HV, dk, dv].  Returns 4-D views of the token tensors, the o
    shape in the caller's rank, and (N, T, HK, HV, dk, dv)."""
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[0] != 1):
        raise ValueError(f"q must be [T,HK,dk] (or [1,T,HK,dk]) for a packed batch, got {_shape_of(q)}")
    lead = q.dim() == 4

    def as4(t, name, r):
        if t is None:
            return None
        if t.dim() == r + (1 if lead else 0) and (not lead or t.shape[0] == 1):
            return t if lead else t.unsqueeze(0)
        raise ValueError(f"{name} must have q's leading layout, got {_shape_of(t)}")

    q4, k4, v4, g4 = (as4(t, n, 3) for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g")))
    b4 = as4(beta, "beta", 2)
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise ValueError(f"cu_seqlens must be [N+1] with N >= 1, got {_shape_of(cu_seqlens)}")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError(f"cu_seqlens must be int32, got {cu_seqlens.dtype}")
    N = cu_seqlens.shape[0] - 1
    _, T, HK, HV, dk, dv = _check_shapes(q4, k4, v4, g4, b4, o=as4(o, "o", 3))
    for name, t in (("h0", h0), ("ht", ht)):
        if t is not None and _shape_of(t) != (N, HV, dk, dv):
            raise ValueError(f"{name} must be {[N, HV, dk, dv]}, got {list(_shape_of(t))}")
    o_shape = (1, T, HV, dv) if lead else (T, HV, dv)
    return q4, k4, v4, g4, b4, o_shape, (N, T, HK, HV, dk, dv)


def chunk_prefill_varlen(q, k, v, g, beta, cu_seqlens, h0=None, chunk: int = 64, o=None, ht=None,
                         workspace=None, want_state: bool = True, stream=None, k_l2norm=False,
                         g_softplus=False, prep: str = "auto", out_dtype=torch.float32):
    """Chunked prefill of a packed batch (gdr_chunk_prefill_varlen): N sequences laid end
    to end in T rows, sequence i on rows ``[cu_seqlens[i], cu_seqlens[i+1])`` (an int32 GPU
    tensor), each run from its own ``h0[i]``.  Token tensors are ``[T, H, d]`` (or with a
    leading 1); states ``[N, HV, dk, dv]``.  Returns ``(o, ht)``."""
    q4, k4, v4, g4, b4, o_shape, (N, T, HK, HV, dk, dv) = _packed(q, k, v, g, beta, cu_seqlens, h0, o, ht)
    _check_inputs(q4, k4, v4, g4, b4)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, o_shape, q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(N, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q4, v4, chunk, g4, k_l2norm, g_softplus, prep)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    d.B = N
    need = int(lib().gdr_chunk_prefill_varlen_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8)
    _check(lib().gdr_chunk_prefill_varlen(ctypes.byref(d), _ptr(cu_seqlens), _ptr(q4), _ptr(k4), _ptr(v4),
                                          _ptr(g4), _ptr(b4), _ptr(h0), _ptr(o), _ptr(ht), _ptr(workspace),
                                          ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return o, ht


def fused_recurrent_varlen(q, k, v, g, beta, cu_seqlens, h0=None, o=None, ht=None, want_state: bool = True,
                           stream=None, k_l2norm=False, g_softplus=False, out_dtype=torch.float32):
    """The fused token recurrence over a packed batch (gdr_fused_recurrent_varlen); layouts
    as for :func:`chunk_prefill_varlen`.  Returns ``(o, ht)``."""
    q4, k4, v4, g4, b4, o_shape, (N, T, HK, HV, dk, dv) = _packed(q, k, v, g, beta, cu_seqlens, h0, o, ht)
    _check_inputs(q4, k4, v4, g4, b4)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, o_shape, q.device, out_dtype)
    if ht is None and want_state:
        ht = torch.empty(N, HV, dk, dv, device=q.device, dtype=torch.float32)
    if ht is not None:
        _need(ht, "ht", torch.float32)
    d = _dims(q4, v4, 0, g4, k_l2norm, g_softplus)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    d.B = N
    _check(lib().gdr_fused_recurrent_varlen(ctypes.byref(d), _ptr(cu_seqlens), _ptr(q4), _ptr(k4), _ptr(v4),
                                            _ptr(g4), _ptr(b4), _ptr(h0), _ptr(o), _ptr(ht), _stream(stream)))
    return o, ht


def tree_verify(q, k, v, g, beta, parent, h0=None, o=None, stream=None, k_l2norm=False,
                g_softplus=False, out_dtype=torch.float32):
    """Tree-verify solve (gdr_tree_verify): ``parent`` is an int32 GPU tensor ``[B,T]`` of
    parent node indices (-1: continues from ``h0``).  Returns ``o`` ``[B,T,HV,dv]``, each
    node's output along its root path."""
    B, T, HK, HV, dk, dv = _check_shapes(q, k, v, g, beta, h0=h0, o=o, parent=parent)
    _check_inputs(q, k, v, g, beta)
    _need(parent, "parent", torch.int32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    o = _out(o, (B, T, HV, dv), q.device, out_dtype)
    d = _dims(q, v, 0, g, k_l2norm, g_softplus)
    d.flags |= O_BF16 if o.dtype == torch.bfloat16 else 0
    _check(lib().gdr_tree_verify(ctypes.byref(d), _ptr(parent), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(h0), _ptr(o), _stream(stream)))
    return o
