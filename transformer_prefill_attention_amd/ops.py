"""Python binding of ``libpfa.so`` (declared in ``include/pfa.h``).

Argument marshalling only: shapes, dtypes and devices are checked, output
tensors are allocated with torch when the caller passes none, and the C entry
point of the same name is called with raw device pointers and the current torch
stream.  Every attention call takes its softmax ``scale`` from the caller (the
pages' models pass 1/sqrt(head_dim)); the binding computes nothing of the method.  Every step of the computation runs in the library's HIP kernels; there
is no fallback of any kind -- if the library is missing, every op raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpfa.so")

PRECISION_F32 = 0
PRECISION_BF16 = 1
PRECISION_BF16X3 = 2
PRECISION_F16 = 3
_PRECISIONS = {"f32": PRECISION_F32, "fp32": PRECISION_F32, "float32": PRECISION_F32,
               "bf16": PRECISION_BF16, "bfloat16": PRECISION_BF16, "bf16x3": PRECISION_BF16X3,
               "f16": PRECISION_F16, "fp16": PRECISION_F16, "float16": PRECISION_F16,
               PRECISION_F32: PRECISION_F32, PRECISION_BF16: PRECISION_BF16,
               PRECISION_BF16X3: PRECISION_BF16X3, PRECISION_F16: PRECISION_F16}

# Every symbol include/pfa.h declares.
EXPORTS = ("qknorm_rope", "gqa_prefill_attn", "qk_prep_attn", "pfa_workspace_bytes",
           "gqa_chunk_attn", "qk_prep_chunk_attn", "pfa_chunk_workspace_bytes",
           "pfa_quantize_rows", "gqa_attn_q8", "qk_prep_attn_q8", "pfa_q8_workspace_bytes",
           "pfa_attn_plan", "pfa_attn_units", "gqa_prefill_attn_noalloc",
           "pfa_noalloc_scratch_bytes", "qk_prep_chunk_attn_tiled", "pfa_kv_tiles_bytes",
           "pfa_last_error", "pfa_version")

# pfa_entry values of the plan report
(ENTRY_PREFILL, ENTRY_PREP, ENTRY_CHUNK, ENTRY_CHUNK_PREP, ENTRY_Q8, ENTRY_Q8_PREP,
 ENTRY_CHUNK_TILED) = range(7)
UNIT_FIELDS = ("workgroup", "pass", "item", "sequence", "super_block", "key_chunk", "kv_head",
               "head_chunk", "tile_begin", "tile_end")


class _Plan(ctypes.Structure):
    """pfa_plan of include/pfa.h."""
    _fields_ = [("items", ctypes.c_int), ("rows_per_item", ctypes.c_int),
                ("waves_per_workgroup", ctypes.c_int), ("tile_keys", ctypes.c_int),
                ("key_chunk_tiles", ctypes.c_int), ("max_key_chunks", ctypes.c_int),
                ("paired", ctypes.c_int), ("merge_in_place", ctypes.c_int),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("kernels", ctypes.c_char * 320)]


class PfaError(RuntimeError):
    """A libpfa entry point returned a non-OK status (or the library is missing)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[pfa status {status}] {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded ``libpfa.so``, with argument types declared.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PfaError(-100, f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                             "g.build()'` first (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp_ = ctypes.c_void_p, ctypes.c_void_p
    i32, f32, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.qknorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    L.qknorm_rope.restype = i32
    L.gqa_prefill_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32,
                                   vp, sz, vp]
    L.gqa_prefill_attn.restype = i32
    L.gqa_prefill_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                           i32, i32, vp]
    L.gqa_prefill_attn_noalloc.restype = i32
    L.pfa_noalloc_scratch_bytes.argtypes = []
    L.pfa_noalloc_scratch_bytes.restype = sz
    L.qk_prep_attn.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                               f32, i32, i32, fp_, vp, sz, vp]
    L.qk_prep_attn.restype = i32
    L.pfa_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32]
    L.pfa_workspace_bytes.restype = sz
    L.gqa_chunk_attn.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                 f32, i32, i32, i32, vp, sz, vp]
    L.gqa_chunk_attn.restype = i32
    L.qk_prep_chunk_attn.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, i32,
                                     i32, i32, i32, i32, i32, f32, f32, f32, i32, i32, i32, vp,
                                     sz, vp]
    L.qk_prep_chunk_attn.restype = i32
    L.pfa_chunk_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
    L.pfa_chunk_workspace_bytes.restype = sz
    L.qk_prep_chunk_attn_tiled.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp,
                                           vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32,
                                           i32, i32, i32, vp, sz, vp]
    L.qk_prep_chunk_attn_tiled.restype = i32
    L.pfa_kv_tiles_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.pfa_kv_tiles_bytes.restype = sz
    L.pfa_last_error.restype = ctypes.c_char_p
    i64 = ctypes.c_int64
    L.pfa_quantize_rows.argtypes = [vp, i64, i32, vp, vp, vp, vp]
    L.pfa_quantize_rows.restype = i32
    L.gqa_attn_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                              i32, i32, f32, i32, i32, vp, sz, vp]
    L.gqa_attn_q8.restype = i32
    L.qk_prep_attn_q8.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                  i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, i32, vp, sz,
                                  vp]
    L.qk_prep_attn_q8.restype = i32
    L.pfa_q8_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32]
    L.pfa_q8_workspace_bytes.restype = sz
    plan_args = [i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, sz]
    L.pfa_attn_plan.argtypes = plan_args + [ctypes.POINTER(_Plan)]
    L.pfa_attn_plan.restype = i32
    L.pfa_attn_units.argtypes = plan_args + [vp, i64]
    L.pfa_attn_units.restype = i64
    L.pfa_last_error.argtypes = []
    L.pfa_version.restype = ctypes.c_char_p
    L.pfa_version.argtypes = []
    _lib = L
    return L


def version() -> str:
    return lib().pfa_version().decode()


def _check(status: int):
    if status != 0:
        raise PfaError(status, lib().pfa_last_error().decode())


def _offsets(seq_offsets, T):
    """Host int32 array for the C call (kept alive by the caller), or None."""
    if seq_offsets is None:
        return None, 0, None
    try:
        import torch
        if isinstance(seq_offsets, torch.Tensor):
            seq_offsets = seq_offsets.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    arr = np.ascontiguousarray(np.asarray(seq_offsets), dtype=np.int32)
    return arr, arr.size - 1, arr.ctypes.data_as(ctypes.c_void_p)


def _dev_f32(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _norm_weights(q_norm_w, k_norm_w, head_dim):
    """The QK-norm weights must hold head_dim floats each (the kernels read all of them):
    checked first, before the device and dtype checks of every tensor."""
    import torch
    ws = ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"))
    for t, n in ws:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.numel() != head_dim:
            raise ValueError(f"{n} must have head_dim = {head_dim} elements, got {t.numel()}")
    for t, n in ws:
        _dev_f32(t, n)


def _heads(t, head_dim, name):
    """(T, heads) of a [T, heads*head_dim] or [T, heads, head_dim] tensor."""
    if t.dim() == 3:
        if t.shape[2] != head_dim:
            raise ValueError(f"{name}: last dim {t.shape[2]} != head_dim {head_dim}")
        return t.shape[0], t.shape[1]
    if t.dim() != 2 or t.shape[1] % head_dim:
        raise ValueError(f"{name} must be [T, heads*head_dim] or [T, heads, head_dim]")
    return t.shape[0], t.shape[1] // head_dim


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _prec(precision):
    try:
        return _PRECISIONS[precision]
    except KeyError:
        raise ValueError(f"precision must be 'f32', 'bf16', 'bf16x3' or 'f16', got {precision!r}") from None


def workspace_bytes(T: int, n_head: int, n_head_kv: int, head_dim: int, precision="f32",
                    seq_offsets: Optional[Sequence[int]] = None, fused: bool = False) -> int:
    """Device workspace ``gqa_prefill_attn`` (``fused=False``) or ``qk_prep_attn``
    (``fused=True``) uses for these arguments (``pfa_workspace_bytes``)."""
    offs, n_seqs, op = _offsets(seq_offsets, T)
    return int(lib().pfa_workspace_bytes(op, n_seqs, T, n_head, n_head_kv, head_dim,
                                         _prec(precision), 1 if fused else 0))


def _workspace(workspace, op, n_seqs, T, H, Hkv, head_dim, prec, fused, device):
    """(tensor, pointer, size) of the caller's workspace, or of a new one from torch's allocator."""
    import torch
    need = int(lib().pfa_workspace_bytes(op, n_seqs, T, H, Hkv, head_dim, prec, 1 if fused else 0))
    if need == 0:
        return None, ctypes.c_void_p(0), 0
    if workspace is None:
        # torch's caching allocator hands out 512-byte aligned blocks
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise TypeError("workspace must be a GPU torch.Tensor")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def qknorm_rope(q, k, q_norm_w, k_norm_w, *, head_dim: int, rope_dim: int,
                rope_freq_base: float, rms_eps: float,
                seq_offsets: Optional[Sequence[int]] = None, q_out=None, k_out=None):
    """QK RMSNorm + NeoX RoPE (``qknorm_rope`` in ``include/pfa.h``).

    Returns ``(q_out, k_out)``; pass ``q_out=q, k_out=k`` to work in place."""
    import torch
    _norm_weights(q_norm_w, k_norm_w, head_dim)
    for t, n in ((q, "q"), (k, "k"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _dev_f32(t, n)
    T, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T:
        raise ValueError(f"q has {T} tokens but k has {Tk}")
    q_out = torch.empty_like(q) if q_out is None else _dev_f32(q_out, "q_out")
    k_out = torch.empty_like(k) if k_out is None else _dev_f32(k_out, "k_out")
    if q_out.numel() != q.numel() or k_out.numel() != k.numel():
        raise ValueError("output shapes must match the inputs")
    offs, n_seqs, op = _offsets(seq_offsets, T)
    _check(lib().qknorm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(q_norm_w),
                             _ptr(k_norm_w), op, n_seqs, T, H, Hkv, head_dim, rope_dim,
                             float(rope_freq_base), float(rms_eps), _stream(q)))
    return q_out, k_out


def gqa_prefill_attn(q, k, v, *, head_dim: int, scale: float,
                     causal: bool = True, precision="f32",
                     seq_offsets: Optional[Sequence[int]] = None, out=None, workspace=None):
    """Causal GQA attention (``gqa_prefill_attn`` in ``include/pfa.h``); returns ``out``.

    The bf16 precisions use a device workspace: ``workspace`` (a GPU tensor of at
    least :func:`workspace_bytes` bytes), else one taken from torch's allocator."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_f32(t, n)
    T, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    offs, n_seqs, op = _offsets(seq_offsets, T)
    prec = _prec(precision)
    ws, wp, wn = _workspace(workspace, op, n_seqs, T, H, Hkv, head_dim, prec, False, q.device)
    _check(lib().gqa_prefill_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), op, n_seqs, T, H, Hkv,
                                  head_dim, float(scale), 1 if causal else 0, prec, wp, wn,
                                  _stream(q)))
    return out


def gqa_prefill_attn_noalloc(q, k, v, *, head_dim: int, scale: float, causal: bool = True,
                             precision="f32", seq_offsets: Optional[Sequence[int]] = None,
                             out=None):
    """``gqa_prefill_attn`` with its workspace in the library's own device array
    (``gqa_prefill_attn_noalloc`` in ``include/pfa.h``): the C call allocates nothing.
    Pass ``out`` too when nothing may be allocated; calls overlapping on one GPU race."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_f32(t, n)
    T, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    offs, n_seqs, op = _offsets(seq_offsets, T)
    _check(lib().gqa_prefill_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), op, n_seqs, T,
                                          H, Hkv, head_dim, float(scale), 1 if causal else 0,
                                          _prec(precision), _stream(q)))
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the device array ``gqa_prefill_attn_noalloc`` uses on each GPU."""
    return int(lib().pfa_noalloc_scratch_bytes())


def qk_prep_attn(q, k, v, q_norm_w, k_norm_w, *, head_dim: int, rope_dim: int,
                 rope_freq_base: float, rms_eps: float, scale: float,
                 causal: bool = True, precision="f32",
                 seq_offsets: Optional[Sequence[int]] = None, out=None, k_rot_out=None,
                 workspace=None):
    """Fused QK-norm + RoPE + causal GQA attention (``qk_prep_attn`` in ``include/pfa.h``).

    Returns ``out`` (and also writes ``k_rot_out`` when one is given).  The device
    workspace (``workspace_bytes(..., fused=True)`` bytes) is ``workspace`` or one
    taken from torch's allocator."""
    import torch
    _norm_weights(q_norm_w, k_norm_w, head_dim)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _dev_f32(t, n)
    T, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    if k_rot_out is not None:
        _dev_f32(k_rot_out, "k_rot_out")
        if k_rot_out.numel() != k.numel():
            raise ValueError("k_rot_out must have k's shape")
    offs, n_seqs, op = _offsets(seq_offsets, T)
    prec = _prec(precision)
    ws, wp, wn = _workspace(workspace, op, n_seqs, T, H, Hkv, head_dim, prec, True, q.device)
    _check(lib().qk_prep_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(q_norm_w),
                              _ptr(k_norm_w), op, n_seqs, T, H, Hkv, head_dim, rope_dim,
                              float(rope_freq_base), float(rms_eps), float(scale),
                              1 if causal else 0, prec, _ptr(k_rot_out), wp, wn, _stream(q)))
    return out


def _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv):
    """Host int32 arrays of a chunk call (both or neither), their count and pointers."""
    if (q_offsets is None) != (kv_offsets is None):
        raise ValueError("give both q_offsets and kv_offsets, or neither")
    qo, n_seqs, qp = _offsets(q_offsets, T_q)
    ko, n_kv, kp = _offsets(kv_offsets, T_kv)
    if qo is not None and n_kv != n_seqs:
        raise ValueError("q_offsets and kv_offsets must have the same length")
    return (qo, ko), n_seqs, qp, kp


def chunk_workspace_bytes(T_q: int, T_kv: int, n_head: int, n_head_kv: int, head_dim: int,
                          precision="f32", q_offsets=None, kv_offsets=None,
                          fused=False) -> int:
    """Device workspace ``gqa_chunk_attn`` (``fused=False``), ``qk_prep_chunk_attn``
    (``fused=True``) or ``qk_prep_chunk_attn_tiled`` (``fused=2``) uses for these
    arguments (``pfa_chunk_workspace_bytes``)."""
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    return int(lib().pfa_chunk_workspace_bytes(qp, kp, n_seqs, T_q, T_kv, n_head, n_head_kv,
                                               head_dim, _prec(precision), _fused_code(fused)))


def _fused_code(fused):
    """The size queries' ``fused`` argument: 0, 1, or 2 (the tiled chunk entry)."""
    if fused is True or fused is False:
        return int(fused)
    if fused in (0, 1, 2):
        return int(fused)
    raise ValueError(f"fused must be False, True or 2 (got {fused!r})")


def _gate(gate, T_q, H, head_dim):
    """(pointer, per-head flag) of an optional output gate: [T_q, H*head_dim] or [T_q, H]."""
    if gate is None:
        return ctypes.c_void_p(0), 0
    _dev_f32(gate, "gate")
    if gate.numel() == T_q * H * head_dim:
        return _ptr(gate), 0
    if gate.numel() == T_q * H:
        return _ptr(gate), 1
    raise ValueError("gate must be [T_q, n_head*head_dim] or [T_q, n_head]")


def _chunk_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, prec, fused,
                     device):
    import torch
    need = int(lib().pfa_chunk_workspace_bytes(qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim,
                                               prec, _fused_code(fused)))
    if need == 0:
        return None, ctypes.c_void_p(0), 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise TypeError("workspace must be a GPU torch.Tensor")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def gqa_chunk_attn(q, k_cache, v_cache, *, head_dim: int, scale: float,
                   causal: bool = True, window: int = 0, gate=None, precision="f32",
                   q_offsets=None, kv_offsets=None, out=None, workspace=None):
    """Attention of new query rows over a K/V cache (``gqa_chunk_attn`` in
    ``include/pfa.h``); returns ``out``.  Sequence s owns query rows
    ``q_offsets[s]..q_offsets[s+1]`` and cache rows ``kv_offsets[s]..kv_offsets[s+1]``,
    its new rows being the last ones of its cache range.  ``window > 0``: each row sees
    only the last ``window`` keys up to its own.  ``gate`` ([T_q, n_head*head_dim] or
    [T_q, n_head]): the output is multiplied by its sigmoid."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_f32(t, n)
    T_q, H = _heads(q, head_dim, "q")
    T_kv, Hkv = _heads(k_cache, head_dim, "k_cache")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    prec = _prec(precision)
    ws, wp, wn = _chunk_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, prec,
                                  False, q.device)
    gp, gh = _gate(gate, T_q, H, head_dim)
    _check(lib().gqa_chunk_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), gp, gh, qp,
                                kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, float(scale),
                                1 if causal else 0, int(window), prec, wp, wn, _stream(q)))
    return out


def qk_prep_chunk_attn(q, k, v, q_norm_w, k_norm_w, k_cache, v_cache, *, head_dim: int,
                       rope_dim: int, rope_freq_base: float, rms_eps: float,
                       scale: float, causal: bool = True, window: int = 0,
                       gate=None, precision="f32", q_offsets=None, kv_offsets=None, out=None,
                       workspace=None):
    """Fused QK-norm + RoPE of the raw new rows at their positions, their K and V written
    into ``k_cache`` / ``v_cache`` (the last rows of each sequence's cache range), then
    attention over the cache (``qk_prep_chunk_attn`` in ``include/pfa.h``); returns
    ``out``."""
    import torch
    _norm_weights(q_norm_w, k_norm_w, head_dim)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_f32(t, n)
    T_q, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T_q or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    T_kv, Hc = _heads(k_cache, head_dim, "k_cache")
    if Hc != Hkv or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [T_kv, n_head_kv*head_dim] like k")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    prec = _prec(precision)
    ws, wp, wn = _chunk_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, prec,
                                  True, q.device)
    gp, gh = _gate(gate, T_q, H, head_dim)
    _check(lib().qk_prep_chunk_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), gp, gh,
                                    _ptr(q_norm_w), _ptr(k_norm_w), _ptr(k_cache), _ptr(v_cache), qp, kp, n_seqs,
                                    T_q, T_kv, H, Hkv, head_dim, rope_dim, float(rope_freq_base),
                                    float(rms_eps), float(scale), 1 if causal else 0,
                                    int(window), prec, wp, wn, _stream(q)))
    return out


def kv_tiles_bytes(n_slots: int, max_rows: int, n_head_kv: int, head_dim: int,
                   precision="bf16") -> int:
    """Bytes of the kept tiles of ``qk_prep_chunk_attn_tiled`` (``pfa_kv_tiles_bytes``)."""
    n = int(lib().pfa_kv_tiles_bytes(int(n_slots), int(max_rows), n_head_kv, head_dim,
                                     _prec(precision)))
    if n == 0:
        raise PfaError(-1, lib().pfa_last_error().decode())
    return n


def qk_prep_chunk_attn_tiled(q, k, v, q_norm_w, k_norm_w, k_cache, v_cache, kv_tiles, *,
                             max_rows: int, head_dim: int, rope_dim: int,
                             rope_freq_base: float, rms_eps: float, scale: float,
                             causal: bool = True, window: int = 0, gate=None,
                             precision="bf16", q_offsets=None, kv_offsets=None, out=None,
                             workspace=None):
    """``qk_prep_chunk_attn`` in the bf16 modes with the cache's bf16 tiles kept in
    ``kv_tiles`` across calls (``qk_prep_chunk_attn_tiled`` in ``include/pfa.h``): a GPU
    tensor of at least :func:`kv_tiles_bytes` bytes, passed to every call on the same
    cache with the same sequence count, ``max_rows`` and head geometry; returns ``out``."""
    import torch
    _norm_weights(q_norm_w, k_norm_w, head_dim)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev_f32(t, n)
    if not isinstance(kv_tiles, torch.Tensor) or kv_tiles.device.type != "cuda":
        raise TypeError("kv_tiles must be a GPU torch.Tensor")
    T_q, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T_q or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    T_kv, Hc = _heads(k_cache, head_dim, "k_cache")
    if Hc != Hkv or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [T_kv, n_head_kv*head_dim] like k")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    prec = _prec(precision)
    need = kv_tiles_bytes(max(n_seqs, 1), max_rows, Hkv, head_dim, precision)
    if kv_tiles.numel() * kv_tiles.element_size() < need:
        raise ValueError(f"kv_tiles holds {kv_tiles.numel() * kv_tiles.element_size()} bytes, "
                         f"{need} needed")
    ws, wp, wn = _chunk_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, prec,
                                  2, q.device)
    gp, gh = _gate(gate, T_q, H, head_dim)
    _check(lib().qk_prep_chunk_attn_tiled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), gp, gh, _ptr(q_norm_w), _ptr(k_norm_w),
        _ptr(k_cache), _ptr(v_cache), ctypes.c_void_p(kv_tiles.data_ptr()), int(max_rows), qp, kp,
        n_seqs, T_q, T_kv, H, Hkv, head_dim, rope_dim, float(rope_freq_base), float(rms_eps),
        float(scale), 1 if causal else 0, int(window), prec, wp, wn, _stream(q)))
    return out


# ---------------------------------------------------------------------------
# 8-bit quantised sessions: stores are (codes int8 [rows, heads*head_dim], scales f32
# [rows, heads]) pairs of GPU tensors.

def _dev(t, name, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _store(codes, scales, head_dim, name):
    """(rows, heads) of an 8-bit store, checked."""
    import torch
    _dev(codes, f"{name} codes", torch.int8)
    _dev(scales, f"{name} scales", torch.float32)
    rows, heads = _heads(codes, head_dim, f"{name} codes")
    if scales.numel() != rows * heads:
        raise ValueError(f"{name} scales must be [rows, heads] = [{rows}, {heads}]")
    return rows, heads


def quantize_rows(x, row_len: int, *, codes=None, scales=None, x_fq=None):
    """8-bit quantisation of every ``row_len`` values of ``x`` (``pfa_quantize_rows`` in
    ``include/pfa.h``); returns ``(codes, scales)``.  ``x_fq``: optional output of the
    fake-quantised values (may be ``x`` for in place)."""
    import torch
    _dev_f32(x, "x")
    if x.numel() % row_len:
        raise ValueError("x does not hold whole rows")
    n = x.numel() // row_len
    codes = torch.empty(x.shape, dtype=torch.int8, device=x.device) if codes is None else \
        _dev(codes, "codes", torch.int8)
    scales = torch.empty(n, dtype=torch.float32, device=x.device) if scales is None else \
        _dev(scales, "scales", torch.float32)
    if codes.numel() != x.numel() or scales.numel() != n:
        raise ValueError("codes must have x's size and scales one value per row")
    if x_fq is not None:
        _dev_f32(x_fq, "x_fq")
        if x_fq.numel() != x.numel():
            raise ValueError("x_fq must have x's size")
    _check(lib().pfa_quantize_rows(_ptr(x), n, int(row_len), _ptr(codes), _ptr(scales),
                                   _ptr(x_fq), _stream(x)))
    return codes, scales


def q8_workspace_bytes(T_q: int, T_kv: int, n_head: int, n_head_kv: int, head_dim: int,
                       q_offsets=None, kv_offsets=None, fused: bool = False) -> int:
    """Device workspace ``gqa_attn_q8`` (``fused=False``) or ``qk_prep_attn_q8``
    (``fused=True``) uses (``pfa_q8_workspace_bytes``)."""
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    return int(lib().pfa_q8_workspace_bytes(qp, kp, n_seqs, T_q, T_kv, n_head, n_head_kv,
                                            head_dim, 1 if fused else 0))


def _q8_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, fused, device):
    import torch
    need = int(lib().pfa_q8_workspace_bytes(qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim,
                                            1 if fused else 0))
    if need == 0:
        return None, ctypes.c_void_p(0), 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda":
        raise TypeError("workspace must be a GPU torch.Tensor")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def gqa_attn_q8(q, q_scale, k_cache, k_scale, v_cache, v_scale, *, head_dim: int,
                scale: float, causal: bool = True, window: int = 0, gate=None,
                q_offsets=None, kv_offsets=None, out=None, workspace=None):
    """Attention through 8-bit stores (``gqa_attn_q8`` in ``include/pfa.h``); returns
    ``out`` (f32).  Offsets, window and gate as for :func:`gqa_chunk_attn`."""
    import torch
    T_q, H = _store(q, q_scale, head_dim, "q")
    T_kv, Hkv = _store(k_cache, k_scale, head_dim, "k_cache")
    if _store(v_cache, v_scale, head_dim, "v_cache") != (T_kv, Hkv):
        raise ValueError("k and v stores must have the same shape")
    out = torch.empty((T_q, H * head_dim), dtype=torch.float32, device=q.device) \
        if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    ws, wp, wn = _q8_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, False,
                               q.device)
    gp, gh = _gate(gate, T_q, H, head_dim)
    _check(lib().gqa_attn_q8(_ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale),
                             _ptr(v_cache), _ptr(v_scale), _ptr(out), gp, gh, qp, kp, n_seqs,
                             T_q, T_kv, H, Hkv, head_dim, float(scale), 1 if causal else 0,
                             int(window), wp, wn, _stream(q)))
    return out


def qk_prep_attn_q8(q, k, v, q_norm_w, k_norm_w, k_cache, k_scale, v_cache, v_scale, *,
                    head_dim: int, rope_dim: int, rope_freq_base: float, rms_eps: float,
                    scale: float, causal: bool = True, window: int = 0,
                    gate=None, q_offsets=None, kv_offsets=None, out=None, workspace=None):
    """A quantised session's step (``qk_prep_attn_q8`` in ``include/pfa.h``): QK-norm +
    RoPE of the raw new rows, Q, K and V quantised per (token, head), K and V appended
    to the 8-bit store (the last rows of each sequence's range), attention through the
    store; returns ``out`` (f32)."""
    import torch
    _norm_weights(q_norm_w, k_norm_w, head_dim)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        _dev_f32(t, n)
    T_q, H = _heads(q, head_dim, "q")
    Tk, Hkv = _heads(k, head_dim, "k")
    if Tk != T_q or v.shape != k.shape:
        raise ValueError("q, k, v must have the same token count and k, v the same shape")
    T_kv, Hc = _store(k_cache, k_scale, head_dim, "k_cache")
    if Hc != Hkv or _store(v_cache, v_scale, head_dim, "v_cache") != (T_kv, Hkv):
        raise ValueError("the K and V stores must be [T_kv, n_head_kv*head_dim] like k")
    out = torch.empty_like(q) if out is None else _dev_f32(out, "out")
    if out.numel() != q.numel():
        raise ValueError("out must have q's shape")
    keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    ws, wp, wn = _q8_workspace(workspace, qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim, True,
                               q.device)
    gp, gh = _gate(gate, T_q, H, head_dim)
    _check(lib().qk_prep_attn_q8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), gp, gh, _ptr(q_norm_w),
                                 _ptr(k_norm_w), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                 _ptr(v_scale), qp, kp, n_seqs, T_q, T_kv, H, Hkv, head_dim,
                                 rope_dim, float(rope_freq_base), float(rms_eps), float(scale),
                                 1 if causal else 0, int(window), wp, wn, _stream(q)))
    return out


# ---------------------------------------------------------------------------
# Plan report (pfa_attn_plan / pfa_attn_units): what an attention call would enqueue.

def _plan_args(entry, T_q, n_head, n_head_kv, head_dim, rope_dim, T_kv, causal, window,
               precision, q_offsets, kv_offsets, has_k_rot_out, workspace_bytes):
    if entry not in (ENTRY_CHUNK, ENTRY_CHUNK_PREP, ENTRY_Q8, ENTRY_Q8_PREP, ENTRY_CHUNK_TILED):
        # the prefill entries (an unknown entry is left to the library to reject)
        keep, n_seqs, qp = _offsets(q_offsets, T_q)
        kp, T_kv = None, T_q
    else:
        if T_kv is None:
            raise ValueError("the chunk and 8-bit entries need T_kv")
        keep, n_seqs, qp, kp = _chunk_offsets(q_offsets, kv_offsets, T_q, T_kv)
    prec = _prec(precision) if entry not in (ENTRY_Q8, ENTRY_Q8_PREP) else PRECISION_BF16
    ws = (1 << 64) - 1 if workspace_bytes is None else int(workspace_bytes)
    return keep, (int(entry), qp, kp, n_seqs, int(T_q), int(T_kv), int(n_head), int(n_head_kv),
                  int(head_dim), int(rope_dim if rope_dim is not None else head_dim),
                  1 if causal else 0, int(window), prec, 1 if has_k_rot_out else 0, ws)


def attn_plan(entry: int, *, T_q: int, n_head: int, n_head_kv: int, head_dim: int,
              rope_dim: Optional[int] = None, T_kv: Optional[int] = None, causal: bool = True,
              window: int = 0, precision="f32", q_offsets=None, kv_offsets=None,
              has_k_rot_out: bool = False, workspace_bytes: Optional[int] = None) -> dict:
    """What one call of entry point ``entry`` (``ENTRY_*``) would enqueue for these
    arguments (``pfa_attn_plan``): work items, key split, pairing, grid, workspace bytes and
    the kernels in launch order.  ``workspace_bytes`` None: the call gets enough."""
    keep, args = _plan_args(entry, T_q, n_head, n_head_kv, head_dim, rope_dim, T_kv, causal,
                            window, precision, q_offsets, kv_offsets, has_k_rot_out,
                            workspace_bytes)
    plan = _Plan()
    _check(lib().pfa_attn_plan(*args, ctypes.byref(plan)))
    res = {name: getattr(plan, name) for name, _ in _Plan._fields_}
    res["kernels"] = plan.kernels.decode()
    return res


def attn_units(entry: int, *, T_q: int, n_head: int, n_head_kv: int, head_dim: int,
               rope_dim: Optional[int] = None, T_kv: Optional[int] = None, causal: bool = True,
               window: int = 0, precision="f32", q_offsets=None, kv_offsets=None,
               has_k_rot_out: bool = False, workspace_bytes: Optional[int] = None) -> np.ndarray:
    """The work unit of every attention workgroup (``pfa_attn_units``): an int32 array of
    one row per (workgroup, item it takes), columns :data:`UNIT_FIELDS`."""
    keep, args = _plan_args(entry, T_q, n_head, n_head_kv, head_dim, rope_dim, T_kv, causal,
                            window, precision, q_offsets, kv_offsets, has_k_rot_out,
                            workspace_bytes)
    n = int(lib().pfa_attn_units(*args, None, 0))
    if n < 0:
        _check(n)
    rec = np.zeros((max(n, 1), len(UNIT_FIELDS)), dtype=np.int32)
    m = int(lib().pfa_attn_units(*args, rec.ctypes.data_as(ctypes.c_void_p), n))
    if m != n:
        raise PfaError(-100, f"pfa_attn_units returned {m} records, then {n}")
    return rec[:n]
