"""CPU oracle for the prefill attention core -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.

``oracle.c`` holds the arithmetic (plain f64 loops, threaded over independent
rows); this module builds it with the host C compiler and wraps it for numpy.

* :func:`qknorm_rope` -- per-(token, head) RMSNorm with a learned scale, then
  NeoX rotary embedding (memra-engine 0.130.0 ``src/forward.rs``,
  ``Model::forward``, QK-norm and RoPE blocks; needle-core ``v3/model.rs``,
  ``rope_at`` / ``rope``).
* :func:`gqa_attn` -- causal grouped-query softmax attention
  (``Model::forward``, SDPA block; memra-engine 0.101.0 ``src/spec.rs``,
  ``full_attn_verify`` per-row fallback for the causal rule).
* :func:`qk_prep_attn` -- the two composed in f64 with no rounding between.
* :func:`chunk_attn`, :func:`qk_prep_chunk_attn` -- new rows over a cached prefix
  (memra-engine 0.101.0 ``src/spec.rs``, ``full_attn_verify``), with a sliding
  window and a gated output.
* :func:`quant_rows`, :func:`q8_chunk_attn`, :func:`qk_prep_q8_attn` -- 8-bit
  per-(token, head) quantisation of Q, K and V and attention through the 8-bit
  store (needle-core ``v3/model.rs``, ``quant_rows`` / ``quantize_rows``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    fp = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_qknorm_rope.argtypes = [fp, fp, fp, fp, ip, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.oracle_qknorm_rope.restype = ctypes.c_int
    lib.oracle_gqa_attn.argtypes = [dp, dp, dp, ip, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                    lp, ctypes.c_int64, dp, ctypes.c_int]
    lib.oracle_gqa_attn.restype = ctypes.c_int
    lib.oracle_qknorm_rope_from.argtypes = [fp, fp, fp, fp, ip, ctypes.c_int, lp, ctypes.c_int64,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_double, ctypes.c_double, dp,
                                            dp, ctypes.c_int]
    lib.oracle_qknorm_rope_from.restype = ctypes.c_int
    lib.oracle_chunk_attn.argtypes = [dp, dp, dp, ip, ip, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_int, ctypes.c_int64, dp,
                                      ctypes.c_int, lp, ctypes.c_int64, dp, ctypes.c_int]
    lib.oracle_chunk_attn.restype = ctypes.c_int
    lib.oracle_quant_rows.argtypes = [fp, ctypes.c_int64, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_int8), fp, fp]
    lib.oracle_quant_rows.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _offsets(seq_offsets, T):
    if seq_offsets is None:
        return np.array([0, T], dtype=np.int32)
    return np.ascontiguousarray(seq_offsets, dtype=np.int32)


def qknorm_rope(q, k, wq, wk, *, n_head, n_head_kv, head_dim, rope_dim, rope_freq_base,
                rms_eps, seq_offsets=None, pos0=None, n_threads=0):
    """O1 + O2 on f32 inputs ``q [T, n_head*head_dim]``, ``k [T, n_head_kv*head_dim]``.
    Row r of sequence s sits at position ``pos0[s] + r`` (``pos0`` None: r).

    Returns ``(q', k')`` as float64 arrays of the same shapes."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    wq = np.ascontiguousarray(wq, dtype=np.float32)
    wk = np.ascontiguousarray(wk, dtype=np.float32)
    T = q.shape[0]
    if q.size != T * n_head * head_dim or k.size != T * n_head_kv * head_dim:
        raise ValueError("q/k shapes do not match the head geometry")
    if wq.size != head_dim or wk.size != head_dim:
        raise ValueError("norm weights must have head_dim entries")
    offs = _offsets(seq_offsets, T)
    qo = np.empty((T, n_head * head_dim), dtype=np.float64)
    ko = np.empty((T, n_head_kv * head_dim), dtype=np.float64)
    if pos0 is None:
        p0 = None
    else:
        p0 = np.ascontiguousarray(pos0, dtype=np.int64)
        if p0.size != len(offs) - 1:
            raise ValueError("pos0 needs one entry per sequence")
    rc = _load().oracle_qknorm_rope_from(_ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                                         _ptr(wq, ctypes.c_float), _ptr(wk, ctypes.c_float),
                                         _ptr(offs, ctypes.c_int32), len(offs) - 1,
                                         None if p0 is None else _ptr(p0, ctypes.c_int64), T,
                                         n_head, n_head_kv, head_dim, rope_dim,
                                         float(rope_freq_base), float(rms_eps),
                                         _ptr(qo, ctypes.c_double), _ptr(ko, ctypes.c_double),
                                         n_threads)
    if rc != 0:
        raise ValueError(f"oracle_qknorm_rope failed ({rc})")
    return qo, ko


def gqa_attn(q, k, v, *, n_head, n_head_kv, head_dim, scale, causal=True, seq_offsets=None,
             rows=None, n_threads=0):
    """O3 on ``q [T, n_head*head_dim]``, ``k``/``v [T, n_head_kv*head_dim]`` (any float
    dtype; converted to f64 exactly).  With ``rows`` only those query rows are computed and
    the result is ``[len(rows), n_head*head_dim]``; otherwise ``[T, n_head*head_dim]``."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    T = q.shape[0]
    if q.size != T * n_head * head_dim or k.size != T * n_head_kv * head_dim or v.size != k.size:
        raise ValueError("q/k/v shapes do not match the head geometry")
    offs = _offsets(seq_offsets, T)
    if rows is None:
        rows_arr, n_rows, rp = None, T, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.size
        rp = _ptr(rows_arr, ctypes.c_int64)
    out = np.empty((n_rows, n_head * head_dim), dtype=np.float64)
    rc = _load().oracle_gqa_attn(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                 _ptr(v, ctypes.c_double), _ptr(offs, ctypes.c_int32),
                                 len(offs) - 1, T, n_head, n_head_kv, head_dim, float(scale),
                                 1 if causal else 0, rp, n_rows, _ptr(out, ctypes.c_double),
                                 n_threads)
    if rc != 0:
        raise ValueError(f"oracle_gqa_attn failed ({rc})")
    return out


def qk_prep_attn(q, k, v, wq, wk, *, n_head, n_head_kv, head_dim, rope_dim, rope_freq_base,
                 rms_eps, scale, causal=True, seq_offsets=None, rows=None, n_threads=0,
                 return_k_rot=False):
    """O3 applied to O1+O2 of the raw f32 Q and K, all in f64 with no rounding between."""
    qn, kn = qknorm_rope(q, k, wq, wk, n_head=n_head, n_head_kv=n_head_kv, head_dim=head_dim,
                         rope_dim=rope_dim, rope_freq_base=rope_freq_base, rms_eps=rms_eps,
                         seq_offsets=seq_offsets, n_threads=n_threads)
    out = gqa_attn(qn, kn, v, n_head=n_head, n_head_kv=n_head_kv, head_dim=head_dim,
                   scale=scale, causal=causal, seq_offsets=seq_offsets, rows=rows,
                   n_threads=n_threads)
    return (out, kn) if return_k_rot else out


def chunk_attn(q, k_cache, v_cache, *, n_head, n_head_kv, head_dim, scale, causal=True,
               q_offsets=None, kv_offsets=None, window=0, gate=None, rows=None, n_threads=0):
    """Attention of the query rows ``q [T_q, n_head*head_dim]`` over a K/V cache
    ``k_cache``/``v_cache [T_kv, n_head_kv*head_dim]``: sequence s owns query rows
    ``q_offsets[s]..q_offsets[s+1]`` and cache rows ``kv_offsets[s]..kv_offsets[s+1]``
    (at least as many); its queries are the last rows of its cache, so query row r sits
    at position ``base_s + r`` with ``base_s`` the rows cached before.  Causal: row r
    sees cache rows 0 .. base_s + r of its sequence, and with ``window > 0`` only the last
    ``window`` of those.  ``gate`` (``[T_q, n_head*head_dim]`` or ``[T_q, n_head]``): the
    output is multiplied by its logistic sigmoid, per element or per head.  Offsets: both
    or neither."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k_cache, dtype=np.float64)
    v = np.ascontiguousarray(v_cache, dtype=np.float64)
    T_q, T_kv = q.shape[0], k.shape[0]
    if q.size != T_q * n_head * head_dim or k.size != T_kv * n_head_kv * head_dim or \
            v.size != k.size:
        raise ValueError("q/k/v shapes do not match the head geometry")
    if (q_offsets is None) != (kv_offsets is None):
        raise ValueError("give both offset arrays or neither")
    qo = _offsets(q_offsets, T_q)
    ko = _offsets(kv_offsets, T_kv)
    gp, per_head = None, 0
    if gate is not None:
        g = np.ascontiguousarray(gate, dtype=np.float64)
        if g.size == T_q * n_head:
            per_head = 1
        elif g.size != T_q * n_head * head_dim:
            raise ValueError("gate must be [T_q, n_head*head_dim] or [T_q, n_head]")
        gp = _ptr(g, ctypes.c_double)
    if rows is None:
        n_rows, rp = T_q, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows, rp = rows_arr.size, _ptr(rows_arr, ctypes.c_int64)
    out = np.empty((n_rows, n_head * head_dim), dtype=np.float64)
    rc = _load().oracle_chunk_attn(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                   _ptr(v, ctypes.c_double), _ptr(qo, ctypes.c_int32),
                                   _ptr(ko, ctypes.c_int32), len(qo) - 1, T_q, T_kv, n_head,
                                   n_head_kv, head_dim, float(scale), 1 if causal else 0,
                                   int(window), gp, per_head, rp, n_rows,
                                   _ptr(out, ctypes.c_double), n_threads)
    if rc != 0:
        raise ValueError(f"oracle_chunk_attn failed ({rc})")
    return out


def qk_prep_chunk_attn(q, k, v, wq, wk, k_cache, v_cache, *, n_head, n_head_kv, head_dim,
                       rope_dim, rope_freq_base, rms_eps, scale, causal=True, q_offsets=None,
                       kv_offsets=None, window=0, gate=None, rows=None, n_threads=0):
    """A block of new rows over a cache: the raw f32 ``q``, ``k``, ``v [T_q, ...]`` are
    normalised and rotated (Q and K) at the positions of the new rows, K and V are
    written into the last rows of each sequence's cache range, and the queries attend
    the cache (:func:`chunk_attn`).  ``k_cache``/``v_cache [T_kv, ...]`` supply the rows
    cached before (their other rows are ignored).  Returns ``(out, k_cache', v_cache')``
    in f64, the caches with the new rows in place."""
    T_q = np.asarray(q).shape[0]
    T_kv = np.asarray(k_cache).shape[0]
    if (q_offsets is None) != (kv_offsets is None):
        raise ValueError("give both offset arrays or neither")
    qo = _offsets(q_offsets, T_q)
    ko = _offsets(kv_offsets, T_kv)
    base = (ko[1:] - ko[:-1]) - (qo[1:] - qo[:-1])
    if np.any(base < 0):
        raise ValueError("a sequence has fewer cache rows than new rows")
    qn, kn = qknorm_rope(q, k, wq, wk, n_head=n_head, n_head_kv=n_head_kv, head_dim=head_dim,
                         rope_dim=rope_dim, rope_freq_base=rope_freq_base, rms_eps=rms_eps,
                         seq_offsets=qo, pos0=base, n_threads=n_threads)
    kc = np.array(k_cache, dtype=np.float64, copy=True).reshape(T_kv, n_head_kv * head_dim)
    vc = np.array(v_cache, dtype=np.float64, copy=True).reshape(T_kv, n_head_kv * head_dim)
    v = np.asarray(v, dtype=np.float64).reshape(T_q, n_head_kv * head_dim)
    for s in range(len(qo) - 1):
        dst = slice(int(ko[s] + base[s]), int(ko[s + 1]))
        kc[dst] = kn[qo[s]:qo[s + 1]]
        vc[dst] = v[qo[s]:qo[s + 1]]
    out = chunk_attn(qn, kc, vc, n_head=n_head, n_head_kv=n_head_kv, head_dim=head_dim,
                     scale=scale, causal=causal, q_offsets=qo, kv_offsets=ko, window=window,
                     gate=gate, rows=rows, n_threads=n_threads)
    return out, kc, vc


def quant_rows(x, row_len):
    """8-bit quantisation of every ``row_len`` consecutive values of ``x`` (one row per
    (token, head) when ``row_len`` is the head size).  Returns ``(codes int8, scales f32,
    fake-quantised f32)`` shaped like ``x``, ``x.size / row_len`` and ``x``.  The input is
    taken as f32 (the integer decisions are made in single precision)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size % row_len:
        raise ValueError("x does not hold whole rows")
    n = x.size // row_len
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(n, dtype=np.float32)
    deq = np.empty(x.shape, dtype=np.float32)
    rc = _load().oracle_quant_rows(_ptr(x, ctypes.c_float), n, int(row_len),
                                   _ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_float),
                                   _ptr(deq, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle_quant_rows failed ({rc})")
    return codes, scales, deq


def _dequant(codes, scales, row_len):
    """codes x their row's scale, in f64 (exact: an 8-bit integer times a float)."""
    c = np.asarray(codes, dtype=np.float64).reshape(-1, row_len)
    return (c * np.asarray(scales, dtype=np.float64).reshape(-1, 1)).reshape(np.shape(codes))


def q8_chunk_attn(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, *, n_head,
                  n_head_kv, head_dim, scale, causal=True, q_offsets=None, kv_offsets=None,
                  window=0, gate=None, rows=None, n_threads=0):
    """Attention through the 8-bit store: every row (one per (token, head)) of Q, K and
    V is its integer codes times its scale.  The store's reader takes the scales out of
    the dot products, which is the attention of the dequantised rows; that is what is
    computed here (f64, :func:`chunk_attn`)."""
    return chunk_attn(_dequant(q_codes, q_scales, head_dim),
                      _dequant(k_codes, k_scales, head_dim),
                      _dequant(v_codes, v_scales, head_dim), n_head=n_head,
                      n_head_kv=n_head_kv, head_dim=head_dim, scale=scale, causal=causal,
                      q_offsets=q_offsets, kv_offsets=kv_offsets, window=window, gate=gate,
                      rows=rows, n_threads=n_threads)


def qk_prep_q8_attn(q, k, v, wq, wk, k_codes, k_scales, v_codes, v_scales, *, n_head,
                    n_head_kv, head_dim, rope_dim, rope_freq_base, rms_eps, scale,
                    causal=True, q_offsets=None, kv_offsets=None, window=0, gate=None,
                    rows=None, n_threads=0):
    """A quantised session's attention over an 8-bit cache: the raw f32 rows are
    normalised and rotated (Q and K, f64) at the positions of the new rows, rounded to
    f32, quantised per (token, head) with V (:func:`quant_rows`), the new K and V codes
    and scales are written into the last rows of each sequence's cache range, and the
    queries attend the cache through the store (:func:`q8_chunk_attn`).  Returns
    ``(out, k_codes', k_scales', v_codes', v_scales', q_codes, q_scales)``."""
    T_q = np.asarray(q).shape[0]
    T_kv = np.asarray(k_codes).shape[0]
    if (q_offsets is None) != (kv_offsets is None):
        raise ValueError("give both offset arrays or neither")
    qo = _offsets(q_offsets, T_q)
    ko = _offsets(kv_offsets, T_kv)
    base = (ko[1:] - ko[:-1]) - (qo[1:] - qo[:-1])
    if np.any(base < 0):
        raise ValueError("a sequence has fewer cache rows than new rows")
    qn, kn = qknorm_rope(q, k, wq, wk, n_head=n_head, n_head_kv=n_head_kv, head_dim=head_dim,
                         rope_dim=rope_dim, rope_freq_base=rope_freq_base, rms_eps=rms_eps,
                         seq_offsets=qo, pos0=base, n_threads=n_threads)
    qc, qs, _ = quant_rows(qn.astype(np.float32), head_dim)
    kq, kqs, _ = quant_rows(kn.astype(np.float32), head_dim)
    vq, vqs, _ = quant_rows(np.asarray(v, dtype=np.float32), head_dim)
    kc = np.array(k_codes, dtype=np.int8, copy=True).reshape(T_kv, n_head_kv * head_dim)
    ks = np.array(k_scales, dtype=np.float32, copy=True).reshape(T_kv, n_head_kv)
    vc = np.array(v_codes, dtype=np.int8, copy=True).reshape(T_kv, n_head_kv * head_dim)
    vs = np.array(v_scales, dtype=np.float32, copy=True).reshape(T_kv, n_head_kv)
    kq = kq.reshape(T_q, -1)
    vq = vq.reshape(T_q, -1)
    for s in range(len(qo) - 1):
        dst = slice(int(ko[s] + base[s]), int(ko[s + 1]))
        src = slice(int(qo[s]), int(qo[s + 1]))
        kc[dst], vc[dst] = kq[src], vq[src]
        ks[dst] = kqs.reshape(T_q, n_head_kv)[src]
        vs[dst] = vqs.reshape(T_q, n_head_kv)[src]
    out = q8_chunk_attn(qc, qs, kc, ks, vc, vs, n_head=n_head, n_head_kv=n_head_kv,
                        head_dim=head_dim, scale=scale, causal=causal, q_offsets=qo,
                        kv_offsets=ko, window=window, gate=gate, rows=rows,
                        n_threads=n_threads)
    return out, kc, ks, vc, vs, qc.reshape(T_q, -1), qs.reshape(T_q, n_head)


def version() -> str:
    return _load().oracle_version().decode()
