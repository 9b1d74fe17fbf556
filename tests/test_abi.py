"""The C ABI boundary, without a GPU: the library loads, exports every function
``include/pfa.h`` declares, and rejects bad arguments with a status code and a
message before anything is enqueued (so these calls never touch a device)."""
import ctypes
import os
import re

import numpy as np
import pytest

import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pfa.h")

OK, INVALID, UNSUPPORTED = 0, -1, -2


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libpfa.so is not built (run __graft_entry__.build())")
    return pfa.lib()


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("qknorm_rope", "gqa_prefill_attn", "qk_prep_attn", "pfa_workspace_bytes",
              "pfa_last_error", "pfa_version"):
        assert n in names
    assert set(names) == set(ops.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), f"libpfa.so does not export {n}"
    assert "gfx950" in pfa.version()


def _attn(L, T=16, H=4, Hkv=2, D=64, scale=0.125, causal=1, prec=0, offs=None, n_seqs=0,
          ptrs=(8, 8, 8, 8 << 20), ws=0, ws_bytes=0):
    q, k, v, o = (ctypes.c_void_p(p) for p in ptrs)
    return L.gqa_prefill_attn(q, k, v, o, offs, n_seqs, T, H, Hkv, D, scale, causal, prec,
                              ctypes.c_void_p(ws), ws_bytes, None)


def _msg(L):
    return L.pfa_last_error().decode()


def test_zero_tokens_is_ok_without_pointers(L):
    assert _attn(L, T=0, ptrs=(0, 0, 0, 0)) == OK
    n = ctypes.c_void_p(0)
    assert L.qknorm_rope(n, n, n, n, n, n, None, 0, 0, 4, 2, 64, 64, 1e6, 1e-6, None) == OK
    assert L.qk_prep_attn(n, n, n, n, n, n, None, 0, 0, 4, 2, 64, 64, 1e6, 1e-6, 0.125, 1, 0, n,
                          n, 0, None) == OK


@pytest.mark.parametrize("kw,status,needle", [
    (dict(H=3, Hkv=2), INVALID, "multiple"),
    (dict(H=0), INVALID, "positive"),
    (dict(T=-1), INVALID, ">= 0"),
    (dict(D=96), UNSUPPORTED, "head_dim"),
    (dict(D=256), UNSUPPORTED, "head_dim"),
    (dict(prec=7), INVALID, "precision"),
    (dict(prec=4), INVALID, "precision"),
    (dict(prec=-1), INVALID, "precision"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(ptrs=(0, 8, 8, 8 << 20)), INVALID, "null"),
    (dict(ptrs=(8, 8, 8, 16)), INVALID, "overlap"),
    (dict(T=1 << 20, H=64, Hkv=8, D=128), UNSUPPORTED, "2^31"),
    (dict(T=4, H=2048, Hkv=8, D=128), UNSUPPORTED, "query heads"),
])
def test_attention_rejects(L, kw, status, needle):
    assert _attn(L, **kw) == status
    assert needle in _msg(L)


def test_bad_seq_offsets(L):
    for offs, n, needle in (([0, 5, 3, 16], 3, "non-decreasing"), ([1, 16], 1, "[0]"),
                            ([0, 8, 15], 2, "T ="), ([0, 16], 0, "n_seqs")):
        arr = (ctypes.c_int32 * len(offs))(*offs)
        assert _attn(L, offs=ctypes.cast(arr, ctypes.c_void_p), n_seqs=n) == INVALID
        assert needle in _msg(L)
    arr = (ctypes.c_int32 * 130)(*([0] * 129 + [16]))
    assert _attn(L, offs=ctypes.cast(arr, ctypes.c_void_p), n_seqs=129) == UNSUPPORTED


@pytest.mark.parametrize("rope_dim,base,eps,needle", [
    (63, 1e6, 1e-6, "rope_dim"), (0, 1e6, 1e-6, "rope_dim"), (130, 1e6, 1e-6, "rope_dim"),
    (64, 0.0, 1e-6, "rope_freq_base"), (64, float("nan"), 1e-6, "rope_freq_base"),
    (64, 1e6, -1.0, "rms_eps"),
])
def test_rope_argument_checks(L, rope_dim, base, eps, needle):
    p = ctypes.c_void_p
    ptrs = [p(8), p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(5 << 20)]
    assert L.qknorm_rope(*ptrs, None, 0, 16, 4, 2, 64, rope_dim, base, eps, None) == INVALID
    assert needle in _msg(L)
    assert L.qk_prep_attn(p(8), p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(5 << 20), None,
                          0, 16, 4, 2, 64, rope_dim, base, eps, 0.125, 1, 0, p(0),
                          p(0), 0, None) == INVALID


def test_qknorm_rope_aliasing_rules(L):
    p = ctypes.c_void_p
    q, k = 1 << 20, 2 << 20  # 16 tokens x 4 heads x 64 dims x 4 B = 16 KiB
    w = 3 << 20
    # partial overlap of q_out with q_in is an error; exact in-place is accepted by the
    # checks (not launched here: only the error path runs on the CPU)
    assert L.qknorm_rope(p(q), p(k), p(q + 64), p(k), p(w), p(w), None, 0, 16, 4, 2, 64, 64,
                         1e6, 1e-6, None) == INVALID
    assert "overlap" in _msg(L)
    assert L.qknorm_rope(p(q), p(k), p(k), p(q), p(w), p(w), None, 0, 16, 4, 2, 64, 64,
                         1e6, 1e-6, None) == INVALID


def test_k_rot_out_must_not_alias(L):
    p = ctypes.c_void_p
    assert L.qk_prep_attn(p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(5 << 20),
                          p(5 << 20), None, 0, 16, 4, 2, 64, 64, 1e6, 1e-6, 0.125, 1, 0,
                          p(2 << 20), p(0), 0, None) == INVALID
    assert "k_rot_out" in _msg(L)


def test_python_binding_raises_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        pfa.gqa_prefill_attn(torch.zeros(4, 128), torch.zeros(4, 64), torch.zeros(4, 64),
                             head_dim=64, scale=0.125)
    with pytest.raises(TypeError):
        pfa.gqa_prefill_attn(torch.zeros(4, 128, dtype=torch.float64), torch.zeros(4, 64),
                             torch.zeros(4, 64), head_dim=64, scale=0.125)


@pytest.mark.parametrize("fn", ["gqa_prefill_attn", "qk_prep_attn", "gqa_chunk_attn",
                                "qk_prep_chunk_attn", "gqa_attn_q8", "qk_prep_attn_q8"])
def test_python_binding_takes_the_scale_from_the_caller(fn):
    """The softmax scale is an argument of every attention call; the binding computes
    no default (that would be the method's arithmetic outside the library)."""
    import inspect
    p = inspect.signature(getattr(pfa, fn)).parameters["scale"]
    assert p.default is inspect.Parameter.empty and p.kind is inspect.Parameter.KEYWORD_ONLY


@pytest.mark.parametrize("fn", ["qknorm_rope", "qk_prep_attn", "qk_prep_chunk_attn",
                                "qk_prep_attn_q8"])
def test_python_binding_checks_norm_weight_sizes(fn):
    """The kernels read head_dim norm weights: a shorter tensor is a Python error, not an
    out-of-bounds device read.  Checked before anything else (these are CPU tensors)."""
    import torch
    d = 64
    q, k = torch.zeros(4, 2 * d), torch.zeros(4, d)
    ok, short = torch.ones(d), torch.ones(d - 1)
    rope = dict(head_dim=d, rope_dim=d, rope_freq_base=1e4, rms_eps=1e-6)
    for wq, wk, bad in ((short, ok, "q_norm_w"), (ok, short, "k_norm_w")):
        with pytest.raises(ValueError, match=bad):
            if fn == "qknorm_rope":
                pfa.qknorm_rope(q, k, wq, wk, **rope)
            elif fn == "qk_prep_attn":
                pfa.qk_prep_attn(q, k, k, wq, wk, scale=0.125, **rope)
            elif fn == "qk_prep_chunk_attn":
                pfa.qk_prep_chunk_attn(q, k, k, wq, wk, k, k, scale=0.125, **rope)
            else:
                c8 = torch.zeros(4, d, dtype=torch.int8)
                s8 = torch.zeros(4, 1)
                pfa.qk_prep_attn_q8(q, k, k, wq, wk, c8, s8, c8, s8, scale=0.125, **rope)


def _ceil(a, b):
    return -(-a // b)


def _expected_workspace(lens, H, Hkv, D, prec, fused, kv_lens=None, chunk=False):
    """The workspace rule pfa_workspace_bytes / pfa_chunk_workspace_bytes document,
    restated: bf16 tiles of every sequence's key rows (plus the rotary table, as long as
    the longest, when Q is prepared in the kernel) or the f32 fused prefill's rotated K,
    then partial results when the (query block, head) items cannot fill the GPU's
    workgroup slots (a target of 512 f32 or 256 bf16 workgroups) and are split by key,
    at least 128 keys a chunk and at most 32 chunks an item (PFA_PREC_BF16 and F16: only
    when a sequence spans at least 2048 keys; shorter ones, with items filling at most a
    quarter of the slots, in two halves).  The chunk length: in the 16-bit modes, the one
    that fills the target with items of n_max tiles each; in f32 the shortest, from that
    floor and 320 keys on, whose non-empty units -- every item's causally visible tiles cut
    into chunks -- fit the target, but no longer than the 16-bit modes' length and, when
    that gives at most 4 chunks an item, no shorter than n_max / 4.
    With at most 4 chunks an item, one 8-byte arrival counter per (item, head group, K/V
    head) follows the partial results, at the next multiple of 256 bytes.  ``lens``:
    query rows per sequence; ``kv_lens``: key rows (default: the same)."""
    kv_lens = lens if kv_lens is None else kv_lens
    bf16 = prec != 0
    waves, tile = (8, 64) if bf16 else (4, 32)
    g = H // Hkv
    hpw = 1
    while hpw < 4 and g % (hpw * 2) == 0:
        hpw *= 2
    chunks, rows = g // hpw, 32 * (waves // hpw)
    items = sum(_ceil(n, rows) for n in lens)
    n_max = _ceil(max(kv_lens), tile)
    wgs, target = items * chunks * Hkv, (1 if bf16 else 2) * 256
    kchunk = 0
    # plain bf16 and f16 split only sequences of at least 32 tiles (2048 keys)
    if wgs < target and n_max >= (32 if prec in (1, 3) else 2):
        # at least 128 keys a chunk, at most 32 chunks an item
        floor = max(_ceil(128, tile), _ceil(n_max, 32))
        k_full = max(floor, _ceil(wgs * n_max, target))
        # each item's visible tiles: its last query row's keys (causal; a chunk's rows are
        # the last of its sequence's key rows)
        tiles = [(min(q0 + rows, n) - 1 + (kn - n)) // tile + 1
                 for n, kn in zip(lens, kv_lens) for q0 in range(0, n, rows)]
        lo = max(floor, _ceil(320, tile))
        if _ceil(n_max, k_full) <= 4:
            lo = max(lo, _ceil(n_max, 4))
        if bf16:
            lo = k_full
        kchunk = next((c for c in range(lo, k_full)
                       if sum(_ceil(t, c) for t in tiles) * chunks * Hkv <= target), k_full)
        if kchunk >= n_max:
            kchunk = 0
    elif prec in (1, 3) and n_max >= 8 and wgs * 4 <= target:
        # shorter inputs in plain bf16 / f16 with few items: two halves, when a half is at
        # least 6 tiles or the items fill at most an eighth of the slots
        half = _ceil(n_max, 2)
        if half >= 6 or wgs * 8 <= target:
            kchunk = half
    parts = 0
    if kchunk and items:
        units = items * _ceil(n_max, kchunk) * chunks * Hkv
        parts = units * waves * 32 * (D * 4 + 8)
        if _ceil(n_max, kchunk) <= 4:
            parts = _ceil(parts, 256) * 256 + items * chunks * Hkv * 8
    base = 0
    if bf16:
        base = Hkv * sum(_ceil(n, 64) for n in kv_lens) * 64 * D * 2 * (3 if prec == 2 else 2)
        if fused:
            base += max(kv_lens) * (D // 2) * 8
    elif fused and not chunk:
        base = sum(lens) * Hkv * D * 4
    if items == 0:
        return 0
    return (_ceil(base, 256) * 256 + parts) if parts else base


def _ws(L, lens, H, Hkv, D, prec, pass_offsets=True, fused=0):
    offs = np.cumsum([0] + list(lens)).astype(np.int32)
    arr = (ctypes.c_int32 * len(offs))(*offs.tolist())
    ptr = ctypes.cast(arr, ctypes.c_void_p) if pass_offsets else None
    return L.pfa_workspace_bytes(ptr, len(lens), int(offs[-1]), H, Hkv, D, prec, fused)


@pytest.mark.parametrize("lens,H,Hkv,D", [
    ((8192,), 32, 8, 128), ((512,), 16, 8, 128), ((512,), 32, 8, 128), ((1024,), 32, 8, 128),
    ((128, 256, 512, 1024, 2048, 3000, 4096, 5000), 16, 4, 128), ((16,), 4, 2, 64),
    ((300,), 8, 2, 128), ((1, 33, 0, 64, 65, 97), 4, 2, 128), ((90,), 6, 2, 64),
    ((2048,), 32, 8, 128), ((3072,), 32, 8, 128), ((2048, 2048), 16, 8, 128),
    ((6000, 100, 100), 32, 8, 128)])
@pytest.mark.parametrize("prec", [0, 1, 2, 3])
@pytest.mark.parametrize("fused", [0, 1])
def test_workspace_bytes_rule(L, lens, H, Hkv, D, prec, fused):
    assert _ws(L, lens, H, Hkv, D, prec, fused=fused) == \
        _expected_workspace(lens, H, Hkv, D, prec, fused)


def test_workspace_bytes_cases():
    # long inputs in f32 need nothing; the T = 512 shapes split their keys
    L = pfa.lib()
    assert _ws(L, (8192,), 32, 8, 128, 0) == 0
    assert _ws(L, (8192,), 32, 8, 128, 0, fused=1) == 8192 * 8 * 128 * 4  # rotated K
    assert _ws(L, (512,), 16, 8, 128, 0) > 0
    assert _ws(L, (8192,), 32, 8, 128, 1, pass_offsets=False) == 8 * 128 * 64 * 128 * 2 * 2
    assert _ws(L, (8192,), 32, 8, 128, 1, pass_offsets=False, fused=1) == \
        8 * 128 * 64 * 128 * 2 * 2 + 8192 * 64 * 8
    assert pfa.workspace_bytes(8192, 32, 8, 128, "bf16x3", fused=True) == \
        8 * 128 * 64 * 128 * 2 * 3 + 8192 * 64 * 8
    # f16 keeps the bf16 mode's tiles (same sizes, binary16 values), and its split rule
    for fused in (False, True):
        for T in (512, 2048, 8192):
            assert pfa.workspace_bytes(T, 32, 8, 128, "f16", fused=fused) == \
                pfa.workspace_bytes(T, 32, 8, 128, "bf16", fused=fused)
    assert pfa.kv_tiles_bytes(2, 3000, 8, 128, "f16") == pfa.kv_tiles_bytes(2, 3000, 8, 128, "bf16")


def test_workspace_bytes_rejects_what_attention_rejects(L):
    assert _ws(L, (16,), 4, 2, 96, 1) == 0
    assert "head_dim" in L.pfa_last_error().decode()
    assert _ws(L, (16,), 4, 2, 64, 7) == 0
    assert "precision" in L.pfa_last_error().decode()
    assert _ws(L, (16,) * 129, 4, 2, 64, 1) == 0
    assert _ws(L, (16,), 3, 2, 64, 1) == 0


@pytest.mark.parametrize("prec", [1, 2, 3])
def test_bf16_modes_check_the_workspace(L, prec):
    # every call below must fail its checks before any launch (the pointers are not real)
    ptrs = (1 << 20, 2 << 20, 3 << 20, 4 << 20)   # q 16x4x64 f32 = 16 KiB, k/v 8 KiB each
    need = _ws(L, (16,), 4, 2, 64, prec)
    exact = (3 if prec == 2 else 2) * 2 * 1 * 64 * 64 * 2   # one 64-key tile per K/V head
    assert exact <= need
    assert _attn(L, prec=prec, ptrs=ptrs) == INVALID
    assert "workspace" in _msg(L)
    assert _attn(L, prec=prec, ptrs=ptrs, ws=8 << 20, ws_bytes=exact - 1) == INVALID
    assert "needed" in _msg(L)
    assert _attn(L, prec=prec, ptrs=ptrs, ws=(8 << 20) + 16, ws_bytes=need) == INVALID
    assert "aligned" in _msg(L)
    assert _attn(L, prec=prec, ptrs=ptrs, ws=(3 << 20) + 4096, ws_bytes=need) == INVALID
    assert "overlap" in _msg(L)


def test_f32_fused_needs_a_workspace_or_k_rot_out(L):
    # the rotated K goes to k_rot_out or the workspace; with neither the call is refused
    # before any launch (the pointers are not real)
    p = ctypes.c_void_p
    assert L.qk_prep_attn(p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(5 << 20),
                          p(5 << 20), None, 0, 16, 4, 2, 64, 64, 1e6, 1e-6, 0.125, 1, 0,
                          p(0), p(0), 0, None) == INVALID
    assert "workspace" in _msg(L)
    need = _ws(L, (16,), 4, 2, 64, 0, fused=1)
    assert need == 16 * 2 * 64 * 4
    assert L.qk_prep_attn(p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(5 << 20),
                          p(5 << 20), None, 0, 16, 4, 2, 64, 64, 1e6, 1e-6, 0.125, 1, 0,
                          p(0), p(8 << 20), need - 1, None) == INVALID
    assert "needed" in _msg(L)


def _i32(a):
    arr = (ctypes.c_int32 * len(a))(*a)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _chunk(L, q_offs, kv_offs, T_q, T_kv, H=4, Hkv=2, D=64, prec=0, ptrs=(8, 8, 8, 8 << 20),
           ws=0, ws_bytes=0, causal=1, window=0, gate=0, gate_per_head=0):
    keep_q, qp = _i32(q_offs) if q_offs is not None else (None, None)
    keep_k, kp = _i32(kv_offs) if kv_offs is not None else (None, None)
    n = len(q_offs) - 1 if q_offs is not None else 0
    q, k, v, o = (ctypes.c_void_p(p) for p in ptrs)
    return L.gqa_chunk_attn(q, k, v, o, ctypes.c_void_p(gate), gate_per_head, qp, kp, n, T_q,
                            T_kv, H, Hkv, D, 0.125, causal, window, prec, ctypes.c_void_p(ws),
                            ws_bytes, None)


def test_chunk_with_no_new_rows_is_ok_without_pointers(L):
    assert _chunk(L, None, None, 0, 0, ptrs=(0, 0, 0, 0)) == OK
    assert _chunk(L, [0, 0], [0, 40], 0, 40, ptrs=(0, 0, 0, 0)) == OK


def test_chunk_rejects_caches_shorter_than_their_queries(L):
    assert _chunk(L, [0, 4], [0, 3], 4, 3) == INVALID
    assert "cache rows" in _msg(L)
    assert _chunk(L, [0, 2, 6], [0, 5, 8], 6, 8) == INVALID   # second sequence: 3 rows for 4
    assert "sequence 1" in _msg(L)


def test_chunk_offsets_come_in_pairs(L):
    assert _chunk(L, [0, 4], None, 4, 9) == INVALID
    assert "both or neither" in _msg(L)
    assert _chunk(L, [0, 4], [0, 9], 4, 8) == INVALID   # kv_offsets must end at T_kv
    assert "T = 8" in _msg(L)


def _chunk_ws(L, q_lens, kv_lens, H, Hkv, D, prec, fused):
    qo = np.cumsum([0] + list(q_lens)).astype(np.int32)
    ko = np.cumsum([0] + list(kv_lens)).astype(np.int32)
    keep_q, qp = _i32(qo.tolist())
    keep_k, kp = _i32(ko.tolist())
    return L.pfa_chunk_workspace_bytes(qp, kp, len(q_lens), int(qo[-1]), int(ko[-1]), H, Hkv, D,
                                       prec, fused)


@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("fused", [0, 1])
def test_chunk_workspace_without_prefix_is_the_prefill_rule(L, prec, fused):
    # no cached rows: the chunk call plans exactly what the prefill call plans, except that
    # the f32 fused chunk entry writes its rotated K into the cache, not the workspace
    for lens in ((512,), (300, 1, 97), (8192,)):
        expect = _expected_workspace(lens, 16, 8, 128, prec, fused and prec != 0)
        assert _chunk_ws(L, lens, lens, 16, 8, 128, prec, fused) == expect


@pytest.mark.parametrize("prec", [0, 1, 2])
@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("q_lens,kv_lens,H,Hkv,D", [
    ((1024,), (8192,), 32, 8, 128), ((1,), (8192,), 32, 8, 128), ((4096,), (8192,), 32, 8, 128),
    ((50, 1, 130, 0), (70, 78, 130, 5), 8, 4, 128), ((90,), (135,), 4, 2, 64),
    ((2048,), (2048,), 32, 8, 128), ((2048,), (2600,), 32, 8, 128)])
def test_chunk_workspace_rule(L, q_lens, kv_lens, H, Hkv, D, prec, fused):
    assert _chunk_ws(L, q_lens, kv_lens, H, Hkv, D, prec, fused) == \
        _expected_workspace(q_lens, H, Hkv, D, prec, fused, kv_lens=kv_lens, chunk=True)


def test_chunk_workspace_tiles_cover_the_cache(L):
    # bf16, 8192 cache rows with 4096 new: no key split, so exactly the tiles of all 8192
    # rows (+ a rotary table as long as the cache for the fused entry)
    tiles = 8 * 128 * 64 * 128 * 2
    assert _chunk_ws(L, (4096,), (8192,), 32, 8, 128, 1, 0) == 2 * tiles
    assert _chunk_ws(L, (4096,), (8192,), 32, 8, 128, 1, 1) == 2 * tiles + 8192 * 64 * 8
    assert _chunk_ws(L, (4096,), (8192,), 32, 8, 128, 2, 0) == 3 * tiles
    assert pfa.chunk_workspace_bytes(4096, 8192, 32, 8, 128, "bf16", fused=True) == \
        2 * tiles + 8192 * 64 * 8


@pytest.mark.parametrize("prec", [1, 2])
@pytest.mark.parametrize("q_lens,kv_lens,H,Hkv,D", [
    ((1024,), (8192,), 32, 8, 128), ((1,), (8192,), 32, 8, 128), ((4096,), (8192,), 32, 8, 128),
    ((50, 1, 130, 0), (70, 78, 130, 5), 8, 4, 128), ((512,), (512,), 16, 8, 128)])
def test_tiled_chunk_workspace_holds_only_the_partials(L, q_lens, kv_lens, H, Hkv, D, prec):
    # qk_prep_chunk_attn_tiled keeps its tiles and rotary table in kv_tiles: its workspace is
    # the key split's part of qk_prep_chunk_attn's (the same plan)
    full = _expected_workspace(q_lens, H, Hkv, D, prec, 1, kv_lens=kv_lens, chunk=True)
    tiles = Hkv * sum(_ceil(n, 64) for n in kv_lens) * 64 * D * 2 * (3 if prec == 2 else 2)
    base = tiles + max(kv_lens) * (D // 2) * 8
    parts = full - _ceil(base, 256) * 256 if full > base else 0
    assert _chunk_ws(L, q_lens, kv_lens, H, Hkv, D, prec, 2) == parts
    assert _chunk_ws(L, q_lens, kv_lens, H, Hkv, D, 0, 2) == 0  # f32: rejected
    assert "PFA_PREC_BF16" in _msg(L)


@pytest.mark.parametrize("n_slots,max_rows,Hkv,D,prec", [
    (1, 1, 1, 64, 1), (1, 8192, 8, 128, 1), (3, 1300, 8, 128, 2), (128, 65, 2, 64, 1)])
def test_kv_tiles_bytes_rule(L, n_slots, max_rows, Hkv, D, prec):
    # slots of ceil(max_rows / 64) tiles per K/V head (K twice for bf16x3, V once, 64 x D
    # bf16 each), then a rotary table of that many rows x D/2 (cos, sin) f32 pairs
    cap = _ceil(max_rows, 64)
    expect = n_slots * cap * Hkv * (3 if prec == 2 else 2) * 64 * D * 2 + cap * 64 * (D // 2) * 8
    assert L.pfa_kv_tiles_bytes(n_slots, max_rows, Hkv, D, prec) == expect
    assert pfa.kv_tiles_bytes(n_slots, max_rows, Hkv, D, "bf16x3" if prec == 2 else "bf16") == expect


@pytest.mark.parametrize("args,needle", [
    ((1, 64, 8, 128, 0), "PFA_PREC_BF16"), ((0, 64, 8, 128, 1), "n_slots"),
    ((129, 64, 8, 128, 1), "n_slots"), ((1, 0, 8, 128, 1), "max_rows"),
    ((1, 64, 8, 96, 1), "head_dim")])
def test_kv_tiles_bytes_rejects(L, args, needle):
    assert L.pfa_kv_tiles_bytes(*args) == 0
    assert needle in _msg(L)


def _tiled(L, q_offs, kv_offs, T_q, T_kv, max_rows=256, prec=1, tiles=1 << 30, Hkv=2, D=64):
    keep_q, qp = _i32(q_offs)
    keep_k, kp = _i32(kv_offs)
    p = ctypes.c_void_p
    # q, k, v, out, weights and caches at distinct fake addresses: only the checks run
    return L.qk_prep_chunk_attn_tiled(p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p(0), 0,
                                      p(5 << 20), p(5 << 20), p(6 << 20), p(7 << 20), p(tiles),
                                      max_rows, qp, kp, len(q_offs) - 1, T_q, T_kv, 4, Hkv, D, D,
                                      1e6, 1e-6, 0.125, 1, 0, prec, p(0), 0, None)


def test_tiled_chunk_argument_checks(L):
    assert _tiled(L, [0, 4], [0, 9], 4, 9, prec=0) == INVALID
    assert "PFA_PREC_BF16" in _msg(L)
    assert _tiled(L, [0, 4], [0, 9], 4, 9, tiles=0) == INVALID
    assert "kv_tiles" in _msg(L)
    assert _tiled(L, [0, 4], [0, 9], 4, 9, tiles=(1 << 30) + 64) == INVALID
    assert "aligned" in _msg(L)
    assert _tiled(L, [0, 4, 8], [0, 9, 300], 8, 300, max_rows=256) == INVALID
    assert "max_rows" in _msg(L)
    assert _tiled(L, [0, 4], [0, 9], 4, 9, max_rows=0) == INVALID
    assert "max_rows" in _msg(L)
    # kv_tiles over out (4 MiB + 8 KiB of f32 rows at 4 << 20)
    assert _tiled(L, [0, 4], [0, 9], 4, 9, tiles=4 << 20) == INVALID
    assert "overlap" in _msg(L)


def test_chunk_window_arguments(L):
    assert _chunk(L, [0, 4], [0, 9], 4, 9, window=-1) == INVALID
    assert "window" in _msg(L)
    assert _chunk(L, [0, 4], [0, 9], 4, 9, window=3, causal=0) == INVALID
    assert "causal" in _msg(L)


def test_chunk_gate_must_not_overlap_out(L):
    # out is [4, 4*64] f32 at 8 MiB; a gate inside it is refused before any launch
    assert _chunk(L, [0, 4], [0, 9], 4, 9, gate=(8 << 20) + 256) == INVALID
    assert "gate" in _msg(L)


# ---------------------------------------------------------------------------
# 8-bit quantised sessions

def _q8_ws(L, q_lens, kv_lens, H, Hkv, D, fused):
    qo = np.cumsum([0] + list(q_lens)).astype(np.int32)
    ko = np.cumsum([0] + list(kv_lens)).astype(np.int32)
    keep_q, qp = _i32(qo.tolist())
    keep_k, kp = _i32(ko.tolist())
    return L.pfa_q8_workspace_bytes(qp, kp, len(q_lens), int(qo[-1]), int(ko[-1]), H, Hkv, D,
                                    fused)


@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("q_lens,kv_lens,H,Hkv,D", [
    ((8192,), (8192,), 32, 8, 128), ((1024,), (8192,), 32, 8, 128), ((512,), (512,), 16, 8, 128),
    ((50, 1, 130, 0), (70, 78, 130, 5), 8, 4, 128), ((90,), (135,), 4, 2, 64)])
def test_q8_workspace_rule(L, q_lens, kv_lens, H, Hkv, D, fused):
    # K tiles (int8 codes for head_dim 128, bf16 for 64) and bf16 V tiles, 256 bytes of
    # key scales per tile and K/V head, (fused) the Q codes and scales, each part 256-byte
    # aligned, then the bf16 plan's partial results
    bf16_chunk = _expected_workspace(q_lens, H, Hkv, D, 1, 0, kv_lens=kv_lens, chunk=True)
    bf16_tiles = Hkv * sum(_ceil(n, 64) for n in kv_lens) * 64 * D * 2 * 2
    parts = bf16_chunk - _ceil(bf16_tiles, 256) * 256 if bf16_chunk > bf16_tiles else 0
    n_t = Hkv * sum(_ceil(n, 64) for n in kv_lens)
    tiles = n_t * (64 * D * (1 if D == 128 else 2) + 64 * D * 2)
    end = tiles + Hkv * sum(_ceil(n, 64) for n in kv_lens) * 256
    if fused:
        T_q = sum(q_lens)
        qs_off = _ceil(_ceil(end, 256) * 256 + T_q * H * D, 256) * 256
        end = qs_off + T_q * H * 4
    expect = (_ceil(end, 256) * 256 + parts) if parts else end
    assert _q8_ws(L, q_lens, kv_lens, H, Hkv, D, fused) == expect


def _q8(L, T_q=4, T_kv=9, H=4, Hkv=2, D=64, scale=0.125, window=0, causal=1, ptrs=None,
        ws=1 << 30, ws_bytes=1 << 24, offs=([0, 4], [0, 9])):
    # q codes, q scales, k codes, k scales, v codes, v scales, out, gate: disjoint by default
    p = ptrs or (1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 6 << 20, 8 << 20, 0)
    keep_q, qp = _i32(offs[0])
    keep_k, kp = _i32(offs[1])
    c = [ctypes.c_void_p(x) for x in p]
    return L.gqa_attn_q8(*c[:7], c[7], 0, qp, kp, len(offs[0]) - 1, T_q, T_kv, H, Hkv, D,
                         scale, causal, window, ctypes.c_void_p(ws), ws_bytes, None)


def test_q8_attention_argument_checks(L):
    assert _q8(L, scale=0.0) == INVALID and "scale > 0" in _msg(L)
    assert _q8(L, scale=-0.5) == INVALID
    assert _q8(L, window=-2) == INVALID and "window" in _msg(L)
    assert _q8(L, ws=0) == INVALID and "workspace" in _msg(L)
    assert _q8(L, ws_bytes=16) == INVALID and "needed" in _msg(L)
    assert _q8(L, ws=(1 << 30) + 64) == INVALID and "256-byte" in _msg(L)
    p = [1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 6 << 20, 8 << 20, 0]
    p[2] += 8   # K codes not 16-byte aligned
    assert _q8(L, ptrs=tuple(p)) == INVALID and "aligned" in _msg(L)
    p = [1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 6 << 20, (3 << 20) + 64, 0]   # out in K
    assert _q8(L, ptrs=tuple(p)) == INVALID and "out must not overlap k_cache" in _msg(L)
    assert _q8(L, ws=(8 << 20)) == INVALID and "overlap" in _msg(L)   # workspace over out
    assert _q8(L, T_q=0, T_kv=0, offs=([0, 0], [0, 0]), ptrs=(0,) * 8, ws=0, ws_bytes=0) == OK
    assert _q8(L, offs=([0, 4], [0, 3]), T_kv=3) == INVALID and "cache rows" in _msg(L)


def test_q8_prep_argument_checks(L):
    keep_q, qp = _i32([0, 4])
    keep_k, kp = _i32([0, 9])
    v = ctypes.c_void_p
    args = [v(1 << 20), v(2 << 20), v(3 << 20), v(8 << 20), v(0), 0, v(4 << 20), v(5 << 20),
            v(6 << 20), v(7 << 20), v(9 << 20), v(10 << 20), qp, kp, 1, 4, 9, 4, 2, 64, 64,
            1e4, 1e-6, 0.125, 1, 0, v(1 << 30), 1 << 24, None]
    a = list(args)
    a[20] = 63   # odd rope_dim
    assert L.qk_prep_attn_q8(*a) == INVALID and "rope_dim" in _msg(L)
    a = list(args)
    a[6] = v(0)   # no norm weights
    assert L.qk_prep_attn_q8(*a) == INVALID and "norm weights" in _msg(L)
    a = list(args)
    a[9] = v((6 << 20) + 16)   # K scales inside the K codes (written)
    assert L.qk_prep_attn_q8(*a) == INVALID and "overlap" in _msg(L)
    a = list(args)
    a[23] = 0.0
    assert L.qk_prep_attn_q8(*a) == INVALID and "scale > 0" in _msg(L)


def test_quantize_rows_argument_checks(L):
    v = ctypes.c_void_p
    assert L.pfa_quantize_rows(v(0), 0, 128, v(0), v(0), v(0), None) == OK
    assert L.pfa_quantize_rows(v(1 << 20), 4, 0, v(2 << 20), v(3 << 20), v(0), None) == INVALID
    assert "row_len" in _msg(L)
    assert L.pfa_quantize_rows(v(1 << 20), -1, 8, v(2 << 20), v(3 << 20), v(0), None) == INVALID
    assert L.pfa_quantize_rows(v(1 << 20), 4, 8, v(0), v(3 << 20), v(0), None) == INVALID
    assert "null" in _msg(L)
    # codes inside x, and an x_fq that overlaps x without being x
    assert L.pfa_quantize_rows(v(1 << 20), 4, 8, v((1 << 20) + 8), v(3 << 20), v(0),
                               None) == INVALID
    assert L.pfa_quantize_rows(v(1 << 20), 4, 8, v(2 << 20), v(3 << 20), v((1 << 20) + 4),
                               None) == INVALID
    assert "overlap" in _msg(L)


def test_tensor_pointers_must_be_16_byte_aligned(L):
    # the header requires 16-byte aligned tensors (the kernels move 16-byte vectors); a
    # misaligned one is rejected on the host, after the other checks, before any launch.
    # (Every call here fails validation: the fake addresses never reach a kernel.)
    p = ctypes.c_void_p
    for bad in range(4):
        ptrs = [(i + 1) << 20 for i in range(4)]
        ptrs[bad] += 4
        assert _attn(L, ptrs=tuple(ptrs)) == INVALID
        assert "16-byte aligned" in _msg(L)
    w = [p((i + 1) << 20) for i in range(6)]
    w[4] = p((5 << 20) + 8)  # q_norm_w
    assert L.qknorm_rope(*w, None, 0, 16, 4, 2, 64, 64, 1e6, 1e-6, None) == INVALID
    assert "16-byte aligned" in _msg(L)
    assert L.qk_prep_attn(p(1 << 20), p(2 << 20), p(3 << 20), p(4 << 20), p((5 << 20) + 4),
                          p(6 << 20), None, 0, 16, 4, 2, 64, 64, 1e6, 1e-6, 0.125, 1, 0,
                          p(7 << 20), p(8 << 20), 16 << 20, None) == INVALID
    assert "16-byte aligned" in _msg(L)


def test_noalloc_rejects_calls_beyond_its_device_array(L):
    """gqa_prefill_attn_noalloc refuses, before anything is enqueued, a call whose workspace
    would not fit in the library's device array (bf16 tiles of 20000 key rows at 8 K/V
    heads of 128 need 82 MB)."""
    p = ctypes.c_void_p
    T = 20000
    assert L.pfa_noalloc_scratch_bytes() == 64 << 20
    assert pfa.workspace_bytes(T, 32, 8, 128, "bf16") > L.pfa_noalloc_scratch_bytes()
    assert L.gqa_prefill_attn_noalloc(p(1 << 30), p(2 << 30), p(3 << 30), p(4 << 30), None, 0,
                                      T, 32, 8, 128, 0.088, 1, 1, None) == UNSUPPORTED
    assert "device array" in _msg(L)
    # argument errors come first, as for gqa_prefill_attn
    assert L.gqa_prefill_attn_noalloc(p(1 << 30), p(2 << 30), p(3 << 30), p(4 << 30), None, 0,
                                      16, 4, 2, 96, 0.125, 1, 0, None) == UNSUPPORTED
    assert "head_dim" in _msg(L)
