"""GPU parity of the two merges of a key split, element by element against the f64 oracle,
through the C ABI.

When a call's (query block, head) items cannot fill the GPU, each item's keys are split
over several workgroups and their partial results merged with the online softmax's own
rescaling (memra-engine 0.130.0 src/forward.rs, ``Model::forward``, SDPA block: one
softmax over each row's visible keys).  With at most 4 key chunks an item, the item's
last workgroup to finish merges them in place (arrival counters in the workspace, tagged
per call); with more, ``attn_combine_kernel`` merges them in a second launch.  Each case
reads the path it takes from the library's plan report (``pfa_attn_plan``), so a change
of the split rules cannot move a case to the other path unnoticed.

Also: one workspace, filled with a byte pattern first (stale counters), shared by calls of
different shapes and paths in a row, each compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity, assert_q8_parity, eps32
from tests.test_gpu_chunk import Case, _chunk_gpu, _chunk_ref, _fused_gpu, _fused_ref

pytestmark = pytest.mark.gpu

IN_PLACE, COMBINE = "in place", "combine"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _check(prec):
    return assert_f32_parity if prec == "f32" else assert_bf16_parity


def _path(entry, q_lens, kv_lens, H, Hkv, d, prec):
    q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    k = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    p = pfa.attn_plan(entry, T_q=int(q[-1]), T_kv=int(k[-1]), n_head=H, n_head_kv=Hkv,
                      head_dim=d, rope_dim=d, precision=prec, q_offsets=q, kv_offsets=k)
    assert p["max_key_chunks"] > 1, "the case must split its keys"
    return IN_PLACE if p["merge_in_place"] else COMBINE


# ---- prefill (gqa_prefill_attn, qk_prep_attn)

PREFILL = [  # name, sequence lengths, H, Hkv, d, precisions
    ("t512", (512,), 16, 8, 128, ("f32", "bf16x3")),
    ("t2048", (2048,), 16, 8, 128, ("bf16",)),
    ("t2048_d64", (2048,), 8, 2, 64, ("f32", "bf16", "bf16x3", "f16")),
    ("packed", (300, 1500, 40), 8, 4, 128, ("f32", "bf16x3")),
]
_prefill_refs = {}


def _prefill_case(name, lens, H, Hkv, d):
    if name not in _prefill_refs:
        w = wl.Workload(f"merge_{name}", lens, H, Hkv, d, d, 1e6, 1e-6, seed=1600 + len(name))
        x = wl.make_inputs(w)
        qn, kn = oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=H, n_head_kv=Hkv, head_dim=d,
                                    rope_dim=d, rope_freq_base=float(np.float32(1e6)),
                                    rms_eps=eps32(w), seq_offsets=w.seq_offsets)
        qn, kn = qn.astype(np.float32), kn.astype(np.float32)
        ref = oracle.gqa_attn(qn, kn, x.v, n_head=H, n_head_kv=Hkv, head_dim=d,
                              scale=w.softmax_scale, seq_offsets=w.seq_offsets)
        ref_fused = oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, n_head=H, n_head_kv=Hkv,
                                        head_dim=d, rope_dim=d,
                                        rope_freq_base=float(np.float32(1e6)), rms_eps=eps32(w),
                                        scale=w.softmax_scale, seq_offsets=w.seq_offsets)
        _prefill_refs.clear()
        _prefill_refs[name] = (w, x, qn, kn, ref, ref_fused)
    return _prefill_refs[name]


@pytest.mark.parametrize("name,lens,H,Hkv,d,precs", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_merged_in_place(name, lens, H, Hkv, d, precs):
    w, x, qn, kn, ref, ref_fused = _prefill_case(name, lens, H, Hkv, d)
    for prec in precs:
        for entry, fused in ((pfa.ENTRY_PREFILL, False), (pfa.ENTRY_PREP, True)):
            assert _path(entry, lens, lens, H, Hkv, d, prec) == IN_PLACE
            what = (f"{'qk_prep_attn' if fused else 'gqa_prefill_attn'} {name}: T={w.T} "
                    f"seqs={w.n_seqs} H={H} Hkv={Hkv} d={d} {prec} (merged in place)")
            print(what, flush=True)
            if fused:
                out = pfa.qk_prep_attn(_dev(x.q), _dev(x.k), _dev(x.v), _dev(x.wq), _dev(x.wk),
                                       head_dim=d, rope_dim=d, rope_freq_base=1e6,
                                       rms_eps=1e-6, scale=w.softmax_scale, precision=prec,
                                       seq_offsets=w.seq_offsets)
            else:
                out = pfa.gqa_prefill_attn(_dev(qn), _dev(kn), _dev(x.v), head_dim=d,
                                           scale=w.softmax_scale, precision=prec,
                                           seq_offsets=w.seq_offsets)
            torch.cuda.synchronize()
            _check(prec)(out.cpu().numpy(), ref_fused if fused else ref, what)


# ---- chunks over a cached prefix (gqa_chunk_attn, qk_prep_chunk_attn), with gates

CHUNKS = [  # name, new rows, prefix rows, path
    ("rows1024_over2048", (1024,), (2048,), IN_PLACE),
    ("rows768_over1792", (768,), (1792,), COMBINE),
]
_chunk_cases = {}


def _chunk_case(name, lens, bases):
    if name not in _chunk_cases:
        _chunk_cases.clear()
        _chunk_cases[name] = Case(name, lens, bases, 16, 8, 128, 128, seed=1700 + len(name))
    return _chunk_cases[name]


@pytest.mark.parametrize("name,lens,bases,path", CHUNKS, ids=[c[0] for c in CHUNKS])
def test_chunk_merges(name, lens, bases, path):
    c = _chunk_case(name, lens, bases)
    full = [b + m for b, m in zip(bases, lens)]
    ref, ref_fused = _chunk_ref(c), _fused_ref(c)[0]
    r = np.random.default_rng(1800)
    gate = (2.0 * r.standard_normal((len(c.new), c.H))).astype(np.float32)
    ref_gated = _chunk_ref(c, gate=gate)
    for prec in ("f32", "bf16", "bf16x3"):
        assert _path(pfa.ENTRY_CHUNK, lens, full, c.H, c.Hkv, c.d, prec) == path
        assert _path(pfa.ENTRY_CHUNK_PREP, lens, full, c.H, c.Hkv, c.d, prec) == path
        _check(prec)(_chunk_gpu(c, prec), ref, c.label("gqa_chunk_attn", prec) + f" ({path})")
        _check(prec)(_chunk_gpu(c, prec, gate=gate), ref_gated,
                     c.label("gqa_chunk_attn", prec) + f" gate/head ({path})")
        got = _fused_gpu(c, prec)[0]
        _check(prec)(got, ref_fused, c.label("qk_prep_chunk_attn", prec) + f" ({path})")


# ---- the 8-bit store (gqa_attn_q8)

Q8 = [("rows1024_over2048", 1024, 2048, IN_PLACE), ("rows768_over1792", 768, 1792, COMBINE)]


@pytest.mark.parametrize("name,n_new,base,path", Q8, ids=[c[0] for c in Q8])
def test_q8_merges(name, n_new, base, path):
    H, Hkv, d = 16, 8, 128
    assert _path(pfa.ENTRY_Q8, [n_new], [base + n_new], H, Hkv, d, "bf16") == path
    q_offs = np.array([0, n_new], dtype=np.int32)
    kv_offs = np.array([0, base + n_new], dtype=np.int32)
    qc, qs = wl.q8_store(n_new, H, d, 1901)
    kc, ks = wl.q8_store(base + n_new, Hkv, d, 1902)
    vc, vs = wl.q8_store(base + n_new, Hkv, d, 1903)
    print(f"gqa_attn_q8 {name}: T_q={n_new} T_kv={base + n_new} H={H} Hkv={Hkv} ({path})",
          flush=True)
    out = pfa.gqa_attn_q8(_dev(qc), _dev(qs), _dev(kc), _dev(ks), _dev(vc), _dev(vs),
                          head_dim=d, scale=d ** -0.5, q_offsets=q_offs, kv_offsets=kv_offs)
    torch.cuda.synchronize()
    ref = oracle.q8_chunk_attn(qc, qs, kc, ks, vc, vs, n_head=H, n_head_kv=Hkv, head_dim=d,
                               scale=d ** -0.5, q_offsets=q_offs, kv_offsets=kv_offs)
    assert_q8_parity(out.cpu().numpy(), ref, f"gqa_attn_q8 {name} ({path})")


# ---- one workspace, stale counters, calls of different shapes in a row

def test_workspace_shared_by_calls_in_a_row():
    """A workspace filled with 0xC3 bytes (every counter word a stale, foreign value),
    then used by in-place merges of two shapes whose counters overlap, a combine-path
    call that overwrites them with partial results, and the first shape again: each
    output is compared with the oracle."""
    a = _prefill_case("t512", (512,), 16, 8, 128)
    wa, xa, qa, ka, refa, _ = a
    c = _chunk_case("rows768_over1792", (768,), (1792,))
    refc = _chunk_ref(c)
    # the second prefill shape: the packed sequences (its own oracle output)
    wb = wl.Workload("merge_ws_b", (200, 700), 16, 8, 128, 128, 1e6, 1e-6, seed=1950)
    xb = wl.make_inputs(wb)
    qb, kb = oracle.qknorm_rope(xb.q, xb.k, xb.wq, xb.wk, n_head=16, n_head_kv=8, head_dim=128,
                                rope_dim=128, rope_freq_base=float(np.float32(1e6)),
                                rms_eps=eps32(wb), seq_offsets=wb.seq_offsets)
    qb, kb = qb.astype(np.float32), kb.astype(np.float32)
    refb = oracle.gqa_attn(qb, kb, xb.v, n_head=16, n_head_kv=8, head_dim=128,
                           scale=wb.softmax_scale, seq_offsets=wb.seq_offsets)
    assert _path(pfa.ENTRY_PREFILL, (200, 700), (200, 700), 16, 8, 128, "f32") == IN_PLACE
    need = max(pfa.workspace_bytes(512, 16, 8, 128, "f32"),
               pfa.workspace_bytes(900, 16, 8, 128, "f32", seq_offsets=wb.seq_offsets),
               pfa.chunk_workspace_bytes(len(c.new), c.w.T, 16, 8, 128, "f32",
                                         q_offsets=c.q_offs, kv_offsets=c.kv_offs))
    ws = torch.full((need,), 0xC3, dtype=torch.uint8, device="cuda:0")
    calls = [
        ("gqa_prefill_attn t512 f32", lambda: pfa.gqa_prefill_attn(
            _dev(qa), _dev(ka), _dev(xa.v), head_dim=128, scale=wa.softmax_scale,
            workspace=ws), refa),
        ("gqa_prefill_attn packed 200+700 f32", lambda: pfa.gqa_prefill_attn(
            _dev(qb), _dev(kb), _dev(xb.v), head_dim=128, scale=wb.softmax_scale,
            seq_offsets=wb.seq_offsets, workspace=ws), refb),
        ("gqa_chunk_attn 768 over 1792 f32 (combine)", lambda: pfa.gqa_chunk_attn(
            _dev(c.q_prep), _dev(c.k_cache), _dev(c.v_cache), head_dim=128,
            scale=c.w.softmax_scale, q_offsets=c.q_offs, kv_offsets=c.kv_offs,
            workspace=ws), refc),
        ("gqa_prefill_attn t512 f32 again", lambda: pfa.gqa_prefill_attn(
            _dev(qa), _dev(ka), _dev(xa.v), head_dim=128, scale=wa.softmax_scale,
            workspace=ws), refa),
    ]
    for what, call, ref in calls:
        print(what, flush=True)
        out = call()
        torch.cuda.synchronize()
        assert_f32_parity(out.cpu().numpy(), ref, what)
