"""GPU parity at the library's packed-sequence limit (PFA_MAX_SEQS = 128), element by
element against the f64 oracle, through the C ABI.

128 sequences of seeded random lengths 0..300 (some empty, some of one row) exercise
the whole sequence table and work schedule the kernels receive by value: the 128-entry
offset tables, the longest-first segment decode over up to 128 segments, the bf16
workspace's per-sequence tile offsets, and positions restarting at every sequence
(multi-sequence rows as in memra-engine 0.101.0 src/spec.rs, `qwen35_tparallel_fa_layer`:
per-row positions and per-sequence K/V).  Every entry point that takes a sequence table
is run: prefill (f32, bf16, bf16x3, f16), fused prefill, chunks over cached prefixes of
random length (plain and fused), and the 8-bit store.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity, assert_q8_parity, eps32
from tests.test_gpu_chunk import Case, _chunk_gpu, _chunk_ref, _fused_gpu as _chunk_fused_gpu
from tests.test_gpu_chunk import _fused_ref as _chunk_fused_ref

pytestmark = pytest.mark.gpu

N_SEQS = 128


def _lens(seed, max_len=300):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=N_SEQS)
    lens[rng.choice(N_SEQS, size=8, replace=False)] = 0   # empty sequences
    lens[rng.choice(N_SEQS, size=4, replace=False)] = 1   # one-row sequences
    return tuple(int(x) for x in lens)


GEOMS = [(8, 2, 128, 128), (8, 4, 64, 64), (12, 4, 128, 64)]


def _workload(i):
    H, Hkv, d, n = GEOMS[i]
    return wl.Workload(f"seqs128_{i}", _lens(1300 + i), H, Hkv, d, n, 1e6, 1e-6, seed=1300 + i)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.mark.parametrize("i", range(len(GEOMS)))
def test_prefill_128_sequences(i):
    w = _workload(i)
    assert w.n_seqs == N_SEQS
    x = wl.make_inputs(w)
    qn, kn = oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=w.n_head, n_head_kv=w.n_head_kv,
                                head_dim=w.head_dim, rope_dim=w.rope_dim,
                                rope_freq_base=float(np.float32(w.rope_freq_base)),
                                rms_eps=eps32(w), seq_offsets=w.seq_offsets)
    qn, kn = qn.astype(np.float32), kn.astype(np.float32)
    ref = oracle.gqa_attn(qn, kn, x.v, n_head=w.n_head, n_head_kv=w.n_head_kv,
                          head_dim=w.head_dim, scale=w.softmax_scale, seq_offsets=w.seq_offsets)
    ref_fused = oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, n_head=w.n_head,
                                    n_head_kv=w.n_head_kv, head_dim=w.head_dim,
                                    rope_dim=w.rope_dim,
                                    rope_freq_base=float(np.float32(w.rope_freq_base)),
                                    rms_eps=eps32(w), scale=w.softmax_scale,
                                    seq_offsets=w.seq_offsets)
    for prec in ("f32", "bf16", "bf16x3", "f16"):
        print(f"gqa_prefill_attn {w.name}: T={w.T} seqs={w.n_seqs} H={w.n_head} "
              f"Hkv={w.n_head_kv} d={w.head_dim} {prec}", flush=True)
        out = pfa.gqa_prefill_attn(_dev(qn), _dev(kn), _dev(x.v), head_dim=w.head_dim,
                                   scale=w.softmax_scale, precision=prec,
                                   seq_offsets=w.seq_offsets)
        torch.cuda.synchronize()
        check = assert_f32_parity if prec == "f32" else assert_bf16_parity
        check(out.cpu().numpy(), ref, f"prefill {prec} {w.name}")
        print(f"qk_prep_attn {w.name}: n={w.rope_dim} {prec}", flush=True)
        out = pfa.qk_prep_attn(_dev(x.q), _dev(x.k), _dev(x.v), _dev(x.wq), _dev(x.wk),
                               head_dim=w.head_dim, rope_dim=w.rope_dim,
                               rope_freq_base=w.rope_freq_base, rms_eps=w.rms_eps,
                               scale=w.softmax_scale, precision=prec, seq_offsets=w.seq_offsets)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), ref_fused, f"fused {prec} {w.name}")


@pytest.mark.parametrize("i", range(len(GEOMS)))
def test_chunk_128_sequences(i):
    """New rows (random, some sequences none) over cached prefixes of random length."""
    H, Hkv, d, n = GEOMS[i]
    rng = np.random.default_rng(1400 + i)
    lens = _lens(1400 + i, max_len=120)
    bases = tuple(int(b) for b in rng.integers(0, 260, size=N_SEQS))
    c = Case(f"seqs128_{i}", lens, bases, H, Hkv, d, n, seed=1400 + i)
    assert c.w.n_seqs == N_SEQS
    ref = _chunk_ref(c)
    ref_fused, kref, _ = _chunk_fused_ref(c)
    for prec in ("f32", "bf16"):
        check = assert_f32_parity if prec == "f32" else assert_bf16_parity
        check(_chunk_gpu(c, prec), ref, c.label("gqa_chunk_attn", prec))
        got, kc, vc = _chunk_fused_gpu(c, prec)
        check(got, ref_fused, c.label("qk_prep_chunk_attn", prec))
        # the cache: new rows' rotated K (f32 gate), V copied, prefix rows untouched
        assert_f32_parity(kc[c.new], kref[c.new], c.label("qk_prep_chunk_attn cache K", prec))
        np.testing.assert_array_equal(vc[c.new], c.v_cache[c.new])
        np.testing.assert_array_equal(kc[~c.is_new], c.k_prefix[~c.is_new])


def test_q8_store_128_sequences():
    rng = np.random.default_rng(1500)
    lens = _lens(1500, max_len=150)
    bases = [int(b) for b in rng.integers(0, 200, size=N_SEQS)]
    full = [b + m for b, m in zip(bases, lens)]
    H, Hkv, d = 8, 2, 128
    q_offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kv_offs = np.concatenate([[0], np.cumsum(full)]).astype(np.int32)
    qc, qs = wl.q8_store(int(q_offs[-1]), H, d, 1501)
    kc, ks = wl.q8_store(int(kv_offs[-1]), Hkv, d, 1502)
    vc, vs = wl.q8_store(int(kv_offs[-1]), Hkv, d, 1503)
    print(f"gqa_attn_q8 seqs={N_SEQS} T_q={q_offs[-1]} T_kv={kv_offs[-1]}", flush=True)
    out = pfa.gqa_attn_q8(_dev(qc), _dev(qs), _dev(kc), _dev(ks), _dev(vc), _dev(vs),
                          head_dim=d, scale=d ** -0.5, q_offsets=q_offs, kv_offsets=kv_offs)
    torch.cuda.synchronize()
    ref = oracle.q8_chunk_attn(qc, qs, kc, ks, vc, vs, n_head=H, n_head_kv=Hkv, head_dim=d,
                               scale=d ** -0.5, q_offsets=q_offs, kv_offsets=kv_offs)
    assert_q8_parity(out.cpu().numpy(), ref, "gqa_attn_q8 128 sequences")
