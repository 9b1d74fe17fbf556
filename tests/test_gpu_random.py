"""GPU parity over seeded random configurations of every entry point, against the oracle:
packed sequences with and without cached prefixes (empty ones included), several head
geometries, head_dim 64 and 128, rotary widths d, d/2 and others, causal or not, sliding
windows, gated outputs -- through qknorm_rope, the prefill entries (f32 / bf16 / bf16x3 / f16,
fused with k_rot_out), the chunk entries, the fused chunk entry and the 8-bit entries.  Each case is
drawn from its own seed (printed first), so a failure names it.
Tolerances: the f32 gate, the bf16 gate, and for the 8-bit path the bf16 gate with its
relative-L2 bound."""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity, assert_q8_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GEOMS = [(4, 2), (8, 2), (8, 8), (16, 4), (6, 2), (12, 4)]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def draw(seed):
    """One configuration: sequences, geometry, flags."""
    r = np.random.default_rng(seed)
    n_seqs = int(r.integers(1, 5))
    lens = [int(r.integers(0, 260)) for _ in range(n_seqs)]
    if sum(lens) == 0:
        lens[0] = 1
    bases = [int(r.integers(0, 400)) if r.random() < 0.6 else 0 for _ in range(n_seqs)]
    H, Hkv = GEOMS[int(r.integers(0, len(GEOMS)))]
    d = 128 if r.random() < 0.7 else 64
    n = [d, d // 2, 2 * int(r.integers(1, d // 2))][int(r.integers(0, 3))]
    causal = bool(r.random() < 0.8)
    window = int(r.integers(1, 300)) if causal and r.random() < 0.3 else 0
    gate = ["none", "elem", "head"][int(r.integers(0, 3))]
    return dict(lens=lens, bases=bases, H=H, Hkv=Hkv, d=d, n=n, causal=causal, window=window,
                gate=gate, seed=seed)


def _offsets(c):
    q_offs = np.concatenate([[0], np.cumsum(c["lens"])]).astype(np.int32)
    full = [b + m for b, m in zip(c["bases"], c["lens"])]
    kv_offs = np.concatenate([[0], np.cumsum(full)]).astype(np.int32)
    new = np.concatenate([np.arange(kv_offs[s] + c["bases"][s], kv_offs[s + 1])
                          for s in range(len(full))]).astype(np.int64)
    return q_offs, kv_offs, new


def _gate(c, T_q, r):
    if c["gate"] == "none":
        return None
    cols = c["H"] * (c["d"] if c["gate"] == "elem" else 1)
    return (2.0 * r.standard_normal((T_q, cols))).astype(np.float32)


@pytest.mark.parametrize("seed", range(100, 124))
@pytest.mark.parametrize("entry", ["chunk_f32", "chunk_bf16", "chunk_bf16x3", "chunk_f16",
                                   "fused_f32", "fused_bf16", "fused_f16"])
def test_random_chunk_entries(seed, entry):
    c = draw(seed)
    q_offs, kv_offs, new = _offsets(c)
    H, Hkv, d, n = c["H"], c["Hkv"], c["d"], c["n"]
    T_kv = int(kv_offs[-1])
    T_q = int(q_offs[-1])
    w = wl.Workload(f"random_{seed}", tuple(int(x) for x in np.diff(kv_offs)), H, Hkv, d, n, 1e4,
                    1e-6, seed=seed)
    x = wl.make_inputs(w)
    r = np.random.default_rng(seed + 1)
    gate = _gate(c, T_q, r)
    prec = entry.split("_")[1]
    print(f"seed {seed} {entry}: {c}", flush=True)
    eps = float(np.float32(1e-6))
    qn, kn = oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=H, n_head_kv=Hkv, head_dim=d,
                                rope_dim=n, rope_freq_base=1e4, rms_eps=eps,
                                seq_offsets=kv_offs)
    scale = d ** -0.5
    if entry.startswith("chunk"):
        k_cache = kn.astype(np.float32)
        v_cache = x.v
        q_prep = qn[new].astype(np.float32)
        out = pfa.gqa_chunk_attn(_t(q_prep), _t(k_cache), _t(v_cache), head_dim=d, scale=scale,
                                 causal=c["causal"], window=c["window"], precision=prec,
                                 q_offsets=q_offs, kv_offsets=kv_offs,
                                 gate=None if gate is None else _t(gate))
        torch.cuda.synchronize()
        ref = oracle.chunk_attn(q_prep, k_cache, v_cache, n_head=H, n_head_kv=Hkv, head_dim=d,
                                scale=scale, causal=c["causal"], q_offsets=q_offs,
                                kv_offsets=kv_offs, window=c["window"], gate=gate)
    else:
        is_new = np.zeros(T_kv, bool)
        is_new[new] = True
        kc = np.where(is_new[:, None], 0.0, kn).astype(np.float32)
        vc = np.where(is_new[:, None], 0.0, x.v).astype(np.float32)
        out = pfa.qk_prep_chunk_attn(_t(x.q[new]), _t(x.k[new]), _t(x.v[new]), _t(x.wq),
                                     _t(x.wk), _t(kc), _t(vc), head_dim=d, rope_dim=n,
                                     rope_freq_base=1e4, rms_eps=1e-6, scale=scale,
                                     causal=c["causal"], window=c["window"], precision=prec,
                                     q_offsets=q_offs, kv_offsets=kv_offs,
                                     gate=None if gate is None else _t(gate))
        torch.cuda.synchronize()
        ref = oracle.qk_prep_chunk_attn(x.q[new], x.k[new], x.v[new], x.wq, x.wk, kc, vc,
                                        n_head=H, n_head_kv=Hkv, head_dim=d, rope_dim=n,
                                        rope_freq_base=1e4, rms_eps=eps, scale=scale,
                                        causal=c["causal"], q_offsets=q_offs,
                                        kv_offsets=kv_offs, window=c["window"], gate=gate)[0]
    got = out.cpu().numpy()
    if prec == "f32":
        assert_f32_parity(got, ref, f"seed {seed} {entry}")
    else:
        assert_bf16_parity(got, ref, f"seed {seed} {entry}")


@pytest.mark.parametrize("seed", range(200, 224))
@pytest.mark.parametrize("entry", ["store", "fused"])
def test_random_q8_entries(seed, entry):
    c = draw(seed)
    q_offs, kv_offs, new = _offsets(c)
    H, Hkv, d, n = c["H"], c["Hkv"], c["d"], c["n"]
    T_kv, T_q = int(kv_offs[-1]), int(q_offs[-1])
    r = np.random.default_rng(seed + 1)
    gate = _gate(c, T_q, r)
    scale = d ** -0.5
    print(f"seed {seed} q8 {entry}: {c}", flush=True)
    kc0, ks0 = wl.q8_store(T_kv, Hkv, d, seed + 2)
    vc0, vs0 = wl.q8_store(T_kv, Hkv, d, seed + 3)
    if entry == "store":
        qc, qs = wl.q8_store(T_q, H, d, seed + 4)
        out = pfa.gqa_attn_q8(_t(qc), _t(qs), _t(kc0), _t(ks0), _t(vc0), _t(vs0), head_dim=d,
                              scale=scale, causal=c["causal"], window=c["window"],
                              gate=None if gate is None else _t(gate), q_offsets=q_offs,
                              kv_offsets=kv_offs)
        torch.cuda.synchronize()
        ref = oracle.q8_chunk_attn(qc, qs, kc0, ks0, vc0, vs0, n_head=H, n_head_kv=Hkv,
                                   head_dim=d, scale=scale, causal=c["causal"],
                                   q_offsets=q_offs, kv_offsets=kv_offs, window=c["window"],
                                   gate=gate)
    else:
        w = wl.Workload(f"random_{seed}", tuple(int(x) for x in np.diff(kv_offs)), H, Hkv, d, n,
                        1e4, 1e-6, seed=seed)
        x = wl.make_inputs(w)
        out = pfa.qk_prep_attn_q8(_t(x.q[new]), _t(x.k[new]), _t(x.v[new]), _t(x.wq), _t(x.wk),
                                  _t(kc0), _t(ks0), _t(vc0), _t(vs0), head_dim=d, rope_dim=n,
                                  rope_freq_base=1e4, rms_eps=1e-6, scale=scale,
                                  causal=c["causal"], window=c["window"],
                                  gate=None if gate is None else _t(gate), q_offsets=q_offs,
                                  kv_offsets=kv_offs)
        torch.cuda.synchronize()
        ref = oracle.qk_prep_q8_attn(x.q[new], x.k[new], x.v[new], x.wq, x.wk, kc0, ks0, vc0,
                                     vs0, n_head=H, n_head_kv=Hkv, head_dim=d, rope_dim=n,
                                     rope_freq_base=1e4, rms_eps=float(np.float32(1e-6)),
                                     scale=scale, causal=c["causal"], q_offsets=q_offs,
                                     kv_offsets=kv_offs, window=c["window"], gate=gate)[0]
    assert_q8_parity(out.cpu().numpy(), ref, f"seed {seed} q8 {entry}")


def draw_prefill(seed):
    r = np.random.default_rng(seed)
    lens = [int(r.integers(0, 300)) for _ in range(int(r.integers(1, 6)))]
    if sum(lens) == 0:
        lens[0] = 1
    H, Hkv = GEOMS[int(r.integers(0, len(GEOMS)))]
    d = 128 if r.random() < 0.7 else 64
    n = [d, d // 2, 2 * int(r.integers(1, d // 2))][int(r.integers(0, 3))]
    return dict(lens=lens, H=H, Hkv=Hkv, d=d, n=n, causal=bool(r.random() < 0.8))


@pytest.mark.parametrize("seed", range(300, 324))
@pytest.mark.parametrize("entry", ["qknorm_rope", "prefill_f32", "prefill_bf16", "prefill_bf16x3",
                                   "prefill_f16", "prep_f32", "prep_bf16", "prep_f16"])
def test_random_prefill_entries(seed, entry):
    c = draw_prefill(seed)
    H, Hkv, d, n = c["H"], c["Hkv"], c["d"], c["n"]
    w = wl.Workload(f"random_{seed}", tuple(c["lens"]), H, Hkv, d, n, 1e6, 1e-6, seed=seed)
    x = wl.make_inputs(w)
    offs = w.seq_offsets
    eps = float(np.float32(1e-6))
    print(f"seed {seed} {entry}: {c}", flush=True)
    kw = dict(head_dim=d, rope_dim=n, rope_freq_base=1e6, rms_eps=1e-6, seq_offsets=offs)
    qn, kn = oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=H, n_head_kv=Hkv, head_dim=d,
                                rope_dim=n, rope_freq_base=1e6, rms_eps=eps, seq_offsets=offs)
    if entry == "qknorm_rope":
        gq, gk = pfa.qknorm_rope(_t(x.q), _t(x.k), _t(x.wq), _t(x.wk), **kw)
        torch.cuda.synchronize()
        assert_f32_parity(gq.cpu().numpy(), qn, f"seed {seed} qknorm_rope Q")
        assert_f32_parity(gk.cpu().numpy(), kn, f"seed {seed} qknorm_rope K")
        return
    prec = entry.split("_")[1]
    if entry.startswith("prefill"):
        q32, k32 = qn.astype(np.float32), kn.astype(np.float32)
        out = pfa.gqa_prefill_attn(_t(q32), _t(k32), _t(x.v), head_dim=d, scale=d ** -0.5,
                                   causal=c["causal"], precision=prec, seq_offsets=offs)
        torch.cuda.synchronize()
        ref = oracle.gqa_attn(q32, k32, x.v, n_head=H, n_head_kv=Hkv, head_dim=d,
                              scale=d ** -0.5, causal=c["causal"], seq_offsets=offs)
    else:
        k_rot = torch.empty(w.T, Hkv * d, device=DEV)
        out = pfa.qk_prep_attn(_t(x.q), _t(x.k), _t(x.v), _t(x.wq), _t(x.wk), scale=d ** -0.5,
                               causal=c["causal"], precision=prec, k_rot_out=k_rot, **kw)
        torch.cuda.synchronize()
        ref = oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, n_head=H, n_head_kv=Hkv,
                                  head_dim=d, rope_dim=n, rope_freq_base=1e6, rms_eps=eps,
                                  scale=d ** -0.5, causal=c["causal"], seq_offsets=offs)
        assert_f32_parity(k_rot.cpu().numpy(), kn, f"seed {seed} {entry} k_rot_out")
    got = out.cpu().numpy()
    if prec == "f32":
        assert_f32_parity(got, ref, f"seed {seed} {entry}")
    else:
        assert_bf16_parity(got, ref, f"seed {seed} {entry}")
