"""GPU parity of the 8-bit quantised session (through the C ABI): ``pfa_quantize_rows``,
``gqa_attn_q8`` and ``qk_prep_attn_q8`` against the oracle's ``quant_rows``,
``q8_chunk_attn`` and ``qk_prep_q8_attn`` (needle-core v3/model.rs: Q, K and V quantised
per (token, head) with 8 bits after RoPE; attention through the int8 store).

* Quantisation is integer work: codes and scales must match the oracle bit for bit on
  the same f32 rows (both take the decision in IEEE single precision).
* Attention through a store: the stores come from the seeded generator (codes shaped like
  quantised unit-variance rows, a +-127 code in every row, scales near 0.022), element
  by element at small sizes (prefill, ragged and tile-aligned prefixes, one new row,
  packed sequences, head_dim 64, a long prefix that takes the key split), non-causal, a
  sliding window and a gated output; the tolerance is the bf16 path's max-abs gate plus a
  relative-L2 bound of 4e-3, since V is dequantised to bf16 and the weights are rounded to
  bf16 (2^-9 relative each; the integer scores are exact).
* The fused step: raw rows normalised and rotated, quantised and appended to the store.
  V codes and scales are exact; a Q or K code may differ by one from the oracle's only
  where the oracle's value / scale lies within 1e-3 of a rounding tie (the two sides
  normalise and rotate with different rounding), and K scales agree to a few ulp.  At
  the benchmark's shape (8192 rows, 32/8 heads) the output is checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_q8_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ---------------------------------------------------------------------------
# pfa_quantize_rows

@pytest.mark.parametrize("rows,row_len,mag", [
    (4096, 128, 1.0), (3000, 64, 1e-3), (257, 1000, 37.0), (999, 17, 1.0), (64, 128, 1e-30),
    (1, 1, 5.0)])
def test_quantize_rows_bit_exact(rows, row_len, mag):
    print(f"pfa_quantize_rows rows={rows} row_len={row_len} mag={mag}", flush=True)
    r = np.random.default_rng(rows + row_len)
    x = (r.standard_normal((rows, row_len)) * mag *
         np.exp(r.standard_normal((rows, 1)))).astype(np.float32)
    x[::7] = 0.0                                   # rows of zeros
    if row_len > 1:
        x[1::11, 0] = np.float32(2.5) * x[1::11, 1]    # ties show up where they can
    c_ref, s_ref, d_ref = oracle.quant_rows(x, row_len)
    xd = _t(x)
    fq = torch.empty_like(xd)
    codes, scales = pfa.quantize_rows(xd, row_len, x_fq=fq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(fq.cpu().numpy(), d_ref)
    # in place, as the session quantises its activations
    codes2, scales2 = pfa.quantize_rows(xd, row_len, x_fq=xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xd.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(codes2.cpu().numpy(), c_ref)


# ---------------------------------------------------------------------------
# gqa_attn_q8 over generated stores

# name: (new rows per sequence, rows stored before them, n_head, n_head_kv, head_dim)
CASES = {
    "prefill": ((300,), (0,), 8, 2, 128),
    "tile_aligned": ((100,), (128,), 8, 2, 128),
    "ragged_prefix": ((70,), (37,), 8, 2, 128),
    "one_new_row": ((1,), (300,), 4, 2, 128),
    "packed": ((50, 1, 130, 0), (20, 77, 0, 5), 8, 4, 128),
    "d64": ((90,), (45,), 4, 2, 64),
    "long_prefix": ((260,), (1500,), 16, 8, 128),
    "mha": ((200,), (60,), 4, 4, 128),
    "group8": ((130,), (70,), 16, 2, 128),
}


class Store:
    """Generated 8-bit stores of a chunk case."""

    def __init__(self, name, lens, bases, H, Hkv, d, seed=900):
        full = [b + m for b, m in zip(bases, lens)]
        self.name, self.H, self.Hkv, self.d = name, H, Hkv, d
        self.q_offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        self.kv_offs = np.concatenate([[0], np.cumsum(full)]).astype(np.int32)
        T_q, T_kv = int(self.q_offs[-1]), int(self.kv_offs[-1])
        self.qc, self.qs = wl.q8_store(T_q, H, d, seed)
        self.kc, self.ks = wl.q8_store(T_kv, Hkv, d, seed + 1)
        self.vc, self.vs = wl.q8_store(T_kv, Hkv, d, seed + 2)
        self.scale = d ** -0.5

    def gpu(self, causal=True, window=0, gate=None):
        print(f"gqa_attn_q8 {self.name}: T_q={self.q_offs[-1]} T_kv={self.kv_offs[-1]} "
              f"H={self.H} Hkv={self.Hkv} d={self.d} seqs={len(self.q_offs) - 1} "
              f"causal={causal} window={window} gate={None if gate is None else gate.shape}",
              flush=True)
        out = pfa.gqa_attn_q8(_t(self.qc), _t(self.qs), _t(self.kc), _t(self.ks), _t(self.vc),
                              _t(self.vs), head_dim=self.d, scale=self.scale, causal=causal,
                              window=window, gate=None if gate is None else _t(gate),
                              q_offsets=self.q_offs, kv_offsets=self.kv_offs)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def ref(self, causal=True, window=0, gate=None):
        return oracle.q8_chunk_attn(self.qc, self.qs, self.kc, self.ks, self.vc, self.vs,
                                    n_head=self.H, n_head_kv=self.Hkv, head_dim=self.d,
                                    scale=self.scale, causal=causal, q_offsets=self.q_offs,
                                    kv_offsets=self.kv_offs, window=window, gate=gate)


@pytest.mark.parametrize("name", list(CASES))
def test_q8_attention_parity(name):
    st = Store(name, *CASES[name])
    assert_q8_parity(st.gpu(), st.ref(), f"gqa_attn_q8 {name}")


@pytest.mark.parametrize("name", ["ragged_prefix", "packed"])
def test_q8_attention_non_causal(name):
    st = Store(name, *CASES[name])
    assert_q8_parity(st.gpu(causal=False), st.ref(causal=False), f"gqa_attn_q8 {name} nc")


@pytest.mark.parametrize("name,window", [("tile_aligned", 64), ("ragged_prefix", 1),
                                         ("packed", 33), ("long_prefix", 700)])
def test_q8_attention_window(name, window):
    st = Store(name, *CASES[name])
    assert_q8_parity(st.gpu(window=window), st.ref(window=window),
                       f"gqa_attn_q8 {name} window {window}")


@pytest.mark.parametrize("name,per_head", [("ragged_prefix", False), ("long_prefix", True),
                                           ("long_prefix", False)])
def test_q8_attention_gate(name, per_head):
    st = Store(name, *CASES[name])
    T_q = int(st.q_offs[-1])
    g = 2.0 * np.random.default_rng(5).standard_normal(
        (T_q, st.H) if per_head else (T_q, st.H * st.d)).astype(np.float32)
    assert_q8_parity(st.gpu(gate=g), st.ref(gate=g), f"gqa_attn_q8 {name} gate")


def test_q8_attention_zero_rows():
    # a query row of zero codes (scale 0) weighs its visible keys equally; zero K rows
    # (scale 0) score 0, zero V rows add nothing -- including a row's own key and the first
    # key of a tile
    st = Store("ragged_prefix", *CASES["ragged_prefix"])
    st.qc[5] = 0
    st.qs[5] = 0.0
    for r in (0, 37 + 5, 64, 100):
        st.kc[r] = 0
        st.ks[r] = 0.0
    for r in (1, 37 + 6, 64):
        st.vc[r] = 0
        st.vs[r] = 0.0
    got, ref = st.gpu(), st.ref()
    assert_q8_parity(got, ref, "gqa_attn_q8 zero rows")


# ---------------------------------------------------------------------------
# qk_prep_attn_q8: raw rows -> norm + RoPE -> 8-bit store -> attention

def _near_tie_ok(got_codes, ref_codes, x_ref, scales_ref, d, what):
    """Codes equal, except +-1 where the oracle's x / scale is within 1e-3 of a tie."""
    g = got_codes.astype(np.int64).reshape(-1, d)
    r = ref_codes.astype(np.int64).reshape(-1, d)
    bad = g != r
    if not bad.any():
        return
    assert np.abs(g - r).max() == 1, f"{what}: a code differs by more than one"
    ratio = x_ref.reshape(-1, d).astype(np.float64) / scales_ref.reshape(-1, 1)
    frac = np.abs(np.abs(ratio - np.floor(ratio)) - 0.5)
    assert np.all(frac[bad] < 1e-3), f"{what}: a code differs away from a rounding tie"
    assert bad.mean() < 1e-3, f"{what}: {bad.sum()} codes differ"


@pytest.mark.parametrize("lens,bases,H,Hkv,d,n", [
    ((300,), (0,), 8, 2, 128, 128), ((70,), (37,), 8, 2, 128, 128),
    ((50, 1, 130, 0), (20, 77, 0, 5), 8, 4, 128, 64), ((90,), (45,), 4, 2, 64, 64),
    ((260,), (1500,), 16, 8, 128, 128)])
def test_qk_prep_attn_q8_parity(lens, bases, H, Hkv, d, n):
    full = [b + m for b, m in zip(bases, lens)]
    w = wl.Workload("q8_prep", tuple(full), H, Hkv, d, n, 1e6, 1e-6, seed=950)
    x = wl.make_inputs(w)
    q_offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kv_offs = w.seq_offsets
    new = np.concatenate([np.arange(kv_offs[s] + bases[s], kv_offs[s + 1])
                          for s in range(len(lens))]).astype(np.int64)
    T_kv = w.T
    kc0, ks0 = wl.q8_store(T_kv, Hkv, d, 951)     # the rows stored before (prefix)
    vc0, vs0 = wl.q8_store(T_kv, Hkv, d, 952)
    print(f"qk_prep_attn_q8: lens={lens} bases={bases} H={H} Hkv={Hkv} d={d} n={n}",
          flush=True)
    kc, ks, vc, vs = _t(kc0), _t(ks0), _t(vc0), _t(vs0)
    out = pfa.qk_prep_attn_q8(_t(x.q[new]), _t(x.k[new]), _t(x.v[new]), _t(x.wq), _t(x.wk),
                              kc, ks, vc, vs, head_dim=d, rope_dim=n, rope_freq_base=1e6,
                              rms_eps=1e-6, scale=w.softmax_scale, q_offsets=q_offs,
                              kv_offsets=kv_offs)
    torch.cuda.synchronize()
    eps = float(np.float32(1e-6))
    ref, rkc, rks, rvc, rvs, rqc, rqs = oracle.qk_prep_q8_attn(
        x.q[new], x.k[new], x.v[new], x.wq, x.wk, kc0, ks0, vc0, vs0, n_head=H, n_head_kv=Hkv,
        head_dim=d, rope_dim=n, rope_freq_base=1e6, rms_eps=eps, scale=w.softmax_scale,
        q_offsets=q_offs, kv_offsets=kv_offs)
    gkc, gks, gvc, gvs = kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(), vs.cpu().numpy()
    old = np.ones(T_kv, bool)
    old[new] = False
    np.testing.assert_array_equal(gkc[old], kc0[old])     # the prefix rows are left alone
    np.testing.assert_array_equal(gvs[old], vs0[old])
    np.testing.assert_array_equal(gvc, rvc)               # V: quantised as given, exact
    np.testing.assert_array_equal(gvs, rvs)
    _, kn = oracle.qknorm_rope(x.q[new], x.k[new], x.wq, x.wk, n_head=H, n_head_kv=Hkv,
                               head_dim=d, rope_dim=n, rope_freq_base=1e6, rms_eps=eps,
                               seq_offsets=q_offs,
                               pos0=(kv_offs[1:] - kv_offs[:-1]) - (q_offs[1:] - q_offs[:-1]))
    np.testing.assert_allclose(gks[new], rks[new], rtol=4e-6, atol=0)
    _near_tie_ok(gkc[new], rkc[new], kn.astype(np.float32), rks[new], d, "K codes")
    assert_q8_parity(out.cpu().numpy(), ref, "qk_prep_attn_q8")


def test_qk_prep_attn_q8_bench_shape_sampled():
    # the benchmark's quantised-session step: one 8192-row sequence, 32/8 heads of 128,
    # prefill (nothing stored before); output rows sampled
    w = wl.Workload("prefill_8192", (8192,), 32, 8, 128, 128, 1e6, 1e-6, seed=0)
    x = wl.make_inputs(w)
    rows = wl.sample_rows(w, n_random=48, seed=3)
    print(f"qk_prep_attn_q8 prefill_8192 sampled rows={len(rows)}", flush=True)
    z8 = np.zeros((w.T, w.n_head_kv * w.head_dim), np.int8)
    zs = np.zeros((w.T, w.n_head_kv), np.float32)
    kc, ks, vc, vs = _t(z8), _t(zs), _t(z8), _t(zs)
    out = pfa.qk_prep_attn_q8(_t(x.q), _t(x.k), _t(x.v), _t(x.wq), _t(x.wk), kc, ks, vc, vs,
                              head_dim=128, rope_dim=128, rope_freq_base=1e6, rms_eps=1e-6,
                              scale=w.softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.qk_prep_q8_attn(x.q, x.k, x.v, x.wq, x.wk, z8, zs, z8, zs, n_head=32,
                                 n_head_kv=8, head_dim=128, rope_dim=128, rope_freq_base=1e6,
                                 rms_eps=float(np.float32(1e-6)), scale=w.softmax_scale,
                                 rows=rows)[0]
    assert_q8_parity(out.cpu().numpy()[rows], ref, "qk_prep_attn_q8 prefill_8192 sampled")


def test_qk_prep_attn_q8_mixed_workload_sampled():
    # the packed mixed-batch workload (8 sequences, positions restarting, 16/4 heads,
    # partial rotary 64 of 128, base 1e4) as one quantised prefill; output rows sampled
    w = wl.CONFIGS["mixed"]
    x = wl.make_inputs(w)
    rows = wl.sample_rows(w, n_random=24, seed=4)
    print(f"qk_prep_attn_q8 mixed T={w.T} seqs={w.n_seqs} sampled rows={len(rows)}", flush=True)
    offs = w.seq_offsets
    z8 = np.zeros((w.T, w.n_head_kv * w.head_dim), np.int8)
    zs = np.zeros((w.T, w.n_head_kv), np.float32)
    kc, ks, vc, vs = _t(z8), _t(zs), _t(z8), _t(zs)
    out = pfa.qk_prep_attn_q8(_t(x.q), _t(x.k), _t(x.v), _t(x.wq), _t(x.wk), kc, ks, vc, vs,
                              head_dim=w.head_dim, rope_dim=w.rope_dim,
                              rope_freq_base=w.rope_freq_base, rms_eps=w.rms_eps,
                              scale=w.softmax_scale, q_offsets=offs, kv_offsets=offs)
    torch.cuda.synchronize()
    ref, rkc, rks, rvc, rvs, _, _ = oracle.qk_prep_q8_attn(
        x.q, x.k, x.v, x.wq, x.wk, z8, zs, z8, zs, n_head=w.n_head, n_head_kv=w.n_head_kv,
        head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
        rms_eps=float(np.float32(w.rms_eps)), scale=w.softmax_scale, q_offsets=offs,
        kv_offsets=offs, rows=rows)
    np.testing.assert_array_equal(vc.cpu().numpy(), rvc)
    np.testing.assert_array_equal(vs.cpu().numpy(), rvs)
    assert_q8_parity(out.cpu().numpy()[rows], ref, "qk_prep_attn_q8 mixed sampled")


def test_q8_attention_chunk_bench_shape_sampled():
    # the benchmark's chunk shape through a generated store: 1024 new rows over 7168 stored
    # (8192 store rows, 32/8 heads of 128; the keys are split in two); output rows sampled
    T_q, T_kv, H, Hkv, d = 1024, 8192, 32, 8, 128
    qc, qs = wl.q8_store(T_q, H, d, 960)
    kc, ks = wl.q8_store(T_kv, Hkv, d, 961)
    vc, vs = wl.q8_store(T_kv, Hkv, d, 962)
    r = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 511, 1022, 1023],
                                     r.integers(0, T_q, 40)])).astype(np.int64)
    print(f"gqa_attn_q8 chunk 1024 over 7168 sampled rows={len(rows)}", flush=True)
    out = pfa.gqa_attn_q8(_t(qc), _t(qs), _t(kc), _t(ks), _t(vc), _t(vs), head_dim=d,
                          scale=d ** -0.5, q_offsets=[0, T_q], kv_offsets=[0, T_kv])
    torch.cuda.synchronize()
    ref = oracle.q8_chunk_attn(qc, qs, kc, ks, vc, vs, n_head=H, n_head_kv=Hkv, head_dim=d,
                               scale=d ** -0.5, q_offsets=[0, T_q], kv_offsets=[0, T_kv],
                               rows=rows)
    assert_q8_parity(out.cpu().numpy()[rows], ref, "gqa_attn_q8 chunk bench shape sampled")


def test_quantize_rows_ties_and_near_ties():
    # codes decided next to rounding ties: exact ties at scale 1 (ties to even), and values
    # within a few ulps of a tie at a scale that is not a power of two (the reciprocal
    # product alone could round the other way there)
    r = np.random.default_rng(17)
    rows = []
    for _ in range(64):                       # scale 1: largest magnitude 127, half-integers
        x = r.integers(-126, 126, 128).astype(np.float32) + np.float32(0.5)
        x[r.integers(0, 128)] = np.float32(127.0 * (1 if r.integers(0, 2) else -1))
        rows.append(x)
    for sc in (0.37, 0.0219, 3.3e-5, 1234.5):     # near ties at other scales
        sc32 = np.float32(sc)
        for _ in range(64):
            k = r.integers(-126, 126, 128).astype(np.float32)
            x = ((k + np.float32(0.5)) * sc32).astype(np.float32)
            ulps = r.integers(-3, 4, 128).astype(np.int32)
            x = (x.view(np.int32) + ulps).view(np.float32)
            x[0] = np.float32(127.0) * sc32          # the row's largest magnitude
            rows.append(x)
    x = np.stack(rows).astype(np.float32)
    print(f"pfa_quantize_rows ties: rows={len(x)}", flush=True)
    c_ref, s_ref, d_ref = oracle.quant_rows(x, 128)
    codes, scales = pfa.quantize_rows(_t(x), 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


def test_q8_attention_prefill_2048_sampled():
    # 2048 rows, 32/8 heads: one round of workgroups exactly fills the slots; sampled rows
    # against the oracle
    T, H, Hkv, d = 2048, 32, 8, 128
    qc, qs = wl.q8_store(T, H, d, 970)
    kc, ks = wl.q8_store(T, Hkv, d, 971)
    vc, vs = wl.q8_store(T, Hkv, d, 972)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 1023, 1024, 2046, 2047],
                                     np.random.default_rng(3).integers(0, T, 40)]))
    print(f"gqa_attn_q8 prefill T=2048 rows={len(rows)}", flush=True)
    out = pfa.gqa_attn_q8(_t(qc), _t(qs), _t(kc), _t(ks), _t(vc), _t(vs), head_dim=d,
                          scale=d ** -0.5)
    torch.cuda.synchronize()
    ref = oracle.q8_chunk_attn(qc, qs, kc, ks, vc, vs, n_head=H, n_head_kv=Hkv, head_dim=d,
                               scale=d ** -0.5, rows=rows)
    assert_q8_parity(out.cpu().numpy()[rows], ref, "gqa_attn_q8 prefill 2048")
