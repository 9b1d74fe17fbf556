"""GPU parity of the chunk entry points, ``gqa_chunk_attn`` and ``qk_prep_chunk_attn``
(through the C ABI): new rows over a K/V cache that already holds each sequence's
earlier rows, against the f64 oracle's ``chunk_attn`` / ``qk_prep_chunk_attn``.

Inputs are whole sequences from the seeded workload generator; each sequence's first
``base`` rows play the cached prefix (its K normalised and rotated by the oracle, as a
cache keeps it, rounded to f32), the rest the new rows.  Element by element at small
sizes (tile-aligned and ragged prefixes, one new row, no prefix, packed sequences with
different prefixes, head_dim 64, a prefix long enough for the key split), and on
sampled rows at the benchmark's chunk shape (8192 cache rows, 1024 new).  The sliding
window (each row sees only the last ``window`` keys up to its own) is checked on the
same cases: windows on and off tile edges, of one key, across packed sequences, with
the key split, and a windowed prefill of 8192 rows on sampled rows; the gated output
(``out = O * sigmoid(gate)``, per element or per head) with and without the key split."""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity, errors

pytestmark = pytest.mark.gpu

# name: (new rows per sequence, cached rows before them, n_head, n_head_kv, head_dim, rope_dim)
CASES = {
    "tile_aligned": ((100,), (128,), 8, 2, 128, 128),
    "ragged_prefix": ((70,), (37,), 8, 2, 128, 128),
    "one_new_row": ((1,), (300,), 4, 2, 128, 128),
    "no_prefix": ((150,), (0,), 8, 2, 128, 128),
    "packed": ((50, 1, 130, 0), (20, 77, 0, 5), 8, 4, 128, 64),
    "d64": ((90,), (45,), 4, 2, 64, 64),
    "long_prefix": ((260,), (1500,), 16, 8, 128, 128),
    # a cache long enough that the bf16 kernel splits its keys too (>= 2048 keys)
    "split_prefix": ((64, 1), (4000, 2500), 8, 2, 128, 128),
}


class Case:
    """Whole sequences (prefix + new rows), their oracle-prepared Q/K, and the split."""

    def __init__(self, name, lens, bases, H, Hkv, d, n, seed=700):
        full = tuple(b + m for b, m in zip(bases, lens))
        self.w = wl.Workload(f"chunk_{name}", full, H, Hkv, d, n, 1e6, 1e-6, seed=seed)
        self.x = wl.make_inputs(self.w)
        self.H, self.Hkv, self.d, self.n = H, Hkv, d, n
        self.kv_offs = np.concatenate([[0], np.cumsum(full)]).astype(np.int32)
        self.q_offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        self.new = np.concatenate(
            [np.arange(self.kv_offs[s] + bases[s], self.kv_offs[s + 1]) for s in range(len(lens))]
        ).astype(np.int64)
        self.is_new = np.zeros(len(self.x.k), dtype=bool)
        self.is_new[self.new] = True
        self.eps = float(np.float32(1e-6))
        self.base_f = float(np.float32(1e6))
        qn, kn = oracle.qknorm_rope(self.x.q, self.x.k, self.x.wq, self.x.wk, n_head=H,
                                    n_head_kv=Hkv, head_dim=d, rope_dim=n,
                                    rope_freq_base=self.base_f, rms_eps=self.eps,
                                    seq_offsets=self.kv_offs)
        self.q_prep = qn[self.new].astype(np.float32)   # prepared new queries, as the GPU gets them
        self.k_cache = kn.astype(np.float32)             # the whole cache, prepared
        self.v_cache = self.x.v.astype(np.float32)
        # what the fused entry starts from: the prefix rows only (new rows zeroed)
        self.k_prefix = np.where(self.is_new[:, None], 0.0, self.k_cache).astype(np.float32)
        self.v_prefix = np.where(self.is_new[:, None], 0.0, self.v_cache).astype(np.float32)

    def label(self, entry, precision, causal=True):
        w = self.w
        return (f"{entry} {w.name}: T_q={len(self.new)} T_kv={w.T} H={self.H} Hkv={self.Hkv} "
                f"d={self.d} n={self.n} seqs={w.n_seqs} causal={causal} {precision}")


def _t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _chunk_gpu(c, precision, causal=True, window=0, gate=None):
    print(c.label("gqa_chunk_attn", precision, causal) + f" window={window}"
          + ("" if gate is None else f" gate{list(gate.shape)}"), flush=True)
    dev = torch.device("cuda:0")
    out = pfa.gqa_chunk_attn(_t(c.q_prep, dev), _t(c.k_cache, dev), _t(c.v_cache, dev),
                             head_dim=c.d, scale=c.w.softmax_scale, causal=causal,
                             window=window, precision=precision, q_offsets=c.q_offs,
                             kv_offsets=c.kv_offs,
                             gate=None if gate is None else _t(gate, dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _chunk_ref(c, causal=True, rows=None, window=0, gate=None):
    return oracle.chunk_attn(c.q_prep, c.k_cache, c.v_cache, n_head=c.H, n_head_kv=c.Hkv,
                             head_dim=c.d, scale=c.w.softmax_scale, causal=causal,
                             q_offsets=c.q_offs, kv_offsets=c.kv_offs, window=window,
                             gate=gate, rows=rows)


def _fused_gpu(c, precision, causal=True, window=0, gate=None):
    print(c.label("qk_prep_chunk_attn", precision, causal) + f" window={window}"
          + ("" if gate is None else f" gate{list(gate.shape)}"), flush=True)
    dev = torch.device("cuda:0")
    kc, vc = _t(c.k_prefix, dev), _t(c.v_prefix, dev)
    out = pfa.qk_prep_chunk_attn(_t(c.x.q[c.new], dev), _t(c.x.k[c.new], dev),
                                 _t(c.x.v[c.new], dev), _t(c.x.wq, dev), _t(c.x.wk, dev), kc, vc,
                                 head_dim=c.d, rope_dim=c.n, rope_freq_base=1e6, rms_eps=1e-6,
                                 scale=c.w.softmax_scale, causal=causal, window=window,
                                 precision=precision, q_offsets=c.q_offs, kv_offsets=c.kv_offs,
                                 gate=None if gate is None else _t(gate, dev))
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()


def _fused_ref(c, causal=True, rows=None, window=0, gate=None):
    return oracle.qk_prep_chunk_attn(c.x.q[c.new], c.x.k[c.new], c.x.v[c.new], c.x.wq, c.x.wk,
                                     c.k_prefix, c.v_prefix, n_head=c.H, n_head_kv=c.Hkv,
                                     head_dim=c.d, rope_dim=c.n, rope_freq_base=c.base_f,
                                     rms_eps=c.eps, scale=c.w.softmax_scale, causal=causal,
                                     q_offsets=c.q_offs, kv_offsets=c.kv_offs, window=window,
                                     gate=gate, rows=rows)


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    return Case(request.param, *CASES[request.param])


@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3", "f16"])
def test_chunk_attn_matches_oracle(case, precision):
    got = _chunk_gpu(case, precision)
    ref = _chunk_ref(case)
    if precision == "f32":
        assert_f32_parity(got, ref, case.label("gqa_chunk_attn", precision))
    else:
        assert_bf16_parity(got, ref, case.label("gqa_chunk_attn", precision))


@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3", "f16"])
def test_prep_chunk_attn_matches_oracle_and_fills_the_cache(case, precision):
    got, kc, vc = _fused_gpu(case, precision)
    ref, kref, vref = _fused_ref(case)
    what = case.label("qk_prep_chunk_attn", precision)
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)
    # the new rows' rotated K in f32 (the K the f32 QK-norm + RoPE path writes), the
    # values copied exactly, the prefix rows untouched
    max_abs, rel = errors(kc[case.new], kref[case.new])
    print(f"{what} cache K: max|err| {max_abs:.3e}  rel L2 {rel:.3e}", flush=True)
    assert max_abs <= 1e-5 and rel <= 2e-6
    np.testing.assert_array_equal(vc[case.new], case.v_cache[case.new])
    keep = ~case.is_new
    np.testing.assert_array_equal(kc[keep], case.k_prefix[keep])
    np.testing.assert_array_equal(vc[keep], case.v_prefix[keep])


def test_chunk_without_prefix_is_prefill_bit_exact():
    # nothing cached before: the chunk entry runs the prefill kernels on the same tables
    c = Case("no_prefix", *CASES["no_prefix"])
    dev = torch.device("cuda:0")
    for precision in ("f32", "bf16"):
        a = _chunk_gpu(c, precision)
        print(f"gqa_prefill_attn {c.w.name}: T={c.w.T} {precision}", flush=True)
        b = pfa.gqa_prefill_attn(_t(c.q_prep, dev), _t(c.k_cache, dev), _t(c.v_cache, dev),
                                 head_dim=c.d, scale=c.w.softmax_scale, precision=precision)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(a, b.cpu().numpy())


def test_chunk_without_prefix_pairs_like_prefill():
    """1536 rows, nothing cached, 32/8 heads of 128: the f32 prefill plan pairs query blocks
    (one workgroup per CU) in place of a split into long key chunks, and the chunk entry --
    whose call is prefill -- takes the same plan, so the two agree bit for bit; the gated
    chunk output and the fused chunk entry on that plan match the oracle on sampled rows."""
    c = Case("no_prefix_1536", (1536,), (0,), 32, 8, 128, 128, seed=702)
    kw = dict(T_q=1536, n_head=32, n_head_kv=8, head_dim=128)
    offs = dict(q_offsets=[0, 1536], kv_offsets=[0, 1536])
    pp = pfa.attn_plan(pfa.ENTRY_PREFILL, **kw)
    pc = pfa.attn_plan(pfa.ENTRY_CHUNK, T_kv=1536, **kw, **offs)
    pf = pfa.attn_plan(pfa.ENTRY_CHUNK_PREP, T_kv=1536, **kw, **offs)
    assert pp["paired"] == pc["paired"] == pf["paired"] == 1
    assert pp["kernels"] == pc["kernels"] == "attn_f32_kernel<128,false,true,false>"
    dev = torch.device("cuda:0")
    a = _chunk_gpu(c, "f32")
    print(f"gqa_prefill_attn {c.w.name}: T={c.w.T} f32 (paired)", flush=True)
    b = pfa.gqa_prefill_attn(_t(c.q_prep, dev), _t(c.k_cache, dev), _t(c.v_cache, dev),
                             head_dim=c.d, scale=c.w.softmax_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, b.cpu().numpy())
    rng = np.random.default_rng(703)
    rows = np.unique(np.concatenate([[0, 31, 32, 767, 768, 1535],
                                     rng.integers(0, 1536, 40)])).astype(np.int64)
    assert_f32_parity(a[rows], _chunk_ref(c, rows=rows), c.label("gqa_chunk_attn", "f32") +
                      " (paired), sampled rows")
    gate = (2.0 * rng.standard_normal((1536, 32))).astype(np.float32)
    g = _chunk_gpu(c, "f32", gate=gate)
    assert_f32_parity(g[rows], _chunk_ref(c, rows=rows, gate=gate),
                      c.label("gqa_chunk_attn", "f32") + " (paired, gate per head), sampled rows")
    f, kc, vc = _fused_gpu(c, "f32")
    assert_f32_parity(f[rows], _fused_ref(c, rows=rows)[0],
                      c.label("qk_prep_chunk_attn", "f32") + " (paired), sampled rows")


@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_chunk_non_causal(precision):
    c = Case("packed_nc", *CASES["packed"], seed=701)
    got = _chunk_gpu(c, precision, causal=False)
    ref = _chunk_ref(c, causal=False)
    what = c.label("gqa_chunk_attn", precision, causal=False)
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)


@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_chunk_benchmark_shape_sampled_rows(precision):
    # 8192 cache rows per the 8B-like heads, the last 1024 new: the launch the benchmark
    # times; 24 query rows spread over the block are checked against the oracle
    c = Case("bench", (1024,), (7168,), 32, 8, 128, 128, seed=702)
    rows = np.linspace(0, 1023, 24).astype(np.int64)
    got, _, _ = _fused_gpu(c, precision)
    ref = _fused_ref(c, rows=rows)[0]
    what = c.label("qk_prep_chunk_attn", precision) + " (sampled rows)"
    if precision == "f32":
        assert_f32_parity(got[rows], ref, what)
    else:
        assert_bf16_parity(got[rows], ref, what)


WINDOWS = [("no_prefix", 64), ("no_prefix", 100), ("ragged_prefix", 1), ("packed", 50),
           ("long_prefix", 300), ("tile_aligned", 128), ("d64", 500)]


@pytest.mark.parametrize("name,window", WINDOWS, ids=[f"{n}-w{w}" for n, w in WINDOWS])
@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_chunk_window_matches_oracle(name, window, precision):
    c = Case(name, *CASES[name])
    got = _chunk_gpu(c, precision, window=window)
    ref = _chunk_ref(c, window=window)
    what = c.label("gqa_chunk_attn", precision) + f" window={window}"
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)
    got, _, _ = _fused_gpu(c, precision, window=window)
    ref = _fused_ref(c, window=window)[0]
    what = c.label("qk_prep_chunk_attn", precision) + f" window={window}"
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)


@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_windowed_prefill_sampled_rows(precision):
    # 8192 rows, no prefix, a window of 1000 keys: the chunk entry as a windowed prefill
    c = Case("win_prefill", (8192,), (0,), 32, 8, 128, 128, seed=703)
    rows = np.concatenate([np.arange(0, 8), np.linspace(990, 8191, 20)]).astype(np.int64)
    got = _chunk_gpu(c, precision, window=1000)
    ref = _chunk_ref(c, rows=rows, window=1000)
    what = c.label("gqa_chunk_attn", precision) + " window=1000 (sampled rows)"
    if precision == "f32":
        assert_f32_parity(got[rows], ref, what)
    else:
        assert_bf16_parity(got[rows], ref, what)


GATES = [("tile_aligned", False), ("long_prefix", True), ("packed", False), ("no_prefix", True)]


@pytest.mark.parametrize("name,per_head", GATES,
                         ids=[f"{n}-{'head' if h else 'elem'}" for n, h in GATES])
@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_chunk_gated_output(name, per_head, precision):
    # out = O * sigmoid(gate), per element or per head; long_prefix splits its keys, so
    # its gate is applied where the combine step stores the rows
    c = Case(name, *CASES[name])
    r = np.random.default_rng(900 + len(name))
    T_q = len(c.new)
    gate = (2.0 * r.standard_normal((T_q, c.H if per_head else c.H * c.d))).astype(np.float32)
    got = _chunk_gpu(c, precision, gate=gate)
    ref = _chunk_ref(c, gate=gate)
    what = c.label("gqa_chunk_attn", precision) + (" gate/head" if per_head else " gate/elem")
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)
    got, _, _ = _fused_gpu(c, precision, gate=gate, window=64 if name == "packed" else 0)
    ref = _fused_ref(c, gate=gate, window=64 if name == "packed" else 0)[0]
    what = c.label("qk_prep_chunk_attn", precision) + (" gate/head" if per_head else " gate/elem")
    if precision == "f32":
        assert_f32_parity(got, ref, what)
    else:
        assert_bf16_parity(got, ref, what)
