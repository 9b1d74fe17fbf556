"""GPU parity of ``gqa_prefill_attn`` and the fused ``qk_prep_attn`` (through the C ABI)
against the f64 oracle: element by element at sizes the oracle finishes in seconds
(several tiles plus ragged tails, group sizes, head sizes, rotary widths, paired items),
and the method's exact invariants.  The workloads at their full sizes are compared in
``test_gpu_full_parity.py``."""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity, eps32, errors

pytestmark = pytest.mark.gpu


def _dev(x, dev):
    return {n: torch.from_numpy(np.ascontiguousarray(getattr(x, n))).to(dev)
            for n in ("q", "k", "v", "wq", "wk")}


def _attn_gpu(w, t, precision="f32", causal=True):
    print(f"gqa_prefill_attn {w.name}: T={w.T} H={w.n_head} Hkv={w.n_head_kv} d={w.head_dim} "
          f"seqs={w.n_seqs} causal={causal} {precision}", flush=True)
    out = pfa.gqa_prefill_attn(t["q"], t["k"], t["v"], head_dim=w.head_dim,
                               scale=w.softmax_scale, causal=causal, precision=precision,
                               seq_offsets=w.seq_offsets)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _fused_gpu(w, t, precision="f32", causal=True, k_rot=None):
    print(f"qk_prep_attn {w.name}: T={w.T} H={w.n_head} Hkv={w.n_head_kv} d={w.head_dim} "
          f"n={w.rope_dim} seqs={w.n_seqs} causal={causal} {precision}", flush=True)
    out = pfa.qk_prep_attn(t["q"], t["k"], t["v"], t["wq"], t["wk"], head_dim=w.head_dim,
                           rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                           rms_eps=w.rms_eps, scale=w.softmax_scale, causal=causal,
                           precision=precision, seq_offsets=w.seq_offsets, k_rot_out=k_rot)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _attn_ref(w, x, rows=None, causal=True):
    return oracle.gqa_attn(x.q, x.k, x.v, n_head=w.n_head, n_head_kv=w.n_head_kv,
                           head_dim=w.head_dim, scale=w.softmax_scale, causal=causal,
                           seq_offsets=w.seq_offsets, rows=rows)


def _fused_ref(w, x, rows=None, causal=True, return_k_rot=False):
    return oracle.qk_prep_attn(x.q, x.k, x.v, x.wq, x.wk, n_head=w.n_head,
                               n_head_kv=w.n_head_kv, head_dim=w.head_dim,
                               rope_dim=w.rope_dim,
                               rope_freq_base=float(np.float32(w.rope_freq_base)),
                               rms_eps=eps32(w), scale=w.softmax_scale, causal=causal,
                               seq_offsets=w.seq_offsets, rows=rows, return_k_rot=return_k_rot)


# Small shapes, compared element by element: group sizes 1, 2, 4, 8 and 3 (odd split),
# head_dim 64 and 128, ragged sequence ends, empty and one-token sequences.
SMALL = [
    wl.Workload("g4_ragged", (300,), 8, 2, 128, 128, 1e6, 1e-6, seed=11),
    wl.Workload("g2_packed", (1, 33, 0, 64, 65, 97), 4, 2, 128, 128, 1e4, 1e-6, seed=12),
    wl.Workload("mha", (130,), 3, 3, 128, 128, 1e6, 1e-6, seed=13),
    wl.Workload("g8", (70, 41), 16, 2, 128, 64, 1e4, 1e-6, seed=14),
    wl.Workload("g3", (90,), 6, 2, 64, 64, 1e6, 1e-6, seed=15),
    wl.Workload("d64_g4", (31, 257), 8, 2, 64, 32, 1e6, 1e-6, seed=16, scale=0.125),
    # a rope_dim that is neither head_dim nor head_dim/2 (the kernels' general pairing)
    wl.Workload("rope96", (150, 70), 8, 2, 128, 96, 1e4, 1e-6, seed=17),
    wl.Workload("d64_rope48", (99,), 4, 2, 64, 48, 1e6, 1e-6, seed=18),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("causal", [True, False])
def test_attn_small_full_compare(gpu_device, w, causal):
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    assert_f32_parity(_attn_gpu(w, t, causal=causal), _attn_ref(w, x, causal=causal),
                      f"attn {w.name} causal={causal}")


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("causal", [True, False])
def test_fused_small_full_compare(gpu_device, w, causal):
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    assert_f32_parity(_fused_gpu(w, t, causal=causal), _fused_ref(w, x, causal=causal),
                      f"fused {w.name} causal={causal}")


def test_fused_k_rot_out_matches_oracle(gpu_device):
    w = wl.CONFIGS["mixed"].with_(seq_lens=(100, 1, 260, 31))
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    k_rot = torch.full_like(t["k"], float("nan"))
    got = _fused_gpu(w, t, k_rot=k_rot)
    ref, ref_k = _fused_ref(w, x, return_k_rot=True)
    assert_f32_parity(got, ref, "fused with k_rot_out")
    assert_f32_parity(k_rot.cpu().numpy(), ref_k, "k_rot_out")


def test_first_row_equals_v_bit_exact(gpu_device):
    """Each sequence's first causal row has one visible key of weight exactly 1."""
    w = wl.Workload("rows0", (5, 64, 1, 200), 8, 2, 128, 128, 1e6, 1e-6, seed=21)
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    got = _attn_gpu(w, t)
    for s in w.seq_offsets[:-1]:
        for h in range(w.n_head):
            kv = h // (w.n_head // w.n_head_kv)
            np.testing.assert_array_equal(got[s, h * 128:(h + 1) * 128],
                                          x.v[s, kv * 128:(kv + 1) * 128])


def test_future_perturbation_bit_exact(gpu_device):
    """Changing tokens >= j (Q, K and V) leaves every earlier row bit-identical."""
    w = wl.Workload("future", (333,), 8, 2, 128, 128, 1e6, 1e-6, seed=22)
    x = wl.make_inputs(w)
    a = _attn_gpu(w, _dev(x, gpu_device))
    j = 150
    x2 = wl.Inputs(x.q.copy(), x.k.copy(), x.v.copy(), x.wq, x.wk, x.outliers)
    x2.q[j:] *= -2
    x2.k[j:] += 1
    x2.v[j:] = 7
    b = _attn_gpu(w, _dev(x2, gpu_device))
    np.testing.assert_array_equal(a[:j], b[:j])
    assert not np.allclose(a[j:], b[j:])


def test_packed_equals_separate(gpu_device):
    w = wl.Workload("packed", (40, 1, 129, 64), 8, 2, 128, 64, 1e4, 1e-6, seed=23)
    x = wl.make_inputs(w)
    packed = _fused_gpu(w, _dev(x, gpu_device))
    offs = w.seq_offsets
    for s in range(w.n_seqs):
        a, b = int(offs[s]), int(offs[s + 1])
        ws = w.with_(seq_lens=(b - a,))
        xs = wl.Inputs(x.q[a:b], x.k[a:b], x.v[a:b], x.wq, x.wk, x.outliers[:0])
        alone = _fused_gpu(ws, _dev(xs, gpu_device))
        np.testing.assert_allclose(packed[a:b], alone, rtol=0, atol=1e-6)


def test_gqa_head_map_probe(gpu_device):
    """V[:, kv, :] = kv: query head h must return h // g."""
    w = wl.Workload("probe", (96,), 8, 2, 64, 64, 1e6, 1e-6, seed=24)
    x = wl.make_inputs(w)
    x.v = np.repeat(np.arange(2, dtype=np.float32), 64)[None, :].repeat(96, 0).copy()
    got = _attn_gpu(w, _dev(x, gpu_device))
    for h in range(8):
        np.testing.assert_allclose(got[:, h * 64:(h + 1) * 64], h // 4, atol=1e-6)


def test_zero_tokens_is_noop(gpu_device):
    z = torch.zeros((0, 256), device=gpu_device)
    zk = torch.zeros((0, 128), device=gpu_device)
    out = pfa.gqa_prefill_attn(z, zk, zk, head_dim=64, scale=0.125)
    torch.cuda.synchronize()
    assert out.numel() == 0


# ----------------------------------------------------------------------------- bf16 inputs
# The contract comparison is against the same f64 oracle on the unrounded f32 inputs
# (gate 2e-2 max abs); the rounding happens inside the kernel.

@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("causal", [True, False])
def test_attn_bf16_small(gpu_device, w, causal):
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    assert_bf16_parity(_attn_gpu(w, t, precision="bf16", causal=causal),
                       _attn_ref(w, x, causal=causal), f"attn bf16 {w.name} causal={causal}")


def _bf16_rounded_inputs(w, x, dtype=torch.bfloat16):
    """Q, K, V as the 16-bit kernel multiplies them: Q * (scale log2 e) rounded to bf16 (or
    ``dtype``, float16 for the f16 mode; then divided back), K and V rounded the same way
    -- for the oracle's comparison of what the mode computes."""
    c = np.float32(np.float32(w.softmax_scale) * np.float32(1.4426950408889634))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(
        torch.float64).numpy()
    q = bf((x.q * c).astype(np.float32)) / np.float64(c)
    return wl.Inputs(q, bf(x.k), bf(x.v), x.wq, x.wk, x.outliers)


# f16 mode: its roundings are those of Q, K, V and of the weights P, each to binary16
# (unit roundoff 2^-11).  Against the oracle on the f16-rounded inputs only the weights'
# rounding remains: the output is an exact weighted mean of V rows with weights off by a
# factor within 1 +- 2^-11 each, which moves it by at most 2^-11 (max V - min V) / (1 -
# 2^-11) (weights below binary16's normal range are off by at most 2^-25 absolute, against
# a sum of weights >= 1; that and the f32 accumulation get the 1e-4 allowance).
F16_U = 2.0 ** -11


def _f16_weight_bound(v):
    return F16_U * float(v.max() - v.min()) / (1.0 - F16_U) + 1e-4


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_attn_f16_small(gpu_device, w):
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    xr = _bf16_rounded_inputs(w, x, torch.float16)
    for causal in (True, False):
        got = _attn_gpu(w, t, precision="f16", causal=causal)
        assert_bf16_parity(got, _attn_ref(w, x, causal=causal), f"attn f16 {w.name} causal={causal}")
        max_abs, rel = errors(got, _attn_ref(w, xr, causal=causal))
        bound = _f16_weight_bound(x.v)
        print(f"attn f16 {w.name} causal={causal} vs oracle on f16-rounded inputs: "
              f"max|err| {max_abs:.3e} (bound {bound:.3e}) rel L2 {rel:.3e}", flush=True)
        assert max_abs <= bound


def test_attn_f16_first_row_is_rounded_v(gpu_device):
    """A first causal row has weight exactly 1 on one key: in the f16 mode the output is
    that key's V rounded to binary16 (and nothing else)."""
    w = wl.Workload("rows0_f16", (5, 64, 1, 200), 8, 2, 128, 128, 1e6, 1e-6, seed=32)
    x = wl.make_inputs(w)
    got = _attn_gpu(w, _dev(x, gpu_device), precision="f16")
    vh = x.v.astype(np.float16).astype(np.float32)
    for s in w.seq_offsets[:-1]:
        for h in range(w.n_head):
            kv = h // 4
            np.testing.assert_array_equal(got[s, h * 128:(h + 1) * 128],
                                          vh[s, kv * 128:(kv + 1) * 128])


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_attn_bf16x3_small(gpu_device, w):
    x = wl.make_inputs(w)
    assert_bf16_parity(_attn_gpu(w, _dev(x, gpu_device), precision="bf16x3"), _attn_ref(w, x),
                       f"attn bf16x3 {w.name}")


def test_attn_bf16_first_row_is_rounded_v(gpu_device):
    """A first causal row has weight exactly 1 on one key: the output is that key's V
    rounded to bf16 (and nothing else)."""
    w = wl.Workload("rows0_bf16", (5, 64, 1, 200), 8, 2, 128, 128, 1e6, 1e-6, seed=31)
    x = wl.make_inputs(w)
    got = _attn_gpu(w, _dev(x, gpu_device), precision="bf16")
    vb = torch.from_numpy(x.v).to(torch.bfloat16).to(torch.float32).numpy()
    for s in w.seq_offsets[:-1]:
        for h in range(w.n_head):
            kv = h // 4
            np.testing.assert_array_equal(got[s, h * 128:(h + 1) * 128],
                                          vb[s, kv * 128:(kv + 1) * 128])


# Short 16-bit inputs whose items fill at most a quarter of the slots cut each item's keys in
# two halves, merged in place by the item's second unit.  Ragged shapes on both branches of
# that rule: a half of at least 6 tiles (T = 700: 11 tiles, halves of 6 and 5; T = 1000:
# 16 tiles), and items filling at most an eighth of the slots (T = 600 with 8/4 heads:
# halves of 5 tiles).  Compared element by element with the oracle, causal and not, through
# the plain and the fused entry.
HALVES = [
    wl.Workload("halves_700", (700,), 16, 8, 128, 128, 1e6, 1e-6, seed=51),
    wl.Workload("halves_1000", (1000,), 16, 8, 128, 128, 1e6, 1e-6, seed=52),
    wl.Workload("halves_600_g2", (600,), 8, 4, 128, 128, 1e6, 1e-6, seed=53),
]


@pytest.mark.parametrize("w", HALVES, ids=[w.name for w in HALVES])
@pytest.mark.parametrize("precision", ["bf16", "f16"])
def test_attn_16bit_key_halves(gpu_device, w, precision):
    plan = pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=w.T, n_head=w.n_head, n_head_kv=w.n_head_kv,
                         head_dim=w.head_dim, causal=True, precision=precision,
                         q_offsets=np.asarray(w.seq_offsets, np.int32))
    n_tiles = -(-w.T // 64)
    assert plan["max_key_chunks"] == 2 and plan["merge_in_place"] == 1, plan
    assert plan["key_chunk_tiles"] == -(-n_tiles // 2), plan
    fplan = pfa.attn_plan(pfa.ENTRY_PREP, T_q=w.T, n_head=w.n_head, n_head_kv=w.n_head_kv,
                          head_dim=w.head_dim, rope_dim=w.rope_dim, causal=True,
                          precision=precision, q_offsets=np.asarray(w.seq_offsets, np.int32))
    assert fplan["max_key_chunks"] == 2 and fplan["merge_in_place"] == 1, fplan
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    for causal in (True, False):
        assert_bf16_parity(_attn_gpu(w, t, precision=precision, causal=causal),
                           _attn_ref(w, x, causal=causal),
                           f"attn {precision} {w.name} causal={causal}")
        assert_bf16_parity(_fused_gpu(w, t, precision=precision, causal=causal),
                           _fused_ref(w, x, causal=causal),
                           f"fused {precision} {w.name} causal={causal}")


# ----------------------------------------------------------------------------- fused, bf16
# qk_prep_attn with bf16 products: K is normalised and rotated in the staging kernel, Q in
# the attention kernel's prologue; compared with the fused f64 oracle on the raw inputs.

@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("precision", ["bf16", "bf16x3", "f16"])
def test_fused_bf16_small(gpu_device, w, precision):
    x = wl.make_inputs(w)
    for causal in (True, False):
        assert_bf16_parity(_fused_gpu(w, _dev(x, gpu_device), precision=precision, causal=causal),
                           _fused_ref(w, x, causal=causal),
                           f"fused {precision} {w.name} causal={causal}")


@pytest.mark.parametrize("precision", ["bf16", "bf16x3", "f16"])
def test_fused_bf16_k_rot_out_is_f32_exact_path(gpu_device, precision):
    """The rotated K copied out by the bf16 staging kernel is f32 and meets the f32 gates."""
    w = wl.CONFIGS["mixed"].with_(seq_lens=(128, 1, 300, 0, 77), name="mixed_small")
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    k_rot = torch.full_like(t["k"], float("nan"))
    got = _fused_gpu(w, t, precision=precision, k_rot=k_rot)
    ref, ref_k = _fused_ref(w, x, return_k_rot=True)
    assert_bf16_parity(got, ref, f"fused {precision} with k_rot_out")
    assert_f32_parity(k_rot.cpu().numpy(), ref_k, f"k_rot_out ({precision} staging)")


def test_fused_bf16_matches_unfused_chain(gpu_device):
    """qk_prep_attn(bf16) against qknorm_rope followed by gqa_prefill_attn(bf16)."""
    w = wl.CONFIGS["mixed"]
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    fused = _fused_gpu(w, t, precision="bf16")
    qn, kn = pfa.qknorm_rope(t["q"], t["k"], t["wq"], t["wk"], head_dim=w.head_dim,
                             rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
                             rms_eps=w.rms_eps, seq_offsets=w.seq_offsets)
    unf = pfa.gqa_prefill_attn(qn, kn, t["v"], head_dim=w.head_dim, scale=w.softmax_scale,
                               precision="bf16", seq_offsets=w.seq_offsets)
    torch.cuda.synchronize()
    assert_bf16_parity(fused, unf.cpu().numpy().astype(np.float64), "fused bf16 vs unfused bf16")


@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3", "f16"])
def test_row_max_covers_both_lane_halves(gpu_device, precision):
    """Keys whose index is 4..7 mod 8 score ~300 (log2 units) above the others.  The two
    lanes of a query hold those two key sets in the score registers; a row max taken
    over only one of them would make exp2 overflow to inf (NaN output)."""
    w = wl.Workload("halves", (64, 40), 2, 1, 64, 64, 1e6, 1e-6, seed=41, scale=1.0)
    T, d = w.T, w.head_dim
    rng = np.random.default_rng(41)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.tile((20.0 * u).astype(np.float32), (T, w.n_head))
    c = np.where(np.arange(T) % 8 >= 4, 10.0, 0.1)
    k = (c[:, None] * u[None, :] + 0.01 * rng.standard_normal((T, d))).astype(np.float32)
    v = rng.standard_normal((T, d)).astype(np.float32)
    x = wl.Inputs(q, k, v, np.ones(d, np.float32), np.ones(d, np.float32), np.zeros(0, np.int64))
    got = _attn_gpu(w, _dev(x, gpu_device), precision=precision)
    assert np.isfinite(got).all()
    ref = _attn_ref(w, x)
    if precision == "f32":
        # scores ~100x those of the workloads: f32 score rounding grows with them, so this
        # stress case gets 1e-4 (max abs and relative L2) rather than the workloads. gates
        max_abs, rel = errors(got, ref)
        print(f"row max over both halves f32: max|err| {max_abs:.3e} rel L2 {rel:.3e}", flush=True)
        assert max_abs <= 1e-4 and rel <= 1e-4
    else:
        # the scores are ~200 (natural units): bf16 inputs move them by ~1 (f16 ones by
        # ~0.1), so compare against the oracle on the rounded inputs (what those modes
        # promise)
        rounded = {"bf16": torch.bfloat16, "f16": torch.float16}
        assert_bf16_parity(got, _attn_ref(w, _bf16_rounded_inputs(w, x, rounded[precision]))
                           if precision in rounded else ref,
                           f"row max over both halves {precision}")


@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3", "f16"])
def test_running_max_moves_mid_row(gpu_device, precision):
    """The attention kernels keep a lazy running max: a tile moves it (and rescales the
    output and the sum) only when one of its scores passes it by more than 8 (log2 units).
    Here every query's component along a unit vector u is 3 (the rest N(0, 1/4)), keys are
    N(0, 1/4), and two keys carry +36.6 u and +68 u, scoring ~14 and ~26 log2 units where
    the others stay within ~2, so every row at or after key 150 moves its max in the middle
    of its key range, and again at key 260 (on a later tile than its first in both tile
    sizes: 32 keys in f32, 64 in the 16-bit kernels).  Scores stay within the long
    workload's range (its x8 outlier keys reach ~29), so the workload gates apply."""
    w = wl.Workload("late_max", (300,), 8, 2, 128, 128, 1e6, 1e-6, seed=43)
    T, d, H, Hkv = w.T, w.head_dim, w.n_head, w.n_head_kv
    rng = np.random.default_rng(43)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = 0.5 * rng.standard_normal((T, H, d))
    q += (3.0 - q @ u)[..., None] * u          # every query: component 3 along u
    k = 0.5 * rng.standard_normal((T, Hkv, d))
    spikes = {150: 36.6, 260: 68.0}
    for j, beta in spikes.items():
        k[j] += beta * u
    v = rng.standard_normal((T, Hkv, d))
    q, k, v = (a.reshape(T, -1).astype(np.float32) for a in (q, k, v))
    # the construction does what it says: for rows past each spike, the spike's score is
    # more than 8 above every key of the tiles before its own (f64, log2 units)
    sc = w.softmax_scale / np.log(2.0)
    qh = q.reshape(T, H, d).astype(np.float64)
    kh = k.reshape(T, Hkv, d).astype(np.float64)
    for j in spikes:
        for h in range(H):
            s = (qh[j:, h] @ kh[:, h // (H // Hkv)].T) * sc   # rows j.. against all keys
            first = (j // 64) * 64                             # the spike's 64-key tile
            assert (s[:, j] - s[:, :first].max(axis=1) > 8.0).all()
    x = wl.Inputs(q, k, v, np.ones(d, np.float32), np.ones(d, np.float32), np.zeros(0, np.int64))
    got = _attn_gpu(w, _dev(x, gpu_device), precision=precision)
    assert np.isfinite(got).all()
    ref = _attn_ref(w, x)
    if precision == "f32":
        assert_f32_parity(got, ref, "running max moved mid-row f32")
    else:
        rounded = {"bf16": torch.bfloat16, "f16": torch.float16}
        assert_bf16_parity(got, _attn_ref(w, _bf16_rounded_inputs(w, x, rounded[precision]))
                           if precision in rounded else ref,
                           f"running max moved mid-row {precision}")


def test_tensors_past_4gb(gpu_device):
    # One sequence whose K and V pass 4 GB each: 128 K/V heads of 128 dims (64 KiB a row),
    # T = 131071 rows, T * heads * head_dim just under 2^31 (the documented limit).  The
    # f32 kernel reads K/V tiles through 32-bit buffer resources; a resource sized to the
    # rest of the sequence wrapped past 4 GB and read key 65535 as zeros.  V of that key is
    # planted large so any such loss shows; rows on both sides of it are checked (f32 and
    # bf16).  Inputs are drawn on the GPU with a seeded torch generator.
    T, H, d = 131071, 128, 128
    assert T * H * d < 2 ** 31
    g = torch.Generator(device=gpu_device).manual_seed(4444)
    q = torch.randn(T, H * d, generator=g, device=gpu_device)
    k = torch.randn(T, H * d, generator=g, device=gpu_device)
    v = torch.randn(T, H * d, generator=g, device=gpu_device)
    v[65535] = 1000.0
    scale = d ** -0.5
    rows = [0, 65534, 65535, 65536, 100000, T - 1]
    print(f"tensors past 4 GB: T={T} H=Hkv={H} d={d} rows={rows}", flush=True)
    kf = k.cpu().numpy().astype(np.float64)
    vf = v.cpu().numpy().astype(np.float64)
    qr = q[rows].cpu().numpy().astype(np.float64)
    ref = np.stack([
        oracle.chunk_attn(qr[i:i + 1], kf[:r + 1], vf[:r + 1], n_head=H, n_head_kv=H,
                          head_dim=d, scale=scale, q_offsets=[0, 1], kv_offsets=[0, r + 1])[0]
        for i, r in enumerate(rows)])
    del kf, vf
    for prec in ("f32", "bf16"):
        out = pfa.gqa_prefill_attn(q, k, v, head_dim=d, scale=scale, precision=prec)
        torch.cuda.synchronize()
        got = out[rows].cpu().numpy()
        del out
        torch.cuda.empty_cache()
        if prec == "f32":
            assert_f32_parity(got, ref, "f32 past 4 GB")
        else:
            assert_bf16_parity(got, ref, "bf16 past 4 GB")


@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_prefill_2048_sampled(gpu_device, precision):
    # 2048 rows with 8B-like heads: one round of workgroups exactly fills the slots (the
    # boundary of the key-split rule); sampled rows against the oracle
    w = wl.sweep_workload(2048)
    x = wl.make_inputs(w)
    rows = wl.sample_rows(w, n_random=64, seed=9)
    print(f"prefill T=2048 {precision} rows={len(rows)}", flush=True)
    dev = gpu_device
    out = pfa.gqa_prefill_attn(torch.from_numpy(x.q).to(dev), torch.from_numpy(x.k).to(dev),
                               torch.from_numpy(x.v).to(dev), head_dim=w.head_dim,
                               scale=w.softmax_scale, precision=precision)
    torch.cuda.synchronize()
    ref = _attn_ref(w, x, rows=rows)
    got = out.cpu().numpy()[rows]
    if precision == "f32":
        assert_f32_parity(got, ref, "prefill 2048 f32")
    else:
        assert_bf16_parity(got, ref, "prefill 2048 bf16")


# Paired items (each f32 workgroup takes the j-th longest and the j-th shortest query
# block of the sequence): these shapes make 256, 512 or 1024 paired workgroups (e.g. 32 K/V heads
# of group 4 and 16 or 31 blocks of 32 rows).  T = 990 has an odd block count, so the middle
# workgroup takes one block.  Compared element by element, plain and fused entry.
PAIRED = [
    wl.Workload("paired_990", (990,), 128, 32, 128, 128, 1e6, 1e-6, seed=31),
    wl.Workload("paired_512", (512,), 128, 32, 128, 128, 1e6, 1e-6, seed=32),
    # group 2: two heads x two 32-row blocks per workgroup (64-row items), 16 items with a
    # ragged last one
    wl.Workload("paired_g2_1000", (1000,), 64, 32, 128, 128, 1e6, 1e-6, seed=33),
    # head_dim 64, partial rotary
    wl.Workload("paired_d64_500", (500,), 128, 32, 64, 32, 1e4, 1e-6, seed=34),
    # group 8: two head chunks per K/V head
    wl.Workload("paired_g8_500", (500,), 128, 16, 128, 64, 1e6, 1e-6, seed=35),
    # 1024 paired workgroups (64 K/V heads, 32 blocks of 32 rows, a ragged last one): two
    # whole rounds of two per CU
    wl.Workload("paired_2rounds_1000", (1000,), 256, 64, 128, 128, 1e6, 1e-6, seed=36),
]


@pytest.mark.parametrize("w", PAIRED, ids=[w.name for w in PAIRED])
def test_paired_items_full_compare(gpu_device, w):
    x = wl.make_inputs(w)
    t = _dev(x, gpu_device)
    ref = _attn_ref(w, x)
    assert_f32_parity(_attn_gpu(w, t), ref, f"attn {w.name}")
    assert_f32_parity(_fused_gpu(w, t), _fused_ref(w, x), f"fused {w.name}")
    # the same shapes through the bf16 kernel
    for prec in ("bf16", "bf16x3", "f16"):
        assert_bf16_parity(_attn_gpu(w, t, precision=prec), ref, f"attn {prec} {w.name}")
