"""GPU parity of ``qk_prep_chunk_attn_tiled``: blocks of new rows appended call after call
to one cache whose bf16 tiles the caller keeps (memra-engine 0.101.0 src/spec.rs,
``full_attn_verify``: a block of rows verified against, and appended to, a persistent
cache), through the C ABI.

Each call is compared with ``qk_prep_chunk_attn`` on the same inputs (the same f32 cache
before the call, the same raw rows): the output and the rows written to the caches must
be the same bits, since the tiles the attention reads are the same conversion of the same
cache rows.  Each output is also compared with the f64 oracle at the bf16 gate.  The
sequences of one ``kv_tiles`` start empty, grow by blocks of 0 .. 700 rows (new rows
starting inside a tile and on a tile edge, a single row, none), with a gate and a
sliding window on one call; the kept tiles sit between 4 KiB sentinel bands that must
stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity

pytestmark = pytest.mark.gpu

GUARD, SENTINEL = 4096, 0xC3

# (new rows per sequence) of each call, three sequences
BLOCKS = [(300, 0, 65), (200, 64, 1), (1, 130, 0), (700, 1, 70)]
MAX_ROWS = 1300


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _session(H, Hkv, d, n, precision, gate_call=2, window_call=3):
    total = tuple(sum(b[s] for b in BLOCKS) for s in range(3))
    w = wl.Workload(f"tiled_{H}_{Hkv}_{d}_{n}", total, H, Hkv, d, n, 1e6, 1e-6, seed=2100 + d + n)
    x = wl.make_inputs(w)  # raw rows of every position of the three sequences
    starts = np.concatenate([[0], np.cumsum(total)])
    nbytes = pfa.kv_tiles_bytes(3, MAX_ROWS, Hkv, d, precision)
    buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda:0")
    kv_tiles = buf[GUARD:GUARD + nbytes]
    # the caller's cache rows per sequence (rotated K, V), as the calls write them
    k_rows = [np.zeros((0, Hkv * d), np.float32) for _ in range(3)]
    v_rows = [np.zeros((0, Hkv * d), np.float32) for _ in range(3)]
    eps = float(np.float32(1e-6))
    for c, block in enumerate(BLOCKS):
        base = [len(r) for r in k_rows]
        full = [b + m for b, m in zip(base, block)]
        q_offs = np.concatenate([[0], np.cumsum(block)]).astype(np.int32)
        kv_offs = np.concatenate([[0], np.cumsum(full)]).astype(np.int32)
        pick = lambda a: np.concatenate(
            [a[starts[s] + base[s]:starts[s] + base[s] + block[s]] for s in range(3)])
        q_new, k_new, v_new = pick(x.q), pick(x.k), pick(x.v)
        T_q, T_kv = int(q_offs[-1]), int(kv_offs[-1])
        # the packed f32 caches before the call: earlier rows, new rows zero
        kc0 = np.zeros((T_kv, Hkv * d), np.float32)
        vc0 = np.zeros((T_kv, Hkv * d), np.float32)
        for s in range(3):
            kc0[kv_offs[s]:kv_offs[s] + base[s]] = k_rows[s]
            vc0[kv_offs[s]:kv_offs[s] + base[s]] = v_rows[s]
        gate = None
        if c == gate_call:
            gate = (2.0 * np.random.default_rng(2200 + c).standard_normal((T_q, H))).astype(np.float32)
        window = 96 if c == window_call else 0
        kw = dict(head_dim=d, rope_dim=n, rope_freq_base=1e6, rms_eps=1e-6, scale=d ** -0.5,
                  window=window, precision=precision, q_offsets=q_offs, kv_offsets=kv_offs,
                  gate=None if gate is None else _dev(gate))
        what = (f"qk_prep_chunk_attn_tiled call {c}: new rows {block} over {base} H={H} "
                f"Hkv={Hkv} d={d} n={n} {precision} window={window} gate={gate is not None}")
        print(what, flush=True)
        kc, vc = _dev(kc0), _dev(vc0)
        got = pfa.qk_prep_chunk_attn_tiled(_dev(q_new), _dev(k_new), _dev(v_new), _dev(x.wq),
                                           _dev(x.wk), kc, vc, kv_tiles, max_rows=MAX_ROWS, **kw)
        kr, vr = _dev(kc0), _dev(vc0)
        ref = pfa.qk_prep_chunk_attn(_dev(q_new), _dev(k_new), _dev(v_new), _dev(x.wq),
                                     _dev(x.wk), kr, vr, **kw)
        torch.cuda.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        kc, vc, kr, vr = (t.cpu().numpy() for t in (kc, vc, kr, vr))
        np.testing.assert_array_equal(got, ref, err_msg=what + ": vs qk_prep_chunk_attn")
        np.testing.assert_array_equal(kc, kr, err_msg=what + ": k_cache")
        np.testing.assert_array_equal(vc, vr, err_msg=what + ": v_cache")
        o = oracle.qk_prep_chunk_attn(q_new, k_new, v_new, x.wq, x.wk, kc0, vc0, n_head=H,
                                      n_head_kv=Hkv, head_dim=d, rope_dim=n,
                                      rope_freq_base=float(np.float32(1e6)), rms_eps=eps,
                                      scale=d ** -0.5, q_offsets=q_offs, kv_offsets=kv_offs,
                                      window=window, gate=gate)[0]
        assert_bf16_parity(got, o, what + " vs oracle")
        for s in range(3):
            k_rows[s] = kc[kv_offs[s]:kv_offs[s + 1]].copy()
            v_rows[s] = vc[kv_offs[s]:kv_offs[s + 1]].copy()
    torch.cuda.synchronize()
    bands = torch.cat([buf[:GUARD], buf[GUARD + nbytes:]]).cpu().numpy()
    assert np.all(bands == SENTINEL), "a write landed outside kv_tiles"


@pytest.mark.parametrize("precision", ["bf16", "bf16x3", "f16"])
def test_tiled_appends_8b_heads(precision):
    _session(32, 8, 128, 128, precision)


@pytest.mark.parametrize("precision", ["bf16", "bf16x3", "f16"])
def test_tiled_appends_d64_half_rotary(precision):
    _session(8, 2, 64, 32, precision, gate_call=0, window_call=1)
