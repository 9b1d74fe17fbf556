"""GPU parity of ``qknorm_rope`` (through the C ABI) against the f64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_f32_parity, eps32

pytestmark = pytest.mark.gpu


def _run(w, x, dev, in_place=False):
    q = torch.from_numpy(x.q).to(dev)
    k = torch.from_numpy(x.k).to(dev)
    wq = torch.from_numpy(x.wq).to(dev)
    wk = torch.from_numpy(x.wk).to(dev)
    print(f"qknorm_rope {w.name}: T={w.T} H={w.n_head} Hkv={w.n_head_kv} d={w.head_dim} "
          f"n={w.rope_dim} seqs={w.n_seqs} in_place={in_place}", flush=True)
    kw = dict(head_dim=w.head_dim, rope_dim=w.rope_dim, rope_freq_base=w.rope_freq_base,
              rms_eps=w.rms_eps, seq_offsets=w.seq_offsets)
    if in_place:
        qo, ko = pfa.qknorm_rope(q, k, wq, wk, q_out=q, k_out=k, **kw)
    else:
        qo, ko = pfa.qknorm_rope(q, k, wq, wk, **kw)
    torch.cuda.synchronize()
    return qo.cpu().numpy(), ko.cpu().numpy()


def _oracle(w, x):
    return oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=w.n_head, n_head_kv=w.n_head_kv,
                              head_dim=w.head_dim, rope_dim=w.rope_dim,
                              rope_freq_base=float(np.float32(w.rope_freq_base)),
                              rms_eps=eps32(w), seq_offsets=w.seq_offsets)


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_qknorm_rope_configs(gpu_device, name):
    """Every workload at full size (the oracle of this step is cheap), raw K (with the
    outlier tokens scaled x8 where the workload has them: the norm must erase them)."""
    w = wl.CONFIGS[name]
    x = wl.make_inputs(w)
    x.k = wl.with_outlier_keys(x.k, x.outliers)
    qo, ko = _run(w, x, gpu_device)
    rq, rk = _oracle(w, x)
    assert_f32_parity(qo, rq, f"{name} Q'")
    assert_f32_parity(ko, rk, f"{name} K'")


@pytest.mark.parametrize("d,n", [(128, 128), (128, 64), (128, 96), (128, 2), (128, 18),
                                 (64, 64), (64, 32), (64, 6)])
def test_qknorm_rope_rope_dims(gpu_device, d, n):
    """Full, half and odd partial rotary widths (in-lane, cross-half and general pairing)."""
    w = wl.Workload(f"rd{d}_{n}", (5, 70, 1, 0, 53), 6, 3, d, n, 1e4, 1e-6, seed=77 + d + n)
    x = wl.make_inputs(w)
    qo, ko = _run(w, x, gpu_device)
    rq, rk = _oracle(w, x)
    assert_f32_parity(qo, rq, f"d={d} n={n} Q'")
    assert_f32_parity(ko, rk, f"d={d} n={n} K'")


def test_qknorm_rope_in_place_and_positions(gpu_device):
    w = wl.CONFIGS["mixed"]
    x = wl.make_inputs(w)
    qo, ko = _run(w, x, gpu_device, in_place=True)
    rq, rk = _oracle(w, x)
    assert_f32_parity(qo, rq, "mixed in place Q'")
    assert_f32_parity(ko, rk, "mixed in place K'")


def test_qknorm_rope_first_token_not_rotated(gpu_device):
    """Position 0 of every packed sequence: only the norm applies (rotation by 0)."""
    w = wl.CONFIGS["mixed"]
    x = wl.make_inputs(w)
    qo, _ = _run(w, x, gpu_device)
    rq0, _ = oracle.qknorm_rope(x.q, x.k, x.wq, x.wk, n_head=w.n_head, n_head_kv=w.n_head_kv,
                                head_dim=w.head_dim, rope_dim=0, rope_freq_base=1e4,
                                rms_eps=eps32(w), seq_offsets=w.seq_offsets)
    starts = w.seq_offsets[:-1]
    assert_f32_parity(qo[starts], rq0[starts], "first tokens")


def test_qknorm_rope_zero_tokens_is_noop(gpu_device):
    q = torch.zeros((0, 256), device=gpu_device)
    k = torch.zeros((0, 128), device=gpu_device)
    w = torch.ones(64, device=gpu_device)
    qo, ko = pfa.qknorm_rope(q, k, w, w, head_dim=64, rope_dim=64, rope_freq_base=1e6,
                             rms_eps=1e-6)
    torch.cuda.synchronize()
    assert qo.numel() == 0 and ko.numel() == 0
