"""gqa_prefill_attn_noalloc, the entry point that allocates nothing (through the C ABI):
its output must equal gqa_prefill_attn's bit for bit (the same kernels and plan, only the
workspace lives in the library's own device array) and meet the oracle's gate, on two
calls in a row, the second smaller than the first (the array keeps the first call's
contents: nothing of it may leak into the second)."""
import numpy as np
import pytest
import torch

import oracle
import transformer_prefill_attention_amd as pfa
from transformer_prefill_attention_amd import workloads as wl
from tests.helpers import assert_bf16_parity, assert_f32_parity

pytestmark = pytest.mark.gpu

# first a larger call, then a smaller one that takes the key split (T = 512, 16/8 heads)
CALLS = [wl.Workload("noalloc_big", (1500, 0, 1, 1499), 32, 8, 128, 128, 1e6, 1e-6, seed=1900),
         wl.Workload("noalloc_small", (512,), 16, 8, 128, 128, 1e6, 1e-6, seed=1901)]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3", "f16"])
def test_noalloc_matches_the_workspace_entry(precision):
    for w in CALLS:
        x = wl.make_inputs(w)
        q, k, v = _dev(x.q), _dev(x.k), _dev(x.v)
        plan = pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=w.T, n_head=w.n_head, n_head_kv=w.n_head_kv,
                             head_dim=w.head_dim, precision=precision, q_offsets=w.seq_offsets)
        print(f"gqa_prefill_attn_noalloc {w.name}: T={w.T} H={w.n_head} Hkv={w.n_head_kv} "
              f"{precision} workspace {plan['workspace_bytes']} of "
              f"{pfa.noalloc_scratch_bytes()} bytes, key chunks {plan['max_key_chunks']}",
              flush=True)
        out = torch.full_like(q, float("nan"))
        pfa.gqa_prefill_attn_noalloc(q, k, v, head_dim=w.head_dim, scale=w.softmax_scale,
                                     precision=precision, seq_offsets=w.seq_offsets, out=out)
        torch.cuda.synchronize()
        want = pfa.gqa_prefill_attn(q, k, v, head_dim=w.head_dim, scale=w.softmax_scale,
                                    precision=precision, seq_offsets=w.seq_offsets)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got, want.cpu().numpy())
        ref = oracle.gqa_attn(x.q, x.k, x.v, n_head=w.n_head, n_head_kv=w.n_head_kv,
                              head_dim=w.head_dim, scale=w.softmax_scale,
                              seq_offsets=w.seq_offsets)
        check = assert_f32_parity if precision == "f32" else assert_bf16_parity
        check(got, ref, f"noalloc {precision} {w.name}")


def test_noalloc_rejects_calls_beyond_its_array():
    # bf16 tiles of 20000 key rows at 8 K/V heads of 128: 82 MB > 64 MiB
    T = 20000
    q = torch.zeros(T, 32 * 128, device="cuda:0")
    k = torch.zeros(T, 8 * 128, device="cuda:0")
    with pytest.raises(pfa.PfaError, match="device array"):
        pfa.gqa_prefill_attn_noalloc(q, k, k, head_dim=128, scale=0.088, precision="bf16")
