"""Attention calls captured in a HIP graph (torch.cuda.graph) and replayed, through the
C ABI.

The library enqueues only kernels (no memset, no allocation), so a call can be captured.
A replay reuses the captured arguments, the key split's per-call tag among them: the
in-place merge must leave its arrival counters at 0 for the next replay to find them so
(see the workspace notes in include/pfa.h).  Each case captures one call, then replays it
four times, each time with new inputs copied into the captured tensors and eager calls of
other shapes in between (sharing the no-alloc entry's device array, for that entry), and
compares every replay bit for bit with an eager call of the same entry point on the same
inputs.  Cases: f32 and bf16 splits merged in place, a split merged by the combine launch,
and the no-alloc entry.
"""
import numpy as np
import pytest
import torch

import transformer_prefill_attention_amd as pfa

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _rand(shape, seed):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


def _prefill_case(T, H, Hkv, d, precision, noalloc=False):
    dev = torch.device("cuda:0")
    q = _rand((T, H * d), 1).to(dev)
    k = _rand((T, Hkv * d), 2).to(dev)
    v = _rand((T, Hkv * d), 3).to(dev)
    out = torch.empty_like(q)
    scale = d ** -0.5
    if noalloc:
        call = lambda o: pfa.gqa_prefill_attn_noalloc(q, k, v, head_dim=d, scale=scale,
                                                       precision=precision, out=o)
    else:
        ws = torch.empty(max(pfa.workspace_bytes(T, H, Hkv, d, precision), 1), dtype=torch.uint8,
                         device=dev)
        call = lambda o: pfa.gqa_prefill_attn(q, k, v, head_dim=d, scale=scale,
                                              precision=precision, out=o, workspace=ws)
    return (q, k, v), out, call


def _chunk_case(precision):
    # one new row over 3000 cached: more key chunks than the in-place merge takes
    dev = torch.device("cuda:0")
    H, Hkv, d, T_kv = 8, 2, 128, 3001
    q = _rand((1, H * d), 4).to(dev)
    kc = _rand((T_kv, Hkv * d), 5).to(dev)
    vc = _rand((T_kv, Hkv * d), 6).to(dev)
    out = torch.empty_like(q)
    offs = dict(q_offsets=[0, 1], kv_offsets=[0, T_kv])
    ws = torch.empty(max(pfa.chunk_workspace_bytes(1, T_kv, H, Hkv, d, precision, **offs), 1),
                     dtype=torch.uint8, device=dev)
    call = lambda o: pfa.gqa_chunk_attn(q, kc, vc, head_dim=d, scale=d ** -0.5,
                                        precision=precision, out=o, workspace=ws, **offs)
    return (q, kc, vc), out, call


def _other_calls():
    """Eager calls of other shapes between replays (their own workspaces, or the no-alloc
    array)."""
    dev = torch.device("cuda:0")
    for T, prec in ((700, "f32"), (300, "bf16")):
        q = _rand((T, 16 * 64), 7).to(dev)
        k = _rand((T, 4 * 64), 8).to(dev)
        pfa.gqa_prefill_attn_noalloc(q, k, k, head_dim=64, scale=0.125, precision=prec)
        pfa.gqa_prefill_attn(q, k, k, head_dim=64, scale=0.125, precision=prec)


CASES = {
    "f32_merge_in_place": (lambda: _prefill_case(512, 16, 8, 128, "f32"),
                           pfa.ENTRY_PREFILL, (512, 16, 8, 128, "f32"), True),
    "bf16_merge_in_place": (lambda: _prefill_case(2048, 16, 8, 128, "bf16"),
                            pfa.ENTRY_PREFILL, (2048, 16, 8, 128, "bf16"), True),
    "f32_combine_launch": (lambda: _chunk_case("f32"), None, None, False),
    "noalloc_f32": (lambda: _prefill_case(512, 16, 8, 128, "f32", noalloc=True),
                    pfa.ENTRY_PREFILL, (512, 16, 8, 128, "f32"), True),
    "noalloc_bf16": (lambda: _prefill_case(2048, 16, 8, 128, "bf16", noalloc=True),
                     pfa.ENTRY_PREFILL, (2048, 16, 8, 128, "bf16"), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_calls(name):
    make, entry, plan_args, in_place = CASES[name]
    if entry is not None:
        T, H, Hkv, d, prec = plan_args
        plan = pfa.attn_plan(entry, T_q=T, n_head=H, n_head_kv=Hkv, head_dim=d, precision=prec)
        assert plan["max_key_chunks"] > 1 and plan["merge_in_place"] == int(in_place)
    inputs, out, call = make()
    print(f"graph {name}: eager call, capture", flush=True)
    call(out)  # first call eager: one-time set-up (device attributes, the array's address)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)  # warm the side stream as torch's capture recipe does
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for i, t in enumerate(inputs):
            t.copy_(_rand(tuple(t.shape), 100 + 10 * r + i).to(t.device))
        torch.cuda.synchronize()
        print(f"graph {name}: replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _other_calls()
        ref = torch.empty_like(out)
        call(ref)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got).all()), f"{name}: replay {r} left unwritten elements"
        assert torch.equal(got, ref), f"{name}: replay {r} differs from the eager call"
