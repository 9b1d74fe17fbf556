"""The attention work schedule, checked on the host (no GPU): ``pfa_attn_units`` decodes
every attention workgroup's unit with the kernels' own decode (compiled for the host
too), so these tests see exactly what the kernels would run.

For random packed-sequence tables of up to PFA_MAX_SEQS = 128 sequences (empty ones
included), head geometries, precisions and entry points:

* every (sequence, super-block) work item is decoded exactly once per (K/V head, head
  chunk) -- twice would compute rows twice, never would leave them unwritten;
* items come longest first: super-block levels never increase along the item order, and
  within a level the sequences with more super-blocks come first;
* the key chunks of an item cover, without gaps or overlap, exactly the key tiles that
  hold a key some row of the super-block may see.  That set is derived here from the
  visibility rule itself -- causal: a row at position p sees the keys at positions
  0..p of its sequence (memra-engine 0.101.0 src/spec.rs, `full_attn_verify`: row r of
  a block appended after base_len rows attends base_len + r + 1 keys); with a window W
  only the last W of them -- not from the kernels' tile formula;
* paired f32 workgroups (slot j takes items j and n-1-j) cover every item once;
* the grid is dense: every workgroup index appears.
"""
import numpy as np
import pytest

import transformer_prefill_attention_amd as pfa

F = {name: i for i, name in enumerate(pfa.UNIT_FIELDS)}


def _visible_tiles(q_lo, q_hi, base, kv_len, tile_keys, causal, window):
    """Key tiles (of the sequence's key rows) holding a key some query row of positions
    base+q_lo .. base+q_hi-1 may see: an interval [first, end)."""
    if not causal:
        return 0, -(-kv_len // tile_keys)
    p_lo, p_hi = base + q_lo, base + q_hi - 1
    key_hi = min(p_hi, kv_len - 1)               # largest key any row sees
    key_lo = max(0, p_lo - window + 1) if window > 0 else 0  # smallest one
    return key_lo // tile_keys, key_hi // tile_keys + 1


def _check_schedule(entry, q_lens, kv_lens, H, Hkv, D, precision, causal=True, window=0,
                    workspace_bytes=None):
    q_offs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv_offs = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    chunk = entry not in (pfa.ENTRY_PREFILL, pfa.ENTRY_PREP)
    kw = dict(T_q=int(q_offs[-1]), n_head=H, n_head_kv=Hkv, head_dim=D, causal=causal,
              precision=precision, q_offsets=q_offs, workspace_bytes=workspace_bytes)
    if chunk:
        kw.update(T_kv=int(kv_offs[-1]), kv_offsets=kv_offs, window=window)
    plan = pfa.attn_plan(entry, **kw)
    rec = pfa.attn_units(entry, **kw)
    rpi, tk = plan["rows_per_item"], plan["tile_keys"]
    n_items = plan["items"]
    # the item set the sequences define
    want = {(s, b) for s, L in enumerate(q_lens) for b in range(-(-L // rpi))}
    assert n_items == len(want)
    if n_items == 0:
        assert len(rec) == 0
        return plan
    # dense grid, pass-0 record per workgroup
    p0 = rec[rec[:, F["pass"]] == 0]
    assert np.array_equal(np.sort(p0[:, F["workgroup"]]), np.arange(plan["workgroups"]))
    # item -> (sequence, super-block) is a bijection onto `want`, the same for every unit
    item_of = {}
    for it, s, b in rec[:, [F["item"], F["sequence"], F["super_block"]]]:
        assert item_of.setdefault(int(it), (int(s), int(b))) == (int(s), int(b))
    assert sorted(item_of) == list(range(n_items))
    assert set(item_of.values()) == want
    # longest first: levels non-increasing; within a level, more super-blocks first
    nsb = [-(-L // rpi) for L in q_lens]
    keyed = [(item_of[i][1], nsb[item_of[i][0]]) for i in range(n_items)]
    assert all(a >= b for a, b in zip(keyed, keyed[1:])), "items not longest first"
    # heads: every (K/V head, head chunk) pair takes every item exactly once, and its key
    # chunks cover exactly the visible tiles
    g = H // Hkv
    n_chunks_head = max(rec[:, F["head_chunk"]]) + 1
    assert g % n_chunks_head == 0
    assert set(rec[:, F["kv_head"]]) == set(range(Hkv))
    # tile ranges per (item, kv, head chunk)
    ranges = {}
    for r in rec:
        key = (int(r[F["item"]]), int(r[F["kv_head"]]), int(r[F["head_chunk"]]))
        tb, te = int(r[F["tile_begin"]]), int(r[F["tile_end"]])
        ranges.setdefault(key, []).append((int(r[F["key_chunk"]]), tb, te))
    assert len(ranges) == n_items * Hkv * n_chunks_head
    for (it, kv, hc), lst in ranges.items():
        s, b = item_of[it]
        base = kv_lens[s] - q_lens[s]
        q_lo, q_hi = b * rpi, min((b + 1) * rpi, q_lens[s])
        first, end = _visible_tiles(q_lo, q_hi, base, kv_lens[s], tk, causal, window)
        got = sorted((tb, te) for kc, tb, te in lst if te > tb)
        # one record per key chunk index, no duplicates
        kcs = [kc for kc, _, _ in lst]
        assert len(kcs) == len(set(kcs))
        assert got, f"item {it} has no key range"
        assert got[0][0] == first and got[-1][1] == end, (it, got, first, end)
        for (a0, a1), (b0, b1) in zip(got, got[1:]):
            assert a1 == b0, f"key chunks of item {it} leave a gap or overlap: {got}"
    return plan


def _random_lens(rng, n, max_len, p_empty=0.15):
    lens = rng.integers(1, max_len + 1, size=n)
    lens[rng.random(n) < p_empty] = 0
    return [int(x) for x in lens]


GEOMS = [(8, 8, 128), (16, 8, 128), (32, 8, 128), (16, 4, 64), (6, 2, 128), (8, 1, 64),
         (32, 4, 128)]


@pytest.mark.parametrize("seed", range(24))
def test_prefill_schedule_random(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.choice([1, 2, 5, 17, 64, 127, 128]))
    H, Hkv, D = GEOMS[seed % len(GEOMS)]
    lens = _random_lens(rng, n, int(rng.choice([40, 300, 2000])))
    if sum(lens) == 0:
        lens[0] = 1
    for precision in ("f32", "bf16"):
        for entry in (pfa.ENTRY_PREFILL, pfa.ENTRY_PREP):
            _check_schedule(entry, lens, lens, H, Hkv, D, precision,
                            causal=bool(seed % 5 != 4))


@pytest.mark.parametrize("seed", range(16))
def test_chunk_schedule_random(seed):
    """New rows over cached prefixes (and sliding windows): the key chunks cover the
    tiles visible from each super-block's rows at their positions base + r."""
    rng = np.random.default_rng(900 + seed)
    n = int(rng.choice([1, 3, 31, 128]))
    H, Hkv, D = GEOMS[(seed * 3) % len(GEOMS)]
    q_lens = _random_lens(rng, n, int(rng.choice([1, 64, 700])))
    if sum(q_lens) == 0:
        q_lens[0] = 1
    kv_lens = [L + int(rng.integers(0, 3000)) for L in q_lens]
    window = int(rng.choice([0, 0, 1, 100, 1024]))
    for precision, entry in (("f32", pfa.ENTRY_CHUNK), ("bf16", pfa.ENTRY_CHUNK_PREP),
                             ("bf16", pfa.ENTRY_Q8)):
        _check_schedule(entry, q_lens, kv_lens, H, Hkv, D, precision, window=window)


def test_paired_items_cover_every_item_once():
    # 8B-like heads at T = 2048 and 4096 take the paired f32 kernel (256 / 512 workgroups)
    for T in (2048, 4096):
        plan = _check_schedule(pfa.ENTRY_PREFILL, [T], [T], 32, 8, 128, "f32")
        assert plan["paired"] == 1
        assert "attn_f32_kernel<128,false,true,false>" in plan["kernels"]
    # odd item count: the middle workgroup takes one item
    plan = _check_schedule(pfa.ENTRY_PREFILL, [990], [990], 128, 32, 128, "f32")
    assert plan["paired"] == 1 and plan["items"] % 2 == 1
    # whole rounds of two paired workgroups per CU: 1024 at T = 8192, 2048 at 16384, and
    # 1024 for 64 K/V heads at T = 1000 (odd item count again)
    for T, H, Hkv in ((8192, 32, 8), (16384, 32, 8), (1000, 256, 64)):
        plan = _check_schedule(pfa.ENTRY_PREFILL, [T], [T], H, Hkv, 128, "f32")
        assert plan["paired"] == 1 and plan["workgroups"] % 512 == 0, (T, H, plan)
        plan = _check_schedule(pfa.ENTRY_PREP, [T], [T], H, Hkv, 128, "f32")
        assert plan["paired"] == 1, (T, H, plan)
    # T = 6144 would make 768 paired workgroups (a round and a half): unpaired; 16-bit calls too
    plan = _check_schedule(pfa.ENTRY_PREFILL, [6144], [6144], 32, 8, 128, "f32")
    assert plan["paired"] == 0
    plan = _check_schedule(pfa.ENTRY_PREFILL, [8192], [8192], 32, 8, 128, "bf16")
    assert plan["paired"] == 0


def test_key_split_at_short_inputs():
    # T = 512 with 0.6B-like heads: the items cannot fill the GPU, so the key range is
    # split (f32 only when the workspace has room for the partial results); with at most
    # 4 chunks an item, each item's last workgroup merges them (no combine launch)
    for prec, kernel in (("f32", "attn_f32_kernel<128,false,false,true>"),
                         ("bf16x3", "attn_bf16_kernel<128,true,false,false,true,false>")):
        plan = _check_schedule(pfa.ENTRY_PREFILL, [512], [512], 16, 8, 128, prec)
        assert 1 < plan["max_key_chunks"] <= 4 and plan["workspace_bytes"] > 0
        assert plan["merge_in_place"] == 1
        assert plan["kernels"].endswith(kernel) and "combine" not in plan["kernels"]
    # plain bf16 and f16 (the same kernel) split sequences of at least 2048 keys to fill
    # the slots; shorter ones whose items fill at most a quarter of them in two halves,
    # when a half is at least 6 tiles (T = 768 and 1024 with 16/8 heads) or the items fill
    # at most an eighth (T = 512 with 16/8 heads), not otherwise (T = 512 with 32/8 heads,
    # T = 1024 with 32/8 heads)
    for prec in ("bf16", "f16"):
        for T, H, halves in ((512, 16, True), (768, 16, True), (1024, 16, True),
                             (512, 32, False), (1024, 32, False), (256, 16, False)):
            plan = _check_schedule(pfa.ENTRY_PREFILL, [T], [T], H, 8, 128, prec)
            if halves:
                assert plan["max_key_chunks"] == 2 and plan["merge_in_place"] == 1, (T, H, plan)
                assert plan["key_chunk_tiles"] == (T // 64 + 1) // 2
            else:
                assert plan["max_key_chunks"] == 1 and plan["merge_in_place"] == 0, (T, H, plan)
        plan = _check_schedule(pfa.ENTRY_PREFILL, [2048], [2048], 16, 8, 128, prec)
        assert 1 < plan["max_key_chunks"] <= 4 and plan["merge_in_place"] == 1
        assert plan["kernels"].endswith(
            f"attn_bf16_kernel<128,false,false,false,true,{'true' if prec == 'f16' else 'false'}>")
    plan = _check_schedule(pfa.ENTRY_PREFILL, [512], [512], 16, 8, 128, "f32",
                           workspace_bytes=0)
    assert plan["max_key_chunks"] == 1 and plan["workspace_bytes"] == 0
    assert plan["merge_in_place"] == 0 and "combine" not in plan["kernels"]
    # new rows over a long cache: the key range of each item is cut into more chunks than
    # the in-place merge takes, merged by the combine launch
    for q_len, chunks in ((1, 32), (256, 8)):
        for prec in ("f32", "bf16"):
            plan = _check_schedule(pfa.ENTRY_CHUNK, [q_len], [8192], 32, 8, 128, prec)
            assert plan["max_key_chunks"] == chunks and plan["merge_in_place"] == 0
            assert plan["kernels"].endswith("attn_combine_kernel<128>")


def test_plan_workspace_matches_the_size_queries():
    for lens, H, Hkv, D in (([512], 16, 8, 128), ([4096], 32, 8, 128),
                            ([128, 256, 0, 5000], 16, 4, 128), ([7, 33], 4, 2, 64)):
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(offs[-1])
        for prec in ("f32", "bf16", "bf16x3"):
            for entry, fused in ((pfa.ENTRY_PREFILL, False), (pfa.ENTRY_PREP, True)):
                plan = pfa.attn_plan(entry, T_q=T, n_head=H, n_head_kv=Hkv, head_dim=D,
                                     precision=prec, q_offsets=offs)
                assert plan["workspace_bytes"] == pfa.workspace_bytes(
                    T, H, Hkv, D, prec, seq_offsets=offs, fused=fused)
            plan = pfa.attn_plan(pfa.ENTRY_CHUNK, T_q=T, T_kv=T, n_head=H, n_head_kv=Hkv,
                                 head_dim=D, precision=prec, q_offsets=offs, kv_offsets=offs)
            assert plan["workspace_bytes"] == pfa.chunk_workspace_bytes(
                T, T, H, Hkv, D, prec, q_offsets=offs, kv_offsets=offs)
        plan = pfa.attn_plan(pfa.ENTRY_Q8_PREP, T_q=T, T_kv=T, n_head=H, n_head_kv=Hkv,
                             head_dim=D, q_offsets=offs, kv_offsets=offs)
        assert plan["workspace_bytes"] == pfa.q8_workspace_bytes(
            T, T, H, Hkv, D, q_offsets=offs, kv_offsets=offs, fused=True)


def test_plan_names_the_kernels_in_launch_order():
    p = pfa.attn_plan(pfa.ENTRY_PREP, T_q=8192, n_head=32, n_head_kv=8, head_dim=128,
                      rope_dim=128)
    # (8192 rows: 1024 paired workgroups, two whole rounds)
    assert p["kernels"] == ("qknorm_rope_kernel<128,0,false> + "
                            "attn_f32_kernel<128,true,true,false>")
    p = pfa.attn_plan(pfa.ENTRY_PREP, T_q=8192, n_head=32, n_head_kv=8, head_dim=128,
                      rope_dim=128, precision="bf16")
    assert p["kernels"] == ("rope_table_kernel<128,false> + "
                            "stage_kv_bf16_kernel<128,false,true,false> + "
                            "attn_bf16_kernel<128,false,true,false,false,false>")
    p = pfa.attn_plan(pfa.ENTRY_PREP, T_q=8192, n_head=32, n_head_kv=8, head_dim=128,
                      rope_dim=128, precision="f16")
    assert p["kernels"] == ("rope_table_kernel<128,false> + "
                            "stage_kv_bf16_kernel<128,false,true,true> + "
                            "attn_bf16_kernel<128,false,true,false,false,true>")
    p = pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=8192, n_head=32, n_head_kv=8, head_dim=128,
                      precision="bf16x3")
    assert p["kernels"] == ("stage_kv_bf16_kernel<128,true,false,false> + "
                            "attn_bf16_kernel<128,true,false,false,false,false>")
    # the tiled chunk entry: the new rows' K/V into the caches, their tiles re-staged into
    # kv_tiles, attention (1024 rows over 8192: two key chunks, merged in place)
    p = pfa.attn_plan(pfa.ENTRY_CHUNK_TILED, T_q=1024, T_kv=8192, n_head=32, n_head_kv=8,
                      head_dim=128, rope_dim=128, precision="bf16", q_offsets=[0, 1024],
                      kv_offsets=[0, 8192])
    assert p["kernels"] == ("qknorm_rope_kernel<128,0,false> + "
                            "append_tiles_kernel<128,false,false> + "
                            "attn_bf16_kernel<128,false,true,false,true,false>")
    assert p["workspace_bytes"] == pfa.chunk_workspace_bytes(
        1024, 8192, 32, 8, 128, "bf16", q_offsets=[0, 1024], kv_offsets=[0, 8192], fused=2)
    p = pfa.attn_plan(pfa.ENTRY_Q8, T_q=8192, T_kv=8192, n_head=32, n_head_kv=8, head_dim=64)
    assert p["kernels"] == ("stage_kv_q8_kernel<64,false> + "
                            "attn_bf16_kernel<64,false,false,true,false,false>")


def test_plan_rejects_what_the_entry_points_reject():
    with pytest.raises(pfa.PfaError, match="head_dim"):
        pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=64, n_head=4, n_head_kv=2, head_dim=96)
    with pytest.raises(pfa.PfaError, match="multiple"):
        pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=64, n_head=5, n_head_kv=2, head_dim=64)
    with pytest.raises(pfa.PfaError, match="packed sequences"):
        lens = np.full(129, 2)
        pfa.attn_plan(pfa.ENTRY_PREFILL, T_q=258, n_head=4, n_head_kv=2, head_dim=64,
                      q_offsets=np.concatenate([[0], np.cumsum(lens)]))
    with pytest.raises(pfa.PfaError, match="window"):
        pfa.attn_plan(pfa.ENTRY_CHUNK, T_q=64, T_kv=64, n_head=4, n_head_kv=2, head_dim=64,
                      causal=False, window=8)
    with pytest.raises(pfa.PfaError, match="unknown entry"):
        pfa.attn_plan(9, T_q=64, n_head=4, n_head_kv=2, head_dim=64)
