"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Selected block indices and counts must match bit for bit; h_full, h_sparse,
delta and the losses within 2e-2 max-abs for bf16 inputs (float32
accumulation) and 1e-5 for float32 problems. Relative-L2 and delta bars are
asserted as well. Small problems are compared in full; the full-size
workloads are compared on every selected index and on sampled rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.ssa_oracle as O
from gpu_common import (BF16_ABS, BF16_DELTA_ABS, BF16_REL_L2, F32_ABS, assert_close,
                        full_compare, gpu_run, np_inputs, sample_rows, to_np64)
from ssa_inputs import CONFIGS, default_head_map, make_inputs, scale_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssa():
    import block_sparse_full_amd as m
    m.load_library()
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- small, full comparison

SMALL = [
    ("gqa_decode_64k", dict(B=2, Hq=16, Hkv=1, N=2048), 5, 1, 1),   # 16 q heads per kv head
    ("tiny_f32", {}, 4, 1, 1),
    ("tiny_f32", {}, 2, 1, 1),
    ("tiny_f32", dict(Hq=2, Hkv=1, N=1024), 5, 2, 1),
    ("mha_4k", dict(Hq=2, Hkv=2, N=1024), 4, 1, 1),
    ("mha_4k", dict(Hq=2, Hkv=1, N=1024, D=64), 3, 1, 1),
    ("mha_4k", dict(Hq=1, Hkv=1, N=64), 1, 0, 1),
    ("mha_4k", dict(Hq=2, Hkv=2, N=640), 3, 0, 0),
    ("gqa_8k_peaked", dict(B=2, Hq=8, Hkv=2, N=1024), 4, 1, 1),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=2048), 6, 2, 2),
    # four q heads per workgroup: G = 8 (two groups per kv head), no forced
    # blocks (the diagonal block may be dropped), several bitmap words, iid
    # inputs (the heads' selections differ widely)
    ("gqa_8k_peaked", dict(B=2, Hq=16, Hkv=2, N=1536), 5, 0, 0),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=4096), 7, 1, 2),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048, planted=False), 6, 1, 1),
    # 9 query blocks: a work-item count that is not a multiple of the 8 XCD
    # queues, so the grouped kernel takes its static one-item-per-workgroup path
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=576), 4, 1, 1),
    ("gqa_decode_64k", dict(B=3, Hq=8, Hkv=2, N=2048), 4, 1, 1),
    ("gqa_decode_64k", dict(B=2, Hq=8, Hkv=1, N=4096, D=64), 5, 1, 1),
    ("gqa_decode_64k", dict(B=2, Hq=2, Hkv=2, N=640), 3, 0, 1),
    ("gqa_decode_64k", dict(dtype="f32", B=2, Hq=4, Hkv=2, N=1024), 4, 1, 1),
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local", SMALL,
                         ids=[f"{s[0]}-{i}" for i, s in enumerate(SMALL)])
def test_small_full_parity(ssa, name, kw, budget, n_sink, n_local):
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, **kw)
    say(f"[parity] {cfg}")
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, want_lse=True)
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, lse=True)


def test_decode_sparse_only_and_pooled_table(ssa):
    cfg = CONFIGS["gqa_decode_64k"].with_sizes(B=3, Hq=8, Hkv=2, N=4096, budget=6)
    say(f"[parity] sparse-only decode {cfg}")
    x = make_inputs(cfg)
    dual = gpu_run(ssa, x, budget=6, k_pooled=True)
    sp = gpu_run(ssa, x, budget=6, k_pooled=True, sparse_only=True)
    xn = np_inputs(x)
    # the pooled table matches the oracle's pooling bit for bit
    assert np.array_equal(dual["k_pooled"].numpy(), O.pool_blocks(xn["k"], 64))
    ref = full_compare(cfg, x, dual, budget=6)
    assert np.array_equal(sp["idx"].numpy(), ref["idx"])
    assert "h_full" not in sp
    assert_close("h_sparse (sparse-only)", to_np64(sp["h_sparse"]), ref["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("sparse-only vs dual", to_np64(sp["h_sparse"]), to_np64(dual["h_sparse"]), 1e-2)


def test_prefill_sparse_only_matches_dual(ssa):
    """Two q heads per kv head: dual mode runs the per-head kernel, sparse-only
    the gather kernel (a different summation order, so not bit for bit); both
    match the oracle and each other."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=4, Hkv=2, N=1024, budget=4)
    x = make_inputs(cfg)
    dual = gpu_run(ssa, x, budget=4)
    sp = gpu_run(ssa, x, budget=4, sparse_only=True)
    ref = full_compare(cfg, x, dual, budget=4)
    assert torch.equal(sp["idx"], dual["idx"])
    assert_close("h_sparse (sparse-only)", to_np64(sp["h_sparse"]), ref["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("sparse-only vs dual", to_np64(sp["h_sparse"]), to_np64(dual["h_sparse"]), 1e-2)


def test_prefill_sparse_only_grouped_shape(ssa):
    """Four q heads per kv head: dual mode runs the grouped kernel, sparse-only
    the per-head kernel; both match the oracle and each other."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=2048, budget=5)
    say(f"[parity] sparse-only prefill {cfg}")
    x = make_inputs(cfg)
    dual = gpu_run(ssa, x, budget=5)
    sp = gpu_run(ssa, x, budget=5, sparse_only=True)
    ref = full_compare(cfg, x, dual, budget=5)
    assert "h_full" not in sp
    assert torch.equal(sp["idx"], dual["idx"])
    assert_close("h_sparse (sparse-only)", to_np64(sp["h_sparse"]), ref["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("sparse-only vs dual", to_np64(sp["h_sparse"]), to_np64(dual["h_sparse"]), 1e-2)


def test_full_budget_gives_identical_streams(ssa):
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=4, Hkv=2, N=1024)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=16)
    assert torch.equal(got["h_sparse"], got["h_full"])
    assert torch.count_nonzero(got["delta"]) == 0
    assert float(got["loss"][0]) == 0.0
    nkb = 16
    assert torch.equal(got["idx"][0, 0, -1], torch.arange(nkb, dtype=torch.int32))


def test_full_budget_gives_identical_streams_grouped(ssa):
    """Four q heads per kv head (one workgroup serves all four): with every
    block selected the walk has no second part and both streams coincide."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=1024)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=20)
    assert torch.equal(got["h_sparse"], got["h_full"])
    assert torch.count_nonzero(got["delta"]) == 0


GROUP_SELECT = [
    # prefill through the grouped kernel (4 q heads per kv head), through the
    # per-head kernel (2 per kv head, D 64), and decode; a custom head map
    ("gqa_8k_peaked", dict(B=2, Hq=8, Hkv=2, N=2048), 6, 1, 1, None),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048, planted=False), 5, 1, 1, [1, 0, 0, 1, 1, 0, 1, 0]),
    ("mha_4k", dict(Hq=4, Hkv=2, N=1024, D=64), 4, 1, 1, None),
    ("gqa_decode_64k", dict(B=3, Hq=8, Hkv=2, N=4096), 6, 1, 1, None),
    ("gqa_decode_64k", dict(dtype="f32", B=2, Hq=4, Hkv=2, N=1024), 4, 1, 1, None),
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local,hm", GROUP_SELECT,
                         ids=[f"{g[0]}-{i}" for i, g in enumerate(GROUP_SELECT)])
def test_group_select_parity(ssa, name, kw, budget, n_sink, n_local, hm):
    """Group-shared selection (one list per GQA group): indices bit-exact,
    identical within each group, streams and lse within the bars."""
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, **kw)
    say(f"[parity] group select {cfg} head_map={hm}")
    x = make_inputs(cfg, head_map=hm)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                  want_lse=True, group_select=True)
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                 lse=True, group_select=True)
    hmap = hm or default_head_map(cfg.Hq, cfg.Hkv)
    idx = got["idx"].numpy()
    for h in range(cfg.Hq):
        first = hmap.index(hmap[h])
        assert np.array_equal(idx[:, h], idx[:, first]), h


# 16-token selection blocks (the pages' model shape): prefill with D 64 and
# 128, GQA 1:1 to 16:1, no forced blocks, iid inputs; decode; sparse-only
BLOCK16 = [
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024), 16, 1, 1, False),
    ("paper_16k_b16", dict(Hq=2, Hkv=2, N=640, D=128), 6, 0, 0, False),
    ("paper_16k_b16", dict(B=2, Hq=32, Hkv=2, N=512), 16, 1, 1, False),
    ("paper_16k_b16", dict(Hq=4, Hkv=2, N=2048, planted=False), 12, 2, 2, False),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024, D=128), 16, 1, 1, True),
    # 16 q heads on one kv head: four four-head workgroups share each kv head
    ("paper_16k_b16", dict(Hq=16, Hkv=1, N=1536), 16, 1, 1, False),
    # 9 query tiles: the static one-item-per-workgroup path of the grouped kernel
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=576), 16, 1, 1, False),
    ("paper_16k_b16", dict(decode=True, B=3, Hq=8, Hkv=2, N=2048), 16, 1, 1, False),
    ("paper_16k_b16", dict(decode=True, B=2, Hq=4, Hkv=1, N=4096, D=128), 9, 1, 1, False),
    # decode with 16 q heads per kv head (two workgroups of 8 per group)
    ("paper_16k_b16", dict(decode=True, B=2, Hq=32, Hkv=2, N=2048), 16, 1, 1, False),
    ("paper_16k_b16", dict(decode=True, B=2, Hq=32, Hkv=2, N=2048), 16, 1, 1, True),
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local,sparse", BLOCK16,
                         ids=[f"b16-{i}" for i in range(len(BLOCK16))])
def test_block16_parity(ssa, name, kw, budget, n_sink, n_local, sparse):
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, **kw)
    say(f"[parity] block 16 {cfg} sparse_only={sparse}")
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, want_lse=not sparse,
                  sparse_only=sparse, block=16)
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, lse=not sparse,
                 sparse_only=sparse)


# Large and growing logits: queries scaled by 4 and keys by a ramp from 1 at
# the first position to 8 at the last, so a row's block maxima climb along
# the walk by far more than the 2^24 rescale slack (logit standard deviation
# from about 6 to 46 in log2 units). The grouped kernels' key-norm bound can
# then no longer rule out a rescale: they compute the block maxima and
# rescale many times. The selection favours the late, large blocks, so the
# selected stream's weights stay within float32 range of the row maximum
# (the 16-token kernel keeps one running maximum for both streams).
LARGE_LOGITS = [
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048), 6, 1, 1, 64),   # D 128, 64-token blocks
    ("paper_16k_b16", dict(Hq=8, Hkv=2, N=2048), 16, 1, 1, 16),       # D 64, 16-token blocks
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local,block", LARGE_LOGITS,
                         ids=["grouped-d128", "grouped-b16"])
def test_large_logits_parity(ssa, name, kw, budget, n_sink, n_local, block):
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, **kw)
    say(f"[parity] large logits {cfg}")
    x = make_inputs(cfg)
    ramp = torch.linspace(1.0, 8.0, cfg.N).view(1, 1, cfg.N, 1)
    x["q"] = x["q"] * 4
    x["k"] = (x["k"].float() * ramp).to(x["k"].dtype)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, want_lse=True,
                  block=block)
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, lse=True)


# Sparse-only prefill with per-block lists (the gather kernel): 16- and
# 64-token blocks, D 64 and 128, GQA 1:1 to 16:1 and 3:1 (workgroups whose
# four lists span query blocks), odd list lengths, no forced blocks (the
# diagonal may be missing), lists that cover every causal block, a head map,
# 9 query tiles; h_sparse and the sparse lse against the oracle
SPARSE_GATHER = [
    ("paper_16k_b16", dict(Hq=16, Hkv=1, N=1024), 16, 1, 1, None),
    ("paper_16k_b16", dict(Hq=4, Hkv=2, N=1024, D=128), 7, 1, 1, None),
    ("paper_16k_b16", dict(Hq=3, Hkv=1, N=576, planted=False), 5, 0, 0, None),
    ("paper_16k_b16", dict(B=2, Hq=8, Hkv=2, N=512), 40, 1, 1, None),
    ("paper_16k_b16", dict(Hq=8, Hkv=2, N=1024), 9, 2, 2, [1, 0, 0, 1, 1, 0, 1, 0]),
    ("gqa_8k_peaked", dict(B=2, Hq=8, Hkv=2, N=1024), 4, 1, 1, None),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=2048, D=64), 5, 0, 0, None),
    ("gqa_8k_peaked", dict(B=1, Hq=3, Hkv=3, N=576, planted=False), 3, 1, 1, None),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=2, N=1024), 16, 1, 1, None),
    ("mha_4k", dict(Hq=2, Hkv=2, N=640), 3, 0, 1, None),
    # eight and sixteen q heads per workgroup
    ("paper_16k_b16", dict(Hq=8, Hkv=1, N=1024), 12, 1, 1, None),
    ("paper_16k_b16", dict(Hq=16, Hkv=1, N=1024, D=128), 16, 1, 1, None),
    ("paper_16k_b16", dict(Hq=32, Hkv=2, N=512), 10, 1, 1, [i % 2 for i in range(32)]),
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local,hm", SPARSE_GATHER,
                         ids=[f"gather-{i}" for i in range(len(SPARSE_GATHER))])
def test_sparse_only_gather_parity(ssa, name, kw, budget, n_sink, n_local, hm):
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, **kw)
    say(f"[parity] sparse-only gather {cfg} head_map={hm}")
    x = make_inputs(cfg, head_map=hm)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                  want_lse=True, sparse_only=True, block=cfg.block)
    assert "h_full" not in got
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                 lse=True, sparse_only=True)


def test_block16_group_select(ssa):
    cfg = CONFIGS["paper_16k_b16"].with_sizes(Hq=8, Hkv=2, N=1024)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=16, want_lse=True, group_select=True, block=16)
    full_compare(cfg, x, got, budget=16, lse=True, group_select=True)


# ---------------------------------------------------------------- hand-built lists

def pattern_lists(B, Hq, Hkv, nqb, seed, head_map):
    """Per-head block lists whose selection patterns over the four heads of a
    work group cover every subset: blocks chosen by nested head sets (the
    runs the grouped kernel walks once), arbitrary partial sets, no head and
    all heads. Block 0 and the diagonal block are in every list (so every row
    has a selected key). Returns idx [B, Hq, nqb, budget] (ascending, padded
    with -1) and cnt."""
    G = Hq // Hkv
    heads = [[h for h in range(Hq) if head_map[h] == g] for g in range(Hkv)]
    lists = {}
    for b in range(B):
        for g in range(Hkv):
            for hg in range(G // 4):
                hs = heads[g][4 * hg:4 * hg + 4]
                for qb in range(nqb):
                    rng = np.random.default_rng([seed, b, g, hg, qb])
                    perm = rng.permutation(4)
                    chain = [1 << perm[0], (1 << perm[0]) | (1 << perm[1]),
                             (1 << perm[0]) | (1 << perm[1]) | (1 << perm[2])]
                    masks = {0: 15, qb: 15}
                    for kb in range(1, qb):
                        r = rng.random()
                        if qb % 7 == 3:        # only all-or-none patterns
                            masks[kb] = 15 if r < 0.3 else 0
                        elif r < 0.4:
                            masks[kb] = chain[int(rng.integers(3))]
                        elif r < 0.7:
                            masks[kb] = int(rng.integers(1, 15))
                        elif r < 0.85:
                            masks[kb] = 0
                        else:
                            masks[kb] = 15
                    for u, h in enumerate(hs):
                        lists[(b, h, qb)] = sorted(kb for kb, m in masks.items() if (m >> u) & 1)
    budget = max(len(v) for v in lists.values())
    idx = np.full((B, Hq, nqb, budget), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    for (b, h, qb), l in lists.items():
        idx[b, h, qb, :len(l)] = l
        cnt[b, h, qb] = len(l)
    return idx, cnt


WALK = [
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048), None),             # 64 items: queues
    ("gqa_8k_peaked", dict(B=2, Hq=16, Hkv=2, N=2112, planted=False),    # 132 items: static
     [h % 2 for h in range(16)]),                                        # interleaved kv heads
]


@pytest.mark.parametrize("name,kw,hm", WALK, ids=["queues", "static_g8_headmap"])
def test_walk_patterns_parity(ssa, name, kw, hm):
    """The grouped D 128 kernel's walk list (per-head snapshot positions, a
    chosen head order, blocks walked once or twice by their selection
    pattern) on lists built to hit every pattern, dual and sparse-only, in
    full against the oracle's attention over the same lists."""
    cfg = CONFIGS[name].with_sizes(**kw)
    x = make_inputs(cfg)
    head_map = hm if hm is not None else default_head_map(cfg.Hq, cfg.Hkv)
    nqb = cfg.N // cfg.block
    idx, cnt = pattern_lists(cfg.B, cfg.Hq, cfg.Hkv, nqb, 7, head_map)
    budget = idx.shape[-1]
    say(f"walk patterns {name} {kw} budget {budget}")
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    p = ssa.problem_for(q, k, budget=budget, n_sink=1, n_local=1, head_map=head_map)
    di, dc = torch.from_numpy(idx).to(dev), torch.from_numpy(cnt).to(dev)
    out = ssa.attn_fwd(p, q, k, v, di, dc)
    sp = ssa.attn_fwd(p, q, k, v, di, dc, sparse_only=True)
    torch.cuda.synchronize()
    xn = np_inputs(x)
    ref = O.dual_attention(xn["q"], xn["k"], xn["v"], idx, block=cfg.block,
                           scale=scale_for(cfg), head_map=head_map)
    want = {n: np.zeros((cfg.B, cfg.Hq, cfg.N) + ((cfg.D,) if n != "delta" else ()))
            for n in ("h_full", "h_sparse", "delta")}
    for (b, h), (r, hf, hs_, dl) in ref.items():
        want["h_full"][b, h, r], want["h_sparse"][b, h, r], want["delta"][b, h, r] = hf, hs_, dl
    assert_close("h_full", to_np64(out["h_full"]), want["h_full"], BF16_ABS, BF16_REL_L2)
    assert_close("h_sparse", to_np64(out["h_sparse"]), want["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("delta", to_np64(out["delta"]), want["delta"], BF16_DELTA_ABS)
    assert_close("h_sparse (sparse-only)", to_np64(sp["h_sparse"]), want["h_sparse"], BF16_ABS,
                 BF16_REL_L2)


def test_attention_timing_hook(ssa):
    """Events handed to ssa_set_attn_timing_events bracket the attention
    kernel of a grouped prefill call: recorded after the V transpose, inside
    the call's own bracket; outputs are unchanged; clearing stops them."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=4096)
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    p = ssa.problem_for(q, k, budget=8, n_sink=1, n_local=1)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    ref = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    ssa.set_attn_timing_events(ev[1], ev[2])
    try:
        ev[0].record()
        out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
        ev[3].record()
    finally:
        ssa.set_attn_timing_events()
    torch.cuda.synchronize()
    call_ms, kern_ms = ev[0].elapsed_time(ev[3]), ev[1].elapsed_time(ev[2])
    say(f"call {call_ms:.4f} ms, attention kernel {kern_ms:.4f} ms")
    assert 0.0 < kern_ms <= call_ms
    assert ev[0].elapsed_time(ev[1]) >= 0.0 and ev[2].elapsed_time(ev[3]) >= 0.0
    for n in ("h_full", "h_sparse", "delta"):
        assert torch.equal(out[n], ref[n]), n
    # cleared: a later call leaves the events where they were
    before = ev[1].elapsed_time(ev[2])
    ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    torch.cuda.synchronize()
    assert ev[1].elapsed_time(ev[2]) == before


DETERMINISM = [
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048, budget=6), dict()),
    ("paper_16k_b16", dict(Hq=8, Hkv=2, N=2048, budget=16), dict(block=16)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048, budget=6), dict(token_select=True)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=2048, budget=6), dict(group_select=True)),
]


@pytest.mark.parametrize("name,kw,run", DETERMINISM, ids=["per_head", "block16", "per_token", "group"])
def test_run_to_run_determinism(ssa, name, kw, run):
    """Two calls on the same inputs give identical bits (fixed-order
    reductions everywhere)."""
    cfg = CONFIGS[name].with_sizes(**kw)
    x = make_inputs(cfg)
    a = gpu_run(ssa, x, budget=cfg.budget, want_lse=True, **run)
    b = gpu_run(ssa, x, budget=cfg.budget, want_lse=True, **run)
    for key in ("idx", "cnt", "h_full", "h_sparse", "delta", "loss", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_head_map_permutation(ssa):
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=1024, budget=4)
    hm = [1, 0, 0, 1, 1, 0, 1, 0]
    x = make_inputs(cfg, head_map=hm)
    got = gpu_run(ssa, x, budget=4, head_map=hm)
    full_compare(cfg, x, got, budget=4, head_map=hm)
    dcfg = CONFIGS["gqa_decode_64k"].with_sizes(B=2, Hq=8, Hkv=2, N=2048, budget=4)
    xd = make_inputs(dcfg, head_map=hm)
    gd = gpu_run(ssa, xd, budget=4, head_map=hm)
    full_compare(dcfg, xd, gd, budget=4, head_map=hm)


def test_exact_ties_go_to_lower_index(ssa):
    """Constant K: every pooled score ties, the free slots take the lowest
    candidate indices. Duplicated key blocks: the lower copy wins."""
    cfg = CONFIGS["mha_4k"].with_sizes(Hq=2, Hkv=1, N=1024, budget=5)
    x = make_inputs(cfg)
    x["k"][:] = x["k"][:, :, :1]
    got = gpu_run(ssa, x, budget=5)
    idx = got["idx"][0, 0]
    for qb in range(16):
        want = [0, 1, 2, 3, qb] if qb >= 4 else list(range(qb + 1))
        assert idx[qb, :len(want)].tolist() == want
    full_compare(cfg, x, got, budget=5)
    y = make_inputs(cfg)
    y["k"][:, :, 5 * 64:6 * 64] = y["k"][:, :, 9 * 64:10 * 64]
    g2 = gpu_run(ssa, y, budget=5)
    full_compare(cfg, y, g2, budget=5)


TIE_RUNS = [
    # (case, Nq, N, block, patterns, budget)
    ("decode_b64_few", 1, 65536, 64, 6, 32),
    ("decode_b64_mid", 1, 65536, 64, 40, 32),
    ("decode_b64_many", 1, 65536, 64, 300, 32),
    ("prefill_b16_mid", 8192, 8192, 16, 40, 16),
    ("prefill_b64_mid", 16384, 16384, 64, 12, 16),
    # more than 64 free slots: the radix select with the direct ranking of its last bin
    ("decode_b64_free98", 1, 65536, 64, 40, 100),
    ("prefill_b64_free88", 8192, 8192, 64, 400, 90),
]


@pytest.mark.parametrize("case", TIE_RUNS, ids=[c[0] for c in TIE_RUNS])
def test_select_tie_runs(ssa, case):
    """Every key block is a copy of one of a few random pattern blocks, so
    the pooled scores come in runs of exactly equal values and the top-k
    boundary falls inside a run: the selection must take the run's lowest
    block indices, bit for bit as the oracle does. Few patterns leave runs of
    hundreds of equal keys (radix passes down to the last byte); tens of
    patterns leave runs of a few dozen (the direct ranking of at most 64
    keys)."""
    name, nq, n, bs, npat, budget = case
    say(f"tie runs {name}: Nq {nq} N {n} block {bs} patterns {npat} budget {budget}")
    r = np.random.default_rng(11 + npat)
    D, Hq, Hkv = 128, 4, 1
    pat = torch.from_numpy(r.standard_normal((npat, bs, D)).astype(np.float32)).to(torch.bfloat16)
    ids = torch.from_numpy(r.integers(0, npat, size=n // bs))
    k = pat[ids].reshape(1, Hkv, n, D).contiguous()
    q = torch.from_numpy(r.standard_normal((1, Hq, nq, D)).astype(np.float32)).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    qd, kd = q.to(dev), k.to(dev)
    p = ssa.problem_for(qd, kd, budget=budget, block_size=bs)
    idx, cnt = ssa.select_blocks(p, qd, kd)
    torch.cuda.synchronize()
    ri, rc = O.select_blocks(q.float().numpy(), k.float().numpy(), block=bs, budget=budget,
                             n_sink=1, n_local=1, head_map=default_head_map(Hq, Hkv))
    assert np.array_equal(cnt.cpu().numpy(), rc), "block counts differ"
    assert np.array_equal(idx.cpu().numpy(), ri), "selected blocks differ"


def test_loss_and_gradient_seeds(ssa):
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=4, Hkv=1, N=1024, budget=4)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=4, want_grads=True)
    hf = got["h_full"].double(); hs = got["h_sparse"].double()
    ls, lc, gf, gs = O.align_loss(hf.numpy(), hs.numpy())
    # the loss kernel on the GPU's own outputs: float64 partials, float32 result
    assert abs(float(got["loss"][0]) - ls) <= 1e-6 * max(ls, 1e-30) + 1e-12
    assert float(got["loss"][1]) == float(got["loss"][0])
    # seeds are stored in bf16: within half a bf16 ulp, at most 2^-8 of the largest seed
    assert_close("grad_full", to_np64(got["grad_full"]), gf, 2.0 ** -8 * np.abs(gf).max() + 1e-12)
    assert_close("grad_sparse", to_np64(got["grad_sparse"]), gs, 2.0 ** -8 * np.abs(gs).max() + 1e-12)


def test_pool_blocks_bit_exact(ssa):
    for name, kw in (("mha_4k", dict(Hq=4, Hkv=4, N=2048)), ("tiny_f32", dict(Hq=2, Hkv=2, N=1024))):
        cfg = CONFIGS[name].with_sizes(**kw)
        x = make_inputs(cfg)
        dev = torch.device("cuda:0")
        q = x["q"].to(dev)
        p = ssa.problem_for(q, q, budget=4)
        got = ssa.pool_blocks(p, q).cpu().numpy()
        assert np.array_equal(got, O.pool_blocks(x["q"].float().numpy(), 64))


# ---------------------------------------------------------------- full-size workloads

def row_loss_check(name, hf_gpu, hs_gpu, hf_ref, hs_ref):
    """Alignment loss on sampled rows ("Bidirectional Attention Alignment":
    both losses are the mean squared difference of the two streams): each
    row's sum over d of (h_full - h_sparse)^2 from the GPU's outputs against
    the oracle's, per row within the 2e-2 bar and summed over the rows within
    the 5e-2 relative bar of the whole-problem comparisons."""
    g = ((np.asarray(hf_gpu, np.float64) - np.asarray(hs_gpu, np.float64)) ** 2).sum(axis=-1)
    w = ((np.asarray(hf_ref, np.float64) - np.asarray(hs_ref, np.float64)) ** 2).sum(axis=-1)
    assert_close(f"row loss {name}", g, w, BF16_ABS)
    if w.sum() > 1e-12:
        rel = abs(g.sum() - w.sum()) / w.sum()
        assert rel <= 5e-2, f"row loss {name}: relative error {rel:.3e} of the sampled sum"


def sampled_compare(cfg, x, got, *, budget, heads, rows_per_head, seed, group_select=False,
                    sparse=None):
    """Every selected index, and sampled rows of the streams, delta and the
    per-row alignment loss, against the oracle. `sparse`: the outputs of a
    sparse-only call on the same inputs, whose h_sparse is checked on the
    same rows."""
    xn = np_inputs(x)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    say(f"[oracle] selection for {cfg.name} budget {budget}")
    ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=cfg.block, budget=budget,
                                       n_sink=cfg.n_sink, n_local=cfg.n_local, head_map=hm,
                                       group_shared=group_select)
    assert np.array_equal(got["idx"].numpy(), ref_idx), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), ref_cnt), "block counts differ"
    if sparse is not None:
        assert np.array_equal(sparse["idx"].numpy(), ref_idx), "sparse-only: selected blocks differ"
        assert np.array_equal(sparse["cnt"].numpy(), ref_cnt), "sparse-only: block counts differ"
        assert "h_full" not in sparse
    rows = {bh: sample_rows(cfg.Nq, rows_per_head, seed + i) for i, bh in enumerate(heads)}
    say(f"[oracle] attention rows for {cfg.name} budget {budget}")
    res = O.dual_attention(xn["q"], xn["k"], xn["v"], ref_idx, block=cfg.block,
                           scale=scale_for(cfg), head_map=hm, rows=rows)
    for (b, h), (r, hf, hs, dl) in res.items():
        gf, gs = to_np64(got["h_full"][b, h, r]), to_np64(got["h_sparse"][b, h, r])
        assert_close(f"h_full[{b},{h}]", gf, hf, BF16_ABS, BF16_REL_L2)
        assert_close(f"h_sparse[{b},{h}]", gs, hs, BF16_ABS, BF16_REL_L2)
        assert_close(f"delta[{b},{h}]", to_np64(got["delta"][b, h, r]), dl, BF16_DELTA_ABS)
        row_loss_check(f"[{b},{h}]", gf, gs, hf, hs)
        if sparse is not None:
            assert_close(f"h_sparse (sparse-only)[{b},{h}]", to_np64(sparse["h_sparse"][b, h, r]),
                         hs, BF16_ABS, BF16_REL_L2)
    # every row of every head: delta is a probability
    d = got["delta"]
    assert float(d.min()) >= 0.0 and float(d.max()) <= 1.0
    # the loss kernel over the whole problem against the mean squared
    # difference of the GPU's own outputs (float64 partials, float32 result)
    ls, _, _, _ = O.align_loss(to_np64(got["h_full"]), to_np64(got["h_sparse"]))
    assert abs(float(got["loss"][0]) - ls) <= 1e-6 * ls + 1e-12
    assert float(got["loss"][1]) == float(got["loss"][0])
    return ref_idx


def test_full_size_mha_4k(ssa):
    cfg = CONFIGS["mha_4k"]
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=cfg.budget)
    full_compare(cfg, x, got, budget=cfg.budget)


def test_full_size_gqa_8k_peaked(ssa):
    cfg = CONFIGS["gqa_8k_peaked"]
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=cfg.budget)
    sampled_compare(cfg, x, got, budget=cfg.budget, heads=[(0, 0), (1, 13), (2, 22), (3, 31)],
                    rows_per_head=384, seed=20)


@pytest.mark.parametrize("budget", [4, 8, 16, 32])
def test_full_size_gqa_32k(ssa, budget):
    """The 32K sweep at the benchmark's launch configuration, dual mode and
    sparse-only (inference) mode on the same inputs."""
    cfg = CONFIGS["gqa_32k_sweep"].with_budget(budget)
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=budget)
    sp = gpu_run(ssa, x, budget=budget, sparse_only=True)
    sampled_compare(cfg, x, got, budget=budget, heads=[(0, 3), (0, 30)], rows_per_head=256,
                    seed=30 + budget, sparse=sp)


def test_full_size_gqa_32k_group_select(ssa):
    """Group-shared selection at the 32K launch configuration: every index,
    sampled rows of two heads of one group and one of another."""
    cfg = CONFIGS["gqa_32k_sweep"].with_budget(16)
    say(f"[parity] full size group select {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=16, group_select=True)
    sampled_compare(cfg, x, got, budget=16, heads=[(0, 4), (0, 6), (0, 29)], rows_per_head=256,
                    seed=77, group_select=True)


def test_full_size_paper_16k_b16(ssa):
    """The pages' model shape at its launch configuration: 16-token blocks,
    D 64, 32 q heads over 2 kv heads, 16K tokens."""
    cfg = CONFIGS["paper_16k_b16"]
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=cfg.budget, block=16)
    sp = gpu_run(ssa, x, budget=cfg.budget, block=16, sparse_only=True)
    sampled_compare(cfg, x, got, budget=cfg.budget, heads=[(0, 0), (0, 17)], rows_per_head=256,
                    seed=91, sparse=sp)


def test_full_size_decode_64k(ssa):
    """The 64K decode workload at the benchmark's launch configuration (the
    caller's pooled-key table, 64 sequences), dual mode and sparse-only mode:
    on 4 sampled sequences (all heads) every output and the alignment loss of
    those sequences against the oracle; the loss kernel over all 64."""
    cfg = CONFIGS["gqa_decode_64k"]
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=cfg.budget, k_pooled=True)
    sp = gpu_run(ssa, x, budget=cfg.budget, k_pooled=True, sparse_only=True)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    seqs = [0, 17, 42, 63]
    xs = {k: v[seqs].float().numpy() for k, v in x.items()}
    say("[oracle] decode selection and attention on sampled sequences")
    assert np.array_equal(got["k_pooled"][seqs].numpy(), O.pool_blocks(xs["k"], 64))
    ref = O.ssa_forward(xs["q"], xs["k"], xs["v"], block=64, budget=cfg.budget, n_sink=1,
                        n_local=1, head_map=hm)
    for tag, r in (("dual", got), ("sparse-only", sp)):
        assert np.array_equal(r["idx"][seqs].numpy(), ref["idx"]), tag
        assert np.array_equal(r["cnt"][seqs].numpy(), ref["cnt"]), tag
        assert_close(f"h_sparse ({tag})", to_np64(r["h_sparse"][seqs]), ref["h_sparse"], BF16_ABS,
                     BF16_REL_L2)
    assert "h_full" not in sp
    assert_close("h_full", to_np64(got["h_full"][seqs]), ref["h_full"], BF16_ABS, BF16_REL_L2)
    assert_close("delta", to_np64(got["delta"][seqs]), ref["delta"], BF16_DELTA_ABS)
    # the alignment loss of the sampled sequences: the GPU outputs' mean
    # squared difference against the oracle's loss on the same sequences
    gh = to_np64(got["h_full"][seqs]) - to_np64(got["h_sparse"][seqs])
    lg = float((gh * gh).mean())
    assert abs(lg - ref["loss_sparsity"]) <= BF16_ABS
    assert abs(lg - ref["loss_sparsity"]) <= 5e-2 * ref["loss_sparsity"], (lg, ref["loss_sparsity"])
    row_loss_check("decode", to_np64(got["h_full"][seqs]), to_np64(got["h_sparse"][seqs]),
                   ref["h_full"], ref["h_sparse"])
    ls, _, _, _ = O.align_loss(to_np64(got["h_full"]), to_np64(got["h_sparse"]))
    assert abs(float(got["loss"][0]) - ls) <= 1e-6 * ls + 1e-12
