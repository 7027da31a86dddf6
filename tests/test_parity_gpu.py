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


def test_prefill_sparse_only_matches_dual_bitwise(ssa):
    """Two q heads per kv head: both modes run the per-head kernel, whose
    sparse-only walk is the first part of the dual walk."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=4, Hkv=2, N=1024, budget=4)
    x = make_inputs(cfg)
    dual = gpu_run(ssa, x, budget=4)
    sp = gpu_run(ssa, x, budget=4, sparse_only=True)
    assert torch.equal(sp["h_sparse"], dual["h_sparse"])


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


def test_block16_group_select(ssa):
    cfg = CONFIGS["paper_16k_b16"].with_sizes(Hq=8, Hkv=2, N=1024)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=16, want_lse=True, group_select=True, block=16)
    full_compare(cfg, x, got, budget=16, lse=True, group_select=True)


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

def sampled_compare(cfg, x, got, *, budget, heads, rows_per_head, seed, group_select=False):
    xn = np_inputs(x)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    say(f"[oracle] selection for {cfg.name} budget {budget}")
    ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=cfg.block, budget=budget,
                                       n_sink=cfg.n_sink, n_local=cfg.n_local, head_map=hm,
                                       group_shared=group_select)
    assert np.array_equal(got["idx"].numpy(), ref_idx), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), ref_cnt), "block counts differ"
    rows = {bh: sample_rows(cfg.Nq, rows_per_head, seed + i) for i, bh in enumerate(heads)}
    say(f"[oracle] attention rows for {cfg.name} budget {budget}")
    res = O.dual_attention(xn["q"], xn["k"], xn["v"], ref_idx, block=cfg.block,
                           scale=scale_for(cfg), head_map=hm, rows=rows)
    for (b, h), (r, hf, hs, dl) in res.items():
        assert_close(f"h_full[{b},{h}]", to_np64(got["h_full"][b, h, r]), hf, BF16_ABS, BF16_REL_L2)
        assert_close(f"h_sparse[{b},{h}]", to_np64(got["h_sparse"][b, h, r]), hs, BF16_ABS, BF16_REL_L2)
        assert_close(f"delta[{b},{h}]", to_np64(got["delta"][b, h, r]), dl, BF16_DELTA_ABS)
    # every row of every head: the streams coincide exactly where all causal
    # blocks are selected, and delta is a probability
    d = got["delta"]
    assert float(d.min()) >= 0.0 and float(d.max()) <= 1.0
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
    # loss over the whole problem against the oracle's loss on the GPU outputs
    ls, _, _, _ = O.align_loss(to_np64(got["h_full"]), to_np64(got["h_sparse"]))
    assert abs(float(got["loss"][0]) - ls) <= 1e-6 * ls + 1e-12


@pytest.mark.parametrize("budget", [4, 8, 16, 32])
def test_full_size_gqa_32k(ssa, budget):
    cfg = CONFIGS["gqa_32k_sweep"].with_budget(budget)
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=budget)
    sampled_compare(cfg, x, got, budget=budget, heads=[(0, 3), (0, 30)], rows_per_head=256,
                    seed=30 + budget)


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
    sampled_compare(cfg, x, got, budget=cfg.budget, heads=[(0, 0), (0, 17)], rows_per_head=256,
                    seed=91)


def test_full_size_decode_64k(ssa):
    cfg = CONFIGS["gqa_decode_64k"]
    say(f"[parity] full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=cfg.budget, k_pooled=True)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    seqs = [0, 17, 42, 63]
    xs = {k: v[seqs].float().numpy() for k, v in x.items()}
    say("[oracle] decode selection and attention on sampled sequences")
    assert np.array_equal(got["k_pooled"][seqs].numpy(), O.pool_blocks(xs["k"], 64))
    ref = O.ssa_forward(xs["q"], xs["k"], xs["v"], block=64, budget=cfg.budget, n_sink=1,
                        n_local=1, head_map=hm)
    assert np.array_equal(got["idx"][seqs].numpy(), ref["idx"])
    assert np.array_equal(got["cnt"][seqs].numpy(), ref["cnt"])
    assert_close("h_full", to_np64(got["h_full"][seqs]), ref["h_full"], BF16_ABS, BF16_REL_L2)
    assert_close("h_sparse", to_np64(got["h_sparse"][seqs]), ref["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("delta", to_np64(got["delta"][seqs]), ref["delta"], BF16_DELTA_ABS)
    ls, _, _, _ = O.align_loss(to_np64(got["h_full"]), to_np64(got["h_sparse"]))
    assert abs(float(got["loss"][0]) - ls) <= 1e-6 * ls + 1e-12
