"""The HIP path at the largest supported key-block count (4096 blocks) against
the fp64 oracle: 16-token blocks at N = 65536 (per-block and per-token
lists), 64-token blocks at N = 262144, and decode over a 262144-token cache.
Selected blocks bit-exact (every list, or sampled rows for per-token lists),
streams and delta on sampled rows within the bf16 bars."""
import sys

import numpy as np
import pytest
import torch

import oracle.ssa_oracle as O
from gpu_common import (BF16_ABS, BF16_DELTA_ABS, BF16_REL_L2, assert_close, gpu_run,
                        np_inputs, sample_rows, to_np64)
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


def check_rows(cfg, xn, got, ref_idx, rows, token_select=False):
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    res = O.dual_attention(xn["q"], xn["k"], xn["v"], ref_idx, block=cfg.block,
                           scale=scale_for(cfg), head_map=hm, rows=rows, chunk=32,
                           per_token=token_select)
    for (b, h), (r, hf, hs, dl) in res.items():
        assert_close(f"h_full[{b},{h}]", to_np64(got["h_full"][b, h, r]), hf, BF16_ABS, BF16_REL_L2)
        assert_close(f"h_sparse[{b},{h}]", to_np64(got["h_sparse"][b, h, r]), hs, BF16_ABS,
                     BF16_REL_L2)
        assert_close(f"delta[{b},{h}]", to_np64(got["delta"][b, h, r]), dl, BF16_DELTA_ABS)


@pytest.mark.parametrize("token_select", [False, True], ids=["per_block", "per_token"])
def test_block16_4096_blocks(ssa, token_select):
    cfg = CONFIGS["paper_16k_b16"].with_sizes(Hq=2, Hkv=1, N=65536, budget=16)
    say(f"[limits] {cfg} token_select={token_select}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=16, block=16, token_select=token_select)
    xn = np_inputs(x)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    rows = {(0, h): sample_rows(cfg.N, 192, 500 + h) for h in range(cfg.Hq)}
    if token_select:
        ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=16, budget=16, n_sink=1,
                                           n_local=1, head_map=hm, per_token=True, rows=rows)
        for (b, h), r in rows.items():
            assert np.array_equal(got["idx"].numpy()[b, h, r], ref_idx[b, h, r]), (b, h)
            assert np.array_equal(got["cnt"].numpy()[b, h, r], ref_cnt[b, h, r]), (b, h)
    else:
        ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=16, budget=16, n_sink=1,
                                           n_local=1, head_map=hm)
        assert np.array_equal(got["idx"].numpy(), ref_idx), "selected blocks differ"
        assert np.array_equal(got["cnt"].numpy(), ref_cnt), "block counts differ"
    check_rows(cfg, xn, got, ref_idx, rows, token_select)


def test_block64_4096_blocks(ssa):
    cfg = CONFIGS["mha_4k"].with_sizes(Hq=1, Hkv=1, N=262144, D=64, budget=16, planted=False)
    say(f"[limits] {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=16)
    xn = np_inputs(x)
    ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=64, budget=16, n_sink=1,
                                       n_local=1, head_map=[0])
    assert np.array_equal(got["idx"].numpy(), ref_idx), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), ref_cnt), "block counts differ"
    check_rows(cfg, xn, got, ref_idx, {(0, 0): sample_rows(cfg.N, 160, 600)})


def test_decode_4096_blocks(ssa):
    cfg = CONFIGS["gqa_decode_64k"].with_sizes(B=2, Hq=8, Hkv=2, N=262144, budget=32)
    say(f"[limits] {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=32, k_pooled=True)
    xn = np_inputs(x)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    ref = O.ssa_forward(xn["q"], xn["k"], xn["v"], block=64, budget=32, n_sink=1, n_local=1,
                        head_map=hm)
    assert np.array_equal(got["idx"].numpy(), ref["idx"])
    assert np.array_equal(got["cnt"].numpy(), ref["cnt"])
    assert_close("h_full", to_np64(got["h_full"]), ref["h_full"], BF16_ABS, BF16_REL_L2)
    assert_close("h_sparse", to_np64(got["h_sparse"]), ref["h_sparse"], BF16_ABS, BF16_REL_L2)
    assert_close("delta", to_np64(got["delta"]), ref["delta"], BF16_DELTA_ABS)
