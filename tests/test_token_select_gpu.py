"""Per-token selection (SSA_SELECT_TOKEN: one block list per query row)
through the C ABI against the fp64 oracle.

Lists and counts must match bit for bit; the two streams, delta, the losses
and lse are held to the same bars as the per-block paths (2e-2 max-abs for
bf16 with float32 accumulation, 1e-5 for float32). The 32K case compares
every list of sampled rows with the oracle, checks properties of every list,
and compares the attention of the sampled rows.
"""
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


# (config, size overrides, budget, n_sink, n_local, block, sparse_only, head_map)
TOKEN_SMALL = [
    ("tiny_f32", {}, 4, 1, 1, 64, False, None),
    ("tiny_f32", dict(Hq=2, Hkv=1, N=1024), 5, 0, 1, 64, False, None),
    ("tiny_f32", dict(Hq=2, Hkv=1, N=768), 3, 1, 1, 64, True, None),
    ("mha_4k", dict(Hq=2, Hkv=2, N=1024), 4, 1, 1, 64, False, None),
    ("mha_4k", dict(Hq=2, Hkv=1, N=1024, D=64), 3, 1, 1, 64, False, None),
    ("mha_4k", dict(Hq=1, Hkv=1, N=64), 1, 0, 1, 64, False, None),
    ("mha_4k", dict(Hq=2, Hkv=2, N=640), 3, 0, 0, 64, False, None),
    ("gqa_8k_peaked", dict(B=2, Hq=8, Hkv=2, N=1024), 4, 1, 1, 64, False, [1, 0, 0, 1, 1, 0, 1, 0]),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=2048, planted=False), 6, 2, 2, 64, False, None),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=2048, planted=False), 6, 1, 1, 64, True, None),
    # longer lists: 32- and 64-entry register lists
    ("gqa_8k_peaked", dict(B=1, Hq=2, Hkv=1, N=4096, planted=False), 24, 1, 1, 64, False, None),
    ("gqa_8k_peaked", dict(B=1, Hq=2, Hkv=1, N=4096, planted=False), 40, 1, 2, 64, False, None),
    # 16-token blocks
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024), 16, 1, 1, 16, False, None),
    ("paper_16k_b16", dict(Hq=2, Hkv=2, N=640, D=128), 6, 0, 0, 16, False, None),
    ("paper_16k_b16", dict(Hq=4, Hkv=2, N=2048, planted=False), 12, 2, 2, 16, False, None),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024, D=128), 16, 1, 1, 16, True, None),
    ("paper_16k_b16", dict(Hq=2, Hkv=1, N=2048, planted=False), 64, 1, 1, 16, False, None),
]


@pytest.mark.parametrize("name,kw,budget,n_sink,n_local,block,sparse,hm", TOKEN_SMALL,
                         ids=[f"tok-{i}-{t[0]}" for i, t in enumerate(TOKEN_SMALL)])
def test_token_parity(ssa, name, kw, budget, n_sink, n_local, block, sparse, hm):
    cfg = CONFIGS[name].with_sizes(budget=budget, n_sink=n_sink, n_local=n_local, block=block, **kw)
    say(f"[parity] per-token {cfg} sparse_only={sparse} head_map={hm}")
    x = make_inputs(cfg, head_map=hm)
    got = gpu_run(ssa, x, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                  want_lse=not sparse, sparse_only=sparse, block=block, token_select=True)
    assert tuple(got["idx"].shape) == (cfg.B, cfg.Hq, cfg.Nq, budget)
    full_compare(cfg, x, got, budget=budget, n_sink=n_sink, n_local=n_local, head_map=hm,
                 lse=not sparse, sparse_only=sparse, token_select=True)


def test_token_rows_of_a_block_differ(ssa):
    """The rows of one query block pick different blocks (the data are iid),
    and a problem whose rows repeat one vector per block gives every row its
    block's per-block list."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=2, Hkv=1, N=2048, budget=5, planted=False)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=5, token_select=True)
    idx = got["idx"].numpy()
    assert any(not np.array_equal(idx[0, 0, r], idx[0, 0, r - 1])
               for r in range(1, 2048) if r % 64), "rows of a block agree everywhere"
    q = x["q"].view(1, 2, 32, 64, 128)[:, :, :, :1].expand(1, 2, 32, 64, 128).reshape(1, 2, 2048, 128)
    xr = dict(x, q=q.contiguous())
    tok = gpu_run(ssa, xr, budget=5, token_select=True)
    blk = gpu_run(ssa, xr, budget=5)
    rows = np.arange(2048) // 64
    assert np.array_equal(tok["idx"].numpy(), blk["idx"].numpy()[:, :, rows])
    assert np.array_equal(tok["cnt"].numpy(), blk["cnt"].numpy()[:, :, rows])
    for key in ("h_full", "h_sparse", "delta"):
        assert torch.equal(tok[key], blk[key]) or \
            float((tok[key].double() - blk[key].double()).abs().max()) <= BF16_ABS, key


def test_token_decode_is_per_head(ssa):
    """One query: per-token and per-head selection are the same problem."""
    cfg = CONFIGS["gqa_decode_64k"].with_sizes(B=2, Hq=8, Hkv=2, N=2048, budget=6)
    x = make_inputs(cfg)
    a = gpu_run(ssa, x, budget=6, want_lse=True, token_select=True)
    b = gpu_run(ssa, x, budget=6, want_lse=True)
    for key in ("idx", "cnt", "h_full", "h_sparse", "delta", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_token_full_size_gqa_32k(ssa):
    """Per-token selection at the 32K GQA launch configuration (budget 16):
    sampled rows of three heads bit-exact against the oracle, every list
    ascending with its forced blocks and the right count, and the attention
    of the sampled rows within the bars."""
    cfg = CONFIGS["gqa_32k_sweep"].with_budget(16)
    say(f"[parity] per-token full size {cfg}")
    x = make_inputs(cfg, workers=16)
    got = gpu_run(ssa, x, budget=16, token_select=True)
    idx, cnt = got["idx"].numpy(), got["cnt"].numpy()
    n, nb = cfg.N, cfg.N // cfg.block
    diag = np.arange(n) // cfg.block
    want_cnt = np.minimum(16, diag + 1)
    assert (cnt == want_cnt[None, None]).all(), "list lengths"
    valid = np.arange(16)[None, None, None, :] < cnt[..., None]
    assert ((idx >= 0) == valid).all()
    steps = np.diff(idx, axis=-1)
    assert ((steps > 0) | ~valid[..., 1:]).all(), "lists ascending"
    assert (idx[..., 0] == 0).all(), "sink block"
    last = np.take_along_axis(idx, (cnt - 1)[..., None], -1)[..., 0]
    assert (last == diag[None, None]).all(), "local block"
    assert (idx[valid] < nb).all()
    xn = np_inputs(x)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    heads = [(0, 3), (0, 17), (0, 30)]
    rows = {bh: sample_rows(n, 256, 400 + i) for i, bh in enumerate(heads)}
    say("[oracle] per-token selection of sampled rows")
    ref_idx, ref_cnt = O.select_blocks(xn["q"], xn["k"], block=64, budget=16, n_sink=1, n_local=1,
                                       head_map=hm, per_token=True, rows=rows)
    for (b, h), r in rows.items():
        assert np.array_equal(idx[b, h, r], ref_idx[b, h, r]), (b, h)
        assert np.array_equal(cnt[b, h, r], ref_cnt[b, h, r]), (b, h)
    say("[oracle] attention of sampled rows")
    res = O.dual_attention(xn["q"], xn["k"], xn["v"], ref_idx, block=64, scale=scale_for(cfg),
                           head_map=hm, rows=rows, per_token=True)
    for (b, h), (r, hf, hs, dl) in res.items():
        assert_close(f"h_full[{b},{h}]", to_np64(got["h_full"][b, h, r]), hf, BF16_ABS, BF16_REL_L2)
        assert_close(f"h_sparse[{b},{h}]", to_np64(got["h_sparse"][b, h, r]), hs, BF16_ABS,
                     BF16_REL_L2)
        assert_close(f"delta[{b},{h}]", to_np64(got["delta"][b, h, r]), dl, BF16_DELTA_ABS)
