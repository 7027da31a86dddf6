"""Parity of the HIP backward pass (through the C ABI) with the fp64 oracle.

The GPU runs selection, the forward (for h_full, h_sparse and lse) and the
backward; the oracle selects its own blocks (which must equal the GPU's bit
for bit) and computes dq, dk, dv from the same seeded inputs and upstream
gradients in float64.

Bars, per gradient tensor: max-abs error at most BWD_NORM times the largest
|oracle value| of that tensor, and relative L2 error at most BWD_REL_L2.
bf16: P and dS enter the bf16 products rounded to bf16 (relative error
2^-8 each, the bf16 unit roundoff), the row sums rowsum(dO * O) use the
bf16-rounded forward output, and every output is rounded once more (2^-8);
summed over a row's keys or a key's rows these give errors of a few 2^-8 of
the largest terms, well inside
2e-2 of the tensor's largest value and 1e-2 in relative L2. float32: exp2,
float32 sums of up to N terms: 1e-5 of the largest value.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.ssa_oracle as O
from gpu_common import to_np64
from ssa_inputs import CONFIGS, default_head_map, make_grads, make_inputs, scale_for

pytestmark = pytest.mark.gpu

BWD_NORM = {"bf16": 2e-2, "f32": 1e-5}
BWD_REL_L2 = {"bf16": 1e-2, "f32": 1e-5}


@pytest.fixture(scope="module")
def ssa():
    import block_sparse_full_amd as m
    m.load_library()
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_bwd(ssa, cfg, x, grads, *, budget, use_full=True, use_sparse=True, head_map=None,
            group_select=False, token_select=False):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    p = ssa.problem_for(q, k, budget=budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                        head_map=head_map, group_select=group_select, block_size=cfg.block,
                        token_select=token_select)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    fwd = ssa.attn_fwd(p, q, k, v, idx, cnt, want_lse=True, ws=ws)
    gf = grads["d_full"].to(dev) if use_full else None
    gs = grads["d_sparse"].to(dev) if use_sparse else None
    out = ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], h_full=fwd["h_full"],
                       h_sparse=fwd["h_sparse"], d_full=gf, d_sparse=gs)
    torch.cuda.synchronize()
    res = {n: out[n].cpu() for n in ("dq", "dk", "dv")}
    res["idx"], res["cnt"] = idx.cpu(), cnt.cpu()
    return res


def check_grad(name, got, want, dtype):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    scale = np.abs(want).max()
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    say(f"  {name}: max|ref| {scale:.3e} max-abs err {err:.3e} ({err / scale:.2e} of max) "
        f"rel-L2 {rel:.2e}")
    assert err <= BWD_NORM[dtype] * scale, f"{name}: max-abs error {err:.3e} > {BWD_NORM[dtype]:.0e} x {scale:.3e}"
    assert rel <= BWD_REL_L2[dtype], f"{name}: relative L2 error {rel:.3e}"


def full_compare(ssa, cfg, *, budget=None, use_full=True, use_sparse=True, head_map=None,
                 group_select=False, token_select=False):
    budget = budget or cfg.budget
    say(f"[bwd] {cfg.name} B{cfg.B} Hq{cfg.Hq} Hkv{cfg.Hkv} N{cfg.N} D{cfg.D} bs{cfg.block} "
        f"budget {budget} full={use_full} sparse={use_sparse} group={group_select} "
        f"token={token_select}")
    x = make_inputs(cfg, head_map=head_map)
    grads = make_grads(cfg)
    got = gpu_bwd(ssa, cfg, x, grads, budget=budget, use_full=use_full, use_sparse=use_sparse,
                  head_map=head_map, group_select=group_select, token_select=token_select)
    hm = head_map or default_head_map(cfg.Hq, cfg.Hkv)
    xn = {n: t.double().numpy() for n, t in x.items()}
    idx, cnt = O.select_blocks(xn["q"], xn["k"], block=cfg.block, budget=budget,
                               n_sink=cfg.n_sink, n_local=cfg.n_local, head_map=hm,
                               group_shared=group_select, per_token=token_select)
    assert np.array_equal(got["idx"].numpy(), idx), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), cnt), "block counts differ"
    gf = grads["d_full"].double().numpy() if use_full else None
    gs = grads["d_sparse"].double().numpy() if use_sparse else None
    dq, dk, dv = O.dual_attention_backward(xn["q"], xn["k"], xn["v"], idx, gf, gs, block=cfg.block,
                                           scale=scale_for(cfg), head_map=hm,
                                           per_token=token_select)
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv)):
        check_grad(name, to_np64(got[name]), want, cfg.dtype)


SMALL = [
    ("tiny_f32", {}, {}),
    ("mha_4k", dict(Hq=2, Hkv=2, N=512), dict(budget=4)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=1024), dict(budget=4)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=1024), dict(budget=4, use_full=False)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=1024), dict(budget=4, use_sparse=False)),
    ("gqa_8k_peaked", dict(B=2, Hq=4, Hkv=2, N=576), dict(budget=3, head_map=[1, 0, 0, 1])),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=704, D=64), dict(budget=4)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=1024), dict(budget=4, group_select=True)),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024), dict(budget=16)),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024), dict(budget=16, use_full=False)),
    ("paper_16k_b16", dict(Hq=2, Hkv=1, N=576, D=128), dict(budget=8)),
    ("tiny_f32", dict(Hq=2, Hkv=1, N=256, D=128), dict(budget=2, use_full=False)),
    # 64 x 32 kv heads x 2 key tiles = 4096 (key tile, kv head) pairs: the
    # full-stream dK/dV pass runs as one head group, writing bfloat16 directly
    # (full stream only) or one float32 slot (both streams)
    ("gqa_8k_peaked", dict(B=64, Hq=32, Hkv=32, N=256, D=64), dict(budget=2, use_sparse=False)),
    ("gqa_8k_peaked", dict(B=64, Hq=32, Hkv=32, N=256, D=64), dict(budget=2)),
    # per-token lists: float32, and bf16 (row masks) with blocks 64 and 16,
    # both streams and each alone, GQA, a permuted head map, D 64 and 128
    ("tiny_f32", dict(Hq=2, Hkv=1, N=512), dict(budget=3, token_select=True)),
    ("tiny_f32", dict(Hq=2, Hkv=2, N=256, D=128), dict(budget=2, token_select=True, use_full=False)),
    ("gqa_8k_peaked", dict(B=1, Hq=8, Hkv=2, N=1024), dict(budget=4, token_select=True)),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=1024, planted=False), dict(budget=5, token_select=True, use_full=False)),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=768, planted=False), dict(budget=5, token_select=True, use_sparse=False)),
    ("gqa_8k_peaked", dict(B=2, Hq=4, Hkv=2, N=576), dict(budget=3, token_select=True, head_map=[1, 0, 0, 1])),
    ("gqa_8k_peaked", dict(B=1, Hq=4, Hkv=1, N=704, D=64, planted=False), dict(budget=4, token_select=True)),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024), dict(budget=16, token_select=True)),
    ("paper_16k_b16", dict(Hq=4, Hkv=1, N=1024, planted=False), dict(budget=12, token_select=True, use_full=False)),
    ("paper_16k_b16", dict(Hq=2, Hkv=1, N=576, D=128, planted=False), dict(budget=8, token_select=True)),
]


@pytest.mark.parametrize("name,sizes,kw", SMALL,
                         ids=[f"{n}-{'-'.join(f'{a}{b}' for a, b in s.items())}-"
                              f"{'-'.join(f'{a}{b}' for a, b in k.items() if a != 'head_map')}"
                              for n, s, k in SMALL])
def test_backward_parity(ssa, name, sizes, kw):
    cfg = CONFIGS[name].with_sizes(**sizes) if sizes else CONFIGS[name]
    full_compare(ssa, cfg, **kw)


def test_backward_mid_size_full_compare(ssa):
    """8192 tokens, 8 q heads over 2 kv heads, budget 16, planted blocks,
    compared element by element in full. The sink block is selected by every
    query row, so its dK and dV sum all 8192 rows of four q heads in both
    streams; they are checked on their own against the largest value of that
    block, not only through the whole tensor's bar."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=8192)
    say(f"[bwd] mid size {cfg.name} B{cfg.B} Hq{cfg.Hq} Hkv{cfg.Hkv} N{cfg.N} budget 16")
    x = make_inputs(cfg, workers=16)
    grads = make_grads(cfg, workers=16)
    got = gpu_bwd(ssa, cfg, x, grads, budget=16)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    xn = {n: t.double().numpy() for n, t in x.items()}
    idx, cnt = O.select_blocks(xn["q"], xn["k"], block=cfg.block, budget=16, n_sink=cfg.n_sink,
                               n_local=cfg.n_local, head_map=hm)
    assert np.array_equal(got["idx"].numpy(), idx), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), cnt), "block counts differ"
    say("[oracle] backward of both streams, 8 heads x 8192 rows")
    dq, dk, dv = O.dual_attention_backward(xn["q"], xn["k"], xn["v"], idx,
                                           grads["d_full"].double().numpy(),
                                           grads["d_sparse"].double().numpy(), block=cfg.block,
                                           scale=scale_for(cfg), head_map=hm)
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv)):
        check_grad(name, to_np64(got[name]), want, "bf16")
    for name, want in (("dk", dk), ("dv", dv)):
        check_grad(f"{name} sink block", to_np64(got[name])[:, :, :cfg.block],
                   want[:, :, :cfg.block], "bf16")


def test_backward_full_budget_streams_agree(ssa):
    """Every causal block selected: a gradient fed to the sparse stream alone
    gives the same dq, dk, dv as the same gradient fed to the full stream."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=4, Hkv=1, N=512)
    x = make_inputs(cfg)
    g = make_grads(cfg)
    a = gpu_bwd(ssa, cfg, x, {"d_full": g["d_full"], "d_sparse": None}, budget=8,
                use_sparse=False)
    b = gpu_bwd(ssa, cfg, x, {"d_full": None, "d_sparse": g["d_full"]}, budget=8, use_full=False)
    for n in ("dq", "dk", "dv"):
        ref = to_np64(a[n])
        err = np.abs(to_np64(b[n]) - ref).max()
        assert err <= 1e-2 * np.abs(ref).max(), (n, err)


@pytest.mark.parametrize("kw", [dict(), dict(token_select=True)], ids=["per_block", "per_token"])
def test_backward_determinism(ssa, kw):
    """dK and dV sum the q heads of a group and the two streams in a fixed
    order (no atomics): two calls give identical bits."""
    cfg = CONFIGS["gqa_8k_peaked"].with_sizes(B=1, Hq=8, Hkv=2, N=1024)
    x = make_inputs(cfg)
    grads = make_grads(cfg)
    a = gpu_bwd(ssa, cfg, x, grads, budget=4, **kw)
    b = gpu_bwd(ssa, cfg, x, grads, budget=4, **kw)
    for name in ("dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("token_select", [False, True], ids=["per_block", "per_token"])
def test_backward_full_size_gqa_32k(ssa, token_select):
    """The 32K GQA workload (budget 16, planted blocks) at full size: dq on
    sampled rows and dk, dv of the last 128 keys of every kv head against the
    oracle restricted to the rows that reach them; over all keys, dk sums to
    zero and dv sums to the upstream gradients summed over rows (per kv
    head), as softmax's shift invariance and unit row sums require. Per-block
    lists, and per-token lists (the oracle selects the sampled rows)."""
    cfg = CONFIGS["gqa_32k_sweep"].with_budget(16)
    say(f"[bwd] full size {cfg.name} budget {cfg.budget} token_select={token_select}")
    x = make_inputs(cfg)
    grads = make_grads(cfg)
    got = gpu_bwd(ssa, cfg, x, grads, budget=cfg.budget, token_select=token_select)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    G = cfg.Hq // cfg.Hkv
    N, nkb = cfg.N, cfg.N // cfg.block
    scale = scale_for(cfg)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                     np.random.default_rng(7).choice(N, 64, replace=False)]))
    tail = np.arange(N - 128, N)
    dq = to_np64(got["dq"]); dk = to_np64(got["dk"]); dv = to_np64(got["dv"])
    gf_all = grads["d_full"].double().numpy(); gs_all = grads["d_sparse"].double().numpy()
    if token_select:
        both = np.union1d(rows, tail)
        tok_idx, _ = O.select_blocks(x["q"].double().numpy(), x["k"].double().numpy(),
                                     block=cfg.block, budget=cfg.budget, n_sink=cfg.n_sink,
                                     n_local=cfg.n_local, head_map=hm, per_token=True,
                                     rows={(0, h): both for h in range(cfg.Hq)})
    err_q = err_k = err_v = 0.0
    max_q = max_k = max_v = 0.0
    for g in range(cfg.Hkv):
        kk = x["k"][0, g].double().numpy(); vv = x["v"][0, g].double().numpy()
        dk_t = np.zeros((128, cfg.D)); dv_t = np.zeros((128, cfg.D))
        for h in [hh for hh in range(cfg.Hq) if hm[hh] == g]:
            qq = x["q"][0, h].double().numpy()
            qbar = O.pool_blocks(qq, cfg.block)
            kbar = O.pool_blocks(kk, cfg.block)
            scores = O.block_score_matrix(qbar, kbar)
            for part, rr in (("rows", rows), ("tail", tail)):
                sel = np.zeros((len(rr), nkb), dtype=bool)
                for i, r in enumerate(rr):
                    qb = r // cfg.block
                    if token_select:
                        lst = [int(v) for v in tok_idx[0, h, r] if v >= 0]
                        want = got["idx"][0, h, r].numpy()
                    else:
                        lst = O.select_row(scores[qb], qb, cfg.budget, cfg.n_sink, cfg.n_local)
                        want = got["idx"][0, h, qb].numpy()
                    sel[i, lst] = True
                    assert sorted(x for x in want.tolist() if x >= 0) == sorted(lst), (h, r)
                a, c, e = O.dual_attention_rows_backward(qq[rr], rr, kk, vv, sel, gf_all[0, h, rr],
                                                         gs_all[0, h, rr], block=cfg.block,
                                                         scale=scale)
                if part == "rows":
                    err_q = max(err_q, np.abs(dq[0, h, rr] - a).max())
                    max_q = max(max_q, np.abs(a).max())
                else:
                    dk_t += c[N - 128:]
                    dv_t += e[N - 128:]
        err_k = max(err_k, np.abs(dk[0, g, N - 128:] - dk_t).max()); max_k = max(max_k, np.abs(dk_t).max())
        err_v = max(err_v, np.abs(dv[0, g, N - 128:] - dv_t).max()); max_v = max(max_v, np.abs(dv_t).max())
        # invariants over all keys of the kv head
        heads = [hh for hh in range(cfg.Hq) if hm[hh] == g]
        want_v = sum((gf_all[0, h] + gs_all[0, h]).sum(axis=0) for h in heads)
        # per-element errors of a few 2^-8 of the terms: bound the sums by
        # 2e-2 of the summed magnitudes, d by d
        sv = dv[0, g].sum(axis=0)
        assert np.all(np.abs(sv - want_v) <= 2e-2 * np.abs(dv[0, g]).sum(axis=0)), (g, sv[:4], want_v[:4])
        sk = dk[0, g].sum(axis=0)
        assert np.all(np.abs(sk) <= 2e-2 * np.abs(dk[0, g]).sum(axis=0)), (g, sk[:4])
    say(f"  dq rows: err {err_q:.3e} of max {max_q:.3e}; dk tail: {err_k:.3e} of {max_k:.3e}; "
        f"dv tail: {err_v:.3e} of {max_v:.3e}")
    assert err_q <= BWD_NORM["bf16"] * max_q
    assert err_k <= BWD_NORM["bf16"] * max_k
    assert err_v <= BWD_NORM["bf16"] * max_v
