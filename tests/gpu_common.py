"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.ssa_oracle as O
from ssa_inputs import default_head_map, scale_for

BF16_ABS = 2e-2      # max-abs bar for bf16 inputs, float32 accumulation
F32_ABS = 1e-5       # max-abs bar for float32 problems
BF16_REL_L2 = 1e-2   # relative L2 bar (informative, asserted)
# delta = l_drop / (l_sel + l_drop) from sums of bf16-rounded weights (each
# within the bf16 unit roundoff 2^-8, an 8-bit significand):
# |d delta| <= delta (1 - delta) * 2 * 2^-8 <= 2^-9
BF16_DELTA_ABS = 2e-3


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_run(ssa, x, *, budget, n_sink=1, n_local=1, head_map=None, want_lse=False,
            want_grads=False, sparse_only=False, k_pooled=False, group_select=False, block=64,
            token_select=False):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kp = None
    if k_pooled:
        p = ssa.problem_for(q, k, budget=budget, n_sink=n_sink, n_local=n_local, head_map=head_map,
                            block_size=block)
        kp = ssa.pool_blocks(p, k)
    out = ssa.dual_attention(q, k, v, budget=budget, n_sink=n_sink, n_local=n_local,
                             head_map=head_map, want_lse=want_lse, want_grads=want_grads,
                             sparse_only=sparse_only, k_pooled=kp, group_select=group_select,
                             block_size=block, token_select=token_select)
    torch.cuda.synchronize()
    res = {}
    for key, val in out.items():
        res[key] = val.cpu()
    if kp is not None:
        res["k_pooled"] = kp.cpu()
    return res


def assert_close(name, got, want, atol, rel_l2=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    err = np.abs(got - want).max() if got.size else 0.0
    assert err <= atol, f"{name}: max-abs error {err:.3e} > {atol:.1e}"
    if rel_l2 is not None and got.size:
        den = np.linalg.norm(want)
        if den > 0:
            r = np.linalg.norm(got - want) / den
            assert r <= rel_l2, f"{name}: relative L2 error {r:.3e} > {rel_l2:.1e}"
    return err


def sample_rows(nq: int, n: int, seed: int) -> np.ndarray:
    """Rows spread over the sequence: the first and last query blocks in
    full, plus random rows, sorted."""
    r = np.random.default_rng(seed)
    fixed = list(range(min(64, nq))) + list(range(max(0, nq - 64), nq))
    extra = r.choice(nq, size=min(nq, max(0, n - len(fixed))), replace=False).tolist()
    return np.array(sorted(set(fixed + extra)), dtype=np.int64)


def np_inputs(x):
    return {k: v.float().numpy() for k, v in x.items()}


def full_compare(cfg, x, got, *, budget, n_sink=1, n_local=1, head_map=None, lse=False,
                 sparse_only=False, group_select=False, token_select=False):
    """Whole-problem comparison with the oracle: indices and counts bit-exact,
    streams, delta, losses (and lse) within the bars."""
    xn = np_inputs(x)
    ref = O.ssa_forward(xn["q"], xn["k"], xn["v"], block=cfg.block, budget=budget, n_sink=n_sink,
                        n_local=n_local, head_map=head_map, group_shared=group_select,
                        per_token=token_select)
    assert np.array_equal(got["idx"].numpy(), ref["idx"]), "selected blocks differ"
    assert np.array_equal(got["cnt"].numpy(), ref["cnt"]), "block counts differ"
    f32 = cfg.dtype == "f32"
    atol = F32_ABS if f32 else BF16_ABS
    rel = 1e-5 if f32 else BF16_REL_L2
    assert_close("h_sparse", to_np64(got["h_sparse"]), ref["h_sparse"], atol, rel)
    if not sparse_only:
        assert_close("h_full", to_np64(got["h_full"]), ref["h_full"], atol, rel)
        assert_close("delta", to_np64(got["delta"]), ref["delta"],
                     F32_ABS if f32 else BF16_DELTA_ABS)
        ls = float(got["loss"][0]); lc = float(got["loss"][1])
        assert ls == lc
        want = ref["loss_sparsity"]
        assert abs(ls - want) <= (F32_ABS if f32 else BF16_ABS)
        if want > 1e-6:
            assert abs(ls - want) / want <= (1e-4 if f32 else 5e-2), (ls, want)
    if lse:
        q = torch.from_numpy(xn["q"]).double(); k = torch.from_numpy(xn["k"]).double()
        hm = head_map or default_head_map(cfg.Hq, cfg.Hkv)
        kk = k[:, hm]
        z = scale_for(cfg) * q @ kk.transpose(-1, -2)
        nq, nk = q.shape[2], k.shape[2]
        pos = torch.arange(nq) + nk - nq
        causal = torch.arange(nk)[None, :] <= pos[:, None]
        full = torch.logsumexp(z.masked_fill(~causal, -math.inf), -1)
        idx = torch.from_numpy(ref["idx"]).long()
        nkb = nk // cfg.block
        sel = torch.zeros(*idx.shape[:3], nkb + 1, dtype=torch.bool)
        sel.scatter_(-1, torch.where(idx >= 0, idx, nkb), True)
        sel = sel[..., :nkb]
        if nq == 1:
            rb = torch.zeros(nq, dtype=torch.long)
        else:
            rb = torch.arange(nq) if token_select else torch.arange(nq) // cfg.block
        tokmask = sel[:, :, rb][..., torch.arange(nk) // cfg.block] & causal
        sparse = torch.logsumexp(z.masked_fill(~tokmask, -math.inf), -1)
        # bf16: the row sums add the bfloat16-rounded weights (relative error
        # <= 2^-8 each, the bf16 unit roundoff), so |d lse| <= ln(1 + 2^-8)
        # ~ 3.9e-3 (reached when one weight dominates a row); fp32 exact sums
        lse_tol = 1e-3 if f32 else 4e-3
        if not sparse_only:   # sparse-only calls leave plane 0 untouched
            assert_close("lse_full", got["lse"][0].double().numpy(), full.numpy(), lse_tol)
        assert_close("lse_sparse", got["lse"][1].double().numpy(), sparse.numpy(), lse_tol)
    return ref
