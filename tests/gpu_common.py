"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.ssa_oracle as O

BF16_ABS = 2e-2      # max-abs bar for bf16 inputs, float32 accumulation
F32_ABS = 1e-5       # max-abs bar for float32 problems
BF16_REL_L2 = 1e-2   # relative L2 bar (informative, asserted)
# delta = l_drop / (l_sel + l_drop) from sums of bf16-rounded weights (each
# relative error <= 2^-9): |d delta| <= delta (1 - delta) * 2 * 2^-9 <= 2^-10
BF16_DELTA_ABS = 1e-3


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_run(ssa, x, *, budget, n_sink=1, n_local=1, head_map=None, want_lse=False,
            want_grads=False, sparse_only=False, k_pooled=False, group_select=False, block=64):
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
                             block_size=block)
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
