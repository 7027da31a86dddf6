"""ssa_align_loss_noalloc (the loss without a workspace, for callers that
cannot allocate device memory) against ssa_align_loss, through the C ABI.

Both run the same kernels with the same number of float64 partials, so the
losses and gradient seeds must agree bit for bit; the losses are also checked
against the oracle's mean squared error. Two calls in a row on one GPU, the
second on a smaller problem, so the second reads a scratch array that still
holds the first call's partials beyond its own range.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.ssa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssa():
    import block_sparse_full_amd as m
    m.load_library()
    return m


def outputs(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    hf = torch.randn(shape, generator=g).to(dtype)
    hs = (hf.float() + 0.1 * torch.randn(shape, generator=g)).to(dtype)
    return hf, hs


CASES = [
    # (shape [B, Hq, N, D], dtype): a problem with the full 1024 partials,
    # then one with 16 of them
    [((1, 8, 4096, 128), torch.bfloat16), ((1, 2, 512, 64), torch.bfloat16)],
    [((2, 4, 2048, 128), torch.float32), ((1, 1, 512, 64), torch.float32)],
]


@pytest.mark.parametrize("case", CASES, ids=["bf16", "f32"])
def test_noalloc_loss_matches_workspace_loss(ssa, case):
    dev = torch.device("cuda:0")
    for i, (shape, dtype) in enumerate(case):
        print(f"[no-alloc] call {i}: shape {shape} {dtype}", flush=True)
        sys.stdout.flush()
        hf, hs = outputs(shape, dtype, 100 + i)
        hfd, hsd = hf.to(dev), hs.to(dev)
        p = ssa.problem_for(hfd, hfd, budget=4)
        want_loss, want_gf, want_gs = ssa.align_loss(p, hfd, hsd, want_grads=True)
        got_loss, got_gf, got_gs = ssa.align_loss_noalloc(p, hfd, hsd, want_grads=True)
        torch.cuda.synchronize()
        assert torch.equal(got_loss.cpu(), want_loss.cpu()), (got_loss, want_loss)
        assert torch.equal(got_gf.cpu(), want_gf.cpu())
        assert torch.equal(got_gs.cpu(), want_gs.cpu())
        ls, _, _, _ = O.align_loss(hf.double().numpy(), hs.double().numpy())
        got = float(got_loss[0].cpu())
        assert float(got_loss[1].cpu()) == got
        # float64 partials rounded once to float32
        assert abs(got - ls) <= 2.0 ** -23 * ls + 1e-30, (got, ls)
