"""The oracle against a pure-Python brute force on Hypothesis-drawn tiny
problems: explicit loops over rows, keys and dimensions, block selection by a
full sort of (-score, index), softmax with math.exp. Queries and keys are
small integers and block sizes powers of two, so every pooled mean and score
is a short dyadic fraction, exact in float64 whatever the summation order:
equal scores are then true ties and both sides must select the same blocks.
(With a block of 3 the means are thirds, the rounding of two mathematically
equal scores can differ with the order of operations, and a tie can break
either way.) The attention outputs agree to rounding.
Also checks the loss bound of the linear error result (the dropped mass
bounds |h_full - h_sparse| by 2 delta max |v|, so the MSE is at most the
mean of 4 delta^2 max|v|^2 / D per row)."""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.ssa_oracle as O


def brute_forward(q, k, v, *, block, budget, n_sink, n_local, head_map, scale, mode):
    """Lists of lists in, plain loops throughout."""
    B, Hq, nq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, nk = len(k[0]), len(k[0][0])
    nkb = nk // block

    def mean_block(x, j):   # x: [N][D]
        return [sum(x[j * block + t][d] for t in range(block)) / block for d in range(D)]

    def dot(a, b):
        return sum(a[d] * b[d] for d in range(D))

    def pick(scores, diag):
        forced = set(range(min(n_sink, diag + 1))) | set(range(max(0, diag - n_local + 1), diag + 1))
        cands = [j for j in range(diag + 1) if j not in forced]
        free = budget - len(forced)
        if len(cands) > free:
            cands = sorted(cands, key=lambda j: (-scores[j], j))[:free]
        return sorted(forced | set(cands))

    lists = {}
    for b in range(B):
        for h in range(Hq):
            g = head_map[h]
            kbar = [mean_block(k[b][g], j) for j in range(nkb)]
            nrep = nq if (mode == "token" or nq == 1) else nq // block
            for r in range(nrep):
                if mode == "token" or nq == 1:
                    rows = [r]
                    diag = (nk - nq + r) // block
                else:
                    rows = list(range(r * block, (r + 1) * block))
                    diag = r
                if mode == "group":
                    heads = [hh for hh in range(Hq) if head_map[hh] == g]
                else:
                    heads = [h]
                scores = [0.0] * nkb
                for hh in heads:
                    if nq == 1 or mode == "token":
                        rep = q[b][hh][r]
                    else:
                        rep = mean_block(q[b][hh], r)
                    for j in range(nkb):
                        scores[j] += dot(rep, kbar[j])
                sel = pick(scores, diag)
                for row in rows:
                    lists[(b, h, row)] = sel
    hf = np.zeros((B, Hq, nq, D)); hs = np.zeros((B, Hq, nq, D)); dl = np.zeros((B, Hq, nq))
    for b in range(B):
        for h in range(Hq):
            g = head_map[h]
            for row in range(nq):
                pos = nk - nq + row
                sel = set(lists[(b, h, row)])
                z = [scale * dot(q[b][h][row], k[b][g][j]) for j in range(pos + 1)]
                m = max(z)
                w = [math.exp(x - m) for x in z]
                ws = [w[j] if (j // block) in sel else 0.0 for j in range(pos + 1)]
                tot, tots = sum(w), sum(ws)
                for d in range(D):
                    hf[b, h, row, d] = sum(w[j] * v[b][g][j][d] for j in range(pos + 1)) / tot
                    hs[b, h, row, d] = sum(ws[j] * v[b][g][j][d] for j in range(pos + 1)) / tots
                dl[b, h, row] = (tot - tots) / tot
    return lists, hf, hs, dl


@st.composite
def problems(draw):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    Hq = Hkv * G
    block = draw(st.sampled_from([1, 2, 4]))
    nb = draw(st.integers(1, 6))
    D = draw(st.integers(1, 4))
    n_sink = draw(st.integers(0, 2))
    n_local = draw(st.integers(0, 2))
    lo = max(1, n_sink + n_local)
    budget = draw(st.integers(lo, max(lo, nb + 2)))
    decode = draw(st.booleans()) and nb > 1
    mode = draw(st.sampled_from(["head", "group", "token"]))
    perm = draw(st.permutations(list(range(Hq))))
    head_map = [perm[i] // G for i in range(Hq)]
    seed = draw(st.integers(0, 2 ** 31 - 1))
    nk = nb * block
    nq = 1 if decode else nk
    r = np.random.default_rng(seed)
    q = r.integers(-3, 4, size=(B, Hq, nq, D)).astype(np.float64)
    k = r.integers(-3, 4, size=(B, Hkv, nk, D)).astype(np.float64)
    v = r.standard_normal((B, Hkv, nk, D))
    scale = draw(st.sampled_from([0.25, 0.5, 1.0 / math.sqrt(D)]))
    return dict(q=q, k=k, v=v, block=block, budget=budget, n_sink=n_sink, n_local=n_local,
                head_map=head_map, scale=scale, mode=mode)


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(problems())
def test_oracle_matches_pure_python(p):
    q, k, v = p["q"], p["k"], p["v"]
    mode = p["mode"]
    lists, hf, hs, dl = brute_forward(q.tolist(), k.tolist(), v.tolist(), block=p["block"],
                                      budget=p["budget"], n_sink=p["n_sink"],
                                      n_local=p["n_local"], head_map=p["head_map"],
                                      scale=p["scale"], mode=mode)
    res = O.ssa_forward(q, k, v, block=p["block"], budget=p["budget"], n_sink=p["n_sink"],
                        n_local=p["n_local"], scale=p["scale"], head_map=p["head_map"],
                        group_shared=mode == "group", per_token=mode == "token")
    B, Hq, nq, D = q.shape
    per_row = mode == "token" or nq == 1
    for (b, h, row), sel in lists.items():
        lr = row if per_row else row // p["block"]
        if nq == 1:
            lr = 0
        got = [int(x) for x in res["idx"][b, h, lr] if x >= 0]
        assert got == sel, (b, h, row, got, sel)
        assert int(res["cnt"][b, h, lr]) == len(sel)
    assert np.allclose(res["h_full"], hf, atol=1e-12)
    assert np.allclose(res["h_sparse"], hs, atol=1e-12)
    assert np.allclose(res["delta"], dl, atol=1e-12)
    # |h_full - h_sparse| <= 2 delta max|v| per row, hence the loss bound
    vmax = np.sqrt((v ** 2).sum(-1)).max()
    diff = np.sqrt(((res["h_full"] - res["h_sparse"]) ** 2).sum(-1))
    assert (diff <= 2 * res["delta"] * vmax + 1e-12).all()
    bound = np.mean(4 * res["delta"] ** 2 * vmax ** 2 / D)
    assert res["loss_sparsity"] <= bound + 1e-12
    assert res["loss_sparsity"] == res["loss_commitment"]
    assert (res["delta"] >= -1e-15).all() and (res["delta"] <= 1 + 1e-15).all()
