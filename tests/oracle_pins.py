"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``check_*`` raises AssertionError when the oracle disagrees with a value
that does not come from the oracle itself: a hand-derived worked example, a
closed form, an exact special case, torch's scaled-dot-product attention in
float64, autograd of torch's MSE, or brute force on tiny inputs. The tests in
test_oracle.py run them; test_oracle_mutations.py plants plausible mistakes in
the oracle and checks that some pin fails for each.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle.ssa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- pooling

def check_pool_closed_form():
    """x[t, d] = t + d/2 -> the mean of block b is b*bs + (bs-1)/2 + d/2."""
    bs, nb, D = 8, 5, 3
    t = np.arange(nb * bs, dtype=np.float64)[:, None]
    d = np.arange(D, dtype=np.float64)[None, :]
    x = (t + 0.5 * d).astype(np.float32)
    got = O.pool_blocks(x, bs)
    want = np.array([[b * bs + (bs - 1) / 2 + 0.5 * dd for dd in range(D)] for b in range(nb)])
    assert got.dtype == np.float32 and got.shape == (nb, D)
    assert np.array_equal(got.astype(np.float64), want), (got, want)


def check_pool_mean_identity():
    """Mean(q K^T) = q Mean(K)^T over a block pair ("SSA: Achieving Sparser
    Attention ...", "Practical Implementation of SSA"), in both indices:
    mean_{i in qb, j in kb} q_i . k_j equals pooled(Q)[qb] . pooled(K)[kb]
    up to the float32 rounding of the pooled vectors."""
    r = _rng(1)
    bs, nb, D = 4, 3, 5
    q = r.standard_normal((nb * bs, D)).astype(np.float32)
    k = r.standard_normal((nb * bs, D)).astype(np.float32)
    qbar, kbar = O.pool_blocks(q, bs), O.pool_blocks(k, bs)
    s = O.block_score_matrix(qbar, kbar)
    for a in range(nb):
        for b in range(nb):
            brute = 0.0
            for i in range(a * bs, (a + 1) * bs):
                for j in range(b * bs, (b + 1) * bs):
                    brute += sum(float(q[i, dd]) * float(k[j, dd]) for dd in range(D))
            brute /= bs * bs
            tol = 1e-6 * (np.linalg.norm(qbar[a]) * np.linalg.norm(kbar[b]) + 1e-30)
            assert abs(s[a, b] - brute) <= tol, (a, b, s[a, b], brute)


def check_scores_exact_integers():
    """Small integer vectors: every summation order is exact, so the scores
    must equal the integer dot products exactly (pins operand order)."""
    r = _rng(2)
    qbar = r.integers(-8, 9, size=(4, 6)).astype(np.float32)
    kbar = r.integers(-8, 9, size=(7, 6)).astype(np.float32)
    s = O.block_score_matrix(qbar, kbar)
    want = qbar.astype(np.int64) @ kbar.astype(np.int64).T
    assert s.shape == (4, 7)
    assert np.array_equal(s, want.astype(np.float64))


# ---------------------------------------------------------------- selection

def check_select_constant_scores():
    """All scores equal: the free slots go to the lowest candidate indices."""
    s = np.zeros(20)
    got = O.select_row(s, diag=19, budget=6, n_sink=1, n_local=1)
    assert got == [0, 1, 2, 3, 4, 19], got
    got = O.select_row(s, diag=19, budget=6, n_sink=2, n_local=2)
    assert got == [0, 1, 2, 3, 18, 19], got


def check_select_duplicate_lower_index():
    """Two blocks with the same score compete for one slot: lower index wins,
    also between +0.0 and -0.0."""
    s = np.array([0.0, 1.0, 5.0, 3.0, 5.0, 2.0, 0.0])
    assert O.select_row(s, diag=6, budget=3, n_sink=1, n_local=1) == [0, 2, 6]
    s = np.array([9.0, -0.0, 0.0, -1.0, 0.0])
    assert O.select_row(s, diag=4, budget=3, n_sink=1, n_local=1) == [0, 1, 4]


def check_select_known_ranking():
    """Distinct scores: the top-`free` candidates by value, forced blocks
    kept even when they score lowest."""
    s = np.array([-100.0, 3.0, 9.0, 1.0, 7.0, 8.0, 2.0, -50.0])
    assert O.select_row(s, diag=7, budget=5, n_sink=1, n_local=1) == [0, 2, 4, 5, 7]
    # diag below the end of the score row: later blocks are not candidates
    assert O.select_row(s, diag=4, budget=3, n_sink=1, n_local=1) == [0, 2, 4]
    # fewer candidates than slots: every causal block
    assert O.select_row(s, diag=3, budget=8, n_sink=1, n_local=1) == [0, 1, 2, 3]


def check_select_invariants(seed=3, trials=200):
    """Brute-force property check on random rows: forced blocks present, list
    ascending and of size min(budget, diag+1), and every picked candidate
    ranks (score desc, index asc) above every candidate left out."""
    r = _rng(seed)
    for _ in range(trials):
        diag = int(r.integers(0, 40))
        n_sink, n_local = int(r.integers(0, 3)), int(r.integers(0, 3))
        budget = n_sink + n_local + int(r.integers(0, 10))
        s = np.round(r.standard_normal(diag + 1), 1)   # rounding makes ties
        sel = O.select_row(s, diag, budget, n_sink, n_local)
        forced = set(range(min(n_sink, diag + 1))) | set(range(max(0, diag - n_local + 1), diag + 1))
        assert sel == sorted(set(sel))
        assert forced <= set(sel)
        assert len(sel) == min(max(budget, len(forced)), diag + 1)
        picked = [x for x in sel if x not in forced]
        left = [x for x in range(diag + 1) if x not in sel]
        for p in picked:
            for o in left:
                assert (s[p] > s[o]) or (s[p] == s[o] and p < o), (s, sel, p, o)


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, mask, scale):
    """torch scaled-dot-product attention in float64 on the CPU."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None, None], t(k)[None, None], t(v)[None, None],
        attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    return out[0, 0].numpy()


def _random_problem(r, nb, bs, D, budget, n_sink, n_local, nq=None):
    n = nb * bs
    q = r.standard_normal((n if nq is None else nq, D))
    k = r.standard_normal((n, D)) * 1.5
    v = r.standard_normal((n, D))
    return q, k, v


def _sel_masks(q, k, bs, budget, n_sink, n_local):
    """Selected-block masks of each query row via the oracle's selection."""
    nq, n = q.shape[0], k.shape[0]
    idx, cnt = O.select_blocks(q[None, None], k[None, None], block=bs, budget=budget,
                               n_sink=n_sink, n_local=n_local, head_map=[0])
    nkb = n // bs
    rows_blocks = (np.arange(nq) // bs) if nq == n else np.zeros(nq, dtype=int)
    sel = np.stack([O.selected_mask(idx[0, 0, x], nkb) for x in rows_blocks])
    return idx[0, 0], sel


def check_attention_vs_sdpa(seed=4, trials=12):
    """Full stream == causal SDPA; sparse stream == SDPA under the boolean
    mask of the selected blocks' causal tokens; delta == full-softmax weight
    outside that mask."""
    r = _rng(seed)
    for _ in range(trials):
        bs = int(r.choice([2, 4, 8])); nb = int(r.integers(1, 7)); D = int(r.integers(1, 9))
        n_sink, n_local = int(r.integers(0, 2)), int(r.integers(1, 3))
        budget = n_sink + n_local + int(r.integers(0, 3))
        scale = float(r.uniform(0.2, 1.5))
        q, k, v = _random_problem(r, nb, bs, D, budget, n_sink, n_local)
        n = nb * bs
        _, sel = _sel_masks(q, k, bs, budget, n_sink, n_local)
        pos = np.arange(n)
        hf, hs, dl = O.dual_attention_rows(q, pos, k, v, sel, block=bs, scale=scale)
        causal = np.tril(np.ones((n, n), dtype=bool))
        smask = causal & sel[:, np.arange(n) // bs]
        assert np.allclose(hf, _sdpa(q, k, v, causal, scale), atol=1e-12, rtol=1e-12)
        assert np.allclose(hs, _sdpa(q, k, v, smask, scale), atol=1e-12, rtol=1e-12)
        z = scale * q @ k.T
        p = np.where(causal, np.exp(z - np.where(causal, z, -np.inf).max(1, keepdims=True)), 0)
        p /= p.sum(1, keepdims=True)
        assert np.allclose(dl, np.where(causal & ~smask, p, 0).sum(1), atol=1e-13)


def check_attention_constant_keys():
    """All keys equal: uniform weights. h_full[t] = mean(v[0..t]); h_sparse[t]
    = mean of v over the selected causal tokens; delta = dropped/(t+1)."""
    r = _rng(5)
    bs, nb, D = 4, 6, 3
    n = bs * nb
    q = r.standard_normal((n, D))
    k = np.tile(r.standard_normal((1, D)), (n, 1))
    v = r.standard_normal((n, D))
    idx, sel = _sel_masks(q, k, bs, 3, 1, 1)
    hf, hs, dl = O.dual_attention_rows(q, np.arange(n), k, v, sel, block=bs, scale=0.7)
    for t in range(n):
        toks = [j for j in range(t + 1) if sel[t, j // bs]]
        assert np.allclose(hf[t], v[:t + 1].mean(0), atol=1e-13)
        assert np.allclose(hs[t], v[toks].mean(0), atol=1e-13)
        assert abs(dl[t] - (t + 1 - len(toks)) / (t + 1)) < 1e-14


def check_attention_graded_logits():
    """Keys chosen so that the scaled logit of key j is ln(j+1): weights are
    (j+1)/sum. Pins the 1/sqrt(D) default scale and the exponential."""
    n, D = 12, 4
    scale = 1.0 / math.sqrt(D)
    q = np.zeros((n, D)); q[:, 0] = 1.0
    k = np.zeros((n, D)); k[:, 0] = np.log(np.arange(1, n + 1)) / scale
    v = np.stack([np.arange(n, dtype=np.float64), np.arange(n) ** 2.0, np.ones(n), -np.arange(n, dtype=np.float64)], 1)
    sel = np.ones((n, 3), dtype=bool)  # block 4, every block selected
    res = O.ssa_forward(q[None, None], k[None, None], v[None, None], block=4, budget=3,
                        n_sink=1, n_local=1)
    for t in range(n):
        w = np.arange(1, t + 2, dtype=np.float64); w /= w.sum()
        assert np.allclose(res["h_full"][0, 0, t], w @ v[:t + 1], atol=1e-12)
    hf, hs, dl = O.dual_attention_rows(q, np.arange(n), k, v, sel, block=4, scale=scale)
    assert np.allclose(hf, res["h_full"][0, 0], atol=1e-14)


def check_full_budget_equals_full(seed=6):
    """Budget covering every causal block: h_sparse == h_full, delta == 0,
    losses 0 (the decomposition's delta = 0 case)."""
    r = _rng(seed)
    bs, nb, D = 4, 5, 6
    q, k, v = _random_problem(r, nb, bs, D, nb, 1, 1)
    res = O.ssa_forward(q[None, None], k[None, None], v[None, None], block=bs,
                        budget=nb, n_sink=1, n_local=1)
    assert np.array_equal(res["idx"][0, 0, -1], np.arange(nb))
    assert np.allclose(res["h_sparse"], res["h_full"], atol=1e-14)
    assert np.all(res["delta"] == 0.0)
    assert res["loss_sparsity"] < 1e-28


def check_decomposition_and_bound(seed=7):
    """h_full = (1-delta) h_sparse + delta h_dropped, with h_dropped the
    attention over the dropped causal tokens alone (torch SDPA), and the
    linear bound ||h_full - h_sparse|| <= 2 delta max_j ||v_j|| (abstract of
    'SSA: Sparse Sparse Attention by Aligning ...': the error scales linearly
    with the dropped mass)."""
    r = _rng(seed)
    bs, nb, D = 4, 8, 5
    q, k, v = _random_problem(r, nb, bs, D, 3, 1, 1)
    n = bs * nb
    _, sel = _sel_masks(q, k, bs, 3, 1, 1)
    hf, hs, dl = O.dual_attention_rows(q, np.arange(n), k, v, sel, block=bs, scale=0.5)
    causal = np.tril(np.ones((n, n), dtype=bool))
    dmask = causal & ~sel[:, np.arange(n) // bs]
    vmax = np.linalg.norm(v, axis=1).max()
    checked = 0
    for t in range(n):
        err = np.linalg.norm(hf[t] - hs[t])
        assert err <= 2 * dl[t] * vmax + 1e-12
        if dmask[t].any():
            hd = _sdpa(q[t:t + 1], k, v, dmask[t:t + 1], 0.5)[0]
            assert np.allclose(hf[t], (1 - dl[t]) * hs[t] + dl[t] * hd, atol=1e-12)
            checked += 1
        else:
            assert dl[t] == 0.0
    assert checked > 0


def check_nested_budgets(seed=8):
    """Growing budgets select nested block sets and drop no more mass."""
    r = _rng(seed)
    bs, nb, D = 4, 12, 6
    q, k, v = _random_problem(r, nb, bs, D, 4, 1, 1)
    prev_idx, prev_delta = None, None
    for budget in (2, 4, 6, 12):
        res = O.ssa_forward(q[None, None], k[None, None], v[None, None], block=bs,
                            budget=budget, n_sink=1, n_local=1)
        if prev_idx is not None:
            for qb in range(nb):
                a = set(prev_idx[0, 0, qb][prev_idx[0, 0, qb] >= 0].tolist())
                b = set(res["idx"][0, 0, qb][res["idx"][0, 0, qb] >= 0].tolist())
                assert a <= b
            assert np.all(res["delta"] <= prev_delta + 1e-15)
        prev_idx, prev_delta = res["idx"], res["delta"]
    assert np.all(prev_delta == 0.0)


def check_gqa_equals_replicated(seed=9):
    """GQA with a head map equals MHA over K/V replicated per q head."""
    r = _rng(seed)
    B, Hq, Hkv, bs, nb, D = 2, 4, 2, 4, 4, 3
    n = bs * nb
    q = r.standard_normal((B, Hq, n, D)); k = r.standard_normal((B, Hkv, n, D)); v = r.standard_normal((B, Hkv, n, D))
    hm = [1, 0, 1, 0]
    a = O.ssa_forward(q, k, v, block=bs, budget=2, n_sink=1, n_local=1, head_map=hm)
    kr, vr = k[:, hm], v[:, hm]
    b = O.ssa_forward(q, kr, vr, block=bs, budget=2, n_sink=1, n_local=1)
    for key in ("idx", "cnt"):
        assert np.array_equal(a[key], b[key])
    for key in ("h_full", "h_sparse", "delta"):
        assert np.allclose(a[key], b[key], atol=1e-14)


def _brute_group_selection(q, k, bs, budget, n_sink, n_local, head_map):
    """Group-shared lists from exact rational arithmetic on the raw inputs:
    pooled means and dot products as Fractions, summed over the group's
    heads, ranked by (-score, index); forced blocks added."""
    B, Hq, nq, D = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    nqb, nkb = (1 if nq == 1 else nq // bs), nk // bs
    out = {}
    for b in range(B):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if head_map[h] == g]
            kbar = [[sum(Fraction(float(k[b, g, j * bs + t, d])) for t in range(bs)) / bs
                     for d in range(D)] for j in range(nkb)]
            for qb in range(nqb):
                diag = O.row_block_diag(nq, nk, bs, qb)
                score = [Fraction(0)] * nkb
                for h in heads:
                    if nq == 1:
                        qv = [Fraction(float(q[b, h, 0, d])) for d in range(D)]
                    else:
                        qv = [sum(Fraction(float(q[b, h, qb * bs + t, d])) for t in range(bs)) / bs
                              for d in range(D)]
                    for j in range(nkb):
                        score[j] += sum(qv[d] * kbar[j][d] for d in range(D))
                forced = O.forced_blocks(diag, n_sink, n_local)
                cands = [j for j in range(diag + 1) if j not in forced]
                free = budget - len(forced)
                picks = cands if len(cands) <= free else \
                    sorted(cands, key=lambda j: (-score[j], j))[:free]
                out[(b, g, qb)] = sorted(forced + picks)
    return out


def check_group_shared_selection(seed=12):
    """Group-shared selection against exact rational brute force (small
    integer inputs keep every float step exact), in prefill and decode; every
    head of a group gets the group's list; with one q head per kv head the
    group mode is the per-head mode."""
    r = _rng(seed)
    for nq_mode in ("prefill", "decode"):
        B, Hq, Hkv, bs, nb, D = 2, 6, 2, 2, 7, 3
        n = bs * nb
        nq = n if nq_mode == "prefill" else 1
        q = r.integers(-4, 5, size=(B, Hq, nq, D)).astype(np.float64)
        k = r.integers(-4, 5, size=(B, Hkv, n, D)).astype(np.float64)
        hm = [0, 1, 1, 0, 0, 1]
        for budget, n_sink, n_local in ((3, 1, 1), (4, 0, 1), (5, 1, 0)):
            idx, cnt = O.select_blocks(q, k, block=bs, budget=budget, n_sink=n_sink,
                                       n_local=n_local, head_map=hm, group_shared=True)
            want = _brute_group_selection(q, k, bs, budget, n_sink, n_local, hm)
            for (b, g, qb), sel in want.items():
                for h in [h for h in range(Hq) if hm[h] == g]:
                    assert int(cnt[b, h, qb]) == len(sel), (nq_mode, b, g, qb)
                    assert idx[b, h, qb, :len(sel)].tolist() == sel, (nq_mode, b, h, qb, sel)
    q = r.standard_normal((1, 2, 16, 4)); k = r.standard_normal((1, 2, 16, 4))
    a = O.select_blocks(q, k, block=4, budget=2, n_sink=1, n_local=0, head_map=[0, 1])
    b2 = O.select_blocks(q, k, block=4, budget=2, n_sink=1, n_local=0, head_map=[0, 1],
                         group_shared=True)
    assert np.array_equal(a[0], b2[0]) and np.array_equal(a[1], b2[1])


def check_decode_vs_sdpa(seed=10):
    """Decode: one query at the last position, its own block representation,
    diag = last block; streams equal SDPA on that single row."""
    r = _rng(seed)
    bs, nb, D = 4, 10, 5
    n = bs * nb
    k = r.standard_normal((n, D)); v = r.standard_normal((n, D)); q = r.standard_normal((1, D))
    res = O.ssa_forward(q[None, None], k[None, None], v[None, None], block=bs, budget=4,
                        n_sink=1, n_local=1)
    sel = O.selected_mask(res["idx"][0, 0, 0], nb)
    assert sel[0] and sel[nb - 1] and sel.sum() == 4
    # the free picks are the two best pooled scores among blocks 1..nb-2
    kbar = O.pool_blocks(k.astype(np.float32), bs).astype(np.float64)
    s = kbar @ q[0].astype(np.float32).astype(np.float64)
    best = sorted(range(1, nb - 1), key=lambda j: -s[j])[:2]
    assert set(np.nonzero(sel)[0].tolist()) == {0, nb - 1, *best}
    mask = sel[np.arange(n) // bs][None]
    scale = 1 / math.sqrt(D)
    assert np.allclose(res["h_full"][0, 0], _sdpa(q, k, v, np.ones((1, n), bool), scale), atol=1e-12)
    assert np.allclose(res["h_sparse"][0, 0], _sdpa(q, k, v, mask, scale), atol=1e-12)


# ---------------------------------------------------------------- losses

def check_loss_vs_torch(seed=11):
    """Loss values equal torch's MSE; gradient seeds equal autograd through
    MSE with the stop-gradient side detached."""
    r = _rng(seed)
    hf = r.standard_normal((2, 3, 5, 4)); hs = r.standard_normal((2, 3, 5, 4))
    ls, lc, gf, gs = O.align_loss(hf, hs)
    tf = torch.tensor(hf, requires_grad=True); ts = torch.tensor(hs, requires_grad=True)
    l_sparsity = torch.nn.functional.mse_loss(tf, ts.detach())
    l_commit = torch.nn.functional.mse_loss(ts, tf.detach())
    (l_sparsity + l_commit).backward()
    assert abs(ls - l_sparsity.item()) < 1e-15 and abs(lc - l_commit.item()) < 1e-15
    assert np.allclose(gf, tf.grad.numpy(), atol=1e-16)
    assert np.allclose(gs, ts.grad.numpy(), atol=1e-16)
    # constant shift c -> loss c^2
    ls2, _, _, _ = O.align_loss(hf, hf + 0.25)
    assert abs(ls2 - 0.0625) < 1e-15


# ---------------------------------------------------------------- worked example

def check_worked_example():
    with open(os.path.join(GOLDEN, "worked_example_6tok.json")) as f:
        ex = json.load(f)
    inp, exp = ex["inputs"], ex["expected"]
    n, D = inp["N"], inp["D"]
    q = np.zeros((n, D)); q[:, 0] = 1.0
    k = np.zeros((n, D)); k[:, 0] = np.log(np.array(inp["a"], dtype=np.float64))
    v = np.array(inp["v"], dtype=np.float64)
    res = O.ssa_forward(q[None, None], k[None, None], v[None, None], block=inp["block"],
                        budget=inp["budget"], n_sink=inp["n_sink"], n_local=inp["n_local"],
                        scale=inp["scale"])
    fr = lambda a: np.array([[float(Fraction(x)) for x in row] for row in a])
    assert res["idx"][0, 0].tolist() == exp["idx"]
    assert res["cnt"][0, 0].tolist() == exp["cnt"]
    assert np.allclose(res["h_full"][0, 0], fr(exp["h_full"]), atol=1e-13)
    assert np.allclose(res["h_sparse"][0, 0], fr(exp["h_sparse"]), atol=1e-13)
    assert np.allclose(res["delta"][0, 0], [float(Fraction(x)) for x in exp["delta"]], atol=1e-14)
    assert abs(res["loss_sparsity"] - float(Fraction(exp["loss"]))) < 1e-14
    assert res["loss_commitment"] == res["loss_sparsity"]


# ---------------------------------------------------------------- backward

def _bwd_problem(seed, B=1, Hq=2, Hkv=1, bs=3, nb=4, D=3, budget=2, hm=None):
    """Tiny GQA problem with a selection that drops blocks, and random
    upstream gradients of both outputs."""
    r = _rng(seed)
    n = bs * nb
    q = r.standard_normal((B, Hq, n, D))
    k = r.standard_normal((B, Hkv, n, D)) * 1.3
    v = r.standard_normal((B, Hkv, n, D))
    hm = hm if hm is not None else [h // (Hq // Hkv) for h in range(Hq)]
    idx, _ = O.select_blocks(q, k, block=bs, budget=budget, n_sink=1, n_local=1, head_map=hm)
    gf = r.standard_normal((B, Hq, n, D))
    gs = r.standard_normal((B, Hq, n, D))
    return q, k, v, idx, gf, gs, hm, bs


def _streams(q, k, v, idx, bs, scale, hm):
    res = O.dual_attention(q, k, v, idx, block=bs, scale=scale, head_map=hm)
    hf = np.zeros(q.shape); hs = np.zeros(q.shape)
    for (b, h), (r, a, c, _) in res.items():
        hf[b, h, r], hs[b, h, r] = a, c
    return hf, hs


def check_backward_finite_differences(seed=13):
    """Central differences (step 1e-6) of F = <d_full, h_full> +
    <d_sparse, h_sparse>, evaluated with the oracle's forward over a fixed
    selection, equal the backward's dq, dk, dv for every input element of a
    two-head GQA group (both heads feed the one kv head)."""
    q, k, v, idx, gf, gs, hm, bs = _bwd_problem(seed)
    scale = 0.8
    dq, dk, dv = O.dual_attention_backward(q, k, v, idx, gf, gs, block=bs, scale=scale, head_map=hm)

    def F(inputs):
        hf, hs = _streams(inputs[0], inputs[1], inputs[2], idx, bs, scale, hm)
        return float((gf * hf).sum() + (gs * hs).sum())

    eps = 1e-6
    for which, grad in enumerate((dq, dk, dv)):
        for pos in np.ndindex(grad.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][pos] += eps
            minus[which][pos] -= eps
            fd = (F(plus) - F(minus)) / (2 * eps)
            assert abs(fd - grad[pos]) < 1e-7, ("qkv"[which], pos, fd, grad[pos])


def _torch_streams_grad(q, k, v, sel_tok, gf, gs, scale, hm, sg_loss_alpha=None):
    """torch float64 autograd through SDPA: full stream under the causal mask,
    sparse stream under the selected-token mask, K/V gathered per q head so
    that autograd sums the group's contributions."""
    t = lambda x: torch.tensor(np.ascontiguousarray(x, dtype=np.float64), requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    kk, vv = tk[:, hm], tv[:, hm]
    n = q.shape[2]
    causal = torch.from_numpy(np.tril(np.ones((n, n), dtype=bool)))
    hf = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=causal, scale=scale)
    hs = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=torch.from_numpy(sel_tok),
                                                          scale=scale)
    if sg_loss_alpha is None:
        L = (torch.from_numpy(gf) * hf).sum() + (torch.from_numpy(gs) * hs).sum()
    else:
        mse = torch.nn.functional.mse_loss
        L = sg_loss_alpha * (mse(hf, hs.detach()) + mse(hs, hf.detach()))
    L.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), hf.detach().numpy(), hs.detach().numpy()


def _sel_tok_masks(idx, n, bs):
    B, Hq = idx.shape[:2]
    causal = np.tril(np.ones((n, n), dtype=bool))
    m = np.zeros((B, Hq, n, n), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for t in range(n):
                blk = O.selected_mask(idx[b, h, t // bs], n // bs)
                m[b, h, t] = causal[t] & blk[np.arange(n) // bs]
    return m


def check_backward_vs_torch_autograd(seed=14):
    """dq, dk, dv equal torch autograd through float64 SDPA of both streams,
    for B 2, a permuted head map and each stream alone."""
    q, k, v, idx, gf, gs, hm, bs = _bwd_problem(seed, B=2, Hq=4, Hkv=2, bs=4, nb=5, D=5, budget=3,
                                                hm=[1, 0, 0, 1])
    n = q.shape[2]
    sel_tok = _sel_tok_masks(idx, n, bs)
    for a, c in ((gf, gs), (gf, None), (None, gs)):
        ta = np.zeros_like(gf) if a is None else a
        tc = np.zeros_like(gs) if c is None else c
        wq, wk, wv, _, _ = _torch_streams_grad(q, k, v, sel_tok, ta, tc, 0.45, hm)
        dq, dk, dv = O.dual_attention_backward(q, k, v, idx, a, c, block=bs, scale=0.45, head_map=hm)
        for got, want in ((dq, wq), (dk, wk), (dv, wv)):
            assert np.allclose(got, want, atol=1e-12, rtol=1e-11), np.abs(got - want).max()


def check_backward_invariants(seed=15):
    """Softmax is unchanged when one vector is added to every key, so dk sums
    to zero over the keys of each kv head; every softmax row sums to one, so
    dv summed over keys equals the upstream gradients summed over the rows of
    the group's q heads. With every causal block selected both streams are
    the same function, so a gradient fed to either stream gives the same
    dq, dk, dv."""
    q, k, v, idx, gf, gs, hm, bs = _bwd_problem(seed, B=2, Hq=4, Hkv=2, nb=5)
    dq, dk, dv = O.dual_attention_backward(q, k, v, idx, gf, gs, block=bs, scale=0.6, head_map=hm)
    for b in range(2):
        for g in range(2):
            assert np.allclose(dk[b, g].sum(axis=0), 0.0, atol=1e-12)
            heads = [h for h in range(4) if hm[h] == g]
            want = sum((gf[b, h] + gs[b, h]).sum(axis=0) for h in heads)
            assert np.allclose(dv[b, g].sum(axis=0), want, atol=1e-12)
    nb = q.shape[2] // bs
    full_idx = np.tile(np.arange(nb), idx.shape[:3] + (1,))
    a = O.dual_attention_backward(q, k, v, full_idx, gf, None, block=bs, scale=0.6, head_map=hm)
    c = O.dual_attention_backward(q, k, v, full_idx, None, gf, block=bs, scale=0.6, head_map=hm)
    for x, y in zip(a, c):
        assert np.allclose(x, y, atol=1e-13)


def check_backward_alignment_seeds(seed=16):
    """Stop-gradient composition: backward fed with alpha times the loss
    seeds (sparsity loss -> h_full, commitment loss -> h_sparse) equals torch
    autograd of alpha (MSE(h_full, sg[h_sparse]) + MSE(h_sparse, sg[h_full]))
    through float64 SDPA, with sg = detach."""
    q, k, v, idx, _, _, hm, bs = _bwd_problem(seed, Hq=2, Hkv=1, bs=4, nb=4, D=4)
    n = q.shape[2]
    alpha = 10.0
    wq, wk, wv, hf, hs = _torch_streams_grad(q, k, v, _sel_tok_masks(idx, n, bs), None, None, 0.5, hm,
                                             sg_loss_alpha=alpha)
    _, _, sf, ss = O.align_loss(hf, hs)
    dq, dk, dv = O.dual_attention_backward(q, k, v, idx, alpha * sf, alpha * ss, block=bs,
                                           scale=0.5, head_map=hm)
    for got, want in ((dq, wq), (dk, wk), (dv, wv)):
        assert np.allclose(got, want, atol=1e-12, rtol=1e-10), np.abs(got - want).max()


# ---------------------------------------------------------------- per-token selection

def _brute_token_selection(q, k, bs, budget, n_sink, n_local, head_map):
    """Per-token lists from exact rational arithmetic on the raw inputs: the
    row's own query and the block means of K as Fractions, ranked by
    (-score, index); the forced blocks of the row's block (first n_sink
    blocks, n_local blocks ending at the block holding the row) are added."""
    B, Hq, nq, D = q.shape
    nk = k.shape[2]
    nkb = nk // bs
    out = {}
    for b in range(B):
        for h in range(Hq):
            g = head_map[h]
            kbar = [[sum(Fraction(float(k[b, g, j * bs + t, d])) for t in range(bs)) / bs
                     for d in range(D)] for j in range(nkb)]
            for t in range(nq):
                diag = (nk - nq + t) // bs
                qv = [Fraction(float(q[b, h, t, d])) for d in range(D)]
                score = [sum(qv[d] * kbar[j][d] for d in range(D)) for j in range(nkb)]
                forced = set(range(min(n_sink, diag + 1)))
                forced |= set(range(max(0, diag - n_local + 1), diag + 1))
                cands = [j for j in range(diag + 1) if j not in forced]
                free = budget - len(forced)
                picks = cands if len(cands) <= free else \
                    sorted(cands, key=lambda j: (-score[j], j))[:free]
                out[(b, h, t)] = sorted(forced | set(picks))
    return out


def check_token_selection_brute(seed=17):
    """Per-token selection against exact rational brute force (small integer
    inputs keep every float step exact), for a permuted GQA head map and
    several forced-block settings; rows of one block must get lists of their
    own (the data are chosen so that some do differ). In decode the single
    query represents itself, so per-token equals per-block selection."""
    r = _rng(seed)
    B, Hq, Hkv, bs, nb, D = 2, 4, 2, 2, 7, 3
    n = bs * nb
    q = r.integers(-4, 5, size=(B, Hq, n, D)).astype(np.float64)
    k = r.integers(-4, 5, size=(B, Hkv, n, D)).astype(np.float64)
    hm = [1, 0, 0, 1]
    differs = 0
    for budget, n_sink, n_local in ((3, 1, 1), (4, 0, 1), (5, 1, 0), (2, 0, 0)):
        idx, cnt = O.select_blocks(q, k, block=bs, budget=budget, n_sink=n_sink,
                                   n_local=n_local, head_map=hm, per_token=True)
        assert idx.shape == (B, Hq, n, budget) and cnt.shape == (B, Hq, n)
        want = _brute_token_selection(q, k, bs, budget, n_sink, n_local, hm)
        for (b, h, t), sel in want.items():
            assert int(cnt[b, h, t]) == len(sel), (budget, b, h, t)
            assert idx[b, h, t, :len(sel)].tolist() == sel, (budget, b, h, t, sel)
            assert (idx[b, h, t, len(sel):] == -1).all()
            if t % bs and want[(b, h, t - 1)] != sel:
                differs += 1
    assert differs > 0
    qd = r.standard_normal((1, 2, 1, 4)).astype(np.float32)
    kd = r.standard_normal((1, 1, 24, 4)).astype(np.float32)
    a = O.select_blocks(qd, kd, block=4, budget=3, n_sink=1, n_local=1, head_map=[0, 0])
    c = O.select_blocks(qd, kd, block=4, budget=3, n_sink=1, n_local=1, head_map=[0, 0],
                        per_token=True)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def check_token_float32_query():
    """The row's query enters the scores as float32, hand-derived: pooled keys
    (0, 1), (1, 0), (0, 1/2) for blocks 0-2, the last row forces its own block
    3 and has one free slot. q = (1 + 2^-10, 1) scores 1, 1 + 2^-10, 1/2 and
    takes block 1 (a bfloat16 copy of q would tie blocks 0 and 1 and take 0);
    q = (1 + 2^-30, 1) rounds to (1, 1) in float32, ties, and takes block 0."""
    k = np.array([[0, 1], [0, 1], [1, 0], [1, 0], [0, 0.5], [0, 0.5], [0, 0], [0, 0]],
                 dtype=np.float64)[None, None]
    for eps, want in ((2.0 ** -10, [1, 3]), (2.0 ** -30, [0, 3])):
        q = np.zeros((1, 1, 8, 2))
        q[0, 0, 7] = [1.0 + eps, 1.0]
        idx, cnt = O.select_blocks(q, k, block=2, budget=2, n_sink=0, n_local=1, head_map=[0],
                                   per_token=True)
        assert idx[0, 0, 7].tolist() == want and int(cnt[0, 0, 7]) == 2, (eps, idx[0, 0, 7])


def check_token_constant_rows(seed=18):
    """When every row of a query block carries the same float32 vector, the
    block's pooled query is that vector exactly, so each row's per-token list
    is its block's per-block list (random float data, ties unlikely)."""
    r = _rng(seed)
    B, Hq, Hkv, bs, nb, D = 1, 2, 1, 4, 9, 5
    base = r.standard_normal((B, Hq, nb, D)).astype(np.float32)
    q = np.repeat(base, bs, axis=2)
    k = r.standard_normal((B, Hkv, nb * bs, D)).astype(np.float32)
    for budget, n_sink, n_local in ((3, 1, 1), (4, 0, 2)):
        ib, cb = O.select_blocks(q, k, block=bs, budget=budget, n_sink=n_sink, n_local=n_local,
                                 head_map=[0, 0])
        it, ct = O.select_blocks(q, k, block=bs, budget=budget, n_sink=n_sink, n_local=n_local,
                                 head_map=[0, 0], per_token=True)
        rows = np.arange(nb * bs)
        assert np.array_equal(it, ib[:, :, rows // bs]), budget
        assert np.array_equal(ct, cb[:, :, rows // bs]), budget


def _token_masks(idx, n, bs):
    """[B, Hq, n, n] selected-token masks of per-token lists, built directly:
    key j is in row t's sparse set when j <= t and j's block is in idx[t]."""
    B, Hq = idx.shape[:2]
    m = np.zeros((B, Hq, n, n), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for t in range(n):
                blocks = {int(x) for x in idx[b, h, t] if x >= 0}
                for j in range(t + 1):
                    m[b, h, t, j] = (j // bs) in blocks
    return m


def check_token_attention_vs_sdpa(seed=19):
    """Both streams and the dropped mass with per-token lists: h_full is
    float64 SDPA under the causal mask, h_sparse SDPA under each row's own
    selected-token mask, delta the full softmax weight outside that mask."""
    r = _rng(seed)
    B, Hq, Hkv, bs, nb, D = 1, 2, 1, 4, 6, 4
    n = bs * nb
    q = r.standard_normal((B, Hq, n, D)); k = r.standard_normal((B, Hkv, n, D)) * 1.5
    v = r.standard_normal((B, Hkv, n, D))
    hm = [0, 0]
    idx, _ = O.select_blocks(q, k, block=bs, budget=3, n_sink=1, n_local=1, head_map=hm,
                             per_token=True)
    sel = _token_masks(idx, n, bs)
    res = O.dual_attention(q, k, v, idx, block=bs, scale=0.4, head_map=hm, per_token=True)
    causal = np.tril(np.ones((n, n), dtype=bool))
    rows_differ = False
    for h in range(Hq):
        _, hf, hs, dl = res[(0, h)]
        assert np.allclose(hf, _sdpa(q[0, h], k[0, 0], v[0, 0], causal, 0.4), atol=1e-13)
        assert np.allclose(hs, _sdpa(q[0, h], k[0, 0], v[0, 0], sel[0, h], 0.4), atol=1e-13)
        z = 0.4 * q[0, h] @ k[0, 0].T
        z = np.where(causal, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.allclose(dl, np.where(causal & ~sel[0, h], p, 0).sum(axis=1), atol=1e-14)
        for t in range(1, n):
            if t % bs and not np.array_equal(sel[0, h, t, :t], sel[0, h, t - 1, :t]):
                rows_differ = True
    assert rows_differ


def check_token_backward_vs_torch_autograd(seed=20):
    """Backward with per-token lists equals torch autograd through float64
    SDPA of both streams under each row's own selected-token mask."""
    r = _rng(seed)
    B, Hq, Hkv, bs, nb, D = 1, 2, 1, 4, 5, 4
    n = bs * nb
    q = r.standard_normal((B, Hq, n, D)); k = r.standard_normal((B, Hkv, n, D)) * 1.3
    v = r.standard_normal((B, Hkv, n, D))
    gf = r.standard_normal((B, Hq, n, D)); gs = r.standard_normal((B, Hq, n, D))
    hm = [0, 0]
    idx, _ = O.select_blocks(q, k, block=bs, budget=2, n_sink=1, n_local=1, head_map=hm,
                             per_token=True)
    wq, wk, wv, _, _ = _torch_streams_grad(q, k, v, _token_masks(idx, n, bs), gf, gs, 0.5, hm)
    dq, dk, dv = O.dual_attention_backward(q, k, v, idx, gf, gs, block=bs, scale=0.5,
                                           head_map=hm, per_token=True)
    for got, want in ((dq, wq), (dk, wk), (dv, wv)):
        assert np.allclose(got, want, atol=1e-12, rtol=1e-11), np.abs(got - want).max()


ALL_CHECKS = [
    check_pool_closed_form, check_pool_mean_identity, check_scores_exact_integers,
    check_select_constant_scores, check_select_duplicate_lower_index,
    check_select_known_ranking, check_select_invariants, check_attention_vs_sdpa,
    check_attention_constant_keys, check_attention_graded_logits,
    check_full_budget_equals_full, check_decomposition_and_bound, check_nested_budgets,
    check_gqa_equals_replicated, check_decode_vs_sdpa, check_loss_vs_torch,
    check_worked_example, check_group_shared_selection,
    check_backward_finite_differences, check_backward_vs_torch_autograd,
    check_backward_invariants, check_backward_alignment_seeds,
    check_token_selection_brute, check_token_float32_query, check_token_constant_rows, check_token_attention_vs_sdpa,
    check_token_backward_vs_torch_autograd,
]
