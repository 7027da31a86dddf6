"""Plain fp64 CPU oracle for the SSA dual-stream block-sparse attention forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or call this module. The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes follows the pages on SSA ("Sparse Sparse Attention"):

* "SSA: Achieving Sparser Attention by Aligning Full and Sparse Attention
  Outputs in Feature Space" (xugj520.cn), section "Practical Implementation
  of SSA": split the sequence into blocks, mean-pool each block, score the
  query against every earlier block representation, keep the top-k blocks and
  attend over the tokens of the kept blocks only; the identity
  Mean(qK^T) = q Mean(K)^T is why pooled scores rank blocks.
* same page, sections "SSA's Dual-Stream Training Mechanism" and
  "Bidirectional Attention Alignment": a full causal attention stream and a
  block-sparse stream per layer, compared by the sparsity loss
  ||a_full - sg[a_sparse]|| and the commitment loss ||a_sparse - sg[a_full]||.
* "Technische Samenvatting: SSA (Sparse Sparse Attention)" (gist.science),
  sections "1. Probleemstelling" and "2. Methodologie": the dropped attention
  mass delta(t), the full-softmax weight on tokens the sparse stream leaves
  out, which bounds the sparse-vs-full error linearly.

Readings where the pages leave a step open (each is also listed with its
reason in the design notes):

* selection is per query block of `block` rows (one list per (b, h, qb)); the
  query-block representation is the mean-pooled Q of that block; in decode the
  single query is its own representation;
* pooled vectors: float64 sum over the block's tokens in ascending order,
  divided by the block size, rounded once to float32; scores: float64 dot
  product of the float32 pooled vectors, summed over d in ascending order,
  without the logit scale; these fix the ranking bit for bit;
* candidates are the causal blocks [0, diag] minus the forced ones (the first
  `n_sink` blocks and the `n_local` blocks ending at the query's own block);
  `budget` counts all selected blocks, forced included; when no more
  candidates remain than free slots, all causal blocks are selected; exact
  score ties go to the lower block index;
* optionally (group-shared selection) one list per GQA group, ranked by the
  sum of the group's per-head scores, added in ascending head order;
* optionally (per-token selection) one list per query row: the row's own
  query vector, taken as float32, is scored against the pooled key blocks
  (the page's identity Mean(qK^T) = q Mean(K)^T is written for a single
  query q); candidates and forced blocks are those of the row's own block,
  so a row of a block and its block-mode list see the same causal range;
* token-level causal masking j <= t inside the query's own block, in both
  streams; logit scale 1/sqrt(D) unless given;
* losses are mean squared errors over all B*Hq*Nq*D elements; their forward
  values coincide, stop-gradient only changes which gradient each one feeds;
* backward: the stop-gradient of "Bidirectional Attention Alignment" blocks
  each loss's gradient at its target side, so the sparsity loss feeds only
  h_full and the commitment loss only h_sparse, and the auxiliary output,
  which is not passed on to later layers ("2. Methodologie"), receives only
  that gradient; both streams therefore run their own attention backward
  from the caller's upstream gradient of each output, and dq, dk, dv are the
  sums over the two streams; the hard top-k selection contributes no
  gradient.

Every function is pinned by the CPU tests against closed forms, exact special
cases, torch's scaled-dot-product attention in float64 (and its autograd for
the backward), central finite differences of the forward, and brute force on
tiny inputs; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# Selection: pool, score, top-k
# --------------------------------------------------------------------------

def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean-pool consecutive `block`-token blocks of x [..., N, D].

    Page: "SSA: Achieving Sparser Attention ..." section "Practical
    Implementation of SSA" (divide into blocks, mean-pool each block).
    float64 running sum over the block's tokens in ascending order, exact
    division by the block size, one rounding to float32. Returns
    [..., N // block, D] float32.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    if n % block:
        raise ValueError("sequence length must be a multiple of the block size")
    xb = x.reshape(x.shape[:-2] + (n // block, block, x.shape[-1]))
    acc = np.zeros(x.shape[:-2] + (n // block, x.shape[-1]), dtype=np.float64)
    for t in range(block):
        acc = acc + xb[..., t, :]
    return (acc / block).astype(np.float32)


def block_score_matrix(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Similarity of every query-block representation with every key-block
    representation: s[i, j] = sum_d qbar[i, d] * kbar[j, d] in float64,
    accumulated over d in ascending order.

    Page: "SSA: Achieving Sparser Attention ..." section "Practical
    Implementation of SSA" (similarity between the query and the earlier
    block representations). The products of two float32 values are exact in
    float64, so only the order of the additions matters, and it is fixed here.
    """
    q64 = np.asarray(qbar, dtype=np.float32).astype(np.float64)
    k64 = np.asarray(kbar, dtype=np.float32).astype(np.float64)
    s = np.zeros((q64.shape[0], k64.shape[0]), dtype=np.float64)
    for d in range(q64.shape[1]):
        s = s + q64[:, d:d + 1] * k64[None, :, d]
    return s


def group_score_matrix(per_head: Sequence[np.ndarray]) -> np.ndarray:
    """Score of a GQA group for group-shared selection: the sum of its q
    heads' score matrices, added in the order given (ascending q head index)
    in float64, starting from zero."""
    s = np.zeros_like(np.asarray(per_head[0], dtype=np.float64))
    for x in per_head:
        s = s + np.asarray(x, dtype=np.float64)
    return s


def forced_blocks(diag: int, n_sink: int, n_local: int) -> List[int]:
    """Blocks every row keeps: the first n_sink blocks and the n_local blocks
    ending at the row's own block `diag`, restricted to [0, diag]."""
    f = set(range(0, min(n_sink, diag + 1)))
    f.update(range(max(0, diag - n_local + 1), diag + 1))
    return sorted(f)


def select_row(scores: np.ndarray, diag: int, budget: int, n_sink: int,
               n_local: int) -> List[int]:
    """Selected key blocks of one row, ascending.

    Page: "SSA: Achieving Sparser Attention ..." section "Practical
    Implementation of SSA" (select the top-k most relevant blocks). Forced
    blocks are kept without being scored; the remaining `budget - |forced|`
    slots go to the highest-scoring causal candidates, ties to the lower
    index; with no more candidates than slots every causal block is kept.
    """
    forced = forced_blocks(diag, n_sink, n_local)
    free = budget - len(forced)
    if free < 0:
        raise ValueError("budget smaller than the number of forced blocks")
    fset = set(forced)
    cands = np.array([kb for kb in range(diag + 1) if kb not in fset], dtype=np.int64)
    if len(cands) <= free:
        picks = cands
    else:
        # np.lexsort sorts by the last key first: descending score, then
        # ascending block index.
        order = np.lexsort((cands, -scores[cands]))
        picks = cands[order[:free]]
    return sorted(forced + [int(x) for x in picks])


def token_representations(q_rows: np.ndarray) -> np.ndarray:
    """Per-token selection: each query row represents itself, rounded once to
    float32 (exact for bfloat16 and float32 inputs). "Practical
    Implementation of SSA" scores the query q against the pooled keys,
    q Mean(K)^T."""
    return np.asarray(q_rows, dtype=np.float64).astype(np.float32)


def token_row_diag(nq: int, nk: int, block: int, t: int) -> int:
    """Key block holding query row t (at key position nk - nq + t): the
    causal range and the forced blocks of a per-token list."""
    if nq != nk and nq != 1:
        raise ValueError("only Nq == Nk (prefill) and Nq == 1 (decode) are defined")
    return (nk - nq + t) // block


def list_row(r: int, block: int, nq: int, per_token: bool) -> int:
    """Selection list that query row r reads: its own list (per-token
    selection), else its row block's list; decode has one list."""
    if nq == 1:
        return 0
    return r if per_token else r // block


def row_block_diag(nq: int, nk: int, block: int, qb: int) -> int:
    """Key block that holds the last query of row block qb (queries are
    aligned to the end of the keys: query i sits at position nk - nq + i)."""
    if nq == nk:
        return qb
    if nq == 1:
        return (nk - 1) // block
    raise ValueError("only Nq == Nk (prefill) and Nq == 1 (decode) are defined")


def select_blocks(q: np.ndarray, k: np.ndarray, *, block: int, budget: int,
                  n_sink: int, n_local: int, head_map: Sequence[int],
                  k_pooled: Optional[np.ndarray] = None, group_shared: bool = False,
                  per_token: bool = False, rows: Optional[Dict] = None):
    """Selection for every (b, q head, row block).

    q [B, Hq, Nq, D], k [B, Hkv, Nk, D]. Returns idx [B, Hq, nQB, budget]
    int32 (ascending, padded with -1) and cnt [B, Hq, nQB] int32.
    In decode (Nq == 1) the query row is its own representation.

    group_shared: one list per (b, kv head, row block), given to every q head
    of the group. The group's score of a key block is the sum of its q heads'
    scores (float64, heads in ascending index order, starting from 0), i.e.
    the pooled key against the sum of the heads' pooled queries. This is the
    GQA-group-shared reading of "the query" in "Practical Implementation of
    SSA" (the pages select per query; a GQA group reads one kv head).

    per_token: one list per (b, q head, query row), idx [B, Hq, Nq, budget]:
    row t scores its own float32 query vector against the pooled keys, with
    the causal range and forced blocks of its block (token_row_diag). In
    decode the single query already represents itself, so per-token and
    per-block selection coincide. `rows` (per_token only) maps (b, h) to the
    query rows to select for; the other lists are left at -1 / 0.
    """
    B, Hq, nq, D = q.shape
    nk = k.shape[2]
    kbar = pool_blocks(k, block) if k_pooled is None else np.asarray(k_pooled, np.float32)
    if per_token:
        if group_shared:
            raise ValueError("per-token selection is per q head")
        qrep = token_representations(q)
        idx = np.full((B, Hq, nq, budget), -1, dtype=np.int32)
        cnt = np.zeros((B, Hq, nq), dtype=np.int32)
        keys = rows.keys() if rows is not None else [(b, h) for b in range(B) for h in range(Hq)]
        for (b, h) in keys:
            ts = np.arange(nq) if rows is None else np.asarray(rows[(b, h)], dtype=np.int64)
            s = block_score_matrix(qrep[b, h, ts], kbar[b, head_map[h]])
            for i, t in enumerate(ts.tolist()):
                sel = select_row(s[i], token_row_diag(nq, nk, block, t), budget, n_sink, n_local)
                idx[b, h, t, :len(sel)] = sel
                cnt[b, h, t] = len(sel)
        return idx, cnt
    if nq == 1:
        qbar = np.asarray(q, dtype=np.float64).astype(np.float32)
    else:
        qbar = pool_blocks(q, block)
    nqb = qbar.shape[2]
    idx = np.full((B, Hq, nqb, budget), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq, nqb), dtype=np.int32)
    for b in range(B):
        if group_shared:
            for g in range(k.shape[1]):
                heads = [h for h in range(Hq) if head_map[h] == g]
                s = group_score_matrix([block_score_matrix(qbar[b, h], kbar[b, g])
                                        for h in heads])
                for qb in range(nqb):
                    diag = row_block_diag(nq, nk, block, qb)
                    sel = select_row(s[qb], diag, budget, n_sink, n_local)
                    for h in heads:
                        idx[b, h, qb, :len(sel)] = sel
                        cnt[b, h, qb] = len(sel)
            continue
        for h in range(Hq):
            s = block_score_matrix(qbar[b, h], kbar[b, head_map[h]])
            for qb in range(nqb):
                diag = row_block_diag(nq, nk, block, qb)
                sel = select_row(s[qb], diag, budget, n_sink, n_local)
                idx[b, h, qb, :len(sel)] = sel
                cnt[b, h, qb] = len(sel)
    return idx, cnt


# --------------------------------------------------------------------------
# Attention: full stream, sparse stream, dropped mass
# --------------------------------------------------------------------------

def _masked_softmax_attend(z: np.ndarray, mask: np.ndarray, v: np.ndarray):
    """softmax of z over the True entries of each row of mask, applied to v."""
    zm = np.where(mask, z, -np.inf)
    m = zm.max(axis=1, keepdims=True)
    p = np.exp(zm - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v, p


def dual_attention_rows(q_rows: np.ndarray, positions: np.ndarray, k: np.ndarray,
                        v: np.ndarray, row_selected: np.ndarray, *, block: int,
                        scale: float):
    """Both attention streams and the dropped mass for a set of query rows of
    one head.

    q_rows [R, D] at key positions `positions` [R]; k, v [Nk, D];
    row_selected [R, nKB] bool: the selected key blocks of each row's block.

    Full stream: softmax over all causal keys j <= t ("SSA: Achieving Sparser
    Attention ...", section "SSA's Dual-Stream Training Mechanism", full
    attention stream). Sparse stream: its own softmax over the causal tokens
    of the selected blocks only (section "Practical Implementation of SSA",
    the concatenated reduced key and value sets). Dropped mass: the full
    softmax weight on causal tokens outside the selected blocks, summed
    directly ("Technische Samenvatting", "2. Methodologie", delta(t)).
    Returns float64 h_full [R, D], h_sparse [R, D], delta [R].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nk = k.shape[0]
    z = scale * (q_rows @ k.T)
    j = np.arange(nk)
    causal = j[None, :] <= np.asarray(positions)[:, None]
    sel_tok = causal & np.asarray(row_selected)[:, j // block]
    h_full, p_full = _masked_softmax_attend(z, causal, v)
    h_sparse, _ = _masked_softmax_attend(z, sel_tok, v)
    delta = np.where(causal & ~sel_tok, p_full, 0.0).sum(axis=1)
    return h_full, h_sparse, delta


def selected_mask(idx_row: np.ndarray, n_kb: int) -> np.ndarray:
    m = np.zeros(n_kb, dtype=bool)
    for x in np.asarray(idx_row).tolist():
        if x >= 0:
            m[x] = True
    return m


def dual_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                   *, block: int, scale: float, head_map: Sequence[int],
                   rows: Optional[Dict] = None, chunk: int = 256, per_token: bool = False):
    """Both streams for every (b, q head) and row, or for a subset of rows.

    q [B, Hq, Nq, D]; k, v [B, Hkv, Nk, D]; idx [B, Hq, nQB, budget], or
    [B, Hq, Nq, budget] with per_token (row r reads list list_row(r)).
    `rows` maps (b, h) -> array of row indices; default: all rows of all
    heads. Returns dicts keyed by (b, h) of (rows, h_full, h_sparse, delta).
    """
    B, Hq, nq, D = q.shape
    nk = k.shape[2]
    n_kb = nk // block
    out = {}
    keys = rows.keys() if rows is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for (b, h) in keys:
        r_all = np.arange(nq) if rows is None else np.asarray(rows[(b, h)])
        g = head_map[h]
        kk = np.asarray(k[b, g], dtype=np.float64)
        vv = np.asarray(v[b, g], dtype=np.float64)
        hf = np.zeros((len(r_all), D))
        hs = np.zeros((len(r_all), D))
        dl = np.zeros(len(r_all))
        for s0 in range(0, len(r_all), chunk):
            r = r_all[s0:s0 + chunk]
            sel = np.stack([selected_mask(idx[b, h, list_row(int(x), block, nq, per_token)], n_kb)
                            for x in r])
            pos = nk - nq + r
            a, c, d = dual_attention_rows(np.asarray(q[b, h, r], dtype=np.float64),
                                          pos, kk, vv, sel, block=block, scale=scale)
            hf[s0:s0 + chunk], hs[s0:s0 + chunk], dl[s0:s0 + chunk] = a, c, d
        out[(b, h)] = (r_all, hf, hs, dl)
    return out


# --------------------------------------------------------------------------
# Backward pass of both streams
# --------------------------------------------------------------------------

def softmax_vjp(p: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Gradient with respect to the logits of a row-wise softmax, given its
    output p and the gradient g with respect to p: the softmax Jacobian
    diag(p) - p p^T applied to g, i.e. p * (g - sum_j p_j g_j) per row.
    Entries where p is 0 (masked keys) get 0."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return p * (g - (p * g).sum(axis=1, keepdims=True))


def dual_attention_rows_backward(q_rows: np.ndarray, positions: np.ndarray, k: np.ndarray,
                                 v: np.ndarray, row_selected: np.ndarray,
                                 d_full: Optional[np.ndarray], d_sparse: Optional[np.ndarray],
                                 *, block: int, scale: float):
    """Gradients of <d_full, h_full> + <d_sparse, h_sparse> for a set of query
    rows of one head, with the block selection held fixed.

    The two streams are those of dual_attention_rows: h_full = P_f v and
    h_sparse = P_s v with P_f, P_s the softmax of z = scale q k^T over the
    causal keys and over the causal keys of the selected blocks. Chain rule,
    stream by stream ("SSA: Achieving Sparser Attention ...", section
    "Bidirectional Attention Alignment": the sparse and the full stream both
    receive gradient, each from the loss term whose target side is not
    stopped):
        dv  = P_f^T d_full + P_s^T d_sparse
        dz  = softmax_vjp(P_f, d_full v^T) + softmax_vjp(P_s, d_sparse v^T)
        dq  = scale dz k,   dk = scale dz^T q.
    The top-k selection is piecewise constant in q and k, so it contributes
    no gradient. d_full or d_sparse None means zero. Returns float64
    dq [R, D], dk [Nk, D], dv [Nk, D] (dk, dv from these rows only).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nk = k.shape[0]
    z = scale * (q_rows @ k.T)
    j = np.arange(nk)
    causal = j[None, :] <= np.asarray(positions)[:, None]
    sel_tok = causal & np.asarray(row_selected)[:, j // block]
    dz = np.zeros_like(z)
    dv = np.zeros_like(v)
    for mask, g in ((causal, d_full), (sel_tok, d_sparse)):
        if g is None:
            continue
        g = np.asarray(g, dtype=np.float64)
        _, p = _masked_softmax_attend(z, mask, v)
        dv += p.T @ g
        dz += softmax_vjp(p, g @ v.T)
    return scale * (dz @ k), scale * (dz.T @ q_rows), dv


def dual_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                            d_full: Optional[np.ndarray], d_sparse: Optional[np.ndarray],
                            *, block: int, scale: float, head_map: Sequence[int],
                            chunk: int = 256, per_token: bool = False):
    """dq [B, Hq, Nq, D], dk and dv [B, Hkv, Nk, D] (float64) of
    sum(d_full * h_full) + sum(d_sparse * h_sparse) for a whole problem, with
    the selection idx [B, Hq, nQB, budget] held fixed. d_full / d_sparse are
    [B, Hq, Nq, D] upstream gradients of the two outputs, or None for zero.
    Each kv head's dk, dv add the contributions of all q heads mapped to it.
    per_token: idx is [B, Hq, Nq, budget], one list per query row.
    """
    B, Hq, nq, D = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    n_kb = nk // block
    dq = np.zeros((B, Hq, nq, D))
    dk = np.zeros((B, Hkv, nk, D))
    dv = np.zeros((B, Hkv, nk, D))
    for b in range(B):
        for h in range(Hq):
            g = head_map[h]
            kk = np.asarray(k[b, g], dtype=np.float64)
            vv = np.asarray(v[b, g], dtype=np.float64)
            for r0 in range(0, nq, chunk):
                r = np.arange(r0, min(nq, r0 + chunk))
                sel = np.stack([selected_mask(idx[b, h, list_row(int(x), block, nq, per_token)],
                                              n_kb) for x in r])
                gf = None if d_full is None else d_full[b, h, r]
                gs = None if d_sparse is None else d_sparse[b, h, r]
                a, c, e = dual_attention_rows_backward(
                    np.asarray(q[b, h, r], dtype=np.float64), nk - nq + r, kk, vv, sel,
                    gf, gs, block=block, scale=scale)
                dq[b, h, r] = a
                dk[b, g] += c
                dv[b, g] += e
    return dq, dk, dv


# --------------------------------------------------------------------------
# Alignment losses
# --------------------------------------------------------------------------

def align_loss(h_full: np.ndarray, h_sparse: np.ndarray):
    """Sparsity and commitment losses with their gradient seeds.

    Page: "SSA: Achieving Sparser Attention ..." section "Bidirectional
    Attention Alignment": L_sparsity = ||a_full - sg[a_sparse]||,
    L_commitment = ||a_sparse - sg[a_full]||, read as mean squared errors
    over all elements. Both forward values equal mean((h_full - h_sparse)^2);
    the stop-gradient makes L_sparsity feed only h_full, with
    dL_sparsity/dh_full = 2 (h_full - h_sparse) / n, and L_commitment feed
    only h_sparse, with dL_commitment/dh_sparse = 2 (h_sparse - h_full) / n.
    Returns (L_sparsity, L_commitment, grad_full, grad_sparse).
    """
    hf = np.asarray(h_full, dtype=np.float64)
    hs = np.asarray(h_sparse, dtype=np.float64)
    diff = hf - hs
    n = diff.size
    loss = float(np.sum(diff * diff) / n)
    return loss, loss, 2.0 * diff / n, -2.0 * diff / n


# --------------------------------------------------------------------------
# Whole forward
# --------------------------------------------------------------------------

def ssa_forward(q, k, v, *, block: int, budget: int, n_sink: int, n_local: int,
                scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None,
                k_pooled: Optional[np.ndarray] = None, group_shared: bool = False,
                per_token: bool = False):
    """Selection, both streams, dropped mass and losses for a whole problem.

    q [B, Hq, Nq, D], k and v [B, Hkv, Nk, D] (any float dtype; used at their
    exact float64 values). Returns a dict with idx, cnt, h_full, h_sparse
    [B, Hq, Nq, D] float64, delta [B, Hq, Nq] float64 and the two losses.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, nq, D = q.shape
    Hkv = k.shape[1]
    if head_map is None:
        head_map = [h // (Hq // Hkv) for h in range(Hq)]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    idx, cnt = select_blocks(q, k, block=block, budget=budget, n_sink=n_sink,
                             n_local=n_local, head_map=head_map, k_pooled=k_pooled,
                             group_shared=group_shared, per_token=per_token)
    res = dual_attention(q, k, v, idx, block=block, scale=scale, head_map=head_map,
                         per_token=per_token)
    h_full = np.zeros((B, Hq, nq, D))
    h_sparse = np.zeros((B, Hq, nq, D))
    delta = np.zeros((B, Hq, nq))
    for (b, h), (r, hf, hs, dl) in res.items():
        h_full[b, h, r], h_sparse[b, h, r], delta[b, h, r] = hf, hs, dl
    l_s, l_c, _, _ = align_loss(h_full, h_sparse)
    return {"idx": idx, "cnt": cnt, "h_full": h_full, "h_sparse": h_sparse,
            "delta": delta, "loss_sparsity": l_s, "loss_commitment": l_c}
