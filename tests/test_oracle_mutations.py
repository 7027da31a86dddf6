"""Plants plausible mistakes in the oracle (on the CPU, by monkeypatching) and
checks that at least one pin catches each of them."""
import numpy as np
import pytest

import oracle.ssa_oracle as O
import oracle_pins as P

_pool, _scores, _select_row, _rows, _loss = (O.pool_blocks, O.block_score_matrix,
                                             O.select_row, O.dual_attention_rows, O.align_loss)
_group = O.group_score_matrix
_vjp, _rows_bwd, _bwd = O.softmax_vjp, O.dual_attention_rows_backward, O.dual_attention_backward
_tok_rep, _tok_diag = O.token_representations, O.token_row_diag


def m_pool_sum(x, block):                      # sum instead of mean
    return (_pool(x, block).astype(np.float64) * block).astype(np.float32)


def m_pool_strided(x, block):                  # blocks taken with a stride
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    xb = x.reshape(x.shape[:-2] + (block, n // block, x.shape[-1]))
    return xb.mean(axis=-3).astype(np.float32)


def m_scores_transposed(qbar, kbar):           # operands swapped
    return _scores(kbar, qbar)


def m_select_high_tie(scores, diag, budget, n_sink, n_local):   # ties to the higher index
    forced = O.forced_blocks(diag, n_sink, n_local)
    free = budget - len(forced)
    c = [kb for kb in range(diag + 1) if kb not in forced]
    picks = c if len(c) <= free else sorted(c, key=lambda kb: (-scores[kb], -kb))[:free]
    return sorted(forced + list(picks))


def m_select_no_forced(scores, diag, budget, n_sink, n_local):  # forced blocks ignored
    c = list(range(diag + 1))
    return sorted(sorted(c, key=lambda kb: (-scores[kb], kb))[:budget])


def m_rows_strict_causal(q, pos, k, v, sel, *, block, scale):   # j < t instead of j <= t
    pos = np.asarray(pos)
    return _rows(q, np.maximum(pos - 1, 0), k, v, sel, block=block, scale=scale)


def m_rows_no_renorm(q, pos, k, v, sel, *, block, scale):       # sparse not renormalised
    hf, hs, dl = _rows(q, pos, k, v, sel, block=block, scale=scale)
    return hf, hs * (1.0 - dl)[:, None], dl


def m_rows_no_scale(q, pos, k, v, sel, *, block, scale):        # logit scale dropped
    return _rows(q, pos, k, v, sel, block=block, scale=1.0)


def m_rows_delta_kept(q, pos, k, v, sel, *, block, scale):      # delta = kept mass
    hf, hs, dl = _rows(q, pos, k, v, sel, block=block, scale=scale)
    return hf, hs, 1.0 - dl


def m_loss_row_mean(hf, hs):                   # mean over rows, not elements
    a, b, c, d = _loss(hf, hs)
    D = np.asarray(hf).shape[-1]
    return a * D, b * D, c * D, d * D


def m_loss_grad_sign(hf, hs):                  # gradient seeds swapped
    a, b, c, d = _loss(hf, hs)
    return a, b, d, c


def m_group_first_head(per_head):             # group score = first head only
    return _group(per_head[:1])


def m_group_max(per_head):                     # max over heads instead of the sum
    return np.maximum.reduce([np.asarray(x, dtype=np.float64) for x in per_head])


def m_vjp_uncentred(p, g):                      # softmax Jacobian without the -p p^T part
    return np.asarray(p) * np.asarray(g)


def m_rows_bwd_no_sparse_dv(q, pos, k, v, sel, gf, gs, *, block, scale):  # P_s^T d_sparse dropped
    dq, dk, dv = _rows_bwd(q, pos, k, v, sel, gf, gs, block=block, scale=scale)
    if gs is not None:
        dv = dv - _rows_bwd(q, pos, k, v, sel, None, gs, block=block, scale=scale)[2]
    return dq, dk, dv


def m_rows_bwd_dk_unscaled(q, pos, k, v, sel, gf, gs, *, block, scale):  # logit scale left off dk
    dq, dk, dv = _rows_bwd(q, pos, k, v, sel, gf, gs, block=block, scale=scale)
    return dq, dk / scale, dv


def m_rows_bwd_streams_swapped(q, pos, k, v, sel, gf, gs, *, block, scale):  # seeds to the wrong stream
    return _rows_bwd(q, pos, k, v, sel, gs, gf, block=block, scale=scale)


def m_bwd_gqa_overwrite(q, k, v, idx, gf, gs, *, block, scale, head_map, chunk=256):
    # dk, dv of a kv head overwritten by each q head instead of summed
    dq, _, _ = _bwd(q, k, v, idx, gf, gs, block=block, scale=scale, head_map=head_map)
    Hq = q.shape[1]
    last = {g: max(h for h in range(Hq) if head_map[h] == g) for g in set(head_map)}
    keep = np.array([last[head_map[h]] == h for h in range(Hq)], dtype=float)[None, :, None, None]
    _, dk, dv = _bwd(q, k, v, idx, None if gf is None else gf * keep,
                     None if gs is None else gs * keep, block=block, scale=scale, head_map=head_map)
    return dq, dk, dv


def m_token_prev_row(q_rows):                 # row t scored with row t-1's query
    return np.roll(_tok_rep(q_rows), 1, axis=-2)


def m_token_rep_bf16(q_rows):                 # representation truncated to bfloat16
    x = _tok_rep(q_rows).view(np.uint32) & np.uint32(0xFFFF0000)
    return x.view(np.float32)


def m_token_diag_next(nq, nk, block, t):       # causal range of the next token's block
    return _tok_diag(nq, nk, block, min(t + 1, nq - 1))


def m_list_row_block(r, block, nq, per_token):  # per-token rows read the block's list
    return 0 if nq == 1 else r // block


MUTATIONS = [
    ("pool_blocks", m_pool_sum), ("pool_blocks", m_pool_strided),
    ("block_score_matrix", m_scores_transposed),
    ("select_row", m_select_high_tie), ("select_row", m_select_no_forced),
    ("dual_attention_rows", m_rows_strict_causal), ("dual_attention_rows", m_rows_no_renorm),
    ("dual_attention_rows", m_rows_no_scale), ("dual_attention_rows", m_rows_delta_kept),
    ("align_loss", m_loss_row_mean), ("align_loss", m_loss_grad_sign),
    ("group_score_matrix", m_group_first_head), ("group_score_matrix", m_group_max),
    ("softmax_vjp", m_vjp_uncentred),
    ("dual_attention_rows_backward", m_rows_bwd_no_sparse_dv),
    ("dual_attention_rows_backward", m_rows_bwd_dk_unscaled),
    ("dual_attention_rows_backward", m_rows_bwd_streams_swapped),
    ("dual_attention_backward", m_bwd_gqa_overwrite),
    ("token_representations", m_token_prev_row), ("token_representations", m_token_rep_bf16),
    ("token_row_diag", m_token_diag_next), ("list_row", m_list_row_block),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # AssertionError, or a shape error
            caught.append(check.__name__)
    assert caught, f"no pin caught mutation {fn.__name__}"
