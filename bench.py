"""Benchmark of the SSA dual-stream attention forward on one MI355X.

A step is one pass of the prefill hot path over the 32K-context GQA workload
(batch 1, 32 q heads / 8 kv heads, N = 32768, D = 128, block 64, budget 16
blocks including the sink and local blocks, planted peaked key blocks):
block pooling + top-k selection, the fused dual-stream attention (h_full,
h_sparse, delta) and the alignment losses. `value` is the algorithmic MFMA
work of the full causal stream, 4*D*64*64 FLOP per (query block, causal key
block) pair (the sparse stream adds none), divided by the step time.

The same run also times the single-query decode path (64 sequences x 32/8
heads, KV length 65536, budget 32) in dual and sparse-only mode, reported in
GB/s of algorithmic HBM bytes, and the fp64 CPU oracle on a bounded sample of
the prefill workload (the `cpu_baseline` object).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP64_PEAK_TFLOPS = 78.6          # MI355X float64 vector FMA

# HBM bytes per launch of the prefill attention kernel, from two rocprofv3
# --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by a plain 1 GiB copy (see the
# HBM-counter summary under profiles/), keyed by the SHA-256 of the kernel
# sources they were taken on (the prefill file and the headers it includes);
# any other source reports traffic as null.
PREFILL_TRAFFIC = {
    # 778032 KiB x 2.000 read + 531942 KiB x 1.000 written per dispatch
    "f64bb4b72ff93a8230594bf1988387fff3206c33c9c756faad6e08e397fdb4e4": int(778032 * 2.0 * 1024 + 531942 * 1.0 * 1024),
}
PREFILL_SRCS = [os.path.join(ROOT, "block_sparse_full_amd", "csrc", f)
                for f in ("ssa_attn_prefill.hip", "ssa_device.h", "ssa_common.h")]


def prefill_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for p in PREFILL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def prefill_traffic():
    try:
        sha = prefill_source_sha()
    except OSError:
        return None
    return PREFILL_TRAFFIC.get(sha)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def token_select_flops(cfg, budget) -> float:
    """float64 FLOPs of per-token selection: one D-long dot product (2 D
    FLOPs) per (query row, candidate block); candidates are the causal
    blocks of the row's block minus the sink and local blocks."""
    nkb = cfg.N // cfg.block
    pairs = 0
    for qb in range(nkb):
        forced = len(set(range(min(cfg.n_sink, qb + 1))) |
                     set(range(max(0, qb - cfg.n_local + 1), qb + 1)))
        pairs += (qb + 1 - forced) * cfg.block
    return 2.0 * cfg.D * pairs * cfg.B * cfg.Hq


def run_token_select(ssa, torch, cfg, q, k, v, steps):
    """Per-token selection (one list per query row) at cfg.budget: selection
    time with its float64 roofline, dual-mode and sparse-only attention."""
    dev = q.device
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                        block_size=cfg.block, token_select=True)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    tsel, tatt, tsp = EventTimer(torch), EventTimer(torch), EventTimer(torch)
    for _ in range(max(3, steps // 4)):
        tsel.start()
        ssa.select_blocks(p, q, k, ws=ws, idx=idx, cnt=cnt)
        tsel.stop()
        tatt.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=out)
        tatt.stop()
        tsp.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out={"h_sparse": out["h_sparse"]},
                     sparse_only=True)
        tsp.stop()
    torch.cuda.synchronize()
    sel_tf = token_select_flops(cfg, cfg.budget) / (tsel.mean_ms() * 1e-3) / 1e12
    att_tf = prefill_flops(cfg) / (tatt.mean_ms() * 1e-3) / 1e12
    res = {"budget": cfg.budget, "block": cfg.block,
           "select_ms": round(tsel.mean_ms(), 4),
           "select_fp64_tflops": round(sel_tf, 2),
           "select_fp64_frac": round(sel_tf / FP64_PEAK_TFLOPS, 4),
           "dual_attn_ms": round(tatt.mean_ms(), 4),
           "attn_tflops": round(att_tf, 2),
           "attn_mfma_frac": round(att_tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "sparse_only_attn_ms": round(tsp.mean_ms(), 4),
           "delta_mean": round(float(out["delta"].mean()), 4)}
    del out, ws, idx, cnt
    torch.cuda.empty_cache()
    return res


def sparse_flops(cfg, cnt) -> float:
    """Algorithmic FLOPs of sparse-only attention: 4 D FLOPs (QK^T and PV) per
    (query row, key) pair of the selected blocks, i.e. 4 D bs^2 per selected
    (query block, key block) pair; cnt holds the list lengths."""
    return 4.0 * cfg.D * cfg.block * cfg.block * float(cnt.sum())


def prefill_flops(cfg) -> float:
    """Algorithmic FLOPs of one dual-stream prefill: QK^T and PV over the
    causal set, 4 D bs^2 per (query block, causal key block) pair; the sparse
    stream reuses those products."""
    nkb = cfg.N // cfg.block
    pairs = nkb * (nkb + 1) // 2
    return 4.0 * cfg.D * cfg.block * cfg.block * pairs * cfg.B * cfg.Hq


class EventTimer:
    """Sums the device time of bracketed regions on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)

    def mean_ms(self):
        return self.total_ms() / max(1, len(self.pairs))


def run_prefill(ssa, torch, cfg, steps, warmup, budgets):
    from ssa_inputs import make_inputs
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = make_inputs(cfg, workers=16)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    del x
    log(f"[bench] prefill inputs ready in {time.time() - t0:.1f}s")
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    loss = torch.empty(2, dtype=torch.float32, device=dev)

    def step(attn_timer=None):
        ssa.select_blocks(p, q, k, ws=ws, idx=idx, cnt=cnt)
        if attn_timer is not None:
            attn_timer.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=out)
        if attn_timer is not None:
            attn_timer.stop()
        ssa.align_loss(p, out["h_full"], out["h_sparse"], ws=ws, loss=loss)

    for _ in range(warmup):
        step()
    # the attention kernel alone, for the roofline: one event pair per step,
    # recorded by the library immediately around the kernel's launch (the V
    # transpose launched before it stays outside the pair); torch creates an
    # event on its first record
    kev = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        kev.append((a, b))
    torch.cuda.synchronize()
    attn_t = EventTimer(torch)
    t0 = time.perf_counter()
    for i in range(steps):
        ssa.set_attn_timing_events(*kev[i])
        step(attn_t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ssa.set_attn_timing_events()
    res = {"ms_per_step": wall * 1e3 / steps, "attn_ms": attn_t.mean_ms(),
           "kernel_ms": sum(a.elapsed_time(b) for a, b in kev) / steps,
           "loss": float(loss[0]), "delta_mean": float(out["delta"].mean())}
    # budget sweep: attention time per budget (selection re-run per budget)
    sweep = {}
    for bgt in budgets:
        pb = ssa.problem_for(q, k, budget=bgt, n_sink=cfg.n_sink, n_local=cfg.n_local)
        ib, cb = ssa.select_blocks(pb, q, k, ws=ws)
        ssa.attn_fwd(pb, q, k, v, ib, cb, ws=ws, out=out)
        tm = EventTimer(torch)
        for _ in range(max(3, steps // 4)):
            tm.start()
            ssa.attn_fwd(pb, q, k, v, ib, cb, ws=ws, out=out)
            tm.stop()
        sp = EventTimer(torch)
        for _ in range(max(3, steps // 4)):
            sp.start()
            ssa.attn_fwd(pb, q, k, v, ib, cb, ws=ws, out={"h_sparse": out["h_sparse"]},
                         sparse_only=True)
            sp.stop()
        torch.cuda.synchronize()
        sp_flops = sparse_flops(cfg, cb)
        sweep[str(bgt)] = {"dual_attn_ms": round(tm.mean_ms(), 4),
                           "sparse_only_attn_ms": round(sp.mean_ms(), 4),
                           "sparse_only_tflops": round(sp_flops / (sp.mean_ms() * 1e-3) / 1e12, 2),
                           "sparse_only_mfma_frac": round(sp_flops / (sp.mean_ms() * 1e-3) / 1e12
                                                          / MFMA_BF16_PEAK_TFLOPS, 4),
                           "delta_mean": round(float(out["delta"].mean()), 4)}
    res["sweep"] = sweep
    # group-shared selection (one list per GQA group) at the headline budget
    pg = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                         group_select=True)
    ig, cg = ssa.select_blocks(pg, q, k, ws=ws)
    ssa.attn_fwd(pg, q, k, v, ig, cg, ws=ws, out=out)
    tsel, tg = EventTimer(torch), EventTimer(torch)
    for _ in range(max(3, steps // 4)):
        tsel.start()
        ssa.select_blocks(pg, q, k, ws=ws, idx=ig, cnt=cg)
        tsel.stop()
        tg.start()
        ssa.attn_fwd(pg, q, k, v, ig, cg, ws=ws, out=out)
        tg.stop()
    torch.cuda.synchronize()
    res["group_select"] = {"budget": cfg.budget, "select_ms": round(tsel.mean_ms(), 4),
                           "dual_attn_ms": round(tg.mean_ms(), 4),
                           "delta_mean": round(float(out["delta"].mean()), 4)}
    del out, ws
    torch.cuda.empty_cache()
    res["token_select"] = run_token_select(ssa, torch, cfg, q, k, v, steps)
    del q, k, v
    torch.cuda.empty_cache()
    return res


def run_paper_shape(ssa, torch, cfg, steps):
    """The pages' model shape (16-token blocks, D 64, 32 q / 2 kv heads):
    selection and dual-mode attention time, plus sparse-only attention."""
    from ssa_inputs import make_inputs
    dev = torch.device("cuda:0")
    x = make_inputs(cfg, workers=16)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    del x
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                        block_size=cfg.block)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    tsel, tatt, tsp = EventTimer(torch), EventTimer(torch), EventTimer(torch)
    for _ in range(max(3, steps // 2)):
        tsel.start()
        ssa.select_blocks(p, q, k, ws=ws, idx=idx, cnt=cnt)
        tsel.stop()
        tatt.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=out)
        tatt.stop()
        tsp.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out={"h_sparse": out["h_sparse"]},
                     sparse_only=True)
        tsp.stop()
    torch.cuda.synchronize()
    flops = prefill_flops(cfg)
    res = {"workload": f"paper shape prefill: B {cfg.B}, {cfg.Hq} q heads / {cfg.Hkv} kv heads, "
                       f"N {cfg.N}, D {cfg.D}, block {cfg.block}, budget {cfg.budget}",
           "select_ms": round(tsel.mean_ms(), 4), "dual_attn_ms": round(tatt.mean_ms(), 4),
           "attn_tflops": round(flops / (tatt.mean_ms() * 1e-3) / 1e12, 2),
           "attn_mfma_frac": round(flops / (tatt.mean_ms() * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "sparse_only_attn_ms": round(tsp.mean_ms(), 4),
           "sparse_only_tflops": round(sparse_flops(cfg, cnt) / (tsp.mean_ms() * 1e-3) / 1e12, 2),
           "delta_mean": round(float(out["delta"].mean()), 4)}
    # backward of both streams on this shape (seeded upstream gradients)
    from ssa_inputs import make_grads
    gr = make_grads(cfg, workers=16)
    gf, gs = gr["d_full"].to(dev), gr["d_sparse"].to(dev)
    del gr
    fwd = ssa.attn_fwd(p, q, k, v, idx, cnt, want_lse=True, ws=ws)
    bws = ssa.alloc_bwd_workspace(p, dev)
    kw = dict(h_full=fwd["h_full"], h_sparse=fwd["h_sparse"], d_full=gf, d_sparse=gs)
    bo = ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], ws=bws, **kw)
    tb = EventTimer(torch)
    for _ in range(max(3, steps // 4)):
        tb.start()
        ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], ws=bws, out=bo, **kw)
        tb.stop()
    torch.cuda.synchronize()
    bflops = 2.5 * flops + sparse_flops(cfg, cnt)   # 5 products per causal pair, 2 per selected
    res["backward_dual_ms"] = round(tb.mean_ms(), 4)
    res["backward_dual_tflops"] = round(bflops / (tb.mean_ms() * 1e-3) / 1e12, 2)
    del out, ws, fwd, bws, bo, gf, gs
    torch.cuda.empty_cache()
    res["token_select"] = run_token_select(ssa, torch, cfg, q, k, v, steps)
    del q, k, v
    torch.cuda.empty_cache()
    res["gqa_16to1"] = run_paper_fwd(ssa, torch, cfg.with_sizes(Hq=16, Hkv=1), steps)
    return res


def run_paper_fwd(ssa, torch, cfg, steps):
    """Dual-mode and sparse-only forward time of a 16-token-block shape."""
    from ssa_inputs import make_inputs
    dev = torch.device("cuda:0")
    x = make_inputs(cfg, workers=16)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    del x
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                        block_size=cfg.block)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    tatt, tsp = EventTimer(torch), EventTimer(torch)
    for _ in range(max(3, steps // 2)):
        tatt.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=out)
        tatt.stop()
        tsp.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out={"h_sparse": out["h_sparse"]},
                     sparse_only=True)
        tsp.stop()
    torch.cuda.synchronize()
    flops = prefill_flops(cfg)
    res = {"workload": f"B {cfg.B}, {cfg.Hq} q heads / {cfg.Hkv} kv head(s), N {cfg.N}, D {cfg.D}, "
                       f"block {cfg.block}, budget {cfg.budget}",
           "dual_attn_ms": round(tatt.mean_ms(), 4),
           "attn_tflops": round(flops / (tatt.mean_ms() * 1e-3) / 1e12, 2),
           "attn_mfma_frac": round(flops / (tatt.mean_ms() * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "sparse_only_attn_ms": round(tsp.mean_ms(), 4),
           "delta_mean": round(float(out["delta"].mean()), 4)}
    del q, k, v, out, ws, idx, cnt
    torch.cuda.empty_cache()
    return res


def run_backward(ssa, torch, cfg, steps, warmup):
    """Backward pass of both streams on the prefill workload, with seeded
    upstream gradients of both outputs (dual mode, as in alignment training),
    plus the full-stream-only and sparse-stream-only backward. FLOPs are
    algorithmic: per causal 64x64 (query block, key block) pair five D-deep
    products for the full stream (S recompute, dP, dV, dQ, dK) and per
    selected pair two more for the sparse stream (dP_s, dV_s)."""
    from ssa_inputs import make_grads, make_inputs
    dev = torch.device("cuda:0")
    x = make_inputs(cfg, workers=16)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    del x
    g = make_grads(cfg, workers=16)
    gf, gs = g["d_full"].to(dev), g["d_sparse"].to(dev)
    del g
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                        block_size=cfg.block)
    ws = ssa.alloc_workspace(p, dev)
    idx, cnt = ssa.select_blocks(p, q, k, ws=ws)
    fwd = ssa.attn_fwd(p, q, k, v, idx, cnt, want_lse=True, ws=ws)
    bws = ssa.alloc_bwd_workspace(p, dev)
    out = ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], h_full=fwd["h_full"],
                       h_sparse=fwd["h_sparse"], d_full=gf, d_sparse=gs, ws=bws)

    def timed(n, **kw):
        for _ in range(warmup):
            ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], ws=bws, out=out, **kw)
        t = EventTimer(torch)
        for _ in range(n):
            t.start()
            ssa.attn_bwd(p, q, k, v, idx, cnt, fwd["lse"], ws=bws, out=out, **kw)
            t.stop()
        torch.cuda.synchronize()
        return t.mean_ms()

    dual_ms = timed(steps, h_full=fwd["h_full"], h_sparse=fwd["h_sparse"], d_full=gf, d_sparse=gs)
    full_ms = timed(max(3, steps // 2), h_full=fwd["h_full"], d_full=gf)
    sparse_ms = timed(max(3, steps // 2), h_sparse=fwd["h_sparse"], d_sparse=gs)
    fwd_t = EventTimer(torch)
    for _ in range(max(3, steps // 2)):
        fwd_t.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, want_lse=True, ws=ws, out=fwd)
        fwd_t.stop()
    torch.cuda.synchronize()
    nkb = cfg.N // 64
    pair = 2.0 * cfg.D * 64 * 64                     # one 64x64xD product
    full_pairs = nkb * (nkb + 1) / 2 * cfg.B * cfg.Hq
    sel_pairs = float(cnt.sum()) * (cfg.block / 64) ** 2
    flops_full = 5 * pair * full_pairs
    flops_dual = flops_full + 2 * pair * sel_pairs
    res = {"workload": f"prefill backward: B {cfg.B}, {cfg.Hq} q heads / {cfg.Hkv} kv heads, "
                       f"N {cfg.N}, D {cfg.D}, block {cfg.block}, budget {cfg.budget}; "
                       f"upstream gradients of both outputs",
           "dual_ms": round(dual_ms, 4),
           "dual_tflops": round(flops_dual / (dual_ms * 1e-3) / 1e12, 2),
           "dual_mfma_frac": round(flops_dual / (dual_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "full_only_ms": round(full_ms, 4),
           "full_only_tflops": round(flops_full / (full_ms * 1e-3) / 1e12, 2),
           "sparse_only_ms": round(sparse_ms, 4),
           "fwd_dual_ms": round(fwd_t.mean_ms(), 4),
           "train_step_attn_ms": round(fwd_t.mean_ms() + dual_ms, 4),
           "sparse_stream_overhead": round((fwd_t.mean_ms() + dual_ms) / (fwd_t.mean_ms() + full_ms) - 1, 4)}
    del fwd, out, ws, bws
    torch.cuda.empty_cache()
    # per-token lists (one per query row): dual-mode backward
    pt = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                         block_size=cfg.block, token_select=True)
    ws = ssa.alloc_workspace(pt, dev)
    it, ct = ssa.select_blocks(pt, q, k, ws=ws)
    fwd = ssa.attn_fwd(pt, q, k, v, it, ct, want_lse=True, ws=ws)
    bws = ssa.alloc_bwd_workspace(pt, dev)
    kw = dict(h_full=fwd["h_full"], h_sparse=fwd["h_sparse"], d_full=gf, d_sparse=gs)
    out = ssa.attn_bwd(pt, q, k, v, it, ct, fwd["lse"], ws=bws, **kw)
    tt = EventTimer(torch)
    for _ in range(max(3, steps // 2)):
        tt.start()
        ssa.attn_bwd(pt, q, k, v, it, ct, fwd["lse"], ws=bws, out=out, **kw)
        tt.stop()
    torch.cuda.synchronize()
    tok_flops = flops_full + 2 * pair * float(ct.sum()) * (cfg.block / 64) / 64
    res["token_select_dual_ms"] = round(tt.mean_ms(), 4)
    res["token_select_dual_tflops"] = round(tok_flops / (tt.mean_ms() * 1e-3) / 1e12, 2)
    del q, k, v, gf, gs, fwd, out, ws, bws
    torch.cuda.empty_cache()
    return res


def run_decode(ssa, torch, cfg, steps, warmup):
    from ssa_inputs import make_inputs
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = make_inputs(cfg, workers=16)
    q = x["q"].to(dev)
    k = x["k"].to(dev)
    v = x["v"].to(dev)
    del x
    log(f"[bench] decode inputs ready in {time.time() - t0:.1f}s")
    p = ssa.problem_for(q, k, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local)
    ws = ssa.alloc_workspace(p, dev)
    kp = ssa.pool_blocks(p, k)   # the pooled-key table kept beside the cache
    idx, cnt = ssa.select_blocks(p, q, None, kp, ws=ws)
    out = ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws)
    loss = torch.empty(2, dtype=torch.float32, device=dev)

    def step(t_sel=None, t_attn=None):
        if t_sel is not None:
            t_sel.start()
        ssa.select_blocks(p, q, None, kp, ws=ws, idx=idx, cnt=cnt)
        if t_sel is not None:
            t_sel.stop()
            t_attn.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=out)
        if t_attn is not None:
            t_attn.stop()
        ssa.align_loss(p, out["h_full"], out["h_sparse"], ws=ws, loss=loss)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ts, ta = EventTimer(torch), EventTimer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(ts, ta)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # sparse-only mode
    sp_out = {"h_sparse": torch.empty_like(out["h_sparse"])}
    for _ in range(warmup):
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=sp_out, sparse_only=True)
    tsp = EventTimer(torch)
    for _ in range(steps):
        tsp.start()
        ssa.attn_fwd(p, q, k, v, idx, cnt, ws=ws, out=sp_out, sparse_only=True)
        tsp.stop()
    torch.cuda.synchronize()

    esz = 2
    kv_bytes = 2 * cfg.B * cfg.Hkv * cfg.N * cfg.D * esz
    table_bytes = cfg.B * cfg.Hkv * (cfg.N // cfg.block) * cfg.D * 4
    q_bytes = cfg.B * cfg.Hq * cfg.D * esz
    out_bytes = 2 * cfg.B * cfg.Hq * cfg.D * esz + cfg.B * cfg.Hq * 4
    idx_bytes = cfg.B * cfg.Hq * (cfg.budget + 1) * 4
    attn_bytes = kv_bytes + q_bytes + out_bytes + idx_bytes
    # sparse-only: the union of the group's selected blocks per (seq, kv head)
    G = cfg.Hq // cfg.Hkv
    ic = idx.view(cfg.B, cfg.Hkv, G, cfg.budget).cpu()
    union = 0
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            s = set(ic[b, g].flatten().tolist())
            s.discard(-1)
            union += len(s)
    sp_bytes = union * 2 * cfg.block * cfg.D * esz + q_bytes + cfg.B * cfg.Hq * cfg.D * esz + idx_bytes
    attn_ms, sel_ms, sp_ms = ta.mean_ms(), ts.mean_ms(), tsp.mean_ms()
    res = {
        "workload": f"gqa decode: {cfg.B} seqs x {cfg.Hq}/{cfg.Hkv} heads, KV {cfg.N}, D {cfg.D}, "
                    f"block {cfg.block}, budget {cfg.budget}",
        "ms_per_step": wall * 1e3 / steps,
        "tokens_per_s": cfg.B / (wall / steps),
        "select_ms": sel_ms,
        "attn_ms": attn_ms,
        "attn_bytes": attn_bytes,
        "attn_GBps": attn_bytes / attn_ms / 1e6,
        "attn_hbm_frac": attn_bytes / attn_ms / 1e6 / HBM_PEAK_GBS,
        "step_GBps": (attn_bytes + table_bytes) / (sel_ms + attn_ms) / 1e6,
        "sparse_only_attn_ms": sp_ms,
        "sparse_only_bytes": sp_bytes + table_bytes,
        "sparse_only_GBps": (sp_bytes + table_bytes) / (sp_ms + sel_ms) / 1e6,
        "sparse_only_union_blocks_per_group": union / (cfg.B * cfg.Hkv),
    }
    del q, k, v, kp, out, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, seconds_target=15.0):
    """The fp64 oracle on a bounded sample of the prefill workload: one q head,
    its selection, and query rows sampled evenly over the sequence."""
    import numpy as np
    from oracle import ssa_oracle as O
    from ssa_inputs import default_head_map, make_head, scale_for
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    h = 5
    x = make_head(cfg, 0, h)
    q = x["q"].float().numpy()[None, None]
    k = x["k"].float().numpy()[None, None]
    v = x["v"].float().numpy()[None, None]
    t0 = time.perf_counter()
    idx, cnt = O.select_blocks(q, k, block=cfg.block, budget=cfg.budget, n_sink=cfg.n_sink,
                               n_local=cfg.n_local, head_map=[0])
    t_sel = time.perf_counter() - t0
    rows_done, flops, t_att = 0, 0.0, 0.0
    # random rows, 256 at a time, until the time target is met
    order = np.random.default_rng(0).permutation(cfg.N)
    pos = 0
    while t_att < seconds_target and pos < cfg.N:
        r = np.sort(order[pos:pos + 256])
        pos += 256
        t1 = time.perf_counter()
        O.dual_attention(q, k, v, idx, block=cfg.block, scale=scale_for(cfg), head_map=[0],
                         rows={(0, 0): r})
        t_att += time.perf_counter() - t1
        flops += float(sum(4.0 * cfg.D * cfg.block * (rr // cfg.block + 1) for rr in r))
        rows_done += len(r)
    # scale: selection share of one head out of Hq heads plus the sampled rows
    sel_share = t_sel * rows_done / cfg.N
    total_s = t_att + sel_share
    return {"value": flops / total_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, q head {h} of {cfg.name} (N={cfg.N}, budget "
                      f"{cfg.budget}): selection for all {cfg.N // cfg.block} query blocks "
                      f"({t_sel:.2f}s, charged pro rata) + both streams and delta for "
                      f"{rows_done} random query rows ({t_att:.1f}s); value = algorithmic "
                      f"full-stream FLOPs of those rows / time",
            "rows": rows_done, "seconds": round(total_s, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--budget", type=int, default=16)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward pass (prints one JSON object)")
    ap.add_argument("--paper-only", action="store_true",
                    help="only time the pages' shape (16-token blocks, D 64): forward, backward, "
                         "per-token selection, 16:1 GQA (prints one JSON object)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (x3), the reference for "
                         "scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written":
                          dst.numel() * 2, "copies": 3}), flush=True)
        return
    import block_sparse_full_amd as ssa
    from ssa_inputs import CONFIGS
    ssa.load_library()

    cfg = CONFIGS["gqa_32k_sweep"].with_budget(args.budget)
    if args.backward_only:
        print(json.dumps({"backward": run_backward(ssa, torch, cfg, args.steps, args.warmup)}),
              flush=True)
        return
    if args.paper_only:
        print(json.dumps({"paper_shape": run_paper_shape(ssa, torch, CONFIGS["paper_16k_b16"],
                                                         args.steps)}), flush=True)
        return
    if args.no_prefill:
        dec = run_decode(ssa, torch, CONFIGS["gqa_decode_64k"], args.steps, args.warmup)
        print(json.dumps({"decode": dec}), flush=True)
        return
    pre = run_prefill(ssa, torch, cfg, args.steps, args.warmup,
                      [] if args.no_sweep else list(cfg.budgets))
    flops = prefill_flops(cfg)
    step_s = pre["ms_per_step"] / 1e3
    value = flops / step_s / 1e12
    kernel_tflops = flops / (pre["kernel_ms"] / 1e3) / 1e12
    result = {
        "metric": "dual-stream attn fwd TFLOP/s + tokens/s at 32K (% MFMA peak); decode GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V with planted peaked key blocks)",
        "config": {"workload": f"gqa prefill 32K: B {cfg.B}, {cfg.Hq} q heads / {cfg.Hkv} kv "
                               f"heads, N {cfg.N}, D {cfg.D}, block {cfg.block}, budget "
                               f"{cfg.budget} (sink + local included)",
                   "global_batch": cfg.B, "seq_len": cfg.N, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(cfg.B * cfg.N / step_s, 1),
        "mfma_frac_step": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "attn_ms": round(pre["attn_ms"], 4),
        "kernel_ms": round(pre["kernel_ms"], 4),
        "roofline": {"bound": "mfma",
                     "kernel": "attn_prefill_bf16_pp_kernel (the attention kernel of ssa_attn_fwd)",
                     "achieved": round(kernel_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": prefill_traffic()},
        "loss_sparsity": pre["loss"],
        "delta_mean": round(pre["delta_mean"], 4),
        "budget_sweep": pre.get("sweep"),
        "group_select": pre.get("group_select"),
        "token_select": pre.get("token_select"),
    }
    if not args.no_backward:
        result["backward"] = run_backward(ssa, torch, cfg, max(5, args.steps // 2), args.warmup)
    if not args.no_sweep:
        result["paper_shape"] = run_paper_shape(ssa, torch, CONFIGS["paper_16k_b16"], args.steps)
    if not args.no_decode:
        dec = run_decode(ssa, torch, CONFIGS["gqa_decode_64k"], max(5, args.steps // 2),
                         args.warmup)
        result["decode"] = {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                            for kk, vv in dec.items()}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
