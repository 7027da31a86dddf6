"""Seeded random problem shapes through the HIP path, each compared in full
with the fp64 oracle (indices bit-exact, streams and delta within the bars).
Covers GQA ratios 1-8, D 64/128, odd block counts, every sink/local mix,
budgets from the forced minimum to above the block count, prefill and
decode, bf16 and float32, planted and iid inputs; a second set draws the
selection mode (per head, per GQA group, per token), 16- or 64-token blocks
and sparse-only calls as well."""
import numpy as np
import pytest

from gpu_common import full_compare, gpu_run
from ssa_inputs import CONFIGS, default_head_map, make_inputs

pytestmark = pytest.mark.gpu


def random_cases(n=14, seed=2024):
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        decode = bool(r.integers(0, 3) == 0)
        f32 = bool(r.integers(0, 5) == 0)
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.choice([1, 2]))
        D = int(r.choice([64, 128]))
        nkb = int(r.integers(1, 25)) if not decode else int(r.integers(2, 70))
        n_sink, n_local = int(r.integers(0, 3)), int(r.integers(0, 3))
        budget = max(1, n_sink + n_local + int(r.integers(0, 6)))
        if r.integers(0, 4) == 0:
            budget = nkb + int(r.integers(0, 3))      # covers every block
        budget = max(budget, n_sink + n_local, 1)
        B = int(r.choice([1, 2, 3])) if decode else int(r.choice([1, 2]))
        base = "gqa_decode_64k" if decode else "gqa_8k_peaked"
        cases.append(dict(base=base, B=B, Hq=G * Hkv, Hkv=Hkv, N=64 * nkb, D=D, budget=budget,
                          n_sink=n_sink, n_local=n_local, dtype="f32" if f32 else "bf16",
                          planted=bool(r.integers(0, 2)), seed=100 + i))
    return cases


CASES = random_cases(24)


def random_mode_cases(n=14, seed=2025):
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        decode = bool(r.integers(0, 4) == 0)
        f32 = bool(r.integers(0, 6) == 0)
        block = 64 if f32 else int(r.choice([16, 64]))
        G = int(r.choice([1, 2, 4, 8]))
        Hkv = int(r.choice([1, 2]))
        D = int(r.choice([64, 128]))
        tiles = int(r.integers(1, 13)) if not decode else int(r.integers(2, 40))
        nkb = tiles * 64 // block
        n_sink, n_local = int(r.integers(0, 3)), int(r.integers(0, 3))
        budget = max(1, n_sink + n_local + int(r.integers(0, 8)))
        if r.integers(0, 5) == 0:
            budget = nkb + int(r.integers(0, 3))
        budget = min(max(budget, n_sink + n_local, 1), 64)
        mode = str(r.choice(["head", "group", "token"]))
        sparse = bool(r.integers(0, 4) == 0)
        B = int(r.choice([1, 2]))
        base = "gqa_decode_64k" if decode else "gqa_8k_peaked"
        cases.append(dict(base=base, B=B, Hq=G * Hkv, Hkv=Hkv, N=64 * tiles, D=D, budget=budget,
                          n_sink=n_sink, n_local=n_local, dtype="f32" if f32 else "bf16",
                          block=block, planted=bool(r.integers(0, 2)), seed=300 + i,
                          mode=mode, sparse=sparse))
    return cases


MODE_CASES = random_mode_cases(24)


@pytest.mark.parametrize("case", CASES, ids=[f"r{i}-{c['base'][:7]}-G{c['Hq'] // c['Hkv']}-"
                                            f"N{c['N']}-D{c['D']}-b{c['budget']}-{c['dtype']}"
                                            for i, c in enumerate(CASES)])
def test_random_shape(case):
    import block_sparse_full_amd as ssa
    ssa.load_library()
    c = dict(case)
    base = c.pop("base")
    cfg = CONFIGS[base].with_sizes(**c)
    print(f"[random] {cfg}", flush=True)
    x = make_inputs(cfg)
    got = gpu_run(ssa, x, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                  want_lse=True)
    full_compare(cfg, x, got, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                 lse=True)


@pytest.mark.parametrize("case", MODE_CASES,
                         ids=[f"m{i}-{c['base'][:7]}-{c['mode']}-bs{c['block']}-G{c['Hq'] // c['Hkv']}-"
                              f"N{c['N']}-D{c['D']}-b{c['budget']}-{c['dtype']}{'-sparse' if c['sparse'] else ''}"
                              for i, c in enumerate(MODE_CASES)])
def test_random_mode(case):
    import block_sparse_full_amd as ssa
    ssa.load_library()
    c = dict(case)
    base, mode, sparse = c.pop("base"), c.pop("mode"), c.pop("sparse")
    cfg = CONFIGS[base].with_sizes(**c)
    print(f"[random] {cfg} mode={mode} sparse_only={sparse}", flush=True)
    x = make_inputs(cfg)
    kw = dict(group_select=mode == "group", token_select=mode == "token")
    got = gpu_run(ssa, x, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                  want_lse=not sparse, sparse_only=sparse, block=cfg.block, **kw)
    full_compare(cfg, x, got, budget=cfg.budget, n_sink=cfg.n_sink, n_local=cfg.n_local,
                 lse=not sparse, sparse_only=sparse, **kw)
