"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ssa.h declares, and rejects invalid problems with the
documented status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_full_amd import ssa
    if not os.path.exists(ssa.lib_path()):
        from block_sparse_full_amd.build import build_library
        build_library()
    return ssa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ssa_select_blocks", "ssa_attn_fwd", "ssa_align_loss", "ssa_pool_blocks",
              "ssa_workspace_bytes", "ssa_status_string", "ssa_last_error_message"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in ssa.h but not exported"


def _p(**kw):
    from block_sparse_full_amd.ssa import Problem
    base = dict(B=1, Hq=8, Hkv=2, Nq=4096, Nk=4096, D=128, budget=16)
    base.update(kw)
    return Problem(**base)


def _status_of(lib, prob, fn="ssa_select_blocks"):
    c, keep = prob.to_c()
    if fn == "ssa_select_blocks":
        return lib.ssa_select_blocks(ctypes.byref(c), 16, 16, None, 16, 16, None, 0, None)
    if fn == "ssa_attn_fwd":
        return lib.ssa_attn_fwd(ctypes.byref(c), 16, 16, 16, 16, 16, 16, 16, None, None, None, 0, None)
    raise ValueError(fn)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(budget=0), 1), (dict(n_sink=-1), 1),
    (dict(Hq=8, Hkv=3), 1), (dict(budget=1, n_sink=1, n_local=1), 1),
    (dict(head_map=[0, 0, 0, 0, 0, 1, 1, 1]), 1), (dict(head_map=[0, 1, 2, 0, 1, 0, 1, 0]), 1),
    (dict(D=96), 2), (dict(block_size=32), 2), (dict(Nk=4000, Nq=4000), 2),
    (dict(Nq=7), 2), (dict(dtype=5), 2), (dict(Hq=64, Hkv=2), 2), (dict(scale=-1.0), 1),
    (dict(Nq=1, Nk=4096, Hq=32, Hkv=2), 3),        # bf16 decode, 16 q heads per kv head: valid
    (dict(selection=3), 1), (dict(selection=-1), 1),
    (dict(selection=2), 3),                         # per-token selection: valid, no workspace
    (dict(selection=2, budget=64), 3),              # longest per-token list
    (dict(selection=2, budget=65), 2),              # per-token lists hold at most 64 blocks
    (dict(selection=2, budget=65, Nq=1), 3),        # decode: per token is per head, no limit
    (dict(block_size=16), 3),                       # 16-token blocks: valid (bf16), no workspace
    (dict(block_size=16, dtype=0), 2),              # 16-token blocks need bf16
    (dict(block_size=16, Nk=200, Nq=200), 2),       # Nk must still be a multiple of 64
    (dict(selection=1), 3),                         # group selection, no workspace
    (dict(), 3),                                    # valid problem, no workspace
])
def test_invalid_problems_are_rejected(lib, kw, status):
    st = _status_of(lib, _p(**kw))
    assert st == status, (kw, st, lib.ssa_last_error_message())
    assert lib.ssa_last_error_message()  # a reason is given


def test_null_pointers(lib):
    c, keep = _p().to_c()
    assert lib.ssa_select_blocks(ctypes.byref(c), None, 16, None, 16, 16, None, 0, None) == 1
    assert lib.ssa_select_blocks(ctypes.byref(c), 16, None, None, 16, 16, None, 0, None) == 1
    assert lib.ssa_attn_fwd(ctypes.byref(c), 16, 16, 16, 16, 16, 16, None, None, None, None, 0, None) == 1
    # delta without h_full (sparse-only mode has no dropped mass)
    assert lib.ssa_attn_fwd(ctypes.byref(c), 16, 16, 16, 16, 16, None, 16, 16, None, None, 0, None) == 1
    assert lib.ssa_align_loss(ctypes.byref(c), None, 16, 16, None, None, None, 0, None) == 1
    assert lib.ssa_align_loss_noalloc(ctypes.byref(c), None, 16, 16, None, None, None) == 1
    assert lib.ssa_align_loss_noalloc(ctypes.byref(c), 16, 16, None, None, None, None) == 1
    assert lib.ssa_pool_blocks(ctypes.byref(c), None, 2, 16, None) == 1
    assert lib.ssa_pool_blocks(ctypes.byref(c), 16, 0, 16, None) == 1
    assert lib.ssa_select_blocks(None, 16, 16, None, 16, 16, None, 0, None) == 1


def test_workspace_checks(lib):
    from block_sparse_full_amd.ssa import workspace_bytes
    p = _p()
    need = workspace_bytes(p)
    # pooled Q + pooled K + transposed V + key-block norms (2 x 64 floats,
    # 512 bytes) + prefill work queues (8 counters on 256-byte lines) + loss
    # partials, each 256-byte aligned
    expect = (8 * 64 * 128 * 4 + 2 * 64 * 128 * 4 + 2 * 128 * 4096 * 2 + 512 + 8 * 256
              + 1024 * 8)
    assert need == expect
    c, keep = p.to_c()
    st = lib.ssa_align_loss(ctypes.byref(c), 16, 16, 16, None, None, 4096, need - 256, None)
    assert st == 3
    st = lib.ssa_align_loss(ctypes.byref(c), 16, 16, 16, None, None, 4096 + 8, need, None)
    assert st == 3  # not 256-byte aligned
    bad = _p(D=96)
    c2, keep2 = bad.to_c()
    assert lib.ssa_workspace_bytes(ctypes.byref(c2)) == 0


def test_status_strings(lib):
    assert lib.ssa_status_string(0) == b"SSA_OK"
    assert lib.ssa_status_string(3) == b"SSA_ERR_WORKSPACE"
    assert lib.ssa_status_string(99) == b"SSA_ERR_UNKNOWN"


def test_binding_refuses_host_tensors(lib):
    """The binding never computes on the CPU: host tensors are rejected."""
    import torch
    from block_sparse_full_amd import ssa
    q = torch.zeros(1, 2, 128, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    p = ssa.problem_for(q, k, budget=2)
    ws = torch.zeros(ssa.workspace_bytes(p) + 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        ssa.select_blocks(p, q, k, ws=ws)
    with pytest.raises(TypeError):
        ssa.problem_for(q.to(torch.float16), k, budget=2)


def test_missing_library_fails_loudly(tmp_path):
    from block_sparse_full_amd import ssa
    with pytest.raises(RuntimeError, match="no fallback"):
        ssa.load_library(str(tmp_path / "libssa.so"))


def _bwd(lib, c, *, q=16, lse=16, hf=16, hs=16, gf=16, gs=16, dq=16, ws=None, wn=0):
    return lib.ssa_attn_bwd(ctypes.byref(c), q, 16, 16, 16, 16, hf, hs, lse, gf, gs, dq, 16, 16,
                            ws, wn, None)


def test_backward_argument_checks(lib):
    c, keep = _p().to_c()
    assert _bwd(lib, c) == 3                       # valid, no workspace
    assert _bwd(lib, c, q=None) == 1
    assert _bwd(lib, c, lse=None) == 1
    assert _bwd(lib, c, dq=None) == 1
    assert _bwd(lib, c, gf=None, gs=None) == 1     # no upstream gradient at all
    assert _bwd(lib, c, hf=None) == 1              # d_full without h_full
    assert _bwd(lib, c, hs=None) == 1              # d_sparse without h_sparse
    assert _bwd(lib, c, hf=None, gf=None) == 3     # sparse stream only: valid
    assert _bwd(lib, c, hs=None, gs=None) == 3     # full stream only: valid
    dec, keep2 = _p(Nq=1).to_c()
    assert _bwd(lib, dec) == 2                     # decode has no backward here
    assert lib.ssa_bwd_workspace_bytes(ctypes.byref(dec)) == 0
    bad, keep3 = _p(D=96).to_c()
    assert _bwd(lib, bad) == 2


def test_token_selection_host(lib):
    """Per-token lists: the backward accepts them (bf16 and float32); the
    forward workspace adds the float64 chunked copy of the pooled keys and
    the bf16 backward workspace one 64-bit row mask per (q head, 128-key
    tile, 32-row step, 32-key block)."""
    from block_sparse_full_amd.ssa import SSA_SELECT_TOKEN, bwd_workspace_bytes, workspace_bytes
    c, keep = _p(selection=SSA_SELECT_TOKEN).to_c()
    assert _bwd(lib, c) == 3                       # valid, no workspace
    extra = bwd_workspace_bytes(_p(selection=SSA_SELECT_TOKEN)) - bwd_workspace_bytes(_p())
    assert extra == 8 * (4096 // 128) * (4096 // 32) * 4 * 8
    c32, keep2 = _p(selection=SSA_SELECT_TOKEN, dtype=0, D=64).to_c()
    assert _bwd(lib, c32) == 3                     # valid, no workspace
    base = workspace_bytes(_p())
    tok = workspace_bytes(_p(selection=SSA_SELECT_TOKEN))
    assert tok - base == 2 * 64 * 128 * 8          # Hkv 2, 64 blocks (4 chunks of 16), D 128
    p = _p(selection=SSA_SELECT_TOKEN)
    assert p.n_qblocks == 4096
    assert _p(selection=SSA_SELECT_TOKEN, Nq=1).n_qblocks == 1


def test_backward_workspace_size(lib):
    from block_sparse_full_amd.ssa import bwd_workspace_bytes
    p = _p()                        # B1 Hq8 Hkv2 N4096 D128 bf16
    need = bwd_workspace_bytes(p)
    stats = 8 * 4096 * 4 * 4
    bits = 8 * (4096 // 128) * (4096 // 32) * 2
    # float32 dQ, and dK, dV per head group of the full-stream pass: 32 key
    # tiles x 2 kv heads = 64 workgroups, below 4096, so each of the four
    # heads of a group gets its own workgroup and slot
    partials = (8 + 4 * 2 * 2) * 4096 * 128 * 4
    slots = 2 * 4 * 2 * 4096 * 128 * 4           # sparse dK, dV per q head of a group (4)
    assert need == stats + bits + partials + slots
    c, keep = p.to_c()
    assert _bwd(lib, c, ws=4096, wn=need - 256) == 3
    assert _bwd(lib, c, ws=4096 + 8, wn=need) == 3   # not 256-byte aligned
    f32 = _p(dtype=0)
    assert bwd_workspace_bytes(f32) == stats        # float32 path keeps statistics only


def test_timing_hook_arguments(lib):
    """The measurement hook takes both event handles or neither; one alone is
    rejected (no device work is involved in setting it)."""
    assert lib.ssa_set_attn_timing_events(ctypes.c_void_p(16), None) == 1
    assert "both" in lib.ssa_last_error_message().decode()
    assert lib.ssa_set_attn_timing_events(None, ctypes.c_void_p(16)) == 1
    assert lib.ssa_set_attn_timing_events(None, None) == 0
    assert lib.ssa_last_error_message().decode() == ""
