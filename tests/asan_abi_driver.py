"""Drives every host-side path of the C ABI in a library built with host
AddressSanitizer: problem validation for valid and invalid problems in each
selection mode, workspace sizing, layout arithmetic, the workspace checks and
the error strings. Every call is built to be rejected before the first HIP
call (NULL or undersized workspace, NULL outputs, H <= 0), so no kernel is
launched and no device is needed. Run by test_host_asan.py in a child process
with the ASan runtime preloaded; argv[1] is the library path."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_full_amd.ssa import (SSA_F32, SSA_SELECT_GROUP, SSA_SELECT_TOKEN,  # noqa: E402
                                       Problem, load_library)

FAKE = 0x1000          # never dereferenced: every call below fails validation first
ALIGNED = 0x100000     # 256-byte aligned, paired with a size below what is needed
MISALIGNED = 0x100010

VARIANTS = [
    dict(), dict(selection=SSA_SELECT_TOKEN), dict(selection=SSA_SELECT_GROUP),
    dict(block_size=16), dict(block_size=16, selection=SSA_SELECT_TOKEN), dict(Nq=1),
    dict(Nq=1, selection=SSA_SELECT_TOKEN), dict(D=64, dtype=SSA_F32),
    dict(D=64, dtype=SSA_F32, selection=SSA_SELECT_TOKEN), dict(budget=64, selection=SSA_SELECT_TOKEN),
    dict(Hq=32, Hkv=8, B=2), dict(head_map=[0, 1, 1, 0, 1, 0, 1, 0]), dict(Nk=262144, Nq=262144, Hq=1, Hkv=1),
    dict(Nk=65536, Nq=65536, block_size=16, Hq=2, Hkv=1, selection=SSA_SELECT_TOKEN),
    # invalid or unsupported problems
    dict(budget=65, selection=SSA_SELECT_TOKEN), dict(Hq=8, Hkv=3), dict(D=96), dict(block_size=32),
    dict(Nk=4000, Nq=4000), dict(Nq=7), dict(budget=1, n_sink=1, n_local=1), dict(n_sink=-1),
    dict(head_map=[0, 0, 0, 0, 0, 1, 1, 1]), dict(head_map=[0, 1, 2, 0, 1, 0, 1, 0]),
    dict(selection=7), dict(scale=float("nan")), dict(scale=-1.0), dict(dtype=9),
    dict(B=0), dict(Nk=2 ** 30, Nq=2 ** 30), dict(Hq=4096, Hkv=1), dict(block_size=16, dtype=SSA_F32),
]


def main():
    lib = load_library(sys.argv[1])
    n = 0
    for kw in VARIANTS:
        base = dict(B=1, Hq=8, Hkv=2, Nq=4096, Nk=4096, D=128, budget=16)
        base.update(kw)
        c, keep = Problem(**base).to_c()
        pc = ctypes.byref(c)
        need = lib.ssa_workspace_bytes(pc)
        need_b = lib.ssa_bwd_workspace_bytes(pc)
        for ws, wsb in ((None, 0), (MISALIGNED, 1 << 40), (ALIGNED, max(need, 1) - 1)):
            lib.ssa_select_blocks(pc, FAKE, FAKE, None, FAKE, FAKE, ws, wsb, None)
            lib.ssa_select_blocks(pc, FAKE, None, FAKE, FAKE, FAKE, ws, wsb, None)
            lib.ssa_attn_fwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, wsb, None)
            lib.ssa_align_loss(pc, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
        for ws, wsb in ((None, 0), (MISALIGNED, 1 << 40), (ALIGNED, max(need_b, 1) - 1)):
            lib.ssa_attn_bwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, ws, wsb, None)
        # argument checks that come before the workspace
        lib.ssa_attn_fwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None)
        lib.ssa_attn_bwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                         FAKE, FAKE, None, 0, None)
        lib.ssa_pool_blocks(pc, FAKE, 0, FAKE, None)
        lib.ssa_pool_blocks(pc, None, 2, FAKE, None)
        lib.ssa_last_error_message()
        n += 1
    for fn in ("ssa_select_blocks", "ssa_attn_fwd", "ssa_align_loss", "ssa_attn_bwd"):
        types = getattr(lib, fn).argtypes
        getattr(lib, fn)(*[0 if t is ctypes.c_size_t else None for t in types])
    lib.ssa_workspace_bytes(None)
    lib.ssa_bwd_workspace_bytes(None)
    for s in range(-1, 12):
        lib.ssa_status_string(s)
    lib.ssa_last_error_message()
    print(f"host paths driven: {n}", flush=True)


if __name__ == "__main__":
    main()
