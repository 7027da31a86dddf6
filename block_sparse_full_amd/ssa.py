"""Python binding of the SSA C ABI (include/ssa.h) over ctypes.

Argument marshalling only: the functions check tensor placement, dtype,
shape and contiguity, allocate outputs and the workspace with torch on the
inputs' device, pass raw device pointers and torch's current HIP stream to
libssa.so, and raise SsaError on a non-OK status. Every step of the
computation runs in the library's HIP kernels; there is no CPU fallback, and
loading fails loudly when the library has not been built.

Function names follow the C entry points: pool_blocks, select_blocks,
attn_fwd, align_loss, workspace_bytes. dual_attention chains them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Dict, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssa.so")
_lib = None

SSA_F32, SSA_BF16 = 0, 1
SSA_SELECT_PER_HEAD, SSA_SELECT_GROUP, SSA_SELECT_TOKEN = 0, 1, 2
STATUS = {0: "SSA_OK", 1: "SSA_ERR_INVALID_ARG", 2: "SSA_ERR_UNSUPPORTED",
          3: "SSA_ERR_WORKSPACE", 4: "SSA_ERR_HIP"}
EXPORTS = ("ssa_workspace_bytes", "ssa_pool_blocks", "ssa_select_blocks", "ssa_attn_fwd",
           "ssa_align_loss", "ssa_align_loss_noalloc", "ssa_set_attn_timing_events",
           "ssa_status_string", "ssa_last_error_message")


class SsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class SsaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("head_map", ctypes.POINTER(ctypes.c_int32)), ("selection", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libssa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m block_sparse_full_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(SsaProblem)
    vp, i32p, f32p, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    lib.ssa_workspace_bytes.argtypes = [P]
    lib.ssa_workspace_bytes.restype = sz
    lib.ssa_pool_blocks.argtypes = [P, vp, ctypes.c_int32, f32p, vp]
    lib.ssa_pool_blocks.restype = ctypes.c_int
    lib.ssa_select_blocks.argtypes = [P, vp, vp, f32p, i32p, i32p, vp, sz, vp]
    lib.ssa_select_blocks.restype = ctypes.c_int
    lib.ssa_attn_fwd.argtypes = [P, vp, vp, vp, i32p, i32p, vp, vp, f32p, f32p, vp, sz, vp]
    lib.ssa_attn_fwd.restype = ctypes.c_int
    lib.ssa_align_loss.argtypes = [P, vp, vp, f32p, vp, vp, vp, sz, vp]
    lib.ssa_align_loss.restype = ctypes.c_int
    lib.ssa_align_loss_noalloc.argtypes = [P, vp, vp, f32p, vp, vp, vp]
    lib.ssa_align_loss_noalloc.restype = ctypes.c_int
    lib.ssa_set_attn_timing_events.argtypes = [vp, vp]
    lib.ssa_set_attn_timing_events.restype = ctypes.c_int
    lib.ssa_bwd_workspace_bytes.argtypes = [P]
    lib.ssa_bwd_workspace_bytes.restype = sz
    lib.ssa_attn_bwd.argtypes = [P, vp, vp, vp, i32p, i32p, vp, vp, f32p, vp, vp, vp, vp, vp, vp,
                                 sz, vp]
    lib.ssa_attn_bwd.restype = ctypes.c_int
    lib.ssa_status_string.argtypes = [ctypes.c_int]
    lib.ssa_status_string.restype = ctypes.c_char_p
    lib.ssa_last_error_message.argtypes = []
    lib.ssa_last_error_message.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


@dataclasses.dataclass
class Problem:
    """Mirror of the C ssa_problem."""
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    budget: int
    n_sink: int = 1
    n_local: int = 1
    block_size: int = 64
    scale: float = 0.0
    dtype: int = SSA_BF16
    head_map: Optional[Sequence[int]] = None
    selection: int = SSA_SELECT_PER_HEAD

    def to_c(self):
        hm = None
        keep = None
        if self.head_map is not None:
            keep = (ctypes.c_int32 * len(self.head_map))(*[int(x) for x in self.head_map])
            hm = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
        c = SsaProblem(self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.D, self.block_size,
                       self.budget, self.n_sink, self.n_local, float(self.scale), self.dtype, hm,
                       int(self.selection))
        return c, keep

    @property
    def n_qblocks(self) -> int:
        """Selection lists per (b, q head): one per query block, one per
        query row with SSA_SELECT_TOKEN, one in decode."""
        if self.Nq == 1:
            return 1
        return self.Nq if self.selection == SSA_SELECT_TOKEN else self.Nq // self.block_size

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == SSA_BF16 else torch.float32


def problem_for(q: torch.Tensor, k: torch.Tensor, *, budget: int, n_sink: int = 1,
                n_local: int = 1, block_size: int = 64, scale: float = 0.0,
                head_map: Optional[Sequence[int]] = None, group_select: bool = False,
                token_select: bool = False) -> Problem:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D [B, H, N, D]")
    dt = {torch.bfloat16: SSA_BF16, torch.float32: SSA_F32}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return Problem(B=q.shape[0], Hq=q.shape[1], Hkv=k.shape[1], Nq=q.shape[2], Nk=k.shape[2],
                   D=q.shape[3], budget=budget, n_sink=n_sink, n_local=n_local,
                   block_size=block_size, scale=scale, dtype=dt, head_map=head_map,
                   selection=(SSA_SELECT_TOKEN if token_select else
                              SSA_SELECT_GROUP if group_select else SSA_SELECT_PER_HEAD))


def _check(status: int):
    if status != 0:
        msg = load_library().ssa_last_error_message().decode(errors="replace")
        raise SsaError(status, msg)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(p: Problem) -> int:
    c, keep = p.to_c()
    n = load_library().ssa_workspace_bytes(ctypes.byref(c))
    if n == 0:
        # ask a call for the reason
        st = load_library().ssa_pool_blocks(ctypes.byref(c), None, 0, None, None)
        _check(st if st != 0 else 1)
    return n


def alloc_workspace(p: Problem, device) -> torch.Tensor:
    n = workspace_bytes(p)
    return torch.empty(n + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws: torch.Tensor):
    base = ws.data_ptr()
    aligned = (base + 255) & ~255
    return aligned, ws.numel() - (aligned - base)


def pool_blocks(p: Problem, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block mean-pool of x [B, H, Nk, D] -> float32 [B, H, Nk/64, D]."""
    B, H, N, D = x.shape
    if out is None:
        out = torch.empty(B, H, N // p.block_size, D, dtype=torch.float32, device=x.device)
    c, keep = p.to_c()
    _check(load_library().ssa_pool_blocks(ctypes.byref(c), _dev(x, "x", p.torch_dtype), H,
                                          _dev(out, "pooled", torch.float32), _stream()))
    return out


def select_blocks(p: Problem, q: torch.Tensor, k: Optional[torch.Tensor] = None,
                  k_pooled: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  idx: Optional[torch.Tensor] = None, cnt: Optional[torch.Tensor] = None):
    """Selected key blocks (idx [B,Hq,nQB,budget] int32, cnt [B,Hq,nQB] int32)."""
    dev = q.device
    nqb = p.n_qblocks
    if idx is None:
        idx = torch.empty(p.B, p.Hq, nqb, p.budget, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty(p.B, p.Hq, nqb, dtype=torch.int32, device=dev)
    _dev(idx, "idx", torch.int32, (p.B, p.Hq, nqb, p.budget))
    _dev(cnt, "cnt", torch.int32, (p.B, p.Hq, nqb))
    ws = ws if ws is not None else alloc_workspace(p, dev)
    wp, wn = _ws_ptr(ws)
    c, keep = p.to_c()
    _check(load_library().ssa_select_blocks(
        ctypes.byref(c), _dev(q, "q", p.torch_dtype, (p.B, p.Hq, p.Nq, p.D)),
        _dev(k, "k", p.torch_dtype, (p.B, p.Hkv, p.Nk, p.D)),
        _dev(k_pooled, "k_pooled", torch.float32, (p.B, p.Hkv, p.Nk // p.block_size, p.D)),
        idx.data_ptr(), cnt.data_ptr(), wp, wn, _stream()))
    return idx, cnt


def attn_fwd(p: Problem, q, k, v, idx, cnt, *, sparse_only: bool = False, want_delta: bool = True,
             want_lse: bool = False, ws: Optional[torch.Tensor] = None,
             out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Dual-stream attention: dict with h_full (unless sparse_only), h_sparse,
    delta (if wanted and not sparse_only) and lse [2,B,Hq,Nq] (if wanted)."""
    dev = q.device
    o = dict(out or {})
    shp = (p.B, p.Hq, p.Nq, p.D)
    if "h_sparse" not in o:
        o["h_sparse"] = torch.empty(shp, dtype=p.torch_dtype, device=dev)
    if not sparse_only and "h_full" not in o:
        o["h_full"] = torch.empty(shp, dtype=p.torch_dtype, device=dev)
    if not sparse_only and want_delta and "delta" not in o:
        o["delta"] = torch.empty(p.B, p.Hq, p.Nq, dtype=torch.float32, device=dev)
    if want_lse and "lse" not in o:
        o["lse"] = torch.empty(2, p.B, p.Hq, p.Nq, dtype=torch.float32, device=dev)
    ws = ws if ws is not None else alloc_workspace(p, dev)
    wp, wn = _ws_ptr(ws)
    c, keep = p.to_c()
    nqb = p.n_qblocks
    _check(load_library().ssa_attn_fwd(
        ctypes.byref(c), _dev(q, "q", p.torch_dtype, shp),
        _dev(k, "k", p.torch_dtype, (p.B, p.Hkv, p.Nk, p.D)),
        _dev(v, "v", p.torch_dtype, (p.B, p.Hkv, p.Nk, p.D)),
        _dev(idx, "idx", torch.int32, (p.B, p.Hq, nqb, p.budget)),
        _dev(cnt, "cnt", torch.int32, (p.B, p.Hq, nqb)),
        None if sparse_only else _dev(o["h_full"], "h_full", p.torch_dtype, shp),
        _dev(o["h_sparse"], "h_sparse", p.torch_dtype, shp),
        _dev(o.get("delta") if not sparse_only else None, "delta", torch.float32),
        _dev(o.get("lse"), "lse", torch.float32), wp, wn, _stream()))
    return o


def set_attn_timing_events(start=None, stop=None) -> None:
    """Record torch.cuda.Event `start` / `stop` around the attention kernel of
    every following bf16 prefill attn_fwd (the V transpose before it stays
    outside the pair); no arguments clears the hook. The events must have been
    recorded once (torch creates them on first use)."""
    if (start is None) != (stop is None):
        raise ValueError("give both events or neither")
    h0 = None if start is None else ctypes.c_void_p(start.cuda_event)
    h1 = None if stop is None else ctypes.c_void_p(stop.cuda_event)
    if start is not None and (not h0.value or not h1.value):
        raise ValueError("record the events once before passing them")
    _check(load_library().ssa_set_attn_timing_events(h0, h1))


def align_loss(p: Problem, h_full, h_sparse, *, want_grads: bool = False,
               ws: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None):
    """(loss float32[2] on the device, grad_full, grad_sparse or None)."""
    dev = h_full.device
    shp = (p.B, p.Hq, p.Nq, p.D)
    if loss is None:
        loss = torch.empty(2, dtype=torch.float32, device=dev)
    _dev(loss, "loss", torch.float32, (2,))
    gf = torch.empty(shp, dtype=p.torch_dtype, device=dev) if want_grads else None
    gs = torch.empty(shp, dtype=p.torch_dtype, device=dev) if want_grads else None
    ws = ws if ws is not None else alloc_workspace(p, dev)
    wp, wn = _ws_ptr(ws)
    c, keep = p.to_c()
    _check(load_library().ssa_align_loss(
        ctypes.byref(c), _dev(h_full, "h_full", p.torch_dtype, shp),
        _dev(h_sparse, "h_sparse", p.torch_dtype, shp), loss.data_ptr(),
        _dev(gf, "grad_full"), _dev(gs, "grad_sparse"), wp, wn, _stream()))
    return loss, gf, gs


def align_loss_noalloc(p: Problem, h_full, h_sparse, *, want_grads: bool = False,
                       loss: Optional[torch.Tensor] = None):
    """align_loss through ssa_align_loss_noalloc: the library's own static
    scratch instead of a workspace. Outputs are allocated here unless given."""
    dev = h_full.device
    shp = (p.B, p.Hq, p.Nq, p.D)
    if loss is None:
        loss = torch.empty(2, dtype=torch.float32, device=dev)
    _dev(loss, "loss", torch.float32, (2,))
    gf = torch.empty(shp, dtype=p.torch_dtype, device=dev) if want_grads else None
    gs = torch.empty(shp, dtype=p.torch_dtype, device=dev) if want_grads else None
    c, keep = p.to_c()
    _check(load_library().ssa_align_loss_noalloc(
        ctypes.byref(c), _dev(h_full, "h_full", p.torch_dtype, shp),
        _dev(h_sparse, "h_sparse", p.torch_dtype, shp), loss.data_ptr(),
        _dev(gf, "grad_full"), _dev(gs, "grad_sparse"), _stream()))
    return loss, gf, gs


def bwd_workspace_bytes(p: Problem) -> int:
    c, keep = p.to_c()
    n = load_library().ssa_bwd_workspace_bytes(ctypes.byref(c))
    if n == 0:
        st = load_library().ssa_attn_bwd(ctypes.byref(c), *([None] * 14), 0, None)
        _check(st if st != 0 else 1)
    return n


def alloc_bwd_workspace(p: Problem, device) -> torch.Tensor:
    return torch.empty(bwd_workspace_bytes(p) + 256, dtype=torch.uint8, device=device)


def attn_bwd(p: Problem, q, k, v, idx, cnt, lse, *, h_full=None, h_sparse=None, d_full=None,
             d_sparse=None, ws: Optional[torch.Tensor] = None,
             out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Backward of both streams: dict with dq [B,Hq,Nq,D], dk and dv
    [B,Hkv,Nk,D] for upstream gradients d_full / d_sparse (either may be
    None for zero) of h_full / h_sparse."""
    dev = q.device
    o = dict(out or {})
    shp = (p.B, p.Hq, p.Nq, p.D)
    kshp = (p.B, p.Hkv, p.Nk, p.D)
    if "dq" not in o:
        o["dq"] = torch.empty(shp, dtype=p.torch_dtype, device=dev)
    for name in ("dk", "dv"):
        if name not in o:
            o[name] = torch.empty(kshp, dtype=p.torch_dtype, device=dev)
    ws = ws if ws is not None else alloc_bwd_workspace(p, dev)
    wp, wn = _ws_ptr(ws)
    c, keep = p.to_c()
    nqb = p.n_qblocks
    _check(load_library().ssa_attn_bwd(
        ctypes.byref(c), _dev(q, "q", p.torch_dtype, shp), _dev(k, "k", p.torch_dtype, kshp),
        _dev(v, "v", p.torch_dtype, kshp),
        _dev(idx, "idx", torch.int32, (p.B, p.Hq, nqb, p.budget)),
        _dev(cnt, "cnt", torch.int32, (p.B, p.Hq, nqb)),
        _dev(h_full, "h_full", p.torch_dtype, shp), _dev(h_sparse, "h_sparse", p.torch_dtype, shp),
        _dev(lse, "lse", torch.float32, (2, p.B, p.Hq, p.Nq)),
        _dev(d_full, "d_full", p.torch_dtype, shp), _dev(d_sparse, "d_sparse", p.torch_dtype, shp),
        _dev(o["dq"], "dq", p.torch_dtype, shp), _dev(o["dk"], "dk", p.torch_dtype, kshp),
        _dev(o["dv"], "dv", p.torch_dtype, kshp), wp, wn, _stream()))
    return o


def dual_attention(q, k, v, *, budget: int, n_sink: int = 1, n_local: int = 1,
                   scale: float = 0.0, head_map=None, k_pooled=None, sparse_only: bool = False,
                   want_lse: bool = False, want_grads: bool = False, ws=None,
                   group_select: bool = False, block_size: int = 64,
                   token_select: bool = False):
    """Selection, both attention streams, dropped mass and alignment losses.
    group_select: one block list per GQA group (SSA_SELECT_GROUP);
    token_select: one block list per query row (SSA_SELECT_TOKEN);
    block_size: selection block in tokens (64 or 16)."""
    p = problem_for(q, k, budget=budget, n_sink=n_sink, n_local=n_local, scale=scale,
                    head_map=head_map, group_select=group_select, block_size=block_size,
                    token_select=token_select)
    ws = ws if ws is not None else alloc_workspace(p, q.device)
    idx, cnt = select_blocks(p, q, None if k_pooled is not None else k, k_pooled, ws=ws)
    out = attn_fwd(p, q, k, v, idx, cnt, sparse_only=sparse_only, want_lse=want_lse, ws=ws)
    out["idx"], out["cnt"] = idx, cnt
    if not sparse_only:
        loss, gf, gs = align_loss(p, out["h_full"], out["h_sparse"], want_grads=want_grads, ws=ws)
        out["loss"] = loss
        if want_grads:
            out["grad_full"], out["grad_sparse"] = gf, gs
    return out
