"""Python binding of libultraep (exact-load MoE expert rebalancing on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI in ``include/ultraep.h``.  PyTorch supplies device memory
and the stream; the functions here take torch tensors, pass their device
pointers and the current HIP stream to the library, and raise on a non-zero
status.  There is no fallback: if ``libultraep.so`` is missing the first call
raises, telling the user to build it.

Names follow the C ABI: ``ultraep_create``, ``ultraep_balance``,
``ultraep_balance_static``,
``ultraep_dispatch_layout``, ``ultraep_permute``, ``ultraep_combine``,
``ultraep_combine_backward``, ``ultraep_weight_sync_plan``,
``ultraep_weight_sync``, ``ultraep_fold_grads``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libultraep.so")

# Plan record fields, in the order of enum ultraep_plan_field_id.
PLAN_FIELDS = ("header", "counts", "master_quota", "slot_expert", "slot_quota", "phys_load",
               "phys_off", "inst_ptr", "inst_phys", "inst_end", "inst_base", "rank_before",
               "rank_after", "inst_local")
REROUTE_RANGES, REROUTE_LOCAL, REROUTE_INTERLEAVE = 0, 1, 2
# Header words, in the order of enum ultraep_header_word.
HEADER_WORDS = ("magic", "E", "R", "S", "D", "M", "P", "N", "total", "dropped", "Q_star", "Q_lb",
                "Q_max", "tol", "grid_index", "floor", "replicas", "rounds")
PLAN_MAGIC = 0x55455031

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape, size or alignment",
          -3: "HIP launch or runtime error", -4: "workspace too small",
          -5: "needs more than the static workspace"}
STATIC_WORKSPACE_BYTES = 32 << 20


class UltraEPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, 'unknown status')} ({status})")
        self.status = status


class _Options(ctypes.Structure):
    _fields_ = [("eps_num", ctypes.c_int32), ("eps_den", ctypes.c_int32),
                ("allow_zero_master", ctypes.c_int32), ("threshold_num", ctypes.c_int32),
                ("threshold_den", ctypes.c_int32), ("reroute_mode", ctypes.c_int32),
                ("min_tokens_per_replica", ctypes.c_int32), ("replica_lean", ctypes.c_int32)]


class _RelayOptions(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("min_replicas", ctypes.c_int32),
                ("max_relays", ctypes.c_int32), ("min_gain", ctypes.c_int32),
                ("domain_gpus", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


RELAY_DIRECT, RELAY_ADAPTIVE, RELAY_FORCE = 0, 1, 2

_lib = None

_I32, _I64, _P, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_SIGNATURES = {
    "ultraep_create": (_I32, [_I32, _I32, _I32, _I32, ctypes.POINTER(_Options), ctypes.POINTER(_P)]),
    "ultraep_destroy": (_I32, [_P]),
    "ultraep_plan_bytes": (_I32, [_P, ctypes.POINTER(_SZ)]),
    "ultraep_plan_field": (_I32, [_P, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "ultraep_workspace_bytes": (_I32, [_P, _I32, _I64, _I32, ctypes.POINTER(_SZ)]),
    "ultraep_balance": (_I32, [_P, _I32, _P, _P, _I64, _I32, _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "ultraep_balance_static": (_I32, [_P, _I32, _P, _P, _I64, _I32, _P, _P, _P, _P, _P, _P]),
    "ultraep_dispatch_layout": (_I32, [_P, _I32, _I64, _I32, _P, _P, _P, _P, _P]),
    "ultraep_permute": (_I32, [_P, _P, _P, _I32, _P, _I64, _I32, _I32, _I32, _P, _I64, _P]),
    "ultraep_fold_grads": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _P]),
    "ultraep_combine": (_I32, [_P, _P, _P, _I32, _P, _I64, _I32, _I64, _I64, _P, _P]),
    "ultraep_combine_backward": (_I32, [_P, _P, _P, _I32, _P, _I64, _I32, _P, _I64, _I64, _P, _P, _P]),
    "ultraep_weight_sync_plan": (_I32, [_P, _P, ctypes.POINTER(_RelayOptions), _P, _P]),
    "ultraep_weight_sync": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "ultraep_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib() -> ctypes.CDLL:
    """Load libultraep.so (built in place by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import "
                               "__graft_entry__ as g; g.build()'` (needs hipcc for gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise UltraEPError(fn, status)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Context:
    """An ``ultraep_ctx``: the shape (E, R, S, D) and planning options."""

    def __init__(self, E: int, R: int, S: int, D: int, eps=(1, 100), allow_zero_master=False,
                 threshold=(1, 1), reroute_mode: int = 0, min_tokens: int = 1, replica_lean: bool = False):
        opt = _Options(int(eps[0]), int(eps[1]), int(bool(allow_zero_master)), int(threshold[0]),
                       int(threshold[1]), int(reroute_mode), int(min_tokens), int(replica_lean))
        self.reroute_mode = int(reroute_mode)
        h = _P()
        _check("ultraep_create", lib().ultraep_create(E, R, S, D, ctypes.byref(opt), ctypes.byref(h)))
        self.handle = h
        self.E, self.R, self.S, self.D = E, R, S, D
        self.M = E // R
        self.P = R * (self.M + S)
        sz = _SZ()
        _check("ultraep_plan_bytes", lib().ultraep_plan_bytes(h, ctypes.byref(sz)))
        self.plan_bytes = sz.value
        self.plan_words = sz.value // 4
        self.fields: Dict[str, tuple] = {}
        for i, name in enumerate(PLAN_FIELDS):
            off, cnt = _SZ(), _SZ()
            _check("ultraep_plan_field", lib().ultraep_plan_field(h, i, ctypes.byref(off), ctypes.byref(cnt)))
            self.fields[name] = (off.value // 4, cnt.value)

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.ultraep_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, L: int, T: int, k: int) -> int:
        sz = _SZ()
        _check("ultraep_workspace_bytes", lib().ultraep_workspace_bytes(self.handle, L, T, k, ctypes.byref(sz)))
        return sz.value

    def decode_plan(self, words: np.ndarray) -> Dict[str, np.ndarray]:
        """Split one plan record (int32 words, host copy) into its fields."""
        w = np.asarray(words, dtype=np.int32).reshape(-1)
        out = {name: w[off:off + cnt].copy() for name, (off, cnt) in self.fields.items()}
        hdr = out["header"]
        for i, name in enumerate(HEADER_WORDS):
            out[name] = int(hdr[i])
        return out


def ultraep_create(E: int, R: int, slots_per_rank: int, D: int, eps=(1, 100),
                   allow_zero_master: bool = False, threshold=(1, 1), reroute_mode: int = 0,
                   min_tokens: int = 1, replica_lean: bool = False) -> Context:
    return Context(E, R, slots_per_rank, D, eps, allow_zero_master, threshold, reroute_mode, min_tokens,
                   replica_lean)


def ultraep_balance(ctx: Context, topk_idx, T: int, k: int, workspace, plans, phys_idx, pos,
                    topk_w=None, inv=None, w_perm=None, L: Optional[int] = None, stream=None) -> None:
    """Count, plan and reroute L layers (topk_idx int32 [L, R*T, k] or [R*T, k]).

    With topk_w, inv and w_perm the dispatch layout is written in the same pass."""
    if L is None:
        L = topk_idx.shape[0] if topk_idx.dim() == 3 else 1
    st = lib().ultraep_balance(ctx.handle, L, _ptr(topk_idx), _ptr(topk_w), T, k, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(plans),
                               _ptr(phys_idx), _ptr(pos), _ptr(inv), _ptr(w_perm), _stream(stream))
    _check("ultraep_balance", st)


def ultraep_balance_static(ctx: Context, topk_idx, T: int, k: int, plans, phys_idx, pos,
                           topk_w=None, inv=None, w_perm=None, L: Optional[int] = None,
                           stream=None) -> None:
    """ultraep_balance with the library's static device workspace (no
    workspace argument; at most STATIC_WORKSPACE_BYTES of it)."""
    if L is None:
        L = topk_idx.shape[0] if topk_idx.dim() == 3 else 1
    st = lib().ultraep_balance_static(ctx.handle, L, _ptr(topk_idx), _ptr(topk_w), T, k, _ptr(plans),
                                      _ptr(phys_idx), _ptr(pos), _ptr(inv), _ptr(w_perm),
                                      _stream(stream))
    _check("ultraep_balance_static", st)


def ultraep_dispatch_layout(ctx: Context, T: int, k: int, pos, topk_w, inv, w_perm,
                            L: Optional[int] = None, stream=None) -> None:
    if L is None:
        L = pos.numel() // max(1, ctx.R * T * k) if T * k else 1
    st = lib().ultraep_dispatch_layout(ctx.handle, L, T, k, _ptr(pos), _ptr(topk_w), _ptr(inv),
                                       _ptr(w_perm), _stream(stream))
    _check("ultraep_dispatch_layout", st)


def ultraep_permute(ctx: Context, plan, inv, k: int, hidden, p_begin: int, p_end: int, out,
                    stream=None) -> None:
    """Gather bf16 rows (any 2-byte dtype; bits are moved untouched)."""
    H = hidden.shape[-1]
    rows = out.shape[0] if out.dim() > 1 else 0
    st = lib().ultraep_permute(ctx.handle, _ptr(plan), _ptr(inv), k, _ptr(hidden), hidden.shape[0],
                               H, p_begin, p_end, _ptr(out), rows, _stream(stream))
    _check("ultraep_permute", st)


def ultraep_fold_grads(ctx: Context, plan, master_ptrs, replica_grads, numel: int,
                       slot_begin: int, slot_end: int, stream=None) -> None:
    """master_ptrs: int64 device tensor [E] of fp32 master-gradient pointers."""
    st = lib().ultraep_fold_grads(ctx.handle, _ptr(plan), _ptr(master_ptrs), _ptr(replica_grads),
                                  numel, slot_begin, slot_end, _stream(stream))
    _check("ultraep_fold_grads", st)


def ultraep_combine(ctx: Context, pos, topk_w, k: int, rows, token_begin: int, token_end: int,
                    out, stream=None) -> None:
    """out[g - token_begin] = sum_j w[g, j] * rows[pos[g*k + j]] (bf16; topk_w None: unweighted)."""
    st = lib().ultraep_combine(ctx.handle, _ptr(pos), _ptr(topk_w), k, _ptr(rows), rows.shape[0],
                               rows.shape[-1], token_begin, token_end, _ptr(out), _stream(stream))
    _check("ultraep_combine", st)


def ultraep_combine_backward(ctx: Context, pos, topk_w, k: int, rows, grad_out, token_begin: int,
                             token_end: int, grad_rows, grad_topk_w, stream=None) -> None:
    """grad_rows[pos[n]] = w[n] * grad_out[g]; grad_topk_w[g, j] = <grad_out[g], rows[pos[n]]>."""
    st = lib().ultraep_combine_backward(ctx.handle, _ptr(pos), _ptr(topk_w), k, _ptr(rows),
                                        rows.shape[0], rows.shape[-1], _ptr(grad_out), token_begin,
                                        token_end, _ptr(grad_rows), _ptr(grad_topk_w), _stream(stream))
    _check("ultraep_combine_backward", st)


def ultraep_weight_sync_plan(ctx: Context, plan, relay, mode: int = RELAY_ADAPTIVE, min_replicas: int = 4,
                             max_relays: int = 8, min_gain: int = 2, domain_gpus: Optional[int] = None,
                             stream=None) -> None:
    """relay: int32 device tensor [2, R*S] (source slot / -1 master / -2 empty; stage)."""
    o = _RelayOptions(mode, min_replicas, max_relays, min_gain, ctx.D if domain_gpus is None else domain_gpus)
    st = lib().ultraep_weight_sync_plan(ctx.handle, _ptr(plan), ctypes.byref(o), _ptr(relay), _stream(stream))
    _check("ultraep_weight_sync_plan", st)


def ultraep_weight_sync(ctx: Context, plan, master_ptrs, replica_weights, numel: int, slot_begin: int,
                        slot_end: int, relay=None, stream=None) -> None:
    """master_ptrs: int64 device tensor [E] of master-weight pointers (16-bit elements)."""
    st = lib().ultraep_weight_sync(ctx.handle, _ptr(plan), _ptr(master_ptrs), _ptr(replica_weights), numel,
                                   slot_begin, slot_end, _ptr(relay), _stream(stream))
    _check("ultraep_weight_sync", st)


def status_string(status: int) -> str:
    return lib().ultraep_status_string(status).decode()


class Buffers:
    """Device buffers for balancing L layers of one shape (torch tensors)."""

    def __init__(self, ctx: Context, L: int, T: int, k: int, device="cuda"):
        import torch
        N = ctx.R * T * k
        self.L, self.T, self.k, self.N = L, T, k, N
        self.workspace = torch.empty(max(1, ctx.workspace_bytes(L, T, k)) // 4, dtype=torch.int32, device=device)
        self.plans = torch.empty((L, ctx.plan_words), dtype=torch.int32, device=device)
        self.phys_idx = torch.empty((L, N), dtype=torch.int32, device=device)
        self.pos = torch.empty((L, N), dtype=torch.int32, device=device)
        self.inv = torch.empty((L, N), dtype=torch.int32, device=device)
        self.w_perm = torch.empty((L, N), dtype=torch.float32, device=device)
