"""The C ABI on the host (no GPU): symbols, argument checks, plan layout.

Every call here either makes no HIP call at all (create, sizes, layout) or
fails its host-side argument check before anything is launched.
"""
import ctypes
import os
import re

import pytest

import moe_expert_load_ultraep_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ultraep.h")

pytestmark = pytest.mark.skipif(not os.path.exists(U.LIB_PATH), reason="libultraep.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ultraep_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 15, names
    lib = ctypes.CDLL(U.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(U._SIGNATURES)


def test_status_strings():
    for code, text in U.STATUS.items():
        assert U.status_string(code) == text
    assert U.status_string(-99) == "unknown status"


@pytest.mark.parametrize("E,R,S,D,code", [
    (8, 3, 1, 1, -1),      # E % R
    (8, 4, 1, 3, -1),      # R % D
    (8, 4, -1, 4, -1),     # S < 0
    (0, 4, 1, 4, -1),
    (2048, 64, 1, 64, -2),  # E beyond limit
    (64, 2, 1, 2, -2),     # M = 32 beyond limit
    (64, 64, 9, 64, -2),   # S beyond limit
    (256, 128, 1, 128, -2),  # D beyond one wave
    (1024, 1024, 2, 64, -2),  # R*S beyond limit
])
def test_create_rejects(E, R, S, D, code):
    with pytest.raises(U.UltraEPError) as ei:
        U.ultraep_create(E, R, S, D)
    assert ei.value.status == code


@pytest.mark.parametrize("E,R,S,D", [(1024, 1024, 1, 64), (1024, 512, 2, 64), (1024, 64, 8, 64),
                                     (256, 64, 2, 64), (160, 40, 3, 8), (8, 4, 1, 4)])
def test_create_accepts_limits(E, R, S, D):
    U.ultraep_create(E, R, S, D).close()


def test_create_rejects_bad_options():
    with pytest.raises(U.UltraEPError):
        U.ultraep_create(8, 4, 1, 4, eps=(1, 0))
    for thr in ((1, 2), (65, 1), (1, 0), (-1, 1)):     # below 1, above 64, zero denominator
        with pytest.raises(U.UltraEPError):
            U.ultraep_create(8, 4, 1, 4, threshold=thr)
    U.ultraep_create(8, 4, 1, 4, threshold=(0, 0)).close()   # 0/0: the default 1
    U.ultraep_create(8, 4, 1, 4, threshold=(64, 1)).close()
    for mode in (0, 1, 2):
        U.ultraep_create(8, 4, 1, 4, reroute_mode=mode).close()
    for mode in (-1, 3):
        with pytest.raises(U.UltraEPError):
            U.ultraep_create(8, 4, 1, 4, reroute_mode=mode)
    U.ultraep_create(8, 4, 1, 4, replica_lean=True).close()
    with pytest.raises(U.UltraEPError):
        U.ultraep_create(8, 4, 1, 4, replica_lean=2)
    U.ultraep_create(8, 4, 1, 4, min_tokens=0).close()       # 0: the default 1
    U.ultraep_create(8, 4, 1, 4, min_tokens=1024).close()
    with pytest.raises(U.UltraEPError):
        U.ultraep_create(8, 4, 1, 4, min_tokens=-1)


def test_plan_layout_fields():
    ctx = U.ultraep_create(256, 64, 2, 64)
    E, R, S, P = 256, 64, 2, ctx.P
    want = {"header": 64, "counts": E, "master_quota": E, "slot_expert": R * S, "slot_quota": R * S,
            "phys_load": P, "phys_off": P + 1, "inst_ptr": E + 1, "inst_phys": E + R * S,
            "inst_end": E + R * S, "inst_base": E + R * S, "rank_before": R, "rank_after": R,
            "inst_local": E + R * S}
    end = 0
    for name in U.PLAN_FIELDS:
        off, cnt = ctx.fields[name]
        assert cnt == want[name] and off % 4 == 0 and off >= end
        end = off + cnt
    assert ctx.plan_bytes % 256 == 0 and end <= ctx.plan_words


def test_workspace_bytes():
    ctx = U.ultraep_create(128, 64, 2, 64)
    ntiles = -(-64 * 8192 * 8 // 8192)
    assert ctx.workspace_bytes(1, 8192, 8) == 2 * 4 * ntiles * 128
    assert ctx.workspace_bytes(3, 8192, 8) == 3 * 2 * 4 * ntiles * 128
    with pytest.raises(U.UltraEPError) as ei:
        ctx.workspace_bytes(1, 8192, 0)
    assert ei.value.status == -1
    with pytest.raises(U.UltraEPError) as ei:
        ctx.workspace_bytes(1, 1 << 30, 8)   # N >= 2^31
    assert ei.value.status == -2


FAKE = 1 << 20   # never dereferenced: every call below fails its host check


def test_balance_argument_checks():
    ctx = U.ultraep_create(8, 4, 1, 4)
    f = U.lib().ultraep_balance
    h, F = ctx.handle, FAKE

    def call(L=1, idx=F, w=None, T=16, k=2, ws=F, wsb=1 << 20, plans=F, phys=F, pos=F, inv=None, wp=None, ctxh=h):
        return f(ctxh, L, idx, w, T, k, ws, wsb, plans, phys, pos, inv, wp, None)

    assert call(L=-1) == -1
    assert call(k=0) == -1
    assert call(k=9) == -1                 # k > E
    assert call(T=-1) == -1
    assert call(idx=None) == -1
    assert call(w=F, inv=F) == -1          # layout outputs given only in part
    assert call(w=F) == -1
    assert call(idx=F + 2) == -2           # misaligned
    assert call(w=F, inv=F, wp=F + 1) == -2
    assert call(wsb=4) == -4               # workspace short
    assert call(T=1 << 28, k=8) == -2      # N >= 2^31
    assert call(ctxh=None) == -1
    assert call(L=0, idx=None, ws=None, plans=None, phys=None, pos=None) == 0   # L = 0: no-op


def test_balance_static_argument_checks():
    """The allocation-free balance checks everything, its size limit
    included, before it looks up its workspace or launches anything."""
    ctx = U.ultraep_create(128, 64, 2, 64)
    f = U.lib().ultraep_balance_static
    h, F = ctx.handle, FAKE

    def call(L=1, idx=F, w=None, T=8192, k=8, plans=F, phys=F, pos=F, inv=None, wp=None):
        return f(h, L, idx, w, T, k, plans, phys, pos, inv, wp, None)

    assert call(L=65) == -5                # 65 x 512 KiB: beyond the static workspace
    assert call(L=1 << 20, T=1) == -5
    assert call(L=-1) == -1
    assert call(k=0) == -1
    assert call(plans=None) == -1
    assert call(w=F) == -1                 # layout outputs given only in part
    assert call(idx=F + 2) == -2
    assert call(T=1 << 28) == -2           # N >= 2^31
    assert call(L=0, idx=None, plans=None, phys=None, pos=None) == 0
    assert U.status_string(-5) == "needs more than the static workspace"


def test_permute_and_fold_argument_checks():
    ctx = U.ultraep_create(8, 4, 1, 4)
    p = U.lib().ultraep_permute
    assert p(ctx.handle, FAKE, FAKE, 2, FAKE, 10, 12, 0, 3, FAKE, 10, None) == -2    # H % 8
    assert p(ctx.handle, FAKE, FAKE, 2, FAKE + 8, 10, 16, 0, 3, FAKE, 10, None) == -2  # hidden not 16-B aligned
    assert p(ctx.handle, FAKE, FAKE, 2, FAKE, 10, 16, 3, 2, FAKE, 10, None) == -1     # p_end < p_begin
    assert p(ctx.handle, FAKE, FAKE, 2, FAKE, 10, 16, 0, ctx.P + 1, FAKE, 10, None) == -1
    assert p(ctx.handle, FAKE, FAKE, 0, FAKE, 10, 16, 0, 3, FAKE, 10, None) == -1     # k = 0
    assert p(ctx.handle, None, FAKE, 2, FAKE, 10, 16, 0, 3, FAKE, 10, None) == -1
    g = U.lib().ultraep_fold_grads
    assert g(ctx.handle, FAKE, FAKE, FAKE, 16, 0, 5, None) == -1     # slot_end > R*S
    assert g(ctx.handle, FAKE, FAKE, FAKE, 16, 2, 1, None) == -1
    assert g(ctx.handle, FAKE, FAKE, FAKE, -1, 0, 1, None) == -1
    assert g(ctx.handle, FAKE, None, FAKE, 16, 0, 1, None) == -1
    assert g(ctx.handle, FAKE, FAKE + 4, FAKE, 16, 0, 1, None) == -2  # pointer table misaligned
    lay = U.lib().ultraep_dispatch_layout
    assert lay(ctx.handle, 1, 16, 2, None, FAKE, FAKE, FAKE, None) == -1
    assert lay(ctx.handle, 1, 16, 2, FAKE + 1, FAKE, FAKE, FAKE, None) == -2


def test_combine_argument_checks():
    ctx = U.ultraep_create(8, 4, 1, 4)
    c = U.lib().ultraep_combine
    F = FAKE
    h = ctx.handle
    #          ctx pos w  k  rows nrows H  g0 g1 out
    assert c(h, F, F, 2, F, 10, 12, 0, 3, F, None) == -2        # H % 8
    assert c(h, F, F, 2, F + 8, 10, 16, 0, 3, F, None) == -2    # rows not 16-B aligned
    assert c(h, F, F, 2, F, 10, 16, 0, 3, F + 8, None) == -2    # out not 16-B aligned
    assert c(h, F + 2, F, 2, F, 10, 16, 0, 3, F, None) == -2    # pos misaligned
    assert c(h, F, F, 2, F, 1 << 31, 16, 0, 3, F, None) == -2   # layout rows >= 2^31
    assert c(h, F, F, 0, F, 10, 16, 0, 3, F, None) == -1        # k = 0
    assert c(h, F, F, 9, F, 10, 16, 0, 3, F, None) == -1        # k > E
    assert c(h, F, F, 2, F, 10, 16, 3, 2, F, None) == -1        # empty range reversed
    assert c(h, F, F, 2, F, 10, -16, 0, 3, F, None) == -1
    assert c(h, None, F, 2, F, 10, 16, 0, 3, F, None) == -1
    assert c(h, F, F, 2, None, 10, 16, 0, 3, F, None) == -1     # rows NULL with rows > 0
    assert c(h, F, F, 2, F, 10, 16, 0, 3, None, None) == -1     # out NULL
    assert c(h, F, None, 2, F, 10, 16, 3, 3, None, None) == 0   # empty range, unweighted: no-op
    b = U.lib().ultraep_combine_backward
    #          ctx pos w  k  rows nrows H  dy g0 g1 grows gw
    assert b(h, F, None, 2, F, 10, 16, F, 0, 3, F, F, None) == -1   # weights required
    assert b(h, F, F, 2, F, 10, 16, None, 0, 3, F, F, None) == -1
    assert b(h, F, F, 2, F, 10, 16, F, 0, 3, None, F, None) == -1
    assert b(h, F, F, 2, F, 10, 16, F, 0, 3, F, None, None) == -1
    assert b(h, F, F, 2, F, 10, 16, F + 8, 0, 3, F, F, None) == -2  # grad_out misaligned
    assert b(h, F, F, 2, F, 10, 16, F, 0, 3, F + 8, F, None) == -2  # grad_rows misaligned
    assert b(h, F, F, 2, F, 10, 16, F, 0, 3, F, F + 2, None) == -2  # grad_topk_w misaligned
    assert b(h, F, F, 2, F, 10, 16, F, 4, 4, F, F, None) == 0       # empty range: no-op


def test_weight_sync_argument_checks():
    ctx = U.ultraep_create(8, 4, 1, 4)
    F = FAKE
    p = U.lib().ultraep_weight_sync_plan
    o = U._RelayOptions(1, 4, 8, 2, 4)
    assert p(ctx.handle, None, ctypes.byref(o), F, None) == -1
    assert p(ctx.handle, F, ctypes.byref(o), None, None) == -1
    assert p(ctx.handle, F, ctypes.byref(U._RelayOptions(3, 4, 8, 2, 4)), F, None) == -1   # mode
    assert p(ctx.handle, F, ctypes.byref(U._RelayOptions(1, -1, 8, 2, 4)), F, None) == -1
    bad = U._RelayOptions(1, 4, 8, 2, 4)
    bad.reserved[1] = 5
    assert p(ctx.handle, F, ctypes.byref(bad), F, None) == -1                             # reserved
    assert p(ctx.handle, F, ctypes.byref(o), F + 2, None) == -2                            # misaligned
    s = U.lib().ultraep_weight_sync
    #          ctx plan masters reps numel s0 s1 relay
    assert s(ctx.handle, F, F, F, 16, 0, 5, None, None) == -1       # slot_end > R*S
    assert s(ctx.handle, F, F, F, 16, 2, 1, None, None) == -1
    assert s(ctx.handle, F, F, F, -1, 0, 1, None, None) == -1
    assert s(ctx.handle, F, None, F, 16, 0, 1, None, None) == -1
    assert s(ctx.handle, F, F, None, 16, 0, 1, None, None) == -1
    assert s(ctx.handle, F, F, F, 16, 0, 2, F, None) == -1          # relay needs every slot
    assert s(ctx.handle, F, F + 4, F, 16, 0, 1, None, None) == -2   # pointer table misaligned
    assert s(ctx.handle, F, F, F + 1, 16, 0, 1, None, None) == -2   # odd element address
    assert s(ctx.handle, F, F, F, 0, 0, 4, None, None) == 0         # numel 0: no-op
