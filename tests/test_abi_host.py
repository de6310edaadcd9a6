"""Host-side checks of the C ABI: the library loads, exports what include/la.h
declares, and rejects bad arguments with the documented status codes before
touching the GPU (so these run on a machine without one)."""
import ctypes
import os
import re

import pytest

import chunkwise_recurrence_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
P16 = ctypes.c_void_p(1 << 20)        # 16-byte aligned fake device address (never dereferenced)
P8 = ctypes.c_void_p((1 << 20) + 8)   # misaligned


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:la_status|size_t|const char\*)\s+(la_\w+)\s*\(", text,
                                 re.M)))


def test_library_exports_every_declared_symbol():
    lib = la.load()
    names = _declared()
    assert set(names) == set(la.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(7):
        assert la.status_string(s).startswith("LA_")
    assert "unknown" in la.status_string(99)


def _fwd(**kw):
    a = dict(q=P16, k=P16, v=P16, dtype=1, B=1, H=1, L=64, dk=64, dv=64, C=64, phi=0, kind=0,
             decay=None, state=None, out=P16, ws=None, ws_bytes=0)
    a.update(kw)
    return la.load().la_chunk_fwd(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"],
                                  a["dk"], a["dv"], a["C"], a["phi"], a["kind"], a["decay"],
                                  a["state"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(out=None), NULL),
    (dict(kind=1, decay=None), NULL), (dict(kind=3, decay=None), NULL),
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(L=-5), SHAPE), (dict(C=0), SHAPE),
    (dict(dk=48), UNSUP), (dict(dv=256), UNSUP), (dict(dk=8), UNSUP), (dict(C=256), UNSUP),
    (dict(C=48), UNSUP), (dict(dtype=2), UNSUP), (dict(phi=2), UNSUP), (dict(kind=5), UNSUP),
    (dict(kind=-1), UNSUP), (dict(kind=4, decay=None), NULL),
    (dict(q=P8), ALIGN), (dict(out=P8), ALIGN), (dict(state=P8), ALIGN),
    (dict(kind=1, decay=ctypes.c_void_p((1 << 20) + 2)), ALIGN),
])
def test_chunk_fwd_rejects(kw, code):
    assert _fwd(**kw) == code


def test_zero_length_is_ok_without_touching_memory():
    assert _fwd(L=0, q=None, k=None, v=None, out=None) == OK


def test_workspace_is_required_when_the_plan_splits_the_sequence():
    # 1 head of 64 x 64 over 64K tokens: the plan splits the sequence
    kernel, tile, P, groups, _ = la.plan(1, 1, 65536, 64, 64, 64)
    assert P > 1
    need = la.chunk_fwd_workspace_bytes(1, 1, 65536, 64, 64, 64)
    assert need >= P * 64 * 64 * 4
    # the token decays add 4 bytes per head-token of prefix sums
    assert la.chunk_fwd_workspace_bytes(1, 1, 65536, 64, 64, 64, la.LA_BF16, 3) >= need + 65536 * 4
    assert _fwd(L=65536, kind=3, decay=P16, ws=P16, ws_bytes=need) == WS
    assert _fwd(L=65536, ws=None, ws_bytes=0) == WS
    # the smallest size the host check accepts (past it the call goes on to the
    # launch, which fails without a GPU): within the query, and one byte less is refused
    lo, hi = 0, need
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if _fwd(L=65536, ws=P16, ws_bytes=mid) == WS:
            lo = mid
        else:
            hi = mid
    assert _fwd(L=65536, ws=P16, ws_bytes=hi) != WS
    assert _fwd(L=65536, ws=P16, ws_bytes=hi - 1) == WS
    # per-segment increments plus the copy of S_0 the output pass reads (the
    # last segment's workgroup overwrites the caller's state with S_L)
    assert P * 64 * 64 * 4 + 64 * 64 * 4 <= hi <= need
    assert _fwd(L=65536, ws=P8, ws_bytes=need) == ALIGN


STRIP, STRIPE, F32 = la.KERNEL_STRIP, la.KERNEL_STRIPE, la.KERNEL_F32


def test_plans_of_the_workloads():
    # the stripe kernel: one workgroup per head (2 waves per 32 value columns)
    # and segment; segments bring the grid to 256 workgroups.  retnet: 64
    # heads x 4 segments
    assert la.plan(2, 32, 16384, 128, 128, 64)[:4] == (STRIPE, 128, 4, 2)
    # gated: 16 heads x 16 segments
    assert la.plan(1, 16, 65536, 128, 128, 64)[:4] == (STRIPE, 128, 16, 2)
    # narrower heads: the strip kernel.  64-wide value heads with d_k >= 64
    # take one 64-column tile in two groups; elu: 64 heads x 2 groups x 4
    # segments, the 512 4-wave units of 32-column tiles
    assert la.plan(4, 16, 4096, 64, 64, 64)[:4] == (STRIP, 64, 4, 2)
    # ... whose 192 state-pass workgroups (64 heads x 3 segments) are split in
    # two to cover the 256 compute units; the stripe kernel's are not split
    assert la.plan(4, 16, 4096, 64, 64, 64)[4] == 2
    assert la.plan(2, 32, 16384, 128, 128, 64)[4] == 1
    assert la.plan(2, 32, 8192, 128, 64, 64)[:4] == (STRIP, 64, 4, 2)
    # d_k = 32 keeps 32-column tiles in one group
    assert la.plan(2, 32, 8192, 32, 64, 64)[:4] == (STRIP, 32, 4, 1)
    assert la.plan(1, 1, 100, 16, 16, 16)[:4] == (STRIP, 16, 1, 1)
    # 16-token chunks, d_k = 16: the strip kernel
    assert la.plan(1, 1, 100, 128, 128, 16)[0] == STRIP
    assert la.plan(1, 1, 100, 16, 128, 64)[0] == STRIP
    # 128-token chunks at d_k = 128 exceed the stripe kernel's LDS
    assert la.plan(1, 1, 100, 128, 128, 128)[:4] == (STRIP, 32, 1, 1)
    assert la.plan(1, 1, 100, 64, 128, 128)[0] == STRIPE
    # fp32: its own kernel, one segment, 16- or 32-wide tiles
    assert la.plan(1, 1, 300, 16, 16, 64, la.LA_F32)[:4] == (F32, 16, 1, 1)
    assert la.chunk_fwd_workspace_bytes(1, 1, 300, 16, 16, 64, la.LA_F32) == 0
    # fp32 with two 32-column value tiles: the normalised form reads z_0 from
    # a copy (the first tile's workgroup writes z_L back), 256 bytes rounded
    assert la.chunk_fwd_workspace_bytes(1, 1, 300, 16, 64, 64, la.LA_F32) == 256
    assert la.chunk_fwd_workspace_bytes(2, 3, 300, 32, 64, 64, la.LA_F32) == 2 * 3 * 32 * 4


def test_plan_requests_and_clamping():
    def got(req, *shape):
        return la.plan(*shape, request=req)
    assert got((STRIP, 64, 3, 1), 1, 1, 64 * 30, 128, 128, 64)[:4] == (STRIP, 64, 3, 1)
    # tile clamped to d_v, P to chunks
    assert got((STRIP, 64, 3, 1), 1, 1, 64 * 2, 128, 32, 64)[:4] == (STRIP, 32, 2, 1)
    assert got((STRIP, 32, 0, 2), 1, 1, 64 * 30, 128, 128, 64)[1::2] == (32, 2)
    # 8-column groups do not exist
    assert got((STRIP, 16, 0, 2), 1, 1, 64 * 30, 128, 128, 64)[1::2] == (16, 1)
    assert got((STRIP, 64, 0, 2), 1, 1, 100, 64, 64, 64)[:4] == (STRIP, 64, 1, 2)
    # two 64-column groups of d_k = 128 exceed the LDS: the tile is halved
    assert got((STRIP, 64, 0, 2), 1, 1, 100, 128, 128, 64)[1::2] == (64, 2)
    assert got((STRIPE, 64, 2), 1, 1, 64 * 30, 128, 128, 64)[:4] == (STRIPE, 64, 2, 2)
    # d_k = 32 keeps one wave per stripe
    assert got((STRIPE,), 1, 1, 100, 32, 32, 64)[:4] == (STRIPE, 32, 1, 1)
    assert got((STRIPE,), 1, 1, 100, 64, 64, 128)[0] == STRIPE
    assert got((STRIPE, 128, 2, 1), 1, 1, 64 * 30, 128, 128, 64)[:4] == (STRIPE, 128, 2, 1)
    # a stripe request the shape does not allow falls back to the strip kernel
    assert got((STRIPE, 128, 2, 1), 1, 1, 64 * 30, 16, 16, 64)[0] == STRIP
    for bad, code in (((STRIP, 48, 0), UNSUP), ((STRIP, 0, -1), SHAPE), ((STRIP, 0, 0, 3), UNSUP),
                      ((7,), UNSUP)):
        with pytest.raises(la.LAError) as e:
            got(bad, 1, 1, 100, 64, 64, 64)
        assert e.value.status == code
    # state-pass splits: reduced to a divisor of the segment's chunk count (24
    # chunks in 3 segments of 8: 3 -> 2), and 1 without a state pass
    L24 = 64 * 23 + 17
    assert got((STRIP, 64, 3, 1, 3), 1, 1, L24, 128, 128, 64) == (STRIP, 64, 3, 1, 2)
    assert got((STRIP, 64, 3, 1, 100), 1, 1, L24, 128, 128, 64)[4] == 8
    assert got((STRIPE, 128, 1, 2, 4), 1, 1, L24, 128, 128, 64)[4] == 1
    # one increment (and one decay total) per state-pass unit in the workspace
    ws = {s: la.plan_workspace_bytes(1, 1, L24, 128, 128, 64, request=(STRIP, 64, 3, 1, s))
          for s in (1, 2, 4)}
    assert ws[2] - ws[1] >= 3 * 128 * 128 * 4 and ws[4] - ws[2] >= 6 * 128 * 128 * 4
    with pytest.raises(la.LAError) as e:
        got((STRIP, 0, 0, 0, -1), 1, 1, 100, 64, 64, 64)
    assert e.value.status == SHAPE
    with pytest.raises(ValueError):
        got((STRIP, 0, 0, 0, 0, 0), 1, 1, 100, 64, 64, 64)
    # the request is per call: the automatic plan is untouched
    assert la.plan(2, 32, 16384, 128, 128, 64)[:4] == (STRIPE, 128, 4, 2)
    # within a using_plan block the binding passes the block's request
    with la.using_plan(STRIP, 32, 2, 1):
        assert la.plan(2, 32, 16384, 128, 128, 64)[:4] == (STRIP, 32, 2, 1)
        # the workspace query follows the request: two segments' states + the S_0 copy
        ws = la.plan_workspace_bytes(2, 32, 16384, 128, 128, 64)
        assert ws >= 64 * 2 * 128 * 128 * 4 + 64 * 128 * 128 * 4
    assert la.plan(2, 32, 16384, 128, 128, 64)[:4] == (STRIPE, 128, 4, 2)


def test_plan_query_rejects():
    lib = la.load()
    p = la.Plan()
    assert lib.la_chunk_fwd_plan(1, 1, 64, 64, 64, 64, 1, 0, 0, None, None) == NULL
    assert lib.la_chunk_fwd_plan(0, 1, 64, 64, 64, 64, 1, 0, 0, ctypes.byref(p), None) == SHAPE
    assert lib.la_chunk_fwd_plan(1, 1, 64, 48, 64, 64, 1, 0, 0, ctypes.byref(p), None) == UNSUP
    assert lib.la_chunk_fwd_plan(1, 1, 64, 64, 64, 64, 1, 9, 0, ctypes.byref(p), None) == UNSUP
    ws = ctypes.c_size_t(7)
    assert lib.la_chunk_fwd_plan(1, 1, 64, 64, 64, 64, 1, 0, 0, ctypes.byref(p),
                                 ctypes.byref(ws)) == OK
    assert ws.value == 0 and p.segments == 1


def _planned(req, **kw):
    a = dict(q=P16, k=P16, v=P16, dtype=1, B=1, H=1, L=64 * 30, dk=128, dv=128, C=64, phi=0,
             kind=0, decay=None, state=None, z=None, norm=0, out=P16, ws=None, ws_bytes=0)
    a.update(kw)
    return la.load().la_chunk_fwd_planned(
        a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"], a["dk"], a["dv"], a["C"],
        a["phi"], a["kind"], a["decay"], a["state"], a["z"], a["norm"],
        None if req is None else ctypes.byref(req), a["out"], a["ws"], a["ws_bytes"], None)


def test_planned_forward_rejects():
    assert _planned(la.Plan(7, 0, 0, 0)) == UNSUP
    assert _planned(la.Plan(STRIP, 24, 0, 0)) == UNSUP
    assert _planned(la.Plan(STRIP, 0, -2, 0)) == SHAPE
    assert _planned(la.Plan(STRIP, 0, 0, 5)) == UNSUP
    # a request that splits the sequence needs its workspace
    assert _planned(la.Plan(STRIPE, 128, 3, 2)) == WS
    assert _planned(la.Plan(STRIPE, 128, 3, 2), q=None) == NULL
    assert _planned(None, L=0, q=None, k=None, v=None, out=None) == OK


def _dec(**kw):
    a = dict(q=P16, k=P16, v=P16, dtype=1, N=2, H=2, dk=128, dv=128, phi=0, kind=0, decay=None,
             state=P16, out=P16)
    a.update(kw)
    return la.load().la_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["N"], a["H"], a["dk"],
                                    a["dv"], a["phi"], a["kind"], a["decay"], a["state"],
                                    a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), NULL), (dict(out=None), NULL), (dict(q=None), NULL),
    (dict(kind=2, decay=None), NULL), (dict(N=0), SHAPE), (dict(H=0), SHAPE),
    (dict(dk=100), UNSUP), (dict(dtype=7), UNSUP), (dict(phi=5), UNSUP), (dict(kind=9), UNSUP),
    (dict(state=P8), ALIGN), (dict(v=P8), ALIGN),
])
def test_decode_step_rejects(kw, code):
    assert _dec(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, 1, 1, 64, 64), NULL), ((P16, 0, 1, 64, 64), SHAPE), ((P16, 1, 1, 64, 20), UNSUP),
    ((P8, 1, 1, 64, 64), ALIGN),
])
def test_state_init_rejects(args, code):
    assert la.load().la_state_init(*args, None) == code


def _fwd_norm(**kw):
    a = dict(q=P16, k=P16, v=P16, dtype=1, B=1, H=1, L=64, dk=64, dv=64, C=64, phi=1, kind=0,
             decay=None, state=None, z=None, out=P16, ws=None, ws_bytes=0)
    a.update(kw)
    return la.load().la_chunk_fwd_norm(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"],
                                       a["dk"], a["dv"], a["C"], a["phi"], a["kind"], a["decay"],
                                       a["state"], a["z"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(B=0), SHAPE), (dict(dk=48), UNSUP),
    # bf16 normalised form: the stripe kernel's shapes only
    (dict(dk=16, dv=16), UNSUP), (dict(dv=16), UNSUP), (dict(C=16), UNSUP),
    (dict(z=P8), ALIGN), (dict(state=P8), ALIGN),
])
def test_chunk_fwd_norm_rejects(kw, code):
    assert _fwd_norm(**kw) == code


def test_chunk_fwd_norm_fp32_takes_every_shape():
    # the fp32 kernel has no shape limits beyond the common ones; L = 0 returns before any launch
    assert _fwd_norm(dtype=0, dk=16, dv=16, C=16, L=0) == OK


def test_decode_norm_requires_its_state():
    lib = la.load()
    assert lib.la_decode_step_norm(P16, P16, P16, 1, 2, 2, 64, 64, 1, 0, None, P16, None, P16,
                                   None) == NULL
    assert lib.la_decode_step_norm(P16, P16, P16, 1, 2, 2, 64, 64, 1, 0, None, P16, P8, P16,
                                   None) == ALIGN


# bf16 per-channel decay: the stripe kernel's layouts whose log-decay
# prefetch stays within 16 tokens per thread and whose tiles fit the LDS
@pytest.mark.parametrize("dk,dv,C", [(128, 128, 128), (64, 64, 128), (128, 32, 64), (32, 32, 128),
                                     (16, 16, 32), (64, 16, 64), (32, 32, 16)])
def test_channel_decay_bf16_unsupported_shapes(dk, dv, C):
    assert _fwd(kind=4, decay=P16, dk=dk, dv=dv, C=C) == UNSUP
    # fp32 inputs take them (the call then fails only on the NULL q)
    assert _fwd(kind=4, decay=P16, dk=dk, dv=dv, C=C, dtype=0, q=None) == NULL


@pytest.mark.parametrize("dk,dv,C", [(128, 128, 64), (128, 128, 32), (64, 64, 64), (32, 128, 128),
                                     (128, 32, 32), (64, 32, 64)])
def test_channel_decay_bf16_supported_shapes(dk, dv, C):
    assert _fwd(kind=4, decay=P16, dk=dk, dv=dv, C=C, q=None) == NULL


def test_channel_decay_bf16_has_no_normalised_form():
    assert _fwd_norm(kind=4, decay=P16, dk=128, dv=128) == UNSUP
    assert _fwd_norm(kind=4, decay=P16, dtype=0, q=None) == NULL


def test_channel_decay_workspace_holds_per_channel_totals():
    # a split sequence keeps one log-decay total per segment, or d_k of them
    # for the per-channel decay (both plans: stripe kernel, same segments)
    B, H, L, d = 1, 1, 65536, 128
    kernel, tile, P, groups, _ = la.plan(B, H, L, d, d, 64)
    assert kernel == la.KERNEL_STRIPE and P > 1
    head = la.chunk_fwd_workspace_bytes(B, H, L, d, d, 64, la.LA_BF16, la.DECAY_HEAD)
    ch = la.chunk_fwd_workspace_bytes(B, H, L, d, d, 64, la.LA_BF16, la.DECAY_CHANNEL)
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # plus one flag per output-pass workgroup (groups of 8 units) for the exact re-run
    flags = r256((P + 7) // 8 * 8 * 4)
    assert ch - head == r256(P * d * 4) - r256(P * 4) + flags


def _delta(**kw):
    a = dict(q=P16, k=P16, v=P16, beta=P16, dtype=1, B=1, H=1, L=64, dk=64, dv=64, C=64, kind=0,
             decay=None, state=None, out=P16, ws=P16, ws_bytes=1 << 30)
    a.update(kw)
    return la.load().la_delta_fwd(a["q"], a["k"], a["v"], a["beta"], a["dtype"], a["B"], a["H"],
                                  a["L"], a["dk"], a["dv"], a["C"], a["kind"], a["decay"],
                                  a["state"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(beta=None), NULL), (dict(out=None), NULL),
    (dict(kind=3, decay=None), NULL), (dict(B=0), SHAPE), (dict(L=-1), SHAPE),
    (dict(C=128), UNSUP), (dict(C=48), UNSUP), (dict(dk=48), UNSUP), (dict(kind=4, decay=P16), UNSUP),
    (dict(dtype=2), UNSUP), (dict(q=P8), ALIGN), (dict(beta=ctypes.c_void_p((1 << 20) + 2)), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS), (dict(ws=P8), ALIGN),
])
def test_delta_fwd_rejects(kw, code):
    assert _delta(**kw) == code


def test_delta_zero_length_and_workspace_size():
    assert _delta(L=0, q=None, k=None, v=None, beta=None, out=None, ws=None) == OK
    B, H, L, dk, dv = 2, 3, 100, 32, 64
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # W and U0, bf16 on the matrix-core path (bf16, 64-token chunks) with the
    # chunks' bf16 score rows and the fp32 in-chunk decay prefix, else fp32
    assert la.delta_fwd_workspace_bytes(B, H, L, dk, dv, 64, la.LA_BF16) == \
        r256(B * H * L * dk * 2) + r256(B * H * L * dv * 2) + r256(B * H * L * 64 * 2) + \
        r256(B * H * L * 4)
    assert la.delta_fwd_workspace_bytes(B, H, L, dk, dv, 32, la.LA_BF16) == \
        r256(B * H * L * dk * 4) + r256(B * H * L * dv * 4)
    assert la.delta_fwd_workspace_bytes(B, H, L, dk, dv, 64, la.LA_F32) == \
        r256(B * H * L * dk * 4) + r256(B * H * L * dv * 4)
    assert la.delta_fwd_workspace_bytes(B, H, L, dk, dv, 128, la.LA_BF16) == 0


def test_delta_decode_rejects():
    lib = la.load()
    call = lambda **kw: lib.la_delta_decode_step(  # noqa: E731
        kw.get("q", P16), P16, P16, kw.get("beta", P16), 1, 2, 2, 64, 64, kw.get("kind", 0),
        kw.get("decay", None), kw.get("state", P16), P16, None)
    assert call(beta=None) == NULL
    assert call(state=None) == NULL
    assert call(kind=4, decay=P16) == UNSUP
    assert call(q=P8) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        la.chunk_fwd(x, x, x)


# The C ABI sees pointers only, so the binding checks every tensor's shape and
# dtype before the call.  These run on CPU tensors: the shape checks come
# before the device check, so each case raises for the reason it names.
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _f(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


@pytest.mark.parametrize("kw,match", [
    (dict(k=("b", 2, 3, 64, 16)), "share a shape"),
    (dict(v=("b", 2, 3, 32, 32)), "last dim"),
    (dict(k=("f", 2, 3, 64, 32)), "share a dtype"),
    (dict(state=("f", 2, 3, 32, 16)), "state"),
    (dict(state=("b", 2, 3, 32, 32)), "state"),
    (dict(out=("b", 2, 3, 64, 16)), "out"),
    (dict(out=("f", 2, 3, 64, 32)), "out"),
    (dict(decay_kind=1, decay=("f", 2)), "decay"),
    (dict(decay_kind=1), "decay"),
    (dict(decay_kind=3, decay=("f", 2, 3, 63)), "decay"),
    (dict(decay_kind=2, decay=("f", 2, 3, 64, 32)), "decay"),
    (dict(decay_kind=4, decay=("f", 2, 3, 64)), "decay"),
    (dict(decay_kind=4, decay=("b", 2, 3, 64, 32)), "decay"),
    (dict(decay_kind=6, decay=("f", 3)), "decay kind"),
    (dict(normalize=True, norm_state=("f", 2, 3, 16)), "norm_state"),
    (dict(norm_state=("f", 2, 3, 32)), "normalize"),
    (dict(workspace=("u", 3)), "workspace"),
])
def test_binding_chunk_fwd_checks_shapes(kw, match):
    import torch
    args = dict(q=("b", 2, 3, 64, 32), k=("b", 2, 3, 64, 32), v=("b", 2, 3, 64, 32))
    args.update(kw)
    mk = {"b": lambda *s: _t(*s), "f": _f, "u": lambda *s: _t(*s, dtype=torch.uint8)}
    call = {n: (mk[x[0]](*x[1:]) if isinstance(x, tuple) else x) for n, x in args.items()}
    if kw.get("workspace"):
        # a workspace that is too small for a split sequence
        call.update(q=_t(1, 1, 65536, 64), k=_t(1, 1, 65536, 64), v=_t(1, 1, 65536, 64))
    with pytest.raises(ValueError, match=match):
        la.chunk_fwd(**call)


@pytest.mark.parametrize("kw,match", [
    (dict(k=("b", 4, 2, 32)), "share a shape"),
    (dict(v=("f", 4, 2, 16)), "share a dtype"),
    (dict(state=("f", 4, 2, 16, 32)), "state"),
    (dict(state=("b", 4, 2, 16, 16)), "state"),
    (dict(state=None), "state"),
    (dict(out=("b", 4, 2, 32)), "out"),
    (dict(decay_kind=1, decay=("f", 4)), "decay"),
    (dict(decay_kind=3, decay=("f", 4)), "decay"),
    (dict(decay_kind=3), "decay"),
    (dict(decay_kind=4, decay=("f", 4, 2)), "decay"),
    (dict(norm_state=("f", 4, 2, 32)), "norm_state"),
])
def test_binding_decode_step_checks_shapes(kw, match):
    args = dict(q=("b", 4, 2, 16), k=("b", 4, 2, 16), v=("b", 4, 2, 16),
                state=("f", 4, 2, 16, 16))
    args.update(kw)
    mk = {"b": lambda *s: _t(*s), "f": _f}
    call = {n: (mk[x[0]](*x[1:]) if isinstance(x, tuple) else x) for n, x in args.items()}
    with pytest.raises(ValueError, match=match):
        la.decode_step(**call)


@pytest.mark.parametrize("kw,match", [
    (dict(beta=("f", 2, 3, 63)), "beta"),
    (dict(beta=("b", 2, 3, 64)), "beta"),
    (dict(state=("f", 2, 3, 16, 32)), "state"),
    (dict(out=("f", 2, 3, 64, 16)), "out"),
    (dict(decay_kind=4, decay=("f", 2, 3, 64, 16)), "decay kind"),
    (dict(decay_kind=3, decay=("f", 2, 3)), "decay"),
])
def test_binding_delta_fwd_checks_shapes(kw, match):
    args = dict(q=("b", 2, 3, 64, 16), k=("b", 2, 3, 64, 16), v=("b", 2, 3, 64, 16),
                beta=("f", 2, 3, 64))
    args.update(kw)
    mk = {"b": lambda *s: _t(*s), "f": _f}
    call = {n: (mk[x[0]](*x[1:]) if isinstance(x, tuple) else x) for n, x in args.items()}
    with pytest.raises(ValueError, match=match):
        la.delta_fwd(**call)


@pytest.mark.parametrize("kw,match", [
    (dict(beta=("f", 4)), "beta"),
    (dict(state=("f", 4, 2, 16, 32)), "state"),
    (dict(state=("b", 4, 2, 16, 16)), "state"),
    (dict(out=("b", 4, 2, 8)), "out"),
    (dict(decay_kind=2, decay=("f", 2)), "decay"),
    (dict(decay_kind=4, decay=("f", 4, 2, 16)), "decay kind"),
])
def test_binding_delta_decode_checks_shapes(kw, match):
    args = dict(q=("b", 4, 2, 16), k=("b", 4, 2, 16), v=("b", 4, 2, 16), beta=("f", 4, 2),
                state=("f", 4, 2, 16, 16))
    args.update(kw)
    mk = {"b": lambda *s: _t(*s), "f": _f}
    call = {n: (mk[x[0]](*x[1:]) if isinstance(x, tuple) else x) for n, x in args.items()}
    with pytest.raises(ValueError, match=match):
        la.delta_decode_step(**call)


def test_binding_well_formed_cpu_call_reaches_the_device_check():
    # every shape right: the only complaint left is that the tensors are not on a GPU
    with pytest.raises(ValueError, match="GPU tensor"):
        la.decode_step(_t(4, 2, 16), _t(4, 2, 16), _t(4, 2, 16), _f(4, 2, 16, 16),
                       decay_kind=la.DECAY_CHANNEL, decay=_f(4, 2, 16), out=_t(4, 2, 16))
    with pytest.raises(ValueError, match="GPU tensor"):
        la.chunk_fwd(_t(2, 3, 64, 32), _t(2, 3, 64, 32), _t(2, 3, 64, 32),
                     decay_kind=la.DECAY_CHANNEL, decay=_f(2, 3, 64, 32),
                     state=_f(2, 3, 32, 32), out=_t(2, 3, 64, 32))


def test_noalloc_host_checks():
    # la_chunk_fwd_noalloc validates like la_chunk_fwd, and refuses a workspace beyond its
    # fixed scratch before touching the device
    lib = la.load()
    call = lambda **kw: lib.la_chunk_fwd_noalloc(  # noqa: E731
        kw.get("q", P16), P16, P16, 1, 1, 1, kw.get("L", 64), 64, 64, 64, 0, kw.get("kind", 0),
        kw.get("decay", None), None, kw.get("out", P16), None)
    assert call(L=0, q=None, out=None) == OK
    assert call(q=None) == NULL
    assert call(out=P8) == ALIGN
    assert call(kind=3) == NULL
    assert call(kind=7, decay=P16) == UNSUP
    # a 16M-token gated head: segment states plus 64 MiB of prefix sums
    assert la.chunk_fwd_workspace_bytes(1, 1, 1 << 24, 64, 64, 64, la.LA_BF16, 3) > \
        la.NOALLOC_SCRATCH_BYTES
    assert call(L=1 << 24, kind=3, decay=P16) == WS
