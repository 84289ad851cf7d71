"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

The library must load, export every function include/taylor_attn.h declares,
size states and workspaces by the closed forms of the paper ("A Taylor-Series
Route to Linear-Time Transformers with a Fixed Number of Recurrent States",
sections 3.4, 4 and 5.8), and reject bad arguments before any HIP call.
"""
import ctypes
import json
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "taylor_attn.h")
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")))


@pytest.fixture(scope="module")
def rsp():
    if not os.path.exists(os.path.join(ROOT, "recurrent_state_phi_amd", "libtaylor_attn.so")):
        import __graft_entry__
        __graft_entry__.build()
    import recurrent_state_phi_amd as rsp
    return rsp


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(taylor_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("taylor_state_init", "taylor_attn_prefill", "taylor_attn_decode"):
        assert want in names


def test_library_exports_every_declared_symbol(rsp):
    lib = ctypes.CDLL(rsp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(rsp.EXPORTED_SYMBOLS)


def test_state_width_closed_form(rsp):
    printed = GOLDEN["symmetric_widths_d16"]["value"]
    for n in range(1, 7):
        assert rsp.state_width(16, n) == sum(printed[:n])
    for d in (1, 2, 6, 64):
        for n in range(1, 6):
            assert rsp.state_width(d, n) == sum(math.comb(d + m - 1, m) for m in range(n))
    assert rsp.state_numel(16, 64, 3) == GOLDEN["state_elements_per_head_n3"]["value"]
    # section 5.8: six terms at d = 16 / d = 64 with bfloat16 elements
    g = GOLDEN["state_size_bf16_MB"]
    assert round(rsp.state_numel(16, 64, 6) * 2 / 2 ** 20, 1) == g["d16_n6"]
    assert round(rsp.state_numel(64, 64, 6) * 2 / 2 ** 30, 1) == g["d64_n6_per_head"]
    assert rsp.state_width(0, 3) == -1 and rsp.state_width(16, 0) == -1


def test_workspace_sizing_n4(rsp):
    """n = 4: segment sums of 969 x 65 floats per segment (rounded up to 4 floats) plus 6 blocks
    of partial outputs, 68 floats per head-token (64 values, the normaliser, 16-byte padding)."""
    BH, N = 2 * 8, 4096
    ws = rsp.prefill_workspace_bytes(2, 8, N, 4, 32)
    out = 6 * BH * N * 68 * 4
    sums = ws - out
    nseg = round(sums / (BH * 969 * 65 * 4))
    assert nseg >= 1 and sums == -(-BH * nseg * 969 * 65 // 4) * 4 * 4
    assert rsp.prefill_workspace_bytes(1, 1, 10, 4, 32) == 6 * 10 * 68 * 4  # one segment: outputs only


@pytest.mark.parametrize("n,D,blocks", [(5, 4845, 28), (6, 20349, 116)])
def test_workspace_sizing_high_orders(rsp, n, D, blocks):
    """n = 5, 6: D rows split into 176-row feature blocks (28, 116); segment sums of D x 65
    floats per segment plus one block of 65 floats per head-token per feature block."""
    BH, N = 2, 333
    ws = rsp.prefill_workspace_bytes(1, 2, N, n, 32)
    out = blocks * BH * N * 68 * 4
    nseg = (ws - out) // (BH * D * 65 * 4)
    assert ws == out + -(-nseg * BH * D * 65 // 4) * 16 and nseg > 1
    assert BH * nseg * blocks <= 512  # at most one round of workgroups
    assert rsp.prefill_workspace_bytes(64, 8, 100, n, 64) == blocks * 512 * 100 * 68 * 4  # one segment


@pytest.mark.parametrize("d,n,D,blocks", [(32, 3, 561, 4), (64, 3, 2145, 13), (64, 2, 65, 1), (32, 1, 1, 1)])
def test_workspace_sizing_wide_heads(rsp, d, n, D, blocks):
    """d = 32, 64 (n <= 3) run feature-blocked: segment sums of D x 65 floats per segment plus,
    when the state spans several 176-row feature blocks, one block of 65 floats per
    head-token per block (a single block writes the outputs directly)."""
    assert rsp.state_width(d, n) == D
    BH, N = 2, 333
    ws = rsp.prefill_workspace_bytes(1, 2, N, n, 32, d=d)
    out = blocks * BH * N * 68 * 4 if blocks > 1 else 0
    nseg = (ws - out) // (BH * D * 65 * 4)
    sums = nseg * BH * D * 65 * 4
    assert ws == out + (-(-sums // 16) * 16 if blocks > 1 else sums) and nseg >= 1
    assert BH * max(nseg, 1) * blocks <= 512


def test_workspace_sizing(rsp):
    # one segment per head when the heads alone fill the GPU: no workspace
    assert rsp.prefill_workspace_bytes(64, 8, 4096, 3, 64) == 0
    assert rsp.prefill_workspace_bytes(1, 1, 0, 3, 64) == 0
    # n = 1, 2 (single-launch kernel, segments of 128 (n = 1) or 256 (n = 2)
    # tokens whatever the chunk): a header of 64 words, one flag word per segment
    # (rounded up to 64 words), then two images per segment (its sum and its
    # inclusive prefix) of 1,108 (n = 2) or 68 floats
    for n, img, seg in ((2, 1108, 256), (1, 68, 128)):
        slots = 4 * 8 * (8192 // seg)
        for chunk in (32, 64):
            assert rsp.prefill_workspace_bytes(4, 8, 8192, n, chunk) == 4 * (64 + -(-slots // 64) * 64 + slots * 2 * img)
    assert rsp.prefill_workspace_bytes(4, 8, 256, 2, 64) == 0  # one segment per head
    assert rsp.prefill_workspace_bytes(4, 8, 128, 1, 64) == 0
    assert rsp.prefill_workspace_bytes(1, 1, 257, 2, 64) == 4 * (64 + 64 + 2 * 2 * 1108)
    assert rsp.prefill_workspace_bytes(1, 1, 129, 1, 32) == 4 * (64 + 64 + 2 * 2 * 68)
    assert rsp.prefill_workspace_bytes(1, 1, 257, 1, 32) == 4 * (64 + 64 + 3 * 2 * 68)
    # n = 3 (single-launch kernel): a header of 64 words plus one 64-word flag
    # slot per segment, then one state image of 10624 floats per segment
    nseg = 512 // 32
    hdr = 64 + 32 * nseg * 64
    assert rsp.prefill_workspace_bytes(4, 8, 8192, 3, 64) == 4 * (hdr + 32 * nseg * 10624)
    # which also covers the generic kernel's need (float32 inputs)
    assert 4 * (hdr + 32 * nseg * 10624) >= 32 * nseg * 153 * 65 * 4


def _prefill_rc(lib, **kw):
    args = dict(q=None, k=None, v=None, o=None, state=None, B=1, H=1, N=64, d=16, d_v=64, n=3, a=1.0,
                chunk=64, ind=0, outd=0, ws=None, wsb=0, stream=None)
    args.update(kw)
    return lib.taylor_attn_prefill(*args.values())


def test_invalid_arguments_are_rejected_before_launch(rsp):
    lib = rsp.raw_library()
    assert _prefill_rc(lib) == -1                       # NULL pointers
    assert b"NULL" in lib.taylor_last_error()
    assert _prefill_rc(lib, d=24) == -2                 # shape not built
    assert _prefill_rc(lib, d_v=128) == -2
    assert _prefill_rc(lib, n=7) == -2                  # orders up to 5 (n <= 6) are built
    assert _prefill_rc(lib, d=32, n=4) == -2            # d = 32, 64: n <= 3
    assert _prefill_rc(lib, d=64, chunk=128, ind=1) == -2
    assert _prefill_rc(lib, d=48) == -2
    assert _prefill_rc(lib, d=64, n=3) == -1            # built: fails on the NULL pointers instead
    assert _prefill_rc(lib, n=0) == -2
    assert _prefill_rc(lib, n=4, chunk=128, ind=1) == -2   # n = 4..6: chunk 32 or 64
    assert _prefill_rc(lib, n=6, chunk=128, ind=1) == -2
    assert _prefill_rc(lib, n=5) == -1                  # built: fails on the NULL pointers instead
    assert _prefill_rc(lib, chunk=48) == -2
    assert _prefill_rc(lib, chunk=128, ind=0) == -2     # float32 path stops at chunk 64
    assert _prefill_rc(lib, a=0.0) == -1
    assert _prefill_rc(lib, a=float("nan")) == -1
    assert _prefill_rc(lib, N=-1) == -1
    assert _prefill_rc(lib, ind=7) == -1
    assert _prefill_rc(lib, N=0) == 0                   # empty sequence: nothing to do
    assert _prefill_rc(lib, B=0) == 0
    # misaligned pointer (never dereferenced: rejected first)
    assert _prefill_rc(lib, q=16, k=16, v=16, o=16, state=8) == -1
    assert b"aligned" in lib.taylor_last_error()
    # workspace too small for a multi-segment plan
    assert _prefill_rc(lib, B=1, H=1, N=4096, q=16, k=16, v=16, o=16, state=16) == -1
    assert b"workspace" in lib.taylor_last_error()
    # n <= 2: at most 2^23 - 1 segment workgroups, segments of 128 (n = 1) or
    # 256 (n = 2) tokens
    big = dict(B=1 << 12, H=1 << 4, N=128 * 128, q=16, k=16, v=16, o=16, state=16)
    assert _prefill_rc(lib, n=1, **big) == -1
    assert b"out of range" in lib.taylor_last_error() and b"N/128" in lib.taylor_last_error()
    assert _prefill_rc(lib, n=2, **big) == -1  # half as many segments: stops at the workspace
    assert b"workspace" in lib.taylor_last_error()
    dec = lib.taylor_attn_decode
    assert dec(None, None, None, None, None, 1, 1, 16, 64, 3, 1.0, 0, 0, None) == -1
    assert dec(None, None, None, None, None, 1, 1, 16, 64, 9, 1.0, 0, 0, None) == -2
    assert dec(None, None, None, None, None, 1, 1, 16, 64, 7, 1.0, 0, 0, None) == -2
    assert dec(None, None, None, None, None, 1, 1, 16, 64, 6, 1.0, 0, 0, None) == -1
    assert dec(None, None, None, None, None, 0, 4, 16, 64, 3, 1.0, 0, 0, None) == 0
    assert lib.taylor_state_init(None, 1, 1, 16, 64, 3, None) == -1
    assert lib.taylor_state_init(None, 0, 1, 16, 64, 3, None) == 0
    assert lib.taylor_set_phase_events(None, 4) == -1
    assert lib.taylor_set_phase_events(None, 0) == 0


def test_wait_limit_hook_and_check_without_workspace(rsp):
    """taylor_set_wait_limit returns the previous limit and rejects negative values;
    taylor_prefill_check has nothing to check without a workspace (no device work)."""
    lib = rsp.raw_library()
    prev = lib.taylor_set_wait_limit(5)
    try:
        assert prev == 1 << 20
        assert lib.taylor_set_wait_limit(7) == 5
        assert lib.taylor_set_wait_limit(-1) == -1
        assert b"polls" in lib.taylor_last_error()
        assert lib.taylor_set_wait_limit(7) == 7  # unchanged by the rejected call
    finally:
        lib.taylor_set_wait_limit(prev)
    assert lib.taylor_prefill_check(None, 0, None) == 0
    assert lib.taylor_prefill_check(None, 1 << 20, None) == 0


def test_state_views_follow_the_header_layout(rsp):
    """The header's state layout: first S[b][h][D][d_v] (value index fastest), then
    T[b][h][D], one flat float32 buffer; state_views must address exactly that."""
    import torch
    for (B, H, d, n) in [(2, 3, 16, 3), (1, 2, 16, 1), (2, 1, 32, 2), (1, 1, 16, 5)]:
        D, dv = rsp.state_width(d, n), 64
        st = torch.arange(B * H * rsp.state_numel(d, dv, n), dtype=torch.float64).float()
        S, T = rsp.state_views(st, B, H, n, d=d, d_v=dv)
        assert tuple(S.shape) == (B, H, D, dv) and tuple(T.shape) == (B, H, D)
        b, h, r, c = B - 1, H - 1, D - 1, 37
        assert int(S[b, h, r, c]) == ((b * H + h) * D + r) * dv + c
        assert int(T[b, h, r]) == B * H * D * dv + (b * H + h) * D + r
        assert int(S[0, 0, 0, 0]) == 0 and int(T[0, 0, 0]) == B * H * D * dv
        assert S.data_ptr() == st.data_ptr() and T.is_contiguous() and S.is_contiguous()


def test_softmax_entry_points_validate_before_launch(rsp):
    """The exact-softmax baseline's entry points: shapes other than d = 16, d_v = 64 are
    not built, bad sizes and pointers are rejected, empty calls do nothing, and the
    decode workspace is one 68-float partial per head per 2048-key range."""
    lib = rsp.raw_library()
    pre = lib.taylor_softmax_prefill
    assert pre(None, None, None, None, 1, 1, 10, 16, 64, 1.0, 1, 0, None) == -1     # NULL
    assert pre(None, None, None, None, 1, 1, 10, 32, 64, 1.0, 1, 0, None) == -2     # d not built
    assert pre(None, None, None, None, 1, 1, 10, 16, 32, 1.0, 1, 0, None) == -2
    assert pre(None, None, None, None, 1, 1, 10, 16, 64, 0.0, 1, 0, None) == -1     # a <= 0
    assert pre(None, None, None, None, 1, 1, -1, 16, 64, 1.0, 1, 0, None) == -1
    assert pre(None, None, None, None, 1, 1, 0, 16, 64, 1.0, 1, 0, None) == 0       # empty
    assert pre(16, 16, 16, 8, 1, 1, 10, 16, 64, 1.0, 1, 0, None) == -1              # misaligned
    assert b"aligned" in lib.taylor_last_error()
    ws = rsp.softmax_decode_workspace_bytes
    assert ws(64, 8, 65792) == 64 * 8 * 33 * 68 * 4
    assert ws(1, 1, 2048) == 68 * 4 and ws(1, 1, 2049) == 2 * 68 * 4
    dec = lib.taylor_softmax_decode
    args = lambda pos, cap, wsb=1 << 20, d=16: (16, 16, 16, 16, 16, 16, 2, 2, pos, cap, d, 64, 1.0, 1, 0, 16, wsb, None)
    assert dec(*args(5, 5)) == -1                        # pos must be < cap
    assert dec(*args(-1, 5)) == -1
    assert dec(*args(1, 4, d=64)) == -2
    assert dec(*args(3000, 4000, wsb=2 * 2 * 68 * 4)) == -1   # two ranges need twice that
    assert b"workspace" in lib.taylor_last_error()
    assert dec(None, None, None, None, None, None, 0, 2, 0, 4, 16, 64, 1.0, 1, 0, None, 0, None) == 0


def test_noalloc_prefill_rejects_before_any_device_work(rsp):
    """taylor_attn_prefill_noalloc: argument errors as taylor_attn_prefill reports them,
    and a plan whose workspace exceeds the fixed 32 MiB scratch (n = 4 at this size
    needs about 121 MiB) is refused with the size in the message; nothing launches."""
    lib = rsp.raw_library()
    f = lib.taylor_attn_prefill_noalloc
    assert f(None, None, None, None, None, 1, 1, 10, 16, 64, 3, 1.0, 64, 1, 0, None) == -1      # NULL
    assert f(None, None, None, None, None, 1, 1, 10, 24, 64, 3, 1.0, 64, 1, 0, None) == -2      # shape
    assert f(None, None, None, None, None, 1, 1, 10, 16, 64, 3, 1.0, 48, 1, 0, None) == -2      # chunk
    assert f(16, 16, 16, 16, 16, 1, 1, 10, 16, 64, 3, 0.0, 64, 1, 0, None) == -1               # a
    assert f(None, None, None, None, None, 0, 1, 10, 16, 64, 3, 1.0, 64, 1, 0, None) == 0       # empty
    assert f(16, 16, 16, 16, 16, 2, 8, 4096, 16, 64, 4, 1.0, 32, 0, 0, None) == -1
    msg = lib.taylor_last_error()
    assert b"33554432" in msg and b"workspace" in msg
