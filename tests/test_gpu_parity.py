"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (max over rows of ||o_t - o_t^oracle||_inf / ||o_t^oracle||_inf):
1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with float32 accumulation.
Inputs come from taylor_inputs (seeded, identical on both sides).  Method:
"A Taylor-Series Route to Linear-Time Transformers with a Fixed Number of
Recurrent States" (arXiv 2610.20637), sections 3.1-3.5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import taylor_inputs as TI
from oracle import recurrent as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


@pytest.fixture(scope="module")
def rsp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recurrent_state_phi_amd as rsp
    return rsp


def say(*a):
    print("[case]", *a, flush=True)


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def run_prefill(rsp, q, k, v, n, a, chunk, dtype, out_dtype=torch.float32, state=None):
    B, H = q.shape[:2]
    if state is None:
        state = rsp.new_state(B, H, n, d=q.shape[-1], device=DEV)
    o = rsp.prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), state, n, a, chunk=chunk,
                    out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), state


def oracle_state(k, v, n):
    """A_m = sum_i phi_m(k_i) [v_i; 1]^T stacked over m (Eq. (6)), float64, per head."""
    k = k.astype(np.float64)
    lead = k.shape[:-2]
    kf, vf = k.reshape((-1,) + k.shape[-2:]), v.reshape((-1,) + v.shape[-2:])
    out = []
    for kh, vh in zip(kf, vf):                       # one head at a time (bounded memory)
        v1 = np.concatenate([vh.astype(np.float64), np.ones((vh.shape[0], 1))], axis=-1)
        feats = np.concatenate([R.phi(kh, m) for m in range(n)], axis=-1)   # [N, D]
        out.append(feats.T @ v1)
    return np.stack(out).reshape(lead + out[0].shape)


# ---------------------------------------------------------------------------
# tiny config: B=1, H=1, N=256, d=16, d_v=64, n=3, a=1, float32
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [32, 64])
def test_tiny_prefill_all_outputs(rsp, chunk):
    say("tiny prefill f32 chunk", chunk)
    q, k, v = TI.make_qkv(TI.SEEDS["tiny"], 1, 1, 256, 16, 64)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0)
    got, _ = run_prefill(rsp, q, k, v, 3, 1.0, chunk, "f32")
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]


def test_tiny_decode_all_outputs(rsp):
    say("tiny decode f32, 256 steps")
    q, k, v = TI.make_qkv(TI.SEEDS["tiny"], 1, 1, 256, 16, 64)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0)
    st = rsp.new_state(1, 1, 3, device=DEV)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = []
    for t in range(256):
        outs.append(rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, 3, 1.0))
    got = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]


# ---------------------------------------------------------------------------
# orders, chunks, dtypes, ragged lengths
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("f32", 64), ("bf16", 32), ("bf16", 64), ("bf16", 128)])
def test_prefill_ragged_vs_oracle(rsp, n, dtype, chunk):
    say("prefill ragged", n, dtype, chunk)
    q, k, v = TI.make_qkv(77, 2, 3, 1000, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    got, st = run_prefill(rsp, q, k, v, n, 1.0, chunk, dtype)
    assert oracle.rel_err_rowwise(got, ref) <= TOL[dtype]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, 2, 3, n))
    A = oracle_state(k, v, n)
    scale = np.abs(A).max(axis=(-1, -2), keepdims=True)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.abs(S - A[..., :64]).max() <= tol * scale.max()
    assert np.abs(T - A[..., 64]).max() <= tol * scale.max()


@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("f32", 64), ("bf16", 32), ("bf16", 64)])
def test_prefill_n4_ragged_vs_oracle(rsp, dtype, chunk):
    """n = 4: the 969-row state is split into feature blocks; outputs and state against the oracle."""
    say("prefill n=4 ragged", dtype, chunk)
    q, k, v = TI.make_qkv(78, 2, 3, 700, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, 4, 1.0)
    got, st = run_prefill(rsp, q, k, v, 4, 1.0, chunk, dtype)
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]  # float32 arithmetic for both input types
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, 2, 3, 4))
    A = oracle_state(k, v, 4)
    scale = np.abs(A).max()
    assert np.abs(S - A[..., :64]).max() <= 1e-5 * scale
    assert np.abs(T - A[..., 64]).max() <= 1e-5 * scale


@pytest.mark.parametrize("N", [1, 17, 65, 300])
def test_prefill_n4_short_and_split(rsp, N):
    say("prefill n=4 short/split", N)
    q, k, v = TI.make_qkv(79, 1, 2, N, 16, 64)
    ref = oracle.taylor_direct(q, k, v, 4, 0.9)
    whole, st_w = run_prefill(rsp, q, k, v, 4, 0.9, 32, "f32")
    assert oracle.rel_err_rowwise(whole, ref) <= TOL["f32"]
    t1 = N // 3
    if t1 > 0:
        a_out, st = run_prefill(rsp, q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], 4, 0.9, 32, "f32")
        b_out, st = run_prefill(rsp, q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], 4, 0.9, 32, "f32", state=st)
        assert oracle.rel_err_rowwise(np.concatenate([a_out, b_out], axis=2), ref) <= TOL["f32"]
        assert np.abs(st.cpu().numpy() - st_w.cpu().numpy()).max() <= 1e-5 * np.abs(st_w.cpu().numpy()).max()


@pytest.mark.parametrize("n", [5, 6])
@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("f32", 64), ("bf16", 64)])
def test_prefill_high_order_vs_oracle(rsp, n, dtype, chunk):
    """n = 5, 6: the 4,845- or 20,349-row state in 28 or 116 feature blocks, each head cut
    into several segments, ragged length, a = 0.8 (so every alpha_m = 1/(m! a^m) up to
    m = 5 matters); outputs and final state against the oracle."""
    say("prefill high order", n, dtype, chunk)
    a = 0.8
    q, k, v = TI.make_qkv(80 + n, 1, 2, 333, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, n, a)
    got, st = run_prefill(rsp, q, k, v, n, a, chunk, dtype)
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]  # float32 arithmetic for both input types
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, 1, 2, n))
    A = oracle_state(k, v, n)
    scale = np.abs(A).max()
    assert np.abs(S - A[..., :64]).max() <= 1e-5 * scale
    assert np.abs(T - A[..., 64]).max() <= 1e-5 * scale


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("bf16", 64)])
def test_wide_heads_vs_oracle(rsp, d, n, dtype, chunk):
    """Head dimensions 32 and 64 (state widths 1/33/561 and 1/65/2,145 rows, in 176-row
    feature blocks): ragged prefill cut into segments, final state, then decode steps
    continuing from it, all against the oracle; a = 1.3."""
    say("wide heads", d, n, dtype, chunk)
    a, N, steps = 1.3, 333, 5
    q, k, v = TI.make_qkv(140 + d + n, 1, 2, N + steps, d, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, n, a)
    got, st = run_prefill(rsp, q[:, :, :N], k[:, :, :N], v[:, :, :N], n, a, chunk, dtype)
    assert oracle.rel_err_rowwise(got, ref[:, :, :N]) <= TOL["f32"]  # float32 arithmetic for both input types
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, 1, 2, n, d=d))
    A = oracle_state(k[:, :, :N], v[:, :, :N], n)
    scale = np.abs(A).max()
    assert np.abs(S - A[..., :64]).max() <= 1e-5 * scale
    assert np.abs(T - A[..., 64]).max() <= 1e-5 * scale
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, a)
            for t in range(N, N + steps)]
    dec = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(dec, ref[:, :, N:]) <= TOL["f32"]


@pytest.mark.parametrize("n", [5, 6])
def test_high_order_split_and_decode(rsp, n):
    """n = 5, 6: prefill in two calls equals one call, and a decode loop continuing from the
    prefilled state matches the oracle (the state carries every order across calls)."""
    say("high order split + decode", n)
    a, N, t1, steps = 1.1, 150, 61, 12
    q, k, v = TI.make_qkv(90 + n, 1, 2, N + steps, 16, 64)
    ref = oracle.taylor_direct(q, k, v, n, a)
    whole, st_w = run_prefill(rsp, q[:, :, :N], k[:, :, :N], v[:, :, :N], n, a, 32, "f32")
    assert oracle.rel_err_rowwise(whole, ref[:, :, :N]) <= TOL["f32"]
    a_out, st = run_prefill(rsp, q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], n, a, 64, "f32")
    b_out, st = run_prefill(rsp, q[:, :, t1:N], k[:, :, t1:N], v[:, :, t1:N], n, a, 32, "f32", state=st)
    assert oracle.rel_err_rowwise(np.concatenate([a_out, b_out], axis=2), ref[:, :, :N]) <= TOL["f32"]
    assert np.abs(st.cpu().numpy() - st_w.cpu().numpy()).max() <= 1e-5 * np.abs(st_w.cpu().numpy()).max()
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, a)
            for t in range(N, N + steps)]
    got = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, ref[:, :, N:]) <= TOL["f32"]


# ---------------------------------------------------------------------------
# closed forms of Eq. (1)-(2) that fix the outputs without the oracle
# ---------------------------------------------------------------------------
def running_mean(v):
    v = v.astype(np.float64)
    return np.cumsum(v, axis=-2) / np.arange(1, v.shape[-2] + 1)[:, None]


@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_n1_is_running_mean(rsp, dtype, chunk):
    """n = 1: the truncated kernel is the constant 1, so o_t is the mean of v_0..v_t for any
    q, k and a; several segments per head, ragged length."""
    say("n=1 running mean", dtype, chunk)
    q, k, v = TI.make_qkv(120, 1, 2, 1500, 16, 64, dtype=dtype)
    got, _ = run_prefill(rsp, q, k, v, 1, 0.7, chunk, dtype)
    assert oracle.rel_err_rowwise(got, running_mean(v)) <= TOL[dtype]


@pytest.mark.parametrize("n,dtype,chunk", [(2, "f32", 64), (3, "f32", 32), (3, "bf16", 64), (3, "bf16", 128),
                                           (4, "f32", 32), (5, "bf16", 64), (6, "f32", 32)])
def test_equal_keys_is_running_mean(rsp, n, dtype, chunk):
    """All keys equal: every weight p_n(q_t.k / a) of row t is the same (and positive at
    a = 2 for unit vectors), so o_t is the mean of v_0..v_t for any n and q; decode steps
    with the same key continue it.  Covers the timed n = 3 bfloat16 kernel across 47
    segments per head."""
    say("equal keys running mean", n, dtype, chunk)
    N, steps = 3000, 4
    q, k, v = TI.make_qkv(121, 1, 2, N + steps, 16, 64, dtype=dtype)
    k = np.ascontiguousarray(np.broadcast_to(k[:, :, :1], k.shape))
    ref = running_mean(v)
    tol = TOL["f32"] if (n >= 4 or dtype == "f32") else TOL["bf16"]
    got, st = run_prefill(rsp, q[:, :, :N], k[:, :, :N], v[:, :, :N], n, 2.0, chunk, dtype)
    assert oracle.rel_err_rowwise(got, ref[:, :, :N]) <= tol
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, 2.0)
            for t in range(N, N + steps)]
    dec = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(dec, ref[:, :, N:]) <= tol


@pytest.mark.parametrize("N", [1, 2, 15, 17, 33, 64, 65, 129])
def test_prefill_short_lengths(rsp, N):
    say("prefill short", N)
    q, k, v = TI.make_qkv(5, 1, 2, N, 16, 64)
    ref = oracle.taylor_direct(q, k, v, 3, 0.8)
    got, _ = run_prefill(rsp, q, k, v, 3, 0.8, 32, "f32")
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]


@pytest.mark.parametrize("n,d,dtype,chunk", [(3, 16, "bf16", 64), (3, 16, "f32", 32), (5, 16, "f32", 32),
                                             (1, 16, "bf16", 128), (3, 64, "bf16", 64)])
def test_empty_calls_leave_state_unchanged(rsp, n, d, dtype, chunk):
    """No tokens (N = 0) and no streams (B = 0): the calls succeed, return empty
    outputs and leave an arbitrary state bit for bit as it was (Eq. (7) adds
    nothing when there is no token)."""
    say("empty calls", n, d, dtype, chunk)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, H = 2, 3
    st = torch.randn(B * H * rsp.state_numel(d, 64, n), device=DEV)
    before = st.clone()
    q0 = torch.zeros(B, H, 0, d, device=DEV, dtype=tdt)
    v0 = torch.zeros(B, H, 0, 64, device=DEV, dtype=tdt)
    o = rsp.prefill(q0, q0.clone(), v0, st, n, 1.0, chunk=chunk)
    st0 = torch.zeros(0, device=DEV)
    od = rsp.decode(torch.zeros(0, H, d, device=DEV, dtype=tdt), torch.zeros(0, H, d, device=DEV, dtype=tdt),
                    torch.zeros(0, H, 64, device=DEV, dtype=tdt), st0, n, 1.0)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, H, 0, 64) and tuple(od.shape) == (0, H, 64)
    assert torch.equal(st, before)


@pytest.mark.parametrize("a", [0.7, 2.0, 3.3])
@pytest.mark.parametrize("chunk", [64, 128])
def test_bf16_prefill_temperatures(rsp, a, chunk):
    """The bfloat16 n = 3 path stages q / a: check temperatures other than 1, ragged N, a resumed state."""
    say("bf16 prefill a", a, "chunk", chunk)
    q, k, v = TI.make_qkv(80, 2, 2, 777, 16, 64, dtype="bf16")
    ref = oracle.taylor_direct(q, k, v, 3, a)
    t1 = 300
    a_out, st = run_prefill(rsp, q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], 3, a, chunk, "bf16")
    b_out, st = run_prefill(rsp, q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], 3, a, chunk, "bf16", state=st)
    assert oracle.rel_err_rowwise(np.concatenate([a_out, b_out], axis=2), ref) <= TOL["bf16"]


@pytest.mark.parametrize("n,in_dtype,chunk", [(3, "bf16", 64), (3, "f32", 32), (4, "bf16", 32), (5, "f32", 64),
                                              (6, "bf16", 32)])
def test_bf16_output(rsp, n, in_dtype, chunk):
    """bfloat16 outputs (rounded once from the float32 result) for every prefill kernel."""
    say("prefill bf16 out", n, in_dtype, chunk)
    q, k, v = TI.make_qkv(6, 1, 4, 700 if n < 6 else 200, 16, 64, dtype=in_dtype)
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    got, _ = run_prefill(rsp, q, k, v, n, 1.0, chunk, in_dtype, out_dtype=torch.bfloat16)
    assert oracle.rel_err_rowwise(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("n", [3, 5, 6])
def test_decode_bf16_io(rsp, n):
    """Decode with bfloat16 q, k, v and bfloat16 outputs (float32 state), after a prefix."""
    say("decode bf16 in/out", n)
    B, H, N0, steps = 1, 3, 40, 5
    q, k, v = TI.make_qkv(7, B, H, N0 + steps, 16, 64, dtype="bf16")
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    _, st = run_prefill(rsp, q[:, :, :N0], k[:, :, :N0], v[:, :, :N0], n, 1.0, 32, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, 1.0,
                       out_dtype=torch.bfloat16) for t in range(N0, N0 + steps)]
    got = torch.stack(outs, dim=2).float().cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, ref[:, :, N0:]) <= TOL["bf16"]


@pytest.mark.parametrize("n", [5, 6])
@pytest.mark.parametrize("N", [1, 2, 33])
def test_high_order_short_lengths(rsp, n, N):
    """n = 5, 6 with one, two and 33 tokens (a partial chunk, padding in every feature block)."""
    say("high order short", n, N)
    q, k, v = TI.make_qkv(8, 2, 1, N, 16, 64)
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    got, _ = run_prefill(rsp, q, k, v, n, 1.0, 32, "f32")
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]


def test_many_heads_single_segment(rsp):
    """600 heads: the plan uses one segment per head (no workspace)."""
    say("prefill 600 heads")
    assert rsp.prefill_workspace_bytes(20, 30, 300, 3, 64) == 0
    q, k, v = TI.make_qkv(8, 20, 30, 300, 16, 64, dtype="bf16")
    rows = np.arange(0, 20 * 30 * 300, 37)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0, rows=rows)
    got, _ = run_prefill(rsp, q, k, v, 3, 1.0, 64, "bf16")
    assert oracle.rel_err_rowwise(got.reshape(-1, 64)[rows], ref) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# additivity, resume and prefill == decode loop (section 5.2, Eq. (7))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_prefill_equals_whole(rsp, dtype):
    say("split prefill", dtype)
    q, k, v = TI.make_qkv(9, 2, 2, 900, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0)
    whole, st_whole = run_prefill(rsp, q, k, v, 3, 1.0, 64, dtype)
    t1 = 333
    a_out, st = run_prefill(rsp, q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], 3, 1.0, 64, dtype)
    # checkpoint/resume: the state goes through host memory and back
    st = st.cpu().to(DEV)
    b_out, st = run_prefill(rsp, q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], 3, 1.0, 64, dtype, state=st)
    split = np.concatenate([a_out, b_out], axis=2)
    assert oracle.rel_err_rowwise(split, ref) <= TOL[dtype]
    assert oracle.rel_err_rowwise(split, whole) <= TOL[dtype]
    sw, ss = st_whole.cpu().numpy(), st.cpu().numpy()
    assert np.abs(sw - ss).max() <= (1e-5 if dtype == "f32" else 1e-2) * np.abs(sw).max()


def test_prefill_equals_decode_loop(rsp):
    say("prefill vs decode loop")
    q, k, v = TI.make_qkv(10, 1, 3, 300, 16, 64)
    pre, st_p = run_prefill(rsp, q, k, v, 3, 1.3, 64, "f32")
    st = rsp.new_state(1, 3, 3, device=DEV)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, 3, 1.3)
            for t in range(300)]
    dec = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(dec, pre) <= 2 * TOL["f32"]
    assert np.abs(st.cpu().numpy() - st_p.cpu().numpy()).max() <= 1e-5 * np.abs(st_p.cpu().numpy()).max()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_after_prefix(rsp, n, dtype):
    say("decode after prefix", n, dtype)
    B, H, N0, steps = 2, 3, 200, 24
    q, k, v = TI.make_qkv(11, B, H, N0 + steps, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    st = rsp.new_state(B, H, n, device=DEV)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    for t in range(N0):  # build the prefix by decode (also covers n >= 4)
        rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, 1.0)
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, 1.0)
            for t in range(N0, N0 + steps)]
    got = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, ref[:, :, N0:]) <= TOL[dtype]


def test_graph_replay_matches_eager(rsp):
    """The calls the bench replays from a HIP graph (state init, n = 3 bfloat16 prefill with
    its workspace, decode steps) captured once and replayed three times, with eager work
    and synchronisations in between: every replay gives the eager outputs and state."""
    say("graph replay vs eager")
    B, H, N, steps, n = 2, 4, 1000, 6, 3
    q, k, v = TI.make_qkv(130, B, H, N + steps, 16, 64, dtype="bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    qp, kp, vp = qd[:, :, :N].contiguous(), kd[:, :, :N].contiguous(), vd[:, :, :N].contiguous()
    qs = [qd[:, :, t].contiguous() for t in range(N, N + steps)]
    ks = [kd[:, :, t].contiguous() for t in range(N, N + steps)]
    vs = [vd[:, :, t].contiguous() for t in range(N, N + steps)]
    st = torch.empty(B * H * rsp.state_numel(16, 64, n), device=DEV)
    ws = torch.empty(rsp.prefill_workspace_bytes(B, H, N, n, 64) // 4 + 4, device=DEV)
    o = torch.empty(B, H, N, 64, device=DEV)
    od = torch.empty(steps, B, H, 64, device=DEV)

    def run():
        rsp.state_init(st, B, H, n)
        rsp.prefill(qp, kp, vp, st, n, 1.0, chunk=64, out=o, workspace=ws)
        for s in range(steps):
            rsp.decode(qs[s], ks[s], vs[s], st, n, 1.0, out=od[s])

    run()
    torch.cuda.synchronize()
    ref_o, ref_od, ref_st = o.clone(), od.clone(), st.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan")), od.fill_(float("nan")), st.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(od, ref_od) and torch.equal(st, ref_st), rep
    exp = oracle.taylor_direct(q, k, v, n, 1.0)
    got = np.concatenate([o.cpu().numpy(), od.permute(1, 2, 0, 3).cpu().numpy()], axis=2).astype(np.float64)
    assert oracle.rel_err_rowwise(got, exp) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# the workloads at full size, on sampled rows
# ---------------------------------------------------------------------------
def sample_rows(B, H, N, per_head, chunk, seed=0):
    """Rows to compare: the first and last token of every chunk of every head
    (every segment of any plan starts and ends on a chunk boundary, so this
    covers the places where a wrong prefix would show first), plus
    `per_head` seeded random positions per head."""
    rng = np.random.default_rng(seed)
    edges = set(range(0, N, chunk)) | set(range(chunk - 1, N, chunk)) | {N - 1}
    rows = []
    for bh in range(B * H):
        pos = set(edges)
        pos.update(rng.integers(0, N, per_head).tolist())
        rows.extend(bh * N + p for p in sorted(pos))
    return np.asarray(rows, np.int64)


def test_prefill_workload_sampled(rsp):
    """B=4, H=8, N=8192, n=3, a=1, chunk=64, bfloat16 inputs, float32 out."""
    say("prefill workload 4x8x8192 bf16")
    B, H, N = 4, 8, 8192
    q, k, v = TI.make_qkv(TI.SEEDS["prefill"], B, H, N, 16, 64, dtype="bf16")
    got, st = run_prefill(rsp, q, k, v, 3, 1.0, 64, "bf16")
    rows = sample_rows(B, H, N, 48, 64)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got.reshape(-1, 64)[rows], ref) <= TOL["bf16"]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, 3))
    A = oracle_state(k[:1, :2], v[:1, :2], 3)
    assert np.abs(T[:1, :2] - A[..., 64]).max() <= 2e-2 * np.abs(A[..., 64]).max()
    assert np.abs(S[:1, :2] - A[..., :64]).max() <= 2e-2 * np.abs(A[..., :64]).max()


@pytest.mark.parametrize("chunk", [64, 128])
def test_one_head_many_segments(rsp, chunk):
    """B=1, H=1, N=32731 (ragged last chunk), bfloat16: the planner cuts the one
    head into 512 (chunk 64) or 256 (chunk 128) segments, so the prefix step
    runs with groups of 23 (16) segments, a short last group and the largest
    number of images per workgroup; sampled rows and the final state against
    the oracle."""
    say("one head, many segments, chunk", chunk)
    B, H, N = 1, 1, 32731
    q, k, v = TI.make_qkv(97, B, H, N, 16, 64, dtype="bf16")
    got, st = run_prefill(rsp, q, k, v, 3, 1.0, chunk, "bf16")
    rows = sample_rows(B, H, N, 96, chunk)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got.reshape(-1, 64)[rows], ref) <= TOL["bf16"]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, 3))
    A = oracle_state(k, v, 3)
    assert np.abs(T - A[..., 64]).max() <= 2e-2 * np.abs(A[..., 64]).max()
    assert np.abs(S - A[..., :64]).max() <= 2e-2 * np.abs(A[..., :64]).max()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_order_sweep_workload(rsp, n):
    """B=2, H=8, N=4096, float32, a=1 (n = 5, 6 beyond the configured sweep, as timed):
    sampled rows against the oracle."""
    say("order sweep", n)
    B, H, N = 2, 8, 4096
    q, k, v = TI.make_qkv(TI.SEEDS["order_sweep"], B, H, N, 16, 64)
    got, _ = run_prefill(rsp, q, k, v, n, 1.0, 64 if n < 3 else 32, "f32")
    rows = sample_rows(B, H, N, 256, 64)
    ref = oracle.taylor_direct(q, k, v, n, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got.reshape(-1, 64)[rows], ref) <= TOL["f32"]


@pytest.mark.parametrize("variant", ["normalised", "unnormalised"])
def test_long_prefill_workload(rsp, variant):
    """B=1, H=16, N=65536, chunk=128, bfloat16 inputs; the unnormalised q,k ~ N(0, 4^2)
    variant must be reported non-converged by the oracle while the GPU still matches it."""
    say("long prefill", variant)
    B, H, N = 1, 16, 65536
    norm = variant == "normalised"
    seed = TI.SEEDS["long" if norm else "long_unnormalised"]
    q, k, v = TI.make_qkv(seed, B, H, N, 16, 64, normalize=norm, scale=4.0, dtype="bf16")
    got, st = run_prefill(rsp, q, k, v, 3, 1.0, 128, "bf16")
    rows = sample_rows(B, H, N, 64, 128)
    ref = oracle.taylor_direct(q, k, v, 3, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got.reshape(-1, 64)[rows], ref) <= TOL["bf16"]
    # the final state of every head against the float64 phi-sum of its 65,536 tokens
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, 3))
    A = oracle_state(k, v, 3)
    assert np.abs(T - A[..., 64]).max() <= 2e-2 * np.abs(A[..., 64]).max()
    assert np.abs(S - A[..., :64]).max() <= 2e-2 * np.abs(A[..., :64]).max()
    rep = oracle.convergence_report(q[:, :1, :256], k[:, :1, :256], v[:, :1, :256], 1.0, 6)
    assert rep["non_converged"] == (not norm)


def test_decode_n5_workload(rsp):
    """B=64 streams, H=8, n=5 (a 645 MB state, as timed): 20 steps from the empty state,
    every output against the oracle."""
    say("decode n=5 workload 64x8, 20 steps")
    B, H, steps, n = 64, 8, 20, 5
    q, k, v = TI.make_qkv(1007, B, H, steps, 16, 64)
    ref = oracle.taylor_direct(q, k, v, n, 1.0)
    st = rsp.new_state(B, H, n, device=DEV)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = [rsp.decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, n, 1.0)
            for t in range(steps)]
    got = torch.stack(outs, dim=2).cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, ref) <= TOL["f32"]


def test_decode_workload_sampled(rsp):
    """B=64 streams, H=8, n=3: states prefilled from an N=65536 context, then 256 steps (float32)."""
    say("decode workload 64x8, ctx 65536, 256 steps")
    B, H, N0, steps, n = 64, 8, 65536, 256, 3
    heads = [(0, 0), (7, 3), (21, 5), (33, 1), (42, 7), (50, 2), (63, 6), (63, 0)]
    # inputs of the sampled heads from the seeded generator; the other heads get
    # seeded torch noise of the same distribution (they are computed but not compared)
    g = torch.Generator(device=DEV).manual_seed(1234)
    qd = torch.randn(B, H, N0 + steps, 16, device=DEV, generator=g)
    kd = torch.randn(B, H, N0 + steps, 16, device=DEV, generator=g)
    vd = torch.randn(B, H, N0 + steps, 64, device=DEV, generator=g)
    qd = qd / qd.norm(dim=-1, keepdim=True)
    kd = kd / kd.norm(dim=-1, keepdim=True)
    host = {}
    for b, h in heads:
        q1, k1, v1 = TI.head_qkv(TI.SEEDS["decode"], b, h, N0 + steps, 16, 64)
        host[(b, h)] = (q1, k1, v1)
        qd[b, h] = torch.from_numpy(q1).to(DEV)
        kd[b, h] = torch.from_numpy(k1).to(DEV)
        vd[b, h] = torch.from_numpy(v1).to(DEV)
    st = rsp.new_state(B, H, n, device=DEV)
    rsp.prefill(qd[:, :, :N0].contiguous(), kd[:, :, :N0].contiguous(), vd[:, :, :N0].contiguous(), st, n, 1.0,
                chunk=64)
    qs = qd[:, :, N0:].permute(2, 0, 1, 3).contiguous()
    ks = kd[:, :, N0:].permute(2, 0, 1, 3).contiguous()
    vs = vd[:, :, N0:].permute(2, 0, 1, 3).contiguous()
    del qd, kd, vd
    outs = torch.empty(steps, B, H, 64, device=DEV)
    for s in range(steps):
        rsp.decode(qs[s], ks[s], vs[s], st, n, 1.0, out=outs[s])
    got = outs.cpu().numpy().astype(np.float64)
    for b, h in heads:
        q1, k1, v1 = host[(b, h)]
        rows = np.arange(N0, N0 + steps)
        ref = oracle.taylor_direct(q1, k1, v1, n, 1.0, rows=rows)
        assert oracle.rel_err_rowwise(got[:, b, h], ref) <= TOL["f32"], (b, h)


# ---------------------------------------------------------------------------
# the bounded waits between the workgroups of one sequence (n = 3, bf16)
# ---------------------------------------------------------------------------
def test_prefill_wait_timeout_is_reported(rsp):
    """With a limit of zero polls every wait between segment workgroups gives up at
    once: the call still completes and taylor_prefill_check reports
    TAYLOR_ETIMEOUT.  With the default limit the same call passes the check and
    matches the oracle."""
    say("prefill wait time-out path")
    B, H, N = 1, 2, 1000  # 16 chunks of 64 per head: one workgroup per chunk-long segment
    q, k, v = TI.make_qkv(91, B, H, N, 16, 64, dtype="bf16")
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    need = rsp.prefill_workspace_bytes(B, H, N, 3, 64)
    assert need > 0
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    prev = rsp.set_wait_limit(0)
    try:
        st = rsp.new_state(B, H, 3, device=DEV)
        rsp.prefill(qd, kd, vd, st, 3, 1.0, chunk=64, workspace=ws)
        with pytest.raises(rsp.TaylorError) as e:
            rsp.prefill_check(ws)
        assert e.value.code == -4
    finally:
        rsp.set_wait_limit(prev)
    st = rsp.new_state(B, H, 3, device=DEV)
    o = rsp.prefill(qd, kd, vd, st, 3, 1.0, chunk=64, workspace=ws)
    rsp.prefill_check(ws)
    got = o.float().cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, 3, 1.0)) <= TOL["bf16"]
