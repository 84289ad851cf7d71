"""The prefill entry point that allocates nothing (taylor_attn_prefill_noalloc: a
fixed per-device scratch array instead of the caller's workspace) against the
existing entry point with a workspace, through the C ABI, on two calls in a row
(the second smaller, so that it runs on whatever the first left in the shared
scratch), and against the float64 oracle.  Method: "A Taylor-Series Route to
Linear-Time Transformers with a Fixed Number of Recurrent States" (arXiv
2610.20637), section 3.5."""
import numpy as np
import pytest
import torch

import oracle
import taylor_inputs as TI

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def rsp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recurrent_state_phi_amd as rsp
    return rsp


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _both(rsp, B, H, N, n, chunk, dtype, seed, a=1.0):
    q, k, v = TI.make_qkv(seed, B, H, N, 16, 64, dtype=dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    st_ref = rsp.new_state(B, H, n, device=DEV)
    st_ref.copy_(torch.randn(st_ref.shape, device=DEV).abs())  # a non-empty incoming state
    st_na = st_ref.clone()
    ws = torch.empty(max(rsp.prefill_workspace_bytes(B, H, N, n, chunk) // 4, 1), device=DEV)
    o_ref = rsp.prefill(qd, kd, vd, st_ref, n, a, chunk=chunk, workspace=ws)
    o_na = torch.empty_like(o_ref)
    rsp.prefill_noalloc(qd, kd, vd, st_na, n, a, chunk=chunk, out=o_na)
    torch.cuda.synchronize()
    return (q, k, v), o_ref, o_na, st_ref, st_na


@pytest.mark.parametrize("n,chunk,dtype", [(3, 64, "bf16"), (3, 128, "bf16"), (2, 64, "f32"), (3, 32, "f32")])
def test_noalloc_matches_workspace_entry_point(rsp, n, chunk, dtype):
    print("[case] noalloc", n, chunk, dtype, flush=True)
    # first call: several segments per head (the scratch holds images / segment sums)
    (q, k, v), o_ref, o_na, st_ref, st_na = _both(rsp, 2, 4, 3000, n, chunk, dtype, 300 + n)
    assert rsp.prefill_workspace_bytes(2, 4, 3000, n, chunk) > 0
    assert torch.equal(o_na, o_ref) and torch.equal(st_na, st_ref)
    # second call, smaller, on the scratch the first one left behind
    (q, k, v), o_ref2, o_na2, st_ref2, st_na2 = _both(rsp, 1, 2, 700, n, chunk, dtype, 310 + n)
    assert rsp.prefill_workspace_bytes(1, 2, 700, n, chunk) > 0
    assert torch.equal(o_na2, o_ref2) and torch.equal(st_na2, st_ref2)
    # and the same result as the oracle for the second call from the empty state
    st = rsp.new_state(1, 2, n, device=DEV)
    o = rsp.prefill_noalloc(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), st, n, 1.0, chunk=chunk)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, 1.0)) <= TOL[dtype]


def test_noalloc_refuses_plans_beyond_the_scratch(rsp):
    """n = 4 at B=2, H=8, N=4096 needs about 121 MiB of workspace: refused, nothing written."""
    print("[case] noalloc too large", flush=True)
    B, H, N = 2, 8, 4096
    q = torch.zeros(B, H, N, 16, device=DEV)
    v = torch.zeros(B, H, N, 64, device=DEV)
    st = rsp.new_state(B, H, 4, device=DEV)
    o = torch.full((B, H, N, 64), 7.0, device=DEV)
    with pytest.raises(rsp.TaylorError) as e:
        rsp.prefill_noalloc(q, q.clone(), v, st, 4, 1.0, chunk=32, out=o)
    assert e.value.code == -1
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(st == 0.0)
