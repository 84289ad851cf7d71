"""GPU checks of the profiling hook (taylor_set_phase_events) that bench.py times
its prefill kernels with: on every prefill path the four events are recorded on
the call's stream, in order, the kernel interval (events 2 -> 3) lies inside the
whole call, and a call with the hook set gives the same bits as one without it.
Outputs are also checked against the float64 oracle (max over rows of
||o_t - o_t^oracle||_inf / ||o_t^oracle||_inf: 1e-4 float32, 2e-2 bfloat16 inputs).
"""
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


# (n, input type, chunk, N): the single-launch n = 3 kernel (chunks of 64 and of
# 128), the single-launch n = 1 and n = 2 kernel, and the three-launch
# feature-blocked path (float32 n = 3, and n = 4), each with several segments
CASES = [(3, "bf16", 64, 3000), (3, "bf16", 128, 3000), (1, "f32", 64, 3000), (2, "f32", 64, 3000),
         (3, "f32", 32, 3000), (4, "f32", 32, 1500)]


@pytest.mark.parametrize("n,dtype,chunk,N", CASES)
def test_phase_events_bracket_the_call(rsp, n, dtype, chunk, N):
    print("[case] phase events", n, dtype, chunk, N, flush=True)
    B, H, a = 1, 4, 1.0
    q, k, v = TI.make_qkv(790 + n, B, H, N, 16, 64, dtype=dtype)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    st0 = rsp.new_state(B, H, n, device=DEV)
    plain = rsp.prefill(qd, kd, vd, st0, n, a, chunk=chunk)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()  # materialise the HIP event handles
    torch.cuda.synchronize()
    st1 = rsp.new_state(B, H, n, device=DEV)
    rsp.set_phase_events(evs)
    try:
        timed = rsp.prefill(qd, kd, vd, st1, n, a, chunk=chunk)
    finally:
        rsp.set_phase_events(None)
    torch.cuda.synchronize()
    gaps = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    whole = evs[0].elapsed_time(evs[3])
    assert all(g >= 0.0 for g in gaps), gaps
    assert gaps[2] > 0.0  # the prefill (or last phase) kernel ran inside events 2 -> 3
    assert gaps[2] <= whole + 1e-3
    assert torch.equal(timed, plain) and torch.equal(st1, st0)
    got = timed.float().cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, a)) <= TOL[dtype]
