"""GPU parity of the eviction-fed hybrid decode ("Tensor Cache: Eviction-conditioned
Associative Memory for Transformers", sections 3.1-3.2: exact softmax over a FIFO
window of the last W pairs, a memory written with the pairs the window evicts;
the memory here is the n-term Taylor state of "A Taylor-Series Route to
Linear-Time Transformers with a Fixed Number of Recurrent States") against the
float64 oracle's direct sum, through the C ABI.  Tolerances (max over rows of
||o_t - o^_t||_inf / ||o^_t||_inf): 1e-4 float32, 2e-2 bfloat16 inputs."""
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


def run(rsp, q, k, v, N0, steps, n, a, W, dtype):
    """Context of N0 tokens (the first N0 - W prefilled into the state, the last W in
    the ring), then `steps` hybrid decode steps; outputs [B, H, steps, d_v] and state."""
    B, H = q.shape[:2]
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    st = rsp.new_state(B, H, n, device=DEV)
    ne = max(0, N0 - W)
    if ne > 0:
        rsp.prefill(qd[:, :, :ne].contiguous(), kd[:, :, :ne].contiguous(), vd[:, :, :ne].contiguous(), st, n, a,
                    chunk=32)
    wk = torch.full((B, H, W, 16), float("nan"), device=DEV, dtype=qd.dtype)  # unwritten slots must not matter
    wv = torch.full((B, H, W, 64), float("nan"), device=DEV, dtype=qd.dtype)
    if N0 > 0:
        rsp.hybrid_fill_window(kd[:, :, :N0].contiguous(), vd[:, :, :N0].contiguous(), wk, wv)
    outs = torch.empty(steps, B, H, 64, device=DEV)
    for s in range(steps):
        t = N0 + s
        rsp.hybrid_decode(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), st, wk, wv,
                          t, n, a, out=outs[s])
    torch.cuda.synchronize()
    return outs.permute(1, 2, 0, 3).cpu().numpy().astype(np.float64), st


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N0,W", [(300, 1), (300, 16), (300, 64), (300, 200), (10, 64), (0, 33)])
def test_hybrid_decode_vs_oracle(rsp, n, dtype, N0, W):
    """Windows of 1 to 200 tokens after a 300-token context, a context shorter than the
    window (nothing evicted at first), and a start from nothing; 90 steps each."""
    print("[case] hybrid decode", n, dtype, N0, W, flush=True)
    steps, a = 90, 0.9
    q, k, v = TI.make_qkv(500 + n + W, 2, 3, N0 + steps, 16, 64, dtype=dtype)
    got, _ = run(rsp, q, k, v, N0, steps, n, a, W, dtype)
    ref = oracle.hybrid_direct(q, k, v, n, a, W)[:, :, N0:]
    assert oracle.rel_err_rowwise(got, ref) <= TOL[dtype]


def test_hybrid_window_longer_than_sequence_is_softmax(rsp):
    """Nothing ever leaves a window longer than the sequence: the outputs are exact
    softmax attention and the Taylor state stays empty."""
    print("[case] hybrid = softmax", flush=True)
    N0, steps, W = 50, 60, 1024
    q, k, v = TI.make_qkv(520, 1, 2, N0 + steps, 16, 64)
    got, st = run(rsp, q, k, v, N0, steps, 3, 1.0, W, "f32")
    assert oracle.rel_err_rowwise(got, oracle.softmax(q, k, v, 1.0)[:, :, N0:]) <= TOL["f32"]
    assert torch.count_nonzero(st).item() == 0


def test_hybrid_state_holds_exactly_the_evicted_tokens(rsp):
    """After the steps the state is the phi-sum of the tokens 0 .. t - W (Eq. (6))."""
    print("[case] hybrid state", flush=True)
    from oracle import recurrent as R
    N0, steps, W, n = 100, 50, 30, 3
    q, k, v = TI.make_qkv(521, 1, 2, N0 + steps, 16, 64)
    _, st = run(rsp, q, k, v, N0, steps, n, 1.0, W, "f32")
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, 1, 2, n))
    ne = N0 + steps - W  # tokens evicted by the end
    for h in range(2):
        kk = k[0, h, :ne].astype(np.float64)
        A = np.concatenate([R.phi(kk, m) for m in range(n)], axis=-1).T @ \
            np.concatenate([v[0, h, :ne].astype(np.float64), np.ones((ne, 1))], axis=1)
        assert np.abs(S[0, h] - A[:, :64]).max() <= 1e-5 * np.abs(A).max()
        assert np.abs(T[0, h] - A[:, 64]).max() <= 1e-5 * np.abs(A).max()


def test_hybrid_decode_workload(rsp):
    """B=64 streams, H=8, n=3, float32: a 65,536-token context (65,280 tokens in the
    state, 256 in the window), then 256 steps; eight sampled heads against the oracle."""
    print("[case] hybrid decode workload 64x8, ctx 65536, W 256, 256 steps", flush=True)
    B, H, N0, steps, n, a, W = 64, 8, 65536, 256, 3, 1.0, 256
    heads = [(0, 0), (7, 3), (21, 5), (33, 1), (42, 7), (50, 2), (63, 6), (63, 0)]
    g = torch.Generator(device=DEV).manual_seed(6789)
    host = {hd: TI.head_qkv(TI.SEEDS["decode"], hd[0], hd[1], N0 + steps, 16, 64) for hd in heads}
    st = rsp.new_state(B, H, n, device=DEV)
    wk = torch.empty(B, H, W, 16, device=DEV)
    wv = torch.empty(B, H, W, 64, device=DEV)
    ne = N0 - W
    for t0 in range(0, N0, 8192):  # context in slices; the last slice also fills the window
        qc = torch.randn(B, H, 8192, 16, device=DEV, generator=g)
        kc = torch.randn(B, H, 8192, 16, device=DEV, generator=g)
        vc = torch.randn(B, H, 8192, 64, device=DEV, generator=g)
        qc, kc = qc / qc.norm(dim=-1, keepdim=True), kc / kc.norm(dim=-1, keepdim=True)
        for (b, h), (q1, k1, v1) in host.items():
            qc[b, h] = torch.from_numpy(q1[t0:t0 + 8192]).to(DEV)
            kc[b, h] = torch.from_numpy(k1[t0:t0 + 8192]).to(DEV)
            vc[b, h] = torch.from_numpy(v1[t0:t0 + 8192]).to(DEV)
        m = min(8192, ne - t0)
        rsp.prefill(qc[:, :, :m].contiguous(), kc[:, :, :m].contiguous(), vc[:, :, :m].contiguous(), st, n, a,
                    chunk=64)
        if t0 + 8192 == N0:
            rsp.hybrid_fill_window(kc, vc, wk, wv)  # positions N0-8192..N0-1: slots i % W
        del qc, kc, vc
    qs = torch.randn(steps, B, H, 16, device=DEV, generator=g)
    ks = torch.randn(steps, B, H, 16, device=DEV, generator=g)
    vs = torch.randn(steps, B, H, 64, device=DEV, generator=g)
    qs, ks = qs / qs.norm(dim=-1, keepdim=True), ks / ks.norm(dim=-1, keepdim=True)
    for (b, h), (q1, k1, v1) in host.items():
        qs[:, b, h] = torch.from_numpy(q1[N0:]).to(DEV)
        ks[:, b, h] = torch.from_numpy(k1[N0:]).to(DEV)
        vs[:, b, h] = torch.from_numpy(v1[N0:]).to(DEV)
    outs = torch.empty(steps, B, H, 64, device=DEV)
    for s in range(steps):
        rsp.hybrid_decode(qs[s], ks[s], vs[s], st, wk, wv, N0 + s, n, a, out=outs[s])
    got = outs.cpu().numpy().astype(np.float64)
    for b, h in heads:
        ref = oracle.hybrid_direct(*host[(b, h)], n, a, W, rows=np.arange(N0, N0 + steps))
        assert oracle.rel_err_rowwise(got[:, b, h], ref) <= TOL["f32"], (b, h)
