"""GPU parity of decode against a bfloat16-stored state (the state sizes of
section 5.8 of "A Taylor-Series Route to Linear-Time Transformers with a Fixed
Number of Recurrent States", arXiv 2610.20637) with an exact window of recent
tokens, against the float64 oracle's direct n-term sum, through the C ABI.

The state's S part is bfloat16, so the bar is the bfloat16 one: max over rows
of ||o_t - o^_t||_inf / ||o^_t||_inf <= 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import taylor_inputs as TI

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


@pytest.fixture(scope="module")
def rsp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recurrent_state_phi_amd as rsp
    return rsp


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def run(rsp, q, k, v, N0, steps, n, a, window, dtype, st32=None):
    """float32 prefill of tokens [0, N0), rounded to a bfloat16 state, then `steps`
    decode steps against it; returns the decode outputs [B, H, steps, d_v]."""
    B, H = q.shape[:2]
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    if st32 is None:
        st32 = rsp.new_state(B, H, n, device=DEV)
        if N0 > 0:
            rsp.prefill(qd[:, :, :N0].contiguous(), kd[:, :, :N0].contiguous(), vd[:, :, :N0].contiguous(), st32,
                        n, a, chunk=32)
    sb = rsp.new_state_bf16(B, H, n, device=DEV)
    rsp.state_to_bf16(st32, sb, B, H, n)
    wk = torch.empty(B, H, window, 16, device=DEV, dtype=qd.dtype)
    wv = torch.empty(B, H, window, 64, device=DEV, dtype=qd.dtype)
    outs = torch.empty(steps, B, H, 64, device=DEV)
    for s in range(steps):
        t = N0 + s
        rsp.decode_bf16state(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), sb, wk,
                             wv, s % window, n, a, out=outs[s])
    torch.cuda.synchronize()
    return outs.permute(1, 2, 0, 3).cpu().numpy().astype(np.float64), sb


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window", [32, 50, 128])
def test_bf16_state_decode_vs_oracle(rsp, n, dtype, window):
    """A 500-token prefill, then 150 steps: several folds and a partly filled window
    at the end; every output against the oracle."""
    print("[case] bf16 state decode", n, dtype, window, flush=True)
    N0, steps, a = 500, 150, 0.9
    q, k, v = TI.make_qkv(400 + n, 2, 3, N0 + steps, 16, 64, dtype=dtype)
    got, _ = run(rsp, q, k, v, N0, steps, n, a, window, dtype)
    ref = oracle.taylor_direct(q, k, v, n, a)[:, :, N0:]
    assert oracle.rel_err_rowwise(got, ref) <= TOL


def test_bf16_state_from_empty_and_after_fold(rsp):
    """From the empty state: the first window-1 steps use only the window (the base is
    zero), so they match the oracle to float32 rounding; after the fold T (float32)
    holds the exact token count and feature sums, S the rounded sums."""
    print("[case] bf16 state from empty", flush=True)
    n, a, window, B, H = 3, 1.0, 16, 1, 2
    q, k, v = TI.make_qkv(410, B, H, 40, 16, 64)
    st32 = rsp.new_state(B, H, n, device=DEV)
    got, sb = run(rsp, q, k, v, 0, window, n, a, window, "f32", st32=st32)
    ref = oracle.taylor_direct(q, k, v, n, a)[:, :, :window]
    assert oracle.rel_err_rowwise(got[:, :, :window - 1], ref[:, :, :window - 1]) <= 1e-5
    assert oracle.rel_err_rowwise(got, ref) <= 1e-5
    from oracle import recurrent as R
    S, T = (x.float().cpu().numpy().astype(np.float64) for x in rsp.state_bf16_views(sb, B, H, n))
    for h in range(H):
        A = np.concatenate([R.phi(k[0, h, :window].astype(np.float64), m) for m in range(n)], axis=-1).T @ \
            np.concatenate([v[0, h, :window].astype(np.float64), np.ones((window, 1))], axis=1)
        assert np.abs(T[0, h] - A[:, 64]).max() <= 1e-5 * np.abs(A[:, 64]).max()
        assert T[0, h, 0] == window                                # the token count, exactly
        assert np.abs(S[0, h] - A[:, :64]).max() <= 2 ** -8 * np.abs(A[:, :64]).max()


def test_bf16_state_decode_workload(rsp):
    """B=64 streams, H=8, n=3: the float32 state of a 65,536-token context rounded to
    bfloat16, then 256 steps with a window of 64 tokens (four folds), float32 q, k, v;
    eight sampled heads against the oracle over all 65,536 + s + 1 keys.  The same run
    with a window of one token (the state rounded after every token) misses the
    bfloat16 bar: the window is what keeps the recent increments."""
    print("[case] bf16 state decode workload 64x8, ctx 65536, 256 steps", flush=True)
    B, H, N0, steps, n, a = 64, 8, 65536, 256, 3, 1.0
    heads = [(0, 0), (7, 3), (21, 5), (33, 1), (42, 7), (50, 2), (63, 6), (63, 0)]
    g = torch.Generator(device=DEV).manual_seed(5678)
    st32 = rsp.new_state(B, H, n, device=DEV)
    host = {hd: TI.head_qkv(TI.SEEDS["decode"], hd[0], hd[1], N0 + steps, 16, 64) for hd in heads}
    for t0 in range(0, N0, 8192):  # context prefill in slices (the state is additive)
        qc = torch.randn(B, H, 8192, 16, device=DEV, generator=g)
        kc = torch.randn(B, H, 8192, 16, device=DEV, generator=g)
        vc = torch.randn(B, H, 8192, 64, device=DEV, generator=g)
        qc, kc = qc / qc.norm(dim=-1, keepdim=True), kc / kc.norm(dim=-1, keepdim=True)
        for (b, h), (q1, k1, v1) in host.items():
            qc[b, h] = torch.from_numpy(q1[t0:t0 + 8192]).to(DEV)
            kc[b, h] = torch.from_numpy(k1[t0:t0 + 8192]).to(DEV)
            vc[b, h] = torch.from_numpy(v1[t0:t0 + 8192]).to(DEV)
        rsp.prefill(qc, kc, vc, st32, n, a, chunk=64)
        del qc, kc, vc
    qs = torch.randn(steps, B, H, 16, device=DEV, generator=g)
    ks = torch.randn(steps, B, H, 16, device=DEV, generator=g)
    vs = torch.randn(steps, B, H, 64, device=DEV, generator=g)
    qs, ks = qs / qs.norm(dim=-1, keepdim=True), ks / ks.norm(dim=-1, keepdim=True)
    for (b, h), (q1, k1, v1) in host.items():
        qs[:, b, h] = torch.from_numpy(q1[N0:]).to(DEV)
        ks[:, b, h] = torch.from_numpy(k1[N0:]).to(DEV)
        vs[:, b, h] = torch.from_numpy(v1[N0:]).to(DEV)
    refs = {hd: oracle.taylor_direct(*host[hd], n, a, rows=np.arange(N0, N0 + steps)) for hd in heads}
    errs = {}
    for window in (64, 1):
        sb = rsp.new_state_bf16(B, H, n, device=DEV)
        rsp.state_to_bf16(st32, sb, B, H, n)
        wk = torch.empty(B, H, window, 16, device=DEV)
        wv = torch.empty(B, H, window, 64, device=DEV)
        outs = torch.empty(steps, B, H, 64, device=DEV)
        for s in range(steps):
            rsp.decode_bf16state(qs[s], ks[s], vs[s], sb, wk, wv, s % window, n, a, out=outs[s])
        got = outs.cpu().numpy().astype(np.float64)
        errs[window] = max(oracle.rel_err_rowwise(got[:, b, h], refs[(b, h)]) for b, h in heads)
        del sb
    print(f"[case] max row error: window 64 {errs[64]:.3e}, window 1 {errs[1]:.3e}", flush=True)
    assert errs[64] <= TOL
    assert errs[1] > TOL
