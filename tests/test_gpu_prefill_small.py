"""GPU parity of the single-launch n = 1, 2 prefill at d = 16 (section 3.5 of "A
Taylor-Series Route to Linear-Time Transformers with a Fixed Number of Recurrent
States", arXiv 2610.20637): segments of 128 (n = 1) or 256 (n = 2) tokens, 16-token chunks inside, a
look-back over the earlier segments of a sequence for the prefix.  Against the
float64 oracle through the C ABI; tolerances (max over rows of
||o_t - o_t^oracle||_inf / ||o_t^oracle||_inf): 1e-4 float32, 2e-2 bfloat16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import taylor_inputs as TI
from oracle import recurrent as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"
SEG = {1: 128, 2: 256}  # tokens per segment, by n


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


def state_of(k, v, n):
    """Stacked phi(k)^T [v, 1] (Eq. (6)) of one head, float64: rows = features."""
    kk = k.astype(np.float64)
    feats = np.concatenate([R.phi(kk, m) for m in range(n)], axis=-1)
    return feats.T @ np.concatenate([v.astype(np.float64), np.ones((v.shape[0], 1))], axis=1)


def edge_rows(N, per_head, heads, seed, seg):
    """Rows of every head: first and last token of every segment of `seg` tokens, of
    every 16-token chunk in the first two and the last two segments, the last token,
    and seeded random positions."""
    rng = np.random.default_rng(seed)
    edges = set(range(0, N, seg)) | set(range(seg - 1, N, seg)) | {N - 1}
    last = (N - 1) // seg * seg
    for lo, hi in ((0, 2 * seg), (max(0, last - seg), N)):
        edges |= set(range(lo, min(hi, N), 16)) | set(range(lo + 15, min(hi, N), 16))
    rows = []
    for bh in range(heads):
        pos = set(edges)
        pos.update(rng.integers(0, N, per_head).tolist())
        rows.extend(bh * N + p for p in sorted(pos))
    return np.asarray(rows, np.int64)


@pytest.mark.parametrize("n", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_segments_per_head(rsp, n, dtype):
    """B=1, H=2, N=70,001: 547 (n = 1) or 274 (n = 2) segments per head (the
    look-back polls 64 flags per read, so it has to move its window back several
    times), a short last segment; sampled rows and the final state against the
    oracle."""
    say("n<=2 many segments", n, dtype)
    B, H, N, a = 1, 2, 70001, 1.3
    q, k, v = TI.make_qkv(700 + n, B, H, N, 16, 64, dtype=dtype)
    st = rsp.new_state(B, H, n, device=DEV)
    o = rsp.prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), st, n, a, chunk=64, check=True)
    got = o.float().cpu().numpy().astype(np.float64).reshape(-1, 64)
    rows = edge_rows(N, 128, B * H, 5, SEG[n])
    ref = oracle.taylor_direct(q, k, v, n, a, rows=rows)
    assert oracle.rel_err_rowwise(got[rows], ref) <= TOL[dtype]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, n))
    for h in range(H):
        A = state_of(k[0, h], v[0, h], n)
        assert T[0, h, 0] == N
        assert np.abs(S[0, h] - A[:, :64]).max() <= 1e-5 * np.abs(A[:, :64]).max()
        assert np.abs(T[0, h] - A[:, 64]).max() <= 1e-5 * np.abs(A[:, 64]).max()


@pytest.mark.parametrize("n", [1, 2])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 127, 128, 129, 255, 256, 257, 511, 513, 1000])
def test_lengths_around_segment_edges(rsp, n, N):
    """Every output row against the oracle for lengths around the 16-token chunk and
    the 128- and 256-token segments (one segment, one full, one plus a token, ...)."""
    say("n<=2 length", n, N)
    q, k, v = TI.make_qkv(710 + N, 2, 3, N, 16, 64)
    st = rsp.new_state(2, 3, n, device=DEV)
    o = rsp.prefill(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), st, n, 0.8, chunk=32, check=True)
    got = o.cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, 0.8)) <= TOL["f32"]


@pytest.mark.parametrize("n", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_resume_through_host(rsp, n, dtype):
    """Three calls (300, 800 and 601 tokens) continuing one state, which goes through
    host memory between calls, equal one call over the 1,701 tokens and the oracle."""
    say("n<=2 split/resume", n, dtype)
    B, H, N, a = 2, 2, 1701, 1.0
    q, k, v = TI.make_qkv(720 + n, B, H, N, 16, 64, dtype=dtype)
    ref = oracle.taylor_direct(q, k, v, n, a)
    stw = rsp.new_state(B, H, n, device=DEV)
    whole = rsp.prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), stw, n, a).cpu().numpy()
    st = rsp.new_state(B, H, n, device=DEV)
    parts = []
    for t0, t1 in ((0, 300), (300, 1100), (1100, N)):
        st = st.cpu().to(DEV)
        sl = (slice(None), slice(None), slice(t0, t1))
        parts.append(rsp.prefill(to_dev(q[sl], dtype), to_dev(k[sl], dtype), to_dev(v[sl], dtype), st, n, a,
                                 chunk=64).cpu().numpy())
    split = np.concatenate(parts, axis=2).astype(np.float64)
    assert oracle.rel_err_rowwise(split, ref) <= TOL[dtype]
    assert oracle.rel_err_rowwise(split, whole.astype(np.float64)) <= TOL[dtype]
    sw, ss = stw.cpu().numpy(), st.cpu().numpy()
    assert np.abs(sw - ss).max() <= 1e-5 * np.abs(sw).max()


@pytest.mark.parametrize("n", [1, 2])
def test_bf16_output(rsp, n):
    """bfloat16 inputs and outputs (16-byte stores of 8 values per lane)."""
    say("n<=2 bf16 out", n)
    B, H, N = 2, 4, 3000
    q, k, v = TI.make_qkv(730 + n, B, H, N, 16, 64, dtype="bf16")
    st = rsp.new_state(B, H, n, device=DEV)
    o = rsp.prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), st, n, 1.0, chunk=64,
                    out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    got = o.float().cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, 1.0)) <= TOL["bf16"]


def test_graph_replay_matches_eager(rsp):
    """n = 2, float32: state init and a prefill with its workspace (flag clearing,
    ticket counter, look-back) captured once in a HIP graph and replayed three times
    with eager work and synchronisations in between: every replay gives the eager
    outputs and state bit for bit."""
    say("n<=2 graph replay")
    B, H, N, n = 2, 4, 3000, 2
    q, k, v = TI.make_qkv(740, B, H, N, 16, 64)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    st = torch.empty(B * H * rsp.state_numel(16, 64, n), device=DEV)
    ws = torch.empty(rsp.prefill_workspace_bytes(B, H, N, n, 64) // 4 + 4, device=DEV)
    o = torch.empty(B, H, N, 64, device=DEV)

    def run():
        rsp.state_init(st, B, H, n)
        rsp.prefill(qd, kd, vd, st, n, 1.0, chunk=64, out=o, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref_o, ref_st = o.clone(), st.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan")), st.fill_(7.0), ws.fill_(3.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(st, ref_st), rep
    got = o.cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, 1.0)) <= TOL["f32"]


def test_wait_timeout_is_reported(rsp):
    """With a limit of zero polls every look-back gives up at once: the call still
    completes and taylor_prefill_check reports TAYLOR_ETIMEOUT; with the default
    limit the same call passes the check and matches the oracle."""
    say("n<=2 wait time-out path")
    B, H, N, n = 1, 2, 2000, 2  # 8 segments per head
    q, k, v = TI.make_qkv(750, B, H, N, 16, 64)
    qd, kd, vd = (to_dev(x, "f32") for x in (q, k, v))
    ws = torch.empty(rsp.prefill_workspace_bytes(B, H, N, n, 64) // 4, device=DEV)
    prev = rsp.set_wait_limit(0)
    try:
        st = rsp.new_state(B, H, n, device=DEV)
        rsp.prefill(qd, kd, vd, st, n, 1.0, chunk=64, workspace=ws)
        with pytest.raises(rsp.TaylorError) as e:
            rsp.prefill_check(ws)
        assert e.value.code == -4
    finally:
        rsp.set_wait_limit(prev)
    st = rsp.new_state(B, H, n, device=DEV)
    o = rsp.prefill(qd, kd, vd, st, n, 1.0, chunk=64, workspace=ws)
    rsp.prefill_check(ws)
    got = o.cpu().numpy().astype(np.float64)
    assert oracle.rel_err_rowwise(got, oracle.taylor_direct(q, k, v, n, 1.0)) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_heads_several_rounds(rsp, dtype):
    """B=16, H=8, N=4096, n = 2: 2,048 segment workgroups, several rounds of them on
    the GPU (later rounds find their predecessors long done); sampled rows of every
    head and the final state of a few heads against the oracle."""
    say("n<=2 many heads", dtype)
    B, H, N, n = 16, 8, 4096, 2
    q, k, v = TI.make_qkv(760, B, H, N, 16, 64, dtype=dtype)
    st = rsp.new_state(B, H, n, device=DEV)
    o = rsp.prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), st, n, 1.0, chunk=64, check=True)
    got = o.float().cpu().numpy().astype(np.float64).reshape(-1, 64)
    rows = edge_rows(N, 8, B * H, 6, SEG[n])
    ref = oracle.taylor_direct(q, k, v, n, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got[rows], ref) <= TOL[dtype]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, n))
    for b, h in ((0, 0), (7, 3), (15, 7)):
        A = state_of(k[b, h], v[b, h], n)
        assert np.abs(S[b, h] - A[:, :64]).max() <= 1e-5 * np.abs(A[:, :64]).max()
        assert np.abs(T[b, h] - A[:, 64]).max() <= 1e-5 * np.abs(A[:, 64]).max()


def test_more_than_4096_segments(rsp):
    """One head of 576,001 tokens, n = 1: 4,501 segments in groups of 68, so both
    parts of the look-back (67 earlier members, 66 earlier groups) wait on more than
    64 flags and poll in two reads; sampled rows (segment starts and ends, the chunks
    around the first group edges, the last segments) and the final state against the
    oracle."""
    say("n<=2 4,501 segments")
    B, H, N, n = 1, 1, SEG[1] * 4500 + 1, 1
    q, k, v = TI.make_qkv(770, B, H, N, 16, 64)
    st = rsp.new_state(B, H, n, device=DEV)
    o = rsp.prefill(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), st, n, 1.0, chunk=64, check=True)
    got = o.cpu().numpy().astype(np.float64).reshape(-1, 64)
    G, L = 68, SEG[1]
    nseg = (N + L - 1) // L
    # first and last token of every segment of the first three groups, of every 40th
    # segment, and of the last two; the chunks on both sides of the first group edges
    segs = set(range(3 * G)) | set(range(0, nseg, 40)) | {nseg - 2, nseg - 1}
    pos = {N - 1}
    for s in segs:
        pos |= {s * L, min(N - 1, s * L + L - 1)}
    for grp in range(3):
        edge = (grp + 1) * G * L
        pos |= set(range(edge - L, min(N, edge + L), 16))
    rows = np.asarray(sorted(pos), np.int64)
    ref = oracle.taylor_direct(q, k, v, n, 1.0, rows=rows)
    assert oracle.rel_err_rowwise(got[rows], ref) <= TOL["f32"]
    S, T = (x.cpu().numpy().astype(np.float64) for x in rsp.state_views(st, B, H, n))
    assert T[0, 0, 0] == N
    vs = v[0, 0].astype(np.float64).sum(0)
    assert np.abs(S[0, 0, 0] - vs).max() <= 1e-5 * np.abs(vs).max() + 1e-3
