"""GPU parity of the backward (dq, dk, dv) through the C ABI against the fp64
oracle's gradients, on the same bf16 inputs and output gradient.

The forward's out and lse come from the library (the backward's inputs);
the oracle recomputes everything from q, k, v and dout.  Bar: max |err| <=
ATOL + RTOL * max |ref| per tensor (bf16 outputs and bf16 P, dS operands
of the products), and exact zeros where no pair contributes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

ATOL = 2e-2
RTOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def pv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_masked_amd as pv
    return pv


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def run_bwd(pv, w, seed=0):
    dt = torch.bfloat16
    q, k, v = (bf16(x).cuda() for x in (w.q, w.k, w.v))
    g = bf16(np.random.default_rng(seed + 77).standard_normal(w.q.shape, dtype=np.float32))
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale))
    dq, dk, dv = pv.attn_bwd(q, k, v, out, lse, g.cuda(), cu, sv, w.n_vec, w.causal, float(w.scale))
    torch.cuda.synchronize()
    return (dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()), g.float().numpy()


def no_pairs(w):
    """Rows that attend no key and keys no row attends (their gradients are
    exactly zero: no pair contributes)."""
    vecs = O.fill_vectors(w.startend, w.n_vec, w.causal, w.N)
    cu = w.cu_seqlens.astype(np.int64)
    row_empty = np.ones(w.N, bool)
    col_empty = np.ones(w.N, bool)
    for b in range(w.B):
        s, e = int(cu[b]), int(cu[b + 1])
        if e > s:
            ok = ~O.element_mask(np.arange(s, e), np.arange(s, e), vecs, w.causal)
            row_empty[s:e] = ~ok.any(axis=1)
            col_empty[s:e] = ~ok.any(axis=0)
    return row_empty, col_empty


def compare(w, got, g, tag=""):
    ref = O.attention_bwd(w.q, w.k, w.v, g, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    row_empty, col_empty = no_pairs(w)
    for nm, a, r, z in zip(("dq", "dk", "dv"), got, ref, (row_empty, col_empty, col_empty)):
        err = float(np.max(np.abs(a - r))) if a.size else 0.0
        mx = float(np.max(np.abs(r))) if r.size else 0.0
        say("  %s %s: max|err|=%.3e max|ref|=%.3e" % (tag, nm, err, mx))
        assert np.all(np.isfinite(a))
        assert err <= ATOL + RTOL * mx, (nm, err, mx)
        assert np.all(a[z] == 0.0), nm
    return ref


@pytest.mark.parametrize("seed", range(6))
def test_bwd_random(pv, seed):
    w = W.random_case(700 + seed, N_max=300, H=2, D=128, dtype=W.BF16, allow_empty=True)
    say("bwd random", seed, "N=%d B=%d causal=%d n_vec=%d" % (w.N, w.B, w.causal, w.n_vec))
    got, g = run_bwd(pv, w, seed)
    compare(w, got, g, "random %d" % seed)


@pytest.mark.parametrize("lens", [[100, 37, 300, 1], [64, 128, 65]])
def test_bwd_documents(pv, lens):
    w = W.document_workload(lens, H=2, seed=21)
    say("bwd documents", lens)
    got, g = run_bwd(pv, w)
    compare(w, got, g, "docs")


@pytest.mark.parametrize("causal,n_vec", [(True, 1), (True, 2), (False, 2), (False, 4)])
def test_bwd_extreme_endpoints(pv, causal, n_vec):
    """Endpoints at the int32 limits and past the token axis on documents of
    several q tiles: dq (whose kernel builds per-key row masks relative to a
    wave's first row) agrees with the oracle as dk and dv do."""
    w = W.extreme_interval_workload([700, 300, 1100], causal, n_vec, H=2, seed=31 + n_vec)
    say("bwd extreme endpoints", w.name)
    got, g = run_bwd(pv, w)
    compare(w, got, g, w.name)


def test_bwd_varlen_workload(pv):
    w = W.make_config(2)
    say("bwd varlen workload N=%d" % w.N)
    got, g = run_bwd(pv, w)
    compare(w, got, g, "cfg2")


@pytest.mark.parametrize("k,N,H", [(3, 3000, 2), (4, 3000, 1), (5, 9000, 1)])
def test_bwd_reduced_configs(pv, k, N, H):
    w = W.make_config(k, N=N, H=H)
    say("bwd config", k, "N=%d H=%d" % (w.N, w.H))
    got, g = run_bwd(pv, w)
    compare(w, got, g, "cfg%d" % k)


def test_bwd_deterministic(pv):
    w = W.document_workload([300, 700], H=2, seed=5)
    a, _ = run_bwd(pv, w)
    b, _ = run_bwd(pv, w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def compare_heads(w, got, g, heads, tag):
    """dq, dk, dv of the given heads against the full oracle (heads are
    independent: each is one single-head problem on the same mask)."""
    for h in heads:
        w1 = W.Workload(w.name + "_h%d" % h, w.N, 1, w.D, w.dtype, w.causal, w.n_vec, w.cu_seqlens, w.startend,
                        w.scale, w.q[:, h:h + 1], w.k[:, h:h + 1], w.v[:, h:h + 1])
        compare(w1, tuple(x[:, h:h + 1] for x in got), g[:, h:h + 1], "%s head %d" % (tag, h))


def test_bwd_sft_full_one_head(pv):
    """SFT packing workload at full size (16384 tokens, 32 heads): dq, dk,
    dv of heads 0 and H - 1 against the full oracle."""
    w = W.make_config(3)
    say("bwd SFT full N=%d H=%d" % (w.N, w.H))
    got, g = run_bwd(pv, w)
    compare_heads(w, got, g, (0, w.H - 1), "cfg3")


def test_bwd_shared_question_full_heads(pv):
    """Shared-question workload at full size (32768 tokens, 32 heads; each
    answer attends to its prompt and itself, not to its siblings): dq, dk,
    dv of heads 0 and H - 1 against the full oracle."""
    w = W.make_config(4)
    say("bwd shared-question full N=%d H=%d" % (w.N, w.H))
    got, g = run_bwd(pv, w)
    compare_heads(w, got, g, (0, w.H - 1), "cfg4")


def test_bwd_short_documents_unchunked(pv):
    """Documents of 1 to 320 tokens filling 16384 tokens at 32 heads, enough
    work that neither launch is cut into chunks: key spans and query tiles
    that visit one to five tiles, so the phase-shifted loops' first and last
    steps (and spans of a single step) run at the full-size launch shapes.
    Heads 0 and H - 1 against the oracle."""
    pattern = [1, 64, 65, 128, 129, 192, 255, 256, 257, 320]
    lens = []
    while sum(lens) + 320 < 16384:
        lens.append(pattern[len(lens) % len(pattern)])
    lens.append(16384 - sum(lens))
    w = W.document_workload(lens, H=32, seed=99)
    say("bwd short documents B=%d N=%d H=%d" % (w.B, w.N, w.H))
    got, g = run_bwd(pv, w)
    compare_heads(w, got, g, (0, w.H - 1), "short docs")


def test_bwd_prefix_window_full_sampled(pv):
    """Prefix-LM + window workload at full size (131072 tokens, 8 heads):
    sampled dq rows against the oracle one by one, and for every sequence and
    head two identities of the exact gradients: sum_j dk_j = 0 (softmax is
    unchanged when all keys move by one vector) and sum_j dv_j = sum of dout
    over the rows that attend (each row's P sums to 1)."""
    w = W.make_config(5)
    say("bwd prefix-window full N=%d H=%d" % (w.N, w.H))
    (dq, dk, dv), g = run_bwd(pv, w)
    rng = np.random.default_rng(3)
    cu = w.cu_seqlens.astype(np.int64)
    rows = sorted(set(int(x) for x in rng.integers(0, w.N, 48)) | {int(cu[b]) for b in range(w.B)} |
                  {int(cu[b + 1]) - 1 for b in range(w.B)})
    heads = [int(x) for x in rng.integers(0, w.H, len(rows))]
    ref = O.attention_bwd_rows(w.q, w.k, w.v, g, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, rows, heads)
    got = np.stack([dq[r, h] for r, h in zip(rows, heads)])
    err, mx = float(np.max(np.abs(got - ref))), float(np.max(np.abs(ref)))
    say("  sampled dq rows: %d, max|err|=%.3e max|ref|=%.3e" % (len(rows), err, mx))
    assert err <= ATOL + RTOL * mx
    row_empty, _ = no_pairs_rows(w)
    for b in range(w.B):
        s, e = int(cu[b]), int(cu[b + 1])
        sk = dk[s:e].astype(np.float64).sum(axis=0)
        sv_ = dv[s:e].astype(np.float64).sum(axis=0)
        gs = g[s:e][~row_empty[s:e]].astype(np.float64).sum(axis=0)
        ek = float(np.max(np.abs(sk)) / max(1.0, float(np.abs(dk[s:e]).sum(axis=0).max())))
        ev = float(np.max(np.abs(sv_ - gs)) / max(1.0, float(np.abs(dv[s:e]).sum(axis=0).max())))
        say("  seq %d (L=%d): |sum dk| / sum|dk| = %.2e, |sum dv - sum dout| / sum|dv| = %.2e" % (b, e - s, ek, ev))
        assert ek <= 1e-2 and ev <= 1e-2


def no_pairs_rows(w):
    """Rows with no allowed key, per token (any size: one pass per row block)."""
    vecs = O.fill_vectors(w.startend, w.n_vec, w.causal, w.N)
    cu = w.cu_seqlens.astype(np.int64)
    empty = np.ones(w.N, bool)
    for b in range(w.B):
        s, e = int(cu[b]), int(cu[b + 1])
        cols = np.arange(s, e)
        for r0 in range(s, e, 1024):
            rr = np.arange(r0, min(r0 + 1024, e))
            empty[rr] = O.element_mask(rr, cols, vecs, w.causal).all(axis=1)
    return empty, None


def test_bwd_bad_cu_and_empty(pv):
    """Decreasing cu_seqlens: the preprocessing sets the status word and the
    backward writes nothing (dq, dk, dv keep their contents).  N = 0: no
    work, no error."""
    w = W.document_workload([100, 100, 56], H=2, seed=8)
    q, k, v = (bf16(x).cuda() for x in (w.q, w.k, w.v))
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    cu = torch.tensor([0, 150, 100, w.N], dtype=torch.int32, device="cuda")
    lse = torch.zeros(w.H, w.N, dtype=torch.float32, device="cuda")
    ws = torch.zeros(pv.bwd_workspace_size(w.N, 3, w.H, w.D, torch.bfloat16), dtype=torch.uint8, device="cuda")
    grads = [torch.full_like(q, 7.0) for _ in range(3)]
    pv.attn_bwd(q, k, v, q, lse, q, cu, sv, w.n_vec, w.causal, workspace=ws, dq=grads[0], dk=grads[1], dv=grads[2])
    assert pv.read_status(ws) & pv.FM_STATUS_ORDER
    for t in grads:
        assert torch.all(t == 7.0).item()
    e = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(2, dtype=torch.int32, device="cuda")
    dq, dk, dv = pv.attn_bwd(e, e, e, e, torch.empty(2, 0, device="cuda"), e, z,
                             torch.empty(1, 0, dtype=torch.int32, device="cuda"), 1, True)
    torch.cuda.synchronize()
    assert dq.shape == (0, 2, 128)


@pytest.mark.parametrize("two_streams", [False, True])
def test_bwd_stream_order(pv, two_streams):
    """Work enqueued after the backward on a (non-default) caller stream
    sees the finished gradients: on one stream, and with the dQ launches on
    a second stream of the caller's (fm_attn_bwd_streams: forked after Delta,
    joined back with the caller's events).  Two streams each run the
    backward and copy dq, dk, dv right after it with no host
    synchronisation; every copy must equal a fully synchronised run, bit for
    bit, three times over."""
    w = W.document_workload([300, 700, 1200], H=2, seed=6)
    ref, _ = run_bwd(pv, w)
    q, k, v = (bf16(x).cuda() for x in (w.q, w.k, w.v))
    g = bf16(np.random.default_rng(77).standard_normal(w.q.shape, dtype=np.float32)).cuda()
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    side = [torch.cuda.Stream(), torch.cuda.Stream()] if two_streams else [None, None]
    copies = []
    for rep in range(3):
        for st, sd in zip(streams, side):
            with torch.cuda.stream(st):
                grads = pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale), dq_stream=sd)
                copies.append([t.clone() for t in grads])
    torch.cuda.synchronize()
    say("stream order (two streams: %s): %d copies" % (two_streams, len(copies)))
    for c in copies:
        for x, y in zip(c, ref):
            assert np.array_equal(x.float().cpu().numpy(), y)
