"""GPU parity of attention dropout (forward and backward) against the fp64
oracle with the same Philox4x32-10 mask (FlashMask article §3.4: the op's
dropout attribute and seed_offset input; the counter layout is this
library's: key = seed, counter = (row, (key - sequence start) >> 4, head,
offset), one byte per pair, dropped below t = round(256 p)).

Bars: lse within 1e-3 (it is the undropped normaliser), gradients within
2e-2 + 1e-2 * max |ref| as without dropout, and out within
2e-2 + 2^-8 |ref| element by element: a kept value is scaled by
256 / (256 - t), so a dropped-out row can leave the range of V that the
plain 2e-2 bar was set for, and the bf16 store of such a value alone may
be off by 2^-8 of it.  The keep mask itself is checked bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def pv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_masked_amd as pv
    return pv


def dev(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    return t(w.q), t(w.k), t(w.v), cu, sv


def cases():
    return [("docs", W.document_workload([100, 37, 300, 1], H=2, seed=31)),
            ("random", W.random_case(811, N_max=300, H=2, D=128, dtype=W.BF16, allow_empty=True)),
            ("noncausal", W.make_config(5, N=3000, H=1))]


@pytest.mark.parametrize("idx", range(3))
@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("S", [0, -1])
def test_dropout_forward(pv, idx, p, S):
    name, w = cases()[idx]
    seed, off = 0x1234_5678_9ABC, 77 + idx
    q, k, v, cu, sv = dev(w)
    say("dropout fwd", name, "N=%d p=%g S=%d" % (w.N, p, S))
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S,
                           dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    oo, ol = O.attention_dropout(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, p, seed, off)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ol))
    fin = np.isfinite(ol)
    err = np.abs(o - oo)
    e_l = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    at = np.unravel_index(np.argmax(err), o.shape)
    small = np.abs(oo) <= 2.0
    e_small = float(np.max(err[small], initial=0.0))
    say("  max|dout|=%.3e at %s (ref %.4f), max|dout| where |ref| <= 2: %.3e, max|dlse|=%.3e"
        % (float(err[at]), at, oo[at], e_small, e_l))
    # the plain bar wherever |ref| <= 2 (the range of the inputs' softmax
    # averages); above it the bf16 store of the inflated kept values adds up
    # to 2^-8 of the value
    assert e_small <= 2e-2
    assert np.all(err <= 2e-2 + 2.0 ** -8 * np.abs(oo)) and e_l <= 1e-3


@pytest.mark.parametrize("idx", range(3))
def test_dropout_backward(pv, idx):
    name, w = cases()[idx]
    p, seed, off = 0.25, 987654321, 5
    q, k, v, cu, sv = dev(w)
    g = np.random.default_rng(idx).standard_normal(w.q.shape, dtype=np.float32)
    g = torch.from_numpy(g).to(torch.bfloat16)
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), dropout_p=p, seed=seed, offset=off)
    grads = pv.attn_bwd(q, k, v, out, lse, g.cuda(), cu, sv, w.n_vec, w.causal, float(w.scale),
                        dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    ref = O.attention_bwd_dropout(w.q, w.k, w.v, g.float().numpy(), w.cu_seqlens, w.startend, w.n_vec, w.causal,
                                  w.scale, p, seed, off)
    say("dropout bwd", name, "N=%d" % w.N)
    for nm, a, r in zip(("dq", "dk", "dv"), grads, ref):
        a = a.float().cpu().numpy()
        err, mx = float(np.max(np.abs(a - r))), float(np.max(np.abs(r)))
        say("  %s max|err|=%.3e max|ref|=%.3e" % (nm, err, mx))
        assert err <= 2e-2 + 1e-2 * mx


@pytest.mark.parametrize("idx", range(3))
def test_dropout_backward_two_streams(pv, idx):
    """fm_attn_bwd_dropout_streams: the dQ launches on a second stream give
    the one-stream call's bits, and everything is ordered before the next
    work on the caller's stream (the gradients are read there)."""
    name, w = cases()[idx]
    p, seed, off = 0.25, 987654321, 5
    q, k, v, cu, sv = dev(w)
    g = torch.from_numpy(np.random.default_rng(idx).standard_normal(w.q.shape, dtype=np.float32))
    g = g.to(torch.bfloat16).cuda()
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), dropout_p=p, seed=seed, offset=off)
    one = pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale),
                      dropout_p=p, seed=seed, offset=off)
    side = torch.cuda.Stream()
    two = pv.attn_bwd(q, k, v, out, lse, g, cu, sv, w.n_vec, w.causal, float(w.scale),
                      dropout_p=p, seed=seed, offset=off, dq_stream=side)
    copies = [t.clone() for t in two]   # on the caller's stream, after the join
    torch.cuda.synchronize()
    say("dropout bwd two streams", name, "N=%d" % w.N)
    for nm, a, b in zip(("dq", "dk", "dv"), one, copies):
        assert torch.equal(a, b), nm


@pytest.mark.parametrize("case", ["docs", "random_causal", "random_intervals"])
def test_dropout_keep_mask_exact(pv, case):
    """The keep mask itself, bit for bit: with q = 0 every visible key gets
    the same weight, and with v_j the unit vector of column j - s (every
    sequence at most D = 128 long) out[i, c] is nonzero exactly when key
    s + c is visible from row i and kept."""
    if case == "docs":
        w = W.document_workload([128, 50, 1, 97, 128], H=2, seed=3)
    else:
        w = W.random_case(4242 if case == "random_causal" else 4243, N_max=128, H=2, D=128, dtype=W.BF16,
                          causal=(case == "random_causal"))
    N, H, D = w.N, w.H, w.D
    cu = w.cu_seqlens.astype(np.int64)
    qz = np.zeros((N, H, D), np.float32)
    one = np.zeros((N, H, D), np.float32)
    for b in range(len(cu) - 1):
        for j in range(cu[b], cu[b + 1]):
            one[j, :, j - cu[b]] = 1.0
    w.q, w.k, w.v = qz, qz.copy(), one
    p, seed, off = 0.4, 0xDEADBEEF_0BADF00D, 123456789
    q, k, v, cucu, sv = dev(w)
    out = pv.attn_fwd(q, k, v, cucu, sv, w.n_vec, w.causal, float(w.scale), dropout_p=p, seed=seed, offset=off)[0]
    torch.cuda.synchronize()
    got = out.float().cpu().numpy() != 0
    t = O.dropout_threshold(p)
    vecs = O.fill_vectors(w.startend, w.n_vec, w.causal, N)
    want = np.zeros((N, H, D), bool)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        rows, cols = np.arange(s, e), np.arange(s, e)
        vis = ~O.element_mask(rows, cols, vecs, w.causal)
        for h in range(H):
            want[s:e, h, :e - s] = vis & O.dropout_keep(rows, cols, s, h, seed, off, t)
    bad = np.argwhere(got != want)
    say("keep mask", case, "N=%d kept=%d mismatches=%d" % (N, int(want.sum()), len(bad)), bad[:8].tolist())
    assert len(bad) == 0


def test_dropout_reproducible(pv):
    """Same (seed, offset): the same bits; another offset: another mask;
    p below 1/512 rounds to no dropout (the plain forward's bits)."""
    w = W.document_workload([300, 200], H=2, seed=9)
    q, k, v, cu, sv = dev(w)
    run = lambda **kw: pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=0, **kw)[0]
    a = run(dropout_p=0.3, seed=11, offset=1)
    b = run(dropout_p=0.3, seed=11, offset=1)
    c = run(dropout_p=0.3, seed=11, offset=2)
    d = run(dropout_p=0.001)
    e = run()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.equal(a, c) and torch.equal(d, e)
