"""GPU parity of the fused rotary embedding (q and k in place, positions
restarting per packed sample) against the fp64 oracle on the same inputs.

Bar: the kernel computes in fp32 and rounds once to the storage type, so
|got - ref| <= 2^-7 |ref| + 1e-5 for bf16 (one bf16 ulp: the rounding is at
most half of it, 2^-8 relative at the bottom of a binade, plus the fp32
products) and <= 1e-6 |ref| + 1e-6 for fp32.  Rows whose position falls
outside the tables must be left bit-identical, with FM_STATUS_POS set.
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


def lengths(seed, N):
    rng = np.random.default_rng(seed)
    cuts = sorted(int(x) for x in rng.integers(0, N, size=int(rng.integers(0, 6)), endpoint=True))
    return np.array([0] + cuts + [N], np.int64)


def check(got, ref, dt):
    err = np.abs(got.astype(np.float64) - ref)
    bound = (2.0 ** -7 * np.abs(ref) + 1e-5) if dt == torch.bfloat16 else (1e-6 * np.abs(ref) + 1e-6)
    say("  max|err| = %.3e (worst err / bound = %.3f)" % (err.max(), float((err / bound).max())))
    assert np.all(err <= bound)


def run(pv, x_q, x_k, cu, cos, sin, dt, inverse=False):
    q = torch.from_numpy(x_q).to(dt).cuda() if x_q is not None else None
    k = torch.from_numpy(x_k).to(dt).cuda() if x_k is not None else None
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    pv.rope_qk_(q, k, torch.from_numpy(cu.astype(np.int32)).cuda(), torch.from_numpy(cos).cuda(),
                torch.from_numpy(sin).cuda(), inverse=inverse, status=st)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float().cpu().numpy()
    return f(q), f(k), int(st.item())


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("seed", range(3))
def test_rope_random(pv, dt, D, seed):
    if dt == torch.bfloat16 and D < 16:
        pytest.skip("bf16 needs D % 16 == 0")
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 700))
    cu = lengths(seed, N)
    Hq, Hk = 4, 2
    q = rng.standard_normal((N, Hq, D), dtype=np.float32)
    k = rng.standard_normal((N, Hk, D), dtype=np.float32)
    q = torch.from_numpy(q).to(dt).float().numpy()   # the exact values the GPU holds
    k = torch.from_numpy(k).to(dt).float().numpy()
    cos, sin = W.rope_tables(N + 1, D)
    inverse = bool(seed % 2)
    say("rope N=%d B=%d D=%d dtype=%s inverse=%d" % (N, len(cu) - 1, D, dt, inverse))
    gq, gk, st = run(pv, q, k, cu, cos, sin, dt, inverse)
    assert st == 0
    check(gq, O.rope(q, cu, cos, sin, inverse), dt)
    check(gk, O.rope(k, cu, cos, sin, inverse), dt)


def test_rope_one_tensor_and_status(pv):
    """k alone; positions past the tables leave their rows unchanged and set
    FM_STATUS_POS, the others are rotated."""
    rng = np.random.default_rng(9)
    D, N = 128, 300
    cu = np.array([0, 40, 300])
    k = torch.from_numpy(rng.standard_normal((N, 3, D), dtype=np.float32)).to(torch.bfloat16).float().numpy()
    cos, sin = W.rope_tables(100, D)   # the second sample (260 rows) runs past position 99
    _, gk, st = run(pv, None, k, cu, cos, sin, torch.bfloat16)
    assert st == pv.FM_STATUS_POS
    ok = np.ones(N, bool)
    ok[40 + 100:] = False
    assert np.array_equal(gk[~ok], k[~ok])
    check(gk[ok], O.rope(k[ok], [0, 40, 140], cos, sin), torch.bfloat16)


def test_rope_sft_full(pv):
    """The SFT packing workload's q and k (16384 tokens, 32 heads, D = 128)
    at full size, forward then inverse."""
    w = W.make_config(3)
    cos, sin = W.rope_tables(int(w.lengths.max()), w.D)
    say("rope SFT full N=%d H=%d" % (w.N, w.H))
    gq, gk, st = run(pv, w.q, w.k, w.cu_seqlens, cos, sin, torch.bfloat16)
    assert st == 0
    check(gq, O.rope(w.q, w.cu_seqlens, cos, sin), torch.bfloat16)
    check(gk, O.rope(w.k, w.cu_seqlens, cos, sin), torch.bfloat16)
    bq, _, st = run(pv, gq, None, w.cu_seqlens, cos, sin, torch.bfloat16, inverse=True)
    check(bq, O.rope(gq, w.cu_seqlens, cos, sin, inverse=True), torch.bfloat16)


def test_rope_empty(pv):
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    cos, sin = (torch.from_numpy(t).cuda() for t in W.rope_tables(4, 64))
    pv.rope_qk_(e, e, torch.zeros(2, dtype=torch.int32, device="cuda"), cos, sin)
    torch.cuda.synchronize()
