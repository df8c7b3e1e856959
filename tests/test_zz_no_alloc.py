"""GPU test of fm_attn_fwd_noalloc, the forward that allocates nothing (its
workspace is the library's own per-device array): through the C ABI its
out and lse equal fm_attn_fwd's with a caller workspace on the same inputs,
call after call with the second input smaller than the first (the array
keeps the previous call's contents), on the fused path with split rows, the
planned path and the fp32 path; both stay within the oracle's bars."""
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
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    return t(w.q), t(w.k), t(w.v), cu, sv


def one(pv, w, **kw):
    q, k, v, cu, sv = dev(w)
    ref_out, ref_lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), **kw)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.H, w.N), float("nan"), dtype=torch.float32, device=q.device)
    pv.attn_fwd_noalloc(q, k, v, cu, sv, w.n_vec, w.causal, out, lse, float(w.scale), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), w.name
    oo, ol = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(ol))
    fin = np.isfinite(ol)
    e_out = float(np.max(np.abs(o - oo)))
    e_lse = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    say("  %s %s: identical to the workspace call; max|dout|=%.3e max|dlse|=%.3e" % (w.name, kw, e_out, e_lse))
    assert e_out <= 2e-2 and e_lse <= 1e-3


def test_noalloc_matches_workspace_call(pv):
    # the varlen [128, 128, 4096] workload (fused path, split rows and the
    # merge), then a smaller one, then the planned path (NO_SKIP forces it)
    # and the page example in fp32
    one(pv, W.make_config(2))
    one(pv, W.document_workload([300, 200, 77], H=2, seed=9))
    one(pv, W.make_config(5, N=3000, H=1), max_kb_per_item=0, flags=pv.FM_FLAG_NO_SKIP)
    one(pv, W.make_config(1), block_q=4, block_k=4)


def test_noalloc_rejects_too_large(pv):
    w = W.make_config(3, with_qkv=False)
    q = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    need = pv.workspace_size(w.N, w.B, w.H, 128, torch.bfloat16, 6)
    assert need > pv.NOALLOC_SCRATCH_BYTES
    rc = pv._lib.fm_attn_fwd_noalloc(pv._ptr(q), pv._ptr(q), pv._ptr(q), pv.FM_BF16, w.N, w.H, 128, pv._ptr(q), w.B,
                                     pv._ptr(q), w.n_vec, 1, pv.ctypes.c_float(0.1), pv._ptr(q), pv._ptr(q), 0, 0, 6,
                                     0, pv._stream())
    assert rc == pv.FM_E_WORKSPACE and str(need) in pv._lib.fm_last_error().decode()
