"""GPU parity of the packings the pages compare, through the same kernels:
documents back to back (varlen), back to back with cu = [0, N] and only the
mask separating them (FlashMask article §6.7, ZeroPadding), zero-padded to
the longest document (Varlen-Packing document §3, the padded baseline), and
zero-padded with the padding masked by the interval.  Every layout is
compared with the oracle run on that same layout: integer plan bit-exact,
out within 2e-2 and lse within 1e-3 with -inf exactly where the oracle has
it; the real tokens of every layout also agree with each other.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from test_gpu_parity import check_plan_ints, compare_full, pv, run, say  # noqa: F401  (pv is a fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", W.PACKINGS)
@pytest.mark.parametrize("S", [0, -1])
def test_packing_small(pv, kind, S):
    w = W.packed_as(W.document_workload([100, 37, 300, 1], H=2, seed=11), kind)
    say("packing", kind, "N=%d B=%d S=%d" % (w.N, w.B, S))
    Br, Bc = pv.tile_config(torch.bfloat16, w.D)
    check_plan_ints(pv, w, Br, Bc, 3 if S else 0)
    out, lse = run(pv, w, max_kb_per_item=S)
    compare_full(w, out, lse, kind)


def test_packings_of_varlen_documents(pv):
    """The [128, 128, 4096] documents (2 heads, D = 128) in all four
    layouts, with the library's default choices (path and splitting) as the
    benchmark runs them."""
    base = W.make_config(2)
    outs = {}
    for kind in W.PACKINGS:
        w = W.packed_as(base, kind)
        say("packing", kind, "N=%d B=%d" % (w.N, w.B))
        out, lse = run(pv, w)
        compare_full(w, out, lse, kind)
        real = w.meta["real_rows"]
        outs[kind] = (out.float().cpu().numpy()[real], lse.cpu().numpy()[:, real])
    ro, rl = outs["varlen"]
    for kind, (o, l) in outs.items():
        e_o = float(np.max(np.abs(o - ro)))
        e_l = float(np.max(np.abs(l - rl)))
        say("  %s against varlen on real rows: max|dout|=%.3e max|dlse|=%.3e" % (kind, e_o, e_l))
        assert e_o <= 2e-2 and e_l <= 1e-3
