"""GPU tests of the fused path (one attention launch in which every
workgroup derives its own work items from cu_seqlens and the mask vectors
of its own q-tile row; split rows combined in split order by a second,
merge launch).

- the header and merge table the fused launch writes into the workspace:
  no plan listed, one merge entry per (q tile, head) with the split count of
  the oracle's work list;
- out / lse are within the parity bars of the fp64 oracle;
- the fused path and the plan-in-workspace path give identical bits (the
  same chunks, the same item code, split merge in split order);
- a workspace is reusable across calls and paths.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
LSE_TOL = 1e-3
BR, BC = 256, 64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def pv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_varlen_masked_amd as pv
    return pv


def dev_inputs(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    return t(w.q), t(w.k), t(w.v), cu, sv


def fused_ws(pv, w, S):
    lay = pv.workspace_layout(w.N, w.B, w.H, w.D, BR, BC, S, False)
    return lay, torch.zeros(lay.bytes, dtype=torch.uint8, device="cuda")


def run_fused(pv, w, S, ws=None):
    q, k, v, cu, sv = dev_inputs(w)
    assert pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal, S)
    if ws is None:
        _, ws = fused_ws(pv, w, S)
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S,
                           workspace=ws)
    torch.cuda.synchronize()
    return out, lse, ws


def run_planned(pv, w, S):
    q, k, v, cu, sv = dev_inputs(w)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16, max_kb_per_item=S)
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    return out, lse


def compare(w, out, lse, tag):
    oo, ol = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(ol)), "lse -inf pattern differs"
    fin = np.isfinite(ol)
    e_out = float(np.max(np.abs(o - oo))) if o.size else 0.0
    e_lse = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    say("  %s max|dout|=%.3e max|dlse|=%.3e" % (tag, e_out, e_lse))
    assert e_out <= OUT_TOL and e_lse <= LSE_TOL


def fused_table(w, S):
    """The fused path's merge table for workload w, from the documented rule:
    q tiles in order (sequences in order, q tiles in order); q tile (b, qt)
    owns ceil(U / S) slots (one when S = 0 or U <= S), U = its key blocks not
    past the causal diagonal (all of them without the causal flag); its entry
    r * H + h is (first slot, h, first row, end row, number of splits of the
    oracle's work list)."""
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, BC)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, BR, BC)
    nsplit = {}
    for it in O.worklist(cls, w.H, S):
        nsplit[(int(it[0]), int(it[2]))] = int(it[6])
    cu = w.cu_seqlens.astype(np.int64)
    rows, slot = [], 0
    for b in range(w.B):
        L = int(cu[b + 1] - cu[b])
        Tc = -(-L // BC)
        for qt in range(-(-L // BR)):
            U = min(Tc, -(-min((qt + 1) * BR, L) // BC)) if w.causal else Tc
            r0 = int(cu[b]) + qt * BR
            for h in range(w.H):
                rows.append([slot, h, r0, min(r0 + BR, int(cu[b + 1])), nsplit[(b, qt)], 0, 0, 0])
            slot += 1 if (S == 0 or U <= S) else -(-U // S)
    return np.array(rows, np.int64).reshape(-1, 8)


def check_header(pv, w, S, ws, lay):
    """Status 0, no plan listed (items, split-row list), and the merge table."""
    hdr = ws[:256].view(torch.int32).cpu().numpy()
    want = fused_table(w, S)
    assert hdr[0] == 0 and hdr[2] == 0 and hdr[3] == 0 and hdr[5] == 0
    if S == 0:
        return
    assert hdr[6] == len(want)
    got = ws[lay.off_merge:lay.off_merge + 32 * len(want)].view(torch.int32).view(-1, 8).cpu().numpy()
    assert np.array_equal(got.astype(np.int64), want)


def test_fused_path_selection(pv):
    w = W.make_config(2, with_qkv=False)
    bf = torch.bfloat16
    assert pv.fused_path(w.N, w.B, w.H, 128, bf, w.n_vec, w.causal)
    assert not pv.fused_path(w.N, w.B, w.H, 128, bf, w.n_vec, w.causal, flags=pv.FM_FLAG_NO_SKIP)
    assert not pv.fused_path(w.N, w.B, w.H, 128, bf, w.n_vec, w.causal, flags=pv.FM_FLAG_PLAN_READY)
    assert not pv.fused_path(w.N, w.B, w.H, 32, torch.float32, w.n_vec, w.causal)
    assert not pv.fused_path(16384, 20, 32, 128, bf, 1, True)          # SFT packing: too big
    assert not pv.fused_path(4096, 300, 1, 128, bf, 1, True)           # too many sequences
    assert not pv.fused_path(20000, 3, 1, 128, bf, 1, True)            # more than 16384 tokens


@pytest.mark.parametrize("S", [-1, 0, 3, 2, 1])
def test_fused_cfg2(pv, S):
    w = W.make_config(2)
    S_eff = pv.auto_split(w.N, w.B, w.H, torch.bfloat16, 128) if S < 0 else S
    say("fused cfg2 S", S, "->", S_eff)
    if not pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal, S_eff):
        assert S_eff == 1, "the headline workload must take the fused path"
        pytest.skip("split bound beyond the fused path")
    lay, ws = fused_ws(pv, w, S_eff)
    out, lse, _ = run_fused(pv, w, S_eff, ws)
    check_header(pv, w, S_eff, ws, lay)
    compare(w, out, lse, "fused cfg2 S=%d" % S_eff)
    o2, l2 = run_planned(pv, w, S_eff)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("seed", range(16))
def test_fused_random(pv, seed):
    rng = np.random.default_rng(1000 + seed)
    w = W.random_case(700 + seed, N_max=1500, H=int(rng.integers(1, 4)), D=128, dtype=W.BF16)
    S = int(rng.choice([0, 1, 2, 6]))
    if not pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal, S):
        pytest.skip("sizes outside the fused path")
    say("fused random", w.name, "N=%d B=%d H=%d causal=%d n_vec=%d S=%d" % (w.N, w.B, w.H, w.causal, w.n_vec, S))
    lay, ws = fused_ws(pv, w, S)
    out, lse, _ = run_fused(pv, w, S, ws)
    check_header(pv, w, S, ws, lay)
    compare(w, out, lse, "fused random")
    o2, l2 = run_planned(pv, w, S)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("k,N,H", [(3, 6000, 2), (4, 4000, 2), (5, 4000, 1)])
def test_fused_reduced_configs(pv, k, N, H):
    w = W.make_config(k, N=N, H=H)
    for S in (0, 3):
        if not pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal, S):
            continue
        say("fused reduced cfg", k, w.N, w.H, w.B, "S", S)
        lay, ws = fused_ws(pv, w, S)
        out, lse, _ = run_fused(pv, w, S, ws)
        check_header(pv, w, S, ws, lay)
        compare(w, out, lse, "fused cfg%d S=%d" % (k, S))


def test_workspace_reuse_across_paths(pv):
    """One workspace serves fused, planned and fused calls again with
    identical results: the planner lists the oracle's split rows for the
    merge (one entry per split row and head), the fused call keeps its own
    table; a ready-plan call right after a fused call finds no plan and
    writes nothing."""
    w = W.make_config(2)
    S = 2
    lay, ws = fused_ws(pv, w, S)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, BC)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, BR, BC)
    oitems = O.worklist(cls, w.H, S)
    want = sorted((int(r[0]), int(r[2]), int(r[1])) for r in oitems if r[5] == 0 and r[6] > 1)

    def merge_rows():
        n = int(ws[20:24].view(torch.int32).item())
        ent = ws[lay.off_merge:lay.off_merge + 32 * n].view(torch.int32).view(n, 8).cpu().numpy()
        cu = w.cu_seqlens.astype(np.int64)
        got = []
        for e in ent:   # (sequence, q tile, head) from the entry's first row
            b = int(np.searchsorted(cu, e[2], side="right") - 1)
            got.append((b, int((e[2] - cu[b]) // BR), int(e[1])))
            assert e[3] == min(e[2] + BR, cu[b + 1]) and e[4] > 1 and np.all(e[5:] == 0)
        return sorted(got)

    o1, l1, _ = run_fused(pv, w, S, ws)
    check_header(pv, w, S, ws, lay)
    q, k, v, cu, sv = dev_inputs(w)
    out = torch.full_like(o1, 3.0)
    lse = torch.full_like(l1, 3.0)
    pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S, workspace=ws,
                flags=pv.FM_FLAG_PLAN_READY, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0).item() and torch.all(lse == 3.0).item()
    pv.build_plan_into(pv.Plan(ws, lay, w.N, w.B, w.H, w.D, torch.bfloat16, w.causal, w.n_vec, S), cu, sv)
    assert merge_rows() == want
    o2, l2 = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S,
                         workspace=ws, flags=pv.FM_FLAG_PLAN_READY)
    torch.cuda.synchronize()
    o3, l3, _ = run_fused(pv, w, S, ws)
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o1, o) and torch.equal(l1, l)
