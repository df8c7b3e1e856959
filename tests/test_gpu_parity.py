"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Integer results (extrema, kb offsets, tile classes, class counts, work
items) must be bit-exact.  Floating point: max |out - out_ref| <= 2e-2 and
max |lse - lse_ref| <= 1e-3, with -inf exactly where the oracle has -inf.
bf16 inputs are compared against the oracle run on the same bf16 values
widened to fp64.
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
    dt = torch.bfloat16 if w.dtype == W.BF16 else torch.float32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda() if a is not None else None
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    sv = torch.from_numpy(np.ascontiguousarray(w.startend.astype(np.int32))).cuda()
    return t(w.q), t(w.k), t(w.v), cu, sv


def oracle_plan(w, Br, Bc, H, S):
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, Bc)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, Br, Bc)
    return kb_off, ext, cls, O.class_counts(cls), O.worklist(cls, H, S)


def check_plan_ints(pv, w, Br, Bc, S, H=None):
    H = w.H if H is None else H
    say("plan ints:", w.name, "N=%d B=%d Br=%d Bc=%d S=%d H=%d" % (w.N, w.B, Br, Bc, S, H))
    _, _, _, cu, sv = dev_inputs(w)
    kb_off, ext, status = pv.preprocess_mask(sv, w.n_vec, w.causal, cu, w.N, Bc)
    okb, oext, ocls, ocnt, oitems = oracle_plan(w, Br, Bc, H, S)
    assert status == 0
    assert np.array_equal(kb_off.cpu().numpy(), okb)
    assert np.array_equal(ext.cpu().numpy().reshape(-1, 8), oext.reshape(-1, 8))
    wl = pv.build_worklist(cu, w.N, H, Br, Bc, kb_off, ext, status, w.causal, S, want_class_map=True)
    assert wl["class_counts"].cpu().tolist() == ocnt.tolist()
    flat = np.concatenate([c.reshape(-1) for c in ocls]) if ocls else np.zeros(0, np.int8)
    assert np.array_equal(wl["tile_class"][:flat.size].cpu().numpy().astype(np.int8), flat)
    items = wl["items"].cpu().numpy()
    assert items.shape == (oitems.shape[0], 16), (items.shape, oitems.shape)
    assert np.array_equal(items[:, :8], oitems)
    # derived words: sequence bounds, extrema base, slot of split 0
    cu = w.cu_seqlens.astype(np.int64)
    b = items[:, 0]
    assert np.array_equal(items[:, 8], cu[b]) and np.array_equal(items[:, 9], cu[b + 1])
    assert np.array_equal(items[:, 10], okb[b]) and np.all(items[:, 12:] == 0)
    key = {}
    for r in items.tolist():     # split s of one (seq, q tile) sits at slot split0_slot + s
        key.setdefault((r[0], r[2]), set()).add(r[11])
    assert all(len(v) == 1 for v in key.values())
    slots = sorted(v.pop() for v in key.values())
    assert len(set(slots)) == len(slots)
    return items[:, :8]


def run(pv, w, **kw):
    q, k, v, cu, sv = dev_inputs(w)
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), **kw)
    torch.cuda.synchronize()
    return out, lse


def compare_full(w, out, lse, tag=""):
    oo, ol = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(ol)), "lse -inf pattern differs"
    fin = np.isfinite(ol)
    assert np.all(np.isfinite(l[fin]))
    e_out = float(np.max(np.abs(o - oo))) if o.size else 0.0
    e_lse = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    say("  %s max|dout|=%.3e max|dlse|=%.3e" % (tag, e_out, e_lse))
    assert e_out <= OUT_TOL and e_lse <= LSE_TOL
    return e_out, e_lse


def compare_rows(w, out, lse, n_rows=64, seed=0):
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens.astype(np.int64)
    rows = set()
    for b in range(w.B):   # first / last rows of sequences and tile edges
        s, e = int(cu[b]), int(cu[b + 1])
        for r in (s, s + 1, e - 1, s + 127, s + 128, e - 2):
            if s <= r < e:
                rows.add(r)
    rows = sorted(rows)
    rows = list(rng.choice(rows, size=min(len(rows), n_rows // 2), replace=False))
    rows += list(rng.integers(0, w.N, size=n_rows - len(rows)))
    heads = list(rng.integers(0, w.H, size=len(rows)))
    oo, ol = O.attention_rows(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale,
                              [int(r) for r in rows], [int(h) for h in heads])
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    go = np.stack([o[r, h] for r, h in zip(rows, heads)]).astype(np.float64)
    gl = np.array([l[h, r] for r, h in zip(rows, heads)], np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(ol))
    fin = np.isfinite(ol)
    e_out = float(np.max(np.abs(go - oo)))
    e_lse = float(np.max(np.abs(gl[fin] - ol[fin]), initial=0.0))
    say("  sampled %d rows: max|dout|=%.3e max|dlse|=%.3e" % (len(rows), e_out, e_lse))
    assert e_out <= OUT_TOL and e_lse <= LSE_TOL


# ---------------------------------------------------------------- integers
@pytest.mark.parametrize("S", [0, 1, 2])
def test_page_example_plan(pv, S):
    w = W.make_config(1, with_qkv=False)
    items = check_plan_ints(pv, w, 4, 4, S)
    if S == 0:
        assert len(items) == 4


@pytest.mark.parametrize("k", [2, 3, 4, 5])
@pytest.mark.parametrize("S", [0, 4, 3])
def test_config_plan_ints(pv, k, S):
    w = W.make_config(k, with_qkv=False)
    items = check_plan_ints(pv, w, 128, 64, S)
    if k == 2 and S == 0:
        assert len(items) == 68


@pytest.mark.parametrize("seed", range(24))
def test_random_plan_ints(pv, seed):
    rng = np.random.default_rng(seed)
    w = W.random_case(seed, N_max=80, with_qkv=False)
    Br, Bc = int(rng.integers(1, 10)), int(rng.integers(1, 10))
    S = int(rng.choice([0, 1, 2, 5]))
    check_plan_ints(pv, w, Br, Bc, S, H=int(rng.integers(1, 4)))


@pytest.mark.parametrize("k,S", [(1, 0), (2, 0), (2, 4), (3, 0), (4, 3), (5, 0)])
def test_fused_plan_matches_oracle(pv, k, S):
    """The plan path (the extrema launch, the tile-class launch with 16
    workgroups per sequence, then the sort) writes the same integers as the
    oracle into the workspace."""
    w = W.make_config(k, with_qkv=False)
    _, _, _, cu, sv = dev_inputs(w)
    dt = torch.float32 if w.dtype == W.F32 else torch.bfloat16
    Br, Bc = (4, 4) if k == 1 else (128, 64)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, dt, block_q=Br, block_k=Bc,
                         max_kb_per_item=S, want_class_map=True)
    hdr = plan.header()
    okb, oext, ocls, ocnt, oitems = oracle_plan(w, Br, Bc, w.H, S)
    assert hdr["status"] == 0 and hdr["n_kblocks"] == len(oext)
    assert np.array_equal(plan.kb_off().cpu().numpy(), okb)
    assert np.array_equal(plan.extrema(len(oext)).cpu().numpy(), oext)
    assert hdr["class_counts"] == ocnt.tolist()
    flat = np.concatenate([c.reshape(-1) for c in ocls])
    assert np.array_equal(plan.tile_class(flat.size).cpu().numpy().astype(np.int8), flat)
    assert hdr["n_items"] == len(oitems)
    assert np.array_equal(plan.items(len(oitems)).cpu().numpy()[:, :8], oitems)


# ----------------------------------------------------------------- fp32
@pytest.mark.parametrize("tiles", [(4, 4), (0, 0), (16, 8)])
def test_cfg1_fp32(pv, tiles):
    w = W.make_config(1)
    say("cfg1 fp32 tiles", tiles)
    out, lse = run(pv, w, block_q=tiles[0], block_k=tiles[1], max_kb_per_item=0)
    e_out, e_lse = compare_full(w, out, lse, "cfg1 fp32")
    assert e_out < 1e-5 and e_lse < 1e-5


@pytest.mark.parametrize("seed", range(8))
def test_random_fp32(pv, seed):
    rng = np.random.default_rng(seed)
    w = W.random_case(seed, N_max=150, H=2, D=int(rng.choice([32, 64, 128])))
    bq, bk = int(rng.integers(1, 65)), int(rng.integers(1, 65))
    say("random fp32", w.name, w.N, w.B, w.D, bq, bk)
    out, lse = run(pv, w, block_q=bq, block_k=bk, max_kb_per_item=0)
    compare_full(w, out, lse, "random fp32")


# ----------------------------------------------------------------- bf16
@pytest.mark.parametrize("S", [0, -1, 2])
def test_cfg2_bf16_full(pv, S):
    w = W.make_config(2)
    say("cfg2 bf16 S", S)
    out, lse = run(pv, w, max_kb_per_item=S)
    compare_full(w, out, lse, "cfg2")


@pytest.mark.parametrize("k,N,H", [(3, 6000, 2), (4, 6000, 2), (5, 12000, 1)])
def test_reduced_configs_full(pv, k, N, H):
    w = W.make_config(k, N=N, H=H)
    say("reduced cfg", k, w.N, w.H, w.B)
    out, lse = run(pv, w, max_kb_per_item=0)
    compare_full(w, out, lse, "cfg%d reduced" % k)
    out2, lse2 = run(pv, w, max_kb_per_item=3)
    compare_full(w, out2, lse2, "cfg%d reduced split3" % k)


# Heads compared on every row at full size: the first and the last (the
# prefix-LM workload, 131072 tokens, only head 0 to keep the oracle's time
# in bounds); every head is covered by the sampled rows.
FULL_HEADS = {3: [0, 31], 4: [0, 31], 5: [0]}


@pytest.mark.parametrize("k", [3, 4, 5])
def test_full_config(pv, k):
    """The full-size workloads through the default call (the path and split
    fm_attn_fwd chooses for them) and through the planned path with a plan
    built beforehand: both give the same bits, every row of the heads in
    FULL_HEADS matches the oracle (out <= 2e-2, lse <= 1e-3, -inf exactly
    where the oracle has it), and 64 sampled (row, head) pairs of all heads
    too."""
    from par_oracle import attention_heads
    w = W.make_config(k)
    fused = pv.fused_path(w.N, w.B, w.H, w.D, torch.bfloat16, w.n_vec, w.causal)
    say("full cfg", k, "N=%d H=%d B=%d fused=%d" % (w.N, w.H, w.B, fused))
    q, kk, v, cu, sv = dev_inputs(w)
    out, lse = pv.attn_fwd(q, kk, v, cu, sv, w.n_vec, w.causal, float(w.scale))
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16)
    out2, lse2 = pv.attn_fwd(q, kk, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    del q, kk, v, out2, lse2
    heads = FULL_HEADS[k]
    oo, ol = attention_heads(w, heads)
    o = out[:, heads].float().cpu().numpy().astype(np.float64)
    l = lse[heads].cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(ol)), "lse -inf pattern differs"
    fin = np.isfinite(ol)
    e_out = float(np.max(np.abs(o - oo)))
    e_lse = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    say("  heads %s, all %d rows: max|dout|=%.3e max|dlse|=%.3e" % (heads, w.N, e_out, e_lse))
    assert e_out <= OUT_TOL and e_lse <= LSE_TOL
    compare_rows(w, out, lse, n_rows=64, seed=k)


@pytest.mark.parametrize("k", [3, 4, 5])
@pytest.mark.parametrize("S", [0, 6])
def test_full_plan_ints_library_tiles(pv, k, S):
    """Extrema, classes, class counts and the work list of the full-size
    workloads at the tiles fm_attn_fwd runs (fm_get_tile_config: 256 x 64),
    bit-exact against the oracle, through the separate calls and through
    fm_build_plan's workspace; S = 0 is the split the library chooses for
    these sizes (fm_auto_split), S = 6 splits long rows."""
    w = W.make_config(k, with_qkv=False)
    Br, Bc = pv.tile_config(torch.bfloat16, 128)
    assert (Br, Bc) == (256, 64)
    assert pv.auto_split(w.N, w.B, w.H, torch.bfloat16, 128) == 0
    check_plan_ints(pv, w, Br, Bc, S)
    _, _, _, cu, sv = dev_inputs(w)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16, max_kb_per_item=S,
                         want_class_map=True)
    hdr = plan.header()
    okb, oext, ocls, ocnt, oitems = oracle_plan(w, Br, Bc, w.H, S)
    assert hdr["status"] == 0 and hdr["n_kblocks"] == len(oext)
    assert np.array_equal(plan.kb_off().cpu().numpy(), okb)
    assert np.array_equal(plan.extrema(len(oext)).cpu().numpy(), oext)
    assert hdr["class_counts"] == ocnt.tolist()
    flat = np.concatenate([c.reshape(-1) for c in ocls])
    assert np.array_equal(plan.tile_class(flat.size).cpu().numpy().astype(np.int8), flat)
    assert hdr["n_items"] == len(oitems)
    assert np.array_equal(plan.items(len(oitems)).cpu().numpy()[:, :8], oitems)


@pytest.mark.parametrize("seed", range(12))
def test_random_bf16(pv, seed):
    w = W.random_case(seed, N_max=700, H=2, D=128, dtype=W.BF16)
    say("random bf16", w.name, w.N, w.B, w.causal, w.n_vec)
    out, lse = run(pv, w, max_kb_per_item=0)
    compare_full(w, out, lse, "random bf16")
    out2, lse2 = run(pv, w, max_kb_per_item=1)
    compare_full(w, out2, lse2, "random bf16 split1")


@pytest.mark.parametrize("causal,n_vec", [(True, 1), (True, 2), (False, 2), (False, 4)])
def test_extreme_endpoints(pv, causal, n_vec):
    """Interval endpoints at the int32 limits and past the token axis
    (INT32_MIN, -1, N + 7, INT32_MAX; FlashMask article §2.1, §2.2: any
    half-open interval, start >= end empty) on documents of several q tiles,
    so that tiles of q tiles after the first are PARTIAL under them: the
    extrema, classes and work list bit-exact, out and lse within the bars on
    the fused path (split and unsplit) and on the planned path."""
    w = W.extreme_interval_workload([700, 300, 1100], causal, n_vec, H=2, seed=31 + n_vec)
    say("extreme endpoints", w.name)
    okb, oext, ocls, _, _ = oracle_plan(w, 256, 64, w.H, 0)
    assert int(w.startend.min()) == W.INT32_MIN or int(w.startend.max()) == W.INT32_MAX
    assert any((c[1:] == O.PARTIAL).any() for c in ocls if c.shape[0] > 1)
    for S in (0, 2):
        check_plan_ints(pv, w, 256, 64, S)
        out, lse = run(pv, w, max_kb_per_item=S)
        compare_full(w, out, lse, "extreme S=%d" % S)
    q, k, v, cu, sv = dev_inputs(w)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16, max_kb_per_item=0)
    out, lse = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    compare_full(w, out, lse, "extreme planned")


# ---------------------------------------------------------- properties
@pytest.mark.parametrize("k,N,H", [(2, None, 2), (4, 6000, 2), (5, 12000, 1)])
def test_no_skip_bit_exact(pv, k, N, H):
    """FlashMask article §3.3: skipping fully masked tiles changes no bit."""
    w = W.make_config(k, N=N, H=H)
    a_out, a_lse = run(pv, w, max_kb_per_item=0)
    b_out, b_lse = run(pv, w, max_kb_per_item=0, flags=pv.FM_FLAG_NO_SKIP)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


@pytest.mark.parametrize("seed", range(6))
def test_no_skip_bit_exact_random(pv, seed):
    w = W.random_case(300 + seed, N_max=500, H=1, D=128, dtype=W.BF16)
    a = run(pv, w, max_kb_per_item=0)
    b = run(pv, w, max_kb_per_item=0, flags=pv.FM_FLAG_NO_SKIP)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    wf = W.random_case(300 + seed, N_max=200, H=1, D=32)
    a = run(pv, wf, block_q=8, block_k=4)
    b = run(pv, wf, block_q=8, block_k=4, flags=pv.FM_FLAG_NO_SKIP)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("S", [0, -1])
def test_deterministic_and_plan_reuse(pv, S):
    w = W.make_config(2)
    q, k, v, cu, sv = dev_inputs(w)
    o1, l1 = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S)
    o2, l2 = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), max_kb_per_item=S)
    plan = pv.build_plan(cu, sv, w.n_vec, w.causal, w.N, w.H, w.D, torch.bfloat16, max_kb_per_item=S)
    o3, l3 = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan)
    o4, l4 = pv.attn_fwd(q, k, v, cu, sv, w.n_vec, w.causal, float(w.scale), plan=plan)
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o1, o) and torch.equal(l1, l)
    assert plan.header()["sched_counter"] == 0


def test_fully_masked_rows(pv):
    """Rows whose every key is masked: out = 0 and lse = -inf."""
    N, H = 300, 2
    cu = np.array([0, 100, 300], np.int32)
    lts = np.zeros(N, np.int32)
    lte = np.zeros(N, np.int32)
    lte[0:100] = 50          # keys of sequence 0 hidden from rows 0..49 -> rows 0..49 empty
    lte[100:300] = 100 + 30  # rows 100..129 of sequence 1 empty
    sv = np.stack([lts, lte])
    for dt, D in ((W.BF16, 128), (W.F32, 32)):
        q, k, v = W.draw_qkv(5, N, H, D, dt)
        w = W.Workload("empty_rows", N, H, D, dt, True, 2, cu, sv, np.float32(0.1), q, k, v)
        out, lse = run(pv, w, max_kb_per_item=0)
        l = lse.cpu().numpy()
        assert np.all(np.isneginf(l[:, 0:50])) and np.all(np.isneginf(l[:, 100:130]))
        assert torch.count_nonzero(out[0:50]).item() == 0
        compare_full(w, out, lse, "empty rows %s" % dt)


def test_bad_cu_sets_status(pv):
    N, H = 256, 1
    w = W.make_config(2, H=1)
    q, k, v, _, sv = dev_inputs(w)
    q, k, v, sv = q[:N].contiguous(), k[:N].contiguous(), v[:N].contiguous(), sv[:, :N].contiguous()
    cu = torch.tensor([0, 200, 100, N], dtype=torch.int32, device="cuda")
    lay = pv.workspace_layout(N, 3, H, 128, 128, 64, 0, False)
    ws = torch.zeros(lay.bytes, dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(q)
    pv.attn_fwd(q, k, v, cu, sv, 2, True, 0.1, max_kb_per_item=0, workspace=ws, out=out)
    assert pv.read_status(ws) & 0x2
    h = ws[:16].view(torch.int32).cpu().tolist()
    assert h[2] == 0 and h[3] == 0          # no items; scheduler counter reset
    assert torch.count_nonzero(out).item() == 0
    cu2 = torch.tensor([0, 100, 200, N + 1], dtype=torch.int32, device="cuda")
    pv.attn_fwd(q, k, v, cu2, sv, 2, True, 0.1, max_kb_per_item=0, workspace=ws, out=out)
    assert pv.read_status(ws) & 0x4


def test_empty_input(pv):
    q = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    sv = torch.empty(1, 0, dtype=torch.int32, device="cuda")
    out, lse = pv.attn_fwd(q, q, q, cu, sv, 1, True)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128) and lse.shape == (2, 0)


# ------------------------------------------------- extrema at large N
@pytest.mark.parametrize("n_vec,causal,aligned", [(4, False, True), (4, False, False), (2, True, False), (1, True, True)])
def test_extrema_large(pv, n_vec, causal, aligned):
    """The extrema pass over 2^22 tokens (65536 key blocks at Bc = 64: more
    than one grid-stride round of the launch), bit-exact against the oracle.
    Documents of random lengths, multiples of 64 when `aligned` (every block
    starts on a 16-byte boundary of the vectors) and arbitrary otherwise;
    uniform random int32 mask values."""
    N = 1 << 22
    rng = np.random.default_rng(4242 + n_vec + 2 * int(aligned))
    lens = []
    while sum(lens) < N:
        L = int(rng.integers(1000, 400000))
        if aligned:
            L = max(64, L // 64 * 64)
        lens.append(min(L, N - sum(lens)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    sv = rng.integers(0, N, size=(n_vec, N), dtype=np.int64).astype(np.int32)
    say("extrema large: N=%d B=%d n_vec=%d causal=%d aligned=%d" % (N, len(lens), n_vec, causal, aligned))
    kb_off, ext, status = pv.preprocess_mask(torch.from_numpy(sv).cuda(), n_vec, causal,
                                             torch.from_numpy(cu).cuda(), N, 64)
    okb, oext = O.extrema(cu, sv, n_vec, causal, 64)
    assert status == 0
    assert np.array_equal(kb_off.cpu().numpy(), okb)
    assert np.array_equal(ext.cpu().numpy().reshape(-1, 8), oext.reshape(-1, 8))


@pytest.mark.parametrize("vexp", [-40, 0, 24, 100])
@pytest.mark.parametrize("S", [2, -1])
def test_split_partials_any_scale(pv, vexp, S):
    """Split rows keep their partials as fp16 with a power-of-two scale per
    row: V multiplied by 2^vexp (exact in bf16) must give out multiplied by
    2^vexp, within the out bar relative to that scale, on rows split into
    many chunks; lse does not depend on V.  Without the per-row scale, 2^24
    and 2^100 would overflow fp16 and 2^-40 would vanish."""
    w = W.document_workload([1500, 300, 700], H=2, seed=21)
    sc = 2.0 ** vexp
    oo, ol = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    q, k, v, cu, sv = dev_inputs(w)
    out, lse = pv.attn_fwd(q, k, (v.float() * sc).to(torch.bfloat16), cu, sv, w.n_vec, w.causal, float(w.scale),
                           max_kb_per_item=S)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64) / sc
    l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ol)
    e_out = float(np.max(np.abs(o - oo)))
    e_lse = float(np.max(np.abs(l[fin] - ol[fin]), initial=0.0))
    say("  V x 2^%d, S=%d: max|dout|/2^%d=%.3e max|dlse|=%.3e" % (vexp, S, vexp, e_out, e_lse))
    assert np.all(np.isfinite(o)) and e_out <= OUT_TOL and e_lse <= LSE_TOL
