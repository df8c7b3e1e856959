"""CPU pins of the oracle against what the pages and the mathematics fix.

Each test names the passage or the mathematical fact it checks.  None of
them re-types an oracle formula: they use printed values, closed forms,
brute force over single elements, and library special cases.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ helpers
_LISTS = {}


def _brute_masked(w, i, j):
    """Element truth straight from the stored vectors, one pair at a time.
    FlashMask article §2.1/§2.2: column j hides rows in [LTS_j, LTE_j) and
    [UTS_j, UTE_j); defaults LTS=UTS=0, LTE=UTE=N; causal hides j > i;
    different sequences never attend (Varlen-Packing document §2)."""
    key = id(w)
    if key not in _LISTS or _LISTS[key][0] is not w:
        _LISTS[key] = (w, [int(x) for x in w.cu_seqlens], [[int(x) for x in row] for row in w.startend])
    _, cu, sv = _LISTS[key]
    if _seq_of(cu, i) != _seq_of(cu, j):
        return True
    N = w.N
    if w.causal:
        lts = sv[0][j]
        lte = sv[1][j] if w.n_vec == 2 else N
        if j > i:
            return True
        return lts <= i < lte
    if w.n_vec == 2:
        lts, lte, uts, ute = sv[0][j], N, 0, sv[1][j]
    else:
        lts, lte, uts, ute = sv[0][j], sv[1][j], sv[2][j], sv[3][j]
    return (lts <= i < lte) or (uts <= i < ute)


def _seq_of(cu, i):
    for b in range(len(cu) - 1):
        if cu[b] <= i < cu[b + 1]:
            return b
    raise ValueError


# ------------------------------------------------------- printed examples
def test_page_table_column0_masks_rows_13_14():
    g = _gold("page_flashmask_16x16.json")
    w = W.make_config(1, with_qkv=False)
    assert w.startend[0].tolist() == g["lts"]["value"]
    assert w.startend[1].tolist() == g["lte"]["value"]
    vecs = O.fill_vectors(w.startend, w.n_vec, w.causal, w.N)
    m = O.element_mask(np.arange(16), np.arange(16), vecs, w.causal)
    # column 0 is below the diagonal everywhere, so only LT masks it
    assert np.nonzero(m[:, 0])[0].tolist() == g["column0_masked_rows"]["value"]


def test_page_block0_extrema():
    g = _gold("page_flashmask_16x16.json")["block0_extrema"]
    w = W.make_config(1, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, g["block_k"])
    assert ext[0, :4].tolist() == [g["lts_min"], g["lts_max"], g["lte_min"], g["lte_max"]]
    # causal: the upper-triangle slots stay 0
    assert ext[:, 4:].tolist() == [[0, 0, 0, 0]] * len(ext)


def test_page_tile_examples():
    g = _gold("page_flashmask_16x16.json")["tile_examples"]
    w = W.make_config(1, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, g["block_k"])
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, g["block_q"], g["block_k"])[0]
    name = {"FULL": O.FULL, "PARTIAL": O.PARTIAL, "UNMASKED": O.UNMASKED}
    for t in g["tiles"]:
        r, c = t["tile"]
        assert cls[r, c] == name[t["class"]], t


def test_page_tiles_agree_with_element_truth():
    """All 16 tiles of the page's example: FULL tiles are entirely masked,
    UNMASKED ones entirely visible (brute force per element)."""
    w = W.make_config(1, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, 2, True, 4)
    cls = O.classify(w.cu_seqlens, kb_off, ext, True, 4, 4)[0]
    for r in range(4):
        for c in range(4):
            el = [_brute_masked(w, i, j) for i in range(4 * r, 4 * r + 4) for j in range(4 * c, 4 * c + 4)]
            if cls[r, c] == O.FULL:
                assert all(el)
            elif cls[r, c] == O.UNMASKED:
                assert not any(el)
            else:  # on this example every PARTIAL tile really is mixed
                assert any(el) and not all(el)


def test_golden_oracle_cfg1_is_current():
    g = _gold("oracle_cfg1.json")
    w = W.make_config(1, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, 2, True, 4)
    cls = O.classify(w.cu_seqlens, kb_off, ext, True, 4, 4)
    assert kb_off.tolist() == g["kb_off"] and ext.tolist() == g["extrema"]
    assert cls[0].tolist() == g["classes"]
    assert O.class_counts(cls).tolist() == g["class_counts"] == [7, 8, 1]
    pairs = sum(not _brute_masked(w, i, j) for i in range(16) for j in range(16))
    assert pairs == g["unmasked_pairs"] == 71


def test_varlen_grid_count_and_items():
    g = _gold("page_varlen_grid.json")
    ge = g["grid_example"]
    assert O.fa_varlen_grid_blocks(ge["lengths"], ge["n_head"], ge["block_q"]) == ge["grid_blocks"]
    assert 3 * max(ge["lengths"]) == g["padded_tokens"]["padded"]
    assert sum(ge["lengths"]) == g["padded_tokens"]["real"]
    w = W.make_config(2, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, 64)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, ge["block_q"], 64)
    items = O.worklist(cls, ge["n_head"], 0)
    # one item per real q tile and head: 2 * (1 + 1 + 32)
    assert len(items) == ge["n_head"] * sum(-(-L // ge["block_q"]) for L in ge["lengths"]) == 68


# ------------------------------------------------------------ closed forms
def _causal_doc_counts(lengths, Br, Bc):
    """Closed form for a causal document mask with every L a multiple of Br
    and Br = 2*Bc: q tile t sees 2t unmasked blocks and 2 diagonal partial
    blocks."""
    f = p = u = 0
    for L in lengths:
        tr, tc = L // Br, L // Bc
        p += 2 * tr
        u += tr * (tr - 1)
        f += tr * tc - 2 * tr - tr * (tr - 1)
    return [f, p, u]


@pytest.mark.parametrize("Bc", [64])
def test_config2_class_counts_closed_form(Bc):
    w = W.make_config(2, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, Bc)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, 128, Bc)
    assert O.class_counts(cls).tolist() == _causal_doc_counts([128, 128, 4096], 128, Bc) == [992, 68, 992]


def test_config2_bc128_counts():
    # Br = Bc = 128: q tile t sees t unmasked blocks and 1 diagonal block
    w = W.make_config(2, with_qkv=False)
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, 128)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, 128, 128)
    tr = [1, 1, 32]
    p = sum(tr); u = sum(t * (t - 1) // 2 for t in tr); f = sum(t * t for t in tr) - p - u
    assert O.class_counts(cls).tolist() == [f, p, u] == [496, 34, 496]


@pytest.mark.parametrize("k", [2, 3])
def test_causal_document_pairs_closed_form(k):
    w = W.make_config(k, with_qkv=False)
    expect = sum(int(L) * (int(L) + 1) // 2 for L in w.lengths)
    assert O.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal) == expect
    if k == 2:
        assert expect == 8407168
        assert O.effective_flops(expect, 2, 128) == 4 * 128 * 2 * 8407168


def test_shared_question_pairs_closed_form():
    """Config 4 at reduced N: per group, the prompt (P tokens) is causal
    (P(P+1)/2); each answer of length A sees the whole prompt and itself
    causally (A*P + A(A+1)/2)."""
    w = W.make_config(4, with_qkv=False, N=6000)
    expect = 0
    for g_start, ends in w.meta["groups"]:
        segs = np.diff([g_start] + list(ends))
        P = int(segs[0])
        expect += P * (P + 1) // 2
        for A in segs[1:]:
            expect += int(A) * P + int(A) * (int(A) + 1) // 2
    assert O.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal) == expect


def test_prefix_window_pairs_closed_form():
    """Config 5 at reduced N: prefix rows see the whole prefix (p^2); a
    suffix row at offset t >= p of its document sees keys t-W+1 .. t."""
    w = W.make_config(5, with_qkv=False, N=20000)
    W_ = w.meta["window"]
    expect = 0
    for L, p in zip(w.lengths, w.meta["prefix"]):
        L = int(L)
        expect += p * p
        for t in range(p, L):
            expect += min(t + 1, W_)
    assert O.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal) == expect


@pytest.mark.parametrize("lens", [[5, 9, 20], [64, 1, 300, 17], [1000]])
def test_bidirectional_document_pairs_closed_form(lens):
    """Non-causal, two stored vectors: the FlashMask article §2.2 defaults
    fill the absent ones (LTE = query length, UTS = 0), so a key of document
    [s, e) stored as LTS = e, UTE = s hides exactly the rows outside its own
    document.  Under one sequence covering every token (cu = [0, N], the
    ZeroPadding packing of §6.7), each row then sees its whole document and
    nothing else: sum_b L_b^2 pairs per head.  Any other reading of the two
    vectors (for instance LTS and LTE) gives a different count."""
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    starts = np.repeat(cu[:-1], lens)
    ends = np.repeat(cu[1:], lens)
    sv = np.stack([ends, starts]).astype(np.int32)
    expect = sum(L * L for L in lens)
    assert O.unmasked_pairs(np.array([0, N], np.int32), sv, 2, False) == expect
    assert O.unmasked_pairs(cu, sv, 2, False) == expect
    # the same documents with the two stored rows swapped hide far more
    assert O.unmasked_pairs(np.array([0, N], np.int32), sv[::-1].copy(), 2, False) != expect or len(lens) == 1


# -------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(8))
def test_extreme_endpoints_brute_force(seed):
    """Endpoints anywhere in the int32 range (FlashMask article §2.1: a
    half-open row interval per column; start >= end is empty): INT32_MIN,
    -1, 0, N, N + 7 and INT32_MAX mixed with ordinary rows.  The oracle's
    attention, extrema and tile classes against pure-Python element truth
    and brute force over single pairs."""
    w = W.random_case(seed, N_max=28, H=2, D=8, extreme=True)
    assert w.startend.min() < -1 or w.startend.max() > w.N
    out, lse = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, chunk=5)
    bo, bl = _brute_attention(w)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - bl[fin]), initial=0) <= 1e-12
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert O.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal) == sum(
        0 if _brute_masked(w, i, j) else 1 for i in range(w.N) for j in range(w.N))
    cu = [int(x) for x in w.cu_seqlens]
    for Br, Bc in ((1, 1), (3, 2), (4, 5)):
        kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, Bc)
        assert ext.dtype.itemsize >= 4 and ext.min() >= W.INT32_MIN and ext.max() <= W.INT32_MAX
        cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, Br, Bc)
        for b, c in enumerate(cls):
            s, e = cu[b], cu[b + 1]
            for qt in range(c.shape[0]):
                for kb in range(c.shape[1]):
                    el = [_brute_masked(w, i, j)
                          for i in range(s + qt * Br, min(s + (qt + 1) * Br, e))
                          for j in range(s + kb * Bc, min(s + (kb + 1) * Bc, e))]
                    if c[qt, kb] == O.FULL:
                        assert all(el)
                    elif c[qt, kb] == O.UNMASKED:
                        assert not any(el)


@pytest.mark.parametrize("seed", range(12))
def test_extrema_brute_force(seed):
    w = W.random_case(seed, with_qkv=False)
    for Bc in (1, 3, 4, 7):
        kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, Bc)
        rows = []
        cu = [int(x) for x in w.cu_seqlens]
        sv = [[int(x) for x in r] for r in w.startend]
        N = w.N
        for b in range(len(cu) - 1):
            for c0 in range(cu[b], cu[b + 1], Bc):
                cols = range(c0, min(c0 + Bc, cu[b + 1]))
                if w.causal:
                    L4 = [[sv[0][j] for j in cols], [sv[1][j] if w.n_vec == 2 else N for j in cols], [0], [0]]
                elif w.n_vec == 2:
                    L4 = [[sv[0][j] for j in cols], [N], [0], [sv[1][j] for j in cols]]
                else:
                    L4 = [[sv[t][j] for j in cols] for t in range(4)]
                rows.append([f(x) for x in L4 for f in (min, max)])
        assert ext.tolist() == rows
        assert int(kb_off[-1]) == len(rows)


@pytest.mark.parametrize("seed", range(40))
def test_classification_sound(seed):
    """FULL => every element masked; UNMASKED => no element masked."""
    w = W.random_case(seed, N_max=48, with_qkv=False)
    rng = np.random.default_rng(seed)
    cu = [int(x) for x in w.cu_seqlens]
    for _ in range(3):
        Br, Bc = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, Bc)
        cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, Br, Bc)
        for b, c in enumerate(cls):
            s, e = cu[b], cu[b + 1]
            for qt in range(c.shape[0]):
                for kb in range(c.shape[1]):
                    el = [_brute_masked(w, i, j)
                          for i in range(s + qt * Br, min(s + (qt + 1) * Br, e))
                          for j in range(s + kb * Bc, min(s + (kb + 1) * Bc, e))]
                    if c[qt, kb] == O.FULL:
                        assert all(el)
                    elif c[qt, kb] == O.UNMASKED:
                        assert not any(el)


def _brute_attention(w):
    """Pure-Python loops, math.exp and math.fsum."""
    N, H, D = w.N, w.H, w.D
    cu = [int(x) for x in w.cu_seqlens]
    sc = float(w.scale)
    out = [[[0.0] * D for _ in range(H)] for _ in range(N)]
    lse = [[-math.inf] * N for _ in range(H)]
    q = w.q.astype(np.float64).tolist(); k = w.k.astype(np.float64).tolist(); v = w.v.astype(np.float64).tolist()
    for i in range(N):
        b = _seq_of(cu, i)
        allowed = [j for j in range(cu[b], cu[b + 1]) if not _brute_masked(w, i, j)]
        for h in range(H):
            if not allowed:
                continue
            s = [sc * math.fsum(q[i][h][d] * k[j][h][d] for d in range(D)) for j in allowed]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            z = math.fsum(p)
            lse[h][i] = m + math.log(z)
            for d in range(D):
                out[i][h][d] = math.fsum(p[t] * v[j][h][d] for t, j in enumerate(allowed)) / z
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", range(10))
def test_attention_brute_force(seed):
    w = W.random_case(seed, N_max=24, H=2, D=8)
    out, lse = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, chunk=5)
    bo, bl = _brute_attention(w)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - bl[fin]), initial=0) <= 1e-12
    assert np.max(np.abs(out - bo)) <= 1e-12
    # sampled evaluation agrees with the dense one
    rows = list(range(w.N)) * w.H
    heads = [h for h in range(w.H) for _ in range(w.N)]
    ro, rl = O.attention_rows(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, rows, heads)
    for t, (i, h) in enumerate(zip(rows, heads)):
        assert np.allclose(ro[t], out[i, h], atol=1e-12, rtol=0)
        assert (rl[t] == lse[h, i]) or abs(rl[t] - lse[h, i]) <= 1e-12


# ----------------------------------------------------- special cases, laws
@pytest.mark.parametrize("k,N", [(2, None), (3, 3000), (4, 3000), (5, 9000)])
def test_q_zero_closed_form(k, N):
    """q = 0: every allowed score is 0, so lse_i = ln|A_i| and out_i is the
    mean of v over A_i."""
    w = W.make_config(k, N=N, H=1)
    q = np.zeros_like(w.q)
    out, lse = O.attention(q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    rng = np.random.default_rng(k)
    cu = [int(x) for x in w.cu_seqlens]
    for i in rng.integers(0, w.N, size=25):
        i = int(i)
        b = _seq_of(cu, i)
        allowed = [j for j in range(cu[b], cu[b + 1]) if not _brute_masked(w, i, j)]
        assert abs(lse[0, i] - math.log(len(allowed))) < 1e-12
        assert np.allclose(out[i, 0], w.v[allowed, 0].astype(np.float64).mean(axis=0), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_empty_intervals_reduce_to_sdpa(causal):
    """With every interval empty the method is plain (causal or full)
    softmax attention per sequence: compare with torch's SDPA in fp64."""
    import torch
    rng = np.random.default_rng(7)
    lens = [5, 17, 1, 30]
    N, H, D = sum(lens), 3, 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = (rng.standard_normal((N, H, D)) for _ in range(3))
    scale = np.float32(0.3)
    if causal:
        sv = np.full((1, N), N, np.int32); n_vec = 1           # LT = [N, N)
    else:
        sv = np.stack([np.full(N, N), np.full(N, N), np.zeros(N), np.zeros(N)]).astype(np.int32); n_vec = 4
    out, lse = O.attention(q, k, v, cu, sv, n_vec, causal, scale)
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x[s:e].transpose(1, 0, 2))) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=float(scale))
        assert np.allclose(out[s:e], ref.numpy().transpose(1, 0, 2), atol=1e-12, rtol=0)
        sc = float(scale) * np.einsum("ihd,jhd->hij", q[s:e], k[s:e])
        if causal:
            sc = np.where(np.tril(np.ones((e - s, e - s), bool))[None], sc, -np.inf)
        ref_lse = np.log(np.exp(sc).sum(-1))
        assert np.allclose(lse[:, s:e], ref_lse, atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(6))
def test_packed_equals_separate(seed):
    """Unsloth packing blog (uncontaminated packing): no attention crosses
    packed samples, so each sequence run alone (indices rebased to its
    start) gives the same out and lse."""
    w = W.random_case(100 + seed, N_max=40, H=2, D=8, allow_empty=True)
    out, lse = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    cu = [int(x) for x in w.cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        sv = w.startend[:, s:e].astype(np.int64) - s
        if (not w.causal) and w.n_vec == 2:
            pass
        o1, l1 = O.attention(w.q[s:e], w.k[s:e], w.v[s:e], np.array([0, e - s]), sv, w.n_vec, w.causal, w.scale)
        # defaults (LTE/UTE = query length) differ between N and e - s only
        # beyond the sequence's rows, where no query lives
        assert np.allclose(o1, out[s:e], atol=1e-12, rtol=0)
        assert np.array_equal(np.isfinite(l1), np.isfinite(lse[:, s:e]))
        f = np.isfinite(l1)
        assert np.allclose(l1[f], lse[:, s:e][f], atol=1e-12, rtol=0)


@pytest.mark.parametrize("k,N", [(2, None), (3, 2500), (4, 2500), (5, 9000)])
def test_mask_only_packing(k, N):
    """FlashMask article §6.7 (ZeroPadding): with global indices the mask
    alone separates documents, so cu = [0, N] gives the varlen result."""
    w = W.make_config(k, N=N, H=1)
    a = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    b = O.attention(w.q, w.k, w.v, np.array([0, w.N]), w.startend, w.n_vec, w.causal, w.scale)
    assert np.allclose(a[0], b[0], atol=1e-12, rtol=0)
    assert np.allclose(a[1], b[1], atol=1e-12, rtol=0)


@pytest.mark.parametrize("lens", [[5, 9, 20], [1, 17, 3, 8], [12], [7, 0, 7]])
def test_packings_agree(lens):
    """Varlen-Packing document §3 (padded batch) and FlashMask article §6.7
    (ZeroPadding): the same causal documents packed back to back, packed
    with cu = [0, N] and a global mask, or zero-padded to the longest one
    give the same out and lse on every real token.  With the padding
    masked by the interval, pad rows are empty rows (out = 0, lse = -inf).
    Pair counts: the masked layouts keep exactly the documents' pairs, the
    plain padded one every causal pair of each padded sample."""
    w = W.document_workload(lens, H=2, D=8, seed=7)
    ref_o, ref_l = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    ref_pairs = O.unmasked_pairs(w.cu_seqlens, w.startend, w.n_vec, w.causal)
    assert ref_pairs == sum(L * (L + 1) // 2 for L in lens)
    Lmax = max(lens)
    for kind in W.PACKINGS:
        p = W.packed_as(w, kind)
        real = p.meta["real_rows"]
        assert np.array_equal(p.q[real], w.q) and np.array_equal(p.v[real], w.v)
        o, l = O.attention(p.q, p.k, p.v, p.cu_seqlens, p.startend, p.n_vec, p.causal, p.scale)
        assert np.allclose(o[real], ref_o, atol=1e-12, rtol=0), kind
        assert np.allclose(l[:, real], ref_l, atol=1e-12, rtol=0), kind
        pad = np.setdiff1d(np.arange(p.N), real)
        pairs = O.unmasked_pairs(p.cu_seqlens, p.startend, p.n_vec, p.causal)
        if kind == "padded":
            assert np.all(np.isfinite(l[:, pad]))
            assert pairs == len(lens) * Lmax * (Lmax + 1) // 2
        else:
            assert pairs == ref_pairs, kind
        if kind == "padded_masked":
            assert np.all(o[pad] == 0.0) and np.all(np.isneginf(l[:, pad]))


# ------------------------------------------------------------- gradients
@pytest.mark.parametrize("seed", range(6))
def test_bwd_finite_differences(seed):
    """FlashMask article §3.4 (the backward returns the gradients of q, k,
    v) and §4.2 (exact: the dense-mask attention's gradients): central
    differences of the forward oracle's L = sum(G * out) match the
    backward for every element of q, k and v, masked pairs, empty rows and
    zero-length sequences included."""
    w = W.random_case(300 + seed, N_max=18, H=2, D=3, dtype=W.F32, allow_empty=True)
    rng = np.random.default_rng(seed)
    G = rng.standard_normal(w.q.shape)
    q, k, v = (x.astype(np.float64) for x in (w.q, w.k, w.v))
    dq, dk, dv = O.attention_bwd(q, k, v, G, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)

    def loss(qq, kk, vv):
        return float(np.sum(G * O.attention(qq, kk, vv, w.cu_seqlens, w.startend, w.n_vec, w.causal,
                                            w.scale)[0]))
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - grad)) < 1e-6, (which, np.max(np.abs(num - grad)))


def test_bwd_q_zero_closed_form():
    """q = 0 makes every allowed key equally likely (P_ij = 1 / |A_i|), so
    dv_j = sum over the rows i that see j of G_i / |A_i|; with the same
    mask written out here as the FlashMask article §2.2 intervals."""
    w = W.make_config(1)
    q = np.zeros_like(w.q)
    G = np.random.default_rng(5).standard_normal(w.q.shape)
    _, _, dv = O.attention_bwd(q, w.k, w.v, G, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    lts, lte = W.PAGE_LTS, W.PAGE_LTE
    allowed = [[j for j in range(16) if j <= i and not (lts[j] <= i < lte[j])] for i in range(16)]
    ref = np.zeros_like(dv)
    for i in range(16):
        for j in allowed[i]:
            ref[j] += G[i] / len(allowed[i])
    assert sum(len(a) for a in allowed) == 71
    assert np.allclose(dv, ref, atol=1e-13, rtol=0)


@pytest.mark.parametrize("seed", range(4))
def test_bwd_rows_match_full(seed):
    """The one-row-at-a-time dq equals the full backward's rows (the same
    definition evaluated two ways), empty rows included."""
    w = W.random_case(500 + seed, N_max=60, H=2, D=8, dtype=W.F32, allow_empty=True)
    G = np.random.default_rng(seed).standard_normal(w.q.shape)
    dq, _, _ = O.attention_bwd(w.q, w.k, w.v, G, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    rows = list(range(w.N)) * 2
    heads = [0] * w.N + [1] * w.N
    r = O.attention_bwd_rows(w.q, w.k, w.v, G, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, rows, heads)
    assert np.allclose(r, np.stack([dq[i, h] for i, h in zip(rows, heads)]), atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(6))
def test_bwd_invariants(seed):
    """Softmax is unchanged when one vector is added to every key of a
    sequence (each score row moves by a constant), so the key gradients of
    a sequence sum to zero per head; rows with no allowed key get dq = 0,
    keys no row attends get dk = dv = 0; packed = separate ([US] packing
    without contamination) holds for the gradients too."""
    w = W.random_case(400 + seed, N_max=40, H=2, D=8, dtype=W.F32, allow_empty=True)
    G = np.random.default_rng(seed).standard_normal(w.q.shape)
    dq, dk, dv = O.attention_bwd(w.q, w.k, w.v, G, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    vecs = O.fill_vectors(w.startend, w.n_vec, w.causal, w.N)
    cu = [int(x) for x in w.cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        assert np.allclose(dk[s:e].sum(axis=0), 0.0, atol=1e-12)
        m = O.element_mask(np.arange(s, e), np.arange(s, e), vecs, w.causal)
        assert np.all(dq[s:e][m.all(axis=1)] == 0.0)
        assert np.all(dk[s:e][m.all(axis=0)] == 0.0) and np.all(dv[s:e][m.all(axis=0)] == 0.0)
        sv = w.startend[:, s:e].astype(np.int64) - s
        one = O.attention_bwd(w.q[s:e], w.k[s:e], w.v[s:e], G[s:e], np.array([0, e - s]), sv, w.n_vec,
                              w.causal, w.scale)
        for a, bb in zip(one, (dq, dk, dv)):
            assert np.allclose(a, bb[s:e], atol=1e-12, rtol=0)


# --------------------------------------------------------------- rotary
def test_rope_2d_rotation():
    """D = 2: each (x0, x1) pair turns by the table's angle, as the 2-D
    rotation matrix [[c, s], [-s, c]] acting on the row vector."""
    rng = np.random.default_rng(0)
    ang = rng.uniform(-np.pi, np.pi, 9)
    cos, sin = np.cos(ang)[:, None], np.sin(ang)[:, None]
    x = rng.standard_normal((9, 3, 2))
    got = O.rope(x, [0, 9], cos, sin)
    for i in range(9):
        M = np.array([[np.cos(ang[i]), np.sin(ang[i])], [-np.sin(ang[i]), np.cos(ang[i])]])
        assert np.allclose(got[i], x[i] @ M, atol=1e-14)


def test_rope_norms_inverse_reset():
    """Every (j, j + D/2) pair keeps its length; the map with sin negated
    (the packing blog's backward) undoes it; positions restart per packed
    sample, so packed = each sample alone."""
    rng = np.random.default_rng(1)
    D, H = 16, 3
    lens = [5, 0, 11, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((int(cu[-1]), H, D))
    cos, sin = W.rope_tables(16, D)
    y = O.rope(x, cu, cos, sin)
    n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2
    assert np.allclose(n0, n1, rtol=1e-6)     # tables are float32: cos^2 + sin^2 = 1 to ~1e-7
    assert np.allclose(O.rope(y, cu, cos, sin, inverse=True), x, atol=1e-6)
    for b in range(len(lens)):
        s, e = int(cu[b]), int(cu[b + 1])
        assert np.array_equal(O.rope(x[s:e], [0, e - s], cos, sin), y[s:e])


def test_rope_relative_positions():
    """With the usual angle tables <rope(q, m), rope(k, n)> depends only on
    m - n: scores see relative positions."""
    rng = np.random.default_rng(2)
    D = 32
    cos, sin = W.rope_tables(64, D)
    q, k = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))

    def at(x, p):   # x placed at position p of a sequence of length p + 1
        z = np.zeros((p + 1, 1, D))
        z[p] = x[0]
        return O.rope(z, [0, p + 1], cos, sin)[p, 0]
    for m, n, c in [(10, 3, 0), (40, 33, 7), (5, 5, 20)]:
        a = at(q, m) @ at(k, n)
        b = at(q, m - n + c) @ at(k, c)
        assert abs(a - b) < 1e-4 * (1 + abs(a))


# --------------------------------------------------------------- dropout
def test_philox_statistics():
    """Philox4x32-10 as a counter-based generator: bytes uniform (chi-square
    over 2^20 bytes), one counter bit flipped changes about half of the 128
    output bits, different keys give unrelated streams, and the same
    (counter, key) always gives the same words."""
    ctr = np.zeros((65536, 4), np.uint64)
    ctr[:, 0] = np.arange(65536)
    ctr[:, 1] = 7
    key = np.array([0x1234567, 0x89ABCDE], np.uint64)
    w = O.philox4x32_10(ctr, key)
    by = w.view(np.uint8).reshape(-1)
    cnt = np.bincount(by, minlength=256)
    chi2 = float(((cnt - by.size / 256) ** 2 / (by.size / 256)).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)
    ctr2 = ctr.copy()
    ctr2[:, 2] ^= np.uint64(1 << 13)
    w2 = O.philox4x32_10(ctr2, key)
    flips = np.unpackbits((w ^ w2).view(np.uint8)).reshape(65536, -1).sum(axis=1)
    assert abs(flips.mean() - 64) < 0.5 and flips.min() > 20
    w3 = O.philox4x32_10(ctr, key + np.uint64(1))
    assert np.mean(w3 == w) < 1e-3
    assert np.array_equal(O.philox4x32_10(ctr, key), w)


def test_dropout_p0_and_keep_fraction():
    """p = 0 is plain attention (to fp64 rounding: the normalisation is
    applied before the product here); the kept fraction of pairs matches
    1 - t/256 within five standard deviations."""
    w = W.document_workload([40, 200, 300], H=2, D=16, seed=3)
    a = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)
    b = O.attention_dropout(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, 0.0, 9, 0)
    assert np.allclose(a[0], b[0], atol=1e-12, rtol=0) and np.array_equal(a[1], b[1])
    for p in (0.1, 0.5):
        t = O.dropout_threshold(p)
        kept = n = 0
        for bb, (s_, e_) in enumerate(zip(w.cu_seqlens[:-1], w.cu_seqlens[1:])):
            km = O.dropout_keep(np.arange(s_, e_), np.arange(s_, e_), s_, 1, 12345, 77, t)
            kept += int(km.sum()); n += km.size
        q = 1 - t / 256
        assert abs(kept / n - q) < 5 * np.sqrt(q * (1 - q) / n)


def test_dropout_expectation():
    """Dropout scales kept values by 256 / (256 - t): averaged over seeds the
    output approaches the output without dropout."""
    w = W.document_workload([24, 40], H=1, D=8, seed=4)
    ref = O.attention(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale)[0]
    n = 400
    acc = sum(O.attention_dropout(w.q, w.k, w.v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, 0.25,
                                  seed, 5)[0] for seed in range(n)) / n
    assert np.max(np.abs(acc - ref)) < 0.15 and np.mean(np.abs(acc - ref)) < 0.03


@pytest.mark.parametrize("seed", range(3))
def test_dropout_bwd_finite_differences(seed):
    """The dropout backward against central differences of the dropout
    forward (the keep mask does not depend on q, k, v)."""
    w = W.random_case(600 + seed, N_max=16, H=2, D=3, dtype=W.F32, allow_empty=True)
    G = np.random.default_rng(seed).standard_normal(w.q.shape)
    q, k, v = (x.astype(np.float64) for x in (w.q, w.k, w.v))
    args = (w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, 0.3, 1000 + seed, 3)
    grads = O.attention_bwd_dropout(q, k, v, G, *args)

    def loss(qq, kk, vv):
        return float(np.sum(G * O.attention_dropout(qq, kk, vv, *args)[0]))
    eps = 1e-6
    for which, grad in enumerate(grads):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            xp = [q.copy(), k.copy(), v.copy()]
            xm = [q.copy(), k.copy(), v.copy()]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            num[idx] = (loss(*xp) - loss(*xm)) / (2 * eps)
        assert np.max(np.abs(num - grad)) < 1e-6, (which, np.max(np.abs(num - grad)))


# ------------------------------------------------------------- worklist
@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("S", [0, 1, 2, 3, 5])
def test_worklist_properties(seed, S):
    w = W.random_case(seed, N_max=64, with_qkv=False)
    H = 3
    kb_off, ext = O.extrema(w.cu_seqlens, w.startend, w.n_vec, w.causal, 4)
    cls = O.classify(w.cu_seqlens, kb_off, ext, w.causal, 8, 4)
    items = O.worklist(cls, H, S)
    keys = [(-it[7], it[0], it[2], it[5], it[1]) for it in items.tolist()]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    n_qt = sum(c.shape[0] for c in cls)
    by = {}
    for it in items.tolist():
        by.setdefault((it[0], it[2], it[1]), []).append(it)
    assert len(by) == n_qt * H
    for (b, qt, h), its in by.items():
        its.sort(key=lambda it: it[5])
        K = [kb for kb in range(cls[b].shape[1]) if cls[b][qt, kb] != O.FULL]
        n = its[0][6]
        assert [it[5] for it in its] == list(range(n))
        sizes = [it[7] for it in its]
        assert sum(sizes) == len(K)
        assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)
        if S:
            assert max(sizes) <= max(S, 0) or n == 1
        covered = []
        for it in its:
            covered += [kb for kb in range(it[3], it[4]) if cls[b][qt, kb] != O.FULL]
            assert it[7] == sum(1 for kb in range(it[3], it[4]) if cls[b][qt, kb] != O.FULL)
        assert covered == K


# ------------------------------------------------------------- generators
def test_generators():
    for k in W.CONFIG_IDS:
        a = W.make_config(k, with_qkv=False)
        b = W.make_config(k, with_qkv=False)
        assert np.array_equal(a.cu_seqlens, b.cu_seqlens) and np.array_equal(a.startend, b.startend)
        assert int(a.cu_seqlens[0]) == 0 and int(a.cu_seqlens[-1]) == a.N
        assert np.all(np.diff(a.cu_seqlens) >= 0)
        assert a.startend.shape == (a.n_vec, a.N)
        assert a.startend.min() >= 0 and a.startend.max() <= a.N
    w3 = W.make_config(3, with_qkv=False)
    L = w3.lengths[:-1]
    assert np.all(((L >= 64) & (L <= 512)) | ((L >= 2048) & (L <= 8192)))
    w5 = W.make_config(5, with_qkv=False)
    assert np.all(w5.lengths[:-1] >= 4096) and np.all(w5.lengths <= 32768)
    q1 = W.make_config(2, H=1).q
    q2 = W.make_config(2, H=1).q
    assert np.array_equal(q1, q2)


_ROCRAND_PROBE = r"""
#include <cstdio>
#include <cstdlib>
#include <rocrand/rocrand_philox4x32_10.h>
// words of rocRAND's Philox4x32-10 engine (host code): seed, subsequence,
// first block, number of blocks; block m of subsequence s is the generator
// at counter (m mod 2^32, m >> 32, s mod 2^32, s >> 32)
int main(int argc, char** argv) {
    const unsigned long long seed = strtoull(argv[1], nullptr, 0), sub = strtoull(argv[2], nullptr, 0);
    const unsigned long long m = strtoull(argv[3], nullptr, 0);
    const int n = atoi(argv[4]);
    rocrand_device::philox4x32_10_engine e(seed, sub, 0);
    if (m) e.discard(4 * m);
    for (int i = 0; i < n; ++i) { const uint4 r = e.next4(); printf("%u %u %u %u\n", r.x, r.y, r.z, r.w); }
    return 0;
}
"""


def test_philox_against_rocrand(tmp_path):
    """Philox4x32-10 bit for bit against an independent implementation, the
    host-callable engine of ROCm's rocRAND library (its header, compiled here
    for the CPU): key = the 64-bit seed's two halves, counter = (block,
    subsequence) as two 64-bit halves, including the carry from word 0 into
    word 1.  Skipped where hipcc or the header is absent."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    import os
    if not (os.path.exists(hipcc) and os.path.exists(hdr)):
        pytest.skip("hipcc or rocRAND header not available")
    src = tmp_path / "probe.cpp"
    src.write_text(_ROCRAND_PROBE)
    exe = tmp_path / "probe"
    subprocess.run([hipcc, "-O1", str(src), "-o", str(exe)], check=True, capture_output=True, timeout=300)
    cases = [(0x0123456789ABCDEF, 0, 0, 64), (7, 0, 0xFFFFFFFE, 4), (2 ** 64 - 1, 5, 0, 8),
             (0xDEADBEEF00000001, 2 ** 32 + 3, 2 ** 32 - 1, 3), (12345, 1, 2 ** 40 + 17, 2)]
    for seed, sub, m0, n in cases:
        out = subprocess.run([str(exe), str(seed), str(sub), str(m0), str(n)], check=True, capture_output=True,
                             text=True, timeout=60).stdout.split()
        got = np.array([int(x) for x in out], np.uint64).reshape(n, 4)
        m = np.arange(m0, m0 + n, dtype=np.uint64)
        ctr = np.stack([m & np.uint64(0xFFFFFFFF), m >> np.uint64(32),
                        np.full(n, sub & 0xFFFFFFFF, np.uint64), np.full(n, sub >> 32, np.uint64)], axis=-1)
        key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
        assert np.array_equal(O.philox4x32_10(ctr, key).astype(np.uint64), got), (seed, sub, m0)
