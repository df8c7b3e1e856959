"""Plain fp64 reference of the FlashMask forward path over packed sequences.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written from the
pages' definitions; no blocking, fusion or reordering beyond what each
definition states.

Conventions shared with the library's public contract (not with its code):
  * cu_seqlens: int [B+1], sequence b owns global rows/columns
    [cu[b], cu[b+1]).  Pairs in different sequences never attend
    ([VP] background and §2: sequences are independent).
  * all interval endpoints are GLOBAL row indices into the packed token axis
    ([FM] §6.7: ZeroPadding adds the running token offset to every stored
    endpoint when it concatenates samples).
  * startend: int [n_vec, N], the stored vectors in the order LTS, LTE, UTS,
    UTE restricted to what n_vec carries (see fill_vectors).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

FULL, PARTIAL, UNMASKED = 0, 1, 2


# ---------------------------------------------------------------- O1 fill
def fill_vectors(startend, n_vec: int, causal: bool, N: int):
    """Expand the stored vectors into the four logical vectors LTS, LTE,
    UTS, UTE (int64, length N each).

    [FM] §2.2: the lower-triangle masked rows of column j are
    [LTS_j, LTE_j), the upper-triangle ones [UTS_j, UTE_j); a causal mask
    needs only LTS and LTE; LTS and UTS default to 0 and LTE and UTE
    default to the query length.  [FM] §3.4/§6.4: one interval endpoint
    per token is stored.

    Readings (the pages leave these open):
      * "query length" is the packed length N, because endpoints are global;
      * causal, n_vec=1: LTS stored, LTE = N;  causal, n_vec=2: LTS, LTE;
      * non-causal, n_vec=2: LTS and UTE stored (LTE = N, UTS = 0): the
        document form; non-causal, n_vec=4: all four;
      * in causal mode the upper triangle is hidden by the causal rule, so
        UTS = UTE = 0 (an empty interval).
    Pinned by: the 16x16 example of [FM] §2.2 (column 0 masks rows 13 and
    14), the extrema example of [FM] §3.1, the brute-force soundness and
    special-case tests.
    """
    sv = np.asarray(startend, dtype=np.int64).reshape(n_vec, N)
    zero = np.zeros(N, np.int64)
    full = np.full(N, N, np.int64)
    if causal and n_vec == 1:
        return sv[0].copy(), full, zero, zero.copy()
    if causal and n_vec == 2:
        return sv[0].copy(), sv[1].copy(), zero, zero.copy()
    if (not causal) and n_vec == 2:
        return sv[0].copy(), full, zero, sv[1].copy()
    if (not causal) and n_vec == 4:
        return sv[0].copy(), sv[1].copy(), sv[2].copy(), sv[3].copy()
    raise ValueError("unsupported (n_vec=%d, causal=%s)" % (n_vec, causal))


# ---------------------------------------------------------------- O2 mask
def element_mask(rows: np.ndarray, cols: np.ndarray, vecs, causal: bool) -> np.ndarray:
    """Dense boolean mask (True = masked) for global rows x global cols of
    ONE sequence.

    [FM] §2.1: column j masks the query rows of one half-open interval
    [start_j, end_j); [FM] §2.2: two such intervals, one per triangle;
    a causal mask additionally hides keys after the query.  Intervals are
    applied as given (not clipped to their triangle); start >= end is empty.
    """
    lts, lte, uts, ute = vecs
    i = np.asarray(rows, np.int64)[:, None]
    j = np.asarray(cols, np.int64)[None, :]
    m = (lts[j] <= i) & (i < lte[j])
    if causal:
        m |= j > i
    else:
        m |= (uts[j] <= i) & (i < ute[j])
    return m


# ------------------------------------------------------------ O3 attention
def _seq_bounds(cu, b):
    return int(cu[b]), int(cu[b + 1])


def attention(q, k, v, cu_seqlens, startend, n_vec: int, causal: bool,
              scale, chunk: int = 512, heads: Optional[Sequence[int]] = None,
              rows: Optional[Tuple[int, int]] = None):
    """Masked softmax attention per sequence, float64.

    q, k, v: [N, H, D] (any float dtype; widened exactly to fp64).
    Returns out [N, H, D] fp64 and lse [H, N] fp64 (natural log of the
    softmax normaliser of the scaled scores).

    Follows FlashAttention-2's definition ([FM] §3 extends FlashAttention-2,
    whose outputs out and softmax_lse are the op's outputs, [FM] §3.4):
    s_ij = scale * <q_i, k_j>; over the allowed keys A_i of row i (same
    sequence, not masked), lse_i = log sum exp s_ij and
    out_i = sum_j exp(s_ij - lse_i) v_j.  Computed per (sequence, head) in
    row chunks of at most `chunk` rows over that sequence's keys.

    `heads` and `rows` (a global row range [lo, hi)) restrict which
    (row, head) results are computed; the others stay out = 0, lse = -inf.

    Reading: a row with no allowed key (possible only for hand-made masks)
    gives out = 0 and lse = -inf (log of an empty sum).
    Pinned by: brute force on tiny inputs, q = 0 closed form, the
    all-intervals-empty reduction to textbook causal/full attention,
    packed = separate ([US] uncontaminated packing) and mask-only packing.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    N, H, D = q.shape
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    out = np.zeros((N, H, D), np.float64)
    lse = np.full((H, N), -np.inf, np.float64)
    heads = range(H) if heads is None else heads
    lo, hi = (0, N) if rows is None else (max(int(rows[0]), 0), min(int(rows[1]), N))
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        s_r, e_r = max(s, lo), min(e, hi)
        if e_r <= s_r:
            continue
        cols = np.arange(s, e)
        for h in heads:
            kh = k[s:e, h, :]
            vh = v[s:e, h, :]
            for r0 in range(s_r, e_r, chunk):
                r1 = min(r0 + chunk, e_r)
                rows = np.arange(r0, r1)
                sc = scale * (q[r0:r1, h, :] @ kh.T)
                msk = element_mask(rows, cols, vecs, causal)
                sc = np.where(msk, -np.inf, sc)
                mx = sc.max(axis=1, keepdims=True)
                ok = np.isfinite(mx[:, 0])
                mx = np.where(np.isfinite(mx), mx, 0.0)
                p = np.exp(sc - mx)
                ssum = p.sum(axis=1, keepdims=True)
                with np.errstate(divide="ignore", invalid="ignore"):
                    o = (p @ vh) / ssum
                    l = mx[:, 0] + np.log(ssum[:, 0])
                out[r0:r1, h, :] = np.where(ok[:, None], o, 0.0)
                lse[h, r0:r1] = np.where(ok, l, -np.inf)
    return out, lse


def attention_rows(q, k, v, cu_seqlens, startend, n_vec: int, causal: bool,
                   scale, rows: Sequence[int], heads: Sequence[int]):
    """The same definition as `attention`, evaluated only at the given
    (row, head) pairs, one by one (for sampled checks at full size).
    Returns out [len(rows), D] and lse [len(rows)] in fp64."""
    N, H, D = np.asarray(q).shape
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    outs = np.zeros((len(rows), D), np.float64)
    lses = np.full(len(rows), -np.inf, np.float64)
    for t, (i, h) in enumerate(zip(rows, heads)):
        b = int(np.searchsorted(cu, i, side="right") - 1)
        s, e = _seq_bounds(cu, b)
        cols = np.arange(s, e)
        msk = element_mask(np.array([i]), cols, vecs, causal)[0]
        allowed = cols[~msk]
        if allowed.size == 0:
            continue
        qi = np.asarray(q[i, h, :], np.float64)
        kk = np.asarray(k[allowed, h, :], np.float64)
        vv = np.asarray(v[allowed, h, :], np.float64)
        sc = scale * (kk @ qi)
        mx = sc.max()
        p = np.exp(sc - mx)
        ssum = p.sum()
        outs[t] = (p @ vv) / ssum
        lses[t] = mx + math.log(ssum)
    return outs, lses


# --------------------------------------------------- backward (gradients)
def attention_bwd(q, k, v, dout, cu_seqlens, startend, n_vec: int, causal: bool,
                  scale, chunk: int = 512):
    """Gradients of `attention`'s out with respect to q, k and v for the
    upstream gradient dout, float64.  Returns dq, dk, dv [N, H, D].

    [FM] §3.4: the backward op takes q, k, v, startend_row_indices, out,
    softmax_lse and out_grad and returns the gradients of q, k and v; §4.2:
    FlashMask is exact, so its gradients are those of the dense-mask
    attention.  This is the chain rule through the forward's definition,
    per (sequence, head), over the same allowed keys A_i:
      P_ij   = exp(s_ij - lse_i) for j in A_i, 0 otherwise;
      dv_j   = sum_i P_ij dout_i;
      dP_ij  = <dout_i, v_j>;
      dS_ij  = P_ij (dP_ij - sum_l P_il dP_il)     (softmax Jacobian);
      dq_i   = scale * sum_j dS_ij k_j;   dk_j = scale * sum_i dS_ij q_i.
    P is recomputed here from q and k (nothing is taken from a forward run).
    Rows with no allowed key have constant out = 0: they contribute nothing.
    Pinned by: central finite differences of `attention` on tiny random
    cases (both modes, empty rows), the q = 0 closed form of dv, the
    softmax shift invariance (sum_j dk_j = 0 per sequence and head) and
    packed = separate.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); g = np.asarray(dout, np.float64)
    N, H, D = q.shape
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    dq = np.zeros((N, H, D), np.float64)
    dk = np.zeros((N, H, D), np.float64)
    dv = np.zeros((N, H, D), np.float64)
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        if e <= s:
            continue
        cols = np.arange(s, e)
        for h in range(H):
            kh = k[s:e, h, :]
            vh = v[s:e, h, :]
            for r0 in range(s, e, chunk):
                r1 = min(r0 + chunk, e)
                rows = np.arange(r0, r1)
                sc = scale * (q[r0:r1, h, :] @ kh.T)
                msk = element_mask(rows, cols, vecs, causal)
                sc = np.where(msk, -np.inf, sc)
                mx = sc.max(axis=1, keepdims=True)
                mx = np.where(np.isfinite(mx), mx, 0.0)
                p = np.exp(sc - mx)                       # 0 on masked pairs
                ssum = p.sum(axis=1, keepdims=True)
                p = np.divide(p, ssum, out=np.zeros_like(p), where=ssum > 0)
                gh = g[r0:r1, h, :]
                dv[s:e, h, :] += p.T @ gh
                dp = gh @ vh.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[r0:r1, h, :] = scale * (ds @ kh)
                dk[s:e, h, :] += scale * (ds.T @ q[r0:r1, h, :])
    return dq, dk, dv


def attention_bwd_rows(q, k, v, dout, cu_seqlens, startend, n_vec: int, causal: bool,
                       scale, rows: Sequence[int], heads: Sequence[int]):
    """dq of `attention_bwd` at the given (row, head) pairs only, one row at a
    time from the same definition (for sampled checks at full size):
    dq_i = scale * sum_j P_ij (<dout_i, v_j> - sum_l P_il <dout_i, v_l>) k_j
    over the row's allowed keys.  Returns dq [len(rows), D] in fp64."""
    N, H, D = np.asarray(q).shape
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    out = np.zeros((len(rows), D), np.float64)
    for t, (i, h) in enumerate(zip(rows, heads)):
        b = int(np.searchsorted(cu, i, side="right") - 1)
        s, e = _seq_bounds(cu, b)
        cols = np.arange(s, e)
        allowed = cols[~element_mask(np.array([i]), cols, vecs, causal)[0]]
        if allowed.size == 0:
            continue
        kk = np.asarray(k[allowed, h, :], np.float64)
        vv = np.asarray(v[allowed, h, :], np.float64)
        sc = scale * (kk @ np.asarray(q[i, h, :], np.float64))
        p = np.exp(sc - sc.max())
        p /= p.sum()
        dp = vv @ np.asarray(dout[i, h, :], np.float64)
        out[t] = scale * ((p * (dp - (p * dp).sum())) @ kk)
    return out


# -------------------------------------------------------------- O4 extrema
def extrema(cu_seqlens, startend, n_vec: int, causal: bool, block_k: int):
    """Per-key-block min/max of the four filled vectors.

    [FM] §3.1: the vectors are split by FlashAttention's column-block size
    and the minimum and maximum over each block's columns give eight
    vectors LTStart^{min,max}, LTEnd^{min,max}, UTStart^{min,max},
    UTEnd^{min,max}.  Readings: key blocks start at each sequence's first
    column (varlen tiles are per sequence, [VP] §2) and the last block of a
    sequence is ragged (min/max over its valid columns only).

    Returns kb_off int64 [B+1] (kb_off[b] = number of key blocks of the
    sequences before b) and ext int64 [n_kb, 8] with columns
    (min LTS, max LTS, min LTE, max LTE, min UTS, max UTS, min UTE, max UTE).
    Pinned by: [FM] §3.1's printed block (LTS 13,5,5,5 -> 5/13; LTE
    15,14,14,15 -> 14/15) and brute force.
    """
    cu = np.asarray(cu_seqlens, np.int64)
    N = int(cu[-1])
    vecs = fill_vectors(startend, n_vec, causal, N)
    kb_off = [0]
    rows = []
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        L = e - s
        tc = -(-L // block_k) if L > 0 else 0
        for kb in range(tc):
            c0 = s + kb * block_k
            c1 = min(c0 + block_k, e)
            rec = []
            for vec in vecs:
                seg = vec[c0:c1]
                rec += [int(seg.min()), int(seg.max())]
            rows.append(rec)
        kb_off.append(kb_off[-1] + tc)
    ext = np.array(rows, np.int64).reshape(-1, 8)
    return np.array(kb_off, np.int64), ext


# ------------------------------------------------------------- O5 classes
def classify(cu_seqlens, kb_off, ext, causal: bool, block_q: int, block_k: int):
    """Class of every (sequence, q tile, key block) tile.

    [FM] §3.2: a block is fully masked when its smallest row is at least
    Start^max and its largest row bound is at most End^min (skipped); it is
    partially masked when its smallest row is below End^max and its largest
    row bound is above Start^min (masked element by element); otherwise it
    is unmasked.  The worked examples of [FM] §3.2 give tile [3,2] FULL,
    [1,1] PARTIAL, [3,1] UNMASKED on the 16x16 example with 4x4 tiles.

    Readings:
      * the "largest row" bound is the tile's EXCLUSIVE end r1: with the
        inclusive last row the FULL rule is unsound (a tile whose last row
        sits at End would be skipped);
      * the comparisons lost in the extracted text of the PARTIAL rule are
        strict (<, >): only that makes the printed example true;
      * the causal rule is a third source: a tile is causal-FULL when its
        first column is at or past its row end, and needs causal element
        masking unless its last column is at or before its first row;
      * FULL is tested first, then PARTIAL (the page's order); the upper
        triangle vectors take part only in non-causal mode.
    Tiles are clipped to their sequence (ragged last q tile / key block).

    Returns a list (one per sequence) of int8 arrays [Tr_b, Tc_b].
    """
    cu = np.asarray(cu_seqlens, np.int64)
    out = []
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        L = e - s
        tr = -(-L // block_q) if L > 0 else 0
        tc = -(-L // block_k) if L > 0 else 0
        # tile bounds, clipped to the sequence: rows [r0, r1), cols [c0, c1)
        r0 = (s + np.arange(tr, dtype=np.int64) * block_q)[:, None]
        r1 = np.minimum(r0 + block_q, e)
        c0 = (s + np.arange(tc, dtype=np.int64) * block_k)[None, :]
        c1 = np.minimum(c0 + block_k, e)
        x = ext[kb_off[b]:kb_off[b] + tc]
        lts_min, lts_max, lte_min, lte_max = (x[:, t][None, :] for t in range(4))
        uts_min, uts_max, ute_min, ute_max = (x[:, t][None, :] for t in range(4, 8))
        causal_full = causal & (c0 >= r1)
        causal_none = (not causal) | (c1 <= r0 + 1)
        lt_full = (r0 >= lts_max) & (r1 <= lte_min)
        lt_touch = (r0 < lte_max) & (r1 > lts_min)
        ut_full = (not causal) & (r0 >= uts_max) & (r1 <= ute_min)
        ut_touch = (not causal) & (r0 < ute_max) & (r1 > uts_min)
        full = causal_full | lt_full | ut_full
        partial = (~causal_none) | lt_touch | ut_touch
        cls = np.where(full, FULL, np.where(partial, PARTIAL, UNMASKED)).astype(np.int8)
        cls = cls.reshape(tr, tc)
        out.append(cls)
    return out


def class_counts(classes) -> np.ndarray:
    """(FULL, PARTIAL, UNMASKED) counts over all tiles, once for all heads."""
    c = np.zeros(3, np.int64)
    for cls in classes:
        for t in (FULL, PARTIAL, UNMASKED):
            c[t] += int((cls == t).sum())
    return c


# ------------------------------------------------------------ O6 worklist
def worklist(classes, H: int, max_kb_per_item: int):
    """Compact work items (one per non-empty q tile, head and split).

    [VP] §2: a FlashAttention varlen launch names each thread block's work by
    the triple (sequence, head, q tile) over a fixed grid of
    seq_count x n_head x ceil(max_seq_len / Br) blocks, short sequences
    leaving blocks empty; [VP] §1.2: the grid is fixed at launch and the
    slowest block sets the end.  Here only real q tiles become items,
    long rows may be cut into splits, and items are ordered longest first.

    For every sequence b, head h and q tile qt: K = ascending key blocks
    whose class is not FULL, cost = |K|.  With S = max_kb_per_item, if S == 0
    or cost <= S there is one item covering [K[0], K[-1] + 1) (or [0, 0)
    when K is empty); otherwise K is cut into n = ceil(cost / S) consecutive
    chunks whose sizes differ by at most one, larger chunks first.
    Record: (seq, head, q_tile, kb_begin, kb_end, split_idx, n_splits, cost).
    Order: ascending (-cost, seq, q_tile, split_idx, head).
    These choices (ordering, split rule, record) are the library's own.
    Pinned by: the [VP] §2 count (192 grid blocks for [128,128,4096],
    2 heads, Br=128, against 68 items) and closed forms.
    """
    items = []
    for b, cls in enumerate(classes):
        tr, tc = cls.shape
        for qt in range(tr):
            K = [kb for kb in range(tc) if cls[qt, kb] != FULL]
            cost = len(K)
            if max_kb_per_item == 0 or cost <= max_kb_per_item:
                n = 1
            else:
                n = -(-cost // max_kb_per_item)
            base, extra = divmod(cost, n)
            pos = 0
            for s in range(n):
                size = base + (1 if s < extra else 0)
                if size == 0:
                    kbb, kbe = 0, 0
                else:
                    kbb, kbe = K[pos], K[pos + size - 1] + 1
                pos += size
                for h in range(H):
                    items.append((b, h, qt, kbb, kbe, s, n, size))
    items.sort(key=lambda it: (-it[7], it[0], it[2], it[5], it[1]))
    return np.array(items, np.int64).reshape(-1, 8)


def fa_varlen_grid_blocks(lengths: Sequence[int], H: int, block_q: int) -> int:
    """[VP] §2: blocks of the fixed FA varlen grid,
    seq_count x n_head x ceil(max_seq_len / Br)."""
    return len(lengths) * H * (-(-max(lengths) // block_q))


# --------------------------------------------------------- O7 flop count
def unmasked_pairs(cu_seqlens, startend, n_vec: int, causal: bool, chunk: int = 2048) -> int:
    """Number of (query, key) pairs that attend, per head (the mask is shared
    by all heads).  Counted on the dense element mask of each sequence."""
    cu = np.asarray(cu_seqlens, np.int64)
    N = int(cu[-1])
    vecs = fill_vectors(startend, n_vec, causal, N)
    total = 0
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        cols = np.arange(s, e)
        for r0 in range(s, e, chunk):
            rows = np.arange(r0, min(r0 + chunk, e))
            total += int((~element_mask(rows, cols, vecs, causal)).sum())
    return total


def effective_flops(pairs_per_head: int, H: int, D: int) -> int:
    """Unmasked FLOPs of the forward: QK^T and PV, one multiply-add (2 flop)
    per (query, key, channel) each, i.e. 4*D per attending pair per head.
    The FlashMask article reports TFLOPs/s (§4.4) without defining the
    count; masked pairs and softmax work are not counted."""
    return 4 * D * H * int(pairs_per_head)


# ------------------------------------------------------ rotary embedding
def rope(x, cu_seqlens, cos, sin, inverse: bool = False):
    """Rotary position embedding of packed rows, float64.

    x: [N, H, D] (D even); cos, sin: [max_pos, D/2] tables (any float
    dtype, widened exactly).  Unsloth packing blog, fused QK RoPE section:
    out = x cos + rotate_half(x) sin, where rotate_half(x) = x R with
    R = [[0, I], [-I, 0]] (halves x1 = x[:D/2], x2 = x[D/2:] give
    [-x2, x1]); the tables repeat over the two halves.  Positions restart
    at 0 in every packed sample (the blog's packing section: the kernel
    resets position ids): row i of sequence b has position i - cu[b].
    The backward of the rotation is the same map with sin negated (the
    blog: R^T replaces R), `inverse=True`.
    Pinned by: the 2-D rotation matrix (D = 2), norm preservation of
    every (j, j + D/2) pair, inverse after forward = identity, relative
    positions (<rope(q, m), rope(k, n)> depends only on m - n) and packed =
    separate sequences.
    """
    x = np.asarray(x, np.float64)
    N, H, D = x.shape
    if D % 2:
        raise ValueError("D must be even")
    cu = np.asarray(cu_seqlens, np.int64)
    c = np.asarray(cos, np.float64)
    s = np.asarray(sin, np.float64)
    if inverse:
        s = -s
    pos = np.zeros(N, np.int64)
    for b in range(len(cu) - 1):
        pos[cu[b]:cu[b + 1]] = np.arange(cu[b + 1] - cu[b])
    if N and pos.max() >= c.shape[0]:
        raise ValueError("position beyond the tables")
    cc = np.concatenate([c[pos], c[pos]], axis=1)[:, None, :]
    ss = np.concatenate([s[pos], s[pos]], axis=1)[:, None, :]
    rot = np.concatenate([-x[..., D // 2:], x[..., :D // 2]], axis=-1)
    return x * cc + rot * ss


# --------------------------------------------------------------- dropout
_PH_M0, _PH_M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 multipliers
_PH_W0, _PH_W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
    as easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 products
    and xors with the key, the key advancing by the Weyl constants between
    rounds.  ctr: uint array [..., 4], key: uint array [..., 2] (broadcast);
    returns uint32 [..., 4].  Arithmetic in uint64 (exact products).

    Pinned by an independent implementation, ROCm's rocRAND Philox4x32-10
    engine (compiled for the CPU in the test; blocks and subsequences as
    the counter's two 64-bit halves, carries included), and by statistics
    (uniform bytes, avalanche on one counter bit, unrelated streams for
    different keys, determinism)."""
    c = [np.asarray(ctr[..., i], np.uint64) & np.uint64(0xFFFFFFFF) for i in range(4)]
    k0 = np.asarray(key[..., 0], np.uint64) & np.uint64(0xFFFFFFFF)
    k1 = np.asarray(key[..., 1], np.uint64) & np.uint64(0xFFFFFFFF)
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_PH_W0)) & mask
            k1 = (k1 + np.uint64(_PH_W1)) & mask
        p0 = np.uint64(_PH_M0) * c[0]
        p1 = np.uint64(_PH_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack(c, axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """Dropout probability p in [0, 1) as the byte threshold t = round(256 p)
    (a key is dropped when its byte is below t): the effective drop
    probability is t / 256 and kept values are scaled by 256 / (256 - t)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(p * 256.0 + 0.5)))


def dropout_keep(rows, cols, seq_start, h: int, seed: int, offset: int, t: int):
    """Keep mask [len(rows), len(cols)] of one head: the byte of pair (i, j)
    is byte (j - s) & 15 (little-endian within the four words) of
    Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter
    (i, (j - s) >> 4, h, offset mod 2^32), s the start of the pair's
    sequence; kept when the byte is >= t.  (The pages name the op's
    dropout attribute and seed_offset input, FlashMask article §3.4; this
    counter layout is this library's.)"""
    i = np.asarray(rows, np.int64)[:, None]
    jl = np.asarray(cols, np.int64)[None, :] - int(seq_start)
    ctr = np.stack(np.broadcast_arrays(i, jl >> 4, np.int64(h), np.int64(offset & 0xFFFFFFFF)), axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint64)
    words = philox4x32_10(ctr.astype(np.uint64), key)
    k = jl & 15
    w = np.take_along_axis(words, np.broadcast_to(k >> 2, words.shape[:-1])[..., None], axis=-1)[..., 0]
    byte = (w >> (8 * (k & 3)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= np.uint32(t)


def attention_dropout(q, k, v, cu_seqlens, startend, n_vec: int, causal: bool, scale, p: float,
                      seed: int, offset: int, chunk: int = 512):
    """Forward with attention dropout, float64: the forward's P (normalised
    over the allowed keys, lse unchanged) times the keep mask and
    256 / (256 - t); out = (P o keep * scale_keep) V.  p = 0 gives
    `attention` exactly."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    N, H, D = q.shape
    t = dropout_threshold(p)
    ks = 256.0 / (256.0 - t)
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    out = np.zeros((N, H, D), np.float64)
    lse = np.full((H, N), -np.inf, np.float64)
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        if e <= s:
            continue
        cols = np.arange(s, e)
        for h in range(H):
            for r0 in range(s, e, chunk):
                r1 = min(r0 + chunk, e)
                rows = np.arange(r0, r1)
                sc = scale * (q[r0:r1, h, :] @ k[s:e, h, :].T)
                sc = np.where(element_mask(rows, cols, vecs, causal), -np.inf, sc)
                mx = sc.max(axis=1, keepdims=True)
                ok = np.isfinite(mx[:, 0])
                mx = np.where(np.isfinite(mx), mx, 0.0)
                pe = np.exp(sc - mx)
                ssum = pe.sum(axis=1, keepdims=True)
                pn = np.divide(pe, ssum, out=np.zeros_like(pe), where=ssum > 0)
                keep = dropout_keep(rows, cols, s, h, seed, offset, t)
                out[r0:r1, h, :] = (pn * keep * ks) @ v[s:e, h, :]
                with np.errstate(divide="ignore"):
                    lse[h, r0:r1] = np.where(ok, mx[:, 0] + np.log(np.where(ok, ssum[:, 0], 1.0)), -np.inf)
    return out, lse


def attention_bwd_dropout(q, k, v, dout, cu_seqlens, startend, n_vec: int, causal: bool, scale, p: float,
                          seed: int, offset: int, chunk: int = 512):
    """Gradients of `attention_dropout` (the keep mask is a constant of the
    inputs): with Z = keep * 256 / (256 - t),
      dv_j = sum_i P_ij Z_ij dout_i,   dP_ij = Z_ij <dout_i, v_j>,
      dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
      dq_i = scale sum_j dS_ij k_j,    dk_j = scale sum_i dS_ij q_i.
    Pinned by central finite differences of `attention_dropout`."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); g = np.asarray(dout, np.float64)
    N, H, D = q.shape
    t = dropout_threshold(p)
    ks = 256.0 / (256.0 - t)
    vecs = fill_vectors(startend, n_vec, causal, N)
    cu = np.asarray(cu_seqlens, np.int64)
    scale = float(np.float64(scale))
    dq = np.zeros((N, H, D)); dk = np.zeros((N, H, D)); dv = np.zeros((N, H, D))
    for b in range(len(cu) - 1):
        s, e = _seq_bounds(cu, b)
        if e <= s:
            continue
        cols = np.arange(s, e)
        for h in range(H):
            kh, vh = k[s:e, h, :], v[s:e, h, :]
            for r0 in range(s, e, chunk):
                r1 = min(r0 + chunk, e)
                rows = np.arange(r0, r1)
                sc = scale * (q[r0:r1, h, :] @ kh.T)
                sc = np.where(element_mask(rows, cols, vecs, causal), -np.inf, sc)
                mx = sc.max(axis=1, keepdims=True)
                mx = np.where(np.isfinite(mx), mx, 0.0)
                pe = np.exp(sc - mx)
                ssum = pe.sum(axis=1, keepdims=True)
                pn = np.divide(pe, ssum, out=np.zeros_like(pe), where=ssum > 0)
                z = dropout_keep(rows, cols, s, h, seed, offset, t) * ks
                gh = g[r0:r1, h, :]
                dv[s:e, h, :] += (pn * z).T @ gh
                dp = (gh @ vh.T) * z
                ds = pn * (dp - (pn * dp).sum(axis=1, keepdims=True))
                dq[r0:r1, h, :] = scale * (ds @ kh)
                dk[s:e, h, :] += scale * (ds.T @ q[r0:r1, h, :])
    return dq, dk, dv
