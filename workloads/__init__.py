"""Seeded synthetic inputs for packed, variable-length, interval-masked attention.

This module is shared by the oracle and the GPU path and therefore holds none
of the method's arithmetic: it draws document lengths, writes down the
per-key-column row intervals that *describe* each workload's mask (the input
encoding), and draws q/k/v.  It never fills defaults, reduces extrema,
classifies tiles or computes attention.

Sources for the shapes and structures (cited by page title and section):
  * PaddleNLP FlashMask article (m.nxbn.cn/news/70198):
      §2.2 the 16x16 causal worked example (LTS/LTE table);
      §5.1 shared-question masks (several answers share one prompt);
      §5.2 mixed masks (global + sliding window, prefix-LM);
      §6.7 ZeroPadding: stored row indices are global (a running offset is
           added per packed sample), so every index below is a global row.
  * Varlen-Packing technical document (www.gsyq.cn/news/432802), §2: the
      worked batch of lengths [128, 128, 4096] with 2 heads and Br=128;
      §3: the padded-batch baseline (every sample zero-padded to the longest).
  * Unsloth packing blog (unsloth.ai, "3x faster training + packing"),
      padding-free packing section: the short/long length mix.

Recipe (stated once, used everywhere):
  * lengths come from numpy.random.default_rng(seed) (PCG64), integer draws
    inclusive of both bounds; "draw until filled" clips the last document to
    the tokens that remain;
  * q, k, v come from numpy.random.default_rng(seed + 1), drawn in that order
    as float32 N(0, 1) of shape [N, H, D]; bf16 configs round them to bf16
    with round-to-nearest-even (torch's float32 -> bfloat16 cast);
  * the default seed of config k is 1000 + k.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = ["Workload", "make_config", "make_lengths", "PAGE_LTS", "PAGE_LTE",
           "causal_document_vectors", "shared_question_vectors", "PACKINGS", "packed_as", "rope_tables",
           "prefix_window_vectors", "random_case", "CONFIG_IDS", "extreme_endpoints",
           "extreme_interval_workload", "INT32_MIN", "INT32_MAX"]

# The 16-column causal example of the FlashMask article, §2.2 (its table is
# flattened to a digit string in the extracted text; these are the 16 values
# per row of that table, column 0 first).
PAGE_LTS = [13, 5, 5, 5, 6, 6, 9, 9, 9, 12, 12, 12, 16, 16, 16, 16]
PAGE_LTE = [15, 14, 14, 15, 12, 12, 11, 11, 16, 16, 16, 16, 16, 16, 16, 16]

CONFIG_IDS = (1, 2, 3, 4, 5)

BF16 = "bf16"
F32 = "f32"


@dataclasses.dataclass
class Workload:
    """One packed attention problem.

    cu_seqlens: int32 [B+1]; startend: int32 [n_vec, N] global row indices.
    q/k/v are float32 numpy arrays [N, H, D] holding exactly the values the
    GPU sees (already rounded to bf16 when dtype == "bf16").
    """
    name: str
    N: int
    H: int
    D: int
    dtype: str
    causal: bool
    n_vec: int
    cu_seqlens: np.ndarray
    startend: np.ndarray
    scale: np.float32
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 -> float32, round-to-nearest-even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def draw_qkv(seed: int, N: int, H: int, D: int, dtype: str):
    rng = np.random.default_rng(seed + 1)
    out = []
    for _ in range(3):
        a = rng.standard_normal((N, H, D), dtype=np.float32)
        if dtype == BF16:
            a = _round_bf16(a)
        out.append(a)
    return out


def _fill_until(rng, N: int, draw_one) -> List[int]:
    lens: List[int] = []
    total = 0
    while total < N:
        L = int(draw_one(rng))
        L = min(L, N - total)
        lens.append(L)
        total += L
    return lens


def make_lengths(k: int, seed: int, N: Optional[int] = None) -> List[int]:
    """Document lengths of config k (configs 3 and 5 take an optional N)."""
    rng = np.random.default_rng(seed)
    if k == 1:
        return [16]
    if k == 2:
        return [128, 128, 4096]
    if k == 3:
        N = 16384 if N is None else N

        def one(r):
            if r.random() < 0.8:
                return r.integers(64, 512, endpoint=True)
            return r.integers(2048, 8192, endpoint=True)
        return _fill_until(rng, N, one)
    if k == 5:
        N = 131072 if N is None else N
        return _fill_until(rng, N, lambda r: r.integers(4096, 32768, endpoint=True))
    raise ValueError("config %d has group structure; use make_config" % k)


def causal_document_vectors(cu: np.ndarray, n_vec: int, N: int) -> np.ndarray:
    """Causal document mask: each key column is masked for rows at or after
    the end of its own document (LTS = document end); LTE is either the
    default (n_vec = 1) or written out as N (n_vec = 2)."""
    cu = np.asarray(cu, dtype=np.int64)
    lts = np.empty(N, np.int64)
    for b in range(len(cu) - 1):
        lts[cu[b]:cu[b + 1]] = cu[b + 1]
    rows = [lts]
    if n_vec == 2:
        rows.append(np.full(N, N, np.int64))
    return np.stack(rows).astype(np.int32)


def shared_question_vectors(groups, N: int) -> np.ndarray:
    """Shared-question (DPO/RM) mask of the FlashMask article §5.1/§6.7.

    groups: list of (group_start, [segment ends...]) with the prompt first.
    Prompt keys are visible to every row of the group (LTS = group end);
    an answer's keys are hidden from rows after that answer (LTS = answer
    end), so sibling answers never see each other.  LTE = N.
    """
    lts = np.empty(N, np.int64)
    for g_start, ends in groups:
        g_end = ends[-1]
        prev = g_start
        for si, e in enumerate(ends):
            lts[prev:e] = g_end if si == 0 else e
            prev = e
    lte = np.full(N, N, np.int64)
    return np.stack([lts, lte]).astype(np.int32)


def prefix_window_vectors(cu: np.ndarray, prefix: List[int], W: int, N: int) -> np.ndarray:
    """Prefix-LM + sliding-window mask (FlashMask article §5.2), non-causal,
    all four vectors.  For a document [s, e) with bidirectional prefix p:
      prefix key j:  UT = [0, s)              LT = [min(max(s+p, j+W), e), N)
      suffix key j:  UT = [0, j)              LT = [min(j+W, e), N)
    so prefix rows see the whole prefix, and a suffix row i sees key j
    (prefix or suffix, j <= i) only while i - j < W."""
    lts = np.empty(N, np.int64); lte = np.full(N, N, np.int64)
    uts = np.zeros(N, np.int64); ute = np.empty(N, np.int64)
    cu = np.asarray(cu, dtype=np.int64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        p = int(prefix[b])
        j = np.arange(s, e, dtype=np.int64)
        pre = j < s + p
        lts[s:e] = np.where(pre, np.minimum(np.maximum(s + p, j + W), e),
                            np.minimum(j + W, e))
        ute[s:e] = np.where(pre, s, j)
    return np.stack([lts, lte, uts, ute]).astype(np.int32)


def make_config(k: int, seed: Optional[int] = None, with_qkv: bool = True,
                N: Optional[int] = None, H: Optional[int] = None) -> Workload:
    """Workload of config k (1..5).  N and H may be reduced for tests; the
    structure (length mix, mask form) stays that of the config."""
    seed = 1000 + k if seed is None else seed
    if k == 1:
        N_, H_, D_ = 16, 1, 32
        cu = np.array([0, 16], np.int32)
        sv = np.array([PAGE_LTS, PAGE_LTE], np.int32)
        w = Workload("cfg1_page_16x16", N_, H_, D_, F32, True, 2, cu, sv,
                     np.float32(1.0 / np.sqrt(np.float32(D_))))
    elif k == 2:
        lens = [128, 128, 4096]
        N_ = sum(lens); H_ = 2 if H is None else H; D_ = 128
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        w = Workload("cfg2_varlen_128_128_4096", N_, H_, D_, BF16, True, 2, cu,
                     causal_document_vectors(cu, 2, N_), np.float32(1.0 / np.sqrt(np.float32(D_))))
    elif k == 3:
        N_ = 16384 if N is None else N; H_ = 32 if H is None else H; D_ = 128
        lens = make_lengths(3, seed, N_)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        w = Workload("cfg3_sft_packing_%d" % N_, N_, H_, D_, BF16, True, 1, cu,
                     causal_document_vectors(cu, 1, N_), np.float32(1.0 / np.sqrt(np.float32(D_))))
    elif k == 4:
        N_ = 32768 if N is None else N; H_ = 32 if H is None else H; D_ = 128
        rng = np.random.default_rng(seed)
        groups = []
        bounds = [0]
        total = 0
        while total < N_:
            segs = [int(rng.integers(512, 2048, endpoint=True))]
            segs += [int(rng.integers(256, 1024, endpoint=True)) for _ in range(4)]
            ends = []
            pos = total
            for L in segs:
                if pos >= N_:
                    break
                pos = min(pos + L, N_)
                ends.append(pos)
            groups.append((total, ends))
            total = ends[-1]
            bounds.append(total)
        cu = np.array(bounds, np.int32)
        w = Workload("cfg4_shared_question_%d" % N_, N_, H_, D_, BF16, True, 2, cu,
                     shared_question_vectors(groups, N_), np.float32(1.0 / np.sqrt(np.float32(D_))))
        w.meta["groups"] = groups
    elif k == 5:
        N_ = 131072 if N is None else N; H_ = 8 if H is None else H; D_ = 128
        W = 4096
        rng = np.random.default_rng(seed)
        lens = _fill_until(rng, N_, lambda r: r.integers(4096, 32768, endpoint=True))
        # prefix fractions: drawn after all lengths, from the same generator
        prefix = [int(np.floor(rng.uniform(0.1, 0.5) * L)) for L in lens]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        w = Workload("cfg5_prefix_window_%d" % N_, N_, H_, D_, BF16, False, 4, cu,
                     prefix_window_vectors(cu, prefix, W, N_), np.float32(1.0 / np.sqrt(np.float32(D_))))
        w.meta.update(prefix=prefix, window=W)
    else:
        raise ValueError("unknown config %r" % k)
    w.meta["seed"] = seed
    w.meta["config"] = k
    if with_qkv:
        w.q, w.k, w.v = draw_qkv(seed, w.N, w.H, w.D, w.dtype)
    return w


def document_workload(lengths: List[int], H: int = 2, D: int = 128, seed: int = 1002,
                      with_qkv: bool = True) -> Workload:
    """Causal documents of the given lengths, encoded as the varlen workload
    encodes them (n_vec = 2: LTS = end of the key's document, LTE = N), bf16
    q/k/v from `seed`: the varlen workload with its documents resized."""
    lens = [int(x) for x in lengths]
    N_ = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    w = Workload("docs_%dx_%d" % (len(lens), N_), N_, H, D, BF16, True, 2, cu,
                 causal_document_vectors(cu, 2, N_), np.float32(1.0 / np.sqrt(np.float32(D))))
    w.meta["seed"] = seed
    if with_qkv:
        w.q, w.k, w.v = draw_qkv(seed, w.N, w.H, w.D, w.dtype)
    return w


INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1


def extreme_endpoints(N: int):
    """Endpoint values at and beyond the ends of the int32 range and of the
    token axis: every int32 is a legal endpoint (half-open intervals,
    start >= end empty; FlashMask article §2.1, §2.2)."""
    return np.array([INT32_MIN, INT32_MIN + 1, -1, 0, N, N + 7, INT32_MAX], np.int64)


def extreme_interval_workload(lengths: List[int], causal: bool, n_vec: int, H: int = 2, D: int = 128,
                              seed: int = 31, with_qkv: bool = True) -> Workload:
    """Documents of the given lengths whose column intervals use endpoints at
    the int32 limits and past the token axis, arranged so that q tiles after
    the first of a long document are cut by them: for a key j of document
    [s, e), one interval in three is [INT32_MIN or -1, r), one in three
    [r, N + 7 or INT32_MAX) with r a random row of [j, e] (of [s, e] for
    the upper triangle), and the rest are empty ([0, 0)).  Causal n_vec = 1
    stores LTS only (LTE = N), drawn as described at that branch.
    bf16 q/k/v from `seed`."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lengths]
    N_ = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    lo_vals = np.array([INT32_MIN, -1], np.int64)
    hi_vals = np.array([N_ + 7, INT32_MAX], np.int64)

    def draw(s, e, first):
        kind = rng.integers(0, 3, size=e - s)
        r = np.array([rng.integers(j if first is None else s, e, endpoint=True) for j in range(s, e)], np.int64)
        st = np.where(kind == 0, lo_vals[rng.integers(0, 2, e - s)], np.where(kind == 1, r, 0))
        en = np.where(kind == 0, r, np.where(kind == 1, hi_vals[rng.integers(0, 2, e - s)], 0))
        return st, en

    lts = np.zeros(N_, np.int64); lte = np.zeros(N_, np.int64)
    uts = np.zeros(N_, np.int64); ute = np.zeros(N_, np.int64)
    for b in range(len(lens)):
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        lts[s:e], lte[s:e] = draw(s, e, None)
        uts[s:e], ute[s:e] = draw(s, e, True)
    if causal and n_vec == 1:
        # LTE = N implicitly, so [LTS, N): half the keys hide the rows from a
        # row r of [j, e] on, 35 % hide nothing (LTS = N + 7 or INT32_MAX),
        # 15 % hide every row (LTS = INT32_MIN or -1)
        u = rng.random(N_)
        r = np.array([rng.integers(j, cu[np.searchsorted(cu, j, side="right")], endpoint=True)
                      for j in range(N_)], np.int64)
        lts = np.where(u < 0.5, r, np.where(u < 0.85, hi_vals[rng.integers(0, 2, N_)],
                                            lo_vals[rng.integers(0, 2, N_)]))
        sv = np.stack([lts])
    elif causal:
        sv = np.stack([lts, lte])
    elif n_vec == 2:
        sv = np.stack([lts, ute])
    else:
        sv = np.stack([lts, lte, uts, ute])
    sv = sv.astype(np.int32)
    w = Workload("extreme_%s%d_%dx%d" % ("c" if causal else "n", n_vec, len(lens), N_), N_, H, D, BF16, causal,
                 n_vec, cu, sv, np.float32(1.0 / np.sqrt(np.float32(D))))
    w.meta["seed"] = seed
    if with_qkv:
        w.q, w.k, w.v = draw_qkv(seed, w.N, w.H, w.D, w.dtype)
    return w


def random_case(seed: int, N_max: int = 64, H: int = 1, D: int = 16,
                causal: Optional[bool] = None, n_vec: Optional[int] = None,
                dtype: str = F32, with_qkv: bool = True, allow_empty: bool = True,
                extreme: bool = False) -> Workload:
    """Tiny adversarial case: random sequence lengths (zero-length ones
    included), random interval endpoints in [0, N] including empty and
    reversed intervals.  Used for brute-force checks.  extreme=True then
    replaces about a third of the stored endpoints by values from
    `extreme_endpoints` (int32 limits, -1, 0, N, N + 7)."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, N_max, endpoint=True))
    n_cuts = int(rng.integers(0, 5, endpoint=True))
    cuts = sorted(int(x) for x in rng.integers(0, N, size=n_cuts, endpoint=True))
    cu = np.array([0] + cuts + [N], np.int32)
    if not allow_empty:
        cu = np.unique(cu).astype(np.int32)
    if causal is None:
        causal = bool(rng.integers(0, 1, endpoint=True))
    if n_vec is None:
        n_vec = int(rng.choice([1, 2]) if causal else rng.choice([2, 4]))
    sv = rng.integers(0, N, size=(n_vec, N), endpoint=True).astype(np.int32)
    # bias some columns towards tidy intervals around their own index
    j = np.arange(N)
    tidy = rng.random(N) < 0.5
    sv[0] = np.where(tidy, np.minimum(j + rng.integers(0, 8, N), N), sv[0])
    if extreme:
        ext = extreme_endpoints(N)
        pick = rng.random(sv.shape) < 0.35
        sv = np.where(pick, ext[rng.integers(0, len(ext), size=sv.shape)], sv.astype(np.int64)).astype(np.int32)
    w = Workload(("random_x%d" if extreme else "random_%d") % seed, N, H, D, dtype, causal, n_vec, cu, sv,
                 np.float32(rng.uniform(0.05, 0.5)))
    w.meta["seed"] = seed
    if with_qkv:
        w.q, w.k, w.v = draw_qkv(seed, N, H, D, dtype)
    return w


PACKINGS = ("varlen", "mask_only", "padded", "padded_masked")


def packed_as(w: Workload, kind: str) -> Workload:
    """The causal documents of `w` (one sequence per document, LTS = the
    document's end) laid out as one of the packings the pages compare:

      varlen         w itself: documents back to back, one sequence each
                     (Varlen-Packing document, §2);
      mask_only      the same tokens and vectors with cu = [0, N]: only the
                     mask keeps documents apart (FlashMask article §6.7,
                     ZeroPadding packing);
      padded         each document right-padded with zero tokens to the
                     longest one, one sequence per document, plain causal
                     mask (Varlen-Packing document §3, the padded baseline):
                     pad rows are attended like real ones;
      padded_masked  the padded layout whose mask also removes the padding:
                     every column of a sample gets LTS = the end of the
                     sample's real tokens (LTE defaults to N), so pad rows
                     attend nowhere (out = 0, lse = -inf) and no real row
                     sees a pad key (they lie above its diagonal).

    meta["real_rows"] holds, in w's token order, the rows of the new layout
    that carry w's tokens; q, k, v of pad rows are zero."""
    if kind not in PACKINGS:
        raise ValueError("unknown packing %r" % (kind,))
    if not w.causal:
        raise ValueError("packings are defined for causal document workloads")
    cu = w.cu_seqlens.astype(np.int64)
    if kind == "varlen":
        out = dataclasses.replace(w, meta=dict(w.meta))
        out.meta.update(packing=kind, real_rows=np.arange(w.N, dtype=np.int64))
        return out
    if kind == "mask_only":
        out = dataclasses.replace(w, name=w.name + "_mask_only", cu_seqlens=np.array([0, w.N], np.int32),
                                  meta=dict(w.meta))
        out.meta.update(packing=kind, real_rows=np.arange(w.N, dtype=np.int64))
        return out
    lens = np.diff(cu)
    Lmax = int(lens.max()) if lens.size else 0
    B = int(lens.size)
    Np = B * Lmax
    cu_p = (np.arange(B + 1, dtype=np.int64) * Lmax).astype(np.int32)
    real = np.concatenate([b * Lmax + np.arange(int(lens[b]), dtype=np.int64) for b in range(B)]) \
        if B else np.zeros(0, np.int64)
    if kind == "padded":
        sv = np.full((1, Np), Np, np.int32)     # [N, N): empty, a plain causal mask
    else:
        sv = np.repeat((np.arange(B, dtype=np.int64) * Lmax + lens).astype(np.int32), Lmax)[None, :]

    def spread(a):
        if a is None:
            return None
        z = np.zeros((Np,) + a.shape[1:], a.dtype)
        z[real] = a
        return z
    out = Workload(w.name + "_" + kind, Np, w.H, w.D, w.dtype, True, 1, cu_p, sv, w.scale,
                   spread(w.q), spread(w.k), spread(w.v), dict(w.meta))
    out.meta.update(packing=kind, real_rows=real)
    return out


def rope_tables(max_pos: int, D: int, base: float = 10000.0):
    """cos / sin tables [max_pos, D/2] (float32) of the usual rotary angles
    p * base^(-2j / D): the input the rotary kernel reads (the pages leave
    the angles to the model; this is the common choice)."""
    j = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-2.0 * j / D)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
