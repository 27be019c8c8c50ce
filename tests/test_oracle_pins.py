"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one step of the path (blocking, summary, estimate, selection,
attention) with a closed form, brute force on tiny inputs, an independent
library routine (torch's scaled_dot_product_attention in fp64) or an
invariant that the mathematics forces.  The last group plants plausible
mistakes in copies of oracle steps and checks that a pin catches each one.

Sources: SPADE technical summary (gist.science page), "Methodology 1.
vDiT-SSR" (3D blocks; Summarizer & Estimator) and "3. Head-wise Sparse
Attention Execution" (flash block-sparse attention, online softmax).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Geometry
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(cfg, x):
    return synth.bf16_bits_to_f64(x) if cfg.dtype == "bf16" else x.astype(np.float64)


def _inputs(name, **kw):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg, **kw)
    g = Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    return cfg, g, {k: _f64(cfg, v) for k, v in x.items()}


# ---------------------------------------------------------------------------
# blocking
# ---------------------------------------------------------------------------

def _read_census(path):
    grid = block = None
    sizes = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = [s.strip() for s in line.split("=", 1)]
            if key == "grid":
                grid = tuple(int(v) for v in val.split("x"))
            elif key == "block":
                block = tuple(int(v) for v in val.split("x"))
            else:
                sizes[int(key)] = int(val)
    return grid, block, sizes


def test_ragged_block_census_golden():
    grid, block, sizes = _read_census(os.path.join(GOLDEN, "ragged_block_census.txt"))
    g = Geometry(*grid, *block)
    toks = oracle.block_tokens(g)
    got = {}
    for t in toks:
        got[len(t)] = got.get(len(t), 0) + 1
    assert got == sizes
    assert sum(k * v for k, v in sizes.items()) == g.N


@pytest.mark.parametrize("name", sorted(synth.TEST_CONFIGS) + ["mid", "large", "ragged", "small"])
def test_blocks_partition_grid_into_boxes(name):
    cfg = synth.get_config(name)
    g = Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    ids = oracle.token_block_ids(g)
    assert (ids >= 0).all()
    toks = oracle.block_tokens(g)
    assert sum(len(t) for t in toks) == g.N
    assert len(toks) == g.nblk
    n = np.arange(g.N)
    t, h, w = n // (g.Hh * g.W), (n // g.W) % g.Hh, n % g.W
    nT, nH, nW = g.counts
    # closed form: the block of token (t, h, w) is (t//bt, h//bh, w//bw)
    expect = ((t // g.bt) * nH + (h // g.bh)) * nW + (w // g.bw)
    assert (ids == expect).all()


# ---------------------------------------------------------------------------
# summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged_p64", "mid_shape", "ragged_small", "big_block"])
def test_summary_closed_form_on_affine_field(name):
    """x[n, c] = a_c t + b_c h + e_c w + f_c: the block mean is that affine map
    at the block's centre ((t0 + t1 - 1)/2, ...)."""
    cfg = synth.get_config(name)
    g = Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    d = 8
    rng = np.random.default_rng(0)
    coef = rng.integers(-3, 4, size=(4, d)).astype(np.float64)
    n = np.arange(g.N)
    t, h, w = n // (g.Hh * g.W), (n // g.W) % g.Hh, n % g.W
    x = (t[:, None] * coef[0] + h[:, None] * coef[1] + w[:, None] * coef[2] + coef[3])
    x = x[None, None]
    got = oracle.summarize(x, g, store_f32=False)[0, 0]
    for j, (t0, t1, h0, h1, w0, w1) in enumerate(oracle.block_extents(g)):
        centre = np.array([(t0 + t1 - 1) / 2, (h0 + h1 - 1) / 2, (w0 + w1 - 1) / 2, 1.0])
        np.testing.assert_allclose(got[j], centre @ coef, rtol=0, atol=1e-12)


def test_summary_stored_f32_is_rounded_exact_mean():
    cfg, g, x = _inputs("ragged_small")
    m64 = oracle.summarize(x["q"], g, store_f32=False)
    m32 = oracle.summarize(x["q"], g, store_f32=True)
    assert (m32 == m64.astype(np.float32).astype(np.float64)).all()
    # bf16 inputs: the fp64 sum of the block is exact, so the fp64 mean is the
    # correctly rounded quotient of an exact sum; check against exact fractions
    from fractions import Fraction
    toks = oracle.block_tokens(g)
    for j in (0, len(toks) - 1):
        for c in (0, 5):
            vals = x["q"][1, 1, toks[j], c]
            exact = sum(Fraction(float(v)) for v in vals) / len(vals)
            assert m64[1, 1, j, c] == float(exact)


# ---------------------------------------------------------------------------
# estimate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged_p64", "ragged_small"])
def test_estimate_is_block_mean_of_token_logits(name):
    """Bilinearity: scale * <mean q, mean k> equals the mean of the token-level
    logits scale * q_a . k_b over the block pair."""
    cfg, g, x = _inputs(name)
    scale = oracle.default_scale(cfg.d)
    qm = oracle.summarize(x["q"], g, store_f32=False)
    km = oracle.summarize(x["k"], g, store_f32=False)
    S = oracle.estimate(qm, km, scale)
    toks = oracle.block_tokens(g)
    b, h = cfg.B - 1, cfg.H - 1
    L = scale * x["q"][b, h] @ x["k"][b, h].T
    for i in range(0, g.nblk, max(1, g.nblk // 5)):
        for j in range(0, g.nblk, max(1, g.nblk // 7)):
            ref = L[np.ix_(toks[i], toks[j])].mean()
            assert abs(S[b, h, i, j] - ref) <= 1e-12 * (1 + abs(ref))


def test_hand_worked_example():
    """Grid 1x2x4, block 1x2x2 (two blocks: tokens {0,1,4,5} and {2,3,6,7}),
    d = 2, keep 1 block.  Worked by hand:
      block-0 keys (1,0),(0,0),(1,0),(2,0) -> mean (1,0); block-1 keys (0,1) -> mean (0,1);
      block-0 queries (2,0) -> mean (2,0); block-1 queries (0,0) -> mean (0,0).
      S = (1/sqrt 2) [[2, 0], [0, 0]]: row 0 keeps block 0 (margin sqrt 2);
      row 1 is a tie and keeps the lower id, block 0.
      Block-0 queries see logits (2,0,2,4)/sqrt 2 over keys 0,1,4,5; block-1
      queries see all-zero logits, i.e. the plain mean of block-0 values."""
    g = Geometry(1, 2, 4, 1, 2, 2)
    q = np.zeros((1, 1, 8, 2))
    q[0, 0, [0, 1, 4, 5]] = [2, 0]
    k = np.zeros((1, 1, 8, 2))
    k[0, 0, [0, 1, 4, 5]] = [[1, 0], [0, 0], [1, 0], [2, 0]]
    k[0, 0, [2, 3, 6, 7]] = [0, 1]
    v = np.arange(16, dtype=np.float64).reshape(1, 1, 8, 2)
    O, sel, S = oracle.spade_attn(q, k, v, g, "count", [1])
    r2 = math.sqrt(2.0)
    np.testing.assert_allclose(S[0, 0], [[r2, 0.0], [0.0, 0.0]], atol=1e-15)
    assert sel.row(0).tolist() == [0] and sel.row(1).tolist() == [0]
    assert abs(sel.margins[0] - r2) < 1e-15 and sel.margins[1] == 0.0
    wts = np.exp(np.array([2, 0, 2, 4]) / r2)
    vb0 = v[0, 0, [0, 1, 4, 5]]
    o0 = (wts[:, None] * vb0).sum(0) / wts.sum()
    for n in (0, 1, 4, 5):
        np.testing.assert_allclose(O[0, 0, n], o0, atol=1e-13)
    for n in (2, 3, 6, 7):
        np.testing.assert_allclose(O[0, 0, n], vb0.mean(0), atol=1e-13)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _random_rows(n_rows, nK, seed):
    rng = np.random.default_rng(seed)
    S = rng.normal(size=(n_rows, nK))
    S[::5] = np.round(S[::5], 1)  # some rows with ties
    return S


@pytest.mark.parametrize("k", [1, 3, 5, 8])
def test_topk_equals_bruteforce_subset(k):
    nK = 8
    S = _random_rows(40, nK, seed=k)
    sel = oracle.select(S[None, None], "count", [k])
    for r in range(S.shape[0]):
        best = None
        for sub in itertools.combinations(range(nK), k):
            key = (S[r, list(sub)].sum(), [-j for j in sub])
            if best is None or key > best[0]:
                best = (key, sub)
        sums = sorted({round(S[r, list(s)].sum(), 12) for s in itertools.combinations(range(nK), k)})
        if sel.margins[r] > 1e-9:
            assert tuple(sel.row(r).tolist()) == best[1]
            assert len(sums) == 1 or sums[-1] - sums[-2] > 1e-12 or k == nK
        else:
            # tie at the boundary: the kept sum is still maximal
            assert abs(S[r, sel.row(r)].sum() - best[0][0]) < 1e-12


def test_tiny_topk_bruteforce():
    cfg, g, x = _inputs("tiny")
    scale = oracle.default_scale(cfg.d)
    S = oracle.estimate(oracle.summarize(x["q"], g), oracle.summarize(x["k"], g), scale)
    sel = oracle.select(S, "count", [3, 3])
    Sr = S.reshape(-1, g.nblk)
    for r in range(Sr.shape[0]):
        sub = max(itertools.combinations(range(8), 3), key=lambda s: Sr[r, list(s)].sum())
        assert sel.margins[r] > 1e-3
        assert tuple(sel.row(r).tolist()) == sub


@pytest.mark.parametrize("tau", [0.05, 0.3, 0.5, 0.9, 0.99, 1.0])
def test_mass_equals_bruteforce_minimal_subset(tau):
    """Smallest subset whose softmax mass reaches tau; among those, the one of
    largest mass.  The greedy prefix is that subset."""
    nK = 8
    S = _random_rows(30, nK, seed=int(tau * 100)) * 2.0
    sel = oracle.select(S[None, None], "mass", [tau])
    tau32 = float(np.float32(tau))
    for r in range(S.shape[0]):
        p = np.exp(S[r] - S[r].max())
        p = p / p.sum()
        best = None
        for m in range(1, nK + 1):
            cands = [s for s in itertools.combinations(range(nK), m) if p[list(s)].sum() >= tau32 - 1e-15]
            if cands:
                best = max(cands, key=lambda s: (p[list(s)].sum(), [-j for j in s]))
                break
        if best is None:
            best = tuple(range(nK))
        if sel.margins[r] > 1e-9:
            assert tuple(sel.row(r).tolist()) == best


def test_mass_prefix_monotone_in_tau():
    S = _random_rows(50, 16, seed=3)
    prev = None
    for tau in (0.1, 0.4, 0.7, 0.95):
        sel = oracle.select(S[None, None], "mass", [tau])
        if prev is not None:
            for r in range(S.shape[0]):
                assert set(prev.row(r).tolist()) <= set(sel.row(r).tolist())
        prev = sel


def test_zero_queries_tie_break_lowest_block_ids():
    cfg, g, x = _inputs("ragged_small")
    q = np.zeros_like(x["q"])
    scale = oracle.default_scale(cfg.d)
    S = oracle.estimate(oracle.summarize(q, g), oracle.summarize(x["k"], g), scale)
    assert (S == 0).all()
    k = oracle.keep_count("ratio", 0.5, g.nblk)
    sel = oracle.select(S, "ratio", [0.5, 0.5])
    for r in range(len(sel.counts)):
        assert sel.row(r).tolist() == list(range(k))
    sel = oracle.select(S, "mass", [0.5, 0.25])
    for r in range(len(sel.counts)):
        h = (r // g.nblk) % cfg.H
        tau = (0.5, 0.25)[h]
        assert sel.row(r).tolist() == list(range(math.ceil(tau * g.nblk)))


def test_keep_count_ratio_rounding():
    assert oracle.keep_count("ratio", 0.25, 455) == 114
    assert oracle.keep_count("ratio", 0.15, 990) == 149
    assert oracle.keep_count("ratio", 0.1, 336) == 34
    assert oracle.keep_count("ratio", 0.5, 336) == 168
    assert oracle.keep_count("ratio", 1.0, 336) == 336
    assert oracle.keep_count("ratio", 0.1, 10) == 1
    assert oracle.keep_count("ratio", 1e-9, 10) == 1


def test_margin_bounds_flip_distance():
    """Perturbing S by less than a fraction of the margin never changes the
    kept set.  Top-k: every score moves by < margin / 2, so the k-th and
    (k+1)-th stay apart.  Mass: with every score moved by at most eps, the
    mass of any fixed subset changes by a factor within exp(+-2 eps), so the
    mass of the best (k-1)- and k-subsets moves by at most exp(2 eps) - 1; for
    eps = 0.1 m that is < 0.23 m, below both mass terms of the margin, and
    2 eps < the score gap, so the prefix length and the kept set stay."""
    S = _random_rows(60, 12, seed=9)
    rng = np.random.default_rng(1)
    checked = {"count": 0, "mass": 0}
    for mode, val in (("count", 4), ("mass", 0.8)):
        sel = oracle.select(S[None, None], mode, [val])
        for r in range(S.shape[0]):
            m = sel.margins[r]
            if not np.isfinite(m) or m <= 1e-9:
                continue
            eps = 0.45 * m if mode == "count" else 0.1 * m
            for _ in range(4):
                pert = S[r] + rng.uniform(-eps, eps, size=S.shape[1])
                sel2 = oracle.select(pert[None, None, None], mode, [val])
                assert sel2.row(0).tolist() == sel.row(r).tolist(), (mode, r, m)
            checked[mode] += 1
    assert checked["count"] > 20 and checked["mass"] > 20


# Hand-worked mass rows (softmax weights in closed form): with
# S = [ln 4, ln 2, 0, 0] the weights are [4, 2, 1, 1] / 8, so the cumulative
# masses in score order are C = [1/2, 3/4, 7/8, 1].
#  * tau = 0.6 keeps 2 blocks (C_1 = 0.5 < 0.6 <= C_2 = 0.75); the three terms
#    are S_(2) - S_(3) = ln 2, C_2 - tau = 0.15, tau - C_1 = 0.1: margin 0.1.
#  * tau = 0.72 keeps 2 blocks; terms ln 2, 0.03, 0.22: margin 0.03.
#  * S = [ln 4, ln 2 + 0.01, ln 2, 0] with tau = 0.5: Z = 7 + 2 e^0.01, C_1 =
#    4 / Z < 0.5 <= C_2, terms 0.01, C_2 - 0.5 = 0.167..., 0.5 - 4/Z = 0.0565...:
#    margin 0.01 (the score gap).
MASS_ROWS = [
    ([math.log(4), math.log(2), 0.0, 0.0], 0.6, 2, lambda t: t - 0.5),
    ([math.log(4), math.log(2), 0.0, 0.0], 0.72, 2, lambda t: 0.75 - t),
    ([math.log(4), math.log(2) + 0.01, math.log(2), 0.0], 0.5, 2, lambda t: 0.01),
]


@pytest.mark.parametrize("row,tau,k,margin", MASS_ROWS)
def test_mass_margin_hand_worked(row, tau, k, margin):
    """Each of the three mass-margin terms is the binding one on one row (tau
    is taken as its fp32 value, the boundary's budget type)."""
    S = np.array(row)[None, None, None]
    sel = oracle.select(S, "mass", [tau])
    assert sel.counts[0] == k
    assert abs(sel.margins[0] - margin(float(np.float32(tau)))) < 1e-12


def _mass_margin_variant(row, tau, drop=None, unnormalised=False):
    """The mass margin restated with one planted mistake: a dropped term
    ("gap", "above", "below") or the cumulative mass compared unnormalised."""
    s = np.sort(np.asarray(row, dtype=np.float64))[::-1]
    p = np.exp(s - s[0])
    Z = p.sum()
    c = np.cumsum(p) if unnormalised else np.cumsum(p) / Z
    k = int(np.nonzero(c >= tau)[0][0]) + 1 if (c >= tau).any() else len(s)
    terms = {"gap": s[k - 1] - s[k] if k < len(s) else math.inf,
             "above": c[k - 1] - tau,
             "below": tau - (c[k - 2] if k >= 2 else 0.0)}
    if drop is not None:
        del terms[drop]
    return min(terms.values())


@pytest.mark.parametrize("drop,unnormalised", [("gap", False), ("above", False), ("below", False), (None, True)])
def test_planted_mass_margin_mistakes_are_caught(drop, unnormalised):
    """Dropping any one term of the mass margin, or comparing unnormalised
    cumulative mass against tau, gives a wrong value on one of the
    hand-worked rows."""
    for row, tau, _, m in MASS_ROWS:  # the restatement itself is right
        assert abs(_mass_margin_variant(row, tau) - m(tau)) < 1e-12
    wrong = [abs(_mass_margin_variant(row, tau, drop, unnormalised) - m(tau)) > 1e-6 for row, tau, _, m in MASS_ROWS]
    assert any(wrong)


def test_shift_of_all_keys_leaves_selection_and_attention():
    cfg, g, x = _inputs("ragged_p64")
    u = np.random.default_rng(5).normal(size=cfg.d)
    O1, s1, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, "ratio", cfg.per_head_budget())
    O2, s2, _ = oracle.spade_attn(x["q"], x["k"] + u, x["v"], g, "ratio", cfg.per_head_budget())
    for r in range(len(s1.counts)):
        if s1.margins[r] > 1e-6:
            assert s1.row(r).tolist() == s2.row(r).tolist()
    # attention on the same CSR is unchanged by the shift
    O3 = oracle.attention_full(x["q"], x["k"] + u, x["v"], g, s1.row_ptr, s1.col_idx,
                               oracle.default_scale(cfg.d))
    np.testing.assert_allclose(O3, O1, atol=1e-10)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, scale, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else t(mask), scale=scale).numpy()


@pytest.mark.parametrize("name", ["tiny", "ragged_small", "ragged_p64"])
def test_ratio_one_is_dense_attention(name):
    cfg, g, x = _inputs(name)
    scale = oracle.default_scale(cfg.d)
    O, sel, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, "ratio", [1.0] * cfg.H)
    assert (sel.counts == g.nblk).all()
    D = oracle.dense_attention(x["q"], x["k"], x["v"], scale)
    ref = _sdpa(x["q"], x["k"], x["v"], scale)
    np.testing.assert_allclose(D, ref, atol=1e-12)
    np.testing.assert_allclose(O, ref, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "ragged_small", "mid_shape"])
def test_block_sparse_equals_explicit_token_mask(name):
    cfg, g, x = _inputs(name)
    scale = oracle.default_scale(cfg.d)
    O, sel, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, cfg.mode, cfg.per_head_budget())
    blk = oracle.token_block_ids(g)
    mask = np.zeros((cfg.B, cfg.H, g.N, g.N), dtype=bool)
    for r in range(len(sel.counts)):
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, cfg.H)
        keep = np.isin(blk, sel.row(r))
        mask[b, h, np.nonzero(blk == i)[0][:, None], np.nonzero(keep)[0][None, :]] = True
    ref = _sdpa(x["q"], x["k"], x["v"], scale, mask)
    np.testing.assert_allclose(O, ref, atol=1e-12)


def test_rows_are_convex_combinations_of_selected_values():
    cfg, g, x = _inputs("mid_shape")
    scale = oracle.default_scale(cfg.d)
    _, sel, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, cfg.mode, cfg.per_head_budget())
    toks = oracle.block_tokens(g)
    for r in range(0, len(sel.counts), 3):
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, cfg.H)
        o, w, keys = oracle.attention_block_row(x["q"][b, h], x["k"][b, h], x["v"][b, h], toks, i,
                                                sel.row(r), scale, return_weights=True)
        assert (w >= 0).all()
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
        assert set(oracle.token_block_ids(g)[keys].tolist()) == set(sel.row(r).tolist())
        vs = x["v"][b, h, keys]
        assert (o >= vs.min(0) - 1e-12).all() and (o <= vs.max(0) + 1e-12).all()


def test_zero_queries_give_mean_of_selected_values():
    cfg, g, x = _inputs("ragged_small")
    q = np.zeros_like(x["q"])
    scale = oracle.default_scale(cfg.d)
    sel = oracle.select(oracle.estimate(oracle.summarize(q, g), oracle.summarize(x["k"], g), scale),
                        "count", [3, 3])
    O = oracle.attention_full(q, x["k"], x["v"], g, sel.row_ptr, sel.col_idx, scale)
    blk = oracle.token_block_ids(g)
    for b in range(cfg.B):
        for h in range(cfg.H):
            keys = np.isin(blk, [0, 1, 2])
            np.testing.assert_allclose(O[b, h], np.broadcast_to(x["v"][b, h, keys].mean(0), O[b, h].shape),
                                       atol=1e-12)


def test_constant_values_give_constant_output():
    cfg, g, x = _inputs("mid_shape")
    v = np.full_like(x["v"], 0.75)
    O, _, _ = oracle.spade_attn(x["q"], x["k"], v, g, cfg.mode, cfg.per_head_budget())
    np.testing.assert_allclose(O, 0.75, atol=1e-12)


def test_onehot_values_measure_block_mass():
    cfg, g, x = _inputs("tiny")
    scale = oracle.default_scale(cfg.d)
    blk = oracle.token_block_ids(g)
    v = np.zeros_like(x["v"])
    v[:, :, np.arange(g.N), blk] = 1.0  # V[m, c] = [block(m) == c]
    O, sel, _ = oracle.spade_attn(x["q"], x["k"], v, g, "count", [3, 3])
    dense_logits = scale * np.matmul(x["q"], np.swapaxes(x["k"], -1, -2))
    for r in range(len(sel.counts)):
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, cfg.H)
        rows = np.nonzero(blk == i)[0]
        kept = sel.row(r).tolist()
        for c in range(g.nblk):
            if c not in kept:
                assert (O[b, h, rows, c] == 0).all()
        L = dense_logits[b, h][rows][:, np.isin(blk, kept)]
        w = np.exp(L - L.max(1, keepdims=True))
        w /= w.sum(1, keepdims=True)
        kb = blk[np.isin(blk, kept)]
        for c in kept:
            np.testing.assert_allclose(O[b, h, rows, c], w[:, kb == c].sum(1), atol=1e-12)


def test_single_block_is_dense_within_that_block():
    cfg, g, x = _inputs("ragged_p64")
    scale = oracle.default_scale(cfg.d)
    O, sel, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, "count", [1] * cfg.H)
    toks = oracle.block_tokens(g)
    for r in range(0, len(sel.counts), 7):
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, cfg.H)
        j = int(sel.row(r)[0])
        ref = _sdpa(x["q"][b, h][toks[i]], x["k"][b, h][toks[j]], x["v"][b, h][toks[j]], scale)
        np.testing.assert_allclose(O[b, h, toks[i]], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# max / min summarizers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged_p64", "mid_shape", "ragged_small"])
def test_max_min_summary_closed_form_on_monotone_field(name):
    """x[n, c] = a_c t + b_c h + e_c w + f_c is monotone along each axis, so its
    block maximum sits at the corner that maximises each term (t1-1 where a_c > 0,
    t0 where a_c < 0, ...) and the minimum at the opposite corner."""
    cfg = synth.get_config(name)
    g = Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    d = 8
    rng = np.random.default_rng(1)
    coef = rng.integers(-3, 4, size=(4, d)).astype(np.float64)
    n = np.arange(g.N)
    t, h, w = n // (g.Hh * g.W), (n // g.W) % g.Hh, n % g.W
    x = (t[:, None] * coef[0] + h[:, None] * coef[1] + w[:, None] * coef[2] + coef[3])[None, None]
    mx = oracle.summarize(x, g, store_f32=False, op="max")[0, 0]
    mn = oracle.summarize(x, g, store_f32=False, op="min")[0, 0]
    for j, (t0, t1, h0, h1, w0, w1) in enumerate(oracle.block_extents(g)):
        lo = np.array([t0, h0, w0], dtype=np.float64)
        hi = np.array([t1 - 1, h1 - 1, w1 - 1], dtype=np.float64)
        a = coef[:3]
        want_max = np.where(a > 0, hi[:, None], lo[:, None]) * a
        want_min = np.where(a > 0, lo[:, None], hi[:, None]) * a
        np.testing.assert_array_equal(mx[j], want_max.sum(0) + coef[3])
        np.testing.assert_array_equal(mn[j], want_min.sum(0) + coef[3])


def test_max_min_mean_order_and_duality():
    cfg, g, x = _inputs("ragged_small")
    q = x["q"]
    mx = oracle.summarize(q, g, op="max")
    mn = oracle.summarize(q, g, op="min")
    me = oracle.summarize(q, g, store_f32=False)
    assert (mn <= me + 1e-12).all() and (me <= mx + 1e-12).all()
    np.testing.assert_array_equal(oracle.summarize(-q, g, op="min"), -mx)
    # a single-token block: all three summarizers return that token
    g1 = Geometry(2, 2, 2, 1, 1, 1)
    y = np.random.default_rng(2).standard_normal((1, 1, 8, 4)).astype(np.float32).astype(np.float64)
    for op in oracle.SUMMARIZERS:
        np.testing.assert_array_equal(oracle.summarize(y, g1, op=op), y)


def test_max_min_are_exact_block_extremes_by_bruteforce():
    cfg, g, x = _inputs("tiny")
    for op, fn in (("max", max), ("min", min)):
        got = oracle.summarize(x["k"], g, op=op)
        for j, tk in enumerate(oracle.block_tokens(g)):
            for c in range(cfg.d):
                assert got[0, 1, j, c] == fn(float(x["k"][0, 1, n, c]) for n in tk)


# ---------------------------------------------------------------------------
# static window united with the dynamic selection
# ---------------------------------------------------------------------------

def _block_coords_from_extents(g):
    """Block coordinates from the token extents of each block (t0 // bt, ...)."""
    return np.array([(t0 // g.bt, h0 // g.bh, w0 // g.bw) for (t0, t1, h0, h1, w0, w1) in oracle.block_extents(g)])


def _static_mask(g, radius):
    c = _block_coords_from_extents(g)
    d = np.abs(c[:, None, :] - c[None, :, :])
    return (d <= np.array(radius)[None, None, :]).all(axis=-1)  # [nQ, nK]


@pytest.mark.parametrize("radius", [(0, 0, 0), (1, 0, 2), (2, 3, 1)])
@pytest.mark.parametrize("mode,zero", [("count", 0), ("ratio", 0.0), ("mass", 0.0)])
def test_zero_budget_with_window_is_the_static_mask(radius, mode, zero):
    cfg, g, x = _inputs("ragged_small")
    S = np.random.default_rng(5).standard_normal((cfg.B, cfg.H, g.nblk, g.nblk))
    sel = oracle.select(S, mode, [zero] * cfg.H, window=radius, g=g)
    m = _static_mask(g, radius)
    for r in range(len(sel.counts)):
        assert sel.row(r).tolist() == np.nonzero(m[r % g.nblk])[0].tolist()


@pytest.mark.parametrize("mode,budget", [("count", 3), ("ratio", 0.2), ("mass", 0.7)])
def test_window_unites_with_the_dynamic_selection(mode, budget):
    cfg, g, x = _inputs("ragged_small")
    S = np.random.default_rng(6).standard_normal((cfg.B, cfg.H, g.nblk, g.nblk))
    radius = (1, 1, 0)
    dyn = oracle.select(S, mode, [budget] * cfg.H)
    hyb = oracle.select(S, mode, [budget] * cfg.H, window=radius, g=g)
    m = _static_mask(g, radius)
    for r in range(len(dyn.counts)):
        want = sorted(set(dyn.row(r).tolist()) | set(np.nonzero(m[r % g.nblk])[0].tolist()))
        assert hyb.row(r).tolist() == want
        assert r % g.nblk in hyb.row(r)  # radius >= 0 always keeps the diagonal block


def test_window_over_the_whole_grid_is_dense_attention():
    cfg, g, x = _inputs("tiny")
    nT, nH, nW = g.counts
    O, sel, S = oracle.spade_attn(x["q"], x["k"], x["v"], g, "count", [0] * cfg.H,
                                  window=(nT, nH, nW))
    assert (sel.counts == g.nblk).all()
    np.testing.assert_allclose(O, _sdpa(x["q"], x["k"], x["v"], oracle.default_scale(cfg.d)), atol=1e-12)


def test_window_grows_with_its_radius():
    g = Geometry(6, 7, 9, 2, 2, 3)
    for i in range(g.nblk):
        small = set(oracle.window_blocks(g, i, (1, 0, 1)).tolist())
        big = set(oracle.window_blocks(g, i, (1, 1, 1)).tolist())
        assert small <= big and i in small


# ---------------------------------------------------------------------------
# intra-block estimate (SICS: Sum of Intra-block Cosine Similarities)
# ---------------------------------------------------------------------------

def _sics_pairs(xb):
    """Brute force over the ordered token pairs of one block, one cosine at a
    time with math.fsum (zero tokens: cosine 0), divided by n^2."""
    n = xb.shape[0]
    norms = [math.sqrt(math.fsum(float(v) * float(v) for v in row)) for row in xb]
    terms = []
    for i in range(n):
        for j in range(n):
            if norms[i] == 0.0 or norms[j] == 0.0:
                continue
            terms.append(math.fsum(float(a) * float(b) for a, b in zip(xb[i], xb[j])) / (norms[i] * norms[j]))
    return math.fsum(terms) / (n * n)


def test_sics_equals_pairwise_bruteforce_on_ragged_blocks():
    g = Geometry(3, 5, 4, 2, 2, 3)  # partial blocks along every axis
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 2, g.N, 6))
    x[0, 1, 5] = 0.0  # a zero token
    got = oracle.sics(x, g, store_f32=False)
    for j, tk in enumerate(oracle.block_tokens(g)):
        for h in range(2):
            assert abs(got[0, h, j] - _sics_pairs(x[0, h, tk])) < 1e-13


def test_sics_online_identity_is_exact():
    """sum_{i,j} <u_i, u_j> = |sum_i u_i|^2 (bilinearity): the O(n d) online
    form of the page reaches the pairwise definition up to rounding."""
    cfg, g, x = _inputs("ragged_small")
    got = oracle.sics(x["k"], g, store_f32=False)
    xk = x["k"]
    norm = np.sqrt((xk * xk).sum(-1, keepdims=True))
    u = np.divide(xk, norm, out=np.zeros_like(xk), where=norm > 0)
    for j, tk in enumerate(oracle.block_tokens(g)):
        s = u[:, :, tk, :].sum(axis=2)
        np.testing.assert_allclose(got[:, :, j], (s * s).sum(-1) / len(tk) ** 2, rtol=1e-12, atol=1e-15)


def test_sics_closed_forms():
    g = Geometry(1, 1, 4, 1, 1, 4)  # one block of 4 tokens
    d = 5
    v = np.array([1.0, -2.0, 0.5, 3.0, 0.25])
    same = np.tile(v, (4, 1))[None, None]
    assert oracle.sics(same, g, store_f32=False)[0, 0, 0] == pytest.approx(1.0, abs=1e-15)
    # a token and its negation, twice: the unit vectors cancel
    opp = np.stack([v, -v, 2 * v, -0.5 * v])[None, None]
    assert abs(oracle.sics(opp, g, store_f32=False)[0, 0, 0]) < 1e-15
    # orthonormal tokens: only the diagonal survives -> n / n^2
    eye = np.eye(d)[:4][None, None] * np.array([1.0, 3.0, 0.2, 7.0])[:, None]
    assert oracle.sics(eye, g, store_f32=False)[0, 0, 0] == pytest.approx(0.25, abs=1e-15)
    # one live token, three zero tokens: |u|^2 / n^2
    one = np.zeros((1, 1, 4, d))
    one[0, 0, 2] = v
    assert oracle.sics(one, g, store_f32=False)[0, 0, 0] == pytest.approx(1.0 / 16, abs=1e-15)
    # two tokens at angle theta: (2 + 2 cos theta) / 4
    g2 = Geometry(1, 1, 2, 1, 1, 2)
    for theta in (0.3, 1.2, 2.9):
        two = np.array([[1.0, 0.0], [math.cos(theta), math.sin(theta)]])[None, None]
        assert oracle.sics(two, g2, store_f32=False)[0, 0, 0] == pytest.approx((2 + 2 * math.cos(theta)) / 4, abs=1e-15)


def test_sics_invariant_to_token_scaling_and_rotation():
    cfg, g, x = _inputs("ragged_p64")
    q = x["q"][:, :1]
    base = oracle.sics(q, g, store_f32=False)
    rng = np.random.default_rng(3)
    scaled = q * rng.uniform(0.1, 10.0, size=q.shape[:-1] + (1,))
    np.testing.assert_allclose(oracle.sics(scaled, g, store_f32=False), base, rtol=1e-12, atol=1e-14)
    rot, _ = np.linalg.qr(rng.standard_normal((cfg.d, cfg.d)))
    np.testing.assert_allclose(oracle.sics(q @ rot, g, store_f32=False), base, rtol=1e-11, atol=1e-13)
    assert (base >= -1e-15).all() and (base <= 1 + 1e-12).all()


# ---------------------------------------------------------------------------
# scheme generation: blocking candidates and head-wise choice
# ---------------------------------------------------------------------------

def test_temporally_constant_field_chooses_the_temporal_blocking():
    """x[t, h, w] = f(h, w): a candidate whose blocks span time only has SICS
    exactly 1; a spatial candidate mixes different columns (aggregate < 1)."""
    T, Hh, W, d = 4, 4, 6, 8
    rng = np.random.default_rng(11)
    col = rng.standard_normal((Hh * W, d))
    x = np.tile(col, (T, 1))[None, None]                     # raster (t, h, w)
    cands = [(1, 2, 3), (4, 1, 1), (2, 2, 2)]
    agg = oracle.scheme_aggregate(x, x, T, Hh, W, cands)
    assert agg[1, 0, 0] == pytest.approx(1.0, abs=1e-7)
    assert agg[0, 0, 0] < 0.9 and agg[2, 0, 0] < 0.9
    choice, margin = oracle.choose_scheme(agg)
    assert choice[0, 0] == 1 and margin[0, 0] > 0.1


def test_frame_constant_field_chooses_the_spatial_blocking():
    T, Hh, W, d = 6, 3, 4, 8
    rng = np.random.default_rng(12)
    frame = rng.standard_normal((T, d))
    x = np.repeat(frame, Hh * W, axis=0)[None, None]         # same vector in every token of a frame
    cands = [(2, 1, 1), (1, 3, 4), (3, 3, 2)]
    agg = oracle.scheme_aggregate(x, x, T, Hh, W, cands)
    assert agg[1, 0, 0] == pytest.approx(1.0, abs=1e-7)
    choice, _ = oracle.choose_scheme(agg)
    assert choice[0, 0] == 1


def test_scheme_aggregate_equals_pairwise_bruteforce():
    T, Hh, W, d = 3, 4, 5, 6
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 1, T * Hh * W, d))
    k = rng.standard_normal((1, 1, T * Hh * W, d))
    cands = [(2, 2, 2), (3, 1, 5)]
    agg = oracle.scheme_aggregate(q, k, T, Hh, W, cands)
    for c, blk in enumerate(cands):
        g = Geometry(T, Hh, W, *blk)
        tot = 0.0
        for tk in oracle.block_tokens(g):
            sq = float(np.float32(_sics_pairs(q[0, 0, tk])))
            sk = float(np.float32(_sics_pairs(k[0, 0, tk])))
            tot += len(tk) * (sq + sk)
        assert agg[c, 0, 0] == pytest.approx(tot / (2 * g.N), rel=1e-12)


def test_single_and_duplicate_candidates():
    cfg, g, x = _inputs("tiny")
    blk = (cfg.bt, cfg.bh, cfg.bw)
    O1, ch1, _ = oracle.spade_attn_schemes(x["q"], x["k"], x["v"], cfg.T, cfg.Hh, cfg.W, [blk], cfg.mode,
                                           cfg.per_head_budget())
    O0, _, _ = oracle.spade_attn(x["q"], x["k"], x["v"], g, cfg.mode, cfg.per_head_budget())
    assert (ch1 == 0).all()
    np.testing.assert_array_equal(O1, O0)
    agg = oracle.scheme_aggregate(x["q"], x["k"], cfg.T, cfg.Hh, cfg.W, [blk, blk])
    choice, margin = oracle.choose_scheme(agg)
    assert (choice == 0).all() and (margin == 0).all()   # a tie goes to the earlier candidate


def test_each_head_equals_its_single_scheme_run():
    cfg, g, x = _inputs("ragged_small")
    cands = [(cfg.bt, cfg.bh, cfg.bw), (1, 4, 4), (4, 2, 2)]
    O, choice, agg = oracle.spade_attn_schemes(x["q"], x["k"], x["v"], cfg.T, cfg.Hh, cfg.W, cands,
                                               cfg.mode, cfg.per_head_budget())
    for c, blk in enumerate(cands):
        gc = Geometry(cfg.T, cfg.Hh, cfg.W, *blk)
        Oc, _, _ = oracle.spade_attn(x["q"], x["k"], x["v"], gc, cfg.mode, cfg.per_head_budget())
        m = choice == c
        np.testing.assert_array_equal(O[m], Oc[m])


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def test_planted_transposed_raster_order_is_caught():
    g = Geometry(3, 4, 5, 2, 2, 2)

    def bad_tokens(g):  # w and h swapped in the flattening
        toks = []
        for (t0, t1, h0, h1, w0, w1) in oracle.block_extents(g):
            t = np.arange(t0, t1)[:, None, None]
            h = np.arange(h0, h1)[None, :, None]
            w = np.arange(w0, w1)[None, None, :]
            toks.append(((t * g.W + w) * g.Hh + h).reshape(-1))
        return toks

    n = np.arange(g.N)
    t, h, w = n // (g.Hh * g.W), (n // g.W) % g.Hh, n % g.W
    nT, nH, nW = g.counts
    expect = ((t // g.bt) * nH + (h // g.bh)) * nW + (w // g.bw)
    ids = np.full(g.N, -1)
    for j, tk in enumerate(bad_tokens(g)):
        ids[tk] = j
    assert not (ids == expect).all()


def test_planted_dropped_scale_is_caught_by_sdpa():
    cfg, g, x = _inputs("tiny")
    scale = oracle.default_scale(cfg.d)
    bad = oracle.dense_attention(x["q"], x["k"], x["v"], 1.0)
    ref = _sdpa(x["q"], x["k"], x["v"], scale)
    assert np.abs(bad - ref).max() > 1e-3


def test_planted_wrong_tie_break_is_caught():
    S = np.zeros((1, 1, 1, 6))
    order_bad = np.argsort(S.reshape(1, 6), axis=1)[:, ::-1]  # ties by descending j
    sel = oracle.select(S, "count", [2])
    assert sorted(order_bad[0, :2].tolist()) != sel.row(0).tolist()


def test_planted_mass_over_kept_only_is_caught():
    """Normalising the mass over the top-k only (instead of all blocks) changes
    the brute-force minimal subset."""
    S = np.array([[[[2.0, 1.0, 0.5, 0.0, -1.0, -3.0]]]])
    sel = oracle.select(S, "mass", [0.9])
    p = np.exp(S[0, 0, 0] - 2.0)
    p /= p.sum()
    assert p[sel.row(0)].sum() >= 0.9 - 1e-15
    assert p[sel.row(0)[:-1]].sum() < 0.9


def test_planted_sics_without_diagonal_is_caught():
    """Dropping the i = j pairs (normalising by n(n-1)) fails the
    orthonormal-tokens closed form (it gives 0 instead of 1/n)."""
    eye = np.eye(4)[None, None]
    n = 4
    u = eye[0, 0]
    bad = (u @ u.T - np.diag(np.diag(u @ u.T))).sum() / (n * (n - 1))
    assert abs(bad - 0.25) > 0.2


def test_planted_sics_dot_products_instead_of_cosines_is_caught():
    """Summing raw dot products (no normalisation) breaks scale invariance."""
    cfg, g, x = _inputs("tiny")
    q = x["q"][:, :1]
    toks = oracle.block_tokens(g)

    def bad(y):
        return np.array([(y[0, 0, tk] @ y[0, 0, tk].T).sum() / len(tk) ** 2 for tk in toks])

    assert np.abs(bad(3.0 * q) - bad(q)).max() > 1e-3


def test_planted_max_over_padded_box_is_caught():
    """Taking the maximum over the full (bt, bh, bw) box instead of the block's
    real tokens reads tokens of the next block on partial edges; the closed
    form of the monotone field catches it."""
    g = Geometry(3, 5, 4, 2, 2, 3)
    n = np.arange(g.N)
    t, h, w = n // (g.Hh * g.W), (n // g.W) % g.Hh, n % g.W
    x = (t + 2.0 * h + 3.0 * w)[None, None, :, None]
    good = oracle.summarize(x, g, store_f32=False, op="max")[0, 0, :, 0]
    bad = []
    for (t0, t1, h0, h1, w0, w1) in oracle.block_extents(g):
        bad.append((t0 + g.bt - 1) + 2.0 * (h0 + g.bh - 1) + 3.0 * (w0 + g.bw - 1))
    assert (np.array(bad) != good).any()


def test_planted_window_in_token_units_is_caught():
    """Measuring the window radius in tokens instead of blocks keeps a
    different set as soon as a block is longer than one token."""
    g = Geometry(4, 6, 8, 2, 3, 4)
    good = _static_mask(g, (1, 1, 1))
    ext = oracle.block_extents(g)
    c = np.array([(t0, h0, w0) for (t0, t1, h0, h1, w0, w1) in ext])
    bad = (np.abs(c[:, None, :] - c[None, :, :]) <= 1).all(axis=-1)
    assert (bad != good).any()

