"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (block-sparse attention contract):
* summaries: the GPU's fp32 means equal the oracle's exact means rounded to
  fp32 (at most one fp32 ulp apart);
* scores: fp64 on both sides, |dS| <= 1e-12 * max(1, |S|max);
* block indices: identical to the oracle's on every row whose oracle margin
  exceeds 1e-3 (the contract) -- and, since both sides decide in fp64, on
  every row whose margin exceeds 1e-9; the oracle's selection run on the GPU's
  own scores reproduces the GPU's CSR on every row;
* outputs, computed with the GPU's CSR fed to the oracle: max-abs error
  <= 2e-2 for bf16 and <= 1e-5 for the fp32 debug path.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import input_adaptive_block_amd as spade  # noqa: E402

BF16_TOL = 2e-2
F32_TOL = 1e-5
SMALL = ["tiny", "tiny_bf16", "ragged_p64", "mid_shape", "small_shape", "ragged_small", "big_block",
         "token_level", "one_block", "d64", "tail24", "ragged_f32", "mid_full", "dense_mixed", "dense_40"]


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def geom(cfg):
    return oracle.Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)


def to_dev(cfg, a):
    if cfg.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(cfg, a):
    return synth.bf16_bits_to_f64(a) if cfg.dtype == "bf16" else a.astype(np.float64)


def dev_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def grid_block(cfg):
    return (cfg.T, cfg.Hh, cfg.W), (cfg.bt, cfg.bh, cfg.bw)


def oracle_means(cfg, x):
    """Oracle block means per head chunk (bounded host memory)."""
    g = geom(cfg)
    out = np.empty((cfg.B, cfg.H, g.nblk, cfg.d))
    for h in range(cfg.H):
        out[:, h:h + 1] = oracle.summarize(to_f64(cfg, x[:, h:h + 1]), g)
    return out


def csr_rows(row_ptr, col_idx):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    return rp, ci


def compare_selection(sel, rp, ci, S_ref, mode, budget, name):
    """Contract check + strict fp64 check; returns number of differing rows."""
    R = len(sel.counts)
    assert rp.shape[0] == R + 1 and rp[0] == 0
    diff = []
    for r in range(R):
        got = ci[rp[r]:rp[r + 1]]
        if not np.array_equal(got, sel.row(r)):
            diff.append(r)
    for r in diff:
        m = sel.margins[r]
        assert m <= 1e-3, f"{name}: row {r} differs with oracle margin {m}"
        assert m <= 1e-9, f"{name}: row {r} differs although both sides decide in fp64 (margin {m})"
    return len(diff)


def run_attn(cfg, x, mode=None, budget=None, scale=None):
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    mode = cfg.mode if mode is None else mode
    budget = cfg.per_head_budget() if budget is None else budget
    o, rp, ci = spade.attn(q, k, v, grid, block, mode, budget, scale=scale)
    torch.cuda.synchronize()
    return o, rp, ci


# ---------------------------------------------------------------------------
# small configurations, every row and every output element
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", SMALL)
def test_summarize_matches_oracle(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qm, km = spade.summarize(to_dev(cfg, x["q"]), to_dev(cfg, x["k"]), grid, block)
    for got, ref in ((qm, oracle_means(cfg, x["q"])), (km, oracle_means(cfg, x["k"]))):
        g = got.cpu().numpy().astype(np.float64)
        ulp = np.abs(ref) * 2.0 ** -23 + 1e-38
        assert (np.abs(g - ref) <= ulp).all(), np.abs(g - ref).max()


def oracle_summaries(cfg, x, op):
    g = geom(cfg)
    out = np.empty((cfg.B, cfg.H, g.nblk, cfg.d))
    for h in range(cfg.H):
        out[:, h:h + 1] = oracle.summarize(to_f64(cfg, x[:, h:h + 1]), g, op=op)
    return out


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("name", SMALL)
def test_max_min_summaries_are_exact(name, op):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    qm, km = spade.summarize(qd, kd, grid, block, summarizer=op)
    assert np.array_equal(qm.cpu().numpy().astype(np.float64), oracle_summaries(cfg, x["q"], op))
    assert np.array_equal(km.cpu().numpy().astype(np.float64), oracle_summaries(cfg, x["k"], op))
    # the SICS pass takes the same summarizer for its summary output
    qm2, km2, qs, ks = spade.summarize_sics(qd, kd, grid, block, summarizer=op)
    assert torch.equal(qm, qm2) and torch.equal(km, km2)


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("name", ["mid_shape", "ragged_small", "tiny", "d64", "ragged_f32"])
def test_whole_path_with_max_min_summarizer(name, op):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, rp, ci = spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget(), summarizer=op)
    torch.cuda.synchronize()
    rp, ci = csr_rows(rp, ci)
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_summaries(cfg, x["q"], op), oracle_summaries(cfg, x["k"], op), scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), f"{name}/{op}")
    ref = oracle.attention_full(*(to_f64(cfg, x[n]) for n in ("q", "k", "v")), geom(cfg), rp, ci, scale)
    tol = BF16_TOL if cfg.dtype == "bf16" else F32_TOL
    assert np.abs(dev_to_f64(o) - ref).max() <= tol


@pytest.mark.parametrize("window,scale_budget", [((0, 0, 0), 0.0), ((1, 1, 2), 0.0), ((1, 0, 1), 1.0),
                                                  ((2, 2, 2), 1.0)])
@pytest.mark.parametrize("name", ["mid_shape", "ragged_small", "tiny", "d64", "dense_40"])
def test_static_window_united_with_selection(name, window, scale_budget):
    """Budget 0 gives the static window alone; otherwise the window is united
    with the scored blocks.  Selection is checked row by row, attention on
    every output element."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    budget = [b * scale_budget for b in cfg.per_head_budget()]
    if cfg.mode == "count":
        budget = [int(b) for b in budget]
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, rp, ci = spade.attn(q, k, v, grid, block, cfg.mode, budget, window=window)
    torch.cuda.synchronize()
    rp, ci = csr_rows(rp, ci)
    g = geom(cfg)
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, cfg.mode, budget, window=window, g=g)
    compare_selection(sel, rp, ci, S_ref, cfg.mode, budget, f"{name}/{window}")
    ref = oracle.attention_full(*(to_f64(cfg, x[n]) for n in ("q", "k", "v")), g, rp, ci, scale)
    tol = BF16_TOL if cfg.dtype == "bf16" else F32_TOL
    assert np.abs(dev_to_f64(o) - ref).max() <= tol


def oracle_sics(cfg, x):
    g = geom(cfg)
    out = np.empty((cfg.B, cfg.H, g.nblk))
    for h in range(cfg.H):
        out[:, h:h + 1] = oracle.sics(to_f64(cfg, x[:, h:h + 1]), g)
    return out


def assert_sics_close(got, ref, name):
    """The GPU takes the online form |sum u|^2 / n^2 in fp64, the oracle the
    pairwise sum: both round once to fp32, so they agree to an ulp of the
    result (plus the fp64 cancellation of nearly balanced blocks)."""
    g = got.cpu().numpy().astype(np.float64)
    tol = np.abs(ref) * 2.0 ** -22 + 1e-12
    bad = np.abs(g - ref) > tol
    assert not bad.any(), f"{name}: {bad.sum()} blocks, max err {np.abs(g - ref).max()}"


@pytest.mark.parametrize("name", SMALL)
def test_summarize_sics_matches_oracle(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    qm, km, qs, ks = spade.summarize_sics(qd, kd, grid, block)
    qm0, km0 = spade.summarize(qd, kd, grid, block)
    # the means are those of the plain summarize, bit for bit
    assert torch.equal(qm, qm0) and torch.equal(km, km0)
    assert_sics_close(qs, oracle_sics(cfg, x["q"]), name + " q")
    assert_sics_close(ks, oracle_sics(cfg, x["k"]), name + " k")
    assert (qs >= 0).all() and (qs <= 1 + 1e-6).all()


def test_sics_closed_forms_on_device():
    """Constructed fp32 tokens: a block of one repeated vector gives 1, a
    block of opposite pairs gives 0, one live token among zeros gives 1/n^2,
    orthogonal one-hot tokens give 1/n (exact in fp64, exact in fp32)."""
    T, Hh, W, bt, bh, bw, d = 1, 1, 16, 1, 1, 4, 64
    p_grid, p_block = (T, Hh, W), (bt, bh, bw)
    x = np.zeros((1, 1, W, d), dtype=np.float32)
    v = np.linspace(-1.0, 2.0, d).astype(np.float32)
    x[0, 0, 0:4] = v                                   # block 0: same vector
    x[0, 0, 4:8] = np.stack([v, -v, 2 * v, -v])        # block 1: cancels
    x[0, 0, 9] = v                                     # block 2: one live token
    x[0, 0, 12:16] = np.eye(d, dtype=np.float32)[:4] * 3.0  # block 3: orthogonal
    xd = torch.from_numpy(x).cuda()
    qm, km, qs, ks = spade.summarize_sics(xd, xd, p_grid, p_block)
    got = qs.cpu().numpy()[0, 0]
    np.testing.assert_allclose(got, [1.0, 0.0, 1.0 / 16, 0.25], rtol=2e-7, atol=1e-12)
    assert torch.equal(qs, ks)


def test_sics_outputs_are_optional():
    cfg = synth.get_config("ragged_small")
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    p = spade.problem_for(qd, grid, block)
    nblk = spade.spade_num_blocks(p)
    qm = torch.empty(cfg.B, cfg.H, nblk, cfg.d, device="cuda")
    km = torch.empty_like(qm)
    ks = torch.full((cfg.B, cfg.H, nblk), -7.0, device="cuda")
    spade.spade_summarize_sics(p, qd, kd, qm, km, None, ks)
    torch.cuda.synchronize()
    assert_sics_close(ks, oracle_sics(cfg, x["k"]), "k only")
    qm0, km0 = spade.summarize(qd, kd, grid, block)
    assert torch.equal(qm, qm0) and torch.equal(km, km0)


@pytest.mark.parametrize("name", SMALL)
def test_scores_and_selection_match_oracle(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    qm, km = spade.summarize(qd, kd, grid, block)
    p = spade.problem_for(qd, grid, block)
    S_gpu = spade.debug_scores(qm, km, p).cpu().numpy()
    scale = oracle.default_scale(cfg.d)
    S_from_gpu_means = oracle.estimate(qm.cpu().numpy().astype(np.float64),
                                       km.cpu().numpy().astype(np.float64), scale)
    tol = 1e-12 * max(1.0, np.abs(S_from_gpu_means).max())
    assert np.abs(S_gpu - S_from_gpu_means).max() <= tol
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    assert np.abs(S_gpu - S_ref).max() <= 1e-9 * max(1.0, np.abs(S_ref).max())

    rp, ci = spade.estimate_select(qm, km, p, cfg.mode, cfg.per_head_budget())
    rp, ci = csr_rows(rp, ci)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    ndiff = compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), name)
    assert ndiff == 0
    # logic check: the oracle's selection on the GPU's own scores
    sel_g = oracle.select(S_gpu, cfg.mode, cfg.per_head_budget())
    assert np.array_equal(sel_g.row_ptr, rp)
    assert np.array_equal(sel_g.col_idx, ci[:rp[-1]])


@pytest.mark.parametrize("name", SMALL)
def test_attention_matches_oracle(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    o, rp, ci = run_attn(cfg, x)
    rp, ci = csr_rows(rp, ci)
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    scale = oracle.default_scale(cfg.d)
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= (BF16_TOL if cfg.dtype == "bf16" else F32_TOL), err
    # and the CSR itself is the oracle's
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    assert compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), name) == 0


# a different budget for every head: each head's rows are selected with its
# own k, ratio or mass
PER_HEAD = [("mid_shape", "mass", [0.5, 0.97]), ("small_shape", "ratio", [0.1, 0.6]),
            ("ragged_small", "count", [2, 9]), ("d64", "mass", [0.95, 0.3])]


@pytest.mark.parametrize("name,mode,budget", PER_HEAD)
def test_per_head_budgets_match_oracle(name, mode, budget):
    cfg = synth.get_config(name)
    assert cfg.H == len(budget)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    o, rp, ci = run_attn(cfg, x, mode=mode, budget=budget)
    rp, ci = csr_rows(rp, ci)
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, mode, budget)
    assert compare_selection(sel, rp, ci, S_ref, mode, budget, name) == 0
    kept = np.diff(rp).reshape(cfg.B, cfg.H, g.nblk).sum(axis=(0, 2))
    assert kept[0] != kept[1]  # the heads really keep different amounts
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= BF16_TOL, err


# the supported limits: 4096 and 1728 blocks per head (the widest selection
# rows), and 1024-token blocks (eight 128-query tiles per row, 32 key subtiles
# per block)
LIMITS = ["max_blocks", "blocks_2k", "max_block_tokens", "max_blocks_mass"]


@pytest.mark.parametrize("name", LIMITS)
def test_limits_selection_and_attention_match_oracle(name):
    # max_blocks_mass: 4096 blocks under a mass budget (the widest rows of the
    # mass search, 64 scores per lane)
    cfg = (synth.get_config("max_blocks").with_budget("mass", 0.5) if name == "max_blocks_mass"
           else synth.get_config(name))
    print(f"[limits] {name}", flush=True)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    qm, km = spade.summarize(qd, kd, grid, block)
    scale = oracle.default_scale(cfg.d)
    qm_ref, km_ref = oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"])
    assert np.array_equal(qm.cpu().numpy().astype(np.float64), qm_ref)
    assert np.array_equal(km.cpu().numpy().astype(np.float64), km_ref)
    S_ref = oracle.estimate(qm_ref, km_ref, scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    o, rp, ci = run_attn(cfg, x)
    rp, ci = csr_rows(rp, ci)
    assert compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), name) == 0
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("name", ["rows_32k", "rows_32k_plus"])
def test_csr_build_on_both_sides_of_its_row_limit(name):
    """Up to 32768 rows the CSR (row_ptr and the ascending kept ids) comes
    from one kernel that also clears the attention kernel's unit counter;
    above it from the chunked scan and the per-row compaction.  Both against
    the oracle's selection, the oracle's selection on the GPU's own scores
    (which must reproduce the CSR exactly), and the attention on that CSR,
    twice in a row (a counter left uncleared would skip every unit)."""
    cfg = synth.get_config(name)
    print(f"[csr] {name} R={cfg.B * cfg.H * 64}", flush=True)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    grid, block = grid_block(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    qm, km = spade.summarize(qd, kd, grid, block)
    p = spade.problem_for(qd, grid, block)
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    rp, ci = csr_rows(*spade.estimate_select(qm, km, p, cfg.mode, cfg.per_head_budget()))
    assert compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), name) == 0
    S_gpu = spade.debug_scores(qm, km, p).cpu().numpy()
    sel_g = oracle.select(S_gpu, cfg.mode, cfg.per_head_budget())
    assert np.array_equal(sel_g.row_ptr, rp)
    assert np.array_equal(sel_g.col_idx, ci[:rp[-1]])
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    for _ in range(2):
        o, rp2, ci2 = run_attn(cfg, x)
        rp2, ci2 = csr_rows(rp2, ci2)
        assert np.array_equal(rp2, rp) and np.array_equal(ci2[:rp[-1]], ci[:rp[-1]])
        ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
        err = np.abs(dev_to_f64(o) - ref).max()
        assert err <= BF16_TOL, err


@pytest.mark.parametrize("name", ["ragged_small", "ragged_p64", "tiny", "ragged_f32", "mid_full", "dense_40"])
def test_ratio_one_equals_dense_attention(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    o, rp, ci = run_attn(cfg, x, mode="ratio", budget=[1.0] * cfg.H)
    g = geom(cfg)
    assert (np.diff(rp.cpu().numpy()) == g.nblk).all()
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref = oracle.dense_attention(xf["q"], xf["k"], xf["v"], oracle.default_scale(cfg.d))
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= (BF16_TOL if cfg.dtype == "bf16" else F32_TOL), err


@pytest.mark.parametrize("name", ["mid_shape", "ragged_small", "tiny", "dense_mixed"])
def test_block_sparse_attn_on_oracle_csr(name):
    """spade_block_sparse_attn alone, fed the oracle's own CSR."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    scale = oracle.default_scale(cfg.d)
    _, sel, _ = oracle.spade_attn(xf["q"], xf["k"], xf["v"], g, cfg.mode, cfg.per_head_budget())
    grid, block = grid_block(cfg)
    rp = torch.from_numpy(sel.row_ptr.astype(np.int32)).cuda()
    ci = torch.from_numpy(sel.col_idx.astype(np.int32)).cuda()
    o = spade.block_sparse_attn(*(to_dev(cfg, x[n]) for n in ("q", "k", "v")), grid, block, rp, ci)
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, sel.row_ptr, sel.col_idx, scale)
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= (BF16_TOL if cfg.dtype == "bf16" else F32_TOL), err


@pytest.mark.parametrize("name", ["mid_shape", "tiny", "mid_full", "dense_mixed"])
def test_arbitrary_csr_is_memory_safe(name):
    """A row is a set (repeated ids count once, order is free), invalid ids are
    skipped, empty rows give zeros."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    R = cfg.B * cfg.H * g.nblk
    rng = np.random.default_rng(7)
    rows, raw = [], []
    for r in range(R):
        if r % 5 == 2:
            ids = []
        else:
            ids = sorted(rng.choice(g.nblk, size=min(g.nblk, 1 + r % 3), replace=False).tolist())
            if r % 4 == 0:
                ids = ids[::-1] + [ids[-1]]  # reversed order and a repeated id
            if r % 3 == 0:
                ids = [-1] + ids + [g.nblk + 5]  # out of range
        raw.append(ids)
        rows.append(sorted(set(j for j in ids if 0 <= j < g.nblk)))
    rp_raw = np.concatenate([[0], np.cumsum([len(a) for a in raw])]).astype(np.int32)
    ci_raw = np.array([j for a in raw for j in a], dtype=np.int32)
    rp_ok = np.concatenate([[0], np.cumsum([len(a) for a in rows])]).astype(np.int64)
    ci_ok = np.array([j for a in rows for j in a], dtype=np.int64)
    grid, block = grid_block(cfg)
    o = spade.block_sparse_attn(*(to_dev(cfg, x[n]) for n in ("q", "k", "v")), grid, block,
                                torch.from_numpy(rp_raw).cuda(), torch.from_numpy(ci_raw).cuda())
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp_ok, ci_ok, oracle.default_scale(cfg.d))
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= (BF16_TOL if cfg.dtype == "bf16" else F32_TOL), err


def test_scale_override():
    cfg = synth.get_config("tiny")
    x = synth.make_inputs(cfg)
    o, rp, ci = run_attn(cfg, x, scale=0.05)
    rp, ci = csr_rows(rp, ci)
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    s = float(np.float32(0.05))
    _, sel, _ = oracle.spade_attn(xf["q"], xf["k"], xf["v"], geom(cfg), cfg.mode, cfg.per_head_budget(), scale=s)
    assert np.array_equal(sel.col_idx, ci[:rp[-1]])
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], geom(cfg), rp, ci, s)
    assert np.abs(dev_to_f64(o) - ref).max() <= F32_TOL


def test_zero_queries_select_lowest_ids():
    cfg = synth.get_config("ragged_small")
    x = synth.make_inputs(cfg)
    x = dict(x, q=np.zeros_like(x["q"]))
    g = geom(cfg)
    for mode, val in (("ratio", 0.5), ("mass", 0.3)):
        _, rp, ci = run_attn(cfg, x, mode=mode, budget=[val] * cfg.H)
        rp, ci = csr_rows(rp, ci)
        k = (oracle.keep_count("ratio", val, g.nblk) if mode == "ratio"
             else math.ceil(float(np.float32(val)) * g.nblk))
        for r in range(len(rp) - 1):
            assert ci[rp[r]:rp[r + 1]].tolist() == list(range(k))


@pytest.mark.parametrize("grid", [(4, 4, 4), (8, 8, 8), (8, 8, 10)])
def test_mass_targets_on_a_whole_number_of_blocks(grid):
    """Zero query summaries make every score 0 and every weight exactly 1, so
    all mass sums are exact integers and every key ties.  With tau * nblk
    exactly an integer m the mass of the top m blocks equals the target
    (kept: the m lowest ids); one fp32 step of tau above, m + 1; one step
    below, m (rows of 64, 512 and 640 blocks: 1, 8 and 10 keys per lane)."""
    nblk = grid[0] * grid[1] * grid[2]
    B, H, d = 1, 3, 64
    q = torch.zeros(B, H, nblk, d, dtype=torch.bfloat16, device="cuda")
    p = spade.problem_for(q, grid, (1, 1, 1))
    assert spade.spade_num_blocks(p) == nblk
    qm = torch.zeros(B, H, nblk, d, dtype=torch.float32, device="cuda")
    km = torch.from_numpy(np.random.default_rng(11).standard_normal((B, H, nblk, d)).astype(np.float32)).cuda()
    m = 5 * (nblk // 40) + 5  # m / nblk is a dyadic fraction: exact in fp32
    t = np.float32(m) / np.float32(nblk)
    assert float(t) * nblk == m
    taus = [t, np.nextafter(t, np.float32(1)), np.nextafter(t, np.float32(0))]
    want = [m, m + 1, m]
    for tau, k in zip(taus, want):
        rp, ci = csr_rows(*spade.estimate_select(qm, km, p, "mass", [float(tau)] * H))
        assert rp[-1] == k * B * H * nblk, (tau, k)
        for r in range(len(rp) - 1):
            assert ci[rp[r]:rp[r + 1]].tolist() == list(range(k)), (tau, r)


@pytest.mark.parametrize("grid", [(4, 4, 4), (8, 8, 8), (8, 8, 10)])
def test_mass_target_next_to_the_mass_of_the_top_blocks(grid):
    """Five blocks score 0 (weight exactly 1), the others score below -1, all
    distinct; tau is the fp32 value nearest 5 / Z and its two fp32 neighbours,
    so the mass of the five top blocks (the first test of each search splits
    them from the rest) lies within a few 1e-7 of the target, on either side:
    five or six blocks kept.  Every row against the oracle's selection, with
    no row allowed to differ: the targets sit 1e-8 to 5e-7 from that mass,
    far beyond the two sides' differences in Z (about 1e-16 relative)."""
    nblk = grid[0] * grid[1] * grid[2]
    B, H, d = 1, 2, 64
    q = torch.zeros(B, H, nblk, d, dtype=torch.bfloat16, device="cuda")
    p = spade.problem_for(q, grid, (1, 1, 1))
    scale = oracle.default_scale(d)
    qm = np.zeros((B, H, nblk, d), np.float32)
    qm[..., 0] = 1.0
    km = np.zeros((B, H, nblk, d), np.float32)
    svals = -1.0 - 0.01 * np.arange(nblk - 5) - 0.001 * np.arange(H)[:, None]
    km[0, :, 5:, 0] = (svals / scale).astype(np.float32)
    S_ref = oracle.estimate(qm.astype(np.float64), km.astype(np.float64), scale)
    Z = np.exp(S_ref[0, :, 0, :] - S_ref[0, :, 0, :].max(axis=1, keepdims=True)).sum(axis=1)
    qd, kd = torch.from_numpy(qm).cuda(), torch.from_numpy(km).cuda()
    for step in (0, 1, -1):
        taus = []
        for h in range(H):
            t = np.float32(5.0 / Z[h])
            if step:
                t = np.nextafter(t, np.float32(1.0 if step > 0 else 0.0))
            assert abs(float(t) * Z[h] - 5.0) < 1e-6 * Z[h]
            taus.append(float(t))
        sel = oracle.select(S_ref, "mass", taus)
        rp, ci = csr_rows(*spade.estimate_select(qd, kd, p, "mass", taus))
        assert compare_selection(sel, rp, ci, S_ref, "mass", taus, f"{grid} step {step}") == 0
        kept = sel.counts.reshape(H, nblk)[:, 0]
        assert set(kept.tolist()) <= {5, 6}


def test_deterministic_and_writes_every_output_once():
    cfg = synth.get_config("mid_shape")
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    p = spade.problem_for(q, grid, block)
    bud = spade.Budget(cfg.mode, cfg.per_head_budget())
    cap = spade.spade_max_nnz(p, bud)
    nblk = spade.spade_num_blocks(p)
    R = cfg.B * cfg.H * nblk
    ws = spade.alloc_workspace(p, q.device)
    G = 4096
    outs = []
    for _ in range(2):
        big = torch.full((q.numel() + 2 * G,), float("nan"), dtype=q.dtype, device=q.device)
        o = big[G:G + q.numel()].view(q.shape)
        rp_big = torch.full((R + 1 + 2 * G,), -7, dtype=torch.int32, device=q.device)
        ci_big = torch.full((cap + 2 * G,), -7, dtype=torch.int32, device=q.device)
        rp = rp_big[G:G + R + 1]
        ci = ci_big[G:G + cap]
        spade.spade_attn(p, q, k, v, bud, o, rp, ci, cap, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all()
        assert torch.isnan(big[:G].float()).all() and torch.isnan(big[-G:].float()).all()
        assert (rp_big[:G] == -7).all() and (rp_big[-G:] == -7).all()
        assert (ci_big[:G] == -7).all() and (ci_big[-G:] == -7).all()
        outs.append((o.clone(), rp.clone(), ci[:int(rp[-1])].clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])


# ---------------------------------------------------------------------------
# full-size workloads in the bench's launch configuration: every row's block
# set, sampled output rows
# ---------------------------------------------------------------------------

FULL = [("small", None), ("mid", None), ("large", None), ("ragged", 1.0), ("ragged", 0.5), ("ragged", 0.1)]


def parity_rows(cfg, nblk, seed):
    """Every row of the first and the last (batch, head) pair plus 256 seeded
    rows of the whole layer, ascending."""
    BH = cfg.B * cfg.H
    R = BH * nblk
    rows = set(range(nblk)) | set(range((BH - 1) * nblk, BH * nblk))
    rng = np.random.default_rng(seed)
    rows |= set(rng.choice(R, size=min(R, 256), replace=False).tolist())
    return sorted(rows)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def check_rows(cfg, x, o, rp, ci, rows, tol, label):
    """Oracle attention of the given rows on the GPU's CSR against the GPU
    output; returns (max-abs error, max |o|, the error in half-ulps of a bf16
    value of that largest magnitude: about 1 means the output's own rounding
    dominates)."""
    g = geom(cfg)
    scale = oracle.default_scale(cfg.d)
    toks = oracle.block_tokens(g)
    of = o.cpu()
    worst = omax = 0.0
    cur = None
    for r in rows:
        bh, i = divmod(r, g.nblk)
        if bh != cur:
            b, h = divmod(bh, cfg.H)
            qh, kh, vh = (to_f64(cfg, x[n][b, h]) for n in ("q", "k", "v"))
            got_h = of[b, h].float().numpy().astype(np.float64)
            cur = bh
        ref = oracle.attention_block_row(qh, kh, vh, toks, i, ci[rp[r]:rp[r + 1]].tolist(), scale)
        err = np.abs(got_h[toks[i]] - ref)
        worst = max(worst, float(err.max()))
        omax = max(omax, float(np.abs(ref).max()))
    ulps = worst / float(bf16_half_ulp(omax))
    print(f"[full] {label}: {len(rows)} rows, max-abs {worst:.3e}, max |o| {omax:.3f}, "
          f"error {ulps:.2f} bf16 half-ulps at max |o|", flush=True)
    assert worst <= tol, (label, worst)
    return worst, omax, ulps


@pytest.mark.slow
@pytest.mark.parametrize("name,ratio", FULL)
def test_full_size_selection_and_sampled_rows(name, ratio):
    """The bench's launch configuration at full size: every row's block set
    against the oracle, and every output element of all rows of the first and
    the last head plus 256 seeded rows (queue stealing, unions of hundreds of
    blocks and the all-head launch only happen at this size)."""
    cfg = synth.get_config(name)
    if ratio is not None:
        cfg = cfg.with_budget("ratio", ratio)
    print(f"[full] {cfg.name}", flush=True)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    o, rp, ci = run_attn(cfg, x)
    rp, ci = csr_rows(rp, ci)
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    ndiff = compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), cfg.name)
    print(f"[full] {cfg.name}: rows {len(sel.counts)}, differing {ndiff}, "
          f"ambiguous(m<=1e-3) {(sel.margins <= 1e-3).sum()}", flush=True)
    check_rows(cfg, x, o, rp, ci, parity_rows(cfg, g.nblk, cfg.seed), BF16_TOL, cfg.name)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mid", "ragged"])
def test_full_size_sics_every_block(name):
    cfg = synth.get_config(name)
    print(f"[full sics] {cfg.name}", flush=True)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    qm, km, qs, ks = spade.summarize_sics(to_dev(cfg, x["q"]), to_dev(cfg, x["k"]), grid, block)
    assert_sics_close(qs, oracle_sics(cfg, x["q"]), name + " q")
    assert_sics_close(ks, oracle_sics(cfg, x["k"]), name + " k")


# ---------------------------------------------------------------------------
# head-wise schemes: blocking candidates, scheme choice, head grouping
# ---------------------------------------------------------------------------

def candidates_for(cfg):
    c0 = (cfg.bt, cfg.bh, cfg.bw)
    c1 = (max(1, cfg.bt // 2), cfg.bh, min(cfg.W, 2 * cfg.bw))
    c2 = (min(cfg.T, 2 * cfg.bt), max(1, cfg.bh // 2), cfg.bw)
    return [c0, c1, c2]


@pytest.mark.parametrize("name", ["tiny", "mid_shape", "ragged_small", "d64", "ragged_f32"])
def test_scheme_select_matches_oracle(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    agg, scheme = spade.scheme_select(qd, kd, (cfg.T, cfg.Hh, cfg.W), cands)
    ref = oracle.scheme_aggregate(to_f64(cfg, x["q"]), to_f64(cfg, x["k"]), cfg.T, cfg.Hh, cfg.W, cands)
    np.testing.assert_allclose(agg.cpu().numpy().astype(np.float64), ref, rtol=1e-6, atol=1e-9)
    choice, margin = oracle.choose_scheme(ref)
    got = scheme.cpu().numpy()
    # both sides decide in fp64 over the same fp32 per-block values
    assert ((got == choice) | (margin <= 1e-9)).all()


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mid", "ragged"])
def test_full_size_scheme_select(name):
    """Scheme selection over the three blocking candidates bench.py times, at
    the full workload: every (b, h) aggregate and choice against the oracle."""
    cfg = synth.get_config(name)
    print(f"[full schemes] {name}", flush=True)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    qd, kd = to_dev(cfg, x["q"]), to_dev(cfg, x["k"])
    agg, scheme = spade.scheme_select(qd, kd, (cfg.T, cfg.Hh, cfg.W), cands)
    ref = oracle.scheme_aggregate(to_f64(cfg, x["q"]), to_f64(cfg, x["k"]), cfg.T, cfg.Hh, cfg.W, cands)
    np.testing.assert_allclose(agg.cpu().numpy().astype(np.float64), ref, rtol=1e-6, atol=1e-9)
    choice, margin = oracle.choose_scheme(ref)
    got = scheme.cpu().numpy()
    assert ((got == choice) | (margin <= 1e-9)).all()
    print(f"[full schemes] {name}: choices {np.bincount(got.ravel(), minlength=len(cands))}, "
          f"min margin {margin.min():.2e}", flush=True)


def test_scheme_choice_follows_constructed_fields():
    """Tokens constant along time pick the temporal blocking; tokens constant
    within each frame pick the spatial one (aggregate 1 exactly)."""
    T, Hh, W, d = 4, 8, 8, 64
    rng = np.random.default_rng(21)
    col = rng.standard_normal((Hh * W, d)).astype(np.float32)
    frame = rng.standard_normal((T, d)).astype(np.float32)
    x = np.stack([np.tile(col, (T, 1)), np.repeat(frame, Hh * W, axis=0)])[None]  # [1, 2, N, d]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    cands = [(4, 1, 1), (1, 2, 2), (2, 1, 2)]
    agg, scheme = spade.scheme_select(xd, xd, (T, Hh, W), cands)
    a = agg.cpu().numpy()
    assert scheme.cpu().tolist() == [[0, 1]]
    assert abs(a[0, 0, 0] - 1.0) < 1e-6 and abs(a[1, 0, 1] - 1.0) < 1e-6


@pytest.mark.parametrize("name", ["tiny", "mid_shape", "ragged_small", "ragged_f32", "mid_full", "dense_mixed"])
def test_attn_schemes_matches_oracle_and_single_scheme_runs(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    grid = (cfg.T, cfg.Hh, cfg.W)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, scheme, agg = spade.attn_schemes(q, k, v, grid, cands, cfg.mode, cfg.per_head_budget())
    torch.cuda.synchronize()
    sch = scheme.cpu().numpy()
    # the choice equals the selection-only call's bit for bit (there, every
    # candidate's SICS come from a SICS-only pass)
    agg_s, scheme_s = spade.scheme_select(q, k, grid, cands)
    assert torch.equal(agg, agg_s) and torch.equal(scheme, scheme_s)
    # per head: bit for bit the single-scheme run with that head's blocking
    for c, blk in enumerate(cands):
        oc, _, _ = spade.attn(q, k, v, grid, blk, cfg.mode, cfg.per_head_budget())
        m = torch.from_numpy(sch == c).cuda()
        assert torch.equal(o[m], oc[m]), f"{name}: heads of candidate {c}"
    # and against the oracle's head-wise path (its own scheme choice)
    ref, choice, _ = oracle.spade_attn_schemes(*(to_f64(cfg, x[n]) for n in ("q", "k", "v")), cfg.T, cfg.Hh,
                                               cfg.W, cands, cfg.mode, cfg.per_head_budget())
    _, margin = oracle.choose_scheme(oracle.scheme_aggregate(to_f64(cfg, x["q"]), to_f64(cfg, x["k"]),
                                                             cfg.T, cfg.Hh, cfg.W, cands))
    same = (sch == choice)
    assert (same | (margin <= 1e-9)).all()
    tol = BF16_TOL if cfg.dtype == "bf16" else F32_TOL
    of = dev_to_f64(o)
    assert np.abs(of[same] - ref[same]).max() <= tol


@pytest.mark.parametrize("name,summarizer", [("mid_shape", "mean"), ("ragged_small", "max"), ("tail24", "min"),
                                             ("d64", "mean"), ("big_block", "mean")])
def test_fused_pack_pass_sics_equal_the_sics_pass(name, summarizer):
    """spade_attn_schemes takes candidate 0's per-block SICS from the pass
    that also summarizes and packs Q/K/V.  With one candidate its workspace
    keeps them at the end (after the fp64 aggregates, 256-byte aligned):
    they equal spade_summarize_sics's bit for bit."""
    from input_adaptive_block_amd import _lib
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    p = spade.problem_for(q, grid, block, summarizer=summarizer)
    bud = spade.Budget(cfg.mode, cfg.per_head_budget())
    n = spade.spade_schemes_workspace_bytes(p, [block], bud)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    agg = torch.empty(1, cfg.B, cfg.H, dtype=torch.float32, device="cuda")
    scheme = torch.empty(cfg.B, cfg.H, dtype=torch.int32, device="cuda")
    _lib.spade_attn_schemes(p, q, k, v, [block], bud, o, agg, scheme, ws, n)
    torch.cuda.synchronize()
    BH, nblk = cfg.B * cfg.H, spade.spade_num_blocks(p)
    a256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    q_off = a256(8 * BH)
    k_off = q_off + a256(4 * BH * nblk)
    fused_q = ws[q_off:q_off + 4 * BH * nblk].view(torch.float32).view(cfg.B, cfg.H, nblk)
    fused_k = ws[k_off:k_off + 4 * BH * nblk].view(torch.float32).view(cfg.B, cfg.H, nblk)
    _, _, qs, ks = spade.summarize_sics(q, k, grid, block, summarizer)
    assert torch.equal(fused_q, qs) and torch.equal(fused_k, ks)
    # and the output is the plain path's
    o_plain, _, _ = spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget(), summarizer=summarizer)
    assert torch.equal(o, o_plain)


@pytest.mark.parametrize("name,window,summarizer", [("mid_shape", (1, 1, 1), "max"), ("ragged_small", (0, 1, 0), "mean"),
                                                     ("tiny", (1, 0, 0), "min")])
def test_attn_schemes_with_window_and_summarizer(name, window, summarizer):
    """The three extensions together: head-wise schemes whose per-candidate
    paths use a static window and a max/min summarizer; every head equals its
    single-scheme run bit for bit and the oracle's head-wise path."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    grid = (cfg.T, cfg.Hh, cfg.W)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    bud = cfg.per_head_budget()
    o, scheme, agg = spade.attn_schemes(q, k, v, grid, cands, cfg.mode, bud, summarizer=summarizer,
                                        window=window)
    torch.cuda.synchronize()
    sch = scheme.cpu().numpy()
    for c, blk in enumerate(cands):
        oc, _, _ = spade.attn(q, k, v, grid, blk, cfg.mode, bud, summarizer=summarizer, window=window)
        m = torch.from_numpy(sch == c).cuda()
        assert torch.equal(o[m], oc[m]), f"{name}: heads of candidate {c}"
    ref, choice, _ = oracle.spade_attn_schemes(*(to_f64(cfg, x[n]) for n in ("q", "k", "v")), cfg.T, cfg.Hh,
                                               cfg.W, cands, cfg.mode, bud, summarizer=summarizer,
                                               window=window)
    _, margin = oracle.choose_scheme(oracle.scheme_aggregate(to_f64(cfg, x["q"]), to_f64(cfg, x["k"]),
                                                             cfg.T, cfg.Hh, cfg.W, cands))
    same = (sch == choice)
    assert (same | (margin <= 1e-9)).all()
    tol = BF16_TOL if cfg.dtype == "bf16" else F32_TOL
    assert np.abs(dev_to_f64(o)[same] - ref[same]).max() <= tol


@pytest.mark.slow
def test_full_size_attn_schemes_ragged():
    """Head-wise schemes at full size (the Ragged layer at ratio 0.5, where
    two of the three candidates win): every head equals its single-scheme run
    bit for bit, and each single-scheme run matches the oracle on all rows of
    the first and last head that chose it plus sampled rows, with its CSR."""
    cfg = synth.get_config("ragged").with_budget("ratio", 0.5)
    print(f"[full schemes attn] {cfg.name}", flush=True)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    grid = (cfg.T, cfg.Hh, cfg.W)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, scheme, agg = spade.attn_schemes(q, k, v, grid, cands, cfg.mode, cfg.per_head_budget())
    torch.cuda.synchronize()
    sch = scheme.cpu().numpy()
    counts = np.bincount(sch.ravel(), minlength=len(cands))
    print(f"[full schemes attn] choices {counts}", flush=True)
    assert (counts > 0).sum() >= 2  # head grouping really splits the launch
    ref = oracle.scheme_aggregate(to_f64(cfg, x["q"]), to_f64(cfg, x["k"]), cfg.T, cfg.Hh, cfg.W, cands)
    choice, margin = oracle.choose_scheme(ref)
    assert ((sch == choice) | (margin <= 1e-9)).all()
    for c, blk in enumerate(cands):
        m = sch == c
        if not m.any():
            continue
        oc, rp, ci = spade.attn(q, k, v, grid, blk, cfg.mode, cfg.per_head_budget())
        assert torch.equal(o[torch.from_numpy(m).cuda()], oc[torch.from_numpy(m).cuda()]), c
        cc = dataclasses.replace(cfg, bt=blk[0], bh=blk[1], bw=blk[2])
        g = geom(cc)
        heads = [b * cfg.H + h for b in range(cfg.B) for h in range(cfg.H) if m[b, h]]
        rows = set(range(heads[0] * g.nblk, (heads[0] + 1) * g.nblk))
        rows |= set(range(heads[-1] * g.nblk, (heads[-1] + 1) * g.nblk))
        rng = np.random.default_rng(cfg.seed + c)
        for bh in rng.choice(heads, size=min(len(heads), 8), replace=False).tolist():
            rows |= set((bh * g.nblk + rng.choice(g.nblk, size=16, replace=False)).tolist())
        rp_h, ci_h = csr_rows(rp, ci)
        check_rows(cc, x, oc, rp_h, ci_h, sorted(rows), BF16_TOL, f"{cfg.name} candidate {blk}")


def f32_logit_bound(xf, scale):
    """(L, bound) for the fp32 path: L = scale max|q| max|k| bounds every
    logit, and fp32 rounding of a d-term dot product moves a logit by at most
    about sqrt(d) 2^-24 L, so the output moves by at most 8 sqrt(d) 2^-24 L
    max|v| (the factor 8 covers the max subtraction, the exponential and the
    normalisation)."""
    d = xf["q"].shape[-1]
    L = scale * np.linalg.norm(xf["q"], axis=-1).max() * np.linalg.norm(xf["k"], axis=-1).max()
    return L, 8 * math.sqrt(d) * 2.0 ** -24 * L * np.abs(xf["v"]).max()


def test_f32_debug_path_with_large_logits():
    """The fp32 debug path on the mid block shape with hot blocks (+3 on every
    channel of some blocks): logits reach about 110, where fp32 rounding of
    the 128-term dot products alone moves a logit by about sqrt(d) 2^-24 |logit|.
    Selection must match the oracle; the output error is held to that
    arithmetic's bound 8 sqrt(d) 2^-24 L max|v| (L the largest scale |q| |k|
    of the layer) and reported, next to the 1e-5 bar of small logits."""
    base = synth.get_config("mid_shape")
    cfg = dataclasses.replace(base, name="mid_shape_f32", dtype="f32")
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    o, rp, ci = run_attn(cfg, x)
    rp, ci = csr_rows(rp, ci)
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    scale = oracle.default_scale(cfg.d)
    S_ref = oracle.estimate(oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"]), scale)
    sel = oracle.select(S_ref, cfg.mode, cfg.per_head_budget())
    assert compare_selection(sel, rp, ci, S_ref, cfg.mode, cfg.per_head_budget(), cfg.name) == 0
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
    err = float(np.abs(dev_to_f64(o) - ref).max())
    L, bound = f32_logit_bound(xf, scale)
    print(f"[f32 large logits] max logit bound {L:.1f}, max-abs error {err:.3e}, bound {bound:.3e}", flush=True)
    assert err <= max(F32_TOL, bound)


def test_single_candidate_equals_the_plain_path():
    cfg = synth.get_config("mid_shape")
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o1, scheme, agg = spade.attn_schemes(q, k, v, grid, [block], cfg.mode, cfg.per_head_budget())
    o0, _, _ = spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget())
    assert (scheme == 0).all()
    assert torch.equal(o1, o0)



@pytest.mark.parametrize("name", ["mid_full", "dense_mixed", "ragged_small"])
def test_whole_path_in_a_hip_graph(name):
    """The whole path (pack, estimate + select, chunked scan, compaction,
    unit counter, attention) records into a HIP graph: every launch is a
    kernel on the caller's stream, with no memset node and no host call.
    Each of three replays, with eager work and synchronisations between
    them, equals the eager call bit for bit."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    p = spade.problem_for(q, grid, block)
    bud = spade.Budget(cfg.mode, cfg.per_head_budget())
    cap = spade.spade_max_nnz(p, bud)
    R = cfg.B * cfg.H * spade.spade_num_blocks(p)
    ws = spade.alloc_workspace(p, q.device)
    o_ref, rp_ref, ci_ref = spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget())
    o = torch.empty_like(q)
    rp = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(cap, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        spade.spade_attn(p, q, k, v, bud, o, rp, ci, cap, ws, ws.numel(), side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        spade.spade_attn(p, q, k, v, bud, o, rp, ci, cap, ws, ws.numel(), side)
    nnz = int(rp_ref[-1])
    for rep in range(3):
        o.fill_(float("nan"))
        ci.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(rp, rp_ref), rep
        assert torch.equal(ci[:nnz], ci_ref[:nnz]), rep
        assert torch.equal(o, o_ref), rep
        # eager work between replays
        spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget())
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# seeded random problems: shapes, ragged tails, head dims, budgets, windows
# and summarizers drawn together, so that combinations no named case lists
# still meet the oracle
# ---------------------------------------------------------------------------

def random_case(seed):
    """A small seeded problem: every grid axis gets a ragged tail with
    probability 2/3, block tokens up to 512, at most 4 (batch, head) pairs and
    6,000 tokens, so the oracle finishes in a second or two."""
    r = np.random.Generator(np.random.PCG64([seed, 71]))
    bt, bh, bw = int(r.integers(1, 5)), int(r.integers(1, 9)), int(r.integers(1, 17))
    while True:
        ext = [b * int(r.integers(1, 7)) + (int(r.integers(0, b)) if r.random() < 2 / 3 else 0)
               for b in (bt, bh, bw)]
        if all(e > 0 for e in ext) and ext[0] * ext[1] * ext[2] <= 6000:
            break
    T, Hh, W = ext
    B, H = [(1, 1), (1, 2), (2, 1), (2, 2), (1, 4)][int(r.integers(0, 5))]
    d = (64, 128)[int(r.integers(0, 2))]
    dtype = "f32" if r.random() < 0.2 else "bf16"
    cfg = synth.Config(f"random{seed}", B=B, H=H, d=d, T=T, Hh=Hh, W=W, bt=bt, bh=bh, bw=bw,
                       dtype=dtype, sigma=float(r.uniform(0.2, 1.0)), amp_kind="uniform",
                       amp_params=(0.2, 2.5), mode="count", budget=(1,), seed=1000 + seed)
    nblk = cfg.nblk
    mode = ("count", "ratio", "mass")[int(r.integers(0, 3))]
    window = None
    if r.random() < 0.4:
        window = tuple(int(x) for x in r.integers(0, 3, size=3))
    lo = 0 if window is not None and r.random() < 0.3 else 1
    if mode == "count":
        budget = [float(r.integers(lo, nblk + 1)) for _ in range(H)]
    elif mode == "ratio":
        budget = [0.0 if lo == 0 and r.random() < 0.5 else float(r.uniform(0.02, 1.0)) for _ in range(H)]
    else:
        budget = [0.0 if lo == 0 and r.random() < 0.5 else float(r.uniform(0.05, 0.999)) for _ in range(H)]
    summarizer = ("mean", "mean", "max", "min")[int(r.integers(0, 4))]
    return cfg, mode, budget, window, summarizer


RANDOM_SEEDS = list(range(48))


@pytest.mark.parametrize("seed", RANDOM_SEEDS)
def test_random_problems_match_oracle(seed):
    cfg, mode, budget, window, summarizer = random_case(seed)
    label = (f"seed {seed}: B{cfg.B} H{cfg.H} d{cfg.d} {cfg.dtype} grid {cfg.T}x{cfg.Hh}x{cfg.W} "
             f"block {cfg.bt}x{cfg.bh}x{cfg.bw} {mode} {budget} window {window} {summarizer}")
    print(label, flush=True)
    x = synth.make_inputs(cfg)
    g = geom(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, rp, ci = spade.attn(q, k, v, grid, block, mode, budget, summarizer=summarizer, window=window)
    torch.cuda.synchronize()
    rp, ci = csr_rows(rp, ci)
    scale = oracle.default_scale(cfg.d)
    if summarizer == "mean":
        qs, ks = oracle_means(cfg, x["q"]), oracle_means(cfg, x["k"])
    else:
        qs, ks = oracle_summaries(cfg, x["q"], summarizer), oracle_summaries(cfg, x["k"], summarizer)
    S_ref = oracle.estimate(qs, ks, scale)
    sel = oracle.select(S_ref, mode, budget, window=window, g=g)
    assert compare_selection(sel, rp, ci, S_ref, mode, budget, label) == 0, label
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], g, rp, ci, scale)
    # fp32: 1e-5, or the rounding bound of the dot products where the drawn
    # amplitudes make logits large
    tol = BF16_TOL if cfg.dtype == "bf16" else max(F32_TOL, f32_logit_bound(xf, scale)[1])
    err = np.abs(dev_to_f64(o) - ref).max()
    assert err <= tol, f"{label}: max error {err} (bar {tol:.2e})"


def random_candidates(r, cfg, n):
    """n further blocking candidates for the grid of cfg: distinct shapes of at
    most 512 tokens, each axis at most the grid's extent; first those with the
    layer block's token count (whose aggregates differ only by the shape, so
    that heads may choose differently), then any."""
    lim = (min(cfg.T, 8), min(cfg.Hh, 8), min(cfg.W, 16))
    n0 = cfg.bt * cfg.bh * cfg.bw
    same = [(a, b, n0 // (a * b)) for a in range(1, lim[0] + 1) for b in range(1, lim[1] + 1)
            if n0 % (a * b) == 0 and n0 // (a * b) <= lim[2] and (a, b, n0 // (a * b)) != (cfg.bt, cfg.bh, cfg.bw)]
    out = [same[i] for i in r.permutation(len(same))[:n]]
    while len(out) < n:
        blk = (int(r.integers(1, min(cfg.T, 8) + 1)), int(r.integers(1, min(cfg.Hh, 8) + 1)),
               int(r.integers(1, min(cfg.W, 16) + 1)))
        if blk[0] * blk[1] * blk[2] <= 512 and blk != (cfg.bt, cfg.bh, cfg.bw) and blk not in out:
            out.append(blk)
    return out


@pytest.mark.parametrize("seed", list(range(16)))
def test_random_head_wise_schemes(seed):
    """Head-wise schemes on seeded random problems with two to four blocking
    candidates: the choice against the oracle's aggregates, every head bit for
    bit the single-scheme run with the blocking it chose, and each of those
    runs against the oracle (selection row by row, outputs on its CSR)."""
    cfg, mode, budget, window, summarizer = random_case(100 + seed)
    # heads of pure noise next to heads of structured tokens, so that heads
    # can choose different blockings
    cfg = dataclasses.replace(cfg, amp_kind="split", amp_params=(max(1, cfg.H // 2), 0.0, 2.5))
    r = np.random.Generator(np.random.PCG64([seed, 72]))
    cands = [(cfg.bt, cfg.bh, cfg.bw)] + random_candidates(r, cfg, int(r.integers(1, 4)))
    geoms = [oracle.Geometry(cfg.T, cfg.Hh, cfg.W, *blk) for blk in cands]
    if mode == "count":
        budget = [min(b, min(gc.nblk for gc in geoms)) for b in budget]
    label = (f"seed {seed}: B{cfg.B} H{cfg.H} d{cfg.d} {cfg.dtype} grid {cfg.T}x{cfg.Hh}x{cfg.W} "
             f"candidates {cands} {mode} {budget} window {window} {summarizer}")
    print(label, flush=True)
    x = synth.make_inputs(cfg)
    grid = (cfg.T, cfg.Hh, cfg.W)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, scheme, agg = spade.attn_schemes(q, k, v, grid, cands, mode, budget, summarizer=summarizer, window=window)
    torch.cuda.synchronize()
    sch = scheme.cpu().numpy()
    xf = {n: to_f64(cfg, x[n]) for n in ("q", "k", "v")}
    ref_agg = oracle.scheme_aggregate(xf["q"], xf["k"], cfg.T, cfg.Hh, cfg.W, cands)
    np.testing.assert_allclose(agg.cpu().numpy().astype(np.float64), ref_agg, rtol=1e-6, atol=1e-9)
    choice, margin = oracle.choose_scheme(ref_agg)
    assert ((sch == choice) | (margin <= 1e-9)).all(), label
    scale = oracle.default_scale(cfg.d)
    tol = BF16_TOL if cfg.dtype == "bf16" else max(F32_TOL, f32_logit_bound(xf, scale)[1])
    for c, (blk, gc) in enumerate(zip(cands, geoms)):
        if not (sch == c).any():
            continue
        oc, rp, ci = spade.attn(q, k, v, grid, blk, mode, budget, summarizer=summarizer, window=window)
        torch.cuda.synchronize()
        m = torch.from_numpy(sch == c).cuda()
        assert torch.equal(o[m], oc[m]), f"{label}: heads of candidate {c}"
        rp, ci = csr_rows(rp, ci)
        qs = np.empty((cfg.B, cfg.H, gc.nblk, cfg.d))
        ks = np.empty_like(qs)
        for h in range(cfg.H):
            qs[:, h:h + 1] = oracle.summarize(xf["q"][:, h:h + 1], gc, op=summarizer)
            ks[:, h:h + 1] = oracle.summarize(xf["k"][:, h:h + 1], gc, op=summarizer)
        S_ref = oracle.estimate(qs, ks, scale)
        sel = oracle.select(S_ref, mode, budget, window=window, g=gc)
        assert compare_selection(sel, rp, ci, S_ref, mode, budget, f"{label} / {blk}") == 0
        ref = oracle.attention_full(xf["q"], xf["k"], xf["v"], gc, rp, ci, scale)
        err = np.abs(dev_to_f64(oc) - ref).max()
        assert err <= tol, f"{label} / {blk}: max error {err}"
