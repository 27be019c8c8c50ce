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
         "token_level", "one_block", "d64", "tail24", "ragged_f32"]


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
@pytest.mark.parametrize("name", ["mid_shape", "ragged_small", "tiny", "d64"])
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
LIMITS = ["max_blocks", "blocks_2k", "max_block_tokens"]


@pytest.mark.parametrize("name", LIMITS)
def test_limits_selection_and_attention_match_oracle(name):
    cfg = synth.get_config(name)
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


@pytest.mark.parametrize("name", ["ragged_small", "ragged_p64", "tiny", "ragged_f32"])
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


@pytest.mark.parametrize("name", ["mid_shape", "ragged_small", "tiny"])
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


def expected_work_queues(cfg, rp):
    """The attention kernel's queue partition, restated: units are 12
    consecutive (row, 32-query subtile) items of a head; a unit costs 1 + the
    kept blocks of each item's row; queue x starts at the first unit whose
    exclusive cost prefix reaches ceil(x * total / 8)."""
    g = geom(cfg)
    ntok = max(len(t) for t in oracle.block_tokens(g))
    nsub = (ntok + 31) // 32
    items = g.nblk * nsub
    per_head = (items + 11) // 12
    kept = np.diff(rp)
    cost = []
    for bh in range(cfg.B * cfg.H):
        for pi in range(per_head):
            its = range(12 * pi, min(items, 12 * pi + 12))
            cost.append(1 + sum(int(kept[bh * g.nblk + it // nsub]) for it in its))
    cost = np.array(cost, dtype=np.int64)
    U = len(cost)
    pre = np.concatenate([[0], np.cumsum(cost)])
    total = int(pre[-1])
    starts = [0]
    for x in range(1, 8):
        t = (x * total + 7) // 8
        hit = np.nonzero(pre[:U] >= t)[0]
        starts.append(int(hit[0]) if len(hit) else U)
    return starts + [U], cost


@pytest.mark.parametrize("name", ["tiny", "ragged_p64", "mid_shape", "small_shape", "ragged_small", "big_block",
                                  "token_level", "max_blocks", "max_block_tokens"])
def test_work_queues_partition_the_units(name):
    """Integer work, checked bit for bit: the eight queue ranges are the
    restated partition, ascending, and cover every unit exactly once."""
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    o, rp, ci = run_attn(cfg, x)
    grid, block = grid_block(cfg)
    p = spade.problem_for(to_dev(cfg, x["q"]), grid, block)
    queue = torch.full((18,), -7, dtype=torch.int32, device="cuda")
    spade.spade_debug_work_queues(p, rp, ci.numel(), queue)
    torch.cuda.synchronize()
    got = queue.cpu().numpy()
    want, cost = expected_work_queues(cfg, rp.cpu().numpy().astype(np.int64))
    assert got[:9].tolist() == want, (got[:9].tolist(), want)
    assert (np.diff(got[:9]) >= 0).all() and got[0] == 0 and got[8] == len(cost)
    assert (got[9:17] == 0).all()  # the cursors (entry 17 is unused)


@pytest.mark.parametrize("name", ["mid_shape", "tiny"])
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


@pytest.mark.slow
@pytest.mark.parametrize("name,ratio", FULL)
def test_full_size_selection_and_sampled_rows(name, ratio):
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
    R = len(sel.counts)
    rng = np.random.default_rng(cfg.seed)
    rows = sorted(set([0, R - 1] + rng.choice(R, size=6, replace=False).tolist()))
    of = o.cpu()
    toks = oracle.block_tokens(g)
    worst = 0.0
    for r in rows:
        bh, i = divmod(r, g.nblk)
        b, h = divmod(bh, cfg.H)
        qh, kh, vh = (to_f64(cfg, x[n][b, h]) for n in ("q", "k", "v"))
        ref = oracle.attention_block_row(qh, kh, vh, toks, i, ci[rp[r]:rp[r + 1]].tolist(), scale)
        got = of[b, h, toks[i]].float().numpy().astype(np.float64)
        worst = max(worst, np.abs(got - ref).max())
    print(f"[full] {cfg.name}: sampled rows {rows} max-abs {worst:.3e}", flush=True)
    assert worst <= BF16_TOL


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


@pytest.mark.parametrize("name", ["tiny", "mid_shape", "ragged_small", "ragged_f32"])
def test_attn_schemes_matches_oracle_and_single_scheme_runs(name):
    cfg = synth.get_config(name)
    x = synth.make_inputs(cfg)
    cands = candidates_for(cfg)
    grid = (cfg.T, cfg.Hh, cfg.W)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o, scheme, agg = spade.attn_schemes(q, k, v, grid, cands, cfg.mode, cfg.per_head_budget())
    torch.cuda.synchronize()
    sch = scheme.cpu().numpy()
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


def test_single_candidate_equals_the_plain_path():
    cfg = synth.get_config("mid_shape")
    x = synth.make_inputs(cfg)
    grid, block = grid_block(cfg)
    q, k, v = (to_dev(cfg, x[n]) for n in ("q", "k", "v"))
    o1, scheme, agg = spade.attn_schemes(q, k, v, grid, [block], cfg.mode, cfg.per_head_budget())
    o0, _, _ = spade.attn(q, k, v, grid, block, cfg.mode, cfg.per_head_budget())
    assert (scheme == 0).all()
    assert torch.equal(o1, o0)

