"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and its validation / sizing helpers behave as include/spade.h states.
Nothing here touches a GPU (only host-only entry points and argument errors
that return before any launch)."""
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

spade = pytest.importorskip("input_adaptive_block_amd")
from input_adaptive_block_amd import _lib  # noqa: E402

OK, INVALID, UNSUP, CAP = (spade.SPADE_OK, spade.SPADE_ERR_INVALID_ARG, spade.SPADE_ERR_UNSUPPORTED,
                           spade.SPADE_ERR_CAPACITY)


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "spade.h")).read()
    return sorted(set(re.findall(
        r"^(?:const\s+char\s*\*|int32_t|int64_t|size_t|spade_status|void)\s+(spade_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert len(names) >= 10
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def _prob(cfg, **kw):
    d = dict(B=cfg.B, H=cfg.H, N=cfg.N, d=cfg.d, T=cfg.T, Hh=cfg.Hh, W=cfg.W, bt=cfg.bt, bh=cfg.bh,
             bw=cfg.bw, dtype=spade.SPADE_BF16 if cfg.dtype == "bf16" else spade.SPADE_F32, scale=0.0)
    d.update(kw)
    return spade.Problem(**d)


@pytest.mark.parametrize("name", ["mid", "large", "small", "ragged", "tiny"])
def test_num_blocks_matches_oracle(name):
    cfg = synth.get_config(name)
    g = oracle.Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    assert spade.spade_num_blocks(_prob(cfg)) == g.nblk


@pytest.mark.parametrize("name", ["mid", "large", "small", "ragged", "tiny", "ragged_p64", "token_level"])
def test_max_nnz_matches_oracle_keep_counts(name):
    cfg = synth.get_config(name)
    g = oracle.Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    p = _prob(cfg)
    for mode, vals in (("ratio", [0.1, 0.25, 0.5, 1.0, 0.15]), ("count", [1, 2, 3])):
        ph = [vals[h % len(vals)] for h in range(cfg.H)]
        if mode == "count":
            ph = [min(v, g.nblk) for v in ph]
        b = spade.Budget(mode, ph)
        expect = cfg.B * g.nblk * sum(oracle.keep_count(mode, v, g.nblk) for v in ph)
        assert spade.spade_max_nnz(p, b) == expect
        assert spade.spade_check(p, b, expect) == OK
        assert spade.spade_check(p, b, expect - 1) == CAP
    b = spade.Budget("mass", [0.9] * cfg.H)
    assert spade.spade_max_nnz(p, b) == cfg.B * cfg.H * g.nblk * g.nblk


def test_workspace_bytes_covers_packed_tiles():
    cfg = synth.get_config("mid")
    p = _prob(cfg)
    n = spade.spade_workspace_bytes(p)
    # three packed bf16 tensors padded to 128-row tiles + fp64 scores
    assert n >= 3 * cfg.H * 630 * 128 * 128 * 2 + cfg.H * 630 * 630 * 8
    assert n < 4 * 1024 ** 3
    pf = _prob(cfg, dtype=spade.SPADE_F32)
    assert spade.spade_workspace_bytes(pf) < n


@pytest.mark.parametrize("change,status", [
    (dict(N=75601), INVALID),
    (dict(d=96), UNSUP),
    (dict(d=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(bt=0), INVALID),
    (dict(T=0, N=0), INVALID),
    (dict(dtype=7), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(bt=21, bh=45, bw=2), UNSUP),  # 1890-token blocks
    (dict(bt=1, bh=1, bw=1), UNSUP),  # 75600 blocks
    (dict(H=300), UNSUP),
    (dict(scale=0.05), OK),
    (dict(B=0), OK),
])
def test_check_rejections(change, status):
    cfg = synth.get_config("mid")
    assert spade.spade_check(_prob(cfg, **change)) == status


@pytest.mark.parametrize("mode,vals,status", [
    ("count", [0], INVALID), ("count", [1.5], INVALID), ("count", [631], INVALID), ("count", [630], OK),
    ("ratio", [0.0], INVALID), ("ratio", [1.01], INVALID), ("ratio", [float("nan")], INVALID),
    ("ratio", [1e-9], OK), ("mass", [0.0], INVALID), ("mass", [1.0], OK), ("mass", [-0.5], INVALID),
])
def test_budget_rejections(mode, vals, status):
    cfg = synth.get_config("mid")
    p = _prob(cfg)
    b = spade.Budget(mode, vals * cfg.H)
    assert spade.spade_check(p, b, -1) == status


def test_summarizer_field_is_validated():
    cfg = synth.get_config("mid")
    for op in (spade.SPADE_SUM_MEAN, spade.SPADE_SUM_MAX, spade.SPADE_SUM_MIN):
        assert spade.spade_check(_prob(cfg, summarizer=op), None, -1) == spade.SPADE_OK
    for bad in (3, -1, 99):
        p = _prob(cfg, summarizer=bad)
        assert spade.spade_check(p, None, -1) == INVALID
        assert spade.spade_num_blocks(p) == -1
        with pytest.raises(spade.SpadeError) as e:
            spade.spade_summarize(p, 1, 1, 1, 1, stream=0)  # rejected before any launch
        assert e.value.status == INVALID


def test_window_budget_validation_and_capacity():
    cfg = synth.get_config("ragged_small")
    p = _prob(cfg)
    g = oracle.Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    # a budget of 0 needs a window; radii must be >= 0
    assert spade.spade_check(p, spade.Budget("count", [0] * cfg.H), -1) == INVALID
    assert spade.spade_check(p, spade.Budget("ratio", [0.0] * cfg.H), -1) == INVALID
    assert spade.spade_check(p, spade.Budget("count", [0] * cfg.H, (1, 0, 1)), -1) == spade.SPADE_OK
    assert spade.spade_check(p, spade.Budget("mass", [0.0] * cfg.H, (0, 0, 0)), -1) == spade.SPADE_OK
    assert spade.spade_check(p, spade.Budget("count", [2] * cfg.H, (1, -1, 0)), -1) == INVALID
    # capacity with a window: sum over rows of min(nK, k + |window|)
    for radius, k in (((0, 0, 0), 0), ((1, 2, 1), 3), ((9, 9, 9), 5)):
        b = spade.Budget("count", [k] * cfg.H, radius)
        sizes = [len(oracle.window_blocks(g, i, radius)) for i in range(g.nblk)]
        want = cfg.B * cfg.H * sum(min(g.nblk, k + n) for n in sizes)
        assert spade.spade_max_nnz(p, b) == want


def test_scheme_entry_points_validate_before_launch():
    cfg = synth.get_config("small")
    p = _prob(cfg)
    good = [(cfg.bt, cfg.bh, cfg.bw), (1, 6, 8)]
    assert spade.spade_schemes_workspace_bytes(p, good) > 0
    b = spade.Budget("ratio", [0.25] * cfg.H)
    assert spade.spade_schemes_workspace_bytes(p, good, b) > spade.spade_schemes_workspace_bytes(p, good)
    assert spade.spade_schemes_workspace_bytes(p, [(0, 1, 1)]) == 0           # invalid candidate
    assert spade.spade_schemes_workspace_bytes(p, []) == 0                    # no candidate
    assert spade.spade_schemes_workspace_bytes(p, [(1, 1, 1)] * 17) == 0      # too many
    # a count larger than one candidate's block count is invalid for the whole call
    coarse = (3, 30, 11)
    nb = spade.spade_num_blocks(_prob(cfg, bt=3, bh=30, bw=11))
    assert 0 < nb < 40
    assert spade.spade_schemes_workspace_bytes(p, good, spade.Budget("count", [40] * cfg.H)) > 0
    assert spade.spade_schemes_workspace_bytes(p, good + [coarse], spade.Budget("count", [40] * cfg.H)) == 0
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_scheme_select(p, 0, 0, good, 0, 0, 0, 0, stream=0)
    assert e.value.status == CAP
    n = spade.spade_schemes_workspace_bytes(p, good)
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_scheme_select(p, 0, 0, good, 0, 0, 0, n, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_attn_schemes(p, 0, 0, 0, good, b, 0, 0, 0, 0, 0, stream=0)
    assert e.value.status == CAP


def test_bad_mode_rejected():
    cfg = synth.get_config("mid")
    b = spade.Budget(9, [1.0] * cfg.H)
    assert spade.spade_check(_prob(cfg), b, -1) == INVALID


def test_compute_entry_points_reject_before_launch():
    """Argument errors return a status with no device call."""
    cfg = synth.get_config("small")
    p = _prob(cfg)
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_summarize(p, 0, 0, 0, 0, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_summarize_sics(p, 0, 0, 0, 0, 0, 0, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_summarize_sics(_prob(cfg, d=32), 1, 1, 1, 1, 0, 0, stream=0)
    assert e.value.status == UNSUP
    b = spade.Budget("ratio", [0.25] * cfg.H)
    cap = spade.spade_max_nnz(p, b)
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_estimate_select(p, 0, 0, b, 0, 0, cap - 1, 0, 0, stream=0)
    assert e.value.status == CAP
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_attn(p, 0, 0, 0, b, 0, 0, 0, cap, 0, 0, stream=0)
    assert e.value.status == CAP  # workspace of 0 bytes
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_block_sparse_attn(p, 0, 0, 0, 0, 0, -1, 0, 0, 0, stream=0)
    assert e.value.status == INVALID
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_debug_scores(_prob(cfg, d=32), 0, 0, 0, stream=0)
    assert e.value.status == UNSUP


def test_empty_batch_is_a_noop():
    cfg = synth.get_config("small")
    p = _prob(cfg, B=0)
    spade.spade_summarize(p, 0, 0, 0, 0, stream=0)  # nothing to do, nothing launched
    spade.spade_summarize_sics(p, 0, 0, 0, 0, 0, 0, stream=0)
    spade.spade_debug_scores(p, 0, 0, 0, stream=0)


def test_status_strings():
    for s in range(5):
        assert spade.status_string(s).startswith("SPADE_")
