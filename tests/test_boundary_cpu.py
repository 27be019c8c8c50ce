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
    # three packed bf16 tensors padded to 128-row tiles; the fp64 scores stay
    # in LDS (630 blocks fit the fused estimate/select tile)
    assert n >= 3 * cfg.H * 630 * 128 * 128 * 2
    assert n < 3 * cfg.H * 630 * 128 * 128 * 2 + cfg.H * 630 * 630 * 8
    # rows wider than the tile keep the fp64 scores in the workspace
    wide = _prob(synth.get_config("max_blocks"))
    assert spade.spade_workspace_bytes(wide) >= 4096 * 4096 * 8
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


def test_misaligned_workspace_rejected_before_launch():
    """Every entry point that takes a workspace needs it on a 256-byte
    boundary; otherwise INVALID_ARG before anything is launched (the other
    pointers here are stand-ins, never dereferenced)."""
    cfg = synth.get_config("small")
    p = _prob(cfg)
    b = spade.Budget("ratio", [0.25] * cfg.H)
    cap = spade.spade_max_nnz(p, b)
    need = spade.spade_workspace_bytes(p)
    good = [(cfg.bt, cfg.bh, cfg.bw), (1, 6, 8)]
    n_sel = spade.spade_schemes_workspace_bytes(p, good)
    n_att = spade.spade_schemes_workspace_bytes(p, good, b)
    d = 0x100000  # a stand-in device address
    for ws in (d + 16, d + 128, d + 4):
        calls = [
            lambda: spade.spade_estimate_select(p, d, d, b, d, d, cap, ws, need, stream=0),
            lambda: spade.spade_block_sparse_attn(p, d, d, d, d, d, cap, d, ws, need, stream=0),
            lambda: spade.spade_attn(p, d, d, d, b, d, d, d, cap, ws, need, stream=0),
            lambda: spade.spade_scheme_select(p, d, d, good, d, d, ws, n_sel, stream=0),
            lambda: spade.spade_attn_schemes(p, d, d, d, good, b, d, d, d, ws, n_att, stream=0),
        ]
        for call in calls:
            with pytest.raises(spade.SpadeError) as e:
                call()
            assert e.value.status == INVALID, ws


def test_empty_batch_is_a_noop():
    cfg = synth.get_config("small")
    p = _prob(cfg, B=0)
    spade.spade_summarize(p, 0, 0, 0, 0, stream=0)  # nothing to do, nothing launched
    spade.spade_summarize_sics(p, 0, 0, 0, 0, 0, 0, stream=0)
    spade.spade_debug_scores(p, 0, 0, 0, stream=0)


def test_status_strings():
    for s in range(5):
        assert spade.status_string(s).startswith("SPADE_")


# ---------------------------------------------------------------------------
# Python wrappers: every tensor's shape, dtype and length is checked before
# any C call (forms before devices, so each check runs without a GPU)
# ---------------------------------------------------------------------------

def _cpu_problem(name="tiny_bf16"):
    torch = pytest.importorskip("torch")
    cfg = synth.get_config(name)
    q = torch.zeros(cfg.B, cfg.H, cfg.N, cfg.d, dtype=torch.bfloat16)
    g = oracle.Geometry(cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw)
    grid, block = (cfg.T, cfg.Hh, cfg.W), (cfg.bt, cfg.bh, cfg.bw)
    return torch, cfg, g, q, grid, block


def _raises(match, status, fn, *a, **kw):
    with pytest.raises(spade.SpadeError, match=match) as ei:
        fn(*a, **kw)
    assert ei.value.status == status


def test_estimate_select_checks_summaries():
    torch, cfg, g, q, grid, block = _cpu_problem()
    p = spade.problem_for(q, grid, block)
    good = torch.zeros(cfg.B, cfg.H, g.nblk, cfg.d)
    bud = ("count", [3] * cfg.H)
    _raises("q_mean has shape", INVALID, spade.estimate_select, good[:, :, :-1], good, p, *bud)
    _raises("k_mean has dtype", INVALID, spade.estimate_select, good, good.double(), p, *bud)
    _raises("k_mean must be contiguous", INVALID, spade.estimate_select, good, good.transpose(2, 3).contiguous().transpose(2, 3), p, *bud)
    _raises("q_mean must be a device tensor", INVALID, spade.estimate_select, good, good, p, *bud)
    _raises("q_mean has shape", INVALID, spade.debug_scores, good[..., :8], good, p)


def test_block_sparse_attn_checks_csr_and_output():
    torch, cfg, g, q, grid, block = _cpu_problem()
    R = cfg.B * cfg.H * g.nblk
    rp = torch.zeros(R + 1, dtype=torch.int32)
    ci = torch.zeros(4, dtype=torch.int32)
    f = spade.block_sparse_attn
    _raises("row_ptr has shape", INVALID, f, q, q, q, grid, block, rp[:-1], ci)
    _raises("row_ptr has dtype", INVALID, f, q, q, q, grid, block, rp.long(), ci)
    _raises("col_idx must be a one-dimensional", INVALID, f, q, q, q, grid, block, rp, ci.view(2, 2))
    _raises("col_idx has dtype", INVALID, f, q, q, q, grid, block, rp, ci.float())
    _raises("out has dtype", INVALID, f, q, q, q, grid, block, rp, ci, out=q.float())
    _raises("out has shape", INVALID, f, q, q, q, grid, block, rp, ci, out=q[:, :1])
    _raises("v has shape", INVALID, f, q, q, q[..., :32], grid, block, rp, ci)
    _raises("q must be a device tensor", INVALID, f, q, q, q, grid, block, rp, ci)


def test_attn_checks_workspace():
    torch, cfg, g, q, grid, block = _cpu_problem()
    p = spade.problem_for(q, grid, block)
    need = spade.spade_workspace_bytes(p)
    small = torch.zeros(need - 1, dtype=torch.uint8)
    _raises("workspace has", CAP, spade.attn, q, q, q, grid, block, "count", [3] * cfg.H, workspace=small)
    wrong = torch.zeros(need, dtype=torch.int8)
    _raises("workspace has dtype", INVALID, spade.attn, q, q, q, grid, block, "count", [3] * cfg.H,
            workspace=wrong)
    _raises("workspace has shape", INVALID, spade.attn, q, q, q, grid, block, "count", [3] * cfg.H,
            workspace=torch.zeros(2, need, dtype=torch.uint8))
    _raises("q must be a device tensor", INVALID, spade.attn, q, q, q, grid, block, "count", [3] * cfg.H,
            workspace=torch.zeros(need, dtype=torch.uint8))


def _static_scratch_need(p, nblk):
    """The selection scratch of spade_estimate_select_static, as the header
    states it."""
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    R = p.B * p.H * nblk
    wide = 8 * R * nblk if nblk > 1024 else 0
    return a(4 * R) + a(4 * R * ((nblk + 31) // 32)) + a(wide) + a(4 * ((R + 4095) // 4096 + 1))


def test_static_select_rejects_before_device():
    """The allocation-free entry point checks its arguments, and the size of
    the static buffer, before it looks up that buffer or launches anything."""
    text = open(os.path.join(ROOT, "include", "spade.h")).read()
    m = re.search(r"#define SPADE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == spade.SPADE_STATIC_SCRATCH_BYTES
    cfg = synth.get_config("mid")
    p = _prob(cfg)
    b = spade.Budget("mass", [0.9] * cfg.H)
    cap = spade.spade_max_nnz(p, b)
    for args, status in [((0, 0, b, 1, 1, cap - 1), CAP), ((0, 0, b, 0, 1, cap), INVALID),
                         ((0, 0, b, 1, 1, cap), INVALID)]:
        with pytest.raises(spade.SpadeError) as e:
            spade.spade_estimate_select_static(p, *args, stream=0)
        assert e.value.status == status, args
    assert _static_scratch_need(p, 630) == 2016000 + 100864 + 256  # 2.02 MiB for the 40-head layer
    # batches of that layer: accepted (then stopped by the null summaries) up
    # to the buffer's size, CAPACITY beyond it
    seen = set()
    for B in range(1, 7):
        q = _prob(cfg, B=B)
        fits = _static_scratch_need(q, 630) <= spade.SPADE_STATIC_SCRATCH_BYTES
        seen.add(fits)
        with pytest.raises(spade.SpadeError) as e:
            spade.spade_estimate_select_static(q, 0, 0, b, 1, 1, spade.spade_max_nnz(q, b), stream=0)
        assert e.value.status == (INVALID if fits else CAP), B
    assert seen == {True, False}
    # rows wider than 1024 blocks would keep their fp64 scores there too,
    # more than the buffer holds even for one head
    q = spade.Problem(1, 1, 32 * 33, 64, 1, 32, 33, 1, 1, 1, spade.SPADE_BF16, 0.0)
    nblk = spade.spade_num_blocks(q)
    assert nblk == 1056 and _static_scratch_need(q, nblk) > spade.SPADE_STATIC_SCRATCH_BYTES
    bw = spade.Budget("ratio", [0.1])
    with pytest.raises(spade.SpadeError) as e:
        spade.spade_estimate_select_static(q, 0, 0, bw, 1, 1, spade.spade_max_nnz(q, bw), stream=0)
    assert e.value.status == CAP


@pytest.mark.parametrize("name,dense", [("small", 1), ("small_shape", 1), ("dense_mixed", 1), ("dense_40", 1),
                                        ("mid", 0), ("large", 0), ("mid_full", 0), ("d64", 0), ("ragged", 0),
                                        ("mid_shape", 0), ("tail24", 0), ("big_block", 0), ("tiny", 0),
                                        ("tiny_bf16", 0), ("token_level", 0)])
def test_attention_walk_by_block_shape(name, dense):
    """Blocks of 72 or 40 tokens (every block a multiple of 8, at least 32)
    are streamed back to back; 120-, 64-, 32- and 256-token blocks, shapes
    with a partial block of 24, 60 or 16 tokens, and fp32 are padded to whole
    32-key subtiles."""
    cfg = synth.get_config(name)
    assert spade.spade_debug_dense_walk(_prob(cfg)) == dense
    assert spade.spade_debug_dense_walk(_prob(cfg, dtype=spade.SPADE_F32)) == 0


def test_device_code_fits_its_registers_without_scratch():
    """Every kernel of the library runs without scratch (private) memory and
    without register spills, so no launch makes the runtime set scratch
    aside (the allocation-free entry point relies on that), and the kernels
    that depend on their occupancy fit it: the attention kernel's twelve
    waves per CU (three per SIMD: at most 168 registers) and the fused
    selection kernel's four waves per SIMD (at most 128)."""
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_spade_build", os.path.join(ROOT, "input_adaptive_block_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    res = mod.kernel_resources()
    assert len(res) >= 40
    for name, r in res.items():
        assert r["scratch"] == 0 and r["vgpr_spill"] == 0, (name, r)
        if "bsattn_bf16_kernel" in name:
            assert r["vgpr"] <= 168, (name, r)
        if "estimate_select_kernel" in name and ("ELi12EE" not in name and "ELi16EE" not in name):
            assert r["vgpr"] <= 128, (name, r)


def test_attention_stage_loop_code_phase():
    """The d = 128 attention kernel's stage loop sits 16 bytes past a 32-byte
    boundary of its code (first MFMA offset = 16 mod 32): at the other 8-byte
    phases the loop measured 1 % slower (Mid: 57.5 ms at phases 16 and 48 of
    64, 58.0-58.5 ms at 0, 8, 24 and 56).  A change to the code before the loop
    moves it; the no-ops at the start of each unit then need retuning."""
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_spade_build", os.path.join(ROOT, "input_adaptive_block_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    offs = mod.first_mfma_offsets()
    key = [k for k in offs if "bsattn_bf16_kernelILi128ELb0E" in k]
    assert len(key) == 1, sorted(offs)
    assert offs[key[0]] % 32 == 16, offs[key[0]]
