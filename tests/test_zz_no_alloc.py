"""The allocation-free estimate + select entry point (library-owned static
scratch) against the workspace entry point, through the C ABI.

Both run the same kernels, so the CSRs must be identical (index work:
bit-exact).  The calls come in a row on one device, each one smaller than the
one before, so a call that relied on the buffer's earlier contents would show
up as a difference.  The first two sit on both sides of the row count where
the CSR moves from one kernel to the chunked scan."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import input_adaptive_block_amd as spade  # noqa: E402


def _summaries(cfg):
    x = synth.make_inputs(cfg)

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    grid, block = (cfg.T, cfg.Hh, cfg.W), (cfg.bt, cfg.bh, cfg.bw)
    q, k = dev(x["q"]), dev(x["k"])
    qm, km = spade.summarize(q, k, grid, block)
    return qm, km, spade.problem_for(q, grid, block)


def _same_csr(a, b):
    rp_a, ci_a = (t.cpu().numpy() for t in a)
    rp_b, ci_b = (t.cpu().numpy() for t in b)
    assert np.array_equal(rp_a, rp_b)
    nnz = int(rp_a[-1])
    assert np.array_equal(ci_a[:nnz], ci_b[:nnz])
    return nnz


# (config, budget mode or None for the config's own, per-head value, window)
CALLS = [
    ("rows_32k_plus", None, None, None),            # 32,832 rows: the chunked scan's chunk sums in the buffer
    ("rows_32k", None, None, None),                 # 32,768 rows: the one-kernel CSR's limit
    ("mid", None, None, None),                      # 25,200 rows, mass 0.9
    ("small", None, None, None),                    # 5,460 rows, ratio 0.25
    ("mid_shape", "count", 3, (1, 1, 1)),           # 24 rows, top-3 united with a window
    ("tiny", "mass", 0.5, None),                    # 16 rows
]


def test_static_scratch_matches_workspace_entry():
    prev_rows = None
    for name, mode, value, window in CALLS:
        cfg = synth.get_config(name)
        print(f"[no-alloc] {name}", flush=True)
        qm, km, p = _summaries(cfg)
        if mode is None:
            mode, per_head = cfg.mode, cfg.per_head_budget()
        else:
            per_head = [value] * cfg.H
        rows = p.B * p.H * spade.spade_num_blocks(p)
        assert prev_rows is None or rows < prev_rows
        prev_rows = rows
        ref = spade.estimate_select(qm, km, p, mode, per_head, window=window)
        got = spade.estimate_select_static(qm, km, p, mode, per_head, window=window)
        torch.cuda.synchronize()
        nnz = _same_csr(ref, got)
        assert nnz > 0
        # again into the same output buffers: nothing allocated on the device
        for t in got:
            t.fill_(-7)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        spade.estimate_select_static(qm, km, p, mode, per_head, window=window, out=got)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        _same_csr(ref, got)
        print(f"[no-alloc] {name}: {rows} rows, nnz {nnz}, identical", flush=True)


def test_static_scratch_rejects_oversize_problems():
    cfg = synth.get_config("mid")
    qm = torch.zeros(5, cfg.H, 630, cfg.d, dtype=torch.float32, device="cuda")
    p = spade.Problem(5, cfg.H, cfg.N, cfg.d, cfg.T, cfg.Hh, cfg.W, cfg.bt, cfg.bh, cfg.bw,
                      spade.SPADE_BF16, 0.0)
    with pytest.raises(spade.SpadeError) as e:
        spade.estimate_select_static(qm, qm, p, "ratio", [0.1] * cfg.H)
    assert e.value.status == spade.SPADE_ERR_CAPACITY


def test_static_scratch_under_graph_capture():
    """The use the entry point exists for: recorded into a HIP graph (after
    one eager call has looked up the device's buffer), its replays equal the
    workspace entry point's CSR, with other selections run eagerly between
    them."""
    cfg = synth.get_config("small")
    qm, km, p = _summaries(cfg)
    per_head = cfg.per_head_budget()
    ref = spade.estimate_select(qm, km, p, cfg.mode, per_head)
    rp, ci = spade.estimate_select_static(qm, km, p, cfg.mode, per_head)  # eager, looks up the buffer
    bud = spade.Budget(cfg.mode, per_head)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        spade.spade_estimate_select_static(p, qm, km, bud, rp, ci, ci.numel(), side)
    other_q, other_k, other_p = _summaries(synth.get_config("mid_shape"))
    for rep in range(3):
        rp.fill_(-1)
        ci.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same_csr(ref, (rp, ci))
        # another problem through the same static buffer, eagerly
        spade.estimate_select_static(other_q, other_k, other_p, "count", [3] * other_p.H)
        torch.cuda.synchronize()
