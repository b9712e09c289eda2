"""Replays of a captured HIP graph of the fused call match eager calls on the same inputs.

A captured graph freezes every kernel argument. The row-team kernel's cross-workgroup exchange
flags therefore come from the workspace, advanced on the device by each launch, so that a replay
never takes units an earlier replay left behind for its own team members' values. The inputs change
between replays (the same buffers, new contents) and eager calls and a sampling verification, which
writes its slice sums over the exchange units, run in between.
"""

import pytest

pytestmark = pytest.mark.gpu

ROWS, VOCAB = 304, 151936  # 19 blocks of 16; four row iterations per team at 85 teams


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _inputs(seed):
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    base = torch.randn(ROWS, VOCAB, device="cuda", generator=g) * 3.0
    z = (base + torch.randn(ROWS, VOCAB, device="cuda", generator=g) * 1.5).to(torch.bfloat16)
    y = base.to(torch.bfloat16)
    return z, y


def _outputs(m, like_z):
    import torch

    return {
        "loss": torch.empty(ROWS, dtype=torch.float32, device="cuda"),
        "target_top1": torch.empty(ROWS, dtype=torch.int32, device="cuda"),
        "draft_top1": torch.empty(ROWS, dtype=torch.int32, device="cuda"),
        "row_stats": torch.empty(ROWS, 8, dtype=torch.float32, device="cuda"),
        "dz": torch.empty_like(like_z),
        "accept_len": torch.empty(ROWS // 16, dtype=torch.int32, device="cuda"),
    }


def test_graph_replays_match_eager(lib):
    import torch

    m = lib
    off = torch.arange(0, ROWS + 1, 16, dtype=torch.int32, device="cuda")
    lens = torch.full((ROWS // 16,), 16, dtype=torch.int32, device="cuda")
    alpha, tau = 0.5, 0.05
    inputs = [_inputs(s) for s in (11, 12, 13)]
    _say("eager references")
    ref = [m.opd_fused_fwd_bwd_verify(z, y, off, lens, alpha, tau) for z, y in inputs]
    torch.cuda.synchronize()
    assert m.read_flags(clear=True) == 0

    zs, ys = torch.empty_like(inputs[0][0]), torch.empty_like(inputs[0][1])
    zs.copy_(inputs[0][0])
    ys.copy_(inputs[0][1])
    out = _outputs(m, zs)
    m.opd_fused_fwd_bwd_verify(zs, ys, off, lens, alpha, tau, out=out)  # warm-up outside the capture
    torch.cuda.synchronize()

    _say("capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.opd_fused_fwd_bwd_verify(zs, ys, off, lens, alpha, tau, out=out)
    torch.cuda.synchronize()

    draft = torch.zeros(ROWS, dtype=torch.int32, device="cuda")
    u_acc = torch.full((ROWS,), 0.5, dtype=torch.float32, device="cuda")
    u_res = torch.full((ROWS // 16,), 0.5, dtype=torch.float32, device="cuda")
    for step, idx in enumerate([1, 0, 2, 2, 1, 0]):
        zs.copy_(inputs[idx][0])
        ys.copy_(inputs[idx][1])
        graph.replay()
        torch.cuda.synchronize()
        _say(f"replay {step} on inputs {idx}")
        for k, v in ref[idx].items():
            assert torch.equal(out[k], v), (step, idx, k)
        # eager work between replays: a fused call on other inputs, and (every other step) a sampling
        # verification whose slice sums overwrite the exchange units
        other = inputs[(idx + 1) % 3]
        e = m.opd_fused_fwd_bwd_verify(other[0], other[1], off, lens, alpha, tau)
        if step % 2 == 0:
            m.verify_sample(other[0], other[1], off, lens, draft, u_acc, u_res, 1.0)
        torch.cuda.synchronize()
        for k, v in ref[(idx + 1) % 3].items():
            assert torch.equal(e[k], v), (step, "eager", k)
    assert m.read_flags(clear=True) == 0


def test_graph_of_separate_calls_replays_match_eager(lib):
    """Forward, backward from its row statistics and verification, captured together in one graph."""
    import torch

    m = lib
    off = torch.arange(0, ROWS + 1, 16, dtype=torch.int32, device="cuda")
    lens = torch.full((ROWS // 16,), 9, dtype=torch.int32, device="cuda")
    alpha, tau = 0.7, 0.02
    inputs = [_inputs(s) for s in (21, 22)]

    def eager(z, y):
        loss, a, d, stats = m.opd_loss_fwd(z, y, alpha, tau)
        dz = m.opd_loss_bwd(z, y, alpha, tau, stats, a)
        a2, d2, acc = m.verify_accept_len(z, y, off, lens)
        return {"loss": loss, "a": a, "d": d, "stats": stats, "dz": dz, "a2": a2, "d2": d2, "acc": acc}

    _say("separate calls: eager references")
    ref = [eager(z, y) for z, y in inputs]
    torch.cuda.synchronize()
    assert m.read_flags(clear=True) == 0

    zs, ys = torch.empty_like(inputs[0][0]), torch.empty_like(inputs[0][1])
    zs.copy_(inputs[0][0])
    ys.copy_(inputs[0][1])
    eager(zs, ys)  # warm-up outside the capture
    torch.cuda.synchronize()
    _say("separate calls: capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = eager(zs, ys)
    torch.cuda.synchronize()
    for step, idx in enumerate([1, 0, 0, 1]):
        zs.copy_(inputs[idx][0])
        ys.copy_(inputs[idx][1])
        graph.replay()
        torch.cuda.synchronize()
        _say(f"separate calls: replay {step} on inputs {idx}")
        for k, v in ref[idx].items():
            assert torch.equal(out[k], v), (step, idx, k)
        e = eager(*inputs[1 - idx])
        torch.cuda.synchronize()
        for k, v in ref[1 - idx].items():
            assert torch.equal(e[k], v), (step, "eager", k)
    assert m.read_flags(clear=True) == 0


def test_graph_replays_across_the_epoch_wrap(lib):
    """The epoch of a fresh workspace set just below 2^31 - 1: replays run across the point where the
    range restarts from 1, and every replay still matches the eager result."""
    import torch

    m = lib
    rows = 96  # two row iterations per team at 85 teams: six flags per launch
    off = torch.arange(0, rows + 1, 16, dtype=torch.int32, device="cuda")
    lens = torch.full((rows // 16,), 16, dtype=torch.int32, device="cuda")
    alpha, tau = 0.5, 0.05
    g = torch.Generator(device="cuda").manual_seed(31)
    base = torch.randn(rows, VOCAB, device="cuda", generator=g) * 3.0
    z = (base + torch.randn(rows, VOCAB, device="cuda", generator=g) * 1.5).to(torch.bfloat16)
    y = base.to(torch.bfloat16)
    ws = torch.zeros(m.load_library().opd_workspace_size(), dtype=torch.uint8, device="cuda")
    ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, alpha, tau, ws=ws)
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    m.opd_fused_fwd_bwd_verify(z, y, off, lens, alpha, tau, ws=ws, out=out)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.opd_fused_fwd_bwd_verify(z, y, off, lens, alpha, tau, ws=ws, out=out)
    torch.cuda.synchronize()
    ws.zero_()  # a fresh workspace whose epoch is 24 below the end of its range
    ws.view(torch.int32)[16] = 0x7FFFFFFF - 24
    torch.cuda.synchronize()
    for step in range(12):
        for v in out.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (step, k)
    epoch = int(ws.view(torch.int32)[16].item())
    _say(f"epoch after the replays: {epoch}")
    assert 0 < epoch < 0x7FFFFFFF - 24  # the range restarted during the replays
    assert m.read_flags(ws, clear=True) == 0
