"""GPU tests of the row-team kernel's shared state and failure reporting:

* calls on two streams at once (each stream has its own default workspace) match serial results;
* check mode turns device flags into errors raised by the call itself;
* the forward and top-1 modes over many row iterations (exchange 1 alternates between two stages by
  row parity, so that a member that moves on cannot overwrite a value a slower member still needs);
* the restart of the host's exchange-flag range and of the device epoch: units left from the range
  that ended, planted here with flags the next range hands out again, are zeroed before they could
  be taken for fresh ones.
"""

import numpy as np
import pytest

import synth
from oracle import opd_oracle as O

pytestmark = pytest.mark.gpu

VOCAB = 151936


def _say(msg):
    print(f"[gpu-robust] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _inputs(rows, seed, vocab=VOCAB, dtype="bf16"):
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    base = torch.randn(rows, vocab, device="cuda", generator=g) * 3.0
    z = base + torch.randn(rows, vocab, device="cuda", generator=g) * 1.5
    y = base
    if dtype == "bf16":
        return z.to(torch.bfloat16), y.to(torch.bfloat16)
    return z.contiguous(), y.contiguous()


def _blocks(rows, L=12):
    import torch

    off = torch.arange(0, rows + 1, 16, dtype=torch.int32, device="cuda")
    lens = torch.full((rows // 16,), L, dtype=torch.int32, device="cuda")
    return off, lens


def test_two_streams_at_once_match_serial(lib):
    """Fused calls on two torch streams at once, each stream with its own default workspace, give
    the bits of the same calls made one after the other."""
    import torch

    m = lib
    rows = 512
    (z1, y1), (z2, y2) = _inputs(rows, 1), _inputs(rows, 2)
    off, lens = _blocks(rows)
    _say("serial references")
    r1 = m.opd_fused_fwd_bwd_verify(z1, y1, off, lens, 0.5, 0.05)
    r2 = m.opd_fused_fwd_bwd_verify(z2, y2, off, lens, 0.5, 0.05)
    torch.cuda.synchronize()
    assert m.read_flags(clear=True) == 0
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    _say("two streams, 4 rounds")
    for _ in range(4):
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            o1 = m.opd_fused_fwd_bwd_verify(z1, y1, off, lens, 0.5, 0.05)
        with torch.cuda.stream(s2):
            o2 = m.opd_fused_fwd_bwd_verify(z2, y2, off, lens, 0.5, 0.05)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    ws1, ws2 = m.workspace(stream=s1), m.workspace(stream=s2)
    assert ws1.data_ptr() != ws2.data_ptr() != m.workspace().data_ptr()
    assert m.read_flags(ws1, clear=True) == 0 and m.read_flags(ws2, clear=True) == 0
    for o1, o2 in outs:
        for k in r1:
            assert torch.equal(o1[k], r1[k]), k
            assert torch.equal(o2[k], r2[k]), k


def test_check_mode_raises_on_device_flags(lib):
    import torch

    m = lib
    rows = 64
    z, y = _inputs(rows, 3, vocab=4096)
    off, _ = _blocks(rows)
    neg = torch.tensor([3, -1, 16, 2], dtype=torch.int32, device="cuda")
    bad_off = torch.tensor([0, 16, 8, 48, 64], dtype=torch.int32, device="cuda")
    lens = torch.full((4,), 16, dtype=torch.int32, device="cuda")
    m.read_flags(clear=True)
    m.set_check(True)
    try:
        _say("check mode: negative L")
        with pytest.raises(m.OpdError) as e:
            m.verify_accept_len(z, y, off, neg)
        assert e.value.status == 8 and "negative L" in str(e.value)
        _say("check mode: malformed offsets")
        with pytest.raises(m.OpdError) as e:
            m.opd_fused_fwd_bwd_verify(z, y, bad_off, lens, 0.5, 0.05)
        assert e.value.status == 8 and "malformed offsets" in str(e.value)
        _say("check mode: clean call")
        a, d, acc = m.verify_accept_len(z, y, off, lens)  # flags were cleared: no error
        assert acc.numel() == 4
    finally:
        m.set_check(False)
    assert m.read_flags(clear=True) == 0


@pytest.mark.parametrize("dtype,vocab", [("bf16", 151936), ("f32", 151937)])
def test_forward_and_top1_modes_over_many_iterations(lib, dtype, vocab):
    """opd_loss_fwd and verify_accept_len over enough rows for many row iterations per team (fp32 at
    V=151,937 has 30 members per team, so its gathers take two passes); both must match the fused
    call bit for bit and raise no flag."""
    import torch

    m = lib
    rows = 1200
    ld = vocab + (-vocab) % (8 if dtype == "bf16" else 4)
    zf, yf = _inputs(rows, 5, vocab=vocab, dtype="f32")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    z = torch.zeros(rows, ld, dtype=tdt, device="cuda")[:, :vocab]
    y = torch.zeros(rows, ld, dtype=tdt, device="cuda")[:, :vocab]
    z.copy_(zf)
    y.copy_(yf)
    del zf, yf
    off, lens = _blocks(rows - rows % 16, L=16)
    _say(f"forward / top-1 modes {dtype} V={vocab}")
    ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.6, 0.03)
    for _ in range(3):
        loss, a, d, stats = m.opd_loss_fwd(z, y, 0.6, 0.03)
        a2, d2, acc = m.verify_accept_len(z, y, off, lens)
        torch.cuda.synchronize()
        assert m.read_flags(clear=True) == 0
        assert torch.equal(loss, ref["loss"]) and torch.equal(stats, ref["row_stats"])
        assert torch.equal(a, ref["target_top1"]) and torch.equal(d, ref["draft_top1"])
        assert torch.equal(a2, a) and torch.equal(d2, d) and torch.equal(acc, ref["accept_len"])
    # the top-1s against the oracle's argmax on every row
    zh = z.float().cpu().numpy()
    yh = y.float().cpu().numpy()
    assert np.array_equal(d.cpu().numpy(), O.top1_rows(zh))
    assert np.array_equal(a.cpu().numpy(), O.top1_rows(yh))


def _plant_units(ws, flags):
    """Fill every exchange unit of a workspace with payload 0 and the given flags in turn: stale units
    that a later launch would take for fresh ones if they were not cleared."""
    import torch

    units = ws[256:].view(torch.int64)
    fl = torch.tensor([int(f) for f in flags], dtype=torch.int64, device="cuda")
    idx = torch.arange(units.numel(), device="cuda") % fl.numel()
    units.copy_((fl[idx] << 32).to(torch.int64))


def _nonzero_units(ws) -> int:
    import torch

    return int(torch.count_nonzero(ws[256:].view(torch.int64)).item())


# A launch writes at most 5 units per stage and workgroup, three stages, and never more than 4096
# workgroups; every unit of the workspace holds a planted value before the restart.
MAX_WRITTEN_UNITS = 4096 * 3 * 5


def test_host_flag_range_restart_clears_units(lib):
    import torch

    m = lib
    rows = 256
    z, y = _inputs(rows, 7)
    off, lens = _blocks(rows)
    ws = torch.zeros(m.load_library().opd_workspace_size(), dtype=torch.uint8, device="cuda")
    _say("host range restart: reference")
    ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, ws=ws)  # ws now known to the host
    torch.cuda.synchronize()
    # flags the restarted range hands out first (the eager range starts at 2^31 + 1)
    _plant_units(ws, [0x80000000 + k for k in range(1, 9)])
    n_units = ws[256:].numel() // 8
    assert _nonzero_units(ws) == n_units > MAX_WRITTEN_UNITS
    # use up the range on another address, so that this workspace's next reservation restarts it
    m.debug_reserve_flags(0x1000, 16, next_offset=(1 << 31) - 8)
    _say("host range restart: call after the restart")
    out = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, ws=ws)
    torch.cuda.synchronize()
    assert m.read_flags(ws, clear=True) == 0
    for k in ref:
        assert torch.equal(out[k], ref[k]), k
    # the units were zeroed before the launch: only what it wrote itself is left
    left = _nonzero_units(ws)
    _say(f"non-zero units after the call: {left} of {n_units}")
    assert left <= MAX_WRITTEN_UNITS


def test_device_epoch_restart_clears_units(lib):
    """Graph replays across the device epoch's restart: the launch whose range passes the restart
    point zeroes every unit when it ends (planted stale units included), and the replays after the
    restart match the eager result."""
    import torch

    m = lib
    rows = 96
    z, y = _inputs(rows, 9)
    off, lens = _blocks(rows)
    ws = torch.zeros(m.load_library().opd_workspace_size(), dtype=torch.uint8, device="cuda")
    ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, ws=ws)
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, ws=ws, out=out)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, ws=ws, out=out)
    torch.cuda.synchronize()
    ws.zero_()
    _plant_units(ws, range(1, 9))  # the flags the restarted range hands out first
    ws.view(torch.int32)[16] = 0x40000000 - 3  # the next launch's range passes the restart point
    torch.cuda.synchronize()
    _say("device epoch restart: replays")
    for step in range(6):
        for v in out.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (step, k)
        epoch = int(ws.view(torch.int32)[16].item())
        left = _nonzero_units(ws)
        _say(f"replay {step}: epoch {epoch}, non-zero units {left}")
        if step == 0:
            assert epoch == 0 and left == 0  # restarted, every unit zeroed at the end of the launch
        else:
            assert 0 < epoch < 64 and left <= MAX_WRITTEN_UNITS
    assert m.read_flags(ws, clear=True) == 0
