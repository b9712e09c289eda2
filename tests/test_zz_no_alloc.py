"""The no-allocation entry point (opd_fused_fwd_bwd_verify_noalloc) against the regular fused call,
through the C ABI: two calls in a row on the library's own workspace array, the second with a
smaller input, each bit-identical to opd_fused_fwd_bwd_verify on a caller workspace (same kernels,
so the results must agree exactly). Runs alone in a fresh process or after the other tests."""

import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _case(rows, vocab, seed, dtype):
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    base = torch.randn(rows, vocab, device="cuda", generator=g) * 3.0
    z = (base + torch.randn(rows, vocab, device="cuda", generator=g) * 1.5).to(dtype)
    y = base.to(dtype)
    nb = max(1, rows // 16)
    off = torch.linspace(0, rows, nb + 1, device="cuda").round().to(torch.int32)
    lens = torch.randint(0, 17, (nb,), generator=g, device="cuda", dtype=torch.int32)
    w = torch.rand(rows, generator=g, device="cuda") + 0.5
    return z, y, off, lens, w


def _outputs(ref):
    """Fresh outputs with the layout (sizes and strides) of the regular call's, filled with 7."""
    import torch

    out = {}
    for k, v in ref.items():
        t = torch.empty_strided(v.size(), v.stride(), dtype=v.dtype, device=v.device)
        t.fill_(7)
        out[k] = t
    return out


@pytest.mark.parametrize("dz_dtype", ["bf16", "f32"])
def test_no_alloc_matches_the_regular_call_twice(lib, dz_dtype):
    import torch

    m = lib
    dzt = torch.bfloat16 if dz_dtype == "bf16" else torch.float32
    cases = [(1100, 151936, 1, torch.bfloat16), (37, 40004, 2, torch.float32)]  # the second is smaller
    for i, (rows, vocab, seed, dt) in enumerate(cases):
        z, y, off, lens, w = _case(rows, vocab, seed, dt)
        _say(f"call {i}: rows={rows} V={vocab} in={dt} dz={dz_dtype}")
        ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.6, 0.03, grad_loss=w, dz_dtype=dzt)
        out = _outputs(ref)
        res = m.opd_fused_fwd_bwd_verify_noalloc(z, y, off, lens, 0.6, 0.03, out=out, grad_loss=w)
        torch.cuda.synchronize()
        assert res is out
        assert m.read_flags(clear=True) == 0
        for k, v in ref.items():
            assert torch.equal(out[k], v), (i, k)
    # check mode reads the library array's flag word: a clean call raises nothing
    m.set_check(True)
    try:
        z, y, off, lens, w = _case(64, 4096, 3, torch.bfloat16)
        ref = m.opd_fused_fwd_bwd_verify(z, y, off, lens, 0.5, 0.05, dz_dtype=dzt)
        out = _outputs(ref)
        m.opd_fused_fwd_bwd_verify_noalloc(z, y, off, lens, 0.5, 0.05, out=out)
        for k, v in ref.items():
            assert torch.equal(out[k], v), ("check mode", k)
    finally:
        m.set_check(False)
