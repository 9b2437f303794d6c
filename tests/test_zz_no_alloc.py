"""The allocation-free matmul backward (gpt2_k_matmul_backward_noalloc) against the
allocating entry point on the same inputs: two calls in a row, the second smaller, then the
first again over the scratch the others left behind; both use the same kernels and plans,
so the results must be bitwise equal. A problem whose plan needs more scratch than the
static array holds is refused before anything runs."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from decoder_only_transformer_05_amd import binding as gb  # noqa: E402


def _problem(seed, N, C, OC, gelu):
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = {
        "dout": torch.randn(N, OC, generator=g) * 0.1,
        "inp": torch.randn(N, C, generator=g),
        "W": torch.randn(OC, C, generator=g) * 0.02,
        "gelu_pre": torch.randn(N, C, generator=g) if gelu else None,
        "dW0": torch.randn(OC, C, generator=g) * 1e-3,
        "db0": torch.randn(OC, generator=g) * 1e-3,
    }
    return {k: (v.cuda() if v is not None else None) for k, v in t.items()}


def _run(fn, p, N, C, OC):
    dinp = torch.full((N, C), float("nan"), device="cuda")
    dW = p["dW0"].clone()
    db = p["db0"].clone()
    fn(dinp, dW, db, p["dout"], p["inp"], p["W"], N, C, OC, gelu_pre=p["gelu_pre"])
    torch.cuda.synchronize()
    return dinp.cpu(), dW.cpu(), db.cpu()


@pytest.mark.parametrize("first,second", [
    ((16384, 768, 768, True), (256, 768, 2304, False)),
    ((16384, 3072, 768, False), (100, 64, 200, True)),
])
def test_noalloc_matches_allocating_entry(first, second):
    runs = [first, second, first]
    for i, (N, C, OC, gelu) in enumerate(runs):
        print(f"noalloc call {i}: N={N} C={C} OC={OC} gelu={gelu}", flush=True)
        p = _problem(100 + i, N, C, OC, gelu)
        want = _run(gb.k_matmul_backward, p, N, C, OC)
        got = _run(gb.k_matmul_backward_noalloc, p, N, C, OC)
        for name, a, b in zip(("dinp", "dW", "dbias"), got, want):
            assert torch.isfinite(a).all(), name
            assert torch.equal(a, b), f"call {i} {name}: max diff {(a - b).abs().max().item()}"


def test_noalloc_refuses_a_plan_above_its_scratch():
    N, C, OC = 16384, 768, 50257  # the tied lm_head weight gradient of GPT-2 124M, B16 T1024
    dout = torch.zeros(N, OC, device="cuda")
    inp = torch.zeros(N, C, device="cuda")
    dW = torch.zeros(OC, C, device="cuda")
    with pytest.raises(gb.GPT2Error) as e:
        gb.k_matmul_backward_noalloc(None, dW, None, dout, inp, None, N, C, OC)
    assert e.value.code == -1 and "scratch" in str(e.value)
    assert float(dW.abs().max()) == 0.0
