"""Parity of the bf16 (mixed-precision) kernels and training step against the fp64 oracle.

The oracle is unchanged (fp64); it is fed exactly the values the GPU sees: inputs are drawn,
rounded to bf16 on the host (torch's CPU conversion, round to nearest even), and the
rounded values are what both sides consume. Tolerances come from the arithmetic:
- a bf16 result is its fp32 value rounded once, |err| <= 2^-9 |x|; the tests allow
  2^-8 |o| for that, on top of the fp32 accumulation term of ``assert_close_mag``;
- fp32 results computed from bf16 inputs (LayerNorm statistics and dx, losses, gradients
  accumulated in fp32) keep the fp32 tolerances;
- whole steps: the loss within 2e-2 relative; logits and gradients by their normwise
  relative error (bf16 keeps 8 significant bits, so every stored activation and weight
  carries up to 2^-9 relative error and these add up over the layers).
"""
import concurrent.futures as cf
import math

import numpy as np
import pytest

import oracle
from decoder_only_transformer_05_amd import synth
from parity import assert_close, assert_close_mag

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from decoder_only_transformer_05_amd import binding as gb  # noqa: E402

BF = 2.0 ** -8  # allowance for one rounding to bf16 (unit roundoff 2^-9, doubled)


def rng(seed):
    return np.random.default_rng(seed)


def bf16_values(a):
    """The bf16 numbers nearest to a (round to nearest even), as float64."""
    t = torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def dev_bf16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is None:
        dtype = torch.int32 if a.dtype.kind in "iu" else torch.float32
    return torch.tensor(a, dtype=dtype, device="cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------------------
# GEMM: C = op(A) op(B) with every storage pattern and epilogue, ragged tiles, split K
# ---------------------------------------------------------------------------------------
CASES = [
    # (M, N, K, a_trans, b_trans)
    (300, 200, 96, 0, 0), (130, 136, 100, 0, 0), (64, 50257, 64, 0, 0),  # forward (NT)
    (300, 96, 200, 0, 1), (64, 80, 50257, 0, 1), (128, 128, 4096, 0, 1),  # grad input (NN)
    (200, 96, 300, 1, 1), (50257, 64, 64, 1, 1), (128, 256, 8192, 1, 1),  # grad weight (TN)
    (136, 72, 130, 1, 0),
    # more tiles than CUs (both tile shapes), with ragged edges
    (4100, 4104, 136, 0, 0), (4100, 4104, 200, 0, 1), (4104, 4100, 72, 1, 1),
    # 1280 output columns (the 774M model's width): seven 192-wide tiles, the last one ragged
    (1000, 1280, 520, 0, 0), (1000, 1280, 520, 0, 1),
    # 5120 output columns (the 774M MLP width): sixteen 320-wide tiles
    (600, 5120, 264, 0, 0), (600, 5120, 264, 0, 1),
]


def stored(op, trans, ld_pad=0):
    """Storage of op (rows, K): row-major (rows, K) or transposed (K, rows), with the
    leading dimension padded up to a multiple of 8 (+ ld_pad)."""
    a = op.T if trans else op
    r, c = a.shape
    ld = (c + 7) // 8 * 8 + ld_pad
    buf = np.zeros((r, ld), np.float64)
    buf[:, :c] = a
    return buf, ld


@pytest.mark.parametrize("tile", ["1", "2", "3", "4"])
@pytest.mark.parametrize("M,N,K,at,bt", CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_gemm_bf16(M, N, K, at, bt, epi, tile, monkeypatch):
    """Every tile shape of the bf16 GEMM: 128 x 128 tiles with 32-deep K slabs, 256 x 256,
    256 x 192 and 256 x 320 tiles with 64-deep slabs (the library picks one per shape; the
    environment variable pins it; the 256 x 320 tile takes no epilogue that reads a tensor,
    so pinned to it those epilogues run split or on 128 x 128 tiles)."""
    monkeypatch.setenv("GPT2_GEMM_BF16_TILE", tile)
    if K > 1000 and epi in (1, 2):
        pytest.skip("long-K shapes run with the epilogues the step uses with them")
    if at and epi in (1, 2) and M * N > 4_000_000:
        pytest.skip("weight-gradient shapes run with the epilogues the step uses with them")
    r = rng(M + 3 * N + 7 * K + 11 * epi + 13 * at + 17 * bt)
    opA = bf16_values(r.normal(size=(M, K)))
    opB = bf16_values(r.normal(0, 0.05, (N, K)))   # op(B)^T as (N, K)
    A, lda = stored(opA, at)
    B, ldb = stored(opB, bt)  # b_trans = 0: stored (N, K); 1: stored (K, N)
    ldc = (N + 7) // 8 * 8
    bias = r.normal(size=N).astype(np.float32) if epi in (0, 1, 2) else None
    ref = oracle.matmul_forward(opA, opB, bias)
    mag = oracle.matmul_forward(np.abs(opA), np.abs(opB), None if bias is None else np.abs(bias))
    Rv = None
    if epi == 2:
        Rv = bf16_values(r.normal(size=(M, N)))
    if epi == 4:
        Rv = bf16_values(r.normal(0, 2, (M, N)))
    Rbuf = None
    if Rv is not None:
        Rbuf = np.zeros((M, ldc))
        Rbuf[:, :N] = Rv
    colsum = None
    if epi == 3:
        C0 = r.normal(size=(M, ldc)).astype(np.float32)
        C = dev(C0)
        if at:
            cs0 = r.normal(size=M).astype(np.float32)
            colsum = dev(cs0)
    else:
        C = torch.full((M, ldc), float("nan"), device="cuda").to(torch.bfloat16)
    C2 = torch.zeros((M, ldc), device="cuda").to(torch.bfloat16) if epi == 1 else None
    gb.k_gemm_bf16(C, dev_bf16(A), dev_bf16(B), M, N, K, lda, ldb, ldc, at, bt, epi,
                   bias=None if bias is None else dev(bias), C2=C2,
                   R=None if Rbuf is None else dev_bf16(Rbuf), colsum=colsum)
    got = host(C)[:, :N]
    if epi == 0:
        assert_close_mag("gemm_bf16 store", got, ref, mag, K, rtol=BF)
    elif epi == 1:
        assert_close_mag("gemm_bf16 gelu pre", got, ref, mag, K, rtol=BF)
        assert_close_mag("gemm_bf16 gelu", host(C2)[:, :N], oracle.gelu_forward(ref), 1.13 * mag,
                         K, rtol=BF)
    elif epi == 2:
        assert_close_mag("gemm_bf16 resid", got, ref + Rv, mag + np.abs(Rv), K, rtol=BF)
    elif epi == 3:
        assert_close_mag("gemm_bf16 accum", got, C0[:, :N] + ref, np.abs(C0[:, :N]) + mag, K,
                         rtol=1e-6)
        if colsum is not None:
            rcs = opA.sum(axis=1)
            assert_close_mag("gemm_bf16 colsum", host(colsum), cs0 + rcs,
                             np.abs(cs0) + np.abs(opA).sum(axis=1), K, rtol=1e-6)
    else:
        rg = oracle.gelu_backward(Rv, ref)
        mg = np.abs(oracle.gelu_backward(Rv, mag))
        assert_close_mag("gemm_bf16 gelu bwd", got, rg, mg, K, rtol=BF)


# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,C", [(300, 768), (64, 16), (77, 100), (33, 1280)])
def test_layernorm_bf16(N, C):
    r = rng(N + C + 1)
    x = bf16_values(r.normal(0.5, 3.0, (N, C)))
    w, b = r.normal(1, 0.3, C).astype(np.float32), r.normal(0, 0.3, C).astype(np.float32)
    out = torch.empty((N, C), device="cuda").to(torch.bfloat16)
    mean = torch.empty(N, device="cuda")
    rstd = torch.empty(N, device="cuda")
    gb.k_layernorm_forward_bf16(out, mean, rstd, dev_bf16(x), dev(w), dev(b), N, C)
    ro, rm, rr = oracle.layernorm_forward(x, w, b)
    assert_close("ln out", host(out), ro, rtol=BF, atol=1e-5)
    assert_close("ln mean", host(mean), rm)
    assert_close("ln rstd", host(rstd), rr)
    dy = bf16_values(r.normal(size=(N, C)))
    dx0 = r.normal(size=(N, C)).astype(np.float32)
    dw0, db0 = r.normal(size=C).astype(np.float32), r.normal(size=C).astype(np.float32)
    dx, dw, db = dev(dx0), dev(dw0), dev(db0)
    dxc = torch.empty((N, C), device="cuda").to(torch.bfloat16)
    gb.k_layernorm_backward_bf16(dx, dxc, dw, db, dev_bf16(dy), dev_bf16(x), dev(w), mean, rstd,
                                 N, C)
    rdx, rdw, rdb = oracle.layernorm_backward(dy, x, w, rm, rr)
    gdx = host(dx)
    assert_close("ln dx", gdx, dx0 + rdx)
    # dw, db are N-term column sums added to the existing values: fp32 bound on their
    # magnitude sums (n = normalised x)
    nrm = (x - rm[:, None]) * rr[:, None]
    assert_close_mag("ln dw", host(dw), dw0 + rdw, np.abs(dw0) + np.abs(nrm * dy).sum(0), N)
    assert_close_mag("ln db", host(db), db0 + rdb, np.abs(db0) + np.abs(dy).sum(0), N)
    assert np.array_equal(host(dxc), bf16_values(gdx))  # the copy is dx rounded once


@pytest.mark.parametrize("B,T,C,NH", [(2, 100, 128, 2), (4, 16, 16, 4), (2, 64, 768, 12),
                                      (1, 1, 64, 1), (3, 257, 64, 1), (2, 130, 48, 2),
                                      (1, 200, 256, 2), (2, 77, 96, 3), (1, 1024, 1280, 20)])
def test_attention_bf16(B, T, C, NH):
    r = rng(B * T + C + NH + 5)
    qkv = bf16_values(r.normal(0, 1.0, (B, T, 3 * C)))
    dy = bf16_values(r.normal(size=(B, T, C)))
    out = torch.full((B, T, C), float("nan"), device="cuda").to(torch.bfloat16)
    lse = torch.empty((B, NH, T), device="cuda")
    gb.k_attention_forward_bf16(out, lse, dev_bf16(qkv), B, T, C, NH)
    ro, ratt = oracle.attention_forward(qkv, NH)
    qabs = qkv.copy()
    qabs[:, :, 2 * C:] = np.abs(qabs[:, :, 2 * C:])
    mag, _ = oracle.attention_forward(qabs, NH)
    # with a head size that is a multiple of 8 the product P V takes P rounded to bf16 (as
    # an MFMA operand): that changes out by up to 2^-9 sum_k P|v| = 2^-9 mag; the bound
    # allows twice that, like the BF allowance for a rounded result
    hs = C // NH
    assert_close_mag("attn out", host(out), ro, mag, T + hs, rtol=BF,
                     operand_u=BF if hs % 8 == 0 else 0.0)
    dqkv = torch.full((B, T, 3 * C), float("nan"), device="cuda").to(torch.bfloat16)
    gb.k_attention_backward_bf16(dqkv, dev_bf16(dy), dev_bf16(qkv), out, lse, B, T, C, NH)
    rd = oracle.attention_backward(dy, qkv, ratt, NH)
    # the kernel forms rowsum(dO * O) from its own bf16 O (within 2^-9 of the exact O), so
    # besides the final rounding dS carries a relative error of that order: the bound is
    # 2^-7 relative plus 2^-8 of the tensor's scale
    scale = np.abs(rd).max()
    assert_close_mag("attn dqkv", host(dqkv), rd, np.full(rd.shape, scale), T, rtol=2 * BF,
                     atol=BF * scale)


@pytest.mark.parametrize("N,V,ld", [(37, 50257, 50304), (64, 27, 28)])
def test_crossentropy_bf16(N, V, ld):
    r = rng(N + V + 9)
    z = np.zeros((N, ld))
    z[:, :V] = bf16_values(r.normal(0, 2.0, (N, V)))
    z[:, V:] = 123.0  # padding must be ignored
    y = r.integers(0, V, N).astype(np.int32)
    logits = dev_bf16(z)
    losses = torch.empty(N, device="cuda")
    lse = torch.empty(N, device="cuda")
    gb.k_crossentropy_forward_bf16(losses, lse, logits, dev(y), N, V, ld)
    rl = oracle.crossentropy_forward(z[:, :V], y)
    assert_close("xent loss", host(losses), rl, rtol=1e-5, atol=1e-6)
    dloss = 1.0 / N
    gb.k_crossentropy_backward_bf16(logits, lse, dev(y), dloss, N, V, ld)
    rg = oracle.crossentropy_softmax_backward(z[:, :V], y, np.full(N, dloss))
    g = host(logits)
    assert_close("xent dlogits", g[:, :V], rg, rtol=BF, atol=1e-9)
    assert np.all(g[:, V:] == 0.0)


def test_encoder_cast_adamw_bf16_rounding():
    """Rounding-only kernels: bitwise equal to fp32 arithmetic then round-to-nearest-even."""
    r = rng(77)
    B, T, C, V = 3, 50, 64, 1000
    wte = r.normal(0, 0.5, (V, C)).astype(np.float32)
    wpe = r.normal(0, 0.5, (T, C)).astype(np.float32)
    tok = r.integers(0, V, (B, T)).astype(np.int32)
    out = torch.empty((B, T, C), device="cuda").to(torch.bfloat16)
    gb.k_encoder_forward_bf16(out, dev(tok), dev(wte), dev(wpe), B, T, C, V)
    want = (torch.tensor(wte)[torch.tensor(tok).long()] + torch.tensor(wpe)[None]).to(torch.bfloat16)
    assert torch.equal(out.cpu(), want)

    n = 10_001
    x = r.normal(0, 3, n).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact ties round to even
    dst = torch.empty(n, device="cuda").to(torch.bfloat16)
    gb.k_cast_bf16(dst, dev(x), n)
    assert torch.equal(dst.cpu(), torch.tensor(x).to(torch.bfloat16))

    p0 = r.normal(0, 0.1, n).astype(np.float32)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    p, m, v = dev(p0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    pb = torch.empty(n, device="cuda").to(torch.bfloat16)
    gb.k_adamw_bf16(p, pb, dev(g), m, v, n, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    assert torch.equal(pb.cpu(), p.cpu().to(torch.bfloat16))
    rp, _, _ = oracle.adamw(p0, g, np.zeros(n), np.zeros(n), 1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
    assert np.abs(host(p) - rp).max() <= 1e-6


# ---------------------------------------------------------------------------------------
# whole steps in GPT2_DTYPE_BF16
# ---------------------------------------------------------------------------------------
from model_harness import (HP, check_losses_and_logits_row, compare_grads_bf16,  # noqa: E402
                           oracle_batch, progress)
from parity import assert_bf16_close  # noqa: E402

LOSS_RTOL_BF16 = 2e-2


def bf16_steps(shape, seed, B, T, steps, mode, scale_residual, grad_r):
    """Each step is compared from the GPU's own fp32 master parameters, so it measures that
    step's bf16 arithmetic alone; logits and every gradient tensor pass the bf16 gate
    (normwise and per entry against the oracle's envelope)."""
    p0 = synth.init_params(shape, seed, scale_residual)
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, dtype="bf16")
    m.set_params(p0)
    rm, rv = np.zeros(p0.size), np.zeros(p0.size)
    for step in range(steps):
        tok, tgt = synth.batch(seed, B, T, shape.V, step=step, mode=mode)
        m.zero_grad()
        loss = m.forward(dev(tok), dev(tgt))
        logits = np.empty((B, T, shape.V), np.float32)
        m.get_logits(logits)
        m.backward()
        grads = m.get_grads()
        got_p = m.get_params()
        m.adamw_step(t=step + 1, **HP)
        ref = oracle.gpt2_step(shape, got_p.astype(np.float64), tok, tgt, want_logits=True,
                               want_mags=True)
        rel = abs(loss - ref["loss"]) / abs(ref["loss"])
        s = assert_bf16_close("logits", logits, ref["logits"], ref["logit_mag"], 2e-2)
        print(f"step {step}: loss {loss:.6f} oracle {ref['loss']:.6f} rel {rel:.2e} "
              f"logits {s}")
        assert rel <= LOSS_RTOL_BF16
        compare_grads_bf16(shape, grads, ref["grads"], ref["grad_mag"], grad_r)
        # AdamW on the GPU's own gradients, checked against the oracle's rule
        rp, rm, rv = oracle.adamw(got_p.astype(np.float64), grads, rm, rv, HP["lr"], HP["beta1"],
                                  HP["beta2"], HP["eps"], HP["weight_decay"], step + 1)
        assert np.abs(m.get_params() - rp).max() <= 1e-6
    m.close()


def test_bf16_tiny_three_steps():
    w = synth.WORKLOADS["tiny"]
    bf16_steps(w.shape, w.seed, w.B, w.T, 3, w.token_mode, w.scale_residual, 5e-2)


def test_bf16_small_multilayer_ragged_two_steps():
    shape = synth.ModelShape(L=2, C=64, H=4, V=1000, maxT=128)
    bf16_steps(shape, 4243, 3, 100, 2, "stream", True, 5e-2)


@pytest.mark.timeout(600)
def test_bf16_774m_b8_t1024_full_rows_and_properties():
    """The 774M bf16 workload in the benchmark's launch configuration: two full T=1024 rows
    (per-position losses and logits) against single-row oracle forwards, the mean loss
    near its value at init, bitwise determinism and a finite step."""
    w = synth.WORKLOADS["gpt2_774m_b8_t1024_bf16"]
    shape = w.shape
    B, T, V = w.B, w.T, shape.V
    p0 = synth.init_params(shape, w.seed, w.scale_residual)
    tok, tgt = synth.batch(w.seed, B, T, V, mode=w.token_mode)
    rows = [0, 7]
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, B, T, dtype="bf16")
    m.set_params(p0)
    m.zero_grad()
    loss = m.forward(dev(tok), dev(tgt))
    losses = torch.empty((B, T), device="cuda")
    m.get_losses(losses)
    got_losses = losses[rows].cpu().numpy()
    logits = torch.empty((B, T, V), device="cuda")
    m.get_logits(logits)
    got_logits = logits[rows].cpu().numpy()
    del logits
    m.backward()
    g1 = torch.empty(m.num_params, device="cuda")
    m.get_grads(g1)
    m.zero_grad()
    assert m.forward(dev(tok), dev(tgt)) == loss  # deterministic
    m.backward()
    g2 = torch.empty(m.num_params, device="cuda")
    m.get_grads(g2)
    assert torch.equal(g1, g2)
    assert bool(torch.isfinite(g1).all())
    del g1, g2
    m.adamw_step(t=1, **HP)
    assert np.isfinite(m.get_params()).all()
    m.close()

    ref = oracle_batch(shape, p0.astype(np.float64), tok[rows], tgt[rows], want_logits=True,
                       want_grads=False, label="774M bf16 rows",
                       row_hook=lambda i, r: check_losses_and_logits_row(
                           rows[i], got_logits[i], r, shape.C, label="774M bf16:", bf16=2e-2))
    rel = np.abs(got_losses - ref["losses"]) / np.abs(ref["losses"])
    progress(f"774M bf16 rows {rows}: per-position loss rel error max {rel.max():.2e} mean "
             f"{rel.mean():.2e}")
    assert rel.max() <= LOSS_RTOL_BF16
    expect = math.log(V) + shape.C * 0.02 ** 2 / 2
    assert abs(loss - expect) < 0.05, (loss, expect)


@pytest.mark.timeout(600)
def test_bf16_774m_b1_t32_gradients():
    """Every parameter gradient of one B1 T32 step of the 774M shape against the oracle."""
    w = synth.WORKLOADS["gpt2_774m_b8_t1024_bf16"]
    shape = w.shape
    p0 = synth.init_params(shape, w.seed, w.scale_residual)
    tok, tgt = synth.batch(w.seed, 1, 32, shape.V, mode=w.token_mode)
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, dtype="bf16")
    m.set_params(p0)
    m.zero_grad()
    loss = m.forward(dev(tok), dev(tgt))
    m.backward()
    grads = m.get_grads()
    m.close()
    ref = oracle.gpt2_step(shape, p0.astype(np.float64), tok, tgt, want_mags=True)
    rel = abs(loss - ref["loss"]) / abs(ref["loss"])
    print(f"loss {loss:.6f} oracle {ref['loss']:.6f} rel {rel:.2e}")
    assert rel <= LOSS_RTOL_BF16
    compare_grads_bf16(shape, grads, ref["grads"], ref["grad_mag"], 5e-2, label="774M B1 T32")
