"""fp16 mixed precision: the GEMM and attention kernels on fp16 MFMA, and whole training
steps in GPT2_DTYPE_FP16 with loss scaling, against the unchanged fp64 oracle.

fp16 keeps 11 significant bits (unit roundoff 2^-11, a quarter of bf16's 2^-9) over a narrow
exponent range (largest finite 65504, normal down to 2^-14). Tolerances follow the bf16
ones scaled by that ratio: a result rounded to fp16 is allowed 2^-10 |o| on top of the fp32
accumulation term; whole steps: loss within 5e-3 relative, logits normwise and per entry
5e-3, parameter gradients 1.25e-2 (the bf16 gates 2e-2 and 5e-2 over four). Gradients are
exchanged unscaled; the loss scale only keeps the fp16 activation gradients above underflow.
"""
import math

import numpy as np
import pytest

import oracle
from decoder_only_transformer_05_amd import synth
from parity import assert_close, assert_close_mag

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from decoder_only_transformer_05_amd import binding as gb  # noqa: E402
from model_harness import (HP, check_losses_and_logits_row, compare_grads_bf16,  # noqa: E402
                           oracle_batch, progress)
from parity import assert_bf16_close  # noqa: E402

F16 = 2.0 ** -10  # allowance for one rounding to fp16 (unit roundoff 2^-11, doubled)
LOSS_RTOL_F16 = 5e-3
LOGITS_R_F16 = 5e-3
GRADS_R_F16 = 1.25e-2


def rng(seed):
    return np.random.default_rng(seed)


def f16_values(a):
    """The fp16 numbers nearest to a (round to nearest even), as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def dev_f16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.float16).cuda()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is None:
        dtype = torch.int32 if a.dtype.kind in "iu" else torch.float32
    return torch.tensor(a, dtype=dtype, device="cuda")


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = [
    (300, 200, 96, 0, 0), (130, 136, 100, 0, 0), (64, 50257, 64, 0, 0),
    (300, 96, 200, 0, 1), (64, 80, 50257, 0, 1), (128, 128, 4096, 0, 1),
    (200, 96, 300, 1, 1), (50257, 64, 64, 1, 1), (128, 256, 8192, 1, 1),
    (136, 72, 130, 1, 0),
    (4100, 4104, 136, 0, 0), (4100, 4104, 200, 0, 1), (4104, 4100, 72, 1, 1),
]


def stored(op, trans):
    a = op.T if trans else op
    r, c = a.shape
    ld = (c + 7) // 8 * 8
    buf = np.zeros((r, ld), np.float64)
    buf[:, :c] = a
    return buf, ld


@pytest.mark.parametrize("tile", ["1", "2", "3", "4"])
@pytest.mark.parametrize("M,N,K,at,bt", CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_gemm_f16(M, N, K, at, bt, epi, tile, monkeypatch):
    monkeypatch.setenv("GPT2_GEMM_BF16_TILE", tile)
    if K > 1000 and epi in (1, 2):
        pytest.skip("long-K shapes run with the epilogues the step uses with them")
    if at and epi in (1, 2) and M * N > 4_000_000:
        pytest.skip("weight-gradient shapes run with the epilogues the step uses with them")
    r = rng(M + 3 * N + 7 * K + 11 * epi + 13 * at + 17 * bt + 1)
    opA = f16_values(r.normal(size=(M, K)))
    opB = f16_values(r.normal(0, 0.05, (N, K)))
    A, lda = stored(opA, at)
    B, ldb = stored(opB, bt)
    ldc = (N + 7) // 8 * 8
    bias = r.normal(size=N).astype(np.float32) if epi in (0, 1, 2) else None
    ref = oracle.matmul_forward(opA, opB, bias)
    mag = oracle.matmul_forward(np.abs(opA), np.abs(opB), None if bias is None else np.abs(bias))
    Rv = None
    if epi == 2:
        Rv = f16_values(r.normal(size=(M, N)))
    if epi == 4:
        Rv = f16_values(r.normal(0, 2, (M, N)))
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
        C = torch.full((M, ldc), float("nan"), device="cuda").to(torch.float16)
    C2 = torch.zeros((M, ldc), device="cuda").to(torch.float16) if epi == 1 else None
    gb.k_gemm_f16(C, dev_f16(A), dev_f16(B), M, N, K, lda, ldb, ldc, at, bt, epi,
                  bias=None if bias is None else dev(bias), C2=C2,
                  R=None if Rbuf is None else dev_f16(Rbuf), colsum=colsum)
    got = host(C)[:, :N]
    if epi == 0:
        assert_close_mag("gemm_f16 store", got, ref, mag, K, rtol=F16)
    elif epi == 1:
        assert_close_mag("gemm_f16 gelu pre", got, ref, mag, K, rtol=F16)
        assert_close_mag("gemm_f16 gelu", host(C2)[:, :N], oracle.gelu_forward(ref), 1.13 * mag,
                         K, rtol=F16)
    elif epi == 2:
        assert_close_mag("gemm_f16 resid", got, ref + Rv, mag + np.abs(Rv), K, rtol=F16)
    elif epi == 3:
        assert_close_mag("gemm_f16 accum", got, C0[:, :N] + ref, np.abs(C0[:, :N]) + mag, K,
                         rtol=1e-6)
        if colsum is not None:
            assert_close_mag("gemm_f16 colsum", host(colsum), cs0 + opA.sum(axis=1),
                             np.abs(cs0) + np.abs(opA).sum(axis=1), K, rtol=1e-6)
    else:
        rg = oracle.gelu_backward(Rv, ref)
        mg = np.abs(oracle.gelu_backward(Rv, mag))
        assert_close_mag("gemm_f16 gelu bwd", got, rg, mg, K, rtol=F16)


@pytest.mark.parametrize("B,T,C,NH", [(2, 100, 128, 2), (4, 16, 16, 4), (2, 64, 768, 12),
                                      (1, 1, 64, 1), (3, 257, 64, 1), (2, 130, 48, 2),
                                      (1, 200, 256, 2), (2, 77, 96, 3), (1, 1024, 1280, 20)])
def test_attention_f16(B, T, C, NH):
    r = rng(B * T + C + NH + 6)
    qkv = f16_values(r.normal(0, 1.0, (B, T, 3 * C)))
    dy = f16_values(r.normal(size=(B, T, C)))
    out = torch.full((B, T, C), float("nan"), device="cuda").to(torch.float16)
    lse = torch.empty((B, NH, T), device="cuda")
    gb.k_attention_forward_f16(out, lse, dev_f16(qkv), B, T, C, NH)
    ro, ratt = oracle.attention_forward(qkv, NH)
    qabs = qkv.copy()
    qabs[:, :, 2 * C:] = np.abs(qabs[:, :, 2 * C:])
    mag, _ = oracle.attention_forward(qabs, NH)
    hs = C // NH
    # P rounded to fp16 as the operand of P V moves out by up to 2^-11 mag (allowed 2^-10)
    assert_close_mag("attn out", host(out), ro, mag, T + hs, rtol=F16,
                     operand_u=F16 if hs % 8 == 0 else 0.0)
    dqkv = torch.full((B, T, 3 * C), float("nan"), device="cuda").to(torch.float16)
    gb.k_attention_backward_f16(dqkv, dev_f16(dy), dev_f16(qkv), out, lse, B, T, C, NH)
    rd = oracle.attention_backward(dy, qkv, ratt, NH)
    # as in the bf16 test: rowsum(dO * O) uses the kernel's own fp16 O, so dS carries an
    # error of that order -- 2^-9 relative plus 2^-10 of the tensor's scale
    scale = np.abs(rd).max()
    assert_close_mag("attn dqkv", host(dqkv), rd, np.full(rd.shape, scale), T, rtol=2 * F16,
                     atol=F16 * scale)


# ---------------------------------------------------------------------------------------
# whole steps in GPT2_DTYPE_FP16
# ---------------------------------------------------------------------------------------
def f16_steps(shape, seed, B, T, steps, mode, scale_residual):
    """Each step is compared from the GPU's own fp32 master parameters."""
    p0 = synth.init_params(shape, seed, scale_residual)
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, dtype="fp16")
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
        scale, skipped = m.get_loss_scale()
        assert not skipped and scale == 65536.0
        ref = oracle.gpt2_step(shape, got_p.astype(np.float64), tok, tgt, want_logits=True,
                               want_mags=True)
        rel = abs(loss - ref["loss"]) / abs(ref["loss"])
        s = assert_bf16_close("logits", logits, ref["logits"], ref["logit_mag"], LOGITS_R_F16)
        progress(f"fp16 step {step}: loss {loss:.6f} oracle {ref['loss']:.6f} rel {rel:.2e} "
                 f"logits {s}")
        assert rel <= LOSS_RTOL_F16
        compare_grads_bf16(shape, grads, ref["grads"], ref["grad_mag"], GRADS_R_F16,
                           label="fp16")
        rp, rm, rv = oracle.adamw(got_p.astype(np.float64), grads, rm, rv, HP["lr"],
                                  HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"],
                                  step + 1)
        assert np.abs(m.get_params() - rp).max() <= 1e-6
    m.close()


def test_f16_tiny_three_steps():
    w = synth.WORKLOADS["tiny"]
    f16_steps(w.shape, w.seed, w.B, w.T, 3, w.token_mode, w.scale_residual)


def test_f16_small_multilayer_ragged_two_steps():
    shape = synth.ModelShape(L=2, C=64, H=4, V=1000, maxT=128)
    f16_steps(shape, 4244, 3, 100, 2, "stream", True)


def test_f16_loss_scaler_skips_overflowing_steps_and_adapts():
    """A scale that overflows fp16 in the backward: the step is skipped (parameters and
    moments unchanged), the scale halves until the gradients fit, and the first applied
    step matches the oracle's AdamW on the unscaled gradients; with a short growth
    interval the scale then doubles after that many clean steps; a fixed scale never
    changes."""
    shape = synth.ModelShape(L=2, C=64, H=4, V=1000, maxT=128)
    B, T = 2, 64
    p0 = synth.init_params(shape, 55, True)
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, dtype="fp16")
    m.set_params(p0)
    tok, tgt = synth.batch(56, B, T, shape.V)
    # (p - 1)/(B T) * 2^24 = 1.3e5 overflows fp16 in dlogits itself
    m.set_loss_scale(2.0 ** 24, growth_interval=3)
    scales, t = [], 1
    for _ in range(12):
        before = m.get_params()
        m.zero_grad()
        m.forward(dev(tok), dev(tgt))
        m.backward()
        m.adamw_step(t=t, **HP)
        scale, skipped = m.get_loss_scale()
        scales.append((scale, skipped))
        if skipped:
            np.testing.assert_array_equal(m.get_params(), before)
            mo, vo = m.get_adam_state()
            assert not mo.any() and not vo.any()
        else:
            break
    assert scales[0] == (2.0 ** 23, True), scales
    assert not scales[-1][1], scales
    for (a, _), (b, _) in zip(scales[:-1], scales[1:]):
        assert b == a / 2 or b == a, scales  # halving while it overflows
    # the applied step: AdamW rule on the unscaled gradients
    g = m.get_grads()
    rp, _, _ = oracle.adamw(before.astype(np.float64), g, np.zeros(p0.size), np.zeros(p0.size),
                            HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                            HP["weight_decay"], 1)
    assert np.abs(m.get_params() - rp).max() <= 1e-6
    ref = oracle.gpt2_step(shape, before.astype(np.float64), tok, tgt, want_mags=True)
    compare_grads_bf16(shape, g, ref["grads"], ref["grad_mag"], GRADS_R_F16, label="scaler")
    # growth: clean steps double the scale after growth_interval of them
    m.set_loss_scale(4.0, growth_interval=2)
    seen = []
    for t in range(2, 7):
        m.zero_grad()
        m.forward(dev(tok), dev(tgt))
        m.backward()
        m.adamw_step(t=t, **HP)
        seen.append(m.get_loss_scale())
    assert [s for s, _ in seen] == [4.0, 8.0, 8.0, 16.0, 16.0], seen
    # a fixed scale (interval 0) stays put even through an overflow, which is still skipped
    m.set_loss_scale(2.0 ** 24, growth_interval=0)
    before = m.get_params()
    m.zero_grad()
    m.forward(dev(tok), dev(tgt))
    m.backward()
    m.adamw_step(t=7, **HP)
    assert m.get_loss_scale() == (2.0 ** 24, True)
    np.testing.assert_array_equal(m.get_params(), before)
    with pytest.raises(gb.GPT2Error):
        m.set_loss_scale(3.0)
    m.close()


@pytest.mark.timeout(600)
def test_f16_774m_b8_t1024_full_rows():
    """The 774M shape in fp16 at B8 T1024: two full T=1024 rows (per-position losses and
    logits) against single-row oracle forwards, and a finite, applied first step."""
    w = synth.WORKLOADS["gpt2_774m_b8_t1024_fp16"]
    shape = w.shape
    B, T, V = w.B, w.T, shape.V
    p0 = synth.init_params(shape, w.seed, w.scale_residual)
    tok, tgt = synth.batch(w.seed, B, T, V, mode=w.token_mode)
    rows = [0, 7]
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, B, T, dtype="fp16")
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
    m.adamw_step(t=1, **HP)
    assert m.get_loss_scale() == (65536.0, False)
    assert np.isfinite(m.get_params()).all()
    m.close()
    ref = oracle_batch(shape, p0.astype(np.float64), tok[rows], tgt[rows], want_logits=True,
                       want_grads=False, label="774M fp16 rows",
                       row_hook=lambda i, r: check_losses_and_logits_row(
                           rows[i], got_logits[i], r, shape.C, label="774M fp16:",
                           bf16=LOGITS_R_F16))
    rel = np.abs(got_losses - ref["losses"]) / np.abs(ref["losses"])
    progress(f"774M fp16 rows {rows}: per-position loss rel error max {rel.max():.2e}")
    assert rel.max() <= LOSS_RTOL_F16
    expect = math.log(V) + shape.C * 0.02 ** 2 / 2
    assert abs(loss - expect) < 0.05, (loss, expect)


@pytest.mark.timeout(600)
def test_f16_774m_b1_t32_gradients():
    w = synth.WORKLOADS["gpt2_774m_b8_t1024_fp16"]
    shape = w.shape
    p0 = synth.init_params(shape, w.seed, w.scale_residual)
    tok, tgt = synth.batch(w.seed, 1, 32, shape.V, mode=w.token_mode)
    m = gb.GPT2(shape.L, shape.C, shape.H, shape.V, shape.maxT, dtype="fp16")
    m.set_params(p0)
    m.zero_grad()
    loss = m.forward(dev(tok), dev(tgt))
    m.backward()
    grads = m.get_grads()
    m.close()
    ref = oracle.gpt2_step(shape, p0.astype(np.float64), tok, tgt, want_mags=True)
    rel = abs(loss - ref["loss"]) / abs(ref["loss"])
    progress(f"774M fp16 B1 T32: loss {loss:.6f} oracle {ref['loss']:.6f} rel {rel:.2e}")
    assert rel <= LOSS_RTOL_F16
    compare_grads_bf16(shape, grads, ref["grads"], ref["grad_mag"], GRADS_R_F16,
                       label="774M fp16 B1 T32")
