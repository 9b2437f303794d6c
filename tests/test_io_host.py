"""Host-side checks (no GPU) of the checkpoint and token-file formats and of the random
number generator the C ABI exposes, against the layouts the llm.c page defines
("llm.c 的中文注解-20240421": 1.22 checkpoint header and parameter order, 1.28 - 1.32
DataLoader, 1.33 / 1.34 random_u32 / random_f32), plus the oracle's sample_mult (1.35)."""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_05_amd import binding as gb
from decoder_only_transformer_05_amd import synth

SHAPE = synth.ModelShape(L=2, C=24, H=3, V=41, maxT=12)


def write_checkpoint_numpy(path, params, shape, magic=20240326, version=1):
    """The file as 1.22 reads it: 256 int32 of header, then the fp32 parameters."""
    hdr = np.zeros(256, np.int32)
    hdr[:7] = [magic, version, shape.maxT, shape.V, shape.L, shape.H, shape.C]
    with open(path, "wb") as f:
        hdr.tofile(f)
        np.asarray(params, np.float32).tofile(f)


def test_checkpoint_written_by_the_library_has_the_pages_layout(tmp_path):
    p = synth.init_params(SHAPE, 5, True)
    path = tmp_path / "m.bin"
    gb.checkpoint_write(path, p, SHAPE.L, SHAPE.C, SHAPE.H, SHAPE.V, SHAPE.maxT)
    raw = np.fromfile(path, np.int32, count=256)
    assert list(raw[:7]) == [20240326, 1, SHAPE.maxT, SHAPE.V, SHAPE.L, SHAPE.H, SHAPE.C]
    assert not raw[7:].any()
    body = np.fromfile(path, np.float32, offset=1024)
    assert body.size == sum(synth.param_sizes(SHAPE.L, SHAPE.C, SHAPE.V, SHAPE.maxT))
    np.testing.assert_array_equal(body, p)


def test_checkpoint_read_of_a_file_written_from_the_layout(tmp_path):
    p = synth.init_params(SHAPE, 6, True)
    path = tmp_path / "m.bin"
    write_checkpoint_numpy(path, p, SHAPE)
    info = gb.checkpoint_info(path)
    assert info == {"maxT": SHAPE.maxT, "V": SHAPE.V, "L": SHAPE.L, "H": SHAPE.H, "C": SHAPE.C,
                    "num_params": p.size}
    np.testing.assert_array_equal(gb.checkpoint_read(path), p)


@pytest.mark.parametrize("defect", ["magic", "version", "truncated", "extra", "short_header",
                                    "zero_size", "missing"])
def test_checkpoint_rejects_malformed_files(tmp_path, defect):
    p = synth.init_params(SHAPE, 7, True)
    path = tmp_path / "m.bin"
    if defect == "magic":
        write_checkpoint_numpy(path, p, SHAPE, magic=20240327)
    elif defect == "version":
        write_checkpoint_numpy(path, p, SHAPE, version=2)
    elif defect == "truncated":
        write_checkpoint_numpy(path, p[:-1], SHAPE)
    elif defect == "extra":
        write_checkpoint_numpy(path, np.concatenate([p, p[:1]]), SHAPE)
    elif defect == "short_header":
        np.zeros(100, np.int32).tofile(path)
    elif defect == "zero_size":
        write_checkpoint_numpy(path, p, synth.ModelShape(L=0, C=24, H=3, V=41, maxT=12))
    with pytest.raises(gb.GPT2Error) as e:
        gb.checkpoint_info(path)
    assert e.value.code == -7
    with pytest.raises(gb.GPT2Error):
        gb.checkpoint_read(path)


def test_dataloader_windows_shift_and_wrap(tmp_path):
    """Batches are consecutive windows of B*T+1 tokens advancing by B*T, targets shifted by
    one, back to the start when the next window would pass the end of the file."""
    B, T, n = 3, 5, 64
    tokens = synth.tokens_uniform(11, 0, n, 50257)
    path = tmp_path / "tok.bin"
    tokens.astype(np.int32).tofile(path)
    dl = gb.DataLoader(path, B, T)
    assert dl.num_batches == n // (B * T)
    pos = 0
    for _ in range(10):
        if pos + B * T + 1 > n:
            pos = 0
        x, y = dl.next_batch()
        np.testing.assert_array_equal(x.ravel(), tokens[pos:pos + B * T])
        np.testing.assert_array_equal(y.ravel(), tokens[pos + 1:pos + B * T + 1])
        pos += B * T
    dl.reset()
    x, y = dl.next_batch()
    np.testing.assert_array_equal(x.ravel(), tokens[:B * T])
    dl.close()


def test_dataloader_exact_fit_and_errors(tmp_path):
    B, T = 2, 4
    path = tmp_path / "tok.bin"
    np.arange(B * T + 1, dtype=np.int32).tofile(path)  # exactly one window
    dl = gb.DataLoader(path, B, T)
    for _ in range(3):  # every call returns the one window
        x, y = dl.next_batch()
        np.testing.assert_array_equal(x.ravel(), np.arange(B * T))
        np.testing.assert_array_equal(y.ravel(), np.arange(1, B * T + 1))
    dl.close()
    np.arange(B * T, dtype=np.int32).tofile(path)  # one token short
    with pytest.raises(gb.GPT2Error) as e:
        gb.DataLoader(path, B, T)
    assert e.value.code == -1
    with pytest.raises(gb.GPT2Error) as e:
        gb.DataLoader(tmp_path / "missing.bin", B, T)
    assert e.value.code == -7


def _xorshift_star(state):
    """xorshift* with shifts 12, 25, 27 and multiplier 0x2545F4914F6CDD1D (Vigna, "An
    experimental exploration of Marsaglia's xorshift generators, scrambled", 2016)."""
    m64 = (1 << 64) - 1
    state ^= state >> 12
    state ^= (state << 25) & m64
    state ^= state >> 27
    return state, ((state * 0x2545F4914F6CDD1D) & m64) >> 32


def test_random_u32_and_f32_follow_xorshift_star():
    r = gb.Rng(1337)
    s = 1337
    for _ in range(1000):
        s, want = _xorshift_star(s)
        assert r.u32() == want
    assert r.state.value == s
    r2 = gb.Rng(42)
    s = 42
    for _ in range(1000):
        s, u = _xorshift_star(s)
        f = r2.f32()
        assert f == np.float32((u >> 8) / 16777216.0) and 0.0 <= f < 1.0


def test_sample_mult_oracle_pins():
    """1.35: the first index whose cumulative probability exceeds coin, else the last."""
    p = np.array([0.125, 0.25, 0.5, 0.125])  # exact binary fractions: the cdf is exact
    cases = {0.0: 0, 0.1249: 0, 0.125: 1, 0.3: 1, 0.375: 2, 0.874: 2, 0.875: 3, 0.9999: 3}
    for coin, want in cases.items():
        assert oracle.sample_mult(p, coin) == want, coin
    # probabilities that sum to slightly less than 1: a coin above the total -> last index
    q = np.array([0.3, 0.3, 0.3999])
    assert oracle.sample_mult(q, 0.99995) == 2
    # a one-hot distribution always returns its index
    h = np.zeros(10)
    h[6] = 1.0
    for coin in (0.0, 0.5, 0.999):
        assert oracle.sample_mult(h, coin) == 6
    # against the inverse-cdf definition with numpy's cumulative sum on random rows
    rng = np.random.default_rng(3)
    for _ in range(200):
        z = rng.normal(0, 2, 50)
        pr = np.exp(z - z.max())
        pr /= pr.sum()
        coin = rng.random()
        cdf = np.cumsum(pr)
        want = int(np.argmax(coin < cdf)) if (coin < cdf).any() else 49
        assert oracle.sample_mult(pr, coin) == want
