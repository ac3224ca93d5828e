"""Pins of the FP8 (E4M3) part of the oracle, on the CPU.

The encoder is checked against torch's float8_e4m3fn conversion (a library routine) on ordinary
values and on exact ties, and against the format's defining values; the FP8 attention path is
checked against the bf16 path on caches whose values E4M3 holds exactly, where the two must agree
bit for bit.  Planted mistakes in the encoder must fail these pins.
"""

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import paged_attention as pa
from workloads import Spec, bf16_bits, build_case


def torch_e4m3(x):
    """torch's conversion; it does not saturate, so callers keep |x| <= 448."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_defining_values():
    t = fp8.decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0      # largest finite
    assert t[0x08] == 2.0 ** -6                         # smallest normal
    assert t[0x01] == 2.0 ** -9                         # smallest subnormal
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x3C] == 1.5
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.all(np.diff(t[:0x7F]) > 0)                # codes 0..0x7E increase
    finite = np.nonzero(~np.isnan(t))[0]
    assert np.array_equal(fp8.encode(t[finite]), finite.astype(np.uint8))  # round trip


def test_encode_matches_library_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(fp8.encode(x), torch_e4m3(x))


def test_ties_go_to_the_even_code():
    t = fp8.decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)  # midpoints are exact in fp32
    assert np.array_equal(fp8.encode(mids), torch_e4m3(mids))
    assert np.all(fp8.encode(mids) % 2 == 0)
    assert np.array_equal(fp8.encode(-mids), torch_e4m3(-mids))


def test_saturation_and_signs():
    assert list(fp8.encode(np.array([449.0, 464.0, 1e6, np.inf]))) == [0x7E] * 4
    assert list(fp8.encode(np.array([-500.0, -np.inf]))) == [0xFE] * 2
    assert fp8.encode(np.array([-0.0]))[0] == 0x80
    assert fp8.encode(np.array([-1e-5]))[0] == 0x80   # rounds to zero, keeps the sign
    assert fp8.encode(np.array([2.0 ** -10]))[0] == 0x00  # tie between 0 and 2^-9: even code
    assert fp8.encode(np.array([3 * 2.0 ** -10]))[0] == 0x02


def test_quantize_divides_in_fp32():
    x = bf16_bits(np.array([1.0, -3.0, 0.3, 1000.0], dtype=np.float32))
    c = fp8.quantize(x, 0.5)
    assert list(fp8.decode(c)) == [2.0, -6.0, fp8.decode(fp8.encode(np.float32(0.30078125) / 0.5)), 448.0]


def _exact_case(seed, scale):
    """A case whose cached values are scale * (E4M3 values), so FP8 holds them exactly."""
    case = build_case(Spec(name="fp8", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           seed=(seed,), decode_lens=[1, 17, 40, 95]))
    rng = np.random.default_rng(seed)
    t = fp8.decode_table()
    finite = t[~np.isnan(t)]
    finite = finite[np.abs(finite) <= 8]  # keep bf16 exact after scaling
    kc8 = rng.integers(0, len(finite), size=case.key_cache.shape)
    vc8 = rng.integers(0, len(finite), size=case.value_cache.shape)
    kv = finite[kc8] * scale
    vv = finite[vc8] * scale
    kc16 = bf16_bits(kv.astype(np.float32))
    vc16 = bf16_bits(vv.astype(np.float32))
    kcode = fp8.encode(finite[kc8])
    vcode = fp8.encode(finite[vc8])
    return case, kc16, vc16, kcode, vcode


@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_fp8_decode_equals_bf16_decode_on_exact_values(scale):
    case, kc16, vc16, kcode, vcode = _exact_case(3, scale)
    d = case.decode
    ref = pa.decode(d.query, kc16, vc16, d.block_tables, d.seq_lens, 2, 64, 16, case.scale)
    got = pa.decode_fp8(d.query, kcode, vcode, d.block_tables, d.seq_lens, 2, 64, 16, case.scale,
                        scale, scale)
    assert np.array_equal(got, ref)


def test_fp8_reshape_places_codes_like_bf16_reshape():
    case = build_case(Spec(name="fp8", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=32,
                           seed=(5,), decode_lens=[33, 70], decode_new_token=True))
    r = case.reshape
    kc8 = np.zeros(case.key_cache.shape, dtype=np.uint8)
    vc8 = np.zeros(case.value_cache.shape, dtype=np.uint8)
    k8, v8 = pa.reshape_and_cache_fp8(kc8, vc8, r.key, r.value, r.slot_mapping, 2, 64, 32, 0.5, 2.0)
    # The written rows, read back through the tables, are the quantised new tokens.
    d = case.decode
    for b in range(2):
        L = int(d.seq_lens[b])
        k, v = pa.gather_kv_fp8(k8, v8, d.block_tables[b], L, 2, 64, 32, 0.5, 2.0)
        assert np.array_equal(k[L - 1], 0.5 * fp8.decode(fp8.quantize(r.key[b], 0.5)))
        assert np.array_equal(v[L - 1], 2.0 * fp8.decode(fp8.quantize(r.value[b], 2.0)))
    assert np.count_nonzero(k8) <= 2 * 2 * 64 and np.count_nonzero(v8) <= 2 * 2 * 64


def _fp8_pins_pass():
    try:
        test_defining_values()
        test_encode_matches_library_conversion()
        test_ties_go_to_the_even_code()
        test_saturation_and_signs()
    except AssertionError:
        return False
    return True


def test_fp8_pins_catch_planted_mistakes(monkeypatch):
    real_table = fp8.decode_table()

    def truncating(x):  # round toward zero instead of to nearest
        x = np.asarray(x, dtype=np.float64)
        a = np.minimum(np.abs(x), 448.0)
        idx = np.searchsorted(real_table[:0x7F], a, side="right") - 1
        return (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    def ties_up(x):  # ties away from zero
        x = np.asarray(x, dtype=np.float64)
        a = np.minimum(np.abs(x), 448.0)
        d = np.abs(real_table[:0x7F][None, :] - a[..., None])
        idx = (d.shape[-1] - 1) - np.argmin(d[..., ::-1], axis=-1)
        return (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    for fake in (truncating, ties_up):
        with monkeypatch.context() as m:
            m.setattr(fp8, "encode", fake)
            assert not _fp8_pins_pass(), fake.__name__
    bias8 = real_table.copy()
    bias8[:0x7F] /= 2  # exponent bias 8 instead of 7
    with monkeypatch.context() as m:
        m.setattr(fp8, "decode_table", lambda: bias8)
        assert not _fp8_pins_pass()


def test_fp8_prefill_equals_bf16_prefill_on_exact_values():
    case = build_case(Spec(name="fp8p", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           seed=(6,), prefill=[(40, 9), (0, 5)]))
    rng = np.random.default_rng(6)
    t = fp8.decode_table()
    finite = t[~np.isnan(t)]
    finite = finite[np.abs(finite) <= 8]
    kc8 = rng.integers(0, len(finite), size=case.key_cache.shape)
    vc8 = rng.integers(0, len(finite), size=case.value_cache.shape)
    p = case.prefill
    for scale in (1.0, 0.5):
        kc16 = bf16_bits((finite[kc8] * scale).astype(np.float32))
        vc16 = bf16_bits((finite[vc8] * scale).astype(np.float32))
        ref = pa.prefill_chunk(p.query, kc16, vc16, p.block_tables, p.query_start_loc, p.seq_lens,
                               2, 64, 16, case.scale)
        got = pa.prefill_chunk_fp8(p.query, fp8.encode(finite[kc8]), fp8.encode(finite[vc8]),
                                   p.block_tables, p.query_start_loc, p.seq_lens, 2, 64, 16,
                                   case.scale, scale, scale)
        assert np.array_equal(got, ref)
