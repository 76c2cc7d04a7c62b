"""Pins of the oracle's FP8 (E4M3) cache functions to facts outside the oracle (CPU only).

The pages name an FP8 E4M3 KV cache (lecture 34 §4.4: one byte per key and value element) but give
no encoding; the format is the OCP 8-bit floating point one (1 sign, 4 exponent bits with bias 7,
3 mantissa bits, subnormals below 2^-6, no infinities, S.1111.111 = NaN, largest value 448). The
pins: torch's float8_e4m3fn number type (decoding all 256 codes; rounding in-range float32 values),
the format's defining constants, brute force over the 254 finite codes (nearest value, ties to the
even code), and a pool whose values are exactly representable, where the FP8 decode must equal the
16-bit decode bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def torch_e4m3_to_f64(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def torch_f32_to_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_matches_torch_for_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_to_double(codes), torch_e4m3_to_f64(codes), equal_nan=True)


def test_defining_constants_of_the_format():
    v = lambda c: float(oracle.e4m3_to_double(np.uint8(c)))
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x3C) == 1.5
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest magnitude 1.75 * 2^8
    assert v(0x08) == 2.0 ** -6                             # smallest normal
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals m * 2^-9
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))    # the only NaNs; no infinities
    assert all(math.isfinite(x) for x in oracle.e4m3_to_double(FINITE))


def test_encode_round_trips_every_finite_code():
    vals = oracle.e4m3_to_double(FINITE).astype(np.float32)
    assert np.array_equal(oracle.e4m3_from_float(vals), FINITE)


def brute_force_code(x):
    """Nearest finite E4M3 value; ties to the even mantissa; beyond 448 saturate."""
    vals = oracle.e4m3_to_double(FINITE)
    if math.isnan(x):
        return None
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = min(abs(x), 448.0)
    pos = [c for c in FINITE if c < 0x80]
    pv = oracle.e4m3_to_double(np.array(pos, np.uint8))
    d = np.abs(pv - a)
    best = np.flatnonzero(d == d.min())
    c = int(pos[best[0]]) if len(best) == 1 else int([pos[i] for i in best if pos[i] % 2 == 0][0])
    return sign | c


def test_encode_equals_brute_force_on_midpoints_and_neighbours():
    pos = oracle.e4m3_to_double(np.arange(0x00, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    xs = []
    for m in mids:
        f = np.float32(m)
        xs += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    xs += [np.float32(v) for v in (449.0, 463.9, 464.0, 470.0, 1e6, 1e-30, 2.0 ** -10)]
    xs = np.array(xs, np.float32)
    xs = np.concatenate([xs, -xs])
    got = oracle.e4m3_from_float(xs)
    want = [brute_force_code(float(x)) for x in xs]
    assert got.tolist() == want


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 150)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(oracle.e4m3_from_float(x), torch_f32_to_e4m3(x))


def test_encode_saturates_and_keeps_signs():
    f = lambda v: int(oracle.e4m3_from_float(np.float32(v)))
    assert f(np.inf) == 0x7E and f(-np.inf) == 0xFE and f(1e30) == 0x7E and f(-500) == 0xFE
    assert f(0.0) == 0x00 and f(-0.0) == 0x80 and f(1e-30) == 0x00 and f(-1e-30) == 0x80
    assert f(np.float32("nan")) == 0x7F and f(-np.float32("nan")) == 0xFF


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -6, 0.0123])
def test_quantize_is_code_of_float32_quotient(dtype, scale):
    rng = np.random.default_rng(11)
    words = W.f32_to_words(rng.standard_normal(4000).astype(np.float32) * 2, dtype)
    x = torch.from_numpy(words.view(np.int16)).view(
        torch.float16 if dtype == "f16" else torch.bfloat16).to(torch.float32)
    q = (x / torch.tensor(scale, dtype=torch.float32)).clamp(-448, 448)
    want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_e4m3(words, dtype, scale), want)


def test_fp8_scatter_writes_codes_of_the_tokens_at_their_slots():
    w = W.build([17, 3, 33], 2, 2, 64, "bf16", seed=51)
    n = w.num_blocks * 2 * 16 * 64
    kc0 = np.full(n, 0x55, np.uint8)
    vc0 = np.full(n, 0xAA, np.uint8)
    kc, vc = oracle.reshape_and_cache_fp8(w.new_key, w.new_value, kc0, vc0, w.slot_mapping,
                                          w.num_blocks, 2, 64, "bf16", 0.25, 0.5)
    k4 = kc.reshape(w.num_blocks, 2, 16, 64)
    v4 = vc.reshape(w.num_blocks, 2, 16, 64)
    touched = np.zeros((w.num_blocks, 16), bool)
    for t, s in enumerate(w.slot_mapping):
        b, o = divmod(int(s), 16)
        touched[b, o] = True
        assert np.array_equal(k4[b, :, o], oracle.quantize_e4m3(w.new_key[t], "bf16", 0.25))
        assert np.array_equal(v4[b, :, o], oracle.quantize_e4m3(w.new_value[t], "bf16", 0.5))
    assert (k4.transpose(0, 2, 1, 3)[~touched] == 0x55).all()
    assert (v4.transpose(0, 2, 1, 3)[~touched] == 0xAA).all()


def test_fp8_copy_blocks_copies_whole_blocks():
    rng = np.random.default_rng(3)
    nb, H, D = 6, 2, 64
    kc = rng.integers(0, 256, nb * H * 16 * D, dtype=np.uint8)
    vc = rng.integers(0, 256, nb * H * 16 * D, dtype=np.uint8)
    k2, v2 = oracle.copy_blocks_fp8(kc, vc, [[1, 4], [0, 5]], nb, H, D)
    per = H * 16 * D
    want_k, want_v = kc.copy(), vc.copy()
    want_k[4 * per:5 * per] = kc[1 * per:2 * per]
    want_k[5 * per:6 * per] = kc[0 * per:1 * per]
    want_v[4 * per:5 * per] = vc[1 * per:2 * per]
    want_v[5 * per:6 * per] = vc[0 * per:1 * per]
    assert np.array_equal(k2, want_k) and np.array_equal(v2, want_v)


def exact_fp8_pool(w, rng, scale):
    """16-bit pool whose values are E4M3 values times a power-of-two scale (exact in f16/bf16),
    and the E4M3 codes it quantizes to without loss."""
    codes = rng.choice(FINITE, size=w.k_cache.size).astype(np.uint8)
    vals = (oracle.e4m3_to_double(codes) * scale).astype(np.float32)
    return W.f32_to_words(vals, w.dtype), codes


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_decode_equals_16bit_decode_on_exactly_representable_pool(dtype):
    w = W.build([1, 40, 77], 4, 2, 64, dtype, seed=52)
    rng = np.random.default_rng(52)
    ks, vs = 2.0 ** -6, 2.0 ** -5
    k16, kcodes = exact_fp8_pool(w, rng, ks)
    v16, vcodes = exact_fp8_pool(w, rng, vs)
    assert np.array_equal(oracle.quantize_e4m3(k16, dtype, ks), kcodes)
    assert np.array_equal(oracle.quantize_e4m3(v16, dtype, vs), vcodes)
    a = oracle.decode(w.query_decode, k16, v16, w.block_tables, w.seq_lens, 4, 2, 64,
                      w.num_blocks, dtype, w.scale)
    b = oracle.decode_fp8(w.query_decode, kcodes, vcodes, w.block_tables, w.seq_lens, 4, 2, 64,
                          w.num_blocks, dtype, w.scale, ks, vs)
    assert np.array_equal(a, b)


def test_fp8_decode_matches_sdpa_on_dequantized_rows():
    """The FP8 decode is softmax attention over code value * scale rows, gathered here with numpy
    from the 4-d pool view and evaluated by torch's sdpa in float64."""
    w = W.build([50, 9], 4, 4, 64, "f16", seed=53)
    ks, vs = 0.02, 0.03
    kc = oracle.quantize_e4m3(w.k_cache, "f16", ks)
    vc = oracle.quantize_e4m3(w.v_cache, "f16", vs)
    out = oracle.decode_fp8(w.query_decode, kc, vc, w.block_tables, w.seq_lens, 4, 4, 64,
                            w.num_blocks, "f16", w.scale, ks, vs)
    k4 = torch_e4m3_to_f64(kc).reshape(w.num_blocks, 4, 16, 64) * ks
    v4 = torch_e4m3_to_f64(vc).reshape(w.num_blocks, 4, 16, 64) * vs
    for s in range(2):
        L = int(w.seq_lens[s])
        pos = np.arange(L)
        blk = w.block_tables[s][pos // 16]
        for h in range(4):
            K = torch.from_numpy(k4[blk, h, pos % 16])[None, None]
            V = torch.from_numpy(v4[blk, h, pos % 16])[None, None]
            q = torch.from_numpy(oracle.to_double(w.query_decode[s, h], "f16"))[None, None, None]
            want = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=w.scale)
            assert np.allclose(out[s, h], want[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_prefill_equals_16bit_prefill_on_exactly_representable_pool(dtype):
    """F7 on a pool that E4M3 codes hold without loss equals the 16-bit prefill (O7) bit for bit."""
    w = W.build([30, 90, 17], 4, 2, 64, dtype, seed=54, n_decode=0, q_lens=[30, 25, 4])
    rng = np.random.default_rng(54)
    ks, vs = 2.0 ** -6, 2.0 ** -4
    k16, kcodes = exact_fp8_pool(w, rng, ks)
    v16, vcodes = exact_fp8_pool(w, rng, vs)
    a = oracle.prefill(w.query_prefill, k16, v16, w.block_tables, w.seq_lens, w.cu_q_lens, 4, 2,
                       64, w.num_blocks, dtype, w.scale)
    b = oracle.prefill_fp8(w.query_prefill, kcodes, vcodes, w.block_tables, w.seq_lens,
                           w.cu_q_lens, 4, 2, 64, w.num_blocks, dtype, w.scale, ks, vs)
    assert np.array_equal(a, b)


def test_fp8_prefill_rows_match_causal_sdpa_on_dequantized_rows():
    """Chunk rows of F7 are causal softmax attention over code value * scale rows (torch sdpa,
    float64, explicit mask), the rows gathered with numpy from the 4-d pool view."""
    w = W.build([70, 33], 4, 2, 64, "bf16", seed=55, n_decode=0, q_lens=[20, 33])
    ks, vs = 0.05, 0.015
    kc = oracle.quantize_e4m3(w.k_cache, "bf16", ks)
    vc = oracle.quantize_e4m3(w.v_cache, "bf16", vs)
    out = oracle.prefill_fp8(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                             4, 2, 64, w.num_blocks, "bf16", w.scale, ks, vs)
    k4 = torch_e4m3_to_f64(kc).reshape(w.num_blocks, 2, 16, 64) * ks
    v4 = torch_e4m3_to_f64(vc).reshape(w.num_blocks, 2, 16, 64) * vs
    for s in range(2):
        L = int(w.seq_lens[s])
        a, b = int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])
        pos = np.arange(L)
        blk = w.block_tables[s][pos // 16]
        mask = torch.from_numpy(np.arange(L)[None, :] <= np.arange(L - (b - a), L)[:, None])
        for h in range(4):
            K = torch.from_numpy(k4[blk, h // 2, pos % 16])[None, None]
            V = torch.from_numpy(v4[blk, h // 2, pos % 16])[None, None]
            q = torch.from_numpy(oracle.to_double(w.query_prefill[a:b, h], "bf16"))[None, None]
            want = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask[None, None],
                                                                    scale=w.scale)
            assert np.allclose(out[a:b, h], want[0, 0].numpy(), rtol=1e-12, atol=1e-13)
