"""Pins of the quantized-KV oracle (CPU only): the E4M3 codec against the format's own
fields and torch's float8_e4m3fn conversion, the affine quantizer of
"LLM 推理优化全景实战" §4.1 against hand-worked codes and its nearest-level property, the
quantized append, and the attention over dequantized caches against torch's SDPA."""

import math

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as orc
from paged_kv_cache_26_amd import workload as wlm
from tests.parity import within


# ---------------------------------------------------------------------------------------
# E4M3 codec
# ---------------------------------------------------------------------------------------

def test_e4m3_decode_fields():
    d = orc.e4m3_decode
    assert d(np.array([0x38]))[0] == 1.0              # exponent 7 = bias, mantissa 0
    assert d(np.array([0x7E]))[0] == 448.0            # largest finite: 1.75 * 2^8
    assert d(np.array([0x08]))[0] == 2.0 ** -6        # smallest normal
    assert d(np.array([0x01]))[0] == 2.0 ** -9        # smallest subnormal
    assert d(np.array([0x07]))[0] == 7 * 2.0 ** -9    # largest subnormal
    assert d(np.array([0xB8]))[0] == -1.0
    assert np.isnan(d(np.array([0x7F, 0xFF]))).all()  # the only NaNs, no infinities
    v = d(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)                     # codes 0..126 increase strictly


def test_e4m3_decode_matches_torch_for_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(0)
    pos = orc.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                   # exact ties: both neighbours equidistant
    y = np.concatenate([
        rng.standard_normal(20000) * 50, rng.uniform(-448, 448, 20000),
        rng.uniform(-2 ** -6, 2 ** -6, 5000),         # subnormal range
        pos, -pos, mids.astype(np.float32), -mids.astype(np.float32),
        np.float32([0.0, -0.0, 448.0, -448.0]),
    ]).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(y), _torch_encode(y))


def test_e4m3_encode_ties_go_to_even():
    # 1.0625 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1): even wins
    assert orc.e4m3_encode(np.float32([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (mantissa 1) and 1.25 (mantissa 2)
    assert orc.e4m3_encode(np.float32([1.1875]))[0] == 0x3A
    assert orc.e4m3_encode(np.float32([500.0]))[0] == 0x7E      # saturates at 448


# ---------------------------------------------------------------------------------------
# Affine INT8 quantizer, Q(x) = round(x / s) + z, x^ = s (Q - z)
# ---------------------------------------------------------------------------------------

def test_int8_hand_worked_row():
    """x = (-1, 0, 0.5, 3): lo = -1, hi = 3, s = 4/255, z = round(63.75) = 64;
    codes round(-63.75) + 64 = 0, 64, round(31.875) + 64 = 96, round(191.25) + 64 = 255."""
    q, s, z = orc.quantize_row(np.float32([-1, 0, 0.5, 3]), "int8")
    assert s == np.float32(np.float32(4.0) / np.float32(255.0)) and z == 64
    assert list(q) == [0, 64, 96, 255]
    x_hat = orc.dequantize(q, s, z, "int8")
    assert x_hat[1] == 0.0                                # zero is exact


@pytest.mark.parametrize("seed", range(5))
def test_int8_nearest_level_and_error_bound(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(128) * rng.uniform(0.01, 10) + rng.uniform(-3, 3)).astype(np.float32)
    q, s, z = orc.quantize_row(x, "int8")
    lo, hi = min(x.min(), 0), max(x.max(), 0)
    assert q[np.argmin(x)] == (0 if x.min() <= 0 else q[np.argmin(x)])
    x_hat = orc.dequantize(q, s, z, "int8")
    # every element within half a step (plus binary32 rounding of x / s)
    assert np.all(np.abs(x_hat - x) <= 0.5 * float(s) * (1 + 1e-5) + 1e-12)
    # and on the nearest of the 256 levels, except at near-ties
    levels = float(s) * (np.arange(256) - float(z))
    dist = np.abs(x[:, None].astype(np.float64) - levels[None, :])
    best = np.argmin(dist, axis=1)
    srt = np.sort(dist, axis=1)
    clear = srt[:, 1] - srt[:, 0] > 1e-5 * float(s)
    assert np.array_equal(q[clear], best[clear])
    assert lo <= x_hat.min() + s and hi >= x_hat.max() - s


def test_int8_degenerate_rows():
    q, s, z = orc.quantize_row(np.zeros(64, np.float32), "int8")
    assert s == 1.0 and z == 0 and not q.any()
    q, s, z = orc.quantize_row(np.full(64, 2.5, np.float32), "int8")
    assert z == 0 and (q == 255).all()                   # lo = 0, hi = 2.5
    q, s, z = orc.quantize_row(np.full(64, -2.5, np.float32), "int8")
    assert z == 255 and (q == 0).all()                   # lo = -2.5, hi = 0


# ---------------------------------------------------------------------------------------
# FP8 quantizer, s = max|x| / 448
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(5))
def test_fp8_quantizer_bounds(seed):
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_normal(128) * rng.uniform(0.01, 10)).astype(np.float32)
    q, s, z = orc.quantize_row(x, "fp8")
    assert z == 0
    assert q[np.argmax(np.abs(x))] & 0x7F == 0x7E        # the largest magnitude maps to 448
    x_hat = orc.dequantize(q, s, z, "fp8")
    y = np.abs(x / float(s))
    normal = y >= 2 ** -6
    # half an ulp of a 3-bit mantissa: relative 2^-4 for normals, 2^-10 * s below
    assert np.all(np.abs(x_hat - x)[normal] <= 2 ** -4 * np.abs(x)[normal] * (1 + 1e-6))
    assert np.all(np.abs(x_hat - x)[~normal] <= 2 ** -10 * float(s) * (1 + 1e-6))
    assert np.array_equal(np.sign(x_hat[x != 0]), np.sign(x[x != 0]))


def test_fp8_zero_row():
    q, s, z = orc.quantize_row(np.zeros(16, np.float32), "fp8")
    assert s == 1.0 and not q.any()


# ---------------------------------------------------------------------------------------
# Quantized append and attention
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", orc.KV_FORMATS)
def test_quantized_append_writes_one_slot(fmt):
    wl = wlm.make_workload(wlm.QUANT_SMALL_SPECS[fmt], seed=3)
    kc, vc, ks, vs = orc.kv_append_quantized(wl.k_pool, wl.v_pool, wl.k_scales, wl.v_scales,
                                             wl.k_new, wl.v_new, wl.block_tables,
                                             wl.positions, 16, fmt, wl.dtype)
    changed = np.zeros(kc.shape[:2], bool)
    for b in range(wl.batch):
        t = int(wl.positions[b])
        phys, off = int(wl.block_tables[b, t // 16]), t % 16
        changed[phys, off] = True
        for j in range(wl.spec.n_kv_heads):
            q, s, z = orc.quantize_row(orc.storage_to_f64(wl.k_new[b, j], wl.dtype), fmt)
            assert np.array_equal(kc[phys, off, j], q) and (ks[phys, j, off] == (s, z)).all()
    assert np.array_equal(kc[~changed], wl.k_pool[~changed])
    assert np.array_equal(vc[~changed], wl.v_pool[~changed])
    keep = ~np.broadcast_to(changed[:, None, :], ks.shape[:3])
    np.testing.assert_array_equal(ks[keep], wl.k_scales[keep])   # NaN-poison compares equal


def _sdpa_dequantized(wl, kc, vc, ks, vs, fmt):
    B, H, d = wl.q.shape
    out = np.empty((B, H, d))
    for b in range(B):
        n = int(wl.context_lens[b])
        t = np.arange(n)
        phys = wl.block_tables[b, t // 16]
        ks_ = ks[phys, :, t % 16]                       # [n, Hkv, 2]
        vs_ = vs[phys, :, t % 16]
        k = orc.dequantize(kc[phys, t % 16], ks_[..., 0], ks_[..., 1], fmt)   # [n, Hkv, d]
        v = orc.dequantize(vc[phys, t % 16], vs_[..., 0], vs_[..., 1], fmt)
        qt = torch.from_numpy(orc.storage_to_f64(wl.q[b], wl.dtype))[None, :, None, :]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt.contiguous(), kt, vt,
                                                             enable_gqa=True)
        out[b] = o[0, :, 0].numpy()
    return out


@pytest.mark.parametrize("fmt", orc.KV_FORMATS)
def test_quantized_attention_equals_library_attention(fmt):
    wl = wlm.make_workload(wlm.QUANT_SMALL_SPECS[fmt], seed=4)
    kc, vc, ks, vs = orc.kv_append_quantized(wl.k_pool, wl.v_pool, wl.k_scales, wl.v_scales,
                                             wl.k_new, wl.v_new, wl.block_tables,
                                             wl.positions, 16, fmt, wl.dtype)
    got = orc.paged_decode_attention_quantized(wl.q, kc, vc, ks, vs, wl.block_tables,
                                               wl.context_lens, 16, wl.scale, fmt, wl.dtype)
    ref = _sdpa_dequantized(wl, kc, vc, ks, vs, fmt)
    assert np.isfinite(got).all()
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-12


def test_int8_cache_of_exact_values_equals_plain_attention():
    """Rows whose values sit exactly on the int8 grid dequantize exactly: the quantized
    attention then equals the plain oracle on an fp32 cache of the same values."""
    rng = np.random.default_rng(7)
    n, d, bs = 37, 64, 16
    s = np.float32(0.03125)                               # a power of two: x / s is exact
    x_codes = rng.integers(0, 256, size=(2, n, d))
    x_codes[..., 0], x_codes[..., 1] = 0, 255             # every row spans the full grid,
    z = 128                                               # so the quantizer finds s and z
    vals = (s * (x_codes - z)).astype(np.float32)         # [K/V, n, d] exact on the grid
    table = np.array([[2, 0, 1]], np.int32)
    kc = np.zeros((3, bs, 1, d), np.uint8)
    vc = np.zeros((3, bs, 1, d), np.uint8)
    ks = np.full((3, 1, bs, 2), np.nan, np.float32)
    vs = np.full((3, 1, bs, 2), np.nan, np.float32)
    kp = np.full((3, bs, 1, d), np.nan, np.float32)
    vp = np.full((3, bs, 1, d), np.nan, np.float32)
    for t in range(n):
        phys, off = table[0, t // bs], t % bs
        for codes, scales, pool, i in ((kc, ks, kp, 0), (vc, vs, vp, 1)):
            q, ss, zz = orc.quantize_row(vals[i, t], "int8")
            assert np.array_equal(orc.dequantize(q, ss, zz, "int8"), vals[i, t])
            codes[phys, off, 0] = q
            scales[phys, 0, off] = (ss, zz)
            pool[phys, off, 0] = vals[i, t]
    qv = rng.standard_normal((1, 2, d)).astype(np.float32)
    lens = np.array([n], np.int32)
    got = orc.paged_decode_attention_quantized(qv, kc, vc, ks, vs, table, lens, bs, 0.125,
                                               "int8", "f32")
    ref = orc.paged_decode_attention(qv, kp, vp, table, lens, bs, 0.125, "f32")
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_quantization_error_of_attention_is_small():
    """Not a definition pin, a sanity property: quantizing the bf16 GQA cache to int8 /
    fp8 moves the attention output by far less than the output scale."""
    wl = wlm.make_workload(3, small=True)
    kp, vp = orc.kv_append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.block_tables,
                           wl.positions, 16)
    ref = orc.paged_decode_attention(wl.q, kp, vp, wl.block_tables, wl.context_lens, 16,
                                     wl.scale, "bf16")
    nb, bs, Hkv, d = kp.shape
    for fmt, tol in (("int8", 0.02), ("fp8", 0.1)):
        codes = [np.zeros((nb, bs, Hkv, d), np.uint8) for _ in range(2)]
        scales = [np.full((nb, Hkv, bs, 2), np.nan, np.float32) for _ in range(2)]
        for src, c, sc in ((kp, codes[0], scales[0]), (vp, codes[1], scales[1])):
            vals = orc.storage_to_f64(src, "bf16")
            for blk in range(nb):
                for off in range(bs):
                    for j in range(Hkv):
                        row = vals[blk, off, j]
                        if np.isnan(row).any():
                            continue
                        q, s, z = orc.quantize_row(row, fmt)
                        c[blk, off, j] = q
                        sc[blk, j, off] = (s, z)
        got = orc.paged_decode_attention_quantized(wl.q, codes[0], codes[1], scales[0],
                                                   scales[1], wl.block_tables,
                                                   wl.context_lens, 16, wl.scale, fmt, "bf16")
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < tol, (fmt, rel)


def test_planted_zero_point_sign_error_is_caught(monkeypatch):
    """A dequantizer that adds z instead of subtracting it fails the library pin."""
    wl = wlm.make_workload(wlm.QUANT_SMALL_SPECS["int8"], seed=4)
    kc, vc, ks, vs = orc.kv_append_quantized(wl.k_pool, wl.v_pool, wl.k_scales, wl.v_scales,
                                             wl.k_new, wl.v_new, wl.block_tables,
                                             wl.positions, 16, "int8", wl.dtype)
    ref = _sdpa_dequantized(wl, kc, vc, ks, vs, "int8")
    real = orc.dequantize
    monkeypatch.setattr(orc, "dequantize", lambda c, s, z, f: real(c, s, -np.asarray(z), f))
    got = orc.paged_decode_attention_quantized(wl.q, kc, vc, ks, vs, wl.block_tables,
                                               wl.context_lens, 16, wl.scale, "int8", wl.dtype)
    assert not within(got, ref, "bf16")[0]


def test_int8_zero_point_is_positive_zero():
    """A row without negative values has lo = 0 and z = 0, stored as +0 (bit pattern 0)."""
    _, s, z = orc.quantize_row(np.float32([0.5, 1.0, 2.0]), "int8")
    assert np.float32(z).view(np.uint32) == 0
