"""Pins for the oracle's exact decode attention and element values.

Attention is softmax(scale * q.K^T) V in fp64 over every cached token (compressed blocks, raw
blocks and the uncompressed tail in one normalisation: GAAC page, §3.2).  Pinned by closed
forms, by torch's own scaled-dot-product attention in float64 (a library routine), and by the
lossless invariant: attention on the decoded cache equals attention on the original cache.
"""
import numpy as np
import pytest
import torch

import synth


def test_bf16_values_match_torch(orc):
    bits = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.values(orc.BF16, bits)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


@pytest.mark.parametrize("fmt,tdt", [(1, torch.float8_e5m2), (2, torch.float8_e4m3fn)])
def test_fp8_values_match_torch(orc, fmt, tdt):
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(tdt).to(torch.float64).numpy()
    got = orc.values(fmt, bits.astype(np.uint16))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def _rand_bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def test_single_token_returns_its_value(orc):
    rng = np.random.default_rng(0)
    q = _rand_bf16(rng, (4, 64))
    k = _rand_bf16(rng, (1, 2, 64))
    v = _rand_bf16(rng, (1, 2, 64))
    o = orc.attention(orc.BF16, q, k, v, 0.125)
    for hq in range(4):
        assert np.array_equal(o[hq], _f(v[0, hq // 2]))


def test_zero_query_or_zero_scale_gives_mean_of_values(orc):
    rng = np.random.default_rng(1)
    k = _rand_bf16(rng, (37, 2, 64), 3.0)
    v = _rand_bf16(rng, (37, 2, 64))
    q0 = np.zeros((4, 64), np.uint16)
    o = orc.attention(orc.BF16, q0, k, v, 0.125)
    for hq in range(4):
        np.testing.assert_allclose(o[hq], _f(v[:, hq // 2]).mean(axis=0), rtol=0, atol=1e-14)
    q = _rand_bf16(rng, (4, 64))
    o = orc.attention(orc.BF16, q, k, v, 0.0)
    for hq in range(4):
        np.testing.assert_allclose(o[hq], _f(v[:, hq // 2]).mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value(orc):
    rng = np.random.default_rng(2)
    L, D = 50, 64
    k = _rand_bf16(rng, (L, 1, D), 0.01)
    v = _rand_bf16(rng, (L, 1, D))
    q = _rand_bf16(rng, (1, D))
    k[17, 0] = synth.f32_to_bf16_bits(_f(q[0]).astype(np.float32) * 8.0)
    o = orc.attention(orc.BF16, q, k, v, 1.0)
    np.testing.assert_allclose(o[0], _f(v[17, 0]), rtol=0, atol=1e-9)


def test_gqa_heads_with_equal_query_are_identical(orc):
    rng = np.random.default_rng(3)
    k = _rand_bf16(rng, (90, 2, 64))
    v = _rand_bf16(rng, (90, 2, 64))
    q = _rand_bf16(rng, (8, 64))
    q[1] = q[0]
    q[7] = q[4]
    o = orc.attention(orc.BF16, q, k, v, 0.125)
    assert np.array_equal(o[0], o[1]) and np.array_equal(o[4], o[7])
    assert not np.array_equal(o[0], o[4])


@pytest.mark.parametrize("L,Hkv,Hq,D", [(1, 1, 1, 64), (17, 2, 4, 64), (203, 2, 8, 128), (64, 8, 32, 128)])
def test_matches_torch_sdpa_float64(orc, L, Hkv, Hq, D):
    rng = np.random.default_rng(L + Hq)
    k = _rand_bf16(rng, (L, Hkv, D), 2.0)
    v = _rand_bf16(rng, (L, Hkv, D))
    q = _rand_bf16(rng, (Hq, D))
    scale = 1.0 / np.sqrt(D)
    o = orc.attention(orc.BF16, q, k, v, scale)
    g = Hq // Hkv
    qt = torch.from_numpy(_f(q)).reshape(1, Hq, 1, D)
    kt = torch.from_numpy(_f(k)).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, Hq, L, D)
    vt = torch.from_numpy(_f(v)).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, Hq, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale).reshape(Hq, D).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_token_order_does_not_matter(orc):
    rng = np.random.default_rng(4)
    k = _rand_bf16(rng, (77, 2, 64))
    v = _rand_bf16(rng, (77, 2, 64))
    q = _rand_bf16(rng, (4, 64))
    perm = rng.permutation(77)
    a = orc.attention(orc.BF16, q, k, v, 0.125)
    b = orc.attention(orc.BF16, q, k[perm], v[perm], 0.125)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_fp8_attention_uses_fp8_values(orc):
    rng = np.random.default_rng(6)
    kb = _rand_bf16(rng, (40, 1, 64))
    vb = _rand_bf16(rng, (40, 1, 64))
    q = _rand_bf16(rng, (2, 64))
    for fmt, tdt in ((1, torch.float8_e5m2), (2, torch.float8_e4m3fn)):
        k8 = synth.bf16_bits_to_fp8_bits(kb, fmt)
        v8 = synth.bf16_bits_to_fp8_bits(vb, fmt)
        o = orc.attention(fmt, q, k8, v8, 0.125)
        kf = torch.from_numpy(k8.astype(np.uint8)).view(tdt).to(torch.float64)
        vf = torch.from_numpy(v8.astype(np.uint8)).view(tdt).to(torch.float64)
        qt = torch.from_numpy(_f(q)).reshape(1, 2, 1, 64)
        kt = kf.permute(1, 0, 2).repeat_interleave(2, dim=0).reshape(1, 2, 40, 64)
        vt = vf.permute(1, 0, 2).repeat_interleave(2, dim=0).reshape(1, 2, 40, 64)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.125).reshape(2, 64).numpy()
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_lossless_invariant_on_cfg0(orc):
    """Attention over the decoded compressed cache equals attention over the original cache,
    bit for bit (decoding is exact)."""
    cfg = synth.config(0)
    g, seqs = synth.sequence_tokens(cfg)
    k, v = seqs[0]
    p = orc.Params(orc.BF16, cfg.T, cfg.D, cfg.G)
    s = orc.Sequence(p, cfg.Hkv, orc.calibrate_layer(p, k[:256], v[:256]))
    s.append(k[:1000], v[:1000])
    s.append(k[1000:], v[1000:])
    kd, vd = s.decoded()
    q = synth.queries(cfg)[0]
    a = orc.attention(orc.BF16, q, k, v, cfg.scale)
    b = orc.attention(orc.BF16, q, kd, vd, cfg.scale)
    assert np.array_equal(a, b)


# ---- exponent concentration (§3.1) ---------------------------------------------------------

def test_window_coverage_pins(orc):
    """The best window of w consecutive exponents, pinned by a different algorithm (a two-pointer
    sweep over the sorted exponents) and by closed forms: w = 2^F covers every token, equal
    exponents are covered by any window, w = 1 is the largest histogram bin."""
    rng = np.random.default_rng(3)
    for fmt, F, MB in ((orc.BF16, 8, 7), (orc.E5M2, 5, 2), (orc.E4M3, 4, 3)):
        p = orc.Params(fmt, 16, 32, 16, esc_cap=0)
        e = np.clip(rng.normal(rng.integers(2, (1 << F) - 2, 32), rng.uniform(0.3, 4, 32), (300, 32)), 0,
                    (1 << F) - 1).astype(np.uint16)
        x = np.ascontiguousarray(e << MB)
        for w in (1, 2, 6, 8, 16, 1 << F):
            if w > (1 << F):
                continue
            got = orc.window_coverage(p, x, w)
            for c in range(32):
                s = np.sort(e[:, c].astype(np.int64))
                best, lo = 0, 0
                for hi in range(len(s)):      # largest run of sorted values within w consecutive ones
                    while s[hi] - s[lo] >= w:
                        lo += 1
                    best = max(best, hi - lo + 1)
                assert got[c] == best, (fmt, w, c)
            if w == (1 << F):
                assert (got == 300).all()
            if w == 1:
                assert all(got[c] == np.bincount(e[:, c]).max() for c in range(32))
        same = np.ascontiguousarray(np.full((50, 32), 3 << MB, np.uint16))
        assert (orc.window_coverage(p, same, 2) == 50).all()

