"""GPU codec parity for FP8 caches through the C ABI (GAAC page App. B: the same base-plus-offset
codec over FP8 E5M2 and E4M3 exponent fields): calibrated bases, encoded bytes and rebuilt
tensors are bit-exact against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import compare_tiles, dev, host, new_cache, oracle_layer

pytestmark = pytest.mark.gpu

FMTS = [oracle.E5M2, oracle.E4M3]


def _small_cfg(fmt):
    return dataclasses.replace(synth.config(0), fmt=fmt)


def _fill(cfg, chunks, esc_cap=-1, compressed=True):
    g, toks = synth.sequence_tokens(cfg)
    L = max(cfg.context)
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=cfg.n_seqs, max_blocks=L // cfg.T + 2,
                      compressed=compressed, esc_cap=esc_cap, fmt=cfg.fmt)
    k0, v0 = toks[0]
    cache.calibrate(dev(k0[:cfg.n_cal], cfg.fmt), dev(v0[:cfg.n_cal], cfg.fmt))
    for a, b in chunks:
        for sid, (k, v) in enumerate(toks):
            if a < min(b, k.shape[0]):
                cache.append([sid], dev(k[None, a:b], cfg.fmt), dev(v[None, a:b], cfg.fmt))
    torch.cuda.synchronize()
    return cache, toks


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_calibration_matches_oracle(fmt):
    cfg = synth.config(4, fmt)
    k, v = synth.LayerGen(cfg).tokens(256)
    cache = new_cache(Hkv=8, Hq=32, D=128, T=64, max_seqs=1, max_blocks=4, fmt=fmt)
    cache.calibrate(dev(k, fmt), dev(v, fmt))
    got = cache.bases().cpu().numpy()
    b3, b4 = oracle.calibrate_layer(oracle.Params(fmt, 64, 128, 16), k, v)
    assert np.array_equal(got[:, 0], b3) and np.array_equal(got[:, 1], b4)
    if fmt == oracle.E4M3:
        assert not got[:, 1].any()  # no 16-wide window in a 4-bit exponent field


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("chunks", [[(0, 1024)], [(0, 100), (100, 101), (101, 700), (700, 1024)]])
def test_fp8_encode_bytes_and_decode(fmt, chunks):
    cfg = _small_cfg(fmt)
    cache, toks = _fill(cfg, chunks)
    p = oracle.Params(fmt, cfg.T, cfg.D, cfg.G)
    k0, v0 = toks[0]
    bases, oseqs = oracle_layer(p, cfg.Hkv, k0[:cfg.n_cal], v0[:cfg.n_cal], toks, chunks)
    assert compare_tiles(cache, p, oseqs, [0]) == 16 * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, 16)
    assert kd.dtype == torch.uint8
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)
    flags, st = cache.status()
    assert flags == 0
    ost = oracle.stats(p, oseqs)
    assert st["raw_tiles"] == ost["raw_tiles"]


@pytest.mark.parametrize("fmt", FMTS)
def test_every_fp8_pattern(fmt):
    """All 256 patterns in sorted, shuffled and repeated (one exponent per group) arrangements,
    including zeros, subnormals and Inf/NaN codes: byte-identical to the oracle, and decoded
    back unchanged, with the default and with zero escape capacity."""
    rng = np.random.default_rng(11)
    allp = np.arange(256, dtype=np.uint16)
    sorted_ = np.tile(allp, 128).reshape(256, 128)                  # 256 tokens x 128 channels
    shuffled = np.concatenate([rng.permutation(allp) for _ in range(128)]).reshape(256, 128)
    t, c = np.meshgrid(np.arange(256), np.arange(128), indexing="ij")
    grouped = (((t // 16) * 128 + c) % 256).astype(np.uint16)       # each 16-token group one pattern
    toks = np.ascontiguousarray(np.concatenate([sorted_, shuffled, grouped])[:, None, :])  # [768][1][128]
    for esc_cap in (-1, 0):
        cache = new_cache(Hkv=1, Hq=1, D=128, T=64, max_seqs=1, max_blocks=toks.shape[0] // 64, esc_cap=esc_cap,
                          fmt=fmt)
        cache.calibrate(dev(toks[:256], fmt), dev(toks[:256], fmt))
        cache.append([0], dev(toks[None], fmt), dev(toks[None], fmt))
        p = oracle.Params(fmt, 64, 128, 16, esc_cap=None if esc_cap < 0 else esc_cap)
        _, oseqs = oracle_layer(p, 1, toks[:256], toks[:256], [(toks, toks)])
        compare_tiles(cache, p, oseqs, [0])
        kd, vd = cache.decode_blocks(0, 0, toks.shape[0] // 64)
        assert np.array_equal(host(kd), toks) and np.array_equal(host(vd), toks)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_uncompressed_cache_is_raw_bytes(fmt):
    cfg = _small_cfg(fmt)
    cache, toks = _fill(cfg, [(0, 1000)], compressed=False)
    flags, st = cache.status()
    assert st["comp_tiles"] == 0 and st["raw_tiles"] == 15 * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, 15)
    assert np.array_equal(host(kd), toks[0][0][:960]) and np.array_equal(host(vd), toks[0][1][:960])


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_full_context_codec(fmt):
    """The 64K-token layer in FP8: a sample of tiles byte-exact, full decode exact, the same
    raw-tile count as the oracle."""
    cfg = synth.config(4, fmt)
    cache, toks = _fill(cfg, [(0, 65536)])
    p = oracle.Params(fmt, 64, 128, 16)
    k0, v0 = toks[0]
    _, oseqs = oracle_layer(p, 8, k0[:256], v0[:256], toks)
    assert compare_tiles(cache, p, oseqs, [0], sample=1024) == 1024
    kd, vd = cache.decode_blocks(0, 0, 1024)
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)
    flags, st = cache.status()
    ost = oracle.stats(p, oseqs)
    assert flags == 0 and st["raw_tiles"] == ost["raw_tiles"]
