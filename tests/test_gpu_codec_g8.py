"""GPU codec parity for 8-token exponent groups (GAAC page §3.1 codes the exponents of small
groups of eight values; the attention path uses 16-token groups): encoded slot bytes, escape
lengths in the block table, rebuilt tensors and tile statistics are bit-exact against the
oracle for BF16, E5M2 and E4M3 at T = 64 and T = 16.  Decode attention over a compressed cache
with 8-token groups is refused before anything runs; an uncompressed one attends normally."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from decode_attention_calibrate_amd._lib import KVCError
from kvtest import compare_tiles, dev, host, new_cache, oracle_layer, row_rel_err

pytestmark = pytest.mark.gpu

FMTS = [oracle.BF16, oracle.E5M2, oracle.E4M3]
CHUNKS = [[(0, 1024)], [(0, 100), (100, 101), (101, 700), (700, 1024)]]


def _cfg(fmt, T):
    return dataclasses.replace(synth.config(0), fmt=fmt, G=8, T=T)


def _fill(cfg, chunks, esc_cap=-1, compressed=True):
    g, toks = synth.sequence_tokens(cfg)
    L = max(cfg.context)
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=cfg.n_seqs, max_blocks=L // cfg.T + 2,
                      compressed=compressed, esc_cap=esc_cap, fmt=cfg.fmt, Gt=cfg.G)
    k0, v0 = toks[0]
    cache.calibrate(dev(k0[:cfg.n_cal], cfg.fmt), dev(v0[:cfg.n_cal], cfg.fmt))
    for a, b in chunks:
        for sid, (k, v) in enumerate(toks):
            if a < min(b, k.shape[0]):
                cache.append([sid], dev(k[None, a:b], cfg.fmt), dev(v[None, a:b], cfg.fmt))
    torch.cuda.synchronize()
    return cache, toks


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [64, 16])
@pytest.mark.parametrize("chunks", CHUNKS)
def test_g8_encode_bytes_decode_and_stats(fmt, T, chunks):
    cfg = _cfg(fmt, T)
    cache, toks = _fill(cfg, chunks)
    p = oracle.Params(fmt, T, cfg.D, 8)
    k0, v0 = toks[0]
    bases, oseqs = oracle_layer(p, cfg.Hkv, k0[:cfg.n_cal], v0[:cfg.n_cal], toks, chunks)
    nb = 1024 // T
    assert compare_tiles(cache, p, oseqs, [0]) == nb * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, nb)
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)
    flags, st = cache.status()
    assert flags == 0
    ost = oracle.stats(p, oseqs)
    assert st["raw_tiles"] == ost["raw_tiles"] and st["comp_tiles"] == ost["tiles"] - ost["raw_tiles"]
    want = np.zeros(3, np.int64)
    esc = 0
    for t in oseqs[0].tiles:
        for kv in range(2):
            for h in range(cfg.Hkv):
                if not t["is_raw"][kv, h]:
                    want += t["modes"][kv, h]
                    esc += int(t["esc"][kv, h])
    assert st["groups"] == want.tolist() and st["esc_bytes"] == esc


def test_g8_every_bf16_pattern_and_escape_capacities():
    """All 65,536 BF16 patterns (sorted, then shuffled) through the 8-token-group encoder and
    decoder at the default, a small and a zero escape capacity: byte-identical to the oracle,
    raw fallback included, and rebuilt unchanged."""
    rng = np.random.default_rng(19)
    allp = np.arange(65536, dtype=np.uint16)
    toks = np.concatenate([allp, rng.permutation(allp)]).reshape(-1, 1, 128)  # 1024 tokens, Hkv = 1
    for esc_cap in (-1, 96, 0):
        cache = new_cache(Hkv=1, Hq=1, D=128, T=64, max_seqs=1, max_blocks=toks.shape[0] // 64, esc_cap=esc_cap, Gt=8)
        cache.calibrate(dev(toks[:256]), dev(toks[:256]))
        cache.append([0], dev(toks[None]), dev(toks[None]))
        p = oracle.Params(oracle.BF16, 64, 128, 8, esc_cap=None if esc_cap < 0 else esc_cap)
        _, oseqs = oracle_layer(p, 1, toks[:256], toks[:256], [(toks, toks)])
        compare_tiles(cache, p, oseqs, [0])
        kd, vd = cache.decode_blocks(0, 0, toks.shape[0] // 64)
        assert np.array_equal(host(kd), toks) and np.array_equal(host(vd), toks)


@pytest.mark.parametrize("fmt", [oracle.E5M2, oracle.E4M3])
def test_g8_every_fp8_pattern(fmt):
    rng = np.random.default_rng(23)
    allp = np.arange(256, dtype=np.uint8)
    toks = np.concatenate([np.tile(allp, 64), rng.permutation(np.tile(allp, 64))]).reshape(-1, 1, 128)  # 256 tokens
    for esc_cap in (-1, 0):
        cache = new_cache(Hkv=1, Hq=1, D=128, T=64, max_seqs=1, max_blocks=4, esc_cap=esc_cap, fmt=fmt, Gt=8)
        cache.calibrate(dev(toks, fmt), dev(toks, fmt))
        cache.append([0], dev(toks[None], fmt), dev(toks[None], fmt))
        p = oracle.Params(fmt, 64, 128, 8, esc_cap=None if esc_cap < 0 else esc_cap)
        _, oseqs = oracle_layer(p, 1, toks, toks, [(toks, toks)])
        compare_tiles(cache, p, oseqs, [0])
        kd, vd = cache.decode_blocks(0, 0, 4)
        assert np.array_equal(host(kd), toks) and np.array_equal(host(vd), toks)


def test_g8_compressed_attention_is_refused_before_anything_runs():
    cfg = _cfg(oracle.BF16, 64)
    cache, toks = _fill(cfg, [(0, 1000)])
    q = dev(synth.queries(cfg))
    with pytest.raises(KVCError) as e:
        cache.attention([0], q, cfg.scale, 4)
    assert e.value.code == -3
    k0, v0 = toks[0]
    with pytest.raises(KVCError) as e:
        cache.decode_step([0], dev(k0[None, 1000:1001]), dev(v0[None, 1000:1001]), q, cfg.scale, 4)
    assert e.value.code == -3
    assert cache.seq_length(0) == 1000


def test_g8_uncompressed_cache_attends():
    cfg = _cfg(oracle.BF16, 64)
    cache, toks = _fill(cfg, [(0, 1000)], compressed=False)
    k0, v0 = toks[0]
    q = synth.queries(cfg)
    out = host(cache.attention([0], dev(q), cfg.scale, 4))
    ref = oracle.attention(oracle.BF16, q[0], k0[:1000], v0[:1000], cfg.scale)
    assert row_rel_err(out[0], ref) <= 4e-3
