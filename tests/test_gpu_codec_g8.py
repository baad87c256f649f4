"""GPU codec parity for 8-token exponent groups (GAAC page §3.1 codes the exponents of small
groups of eight values; the attention path uses 16-token groups): encoded slot bytes, escape
lengths in the block table, rebuilt tensors and tile statistics are bit-exact against the
oracle for BF16, E5M2 and E4M3 at T = 64 and T = 16.  Decode attention over compressed caches
with 8-token groups (GAAC page §3.2; blocks rebuilt into LDS) matches the oracle's fp64
attention within 4e-3 per row, and its decode step matches append + attention bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
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
    assert st["groups"][:3] == want.tolist() and st["groups"][3] == 0 and st["esc_bytes"] == esc


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


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [16, 32, 64])
def test_g8_compressed_attention_matches_oracle(fmt, T):
    """Decode attention over caches with 8-token groups (the kernel that rebuilds each block's
    tiles into LDS): lengths ending before the first block, just past a block and inside one,
    split counts 1 to 64, and a small escape capacity that turns tiles raw; against the oracle's
    exact fp64 attention over the stored values."""
    cfg = _cfg(fmt, T)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    for esc_cap in (-1, 16):
        cache, _ = _fill(cfg, CHUNKS[1], esc_cap=esc_cap)
        if esc_cap == 16:
            assert cache.status()[1]["raw_tiles"] > 0
        for L in (T - 1, 4 * T + 1, 1000, 1024):
            sub = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=T, max_seqs=1, max_blocks=L // T + 2,
                            esc_cap=esc_cap, fmt=fmt, Gt=8) if L != 1024 else cache
            if L != 1024:
                sub.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
                sub.append([0], dev(k[None, :L], fmt), dev(v[None, :L], fmt))
            q = synth.queries(cfg, step=L)
            ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
            for S in (1, 3, 64):
                out = host(sub.attention([0], dev(q), cfg.scale, S))
                assert row_rel_err(out[0], ref) <= 4e-3, (esc_cap, L, S)
    assert cache.status()[0] == 0


def test_g8_head_dim_128_and_gqa_group_of_4():
    """The 8-token-group kernel at D = 128 with four query heads per KV head (the benchmark
    geometry at a 2,048-token context)."""
    cfg = dataclasses.replace(synth.config(1), G=8)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    L = 2048
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=1, max_blocks=L // cfg.T + 2, Gt=8)
    cache.calibrate(dev(k[:cfg.n_cal]), dev(v[:cfg.n_cal]))
    cache.append([0], dev(k[None, :L - 5]), dev(v[None, :L - 5]))
    for t in range(L - 5, L):
        cache.append([0], dev(k[None, t:t + 1]), dev(v[None, t:t + 1]))
    q = synth.queries(cfg, step=L)
    out = host(cache.attention([0], dev(q), cfg.scale, 32))
    assert row_rel_err(out[0], oracle.attention(oracle.BF16, q[0], k[:L], v[:L], cfg.scale)) <= 4e-3


@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.E4M3])
def test_g8_gqa_group_of_16_at_32_token_blocks(fmt):
    """Sixteen query heads per KV head (every row of the kernel's 16-row MFMA tiles a real head),
    128 channels, 32-token blocks (two of the four waves score each block), a ragged length and
    a tail; against the oracle."""
    cfg = dataclasses.replace(synth.config(0), fmt=fmt, G=8, T=32, Hkv=1, Hq=16, D=128)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    L = 1000
    cache = new_cache(Hkv=1, Hq=16, D=128, T=32, max_seqs=1, max_blocks=L // 32 + 2, fmt=fmt, Gt=8)
    cache.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
    cache.append([0], dev(k[None, :L], fmt), dev(v[None, :L], fmt))
    q = synth.queries(cfg, step=L)
    ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
    for S in (1, 7):
        out = host(cache.attention([0], dev(q), cfg.scale, S))
        assert row_rel_err(out[0], ref) <= 4e-3, S
    assert cache.status()[0] == 0


@pytest.mark.parametrize("fmt", FMTS)
def test_g8_decode_step_equals_append_then_attention(fmt):
    """kv_decode_step (the kernel stores the new token into the tail, the merge attends it) gives
    the bits of kv_encode_append followed by kv_decode_attention, across a block completion
    (T = 16: tokens 1022..1025), and matches the oracle."""
    cfg = _cfg(fmt, 16)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    a, _ = _fill(cfg, [(0, 1020)])
    b, _ = _fill(cfg, [(0, 1020)])
    for t in range(1020, 1024):
        q = dev(synth.queries(cfg, step=t))
        kn, vn = dev(k[None, t:t + 1], fmt), dev(v[None, t:t + 1], fmt)
        out_a = host(a.decode_step([0], kn, vn, q, cfg.scale, 8))
        b.append([0], kn, vn)
        out_b = host(b.attention([0], q, cfg.scale, 8))
        assert np.array_equal(out_a, out_b), t
        ref = oracle.attention(fmt, synth.queries(cfg, step=t)[0], k[:t + 1], v[:t + 1], cfg.scale)
        assert row_rel_err(out_a[0], ref) <= 4e-3, t
    assert a.seq_length(0) == 1024 and a.status()[0] == 0


def test_g8_uncompressed_cache_attends():
    cfg = _cfg(oracle.BF16, 64)
    cache, toks = _fill(cfg, [(0, 1000)], compressed=False)
    k0, v0 = toks[0]
    q = synth.queries(cfg)
    out = host(cache.attention([0], dev(q), cfg.scale, 4))
    ref = oracle.attention(oracle.BF16, q[0], k0[:1000], v0[:1000], cfg.scale)
    assert row_rel_err(out[0], ref) <= 4e-3
