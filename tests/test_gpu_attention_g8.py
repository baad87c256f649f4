"""Decode attention over compressed caches with 8-token exponent groups in 64-token blocks (GAAC
page §3.1: exponents coded in groups of eight; §3.2: compressed, raw and tail tokens attended in
one softmax, the values rebuilt on chip).  These caches take a split kernel that rebuilds whole
8-token CODE units in registers.  Its results match the oracle's exact fp64 attention within
4e-3 per (sequence, query head) row.  The kernel adds the same per-split sequence of MFMA
contractions and softmax updates whether a tile is compressed or stored raw, so caches of the
same tokens give the same bits whatever form their tiles take."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import dev, host, new_cache, row_rel_err

pytestmark = pytest.mark.gpu

TOL = 4e-3


def _cache(cfg, L, esc_cap=-1, fmt=oracle.BF16, max_seqs=1):
    return new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=64, max_seqs=max_seqs, max_blocks=L // 64 + 2,
                     esc_cap=esc_cap, fmt=fmt, Gt=8)


def _filled(cfg, k, v, L, esc_cap=-1, fmt=oracle.BF16):
    c = _cache(cfg, L, esc_cap, fmt)
    c.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
    c.append([0], dev(k[None, :L], fmt), dev(v[None, :L], fmt))
    return c


@pytest.mark.parametrize("cfg_i", [0, 1])
def test_g8_tile_forms_give_the_same_bits(cfg_i):
    """BF16, 8-token groups, 64-token blocks: all tiles compressed, many tiles raw (a 16-byte
    escape capacity) and every tile raw (no escape capacity) give bit-identical outputs for
    lengths with tails of 0, 1 and 63 tokens and 1 to 256 splits; against the oracle."""
    cfg = dataclasses.replace(synth.config(cfg_i), G=8, T=64)
    print(f"[g8 forms] cfg{cfg_i} D={cfg.D} Hq={cfg.Hq}", flush=True)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    raw_seen = 0
    for L in (63, 256, 257, 1000, 4097):
        q = synth.queries(cfg, step=L)
        outs = []
        for esc_cap in (-1, 16, 0):
            c = _filled(cfg, k, v, L, esc_cap)
            st = c.status()[1]
            if esc_cap == 16:
                raw_seen += st["raw_tiles"]
            if esc_cap == 0 and L >= 64:
                assert st["raw_tiles"] > 0
            outs.append([host(c.attention([0], dev(q), cfg.scale, S)) for S in (1, 3, 16, 256)])
            assert c.status()[0] == 0
        ref = oracle.attention(oracle.BF16, q[0], k[:L], v[:L], cfg.scale)
        assert row_rel_err(outs[0][0][0], ref) <= TOL, L
        for S_i in range(4):
            assert np.array_equal(outs[0][S_i], outs[1][S_i]), (L, S_i, "raw fallbacks")
            assert np.array_equal(outs[0][S_i], outs[2][S_i]), (L, S_i, "all raw")
    assert raw_seen > 0


@pytest.mark.parametrize("fmt", [oracle.E5M2, oracle.E4M3])
def test_g8_fp8_head_dim_128(fmt):
    """FP8 caches with 8-token groups at 128 channels and four query heads per KV head: against
    the oracle, and bit-identical with a cache whose small escape capacity turns tiles raw."""
    cfg = dataclasses.replace(synth.config(1), G=8, T=64, fmt=fmt)
    print(f"[g8 fp8] fmt={fmt}", flush=True)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    L = 2048 + 37
    q = synth.queries(cfg, step=L)
    ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
    outs = []
    for esc_cap in (-1, 16):
        c = _filled(cfg, k, v, L, esc_cap, fmt)
        if esc_cap == 16:
            assert c.status()[1]["raw_tiles"] > 0
        outs.append([host(c.attention([0], dev(q), cfg.scale, S)) for S in (1, 32)])
        assert c.status()[0] == 0
    for S_i in range(2):
        assert row_rel_err(outs[0][S_i][0], ref) <= TOL, S_i
        assert np.array_equal(outs[0][S_i], outs[1][S_i]), S_i


def test_g8_full_context_all_heads():
    """The 64K-token Qwen3-8B-like layer with 8-token groups at 256 splits, all 32 query heads
    against the oracle; then 27 single-token appends and the same again."""
    cfg = dataclasses.replace(synth.config(2), G=8)
    print("[g8 64k] all heads", flush=True)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    L = k.shape[0]
    kn, vn = g.tokens(27)
    q = synth.queries(cfg)
    q2 = synth.queries(cfg, step=27)
    c = _filled(cfg, k, v, L)
    out = host(c.attention([0], dev(q), cfg.scale, 256))
    assert row_rel_err(out[0], oracle.attention(oracle.BF16, q[0], k, v, cfg.scale)) <= TOL
    for i in range(27):
        c.append([0], dev(kn[None, i:i + 1]), dev(vn[None, i:i + 1]))
    out = host(c.attention([0], dev(q2), cfg.scale, 256))
    ref = oracle.attention(oracle.BF16, q2[0], np.concatenate([k, kn]), np.concatenate([v, vn]), cfg.scale)
    assert row_rel_err(out[0], ref) <= TOL
    assert c.status()[0] == 0
    del c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.E4M3])
def test_g8_decode_step_equals_append_then_attention(fmt):
    """kv_decode_step on 64-token blocks with 8-token groups (the split kernel stores the new token
    into the tail, the merge attends it; a block-completing step appends, then attends) gives the
    bits of kv_encode_append followed by kv_decode_attention for three sequences at different
    tail positions, across block boundaries; the final state matches the oracle."""
    cfg = dataclasses.replace(synth.config(0), G=8, T=64, fmt=fmt)
    print(f"[g8 step] fmt={fmt}", flush=True)
    lg = synth.LayerGen(cfg)
    starts = [61, 133, 1]
    toks = [lg.tokens(L0 + 70) for L0 in starts]
    caches = []
    for _ in range(2):
        c = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=64, max_seqs=3, max_blocks=5, fmt=fmt, Gt=8)
        c.calibrate(dev(toks[0][0][:cfg.n_cal], fmt), dev(toks[0][1][:cfg.n_cal], fmt))
        for sid, (k, v) in enumerate(toks):
            c.append([sid], dev(k[None, :starts[sid]], fmt), dev(v[None, :starts[sid]], fmt))
        caches.append(c)
    step_cache, ref_cache = caches
    ids = [2, 0, 1]
    for st in range(70):
        kn = np.stack([toks[s][0][starts[s] + st] for s in ids])[:, None]
        vn = np.stack([toks[s][1][starts[s] + st] for s in ids])[:, None]
        q = dev(synth.queries(cfg, step=st)[:1].repeat(3, axis=0))
        a = step_cache.decode_step(ids, dev(kn, fmt), dev(vn, fmt), q, cfg.scale, 3)
        ref_cache.append(ids, dev(kn, fmt), dev(vn, fmt))
        b = ref_cache.attention(ids, q, cfg.scale, 3)
        assert np.array_equal(host(a), host(b)), st
    qh = synth.queries(cfg, step=99)
    out = host(step_cache.attention(ids, dev(qh[:1].repeat(3, axis=0)), cfg.scale, 2))
    for row, s in enumerate(ids):
        L = starts[s] + 70
        ref = oracle.attention(fmt, qh[0], toks[s][0][:L], toks[s][1][:L], cfg.scale)
        assert row_rel_err(out[row], ref) <= TOL, s
    assert step_cache.status()[0] == 0


@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.E5M2])
def test_g8_gqa_group_of_16(fmt):
    """Sixteen query heads per KV head (every row of the 16-row MFMA tiles a real head), 128
    channels, a ragged length with a tail, split counts 1 and 7; against the oracle."""
    cfg = dataclasses.replace(synth.config(0), fmt=fmt, G=8, T=64, Hkv=1, Hq=16, D=128)
    print(f"[g8 gqa16] fmt={fmt}", flush=True)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    L = 1000
    c = _filled(cfg, k, v, L, fmt=fmt)
    q = synth.queries(cfg, step=L)
    ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
    for S in (1, 7):
        out = host(c.attention([0], dev(q), cfg.scale, S))
        assert row_rel_err(out[0], ref) <= TOL, S
    assert c.status()[0] == 0
