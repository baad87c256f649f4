"""GPU causal prefill attention over blocks rebuilt by kv_decode_blocks (GAAC page §3.3 encodes a
prompt's complete blocks during prefill; attending the rebuilt blocks with standard causal
attention is this library's reading) through the C ABI.  Every query row against
the oracle's exact fp64 attention over the tokens up to its position: per (query, head) row,
max_c |o - r| / max_c |r| <= 4e-3."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import dev, host, new_cache, row_rel_err

pytestmark = pytest.mark.gpu

TOL = 4e-3


@pytest.mark.parametrize("cfg_i,D,fmt", [(0, 64, oracle.BF16), (1, 128, oracle.BF16), (0, 256, oracle.BF16),
                                         (0, 64, oracle.E5M2), (0, 128, oracle.E4M3)])
def test_prefill_over_decoded_blocks(cfg_i, D, fmt):
    cfg = dataclasses.replace(synth.config(cfg_i), D=D, fmt=fmt)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    T, n_kv = cfg.T, 4 * cfg.T
    halves = 2 if D == 256 else 1
    n_tiles = (n_kv // T + 1) * 2 * cfg.Hkv * halves
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=D, T=T, max_seqs=1, max_blocks=n_kv // T + 1, comp_slots=n_tiles,
                      raw_slots=n_tiles, fmt=fmt)
    cache.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
    cache.append([0], dev(k[None, :n_kv], fmt), dev(v[None, :n_kv], fmt))
    kd, vd = cache.decode_blocks(0, 0, n_kv // T)
    assert np.array_equal(host(kd), k[:n_kv]) and np.array_equal(host(vd), v[:n_kv])  # lossless
    qall = synth.queries(dataclasses.replace(cfg, n_seqs=n_kv))  # one query set per position
    for n_q in (n_kv, 37, 1):
        q = qall[n_kv - n_q:]
        out = host(cache.prefill_attention(kd, vd, dev(q), cfg.scale))
        for i in range(n_q):
            pos = n_kv - n_q + i
            ref = oracle.attention(fmt, q[i], k[:pos + 1], v[:pos + 1], cfg.scale)
            assert row_rel_err(out[i], ref) <= TOL, (n_q, i)


def test_prefill_single_token_returns_its_value():
    """The first position attends only itself: its output is its own V row, bit for bit."""
    cfg = synth.config(0)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=1, max_blocks=2)
    q = synth.queries(dataclasses.replace(cfg, n_seqs=5))
    out = host(cache.prefill_attention(dev(k[:5]), dev(v[:5]), dev(q), cfg.scale))
    for hq in range(cfg.Hq):
        assert np.array_equal(out[0, hq], v[0, hq // (cfg.Hq // cfg.Hkv)])
