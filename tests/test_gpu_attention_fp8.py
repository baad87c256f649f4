"""GPU decode attention over FP8 caches through the C ABI (GAAC page App. B with §3.2): the
kernel rebuilds the FP8 elements of compressed tiles, converts them exactly to BF16 and
accumulates in fp32.  The bar is the same as for BF16 caches: per (sequence, query head) row,
max_c |o - r| / max_c |r| <= 4e-3 against the oracle's exact fp64 attention over the FP8
values."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import dev, host, new_cache, row_rel_err

pytestmark = pytest.mark.gpu

TOL = 4e-3
FMTS = [oracle.E5M2, oracle.E4M3]


def _fill(cfg, toks, compressed=True, chunks=None, esc_cap=-1, perm_seed=0, max_blocks=None):
    L = max(k.shape[0] for k, _ in toks)
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=len(toks),
                      max_blocks=max_blocks or (L // cfg.T + 2), compressed=compressed, esc_cap=esc_cap,
                      perm_seed=perm_seed, fmt=cfg.fmt)
    k0, v0 = toks[0]
    cache.calibrate(dev(k0[:cfg.n_cal], cfg.fmt), dev(v0[:cfg.n_cal], cfg.fmt))
    for sid, (k, v) in enumerate(toks):
        for a, b in (chunks or [(0, k.shape[0])]):
            b = min(b, k.shape[0])
            if a < b:
                cache.append([sid], dev(k[None, a:b], cfg.fmt), dev(v[None, a:b], cfg.fmt))
    return cache


def _oracle(cfg, toks, q, heads=None):
    out = []
    g = cfg.Hq // cfg.Hkv
    for sid, (k, v) in enumerate(toks):
        if heads is None:
            out.append(oracle.attention(cfg.fmt, q[sid], k, v, cfg.scale))
        else:
            rows = [oracle.attention(cfg.fmt, q[sid][hq:hq + 1], k[:, hq // g:hq // g + 1], v[:, hq // g:hq // g + 1],
                                     cfg.scale)[0] for hq in heads]
            out.append(np.stack(rows))
    return np.stack(out)


def _cfg0(fmt):
    return dataclasses.replace(synth.config(0), fmt=fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("compressed", [True, False])
@pytest.mark.parametrize("S", [1, 3, 16])
def test_fp8_cfg0_matches_oracle(fmt, compressed, S):
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    cache = _fill(cfg, toks, compressed)
    q = synth.queries(cfg)
    out = cache.attention([0], dev(q), cfg.scale, S)
    err = row_rel_err(host(out), _oracle(cfg, toks, q))
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("L", [1, 17, 64, 65, 200, 1024])
def test_fp8_ragged_lengths_and_tail(fmt, L):
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    k, v = k[:L], v[:L]
    chunks = [(0, max(L - 3, 0))] + [(i, i + 1) for i in range(max(L - 3, 0), L)]
    q = synth.queries(cfg, step=L)
    ref = _oracle(cfg, [(k, v)], q)
    for compressed in (True, False):
        cache = _fill(cfg, [(k, v)], compressed, chunks=chunks, max_blocks=17)
        for S in (1, 4):
            err = row_rel_err(host(cache.attention([0], dev(q), cfg.scale, S)), ref)
            assert err <= TOL, (compressed, S, err)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_single_token_returns_its_value(fmt):
    """One cached token: the output is that token's V converted to BF16, exactly."""
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    cache = _fill(cfg, [(k[:1], v[:1])])
    out = host(cache.attention([0], dev(synth.queries(cfg)), cfg.scale, 2))
    want = synth.f32_to_bf16_bits(oracle.values(fmt, v[0]).astype(np.float32))
    for hq in range(cfg.Hq):
        assert np.array_equal(out[0, hq], want[hq // 2])


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_raw_fallback_tiles(fmt):
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    cache = _fill(cfg, toks, esc_cap=96 if fmt == oracle.E5M2 else 64)  # about 40 of 64 tiles raw
    flags, st = cache.status()
    assert st["raw_tiles"] > 0 and st["comp_tiles"] > 0
    q = synth.queries(cfg, step=5)
    assert row_rel_err(host(cache.attention([0], dev(q), cfg.scale, 4)), _oracle(cfg, toks, q)) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_paged_t16_permuted_pool(fmt):
    cfg = dataclasses.replace(synth.config(3), fmt=fmt)
    g = synth.LayerGen(cfg)
    lens = [1, 100, 1000, 2049]
    toks = [g.tokens(L) for L in lens]
    cache = _fill(cfg, toks, perm_seed=5, max_blocks=2049 // 16 + 2)
    q = synth.queries(dataclasses.replace(cfg, n_seqs=len(lens)), step=2)
    out = cache.attention(list(range(len(lens))), dev(q), cfg.scale, 8)
    assert row_rel_err(host(out), _oracle(cfg, toks, q)) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_full_context_all_heads(fmt):
    """The 64K-token layer in FP8 (compressed and uncompressed) at the benchmark's split count,
    all 32 query heads against the oracle."""
    cfg = synth.config(4, fmt)
    g, toks = synth.sequence_tokens(cfg)
    q = synth.queries(cfg)
    ref = _oracle(cfg, toks, q)
    for compressed in (True, False):
        cache = _fill(cfg, toks, compressed)
        out = host(cache.attention([0], dev(q), cfg.scale, 256))
        assert row_rel_err(out, ref) <= TOL, compressed
        del cache
        torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_decode_step_equals_append_then_attention(fmt):
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    kx, vx = g.tokens(40)  # the stream continues past the configured 1,024 tokens
    k, v = np.concatenate([toks[0][0], kx]), np.concatenate([toks[0][1], vx])
    L0 = 1000
    caches = [_fill(cfg, [(k[:L0], v[:L0])], max_blocks=18) for _ in range(2)]
    for st in range(40):  # crosses the block boundary at 1024
        kn, vn = dev(k[None, L0 + st:L0 + st + 1], fmt), dev(v[None, L0 + st:L0 + st + 1], fmt)
        q = dev(synth.queries(cfg, step=st))
        a = caches[0].decode_step([0], kn, vn, q, cfg.scale, 4)
        caches[1].append([0], kn, vn)
        b = caches[1].attention([0], q, cfg.scale, 4)
        assert np.array_equal(host(a), host(b)), st
    q = synth.queries(cfg, step=77)
    ref = _oracle(cfg, [(k[:L0 + 40], v[:L0 + 40])], q)
    assert row_rel_err(host(caches[0].attention([0], dev(q), cfg.scale, 4)), ref) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [16, 64])
def test_fp8_compressed_and_uncompressed_caches_give_the_same_bits(fmt, T):
    """Lossless end to end for FP8 caches (GAAC page App. B with §3.2): compressed tiles, raw
    fallback tiles (a small escape capacity) and an uncompressed cache of the same tokens give
    bit-identical outputs; split counts 1 to 256."""
    cfg = _cfg0(fmt)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    raw_seen = 0
    for L in (T - 1, 4 * T + 1, 1000):
        kk, vv = k[:L], v[:L]
        q = dev(synth.queries(cfg, step=L))
        outs = []
        for compressed, esc_cap in ((True, -1), (True, 16), (False, -1)):
            cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=T, max_seqs=1, max_blocks=L // T + 2,
                              compressed=compressed, esc_cap=esc_cap, fmt=fmt)
            cache.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
            cache.append([0], dev(kk[None], fmt), dev(vv[None], fmt))
            if compressed and esc_cap == 16:
                raw_seen += cache.status()[1]["raw_tiles"]
            outs.append([host(cache.attention([0], q, cfg.scale, S)) for S in (1, 3, 16, 256)])
        assert row_rel_err(outs[2][0], _oracle(cfg, [(kk, vv)], synth.queries(cfg, step=L))) <= TOL, L
        for S_i in range(4):
            assert np.array_equal(outs[0][S_i], outs[2][S_i]), (L, S_i, "compressed")
            assert np.array_equal(outs[1][S_i], outs[2][S_i]), (L, S_i, "raw fallbacks")
    assert raw_seen > 0
