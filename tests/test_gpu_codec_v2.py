"""GPU parity for FORMAT v2, the nested precision modes of the GAAC page (§4.7.2 / Table 4): a 2-bit
mode added to the 3-bit, 4-bit and raw modes (mode set 1), the 3-bit mode removed (mode set 2),
and the v1 modes in the v2 layout (mode set 3).  Through the C ABI: calibrated bases, every
stored tile's bytes and code length against the oracle's FORMAT v2 encoding, every BF16 bit
pattern, raw fallback, statistics, kv_decode_blocks bit for bit, decode attention against the
oracle's exact attention, and decode steps bit-identical to append + attention."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import _stored_tiles, dev, host, new_cache, row_rel_err

pytestmark = pytest.mark.gpu
TOL = 4e-3


def _cache(cfg, T, Gt, ms, max_seqs=1, max_blocks=None, esc_cap=-1, **kw):
    return new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=T, max_seqs=max_seqs,
                     max_blocks=max_blocks or 1024 // T + 2, Gt=Gt, esc_cap=esc_cap, mode_set=ms, **kw)


def _oracle_bases(p, k_cal, v_cal):
    return oracle.v2_calibrate_layer(p, k_cal, v_cal)  # (b2, b3, b4) each [2][Hkv][D]


def _compare_all_tiles(cache, p, ms, bases, toks):
    """Every finished tile of every sequence: stored bytes == the oracle's FORMAT v2 encoding."""
    b2, b3, b4 = bases
    lay = oracle.v2_layout(p, ms)
    jobs = [(sid, blk, kv, h) for sid, (k, _) in enumerate(toks) for blk in range(k.shape[0] // p.T)
            for kv in range(2) for h in range(cache.Hkv)]
    tiles = np.stack([toks[sid][kv][blk * p.T:(blk + 1) * p.T, h] for sid, blk, kv, h in jobs])
    data, is_raw, used, modes = oracle.v2_encode_tiles(
        p, ms, tiles, np.stack([b2[kv, h] for _, _, kv, h in jobs]), np.stack([b3[kv, h] for _, _, kv, h in jobs]),
        np.stack([b4[kv, h] for _, _, kv, h in jobs]), np.array([kv for _, _, kv, _ in jobs], np.int32))
    for n, (job, (raw, units, got)) in enumerate(zip(jobs, _stored_tiles(cache, jobs))):
        assert raw == bool(is_raw[n]), job
        size = lay["raw_bytes"] if raw else lay["stride"]
        assert units == 0, job
        if not np.array_equal(got[:size], data[n, :size]):
            raise AssertionError(f"tile {job} raw={raw}: bytes differ from the oracle")
    return is_raw, used, modes


@pytest.mark.parametrize("ms", [1, 2, 3])
@pytest.mark.parametrize("T,Gt", [(64, 8), (64, 16), (16, 8), (16, 16)])
def test_v2_codec_matches_oracle(ms, T, Gt):
    print(f"[v2 codec] mode set {ms} T={T} G={Gt}", flush=True)
    cfg = synth.config(0)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    c = _cache(cfg, T, Gt, ms)
    c.calibrate(dev(k[:cfg.n_cal]), dev(v[:cfg.n_cal]))
    p = oracle.Params(oracle.BF16, T, cfg.D, Gt)
    bases = _oracle_bases(p, k[:cfg.n_cal], v[:cfg.n_cal])
    got_b = c.bases().cpu().numpy()
    assert np.array_equal(got_b[:, 0], bases[1]) and np.array_equal(got_b[:, 1], bases[2])
    if ms == 1:
        assert np.array_equal(c.bases2().cpu().numpy(), bases[0])
    for a, b in ((0, 300), (300, 301), (301, 1000)):  # a bulk append, a single token, another bulk
        c.append([0], dev(k[None, a:b]), dev(v[None, a:b]))
    L = 1000
    is_raw, used, modes = _compare_all_tiles(c, p, ms, bases, [(k[:L], v[:L])])
    kd, vd = c.decode_blocks(0, 0, L // T)
    assert np.array_equal(host(kd), k[:L // T * T]) and np.array_equal(host(vd), v[:L // T * T])
    flags, st = c.status()
    assert flags == 0
    comp = is_raw == 0
    assert st["raw_tiles"] == int((~comp).sum())
    assert st["groups"] == modes[comp].sum(0).tolist()
    assert st["esc_bytes"] == int(used[comp].sum())


@pytest.mark.parametrize("ms", [1, 2])
def test_v2_every_bf16_pattern(ms):
    """All 65,536 BF16 patterns (±0, subnormals, Inf, NaN payloads) through the v2 encoder and
    decoder: bytes equal the oracle's, blocks decode bit for bit."""
    cfg = synth.config(0)
    allp = np.arange(65536, dtype=np.uint16)
    rng = np.random.default_rng(5)
    pat = rng.permutation(allp).reshape(-1, 2, 64)            # [512 tokens][2 heads][64]
    k, v = pat, np.ascontiguousarray(pat[::-1])
    for Gt in (8, 16):
        c = _cache(cfg, 64, Gt, ms, max_blocks=10)
        c.calibrate(dev(k[:256]), dev(v[:256]))
        c.append([0], dev(k[None]), dev(v[None]))
        p = oracle.Params(oracle.BF16, 64, 64, Gt)
        _compare_all_tiles(c, p, ms, _oracle_bases(p, k[:256], v[:256]), [(k, v)])
        kd, vd = c.decode_blocks(0, 0, 8)
        assert np.array_equal(host(kd), k) and np.array_equal(host(vd), v)


def test_v2_raw_fallback():
    """Tiles whose codes overflow the capacity are stored raw: a block whose K head 0 alternates
    exponents 100 and 130 token by token (every group raw: 8 bits per offset), with no escape
    allowance; attention and decode over the mix are still exact."""
    cfg = synth.config(0)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    k = k.copy()
    rng = np.random.default_rng(3)
    e = np.where(np.arange(64)[:, None] % 2 == 0, 100, 130) * np.ones((64, 64), np.int64)
    k[320:384, 0] = (rng.integers(0, 2, (64, 64)) << 15 | e << 7 | rng.integers(0, 128, (64, 64))).astype(np.uint16)
    for ms in (1, 2):
        c = _cache(cfg, 64, 8, ms, esc_cap=0)
        c.calibrate(dev(k[:256]), dev(v[:256]))
        c.append([0], dev(k[None, :1000]), dev(v[None, :1000]))
        p = oracle.Params(oracle.BF16, 64, cfg.D, 8, esc_cap=0)
        is_raw, _, _ = _compare_all_tiles(c, p, ms, _oracle_bases(p, k[:256], v[:256]), [(k[:1000], v[:1000])])
        assert is_raw.any() and not is_raw.all()
        kd, vd = c.decode_blocks(0, 0, 15)
        assert np.array_equal(host(kd), k[:960]) and np.array_equal(host(vd), v[:960])
        q = synth.queries(cfg)
        ref = oracle.attention(oracle.BF16, q[0], k[:1000], v[:1000], cfg.scale)
        assert row_rel_err(host(c.attention([0], dev(q), cfg.scale, 4))[0], ref) <= TOL


@pytest.mark.parametrize("ms,T", [(1, 64), (2, 64), (3, 64), (1, 32)])
@pytest.mark.parametrize("Gt", [8, 16])
def test_v2_attention_and_decode_step(ms, T, Gt):
    """Decode attention over FORMAT v2 caches against the oracle (three sequences of ragged
    lengths, several split counts), then decode steps bit-identical to append + attention."""
    cfg = dataclasses.replace(synth.config(0), T=T)
    g = synth.LayerGen(cfg)
    lens = [1, 200, 777]
    toks = [g.tokens(L + 20) for L in lens]
    cal = toks[2]
    caches = []
    for _ in range(2):
        c = _cache(cfg, T, Gt, ms, max_seqs=3, max_blocks=800 // T + 3)
        c.calibrate(dev(cal[0][:256]), dev(cal[1][:256]))
        for sid, (k, v) in enumerate(toks):
            c.append([sid], dev(k[None, :lens[sid]]), dev(v[None, :lens[sid]]))
        caches.append(c)
    q = synth.queries(dataclasses.replace(cfg, n_seqs=3))
    ref = np.stack([oracle.attention(oracle.BF16, q[s], toks[s][0][:lens[s]], toks[s][1][:lens[s]], cfg.scale)
                    for s in range(3)])
    for S in (1, 3, 8):
        out = host(caches[0].attention([0, 1, 2], dev(q), cfg.scale, S))
        assert row_rel_err(out, ref) <= TOL, S
    ids = [0, 1, 2]
    for st in range(20):  # crosses block boundaries for every sequence
        kn = np.stack([toks[s][0][lens[s] + st] for s in range(3)])
        vn = np.stack([toks[s][1][lens[s] + st] for s in range(3)])
        qs = dev(synth.queries(dataclasses.replace(cfg, n_seqs=3), step=st + 1))
        a = caches[0].decode_step(ids, dev(kn[:, None]), dev(vn[:, None]), qs, cfg.scale, 4)
        caches[1].append(ids, dev(kn[:, None]), dev(vn[:, None]))
        b = caches[1].attention(ids, qs, cfg.scale, 4)
        assert torch.equal(a, b), st
    flags, _ = caches[0].status()
    assert flags == 0
