"""GPU codec parity through the C ABI: calibrated bases, encoded bytes and rebuilt tensors are
bit-exact against the oracle (GAAC page §3.1 codec, §3.3 blocks and slots)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import compare_tiles, dev, host, new_cache, oracle_layer, row_rel_err

pytestmark = pytest.mark.gpu


def _cfg_cache(cfg, chunks, compressed=True, esc_cap=-1, **kw):
    g, toks = synth.sequence_tokens(cfg)
    L = max(cfg.context)
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=cfg.n_seqs, max_blocks=L // cfg.T + 2,
                      compressed=compressed, esc_cap=esc_cap, **kw)
    k0, v0 = toks[0]
    cache.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
    for a, b in chunks:
        for sid, (k, v) in enumerate(toks):
            if a < min(b, k.shape[0]):
                cache.append([sid], dev(k[None, a:b]), dev(v[None, a:b]))
    torch.cuda.synchronize()
    return cache, toks


def test_calibration_matches_oracle():
    cfg = synth.config(2)
    g = synth.LayerGen(cfg)
    k, v = g.tokens(256)
    cache = new_cache(Hkv=8, Hq=32, D=128, T=64, max_seqs=1, max_blocks=4)
    cache.calibrate(dev(k), dev(v))
    got = cache.bases().cpu().numpy()
    b3, b4 = oracle.calibrate_layer(oracle.Params(oracle.BF16, 64, 128, 16), k, v)
    assert np.array_equal(got[:, 0], b3) and np.array_equal(got[:, 1], b4)


@pytest.mark.parametrize("chunks", [[(0, 1024)], [(0, 100), (100, 101), (101, 700), (700, 1024)]])
def test_cfg0_encode_bytes_and_decode(chunks):
    cfg = synth.config(0)
    cache, toks = _cfg_cache(cfg, chunks)
    p = oracle.Params(oracle.BF16, cfg.T, cfg.D, cfg.G)
    k0, v0 = toks[0]
    bases, oseqs = oracle_layer(p, cfg.Hkv, k0[:cfg.n_cal], v0[:cfg.n_cal], toks, chunks)
    assert np.array_equal(cache.bases().cpu().numpy()[:, 0], bases[0])
    assert compare_tiles(cache, p, oseqs, [0]) == 16 * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, 16)
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)
    flags, st = cache.status()
    assert flags == 0
    ost = oracle.stats(p, oseqs)
    assert st["comp_tiles"] + st["raw_tiles"] == ost["tiles"] and st["raw_tiles"] == ost["raw_tiles"]
    want = np.zeros(3, np.int64)
    for t in oseqs[0].tiles:
        for kv in range(2):
            for h in range(cfg.Hkv):
                if not t["is_raw"][kv, h]:
                    want += t["modes"][kv, h]
    assert st["groups"][:3] == want.tolist() and st["groups"][3] == 0  # FORMAT v1: three modes


def test_every_bf16_pattern_and_special_values():
    """All 65,536 BF16 patterns (sorted, shuffled) plus tiles of Inf/NaN/zero/subnormal groups
    go through the GPU encoder and decoder unchanged, byte-identical to the oracle."""
    rng = np.random.default_rng(9)
    allp = np.arange(65536, dtype=np.uint16)
    data = np.concatenate([allp, rng.permutation(allp)]).reshape(-1, 1, 128)  # 1024 tokens, Hkv=1
    # specials: channels 0..31 exponent 255, 32..63 exponent 0, 64..95 mixed, rest normal
    sp = synth.f32_to_bf16_bits(rng.standard_normal((256, 1, 128)).astype(np.float32))
    man = rng.integers(0, 1 << 16, (256, 1, 128)).astype(np.uint16) & np.uint16(0x807F)
    sp[:, :, 0:32] = man[:, :, 0:32] | np.uint16(0x7F80)
    sp[:, :, 32:64] = man[:, :, 32:64]
    sp[:, :, 64:96] = np.where(rng.integers(0, 2, (256, 1, 32)) == 1, man[:, :, 64:96] | np.uint16(0x7F80),
                               man[:, :, 64:96])
    for esc_cap in (-1, 0):
        for toks in (data, sp):
            cache = new_cache(Hkv=1, Hq=1, D=128, T=64, max_seqs=1, max_blocks=toks.shape[0] // 64,
                              esc_cap=esc_cap)
            cache.calibrate(dev(toks[:256]), dev(toks[:256]))
            cache.append([0], dev(toks[None]), dev(toks[None]))
            p = oracle.Params(oracle.BF16, 64, 128, 16, esc_cap=None if esc_cap < 0 else esc_cap)
            _, oseqs = oracle_layer(p, 1, toks[:256], toks[:256], [(toks, toks)])
            compare_tiles(cache, p, oseqs, [0])
            kd, vd = cache.decode_blocks(0, 0, toks.shape[0] // 64)
            assert np.array_equal(host(kd), toks) and np.array_equal(host(vd), toks)


def test_small_escape_capacity_forces_raw_tiles():
    cfg = synth.config(0)
    cache, toks = _cfg_cache(cfg, [(0, 1024)], esc_cap=64)
    p = oracle.Params(oracle.BF16, cfg.T, cfg.D, cfg.G, esc_cap=64)
    k0, v0 = toks[0]
    _, oseqs = oracle_layer(p, cfg.Hkv, k0[:256], v0[:256], toks)
    assert oracle.stats(p, oseqs)["raw_tiles"] > 0
    compare_tiles(cache, p, oseqs, [0])
    kd, vd = cache.decode_blocks(0, 0, 16)
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)


def test_uncompressed_cache_stores_every_tile_raw():
    cfg = synth.config(0)
    cache, toks = _cfg_cache(cfg, [(0, 1000)], compressed=False)
    flags, st = cache.status()
    assert st["comp_tiles"] == 0 and st["raw_tiles"] == 15 * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, 15)
    assert np.array_equal(host(kd), toks[0][0][:960]) and np.array_equal(host(vd), toks[0][1][:960])


def test_pool_exhaustion_and_release():
    cfg = synth.config(0)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    cache = new_cache(Hkv=2, Hq=4, D=64, T=64, max_seqs=2, max_blocks=16, comp_slots=6, raw_slots=2)
    cache.calibrate(dev(k[:256]), dev(v[:256]))
    cache.append([0], dev(k[None, :256]), dev(v[None, :256]))   # 4 blocks x 4 tiles = 16 tiles > 8 slots
    flags, st = cache.status()
    assert flags & 1 and flags & 2
    assert st["comp_tiles"] == 6 and st["raw_tiles"] == 2 and st["comp_free"] == 0 and st["raw_free"] == 0
    cache.release(0)
    flags, st = cache.status()
    assert st["comp_free"] == 6 and st["raw_free"] == 2 and cache.seq_length(0) == 0
    cache.append([1], dev(k[None, :128]), dev(v[None, :128]))
    kd, vd = cache.decode_blocks(1, 0, 2)
    assert np.array_equal(host(kd), k[:128]) and np.array_equal(host(vd), v[:128])


def test_cfg3_paged_mix_codec_sample():
    """32 sequences, T=16 blocks over a permuted shared pool: a sample of tiles byte-exact."""
    cfg = synth.config(3)
    g = synth.LayerGen(cfg)
    lens = [int(x) // 8 for x in cfg.context[:6]]            # shortened for the test
    toks = [g.tokens(L) for L in lens]
    cache = new_cache(Hkv=8, Hq=32, D=128, T=16, max_seqs=6, max_blocks=max(lens) // 16 + 1, perm_seed=77)
    cache.calibrate(dev(toks[0][0][:256]), dev(toks[0][1][:256]))
    for sid, (k, v) in enumerate(toks):
        cache.append([sid], dev(k[None]), dev(v[None]))
    p = oracle.Params(oracle.BF16, 16, 128, 16)
    _, oseqs = oracle_layer(p, 8, toks[0][0][:256], toks[0][1][:256], toks)
    assert compare_tiles(cache, p, oseqs, list(range(6)), sample=600) == 600
    for sid in (0, 5):
        nb = lens[sid] // 16
        kd, vd = cache.decode_blocks(sid, 0, nb)
        assert np.array_equal(host(kd), toks[sid][0][:nb * 16])


def test_cfg2_full_context_codec():
    """The 64K-token headline layer: all 16,384 tiles byte-exact against the oracle, every block
    decoded bit for bit, the same raw tiles and escape bytes."""
    cfg = synth.config(2)
    cache, toks = _cfg_cache(cfg, [(0, 65536)])
    p = oracle.Params(oracle.BF16, 64, 128, 16)
    k0, v0 = toks[0]
    _, oseqs = oracle_layer(p, 8, k0[:256], v0[:256], toks)
    assert compare_tiles(cache, p, oseqs, [0]) == 16384
    kd, vd = cache.decode_blocks(0, 0, 1024)
    assert np.array_equal(host(kd), k0) and np.array_equal(host(vd), v0)
    flags, st = cache.status()
    ost = oracle.stats(p, oseqs)
    assert st["raw_tiles"] == ost["raw_tiles"]
    assert st["esc_bytes"] == sum(int(t["esc"].sum()) for t in oseqs[0].tiles)


def test_head_dim_256_half_heads():
    """A 256-channel head (GAAC page App. D: two 128-channel half-heads): encoded bytes equal the
    oracle's for the half-head view of the same tokens, and blocks decode back bit for bit."""
    import dataclasses
    cfg = dataclasses.replace(synth.config(0), D=256)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    n_tiles = 17 * 2 * 2 * cfg.Hkv  # a block holds two half-head tiles per head, for K and V
    cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=256, T=cfg.T, max_seqs=1, max_blocks=17, comp_slots=n_tiles,
                      raw_slots=n_tiles)
    cache.calibrate(dev(k[:cfg.n_cal]), dev(v[:cfg.n_cal]))
    cache.append([0], dev(k[None, :1000]), dev(v[None, :1000]))
    half = lambda a: a.reshape(a.shape[0], 2 * cfg.Hkv, 128)  # the same memory as half-heads
    p = oracle.Params(oracle.BF16, cfg.T, 128, cfg.G)
    _, oseqs = oracle_layer(p, 2 * cfg.Hkv, half(k[:cfg.n_cal]), half(v[:cfg.n_cal]), [(half(k[:1000]), half(v[:1000]))])
    view = new_cache(Hkv=2 * cfg.Hkv, Hq=2 * cfg.Hq, D=128, T=cfg.T, max_seqs=1, max_blocks=17)  # for its metadata
    view.buffers = cache.buffers
    view.slot_stride = cache.slot_stride
    assert compare_tiles(view, p, oseqs, [0]) == 15 * 2 * 2 * cfg.Hkv
    kd, vd = cache.decode_blocks(0, 0, 15)
    assert np.array_equal(host(kd), k[:960]) and np.array_equal(host(vd), v[:960])
    flags, st = cache.status()
    assert flags == 0 and st["comp_tiles"] == 15 * 2 * 2 * cfg.Hkv and st["raw_tiles"] == 0


@pytest.mark.parametrize("fmt,Gt,T", [(oracle.BF16, 16, 64), (oracle.BF16, 8, 16), (oracle.E5M2, 16, 64),
                                      (oracle.E4M3, 8, 64)])
def test_head_dim_256_attention(fmt, Gt, T):
    """Decode attention over 256-channel heads (both half-heads of a head in one softmax; the
    tail attended by the last split): compressed, raw-fallback and uncompressed caches against
    the oracle's fp64 attention, lengths with tails of 0, 1 and T - 1 tokens, split counts 1 to
    16, and a decode step equal to append + attention bit for bit."""
    import dataclasses
    cfg = dataclasses.replace(synth.config(0), D=256, fmt=fmt)
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    for L in (T - 1, 3 * T, 3 * T + 1, 700):
        q = synth.queries(cfg, step=L)
        ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
        for compressed, esc_cap in ((True, -1), (True, 16), (False, -1)):
            n_tiles = (L // T + 2) * 2 * 2 * cfg.Hkv
            cache = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=256, T=T, max_seqs=1, max_blocks=L // T + 2,
                              comp_slots=n_tiles if compressed else None, raw_slots=n_tiles, compressed=compressed,
                              esc_cap=esc_cap, fmt=fmt, Gt=Gt)
            cache.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
            cache.append([0], dev(k[None, :L], fmt), dev(v[None, :L], fmt))
            for S in (1, 3, 16):
                out = host(cache.attention([0], dev(q), cfg.scale, S))
                assert row_rel_err(out[0], ref) <= 4e-3, (L, compressed, esc_cap, S)
            assert cache.status()[0] == 0
    # decode step against append + attention
    L = 3 * T - 2
    a, b = [new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=256, T=T, max_seqs=1, max_blocks=L // T + 3,
                      comp_slots=(L // T + 3) * 4 * cfg.Hkv, raw_slots=(L // T + 3) * 4 * cfg.Hkv, fmt=fmt, Gt=Gt)
            for _ in range(2)]
    for c in (a, b):
        c.calibrate(dev(k[:cfg.n_cal], fmt), dev(v[:cfg.n_cal], fmt))
        c.append([0], dev(k[None, :L], fmt), dev(v[None, :L], fmt))
    for t in range(L, L + 4):
        q = dev(synth.queries(cfg, step=t))
        kn, vn = dev(k[None, t:t + 1], fmt), dev(v[None, t:t + 1], fmt)
        out_a = host(a.decode_step([0], kn, vn, q, cfg.scale, 4))
        b.append([0], kn, vn)
        assert np.array_equal(out_a, host(b.attention([0], q, cfg.scale, 4))), t
        ref = oracle.attention(fmt, synth.queries(cfg, step=t)[0], k[:t + 1], v[:t + 1], cfg.scale)
        assert row_rel_err(out_a[0], ref) <= 4e-3, t
