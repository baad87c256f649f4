"""Recalibration of a live cache through the C ABI (GAAC page App. C: exponent windows
calibrated near the start of a context drift away from later keys).  A cache calibrated on its
first tokens is recalibrated (kv_recalibrate) twice as the token distribution changes (each
segment comes from a layer with other channel scales); every block is encoded with the base
version current when it finished, and every decoder reads a tile's version from its table
entry.  Against the oracle: each version's bases, every stored tile's bytes (the oracle's
encoding with the bases of that tile's version), kv_decode_blocks bit for bit, the version field
of kv_tile_stats, decode attention within the tolerance, and decode steps across a
recalibration bit-identical to append + attention -- for every kernel family: register rebuild
at T = 64 and at T = 16 (versions change inside a 64-token super-block), FP8, 8-token groups,
FORMAT v2 and 256-channel heads.  Then the version bookkeeping: exhaustion, release, a
single-version cache."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from decode_attention_calibrate_amd import KVCError
from kvtest import _stored_tiles, dev, host, new_cache, row_rel_err, stored_versions

pytestmark = pytest.mark.gpu
TOL = 4e-3
CUTS = (400, 900)  # tokens stored before the first and before the second recalibration
L = 1290           # 20 blocks of 64 tokens and a 10-token tail
ESTATE = -6

CASES = [  # (fmt, T, Gt, mode_set, D)
    (oracle.BF16, 64, 16, 0, 128),
    (oracle.BF16, 16, 16, 0, 128),
    (oracle.E5M2, 64, 16, 0, 128),
    (oracle.BF16, 64, 8, 0, 128),
    (oracle.BF16, 64, 8, 1, 128),
    (oracle.BF16, 64, 16, 0, 256),
]


def _tokens(fmt, D):
    cfg = dataclasses.replace(synth.config(0), D=D, Hq=8, fmt=fmt, context=(L,))
    parts = [synth.LayerGen(cfg, layer).tokens(n) for layer, n in ((0, CUTS[0]), (1, CUTS[1] - CUTS[0]), (2, L - CUTS[1]))]
    return cfg, np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


CAL = [(0, 256), (CUTS[0], CUTS[0] + 256), (CUTS[1], CUTS[1] + 256)]  # calibration rows per version


def _version_of_block(b, T):
    end = (b + 1) * T  # the block finishes when its last token is stored
    return 0 if end <= CUTS[0] else 1 if end <= CUTS[1] else 2


def _stored_heads(x, D):
    """[n][Hkv][D] -> the stored [n][stored heads][128 or D] view (256-channel heads as halves)."""
    return x.reshape(x.shape[0], -1, 128) if D == 256 else x


def _cache(cfg, T, Gt, ms, D, max_blocks, versions):
    heads = cfg.Hkv * (2 if D == 256 else 1)
    n = max_blocks * 2 * heads
    return new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=D, T=T, max_seqs=1, max_blocks=max_blocks, comp_slots=n, raw_slots=n,
                     fmt=cfg.fmt, Gt=Gt, mode_set=ms, base_versions=versions)


def _fill(c, k, v, fmt, upto=L):
    """calibrate, append up to CUTS[0], recalibrate, append up to CUTS[1], recalibrate, append."""
    c.calibrate(dev(k[:256], fmt), dev(v[:256], fmt))
    bounds = [0, CUTS[0], CUTS[1], upto]
    for i in range(3):
        if i > 0:
            a, b = CAL[i]
            c.recalibrate(dev(k[a:b], fmt), dev(v[a:b], fmt))
        c.append([0], dev(k[None, bounds[i]:bounds[i + 1]], fmt), dev(v[None, bounds[i]:bounds[i + 1]], fmt))


@pytest.mark.parametrize("fmt,T,Gt,ms,D", CASES)
def test_recalibrated_cache_matches_oracle(fmt, T, Gt, ms, D):
    print(f"[recalibrate] fmt={fmt} T={T} G={Gt} mode_set={ms} D={D}", flush=True)
    cfg, k, v = _tokens(fmt, D)
    nb = L // T
    c = _cache(cfg, T, Gt, ms, D, nb + 1, versions=3)
    _fill(c, k, v, fmt)
    ks, vs = _stored_heads(k, D), _stored_heads(v, D)
    heads = ks.shape[1]
    p = oracle.Params(fmt, T, ks.shape[2], Gt)
    # each version's bases equal the oracle's calibration on that version's rows
    vb = []
    for ver, (a, b) in enumerate(CAL):
        if ms == 0:
            b3, b4 = oracle.calibrate_layer(p, ks[a:b], vs[a:b])
            vb.append((None, b3, b4))
        else:
            vb.append(oracle.v2_calibrate_layer(p, ks[a:b], vs[a:b]))
        got = c.bases(ver).cpu().numpy().reshape(2, 2, heads, -1)
        assert np.array_equal(got[:, 0], vb[ver][1]) and np.array_equal(got[:, 1], vb[ver][2]), ver
        if ms == 1:
            assert np.array_equal(c.bases2(ver).cpu().numpy().reshape(2, heads, -1), vb[ver][0]), ver
    # every stored tile: its version, and its bytes as the oracle encodes it with those bases
    jobs = [(0, b, kv, h) for b in range(nb) for kv in range(2) for h in range(heads)]
    want_ver = np.array([_version_of_block(b, T) for _, b, _, _ in jobs])
    tiles = np.stack([(ks, vs)[kv][b * T:(b + 1) * T, h] for _, b, kv, h in jobs])
    isv = np.array([kv for _, _, kv, _ in jobs], np.int32)
    pick = lambda w: np.stack([vb[ver][w][kv, h] for ver, (_, _, kv, h) in zip(want_ver, jobs)])
    if ms == 0:
        data, is_raw, used, _ = oracle.encode_tiles(p, tiles, pick(1), pick(2), isv)
        lay = oracle.layout(p)
    else:
        data, is_raw, used, _ = oracle.v2_encode_tiles(p, ms, tiles, pick(0), pick(1), pick(2), isv)
        lay = oracle.v2_layout(p, ms)
    got_ver = np.array(stored_versions(c, jobs))
    assert np.array_equal(got_ver[is_raw == 0], want_ver[is_raw == 0]), "base versions in the table entries"
    assert (got_ver[is_raw == 1] == -1).all()
    for n, (job, (raw, units, got)) in enumerate(zip(jobs, _stored_tiles(c, jobs))):
        assert raw == bool(is_raw[n]), job
        size = lay["raw_bytes"] if raw else lay["stride"]
        if not np.array_equal(got[:size], data[n, :size]):
            raise AssertionError(f"tile {job} (version {want_ver[n]}): bytes differ from the oracle")
        if not raw and ms == 0:
            assert units == (int(used[n]) + 15) // 16, job
    assert len(set(want_ver[is_raw == 0])) == 3, "every version holds compressed tiles"
    # the tile statistics carry the version
    st = c.tile_stats(0, 0, nb).cpu().numpy().reshape(-1, 7)
    assert np.array_equal(st[:, 6], got_ver)
    # decode back to the original tokens, bit for bit
    kd, vd = c.decode_blocks(0, 0, nb)
    assert np.array_equal(host(kd), k[:nb * T]) and np.array_equal(host(vd), v[:nb * T])
    # decode attention over blocks of three base versions plus the tail
    q = synth.queries(cfg)
    ref = oracle.attention(fmt, q[0], k[:L], v[:L], cfg.scale)
    for S in (1, 4, 16):
        out = host(c.attention([0], dev(q), cfg.scale, S))
        assert row_rel_err(out[0], ref) <= TOL, S
    flags, _ = c.status()
    assert flags == 0


@pytest.mark.parametrize("fmt,T,Gt,ms,D", CASES)
def test_decode_steps_across_a_recalibration(fmt, T, Gt, ms, D):
    """Two caches filled alike; a third recalibration in the middle of a run of decode steps,
    one of which then completes a block (encoded with the new version): kv_decode_step equals
    append + attention bit for bit at every step."""
    print(f"[recalibrate steps] fmt={fmt} T={T} G={Gt} mode_set={ms} D={D}", flush=True)
    cfg, k, v = _tokens(fmt, D)
    L0 = 1270
    caches = [_cache(cfg, T, Gt, ms, D, L // T + 2, versions=4) for _ in range(2)]
    for c in caches:
        _fill(c, k, v, fmt, upto=L0)
    for t in range(L0, L):
        if t == L0 + 5:
            for c in caches:
                c.recalibrate(dev(k[1000:1256], fmt), dev(v[1000:1256], fmt))
        q = dev(synth.queries(cfg, step=t))
        kn, vn = dev(k[None, t:t + 1], fmt), dev(v[None, t:t + 1], fmt)
        out_a = caches[0].decode_step([0], kn, vn, q, cfg.scale, 4)
        caches[1].append([0], kn, vn)
        out_b = caches[1].attention([0], q, cfg.scale, 4)
        assert torch.equal(out_a, out_b), t
    ref = oracle.attention(fmt, synth.queries(cfg, step=L - 1)[0], k[:L], v[:L], cfg.scale)
    assert row_rel_err(host(out_a)[0], ref) <= TOL
    heads = cfg.Hkv * (2 if D == 256 else 1)
    last = [(0, L // T - 1, kv, h) for kv in range(2) for h in range(heads)]
    assert set(x for x in stored_versions(caches[0], last) if x >= 0) == {3}  # the block finished after it
    kd, vd = caches[0].decode_blocks(0, 0, L // T)
    assert np.array_equal(host(kd), k[:L // T * T]) and np.array_equal(host(vd), v[:L // T * T])
    assert caches[0].status()[0] == 0


def test_version_bookkeeping():
    """Versions in use cannot be recalibrated; releasing a sequence frees its versions; a
    single-version cache and an uncalibrated cache refuse; after a release and a recalibration
    the reused version's new bases encode the new blocks."""
    cfg, k, v = _tokens(oracle.BF16, 128)
    c = _cache(cfg, 64, 16, 0, 128, L // 64 + 1, versions=3)
    with pytest.raises(KVCError) as e:
        c.recalibrate(dev(k[:256]), dev(v[:256]))            # before kv_calibrate
    assert e.value.code == ESTATE
    _fill(c, k, v, oracle.BF16)                              # versions 0, 1, 2 all hold blocks
    with pytest.raises(KVCError) as e:
        c.recalibrate(dev(k[:256]), dev(v[:256]))
    assert e.value.code == ESTATE
    c.release(0)
    c.recalibrate(dev(k[CUTS[1]:CUTS[1] + 256]), dev(v[CUTS[1]:CUTS[1] + 256]))  # reuses version 0
    c.append([0], dev(k[None, :640]), dev(v[None, :640]))
    p = oracle.Params(oracle.BF16, 64, 128, 16)
    b3, b4 = oracle.calibrate_layer(p, k[CUTS[1]:CUTS[1] + 256], v[CUTS[1]:CUTS[1] + 256])
    jobs = [(0, b, kv, h) for b in range(10) for kv in range(2) for h in range(cfg.Hkv)]
    tiles = np.stack([(k, v)[kv][b * 64:(b + 1) * 64, h] for _, b, kv, h in jobs])
    data, is_raw, _, _ = oracle.encode_tiles(p, tiles, np.stack([b3[kv, h] for _, _, kv, h in jobs]),
                                             np.stack([b4[kv, h] for _, _, kv, h in jobs]),
                                             np.array([kv for _, _, kv, _ in jobs], np.int32))
    lay = oracle.layout(p)
    vers = stored_versions(c, jobs)
    for n, (raw, _, got) in enumerate(_stored_tiles(c, jobs)):
        size = lay["raw_bytes"] if raw else lay["stride"]
        assert raw == bool(is_raw[n]) and np.array_equal(got[:size], data[n, :size]), jobs[n]
        assert vers[n] == (-1 if raw else 0)
    one = _cache(cfg, 64, 16, 0, 128, 4, versions=1)
    one.calibrate(dev(k[:256]), dev(v[:256]))
    with pytest.raises(KVCError) as e:
        one.recalibrate(dev(k[:256]), dev(v[:256]))
    assert e.value.code == ESTATE
