"""The diagnostics behind the positional-drift study (GAAC page App. C: escape bytes per tile and
raw fallbacks along a context of rotated keys) and the exponent-concentration claim (§3.1),
through the C ABI against the oracle: kv_tile_stats on RoPE-rotated keys equals the oracle's
encoding of the same tiles, tile by tile (storage mode, escape or code bytes, mode counts), so
the per-segment figures the study reports are the oracle's; kv_window_coverage equals the
oracle's best-window counts for every format."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import dev, new_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ms", [0, 1])
def test_rope_drift_tile_stats_match_oracle(ms):
    cfg = synth.config(2)
    g = synth.LayerGen(cfg)
    kc, vc = g.tokens(256)
    k, v = g.tokens(4096)
    cal_k = synth.rope_keys(kc, first_pos=0)                 # calibrated at the start of a context
    kr = synth.rope_keys(k, first_pos=56 * 1024)             # keys 56K positions later: drifted
    Gt = 8 if ms else 16
    p = oracle.Params(oracle.BF16, 64, 128, Gt)
    nb = 4096 // 64
    print(f"[rope stats] mode set {ms}", flush=True)
    c = new_cache(Hkv=8, Hq=32, D=128, T=64, max_seqs=1, max_blocks=nb + 1, Gt=Gt, mode_set=ms)
    c.calibrate(dev(cal_k), dev(vc))
    c.append([0], dev(kr[None]), dev(v[None]))
    got = c.tile_stats(0, 0, nb).cpu().numpy()               # [nb][2][8][7]
    tiles = np.stack([x[b * 64:(b + 1) * 64, h] for b in range(nb) for x in (kr, v) for h in range(8)])
    isv = np.array([kv for b in range(nb) for kv in (0, 1) for h in range(8)], np.int32)
    kvh = [(kv, h) for b in range(nb) for kv in (0, 1) for h in range(8)]
    if ms == 0:
        b3, b4 = oracle.calibrate_layer(p, cal_k, vc)
        _, is_raw, nbytes, modes = oracle.encode_tiles(p, tiles, np.stack([b3[a, h] for a, h in kvh]),
                                                       np.stack([b4[a, h] for a, h in kvh]), isv)
        modes = np.concatenate([modes, np.zeros((len(kvh), 1), np.int32)], axis=1)
    else:
        b2, b3, b4 = oracle.v2_calibrate_layer(p, cal_k, vc)
        _, is_raw, nbytes, modes = oracle.v2_encode_tiles(p, ms, tiles, *[np.stack([b[a, h] for a, h in kvh])
                                                                           for b in (b2, b3, b4)], isv)
    got = got.reshape(-1, 7)
    assert np.array_equal(got[:, 0], is_raw), "storage modes differ"
    comp = is_raw == 0
    assert np.array_equal(got[comp, 1], nbytes[comp]), "escape/code bytes differ"
    assert np.array_equal(got[comp, 2:6], modes[comp]), "mode counts differ"
    assert (got[~comp, 1:6] == 0).all()
    assert (got[comp, 6] == 0).all() and (got[~comp, 6] == -1).all()  # one base version
    if ms == 0:  # the drifted keys need more escape bytes than the unrotated values
        kt = got.reshape(nb, 2, 8, 7)
        assert kt[:, 0, :, 1].mean() > kt[:, 1, :, 1].mean()
    flags, st = c.status()
    assert flags == 0 and st["raw_tiles"] == int((~comp).sum())


@pytest.mark.parametrize("fmt", [synth.BF16, synth.E5M2, synth.E4M3])
def test_window_coverage_matches_oracle(fmt):
    import dataclasses
    cfg = dataclasses.replace(synth.config(2), fmt=fmt)
    k, v = synth.LayerGen(cfg).tokens(2048)
    c = new_cache(Hkv=8, Hq=32, D=128, T=64, max_seqs=1, max_blocks=2, fmt=fmt)
    p = oracle.Params(fmt, 64, 128, 16)
    F = {synth.BF16: 8, synth.E5M2: 5, synth.E4M3: 4}[fmt]
    for x in (k, v):
        xd = dev(x, fmt)
        for w in sorted({1, 6, 8, 16, 1 << F}):
            got = c.window_coverage(xd, w).cpu().numpy()
            want = np.stack([oracle.window_coverage(p, np.ascontiguousarray(x[:, h]), w) for h in range(8)])
            assert np.array_equal(got, want), (fmt, w)
    with pytest.raises(Exception):
        c.window_coverage(dev(k, fmt), (1 << F) + 1)


def test_read_probe_reads_every_byte():
    """kv_read_probe: every lane's checksum equals the fold of exactly the 16-byte words the
    probe is documented to read (wave w's region, batch by batch, four words per lane), and
    misshaped requests are refused."""
    import decode_attention_calibrate_amd as K
    rng = np.random.default_rng(11)
    waves, per = 5, 3 * 8192
    words = rng.integers(0, 1 << 32, size=(waves * per) // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    got = K.read_probe(src, per, waves).cpu().numpy().view(np.uint32)
    w4 = words.reshape(waves, per // 16, 4)
    x = (w4[..., 0] ^ w4[..., 1] ^ w4[..., 2] ^ w4[..., 3]).astype(np.uint64)   # [wave][16-byte word]
    want = np.zeros((waves, 64), np.uint64)
    for i in range(per // 8192):
        for u in range(8):
            want = (want * 31 + x[:, i * 512 + 64 * u + np.arange(64)]) & 0xFFFFFFFF
    assert np.array_equal(got, want.astype(np.uint32))
    for nbytes, nw in ((8192 + 4096, 1), (0, 1), (8192, 0)):  # refused by the library's own checks
        with pytest.raises(K.KVCError):
            K.read_probe(src, nbytes, nw)
