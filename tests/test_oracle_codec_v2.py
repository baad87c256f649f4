"""Pins for the oracle's FORMAT v2 codec: the nested precision modes of the GAAC page (§4.7.2 /
Table 4: a 2-bit mode added to the 3-bit, 4-bit and raw modes, or the 3-bit mode removed), each
group's offsets stored at its own mode's width.  Hand-derived golden tiles, planted layout
mistakes they catch, exhaustive round trips of every BF16 pattern, brute-force mode choice and
2-bit calibration, closed-form sizes, and the v1 modes in the v2 layout giving v1's bit count."""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
V2_GOLDEN = ["tile_v2_bf16_t16_d2_g8_modes_2_3_4_raw", "tile_v2_bf16_t16_d2_modes_4_raw"]


def _golden(orc, name):
    d = json.load(open(os.path.join(GOLDEN, name + ".json")))
    p = orc.Params(**d["params"])
    x = np.array(d["x"], np.uint16)
    bases = [np.array(d[k], np.uint8) for k in ("b2", "b3", "b4")]
    want = bytes.fromhex(d["expected_hex"].replace(" ", ""))
    return p, d["mode_set"], x, bases, want, d["stride"], d["code_bytes"]


@pytest.mark.parametrize("name", V2_GOLDEN)
def test_v2_golden_tile_bytes(orc, name):
    p, ms, x, (b2, b3, b4), want, stride, used = _golden(orc, name)
    assert orc.v2_layout(p, ms)["stride"] == stride == len(want)
    data, is_raw, code_bytes, modes = orc.v2_encode_tiles(p, ms, x[None], b2, b3, b4, 0)
    assert is_raw[0] == 0 and code_bytes[0] == used
    assert bytes(data[0, :stride]) == want
    back, st = orc.v2_decode_tiles(p, ms, np.frombuffer(want, np.uint8)[None], [0], 0, b2, b3, b4)
    assert st[0] == 0 and np.array_equal(back[0], x)


PLANTED_V2 = {
    "offsets of a group in reverse token order": [
        ("put_bit(code, O + (long)tau * w + b, o >> b);", "put_bit(code, O + (long)(G - 1 - tau) * w + b, o >> b);"),
        ("o |= get_bit(code, O + (long)tau * w + b) << b;", "o |= get_bit(code, O + (long)(G - 1 - tau) * w + b) << b;")],
    "offset bits most significant first": [
        ("put_bit(code, O + (long)tau * w + b, o >> b);", "put_bit(code, O + (long)tau * w + (w - 1 - b), o >> b);"),
        ("o |= get_bit(code, O + (long)tau * w + b) << b;", "o |= get_bit(code, O + (long)tau * w + (w - 1 - b)) << b;")],
    "mode-index planes swapped": [
        ("put_bit(tag0, q, (uint32_t)k & 1u);\n    put_bit(tag1, q, ((uint32_t)k >> 1) & 1u);",
         "put_bit(tag1, q, (uint32_t)k & 1u);\n    put_bit(tag0, q, ((uint32_t)k >> 1) & 1u);"),
        ("int k = (int)(get_bit(tag0, q) | (get_bit(tag1, q) << 1));",
         "int k = (int)(get_bit(tag1, q) | (get_bit(tag0, q) << 1));")],
    "codes before the sign/mantissa bytes": [
        ("  L->sm_off = align16(L->tag_bytes);\n  L->code_off = L->sm_off + align16(L->sm_bytes);\n  L->stride = L->code_off + align16(L->code_cap);",
         "  L->code_off = align16(L->tag_bytes);\n  L->sm_off = L->code_off + align16(L->code_cap);\n  L->stride = L->sm_off + align16(L->sm_bytes);")],
}


def _planted(tmp_path, edits):
    src = open(os.path.join(ROOT, "oracle", "kvc_oracle.c")).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"planted edit not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / "planted_v2.c"
    so = tmp_path / "planted_v2.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(c), "-o", str(so), "-lm"])
    return ctypes.CDLL(str(so))


@pytest.mark.parametrize("mistake", sorted(PLANTED_V2))
def test_v2_goldens_catch_planted_mistakes(orc, tmp_path, mistake):
    lib = _planted(tmp_path, PLANTED_V2[mistake])
    P = ctypes.POINTER
    lib.orc_v2_encode_tile.argtypes = [P(orc._Params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                       P(ctypes.c_int32), P(ctypes.c_int32), ctypes.c_void_p]
    lib.orc_v2_decode_tile.argtypes = [P(orc._Params), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    caught = []
    for name in V2_GOLDEN:
        p, ms, x, (b2, b3, b4), want, stride, _ = _golden(orc, name)
        out = np.zeros(4096, np.uint8)
        isr, used = ctypes.c_int32(), ctypes.c_int32()
        modes = np.zeros(4, np.int32)
        assert lib.orc_v2_encode_tile(ctypes.byref(p.c()), ms, x.ctypes.data, b2.ctypes.data, b3.ctypes.data,
                                      b4.ctypes.data, 0, out.ctypes.data, ctypes.byref(isr), ctypes.byref(used),
                                      modes.ctypes.data) == 0
        back = np.zeros_like(x)
        assert lib.orc_v2_decode_tile(ctypes.byref(p.c()), ms, out.ctypes.data, isr.value, 0, b2.ctypes.data,
                                      b3.ctypes.data, b4.ctypes.data, back.ctypes.data) == 0
        assert np.array_equal(back, x)  # the planted copy still round-trips its own bytes
        if bytes(out[:stride]) != want:
            caught.append(name)
    assert caught, f"no golden tile detects: {mistake}"


@pytest.mark.parametrize("G", [8, 16])
@pytest.mark.parametrize("ms", [1, 2, 3])
def test_v2_every_bf16_pattern_roundtrips(orc, ms, G):
    p = orc.Params(orc.BF16, 64, 128, G)
    rng = np.random.default_rng(41 + ms)
    allp = np.arange(65536, dtype=np.uint16)
    for pat in (allp, rng.permutation(allp), np.repeat(allp[::G], G)):
        tiles = pat[: len(pat) // 8192 * 8192].reshape(-1, 64, 128)
        n = tiles.shape[0]
        for lo in (0, 120):
            b = [rng.integers(lo, min(lo + 100, 256 - (1 << w)) + 1, (n, 128)).astype(np.uint8) for w in (2, 3, 4)]
            for is_v in (0, 1):
                data, is_raw, used, modes = orc.v2_encode_tiles(p, ms, tiles, *b, is_v)
                back, st = orc.v2_decode_tiles(p, ms, data, is_raw, is_v, *b)
                assert (st == 0).all() and np.array_equal(back, tiles)


def _brute_mode(widths, bases, mn, mx):
    for k, w in enumerate(widths[:-1]):
        b = bases[w]
        if b <= mn and mx <= b + (1 << w) - 1:
            return k
    return len(widths) - 1


@pytest.mark.parametrize("ms", [1, 2, 3])
def test_v2_mode_choice_is_the_narrowest_fitting_window(orc, ms):
    """Every (min, max) exponent pair of a group against a grid of bases: the oracle's mode
    index equals the first window of the set that holds both."""
    p = orc.Params(orc.BF16, 16, 32, 16)
    widths = orc.MODE_SETS[ms]
    rng = np.random.default_rng(ms)
    pairs = [(mn, mx) for mn in range(0, 256, 3) for mx in range(mn, min(mn + 40, 256), 2)]
    for start in range(0, len(pairs), 32):
        chunk = pairs[start:start + 32]
        x = np.zeros((16, 32), np.uint16)
        for c, (mn, mx) in enumerate(chunk):
            x[:, c] = ((np.linspace(mn, mx, 16).round().astype(np.uint16)) << 7)
            x[0, c], x[15, c] = mn << 7, mx << 7
        bases = {w: rng.integers(0, 256 - (1 << w) + 1, 32).astype(np.uint8) for w in (2, 3, 4)}
        # put some bases exactly at the group's minimum so that windows fit
        for c, (mn, mx) in enumerate(chunk):
            if c % 2 == 0:
                for w in (2, 3, 4):
                    bases[w][c] = min(mn, 256 - (1 << w))
        _, _, _, modes = orc.v2_encode_tiles(p, ms, x[None], bases[2], bases[3], bases[4], 0)
        want = np.zeros(4, np.int64)
        for c in range(32):  # channels past the chunk hold exponent 0 throughout
            mn, mx = chunk[c] if c < len(chunk) else (0, 0)
            want[_brute_mode(widths, {w: int(bases[w][c]) for w in (2, 3, 4)}, mn, mx)] += 1
        got = modes[0].astype(np.int64)
        assert np.array_equal(got, want), (ms, start)


@pytest.mark.parametrize("w", [2, 3, 4])
def test_v2_calibration_bruteforce(orc, w):
    """The base of every window width (2-, 3- and 4-bit offsets) against a brute force over all
    window starts: the lower median of the starts of maximal coverage."""
    p = orc.Params(orc.BF16, 16, 4, 16, esc_cap=0)
    rng = np.random.default_rng(9 + w)
    n = 1 << w
    for trial in range(40):
        e = rng.integers(100, 140, (256, 4)) if trial % 2 else rng.normal(120, 3, (256, 4)).astype(int)
        if trial % 5 == 0:
            e[:, 1] = 0          # a window that must start at 0
            e[:, 2] = 255        # and one pressed against the top of the field
        x = (np.clip(e, 0, 255).astype(np.uint16) << 7)
        b = orc.v2_calibrate(p, x, w)
        for c in range(4):
            hist = np.bincount((x[:, c] >> 7) & 0xFF, minlength=256)
            cov = np.array([hist[s:s + n].sum() for s in range(256 - n + 1)])
            ties = np.nonzero(cov == cov.max())[0]
            assert b[c] == ties[(len(ties) - 1) // 2], (w, trial, c)
    if w > 2:  # the 3- and 4-bit bases are FORMAT v1's b3 and b4
        x = (rng.integers(90, 150, (256, 4)).astype(np.uint16) << 7)
        b3, b4 = orc.calibrate(p, x)
        assert np.array_equal(orc.v2_calibrate(p, x, w), b3 if w == 3 else b4)


@pytest.mark.parametrize("G", [8, 16])
def test_v2_sizes_closed_form(orc, G):
    """All-2-bit and all-raw tiles: CODES bytes = G * sum of widths / 8; a tile whose codes exceed
    3*T*D/8 + esc_cap stays raw; the v1 modes in the v2 layout cost exactly v1's CODE + ESC bits."""
    p = orc.Params(orc.BF16, 64, 128, G)
    lay = orc.v2_layout(p, 1)
    assert lay["code_cap"] == 64 * 128 * 3 // 8 + 512 == orc.v2_layout(p, 3)["code_cap"]
    assert orc.v2_layout(p, 2)["code_cap"] == 64 * 128 * 4 // 8 + 512
    e = np.full((64, 128), 100, np.uint16)
    x = (e << 7)[None]
    b = np.full(128, 100, np.uint8)
    _, is_raw, used, modes = orc.v2_encode_tiles(p, 1, x, b, b, b, 0)
    assert is_raw[0] == 0 and used[0] == 64 * 128 * 2 // 8 and modes[0, 0] == lay["n_groups"]
    _, is_raw, used, modes = orc.v2_encode_tiles(p, 2, x, b, b, b, 0)
    assert used[0] == 64 * 128 * 4 // 8 and modes[0, 0] == lay["n_groups"]
    # every group raw: 8 bits per element > 3/8 + 1/16 bytes per element -> RAW tile
    xr = (np.arange(64 * 128, dtype=np.uint16).reshape(64, 128) % 256 << 7)[None]
    _, is_raw, _, modes = orc.v2_encode_tiles(p, 1, xr, b, b, b, 0)
    assert is_raw[0] == 1
    # v1 modes in the v2 layout: the same stored bits as FORMAT v1 on the same data
    import synth
    cfg = synth.config(2)
    g = synth.LayerGen(cfg)
    k, v = g.tokens(2048)
    p1 = orc.Params(orc.BF16, 64, 128, G)
    b3, b4 = orc.calibrate(p1, np.ascontiguousarray(k[:256, 0]))
    tiles = np.ascontiguousarray(k[:, 0].reshape(-1, 64, 128))
    _, raw1, esc1, modes1 = orc.encode_tiles(p1, tiles, b3, b4, 0)
    _, raw2, used2, modes2 = orc.v2_encode_tiles(p1, 3, tiles, b3, b3, b4, 0)
    assert (raw1 == raw2).all() and np.array_equal(modes1, modes2[:, :3])
    assert (used2 == 3 * 64 * 128 // 8 + esc1).all()      # v1's CODE bytes + its used ESC bytes
