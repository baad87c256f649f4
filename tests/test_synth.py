"""The seeded input generators: rotated keys are an exact rotation of the unrotated ones up to
the final BF16 rounding (position 0 leaves them unchanged; every channel pair keeps its norm)."""
import numpy as np

import synth


def test_rope_keys_position_zero_is_identity_and_pairs_keep_their_norm():
    cfg = synth.config(0)
    k, _ = synth.LayerGen(cfg).tokens(300)
    r = synth.rope_keys(k, theta=1.0e4)
    assert np.array_equal(r[0], k[0])
    D = cfg.D
    x, y = synth.bf16_bits_to_f32(k).astype(np.float64), synth.bf16_bits_to_f32(r).astype(np.float64)
    nx = np.hypot(x[..., : D // 2], x[..., D // 2:])
    ny = np.hypot(y[..., : D // 2], y[..., D // 2:])
    assert np.all(np.abs(ny - nx) <= 2.0 ** -7 * nx + 1e-30)  # two BF16 roundings at most
    # a later position really turns the fast pairs: channel 0 differs somewhere
    assert not np.array_equal(r[1:, :, 0], k[1:, :, 0])


def test_rope_keys_continue_across_calls():
    cfg = synth.config(0)
    k, _ = synth.LayerGen(cfg).tokens(64)
    whole = synth.rope_keys(k)
    parts = np.concatenate([synth.rope_keys(k[:20]), synth.rope_keys(k[20:], first_pos=20)])
    assert np.array_equal(whole, parts)
