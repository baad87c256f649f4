"""kv_decode_attention_noalloc: decode attention whose split partials live in the library's fixed
per-GPU workspace instead of a caller buffer, for callers that cannot allocate.  Through the C
ABI it must give kv_decode_attention's output bit for bit (the same kernels) on two calls in a
row, the second over a smaller input (the array keeps the first call's partials), allocate
nothing, and refuse a split count whose partials do not fit, before enqueuing anything."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kvtest import dev, host, new_cache, row_rel_err

pytestmark = pytest.mark.gpu


def _filled_cache(cfg, n_tokens, seed_layer=0):
    g = synth.LayerGen(cfg, seed_layer)
    k, v = g.tokens(n_tokens)
    c = new_cache(Hkv=cfg.Hkv, Hq=cfg.Hq, D=cfg.D, T=cfg.T, max_seqs=1, max_blocks=n_tokens // cfg.T + 2)
    c.calibrate(dev(k[:cfg.n_cal]), dev(v[:cfg.n_cal]))
    c.append([0], dev(k[None]), dev(v[None]))
    return c, k, v


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    from decode_attention_calibrate_amd import _lib
    cases = [  # (workload, tokens, splits): the second is smaller in every dimension
        (synth.config(2), 16421, 256),   # 8 KV / 32 query heads, D = 128, T = 64: 4.26 MB of partials
        (synth.config(0), 1000, 16),     # 2 KV / 4 query heads, D = 64
    ]
    for cfg, n_tokens, S in cases:
        print(f"[noalloc] {cfg.name} tokens={n_tokens} splits={S}", flush=True)
        c, k, v = _filled_cache(cfg, n_tokens)
        q = dev(synth.queries(cfg))
        need = c.lib.kv_attention_workspace_bytes(c.params, 1, S)
        assert need <= _lib.NOALLOC_WS_BYTES
        want = c.attention([0], q, cfg.scale, S)
        out = torch.full_like(want, 0x7FC1)  # NaN pattern: every element must be written
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        c.attention_noalloc([0], q, cfg.scale, S, out)
        after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        torch.cuda.synchronize()
        assert after == before, "the allocation-free entry point allocated through torch"
        assert torch.equal(out, want), f"{cfg.name}: differs from kv_decode_attention"
        ref = oracle.attention(oracle.BF16, synth.queries(cfg)[0], k, v, cfg.scale)
        err = row_rel_err(host(out)[0], ref)
        assert err <= 4e-3, err
        flags, _ = c.status()
        assert flags == 0


def test_noalloc_refuses_oversized_partials():
    cfg = synth.config(2)
    c, _, _ = _filled_cache(cfg, 4096 + 5)
    q = dev(synth.queries(cfg))
    out = torch.zeros((1, cfg.Hq, cfg.D), dtype=torch.int16, device="cuda")
    from decode_attention_calibrate_amd import _lib
    S = 1024  # 32 heads x 1024 splits x 130 floats = 17.0 MB > 16 MiB
    assert c.lib.kv_attention_workspace_bytes(c.params, 1, S) > _lib.NOALLOC_WS_BYTES
    with pytest.raises(_lib.KVCError) as ei:
        c.attention_noalloc([0], q, cfg.scale, S, out)
    assert ei.value.code == _lib.ESMALLWS
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0  # nothing ran
    # the largest split count that fits still works and matches
    S = 1008
    want = c.attention([0], q, cfg.scale, S)
    got = c.attention_noalloc([0], q, cfg.scale, S, torch.empty_like(want))
    assert torch.equal(got, want)
