"""Corrupt stored tiles on the GPU (GAAC page §3.1: tags 3 is not a mode; the escape area has a
fixed capacity): one compressed tile's tag words are overwritten on the device with either
raw-without-escape pairs (an invalid tag) or every group raw (escape units far past the
capacity).  Decode attention and kv_decode_blocks must set the sticky corrupt bit, stay inside
the tile (every tag-driven read is bounded: the escape pieces by the capacity, the rebuild's
escape units by the staged pieces), and leave every other KV head's results bit-identical.  The
oracle's decoder rejects the same corruptions (tests/test_oracle_codec.py)."""
import numpy as np
import pytest
import torch

import synth
from kvtest import dev, host, new_cache

pytestmark = pytest.mark.gpu

CORRUPT = 8  # KVC_STATUS_CORRUPT


def _cache(T, Gt):
    cfg = synth.config(0)  # 2 KV heads, 4 query heads, D = 64
    g, toks = synth.sequence_tokens(cfg)
    k, v = toks[0]
    c = new_cache(Hkv=2, Hq=4, D=64, T=T, max_seqs=1, max_blocks=1024 // T + 2, Gt=Gt)
    c.calibrate(dev(k[:256]), dev(v[:256]))
    c.append([0], dev(k[None, :1000]), dev(v[None, :1000]))
    return cfg, c, k, v


def _corrupt(c, blk, kv, h, how):
    """Overwrite the tag planes of one compressed tile in place on the device."""
    e = int(c.table()[((0 * c.params.max_blocks_per_seq + blk) * 2 + kv) * c.Hkv + h].item()) & 0xFFFFFFFF
    assert e != 0xFFFFFFFF and not (e >> 31), "need a compressed tile"
    slot = e & 0xFFFFFF
    n_groups = c.T // c.params.group_tokens * c.D
    pw = (n_groups + 31) // 32  # 32-bit words per tag plane
    tags = c.buffers["comp_pool"].view(-1, c.slot_stride)[slot, :8 * pw].view(torch.int32)
    if how == "raw_without_escape":
        tags[:pw] = 0                       # plane E
        tags[pw:] = -1                      # plane R
    else:                                   # every group raw: escape units far past the capacity
        tags[:] = -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("how", ["raw_without_escape", "escape_overrun"])
@pytest.mark.parametrize("T,Gt", [(64, 16), (16, 16), (64, 8)])
def test_corrupt_tags_flagged_and_contained(T, Gt, how):
    print(f"[corrupt] T={T} G={Gt} {how}", flush=True)
    cfg, c, k, v = _cache(T, Gt)
    q = dev(synth.queries(cfg))
    clean = host(c.attention([0], q, cfg.scale, 4))
    kd0, vd0 = c.decode_blocks(0, 0, 1000 // T)
    flags, _ = c.status()
    assert flags == 0
    _corrupt(c, blk=3, kv=0, h=1, how=how)   # K tile of block 3, KV head 1 (query heads 2, 3)
    out = host(c.attention([0], q, cfg.scale, 4))
    flags, _ = c.status()
    assert flags & CORRUPT, "attention did not flag the corrupt tile"
    assert np.array_equal(out[0, :2], clean[0, :2]), "KV head 0 changed"
    # kv_decode_blocks on a second cache with the same corruption
    cfg, c2, _, _ = _cache(T, Gt)
    _corrupt(c2, blk=3, kv=0, h=1, how=how)
    kd, vd = c2.decode_blocks(0, 0, 1000 // T)
    flags, _ = c2.status()
    assert flags & CORRUPT, "decode_blocks did not flag the corrupt tile"
    kd, vd, kd0, vd0 = host(kd), host(vd), host(kd0), host(vd0)
    assert np.array_equal(vd, vd0) and np.array_equal(kd[:, 0], kd0[:, 0]), "other tiles changed"
    bad = slice(3 * T, 4 * T)
    keep = np.ones(kd.shape[0], bool)
    keep[bad] = False
    assert np.array_equal(kd[keep, 1], kd0[keep, 1]), "other blocks of head 1 changed"
