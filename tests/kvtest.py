"""Helpers shared by the GPU tests: move seeded inputs to the device, build a cache through the
C ABI, build the matching oracle state, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def dev(a: np.ndarray, fmt: int = oracle.BF16) -> torch.Tensor:
    """Element bits to the device: BF16 as 16-bit words, FP8 as bytes."""
    if fmt == oracle.BF16:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.uint8)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device element bits back as uint16 (FP8 bytes widened)."""
    if t.dtype == torch.uint8:
        return t.cpu().numpy().astype(np.uint16)
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def new_cache(*, Hkv, Hq, D, T, max_seqs, max_blocks, comp_slots=None, raw_slots=None, compressed=True,
              esc_cap=-1, perm_seed=0, fmt=oracle.BF16, Gt=16, mode_set=0, base_versions=1):
    from decode_attention_calibrate_amd import KVCache
    n_tiles = max_seqs * max_blocks * 2 * Hkv
    return KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=max_seqs,
                   max_blocks_per_seq=max_blocks, group_tokens=Gt,
                   num_comp_slots=(n_tiles if comp_slots is None else comp_slots) if compressed else 0,
                   num_raw_slots=(n_tiles if raw_slots is None else raw_slots), compressed=compressed,
                   esc_cap_bytes=esc_cap, perm_seed=perm_seed, dtype=fmt, mode_set=mode_set,
                   base_versions=base_versions)


# table entry fields (include/kvc.h): bit 31 raw, bits 29..30 base version, bits 23..28 escape
# units of 16 bytes, bits 0..22 slot
SLOT_MASK = 0x7FFFFF


def esc_units(e: int) -> int:
    return (e >> 23) & 0x3F


def row_rel_err(out_bits: np.ndarray, ref: np.ndarray) -> float:
    """max over (seq, head) rows of max_c |o - r| / max_c |r|."""
    o = bf16_to_f64(out_bits).reshape(-1, out_bits.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    return float(np.max(np.max(np.abs(o - r), axis=1) / np.max(np.abs(r), axis=1)))


def gpu_tile_bytes(cache, seq, blk, kv, h):  # one tile; compare_tiles reads many at once
    """(is_raw, esc_units, bytes) of one finished tile as the GPU stored it."""
    e = int(cache.table()[((seq * cache.params.max_blocks_per_seq + blk) * 2 + kv) * cache.Hkv + h].item()) & 0xFFFFFFFF
    assert e != 0xFFFFFFFF, "unallocated tile"
    slot = e & SLOT_MASK
    if e >> 31:
        n = cache.T * cache.D * cache.EB
        return True, 0, cache.buffers["raw_pool"][slot * n:(slot + 1) * n].cpu().numpy()
    st = cache.slot_stride
    return False, esc_units(e), cache.buffers["comp_pool"][slot * st:(slot + 1) * st].cpu().numpy()


def oracle_layer(p: oracle.Params, Hkv: int, k_cal: np.ndarray, v_cal: np.ndarray, seq_tokens, chunks=None):
    """Oracle bases and Sequences fed the same appends as the GPU cache."""
    bases = oracle.calibrate_layer(p, k_cal, v_cal)
    seqs = []
    for k, v in seq_tokens:
        s = oracle.Sequence(p, Hkv, bases)
        for a, b in (chunks or [(0, k.shape[0])]):
            if a < min(b, k.shape[0]):
                s.append(k[a:b], v[a:b])
        seqs.append(s)
    return bases, seqs


def _stored_heads(cache) -> int:
    """Heads the table rows count: a 256-channel head is stored as two 128-channel half-heads."""
    return cache.Hkv * (2 if cache.D == 256 else 1)


def _stored_tiles(cache, jobs):
    """(is_raw, esc_units, bytes) per (seq, blk, kv, h) job as the GPU stored them: the table is
    read once and the slots are gathered on the device, so large samples cost one copy."""
    tab = cache.table().cpu().numpy().view(np.uint32)
    Hkv, MB = _stored_heads(cache), cache.params.max_blocks_per_seq
    ent = np.array([tab[((sid * MB + b) * 2 + kv) * Hkv + h] for sid, b, kv, h in jobs], np.uint32)
    assert (ent != 0xFFFFFFFF).all(), "unallocated tile"
    raw = (ent >> 31).astype(bool)
    slot = torch.from_numpy((ent & SLOT_MASK).astype(np.int64)).cuda()
    n_raw = cache.T * min(cache.D, 128) * cache.EB
    comp = cache.buffers["comp_pool"].view(-1, cache.slot_stride) if cache.compressed else None
    rawp = cache.buffers["raw_pool"][: (cache.buffers["raw_pool"].numel() // n_raw) * n_raw].view(-1, n_raw)
    rb = torch.from_numpy(raw).cuda()
    got_c = comp[torch.where(rb, torch.zeros_like(slot), slot)].cpu().numpy() if comp is not None else None
    got_r = rawp[torch.where(rb, slot, torch.zeros_like(slot))].cpu().numpy()
    return [(bool(raw[i]), esc_units(int(ent[i])), got_r[i] if raw[i] else got_c[i]) for i in range(len(jobs))]


def stored_versions(cache, jobs):
    """Base version of each (seq, blk, kv, h) job's compressed tile (-1 for raw tiles)."""
    tab = cache.table().cpu().numpy().view(np.uint32)
    Hkv, MB = _stored_heads(cache), cache.params.max_blocks_per_seq
    out = []
    for sid, b, kv, h in jobs:
        e = int(tab[((sid * MB + b) * 2 + kv) * Hkv + h])
        assert e != 0xFFFFFFFF, "unallocated tile"
        out.append(-1 if e >> 31 else (e >> 29) & 3)
    return out


def compare_tiles(cache, p: oracle.Params, oseqs, seq_ids, sample=None, rng=None):
    """Every (or a sample of) finished tiles: GPU bytes == oracle bytes, same storage form and
    escape length.  Returns the number of tiles compared."""
    lay = oracle.layout(p)
    jobs = []
    for sid, s in zip(seq_ids, oseqs):
        for b in range(len(s.tiles)):
            for kv in range(2):
                for h in range(s.Hkv):
                    jobs.append((sid, s, b, kv, h))
    if sample is not None and len(jobs) > sample:
        idx = (rng or np.random.default_rng(0)).choice(len(jobs), sample, replace=False)
        jobs = [jobs[i] for i in sorted(idx)]
    stored = _stored_tiles(cache, [(sid, b, kv, h) for sid, s, b, kv, h in jobs])
    for (sid, s, b, kv, h), (raw, units, got) in zip(jobs, stored):
        t = s.tiles[b]
        assert raw == bool(t["is_raw"][kv, h]), (sid, b, kv, h)
        if raw:
            want = t["data"][kv, h][:lay["raw_bytes"]]
            got = got[:lay["raw_bytes"]]
        else:
            want = t["data"][kv, h][:lay["stride"]]
            assert units == (int(t["esc"][kv, h]) + 15) // 16, (sid, b, kv, h)
        if not np.array_equal(got, want):
            diff = np.nonzero(got != want)[0]
            raise AssertionError(f"tile seq={sid} blk={b} kv={kv} h={h} raw={raw}: {diff.size} bytes differ, "
                                 f"first at {diff[:8].tolist()}")
    return len(jobs)


def compare_sampled_tiles(cache, p: oracle.Params, bases, toks, n_sample: int, rng):
    """n_sample finished tiles drawn over all sequences: GPU bytes == the oracle's encoding of the
    same tokens with the same bases (only the sampled tiles are encoded by the oracle)."""
    lay = oracle.layout(p)
    b3, b4 = bases
    jobs = []
    per_seq = [k.shape[0] // p.T for k, _ in toks]
    total = sum(per_seq) * 2 * cache.Hkv
    for i in sorted(rng.choice(total, n_sample, replace=False)):
        h = i % cache.Hkv
        kv = (i // cache.Hkv) % 2
        blk = i // (2 * cache.Hkv)
        sid = 0
        while blk >= per_seq[sid]:
            blk -= per_seq[sid]
            sid += 1
        jobs.append((sid, blk, kv, h))
    tiles = np.stack([toks[sid][kv][blk * p.T:(blk + 1) * p.T, h] for sid, blk, kv, h in jobs])
    data, is_raw, esc, _ = oracle.encode_tiles(p, tiles, np.stack([b3[kv, h] for _, _, kv, h in jobs]),
                                               np.stack([b4[kv, h] for _, _, kv, h in jobs]),
                                               np.array([kv for _, _, kv, _ in jobs], np.int32))
    for n, ((sid, blk, kv, h), (raw, units, got)) in enumerate(zip(jobs, _stored_tiles(cache, jobs))):
        assert raw == bool(is_raw[n]), (sid, blk, kv, h)
        size = lay["raw_bytes"] if raw else lay["stride"]
        if not raw:
            assert units == (int(esc[n]) + 15) // 16, (sid, blk, kv, h)
        if not np.array_equal(got[:size], data[n, :size]):
            raise AssertionError(f"tile seq={sid} blk={blk} kv={kv} h={h} raw={raw} differs from the oracle")
    return len(jobs)
