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
              esc_cap=-1, perm_seed=0, fmt=oracle.BF16, Gt=16):
    from decode_attention_calibrate_amd import KVCache
    n_tiles = max_seqs * max_blocks * 2 * Hkv
    return KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=max_seqs,
                   max_blocks_per_seq=max_blocks, group_tokens=Gt,
                   num_comp_slots=(n_tiles if comp_slots is None else comp_slots) if compressed else 0,
                   num_raw_slots=(n_tiles if raw_slots is None else raw_slots), compressed=compressed,
                   esc_cap_bytes=esc_cap, perm_seed=perm_seed, dtype=fmt)


def row_rel_err(out_bits: np.ndarray, ref: np.ndarray) -> float:
    """max over (seq, head) rows of max_c |o - r| / max_c |r|."""
    o = bf16_to_f64(out_bits).reshape(-1, out_bits.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    return float(np.max(np.max(np.abs(o - r), axis=1) / np.max(np.abs(r), axis=1)))


def gpu_tile_bytes(cache, seq, blk, kv, h):
    """(is_raw, esc_units, bytes) of one finished tile as the GPU stored it."""
    e = int(cache.table()[((seq * cache.params.max_blocks_per_seq + blk) * 2 + kv) * cache.Hkv + h].item()) & 0xFFFFFFFF
    assert e != 0xFFFFFFFF, "unallocated tile"
    slot = e & 0xFFFFFF
    if e >> 31:
        n = cache.T * cache.D * cache.EB
        return True, 0, cache.buffers["raw_pool"][slot * n:(slot + 1) * n].cpu().numpy()
    st = cache.slot_stride
    return False, (e >> 24) & 0x7F, cache.buffers["comp_pool"][slot * st:(slot + 1) * st].cpu().numpy()


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
    for sid, s, b, kv, h in jobs:
        raw, units, got = gpu_tile_bytes(cache, sid, b, kv, h)
        t = s.tiles[b]
        assert raw == bool(t["is_raw"][kv, h]), (sid, b, kv, h)
        if raw:
            want = t["data"][kv, h][:lay["raw_bytes"]]
        else:
            want = t["data"][kv, h][:lay["stride"]]
            assert units == (int(t["esc"][kv, h]) + 15) // 16, (sid, b, kv, h)
        if not np.array_equal(got, want):
            diff = np.nonzero(got != want)[0]
            raise AssertionError(f"tile seq={sid} blk={b} kv={kv} h={h} raw={raw}: {diff.size} bytes differ, "
                                 f"first at {diff[:8].tolist()}")
    return len(jobs)
