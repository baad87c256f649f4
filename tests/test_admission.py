"""kv_admit_fcfs (host only, no GPU): equal-memory admission (GAAC page §4.5).  The pools it plans
fit the budget and the slot sizes the cache itself reports; requests are admitted first come,
first served until the first one whose blocks plus one spare block no longer fit; the same
budget admits at least as many requests compressed as uncompressed."""
import ctypes

import numpy as np
import pytest


@pytest.fixture(scope="module")
def K():
    import decode_attention_calibrate_amd as K
    return K


def _stride(K, T, Hkv=8, D=128, Gt=16, ms=0):
    lib = K.load()
    p = K._lib.Params(0, Hkv, 4 * Hkv, D, T, Gt, -1, 1, 1, 1, 1, 1, ms)
    sz = (ctypes.c_size_t * 8)()
    st = ctypes.c_size_t()
    assert lib.kv_buffer_sizes(ctypes.byref(p), sz, ctypes.byref(st)) == 0
    return st.value


@pytest.mark.parametrize("T", [16, 64])
@pytest.mark.parametrize("compressed", [True, False])
def test_pools_fit_the_budget_and_admission_is_fcfs(K, T, compressed):
    rng = np.random.default_rng(T + compressed)
    lens = rng.integers(4096, 32768, size=64, endpoint=True).tolist()
    Hkv, D = 8, 128
    raw_tile = T * D * 2
    stride = _stride(K, T)
    for budget in (1 << 28, 1536 << 20, 6 << 30):
        n, nc, nr = K.admit_fcfs(num_kv_heads=Hkv, head_dim=D, block_tokens=T, budget_bytes=budget, lengths=lens,
                                 compressed=compressed)
        used = nc * stride + nr * raw_tile
        assert used <= budget
        if compressed:
            assert nr == int(budget / 64) // raw_tile and nc == (budget - nr * raw_tile) // stride
        else:
            assert nc == 0 and nr == budget // raw_tile
        pool = nc if compressed else nr
        need = [(L // T + 1) * 2 * Hkv for L in lens]
        assert sum(need[:n]) <= pool
        assert n == len(lens) or sum(need[:n + 1]) > pool     # stops at the first request that does not fit


def test_compressed_admits_at_least_as_many(K):
    rng = np.random.default_rng(7)
    for _ in range(20):
        lens = rng.integers(1, 40000, size=50).tolist()
        budget = int(rng.integers(1 << 26, 1 << 32))
        kw = dict(num_kv_heads=8, head_dim=128, block_tokens=16, budget_bytes=budget, lengths=lens)
        assert K.admit_fcfs(**kw)[0] >= K.admit_fcfs(compressed=False, **kw)[0]
        # more budget never admits fewer
        assert K.admit_fcfs(**{**kw, "budget_bytes": 2 * budget})[0] >= K.admit_fcfs(**kw)[0]


def test_admission_argument_errors(K):
    kw = dict(num_kv_heads=8, head_dim=128, block_tokens=16, budget_bytes=1 << 30)
    with pytest.raises(K.KVCError):
        K.admit_fcfs(lengths=[100, 0], **kw)          # a request needs at least one token
    with pytest.raises(K.KVCError):
        K.admit_fcfs(lengths=[100], raw_share=1.5, **kw)
    with pytest.raises(K.KVCError):
        K.admit_fcfs(lengths=[100], budget_bytes=1 << 40, num_kv_heads=8, head_dim=128, block_tokens=16)
