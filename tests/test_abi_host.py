"""The C-ABI library loads, exports every entry point of include/kvc.h, and validates
arguments on the host (no GPU needed: none of these calls reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    import decode_attention_calibrate_amd as K
    if not os.path.exists(K.LIB_PATH):
        pytest.fail("libkvc.so is not built: run __graft_entry__.build()")
    return K


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(kv_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(K):
    lib = ctypes.CDLL(K.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K._lib.SIGNATURES), "binding and header disagree"


def _params(K, **kw):
    d = dict(dtype=0, num_kv_heads=8, num_q_heads=32, head_dim=128, block_tokens=64, group_tokens=16,
             esc_cap_bytes=-1, compressed=1, max_seqs=2, max_blocks_per_seq=1024, num_comp_slots=2048,
             num_raw_slots=64, mode_set=0, base_versions=1)
    d.update(kw)
    return K._lib.Params(*[d[f] for f, _ in K._lib.Params._fields_])


def _sizes(K, p):
    lib = K.load()
    sz = (ctypes.c_size_t * 8)()
    st = ctypes.c_size_t()
    rc = lib.kv_buffer_sizes(ctypes.byref(p), sz, ctypes.byref(st))
    return rc, list(sz), st.value, lib.kv_last_error().decode()


@pytest.mark.parametrize("Gt", [16, 8])
@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.E5M2, oracle.E4M3])
@pytest.mark.parametrize("T,D", [(64, 128), (16, 128), (64, 64), (32, 128)])
def test_slot_stride_matches_format(K, T, D, fmt, Gt):
    """The library's slot stride equals the stride of FORMAT v1 as the oracle lays it out."""
    rc, sz, stride, _ = _sizes(K, _params(K, block_tokens=T, head_dim=D, dtype=fmt, group_tokens=Gt))
    assert rc == 0
    lay = oracle.layout(oracle.Params(fmt, T, D, Gt))
    eb = 2 if fmt == oracle.BF16 else 1
    assert stride == lay["stride"]
    assert sz[0] == 2048 * stride
    assert sz[1] == 64 * T * D * eb == 64 * lay["raw_bytes"]
    assert sz[2] == 2 * 2 * 8 * T * D * eb
    assert sz[3] == 4 * 8 * D
    assert sz[4] == 2 * 1024 * 2 * 8 * 4
    assert sz[5] == 2048 * 4 and sz[6] == 64 * 4 and sz[7] == 128 * (2 * 16 + 1 + 64)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -1), (dict(num_q_heads=12), -1), (dict(num_q_heads=8 * 17), -1),
    (dict(block_tokens=40), -1), (dict(esc_cap_bytes=24), -1), (dict(max_seqs=0), -1),
    (dict(num_comp_slots=0), -1), (dict(compressed=0, num_raw_slots=0), -1), (dict(dtype=7), -1),
    (dict(group_tokens=4), -3), (dict(group_tokens=32), -3), (dict(block_tokens=128), -3),
    (dict(block_tokens=48), -3),
])
def test_parameter_validation(K, kw, code):
    rc, _, _, msg = _sizes(K, _params(K, **kw))
    assert rc == code and msg


def test_workspace_bytes(K):
    lib = K.load()
    p = _params(K)
    assert lib.kv_attention_workspace_bytes(ctypes.byref(p), 3, 64) == 3 * 32 * 64 * (128 + 2) * 4
    assert lib.kv_attention_workspace_bytes(ctypes.byref(p), 0, 64) == 0


def test_null_handles_rejected(K):
    lib = K.load()
    ids = (ctypes.c_int32 * 1)(0)
    assert lib.kv_calibrate(None, None, None, 1, None) == -1
    assert lib.kv_encode_append(None, ids, 1, None, None, 1, None) == -1
    assert lib.kv_decode_attention(None, ids, 1, None, 1.0, 1, None, 0, None, None) == -1
    assert lib.kv_get_status(None, None, None, None) == -1
    assert b"NULL" in lib.kv_last_error()


def test_head_dim_256_is_stored_as_half_heads(K):
    """A 256-channel head is two 128-channel half-heads: every buffer size and the slot stride are
    those of the same cache with twice the KV heads at head_dim 128."""
    rc, sz, stride, _ = _sizes(K, _params(K, head_dim=256, num_kv_heads=8, num_q_heads=32))
    rc2, sz2, stride2, _ = _sizes(K, _params(K, head_dim=128, num_kv_heads=16, num_q_heads=64))
    assert rc == 0 and rc2 == 0
    assert sz == sz2 and stride == stride2 == oracle.layout(oracle.Params(oracle.BF16, 64, 128, 16))["stride"]
