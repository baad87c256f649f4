"""KVCache: one layer of lossless compressed (or uncompressed) paged KV cache on one GPU.

A thin wrapper over the C ABI: it allocates the device buffers as torch tensors, passes
pointers, sizes and the current HIP stream, and raises on error codes.  All computation runs
in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _elem(t: torch.Tensor, what: str, nbytes: int = 2) -> torch.Tensor:
    if not t.is_cuda or not t.is_contiguous() or t.element_size() != nbytes:
        kind = "2-byte (BF16 bits)" if nbytes == 2 else "1-byte (FP8 bits)"
        raise ValueError(f"{what} must be a contiguous {kind} CUDA tensor")
    return t


class KVCache:
    def __init__(self, *, num_kv_heads: int, num_q_heads: int, head_dim: int, block_tokens: int,
                 max_seqs: int, max_blocks_per_seq: int, num_comp_slots: int, num_raw_slots: int,
                 compressed: bool = True, group_tokens: int = 16, esc_cap_bytes: int = -1, dtype: int = L.BF16,
                 device: str | torch.device = "cuda", perm_seed: int = 0, mode_set: int = 0, base_versions: int = 1):
        self.lib = L.load()
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.params = L.Params(dtype, num_kv_heads, num_q_heads, head_dim, block_tokens, group_tokens, esc_cap_bytes,
                               1 if compressed else 0, max_seqs, max_blocks_per_seq, num_comp_slots, num_raw_slots,
                               mode_set, base_versions)
        self.mode_set = mode_set
        self.base_versions = max(1, base_versions)
        sizes = (ctypes.c_size_t * L.NUM_BUFFERS)()
        stride = ctypes.c_size_t()
        L.check(self.lib.kv_buffer_sizes(ctypes.byref(self.params), sizes, ctypes.byref(stride)))
        self.slot_stride = stride.value
        self.T, self.D, self.Hkv, self.Hq = block_tokens, head_dim, num_kv_heads, num_q_heads
        self.dtype = dtype
        self.EB = 2 if dtype == L.BF16 else 1  # bytes per cached element
        self.compressed = bool(compressed)
        self.buffers = {}
        for name, sz in zip(L.BUFFER_NAMES, sizes):
            self.buffers[name] = torch.empty(max(int(sz), 16), dtype=torch.uint8, device=self.device)
        self._bufs = L.Buffers(*[_ptr(self.buffers[n]) if sizes[i] else None for i, n in enumerate(L.BUFFER_NAMES)])
        h = ctypes.c_void_p()
        L.check(self.lib.kv_cache_create(ctypes.byref(self.params), ctypes.byref(self._bufs), perm_seed,
                                         self._stream(), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.kv_cache_destroy(h)
            self.handle = None

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    # ---- the four calls of the method ----
    def _shape(self, t: torch.Tensor, what: str, lead: int):
        if t.dim() != lead + 2 or tuple(t.shape[lead:]) != (self.Hkv, self.D) or t.device != self.device:
            raise ValueError(f"{what} must have shape [...{lead} dims...][{self.Hkv}][{self.D}] on {self.device}")

    def calibrate(self, k: torch.Tensor, v: torch.Tensor):
        """k, v: [n][Hkv][D] element bits."""
        _elem(k, "k", self.EB), _elem(v, "v", self.EB)
        self._shape(k, "k", 1), self._shape(v, "v", 1)
        if k.shape != v.shape:
            raise ValueError("k and v differ in shape")
        L.check(self.lib.kv_calibrate(self.handle, _ptr(k), _ptr(v), k.shape[0], self._stream()))

    def recalibrate(self, k: torch.Tensor, v: torch.Tensor):
        """kv_recalibrate: a new base version from k, v [n][Hkv][D] element bits for the blocks
        finished from now on; stored blocks keep theirs."""
        _elem(k, "k", self.EB), _elem(v, "v", self.EB)
        self._shape(k, "k", 1), self._shape(v, "v", 1)
        if k.shape != v.shape:
            raise ValueError("k and v differ in shape")
        L.check(self.lib.kv_recalibrate(self.handle, _ptr(k), _ptr(v), k.shape[0], self._stream()))

    def append(self, seq_ids, k: torch.Tensor, v: torch.Tensor):
        """k, v: [n_seqs][n_tokens][Hkv][D] element bits."""
        _elem(k, "k", self.EB), _elem(v, "v", self.EB)
        self._shape(k, "k", 2), self._shape(v, "v", 2)
        if k.shape[0] != len(seq_ids) or k.shape != v.shape:
            raise ValueError("k, v must be [n_seqs][n_tokens][Hkv][D] with n_seqs = len(seq_ids)")
        ids = (ctypes.c_int32 * len(seq_ids))(*seq_ids)
        L.check(self.lib.kv_encode_append(self.handle, ids, len(seq_ids), _ptr(k), _ptr(v), k.shape[1],
                                          self._stream()))

    def decode_blocks(self, seq: int, first: int, n: int, out=None):
        if out is None:
            k = torch.empty((n * self.T, self.Hkv, self.D), dtype=torch.int16 if self.EB == 2 else torch.uint8,
                            device=self.device)
            v = torch.empty_like(k)
        else:
            k, v = out
            for t in (k, v):
                _elem(t, "out", self.EB)
                if tuple(t.shape) != (n * self.T, self.Hkv, self.D):
                    raise ValueError("decode_blocks outputs must be [n*T][Hkv][D]")
        L.check(self.lib.kv_decode_blocks(self.handle, seq, first, n, _ptr(k), _ptr(v), self._stream()))
        return k, v

    def prefill_attention(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, scale: float, out=None) -> torch.Tensor:
        """Causal attention of q ([n_q][Hq][D] BF16 bits, the last n_q positions) over k, v
        ([n_kv][Hkv][D] elements, e.g. from decode_blocks) -> [n_q][Hq][D] BF16 bits."""
        n_kv, n_q = k.shape[0], q.shape[0]
        for t in (k, v):
            _elem(t, "k/v", self.EB)
            if tuple(t.shape) != (n_kv, self.Hkv, self.D):
                raise ValueError("k and v must be [n_kv][Hkv][D]")
        if tuple(q.shape) != (n_q, self.Hq, self.D) or q.device != self.device:
            raise ValueError(f"q must be [n_q][{self.Hq}][{self.D}] on {self.device}")
        if out is None:
            out = torch.empty((n_q, self.Hq, self.D), dtype=torch.int16, device=self.device)
        L.check(self.lib.kv_prefill_attention(self.handle, _ptr(k), _ptr(v), n_kv, _ptr(q), n_q, float(scale), _ptr(out),
                                              self._stream()))
        return out

    def workspace(self, n_seqs: int, n_splits: int) -> torch.Tensor:
        nb = self.lib.kv_attention_workspace_bytes(ctypes.byref(self.params), n_seqs, n_splits)
        return torch.empty(max(nb, 16), dtype=torch.uint8, device=self.device)

    def attention(self, seq_ids, q: torch.Tensor, scale: float, n_splits: int, ws=None, out=None) -> torch.Tensor:
        """q: [n_seqs][Hq][D] BF16 bits -> out [n_seqs][Hq][D] BF16 bits."""
        n = len(seq_ids)
        self._check_q(q, n)
        if ws is None:
            ws = self.workspace(n, n_splits)
        if out is None:
            out = torch.empty((n, self.Hq, self.D), dtype=torch.int16, device=self.device)
        self._check_out(out, n)
        ids = (ctypes.c_int32 * n)(*seq_ids)
        L.check(self.lib.kv_decode_attention(self.handle, ids, n, _ptr(q), float(scale), n_splits, _ptr(ws),
                                             ws.numel(), _ptr(out), self._stream()))
        return out

    def attention_noalloc(self, seq_ids, q: torch.Tensor, scale: float, n_splits: int, out: torch.Tensor) -> torch.Tensor:
        """kv_decode_attention_noalloc: as attention(), with the split partials in the library's fixed
        per-GPU workspace (no workspace argument; out must be given, so nothing is allocated)."""
        n = len(seq_ids)
        self._check_q(q, n)
        self._check_out(out, n)
        ids = (ctypes.c_int32 * n)(*seq_ids)
        L.check(self.lib.kv_decode_attention_noalloc(self.handle, ids, n, _ptr(q), float(scale), n_splits, _ptr(out),
                                                     self._stream()))
        return out

    def _check_q(self, q: torch.Tensor, n: int):
        _elem(q, "q")
        if tuple(q.shape) != (n, self.Hq, self.D) or q.device != self.device:
            raise ValueError(f"q must be [{n}][{self.Hq}][{self.D}] on {self.device}")

    def _check_out(self, out: torch.Tensor, n: int):
        _elem(out, "out")
        if tuple(out.shape) != (n, self.Hq, self.D) or out.device != self.device:
            raise ValueError(f"out must be [{n}][{self.Hq}][{self.D}] on {self.device}")

    def attention_partials(self, seq_ids, q: torch.Tensor, scale: float, n_splits: int, ws: torch.Tensor):
        self._check_q(q, len(seq_ids))
        ids = (ctypes.c_int32 * len(seq_ids))(*seq_ids)
        L.check(self.lib.kv_attention_partials(self.handle, ids, len(seq_ids), _ptr(q), float(scale), n_splits,
                                               _ptr(ws), ws.numel(), self._stream()))

    def attention_combine(self, seq_ids, q: torch.Tensor, scale: float, n_splits: int, ws: torch.Tensor,
                          out: torch.Tensor):
        n = len(seq_ids)
        self._check_q(q, n)
        self._check_out(out, n)
        ids = (ctypes.c_int32 * n)(*seq_ids)
        L.check(self.lib.kv_attention_combine(self.handle, ids, n, _ptr(q), float(scale), n_splits, _ptr(ws),
                                              ws.numel(), _ptr(out), self._stream()))
        return out

    def decode_step(self, seq_ids, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, scale: float,
                    n_splits: int, ws=None, out=None) -> torch.Tensor:
        """Append one token per sequence (k_new, v_new: [n][1][Hkv][D] or [n][Hkv][D] elements)
        and attend over every token including it."""
        n = len(seq_ids)
        self._check_q(q, n)
        for t, what in ((k_new, "k_new"), (v_new, "v_new")):
            _elem(t, what, self.EB)
            if t.numel() != n * self.Hkv * self.D or not t.is_contiguous() or t.device != self.device:
                raise ValueError(f"{what} must be a contiguous [{n}][{self.Hkv}][{self.D}] tensor on {self.device}")
        if ws is None:
            ws = self.workspace(n, n_splits)
        if out is None:
            out = torch.empty((n, self.Hq, self.D), dtype=torch.int16, device=self.device)
        self._check_out(out, n)
        ids = (ctypes.c_int32 * n)(*seq_ids)
        L.check(self.lib.kv_decode_step(self.handle, ids, n, _ptr(k_new), _ptr(v_new), _ptr(q), float(scale), n_splits,
                                        _ptr(ws), ws.numel(), _ptr(out), self._stream()))
        return out

    # ---- diagnostics ----
    def tile_stats(self, seq: int, first: int, n: int) -> torch.Tensor:
        """kv_tile_stats: [n][2][stored heads][7] int32 {state, bytes, groups per mode index [4], base
        version}; a 256-channel head is stored as two half-heads (2 Hkv rows)."""
        out = torch.empty((n, 2, self.Hkv * (2 if self.D == 256 else 1), 7), dtype=torch.int32, device=self.device)
        L.check(self.lib.kv_tile_stats(self.handle, seq, first, n, _ptr(out), self._stream()))
        return out

    def window_coverage(self, x: torch.Tensor, window: int) -> torch.Tensor:
        """kv_window_coverage of x [n][Hkv][D] elements -> [Hkv][D] int32 counts."""
        _elem(x, "x", self.EB)
        self._shape(x, "x", 1)
        out = torch.empty((self.Hkv, self.D), dtype=torch.int32, device=self.device)
        L.check(self.lib.kv_window_coverage(self.handle, _ptr(x), x.shape[0], window, _ptr(out), self._stream()))
        return out

    # ---- bookkeeping ----
    def release(self, seq: int):
        L.check(self.lib.kv_release_seq(self.handle, seq, self._stream()))

    def seq_length(self, seq: int) -> int:
        n = ctypes.c_int32()
        L.check(self.lib.kv_seq_length(self.handle, seq, ctypes.byref(n)))
        return n.value

    def status(self):
        flags = ctypes.c_uint32()
        st = L.Stats()
        L.check(self.lib.kv_get_status(self.handle, ctypes.byref(flags), ctypes.byref(st), self._stream()))
        return flags.value, dict(comp_tiles=st.comp_tiles, raw_tiles=st.raw_tiles, groups=list(st.groups),
                                 esc_bytes=st.esc_bytes, comp_free=st.comp_free, raw_free=st.raw_free)

    # ---- raw views of the device state (tests) ----
    def table(self) -> torch.Tensor:
        return self.buffers["block_table"].view(torch.int32)

    def _version_offset(self, version: int) -> int:
        if not 0 <= version < self.base_versions:
            raise ValueError("no such base version")
        return version * (6 if self.mode_set == 1 else 4) * self.Hkv * self.D

    def bases(self, version: int = 0) -> torch.Tensor:
        """The b3 and b4 bases of one base version, [2 (K, V)][2 (b3, b4)][Hkv][D]."""
        n = self._version_offset(version)
        return self.buffers["bases"][n: n + 4 * self.Hkv * self.D].view(2, 2, self.Hkv, self.D)

    def bases2(self, version: int = 0) -> torch.Tensor:
        """The 2-bit-window bases of mode set 1, [2 (K, V)][Hkv][D]."""
        n = self._version_offset(version) + 4 * self.Hkv * self.D
        return self.buffers["bases"][n: n + 2 * self.Hkv * self.D].view(2, self.Hkv, self.D)


def admit_fcfs(*, num_kv_heads: int, head_dim: int, block_tokens: int, budget_bytes: int, lengths,
               compressed: bool = True, raw_share: float = 1.0 / 64, group_tokens: int = 16, dtype: int = L.BF16,
               mode_set: int = 0, num_q_heads: int | None = None):
    """kv_admit_fcfs: (admitted count, compressed slots, raw slots) for one layer's KV byte budget
    and requests admitted first come, first served (host only)."""
    lib = L.load()
    p = L.Params(dtype, num_kv_heads, num_q_heads or num_kv_heads, head_dim, block_tokens, group_tokens, -1,
                 1 if compressed else 0, 1, 1, 1, 1, mode_set, 1)
    arr = (ctypes.c_int32 * len(lengths))(*[int(x) for x in lengths])
    n, nc, nr = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    L.check(lib.kv_admit_fcfs(ctypes.byref(p), int(budget_bytes), float(raw_share), arr, len(lengths), ctypes.byref(n),
                              ctypes.byref(nc), ctypes.byref(nr)))
    return n.value, nc.value, nr.value



def read_probe(src: torch.Tensor, bytes_per_wave: int, waves: int, sink: torch.Tensor | None = None) -> torch.Tensor:
    """kv_read_probe over the first waves * bytes_per_wave bytes of the contiguous device tensor
    src, enqueued on src's current stream; returns the [waves][64] int32 checksum words (sink)."""
    lib = L.load()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if src.numel() * src.element_size() < waves * bytes_per_wave:
        raise ValueError("src holds fewer than waves * bytes_per_wave bytes")
    if sink is None:
        sink = torch.empty((waves, 64), dtype=torch.int32, device=src.device)
    elif not sink.is_cuda or not sink.is_contiguous() or sink.numel() * sink.element_size() < waves * 256:
        raise ValueError("sink must be a contiguous device tensor of waves * 64 32-bit words")
    L.check(lib.kv_read_probe(_ptr(src), int(bytes_per_wave), int(waves), _ptr(sink),
                              ctypes.c_void_p(torch.cuda.current_stream(src.device).cuda_stream)))
    return sink
