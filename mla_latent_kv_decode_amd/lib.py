"""Thin ctypes binding over the MLA C ABI (``include/mla.h``).

Argument marshalling only: tensors are passed as device pointers
(``tensor.data_ptr()``), ragged metadata as host arrays, streams as the raw
``hipStream_t`` of torch's current stream.  Every step of the computation runs
in the HIP library; this module raises if the library is missing.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB selects another build of the same library (the host-sanitized one
# in the CPU tests); by default the in-tree libmla.so
LIB_PATH = os.environ.get("MLA_LIB") or os.path.join(_PKG, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_SHAPE = -2
MLA_ERR_CAPACITY = -3
MLA_ERR_STATE = -4
MLA_ERR_HIP = -5
MLA_ERR_WORKSPACE = -6
MLA_BF16 = 0
MLA_F32 = 1
MLA_KV_DTYPE = 0
MLA_KV_FP8_E4M3 = 1
MLA_ABSORB_FACTORED = 0
MLA_ABSORB_MATERIALIZED = 1

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class MLAConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("qk_nope", ctypes.c_int32), ("qk_rope", ctypes.c_int32),
                ("v_head", ctypes.c_int32), ("kv_lora", ctypes.c_int32),
                ("q_lora", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("kv_storage", ctypes.c_int32),
                ("rope_scale", ctypes.c_float), ("rope_orig_max", ctypes.c_int32),
                ("yarn_beta_fast", ctypes.c_float), ("yarn_beta_slow", ctypes.c_float),
                ("yarn_mscale", ctypes.c_float), ("absorb", ctypes.c_int32)]


class MLADecodeArgs(ctypes.Structure):
    """struct mla_decode_args (include/mla.h)."""
    _fields_ = [("hidden", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("seq_len", ctypes.POINTER(ctypes.c_int32)),
                ("seq_off", ctypes.POINTER(ctypes.c_int64)),
                ("block_table", ctypes.POINTER(ctypes.c_int32)),
                ("max_pages", ctypes.c_int32), ("page_rows", ctypes.c_int32),
                ("cache", ctypes.c_void_p), ("cache_rows", ctypes.c_int64),
                ("append", ctypes.c_int32), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


MLA_MAX_Q_LEN = 16

# name -> (restype, argtypes)
_SIGS = {
    "mla_abi_version": (ctypes.c_int, []),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, [_P]),
    "mla_config_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig)]),
    "mla_cache_row_bytes": (ctypes.c_size_t, [ctypes.POINTER(MLAConfig)]),
    "mla_append_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I64P, ctypes.c_int32,
                                        ctypes.c_int64]),
    "mla_decode_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I64P, _I32P,
                                        ctypes.c_int32, ctypes.c_int64]),
    "mla_prefill_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I32P, _I64P,
                                         ctypes.c_int32, ctypes.c_int64]),
    "mla_decode_paged_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I32P,
                                              ctypes.c_int32, ctypes.c_int32, _I32P,
                                              ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]),
    "mla_prefill_paged_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I32P, _I32P,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64]),
    "mla_create": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _P, ctypes.POINTER(_P)]),
    "mla_destroy": (ctypes.c_int, [_P]),
    "mla_set_stream": (ctypes.c_int, [_P, _P]),
    "mla_absorb_weights": (ctypes.c_int, [_P] * 9),
    "mla_append_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32]),
    "mla_append_latent": (ctypes.c_int, [_P, _P, _I32P, _I64P, ctypes.c_int32, _P,
                                         ctypes.c_int64, _P, ctypes.c_size_t]),
    "mla_cache_write_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32]),
    "mla_cache_write": (ctypes.c_int, [_P, _P, _I64P, ctypes.c_int32, _P, ctypes.c_int64, _P,
                                       ctypes.c_size_t]),
    "mla_cache_store": (ctypes.c_int, [_P, _P, _I64P, ctypes.c_int32, _P, ctypes.c_int64, _P,
                                       ctypes.c_size_t]),
    "mla_decode_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int64]),
    "mla_decode": (ctypes.c_int, [_P, _P, _I32P, _I64P, _I32P, ctypes.c_int32, _P,
                                  ctypes.c_int64, _P, _P, ctypes.c_size_t]),
    "mla_decode_step_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int64]),
    "mla_decode_step": (ctypes.c_int, [_P, _P, _I32P, _I64P, _I32P, ctypes.c_int32, _P,
                                       ctypes.c_int64, _P, _P, ctypes.c_size_t]),
    "mla_decode_step_noalloc": (ctypes.c_int, [_P, _P, _I32P, _I64P, _I32P, ctypes.c_int32, _P,
                                               ctypes.c_int64, _P]),
    "mla_decode_paged": (ctypes.c_int, [_P, _P, _I32P, _I32P, ctypes.c_int32, ctypes.c_int32,
                                        _I32P, ctypes.c_int32, _P, ctypes.c_int64, _P, _P,
                                        ctypes.c_size_t]),
    "mla_decode_step_paged": (ctypes.c_int, [_P, _P, _I32P, _I32P, ctypes.c_int32,
                                             ctypes.c_int32, _I32P, ctypes.c_int32, _P,
                                             ctypes.c_int64, _P, _P, ctypes.c_size_t]),
    "mla_decode_ex_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig),
                                           ctypes.POINTER(MLADecodeArgs)]),
    "mla_decode_ex_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_int64, ctypes.c_int32]),
    "mla_decode_ex": (ctypes.c_int, [_P, ctypes.POINTER(MLADecodeArgs)]),
    "mla_decode_stage_offsets": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "mla_decode_plan_tokens": (ctypes.c_int, [ctypes.c_int32, _I32P, ctypes.c_int32,
                                              ctypes.c_int32, _I32P, _I32P, _I32P, _I32P,
                                              _I32P, _I32P]),
    "mla_decode_plan": (ctypes.c_int, [ctypes.c_int32, _I32P, ctypes.c_int32, _I32P, _I32P,
                                       _I32P, _I32P, _I32P, _I32P]),
    "mla_core_timing": (ctypes.c_int, [_P, ctypes.c_int32]),
    "mla_core_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                            _I32P]),
    "mla_prefill_step_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32,
                                                           ctypes.c_int64]),
    "mla_prefill_step_check": (ctypes.c_int, [ctypes.POINTER(MLAConfig), _I32P, _I32P, _I64P,
                                              ctypes.c_int32, ctypes.c_int64]),
    "mla_prefill_step": (ctypes.c_int, [_P, _P, _I32P, _I32P, _I64P, ctypes.c_int32, _P,
                                        ctypes.c_int64, _P, _P, ctypes.c_size_t]),
    "mla_prefill_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int64]),
    "mla_prefill": (ctypes.c_int, [_P, _P, _I32P, _I32P, _I64P, ctypes.c_int32, _P,
                                   ctypes.c_int64, _P, _P, ctypes.c_size_t]),
    "mla_prefill_paged_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int64]),
    "mla_prefill_paged": (ctypes.c_int, [_P, _P, _I32P, _I32P, _I32P, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P,
                                         _P, ctypes.c_size_t]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"MLA HIP library not found at {path}; build it with "
                           "`python -m mla_latent_kv_decode_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def make_config(dims, dtype: str, softmax_scale: float = 0.0, kv: str = "dtype",
                absorb: str = "factored") -> MLAConfig:
    """kv: "dtype" (cache rows in the layer dtype) or "fp8" (FP8 E4M3 rows);
    absorb: "factored" or "materialized" (mla_absorb)."""
    return MLAConfig(dims.hidden, dims.n_heads, dims.qk_nope, dims.qk_rope, dims.v_head,
                     dims.kv_lora, dims.q_lora, float(dims.rope_base), float(dims.rms_eps),
                     float(softmax_scale), MLA_BF16 if dtype == "bf16" else MLA_F32,
                     MLA_KV_FP8_E4M3 if kv == "fp8" else MLA_KV_DTYPE,
                     float(getattr(dims, "rope_scale", 1.0)),
                     int(getattr(dims, "rope_orig_max", 4096)),
                     float(getattr(dims, "yarn_beta_fast", 32.0)),
                     float(getattr(dims, "yarn_beta_slow", 1.0)),
                     float(getattr(dims, "yarn_mscale", 0.0)),
                     MLA_ABSORB_MATERIALIZED if absorb == "materialized" else MLA_ABSORB_FACTORED)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_I32P)


def _i64(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(_I64P)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream_ptr():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Workspace:
    """Grow-only device scratch buffer (256-byte aligned view of a torch tensor)."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        import torch
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        addr = self.buf.data_ptr()
        pad = (-addr) % 256
        return ctypes.c_void_p(addr + pad), self.buf.numel() - pad


class MLALayer:
    """One MLA layer bound to a library handle on the current device/stream."""

    def __init__(self, dims, dtype: str = "bf16", softmax_scale: float = 0.0, device="cuda",
                 kv: str = "dtype", absorb: str = "factored"):
        import torch
        self.lib = load()
        self.dims = dims
        self.dtype = dtype
        self.kv = kv
        self.absorb = absorb
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.cfg = make_config(dims, dtype, softmax_scale, kv, absorb)
        self.device = torch.device(device)
        h = ctypes.c_void_p()
        self._check(self.lib.mla_create(ctypes.byref(self.cfg), _stream_ptr(), ctypes.byref(h)),
                    None, "mla_create")
        self.h = h
        self.ws = Workspace(self.device)

    # -- helpers
    def _check(self, rc, h, what):
        if rc != MLA_OK:
            detail = self.lib.mla_last_error(h).decode() if h else ""
            raise MLAError(rc, f"{what}: {self.lib.mla_status_string(rc).decode()} {detail}")

    def _sync_stream(self):
        self.lib.mla_set_stream(self.h, _stream_ptr())

    def close(self):
        if getattr(self, "h", None):
            self.lib.mla_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def core_timing(self, n_slots: int):
        """Time the next attention-core launches in a ring of n_slots (0 = off)."""
        self._check(self.lib.mla_core_timing(self.h, int(n_slots)), self.h, "core timing")

    def core_timing_read(self, n: int) -> np.ndarray:
        """Durations (ms) of the last n timed core launches, oldest first."""
        ms = np.zeros(max(int(n), 1), np.float32)
        got = ctypes.c_int32()
        self._check(self.lib.mla_core_timing_read(
            self.h, ms.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(n),
            ctypes.byref(got)), self.h, "core timing read")
        return ms[:got.value].copy()

    # -- A1
    def absorb_weights(self, w: dict):
        """w: dict of device tensors in the layer dtype (keys as synth.make_weights)."""
        self._sync_stream()
        rc = self.lib.mla_absorb_weights(
            self.h, _ptr(w.get("w_q")), _ptr(w.get("w_qa")), _ptr(w.get("q_norm_g")),
            _ptr(w.get("w_qb")), _ptr(w["w_kva"]), _ptr(w.get("kv_norm_g")), _ptr(w["w_kvb"]),
            _ptr(w["w_o"]))
        self._check(rc, self.h, "mla_absorb_weights")

    # -- A2
    def append(self, hidden, pos, slot, cache, check_only=False):
        self._sync_stream()
        T = int(hidden.shape[0])
        pos_a, pos_p = _i32(pos)
        slot_a, slot_p = _i64(slot)
        wsp, wsn = self.ws.get(self.lib.mla_append_workspace_bytes(self.h, T))
        rc = self.lib.mla_append_latent(self.h, _ptr(hidden), pos_p, slot_p, T, _ptr(cache),
                                        int(cache.shape[0]), wsp, wsn)
        self._check(rc, self.h, "mla_append_latent")

    def cache_write(self, rows, slot, cache):
        self._sync_stream()
        T = int(rows.shape[0])
        slot_a, slot_p = _i64(slot)
        wsp, wsn = self.ws.get(self.lib.mla_cache_write_workspace_bytes(self.h, T))
        rc = self.lib.mla_cache_write(self.h, _ptr(rows), slot_p, T, _ptr(cache),
                                      int(cache.shape[0]), wsp, wsn)
        self._check(rc, self.h, "mla_cache_write")

    def cache_store(self, rows, slot, cache):
        """rows (T, R) in the layer dtype, stored in the cache's own format."""
        self._sync_stream()
        T = int(rows.shape[0])
        slot_a, slot_p = _i64(slot)
        wsp, wsn = self.ws.get(self.lib.mla_cache_write_workspace_bytes(self.h, T))
        rc = self.lib.mla_cache_store(self.h, _ptr(rows), slot_p, T, _ptr(cache),
                                      int(cache.shape[0]), wsp, wsn)
        self._check(rc, self.h, "mla_cache_store")

    def row_bytes(self) -> int:
        return int(self.lib.mla_cache_row_bytes(ctypes.byref(self.cfg)))

    def new_cache(self, rows: int, fill=None):
        """An empty latent cache of `rows` rows on the layer's device: (rows, R)
        of the layer dtype, or (rows, row_bytes) uint8 for FP8 rows."""
        import torch
        if self.kv == "fp8":
            return torch.zeros((rows, self.row_bytes()), dtype=torch.uint8, device=self.device)
        return torch.zeros((rows, self.dims.row), dtype=self.torch_dtype, device=self.device)

    # -- A3..A8
    def decode(self, hidden, pos, seq_off, seq_len, cache, out=None, stages=False):
        import torch
        self._sync_stream()
        B = int(hidden.shape[0])
        pos_a, pos_p = _i32(pos)
        so_a, so_p = _i64(seq_off)
        sl_a, sl_p = _i32(seq_len)
        total = int(sl_a.astype(np.int64).sum())
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_decode_workspace_bytes(self.h, B, max(total, 1)))
        rc = self.lib.mla_decode(self.h, _ptr(hidden), pos_p, so_p, sl_p, B, _ptr(cache),
                                 int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_decode")
        if not stages:
            return out
        return (out,) + self._stages(B, total, wsp)

    def _stages(self, B, total, wsp):
        qo, oo = ctypes.c_size_t(), ctypes.c_size_t()
        self._check(self.lib.mla_decode_stage_offsets(self.h, B, total, ctypes.byref(qo),
                                                      ctypes.byref(oo)), self.h, "stages")
        d = self.dims
        es = 2 if self.dtype == "bf16" else 4
        base = wsp.value - self.ws.buf.data_ptr()
        raw = self.ws.buf
        q_cat = raw[base + qo.value: base + qo.value + B * d.n_heads * d.row * es]
        o_lat = raw[base + oo.value: base + oo.value + B * d.n_heads * d.kv_lora * es]
        q_cat = q_cat.view(self.torch_dtype).reshape(B, d.n_heads, d.row).clone()
        o_lat = o_lat.view(self.torch_dtype).reshape(B, d.n_heads, d.kv_lora).clone()
        return q_cat, o_lat

    # -- A3..A8 over a paged cache
    def decode_paged(self, hidden, pos, block_table, page_rows, seq_len, cache, out=None,
                     stages=False):
        """mla_decode_paged: block_table (B, max_pages) int32 host array; page
        k of the cache is rows [k * page_rows, (k + 1) * page_rows)."""
        import torch
        self._sync_stream()
        B = int(hidden.shape[0])
        pos_a, pos_p = _i32(pos)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_a, bt_p = _i32(bt.reshape(-1))
        sl_a, sl_p = _i32(seq_len)
        total = int(sl_a.astype(np.int64).sum())
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_decode_workspace_bytes(self.h, B, max(total, 1)))
        rc = self.lib.mla_decode_paged(self.h, _ptr(hidden), pos_p, bt_p, int(bt.shape[1]),
                                       int(page_rows), sl_p, B, _ptr(cache),
                                       int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_decode_paged")
        if not stages:
            return out
        return (out,) + self._stages(B, total, wsp)

    def decode_ex(self, hidden, seq_len, cache, q_len=1, seq_off=None, block_table=None,
                  page_rows=0, append=False, out=None):
        """mla_decode_ex: q_len new tokens per sequence (hidden / out rows
        b * q_len + j), over a contiguous (seq_off) or paged (block_table,
        page_rows) cache, appending the new rows first if `append`."""
        import torch
        self._sync_stream()
        args, keep = decode_args(hidden.shape[0] // q_len, q_len, seq_len, seq_off, block_table,
                                 page_rows, cache, append)
        B = args.B
        if out is None:
            out = torch.empty((B * q_len, self.dims.hidden), dtype=self.torch_dtype,
                              device=self.device)
        total = int(keep[0].astype(np.int64).sum())
        wsp, wsn = self.ws.get(self.lib.mla_decode_ex_workspace_bytes(self.h, B, q_len,
                                                                      max(total, 1),
                                                                      int(bool(append))))
        args.hidden, args.out = hidden.data_ptr(), out.data_ptr()
        args.ws, args.ws_bytes = wsp.value, wsn
        rc = self.lib.mla_decode_ex(self.h, ctypes.byref(args))
        self._check(rc, self.h, "mla_decode_ex")
        return out

    def decode_step_paged(self, hidden, block_table, page_rows, seq_len, cache, out=None):
        """mla_decode_step_paged: appends each new token at position
        seq_len[b] - 1 through the block table, then decodes."""
        import torch
        self._sync_stream()
        B = int(hidden.shape[0])
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_a, bt_p = _i32(bt.reshape(-1))
        sl_a, sl_p = _i32(seq_len)
        pos_a, pos_p = _i32(sl_a - 1)
        total = int(sl_a.astype(np.int64).sum())
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_decode_step_workspace_bytes(self.h, B, max(total, 1)))
        rc = self.lib.mla_decode_step_paged(self.h, _ptr(hidden), pos_p, bt_p, int(bt.shape[1]),
                                            int(page_rows), sl_p, B, _ptr(cache),
                                            int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_decode_step_paged")
        return out

    def decode_step(self, hidden, seq_off, seq_len, cache, out=None):
        """Append each sequence's new token (row seq_off[b] + seq_len[b] - 1,
        position seq_len[b] - 1) and decode it, in one call."""
        import torch
        self._sync_stream()
        B = int(hidden.shape[0])
        sl_a, sl_p = _i32(seq_len)
        pos_a, pos_p = _i32(sl_a - 1)
        so_a, so_p = _i64(seq_off)
        total = int(sl_a.astype(np.int64).sum())
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_decode_step_workspace_bytes(self.h, B, max(total, 1)))
        rc = self.lib.mla_decode_step(self.h, _ptr(hidden), pos_p, so_p, sl_p, B, _ptr(cache),
                                      int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_decode_step")
        return out

    def decode_step_noalloc(self, hidden, seq_off, seq_len, cache, out=None):
        """decode_step with the library's static scratch instead of a
        workspace (mla_decode_step_noalloc)."""
        import torch
        self._sync_stream()
        B = int(hidden.shape[0])
        sl_a, sl_p = _i32(seq_len)
        pos_a, pos_p = _i32(sl_a - 1)
        so_a, so_p = _i64(seq_off)
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        rc = self.lib.mla_decode_step_noalloc(self.h, _ptr(hidden), pos_p, so_p, sl_p, B,
                                              _ptr(cache), int(cache.shape[0]), _ptr(out))
        self._check(rc, self.h, "mla_decode_step_noalloc")
        return out

    # -- P1
    def prefill(self, hidden, cu_new, prior_len, seq_off, cache, out=None):
        import torch
        self._sync_stream()
        cu_a, cu_p = _i32(cu_new)
        pr_a, pr_p = _i32(prior_len)
        so_a, so_p = _i64(seq_off)
        B = len(pr_a)
        T = int(cu_a[-1])
        rows = int((pr_a.astype(np.int64) + np.diff(cu_a)).sum())
        if out is None:
            out = torch.empty((T, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_prefill_workspace_bytes(self.h, T, B, max(rows, 1)))
        rc = self.lib.mla_prefill(self.h, _ptr(hidden), cu_p, pr_p, so_p, B, _ptr(cache),
                                  int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_prefill")
        return out

    def prefill_step(self, hidden, cu_new, prior_len, seq_off, cache, out=None):
        """mla_prefill_step: appends the new tokens' latent rows (position
        prior_len[b] + i at cache row seq_off[b] + prior_len[b] + i), then the
        prefill, in one call."""
        import torch
        self._sync_stream()
        cu_a, cu_p = _i32(cu_new)
        pr_a, pr_p = _i32(prior_len)
        so_a, so_p = _i64(seq_off)
        B = len(pr_a)
        T = int(cu_a[-1])
        rows = int((pr_a.astype(np.int64) + np.diff(cu_a)).sum())
        if out is None:
            out = torch.empty((T, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_prefill_step_workspace_bytes(self.h, T, B,
                                                                         max(rows, 1)))
        rc = self.lib.mla_prefill_step(self.h, _ptr(hidden), cu_p, pr_p, so_p, B, _ptr(cache),
                                       int(cache.shape[0]), _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_prefill_step")
        return out

    def prefill_paged(self, hidden, cu_new, prior_len, block_table, page_rows, cache, out=None):
        """mla_prefill_paged: block_table (B, max_pages) int32 host array; page
        k of the cache is rows [k * page_rows, (k + 1) * page_rows)."""
        import torch
        self._sync_stream()
        cu_a, cu_p = _i32(cu_new)
        pr_a, pr_p = _i32(prior_len)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_a, bt_p = _i32(bt.reshape(-1))
        B = len(pr_a)
        T = int(cu_a[-1])
        rows = int((pr_a.astype(np.int64) + np.diff(cu_a)).sum())
        if out is None:
            out = torch.empty((T, self.dims.hidden), dtype=self.torch_dtype, device=self.device)
        wsp, wsn = self.ws.get(self.lib.mla_prefill_paged_workspace_bytes(self.h, T, B,
                                                                          max(rows, 1)))
        rc = self.lib.mla_prefill_paged(self.h, _ptr(hidden), cu_p, pr_p, bt_p, int(bt.shape[1]),
                                        int(page_rows), B, _ptr(cache), int(cache.shape[0]),
                                        _ptr(out), wsp, wsn)
        self._check(rc, self.h, "mla_prefill_paged")
        return out


def decode_plan(seq_len, max_parts: int, q_len: int = 1):
    """The split-S work list for these lengths (host only), q_len new tokens
    per sequence: returns (part_begin, seg_b, seg_r0, seg_r1) as int32 arrays."""
    lib = load()
    sl, slp = _i32(seq_len)
    B = len(sl)
    nseg_max = B + max_parts - 1
    pb = np.zeros(max_parts + 1, np.int32)
    sb, r0, r1 = (np.zeros(nseg_max, np.int32) for _ in range(3))
    npart, nseg = ctypes.c_int32(), ctypes.c_int32()
    st = lib.mla_decode_plan_tokens(B, slp, int(q_len), max_parts, pb.ctypes.data_as(_I32P),
                             sb.ctypes.data_as(_I32P), r0.ctypes.data_as(_I32P),
                             r1.ctypes.data_as(_I32P), ctypes.byref(npart), ctypes.byref(nseg))
    if st != 0:
        raise MLAError(st, lib.mla_status_string(st).decode())
    p, n = npart.value, nseg.value
    return pb[:p + 1].copy(), sb[:n].copy(), r0[:n].copy(), r1[:n].copy()


def decode_args(B, q_len, seq_len, seq_off=None, block_table=None, page_rows=0, cache=None,
                append=False):
    """An MLADecodeArgs for the host metadata (tensors and workspace left for
    the caller); returns (args, arrays that must stay alive)."""
    sl_a, sl_p = _i32(seq_len)
    keep = [sl_a]
    a = MLADecodeArgs()
    a.B, a.q_len, a.seq_len = int(B), int(q_len), sl_p
    if seq_off is not None:
        so_a, a.seq_off = _i64(seq_off)
        keep.append(so_a)
    if block_table is not None:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_a, a.block_table = _i32(bt.reshape(-1))
        a.max_pages, a.page_rows = int(bt.shape[1]), int(page_rows)
        keep.append(bt_a)
    if cache is not None:
        a.cache, a.cache_rows = cache.data_ptr(), int(cache.shape[0])
    a.append = int(bool(append))
    return a, keep


def header_functions(header: str = None) -> list:
    """Names of the functions include/mla.h declares."""
    import re
    header = header or os.path.join(os.path.dirname(_PKG), "include", "mla.h")
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))
