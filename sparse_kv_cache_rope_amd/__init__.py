"""Python binding of libfasa, the FASA decode hot path for MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libfasa.so`` (built in-tree by ``python sparse_kv_cache_rope_amd/build.py``).
PyTorch provides device memory and the current stream.  Importing this module
without the built library raises ImportError; there is no fallback.

The calls mirror ``include/fasa.h`` (same names without the ``fasa_`` prefix)
and take torch tensors on the context's device.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfasa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing; build it with `python sparse_kv_cache_rope_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "fasa_create": (_c_int, [ctypes.POINTER(_vp), _c_int, _c_int, _c_int, _c_int, _c_int,
                             ctypes.c_double, _c_int, _i32p, _c_int, _c_int]),
    "fasa_create_partial_rope": (_c_int, [ctypes.POINTER(_vp), _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, ctypes.c_double, _c_int, _i32p, _c_int,
                                          _c_int]),
    "fasa_destroy": (None, [_vp]),
    "fasa_kv_cache_bytes": (_c_size, [_vp]),
    "fasa_sidecar_bytes": (_c_size, [_vp]),
    "fasa_workspace_bytes": (_c_size, [_vp]),
    "fasa_sidecar_layout": (_c_int, [_vp, _i32p, _i32p]),
    "fasa_workspace_init": (_c_int, [_vp, _vp, _vp]),
    "fasa_append_kv": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp]),
    "fasa_tip_scores": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]),
    "fasa_topk": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp]),
    "fasa_topk_per_head": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _vp, _vp]),
    "fasa_sparse_attn": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]),
    "fasa_decode_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                  _vp, _vp, _vp, ctypes.c_uint, _vp]),
    "fasa_decode_step_per_head": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp,
                                           _c_int, _vp, _vp, _vp, ctypes.c_uint, _vp]),
    "fasa_decode_step_static": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                         _vp, _vp, _vp, ctypes.c_uint, _vp]),
    "fasa_dense_attn": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]),
    "fasa_calibrate_workspace_bytes": (_c_size, [_vp, _c_int]),
    "fasa_calibrate": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp]),
    "fasa_select_dominant": (_c_int, [ctypes.POINTER(ctypes.c_float), _c_int, _c_int, _c_int,
                                      _c_int, _i32p]),
    "fasa_pointer_kind": (_c_int, [_vp]),
    "fasa_read_probe": (_c_int, [_vp, _c_size, _vp, _vp]),
    "fasa_select_layout": (_c_int, [_c_int, _c_int, ctypes.POINTER(_c_int),
                                    ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "fasa_decode_layout": (_c_int, [_c_int, _c_int, ctypes.POINTER(_c_int),
                                    ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "fasa_check": (_c_int, [_vp, _vp, _vp, ctypes.POINTER(ctypes.c_uint32)]),
    "fasa_timing_enable": (_c_int, [_vp, _c_int]),
    "fasa_timing_collect": (_c_int, [_vp, ctypes.POINTER(ctypes.c_double), _i32p]),
    "fasa_status_string": (ctypes.c_char_p, [_c_int]),
    "fasa_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    try:
        _fn = getattr(_lib, _name)
    except AttributeError as _e:
        raise ImportError(f"{LIB_PATH} lacks {_name}: stale build, rebuild it") from _e
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)

F32, BF16 = 0, 1
ADVANCE_SEQ_LENS = 1
STATIC_SCRATCH_BYTES = 64 << 20  # FASA_STATIC_SCRATCH_BYTES
DEVFLAG_SEQ_LEN, DEVFLAG_INDEX, DEVFLAG_APPEND, DEVFLAG_BUDGET, DEVFLAG_SELECT = 1, 2, 4, 8, 16
_DTYPES = {"f32": (F32, torch.float32), "bf16": (BF16, torch.bfloat16)}


class FasaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.fasa_status_string(status).decode()
        detail = _lib.fasa_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def _chk(status, where):
    if status != 0:
        raise FasaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Context:
    """One attention layer's FASA context (``fasa_create``; with rotary_dim,
    partial RoPE over the first rotary_dim dims, ``fasa_create_partial_rope``)."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, capacity, rope_theta,
                 dtype, dom_fc, max_budget, device=None, rotary_dim=None):
        if dtype not in _DTYPES:
            raise ValueError(f"dtype must be one of {list(_DTYPES)}")
        self.dtype_name = dtype
        self.dtype_code, self.torch_dtype = _DTYPES[dtype]
        self.batch, self.n_q_heads, self.n_kv_heads = batch, n_q_heads, n_kv_heads
        self.head_dim, self.capacity, self.max_budget = head_dim, capacity, max_budget
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        dom = np.ascontiguousarray(np.asarray(dom_fc, dtype=np.int32))
        if dom.ndim != 2 or dom.shape[0] != n_q_heads:
            raise ValueError("dom_fc must be [n_q_heads, n_dom]")
        self.dom_fc = dom
        self.rotary_dim = head_dim if rotary_dim is None else int(rotary_dim)
        handle = _vp()
        with torch.cuda.device(self.device):
            if rotary_dim is None:
                _chk(_lib.fasa_create(ctypes.byref(handle), batch, n_q_heads, n_kv_heads,
                                      head_dim, capacity, float(rope_theta), self.dtype_code,
                                      dom.ctypes.data_as(_i32p), dom.shape[1], max_budget),
                     "fasa_create")
            else:
                _chk(_lib.fasa_create_partial_rope(
                    ctypes.byref(handle), batch, n_q_heads, n_kv_heads, head_dim,
                    self.rotary_dim, capacity, float(rope_theta), self.dtype_code,
                    dom.ctypes.data_as(_i32p), dom.shape[1], max_budget),
                    "fasa_create_partial_rope")
        self._h = handle

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            _lib.fasa_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- sizes and layout -------------------------------------------------
    @property
    def kv_cache_bytes(self):
        return _lib.fasa_kv_cache_bytes(self._h)

    @property
    def sidecar_bytes(self):
        return _lib.fasa_sidecar_bytes(self._h)

    @property
    def workspace_bytes(self):
        return _lib.fasa_workspace_bytes(self._h)

    def sidecar_layout(self):
        """(plane_offset [Hkv+1], plane_fc [P]) as NumPy int32 arrays."""
        P = _lib.fasa_sidecar_layout(self._h, None, None)
        off = np.zeros(self.n_kv_heads + 1, dtype=np.int32)
        fc = np.zeros(max(P, 1), dtype=np.int32)
        _lib.fasa_sidecar_layout(self._h, off.ctypes.data_as(_i32p), fc.ctypes.data_as(_i32p))
        return off, fc[:P]

    # -- allocation helpers (plain torch memory) ----------------------------
    def new_cache(self, kv_on_host=False):
        """Zeroed K cache, V cache and sidecar tensors.  With kv_on_host the K
        and V caches are pinned host memory the GPU reads and writes in place
        (FASA-M); the sidecar, which TIP streams, stays on the device."""
        shape = (self.batch, self.n_kv_heads, self.capacity, self.head_dim)
        if kv_on_host:
            k = torch.zeros(shape, dtype=self.torch_dtype, pin_memory=True)
            v = torch.zeros(shape, dtype=self.torch_dtype, pin_memory=True)
            for name, t in (("K", k), ("V", v)):
                kind = pointer_kind(t)
                if kind != PTR_HOST_MAPPED:
                    raise RuntimeError(f"pinned {name} cache is not reachable from the device "
                                       f"at its host address (kind {kind})")
        else:
            k = torch.zeros(shape, dtype=self.torch_dtype, device=self.device)
            v = torch.zeros(shape, dtype=self.torch_dtype, device=self.device)
        P = _lib.fasa_sidecar_layout(self._h, None, None)
        side = torch.zeros((self.batch, P, self.capacity, 2), dtype=self.torch_dtype,
                           device=self.device)
        assert side.numel() * side.element_size() == self.sidecar_bytes
        return k, v, side

    def new_workspace(self):
        return torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=self.device)

    # -- calls ----------------------------------------------------------------
    def _stream(self, stream):
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        return _vp(s.cuda_stream)

    def _cache(self, t, name):
        """A K or V cache: on the context's device, or pinned host memory the
        device maps at the same address (FASA-M); anything else would fault."""
        shape = (self.batch, self.n_kv_heads, self.capacity, self.head_dim)
        if t.dtype != self.torch_dtype or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a contiguous {self.torch_dtype} tensor of shape "
                             f"{shape} (got {t.dtype}, {tuple(t.shape)})")
        if t.device == self.device:
            return _ptr(t)
        if t.device.type == "cpu" and pointer_kind(t) == PTR_HOST_MAPPED:
            return _ptr(t)
        raise ValueError(f"{name} must be on {self.device} or pinned host memory mapped "
                         f"into it (got {t.device})")

    def _want(self, t, name, dtype, shape=None):
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, context on {self.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def workspace_init(self, workspace, stream=None):
        _chk(_lib.fasa_workspace_init(self._h, _ptr(workspace), self._stream(stream)),
             "fasa_workspace_init")

    def append_kv(self, k_cache, v_cache, sidecar, k_new, v_new, start_pos, workspace,
                  stream=None):
        b, hkv, d = self.batch, self.n_kv_heads, self.head_dim
        n_new = k_new.shape[2]
        self._want(k_new, "k_new", self.torch_dtype, (b, hkv, n_new, d))
        self._want(v_new, "v_new", self.torch_dtype, (b, hkv, n_new, d))
        self._want(start_pos, "start_pos", torch.int32, (b,))
        _chk(_lib.fasa_append_kv(self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'), _ptr(sidecar),
                                 _ptr(k_new), _ptr(v_new), _ptr(start_pos), n_new,
                                 _ptr(workspace), self._stream(stream)), "fasa_append_kv")

    def tip_scores(self, sidecar, q, seq_lens, max_seq_len, scores, workspace, stream=None):
        self._want(q, "q", self.torch_dtype, (self.batch, self.n_q_heads, self.head_dim))
        self._want(scores, "scores", torch.float32,
                   (self.batch, self.n_q_heads, self.capacity))
        self._want(seq_lens, "seq_lens", torch.int32, (self.batch,))
        _chk(_lib.fasa_tip_scores(self._h, _ptr(sidecar), _ptr(q), _ptr(seq_lens),
                                  int(max_seq_len), _ptr(scores), _ptr(workspace),
                                  self._stream(stream)), "fasa_tip_scores")

    def topk(self, scores, seq_lens, max_seq_len, budget, idx, workspace, stream=None,
             head_budgets=None):
        """Top-B per (b, h).  head_budgets (device int32 [Hq], each in
        [0, budget]) gives each query head its own B; idx rows stay budget wide."""
        self._want(scores, "scores", torch.float32,
                   (self.batch, self.n_q_heads, self.capacity))
        self._want(idx, "idx", torch.int32, (self.batch, self.n_q_heads, budget))
        self._want(seq_lens, "seq_lens", torch.int32, (self.batch,))
        if head_budgets is None:
            _chk(_lib.fasa_topk(self._h, _ptr(scores), _ptr(seq_lens), int(max_seq_len),
                                int(budget), _ptr(idx), _ptr(workspace), self._stream(stream)),
                 "fasa_topk")
            return
        self._want(head_budgets, "head_budgets", torch.int32, (self.n_q_heads,))
        _chk(_lib.fasa_topk_per_head(self._h, _ptr(scores), _ptr(seq_lens), int(max_seq_len),
                                     _ptr(head_budgets), int(budget), _ptr(idx),
                                     _ptr(workspace), self._stream(stream)),
             "fasa_topk_per_head")

    def sparse_attn(self, k_cache, v_cache, q, seq_lens, idx, budget, out, workspace,
                    stream=None):
        self._want(q, "q", self.torch_dtype, (self.batch, self.n_q_heads, self.head_dim))
        self._want(idx, "idx", torch.int32, (self.batch, self.n_q_heads, budget))
        self._want(out, "out", torch.float32, (self.batch, self.n_q_heads, self.head_dim))
        self._want(seq_lens, "seq_lens", torch.int32, (self.batch,))
        _chk(_lib.fasa_sparse_attn(self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'), _ptr(q),
                                   _ptr(seq_lens), _ptr(idx), int(budget), _ptr(out),
                                   _ptr(workspace), self._stream(stream)), "fasa_sparse_attn")

    def decode_step(self, k_cache, v_cache, sidecar, q, k_new, v_new, seq_lens, max_seq_len,
                    budget, out, workspace, idx_out=None, advance=False, stream=None,
                    head_budgets=None):
        """One decode step.  head_budgets (device int32 [Hq], each in
        [0, budget]) gives each query head its own B."""
        b, hq, hkv, d = self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim
        self._want(q, "q", self.torch_dtype, (b, hq, d))
        self._want(k_new, "k_new", self.torch_dtype, (b, hkv, d))
        self._want(v_new, "v_new", self.torch_dtype, (b, hkv, d))
        self._want(seq_lens, "seq_lens", torch.int32, (b,))
        self._want(out, "out", torch.float32, (b, hq, d))
        if idx_out is not None:
            self._want(idx_out, "idx_out", torch.int32, (b, hq, budget))
        if head_budgets is not None:
            self._want(head_budgets, "head_budgets", torch.int32, (hq,))
            _chk(_lib.fasa_decode_step_per_head(
                self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'),
                _ptr(sidecar), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                int(max_seq_len), _ptr(head_budgets), int(budget), _ptr(out), _ptr(idx_out),
                _ptr(workspace), ADVANCE_SEQ_LENS if advance else 0, self._stream(stream)),
                "fasa_decode_step_per_head")
            return
        _chk(_lib.fasa_decode_step(self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'), _ptr(sidecar),
                                   _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                   int(max_seq_len), int(budget), _ptr(out), _ptr(idx_out),
                                   _ptr(workspace), ADVANCE_SEQ_LENS if advance else 0,
                                   self._stream(stream)), "fasa_decode_step")

    def decode_step_static(self, k_cache, v_cache, sidecar, q, k_new, v_new, seq_lens,
                           max_seq_len, budget, out, idx_out=None, dev_flags=None,
                           advance=False, stream=None):
        """fasa_decode_step_static: one decode step whose workspace is the
        library's own per-GPU array (no workspace argument, nothing
        allocated).  dev_flags: optional device uint32 [1] that receives the
        step's device flag bits."""
        b, hq, hkv, d = self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim
        self._want(q, "q", self.torch_dtype, (b, hq, d))
        self._want(k_new, "k_new", self.torch_dtype, (b, hkv, d))
        self._want(v_new, "v_new", self.torch_dtype, (b, hkv, d))
        self._want(seq_lens, "seq_lens", torch.int32, (b,))
        self._want(out, "out", torch.float32, (b, hq, d))
        if idx_out is not None:
            self._want(idx_out, "idx_out", torch.int32, (b, hq, budget))
        if dev_flags is not None:
            self._want(dev_flags, "dev_flags", torch.int32, (1,))
        _chk(_lib.fasa_decode_step_static(
            self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'),
            _ptr(sidecar), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(seq_lens), int(max_seq_len),
            int(budget), _ptr(out), _ptr(idx_out), _ptr(dev_flags),
            ADVANCE_SEQ_LENS if advance else 0, self._stream(stream)), "fasa_decode_step_static")

    def dense_attn(self, k_cache, v_cache, q, seq_lens, max_seq_len, out, workspace,
                   stream=None):
        self._want(q, "q", self.torch_dtype, (self.batch, self.n_q_heads, self.head_dim))
        self._want(out, "out", torch.float32, (self.batch, self.n_q_heads, self.head_dim))
        self._want(seq_lens, "seq_lens", torch.int32, (self.batch,))
        _chk(_lib.fasa_dense_attn(self._h, self._cache(k_cache, 'k_cache'), self._cache(v_cache, 'v_cache'), _ptr(q),
                                  _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(workspace),
                                  self._stream(stream)), "fasa_dense_attn")

    def calibrate_workspace_bytes(self, topk):
        return int(_lib.fasa_calibrate_workspace_bytes(self._h, int(topk)))

    def new_calibration_workspace(self, topk):
        return torch.zeros(self.calibrate_workspace_bytes(topk), dtype=torch.uint8,
                           device=self.device)

    def calibrate(self, k_cache, q, seq_lens, max_seq_len, topk, ca, workspace, stream=None):
        """Contextual agreement ca[b][h][c] of every FC with the full head (see
        fasa_calibrate in include/fasa.h); each sequence is one sample."""
        self._want(q, "q", self.torch_dtype, (self.batch, self.n_q_heads, self.head_dim))
        self._want(ca, "ca", torch.float32, (self.batch, self.n_q_heads, self.head_dim // 2))
        self._want(seq_lens, "seq_lens", torch.int32, (self.batch,))
        _chk(_lib.fasa_calibrate(self._h, self._cache(k_cache, 'k_cache'), _ptr(q), _ptr(seq_lens),
                                 int(max_seq_len), int(topk), _ptr(ca), _ptr(workspace),
                                 self._stream(stream)), "fasa_calibrate")

    KERNEL_FAMILIES = ("append", "prologue", "tip", "topk", "fac", "dense", "select_fac",
                       "calibrate")

    def timing_enable(self, enable=True):
        _chk(_lib.fasa_timing_enable(self._h, 1 if enable else 0), "fasa_timing_enable")

    def timing_collect(self):
        """{family: (total_ms, launches)} since the last collect (waits)."""
        n = len(self.KERNEL_FAMILIES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int32 * n)()
        _chk(_lib.fasa_timing_collect(self._h, ms, cnt), "fasa_timing_collect")
        return {f: (ms[i], cnt[i]) for i, f in enumerate(self.KERNEL_FAMILIES)}

    def check(self, workspace, stream=None):
        """Synchronise; return the device error-flag bits (and clear them)."""
        flags = ctypes.c_uint32(0)
        st = _lib.fasa_check(self._h, _ptr(workspace), self._stream(stream), ctypes.byref(flags))
        if st not in (0, -5):
            raise FasaError(st, "fasa_check")
        return int(flags.value)


PTR_UNUSABLE, PTR_DEVICE, PTR_HOST_MAPPED = 0, 1, 2


def pointer_kind(t):
    """fasa_pointer_kind of a tensor's storage."""
    return int(_lib.fasa_pointer_kind(_vp(t.data_ptr())))


def read_probe(buf, sink, stream=None):
    """fasa_read_probe: one streaming read pass over a device tensor's bytes
    (a measurement aid); `sink` is a device float tensor of at least one
    element."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    _chk(_lib.fasa_read_probe(_vp(buf.data_ptr()), buf.numel() * buf.element_size(),
                              _vp(sink.data_ptr()), _vp(st.cuda_stream)), "fasa_read_probe")


SELECT_LAYOUTS = {0: "none", 1: "whole", 2: "chunked", 3: "whole_wide", 4: "per_row",
                  5: "group_filter"}


def select_layout(max_seq_len, budget):
    """fasa_select_layout (host only): the top-B layout for rows of up to
    max_seq_len positions at `budget`, as (name, threads, per_thread, chunk)."""
    t, e, ch = _c_int(0), _c_int(0), _c_int(0)
    k = _lib.fasa_select_layout(int(max_seq_len), int(budget), ctypes.byref(t), ctypes.byref(e),
                                ctypes.byref(ch))
    return SELECT_LAYOUTS[k], t.value, e.value, ch.value


def decode_layout(max_seq_len, budget):
    """fasa_decode_layout (host only): the top-B layout of a decode step, as
    (name, threads, per_thread, chunk); "group_filter" where the step selects
    through TIP's group maxima."""
    t, e, ch = _c_int(0), _c_int(0), _c_int(0)
    k = _lib.fasa_decode_layout(int(max_seq_len), int(budget), ctypes.byref(t), ctypes.byref(e),
                                ctypes.byref(ch))
    return SELECT_LAYOUTS[k], t.value, e.value, ch.value


def select_dominant(ca, n_dom):
    """I_dom from agreement values (host, fasa_select_dominant): ca is a host
    array [samples, heads, C] (or [heads, C]); returns int32 [heads, n_dom]."""
    a = np.ascontiguousarray(np.asarray(ca, dtype=np.float32))
    if a.ndim == 2:
        a = a[None]
    samples, heads, n_fc = a.shape
    out = np.empty((heads, int(n_dom)), dtype=np.int32)
    _chk(_lib.fasa_select_dominant(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), samples,
                                   heads, n_fc, int(n_dom), out.ctypes.data_as(_i32p)),
         "fasa_select_dominant")
    return out


def status_string(status):
    return _lib.fasa_status_string(status).decode()


def raw_create(batch, n_q_heads, n_kv_heads, head_dim, capacity, rope_theta, dtype_code,
               dom_fc, n_dom, max_budget, rotary_dim=None):
    """fasa_create (fasa_create_partial_rope with rotary_dim) with raw
    arguments: (status, message)."""
    dom = np.ascontiguousarray(np.asarray(dom_fc, dtype=np.int32)) if dom_fc is not None else None
    dp = dom.ctypes.data_as(_i32p) if dom is not None else None
    handle = _vp()
    if rotary_dim is None:
        st = _lib.fasa_create(ctypes.byref(handle), batch, n_q_heads, n_kv_heads, head_dim,
                              capacity, float(rope_theta), dtype_code, dp, n_dom, max_budget)
    else:
        st = _lib.fasa_create_partial_rope(ctypes.byref(handle), batch, n_q_heads, n_kv_heads,
                                           head_dim, rotary_dim, capacity, float(rope_theta),
                                           dtype_code, dp, n_dom, max_budget)
    msg = _lib.fasa_last_error().decode()
    if st == 0:
        _lib.fasa_destroy(handle)
    return st, msg
