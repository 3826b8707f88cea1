"""Python binding of libnatsl (the NAtS-L hybrid attention layer for MI355X).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libnatsl.so.  PyTorch supplies device memory and the current stream.  The
names mirror the C ABI in include/natsl.h: route, gdn_chunk, softmax_masked,
merge, forward, decode_step, workspace_size, plus profile_* for measurement.

If the library is missing every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnatsl.so")

F32, BF16 = 0, 1
ROUTE_SOFTMAX, ROUTE_LINEAR = 0, 1
ENTRY_ROUTE, ENTRY_GDN_CHUNK, ENTRY_SOFTMAX_MASKED, ENTRY_MERGE, ENTRY_FORWARD, ENTRY_DECODE_STEP, \
    ENTRY_DECODE_HANDOFF, ENTRY_SOFTMAX_BACKWARD, ENTRY_GDN_BACKWARD, ENTRY_MERGE_BACKWARD, \
    ENTRY_ROUTE_BACKWARD, ENTRY_GDN_BACKWARD_OVERLAP = range(12)
STATUS = {0: "NATSL_OK", 1: "NATSL_ERR_INVALID_ARG", 2: "NATSL_ERR_UNSUPPORTED",
          3: "NATSL_ERR_WORKSPACE", 4: "NATSL_ERR_DEVICE", 5: "NATSL_ERR_CAPACITY"}
EXPORTS = ["natsl_version", "natsl_last_error", "natsl_workspace_size", "natsl_route", "natsl_gdn_chunk",
           "natsl_softmax_masked", "natsl_merge", "natsl_forward", "natsl_decode_step",
           "natsl_decode_handoff", "natsl_softmax_masked_backward", "natsl_gdn_backward", "natsl_merge_backward",
           "natsl_decode_step_noalloc", "natsl_route_backward", "natsl_nha_workspace_size", "natsl_nha_attention", "natsl_profile_enable", "natsl_profile_reset", "natsl_profile_read",
           "natsl_profile_select", "natsl_set_sync_check", "natsl_get_sync_check"]
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


class NatslError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("L", C.c_int32), ("Dk", C.c_int32), ("Dv", C.c_int32),
                ("d_model", C.c_int32), ("chunk", C.c_int32), ("route_groups", C.c_int32), ("io", C.c_int),
                ("sm_scale", C.c_float), ("rms_eps", C.c_float)]


class ForwardArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("alpha", C.c_void_p), ("beta", C.c_void_p), ("w_score", C.c_void_p), ("b_score", C.c_void_p),
                ("w_mix", C.c_void_p), ("w_mix_head_stride", C.c_int64), ("g_sm", C.c_void_p),
                ("g_lin", C.c_void_p), ("route_override", C.c_void_p), ("S_init", C.c_void_p),
                ("branch_dtype", C.c_int), ("route_out", C.c_void_p), ("scores_out", C.c_void_p),
                ("o_sm_dbg", C.c_void_p), ("o_gdn_dbg", C.c_void_p), ("S_final", C.c_void_p),
                ("out", C.c_void_p), ("prefix", C.c_void_p)]


class DecodeCache(C.Structure):
    _fields_ = [("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("cap", C.c_int32),
                ("n_committed", C.c_void_p), ("n_open", C.c_void_p), ("S_carry", C.c_void_p),
                ("S_work", C.c_void_p), ("x_sum", C.c_void_p), ("err_flag", C.c_void_p)]


class DecodeArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("alpha", C.c_void_p), ("beta", C.c_void_p), ("w_score", C.c_void_p), ("b_score", C.c_void_p),
                ("w_mix", C.c_void_p), ("w_mix_head_stride", C.c_int64), ("g_sm", C.c_void_p),
                ("g_lin", C.c_void_p), ("out", C.c_void_p), ("route_out", C.c_void_p),
                ("o_sm_dbg", C.c_void_p), ("o_gdn_dbg", C.c_void_p)]


_lib = None


def lib():
    """Load libnatsl.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_natsl_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        vp, i32, st = C.c_void_p, C.c_int32, C.c_int
        L.natsl_version.restype = C.c_int
        L.natsl_last_error.restype = C.c_char_p
        L.natsl_workspace_size.argtypes = [C.c_int, C.POINTER(Dims), C.POINTER(C.c_size_t)]
        L.natsl_route.argtypes = [C.POINTER(Dims)] + [vp] * 8 + [vp]
        L.natsl_gdn_chunk.argtypes = [C.POINTER(Dims)] + [vp] * 8 + [C.c_int, vp, vp, C.c_size_t, vp]
        L.natsl_softmax_masked.argtypes = [C.POINTER(Dims)] + [vp] * 6 + [C.c_int, vp, vp, C.c_size_t, vp]
        L.natsl_merge.argtypes = [C.POINTER(Dims), vp, vp, vp, C.c_int, vp, C.c_int64, vp, vp, vp, vp]
        L.natsl_forward.argtypes = [C.POINTER(Dims), C.POINTER(ForwardArgs), vp, C.c_size_t, vp]
        L.natsl_decode_step.argtypes = [C.POINTER(Dims), C.POINTER(DecodeCache), C.POINTER(DecodeArgs), vp,
                                        C.c_size_t, vp]
        L.natsl_decode_step_noalloc.argtypes = [C.POINTER(Dims), C.POINTER(DecodeCache), C.POINTER(DecodeArgs), vp]
        L.natsl_nha_workspace_size.argtypes = [C.POINTER(Dims), C.c_int, C.c_int, C.POINTER(C.c_size_t)]
        L.natsl_nha_attention.argtypes = [C.POINTER(Dims), vp, vp, vp, vp, C.c_int, C.c_int, vp, vp, C.c_size_t, vp]
        L.natsl_decode_handoff.argtypes = [C.POINTER(Dims), vp, vp, vp, vp, C.c_int, C.POINTER(DecodeCache), vp,
                                           C.c_size_t, vp]
        L.natsl_softmax_masked_backward.argtypes = [C.POINTER(Dims)] + [vp] * 13 + [C.c_size_t, vp]
        L.natsl_gdn_backward.argtypes = [C.POINTER(Dims)] + [vp] * 17 + [C.c_size_t, vp]
        L.natsl_route_backward.argtypes = [C.POINTER(Dims)] + [vp] * 9 + [C.c_size_t, vp]
        L.natsl_merge_backward.argtypes = [C.POINTER(Dims), vp, vp, vp, C.c_int, vp, C.c_int64] + [vp] * 10 + \
            [C.c_size_t, vp]
        L.natsl_profile_enable.argtypes = [C.c_int]
        L.natsl_profile_read.argtypes = [C.c_char_p, C.POINTER(C.c_int), C.POINTER(C.c_double)]
        L.natsl_profile_select.argtypes = [C.c_char_p]
        L.natsl_set_sync_check.argtypes = [C.c_int]
        L.natsl_get_sync_check.argtypes = []
        L.natsl_get_sync_check.restype = C.c_int
        for name in ("natsl_workspace_size", "natsl_route", "natsl_gdn_chunk", "natsl_softmax_masked",
                     "natsl_merge", "natsl_forward", "natsl_decode_step", "natsl_decode_step_noalloc",
                     "natsl_nha_workspace_size", "natsl_nha_attention", "natsl_route_backward",
                     "natsl_decode_handoff",
                     "natsl_softmax_masked_backward", "natsl_gdn_backward", "natsl_merge_backward",
                     "natsl_profile_enable",
                     "natsl_profile_reset", "natsl_profile_read", "natsl_profile_select",
                     "natsl_set_sync_check"):
            getattr(L, name).restype = st
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise NatslError(status, lib().natsl_last_error().decode())


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t, dtype=None, name="tensor", shape=None):
    """Device pointer of a contiguous CUDA tensor (None -> NULL), after
    checking dtype and shape on the host: the kernels index these buffers by
    the dims alone, so a wrong shape must never reach them."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _io_t(dm):
    return torch.bfloat16 if dm.io == BF16 else torch.float32


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def dims(B, H, L, D, d_model, io, groups=1, sm_scale=0.0, rms_eps=0.0):
    return Dims(B, H, L, D, D, d_model, 64, groups, io, sm_scale, rms_eps)


def version():
    return lib().natsl_version()


def workspace_size(entry, dm: Dims):
    n = C.c_size_t(0)
    _check(lib().natsl_workspace_size(entry, C.byref(dm), C.byref(n)))
    return n.value


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned workspace (torch allocations are 512-byte aligned)."""
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def route(dm: Dims, x, w_score, b_score=None, route_in=None, scores=True, stream=None):
    B, G, nc = dm.B, dm.route_groups, dm.L // 64
    dev = (x if x is not None else route_in).device
    route_out = torch.empty(B, G, nc, dtype=torch.int32, device=dev)
    sel = torch.empty(B, G, nc, dtype=torch.int32, device=dev)
    nsb = torch.empty(B, G, nc + 1, dtype=torch.int32, device=dev)
    sc = torch.empty(B, G, nc, 2, dtype=torch.float32, device=dev) if scores and route_in is None else None
    G2 = 2 * G
    _check(lib().natsl_route(C.byref(dm), _p(x, _io_t(dm), "x", (B, dm.L, dm.d_model)),
                             _p(w_score, torch.float32, "w_score", (dm.d_model, G2)),
                             _p(b_score, torch.float32, "b_score", (G2,)),
                             _p(route_in, torch.int32, "route_in", (B, G, nc)),
                             _p(route_out), _p(sel), _p(nsb), _p(sc), _stream(stream)))
    return route_out, sel, nsb, sc


def gdn_chunk(dm: Dims, q, k, v, alpha, beta, route_bgc, S_init=None, o_dtype=torch.float32,
              want_state=True, stream=None):
    o = torch.empty(q.shape[:3] + (dm.Dv,), dtype=o_dtype, device=q.device)
    Sf = torch.empty(dm.B, dm.H, dm.Dk, dm.Dv, dtype=torch.float32, device=q.device) if want_state else None
    nb = workspace_size(ENTRY_GDN_CHUNK, dm)
    ws = workspace(nb, q.device)
    io, qs, ts = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk), (dm.B, dm.H, dm.L)
    _check(lib().natsl_gdn_chunk(C.byref(dm), _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs),
                                 _p(alpha, torch.float32, "alpha", ts), _p(beta, torch.float32, "beta", ts),
                                 _p(route_bgc, torch.int32, "route", (dm.B, dm.route_groups, dm.L // 64)),
                                 _p(S_init, torch.float32, "S_init", (dm.B, dm.H, dm.Dk, dm.Dv)),
                                 _p(o), _dt(o), _p(Sf), _p(ws), nb, _stream(stream)))
    return o, Sf


def softmax_masked(dm: Dims, q, k, v, sel_idx, nsel_before, o_dtype=torch.float32, want_lse=False,
                   stream=None):
    o = torch.empty(q.shape[:3] + (dm.Dv,), dtype=o_dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    io, qs, nc = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk), dm.L // 64
    _check(lib().natsl_softmax_masked(C.byref(dm), _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs),
                                      _p(sel_idx, torch.int32, "sel_idx", (dm.B, dm.route_groups, nc)),
                                      _p(nsel_before, torch.int32, "nsel_before", (dm.B, dm.route_groups, nc + 1)),
                                      _p(o), _dt(o), _p(lse),
                                      None, 0, _stream(stream)))
    return o, lse


def merge(dm: Dims, q, o_sm, o_gdn, w_mix, w_mix_head_stride=0, g_sm=None, g_lin=None, stream=None):
    out = torch.empty(q.shape[:3] + (dm.Dv,), dtype=q.dtype, device=q.device)
    if o_sm.dtype != o_gdn.dtype:
        raise TypeError("o_sm and o_gdn must share a dtype")
    qs = (dm.B, dm.H, dm.L, dm.Dk)
    wm_shape = (dm.Dk, 2) if w_mix_head_stride == 0 else (dm.H, dm.Dk, 2)
    if w_mix_head_stride not in (0, 2 * dm.Dk):
        raise ValueError("w_mix_head_stride must be 0 or 2*Dk")
    _check(lib().natsl_merge(C.byref(dm), _p(q, _io_t(dm), "q", qs), _p(o_sm, None, "o_sm", qs),
                             _p(o_gdn, None, "o_gdn", qs),
                             _dt(o_sm), _p(w_mix, torch.float32, "w_mix", wm_shape), w_mix_head_stride,
                             _p(g_sm, torch.float32, "g_sm", (dm.Dv,)), _p(g_lin, torch.float32, "g_lin", (dm.Dv,)),
                             _p(out),
                             _stream(stream)))
    return out


def nha_workspace_size(dm: Dims, slots, window):
    n = C.c_size_t(0)
    _check(lib().natsl_nha_workspace_size(C.byref(dm), slots, window, C.byref(n)))
    return n.value


def nha_attention(dm: Dims, q, k, v, slot_gate, window, ws=None, stream=None):
    """Native Hybrid Attention: one softmax over gated key-value slots and a
    sliding window of `window` tokens (a multiple of 64).  slot_gate is
    [B, H, L, slots] fp32 with slots in {16, 32, 64}.  Returns out in the io
    dtype."""
    io, qs = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk)
    slots = slot_gate.shape[-1] if slot_gate.dim() == 4 else -1
    nbytes = nha_workspace_size(dm, slots, window)
    if ws is None:
        ws = workspace(nbytes, q.device)
    elif ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    out = torch.empty(qs, dtype=io, device=q.device)
    _check(lib().natsl_nha_attention(C.byref(dm), _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs),
                                     _p(slot_gate, torch.float32, "slot_gate", (dm.B, dm.H, dm.L, slots)), slots,
                                     window, _p(out), _p(ws), nbytes, _stream(stream)))
    return out


class Forward:
    """Reusable forward call: owns its workspace and output buffers so that
    repeated calls (benchmarks, graphs) allocate nothing."""

    def __init__(self, dm: Dims, device="cuda", branch_dtype=None, debug=False, want_state=False):
        self.dm = dm
        io_t = torch.bfloat16 if dm.io == BF16 else torch.float32
        # branch intermediates in the io dtype by default (the kernels
        # accumulate in fp32 either way); fp32 storage on request
        self.branch_dtype = branch_dtype if branch_dtype is not None else io_t
        self.ws_bytes = workspace_size(ENTRY_FORWARD, dm)
        self.ws = workspace(self.ws_bytes, device)
        shp = (dm.B, dm.H, dm.L, dm.Dv)
        self.out = torch.empty(shp, dtype=io_t, device=device)
        self.route = torch.empty(dm.B, dm.route_groups, dm.L // 64, dtype=torch.int32, device=device)
        self.scores = torch.empty(dm.B, dm.route_groups, dm.L // 64, 2, dtype=torch.float32, device=device)
        self.o_sm = torch.empty(shp, dtype=self.branch_dtype, device=device) if debug else None
        self.o_gdn = torch.empty(shp, dtype=self.branch_dtype, device=device) if debug else None
        self.S_final = torch.empty(dm.B, dm.H, dm.Dk, dm.Dv, dtype=torch.float32, device=device) \
            if want_state else None

    def __call__(self, x, q, k, v, alpha, beta, w_score, w_mix, b_score=None, g_sm=None, g_lin=None,
                 route_override=None, S_init=None, w_mix_head_stride=0, stream=None, prefix=None):
        """prefix: a DecodeState at a chunk boundary that these L tokens
        continue (chunked prefill): the softmax branch also attends to its
        committed rows and the Gated DeltaNet branch starts from its S_carry."""
        dm = self.dm
        io, qs, ts, nc, G2 = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk), (dm.B, dm.H, dm.L), dm.L // 64, 2 * dm.route_groups
        if w_mix_head_stride not in (0, 2 * dm.Dk):
            raise ValueError("w_mix_head_stride must be 0 or 2*Dk")
        a = ForwardArgs()
        a.x = _p(x, io, "x", (dm.B, dm.L, dm.d_model))
        a.q, a.k, a.v = _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs)
        a.alpha, a.beta = _p(alpha, torch.float32, "alpha", ts), _p(beta, torch.float32, "beta", ts)
        a.w_score = _p(w_score, torch.float32, "w_score", (dm.d_model, G2))
        a.b_score = _p(b_score, torch.float32, "b_score", (G2,))
        a.w_mix = _p(w_mix, torch.float32, "w_mix", (dm.Dk, 2) if w_mix_head_stride == 0 else (dm.H, dm.Dk, 2))
        a.w_mix_head_stride = w_mix_head_stride
        a.g_sm, a.g_lin = _p(g_sm, torch.float32, "g_sm", (dm.Dv,)), _p(g_lin, torch.float32, "g_lin", (dm.Dv,))
        a.route_override = _p(route_override, torch.int32, "route_override", (dm.B, dm.route_groups, nc))
        a.S_init = _p(S_init, torch.float32, "S_init", (dm.B, dm.H, dm.Dk, dm.Dv))
        a.branch_dtype = F32 if self.branch_dtype == torch.float32 else BF16
        a.route_out, a.scores_out = _p(self.route), (_p(self.scores) if route_override is None else None)
        a.o_sm_dbg, a.o_gdn_dbg = _p(self.o_sm), _p(self.o_gdn)
        a.S_final, a.out = _p(self.S_final), _p(self.out)
        pre = None
        if prefix is not None:
            if prefix.k.dtype != io or tuple(prefix.k.shape[:2]) != (dm.B, dm.H) or prefix.k.shape[3] != dm.Dk:
                raise ValueError("prefix cache does not match the dims")
            if tuple(prefix.n_committed.shape) != (dm.B, dm.route_groups):
                raise ValueError("prefix cache counters do not match the dims")
            pre = prefix.struct()
            a.prefix = C.cast(C.pointer(pre), C.c_void_p)
        _check(lib().natsl_forward(C.byref(self.dm), C.byref(a), _p(self.ws), self.ws_bytes, _stream(stream)))
        del pre
        return self.out


def forward(dm: Dims, *args, debug=False, want_state=False, branch_dtype=None, **kw):
    f = Forward(dm, device=args[1].device, branch_dtype=branch_dtype, debug=debug, want_state=want_state)
    f(*args, **kw)
    return f


class DecodeState:
    """Device-resident decode cache (layout of natsl_decode_cache)."""

    def __init__(self, B, H, D, d_model, cap, groups=1, io=torch.bfloat16, device="cuda"):
        self.k = torch.zeros(B, H, cap, D, dtype=io, device=device)
        self.v = torch.zeros(B, H, cap, D, dtype=io, device=device)
        self.cap = cap
        self.n_committed = torch.zeros(B, groups, dtype=torch.int32, device=device)
        self.n_open = torch.zeros(B, dtype=torch.int32, device=device)
        self.S_carry = torch.zeros(B, H, D, D, dtype=torch.float32, device=device)
        self.S_work = torch.zeros(B, H, D, D, dtype=torch.float32, device=device)
        self.x_sum = torch.zeros(B, d_model, dtype=torch.float32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)

    def struct(self):
        return DecodeCache(_p(self.k), _p(self.v), self.cap, _p(self.n_committed), _p(self.n_open),
                           _p(self.S_carry), _p(self.S_work), _p(self.x_sum), _p(self.err))


class Decode:
    """Reusable decode step bound to a DecodeState (allocates only at init).
    noalloc=True calls natsl_decode_step_noalloc: no workspace, the library's
    per-device scratch array instead."""

    def __init__(self, dm: Dims, state: DecodeState, device="cuda", debug=False, noalloc=False):
        self.dm = Dims.from_buffer_copy(dm)
        self.dm.L = state.cap
        exp = (dm.B, dm.H, state.cap, dm.Dk)
        if tuple(state.k.shape) != exp or tuple(state.v.shape) != exp:
            raise ValueError(f"cache k/v must have shape {exp}")
        if tuple(state.n_committed.shape) != (dm.B, dm.route_groups) or tuple(state.n_open.shape) != (dm.B,):
            raise ValueError("cache counters do not match the dims")
        if tuple(state.S_carry.shape) != (dm.B, dm.H, dm.Dk, dm.Dv) or tuple(state.x_sum.shape) != (dm.B, dm.d_model):
            raise ValueError("cache states do not match the dims")
        if state.k.dtype != _io_t(dm):
            raise TypeError("cache dtype must be the io dtype")
        self.state = state
        self.cstruct = state.struct()
        self.noalloc = noalloc
        self.ws_bytes = 0 if noalloc else workspace_size(ENTRY_DECODE_STEP, self.dm)
        self.ws = None if noalloc else workspace(self.ws_bytes, device)
        io_t = torch.bfloat16 if dm.io == BF16 else torch.float32
        self.out = torch.empty(dm.B, dm.H, dm.Dv, dtype=io_t, device=device)
        self.route = torch.empty(dm.B, dm.route_groups, dtype=torch.int32, device=device)
        self.o_sm = torch.empty(dm.B, dm.H, dm.Dv, dtype=torch.float32, device=device) if debug else None
        self.o_gdn = torch.empty(dm.B, dm.H, dm.Dv, dtype=torch.float32, device=device) if debug else None

    def __call__(self, x, q, k, v, alpha, beta, w_score, w_mix, b_score=None, g_sm=None, g_lin=None,
                 w_mix_head_stride=0, stream=None):
        dm = self.dm
        io, hs, G2 = _io_t(dm), (dm.B, dm.H, dm.Dk), 2 * dm.route_groups
        if w_mix_head_stride not in (0, 2 * dm.Dk):
            raise ValueError("w_mix_head_stride must be 0 or 2*Dk")
        a = DecodeArgs()
        a.x = _p(x, io, "x", (dm.B, dm.d_model))
        a.q, a.k, a.v = _p(q, io, "q", hs), _p(k, io, "k", hs), _p(v, io, "v", hs)
        a.alpha = _p(alpha, torch.float32, "alpha", (dm.B, dm.H))
        a.beta = _p(beta, torch.float32, "beta", (dm.B, dm.H))
        a.w_score = _p(w_score, torch.float32, "w_score", (dm.d_model, G2))
        a.b_score = _p(b_score, torch.float32, "b_score", (G2,))
        a.w_mix = _p(w_mix, torch.float32, "w_mix", (dm.Dk, 2) if w_mix_head_stride == 0 else (dm.H, dm.Dk, 2))
        a.w_mix_head_stride = w_mix_head_stride
        a.g_sm, a.g_lin = _p(g_sm, torch.float32, "g_sm", (dm.Dv,)), _p(g_lin, torch.float32, "g_lin", (dm.Dv,))
        a.out, a.route_out = _p(self.out), _p(self.route)
        a.o_sm_dbg, a.o_gdn_dbg = _p(self.o_sm), _p(self.o_gdn)
        if self.noalloc:
            _check(lib().natsl_decode_step_noalloc(C.byref(self.dm), C.byref(self.cstruct), C.byref(a),
                                                   _stream(stream)))
        else:
            _check(lib().natsl_decode_step(C.byref(self.dm), C.byref(self.cstruct), C.byref(a), _p(self.ws),
                                           self.ws_bytes, _stream(stream)))
        return self.out


def decode_step(dm: Dims, state: DecodeState, *args, debug=False, **kw):
    d = Decode(dm, state, device=args[1].device, debug=debug)
    d(*args, **kw)
    return d


def softmax_masked_backward(dm: Dims, q, k, v, sel_idx, nsel_before, o_sm, lse, d_o, stream=None, want_gate=False):
    """Gradient of the softmax branch: returns fp32 (dq, dk, dv), and the
    per-chunk softmax-gate derivative [B, H, Nc] as a fourth value when
    want_gate.  o_sm and lse are the forward's outputs (softmax_masked(...,
    o_dtype=io, want_lse=True)), d_o the upstream gradient, both in the io
    dtype."""
    io, qs, nc = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk), dm.L // 64
    dq = torch.empty(qs, dtype=torch.float32, device=q.device)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    dg = torch.empty(dm.B, dm.H, nc, dtype=torch.float32, device=q.device) if want_gate else None
    ws_bytes = workspace_size(ENTRY_SOFTMAX_BACKWARD, dm)
    ws = workspace(ws_bytes, q.device)
    _check(lib().natsl_softmax_masked_backward(
        C.byref(dm), _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs),
        _p(sel_idx, torch.int32, "sel_idx", (dm.B, dm.route_groups, nc)),
        _p(nsel_before, torch.int32, "nsel_before", (dm.B, dm.route_groups, nc + 1)),
        _p(o_sm, io, "o_sm", qs), _p(lse, torch.float32, "lse", qs[:3]), _p(d_o, io, "d_o", qs),
        _p(dq), _p(dk), _p(dv), _p(dg), _p(ws), ws_bytes, _stream(stream)))
    return (dq, dk, dv, dg) if want_gate else (dq, dk, dv)


def gdn_backward(dm: Dims, q, k, v, alpha, beta, route_bgc, d_o, S_init=None, dS_final=None, want_dS_init=True,
                 stream=None, want_gate=False, overlap=False):
    """Gradient of the Gated DeltaNet branch through the rollback: returns fp32
    (dq, dk, dv, dalpha, dbeta, dS_init).  q, k, v, alpha, beta, route_bgc and
    S_init are the forward's inputs (gdn_chunk), d_o the fp32 upstream gradient
    of o_gdn, dS_final that of the final carried state (None: zero).  overlap:
    pass the larger workspace of ENTRY_GDN_BACKWARD_OVERLAP, with which the
    library runs its two sweeps at the same time (same results)."""
    io, qs, ts = _io_t(dm), (dm.B, dm.H, dm.L, dm.Dk), (dm.B, dm.H, dm.L)
    ss = (dm.B, dm.H, dm.Dk, dm.Dv)
    dq = torch.empty(qs, dtype=torch.float32, device=q.device)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    da = torch.empty(ts, dtype=torch.float32, device=q.device)
    db = torch.empty_like(da)
    dS0 = torch.empty(ss, dtype=torch.float32, device=q.device) if want_dS_init else None
    dg = torch.empty(dm.B, dm.H, dm.L // 64, dtype=torch.float32, device=q.device) if want_gate else None
    ws_bytes = workspace_size(ENTRY_GDN_BACKWARD_OVERLAP if overlap else ENTRY_GDN_BACKWARD, dm)
    ws = workspace(ws_bytes, q.device)
    _check(lib().natsl_gdn_backward(
        C.byref(dm), _p(q, io, "q", qs), _p(k, io, "k", qs), _p(v, io, "v", qs),
        _p(alpha, torch.float32, "alpha", ts), _p(beta, torch.float32, "beta", ts),
        _p(route_bgc, torch.int32, "route", (dm.B, dm.route_groups, dm.L // 64)),
        _p(S_init, torch.float32, "S_init", ss), _p(d_o, torch.float32, "d_o", qs),
        _p(dS_final, torch.float32, "dS_final", ss), _p(dq), _p(dk), _p(dv), _p(da), _p(db), _p(dS0), _p(dg),
        _p(ws), ws_bytes, _stream(stream)))
    return (dq, dk, dv, da, db, dS0, dg) if want_gate else (dq, dk, dv, da, db, dS0)


def route_backward(dm: Dims, x, w_score, scores, dgate_sm, dgate_lin, want_dx=True, want_db=True, stream=None):
    """Router gradient under the straight-through reading (natsl_route_backward):
    returns fp32 (dx or None, dw_score, db_score or None)."""
    io, nc, G = _io_t(dm), dm.L // 64, dm.route_groups
    dx = torch.empty(dm.B, dm.L, dm.d_model, dtype=torch.float32, device=x.device) if want_dx else None
    dw = torch.empty(dm.d_model, 2 * G, dtype=torch.float32, device=x.device)
    db = torch.empty(2 * G, dtype=torch.float32, device=x.device) if want_db else None
    ws_bytes = workspace_size(ENTRY_ROUTE_BACKWARD, dm)
    ws = workspace(ws_bytes, x.device)
    _check(lib().natsl_route_backward(
        C.byref(dm), _p(x, io, "x", (dm.B, dm.L, dm.d_model)), _p(w_score, torch.float32, "w_score", (dm.d_model, 2 * G)),
        _p(scores, torch.float32, "scores", (dm.B, G, nc, 2)),
        _p(dgate_sm, torch.float32, "dgate_sm", (dm.B, dm.H, nc)), _p(dgate_lin, torch.float32, "dgate_lin", (dm.B, dm.H, nc)),
        _p(dx), _p(dw), _p(db), _p(ws), ws_bytes, _stream(stream)))
    return dx, dw, db


def merge_backward(dm: Dims, q, o_sm, o_gdn, w_mix, d_out, w_mix_head_stride=0, g_sm=None, g_lin=None,
                   stream=None):
    """Gradient of the merge: returns fp32 (d_o_sm, d_o_gdn, dq, dw_mix, dg_sm,
    dg_lin); dq is the mixing weights' share of q's gradient.  d_out is the
    fp32 upstream gradient of out."""
    if o_sm.dtype != o_gdn.dtype:
        raise TypeError("o_sm and o_gdn must share a dtype")
    if w_mix_head_stride not in (0, 2 * dm.Dk):
        raise ValueError("w_mix_head_stride must be 0 or 2*Dk")
    qs = (dm.B, dm.H, dm.L, dm.Dk)
    wm_shape = (dm.Dk, 2) if w_mix_head_stride == 0 else (dm.H, dm.Dk, 2)
    d_sm = torch.empty(qs, dtype=torch.float32, device=q.device)
    d_gdn, dq = torch.empty_like(d_sm), torch.empty_like(d_sm)
    dwm = torch.empty(wm_shape, dtype=torch.float32, device=q.device)
    dgs = torch.empty(dm.Dv, dtype=torch.float32, device=q.device)
    dgl = torch.empty_like(dgs)
    ws_bytes = workspace_size(ENTRY_MERGE_BACKWARD, dm)
    ws = workspace(ws_bytes, q.device)
    _check(lib().natsl_merge_backward(
        C.byref(dm), _p(q, _io_t(dm), "q", qs), _p(o_sm, None, "o_sm", qs), _p(o_gdn, None, "o_gdn", qs), _dt(o_sm),
        _p(w_mix, torch.float32, "w_mix", wm_shape), w_mix_head_stride,
        _p(g_sm, torch.float32, "g_sm", (dm.Dv,)), _p(g_lin, torch.float32, "g_lin", (dm.Dv,)),
        _p(d_out, torch.float32, "d_out", qs), _p(d_sm), _p(d_gdn), _p(dq), _p(dwm), _p(dgs), _p(dgl),
        _p(ws), ws_bytes, _stream(stream)))
    return d_sm, d_gdn, dq, dwm, dgs, dgl


def decode_handoff(dm: Dims, route, k, v, S_final, state: DecodeState, append=False, stream=None):
    """Fill `state` as the decode cache after a prefill of dm.L tokens: the
    K/V rows of its softmax-routed chunks, S_carry = S_final (None: zero),
    empty open chunk.  `route` is the forward's route [B, G, L/64].  With
    append=True the tokens were a segment prefilled on top of `state`
    (Forward(..., prefix=state)) and its rows are added after the cached ones."""
    B, H, G, nc, D = dm.B, dm.H, dm.route_groups, dm.L // 64, dm.Dk
    io = _io_t(dm)
    if state.k.dtype != io or tuple(state.k.shape[:2]) != (B, H) or state.k.shape[3] != D:
        raise ValueError("decode state does not match the dims")
    if tuple(state.n_committed.shape) != (B, G) or tuple(state.x_sum.shape) != (B, dm.d_model):
        raise ValueError("decode state counters do not match the dims")
    ws_bytes = workspace_size(ENTRY_DECODE_HANDOFF, dm)
    ws = workspace(ws_bytes, k.device)
    cs = state.struct()
    _check(lib().natsl_decode_handoff(C.byref(dm), _p(route, torch.int32, "route", (B, G, nc)),
                                      _p(k, io, "k", (B, H, dm.L, D)), _p(v, io, "v", (B, H, dm.L, D)),
                                      _p(S_final, torch.float32, "S_final", (B, H, D, D)), 1 if append else 0,
                                      C.byref(cs),
                                      _p(ws), ws_bytes, _stream(stream)))
    return state


def profile_enable(on=True):
    _check(lib().natsl_profile_enable(1 if on else 0))


def set_sync_check(level):
    """Debug mode: 0 off, 1 each call waits for its stream and reports the
    first device error by entry point, 2 also names the call on stderr first."""
    _check(lib().natsl_set_sync_check(int(level)))


def get_sync_check():
    return lib().natsl_get_sync_check()


def profile_reset():
    _check(lib().natsl_profile_reset())


def profile_select(name=None):
    """Record only kernel `name` (None: every kernel)."""
    _check(lib().natsl_profile_select(name.encode() if name else None))


def profile_read(name):
    n, ms = C.c_int(0), C.c_double(0.0)
    _check(lib().natsl_profile_read(name.encode(), C.byref(n), C.byref(ms)))
    return n.value, ms.value
