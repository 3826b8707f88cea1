"""C ABI checks that need no GPU: the library loads, exports every function
include/natsl.h declares, and rejects bad arguments with the documented
status before anything is enqueued (the fake device pointers used here are
never dereferenced because validation fails first)."""
import ctypes as C
import os
import re
import threading

import pytest

import linear_attention_natsl_amd as N

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
HDR = os.path.join(ROOT, "include", "natsl.h")
FAKE = 0x10000  # stands in for a device pointer; never dereferenced

# Every call below must fail validation before anything is enqueued.  As a
# safety net these fake-pointer tests never run where a GPU is visible.
pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="fake-pointer validation tests run without a GPU only")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(N.LIB_PATH):
        from linear_attention_natsl_amd import build
        build.build()
    return N.lib()


def declared():
    src = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:natsl_status|int|const char\*)\s+(natsl_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(N.EXPORTS)


def test_version(L):
    assert N.version() == 100


def good(io=N.BF16):
    return N.dims(2, 4, 256, 128, 256, io)


@pytest.mark.parametrize("mut,status", [
    (lambda d: setattr(d, "chunk", 32), 2),
    (lambda d: setattr(d, "Dv", 64), 2),
    (lambda d: (setattr(d, "Dk", 96), setattr(d, "Dv", 96)), 2),
    (lambda d: setattr(d, "L", 100), 2),
    (lambda d: setattr(d, "L", 0), 2),
    (lambda d: setattr(d, "route_groups", 3), 2),
    (lambda d: setattr(d, "H", 0), 1),
    (lambda d: setattr(d, "B", -1), 1),
    (lambda d: setattr(d, "io", 7), 1),
])
def test_dims_validation(L, mut, status):
    d = good()
    mut(d)
    n = C.c_size_t(0)
    assert L.natsl_workspace_size(N.ENTRY_FORWARD, C.byref(d), C.byref(n)) == status
    assert L.natsl_last_error()


def test_dmodel_and_heads_limits(L):
    # the router keeps d_model floats of chunk mean plus 2G scores in LDS: the
    # dims check rejects larger shapes (2) before the NULL x is noticed (1)
    for dm, H, status in ((32768, 4, 1), (32776, 4, 2), (256, 1024, 1), (256, 1025, 2)):
        d = N.dims(1, H, 64, 128, dm, N.BF16)
        got = L.natsl_route(C.byref(d), None, None, None, None, None, None, None, None, None)
        assert got == status, (dm, H, got, L.natsl_last_error())


def test_route_validation(L):
    d = good()
    # x, w_score, b_score, route_in(NULL), route_out, sel_idx, nsel_before, scores, stream
    args = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None]
    assert L.natsl_route(None, *args) == 1
    bad = list(args)
    bad[0] = None  # x without route_in
    assert L.natsl_route(C.byref(d), *bad) == 1 and b"x" in L.natsl_last_error()
    d.d_model = 12  # router input width must be a multiple of 8
    assert L.natsl_route(C.byref(d), *args) == 2
    d.d_model = 256
    bad = list(args)
    bad[5] = None  # sel_idx
    assert L.natsl_route(C.byref(d), *bad) == 1 and b"sel_idx" in L.natsl_last_error()
    bad[3] = FAKE  # forced routes still need the outputs
    assert L.natsl_route(C.byref(d), *bad) == 1


def test_gdn_workspace_checks(L):
    d = good()
    need = N.workspace_size(N.ENTRY_GDN_CHUNK, d)
    assert need > 0
    base = [C.byref(d)] + [FAKE] * 8 + [N.F32, None]
    assert L.natsl_gdn_chunk(*base, None, need, None) == 3
    assert L.natsl_gdn_chunk(*base, FAKE + 8, need, None) == 3  # misaligned
    assert L.natsl_gdn_chunk(*base, FAKE, need - 1, None) == 3
    assert b"too small" in L.natsl_last_error()
    b2 = list(base)
    b2[6] = None  # route (base = dims, q, k, v, alpha, beta, route, S_init, o_gdn, o_dtype, S_final)
    assert L.natsl_gdn_chunk(*b2, FAKE, need, None) == 1
    b3 = list(base)
    b3[9] = 5  # bad o_dtype
    assert L.natsl_gdn_chunk(*b3, FAKE, need, None) == 1


def test_softmax_and_merge_validation(L):
    d = good()
    assert L.natsl_softmax_masked(C.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, None, None, 0, None) == 1
    assert L.natsl_softmax_masked(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 9, None, None, 0, None) == 1
    assert L.natsl_merge(C.byref(d), FAKE, FAKE, FAKE, 0, None, 0, None, None, FAKE, None) == 1
    assert L.natsl_merge(C.byref(d), FAKE, FAKE, FAKE, 0, FAKE, -2, None, None, FAKE, None) == 1


def test_forward_validation(L):
    d = good()
    a = N.ForwardArgs()
    assert L.natsl_forward(C.byref(d), None, FAKE, 1 << 30, None) == 1
    a.q = a.k = a.v = a.alpha = a.beta = a.w_mix = a.out = FAKE
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, 1 << 30, None) == 1  # no x, no override
    a.route_override = FAKE
    need = N.workspace_size(N.ENTRY_FORWARD, d)
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, need // 4, None) == 3
    a.branch_dtype = 3
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, need, None) == 1


def test_decode_validation(L):
    d = good()
    c = N.DecodeCache()
    a = N.DecodeArgs()
    assert L.natsl_decode_step(C.byref(d), C.byref(c), C.byref(a), None, 0, None) == 1
    for f in ("k_cache", "v_cache", "n_committed", "n_open", "S_carry", "S_work", "x_sum", "err_flag"):
        setattr(c, f, FAKE)
    c.cap = 0
    assert L.natsl_decode_step(C.byref(d), C.byref(c), C.byref(a), None, 0, None) == 1
    c.cap = 1024
    for f in ("x", "q", "k", "v", "alpha", "beta", "w_score", "w_mix", "out"):
        setattr(a, f, FAKE)
    assert L.natsl_decode_step(C.byref(d), C.byref(c), C.byref(a), None, 0, None) == 3
    d2 = N.dims(2, 4, 1024, 128, 256, N.BF16)
    need = N.workspace_size(N.ENTRY_DECODE_STEP, d2)
    assert need > 0
    assert L.natsl_decode_step(C.byref(d), C.byref(c), C.byref(a), FAKE, need - 256, None) == 3


def test_decode_handoff_validation(L):
    d = good()
    c = N.DecodeCache()
    for f in ("k_cache", "v_cache", "n_committed", "n_open", "S_carry", "S_work", "x_sum", "err_flag"):
        setattr(c, f, FAKE)
    c.cap = 1024
    need = N.workspace_size(N.ENTRY_DECODE_HANDOFF, d)
    assert need == d.B * d.route_groups * (2 * (d.L // 64) + 1) * 4
    call = lambda dd, route, cc, ws, nbytes, append=0, S=None: L.natsl_decode_handoff(
        C.byref(dd), route, FAKE, FAKE, S, append, C.byref(cc), ws, nbytes, None)
    assert call(d, None, c, FAKE, need) == 1             # route missing
    assert call(d, FAKE, c, FAKE, need - 4) == 3         # workspace too small
    bad = good()
    bad.L = 100
    assert call(bad, FAKE, c, FAKE, need) == 2           # L not a whole number of chunks
    c0 = N.DecodeCache()
    assert call(d, FAKE, c0, FAKE, need) == 1            # cache tensors missing
    c.cap = 0
    assert call(d, FAKE, c, FAKE, need) == 1             # no capacity
    empty = good()
    empty.B = 0
    assert call(empty, None, N.DecodeCache(), None, 0) == 0  # empty batch is a no-op
    c.cap = 1024
    assert call(d, FAKE, c, FAKE, need, append=1) == 1   # appending needs S_final
    assert call(d, FAKE, c, FAKE, need, append=2, S=FAKE) == 1  # append is 0 or 1


def test_forward_prefix_validation(L):
    d = good()
    a = N.ForwardArgs()
    for f in ("x", "q", "k", "v", "alpha", "beta", "w_score", "w_mix", "out"):
        setattr(a, f, FAKE)
    c = N.DecodeCache()
    a.prefix = C.cast(C.pointer(c), C.c_void_p)
    need = N.workspace_size(N.ENTRY_FORWARD, d)
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, need, None) == 1      # prefix tensors missing
    for f in ("k_cache", "v_cache", "n_committed", "n_open", "S_carry", "S_work", "x_sum", "err_flag"):
        setattr(c, f, FAKE)
    c.cap = -1
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, need, None) == 1      # bad capacity
    c.cap = 1024
    a.S_init = FAKE
    assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, need, None) == 1      # S_init with a prefix
    assert b"exclusive" in L.natsl_last_error()


def test_workspace_sizes_monotone(L):
    prev = 0
    for Lq in (64, 128, 1024, 4096):
        n = N.workspace_size(N.ENTRY_FORWARD, N.dims(1, 16, Lq, 128, 2048, N.BF16))
        assert n > prev
        prev = n
    a = N.workspace_size(N.ENTRY_GDN_CHUNK, N.dims(1, 16, 4096, 128, 2048, N.BF16))
    b = N.workspace_size(N.ENTRY_GDN_CHUNK, N.dims(2, 16, 4096, 128, 2048, N.BF16))
    assert b > a
    assert N.workspace_size(N.ENTRY_SOFTMAX_MASKED, N.dims(1, 16, 4096, 128, 2048, N.BF16)) == 0


def test_gdn_backward_overlap_workspace(L):
    """natsl_gdn_backward's overlapping layout gives the forward prep's output
    and the backward prep's output plus Gc regions of their own: on the long
    prefill (B 1, H 16, L 32768, bf16 D 128) 0.877 GB shared, 1.352 GB apart
    (each region 57920 bytes per chunk-head, S0 32768 and U 16384)."""
    d = N.dims(1, 16, 32768, 128, 2048, N.BF16)
    a = N.workspace_size(N.ENTRY_GDN_BACKWARD, d)
    b = N.workspace_size(N.ENTRY_GDN_BACKWARD_OVERLAP, d)
    nch = 16 * 512
    assert abs(a - nch * (32768 + 16384 + 57920)) <= 4 * 256
    assert abs(b - nch * (32768 + 16384 + 2 * 57920)) <= 8 * 256
    for io, D in ((N.F32, 64), (N.F32, 128), (N.BF16, 64)):
        d = N.dims(2, 4, 640, D, 256, io)
        assert N.workspace_size(N.ENTRY_GDN_BACKWARD_OVERLAP, d) > N.workspace_size(N.ENTRY_GDN_BACKWARD, d)


def test_last_error_is_thread_local(L):
    L.natsl_route(None, *([None] * 9))
    assert L.natsl_last_error() != b""
    seen = []
    t = threading.Thread(target=lambda: seen.append(L.natsl_last_error()))
    t.start()
    t.join()
    assert seen == [b""]


def test_binding_rejects_without_gpu_tensor():
    import torch
    with pytest.raises(ValueError):
        N._p(torch.zeros(3), name="x")


def test_profile_select(L):
    # selecting a kernel only sets host state: no GPU involved
    assert L.natsl_profile_select(b"no_such_kernel") == 1
    assert b"no_such_kernel" in N.lib().natsl_last_error()
    for name in (b"softmax_masked", b"decode_attn", b"", None):
        assert L.natsl_profile_select(name) == 0
    with pytest.raises(N.NatslError):
        N.profile_select("gdn_everything")
    N.profile_select("merge")
    N.profile_select(None)


def test_binding_argtypes_match_prototypes(L):
    """The ctypes argument list of every declared function has the length of
    its C prototype (a short list passes the trailing stream handle as a
    32-bit int)."""
    src = open(HDR).read()
    protos = {m.group(1): m.group(2) for m in re.finditer(r"natsl_status\s+(natsl_\w+)\s*\(([^;]*?)\);", src, re.S)}
    assert len(protos) >= 12
    for name, args in protos.items():
        n = 0 if args.strip() == "void" else len([a for a in args.split(",") if a.strip()])
        at = getattr(L, name).argtypes
        assert (at is None and n == 0) or (at is not None and len(at) == n), (name, n, at)


def test_gdn_length_limit_rejected_before_enqueue(L):
    """bf16 D = 128 keeps one route byte per chunk in the scan's LDS: up to
    15232 chunks (L = 974848) are accepted, one chunk more is UNSUPPORTED in
    natsl_workspace_size, natsl_gdn_chunk and natsl_forward, before anything
    is enqueued (the fake pointers are never touched); a 128k-token prefill
    is accepted; fp32 io has no such limit."""
    lim = 15232
    for nch, io, ok in ((lim, N.BF16, True), (lim + 1, N.BF16, False), (2048, N.BF16, True), (lim + 1, N.F32, True)):
        d = N.dims(1, 1, 64 * nch, 128, 256, io)
        n = C.c_size_t(0)
        for entry in (N.ENTRY_FORWARD, N.ENTRY_GDN_CHUNK):
            got = L.natsl_workspace_size(entry, C.byref(d), C.byref(n))
            assert got == (0 if ok else 2), (nch, io, entry, got)
        if not ok:
            assert b"15232" in L.natsl_last_error()
            assert L.natsl_gdn_chunk(C.byref(d), *([FAKE] * 6), None, FAKE, 0, None, FAKE, 1 << 40, None) == 2
            a = N.ForwardArgs()
            a.q = a.k = a.v = a.alpha = a.beta = a.w_mix = a.out = a.route_override = FAKE
            assert L.natsl_forward(C.byref(d), C.byref(a), FAKE, 1 << 40, None) == 2


def test_decode_noalloc_rejects_oversized_before_enqueue(L):
    """The allocation-free decode step holds 16 MiB of scratch per device: dims
    that need more are NATSL_ERR_WORKSPACE before anything is enqueued (the
    fake pointers are never touched)."""
    assert N.DECODE_NOALLOC_SCRATCH_BYTES == 16 << 20
    d = N.dims(64, 16, 40000, 128, 256, N.BF16)
    assert N.workspace_size(N.ENTRY_DECODE_STEP, d) > N.DECODE_NOALLOC_SCRATCH_BYTES
    c = N.DecodeCache(FAKE, FAKE, 40000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    a = N.DecodeArgs()
    a.x = a.q = a.k = a.v = a.alpha = a.beta = a.w_score = a.w_mix = a.out = FAKE
    d.L = 1
    assert L.natsl_decode_step_noalloc(C.byref(d), C.byref(c), C.byref(a), None) == 3
    assert b"16777216" in L.natsl_last_error()
    assert L.natsl_decode_step_noalloc(C.byref(d), None, C.byref(a), None) == 1


def test_sync_check_level(L):
    """The synchronous-check debug level is host state: 0..2 are accepted and
    read back, anything else is INVALID_ARG and changes nothing; without a
    call, NATSL_SYNC_CHECK in the environment sets it (read in a fresh
    process)."""
    import subprocess
    import sys
    try:
        assert L.natsl_set_sync_check(3) == 1 and b"sync check level" in L.natsl_last_error()
        assert L.natsl_set_sync_check(-1) == 1
        for lv in (1, 2, 0):
            assert L.natsl_set_sync_check(lv) == 0 and L.natsl_get_sync_check() == lv
        N.set_sync_check(1)
        assert N.get_sync_check() == 1
        with pytest.raises(N.NatslError):
            N.set_sync_check(7)
        assert N.get_sync_check() == 1
    finally:
        N.set_sync_check(0)
    code = "import linear_attention_natsl_amd as N; print(N.get_sync_check())"
    for env_val, want in (("2", 2), ("1", 1), ("yes", 1), ("0", 0), ("", 0), (None, 0)):
        env = dict(os.environ)
        env.pop("NATSL_SYNC_CHECK", None)
        if env_val is not None:
            env["NATSL_SYNC_CHECK"] = env_val
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        assert r.stdout.strip().splitlines()[-1] == str(want), (env_val, r.stdout)


def test_missing_library_fails_loudly():
    """Without the built library the binding raises (no CPU fallback exists):
    run in a fresh interpreter whose loader points at a file that is not there."""
    import subprocess
    import sys
    code = ("import linear_attention_natsl_amd as N\n"
            "N._lib = None\n"
            "N.LIB_PATH = N.LIB_PATH + '.not_built'\n"
            "try:\n"
            "    N.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "no fallback" in r.stdout
