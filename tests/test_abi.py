"""CPU checks of the C ABI: the library loads, exports every function that
include/miep.h declares, and its host-only helpers and argument validation
behave as documented.  No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from combine_get_dispatch_histogram_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miep.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(miep_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from combine_get_dispatch_histogram_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared()
    for f in ("miep_get_dispatch_layout", "miep_dispatch", "miep_cached_dispatch", "miep_combine",
              "miep_relay_dispatch", "miep_relay_cached_dispatch", "miep_relay_combine",
              "miep_ll_dispatch", "miep_ll_combine", "miep_mask_update", "miep_mask_clean", "miep_mask_query"):
        assert f in names
    assert set(names) == set(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(miep_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_host_helpers(lib):
    assert lib.miep_ll_msg_bytes(7168, 1) == 7408
    assert lib.miep_ll_msg_bytes(7168, 0) == 14352
    assert lib.miep_ll_msg_bytes(128, 1) == 160 and lib.miep_ll_msg_bytes(640, 1) == 688   # 16-byte stride
    assert lib.miep_ll_msg_bytes(0, 1) == -1
    assert b"gfx950" in lib.miep_version()


def _problem(**kw):
    d = dict(num_src=8, num_tokens=512, hidden=7168, num_topk=8, num_experts=256, num_ranks=8, num_channels=24,
             expert_alignment=1)
    d.update(kw)
    return _lib.Problem(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(num_experts=250), _lib.MIEP_EINVAL),          # E % R != 0
    (dict(num_ranks=12, num_experts=240), _lib.MIEP_EINVAL),   # R > 8, R % 8 != 0
    (dict(num_ranks=512, num_experts=512), _lib.MIEP_EUNSUPPORTED),
    (dict(num_experts=16384, num_ranks=8), _lib.MIEP_EUNSUPPORTED),
    (dict(expert_alignment=0), _lib.MIEP_EINVAL),
    (dict(num_channels=0), _lib.MIEP_EINVAL),
    (dict(num_tokens=-1), _lib.MIEP_EINVAL),
    (dict(num_topk=65), _lib.MIEP_EUNSUPPORTED),
])
def test_layout_rejects_bad_problems(lib, kw, status):
    p = _problem(**kw)
    rc = lib.miep_get_dispatch_layout(ctypes.byref(p), 16, 16, None, 16, 16, None)
    assert rc == status, lib.miep_last_error()
    assert lib.miep_last_error()


def test_layout_rejects_null_and_rdma_mismatch(lib):
    p = _problem()
    assert lib.miep_get_dispatch_layout(None, 16, 16, None, 16, 16, None) == _lib.MIEP_EINVAL
    assert lib.miep_get_dispatch_layout(ctypes.byref(p), None, 16, None, 16, 16, None) == _lib.MIEP_EINVAL
    # R = 8: the RDMA counts must be NULL; R = 16: they are required
    assert lib.miep_get_dispatch_layout(ctypes.byref(p), 16, 16, 16, 16, 16, None) == _lib.MIEP_EINVAL
    p16 = _problem(num_ranks=16)
    assert lib.miep_get_dispatch_layout(ctypes.byref(p16), 16, 16, None, 16, 16, None) == _lib.MIEP_EINVAL


def _dispatch(lib, p, h, x=16, kind=0, x_scales=None, round_scale=0, use_ue8m0=0, recv_x_scales=None, ue=None,
              status=None):
    # p, x, kind, x_scales, round_scale, use_ue8m0, topk_idx, topk_weights, num_tokens_per_rank,
    # num_tokens_per_expert, recv_x, recv_x_scales, recv_x_scales_ue8m0, recv_topk_idx, recv_topk_weights,
    # num_recv_tokens_per_expert, status, handle, stream
    return lib.miep_dispatch(ctypes.byref(p), x, kind, x_scales, round_scale, use_ue8m0, 16, 16, 16, 16, 16,
                             recv_x_scales, ue, 16, 16, None, status, ctypes.byref(h), None)


def test_dispatch_validation(lib):
    p = _problem()
    h = _lib.HandleC(16, 16, 16, 16, 16, 16, 16, 100)
    assert _dispatch(lib, p, h, x=8) == _lib.MIEP_EUNSUPPORTED                  # misaligned x
    assert _dispatch(lib, p, h, kind=1) == _lib.MIEP_EINVAL                     # FP8 payload without scales
    assert _dispatch(lib, p, h, kind=7) == _lib.MIEP_EINVAL                     # unknown kind
    hbad = _lib.HandleC(None, 16, 16, 16, 16, 16, 16, 100)
    assert _dispatch(lib, p, hbad) == _lib.MIEP_EINVAL                         # handle missing arrays
    p2 = _problem(hidden=200)
    assert _dispatch(lib, p2, h, kind=2, recv_x_scales=16) == _lib.MIEP_EINVAL  # FP8 cast needs hidden % 128 == 0
    # use_ue8m0: only with the fused cast and power-of-two scales, and with somewhere to put the bytes
    assert _dispatch(lib, p, h, kind=2, recv_x_scales=16, use_ue8m0=1, ue=16) == _lib.MIEP_EINVAL
    assert _dispatch(lib, p, h, kind=0, round_scale=1, use_ue8m0=1, ue=16) == _lib.MIEP_EINVAL
    assert _dispatch(lib, p, h, kind=2, recv_x_scales=16, round_scale=1, use_ue8m0=1) == _lib.MIEP_EINVAL
    assert "ue8m0" in lib.miep_last_error().decode()
    # receive rows are int32: N * min(K, R) must stay below 2^31 (here 2^28 tokens reach up to 8 ranks each)
    big = _problem(num_src=1 << 10, num_tokens=1 << 18, num_topk=8, num_ranks=8, num_experts=64)
    assert _dispatch(lib, big, h) == _lib.MIEP_EUNSUPPORTED
    assert "receive rows" in lib.miep_last_error().decode()
    assert _dispatch(lib, _problem(num_src=1 << 10, num_tokens=1 << 18, num_topk=7, num_ranks=8, num_experts=64),
                     h, x=8) == _lib.MIEP_EUNSUPPORTED and "aligned" in lib.miep_last_error().decode()
    # negative capacity
    hneg = _lib.HandleC(16, 16, 16, 16, 16, 16, 16, -1)
    rc = lib.miep_cached_dispatch(ctypes.byref(p), 16, 0, None, 0, 0, ctypes.byref(hneg), 16, None, None, None)
    assert rc == _lib.MIEP_EINVAL
    rc = lib.miep_cached_dispatch(ctypes.byref(p), 16, 2, None, 0, 1, ctypes.byref(h), 16, 16, 16, None)
    assert rc == _lib.MIEP_EINVAL                                              # ue8m0 without round_scale


def test_status_codes_and_check(lib):
    """The capacity status code matches the header, and reading a status word validates its pointer."""
    text = open(HEADER).read()
    assert re.search(r"MIEP_ECAPACITY\s*=\s*4", text) and _lib.MIEP_ECAPACITY == 4
    assert lib.miep_check_status(None, None) == _lib.MIEP_EINVAL
    assert lib.miep_last_error()


def test_problem_bounds(lib):
    h = _lib.HandleC(16, 16, 16, 16, 16, 16, 16, 0)
    for bad, code in ((dict(num_src=(1 << 20) + 1, num_tokens=0), _lib.MIEP_EUNSUPPORTED),
                      (dict(num_channels=1025), _lib.MIEP_EUNSUPPORTED),
                      (dict(num_topk=65), _lib.MIEP_EUNSUPPORTED),
                      (dict(num_ranks=512, num_experts=512), _lib.MIEP_EUNSUPPORTED),
                      (dict(num_src=70000, num_tokens=40000), _lib.MIEP_EUNSUPPORTED)):
        p = _problem(**bad)
        assert lib.miep_combine(ctypes.byref(p), 16, None, None, None, ctypes.byref(h), 16, None, None) == code, bad


def test_combine_validation(lib):
    p = _problem()
    h = _lib.HandleC(16, 16, 16, 16, 16, 16, 16, 100)
    def c(y, w, b0, b1, out, cw):
        return lib.miep_combine(ctypes.byref(p), y, w, b0, b1, ctypes.byref(h), out, cw, None)

    assert c(None, None, None, None, 16, None) == _lib.MIEP_EINVAL        # y NULL
    assert c(16, 16, None, None, 16, None) == _lib.MIEP_EINVAL            # weights without their output
    assert c(8, None, None, None, 16, None) == _lib.MIEP_EUNSUPPORTED     # misaligned y
    assert c(16, None, 8, None, 16, None) == _lib.MIEP_EUNSUPPORTED       # misaligned bias_0
    assert c(16, None, None, 24, 16, None) == _lib.MIEP_EUNSUPPORTED      # misaligned bias_1


def test_relay_validation(lib):
    p = _problem(num_ranks=64)
    h = _lib.HandleC(16, 16, 16, 16, 16, 16, 16, 100)
    rh = _lib.RelayHandleC(16, 16, 16, 16, 16, 16, 16, 50)

    def d(prob, handle, relay, rdma_x=16):
        return lib.miep_relay_dispatch(ctypes.byref(prob), 16, 0, None, 0, 16, 16, 16, 16, 16, rdma_x, None, 16,
                                       None, 16, 16, None, None, ctypes.byref(handle), relay, None)

    assert d(_problem(num_ranks=8), h, ctypes.byref(rh)) == _lib.MIEP_EUNSUPPORTED      # one group only
    assert d(_problem(num_ranks=12), h, ctypes.byref(rh)) == _lib.MIEP_EINVAL          # R > 8 not a multiple of 8
    assert d(p, h, None) == _lib.MIEP_EINVAL                                          # no relay handle
    assert d(p, h, ctypes.byref(rh), rdma_x=None) == _lib.MIEP_EINVAL                  # rdma_x NULL
    assert d(p, h, ctypes.byref(rh), rdma_x=8) == _lib.MIEP_EUNSUPPORTED               # misaligned rdma_x
    bad = _lib.RelayHandleC(16, 16, 16, 16, 16, 16, 24, 50)                           # misaligned send_nvl_head
    assert d(p, h, ctypes.byref(bad)) == _lib.MIEP_EUNSUPPORTED
    neg = _lib.RelayHandleC(16, 16, 16, 16, 16, 16, 16, -1)
    assert d(p, h, ctypes.byref(neg)) == _lib.MIEP_EINVAL

    def c(relay, y=16, w=None, rdma_y=16, rdma_w=None, out=16, cw=None, f32=0):
        return lib.miep_relay_combine(ctypes.byref(p), y, w, None, None, ctypes.byref(h), relay, f32, rdma_y, rdma_w,
                                      out, cw, None)

    assert c(ctypes.byref(rh), y=None) == _lib.MIEP_EINVAL
    assert c(ctypes.byref(rh), rdma_y=None) == _lib.MIEP_EINVAL
    assert c(ctypes.byref(rh), w=16) == _lib.MIEP_EINVAL                               # weights without rdma_w
    assert c(ctypes.byref(rh), y=8) == _lib.MIEP_EUNSUPPORTED
    assert c(ctypes.byref(rh), rdma_y=8, f32=1) == _lib.MIEP_EUNSUPPORTED              # misaligned fp32 partials


def test_ll_validation(lib):
    def q(**kw):
        d = dict(num_ranks=32, num_tokens=128, max_tokens=128, hidden=7168, num_topk=8, num_experts=256, dest_rank=0)
        d.update(kw)
        return _lib.LLProblem(**d)

    args = [16, 16, 1, 1, 1, 16, 16, 16, 16, 16, 16, 16, 16, None, None, None]
    assert lib.miep_ll_dispatch(ctypes.byref(q(num_tokens=129)), *args) == _lib.MIEP_EINVAL
    assert lib.miep_ll_dispatch(ctypes.byref(q(num_topk=65)), *args) == _lib.MIEP_EUNSUPPORTED
    assert lib.miep_ll_dispatch(ctypes.byref(q(num_experts=250)), *args) == _lib.MIEP_EINVAL
    assert lib.miep_ll_dispatch(ctypes.byref(q(dest_rank=32)), *args) == _lib.MIEP_EINVAL
    assert lib.miep_ll_dispatch(ctypes.byref(q(hidden=7000)), *args) == _lib.MIEP_EINVAL   # FP8 needs H % 128 == 0
    bad = list(args)
    bad[3], bad[4] = 0, 1                      # ue8m0 without round_scale
    assert lib.miep_ll_dispatch(ctypes.byref(q()), *bad) == _lib.MIEP_EINVAL
    nul = list(args)
    nul[5] = None                              # msg_buf NULL
    assert lib.miep_ll_dispatch(ctypes.byref(q()), *nul) == _lib.MIEP_EINVAL

    cargs = [16, 16, 16, 16, None, 16, None]   # y, src_info, layout_range, topk_idx, weights, out, stream
    assert lib.miep_ll_combine(None, *cargs) == _lib.MIEP_EINVAL
    assert lib.miep_ll_combine(ctypes.byref(q(dest_rank=-1)), *cargs) == _lib.MIEP_EINVAL
    assert lib.miep_ll_combine(ctypes.byref(q(max_tokens=8192, num_tokens=8)), *cargs) == _lib.MIEP_EUNSUPPORTED
    bad = list(cargs)
    bad[1] = None                              # src_info NULL
    assert lib.miep_ll_combine(ctypes.byref(q()), *bad) == _lib.MIEP_EINVAL
    bad = list(cargs)
    bad[0] = 8                                 # misaligned y
    assert lib.miep_ll_combine(ctypes.byref(q()), *bad) == _lib.MIEP_EUNSUPPORTED


def test_ll_noalloc_validation(lib):
    """The allocation-free low-latency dispatch checks its sizes before touching the device: more experts
    than its count array holds (65536) is EUNSUPPORTED, and the usual argument errors are reported."""
    def q(**kw):
        d = dict(num_ranks=32, num_tokens=128, max_tokens=128, hidden=7168, num_topk=8, num_experts=256, dest_rank=0)
        d.update(kw)
        return _lib.LLProblem(**d)

    # x, topk_idx, use_fp8, round_scale, use_ue8m0, packed_recv_x, scales, ue8m0, src_info, layout_range, count,
    # cumulative stats, mask, stream
    args = [16, 16, 0, 0, 0, 16, None, None, 16, 16, 16, None, None, None]
    assert lib.miep_ll_dispatch_noalloc(ctypes.byref(q(num_ranks=2, num_tokens=4, max_tokens=8,
                                                       num_experts=2 * 65536)), *args) == _lib.MIEP_EUNSUPPORTED
    assert "65536" in lib.miep_last_error().decode()
    assert lib.miep_ll_dispatch_noalloc(ctypes.byref(q(num_tokens=129)), *args) == _lib.MIEP_EINVAL
    bad = list(args)
    bad[5] = None                              # packed_recv_x NULL
    assert lib.miep_ll_dispatch_noalloc(ctypes.byref(q()), *bad) == _lib.MIEP_EINVAL
    bad = list(args)
    bad[2] = 1                                 # FP8 without scales
    assert lib.miep_ll_dispatch_noalloc(ctypes.byref(q()), *bad) == _lib.MIEP_EINVAL


def test_mask_validation(lib):
    assert lib.miep_mask_update(None, 8, 0, 1, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_update(16, 8, 8, 1, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_update(16, 8, -1, 1, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_update(16, 0, 0, 1, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_clean(None, 8, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_clean(16, 0, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_query(16, 8, None, None) == _lib.MIEP_EINVAL
    assert lib.miep_mask_query(None, 8, 16, None) == _lib.MIEP_EINVAL


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_binding_rejects_host_and_mixed_device_tensors():
    """The binding refuses host tensors before anything reaches the library,
    and refuses a call whose tensors sit on two different GPUs."""
    import types

    import torch

    import combine_get_dispatch_histogram_amd as miep
    idx = torch.zeros((8, 2), dtype=torch.int64)
    with pytest.raises(ValueError, match="device tensors"):
        miep.get_dispatch_layout(idx, 8, 4, 4)
    a = miep._Args()
    a._see(types.SimpleNamespace(is_cuda=True, device="cuda:0"))
    a._see(types.SimpleNamespace(is_cuda=True, device="cuda:0"))
    with pytest.raises(ValueError, match="one device"):
        a._see(types.SimpleNamespace(is_cuda=True, device="cuda:1"))
