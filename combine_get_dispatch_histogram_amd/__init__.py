"""miep -- MI355X-native MoE expert-parallel core: layout, dispatch, handle, combine.

A thin Python face over ``libmiep.so`` (C ABI in ``include/miep.h``).  This
module only checks tensor shapes / dtypes / devices, allocates outputs with
PyTorch and passes raw device pointers plus the current HIP stream; every step
of the computation runs in the library's gfx950 kernels.  There is no
fallback: without the built library every call raises.

Calls (the API surface of "Chapter 4  V1: layout, dispatch and combine",
sections 4.1-4.3, for ranks that are partitions of one GPU):
  get_dispatch_layout(topk_idx, num_experts, num_ranks)            section 4.1
  dispatch(x, topk_idx, topk_weights, <layout>, ...) -> (..., handle)  4.1
  cached_dispatch(x, handle)                                        4.1 (cached)
  combine(y, handle, topk_weights, bias)                            4.2, 4.4
  relay_dispatch / relay_combine: the same through one buffer per group of 8
  ranks (the two-level RDMA + NVLink relay), with a RelayHandle
  low_latency_dispatch(x, topk_idx, max_tokens, num_experts, dest_rank, ...)  4.3
  low_latency_combine(y, topk_idx, topk_weights, <dispatch outputs>, ...)     4.3
  update_mask_buffer / clean_mask_buffer / query_mask_buffer        rank masking
The ``*_into`` variants take preallocated outputs and allocate nothing.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import MIEP_ECAPACITY, MiepError, X_BF16, X_BF16_CAST_FP8, X_FP8  # noqa: F401

__all__ = ["Handle", "MiepError", "get_dispatch_layout", "get_dispatch_layout_into", "dispatch", "dispatch_into", "cached_dispatch",
           "cached_dispatch_into", "combine", "combine_into", "low_latency_dispatch", "low_latency_dispatch_into",
           "low_latency_dispatch_noalloc", "low_latency_combine", "low_latency_combine_into", "update_mask_buffer",
           "clean_mask_buffer",
           "RelayHandle", "relay_dispatch", "relay_dispatch_into", "relay_cached_dispatch",
           "relay_cached_dispatch_into", "relay_combine", "relay_combine_into",
           "query_mask_buffer", "check_status", "ll_msg_bytes", "version", "MIEP_ECAPACITY"]


class _Args:
    """Pointer marshalling for one library call: every tensor it passes must be
    a contiguous device tensor on one and the same GPU, and the call runs with
    that GPU current and on its current stream."""

    def __init__(self):
        self.dev = None

    def _see(self, t: torch.Tensor) -> None:
        if not t.is_cuda:
            raise ValueError("miep expects device tensors")
        if self.dev is None:
            self.dev = t.device
        elif t.device != self.dev:
            raise ValueError("miep expects every tensor of a call on one device (%s and %s)" % (self.dev, t.device))

    def p(self, t: Optional[torch.Tensor]):
        if t is None:
            return None
        self._see(t)
        if not t.is_contiguous():
            raise ValueError("miep expects contiguous tensors")
        return ctypes.c_void_p(t.data_ptr())

    def handle(self, h) -> None:
        for t in h.tensors():
            self.p(t)


def _run(a: _Args, name: str, *args) -> None:
    if a.dev is None:
        raise ValueError("miep call without device tensors")
    with torch.cuda.device(a.dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(a.dev).cuda_stream)
        _lib.check(getattr(_lib.load(), name)(*args, stream))


def _want(t: Optional[torch.Tensor], name: str, dtype, shape=None):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def version() -> str:
    return _lib.load().miep_version().decode()


def check_status(status: torch.Tensor) -> None:
    """Read a dispatch's device status word (synchronous: waits for the
    current stream); raises MiepError(MIEP_ECAPACITY) if the receive rows
    exceeded their fixed capacity."""
    _want(status, "status", torch.int32, (1,))
    a = _Args()
    _run(a, "miep_check_status", a.p(status))


def ll_msg_bytes(hidden: int, use_fp8: bool) -> int:
    return int(_lib.load().miep_ll_msg_bytes(hidden, int(bool(use_fp8))))


# --------------------------------------------------------------------------- handle
@dataclass
class Handle:
    """The reverse-routing record of a normal dispatch (section 4.2).

    rank_prefix_matrix [S,R], channel_prefix_matrix [S,R,C],
    recv_channel_prefix_matrix [R,S,C], recv_rank_offset [R+1] (last = total
    rows), recv_src_idx [cap], is_token_in_rank [N,R] bool, send_head [N,R].
    Rank r's rows are receive rows recv_rank_offset[r] .. recv_rank_offset[r+1].
    """
    rank_prefix_matrix: torch.Tensor
    channel_prefix_matrix: torch.Tensor
    recv_channel_prefix_matrix: torch.Tensor
    recv_rank_offset: torch.Tensor
    recv_src_idx: torch.Tensor
    is_token_in_rank: torch.Tensor
    send_head: torch.Tensor
    num_src: int
    num_tokens: int
    num_topk: int
    num_experts: int
    num_ranks: int
    num_channels: int

    @property
    def recv_capacity(self) -> int:
        return self.recv_src_idx.numel()

    @staticmethod
    def allocate(is_token_in_rank: torch.Tensor, num_src: int, num_topk: int, num_experts: int, num_channels: int,
                 capacity: int) -> "Handle":
        N, R = is_token_in_rank.shape
        S = num_src
        dev = is_token_in_rank.device
        i32 = dict(dtype=torch.int32, device=dev)
        return Handle(torch.empty((S, R), **i32), torch.empty((S, R, num_channels), **i32),
                      torch.empty((R, S, num_channels), **i32), torch.empty((R + 1,), **i32),
                      torch.empty((capacity,), **i32), is_token_in_rank, torch.empty((N, R), **i32), S,
                      N // S if S else 0, num_topk, num_experts, R, num_channels)

    def tensors(self):
        return (self.rank_prefix_matrix, self.channel_prefix_matrix, self.recv_channel_prefix_matrix,
                self.recv_rank_offset, self.recv_src_idx, self.is_token_in_rank, self.send_head)

    def c(self) -> _lib.HandleC:
        return _lib.HandleC(self.rank_prefix_matrix.data_ptr(), self.channel_prefix_matrix.data_ptr(),
                            self.recv_channel_prefix_matrix.data_ptr(), self.recv_rank_offset.data_ptr(),
                            self.recv_src_idx.data_ptr(), self.is_token_in_rank.data_ptr(),
                            self.send_head.data_ptr(), self.recv_capacity)

    def problem(self, hidden: int, expert_alignment: int = 1) -> _lib.Problem:
        return _lib.Problem(self.num_src, self.num_tokens, hidden, self.num_topk, self.num_experts, self.num_ranks,
                            self.num_channels, expert_alignment)


def _x_kind(x: torch.Tensor, cast_to_fp8: bool) -> int:
    if x.dtype == torch.bfloat16:
        return X_BF16_CAST_FP8 if cast_to_fp8 else X_BF16
    if x.dtype in (torch.float8_e4m3fn, torch.uint8):
        if cast_to_fp8:
            raise ValueError("x is already FP8")
        return X_FP8
    raise TypeError("x must be bf16 or float8_e4m3fn/uint8 codes, got %s" % x.dtype)


# --------------------------------------------------------------------------- layout
def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int, num_src: Optional[int] = None):
    """Per-rank, per-RDMA-rank, per-expert token counts and the token-in-rank matrix.

    topk_idx [N, K] int64 on the GPU (negative = masked); the N tokens are
    ``num_src`` (default: num_ranks) consecutive source partitions.  Returns
    (num_tokens_per_rank [S,R] i32, num_tokens_per_rdma_rank [S,R/8] i32 or
    None when R <= 8, num_tokens_per_expert [S,E] i32, is_token_in_rank [N,R] bool).
    """
    _want(topk_idx, "topk_idx", torch.int64)
    N, K = topk_idx.shape
    S = num_ranks if num_src is None else num_src
    if S <= 0 or N % S:
        raise ValueError("the %d tokens do not split into %d source partitions" % (N, S))
    dev = topk_idx.device
    i32 = dict(dtype=torch.int32, device=dev)
    ntpr = torch.empty((S, num_ranks), **i32)
    ntp_rdma = torch.empty((S, num_ranks // 8), **i32) if num_ranks > 8 else None
    ntpe = torch.empty((S, num_experts), **i32)
    itr = torch.empty((N, num_ranks), dtype=torch.bool, device=dev)
    get_dispatch_layout_into(topk_idx, num_experts, num_ranks, S, ntpr, ntp_rdma, ntpe, itr)
    return ntpr, ntp_rdma, ntpe, itr


def get_dispatch_layout_into(topk_idx, num_experts: int, num_ranks: int, num_src: int, num_tokens_per_rank,
                             num_tokens_per_rdma_rank, num_tokens_per_expert, is_token_in_rank) -> None:
    """get_dispatch_layout into preallocated outputs (allocates nothing)."""
    N, K = topk_idx.shape
    S, R = num_src, num_ranks
    if S <= 0 or N % S:
        raise ValueError("the %d tokens do not split into %d source partitions" % (N, S))
    _want(topk_idx, "topk_idx", torch.int64)
    _want(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (S, R))
    _want(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (S, num_experts))
    _want(is_token_in_rank, "is_token_in_rank", torch.bool, (N, R))
    if R > 8:
        _want(num_tokens_per_rdma_rank, "num_tokens_per_rdma_rank", torch.int32, (S, R // 8))
    p = _lib.Problem(S, N // S, 8, K, num_experts, R, 1, 1)
    a = _Args()
    _run(a, "miep_get_dispatch_layout", ctypes.byref(p), a.p(topk_idx), a.p(num_tokens_per_rank),
         a.p(num_tokens_per_rdma_rank), a.p(num_tokens_per_expert), a.p(is_token_in_rank))


# --------------------------------------------------------------------------- dispatch
def dispatch_into(x, topk_idx, topk_weights, num_tokens_per_rank, num_tokens_per_expert, handle: Handle, recv_x,
                  recv_x_scales=None, recv_topk_idx=None, recv_topk_weights=None, num_recv_tokens_per_expert=None,
                  x_scales=None, cast_to_fp8: bool = False, round_scale: bool = False,
                  expert_alignment: int = 1, use_ue8m0: bool = False, recv_x_scales_ue8m0=None,
                  status=None) -> None:
    """Fresh dispatch into preallocated outputs (allocates nothing).  ``status`` ([1] int32, optional) receives
    0 or MIEP_ECAPACITY (read it with ``check_status``); ``recv_x_scales_ue8m0`` ([cap, H/128] uint8) receives
    the scales' exponent bytes when ``use_ue8m0``."""
    kind = _x_kind(x, cast_to_fp8)
    _check_payload_shapes(x, kind, x_scales, handle, recv_x, recv_x_scales)
    _check_ue8m0(x, kind, round_scale, use_ue8m0, handle, recv_x_scales_ue8m0)
    _want(status, "status", torch.int32, (1,))
    N, S, R, K = x.shape[0], handle.num_src, handle.num_ranks, handle.num_topk
    _want(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (S, R))
    _want(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (S, handle.num_experts))
    _want(topk_idx, "topk_idx", torch.int64, (N, K))
    _want(topk_weights, "topk_weights", torch.float32, (N, K))
    _want(recv_topk_idx, "recv_topk_idx", torch.int64)
    _want(recv_topk_weights, "recv_topk_weights", torch.float32)
    _want(num_recv_tokens_per_expert, "num_recv_tokens_per_expert", torch.int32, (R, handle.num_experts // R))
    for t, name in ((recv_topk_idx, "recv_topk_idx"), (recv_topk_weights, "recv_topk_weights")):
        if t is not None and (t.dim() != 2 or t.shape[0] < handle.recv_capacity or t.shape[1] != K):
            raise ValueError("%s must be [>= %d, %d]" % (name, handle.recv_capacity, K))
    p = handle.problem(x.shape[1], expert_alignment)
    h = handle.c()
    a = _Args()
    a.handle(handle)
    _run(a, "miep_dispatch", ctypes.byref(p), a.p(x), kind, a.p(x_scales), int(round_scale), int(use_ue8m0),
         a.p(topk_idx), a.p(topk_weights), a.p(num_tokens_per_rank), a.p(num_tokens_per_expert), a.p(recv_x),
         a.p(recv_x_scales), a.p(recv_x_scales_ue8m0 if use_ue8m0 else None), a.p(recv_topk_idx),
         a.p(recv_topk_weights), a.p(num_recv_tokens_per_expert), a.p(status), ctypes.byref(h))


def _check_ue8m0(x, kind, round_scale, use_ue8m0, handle: Handle, out):
    if not use_ue8m0:
        return
    if kind != X_BF16_CAST_FP8 or not round_scale:
        raise ValueError("use_ue8m0 needs the FP8 cast (cast_to_fp8=True) with round_scale=True")
    H = x.shape[1]
    if out is None or out.dtype != torch.uint8 or out.dim() != 2 or out.shape[1] != H // 128 or \
            out.shape[0] < handle.recv_capacity:
        raise ValueError("recv_x_scales_ue8m0 must be uint8 [>= %d, %d]" % (handle.recv_capacity, H // 128))


def _check_payload_shapes(x, kind, x_scales, handle: Handle, recv_x, recv_x_scales):
    N, H = x.shape
    if N != handle.send_head.shape[0] or N != handle.num_src * handle.num_tokens:
        raise ValueError("x has %d tokens, the handle %d" % (N, handle.send_head.shape[0]))
    if recv_x.dim() != 2 or recv_x.shape[1] != H or recv_x.shape[0] < handle.recv_capacity:
        raise ValueError("recv_x must be [>= %d, %d]" % (handle.recv_capacity, H))
    if kind == X_BF16:
        _want(recv_x, "recv_x", torch.bfloat16)
    else:
        if recv_x.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError("recv_x must hold E4M3 codes for an FP8 dispatch")
        if recv_x_scales is None or tuple(recv_x_scales.shape[1:]) != (H // 128,) or \
                recv_x_scales.shape[0] < handle.recv_capacity:
            raise ValueError("recv_x_scales must be [>= %d, %d]" % (handle.recv_capacity, H // 128))
        _want(recv_x_scales, "recv_x_scales", torch.float32)
    if kind == X_FP8:
        _want(x_scales, "x_scales", torch.float32, (N, H // 128))
        if x_scales is None:
            raise ValueError("x_scales are required for pre-quantised FP8 x")
    if handle.is_token_in_rank.shape != (N, handle.num_ranks):
        raise ValueError("handle.is_token_in_rank must be [%d, %d]" % (N, handle.num_ranks))


def _recv_buffers(x, kind, cap, dev):
    H = x.shape[1]
    if kind == X_BF16:
        return torch.empty((cap, H), dtype=torch.bfloat16, device=dev), None
    codes = torch.empty((cap, H), dtype=torch.float8_e4m3fn, device=dev)
    return codes, torch.empty((cap, H // 128), dtype=torch.float32, device=dev)


def dispatch(x: torch.Tensor, topk_idx: Optional[torch.Tensor], topk_weights: Optional[torch.Tensor],
             num_tokens_per_rank: torch.Tensor, is_token_in_rank: torch.Tensor,
             num_tokens_per_expert: Optional[torch.Tensor], num_experts: int, num_channels: int = 24,
             expert_alignment: int = 1, num_worst_tokens: int = 0, x_scales: Optional[torch.Tensor] = None,
             cast_to_fp8: bool = False, round_scale: bool = False, use_ue8m0: bool = False,
             check_capacity: bool = True):
    """Normal-mode dispatch (section 4.1, fresh branch).

    Receive buffers are sized exactly from num_tokens_per_rank (one host
    read, the CPU-sync mode) unless ``num_worst_tokens`` > 0 gives a fixed
    capacity; then, with ``check_capacity``, the device status word is read
    back (synchronously) and an overflow raises MiepError(MIEP_ECAPACITY).
    Returns (recv_x, recv_x_scales, recv_topk_idx, recv_topk_weights,
    num_recv_tokens_per_expert [R, E/R], handle), and with ``use_ue8m0``
    (FP8 cast with round_scale) a seventh item, the scales' exponent bytes
    [cap, H/128] uint8.
    """
    kind = _x_kind(x, cast_to_fp8)
    N, H = x.shape
    S, R = num_tokens_per_rank.shape
    _want(is_token_in_rank, "is_token_in_rank", torch.bool, (N, R))
    _want(num_tokens_per_rank, "num_tokens_per_rank", torch.int32)
    _want(topk_idx, "topk_idx", torch.int64)
    _want(topk_weights, "topk_weights", torch.float32)
    K = topk_idx.shape[1] if topk_idx is not None else 1
    cap = int(num_worst_tokens) if num_worst_tokens > 0 else int(num_tokens_per_rank.sum().item())
    dev = x.device
    handle = Handle.allocate(is_token_in_rank, S, K, num_experts, num_channels, cap)
    recv_x, recv_x_scales = _recv_buffers(x, kind, cap, dev)
    recv_topk_idx = torch.empty((cap, K), dtype=torch.int64, device=dev) if topk_idx is not None else None
    recv_topk_weights = torch.empty((cap, K), dtype=torch.float32, device=dev) if topk_weights is not None else None
    nrte = torch.empty((R, num_experts // R), dtype=torch.int32, device=dev) if num_tokens_per_expert is not None \
        else None
    ue = torch.empty((cap, H // 128), dtype=torch.uint8, device=dev) if use_ue8m0 else None
    status = torch.empty((1,), dtype=torch.int32, device=dev) if num_worst_tokens > 0 else None
    dispatch_into(x, topk_idx, topk_weights, num_tokens_per_rank, num_tokens_per_expert, handle, recv_x,
                  recv_x_scales, recv_topk_idx, recv_topk_weights, nrte, x_scales, cast_to_fp8, round_scale,
                  expert_alignment, use_ue8m0, ue, status)
    if status is not None and check_capacity:
        check_status(status)
    out = (recv_x, recv_x_scales, recv_topk_idx, recv_topk_weights, nrte, handle)
    return out + (ue,) if use_ue8m0 else out


def cached_dispatch_into(x, handle: Handle, recv_x, recv_x_scales=None, x_scales=None, cast_to_fp8: bool = False,
                         round_scale: bool = False, use_ue8m0: bool = False, recv_x_scales_ue8m0=None) -> None:
    kind = _x_kind(x, cast_to_fp8)
    _check_payload_shapes(x, kind, x_scales, handle, recv_x, recv_x_scales)
    _check_ue8m0(x, kind, round_scale, use_ue8m0, handle, recv_x_scales_ue8m0)
    p = handle.problem(x.shape[1])
    h = handle.c()
    a = _Args()
    a.handle(handle)
    _run(a, "miep_cached_dispatch", ctypes.byref(p), a.p(x), kind, a.p(x_scales), int(round_scale), int(use_ue8m0),
         ctypes.byref(h), a.p(recv_x), a.p(recv_x_scales), a.p(recv_x_scales_ue8m0 if use_ue8m0 else None))


def cached_dispatch(x: torch.Tensor, handle: Handle, x_scales: Optional[torch.Tensor] = None,
                    cast_to_fp8: bool = False, round_scale: bool = False, use_ue8m0: bool = False):
    """Dispatch a new x along a handle's routing (section 4.1, cached branch): no top-k inputs.
    Returns (recv_x, recv_x_scales), plus the exponent bytes with ``use_ue8m0``."""
    kind = _x_kind(x, cast_to_fp8)
    recv_x, recv_x_scales = _recv_buffers(x, kind, handle.recv_capacity, x.device)
    ue = torch.empty((handle.recv_capacity, x.shape[1] // 128), dtype=torch.uint8, device=x.device) \
        if use_ue8m0 else None
    cached_dispatch_into(x, handle, recv_x, recv_x_scales, x_scales, cast_to_fp8, round_scale, use_ue8m0, ue)
    return (recv_x, recv_x_scales, ue) if use_ue8m0 else (recv_x, recv_x_scales)


# --------------------------------------------------------------------------- combine
def _unpack_bias(bias):
    """``bias`` is None, one [N, H] bf16 tensor, or a pair (bias_0, bias_1) with None allowed in either place."""
    if bias is None:
        return None, None
    if isinstance(bias, torch.Tensor):
        return bias, None
    if isinstance(bias, (tuple, list)) and len(bias) == 2:
        return bias[0], bias[1]
    raise TypeError("bias must be a tensor or a pair of tensors")


def combine_into(y, handle: Handle, combined_x, recv_topk_weights=None, combined_topk_weights=None,
                 bias=None) -> None:
    N, H, K = handle.send_head.shape[0], y.shape[1], handle.num_topk
    _want(y, "y", torch.bfloat16)
    if y.dim() != 2 or y.shape[0] < handle.recv_capacity:
        raise ValueError("y must be [>= %d, H]" % handle.recv_capacity)
    _want(combined_x, "combined_x", torch.bfloat16, (N, H))
    _want(recv_topk_weights, "recv_topk_weights", torch.float32)
    if recv_topk_weights is not None and (recv_topk_weights.dim() != 2 or recv_topk_weights.shape[1] != K or
                                          recv_topk_weights.shape[0] < handle.recv_capacity):
        raise ValueError("recv_topk_weights must be [>= %d, %d]" % (handle.recv_capacity, K))
    _want(combined_topk_weights, "combined_topk_weights", torch.float32, (N, K))
    b0, b1 = _unpack_bias(bias)
    _want(b0, "bias_0", torch.bfloat16, (N, H))
    _want(b1, "bias_1", torch.bfloat16, (N, H))
    p = handle.problem(y.shape[1])
    h = handle.c()
    a = _Args()
    a.handle(handle)
    _run(a, "miep_combine", ctypes.byref(p), a.p(y), a.p(recv_topk_weights), a.p(b0), a.p(b1), ctypes.byref(h),
         a.p(combined_x), a.p(combined_topk_weights))


def combine(y: torch.Tensor, handle: Handle, topk_weights: Optional[torch.Tensor] = None, bias=None):
    """Sum expert outputs back into source-token order (sections 4.2, 4.4).

    y [cap, H] bf16 in the receive layout; ``topk_weights`` are the received
    top-k weights [cap, K], reduced the same way; ``bias`` (one [N, H] bf16
    tensor or a pair) is added to each token's sum after the received rows.
    Returns (combined_x [N, H] bf16, combined_topk_weights [N, K] fp32 or None).
    """
    _want(y, "y", torch.bfloat16)
    if y.shape[0] != handle.recv_capacity:
        raise ValueError("y must have the handle's %d receive rows" % handle.recv_capacity)
    N = handle.send_head.shape[0]
    combined_x = torch.empty((N, y.shape[1]), dtype=torch.bfloat16, device=y.device)
    cw = None
    if topk_weights is not None:
        _want(topk_weights, "topk_weights", torch.float32)
        cw = torch.empty((N, topk_weights.shape[1]), dtype=torch.float32, device=y.device)
        if topk_weights.shape[1] != handle.num_topk:
            raise ValueError("topk_weights must have num_topk columns")
    combine_into(y, handle, combined_x, topk_weights, cw, bias)
    return combined_x, cw


# --------------------------------------------------------------------------- low-latency
def low_latency_dispatch_into(x, topk_idx, num_ranks: int, max_tokens: int, num_experts: int, dest_rank: int,
                              use_fp8: bool, round_scale: bool, use_ue8m0: bool, msg_buf, msg_count, packed_recv_x,
                              packed_recv_x_scales, packed_recv_x_scales_ue8m0, packed_recv_src_info,
                              packed_recv_layout_range, packed_recv_count,
                              cumulative_local_expert_recv_stats=None, mask_buffer=None) -> None:
    N, H = x.shape
    R, M, L, K = num_ranks, max_tokens, num_experts // num_ranks, topk_idx.shape[1]
    if N % R:
        raise ValueError("x rows must split evenly over the source ranks")
    _want(x, "x", torch.bfloat16)
    _want(topk_idx, "topk_idx", torch.int64, (N, K))
    _want(msg_buf, "msg_buf", torch.uint8, (L, R, M, ll_msg_bytes(H, use_fp8)))
    _want(msg_count, "msg_count", torch.int32, (L, R))
    if use_fp8:
        if packed_recv_x.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(packed_recv_x.shape) != (L, R * M, H):
            raise ValueError("packed_recv_x must be [%d, %d, %d] E4M3 codes" % (L, R * M, H))
        _want(packed_recv_x_scales, "packed_recv_x_scales", torch.float32, (L, R * M, H // 128))
        _want(packed_recv_x_scales_ue8m0, "packed_recv_x_scales_ue8m0", torch.uint8, (L, R * M, H // 128))
    else:
        _want(packed_recv_x, "packed_recv_x", torch.bfloat16, (L, R * M, H))
    _want(packed_recv_src_info, "packed_recv_src_info", torch.int32, (L, R * M))
    _want(packed_recv_layout_range, "packed_recv_layout_range", torch.int64, (L, R))
    _want(packed_recv_count, "packed_recv_count", torch.int32, (L,))
    _want(cumulative_local_expert_recv_stats, "cumulative_local_expert_recv_stats", torch.int32, (L,))
    _want(mask_buffer, "mask_buffer", torch.int32, (R,))
    q = _lib.LLProblem(num_ranks, N // num_ranks, max_tokens, H, K, num_experts, dest_rank)
    a = _Args()
    _run(a, "miep_ll_dispatch", ctypes.byref(q), a.p(x), a.p(topk_idx), int(use_fp8), int(round_scale),
         int(use_ue8m0), a.p(msg_buf), a.p(msg_count), a.p(packed_recv_x), a.p(packed_recv_x_scales),
         a.p(packed_recv_x_scales_ue8m0), a.p(packed_recv_src_info), a.p(packed_recv_layout_range),
         a.p(packed_recv_count), a.p(cumulative_local_expert_recv_stats), a.p(mask_buffer))


def low_latency_dispatch_noalloc(x, topk_idx, num_ranks: int, max_tokens: int, num_experts: int, dest_rank: int,
                                 use_fp8: bool, round_scale: bool, use_ue8m0: bool, packed_recv_x,
                                 packed_recv_x_scales, packed_recv_x_scales_ue8m0, packed_recv_src_info,
                                 packed_recv_layout_range, packed_recv_count, cumulative_local_expert_recv_stats=None,
                                 mask_buffer=None) -> None:
    """low_latency_dispatch_into without the message buffer and counts, for callers that cannot allocate:
    the library keeps the counts in a device array of its own (at most 65536 = num_experts, shared by every
    call on the device, so calls on concurrent streams race).  Fills the same packed receive side."""
    N, H = x.shape
    R, M, L, K = num_ranks, max_tokens, num_experts // num_ranks, topk_idx.shape[1]
    if N % R:
        raise ValueError("x rows must split evenly over the source ranks")
    _want(x, "x", torch.bfloat16)
    _want(topk_idx, "topk_idx", torch.int64, (N, K))
    if use_fp8:
        if packed_recv_x.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(packed_recv_x.shape) != (L, R * M, H):
            raise ValueError("packed_recv_x must be [%d, %d, %d] E4M3 codes" % (L, R * M, H))
        _want(packed_recv_x_scales, "packed_recv_x_scales", torch.float32, (L, R * M, H // 128))
        _want(packed_recv_x_scales_ue8m0, "packed_recv_x_scales_ue8m0", torch.uint8, (L, R * M, H // 128))
    else:
        _want(packed_recv_x, "packed_recv_x", torch.bfloat16, (L, R * M, H))
    _want(packed_recv_src_info, "packed_recv_src_info", torch.int32, (L, R * M))
    _want(packed_recv_layout_range, "packed_recv_layout_range", torch.int64, (L, R))
    _want(packed_recv_count, "packed_recv_count", torch.int32, (L,))
    _want(cumulative_local_expert_recv_stats, "cumulative_local_expert_recv_stats", torch.int32, (L,))
    _want(mask_buffer, "mask_buffer", torch.int32, (R,))
    q = _lib.LLProblem(num_ranks, N // num_ranks, max_tokens, H, K, num_experts, dest_rank)
    a = _Args()
    _run(a, "miep_ll_dispatch_noalloc", ctypes.byref(q), a.p(x), a.p(topk_idx), int(use_fp8), int(round_scale),
         int(use_ue8m0), a.p(packed_recv_x), a.p(packed_recv_x_scales), a.p(packed_recv_x_scales_ue8m0),
         a.p(packed_recv_src_info), a.p(packed_recv_layout_range), a.p(packed_recv_count),
         a.p(cumulative_local_expert_recv_stats), a.p(mask_buffer))


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_max_dispatch_tokens_per_rank: int,
                         num_experts: int, dest_rank: int, num_ranks: int, use_fp8: bool = True,
                         round_scale: bool = False, use_ue8m0: bool = False,
                         cumulative_local_expert_recv_stats: Optional[torch.Tensor] = None,
                         mask_buffer: Optional[torch.Tensor] = None) -> dict:
    """Low-latency dispatch received by rank ``dest_rank`` (section 4.3).

    x [R*T, H] bf16 and topk_idx [R*T, K] int64 hold every source rank's
    tokens.  Returns a dict with packed_recv_x [L, R*M, H] (E4M3 or bf16),
    packed_recv_x_scales [L, R*M, H/128], packed_recv_x_scales_ue8m0 (or None),
    packed_recv_src_info [L, R*M], packed_recv_layout_range [L, R] int64,
    packed_recv_count [L], and the expert-major message buffer and counts.
    ``mask_buffer`` [R] int32 (nonzero = masked rank) stops every message from
    or to a masked rank.
    """
    _want(x, "x", torch.bfloat16)
    _want(topk_idx, "topk_idx", torch.int64)
    N, H = x.shape
    R, M = num_ranks, num_max_dispatch_tokens_per_rank
    L = num_experts // R
    dev = x.device
    mb = ll_msg_bytes(H, use_fp8)
    msg_buf = torch.empty((L, R, M, mb), dtype=torch.uint8, device=dev)
    msg_count = torch.empty((L, R), dtype=torch.int32, device=dev)
    if use_fp8:
        prx = torch.empty((L, R * M, H), dtype=torch.float8_e4m3fn, device=dev)
        prs = torch.empty((L, R * M, H // 128), dtype=torch.float32, device=dev)
        pue = torch.empty((L, R * M, H // 128), dtype=torch.uint8, device=dev) if use_ue8m0 else None
    else:
        prx = torch.empty((L, R * M, H), dtype=torch.bfloat16, device=dev)
        prs = pue = None
    src = torch.empty((L, R * M), dtype=torch.int32, device=dev)
    lr = torch.empty((L, R), dtype=torch.int64, device=dev)
    cnt = torch.empty((L,), dtype=torch.int32, device=dev)
    low_latency_dispatch_into(x, topk_idx, R, M, num_experts, dest_rank, use_fp8, round_scale, use_ue8m0, msg_buf,
                              msg_count, prx, prs, pue, src, lr, cnt, cumulative_local_expert_recv_stats, mask_buffer)
    return dict(packed_recv_x=prx, packed_recv_x_scales=prs, packed_recv_x_scales_ue8m0=pue,
                packed_recv_src_info=src, packed_recv_layout_range=lr, packed_recv_count=cnt, msg_buf=msg_buf,
                msg_count=msg_count, cumulative_local_expert_recv_stats=cumulative_local_expert_recv_stats)


def low_latency_combine_into(y, topk_idx, topk_weights, packed_recv_src_info, packed_recv_layout_range,
                             num_ranks: int, max_tokens: int, num_experts: int, dest_rank: int, combined_x) -> None:
    R, M = num_ranks, max_tokens
    L = num_experts // R if R > 0 else 0
    _want(topk_idx, "topk_idx", torch.int64)
    if topk_idx.dim() != 2 or R <= 0 or topk_idx.shape[0] % R:
        raise ValueError("topk_idx must be [R*T, K]")
    N, K = topk_idx.shape
    _want(y, "y", torch.bfloat16)
    if y.dim() != 3 or tuple(y.shape[:2]) != (L, R * M):
        raise ValueError("y must be [%d, %d, H]" % (L, R * M))
    H = y.shape[2]
    _want(topk_weights, "topk_weights", torch.float32, (N, K))
    _want(packed_recv_src_info, "packed_recv_src_info", torch.int32, (L, R * M))
    _want(packed_recv_layout_range, "packed_recv_layout_range", torch.int64, (L, R))
    _want(combined_x, "combined_x", torch.bfloat16, (N, H))
    q = _lib.LLProblem(R, N // R, M, H, K, num_experts, dest_rank)
    a = _Args()
    _run(a, "miep_ll_combine", ctypes.byref(q), a.p(y), a.p(packed_recv_src_info), a.p(packed_recv_layout_range),
         a.p(topk_idx), a.p(topk_weights), a.p(combined_x))


def low_latency_combine(y: torch.Tensor, topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                        packed_recv_src_info: torch.Tensor, packed_recv_layout_range: torch.Tensor,
                        num_max_dispatch_tokens_per_rank: int, num_experts: int, dest_rank: int,
                        num_ranks: int) -> torch.Tensor:
    """Low-latency combine: rank ``dest_rank``'s expert outputs back to token order (section 4.3).

    y [L, R*M, H] bf16 in the packed layout of ``low_latency_dispatch``;
    topk_idx [R*T, K] is the routing that dispatch was given and
    packed_recv_src_info / packed_recv_layout_range are its outputs.  Each
    token sums, in ascending k, the rows its entries on d's experts were sent
    to, times the entry's weight when ``topk_weights`` is given.  Returns
    combined_x [R*T, H] bf16 (zero for tokens without a row on rank d).
    """
    _want(y, "y", torch.bfloat16)
    combined_x = torch.empty((topk_idx.shape[0], y.shape[-1]), dtype=torch.bfloat16, device=y.device)
    low_latency_combine_into(y, topk_idx, topk_weights, packed_recv_src_info, packed_recv_layout_range, num_ranks,
                             num_max_dispatch_tokens_per_rank, num_experts, dest_rank, combined_x)
    return combined_x


# --------------------------------------------------------------------------- rank mask
def _mask_check(mask_buffer):
    _want(mask_buffer, "mask_buffer", torch.int32)
    if mask_buffer.dim() != 1:
        raise ValueError("mask_buffer must be [num_ranks] int32")


def update_mask_buffer(mask_buffer: torch.Tensor, rank: int, mask: bool) -> None:
    """Set (mask=True) or clear rank ``rank``'s entry of the [R] int32 mask."""
    _mask_check(mask_buffer)
    a = _Args()
    _run(a, "miep_mask_update", a.p(mask_buffer), mask_buffer.shape[0], int(rank), int(bool(mask)))


def clean_mask_buffer(mask_buffer: torch.Tensor) -> None:
    """Clear every entry of the [R] int32 mask."""
    _mask_check(mask_buffer)
    a = _Args()
    _run(a, "miep_mask_clean", a.p(mask_buffer), mask_buffer.shape[0])


def query_mask_buffer(mask_buffer: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Copy the [R] int32 mask into ``out`` (allocated when None) and return it."""
    _mask_check(mask_buffer)
    if out is None:
        out = torch.empty_like(mask_buffer)
    _want(out, "out", torch.int32, tuple(mask_buffer.shape))
    a = _Args()
    _run(a, "miep_mask_query", a.p(mask_buffer), mask_buffer.shape[0], a.p(out))
    return out


# --------------------------------------------------------------------------- two-level relay
@dataclass
class RelayHandle:
    """The group rows of a relay dispatch (groups of 8 ranks standing for the nodes).

    rdma_rank_prefix_matrix [S,G], rdma_channel_prefix_matrix [S,G,C],
    recv_rdma_channel_prefix_matrix [G,S,C], recv_rdma_offset [G+1] (last =
    total group rows), send_rdma_head [N,G], rdma_src_idx [rcap] (source token
    of each group row), send_nvl_head [rcap, 8] (its row in each of the group's
    ranks, or -1).
    """
    rdma_rank_prefix_matrix: torch.Tensor
    rdma_channel_prefix_matrix: torch.Tensor
    recv_rdma_channel_prefix_matrix: torch.Tensor
    recv_rdma_offset: torch.Tensor
    send_rdma_head: torch.Tensor
    rdma_src_idx: torch.Tensor
    send_nvl_head: torch.Tensor

    @property
    def rdma_capacity(self) -> int:
        return self.rdma_src_idx.numel()

    @staticmethod
    def allocate(num_tokens: int, num_src: int, num_ranks: int, num_channels: int, rdma_capacity: int,
                 device) -> "RelayHandle":
        G = num_ranks // 8
        i32 = dict(dtype=torch.int32, device=device)
        return RelayHandle(torch.empty((num_src, G), **i32), torch.empty((num_src, G, num_channels), **i32),
                           torch.empty((G, num_src, num_channels), **i32), torch.empty((G + 1,), **i32),
                           torch.empty((num_tokens, G), **i32), torch.empty((rdma_capacity,), **i32),
                           torch.empty((rdma_capacity, 8), **i32))

    def tensors(self):
        return (self.rdma_rank_prefix_matrix, self.rdma_channel_prefix_matrix, self.recv_rdma_channel_prefix_matrix,
                self.recv_rdma_offset, self.send_rdma_head, self.rdma_src_idx, self.send_nvl_head)

    def c(self) -> _lib.RelayHandleC:
        return _lib.RelayHandleC(self.rdma_rank_prefix_matrix.data_ptr(), self.rdma_channel_prefix_matrix.data_ptr(),
                                 self.recv_rdma_channel_prefix_matrix.data_ptr(), self.recv_rdma_offset.data_ptr(),
                                 self.send_rdma_head.data_ptr(), self.rdma_src_idx.data_ptr(),
                                 self.send_nvl_head.data_ptr(), self.rdma_capacity)


def relay_dispatch_into(x, topk_idx, topk_weights, num_tokens_per_rank, num_tokens_per_rdma_rank,
                        num_tokens_per_expert, handle: Handle, relay: RelayHandle, rdma_x, recv_x,
                        rdma_x_scales=None, recv_x_scales=None, recv_topk_idx=None, recv_topk_weights=None,
                        num_recv_tokens_per_expert=None, x_scales=None, cast_to_fp8: bool = False,
                        round_scale: bool = False, expert_alignment: int = 1, status=None) -> None:
    """Relay dispatch into preallocated outputs (allocates nothing).  ``status`` ([1] int32, optional) receives
    0 or MIEP_ECAPACITY (group rows or receive rows past their capacity)."""
    kind = _x_kind(x, cast_to_fp8)
    _check_payload_shapes(x, kind, x_scales, handle, recv_x, recv_x_scales)
    N, H = x.shape
    S, R, K = handle.num_src, handle.num_ranks, handle.num_topk
    G = R // 8
    if R % 8 or R <= 8:
        raise ValueError("the relay needs num_ranks > 8 and a multiple of 8")
    _want(num_tokens_per_rank, "num_tokens_per_rank", torch.int32, (S, R))
    _want(num_tokens_per_rdma_rank, "num_tokens_per_rdma_rank", torch.int32, (S, G))
    _want(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, (S, handle.num_experts))
    _want(topk_idx, "topk_idx", torch.int64, (N, K))
    _want(topk_weights, "topk_weights", torch.float32, (N, K))
    _want(num_recv_tokens_per_expert, "num_recv_tokens_per_expert", torch.int32, (R, handle.num_experts // R))
    for t, name in ((recv_topk_idx, "recv_topk_idx"), (recv_topk_weights, "recv_topk_weights")):
        if t is not None and (t.dim() != 2 or t.shape[0] < handle.recv_capacity or t.shape[1] != K):
            raise ValueError("%s must be [>= %d, %d]" % (name, handle.recv_capacity, K))
    _want(recv_topk_idx, "recv_topk_idx", torch.int64)
    _want(recv_topk_weights, "recv_topk_weights", torch.float32)
    rc = relay.rdma_capacity
    if rdma_x.dim() != 2 or rdma_x.shape[0] < rc or rdma_x.shape[1] != H:
        raise ValueError("rdma_x must be [>= %d, %d]" % (rc, H))
    if kind == X_BF16:
        _want(rdma_x, "rdma_x", torch.bfloat16)
    else:
        if rdma_x.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError("rdma_x must hold E4M3 codes for an FP8 dispatch")
        if rdma_x_scales is None or rdma_x_scales.dim() != 2 or rdma_x_scales.shape[0] < rc or \
                rdma_x_scales.shape[1] != H // 128:
            raise ValueError("rdma_x_scales must be [>= %d, %d]" % (rc, H // 128))
        _want(rdma_x_scales, "rdma_x_scales", torch.float32)
    if relay.send_rdma_head.shape != (N, G):
        raise ValueError("relay.send_rdma_head must be [%d, %d]" % (N, G))
    _want(status, "status", torch.int32, (1,))
    p = handle.problem(H, expert_alignment)
    h = handle.c()
    rh = relay.c()
    a = _Args()
    a.handle(handle)
    a.handle(relay)
    _run(a, "miep_relay_dispatch", ctypes.byref(p), a.p(x), kind, a.p(x_scales), int(round_scale), a.p(topk_idx),
         a.p(topk_weights), a.p(num_tokens_per_rank), a.p(num_tokens_per_rdma_rank), a.p(num_tokens_per_expert),
         a.p(rdma_x), a.p(rdma_x_scales), a.p(recv_x), a.p(recv_x_scales), a.p(recv_topk_idx), a.p(recv_topk_weights),
         a.p(num_recv_tokens_per_expert), a.p(status), ctypes.byref(h), ctypes.byref(rh))


def relay_dispatch(x: torch.Tensor, topk_idx: Optional[torch.Tensor], topk_weights: Optional[torch.Tensor],
                   num_tokens_per_rank: torch.Tensor, num_tokens_per_rdma_rank: torch.Tensor,
                   is_token_in_rank: torch.Tensor, num_tokens_per_expert: Optional[torch.Tensor], num_experts: int,
                   num_channels: int = 24, expert_alignment: int = 1, x_scales: Optional[torch.Tensor] = None,
                   cast_to_fp8: bool = False, round_scale: bool = False):
    """Dispatch through the two-level relay: each token once per destination group of 8 ranks (the FP8 cast,
    if any, happens once before this hop), then forwarded to the group's receiving ranks.

    The receive side equals ``dispatch``'s.  Buffers are sized exactly (one host read of the rank and group
    counts).  Returns (recv_x, recv_x_scales, recv_topk_idx, recv_topk_weights, num_recv_tokens_per_expert,
    handle, relay_handle, rdma_x, rdma_x_scales).
    """
    kind = _x_kind(x, cast_to_fp8)
    N, H = x.shape
    S, R = num_tokens_per_rank.shape
    _want(is_token_in_rank, "is_token_in_rank", torch.bool, (N, R))
    _want(num_tokens_per_rank, "num_tokens_per_rank", torch.int32)
    _want(num_tokens_per_rdma_rank, "num_tokens_per_rdma_rank", torch.int32)
    _want(topk_idx, "topk_idx", torch.int64)
    _want(topk_weights, "topk_weights", torch.float32)
    K = topk_idx.shape[1] if topk_idx is not None else 1
    cap = int(num_tokens_per_rank.sum().item())
    rcap = int(num_tokens_per_rdma_rank.sum().item())
    dev = x.device
    handle = Handle.allocate(is_token_in_rank, S, K, num_experts, num_channels, cap)
    relay = RelayHandle.allocate(N, S, R, num_channels, rcap, dev)
    recv_x, recv_x_scales = _recv_buffers(x, kind, cap, dev)
    rdma_x, rdma_x_scales = _recv_buffers(x, kind, rcap, dev)
    recv_topk_idx = torch.empty((cap, K), dtype=torch.int64, device=dev) if topk_idx is not None else None
    recv_topk_weights = torch.empty((cap, K), dtype=torch.float32, device=dev) if topk_weights is not None else None
    nrte = torch.empty((R, num_experts // R), dtype=torch.int32, device=dev) if num_tokens_per_expert is not None \
        else None
    relay_dispatch_into(x, topk_idx, topk_weights, num_tokens_per_rank, num_tokens_per_rdma_rank,
                        num_tokens_per_expert, handle, relay, rdma_x, recv_x, rdma_x_scales, recv_x_scales,
                        recv_topk_idx, recv_topk_weights, nrte, x_scales, cast_to_fp8, round_scale, expert_alignment)
    return recv_x, recv_x_scales, recv_topk_idx, recv_topk_weights, nrte, handle, relay, rdma_x, rdma_x_scales


def relay_cached_dispatch_into(x, handle: Handle, relay: RelayHandle, rdma_x, recv_x, rdma_x_scales=None,
                               recv_x_scales=None, x_scales=None, cast_to_fp8: bool = False,
                               round_scale: bool = False) -> None:
    """Cached dispatch through the relay into preallocated buffers (allocates nothing)."""
    kind = _x_kind(x, cast_to_fp8)
    _check_payload_shapes(x, kind, x_scales, handle, recv_x, recv_x_scales)
    H = x.shape[1]
    rc = relay.rdma_capacity
    if rdma_x.dim() != 2 or rdma_x.shape[0] < rc or rdma_x.shape[1] != H:
        raise ValueError("rdma_x must be [>= %d, %d]" % (rc, H))
    if kind != X_BF16 and (rdma_x_scales is None or rdma_x_scales.shape[0] < rc):
        raise ValueError("rdma_x_scales must be [>= %d, %d]" % (rc, H // 128))
    p = handle.problem(H)
    h = handle.c()
    rh = relay.c()
    a = _Args()
    a.handle(handle)
    a.handle(relay)
    _run(a, "miep_relay_cached_dispatch", ctypes.byref(p), a.p(x), kind, a.p(x_scales), int(round_scale),
         ctypes.byref(h), ctypes.byref(rh), a.p(rdma_x), a.p(rdma_x_scales), a.p(recv_x), a.p(recv_x_scales))


def relay_cached_dispatch(x: torch.Tensor, handle: Handle, relay: RelayHandle, x_scales: Optional[torch.Tensor] = None,
                          cast_to_fp8: bool = False, round_scale: bool = False):
    """Dispatch a new x along the handles of an earlier relay dispatch (no top-k inputs).
    Returns (recv_x, recv_x_scales)."""
    kind = _x_kind(x, cast_to_fp8)
    recv_x, recv_x_scales = _recv_buffers(x, kind, handle.recv_capacity, x.device)
    rdma_x, rdma_x_scales = _recv_buffers(x, kind, relay.rdma_capacity, x.device)
    relay_cached_dispatch_into(x, handle, relay, rdma_x, recv_x, rdma_x_scales, recv_x_scales, x_scales, cast_to_fp8,
                               round_scale)
    return recv_x, recv_x_scales


def relay_combine_into(y, handle: Handle, relay: RelayHandle, rdma_y, combined_x, recv_topk_weights=None,
                       rdma_w=None, combined_topk_weights=None, bias=None) -> None:
    """Two-level combine into preallocated buffers (allocates nothing).  The partials' type follows rdma_y:
    bfloat16 (rounded between the levels) or float32 (kept unrounded)."""
    N, H, K = handle.send_head.shape[0], y.shape[1], handle.num_topk
    _want(y, "y", torch.bfloat16)
    if y.dim() != 2 or y.shape[0] < handle.recv_capacity:
        raise ValueError("y must be [>= %d, H]" % handle.recv_capacity)
    if rdma_y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("rdma_y must be bfloat16 or float32, got %s" % rdma_y.dtype)
    partial_f32 = rdma_y.dtype == torch.float32
    if rdma_y.dim() != 2 or rdma_y.shape[0] < relay.rdma_capacity or rdma_y.shape[1] != H:
        raise ValueError("rdma_y must be [>= %d, %d]" % (relay.rdma_capacity, H))
    _want(combined_x, "combined_x", torch.bfloat16, (N, H))
    _want(recv_topk_weights, "recv_topk_weights", torch.float32)
    if recv_topk_weights is not None:
        if recv_topk_weights.dim() != 2 or recv_topk_weights.shape[1] != K or \
                recv_topk_weights.shape[0] < handle.recv_capacity:
            raise ValueError("recv_topk_weights must be [>= %d, %d]" % (handle.recv_capacity, K))
        if rdma_w is None or rdma_w.dim() != 2 or rdma_w.shape[0] < relay.rdma_capacity or rdma_w.shape[1] != K:
            raise ValueError("rdma_w must be [>= %d, %d] when weights are combined" % (relay.rdma_capacity, K))
    _want(rdma_w, "rdma_w", torch.float32)
    _want(combined_topk_weights, "combined_topk_weights", torch.float32, (N, K))
    b0, b1 = _unpack_bias(bias)
    _want(b0, "bias_0", torch.bfloat16, (N, H))
    _want(b1, "bias_1", torch.bfloat16, (N, H))
    p = handle.problem(H)
    h = handle.c()
    rh = relay.c()
    a = _Args()
    a.handle(handle)
    a.handle(relay)
    _run(a, "miep_relay_combine", ctypes.byref(p), a.p(y), a.p(recv_topk_weights), a.p(b0), a.p(b1), ctypes.byref(h),
         ctypes.byref(rh), int(partial_f32), a.p(rdma_y), a.p(rdma_w), a.p(combined_x), a.p(combined_topk_weights))


def relay_combine(y: torch.Tensor, handle: Handle, relay: RelayHandle, topk_weights: Optional[torch.Tensor] = None,
                  bias=None, partial_f32: bool = False):
    """Two-level combine: each group row sums its group's ranks (rounded to bf16, the partial's travel type,
    or kept fp32 with ``partial_f32``), then each token sums its groups' partials and the bias.  Returns
    (combined_x [N, H] bf16, combined_topk_weights [N, K] fp32 or None)."""
    _want(y, "y", torch.bfloat16)
    N, H = handle.send_head.shape[0], y.shape[1]
    dev = y.device
    rdma_y = torch.empty((relay.rdma_capacity, H), dtype=torch.float32 if partial_f32 else torch.bfloat16,
                         device=dev)
    combined_x = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    rdma_w = cw = None
    if topk_weights is not None:
        K = topk_weights.shape[1]
        rdma_w = torch.empty((relay.rdma_capacity, K), dtype=torch.float32, device=dev)
        cw = torch.empty((N, K), dtype=torch.float32, device=dev)
    relay_combine_into(y, handle, relay, rdma_y, combined_x, topk_weights, rdma_w, cw, bias)
    return combined_x, cw
