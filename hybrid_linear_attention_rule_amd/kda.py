"""Python binding of libkda.so (ctypes): argument marshalling only.

Every step of the mixer runs in the HIP library; this module turns torch
tensors into device pointers and the current HIP stream, and raises when the
library returns an error code.  PyTorch supplies device memory and streams.
The binding never falls back to another implementation: if libkda.so is
missing it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
GATE_SIGMOID, GATE_SILU = 0, 1
GATES_VALUES, GATES_LOGITS = 0, 1
STATUS_BAD_SLOT = 1
STATUS_BAD_POSITION = 2
STATUS_BAD_ACCEPTED = 4
STATUS_BAD_SEQLENS = 8
STATUS_STALLED = 16
ERR_TOO_LARGE = -7
PREFILL_SCRATCH_BYTES = 128 << 20      # KDA_PREFILL_SCRATCH_BYTES in kda.h

_DT = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.float8_e4m3fn}


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_k", ctypes.c_int32),
                ("head_v", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("q_scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("gate_inputs", ctypes.c_int32), ("qkv_row_stride", ctypes.c_int32),
                ("g_row_stride", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("conv_w_q", ctypes.c_void_p), ("conv_w_k", ctypes.c_void_p),
                ("conv_w_v", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("qkv_scale", ctypes.c_float * 3)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SP = ctypes.POINTER(_Shape)
_PP = ctypes.POINTER(_Params)

# exported symbol -> (restype, argtypes); the header declares exactly these
SIGNATURES = {
    "kda_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_state_bytes": (_sz, [_SP, _i64]),
    "kda_conv_bytes": (_sz, [_SP, _i64]),
    "kda_draft_state_bytes": (_sz, [_SP, _i32, _i32]),
    "kda_draft_conv_bytes": (_sz, [_SP, _i32, _i32]),
    "kda_prefill_workspace_bytes": (_sz, [_SP, _i32, _i64]),
    "kda_state_write": (ctypes.c_int, [_SP, _vp, _i64, _vp, _i32, _vp, _vp, _vp]),
    "kda_state_read": (ctypes.c_int, [_SP, _vp, _i64, _vp, _i32, _vp, _vp, _vp]),
    "kda_conv_write": (ctypes.c_int, [_SP, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _vp]),
    "kda_conv_read": (ctypes.c_int, [_SP, _vp, _i64, _vp, _vp, _i32, _vp, _vp, _vp]),
    "kda_decode": (ctypes.c_int, [_SP, _PP, _i32, _i64, _vp, _vp] + [_vp] * 6 +
                   [_vp, _vp, _vp, _vp, _vp]),
    "kda_verify": (ctypes.c_int, [_SP, _PP, _i32, _i32, _i64, _vp, _vp] + [_vp] * 6 +
                   [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_commit_accepted": (ctypes.c_int, [_SP, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp]),
    "kda_commit_recompute": (ctypes.c_int, [_SP, _PP, _i32, _i32, _i64, _vp, _vp, _vp] +
                             [_vp] * 6 + [_vp, _vp, _vp, _vp]),
    "kda_prefill": (ctypes.c_int, [_SP, _PP, _i32, _vp, _i64, _i32, _i64, _vp, _vp] +
                    [_vp] * 6 + [_vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "kda_prefill_noalloc": (ctypes.c_int, [_SP, _PP, _i32, _vp, _i64, _i32, _i64, _vp, _vp] +
                            [_vp] * 6 + [_vp, _vp, _vp, _vp, _vp]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libkda.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with __graft_entry__.build() or "
                "python hybrid_linear_attention_rule_amd/build_lib.py")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        raise KdaError(rc, load().kda_status_str(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, numel, dtype, name):
    """Host-side guard: a tensor the kernels will index must be a contiguous
    device tensor of exactly the size and dtype the call implies."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _expect_rows(t, lead, H, d, dtype, rs, name):
    """A [.., H, d] device tensor whose `lead` token rows start rs elements
    apart (rs = 0: contiguous, H*d), as the kernels index it."""
    if rs == 0:
        return _expect(t, lead * H * d, dtype, name)
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dtype != dtype or t.dim() < 3 or tuple(t.shape[-2:]) != (H, d):
        raise ValueError(f"{name}: expected a {dtype} device tensor [.., {H}, {d}]")
    want, step = [], rs
    for n in reversed(t.shape[:-2]):
        want.append(step)
        step *= n
    if (t.stride(-1), t.stride(-2)) != (1, d) or tuple(t.stride()[:-2]) != tuple(reversed(want)) \
            or t.numel() != lead * H * d:
        raise ValueError(f"{name}: token rows must be {rs} elements apart, heads {d}, "
                         f"channels contiguous (strides {tuple(t.stride())})")


def _check_tokens(shape, lead, q, k, v, alpha, beta, g):
    H, dk, dv, a = shape.num_heads, shape.head_k, shape.head_v, shape.act_dtype
    ga = shape.gate_dtype
    _expect_rows(q, lead, H, dk, a, shape.qkv_row_stride, "q")
    _expect_rows(k, lead, H, dk, a, shape.qkv_row_stride, "k")
    _expect_rows(v, lead, H, dv, a, shape.qkv_row_stride, "v")
    _expect(alpha, lead * H * dk, ga, "alpha")
    _expect(beta, lead * H, ga, "beta")
    _expect_rows(g, lead, H, dv, ga, shape.g_row_stride, "g")


def _check_pool_ring(shape, pool, ring):
    H, dk, dv = shape.num_heads, shape.head_k, shape.head_v
    n = pool.shape[0]
    _expect(pool, n * H * dk * dv, shape.state_dtype, "pool")
    _expect(ring, n * shape.conv_width * H * shape.channels, shape.act_dtype, "ring")


def _check_params(shape, params):
    H, dk, dv, W = shape.num_heads, shape.head_k, shape.head_v, shape.conv_width
    _expect(params.conv_w_q, H * dk * W, torch.float32, "conv_w_q")
    _expect(params.conv_w_k, H * dk * W, torch.float32, "conv_w_k")
    _expect(params.conv_w_v, H * dv * W, torch.float32, "conv_w_v")
    if params.norm_w is not None:
        _expect(params.norm_w, dv, torch.float32, "norm_w")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class KdaShape:
    num_heads: int
    head_k: int
    head_v: int
    act: str = "bf16"
    state: str = "f32"
    gate: int = GATE_SIGMOID
    q_scale: float = 1.0
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6
    conv_width: int = 4
    gate_inputs: int = GATES_VALUES
    qkv_row_stride: int = 0   # elements between token rows of q, k, v; 0 = contiguous
    g_row_stride: int = 0     # the same for g

    def c(self) -> _Shape:
        return _Shape(self.num_heads, self.head_k, self.head_v, self.conv_width,
                      _DT[self.act], _DT[self.state], self.gate, self.q_scale,
                      self.l2_eps, self.norm_eps, self.gate_inputs, self.qkv_row_stride,
                      self.g_row_stride)

    @property
    def channels(self) -> int:
        return 2 * self.head_k + self.head_v

    @property
    def act_dtype(self) -> torch.dtype:
        """dtype of q, k, v, the ring and the raw drafts"""
        return _TORCH_DT[_DT[self.act]]

    @property
    def gate_dtype(self) -> torch.dtype:
        """dtype of alpha, beta and g (BF16 when the activations are FP8)"""
        return torch.bfloat16 if self.act == "fp8" else self.act_dtype

    @property
    def state_dtype(self) -> torch.dtype:
        return _TORCH_DT[_DT[self.state]]


@dataclass
class KdaParams:
    conv_w_q: torch.Tensor  # [H*dk, 4] fp32
    conv_w_k: torch.Tensor  # [H*dk, 4] fp32
    conv_w_v: torch.Tensor  # [H*dv, 4] fp32
    norm_w: torch.Tensor | None = None  # [dv] fp32
    qkv_scale: tuple = (1.0, 1.0, 1.0)  # FP8 activations: dequantisation scales

    def c(self) -> _Params:
        return _Params(self.conv_w_q.data_ptr(), self.conv_w_k.data_ptr(),
                       self.conv_w_v.data_ptr(),
                       None if self.norm_w is None else self.norm_w.data_ptr(),
                       (ctypes.c_float * 3)(*self.qkv_scale))


# ------------------------------------------------------------------ sizes

def state_bytes(shape: KdaShape, num_slots: int) -> int:
    return load().kda_state_bytes(ctypes.byref(shape.c()), num_slots)


def conv_bytes(shape: KdaShape, num_slots: int) -> int:
    return load().kda_conv_bytes(ctypes.byref(shape.c()), num_slots)


def draft_state_bytes(shape: KdaShape, batch: int, n: int) -> int:
    return load().kda_draft_state_bytes(ctypes.byref(shape.c()), batch, n)


def draft_conv_bytes(shape: KdaShape, batch: int, n: int) -> int:
    return load().kda_draft_conv_bytes(ctypes.byref(shape.c()), batch, n)


def prefill_workspace_bytes(shape: KdaShape, num_seqs: int, total_tokens: int) -> int:
    return load().kda_prefill_workspace_bytes(ctypes.byref(shape.c()), num_seqs,
                                              total_tokens)


# ------------------------------------------------------- device buffers

def alloc_pool(shape: KdaShape, num_slots: int, device="cuda") -> torch.Tensor:
    """State pool [num_slots, H, dk, dv] in the storage dtype."""
    return torch.zeros((num_slots, shape.num_heads, shape.head_k, shape.head_v),
                       dtype=shape.state_dtype, device=device)


def alloc_ring(shape: KdaShape, num_slots: int, device="cuda") -> torch.Tensor:
    """Conv ring [num_slots, 4, H, 2dk+dv] in the activation dtype."""
    return torch.zeros((num_slots, shape.conv_width, shape.num_heads, shape.channels),
                       dtype=shape.act_dtype, device=device)


# -------------------------------------------------------------- calls

def state_write(shape, pool, slot_ids, src, status=None, stream=None):
    _expect(pool, pool.numel(), shape.state_dtype, "pool")
    _expect(slot_ids, slot_ids.numel(), torch.int32, "slot_ids")
    _expect(src, slot_ids.numel() * shape.num_heads * shape.head_k * shape.head_v,
            torch.float32, "src")
    _check(load().kda_state_write(ctypes.byref(shape.c()), _ptr(pool), pool.shape[0],
                                  _ptr(slot_ids), slot_ids.numel(), _ptr(src),
                                  _ptr(status), _stream(stream)))


def state_read(shape, pool, slot_ids, dst, status=None, stream=None):
    _expect(pool, pool.numel(), shape.state_dtype, "pool")
    _expect(slot_ids, slot_ids.numel(), torch.int32, "slot_ids")
    _expect(dst, slot_ids.numel() * shape.num_heads * shape.head_k * shape.head_v,
            torch.float32, "dst")
    _check(load().kda_state_read(ctypes.byref(shape.c()), _ptr(pool), pool.shape[0],
                                 _ptr(slot_ids), slot_ids.numel(), _ptr(dst),
                                 _ptr(status), _stream(stream)))


def conv_write(shape, ring, slot_ids, positions, window, status=None, stream=None):
    _conv_io_checks(shape, ring, slot_ids, positions, window)
    _check(load().kda_conv_write(ctypes.byref(shape.c()), _ptr(ring), ring.shape[0],
                                 _ptr(slot_ids), _ptr(positions), slot_ids.numel(),
                                 _ptr(window), _ptr(status), _stream(stream)))


def _conv_io_checks(shape, ring, slot_ids, positions, window):
    n = slot_ids.numel()
    _expect(ring, ring.numel(), shape.act_dtype, "ring")
    _expect(slot_ids, n, torch.int32, "slot_ids")
    _expect(positions, n, torch.int32, "positions")
    _expect(window, n * (shape.conv_width - 1) * shape.num_heads * shape.channels,
            shape.act_dtype, "window")


def conv_read(shape, ring, slot_ids, positions, window, status=None, stream=None):
    _conv_io_checks(shape, ring, slot_ids, positions, window)
    _check(load().kda_conv_read(ctypes.byref(shape.c()), _ptr(ring), ring.shape[0],
                                _ptr(slot_ids), _ptr(positions), slot_ids.numel(),
                                _ptr(window), _ptr(status), _stream(stream)))


def decode(shape, params, slot_ids, positions, q, k, v, alpha, beta, g, pool, ring,
           y, status=None, stream=None):
    B = slot_ids.numel()
    _check_params(shape, params)
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _check_tokens(shape, B, q, k, v, alpha, beta, g)
    _check_pool_ring(shape, pool, ring)
    _expect(y, B * shape.num_heads * shape.head_v, torch.float32, "y")
    _check(load().kda_decode(ctypes.byref(shape.c()), ctypes.byref(params.c()),
                             slot_ids.numel(), pool.shape[0], _ptr(slot_ids),
                             _ptr(positions), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(g), _ptr(pool), _ptr(ring), _ptr(y),
                             _ptr(status), _stream(stream)))


def verify(shape, params, slot_ids, positions, q, k, v, alpha, beta, g, pool, ring,
           draft_states, draft_conv, y, status=None, stream=None):
    B = slot_ids.numel()
    n = q.shape[1]
    H, dk, dv = shape.num_heads, shape.head_k, shape.head_v
    _check_params(shape, params)
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _check_tokens(shape, B * n, q, k, v, alpha, beta, g)
    _check_pool_ring(shape, pool, ring)
    # draft_states / draft_conv may be None: no records / raw drafts kept
    if draft_states is not None:
        _expect(draft_states, B * n * H * dv * dk, torch.float32, "draft_states")
    if draft_conv is not None:
        _expect(draft_conv, B * n * H * shape.channels, shape.act_dtype, "draft_conv")
    _expect(y, B * n * H * dv, torch.float32, "y")
    _check(load().kda_verify(ctypes.byref(shape.c()), ctypes.byref(params.c()),
                             slot_ids.numel(), n, pool.shape[0], _ptr(slot_ids),
                             _ptr(positions), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(g), _ptr(pool), _ptr(ring),
                             _ptr(draft_states), _ptr(draft_conv), _ptr(y),
                             _ptr(status), _stream(stream)))


def commit_accepted(shape, slot_ids, positions, accepted, draft_states, draft_conv,
                    pool, ring, status=None, stream=None):
    B = slot_ids.numel()
    n = draft_states.shape[1]
    H, dk, dv = shape.num_heads, shape.head_k, shape.head_v
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _expect(accepted, B, torch.int32, "accepted")
    _expect(draft_states, B * n * H * dv * dk, torch.float32, "draft_states")
    _expect(draft_conv, B * n * H * shape.channels, shape.act_dtype, "draft_conv")
    _check_pool_ring(shape, pool, ring)
    _check(load().kda_commit_accepted(ctypes.byref(shape.c()), slot_ids.numel(), n,
                                      pool.shape[0], _ptr(slot_ids), _ptr(positions),
                                      _ptr(accepted), _ptr(draft_states),
                                      _ptr(draft_conv), _ptr(pool), _ptr(ring),
                                      _ptr(status), _stream(stream)))


def commit_recompute(shape, params, slot_ids, positions, accepted, q, k, v, alpha, beta, g,
                     pool, ring, status=None, stream=None):
    """Commit accepted[b] of the verify's n draft tokens by running them
    again from the stored state (q, k, v, alpha, beta, g: the verify's inputs,
    [B, n, H, .])."""
    B = slot_ids.numel()
    n = q.shape[1]
    _check_params(shape, params)
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _expect(accepted, B, torch.int32, "accepted")
    _check_tokens(shape, B * n, q, k, v, alpha, beta, g)
    _check_pool_ring(shape, pool, ring)
    _check(load().kda_commit_recompute(ctypes.byref(shape.c()), ctypes.byref(params.c()),
                                       B, n, pool.shape[0], _ptr(slot_ids), _ptr(positions),
                                       _ptr(accepted), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(g), _ptr(pool),
                                       _ptr(ring), _ptr(status), _stream(stream)))


def prefill(shape, params, cu_seqlens, max_seqlen, slot_ids, positions, q, k, v,
            alpha, beta, g, pool, ring, y, workspace, status=None, stream=None):
    """Chunked prefill of the packed sequences cu_seqlens describes.
    workspace: a device tensor of at least prefill_workspace_bytes() bytes."""
    B = slot_ids.numel()
    T = q.shape[0]
    _check_params(shape, params)
    _expect(cu_seqlens, B + 1, torch.int32, "cu_seqlens")
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _check_tokens(shape, T, q, k, v, alpha, beta, g)
    _check_pool_ring(shape, pool, ring)
    _expect(y, T * shape.num_heads * shape.head_v, torch.float32, "y")
    ws_bytes = 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().kda_prefill(ctypes.byref(shape.c()), ctypes.byref(params.c()), B,
                              _ptr(cu_seqlens), T, int(max_seqlen), pool.shape[0],
                              _ptr(slot_ids), _ptr(positions), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(alpha), _ptr(beta), _ptr(g), _ptr(pool), _ptr(ring),
                              _ptr(y), _ptr(workspace), ws_bytes, _ptr(status),
                              _stream(stream)))


def prefill_noalloc(shape, params, cu_seqlens, max_seqlen, slot_ids, positions, q, k, v,
                    alpha, beta, g, pool, ring, y, status=None, stream=None):
    """kda_prefill with the library's fixed scratch array as its workspace
    (no allocation; calls needing more than PREFILL_SCRATCH_BYTES of
    workspace raise KdaError with code ERR_TOO_LARGE)."""
    B = slot_ids.numel()
    T = q.shape[0]
    _check_params(shape, params)
    _expect(cu_seqlens, B + 1, torch.int32, "cu_seqlens")
    _expect(slot_ids, B, torch.int32, "slot_ids")
    _expect(positions, B, torch.int32, "positions")
    _check_tokens(shape, T, q, k, v, alpha, beta, g)
    _check_pool_ring(shape, pool, ring)
    _expect(y, T * shape.num_heads * shape.head_v, torch.float32, "y")
    _check(load().kda_prefill_noalloc(ctypes.byref(shape.c()), ctypes.byref(params.c()), B,
                                      _ptr(cu_seqlens), T, int(max_seqlen), pool.shape[0],
                                      _ptr(slot_ids), _ptr(positions), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(alpha), _ptr(beta), _ptr(g), _ptr(pool),
                                      _ptr(ring), _ptr(y), _ptr(status), _stream(stream)))
