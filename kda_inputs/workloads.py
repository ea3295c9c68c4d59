"""Seeded synthetic inputs for the KDA mixer.

This module draws inputs and nothing else.  It holds none of the mixer's
arithmetic, so both the HIP path and the CPU oracle may consume what it
produces.  It imports neither of them.

Distributions, following the workloads the mixer is measured on:
  * raw q, k, v          N(0, 1)
  * decay alpha          exp(-softplus(a)), a ~ N(0, 1), one per key channel
  * write strength beta  sigmoid(b), b ~ N(0, 1), one per head
  * output gate g        N(0, 1), one per value channel
  * conv weights         N(0, 0.5) (second argument = standard deviation)
  * initial state        N(0, 0.1) where a workload starts from a random state
  * conv history         N(0, 1)   where a workload starts mid-sequence

A workload with gates="logits" hands the mixer the logits a and b
themselves (rounded to the activation dtype) in place of alpha and beta;
the mixer then forms alpha and beta.

Draws are fp64 from numpy's PCG64 and are then rounded to the activation
dtype: float32 (round to nearest even), bfloat16 (round to float32, then
to nearest even on the upper 16 bits), or for "fp8" q, k, v and the history
to E4M3 values times FP8_SCALE with alpha, beta and g in bfloat16.  Conv and norm weights stay float32.
Every array here holds values that are exact in its dtype, stored as float32
(bfloat16 values are float32 values with 16 zero low bits); ``bf16_bits``
gives the 16-bit patterns the device buffers hold.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ACT_DTYPES = ("f32", "bf16", "fp8")

# FP8 workloads store q, k, v (and the raw history) as E4M3 values times this
# per-tensor dequantisation scale; N(0, 1) draws then sit far inside E4M3's
# range (|x| / scale <= 448 for |x| <= 14).
FP8_SCALE = 2.0 ** -5
STATE_DTYPES = ("f32", "bf16")


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of the float32 rounding of x, as float32 values."""
    u = round_f32(x).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest OCP FP8 E4M3 value (bias 7, three mantissa bits, no
    infinities, largest finite 448), ties to even, saturating at +-448, as
    float32.  A binade [2^e, 2^(e+1)) holds steps of 2^(e-3); below 2^-6 the
    subnormals keep the step 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = 2.0 ** (np.clip(e, -6, 8) - 3)
    r = np.minimum(np.round(a / step) * step, 448.0)     # np.round: ties to even
    return (np.sign(x) * r).astype(np.float32)


def gate_dtype(act: str) -> str:
    """dtype of alpha, beta and g: FP8 activations keep the gates in BF16."""
    return "bf16" if act == "fp8" else act


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp8":
        return (round_e4m3(np.asarray(x, dtype=np.float64) / FP8_SCALE) *
                np.float32(FP8_SCALE)).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 arrays that hold bfloat16 values."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bfloat16")
    return (u >> 16).astype(np.uint16)


def _softplus(a: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, a)


def _sigmoid(b: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-b))


@dataclass
class Weights:
    """Per-layer parameters: depthwise conv taps and the norm weight."""
    conv_q: np.ndarray  # [H, dk, W] float32
    conv_k: np.ndarray  # [H, dk, W] float32
    conv_v: np.ndarray  # [H, dv, W] float32
    norm_w: np.ndarray  # [dv] float32


@dataclass
class TokenInputs:
    """Per-token mixer inputs; leading dims are whatever the caller asked."""
    q: np.ndarray      # [..., H, dk]
    k: np.ndarray      # [..., H, dk]
    v: np.ndarray      # [..., H, dv]
    alpha: np.ndarray  # [..., H, dk]  (the logit a when gates == "logits")
    beta: np.ndarray   # [..., H]      (the logit b when gates == "logits")
    g: np.ndarray      # [..., H, dv]


@dataclass
class Case:
    """One workload: shapes, weights, starting state and the token stream."""
    name: str
    mode: str               # "decode" | "verify" | "prefill"
    H: int
    dk: int
    dv: int
    width: int
    act: str
    state: str
    weights: Weights
    batch: int
    S0: np.ndarray          # [batch, H, dk, dv] logical, exact in `state`
    hist0: np.ndarray       # [batch, width-1, H, 2dk+dv] raw, oldest first
    pos0: np.ndarray        # [batch] int64 tokens already consumed
    steps: int = 0          # decode
    n_draft: int = 0        # verify
    tokens: TokenInputs | None = None  # decode [steps,B,...]; verify [B,n,...]
    active: np.ndarray | None = None   # decode [steps, B] bool
    accepted: np.ndarray | None = None  # verify [B] int32
    lens: list = field(default_factory=list)   # prefill lengths
    cu_seqlens: np.ndarray | None = None       # prefill [B+1] int32
    chunk: int = 64
    slice_seq: int = -1    # prefill: sequence and start of the checked slice
    slice_start: int = -1
    slice_len: int = 0
    gates: str = "values"  # "logits": tokens.alpha / tokens.beta hold a and b


def _weights(rng, H, dk, dv, W):
    cq = round_f32(rng.normal(0.0, 0.5, size=(H, dk, W)))
    ck = round_f32(rng.normal(0.0, 0.5, size=(H, dk, W)))
    cv = round_f32(rng.normal(0.0, 0.5, size=(H, dv, W)))
    return Weights(cq, ck, cv, np.ones(dv, dtype=np.float32))


def _tokens(rng, lead, H, dk, dv, act, gates="values") -> TokenInputs:
    q = round_to(rng.standard_normal(lead + (H, dk)), act)
    k = round_to(rng.standard_normal(lead + (H, dk)), act)
    v = round_to(rng.standard_normal(lead + (H, dv)), act)
    a = rng.standard_normal(lead + (H, dk))
    b = rng.standard_normal(lead + (H,))
    ga = gate_dtype(act)
    if gates == "logits":
        alpha, beta = round_to(a, ga), round_to(b, ga)
    elif gates == "values":
        alpha = round_to(np.exp(-_softplus(a)), ga)
        beta = round_to(_sigmoid(b), ga)
    else:
        raise ValueError(f"unknown gate inputs {gates!r}")
    g = round_to(rng.standard_normal(lead + (H, dv)), ga)
    return TokenInputs(q, k, v, alpha, beta, g)


def _start(rng, B, H, dk, dv, W, act, state, init):
    C = 2 * dk + dv
    if init == "zero":
        S0 = np.zeros((B, H, dk, dv), dtype=np.float32)
        hist0 = np.zeros((B, W - 1, H, C), dtype=np.float32)
        pos0 = np.zeros(B, dtype=np.int64)
    elif init == "random":
        S0 = round_to(rng.normal(0.0, 0.1, size=(B, H, dk, dv)), state)
        hist0 = round_to(rng.standard_normal((B, W - 1, H, C)), act)
        pos0 = (W - 1) + (np.arange(B, dtype=np.int64) % 4)
    else:
        raise ValueError(init)
    return S0, hist0, pos0


def make_decode(seed, *, B, H, dk, dv, steps, act, state, init,
                active_per_step=None, width=4, name="decode", norm_w=None,
                gates="values"):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = _weights(rng, H, dk, dv, width)
    if norm_w is not None:
        w.norm_w = round_f32(norm_w)
    S0, hist0, pos0 = _start(rng, B, H, dk, dv, width, act, state, init)
    toks = _tokens(rng, (steps, B), H, dk, dv, act, gates)
    active = np.ones((steps, B), dtype=bool)
    if active_per_step is not None:
        active[:] = False
        for s in range(steps):
            active[s, rng.permutation(B)[:active_per_step]] = True
    return Case(name=name, mode="decode", H=H, dk=dk, dv=dv, width=width,
                act=act, state=state, weights=w, batch=B, S0=S0, hist0=hist0,
                pos0=pos0, steps=steps, tokens=toks, active=active, gates=gates)


def make_verify(seed, *, B, H, dk, dv, n_draft, act, state, init, width=4,
                name="verify", gates="values"):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = _weights(rng, H, dk, dv, width)
    S0, hist0, pos0 = _start(rng, B, H, dk, dv, width, act, state, init)
    toks = _tokens(rng, (B, n_draft), H, dk, dv, act, gates)
    accepted = rng.integers(0, n_draft + 1, size=B).astype(np.int32)
    return Case(name=name, mode="verify", H=H, dk=dk, dv=dv, width=width,
                act=act, state=state, weights=w, batch=B, S0=S0, hist0=hist0,
                pos0=pos0, n_draft=n_draft, tokens=toks, accepted=accepted,
                gates=gates)


def make_prefill(seed, *, lens, H, dk, dv, act, state, init="zero", width=4,
                 chunk=64, slice_len=512, name="prefill", gates="values"):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = _weights(rng, H, dk, dv, width)
    B = len(lens)
    S0, hist0, pos0 = _start(rng, B, H, dk, dv, width, act, state, init)
    total = int(sum(lens))
    toks = _tokens(rng, (total,), H, dk, dv, act, gates)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    # a slice of consecutive outputs to check at full size
    fits = [i for i, n in enumerate(lens) if n >= slice_len]
    if fits:
        s = int(fits[rng.integers(0, len(fits))])
        start = int(rng.integers(0, lens[s] - slice_len + 1))
    else:
        s, start, slice_len = 0, 0, int(lens[0])
    return Case(name=name, mode="prefill", H=H, dk=dk, dv=dv, width=width,
                act=act, state=state, weights=w, batch=B, S0=S0, hist0=hist0,
                pos0=pos0, tokens=toks, lens=list(lens), cu_seqlens=cu,
                chunk=chunk, slice_seq=s, slice_start=start,
                slice_len=slice_len, gates=gates)


# The five measured workloads.  The seed of each is its index.
CONFIG_NAMES = {
    0: "tiny_decode_B1_H4_d64_fp32",
    1: "batched_decode_B64_H32_d128_bf16act_f32state",
    2: "spec_verify_B16_H32_d128_n4_f32state",
    3: "large_batch_decode_B256_active192_H32_d128_bf16state",
    4: "chunked_prefill_lens8192_4096_2048_1024_H32_d128_C64",
}


def config(i: int) -> Case:
    if i == 0:
        return make_decode(0, B=1, H=4, dk=64, dv=64, steps=16, act="f32",
                           state="f32", init="zero", name=CONFIG_NAMES[0])
    if i == 1:
        return make_decode(1, B=64, H=32, dk=128, dv=128, steps=32,
                           act="bf16", state="f32", init="random",
                           name=CONFIG_NAMES[1])
    if i == 2:
        return make_verify(2, B=16, H=32, dk=128, dv=128, n_draft=4,
                           act="bf16", state="f32", init="random",
                           name=CONFIG_NAMES[2])
    if i == 3:
        return make_decode(3, B=256, H=32, dk=128, dv=128, steps=16,
                           act="bf16", state="bf16", init="random",
                           active_per_step=192, name=CONFIG_NAMES[3])
    if i == 4:
        return make_prefill(4, lens=[8192, 4096, 2048, 1024], H=32, dk=128,
                            dv=128, act="bf16", state="f32", init="zero",
                            chunk=64, name=CONFIG_NAMES[4])
    raise ValueError(f"no config {i}")


COMPACT_HEADS_NAME = "compact_heads_decode_B256_H2_d128_bf16act_{}state"


def compact_heads(state: str = "f32") -> Case:
    """Decode at a small per-GPU head count (two heads, as when the heads are
    split over many GPUs) with a large batch: 256 rows, 16 steps, inputs and
    start states drawn as in the batched-decode workload."""
    return make_decode(5, B=256, H=2, dk=128, dv=128, steps=16, act="bf16", state=state,
                       init="random", name=COMPACT_HEADS_NAME.format(state))


def fp8_decode() -> Case:
    """The batched-decode workload (64 rows, 32 heads, 32 steps, FP32 state)
    with FP8 E4M3 q, k, v and BF16 gates."""
    return make_decode(1, B=64, H=32, dk=128, dv=128, steps=32, act="fp8", state="f32",
                       init="random", name="batched_decode_B64_H32_d128_fp8act_f32state")


def fp8_prefill() -> Case:
    """The chunked-prefill workload with FP8 E4M3 q, k, v and BF16 gates."""
    return make_prefill(4, lens=[8192, 4096, 2048, 1024], H=32, dk=128, dv=128, act="fp8",
                        state="f32", name="chunked_prefill_lens8192_4096_2048_1024_H32_d128_C64_fp8act")

