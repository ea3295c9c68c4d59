"""GPU parity with gate logits as inputs (kda_shape.gate_inputs = LOGITS):
the kernels form alpha = exp(-softplus(a)) and beta = sigmoid(b) themselves,
and every mode matches the oracle run on the same logits."""
import numpy as np
import pytest

from gpu_util import need_gpu
from kda_inputs import workloads as wl
from test_gpu_decode import check_decode
from test_gpu_prefill import check_prefill
from test_gpu_verify import check_verify_commit

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("act,state,d", [("bf16", "f32", 128), ("f32", "bf16", 128),
                                         ("f32", "f32", 64)])
def test_decode_from_gate_logits(act, state, d):
    need_gpu()
    case = wl.make_decode(61, B=5, H=3, dk=d, dv=d, steps=6, act=act, state=state,
                          init="random", active_per_step=4, gates="logits",
                          name=f"decode_logits_{act}_{state}_{d}")
    check_decode(case)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_verify_commit_from_gate_logits(state):
    need_gpu()
    case = wl.make_verify(62, B=6, H=3, dk=128, dv=128, n_draft=4, act="bf16",
                          state=state, init="random", gates="logits",
                          name=f"verify_logits_{state}")
    check_verify_commit(case)


@pytest.mark.parametrize("act,state", [("bf16", "f32"), ("f32", "bf16")])
def test_prefill_from_gate_logits(act, state):
    need_gpu()
    case = wl.make_prefill(63, lens=[150, 1, 77], H=2, dk=128, dv=128, act=act,
                           state=state, init="random", slice_len=32, gates="logits",
                           name=f"prefill_logits_{act}_{state}")
    check_prefill(case)


def test_prefill_from_large_logits_stays_finite():
    """Decay logits up to +12 (alpha ~ 6e-6 per token) and write logits of
    either sign far from zero: the in-kernel maps stay in (0, 1] and the
    chunk form matches the oracle."""
    need_gpu()
    case = wl.make_prefill(64, lens=[128, 64], H=2, dk=128, dv=128, act="f32",
                           state="f32", slice_len=32, gates="logits",
                           name="prefill_large_logits")
    rng = np.random.default_rng(6)
    case.tokens.alpha[:] = wl.round_f32(rng.uniform(-4.0, 12.0, case.tokens.alpha.shape))
    case.tokens.beta[:] = wl.round_f32(rng.uniform(-8.0, 8.0, case.tokens.beta.shape))
    check_prefill(case)
