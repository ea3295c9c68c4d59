"""GPU parity with FP8 E4M3 activations: q, k, v, the ring and the raw
drafts are E4M3 bytes times a per-tensor scale, alpha, beta and g BF16.  The
oracle runs on the same (exact) values, so every bar is the usual one."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
from test_gpu_decode import check_decode
from test_gpu_prefill import check_prefill
from test_gpu_recompute import recompute, verify_no_records
from test_gpu_verify import check_verify_commit
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("state,d", [("f32", 128), ("bf16", 128), ("f32", 64)])
def test_decode_fp8_activations(state, d):
    need_gpu()
    case = wl.make_decode(91, B=5, H=3, dk=d, dv=d, steps=6, act="fp8", state=state,
                          init="random", active_per_step=4, name=f"decode_fp8_{state}_{d}")
    check_decode(case)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_verify_commit_and_recompute_fp8_activations(state):
    torch = need_gpu()
    case = wl.make_verify(92, B=6, H=3, dk=128, dv=128, n_draft=4, act="fp8", state=state,
                          init="random", name=f"verify_fp8_{state}")
    case.accepted = np.array([0, 1, 2, 3, 4, 4], dtype=np.int32)
    ds_r = check_verify_commit(case)
    ds = dev.make_state(case)
    tok, slot_t, pos_t, _, st = verify_no_records(case, ds)
    assert st == 0
    assert recompute(ds, tok, slot_t, pos_t, case.accepted) == 0
    assert torch.equal(ds.pool.view(torch.uint8), ds_r.pool.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ds_r.ring.view(torch.uint8))


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_prefill_fp8_activations(state):
    need_gpu()
    case = wl.make_prefill(93, lens=[150, 1, 77, 64], H=2, dk=128, dv=128, act="fp8",
                           state=state, init="random", slice_len=32, name=f"prefill_fp8_{state}")
    check_prefill(case)


def test_fp8_large_prefill_against_sampled_oracle():
    """The chunked-prefill shape of the benchmark on FP8 inputs, shortened to
    two sequences of 2048 and 640 tokens: final states and a 512-token slice."""
    need_gpu()
    case = wl.make_prefill(94, lens=[2048, 640], H=8, dk=128, dv=128, act="fp8", state="f32",
                           slice_len=512, name="prefill_fp8_long")
    check_prefill(case, full_outputs=False)


def test_conv_history_roundtrip_fp8():
    """kda_conv_write then kda_conv_read gives the window back bit for bit."""
    torch = need_gpu()
    case = wl.make_decode(95, B=4, H=2, dk=128, dv=128, steps=1, act="fp8", state="f32",
                          init="random", name="conv_io_fp8")
    ds = dev.make_state(case)
    n, C = case.batch, 2 * case.dk + case.dv
    win = torch.empty((n, 3, case.H, C), device="cuda", dtype=torch.float8_e4m3fn)
    pos = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    kda.conv_read(ds.shape, ds.ring, ds.slot_ids, pos, win)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.acts_to_numpy(win, "fp8"), case.hist0)
    ring2 = kda.alloc_ring(ds.shape, ds.num_slots)
    kda.conv_write(ds.shape, ring2, ds.slot_ids, pos, win)
    win2 = torch.empty_like(win)
    kda.conv_read(ds.shape, ring2, ds.slot_ids, pos, win2)
    torch.cuda.synchronize()
    assert torch.equal(win.view(torch.uint8), win2.view(torch.uint8))


def test_every_finite_e4m3_code_decodes_exactly():
    """q, k and v built from all 254 finite E4M3 codes (subnormals, 448 and
    both signs included), shuffled over a decode workload: the kernels'
    conversion of every code matches the oracle run on the codes' values."""
    torch = need_gpu()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.float().numpy().astype(np.float64)
    vals = vals[np.isfinite(vals)] * wl.FP8_SCALE
    assert len(vals) == 254
    case = wl.make_decode(96, B=4, H=2, dk=128, dv=128, steps=3, act="fp8", state="f32",
                          init="random", name="decode_fp8_all_codes")
    rng = np.random.default_rng(96)
    for name in ("q", "k", "v"):
        arr = getattr(case.tokens, name)
        arr[...] = rng.permutation(np.resize(vals, arr.size)).reshape(arr.shape)
    check_decode(case)


def test_fp8_activations_with_gate_logits():
    """FP8 q, k, v together with BF16 gate logits, in decode and in a
    continued prefill."""
    need_gpu()
    case = wl.make_decode(97, B=4, H=2, dk=128, dv=128, steps=4, act="fp8", state="bf16",
                          init="random", gates="logits", name="decode_fp8_logits")
    check_decode(case)
    case = wl.make_prefill(98, lens=[90, 3, 140], H=2, dk=128, dv=128, act="fp8", state="f32",
                           init="random", gates="logits", slice_len=32,
                           name="prefill_fp8_logits")
    check_prefill(case)
