"""kda_prefill_noalloc, the prefill for callers that cannot allocate (its
workspace is the library's fixed per-GPU scratch array), against kda_prefill
with a caller's workspace: two calls in a row through the C-ABI, the second
with a smaller input, each equal bit for bit to kda_prefill's result and
within the FP32 parity bar of the oracle."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
import oracle

pytestmark = pytest.mark.gpu


def _call(case, noalloc):
    torch = need_gpu()
    ds = dev.make_state(case)
    tok = dev.tokens_to_device(case.tokens, case.act)
    T = int(case.cu_seqlens[-1])
    y = torch.full((T, case.H, case.dv), float("nan"), device="cuda")
    cu_t = torch.from_numpy(case.cu_seqlens.astype(np.int32)).cuda()
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (ds.shape, ds.params, cu_t, max(case.lens), ds.slot_ids, pos_t, tok["q"],
            tok["k"], tok["v"], tok["alpha"], tok["beta"], tok["g"], ds.pool, ds.ring, y)
    if noalloc:
        kda.prefill_noalloc(*args, status=status)
    else:
        nbytes = kda.prefill_workspace_bytes(ds.shape, case.batch, T)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        kda.prefill(*args, ws, status=status)
    torch.cuda.synchronize()
    end = case.pos0 + np.asarray(case.lens)
    return (y.cpu().numpy(), dev.read_states(ds), dev.read_window(ds, end),
            int(status.item()))


def test_noalloc_prefill_two_calls_second_smaller():
    need_gpu()
    big = wl.make_prefill(91, lens=[900, 300, 64, 1], H=4, dk=128, dv=128, act="bf16",
                          state="f32", init="random", slice_len=32, name="noalloc_big")
    small = wl.make_prefill(92, lens=[130, 5], H=4, dk=128, dv=128, act="bf16",
                            state="f32", init="random", slice_len=32, name="noalloc_small")
    refs = [_call(c, noalloc=False) for c in (big, small)]
    got = [_call(c, noalloc=True) for c in (big, small)]     # back to back, shared scratch
    for case, r, o in zip((big, small), refs, got):
        print(f"case {case.name}: lens={case.lens}", flush=True)
        assert r[3] == 0 and o[3] == 0
        np.testing.assert_array_equal(o[0], r[0])            # outputs
        np.testing.assert_array_equal(o[1], r[1])            # final states
        np.testing.assert_array_equal(o[2], r[2])            # conv history
        y_ref, S_ref, _ = oracle.prefill_case(case)
        assert_parity(o[0], y_ref, 2e-5, "outputs vs oracle")
        assert_parity(o[1], S_ref, 2e-5, "final states vs oracle")


def test_noalloc_prefill_rejects_calls_beyond_its_scratch():
    torch = need_gpu()
    lens = [kda.PREFILL_SCRATCH_BYTES // (147456 * 32) * 64]     # one chunk slot too many
    case = wl.make_prefill(93, lens=lens, H=32, dk=128, dv=128, act="bf16", state="f32",
                           slice_len=32, name="noalloc_too_large")
    assert kda.prefill_workspace_bytes(dev.shape_of(case), 1, lens[0]) > \
        kda.PREFILL_SCRATCH_BYTES
    with pytest.raises(kda.KdaError) as e:
        _call(case, noalloc=True)
    assert e.value.code == kda.ERR_TOO_LARGE
    torch.cuda.synchronize()
