"""GPU parity of kda_verify and kda_commit_accepted against the CPU oracle,
and the decode == verify + commit(m) property on the device."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
import oracle

pytestmark = pytest.mark.gpu


def run_verify_gpu(case, ds, slots=None):
    torch = need_gpu()
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, n, H, dk, dv = case.batch, case.n_draft, case.H, case.dk, case.dv
    C = 2 * dk + dv
    slots = ds.slots if slots is None else slots
    slot_t = torch.from_numpy(slots.astype(np.int32)).cuda()
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    rec = torch.full((B, n, H, dk, dv), float("nan"), device="cuda")
    dconv = torch.full((B, n, H, C), float("nan"), device="cuda",
                       dtype=ds.shape.act_dtype)
    y = torch.full((B, n, H, dv), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool0 = ds.pool.clone()
    ring0 = ds.ring.clone()
    kda.verify(ds.shape, ds.params, slot_t, pos_t, tok["q"], tok["k"], tok["v"],
               tok["alpha"], tok["beta"], tok["g"], ds.pool, ds.ring, rec, dconv, y,
               status)
    torch.cuda.synchronize()
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8)), \
        "verify must not write the pool"
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8)), \
        "verify must not write the ring"
    return rec, dconv, y, slot_t, pos_t, status


def commit_gpu(case, ds, rec, dconv, slot_t, pos_t, accepted):
    torch = need_gpu()
    acc_t = torch.from_numpy(np.asarray(accepted, dtype=np.int32)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.commit_accepted(ds.shape, slot_t, pos_t, acc_t, rec, dconv, ds.pool, ds.ring,
                        status)
    torch.cuda.synchronize()
    return int(status.item())


def check_verify_commit(case):
    print(f"case {case.name}: B={case.batch} H={case.H} d={case.dk} n={case.n_draft} "
          f"act={case.act} state={case.state}", flush=True)
    ds = dev.make_state(case)
    rec, dconv, y, slot_t, pos_t, status = run_verify_gpu(case, ds)
    assert int(status.item()) == 0
    y_ref, rec_ref, S_ref, h_ref = oracle.verify_case(case)
    # records and outputs are FP32 under either storage dtype; with BF16
    # storage the start state is the dequantised BF16 pool, shared by both
    assert_parity(y.cpu().numpy(), y_ref, 2e-5, "verify y")
    rec_l = rec.cpu().numpy()
    assert_parity(rec_l, rec_ref, 2e-5, "verify records")
    # raw drafts are kept bit for bit
    raw = np.concatenate([case.tokens.q, case.tokens.k, case.tokens.v], axis=-1)
    np.testing.assert_array_equal(dev.acts_to_numpy(dconv, case.act), raw)
    assert commit_gpu(case, ds, rec, dconv, slot_t, pos_t, case.accepted) == 0
    assert_parity(dev.read_states(ds), S_ref, tol_for(case.state), "committed states")
    win = dev.read_window(ds, case.pos0 + case.accepted)
    np.testing.assert_array_equal(win, h_ref)
    return ds


def test_config2_verify_commit():
    need_gpu()
    check_verify_commit(wl.config(2))


@pytest.mark.parametrize("act,state,d,n", [("bf16", "bf16", 128, 4), ("f32", "f32", 64, 8),
                                           ("bf16", "f32", 64, 1), ("f32", "bf16", 128, 6)])
def test_verify_matrix(act, state, d, n):
    need_gpu()
    case = wl.make_verify(40 + n, B=6, H=3, dk=d, dv=d, n_draft=n, act=act, state=state,
                          init="random", name=f"verify_{act}_{state}_{d}_{n}")
    check_verify_commit(case)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_verify_commit_equals_decode_steps(state):
    """For every m in 0..n: verify + commit(m) against m device decode steps.
    FP32 storage: bitwise.  BF16 storage: one rounding at commit against one
    per step, so within the BF16 bar."""
    torch = need_gpu()
    n = 5
    base = wl.make_verify(50, B=n + 1, H=4, dk=128, dv=128, n_draft=n, act="bf16",
                          state=state, init="random", name=f"v_eq_d_{state}")
    base.accepted = np.arange(n + 1, dtype=np.int32)       # row b accepts b tokens
    ds_v = dev.make_state(base)
    rec, dconv, _, slot_t, pos_t, _ = run_verify_gpu(base, ds_v)
    assert commit_gpu(base, ds_v, rec, dconv, slot_t, pos_t, base.accepted) == 0

    ds_d = dev.make_state(base)                             # same start, same slots
    tok = dev.tokens_to_device(base.tokens, base.act)
    y = torch.empty((base.batch, base.H, base.dv), device="cuda")
    for t in range(n):
        active = base.accepted > t
        slots = torch.from_numpy(np.where(active, ds_d.slots, -1).astype(np.int32)).cuda()
        pos = torch.from_numpy((base.pos0 + t).astype(np.int32)).cuda()
        kda.decode(ds_d.shape, ds_d.params, slots, pos,
                   *[tok[name][:, t].contiguous() for name in
                     ("q", "k", "v", "alpha", "beta", "g")],
                   ds_d.pool, ds_d.ring, y)
    torch.cuda.synchronize()
    if state == "f32":
        assert torch.equal(ds_v.pool.view(torch.uint8), ds_d.pool.view(torch.uint8))
    else:
        assert_parity(dev.read_states(ds_v), dev.read_states(ds_d), 1e-2, "v+c vs decode")
    np.testing.assert_array_equal(dev.read_window(ds_v, base.pos0 + base.accepted),
                                  dev.read_window(ds_d, base.pos0 + base.accepted))


def test_commit_zero_is_noop_and_bad_accepted_is_reported():
    torch = need_gpu()
    case = wl.make_verify(51, B=3, H=2, dk=64, dv=64, n_draft=3, act="bf16", state="f32",
                          init="random", name="commit_edges")
    ds = dev.make_state(case)
    rec, dconv, _, slot_t, pos_t, _ = run_verify_gpu(case, ds)
    pool0, ring0 = ds.pool.clone(), ds.ring.clone()
    assert commit_gpu(case, ds, rec, dconv, slot_t, pos_t, [0, 0, 0]) == 0
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8))
    st = commit_gpu(case, ds, rec, dconv, slot_t, pos_t, [4, -1, 0])
    assert st == kda.STATUS_BAD_ACCEPTED
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))


def test_verify_inactive_rows_write_nothing():
    torch = need_gpu()
    case = wl.make_verify(52, B=4, H=2, dk=128, dv=128, n_draft=2, act="bf16",
                          state="bf16", init="random", name="verify_inactive")
    ds = dev.make_state(case)
    slots = ds.slots.copy()
    slots[[1, 3]] = -1
    rec, dconv, y, _, _, status = run_verify_gpu(case, ds, slots=slots)
    assert int(status.item()) == 0
    assert torch.isnan(rec[[1, 3]]).all() and torch.isnan(y[[1, 3]]).all()
    assert torch.isnan(dconv[[1, 3]].float()).all()
    assert not torch.isnan(rec[[0, 2]]).any()
