"""GPU parity of kda_decode against the CPU oracle (token by token)."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
import oracle

pytestmark = pytest.mark.gpu


def run_decode_gpu(case, ds, *, steps=None):
    torch = need_gpu()
    steps = case.steps if steps is None else steps
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, H, dv = case.batch, case.H, case.dv
    y = torch.full((steps, B, H, dv), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = case.pos0.copy()
    for s in range(steps):
        act = case.active[s]
        slot_t = torch.from_numpy(np.where(act, ds.slots, -1).astype(np.int32)).cuda()
        pos_t = torch.from_numpy(pos.astype(np.int32)).cuda()
        kda.decode(ds.shape, ds.params, slot_t, pos_t, tok["q"][s], tok["k"][s],
                   tok["v"][s], tok["alpha"][s], tok["beta"][s], tok["g"][s],
                   ds.pool, ds.ring, y[s], status)
        pos += act
    torch.cuda.synchronize()
    return y.cpu().numpy(), pos, int(status.item())


def check_decode(case, *, gate="sigmoid", q_scale=1.0, device_S0=None):
    print(f"case {case.name}: B={case.batch} H={case.H} d={case.dk} "
          f"act={case.act} state={case.state} steps={case.steps}", flush=True)
    dcase = case if device_S0 is None else _with_S0(case, device_S0)
    ds = dev.make_state(dcase, gate=gate, q_scale=q_scale)
    y, pos, status = run_decode_gpu(case, ds)
    assert status == 0
    y_ref, S_ref, h_ref = oracle.decode_case(case, gate=gate) if q_scale == 1.0 else \
        _oracle_qscale(case, gate, q_scale)
    tol = tol_for(case.state)
    act = case.active[:, :, None, None].repeat(case.H, 2).repeat(case.dv, 3)
    assert np.all(np.isnan(y[~act])), "inactive rows must leave y untouched"
    assert_parity(y[act], y_ref[act], tol, "y")
    assert_parity(dev.read_states(ds), S_ref, tol, "final states")
    win = dev.read_window(ds, pos)
    np.testing.assert_array_equal(win, h_ref)
    spare = np.setdiff1d(np.arange(ds.num_slots), ds.slots)
    assert np.all(np.isnan(ds.pool[spare].float().cpu().numpy()))
    assert np.all(np.isnan(ds.ring[spare].float().cpu().numpy()))
    return ds


def _with_S0(case, S0):
    import copy
    c = copy.copy(case)
    c.S0 = S0
    return c


def _oracle_qscale(case, gate, q_scale):
    import copy
    from oracle.ref import OracleCfg, run_heads
    cfg = OracleCfg(case.dk, case.dv, case.width, gate, q_scale)
    S = case.S0.astype(np.float64)
    h = case.hist0.astype(np.float64)
    y, _ = run_heads(cfg, S, h, case.tokens, case.weights,
                     round_each_token=case.state == "bf16")
    return np.transpose(y, (1, 0, 2, 3)), S, h


def test_config0_tiny_decode():
    need_gpu()
    check_decode(wl.config(0))


def test_config1_batched_decode():
    need_gpu()
    check_decode(wl.config(1))


def test_config3_bf16_state_ragged():
    need_gpu()
    check_decode(wl.config(3))


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_two_head_large_batch_decode(state):
    """The small per-GPU head count (two heads, 256 rows), with both storage
    dtypes, as the benchmark's two-head mode launches it (one 256-row
    launch per step, 512 workgroups)."""
    need_gpu()
    check_decode(wl.compact_heads(state))


@pytest.mark.parametrize("act,state,d", [("f32", "f32", 128), ("bf16", "bf16", 64),
                                         ("f32", "bf16", 128), ("bf16", "f32", 64)])
def test_decode_dtype_and_size_matrix(act, state, d):
    need_gpu()
    case = wl.make_decode(20 + d, B=5, H=3, dk=d, dv=d, steps=7, act=act, state=state,
                          init="random", active_per_step=4, name=f"mix_{act}_{state}_{d}")
    check_decode(case)


def test_decode_silu_gate_norm_weight_and_q_scale():
    need_gpu()
    rng = np.random.default_rng(3)
    case = wl.make_decode(31, B=4, H=2, dk=128, dv=128, steps=5, act="bf16", state="f32",
                          init="random", norm_w=rng.uniform(0.5, 1.5, 128),
                          name="silu_normw")
    check_decode(case, gate="silu", q_scale=0.75)


def test_decode_fresh_and_short_histories():
    """positions 0..5: position 0 ignores the (random) pool and the ring;
    positions 1..2 read only the part of the history that exists."""
    need_gpu()
    case = wl.make_decode(32, B=6, H=4, dk=128, dv=128, steps=4, act="bf16",
                          state="f32", init="random", name="short_history")
    device_S0 = case.S0.copy()
    case.pos0 = np.arange(6, dtype=np.int64)
    for b in range(6):
        if case.pos0[b] == 0:
            case.S0[b] = 0.0
        for j in range(3):
            if case.pos0[b] - 3 + j < 0:
                case.hist0[b, j] = 0.0
    check_decode(case, device_S0=device_S0)


def test_decode_bad_slot_sets_status_and_writes_nothing():
    torch = need_gpu()
    case = wl.make_decode(33, B=3, H=2, dk=64, dv=64, steps=1, act="bf16", state="f32",
                          init="random", name="bad_slot")
    ds = dev.make_state(case)
    tok = dev.tokens_to_device(case.tokens, case.act)
    pool0 = ds.pool.clone()
    ring0 = ds.ring.clone()
    slots = torch.tensor([ds.num_slots, ds.num_slots + 7, -1], dtype=torch.int32,
                         device="cuda")
    pos = torch.tensor([3, 4, 5], dtype=torch.int32, device="cuda")
    y = torch.full((3, 2, 64), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.decode(ds.shape, ds.params, slots, pos, tok["q"][0], tok["k"][0], tok["v"][0],
               tok["alpha"][0], tok["beta"][0], tok["g"][0], ds.pool, ds.ring, y, status)
    torch.cuda.synchronize()
    assert status.item() == kda.STATUS_BAD_SLOT
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8))
    assert torch.isnan(y).all()
    # a negative position is reported too
    slots = torch.tensor([int(ds.slots[0]), -1, -1], dtype=torch.int32, device="cuda")
    pos = torch.tensor([-2, 0, 0], dtype=torch.int32, device="cuda")
    status.zero_()
    kda.decode(ds.shape, ds.params, slots, pos, tok["q"][0], tok["k"][0], tok["v"][0],
               tok["alpha"][0], tok["beta"][0], tok["g"][0], ds.pool, ds.ring, y, status)
    torch.cuda.synchronize()
    assert status.item() == kda.STATUS_BAD_POSITION
    assert torch.isnan(y).all()


def test_decode_is_bitwise_deterministic():
    torch = need_gpu()
    case = wl.make_decode(34, B=16, H=8, dk=128, dv=128, steps=3, act="bf16",
                          state="bf16", init="random", name="determinism")
    outs = []
    for _ in range(2):
        ds = dev.make_state(case)
        y, _, _ = run_decode_gpu(case, ds)
        outs.append((y, ds.pool.float().cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("act,state", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
                                       ("fp8", "bf16")])
def test_decode_many_rows_matches_small_calls(act, state):
    """64 rows x 32 heads (2,048 row-head items) in one launch, with ragged
    activity and rows starting at positions 0..7 (fresh sequences and short
    histories).  The outputs, states and histories match the oracle, and
    equal bit for bit what the same rows give when decoded four at a time:
    the grid size changes nothing about a row's arithmetic."""
    torch = need_gpu()
    case = wl.make_decode(35, B=64, H=32, dk=128, dv=128, steps=3, act=act, state=state,
                          init="random", active_per_step=48,
                          name=f"many_rows_{act}_{state}")
    device_S0 = case.S0.copy()
    case.pos0 = (np.arange(64) % 8).astype(np.int64)
    for b in range(64):
        if case.pos0[b] == 0:
            case.S0[b] = 0.0
        for j in range(3):
            if case.pos0[b] - 3 + j < 0:
                case.hist0[b, j] = 0.0
    ds = check_decode(case, device_S0=device_S0)
    # the same steps, four rows per call
    ds4 = dev.make_state(_with_S0(case, device_S0))
    tok = dev.tokens_to_device(case.tokens, case.act)
    y4 = torch.full((case.steps, 64, 32, 128), float("nan"), device="cuda")
    pos = case.pos0.copy()
    for s in range(case.steps):
        act_s = case.active[s]
        for r0 in range(0, 64, 4):
            rows = slice(r0, r0 + 4)
            slot_t = torch.from_numpy(np.where(act_s[rows], ds4.slots[rows], -1)
                                      .astype(np.int32)).cuda()
            pos_t = torch.from_numpy(pos[rows].astype(np.int32)).cuda()
            kda.decode(ds4.shape, ds4.params, slot_t, pos_t, tok["q"][s][rows].contiguous(),
                       tok["k"][s][rows].contiguous(), tok["v"][s][rows].contiguous(),
                       tok["alpha"][s][rows].contiguous(), tok["beta"][s][rows].contiguous(),
                       tok["g"][s][rows].contiguous(), ds4.pool, ds4.ring, y4[s][rows])
        pos += act_s
    torch.cuda.synchronize()
    y_all, _, _ = run_decode_gpu(case, dev.make_state(_with_S0(case, device_S0)))
    np.testing.assert_array_equal(y4.cpu().numpy(), y_all)
    assert torch.equal(ds4.pool.view(torch.uint8), ds.pool.view(torch.uint8))
    assert torch.equal(ds4.ring.view(torch.uint8), ds.ring.view(torch.uint8))


def test_decode_bad_rows_among_many():
    """Bad slots and negative positions among 64 rows x 32 heads: reported,
    those rows untouched, the others as the oracle has them."""
    torch = need_gpu()
    case = wl.make_decode(36, B=64, H=32, dk=128, dv=128, steps=1, act="bf16", state="bf16",
                          init="random", name="many_rows_bad_rows")
    ds = dev.make_state(case)
    tok = dev.tokens_to_device(case.tokens, case.act)
    pool0 = ds.pool.clone()
    slots = ds.slots.astype(np.int32).copy()
    pos = case.pos0.astype(np.int32).copy()
    slots[5] = ds.num_slots + 1
    slots[17] = -1
    pos[40] = -3
    y = torch.full((64, 32, 128), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.decode(ds.shape, ds.params, torch.from_numpy(slots).cuda(),
               torch.from_numpy(pos).cuda(), tok["q"][0], tok["k"][0], tok["v"][0],
               tok["alpha"][0], tok["beta"][0], tok["g"][0], ds.pool, ds.ring, y, status)
    torch.cuda.synchronize()
    assert status.item() == kda.STATUS_BAD_SLOT | kda.STATUS_BAD_POSITION
    y = y.cpu().numpy()
    bad = [5, 17, 40]
    assert np.isnan(y[bad]).all()
    for b in bad:
        if slots[b] >= 0 and slots[b] < ds.num_slots:
            assert torch.equal(ds.pool[slots[b]].view(torch.uint8),
                               pool0[slots[b]].view(torch.uint8))
    good = np.setdiff1d(np.arange(64), bad)
    y_ref, S_ref, _ = oracle.decode_case(case)
    assert_parity(y[good], y_ref[0][good], tol_for(case.state), "y of the good rows")
    assert_parity(dev.read_states(ds)[good], S_ref[good], tol_for(case.state),
                  "states of the good rows")
