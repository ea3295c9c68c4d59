"""Speculative verify without per-token records, then kda_commit_recompute:
the accepted tokens run again from the stored state.  Checked against the
oracle's verify + commit and, bit for bit, against the records path
(kda_verify with records + kda_commit_accepted)."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
import oracle
from test_gpu_verify import commit_gpu, run_verify_gpu

pytestmark = pytest.mark.gpu


def verify_no_records(case, ds, slots=None):
    torch = need_gpu()
    tok = dev.tokens_to_device(case.tokens, case.act)
    slots = ds.slots if slots is None else slots
    slot_t = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    y = torch.full((case.batch, case.n_draft, case.H, case.dv), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool0, ring0 = ds.pool.clone(), ds.ring.clone()
    kda.verify(ds.shape, ds.params, slot_t, pos_t, tok["q"], tok["k"], tok["v"],
               tok["alpha"], tok["beta"], tok["g"], ds.pool, ds.ring, None, None, y, status)
    torch.cuda.synchronize()
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8))
    return tok, slot_t, pos_t, y, int(status.item())


def recompute(ds, tok, slot_t, pos_t, accepted):
    torch = need_gpu()
    acc_t = torch.from_numpy(np.asarray(accepted, dtype=np.int32)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.commit_recompute(ds.shape, ds.params, slot_t, pos_t, acc_t, tok["q"], tok["k"],
                         tok["v"], tok["alpha"], tok["beta"], tok["g"], ds.pool, ds.ring,
                         status)
    torch.cuda.synchronize()
    return int(status.item())


@pytest.mark.parametrize("act,state,d,n", [("bf16", "f32", 128, 4), ("bf16", "bf16", 128, 4),
                                           ("f32", "f32", 64, 7), ("f32", "bf16", 64, 3)])
def test_recompute_commit_matches_oracle_and_records_path(act, state, d, n):
    torch = need_gpu()
    case = wl.make_verify(53, B=n + 3, H=3, dk=d, dv=d, n_draft=n, act=act, state=state,
                          init="random", name=f"recompute_{act}_{state}_{d}_{n}")
    case.accepted = np.concatenate([np.arange(n + 1), [n, 0]]).astype(np.int32)
    print(f"case {case.name}: accepted={case.accepted.tolist()}", flush=True)
    # records path
    ds_r = dev.make_state(case)
    rec, dconv, y_r, slot_t, pos_t, st = run_verify_gpu(case, ds_r)
    assert int(st.item()) == 0
    assert commit_gpu(case, ds_r, rec, dconv, slot_t, pos_t, case.accepted) == 0
    # no records, commit by recompute
    ds = dev.make_state(case)
    tok, slot_t, pos_t, y, st = verify_no_records(case, ds)
    assert st == 0
    assert torch.equal(y, y_r), "verify outputs must not depend on keeping records"
    assert recompute(ds, tok, slot_t, pos_t, case.accepted) == 0
    y_ref, _, S_ref, h_ref = oracle.verify_case(case)
    assert_parity(y.cpu().numpy(), y_ref, 2e-5, "verify y")
    assert_parity(dev.read_states(ds), S_ref, tol_for(state), "recomputed commit states")
    np.testing.assert_array_equal(dev.read_window(ds, case.pos0 + case.accepted), h_ref)
    # the same per-token arithmetic, FP32 across the tokens, one rounding on store
    assert torch.equal(ds.pool.view(torch.uint8), ds_r.pool.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ds_r.ring.view(torch.uint8))


def test_recompute_from_fresh_sequences():
    """Position 0: zero state, empty history; every draft accepted."""
    need_gpu()
    case = wl.make_verify(54, B=3, H=2, dk=128, dv=128, n_draft=5, act="bf16", state="f32",
                          init="zero", name="recompute_fresh")
    case.accepted = np.array([5, 3, 1], dtype=np.int32)
    ds = dev.make_state(case)
    tok, slot_t, pos_t, _, _ = verify_no_records(case, ds)
    assert recompute(ds, tok, slot_t, pos_t, case.accepted) == 0
    _, _, S_ref, h_ref = oracle.verify_case(case)
    assert_parity(dev.read_states(ds), S_ref, 2e-5, "states")
    np.testing.assert_array_equal(dev.read_window(ds, case.pos0 + case.accepted), h_ref)


def test_recompute_zero_inactive_and_bad_accepted_write_nothing():
    torch = need_gpu()
    case = wl.make_verify(55, B=4, H=2, dk=64, dv=64, n_draft=3, act="bf16", state="bf16",
                          init="random", name="recompute_edges")
    ds = dev.make_state(case)
    slots = ds.slots.copy()
    slots[2] = -1
    tok, slot_t, pos_t, _, _ = verify_no_records(case, ds, slots=slots)
    pool0, ring0 = ds.pool.clone(), ds.ring.clone()
    assert recompute(ds, tok, slot_t, pos_t, [0, 0, 3, 0]) == 0
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8))
    st = recompute(ds, tok, slot_t, pos_t, [4, -1, 3, 0])
    assert st == kda.STATUS_BAD_ACCEPTED
    assert torch.equal(ds.pool.view(torch.uint8), pool0.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ring0.view(torch.uint8))


def test_longest_draft_block_records_and_recompute_agree():
    """n_draft = 16, the longest block the library takes: accepted lengths
    past the ring's four entries overwrite ring entries several times, and
    both commits keep the last three raw tokens."""
    torch = need_gpu()
    n = 16
    case = wl.make_verify(56, B=6, H=2, dk=128, dv=128, n_draft=n, act="bf16", state="f32",
                          init="random", name="recompute_n16")
    case.accepted = np.array([16, 15, 5, 4, 3, 0], dtype=np.int32)
    ds_r = dev.make_state(case)
    rec, dconv, y_r, slot_t, pos_t, st = run_verify_gpu(case, ds_r)
    assert int(st.item()) == 0
    assert commit_gpu(case, ds_r, rec, dconv, slot_t, pos_t, case.accepted) == 0
    ds = dev.make_state(case)
    tok, slot_t, pos_t, y, _ = verify_no_records(case, ds)
    assert recompute(ds, tok, slot_t, pos_t, case.accepted) == 0
    y_ref, rec_ref, S_ref, h_ref = oracle.verify_case(case)
    assert_parity(y_r.cpu().numpy(), y_ref, 2e-5, "verify y")
    assert_parity(rec.cpu().numpy(), rec_ref, 2e-5, "records")
    assert_parity(dev.read_states(ds), S_ref, 2e-5, "recomputed states")
    np.testing.assert_array_equal(dev.read_window(ds, case.pos0 + case.accepted), h_ref)
    assert torch.equal(y, y_r)
    assert torch.equal(ds.pool.view(torch.uint8), ds_r.pool.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ds_r.ring.view(torch.uint8))
