"""State semantics and call sequences on the GPU: the typed state store's
export/import round trip, interleaved pools over layers and steps, a
negative control for the commit check, and prefill determinism."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, rel_linf, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
from test_gpu_prefill import run_prefill_gpu
from test_gpu_verify import commit_gpu, run_verify_gpu
import oracle

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "beta", "g")


@pytest.mark.parametrize("act,state", [("bf16", "f32"), ("f32", "bf16")])
def test_state_and_history_export_import_round_trip(act, state):
    """kda_state_read returns the stored states exactly; kda_state_write
    stores FP32 values as they are (FP32) or rounded to nearest even (BF16)
    into the named slots only; the conv history round trip is bit exact."""
    torch = need_gpu()
    case = wl.make_decode(111, B=4, H=3, dk=128, dv=128, steps=1, act=act, state=state,
                          init="random", name="state_io")
    ds = dev.make_state(case)
    n, H, d = case.batch, case.H, case.dk
    got = torch.empty((n, H, d, d), device="cuda")
    kda.state_read(ds.shape, ds.pool, ds.slot_ids, got)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), case.S0)
    # import values that are not exact in the storage dtype into fresh slots
    rng = np.random.default_rng(5)
    x = rng.normal(0, 0.1, (n, H, d, d)).astype(np.float32)
    pool = torch.full_like(ds.pool, float("nan"))
    kda.state_write(ds.shape, pool, ds.slot_ids, torch.from_numpy(x).cuda())
    kda.state_read(ds.shape, pool, ds.slot_ids, got)
    torch.cuda.synchronize()
    want = x if state == "f32" else wl.round_bf16(x)
    np.testing.assert_array_equal(got.cpu().numpy(), want)
    spare = np.setdiff1d(np.arange(ds.num_slots), ds.slots)
    assert torch.isnan(pool[spare].float()).all(), "only the named slots are written"
    # conv history: read, write into a fresh ring, read again
    C = 2 * d + d
    pos = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    win = torch.empty((n, 3, H, C), device="cuda", dtype=ds.shape.act_dtype)
    kda.conv_read(ds.shape, ds.ring, ds.slot_ids, pos, win)
    ring2 = kda.alloc_ring(ds.shape, ds.num_slots)
    kda.conv_write(ds.shape, ring2, ds.slot_ids, pos, win)
    win2 = torch.empty_like(win)
    kda.conv_read(ds.shape, ring2, ds.slot_ids, pos, win2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.acts_to_numpy(win, act), case.hist0)
    assert torch.equal(win.view(torch.uint8), win2.view(torch.uint8))


def test_interleaved_pools_over_layers_and_steps():
    """Two models x three layers, each layer its own pool and inputs, run
    step by step with the calls interleaved (step, then layer, then model):
    every layer ends where its own token-by-token oracle run ends."""
    torch = need_gpu()
    steps, cases, states = 12, [], []
    for m in range(2):
        for layer in range(3):
            c = wl.make_decode(120 + 3 * m + layer, B=3, H=2, dk=64, dv=64, steps=steps,
                               act="bf16", state="f32" if m == 0 else "bf16", init="random",
                               name=f"model{m}_layer{layer}")
            cases.append(c)
            states.append(dev.make_state(c))
    toks = [dev.tokens_to_device(c.tokens, c.act) for c in cases]
    ys = [torch.full((steps, c.batch, c.H, c.dv), float("nan"), device="cuda") for c in cases]
    for s in range(steps):
        for layer in range(3):
            for m in range(2):
                i = 3 * m + layer
                c, ds, tok = cases[i], states[i], toks[i]
                pos = torch.from_numpy((c.pos0 + s).astype(np.int32)).cuda()
                kda.decode(ds.shape, ds.params, ds.slot_ids, pos, *[tok[x][s] for x in NAMES],
                           ds.pool, ds.ring, ys[i][s])
    torch.cuda.synchronize()
    for c, ds, y in zip(cases, states, ys):
        y_ref, S_ref, h_ref = oracle.decode_case(c)
        assert_parity(y.cpu().numpy(), y_ref, tol_for(c.state), f"{c.name} outputs")
        assert_parity(dev.read_states(ds), S_ref, tol_for(c.state), f"{c.name} states")
        np.testing.assert_array_equal(dev.read_window(ds, c.pos0 + steps), h_ref)


def test_negative_control_wrong_accepted_length_is_caught():
    """Committing one more (or one fewer) draft token than accepted must
    fail the committed-state check that the parity tests use."""
    need_gpu()
    case = wl.make_verify(130, B=4, H=2, dk=128, dv=128, n_draft=4, act="bf16", state="f32",
                          init="random", name="negative_control")
    case.accepted = np.array([2, 1, 3, 2], dtype=np.int32)
    _, _, S_ref, _ = oracle.verify_case(case)
    ds = dev.make_state(case)
    rec, dconv, _, slot_t, pos_t, _ = run_verify_gpu(case, ds)
    wrong = case.accepted.copy()
    wrong[1] += 1
    wrong[2] -= 1
    assert commit_gpu(case, ds, rec, dconv, slot_t, pos_t, wrong) == 0
    got = dev.read_states(ds)
    for b in (1, 2):
        assert rel_linf(got[b], S_ref[b]) > 100 * tol_for("f32"), f"row {b}: not caught"
    for b in (0, 3):
        assert rel_linf(got[b], S_ref[b]) <= tol_for("f32")


def test_prefill_is_bitwise_deterministic():
    torch = need_gpu()
    case = wl.make_prefill(131, lens=[300, 17, 129], H=4, dk=128, dv=128, act="bf16",
                           state="f32", init="random", slice_len=16, name="prefill_det")
    ds1, y1, s1 = run_prefill_gpu(case)
    ds2, y2, s2 = run_prefill_gpu(case)
    assert s1 == s2 == 0
    assert np.array_equal(y1, y2)
    assert torch.equal(ds1.pool.view(torch.uint8), ds2.pool.view(torch.uint8))
