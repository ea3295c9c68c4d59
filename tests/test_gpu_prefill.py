"""GPU parity of kda_prefill (chunkwise WY/UT form on the matrix cores)
against the CPU oracle's token-by-token recurrence."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
import oracle

pytestmark = pytest.mark.gpu


def run_prefill_gpu(case, ds=None, *, slots=None, max_seqlen=None, cu=None, q_scale=1.0):
    torch = need_gpu()
    ds = dev.make_state(case, q_scale=q_scale) if ds is None else ds
    tok = dev.tokens_to_device(case.tokens, case.act)
    T = int(case.cu_seqlens[-1])
    y = torch.full((T, case.H, case.dv), float("nan"), device="cuda")
    slots = ds.slots if slots is None else slots
    slot_t = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    cu_t = torch.from_numpy(np.asarray(case.cu_seqlens if cu is None else cu,
                                       dtype=np.int32)).cuda()
    nbytes = kda.prefill_workspace_bytes(ds.shape, case.batch, T)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mx = max(case.lens) if max_seqlen is None else max_seqlen
    kda.prefill(ds.shape, ds.params, cu_t, mx, slot_t, pos_t, tok["q"], tok["k"],
                tok["v"], tok["alpha"], tok["beta"], tok["g"], ds.pool, ds.ring, y, ws,
                status)
    torch.cuda.synchronize()
    return ds, y.cpu().numpy(), int(status.item())


def check_prefill(case, *, full_outputs=True, q_scale=1.0):
    print(f"case {case.name}: lens={case.lens} H={case.H} d={case.dk} act={case.act} "
          f"state={case.state} q_scale={q_scale}", flush=True)
    ds, y, status = run_prefill_gpu(case, q_scale=q_scale)
    assert status == 0
    y_ref, S_ref, h_ref = oracle.prefill_case(case, q_scale=q_scale)
    tol = tol_for(case.state)
    assert_parity(dev.read_states(ds), S_ref, tol, "final states")
    if full_outputs:
        assert_parity(y, y_ref, 2e-5, "all outputs")
    lo = int(case.cu_seqlens[case.slice_seq]) + case.slice_start
    sl = slice(lo, lo + case.slice_len)
    assert_parity(y[sl], y_ref[sl], 2e-5, f"{case.slice_len}-token output slice")
    end_pos = case.pos0 + np.asarray(case.lens)
    np.testing.assert_array_equal(dev.read_window(ds, end_pos), h_ref)
    spare = np.setdiff1d(np.arange(ds.num_slots), ds.slots)
    assert np.all(np.isnan(ds.pool[spare].float().cpu().numpy()))
    return ds


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 130], [200, 3, 2]])
def test_prefill_ragged_lengths(lens):
    need_gpu()
    case = wl.make_prefill(70 + len(lens), lens=lens, H=3, dk=128, dv=128, act="bf16",
                           state="f32", slice_len=32, name=f"prefill_ragged_{len(lens)}")
    check_prefill(case)


@pytest.mark.parametrize("act,state", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_prefill_dtypes(act, state):
    need_gpu()
    case = wl.make_prefill(80, lens=[150, 77], H=2, dk=128, dv=128, act=act, state=state,
                           slice_len=32, name=f"prefill_{act}_{state}")
    check_prefill(case)


def test_prefill_continues_from_stored_state_and_history():
    """positions > 0: the chunk pass reads the ring for the first tokens and
    the state pass starts from the stored state."""
    need_gpu()
    case = wl.make_prefill(81, lens=[70, 5, 129], H=2, dk=128, dv=128, act="bf16",
                           state="f32", init="random", slice_len=32,
                           name="prefill_continued")
    check_prefill(case)


@pytest.mark.parametrize("act", ["f32", "bf16", "fp8"])
def test_prefill_from_positions_zero_one_two(act):
    """Start positions 0, 1 and 2: the conv taps before position 0 count as
    zero (the ring holds NaN there) and the later ones come from the ring;
    lengths 1-3 also leave raw taps past the chunk's end in the same lanes."""
    need_gpu()
    case = wl.make_prefill(87, lens=[1, 2, 3, 70, 65, 5, 2], H=2, dk=128, dv=128, act=act,
                           state="f32", init="random", slice_len=32,
                           name=f"prefill_short_history_{act}")
    case.pos0[:] = [1, 2, 1, 2, 0, 1, 0]
    for b, p in enumerate(case.pos0):
        if p == 0:
            case.S0[b] = 0.0               # position 0 starts from the zero state
        for j in range(case.width - 1):
            if p - (case.width - 1) + j < 0:
                case.hist0[b, j] = 0.0     # no token before position 0
    check_prefill(case)


def test_prefill_strong_decay_stays_finite():
    """Decays down to alpha ~ e^-12 per token: the factorised exponentials
    stay <= 1, nothing overflows."""
    need_gpu()
    case = wl.make_prefill(82, lens=[128, 64], H=2, dk=128, dv=128, act="f32",
                           state="f32", slice_len=32, name="prefill_strong_decay")
    rng = np.random.default_rng(5)
    case.tokens.alpha[:] = wl.round_f32(np.exp(-rng.uniform(0.0, 12.0,
                                                            case.tokens.alpha.shape)))
    check_prefill(case)


@pytest.mark.parametrize("ev,es,state", [(-12, -12, "f32"), (12, 12, "f32"),
                                         (-24, -24, "f32"), (24, 24, "f32"),
                                         (12, -12, "f32"), (-3, 3, "f32"),
                                         (12, 12, "bf16")])
def test_prefill_value_and_state_magnitudes(ev, es, state):
    """v (and the v channels of the stored history) scaled by 2^ev and the
    stored start state by 2^es, exactly (powers of two).  The recurrence
    takes them at any magnitude; the prefill's split matrix-core operands
    keep FP32-level accuracy on the value side whatever the common
    magnitude is, with a start state much smaller than the values, and with
    one up to 2^6 larger (the stated domain allows about 2^9 between the
    largest write of a chunk and the ones that set its result)."""
    need_gpu()
    case = wl.make_prefill(88, lens=[200, 64, 37], H=2, dk=128, dv=128, act="bf16",
                           state=state, init="random", slice_len=32,
                           name=f"prefill_magnitudes_v{ev}_s{es}_{state}")
    case.tokens.v[:] *= 2.0 ** ev
    case.hist0[..., 2 * case.dk:] *= 2.0 ** ev
    case.S0[:] *= 2.0 ** es
    if state == "bf16":
        case.S0[:] = wl.round_bf16(case.S0)
    check_prefill(case)


def test_prefill_near_collinear_keys_full_writes():
    """Keys of one sequence and head all close to one direction (head 0) or
    to one direction with alternating sign (head 1), beta close to 1 and no
    decay: A is close to a block of ones (or of alternating signs) under the
    diagonal, the hardest case for the diagonal inverses T_bb and for W."""
    need_gpu()
    case = wl.make_prefill(89, lens=[192, 80, 17], H=2, dk=128, dv=128, act="f32",
                           state="f32", init="random", slice_len=32,
                           name="prefill_collinear_keys")
    rng = np.random.default_rng(9)
    k = case.tokens.k                         # [T, H, dk]
    T = k.shape[0]
    sign = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
    for h in range(case.H):
        base = rng.standard_normal(case.dk)
        noise = 1e-3 * rng.standard_normal((T, case.dk))
        k[:, h] = (sign[:, None] if h == 1 else 1.0) * base[None, :] + noise
    case.tokens.k[:] = wl.round_f32(k)
    case.tokens.beta[:] = wl.round_f32(np.full_like(case.tokens.beta, 0.999))
    case.tokens.alpha[:] = 1.0
    case.hist0[..., case.dk:2 * case.dk] = 0.0   # history keys do not spoil the first block
    check_prefill(case)


@pytest.mark.parametrize("q_scale", [0.08838834764831845, 40.0])
def test_prefill_query_scale(q_scale):
    """A query scale other than 1 (1/sqrt(dk), and a large one): the prefill
    applies it to the read-outs, and the outputs match the oracle's."""
    need_gpu()
    case = wl.make_prefill(90, lens=[130, 7], H=2, dk=128, dv=128, act="bf16", state="f32",
                           init="random", slice_len=32, name=f"prefill_q_scale_{q_scale:g}")
    check_prefill(case, q_scale=q_scale)


def test_prefill_many_sequences_several_items_per_workgroup():
    """37 sequences of 1..300 tokens over 16 heads continuing stored states:
    more chunk items than workgroups, so each workgroup runs several items
    and prefetches the next one's inputs; first, interior and partial chunks
    mix, and the unused slot between sequences is skipped."""
    need_gpu()
    rng = np.random.default_rng(37)
    lens = [int(x) for x in rng.integers(1, 301, 37)]
    case = wl.make_prefill(84, lens=lens, H=16, dk=128, dv=128, act="bf16", state="f32",
                           init="random", slice_len=64, name="prefill_many_seqs")
    check_prefill(case, full_outputs=True)


@pytest.mark.parametrize("act", ["f32", "fp8"])
def test_prefill_several_items_per_workgroup_other_inputs(act):
    """FP32 and FP8 inputs with more chunk items than workgroups: each
    workgroup requests the next item's inputs (q, k and v/alpha/beta at
    three different steps) while it works on the current one."""
    need_gpu()
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 301, 24)]
    case = wl.make_prefill(95, lens=lens, H=8, dk=128, dv=128, act=act, state="f32",
                           init="random", slice_len=64, name=f"prefill_many_seqs_{act}")
    check_prefill(case, full_outputs=True)


def test_prefill_inactive_and_bad_rows_among_many():
    """Inactive sequences scattered among active ones are untouched, a bad
    slot is reported once and skipped, and the others still match."""
    torch = need_gpu()
    lens = [70, 1, 200, 64, 3, 129, 40, 90]
    case = wl.make_prefill(85, lens=lens, H=4, dk=128, dv=128, act="bf16", state="f32",
                           init="random", slice_len=32, name="prefill_mixed_rows")
    ds = dev.make_state(case)
    slots = ds.slots.copy()
    skip = [1, 4, 6]
    keep_pool = {i: ds.pool[ds.slots[i]].clone() for i in skip}
    slots[1] = -1
    slots[4] = -1
    slots[6] = ds.num_slots + 5            # out of range: reported and skipped
    ds, y, status = run_prefill_gpu(case, ds, slots=slots)
    assert status == kda.STATUS_BAD_SLOT
    y_ref, S_ref, _ = oracle.prefill_case(case)
    got = dev.read_states(ds)
    cu = case.cu_seqlens
    for i in range(len(lens)):
        rows = slice(int(cu[i]), int(cu[i + 1]))
        if i in skip:
            assert np.isnan(y[rows]).all()
            assert torch.equal(ds.pool[ds.slots[i]].view(torch.uint8),
                               keep_pool[i].view(torch.uint8))
        else:
            assert_parity(got[i], S_ref[i], tol_for(case.state), f"state of sequence {i}")
            assert_parity(y[rows], y_ref[rows], 2e-5, f"outputs of sequence {i}")


def test_config4_chunked_prefill():
    need_gpu()
    check_prefill(wl.config(4))


def test_prefill_bad_seqlens_and_inactive_sequences():
    torch = need_gpu()
    case = wl.make_prefill(83, lens=[40, 30], H=2, dk=128, dv=128, act="bf16",
                           state="f32", slice_len=8, name="prefill_bad")
    # sequence 1 inactive: untouched; sequence 0 checked
    ds = dev.make_state(case)
    slots = ds.slots.copy()
    slots[1] = -1
    pool1 = ds.pool[ds.slots[1]].clone()
    ds, y, status = run_prefill_gpu(case, ds, slots=slots)
    assert status == 0
    assert np.isnan(y[40:]).all()
    assert torch.equal(ds.pool[ds.slots[1]].view(torch.uint8), pool1.view(torch.uint8))
    # non-monotone cu_seqlens: reported, that sequence skipped
    ds = dev.make_state(case)
    pool0 = ds.pool.clone()
    ds, y, status = run_prefill_gpu(case, ds, cu=[0, 50, 40])
    assert status & kda.STATUS_BAD_SEQLENS
    # a sequence longer than max_seqlen is reported too
    ds = dev.make_state(case)
    ds, y, status = run_prefill_gpu(case, ds, max_seqlen=32)
    assert status & kda.STATUS_BAD_SEQLENS


def test_mixed_launch_decode_rows_as_length_one_sequences():
    """One kda_prefill launch that mixes decode rows (length-1 sequences
    continuing a stored state and history) with multi-chunk sequences: every
    row matches the oracle, and each decode row also matches kda_decode of
    the same token from the same start."""
    torch = need_gpu()
    lens = [1, 200, 1, 1, 70, 1]
    case = wl.make_prefill(86, lens=lens, H=4, dk=128, dv=128, act="bf16", state="f32",
                           init="random", slice_len=32, name="prefill_mixed_decode_rows")
    ds_p = check_prefill(case)
    _, y_p, _ = run_prefill_gpu(case)          # fresh state, same launch again
    singles = [i for i, n in enumerate(lens) if n == 1]
    cu = case.cu_seqlens
    ds_d = dev.make_state(case)
    slots = np.where(np.asarray(lens) == 1, ds_d.slots, -1).astype(np.int32)
    tok = dev.tokens_to_device(case.tokens, case.act)
    first = torch.from_numpy(cu[:-1].astype(np.int64)).cuda()
    rows = {k: t.index_select(0, first).contiguous() for k, t in tok.items()}
    y_d = torch.full((len(lens), case.H, case.dv), float("nan"), device="cuda")
    kda.decode(ds_d.shape, ds_d.params, torch.from_numpy(slots).cuda(),
               torch.from_numpy(case.pos0.astype(np.int32)).cuda(), rows["q"], rows["k"],
               rows["v"], rows["alpha"], rows["beta"], rows["g"], ds_d.pool, ds_d.ring, y_d)
    torch.cuda.synchronize()
    y_d = y_d.cpu().numpy()
    S_p = dev.read_states(ds_p)
    S_d = dev.read_states(ds_d)
    for i in singles:
        assert_parity(y_d[i], y_p[int(cu[i])], 2e-5, f"decode row {i}: output")
        assert_parity(S_d[i], S_p[i], 2e-5, f"decode row {i}: state")
    np.testing.assert_array_equal(dev.read_window(ds_d, case.pos0 + 1)[singles],
                                  dev.read_window(ds_p, case.pos0 + 1)[singles])
