"""HIP-graph capture and replay of decode, verify, commit and prefill.

The calls read slots, positions, accepted lengths and token inputs on the
device, so one captured call replays correctly after those buffers are
rewritten in place.  Each replay is checked bitwise against the same call run
eagerly, with eager work (the input copies) between replays."""
import numpy as np
import pytest

from gpu_util import need_gpu
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "alpha", "beta", "g")


def _bits(t):
    return t.contiguous().view(-1).view(dtype=__import__("torch").uint8)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_decode_graph_replay_matches_eager(state):
    torch = need_gpu()
    case = wl.make_decode(60, B=8, H=4, dk=128, dv=128, steps=6, act="bf16",
                          state=state, init="random", active_per_step=6,
                          name=f"graph_decode_{state}")
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, H, dv = case.batch, case.H, case.dv
    pos = np.zeros((case.steps + 1, B), dtype=np.int64)
    pos[0] = case.pos0
    for s in range(case.steps):
        pos[s + 1] = pos[s] + case.active[s]

    def step_slots(ds, s):
        return torch.from_numpy(np.where(case.active[s], ds.slots, -1)
                                .astype(np.int32)).cuda()

    # eager
    ds_e = dev.make_state(case)
    ys_e = []
    for s in range(case.steps):
        y = torch.full((B, H, dv), float("nan"), device="cuda")
        kda.decode(ds_e.shape, ds_e.params, step_slots(ds_e, s),
                   torch.from_numpy(pos[s].astype(np.int32)).cuda(),
                   *[tok[n][s] for n in NAMES], ds_e.pool, ds_e.ring, y)
        ys_e.append(y)
    torch.cuda.synchronize()

    # captured once, replayed per step with the inputs rewritten in place
    ds_g = dev.make_state(case)
    slot_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    pos_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    in_buf = {n: torch.empty_like(tok[n][0]) for n in NAMES}
    y_buf = torch.full((B, H, dv), float("nan"), device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        kda.decode(ds_g.shape, ds_g.params, slot_buf, pos_buf,
                   *[in_buf[n] for n in NAMES], ds_g.pool, ds_g.ring, y_buf)
    torch.cuda.synchronize()
    for s in range(case.steps):
        slot_buf.copy_(step_slots(ds_g, s))
        pos_buf.copy_(torch.from_numpy(pos[s].astype(np.int32)))
        for n in NAMES:
            in_buf[n].copy_(tok[n][s])
        y_buf.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_buf), _bits(ys_e[s])), f"replay {s}: y differs"
    assert torch.equal(_bits(ds_g.pool), _bits(ds_e.pool))
    assert torch.equal(_bits(ds_g.ring), _bits(ds_e.ring))


def test_verify_commit_graph_replay_matches_eager():
    torch = need_gpu()
    n = 4
    cases = [wl.make_verify(61 + i, B=6, H=4, dk=128, dv=128, n_draft=n, act="bf16",
                            state="f32", init="random", name=f"graph_verify_{i}")
             for i in range(3)]
    base = cases[0]
    B, H, dk, dv = base.batch, base.H, base.dk, base.dv
    C = 2 * dk + dv

    def fresh():
        return dev.make_state(base)

    # eager: three rounds of verify + commit on one pool, each round with its
    # own drafts and accepted lengths; positions advance by the accepted count
    ds_e = fresh()
    pos = base.pos0.astype(np.int64).copy()
    outs_e = []
    for c in cases:
        tok = dev.tokens_to_device(c.tokens, c.act)
        rec = torch.empty((B, n, H, dk, dv), device="cuda")
        dconv = torch.empty((B, n, H, C), device="cuda", dtype=torch.bfloat16)
        y = torch.empty((B, n, H, dv), device="cuda")
        p_t = torch.from_numpy(pos.astype(np.int32)).cuda()
        kda.verify(ds_e.shape, ds_e.params, ds_e.slot_ids, p_t,
                   *[tok[x] for x in NAMES], ds_e.pool, ds_e.ring, rec, dconv, y)
        kda.commit_accepted(ds_e.shape, ds_e.slot_ids, p_t,
                            torch.from_numpy(c.accepted).cuda(), rec, dconv,
                            ds_e.pool, ds_e.ring)
        outs_e.append((y, rec))
        pos += c.accepted
    torch.cuda.synchronize()

    ds_g = fresh()
    pos = base.pos0.astype(np.int64).copy()
    pos_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    acc_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    tok0 = dev.tokens_to_device(base.tokens, base.act)
    in_buf = {x: torch.empty_like(tok0[x]) for x in NAMES}
    rec = torch.empty((B, n, H, dk, dv), device="cuda")
    dconv = torch.empty((B, n, H, C), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((B, n, H, dv), device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        kda.verify(ds_g.shape, ds_g.params, ds_g.slot_ids, pos_buf,
                   *[in_buf[x] for x in NAMES], ds_g.pool, ds_g.ring, rec, dconv, y)
        kda.commit_accepted(ds_g.shape, ds_g.slot_ids, pos_buf, acc_buf, rec, dconv,
                            ds_g.pool, ds_g.ring)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        tok = dev.tokens_to_device(c.tokens, c.act)
        for x in NAMES:
            in_buf[x].copy_(tok[x])
        pos_buf.copy_(torch.from_numpy(pos.astype(np.int32)))
        acc_buf.copy_(torch.from_numpy(c.accepted))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(outs_e[i][0])), f"replay {i}: y differs"
        assert torch.equal(_bits(rec), _bits(outs_e[i][1])), f"replay {i}: records"
        pos += c.accepted
    assert torch.equal(_bits(ds_g.pool), _bits(ds_e.pool))
    assert torch.equal(_bits(ds_g.ring), _bits(ds_e.ring))


def test_records_free_verify_and_recompute_graph_replay_matches_eager():
    """verify without records + kda_commit_recompute captured once and
    replayed for three rounds with drafts, positions and accepted lengths
    rewritten in place: every replay matches the eager records path."""
    torch = need_gpu()
    n = 4
    cases = [wl.make_verify(71 + i, B=6, H=4, dk=128, dv=128, n_draft=n, act="bf16",
                            state="bf16", init="random", name=f"graph_recompute_{i}")
             for i in range(3)]
    base = cases[0]
    B, H, dk, dv = base.batch, base.H, base.dk, base.dv
    C = 2 * dk + dv

    ds_e = dev.make_state(base)
    pos = base.pos0.astype(np.int64).copy()
    ys_e = []
    for c in cases:
        tok = dev.tokens_to_device(c.tokens, c.act)
        rec = torch.empty((B, n, H, dk, dv), device="cuda")
        dconv = torch.empty((B, n, H, C), device="cuda", dtype=torch.bfloat16)
        y = torch.empty((B, n, H, dv), device="cuda")
        p_t = torch.from_numpy(pos.astype(np.int32)).cuda()
        kda.verify(ds_e.shape, ds_e.params, ds_e.slot_ids, p_t,
                   *[tok[x] for x in NAMES], ds_e.pool, ds_e.ring, rec, dconv, y)
        kda.commit_accepted(ds_e.shape, ds_e.slot_ids, p_t,
                            torch.from_numpy(c.accepted).cuda(), rec, dconv,
                            ds_e.pool, ds_e.ring)
        ys_e.append(y)
        pos += c.accepted
    torch.cuda.synchronize()

    ds_g = dev.make_state(base)
    pos = base.pos0.astype(np.int64).copy()
    pos_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    acc_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    tok0 = dev.tokens_to_device(base.tokens, base.act)
    in_buf = {x: torch.empty_like(tok0[x]) for x in NAMES}
    y = torch.empty((B, n, H, dv), device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        kda.verify(ds_g.shape, ds_g.params, ds_g.slot_ids, pos_buf,
                   *[in_buf[x] for x in NAMES], ds_g.pool, ds_g.ring, None, None, y)
        kda.commit_recompute(ds_g.shape, ds_g.params, ds_g.slot_ids, pos_buf, acc_buf,
                             *[in_buf[x] for x in NAMES], ds_g.pool, ds_g.ring)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        tok = dev.tokens_to_device(c.tokens, c.act)
        for x in NAMES:
            in_buf[x].copy_(tok[x])
        pos_buf.copy_(torch.from_numpy(pos.astype(np.int32)))
        acc_buf.copy_(torch.from_numpy(c.accepted))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ys_e[i])), f"replay {i}: y differs"
        pos += c.accepted
    assert torch.equal(_bits(ds_g.pool), _bits(ds_e.pool))
    assert torch.equal(_bits(ds_g.ring), _bits(ds_e.ring))


def test_prefill_graph_replay_with_new_lengths_matches_eager():
    """kda_prefill captured once (host sizes: 3 sequences, 180 tokens,
    lengths at most 128) and replayed with cu_seqlens, tokens and start
    states rewritten in place: the sequence lengths change between replays
    and every replay equals the eager call bit for bit."""
    torch = need_gpu()
    splits = [[100, 50, 30], [60, 90, 30], [1, 128, 51]]
    cases = [wl.make_prefill(81 + i, lens=l, H=2, dk=128, dv=128, act="bf16", state="f32",
                             init="random", slice_len=16, name=f"graph_prefill_{i}")
             for i, l in enumerate(splits)]
    for c in cases[1:]:
        c.weights = cases[0].weights      # one layer: the captured call's weights
    T, B, H, dv, mx = 180, 3, 2, 128, 128
    nbytes = kda.prefill_workspace_bytes(dev.shape_of(cases[0]), B, T)

    def eager(c):
        ds = dev.make_state(c)
        tok = dev.tokens_to_device(c.tokens, c.act)
        y = torch.full((T, H, dv), float("nan"), device="cuda")
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        kda.prefill(ds.shape, ds.params, torch.from_numpy(c.cu_seqlens).cuda(), mx,
                    ds.slot_ids, torch.from_numpy(c.pos0.astype(np.int32)).cuda(),
                    *[tok[x] for x in NAMES], ds.pool, ds.ring, y, ws)
        torch.cuda.synchronize()
        return ds, y

    outs = [eager(c) for c in cases]

    ds_g = dev.make_state(cases[0])
    tok0 = dev.tokens_to_device(cases[0].tokens, cases[0].act)
    in_buf = {x: torch.empty_like(tok0[x]) for x in NAMES}
    cu_buf = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    pos_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    y = torch.empty((T, H, dv), device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        kda.prefill(ds_g.shape, ds_g.params, cu_buf, mx, ds_g.slot_ids, pos_buf,
                    *[in_buf[x] for x in NAMES], ds_g.pool, ds_g.ring, y, ws)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        start = dev.make_state(c)                     # this case's start state
        ds_g.pool.copy_(start.pool)
        ds_g.ring.copy_(start.ring)
        tok = dev.tokens_to_device(c.tokens, c.act)
        for x in NAMES:
            in_buf[x].copy_(tok[x])
        cu_buf.copy_(torch.from_numpy(c.cu_seqlens))
        pos_buf.copy_(torch.from_numpy(c.pos0.astype(np.int32)))
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ds_e, y_e = outs[i]
        assert torch.equal(_bits(y), _bits(y_e)), f"replay {i}: y differs"
        assert torch.equal(_bits(ds_g.pool), _bits(ds_e.pool)), f"replay {i}: states differ"
        assert torch.equal(_bits(ds_g.ring), _bits(ds_e.ring)), f"replay {i}: ring differs"
