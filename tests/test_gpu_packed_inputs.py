"""GPU parity with q, k, v and g read as column ranges of one packed
projection output (kda_shape.qkv_row_stride / g_row_stride): the same
results as contiguous inputs, bit for bit, and the oracle's."""
import numpy as np
import pytest

from gpu_util import assert_parity, need_gpu, tol_for
from kda_inputs import device as dev
from hybrid_linear_attention_rule_amd import kda
from kda_inputs import workloads as wl
from test_gpu_prefill import run_prefill_gpu
import oracle

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "alpha", "beta", "g")


def pack(tok, act, H, d, pad=8):
    """q | k | v | (g when it shares the dtype) | pad per token row, as one
    buffer, and views of it with the input shapes; the row strides used."""
    torch = need_gpu()
    q = tok["q"]
    lead = q.shape[:-2]
    rows = int(np.prod(lead))
    g_in = tok["g"].dtype == q.dtype
    W = (4 if g_in else 3) * H * d + pad
    buf = torch.full((rows, W), float("nan"), device="cuda").to(q.dtype)
    out = dict(tok)
    for i, name in enumerate(("q", "k", "v") + (("g",) if g_in else ())):
        buf[:, i * H * d:(i + 1) * H * d] = tok[name].reshape(rows, H * d)
        out[name] = buf[:, i * H * d:(i + 1) * H * d].view(*lead, H, d)
    g_rs = W
    if not g_in:                                   # FP8 inputs: g (BF16) on its own, strided
        g_rs = 2 * H * d
        gbuf = torch.full((rows, g_rs), float("nan"), device="cuda", dtype=tok["g"].dtype)
        gbuf[:, H * d:] = tok["g"].reshape(rows, H * d)
        out["g"] = gbuf[:, H * d:].view(*lead, H, d)
    return out, W, g_rs


@pytest.mark.parametrize("act,state", [("bf16", "f32"), ("fp8", "bf16"), ("f32", "f32")])
def test_decode_from_packed_projection(act, state):
    torch = need_gpu()
    case = wl.make_decode(101, B=5, H=3, dk=128, dv=128, steps=4, act=act, state=state,
                          init="random", name=f"decode_packed_{act}")
    outs = []
    for packed in (False, True):
        ds = dev.make_state(case)
        y = torch.full((case.steps, case.batch, case.H, case.dv), float("nan"), device="cuda")
        tok_all = dev.tokens_to_device(case.tokens, case.act)
        for s in range(case.steps):
            tok = {x: tok_all[x][s] for x in NAMES}
            if packed:
                tok, W, gW = pack(tok, case.act, case.H, case.dk)
                ds.shape.qkv_row_stride, ds.shape.g_row_stride = W, gW
            pos = torch.from_numpy((case.pos0 + s).astype(np.int32)).cuda()
            kda.decode(ds.shape, ds.params, ds.slot_ids, pos, *[tok[x] for x in NAMES],
                       ds.pool, ds.ring, y[s])
        torch.cuda.synchronize()
        outs.append((y, ds))
    (y0, ds0), (y1, ds1) = outs
    assert torch.equal(y0, y1) and torch.equal(ds0.pool.view(torch.uint8), ds1.pool.view(torch.uint8))
    y_ref, S_ref, _ = oracle.decode_case(case)
    assert_parity(y1.cpu().numpy(), y_ref, tol_for(state), "y")
    assert_parity(dev.read_states(ds1), S_ref, tol_for(state), "states")


def test_verify_commit_from_packed_projection():
    torch = need_gpu()
    case = wl.make_verify(102, B=4, H=2, dk=128, dv=128, n_draft=3, act="bf16", state="f32",
                          init="random", name="verify_packed")
    ds = dev.make_state(case)
    tok, W, gW = pack(dev.tokens_to_device(case.tokens, case.act), case.act, case.H, case.dk)
    ds.shape.qkv_row_stride, ds.shape.g_row_stride = W, gW
    B, n, H, d = case.batch, case.n_draft, case.H, case.dk
    rec = torch.empty((B, n, H, d, d), device="cuda")
    dconv = torch.empty((B, n, H, 3 * d), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((B, n, H, d), device="cuda")
    pos = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    kda.verify(ds.shape, ds.params, ds.slot_ids, pos, *[tok[x] for x in NAMES], ds.pool,
               ds.ring, rec, dconv, y)
    kda.commit_accepted(ds.shape, ds.slot_ids, pos, torch.from_numpy(case.accepted).cuda(),
                        rec, dconv, ds.pool, ds.ring)
    torch.cuda.synchronize()
    y_ref, rec_ref, S_ref, h_ref = oracle.verify_case(case)
    assert_parity(y.cpu().numpy(), y_ref, 2e-5, "y")
    assert_parity(rec.cpu().numpy(), rec_ref, 2e-5, "records")
    assert_parity(dev.read_states(ds), S_ref, 2e-5, "committed states")
    np.testing.assert_array_equal(dev.read_window(ds, case.pos0 + case.accepted), h_ref)


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_prefill_from_packed_projection(act):
    torch = need_gpu()
    case = wl.make_prefill(103, lens=[150, 1, 77], H=2, dk=128, dv=128, act=act, state="f32",
                           init="random", slice_len=32, name=f"prefill_packed_{act}")
    ds_c, y_c, st = run_prefill_gpu(case)
    assert st == 0
    ds = dev.make_state(case)
    tok, W, gW = pack(dev.tokens_to_device(case.tokens, case.act), case.act, case.H, case.dk)
    ds.shape.qkv_row_stride, ds.shape.g_row_stride = W, gW
    T = int(case.cu_seqlens[-1])
    y = torch.full((T, case.H, case.dv), float("nan"), device="cuda")
    ws = torch.empty(kda.prefill_workspace_bytes(ds.shape, case.batch, T), dtype=torch.uint8,
                     device="cuda")
    kda.prefill(ds.shape, ds.params, torch.from_numpy(case.cu_seqlens).cuda(), max(case.lens),
                ds.slot_ids, torch.from_numpy(case.pos0.astype(np.int32)).cuda(),
                *[tok[x] for x in NAMES], ds.pool, ds.ring, y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_c), "packed inputs must give the same outputs"
    assert torch.equal(ds.pool.view(torch.uint8), ds_c.pool.view(torch.uint8))
    assert torch.equal(ds.ring.view(torch.uint8), ds_c.ring.view(torch.uint8))
    y_ref, S_ref, _ = oracle.prefill_case(case)
    assert_parity(y.cpu().numpy(), y_ref, 2e-5, "y")
    assert_parity(dev.read_states(ds), S_ref, 2e-5, "states")
