"""Pins of the CPU oracle against facts that do not come from its own code.

Each test is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a transposed state, a reversed conv tap, a read-out before the
write, a sum where a mean belongs, a gate applied before the norm) fails at
least one of them.  All run on the CPU in fp64.
"""
import os

import numpy as np
import pytest

from oracle import ref
from oracle.ref import OracleCfg
from kda_inputs import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = line.split("=", 1)
            vals[key.strip()] = np.array([float(x) for x in rhs.split()])
    return vals


def _identity_taps(n, W=4):
    w = np.zeros((n, W))
    w[:, W - 1] = 1.0
    return w


def _rand_stream(rng, T, dk, dv, *, beta_lo=0.0):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    alpha = np.exp(-np.logaddexp(0.0, rng.standard_normal((T, dk))))
    beta = rng.uniform(beta_lo, 1.0, T)
    g = rng.standard_normal((T, dv))
    return q, k, v, alpha, beta, g


def _run(cfg, S0, hist0, stream, wconv, norm_w=None, **kw):
    S = np.array(S0, dtype=np.float64, order="C", copy=True)
    h = np.array(hist0, dtype=np.float64, order="C", copy=True)
    y, rec = ref.run_one(cfg, S, h, *stream, np.ascontiguousarray(wconv,
                         dtype=np.float64),
                         None if norm_w is None else np.ascontiguousarray(norm_w, float),
                         **kw)
    return S, h, y, rec


# ----------------------------------------------------------------- golden

def test_golden_hand_worked_three_tokens():
    gd = _read_golden("hand_three_tokens.txt")
    cfg = OracleCfg(2, 2, 4, "sigmoid", 1.0, 0.0, 0.0)
    T = 3
    stream = (gd["q"].reshape(T, 2), gd["k"].reshape(T, 2),
              gd["v"].reshape(T, 2), gd["alpha"].reshape(T, 2), gd["beta"],
              gd["g"].reshape(T, 2))
    S, _, y, rec = _run(cfg, np.zeros((2, 2)), np.zeros((3, 6)), stream,
                        _identity_taps(6), np.ones(2), want_records=True)
    for t in range(3):
        np.testing.assert_allclose(rec[t].ravel(), gd[f"S{t + 1}"],
                                   rtol=0, atol=1e-15)
        np.testing.assert_allclose(y[t], gd[f"y{t + 1}"], rtol=1e-14,
                                   atol=1e-15)


def test_golden_query_scale():
    gd = _read_golden("q_scale_two_tokens.txt")
    cfg = OracleCfg(2, 2, 4, "sigmoid", float(gd["q_scale"][0]),
                    float(gd["l2_eps"][0]), float(gd["norm_eps"][0]))
    T = 2
    stream = (gd["q"].reshape(T, 2), gd["k"].reshape(T, 2),
              gd["v"].reshape(T, 2), gd["alpha"].reshape(T, 2), gd["beta"],
              gd["g"].reshape(T, 2))
    S, _, y, rec = _run(cfg, gd["S0"].reshape(2, 2), np.zeros((3, 6)), stream,
                        _identity_taps(6), np.ones(2), want_records=True)
    for t in range(T):
        np.testing.assert_allclose(rec[t].ravel(), gd[f"S{t + 1}"],
                                   rtol=0, atol=1e-15)
        np.testing.assert_allclose(y[t], gd[f"y{t + 1}"], rtol=1e-14,
                                   atol=1e-15)
    # the chunkwise form applies the same scale
    y_c = ref.run_one_chunked(cfg, 2, gd["S0"].reshape(2, 2).copy(),
                              np.zeros((3, 6)), *stream,
                              _identity_taps(6).astype(np.float64), np.ones(2))
    np.testing.assert_allclose(y_c, y, rtol=1e-13, atol=1e-15)


def test_golden_conv_taps():
    gd = _read_golden("conv_taps.txt")
    cfg = OracleCfg(1, 1, 4, "sigmoid", 1.0, 0.0, 0.0)
    T = 5
    w = _identity_taps(3)
    w[2] = gd["w_v"]
    ones = np.ones((T, 1))
    stream = (ones, ones, gd["v"].reshape(T, 1), ones, np.ones(T),
              np.zeros((T, 1)))
    _, hist, _, rec = _run(cfg, np.zeros((1, 1)), np.zeros((3, 3)), stream,
                           w, want_records=True)
    np.testing.assert_array_equal(rec.ravel(), gd["S"])
    np.testing.assert_array_equal(hist[:, 2], gd["hist_v"])


# -------------------------------------------------------- bf16 rounding

def test_bf16_rounding_hand_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even one
    assert ref.bf16(1.0 + 2.0 ** -8) == 1.0
    assert ref.bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert ref.bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert ref.bf16(-(1.0 + 2.0 ** -8)) == -1.0
    assert ref.bf16(0.0) == 0.0
    assert ref.bf16(3.0) == 3.0


def test_fp8_e4m3_rounding_matches_torch():
    """The generator's E4M3 rounding (ties to even, subnormals below 2^-6,
    saturation at 448) against torch's float8_e4m3fn cast, on float32
    inputs across the whole finite range, exact ties included."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = rng.standard_normal(50000) * np.exp2(rng.uniform(-12, 9, 50000))
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    vals = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    ties = (vals[:-1] + vals[1:]) / 2.0                  # halfway between neighbours
    x = wl.round_f32(np.concatenate([x, ties, -ties, vals, -vals]))
    x = x[np.abs(x) <= 448.0]
    got = wl.round_e4m3(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(got, want)
    assert wl.round_e4m3(np.array([1000.0, -460.0]))[0] == 448.0


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x32 = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(
        -20, 20, 20000)]).astype(np.float32)
    # exact ties too: values with bit 15 set and bits 0..14 clear
    u = x32.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, ties])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = ref.round_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("dk,dv", [(8, 8), (6, 10), (12, 4)])
def test_beta0_alpha1_leaves_state_and_reads_rows(dk, dv):
    rng = np.random.default_rng(1)
    cfg = OracleCfg(dk, dv, 4, "sigmoid", 1.0, 0.0, 0.0)
    S0 = rng.standard_normal((dk, dv))
    T = 5
    q = np.zeros((T, dk))
    q[np.arange(T), np.arange(T) % dk] = 2.0     # qh = e_i
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g = rng.standard_normal((T, dv))
    stream = (q, k, v, np.ones((T, dk)), np.zeros(T), g)
    S, _, y, _ = _run(cfg, S0, np.zeros((3, 2 * dk + dv)), stream,
                      _identity_taps(2 * dk + dv))
    np.testing.assert_array_equal(S, S0)
    for t in range(T):
        o = S0[t % dk]                               # S^T e_i = row i
        want = o / np.sqrt(np.mean(o * o)) / (1.0 + np.exp(-g[t]))
        np.testing.assert_allclose(y[t], want, rtol=1e-13)


@pytest.mark.parametrize("dk,dv", [(5, 7), (8, 3)])
def test_brute_force_matrix_form(dk, dv):
    """Explicit dk x dk products (I - b k k^T) Diag(a) applied to S, with the
    conv done by numpy's convolve and the norms by numpy.linalg."""
    rng = np.random.default_rng(2)
    W, T = 4, 9
    cfg = OracleCfg(dk, dv, W, "sigmoid", 1.0, 1e-6, 1e-6)
    q, k, v, alpha, beta, g = _rand_stream(rng, T, dk, dv)
    wconv = rng.normal(0, 0.5, (2 * dk + dv, W))
    norm_w = rng.uniform(0.5, 1.5, dv)
    S0 = rng.normal(0, 0.1, (dk, dv))
    _, _, y, rec = _run(cfg, S0, np.zeros((W - 1, 2 * dk + dv)),
                        (q, k, v, alpha, beta, g), wconv, norm_w,
                        want_records=True)

    raw = np.concatenate([q, k, v], axis=1)
    conv = np.stack([np.convolve(raw[:, ch], wconv[ch, ::-1])[:T]
                     for ch in range(2 * dk + dv)], axis=1)
    S = S0.copy()
    for t in range(T):
        cq, ck, cv = conv[t, :dk], conv[t, dk:2 * dk], conv[t, 2 * dk:]
        kh = ck / np.sqrt(np.linalg.norm(ck) ** 2 + 1e-6)
        qh = cq / np.sqrt(np.linalg.norm(cq) ** 2 + 1e-6)
        M = (np.eye(dk) - beta[t] * np.outer(kh, kh)) @ np.diag(alpha[t])
        S = M @ S + beta[t] * np.outer(kh, cv)
        o = S.T @ qh
        yy = norm_w * o / np.sqrt(np.mean(o ** 2) + 1e-6) / (1 + np.exp(-g[t]))
        np.testing.assert_allclose(rec[t], S, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(y[t], yy, rtol=1e-11, atol=1e-13)


def test_delta_write_identity():
    """S'^T kh = (1 - b|kh|^2) (Diag(a) S)^T kh + b |kh|^2 vt."""
    rng = np.random.default_rng(3)
    dk, dv = 7, 5
    cfg = OracleCfg(dk, dv, 4, "sigmoid", 1.0, 0.5, 1e-6)   # |kh| < 1
    S0 = rng.standard_normal((dk, dv))
    q, k, v, alpha, beta, g = _rand_stream(rng, 1, dk, dv)
    _, _, _, rec = _run(cfg, S0, np.zeros((3, 2 * dk + dv)),
                        (q, k, v, alpha, beta, g), _identity_taps(2 * dk + dv),
                        want_records=True)
    kh = k[0] / np.sqrt(k[0] @ k[0] + 0.5)
    n2 = kh @ kh
    lhs = rec[0].T @ kh
    rhs = (1 - beta[0] * n2) * ((alpha[0][:, None] * S0).T @ kh) + \
        beta[0] * n2 * v[0]
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


def test_linearity_in_state_and_values():
    rng = np.random.default_rng(4)
    dk, dv, T = 6, 4, 7
    cfg = OracleCfg(dk, dv)
    q, k, v1, alpha, beta, g = _rand_stream(rng, T, dk, dv)
    v2 = rng.standard_normal((T, dv))
    S1, S2 = rng.standard_normal((2, dk, dv))
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    h0 = np.zeros((3, 2 * dk + dv))
    a, b = 0.7, -1.3
    r1 = _run(cfg, S1, h0, (q, k, v1, alpha, beta, g), w)[0]
    r2 = _run(cfg, S2, h0, (q, k, v2, alpha, beta, g), w)[0]
    r3 = _run(cfg, a * S1 + b * S2, h0,
              (q, k, a * v1 + b * v2, alpha, beta, g), w)[0]
    np.testing.assert_allclose(r3, a * r1 + b * r2, rtol=1e-12, atol=1e-12)


def test_value_columns_independent():
    rng = np.random.default_rng(5)
    dk, dv, T = 6, 8, 6
    cols = [1, 4, 5]
    q, k, v, alpha, beta, g = _rand_stream(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    h0 = np.zeros((3, 2 * dk + dv))
    full = _run(OracleCfg(dk, dv), S0, h0, (q, k, v, alpha, beta, g), w,
                want_records=True)[3]
    wsub = np.concatenate([w[:2 * dk], w[2 * dk:][cols]])
    sub = _run(OracleCfg(dk, len(cols)), S0[:, cols],
               np.zeros((3, 2 * dk + len(cols))),
               (q, k, v[:, cols], alpha, beta, g[:, cols]), wsub,
               want_records=True)[3]
    np.testing.assert_array_equal(full[:, :, cols], sub)


def test_contraction_bound():
    rng = np.random.default_rng(6)
    dk, dv, T = 8, 6, 40
    cfg = OracleCfg(dk, dv, 4, "sigmoid", 1.0, 1e-6, 1e-6)
    q, k, v, alpha, beta, g = _rand_stream(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv)) * 3
    _, _, _, rec = _run(cfg, S0, np.zeros((3, 2 * dk + dv)),
                        (q, k, v, alpha, beta, g), _identity_taps(2 * dk + dv),
                        want_records=True)
    prev = np.linalg.norm(S0, 2)
    for t in range(T):
        cur = np.linalg.norm(rec[t], 2)
        assert cur <= prev + beta[t] * np.linalg.norm(v[t]) + 1e-12
        prev = cur


def test_orthonormal_keys_store_values():
    dk, dv = 4, 3
    rng = np.random.default_rng(8)
    cfg = OracleCfg(dk, dv, 4, "sigmoid", 1.0, 0.0, 0.0)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q.T                                 # orthonormal rows
    vals = rng.standard_normal((dk, dv))
    stream = (keys, keys, vals, np.ones((dk, dk)), np.ones(dk),
              np.zeros((dk, dv)))
    S, _, _, _ = _run(cfg, np.zeros((dk, dv)), np.zeros((3, 2 * dk + dv)),
                      stream, _identity_taps(2 * dk + dv))
    for i in range(dk):
        np.testing.assert_allclose(S.T @ keys[i], vals[i], atol=1e-13)


def test_gated_norm_unit_rms_and_silu_ratio():
    rng = np.random.default_rng(9)
    dk, dv, T = 6, 16, 4
    q, k, v, alpha, beta, _ = _rand_stream(rng, T, dk, dv)
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    h0 = np.zeros((3, 2 * dk + dv))
    S0 = rng.standard_normal((dk, dv))
    big = np.full((T, dv), 40.0)
    y = _run(OracleCfg(dk, dv, 4, "sigmoid", 1.0, 1e-6, 0.0), S0, h0,
             (q, k, v, alpha, beta, big), w)[2]
    np.testing.assert_allclose(np.sqrt(np.mean(y ** 2, axis=1)), 1.0,
                               rtol=1e-14)
    g = rng.standard_normal((T, dv))
    ys = _run(OracleCfg(dk, dv, 4, "sigmoid"), S0, h0,
              (q, k, v, alpha, beta, g), w)[2]
    yl = _run(OracleCfg(dk, dv, 4, "silu"), S0, h0,
              (q, k, v, alpha, beta, g), w)[2]
    np.testing.assert_allclose(yl, ys * g, rtol=1e-13, atol=1e-15)


def test_history_holds_last_raw_tokens_and_split_runs_agree():
    rng = np.random.default_rng(10)
    dk, dv, T = 5, 4, 11
    cfg = OracleCfg(dk, dv)
    st = _rand_stream(rng, T, dk, dv)
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    S0 = rng.standard_normal((dk, dv))
    h0 = rng.standard_normal((3, 2 * dk + dv))
    S, h, y, _ = _run(cfg, S0, h0, st, w)
    raw = np.concatenate(st[:3], axis=1)
    np.testing.assert_array_equal(h, raw[-3:])
    for cut in (1, 3, 7):
        Sa, ha, ya, _ = _run(cfg, S0, h0, tuple(a[:cut] for a in st), w)
        Sb, hb, yb, _ = _run(cfg, Sa, ha, tuple(a[cut:] for a in st), w)
        np.testing.assert_array_equal(Sb, S)
        np.testing.assert_array_equal(hb, h)
        np.testing.assert_array_equal(np.concatenate([ya, yb]), y)


# ------------------------------------------------ the mixer's three modes

@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_verify_then_commit_equals_decode_steps(state):
    n = 5
    case = wl.make_verify(11, B=3, H=2, dk=8, dv=6, n_draft=n, act="bf16",
                          state=state, init="random")
    cfg = OracleCfg(case.dk, case.dv)
    S0 = case.S0.astype(np.float64)
    h0 = case.hist0.astype(np.float64)
    Sv, hv = S0.copy(), h0.copy()
    y, rec = ref.run_heads(cfg, Sv, hv, case.tokens, case.weights,
                           token_axis=1, want_records=True)
    # verify leaves the stored state alone (it works on copies) and its
    # records and outputs equal FP32 decode steps from the same state
    yd = np.empty_like(y)
    Sd, hd = S0.copy(), h0.copy()
    for t in range(n):
        sub = wl.TokenInputs(*[a[:, t:t + 1] for a in (
            case.tokens.q, case.tokens.k, case.tokens.v, case.tokens.alpha,
            case.tokens.beta, case.tokens.g)])
        yy, _ = ref.run_heads(cfg, Sd, hd, sub, case.weights, token_axis=1)
        yd[:, t] = yy[:, 0]
        np.testing.assert_array_equal(rec[:, t], Sd)
    np.testing.assert_array_equal(y, yd)

    for m in range(n + 1):
        Sc, hc = S0.copy(), h0.copy()
        ref.commit(cfg, Sc, hc, rec, case.tokens, np.full(case.batch, m),
                   state == "bf16")
        Sm, hm = S0.copy(), h0.copy()
        if m:
            sub = wl.TokenInputs(*[a[:, :m] for a in (
                case.tokens.q, case.tokens.k, case.tokens.v,
                case.tokens.alpha, case.tokens.beta, case.tokens.g)])
            ref.run_heads(cfg, Sm, hm, sub, case.weights, token_axis=1,
                          round_each_token=(state == "bf16"))
        np.testing.assert_array_equal(hc, hm)
        if state == "f32" or m <= 1:
            np.testing.assert_array_equal(Sc, Sm)
        else:
            # BF16 storage: one rounding at commit against one per step
            scale = np.abs(Sm).max()
            assert np.abs(Sc - Sm).max() <= 1e-2 * scale
        if m == 0:
            np.testing.assert_array_equal(Sc, S0)
            np.testing.assert_array_equal(hc, h0)


def test_bf16_storage_is_fp32_step_then_rounding():
    case = wl.make_decode(12, B=2, H=2, dk=8, dv=8, steps=6, act="bf16",
                          state="bf16", init="random")
    cfg = OracleCfg(8, 8)
    S, h = case.S0.astype(np.float64), case.hist0.astype(np.float64)
    for s in range(case.steps):
        sub = wl.TokenInputs(*[a[s:s + 1] for a in (
            case.tokens.q, case.tokens.k, case.tokens.v, case.tokens.alpha,
            case.tokens.beta, case.tokens.g)])
        Sb, hb = S.copy(), h.copy()
        yb, _ = ref.run_heads(cfg, Sb, hb, sub, case.weights,
                              round_each_token=True)
        Sf, hf = S.copy(), h.copy()
        yf, _ = ref.run_heads(cfg, Sf, hf, sub, case.weights)
        np.testing.assert_array_equal(yb, yf)       # rounding after y
        np.testing.assert_array_equal(Sb, ref.round_bf16(Sf))
        assert np.all(wl.round_bf16(Sb) == Sb)      # stored values are bf16
        S, h = Sb, hb


@pytest.mark.parametrize("C", [1, 2, 16, 64])
def test_chunked_form_equals_sequential(C):
    rng = np.random.default_rng(13 + C)
    dk, dv = 16, 12
    cfg = OracleCfg(dk, dv)
    for T in (1, C - 1 if C > 1 else 2, C + 1, 3 * C + 5, 150):
        st = _rand_stream(rng, T, dk, dv)
        w = rng.normal(0, 0.5, (2 * dk + dv, 4))
        S0 = rng.normal(0, 0.1, (dk, dv))
        h0 = rng.standard_normal((3, 2 * dk + dv))
        S, h, y, _ = _run(cfg, S0, h0, st, w)
        Sc, hc = S0.copy(), h0.copy()
        yc = ref.run_one_chunked(cfg, C, Sc, hc, *st, w, None)
        np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-12 * np.abs(S).max())
        np.testing.assert_allclose(yc, y, rtol=0, atol=1e-11 * np.abs(y).max())
        np.testing.assert_array_equal(hc, h)


def test_chunked_form_strong_decay():
    """|log alpha| up to about 6 per token, as the workloads reach."""
    rng = np.random.default_rng(14)
    dk, dv, T, C = 16, 8, 200, 64
    cfg = OracleCfg(dk, dv)
    q, k, v, _, beta, g = _rand_stream(rng, T, dk, dv)
    alpha = np.exp(-rng.uniform(0, 6, (T, dk)))
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    S0 = rng.normal(0, 0.1, (dk, dv))
    h0 = np.zeros((3, 2 * dk + dv))
    S, _, y, _ = _run(cfg, S0, h0, (q, k, v, alpha, beta, g), w)
    Sc = S0.copy()
    yc = ref.run_one_chunked(cfg, C, Sc, h0.copy(), q, k, v, alpha, beta, g,
                             w, None)
    np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-12 * np.abs(S).max())
    np.testing.assert_allclose(yc, y, rtol=0, atol=1e-11 * np.abs(y).max())


# ----------------------------------------------------------------- gate logits

@pytest.mark.parametrize("chunk", [None, 16])
def test_gate_logits_match_library_logistic(chunk):
    """Logit inputs: alpha = exp(-softplus(a)) = logistic(-a) and beta =
    logistic(b).  A run on logits equals a run on the values scipy's expit
    (an independent library routine) gives for them, token by token and in
    the chunk form.  Logits up to |6| reach both sides of softplus's split."""
    from scipy.special import expit
    rng = np.random.default_rng(91)
    dk, dv, T = 8, 6, 40
    q, k, v, _, _, g = _rand_stream(rng, T, dk, dv)
    a = rng.normal(0.0, 2.0, (T, dk))
    b = rng.normal(0.0, 2.0, T)
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    S0 = rng.normal(0, 0.1, (dk, dv))
    h0 = rng.standard_normal((3, 2 * dk + dv))
    cfg_l, cfg_v = OracleCfg(dk, dv, gates="logits"), OracleCfg(dk, dv)
    if chunk is None:
        S_l, h_l, y_l, _ = _run(cfg_l, S0, h0, (q, k, v, a, b, g), w)
        S_v, h_v, y_v, _ = _run(cfg_v, S0, h0, (q, k, v, expit(-a), expit(b), g), w)
    else:
        S_l, h_l, S_v, h_v = S0.copy(), h0.copy(), S0.copy(), h0.copy()
        y_l = ref.run_one_chunked(cfg_l, chunk, S_l, h_l, q, k, v, a, b, g, w, None)
        y_v = ref.run_one_chunked(cfg_v, chunk, S_v, h_v, q, k, v, expit(-a),
                                  expit(b), g, w, None)
    np.testing.assert_allclose(S_l, S_v, rtol=0, atol=1e-13 * np.abs(S_v).max())
    np.testing.assert_allclose(y_l, y_v, rtol=0, atol=1e-12 * np.abs(y_v).max())
    np.testing.assert_array_equal(h_l, h_v)


def test_gate_logits_special_values():
    """a = 0 halves the state (alpha = 1/2) and b = 0 writes at beta = 1/2;
    a = -60 keeps the state (alpha = 1 in fp64) and b = -60 writes nothing
    measurable (beta ~ 1e-26), so the state stays as it was."""
    rng = np.random.default_rng(92)
    dk, dv, T = 6, 5, 4
    q, k, v, _, _, g = _rand_stream(rng, T, dk, dv)
    w = rng.normal(0, 0.5, (2 * dk + dv, 4))
    S0 = rng.normal(0, 0.1, (dk, dv))
    h0 = np.zeros((3, 2 * dk + dv))
    cfg_l, cfg_v = OracleCfg(dk, dv, gates="logits"), OracleCfg(dk, dv)
    S_l, _, y_l, _ = _run(cfg_l, S0, h0, (q, k, v, np.zeros((T, dk)), np.zeros(T), g), w)
    S_v, _, y_v, _ = _run(cfg_v, S0, h0, (q, k, v, np.full((T, dk), 0.5),
                                          np.full(T, 0.5), g), w)
    np.testing.assert_allclose(S_l, S_v, rtol=1e-14, atol=0)
    np.testing.assert_allclose(y_l, y_v, rtol=1e-13, atol=0)
    S_k, _, _, _ = _run(cfg_l, S0, h0, (q, k, v, np.full((T, dk), -60.0),
                                        np.full(T, -60.0), g), w)
    np.testing.assert_allclose(S_k, S0, rtol=0, atol=1e-20)


def test_prefill_case_equals_decode_of_same_tokens():
    case = wl.make_prefill(15, lens=[7, 1, 70], H=2, dk=8, dv=8, act="bf16",
                           state="f32", chunk=16, slice_len=4)
    y, S, h = ref.prefill_case(case, threads=1)
    cfg = OracleCfg(8, 8)
    for b, n in enumerate(case.lens):
        lo = int(case.cu_seqlens[b])
        Sd = np.zeros((1, 2, 8, 8))
        hd = np.zeros((1, 3, 2, 24))
        for t in range(n):
            sub = wl.TokenInputs(*[a[lo + t:lo + t + 1][None] for a in (
                case.tokens.q, case.tokens.k, case.tokens.v,
                case.tokens.alpha, case.tokens.beta, case.tokens.g)])
            yy, _ = ref.run_heads(cfg, Sd, hd, sub, case.weights,
                                  token_axis=1, threads=1)
            np.testing.assert_array_equal(yy[0, 0], y[lo + t])
        np.testing.assert_array_equal(Sd[0], S[b])
        np.testing.assert_array_equal(hd[0], h[b])
    yc, Sc, _ = ref.prefill_case(case, threads=1, chunk=16)
    np.testing.assert_allclose(Sc, S, atol=1e-12 * np.abs(S).max(), rtol=0)
    np.testing.assert_allclose(yc, y, atol=1e-11 * np.abs(y).max(), rtol=0)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import ctypes
    c = OracleCfg(4, 4).c()
    c.dk = 0
    assert oracle_lib.kda_ref_run(ctypes.byref(c), 1, *([None] * 10), 0, None,
                                  None) == -1
    c = OracleCfg(4, 4).c()
    S = np.zeros((4, 4))
    h = np.zeros((3, 12))
    with pytest.raises(RuntimeError):
        ref.commit_one(OracleCfg(4, 4), 2, 3, 0, S, h, np.zeros((2, 4, 4)),
                       np.zeros((2, 4)), np.zeros((2, 4)), np.zeros((2, 4)))
