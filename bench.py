"""Benchmark of the KDA mixer on one MI355X.

The timed step is one decode call (conv, L2 norms, decay, delta-rule write,
read-out, gated RMSNorm and the typed state store) over the large-batch
decode workload: 256 sequences x 32 heads, dk = dv = 128, bf16 activations,
BF16 state storage (32 KiB per head), 192 of the 256 rows active per step.
Four independent state pools ("layers", 256 MiB each) are rotated so the
working set (1 GiB) is far larger than the 256 MB Infinity Cache and every
step streams its state from HBM.

Printed: one JSON line with the throughput (active token-head state updates
per second), the roofline of the decode kernel (algorithmic bytes per launch
over its median launch time, HIP events on the launch stream), the CPU
oracle's throughput on a bounded sample of the same workload, and the same
figures for the other modes (batched decode with FP32 state, speculative
verify + commit, chunked prefill with its algorithmic and issued matrix-core
rates, two-head decode, FP8 inputs).

Exactly --steps launches are timed, in five groups; each group is a captured
HIP graph replayed once between HIP events, so the host never sits between
two kernels.  The per-launch time is the median over the groups.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E peak, GB/s
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=4,
                    help="state pools of the headline workload rotated to defeat the "
                         "Infinity Cache (4 x 256 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-modes", action="store_true",
                    help="time only the headline decode workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of the extra modes to run (f32, verify, recompute, "
                         "compact, fp8, prefill); all when empty")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (a known byte count "
                         "for scaling the HBM byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------ byte models
# Algorithmic bytes: every tensor the step must touch, counted once.

def act_bytes(act):
    """Bytes per element of q, k, v (and the ring, raw drafts) and of alpha,
    beta, g: FP8 activations keep the gates in BF16."""
    a = {"f32": 4, "bf16": 2, "fp8": 1}[act]
    return a, (2 if act == "fp8" else a)


def decode_bytes_per_th(dk, dv, act_b, state_b, gate_b=None):
    C = 2 * dk + dv
    gate_b = act_b if gate_b is None else gate_b
    return (2 * dk * dv * state_b          # state read + write
            + C * act_b                    # raw q, k, v
            + dk * gate_b + gate_b         # alpha, beta
            + dv * gate_b                  # g
            + 3 * C * act_b                # conv history read (3 ring entries)
            + C * act_b                    # new ring entry
            + dv * 4)                      # y (FP32)


def per_call_bytes(H, dk, dv, rows):
    return H * (2 * dk + dv) * 4 * 4 + dv * 4 + rows * 8   # conv taps, norm_w, ids


def verify_bytes_per_head(n, dk, dv, act_b, state_b, gate_b=None):
    C = 2 * dk + dv
    gate_b = act_b if gate_b is None else gate_b
    return (dk * dv * state_b              # state read
            + n * dk * dv * 4              # FP32 records
            + n * (C * act_b + (dk + 1 + dv) * gate_b)  # q, k, v, alpha, beta, g
            + 3 * C * act_b                # conv history
            + n * C * act_b                # raw drafts kept
            + n * dv * 4)                  # y


def prefill_flops_per_chunk(C, d, L=None):
    """Algorithmic FLOPs of the chunk form for one (chunk, head), counting
    triangles once: A (strictly lower) and P (lower incl. diagonal) as
    d-deep dot products, T applied to [beta K_G | beta V], then
    U = Ut - W S, O = Qg S + P U and S <- gamma S + Kc^T U."""
    L = C if L is None else L
    tri_lo, tri_le = L * (L - 1) // 2, L * (L + 1) // 2
    return 2 * (tri_lo * d + tri_le * d       # A, P
                + tri_le * 2 * d              # T [beta K_G | beta V]
                + 3 * L * d * d               # W S, Qg S, Kc^T U
                + tri_le * d)                 # P U


# MFMA instructions the prefill kernels issue per (chunk, head): chunk kernel
# A/P products 336 and solve 96 of 16x16x32 plus 288 of 16x16x16; state
# kernel 2 workgroups x 4 waves x 162 of 16x16x32 (three passes per product).
PREFILL_MFMA_32_PER_CHUNK = 336 + 96 + 2 * 4 * 162
PREFILL_MFMA_16_PER_CHUNK = 288


def prefill_bytes(lens, H, dk, dv, act_b, st_b, gate_b=None):
    """Algorithmic HBM bytes of one prefill call from position 0: q, k, v,
    alpha, g and beta read once, y (FP32) written once, the final state and
    the ring's last three raw tokens written once per (sequence, head),
    conv taps and norm weight once."""
    T = int(np.sum(lens))
    C = 2 * dk + dv
    gate_b = act_b if gate_b is None else gate_b
    per_th = C * act_b + (dk + dv + 1) * gate_b + dv * 4
    per_sh = dk * dv * st_b + 3 * C * act_b
    return T * H * per_th + len(lens) * H * per_sh + H * C * 4 * 4 + dv * 4


# ------------------------------------------------------------ measured traffic

PROFILES = os.path.join(ROOT, "profiles")
DECODE_BF16_TRAFFIC = ("token_kernel_large_batch_decode_bf16_state_hbm_traffic.md",
                       ("kda_token.hip", "kda_device.h", "kda_internal.h"))
DECODE_F32_TRAFFIC = ("token_kernel_batched_decode_hbm_traffic.md",
                      ("kda_token.hip", "kda_device.h", "kda_internal.h"))
PREFILL_TRAFFIC = ("prefill_kernels_chunked_prefill_hbm_traffic.md",
                   ("kda_prefill.hip", "kda_mfma.h", "kda_device.h", "kda_internal.h"))


def measured_traffic(which):
    """HBM bytes per launch of a kernel (or, for the prefill, of one call's
    kernels), from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded under
    profiles/ (each scaled by the same counter's reading for a 1 GiB copy).
    None when the file is missing or the kernels' sources have changed since
    the counters were taken."""
    import hashlib
    name, sources = which
    try:
        text = open(os.path.join(PROFILES, name)).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256:")))
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "hybrid_linear_attention_rule_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256", "").strip() != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


# ------------------------------------------------------------ helpers

def timed_loop(torch, launch, K, W, groups=5):
    """Time exactly K launches (at least `groups` of them, so K is raised to
    `groups` when smaller), after W warm-up launches outside any graph.

    The K launches are split into `groups` consecutive groups of K // groups
    or K // groups + 1 launches.  Each group is captured as one HIP graph (the
    launch index keeps counting across groups, so state pools and steps
    rotate as in eager order) and replayed once untimed, then timed once:
    device synchronisation, a short spin kernel that keeps the GPU busy while
    the host queues the start event, the replay and the end event, then
    synchronisation again.  The events sit on the launch stream.  Returns
    (total seconds, median seconds per launch over the groups, launches
    timed, spread)."""
    K = max(K, groups)
    for i in range(W):
        launch(i)
    torch.cuda.synchronize()
    sizes = [K // groups + (1 if g < K % groups else 0) for g in range(groups)]
    graphs, first = [], W
    for n in sizes:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + n):
                launch(i)
        graphs.append((g, n))
        first += n
    for g, _ in graphs:                   # one untimed replay of each
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    total, per = 0.0, []
    for g, n in graphs:
        torch.cuda.synchronize()
        torch.cuda._sleep(200000)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        dt = t0.elapsed_time(t1) / 1e3
        total += dt
        per.append(dt / n)
    per.sort()
    med = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    spread = {"repeats": len(per), "min_us": per[0] * 1e6, "max_us": per[-1] * 1e6,
              "launches_per_group": sizes}
    return total, med, K, spread


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Achievable device-memory bandwidth: a plain device-to-device copy of
    `nbytes` (reads and writes nbytes each), timed with HIP events."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    dt = t0.elapsed_time(t1) / 1e3
    del src, dst
    return 2.0 * nbytes * reps / dt / 1e9


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


# ------------------------------------------------------------ decode

def run_decode_mode(torch, case, K, W, layers):
    from kda_inputs import device as dev
    from hybrid_linear_attention_rule_amd import kda
    import oracle

    pools = [dev.make_state(case, spare_slots=0, fill_nan=False) for _ in range(layers)]
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, H, dk, dv, S = case.batch, case.H, case.dk, case.dv, case.steps
    y = torch.empty((B, H, dv), device="cuda")
    slot_steps = [torch.from_numpy(np.where(case.active[s], pools[0].slots, -1)
                                   .astype(np.int32)).cuda() for s in range(S)]
    pos = np.zeros((S, B), dtype=np.int64)
    pos[0] = case.pos0
    for s in range(1, S):
        pos[s] = pos[s - 1] + case.active[s - 1]
    pos_steps = [torch.from_numpy(pos[s].astype(np.int32)).cuda() for s in range(S)]
    ds0 = pools[0]

    def launch(i):
        layer = i % layers
        s = (i // layers) % S
        d = pools[layer]
        kda.decode(d.shape, d.params, slot_steps[s], pos_steps[s], tok["q"][s],
                   tok["k"][s], tok["v"][s], tok["alpha"][s], tok["beta"][s],
                   tok["g"][s], d.pool, d.ring, y)

    # parity of the first step on layer 0 before any timing
    launch(0)
    torch.cuda.synchronize()
    y_ref, S_ref, _ = oracle.decode_case(case, steps=1)
    act0 = case.active[0]
    tol = 2e-5 if case.state == "f32" else 1e-2
    e_y = rel_err(y.cpu().numpy()[act0], y_ref[0][act0])
    e_s = rel_err(dev.read_states(ds0)[act0], S_ref[act0])
    assert e_y <= tol and e_s <= tol, f"parity failed before timing: {e_y} {e_s}"
    # restore layer 0 so that every layer starts from the same state
    pools[0] = dev.make_state(case, spare_slots=0, fill_nan=False)

    total, per_launch, n_timed, spread = timed_loop(torch, launch, K, W)
    act_b, gate_b = act_bytes(case.act)
    st_b = 2 if case.state == "bf16" else 4
    n_active = int(case.active.sum(axis=1).mean())
    th_per_step = n_active * H
    bytes_launch = th_per_step * decode_bytes_per_th(dk, dv, act_b, st_b, gate_b) + \
        per_call_bytes(H, dk, dv, B)
    return dict(
        workload=case.name, rows=B, active_rows=n_active, heads=H, dk=dk, dv=dv,
        act=case.act, state=case.state, layers=layers, launches_timed=n_timed,
        warmup=W, ms_per_step=per_launch * 1e3, kernel_us=per_launch * 1e6,
        th_per_s=th_per_step / per_launch, bytes_per_launch=bytes_launch,
        hbm_gbs=bytes_launch / per_launch / 1e9,
        hbm_frac=bytes_launch / per_launch / 1e9 / HBM_PEAK_GBS,
        spread=spread, parity_rel_err={"y": e_y, "state": e_s})


# ------------------------------------------------------------ verify

def run_verify_mode(torch, case, K, W, layers):
    from kda_inputs import device as dev
    from hybrid_linear_attention_rule_amd import kda
    import oracle

    pools = [dev.make_state(case, spare_slots=0, fill_nan=False) for _ in range(layers)]
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, n, H, dk, dv = case.batch, case.n_draft, case.H, case.dk, case.dv
    C = 2 * dk + dv
    recs = [torch.empty((B, n, H, dk, dv), device="cuda") for _ in range(2)]
    dconv = torch.empty((B, n, H, C), device="cuda", dtype=pools[0].shape.act_dtype)
    y = torch.empty((B, n, H, dv), device="cuda")
    slot_t = pools[0].slot_ids
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    acc_t = torch.from_numpy(case.accepted.astype(np.int32)).cuda()

    def verify(i):
        d = pools[i % layers]
        kda.verify(d.shape, d.params, slot_t, pos_t, tok["q"], tok["k"], tok["v"],
                   tok["alpha"], tok["beta"], tok["g"], d.pool, d.ring, recs[i % 2],
                   dconv, y)

    verify(0)
    torch.cuda.synchronize()
    y_ref, rec_ref, _, _ = oracle.verify_case(case)
    e_y = rel_err(y.cpu().numpy(), y_ref)
    e_r = rel_err(recs[0].cpu().numpy(), rec_ref)
    assert e_y <= 2e-5 and e_r <= 2e-5, f"verify parity failed: {e_y} {e_r}"
    total, v_launch, _, v_spread = timed_loop(torch, verify, K, W)
    act_b, gate_b = act_bytes(case.act)
    st_b = 2 if case.state == "bf16" else 4
    per_head = verify_bytes_per_head(n, dk, dv, act_b, st_b, gate_b)
    bytes_launch = B * H * per_head + per_call_bytes(H, dk, dv, B)

    # commit: copies record m-1 of rows with m >= 1 (m = accepted)
    def commit(i):
        d = pools[i % layers]
        kda.commit_accepted(d.shape, slot_t, pos_t, acc_t, recs[0], dconv, d.pool,
                            d.ring)
    c_total, c_launch, _, c_spread = timed_loop(torch, commit, K, W)
    m = case.accepted
    commit_bytes = int((m > 0).sum()) * H * (dk * dv * 4 + dk * dv * st_b) + \
        int(np.minimum(m, 4).sum()) * H * 2 * C * act_b
    return dict(
        workload=case.name, rows=B, heads=H, n_draft=n, state=case.state,
        verify_kernel_us=v_launch * 1e6, th_per_s=B * H * n / v_launch,
        bytes_per_launch=bytes_launch, hbm_gbs=bytes_launch / v_launch / 1e9,
        hbm_frac=bytes_launch / v_launch / 1e9 / HBM_PEAK_GBS,
        commit_kernel_us=c_launch * 1e6, commit_bytes=commit_bytes,
        commit_hbm_gbs=commit_bytes / c_launch / 1e9,
        verify_spread=v_spread, commit_spread=c_spread,
        parity_rel_err={"y": e_y, "records": e_r})


def run_verify_recompute_mode(torch, case, K, W, layers):
    """The records-free alternative on the same workload: verify writes only
    y, and the commit runs the accepted tokens again from the stored state."""
    from kda_inputs import device as dev
    from hybrid_linear_attention_rule_amd import kda
    import oracle

    pools = [dev.make_state(case, spare_slots=0, fill_nan=False) for _ in range(layers)]
    tok = dev.tokens_to_device(case.tokens, case.act)
    B, n, H, dk, dv = case.batch, case.n_draft, case.H, case.dk, case.dv
    C = 2 * dk + dv
    y = torch.empty((B, n, H, dv), device="cuda")
    slot_t = pools[0].slot_ids
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()
    acc_t = torch.from_numpy(case.accepted.astype(np.int32)).cuda()

    def verify(i):
        d = pools[i % layers]
        kda.verify(d.shape, d.params, slot_t, pos_t, tok["q"], tok["k"], tok["v"],
                   tok["alpha"], tok["beta"], tok["g"], d.pool, d.ring, None, None, y)

    def commit(i):
        d = pools[i % layers]
        kda.commit_recompute(d.shape, d.params, slot_t, pos_t, acc_t, tok["q"], tok["k"],
                             tok["v"], tok["alpha"], tok["beta"], tok["g"], d.pool, d.ring)

    verify(0)
    commit(0)
    torch.cuda.synchronize()
    y_ref, _, S_ref, _ = oracle.verify_case(case)
    tol = 2e-5 if case.state == "f32" else 1e-2
    e_y = rel_err(y.cpu().numpy(), y_ref)
    e_s = rel_err(dev.read_states(pools[0]), S_ref)
    assert e_y <= 2e-5 and e_s <= tol, f"verify/recompute parity failed: {e_y} {e_s}"
    pools[0] = dev.make_state(case, spare_slots=0, fill_nan=False)

    _, v_launch, _, v_spread = timed_loop(torch, verify, K, W)
    _, c_launch, _, c_spread = timed_loop(torch, commit, K, W)
    act_b, gate_b = act_bytes(case.act)
    st_b = 2 if case.state == "bf16" else 4
    per_tok_in = C * act_b + (dk + 1 + dv) * gate_b
    v_bytes = B * H * (dk * dv * st_b + n * per_tok_in + 3 * C * act_b + n * dv * 4) + \
        per_call_bytes(H, dk, dv, B)
    m = case.accepted
    c_bytes = int((m > 0).sum()) * H * (2 * dk * dv * st_b + 3 * C * act_b) + \
        int(m.sum()) * H * per_tok_in + int(np.minimum(m, 4).sum()) * H * C * act_b + \
        per_call_bytes(H, dk, dv, B)
    return dict(
        workload=case.name, rows=B, heads=H, n_draft=n, state=case.state,
        verify_kernel_us=v_launch * 1e6, th_per_s=B * H * n / v_launch,
        verify_bytes=v_bytes, verify_hbm_gbs=v_bytes / v_launch / 1e9,
        commit_kernel_us=c_launch * 1e6, commit_bytes=c_bytes,
        commit_hbm_gbs=c_bytes / c_launch / 1e9,
        verify_plus_commit_us=(v_launch + c_launch) * 1e6,
        verify_spread=v_spread, commit_spread=c_spread,
        parity_rel_err={"y": e_y, "committed_state": e_s})


# ------------------------------------------------------------ prefill

def run_prefill_mode(torch, case, K, W):
    from kda_inputs import device as dev
    from hybrid_linear_attention_rule_amd import kda
    import oracle

    ds = dev.make_state(case, spare_slots=0, fill_nan=False)
    tok = dev.tokens_to_device(case.tokens, case.act)
    T = int(case.cu_seqlens[-1])
    H, dk, dv = case.H, case.dk, case.dv
    y = torch.empty((T, H, dv), device="cuda")
    ws = torch.empty(kda.prefill_workspace_bytes(ds.shape, case.batch, T),
                     dtype=torch.uint8, device="cuda")
    cu_t = torch.from_numpy(case.cu_seqlens.astype(np.int32)).cuda()
    pos_t = torch.from_numpy(case.pos0.astype(np.int32)).cuda()

    def launch(i):
        # from position 0 the pool is written, not read: every call is the same
        kda.prefill(ds.shape, ds.params, cu_t, max(case.lens), ds.slot_ids, pos_t,
                    tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], tok["g"],
                    ds.pool, ds.ring, y, ws)

    launch(0)
    torch.cuda.synchronize()
    y_ref, S_ref, _ = oracle.prefill_case(case)
    e_y = rel_err(y.cpu().numpy(), y_ref)
    tol = 2e-5 if case.state == "f32" else 1e-2
    e_s = rel_err(dev.read_states(ds), S_ref)
    assert e_y <= 2e-5 and e_s <= tol, f"prefill parity failed: {e_y} {e_s}"
    total, per_launch, n_timed, spread = timed_loop(torch, launch, 10, 2)
    act_b, gate_b = act_bytes(case.act)
    st_b = 2 if case.state == "bf16" else 4
    lens = np.asarray(case.lens)
    flops = sum(H * (prefill_flops_per_chunk(64, dk) * (int(L) // 64) +
                     (prefill_flops_per_chunk(64, dk, int(L) % 64) if L % 64 else 0))
                for L in lens)
    chunks = int(sum((int(L) + 63) // 64 for L in lens)) * H
    issued = chunks * (PREFILL_MFMA_32_PER_CHUNK * 16 * 16 * 32 * 2 +
                       PREFILL_MFMA_16_PER_CHUNK * 16 * 16 * 16 * 2)
    nbytes = prefill_bytes(lens, H, dk, dv, act_b, st_b, gate_b)
    floor_s = max(flops / (MFMA_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
    return dict(
        workload=case.name, seq_lens=[int(x) for x in lens], heads=H, dk=dk, dv=dv,
        chunk=64, act=case.act, state=case.state, launches_timed=n_timed,
        prefill_us=per_launch * 1e6, tokens_per_s=T / per_launch,
        th_per_s=T * H / per_launch,
        algorithmic_gflop=flops / 1e9, mfma_tflops_algorithmic=flops / per_launch / 1e12,
        mfma_frac_algorithmic=flops / per_launch / 1e12 / MFMA_PEAK_TFLOPS,
        issued_gflop=issued / 1e9, mfma_tflops_issued=issued / per_launch / 1e12,
        mfma_frac_issued=issued / per_launch / 1e12 / MFMA_PEAK_TFLOPS,
        bytes_per_launch=nbytes, hbm_gbs=nbytes / per_launch / 1e9,
        hbm_frac=nbytes / per_launch / 1e9 / HBM_PEAK_GBS,
        roofline_floor_us=floor_s * 1e6, roofline_frac=floor_s / per_launch,
        spread=spread, parity_rel_err={"y": e_y, "state": e_s})


# ------------------------------------------------------------ CPU oracle

def cpu_info():
    """The host's logical CPU count, the share this process may run on, and
    the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        share = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        share = os.cpu_count() or 1
    return os.cpu_count() or 1, share, model


def cpu_baseline(case, seconds, max_threads=16):
    """The oracle as it stands (fp64 C, threaded over (sequence, head)) on the
    same workload: whole passes over its decode steps until `seconds`
    elapse, on the host cores this process may use (at most `max_threads`,
    one GPU's share of the host); then one pass on a single thread."""
    import oracle

    def passes(th, secs):
        done, n = 0, 0
        t0 = time.perf_counter()
        while True:
            oracle.decode_case(case, threads=th)
            n += 1
            done += int(case.active.sum()) * case.H
            if time.perf_counter() - t0 >= secs:
                break
        return done / (time.perf_counter() - t0), n, time.perf_counter() - t0

    nproc, share, model = cpu_info()
    th = max(1, min(share, max_threads))
    rate, n, dt = passes(th, seconds)
    rate1, n1, dt1 = passes(1, 0.0)
    return {"value": rate, "unit": "token-head updates/s", "cores": th,
            "kind": "oracle",
            "sample": f"{n} full pass(es) of the {case.name} workload "
                      f"({case.steps} decode steps, {int(case.active.sum(axis=1).mean())} "
                      f"active of {case.batch} rows, {case.H} heads), fp64 C oracle on {th} "
                      f"threads, {dt:.1f} s",
            "host": {"nproc": nproc, "usable_cpus": share, "cpu_model": model},
            "single_thread": {"value": rate1, "sample": f"{n1} pass on 1 thread, {dt1:.1f} s"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer shards over heads and sequences with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from hybrid_linear_attention_rule_amd import kda
    from kda_inputs import workloads as wl

    if not os.path.exists(kda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kda.load()
    torch.cuda.init()

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)        # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    copy_gbs = copy_bandwidth(torch)
    print(f"# device copy of 1 GiB: {copy_gbs:.0f} GB/s", file=sys.stderr, flush=True)

    case3 = wl.config(3)
    print(f"# decode {case3.name}: steps={args.steps} warmup={args.warmup} "
          f"layers={args.layers}", file=sys.stderr, flush=True)
    head = run_decode_mode(torch, case3, args.steps, args.warmup, args.layers)
    print(f"# decode kernel {head['kernel_us']:.2f} us, {head['hbm_gbs']:.0f} GB/s",
          file=sys.stderr, flush=True)

    modes = {}
    only = set(x for x in args.only.split(",") if x)
    want = (lambda m: not args.no_modes and (not only or m in only))
    if want("f32"):
        case1 = wl.config(1)
        print(f"# decode {case1.name}", file=sys.stderr, flush=True)
        modes["batched_decode_f32_state"] = run_decode_mode(
            torch, case1, args.steps, args.warmup, 8)
        modes["batched_decode_f32_state"]["traffic"] = measured_traffic(DECODE_F32_TRAFFIC)
    if want("verify"):
        case2 = wl.config(2)
        print(f"# verify {case2.name}", file=sys.stderr, flush=True)
        modes["spec_verify_commit"] = run_verify_mode(torch, case2, args.steps,
                                                      args.warmup, 8)
        modes["spec_verify_commit"]["verify_plus_commit_us"] = (
            modes["spec_verify_commit"]["verify_kernel_us"] +
            modes["spec_verify_commit"]["commit_kernel_us"])
    if want("recompute"):
        print(f"# verify without records, commit by recompute", file=sys.stderr, flush=True)
        modes["spec_verify_recompute"] = run_verify_recompute_mode(
            torch, wl.config(2), args.steps, args.warmup, 8)
    if want("compact"):
        for st, layers in (("f32", 32), ("bf16", 48)):
            casec = wl.compact_heads(st)
            print(f"# decode {casec.name}", file=sys.stderr, flush=True)
            modes[f"compact_heads_decode_{st}_state"] = run_decode_mode(
                torch, casec, args.steps, args.warmup, layers)
    if want("fp8"):
        casef = wl.fp8_decode()
        print(f"# decode {casef.name}", file=sys.stderr, flush=True)
        modes["batched_decode_fp8_act"] = run_decode_mode(torch, casef, args.steps,
                                                          args.warmup, 8)
        casefp = wl.fp8_prefill()
        print(f"# prefill {casefp.name}", file=sys.stderr, flush=True)
        modes["chunked_prefill_fp8_act"] = run_prefill_mode(torch, casefp, args.steps,
                                                            args.warmup)
    if want("prefill"):
        case4 = wl.config(4)
        print(f"# prefill {case4.name}", file=sys.stderr, flush=True)
        modes["chunked_prefill"] = pf = run_prefill_mode(torch, case4, args.steps, args.warmup)
        t = measured_traffic(PREFILL_TRAFFIC)
        pf["traffic"] = t
        pf["traffic_over_algorithmic"] = None if t is None else t / pf["bytes_per_launch"]
        print(f"# prefill {pf['prefill_us']:.1f} us", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        print("# cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case3, args.cpu_seconds)

    line = {
        "metric": "KDA decode/verify token-head updates/s + achieved HBM GB/s (% peak), 1 GPU",
        "value": head["th_per_s"],
        "unit": "token-head updates/s",
        "n_gpus": 1,
        "steps": head["launches_timed"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; distributions of the large-batch decode workload)",
        "config": {"workload": case3.name, "batch": case3.batch,
                   "active_rows_per_step": head["active_rows"], "heads": case3.H,
                   "head_k": case3.dk, "head_v": case3.dv, "act": case3.act,
                   "state": case3.state, "state_pools_rotated": args.layers,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": head["hbm_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": measured_traffic(DECODE_BF16_TRAFFIC),
                     "kernel": "kda::token_kernel<128,128,bf16,bf16,decode>",
                     "kernel_us": head["kernel_us"],
                     "kernel_us_spread": head["spread"],
                     "bytes_per_launch": head["bytes_per_launch"],
                     "achievable_copy_gbs": copy_gbs,
                     "frac_of_copy": head["hbm_gbs"] / copy_gbs},
        "cpu_baseline": cpu,
        "parity_rel_err": head["parity_rel_err"],
        "modes": modes,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
