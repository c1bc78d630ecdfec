"""Throughput of the chunked TTT / Titans memory forward on one MI355X.

A step is one forward pass of the whole memory layer -- every (batch, head)
sequence, every chunk -- over one batch of synthetic inputs that are already
resident in HBM.  By default: the Titans linear-memory workload, B=4 H=16
T=8192 d=128 b=64, bf16 q/k/v and z, float32 gates and state (``--z-f32``:
float32 z).  ``--workload 2`` and ``--workload 4`` time the TTT-Linear-style
(B=8 H=12 T=2048 d=64 b=16) and long-context (B=1 H=32 T=131072 d=128 b=64)
linear workloads; ``--workload 5`` the deep (2-layer MLP) memory workload,
B=4 H=8 T=4096 d=64 hidden=256 b=16.  ``--decode`` times token-by-token generation on the Titans shapes
instead: a step is one call of the primal form for one token of every
(batch, head) sequence (B=4 H=16 d=128), with the state carried in place from
step to step.  ``--varlen`` times packed variable-length documents with the
Titans recipe (32768 tokens per head in documents of seeded lengths, each
from its own state); with ``--backward`` as well, one training step over
those documents.  ``--backward`` times one training step of the Titans
linear memory: the forward that saves the chunk-start states plus the
backward pass (gradients for q, k, v, the three gates and the initial state),
with a seeded synthetic outer-loss derivative dz (with ``--chunk-gates`` as
well, that step with chunk-shared gates).  ``--chunk-gates`` times
the Titans forward with gates shared by each chunk's tokens (one theta, eta,
alpha per 64-token chunk, drawn from the same distributions).  Prints ONE
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload {2,3,4,5} | --decode | --varlen [--backward] | [--chunk-gates] [--backward]]
                    [--z-f32] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from test_neural_memory_amd import memory as tm  # noqa: E402
from test_neural_memory_amd.workloads import (WORKLOADS, make_cotangents, make_deep_layers, make_inputs,  # noqa: E402
                                              set_chunk_gates, to_numpy64, varlen_lengths)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cores():
    """CPU cores this process may run on (the oracle baseline uses up to 16
    worker processes of one thread each, the machine's CPU share for one GPU)."""
    return len(os.sched_getaffinity(0))


def algorithmic_work(w, in_bytes=2, z_bytes=4, reads_state=False):
    """Bytes and flops the method itself must move / do for one forward.

    Per (batch, head, token): read q, k, v (d elements each) and three gates,
    write z (d elements); per chunk the dual form does 2 b d^2 flops for each of
    K M0^T, Q M0^T, Q S0^T, dM, dS and 2 b^2 d for each of Q K^T and P E, i.e.
    10 d^2 + 4 b d flops per head-token.  Per (batch, head): write M_T, S_T
    (and read M0, S0 when given: 16 d^2 bytes of state in all).  With bf16
    q, k, v and z at d = 128, b = 64, T = 8192 that is 1036 bytes per
    head-token plus 32 of state = 1068.
    """
    ht = w.B * w.H * w.T
    per_tok = 3 * w.d * in_bytes + 3 * 4 + w.d * z_bytes
    state = w.B * w.H * w.d * w.d * 4 * (4 if reads_state else 2)
    flops = ht * (10 * w.d * w.d + 4 * w.b * w.d)
    return ht * per_tok + state, flops, per_tok


def algorithmic_work_mlp(w, in_bytes=2, z_bytes=4, depth=2):
    """Bytes and flops of one deep-memory forward (f(u) = u + SiLU(...SiLU(u W_1)...) W_L, hidden h).

    Per (batch, head, token), per chunk of b tokens in the dual form, for the
    two outer layers: 2dh flops for each of K W1, X W_L, R W_L^T, Q W1, Q S1,
    Y W_L, Y S_L and for each of the four weight/momentum carries (22 dh = 88
    d^2 at h = 4d), plus 2bd or 2bh for each of Q K^T, (L.QK^T) D_1, Y X^T and
    (L.G) R (4b(d + h) = 20bd).  Each of the depth - 2 hidden-to-hidden layers
    adds 2h^2 for each of X W, D W^T, Y W, Y S and the two carries (12 h^2)
    and 2bh for each of Y X^T and (L.G) D (4bh).
    Bytes: q, k, v, three gates and z per token; every weight and momentum
    tensor read and written once per (batch, head).
    """
    ht = w.B * w.H * w.T
    d, h = w.d, w.hidden
    nm = depth - 2
    per_tok = 3 * d * in_bytes + 3 * 4 + d * z_bytes
    state = w.B * w.H * 4 * (2 * d * h + nm * h * h) * 4
    flops = ht * (22 * d * h + 4 * w.b * (d + h) + nm * (12 * h * h + 4 * w.b * h))
    return ht * per_tok + state, flops, per_tok


def algorithmic_work_decode(w, in_bytes=2, z_bytes=4):
    """Bytes and flops of one token-by-token step for every (batch, head).

    Per (batch, head): read and write M and S (4 d^2 floats), read q, k, v and
    three gates, write z.  Flops: M k, the S and M updates and M q, 2 d^2 each.
    """
    bh = w.B * w.H
    per_seq = 16 * w.d * w.d + 3 * w.d * in_bytes + 3 * 4 + w.d * z_bytes
    return bh * per_seq, bh * 8 * w.d * w.d, per_seq


FWD_PROFILES = {2: "linear_memory_fwd_ttt_linear_d64_b16", 3: "linear_memory_fwd_titans_d128_b64",
                4: "linear_memory_fwd_long_context_d128_b64"}


def measured_traffic(w, kind="forward"):
    """HBM bytes per launch from the committed counter summary under profiles/
    (TCC read and write requests by size, from separate rocprofv3 runs; see the
    summary for the commands), not measured in this run.

    The summary records the sha256 of the kernel source it was measured on; if
    the source has changed since (or the workload differs), the figure no
    longer describes this kernel and None is returned.
    """
    import hashlib
    if kind == "forward":
        if w.id not in FWD_PROFILES:
            return None
    elif w.id != (5 if kind in ("mlp", "deep3", "deep4") else 3):
        return None
    if kind in ("mlp", "deep3", "deep4"):
        name = {"mlp": "mlp_memory_fwd_deep_d64_h256_b16", "deep3": "deep_memory_fwd_depth3_d64_h256_b16",
                "deep4": "deep_memory_fwd_depth4_d64_h256_b16"}[kind]
        path = os.path.join(ROOT, "profiles", name + "_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_deep.hip")
    elif kind == "decode":
        path = os.path.join(ROOT, "profiles", "linear_memory_decode_titans_d128_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_decode.hip")
    elif kind == "cg_forward":
        path = os.path.join(ROOT, "profiles", "linear_memory_fwd_chunk_gates_titans_d128_b64_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_linear.hip")
    elif kind == "varlen":
        path = os.path.join(ROOT, "profiles", "linear_memory_fwd_varlen_titans_d128_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_linear.hip")
    elif kind in ("backward", "varlen_backward", "cg_backward"):
        name = {"backward": "linear_memory_train_titans_d128_b64",
                "varlen_backward": "linear_memory_train_varlen_titans_d128",
                "cg_backward": "linear_memory_train_chunk_gates_titans_d128_b64"}[kind]
        path = os.path.join(ROOT, "profiles", name + "_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_linear_bwd.hip")
    else:
        path = os.path.join(ROOT, "profiles", FWD_PROFILES[w.id] + "_traffic.json")
        src = os.path.join(ROOT, "test_neural_memory_amd", "csrc", "ttt_mem_linear.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def _oracle_worker(args):
    # Runs in a separate process: one BLAS thread, the oracle as it stands.
    q, k, v, th, et, al, b, W1, W2 = args[:9]
    chunk_gates = len(args) > 9 and args[9]
    M0 = args[10] if len(args) > 10 else None
    layers = args[11] if len(args) > 11 else None
    from threadpoolctl import threadpool_limits
    from oracle import deep_forward, linear_forward, linear_forward_chunk_gates, mlp_forward
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if layers is not None:
            deep_forward(q, k, v, th, et, al, layers, None, b=b)
        elif chunk_gates:
            linear_forward_chunk_gates(q, k, v, th, et, al, M0, None, b=b)
        elif W1 is None:
            linear_forward(q, k, v, th, et, al, M0, None, b=b)
        else:
            mlp_forward(q, k, v, th, et, al, W1, W2, None, None, b=b)
        return time.perf_counter() - t0


def cpu_baseline_decode(w, inp, tokens):
    """Time the float64 oracle with b = 1 (the token-by-token form) on every
    (batch, head) sequence for ``tokens`` tokens, in a process pool."""
    import multiprocessing as mp
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16))
    g = {k: to_numpy64(v) for k, v in inp.items() if k in ("q", "k", "v", "theta", "eta", "alpha")}
    B, H = w.B, w.H
    pairs = [(i // H, i % H) for i in range(B * H)]
    groups = [pairs[i::ncores] for i in range(ncores)]
    jobs = []
    for grp in groups:
        if not grp:
            continue
        bi = np.array([p[0] for p in grp])
        hi = np.array([p[1] for p in grp])
        jobs.append(tuple(g[x][bi, hi][..., :tokens, :] if g[x].ndim == 4 else g[x][bi, hi][..., :tokens]
                          for x in ("q", "k", "v", "theta", "eta", "alpha")) + (1, None, None))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(len(jobs)) as pool:
        per_job = pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    return {
        "value": B * tokens / wall,   # tokens/s, each token covering all H heads
        "unit": "tokens/s",
        "cores": len(jobs),
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"all {B * H} (batch, head) sequences, {tokens} tokens each, b=1 (token by token); "
                  f"float64 per-token NumPy loop, {len(jobs)} processes x 1 thread; wall {wall:.2f} s, "
                  f"busiest process {max(per_job):.2f} s; tokens/s = B * tokens / wall",
    }


def decode_main(args):
    """Token-by-token generation on the Titans shapes (one token per step, state carried in place)."""
    steps_total = 1 + args.steps   # token 0: parity step; then the K captured steps
    w = WORKLOADS[3].replace(T=steps_total)
    log(f"decode workload: {w} (one token per step, {steps_total} steps)")
    inp = make_inputs(w)
    B, H, d = w.B, w.H, w.d
    rng = np.random.default_rng(2003)
    M0 = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32))
    S0 = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.005).astype(np.float32))
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    # One [B, H, 1, d] slice per token, contiguous, prepared before timing.
    toks = []
    for t in range(steps_total):
        toks.append(tuple(dev[x][:, :, t:t + 1, :].contiguous() if dev[x].dim() == 4
                          else dev[x][:, :, t:t + 1].contiguous() for x in ("q", "k", "v", "theta", "eta", "alpha")))
    M = M0.cuda()
    S = S0.cuda()
    z = torch.empty(B, H, 1, d, dtype=torch.float32, device="cuda")

    # Parity of one step from the initial state, every row of sequence 0.
    from oracle import linear_forward
    tm.decode(*toks[0], M, S, out=(z, M, S))
    torch.cuda.synchronize()
    g = [to_numpy64(x[0, 0].cpu()) for x in toks[0]]
    zo, Mo, So = linear_forward(*g, to_numpy64(M0[0, 0]), to_numpy64(S0[0, 0]), b=1)
    errs = [float(np.max(np.abs(to_numpy64(x[0, 0].cpu()) - r)) / np.sqrt(np.mean(r ** 2)))
            for x, r in ((z[:, :, 0], zo[0]), (M, Mo), (S, So))]
    parity = max(errs)
    log(f"parity of step 0 (sequence 0, all rows): z {errs[0]:.3e}, M {errs[1]:.3e}, S {errs[2]:.3e}")

    # Eager steps are bound by host submission (microsecond kernels); a
    # generation loop replays captured steps.  The K steps are captured once
    # into a HIP graph (kernel launches only); the warmup replays it until W
    # untimed steps have run, then one replay is timed.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            tm.decode(*toks[1 + i], M, S, out=(z, M, S))
    torch.cuda.synchronize()
    for _ in range((args.warmup + args.steps - 1) // args.steps):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    avg_launch_ms = ms_per_step
    nbytes, flops, per_seq = algorithmic_work_decode(w)
    achieved_gbs = nbytes / (avg_launch_ms * 1e-3) / 1e9
    log(f"graph of {args.steps} steps: {ms_per_step * 1e3:.2f} us per step; wall/step {t_wall / args.steps * 1e3:.4f} ms")
    log(f"algorithmic bytes/step {nbytes / 1e6:.2f} MB -> {achieved_gbs:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        wc = WORKLOADS[3].replace(T=4096)   # a longer token stream of the same recipe for the host sample
        cpu = cpu_baseline_decode(wc, make_inputs(wc), wc.T)
        log(f"cpu baseline: {cpu}")
    result = {
        "metric": "decode tokens/s at B=4,H=16,d=128 (one token per step, state carried)",
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "titans-linear-decode", "B": B, "H": H, "d": d, "tokens_per_step": 1,
                   "inputs": "bf16 q,k,v; f32 gates", "arithmetic": "f32", "state": "f32 in place",
                   "z": "f32", "head_tokens_per_s": B * H / (ms_per_step * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(w, "decode"),
                     "traffic_unit": "bytes/launch", "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(result), flush=True)


def algorithmic_work_backward(w, in_bytes=2, chunk_gates=False):
    """Bytes and flops the method must move / do for one backward pass.

    Per (batch, head, token): read q, k, v, three gates and dz; write dq, dk,
    dv (float32) and three gate gradients.  Per (batch, head): write dM0, dS0
    (no state cotangent is given).  Flops, per head-token in the dual form:
    the carry's dE and state updates (5 products of 2 b d^2 per chunk: K dM^T,
    K dS^T, Q^T (A.dZ), Q^T (c.dZ), K^T dE) and the chunk gradients (6: K M0^T,
    dZ M0, dZ S0, dE M0, E dM, E dS) are 22 d^2; the intra-chunk products
    (P^T dZ, Q K^T twice, dZ E^T, DL K, DL^T Q) add 12 b d.  The checkpointed
    states the implementation writes and reads are not counted.  With chunk
    gates, the gates and their gradients are one triple per chunk.
    """
    ht = w.B * w.H * w.T
    gate_tok = 0 if chunk_gates else 3 * 4 + 3 * 4
    per_tok = 3 * w.d * in_bytes + w.d * 4 + 3 * w.d * 4 + gate_tok
    gates = w.B * w.H * ((w.T + w.b - 1) // w.b) * (3 * 4 + 3 * 4) if chunk_gates else 0
    state = w.B * w.H * w.d * w.d * 4 * 2
    flops = ht * (22 * w.d * w.d + 12 * w.b * w.d)
    return ht * per_tok + gates + state, flops, per_tok


def _oracle_train_worker(args):
    # One BLAS thread; the oracle's forward and backward, one sequence at a time.
    seqs, b = args[:2]
    chunk_gates = len(args) > 2 and args[2]
    from threadpoolctl import threadpool_limits
    from oracle import linear_backward, linear_backward_chunk_gates, linear_forward, linear_forward_chunk_gates
    fwd = linear_forward_chunk_gates if chunk_gates else linear_forward
    bwd = linear_backward_chunk_gates if chunk_gates else linear_backward
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for q, k, v, th, et, al, dz in seqs:
            fwd(q, k, v, th, et, al, None, None, b=b)
            bwd(q, k, v, th, et, al, dz, None, None, None, None, b=b)
        return time.perf_counter() - t0


def cpu_baseline_backward(w, inp, cot, pairs=64, tokens=2048, chunk_gates=False):
    """Time the float64 oracle (forward, then backward) on `pairs` (batch, head)
    sequences cut to their first `tokens` tokens, in a process pool."""
    import multiprocessing as mp
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16))
    g = {k: to_numpy64(v) for k, v in inp.items() if k in ("q", "k", "v", "theta", "eta", "alpha")}
    dz = to_numpy64(cot["dz"])
    B, H = w.B, w.H
    sel = [(i // H, i % H) for i in range(B * H)][:pairs]
    jobs = [([], w.b, chunk_gates) for _ in range(ncores)]
    gt = (tokens + w.b - 1) // w.b if chunk_gates else tokens
    for i, (bi, hi) in enumerate(sel):
        jobs[i % ncores][0].append(tuple(g[x][bi, hi, :tokens] for x in ("q", "k", "v"))
                                   + tuple(g[x][bi, hi, :gt] for x in ("theta", "eta", "alpha"))
                                   + (dz[bi, hi, :tokens],))
    jobs = [j for j in jobs if j[0]]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(len(jobs)) as pool:
        per_job = pool.map(_oracle_train_worker, jobs)
    wall = time.perf_counter() - t0
    head_tokens = len(sel) * tokens
    return {
        "value": head_tokens / H / wall,   # training tokens/s, each token covering all H heads
        "unit": "tokens/s",
        "cores": len(jobs),
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"{len(sel)} of {B * H} (batch, head) sequences, first {tokens} of T={w.T} tokens, all "
                  f"d={w.d} rows; float64 per-token NumPy forward then reverse-mode backward"
                  f"{' (chunk-shared gates)' if chunk_gates else ''}, "
                  f"{len(jobs)} processes x 1 thread; wall {wall:.2f} s, busiest process {max(per_job):.2f} s; "
                  f"tokens/s = sampled head-tokens / H / wall",
    }


def backward_main(args):
    """One training step of the Titans linear memory: forward with checkpoints +
    backward; with ``--chunk-gates``, gates shared by each chunk's tokens."""
    w = WORKLOADS[3]
    cg = args.chunk_gates
    B, H, T, d = w.B, w.H, w.T, w.d
    log(f"training step workload {w}{' with chunk-shared gates' if cg else ''}")
    inp = make_inputs(w)
    if cg:
        set_chunk_gates(w, inp)
    cot = make_cotangents(w, states=False)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    dz = cot["dz"].cuda()
    args_ = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    z = torch.empty(B, H, T, d, dtype=torch.float32, device="cuda")
    MT = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
    ST = torch.empty_like(MT)
    nch = (T + w.b - 1) // w.b
    ckpt = tm.new_ckpt(dev["q"], w.b)
    work = torch.empty(tm.backward_work_bytes(dev["q"], w.b), dtype=torch.uint8, device="cuda")
    gl = nch if cg else T
    outs = [torch.empty(B, H, T, d, dtype=torch.float32, device="cuda") for _ in range(3)] + \
           [torch.empty(B, H, gl, dtype=torch.float32, device="cuda") for _ in range(3)] + \
           [torch.empty(B, H, d, d, dtype=torch.float32, device="cuda") for _ in range(2)]
    if cg:
        fwd = lambda: tm.forward_chunk_gates(*args_, b=w.b, out=(z, MT, ST), ckpt=ckpt)  # noqa: E731
    else:
        fwd = lambda: tm.forward_train(*args_, b=w.b, out=(z, MT, ST), ckpt=ckpt)  # noqa: E731
    bwd = lambda: tm.backward(*args_, ckpt, dz, b=w.b, work=work, out=outs, chunk_gates=cg)  # noqa: E731
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    # Timed region: K training steps on torch's current stream (the stream
    # the library launches on), events around the forward and the backward.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        fwd()
        ev[i][1].record()
        bwd()
        ev[i][2].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    nbytes, flops, _ = algorithmic_work_backward(w, chunk_gates=cg)
    fbytes, _, _ = algorithmic_work(w)
    achieved_gbs = nbytes / (bwd_ms * 1e-3) / 1e9
    achieved_tflops = flops / (bwd_ms * 1e-3) / 1e12
    ck_bytes = ckpt.numel() * ckpt.element_size()
    log(f"forward with checkpoints {fwd_ms * 1e3:.1f} us (algorithmic {fbytes / (fwd_ms * 1e-3) / 1e9:.0f} GB/s "
        f"+ {ck_bytes / 1e9:.2f} GB of checkpoints), backward {bwd_ms * 1e3:.1f} us; wall/step "
        f"{t_wall / args.steps * 1e3:.3f} ms")
    log(f"backward algorithmic bytes {nbytes / 1e9:.3f} GB -> {achieved_gbs:.0f} GB/s; flops {flops / 1e9:.1f} "
        f"GFLOP -> {achieved_tflops:.1f} TFLOP/s")

    # Sampled parity: the last two chunks of sequences (0, 0) and (B-1, H-1).
    # No loss reaches past them, so their gradients are the oracle's on that
    # window started from the oracle's own state after the chunks before it.
    from oracle import linear_backward, linear_backward_chunk_gates, linear_forward, linear_forward_chunk_gates
    lf = linear_forward_chunk_gates if cg else linear_forward
    lb = linear_backward_chunk_gates if cg else linear_backward
    t0 = (nch - 2) * w.b
    g0 = nch - 2 if cg else t0   # first gate entry of the window
    errs = []
    for (bi, hi) in ((0, 0), (B - 1, H - 1)):
        g = {k: to_numpy64(v[bi, hi]) for k, v in inp.items() if v is not None}
        _, Ms, Ss = lf(g["q"][:t0], g["k"][:t0], g["v"][:t0], g["theta"][:g0], g["eta"][:g0],
                       g["alpha"][:g0], None, None, b=w.b)
        ref = lb(g["q"][t0:], g["k"][t0:], g["v"][t0:], g["theta"][g0:], g["eta"][g0:],
                 g["alpha"][g0:], to_numpy64(cot["dz"][bi, hi, t0:]), None, None, Ms, Ss, b=w.b)
        for i, (x, r) in enumerate(zip(outs[:6], ref[:6])):
            xg = x[bi, hi, (t0 if i < 3 else g0):].double().cpu().numpy()
            errs.append(float(np.max(np.abs(xg - r)) / np.sqrt(np.mean(r ** 2))))
    parity = max(errs)
    log(f"sampled parity (last two chunks of two sequences, every gradient): max|d|/rms = {parity:.3e}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_backward(w, inp, cot, chunk_gates=cg)
        log(f"cpu baseline: {cpu}")
    result = {
        "metric": "training tokens/s (forward + backward) at H=16,d=128,b=64" + (" (chunk-shared gates)" if cg else ""),
        "value": B * T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "titans-linear-train" + ("-chunk-gates" if cg else ""), "B": B, "H": H, "T": T,
                   "d": d, "b": w.b,
                   "inputs": f"bf16 q,k,v; f32 gates{' per chunk' if cg else ''}; f32 dz (seeded N(0,1))",
                   "accumulate": "f32",
                   "gradients": "f32", "checkpoints": "fp16", "forward_ms": fwd_ms, "backward_ms": bwd_ms,
                   "checkpoint_bytes": ck_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(w, "cg_backward" if cg else "backward"),
                     "traffic_unit": "bytes/launch",
                     "algorithmic_bytes": nbytes, "kernel": "backward pass (carry walk + chunk gradients)",
                     "mfma_frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(result), flush=True)


def varlen_main(args):
    """Packed variable-length documents with the Titans recipe: H=16, d=128, b=64,
    B*T = 32768 tokens per head split into documents of seeded lengths."""
    wv = WORKLOADS[3].replace(B=1, T=4 * 8192)
    lengths = varlen_lengths(wv.T, mean=args.doc_mean)
    N, H, T, d = len(lengths), wv.H, wv.T, wv.d
    log(f"varlen workload: {N} documents, lengths min {min(lengths)} median {int(np.median(lengths))} "
        f"max {max(lengths)}, {T} tokens per head, H={H} d={d} b={wv.b}")
    inp = make_inputs(wv)
    dev = {k: v[0].cuda() for k, v in inp.items() if v is not None}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    z = torch.empty(H, T, d, dtype=torch.float32, device="cuda")
    MT = torch.empty(N, H, d, d, dtype=torch.float32, device="cuda")
    ST = torch.empty_like(MT)
    call = lambda: tm.forward_varlen(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],  # noqa: E731
                                     cu, b=wv.b, out=(z, MT, ST))
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # Timed region: K back-to-back launches between two HIP events on the
    # library's stream (no event between launches).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    avg_launch_ms = ms_per_step
    per_tok = 3 * d * 2 + 3 * 4 + d * 4
    nbytes = H * T * per_tok + N * H * d * d * 4 * 2
    achieved_gbs = nbytes / (avg_launch_ms * 1e-3) / 1e9
    log(f"launch average {avg_launch_ms * 1e3:.1f} us; "
        f"algorithmic bytes/launch {nbytes / 1e6:.1f} MB -> {achieved_gbs:.0f} GB/s")
    # Parity: the first two documents of head 0, every row.
    from oracle import linear_forward
    g = {k: to_numpy64(v[0, 0]) for k, v in inp.items() if v is not None}
    errs = []
    for s_ in range(min(2, N)):
        t0, t1 = int(sum(lengths[:s_])), int(sum(lengths[:s_ + 1]))
        zo = linear_forward(g["q"][t0:t1], g["k"][t0:t1], g["v"][t0:t1], g["theta"][t0:t1], g["eta"][t0:t1],
                            g["alpha"][t0:t1], None, None, b=wv.b)[0]
        errs.append(float(np.max(np.abs(z[0, t0:t1].double().cpu().numpy() - zo)) / np.sqrt(np.mean(zo ** 2))))
    parity = max(errs)
    log(f"sampled parity (documents 0-1, head 0): max|dz|/rms = {parity:.3e}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_varlen(inp, lengths, H, wv.b)
        log(f"cpu baseline: {cpu}")
    result = {
        "metric": "packed-document tokens/s at H=16,d=128,b=64 (variable-length documents)",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "titans-linear-varlen", "documents": N, "tokens_per_head": T, "H": H, "d": d,
                   "b": wv.b, "lengths": f"lognormal(sigma 1) around {args.doc_mean}, clipped to [1, 8192], seed 3001",
                   "inputs": "bf16 q,k,v; f32 gates", "accumulate": "f32", "state": "f32", "z": "f32"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS,
                     # the committed counters describe the default length mix only
                     "traffic": measured_traffic(wv, "varlen") if args.doc_mean == 1024 else None,
                     "traffic_unit": "bytes/launch", "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(result), flush=True)


def varlen_train_main(args):
    """One training step over packed documents with the Titans recipe (the
    ``--varlen`` workload): the forward that keeps every document's chunk-start
    states, then the backward pass over the same documents."""
    wv = WORKLOADS[3].replace(B=1, T=4 * 8192)
    lengths = varlen_lengths(wv.T, mean=args.doc_mean)
    N, H, T, d, b = len(lengths), wv.H, wv.T, wv.d, wv.b
    log(f"varlen training workload: {N} documents, lengths min {min(lengths)} median {int(np.median(lengths))} "
        f"max {max(lengths)}, {T} tokens per head, H={H} d={d} b={b}")
    inp = make_inputs(wv)
    dev = {k: v[0].cuda() for k, v in inp.items() if v is not None}
    dz_h = make_cotangents(wv, states=False)["dz"][0]
    dz = dz_h.cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    args_ = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    z = torch.empty(H, T, d, dtype=torch.float32, device="cuda")
    MT = torch.empty(N, H, d, d, dtype=torch.float32, device="cuda")
    ST = torch.empty_like(MT)
    ckpt = tm.new_ckpt_varlen(dev["q"], cu, b)
    work = torch.empty(tm.backward_work_bytes(dev["q"], b, cu), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(H, T, d, dtype=torch.float32, device="cuda") for _ in range(3)] + \
           [torch.empty(H, T, dtype=torch.float32, device="cuda") for _ in range(3)] + \
           [torch.empty(N, H, d, d, dtype=torch.float32, device="cuda") for _ in range(2)]
    fwd = lambda: tm.forward_varlen(*args_, cu, b=b, out=(z, MT, ST), ckpt=ckpt)  # noqa: E731
    bwd = lambda: tm.backward_varlen(*args_, cu, ckpt, dz, b=b, work=work, out=outs)  # noqa: E731
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        fwd()
        ev[i][1].record()
        bwd()
        ev[i][2].record()
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    # Algorithmic bytes of the backward, as for the dense step: inputs and dz
    # read once, every token gradient written once, dM0 and dS0 per document.
    per_tok = 3 * d * 2 + 3 * 4 + d * 4 + 3 * d * 4 + 3 * 4
    nbytes = H * T * per_tok + N * H * d * d * 4 * 2
    achieved_gbs = nbytes / (bwd_ms * 1e-3) / 1e9
    log(f"forward with checkpoints {fwd_ms * 1e3:.1f} us, backward {bwd_ms * 1e3:.1f} us; backward algorithmic "
        f"bytes {nbytes / 1e9:.3f} GB -> {achieved_gbs:.0f} GB/s")
    # Parity: documents 0 and 1 on heads 0 and H-1, every gradient, against the
    # oracle's backward of each document from a zero state.
    from oracle import linear_backward
    errs = []
    for h in (0, H - 1):
        g = {k: to_numpy64(v[0, h]) for k, v in inp.items() if v is not None}
        dzn = to_numpy64(dz_h[h])
        for s_ in range(min(2, N)):
            t0, t1 = int(sum(lengths[:s_])), int(sum(lengths[:s_ + 1]))
            ref = linear_backward(g["q"][t0:t1], g["k"][t0:t1], g["v"][t0:t1], g["theta"][t0:t1],
                                  g["eta"][t0:t1], g["alpha"][t0:t1], dzn[t0:t1], None, None, None, None, b=b)
            got = [x[h, t0:t1] for x in outs[:6]] + [outs[6][s_, h], outs[7][s_, h]]
            for x, r in zip(got, ref):
                xg = x.double().cpu().numpy()
                errs.append(float(np.max(np.abs(xg - r)) / np.sqrt(np.mean(r ** 2))))
    parity = max(errs)
    log(f"sampled parity (documents 0-1, heads 0 and {H - 1}, every gradient): max|d|/rms = {parity:.3e}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_varlen_train(inp, dz_h, lengths, H, b)
        log(f"cpu baseline: {cpu}")
    result = {
        "metric": "packed-document training tokens/s (forward + backward) at H=16,d=128,b=64",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "titans-linear-varlen-train", "documents": N, "tokens_per_head": T, "H": H,
                   "d": d, "b": b, "lengths": f"lognormal(sigma 1) around {args.doc_mean}, clipped to [1, 8192], seed 3001",
                   "inputs": "bf16 q,k,v; f32 gates; f32 dz (seeded N(0,1))", "accumulate": "f32",
                   "gradients": "f32", "checkpoints": "fp16", "forward_ms": fwd_ms, "backward_ms": bwd_ms,
                   "checkpoint_bytes": ckpt.numel() * ckpt.element_size()},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wv, "varlen_backward") if args.doc_mean == 1024 else None,
                     "traffic_unit": "bytes/launch", "algorithmic_bytes": nbytes,
                     "kernel": "backward pass (carry walk + chunk gradients)"},
        "cpu_baseline": cpu,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_varlen_train(inp, dz, lengths, H, b, docs=8):
    """Time the float64 oracle (forward, then backward) on the first `docs`
    documents of every head, in a process pool."""
    import multiprocessing as mp
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16))
    g = {k: to_numpy64(v[0]) for k, v in inp.items() if k in ("q", "k", "v", "theta", "eta", "alpha")}
    dzn = to_numpy64(dz)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    nd = min(docs, len(lengths))
    jobs = [([], b) for _ in range(ncores)]
    for i, (s_, h) in enumerate((s_, h) for s_ in range(nd) for h in range(H)):
        t0, t1 = cu[s_], cu[s_ + 1]
        jobs[i % ncores][0].append(tuple(g[x][h, t0:t1] for x in ("q", "k", "v", "theta", "eta", "alpha"))
                                   + (dzn[h, t0:t1],))
    jobs = [j for j in jobs if j[0]]
    ctx = mp.get_context("fork")
    t0w = time.perf_counter()
    with ctx.Pool(len(jobs)) as pool:
        per_job = pool.map(_oracle_train_worker, jobs)
    wall = time.perf_counter() - t0w
    tokens = int(cu[nd])
    return {
        "value": tokens / wall,   # training tokens/s, each token covering all H heads
        "unit": "tokens/s",
        "cores": len(jobs),
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"first {nd} of {len(lengths)} documents ({tokens} tokens) on all {H} heads; float64 per-token "
                  f"NumPy forward then reverse-mode backward, {len(jobs)} processes x 1 thread; wall {wall:.2f} s, "
                  f"busiest process {max(per_job):.2f} s; tokens/s = sampled tokens / wall",
    }


def cpu_baseline_varlen(inp, lengths, H, b, docs=12):
    """Time the float64 oracle on the first `docs` documents of every head, in a process pool."""
    import multiprocessing as mp
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16))
    g = {k: to_numpy64(v[0]) for k, v in inp.items() if k in ("q", "k", "v", "theta", "eta", "alpha")}
    cu = np.concatenate([[0], np.cumsum(lengths)])
    pairs = [(s_, h) for s_ in range(min(docs, len(lengths))) for h in range(H)]
    jobs = [[] for _ in range(ncores)]
    for i, (s_, h) in enumerate(pairs):
        t0, t1 = cu[s_], cu[s_ + 1]
        jobs[i % ncores].append(tuple(g[x][h:h + 1, t0:t1] for x in ("q", "k", "v", "theta", "eta", "alpha")))
    work = []
    for grp in jobs:
        for item in grp:
            work.append(item + (b, None, None))
    ctx = mp.get_context("fork")
    t0w = time.perf_counter()
    with ctx.Pool(ncores) as pool:
        per_job = pool.map(_oracle_worker, work)
    wall = time.perf_counter() - t0w
    tokens = int(cu[min(docs, len(lengths))])
    return {
        "value": tokens / wall,   # tokens/s, each token covering all H heads
        "unit": "tokens/s",
        "cores": ncores,
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"first {min(docs, len(lengths))} of {len(lengths)} documents ({tokens} tokens) on all {H} heads; "
                  f"float64 per-token NumPy loop, {ncores} processes x 1 thread; wall {wall:.2f} s, "
                  f"busiest task {max(per_job):.2f} s; tokens/s = sampled tokens / wall",
    }


def cpu_baseline(w, inp, heads, chunk_gates=False, layers=None):
    """Time the float64 oracle on ``heads`` (batch, head) pairs with full T, in a process pool
    (``layers``: the initial layers of a deeper memory, run by the oracle's deep_forward)."""
    import multiprocessing as mp
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16))
    g = {k: to_numpy64(v) for k, v in inp.items()
         if v is not None and k in ("q", "k", "v", "theta", "eta", "alpha", "W1", "W2", "M0")}
    B, H = w.B, w.H
    pairs = [(i // H, i % H) for i in range(B * H)][:heads]
    groups = [pairs[i::ncores] for i in range(ncores)]
    jobs = []
    for grp in groups:
        if not grp:
            continue
        bi = np.array([p[0] for p in grp])
        hi = np.array([p[1] for p in grp])
        jobs.append(tuple(g[x][bi, hi] for x in ("q", "k", "v", "theta", "eta", "alpha")) + (w.b,)
                    + ((g["W1"][bi, hi], g["W2"][bi, hi]) if w.hidden else (None, None)) + (chunk_gates,)
                    + ((g["M0"][bi, hi] if "M0" in g else None),)
                    + ((None if layers is None else [to_numpy64(x)[bi, hi] for x in layers]),))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(len(jobs)) as pool:
        per_job = pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    head_tokens = len(pairs) * w.T
    return {
        "value": head_tokens / H / wall,   # tokens/s, each token covering all H heads
        "unit": "tokens/s",
        "cores": len(jobs),
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"{len(pairs)} of {B * H} (batch, head) sequences, full T={w.T}"
                  f"{'' if w.hidden else f', all d={w.d} rows'}; "
                  f"float64 per-token NumPy loop, {len(jobs)} processes x 1 thread; "
                  f"wall {wall:.2f} s, busiest process {max(per_job):.2f} s; "
                  f"tokens/s = sampled head-tokens / H / wall",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU's clocks ramp up over the first ~20 ms of back-to-back launches
    # (a launch of the Titans workload falls from ~290 us to ~220 us); the
    # default warmup runs past that ramp.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--depth", type=int, default=2, choices=[1, 2, 3, 4],
                    help="layers of the deep memory (workload 5); 3 and 4 start from seeded N(0, 1/fan_in) layers, "
                         "1 is the linear memory on the same inputs (the depth sweep's first point)")
    ap.add_argument("--decode", action="store_true",
                    help="time token-by-token generation (primal form) on the Titans shapes instead")
    ap.add_argument("--varlen", action="store_true",
                    help="time packed variable-length documents with the Titans recipe instead")
    ap.add_argument("--backward", action="store_true",
                    help="time one training step (forward with checkpoints + backward) on the Titans workload")
    ap.add_argument("--doc-mean", type=int, default=1024,
                    help="--varlen: mean document length (lognormal lengths; 1024 packs 31 documents per head)")
    ap.add_argument("--chunk-gates", action="store_true",
                    help="time the Titans forward with gates shared by each chunk's tokens instead")
    ap.add_argument("--z-f32", action="store_true",
                    help="time the float32-z entry point (bf16 inputs) instead of the bf16-z one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="(batch, head) sequences in the oracle sample (0: 64 for the linear memory, "
                         "16 for the deep memory)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed region, run 3 plain device copies of MIB MiB (float32 read once, "
                         "written once) so that hardware byte counters can be scaled against known traffic")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the memory forward needs no "
              "collective and this implementation runs on a single MI355X; shard (batch, head) pairs across "
              "processes to use more GPUs.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x elementwise copy of {n * 4} bytes read + {n * 4} bytes written")
        del src, dst
    if args.decode:
        decode_main(args)
        return
    if args.varlen and args.backward:
        varlen_train_main(args)
        return
    if args.varlen:
        varlen_main(args)
        return
    if args.backward:
        backward_main(args)
        return
    w = WORKLOADS[args.workload]
    if args.depth == 1 and w.hidden:
        # Memory depth 1: the linear memory (d x d state) on the deep workload's inputs.
        w = w.replace(hidden=0)
    if args.chunk_gates and args.workload != 3:
        print("--chunk-gates runs on the Titans workload (3)", file=sys.stderr)
        sys.exit(2)
    deep = w.hidden > 0
    zdt = torch.float32 if args.z_f32 else torch.bfloat16
    zname = "f32" if args.z_f32 else "bf16"
    log(f"workload {w}{' with chunk-shared gates' if args.chunk_gates else ''}; z {zname}")
    inp = make_inputs(w)
    if args.chunk_gates:
        set_chunk_gates(w, inp)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    B, H, T, d = w.B, w.H, w.T, w.d
    z = torch.empty(B, H, T, d, dtype=zdt, device="cuda")
    if args.depth != 2 and args.workload != 5:
        print("--depth applies to the deep-memory workload (5)", file=sys.stderr)
        sys.exit(2)
    deep_layers = None
    if deep and args.depth > 2:
        if args.z_f32:
            print("--depth 3 and 4 write bf16 z", file=sys.stderr)
            sys.exit(2)
        deep_layers = make_deep_layers(w, args.depth)
        W0 = tm.deep_pack([x.cuda() for x in deep_layers])
        WT, ST = torch.empty_like(W0), torch.empty_like(W0)
        dwork = tm.new_deep_work(B, H, d, w.hidden, args.depth, "cuda")
        call = lambda: tm.deep_forward(  # noqa: E731
            dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], W0, None, hidden=w.hidden,
            depth=args.depth, b=w.b, work=dwork, out=(z, WT, ST))
    elif deep:
        outs = (z,) + tuple(torch.empty_like(dev[k]) for k in ("W1", "W2", "W1", "W2"))
        call = lambda: tm.ttt_mem_mlp_forward_bf16(  # noqa: E731
            dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], dev["W1"], dev["W2"],
            b=w.b, out=outs, z_dtype=zdt)
    else:
        # The workloads start from explicit states (zeros where the recipe
        # gives none), so the launch reads M0 and S0 as the algorithmic
        # bytes count them.
        M0 = dev["M0"] if dev.get("M0") is not None else torch.zeros(B, H, d, d, device="cuda")
        S0 = torch.zeros(B, H, d, d, device="cuda")
        MT = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
        ST = torch.empty(B, H, d, d, dtype=torch.float32, device="cuda")
        if args.chunk_gates:
            if args.z_f32:
                print("--chunk-gates writes float32 z already", file=sys.stderr)
                sys.exit(2)
            z = torch.empty(B, H, T, d, dtype=torch.float32, device="cuda")
            zname = "f32"
            call = lambda: tm.forward_chunk_gates(  # noqa: E731
                dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], M0, S0, b=w.b,
                out=(z, MT, ST))
        else:
            call = lambda: tm.forward(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"],  # noqa: E731
                                      dev["alpha"], M0, S0, b=w.b, out=(z, MT, ST), z_dtype=zdt)
    z_bytes = 2 if zname == "bf16" else 4

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # Timed region: K steps, one kernel launch each, back to back on torch's
    # current stream (the stream the library launches on), between two HIP
    # events; no event sits between launches, so the launch average is the
    # events' interval over K (launch gaps included).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    avg_launch_ms = ms_per_step

    if deep:
        nbytes, flops, per_tok = algorithmic_work_mlp(w, z_bytes=z_bytes, depth=args.depth)
        traffic = measured_traffic(w, "mlp" if args.depth == 2 else f"deep{args.depth}") if not args.z_f32 else None
    else:
        nbytes, flops, per_tok = algorithmic_work(w, z_bytes=z_bytes, reads_state=True)
        traffic = measured_traffic(w) if not args.z_f32 else None
        if args.chunk_gates:
            # Three gate floats per chunk instead of per token.
            nbytes -= w.B * w.H * (w.T - (w.T + w.b - 1) // w.b) * 12
            traffic = measured_traffic(w, "cg_forward")
    achieved_gbs = nbytes / (avg_launch_ms * 1e-3) / 1e9
    achieved_tflops = flops / (avg_launch_ms * 1e-3) / 1e12
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    log(f"launch average {avg_launch_ms * 1e3:.1f} us; wall/step {t_wall / args.steps * 1e3:.3f} ms")
    log(f"algorithmic bytes/launch {nbytes / 1e6:.1f} MB ({per_tok} B per head-token + state) -> "
        f"{achieved_gbs:.0f} GB/s; flops/launch {flops / 1e9:.1f} GFLOP -> {achieved_tflops:.1f} TFLOP/s")

    # Sampled parity check of the timed outputs against the oracle: the first
    # and last (batch, head) sequences, and for the linear memory a few value
    # rows of each (rows are independent problems).
    from oracle import deep_forward, linear_forward, linear_forward_chunk_gates, mlp_forward
    errs = []
    for (bi, hi) in ((0, 0), (B - 1, H - 1)):
        g = {k: to_numpy64(v[bi, hi]) for k, v in inp.items() if v is not None}
        if deep_layers is not None:
            zo = deep_forward(g["q"], g["k"], g["v"], g["theta"], g["eta"], g["alpha"],
                              [to_numpy64(x[bi, hi]) for x in deep_layers], None, b=w.b)[0]
            zg = z[bi, hi].double().cpu().numpy()
            what = "sequences (0,0) and (B-1,H-1), all columns"
        elif deep:
            zo = mlp_forward(g["q"], g["k"], g["v"], g["theta"], g["eta"], g["alpha"], g["W1"], g["W2"], b=w.b)[0]
            zg = z[bi, hi].double().cpu().numpy()
            what = "sequences (0,0) and (B-1,H-1), all columns"
        else:
            rows = np.r_[0:4, d - 4:d]
            M0s = g["M0"][rows] if "M0" in g else None
            lf = linear_forward_chunk_gates if args.chunk_gates else linear_forward
            zo = lf(g["q"], g["k"], g["v"][:, rows], g["theta"], g["eta"], g["alpha"], M0s, None, b=w.b)[0]
            zg = z[bi, hi][:, rows].double().cpu().numpy()
            what = f"sequences (0,0) and (B-1,H-1), rows {[int(r) for r in rows]}"
        errs.append(float(np.max(np.abs(zg - zo)) / np.sqrt(np.mean(zo ** 2))))
    parity = max(errs)
    log(f"sampled parity ({what}): max|dz|/rms = {parity:.3e}")

    cpu = None
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or (16 if deep else min(64, B * H))
        cw = w if w.T <= 8192 else w.replace(T=8192)   # long sequences: the oracle on their first 8192 tokens
        cpu = cpu_baseline(cw, inp if cw is w else _head_slice(inp, cw.T), heads, chunk_gates=args.chunk_gates,
                           layers=deep_layers)
        log(f"cpu baseline: {cpu}")

    if deep:
        metric = f"deep-memory tokens/s at H={H},d={d},hidden={w.hidden},b={w.b}" + (
            f",depth={args.depth}" if args.depth != 2 else "")
        roofline = {"bound": "mfma", "achieved": achieved_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                    "traffic_unit": "bytes/launch", "traffic_source": "profiles/ counter summary",
                    "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                    "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
                    "launch_us": avg_launch_ms * 1e3}
        cfg = {"workload": w.name + (f"-depth{args.depth}" if args.depth != 2 else ""), "B": B, "H": H, "T": T,
               "d": d, "hidden": w.hidden, "depth": args.depth, "b": w.b,
               "inputs": "bf16 q,k,v; f32 gates", "accumulate": "f32", "weights": "f32", "z": zname,
               "head_tokens_per_s": B * H * T / (ms_per_step * 1e-3)}
    else:
        metric = (f"memory-layer tokens/s at H={H},d={d},b={w.b}"
                  + (" (chunk-shared gates)" if args.chunk_gates else "")
                  + (" (memory depth 1 on the deep-memory inputs)" if args.depth == 1 else ""))
        roofline = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved_gbs / HBM_PEAK_GBS,
                    "traffic": traffic, "traffic_unit": "bytes/launch",
                    "traffic_source": "profiles/ counter summary", "algorithmic_bytes": nbytes,
                    "algorithmic_flops": flops,
                    "frac_of_step": nbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "mfma_frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS,
                    "launch_us": avg_launch_ms * 1e3}
        cfg = {"workload": w.name + ("-chunk-gates" if args.chunk_gates else "") + ("-depth1" if args.depth == 1 else ""),
               "B": B, "H": H, "T": T, "d": d,
               "b": w.b, "inputs": "bf16 q,k,v; f32 gates" + (" per chunk" if args.chunk_gates else ""),
               "accumulate": "f32", "state": "f32 (M0, S0 read)", "z": zname,
               "head_tokens_per_s": B * H * T / (ms_per_step * 1e-3)}
    result = {
        "metric": metric,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(result), flush=True)


def _head_slice(inp, T):
    """The inputs cut to their first T tokens (for the oracle sample of long sequences)."""
    out = {}
    for k, v in inp.items():
        if v is None or k in ("M0", "S0", "W1", "W2", "S1", "S2"):
            out[k] = v
        elif v.dim() == 4:
            out[k] = v[:, :, :T].contiguous()
        else:
            out[k] = v[:, :, :T].contiguous()
    return out


if __name__ == "__main__":
    main()
