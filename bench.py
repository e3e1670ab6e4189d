#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X: decode state GB/s and prompt-form tokens/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one gdn_decode_step call over the batched-decode workload (B = 64
sequences x H = 16 heads, bf16 q/k/v, fp32 g/beta, fp32 state [64,16,128,128]
updated in place), each step with its own freshly drawn token.  W untimed
steps run first; the K steps are captured as one HIP graph (so that host
launch cost does not pace the GPU), replayed once untimed, and then replayed
once more between two device synchronisations, timed by device events on the
replay's stream.  `value` is the state traffic those K steps move (2 x 64 KiB
per head-step) per second, `ms_per_step` their time over K and
`roofline.achieved` their algorithmic bytes per launch over the same time.
With one state batch updated in place, the 64 MiB state stays in the 256 MB
last-level cache; the same steps over eight batches in turn (512 MiB), with
the non-temporal state form, give `roofline_state_from_hbm`.

The same run times the prompt form (gdn_chunk_prefill) on the large prefill
(B=8, H=32, T=16384, chunk 64, bf16, zero S0) and on the long, packed
variable-length and speculative-verify workloads, and reports their tokens/s
and roofline fractions under "prefill".  Each such figure is the median over
three runs of --prefill-iters back-to-back calls between one pair of events,
so that the host's launch work overlaps the GPU's.  All inputs are seeded
synthetic draws made on the device before any timing starts.

The CPU oracle is timed on a bounded sample of the decode workload (and of the
large prefill) on this host's cores as `cpu_baseline`; it is a reported
baseline, not a target.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
BF16_PEAK = 2.5166e15        # flop/s, dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
DK = DV = 128
STATE_BYTES = DK * DV * 4    # one fp32 head state


# What the bf16 prompt-form legs compute in: matrix-core products on fp16
# operands (hi + lo pairs where the recurrence needs them) and bf16 values,
# fp32 accumulation, fp32 state.
PREFILL_ARITH = ("bf16 io; matrix-core products on fp16 operands (split into hi + lo "
                 "pairs where needed) and bf16 values, fp32 accumulation and state")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(lengths, H, C):
    """Algorithmic flops of the chunk form: per chunk of c real tokens,
    6 c dk dv (state products and the state update) + 2 c^2 (dk + dv) (the
    in-chunk triangular products, counted once)."""
    total = 0
    for L in lengths:
        full, tail = divmod(int(L), C)
        for c in [C] * full + ([tail] if tail else []):
            total += 6 * c * DK * DV + 2 * c * c * (DK + DV)
    return total * H


def prefill_bytes(tokens, H, n_seqs, s0, esz=2):
    """q, k, v, O rows (esz bytes per element) + g, beta (fp32) per head-token,
    plus one state read (if S0) and one state write per (sequence, head)."""
    per_tok = 4 * DK * esz + 8
    return tokens * H * per_tok + n_seqs * H * STATE_BYTES * (2 if s0 else 1)


def decode_bytes(units, esz=2):
    """State read + write, plus q, k, v, o rows and g, beta, per head-step."""
    return units * (2 * STATE_BYTES + 4 * DK * esz + 8)


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic}


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_recurrence_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag, digest):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k_, v_ = line.split("=", 1)
            vals[k_.strip()] = v_.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_decode(torch, gdn, inputs, steps, warmup, cold, streaming=False):
    w = inputs.batched_decode(device="cuda", steps=steps)
    B, H = w.meta["B"], w.meta["H"]
    units = B * H
    nbuf = 8 if cold else 1
    states = [w.S0.clone() for _ in range(nbuf)]
    outs = torch.empty_like(w.v)
    # warmup (eager) on a scratch state
    scratch = w.S0.clone()
    for i in range(warmup):
        s = i % steps
        gdn.gdn_decode_step(w.q[s], w.k[s], w.v[s], w.g[s], w.beta[s], scratch, o=outs[s],
                            streaming=streaming)
    torch.cuda.synchronize()
    # capture the K steps once
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        for s in range(steps):
            gdn.gdn_decode_step(w.q[s], w.k[s], w.v[s], w.g[s], w.beta[s],
                                states[s % nbuf], o=outs[s], streaming=streaming)
    torch.cuda.synchronize()
    # one untimed replay (first-replay setup cost); the timed replay follows it
    # directly, so each state batch starts where that replay left it, as in a
    # steady stream of steps (with one batch, the 64 MiB state then sits in the
    # 256 MB last-level cache)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    # eager launches of the same K steps, for reference
    for st in states:
        st.copy_(w.S0)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(steps):
        gdn.gdn_decode_step(w.q[s], w.k[s], w.v[s], w.g[s], w.beta[s], states[s % nbuf],
                            o=outs[s], streaming=streaming)
    torch.cuda.synchronize()
    eager = time.perf_counter() - t1
    return dict(units=units, wall_s=wall, gpu_ms=gpu_ms, eager_s=eager, workload=w)


def state_traffic_ceiling(torch, S0, steps, nbuf=1):
    """Microseconds per launch for torch's in-place elementwise pass over a
    tensor of the decode state's size (read once, written once) and for a
    device copy of it, each captured ``steps`` times in a graph like the decode
    steps, over ``nbuf`` such tensors in turn: what moving the same bytes
    costs without any arithmetic (nbuf = 8 puts 512 MiB in play, more than the
    last-level cache holds)."""
    xs = [S0.clone() for _ in range(nbuf)]
    ys = [torch.empty_like(S0) for _ in range(nbuf)]
    out = {}
    pre = "" if nbuf == 1 else "cold_"
    for tag, op in ((pre + "state_rmw_ceiling_us", lambda i: xs[i % nbuf].mul_(1.0)),
                    (pre + "state_copy_ceiling_us", lambda i: ys[i % nbuf].copy_(xs[i % nbuf]))):
        op(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
            for i in range(steps):
                op(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[tag] = e0.elapsed_time(e1) * 1e3 / steps
        del graph
    del xs, ys
    torch.cuda.empty_cache()
    return out


def time_calls(torch, call, iters, reps=3):
    """Seconds per call: ``iters`` calls back to back between one pair of events
    on the current stream (so that the host's launch work overlaps the GPU's),
    the median over ``reps`` such runs."""
    per_call = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            call()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) / 1e3 / iters)
    return statistics.median(per_call)


def bench_decode_preop(torch, gdn, inputs, steps):
    """Decode steps from the raw projections at the batched-decode shape (64 x 16),
    each form captured as one graph of ``steps`` steps: the fused
    gdn_decode_step_preop (one kernel a step; also with the gated norm on the
    output) against gdn_preop followed by gdn_decode_step (three).  The same token's projections feed every step (the
    time does not depend on the values).  Returns microseconds per step."""
    p = inputs.preop_inputs(64, 1, 16, seed=5, device="cuda")
    S = inputs.decode_workload(1, 64, 16, seed=6, device="cuda").S0.clone()
    state = p.state.clone()
    x3 = [t[:, 0].contiguous() for t in (p.xq, p.xk, p.xv)]
    a2, b2 = p.a[:, 0].contiguous(), p.b[:, 0].contiguous()
    o = torch.empty_like(x3[2])
    pre = [torch.empty_like(p.xq) for _ in range(3)] + [torch.empty_like(p.a) for _ in range(2)]

    gen = torch.Generator(device="cuda").manual_seed(7)
    gate = (torch.randn(64, 16, 128, generator=gen, device="cuda").to(p.xq.dtype),
            0.5 + torch.rand(128, generator=gen, device="cuda"), 1e-6)

    def fused():
        gdn.gdn_decode_step_preop(*x3, a2, b2, p.conv_w, state, S, o=o)

    def fused_gated():
        gdn.gdn_decode_step_preop(*x3, a2, b2, p.conv_w, state, S, gate=gate, o=o)

    def separate():
        gdn.gdn_preop(p.xq, p.xk, p.xv, p.a, p.b, p.conv_w, state, out=pre)
        gdn.gdn_decode_step(pre[0][:, 0], pre[1][:, 0], pre[2][:, 0], pre[3][:, 0],
                            pre[4][:, 0], S, o=o)

    out = {}
    for name, f in (("fused", fused), ("fused_gated", fused_gated), ("separate", separate)):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        graph, cap = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(steps):
                f()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / steps
        del graph
    return out


def bench_prefill(torch, gdn, w, iters, warmup, gate=None, segment_len=None, columns=None):
    """The prompt form over workload w; with gate = (z, norm_w, eps) the form
    with the gated RMS norm on the output (gdn_chunk_prefill_gated); with
    segment_len the segmented form (gdn_chunk_prefill_segmented; its
    workspace is allocated before the timed calls); with columns a
    GDN_COLUMNS_* choice (gdn_chunk_prefill_ex)."""
    O = torch.empty_like(w.v)
    N = w.q.shape[0] if w.cu_seqlens is None else w.cu_seqlens.numel() - 1
    S_T = torch.empty((N, w.q.shape[2], DK, DV), dtype=torch.float32, device="cuda")
    ws = None
    if segment_len is not None:
        need = gdn.segmented_workspace_bytes(w.q, segment_len, w.cu_seqlens)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def call():
        if segment_len is not None:
            gdn.gdn_chunk_prefill_segmented(w.q, w.k, w.v, w.g, w.beta, w.S0, w.chunk,
                                            segment_len, cu_seqlens=w.cu_seqlens,
                                            workspace=ws, O=O, S_T=S_T)
        elif gate is None:
            gdn.gdn_chunk_prefill(w.q, w.k, w.v, w.g, w.beta, w.S0, w.cu_seqlens, w.chunk,
                                  O=O, S_T=S_T, columns=columns)
        else:
            gdn.gdn_chunk_prefill_gated(w.q, w.k, w.v, w.g, w.beta, *gate, w.S0,
                                        w.cu_seqlens, w.chunk, Y=O, S_T=S_T)
    # Warm up for at least `warmup` calls and about 0.25 s of GPU time, so that
    # the clocks have settled before the timed calls.
    t_end = time.perf_counter() + 0.25
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        call()
        torch.cuda.synchronize()
        n += 1
    t = time_calls(torch, call, iters)
    H = w.q.shape[2]
    if w.cu_seqlens is None:
        lengths = [w.q.shape[1]] * w.q.shape[0]
    else:
        lengths = w.meta["lengths"]
    tokens = sum(lengths)
    esz = w.q.element_size()
    flops = prefill_flops(lengths, H, w.chunk)
    nbytes = prefill_bytes(tokens, H, len(lengths), w.S0 is not None, esz)
    if gate is not None:
        nbytes += tokens * H * DV * esz          # the gate rows z
    return {
        "workload": w.name + ("_gated_norm" if gate is not None else "")
                    + (f"_segmented_{segment_len}" if segment_len is not None else "")
                    + ({gdn.GDN_COLUMNS_WHOLE: "_whole_columns",
                        gdn.GDN_COLUMNS_SPLIT: "_split_columns"}.get(columns, "")),
        "arith": PREFILL_ARITH if esz == 2 else "fp32 arithmetic (vector kernel)",
        "tokens": tokens, "heads": H, "chunk": w.chunk,
        "seconds": t, "tokens_per_s": tokens / t,
        "mfma_frac": flops / t / BF16_PEAK, "hbm_frac": nbytes / t / HBM_PEAK,
        "alg_flops": flops, "alg_bytes": nbytes,
        "roofline": roofline("hbm", nbytes / t / 1e9, HBM_PEAK / 1e9, "GB/s"),
    }


def bench_states(torch, gdn, w, iters):
    """The rewindable verify form: gdn_prefill_states over a verify workload;
    the figure is the state bytes it writes (plus the state and token bytes it
    reads) per second."""
    O = torch.empty_like(w.v)
    B, T, H = w.q.shape[:3]
    S_tok = torch.empty((B, T, H, DK, DV), dtype=torch.float32, device="cuda")
    t_end = time.perf_counter() + 0.25
    n = 0
    while n < 2 or time.perf_counter() < t_end:
        gdn.gdn_prefill_states(w.q, w.k, w.v, w.g, w.beta, w.S0, w.cu_seqlens, O=O,
                               S_tok=S_tok)
        torch.cuda.synchronize()
        n += 1
    t = time_calls(torch, lambda: gdn.gdn_prefill_states(w.q, w.k, w.v, w.g, w.beta, w.S0,
                                                         w.cu_seqlens, O=O, S_tok=S_tok),
                   iters)
    rows = B * T
    nseq = len(w.meta["lengths"]) if w.cu_seqlens is not None else B
    esz = w.q.element_size()
    state_out = rows * H * STATE_BYTES
    nbytes = state_out + (nseq * H * STATE_BYTES if w.S0 is not None else 0) \
        + rows * H * (4 * DK * esz + 8)
    return {
        "workload": w.name + "_token_states", "tokens": rows, "heads": H, "seconds": t,
        "tokens_per_s": rows / t, "state_write_gbs": state_out / t / 1e9,
        "hbm_frac": nbytes / t / HBM_PEAK, "alg_bytes": nbytes,
        "roofline": roofline("hbm", nbytes / t / 1e9, HBM_PEAK / 1e9, "GB/s"),
    }


def bench_preop(torch, gdn, p, iters):
    """The block's pre-operations (gdn_preop) over one call's projections; the
    figure is the HBM bytes it must move per second."""
    B, T, H = p.xq.shape[:3]
    st = p.state.clone()
    out = (torch.empty_like(p.xq), torch.empty_like(p.xk), torch.empty_like(p.xv),
           torch.empty_like(p.a), torch.empty_like(p.b))

    def call():
        gdn.gdn_preop(p.xq, p.xk, p.xv, p.a, p.b, p.conv_w, st, p.cu_seqlens, out=out)

    t_end = time.perf_counter() + 0.25
    n = 0
    while n < 2 or time.perf_counter() < t_end:
        call()
        torch.cuda.synchronize()
        n += 1
    t = time_calls(torch, call, iters)
    rows = B * T
    esz = p.xq.element_size()
    # projections in and q/k/v out, gate inputs in and g/beta out, plus each
    # sequence's FIFO read and written (conv weights are negligible)
    nbytes = rows * H * (6 * DK * esz + 16) + 2 * p.state.numel() * esz
    return {
        "workload": f"preop_{B}x{T}x{H}", "tokens": rows, "heads": H, "seconds": t,
        "tokens_per_s": rows / t, "hbm_frac": nbytes / t / HBM_PEAK, "alg_bytes": nbytes,
        "roofline": roofline("hbm", nbytes / t / 1e9, HBM_PEAK / 1e9, "GB/s"),
    }


def bench_prefill_preop(torch, gdn, p, iters):
    """The prompt form from the raw projections, gdn_chunk_prefill_preop (the
    pre-operations inside the prompt kernel's chunk load), against the two
    calls gdn_preop then gdn_chunk_prefill on the same inputs."""
    B, T, H = p.xq.shape[:3]
    st = p.state.clone()
    S0 = torch.zeros(B, H, DK, DK, device="cuda")
    O = torch.empty_like(p.xq)
    S_T = torch.empty_like(S0)
    pre = (torch.empty_like(p.xq), torch.empty_like(p.xk), torch.empty_like(p.xv),
           torch.empty_like(p.a), torch.empty_like(p.b))

    def fused():
        gdn.gdn_chunk_prefill_preop(p.xq, p.xk, p.xv, p.a, p.b, p.conv_w, st, S0, O=O, S_T=S_T)

    def separate():
        q, k, v, g, b = gdn.gdn_preop(p.xq, p.xk, p.xv, p.a, p.b, p.conv_w, st, out=pre)
        gdn.gdn_chunk_prefill(q, k, v, g, b, S0, None, 64, O=O, S_T=S_T)

    for call in (fused, separate):
        for _ in range(2):
            call()
        torch.cuda.synchronize()
    t_sep = time_calls(torch, separate, iters)
    t = time_calls(torch, fused, iters)
    rows = B * T
    esz = p.xq.element_size()
    # projections and gate inputs in, O out, the states in and out, the FIFO
    nbytes = rows * H * (4 * DK * esz + 8) + 2 * B * H * DK * DK * 4 + 2 * p.state.numel() * esz
    return {
        "workload": f"prefill_preop_{B}x{T}x{H}", "tokens": rows, "heads": H, "seconds": t,
        "tokens_per_s": rows / t, "two_call_seconds": t_sep, "hbm_frac": nbytes / t / HBM_PEAK,
        "alg_bytes": nbytes, "arith": PREFILL_ARITH + "; pre-operations in fp32",
        "roofline": roofline("hbm", nbytes / t / 1e9, HBM_PEAK / 1e9, "GB/s"),
    }


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_decode(w, target_s=12.0):
    """The oracle, as it stands, on the first n steps of the decode workload,
    n sized from a timed probe so that the sample takes about target_s."""
    import oracle
    threads = oracle.default_threads()
    host = lambda x, n: x[:n].cpu()
    probe = min(20, w.q.shape[0])
    t0 = time.perf_counter()
    oracle.decode(host(w.q, probe), host(w.k, probe), host(w.v, probe), host(w.g, probe),
                  host(w.beta, probe), w.S0.cpu(), nthreads=threads)
    per_step = max(time.perf_counter() - t0, 1e-3) / probe
    n = int(max(1, min(w.q.shape[0], target_s / per_step)))
    t0 = time.perf_counter()
    oracle.decode(host(w.q, n), host(w.k, n), host(w.v, n), host(w.g, n), host(w.beta, n),
                  w.S0.cpu(), nthreads=threads)
    dt = time.perf_counter() - t0
    units = w.q.shape[1] * w.q.shape[2]
    return {"value": n * units * 2 * STATE_BYTES / dt / 1e9, "unit": "GB/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {n} steps of the B=64 x H=16 decode batch "
                      f"({dt:.1f} s, fp64, {threads} threads)"}


def cpu_baseline_prefill(w, target_s=12.0):
    """The oracle on whole (sequence, head) units of the large prefill: a probe
    of one unit sizes a sample of about target_s, run on all threads."""
    import oracle
    threads = oracle.default_threads()
    B, T, H = w.q.shape[0], w.q.shape[1], w.q.shape[2]
    sl = lambda x, b, hs: x[b:b + 1, :, hs].cpu()
    t0 = time.perf_counter()
    oracle.prefill(sl(w.q, 0, [0]), sl(w.k, 0, [0]), sl(w.v, 0, [0]), sl(w.g, 0, [0]),
                   sl(w.beta, 0, [0]), None, nthreads=1)
    per_unit = max(time.perf_counter() - t0, 1e-3)
    n_units = int(max(1, min(B * H, target_s * threads / per_unit)))
    n_units = max(threads, (n_units // threads) * threads) if n_units >= threads else n_units
    n_units = min(n_units, B * H)
    done, dt = 0, 0.0
    while done < n_units:
        b, h0 = divmod(done, H)
        hs = list(range(h0, min(H, h0 + n_units - done)))
        t0 = time.perf_counter()
        oracle.prefill(sl(w.q, b, hs), sl(w.k, b, hs), sl(w.v, b, hs), sl(w.g, b, hs),
                       sl(w.beta, b, hs), None, nthreads=threads)
        dt += time.perf_counter() - t0
        done += len(hs)
    return {"value": n_units * T / H / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n_units} (sequence, head) units x {T} tokens of the large prefill "
                      f"({dt:.1f} s of oracle time), scaled to tokens of {H} heads"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-iters", type=int, default=10)
    ap.add_argument("--cold", action="store_true",
                    help="rotate 8 state batches (512 MiB) so the state cannot stay in cache")
    ap.add_argument("--streaming", action="store_true",
                    help="time the decode with non-temporal state loads and stores "
                         "(gdn_decode_step_ex, GDN_STATE_STREAMING)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "decode-step", "prefill"], default=None,
                    help="decode: the decode legs; decode-step: only the headline decode "
                         "steps (the command the kernel trace in profiles/ is taken on); "
                         "prefill: the prompt-form legs")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB "
                         "(5 times), to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libgdn runs on one GPU and has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 4 * n, "dispatches": 5}), flush=True)
        return

    from linear_attention_recurrence_02_amd import binding as gdn
    from linear_attention_recurrence_02_amd import inputs
    gdn.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    result = {
        "metric": "prefill tokens/s (MFMA %) and decode state GB/s (HBM %) on 1 MI355X",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 io; decode step in fp32 arithmetic, fp32 state",
        "data": "synthetic (seeded device draws; q,k unit-norm, g=-softplus(N(0,1)), "
                "beta=sigmoid(N(0,1)), S0~0.1*N(0,1))",
        "config": {"workload": "batched decode step: B=64 sequences x H=16 heads, "
                               "dk=dv=128, bf16 q/k/v, fp32 state updated in place",
                   "global_batch": 64, "heads": 16, "seq_len": 1,
                   "parallelism": "single GPU"},
    }

    dec = None
    if args.only in (None, "decode", "decode-step"):
        log("decode: generating inputs and capturing the step graph ...")
        dec = bench_decode(torch, gdn, inputs, args.steps, args.warmup, args.cold,
                           args.streaming)
        K = args.steps
        units = dec["units"]
        # one timer for the value, ms_per_step and the roofline: the device
        # events around the timed replay of the K steps (the host clock around
        # the same replay is reported beside it)
        gpu_s = dec["gpu_ms"] / 1e3
        state_gbs = K * units * 2 * STATE_BYTES / gpu_s / 1e9
        avg_launch = gpu_s / K
        alg = decode_bytes(units)
        traffic = read_traffic(
            "decode_bf16_b64h16" + ("_streaming" if args.streaming else ""),
            source_digest("gdn_decode.hip"))
        result.update(value=state_gbs, ms_per_step=avg_launch * 1e3)
        result["roofline"] = roofline("hbm", alg / avg_launch / 1e9, HBM_PEAK / 1e9, "GB/s",
                                      traffic)
        result["decode"] = {
            "steps_per_s": K / gpu_s,
            "avg_launch_us": avg_launch * 1e6,
            "wall_us_per_step": dec["wall_s"] * 1e6 / K,
            "alg_bytes_per_launch": alg,
            "eager_launch_state_gbs": K * units * 2 * STATE_BYTES / dec["eager_s"] / 1e9,
            "cold_rotating_8_batches": bool(args.cold),
            "streaming_state": bool(args.streaming),
            "state_residency": ("8 state batches of 64 MiB in turn (512 MiB): read from HBM"
                                if args.cold else
                                "one 64 MiB batch updated in place: after the first step it "
                                "sits in the 256 MB last-level cache"),
        }
        log(f"decode: {state_gbs:.1f} GB/s state, {avg_launch*1e6:.2f} us/step "
            f"(host clock {dec['wall_s']*1e6/K:.2f} us/step, eager {dec['eager_s']*1e6/K:.2f} us/step)")
        if not args.cold and not args.streaming and args.only != "decode-step":
            # the same steps over eight state batches in turn (512 MiB, twice the
            # last-level cache), so that every step reads its state from HBM;
            # with plain and with non-temporal state access, and the latter on
            # the one batch too
            for tag, cold_, streaming_ in (("cold", True, False),
                                           ("cold_streaming", True, True),
                                           ("streaming", False, True)):
                r_ = bench_decode(torch, gdn, inputs, K, args.warmup, cold_, streaming_)
                launch = r_["gpu_ms"] / 1e3 / K
                result["decode"][f"{tag}_avg_launch_us"] = launch * 1e6
                result["decode"][f"{tag}_state_gbs"] = K * units * 2 * STATE_BYTES / (r_["gpu_ms"] / 1e3) / 1e9
                result["decode"][f"{tag}_hbm_frac"] = alg / launch / HBM_PEAK
                if tag == "cold_streaming":
                    # the state read from HBM on every step: the roofline of the
                    # decode step when the cache cannot hold the state
                    result["roofline_state_from_hbm"] = dict(
                        roofline("hbm", alg / launch / 1e9, HBM_PEAK / 1e9, "GB/s",
                                 read_traffic("decode_bf16_b64h16_streaming",
                                              source_digest("gdn_decode.hip"))),
                        call="gdn_decode_step_ex (GDN_STATE_STREAMING)",
                        workload="the same steps over 8 state batches of 64 MiB in turn")
                log(f"decode, {'8 rotating state batches' if cold_ else 'one batch'}"
                    f"{', non-temporal state' if streaming_ else ''}: {launch*1e6:.2f} us/step, "
                    f"HBM {100*alg/launch/HBM_PEAK:.1f}%")
                del r_
                torch.cuda.empty_cache()
            # the practical ceiling for these bytes: the same 64 MiB state read and
            # written once per launch by torch's own kernels (an in-place
            # elementwise pass, and a device copy into a second buffer), captured
            # and replayed like the decode steps
            ceil = state_traffic_ceiling(torch, dec["workload"].S0, K)
            ceil.update(state_traffic_ceiling(torch, dec["workload"].S0, K, nbuf=8))
            result["decode"].update(ceil)
            log(f"same state bytes by torch, one batch: in-place pass "
                f"{ceil['state_rmw_ceiling_us']:.2f} us, copy {ceil['state_copy_ceiling_us']:.2f} us; "
                f"8 batches in turn: {ceil['cold_state_rmw_ceiling_us']:.2f} us, "
                f"{ceil['cold_state_copy_ceiling_us']:.2f} us per launch")

    if args.only in (None, "decode") and not args.cold and not args.streaming:
        dp = bench_decode_preop(torch, gdn, inputs, min(args.steps, 200))
        result["decode"]["preop_fused_us"] = dp["fused"]
        result["decode"]["preop_gated_fused_us"] = dp["fused_gated"]
        result["decode"]["preop_then_decode_us"] = dp["separate"]
        log(f"decode from raw projections: fused {dp['fused']:.2f} us/step "
            f"({dp['fused_gated']:.2f} with the gated norm), "
            f"pre-operations then decode {dp['separate']:.2f} us/step")
        torch.cuda.empty_cache()

    if args.only in (None, "prefill"):
        pre = {}
        for make in (inputs.large_prefill, inputs.long_prefill, inputs.varlen_prefill,
                     inputs.verify_blocks):
            w = make(device="cuda")
            r = bench_prefill(torch, gdn, w, args.prefill_iters, 2)
            log(f"prefill {r['workload']}: {r['tokens_per_s']:.3e} tok/s, "
                f"{r['seconds']*1e3:.3f} ms, MFMA {100*r['mfma_frac']:.1f}%, "
                f"HBM {100*r['hbm_frac']:.1f}%")
            pre[r["workload"]] = r
            if w.name == "verify":
                r["roofline"]["traffic"] = read_traffic(
                    "prefill_short_verify",
                    source_digest("gdn_prefill_short.hip", "gdn_mfma.hpp"))
            if w.name == "long_prefill":
                # the default splits each (sequence, head) over two workgroups of
                # 64 value columns (16 units on 256 CUs); the unsplit form beside
                # it, then the segmented form
                rw = bench_prefill(torch, gdn, w, args.prefill_iters, 2,
                                   columns=gdn.GDN_COLUMNS_WHOLE)
                log(f"prefill {rw['workload']}: {rw['tokens_per_s']:.3e} tok/s, "
                    f"{rw['seconds']*1e3:.3f} ms")
                pre[rw["workload"]] = rw
                for seg_len in (256, 512):
                    rs = bench_prefill(torch, gdn, w, args.prefill_iters, 2, segment_len=seg_len)
                    log(f"prefill {rs['workload']}: {rs['tokens_per_s']:.3e} tok/s, "
                        f"{rs['seconds']*1e3:.3f} ms, MFMA {100*rs['mfma_frac']:.1f}%, "
                        f"HBM {100*rs['hbm_frac']:.1f}%")
                    pre[rs["workload"]] = rs
                # a packed serving batch: one 16384-token prompt among 31 of 256
                # tokens (not one of the specified workloads: it shows where the
                # packed segmented form pays)
                wp = inputs.varlen_workload([16384] + [256] * 31, H=16, seed=0,
                                            name="packed_long_among_short", device="cuda")
                for seg_len in (None, 2048):
                    rp = bench_prefill(torch, gdn, wp, args.prefill_iters, 2, segment_len=seg_len)
                    log(f"prefill {rp['workload']}: {rp['tokens_per_s']:.3e} tok/s, "
                        f"{rp['seconds']*1e3:.3f} ms")
                    pre[rp["workload"]] = rp
                del wp
            if w.name == "large_prefill":
                r["roofline"]["traffic"] = read_traffic(
                    "prefill_large", source_digest("gdn_prefill_mfma.hip", "gdn_mfma.hpp"))
                if not args.no_cpu_baseline:
                    r["cpu_baseline"] = cpu_baseline_prefill(w)
                    r["cpu_baseline"]["gpu_over_cpu"] = r["tokens_per_s"] / r["cpu_baseline"]["value"]
                # the same workload with the gated RMS norm fused on the output
                rg = bench_prefill(torch, gdn, w, args.prefill_iters, 2,
                                   gate=inputs.norm_gate(w))
                rg["roofline"]["traffic"] = read_traffic(
                    "prefill_large_gated", source_digest("gdn_prefill_mfma.hip", "gdn_mfma.hpp"))
                log(f"prefill {rg['workload']}: {rg['tokens_per_s']:.3e} tok/s, "
                    f"{rg['seconds']*1e3:.3f} ms, HBM {100*rg['hbm_frac']:.1f}%")
                pre[rg["workload"]] = rg
            del w
            torch.cuda.empty_cache()
        p = inputs.preop_inputs(8, 16384, 32, device="cuda")
        r = bench_preop(torch, gdn, p, args.prefill_iters)
        r["roofline"]["traffic"] = read_traffic("preop_large", source_digest("gdn_preop.hip"))
        log(f"pre-operations {r['workload']}: {r['seconds']*1e3:.3f} ms, "
            f"{r['roofline']['achieved']:.0f} GB/s, HBM {100*r['hbm_frac']:.1f}%")
        pre[r["workload"]] = r
        r = bench_prefill_preop(torch, gdn, p, args.prefill_iters)
        r["roofline"]["traffic"] = read_traffic(
            "prefill_preop_large", source_digest("gdn_prefill_mfma.hip", "gdn_mfma.hpp"))
        log(f"prompt form from the projections {r['workload']}: {r['seconds']*1e3:.3f} ms fused, "
            f"{r['two_call_seconds']*1e3:.3f} ms as two calls")
        pre[r["workload"]] = r
        del p
        torch.cuda.empty_cache()
        w = inputs.verify_blocks(device="cuda")
        r = bench_states(torch, gdn, w, args.prefill_iters)
        r["roofline"]["traffic"] = read_traffic("token_states_verify",
                                                source_digest("gdn_states.hip"))
        log(f"token states {r['workload']}: {r['state_write_gbs']:.1f} GB/s of states, "
            f"{r['seconds']*1e3:.3f} ms, HBM {100*r['hbm_frac']:.1f}%")
        pre[r["workload"]] = r
        del w
        torch.cuda.empty_cache()
        result["prefill"] = pre

    if dec is not None and not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample of the decode workload ...")
        result["cpu_baseline"] = cpu_baseline_decode(dec["workload"])
        result["cpu_baseline"]["gpu_over_cpu"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
