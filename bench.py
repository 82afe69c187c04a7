"""Benchmark: streaming chunk attention on one MI355X.

One step = one steady-state chunk of a stream through the whole hot path:
  sa_chunk_attend  -> rope_apply (RoPE of Q and K fused into their writes,
                      V transposed into the cache) + chunk_attention
                      (+ attn_combine when the key range is split)
  sa_kv_append     -> kv_ring_append (RoPE of K fused, V transposed), evicting
                      the oldest window chunk
over seeded synthetic bf16 inputs already resident in HBM (a pool of 8
distinct chunks cycled). The stream is filled to steady state (sink + full
window) before the warm-up, so every timed chunk attends to
(S + W + 1) * Nc keys. RoPE refresh and sink replacement do not occur in the
default workload's schedule; they are timed separately and reported as extra
fields.

Output: one JSON line. value = attended query tokens/s (B * Nc per step);
ms_per_step = ms per chunk. roofline = the chunk_attention kernel alone,
algorithmic FLOPs 4*B*H*D*Nc*Nk over visible keys / its mean duration from
HIP events recorded on the launch stream, against the MI355X dense bf16 peak.
cpu_baseline = the fp64 NumPy oracle on a bounded sample of one steady chunk.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan1.3b]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attended query tokens/sec + ms/chunk; % bf16 MFMA peak (1 MI355X)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3  # MI355X fp32, vector and dense MFMA alike
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan1.3b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--deadline-ms", type=float, default=1.0,
                    help="per-call deadline for the ragged-batch size choice (an example SLO)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget for the oracle baseline sample")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--variant", type=int, default=0,
                    help="bf16 attention kernel variant (0 automatic, 1 = 32 rows/wave, 2 = 64 rows/wave)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline workload only (a profiler's per-kernel averages then cover it alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 4 times (scales the HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 4 x (read 1 GiB + write 1 GiB)."""
    import torch
    torch.cuda.set_device(0)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n}), flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("attention_kernels.hip", "sa_internal.h"):
        h.update(open(os.path.join(ROOT, "causal_windowed_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, src_hash):
    """HBM bytes per chunk_attention launch from a committed rocprofv3 --pmc summary, or None.

    The summary records the kernel source hash it was taken with; a different
    hash means the kernel changed since, and the figure is not reported.
    """
    path = os.path.join(PROFILES, f"chunk_attention_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle on a bounded sample of one steady-state chunk."""
    import numpy as np
    import synth
    from oracle import HistoryOracle, StreamSpec
    from dataclasses import replace
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = []
    threads = max([t for _, t in blas if t] or [1])
    steady = w.sink_chunks + w.window_chunks
    heads_done, elapsed = 0, 0.0
    for h in range(w.heads):
        spec = replace(StreamSpec.from_workload(w), heads=1)
        orc = HistoryOracle(spec)
        for c in range(steady):
            _, k, v = synth.chunk_qkv(w, c)
            orc.append(k[:, :, h:h + 1], v[:, :, h:h + 1])
        q, k, v = synth.chunk_qkv(w, steady)
        t0 = time.perf_counter()
        orc.attend(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1])
        elapsed += time.perf_counter() - t0
        heads_done += 1
        if elapsed >= budget_s:
            break
    per_chunk_s = elapsed * w.heads / heads_done
    return {
        "value": w.batch * w.tokens_per_chunk / per_chunk_s,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{heads_done} of {w.heads} heads of one steady-state chunk "
                   f"({w.tokens_per_chunk} query rows x {(steady + 1) * w.tokens_per_chunk} keys, fp64 "
                   f"NumPy incl. RoPE), {elapsed:.1f} s, scaled to all heads"),
        "seconds_per_chunk": per_chunk_s,
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": blas,
    }


def write_reference(torch, traffic, reps=30):
    """A plain device copy moving the same bytes as each write kernel (traffic = read + write
    bytes; the copy reads and writes half each), timed two ways: with one HIP event pair around
    each launch, as the library's kernel profile times its kernels, and back to back (one event
    pair around reps launches)."""
    def per_launch(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for _ in range(3):
            fn()
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps
    copies = {}
    for name, nbytes in traffic.items():
        src = torch.ones(nbytes // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        ms = per_launch(lambda: dst.copy_(src))
        ms_b2b = back_to_back(torch, lambda: dst.copy_(src), reps)
        copies[name] = {"traffic_bytes": nbytes, "copy_ms": ms, "copy_ms_back_to_back": ms_b2b}
        del src, dst
    return copies


def back_to_back(torch, fn, reps):
    """Mean time of reps launches of fn issued back to back between one event pair."""
    for _ in range(3):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def probe_mfma(torch, cwa, blocks=512, iters=20000, reps=3):
    """The MFMA rate the part sustains on a pure v_mfma_f32_32x32x16_bf16 stream, on this machine
    and in this run, for two kinds of operands: fixed per lane (benign, low toggle) and normally
    distributed bf16 data that changes between consecutive MFMAs (the realistic case); timed
    with events around the library's measurement kernels (best of reps)."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(11)
    ops = torch.randn(6 * 64 * 8, generator=g).to(torch.bfloat16).cuda()
    flops = blocks * 4 * iters * 8 * 32768.0
    res = {"blocks": blocks, "iters": iters}
    for kind, launch in (("fixed_operands", lambda: cwa.sa_probe_mfma_bf16(out, blocks, iters)),
                         ("normal_operands", lambda: cwa.sa_probe_mfma_bf16_data(out, ops, blocks, iters))):
        launch()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        tf = flops / (best * 1e-3) / 1e12
        res[kind] = {"tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS}
    return res


def box_identity(torch):
    """Which box a run measured: host name, device name and the device's UUID."""
    import socket
    p = torch.cuda.get_device_properties(0)
    return {"host": socket.gethostname(), "device": p.name, "uuid": str(getattr(p, "uuid", "")),
            "gcn_arch": getattr(p, "gcnArchName", "")}


def bench_buffer(torch, cwa, synth, name="long512p", n=4, steps=20, steps_mode=False):
    """Buffer attend (n chunks as queries in one call; the moving buffer, or with steps_mode
    Stream-Batch over denoising steps) at steady state: call time, kernel time, and
    algorithmic FLOPs over each chunk's visible keys (from sa_buffer_plan)."""
    import numpy as np
    w = synth.WORKLOADS[name]
    cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                          w.sink_chunks, w.window_chunks, dtype="bf16", max_buffer_chunks=n)
    s = cwa.Stream(cfg, device="cuda")
    nc = w.tokens_per_chunk
    for c in range(w.sink_chunks + w.window_chunks + 1):
        _, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in synth.chunk_qkv(w, c))
        s.kv_append(k, v)
    parts = [synth.chunk_qkv(w, 200 + j) for j in range(n)]
    q, k, v = (torch.from_numpy(np.concatenate([p_[i] for p_ in parts], axis=1)).to(torch.bfloat16).cuda()
               for i in range(3))
    out = torch.empty_like(q)
    keys = [sum(hi - lo for lo, hi in segs) for segs in s.buffer_plan(n, steps=steps_mode)]
    flops = sum(4.0 * w.batch * w.heads * w.head_dim * nc * kj for kj in keys)
    for _ in range(3):
        s.buffer_attend(q, k, v, out=out, steps=steps_mode)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        s.buffer_attend(q, k, v, out=out, steps=steps_mode)
    b.record()
    torch.cuda.synchronize()
    call_ms = a.elapsed_time(b) / steps
    s.set_option(cwa.SA_OPT_PROFILE, 1)
    for k_id in range(cwa.SA_K_COUNT):
        s.profile_read(k_id, reset=True)
    for _ in range(steps):
        s.buffer_attend(q, k, v, out=out, steps=steps_mode)
    attn_ms, na = s.profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
    rope_ms, nr = s.profile_read(cwa.SA_K_ROPE_APPLY, reset=True)
    s.close()
    attn_ms /= max(na, 1)
    tf = flops / (attn_ms * 1e-3) / 1e12
    return {"workload": name, "mode": "steps" if steps_mode else "moving buffer",
            "buffer_chunks": n, "tokens_per_call": w.batch * n * nc,
            "tokens_per_s": w.batch * n * nc / (call_ms * 1e-3), "ms_per_call": call_ms,
            "attention_ms": attn_ms, "rope_apply_ms_per_call": rope_ms / max(nr, 1),
            "visible_keys_per_chunk": keys, "flops_per_call": flops, "tflops": tf,
            "frac_of_peak": tf / PEAK_BF16_TFLOPS, "kernel": "chunk_attention_bf16_d128_ppg"}


def bench_fp8(torch, cwa, synth, name="wan1.3b", steps=30):
    """The same steady-state step (attend + commit) on a stream with an fp8 (E4M3) cache:
    bf16 inputs and outputs, fp8 MFMAs. Step time, the attention kernel's time and its
    algorithmic FLOP rate against the fp8 peak; the bf16 step is the headline line."""
    w = synth.WORKLOADS[name]
    cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                          w.sink_chunks, w.window_chunks, dtype="fp8")
    s = cwa.Stream(cfg, device="cuda")
    nc = w.tokens_per_chunk
    pool = [tuple(torch.from_numpy(x).to(torch.bfloat16).cuda() for x in synth.chunk_qkv(w, c)) for c in range(8)]
    out = torch.empty_like(pool[0][0])
    for c in range(w.sink_chunks + w.window_chunks + 1):
        q, k, v = pool[c % 8]
        s.chunk_attend(q, k, v, out=out)
        s.kv_append()
    def step(i):
        q, k, v = pool[i % 8]
        s.chunk_attend(q, k, v, out=out)
        s.kv_append()
    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / steps
    s.set_option(cwa.SA_OPT_PROFILE, 1)
    s.profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
    for i in range(steps):
        step(i)
    attn_ms, na = s.profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
    keys = s.query()["visible_keys"]
    s.close()
    attn_ms /= max(na, 1)
    flops = 4.0 * w.batch * w.heads * w.head_dim * nc * keys
    tf = flops / (attn_ms * 1e-3) / 1e12
    return {"workload": name, "dtype": "fp8 e4m3 cache (bf16 in/out)", "ms_per_step": step_ms,
            "tokens_per_s": w.batch * nc / (step_ms * 1e-3), "attention_ms": attn_ms, "visible_keys": keys,
            "tflops": tf, "frac_of_fp8_peak": tf / PEAK_FP8_TFLOPS, "kernel": "chunk_attention_fp8_d128_pp"}


def gdn_flops(N, H, D, B=1, C=64):
    """Algorithmic FLOPs of the chunkwise gated delta rule per call: per 64-token block and
    head, K K^T (C^2 D), the triangular solve (C^3 / 6), T V and T diag(gam) K (2 C^2 D),
    U = Up - W S^T and the state update (2 C D^2), Q S^T (C D^2), Q K^T and P U (2 C^2 D);
    two FLOPs per multiply-add."""
    nb = -(-N // C)
    mac = 5 * C * C * D + C ** 3 / 6 + 3 * C * D * D
    return 2.0 * B * H * nb * mac


def bench_gdn(torch, cwa, synth, name="hybrid1280x704", steps=20):
    """GDN block (gated delta rule) forward over one video chunk of a workload shape with a
    carried state: call time and FLOP rate (chunkwise count) against the fp32 peak (its state
    products run on the fp32 MFMA; the sequential scan, not arithmetic, bounds the call)."""
    w = synth.WORKLOADS[name]
    B, N, H, D = w.batch, w.tokens_per_chunk, w.heads, w.head_dim
    q, k, v, a, b, s0 = synth.gdn_inputs(B, N, H, D, seed=1)
    d16 = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    d32 = lambda x: torch.from_numpy(x).cuda()
    q, k, v, a, b, state = d16(q), d16(k), d16(v), d32(a), d32(b), d32(s0)
    out = torch.empty_like(v)
    ws = torch.empty(cwa.sa_gdn_workspace_bytes(B, N, H, D), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        cwa.gdn_forward(q, k, v, a, b, state=state, out=out, state_out=state, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        cwa.gdn_forward(q, k, v, a, b, state=state, out=out, state_out=state, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = gdn_flops(N, H, D, B)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": name, "tokens_per_call": B * N, "heads": H, "head_dim": D, "ms_per_call": ms,
            "tokens_per_s": B * N / (ms * 1e-3), "flops_per_call": fl, "tflops": tf,
            "frac_of_fp32_peak": tf / PEAK_FP32_TFLOPS,
            "kernels": ["gdn_prep", "gdn_scan", "gdn_out"]}


BF16_CONFIGS = ("wan1.3b", "wan14b_b1", "wan14b_b2", "wan14b_b4", "hybrid1280x704", "long512p")


def bench_configs(torch, cwa, synth, steps=20):
    """Every bf16 workload shape at steady state (a full sink and window): the step (attend +
    commit) and the attend alone per chunk as p50 / p99 of per-step events, the attention kernel's time and its
    algorithmic FLOP rate (visible keys only), and misses against the per-chunk budgets of
    24 and 16 frames/s. A pool of two distinct chunks cycles through the stream."""
    res = {}
    for name in BF16_CONFIGS:
        w = synth.WORKLOADS[name]
        cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                              w.sink_chunks, w.window_chunks, dtype="bf16")
        s = cwa.Stream(cfg, device="cuda")
        pool = [tuple(torch.from_numpy(x).to(torch.bfloat16).cuda() for x in synth.chunk_qkv(w, 300 + i))
                for i in range(2)]
        out = torch.empty_like(pool[0][0])

        def step(i, mid=None):
            q, k, v = pool[i % 2]
            s.chunk_attend(q, k, v, out=out)
            if mid is not None:
                mid.record()
            s.kv_append(k, v)
        for i in range(w.sink_chunks + w.window_chunks + 3):
            step(i)
        torch.cuda.synchronize()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            step(i, evs[i][1])
            evs[i][2].record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(c) for a, _, c in evs)
        ta = sorted(a.elapsed_time(b) for a, b, _ in evs)
        s.set_option(cwa.SA_OPT_PROFILE, 1)
        s.profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
        for i in range(steps):
            step(i)
        attn_ms, na = s.profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
        keys = s.query()["visible_keys"]
        s.close()
        attn_ms /= max(na, 1)
        nc = w.tokens_per_chunk
        flops = 4.0 * w.batch * w.heads * w.head_dim * nc * keys
        tf = flops / (attn_ms * 1e-3) / 1e12
        budgets = {fps: w.frames_per_chunk * 1000.0 / fps for fps in (24, 16)}
        res[name] = {"batch": w.batch, "heads": w.heads, "tokens_per_chunk": nc, "visible_keys": keys,
                     "step_ms_p50": t[len(t) // 2], "step_ms_p99": t[min(len(t) - 1, int(round(0.99 * (len(t) - 1))))],
                     "attend_ms_p50": ta[len(ta) // 2],
                     "attend_ms_p99": ta[min(len(ta) - 1, int(round(0.99 * (len(ta) - 1))))],
                     "attention_ms": attn_ms, "tokens_per_s": w.batch * nc / (t[len(t) // 2] * 1e-3),
                     "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS,
                     "deadline_misses": {fps: sum(x > b for x in t) for fps, b in budgets.items()}}
    return res


def _tiny_schedule(w, attend, append, refresh):
    """The tiny workload's whole stream: attend and commit every chunk, with the refresh its
    schedule puts before some chunks."""
    for c in range(w.n_chunks):
        if w.refresh_before(c):
            refresh()
        attend(c)
        append(c)


def bench_tiny(torch, cwa, synth, reps=20):
    """The tiny fp32 workload (B 1, H 2, D 64, 8 x 8 frames, F 2 -> Nc 128; S 1, W 2): its whole
    stream of 6 chunks, refresh included, on a fresh stream each repetition (created and zeroed
    outside the timed region). Launch-latency bound: a correctness shape, with no fraction of peak."""
    w = synth.WORKLOADS["tiny_f32"]
    cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                          w.sink_chunks, w.window_chunks, dtype="f32")
    data = [tuple(torch.from_numpy(x).cuda() for x in synth.chunk_qkv(w, c)) for c in range(w.n_chunks)]
    out = torch.empty_like(data[0][0])
    times = []
    for _ in range(reps + 2):
        s = cwa.Stream(cfg, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _tiny_schedule(w, lambda c: s.chunk_attend(*data[c], out=out), lambda c: s.kv_append(*data[c][1:]),
                       lambda: s.rope_refresh(-1, 0))
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
        s.close()
    t = sorted(times[2:])
    return {"workload": w.name, "chunks": w.n_chunks, "tokens_per_chunk": w.tokens_per_chunk,
            "ms_per_stream_p50": t[len(t) // 2], "ms_per_stream_min": t[0],
            "ms_per_chunk": t[len(t) // 2] / w.n_chunks,
            "tokens_per_s": w.batch * w.tokens_per_chunk * w.n_chunks / (t[len(t) // 2] * 1e-3),
            "what": "host wall time of the whole stream (attend + commit per chunk, one refresh), launch-latency bound"}


def tiny_oracle(synth, reps=3):
    """The fp64 oracle over the tiny workload's whole stream (the same schedule), best of reps."""
    from oracle import HistoryOracle, StreamSpec
    w = synth.WORKLOADS["tiny_f32"]
    data = [synth.chunk_qkv(w, c) for c in range(w.n_chunks)]
    best = None
    for _ in range(reps):
        orc = HistoryOracle(StreamSpec.from_workload(w))
        t0 = time.perf_counter()
        _tiny_schedule(w, lambda c: orc.attend(*data[c]), lambda c: orc.append(*data[c][1:]),
                       lambda: orc.refresh(None, 0))
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return best


def bench_batch(torch, cwa, synth, name="long512p", sizes=(1, 2, 3, 4, 6, 8), steps=20, deadline_ms=1.0,
                model_calls=60, calls=1000, margin=0.10):
    """Ragged batch: n steady-state streams (each its own cache and position) attended in one
    launch; per n the call time, attended tokens/s and the attention kernel's TFLOP/s.

    Then a deadline-driven choice of n (Stream-Batch: adapt the batch to the load without
    breaking the latency bound). The latency model is measured on the running box at start-up:
    per n, model_calls calls each timed by its own events, and the model is their p99 (a tail
    quantile, not a mean fit). The chosen n is the largest whose p99 times (1 + margin) meets the
    deadline; margin covers drift between the model's measurement and the run (boxes differ by
    up to 10 %). The chosen batch then runs `calls` calls, each timed by its own events; the
    miss rate (calls over the deadline), p50 / p99 / max and the mean jitter (mean |difference|
    of consecutive call times) are reported beside the prediction."""
    import numpy as np
    w = synth.WORKLOADS[name]
    cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                          w.sink_chunks, w.window_chunks, dtype="bf16")
    nc = w.tokens_per_chunk
    streams, qs, ks, vs, outs = [], [], [], [], []
    for i in range(max(sizes)):
        s = cwa.Stream(cfg, device="cuda")
        for c in range(w.sink_chunks + w.window_chunks + i):   # full windows, different positions
            _, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in synth.chunk_qkv(w, 50 * i + c))
            s.kv_append(k, v)
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in synth.chunk_qkv(w, 900 + i))
        streams.append(s); qs.append(q); ks.append(k); vs.append(v); outs.append(torch.empty_like(q))

    def timed_calls(n, count):
        args = (streams[:n], qs[:n], ks[:n], vs[:n], outs[:n])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]
        for a, b in ev:
            a.record()
            cwa.sa_batch_attend(*args)
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    res = {}
    model = {}
    for n in sizes:
        args = (streams[:n], qs[:n], ks[:n], vs[:n], outs[:n])
        for _ in range(3):
            cwa.sa_batch_attend(*args)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            cwa.sa_batch_attend(*args)
        b.record()
        torch.cuda.synchronize()
        call_ms = a.elapsed_time(b) / steps
        streams[0].set_option(cwa.SA_OPT_PROFILE, 1)
        streams[0].profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
        streams[0].profile_read(cwa.SA_K_ROPE_APPLY, reset=True)
        for _ in range(steps):
            cwa.sa_batch_attend(*args)
        attn_ms, na = streams[0].profile_read(cwa.SA_K_CHUNK_ATTENTION, reset=True)
        rope_ms, nr = streams[0].profile_read(cwa.SA_K_ROPE_APPLY, reset=True)
        streams[0].set_option(cwa.SA_OPT_PROFILE, 0)
        attn_ms /= max(na, 1)
        t = timed_calls(n, model_calls)
        model[n] = {"p50_ms": float(np.percentile(t, 50)), "p99_ms": float(np.percentile(t, 99)),
                    "max_ms": float(t.max())}
        flops = sum(4.0 * w.batch * w.heads * w.head_dim * nc * st.query()["visible_keys"] for st in streams[:n])
        tf = flops / (attn_ms * 1e-3) / 1e12
        res[n] = {"ms_per_call": call_ms, "tokens_per_s": n * w.batch * nc / (call_ms * 1e-3),
                  "attention_ms": attn_ms, "rope_launches_per_call": nr / max(steps, 1),
                  "rope_ms": rope_ms / max(nr, 1), "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS,
                  "call_p50_ms": model[n]["p50_ms"], "call_p99_ms": model[n]["p99_ms"]}
    fits = [n for n in sizes if model[n]["p99_ms"] * (1.0 + margin) <= deadline_ms]
    # the largest batch that meets the deadline: the most work per call within the latency bound
    n = max(fits) if fits else min(sizes)
    t = timed_calls(n, calls)
    sched = {"deadline_ms_per_call": deadline_ms, "model": "p99 of %d calls per size, measured at start-up" % model_calls,
             "margin": margin, "model_p99_ms": {k: v["p99_ms"] for k, v in model.items()},
             "chosen_streams": n, "rule": "largest n with model p99 x (1 + margin) <= deadline",
             "deadline_met_by_model": bool(fits),
             "predicted_p99_ms": model[n]["p99_ms"], "calls": calls,
             "p50_ms": float(np.percentile(t, 50)), "p99_ms": float(np.percentile(t, 99)), "max_ms": float(t.max()),
             "miss_rate": float(np.mean(t > deadline_ms)), "mean_jitter_ms": float(np.mean(np.abs(np.diff(t)))),
             "tokens_per_s": n * w.batch * nc / (float(np.mean(t)) * 1e-3)}
    for s in streams:
        s.close()
    return {"workload": name, "streams": res, "deadline_schedule": sched,
            "kernel": "chunk_attention_bf16_d128_ppg"}


def note(msg):
    """Progress of a long run, on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(a stream's caches live on one GPU; streams and heads would shard across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import causal_windowed_attention_amd as cwa
    import synth

    w = synth.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("the benchmark workloads are bf16")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w, w.frames_per_chunk,
                          w.sink_chunks, w.window_chunks, dtype="bf16")
    s = cwa.Stream(cfg, device=dev)
    s.set_option(cwa.SA_OPT_ATTN_VARIANT, args.variant)
    nc = w.tokens_per_chunk
    steady = w.sink_chunks + w.window_chunks
    pool = []
    for i in range(8):
        q, k, v = synth.chunk_qkv(w, 100 + i)
        pool.append(tuple(torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v)))
    out = torch.empty_like(pool[0][0])

    def step(i, mid=None):
        q, k, v = pool[i % len(pool)]
        s.chunk_attend(q, k, v, out=out)
        if mid is not None:
            mid.record()                         # attend done, append next
        s.kv_append(k, v)

    # ---- full stream from empty (warm-up chunks included), once -----------------
    note(f"{w.name}: stream from empty, then {args.warmup} + {args.steps} timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(w.n_chunks):
        step(i)
    torch.cuda.synchronize()
    stream_ms = (time.perf_counter() - t0) * 1e3
    # after n_chunks >= S + W commits the stream is in steady state
    assert s.query()["visible_keys"] == (steady + 1) * nc

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    value = w.batch * nc * args.steps / dt

    # ---- the same step committing the staged K/V (sa_kv_append(NULL, NULL): the attend
    # already wrote the rotated K and V^T into the slot the commit makes visible) ---------
    def step_zero_copy(i):
        q, k, v = pool[i % len(pool)]
        s.chunk_attend(q, k, v, out=out)
        s.kv_append(None, None)
    for i in range(args.warmup):
        step_zero_copy(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_zero_copy(i)
    torch.cuda.synchronize()
    dt_zc = time.perf_counter() - t0

    # ---- per-step GPU time distribution (events on the stream the library uses) ---
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        step(i, evs[i][1])
        evs[i][2].record()
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(c) for a, _, c in evs)
    attend_only_ms = sorted(a.elapsed_time(b) for a, b, _ in evs)
    pct = lambda q, v=step_ms: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]

    # ---- per-kernel durations: HIP events on the launch stream ------------------
    note("per-kernel durations")
    s.set_option(cwa.SA_OPT_PROFILE, 1)
    for k_id in range(cwa.SA_K_COUNT):
        s.profile_read(k_id, reset=True)
    for i in range(args.profile_steps):
        step(i)
    kern = {}
    for name, k_id in (("rope_apply", cwa.SA_K_ROPE_APPLY), ("chunk_attention", cwa.SA_K_CHUNK_ATTENTION),
                       ("attn_combine", cwa.SA_K_ATTN_COMBINE), ("kv_ring_append", cwa.SA_K_KV_APPEND)):
        ms, n = s.profile_read(k_id, reset=True)
        if n:
            kern[name] = ms / n
    st = s.query()
    # refresh and sink update (not in this workload's schedule): timed separately
    base = w.sink_chunks * w.frames_per_chunk
    for i in range(4):
        s.rope_refresh(base + (i % 2) * w.frames_per_chunk, 0)   # alternate bases: Delta != 0 each time
        s.sink_update(*[torch.cat([pool[0][j]] * w.sink_chunks, dim=1) for j in (1, 2)])
    for name, k_id in (("rope_refresh", cwa.SA_K_ROPE_REFRESH), ("sink_update", cwa.SA_K_SINK_UPDATE)):
        ms, n = s.profile_read(k_id, reset=True)
        if n:
            kern[name] = ms / n
    s.set_option(cwa.SA_OPT_PROFILE, 0)
    # back to back: commits of a chunk (each writes the next ring slot) and refreshes
    b2b_ms = {"kv_ring_append": back_to_back(torch, lambda: s.kv_append(pool[0][1], pool[0][2]), 20)}
    flip = [0]

    def refresh():
        flip[0] ^= 1
        s.rope_refresh(base + flip[0] * w.frames_per_chunk, 0)
    b2b_ms["rope_refresh"] = back_to_back(torch, refresh, 20)

    buffer_res = fp8_res = gdn_res = configs_res = steps_res = batch_res = tiny_res = None
    note("mfma probe")
    mfma_probe = probe_mfma(torch, cwa)
    if not args.headline_only:
        note("moving buffer")
        buffer_res = bench_buffer(torch, cwa, synth)
        note("fp8 cache")
        fp8_res = bench_fp8(torch, cwa, synth)
        note("gdn block")
        gdn_res = bench_gdn(torch, cwa, synth)
        note("bf16 shapes")
        configs_res = bench_configs(torch, cwa, synth)
        note("steps mode")
        steps_res = bench_buffer(torch, cwa, synth, steps_mode=True)
        note("ragged batches")
        batch_res = bench_batch(torch, cwa, synth, deadline_ms=args.deadline_ms)
        note("tiny fp32 stream")
        tiny_res = bench_tiny(torch, cwa, synth)

    nk = st["visible_keys"]
    flops = 4.0 * w.batch * w.heads * w.head_dim * nc * nk
    attn_ms = kern["chunk_attention"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    elem = w.batch * nc * w.heads * w.head_dim * 2
    d_t = w.head_dim - 4 * (w.head_dim // 6)
    gbs = lambda bytes_, ms: bytes_ / (ms * 1e-3) / 1e9
    write_bytes = {"rope_apply": 6 * elem, "kv_ring_append": 4 * elem,
                   # temporal pairs of the window's rows, read and written
                   "rope_refresh": 2 * w.batch * w.heads * w.window_chunks * nc * d_t * 2}
    copy_ref = write_reference(torch, write_bytes)
    write_kernels = {}
    for name, nbytes in write_bytes.items():
        if name not in kern:
            continue
        ms, c = kern[name], copy_ref[name]
        write_kernels[name] = {"ms": ms, "gbs": gbs(nbytes, ms), "copy_gbs": gbs(nbytes, c["copy_ms"]),
                               "frac_of_copy": c["copy_ms"] / ms}
        b2b = b2b_ms.get(name)
        if b2b is not None:
            write_kernels[name].update({"ms_back_to_back": b2b, "gbs_back_to_back": gbs(nbytes, b2b),
                                        "copy_gbs_back_to_back": gbs(nbytes, c["copy_ms_back_to_back"]),
                                        "frac_of_copy_back_to_back": c["copy_ms_back_to_back"] / b2b})
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(w.name, src_hash)
    attend_ms = attn_ms + kern.get("rope_apply", 0.0) + kern.get("attn_combine", 0.0)

    res = {
        "metric": METRIC,
        "value": value,
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
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
            "frame": [w.frame_h, w.frame_w], "frames_per_chunk": w.frames_per_chunk,
            "tokens_per_chunk": nc, "sink_chunks": w.sink_chunks, "window_chunks": w.window_chunks,
            "visible_keys": nk, "step": "one steady-state chunk: attend (rope_apply + chunk_attention"
            + (" + attn_combine" if st["last_kv_splits"] > 1 else "") + ") + append (kv_ring_append)",
            "kv_splits": st["last_kv_splits"], "q_tiles": st["last_q_tiles"],
            "attn_variant": args.variant,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel": {1: "chunk_attention_bf16_d128", 2: "chunk_attention_bf16_d128_q64",
                       3: "chunk_attention_bf16_d128_pp"}[args.variant or 3],
            "flops_per_launch": flops,
            "mean_ms": attn_ms,
            "kernel_source_hash": src_hash,
            # the same rate against this box's measured pure-MFMA ceiling on normally distributed
            # operands (mfma_probe.normal_operands, same run)
            "frac_of_measured_ceiling": achieved / mfma_probe["normal_operands"]["tflops"],
        },
        "kernels_ms": kern,
        "kernels_gbs": {name: v["gbs"] for name, v in write_kernels.items()},
        # per-launch event timing (the library's profile) and, for the kernels a call can issue
        # alone, back-to-back launches; a device copy of the same bytes under each timing is
        # the practical ceiling
        "write_kernels": write_kernels,
        "step_zero_copy_commit": {"ms_per_step": dt_zc * 1e3 / args.steps,
                                  "tokens_per_s": w.batch * nc * args.steps / dt_zc,
                                  "what": "attend + sa_kv_append(NULL, NULL): the staged K/V committed "
                                          "without device work"},
        "attend_ms": attend_ms,
        "attend_tokens_per_s": w.batch * nc / (attend_ms * 1e-3),
        "pct_bf16_peak_attend": flops / (attend_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stream_cold_start": {"chunks": w.n_chunks, "ms": stream_ms, "ms_per_chunk": stream_ms / w.n_chunks},
        "step_ms": {"p50": pct(0.5), "p99": pct(0.99), "max": step_ms[-1], "n": len(step_ms)},
        "attend_step_ms": {"p50": pct(0.5, attend_only_ms), "p99": pct(0.99, attend_only_ms),
                           "max": attend_only_ms[-1], "n": len(attend_only_ms)},
        # a chunk of F latent frames must be produced within F frame periods; this layer's
        # attention step is one of many inside that budget
        "chunk_budget_ms": {fps: w.frames_per_chunk * 1000.0 / fps for fps in (24, 16)},
        "steps_within_chunk_budget_p99": {fps: w.frames_per_chunk * 1000.0 / fps / pct(0.99) for fps in (24, 16)},
        "mfma_probe": mfma_probe,
        "box": box_identity(torch),
        "configs": configs_res,
        "fp8_attend": fp8_res,
        "gdn_forward": gdn_res,
        "buffer_attend": buffer_res,
        "steps_attend": steps_res,
        "batch_attend": batch_res,
        "tiny_stream": tiny_res,
    }
    if not args.no_cpu_baseline:
        note("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        if configs_res is not None:
            # the oracle beside every bf16 shape: heads of one steady chunk for about 1.5 s each
            for name, c in configs_res.items():
                o = cpu_baseline(synth.WORKLOADS[name], 1.5)
                c["oracle"] = {"seconds_per_chunk": o["seconds_per_chunk"], "tokens_per_s": o["value"],
                               "sample": o["sample"], "cores": o["cores"],
                               "gpu_over_oracle": c["tokens_per_s"] / o["value"]}
        if tiny_res is not None:
            # the tiny workload's whole stream, the same schedule through the oracle
            o_s = tiny_oracle(synth)
            tiny_res["oracle"] = {"seconds_per_stream": o_s, "gpu_over_oracle": o_s * 1e3 / tiny_res["ms_per_stream_p50"]}
    s.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
