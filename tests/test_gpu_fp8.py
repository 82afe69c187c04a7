"""GPU parity of the fp8 cache variant (SA_FP8) against the fp64 oracle.

What the device stores is checked code by code: V is a plain bf16 -> E4M3 rounding and
must match the oracle's E4M3 rounding exactly; rotated K and Q (Q times the factor
fp8_q_scale) come from fp32 arithmetic on the device and fp64 in the oracle, so an
element may take the other neighbour only where the fp32 error can reach an E4M3
rounding boundary.

Attention is compared with the storage-emulating oracle (RingOracle, storage 'fp8':
exact softmax over the E4M3-rounded Q, K and V the device holds). The device also
rounds the softmax weights to E4M3 and normalises by the sum of the rounded weights
(O_i = sum_j p~_ij v_j / sum_j p~_ij, LSE from the same sum), which the oracle does not;
the tolerance is derived from that rounding. Weight j of row i, in units of the
normalised weights P_ij, is rounded with an error e_ij of at most h_ij =
max(2^-4 P_ij, 2^-10 max_j P_ij / 2^4): a relative half-step of 2^-4 in E4M3's normal
range, or half the subnormal step 2^-9 at the kernel's weight scale (the largest weight
of a row is at least 2^4 there). To first order O_i moves by sum_j e_ij (v_j - O_i) and
LSE_i by sum_j e_ij. The errors are independent; with a uniform-error variance bound
h^2 / 3 their standard deviations are at most sigma_id = sqrt(sum_j h_ij^2 (v_jd -
O_id)^2 / 3) and sqrt(sum_j h_ij^2 / 3). Round to nearest even is unbiased only for a
flat density across a rounding step; exponentials of smooth scores are denser at the
low end of a step, which biases each normal-range weight low by about (step / value)^2
/ 24 <= 2^-6 / 24 of itself: at most beta = 2^-6 / 24 on the LSE and beta sum_j P_ij
|v_j - O_i| <= beta (P|V| + |O|) on an output. The test allows 6 sigma plus that bias,
plus 2^-8 |O| for the bf16 output rounding and 2e-3 (outputs) or 1e-4 (LSE) for fp32
accumulation and the fp8 MFMA's own (measured on N(0,1)-like E4M3 data: at most 5e-5
of sum |products|, unbiased). The error against the pure fp64 oracle (dominated by the
E4M3 rounding of Q and K) is printed.
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from gpu_util import (check_fp8_attend, check_fp8_pure, config_for, dev, fp8_pure_tolerance, fp8_tolerance,
                      host, say, spec_for)
from oracle import HistoryOracle, RingOracle, fp8_q_scale, round_e4m3

pytestmark = pytest.mark.gpu

CASES = {
    # Nc = 180 and 70: key tiles straddle chunk boundaries, the last query tile is ragged
    "d128_s1w3": dict(heads=2, frame_h=6, frame_w=10, frames_per_chunk=3, window_chunks=3),
    "d128_s2w2": dict(heads=1, frame_h=5, frame_w=7, frames_per_chunk=2, sink_chunks=2, window_chunks=2),
}


def _workload(**kw):
    return synth.small_variant(synth.WORKLOADS["wan1.3b"], dtype="fp8", **kw)


def _check_codes(what, got, want_fp64, delta):
    """got: E4M3 values from the device; want_fp64: the exact (unrounded) values; delta:
    bound on the device's fp32 error of each element (0 where its value is exact)."""
    lo, hi = round_e4m3(want_fp64 - delta), round_e4m3(want_fp64 + delta)
    ok = (got == lo) | (got == hi)
    exact = (delta == 0)
    say(f"  {what}: {int((~ok).sum())} codes outside the rounding interval of {ok.size}; "
        f"{int((lo != hi).sum())} elements near a boundary")
    assert ok.all(), what
    assert np.array_equal(got[exact], round_e4m3(want_fp64[exact])), what


def _pair_delta(x):
    """fp32 error bound of a rotated pair element: 2^-21 (|u0| + |u1|) of its input pair."""
    a = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    return np.repeat(a, 2, axis=-1) * 2.0 ** -21


@pytest.mark.parametrize("case", list(CASES))
def test_fp8_stream_matches_oracle(case):
    w = _workload(**CASES[case])
    nc = w.tokens_per_chunk
    say(f"fp8 {case}: H {w.heads} D {w.head_dim} Nc {nc} S {w.sink_chunks} W {w.window_chunks}")
    s = cwa.Stream(config_for(w))
    spec = spec_for(w)
    emu, pure_ring, hist = RingOracle(spec, storage="fp8"), RingOracle(spec), HistoryOracle(spec)
    n_chunks = w.sink_chunks + w.window_chunks + 4
    for c in range(n_chunks):
        if c == w.sink_chunks + w.window_chunks + 1:
            d = s.rope_refresh(-1, 0)
            assert d == emu.refresh(None, 0) == pure_ring.refresh(None, 0) == hist.refresh(None, 0)
        if c == n_chunks - 2:
            ks, vs = synth.sink_kv(w, 0)
            s.sink_update(dev(ks, w.dtype), dev(vs, w.dtype))
            for o in (emu, pure_ring, hist):
                o.sink_update(ks, vs)
        q, k, v = synth.chunk_qkv(w, c)
        lse = torch.empty((w.batch, w.heads, nc), dtype=torch.float32, device="cuda")
        out = s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse)
        torch.cuda.synchronize()
        qrot, keys, vals = emu.operands(q, k, v)
        tol, ltol, emu_out = fp8_tolerance(qrot, keys, vals, spec.softmax_scale)
        _, emu_lse = emu.attend(q, k, v)
        pure_out, pure_lse = hist.attend(q, k, v)
        check_fp8_attend(f"chunk {c}", out, lse, emu_out, emu_lse, tol, ltol, pure_out)
        ptol, pltol = fp8_pure_tolerance(*pure_ring.operands(q, k, v), spec.softmax_scale, fp8_q_scale(spec))
        check_fp8_pure(f"chunk {c}", out, lse, pure_out, pure_lse, ptol, pltol)
        if c == 1:                               # the Q scratch of this attend, before any refresh
            qs = s.q_scratch_view().cpu().float().numpy().astype(np.float64).reshape(w.batch, w.heads, nc, -1)
            kappa = fp8_q_scale(spec)
            qwant = kappa * pure_ring.staged(q, k, v)[0]
            qin = np.transpose(q, (0, 2, 1, 3)).astype(np.float64)
            # rotation error times the factor, plus the fp32 product and the fp32 factor itself
            _check_codes("Q scratch", qs, qwant, kappa * _pair_delta(qin) + 2.0 ** -22 * np.abs(qwant))
        s.kv_append()                            # commit the staged chunk
        for o in (emu, pure_ring, hist):
            o.append(k, v)
        if c == w.sink_chunks + 1:               # cache codes of every committed chunk so far
            kc = s.k_cache_view().cpu().float().numpy().astype(np.float64)
            vt = s.vt_cache_view().cpu().float().numpy().astype(np.float64)
            for slot in range(s.query()["n_slots"]):
                info = s.slot(slot)
                if info["kind"] not in (cwa.SA_SLOT_SINK, cwa.SA_SLOT_WINDOW):
                    continue
                cid = info["chunk_id"]
                _, kraw, vraw = synth.chunk_qkv(w, cid)
                rows = slice(slot * nc, (slot + 1) * nc)
                kdev = kc[:, rows].reshape(w.batch, w.heads, nc, -1)
                kin = np.transpose(kraw, (0, 2, 1, 3)).astype(np.float64)
                _check_codes(f"K slot {slot} (chunk {cid})", kdev, pure_ring.stored_k(cid), _pair_delta(kin))
                vdev = np.transpose(vt[:, :, rows], (0, 2, 1)).reshape(w.batch, w.heads, nc, -1)
                vwant = pure_ring.stored_v(cid)
                _check_codes(f"V slot {slot} (chunk {cid})", vdev, vwant, np.zeros_like(vwant))
    s.close()


@pytest.mark.parametrize("name", ["wan1.3b", "wan14b_b2", "hybrid1280x704", "long512p"])
def test_fp8_full_size_sampled(name):
    """Full workload shapes with an fp8 cache (wan1.3b: H = 12, Nc = 4680, S = 1, W = 6;
    wan14b_b2: two streams of 40 heads; hybrid1280x704: outlier channels scaled x8 in Q and
    K; long512p: H = 24, Nc = 2048), after the ring has wrapped: sampled rows of two heads
    against the storage-emulating oracle."""
    w = synth.small_variant(synth.WORKLOADS[name], dtype="fp8")
    nc = w.tokens_per_chunk
    heads = [0, w.heads - 1]
    say(f"fp8 {name} full size: B {w.batch} H {w.heads} Nc {nc}; heads {heads}")
    s = cwa.Stream(config_for(w))
    spec = spec_for(w, heads)
    emu, hist, pure = RingOracle(spec, storage="fp8"), HistoryOracle(spec), RingOracle(spec)
    n = w.sink_chunks + w.window_chunks + 2
    for c in range(n):
        q, k, v = synth.chunk_qkv(w, c)
        if c < n - 1:
            s.kv_append(dev(k, w.dtype), dev(v, w.dtype))
            for o in (emu, hist, pure):
                o.append(k[:, :, heads], v[:, :, heads])
    lse = torch.empty((w.batch, w.heads, nc), dtype=torch.float32, device="cuda")
    out = s.chunk_attend(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), lse=lse)
    torch.cuda.synchronize()
    g = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(nc - 8, nc), g.choice(nc, 40, replace=False)]))
    qh, kh, vh = q[:, :, heads], k[:, :, heads], v[:, :, heads]
    qrot, keys, vals = emu.operands(qh, kh, vh)
    tol, ltol, emu_out = fp8_tolerance(qrot, keys, vals, spec.softmax_scale, rows=rows)
    _, emu_lse = emu.attend(qh, kh, vh, rows=list(rows))
    pure_out, pure_lse = hist.attend(qh, kh, vh, rows=list(rows))
    check_fp8_attend(f"{name} fp8 sampled", out, lse, emu_out, emu_lse[:, :, rows], tol, ltol, pure_out[:, rows],
                  rows=rows, heads=heads)
    if not w.outlier_channels:
        # N(0, 1) activations: held to the fp64 definition within the derived E4M3 budget (the
        # outlier workload's logits are beyond E4M3's 3 mantissa bits; see fp8_pure_tolerance)
        ptol, pltol = fp8_pure_tolerance(*pure.operands(qh, kh, vh), spec.softmax_scale, fp8_q_scale(spec),
                                         rows=rows, k_double=False)
        check_fp8_pure(f"{name} fp8 sampled", out, lse, pure_out[:, rows], pure_lse[:, :, rows], ptol, pltol,
                       rows=rows, heads=heads)
    s.close()
