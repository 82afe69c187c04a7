"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from ``synth`` (seeded, host-side); expected values come from the
fp64 oracle only. The HIP path is reached through the C ABI
(causal_windowed_attention_amd), never through the oracle.
"""
import sys

import numpy as np
import torch

import causal_windowed_attention_amd as cwa
import synth
from oracle import StreamSpec, attention_probs


def say(*a):
    """Progress line that names the case before a GPU step (flushed)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def config_for(w: synth.Workload, **kw):
    return cwa.make_config(w.batch, w.heads, w.head_dim, w.frame_h, w.frame_w,
                           w.frames_per_chunk, w.sink_chunks, w.window_chunks, dtype=w.dtype, **kw)


def spec_for(w: synth.Workload, heads=None) -> StreamSpec:
    s = StreamSpec.from_workload(w)
    if heads is not None:
        from dataclasses import replace
        s = replace(s, heads=len(heads))
    return s


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype in ("bf16", "fp8"):
        t = t.to(torch.bfloat16)            # exact: the inputs are bf16-representable
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def err(got: np.ndarray, want: np.ndarray):
    """(max abs error, relative L2 error) over the entries that are not NaN in want."""
    m = ~np.isnan(want)
    d = got[m] - want[m]
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(want[m]), 1e-30))


def bf16_ulp_distance(a: torch.Tensor, b: np.ndarray) -> int:
    """Max distance in bf16 representable steps between a bf16 tensor and bf16-exact fp64 values."""
    bb = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(bb.float().double(), torch.from_numpy(np.ascontiguousarray(b)).double()), \
        "expected values must be bf16-exact"

    def ordered(t):
        i = t.contiguous().view(torch.int16).to(torch.int32)
        return torch.where(i < 0, -(i & 0x7FFF), i)
    return int((ordered(a.cpu()) - ordered(bb)).abs().max().item())


# bf16 tolerances (fp32 accumulation): max abs and relative L2 must both hold
BF16_ABS, BF16_REL = 2e-2, 1e-2
F32_ABS = 1e-4


def fp8_tolerance(qrot, keys, vals, scale, rows=None):
    """Per-element output tolerance [B, Nq, H, D], LSE tolerance [B, H, Nq] and the
    emulated output, from the stored operands of one attend of an fp8 stream.

    Derivation (the device rounds the softmax weights to E4M3 and normalises by the sum
    of the rounded weights, which the storage-emulating oracle does not): weight j of
    row i, in units of the normalised weights P_ij, is off by e_ij with |e_ij| <= h_ij =
    max(2^-4 P_ij, 2^-10 max_j P_ij / 2^4) (relative half-step of E4M3's normal range;
    half the subnormal step at the kernel's weight scale, where a row's largest weight
    is at least 2^4). To first order O_i moves by sum_j e_ij (v_j - O_i) and LSE_i by
    sum_j e_ij; independent errors with variance <= h^2 / 3 give 6-sigma bounds. Round
    to nearest is biased low on the falling density of exponentials by at most
    beta = 2^-6 / 24 per weight (relative), added as beta (P|V| + |O|) and beta. Plus
    2^-8 |O| for the bf16 output and 2e-3 / 1e-4 for fp32 accumulation and the fp8
    MFMA's own (at most 5e-5 of sum |products| on N(0,1)-like E4M3 data, unbiased)."""
    B, H, Nc, D = qrot.shape
    r = np.arange(Nc) if rows is None else np.asarray(rows)
    tol = np.zeros((B, len(r), H, D))
    ltol = np.zeros((B, H, len(r)))
    out = np.zeros((B, len(r), H, D))
    for b in range(B):
        for h in range(H):
            K = np.concatenate([k[b, h] for k in keys], axis=0)
            V = np.concatenate([v[b, h] for v in vals], axis=0)
            P = attention_probs(qrot[b, h, r], K, scale)
            h2 = np.maximum(2.0 ** -4 * P, 2.0 ** -10 * P.max(axis=1, keepdims=True) / 16.0) ** 2
            o = P @ V
            # sum_j h_ij^2 (v_jd - o_id)^2 expanded so no [Nq, Nk, D] array is formed
            var = (h2 @ V ** 2 - 2.0 * o * (h2 @ V) + o ** 2 * h2.sum(axis=1, keepdims=True)) / 3.0
            beta = 2.0 ** -6 / 24.0
            out[b, :, h] = o
            tol[b, :, h] = (6.0 * np.sqrt(np.maximum(var, 0.0)) + beta * (P @ np.abs(V) + np.abs(o))
                            + 2.0 ** -8 * np.abs(o) + 2e-3)
            ltol[b, h] = 6.0 * np.sqrt(h2.sum(axis=1) / 3.0) + beta + 1e-4
    return tol, ltol, out


def fp8_pure_tolerance(qrot, keys, vals, scale, kappa, rows=None, k_double=True):
    """Per-element output tolerance [B, Nq, H, D] and LSE tolerance [B, H, Nq] of the fp8 variant
    against the fp64 definition, from the exact operands of one attend (rotated Q, visible keys
    and values as the pure fp64 oracle holds them) and the Q factor kappa.

    Derivation. The device holds Q~ = E4M3(kappa Q) / kappa, K~ = E4M3(K), V~ = E4M3(V). An
    E4M3 rounding moves x by at most h(x) = max(2^-4 |x|, 2^-10) (half a step of 3 mantissa
    bits; half the subnormal step 2^-9), kappa-scaled for Q: h_q = max(2^-4 |Q|, 2^-10 / kappa).
    A re-rotated key (after a refresh) is rounded twice, so the key variance is doubled
    (k_double). Treating the roundings as independent, zero-mean, with variance <= h^2 / 3:
    * score s_ij = scale <Q_i, K_j> moves by scale sum_d (dq_id K_jd + Q_id dk_jd);
    * to first order O_i moves by sum_j P_ij ds_ij (V_j - O_i) + sum_j P_ij dv_j. The key and
      value parts are independent across j: variances sum_j P_ij^2 Var(ds_ij^K) (V_j - O_i)^2
      and sum_j P_ij^2 h(V_j)^2 / 3. The query part is shared by all keys of row i:
      scale sum_d dq_id C_i[d], C_i = sum_j P_ij K_jd (V_j - O_i), variance
      scale^2 / 3 sum_d h_q,id^2 C_i[d]^2;
    * LSE_i moves by sum_j P_ij ds_ij, with the same split;
    * second order: e^ds - 1 has mean Var(ds) / 2, bounded by half the largest score variance of
      the row, times sum_j P_ij |V_j - O_i| (outputs) or itself (LSE).
    The device also rounds the weights to E4M3 and normalises by their rounded sum; that part is
    fp8_tolerance's model (variance and bias), added here. The tolerance is 6 standard
    deviations of the sum plus the biases, 2^-8 |O| for the bf16 output and 2e-3 (1e-4 on LSE)
    for fp32 accumulation. The first-order model needs small score errors: it is meant for
    N(0, 1)-like activations, not for logits far beyond E4M3's 3 mantissa bits."""
    B, H, Nc, D = qrot.shape
    r = np.arange(Nc) if rows is None else np.asarray(rows)
    tol = np.zeros((B, len(r), H, D))
    ltol = np.zeros((B, H, len(r)))
    kf = 2.0 if k_double else 1.0
    for b in range(B):
        for h in range(H):
            K = np.concatenate([k[b, h] for k in keys], axis=0)
            V = np.concatenate([v[b, h] for v in vals], axis=0)
            Q = qrot[b, h, r]
            P = attention_probs(Q, K, scale)
            O = P @ V
            hq2 = np.maximum(2.0 ** -4 * np.abs(Q), 2.0 ** -10 / kappa) ** 2
            hk2 = kf * np.maximum(2.0 ** -4 * np.abs(K), 2.0 ** -10) ** 2
            hv2 = np.maximum(2.0 ** -4 * np.abs(V), 2.0 ** -10) ** 2
            var_sk = scale ** 2 / 3.0 * ((Q ** 2) @ hk2.T)          # [Nq, Nk] key part of ds
            var_sq = scale ** 2 / 3.0 * (hq2 @ (K ** 2).T)          # [Nq, Nk] query part of ds
            A = P ** 2 * var_sk
            var_ok = A @ V ** 2 - 2.0 * O * (A @ V) + O ** 2 * A.sum(axis=1, keepdims=True)
            var_ov = (P ** 2) @ hv2 / 3.0
            var_oq = np.empty_like(O)
            for i in range(len(r)):
                Ci = (K * P[i, :, None]).T @ V - np.outer(P[i] @ K, O[i])   # [D, D]
                var_oq[i] = scale ** 2 / 3.0 * (hq2[i] @ Ci ** 2)
            pk = P @ K
            var_l = scale ** 2 / 3.0 * (hq2 * pk ** 2).sum(axis=1) + A.sum(axis=1)
            second = 0.5 * (var_sk + var_sq).max(axis=1)            # [Nq]
            absdev = P @ np.abs(V) + np.abs(O)                       # >= sum_j P_ij |V_j - O_i|
            # weight rounding (the kernel's E4M3 weights), as in fp8_tolerance
            hp2 = np.maximum(2.0 ** -4 * P, 2.0 ** -10 * P.max(axis=1, keepdims=True) / 16.0) ** 2
            var_p = (hp2 @ V ** 2 - 2.0 * O * (hp2 @ V) + O ** 2 * hp2.sum(axis=1, keepdims=True)) / 3.0
            beta = 2.0 ** -6 / 24.0
            sd = np.sqrt(np.maximum(var_ok + var_ov + var_oq + var_p, 0.0))
            tol[b, :, h] = (6.0 * sd + (second[:, None] + beta) * absdev + 2.0 ** -8 * np.abs(O) + 2e-3)
            ltol[b, h] = (6.0 * np.sqrt(var_l + hp2.sum(axis=1) / 3.0) + second + beta + 1e-4)
    return tol, ltol


def check_fp8_pure(what, got, got_lse, pure_out, pure_lse, tol, ltol, rows=None, heads=None):
    """The fp8 output against the fp64 definition within fp8_pure_tolerance's bound."""
    g = host(got)
    gl = host(got_lse)
    if rows is not None:
        g = g[:, rows][:, :, heads]
        gl = gl[:, heads][:, :, rows]
    d = np.abs(g - pure_out)
    ratio = float((d / tol).max())
    ld = np.abs(gl - pure_lse)
    lratio = float((ld / ltol).max())
    rel = float(np.linalg.norm(g - pure_out) / max(np.linalg.norm(pure_out), 1e-30))
    say(f"  {what} vs fp64 definition: max err {d.max():.2e}, rel L2 {rel:.2e}, err/tol {ratio:.3f}; "
        f"lse max err {ld.max():.2e}, err/tol {lratio:.3f}")
    assert ratio <= 1.0 and lratio <= 1.0, (what, ratio, lratio)


def check_fp8_attend(what, got, got_lse, emu_out, emu_lse, tol, ltol, pure_out=None, rows=None, heads=None):
    g = host(got)
    gl = host(got_lse)
    if rows is not None:
        g = g[:, rows][:, :, heads]
        gl = gl[:, heads][:, :, rows]
    d = np.abs(g - emu_out)
    ratio = float((d / tol).max())
    ld = np.abs(gl - emu_lse)
    lratio = float((ld / ltol).max())
    msg = (f"  {what}: max err {d.max():.2e}, max err/tol {ratio:.3f}; lse max err {ld.max():.2e}, "
           f"err/tol {lratio:.3f}")
    if pure_out is not None:
        msg += f"; vs pure fp64 max {np.abs(g - pure_out).max():.2e}"
    say(msg)
    assert ratio <= 1.0 and lratio <= 1.0, (what, ratio, lratio)
