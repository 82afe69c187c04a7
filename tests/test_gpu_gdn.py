"""GPU parity of the gated delta rule forward (sa_gdn_forward) against the fp64 oracle.

The oracle (oracle/gdn.py) runs the published recurrence token by token; the GPU path runs
the chunkwise rewriting in fp32 (64-token blocks). Tolerance, derived: outputs are bf16,
so 2^-8 |o| covers their rounding; the fp32 path's own error is bounded per block by its
longest fp32 sums (128 products, relative 128 * 2^-24 ~ 8e-6) and, the recurrence being a
contraction for unit keys with alpha, beta <= 1, adds up over at most nb blocks
(nb * 8e-6 of the largest magnitude). So |o - o_ref| <= 2^-8 |o_ref| + nb * 1e-5 * max|o_ref|
per (b, h) and |S - S_ref| <= nb * 1e-5 * max|S_ref|.
"""
import numpy as np
import pytest
import torch

import causal_windowed_attention_amd as cwa
import synth
from gpu_util import host, say
from oracle import gdn_recurrent

pytestmark = pytest.mark.gpu


def _dev(x, bf16):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


def _check(what, o, S, o_ref, S_ref, nb):
    o, S = host(o), host(S)
    B, N, H, D = o_ref.shape
    worst_o = worst_s = 0.0
    for b in range(B):
        for h in range(H):
            ref = o_ref[b, :, h]
            tol = 2.0 ** -8 * np.abs(ref) + max(nb, 1) * 1e-5 * np.abs(ref).max()
            worst_o = max(worst_o, float((np.abs(o[b, :, h] - ref) / tol).max()) if N else 0.0)
            sref = S_ref[b, h]
            worst_s = max(worst_s, float(np.abs(S[b, h] - sref).max() / (max(nb, 1) * 1e-5 * np.abs(sref).max())))
    say(f"  {what}: max |o err| / tol {worst_o:.3f}, max |S err| / tol {worst_s:.3f}")
    assert worst_o <= 1.0 and worst_s <= 1.0, (what, worst_o, worst_s)


@pytest.mark.parametrize("B,N,H,D", [(1, 150, 2, 64), (2, 64, 1, 128), (1, 333, 3, 128), (1, 1, 2, 64),
                                     (1, 63, 1, 128)])
def test_gdn_matches_recurrence(B, N, H, D):
    say(f"gdn B {B} N {N} H {H} D {D}")
    q, k, v, a, b_, s0 = synth.gdn_inputs(B, N, H, D, seed=N + D)
    o, S = cwa.gdn_forward(_dev(q, True), _dev(k, True), _dev(v, True), _dev(a, False), _dev(b_, False),
                           state=_dev(s0, False))
    torch.cuda.synchronize()
    o_ref, S_ref = gdn_recurrent(q, k, v, a, b_, s0)
    _check(f"B {B} N {N} H {H} D {D}", o, S, o_ref, S_ref, -(-N // 64))


def test_gdn_carried_state_in_place_and_zero_state():
    """Two calls with the state carried (in place) equal one call over both token ranges;
    no initial state means zeros; N = 0 passes the state through (zeros without one)."""
    B, N, H, D = 1, 200, 2, 128
    q, k, v, a, b_, _ = synth.gdn_inputs(B, N, H, D, seed=9, state=False)
    o_ref, S_ref = gdn_recurrent(q, k, v, a, b_)
    d = lambda x, bf=True: _dev(x, bf)
    state = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    o1, _ = cwa.gdn_forward(d(q[:, :70]), d(k[:, :70]), d(v[:, :70]), d(a[:, :, :70], False), d(b_[:, :, :70], False),
                            state=None, state_out=state)
    o2, _ = cwa.gdn_forward(d(q[:, 70:]), d(k[:, 70:]), d(v[:, 70:]), d(a[:, :, 70:], False), d(b_[:, :, 70:], False),
                            state=state, state_out=state)
    torch.cuda.synchronize()
    _check("split 70 + 130, state in place", torch.cat([o1, o2], dim=1), state, o_ref, S_ref, 4)
    before = state.clone()
    e = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    ea = torch.empty((B, H, 0), dtype=torch.float32, device="cuda")
    _, s_out = cwa.gdn_forward(e, e, e, ea, ea, state=state)
    z = torch.full_like(state, 7.0)
    _, z_out = cwa.gdn_forward(e, e, e, ea, ea, state=None, state_out=z)     # no state in: zeros out
    torch.cuda.synchronize()
    assert torch.equal(s_out, before)
    assert z_out.data_ptr() == z.data_ptr() and not torch.any(z)


@pytest.mark.parametrize("name", ["hybrid1280x704", "wan1.3b"])
def test_gdn_full_chunk_sampled_heads(name):
    """One video chunk of a workload shape (hybrid1280x704: Nc = 3520, H = 16; wan1.3b:
    Nc = 4680, H = 12; D = 128) through the GDN block; the oracle runs the first and last
    heads (heads are independent) over every token."""
    w = synth.WORKLOADS[name]
    B, N, H, D = w.batch, w.tokens_per_chunk, w.heads, w.head_dim
    say(f"gdn full chunk {name}: B {B} N {N} H {H} D {D}")
    q, k, v, a, b_, s0 = synth.gdn_inputs(B, N, H, D, seed=w.cfg_id)
    o, S = cwa.gdn_forward(_dev(q, True), _dev(k, True), _dev(v, True), _dev(a, False), _dev(b_, False),
                           state=_dev(s0, False))
    torch.cuda.synchronize()
    hs = [0, H - 1]
    o_ref, S_ref = gdn_recurrent(q[:, :, hs], k[:, :, hs], v[:, :, hs], a[:, hs], b_[:, hs], s0[:, hs])
    _check(f"{name} heads {hs}", o[:, :, hs], S[:, hs], o_ref, S_ref, -(-N // 64))
