"""Planted mistakes in the oracle, on the CPU: each one must fail at least one pin.

Every entry below is one plausible error (a sign, an exponent, a swapped axis or index,
a dropped term, a wrong direction or order) written as a textual change to a file of
oracle/. The oracle package, synth/ and the oracle pin files are copied into a temporary
tree, the change is applied there, and the pins run in a subprocess; the test fails if
any planted mistake lets every pin pass. The unchanged copy must pass. Changes that
cannot alter any result (a slice the surrounding code already bounds) are not listed: the
window entry changes both the trimming and the selection of the history, since either
alone is masked by the other.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_attention.py", "test_oracle_fp8.py", "test_oracle_gdn.py", "test_oracle_rope_bf16.py",
        "test_oracle_stream.py"]

# (file under oracle/, [(text, replacement), ...], what the mistake is)
M = [
 ("rope.py", [("u[..., offset:offset + seg_len:2] = a * c - b * s", "u[..., offset:offset + seg_len:2] = a * c + b * s")], "rotation sign"),
 ("rope.py", [("np.power(float(theta), -2.0 * j / seg_len)", "np.power(float(theta), -1.0 * j / seg_len)")], "frequency exponent"),
 ("rope.py", [("_rotate_segment(out, dt, dh, y, theta)", "_rotate_segment(out, dt, dh, x, theta)")], "h segment rotated by x"),
 ("rope.py", [("return n // per_frame, (n // frame_w) % frame_h, n % frame_w", "return n // per_frame, (n // frame_h) % frame_w, n % frame_h")], "column-major raster"),
 ("attention.py", [("        p = np.exp(s - m)\n        denom", "        p = np.exp(s)\n        denom")], "softmax without the max"),
 ("attention.py", [("lse[r0:r0 + block_rows] = (m + np.log(denom))[:, 0]", "lse[r0:r0 + block_rows] = (np.log(denom))[:, 0]")], "LSE without the max"),
 ("attention.py", [("s = (q[r0:r0 + block_rows] @ k.T) * scale", "s = (q[r0:r0 + block_rows] @ k.T)")], "scale dropped"),
 ("attention.py", [("out[r0:r0 + block_rows] = (p @ v) / denom", "out[r0:r0 + block_rows] = (p @ v)")], "unnormalised output"),
 ("stream.py", [("            e[1] -= delta\n        self.t_next -= delta", "            e[1] += delta\n        self.t_next -= delta")], "history refresh direction"),
 ("stream.py", [("rotate_temporal(self.ring_k[j], -delta, s.rope, s.theta)", "rotate_temporal(self.ring_k[j], delta, s.rope, s.theta)")], "ring re-rotation direction"),
 ("stream.py", [("self.ring_meta[j][2] -= delta", "self.ring_meta[j][2] += delta")], "ring t0 update"),
 ("stream.py", [("return self.ring[max(0, len(self.ring) - W):] if W > 0 else []", "return self.ring[max(0, len(self.ring) - W - 1):] if W > 0 else []"),
                ("if len(self.ring) > s.window_chunks:", "if len(self.ring) > s.window_chunks + 1:"),
                ("self.ring = self.ring[len(self.ring) - s.window_chunks:]", "self.ring = self.ring[len(self.ring) - s.window_chunks - 1:]")], "history window one chunk too long"),
 ("stream.py", [("self.ring_next = (self.ring_next + 1) % s.window_chunks", "self.ring_next = (self.ring_next + 2) % s.window_chunks")], "ring slot order"),
 ("stream.py", [("            self.sink_meta[j] = [True, self.n_appends, self.t_next]", "            self.sink_meta[j] = [True, self.n_appends, 0]")], "ring sink chunks all at t = 0"),
 ("stream.py", [("entry = [self.n_appends, self.t_next, np.array(k", "entry = [self.n_appends, self.t_next + 1, np.array(k")], "chunks committed one frame late"),
 ("stream.py", [("                tmp.t_next = self.t_next + j * s.frames_per_chunk", "                tmp.t_next = self.t_next")], "steps: every chunk at t_next"),
 ("stream.py", [("            if not steps and j + 1 < n:\n                tmp.append(k[:, sl], v[:, sl])", "            if not steps and j + 1 < n:\n                tmp.t_next += s.frames_per_chunk")], "buffer: earlier chunks not visible"),
 ("stream.py", [("            self.sink[j] = [-1, j * s.frames_per_chunk,", "            self.sink[j] = [-1, 0,")], "history sink update: all at t = 0"),
 ("stream.py", [("    k = -math.floor(math.log2(c))", "    k = -math.ceil(math.log2(c))")], "fp8 query factor in [0.5, 1)"),
 ("stream.py", [("            return self.spec.sink_chunks * self.spec.frames_per_chunk", "            return self.spec.sink_chunks")], "refresh default base in chunks"),
 ("rope.py", [("        dh = 2 * (head_dim // 6)", "        dh = 2 * (head_dim // 8)")], "default RoPE split"),
 ("attention.py", [("            scores.append(acc * scale)", "            scores.append(acc)")], "scalar twin without scale"),
 ("attention.py", [("    s = (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T) * scale",
                   "    s = (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)")], "weights: scale dropped"),
 ("attention.py", [("    s = (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T) * scale",
                   "    s = (np.asarray(k, dtype=np.float64) @ np.asarray(q, dtype=np.float64).T) * scale")], "weights: transposed score product"),
 ("attention.py", [("    return p / p.sum(axis=1, keepdims=True)", "    return p / p.sum(axis=0, keepdims=True)")], "weights: normalised over queries"),
 ("attention.py", [("    m = s.max(axis=1, keepdims=True)\n    p = np.exp(s - m)\n    return",
                   "    m = s.max(axis=0, keepdims=True)\n    p = np.exp(s - m)\n    return")], "weights: maximum over queries"),
 ("bf16.py", [("spacing_exp = np.maximum(e - 8, -133)", "spacing_exp = np.maximum(e - 9, -133)")], "bf16 spacing"),
 ("bf16.py", [("np.rint(np.ldexp(v, -spacing_exp))", "np.trunc(np.ldexp(v, -spacing_exp))")], "bf16 truncation"),
 ("fp8.py", [("spacing_exp = np.maximum(e - 4, -9)", "spacing_exp = np.maximum(e - 3, -9)")], "E4M3 spacing"),
 ("fp8.py", [("spacing_exp = np.maximum(e - 4, -9)", "spacing_exp = np.maximum(e - 4, -10)")], "E4M3 subnormal spacing"),
 ("fp8.py", [("np.rint(np.ldexp(v, -spacing_exp))", "np.trunc(np.ldexp(v, -spacing_exp))")], "E4M3 truncation"),
 ("gdn.py", [("S = a * (S - b * Sk", "S = a * (S + b * Sk")], "delta-rule sign"),
 ("gdn.py", [("S = a * (S - b * Sk[..., None] * kt[:, :, None, :]) + b", "S = (S - b * Sk[..., None] * kt[:, :, None, :]) + b")], "decay dropped"),
 ("gdn.py", [("S = a * (S - b * Sk[..., None] * kt[:, :, None, :]) + b * vt[..., None] * kt[:, :, None, :]",
              "S = a * (S - b * Sk[..., None] * kt[:, :, None, :] + b * vt[..., None] * kt[:, :, None, :])")], "decay on the write"),
 ("gdn.py", [(") + b * vt[..., None]", ") + vt[..., None]")], "write strength dropped"),
 ("gdn.py", [("        Sk = np.einsum", "        S_old = S\n        Sk = np.einsum"),
             ('o[:, t] = np.einsum("bhvk,bhk->bhv", S, qt)', 'o[:, t] = np.einsum("bhvk,bhk->bhv", S_old, qt)')], "output from the old state"),
]

def _tree(dst, edits=(), fname=None):
    for d in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in ["conftest.py"] + PINS:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    if fname is not None:
        p = os.path.join(dst, "oracle", fname)
        with open(p) as fh:
            s = fh.read()
        for old, new in edits:
            assert s.count(old) == 1, f"oracle/{fname} changed: update the planted mistake {old!r}"
            s = s.replace(old, new)
        with open(p, "w") as fh:
            fh.write(s)


def _pins_pass(dst) -> bool:
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + ["tests/" + p for p in PINS], cwd=dst, capture_output=True, text=True, timeout=600)
    return r.returncode == 0


def test_unchanged_copy_passes(tmp_path):
    _tree(str(tmp_path))
    assert _pins_pass(str(tmp_path))


def test_every_planted_mistake_fails_a_pin(tmp_path):
    def caught(i):
        fname, edits, what = M[i]
        dst = os.path.join(str(tmp_path), f"m{i}")
        _tree(dst, edits, fname)
        return what, not _pins_pass(dst)
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(caught, range(len(M))))
    survivors = [what for what, ok in results if not ok]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
