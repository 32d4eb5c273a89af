"""The oracle under the address and undefined-behaviour sanitizers (CPU only).

tests/oracle_sanitize.c compiles the oracle source into a program of its own
with gcc's -fsanitize=address,undefined (the runtimes linked statically, so
they come first), reads a problem from a file into heap blocks of exactly the
sizes the oracle may touch, and writes every output and term sum. Each case
here is an input family of the pins and the parity tests -- random locations
around the levels, far and non-finite locations, one-pixel, one-row and
one-column levels, sixteen levels, empty batches, queries and points, the
fused front-end with extreme logits, DCNv3 grids with padding, stride and
dilation -- and the sanitized run must finish cleanly and agree with the
in-tree build bit for bit.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize.c")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sanitize") / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-static-libasan", "-static-libubsan", DRIVER, "-o", exe, "-lm"], check=True)
    return exe


def _run(exe, tmp_path, header, arrays, n_out):
    prob, res = str(tmp_path / "problem.bin"), str(tmp_path / "result.bin")
    with open(prob, "wb") as f:
        np.asarray(header, np.int64).tofile(f)
        for a in arrays:
            np.ascontiguousarray(a).tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, prob, res], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"sanitized oracle failed ({r.returncode}):\n{r.stderr[-4000:]}"
    flat = np.fromfile(res, np.float64)
    assert flat.size == sum(n_out), "result size"
    return np.split(flat, np.cumsum(n_out)[:-1])


def _same(got, want, what):
    for i, (g, w) in enumerate(zip(got, want)):
        w = np.asarray(w, np.float64).reshape(-1)
        assert np.array_equal(g, w, equal_nan=True), f"{what}: output {i} differs from the in-tree build"


def _core_case(exe, tmp_path, value, shapes, lsi, loc, attn, g, what):
    B, Nv, M, D = value.shape
    L, K, Nq = loc.shape[3], loc.shape[4], loc.shape[1]
    header = [0, B, Nv, M, D, L, Nq, K]
    arrays = [np.asarray(shapes, np.int64), np.asarray(lsi, np.int64), value.astype(np.float64),
              loc.astype(np.float32), attn.astype(np.float64), g.astype(np.float64)]
    o, oa = oracle.forward(value, shapes, lsi, loc, attn, with_abs=True)
    want = [o] + list(oracle.backward(value, shapes, lsi, loc, attn, g, with_abs=True)[:3]) + \
        [oa] + list(oracle.backward(value, shapes, lsi, loc, attn, g, with_abs=True)[3:])
    got = _run(exe, tmp_path, header, arrays, [np.size(w) for w in want])
    _same(got, want, what)


def _core_inputs(rng, shapes, B=2, M=3, D=4, Nq=5, K=3, lo=-0.3, hi=1.3):
    shapes, lsi = pins.level_tables(shapes)
    L = shapes.shape[0]
    Nv = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((B, Nv, M, D))
    loc = rng.uniform(lo, hi, size=(B, Nq, M, L, K, 2)).astype(np.float32)
    attn = rng.standard_normal((B, Nq, M, L, K))
    g = rng.standard_normal((B, Nq, M, D))
    return value, shapes, lsi, loc, attn, g


def test_core_random(driver, tmp_path):
    for seed in (1, 2):
        rng = np.random.default_rng(seed)
        _core_case(driver, tmp_path, *_core_inputs(rng, ((5, 7), (3, 4), (2, 2))), f"core {seed}")


def test_core_far_and_nonfinite(driver, tmp_path):
    rng = np.random.default_rng(3)
    value, shapes, lsi, loc, attn, g = _core_inputs(rng, ((4, 6), (2, 3)), Nq=6, K=2)
    specials = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, -1.0, 2.0, 0.0, 1.0], np.float32)
    loc.reshape(-1)[:] = rng.choice(specials, size=loc.size)
    _core_case(driver, tmp_path, value, shapes, lsi, loc, attn, g, "core far / non-finite")


def test_core_thin_and_many_levels(driver, tmp_path):
    rng = np.random.default_rng(4)
    _core_case(driver, tmp_path, *_core_inputs(rng, ((1, 1), (1, 9), (7, 1), (3, 3))),
               "one-pixel, one-row, one-column levels")
    sixteen = tuple((1 + (i % 4), 1 + (i * 3) % 5) for i in range(16))
    _core_case(driver, tmp_path, *_core_inputs(rng, sixteen, B=1, M=2, Nq=3, K=2), "16 levels")


def test_core_empty(driver, tmp_path):
    rng = np.random.default_rng(5)
    for kw in (dict(Nq=0), dict(B=0), dict(K=0)):
        _core_case(driver, tmp_path, *_core_inputs(rng, ((3, 4), (2, 2)), **kw), f"empty {kw}")


def _fused_case(exe, tmp_path, value, shapes, lsi, ref, off, logits, g, what):
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = off.shape
    header = [1, B, Nv, M, D, L, Nq, K]
    arrays = [np.asarray(shapes, np.int64), np.asarray(lsi, np.int64), value.astype(np.float64),
              ref.astype(np.float32), off.astype(np.float32), logits.astype(np.float32),
              g.astype(np.float64)]
    o, oa = oracle.forward_fused(value, shapes, lsi, ref, off, logits, with_abs=True)
    b = oracle.backward_fused(value, shapes, lsi, ref, off, logits, g, with_abs=True)
    want = [o] + list(b[:4]) + [oa] + list(b[4:])
    got = _run(exe, tmp_path, header, arrays, [np.size(w) for w in want])
    _same(got, want, what)


def test_fused(driver, tmp_path):
    rng = np.random.default_rng(6)
    case = pins.random_fused_case(rng)
    _fused_case(driver, tmp_path, *case, "fused random")
    value, shapes, lsi, ref, off, logits, g = case
    logits = (rng.standard_normal(logits.shape) * 300.0).astype(np.float32)
    off = (rng.standard_normal(off.shape) * 50.0).astype(np.float32)
    _fused_case(driver, tmp_path, value, shapes, lsi, ref, off, logits, g,
                "fused extreme logits, far offsets")


def _dcn_case(exe, tmp_path, x, off, mask, g, kernel, stride, pad, dil, what):
    B, H, W, G, D = x.shape
    Ho, Wo = off.shape[1], off.shape[2]
    header = [2, B, H, W, G, D, kernel[0], kernel[1], stride[0], stride[1], pad[0], pad[1],
              dil[0], dil[1], Ho, Wo]
    arrays = [x.astype(np.float64), off.astype(np.float32), mask.astype(np.float64),
              g.astype(np.float64)]
    o, oa = oracle.dcn_forward(x, off, mask, kernel, stride, pad, dil, with_abs=True)
    b = oracle.dcn_backward(x, off, mask, g, kernel, stride, pad, dil, with_abs=True)
    want = [o] + list(b[:3]) + [oa] + list(b[3:])
    got = _run(exe, tmp_path, header, arrays, [np.size(w) for w in want])
    _same(got, want, what)


def test_dcn(driver, tmp_path):
    rng = np.random.default_rng(7)
    for kernel, stride, pad, dil in pins.DCN_CONFIGS:
        H, W, G, D, B = 6, 7, 2, 3, 2
        Ho, Wo = pins._dcn_out_size(H, W, kernel, stride, pad, dil)
        K = kernel[0] * kernel[1]
        x = rng.standard_normal((B, H, W, G, D))
        off = (rng.standard_normal((B, Ho, Wo, G, K, 2)) * 2.0).astype(np.float32)
        off.reshape(-1)[::7] = np.nan
        off.reshape(-1)[3::11] = 1e30
        mask = rng.standard_normal((B, Ho, Wo, G, K))
        g = rng.standard_normal((B, Ho, Wo, G, D))
        _dcn_case(driver, tmp_path, x, off, mask, g, kernel, stride, pad, dil,
                  f"dcn {kernel} {stride} {pad} {dil}")
