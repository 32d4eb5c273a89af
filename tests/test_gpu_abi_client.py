"""The C ABI from a plain C99 program (tests/abi_client.c: gcc, the HIP
runtime and libmsda.so, no PyTorch): forward and backward on the GPU,
compared element by element with the CPU oracle at the fp32 tolerance
|x - r| <= 1e-5 |r| + 1e-5 S."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from scale_deformable_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_client")


def check(name, got, ref, ref_abs):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    bad = ~(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-5 * ref_abs)
    assert not bad.any(), f"{name}: {bad.sum()} of {bad.size} elements outside tolerance"


def test_c_client_matches_oracle(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BINARY):
        import abi_client   # normally built by __graft_entry__.build(); a gcc
        abi_client.build()  # compile of one C file, on the host
    w = wl.Workload("c_client", B=2, M=4, D=32, K=3, shapes=((13, 21), (7, 11), (4, 6)),
                    ref="uniform", sigma_px=2.0, Nq=45, seed=640)
    x = wl.generate(w)
    (tmp_path / "dims.txt").write_text(
        f"{w.B} {w.Nv} {w.M} {w.D} {w.L} {w.num_queries} {w.K}\n")
    for name, key, dt in (("value.bin", "value", np.float32), ("shapes.bin", "spatial_shapes",
                          np.int64), ("lsi.bin", "level_start_index", np.int64),
                          ("loc.bin", "sampling_locations", np.float32),
                          ("attn.bin", "attention_weights", np.float32),
                          ("gout.bin", "grad_output", np.float32)):
        np.ascontiguousarray(x[key], dtype=dt).tofile(tmp_path / name)
    print(f"[abi_client] {w.name}: B={w.B} M={w.M} D={w.D} L={w.L} K={w.K} "
          f"Nq={w.num_queries}", flush=True)
    r = subprocess.run([BINARY, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    print(r.stdout.strip(), flush=True)
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
            x["attention_weights"])
    ref, ref_abs = oracle.forward(*args, with_abs=True)
    check("output", np.fromfile(tmp_path / "out.bin", np.float32), ref, ref_abs)
    rgv, rgl, rga, agv, agl, aga = oracle.backward(*args, x["grad_output"], with_abs=True)
    check("grad_value", np.fromfile(tmp_path / "gvalue.bin", np.float32), rgv, agv)
    check("grad_sampling_locations", np.fromfile(tmp_path / "gloc.bin", np.float32), rgl, agl)
    check("grad_attention_weights", np.fromfile(tmp_path / "gattn.bin", np.float32), rga, aga)
