"""The C ABI used from plain C (tests/c_abi/forward.c), without Python in between.

CPU: the header compiles as C99 and the caller links against libmoe.so.
GPU: the caller runs one layer on seeded inputs handed over in a file; its
top-k ids must equal the oracle's exactly, its weights within 2e-6 and y
within 2e-2 * rms(y) (the bars of the other parity tests), and it must see
MOE_ERR_INVALID_ARG for k > E.
"""
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest

import gen
import oracle
from top_routing_grouped_gemm_amd import build as hipbuild

HERE = os.path.dirname(os.path.abspath(__file__))


def _lib_built():
    return os.path.exists(hipbuild.LIB)


@pytest.mark.skipif(not _lib_built(), reason="libmoe.so not built")
def test_c_caller_compiles_and_links():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "forward")
        res = subprocess.run(hipbuild.c_example_cmd(hipbuild.C_EXAMPLE, out), capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        assert res.stderr.strip() == "", f"warnings compiling the C caller:\n{res.stderr}"
        assert os.path.exists(out)


def _write_inputs(path, I):
    with open(path, "wb") as f:
        dt = 1 if I.dtype == "bf16" else 0
        has_bias = I.bias is not None
        f.write(struct.pack("<7i", I.T, I.H, I.F, I.E, I.k, dt, int(has_bias)))
        f.write(struct.pack("<f", I.drop))
        f.write(np.ascontiguousarray(I.x).tobytes())
        f.write(np.ascontiguousarray(I.Wr).tobytes())
        if has_bias:
            f.write(np.ascontiguousarray(I.bias, dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(I.W1()).tobytes())
        f.write(np.ascontiguousarray(I.W2()).tobytes())


@pytest.mark.gpu
@pytest.mark.parametrize("over", [
    dict(T=96, H=128, F=192, E=8, k=2, dtype="bf16", seed=801),
    dict(T=40, H=64, F=64, E=16, k=4, dtype="f32", seed=802, drop=0.1, zipf=1.2),   # router bias
    dict(T=700, H=128, F=192, E=5, k=2, dtype="bf16", seed=803),   # 256-row tiles
], ids=["bf16", "f32-drop-bias", "bf16-large"])
def test_c_caller_runs_layer(over):
    exe = hipbuild.C_EXAMPLE_BIN
    if not os.path.exists(exe):
        pytest.skip("tests/c_abi/forward not built (build() makes it)")
    I = gen.make_inputs("tiny", **over)
    print(f"case {over}", flush=True)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        _write_inputs(fin, I)
        res = subprocess.run([exe, fin, fout], capture_output=True, text=True, timeout=120)
        print(res.stdout, res.stderr, flush=True)
        assert res.returncode == 0, res.stderr
        assert "k > E rejected: MOE_ERR_INVALID_ARG" in res.stdout
        raw = open(fout, "rb").read()
    T, H, k = I.T, I.H, I.k
    y = np.frombuffer(raw, dtype=np.float32, count=T * H).reshape(T, H)
    ids = np.frombuffer(raw, dtype=np.int32, count=T * k, offset=4 * T * H).reshape(T, k)
    w = np.frombuffer(raw, dtype=np.float32, count=T * k, offset=4 * T * H + 4 * T * k).reshape(T, k)
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), I.f64(I.W2()), k, I.drop)
    assert np.array_equal(ids, ref.route.ids)
    assert np.abs(w - ref.route.w).max() <= 2e-6
    rms = float(np.sqrt((ref.y ** 2).mean()))
    assert float(np.abs(y - ref.y).max()) <= 2e-2 * rms
