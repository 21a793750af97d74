"""The C ABI from plain C: tests/abi_step.c (built by __graft_entry__.build()
into tests/_build/abi_step) runs a whole step on buffers it allocates itself,
with no Python or torch in the process, and its outputs must equal the
Python binding's on the same inputs bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import synth
from gpu_harness import gpu_step, upload

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "abi_step")


def _write_inputs(path, inp):
    with open(path, "wb") as f:
        f.write(np.array([inp.R, inp.gamma, inp.V, inp.rank], np.int32).tobytes())
        f.write(np.array([inp.K], np.int64).tobytes())
        for a, dt in ((inp.U, np.float32), (inp.target, np.float32), (inp.W1, np.uint16), (inp.W2, np.uint16),
                      (inp.anchor, np.int32), (inp.temp, np.float32), (inp.u_draft, np.float32),
                      (inp.u_accept, np.float32), (inp.u_final, np.float32), (inp.c, np.float32)):
            f.write(np.ascontiguousarray(a, dtype=dt).tobytes())


def _read_outputs(path, R, gamma):
    raw = open(path, "rb").read()
    out, o = {}, 0
    for name, dt, n in (("y", np.int32, R * gamma), ("q_tok", np.float32, R * gamma),
                        ("q_stats", np.float32, R * gamma * 2), ("l", np.int32, R), ("row_offsets", np.int32, R + 1),
                        ("n_accept", np.int32, R), ("out_tok", np.int32, R), ("p_tok", np.float32, R * gamma)):
        b = n * np.dtype(dt).itemsize
        out[name] = np.frombuffer(raw[o:o + b], dt)
        o += b
    assert o == len(raw)
    return out


@pytest.mark.parametrize("R,V,rank", [(5, 3000, 64), (70, 2000, 128)], ids=["seg16", "seg64"])
def test_c_client_matches_the_binding(tmp_path, R, V, rank):
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build()"
    inp = synth.make_custom(77 + R, R, 4, V, rank, policy="mixed", K_mode="uniformK")
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_inputs(fin, inp)
    r = subprocess.run([EXE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    c = _read_outputs(fout, inp.R, inp.gamma)
    g = gpu_step(upload(inp), inp.K, inp.gamma)
    for k in c:
        np.testing.assert_array_equal(c[k], np.asarray(g[k]).reshape(-1), err_msg=k)
    print(f"[c abi R={R}] {inp.K=} rows={int(c['row_offsets'][-1])} identical to the binding", flush=True)
