"""The C ABI from plain C: tests/capi/adam_from_c.c (C99, built by
__graft_entry__.build() against liblso.so) runs three Adam steps over one
ragged block through lso_adam_step; its outputs must equal the binary32
emulation of the kernel's arithmetic bit for bit and the FP64 oracle
within the parity bound."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import fp32_exact as fx
import oracle
import synth

from gpu_util import assert_parity, log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "capi", "adam_from_c")


def test_adam_step_from_plain_c():
    assert os.path.exists(EXE), f"{EXE} is missing: build it with __graft_entry__.build()"
    n, steps = 1000 * 1024 + 3, 3
    master = synth.normal_f32(n, stream=98, block=0, purpose=synth.PURPOSE_MASTER, step=0, sigma=0.02)
    master[::2] = 0.0
    grads = [synth.normal_bf16(n, stream=98, block=0, purpose=synth.PURPOSE_GRAD, step=t, sigma=1e-3)
             for t in range(1, steps + 1)]
    with tempfile.TemporaryDirectory() as d:
        master.tofile(os.path.join(d, "master.f32"))
        for t, g in enumerate(grads, 1):
            g.tofile(os.path.join(d, f"grad_{t}.bf16"))
        log("capi", f"running {EXE} on {n} elements, {steps} steps")
        r = subprocess.run([EXE, d, str(n), str(steps)], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        got = {q: np.fromfile(os.path.join(d, f"out_{q}.f32"), np.float32) for q in ("master", "m", "v")}
        got["weight"] = np.fromfile(os.path.join(d, "out_weight.bf16"), np.uint16)
    p, m, v = master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    ref = dict(master=master.copy(), m=np.zeros(n, np.float32), v=np.zeros(n, np.float32),
               weight=np.zeros(n, np.uint16))
    for t, g in enumerate(grads, 1):
        p, m, v, w = fx.adam_binary32_v(p, m, v, g, fx.adam_constants(t, 1e-3, 0.9, 0.999, 1e-8))
        oracle.adam_step(ref["master"], ref["m"], ref["v"], g, ref["weight"], t, 1e-3, 0.9, 0.999, 1e-8)
    for q, want in (("master", p), ("m", m), ("v", v), ("weight", w)):
        dt = np.uint16 if want.dtype == np.uint16 else np.uint32
        bad = np.count_nonzero(got[q].view(dt) != want.view(dt))
        assert bad == 0, f"{q}: {bad} elements differ from the binary32 emulation"
    assert_parity(got, ref, 1e-6, "lso_adam_step from C")
