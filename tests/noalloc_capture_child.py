"""Child process of the capture-rule test (run by tests/test_zz_no_alloc.py,
not collected by pytest): in a fresh process, the first
lso_adam_step_noalloc call on the device is made under stream capture and
must be refused (LSO_E_INVALID, nothing enqueued); after one call outside
the capture, captured calls work and a replay equals the eager update."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import layer_streamed_optimizer_amd as lso  # noqa: E402
import synth  # noqa: E402
from gpu_util import Arena  # noqa: E402


def main():
    torch.cuda.set_device(0)
    sizes = [1000 + 37 * i for i in range(8)]   # more than 4 blocks: the table goes to the array
    a, b = Arena(sizes), Arena(sizes)
    for i, n in enumerate(sizes):
        m0 = synth.normal_f32(n, stream=98, block=i, purpose=0, step=0, sigma=0.02)
        g = synth.normal_bf16(n, stream=98, block=i, purpose=2, step=1, sigma=1e-3)
        for x in (a, b):
            x.put(i, "master", m0)
            x.put(i, "m", np.zeros(n, np.float32))
            x.put(i, "v", np.zeros(n, np.float32))
            x.put(i, "grad", g)
    before = a.buf.clone()
    ta, tb = a.table(), b.table()
    lib = lso._native.lib()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = lib.lso_adam_step_noalloc(ta.ptr, len(ta), torch.cuda.current_stream().cuda_stream)
        err = lso.last_error()
    torch.cuda.synchronize()
    assert st == lso._native.LSO_E_INVALID, st
    assert "capture" in err, err
    graph.replay()                                   # it captured nothing
    torch.cuda.synchronize()
    assert torch.equal(before, a.buf), "the refused call wrote something"
    # one call outside any capture, then the capture works
    lso.adam_step_noalloc(ta)
    lso.adam_step(tb)
    torch.cuda.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2):
        ta.set_step(2)
        lso.adam_step_noalloc(ta, torch.cuda.current_stream())
    graph2.replay()
    tb.set_step(2)
    lso.adam_step(tb)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        for q in ("master", "m", "v", "weight"):
            assert np.array_equal(a.get(i, q).view(np.uint8), b.get(i, q).view(np.uint8)), (i, q)
    print("capture rule ok", flush=True)


if __name__ == "__main__":
    main()
