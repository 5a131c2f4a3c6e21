"""Child process of the crash test (run by tests/test_gpu_shadow.py, not
collected by pytest): one step over shadow files whose gradient producer,
at layer K, waits until the device is idle and then kills its own process
with SIGKILL, while the write-backs of earlier layers may be in flight.

    python shadow_crash_child.py DIR K STREAM_ID
"""
import ctypes
import os
import signal
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import layer_streamed_optimizer_amd as lso  # noqa: E402
import synth  # noqa: E402
from layer_streamed_optimizer_amd import configs  # noqa: E402
from layer_streamed_optimizer_amd.disk import LayerFiles  # noqa: E402


def main(directory: str, kill_at: int, sid: int) -> int:
    files = LayerFiles.open(directory)
    hip = ctypes.CDLL("libamdhip64.so")
    fill = synth._dev_lib().synth_fill_normal_bf16

    def producer(layer, dev_grad, n, stream):
        if layer == kill_at:
            # every kernel and copy enqueued so far finishes first; only
            # host-side file writes can still be running
            assert hip.hipDeviceSynchronize() == 0
            print(f"killing the process at layer {layer}", flush=True)
            time.sleep(0.01)
            os.kill(os.getpid(), signal.SIGKILL)
        return fill(dev_grad, n, 0, synth.SEED, sid, layer, synth.PURPOSE_GRAD, 1,
                    synth.scale_for(1e-3), stream)

    ls = lso.LayerStream(files.bytes(0), files.sizes[0], producer)
    ls.stream_files(files.table(1, configs.LR, configs.BETA1, configs.BETA2, configs.EPS))
    print("the step finished without being killed", flush=True)
    return 3


if __name__ == "__main__":
    sys.exit(main(sys.argv[1], int(sys.argv[2]), int(sys.argv[3])))
