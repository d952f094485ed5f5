"""Run as a script by test_gpu_reentrancy.py, in a fresh process: the first
GEMV and skinny calls of the process come from 4 Python threads at once, each
on a stream of its own (the ctypes calls release the GIL, so the library's
host code runs concurrently), and each result is checked against the oracle.
Prints one line per thread and exits non-zero on any mismatch."""

import os
import sys
import threading

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import torch  # noqa: E402

import fp8_weight_only_fp4w_amd as fw  # noqa: E402
import workloads  # noqa: E402
from gpu_helpers import assert_parity, dev_to_bits, fp4_device, fp8_device, ref_fp4, ref_fp8  # noqa: E402


def main():
    assert torch.cuda.is_available()
    fw.load_library()
    # (kind, problem): two threads share one GEMV variant, the others take
    # the FP4 skinny kernel and the FP8 GEMV
    jobs = [
        ("fp4", workloads.make_fp4(4, 1000, 1024, 16, "bf16", seed=31, with_bias=True)),
        ("fp4", workloads.make_fp4(4, 1000, 1024, 16, "bf16", seed=32, with_bias=True)),
        ("fp4", workloads.make_fp4(24, 800, 512, 16, "fp16", seed=33, with_bias=True)),
        ("fp8", workloads.make_fp8(3, 600, 1024, 128, "bf16", seed=34, with_bias=False)),
    ]
    devs = [fp4_device(p) if k == "fp4" else fp8_device(p) for k, p in jobs]
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    start = threading.Barrier(len(jobs))
    out = [None] * len(jobs)
    err = [None] * len(jobs)

    def run(i):
        try:
            kind, p = jobs[i]
            d = devs[i]
            with torch.cuda.stream(streams[i]):
                start.wait()
                if kind == "fp4":
                    Y = fw.fp4w_matmul(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], 16)
                else:
                    Y = fw.fp8w_matmul(d["A"], d["B"], d["bs"], d["bias"], 128)
                streams[i].synchronize()
                out[i] = dev_to_bits(Y)
        except Exception as e:  # noqa: BLE001 - reported by the main thread
            err[i] = e

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    ok = True
    for i, (kind, p) in enumerate(jobs):
        if err[i] is not None:
            print(f"thread {i} {kind} M={p.M}: error {err[i]!r}", flush=True)
            ok = False
            continue
        Y_ref, S = ref_fp4(p) if kind == "fp4" else ref_fp8(p)
        try:
            assert_parity(out[i], p.dtype, Y_ref, S, f"thread {i}")
            print(f"thread {i} {kind} M={p.M} N={p.N} K={p.K}: ok", flush=True)
        except AssertionError as e:
            print(f"thread {i} {kind}: {e}", flush=True)
            ok = False
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
