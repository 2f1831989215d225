"""The library called from several host threads at once.

Two threads, each with its own stream and its own stream-K workspace, run a
dense training step of their own (the paired forward-operand quantizer, the
grad_out quantizer, forward, dgrad and the stream-K wgrad) several times while
the other does the same; every output must equal, byte for byte, what the
same calls wrote when run one after the other on one stream.  ctypes releases
the interpreter lock during each call, so the threads are inside the library
together (validation, the launch-size cache, the launches).
"""

import threading

import pytest
import torch

import blockwise_scaled_fp8_bs_amd as bs
from blockwise_scaled_fp8_bs_amd import inputs
from gpu_support import need_gpu

pytestmark = pytest.mark.gpu

REPEATS = 4


class DenseStep:
    """Buffers and calls of one dense training step, wgrad through its own workspace."""

    def __init__(self, M, K, N, seed):
        dev = "cuda"
        u8, f32 = torch.uint8, torch.float32
        r4 = lambda n: (n + 3) // 4 * 4  # noqa: E731
        self.x = inputs.bf16_normal((M, K), 1.0, seed, device=dev)
        self.w = inputs.bf16_normal((N, K), 0.02, seed + 1, device=dev)
        self.dy = inputs.bf16_normal((M, N), 0.01, seed + 2, device=dev)
        self.out = {
            "qx": torch.empty((M, K), dtype=u8, device=dev), "sx": torch.empty((K // 128, r4(M)), dtype=f32, device=dev),
            "qxt": torch.empty((K, M), dtype=u8, device=dev), "sxt": torch.empty((M // 128, r4(K)), dtype=f32, device=dev),
            "qw": torch.empty((N, K), dtype=u8, device=dev), "sw": torch.empty((K // 128, r4(N // 128)), dtype=f32, device=dev),
            "qwt": torch.empty((K, N), dtype=u8, device=dev), "swt": torch.empty((N // 128, r4(K // 128)), dtype=f32, device=dev),
            "qg": torch.empty((M, N), dtype=u8, device=dev), "sg": torch.empty((N // 128, r4(M)), dtype=f32, device=dev),
            "qgt": torch.empty((N, M), dtype=u8, device=dev), "sgt": torch.empty((M // 128, r4(N)), dtype=f32, device=dev),
            "y": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            "dx": torch.empty((M, K), dtype=torch.bfloat16, device=dev),
            "dw": torch.empty((N, K), dtype=torch.bfloat16, device=dev),
        }
        nbytes = bs.bs_scaled_mm_workspace_bytes(N, K, M, bs.BS_SCALE_1X128)
        self.ws = torch.empty(max(nbytes, 256), dtype=u8, device=dev)

    def run(self):
        o = self.out
        bs.bs_quant_fwd_operands(self.x, o["qx"], o["sx"], o["qxt"], o["sxt"], self.w, o["qw"], o["sw"],
                                 o["qwt"][None], o["swt"][None])
        bs.bs_scaled_mm(o["qx"], o["sx"], o["qw"], o["sw"], bs.BS_SCALE_128X128, out=o["y"])
        bs.bs_quant_1x128(self.dy, o["qg"], o["sg"], o["qgt"], o["sgt"])
        bs.bs_scaled_mm(o["qg"], o["sg"], o["qwt"], o["swt"], bs.BS_SCALE_128X128, out=o["dx"])
        bs.bs_scaled_mm_ws(o["qgt"], o["sgt"], o["qxt"], o["sxt"], bs.BS_SCALE_1X128, workspace=self.ws,
                           out=o["dw"])

    def snapshot(self):
        return {k: t.view(torch.uint8).clone() for k, t in self.out.items()}


def test_two_threads_match_serial():
    need_gpu()
    steps = [DenseStep(1280, 640, 768, seed=21), DenseStep(1152, 896, 512, seed=31)]

    def poison():  # scale padding is never written: it keeps this pattern in both runs
        for s in steps:
            for t in s.out.values():
                t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()

    poison()
    for s in steps:
        s.run()
    torch.cuda.synchronize()
    ref = [s.snapshot() for s in steps]
    poison()

    errors = []
    start = threading.Barrier(len(steps))

    def worker(step):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                start.wait()
                for _ in range(REPEATS):
                    step.run()
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(s,)) for s in steps]
    print(f"threads: {len(threads)}, {REPEATS} steps each", flush=True)
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, s in enumerate(steps):
        got = s.snapshot()
        for k in ref[i]:
            bad = int((got[k] != ref[i][k]).sum())
            assert bad == 0, f"step {i}: {k} differs from the serial run in {bad} bytes"
