"""qgemv_time_next_launch on the GPU: the armed launch records the caller's
events around its own kernel, the setting is used by exactly one launch,
disarming leaves the events alone, and a timed launch computes the same
bits as an untimed one."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, host, quantize, say

pytestmark = pytest.mark.gpu

FENCE_OFF = 0x20000000  # hipEventDisableSystemFence


class Events:
    """Raw hipEvent_t handles (the library takes them as plain pointers)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p] * 3
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), FENCE_OFF) == 0
            self.ev.append(e)

    def record(self, i):
        sh = torch.cuda.current_stream().cuda_stream
        assert self.hip.hipEventRecord(self.ev[i], sh) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(self.ev[b]) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


@pytest.fixture(scope="module")
def problem(qg):
    """A Q4_K product large enough to take tens of microseconds, and a small
    one (same K) that takes a few."""
    g = np.random.default_rng(4242)
    K = 4096
    big, small = 65536, 64
    w = synth.q4_k_weights(g, big, K)
    act = quantize(qg, synth.activation(g, 1, K)[0])
    wd = dev(w)
    rb = synth.row_bytes("q4_k", K)
    return wd, wd.view(big, rb)[:small].reshape(-1), big, small, K, act


def run(qg, w, N, K, act):
    q, d, s = act
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda:0")
    qg.qgemv_q4_k(w, N, K, q, d, s, y)
    return y


def test_timed_launch_is_the_kernel_and_same_bits(qg, problem):
    w, _, N, _, K, act = problem
    say("time_next_launch kernel vs bracket", N, K)
    y0 = host(run(qg, w, N, K, act))
    ev = Events(4)
    try:
        for _ in range(3):
            ev.record(0)
            qg.qgemv_time_next_launch(ev.ev[2], ev.ev[3])
            y1 = run(qg, w, N, K, act)
            ev.record(1)
            kernel, bracket = ev.ms(2, 3), ev.ms(0, 1)
            assert 0.0 < kernel <= bracket + 1e-3, (kernel, bracket)
            assert np.array_equal(host(y1).view(np.uint32), y0.view(np.uint32))
    finally:
        torch.cuda.synchronize()
        ev.close()


def test_setting_is_used_by_one_launch(qg, problem):
    w, w_small, N, n_small, K, act = problem
    say("time_next_launch consumed by one launch", n_small, N, K)
    ev = Events(4)
    try:
        # the small product alone, then the big one alone, both timed
        qg.qgemv_time_next_launch(ev.ev[0], ev.ev[1])
        run(qg, w_small, n_small, K, act)
        qg.qgemv_time_next_launch(ev.ev[2], ev.ev[3])
        run(qg, w, N, K, act)
        small_ms, big_ms = ev.ms(0, 1), ev.ms(2, 3)
        assert small_ms < 0.5 * big_ms, (small_ms, big_ms)
        # armed once, then two launches: the events keep the first (small) one
        qg.qgemv_time_next_launch(ev.ev[0], ev.ev[1])
        run(qg, w_small, n_small, K, act)
        run(qg, w, N, K, act)
        again = ev.ms(0, 1)
        assert again < 0.5 * big_ms, (again, small_ms, big_ms)
    finally:
        torch.cuda.synchronize()
        ev.close()


def test_disarm_leaves_events_alone(qg, problem):
    w, _, N, _, K, act = problem
    say("time_next_launch disarmed", N, K)
    ev = Events(3)
    try:
        ev.record(0)
        ev.record(1)
        torch.cuda.synchronize()
        qg.qgemv_time_next_launch(ev.ev[0], ev.ev[1])
        qg.qgemv_time_next_launch(None, None)
        run(qg, w, N, K, act)
        ev.record(2)
        # neither event moved to the launch: they still lie before it
        assert ev.ms(0, 1) <= ev.ms(0, 2)
        assert abs(ev.ms(0, 1)) < 0.01
    finally:
        torch.cuda.synchronize()
        ev.close()
