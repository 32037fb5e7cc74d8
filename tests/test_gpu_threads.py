"""Concurrent calls from several host threads, each on its own stream, give the
results of the same calls made one at a time (bitwise: the kernels use no
atomics and no shared state)."""
import threading

import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I

from gpu_util import run_case

pytestmark = pytest.mark.gpu


def test_threads_on_separate_streams_match_serial():
    cases = [I.make_case(f"thr{i}", 2, 8, 384 + 64 * i, 64, I.BF16, i % 2 == 0, 300 + i) for i in range(4)]
    serial = [run_case(c, fa.FA_PREC_BF16) for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    results = [None] * len(cases)
    errors = []

    def work(i):
        try:
            # allocation, upload and launches all on this thread's stream
            with torch.cuda.stream(streams[i]):
                results[i] = run_case(cases[i], fa.FA_PREC_BF16, stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (a, b) in enumerate(zip(serial, results)):
        for n in a:
            assert torch.equal(a[n], b[n]), (i, n)
