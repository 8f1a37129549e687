"""Entry points called from several host threads at once.

The library keeps no per-device state filled on first use, so concurrent
first launches from different threads (each on its own stream) must give the
same results as the same launches made one after the other.  ctypes releases
the interpreter lock for the duration of each foreign call, so the threads'
calls into the library do overlap.
"""
import threading

import pytest
import torch

from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d

from parity_util import note

pytestmark = pytest.mark.gpu

PROBLEMS = [I.Problem(4, 2, 56, 56, 32, 7, 1, "bf16"),    # general kernel
            I.Problem(4, 2, 56, 56, 32, 7, 8, "bf16"),    # whole-class kernel
            I.Problem(2, 3, 40, 37, 32, 5, 2, "f16"),
            I.Problem(1, 2, 20, 21, 32, 3, 1, "f32")]     # per-lane kernel


def test_concurrent_forward_from_host_threads():
    note("forward from %d host threads" % len(PROBLEMS))
    ins = []
    for i, p in enumerate(PROBLEMS):
        q, k, v, rpb = (t.cuda() for t in I.make_inputs(p, seed=10 + i))
        ins.append((p, q, k, v, rpb))
    torch.cuda.synchronize()
    results = [None] * len(ins)
    errors = []
    start = threading.Barrier(len(ins))

    def work(i):
        p, q, k, v, rpb = ins[i]
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                outs = [na2d.forward(q, k, v, rpb, p.kernel_size, p.dilation) for _ in range(4)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(ins))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for (p, q, k, v, rpb), outs in zip(ins, results):
        ref = na2d.forward(q, k, v, rpb, p.kernel_size, p.dilation)
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, ref), p.describe()
