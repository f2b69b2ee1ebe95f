"""Library calls in flight at the same time: on two streams of one device,
issued from two host threads.  Each stream has its own split-K workspace
(the Python binding keys workspaces by device and stream), so split-K
products overlapping on the two streams must not disturb each other; each
result must equal the same call made alone, bit for bit."""
import sys
import threading

import pytest
import torch

from workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_03_amd as t
    return t


def test_two_streams_two_threads(tdg):
    print("CASE two streams, two threads", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda:0")
    # split-K shapes (few 128 x 128 tiles, long K) and a plain one
    shapes = [("nn", 300, 520, 16384, torch.float32), ("tn", 257, 264, 16384, torch.bfloat16),
              ("nn", 1024, 2048, 512, torch.float16)]
    assert tdg.tdg_gemm_workspace_size(0, 300, 520, 16384, 1, 0) > 0
    work = []
    for t in range(2):
        per = []
        for i, (layout, M, N, K, odt) in enumerate(shapes * 2):
            a, b = make_inputs(M, N, K, layout, "bf16" if odt == torch.bfloat16 else "f16", "uniform",
                               seed=1000 * t + i)
            per.append((layout, a.to(dev), b.to(dev), odt))
        work.append(per)
    ref = [[tdg.gemm(a, b, layout=layout, out_dtype=odt) for (layout, a, b, odt) in per] for per in work]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * len(work[0]) for _ in range(2)]
    errors = []

    def run(t):
        try:
            with torch.cuda.stream(streams[t]):
                for rep in range(3):
                    for i, (layout, a, b, odt) in enumerate(work[t]):
                        outs[t][i] = tdg.gemm(a, b, layout=layout, out_dtype=odt)
        except Exception as e:                  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for i in range(len(work[t])):
            assert torch.equal(outs[t][i], ref[t][i]), "stream %d, call %d" % (t, i)
