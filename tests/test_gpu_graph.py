"""Library calls captured in a HIP graph (torch.cuda.graph) and replayed.

The library allocates nothing, never synchronises and records no memset, so
its calls can be captured; the split-K schedule's arrival counters are reset
by the kernel itself, so every replay starts from zeros.  Each replay runs on
new operands (copied into the captured input buffers), with eager library
calls and a synchronisation between replays, and must equal the eager result
on the same operands bit for bit (the kernels' summation order is fixed)."""
import sys

import numpy as np
import pytest
import torch

from workloads import make_f8_inputs, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_03_amd as t
    return t


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def test_graph_replays_match_eager(tdg):
    announce("graph capture and replay")
    dev = torch.device("cuda:0")
    # (layout, M, N, K, batch, in, out): a split-K problem (few tiles, long K),
    # a batched TN product and a small NN one
    probs = [("nn", 300, 520, 16384, 0, torch.float16, torch.float32),
             ("tn", 512, 512, 256, 4, torch.bfloat16, torch.float32),
             ("nn", 128, 256, 192, 0, torch.float16, torch.float32)]
    assert tdg.tdg_gemm_workspace_size(0, 300, 520, 16384, 1, 0) > 0, "the first problem should split K"
    sets = 4                                     # operand sets: eager reference for each
    inputs = []
    for p, (layout, M, N, K, batch, dt, odt) in enumerate(probs):
        per = []
        for s in range(sets):
            a, b = make_inputs(M, N, K, layout, "f16" if dt == torch.float16 else "bf16", "uniform",
                               seed=100 * p + s, batch=batch)
            per.append((a.to(dev), b.to(dev)))
        inputs.append(per)
    a8s, b8s = [], []
    for s in range(sets):
        a8, b8, _, _, _, _ = make_f8_inputs(256, 384, 512, dist="normal", seed=700 + s)
        a8s.append(torch.from_numpy(a8).to(dev).view(torch.float8_e4m3fn))
        b8s.append(torch.from_numpy(b8).to(dev).view(torch.float8_e4m3fn))

    # eager references
    ref = [[tdg.gemm(a, b, layout=probs[p][0], out_dtype=probs[p][6]) for (a, b) in inputs[p]]
           for p in range(len(probs))]
    ref8 = [tdg.gemm_f8(a8s[s], b8s[s], out_dtype=torch.bfloat16) for s in range(sets)]
    torch.cuda.synchronize()

    # captured buffers, filled with set 0; warm-up on the capture stream first
    # (the split-K workspace of that stream is allocated outside the capture)
    bufs = [(inputs[p][0][0].clone(), inputs[p][0][1].clone()) for p in range(len(probs))]
    outs = [torch.empty_like(ref[p][0]) for p in range(len(probs))]
    a8, b8 = a8s[0].clone(), b8s[0].clone()
    out8 = torch.empty_like(ref8[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def body():
        for p, (layout, *_rest) in enumerate(probs):
            tdg.gemm(bufs[p][0], bufs[p][1], layout=layout, out=outs[p])
        tdg.gemm_f8(a8, b8, out=out8)

    with torch.cuda.stream(s):
        body()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        body()
    torch.cuda.synchronize()

    for rep in range(sets):
        for p in range(len(probs)):
            bufs[p][0].copy_(inputs[p][rep][0])
            bufs[p][1].copy_(inputs[p][rep][1])
            outs[p].fill_(float("nan"))
        a8.copy_(a8s[rep])
        b8.copy_(b8s[rep])
        out8.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for p in range(len(probs)):
            assert torch.equal(outs[p], ref[p][rep]), "replay %d, problem %d" % (rep, p)
        assert torch.equal(out8, ref8[rep]), "replay %d, 8-bit product" % rep
        # eager work between replays, on the default stream
        x = tdg.gemm(inputs[0][(rep + 1) % sets][0], inputs[0][(rep + 1) % sets][1], layout="nn",
                     out_dtype=probs[0][6])
        torch.cuda.synchronize()
        assert torch.equal(x, ref[0][(rep + 1) % sets])
    assert np.isfinite(outs[0].float().cpu().numpy()).all()
