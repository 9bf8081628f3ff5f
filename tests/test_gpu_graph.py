"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: every replay equals the eager result bit for bit, with eager calls
on other inputs and host synchronisations between the replays. The library's
entry points launch kernels only (no memset, allocation or synchronisation),
so a caller may capture them."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import bit_block_quantized_rocmfp2_amd as qm  # noqa: E402
from synth import gen  # noqa: E402


def test_graph_replay_decode():
    spec = gen.LayerSpec(hidden=1024, inter=512, n_experts=32, topk=6, rot_down=1)
    dl = qm.device.DeviceLayer(spec, seed=21)
    ws = dl.workspace(4)
    xs = [torch.from_numpy(gen.tokens(q, spec.hidden, seed=210 + i, stream=q)).cuda()
          for i, q in enumerate([1, 1, 4, 2, 1])]
    outs = [torch.empty_like(x) for x in xs]
    # eager reference
    ref = []
    for x, o in zip(xs, outs):
        qm.qmoe_decode_layer(dl.desc, x, o, ws)
        torch.cuda.synchronize()
        ref.append(o.cpu().numpy().copy())
    other = torch.from_numpy(gen.tokens(4, spec.hidden, seed=299, stream=4)).cuda()
    other_out = torch.empty_like(other)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):     # warm-up on the capture stream
        for x, o in zip(xs, outs):
            qm.qmoe_decode_layer(dl.desc, x, o, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, o in zip(xs, outs):
            qm.qmoe_decode_layer(dl.desc, x, o, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(o.cpu().numpy(), ref[i]), (rep, i)
        qm.qmoe_decode_layer(dl.desc, other, other_out, ws)   # eager work on the same workspace
        torch.cuda.synchronize()
