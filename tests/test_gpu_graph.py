"""A shared round captured as one HIP graph (the table upload and every
launch of the library on the capture stream) gives, replay after replay,
the bits of the same round run eagerly. Each replay starts from the same
conv states (restored outside the graph), with eager work of the program
and synchronisations between the replays."""

import numpy as np
import pytest
import torch

import attention_stream_verify_amd as asv
import workloads

pytestmark = pytest.mark.gpu


def _u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("streams", [
    None,                                               # the tiny round
    [(16, 20000, 20000), (8, 9000, 9024), (1, 3000, 3008)],   # 16-row tiles with two split sizes
])
def test_graph_replays_equal_the_eager_round(streams):
    rnd = workloads.Round(0, device="cuda", streams=streams, n_conv=1, n_attn=1)
    X, W, states = rnd.conv[0]
    Q, ks, vs = rnd.attn[0]
    rb = asv.RoundBuffers(rnd.streams, [states], [ks], [vs], device="cuda", vocab=rnd.logits.shape[1])
    saved = [s.clone() for s in states]

    def restore():
        for s, v in zip(states, saved):
            s.copy_(v)

    def round_():
        rb.upload()
        rb.conv(0, X, W)
        rb.attn(0, Q)
        rb.merge()
        rb.argmax(rnd.logits)
        rb.draft()

    def outputs():
        torch.cuda.synchronize()
        return [_u16(rb.y), _u16(rb.o), rb.pick.cpu().numpy(), rb.flag.cpu().numpy(), rb.ids.cpu().numpy(),
                rb.fail.cpu().numpy()] + [_u16(s) for s in states]

    round_()
    want = outputs()
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    for rep in range(4):
        restore()
        rb.y.zero_()
        rb.o.zero_()
        rb.pick.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        got = outputs()
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {rep}"
        round_()                                   # eager work between replays
        torch.cuda.synchronize()
