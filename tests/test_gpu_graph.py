"""HIP-graph capture of the library's calls (GPU).

Callers replay decode steps and whole prefills from captured graphs to drop the host
launch cost.  Each test captures the calls on torch's capture stream, replays the graph
several times with eager work and synchronisations between the replays (a state reset,
a copy), and checks every replay bit for bit against the same calls made eagerly: the
kernels are deterministic, so a replay must reproduce the eager result exactly.
"""
import pytest
import torch

import gated_delta_rule_70_amd as gdr
from gpu_util import dev, note, small_inputs

pytestmark = pytest.mark.gpu


def test_decode_steps_replayed_from_a_graph():
    B, HK, HV, dk, dv, nstep = 4, 2, 4, 64, 64, 6
    x = dev(small_inputs(B, nstep, HK, HV, dk, dv, seed=71))
    step = [{n: x[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")} for t in range(nstep)]
    note(f"graph decode B={B} HV={HV} {dk}x{dv} steps={nstep}")

    eager = x["h0"].clone()
    o_eager = []
    for t in range(nstep):
        o = torch.empty(B, 1, HV, dv, device="cuda")
        gdr.decode_step(step[t]["q"], step[t]["k"], step[t]["v"], step[t]["g"], step[t]["beta"], eager,
                        o=o, out_state=eager)
        o_eager.append(o)
    torch.cuda.synchronize()

    state = x["h0"].clone()
    outs = [torch.empty(B, 1, HV, dv, device="cuda") for _ in range(nstep)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(nstep):
            gdr.decode_step(step[t]["q"], step[t]["k"], step[t]["v"], step[t]["g"], step[t]["beta"], state,
                            o=outs[t], out_state=state)
    for rep in range(3):
        state.copy_(x["h0"])          # eager work between replays
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, eager), f"replay {rep}: state differs"
        for t in range(nstep):
            assert torch.equal(outs[t], o_eager[t]), f"replay {rep}: o of step {t} differs"


# (B, T, HK, HV, dk, chunk): column-split carry; whole-head carry (> 128 heads); the
# segmented carry (summary, combine and full launches; 2 heads x 2048 chunks, 128 segments)
GRAPH_PREFILLS = [(2, 97, 2, 4, 128, 64), (2, 200, 2, 4, 128, 64), (2, 97, 40, 80, 64, 32),
                  (1, 32768, 1, 2, 64, 16)]


@pytest.mark.parametrize("case", GRAPH_PREFILLS, ids=lambda c: "B{}T{}HV{}dk{}C{}".format(c[0], c[1], c[3], c[4], c[5]))
def test_prefill_replayed_from_a_graph(case):
    B, T, HK, HV, dk, C = case
    dv = dk
    x = dev(small_inputs(B, T, HK, HV, dk, dv, seed=72))
    note(f"graph prefill B={B} T={T} HV={HV} {dk}x{dv} C={C}")
    ws = torch.empty(gdr.workspace_bytes(B, T, HK, HV, dk, dv, C), dtype=torch.uint8, device="cuda")

    def call(o, ht):
        gdr.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"], chunk=C, o=o, ht=ht,
                          workspace=ws)

    o_e = torch.empty(B, T, HV, dv, device="cuda")
    ht_e = torch.empty(B, HV, dk, dv, device="cuda")
    call(o_e, ht_e)
    torch.cuda.synchronize()

    o = torch.empty_like(o_e)
    ht = torch.empty_like(ht_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o, ht)
    for rep in range(3):
        o.fill_(float("nan"))          # eager work between replays
        ht.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), f"replay {rep}: o differs"
        assert torch.equal(ht, ht_e), f"replay {rep}: final state differs"


def test_fused_recurrence_and_tree_verify_replayed_from_a_graph():
    from gdr_synth import make_tree

    B, T, HK, HV, dk, dv = 2, 12, 2, 4, 128, 64
    x = dev(small_inputs(B, T, HK, HV, dk, dv, seed=73))
    par = make_tree(B, T, "random", seed=5).cuda()
    note(f"graph fused recurrence + tree verify B={B} T={T}")
    o_r, ht_r = gdr.fused_recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    o_t = gdr.tree_verify(x["q"], x["k"], x["v"], x["g"], x["beta"], par, h0=x["h0"])
    torch.cuda.synchronize()

    o1 = torch.empty_like(o_r)
    ht1 = torch.empty_like(ht_r)
    o2 = torch.empty_like(o_t)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdr.fused_recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"], o=o1, ht=ht1)
        gdr.tree_verify(x["q"], x["k"], x["v"], x["g"], x["beta"], par, h0=x["h0"], o=o2)
    for rep in range(3):
        for t in (o1, ht1, o2):
            t.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, o_r) and torch.equal(ht1, ht_r), f"replay {rep}: fused recurrence differs"
        assert torch.equal(o2, o_t), f"replay {rep}: tree verify differs"
