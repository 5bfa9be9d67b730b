"""The hot path inside a HIP graph.

A segmented, decayed prefill (segment pass, slot composition, full pass) followed by
a decode step that advances the prefill's end state in place is captured once and
replayed.  Every replay, with eager work and synchronizations between replays,
must give the eager result bit for bit: the kernels are deterministic and record no
memset, copy or allocation.  The entry point without allocation is captured the
same way (it is meant for callers that capture), and so is the chunk-parallel path.
"""
import pytest
import torch

from selective_state_space_hm_amd import hm, inputs

pytestmark = pytest.mark.gpu


def _case():
    c = inputs.make_prefill("graph", 2, 4, 700, 128, 64, 128, torch.bfloat16, None, "mamba", seed=31)
    g = {k: getattr(c, k).cuda() for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    gen = torch.Generator().manual_seed(32)
    B, H = c.B, c.H
    step = {
        "q": torch.randn((B, H, 128), generator=gen).to(torch.bfloat16).cuda(),
        "k": torch.randn((B, H, 128), generator=gen).to(torch.bfloat16).cuda(),
        "v": torch.randn((B, H, 128), generator=gen).to(torch.bfloat16).cuda(),
        "dt": torch.randn((B, H), generator=gen).cuda(),
    }
    return c, g, step


def _replays_match(run, outs, reps=3):
    """Eager run, capture, then `reps` replays each checked against the eager outputs."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(reps):
        for t in outs:  # eager work between replays: overwrite every output
            if t.is_floating_point():
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"replay {rep}, output {i}"
    print(f"[parity] graph: {reps} replays equal the eager run bit for bit", flush=True)


def test_prefill_and_decode_step_replay_in_a_graph():
    c, g, s = _case()
    B, H = c.B, c.H
    o = torch.empty_like(g["v"])
    state = torch.empty((B, H, hm.state_numel(64, 128)), dtype=torch.float32, device="cuda")
    o1 = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    plan = hm.hm_linattn_fwd_plan(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], segments=4)
    assert plan[1] == 4, plan

    def run():
        hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=state, o=o,
                          segments=4, workspace=ws)
        hm.hm_linattn_step(s["q"], s["k"], s["v"], g["w_q"], g["w_k"], state, s["dt"], g["a_log"], o=o1)

    _replays_match(run, [o, state, o1])


def test_noalloc_prefill_replays_in_a_graph():
    c, g, _ = _case()
    B, H = c.B, c.H
    o = torch.empty_like(g["v"])
    state = torch.empty((B, H, hm.state_numel(64, 128)), dtype=torch.float32, device="cuda")

    def run():
        hm.hm_linattn_fwd_noalloc(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_final=state,
                                  o=o)

    _replays_match(run, [o, state])


def test_chunk_parallel_prefill_replays_in_a_graph():
    """The chunk-parallel path (chunk 256: local states, their scan, outputs) with an
    initial state that the same buffer receives back as s_final, then a decode step
    on it; the replays must equal the eager run."""
    c, g, s = _case()
    B, H = c.B, c.H
    o = torch.empty_like(g["v"])
    gen = torch.Generator().manual_seed(33)
    s0 = (torch.rand((B, H, hm.state_numel(64, 128)), generator=gen) + 0.5).cuda()
    state = torch.empty_like(s0)
    o1 = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    assert hm.hm_linattn_fwd_plan(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], chunk=256)[0] == 256

    def run():
        torch.mul(s0, 1.0, out=state)  # the state starts from s0 at every replay (an element-wise kernel, no memcpy node)
        hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], s_init=state,
                          s_final=state, o=o, chunk=256, workspace=ws)
        hm.hm_linattn_step(s["q"], s["k"], s["v"], g["w_q"], g["w_k"], state, s["dt"], g["a_log"], o=o1)

    _replays_match(run, [o, state, o1])
