"""The prolog captured into a HIP graph (through torch.cuda.CUDAGraph) and replayed.

mlap_run only enqueues kernels on the caller's stream, so a bound run can be captured.
Each replay must reproduce the eager run bit for bit; replays are separated by other
eager GPU work and host synchronisations, and the outputs are cleared before each
replay so a replay that does nothing cannot pass."""
import pytest
import torch

import mla_prolog_amd as mlap
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _diff(a, b):
    """Where two equal-shaped tensors differ: count and the first few indexes and values."""
    ne = (a != b).nonzero()
    first = [(tuple(i.tolist()), a[tuple(i)].item(), b[tuple(i)].item()) for i in ne[:6]]
    rows = sorted(set(ne[:, 0].tolist()))
    return {"count": int(ne.shape[0]), "rows": rows[:12], "n_rows": len(rows), "first": first}


# v3_w8a8 at T=2048 adds the activation quant and the int8 tiles with their dequantisation;
# the MXFP8 cases add the weight decode / activation conversion launches of both routes; the
# V4 shape its head norm spread over several workgroups per token
@pytest.mark.parametrize("name,T,var", [("v3_decode", 64, {}), ("v3_decode", 256, {}),
                                        ("v2lite_kv_decode", None, {}), ("v3_prefill", 1000, {}),
                                        ("v3_w8a8", 2048, {}), ("v3_mxfp8", 300, {}),
                                        ("v3_mxfp8", 1000, {"mxfp8_mfma": True}),
                                        ("v4_decode", None, {}), ("v4_decode", 64, {"q_quant_per_head": True})])
def test_graph_replay_matches_eager(name, T, var):
    cfg = synth.get_config(name, T=T, **var)
    say("graph replay", name, "T=%d" % cfg.T)
    inp = {k: v.cuda() for k, v in synth.make_inputs(cfg).items()}
    other = {k: v.cuda() for k, v in synth.make_inputs(cfg, seed=synth.seed_for(cfg) + 7).items()}
    p = mlap.Prolog.from_config(cfg)
    ref = {k: v.clone() for k, v in p.run(inp).items()}
    outs = p.alloc_outputs(cfg.T)
    ws = torch.empty(p.workspace_size(cfg.T), dtype=torch.uint8, device="cuda")
    side_outs = p.alloc_outputs(cfg.T)
    side_ws = torch.empty_like(ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bound = p.bind(inp, outputs=outs, workspace=ws)  # binds the capture stream
        bound()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        # unrelated eager work between replays, on the same buffers' neighbours
        p.run(other, outputs=side_outs, workspace=side_ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = {k: _diff(outs[k], v) for k, v in ref.items() if not torch.equal(outs[k], v)}
        assert not bad, "replay %d differs from the eager run: %s" % (rep, bad)
    say("  3 replays bit-identical to eager")
