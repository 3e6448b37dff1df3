"""The DSA decode step (indexer, top-k, sparse MLA) captured once as a HIP graph and replayed, as a serving loop
would run a launch-bound decode step: every replay, with eager work on other inputs between the replays, gives
the eager step's outputs bit for bit (the kernels are deterministic and take all inputs by pointer). The eager step
itself is checked against the oracle in the DSA tests."""
import dataclasses

import numpy as np
import pytest
import torch

from synth import WORKLOADS, dsa_inputs
from gpu_util import require_gpu, say, dev, dev_bf16

pytestmark = pytest.mark.gpu


def make_step(ta, w, inp):
    """Device inputs and outputs of one DSA decode step, and a function that enqueues the step on the current
    stream (no allocation, no synchronisation)."""
    t = {n: dev_bf16(inp[n]) for n in ("q_idx", "k_idx", "q_lat", "q_pe", "c_kv", "k_pe")}
    t["w_idx"], t["lens"] = dev(inp["w_idx"]), dev(inp["seq_lens"])
    b, heads = inp["q_lat"].shape[:2]
    t["scores"] = torch.empty((b, inp["k_idx"].shape[1]), dtype=torch.float32, device="cuda")
    t["idx"] = torch.empty((b, w.topk), dtype=torch.int32, device="cuda")
    t["o"] = torch.empty_like(t["q_lat"])
    t["lse"] = torch.empty((b, heads), dtype=torch.float32, device="cuda")
    t["ws"] = torch.empty(ta.attn_mla_sparse_decode_workspace_size(b, heads, w.latent, w.topk), dtype=torch.uint8,
                          device="cuda")

    def step():
        ta.attn_dsa_indexer(t["q_idx"], t["w_idx"], t["k_idx"], t["lens"], scores=t["scores"])
        ta.attn_topk(t["scores"], t["lens"], w.topk, indices=t["idx"])
        ta.attn_mla_sparse_decode(t["q_lat"], t["q_pe"], t["c_kv"], t["k_pe"], t["lens"], t["idx"], w.scale,
                                  o=t["o"], lse=t["lse"], workspace=t["ws"])
    return t, step


def outputs(t):
    return [t[n].cpu().clone() for n in ("scores", "idx", "o", "lse")]


@pytest.mark.parametrize("batch,seqlen,lens", [(4, 3000, [3000, 2500, 700, 1]), (32, 32768, None)])
def test_dsa_step_graph_replays_match_eager(batch, seqlen, lens):
    ta = require_gpu()
    w = WORKLOADS["dsa_decode_b32"]
    say(f"dsa step graph B={batch} T={seqlen}")
    t, step = make_step(ta, w, dsa_inputs(w, seed=7, batch=batch, seqlen=seqlen, seq_lens=lens))
    step()
    torch.cuda.synchronize()
    eager = outputs(t)
    # other inputs, run eagerly between the replays
    w2 = dataclasses.replace(w)
    t2, step2 = make_step(ta, w2, dsa_inputs(w2, seed=8, batch=2, seqlen=1000, seq_lens=[1000, 333]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for n in ("scores", "idx", "o", "lse"):
        t[n].zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for n in ("scores", "idx", "o", "lse"):
            t[n].zero_()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(t)
        for name, a, b in zip(("scores", "idx", "o", "lse"), got, eager):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager step"
        step2()
        torch.cuda.synchronize()
