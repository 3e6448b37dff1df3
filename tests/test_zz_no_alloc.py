"""attn_decode_paged_noalloc (library-owned static scratch, no workspace argument) against attn_decode_paged on the
same inputs: bitwise equal outputs and lse, on two calls in a row with the second one smaller (the scratch keeps
the first call's partials, which must not leak into the second), at head dims 128 and 64, and at the largest
sequence length the scratch admits for the paged-decode workload's batch and heads."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, paged_decode_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check_bf16

pytestmark = pytest.mark.gpu


def both(ta, w, inp):
    q = dev_bf16(inp["q"])
    ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table, lens = dev(inp["block_table"]), dev(inp["seq_lens"])
    o1, l1 = ta.attn_decode_paged(q, kc, vc, table, lens, inp["max_len"], softmax_scale=w.scale, return_lse=True)
    o2, l2 = ta.attn_decode_paged_noalloc(q, kc, vc, table, lens, inp["max_len"], softmax_scale=w.scale,
                                          return_lse=True)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2), q


@pytest.mark.parametrize("d", [128, 64])
def test_noalloc_equals_workspace_decode_twice(d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    lens = np.random.default_rng(90).integers(1024, 9000, size=16, endpoint=True)
    big = paged_decode_inputs(w, seed=91, seq_lens=lens, max_len=9000)
    small = paged_decode_inputs(w, seed=92, seq_lens=[1, 300, 2047, 5], max_len=2048)
    for name, inp in (("first, larger", big), ("second, smaller", small)):
        say(f"noalloc d={d} {name}: lens {inp['seq_lens'].tolist()}")
        (o1, l1), (o2, l2), q = both(ta, w, inp)
        assert torch.equal(o1, o2), name
        assert torch.equal(l1, l2), name
    # the second (small) result is also right against the oracle
    qr = oracle.rope(bits_to_f32(small["q"])[:, None], small["positions"][:, None], w.theta)[:, 0]
    o_ref, _ = oracle.decode_paged(qr, bits_to_f32(small["k_cache"]), bits_to_f32(small["v_cache"]),
                                   small["block_table"], small["seq_lens"], w.scale)
    check_bf16("noalloc o (second call)", host_bf16(o2), o_ref)


def test_noalloc_at_the_scratch_limit():
    """64 sequences x 32 query heads x 128 dims with max_seqlen_kv 64512: the largest request the 64 MiB scratch
    serves (a few sequences are that long, the rest short)."""
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    lens = [64512, 64000, 1] + [100 + 37 * i for i in range(61)]
    inp = paged_decode_inputs(w, seed=93, seq_lens=lens, max_len=64512)
    assert ta.attn_decode_paged_workspace_size(64, 32, 128, 64512) <= ta.DECODE_SCRATCH_BYTES
    say("noalloc at the scratch limit")
    (o1, l1), (o2, l2), _ = both(ta, w, inp)
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
