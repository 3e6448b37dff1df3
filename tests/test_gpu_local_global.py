"""attn_prefill_local_global on the GPU against the fp64 oracle: sliding windows, leading global tokens and periodic
anchors (alone and combined), the degenerate cases (window 1, window >= S, anchor stride 1), bit-identity with the
plain causal kernel when the window covers the sequence, and sampled rows of the 131072-token workload."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, prefill_inputs, sampled_rows
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu


def rotated(ta, w, inp):
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    pos = dev(inp["positions"])
    ta.attn_rope_apply(q, pos, w.theta)
    ta.attn_rope_apply(k, pos, w.theta)
    return q, k, v


def oracle_inputs(w, inp):
    s_len = inp["q"].shape[1]
    pos = np.broadcast_to(np.arange(s_len), inp["q"].shape[:2])
    return (oracle.rope(bits_to_f32(inp["q"]), pos, w.theta), oracle.rope(bits_to_f32(inp["k"]), pos, w.theta),
            bits_to_f32(inp["v"]))


CASES = [  # (window, n_lead, anchor_stride)
    (64, 0, 0), (100, 5, 0), (128, 0, 32), (50, 3, 7), (200, 64, 100), (1, 0, 0), (16, 0, 1), (5000, 0, 0),
    (65, 130, 0), (33, 0, 200),
]


@pytest.mark.parametrize("hq,hkv,d,s_len", [(32, 8, 128, 300), (16, 16, 64, 517), (12, 4, 128, 1000)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_local_global_small(hq, hkv, d, s_len, case):
    ta = require_gpu()
    W, G, P = CASES[case]
    w = dataclasses.replace(WORKLOADS["swa_prefill_s131072"], batch=2, seqlen=s_len, hq=hq, hkv=hkv, head_dim=d,
                            window=W, n_lead=G, anchor_stride=P, scale=1.0 / np.sqrt(d))
    say(f"local+global hq={hq} hkv={hkv} d={d} S={s_len} window={W} lead={G} stride={P}")
    inp = prefill_inputs(w, seed=95 + case)
    q, k, v = rotated(ta, w, inp)
    o, lse = ta.attn_prefill_local_global(q, k, v, W, G, P, softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_local_global(*oracle_inputs(w, inp), W, G, P, w.scale)
    check_bf16("o", host_bf16(o), o_ref)
    check("lse", lse.cpu().numpy(), lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("s_len,hq,hkv,d", [(777, 32, 8, 128), (300, 8, 8, 64)])
def test_full_window_is_bit_identical_to_causal(s_len, hq, hkv, d):
    """A window covering the sequence visits the causal kernel's tiles in its order with the same masks."""
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["swa_prefill_s131072"], batch=2, seqlen=s_len, hq=hq, hkv=hkv, head_dim=d,
                            scale=1.0 / np.sqrt(d))
    inp = prefill_inputs(w, seed=99)
    q, k, v = rotated(ta, w, inp)
    o1, l1 = ta.attn_prefill_local_global(q, k, v, s_len, 0, 0, softmax_scale=w.scale, return_lse=True)
    o2, l2 = ta.attn_prefill(q, k, v, causal=True, softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(o1), host_bf16(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_full_size_sampled_rows():
    """The benchmark workload (S=131072, window 4096, anchors every 32 tokens) in the bench's launch configuration,
    checked on 64 seeded rows (including the first and the last) for every head."""
    ta = require_gpu()
    w = WORKLOADS["swa_prefill_s131072"]
    say(f"local+global full size S={w.seqlen} window={w.window} stride={w.anchor_stride}")
    inp = prefill_inputs(w, seed=0)
    q, k, v = rotated(ta, w, inp)
    o, lse = ta.attn_prefill_local_global(q, k, v, w.window, w.n_lead, w.anchor_stride, softmax_scale=w.scale,
                                         return_lse=True)
    torch.cuda.synchronize()
    rows = sampled_rows(w.seqlen, 64, seed=3)
    o = host_bf16(o)[:, rows]
    lse = lse.cpu().numpy()[:, :, rows]
    pos = np.broadcast_to(np.arange(w.seqlen), (w.batch, w.seqlen))
    qr = np.zeros((w.batch, w.seqlen, w.hq, w.head_dim))
    qr[:, rows] = oracle.rope(bits_to_f32(inp["q"][:, rows]), pos[:, rows], w.theta)
    kr = oracle.rope(bits_to_f32(inp["k"]), pos, w.theta)
    o_ref, lse_ref = oracle.attention_local_global_rows(qr, kr, bits_to_f32(inp["v"]), rows, w.window, w.n_lead,
                                                        w.anchor_stride, w.scale)
    check_bf16("o (sampled rows)", o, o_ref)
    check("lse (sampled rows)", lse, lse_ref, BF16_MAX, BF16_MEAN)
