"""attn_mla_decode on the GPU against the fp64 oracle (absorbed form as plain attention over [c_kv ; k_pe])."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, mla_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu


def run_gpu(ta, w, inp):
    o, lse = ta.attn_mla_decode(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev_bf16(inp["c_kv"]),
                                dev_bf16(inp["k_pe"]), dev(inp["seq_lens"]), w.scale, return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(o), lse.cpu().numpy()


def run_oracle(w, inp):
    f = bits_to_f32
    return oracle.mla_decode(f(inp["q_lat"]), f(inp["q_pe"]), f(inp["c_kv"]), f(inp["k_pe"]), inp["seq_lens"], w.scale)


@pytest.mark.parametrize("heads,t,lens", [(128, 300, [300, 37, 1]), (32, 100, [100, 64]), (64, 1000, [999, 1000])])
def test_mla_small(heads, t, lens):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["mla_decode_b32"], heads=heads)
    say(f"mla heads={heads} T={t} lens={lens}")
    inp = mla_inputs(w, seed=31, batch=len(lens), seqlen=t, seq_lens=lens)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


def test_mla_length_one_and_zero():
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=32, batch=2, seqlen=64, seq_lens=[1, 0])
    o, lse = run_gpu(ta, w, inp)
    for h in range(w.heads):
        assert np.array_equal(o[0, h], inp["c_kv"][0, 0])
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_mla_tokens_past_the_length_are_invisible():
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=33, batch=2, seqlen=256, seq_lens=[200, 77])
    o1, l1 = run_gpu(ta, w, inp)
    inp["c_kv"][0, 200:] = 0x7FC0          # NaN after the length: must never be read
    inp["k_pe"][1, 77:] = 0x7FC0
    o2, l2 = run_gpu(ta, w, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_mla_is_deterministic():
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=34, batch=2, seqlen=3000)
    a = run_gpu(ta, w, inp)
    b = run_gpu(ta, w, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_full_size_mla_decode():
    """The benchmark's workload: 32 sequences x 32768 latent tokens, 128 heads, full oracle."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    say("full-size MLA decode: generating inputs")
    inp = mla_inputs(w, seed=0)
    say("  gpu")
    o, lse = run_gpu(ta, w, inp)
    say("  oracle")
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)
