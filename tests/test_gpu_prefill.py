"""attn_prefill on the GPU against the fp64 oracle: RoPE on the GPU, then attention, compared element by element
(or on seeded sampled rows at the full long-context sizes)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, prefill_inputs, sampled_rows
from gpu_util import (require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, scale_for,
                      FP32_MAX, BF16_MAX, BF16_MEAN)

pytestmark = pytest.mark.gpu


def run_gpu(ta, w, inp, causal=True, lse=True):
    """RoPE(q), RoPE(k) at positions 0..S-1, then prefill; returns (o bits or floats, lse)."""
    bf = w.dtype == "bf16"
    q = dev_bf16(inp["q"]) if bf else dev(inp["q"])
    k = dev_bf16(inp["k"]) if bf else dev(inp["k"])
    v = dev_bf16(inp["v"]) if bf else dev(inp["v"])
    pos = dev(inp["positions"])
    ta.attn_rope_apply(q, pos, w.theta)
    ta.attn_rope_apply(k, pos, w.theta)
    o, l = ta.attn_prefill(q, k, v, causal=causal, softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    o_h = host_bf16(o) if bf else o.cpu().numpy()
    return o_h, l.cpu().numpy()


def oracle_inputs(w, inp):
    conv = bits_to_f32 if w.dtype == "bf16" else (lambda a: a)
    b, s = inp["q"].shape[:2]
    pos = inp["positions"].reshape(b, s)
    q = oracle.rope(conv(inp["q"]), pos, w.theta)
    k = oracle.rope(conv(inp["k"]), pos, w.theta)
    return q, k, conv(inp["v"]).astype(np.float64)


def test_mha_fp32_s256_full():
    ta = require_gpu()
    w = WORKLOADS["mha_fp32_s256"]
    say(f"prefill fp32 {w}")
    inp = prefill_inputs(w, seed=0)
    o, lse = run_gpu(ta, w, inp)
    q, k, v = oracle_inputs(w, inp)
    o_ref, lse_ref = oracle.attention_prefill(q, k, v, True, w.scale)
    check("o", o, o_ref, FP32_MAX)
    check("lse", lse, lse_ref, FP32_MAX)


FP32_CASES = [  # (batch, seqlen, hq, hkv, head_dim, causal)
    (1, 300, 8, 2, 128, True),     # head_dim 128, 4 query heads per KV head, ragged tail
    (2, 513, 4, 4, 64, False),     # no causal mask, ragged
    (1, 300, 8, 2, 64, False),     # GQA without the mask
    (1, 513, 6, 3, 128, True),     # 2 query heads per KV head, ragged
    (1, 1, 4, 2, 128, True),       # a single token
    (1, 64, 8, 1, 128, False),     # one KV head for all query heads, exactly two 32-key tiles
]


@pytest.mark.parametrize("case", FP32_CASES, ids=lambda c: "b{}_s{}_hq{}_hkv{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full"))
def test_fp32_prefill_small(case):
    """The fp32 path against the oracle at the fp32 bound (max abs <= 1e-5) beyond the 256-token MHA workload."""
    ta = require_gpu()
    b, s, hq, hkv, d, causal = case
    w = dataclasses.replace(WORKLOADS["mha_fp32_s256"], batch=b, seqlen=s, hq=hq, hkv=hkv, head_dim=d,
                            scale=scale_for(d), causal=causal)
    say(f"prefill fp32 {case}")
    inp = prefill_inputs(w, seed=12)
    o, lse = run_gpu(ta, w, inp, causal=causal)
    q, k, v = oracle_inputs(w, inp)
    o_ref, lse_ref = oracle.attention_prefill(q, k, v, causal, w.scale)
    check("o", o, o_ref, FP32_MAX)
    check("lse", lse, lse_ref, FP32_MAX)


SMALL = [  # (batch, seqlen, hq, hkv, head_dim, causal)
    (2, 300, 8, 2, 128, True),     # 4 query heads per KV head: heads mode; ragged tail
    (1, 200, 4, 4, 64, True),      # MHA: positions mode, head_dim 64
    (1, 130, 6, 3, 128, True),     # 2 query heads per KV head
    (1, 257, 16, 2, 128, True),    # 8 per KV head: two workgroups share a KV head
    (2, 190, 8, 2, 128, False),    # no causal mask
    (1, 1, 8, 2, 128, True),       # a single token
    (1, 64, 4, 1, 64, True),       # exactly one tile
    (1, 513, 4, 4, 128, False),    # MHA, full attention, ragged
    # more workgroups than the device holds at once (256 compute units, one each): two or three rounds
    (3, 2000, 32, 8, 128, True),   # 504 units
    (4, 1600, 32, 8, 64, True),    # 544 units, head_dim 64
    (1, 2000, 80, 80, 64, True),   # positions mode, 480 units over 80 head groups
    (3, 1200, 32, 8, 128, False),  # no causal mask, 312 units
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}_s{}_hq{}_hkv{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full"))
def test_bf16_prefill_small(case):
    ta = require_gpu()
    b, s, hq, hkv, d, causal = case
    w = dataclasses.replace(WORKLOADS["gqa_prefill_s8192"], batch=b, seqlen=s, hq=hq, hkv=hkv, head_dim=d,
                            scale=scale_for(d), causal=causal)
    say(f"prefill bf16 {case}")
    inp = prefill_inputs(w, seed=11)
    o, lse = run_gpu(ta, w, inp, causal=causal)
    q, k, v = oracle_inputs(w, inp)
    o_ref, lse_ref = oracle.attention_prefill(q, k, v, causal, w.scale)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


def test_causal_row_zero_is_v0_exactly():
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["gqa_prefill_s8192"], batch=2, seqlen=130)
    inp = prefill_inputs(w, seed=5)
    o, _ = run_gpu(ta, w, inp)
    grp = w.hq // w.hkv
    for h in range(w.hq):
        assert np.array_equal(o[:, 0, h], inp["v"][:, 0, h // grp]), h


def test_future_keys_do_not_change_earlier_rows():
    """Finite extreme values in keys/values after position 127 leave rows 0..127 bitwise unchanged."""
    ta = require_gpu()
    for hq, hkv in ((8, 2), (4, 4)):
        w = dataclasses.replace(WORKLOADS["gqa_prefill_s8192"], batch=1, seqlen=256, hq=hq, hkv=hkv)
        say(f"poison hq={hq} hkv={hkv}")
        inp = prefill_inputs(w, seed=6)
        o1, _ = run_gpu(ta, w, inp)
        rng = np.random.default_rng(7)
        for name in ("k", "v"):
            poison = np.where(rng.random(inp[name][:, 128:].shape) < 0.5, 0xC6EA, 0x46EA).astype(np.uint16)  # +-3e4
            inp[name][:, 128:] = poison
        o2, _ = run_gpu(ta, w, inp)
        assert np.array_equal(o1[:, :128], o2[:, :128])


def test_prefill_is_deterministic():
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["gqa_prefill_s8192"], batch=1, seqlen=700)
    inp = prefill_inputs(w, seed=8)
    o1, l1 = run_gpu(ta, w, inp)
    o2, l2 = run_gpu(ta, w, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name,n_rows", [("gqa_prefill_s8192", 64), ("gqa_prefill_s131072", 256)])
def test_full_size_sampled_rows(name, n_rows):
    """The benchmark's launch configuration at full size; the oracle computes seeded sampled query rows for every
    head (the first and last row always included)."""
    ta = require_gpu()
    w = WORKLOADS[name]
    say(f"full-size prefill {name}: generating inputs")
    inp = prefill_inputs(w, seed=0)
    say("  gpu")
    o, lse = run_gpu(ta, w, inp)
    rows = sampled_rows(w.seqlen, n_rows, seed=0)
    say(f"  oracle on {rows.size} rows")
    pos = np.arange(w.seqlen)
    k = oracle.rope(bits_to_f32(inp["k"]), np.broadcast_to(pos, (w.batch, w.seqlen)), w.theta)
    v = bits_to_f32(inp["v"]).astype(np.float64)
    qr = np.zeros((w.batch, w.seqlen, w.hq, w.head_dim))
    qr[:, rows] = oracle.rope(bits_to_f32(inp["q"][:, rows]), np.broadcast_to(rows, (w.batch, rows.size)), w.theta)
    o_ref, lse_ref = oracle.attention_prefill_rows(qr, k, v, rows, True, w.scale)
    check_bf16("o rows", o[:, rows], o_ref)
    check("lse rows", lse[:, :, rows], lse_ref, BF16_MAX, BF16_MEAN)
