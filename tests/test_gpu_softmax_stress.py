"""The online softmax under stress, against the fp64 oracle: scores that grow by far more than the lazy-rescale
threshold from one key tile to the next (the running max moves and O, l are rescaled at nearly every tile), and
scores that fall steeply (later tiles underflow to P = 0 against the first tile's max). Prefill (bf16 and the
local + global kernel), paged decode (bf16 and FP8 caches) and MLA decode. Inputs carry a seeded N(0,1) part plus a
ramp along one dimension, so the expected result is far from the mean of V and a missed rescale shows."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, prefill_inputs, paged_decode_inputs, mla_inputs, f32_to_bf16_bits, f32_to_e4m3_bits
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu


def ramp(n, slope):
    """Per-token ramp: +slope*j (growing) or -slope*j (falling) along the last dimension."""
    return slope * np.arange(n, dtype=np.float32)


@pytest.mark.parametrize("slope", [0.4, -0.4])
def test_prefill_rescale_every_tile(slope):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["gqa_prefill_s8192"], batch=1, seqlen=700, hq=8, hkv=2, head_dim=128,
                            scale=1.0 / np.sqrt(128))
    say(f"prefill stress slope={slope}")
    inp = prefill_inputs(w, seed=150)
    q = bits_to_f32(inp["q"]).copy(); k = bits_to_f32(inp["k"]).copy(); v = bits_to_f32(inp["v"])
    q[..., -1] = 8.0                                   # every query points along the last dimension
    k[0, :, :, -1] += ramp(w.seqlen, slope)[:, None]   # key j's score rises (or falls) by ~3.2*slope*j
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    o, lse = ta.attn_prefill(dev_bf16(qb), dev_bf16(kb), dev_bf16(inp["v"]), causal=True, softmax_scale=w.scale,
                             return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_prefill(bits_to_f32(qb), bits_to_f32(kb), v.astype(np.float64), True, w.scale)
    check_bf16("o", host_bf16(o), o_ref)
    check("lse", lse.cpu().numpy(), lse_ref, BF16_MAX, BF16_MEAN)
    # the local + global kernel on the same inputs: window 300 with anchors every 50 tokens
    o2, l2 = ta.attn_prefill_local_global(dev_bf16(qb), dev_bf16(kb), dev_bf16(inp["v"]), 300, 2, 50,
                                          softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    o2_ref, l2_ref = oracle.attention_local_global(bits_to_f32(qb), bits_to_f32(kb), v.astype(np.float64), 300, 2, 50,
                                                   w.scale)
    check_bf16("o (local + global)", host_bf16(o2), o2_ref)
    check("lse (local + global)", l2.cpu().numpy(), l2_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("slope", [0.05, -0.05])
def test_paged_decode_rescale_across_blocks(kind, slope):
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    lens = [3000, 1100, 64]
    say(f"decode stress kind={kind} slope={slope}")
    inp = paged_decode_inputs(w, seed=151, seq_lens=lens, max_len=3072)
    q = bits_to_f32(inp["q"]).copy()
    q[..., -1] = 8.0
    kc = bits_to_f32(inp["k_cache"]).copy()
    # logical token t of sequence b sits in page block_table[b, t // page] slot t % page
    ps = w.page_size
    for b, L in enumerate(lens):
        t = np.arange(L)
        kc[inp["block_table"][b, t // ps], t % ps, :, -1] += ramp(L, slope)[:, None]
    qb = f32_to_bf16_bits(q)
    if kind == "bf16":
        kb = f32_to_bf16_bits(kc)
        o, lse = ta.attn_decode_paged(dev_bf16(qb), dev_bf16(kb), dev_bf16(inp["v_cache"]), dev(inp["block_table"]),
                                      dev(inp["seq_lens"]), inp["max_len"], softmax_scale=w.scale, return_lse=True)
        k_ref, v_ref = bits_to_f32(kb), bits_to_f32(inp["v_cache"])
    else:   # FP8 codes with unit scales (values up to ~160 fit E4M3's 448)
        k8 = f32_to_e4m3_bits(kc)
        v8 = f32_to_e4m3_bits(bits_to_f32(inp["v_cache"]))
        ones = np.ones((w.hkv, w.head_dim), np.float32)
        o, lse = ta.attn_decode_paged_q8(dev_bf16(qb), dev(k8), dev(v8), dev(ones), dev(ones), "fp8",
                                         dev(inp["block_table"]), dev(inp["seq_lens"]), inp["max_len"],
                                         softmax_scale=w.scale, return_lse=True)
        k_ref, v_ref = oracle.fp8_e4m3_decode(k8), oracle.fp8_e4m3_decode(v8)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged(bits_to_f32(qb), k_ref, v_ref, inp["block_table"], inp["seq_lens"], w.scale)
    check_bf16("o", host_bf16(o), o_ref)
    check("lse", lse.cpu().numpy(), lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("slope", [0.03, -0.03])
def test_mla_rescale_across_tiles(kind, slope):
    """The FP8 latent cache runs on its own kernel (FP8 products, probabilities carried x 2^7 with the reference
    max moved whenever the max doubles), so it gets the same stress: the ramp moves the max by more than that at
    every 64-token tile."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    lens = [2000, 700]
    say(f"mla stress kind={kind} slope={slope}")
    inp = mla_inputs(w, seed=152, batch=2, seqlen=2048, seq_lens=lens)
    qp = bits_to_f32(inp["q_pe"]).copy(); kp = bits_to_f32(inp["k_pe"]).copy()
    qp[..., -1] = 8.0
    kp[:, :, -1] += ramp(2048, slope)[None]
    qpb, kpb = f32_to_bf16_bits(qp), f32_to_bf16_bits(kp)
    f = bits_to_f32
    if kind == "bf16":
        o, lse = ta.attn_mla_decode(dev_bf16(inp["q_lat"]), dev_bf16(qpb), dev_bf16(inp["c_kv"]), dev_bf16(kpb),
                                    dev(inp["seq_lens"]), w.scale, return_lse=True)
        ckv_ref, kpe_ref = f(inp["c_kv"]), f(kpb)
    else:   # FP8 codes with unit scales (the ramp reaches about 61, within E4M3's 448)
        c8, k8 = f32_to_e4m3_bits(f(inp["c_kv"])), f32_to_e4m3_bits(f(kpb))
        o, lse = ta.attn_mla_decode_q8(dev_bf16(inp["q_lat"]), dev_bf16(qpb), dev(c8), dev(k8),
                                       dev(np.ones(w.latent, np.float32)), dev(np.ones(w.rope, np.float32)), "fp8",
                                       dev(inp["seq_lens"]), w.scale, return_lse=True)
        ckv_ref, kpe_ref = oracle.fp8_e4m3_decode(c8), oracle.fp8_e4m3_decode(k8)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.mla_decode(f(inp["q_lat"]), f(qpb), ckv_ref, kpe_ref, inp["seq_lens"], w.scale)
    check_bf16("o", host_bf16(o), o_ref)
    check("lse", lse.cpu().numpy(), lse_ref, BF16_MAX, BF16_MEAN)


def test_mla_fp8_query_scales_span_many_binades():
    """The FP8 kernel brings each head's query into E4M3 range with its own power of two: heads whose queries
    differ by factors up to 2^16 (from uniform attention to a score spread of about 4) all match the oracle. The
    range stops there because the query enters the products as two E4M3 terms (about 8 significant bits of
    query x scale), so each score carries a relative error near 2^-9: harmless at ordinary score sizes, but with
    scores spread over tens of units (this workload's query x 2^5) the output moves by about 0.04."""
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["mla_decode_b32"], heads=64)
    inp = mla_inputs(w, seed=153, batch=2, seqlen=900, seq_lens=[900, 333], kv="fp8")
    f = bits_to_f32
    mult = (2.0 ** np.linspace(-14, 2, w.heads)).astype(np.float32)[None, :, None]
    ql = f32_to_bf16_bits(f(inp["q_lat"]) * mult)
    qp = f32_to_bf16_bits(f(inp["q_pe"]) * mult)
    o, lse = ta.attn_mla_decode_q8(dev_bf16(ql), dev_bf16(qp), dev(inp["c_kv"]), dev(inp["k_pe"]),
                                   dev(inp["c_scale"]), dev(inp["pe_scale"]), "fp8", dev(inp["seq_lens"]), w.scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.mla_decode_q8(f(ql), f(qp), inp["c_kv"], inp["k_pe"], inp["c_scale"], inp["pe_scale"],
                                          "fp8", inp["seq_lens"], w.scale)
    check_bf16("o", host_bf16(o), o_ref)
    lse = lse.cpu().numpy()
    rel = np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    say(f"  lse: max relative difference {rel.max():.3e}")
    assert rel.max() <= 1e-3, rel.max()
