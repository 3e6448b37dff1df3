"""attn_mla_decode_q8 on the GPU against the fp64 oracle over the dequantised latent cache: FP8 E4M3 and int8 codes
with per-channel scales, ragged and degenerate lengths, head counts, poisoned tokens past the length, the unit-scale
case against the bf16 kernel on the decoded cache, determinism, and the full benchmark workload."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, mla_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu


def run_gpu(ta, w, inp):
    o, lse = ta.attn_mla_decode_q8(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev(inp["c_kv"]), dev(inp["k_pe"]),
                                   dev(inp["c_scale"]), dev(inp["pe_scale"]), inp["kv"], dev(inp["seq_lens"]), w.scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(o), lse.cpu().numpy()


def run_oracle(w, inp):
    f = bits_to_f32
    return oracle.mla_decode_q8(f(inp["q_lat"]), f(inp["q_pe"]), inp["c_kv"], inp["k_pe"], inp["c_scale"],
                                inp["pe_scale"], inp["kv"], inp["seq_lens"], w.scale)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("heads,t,lens", [(128, 300, [300, 37, 1]), (32, 100, [100, 64]), (64, 1000, [999, 1000]),
                                          (96, 130, [65, 130])])
def test_mla_q8_small(kind, heads, t, lens):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["mla_decode_b32"], heads=heads)
    say(f"mla q8 {kind} heads={heads} T={t} lens={lens}")
    inp = mla_inputs(w, seed=41, batch=len(lens), seqlen=t, seq_lens=lens, kv=kind)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_mla_q8_length_zero_and_poison_past_the_length(kind):
    """A sequence of length 0 gives O = 0, lse = -inf; codes past a sequence's length (NaN for FP8, extreme for
    int8) change nothing."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=42, batch=3, seqlen=256, seq_lens=[200, 0, 77], kv=kind)
    o1, l1 = run_gpu(ta, w, inp)
    assert np.all(o1[1] == 0) and np.all(np.isneginf(l1[1]))
    inp["c_kv"][0, 200:] = 0x7F
    inp["k_pe"][2, 77:] = 0xFF
    o2, l2 = run_gpu(ta, w, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, lse_ref = run_oracle(w, dict(inp, seq_lens=np.array([200, 0, 77], np.int32)))
    check_bf16("o", o1[[0, 2]], o_ref[[0, 2]])


def test_mla_fp8_unit_scales_match_bf16_kernel_on_decoded_cache():
    """FP8 codes are exact in bf16: with unit scales the 8-bit kernel and the bf16 kernel on the decoded cache compute
    the same attention. Unit scales make the latent values, and so the outputs, as large as the codes (up to 448),
    so the bound is relative to each head's output scale (its largest |o|): the FP8 kernel carries the query and
    the probabilities as two E4M3 terms (about the 8 significant bits of bf16) and rounds in other places than the
    bf16 kernel, and two such results agree to a few units of bf16 rounding of that scale (2^-6 allowed; mean
    2^-9). The lse agrees to 1e-4 relative."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=43, batch=2, seqlen=700, seq_lens=[700, 333], kv="fp8")
    inp["c_scale"] = np.ones_like(inp["c_scale"])
    inp["pe_scale"] = np.ones_like(inp["pe_scale"])
    o8, l8 = run_gpu(ta, w, inp)
    to_bits = lambda c: (oracle.fp8_e4m3_decode(c).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ob, lb = ta.attn_mla_decode(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev_bf16(to_bits(inp["c_kv"])),
                                dev_bf16(to_bits(inp["k_pe"])), dev(inp["seq_lens"]), w.scale, return_lse=True)
    torch.cuda.synchronize()
    a, b = bits_to_f32(o8).astype(np.float64), bits_to_f32(host_bf16(ob)).astype(np.float64)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    scale = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-3)      # per (sequence, head)
    rel = np.abs(a - b) / scale
    say(f"  q8 vs bf16: max {rel.max():.3e}, mean {rel.mean():.3e} of each head's output scale "
        f"(max |o| {np.abs(b).max():.1f})")
    assert rel.max() <= 2.0 ** -6 and rel.mean() <= 2.0 ** -9, (rel.max(), rel.mean())
    la, lb_ = l8.astype(np.float64), lb.cpu().numpy().astype(np.float64)
    lrel = np.abs(la - lb_) / np.maximum(np.abs(lb_), 1.0)
    say(f"  lse: max relative difference {lrel.max():.3e}")
    assert lrel.max() <= 1e-4, lrel.max()


def test_mla_q8_is_deterministic():
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    inp = mla_inputs(w, seed=44, batch=2, seqlen=3000, kv="int8")
    a = run_gpu(ta, w, inp)
    b = run_gpu(ta, w, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_full_size_mla_q8_decode(kind):
    """The benchmark's workload with an 8-bit latent cache (32 sequences x 32768 tokens, 128 heads) in the bench's
    launch configuration; the oracle checks three sequences."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    say(f"full-size MLA {kind} decode: generating inputs")
    inp = mla_inputs(w, seed=0, kv=kind)
    o, lse = run_gpu(ta, w, inp)
    seqs = [0, 13, 31]
    say(f"  oracle on sequences {seqs}")
    sub = dict(inp, q_lat=inp["q_lat"][seqs], q_pe=inp["q_pe"][seqs], c_kv=inp["c_kv"][seqs], k_pe=inp["k_pe"][seqs],
               seq_lens=inp["seq_lens"][seqs])
    o_ref, lse_ref = run_oracle(w, sub)
    check_bf16("o", o[seqs], o_ref)
    check("lse", lse[seqs], lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_mla_q8_every_code_value(kind):
    """Every code byte of the latent and rope caches (int8 including -128, every finite E4M3 code with subnormals)
    against the oracle's decoding of the same bytes; per-channel scales put the largest code near magnitude 1."""
    ta = require_gpu()
    w = WORKLOADS["mla_decode_b32"]
    say(f"mla q8 every code value {kind}")
    inp = mla_inputs(w, seed=43, batch=2, seqlen=320, seq_lens=[320, 129], kv=kind)
    r = np.random.default_rng(5)
    top = 448.0 if kind == "fp8" else 128.0
    for name, sc in (("c_kv", "c_scale"), ("k_pe", "pe_scale")):
        n = inp[name].size
        b = np.concatenate([r.permutation(256) for _ in range((n + 255) // 256)])[:n].astype(np.uint8)
        if kind == "fp8":
            b[b == 0x7F] = 0x7E
            b[b == 0xFF] = 0xFE
        inp[name] = b.reshape(inp[name].shape)
        inp[sc] = (r.uniform(0.5, 1.5, inp[sc].shape) / top).astype(np.float32)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)
