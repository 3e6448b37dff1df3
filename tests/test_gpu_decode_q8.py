"""attn_decode_paged_q8 on the GPU against the fp64 oracle over the dequantised caches: FP8 E4M3 and int8 codes with
per-(KV head, channel) scales, ragged lengths, several head groups and page sizes, physical placement and poisoned
unused pages, the unit-scale case against the bf16 kernel, and the full benchmark workload."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, paged_decode_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu

LENS = [1, 17, 64, 65, 600, 1300, 511, 512, 513, 1024]


def run_gpu(ta, w, inp, rotate=True):
    q = dev_bf16(inp["q"])
    if rotate:
        ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    o, lse = ta.attn_decode_paged_q8(q, dev(inp["k_cache"]), dev(inp["v_cache"]), dev(inp["k_scale"]),
                                     dev(inp["v_scale"]), inp["kv"], dev(inp["block_table"]), dev(inp["seq_lens"]),
                                     inp["max_len"], softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(o), lse.cpu().numpy()


def run_oracle(w, inp):
    q = oracle.rope(bits_to_f32(inp["q"])[:, None], inp["positions"][:, None], w.theta)[:, 0]
    return oracle.decode_paged_q8(q, inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["kv"],
                                  inp["block_table"], inp["seq_lens"], w.scale)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
# One KV head per wave; the cases cover head-group counts that 8 (the XCD grouping of the unit order) divides
# and ones it does not (12/3, 5/5, 16/1), at both head dims.
@pytest.mark.parametrize("hq,hkv,page,d", [(32, 8, 64, 128), (32, 8, 16, 128), (32, 2, 128, 128), (8, 8, 32, 128),
                                         (12, 4, 64, 128), (12, 3, 64, 128), (5, 5, 16, 128), (32, 8, 64, 64),
                                         (32, 8, 16, 64), (16, 1, 128, 64), (12, 4, 32, 64), (8, 2, 64, 64)])
def test_q8_decode_small(kind, hq, hkv, page, d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], hq=hq, hkv=hkv, page_size=page, head_dim=d,
                            scale=1.0 / np.sqrt(d))
    say(f"q8 decode {kind} hq={hq} hkv={hkv} page={page} d={d} lens={LENS}")
    inp = paged_decode_inputs(w, seed=81, seq_lens=LENS, max_len=2048, kv=kind)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("d", [128, 64])
def test_q8_placement_and_poison_are_invisible(kind, d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    say(f"q8 decode placement / poison {kind} d={d}")
    inp = paged_decode_inputs(w, seed=82, seq_lens=[3, 70, 999, 1500, 64, 1], max_len=1600, kv=kind)
    o1, l1 = run_gpu(ta, w, inp)
    ps = w.page_size
    perm = np.random.default_rng(5).permutation(inp["k_cache"].shape[0])
    kc = np.full_like(inp["k_cache"], 0x7F)          # NaN (fp8) / 127 (int8) in every page not in use
    vc = np.full_like(inp["v_cache"], 0x7F)
    table = np.full_like(inp["block_table"], 1 << 30)
    off = 0
    for b, L in enumerate(inp["seq_lens"]):
        for j in range((int(L) + ps - 1) // ps):
            src, dst = inp["block_table"][b, j], perm[off]
            off += 1
            kc[dst], vc[dst] = inp["k_cache"][src], inp["v_cache"][src]
            table[b, j] = dst
    inp2 = dict(inp, k_cache=kc, v_cache=vc, block_table=table)
    o2, l2 = run_gpu(ta, w, inp2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_q8_with_unit_scales_matches_bf16_decode():
    """FP8 codes are exact in bf16: with unit scales the 8-bit kernel and the bf16 kernel on the decoded cache agree
    to the rounding of their bf16 outputs. Unit scales make the cached values (and outputs) as large as the codes
    (up to 448), so the bound is relative: two roundings to bf16 of nearly the same value differ by at most one
    unit in the last place, 2^-7 of the value (2^-6 allowed); the kernels' split sizes and contraction orders
    differ, so the fp32 results themselves differ slightly. The lse agrees to fp32 summation order (1e-4 relative)."""
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    inp = paged_decode_inputs(w, seed=83, seq_lens=[700, 2048, 5], max_len=2048, kv="fp8")
    inp["k_scale"] = np.ones_like(inp["k_scale"])
    inp["v_scale"] = np.ones_like(inp["v_scale"])
    o8, l8 = run_gpu(ta, w, inp)
    kb = (oracle.fp8_e4m3_decode(inp["k_cache"]).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (oracle.fp8_e4m3_decode(inp["v_cache"]).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = dev_bf16(inp["q"])
    ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    ob, lb = ta.attn_decode_paged(q, dev_bf16(kb), dev_bf16(vb), dev(inp["block_table"]), dev(inp["seq_lens"]),
                                  inp["max_len"], softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    a, b = bits_to_f32(o8).astype(np.float64), bits_to_f32(host_bf16(ob)).astype(np.float64)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    rel = np.abs(a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-3)
    say(f"  q8 vs bf16: max relative difference {rel.max():.3e} (max |o| {np.abs(b).max():.1f})")
    assert rel.max() <= 2.0 ** -6, rel.max()
    la, lb_ = l8.astype(np.float64), lb.cpu().numpy().astype(np.float64)
    lrel = np.abs(la - lb_) / np.maximum(np.abs(lb_), 1.0)
    say(f"  lse: max relative difference {lrel.max():.3e}")
    assert lrel.max() <= 1e-4, lrel.max()


def compact(inp, seqs):
    """The inputs of a subset of sequences with their pages copied into a small pool (same logical contents)."""
    ps = inp["k_cache"].shape[1]
    pages = [inp["block_table"][b, : (int(inp["seq_lens"][b]) + ps - 1) // ps] for b in seqs]
    table = np.full((len(seqs), max(len(p) for p in pages)), -1, np.int32)
    off = 0
    for i, p in enumerate(pages):
        table[i, : len(p)] = np.arange(off, off + len(p))
        off += len(p)
    allp = np.concatenate(pages)
    return dict(inp, q=inp["q"][seqs], positions=inp["positions"][seqs], seq_lens=inp["seq_lens"][seqs],
                k_cache=inp["k_cache"][allp], v_cache=inp["v_cache"][allp], block_table=table)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_full_size_q8_decode(kind):
    """The benchmark's workload with an 8-bit cache (64 sequences, lengths U[1024, 32768], 64-token pages) in the
    bench's launch configuration; the oracle checks the shortest, the longest and five seeded sequences."""
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    say(f"full-size {kind} paged decode: generating inputs")
    inp = paged_decode_inputs(w, seed=0, kv=kind)
    o, lse = run_gpu(ta, w, inp)
    lens = inp["seq_lens"]
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))} |
                  set(np.random.default_rng(84).choice(len(lens), 5, replace=False).tolist()))
    say(f"  oracle on sequences {seqs}")
    o_ref, lse_ref = run_oracle(w, compact(inp, seqs))
    check_bf16("o", o[seqs], o_ref)
    check("lse", lse[seqs], lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "int8"])
def test_many_sequences_with_empty_ones(kind):
    """150 sequences (the 8-bit kernels enumerate the (sequence, chunk) pairs that hold keys 64 sequences at a
    time), lengths from 0 to 2500 with empty sequences between long ones: every head of every sequence against the
    oracle, empty sequences give O = 0 and lse = -inf."""
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], batch=150, hq=8, hkv=2, page_size=16)
    lens = np.random.default_rng(85).integers(1, 2500, 150)
    lens[::7] = 0
    lens[[63, 64, 127, 128]] = [0, 2500, 1025, 0]
    say(f"{kind} decode, 150 sequences, {int((lens == 0).sum())} empty")
    inp = paged_decode_inputs(w, seed=85, seq_lens=lens.tolist(), max_len=2500, kv=kind)
    q = dev_bf16(inp["q"])
    ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    if kind == "bf16":
        o, lse = ta.attn_decode_paged(q, dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"]), dev(inp["block_table"]),
                                      dev(inp["seq_lens"]), inp["max_len"], softmax_scale=w.scale, return_lse=True)
    else:
        o, lse = ta.attn_decode_paged_q8(q, dev(inp["k_cache"]), dev(inp["v_cache"]), dev(inp["k_scale"]),
                                         dev(inp["v_scale"]), kind, dev(inp["block_table"]), dev(inp["seq_lens"]),
                                         inp["max_len"], softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    o, lse = host_bf16(o), lse.cpu().numpy()
    qr = oracle.rope(bits_to_f32(inp["q"])[:, None], inp["positions"][:, None], w.theta)[:, 0]
    full = lens > 0
    if kind == "bf16":
        o_ref, lse_ref = oracle.decode_paged(qr[full], bits_to_f32(inp["k_cache"]), bits_to_f32(inp["v_cache"]),
                                             inp["block_table"][full], inp["seq_lens"][full], w.scale)
    else:
        o_ref, lse_ref = oracle.decode_paged_q8(qr[full], inp["k_cache"], inp["v_cache"], inp["k_scale"],
                                                inp["v_scale"], kind, inp["block_table"][full], inp["seq_lens"][full],
                                                w.scale)
    check_bf16("o", o[full], o_ref)
    check("lse", lse[full], lse_ref, BF16_MAX, BF16_MEAN)
    assert np.all(o[~full] == 0) and np.all(np.isneginf(lse[~full]))


def every_code(shape, kind, seed):
    """Cache bytes taking every code value: seeded permutations of all 256 bytes, repeated. For int8 this includes
    0x80 (-128), which the generator's [-127, 127] never produces; for FP8 the two NaN codes are replaced by the
    largest finite ones (every other E4M3 code, subnormals included, occurs)."""
    r = np.random.default_rng(seed)
    n = int(np.prod(shape))
    b = np.concatenate([r.permutation(256) for _ in range((n + 255) // 256)])[:n].astype(np.uint8)
    if kind == "fp8":
        b[b == 0x7F] = 0x7E
        b[b == 0xFF] = 0xFE
    return b.reshape(shape)


def unit_range_scales(shape, kind, seed):
    """Per-channel scales that put the largest code near magnitude 1 (0.5x to 1.5x, seeded per channel)."""
    top = 448.0 if kind == "fp8" else 128.0
    return (np.random.default_rng(seed).uniform(0.5, 1.5, shape) / top).astype(np.float32)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("d", [128, 64])
def test_q8_decode_every_code_value(kind, d):
    """Every code byte through the GPU's code conversion (int8 sign extension including -128; every finite E4M3
    code) against the oracle's decoding of the same bytes."""
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    say(f"q8 decode every code value {kind} d={d}")
    inp = paged_decode_inputs(w, seed=83, seq_lens=[300, 1, 700, 64], max_len=768, kv=kind)
    inp["k_cache"] = every_code(inp["k_cache"].shape, kind, 1)
    inp["v_cache"] = every_code(inp["v_cache"].shape, kind, 2)
    inp["k_scale"] = unit_range_scales(inp["k_scale"].shape, kind, 3)
    inp["v_scale"] = unit_range_scales(inp["v_scale"].shape, kind, 4)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)
