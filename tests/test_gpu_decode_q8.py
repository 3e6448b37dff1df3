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
@pytest.mark.parametrize("hq,hkv,page", [(32, 8, 64), (32, 8, 16), (32, 2, 128), (8, 8, 32), (12, 4, 64)])
def test_q8_decode_small(kind, hq, hkv, page):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], hq=hq, hkv=hkv, page_size=page)
    say(f"q8 decode {kind} hq={hq} hkv={hkv} page={page} lens={LENS}")
    inp = paged_decode_inputs(w, seed=81, seq_lens=LENS, max_len=2048, kv=kind)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_q8_placement_and_poison_are_invisible(kind):
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
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
    within the bf16 tolerance (their contraction orders differ)."""
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
    check("q8 vs bf16", bits_to_f32(o8), bits_to_f32(host_bf16(ob)), BF16_MAX, BF16_MEAN)
    check("lse", l8, lb.cpu().numpy(), BF16_MAX, BF16_MEAN)


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
