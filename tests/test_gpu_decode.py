"""attn_decode_paged on the GPU against the fp64 oracle, plus the bit-exact indexing properties of the paged
cache (physical placement, poisoned unused pages and slots, out-of-range unused table entries)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, paged_decode_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu


def run_gpu(ta, w, inp, rotate=True):
    q = dev_bf16(inp["q"])
    if rotate:
        ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    o, lse = ta.attn_decode_paged(q, dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"]), dev(inp["block_table"]),
                                  dev(inp["seq_lens"]), inp["max_len"], softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(o), lse.cpu().numpy()


def run_oracle(w, inp):
    q = oracle.rope(bits_to_f32(inp["q"])[:, None], inp["positions"][:, None], w.theta)[:, 0]
    return oracle.decode_paged(q, bits_to_f32(inp["k_cache"]), bits_to_f32(inp["v_cache"]), inp["block_table"],
                               inp["seq_lens"], w.scale)


LENS = [1, 17, 64, 65, 600, 1300, 511, 512, 513, 1024]


@pytest.mark.parametrize("hq,hkv,page,d", [(32, 8, 64, 128), (32, 8, 16, 128), (32, 2, 128, 128), (8, 8, 32, 128),
                                         (12, 4, 64, 128), (32, 8, 64, 64), (32, 8, 16, 64), (16, 1, 128, 64),
                                         (12, 4, 32, 64)])
def test_decode_small(hq, hkv, page, d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], hq=hq, hkv=hkv, page_size=page, head_dim=d,
                            scale=1.0 / np.sqrt(d))
    say(f"decode hq={hq} hkv={hkv} page={page} d={d} lens={LENS}")
    inp = paged_decode_inputs(w, seed=21, seq_lens=LENS, max_len=2048)
    o, lse = run_gpu(ta, w, inp)
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


def relayout(inp, seed, poison_spare=True, bad_unused=True):
    """Same logical K/V in a new random physical placement; spare pages NaN, unused table entries out of range."""
    ps = inp["k_cache"].shape[1]
    n_pool = inp["k_cache"].shape[0]
    perm = np.random.default_rng(seed).permutation(n_pool)
    kc = np.full_like(inp["k_cache"], 0x7FC0 if poison_spare else 0)     # bf16 NaN
    vc = np.full_like(inp["v_cache"], 0x7FC0 if poison_spare else 0)
    table = np.full_like(inp["block_table"], (1 << 30) if bad_unused else -1)
    off = 0
    for b, L in enumerate(inp["seq_lens"]):
        for j in range((int(L) + ps - 1) // ps):
            src = inp["block_table"][b, j]
            dst = perm[off]; off += 1
            kc[dst] = inp["k_cache"][src]; vc[dst] = inp["v_cache"][src]
            table[b, j] = dst
    out = dict(inp); out.update(k_cache=kc, v_cache=vc, block_table=table)
    return out


@pytest.mark.parametrize("d", [128, 64])
def test_physical_placement_and_poison_are_invisible(d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    say(f"decode placement / poison d={d}")
    inp = paged_decode_inputs(w, seed=22, seq_lens=[3, 70, 999, 1500, 64, 1], max_len=1600)
    o1, l1 = run_gpu(ta, w, inp)
    for seed in (1, 2):
        o2, l2 = run_gpu(ta, w, relayout(inp, seed))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), seed


@pytest.mark.parametrize("d", [128, 64])
def test_slots_past_the_length_are_invisible(d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    inp = paged_decode_inputs(w, seed=23, seq_lens=[5, 130, 1001], max_len=1024)
    o1, l1 = run_gpu(ta, w, inp)
    ps = w.page_size
    for b, L in enumerate(inp["seq_lens"]):
        last = inp["block_table"][b, (L - 1) // ps]
        inp["k_cache"][last, L % ps if L % ps else ps:] = 0x46EA      # +3e4 (finite): masked, P = 0
        inp["v_cache"][last, L % ps if L % ps else ps:] = 0xC6EA      # -3e4
    o2, l2 = run_gpu(ta, w, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("d", [128, 64])
def test_length_one_is_v0_and_length_zero_is_empty(d):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["paged_decode_b64"], head_dim=d, scale=1.0 / np.sqrt(d))
    inp = paged_decode_inputs(w, seed=24, seq_lens=[1, 0, 1], max_len=64)
    o, lse = run_gpu(ta, w, inp)
    grp = w.hq // w.hkv
    for b in (0, 2):
        v0 = inp["v_cache"][inp["block_table"][b, 0], 0]
        for h in range(w.hq):
            assert np.array_equal(o[b, h], v0[h // grp])
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_decode_matches_last_row_of_prefill():
    """Cross-kernel: decode over a paged copy equals (within tolerance) the last causal row of prefill."""
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    L = 777
    inp = paged_decode_inputs(w, seed=25, seq_lens=[L], max_len=1024)
    k = oracle.gather_paged(inp["k_cache"], inp["block_table"][0], L)[None]     # [1, L, Hkv, D] bits
    v = oracle.gather_paged(inp["v_cache"], inp["block_table"][0], L)[None]
    qfull = np.zeros((1, L, w.hq, w.head_dim), np.uint16)
    qfull[0, L - 1] = inp["q"][0]
    qd = dev_bf16(qfull)
    ta.attn_rope_apply(qd, dev(np.arange(L, dtype=np.int32)), w.theta)
    o_pre = ta.attn_prefill(qd, dev_bf16(k), dev_bf16(v), causal=True, softmax_scale=w.scale)
    o_dec, _ = run_gpu(ta, w, inp)
    torch.cuda.synchronize()
    check("decode vs prefill", bits_to_f32(o_dec[0]), bits_to_f32(host_bf16(o_pre)[0, L - 1]), BF16_MAX, BF16_MEAN)


def test_decode_is_deterministic():
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    inp = paged_decode_inputs(w, seed=26, seq_lens=[2000, 33, 4097], max_len=4200)
    a = run_gpu(ta, w, inp)
    b = run_gpu(ta, w, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_full_size_paged_decode():
    """The benchmark's workload: 64 sequences, lengths U[1024, 32768], 64-token pages, full oracle."""
    ta = require_gpu()
    w = WORKLOADS["paged_decode_b64"]
    say("full-size paged decode: generating inputs")
    inp = paged_decode_inputs(w, seed=0)
    say(f"  tokens {int(inp['seq_lens'].sum())}, pool pages {inp['k_cache'].shape[0]}; gpu")
    o, lse = run_gpu(ta, w, inp)
    say("  oracle")
    o_ref, lse_ref = run_oracle(w, inp)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)
