"""DeepSeek Sparse Attention decode on the GPU against the fp64 oracle: attn_dsa_indexer (scores within an fp32
error bound derived from the arithmetic), attn_topk (bit-exact: the oracle's selection applied to the same fp32
scores the kernel selected from), attn_mla_sparse_decode (bf16 tolerance over the selected tokens), and the
three chained at the full workload size."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, dsa_inputs
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu

NAN = 0x7FC0
U = 2.0 ** -24          # fp32 unit roundoff


def indexer_bound(q, w, k, lens):
    """Elementwise bound on |fp32 score - exact score|: each head's dot is an fp32 sum of D exact bf16 products
    (error <= (D+1) u sum_i |q_i k_i|), then w_j * ReLU(.) and a sum over the H heads in fp32
    (<= (H+2) u sum_j |w_j ReLU_j|); doubled for safety."""
    aq, ak = np.abs(q.astype(np.float64)), np.abs(k.astype(np.float64))
    bsz, hi, d = q.shape
    out = np.zeros((bsz, k.shape[1]))
    for b in range(bsz):
        n = int(lens[b])
        dot_abs = ak[b, :n] @ aq[b].T                                           # [L, H]
        relu = np.maximum(k[b, :n].astype(np.float64) @ q[b].astype(np.float64).T, 0)
        out[b, :n] = 2 * U * ((d + 1) * dot_abs @ np.abs(w[b]) + (hi + 2) * relu @ np.abs(w[b]))
    return out


def check_scores(got, ref, bound, lens):
    for b in range(got.shape[0]):
        n = int(lens[b])
        assert np.all(np.isneginf(got[b, n:])), "slots past the length must be -inf"
        err = np.abs(got[b, :n].astype(np.float64) - ref[b, :n])
        assert np.all(err <= bound[b, :n]), f"seq {b}: score error {err.max()} above its fp32 bound"
    say(f"  scores: max err {max(float(np.abs(got[b, :int(lens[b])] - ref[b, :int(lens[b])]).max(initial=0)) for b in range(got.shape[0])):.3e}")


@pytest.mark.parametrize("hi,di", [(64, 128), (32, 128), (64, 64), (32, 64)])
def test_indexer_small(hi, di):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["dsa_decode_b32"], idx_heads=hi, idx_dim=di)
    lens = [1000, 1, 0, 257, 1024, 33]
    say(f"dsa indexer H_I={hi} D_I={di} lens={lens}")
    inp = dsa_inputs(w, seed=61, batch=len(lens), seqlen=1030, seq_lens=lens)
    sc = ta.attn_dsa_indexer(dev_bf16(inp["q_idx"]), dev(inp["w_idx"]), dev_bf16(inp["k_idx"]), dev(inp["seq_lens"]))
    torch.cuda.synchronize()
    q, k = bits_to_f32(inp["q_idx"]), bits_to_f32(inp["k_idx"])
    ref = oracle.dsa_indexer_scores(q, inp["w_idx"], k, inp["seq_lens"])
    check_scores(sc.cpu().numpy(), ref, indexer_bound(q, inp["w_idx"], k, inp["seq_lens"]), inp["seq_lens"])


def run_topk(ta, scores, lens, k):
    idx = ta.attn_topk(dev(scores.astype(np.float32)), dev(np.asarray(lens, np.int32)), k)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


@pytest.mark.parametrize("k", [1, 7, 64, 2048])
def test_topk_matches_oracle_selection(k):
    ta = require_gpu()
    rng = np.random.default_rng(62)
    lens = [3000, 1, 0, k, k + 1, 4096, 2 * k + 3]
    t = max(lens)
    sc = rng.standard_normal((len(lens), t)).astype(np.float32) * 100
    sc[:, ::5] = -sc[:, ::5]
    say(f"topk k={k} lens={lens}")
    got = run_topk(ta, sc, lens, k)
    np.testing.assert_array_equal(got, oracle.topk_indices(sc, lens, k))


def test_topk_ties_signed_zeros_and_infinities():
    """Heavy ties (few distinct values), -0.0 equal to +0.0, infinities: the lower index wins every tie."""
    ta = require_gpu()
    rng = np.random.default_rng(63)
    t = 5000
    lens = [t, t, t, 999]
    sc = np.zeros((4, t), np.float32)
    sc[0] = rng.integers(0, 7, t).astype(np.float32)                 # 7 distinct values
    sc[1] = np.where(rng.random(t) < 0.5, 0.0, -0.0).astype(np.float32)
    sc[1, 4000:] = 1.0
    sc[2] = rng.standard_normal(t).astype(np.float32)
    sc[2, rng.choice(t, 30, replace=False)] = np.inf
    sc[2, rng.choice(t, 30, replace=False)] = -np.inf
    sc[3] = 5.0                                                       # all equal
    for k in (1, 100, 999, 1000, 4999):
        got = run_topk(ta, sc, lens, k)
        ref = oracle.topk_indices(sc, lens, k)
        np.testing.assert_array_equal(got, ref, err_msg=f"k={k}")


def test_topk_nan_scores_rank_below_every_number():
    """NaN scores of either sign (several payloads) among numbers and infinities: every NaN ranks below -inf and
    NaNs tie among themselves (lower index first), index-exact against the oracle's selection on the same scores."""
    ta = require_gpu()
    rng = np.random.default_rng(64)
    t = 3000
    lens = [t, t, t, 40]
    sc = rng.standard_normal((4, t)).astype(np.float32)
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], np.uint32)   # +qNaN, -qNaN, sNaN, -NaN
    for b in range(3):
        pos = rng.choice(t, 200, replace=False)
        sc[b, pos] = nan_bits[rng.integers(0, 4, 200)].view(np.float32)
    sc[1, rng.choice(t, 50, replace=False)] = -np.inf
    sc[1, rng.choice(t, 50, replace=False)] = np.inf
    sc[2, :] = nan_bits[rng.integers(0, 4, t)].view(np.float32)                     # mostly NaN ...
    sc[2, rng.choice(t, 10, replace=False)] = -np.inf                                # ... a few -inf
    sc[3, :] = nan_bits[0].view(np.float32)
    sc[3, 7] = -np.inf
    for k in (1, 5, 100, 2799, 2800, 2801, 2990, 2999):
        say(f"topk NaN k={k}")
        got = run_topk(ta, sc, lens, k)
        ref = oracle.topk_indices(sc, lens, k)
        np.testing.assert_array_equal(got, ref, err_msg=f"k={k}")
    # no NaN is selected while numbers remain unselected
    got = run_topk(ta, sc, lens, 2800)
    assert not np.isnan(sc[0, got[0]]).any()


def test_topk_long_rows_in_rounds():
    """Rows longer than one register-resident round (32768 scores), with ties spread across rounds."""
    ta = require_gpu()
    rng = np.random.default_rng(69)
    lens = [70000, 32769, 32768, 65536]
    sc = rng.standard_normal((4, 70000)).astype(np.float32)
    sc[1] = rng.integers(0, 50, 70000).astype(np.float32)             # ties everywhere
    sc[3] = np.round(sc[3] * 4) / 4
    for k in (5, 2048, 40000):
        say(f"topk rounds k={k} lens={lens}")
        np.testing.assert_array_equal(run_topk(ta, sc, lens, k), oracle.topk_indices(sc, lens, k), err_msg=f"k={k}")


def run_sparse(ta, w, inp, idx):
    o, lse = ta.attn_mla_sparse_decode(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev_bf16(inp["c_kv"]),
                                       dev_bf16(inp["k_pe"]), dev(inp["seq_lens"]), dev(np.asarray(idx, np.int32)),
                                       w.scale, return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(o), lse.cpu().numpy()


def sparse_oracle(w, inp, idx):
    f = bits_to_f32
    return oracle.mla_sparse_decode(f(inp["q_lat"]), f(inp["q_pe"]), f(inp["c_kv"]), f(inp["k_pe"]), inp["seq_lens"],
                                    idx, w.scale)


@pytest.mark.parametrize("heads,topk", [(128, 256), (128, 100), (64, 70), (32, 1)])
def test_sparse_mla_small(heads, topk):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["dsa_decode_b32"], heads=heads)
    lens = [600, 37, 1, 0, 600]
    rng = np.random.default_rng(64)
    inp = dsa_inputs(w, seed=65, batch=len(lens), seqlen=600, seq_lens=lens)
    idx = np.full((len(lens), topk), -1, np.int32)
    for b, n in enumerate(lens):
        m = min(topk, n)
        idx[b, :m] = rng.choice(n, m, replace=False) if n else []
    idx[0, ::3] = -1                                                  # padding in the middle
    idx[4, 1::4] = 600 + np.arange(len(idx[4, 1::4]))                 # at and past the length: ignored
    if topk > 2:
        idx[4, 2] = idx[4, 0]                                         # a repeated token counts twice
    say(f"sparse mla heads={heads} topk={topk} lens={lens}")
    o, lse = run_sparse(ta, w, inp, idx)
    o_ref, lse_ref = sparse_oracle(w, inp, idx)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN, mask_inf=True)
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3]))          # nothing selected


def test_sparse_mla_reads_only_selected_tokens():
    """NaN in every token that is not selected (and in the slots past each length) changes no bit of the output."""
    ta = require_gpu()
    w = WORKLOADS["dsa_decode_b32"]
    lens = [500, 300]
    inp = dsa_inputs(w, seed=66, batch=2, seqlen=512, seq_lens=lens)
    rng = np.random.default_rng(67)
    idx = np.full((2, 200), -1, np.int32)
    idx[0] = rng.choice(500, 200, replace=False)
    idx[1, :150] = rng.choice(300, 150, replace=False)
    o1, l1 = run_sparse(ta, w, inp, idx)
    for b in range(2):
        keep = np.zeros(512, bool)
        keep[idx[b][(idx[b] >= 0)]] = True
        inp["c_kv"][b, ~keep] = NAN
        inp["k_pe"][b, ~keep] = NAN
    o2, l2 = run_sparse(ta, w, inp, idx)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_with_every_token_matches_dense_mla():
    ta = require_gpu()
    w = WORKLOADS["dsa_decode_b32"]
    lens = [777, 128]
    inp = dsa_inputs(w, seed=68, batch=2, seqlen=800, seq_lens=lens)
    idx = np.full((2, 800), -1, np.int32)
    for b, n in enumerate(lens):
        idx[b, :n] = np.random.default_rng(b).permutation(n)
    o_s, l_s = run_sparse(ta, w, inp, idx)
    o_d, l_d = ta.attn_mla_decode(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev_bf16(inp["c_kv"]),
                                  dev_bf16(inp["k_pe"]), dev(inp["seq_lens"]), w.scale, return_lse=True)
    torch.cuda.synchronize()
    check("sparse vs dense", bits_to_f32(o_s), bits_to_f32(host_bf16(o_d)), BF16_MAX, BF16_MEAN)
    check("lse", l_s, l_d.cpu().numpy(), BF16_MAX, BF16_MEAN)


def test_dsa_pipeline_full_size():
    """The workload in the bench's launch configuration: B=32, 32768 cached tokens each, 64 indexer heads of 128,
    top 2048, 128 MLA heads. Indexer scores checked on sampled sequences (fp64 oracle, fp32 bound), the top-k of
    every sequence bit-exact against the oracle's selection from the same scores, sparse attention on sampled
    sequences against the oracle over the selected tokens."""
    ta = require_gpu()
    w = WORKLOADS["dsa_decode_b32"]
    say(f"dsa full size B={w.batch} T={w.seqlen} topk={w.topk}")
    inp = dsa_inputs(w, seed=0)
    lens_d = dev(inp["seq_lens"])
    sc = ta.attn_dsa_indexer(dev_bf16(inp["q_idx"]), dev(inp["w_idx"]), dev_bf16(inp["k_idx"]), lens_d)
    idx = ta.attn_topk(sc, lens_d, w.topk)
    o, lse = ta.attn_mla_sparse_decode(dev_bf16(inp["q_lat"]), dev_bf16(inp["q_pe"]), dev_bf16(inp["c_kv"]),
                                       dev_bf16(inp["k_pe"]), lens_d, idx, w.scale, return_lse=True)
    torch.cuda.synchronize()
    sc, idx, o, lse = sc.cpu().numpy(), idx.cpu().numpy(), host_bf16(o), lse.cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.topk_indices(sc, inp["seq_lens"], w.topk))
    for b in (0, 17, 31):
        q, k = bits_to_f32(inp["q_idx"][b:b + 1]), bits_to_f32(inp["k_idx"][b:b + 1])
        ref = oracle.dsa_indexer_scores(q, inp["w_idx"][b:b + 1], k, inp["seq_lens"][b:b + 1])
        check_scores(sc[b:b + 1], ref, indexer_bound(q, inp["w_idx"][b:b + 1], k, inp["seq_lens"][b:b + 1]),
                     inp["seq_lens"][b:b + 1])
        sel = idx[b]
        f = bits_to_f32
        o_ref, lse_ref = oracle.mla_sparse_decode(f(inp["q_lat"][b:b + 1]), f(inp["q_pe"][b:b + 1]),
                                                  f(inp["c_kv"][b:b + 1]), f(inp["k_pe"][b:b + 1]),
                                                  inp["seq_lens"][b:b + 1], sel[None], w.scale)
        check_bf16(f"o seq {b}", o[b:b + 1], o_ref)
        check(f"lse seq {b}", lse[b:b + 1], lse_ref, BF16_MAX, BF16_MEAN)
