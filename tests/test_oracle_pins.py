"""Pins for the fp64 oracle: each check ties it to something other than itself — values the pages print, closed
forms, brute force on tiny inputs, invariants the mathematics fixes, and a library routine in a special case.
Chosen so that a dropped term, a wrong sign or index, or a transposed operand anywhere in the oracle fails one.
CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------------------------------- RoPE ----

def test_rope_frequencies_match_printed_formula():
    with open(os.path.join(GOLDEN, "rope_frequencies.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        np.testing.assert_allclose(oracle.rope_inv_freq(case["d"], case["base"]), case["inv_freq"], rtol=1e-15)


def test_rope_pair_angles_closed_form():
    # D = 8, base 10000: pair i rotates by p * 10**(-i). A unit vector (1, 0) in every pair lands on (cos, sin).
    x = np.zeros((1, 1, 8)); x[..., 0::2] = 1.0
    for p in (0, 1, 3, 255, 131071):
        y = oracle.rope(x, np.array([p]), 10000.0)[0, 0]
        for i in range(4):
            a = p * 10.0 ** (-i)
            assert abs(y[2 * i] - math.cos(a)) < 1e-12 and abs(y[2 * i + 1] - math.sin(a)) < 1e-12, (p, i)


def test_rope_d2_is_rotation_matrix():
    x = rnd(1, 5, 3, 2)
    pos = np.array([0, 1, 7, 1000, 131071])
    y = oracle.rope(x, pos, 10000.0)
    for t, p in enumerate(pos):
        c, s = math.cos(p), math.sin(p)
        r = np.array([[c, -s], [s, c]])
        np.testing.assert_allclose(y[t], x[t] @ r.T, atol=1e-13)


def test_rope_position_zero_is_identity():
    x = rnd(2, 4, 3, 64)
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(4, int), 10000.0), x)


def test_rope_preserves_norm():
    x = rnd(3, 6, 2, 128)
    pos = np.array([0, 5, 300, 8191, 65536, 131071])
    for inter in (True, False):
        y = oracle.rope(x, pos, 40889.94, interleaved=inter)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 128)); k = rng.standard_normal((1, 1, 128))
    for _ in range(10):
        m, n, s = (int(v) for v in rng.integers(0, 131072, 3))
        for theta in (10000.0, WORKLOADS["gqa_prefill_s131072"].theta):
            for inter in (True, False):
                a = np.sum(oracle.rope(q, [m], theta, inter) * oracle.rope(k, [n], theta, inter))
                b = np.sum(oracle.rope(q, [m + s], theta, inter) * oracle.rope(k, [n + s], theta, inter))
                assert abs(a - b) < 1e-8 * (1 + abs(a)), (m, n, s)


def test_rope_half_split_is_a_permutation_of_interleaved():
    # Pairing (i, i + D/2) equals pairing (2i, 2i+1) after moving element i -> 2i and i + D/2 -> 2i + 1.
    d = 16
    x = rnd(5, 3, 2, d)
    perm = np.empty(d, int); perm[0::2] = np.arange(d // 2); perm[1::2] = np.arange(d // 2) + d // 2
    pos = np.array([1, 17, 4000])
    np.testing.assert_allclose(oracle.rope(x[..., perm], pos, 10000.0, True),
                               oracle.rope(x, pos, 10000.0, False)[..., perm], atol=1e-14)


def test_ntk_base_closed_form():
    assert abs(WORKLOADS["gqa_prefill_s131072"].theta - 40889.94243248622) < 1e-8


# ------------------------------------------------------------------------------------------ softmax/attention ----

def brute_attention(q, k, v, causal, scale):
    """Nested loops; exp without max subtraction; p = exp(s) / sum exp(s)."""
    bsz, s_len, hq, _ = q.shape
    hkv = k.shape[2]
    o = np.zeros(q.shape[:3] + (v.shape[-1],)); lse = np.zeros((bsz, hq, s_len))
    for b in range(bsz):
        for h in range(hq):
            g = h * hkv // hq
            for i in range(s_len):
                w = []
                for j in range(k.shape[1]):
                    if causal and j > i:
                        w.append(0.0)
                        continue
                    w.append(math.exp(scale * sum(q[b, i, h, d] * k[b, j, g, d] for d in range(q.shape[-1]))))
                tot = sum(w)
                lse[b, h, i] = math.log(tot)
                for j in range(k.shape[1]):
                    o[b, i, h] += (w[j] / tot) * v[b, j, g]
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_prefill_matches_brute_force(causal, hq, hkv):
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 5, hq, 3)); k = rng.standard_normal((2, 5, hkv, 3)); v = rng.standard_normal((2, 5, hkv, 4))
    o, lse = oracle.attention_prefill(q, k, v, causal, 0.7)
    ob, lb = brute_attention(q, k, v, causal, 0.7)
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_allclose(lse, lb, atol=1e-13)


def online_softmax_attention(q, k, v, causal, scale, tiles):
    """Independent fp64 implementation of the page's online-softmax recurrence (block max m_c, block exp-sum l_c;
    m_new = max(m_old, m_c); l_new = l_old e^(m_old-m_new) + l_c e^(m_c-m_new)), with the output accumulator
    rescaled by the same factors and divided by l at the end."""
    bsz, s_len, hq, _ = q.shape
    hkv = k.shape[2]
    o = np.zeros(q.shape[:3] + (v.shape[-1],)); lse = np.zeros((bsz, hq, s_len))
    for b in range(bsz):
        for h in range(hq):
            g = h * hkv // hq
            for i in range(s_len):
                m, l, acc = -np.inf, 0.0, np.zeros(v.shape[-1])
                j0 = 0
                for t in tiles:
                    j1 = min(j0 + t, s_len)
                    if j0 >= j1:
                        break
                    s = np.array([scale * q[b, i, h] @ k[b, j, g] if (not causal or j <= i) else -np.inf
                                  for j in range(j0, j1)])
                    m_c = s.max()
                    if np.isfinite(m_c):
                        e = np.exp(s - m_c)
                        l_c = e.sum()
                        m_new = max(m, m_c)
                        a_old = math.exp(m - m_new) if np.isfinite(m) else 0.0
                        a_c = math.exp(m_c - m_new)
                        l = l * a_old + l_c * a_c
                        acc = acc * a_old + a_c * (e @ v[b, j0:j1, g])
                        m = m_new
                    j0 = j1
                o[b, i, h] = acc / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_online_recurrence_equals_two_pass(causal):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 37, 4, 8)) * 2; k = rng.standard_normal((1, 37, 2, 8)); v = rng.standard_normal((1, 37, 2, 8))
    o, lse = oracle.attention_prefill(q, k, v, causal, 0.9)
    for trial in range(3):
        tiles = list(rng.integers(1, 12, size=40))
        o2, l2 = online_softmax_attention(q, k, v, causal, 0.9, tiles)
        np.testing.assert_allclose(o, o2, atol=1e-12)
        np.testing.assert_allclose(lse, l2, atol=1e-12)


def test_rows_of_p_sum_to_one_and_respect_mask():
    # With V = identity (value j = e_j) the output row is the probability row itself.
    s_len = 9
    q = rnd(8, 1, s_len, 2, 4); k = rnd(9, 1, s_len, 2, 4)
    v = np.broadcast_to(np.eye(s_len)[None, :, None, :], (1, s_len, 2, s_len)).copy()
    p, _ = oracle.attention_prefill(q, k, v, True, 1.3)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    assert (p >= 0).all()
    for i in range(s_len):
        assert np.all(p[0, i, :, i + 1:] == 0.0)


def test_constant_v_gives_constant_o():
    q = rnd(10, 2, 11, 4, 8); k = rnd(11, 2, 11, 2, 8)
    c = rnd(12, 8)
    v = np.broadcast_to(c, (2, 11, 2, 8)).copy()
    o, _ = oracle.attention_prefill(q, k, v, True, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)


def test_causal_row_zero_is_v0():
    q = rnd(13, 1, 6, 4, 8); k = rnd(14, 1, 6, 2, 8); v = rnd(15, 1, 6, 2, 8)
    o, lse = oracle.attention_prefill(q, k, v, True, 0.35)
    for h in range(4):
        np.testing.assert_array_equal(o[0, 0, h], v[0, 0, h // 2])
        assert abs(lse[0, h, 0] - 0.35 * q[0, 0, h] @ k[0, 0, h // 2]) < 1e-14


def test_large_query_along_a_key_selects_its_value():
    k = np.zeros((1, 4, 1, 4)); k[0, :, 0, :] = np.eye(4)
    v = rnd(16, 1, 4, 1, 5)
    q = np.zeros((1, 4, 1, 4)); q[0, 3, 0, 2] = 60.0         # last query points at key 2
    o, _ = oracle.attention_prefill(q, k, v, True, 1.0)
    np.testing.assert_allclose(o[0, 3, 0], v[0, 2, 0], atol=1e-20 + 1e-24)


def test_gqa_head_mapping_matches_printed_examples():
    with open(os.path.join(GOLDEN, "gqa_head_mapping.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        hq, hkv = case["hq"], case["hkv"]
        q = rnd(17, 1, 3, hq, 4); k = rnd(18, 1, 3, hkv, 4)
        v = np.zeros((1, 3, hkv, 1))
        for g in range(hkv):
            v[:, :, g, 0] = 10.0 * (g + 1)                      # each KV head carries a distinct constant
        o, _ = oracle.attention_prefill(q, k, v, True, 1.0)
        got = [int(round(o[0, 2, h, 0] / 10.0)) - 1 for h in range(hq)]
        assert got == case["kv_of_q"], case["cite"]


def test_gqa_equals_mha_on_repeated_kv():
    q = rnd(19, 2, 7, 8, 8); k = rnd(20, 2, 7, 2, 8); v = rnd(21, 2, 7, 2, 8)
    o, lse = oracle.attention_prefill(q, k, v, True, 0.4)
    o2, lse2 = oracle.attention_prefill(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), True, 0.4)
    np.testing.assert_allclose(o, o2, atol=1e-15); np.testing.assert_allclose(lse, lse2, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_torch_sdpa_fp64(causal):
    torch = pytest.importorskip("torch")
    q = rnd(22, 2, 19, 8, 16); k = rnd(23, 2, 19, 2, 16); v = rnd(24, 2, 19, 2, 16)
    o, _ = oracle.attention_prefill(q, k, v, causal, 0.3)
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(np.repeat(k, 4, axis=2)).transpose(1, 2)
    tv = torch.from_numpy(np.repeat(v, 4, axis=2)).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), atol=1e-12)


def test_prefill_rows_equals_full():
    q = rnd(25, 2, 40, 4, 8); k = rnd(26, 2, 40, 2, 8); v = rnd(27, 2, 40, 2, 8)
    o, lse = oracle.attention_prefill(q, k, v, True, 0.6)
    rows = np.array([0, 3, 17, 39])
    o_r, lse_r = oracle.attention_prefill_rows(q, k, v, rows, True, 0.6)
    np.testing.assert_allclose(o_r, o[:, rows], atol=1e-14); np.testing.assert_allclose(lse_r, lse[:, :, rows], atol=1e-14)


def test_lse_merge_of_key_splits_equals_unsplit():
    """Split the keys into random chunks, attend each chunk separately (normalised O_c, lse_c), merge:
    M = max lse_c, w_c = exp(lse_c - M), O = sum w_c O_c / sum w_c, lse = M + log sum w_c."""
    rng = np.random.default_rng(28)
    L = 50
    q = rng.standard_normal((1, 1, 4, 8)) * 3; k = rng.standard_normal((1, L, 2, 8)); v = rng.standard_normal((1, L, 2, 8))
    o_full, lse_full = oracle.attention_prefill(q, k, v, False, 0.8)
    cuts = np.sort(rng.choice(np.arange(1, L), 5, replace=False))
    bounds = [0, *cuts, L]
    parts = [oracle.attention_prefill(q, k[:, a:b], v[:, a:b], False, 0.8) for a, b in zip(bounds[:-1], bounds[1:])]
    lses = np.stack([p[1] for p in parts])                      # [C, 1, H, 1]
    outs = np.stack([p[0] for p in parts])                      # [C, 1, 1, H, D]
    mx = lses.max(axis=0)
    w = np.exp(lses - mx)
    o = (w.transpose(0, 1, 3, 2)[..., None] * outs).sum(0) / w.sum(0).transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(o, o_full, atol=1e-13)
    np.testing.assert_allclose(mx + np.log(w.sum(0)), lse_full, atol=1e-13)


# ------------------------------------------------------------------------------------------------ paged decode ----

def _paged_layout(k_dense, v_dense, page, rng, n_spare=3):
    """Scatter dense [L, Hkv, D] K/V into a randomly permuted page pool; returns caches and a one-row table."""
    L = k_dense.shape[0]
    n_pages = (L + page - 1) // page
    pool = n_pages + n_spare
    perm = rng.permutation(pool)
    kc = rng.standard_normal((pool, page) + k_dense.shape[1:]) * 100
    vc = rng.standard_normal((pool, page) + v_dense.shape[1:]) * 100
    for j in range(n_pages):
        n = min(page, L - j * page)
        kc[perm[j], :n] = k_dense[j * page: j * page + n]
        vc[perm[j], :n] = v_dense[j * page: j * page + n]
    table = np.full((1, n_pages + 2), -1); table[0, :n_pages] = perm[:n_pages]
    return kc, vc, table


def test_decode_equals_last_row_of_causal_prefill():
    rng = np.random.default_rng(29)
    for L in (1, 5, 16, 37):
        k = rng.standard_normal((L, 2, 8)); v = rng.standard_normal((L, 2, 8)); qd = rng.standard_normal((4, 8))
        kc, vc, table = _paged_layout(k, v, 8, rng)
        o, lse = oracle.decode_paged(qd[None], kc, vc, table, np.array([L]), 0.5)
        qfull = np.zeros((1, L, 4, 8)); qfull[0, L - 1] = qd
        o_ref, lse_ref = oracle.attention_prefill_rows(qfull, k[None], v[None], [L - 1], True, 0.5)
        np.testing.assert_allclose(o[0], o_ref[0, 0], atol=1e-13); np.testing.assert_allclose(lse[0], lse_ref[0, :, 0], atol=1e-13)


def test_decode_is_independent_of_page_placement():
    rng = np.random.default_rng(30)
    k = rng.standard_normal((45, 2, 8)); v = rng.standard_normal((45, 2, 8)); qd = rng.standard_normal((1, 4, 8))
    outs = []
    for s in range(3):
        kc, vc, table = _paged_layout(k, v, 16, np.random.default_rng(100 + s))
        outs.append(oracle.decode_paged(qd, kc, vc, table, np.array([45]), 0.5)[0])
    np.testing.assert_array_equal(outs[0], outs[1]); np.testing.assert_array_equal(outs[0], outs[2])


def test_decode_length_one_gives_v0_and_brute_force():
    rng = np.random.default_rng(31)
    kc = rng.standard_normal((4, 8, 2, 4)); vc = rng.standard_normal((4, 8, 2, 4)); q = rng.standard_normal((2, 4, 4))
    table = np.array([[2, -1, -1], [3, 0, 1]])
    o, lse = oracle.decode_paged(q, kc, vc, table, np.array([1, 19]), 0.9)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], vc[2, 0, h // 2])
    # brute force for sequence 1: token t at page table[1][t // 8], slot t % 8
    for h in range(4):
        w = [math.exp(0.9 * q[1, h] @ kc[table[1, t // 8], t % 8, h // 2]) for t in range(19)]
        ref = sum(wi * vc[table[1, t // 8], t % 8, h // 2] for t, wi in enumerate(w)) / sum(w)
        np.testing.assert_allclose(o[1, h], ref, atol=1e-13)
        assert abs(lse[1, h] - math.log(sum(w))) < 1e-13


def test_empty_key_set_gives_zero_and_minus_inf():
    kc = np.ones((2, 4, 1, 4)); vc = np.ones((2, 4, 1, 4)); q = np.ones((1, 2, 4))
    o, lse = oracle.decode_paged(q, kc, vc, np.array([[0, 1]]), np.array([0]), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------------------------------------ chunked prefill from pages ----

def _paged_multi(seqs_k, seqs_v, page, rng, n_spare=4):
    """Scatter dense per-sequence K/V [L_b, Hkv, D] into one randomly permuted pool of distinct pages (junk
    elsewhere); returns caches and the block table (-1 past each sequence's pages)."""
    n_pages = [(k.shape[0] + page - 1) // page for k in seqs_k]
    pool = sum(n_pages) + n_spare
    perm = rng.permutation(pool)
    kc = rng.standard_normal((pool, page) + seqs_k[0].shape[1:]) * 100
    vc = rng.standard_normal((pool, page) + seqs_v[0].shape[1:]) * 100
    table = np.full((len(seqs_k), max(n_pages) + 1), -1)
    used = 0
    for b, (k, v) in enumerate(zip(seqs_k, seqs_v)):
        for j in range(n_pages[b]):
            phys = perm[used]; used += 1
            n = min(page, k.shape[0] - j * page)
            kc[phys, :n] = k[j * page: j * page + n]
            vc[phys, :n] = v[j * page: j * page + n]
            table[b, j] = phys
    return kc, vc, table


CHUNKS = [(0, 7), (5, 1), (13, 11), (20, 20), (8, 9)]    # (cached tokens, new tokens) per sequence


def _chunked_case(seed, hq=4, hkv=2, d=8, page=8):
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((c + n, hkv, d)) for c, n in CHUNKS]
    vs = [rng.standard_normal((c + n, hkv, d)) for c, n in CHUNKS]
    qs = [rng.standard_normal((c + n, hq, d)) for c, n in CHUNKS]
    kc, vc, table = _paged_multi(ks, vs, page, rng)
    cu = np.concatenate([[0], np.cumsum([n for _, n in CHUNKS])])
    ctx = np.array([c for c, _ in CHUNKS])
    q_new = np.concatenate([qs[b][c:] for b, (c, _) in enumerate(CHUNKS)])
    return ks, vs, qs, kc, vc, table, cu, ctx, q_new


def test_chunked_prefill_equals_tail_rows_of_full_prefill():
    # The last n of c + n tokens as queries against all c + n keys are rows c .. c+n-1 of the ordinary causal
    # prefill over the whole sequence (where the mask j <= i is exact because Sq == Sk).
    ks, vs, qs, kc, vc, table, cu, ctx, q_new = _chunked_case(40)
    o, lse = oracle.prefill_paged(q_new, kc, vc, table, cu, ctx, 0.6)
    for b, (c, n) in enumerate(CHUNKS):
        o_ref, lse_ref = oracle.attention_prefill(qs[b][None], ks[b][None], vs[b][None], True, 0.6)
        np.testing.assert_allclose(o[cu[b]:cu[b + 1]], o_ref[0, c:], atol=1e-12)
        np.testing.assert_allclose(lse[:, cu[b]:cu[b + 1]], lse_ref[0, :, c:], atol=1e-12)


def test_chunked_prefill_of_one_new_token_is_decode():
    rng = np.random.default_rng(41)
    lens = [1, 9, 17, 33]
    ks = [rng.standard_normal((L, 2, 8)) for L in lens]; vs = [rng.standard_normal((L, 2, 8)) for L in lens]
    kc, vc, table = _paged_multi(ks, vs, 8, rng)
    q = rng.standard_normal((len(lens), 4, 8))
    o, lse = oracle.prefill_paged(q, kc, vc, table, np.arange(len(lens) + 1), np.array(lens) - 1, 0.7)
    o_d, lse_d = oracle.decode_paged(q, kc, vc, table, np.array(lens), 0.7)
    np.testing.assert_allclose(o, o_d, atol=1e-13)
    np.testing.assert_allclose(lse, lse_d.T, atol=1e-13)


def test_chunked_prefill_brute_force_tiny():
    # explicit loops: 3 cached + 2 new tokens, one KV head shared by 2 query heads, keys after the query hidden
    rng = np.random.default_rng(42)
    k = rng.standard_normal((5, 1, 4)); v = rng.standard_normal((5, 1, 4)); q = rng.standard_normal((2, 2, 4))
    kc, vc, table = _paged_multi([k], [v], 4, rng)
    o, lse = oracle.prefill_paged(q, kc, vc, table, np.array([0, 2]), np.array([3]), 0.9)
    for i in range(2):
        for h in range(2):
            w = [math.exp(0.9 * q[i, h] @ k[j, 0]) for j in range(3 + i + 1)]
            ref = sum(wj * v[j, 0] for j, wj in enumerate(w)) / sum(w)
            np.testing.assert_allclose(o[i, h], ref, atol=1e-13)
            assert abs(lse[h, i] - math.log(sum(w))) < 1e-13


def test_chunked_prefill_with_no_new_tokens_leaves_other_rows():
    ks, vs, qs, kc, vc, table, cu, ctx, q_new = _chunked_case(43)
    cu2 = np.concatenate([cu[:2], cu[1:]])             # insert an empty sequence after the first one
    table2 = np.concatenate([table[:1], table[:1], table[1:]])
    ctx2 = np.concatenate([ctx[:1], [4], ctx[1:]])
    o, lse = oracle.prefill_paged(q_new, kc, vc, table, cu, ctx, 0.5)
    o2, lse2 = oracle.prefill_paged(q_new, kc, vc, table2, cu2, ctx2, 0.5)
    np.testing.assert_array_equal(o, o2); np.testing.assert_array_equal(lse, lse2)


def test_kv_append_places_rotated_keys_at_absolute_positions():
    rng = np.random.default_rng(44)
    page, hkv, d, theta = 8, 2, 8, 500.0
    ctx = np.array([0, 6, 13]); n = np.array([5, 9, 3])
    dense_k = [rng.standard_normal((c, hkv, d)) for c in ctx]; dense_v = [rng.standard_normal((c, hkv, d)) for c in ctx]
    # reserve pages for the final lengths; the cached prefix is already in place
    full = [np.concatenate([dk, np.zeros((m, hkv, d))]) for dk, m in zip(dense_k, n)]
    kc, vc, table = _paged_multi(full, [np.concatenate([dv, np.zeros((m, hkv, d))]) for dv, m in zip(dense_v, n)],
                                 page, rng)
    k_new = rng.standard_normal((n.sum(), hkv, d)); v_new = rng.standard_normal((n.sum(), hkv, d))
    cu = np.concatenate([[0], np.cumsum(n)])
    kc2, vc2 = oracle.kv_append_paged(kc, vc, table, ctx, k_new, v_new, cu, theta)
    for b in range(3):
        L = ctx[b] + n[b]
        kg = oracle.gather_paged(kc2, table[b], L); vg = oracle.gather_paged(vc2, table[b], L)
        np.testing.assert_array_equal(kg[:ctx[b]], dense_k[b]); np.testing.assert_array_equal(vg[:ctx[b]], dense_v[b])
        # one vectorised rotation of the whole new block at positions ctx .. ctx+n-1
        np.testing.assert_allclose(kg[ctx[b]:], oracle.rope(k_new[cu[b]:cu[b + 1]], np.arange(ctx[b], L), theta),
                                   atol=1e-14)
        np.testing.assert_array_equal(vg[ctx[b]:], v_new[cu[b]:cu[b + 1]])
    used = set(table[table >= 0].tolist())
    for p in range(kc.shape[0]):
        if p not in used:
            np.testing.assert_array_equal(kc2[p], kc[p]); np.testing.assert_array_equal(vc2[p], vc[p])


def test_kv_append_in_two_chunks_equals_one():
    rng = np.random.default_rng(45)
    kc = rng.standard_normal((6, 4, 1, 4)); vc = rng.standard_normal((6, 4, 1, 4))
    table = np.array([[4, 1, 5, 0]])
    k_new = rng.standard_normal((9, 1, 4)); v_new = rng.standard_normal((9, 1, 4))
    one = oracle.kv_append_paged(kc, vc, table, np.array([3]), k_new, v_new, np.array([0, 9]), 1000.0)
    a = oracle.kv_append_paged(kc, vc, table, np.array([3]), k_new[:4], v_new[:4], np.array([0, 4]), 1000.0)
    two = oracle.kv_append_paged(a[0], a[1], table, np.array([7]), k_new[4:], v_new[4:], np.array([0, 5]), 1000.0)
    np.testing.assert_array_equal(one[0], two[0]); np.testing.assert_array_equal(one[1], two[1])


# ------------------------------------------------------------------------------------------------------ MLA ----

def test_mla_absorbed_equals_naive_up_projection():
    rng = np.random.default_rng(32)
    B, H, C, R, Dn, Dv, T = 2, 3, 16, 4, 6, 5, 11
    q_nope = rng.standard_normal((B, H, Dn)); q_pe = rng.standard_normal((B, H, R))
    c_kv = rng.standard_normal((B, T, C)); k_pe = rng.standard_normal((B, T, R))
    w_uk = rng.standard_normal((H, C, Dn)) * 0.3; w_uv = rng.standard_normal((H, C, Dv))
    lens = np.array([T, 7])
    o_naive = oracle.mla_naive(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, lens, 0.4)
    q_lat = np.einsum("hcn,bhn->bhc", w_uk, q_nope)                  # W^K_up absorbed into the query
    o_lat, _ = oracle.mla_decode(q_lat, q_pe, c_kv, k_pe, lens, 0.4)
    o_abs = np.einsum("bhc,hcv->bhv", o_lat, w_uv)                   # W^V_up applied after attention
    np.testing.assert_allclose(o_abs, o_naive, atol=1e-12)


def test_mla_scores_match_printed_absorb_einsums():
    """The absorbed scores written with the page's own einsum index strings, then a softmax and P.c_kv."""
    rng = np.random.default_rng(33)
    B, H, C, R, T = 2, 4, 12, 3, 9
    q_nope = rng.standard_normal((B, 1, H, C)); q_pe = rng.standard_normal((B, 1, H, R))
    kv = rng.standard_normal((B, T, C)); pe = rng.standard_normal((B, T, R))
    scores = (np.einsum("bshc,btc->bsht", q_nope, kv) + np.einsum("bshr,btr->bsht", q_pe, pe)) * 0.25
    p = np.exp(scores - scores.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
    ref = np.einsum("bsht,btc->bshc", p, kv)[:, 0]
    o, _ = oracle.mla_decode(q_nope[:, 0], q_pe[:, 0], kv, pe, np.array([T, T]), 0.25)
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_mla_zero_rope_key_is_single_kv_head_attention():
    rng = np.random.default_rng(34)
    B, H, C, R, T = 2, 4, 16, 4, 13
    q_lat = rng.standard_normal((B, H, C)); q_pe = rng.standard_normal((B, H, R)); c_kv = rng.standard_normal((B, T, C))
    o, lse = oracle.mla_decode(q_lat, q_pe, c_kv, np.zeros((B, T, R)), np.array([T, T]), 0.3)
    o_ref, lse_ref = oracle.attention_prefill(q_lat[:, None], c_kv[:, :, None], c_kv[:, :, None], False, 0.3)
    np.testing.assert_allclose(o, o_ref[:, 0], atol=1e-13); np.testing.assert_allclose(lse, lse_ref[:, :, 0], atol=1e-13)


def test_mla_zero_query_averages_latent_cache():
    rng = np.random.default_rng(35)
    c_kv = rng.standard_normal((2, 10, 16)); k_pe = rng.standard_normal((2, 10, 4))
    o, lse = oracle.mla_decode(np.zeros((2, 3, 16)), np.zeros((2, 3, 4)), c_kv, k_pe, np.array([10, 6]), 0.5)
    np.testing.assert_allclose(o[0], np.broadcast_to(c_kv[0].mean(0), (3, 16)), atol=1e-14)
    np.testing.assert_allclose(o[1], np.broadcast_to(c_kv[1, :6].mean(0), (3, 16)), atol=1e-14)
    np.testing.assert_allclose(lse[1], math.log(6), atol=1e-14)


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625                                        # 0x4049 = 1.5703125 * 2
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127                      # largest finite bf16
    assert vals[5] == 2.0 ** -133                                     # smallest subnormal bf16


# ------------------------------------------------------------------------------ DSA indexer, top-k, sparse MLA ----

def test_indexer_brute_force_loops():
    """The page's formula with explicit loops: sum over heads j of w_j * max(0, sum_d q_jd * k_sd)."""
    rng = np.random.default_rng(50)
    B, H, D, T = 2, 3, 4, 6
    q = rng.standard_normal((B, H, D)); w = rng.standard_normal((B, H)); k = rng.standard_normal((B, T, D))
    lens = np.array([6, 4])
    got = oracle.dsa_indexer_scores(q, w, k, lens)
    for b in range(B):
        for s in range(T):
            if s >= lens[b]:
                assert got[b, s] == -np.inf
                continue
            ref = 0.0
            for j in range(H):
                dot = sum(q[b, j, d] * k[b, s, d] for d in range(D))
                ref += w[b, j] * (dot if dot > 0 else 0.0)
            assert abs(got[b, s] - ref) < 1e-13


def test_indexer_relu_and_weights():
    # one head with w = 1 is ReLU(q . k); a head whose dots are all negative contributes nothing; w is linear
    rng = np.random.default_rng(51)
    q = rng.standard_normal((1, 1, 8)); k = rng.standard_normal((1, 20, 8))
    got = oracle.dsa_indexer_scores(q, np.ones((1, 1)), k, [20])
    np.testing.assert_allclose(got[0], np.maximum(k[0] @ q[0, 0], 0), atol=1e-14)
    q2 = np.concatenate([q, np.zeros_like(q)], axis=1)          # second head: q = 0, so ReLU(q . k) = 0
    got2 = oracle.dsa_indexer_scores(q2, np.array([[1.0, 5.0]]), k, [20])
    np.testing.assert_allclose(got2, got, atol=1e-14)
    w = rng.standard_normal((1, 2)); qq = rng.standard_normal((1, 2, 8))
    a = oracle.dsa_indexer_scores(qq, w, k, [20]); b2 = oracle.dsa_indexer_scores(qq, -2.5 * w, k, [20])
    np.testing.assert_allclose(b2, -2.5 * a, atol=1e-13)
    # heads are an unordered sum: permuting heads together with their weights changes nothing
    perm = [1, 0]
    np.testing.assert_allclose(oracle.dsa_indexer_scores(qq[:, perm], w[:, perm], k, [20]), a, atol=1e-13)


def test_topk_distinct_values_is_argsort():
    rng = np.random.default_rng(52)
    x = rng.standard_normal((3, 50))
    lens = np.array([50, 30, 7])
    got = oracle.topk_indices(x, lens, 10)
    for b in range(3):
        ref = np.sort(np.argsort(-x[b, :lens[b]], kind="stable")[:10])
        n = min(10, lens[b])
        np.testing.assert_array_equal(got[b, :n], ref)
        assert np.all(got[b, n:] == -1)
        sel = np.zeros(lens[b], bool); sel[got[b, :n]] = True
        if n < lens[b]:
            assert x[b, :lens[b]][sel].min() > x[b, :lens[b]][~sel].max()


def test_topk_ties_and_short_rows():
    x = np.array([[3.0, 1.0, 3.0, 3.0, 0.0, 7.0], [2.0, 2.0, 2.0, 2.0, 2.0, 2.0]])
    got = oracle.topk_indices(x, [5, 6], 3)
    np.testing.assert_array_equal(got[0], [0, 2, 3])           # 7.0 is past the length; three 3.0 ties fill it
    np.testing.assert_array_equal(got[1], [0, 1, 2])           # all equal: the lowest indices
    got = oracle.topk_indices(x, [2, 0], 4)
    np.testing.assert_array_equal(got[0], [0, 1, -1, -1])      # fewer tokens than k: all of them
    np.testing.assert_array_equal(got[1], [-1, -1, -1, -1])


def test_topk_nan_ranks_below_every_number():
    """Reading: a NaN score is less relevant than any number, -inf included; NaNs tie (lower index first)."""
    nan, inf = np.nan, np.inf
    x = np.array([[nan, -inf, 2.0, -nan, inf, nan, -1.0]])
    np.testing.assert_array_equal(oracle.topk_indices(x, [7], 2), [[2, 4]])
    np.testing.assert_array_equal(oracle.topk_indices(x, [7], 4), [[1, 2, 4, 6]])          # -inf before any NaN
    np.testing.assert_array_equal(oracle.topk_indices(x, [7], 5), [[0, 1, 2, 4, 6]])       # first NaN by index
    np.testing.assert_array_equal(oracle.topk_indices(x, [7], 6), [[0, 1, 2, 3, 4, 6]])
    y = np.full((1, 5), nan)
    np.testing.assert_array_equal(oracle.topk_indices(y, [5], 2), [[0, 1]])                 # all NaN: lowest indices


def _mla_case(seed, B=2, H=3, C=16, R=4, T=12):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, C)), rng.standard_normal((B, H, R)), rng.standard_normal((B, T, C)),
            rng.standard_normal((B, T, R)))


def test_sparse_mla_with_every_token_is_dense():
    q_lat, q_pe, c_kv, k_pe = _mla_case(53)
    lens = np.array([12, 5])
    idx = np.array([np.arange(12), np.concatenate([np.arange(5), -np.ones(7, int)])])
    o, lse = oracle.mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, lens, idx, 0.35)
    o_ref, lse_ref = oracle.mla_decode(q_lat, q_pe, c_kv, k_pe, lens, 0.35)
    np.testing.assert_allclose(o, o_ref, atol=1e-13); np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


def test_sparse_mla_equals_dense_on_a_compacted_cache():
    q_lat, q_pe, c_kv, k_pe = _mla_case(54)
    lens = np.array([12, 9])
    idx = np.array([[7, 2, 11, -1, 0, 40], [8, 3, 9, 5, -1, 1]])  # unordered, padding, entries at / past the length
    o, lse = oracle.mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, lens, idx, 0.35)
    for b in range(2):
        keep = [i for i in idx[b] if 0 <= i < lens[b]]
        ck = np.zeros((1, len(keep), c_kv.shape[2])); kp = np.zeros((1, len(keep), k_pe.shape[2]))
        for j, i in enumerate(keep):                              # explicit copy of the selected rows
            ck[0, j] = c_kv[b, i]; kp[0, j] = k_pe[b, i]
        o_ref, lse_ref = oracle.mla_decode(q_lat[b:b + 1], q_pe[b:b + 1], ck, kp, [len(keep)], 0.35)
        np.testing.assert_allclose(o[b], o_ref[0], atol=1e-13); np.testing.assert_allclose(lse[b], lse_ref[0], atol=1e-13)
    # the order of the index list does not matter
    o2, _ = oracle.mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, lens, idx[:, ::-1], 0.35)
    np.testing.assert_allclose(o2, o, atol=1e-13)


def test_sparse_mla_with_nothing_selected_is_empty():
    q_lat, q_pe, c_kv, k_pe = _mla_case(55)
    o, lse = oracle.mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, np.array([12, 3]), np.array([[-1, -1], [5, 7]]), 0.3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_dsa_pipeline_with_large_k_is_dense_mla():
    # top_k >= L keeps every token, so indexer -> top-k -> sparse attention is dense MLA whatever the scores are
    q_lat, q_pe, c_kv, k_pe = _mla_case(56)
    rng = np.random.default_rng(57)
    lens = np.array([12, 10])
    sc = oracle.dsa_indexer_scores(rng.standard_normal((2, 4, 8)), rng.standard_normal((2, 4)),
                                   rng.standard_normal((2, 12, 8)), lens)
    idx = oracle.topk_indices(sc, lens, 16)
    o, _ = oracle.mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, lens, idx, 0.3)
    o_ref, _ = oracle.mla_decode(q_lat, q_pe, c_kv, k_pe, lens, 0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)


# ---------------------------------------------------------------------------------------------- 8-bit KV ----

def test_fp8_e4m3_printed_maximum_and_closed_forms():
    v = oracle.fp8_e4m3_decode
    assert v([0x7E])[0] == 448.0 and v([0xFE])[0] == -448.0          # the largest finite E4M3 value the page prints
    assert v([0x38])[0] == 1.0 and v([0x40])[0] == 2.0 and v([0x30])[0] == 0.5
    assert v([0x08])[0] == 2.0 ** -6 and v([0x01])[0] == 2.0 ** -9    # smallest normal, smallest subnormal
    assert v([0x07])[0] == 7 * 2.0 ** -9                              # largest subnormal
    assert np.isnan(v([0x7F])[0]) and np.isnan(v([0xFF])[0])
    assert v([0x80])[0] == 0.0 and np.signbit(v([0x80])[0])


def test_fp8_e4m3_all_codes_match_torch_and_are_monotone():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    pos = got[:0x7F]                                                   # 0x00 .. 0x7E increase strictly
    assert np.all(np.diff(pos) > 0)


def test_int8_decode_is_twos_complement():
    np.testing.assert_array_equal(oracle.int8_decode([0, 1, 127, 128, 255, 0x81]), [0, 1, 127, -128, -1, -127])


def test_q8_decode_scales_are_per_channel_and_linear():
    """Scaling K's channel d by s_d equals scaling the query's channel d; scaling V's channel d scales output
    channel d; with unit scales the 8-bit decode is decode_paged on the decoded codes."""
    rng = np.random.default_rng(70)
    B, Hq, Hkv, D, page, T = 2, 4, 2, 8, 4, 10
    lens = np.array([10, 7])
    kc = rng.integers(0, 256, (6, page, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0, 256, (6, page, Hkv, D)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C                                       # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    table = np.array([[0, 3, 5], [1, 4, -1]], np.int32)
    q = rng.standard_normal((B, Hq, D))
    ones = np.ones((Hkv, D))
    sk = rng.uniform(0.01, 0.1, (Hkv, D)); sv = rng.uniform(0.01, 0.1, (Hkv, D))
    for kind in ("fp8", "int8"):
        dec = oracle.fp8_e4m3_decode if kind == "fp8" else oracle.int8_decode
        o1, l1 = oracle.decode_paged_q8(q, kc, vc, ones, ones, kind, table, lens, 0.3)
        o2, l2 = oracle.decode_paged(q, dec(kc), dec(vc), table, lens, 0.3)
        np.testing.assert_array_equal(o1, o2); np.testing.assert_array_equal(l1, l2)
        # K scale == query scaled per channel by the scale of its KV head
        o3, l3 = oracle.decode_paged_q8(q, kc, vc, sk, ones, kind, table, lens, 0.3)
        qs = q * sk[np.arange(Hq) // (Hq // Hkv)][None]
        o4, l4 = oracle.decode_paged_q8(qs, kc, vc, ones, ones, kind, table, lens, 0.3)
        np.testing.assert_allclose(o3, o4, atol=1e-13); np.testing.assert_allclose(l3, l4, atol=1e-13)
        # V scale == output scaled per channel
        o5, _ = oracle.decode_paged_q8(q, kc, vc, ones, sv, kind, table, lens, 0.3)
        np.testing.assert_allclose(o5, o1 * sv[np.arange(Hq) // (Hq // Hkv)][None], atol=1e-13)


def test_mla_q8_single_token_and_constant_value_closed_forms():
    """One token: the output is its dequantised latent row (softmax over one key is 1), per channel. Identical
    latent rows: the output is that row whatever the scores. FP8 0x38 = 1, 0x40 = 2, 0xC4 = -3; int8 codes are the
    integers; distinct per-channel scales catch a misplaced or transposed scale."""
    C, R, H = 6, 2, 3
    rng = np.random.default_rng(71)
    q_lat = rng.standard_normal((1, H, C)); q_pe = rng.standard_normal((1, H, R))
    cs = np.array([0.5, 0.25, 2.0, 1.5, 0.75, 3.0]); ps = np.array([0.1, 0.2])
    row8 = np.array([0x38, 0x40, 0xC4, 0x38, 0x40, 0xC4], np.uint8)          # 1, 2, -3, 1, 2, -3
    row_i = np.array([1, 2, -3, 1, 2, -3], np.int8).view(np.uint8)
    want = np.array([1, 2, -3, 1, 2, -3]) * cs
    pe = rng.integers(0, 0x70, (1, 5, R)).astype(np.uint8)                     # finite codes (FP8 and int8)
    for kind, row in (("fp8", row8), ("int8", row_i)):
        o, _ = oracle.mla_decode_q8(q_lat, q_pe, row[None, None], pe[:, :1], cs, ps, kind, [1], 0.2)
        np.testing.assert_allclose(o[0], np.broadcast_to(want, (H, C)), rtol=0, atol=1e-15)
        o, _ = oracle.mla_decode_q8(q_lat, q_pe, np.repeat(row[None, None], 5, axis=1), pe, cs, ps, kind, [5], 0.2)
        np.testing.assert_allclose(o[0], np.broadcast_to(want, (H, C)), rtol=0, atol=1e-13)


def test_mla_q8_rope_scale_sits_on_the_scores():
    """Two tokens, zero latent query: the scores are scale * q_pe . (code * pe_scale), so the weights are a
    two-way softmax written out by hand."""
    C, R = 4, 2
    q_lat = np.zeros((1, 1, C)); q_pe = np.array([[[1.5, -0.5]]])
    cs = np.ones(C); ps = np.array([0.7, 0.3])
    c = np.array([[[0x38, 0x38, 0x38, 0x38], [0x40, 0xC4, 0x38, 0x40]]], np.uint8)   # rows (1,1,1,1), (2,-3,1,2)
    pe = np.array([[[0x40, 0x38], [0xC4, 0x40]]], np.uint8)                             # (2, 1), (-3, 2)
    o, lse = oracle.mla_decode_q8(q_lat, q_pe, c, pe, cs, ps, "fp8", [2], 0.5)
    s0 = 0.5 * (1.5 * 2 * 0.7 - 0.5 * 1 * 0.3)
    s1 = 0.5 * (1.5 * -3 * 0.7 - 0.5 * 2 * 0.3)
    w0, w1 = np.exp(s0), np.exp(s1)
    want = (w0 * np.array([1, 1, 1, 1]) + w1 * np.array([2, -3, 1, 2])) / (w0 + w1)
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(w0 + w1), rtol=1e-14)


# --------------------------------------------------------------------------------------- local + global mask ----

def _lg_case(seed, B=1, S=40, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)), rng.standard_normal((B, S, Hkv, D))


def test_local_global_reduces_to_causal():
    q, k, v = _lg_case(90)
    ref = oracle.attention_prefill(q, k, v, True, 0.4)
    for w, g, p in [(40, 0, 0), (1000, 3, 7), (1, 40, 0), (1, 0, 1), (5, 0, 1)]:   # window >= S, all lead, stride 1
        o, lse = oracle.attention_local_global(q, k, v, w, g, p, 0.4)
        np.testing.assert_allclose(o, ref[0], atol=1e-13); np.testing.assert_allclose(lse, ref[1], atol=1e-13)


def test_window_one_sees_only_itself():
    q, k, v = _lg_case(91)
    o, lse = oracle.attention_local_global(q, k, v, 1, 0, 0, 0.4)
    grp = q.shape[2] // k.shape[2]
    for h in range(q.shape[2]):
        np.testing.assert_allclose(o[0, :, h], v[0, :, h // grp], atol=1e-14)
        np.testing.assert_allclose(lse[0, h], 0.4 * np.einsum("sd,sd->s", q[0, :, h], k[0, :, h // grp]), atol=1e-13)


def test_local_global_mask_brute_force():
    """Explicit loops over (i, j) with the rule written out, softmax with exp and no max subtraction."""
    q, k, v = _lg_case(92, S=23, Hq=2, Hkv=1, D=4)
    W, G, P = 4, 2, 5
    o, lse = oracle.attention_local_global(q, k, v, W, G, P, 0.5)
    for i in range(23):
        for h in range(2):
            num, den = np.zeros(4), 0.0
            for j in range(23):
                if j <= i and (i - j < W or j < G or j % P == 0):
                    e = math.exp(0.5 * float(q[0, i, h] @ k[0, j, 0]))
                    num += e * v[0, j, 0]; den += e
            np.testing.assert_allclose(o[0, i, h], num / den, atol=1e-12)
            assert abs(lse[0, h, i] - math.log(den)) < 1e-12


def test_local_global_visible_counts():
    # the page's hybrid configuration: window 32 with global sampling rate 1/32 on a 512-token sequence
    vis = oracle.local_global_visible(np.arange(512), 512, 32, 0, 32)
    i = 511
    assert vis[i].sum() == 32 + len([j for j in range(0, 512 - 32) if j % 32 == 0])      # window + 15 anchors
    assert vis[i, 0] and vis[i, 32] and not vis[i, 33] and vis[i, 480] and vis[i, 511] and not vis[i, 479]
    assert np.all(vis.sum(1) >= 1) and np.all(np.diag(vis))
