"""Plain fp64 attention, RoPE and MLA — the oracle (test infrastructure only; see the package docstring).

Everything is the plain definition written out: scores are materialised, the softmax takes two passes (max, then
exp-and-sum), RoPE is an explicit cos/sin rotation, the paged cache is gathered with an explicit loop over pages,
and MLA is computed either in its absorbed form as plain attention or naively through per-head up-projections.
Library primitives used as steps: numpy matmul, exp, log, sin, cos.

Pages cited (by title, as they appear on the web):
  [AN]  "Attention" notes, makinaruto.github.io (posts/nlp/llm_learning/attention): sections "FlashAttention",
        "online-softmax", "Page Attention", "Group-Query Attention", "Multi-Head Latent Attention", "RoPE".
  [LC]  "DeepSeek 32K to 256K long context" (tqpw.cn): §2.1 RoPE definition, §2.2 frequency code, §2.5 rope cache.
  [V3]  "DeepSeek-V3 attention guide: einsum vs manual optimisation" (dksg.cn): the naive and the absorbed
        score einsums quoted from the model's inference code.
  [AP]  "7 anti-patterns of DeepSeek attention optimisation" (lpnh.cn): §4.2 GQA cache reorder.
  [LC-SW] [LC] §4.1: hybrid sparse attention, a sliding window for the local neighbourhood plus a few global
        tokens (a leading token such as CLS, periodic anchors at a global sampling rate).
  [LC-KV] [LC] §2.5, KV-cache compression: keys and values stored as 8-bit integers with a per-channel scale.
  [AP-F8] [AP] §3.3: FP8 E4M3, whose largest finite value is 448.
  [AN-LI] the "Lighting Indexer" section of [AN]: DeepSeek Sparse Attention scores every earlier token with
        sum over indexer heads j of w_j * ReLU(q_j . k_s) and attends only the most relevant tokens.

Readings taken where the pages are silent or garbled:
  * online-softmax running max is max(m_old, m_c) ([AN] prints a minus sign inside the max);
  * the softmax scale multiplies the scores inside the softmax ([V3] "* softmax_scale" on the scores);
  * query head h reads KV head h // (Hq/Hkv) ([AN] GQA table: Q1..Q4 use K1,K1,K2,K2; [AP] repeat_interleave);
  * causal: key j is visible to query i iff j <= i (Sq == Sk);
  * RoPE pairs are adjacent (2i, 2i+1) by default ([LC] §2.1 views the last dim as (-1, 2)); the half-split
    pairing (i, i + D/2) is available with interleaved=False;
  * RoPE angle = position * theta**(-2i/D) computed directly from the integer position in fp64 ([LC] §2.5);
  * an empty key set (sequence length 0) gives O = 0 and lse = -inf;
  * chunked prefill from a paged cache: the new tokens of a sequence follow its cached ones, new token i sits at
    absolute position cache_len + i and sees keys 0 .. cache_len + i ([AN]: later tokens attend to all earlier
    ones; with fewer queries than keys the mask is aligned to the last query, the bottom-right corner); appended
    keys are rotated at that absolute position and values are copied unrotated;
  * the indexer ([AN-LI]) is taken literally: no scale and no rotation beyond what its inputs already carry, one
    key per token shared by all indexer heads, one weight per (query token, indexer head); "the most relevant
    tokens" are the top_k largest scores, ties broken towards the lower token index (the page names no rule);
    a sequence with at most top_k tokens keeps all of them; sparse attention is the absorbed MLA attention
    restricted to the selected tokens;
  * 8-bit KV caches ([LC-KV], [AP-F8]): a cached value is code * scale[kv_head, channel], the code being an int8
    (two's complement) or an OCP FP8 E4M3 byte (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal; no infinities, S.1111.111 is NaN) and the scale an fp32 per (KV head, channel) for K and for V;
    attention is then exactly decode_paged on the dequantised caches;
  * 8-bit MLA latent cache (the same passages, for the shared latent cache): c_kv and k_pe are stored as codes with
    one fp32 scale per latent channel (c_scale [C]) and per rope channel (pe_scale [R]), shared by every head and
    token; attention is exactly mla_decode on the dequantised caches;
  * local + global mask ([LC-SW]): key j is visible to query i iff j <= i and (i - j < window, or j < n_lead, or
    anchor_stride > 0 and j % anchor_stride == 0); window >= 1 (a query always sees itself); the global sampling
    rate is 1 / anchor_stride, and j = 0 is an anchor whenever anchor_stride > 0.
"""
import numpy as np

__all__ = [
    "bf16_bits_to_f64", "rope_inv_freq", "rope", "attention_prefill", "attention_prefill_rows", "gather_paged",
    "decode_paged", "mla_decode", "mla_naive", "kv_append_paged", "prefill_paged", "dsa_indexer_scores",
    "topk_indices", "mla_sparse_decode", "fp8_e4m3_decode", "int8_decode", "dequantize_kv", "decode_paged_q8",
    "local_global_visible", "attention_local_global", "attention_local_global_rows", "mla_decode_q8",
]


def bf16_bits_to_f64(bits):
    """Decode IEEE bfloat16 bit patterns (uint16) to float64, exactly: bf16 is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def rope_inv_freq(head_dim, theta):
    """[LC] §2.1: theta_i = theta ** (-2i/d) for i = 0 .. d/2 - 1 (the rotation frequency of pair i)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * i / np.float64(head_dim))


def rope(x, positions, theta, interleaved=True):
    """Rotary position embedding by explicit rotation ([LC] §2.1: each pair (a, b) is multiplied by the
    matrix [[cos, -sin], [sin, cos]] of angle position * theta_i).

    x: [..., H, D] float (token axes first, then head, then dim). positions: integer array broadcastable to
    x.shape[:-2]. Returns a new float64 array; nothing is rounded.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0, "RoPE needs an even head dimension"
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[..., None] * rope_inv_freq(d, theta)           # [..tokens.., D/2], integer position times frequency
    c = np.cos(ang)[..., None, :]                             # broadcast over the head axis
    s = np.sin(ang)[..., None, :]
    if interleaved:
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        a, b = x[..., : d // 2], x[..., d // 2:]
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty_like(x)
    if interleaved:
        out[..., 0::2], out[..., 1::2] = ra, rb
    else:
        out[..., : d // 2], out[..., d // 2:] = ra, rb
    return out


def _softmax_rows_then_v(s, v):
    """Two-pass softmax over the last axis of materialised scores s [R, T] (pass 1: row max; pass 2: exp and sum),
    then P @ v. Rows whose every score is -inf (no visible key) give O = 0 and lse = -inf.
    Returns (o [R, Dv], lse [R])."""
    m = np.max(s, axis=-1) if s.shape[-1] else np.full(s.shape[:-1], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])                           # exp(-inf) = 0 for masked keys
    l = e.sum(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p @ v, lse


def attention_prefill(q, k, v, causal, scale):
    """softmax(scale * Q K^T [+ causal mask]) V per (batch, query head), with S materialised ([AN] conventional
    tiled computation: S = Q K^T, P = softmax(S), O = P V).

    q: [B, S, Hq, D]; k, v: [B, S, Hkv, D] (any float; computed in float64). Query head h reads KV head
    h // (Hq // Hkv). Returns (o [B, S, Hq, D] float64, lse [B, Hq, S] float64 natural-log sum-exp).
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    bsz, s_len, hq, _ = q.shape
    hkv = k.shape[2]
    assert hq % hkv == 0
    grp = hq // hkv
    o = np.zeros(q.shape[:3] + (v.shape[-1],), np.float64)
    lse = np.zeros((bsz, hq, s_len), np.float64)
    mask = np.triu(np.ones((s_len, s_len), dtype=bool), k=1) if causal else None   # True where key j > query i
    for b in range(bsz):
        for h in range(hq):
            g = h // grp
            sc = scale * (q[b, :, h, :] @ k[b, :, g, :].T)    # [S, S] materialised
            if causal:
                sc[mask] = -np.inf
            o[b, :, h, :], lse[b, h, :] = _softmax_rows_then_v(sc, v[b, :, g, :])
    return o, lse


def attention_prefill_rows(q, k, v, rows, causal, scale):
    """attention_prefill restricted to the query positions `rows` (same rows for every batch and head); used where
    the full S x S score matrix is too large for the CPU. Returns (o [B, R, Hq, Dv], lse [B, Hq, R])."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    bsz, s_len, hq, _ = q.shape
    hkv = k.shape[2]
    grp = hq // hkv
    o = np.zeros((bsz, rows.size, hq, v.shape[-1]), np.float64)
    lse = np.zeros((bsz, hq, rows.size), np.float64)
    keys = np.arange(s_len)
    for b in range(bsz):
        for h in range(hq):
            g = h // grp
            sc = scale * (q[b, rows, h, :] @ k[b, :, g, :].T)  # [R, S]
            if causal:
                sc[keys[None, :] > rows[:, None]] = -np.inf
            o[b, :, h, :], lse[b, h, :] = _softmax_rows_then_v(sc, v[b, :, g, :])
    return o, lse


def gather_paged(cache, block_table_row, seq_len):
    """[AN] Page Attention: logical token t of a sequence lives in physical page block_table_row[t // page_size],
    slot t % page_size. cache: [num_pages, page_size, ...]. Returns the logical [seq_len, ...] view, gathered with
    an explicit loop over pages."""
    page_size = cache.shape[1]
    out = np.empty((seq_len,) + cache.shape[2:], dtype=cache.dtype)
    n_pages = (seq_len + page_size - 1) // page_size
    for j in range(n_pages):
        phys = int(block_table_row[j])
        n = min(page_size, seq_len - j * page_size)
        out[j * page_size: j * page_size + n] = cache[phys, :n]
    return out


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale):
    """One query token per sequence attending all seq_lens[b] cached tokens of a paged KV cache.

    q: [B, Hq, D] (already rotated); k_cache, v_cache: [num_pages, page_size, Hkv, D]; block_table:
    [B, max_pages] int; seq_lens: [B] int. Query head h reads KV head h // (Hq // Hkv).
    Returns (o [B, Hq, D] float64, lse [B, Hq] float64).
    """
    q = np.asarray(q, np.float64)
    bsz, hq, _ = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    o = np.zeros((bsz, hq, v_cache.shape[-1]), np.float64)
    lse = np.zeros((bsz, hq), np.float64)
    for b in range(bsz):
        n = int(seq_lens[b])
        kb = np.asarray(gather_paged(k_cache, block_table[b], n), np.float64)   # [L, Hkv, D]
        vb = np.asarray(gather_paged(v_cache, block_table[b], n), np.float64)
        for h in range(hq):
            g = h // grp
            sc = scale * (kb[:, g, :] @ q[b, h, :])[None, :]     # [1, L]
            ob, lb = _softmax_rows_then_v(sc, vb[:, g, :])
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def mla_decode(q_lat, q_pe, c_kv, k_pe, seq_lens, scale):
    """MLA decode in the absorbed form, written as plain attention ([V3] absorb-mode scores:
    scale * (q_nope . kv_cache + q_pe . pe_cache); [AN] MLA: the value up-projection folds into W^O, so the
    output stays in the latent space: O = P . c_kv).

    q_lat: [B, H, C] (query already projected into the latent space), q_pe: [B, H, R]; c_kv: [B, T, C],
    k_pe: [B, T, R] (one rope key shared by all heads, [AN] partial RoPE); seq_lens: [B].
    Every head uses key [c_kv ; k_pe] (C+R wide) and value c_kv. Returns (o [B, H, C], lse [B, H]).
    """
    q_lat = np.asarray(q_lat, np.float64); q_pe = np.asarray(q_pe, np.float64)
    c_kv = np.asarray(c_kv, np.float64); k_pe = np.asarray(k_pe, np.float64)
    bsz, nh, c = q_lat.shape
    o = np.zeros((bsz, nh, c), np.float64)
    lse = np.zeros((bsz, nh), np.float64)
    for b in range(bsz):
        n = int(seq_lens[b])
        keys = np.concatenate([c_kv[b, :n], k_pe[b, :n]], axis=-1)        # [L, C+R]
        qry = np.concatenate([q_lat[b], q_pe[b]], axis=-1)                  # [H, C+R]
        sc = scale * (qry @ keys.T)                                         # [H, L] materialised
        o[b], lse[b] = _softmax_rows_then_v(sc, c_kv[b, :n])
    return o, lse


def mla_naive(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, seq_lens, scale):
    """MLA with explicit per-head up-projections ([AN] MLA: K = C^KV W^K_up, V = C^KV W^V_up; partial RoPE
    concatenates a rotated part whose key is shared across heads; [V3] naive-mode score einsum over full keys).

    q_nope: [B, H, Dn], q_pe: [B, H, R], c_kv: [B, T, C], k_pe: [B, T, R], w_uk: [H, C, Dn], w_uv: [H, C, Dv].
    Head h: key_t = [c_kv_t W_uk[h] ; k_pe_t], value_t = c_kv_t W_uv[h], query [q_nope_h ; q_pe_h].
    Returns o [B, H, Dv].
    """
    q_nope = np.asarray(q_nope, np.float64); q_pe = np.asarray(q_pe, np.float64)
    c_kv = np.asarray(c_kv, np.float64); k_pe = np.asarray(k_pe, np.float64)
    w_uk = np.asarray(w_uk, np.float64); w_uv = np.asarray(w_uv, np.float64)
    bsz, nh, _ = q_nope.shape
    o = np.zeros((bsz, nh, w_uv.shape[-1]), np.float64)
    for b in range(bsz):
        n = int(seq_lens[b])
        for h in range(nh):
            k_h = np.concatenate([c_kv[b, :n] @ w_uk[h], k_pe[b, :n]], axis=-1)   # [L, Dn+R]
            v_h = c_kv[b, :n] @ w_uv[h]                                          # [L, Dv]
            q_h = np.concatenate([q_nope[b, h], q_pe[b, h]])
            sc = scale * (k_h @ q_h)[None, :]
            ob, _ = _softmax_rows_then_v(sc, v_h)
            o[b, h] = ob[0]
    return o


def kv_append_paged(k_cache, v_cache, block_table, cache_lens, k_new, v_new, cu_new, theta, interleaved=True):
    """Append new tokens to a paged KV cache ([AN] Page Attention: logical token t of a sequence lives in page
    block_table[b][t // page_size], slot t % page_size). New token i of sequence b (rows cu_new[b] .. cu_new[b+1]-1
    of k_new / v_new) has absolute position cache_lens[b] + i; its key is rotated at that position ([LC] §2.1, §2.5:
    the angle comes straight from the integer position) and its value is stored as is.

    k_cache, v_cache: [num_pages, page_size, Hkv, D]; k_new, v_new: [total_new, Hkv, D]; cu_new: [B+1];
    cache_lens: [B]. Returns new float64 caches (the inputs are not modified); slots not written keep their values.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    page_size = kc.shape[1]
    for b in range(len(cache_lens)):
        for row in range(int(cu_new[b]), int(cu_new[b + 1])):
            pos = int(cache_lens[b]) + row - int(cu_new[b])
            page, slot = int(block_table[b][pos // page_size]), pos % page_size
            kc[page, slot] = rope(np.asarray(k_new[row], np.float64)[None], np.array([pos]), theta, interleaved)[0]
            vc[page, slot] = v_new[row]
    return kc, vc


def prefill_paged(q, k_cache, v_cache, block_table, cu_new, cache_lens, scale):
    """Chunked / variable-length causal prefill against a paged KV cache that already holds, for each sequence b,
    its cache_lens[b] earlier tokens followed by its n_b = cu_new[b+1] - cu_new[b] new ones. The new tokens are the
    queries: query i of sequence b (row cu_new[b] + i of q, already rotated) sits at absolute position
    cache_lens[b] + i and sees keys 0 .. cache_lens[b] + i. Scores are materialised per (sequence, head).

    q: [total_new, Hq, D]; caches: [num_pages, page_size, Hkv, D]. Query head h reads KV head h // (Hq // Hkv).
    Returns (o [total_new, Hq, D] float64, lse [Hq, total_new] float64).
    """
    q = np.asarray(q, np.float64)
    total, hq, _ = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    o = np.zeros((total, hq, v_cache.shape[-1]), np.float64)
    lse = np.zeros((hq, total), np.float64)
    for b in range(len(cache_lens)):
        r0, r1 = int(cu_new[b]), int(cu_new[b + 1])
        n, ctx = r1 - r0, int(cache_lens[b])
        if n == 0:
            continue
        kb = np.asarray(gather_paged(k_cache, block_table[b], ctx + n), np.float64)    # [ctx + n, Hkv, D]
        vb = np.asarray(gather_paged(v_cache, block_table[b], ctx + n), np.float64)
        hidden = np.arange(ctx + n)[None, :] > (ctx + np.arange(n))[:, None]           # key after the query
        for h in range(hq):
            g = h // grp
            sc = scale * (q[r0:r1, h, :] @ kb[:, g, :].T)                               # [n, ctx + n]
            sc[hidden] = -np.inf
            o[r0:r1, h, :], lse[h, r0:r1] = _softmax_rows_then_v(sc, vb[:, g, :])
    return o, lse


def dsa_indexer_scores(q_idx, w, k_idx, seq_lens):
    """Lightning-indexer scores of one query token per sequence against every cached token ([AN-LI]):
    I[b, s] = sum_j w[b, j] * ReLU(q_idx[b, j] . k_idx[b, s]) for s < seq_lens[b], -inf past the length.

    q_idx: [B, H_I, D_I] (indexer queries), w: [B, H_I] (per-head weights), k_idx: [B, T, D_I] (one indexer key per
    token). Returns [B, T] float64.
    """
    q_idx = np.asarray(q_idx, np.float64); w = np.asarray(w, np.float64); k_idx = np.asarray(k_idx, np.float64)
    bsz, t = k_idx.shape[0], k_idx.shape[1]
    out = np.full((bsz, t), -np.inf)
    for b in range(bsz):
        n = int(seq_lens[b])
        dots = k_idx[b, :n] @ q_idx[b].T                  # [L, H_I]: q_j . k_s for every head and token
        out[b, :n] = np.maximum(dots, 0.0) @ w[b]         # weighted sum of the ReLU'd dots over the heads
    return out


def topk_indices(scores, seq_lens, k):
    """Indices of the k largest scores among the first seq_lens[b] of each row ([AN-LI]: keep the most relevant
    tokens). Ties at the cut go to the lower index. A NaN score (either sign) counts as less relevant than every
    number, -inf included, and NaNs tie among themselves (the page is silent; a NaN carries no relevance).
    All min(k, L) selected indices are returned in ascending order, the rest of the k slots hold -1.
    Returns int32 [B, k].
    """
    scores = np.asarray(scores)
    out = np.full((scores.shape[0], k), -1, np.int32)
    for b in range(scores.shape[0]):
        n = int(seq_lens[b])
        idx = np.arange(n)
        with np.errstate(invalid="ignore"):                 # signalling NaNs convert quietly
            sc = scores[b, :n].astype(np.float64)
        nan = np.isnan(sc)
        # numbers before NaNs, then by descending score, then by index (lexsort sorts by its last key first)
        order = np.lexsort((idx, -np.where(nan, 0.0, sc), nan))
        sel = np.sort(order[: min(k, n)])
        out[b, : sel.size] = sel
    return out


def mla_sparse_decode(q_lat, q_pe, c_kv, k_pe, seq_lens, indices, scale):
    """Absorbed MLA decode over the selected tokens only (DeepSeek Sparse Attention, [AN-LI]): for sequence b the
    keys and values are the rows indices[b, i] of its caches, for the entries with 0 <= index < seq_lens[b]
    (others, e.g. -1 padding, are ignored). Otherwise exactly mla_decode. Returns (o [B, H, C], lse [B, H]).
    """
    q_lat = np.asarray(q_lat, np.float64); q_pe = np.asarray(q_pe, np.float64)
    c_kv = np.asarray(c_kv, np.float64); k_pe = np.asarray(k_pe, np.float64)
    bsz, nh, c = q_lat.shape
    o = np.zeros((bsz, nh, c), np.float64)
    lse = np.zeros((bsz, nh), np.float64)
    for b in range(bsz):
        n = int(seq_lens[b])
        sel = np.array([int(i) for i in indices[b] if 0 <= int(i) < n], dtype=np.int64)
        keys = np.concatenate([c_kv[b, sel], k_pe[b, sel]], axis=-1)        # [n_sel, C+R], gathered rows
        qry = np.concatenate([q_lat[b], q_pe[b]], axis=-1)
        sc = scale * (qry @ keys.T)
        o[b], lse[b] = _softmax_rows_then_v(sc, c_kv[b, sel])
    return o, lse


def fp8_e4m3_decode(codes):
    """Value of each OCP FP8 E4M3 byte ([AP-F8]): bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
    e = 0 is subnormal (m/8 * 2^-6), otherwise (1 + m/8) * 2^(e-7); e = 15 with m = 7 is NaN (no infinities, so
    the largest finite value is 1.75 * 2^8 = 448). Returns float64."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def int8_decode(codes):
    """Value of each int8 byte (two's complement). Returns float64."""
    return np.asarray(codes, np.uint8).view(np.int8).astype(np.float64)


def dequantize_kv(codes, scale, kind):
    """8-bit cache [num_pages, page_size, Hkv, D] -> float64 values code * scale[kv_head, channel] ([LC-KV])."""
    dec = fp8_e4m3_decode(codes) if kind == "fp8" else int8_decode(codes)
    return dec * np.asarray(scale, np.float64)[None, None]


def decode_paged_q8(q, k_codes, v_codes, k_scale, v_scale, kind, block_table, seq_lens, scale):
    """Paged decode over 8-bit K/V caches: decode_paged on the dequantised caches. kind: "fp8" or "int8"."""
    return decode_paged(q, dequantize_kv(k_codes, k_scale, kind), dequantize_kv(v_codes, v_scale, kind), block_table,
                        seq_lens, scale)


def mla_decode_q8(q_lat, q_pe, c_codes, pe_codes, c_scale, pe_scale, kind, seq_lens, scale):
    """Absorbed MLA decode over an 8-bit latent cache: mla_decode on c_kv = code * c_scale[channel] and
    k_pe = code * pe_scale[channel] ([LC-KV], [AP-F8] applied to the latent cache). kind: "fp8" or "int8"."""
    dec = fp8_e4m3_decode if kind == "fp8" else int8_decode
    c_kv = dec(c_codes) * np.asarray(c_scale, np.float64)
    k_pe = dec(pe_codes) * np.asarray(pe_scale, np.float64)
    return mla_decode(q_lat, q_pe, c_kv, k_pe, seq_lens, scale)


def local_global_visible(rows, n_keys, window, n_lead, anchor_stride):
    """Boolean [len(rows), n_keys]: key j visible to query i ([LC-SW] reading above)."""
    i = np.asarray(rows, np.int64)[:, None]
    j = np.arange(n_keys)[None, :]
    glob = j < n_lead
    if anchor_stride > 0:
        glob = glob | (j % anchor_stride == 0)
    return (j <= i) & ((i - j < window) | glob)


def attention_local_global_rows(q, k, v, rows, window, n_lead, anchor_stride, scale):
    """Causal attention with the local + global mask for the query positions `rows`, scores materialised.
    q: [B, S, Hq, D]; k, v: [B, S, Hkv, D]. Returns (o [B, R, Hq, Dv], lse [B, Hq, R])."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    bsz, s_len, hq, _ = q.shape
    grp = hq // k.shape[2]
    hidden = ~local_global_visible(rows, s_len, window, n_lead, anchor_stride)
    o = np.zeros((bsz, rows.size, hq, v.shape[-1]), np.float64)
    lse = np.zeros((bsz, hq, rows.size), np.float64)
    for b in range(bsz):
        for h in range(hq):
            g = h // grp
            sc = scale * (q[b, rows, h, :] @ k[b, :, g, :].T)        # [R, S] materialised
            sc[hidden] = -np.inf
            o[b, :, h, :], lse[b, h, :] = _softmax_rows_then_v(sc, v[b, :, g, :])
    return o, lse


def attention_local_global(q, k, v, window, n_lead, anchor_stride, scale):
    """attention_local_global_rows over every query position. Returns (o [B, S, Hq, Dv], lse [B, Hq, S])."""
    return attention_local_global_rows(q, k, v, np.arange(np.asarray(q).shape[1]), window, n_lead, anchor_stride,
                                       scale)
