"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

Holds none of the method's arithmetic: it draws iid N(0, 1) values, rounds them to bfloat16 (round to nearest
even) or encodes them as 8-bit cache codes (FP8 E4M3 or int8, nearest-even, with per-channel scales), and builds
block tables, sequence lengths, positions and sampled rows. Every tensor has its own random
stream: numpy PCG64 seeded by SeedSequence(seed, spawn_key=(tensor id, chunk)), so values do not depend on how many
threads draw them. bf16 tensors are returned as their uint16 bit patterns, fp32 tensors as float32.
"""
from concurrent.futures import ThreadPoolExecutor
import os
import zlib

import numpy as np

from .workloads import Prefill, PagedDecode, MLADecode

_CHUNK = 1 << 22          # elements per independently seeded chunk


def _tensor_id(name):
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16, nearest-even, returning the uint16 bit pattern (inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_e4m3_bits(x):
    """Round float32 to the OCP FP8 E4M3 byte, nearest-even, saturating at +-448 (never produces the NaN code)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    sign = (x.view(np.uint32) >> np.uint32(24)) & np.uint32(0x80)
    a = np.abs(x)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = (u + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)           # float32 exponent and top 3 mantissa bits, rounded
    normal_code = np.minimum(r.astype(np.int64) - (120 << 3), 0x7E)  # rebias 127 -> 7; saturate at 448
    sub_code = np.rint(a * np.float32(512.0)).astype(np.int64)       # below 2^-6: m * 2^-9, m = 0..8
    code = np.where(a < np.float32(2.0 ** -6), sub_code, normal_code)
    return (code.astype(np.uint32) | sign).astype(np.uint8)


def f32_to_int8_bits(x):
    """Round float32 to int8, nearest-even, clipped to [-127, 127]; returned as the uint8 byte."""
    return np.clip(np.rint(np.asarray(x, np.float32)), -127, 127).astype(np.int8).view(np.uint8)


def normal(seed, name, shape, dtype, q8=None):
    """iid N(0, 1) of the given shape; dtype "bf16" -> uint16 bits, "fp32" -> float32. With q8 = (scale, kind) the
    values are divided by scale (broadcast over the trailing dimensions) and stored as 8-bit codes, kind "fp8"
    (E4M3) or "int8"."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint8 if q8 else (np.uint16 if dtype == "bf16" else np.float32))
    tid = _tensor_id(name)
    if q8:
        inv = (1.0 / np.asarray(q8[0], np.float64)).astype(np.float32).ravel()
        enc = f32_to_e4m3_bits if q8[1] == "fp8" else f32_to_int8_bits

    def fill(ci):
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, ci))))
        vals = rng.standard_normal(hi - lo, dtype=np.float32)
        if q8:
            out[lo:hi] = enc(vals * inv[np.arange(lo, hi) % inv.size])
        else:
            out[lo:hi] = f32_to_bf16_bits(vals) if dtype == "bf16" else vals

    n_chunks = (n + _CHUNK - 1) // _CHUNK
    if n_chunks <= 1:
        for ci in range(n_chunks):
            fill(ci)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _rng(seed, name):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_tensor_id(name),))))


def prefill_inputs(w: Prefill, seed=0, seqlen=None, batch=None):
    """q [B, S, Hq, D], k and v [B, S, Hkv, D]; positions [B*S] int32 (0..S-1 for each sequence).
    seqlen / batch override the workload's sizes (for scaled-down cases of the same shape family)."""
    s = w.seqlen if seqlen is None else seqlen
    b = w.batch if batch is None else batch
    q = normal(seed, "prefill.q", (b, s, w.hq, w.head_dim), w.dtype)
    k = normal(seed, "prefill.k", (b, s, w.hkv, w.head_dim), w.dtype)
    v = normal(seed, "prefill.v", (b, s, w.hkv, w.head_dim), w.dtype)
    positions = np.tile(np.arange(s, dtype=np.int32), b)
    return dict(q=q, k=k, v=v, positions=positions)


def sampled_rows(seqlen, n, seed=0):
    """n distinct query positions in [0, seqlen), always including the first and the last, sorted."""
    if n >= seqlen:
        return np.arange(seqlen, dtype=np.int64)
    rng = _rng(seed, "prefill.rows")
    inner = rng.choice(np.arange(1, seqlen - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, seqlen - 1], inner])).astype(np.int64)


def kv_scales(seed, w, kind):
    """Per-(KV head, channel) fp32 scales for an 8-bit cache of N(0,1) values: 4 / code_max times a seeded factor in
    [0.75, 1.25] (so about 4 standard deviations fill the code range), as k_scale, v_scale [Hkv, D]."""
    top = 448.0 if kind == "fp8" else 127.0
    f = _rng(seed, "decode.kv_scale").uniform(0.75, 1.25, size=(2, w.hkv, w.head_dim))
    return (4.0 / top * f).astype(np.float32)


def paged_decode_inputs(w: PagedDecode, seed=0, batch=None, seq_lens=None, page_size=None, max_len=None, kv="bf16"):
    """A paged KV cache placed by a seeded random block table.

    Returns dict with q [B, Hq, D] (not yet rotated), k_cache / v_cache [N_pool, page, Hkv, D], block_table
    [B, max_pages] int32 (-1 for unused entries), seq_lens [B] int32, positions [B] int32 (= seq_len - 1),
    spare_pages (physical pages no table references), max_len.
    Each sequence of length L needs ceil(L / page) pages; a seeded permutation of a pool of N_used + spares
    pages hands out distinct pages, never shared between sequences.
    """
    b = w.batch if batch is None else batch
    ps = w.page_size if page_size is None else page_size
    if seq_lens is None:
        seq_lens = _rng(seed, "decode.lens").integers(w.len_lo, w.len_hi, size=b, endpoint=True)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    b = seq_lens.size
    max_len = int(max(w.len_hi, seq_lens.max(initial=0)) if max_len is None else max_len)
    max_pages = max(1, (max_len + ps - 1) // ps)
    n_pages = (seq_lens.astype(np.int64) + ps - 1) // ps
    n_used = int(n_pages.sum())
    n_pool = n_used + int(np.ceil(n_used * w.spare_frac)) + 1
    perm = _rng(seed, "decode.perm").permutation(n_pool).astype(np.int32)
    table = np.full((b, max_pages), -1, dtype=np.int32)
    off = 0
    for i in range(b):
        table[i, : n_pages[i]] = perm[off: off + n_pages[i]]
        off += int(n_pages[i])
    spare = np.sort(perm[off:])
    q = normal(seed, "decode.q", (b, w.hq, w.head_dim), "bf16")
    out = dict(q=q, block_table=table, seq_lens=seq_lens, positions=(seq_lens - 1).astype(np.int32),
               spare_pages=spare, max_len=max_len)
    shape = (n_pool, ps, w.hkv, w.head_dim)
    if kv == "bf16":
        out.update(k_cache=normal(seed, "decode.k", shape, "bf16"), v_cache=normal(seed, "decode.v", shape, "bf16"))
    else:                     # 8-bit codes of the same N(0,1) draws, with per-channel scales
        sk, sv = kv_scales(seed, w, kv)
        out.update(k_cache=normal(seed, "decode.k", shape, None, q8=(sk, kv)),
                   v_cache=normal(seed, "decode.v", shape, None, q8=(sv, kv)), k_scale=sk, v_scale=sv, kv=kv)
    return out


def mla_scales(seed, w, kind):
    """Per-channel fp32 scales of an 8-bit latent cache of N(0,1) values: 4 / code_max times a seeded factor in
    [0.75, 1.25], as (c_scale [C], pe_scale [R])."""
    top = 448.0 if kind == "fp8" else 127.0
    f = _rng(seed, "mla.scale").uniform(0.75, 1.25, size=w.latent + w.rope)
    s = (4.0 / top * f).astype(np.float32)
    return s[: w.latent].copy(), s[w.latent:].copy()


def mla_inputs(w: MLADecode, seed=0, batch=None, seqlen=None, seq_lens=None, kv="bf16"):
    """q_lat [B, H, C], q_pe [B, H, R], c_kv [B, T, C], k_pe [B, T, R] (bf16 bits), seq_lens [B] int32.
    kv "fp8" / "int8": c_kv and k_pe hold 8-bit codes of the same draws divided by per-channel scales c_scale [C]
    and pe_scale [R] (also returned, with kv)."""
    b = w.batch if batch is None else batch
    t = w.seqlen if seqlen is None else seqlen
    q_lat = normal(seed, "mla.q_lat", (b, w.heads, w.latent), "bf16")
    q_pe = normal(seed, "mla.q_pe", (b, w.heads, w.rope), "bf16")
    lens = np.full(b, t, dtype=np.int32) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if kv == "bf16":
        c_kv = normal(seed, "mla.c_kv", (b, t, w.latent), "bf16")
        k_pe = normal(seed, "mla.k_pe", (b, t, w.rope), "bf16")
        return dict(q_lat=q_lat, q_pe=q_pe, c_kv=c_kv, k_pe=k_pe, seq_lens=lens)
    cs, ps = mla_scales(seed, w, kv)
    c_kv = normal(seed, "mla.c_kv", (b, t, w.latent), None, q8=(cs, kv))
    k_pe = normal(seed, "mla.k_pe", (b, t, w.rope), None, q8=(ps, kv))
    return dict(q_lat=q_lat, q_pe=q_pe, c_kv=c_kv, k_pe=k_pe, seq_lens=lens, c_scale=cs, pe_scale=ps, kv=kv)


def chunked_prefill_inputs(w, seed=0, ctx_lens=None, new_lens=None, page_size=None, hq=None, hkv=None,
                           head_dim=None):
    """A paged cache holding ctx_lens[b] tokens per sequence (already-rotated keys: the N(0,1) values), placed by a
    seeded random block table with room for the new tokens, plus the new tokens' q, k, v (not yet rotated).

    Returns dict with q [T, Hq, D], k_new / v_new [T, Hkv, D] (T = total new tokens, sequences packed in order),
    k_cache / v_cache [N_pool, page, Hkv, D], block_table [B, max_pages] int32 (-1 unused), cu_new [B+1],
    ctx_lens [B], positions [T] (absolute position of each new token), spare_pages, max_new.
    """
    ctx = np.asarray(w.ctx_lens if ctx_lens is None else ctx_lens, dtype=np.int32)
    new = np.asarray(w.new_lens if new_lens is None else new_lens, dtype=np.int32)
    ps = w.page_size if page_size is None else page_size
    hq = w.hq if hq is None else hq
    hkv = w.hkv if hkv is None else hkv
    d = w.head_dim if head_dim is None else head_dim
    b = ctx.size
    total = (ctx + new).astype(np.int64)
    n_pages = (total + ps - 1) // ps
    max_pages = max(1, int(n_pages.max(initial=1)))
    n_used = int(n_pages.sum())
    n_pool = n_used + int(np.ceil(n_used * w.spare_frac)) + 1
    perm = _rng(seed, "chunked.perm").permutation(n_pool).astype(np.int32)
    table = np.full((b, max_pages), -1, dtype=np.int32)
    off = 0
    for i in range(b):
        table[i, : n_pages[i]] = perm[off: off + n_pages[i]]
        off += int(n_pages[i])
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    t = int(cu[-1])
    positions = np.concatenate([np.arange(c, c + n) for c, n in zip(ctx, new)] or [np.zeros(0)]).astype(np.int32)
    return dict(q=normal(seed, "chunked.q", (t, hq, d), "bf16"),
                k_new=normal(seed, "chunked.k_new", (t, hkv, d), "bf16"),
                v_new=normal(seed, "chunked.v_new", (t, hkv, d), "bf16"),
                k_cache=normal(seed, "chunked.k", (n_pool, ps, hkv, d), "bf16"),
                v_cache=normal(seed, "chunked.v", (n_pool, ps, hkv, d), "bf16"),
                block_table=table, cu_new=cu, ctx_lens=ctx, positions=positions,
                spare_pages=np.sort(perm[off:]), max_new=int(new.max(initial=0)))


def dsa_inputs(w, seed=0, batch=None, seqlen=None, seq_lens=None):
    """The MLA decode inputs (q_lat, q_pe, c_kv, k_pe, seq_lens as mla_inputs) plus the lightning indexer's:
    q_idx [B, H_I, D_I] and k_idx [B, T, D_I] bf16 bits, head weights w_idx [B, H_I] float32; all iid N(0, 1)."""
    b = w.batch if batch is None else batch
    t = w.seqlen if seqlen is None else seqlen
    out = mla_inputs(w, seed=seed, batch=b, seqlen=t, seq_lens=seq_lens)
    out["q_idx"] = normal(seed, "dsa.q_idx", (b, w.idx_heads, w.idx_dim), "bf16")
    out["k_idx"] = normal(seed, "dsa.k_idx", (b, t, w.idx_dim), "bf16")
    out["w_idx"] = normal(seed, "dsa.w_idx", (b, w.idx_heads), "fp32")
    return out
