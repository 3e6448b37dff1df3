"""Thin Python binding over libattn's C ABI (include/attn.h), with the same entry-point names.

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C ABI. PyTorch
provides device memory and the current stream. If libattn.so is missing or cannot be loaded, every call raises
(there is no fallback path).
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_BF16, ATTN_FP32 = 0, 1
ATTN_KV_FP8_E4M3, ATTN_KV_INT8 = 1, 2
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_WORKSPACE",
          4: "ATTN_ERR_HIP"}

# (name, restype, argtypes) for every symbol include/attn.h declares.
_P, _I, _I64, _D, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_rope_apply": (_I, [_P, _I, _I64, _I, _I, _P, _D, _I, _P]),
    "attn_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_rope_table": (_I, [_P, _I, _I, _D, _P]),
    "attn_prefill_rope": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _I, _P]),
    "attn_prefill_local_global": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_decode_paged_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _I, _F, _P, _SZ, _P]),
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _I, _F, _P]),
    "attn_decode_paged_q8": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _I, _F, _P, _SZ,
                                  _P]),
    "attn_mla_decode_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "attn_mla_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "attn_mla_decode_q8": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "attn_kv_append_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _D, _I, _P]),
    "attn_prefill_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I64, _F, _P]),
    "attn_prefill_paged_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I64, _F, _P,
                                     _P, _I, _I, _P]),
    "attn_dsa_indexer": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_topk": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "attn_mla_sparse_decode_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "attn_mla_sparse_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
}


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None


def load_library(path=LIB_PATH):
    """Load libattn.so (once) and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m transformer_attention_causal_amd.build` "
                           "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise AttnError(fn, status)


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name):
    """Raise unless tensor t has exactly this shape (the kernels index every buffer by the sizes passed)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _code(dtype):
    if dtype == torch.bfloat16:
        return ATTN_BF16
    if dtype == torch.float32:
        return ATTN_FP32
    raise ValueError(f"unsupported dtype {dtype}")


def attn_rope_apply(x, positions, theta, interleaved=True, stream=None):
    """Rotate x ([..., H, D], bf16 or fp32, contiguous) in place; positions: int32 [prod(x.shape[:-2])]."""
    lib = load_library()
    n_tokens = x.numel() // (x.shape[-1] * x.shape[-2]) if x.dim() >= 2 else 0
    if positions.numel() != n_tokens:
        raise ValueError("positions must have one entry per token row")
    _check("attn_rope_apply", lib.attn_rope_apply(_dev(x, "x"), _code(x.dtype), n_tokens, x.shape[-2], x.shape[-1],
                                                   _dev(positions, "positions", torch.int32), float(theta),
                                                   1 if interleaved else 0, _stream(x, stream)))
    return x


def attn_prefill(q, k, v, causal=True, softmax_scale=None, o=None, lse=None, return_lse=False, stream=None):
    """q [B, S, Hq, D], k/v [B, S, Hkv, D] (bf16 or fp32) -> o [B, S, Hq, D] (and lse [B, Hq, S] fp32)."""
    lib = load_library()
    bsz, s_len, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (bsz, s_len, hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, S, Hkv, D] with q's dtype")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq, s_len), dtype=torch.float32, device=q.device)
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq, s_len), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_prefill", lib.attn_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o", q.dtype), lse_p,
                                             _code(q.dtype), bsz, s_len, hq, hkv, d, 1 if causal else 0, scale,
                                             _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_rope_table(n_positions, head_dim, theta, device=None, table=None, stream=None):
    """(cos, sin) fp32 table [n_positions, head_dim/2, 2] of the rotation by integer position (the values
    attn_rope_apply uses)."""
    lib = load_library()
    if table is None:
        table = torch.empty((n_positions, head_dim // 2, 2), dtype=torch.float32,
                            device=device if device is not None else "cuda")
    _check("attn_rope_table", lib.attn_rope_table(_dev(table, "table", torch.float32) if table.numel() else None,
                                                   int(n_positions), int(head_dim), float(theta),
                                                   _stream(table, stream)))
    return table


def attn_prefill_rope(q, k, v, rope_table, q_positions=None, interleaved=True, causal=True, softmax_scale=None,
                      o=None, lse=None, return_lse=False, stream=None):
    """attn_prefill (bf16) with q UNROTATED: each query is rotated as the kernel loads it, by the cos/sin of its
    position (q_positions int32 [B*S], or 0..S-1 per sequence when None) from rope_table [n_pos, D/2, 2] fp32.
    k must be rotated already. Returns o [B, S, Hq, D] (and lse [B, Hq, S])."""
    lib = load_library()
    bsz, s_len, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (bsz, s_len, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, S, Hkv, D]")
    if rope_table.dim() != 3 or rope_table.shape[1:] != (d // 2, 2):
        raise ValueError("rope_table must be [n_positions, head_dim/2, 2]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq, s_len), dtype=torch.float32, device=q.device)
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq, s_len), "lse")
    if q_positions is not None and q_positions.numel() != bsz * s_len:
        raise ValueError("q_positions must have one entry per query row (B*S)")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    pos_p = _dev(q_positions, "q_positions", torch.int32) if q_positions is not None else None
    _check("attn_prefill_rope", lib.attn_prefill_rope(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        _dev(o, "o", torch.bfloat16), lse_p, bsz, s_len, hq, hkv, d, 1 if causal else 0, scale, pos_p,
        _dev(rope_table, "rope_table", torch.float32), rope_table.shape[0], 1 if interleaved else 0,
        _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_prefill_local_global(q, k, v, window, n_lead=0, anchor_stride=0, softmax_scale=None, o=None, lse=None,
                              return_lse=False, stream=None):
    """Causal prefill with a local + global mask: q [B, S, Hq, D], k/v [B, S, Hkv, D] bf16 -> o [B, S, Hq, D]
    (and lse [B, Hq, S]). Key j is visible to query i iff j <= i and (i - j < window or j < n_lead or
    (anchor_stride > 0 and j % anchor_stride == 0))."""
    lib = load_library()
    bsz, s_len, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (bsz, s_len, hkv, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes do not match")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq, s_len), dtype=torch.float32, device=q.device)
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq, s_len), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_prefill_local_global", lib.attn_prefill_local_global(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
        _dev(o, "o", torch.bfloat16), lse_p, bsz, s_len, hq, hkv, d, int(window), int(n_lead), int(anchor_stride),
        scale, _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_decode_paged_workspace_size(batch, n_heads_q, head_dim, max_seqlen_kv):
    return int(load_library().attn_decode_paged_workspace_size(batch, n_heads_q, head_dim, max_seqlen_kv))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, max_seqlen_kv, softmax_scale=None, o=None,
                      lse=None, workspace=None, return_lse=False, stream=None):
    """q [B, Hq, D] bf16 (rotated); caches [num_pages, page, Hkv, D] bf16; block_table [B, max_pages] int32;
    seq_lens [B] int32 (device). Returns o [B, Hq, D] bf16 (and lse [B, Hq] fp32)."""
    lib = load_library()
    bsz, hq, d = q.shape
    num_pages, page, hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    need = attn_decode_paged_workspace_size(bsz, hq, d, max(1, int(max_seqlen_kv)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if k_cache.dim() != 4 or k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_pages, page, Hkv, D] with q's D")
    if block_table.dim() != 2 or block_table.shape[0] != bsz or tuple(seq_lens.shape) != (bsz,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_decode_paged", lib.attn_decode_paged(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(o, "o", torch.bfloat16), lse_p, bsz, hq, hkv, d, page, block_table.shape[1], num_pages,
        int(max_seqlen_kv), scale, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(q, stream)))
    return (o, lse) if return_lse else o


DECODE_SCRATCH_BYTES = 64 << 20     # ATTN_DECODE_SCRATCH_BYTES


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seqlen_kv, softmax_scale=None, o=None,
                              lse=None, return_lse=False, stream=None):
    """attn_decode_paged with the library's static per-GPU scratch instead of a workspace (no device allocation in
    the call; pass o and lse to allocate nothing here either). Calls that overlap on one GPU race on the scratch."""
    lib = load_library()
    bsz, hq, d = q.shape
    num_pages, page, hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    if k_cache.dim() != 4 or k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_pages, page, Hkv, D] with q's D")
    if block_table.dim() != 2 or block_table.shape[0] != bsz or tuple(seq_lens.shape) != (bsz,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_decode_paged_noalloc", lib.attn_decode_paged_noalloc(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(o, "o", torch.bfloat16), lse_p, bsz, hq, hkv, d, page, block_table.shape[1], num_pages,
        int(max_seqlen_kv), scale, _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_mla_decode_workspace_size(batch, n_heads, kv_lora_rank, max_seqlen_kv):
    return int(load_library().attn_mla_decode_workspace_size(batch, n_heads, kv_lora_rank, max_seqlen_kv))


def attn_mla_decode(q_latent, q_pe, c_kv, k_pe, seq_lens, softmax_scale, o=None, lse=None, workspace=None,
                    return_lse=False, stream=None):
    """q_latent [B, H, C], q_pe [B, H, R], c_kv [B, T, C], k_pe [B, T, R] bf16; seq_lens [B] int32 (device).
    Returns o_latent [B, H, C] bf16 (and lse [B, H] fp32)."""
    lib = load_library()
    bsz, nh, c = q_latent.shape
    r = q_pe.shape[-1]
    t = c_kv.shape[1]
    if o is None:
        o = torch.empty_like(q_latent)
    if lse is None and return_lse:
        lse = torch.empty((bsz, nh), dtype=torch.float32, device=q_latent.device)
    need = attn_mla_decode_workspace_size(bsz, nh, c, max(1, t))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_latent.device)
    if q_pe.shape[:2] != (bsz, nh) or c_kv.shape[0] != bsz or c_kv.shape[2] != c or k_pe.shape != (bsz, t, r):
        raise ValueError("q_pe [B, H, R], c_kv [B, T, C] and k_pe [B, T, R] must agree with q_latent [B, H, C]")
    if tuple(seq_lens.shape) != (bsz,):
        raise ValueError("seq_lens must be [B]")
    _shape(o, q_latent.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, nh), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_mla_decode", lib.attn_mla_decode(
        _dev(q_latent, "q_latent", torch.bfloat16), _dev(q_pe, "q_pe", torch.bfloat16),
        _dev(c_kv, "c_kv", torch.bfloat16), _dev(k_pe, "k_pe", torch.bfloat16),
        _dev(seq_lens, "seq_lens", torch.int32), _dev(o, "o_latent", torch.bfloat16), lse_p, bsz, nh, c, r, t,
        float(softmax_scale), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(q_latent, stream)))
    return (o, lse) if return_lse else o


def attn_mla_decode_q8(q_latent, q_pe, c_kv, k_pe, c_scale, pe_scale, kv_kind, seq_lens, softmax_scale, o=None,
                       lse=None, workspace=None, return_lse=False, stream=None):
    """MLA decode over an 8-bit latent cache: c_kv [B, T, C] and k_pe [B, T, R] uint8 codes of kv_kind ("fp8" or
    "int8") with per-channel fp32 scales c_scale [C], pe_scale [R]; q_latent [B, H, C],
    q_pe [B, H, R] bf16; seq_lens [B] int32. Returns o_latent [B, H, C] bf16 (and lse [B, H] fp32)."""
    lib = load_library()
    bsz, nh, c = q_latent.shape
    r = q_pe.shape[-1]
    t = c_kv.shape[1]
    kind = {"fp8": ATTN_KV_FP8_E4M3, "int8": ATTN_KV_INT8}[kv_kind]
    if o is None:
        o = torch.empty_like(q_latent)
    if lse is None and return_lse:
        lse = torch.empty((bsz, nh), dtype=torch.float32, device=q_latent.device)
    need = attn_mla_decode_workspace_size(bsz, nh, c, max(1, t))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_latent.device)
    if q_pe.shape[:2] != (bsz, nh) or c_kv.shape[0] != bsz or c_kv.shape[2] != c or k_pe.shape != (bsz, t, r):
        raise ValueError("q_pe [B, H, R], c_kv [B, T, C] and k_pe [B, T, R] must agree with q_latent [B, H, C]")
    if tuple(seq_lens.shape) != (bsz,):
        raise ValueError("seq_lens must be [B]")
    _shape(c_scale, (c,), "c_scale")
    _shape(pe_scale, (r,), "pe_scale")
    _shape(o, q_latent.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, nh), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_mla_decode_q8", lib.attn_mla_decode_q8(
        _dev(q_latent, "q_latent", torch.bfloat16), _dev(q_pe, "q_pe", torch.bfloat16),
        _dev(c_kv, "c_kv", torch.uint8), _dev(k_pe, "k_pe", torch.uint8), _dev(c_scale, "c_scale", torch.float32),
        _dev(pe_scale, "pe_scale", torch.float32), int(kind), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(o, "o_latent", torch.bfloat16), lse_p, bsz, nh, c, r, t, float(softmax_scale),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(q_latent, stream)))
    return (o, lse) if return_lse else o


def attn_kv_append_paged(k_new, v_new, cu_new, cache_lens, k_cache, v_cache, block_table, theta, interleaved=True,
                         stream=None):
    """Write new rows k_new/v_new [total_new, Hkv, D] bf16 into the paged caches [num_pages, page, Hkv, D] bf16 at
    positions cache_lens[b] + i (keys rotated with base theta); cu_new [B+1] and cache_lens [B] are int32 device
    tensors, block_table [B, max_pages] int32. The caches are updated in place."""
    lib = load_library()
    total, hkv, d = k_new.shape
    num_pages, page = k_cache.shape[0], k_cache.shape[1]
    if v_new.shape != k_new.shape or k_cache.shape[2:] != (hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("k_new/v_new [total, Hkv, D] and caches [num_pages, page, Hkv, D] must agree")
    _check("attn_kv_append_paged", lib.attn_kv_append_paged(
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16), _dev(cu_new, "cu_new", torch.int32),
        _dev(cache_lens, "cache_lens", torch.int32), _dev(k_cache, "k_cache", torch.bfloat16),
        _dev(v_cache, "v_cache", torch.bfloat16), _dev(block_table, "block_table", torch.int32), cu_new.numel() - 1,
        total, hkv, d, page, block_table.shape[1], num_pages, float(theta), 1 if interleaved else 0,
        _stream(k_new, stream)))
    return k_cache, v_cache


def _check_paged_prefill(q, k_cache, v_cache, block_table, cu_new, cache_lens, o, lse):
    total, hq, d = q.shape
    if k_cache.dim() != 4 or k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_pages, page, Hkv, D] with q's D")
    bsz = cu_new.numel() - 1
    if bsz < 0 or tuple(cache_lens.shape) != (bsz,) or block_table.dim() != 2 or block_table.shape[0] != bsz:
        raise ValueError("cu_new [B+1], cache_lens [B] and block_table [B, max_pages] must agree")
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (hq, total), "lse")


def attn_prefill_paged(q, k_cache, v_cache, block_table, cu_new, cache_lens, max_new, softmax_scale=None, o=None,
                       lse=None, return_lse=False, stream=None):
    """q [total_new, Hq, D] bf16 (rotated at absolute positions) against the paged caches that already hold each
    sequence's cache_lens[b] earlier tokens plus its new ones. Returns o [total_new, Hq, D] bf16 (and lse
    [Hq, total_new] fp32). max_new (host int) must be at least every sequence's number of new tokens."""
    lib = load_library()
    total, hq, d = q.shape
    num_pages, page, hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((hq, total), dtype=torch.float32, device=q.device)
    _check_paged_prefill(q, k_cache, v_cache, block_table, cu_new, cache_lens, o, lse)
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_prefill_paged", lib.attn_prefill_paged(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_table, "block_table", torch.int32), _dev(cu_new, "cu_new", torch.int32),
        _dev(cache_lens, "cache_lens", torch.int32), _dev(o, "o", torch.bfloat16), lse_p, cu_new.numel() - 1, total,
        int(max_new), hq, hkv, d, page, block_table.shape[1], num_pages, scale, _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_prefill_paged_rope(q, k_cache, v_cache, block_table, cu_new, cache_lens, max_new, rope_table,
                            q_positions=None, interleaved=True, softmax_scale=None, o=None, lse=None,
                            return_lse=False, stream=None):
    """attn_prefill_paged with q UNROTATED: each query is rotated as the kernel loads it, by the cos/sin of its
    position (q_positions int32 [total_new], or cache_lens[b] + i when None) from rope_table [n_pos, D/2, 2] fp32."""
    lib = load_library()
    total, hq, d = q.shape
    num_pages, page, hkv, _ = k_cache.shape
    if rope_table.dim() != 3 or rope_table.shape[1:] != (d // 2, 2):
        raise ValueError("rope_table must be [n_positions, head_dim/2, 2]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((hq, total), dtype=torch.float32, device=q.device)
    _check_paged_prefill(q, k_cache, v_cache, block_table, cu_new, cache_lens, o, lse)
    if q_positions is not None and q_positions.numel() != total:
        raise ValueError("q_positions must have one entry per new token (total_new)")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    pos_p = _dev(q_positions, "q_positions", torch.int32) if q_positions is not None else None
    _check("attn_prefill_paged_rope", lib.attn_prefill_paged_rope(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_table, "block_table", torch.int32), _dev(cu_new, "cu_new", torch.int32),
        _dev(cache_lens, "cache_lens", torch.int32), _dev(o, "o", torch.bfloat16), lse_p, cu_new.numel() - 1, total,
        int(max_new), hq, hkv, d, page, block_table.shape[1], num_pages, scale, pos_p,
        _dev(rope_table, "rope_table", torch.float32), rope_table.shape[0], 1 if interleaved else 0,
        _stream(q, stream)))
    return (o, lse) if return_lse else o


def attn_dsa_indexer(q_idx, w_idx, k_idx, seq_lens, scores=None, stream=None):
    """q_idx [B, H_I, D_I] bf16, w_idx [B, H_I] fp32, k_idx [B, T, D_I] bf16, seq_lens [B] int32 (device).
    Returns scores [B, T] fp32 (-inf past each sequence's length)."""
    lib = load_library()
    bsz, hi, di = q_idx.shape
    t = k_idx.shape[1]
    if k_idx.shape != (bsz, t, di) or tuple(w_idx.shape) != (bsz, hi):
        raise ValueError("shape mismatch between q_idx, w_idx and k_idx")
    if scores is None:
        scores = torch.empty((bsz, t), dtype=torch.float32, device=q_idx.device)
    _shape(scores, (bsz, t), "scores")
    _shape(seq_lens, (bsz,), "seq_lens")
    _check("attn_dsa_indexer", lib.attn_dsa_indexer(
        _dev(q_idx, "q_idx", torch.bfloat16), _dev(w_idx, "w_idx", torch.float32), _dev(k_idx, "k_idx", torch.bfloat16),
        _dev(seq_lens, "seq_lens", torch.int32), _dev(scores, "scores", torch.float32), bsz, hi, di, t,
        _stream(q_idx, stream)))
    return scores


def attn_topk(scores, seq_lens, topk, indices=None, stream=None):
    """scores [B, T] fp32, seq_lens [B] int32 (device) -> indices [B, topk] int32: the selected tokens ascending,
    then -1."""
    lib = load_library()
    bsz, t = scores.shape
    if indices is None:
        indices = torch.empty((bsz, topk), dtype=torch.int32, device=scores.device)
    _shape(indices, (bsz, topk), "indices")
    _shape(seq_lens, (bsz,), "seq_lens")
    _check("attn_topk", lib.attn_topk(_dev(scores, "scores", torch.float32), _dev(seq_lens, "seq_lens", torch.int32),
                                      _dev(indices, "indices", torch.int32), bsz, t, int(topk),
                                      _stream(scores, stream)))
    return indices


def attn_mla_sparse_decode_workspace_size(batch, n_heads, kv_lora_rank, topk):
    return int(load_library().attn_mla_sparse_decode_workspace_size(batch, n_heads, kv_lora_rank, topk))


def attn_mla_sparse_decode(q_latent, q_pe, c_kv, k_pe, seq_lens, indices, softmax_scale, o=None, lse=None,
                           workspace=None, return_lse=False, stream=None):
    """As attn_mla_decode, over the tokens indices [B, topk] int32 (device) of each sequence only."""
    lib = load_library()
    bsz, nh, c = q_latent.shape
    r = q_pe.shape[-1]
    t = c_kv.shape[1]
    topk = indices.shape[1]
    if o is None:
        o = torch.empty_like(q_latent)
    if lse is None and return_lse:
        lse = torch.empty((bsz, nh), dtype=torch.float32, device=q_latent.device)
    need = attn_mla_sparse_decode_workspace_size(bsz, nh, c, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_latent.device)
    if q_pe.shape[:2] != (bsz, nh) or c_kv.shape[0] != bsz or c_kv.shape[2] != c or k_pe.shape != (bsz, t, r):
        raise ValueError("q_pe [B, H, R], c_kv [B, T, C] and k_pe [B, T, R] must agree with q_latent [B, H, C]")
    if tuple(seq_lens.shape) != (bsz,) or indices.dim() != 2 or indices.shape[0] != bsz:
        raise ValueError("seq_lens must be [B] and indices [B, topk]")
    _shape(o, q_latent.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, nh), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_mla_sparse_decode", lib.attn_mla_sparse_decode(
        _dev(q_latent, "q_latent", torch.bfloat16), _dev(q_pe, "q_pe", torch.bfloat16),
        _dev(c_kv, "c_kv", torch.bfloat16), _dev(k_pe, "k_pe", torch.bfloat16),
        _dev(seq_lens, "seq_lens", torch.int32), _dev(indices, "indices", torch.int32),
        _dev(o, "o_latent", torch.bfloat16), lse_p, bsz, nh, c, r, t, topk, float(softmax_scale),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(q_latent, stream)))
    return (o, lse) if return_lse else o


def attn_decode_paged_q8(q, k_cache, v_cache, k_scale, v_scale, kv_kind, block_table, seq_lens, max_seqlen_kv,
                         softmax_scale=None, o=None, lse=None, workspace=None, return_lse=False, stream=None):
    """As attn_decode_paged over 8-bit caches: k_cache / v_cache uint8 [num_pages, page, Hkv, D] holding FP8 E4M3
    (kv_kind "fp8") or int8 ("int8") codes, k_scale / v_scale fp32 [Hkv, D]."""
    lib = load_library()
    bsz, hq, d = q.shape
    num_pages, page, hkv, _ = k_cache.shape
    kind = {"fp8": ATTN_KV_FP8_E4M3, "int8": ATTN_KV_INT8}[kv_kind]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    need = attn_decode_paged_workspace_size(bsz, hq, d, max(1, int(max_seqlen_kv)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if k_cache.dim() != 4 or k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_pages, page, Hkv, D] with q's D")
    if block_table.dim() != 2 or block_table.shape[0] != bsz or tuple(seq_lens.shape) != (bsz,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    _shape(k_scale, (hkv, d), "k_scale")
    _shape(v_scale, (hkv, d), "v_scale")
    _shape(o, q.shape, "o")
    if lse is not None:
        _shape(lse, (bsz, hq), "lse")
    lse_p = _dev(lse, "lse", torch.float32) if lse is not None else None
    _check("attn_decode_paged_q8", lib.attn_decode_paged_q8(
        _dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32), kind,
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(o, "o", torch.bfloat16), lse_p, bsz, hq, hkv, d, page, block_table.shape[1], num_pages,
        int(max_seqlen_kv), scale, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(q, stream)))
    return (o, lse) if return_lse else o
