"""The C ABI on the CPU: libattn.so loads, exports every function include/attn.h declares, sizes workspaces, and
rejects invalid arguments with the documented status before any device work (so no GPU is needed here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
# ATTN_LIB selects another build of the library (e.g. the host-ASan build of the validation code)
LIB = os.environ.get("ATTN_LIB") or os.path.join(ROOT, "transformer_attention_causal_amd", "libattn.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
NULL = None
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libattn.so is not built: run python -m transformer_attention_causal_amd.build")
    from transformer_attention_causal_amd import load_library
    return load_library(LIB)


def test_header_declares_the_operations():
    names = declared_functions()
    for n in ("attn_rope_apply", "attn_prefill", "attn_decode_paged", "attn_mla_decode", "attn_kv_append_paged",
              "attn_prefill_paged", "attn_dsa_indexer", "attn_topk", "attn_mla_sparse_decode", "attn_decode_paged_q8",
              "attn_prefill_local_global", "attn_rope_table", "attn_prefill_rope", "attn_mla_decode_q8",
              "attn_prefill_paged_rope"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from transformer_attention_causal_amd import SIGNATURES
    names = declared_functions()
    assert sorted(SIGNATURES) == names, "binding signatures and header disagree"
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, word in [(0, b"ATTN_OK"), (1, b"INVALID_ARG"), (2, b"UNSUPPORTED"), (3, b"WORKSPACE"), (4, b"HIP")]:
        assert word in lib.attn_status_string(code)
    assert lib.attn_status_string(99)


def test_workspace_sizes(lib):
    # decode: [B, Hq, ceil(L/1024), D] fp32 partial outputs (256-byte aligned) + [B, Hq, chunks] fp32 lse
    b, hq, d, lmax = 64, 32, 128, 32768
    chunks = (lmax + 1023) // 1024
    o_bytes = (b * hq * chunks * d * 4 + 255) // 256 * 256
    assert lib.attn_decode_paged_workspace_size(b, hq, d, lmax) == o_bytes + b * hq * chunks * 4
    assert lib.attn_decode_paged_workspace_size(0, hq, d, lmax) == 0
    assert lib.attn_decode_paged_workspace_size(b, hq, d, 0) == 0
    # MLA: grows with the number of splits, which never exceeds ceil(L/32)
    assert lib.attn_mla_decode_workspace_size(32, 128, 512, 32768) > 32 * 128 * 512 * 4
    assert lib.attn_mla_decode_workspace_size(1, 128, 512, 32) == 128 * 512 * 4 + 128 * 4
    assert lib.attn_mla_decode_workspace_size(-1, 128, 512, 32) == 0


def test_rope_validation(lib):
    f = lib.attn_rope_apply
    assert f(FAKE, 0, 4, 2, 63, FAKE, 10000.0, 1, NULL) == INVALID        # odd head_dim
    assert f(FAKE, 0, 4, 0, 64, FAKE, 10000.0, 1, NULL) == INVALID        # no heads
    assert f(FAKE, 0, -1, 2, 64, FAKE, 10000.0, 1, NULL) == INVALID       # negative tokens
    assert f(FAKE, 0, 4, 2, 64, FAKE, 1.0, 1, NULL) == INVALID            # base must exceed 1
    assert f(FAKE, 0, 4, 2, 64, FAKE, float("nan"), 1, NULL) == INVALID
    assert f(NULL, 0, 4, 2, 64, FAKE, 10000.0, 1, NULL) == INVALID        # null tensor
    assert f(FAKE, 0, 4, 2, 64, NULL, 10000.0, 1, NULL) == INVALID        # null positions
    assert f(FAKE, 7, 4, 2, 64, FAKE, 10000.0, 1, NULL) == UNSUPPORTED    # dtype
    assert f(FAKE, 0, 4, 2, 2048, FAKE, 10000.0, 1, NULL) == UNSUPPORTED  # head_dim > 1024
    assert f(NULL, 0, 0, 2, 64, NULL, 10000.0, 1, NULL) == OK             # nothing to do


def test_prefill_validation(lib):
    f = lib.attn_prefill
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=NULL, dt=0, b=1, s=16, hq=8, hkv=2, d=128,
                                  causal=1, scale=0.088), **kw)
    call = lambda a: f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dt"], a["b"], a["s"], a["hq"], a["hkv"], a["d"],
                       a["causal"], a["scale"], NULL)
    assert call(args(hq=6, hkv=4)) == INVALID            # Hq % Hkv != 0
    assert call(args(hkv=0)) == INVALID
    assert call(args(s=-1)) == INVALID
    assert call(args(scale=0.0)) == INVALID
    assert call(args(scale=float("inf"))) == INVALID
    assert call(args(q=NULL)) == INVALID
    assert call(args(o=NULL)) == INVALID
    assert call(args(d=96)) == UNSUPPORTED
    assert call(args(dt=3)) == UNSUPPORTED
    assert call(args(q=NULL, k=NULL, v=NULL, o=NULL, s=0)) == OK     # empty: nothing launched


def test_rope_table_validation(lib):
    f = lib.attn_rope_table
    assert f(FAKE, 16, 63, 10000.0, NULL) == INVALID          # odd head_dim
    assert f(FAKE, 16, 0, 10000.0, NULL) == INVALID
    assert f(FAKE, -1, 64, 10000.0, NULL) == INVALID          # negative count
    assert f(FAKE, 16, 64, 0.5, NULL) == INVALID              # base must exceed 1
    assert f(FAKE, 16, 64, float("inf"), NULL) == INVALID
    assert f(NULL, 16, 64, 10000.0, NULL) == INVALID          # null table
    assert f(FAKE, 16, 2048, 10000.0, NULL) == UNSUPPORTED    # head_dim > 1024
    assert f(NULL, 0, 64, 10000.0, NULL) == OK                # nothing to do


def test_prefill_rope_validation(lib):
    f = lib.attn_prefill_rope
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=NULL, b=1, s=16, hq=8, hkv=2, d=128, causal=1,
                                  scale=0.088, pos=NULL, tab=FAKE, tlen=16, il=1), **kw)
    call = lambda a: f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["b"], a["s"], a["hq"], a["hkv"], a["d"],
                       a["causal"], a["scale"], a["pos"], a["tab"], a["tlen"], a["il"], NULL)
    assert call(args(hq=6, hkv=4)) == INVALID
    assert call(args(scale=-1.0)) == INVALID
    assert call(args(q=NULL)) == INVALID
    assert call(args(tab=NULL)) == INVALID                     # table required
    assert call(args(tlen=0)) == INVALID
    assert call(args(tab=ctypes.c_void_p(0x1008))) == INVALID  # table must be 16-byte aligned
    assert call(args(d=96)) == UNSUPPORTED
    assert call(args(q=NULL, k=NULL, v=NULL, o=NULL, tab=NULL, b=0)) == OK


def test_prefill_paged_rope_validation(lib):
    f = lib.attn_prefill_paged_rope
    args = lambda **kw: dict(dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cu=FAKE, cl=FAKE, o=FAKE, lse=NULL, b=2, tot=100,
                                  mx=60, hq=8, hkv=2, d=128, page=64, mp=4, np_=8, scale=0.088, pos=NULL, tab=FAKE,
                                  tlen=300, il=1), **kw)
    call = lambda a: f(a["q"], a["kc"], a["vc"], a["bt"], a["cu"], a["cl"], a["o"], a["lse"], a["b"], a["tot"],
                       a["mx"], a["hq"], a["hkv"], a["d"], a["page"], a["mp"], a["np_"], a["scale"], a["pos"],
                       a["tab"], a["tlen"], a["il"], NULL)
    assert call(args(hq=6, hkv=4)) == INVALID
    assert call(args(mx=101)) == INVALID                       # max_new > total_new
    assert call(args(bt=NULL)) == INVALID
    assert call(args(tab=NULL)) == INVALID                     # table required
    assert call(args(tlen=0)) == INVALID
    assert call(args(tab=ctypes.c_void_p(0x1008))) == INVALID  # table must be 16-byte aligned
    assert call(args(page=48)) == UNSUPPORTED
    assert call(args(d=96)) == UNSUPPORTED
    assert call(args(q=NULL, kc=NULL, vc=NULL, bt=NULL, cu=NULL, cl=NULL, o=NULL, tab=NULL, tot=0, mx=0)) == OK


def test_decode_validation(lib):
    f = lib.attn_decode_paged
    ws_need = lib.attn_decode_paged_workspace_size(2, 8, 128, 100)

    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=NULL, b=2, hq=8, hkv=2, d=128, ps=64,
                 maxp=2, npages=4, maxlen=100, scale=0.088, ws=FAKE, wsb=ws_need)
        a.update(kw)
        return f(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["b"], a["hq"], a["hkv"], a["d"],
                 a["ps"], a["maxp"], a["npages"], a["maxlen"], a["scale"], a["ws"], a["wsb"], NULL)
    assert call(hq=6, hkv=4) == INVALID
    assert call(maxlen=-1) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(ps=0) == INVALID
    assert call(q=NULL) == INVALID
    assert call(sl=NULL) == INVALID
    assert call(bt=NULL) == INVALID
    assert call(npages=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(d=64, ws=NULL) == WORKSPACE              # head_dim 64 is supported: validation reaches the workspace
    assert call(d=64, b=0) == OK
    assert call(hq=64, hkv=2) == UNSUPPORTED             # group of 32 query heads > 16
    assert call(ps=48) == UNSUPPORTED                    # not a power of two
    assert call(ps=8) == UNSUPPORTED
    assert call(wsb=ws_need - 1) == WORKSPACE
    assert call(ws=NULL) == WORKSPACE
    assert call(b=0) == OK


def test_decode_noalloc_validation(lib):
    """The no-allocation decode validates exactly as attn_decode_paged, and refuses a request whose workspace would
    exceed the static scratch (64 MiB), all before any HIP call."""
    f = lib.attn_decode_paged_noalloc
    scratch = 64 << 20

    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=NULL, b=2, hq=8, hkv=2, d=128, ps=64,
                 maxp=2, npages=4, maxlen=100, scale=0.088)
        a.update(kw)
        return f(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["b"], a["hq"], a["hkv"], a["d"],
                 a["ps"], a["maxp"], a["npages"], a["maxlen"], a["scale"], NULL)
    assert call(hq=6, hkv=4) == INVALID
    assert call(maxlen=-1) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(q=NULL) == INVALID
    assert call(bt=NULL) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(ps=48) == UNSUPPORTED
    assert call(b=0) == OK
    # 64 sequences x 32 heads x D=128: 64512 cached tokens fit the scratch, one more chunk does not
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 64512) <= scratch
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 64513) > scratch
    assert call(b=64, hq=32, hkv=8, maxp=1100, npages=70000, maxlen=64513) == WORKSPACE
    assert call(b=64, hq=32, hkv=8, maxp=1100, npages=70000, maxlen=1 << 30) == WORKSPACE


def test_mla_validation(lib):
    f = lib.attn_mla_decode
    ws_need = lib.attn_mla_decode_workspace_size(2, 128, 512, 64)

    def call(**kw):
        a = dict(ql=FAKE, qp=FAKE, ckv=FAKE, kpe=FAKE, sl=FAKE, o=FAKE, lse=NULL, b=2, h=128, c=512, r=64, t=64,
                 scale=0.072, ws=FAKE, wsb=ws_need)
        a.update(kw)
        return f(a["ql"], a["qp"], a["ckv"], a["kpe"], a["sl"], a["o"], a["lse"], a["b"], a["h"], a["c"], a["r"],
                 a["t"], a["scale"], a["ws"], a["wsb"], NULL)
    assert call(h=0) == INVALID
    assert call(t=-2) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(ql=NULL) == INVALID
    assert call(ckv=NULL) == INVALID
    assert call(c=256) == UNSUPPORTED
    assert call(r=32) == UNSUPPORTED
    assert call(h=48) == UNSUPPORTED
    assert call(h=256) == UNSUPPORTED
    assert call(wsb=ws_need - 4) == WORKSPACE
    assert call(b=0) == OK


def test_mla_q8_validation(lib):
    f = lib.attn_mla_decode_q8
    WS = ctypes.c_size_t(1 << 40)
    args = lambda **kw: dict(dict(ql=FAKE, qp=FAKE, ckv=FAKE, kpe=FAKE, cs=FAKE, ps=FAKE, kind=1, sl=FAKE, o=FAKE,
                                  b=2, h=128, c=512, r=64, t=100, scale=0.07, ws=FAKE), **kw)
    call = lambda **kw: (lambda a: f(a["ql"], a["qp"], a["ckv"], a["kpe"], a["cs"], a["ps"], a["kind"], a["sl"],
                                     a["o"], NULL, a["b"], a["h"], a["c"], a["r"], a["t"], a["scale"], a["ws"], WS,
                                     NULL))(args(**kw))
    assert call(kind=0) == UNSUPPORTED                  # bf16 has its own entry point
    assert call(kind=3) == UNSUPPORTED
    assert call(cs=NULL) == INVALID
    assert call(ps=NULL) == INVALID
    assert call(cs=ctypes.c_void_p(0x1004)) == INVALID  # scales must be 16-byte aligned
    assert call(ckv=ctypes.c_void_p(0x1008)) == INVALID
    assert call(h=48) == UNSUPPORTED
    assert call(c=256) == UNSUPPORTED
    assert call(scale=0.0) == INVALID
    assert call(t=-1) == INVALID
    assert call(ws=NULL) == WORKSPACE
    assert call(b=0, ql=NULL, qp=NULL, ckv=NULL, kpe=NULL, cs=NULL, ps=NULL, sl=NULL, o=NULL) == OK


def test_binding_refuses_without_library(tmp_path):
    from transformer_attention_causal_amd import binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            binding.load_library(str(tmp_path / "missing.so"))
    finally:
        binding._lib = saved


def test_kv_append_validation(lib):
    f = lib.attn_kv_append_paged
    A = ctypes.c_void_p(0x10000)                    # 16-byte aligned fake pointer (never dereferenced)
    U = ctypes.c_void_p(0x10008)                    # misaligned
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("k_new", A), ("v_new", A), ("cu", FAKE), ("lens", FAKE), ("kc", A), ("vc", A), ("table", FAKE),
        ("batch", 2), ("total", 10), ("hkv", 8), ("d", 128), ("page", 64), ("maxp", 4), ("npages", 16),
        ("theta", 10000.0), ("inter", 1), ("stream", NULL)]]
    assert f(*args(d=127)) == INVALID
    assert f(*args(batch=-1)) == INVALID
    assert f(*args(theta=0.5)) == INVALID
    assert f(*args(k_new=NULL)) == INVALID
    assert f(*args(k_new=U)) == INVALID               # rows must be 16-byte aligned
    assert f(*args(npages=0)) == INVALID
    assert f(*args(d=72)) == UNSUPPORTED              # not a multiple of 16
    assert f(*args(page=48)) == UNSUPPORTED           # not a power of two
    assert f(*args(total=0, k_new=NULL)) == OK        # nothing to append


def test_prefill_paged_validation(lib):
    f = lib.attn_prefill_paged
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("q", FAKE), ("kc", FAKE), ("vc", FAKE), ("table", FAKE), ("cu", FAKE), ("lens", FAKE), ("o", FAKE),
        ("lse", NULL), ("batch", 2), ("total", 100), ("maxnew", 60), ("hq", 32), ("hkv", 8), ("d", 128),
        ("page", 64), ("maxp", 8), ("npages", 32), ("scale", 0.088), ("stream", NULL)]]
    assert f(*args(hq=30)) == INVALID                 # Hq % Hkv
    assert f(*args(scale=0.0)) == INVALID
    assert f(*args(maxnew=101)) == INVALID            # more than the total
    assert f(*args(q=NULL)) == INVALID
    assert f(*args(cu=NULL)) == INVALID
    assert f(*args(npages=0)) == INVALID
    assert f(*args(d=96)) == UNSUPPORTED
    assert f(*args(page=32)) == UNSUPPORTED           # tiles of 64 keys may not straddle pages
    assert f(*args(page=96)) == UNSUPPORTED
    assert f(*args(total=0, maxnew=0, q=NULL)) == OK


def test_dsa_indexer_validation(lib):
    f = lib.attn_dsa_indexer
    A = ctypes.c_void_p(0x10000)
    U = ctypes.c_void_p(0x10004)
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("q", A), ("w", FAKE), ("k", A), ("lens", FAKE), ("scores", FAKE), ("batch", 2), ("hi", 64), ("di", 128),
        ("t", 1000), ("stream", NULL)]]
    assert f(*args(batch=-1)) == INVALID
    assert f(*args(t=-1)) == INVALID
    assert f(*args(hi=0)) == INVALID
    assert f(*args(w=NULL)) == INVALID
    assert f(*args(scores=NULL)) == INVALID
    assert f(*args(k=U)) == INVALID                   # 16-byte rows
    assert f(*args(hi=48)) == UNSUPPORTED
    assert f(*args(di=96)) == UNSUPPORTED
    assert f(*args(t=0, q=NULL)) == OK                # no tokens: nothing to score


def test_topk_validation(lib):
    f = lib.attn_topk
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("scores", FAKE), ("lens", FAKE), ("out", FAKE), ("batch", 2), ("t", 100), ("k", 10), ("stream", NULL)]]
    assert f(*args(k=0)) == INVALID
    assert f(*args(batch=-2)) == INVALID
    assert f(*args(out=NULL)) == INVALID
    assert f(*args(scores=NULL)) == INVALID
    assert f(*args(batch=0, out=NULL)) == OK


def test_mla_sparse_validation(lib):
    f = lib.attn_mla_sparse_decode
    need = lib.attn_mla_sparse_decode_workspace_size(2, 128, 512, 256)
    assert need >= 2 * 128 * 512 * 4                 # at least one fp32 partial per (sequence, head)
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("ql", FAKE), ("qp", FAKE), ("ckv", FAKE), ("kpe", FAKE), ("lens", FAKE), ("idx", FAKE), ("o", FAKE),
        ("lse", NULL), ("b", 2), ("h", 128), ("c", 512), ("r", 64), ("t", 4096), ("k", 256), ("scale", 0.07),
        ("ws", FAKE), ("wsb", need), ("stream", NULL)]]
    assert f(*args(k=0)) == INVALID
    assert f(*args(t=0)) == INVALID
    assert f(*args(idx=NULL)) == INVALID
    assert f(*args(scale=-1.0)) == INVALID
    assert f(*args(c=256)) == UNSUPPORTED
    assert f(*args(h=40)) == UNSUPPORTED
    assert f(*args(t=1 << 23)) == UNSUPPORTED         # latent rows of one sequence beyond a 32-bit resource
    assert f(*args(wsb=need - 1)) == WORKSPACE
    assert f(*args(b=0)) == OK


def test_decode_q8_validation(lib):
    f = lib.attn_decode_paged_q8
    A = ctypes.c_void_p(0x10000)
    U = ctypes.c_void_p(0x10008)
    need = lib.attn_decode_paged_workspace_size(2, 32, 128, 4096)
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("q", A), ("kc", A), ("vc", A), ("ks", A), ("vs", A), ("kind", 1), ("table", FAKE), ("lens", FAKE),
        ("o", FAKE), ("lse", NULL), ("b", 2), ("hq", 32), ("hkv", 8), ("d", 128), ("page", 64), ("maxp", 64),
        ("npages", 200), ("t", 4096), ("scale", 0.088), ("ws", FAKE), ("wsb", need), ("stream", NULL)]]
    assert f(*args(hq=30)) == INVALID
    assert f(*args(ks=NULL)) == INVALID
    assert f(*args(kc=U)) == INVALID                  # 16-byte aligned rows
    assert f(*args(scale=0.0)) == INVALID
    assert f(*args(kind=0)) == UNSUPPORTED            # bf16 caches go through attn_decode_paged
    assert f(*args(kind=3)) == UNSUPPORTED
    assert f(*args(d=96)) == UNSUPPORTED
    assert f(*args(d=64, ws=NULL)) == WORKSPACE       # head_dim 64 is supported: validation reaches the workspace
    assert f(*args(wsb=need - 1)) == WORKSPACE
    assert f(*args(b=0)) == OK


def test_prefill_local_global_validation(lib):
    f = lib.attn_prefill_local_global
    args = lambda **kw: [kw.get(n, d) for n, d in [
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE), ("lse", NULL), ("b", 1), ("s", 1000), ("hq", 32),
        ("hkv", 8), ("d", 128), ("w", 128), ("g", 0), ("p", 32), ("scale", 0.088), ("stream", NULL)]]
    assert f(*args(w=0)) == INVALID                   # a query must see at least itself
    assert f(*args(g=-1)) == INVALID
    assert f(*args(p=-2)) == INVALID
    assert f(*args(hq=12, hkv=8)) == INVALID
    assert f(*args(q=NULL)) == INVALID
    assert f(*args(d=96)) == UNSUPPORTED
    assert f(*args(p=1 << 20)) == UNSUPPORTED         # strided anchor tile beyond 32-bit offsets
    assert f(*args(s=0, q=NULL)) == OK
