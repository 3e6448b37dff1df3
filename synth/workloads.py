"""The workloads: shapes, RoPE base and softmax scale, as constants.

Nothing here computes attention. A workload is named by what it is; `WORKLOADS` maps the short name to its
description. Long-context RoPE uses the NTK-scaled base 10000 * 4**(128/126) (the base stretched for a 4x longer
context at head dim 128).
"""
from dataclasses import dataclass
import math

import numpy as np


@dataclass(frozen=True)
class Prefill:
    name: str
    batch: int
    seqlen: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str            # "fp32" or "bf16"
    theta: float
    scale: float
    causal: bool = True
    sampled_rows: int = 0  # > 0: the oracle checks only this many seeded query rows (for every head)

    @property
    def flops(self):
        """Algorithmic flops: QK^T and PV at 2 flop per multiply-add over the unmasked (query, key) pairs."""
        pairs = self.seqlen * (self.seqlen + 1) // 2 if self.causal else self.seqlen * self.seqlen
        return 4 * self.batch * self.hq * self.head_dim * pairs


@dataclass(frozen=True)
class PagedDecode:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    page_size: int
    len_lo: int
    len_hi: int
    theta: float
    scale: float
    spare_frac: float = 0.125   # extra physical pages in the pool, never referenced by a block table


@dataclass(frozen=True)
class MLADecode:
    name: str
    batch: int
    heads: int
    latent: int            # kv_lora_rank: width of c_kv and of the absorbed query
    rope: int              # width of the shared rope key k_pe and of q_pe
    seqlen: int
    scale: float


@dataclass(frozen=True)
class ChunkedPrefill:
    """New tokens of several sequences appended to a paged cache that already holds ctx_lens[b] tokens each, then
    attending (causally, bottom-right aligned) to everything before them."""
    name: str
    hq: int
    hkv: int
    head_dim: int
    page_size: int
    ctx_lens: tuple        # tokens already cached per sequence
    new_lens: tuple        # new tokens per sequence (the queries)
    theta: float
    scale: float
    spare_frac: float = 0.125

    @property
    def batch(self):
        return len(self.ctx_lens)

    @property
    def flops(self):
        """Algorithmic flops: QK^T and PV at 2 flop per multiply-add over the unmasked (query, key) pairs; new token
        i of a sequence with c cached tokens sees c + i + 1 keys."""
        pairs = sum(n * c + n * (n + 1) // 2 for c, n in zip(self.ctx_lens, self.new_lens))
        return 4 * self.hq * self.head_dim * pairs


@dataclass(frozen=True)
class DSADecode:
    """DeepSeek Sparse Attention decode: a lightning indexer scores every cached token of each sequence, the top_k
    are kept, and absorbed MLA attends only those (latent / rope widths as MLADecode)."""
    name: str
    batch: int
    heads: int
    latent: int
    rope: int
    seqlen: int
    idx_heads: int         # indexer heads H_I
    idx_dim: int           # indexer query / key width D_I
    topk: int
    scale: float


@dataclass(frozen=True)
class LocalGlobalPrefill:
    """Causal prefill with a local + global mask: key j visible to query i iff j <= i and (i - j < window, or
    j < n_lead, or anchor_stride > 0 and j % anchor_stride == 0)."""
    name: str
    batch: int
    seqlen: int
    hq: int
    hkv: int
    head_dim: int
    window: int
    n_lead: int
    anchor_stride: int
    theta: float
    scale: float
    dtype: str = "bf16"

    def visible_pairs(self, seqlen=None):
        s = self.seqlen if seqlen is None else seqlen
        i = np.arange(s, dtype=np.int64)
        lo = i - self.window + 1                       # first key of the window
        outside = np.maximum(lo, 0)                    # keys 0 .. lo-1 lie outside the window
        lead = np.minimum(self.n_lead, outside)
        anchors = np.zeros_like(i)
        if self.anchor_stride > 0:
            p = self.anchor_stride
            first = -(-self.n_lead // p)                 # first anchor index at or past n_lead
            anchors = np.maximum(0, (outside - 1) // p - first + 1) * (outside > 0)
        return int((np.minimum(self.window, i + 1) + lead + anchors).sum())

    @property
    def flops(self):
        """4 * D flop per visible (query, key) pair per query head and sequence."""
        return 4 * self.batch * self.hq * self.head_dim * self.visible_pairs()


WORKLOADS = {
    "mha_fp32_s256": Prefill("mha_fp32_s256", batch=1, seqlen=256, hq=4, hkv=4, head_dim=64, dtype="fp32",
                             theta=10000.0, scale=1.0 / math.sqrt(64)),
    "gqa_prefill_s8192": Prefill("gqa_prefill_s8192", batch=2, seqlen=8192, hq=32, hkv=8, head_dim=128,
                                 dtype="bf16", theta=10000.0, scale=1.0 / math.sqrt(128)),
    "paged_decode_b64": PagedDecode("paged_decode_b64", batch=64, hq=32, hkv=8, head_dim=128, page_size=64,
                                    len_lo=1024, len_hi=32768, theta=10000.0, scale=1.0 / math.sqrt(128)),
    "mla_decode_b32": MLADecode("mla_decode_b32", batch=32, heads=128, latent=512, rope=64, seqlen=32768,
                                scale=1.0 / math.sqrt(192)),
    "dsa_decode_b32": DSADecode("dsa_decode_b32", batch=32, heads=128, latent=512, rope=64, seqlen=32768,
                                idx_heads=64, idx_dim=128, topk=2048, scale=1.0 / math.sqrt(192)),
    "swa_prefill_s131072": LocalGlobalPrefill("swa_prefill_s131072", batch=1, seqlen=131072, hq=32, hkv=8,
                                              head_dim=128, window=4096, n_lead=0, anchor_stride=32, theta=10000.0,
                                              scale=1.0 / math.sqrt(128)),
    "chunked_prefill_b4": ChunkedPrefill("chunked_prefill_b4", hq=32, hkv=8, head_dim=128, page_size=64,
                                         ctx_lens=(0, 4096, 8192, 14336), new_lens=(2048, 2048, 2048, 2048),
                                         theta=10000.0, scale=1.0 / math.sqrt(128)),
    "gqa_prefill_s131072": Prefill("gqa_prefill_s131072", batch=1, seqlen=131072, hq=32, hkv=8, head_dim=128,
                                   dtype="bf16", theta=10000.0 * 4.0 ** (128.0 / 126.0),
                                   scale=1.0 / math.sqrt(128), sampled_rows=256),
}
