"""Chunked / variable-length prefill from a paged cache on the GPU against the fp64 oracle: attn_kv_append_paged
(keys rotated at their absolute positions, values copied, nothing else touched) followed by attn_prefill_paged
(bottom-right causal attention of the new tokens over cache + new keys)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, chunked_prefill_inputs, sampled_rows
from gpu_util import require_gpu, say, dev, dev_bf16, host_bf16, bits_to_f32, check, check_bf16, BF16_MAX, BF16_MEAN

pytestmark = pytest.mark.gpu

NAN = 0x7FC0


def run_gpu(ta, w, inp, interleaved=True):
    """Append the new tokens, rotate q at the same positions, then attend. Returns host (k_cache, v_cache, o, lse)."""
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table, cu, ctx = dev(inp["block_table"]), dev(inp["cu_new"]), dev(inp["ctx_lens"])
    ta.attn_kv_append_paged(dev_bf16(inp["k_new"]), dev_bf16(inp["v_new"]), cu, ctx, kc, vc, table, w.theta,
                            interleaved=interleaved)
    q = dev_bf16(inp["q"])
    if q.shape[0]:
        ta.attn_rope_apply(q, dev(inp["positions"]), w.theta, interleaved=interleaved)
    o, lse = ta.attn_prefill_paged(q, kc, vc, table, cu, ctx, inp["max_new"], softmax_scale=w.scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    return host_bf16(kc), host_bf16(vc), host_bf16(o), lse.cpu().numpy()


def run_oracle(w, inp, interleaved=True):
    kc, vc = oracle.kv_append_paged(bits_to_f32(inp["k_cache"]), bits_to_f32(inp["v_cache"]), inp["block_table"],
                                    inp["ctx_lens"], bits_to_f32(inp["k_new"]), bits_to_f32(inp["v_new"]),
                                    inp["cu_new"], w.theta, interleaved)
    q = oracle.rope(bits_to_f32(inp["q"]), inp["positions"], w.theta, interleaved)
    o, lse = oracle.prefill_paged(q, kc, vc, inp["block_table"], inp["cu_new"], inp["ctx_lens"], w.scale)
    return kc, vc, o, lse


def written_slots(inp):
    """(page, slot) of every new token, in row order."""
    ps = inp["k_cache"].shape[1]
    out = []
    for b in range(len(inp["ctx_lens"])):
        for i in range(int(inp["cu_new"][b + 1] - inp["cu_new"][b])):
            p = int(inp["ctx_lens"][b]) + i
            out.append((int(inp["block_table"][b, p // ps]), p % ps))
    return out


def check_cache(inp, kc, vc, kc_ref):
    """New keys within bf16 rounding of the oracle's rotation, new values bit-exact, every other slot untouched."""
    slots = written_slots(inp)
    untouched = np.ones(inp["k_cache"].shape[:2], bool)
    for r, (pg, sl) in enumerate(slots):
        untouched[pg, sl] = False
        assert np.array_equal(vc[pg, sl], inp["v_new"][r]), f"value row {r} not copied exactly"
    if slots:
        pg, sl = np.array(slots).T
        check("k_cache (new slots)", bits_to_f32(kc[pg, sl]), kc_ref[pg, sl], BF16_MAX, BF16_MEAN)
    assert np.array_equal(kc[untouched], inp["k_cache"][untouched]), "append touched a key slot it does not own"
    assert np.array_equal(vc[untouched], inp["v_cache"][untouched]), "append touched a value slot it does not own"


# (ctx_lens, new_lens): empty context, one new token, chunks that start mid-page, a sequence with nothing new,
# a ragged tail in every sequence, and a chunk longer than its context.
CASES = [
    ((0, 5, 130, 64, 1000, 7), (7, 1, 200, 64, 129, 0)),
    ((300,), (517,)),
    ((0, 0), (1, 333)),
]


@pytest.mark.parametrize("hq,hkv,d,page", [(32, 8, 128, 64), (16, 2, 64, 128), (12, 4, 128, 64), (8, 8, 64, 256),
                                           (20, 4, 128, 64)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_chunked_prefill_small(hq, hkv, d, page, case):
    ta = require_gpu()
    w = dataclasses.replace(WORKLOADS["chunked_prefill_b4"], hq=hq, hkv=hkv, head_dim=d, page_size=page,
                            scale=1.0 / np.sqrt(d))
    ctx, new = CASES[case]
    say(f"chunked hq={hq} hkv={hkv} d={d} page={page} ctx={ctx} new={new}")
    inp = chunked_prefill_inputs(w, seed=31 + case, ctx_lens=ctx, new_lens=new)
    kc, vc, o, lse = run_gpu(ta, w, inp)
    kc_ref, vc_ref, o_ref, lse_ref = run_oracle(w, inp)
    check_cache(inp, kc, vc, kc_ref)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


def test_half_split_pairing():
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    inp = chunked_prefill_inputs(w, seed=40, ctx_lens=(70, 3), new_lens=(90, 150))
    say("chunked half-split pairing")
    kc, vc, o, lse = run_gpu(ta, w, inp, interleaved=False)
    kc_ref, _, o_ref, lse_ref = run_oracle(w, inp, interleaved=False)
    check_cache(inp, kc, vc, kc_ref)
    check_bf16("o", o, o_ref)
    check("lse", lse, lse_ref, BF16_MAX, BF16_MEAN)


def relayout(inp, seed):
    """Same logical cache in a new random physical placement: pages not in use (and slots past each sequence's
    end) hold NaN, table entries past each sequence's pages are out of range."""
    ps = inp["k_cache"].shape[1]
    n_pool = inp["k_cache"].shape[0]
    perm = np.random.default_rng(seed).permutation(n_pool)
    kc = np.full_like(inp["k_cache"], NAN)
    vc = np.full_like(inp["v_cache"], NAN)
    table = np.full_like(inp["block_table"], 1 << 30)
    off = 0
    for b in range(len(inp["ctx_lens"])):
        total = int(inp["ctx_lens"][b]) + int(inp["cu_new"][b + 1] - inp["cu_new"][b])
        for j in range((total + ps - 1) // ps):
            src, dst = inp["block_table"][b, j], perm[off]
            off += 1
            n = min(ps, total - j * ps)
            kc[dst, :n] = inp["k_cache"][src, :n]
            vc[dst, :n] = inp["v_cache"][src, :n]
            table[b, j] = dst
    out = dict(inp)
    out.update(k_cache=kc, v_cache=vc, block_table=table)
    return out


def test_placement_and_poison_are_invisible():
    """Outputs are bit-identical under any physical placement, with NaN in every unused page and every slot past a
    sequence's end, and out-of-range table entries past its pages."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    inp = chunked_prefill_inputs(w, seed=41, ctx_lens=(3, 0, 190, 64), new_lens=(100, 65, 1, 63))
    say("chunked placement / poison")
    _, _, o1, l1 = run_gpu(ta, w, inp)
    for seed in (1, 2):
        _, _, o2, l2 = run_gpu(ta, w, relayout(inp, seed))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), seed


def test_one_chunk_equals_plain_causal_prefill():
    """Cross-kernel: with empty caches the chunked path is plain causal prefill of each sequence (bit-identical:
    the same tile order, masks and arithmetic)."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    n = 700
    inp = chunked_prefill_inputs(w, seed=42, ctx_lens=(0, 0), new_lens=(n, n))
    say("chunked vs plain prefill")
    _, _, o, lse = run_gpu(ta, w, inp)
    q = dev_bf16(inp["q"].reshape(2, n, w.hq, w.head_dim))
    ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    k = dev_bf16(inp["k_new"].reshape(2, n, w.hkv, w.head_dim))
    ta.attn_rope_apply(k, dev(inp["positions"]), w.theta)
    o2, lse2 = ta.attn_prefill(q, k, dev_bf16(inp["v_new"].reshape(2, n, w.hkv, w.head_dim)), causal=True,
                               softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(o.reshape(2, n, w.hq, w.head_dim), host_bf16(o2))
    lse2 = lse2.cpu().numpy()                                  # [B, Hq, n] -> [Hq, B*n]
    assert np.array_equal(lse, lse2.transpose(1, 0, 2).reshape(w.hq, 2 * n))


def test_chunks_in_sequence_equal_one_prefill():
    """Prefilling a sequence in three chunks (append, attend, repeat) gives the rows of one causal prefill of the
    whole sequence, within the bf16 tolerance."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    cuts = [0, 150, 151, 600]
    L = cuts[-1]
    inp = chunked_prefill_inputs(w, seed=43, ctx_lens=(0,), new_lens=(L,))
    say(f"chunked in sequence {cuts}")
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table = dev(inp["block_table"])
    outs = []
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        cu, ctx = dev(np.array([0, c1 - c0], np.int32)), dev(np.array([c0], np.int32))
        ta.attn_kv_append_paged(dev_bf16(inp["k_new"][c0:c1]), dev_bf16(inp["v_new"][c0:c1]), cu, ctx, kc, vc, table,
                                w.theta)
        q = dev_bf16(inp["q"][c0:c1])
        ta.attn_rope_apply(q, dev(inp["positions"][c0:c1]), w.theta)
        outs.append(host_bf16(ta.attn_prefill_paged(q, kc, vc, table, cu, ctx, c1 - c0, softmax_scale=w.scale)))
    torch.cuda.synchronize()
    o = np.concatenate(outs)
    _, _, o_ref, _ = run_oracle(w, inp)
    check_bf16("o (three chunks)", o, o_ref)


def test_max_new_smaller_than_a_sequence_leaves_its_tail_unwritten():
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    inp = chunked_prefill_inputs(w, seed=44, ctx_lens=(10, 20), new_lens=(40, 300))
    say("chunked max_new < n_b")
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table, cu, ctx = dev(inp["block_table"]), dev(inp["cu_new"]), dev(inp["ctx_lens"])
    ta.attn_kv_append_paged(dev_bf16(inp["k_new"]), dev_bf16(inp["v_new"]), cu, ctx, kc, vc, table, w.theta)
    q = dev_bf16(inp["q"])
    ta.attn_rope_apply(q, dev(inp["positions"]), w.theta)
    o = torch.full((q.shape[0], w.hq, w.head_dim), 7.0, dtype=torch.bfloat16, device=q.device)
    ta.attn_prefill_paged(q, kc, vc, table, cu, ctx, 64, softmax_scale=w.scale, o=o)
    torch.cuda.synchronize()
    o = host_bf16(o)
    _, _, o_ref, _ = run_oracle(w, inp)
    check_bf16("o rows below max_new", np.concatenate([o[:40], o[40:104]]),
               np.concatenate([o_ref[:40], o_ref[40:104]]))
    assert np.all(bits_to_f32(o[104:]) == 7.0)


def test_full_size_sampled():
    """The bench workload (4 sequences x 2048 new tokens on 0 / 4096 / 8192 / 14336 cached ones) in the bench's
    launch configuration. The oracle appends the new tokens to its own copy of the caches (keys rotated at their
    absolute positions); every appended key and value of all four sequences is compared with it, every other slot
    must be untouched, and sampled query rows are computed one by one against the oracle's caches."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    inp = chunked_prefill_inputs(w, seed=0)
    say(f"chunked full size ctx={w.ctx_lens} new={w.new_lens}")
    kc, vc, o, lse = run_gpu(ta, w, inp)
    say("  oracle append")
    kc_ref, vc_ref = oracle.kv_append_paged(bits_to_f32(inp["k_cache"]), bits_to_f32(inp["v_cache"]),
                                            inp["block_table"], inp["ctx_lens"], bits_to_f32(inp["k_new"]),
                                            bits_to_f32(inp["v_new"]), inp["cu_new"], w.theta)
    check_cache(inp, kc, vc, kc_ref)
    # sampled rows: first, last and three seeded others of each sequence; all heads
    rows = []
    for b in range(w.batch):
        r0, r1 = int(inp["cu_new"][b]), int(inp["cu_new"][b + 1])
        rows += [r0 + int(i) for i in sampled_rows(r1 - r0, 5, seed=b)]
    say(f"  oracle on {len(rows)} rows")
    q_all = oracle.rope(bits_to_f32(inp["q"][rows]), inp["positions"][rows], w.theta)
    for j, r in enumerate(rows):
        b = int(np.searchsorted(inp["cu_new"], r, side="right") - 1)
        L = int(inp["positions"][r]) + 1
        k = oracle.gather_paged(kc_ref, inp["block_table"][b], L)
        v = oracle.gather_paged(vc_ref, inp["block_table"][b], L)
        o_ref, lse_ref = _one_row(q_all[j], k, v, w)
        check_bf16(f"o row {r}", o[r], o_ref)
        check(f"lse row {r}", lse[:, r], lse_ref, BF16_MAX)


def _one_row(q, k, v, w):
    """One query (all heads) against L keys: the oracle's paged prefill on a single-query sequence."""
    L = k.shape[0]
    table = np.arange((L + w.page_size - 1) // w.page_size, dtype=np.int32)[None]
    pad = table.shape[1] * w.page_size - L
    kp = np.concatenate([k, np.zeros((pad,) + k.shape[1:])]).reshape(-1, w.page_size, *k.shape[1:])
    vp = np.concatenate([v, np.zeros((pad,) + v.shape[1:])]).reshape(-1, w.page_size, *v.shape[1:])
    o, lse = oracle.prefill_paged(q[None], kp, vp, table, np.array([0, 1]), np.array([L - 1]), w.scale)
    return o[0], lse[:, 0]


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("explicit_pos", [True, False])
@pytest.mark.parametrize("ctx,new,hq,hkv,d", [((0, 4096, 8192, 14336), (2048,) * 4, 32, 8, 128),
                                              ((3, 0, 190, 64), (100, 65, 1, 63), 32, 8, 128),
                                              ((70, 500), (90, 150), 16, 16, 64)])
def test_fused_rope_equals_rotate_then_attend(ctx, new, hq, hkv, d, interleaved, explicit_pos):
    """attn_prefill_paged_rope on unrotated q gives attn_rope_apply(q) then attn_prefill_paged bit for bit, with
    the default positions (cache_lens[b] + i) or the same positions passed explicitly; q itself is not rotated."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    say(f"chunked fused rope ctx={ctx} new={new} hq={hq} hkv={hkv} d={d} interleaved={interleaved}")
    inp = chunked_prefill_inputs(w, seed=50, ctx_lens=ctx, new_lens=new, hq=hq, hkv=hkv, head_dim=d)
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table, cu, cl = dev(inp["block_table"]), dev(inp["cu_new"]), dev(inp["ctx_lens"])
    ta.attn_kv_append_paged(dev_bf16(inp["k_new"]), dev_bf16(inp["v_new"]), cu, cl, kc, vc, table, w.theta,
                            interleaved=interleaved)
    pos = dev(inp["positions"])
    q1 = dev_bf16(inp["q"])
    ta.attn_rope_apply(q1, pos, w.theta, interleaved=interleaved)
    o1, l1 = ta.attn_prefill_paged(q1, kc, vc, table, cu, cl, inp["max_new"], softmax_scale=w.scale,
                                   return_lse=True)
    rope_tab = ta.attn_rope_table(int(inp["positions"].max()) + 1, d, w.theta)
    q2 = dev_bf16(inp["q"])
    o2, l2 = ta.attn_prefill_paged_rope(q2, kc, vc, table, cu, cl, inp["max_new"], rope_tab,
                                        q_positions=pos if explicit_pos else None, interleaved=interleaved,
                                        softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
    assert np.array_equal(host_bf16(q2), inp["q"])


def test_fused_rope_at_other_positions_and_clamped():
    """Explicit query positions that differ from cache_lens[b] + i (shifted per sequence, permuted within it, some
    negative, some past the table) give the same bits as attn_rope_apply at the positions clamped into the table
    followed by attn_prefill_paged: the kernel rotates by the positions it is given, clamped into [0, rows)."""
    ta = require_gpu()
    w = WORKLOADS["chunked_prefill_b4"]
    inp = chunked_prefill_inputs(w, seed=51, ctx_lens=(3, 0, 190, 64), new_lens=(100, 65, 1, 63))
    say("chunked fused rope at shifted / permuted / clamped positions")
    kc, vc = dev_bf16(inp["k_cache"]), dev_bf16(inp["v_cache"])
    table, cu, cl = dev(inp["block_table"]), dev(inp["cu_new"]), dev(inp["ctx_lens"])
    ta.attn_kv_append_paged(dev_bf16(inp["k_new"]), dev_bf16(inp["v_new"]), cu, cl, kc, vc, table, w.theta)
    rng = np.random.default_rng(52)
    pos = inp["positions"].astype(np.int64).copy()
    for b, shift in enumerate((37, -20, 1000, 5)):
        r0, r1 = int(inp["cu_new"][b]), int(inp["cu_new"][b + 1])
        pos[r0:r1] = rng.permutation(pos[r0:r1]) + shift
    pos = pos.astype(np.int32)
    n_tab = 200
    assert pos.min() < 0 and pos.max() >= n_tab
    rope_tab = ta.attn_rope_table(n_tab, w.head_dim, w.theta)
    q1 = dev_bf16(inp["q"])
    ta.attn_rope_apply(q1, dev(np.clip(pos, 0, n_tab - 1)), w.theta)
    o1, l1 = ta.attn_prefill_paged(q1, kc, vc, table, cu, cl, inp["max_new"], softmax_scale=w.scale, return_lse=True)
    o2, l2 = ta.attn_prefill_paged_rope(dev_bf16(inp["q"]), kc, vc, table, cu, cl, inp["max_new"], rope_tab,
                                        q_positions=dev(pos), softmax_scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
