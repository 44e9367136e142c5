"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test names the pin it implements:
  P1 chunked prefill == one-shot prefill, outputs and KV cache (chunked-prefill
     post, section "correctness");
  P2 merge of two disjoint partitions == attention over their union (same
     section, softmax_merge);
  P3 brute force: scalar loops with math.exp on tiny inputs, with the test's own
     page placement;
  P4 a library routine: torch float64 scaled_dot_product_attention with an
     explicit bottom-right mask on contiguous K/V, and torch.logsumexp;
  P5 closed forms (one key; all keys zero; all values equal; two keys with
     known weights);
  P6 invariances (page permutation, page size, request order, GQA vs MHA with
     copied KV heads, shared latent V vs explicit copy);
  P7 append touches exactly its target slots; HND head slices are contiguous;
  P8 FLOP identity and the pages' closed form (section "flops");
  P9 the pages' IO worked example (section "io-overhead");
  P10 verify shapes: n drafts give qo_len n + 1; MTP verify gives 2 rows per
     request.
  P2s split execution (cache part over the pages before the append, chunk
     part over the new keys, merged) == attention after the append, and == the
     torch SDPA reference over the concatenated keys.
  PC page copies: an element loop over (page, head, slot, dim) with its own
     index arithmetic; two half-head shards rebuild the full pages; NHD is the
     slot/head transpose (element loop); nothing outside the target changes;
     copying a shared partly filled prefix page before two requests append
     gives the attention of private copies (torch SDPA reference).
  PT tree masks among the new tokens: a chain mask == causal attention; any
     mask == torch SDPA with the test's own boolean mask; relabeling the draft
     nodes permutes the outputs.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import Batch


# ----------------------------------------------------------------------------
# Helpers: the test's own placement of logical K/V into pages
# ----------------------------------------------------------------------------


def place(seqs, page_size, num_heads, dim, rng, extra_pages=0, slack=3, fill=np.nan):
    """Lay logical per-request sequences [L_r, H, d] out in a paged HND pool.

    Page ids are a random permutation; unused pages and tail slots hold
    ``fill``.  Returns (pool [num_pages, H, P, d], kv_page_indptr, kv_page_indices).
    """
    need = [-(-s.shape[0] // page_size) + extra_pages for s in seqs]
    total = sum(need)
    num_pages = total + slack
    perm = rng.permutation(num_pages)
    pool = np.full((num_pages, num_heads, page_size, dim), fill, dtype=np.float64)
    indptr = [0]
    indices = []
    cursor = 0
    for s, n_p in zip(seqs, need):
        pages = perm[cursor:cursor + n_p]
        cursor += n_p
        for j in range(s.shape[0]):
            pg = pages[j // page_size]
            sl = j % page_size
            for h in range(num_heads):
                pool[pg, h, sl, :] = s[j, h, :]
        indices.extend(int(p) for p in pages)
        indptr.append(len(indices))
    return pool, np.array(indptr), np.array(indices)


def random_case(rng, qo_lens, kv_lens, hq, hkv, d, dv, page_size, extra_pages=0):
    seqs_k = [rng.standard_normal((L, hkv, d)) for L in kv_lens]
    seqs_v = [rng.standard_normal((L, hkv, dv)) for L in kv_lens]
    seed_perm = int(rng.integers(1 << 30))
    k_pool, indptr, indices = place(seqs_k, page_size, hkv, d, np.random.default_rng(seed_perm),
                                    extra_pages)
    v_pool, indptr2, indices2 = place(seqs_v, page_size, hkv, dv,
                                      np.random.default_rng(seed_perm), extra_pages)
    assert np.array_equal(indices, indices2)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)])
    batch = Batch(qo_indptr, kv_lens, indptr, indices, page_size)
    q = rng.standard_normal((int(qo_indptr[-1]), hq, d))
    return q, seqs_k, seqs_v, k_pool, v_pool, batch


def torch_reference(q, seqs_k, seqs_v, qo_lens, kv_lens, hq, hkv, scale, causal=True,
                    new_masks=None):
    """Attention by torch's SDPA (float64) on contiguous logical K/V."""
    G = hq // hkv
    outs, lses = [], []
    i0 = 0
    for n, L, K, V in zip(qo_lens, kv_lens, seqs_k, seqs_v):
        if n == 0:
            continue
        c = L - n
        qt = torch.from_numpy(q[i0:i0 + n]).permute(1, 0, 2)            # [hq, n, d]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)  # [hq, L, d]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        t = torch.arange(n)[:, None]
        j = torch.arange(L)[None, :]
        mask = (j <= c + t) if causal else torch.ones(n, L, dtype=torch.bool)
        if new_masks is not None and new_masks[len(outs)] is not None:
            mask = mask.clone()
            mask[:, c:] = torch.from_numpy(np.asarray(new_masks[len(outs)], dtype=bool))
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=scale)
        s = (qt @ kt.transpose(1, 2)) * scale
        s = s.masked_fill(~mask, float("-inf"))
        lse = torch.logsumexp(s, dim=-1)
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(lse.permute(1, 0).numpy())
        i0 += n
    return np.concatenate(outs), np.concatenate(lses)


CASES = [
    # qo_lens, kv_lens, hq, hkv, d, dv, P
    ([1, 16], [37, 36], 4, 2, 64, 64, 16),
    ([3, 0, 5, 1], [3, 9, 40, 1], 8, 2, 16, 16, 4),
    ([7], [20], 4, 4, 8, 8, 1),
    ([2, 2, 2], [50, 2, 17], 8, 1, 24, 16, 16),
    ([4, 1], [70, 64], 4, 1, 32, 32, 64),
]


# ----------------------------------------------------------------------------
# bf16 helpers, pinned to torch's conversions
# ----------------------------------------------------------------------------


def test_bf16_conversions_match_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(10000).astype(np.float32) * 10,
        np.array([1.0, -2.5, 3.00390625, 1.00390625, 1.01171875, 0.0, -0.0, 65504.0,
                  1e-40, 3.4e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16)
    bits_ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits_rne(x), bits_ref)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits_ref), ref.to(torch.float64).numpy())


# ----------------------------------------------------------------------------
# P4: library routine
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_p4_attend_matches_torch_sdpa(case, causal):
    qo, kv, hq, hkv, d, dv, P = case
    rng = np.random.default_rng(hash((tuple(qo), tuple(kv), hq, causal)) % (1 << 31))
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, hq, hkv, d, dv, P, extra_pages=1)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attend(q, kp, vp, batch, hq, hkv, scale, causal=causal)
    o_ref, lse_ref = torch_reference(q, sk, sv, qo, kv, hq, hkv, scale, causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P3: brute force with scalar loops
# ----------------------------------------------------------------------------


def brute_force(q, k_pool, v_pool, qo_indptr, kv_len, indptr, indices, P, hq, hkv, scale):
    G = hq // hkv
    total = qo_indptr[-1]
    dv = v_pool.shape[-1]
    o = [[[0.0] * dv for _ in range(hq)] for _ in range(total)]
    lse = [[0.0] * hq for _ in range(total)]
    for r in range(len(kv_len)):
        n = qo_indptr[r + 1] - qo_indptr[r]
        c = kv_len[r] - n
        for t in range(n):
            i = qo_indptr[r] + t
            for h in range(hq):
                g = h // G
                scores = []
                vals = []
                for j in range(c + t + 1):
                    page = indices[indptr[r] + j // P]
                    slot = j % P
                    s = 0.0
                    for e in range(q.shape[2]):
                        s += float(q[i, h, e]) * float(k_pool[page, g, slot, e])
                    scores.append(s * scale)
                    vals.append([float(x) for x in v_pool[page, g, slot, :]])
                m = max(scores)
                z = sum(math.exp(s - m) for s in scores)
                lse[i][h] = m + math.log(z)
                for e in range(dv):
                    o[i][h][e] = sum(math.exp(s - m) / z * v[e] for s, v in zip(scores, vals))
    return np.array(o), np.array(lse)


def test_p3_brute_force_tiny():
    rng = np.random.default_rng(3)
    for qo, kv, hq, hkv, d, P in [([1, 3], [5, 9], 2, 1, 4, 4), ([2], [2], 4, 2, 3, 1),
                                  ([4, 1, 0], [11, 20, 3], 2, 2, 5, 16)]:
        q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, hq, hkv, d, d, P)
        scale = 0.7
        o, lse = oracle.attend(q, kp, vp, batch, hq, hkv, scale)
        o_b, lse_b = brute_force(q, kp, vp, list(batch.qo_indptr), list(batch.kv_len),
                                 list(batch.kv_page_indptr), list(batch.kv_page_indices), P,
                                 hq, hkv, scale)
        np.testing.assert_allclose(o, o_b, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P5: closed forms
# ----------------------------------------------------------------------------


def test_p5_single_key():
    rng = np.random.default_rng(5)
    q, sk, sv, kp, vp, batch = random_case(rng, [1], [1], 2, 1, 8, 6, 16)
    scale = 0.37
    o, lse = oracle.attend(q, kp, vp, batch, 2, 1, scale)
    for h in range(2):
        np.testing.assert_allclose(o[0, h], sv[0][0, 0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, h], scale * q[0, h] @ sk[0][0, 0], rtol=0, atol=1e-14)


def test_p5_zero_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(6)
    q, sk, sv, kp, vp, batch = random_case(rng, [4], [10], 2, 2, 8, 5, 4)
    kp = np.where(np.isnan(kp), np.nan, 0.0)
    o, lse = oracle.attend(q, kp, vp, batch, 2, 2, 1.0)
    for t in range(4):
        p = 6 + t
        for h in range(2):
            np.testing.assert_allclose(o[t, h], sv[0][:p + 1, h].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[t, h], math.log(p + 1), rtol=0, atol=1e-14)


def test_p5_equal_values_pass_through():
    rng = np.random.default_rng(7)
    q, sk, sv, kp, vp, batch = random_case(rng, [3, 2], [8, 30], 4, 2, 8, 8, 16)
    vconst = rng.standard_normal(8)
    vp = np.where(np.isnan(vp), np.nan, vconst[None, None, None, :])
    o, _ = oracle.attend(q, kp, vp, batch, 4, 2, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(vconst, o.shape), rtol=0, atol=1e-13)


def test_p5_two_keys_known_weights():
    # q.k0 = 0 and q.k1 = ln 3 (scale 1): weights 1/4 and 3/4, lse = ln 4.
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[0.0, 5.0]], [[math.log(3.0), -1.0]]])        # [L=2, H=1, d=2]
    v = np.array([[[4.0, -8.0]], [[0.0, 8.0]]])
    kp, indptr, indices = place([k], 2, 1, 2, np.random.default_rng(0))
    vp, _, _ = place([v], 2, 1, 2, np.random.default_rng(0))
    batch = Batch([0, 1], [2], indptr, indices, 2)
    o, lse = oracle.attend(q, kp, vp, batch, 1, 1, 1.0)
    np.testing.assert_allclose(o[0, 0], [1.0, 4.0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(4.0), rtol=0, atol=1e-15)


def test_p5_decode_sees_all_keys_and_causal_row_sees_itself():
    # A decode row (qo 1) must see every one of its kv_len keys; the first row of
    # a chunk with no cache sees exactly its own key.
    rng = np.random.default_rng(8)
    q, sk, sv, kp, vp, batch = random_case(rng, [1, 3], [9, 3], 1, 1, 4, 4, 4)
    o, _ = oracle.attend(q, kp, vp, batch, 1, 1, 1.0)
    np.testing.assert_allclose(o[1, 0], sv[1][0, 0], rtol=0, atol=1e-15)
    s = q[0, 0] @ sk[0][:, 0].T
    w = np.exp(s - s.max())
    w /= w.sum()
    np.testing.assert_allclose(o[0, 0], w @ sv[0][:, 0], rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# P2: merge of disjoint partitions
# ----------------------------------------------------------------------------


def test_p2_merge_equals_union():
    rng = np.random.default_rng(11)
    for trial in range(40):
        n, m, d, dv = int(rng.integers(1, 6)), int(rng.integers(1, 40)), 8, 5
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((m, d)) * 2
        v = rng.standard_normal((m, dv))
        base = rng.random((n, m)) < 0.8
        base[:, 0] = True                   # every row sees at least one key in the union
        part = rng.random(m) < rng.random()  # arbitrary partition, possibly empty
        if trial % 7 == 0:
            part[:] = False                  # A empty
        if trial % 11 == 0:
            part[:] = True                   # B empty
        vis_a = base & part[None, :]
        vis_b = base & ~part[None, :]
        o_a, l_a = oracle.attend_dense(q, k, v, 0.9, vis_a)
        o_b, l_b = oracle.attend_dense(q, k, v, 0.9, vis_b)
        o_u, l_u = oracle.attend_dense(q, k, v, 0.9, base)
        o_m, l_m = oracle.merge(o_a, l_a, o_b, l_b)
        np.testing.assert_allclose(o_m, o_u, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l_m, l_u, rtol=0, atol=1e-13)
        o_m2, l_m2 = oracle.merge(o_b, l_b, o_a, l_a)    # symmetric
        np.testing.assert_allclose(o_m2, o_u, rtol=0, atol=1e-13)


@pytest.mark.parametrize("qo,kv,hq,hkv,P", [
    ([1, 16, 0, 5], [37, 36, 4, 5], 4, 2, 16),     # decode, chunk on a cache, empty, first chunk
    ([3, 7], [40, 7], 8, 1, 4),
    ([2, 1, 6], [9, 64, 70], 2, 2, 64),
])
def test_p2s_split_execution_equals_attention_after_append(qo, kv, hq, hkv, P):
    rng = np.random.default_rng(sum(kv))
    d, dv, scale = 16, 8, 0.3
    seqs_k = [rng.standard_normal((L, hkv, d)) for L in kv]
    seqs_v = [rng.standard_normal((L, hkv, dv)) for L in kv]
    seed = int(rng.integers(1 << 30))
    kp, indptr, indices = place(seqs_k, P, hkv, d, np.random.default_rng(seed))
    vp, _, _ = place(seqs_v, P, hkv, dv, np.random.default_rng(seed))
    qo_indptr = np.concatenate([[0], np.cumsum(qo)])
    batch = Batch(qo_indptr, kv, indptr, indices, P)
    # the pool before the append: the new tokens' slots are NaN, so the split
    # form must not read them
    kp0 = kp.copy()
    vp0 = vp.copy()
    for r, (n, L) in enumerate(zip(qo, kv)):
        for t in range(L - n, L):
            pg, sl = oracle.slot_of(batch, r, t)
            kp0[pg, :, sl, :] = np.nan
            vp0[pg, :, sl, :] = np.nan
    k_new = np.concatenate([s[L - n:] for s, L, n in zip(seqs_k, kv, qo)])
    v_new = np.concatenate([s[L - n:] for s, L, n in zip(seqs_v, kv, qo)])
    q = rng.standard_normal((int(qo_indptr[-1]), hq, d))
    o_s, l_s = oracle.split_attention(q, kp0, vp0, k_new, v_new, batch, hq, hkv, scale)
    kp1, vp1 = oracle.append(kp0, vp0, k_new, v_new, batch)
    np.testing.assert_array_equal(kp1, kp)           # the append restores the full pool
    o_a, l_a = oracle.attend(q, kp1, vp1, batch, hq, hkv, scale)
    np.testing.assert_allclose(o_s, o_a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_s, l_a, rtol=0, atol=1e-12)
    o_t, l_t = torch_reference(q, seqs_k, seqs_v, qo, kv, hq, hkv, scale)
    rows = np.concatenate([np.arange(qo_indptr[r], qo_indptr[r + 1]) for r in range(len(qo))])
    np.testing.assert_allclose(o_s[rows], o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_s[rows], l_t, rtol=0, atol=1e-12)


def test_p2_merge_of_two_empty_partials_is_empty():
    o, lse = oracle.merge(np.zeros((2, 3)), np.full(2, -np.inf), np.zeros((2, 3)),
                          np.full(2, -np.inf))
    assert np.all(lse == -np.inf) and np.all(o == 0) and not np.any(np.isnan(o))


def test_p2_merge_is_associative():
    rng = np.random.default_rng(12)
    parts = [(rng.standard_normal((4, 3)), rng.standard_normal(4) * 3) for _ in range(3)]
    (a, la), (b, lb), (c, lc) = parts
    x1 = oracle.merge(*oracle.merge(a, la, b, lb), c, lc)
    x2 = oracle.merge(a, la, *oracle.merge(b, lb, c, lc))
    np.testing.assert_allclose(x1[0], x2[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(x1[1], x2[1], rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# P1: chunked == one-shot
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("L,C,P,hq,hkv,bits", [
    (1, 4, 16, 2, 1, False), (7, 3, 4, 2, 2, False), (100, 16, 16, 4, 1, True),
    (257, 64, 16, 8, 1, True), (300, 100, 1, 2, 1, False), (130, 130, 64, 4, 2, True),
    (1024, 128, 16, 8, 1, True),
])
def test_p1_chunked_equals_one_shot(L, C, P, hq, hkv, bits):
    rng = np.random.default_rng(L * 31 + C)
    d = 16
    q = rng.standard_normal((L, hq, d))
    kn = rng.standard_normal((L, hkv, d))
    vn = rng.standard_normal((L, hkv, d))
    n_pages = -(-L // P)
    num_pages = n_pages + 5
    pages = rng.permutation(num_pages)[:n_pages]
    if bits:
        to64 = oracle.bf16_bits_to_f64
        q, kn, vn = (oracle.f32_to_bf16_bits_rne(x.astype(np.float32)) for x in (q, kn, vn))
        kp = np.full((num_pages, hkv, P, d), 0x7FC0, dtype=np.uint16)
        vp = kp.copy()
    else:
        to64 = None
        kp = np.full((num_pages, hkv, P, d), np.nan)
        vp = kp.copy()
    o_c, l_c, kp_c, vp_c = oracle.chunked_prefill(q, kn, vn, kp, vp, pages, P, C, hq, hkv,
                                                  0.25, to_f64=to64)
    o_1, l_1, kp_1, vp_1 = oracle.one_shot_prefill(q, kn, vn, kp, vp, pages, P, hq, hkv, 0.25,
                                                   to_f64=to64)
    assert kp_c.tobytes() == kp_1.tobytes() and vp_c.tobytes() == vp_1.tobytes()
    np.testing.assert_allclose(o_c, o_1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_1, rtol=0, atol=1e-12)
    # The cache holds the prompt's K at the slots the layout defines.
    kc = kp_c if not bits else kp_c
    for j in [0, L // 2, L - 1]:
        assert kc[pages[j // P], :, j % P, :].tobytes() == kn[j].tobytes()


# ----------------------------------------------------------------------------
# P6: invariances
# ----------------------------------------------------------------------------


def test_p6_page_permutation_and_page_size_invariance():
    rng = np.random.default_rng(21)
    qo, kv, hq, hkv, d = [1, 5, 2], [33, 40, 2], 4, 2, 8
    seqs_k = [rng.standard_normal((L, hkv, d)) for L in kv]
    seqs_v = [rng.standard_normal((L, hkv, d)) for L in kv]
    q = rng.standard_normal((sum(qo), hq, d))
    results = []
    for P, seed in [(1, 1), (4, 2), (16, 3), (16, 4), (64, 5)]:
        kp, ip, ix = place(seqs_k, P, hkv, d, np.random.default_rng(seed), extra_pages=seed % 2)
        vp, _, _ = place(seqs_v, P, hkv, d, np.random.default_rng(seed), extra_pages=seed % 2)
        batch = Batch(np.concatenate([[0], np.cumsum(qo)]), kv, ip, ix, P)
        results.append(oracle.attend(q, kp, vp, batch, hq, hkv, 0.3))
    for o, lse in results[1:]:
        np.testing.assert_allclose(o, results[0][0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, results[0][1], rtol=0, atol=1e-13)


def test_p6_request_order_invariance():
    rng = np.random.default_rng(22)
    qo, kv = [1, 3, 2], [10, 12, 5]
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, 2, 1, 8, 8, 4)
    o, lse = oracle.attend(q, kp, vp, batch, 2, 1, 0.4)
    order = [2, 0, 1]
    qo_p = [qo[r] for r in order]
    kv_p = [kv[r] for r in order]
    starts = np.concatenate([[0], np.cumsum(qo)])
    q_p = np.concatenate([q[starts[r]:starts[r + 1]] for r in order])
    ip = [0]
    ix = []
    for r in order:
        ix.extend(batch.pages(r))
        ip.append(len(ix))
    b_p = Batch(np.concatenate([[0], np.cumsum(qo_p)]), kv_p, ip, ix, 4)
    o_p, lse_p = oracle.attend(q_p, kp, vp, b_p, 2, 1, 0.4)
    o_back = np.concatenate([o[starts[r]:starts[r + 1]] for r in order])
    np.testing.assert_allclose(o_p, o_back, rtol=0, atol=0)


def test_p6_gqa_equals_mha_with_copied_kv_heads():
    rng = np.random.default_rng(23)
    qo, kv, hq, hkv, d = [2, 1], [9, 20], 8, 2, 8
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, hq, hkv, d, d, 4)
    o_g, l_g = oracle.attend(q, kp, vp, batch, hq, hkv, 0.5)
    G = hq // hkv
    kp_m = np.repeat(kp, G, axis=1)    # KV head g copied to heads gG .. gG+G-1
    vp_m = np.repeat(vp, G, axis=1)
    o_m, l_m = oracle.attend(q, kp_m, vp_m, batch, hq, hq, 0.5)
    np.testing.assert_allclose(o_g, o_m, rtol=0, atol=0)
    np.testing.assert_allclose(l_g, l_m, rtol=0, atol=0)


def test_p6_shared_latent_equals_explicit_value_copy():
    rng = np.random.default_rng(24)
    qo, kv, hq, d, dv = [2, 2], [70, 9], 16, 24, 16
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, hq, 1, d, d, 64)
    o_s, l_s = oracle.attend(q, kp, None, batch, hq, 1, 0.2, head_dim_v=dv)
    o_e, l_e = oracle.attend(q, kp, kp[..., :dv].copy(), batch, hq, 1, 0.2)
    np.testing.assert_allclose(o_s, o_e, rtol=0, atol=0)
    np.testing.assert_allclose(l_s, l_e, rtol=0, atol=0)


# ----------------------------------------------------------------------------
# P7: append bits
# ----------------------------------------------------------------------------


def test_p7_append_touches_exactly_the_target_slots():
    rng = np.random.default_rng(31)
    qo, kv, P, hkv, d = [1, 4, 0, 3], [6, 9, 4, 3], 4, 2, 8
    meta = workloads.make_meta(qo, kv, P, seed=5, extra_pages_per_req=1)
    batch = Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices, P)
    kp = rng.integers(0, 1 << 16, size=(meta.num_pages, hkv, P, d), dtype=np.uint16)
    kp[0, 0, 0, 0] = 0x7FC0
    vp = rng.integers(0, 1 << 16, size=(meta.num_pages, hkv, P, d), dtype=np.uint16)
    kn = rng.integers(0, 1 << 16, size=(sum(qo), hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, size=(sum(qo), hkv, d), dtype=np.uint16)
    k2, v2 = oracle.append(kp, vp, kn, vn, batch)
    expect_k = kp.copy()
    expect_v = vp.copy()
    i = 0
    for r in range(len(qo)):
        pages = meta.kv_page_indices[meta.kv_page_indptr[r]:meta.kv_page_indptr[r + 1]]
        for t in range(qo[r]):
            pos = kv[r] - qo[r] + t
            expect_k[pages[pos // P], :, pos % P, :] = kn[i]
            expect_v[pages[pos // P], :, pos % P, :] = vn[i]
            i += 1
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    changed = np.argwhere(np.any(k2 != kp, axis=-1))
    assert len(changed) <= sum(qo) * hkv


def test_p7_append_shared_latent_writes_only_k():
    rng = np.random.default_rng(32)
    meta = workloads.make_meta([2], [66], 64, seed=1)
    batch = Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices, 64)
    kp = np.full((meta.num_pages, 1, 64, 12), 0x7FC0, dtype=np.uint16)
    kn = rng.integers(0, 1 << 15, size=(2, 1, 12), dtype=np.uint16)
    k2, v2 = oracle.append(kp, None, kn, None, batch)
    assert v2 is None
    pg = meta.kv_page_indices[1]
    assert np.array_equal(k2[pg, 0, 0:2], kn[:, 0])
    assert np.sum(k2 != kp) == 24


def test_p7_hnd_head_slice_is_contiguous():
    # In an HND pool [pages][H][P][d] (C order), heads h0..h1-1 of one page are
    # one contiguous run of (h1 - h0) * P * d elements.
    H, P, d = 8, 16, 128
    pool = np.arange(3 * H * P * d).reshape(3, H, P, d)
    for h0, h1 in [(0, 8), (2, 5), (7, 8)]:
        sl = pool[1, h0:h1]
        assert sl.flags["C_CONTIGUOUS"]
        flat = sl.reshape(-1)
        assert np.array_equal(flat, np.arange(flat[0], flat[0] + (h1 - h0) * P * d))


# ----------------------------------------------------------------------------
# P8, P9: the pages' accounting
# ----------------------------------------------------------------------------


def test_p8_flop_identity(golden_dir):
    with open(os.path.join(golden_dir, "flops_identity.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        L, C, d, hq = case["L"], case["C"], case["head_dim"], case["num_qo_heads"]
        one = oracle.accounting(Batch([0, L], [L], [0, 1], [0], L + 1), hq, 1, d, d, 2)
        tot_pairs = 0
        tot_flops = 0
        for s in range(-(-L // C)):
            n = min(C, L - s * C)
            acc = oracle.accounting(Batch([0, n], [s * C + n], [0, 1], [0], L + 1), hq, 1, d, d, 2)
            tot_pairs += acc["pairs"]
            tot_flops += acc["flops"]
        assert one["pairs"] == tot_pairs == case["pairs_per_head"] == L * (L + 1) // 2
        assert one["flops"] == tot_flops == case["attention_flops"]


def test_p8_accounting_counts_visible_pairs():
    rng = np.random.default_rng(41)
    q, sk, sv, kp, vp, batch = random_case(rng, [3, 1, 0], [10, 4, 2], 2, 1, 4, 4, 4)
    acc = oracle.accounting(batch, 2, 1, 4, 4, 2)
    assert acc["pairs"] == (8 + 9 + 10) + 4
    assert acc["kv_bytes"] == 16 * 1 * 8 * 2
    assert acc["append_bytes"] == 4 * 1 * 8 * 2
    acc_nc = oracle.accounting(batch, 2, 1, 4, 4, 2, causal=False)
    assert acc_nc["pairs"] == 3 * 10 + 4


def test_p9_io_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "io_overhead_example.json")) as f:
        g = json.load(f)
    assert oracle.kv_write_bytes_per_chunk(g["chunk"], g["n_layers"], g["n_kv_heads"],
                                           g["head_dim"], g["elem_bytes"]) == g["bytes"]
    # Per layer, the same bytes are what the append of one chunk writes.
    b = Batch([0, 512], [512], [0, 32], np.arange(32), 16)
    acc = oracle.accounting(b, 32, 8, 128, 128, 2)
    assert acc["append_bytes"] * g["n_layers"] == g["bytes"]


def test_chunk_schedule(golden_dir):
    with open(os.path.join(golden_dir, "chunk_schedule.json")) as f:
        g = json.load(f)
    L, C = g["prompt_len"], g["chunk"]
    n = -(-L // C)
    assert n == g["iterations"]
    got = [[s * C, min(L, s * C + C) - 1] for s in range(n)]
    assert got == g["chunks_0_indexed_inclusive"]


# ----------------------------------------------------------------------------
# P10: verify shapes
# ----------------------------------------------------------------------------


def test_p10_verify_shapes():
    qo, kv = workloads.lengths("decode_verify_gqa")
    assert set(qo[1::2]) == {3 + 1} and set(qo[0::2]) == {1}
    assert np.all(kv >= 1024) and np.all(kv <= 32768)
    qo5, _ = workloads.lengths("mla_absorbed")
    assert int(qo5.sum()) == 2 * len(qo5) == 128
    qo2, kv2 = workloads.lengths("mixed_7b")
    assert qo2[-1] == 512 and kv2[-1] == 1536 and np.all(qo2[:-1] == 1)



# ----------------------------------------------------------------------------
# PT: tree masks among the new tokens
# ----------------------------------------------------------------------------


def random_tree(rng, n):
    """Ancestor-or-self mask of a random rooted tree on n nodes labelled in
    creation order (a node's parent has a smaller label)."""
    parent = [-1] + [int(rng.integers(0, u)) for u in range(1, n)]
    m = np.zeros((n, n), dtype=bool)
    for t in range(n):
        u = t
        while u >= 0:
            m[t, u] = True
            u = parent[u]
    return m


def test_pt_chain_mask_equals_causal():
    rng = np.random.default_rng(41)
    qo, kv = [4, 1, 7], [40, 9, 7]
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, 8, 2, 16, 16, 16)
    chains = [np.tril(np.ones((n, n), dtype=bool)) for n in qo]
    o_t, l_t = oracle.attend(q, kp, vp, batch, 8, 2, 0.4, tree=chains)
    o_c, l_c = oracle.attend(q, kp, vp, batch, 8, 2, 0.4)
    np.testing.assert_allclose(o_t, o_c, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_t, l_c, rtol=0, atol=1e-13)


def test_pt_tree_mask_matches_torch_sdpa():
    rng = np.random.default_rng(42)
    qo, kv = [5, 0, 9, 3], [30, 4, 9, 70]
    q, sk, sv, kp, vp, batch = random_case(rng, qo, kv, 4, 2, 16, 8, 4)
    masks = [random_tree(rng, 5), None, random_tree(rng, 9), None]
    o, lse = oracle.attend(q, kp, vp, batch, 4, 2, 0.3, tree=masks)
    o_t, l_t = torch_reference(q, sk, sv, qo, kv, 4, 2, 0.3,
                               new_masks=[m for m, n in zip(masks, qo) if n > 0])
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_t, rtol=0, atol=1e-12)
    # a non-causal pattern (a node seeing a later sibling) is honoured too
    odd = [np.eye(5, dtype=bool) | np.eye(5, k=1, dtype=bool), None, random_tree(rng, 9), None]
    o2, l2 = oracle.attend(q, kp, vp, batch, 4, 2, 0.3, tree=odd)
    o_t2, l_t2 = torch_reference(q, sk, sv, qo, kv, 4, 2, 0.3,
                                 new_masks=[m for m, n in zip(odd, qo) if n > 0])
    np.testing.assert_allclose(o2, o_t2, rtol=0, atol=1e-12)


def test_pt_relabeling_draft_nodes_permutes_outputs():
    rng = np.random.default_rng(43)
    n, c, hq, hkv, d = 6, 25, 4, 1, 8
    k_all = rng.standard_normal((c + n, hkv, d))
    v_all = rng.standard_normal((c + n, hkv, d))
    q = rng.standard_normal((n, hq, d))
    m = random_tree(rng, n)
    perm = rng.permutation(n)          # new label of node u is perm[u]
    inv = np.argsort(perm)
    k2 = np.concatenate([k_all[:c], k_all[c:][inv]])
    v2 = np.concatenate([v_all[:c], v_all[c:][inv]])
    m2 = m[np.ix_(inv, inv)]
    outs = []
    for kk, vv, qq, mm in ((k_all, v_all, q, m), (k2, v2, q[inv], m2)):
        kp, indptr, indices = place([kk], 4, hkv, d, np.random.default_rng(1))
        vp, _, _ = place([vv], 4, hkv, d, np.random.default_rng(1))
        b = Batch([0, n], [c + n], indptr, indices, 4)
        outs.append(oracle.attend(qq, kp, vp, b, hq, hkv, 0.5, tree=[mm]))
    np.testing.assert_allclose(outs[1][0], outs[0][0][inv], rtol=0, atol=1e-13)
    np.testing.assert_allclose(outs[1][1], outs[0][1][inv], rtol=0, atol=1e-13)



# ----------------------------------------------------------------------------
# PC: page copies
# ----------------------------------------------------------------------------


def test_pc_copy_pages_element_loop_and_untouched_bytes():
    rng = np.random.default_rng(51)
    src = rng.standard_normal((7, 4, 8, 6))
    dst = np.full((9, 4, 8, 6), np.nan)
    sp, dp = [3, 0, 6], [8, 2, 5]
    out = oracle.copy_pages(src, dst, sp, dp, 1, 2, 2)
    want = dst.copy()
    for i in range(3):
        for hh in range(2):
            for sl in range(8):
                for e in range(6):
                    want[dp[i], 2 + hh, sl, e] = src[sp[i], 1 + hh, sl, e]
    np.testing.assert_array_equal(out, want)
    assert np.isnan(out[[0, 1, 3, 4, 6, 7]]).all()
    assert np.isnan(out[dp][:, [0, 1]]).all()


def test_pc_half_shards_rebuild_full_pages_and_nhd_is_a_transpose():
    rng = np.random.default_rng(52)
    H, P, d = 8, 16, 4
    pool = rng.standard_normal((20, H, P, d))
    pages = rng.permutation(20)[:6]
    ident = np.arange(6)
    lo = oracle.copy_pages(pool, np.zeros((6, H // 2, P, d)), pages, ident, 0, 0, H // 2)
    hi = oracle.copy_pages(pool, np.zeros((6, H // 2, P, d)), pages, ident, H // 2, 0, H // 2)
    rebuilt = np.full((30, H, P, d), np.nan)
    dst_pages = rng.permutation(30)[:6]
    rebuilt = oracle.copy_pages(lo, rebuilt, ident, dst_pages, 0, 0, H // 2)
    rebuilt = oracle.copy_pages(hi, rebuilt, ident, dst_pages, 0, H // 2, H // 2)
    np.testing.assert_array_equal(rebuilt[dst_pages], pool[pages])
    nhd = oracle.hnd_to_nhd(pool[pages])
    for i in range(6):
        for sl in range(P):
            for h in range(H):
                np.testing.assert_array_equal(nhd[i, sl, h], pool[pages[i], h, sl])


def test_pc_copy_shared_tail_page_then_append_matches_private_copies():
    # Two requests share a 40-token prefix over pages of 16: pages 0, 1 are
    # full and shared read-only; the tail page (8 tokens) is copied for the
    # second request before both append their own tokens.
    rng = np.random.default_rng(53)
    H, P, d, hq = 2, 16, 8, 4
    prefix_k = rng.standard_normal((40, H, d))
    prefix_v = rng.standard_normal((40, H, d))
    own = [rng.standard_normal((n, H, d)) for n in (5, 12)]
    own_v = [rng.standard_normal((n, H, d)) for n in (5, 12)]
    kp, indptr, indices = place([prefix_k], P, H, d, np.random.default_rng(3), slack=4)
    vp, _, _ = place([prefix_v], P, H, d, np.random.default_rng(3), slack=4)
    shared = [int(x) for x in indices]            # 3 pages
    free = [x for x in range(kp.shape[0]) if x not in shared]
    tail_copy = free[0]
    kp = oracle.copy_pages(kp, kp, [shared[2]], [tail_copy], 0, 0, H)
    vp = oracle.copy_pages(vp, vp, [shared[2]], [tail_copy], 0, 0, H)
    extra = free[1:3]                             # the second request grows past its tail
    tables = [shared, shared[:2] + [tail_copy, extra[0]]]
    batch = Batch([0, 5, 17], [45, 52], [0, 3, 7], tables[0] + tables[1], P)
    k_new = np.concatenate(own)
    v_new = np.concatenate(own_v)
    kp2, vp2 = oracle.append(kp, vp, k_new, v_new, batch)
    q = rng.standard_normal((17, hq, d))
    o, lse = oracle.attend(q, kp2, vp2, batch, hq, H, 0.35)
    seqs_k = [np.concatenate([prefix_k, own[0]]), np.concatenate([prefix_k, own[1]])]
    seqs_v = [np.concatenate([prefix_v, own_v[0]]), np.concatenate([prefix_v, own_v[1]])]
    o_t, l_t = torch_reference(q, seqs_k, seqs_v, [5, 12], [45, 52], hq, H, 0.35)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_t, rtol=0, atol=1e-12)
    # the shared full pages are unchanged by either append
    np.testing.assert_array_equal(kp2[shared[:2]], kp[shared[:2]])
