"""fp64 reference for ragged paged attention with KV append (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module.  It is written straight from the definitions on the pages, with no
blocking, fusion or reordering beyond what those definitions state; numpy's
matmul, exp and log are the only library steps.

Notation (per request r of a batch):
  n_r   = qo_len, the number of new query tokens;
  L_r   = kv_len, cached plus new keys (the new tokens are the last n_r);
  c_r   = L_r - n_r, the number of keys already in the cache;
  P     = page size in tokens;
  G     = num_qo_heads / num_kv_heads (query heads per KV head).
The new token t of request r has global index i = qo_indptr[r] + t and sits at
absolute position p = c_r + t.

Readings of points the pages leave open (each is also listed in the design
notes of the repository):
  * kv_len counts the new tokens as well ("history cache + current chunk" in
    the chunked-prefill post, section "correctness");
  * causal alignment is bottom-right: query t sees keys j <= c_r + t;
  * consecutive query heads share a KV head: kv head of query head h is h // G;
  * the log-sum-exp is the natural log of the sum of exp(scaled score);
  * the page table is CSR (kv_page_indptr, kv_page_indices); page entries
    past ceil(L_r / P) are ignored;
  * a row with no visible key (only possible for a partial over a key subset)
    has lse = -inf and output 0; merging with such a partial returns the
    other one.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# Batch description
# ----------------------------------------------------------------------------


@dataclass
class Batch:
    """Ragged batch metadata: per-request qo_len and kv_len plus a CSR page table.

    Follows "Accelerating Sonar through speculation" (Perplexity), runtime
    section: the batch carries the new tokens and the page information of
    every request; and "Disaggregated prefill and decode", performance section:
    qo_len new tokens against kv_len cached entries.
    """

    qo_indptr: np.ndarray
    kv_len: np.ndarray
    kv_page_indptr: np.ndarray
    kv_page_indices: np.ndarray
    page_size: int

    def __post_init__(self):
        self.qo_indptr = np.asarray(self.qo_indptr, dtype=np.int64)
        self.kv_len = np.asarray(self.kv_len, dtype=np.int64)
        self.kv_page_indptr = np.asarray(self.kv_page_indptr, dtype=np.int64)
        self.kv_page_indices = np.asarray(self.kv_page_indices, dtype=np.int64)

    @property
    def batch_size(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    def qo_len(self, r: int) -> int:
        return int(self.qo_indptr[r + 1] - self.qo_indptr[r])

    def cached_len(self, r: int) -> int:
        return int(self.kv_len[r]) - self.qo_len(r)

    def pages(self, r: int) -> np.ndarray:
        return self.kv_page_indices[self.kv_page_indptr[r]:self.kv_page_indptr[r + 1]]


# ----------------------------------------------------------------------------
# dtype handling
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their raw uint16 bit patterns.

    A bfloat16 number is the upper half of an IEEE binary32 number, so
    shifting the 16 bits into the top of a 32-bit word gives the same value
    as a float32, which widens to float64 exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Used only where a test needs the oracle's own rounding of an fp64 result
    to the output dtype.  NaN stays NaN (quiet).
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    out[nan] = np.uint16(0x7FC0)
    return out


# ----------------------------------------------------------------------------
# O0: page-table gather (HND layout)
# ----------------------------------------------------------------------------


def slot_of(batch: Batch, r: int, pos: int) -> tuple[int, int]:
    """Physical (page id, slot) of absolute position ``pos`` of request ``r``.

    Logical key j of a request lives in the (j // P)-th page of its page list,
    at slot j % P of that page.
    """
    P = batch.page_size
    return int(batch.pages(r)[pos // P]), pos % P


def gather(pool: np.ndarray, batch: Batch, r: int, head: int, n_tokens: int) -> np.ndarray:
    """Keys (or values) 0..n_tokens-1 of request r for one KV head.

    ``pool`` has the HND shape [num_pages, num_kv_heads, page_size, dim]: the
    head dimension comes before the token dimension inside a page
    ("Disaggregated prefill and decode", sharded-transfer section).
    Returns an array [n_tokens, dim] of the pool's dtype.
    """
    P = batch.page_size
    j = np.arange(n_tokens)
    pages = batch.pages(r)[j // P]
    return pool[pages, head, j % P, :]


# ----------------------------------------------------------------------------
# O1: KV append
# ----------------------------------------------------------------------------


def append(k_pool: np.ndarray, v_pool, k_new: np.ndarray, v_new, batch: Batch):
    """Write every new token's K (and V) into its page slot; return new pools.

    For request r, new token t and KV head h the K row k_new[i, h, :] goes to
    page pages_r[(c_r + t) // P], head h, slot (c_r + t) % P (and the same for
    V).  This is the per-layer append of "Disaggregated prefill and decode"
    (KV Messenger section) and the cache update K_cache += [k ...] of the
    chunked-prefill post (section "correctness").

    The copy is a raw copy of the stored elements (pass bfloat16 data as its
    uint16 bits), so every byte outside the target slots is left unchanged.
    ``v_new`` / ``v_pool`` may be None for a shared latent cache (only the
    latent rows are stored; values are a view of them).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = None if v_pool is None else np.array(v_pool, copy=True)
    num_kv_heads = k_pool.shape[1]
    for r in range(batch.batch_size):
        n = batch.qo_len(r)
        c = batch.cached_len(r)
        for t in range(n):
            i = int(batch.qo_indptr[r]) + t
            page, slot = slot_of(batch, r, c + t)
            for h in range(num_kv_heads):
                k_out[page, h, slot, :] = k_new[i, h, :]
                if v_new is not None and v_out is not None:
                    v_out[page, h, slot, :] = v_new[i, h, :]
    return k_out, v_out


# ----------------------------------------------------------------------------
# O2: attention
# ----------------------------------------------------------------------------


def attend_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 visible: np.ndarray):
    """Softmax attention of query rows over key rows, restricted to a mask.

    q [n, d_qk], k [m, d_qk], v [m, d_v], visible [n, m] (bool).  For each
    row: s_j = scale * <q, k_j> over visible j, lse = ln sum_j exp(s_j), and
    o = sum_j exp(s_j - lse) v_j.  A row with no visible key gets lse = -inf
    and o = 0.  Everything in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    if n == 0 or k.shape[0] == 0:
        return o, lse
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1)
    has = np.isfinite(m)
    if not np.any(has):
        return o, lse
    sh = s[has]
    mh = m[has]
    e = np.exp(sh - mh[:, None])
    tot = np.sum(e, axis=1)
    lse_h = mh + np.log(tot)
    w = np.exp(sh - lse_h[:, None])
    o[has] = w @ v
    lse[has] = lse_h
    return o, lse


def attend(q: np.ndarray, k_pool: np.ndarray, v_pool, batch: Batch,
           num_qo_heads: int, num_kv_heads: int, sm_scale: float,
           head_dim_v: int | None = None, causal: bool = True, tree=None):
    """Batched ragged causal attention over a paged KV cache, in float64.

    q: [total_q, num_qo_heads, d_qk] (float64).  k_pool / v_pool: HND pools
    [num_pages, num_kv_heads, P, d] (float64).  ``v_pool=None`` means values
    are the first ``head_dim_v`` dims of the key rows (shared latent cache).

    Query token t of request r, head h, attends to keys j = 0 .. c_r + t of KV
    head h // G of its own request (all kv_len keys when causal is False).

    ``tree``: optional list with one entry per request, None or a boolean
    [n_r, n_r] matrix; for such a request new token t sees every cached key
    and new token u iff tree[r][t, u] (verification of a draft tree under a
    custom attention mask, "Accelerating Sonar through speculation", EAGLE
    section).
    Returns (o [total_q, num_qo_heads, d_v], lse [total_q, num_qo_heads]).
    """
    if num_qo_heads % num_kv_heads != 0:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = num_qo_heads // num_kv_heads
    d_v = head_dim_v if head_dim_v is not None else (
        v_pool.shape[-1] if v_pool is not None else k_pool.shape[-1])
    total_q = batch.total_q
    o = np.zeros((total_q, num_qo_heads, d_v), dtype=np.float64)
    lse = np.full((total_q, num_qo_heads), -np.inf, dtype=np.float64)
    for r in range(batch.batch_size):
        n = batch.qo_len(r)
        if n == 0:
            continue
        L = int(batch.kv_len[r])
        c = L - n
        i0 = int(batch.qo_indptr[r])
        t_idx = np.arange(n)[:, None]
        j_idx = np.arange(L)[None, :]
        visible = (j_idx <= c + t_idx) if causal else np.ones((n, L), dtype=bool)
        if tree is not None and tree[r] is not None:
            among_new = np.asarray(tree[r], dtype=bool)
            visible = np.concatenate([np.ones((n, c), dtype=bool), among_new], axis=1)
        for g in range(num_kv_heads):
            kk = gather(k_pool, batch, r, g, L)
            if v_pool is None:
                vv = kk[:, :d_v]
            else:
                vv = gather(v_pool, batch, r, g, L)[:, :d_v]
            for hh in range(group):
                h = g * group + hh
                o_r, lse_r = attend_dense(q[i0:i0 + n, h, :], kk, vv, sm_scale, visible)
                o[i0:i0 + n, h, :] = o_r
                lse[i0:i0 + n, h] = lse_r
    return o, lse


# ----------------------------------------------------------------------------
# O3: softmax merge
# ----------------------------------------------------------------------------


def merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """Combine attention states of two disjoint key partitions.

    The chunked-prefill post (section "correctness") joins the attention to
    the cache and the attention within the chunk with an online-softmax
    merge.  With partial results (o_x, lse_x), x in {a, b}:
    lse = ln(e^{lse_a} + e^{lse_b}) and o = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b.
    A partition with lse = -inf contributes nothing; both -inf gives
    (-inf, 0).  Shapes: o_* [..., d], lse_* [...].
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    ea = np.where(np.isfinite(lse_a), np.exp(lse_a - m_safe), 0.0)
    eb = np.where(np.isfinite(lse_b), np.exp(lse_b - m_safe), 0.0)
    tot = ea + eb
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wa = np.where(finite, ea / np.where(finite, tot, 1.0), 0.0)
    wb = np.where(finite, eb / np.where(finite, tot, 1.0), 0.0)
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse


# ----------------------------------------------------------------------------
# O3b: split execution (cache part + chunk part, merged)
# ----------------------------------------------------------------------------


def split_attention(q: np.ndarray, k_pool: np.ndarray, v_pool, k_new: np.ndarray, v_new,
                    batch: Batch, num_qo_heads: int, num_kv_heads: int, sm_scale: float,
                    head_dim_v: int | None = None):
    """The chunked-prefill post's split form of one step (section "correctness").

    The step's new tokens of request r attend to the c_r cached keys held in
    the pages, each new token seeing all of them (the "history cache"), and,
    causally, to the step's own keys k_new / v_new (token t sees new tokens
    0 .. t: the "current chunk"); the two partial states are joined with the
    softmax merge (O3).  The pages are read without the new tokens, so the
    result does not depend on whether the append has run.  All inputs are
    float64; k_new / v_new are token-major [total_q, num_kv_heads, d].
    Returns (o, lse) like ``attend``.
    """
    group = num_qo_heads // num_kv_heads
    d_v = head_dim_v if head_dim_v is not None else v_new.shape[-1]
    cached = np.array([batch.cached_len(r) for r in range(batch.batch_size)], dtype=np.int64)
    cache_batch = Batch(batch.qo_indptr, cached, batch.kv_page_indptr, batch.kv_page_indices,
                        batch.page_size)
    o_a, lse_a = attend(q, k_pool, v_pool, cache_batch, num_qo_heads, num_kv_heads, sm_scale,
                        head_dim_v=d_v, causal=False)
    o_b = np.zeros_like(o_a)
    lse_b = np.full_like(lse_a, -np.inf)
    for r in range(batch.batch_size):
        n = batch.qo_len(r)
        if n == 0:
            continue
        i0 = int(batch.qo_indptr[r])
        visible = np.arange(n)[None, :] <= np.arange(n)[:, None]
        for g in range(num_kv_heads):
            kk = k_new[i0:i0 + n, g, :]
            vv = v_new[i0:i0 + n, g, :d_v]
            for hh in range(group):
                h = g * group + hh
                o_r, lse_r = attend_dense(q[i0:i0 + n, h, :], kk, vv, sm_scale, visible)
                o_b[i0:i0 + n, h, :] = o_r
                lse_b[i0:i0 + n, h] = lse_r
    return merge(o_a, lse_a, o_b, lse_b)


# ----------------------------------------------------------------------------
# O4: chunked prefill driver
# ----------------------------------------------------------------------------


def _prefill_steps(q, k_new, v_new, k_pool, v_pool, pages, page_size, chunk,
                   num_qo_heads, num_kv_heads, sm_scale, to_f64, head_dim_v=None):
    L = q.shape[0]
    pages = np.asarray(pages, dtype=np.int64)
    d_v = head_dim_v if head_dim_v is not None else (
        v_new.shape[-1] if v_new is not None else k_new.shape[-1])
    o = np.zeros((L, num_qo_heads, d_v), dtype=np.float64)
    lse = np.zeros((L, num_qo_heads), dtype=np.float64)
    n_chunks = -(-L // chunk)
    for s in range(n_chunks):
        start = s * chunk
        n = min(chunk, L - start)
        batch = Batch(qo_indptr=[0, n], kv_len=[start + n],
                      kv_page_indptr=[0, len(pages)], kv_page_indices=pages,
                      page_size=page_size)
        k_pool, v_pool = append(k_pool, v_pool, k_new[start:start + n],
                                None if v_new is None else v_new[start:start + n], batch)
        o_s, lse_s = attend(to_f64(q[start:start + n]), to_f64(k_pool),
                            None if v_pool is None else to_f64(v_pool), batch,
                            num_qo_heads, num_kv_heads, sm_scale, head_dim_v=d_v)
        o[start:start + n] = o_s
        lse[start:start + n] = lse_s
    return o, lse, k_pool, v_pool


def chunked_prefill(q, k_new, v_new, k_pool, v_pool, pages, page_size, chunk,
                    num_qo_heads, num_kv_heads, sm_scale, to_f64=None, head_dim_v=None):
    """Prefill one prompt of L tokens in ceil(L/C) chunks of size C.

    Chunk s (0-indexed) holds tokens [sC, min(sC + C, L)); its step appends
    those tokens' K/V (O1) and then attends them over kv_len = sC + n keys
    (O2), as in the chunked-prefill post, sections "core-idea" and
    "correctness".  ``k_pool``/``v_pool`` are raw pools (any dtype); ``to_f64``
    converts raw stored values to float64 (identity for float arrays).
    Returns (o, lse, final k_pool, final v_pool).
    """
    conv = to_f64 if to_f64 is not None else (lambda a: np.asarray(a, dtype=np.float64))
    return _prefill_steps(q, k_new, v_new, k_pool, v_pool, pages, page_size, chunk,
                          num_qo_heads, num_kv_heads, sm_scale, conv, head_dim_v)


def one_shot_prefill(q, k_new, v_new, k_pool, v_pool, pages, page_size,
                     num_qo_heads, num_kv_heads, sm_scale, to_f64=None, head_dim_v=None):
    """Prefill the whole prompt in one step (C = L)."""
    conv = to_f64 if to_f64 is not None else (lambda a: np.asarray(a, dtype=np.float64))
    return _prefill_steps(q, k_new, v_new, k_pool, v_pool, pages, page_size, q.shape[0],
                          num_qo_heads, num_kv_heads, sm_scale, conv, head_dim_v)


# ----------------------------------------------------------------------------
# O6: page copies (sharded transfer, prefix reuse)
# ----------------------------------------------------------------------------


def copy_pages(src: np.ndarray, dst: np.ndarray, src_pages, dst_pages, src_head0: int,
               dst_head0: int, num_heads: int) -> np.ndarray:
    """Copy head ranges of whole pages; returns the new destination.

    ``src`` and ``dst`` are indexed [page, head, slot, dim] whatever their
    storage order (an NHD buffer is passed as its [page, head, slot, dim]
    view).  For each i, heads src_head0 .. src_head0 + num_heads - 1 of page
    src_pages[i] go to heads dst_head0 .. of page dst_pages[i]; nothing else
    of the destination changes.  This is the page split and reconstruction of
    "Disaggregated prefill and decode" (sharded-transfer section: a decoder
    rebuilds full pages from the halves sent by two prefill devices, and HND
    keeps a head range of a page contiguous), and the copy of a shared,
    partly filled prefix block before two requests append to it (chunked-
    prefill post, prefix-cache section).  Raw elements move unchanged.
    """
    out = np.array(dst, copy=True)
    for sp, dp in zip(np.asarray(src_pages).tolist(), np.asarray(dst_pages).tolist()):
        out[dp, dst_head0:dst_head0 + num_heads] = src[sp, src_head0:src_head0 + num_heads]
    return out


def hnd_to_nhd(pages: np.ndarray) -> np.ndarray:
    """Pages [n, heads, slots, dim] (HND) re-laid as [n, slots, heads, dim] (NHD)."""
    return np.ascontiguousarray(np.swapaxes(pages, 1, 2))


# ----------------------------------------------------------------------------
# O5: accounting
# ----------------------------------------------------------------------------


def accounting(batch: Batch, num_qo_heads: int, num_kv_heads: int, head_dim_qk: int,
               head_dim_v: int, elem_bytes: int, shared_latent: bool = False,
               causal: bool = True) -> dict:
    """Algorithmic work of one attention call over a batch.

    * pairs: visible (query token, key) pairs per query head; a causal query
      at position p sees p + 1 keys (chunked-prefill post, section "flops").
    * flops: each pair and query head costs 2*d_qk for q.k and 2*d_v for the
      weighted sum of values; with d_qk = d_v = d this is the page's 4d per
      pair.  Projections are not attention work and are not counted.
    * kv_bytes: every valid key (and value) row of every KV head read once; a
      shared latent stores and reads d_qk elements only.
    * append_bytes: bytes written by the append (section "io-overhead" counts
      K and V, hence the factor 2 there).
    """
    pairs = 0
    for r in range(batch.batch_size):
        n = batch.qo_len(r)
        L = int(batch.kv_len[r])
        c = L - n
        if causal:
            pairs += sum(c + t + 1 for t in range(n))
        else:
            pairs += n * L
    row_elems = head_dim_qk + (0 if shared_latent else head_dim_v)
    kv_tokens = int(np.sum(batch.kv_len))
    return {
        "pairs": pairs,
        "flops": num_qo_heads * pairs * 2 * (head_dim_qk + head_dim_v),
        "kv_bytes": kv_tokens * num_kv_heads * row_elems * elem_bytes,
        "append_bytes": batch.total_q * num_kv_heads * row_elems * elem_bytes,
    }


def kv_write_bytes_per_chunk(chunk: int, n_layers: int, n_kv_heads: int, head_dim: int,
                             elem_bytes: int = 2) -> int:
    """KV bytes a model writes for one prefill chunk, over all layers.

    Chunked-prefill post, section "io-overhead": C tokens, K and V (2), every
    layer, every KV head, head_dim elements of elem_bytes each.
    """
    return chunk * 2 * n_layers * n_kv_heads * head_dim * elem_bytes


__all__ = [
    "Batch", "bf16_bits_to_f64", "f32_to_bf16_bits_rne", "slot_of", "gather", "append",
    "attend_dense", "attend", "merge", "split_attention", "chunked_prefill", "one_shot_prefill",
    "accounting", "kv_write_bytes_per_chunk", "copy_pages", "hnd_to_nhd",
]
