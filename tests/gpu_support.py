"""Helpers for the GPU parity tests: run a batch through the HIP library and
build the oracle's expected values from the same seeded inputs.

The expected values come only from ``oracle``; the HIP path's outputs are
compared to them and never feed them.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
import ragged_paged_kv_append_amd as rpa

TOL = {"bf16": 2e-2, "f32": 1e-4}


def raw(t: torch.Tensor) -> np.ndarray:
    """Stored elements of a tensor as a numpy array (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of stored elements."""
    if a.dtype == np.uint16:
        return oracle.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def config_of(spec: workloads.Spec):
    return rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                           spec.page_size, spec.dtype, spec.causal, spec.sm_scale)


def batch_of(meta: workloads.Meta) -> oracle.Batch:
    return oracle.Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                        meta.page_size)


def poison_tail_slots(meta: workloads.Meta, tensors: dict):
    """NaN in the slots past kv_len of each request's last page (never read)."""
    b = batch_of(meta)
    P = meta.page_size
    for r in range(meta.batch_size):
        L = int(meta.kv_len[r])
        if L == 0:
            continue
        last_page_end = -(-L // P) * P
        for pos in range(L, last_page_end):
            page, slot = oracle.slot_of(b, r, pos)
            for key in ("k_pool", "v_pool"):
                if tensors.get(key) is not None:
                    tensors[key][page, :, slot, :] = float("nan")


def run_library(spec, meta, tensors, num_cus=0, device="cuda"):
    """Plan, upload, append and attend on the GPU.  Mutates the pools in place;
    returns (o, lse, plan)."""
    cfg = config_of(spec)
    plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages, device=device, num_cus=num_cus)
    plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
    o, lse = plan.attention(tensors["q"], tensors["k_pool"], tensors["v_pool"])
    torch.cuda.synchronize()
    return o, lse, plan


def compact(meta: workloads.Meta, requests, pools: dict, rows: dict):
    """Sub-batch of the given requests with its pages renumbered 0..m-1.

    pools: name -> full pool array (numpy raw); rows: name -> [total_q, ...] arrays.
    Returns (sub-meta, sub-pools, sub-rows).  Pure slicing, no arithmetic of the method.
    """
    requests = list(requests)
    qo_lens = [int(meta.qo_indptr[r + 1] - meta.qo_indptr[r]) for r in requests]
    page_lists = [meta.kv_page_indices[meta.kv_page_indptr[r]:meta.kv_page_indptr[r + 1]]
                  for r in requests]
    all_pages = np.concatenate(page_lists) if page_lists else np.zeros(0, dtype=np.int64)
    indptr = np.concatenate([[0], np.cumsum([len(p) for p in page_lists])]).astype(np.int32)
    sub_meta = workloads.Meta(
        qo_indptr=np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32),
        kv_len=np.array([meta.kv_len[r] for r in requests], dtype=np.int32),
        kv_page_indptr=indptr,
        kv_page_indices=np.arange(len(all_pages), dtype=np.int32),
        num_pages=len(all_pages), page_size=meta.page_size)
    sub_pools = {k: (None if v is None else v[all_pages]) for k, v in pools.items()}
    sel = np.concatenate([np.arange(meta.qo_indptr[r], meta.qo_indptr[r + 1]) for r in requests]) \
        if requests else np.zeros(0, dtype=np.int64)
    sub_rows = {k: (None if v is None else v[sel]) for k, v in rows.items()}
    return sub_meta, sub_pools, sub_rows, sel


def expected(spec, meta, q_raw, kn_raw, vn_raw, kp_raw, vp_raw):
    """The oracle's pools after append and its attention output (float64)."""
    b = batch_of(meta)
    kp2, vp2 = oracle.append(kp_raw, vp_raw, kn_raw, vn_raw, b)
    o, lse = oracle.attend(f64(q_raw), f64(kp2), None if vp2 is None else f64(vp2), b,
                           spec.num_qo_heads, spec.num_kv_heads, spec.sm_scale,
                           head_dim_v=spec.head_dim_v, causal=spec.causal)
    return kp2, vp2, o, lse


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want)))


def full_parity(spec, meta, tensors, label, tree_masks=None, num_cus=0, group_bytes=1 << 29,
                log=print, split=False):
    """Runs the batch through the library once (the launch configuration the
    benchmark times), then checks the pools bit-exactly over the whole pool
    and O / LSE of every request against the oracle.  The oracle runs over
    groups of requests of at most `group_bytes` of float64 keys, so host
    memory stays bounded at any batch size.  With `split`, the step runs in
    split form (rpa_split_attention before the append, which then must not
    matter).  Returns (max|dO|, max|dLSE|)."""
    q_raw, kn_raw = raw(tensors["q"]), raw(tensors["k_new"])
    vn_raw = None if tensors["v_new"] is None else raw(tensors["v_new"])
    kp_raw = raw(tensors["k_pool"])
    vp_raw = None if tensors["v_pool"] is None else raw(tensors["v_pool"])
    b = batch_of(meta)
    kp2, vp2 = oracle.append(kp_raw, vp_raw, kn_raw, vn_raw, b)
    cfg = config_of(spec)
    if split:
        plan = rpa.SplitChunkAttention(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                                       meta.kv_page_indices, meta.num_pages, num_cus=num_cus)
        o, lse = plan.run(tensors["q"], tensors["k_new"], tensors["v_new"], tensors["k_pool"],
                          tensors["v_pool"])
        plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
    else:
        plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                        meta.kv_page_indices, meta.num_pages, num_cus=num_cus,
                        tree_masks=tree_masks)
        plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
        o, lse = plan.attention(tensors["q"], tensors["k_pool"], tensors["v_pool"])
    torch.cuda.synchronize()
    log(f"[{label}] summary={plan.debug('summary').tolist()}")
    assert np.array_equal(raw(tensors["k_pool"]), kp2), "K pool differs from the oracle"
    if vp2 is not None:
        assert np.array_equal(raw(tensors["v_pool"]), vp2), "V pool differs from the oracle"
    o_g = o.float().cpu().numpy().astype(np.float64)
    lse_g = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g)), "non-finite output"
    per_token = spec.num_kv_heads * (spec.head_dim_qk + (0 if vp2 is None else spec.head_dim_v)) * 8
    eo = el = 0.0
    r0 = 0
    B = meta.batch_size
    while r0 < B:
        r1, acc = r0, 0
        while r1 < B and (r1 == r0 or acc + int(meta.kv_len[r1]) * per_token <= group_bytes):
            acc += int(meta.kv_len[r1]) * per_token
            r1 += 1
        reqs = list(range(r0, r1))
        sub_meta, sub_pools, sub_rows, sel = compact(meta, reqs, {"k": kp2, "v": vp2},
                                                     {"q": q_raw})
        o_ref, lse_ref = oracle.attend(
            f64(sub_rows["q"]), f64(sub_pools["k"]),
            None if sub_pools["v"] is None else f64(sub_pools["v"]), batch_of(sub_meta),
            spec.num_qo_heads, spec.num_kv_heads, spec.sm_scale, head_dim_v=spec.head_dim_v,
            causal=spec.causal,
            tree=None if tree_masks is None else [tree_masks[r] for r in reqs])
        if len(sel):
            eo = max(eo, float(np.max(np.abs(o_g[sel] - o_ref))))
            el = max(el, float(np.max(np.abs(lse_g[sel] - lse_ref))))
        r0 = r1
    log(f"[{label}] all {B} requests: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= TOL[spec.dtype] and el <= TOL[spec.dtype]
    return eo, el
