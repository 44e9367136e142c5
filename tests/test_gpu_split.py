"""GPU parity of the split execution ("Chunked prefill", section
"correctness"): the new tokens attend to the cached keys (a cross-attention
plan: causal masking off, kv_len = cached length, possibly 0) and causally to
their own keys read straight from the projection buffers, and the two states
are merged.  Compared with the fp64 oracle's split form, and with the oracle's
attention after the append, on the same seeded inputs.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import ragged_paged_kv_append_amd as rpa
from tests.gpu_support import (TOL, batch_of, config_of, f64, full_parity, max_err,
                               poison_tail_slots, raw)

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rpa.lib()
    yield


def spec_of(dtype, hq, hkv, d, P, seed):
    return workloads.Spec(f"split{seed}", hq, hkv, d, d, P, dtype, 1.0 / math.sqrt(d), seed)


def new_slots_nan(meta, tensors):
    """NaN in the slots the append would write: the split form must not read them."""
    b = batch_of(meta)
    for r in range(meta.batch_size):
        n = int(meta.qo_indptr[r + 1] - meta.qo_indptr[r])
        L = int(meta.kv_len[r])
        for pos in range(L - n, L):
            page, slot = oracle.slot_of(b, r, pos)
            for key in ("k_pool", "v_pool"):
                tensors[key][page, :, slot, :] = float("nan")


CROSS = [
    # dtype, hq, hkv, d, P, qo lens, cached lens
    ("bf16", 8, 2, 128, 16, [1, 4, 300, 7], [700, 0, 513, 33]),    # decode / prefill classes
    ("bf16", 32, 32, 128, 16, [1, 2, 1], [0, 90, 4000]),
    ("f32", 4, 2, 64, 16, [3, 16, 1], [37, 0, 5]),                 # generic kernel
    ("bf16", 4, 4, 64, 4, [5, 2], [19, 0]),
]


@pytest.mark.parametrize("case", CROSS, ids=[f"x{i}" for i in range(len(CROSS))])
def test_cross_attention_over_cached_keys(case):
    dtype, hq, hkv, d, P, qo, cached = case
    seed = 500 + sum(cached)
    spec = spec_of(dtype, hq, hkv, d, P, seed)
    meta = workloads.make_meta(qo, cached, P, seed)
    t = workloads.make_tensors(spec, meta, seed, device="cuda")
    poison_tail_slots(meta, t)
    cfg = rpa.make_config(hq, hkv, d, d, P, dtype, False, spec.sm_scale)
    log(f"cross {case}")
    plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages)
    o, lse = plan.attention(t["q"], t["k_pool"], t["v_pool"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attend(f64(raw(t["q"])), f64(raw(t["k_pool"])),
                                   f64(raw(t["v_pool"])), batch_of(meta), hq, hkv, spec.sm_scale,
                                   causal=False)
    lse_g = lse.cpu().numpy().astype(np.float64)
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(np.isinf(lse_g) & (lse_g < 0), empty), "empty rows must be -inf"
    assert torch.all(o.float()[torch.from_numpy(empty).cuda()] == 0)
    eo = max_err(o, o_ref)
    el = float(np.max(np.abs(lse_g[~empty] - lse_ref[~empty]))) if np.any(~empty) else 0.0
    log(f"  max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    # a plan with kv_len < qo_len has no append slots
    with pytest.raises(rpa.RpaError) as ei:
        plan.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
    assert ei.value.status == rpa.RPA_ERR_INVALID_ARG


SPLIT = [
    ("bf16", 32, 32, 128, 16, [1, 1, 512, 40], [3000, 17, 1536, 40]),   # decodes, chunk, first chunk
    ("bf16", 8, 1, 128, 16, [512, 4, 3], [2048, 700, 3]),
    ("f32", 4, 2, 64, 16, [1, 16, 5], [37, 36, 5]),
    ("bf16", 16, 2, 128, 64, [129, 0, 33], [1000, 64, 97]),
]


@pytest.mark.parametrize("case", SPLIT, ids=[f"s{i}" for i in range(len(SPLIT))])
def test_split_execution_matches_oracle(case):
    dtype, hq, hkv, d, P, qo, kv = case
    seed = 600 + sum(kv)
    spec = spec_of(dtype, hq, hkv, d, P, seed)
    meta = workloads.make_meta(qo, kv, P, seed)
    t = workloads.make_tensors(spec, meta, seed, device="cuda")
    poison_tail_slots(meta, t)
    new_slots_nan(meta, t)
    log(f"split {case}")
    host = {k: raw(v) for k, v in t.items()}
    split = rpa.SplitChunkAttention(config_of(spec), meta.qo_indptr, meta.kv_len,
                                    meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)
    o, lse = split.run(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
    torch.cuda.synchronize()
    b = batch_of(meta)
    o_ref, lse_ref = oracle.split_attention(f64(host["q"]), f64(host["k_pool"]),
                                            f64(host["v_pool"]), f64(host["k_new"]),
                                            f64(host["v_new"]), b, hq, hkv, spec.sm_scale)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    log(f"  split vs oracle split form: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    # the same step through the append and the paged attention
    kp2, vp2 = oracle.append(host["k_pool"], host["v_pool"], host["k_new"], host["v_new"], b)
    o_app, lse_app = oracle.attend(f64(host["q"]), f64(kp2), f64(vp2), b, hq, hkv, spec.sm_scale)
    eo2, el2 = max_err(o, o_app), max_err(lse, lse_app)
    log(f"  split vs attention after append: max|dO|={eo2:.3g} max|dLSE|={el2:.3g}")
    assert eo2 <= TOL[dtype] and el2 <= TOL[dtype]


def test_split_execution_chunked_prompt_equals_one_shot():
    # the 8192-token GQA prompt in 16 chunks of 512, each chunk attended in
    # split form before its append; outputs against the one-shot oracle
    spec = workloads.SPECS["chunked_gqa"]
    L, C = spec.extra["prompt_len"], spec.extra["chunk"]
    q, k, v = workloads.make_prompt(spec, spec.seed, device="cuda")
    meta = workloads.make_meta([L], [L], 16, spec.seed)
    pages = meta.kv_page_indices
    shape = (meta.num_pages, 1, 16, 128)
    kp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    o = torch.empty((L, 8, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, 8), dtype=torch.float32, device="cuda")
    cfg = config_of(spec)
    for s in range(L // C):
        a = s * C
        split = rpa.SplitChunkAttention(cfg, [0, C], [a + C], [0, len(pages)], pages,
                                        meta.num_pages)
        split.run(q[a:a + C], k[a:a + C], v[a:a + C], kp, vp, o=o[a:a + C], lse=lse[a:a + C])
        plan = rpa.Plan(cfg, [0, C], [a + C], [0, len(pages)], pages, meta.num_pages)
        plan.append(k[a:a + C], v[a:a + C], kp, vp)
    torch.cuda.synchronize()
    kp0 = np.full(shape, 0x7FC0, dtype=np.uint16)
    b = oracle.Batch([0, L], [L], [0, len(pages)], pages, 16)
    kp2, vp2 = oracle.append(kp0, kp0.copy(), raw(k), raw(v), b)
    assert raw(kp).tobytes() == kp2.tobytes() and raw(vp).tobytes() == vp2.tobytes()
    o_ref, lse_ref = oracle.attend(f64(raw(q)), f64(kp2), f64(vp2), b, 8, 1, spec.sm_scale)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    log(f"[chunked_gqa split] max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= 2e-2 and el <= 2e-2


@pytest.mark.parametrize("name", ["mixed_7b", "decode_verify_gqa"])
def test_split_execution_full_workload(name):
    """Every request of a full benchmark batch in split form (decodes, the
    prefill chunk, verifications), element by element against the oracle's
    attention after the append; the split attention runs before the append."""
    spec, meta, tensors = workloads.workload(name, device="cuda")
    new_slots_nan(meta, tensors)
    log(f"split full {name}")
    full_parity(spec, meta, tensors, f"split {name}", log=log, split=True)


def test_split_execution_plan_reuse_and_append_order():
    """One split plan, called twice with different inputs, the append run
    before the first call and after the second: both match the oracle."""
    spec = spec_of("bf16", 16, 4, 128, 16, 4242)
    qo, kv = [300, 1, 4, 64], [2000, 513, 37, 64]
    meta = workloads.make_meta(qo, kv, 16, 4242)
    split = rpa.SplitChunkAttention(config_of(spec), meta.qo_indptr, meta.kv_len,
                                    meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)
    b = batch_of(meta)
    for it, seed in enumerate((4242, 4243)):
        t = workloads.make_tensors(spec, meta, seed, device="cuda")
        host = {k: raw(v) for k, v in t.items()}
        if it == 0:
            split.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
        o, lse = split.run(t["q"], t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
        if it == 1:
            split.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
        torch.cuda.synchronize()
        kp2, vp2 = oracle.append(host["k_pool"], host["v_pool"], host["k_new"], host["v_new"], b)
        assert np.array_equal(raw(t["k_pool"]), kp2) and np.array_equal(raw(t["v_pool"]), vp2)
        o_ref, lse_ref = oracle.attend(f64(host["q"]), f64(kp2), f64(vp2), b, 16, 4,
                                       spec.sm_scale)
        eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
        log(f"  call {it}: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        assert eo <= TOL["bf16"] and el <= TOL["bf16"]
