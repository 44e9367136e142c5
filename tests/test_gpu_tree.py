"""GPU parity of tree-masked verification ("Accelerating Sonar through
speculation", EAGLE section: draft trees are verified under a custom
attention mask).  The mask applies among a request's new tokens only; cached
keys stay visible.  Decode-class, prefill-class, generic and latent-form
requests against the fp64 oracle on the same seeded inputs.
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


def random_tree(rng, n):
    parent = [-1] + [int(rng.integers(0, u)) for u in range(1, n)]
    m = np.zeros((n, n), dtype=bool)
    for t in range(n):
        u = t
        while u >= 0:
            m[t, u] = True
            u = parent[u]
    return m


CASES = [
    # dtype, hq, hkv, dqk, dv, P, qo lens, kv lens, which requests carry a tree, num_cus
    ("bf16", 32, 8, 128, 128, 16, [4, 1, 4, 4], [5000, 300, 4, 1200], [0, 2, 3], 0),   # decode class
    ("bf16", 32, 8, 128, 128, 16, [4, 4, 4], [4, 6, 20], [0, 1, 2], 0),               # short contexts
    ("bf16", 8, 1, 128, 128, 16, [16, 64, 3, 40], [900, 64, 2000, 3000], [0, 1, 3], 0),  # prefill class
    ("bf16", 8, 1, 128, 128, 16, [64], [8192], [0], 100000),                       # many splits
    ("f32", 4, 2, 64, 64, 16, [7, 2, 5], [37, 2, 90], [0, 2], 0),                  # generic
    ("bf16", 128, 1, 576, 512, 64, [4, 2], [3000, 700], [0], 0),                   # latent -> generic
]


@pytest.mark.parametrize("case", CASES, ids=[f"t{i}" for i in range(len(CASES))])
def test_tree_masked_verify_matches_oracle(case):
    dtype, hq, hkv, dqk, dv, P, qo, kv, masked, num_cus = case
    seed = 700 + sum(kv)
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(192 if dqk == 576 else dqk)
    spec = workloads.Spec(f"tree{seed}", hq, hkv, dqk, dv, P, dtype, scale, seed,
                          shared_latent=(dqk == 576))
    meta = workloads.make_meta(qo, kv, P, seed)
    t = workloads.make_tensors(spec, meta, seed, device="cuda")
    poison_tail_slots(meta, t)
    masks = [random_tree(rng, n) if r in masked else None for r, n in enumerate(qo)]
    log(f"tree {case}")
    host = {k: (None if v is None else raw(v)) for k, v in t.items()}
    plan = rpa.Plan(config_of(spec), meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                    meta.kv_page_indices, meta.num_pages, num_cus=num_cus, tree_masks=masks)
    plan.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
    o, lse = plan.attention(t["q"], t["k_pool"], t["v_pool"])
    torch.cuda.synchronize()
    b = batch_of(meta)
    kp2, vp2 = oracle.append(host["k_pool"], host["v_pool"], host["k_new"], host["v_new"], b)
    assert raw(t["k_pool"]).tobytes() == kp2.tobytes()
    o_ref, lse_ref = oracle.attend(f64(host["q"]), f64(kp2), None if vp2 is None else f64(vp2), b,
                                   hq, hkv, scale, head_dim_v=dv, tree=masks)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    log(f"  max|dO|={eo:.3g} max|dLSE|={el:.3g} summary={plan.debug('summary').tolist()}")
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    # where the mask changes the answer, the GPU follows the mask
    o_c, _ = oracle.attend(f64(host["q"]), f64(kp2), None if vp2 is None else f64(vp2), b, hq,
                           hkv, scale, head_dim_v=dv)
    o_g = o.float().cpu().numpy().astype(np.float64)
    moved = np.abs(o_c - o_ref) > 0.1
    assert np.all(np.abs(o_g - o_c)[moved] > 0.05)


def test_chain_mask_reproduces_causal_verify():
    spec = workloads.Spec("chain", 32, 8, 128, 128, 16, "bf16", 1 / math.sqrt(128), 9)
    qo, kv = [4, 4, 1, 4], [4096, 900, 2000, 4]
    meta = workloads.make_meta(qo, kv, 16, 9)
    chains = [np.tril(np.ones((n, n), dtype=bool)) for n in qo]
    outs = []
    for masks in (chains, None):
        t = workloads.make_tensors(spec, meta, 9, device="cuda")
        plan = rpa.Plan(config_of(spec), meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                        meta.kv_page_indices, meta.num_pages, tree_masks=masks)
        plan.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
        outs.append(plan.attention(t["q"], t["k_pool"], t["v_pool"]))
    torch.cuda.synchronize()
    d = (outs[0][0].float() - outs[1][0].float()).abs().max().item()
    dl = (outs[0][1] - outs[1][1]).abs().max().item()
    log(f"chain vs causal: max|dO|={d:.3g} max|dLSE|={dl:.3g}")
    assert d <= 2e-2 and dl <= 2e-2


def test_tree_verify_full_size_workload():
    """The verify workload at full size (256 requests, 32/8 heads) with every
    4-token verification as the draft tree the benchmark times (parents
    -1, 0, 0, 1: a root, its two children, one grandchild), every request
    compared with the oracle's tree-masked attention."""
    spec, meta, tensors = workloads.workload("decode_verify_gqa", device="cuda")
    parents = [-1, 0, 0, 1]
    tree = np.zeros((4, 4), dtype=bool)
    for t_ in range(4):
        u = t_
        while u >= 0:
            tree[t_, u] = True
            u = parents[u]
    qo = np.diff(meta.qo_indptr)
    masks = [tree if int(qo[r]) == 4 else None for r in range(meta.batch_size)]
    full_parity(spec, meta, tensors, "decode_verify_gqa tree", tree_masks=masks, log=log)
