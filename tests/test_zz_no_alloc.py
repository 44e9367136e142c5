"""The allocation-free attention entry point (rpa_batch_attention_noalloc)
against rpa_batch_attention with an uploaded workspace: two calls in a row
through the C ABI, the second on a smaller batch (the static scratch keeps the
first call's contents), each bit-identical to the workspace path and within
tolerance of the fp64 oracle.
"""

import math
import sys

import numpy as np
import pytest
import torch

import workloads
import ragged_paged_kv_append_amd as rpa
from tests.gpu_support import TOL, config_of, expected, max_err, raw

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


# Two batches per class mix, the second smaller; long keys force split pieces
# (partials in the scratch) and the chunk runs on the prefill kernel.
CALLS = [
    ("bf16 decode + chunk", (32, 8, 128, 128, 16, "bf16"),
     [([1, 4, 1, 512, 4], [30000, 9000, 700, 3000, 6000]), ([1, 64, 4], [5000, 2100, 40])]),
    ("latent", (128, 1, 576, 512, 64, "bf16"),
     [([2, 2, 2, 2], [20000, 9000, 4100, 30000]), ([2, 2], [6000, 700])]),
    ("fp32 generic", (4, 2, 64, 64, 16, "f32"),
     [([3, 1, 17], [2000, 900, 3000]), ([1, 5], [300, 40])]),
]


@pytest.mark.parametrize("case", CALLS, ids=[c[0] for c in CALLS])
def test_noalloc_matches_workspace_path_twice(case):
    label, (hq, hkv, dqk, dv, P, dtype), batches = case
    for call, (qo, kv) in enumerate(batches):
        seed = 900 + 10 * call + hq
        scale = 1.0 / math.sqrt(192 if dqk == 576 else dqk)
        spec = workloads.Spec(f"noalloc{seed}", hq, hkv, dqk, dv, P, dtype, scale, seed,
                              shared_latent=(dqk == 576))
        meta = workloads.make_meta(qo, kv, P, seed)
        t = workloads.make_tensors(spec, meta, seed, device="cuda")
        host = {k: (None if v is None else raw(v)) for k, v in t.items()}
        cfg = config_of(spec)
        plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                        meta.kv_page_indices, meta.num_pages, num_cus=64)
        log(f"{label} call {call}: qo={qo} kv={kv} workspace={plan.ws_bytes} "
            f"summary={plan.debug('summary').tolist()}")
        plan.append(t["k_new"], t["v_new"], t["k_pool"], t["v_pool"])
        o_ws, lse_ws = plan.attention(t["q"], t["k_pool"], t["v_pool"])
        o_na = torch.full_like(o_ws, float("nan"))
        lse_na = torch.full_like(lse_ws, float("nan"))
        ks = rpa.strides_of(t["k_pool"])
        vs = None if t["v_pool"] is None else rpa.strides_of(t["v_pool"])
        rpa.check_attention_args(cfg, plan.total_q, plan.num_pages, t["q"], t["k_pool"],
                                 t["v_pool"], o_na, lse_na)
        rpa.rpa_batch_attention_noalloc(plan.handle, t["q"], t["k_pool"], t["v_pool"], ks, vs,
                                        o_na, lse_na)
        torch.cuda.synchronize()
        assert torch.equal(raw_t(o_na), raw_t(o_ws)), "O differs from the workspace path"
        assert torch.equal(lse_na.view(torch.int32), lse_ws.view(torch.int32)), \
            "LSE differs from the workspace path"
        _, _, o_ref, lse_ref = expected(spec, meta, host["q"], host["k_new"], host["v_new"],
                                        host["k_pool"], host["v_pool"])
        eo, el = max_err(o_na, o_ref), max_err(lse_na, lse_ref)
        log(f"  max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        assert eo <= TOL[dtype] and el <= TOL[dtype]


def raw_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
