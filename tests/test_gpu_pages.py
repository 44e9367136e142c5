"""GPU parity of page copies (bit-exact against the oracle's copy_pages):
shard export and reconstruction of full pages from half-head shards
("Disaggregated prefill and decode", sharded-transfer section), HND <-> NHD
transfer buffers, and the copy of a shared partly filled prefix page before
two requests append to it (chunked-prefill post, prefix-cache section).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import ragged_paged_kv_append_amd as rpa
from tests.gpu_support import TOL, batch_of, config_of, f64, max_err, raw

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


def ids(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


@pytest.mark.parametrize("dtype,H,P,d", [(torch.bfloat16, 8, 16, 128), (torch.float32, 4, 16, 64),
                                         (torch.bfloat16, 1, 64, 576), (torch.bfloat16, 32, 16, 128)])
def test_shard_export_and_rebuild(dtype, H, P, d):
    g = torch.Generator(device="cuda").manual_seed(H * P + d)
    n_pool = 300
    pool = torch.randn((n_pool, H, P, d), generator=g, device="cuda").to(dtype)
    rng = np.random.default_rng(H + d)
    pages = rng.permutation(n_pool)[:97]
    parts = [(0, H)] if H == 1 else [(0, H // 2), (H // 2, H - H // 2)]
    # export: each shard into a packed HND buffer [n, heads of shard, P, d]
    shards = []
    for h0, nh in parts:
        buf = torch.full((len(pages), nh, P, d), float("nan"), dtype=dtype, device="cuda")
        rpa.copy_pages(pool, buf, src_pages=ids(pages), src_head0=h0, num_heads=nh)
        shards.append(buf)
    torch.cuda.synchronize()
    host_pool = raw(pool)
    for (h0, nh), buf in zip(parts, shards):
        want = oracle.copy_pages(host_pool, np.zeros_like(raw(buf)), pages, np.arange(len(pages)),
                                 h0, 0, nh)
        assert raw(buf).tobytes() == want.tobytes()
    # rebuild full pages on the other side at other page ids, from the shards
    dst = torch.full((400, H, P, d), float("nan"), dtype=dtype, device="cuda")
    dpages = rng.permutation(400)[:97]
    for (h0, nh), buf in zip(parts, shards):
        rpa.copy_pages(buf, dst, dst_pages=ids(dpages), dst_head0=h0, num_heads=nh)
    torch.cuda.synchronize()
    want = raw(torch.full((400, H, P, d), float("nan"), dtype=dtype))
    for (h0, nh), buf in zip(parts, shards):
        want = oracle.copy_pages(raw(buf), want, np.arange(len(pages)), dpages, 0, h0, nh)
    assert raw(dst).tobytes() == want.tobytes()
    assert raw(dst)[dpages].tobytes() == host_pool[pages].tobytes()


def test_hnd_to_nhd_transfer_buffer_and_back():
    g = torch.Generator(device="cuda").manual_seed(5)
    H, P, d = 8, 16, 128
    pool = torch.randn((200, H, P, d), generator=g, device="cuda").to(torch.bfloat16)
    pages = np.random.default_rng(5).permutation(200)[:50]
    nhd = torch.empty((50, P, H, d), dtype=torch.bfloat16, device="cuda")
    rpa.copy_pages(pool, nhd.permute(0, 2, 1, 3), src_pages=ids(pages))
    back = torch.full_like(pool, float("nan"))
    rpa.copy_pages(nhd.permute(0, 2, 1, 3), back, dst_pages=ids(pages))
    torch.cuda.synchronize()
    assert raw(nhd).tobytes() == oracle.hnd_to_nhd(raw(pool)[pages]).tobytes()
    assert raw(back)[pages].tobytes() == raw(pool)[pages].tobytes()
    others = np.setdiff1d(np.arange(200), pages)
    assert torch.isnan(back[torch.as_tensor(others, device="cuda")].float()).all()


def test_prefix_tail_copy_then_append_and_attend():
    # two requests share a prefix of 40 tokens (pages of 16): two full pages
    # are shared read-only; the partly filled tail page is copied for the
    # second request before both append their own tokens
    H, hq, d, P = 2, 8, 128, 16
    spec = workloads.Spec("prefix", hq, H, d, d, P, "bf16", 1 / math.sqrt(d), 31)
    g = torch.Generator(device="cuda").manual_seed(31)
    n_pool = 12
    kp = torch.full((n_pool, H, P, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    shared = [7, 2, 9]
    pre_k = torch.randn((40, H, d), generator=g, device="cuda").to(torch.bfloat16)
    pre_v = torch.randn((40, H, d), generator=g, device="cuda").to(torch.bfloat16)
    for j in range(40):
        kp[shared[j // P], :, j % P] = pre_k[j]
        vp[shared[j // P], :, j % P] = pre_v[j]
    tail_copy, extra = 4, 11
    rpa.copy_pages(kp, kp, src_pages=ids([shared[2]]), dst_pages=ids([tail_copy]))
    rpa.copy_pages(vp, vp, src_pages=ids([shared[2]]), dst_pages=ids([tail_copy]))
    qo, kv = [5, 12], [45, 52]
    indptr = [0, 3, 7]
    indices = shared + [shared[0], shared[1], tail_copy, extra]
    meta = workloads.Meta(np.array([0, 5, 17], np.int32), np.array(kv, np.int32),
                          np.array(indptr, np.int32), np.array(indices, np.int32), n_pool, P)
    q = torch.randn((17, hq, d), generator=g, device="cuda").to(torch.bfloat16)
    k_new = torch.randn((17, H, d), generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((17, H, d), generator=g, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    host_k, host_v = raw(kp), raw(vp)
    plan = rpa.Plan(config_of(spec), meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                    meta.kv_page_indices, n_pool)
    plan.append(k_new, v_new, kp, vp)
    o, lse = plan.attention(q, kp, vp)
    torch.cuda.synchronize()
    b = batch_of(meta)
    kp2, vp2 = oracle.append(host_k, host_v, raw(k_new), raw(v_new), b)
    assert raw(kp).tobytes() == kp2.tobytes() and raw(vp).tobytes() == vp2.tobytes()
    o_ref, lse_ref = oracle.attend(f64(raw(q)), f64(kp2), f64(vp2), b, hq, H, spec.sm_scale)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    log(f"prefix tail copy: max|dO|={eo:.3g} max|dLSE|={el:.3g}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]


def test_page_copy_argument_checks_launch_nothing():
    pool = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    st = rpa.strides_of(pool)
    with pytest.raises(rpa.RpaError):   # dim not a whole number of 16-byte chunks
        rpa.rpa_page_copy(pool, st, 4, 2, None, pool, st, 4, 2, None, 4, 0, 0, 2, 16, 100,
                          rpa.RPA_DTYPE_BF16)
    with pytest.raises(rpa.RpaError):   # misaligned destination
        rpa.rpa_page_copy(pool, st, 4, 2, None, pool.data_ptr() + 2, st, 4, 2, None, 4, 0, 0, 2,
                          16, 128, rpa.RPA_DTYPE_BF16)
    with pytest.raises(rpa.RpaError) as ei:   # identity list longer than the destination pool
        rpa.rpa_page_copy(pool, st, 4, 2, None, pool, st, 3, 2, None, 4, 0, 0, 2, 16, 128,
                          rpa.RPA_DTYPE_BF16)
    assert ei.value.status == rpa.RPA_ERR_PAGE_OOB
    with pytest.raises(rpa.RpaError):   # head range past the source's heads
        rpa.rpa_page_copy(pool, st, 4, 2, None, pool, st, 4, 2, None, 4, 1, 0, 2, 16, 128,
                          rpa.RPA_DTYPE_BF16)
    rpa.rpa_page_copy(None, st, 4, 2, None, None, st, 4, 2, None, 0, 0, 0, 2, 16, 128,
                      rpa.RPA_DTYPE_BF16)


def test_page_copy_skips_out_of_range_device_ids():
    """Device page ids outside a pool are skipped in the kernel: those pairs
    write nothing, the others are copied as usual."""
    g = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randn((20, 2, 16, 128), generator=g, device="cuda").to(torch.bfloat16)
    dst = torch.zeros((12, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    sp = [3, 25, 7, -1, 19, 4]
    dp = [0, 1, 12, 3, 11, -5]
    rpa.copy_pages(src, dst, src_pages=ids(sp), dst_pages=ids(dp))
    torch.cuda.synchronize()
    want = np.zeros_like(raw(dst))
    host = raw(src)
    for s_, d_ in zip(sp, dp):
        if 0 <= s_ < 20 and 0 <= d_ < 12:
            want[d_] = host[s_]
    assert raw(dst).tobytes() == want.tobytes()
