"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

KV pools must match the oracle's append bit for bit (the whole pool, NaN
sentinels in unreferenced pages included); attention outputs and LSE must be
within max-abs 2e-2 (bf16) or 1e-4 (fp32) of the oracle.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import ragged_paged_kv_append_amd as rpa
from tests.gpu_support import (TOL, config_of, expected, f64, full_parity, max_err,
                               poison_tail_slots, raw, run_library)

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rpa.lib()  # fail loudly if the library is missing
    yield


def check_full(spec, meta, tensors, num_cus=0, label=""):
    """Whole-batch parity: pools bit-exact, O and LSE within tolerance."""
    poison_tail_slots(meta, tensors)
    host = {k: (None if v is None else raw(v)) for k, v in tensors.items()}
    kp2, vp2, o_ref, lse_ref = expected(spec, meta, host["q"], host["k_new"], host["v_new"],
                                        host["k_pool"], host["v_pool"])
    o, lse, plan = run_library(spec, meta, tensors, num_cus=num_cus)
    assert raw(tensors["k_pool"]).tobytes() == kp2.tobytes(), "K pool differs from the oracle"
    if vp2 is not None:
        assert raw(tensors["v_pool"]).tobytes() == vp2.tobytes(), "V pool differs from the oracle"
    eo = max_err(o, o_ref)
    el = max_err(lse, lse_ref)
    log(f"[{label}] max|dO|={eo:.3g} max|dLSE|={el:.3g} summary={plan.debug('summary').tolist()}")
    tol = TOL[spec.dtype]
    assert eo <= tol and el <= tol, (eo, el)
    return o, lse, plan


def small_spec(dtype, hq, hkv, dqk, dv, P, causal=True, seed=0):
    scale = 1.0 / math.sqrt(192 if dqk == 576 else dqk)
    return workloads.Spec(f"small{seed}", hq, hkv, dqk, dv, P, dtype, scale, seed,
                          shared_latent=(dqk == 576), causal=causal)


# ----------------------------------------------------------------------------
# Small cases: several tiles and a ragged tail, every supported layout
# ----------------------------------------------------------------------------


def test_tiny_fp32_workload():
    spec, meta, tensors = workloads.workload("tiny_fp32", device="cuda")
    check_full(spec, meta, tensors, label="tiny_fp32")


SMALL = []
for seed in range(24):
    rng = np.random.default_rng(100 + seed)
    dtype = ["bf16", "f32"][seed % 2]
    dims = [(128, 128), (64, 64), (128, 128), (576, 512)][(seed // 2) % 4]
    if dims == (576, 512):
        dtype = "bf16"
    P = int([16, 64, 4, 1, 16, 32][seed % 6])
    hkv = 1 if dims[0] == 576 else int(rng.choice([1, 2, 4]))
    G = int(rng.choice([16, 32])) if dims[0] == 576 else int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 6))
    qo = rng.integers(0, 18, size=B)
    if seed % 5 == 0:
        qo[0] = 0
    kv = qo + rng.integers(0, 400, size=B)
    causal = seed % 4 != 3
    num_cus = [0, 100000, 4][seed % 3]
    SMALL.append((seed, dtype, dims, P, hkv, G, qo.tolist(), kv.tolist(), causal, num_cus))


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_small_random_batches(case):
    seed, dtype, dims, P, hkv, G, qo, kv, causal, num_cus = case
    spec = small_spec(dtype, hkv * G, hkv, dims[0], dims[1], P, causal, seed)
    meta = workloads.make_meta(qo, kv, P, seed, extra_pages_per_req=seed % 2)
    tensors = workloads.make_tensors(spec, meta, seed, device="cuda")
    log(f"case {case}")
    check_full(spec, meta, tensors, num_cus=num_cus, label=f"small{seed}")


def test_prefill_tiles_and_splits_bf16():
    # several 128-row tiles, a ragged tail, GQA folding and forced kv splits
    spec = small_spec("bf16", 8, 2, 128, 128, 16, True, 7)
    meta = workloads.make_meta([300, 1, 4, 129], [900, 700, 50, 129], 16, 7)
    tensors = workloads.make_tensors(spec, meta, 7, device="cuda")
    check_full(spec, meta, tensors, num_cus=100000, label="prefill-splits")
    tensors = workloads.make_tensors(spec, meta, 8, device="cuda")
    check_full(spec, meta, tensors, num_cus=0, label="prefill-default")


@pytest.mark.parametrize("scale", [0.01, 0.1, 0.3])
def test_prefill_rows_without_keys_in_a_piece(scale):
    """An MHA chunk whose key pieces start past the first rows of a row tile
    (those rows see no key of the piece: the piece's items must still run once,
    and the merge skips those rows' empty partial states), at softmax scales
    where a masked score's scaled value lies above -5e29."""
    spec = workloads.Spec("nokey", 16, 16, 128, 128, 16, "bf16", scale, 41)
    meta = workloads.make_meta([512, 300], [1636, 1000], 16, 41)
    tensors = workloads.make_tensors(spec, meta, 41, device="cuda")
    check_full(spec, meta, tensors, num_cus=0, label=f"nokey{scale}")


def test_interleaved_kv_pages():
    # K and V of a page interleaved in one allocation: [pages][2][H][P][d]
    spec = small_spec("bf16", 8, 2, 128, 128, 16, True, 11)
    meta = workloads.make_meta([1, 5, 33], [70, 40, 90], 16, 11)
    t = workloads.make_tensors(spec, meta, 11, device="cuda")
    both = torch.empty((meta.num_pages, 2, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    both[:, 0] = t["k_pool"]
    both[:, 1] = t["v_pool"]
    tensors = dict(t, k_pool=both[:, 0], v_pool=both[:, 1])
    o, lse, _ = check_full(spec, meta, tensors, label="interleaved")


def test_step_without_new_tokens_changes_nothing():
    """Requests with cached keys but no new token: the append writes no slot,
    attention has no query row, and the pools keep every byte (fused and split
    execution alike)."""
    spec = small_spec("bf16", 8, 2, 128, 128, 16, True, 13)
    meta = workloads.make_meta([0, 0, 0], [70, 0, 33], 16, 13)
    tensors = workloads.make_tensors(spec, meta, 13, device="cuda")
    kp0, vp0 = raw(tensors["k_pool"]).tobytes(), raw(tensors["v_pool"]).tobytes()
    cfg = config_of(spec)
    plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages)
    plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
    o, lse = plan.attention(tensors["q"], tensors["k_pool"], tensors["v_pool"])
    split = rpa.SplitChunkAttention(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                                    meta.kv_page_indices, meta.num_pages)
    o2, lse2 = split.run(tensors["q"], tensors["k_new"], tensors["v_new"], tensors["k_pool"],
                         tensors["v_pool"])
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 128) and lse.shape == (0, 8)
    assert o2.shape == (0, 8, 128) and lse2.shape == (0, 8)
    assert raw(tensors["k_pool"]).tobytes() == kp0 and raw(tensors["v_pool"]).tobytes() == vp0


def test_deterministic_outputs():
    spec = small_spec("bf16", 16, 4, 128, 128, 16, True, 3)
    meta = workloads.make_meta([1, 4, 40], [3000, 2000, 800], 16, 3)
    outs = []
    for _ in range(2):
        tensors = workloads.make_tensors(spec, meta, 3, device="cuda")
        o, lse, _ = run_library(spec, meta, tensors)
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_plan_reuse_across_layers():
    # one plan, two "layers" with different pools and queries
    spec = small_spec("bf16", 8, 2, 128, 128, 16, True, 5)
    meta = workloads.make_meta([1, 4, 20], [500, 300, 64], 16, 5)
    cfg = config_of(spec)
    plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages, num_cus=100000)
    for layer in range(2):
        tensors = workloads.make_tensors(spec, meta, 50 + layer, device="cuda")
        host = {k: (None if v is None else raw(v)) for k, v in tensors.items()}
        kp2, vp2, o_ref, lse_ref = expected(spec, meta, host["q"], host["k_new"], host["v_new"],
                                            host["k_pool"], host["v_pool"])
        plan.append(tensors["k_new"], tensors["v_new"], tensors["k_pool"], tensors["v_pool"])
        o, lse = plan.attention(tensors["q"], tensors["k_pool"], tensors["v_pool"])
        torch.cuda.synchronize()
        assert raw(tensors["k_pool"]).tobytes() == kp2.tobytes()
        assert max_err(o, o_ref) <= 2e-2 and max_err(lse, lse_ref) <= 2e-2


def test_merge_state_matches_oracle():
    rng = np.random.default_rng(9)
    for dtype, tol in (("f32", 1e-5), ("bf16", 2e-2)):
        rows, heads, dim = 37, 5, 64
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        o_a = torch.randn(rows, heads, dim, device="cuda").to(tdt)
        o_b = torch.randn(rows, heads, dim, device="cuda").to(tdt)
        la = torch.from_numpy(rng.standard_normal((rows, heads)).astype(np.float32) * 3).cuda()
        lb = torch.from_numpy(rng.standard_normal((rows, heads)).astype(np.float32) * 3).cuda()
        la[0, :] = float("-inf")           # empty partition A
        lb[1, :] = float("-inf")           # empty partition B
        la[2, :] = float("-inf")
        lb[2, :] = float("-inf")           # both empty
        o, lse = rpa.merge_state(o_a, la, o_b, lb)
        torch.cuda.synchronize()
        want_o, want_l = oracle.merge(f64(raw(o_a)), la.double().cpu().numpy(), f64(raw(o_b)),
                                      lb.double().cpu().numpy())
        got_l = lse.double().cpu().numpy()
        assert np.all(got_l[2] == -np.inf)
        fin = np.isfinite(want_l)
        assert np.max(np.abs(got_l[fin] - want_l[fin])) <= 1e-5
        assert max_err(o, want_o) <= tol
        # in place: o aliases o_a
        o_alias = o_a.clone()
        rpa.rpa_merge_state(o_alias, la, o_b, lb, o_alias, None, rows, heads, dim,
                            rpa.RPA_DTYPE_F32 if dtype == "f32" else rpa.RPA_DTYPE_BF16)
        torch.cuda.synchronize()
        assert torch.equal(o_alias, o)


GROWING = [
    # (dtype, hq, hkv, dqk, dv, P, qo, kv, num_cus, key scale per 512-key segment)
    ("bf16", 128, 1, 576, 512, 64, [2, 1, 2], [3000, 1800, 700], 4, [1, 32, 1024]),  # latent
    ("bf16", 128, 1, 576, 512, 64, [2, 1, 2], [3000, 1800, 700], 0, [1, 32, 1024]),  # split
    ("bf16", 16, 2, 128, 128, 16, [1, 5, 40], [2500, 1200, 900], 4, [1, 32, 1024]),  # GQA
    # fp32 keeps the scores small enough for its 1e-4 bound (fp32 dot products)
    ("f32", 8, 2, 64, 64, 16, [1, 3], [1100, 600], 0, [1, 8]),                      # generic
]


@pytest.mark.parametrize("case", GROWING, ids=[f"g{i}" for i in range(len(GROWING))])
def test_scores_jump_far_above_the_first_tiles(case):
    # Later keys are scaled up by powers of two (values are not): a row's max
    # rises by tens to hundreds of log2 units after its first tiles, far past
    # any lazy-rescale slack, so every kernel must move its reference (or redo
    # its pass).
    dtype, hq, hkv, dqk, dv, P, qo, kv, num_cus, scales = case
    spec = small_spec(dtype, hq, hkv, dqk, dv, P, True, 31)
    meta = workloads.make_meta(qo, kv, P, 31)
    tensors = workloads.make_tensors(spec, meta, 31, device="cuda")
    # Near one-hot rows return a single value row: values of magnitude <~ 1
    # keep the bf16 output rounding (half an ulp) well inside the bound.
    for name in (("k_pool", "k_new") if dqk == 576 else ("v_pool", "v_new")):
        tensors[name] *= 0.25
    for r in range(meta.batch_size):
        ids = meta.kv_page_indices[meta.kv_page_indptr[r]:meta.kv_page_indptr[r + 1]]
        for i, pg in enumerate(ids):
            f = float(scales[min((i * P) // 512, len(scales) - 1)])
            if dqk == 576:
                # the latent's values are its first 512 dims: scale only the
                # 64 key-only dims so O keeps its magnitude
                tensors["k_pool"][int(pg), :, :, 512:] *= f
            else:
                tensors["k_pool"][int(pg)] *= f
    log(f"case {case}")
    check_full(spec, meta, tensors, num_cus=num_cus, label=f"growing {dtype} d{dqk}")



DEEP = [
    # (dtype, hq, hkv, dqk, dv, P, qo, kv, log2 score of every key against 0)
    ("bf16", 16, 2, 128, 128, 16, [1, 5, 40], [700, 300, 500], -300.0),  # every P underflows
    ("bf16", 16, 2, 128, 128, 16, [1, 5, 40], [700, 300, 500], -80.0),   # sums below 2^-64
    ("bf16", 128, 1, 576, 512, 64, [2, 1], [900, 400], -300.0),          # latent
    ("f32", 8, 2, 64, 64, 16, [1, 3], [300, 200], -300.0),               # generic
]


@pytest.mark.parametrize("case", DEEP, ids=[f"d{i}" for i in range(len(DEEP))])
def test_scores_far_below_zero(case):
    # Every key close to one vector u and every query -beta u: all scores of a
    # row sit near one large negative value, so that against a reference of 0
    # every P underflows (or every row sum falls below 2^-64).  The softmax is
    # well defined (weights near uniform): each kernel must move its reference
    # down to the scores.
    dtype, hq, hkv, dqk, dv, P, qo, kv, target = case
    spec = small_spec(dtype, hq, hkv, dqk, dv, P, True, 53)
    meta = workloads.make_meta(qo, kv, P, 53)
    tensors = workloads.make_tensors(spec, meta, 53, device="cuda")
    gen = torch.Generator().manual_seed(53)
    u = torch.randn(dqk, generator=gen)
    u *= math.sqrt(dqk) / float(u.norm())  # |u|^2 = dqk
    beta = -target / (dqk * spec.sm_scale * math.log2(math.e))
    used = torch.from_numpy(workloads.referenced_pages(meta))
    kp = tensors["k_pool"]
    keys = (u + 0.02 * torch.randn(tuple(kp.shape), generator=gen)).to(kp.dtype)
    kp[used.cuda()] = keys[used].cuda()
    kn = tensors["k_new"]
    kn.copy_((u + 0.02 * torch.randn(tuple(kn.shape), generator=gen)).to(kn.dtype).cuda())
    tensors["q"].copy_((-beta * u).expand(tuple(tensors["q"].shape)).to(tensors["q"].dtype).cuda())
    log(f"case {case}")
    check_full(spec, meta, tensors, label=f"deep {dtype} d{dqk} {target}")


LONG = [
    # (dtype, hq, hkv, dqk, dv, P, qo, kv, num_cus): few compute units, so pieces stay long
    ("bf16", 32, 8, 128, 128, 16, [1, 4], [40000, 9000], 1),    # decode pieces past 256 pages
    ("bf16", 8, 1, 128, 128, 16, [300], [12000], 2),            # prefill split at 8192 keys
    ("bf16", 16, 1, 576, 512, 64, [2], [40000], 1),             # latent split at 32768 keys
]


@pytest.mark.parametrize("case", LONG, ids=[f"long{i}" for i in range(len(LONG))])
def test_long_requests(case):
    dtype, hq, hkv, dqk, dv, P, qo, kv, num_cus = case
    spec = small_spec(dtype, hq, hkv, dqk, dv, P, True, 43)
    meta = workloads.make_meta(qo, kv, P, 43)
    tensors = workloads.make_tensors(spec, meta, 43, device="cuda")
    log(f"case {case}")
    check_full(spec, meta, tensors, num_cus=num_cus, label=f"long d{dqk}")


@pytest.mark.parametrize("dqk", [576, 128])
def test_pool_base_with_bit_31_of_its_low_word_set(dqk):
    # Kernels that keep a wave-uniform 64-bit base in scalar registers must
    # widen its halves without sign extension: put the pool at an address
    # whose low 32 bits are >= 2^31 (and, for contrast, below it).
    dv = 512 if dqk == 576 else 128
    hq, hkv, P = (16, 1, 64) if dqk == 576 else (8, 2, 16)
    spec = small_spec("bf16", hq, hkv, dqk, dv, P, True, 41)
    meta = workloads.make_meta([2, 1, 9], [900, 700, 300], P, 41)
    base_tensors = workloads.make_tensors(spec, meta, 41, device="cuda")
    pool = base_tensors["k_pool"]
    need = pool.numel() * 2
    for high in (True, False):
        buf = torch.empty(need + (1 << 32) + 4096, dtype=torch.uint8, device="cuda")
        addr = buf.data_ptr()
        want = (addr & ~0xFFFFFFFF) + (0x80000000 if high else 0)
        while want < addr:
            want += 1 << 32
        off = want - addr
        assert off + need <= buf.numel() and ((want & 0xFFFFFFFF) >= 0x80000000) == high
        k_pool = buf[off:off + need].view(torch.bfloat16).view(pool.shape)
        k_pool.copy_(pool)
        tensors = dict(base_tensors, k_pool=k_pool)
        if base_tensors["v_pool"] is not None:
            tensors["v_pool"] = base_tensors["v_pool"].clone()
        log(f"dqk {dqk} pool at {want:#x} (bit 31 of the low word {'set' if high else 'clear'})")
        check_full(spec, meta, tensors, num_cus=4, label=f"pool-address d{dqk} high={high}")
        del buf, k_pool, tensors
        torch.cuda.empty_cache()


def test_invalid_calls_launch_nothing():
    spec = small_spec("bf16", 4, 2, 128, 128, 16, True, 1)
    meta = workloads.make_meta([2], [10], 16, 1)
    tensors = workloads.make_tensors(spec, meta, 1, device="cuda")
    before = tensors["k_pool"].clone()
    cfg = config_of(spec)
    plan = rpa.Plan(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                    meta.num_pages)
    bad = rpa.rpa_cache_strides(1, 1, 1)
    with pytest.raises(rpa.RpaError) as ei:
        rpa.rpa_kv_append(plan.handle, tensors["k_new"], tensors["v_new"], tensors["k_pool"],
                          tensors["v_pool"], bad, bad)
    assert ei.value.status == rpa.RPA_ERR_INVALID_ARG
    o = torch.full((2, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rpa.RpaError):
        rpa.rpa_batch_attention(plan.handle, tensors["q"], tensors["k_pool"], None,
                                rpa.strides_of(tensors["k_pool"]), None, o, None)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), tensors["k_pool"].view(torch.int16))
    assert torch.all(o == 7.0)


# ----------------------------------------------------------------------------
# Full-size workloads (the launch configuration the benchmark times)
# ----------------------------------------------------------------------------


def test_workload_mixed_7b_full():
    spec, meta, tensors = workloads.workload("mixed_7b", device="cuda")
    full_parity(spec, meta, tensors, "mixed_7b", log=log)


def test_workload_decode_verify_gqa_full():
    """All 256 requests (128 decodes, 128 four-token verifications) element by
    element, in the launch configuration the benchmark times."""
    spec, meta, tensors = workloads.workload("decode_verify_gqa", device="cuda")
    full_parity(spec, meta, tensors, "decode_verify_gqa", log=log)


def test_workload_mla_absorbed_full():
    """All 64 latent requests (two query tokens over 128 heads each) element by
    element, in the launch configuration the benchmark times."""
    spec, meta, tensors = workloads.workload("mla_absorbed", device="cuda")
    full_parity(spec, meta, tensors, "mla_absorbed", log=log)


def _chunked_run(spec, pages, num_pages, q, k, v, C, stop_after=None, pools=None):
    """GPU chunked prefill of one prompt; returns (o, lse, k_pool, v_pool)."""
    L = q.shape[0]
    dev = q.device
    if pools is None:
        k_pool = torch.full((num_pages, 1, 16, 128), float("nan"), dtype=torch.bfloat16, device=dev)
        v_pool = k_pool.clone()
    else:
        k_pool, v_pool = pools
    o = torch.empty((L, spec.num_qo_heads, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((L, spec.num_qo_heads), dtype=torch.float32, device=dev)
    cfg = config_of(spec)
    n_chunks = -(-L // C)
    start_chunk = 0 if stop_after is None else 0
    for s in range(start_chunk, n_chunks):
        if stop_after is not None and s > stop_after:
            break
        a = s * C
        n = min(C, L - a)
        plan = rpa.Plan(cfg, [0, n], [a + n], [0, len(pages)], pages, num_pages)
        plan.append(k[a:a + n], v[a:a + n], k_pool, v_pool)
        plan.attention(q[a:a + n], k_pool, v_pool, o=o[a:a + n], lse=lse[a:a + n])
    torch.cuda.synchronize()
    return o, lse, k_pool, v_pool


def test_workload_chunked_equals_one_shot():
    spec = workloads.SPECS["chunked_gqa"]
    L, C = spec.extra["prompt_len"], spec.extra["chunk"]
    q, k, v = workloads.make_prompt(spec, spec.seed, device="cuda")
    meta = workloads.make_meta([L], [L], 16, spec.seed)
    pages = meta.kv_page_indices
    o_c, l_c, kp_c, vp_c = _chunked_run(spec, pages, meta.num_pages, q, k, v, C)
    o_1, l_1, kp_1, vp_1 = _chunked_run(spec, pages, meta.num_pages, q, k, v, L)
    # identical caches, both equal to the oracle's append
    assert torch.equal(kp_c.view(torch.int16), kp_1.view(torch.int16))
    assert torch.equal(vp_c.view(torch.int16), vp_1.view(torch.int16))
    kp0 = np.full((meta.num_pages, 1, 16, 128), 0x7FC0, dtype=np.uint16)
    b = oracle.Batch([0, L], [L], [0, len(pages)], pages, 16)
    kp2, vp2 = oracle.append(kp0, kp0.copy(), raw(k), raw(v), b)
    assert raw(kp_c).tobytes() == kp2.tobytes() and raw(vp_c).tobytes() == vp2.tobytes()
    # outputs of both GPU runs within tolerance of the oracle's one-shot prefill
    o_ref, lse_ref = oracle.attend(f64(raw(q)), f64(kp2), f64(vp2), b, 8, 1, spec.sm_scale)
    for name, o, lse in (("chunked", o_c, l_c), ("one-shot", o_1, l_1)):
        eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
        log(f"[chunked_gqa {name}] max|dO|={eo:.3g} max|dLSE|={el:.3g}")
        assert eo <= 2e-2 and el <= 2e-2


def test_chunked_prefill_resumes_from_the_cache_alone():
    # stop after chunk 5, move the cache through host memory into a fresh pool,
    # continue: bit-identical to the uninterrupted run
    spec = workloads.SPECS["chunked_gqa"]
    L, C = 2048, 256
    q, k, v = workloads.make_prompt(spec, 77, device="cuda")
    q, k, v = q[:L].contiguous(), k[:L].contiguous(), v[:L].contiguous()
    meta = workloads.make_meta([L], [L], 16, 77)
    pages = meta.kv_page_indices
    o_full, l_full, kp_full, vp_full = _chunked_run(spec, pages, meta.num_pages, q, k, v, C)
    o_a, l_a, kp_a, vp_a = _chunked_run(spec, pages, meta.num_pages, q, k, v, C, stop_after=5)
    kp_host, vp_host = kp_a.cpu(), vp_a.cpu()
    kp_b, vp_b = kp_host.cuda(), vp_host.cuda()
    cfg = config_of(spec)
    for s in range(6, L // C):
        a = s * C
        plan = rpa.Plan(cfg, [0, C], [a + C], [0, len(pages)], pages, meta.num_pages)
        plan.append(k[a:a + C], v[a:a + C], kp_b, vp_b)
        plan.attention(q[a:a + C], kp_b, vp_b, o=o_a[a:a + C], lse=l_a[a:a + C])
    torch.cuda.synchronize()
    assert torch.equal(kp_b.view(torch.int16), kp_full.view(torch.int16))
    assert torch.equal(o_a.view(torch.int16), o_full.view(torch.int16))
    assert torch.equal(l_a, l_full)
