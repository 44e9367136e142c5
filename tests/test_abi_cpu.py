"""C-ABI library checks that need no GPU: exports, planner properties, error paths.

The planner is pure host code, so plans are built and inspected here through
rpa_plan_debug_dump; calls that would touch the device are only exercised on
their argument-validation paths, which return before any HIP call.
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
import workloads
import ragged_paged_kv_append_amd as rpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rpa.LIB_PATH):
        from ragged_paged_kv_append_amd import build
        build.build()
    return rpa.lib()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "rpa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rpa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(rpa.EXPORTED_SYMBOLS)


def test_abi_version_and_status_strings(L):
    assert rpa.rpa_abi_version() == 3
    for code, name in [(0, "RPA_OK"), (-1, "RPA_ERR_INVALID_ARG"), (-2, "RPA_ERR_UNSUPPORTED"),
                       (-3, "RPA_ERR_WORKSPACE_TOO_SMALL"), (-4, "RPA_ERR_PAGE_OOB"),
                       (-5, "RPA_ERR_DUPLICATE_WRITE_PAGE"), (-6, "RPA_ERR_HIP"),
                       (-7, "RPA_ERR_NOT_UPLOADED"), (-8, "RPA_ERR_HOST_ALLOC"),
                       (-9, "RPA_ERR_INTERNAL")]:
        assert rpa.rpa_status_string(code) == name


# ----------------------------------------------------------------------------
# Planner properties
# ----------------------------------------------------------------------------


def plan_for(meta, cfg, num_cus=0):
    return rpa.rpa_plan_create(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                               meta.kv_page_indices, meta.num_pages, num_cus)


def check_plan(plan, meta, cfg):
    """Every (row, visible key) pair is in exactly one item; items stay inside
    their request; splits, merge rows and the append map are consistent."""
    G = cfg.num_qo_heads // cfg.num_kv_heads
    items = rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8)
    splits = rpa.rpa_plan_debug_dump(plan, "splits").reshape(-1, 3)
    merge_rows = set(rpa.rpa_plan_debug_dump(plan, "merge_rows").tolist())
    app = rpa.rpa_plan_debug_dump(plan, "append").reshape(-1, 2)
    summary = rpa.rpa_plan_debug_dump(plan, "summary")
    assert summary[2] == len(items)
    B = meta.batch_size
    batch = oracle.Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices,
                         meta.page_size)
    cover = {}
    piece = {}  # (request, piece) -> its key range, the same in every item
    for r_, g, row0, row1, k0, k1, s, kc in items.tolist():
        n = batch.qo_len(r_)
        Lr = int(meta.kv_len[r_])
        assert 0 <= r_ < B and 0 <= g < cfg.num_kv_heads
        assert 0 <= row0 < row1 <= n * G
        assert 0 <= k0 < k1 <= Lr
        S, chunk, base = splits[r_]
        assert 0 <= s < S and piece.setdefault((r_, s), (k0, k1)) == (k0, k1)
        if chunk > 0:  # equal pieces
            assert k0 == s * chunk and k1 == min(Lr, k0 + chunk)
        for row in range(row0, row1):
            key = (r_, g, row)
            cover.setdefault(key, []).append((k0, k1))
    # pieces of unequal length (chunk 0) tile the request in order, starting at
    # multiples of 64
    starts = {}
    for r_ in range(B):
        S, chunk, base = splits[r_]
        if chunk == 0 and S > 0:
            rng = [piece[(r_, s)] for s in range(S)]
            assert rng[0][0] == 0 and rng[-1][1] == int(meta.kv_len[r_])
            assert all(a[1] == b[0] for a, b in zip(rng, rng[1:]))
            assert all(a[0] % 64 == 0 for a in rng)
            starts[r_] = [a[0] for a in rng]

    def live(r_, S, chunk, pmax):
        """Pieces that hold a key at or below pmax."""
        if pmax < 0:
            return 0
        if chunk > 0:
            return min(S, pmax // chunk + 1)
        return sum(1 for k0 in starts[r_] if k0 <= pmax)
    for r_ in range(B):
        n = batch.qo_len(r_)
        Lr = int(meta.kv_len[r_])
        c = Lr - n
        S, chunk, base = splits[r_]
        for g in range(cfg.num_kv_heads):
            for row in range(n * G):
                t = row // G
                pmax = c + t if cfg.causal else Lr - 1
                everything = sorted(cover.get((r_, g, row), []))
                assert len(set(everything)) == len(everything), "a piece covers a row twice"
                # the merge reads the pieces that hold a key the row sees: they
                # start at 0, are contiguous and end past the last visible key
                ranges = [x for x in everything if x[0] <= pmax]
                assert ranges, (r_, g, row)
                assert ranges[0][0] == 0
                for (a0, a1), (b0, b1) in zip(ranges, ranges[1:]):
                    assert a1 == b0
                assert ranges[-1][1] > pmax
                assert len(ranges) == live(r_, S, chunk, pmax)
        for t in range(n):
            i = int(meta.qo_indptr[r_]) + t
            assert (i in merge_rows) == (S > 1)
            assert tuple(app[i]) == oracle.slot_of(batch, r_, c + t)
    # every decode item sits in exactly one workgroup list
    n_dec = int(np.sum(items[:, 7] == 1))
    if n_dec:
        wg = rpa.rpa_plan_debug_dump(plan, "wg_decode")
        assert wg[0] == 0 and wg[-1] == n_dec and np.all(np.diff(wg) >= 0)
    # each merge row's first partial row, piece stride and live piece count
    mrows = rpa.rpa_plan_debug_dump(plan, "merge_rows").tolist()
    minfo = rpa.rpa_plan_debug_dump(plan, "merge_info").reshape(-1, 4)
    assert len(minfo) == len(mrows)
    for x, i in enumerate(mrows):
        r_ = int(np.searchsorted(np.asarray(meta.qo_indptr), i, side="right")) - 1
        n = batch.qo_len(r_)
        t = i - int(meta.qo_indptr[r_])
        Lr = int(meta.kv_len[r_])
        S, chunk, base = splits[r_]
        pmax = Lr - n + t if cfg.causal else Lr - 1
        assert tuple(minfo[x].tolist()) == (base + t, n, live(r_, S, chunk, pmax), 0), (i, minfo[x])
    return items, splits


@pytest.mark.parametrize("name", ["tiny_fp32", "mixed_7b", "decode_verify_gqa", "mla_absorbed"])
def test_planner_covers_workloads(L, name):
    spec = workloads.SPECS[name]
    qo, kv = workloads.lengths(name)
    meta = workloads.make_meta(qo, kv, spec.page_size, spec.seed)
    cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk, spec.head_dim_v,
                          spec.page_size, spec.dtype, spec.causal, spec.sm_scale)
    if name in ("mixed_7b", "decode_verify_gqa", "mla_absorbed"):
        # full coverage check is quadratic in rows; check a sub-batch plus the summary
        sub = workloads.make_meta(qo[:6], kv[:6], spec.page_size, spec.seed)
        check_plan(plan_for(sub, cfg), sub, cfg)
        plan = plan_for(meta, cfg)
        summary = rpa.rpa_plan_debug_dump(plan, "summary")
        assert summary[0] == len(kv) and summary[1] == int(np.sum(qo))
    else:
        check_plan(plan_for(meta, cfg), meta, cfg)


@pytest.mark.parametrize("seed", range(12))
def test_planner_random_batches(L, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    qo = rng.integers(0, 18, size=B)
    kv = qo + rng.integers(0, 300, size=B)
    P = int(rng.choice([1, 4, 16, 64]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    dims = [(64, 64), (128, 128)][seed % 2]
    dtype = ["bf16", "f32"][(seed // 2) % 2]
    causal = seed % 3 != 0
    meta = workloads.make_meta(qo, kv, P, seed, extra_pages_per_req=seed % 2)
    cfg = rpa.make_config(hkv * G, hkv, dims[0], dims[1], P, dtype, causal)
    for cus in (0, 1, 100000):
        check_plan(plan_for(meta, cfg, cus), meta, cfg)


def test_planner_splits_long_requests(L):
    meta = workloads.make_meta([1, 1], [40000, 100], 16, 1)
    cfg = rpa.make_config(8, 8, 128, 128, 16, "bf16")
    plan = plan_for(meta, cfg)
    splits = rpa.rpa_plan_debug_dump(plan, "splits").reshape(-1, 3)
    assert splits[0][0] > 1 and splits[1][0] == 1
    items = rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8)
    costs = (items[:, 5] - items[:, 4]) * (items[:, 3] - items[:, 2])
    # heaviest items are listed first within each kernel class, or within each
    # workgroup's list where the class has them
    lists = {1: "wg_decode", 2: "wg_prefill", 3: "wg_mla"}
    for k in set(items[:, 7].tolist()):
        ck = costs[items[:, 7] == k]
        if k in lists:
            wg = rpa.rpa_plan_debug_dump(plan, lists[k])
            assert wg[0] == 0 and wg[-1] == len(ck)
            for b in range(len(wg) - 1):
                assert np.all(np.diff(ck[wg[b]:wg[b + 1]]) <= 0)
        else:
            assert np.all(np.diff(ck) <= 0)


@pytest.mark.parametrize("case", ["one_shot_8192", "mixed_7b", "mla_absorbed", "chunk_15"])
def test_planner_packs_tile_items_onto_workgroups(L, case):
    """Tile-class items are grouped per workgroup (wg_indptr); the grouping is a
    longest-first packing, so no workgroup carries more than the average load
    plus one item."""
    if case == "one_shot_8192":
        meta = workloads.make_meta([8192], [8192], 16, 3)
        cfg = rpa.make_config(8, 1, 128, 128, 16, "bf16")
        k, table = 2, "wg_prefill"
    elif case == "chunk_15":
        meta = workloads.make_meta([512], [8192], 16, 3)
        cfg = rpa.make_config(8, 1, 128, 128, 16, "bf16")
        k, table = 2, "wg_prefill"
    else:
        spec = workloads.SPECS[case]
        qo, kv = workloads.lengths(case)
        meta = workloads.make_meta(qo, kv, spec.page_size, spec.seed)
        cfg = rpa.make_config(spec.num_qo_heads, spec.num_kv_heads, spec.head_dim_qk,
                              spec.head_dim_v, spec.page_size, spec.dtype, spec.causal,
                              spec.sm_scale)
        k, table = (3, "wg_mla") if case == "mla_absorbed" else (2, "wg_prefill")
    for cus in (0, 7, 100000):
        plan = plan_for(meta, cfg, cus)
        items = rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8)
        items = items[items[:, 7] == k]
        wg = rpa.rpa_plan_debug_dump(plan, table)
        per_cu = {2: 1, 3: 1}[k]  # resident workgroups per compute unit of each class
        slots = per_cu * (cus if cus > 0 else 256)
        paired = k == 3 and slots % 16 == 0
        assert wg[0] == 0 and wg[-1] == len(items)
        if paired:
            # latent row tiles of one key range sit on workgroups b and b + 8
            # (one XCD), at the same place in both lists; in this workload every
            # key range has two row tiles (two query tokens of 128 heads)
            n_wgs = len(wg) - 1
            assert n_wgs % 16 == 0 and n_wgs <= slots and np.all(np.diff(wg) >= 0)
            pairs = 0
            for b in range(n_wgs):
                if b % 16 >= 8:
                    continue
                ka = items[wg[b]:wg[b + 1]][:, [0, 1, 4, 5]]
                kb = items[wg[b + 8]:wg[b + 9]][:, [0, 1, 4, 5]]
                n_ = min(len(ka), len(kb))
                pairs += int(np.sum(np.all(ka[:n_] == kb[:n_], axis=1)))
            assert pairs == len(items) // 2
            continue
        assert np.all(np.diff(wg) >= 1)
        assert len(wg) - 1 == min(slots, len(items))
        G = cfg.num_qo_heads // cfg.num_kv_heads
        cached = {r: int(meta.kv_len[r]) - int(meta.qo_indptr[r + 1] - meta.qo_indptr[r])
                  for r in range(meta.batch_size)}
        cost = []
        for r_, g, row0, row1, k0, k1, s, kc in items.tolist():
            last = cached[r_] + (row1 - 1) // G if cfg.causal else int(meta.kv_len[r_]) - 1
            cost.append((min(k1, last + 1) - k0) * (-(-(row1 - row0) // 32) * 32))
        cost = np.array(cost)
        loads = np.array([cost[wg[b]:wg[b + 1]].sum() for b in range(len(wg) - 1)])
        assert loads.max() <= cost.sum() / len(loads) + cost.max()
        # every list runs its items longest first
        for b in range(len(wg) - 1):
            assert np.all(np.diff(cost[wg[b]:wg[b + 1]]) <= 0)
        # lists are handed out XCD by XCD (workgroup w runs on XCD w % 8) in the
        # order of (request, KV head, first key, first row) of their first item
        n_wgs = len(wg) - 1
        order = [w for x in range(8) for w in range(x, n_wgs, 8)]
        firsts = [tuple(items[wg[w]][[0, 1, 4, 2]].tolist()) for w in order]
        assert firsts == sorted(firsts)


def test_planner_empty_batch_and_empty_requests(L):
    cfg = rpa.make_config(4, 2, 64, 64, 16, "f32")
    plan = rpa.rpa_plan_create(cfg, [0], [], [0], [], 0)
    assert rpa.rpa_plan_debug_dump(plan, "summary")[2] == 0
    meta = workloads.make_meta([0, 3, 0], [5, 3, 0], 16, 2)
    plan = plan_for(meta, cfg)
    check_plan(plan, meta, cfg)


def test_planner_is_deterministic(L):
    spec = workloads.SPECS["mixed_7b"]
    qo, kv = workloads.lengths("mixed_7b")
    meta = workloads.make_meta(qo, kv, 16, 3)
    cfg = rpa.make_config(32, 32, 128, 128, 16, "bf16")
    a = rpa.rpa_plan_debug_dump(plan_for(meta, cfg), "items")
    b = rpa.rpa_plan_debug_dump(plan_for(meta, cfg), "items")
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# Error paths: each invalid input returns its code and builds nothing
# ----------------------------------------------------------------------------


def expect(status, fn, *args):
    with pytest.raises(rpa.RpaError) as ei:
        fn(*args)
    assert ei.value.status == status, str(ei.value)
    assert rpa.rpa_last_error_message() != ""


def test_plan_create_error_paths(L):
    cfg = rpa.make_config(4, 2, 64, 64, 16, "f32")
    ok = dict(qo=[0, 1, 3], kv=[5, 20], pip=[0, 1, 3], pix=[0, 1, 2], num_pages=4)

    def call(cfg=cfg, **kw):
        a = dict(ok)
        a.update(kw)
        return rpa.rpa_plan_create(cfg, a["qo"], a["kv"], a["pip"], a["pix"], a["num_pages"])

    call()  # the baseline is valid
    expect(rpa.RPA_ERR_INVALID_ARG, lambda: call(qo=[1, 2, 3]))            # indptr not from 0
    expect(rpa.RPA_ERR_INVALID_ARG, lambda: call(qo=[0, 3, 1]))            # decreasing
    expect(rpa.RPA_ERR_INVALID_ARG, lambda: call(kv=[0, 20]))              # kv_len < qo_len, causal
    expect(rpa.RPA_ERR_INVALID_ARG, lambda: call(kv=[-1, 20]))             # negative kv_len
    expect(rpa.RPA_ERR_INVALID_ARG, lambda: call(pip=[0, 2, 1]))           # page indptr decreasing
    expect(rpa.RPA_ERR_PAGE_OOB, lambda: call(kv=[17, 20]))                # missing page
    expect(rpa.RPA_ERR_PAGE_OOB, lambda: call(pix=[0, 1, 4]))              # page id >= num_pages
    expect(rpa.RPA_ERR_PAGE_OOB, lambda: call(pix=[0, -1, 2]))             # negative page id
    expect(rpa.RPA_ERR_DUPLICATE_WRITE_PAGE, lambda: call(pix=[0, 1, 0]))  # written page twice
    expect(rpa.RPA_ERR_DUPLICATE_WRITE_PAGE, lambda: call(pix=[2, 1, 2]))
    # a shared page that nobody writes is fine (prefix sharing)
    rpa.rpa_plan_create(cfg, [0, 1, 2], [20, 20], [0, 2, 4], [0, 1, 0, 2], 3)
    bad = [
        (rpa.RPA_ERR_UNSUPPORTED, rpa.make_config(4, 2, 96, 96, 16, "f32")),
        (rpa.RPA_ERR_UNSUPPORTED, rpa.make_config(4, 2, 64, 64, 12, "f32")),
        (rpa.RPA_ERR_UNSUPPORTED, rpa.make_config(4, 2, 64, 64, 512, "f32")),
        (rpa.RPA_ERR_UNSUPPORTED, rpa.make_config(4, 2, 576, 512, 64, "bf16")),
        (rpa.RPA_ERR_INVALID_ARG, rpa.make_config(3, 2, 64, 64, 16, "f32")),
        (rpa.RPA_ERR_INVALID_ARG, rpa.make_config(0, 2, 64, 64, 16, "f32")),
        (rpa.RPA_ERR_INVALID_ARG, rpa.rpa_attn_config(4, 2, 64, 64, 16, 7, 1, 0.1)),
        (rpa.RPA_ERR_INVALID_ARG, rpa.rpa_attn_config(4, 2, 64, 64, 16, 0, 2, 0.1)),
        (rpa.RPA_ERR_INVALID_ARG, rpa.rpa_attn_config(4, 2, 64, 64, 16, 0, 1, float("nan"))),
        (rpa.RPA_ERR_INVALID_ARG, rpa.rpa_attn_config(4, 2, 64, 64, 16, 0, 1, 0.0)),
        (rpa.RPA_ERR_INVALID_ARG, rpa.rpa_attn_config(4, 2, 64, 64, 16, 0, 1, -0.125)),
    ]
    for status, c in bad:
        expect(status, lambda c=c: call(cfg=c))
    # null pointers through the raw C entry point
    out = ctypes.c_void_p()
    assert L.rpa_plan_create(None, None, 0, ctypes.byref(out)) == rpa.RPA_ERR_INVALID_ARG
    batch = rpa.rpa_batch_desc(2, None, None, None, None, 4)
    assert L.rpa_plan_create(ctypes.byref(cfg), ctypes.byref(batch), 0,
                             ctypes.byref(out)) == rpa.RPA_ERR_INVALID_ARG
    assert out.value is None


def test_device_calls_validate_before_touching_the_device(L):
    cfg = rpa.make_config(4, 2, 64, 64, 16, "f32")
    plan = rpa.rpa_plan_create(cfg, [0, 1], [5], [0, 1], [0], 1)
    st = rpa.rpa_cache_strides(2 * 16 * 64, 16 * 64, 64)
    fake = 1 << 40  # never dereferenced: validation fails first
    expect(rpa.RPA_ERR_NOT_UPLOADED, rpa.rpa_batch_attention, plan, fake, fake, fake, st, st, fake,
           None, 0)
    expect(rpa.RPA_ERR_NOT_UPLOADED, rpa.rpa_kv_append, plan, fake, fake, fake, fake, st, st, 0)
    size = rpa.rpa_plan_workspace_size(plan)
    assert size > 0 and size % 256 == 0
    expect(rpa.RPA_ERR_WORKSPACE_TOO_SMALL, rpa.rpa_plan_upload, plan, fake, size - 1, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_plan_upload, plan, fake + 16, size, 0)
    assert L.rpa_plan_upload(None, fake, size, None) == rpa.RPA_ERR_INVALID_ARG
    # standalone merge argument checks
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake, fake, fake, fake, fake, fake, 4, 2,
           12, rpa.RPA_DTYPE_F32, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake, fake, fake, fake, fake, fake, -1, 2,
           8, rpa.RPA_DTYPE_F32, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, None, fake, fake, fake, fake, fake, 4, 2,
           8, rpa.RPA_DTYPE_F32, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake + 4, fake, fake, fake, fake, fake,
           4, 2, 8, rpa.RPA_DTYPE_F32, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake, fake, fake, fake, fake, fake, 4, 2,
           8, 9, 0)
    # an output lse over an input lse would race between the threads of a row
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake, fake + 4096, fake + 8192,
           fake + 12288, fake, fake + 4096, 4, 2, 8, rpa.RPA_DTYPE_F32, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_merge_state, fake, fake + 4096, fake + 8192,
           fake + 12288, fake, fake + 12288, 4, 2, 8, rpa.RPA_DTYPE_F32, 0)
    with pytest.raises(rpa.RpaError):
        rpa.rpa_plan_debug_dump(plan, "no_such_table")


def test_page_copy_validates_pools_before_touching_the_device(L):
    st = rpa.rpa_cache_strides(2 * 16 * 128, 16 * 128, 128)
    fake = 1 << 40  # never dereferenced: validation fails first
    bf16 = rpa.RPA_DTYPE_BF16
    # (src_pool_pages, src_pool_heads, src_pages, dst_pool_pages, dst_pool_heads, dst_pages,
    #  num_pages, src_head0, dst_head0, num_heads) -> status
    cases = [
        ((10, 2, None, 9, 2, None, 10, 0, 0, 2), rpa.RPA_ERR_PAGE_OOB),   # identity past dst
        ((9, 2, None, 10, 2, None, 10, 0, 0, 2), rpa.RPA_ERR_PAGE_OOB),   # identity past src
        ((10, 2, None, 10, 2, None, 4, 1, 0, 2), rpa.RPA_ERR_INVALID_ARG),  # src heads 1..2 of 2
        ((10, 2, None, 10, 1, None, 4, 0, 0, 2), rpa.RPA_ERR_INVALID_ARG),  # dst has one head
        ((10, 0, None, 10, 2, None, 4, 0, 0, 1), rpa.RPA_ERR_INVALID_ARG),  # no heads
        ((-1, 2, None, 10, 2, None, 0, 0, 0, 1), rpa.RPA_ERR_INVALID_ARG),  # negative pool
    ]
    for (sp, sh, sids, dp, dh, dids, n, h0s, h0d, nh), want in cases:
        got = L.rpa_page_copy(fake, ctypes.byref(st), sp, sh, sids, fake, ctypes.byref(st), dp,
                              dh, dids, n, h0s, h0d, nh, 16, 128, bf16, None)
        assert got == want, ((sp, sh, dp, dh, n, h0s, h0d, nh), got, want)
    # device page lists are checked in the kernel, so the host accepts any count
    # of them; a zero-length copy returns before any device work
    assert L.rpa_page_copy(fake, ctypes.byref(st), 1, 2, fake, fake, ctypes.byref(st), 1, 2,
                           fake, 0, 0, 0, 2, 16, 128, bf16, None) == rpa.RPA_OK


def test_binding_checks_tensors_before_any_launch():
    """The binding's checks of dtype, shape, contiguity, pool size and device
    raise INVALID_ARG before the C ABI is called (CPU tensors here: each case
    has exactly one thing wrong, and the all-correct case fails on the device)."""
    import torch
    cfg = rpa.make_config(8, 2, 128, 128, 16, "bf16")
    T, P, npg = 5, 16, 7
    bf = torch.bfloat16

    def good():
        return {"k_new": torch.zeros((T, 2, 128), dtype=bf), "v_new": torch.zeros((T, 2, 128), dtype=bf),
                "k_cache": torch.zeros((npg, 2, P, 128), dtype=bf),
                "v_cache": torch.zeros((npg, 2, P, 128), dtype=bf),
                "q": torch.zeros((T, 8, 128), dtype=bf), "o": torch.zeros((T, 8, 128), dtype=bf),
                "lse": torch.zeros((T, 8), dtype=torch.float32)}

    def append(t):
        rpa.check_append_args(cfg, T, npg, t["k_new"], t["v_new"], t["k_cache"], t["v_cache"])

    def attend(t):
        rpa.check_attention_args(cfg, T, npg, t["q"], t["k_cache"], t["v_cache"], t["o"], t["lse"])

    bad = {
        "k_new dtype": ("k_new", lambda t: t.float()),
        "k_new shape": ("k_new", lambda t: t[:T - 1]),
        "v_new heads": ("v_new", lambda t: torch.zeros((T, 1, 128), dtype=bf)),
        "q non-contiguous": ("q", lambda t: torch.zeros((T, 128, 8), dtype=bf).transpose(1, 2)),
        "o dtype": ("o", lambda t: t.float()),
        "lse dtype": ("lse", lambda t: t.double()),
        "k_cache too few pages": ("k_cache", lambda t: t[:npg - 1]),
        "v_cache page size": ("v_cache", lambda t: torch.zeros((npg, 2, 8, 128), dtype=bf)),
        "k_cache row": ("k_cache", lambda t: torch.zeros((npg, 2, P, 64), dtype=bf)),
        "v_cache last dim strided": ("v_cache",
                                     lambda t: torch.zeros((npg, 2, P, 256), dtype=bf)[..., ::2]),
    }
    for label, (key, mutate) in bad.items():
        t = good()
        t[key] = mutate(t[key])
        fns = [append] if key in ("k_new", "v_new") else [attend] if key in ("q", "o", "lse") \
            else [append, attend]
        for fn in fns:
            with pytest.raises(rpa.RpaError) as ei:
                fn(t)
            assert ei.value.status == rpa.RPA_ERR_INVALID_ARG, label
            assert "GPU" not in str(ei.value), (label, str(ei.value))
    for fn in (append, attend):
        with pytest.raises(rpa.RpaError) as ei:
            fn(good())
        assert "not a GPU" in str(ei.value)


def test_plan_debug_dump_append_matches_oracle(L):
    meta = workloads.make_meta([3, 1, 4], [10, 17, 4], 4, 9)
    cfg = rpa.make_config(2, 1, 64, 64, 4, "f32")
    plan = plan_for(meta, cfg)
    app = rpa.rpa_plan_debug_dump(plan, "append").reshape(-1, 2)
    batch = oracle.Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices, 4)
    i = 0
    for r in range(3):
        for t in range(batch.qo_len(r)):
            assert tuple(app[i]) == oracle.slot_of(batch, r, batch.cached_len(r) + t)
            i += 1


def test_cross_attention_plan_without_causal_mask(L):
    """Without causal masking kv_len may be below qo_len (the new tokens attend
    to cached keys only); kv_len = 0 rows go to the merge pass as empty states."""
    cfg = rpa.make_config(4, 2, 64, 64, 16, "f32", causal=False)
    plan = rpa.rpa_plan_create(cfg, [0, 3, 8, 9], [0, 2, 40], [0, 0, 1, 4], [3, 0, 1, 2], 4)
    items = rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8)
    assert 0 not in set(items[:, 0].tolist())          # kv_len 0: no work item
    assert {1, 2} <= set(items[:, 0].tolist())
    merge = set(rpa.rpa_plan_debug_dump(plan, "merge_rows").tolist())
    assert {0, 1, 2} <= merge                          # rows of the kv_len = 0 request
    noncausal = rpa.make_config(4, 2, 64, 64, 16, "f32", causal=False)
    with pytest.raises(rpa.RpaError):
        rpa.rpa_plan_create(noncausal, [0, 3], [-2], [0, 0], [0], 1)


def test_tree_mask_plan_validation(L):
    cfg = rpa.make_config(8, 2, 128, 128, 16, "bf16")
    qo, kv, pip, pix = [0, 4, 5], [40, 9], [0, 3, 4], [0, 1, 2, 3]
    tree = np.array([[1, 0, 0, 0], [1, 1, 0, 0], [1, 0, 1, 0], [1, 0, 1, 1]], dtype=bool)
    ti, tw = rpa.tree_mask_words([tree, None])
    assert ti.tolist() == [0, 4, 4] and tw.tolist() == [0b1, 0b11, 0b101, 0b1101]
    plan = rpa.rpa_plan_create_tree(cfg, qo, kv, pip, pix, 4, ti, tw)
    items = rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8)
    # the masked request's items reach its last key (the tree may see any draft token)
    assert items[items[:, 0] == 0][:, 5].max() == 40
    bad_diag = tw.copy()
    bad_diag[1] = 0b01
    expect(rpa.RPA_ERR_INVALID_ARG,
           lambda: rpa.rpa_plan_create_tree(cfg, qo, kv, pip, pix, 4, ti, bad_diag))
    past = tw.copy()
    past[0] |= 1 << 7
    expect(rpa.RPA_ERR_INVALID_ARG,
           lambda: rpa.rpa_plan_create_tree(cfg, qo, kv, pip, pix, 4, ti, past))
    expect(rpa.RPA_ERR_INVALID_ARG,
           lambda: rpa.rpa_plan_create_tree(cfg, qo, kv, pip, pix, 4, [0, 3, 3], tw[:3]))
    noncausal = rpa.make_config(8, 2, 128, 128, 16, "bf16", causal=False)
    expect(rpa.RPA_ERR_INVALID_ARG,
           lambda: rpa.rpa_plan_create_tree(noncausal, qo, kv, pip, pix, 4, ti, tw))
    big = np.tril(np.ones((65, 65), dtype=bool))
    ti2, tw2 = rpa.tree_mask_words([big])
    expect(rpa.RPA_ERR_UNSUPPORTED,
           lambda: rpa.rpa_plan_create_tree(cfg, [0, 65], [70], [0, 5], [0, 1, 2, 3, 4], 5,
                                            ti2, tw2))


def test_noalloc_attention_rejects_plans_beyond_the_static_scratch(L):
    """The allocation-free entry point checks the plan's workspace against the
    static scratch (128 MiB) before any device work."""
    cfg = rpa.make_config(8, 1, 128, 128, 16, "bf16")
    n = 32768
    plan = rpa.rpa_plan_create(cfg, [0, n], [n], [0, n // 16], np.arange(n // 16), n // 16)
    assert rpa.rpa_plan_workspace_size(plan) > (128 << 20)
    st = rpa.rpa_cache_strides(16 * 128, 16 * 128, 128)
    fake = 1 << 40  # never dereferenced: the size check fails first
    expect(rpa.RPA_ERR_WORKSPACE_TOO_SMALL, rpa.rpa_batch_attention_noalloc, plan, fake, fake,
           fake, st, st, fake, None, 0)
    assert "static scratch" in rpa.rpa_last_error_message()
    # argument checks come first, as in rpa_batch_attention
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_batch_attention_noalloc, plan, None, fake, fake, st,
           st, fake, None, 0)


def split_plan_for(meta, cfg, num_cus=0):
    return rpa.rpa_plan_create_split(cfg, meta.qo_indptr, meta.kv_len, meta.kv_page_indptr,
                                     meta.kv_page_indices, meta.num_pages, num_cus)


SPLIT_BATCHES = [
    # hq, hkv, d, P, qo lens, kv lens
    (32, 32, 128, 16, [1, 1, 512, 40], [3000, 17, 1536, 40]),
    (8, 1, 128, 16, [512], [8192]),
    (8, 1, 128, 16, [512, 4, 3], [2048, 700, 3]),
    (16, 2, 128, 64, [129, 0, 33], [1000, 64, 97]),
    (4, 2, 64, 16, [1, 16, 5], [37, 36, 5]),
    (32, 8, 128, 16, [4, 1, 4096], [9000, 1, 4096 + 700]),
]


@pytest.mark.parametrize("case", SPLIT_BATCHES, ids=[f"b{i}" for i in range(len(SPLIT_BATCHES))])
def test_split_plan_covers_cache_and_own_keys(L, case):
    """Split execution ("Chunked prefill", section "correctness"): the cache
    part covers each row's c_r cached keys once, the own part its new keys
    0 .. t once, their pieces share one block of partial rows (cache pieces
    first), and the merge reads exactly the pieces that hold a visible key."""
    hq, hkv, d, P, qo, kv = case
    dtype = "f32" if d == 64 else "bf16"
    cfg = rpa.make_config(hq, hkv, d, d, P, dtype, True, 1.0 / math.sqrt(d))
    meta = workloads.make_meta(qo, kv, P, 11 + sum(kv))
    plan = split_plan_for(meta, cfg)
    G = hq // hkv
    B = meta.batch_size
    batch = oracle.Batch(meta.qo_indptr, meta.kv_len, meta.kv_page_indptr, meta.kv_page_indices, P)
    parts = {"cache": rpa.rpa_plan_debug_dump(plan, "items").reshape(-1, 8),
             "own": rpa.rpa_plan_debug_dump(plan, "own:items").reshape(-1, 8)}
    sp_c = rpa.rpa_plan_debug_dump(plan, "splits").reshape(-1, 3)
    sp_o = rpa.rpa_plan_debug_dump(plan, "own:splits").reshape(-1, 3)
    assert len(rpa.rpa_plan_debug_dump(plan, "own:merge_rows")) == 0
    cover = {"cache": {}, "own": {}}
    pieces = {}  # (r, s) -> key range and part
    for part, items in parts.items():
        for r_, g, row0, row1, k0, k1, s, kc in items.tolist():
            n = batch.qo_len(r_)
            lim = int(meta.kv_len[r_]) - n if part == "cache" else n
            assert 0 <= k0 < k1 <= lim and 0 <= row0 < row1 <= n * G
            assert pieces.setdefault((r_, s), (part, k0, k1)) == (part, k0, k1)
            for row in range(row0, row1):
                cover[part].setdefault((r_, g, row), []).append((k0, k1))
    mrows = rpa.rpa_plan_debug_dump(plan, "merge_rows").tolist()
    minfo = rpa.rpa_plan_debug_dump(plan, "merge_info").reshape(-1, 4)
    info_of = {i: tuple(minfo[x].tolist()) for x, i in enumerate(mrows)}
    assert len(info_of) == len(mrows)
    app = rpa.rpa_plan_debug_dump(plan, "append").reshape(-1, 2)
    expected_rows = 0
    for r_ in range(B):
        n = batch.qo_len(r_)
        c = int(meta.kv_len[r_]) - n
        S = int(sp_c[r_][0])
        if n > 0:
            assert (sp_c[r_][0], sp_c[r_][2]) == (sp_o[r_][0], sp_o[r_][2])
        n_cache = len({s for (rr, s), v in pieces.items() if rr == r_ and v[0] == "cache"})
        n_own = len({s for (rr, s), v in pieces.items() if rr == r_ and v[0] == "own"})
        if n == 0:
            assert n_cache == n_own == 0
            continue
        assert n_cache == (0 if c == 0 else n_cache) and n_own >= 1
        assert S == max(1, n_cache + n_own)
        # cache pieces are 0 .. S_c - 1, own pieces follow
        for (rr, s), v in pieces.items():
            if rr == r_:
                assert (s < n_cache) == (v[0] == "cache")
        for g in range(hkv):
            for row in range(n * G):
                t = row // G
                cr = sorted(cover["cache"].get((r_, g, row), []))
                if c > 0:
                    assert cr[0][0] == 0 and cr[-1][1] == c and len(cr) == n_cache
                    assert all(a[1] == b[0] for a, b in zip(cr, cr[1:]))
                else:
                    assert not cr
                orng = sorted(cover["own"].get((r_, g, row), []))
                assert orng[0][0] == 0 and orng[-1][1] > t
                assert all(a[1] == b[0] for a, b in zip(orng, orng[1:]))
                live_own = sum(1 for (rr, s), v in pieces.items()
                               if rr == r_ and v[0] == "own" and v[1] <= t)
                assert len(orng) == live_own
                i = int(meta.qo_indptr[r_]) + t
                if S > 1:
                    assert info_of[i] == (int(sp_c[r_][2]) + t, n, n_cache + live_own, 0)
                else:
                    assert i not in info_of
        for t in range(n):
            assert tuple(app[int(meta.qo_indptr[r_]) + t]) == oracle.slot_of(batch, r_, c + t)
        if S > 1:
            expected_rows += S * n
    summary = rpa.rpa_plan_debug_dump(plan, "summary")
    assert summary[3] == expected_rows


def test_split_plan_validation(L):
    cfg = rpa.make_config(8, 2, 128, 128, 16, "bf16", True, 0.1)
    meta = workloads.make_meta([4, 1], [20, 9], 16, 3)
    plan = split_plan_for(meta, cfg)
    fused = plan_for(meta, cfg)
    st = rpa.rpa_cache_strides(2 * 16 * 128, 16 * 128, 128)
    fake = 1 << 40  # never dereferenced: validation fails first
    # each plan kind runs only through its own entry point
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_batch_attention, plan, fake, fake, fake, st, st, fake,
           None, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_batch_attention_noalloc, plan, fake, fake, fake, st,
           st, fake, None, 0)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_split_attention, fused, fake, fake, fake, fake, fake,
           st, st, fake, None, 0)
    expect(rpa.RPA_ERR_NOT_UPLOADED, rpa.rpa_split_attention, plan, fake, fake, fake, fake, fake,
           st, st, fake, None, 0)
    expect(rpa.RPA_ERR_NOT_UPLOADED, rpa.rpa_kv_append, plan, fake, fake, fake, fake, st, st, 0)
    # the whole step is checked as by rpa_plan_create
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_plan_create_split,
           rpa.make_config(8, 2, 128, 128, 16, "bf16", False, 0.1), meta.qo_indptr, meta.kv_len,
           meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)
    expect(rpa.RPA_ERR_UNSUPPORTED, rpa.rpa_plan_create_split,
           rpa.make_config(16, 1, 576, 512, 16, "bf16", True, 0.1), meta.qo_indptr, meta.kv_len,
           meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)
    expect(rpa.RPA_ERR_PAGE_OOB, rpa.rpa_plan_create_split, cfg, meta.qo_indptr, meta.kv_len,
           meta.kv_page_indptr, meta.kv_page_indices, 1)
    expect(rpa.RPA_ERR_INVALID_ARG, rpa.rpa_plan_create_split, cfg, [0, 4, 5], [3, 9],
           meta.kv_page_indptr, meta.kv_page_indices, meta.num_pages)
    with pytest.raises(rpa.RpaError):
        rpa.rpa_plan_debug_dump(fused, "own:items")
    # two requests may share a cached prefix page: only pages the append
    # writes must be unshared
    shared = split_plan_for(workloads.Meta(np.array([0, 2, 4], np.int32),
                                           np.array([18, 18], np.int32),
                                           np.array([0, 2, 4], np.int32),
                                           np.array([0, 1, 0, 2], np.int32), 3, 16), cfg)
    assert rpa.rpa_plan_workspace_size(shared) > 0
