"""Seeded synthetic inputs for ragged paged attention with KV append.

This module only draws inputs: request lengths, page tables, and random
Q / K / V / cache contents.  It holds none of the method's arithmetic (no
append, no attention, no merge), so both the HIP library's tests and the fp64
oracle can take their inputs from it.

Workloads (shapes follow the pages' regimes: decode qo_len = 1, prefill chunk
qo_len = C = 512, speculative verify qo_len = n + 1, MTP verify qo_len = 2):

  tiny_fp32          2 requests: decode (qo 1, kv 37) and a prefill chunk (qo 16 on
                     20 cached, kv 36); 4 q / 2 kv heads, d 64, P 16, fp32.
  mixed_7b           32 decodes with kv_len ~ U{512..4096} plus one C=512 chunk at
                     positions 1024..1535 (kv 1536); 32/32 heads, d 128, P 16, bf16.
  chunked_gqa        one 8192-token prompt, 8 q / 1 kv heads, d 128, P 16, bf16, run
                     as 16 chunks of 512 and one-shot.
  decode_verify_gqa  256 requests, kv_len lognormal (median 4096, sigma 1) clipped
                     to [1024, 32768]; even requests decode (qo 1), odd verify
                     (qo 4); 32/8 heads, d 128, P 16, bf16.
  mla_absorbed       64 requests, kv_len ~ U{4096..16384}, qo 2; 128 q heads over one
                     latent head (key 576, value = first 512 dims), P 64, bf16,
                     scale 1/sqrt(192).

Random values are N(0, 1) float32 draws, rounded to bfloat16 with
round-to-nearest-even where the dtype is bf16.  Cache pages that no request
references are filled with NaN, so a read of a wrong page shows up.  Physical
page ids are a seeded random permutation of the pool.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NAN_BF16_BITS = 0x7FC0


@dataclass
class Spec:
    name: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    dtype: str  # "bf16" or "f32"
    sm_scale: float
    seed: int
    shared_latent: bool = False
    causal: bool = True
    extra: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


SPECS = {
    "tiny_fp32": Spec("tiny_fp32", 4, 2, 64, 64, 16, "f32", 1.0 / math.sqrt(64), 1001),
    "mixed_7b": Spec("mixed_7b", 32, 32, 128, 128, 16, "bf16", 1.0 / math.sqrt(128), 1002),
    "chunked_gqa": Spec("chunked_gqa", 8, 1, 128, 128, 16, "bf16", 1.0 / math.sqrt(128), 1003,
                        extra={"prompt_len": 8192, "chunk": 512}),
    "decode_verify_gqa": Spec("decode_verify_gqa", 32, 8, 128, 128, 16, "bf16",
                              1.0 / math.sqrt(128), 1004),
    "mla_absorbed": Spec("mla_absorbed", 128, 1, 576, 512, 64, "bf16", 1.0 / math.sqrt(192),
                         1005, shared_latent=True),
}


def lengths(name: str, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(qo_len, kv_len) per request for a named workload, drawn from its seed."""
    spec = SPECS[name]
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    if name == "tiny_fp32":
        return np.array([1, 16]), np.array([37, 36])
    if name == "mixed_7b":
        kv = rng.integers(512, 4096, size=32, endpoint=True)
        return np.concatenate([np.ones(32, dtype=np.int64), [512]]), np.concatenate([kv, [1536]])
    if name == "chunked_gqa":
        L = spec.extra["prompt_len"]
        return np.array([L]), np.array([L])
    if name == "decode_verify_gqa":
        raw = rng.lognormal(mean=math.log(4096.0), sigma=1.0, size=256)
        kv = np.rint(np.clip(raw, 1024, 32768)).astype(np.int64)
        qo = np.where(np.arange(256) % 2 == 0, 1, 4)
        return qo.astype(np.int64), kv
    if name == "mla_absorbed":
        kv = rng.integers(4096, 16384, size=64, endpoint=True)
        return np.full(64, 2, dtype=np.int64), kv
    raise KeyError(name)


@dataclass
class Meta:
    """Batch metadata as host int32 arrays (CSR page table)."""
    qo_indptr: np.ndarray
    kv_len: np.ndarray
    kv_page_indptr: np.ndarray
    kv_page_indices: np.ndarray
    num_pages: int
    page_size: int

    @property
    def batch_size(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])


def make_meta(qo_lens, kv_lens, page_size: int, seed: int, extra_pages_per_req: int = 0,
              slack_frac: float = 0.05, min_slack: int = 2) -> Meta:
    """CSR page table over a seeded random permutation of a pool with slack.

    Request r gets ceil(kv_len / P) pages (plus ``extra_pages_per_req`` unused
    trailing entries, which the method must ignore).  The pool has 5% slack
    pages (at least two) that no request references.
    """
    qo = np.asarray(qo_lens, dtype=np.int64)
    kv = np.asarray(kv_lens, dtype=np.int64)
    need = (kv + page_size - 1) // page_size + extra_pages_per_req
    total = int(need.sum())
    num_pages = total + max(min_slack, int(math.ceil(slack_frac * total)))
    rng = np.random.default_rng(seed + 7919)
    perm = rng.permutation(num_pages)
    page_indptr = np.zeros(len(kv) + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(need)
    qo_indptr = np.zeros(len(qo) + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(qo)
    return Meta(qo_indptr.astype(np.int32), kv.astype(np.int32), page_indptr.astype(np.int32),
                perm[:total].astype(np.int32), int(num_pages), int(page_size))


def referenced_pages(meta: Meta) -> np.ndarray:
    """Boolean mask over the pool: True for pages some request lists."""
    used = np.zeros(meta.num_pages, dtype=bool)
    used[meta.kv_page_indices] = True
    return used


def _torch():
    import torch  # local import: the generator is usable without a GPU
    return torch


def _randn(shape, gen, device, dtype_name):
    torch = _torch()
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if dtype_name == "bf16":
        x = x.to(torch.bfloat16)
    return x


def make_tensors(spec: Spec, meta: Meta, seed: int, device="cpu", chunk_pages: int = 4096):
    """Random Q, new K/V and cache pools for a batch, as torch tensors on ``device``.

    Shapes: q [total_q, Hq, d_qk]; k_new [total_q, Hkv, d_qk]; v_new
    [total_q, Hkv, d_v] (None for a shared latent); k_pool / v_pool
    [num_pages, Hkv, P, d] (HND; v_pool None for a shared latent).  Pool pages
    no request references hold NaN.
    """
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    T = meta.total_q
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    q = _randn((T, spec.num_qo_heads, spec.head_dim_qk), gen, device, spec.dtype)
    k_new = _randn((T, spec.num_kv_heads, spec.head_dim_qk), gen, device, spec.dtype)
    v_new = None if spec.shared_latent else _randn((T, spec.num_kv_heads, spec.head_dim_v), gen,
                                                  device, spec.dtype)
    used = torch.from_numpy(referenced_pages(meta)).to(device)

    def pool(dim):
        p = torch.empty((meta.num_pages, spec.num_kv_heads, meta.page_size, dim), dtype=tdt,
                        device=device)
        for s in range(0, meta.num_pages, chunk_pages):
            e = min(meta.num_pages, s + chunk_pages)
            p[s:e] = _randn((e - s, spec.num_kv_heads, meta.page_size, dim), gen, device,
                            spec.dtype)
        p[~used] = float("nan")
        return p

    k_pool = pool(spec.head_dim_qk)
    v_pool = None if spec.shared_latent else pool(spec.head_dim_v)
    return {"q": q, "k_new": k_new, "v_new": v_new, "k_pool": k_pool, "v_pool": v_pool}


def make_prompt(spec: Spec, seed: int, device="cpu"):
    """Q, K, V of one whole prompt (chunked_gqa): [L, H, d] tensors."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    L = spec.extra["prompt_len"]
    q = _randn((L, spec.num_qo_heads, spec.head_dim_qk), gen, device, spec.dtype)
    k = _randn((L, spec.num_kv_heads, spec.head_dim_qk), gen, device, spec.dtype)
    v = _randn((L, spec.num_kv_heads, spec.head_dim_v), gen, device, spec.dtype)
    return q, k, v


def workload(name: str, device="cpu"):
    """Spec, metadata and tensors of a named workload (chunked_gqa: one-shot batch)."""
    spec = SPECS[name]
    qo, kv = lengths(name)
    meta = make_meta(qo, kv, spec.page_size, spec.seed)
    tensors = make_tensors(spec, meta, spec.seed, device=device)
    return spec, meta, tensors
