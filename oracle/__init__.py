"""Plain, slow fp64 CPU oracle for ragged paged attention with KV append.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code, tables or helpers with the HIP
library under ``ragged_paged_kv_append_amd``.

What it computes, and the passages it follows (sources are the web pages the
method is described on):

* page-table gather and the HND page layout -- "Disaggregated prefill and
  decode" (Perplexity), section on sharded KV transfers: a page keeps the head
  dimension ahead of the token dimension, so one head's slice of a page is one
  contiguous run;
* KV append -- same post, KV Messenger section: a layer appends its new KV
  entries to the cache, and they are valid after the append and before the
  attention that reads them;
* causal attention per request with qo_len new tokens over kv_len keys --
  same post, prefill/decode performance section (qo_len, kv_len), and the
  chunked-prefill post (k4i.top), section "correctness" (position i sees keys
  j <= i, scores q.K^T/sqrt(d_k), softmax, times V);
* softmax merge of two disjoint key partitions -- chunked-prefill post,
  section "correctness" (softmax_merge of the cache part and the chunk part),
  and the split execution built on it (the new tokens attend to the cache
  and, causally, to their own keys; the two states are merged);
* page copies: head ranges of pages between pools and transfer buffers --
  disaggregation post, sharded-transfer section (pages split and rebuilt by
  the shard ratio; HND keeps a head range contiguous), and the copy of a
  shared partly filled prefix block (chunked-prefill post, prefix cache);
* chunked driver over ceil(L/C) chunks -- chunked-prefill post, sections
  "core-idea" and "correctness";
* FLOP and IO accounting -- chunked-prefill post, sections "flops" and
  "io-overhead".

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
closed forms, invariants, a library routine and the pages' printed numbers.
"""

from .rpa_oracle import (  # noqa: F401
    Batch,
    bf16_bits_to_f64,
    f32_to_bf16_bits_rne,
    gather,
    slot_of,
    append,
    attend,
    attend_dense,
    merge,
    split_attention,
    chunked_prefill,
    one_shot_prefill,
    accounting,
    kv_write_bytes_per_chunk,
    copy_pages,
    hnd_to_nhd,
)
