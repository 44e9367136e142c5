"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a private copy of the oracle's source (a
dropped term, a wrong sign or index, a swapped operand) and runs the pin tests
against that copy: at least one pin must fail.  The real oracle is untouched.
"""

import inspect
import sys
import types

import numpy as np
import pytest

import oracle.rpa_oracle as ro
from tests import test_oracle_pins as pins

MUTATIONS = {
    "gqa_mapping_modulo": ("h = g * group + hh", "h = hh * num_kv_heads + g"),
    "causal_top_left": ("visible = (j_idx <= c + t_idx)", "visible = (j_idx <= t_idx)"),
    "causal_off_by_one": ("visible = (j_idx <= c + t_idx)", "visible = (j_idx < c + t_idx)"),
    "scale_dropped": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "lse_drops_max": ("lse_h = mh + np.log(tot)", "lse_h = np.log(tot)"),
    "k_v_swapped": ("o[has] = w @ v", "o[has] = w @ k[:, :v.shape[1]]"),
    "merge_sign": ("eb = np.where(np.isfinite(lse_b), np.exp(lse_b - m_safe), 0.0)",
                   "eb = np.where(np.isfinite(lse_b), np.exp(m_safe - lse_b), 0.0)"),
    "merge_drops_b": ("o = wa[..., None] * o_a + wb[..., None] * o_b", "o = wa[..., None] * o_a"),
    "slot_modulo_page": ("return int(batch.pages(r)[pos // P]), pos % P",
                         "return int(batch.pages(r)[pos % len(batch.pages(r))]), pos % P"),
    "gather_wrong_page": ("pages = batch.pages(r)[j // P]", "pages = batch.pages(r)[j % P]"),
    "append_cached_offset": ("page, slot = slot_of(batch, r, c + t)",
                             "page, slot = slot_of(batch, r, t)"),
    "kv_len_excludes_new": ("return int(self.kv_len[r]) - self.qo_len(r)",
                            "return int(self.kv_len[r])"),
    "flops_drop_pv": ("2 * (head_dim_qk + head_dim_v)", "2 * head_dim_qk"),
    "pairs_off_by_one": ("pairs += sum(c + t + 1 for t in range(n))",
                         "pairs += sum(c + t for t in range(n))"),
    "io_drops_v": ("return chunk * 2 * n_layers", "return chunk * n_layers"),
    "split_cache_part_causal": ("head_dim_v=d_v, causal=False)", "head_dim_v=d_v, causal=True)"),
    "split_chunk_part_sees_all": ("visible = np.arange(n)[None, :] <= np.arange(n)[:, None]",
                                  "visible = np.ones((n, n), dtype=bool)"),
    "tree_mask_transposed": ("among_new = np.asarray(tree[r], dtype=bool)",
                             "among_new = np.asarray(tree[r], dtype=bool).T"),
    "tree_hides_cache": ("visible = np.concatenate([np.ones((n, c), dtype=bool), among_new], axis=1)",
                         "visible = np.concatenate([np.zeros((n, c), dtype=bool), among_new], axis=1)"),
    "copy_pages_wrong_head_offset": (
        "out[dp, dst_head0:dst_head0 + num_heads] = src[sp, src_head0:src_head0 + num_heads]",
        "out[dp, dst_head0:dst_head0 + num_heads] = src[sp, dst_head0:dst_head0 + num_heads]"),
    "nhd_wrong_axes": ("np.swapaxes(pages, 1, 2)", "np.swapaxes(pages, 2, 3)"),
    "bf16_truncates": ("rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)",
                       "rounded = u >> np.uint64(16)"),
}


def _mutant(old, new):
    src = inspect.getsource(ro)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    sys.modules["oracle_mutant"] = mod  # dataclasses look their module up here
    try:
        exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


def _pin_calls(golden):
    calls = []
    for case in pins.CASES[:3]:
        calls.append(lambda c=case: pins.test_p4_attend_matches_torch_sdpa(c, True))
    calls += [
        pins.test_bf16_conversions_match_torch,
        pins.test_p3_brute_force_tiny,
        pins.test_p5_single_key,
        pins.test_p5_zero_keys_give_mean_of_visible_values,
        pins.test_p5_equal_values_pass_through,
        pins.test_p5_two_keys_known_weights,
        pins.test_p5_decode_sees_all_keys_and_causal_row_sees_itself,
        pins.test_p2_merge_equals_union,
        pins.test_p6_page_permutation_and_page_size_invariance,
        pins.test_p6_gqa_equals_mha_with_copied_kv_heads,
        pins.test_p7_append_touches_exactly_the_target_slots,
        lambda: pins.test_p1_chunked_equals_one_shot(100, 16, 16, 4, 1, True),
        lambda: pins.test_p8_flop_identity(golden),
        pins.test_p8_accounting_counts_visible_pairs,
        lambda: pins.test_p9_io_worked_example(golden),
        pins.test_pt_tree_mask_matches_torch_sdpa,
        pins.test_pc_copy_pages_element_loop_and_untouched_bytes,
        pins.test_pc_half_shards_rebuild_full_pages_and_nhd_is_a_transpose,
        lambda: pins.test_p2s_split_execution_equals_attention_after_append(
            [1, 16, 0, 5], [37, 36, 4, 5], 4, 2, 16),
    ]
    return calls


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches_mutation(name, monkeypatch, golden_dir):
    mod = _mutant(*MUTATIONS[name])
    monkeypatch.setattr(pins, "oracle", mod)
    monkeypatch.setattr(pins, "Batch", mod.Batch)
    caught = []
    for call in _pin_calls(golden_dir):
        try:
            with np.errstate(all="ignore"):
                call()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(call)
            break
    assert caught, f"no pin caught mutation {name}"


def test_unmutated_copy_passes_every_pin(monkeypatch, golden_dir):
    mod = _mutant("import math", "import math")
    monkeypatch.setattr(pins, "oracle", mod)
    monkeypatch.setattr(pins, "Batch", mod.Batch)
    for call in _pin_calls(golden_dir):
        call()
