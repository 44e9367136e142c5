// Host-side plan object and planner entry point (pure C++, no HIP calls).
#pragma once

#include <memory>
#include <string>
#include <vector>

#include "rpa_internal.h"

struct rpa_plan {
  rpa_attn_config cfg{};
  int32_t batch_size = 0;
  int32_t total_q = 0;
  int32_t num_pages = 0;
  int32_t group = 1;
  bool can_append = true;  // false if a request has kv_len < qo_len

  // Metadata in the order it is laid out in the device workspace (int32 words).
  std::vector<int32_t> blob;
  int64_t off_qo_indptr = 0, off_kv_len = 0, off_page_indptr = 0, off_page_indices = 0;
  int64_t off_split = 0, off_append = 0, off_merge = 0, off_merge_info = 0;
  int64_t off_tree_mask = -1, off_tree_req = -1;  // -1: the plan has no tree masks
  int64_t off_items[rpa::KC_COUNT] = {0, 0, 0, 0};
  int32_t n_items[rpa::KC_COUNT] = {0, 0, 0, 0};
  int64_t off_wg[rpa::KC_COUNT] = {0, 0, 0, 0};   // wg_indptr tables (tile classes)
  int32_t n_wgs[rpa::KC_COUNT] = {0, 0, 0, 0};
  int32_t n_merge_rows = 0;
  int32_t dec_stages = 3;  // decode ring depth the plan's decode lists are sized for
  int64_t partial_rows = 0;

  // Workspace layout (bytes from the workspace base).
  size_t meta_bytes = 0;
  size_t part_o_off = 0;
  size_t part_lse_off = 0;
  size_t ws_bytes = 0;

  // Split execution ("Chunked prefill", section "correctness"): this plan is
  // the cache part (cross attention over the pages, kv_len = c_r, no causal
  // mask) and carries the merge of both parts; own_part is the causal
  // attention over the step's own rows, read token-major from its K/V
  // buffers.  Its metadata follows this plan's in the workspace, at byte
  // own_off; both parts write the same partial rows.  Null for other plans.
  std::unique_ptr<rpa_plan> own_part;
  size_t own_off = 0;

  // Upload state (set by rpa_plan_upload).
  void* d_ws = nullptr;
  void* staging = nullptr;   // pinned host buffer, meta_bytes long
  void* event = nullptr;     // hipEvent_t recorded after the upload copy
  bool uploaded = false;
};

namespace rpa {

// Validates cfg and batch and fills `plan` (metadata, offsets, sizes).
// On failure returns the status and sets *err.
// tree_indptr / tree_words: optional per-request visibility masks among the
// new tokens (both NULL for plain causal or non-causal attention).
rpa_status build_plan(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                      const int32_t* tree_indptr, const uint32_t* tree_words, int32_t num_cus,
                      rpa_plan* plan, std::string* err);

// Plans the split execution of one causal step (see own_part above).  The
// whole step is checked as by build_plan; the result is the cache part with
// its own_part set.
rpa_status build_split_plan(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                            int32_t num_cus, rpa_plan* plan, std::string* err);

}  // namespace rpa
