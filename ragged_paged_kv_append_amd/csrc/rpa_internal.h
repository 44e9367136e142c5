// Internal definitions shared by the host planner (plan.cpp), the C ABI
// (api.cpp) and the HIP kernels.  Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/rpa.h"

namespace rpa {

// Kernel classes a work item can be routed to.
enum KernelClass : int32_t {
  KC_GENERIC = 0,  // any dtype / head dim / page size; one wave per query row
  KC_DECODE = 1,   // bf16, d 128, P % 16 == 0, at most DEC_MAX_ROWS rows per KV head
  KC_PREFILL = 2,  // bf16, d 128, P % 16 == 0, many rows per KV head (prefill chunks)
  KC_MLA = 3,      // bf16, 576/512 shared latent, P % 16 == 0
  KC_COUNT = 4
};

// A work item: 8 int32 values.
//   request r, KV head g, rows [row0, row1) of that (r, g) group
//   (row = t * G + hh, i.e. token-major then query head within the group),
//   keys [k0, k1) of the request, split piece s, kernel class.
enum ItemField : int32_t {
  IT_REQ = 0, IT_KVHEAD, IT_ROW0, IT_ROW1, IT_K0, IT_K1, IT_SPLIT, IT_CLASS, IT_WORDS
};

// Per-request split record: 3 int32 values.
//   number of pieces S_r, keys per piece (pieces are [s*kc, (s+1)*kc) clipped
//   to kv_len; 0 when the pieces differ in length, whose bounds the items
//   carry), first partial row of the request (partial row of token t in
//   piece s is base + s * n_r + t).  S_r == 1 means items write the final
//   output directly and there is nothing to merge.
enum SplitField : int32_t { SP_COUNT = 0, SP_CHUNK, SP_BASE, SP_WORDS };

constexpr int GEN_ROWS = 4;        // rows per generic item (one wave each)
constexpr int DEC_MAX_ROWS = 16;   // rows per decode item (one MFMA column block)
constexpr int PRE_ROWS = 256;      // rows per prefill item
constexpr int PRE_MAX_KEYS = 4096; // keys per prefill item (64 tiles: one page-id register)
constexpr int MLA_MAX_KEYS = 32768; // keys per latent item (its page ids fit an LDS table)
constexpr int TREE_MAX_NEW = 64;   // new tokens of a request with a tree mask (one 64-bit row)
constexpr int MLA_ROWS = 128;      // rows per latent-attention item
constexpr int KEY_ALIGN = 64;      // split pieces start at multiples of this
constexpr int PRE_WGS_PER_CU = 1;  // prefill workgroups resident per compute unit
constexpr int MLA_WGS_PER_CU = 1;  // latent-attention workgroups resident per compute unit

// Device view of an uploaded plan, passed to kernels by value.
struct DevPlan {
  const int32_t* qo_indptr;     // [B+1]
  const int32_t* kv_len;        // [B]
  const int32_t* page_indptr;   // [B+1]
  const int32_t* page_indices;  // [nnz]
  const int32_t* split;         // [B][SP_WORDS]
  const int32_t* append;        // [total_q][2]: page id, slot
  const int32_t* items[KC_COUNT];
  // Tile classes (prefill, latent): workgroup b runs items
  // wg_indptr[b] .. wg_indptr[b + 1] - 1 of its class, in that order.
  const int32_t* wg_indptr[KC_COUNT];
  const int32_t* merge_rows;    // tokens whose request has S_r > 1 (or kv_len 0)
  // merge_info[4 x + 0..3] for merge row x: its first partial row, the
  // partial-row stride between pieces (qo_len of its request), and the number
  // of pieces that hold a key the row sees (0: an empty state).
  const int32_t* merge_info;
  // Tree masks (nullptr when the plan has none).  tree_req[r] = 1 if request
  // r has a mask; then tree_mask[2 i], tree_mask[2 i + 1] are the low and high
  // 32 bits of new token i's row: bit u = it sees new token u of its request.
  const int32_t* tree_req;
  const uint32_t* tree_mask;
  float* part_o;                // [partial rows][num_qo_heads][head_dim_v], float32
  float* part_lse;              // [partial rows][num_qo_heads]
  int32_t n_items[KC_COUNT];
  int32_t n_wgs[KC_COUNT];      // workgroups of each class's launch
  int32_t n_merge_rows;
  int32_t dec_stages;           // decode LDS ring depth (2 or 3) chosen by the planner
  int32_t batch_size;
  int32_t total_q;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t page_size;
  int32_t page_shift;
  int32_t causal;
  int32_t dtype;
  float sm_scale;
};

// Cache addressing (elements).
struct Strides {
  int64_t page, head, token;
};

}  // namespace rpa
