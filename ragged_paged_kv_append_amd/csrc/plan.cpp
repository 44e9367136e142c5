// Host planner: validation, append map, split of long kv ranges into work
// items, merge map, workspace layout.  Pure C++ (no HIP), so it also builds
// and runs on a machine without a GPU.
//
// Follows "Accelerating Sonar through speculation" (Perplexity), runtime
// section: per step, the host packs the new tokens and page information and
// builds the attention metadata and intermediate buffers once for prefill,
// decode and verification; and "Disaggregated prefill and decode",
// performance section: attention parallelises over requests and over kv_len
// in proportion to the sequence lengths.

#include "plan.h"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <numeric>

namespace rpa {

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Resident decode waves per CU that a cut decode batch is planned for: the
// two-slot ring (16 KiB of LDS per wave) and ~150 VGPRs admit eight.
constexpr int64_t kDecodeWavesPerCu = 8;

int64_t wgs_per_cu(int32_t cls) {
  switch (cls) {
    case KC_PREFILL: return PRE_WGS_PER_CU;
    case KC_MLA: return MLA_WGS_PER_CU;
    default: return 1;
  }
}

int32_t rows_per_item(int32_t cls, int32_t rows_total) {
  switch (cls) {
    case KC_DECODE: return DEC_MAX_ROWS;
    case KC_PREFILL: return PRE_ROWS;
    case KC_MLA: return MLA_ROWS;
    default: return GEN_ROWS;
  }
  (void)rows_total;
}

// Latent packing with XCD pairs.  `items` are sorted by decreasing cost and
// `cost` holds the same costs in any order.  Items with the same request, KV
// head and key range form units of two; units go longest first to the pair of
// workgroups (b, b + 8) with the least work, one item to each.  Returns false
// (and changes nothing) when no unit has two items or the workgroup count is
// not a multiple of 16.
bool pack_latent_pairs(std::vector<int32_t>& items, const std::vector<int64_t>& cost,
                       int64_t max_wgs, std::vector<int32_t>* wg_indptr) {
  const int64_t m = (int64_t)cost.size();
  if (max_wgs < 16 || max_wgs % 16 != 0) return false;
  std::vector<int64_t> c(cost);
  std::sort(c.begin(), c.end(), std::greater<int64_t>());
  // units: consecutive pairing within each (request, head, k0, k1) group, in
  // decreasing cost order
  struct Unit {
    int64_t a, b;  // item indices (b < 0: single)
    int64_t cost;
  };
  std::vector<Unit> units;
  std::vector<int64_t> open;  // per group: index of the unit waiting for a partner
  std::vector<std::array<int32_t, 4>> keys;
  bool any_pair = false;
  for (int64_t j = 0; j < m; ++j) {
    const int32_t* it = &items[(size_t)j * IT_WORDS];
    const std::array<int32_t, 4> key = {it[IT_REQ], it[IT_KVHEAD], it[IT_K0], it[IT_K1]};
    size_t g = 0;
    while (g < keys.size() && keys[g] != key) ++g;
    if (g == keys.size()) {
      keys.push_back(key);
      open.push_back(-1);
    }
    if (open[g] >= 0) {
      units[(size_t)open[g]].b = j;
      open[g] = -1;
      any_pair = true;
    } else {
      open[g] = (int64_t)units.size();
      units.push_back({j, -1, c[(size_t)j]});
    }
  }
  if (!any_pair) return false;
  const int64_t npairs = std::min<int64_t>(max_wgs / 2, round_up((int64_t)units.size(), 8));
  const int64_t n_wgs = 2 * npairs;
  std::vector<int64_t> load((size_t)n_wgs, 0);
  std::vector<std::vector<int64_t>> lists((size_t)n_wgs);
  auto wg_of = [](int64_t pair, int side) { return 16 * (pair / 8) + pair % 8 + 8 * side; };
  std::vector<std::pair<int64_t, int64_t>> heap;  // (pair load, pair), min-heap
  for (int64_t q = 0; q < npairs; ++q) heap.push_back({0, q});
  auto greater = [](const std::pair<int64_t, int64_t>& x, const std::pair<int64_t, int64_t>& y) {
    return x > y;
  };
  std::make_heap(heap.begin(), heap.end(), greater);
  for (const Unit& u : units) {
    std::pop_heap(heap.begin(), heap.end(), greater);
    auto& top = heap.back();
    const int64_t w0 = wg_of(top.second, 0), w1 = wg_of(top.second, 1);
    if (u.b >= 0) {
      lists[(size_t)w0].push_back(u.a);
      lists[(size_t)w1].push_back(u.b);
      load[(size_t)w0] += c[(size_t)u.a];
      load[(size_t)w1] += c[(size_t)u.b];
    } else {
      const int64_t w = load[(size_t)w0] <= load[(size_t)w1] ? w0 : w1;
      lists[(size_t)w].push_back(u.a);
      load[(size_t)w] += c[(size_t)u.a];
    }
    top.first = std::max(load[(size_t)w0], load[(size_t)w1]);
    std::push_heap(heap.begin(), heap.end(), greater);
  }
  std::vector<int32_t> grouped;
  grouped.reserve(items.size());
  wg_indptr->assign(1, 0);
  for (int64_t b = 0; b < n_wgs; ++b) {
    for (int64_t j : lists[(size_t)b])
      grouped.insert(grouped.end(), items.begin() + j * IT_WORDS,
                     items.begin() + (j + 1) * IT_WORDS);
    wg_indptr->push_back((int32_t)(grouped.size() / IT_WORDS));
  }
  items.swap(grouped);
  return true;
}

// Plans one batch.  A part plan (one half of the split execution) skips two
// checks that belong to the whole step: the page-size bound (the step's own
// rows form one page per request, of 2^30 tokens) and the check of the pages
// the append writes (the whole step has been checked for those).
// prefill_cus (> 0) replaces num_cus for the prefill class only: the
// compute units that class's workgroups get in a launch shared with another
// plan's.
rpa_status build_plan_impl(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                           const int32_t* tree_indptr, const uint32_t* tree_words,
                           int32_t num_cus, bool part, int32_t prefill_cus, rpa_plan* plan,
                           std::string* err) {
  if (!cfg || !batch || !plan) {
    *err = "null cfg, batch or plan pointer";
    return RPA_ERR_INVALID_ARG;
  }
  const rpa_attn_config c = *cfg;
  if (c.num_qo_heads <= 0 || c.num_kv_heads <= 0 || c.num_qo_heads % c.num_kv_heads != 0) {
    *err = "num_qo_heads must be a positive multiple of num_kv_heads";
    return RPA_ERR_INVALID_ARG;
  }
  if (c.dtype != RPA_DTYPE_F32 && c.dtype != RPA_DTYPE_BF16) {
    *err = "dtype must be RPA_DTYPE_F32 or RPA_DTYPE_BF16";
    return RPA_ERR_INVALID_ARG;
  }
  if (c.causal != 0 && c.causal != 1) {
    *err = "causal must be 0 or 1";
    return RPA_ERR_INVALID_ARG;
  }
  // The kernels take a row's maximum score before scaling, which is the
  // maximum scaled score only for a positive scale.
  if (!std::isfinite(c.sm_scale) || !(c.sm_scale > 0.f)) {
    *err = "sm_scale must be finite and positive";
    return RPA_ERR_INVALID_ARG;
  }
  const bool dims_ok = (c.head_dim_qk == 64 && c.head_dim_v == 64) ||
                       (c.head_dim_qk == 128 && c.head_dim_v == 128) ||
                       (c.head_dim_qk == 576 && c.head_dim_v == 512);
  if (!dims_ok) {
    *err = "unsupported head dims (supported: 64/64, 128/128, 576/512)";
    return RPA_ERR_UNSUPPORTED;
  }
  if (c.head_dim_qk == 576 && c.num_kv_heads != 1) {
    *err = "the 576/512 latent form has exactly one KV head";
    return RPA_ERR_UNSUPPORTED;
  }
  if (!is_pow2(c.page_size) || (c.page_size > 256 && !part)) {
    *err = "page_size must be a power of two in [1, 256]";
    return RPA_ERR_UNSUPPORTED;
  }
  const int32_t B = batch->batch_size;
  if (B < 0) {
    *err = "batch_size must be >= 0";
    return RPA_ERR_INVALID_ARG;
  }
  if (B > 0 && (!batch->qo_indptr || !batch->kv_len || !batch->kv_page_indptr ||
                !batch->kv_page_indices)) {
    *err = "null batch array";
    return RPA_ERR_INVALID_ARG;
  }
  if (batch->num_pages < 0) {
    *err = "num_pages must be >= 0";
    return RPA_ERR_INVALID_ARG;
  }
  const int32_t P = c.page_size;
  const int32_t G = c.num_qo_heads / c.num_kv_heads;
  const int32_t* qo = batch->qo_indptr;
  const int32_t* kvl = batch->kv_len;
  const int32_t* pip = batch->kv_page_indptr;
  const int32_t* pix = batch->kv_page_indices;

  if (B > 0 && (qo[0] != 0 || pip[0] != 0)) {
    *err = "qo_indptr[0] and kv_page_indptr[0] must be 0";
    return RPA_ERR_INVALID_ARG;
  }
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    if (n < 0) {
      *err = "qo_indptr must be non-decreasing (request " + std::to_string(r) + ")";
      return RPA_ERR_INVALID_ARG;
    }
    if (kvl[r] < 0 || (c.causal && kvl[r] < n)) {
      *err = (kvl[r] < 0 ? "kv_len < 0" : "kv_len < qo_len with causal attention") +
             std::string(" for request ") + std::to_string(r);
      return RPA_ERR_INVALID_ARG;
    }
    if (pip[r + 1] < pip[r]) {
      *err = "kv_page_indptr must be non-decreasing (request " + std::to_string(r) + ")";
      return RPA_ERR_INVALID_ARG;
    }
    const int64_t need = ceil_div(kvl[r], P);
    if ((int64_t)pip[r + 1] - pip[r] < need) {
      *err = "request " + std::to_string(r) + " has fewer than ceil(kv_len/page_size) pages";
      return RPA_ERR_PAGE_OOB;
    }
    for (int64_t j = 0; j < need; ++j) {
      const int32_t pg = pix[pip[r] + j];
      if (pg < 0 || pg >= batch->num_pages) {
        *err = "page id " + std::to_string(pg) + " of request " + std::to_string(r) +
               " outside [0, num_pages)";
        return RPA_ERR_PAGE_OOB;
      }
    }
  }
  // Tree masks ("Accelerating Sonar through speculation", tree drafts: the
  // verification attends each draft token to its ancestors only).  Request r
  // has a mask iff tree_indptr[r + 1] > tree_indptr[r]; it then holds n_r rows
  // of ceil(n_r / 32) words, row t bit u set iff new token t sees new token u.
  const bool has_tree = tree_indptr != nullptr || tree_words != nullptr;
  std::vector<uint8_t> tree_req;
  if (has_tree) {
    if (!tree_indptr || (!tree_words && B > 0 && tree_indptr[B] > 0)) {
      *err = "tree masks need both tree_indptr and tree_words";
      return RPA_ERR_INVALID_ARG;
    }
    if (!c.causal) {
      *err = "tree masks refine causal attention (causal must be 1)";
      return RPA_ERR_INVALID_ARG;
    }
    if (B > 0 && tree_indptr[0] != 0) {
      *err = "tree_indptr[0] must be 0";
      return RPA_ERR_INVALID_ARG;
    }
    tree_req.assign((size_t)B, 0);
    for (int32_t r = 0; r < B; ++r) {
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      const int64_t words = (int64_t)tree_indptr[r + 1] - tree_indptr[r];
      if (words == 0) continue;
      const int64_t wpr = (n + 31) / 32;
      if (n > TREE_MAX_NEW) {
        *err = "request " + std::to_string(r) + " has a tree mask over more than " +
               std::to_string(TREE_MAX_NEW) + " new tokens";
        return RPA_ERR_UNSUPPORTED;
      }
      if (words != n * wpr) {
        *err = "tree mask of request " + std::to_string(r) + " must hold qo_len * ceil(qo_len/32) words";
        return RPA_ERR_INVALID_ARG;
      }
      for (int64_t t = 0; t < n; ++t) {
        const uint32_t* row = tree_words + tree_indptr[r] + t * wpr;
        if (!((row[t / 32] >> (t % 32)) & 1u)) {
          *err = "tree mask of request " + std::to_string(r) + ": token " + std::to_string(t) +
                 " must see itself";
          return RPA_ERR_INVALID_ARG;
        }
        for (int64_t u = n; u < wpr * 32; ++u)
          if ((row[u / 32] >> (u % 32)) & 1u) {
            *err = "tree mask of request " + std::to_string(r) + " has bits past qo_len";
            return RPA_ERR_INVALID_ARG;
          }
      }
      tree_req[(size_t)r] = 1;
    }
  }

  // A page the append writes must be referenced exactly once in the batch.
  if (B > 0 && !part) {
    std::vector<uint8_t> refs((size_t)batch->num_pages, 0);
    for (int32_t r = 0; r < B; ++r) {
      const int64_t need = ceil_div(kvl[r], P);
      for (int64_t j = 0; j < need; ++j) {
        uint8_t& x = refs[(size_t)pix[pip[r] + j]];
        if (x < 255) ++x;
      }
    }
    for (int32_t r = 0; r < B; ++r) {
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      if (n == 0 || kvl[r] < n) continue;  // nothing to append (cross attention)
      const int64_t cached = kvl[r] - n;
      for (int64_t j = cached / P; j <= (kvl[r] - 1) / P; ++j) {
        const int32_t pg = pix[pip[r] + j];
        if (refs[(size_t)pg] > 1) {
          *err = "page " + std::to_string(pg) + " written by request " + std::to_string(r) +
                 " is referenced more than once";
          return RPA_ERR_DUPLICATE_WRITE_PAGE;
        }
      }
    }
  }

  const int64_t total_q = B > 0 ? qo[B] : 0;
  const int64_t nnz = B > 0 ? pip[B] : 0;

  // ---- kernel class per request --------------------------------------------
  std::vector<int32_t> cls(B, KC_GENERIC);
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    int32_t k = KC_GENERIC;
    if (c.dtype == RPA_DTYPE_BF16 && P % 16 == 0) {
      if (c.head_dim_qk == 128 && c.head_dim_v == 128) {
        k = (n * G <= DEC_MAX_ROWS) ? KC_DECODE : KC_PREFILL;
      } else if (c.head_dim_qk == 576) {
        k = KC_MLA;
      }
    }
    if (k == KC_MLA && has_tree && tree_req[(size_t)r]) k = KC_GENERIC;
    cls[r] = k;
  }

  // ---- split of kv ranges into pieces ----------------------------------------
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  auto cus_of = [&](int k) -> int64_t {
    return (k == KC_PREFILL && prefill_cus > 0) ? prefill_cus : cus;
  };
  // Streaming classes (generic, decode): pieces sized so the whole batch makes
  // about 8 items per compute unit.  Tile classes (prefill, latent): pieces
  // sized so that one piece of a full row tile carries about the average load
  // of one resident workgroup; the items are then packed onto the resident
  // workgroups longest first (below).
  int64_t stream_work = 0;
  int64_t tile_work[KC_COUNT] = {0, 0, 0, 0};
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    if (n == 0) continue;
    const int64_t R = rows_per_item(cls[r], (int32_t)(n * G));
    if (cls[r] == KC_GENERIC || cls[r] == KC_DECODE) {
      stream_work += (int64_t)kvl[r] * c.num_kv_heads * ceil_div(n * G, R);
    } else {
      const int64_t cached = (int64_t)kvl[r] - n;
      for (int64_t row0 = 0; row0 < n * G; row0 += R) {
        const int64_t row1 = std::min(n * G, row0 + R);
        const int64_t visible = (c.causal && !(has_tree && tree_req[(size_t)r]))
                                    ? cached + (row1 - 1) / G + 1 : kvl[r];
        tile_work[cls[r]] += visible * round_up(row1 - row0, 32) * c.num_kv_heads;
      }
    }
  }
  const int64_t stream_piece =
      std::max<int64_t>(KEY_ALIGN, round_up(ceil_div(std::max<int64_t>(stream_work, 1), 8 * cus),
                                            KEY_ALIGN));
  int64_t tile_piece[KC_COUNT] = {0, 0, 0, 0};
  for (int k : {(int)KC_PREFILL, (int)KC_MLA}) {
    const int64_t slots = wgs_per_cu(k) * cus_of(k);
    tile_piece[k] = std::max<int64_t>(
        4 * KEY_ALIGN, round_up(ceil_div(std::max<int64_t>(tile_work[k], 1),
                                         slots * rows_per_item(k, 0)), KEY_ALIGN));
  }

  // Requests cut into equal runs of keys, one run per "bin" of workgroups
  // that run side by side: the requests, longest first, are laid end to end
  // and cut at multiples of KEY_ALIGN (no piece under kMinPiece keys unless
  // the request is shorter, none over max_piece; kMinPiece is 4 KEY_ALIGN for
  // latent pieces, each of which costs a 144 KiB Q load and a 256 KiB partial).  cut_k0[r] holds the first
  // key of each piece of a cut request and cut_bin[r] its bin.
  //   Latent requests of two row tiles (a query token pair over 128 heads):
  //   a bin is a pair of workgroups on one XCD.  Equal pieces packed longest
  //   first left the busiest pair with 40% more keys than the average.
  std::vector<std::vector<int64_t>> cut_k0((size_t)B), cut_bin((size_t)B);
  int64_t cut_bins[KC_COUNT] = {0, 0, 0, 0};
  auto cut_requests = [&](std::vector<int32_t> reqs, int64_t bins, int64_t max_piece,
                          int64_t kMinPiece) {
    int64_t total = 0;
    for (int32_t r : reqs) total += kvl[r];
    bins = std::min<int64_t>(bins, std::max<int64_t>(1, total / kMinPiece));
    const int64_t cap = round_up(ceil_div(total, bins), KEY_ALIGN);
    std::stable_sort(reqs.begin(), reqs.end(), [&](int32_t a, int32_t b) { return kvl[a] > kvl[b]; });
    int64_t bin = 0, room = cap;
    for (int32_t r : reqs) {
      const int64_t L = kvl[r];
      for (int64_t k0 = 0; k0 < L;) {
        // Pieces start at multiples of KEY_ALIGN: a bin takes whole KEY_ALIGN
        // runs of what it has left, or a request's whole rest.
        int64_t avail = std::max<int64_t>(room, 0) / KEY_ALIGN * KEY_ALIGN;
        // A run that would start a bin's list with a sliver goes to the next bin.
        if (avail < kMinPiece && avail < L - k0 && bin + 1 < bins) {
          ++bin;
          room = avail = cap;
        }
        const bool last_bin = bin + 1 == bins;
        int64_t take = last_bin ? L - k0 : std::min(L - k0, avail);
        if (L - (k0 + take) < kMinPiece) take = L - k0;  // no sliver at the end either
        take = std::min<int64_t>(take, max_piece);
        cut_k0[(size_t)r].push_back(k0);
        cut_bin[(size_t)r].push_back(bin);
        k0 += take;
        room -= take;
        if (room <= 0 && !last_bin) {
          ++bin;
          room = cap;
        }
      }
    }
    return bins;
  };
  {
    const int64_t max_wgs = wgs_per_cu(KC_MLA) * cus;
    bool ok = max_wgs >= 16 && max_wgs % 16 == 0 && c.num_kv_heads == 1;
    std::vector<int32_t> reqs;
    for (int32_t r = 0; r < B && ok; ++r) {
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      if (cls[r] != KC_MLA || n == 0 || kvl[r] == 0) continue;
      if (n * G <= MLA_ROWS || n * G > 2 * MLA_ROWS) ok = false;  // two row tiles each
      reqs.push_back(r);
    }
    if (ok && !reqs.empty())
      cut_bins[KC_MLA] = cut_requests(reqs, max_wgs / 2, MLA_MAX_KEYS, 4 * KEY_ALIGN);
  }
  // Decode batches whose items all hold a GQA group or verify rows (n G >= 4)
  // are cut the same way into one equal run per resident workgroup (eight
  // per CU with a two-slot ring), each workgroup running its bin's pieces for
  // one KV head in turn: 5% faster than one item per workgroup on the long
  // GQA verify batch, but 10% slower on single-row (MHA) decode batches,
  // which keep one item per workgroup.
  plan->dec_stages = 3;
  {
    std::vector<int32_t> reqs;
    bool ok = true;
    for (int32_t r = 0; r < B; ++r) {
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      if (cls[r] != KC_DECODE || n == 0 || kvl[r] == 0) continue;
      if (n * G < 4) ok = false;
      reqs.push_back(r);
    }
    if (ok && !reqs.empty()) {
      const int64_t bins = std::max<int64_t>(1, kDecodeWavesPerCu * cus / c.num_kv_heads);
      cut_bins[KC_DECODE] = cut_requests(reqs, bins, INT32_MAX / 2, KEY_ALIGN);
      plan->dec_stages = 2;
    }
  }

  std::vector<int32_t> split((size_t)B * SP_WORDS, 0);
  int64_t partial_rows = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    const int64_t L = kvl[r];
    int64_t S = 1, kc = std::max<int64_t>(L, 1);
    if (n > 0 && L > 0) {
      if (cls[r] == KC_GENERIC || cls[r] == KC_DECODE) {
        S = ceil_div(L, stream_piece);
      } else {
        S = ceil_div(L, tile_piece[cls[r]]);
        if (cls[r] == KC_PREFILL) S = std::max<int64_t>(S, ceil_div(L, PRE_MAX_KEYS));
        if (cls[r] == KC_MLA) S = std::max<int64_t>(S, ceil_div(L, MLA_MAX_KEYS));
      }
      S = std::max<int64_t>(S, 1);
      kc = round_up(ceil_div(L, S), KEY_ALIGN);
      S = ceil_div(L, kc);
      if (!cut_k0[(size_t)r].empty()) {
        S = (int64_t)cut_k0[(size_t)r].size();
        kc = 0;  // pieces of unequal length: cut_k0
      }
    }
    split[(size_t)r * SP_WORDS + SP_COUNT] = (int32_t)S;
    split[(size_t)r * SP_WORDS + SP_CHUNK] = (int32_t)kc;
    split[(size_t)r * SP_WORDS + SP_BASE] = (int32_t)(S > 1 ? partial_rows : -1);
    if (S > 1) partial_rows += S * n;
  }
  if (partial_rows > INT32_MAX / 2) {
    *err = "batch too large: partial rows overflow";
    return RPA_ERR_INVALID_ARG;
  }

  // ---- work items ----------------------------------------------------------------
  std::vector<std::vector<int32_t>> items(KC_COUNT);
  std::vector<std::vector<int64_t>> cost(KC_COUNT);
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    if (n == 0) continue;
    const int64_t L = kvl[r];
    const int64_t cached = L - n;
    const int32_t k = cls[r];
    const int64_t rows_total = n * G;
    const int64_t R = rows_per_item(k, (int32_t)rows_total);
    const int64_t S = split[(size_t)r * SP_WORDS + SP_COUNT];
    const int64_t kc = split[(size_t)r * SP_WORDS + SP_CHUNK];
    for (int32_t g = 0; g < c.num_kv_heads; ++g) {
      for (int64_t row0 = 0; row0 < rows_total; row0 += R) {
        const int64_t row1 = std::min(rows_total, row0 + R);
        const int64_t t_last = (row1 - 1) / G;
        const bool masked = has_tree && tree_req[(size_t)r];
        const int64_t p_last = (c.causal && !masked) ? cached + t_last : L - 1;
        const std::vector<int64_t>& cuts = cut_k0[(size_t)r];
        for (int64_t s = 0; s < S; ++s) {
          const int64_t k0 = kc > 0 ? s * kc : cuts[(size_t)s];
          if (k0 > p_last) break;
          const int64_t k1 =
              kc > 0 ? std::min(L, k0 + kc) : (s + 1 < S ? cuts[(size_t)s + 1] : L);
          const int32_t it[IT_WORDS] = {r, g, (int32_t)row0, (int32_t)row1, (int32_t)k0,
                                        (int32_t)k1, (int32_t)s, k};
          items[k].insert(items[k].end(), it, it + IT_WORDS);
          const int64_t rows_cost = (k == KC_PREFILL || k == KC_MLA) ? round_up(row1 - row0, 32)
                                                                      : row1 - row0;
          // A prefill item also costs a fixed start and finish (its Q and
          // first tiles, its stores), about what 256 keys take: without it
          // the packing put short items on workgroups that were already
          // among the busiest (one-shot prompt: 154 -> 150 us).
          const int64_t fixed = k == KC_PREFILL ? 256 : 0;
          cost[k].push_back((std::min(k1, p_last + 1) - k0 + fixed) * rows_cost);
        }
      }
    }
  }
  // Heaviest items first, so the tail of the launch holds the short ones.
  for (int k = 0; k < KC_COUNT; ++k) {
    const size_t m = cost[k].size();
    std::vector<size_t> order(m);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](size_t a, size_t b) { return cost[k][a] > cost[k][b]; });
    std::vector<int32_t> sorted(items[k].size());
    for (size_t j = 0; j < m; ++j)
      std::memcpy(&sorted[j * IT_WORDS], &items[k][order[j] * IT_WORDS], IT_WORDS * sizeof(int32_t));
    items[k].swap(sorted);
  }

  // Tile classes: pack the items onto the resident workgroups, longest first,
  // each to the workgroup with the least work so far.  Items are then stored
  // grouped by workgroup; wg_indptr delimits each workgroup's list.
  //
  // Latent items that read the same key range (the row tiles of one request:
  // its query tokens all read the one latent head) are packed as a pair onto
  // workgroups b and b + 8.  Workgroups are dealt to the eight XCDs round
  // robin, so both run on one XCD, start together and stream the same latent
  // tiles in step: the second read of each tile is served by that XCD's L2.
  std::vector<std::vector<int32_t>> wg_indptr(KC_COUNT);
  for (int k : {(int)KC_PREFILL, (int)KC_MLA}) {
    const int64_t m = (int64_t)cost[k].size();
    if (m == 0) continue;
    if (k == KC_MLA && cut_bins[KC_MLA] > 0) {
      // Cut latent requests: each piece's two row tiles go to its pair's
      // workgroups b and b + 8 (one XCD); a pair runs its pieces in turn.
      const int64_t n_wgs = 16 * ceil_div(cut_bins[KC_MLA], 8);
      std::vector<std::vector<int64_t>> lists((size_t)n_wgs);
      for (int64_t j = 0; j < m; ++j) {
        const int32_t* it = &items[k][(size_t)j * IT_WORDS];
        const int64_t pr = cut_bin[(size_t)it[IT_REQ]][(size_t)it[IT_SPLIT]];
        const int64_t side = it[IT_ROW0] / MLA_ROWS;
        lists[(size_t)(16 * (pr / 8) + pr % 8 + 8 * side)].push_back(j);
      }
      std::vector<int32_t> grouped;
      grouped.reserve(items[k].size());
      wg_indptr[k].push_back(0);
      for (int64_t w = 0; w < n_wgs; ++w) {
        for (int64_t j : lists[(size_t)w])
          grouped.insert(grouped.end(), items[k].begin() + j * IT_WORDS,
                         items[k].begin() + (j + 1) * IT_WORDS);
        wg_indptr[k].push_back((int32_t)(grouped.size() / IT_WORDS));
      }
      items[k].swap(grouped);
      continue;
    }
    if (k == KC_MLA && pack_latent_pairs(items[k], cost[k], wgs_per_cu(k) * cus, &wg_indptr[k]))
      continue;
    const int64_t slots = std::min<int64_t>(m, wgs_per_cu(k) * cus_of(k));
    std::vector<int64_t> load(slots, 0);
    std::vector<std::vector<int64_t>> lists(slots);
    // costs are already sorted in decreasing order
    std::vector<std::pair<int64_t, int64_t>> heap;  // (load, slot), min-heap
    heap.reserve(slots);
    for (int64_t b = 0; b < slots; ++b) heap.push_back({0, b});
    auto greater = [](const std::pair<int64_t, int64_t>& a, const std::pair<int64_t, int64_t>& b) {
      return a > b;
    };
    std::make_heap(heap.begin(), heap.end(), greater);
    std::vector<int64_t> sorted_cost(cost[k].begin(), cost[k].end());
    std::sort(sorted_cost.begin(), sorted_cost.end(), std::greater<int64_t>());
    for (int64_t j = 0; j < m; ++j) {
      std::pop_heap(heap.begin(), heap.end(), greater);
      auto& top = heap.back();
      lists[top.second].push_back(j);
      top.first += sorted_cost[j];
      std::push_heap(heap.begin(), heap.end(), greater);
    }
    // Workgroup w runs on XCD w % 8.  Lists are handed to the workgroups of
    // XCD 0 first, then XCD 1, ..., in the order of the request, KV head, key
    // range and row tile of their first (longest) item: the row tiles that
    // read one key range, and the pieces of one KV head, then share an XCD, so
    // the K/V tiles (and Q rows) they have in common come from HBM once and
    // from that XCD's L2 after.
    std::vector<int64_t> by_key((size_t)slots);
    for (int64_t b = 0; b < slots; ++b) by_key[(size_t)b] = b;
    auto key_of = [&](int64_t b) {
      const int32_t* it = &items[k][(size_t)lists[(size_t)b][0] * IT_WORDS];
      return std::array<int32_t, 4>{it[IT_REQ], it[IT_KVHEAD], it[IT_K0], it[IT_ROW0]};
    };
    std::stable_sort(by_key.begin(), by_key.end(),
                     [&](int64_t a, int64_t b) { return key_of(a) < key_of(b); });
    std::vector<int64_t> list_of_wg((size_t)slots);
    {
      int64_t i = 0;
      for (int64_t x = 0; x < 8; ++x)
        for (int64_t w = x; w < slots; w += 8) list_of_wg[(size_t)w] = by_key[(size_t)i++];
    }
    std::vector<int32_t> grouped;
    grouped.reserve(items[k].size());
    wg_indptr[k].push_back(0);
    for (int64_t w = 0; w < slots; ++w) {
      for (int64_t j : lists[(size_t)list_of_wg[(size_t)w]])
        grouped.insert(grouped.end(), items[k].begin() + j * IT_WORDS,
                       items[k].begin() + (j + 1) * IT_WORDS);
      wg_indptr[k].push_back((int32_t)(grouped.size() / IT_WORDS));
    }
    items[k].swap(grouped);
  }

  // Decode: cut batches run workgroup bin * H_kv + g over the pieces of its
  // bin for KV head g; others one item per workgroup, in the heaviest-first
  // order above, so the dispatcher hands each freed slot the next item.
  if (cut_bins[KC_DECODE] > 0 && !items[KC_DECODE].empty()) {
    const int64_t H = c.num_kv_heads;
    const int64_t n_wgs = cut_bins[KC_DECODE] * H;
    const int64_t m = (int64_t)items[KC_DECODE].size() / IT_WORDS;
    std::vector<std::vector<int64_t>> lists((size_t)n_wgs);
    for (int64_t j = 0; j < m; ++j) {
      const int32_t* it = &items[KC_DECODE][(size_t)j * IT_WORDS];
      const int64_t bin = cut_bin[(size_t)it[IT_REQ]][(size_t)it[IT_SPLIT]];
      lists[(size_t)(bin * H + it[IT_KVHEAD])].push_back(j);
    }
    std::vector<int32_t> grouped;
    grouped.reserve(items[KC_DECODE].size());
    wg_indptr[KC_DECODE].push_back(0);
    for (int64_t w = 0; w < n_wgs; ++w) {
      for (int64_t j : lists[(size_t)w])
        grouped.insert(grouped.end(), items[KC_DECODE].begin() + j * IT_WORDS,
                       items[KC_DECODE].begin() + (j + 1) * IT_WORDS);
      wg_indptr[KC_DECODE].push_back((int32_t)(grouped.size() / IT_WORDS));
    }
    items[KC_DECODE].swap(grouped);
  } else if (!items[KC_DECODE].empty()) {
    const int32_t m = (int32_t)(items[KC_DECODE].size() / IT_WORDS);
    for (int32_t j = 0; j <= m; ++j) wg_indptr[KC_DECODE].push_back(j);
  }

  // ---- append map and merge rows --------------------------------------------------
  // A request with kv_len < qo_len (allowed without causal masking: the new
  // tokens attend to cached keys only) has no append slots, so such a plan
  // cannot append.  Its rows with kv_len = 0 have no work item; the merge
  // pass writes them as empty states (O = 0, lse = -inf).
  std::vector<int32_t> append((size_t)total_q * 2, -1);
  std::vector<int32_t> merge_rows, merge_info;
  plan->can_append = true;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    const int64_t cached = (int64_t)kvl[r] - n;
    if (cached < 0) plan->can_append = false;
    for (int64_t t = 0; t < n; ++t) {
      const int64_t p = cached + t;
      const int64_t i = qo[r] + t;
      if (p >= 0) {
        append[(size_t)i * 2 + 0] = pix[pip[r] + p / P];
        append[(size_t)i * 2 + 1] = (int32_t)(p % P);
      }
      const int32_t S = split[(size_t)r * SP_WORDS + SP_COUNT];
      if (S > 1 || kvl[r] == 0) {
        // Piece s holds keys [s chunk, (s + 1) chunk) (or from cut_k0[s] for a
        // cut request); the row sees keys up to pmax, so pieces that start
        // past pmax hold nothing for it.
        const bool masked = c.causal && !(has_tree && tree_req[(size_t)r]);
        const int64_t pmax = masked ? p : (int64_t)kvl[r] - 1;
        const int64_t chunk = split[(size_t)r * SP_WORDS + SP_CHUNK];
        int64_t s_eff = 0;
        if (pmax >= 0 && chunk > 0) {
          s_eff = std::min<int64_t>(S, pmax / chunk + 1);
        } else if (pmax >= 0) {
          for (int64_t k0c : cut_k0[(size_t)r]) s_eff += k0c <= pmax ? 1 : 0;
        }
        merge_rows.push_back((int32_t)i);
        merge_info.push_back(split[(size_t)r * SP_WORDS + SP_BASE] + (int32_t)t);
        merge_info.push_back((int32_t)n);
        merge_info.push_back((int32_t)s_eff);
        merge_info.push_back(0);
      }
    }
  }

  // ---- blob -------------------------------------------------------------------------
  plan->cfg = c;
  plan->batch_size = B;
  plan->total_q = (int32_t)total_q;
  plan->num_pages = batch->num_pages;
  plan->group = G;
  std::vector<int32_t>& blob = plan->blob;
  blob.clear();
  auto push = [&](const int32_t* p, int64_t count) {
    const int64_t off = (int64_t)blob.size();
    if (count > 0) blob.insert(blob.end(), p, p + count);
    // keep every table 16-byte aligned
    while (blob.size() % 4) blob.push_back(0);
    return off;
  };
  const int32_t zero = 0;
  plan->off_qo_indptr = B > 0 ? push(qo, B + 1) : push(&zero, 1);
  plan->off_kv_len = push(kvl, B);
  plan->off_page_indptr = B > 0 ? push(pip, B + 1) : push(&zero, 1);
  plan->off_page_indices = push(pix, nnz);
  plan->off_split = push(split.data(), (int64_t)split.size());
  plan->off_append = push(append.data(), (int64_t)append.size());
  for (int k = 0; k < KC_COUNT; ++k) {
    plan->off_items[k] = push(items[k].data(), (int64_t)items[k].size());
    plan->n_items[k] = (int32_t)(items[k].size() / IT_WORDS);
    plan->off_wg[k] = push(wg_indptr[k].data(), (int64_t)wg_indptr[k].size());
    plan->n_wgs[k] = wg_indptr[k].empty() ? plan->n_items[k] : (int32_t)wg_indptr[k].size() - 1;
  }
  plan->off_merge = push(merge_rows.data(), (int64_t)merge_rows.size());
  plan->off_merge_info = push(merge_info.data(), (int64_t)merge_info.size());
  plan->off_tree_mask = plan->off_tree_req = -1;
  if (has_tree) {
    std::vector<int32_t> treq(tree_req.begin(), tree_req.end());
    std::vector<int32_t> tmask((size_t)total_q * 2, 0);
    for (int32_t r = 0; r < B; ++r) {
      if (!tree_req[(size_t)r]) continue;
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      const int64_t wpr = (n + 31) / 32;
      for (int64_t t = 0; t < n; ++t) {
        const uint32_t* row = tree_words + tree_indptr[r] + t * wpr;
        tmask[(size_t)(qo[r] + t) * 2 + 0] = (int32_t)row[0];
        tmask[(size_t)(qo[r] + t) * 2 + 1] = wpr > 1 ? (int32_t)row[1] : 0;
      }
    }
    plan->off_tree_req = push(treq.data(), (int64_t)treq.size());
    plan->off_tree_mask = push(tmask.data(), (int64_t)tmask.size());
  }
  plan->n_merge_rows = (int32_t)merge_rows.size();
  plan->partial_rows = partial_rows;

  plan->meta_bytes = (size_t)round_up((int64_t)blob.size() * 4, 256);
  plan->part_o_off = plan->meta_bytes;
  plan->part_lse_off =
      plan->part_o_off + (size_t)round_up(partial_rows * c.num_qo_heads * c.head_dim_v * 4, 256);
  plan->ws_bytes = plan->part_lse_off + (size_t)round_up(partial_rows * c.num_qo_heads * 4, 256);
  return RPA_OK;
}

// Appends a table to a plan blob, 16-byte aligned; returns its word offset.
int64_t push_table(std::vector<int32_t>& blob, const std::vector<int32_t>& t) {
  const int64_t off = (int64_t)blob.size();
  blob.insert(blob.end(), t.begin(), t.end());
  while (blob.size() % 4) blob.push_back(0);
  return off;
}

// Work of the busiest prefill workgroup of a plan: per item its (row,
// visible key) pairs, rows rounded up to the 32-row blocks the kernel
// computes, plus a fixed cost of 256 keys per item.
int64_t prefill_busiest(const rpa_plan& pl, bool causal) {
  if (pl.n_items[KC_PREFILL] == 0) return 0;
  const int32_t* blob = pl.blob.data();
  const int32_t* items = blob + pl.off_items[KC_PREFILL];
  const int32_t* wg = blob + pl.off_wg[KC_PREFILL];
  const int32_t* qo = blob + pl.off_qo_indptr;
  const int32_t* kvl = blob + pl.off_kv_len;
  int64_t worst = 0;
  for (int32_t b = 0; b < pl.n_wgs[KC_PREFILL]; ++b) {
    int64_t load = 0;
    for (int32_t j = wg[b]; j < wg[b + 1]; ++j) {
      const int32_t* it = items + (int64_t)j * IT_WORDS;
      const int32_t r = it[IT_REQ];
      const int64_t cached = (int64_t)kvl[r] - (qo[r + 1] - qo[r]);
      const int64_t kend = causal ? std::min<int64_t>(it[IT_K1], cached + (it[IT_ROW1] - 1) / pl.group + 1)
                                  : it[IT_K1];
      load += (std::max<int64_t>(kend - it[IT_K0], 0) + 256) * round_up(it[IT_ROW1] - it[IT_ROW0], 32);
    }
    worst = std::max(worst, load);
  }
  return worst;
}

}  // namespace

rpa_status build_plan(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                      const int32_t* tree_indptr, const uint32_t* tree_words, int32_t num_cus,
                      rpa_plan* plan, std::string* err) {
  return build_plan_impl(cfg, batch, tree_indptr, tree_words, num_cus, false, 0, plan, err);
}

rpa_status build_split_plan(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                            int32_t num_cus, rpa_plan* plan, std::string* err) {
  // The whole step, planned as one batch: every check of lengths and pages,
  // and the append map, which the split plan keeps.
  rpa_plan whole;
  rpa_status s = build_plan(cfg, batch, nullptr, nullptr, num_cus, &whole, err);
  if (s != RPA_OK) return s;
  const rpa_attn_config c = *cfg;
  if (!c.causal) {
    *err = "split execution is defined for causal attention (causal must be 1)";
    return RPA_ERR_INVALID_ARG;
  }
  if (c.head_dim_qk == 576) {
    *err = "split execution of the shared latent form is not supported";
    return RPA_ERR_UNSUPPORTED;
  }
  const int32_t B = batch->batch_size;
  const int32_t* qo = batch->qo_indptr;
  const int64_t total_q = B > 0 ? qo[B] : 0;

  // Cache part: every new token sees all c_r cached keys of its request.
  std::vector<int32_t> cached((size_t)B), own_len((size_t)B), own_indptr((size_t)B + 1, 0),
      own_pages;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t n = qo[r + 1] - qo[r];
    cached[(size_t)r] = batch->kv_len[r] - n;
    own_len[(size_t)r] = n;
    // Own part: the request's n_r new rows, token-major from row qo[r] of
    // the step's K/V buffers, as one page whose id is that row.
    if (n > 0) own_pages.push_back(qo[r]);
    own_indptr[(size_t)r + 1] = (int32_t)own_pages.size();
  }
  if (own_pages.empty()) own_pages.push_back(0);
  // The prefill-class items of both parts run in one launch, so the compute
  // units are shared between them, each part's prefill items balanced over
  // its share.  The other classes run part after part, each over every
  // compute unit.  The share starts from the parts' (row, visible key) pairs;
  // a few larger own shares are planned too and the one whose busiest
  // workgroup has the least work is kept: an item's fixed cost (its Q load,
  // first tiles and output stores take about as long as four 64-key steps)
  // weighs most on the own part, whose items are short.
  double w_cache = 0.0, w_own = 0.0;
  const int32_t G = c.num_qo_heads / c.num_kv_heads;
  for (int32_t r = 0; r < B; ++r) {
    const double n = (double)own_len[(size_t)r];
    if (n * G <= DEC_MAX_ROWS) continue;
    w_cache += n * (double)cached[(size_t)r];
    w_own += n * (n + 1.0) / 2.0;
  }
  const int32_t cus = num_cus > 0 ? num_cus : 256;
  rpa_attn_config cc = c;
  cc.causal = 0;
  const rpa_batch_desc cb{B, qo, cached.data(), batch->kv_page_indptr, batch->kv_page_indices,
                          batch->num_pages};
  rpa_attn_config oc = c;
  oc.page_size = 1 << 30;
  const rpa_batch_desc ob{B, qo, own_len.data(), own_indptr.data(), own_pages.data(),
                          (int32_t)std::max<int64_t>(total_q, 1)};
  std::unique_ptr<rpa_plan> own(new rpa_plan());
  if (w_cache > 0.0 && w_own > 0.0 && cus > 1) {
    const int32_t c0 = std::min(cus - 1, std::max<int32_t>(
        1, (int32_t)std::lround((double)cus * w_own / (w_own + w_cache))));
    int64_t best = -1;
    int32_t best_own = c0;
    for (const double f : {1.0, 1.5, 2.0, 3.0}) {
      const int32_t co = std::min(cus - 1, std::max<int32_t>(1, (int32_t)std::lround(c0 * f)));
      if (f > 1.0 && co == best_own) continue;
      rpa_plan pc, po;
      s = build_plan_impl(&cc, &cb, nullptr, nullptr, cus, true, cus - co, &pc, err);
      if (s != RPA_OK) return s;
      s = build_plan_impl(&oc, &ob, nullptr, nullptr, cus, true, co, &po, err);
      if (s != RPA_OK) return s;
      const int64_t span = std::max(prefill_busiest(pc, false), prefill_busiest(po, true));
      if (best < 0 || span < best) {
        best = span;
        best_own = co;
      }
    }
    s = build_plan_impl(&cc, &cb, nullptr, nullptr, cus, true, cus - best_own, plan, err);
    if (s != RPA_OK) return s;
    s = build_plan_impl(&oc, &ob, nullptr, nullptr, cus, true, best_own, own.get(), err);
  } else {
    s = build_plan_impl(&cc, &cb, nullptr, nullptr, cus, true, cus, plan, err);
    if (s != RPA_OK) return s;
    s = build_plan_impl(&oc, &ob, nullptr, nullptr, cus, true, cus, own.get(), err);
  }
  if (s != RPA_OK) return s;

  // Pieces of request r: the cache part's S_c pieces (keys 0 .. c_r - 1),
  // then the own part's S_o pieces (the new keys), numbered after them, all
  // in one block of partial rows.  A row sees every cache piece and a prefix
  // of the own pieces, so its live pieces are again a prefix.
  int32_t* csplit = plan->blob.data() + plan->off_split;
  int32_t* osplit = own->blob.data() + own->off_split;
  std::vector<int32_t> own_live((size_t)total_q, 1);
  for (int32_t x = 0; x < own->n_merge_rows; ++x) {
    const int32_t i = own->blob[(size_t)(own->off_merge + x)];
    own_live[(size_t)i] = own->blob[(size_t)(own->off_merge_info + 4 * x + 2)];
  }
  std::vector<int32_t> shift((size_t)B, 0), merge_rows, merge_info;
  int64_t partial_rows = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t n = qo[r + 1] - qo[r];
    int32_t* cs = csplit + (size_t)r * SP_WORDS;
    int32_t* os = osplit + (size_t)r * SP_WORDS;
    const int32_t sc = (n > 0 && cached[(size_t)r] > 0) ? cs[SP_COUNT] : 0;
    const int32_t so = n > 0 ? os[SP_COUNT] : 0;
    if (sc + so <= 1) {
      // nothing to merge: the own part (if any) writes the output
      cs[SP_COUNT] = os[SP_COUNT] = 1;
      cs[SP_BASE] = os[SP_BASE] = -1;
      continue;
    }
    const int64_t base = partial_rows;
    partial_rows += (int64_t)(sc + so) * n;
    for (int32_t* x : {cs, os}) {
      x[SP_COUNT] = sc + so;
      x[SP_CHUNK] = 0;
      x[SP_BASE] = (int32_t)base;
    }
    shift[(size_t)r] = sc;
    for (int32_t t = 0; t < n; ++t) {
      const int32_t i = qo[r] + t;
      merge_rows.push_back(i);
      merge_info.push_back((int32_t)base + t);
      merge_info.push_back(n);
      merge_info.push_back(sc + (so > 1 ? own_live[(size_t)i] : 1));
      merge_info.push_back(0);
    }
  }
  if (partial_rows > INT32_MAX / 2) {
    *err = "batch too large: partial rows overflow";
    return RPA_ERR_INVALID_ARG;
  }
  for (int k = 0; k < KC_COUNT; ++k) {
    int32_t* it = own->blob.data() + own->off_items[k];
    for (int32_t j = 0; j < own->n_items[k]; ++j, it += IT_WORDS) it[IT_SPLIT] += shift[(size_t)it[IT_REQ]];
  }
  // The cache part's plan carries the merge of both parts and the whole
  // step's append map; the own part merges nothing.
  std::copy(whole.blob.begin() + whole.off_append,
            whole.blob.begin() + whole.off_append + total_q * 2,
            plan->blob.begin() + plan->off_append);
  plan->can_append = whole.can_append;
  plan->blob.resize((size_t)plan->off_merge);
  plan->off_merge = push_table(plan->blob, merge_rows);
  plan->off_merge_info = push_table(plan->blob, merge_info);
  plan->n_merge_rows = (int32_t)merge_rows.size();
  own->blob.resize((size_t)own->off_merge);
  own->off_merge = own->off_merge_info = (int64_t)own->blob.size();
  own->n_merge_rows = 0;

  // Workspace: the cache part's metadata, the own part's, then the shared
  // partial rows.
  const int64_t c_words = round_up((int64_t)plan->blob.size(), 64);
  plan->blob.resize((size_t)c_words, 0);
  plan->own_off = (size_t)c_words * 4;
  plan->blob.insert(plan->blob.end(), own->blob.begin(), own->blob.end());
  plan->meta_bytes = (size_t)round_up((int64_t)plan->blob.size() * 4, 256);
  plan->partial_rows = own->partial_rows = partial_rows;
  plan->part_o_off = plan->meta_bytes;
  plan->part_lse_off =
      plan->part_o_off + (size_t)round_up(partial_rows * c.num_qo_heads * c.head_dim_v * 4, 256);
  plan->ws_bytes = plan->part_lse_off + (size_t)round_up(partial_rows * c.num_qo_heads * 4, 256);
  own->part_o_off = plan->part_o_off - plan->own_off;
  own->part_lse_off = plan->part_lse_off - plan->own_off;
  own->meta_bytes = plan->meta_bytes - plan->own_off;
  own->ws_bytes = plan->ws_bytes - plan->own_off;
  plan->own_part = std::move(own);
  return RPA_OK;
}

}  // namespace rpa
