// C ABI of librpa.so: argument validation, plan upload and kernel dispatch.
// Every step of the path runs in the HIP kernels launched from here.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <exception>
#include <map>
#include <memory>
#include <set>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "launch.h"
#include "plan.h"

#define RPA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// Message of the last failure on this thread.  A fixed buffer, so that
// recording a failure never allocates (the handlers below run after an
// allocation has failed).
thread_local char g_last_error[512];

void set_error(const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
}
void clear_error() { g_last_error[0] = '\0'; }

rpa_status fail(rpa_status s, const std::string& msg) {
  set_error(msg.c_str());
  return s;
}

rpa_status hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return RPA_ERR_HIP;
}

// Runs an entry point's body; no C++ exception leaves the library.
template <class F>
rpa_status guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    set_error("out of host memory");
    return RPA_ERR_HOST_ALLOC;
  } catch (const std::exception& e) {
    set_error(e.what());
    return RPA_ERR_INTERNAL;
  } catch (...) {
    set_error("unexpected internal error");
    return RPA_ERR_INTERNAL;
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device view of a plan whose workspace (metadata, then partials) starts at ws.
rpa::DevPlan dev_plan(const rpa_plan* plan, void* ws_base) {
  rpa::DevPlan p{};
  const int32_t* base = static_cast<const int32_t*>(ws_base);
  p.qo_indptr = base + plan->off_qo_indptr;
  p.kv_len = base + plan->off_kv_len;
  p.page_indptr = base + plan->off_page_indptr;
  p.page_indices = base + plan->off_page_indices;
  p.split = base + plan->off_split;
  p.append = base + plan->off_append;
  for (int k = 0; k < rpa::KC_COUNT; ++k) {
    p.items[k] = base + plan->off_items[k];
    p.n_items[k] = plan->n_items[k];
    p.wg_indptr[k] = base + plan->off_wg[k];
    p.n_wgs[k] = plan->n_wgs[k];
  }
  p.merge_rows = base + plan->off_merge;
  p.merge_info = base + plan->off_merge_info;
  p.tree_req = plan->off_tree_req >= 0 ? base + plan->off_tree_req : nullptr;
  p.tree_mask = plan->off_tree_mask >= 0
                    ? reinterpret_cast<const uint32_t*>(base + plan->off_tree_mask) : nullptr;
  p.n_merge_rows = plan->n_merge_rows;
  p.dec_stages = plan->dec_stages;
  char* ws = static_cast<char*>(ws_base);
  p.part_o = reinterpret_cast<float*>(ws + plan->part_o_off);
  p.part_lse = reinterpret_cast<float*>(ws + plan->part_lse_off);
  p.batch_size = plan->batch_size;
  p.total_q = plan->total_q;
  p.num_qo_heads = plan->cfg.num_qo_heads;
  p.num_kv_heads = plan->cfg.num_kv_heads;
  p.group = plan->group;
  p.head_dim_qk = plan->cfg.head_dim_qk;
  p.head_dim_v = plan->cfg.head_dim_v;
  p.page_size = plan->cfg.page_size;
  int32_t s = 0;
  while ((1 << s) < plan->cfg.page_size) ++s;
  p.page_shift = s;
  p.causal = plan->cfg.causal;
  p.dtype = plan->cfg.dtype;
  p.sm_scale = plan->cfg.sm_scale;
  return p;
}

// Checks a pool's strides for a row of `row_len` elements.
bool strides_ok(const rpa_cache_strides* st, int32_t row_len, int32_t dtype, std::string* why) {
  if (!st) {
    *why = "null strides";
    return false;
  }
  const int64_t vec = dtype == RPA_DTYPE_BF16 ? 8 : 4;
  if (st->token_stride < row_len || st->head_stride <= 0 || st->page_stride <= 0) {
    *why = "strides must be positive and token_stride >= the stored row length";
    return false;
  }
  if (st->token_stride % vec || st->head_stride % vec || st->page_stride % vec) {
    *why = "strides must be multiples of 16 bytes";
    return false;
  }
  return true;
}

rpa_status check_uploaded(const rpa_plan* plan) {
  if (!plan) return fail(RPA_ERR_INVALID_ARG, "null plan");
  if (!plan->uploaded || !plan->d_ws)
    return fail(RPA_ERR_NOT_UPLOADED, "plan has not been uploaded (call rpa_plan_upload)");
  return RPA_OK;
}

bool shared_latent(const rpa_attn_config& c) { return c.head_dim_qk == 576; }

constexpr const char* kSplitPlanMsg =
    "a split plan runs through rpa_split_attention (it reads the step's own K/V rows)";

// ---- optional per-kernel event timing -------------------------------------------

struct ProfRecord {
  std::string name;
  hipEvent_t start, stop;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::set<std::string> g_prof_only;  // kernels to time (empty: all)
std::vector<ProfRecord> g_prof_pending;
std::vector<hipEvent_t> g_prof_free;
std::map<std::string, std::pair<double, int64_t>> g_prof_totals;

hipError_t prof_event(hipEvent_t* ev) {
  if (!g_prof_free.empty()) {
    *ev = g_prof_free.back();
    g_prof_free.pop_back();
    return hipSuccess;
  }
  // Timing-only events: no system-scope fence (cache writeback and
  // invalidate) when they are recorded, which otherwise costs several
  // microseconds per event between the kernels being timed.
  return hipEventCreateWithFlags(ev, hipEventDisableSystemFence);
}

// Runs `launch`, bracketed by timing events when profiling is on.
template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  std::unique_lock<std::mutex> lock(g_prof_mu);
  if (!g_prof_on || (!g_prof_only.empty() && g_prof_only.count(name) == 0)) {
    lock.unlock();
    return launch();
  }
  hipEvent_t a, b;
  hipError_t e = prof_event(&a);
  if (e != hipSuccess) return e;
  e = prof_event(&b);
  if (e != hipSuccess) return e;
  e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  if (e != hipSuccess) return e;
  g_prof_pending.push_back({name, a, b});
  return hipSuccess;
}

hipError_t prof_drain() {
  for (ProfRecord& rec : g_prof_pending) {
    hipError_t e = hipEventSynchronize(rec.stop);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, rec.start, rec.stop);
    if (e != hipSuccess) return e;
    auto& tot = g_prof_totals[rec.name];
    tot.first += ms;
    tot.second += 1;
    g_prof_free.push_back(rec.start);
    g_prof_free.push_back(rec.stop);
  }
  g_prof_pending.clear();
  return hipSuccess;
}

}  // namespace

RPA_EXPORT int32_t rpa_abi_version(void) { return RPA_ABI_VERSION; }

RPA_EXPORT const char* rpa_status_string(rpa_status s) {
  switch (s) {
    case RPA_OK: return "RPA_OK";
    case RPA_ERR_INVALID_ARG: return "RPA_ERR_INVALID_ARG";
    case RPA_ERR_UNSUPPORTED: return "RPA_ERR_UNSUPPORTED";
    case RPA_ERR_WORKSPACE_TOO_SMALL: return "RPA_ERR_WORKSPACE_TOO_SMALL";
    case RPA_ERR_PAGE_OOB: return "RPA_ERR_PAGE_OOB";
    case RPA_ERR_DUPLICATE_WRITE_PAGE: return "RPA_ERR_DUPLICATE_WRITE_PAGE";
    case RPA_ERR_HIP: return "RPA_ERR_HIP";
    case RPA_ERR_NOT_UPLOADED: return "RPA_ERR_NOT_UPLOADED";
    case RPA_ERR_HOST_ALLOC: return "RPA_ERR_HOST_ALLOC";
    case RPA_ERR_INTERNAL: return "RPA_ERR_INTERNAL";
  }
  return "RPA_ERR_UNKNOWN";
}

RPA_EXPORT const char* rpa_last_error_message(void) { return g_last_error; }

namespace {

rpa_status create_plan(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                       const int32_t* tree_indptr, const uint32_t* tree_words, int32_t num_cus,
                       rpa_plan** out) {
  if (!out) return fail(RPA_ERR_INVALID_ARG, "null output pointer");
  *out = nullptr;
  std::unique_ptr<rpa_plan> plan(new rpa_plan());
  std::string err;
  const rpa_status s = rpa::build_plan(cfg, batch, tree_indptr, tree_words, num_cus, plan.get(),
                                       &err);
  if (s != RPA_OK) return fail(s, err);
  *out = plan.release();
  clear_error();
  return RPA_OK;
}

}  // namespace

RPA_EXPORT rpa_status rpa_plan_create(const rpa_attn_config* cfg, const rpa_batch_desc* batch,
                                      int32_t num_cus, rpa_plan** out) {
  return guarded([&] { return create_plan(cfg, batch, nullptr, nullptr, num_cus, out); });
}

RPA_EXPORT rpa_status rpa_plan_create_tree(const rpa_attn_config* cfg,
                                           const rpa_batch_desc* batch,
                                           const int32_t* tree_indptr,
                                           const uint32_t* tree_words, int32_t num_cus,
                                           rpa_plan** out) {
  return guarded([&] {
    if (out) *out = nullptr;
    if (!tree_indptr) return fail(RPA_ERR_INVALID_ARG, "null tree_indptr");
    return create_plan(cfg, batch, tree_indptr, tree_words, num_cus, out);
  });
}

RPA_EXPORT rpa_status rpa_plan_create_split(const rpa_attn_config* cfg,
                                            const rpa_batch_desc* batch, int32_t num_cus,
                                            rpa_plan** out) {
  return guarded([&] {
    if (!out) return fail(RPA_ERR_INVALID_ARG, "null output pointer");
    *out = nullptr;
    std::unique_ptr<rpa_plan> plan(new rpa_plan());
    std::string err;
    const rpa_status s = rpa::build_split_plan(cfg, batch, num_cus, plan.get(), &err);
    if (s != RPA_OK) return fail(s, err);
    *out = plan.release();
    clear_error();
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_plan_workspace_size(const rpa_plan* plan, size_t* bytes) {
  if (!plan || !bytes) {
    set_error("null plan or bytes pointer");
    return RPA_ERR_INVALID_ARG;
  }
  *bytes = plan->ws_bytes;
  return RPA_OK;
}

RPA_EXPORT rpa_status rpa_plan_upload(rpa_plan* plan, void* d_workspace, size_t bytes,
                                      void* stream) {
  return guarded([&] {
    if (!plan || !d_workspace) return fail(RPA_ERR_INVALID_ARG, "null plan or workspace");
    if (!aligned(d_workspace, 256))
      return fail(RPA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (bytes < plan->ws_bytes)
      return fail(RPA_ERR_WORKSPACE_TOO_SMALL,
                  "workspace has " + std::to_string(bytes) + " bytes, plan needs " +
                      std::to_string(plan->ws_bytes));
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (!plan->event) {
      hipEvent_t ev;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
      plan->event = ev;
    } else {
      // The previous upload may still be reading the staging buffer.
      e = hipEventSynchronize(static_cast<hipEvent_t>(plan->event));
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    }
    if (!plan->staging) {
      e = hipHostMalloc(&plan->staging, plan->meta_bytes, hipHostMallocDefault);
      if (e != hipSuccess) {
        plan->staging = nullptr;
        return hip_fail(e, "hipHostMalloc");
      }
    }
    std::memset(plan->staging, 0, plan->meta_bytes);
    std::memcpy(plan->staging, plan->blob.data(), plan->blob.size() * sizeof(int32_t));
    e = hipMemcpyAsync(d_workspace, plan->staging, plan->meta_bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipEventRecord(static_cast<hipEvent_t>(plan->event), st);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    plan->d_ws = d_workspace;
    plan->uploaded = true;
    clear_error();
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_kv_append(const rpa_plan* plan, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const rpa_cache_strides* ks,
                                    const rpa_cache_strides* vs, void* stream) {
  return guarded([&] {
    rpa_status s = check_uploaded(plan);
    if (s != RPA_OK) return s;
    const rpa_attn_config& c = plan->cfg;
    const bool latent = shared_latent(c);
    std::string why;
    if (plan->total_q == 0) return RPA_OK;  // no new tokens: nothing to read or write
    if (!plan->can_append)
      return fail(RPA_ERR_INVALID_ARG,
                  "the plan has a request with kv_len < qo_len (cross attention): no append slots");
    if (!k_new || !k_cache) return fail(RPA_ERR_INVALID_ARG, "null k_new or k_cache");
    if (!aligned(k_new, 16) || !aligned(k_cache, 16))
      return fail(RPA_ERR_INVALID_ARG, "k_new and k_cache must be 16-byte aligned");
    if (!strides_ok(ks, c.head_dim_qk, c.dtype, &why))
      return fail(RPA_ERR_INVALID_ARG, "k: " + why);
    if (latent) {
      if (v_new) return fail(RPA_ERR_INVALID_ARG, "shared latent cache: v_new must be NULL");
      if (v_cache && v_cache != k_cache)
        return fail(RPA_ERR_INVALID_ARG, "shared latent cache: v_cache must be NULL or k_cache");
    } else {
      if (!v_new || !v_cache) return fail(RPA_ERR_INVALID_ARG, "null v_new or v_cache");
      if (!aligned(v_new, 16) || !aligned(v_cache, 16))
        return fail(RPA_ERR_INVALID_ARG, "v_new and v_cache must be 16-byte aligned");
      if (!strides_ok(vs, c.head_dim_v, c.dtype, &why))
        return fail(RPA_ERR_INVALID_ARG, "v: " + why);
    }
    rpa::DevPlan p = dev_plan(plan, plan->d_ws);
    rpa::Strides k_st{ks->page_stride, ks->head_stride, ks->token_stride};
    rpa::Strides v_st =
        latent ? k_st : rpa::Strides{vs->page_stride, vs->head_stride, vs->token_stride};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = timed("append", st, [&] {
      return rpa::launch_append(p, k_new, latent ? nullptr : v_new, k_cache,
                                latent ? nullptr : v_cache, k_st, v_st, st);
    });
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    return RPA_OK;
  });
}

namespace {

// Pool views of an attention call, after validation.
struct AttnPools {
  rpa::Strides k_st, v_st;
  const void* vc;
};

// Validates the tensor arguments of an attention call against the plan.
rpa_status attention_args(const rpa_plan* plan, const void* q, const void* k_cache,
                          const void* v_cache, const rpa_cache_strides* ks,
                          const rpa_cache_strides* vs, const void* o, const float* lse,
                          AttnPools* out) {
  const rpa_attn_config& c = plan->cfg;
  const bool latent = shared_latent(c);
  std::string why;
  if (!q || !k_cache || !o) return fail(RPA_ERR_INVALID_ARG, "null q, k_cache or o");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(o, 16))
    return fail(RPA_ERR_INVALID_ARG, "q, k_cache and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(RPA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!strides_ok(ks, c.head_dim_qk, c.dtype, &why)) return fail(RPA_ERR_INVALID_ARG, "k: " + why);
  out->k_st = rpa::Strides{ks->page_stride, ks->head_stride, ks->token_stride};
  out->v_st = out->k_st;
  out->vc = v_cache;
  if (latent) {
    if (v_cache && v_cache != k_cache)
      return fail(RPA_ERR_UNSUPPORTED, "576/512 needs the shared latent cache (v_cache == k_cache)");
    if (vs && (vs->page_stride != ks->page_stride || vs->head_stride != ks->head_stride ||
               vs->token_stride != ks->token_stride))
      return fail(RPA_ERR_UNSUPPORTED, "576/512 needs vs == ks (shared latent cache)");
    out->vc = k_cache;
  } else {
    if (!v_cache) return fail(RPA_ERR_INVALID_ARG, "null v_cache");
    if (!aligned(v_cache, 16)) return fail(RPA_ERR_INVALID_ARG, "v_cache must be 16-byte aligned");
    if (!strides_ok(vs, c.head_dim_v, c.dtype, &why)) return fail(RPA_ERR_INVALID_ARG, "v: " + why);
    out->v_st = rpa::Strides{vs->page_stride, vs->head_stride, vs->token_stride};
  }
  return RPA_OK;
}

// Launches the attention kernels of every class the plan uses, then (with
// `merge`) the merge of split pieces, on one stream.
rpa_status run_attention(const rpa::DevPlan& p, const void* q, const void* k_cache,
                         const AttnPools& a, void* o, float* lse, hipStream_t st,
                         bool merge = true) {
  hipError_t e;
  if (p.n_items[rpa::KC_GENERIC] > 0) {
    e = timed("generic", st, [&] {
      return rpa::launch_generic(p, q, k_cache, a.vc, a.k_st, a.v_st, o, lse, st);
    });
    if (e != hipSuccess) return hip_fail(e, "generic attention launch");
  }
  if (p.n_items[rpa::KC_DECODE] > 0) {
    e = timed("decode", st, [&] {
      return rpa::launch_decode(p, q, k_cache, a.vc, a.k_st, a.v_st, o, lse, st);
    });
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  }
  if (p.n_items[rpa::KC_PREFILL] > 0) {
    e = timed("prefill", st, [&] {
      return rpa::launch_prefill(p, q, k_cache, a.vc, a.k_st, a.v_st, o, lse, st);
    });
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  }
  if (p.n_items[rpa::KC_MLA] > 0) {
    e = timed("mla", st, [&] { return rpa::launch_mla(p, q, k_cache, a.k_st, o, lse, st); });
    if (e != hipSuccess) return hip_fail(e, "latent attention launch");
  }
  if (merge && p.n_merge_rows > 0) {
    e = timed("merge", st, [&] { return rpa::launch_merge_rows(p, o, lse, st); });
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return RPA_OK;
}

// Split execution: the cache part's and the own part's kernels, then the
// merge of both.  Streaming classes run part after part; the prefill items of
// both parts share one launch, each part's workgroups planned for its share
// of the compute units.
rpa_status run_split(const rpa::DevPlan& cp, const AttnPools& ca, const rpa::DevPlan& op,
                     const AttnPools& oa, const void* q, const void* k_cache, const void* k_new,
                     void* o, float* lse, hipStream_t st) {
  hipError_t e;
  for (const bool own : {false, true}) {
    const rpa::DevPlan& p = own ? op : cp;
    const AttnPools& a = own ? oa : ca;
    const void* kc = own ? k_new : k_cache;
    if (p.n_items[rpa::KC_GENERIC] > 0) {
      e = timed("generic", st, [&] {
        return rpa::launch_generic(p, q, kc, a.vc, a.k_st, a.v_st, o, lse, st);
      });
      if (e != hipSuccess) return hip_fail(e, "generic attention launch");
    }
    if (p.n_items[rpa::KC_DECODE] > 0) {
      e = timed("decode", st, [&] {
        return rpa::launch_decode(p, q, kc, a.vc, a.k_st, a.v_st, o, lse, st);
      });
      if (e != hipSuccess) return hip_fail(e, "decode attention launch");
    }
  }
  const bool pc = cp.n_items[rpa::KC_PREFILL] > 0, po = op.n_items[rpa::KC_PREFILL] > 0;
  if (pc || po) {
    e = timed("prefill", st, [&] {
      if (pc && po)
        return rpa::launch_prefill2(cp, k_cache, ca.vc, ca.k_st, ca.v_st, op, k_new, oa.vc,
                                    oa.k_st, oa.v_st, q, o, lse, st);
      const rpa::DevPlan& p = pc ? cp : op;
      const AttnPools& a = pc ? ca : oa;
      return rpa::launch_prefill(p, q, pc ? k_cache : k_new, a.vc, a.k_st, a.v_st, o, lse, st);
    });
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  }
  if (cp.n_merge_rows > 0) {
    e = timed("merge", st, [&] { return rpa::launch_merge_rows(cp, o, lse, st); });
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return RPA_OK;
}

}  // namespace

RPA_EXPORT rpa_status rpa_batch_attention(const rpa_plan* plan, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const rpa_cache_strides* ks,
                                          const rpa_cache_strides* vs, void* o, float* lse,
                                          void* stream) {
  return guarded([&] {
    if (plan && plan->own_part) return fail(RPA_ERR_INVALID_ARG, kSplitPlanMsg);
    rpa_status s = check_uploaded(plan);
    if (s != RPA_OK) return s;
    if (plan->total_q == 0) return RPA_OK;  // no query rows: nothing to compute
    AttnPools a;
    s = attention_args(plan, q, k_cache, v_cache, ks, vs, o, lse, &a);
    if (s != RPA_OK) return s;
    return run_attention(dev_plan(plan, plan->d_ws), q, k_cache, a, o, lse,
                         static_cast<hipStream_t>(stream));
  });
}

RPA_EXPORT rpa_status rpa_split_attention(const rpa_plan* plan, const void* q,
                                          const void* k_new, const void* v_new,
                                          const void* k_cache, const void* v_cache,
                                          const rpa_cache_strides* ks,
                                          const rpa_cache_strides* vs, void* o, float* lse,
                                          void* stream) {
  return guarded([&] {
    if (plan && !plan->own_part)
      return fail(RPA_ERR_INVALID_ARG, "not a split plan (create it with rpa_plan_create_split)");
    rpa_status s = check_uploaded(plan);
    if (s != RPA_OK) return s;
    if (plan->total_q == 0) return RPA_OK;  // no query rows: nothing to compute
    AttnPools a;
    s = attention_args(plan, q, k_cache, v_cache, ks, vs, o, lse, &a);
    if (s != RPA_OK) return s;
    if (!k_new || !v_new) return fail(RPA_ERR_INVALID_ARG, "null k_new or v_new");
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
      return fail(RPA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    const rpa_attn_config& c = plan->cfg;
    // The step's own rows, token-major [total_q, num_kv_heads, d]: request
    // r's page (id qo_indptr[r]) starts at its first row, so the page stride
    // is one row.
    const int64_t krow = (int64_t)c.num_kv_heads * c.head_dim_qk;
    const int64_t vrow = (int64_t)c.num_kv_heads * c.head_dim_v;
    AttnPools own;
    own.k_st = rpa::Strides{krow, c.head_dim_qk, krow};
    own.v_st = rpa::Strides{vrow, c.head_dim_v, vrow};
    own.vc = v_new;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(plan->d_ws);
    return run_split(dev_plan(plan, ws), a, dev_plan(plan->own_part.get(), ws + plan->own_off),
                     own, q, k_cache, k_new, o, lse, st);
  });
}

RPA_EXPORT rpa_status rpa_batch_attention_noalloc(const rpa_plan* plan, const void* q,
                                                  const void* k_cache, const void* v_cache,
                                                  const rpa_cache_strides* ks,
                                                  const rpa_cache_strides* vs, void* o,
                                                  float* lse, void* stream) {
  return guarded([&] {
    if (!plan) return fail(RPA_ERR_INVALID_ARG, "null plan");
    if (plan->own_part) return fail(RPA_ERR_INVALID_ARG, kSplitPlanMsg);
    if (plan->total_q == 0) return RPA_OK;  // no query rows: nothing to compute
    AttnPools a;
    rpa_status s = attention_args(plan, q, k_cache, v_cache, ks, vs, o, lse, &a);
    if (s != RPA_OK) return s;
    if (plan->ws_bytes > rpa::kStaticScratchBytes)
      return fail(RPA_ERR_WORKSPACE_TOO_SMALL,
                  "the plan needs " + std::to_string(plan->ws_bytes) +
                      " bytes of workspace; the static scratch holds " +
                      std::to_string(rpa::kStaticScratchBytes) +
                      " (use rpa_batch_attention with a workspace)");
    void* ws = nullptr;
    hipError_t e = rpa::static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The metadata goes from the plan's host copy into the scratch, ordered
    // on the stream before the kernels that read it.  Nothing in the scratch
    // needs to start at zero: every partial the merge reads is written by
    // this call's attention kernels first.
    e = hipMemcpyAsync(ws, plan->blob.data(), plan->blob.size() * sizeof(int32_t),
                       hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of the plan metadata");
    return run_attention(dev_plan(plan, ws), q, k_cache, a, o, lse, st);
  });
}

RPA_EXPORT rpa_status rpa_merge_state(const void* o_a, const float* lse_a, const void* o_b,
                                      const float* lse_b, void* o, float* lse, int64_t rows,
                                      int32_t heads, int32_t dim, int32_t dtype, void* stream) {
  return guarded([&] {
    if (dtype != RPA_DTYPE_F32 && dtype != RPA_DTYPE_BF16)
      return fail(RPA_ERR_INVALID_ARG, "dtype must be RPA_DTYPE_F32 or RPA_DTYPE_BF16");
    if (rows < 0 || heads <= 0 || dim <= 0)
      return fail(RPA_ERR_INVALID_ARG, "bad rows/heads/dim");
    if (dim % 8 != 0) return fail(RPA_ERR_INVALID_ARG, "dim must be a multiple of 8");
    if (rows == 0) return RPA_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o)
      return fail(RPA_ERR_INVALID_ARG, "null o_a, lse_a, o_b, lse_b or o");
    if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16))
      return fail(RPA_ERR_INVALID_ARG, "o_a, o_b and o must be 16-byte aligned");
    // Several threads read each input lse value; one of them writes the
    // output lse.  An output lse over an input would race.
    if (lse && (lse == lse_a || lse == lse_b))
      return fail(RPA_ERR_INVALID_ARG, "lse must not alias lse_a or lse_b");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = timed("merge_state", st, [&] {
      return rpa::launch_merge_state(o_a, lse_a, o_b, lse_b, o, lse, rows, heads, dim, dtype, st);
    });
    if (e != hipSuccess) return hip_fail(e, "merge_state launch");
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_page_copy(const void* src, const rpa_cache_strides* src_strides,
                                    int32_t src_pool_pages, int32_t src_pool_heads,
                                    const int32_t* src_pages, void* dst,
                                    const rpa_cache_strides* dst_strides, int32_t dst_pool_pages,
                                    int32_t dst_pool_heads, const int32_t* dst_pages,
                                    int32_t num_pages, int32_t src_head0, int32_t dst_head0,
                                    int32_t num_heads, int32_t page_size, int32_t dim,
                                    int32_t dtype, void* stream) {
  return guarded([&] {
    if (dtype != RPA_DTYPE_F32 && dtype != RPA_DTYPE_BF16)
      return fail(RPA_ERR_INVALID_ARG, "dtype must be RPA_DTYPE_F32 or RPA_DTYPE_BF16");
    if (num_pages < 0 || num_heads <= 0 || page_size <= 0 || dim <= 0 || src_head0 < 0 ||
        dst_head0 < 0)
      return fail(RPA_ERR_INVALID_ARG, "bad num_pages, heads, page_size or dim");
    if (src_pool_pages < 0 || dst_pool_pages < 0 || src_pool_heads <= 0 || dst_pool_heads <= 0)
      return fail(RPA_ERR_INVALID_ARG, "bad pool page or head counts");
    if ((int64_t)src_head0 + num_heads > src_pool_heads ||
        (int64_t)dst_head0 + num_heads > dst_pool_heads)
      return fail(RPA_ERR_INVALID_ARG, "head range outside the pool's heads");
    if ((!src_pages && num_pages > src_pool_pages) || (!dst_pages && num_pages > dst_pool_pages))
      return fail(RPA_ERR_PAGE_OOB, "identity page list longer than the pool");
    const int32_t vec = dtype == RPA_DTYPE_BF16 ? 8 : 4;
    if (dim % vec) return fail(RPA_ERR_INVALID_ARG, "dim must fill whole 16-byte chunks");
    if (num_pages == 0) return RPA_OK;
    if (!src || !dst) return fail(RPA_ERR_INVALID_ARG, "null src or dst");
    if (!aligned(src, 16) || !aligned(dst, 16))
      return fail(RPA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    if ((src_pages && !aligned(src_pages, 4)) || (dst_pages && !aligned(dst_pages, 4)))
      return fail(RPA_ERR_INVALID_ARG, "page id arrays must be 4-byte aligned");
    std::string why;
    if (!strides_ok(src_strides, dim, dtype, &why))
      return fail(RPA_ERR_INVALID_ARG, "src: " + why);
    if (!strides_ok(dst_strides, dim, dtype, &why))
      return fail(RPA_ERR_INVALID_ARG, "dst: " + why);
    const int64_t es = dtype == RPA_DTYPE_BF16 ? 2 : 4;
    if ((int64_t)num_heads * page_size * (dim * es / 16) > INT32_MAX)
      return fail(RPA_ERR_INVALID_ARG, "page too large");
    const rpa::Strides sb{src_strides->page_stride * es, src_strides->head_stride * es,
                          src_strides->token_stride * es};
    const rpa::Strides db{dst_strides->page_stride * es, dst_strides->head_stride * es,
                          dst_strides->token_stride * es};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = timed("page_copy", st, [&] {
      return rpa::launch_page_copy(src, sb, src_pages, src_pool_pages, dst, db, dst_pages,
                                   dst_pool_pages, num_pages, src_head0, dst_head0, num_heads,
                                   page_size, (int32_t)(dim * es), st);
    });
    if (e != hipSuccess) return hip_fail(e, "page_copy launch");
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_profile_enable(int32_t on) {
  return guarded([&] {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = on != 0;
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_profile_select(const char* kernels) {
  return guarded([&] {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_only.clear();
    if (kernels == nullptr) return RPA_OK;
    std::string cur;
    for (const char* c = kernels;; ++c) {
      if (*c == ',' || *c == '\0') {
        if (!cur.empty()) g_prof_only.insert(cur);
        cur.clear();
        if (*c == '\0') break;
      } else {
        cur.push_back(*c);
      }
    }
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  return guarded([&] {
    if (!kernel || !total_ms || !launches) return fail(RPA_ERR_INVALID_ARG, "null argument");
    std::lock_guard<std::mutex> lock(g_prof_mu);
    hipError_t e = prof_drain();
    if (e != hipSuccess) return hip_fail(e, "profile events");
    auto it = g_prof_totals.find(kernel);
    *total_ms = it == g_prof_totals.end() ? 0.0 : it->second.first;
    *launches = it == g_prof_totals.end() ? 0 : it->second.second;
    return RPA_OK;
  });
}

RPA_EXPORT rpa_status rpa_profile_reset(void) {
  return guarded([&] {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    hipError_t e = prof_drain();
    g_prof_totals.clear();
    if (e != hipSuccess) return hip_fail(e, "profile events");
    return RPA_OK;
  });
}

RPA_EXPORT void rpa_plan_destroy(rpa_plan* plan) {
  if (!plan) return;
  if (plan->event) {
    (void)hipEventSynchronize(static_cast<hipEvent_t>(plan->event));
    (void)hipEventDestroy(static_cast<hipEvent_t>(plan->event));
  }
  if (plan->staging) (void)hipHostFree(plan->staging);
  delete plan;  // vectors only: their destructors do not throw
}

RPA_EXPORT rpa_status rpa_plan_debug_dump(const rpa_plan* plan, const char* name, int32_t* dst,
                                          int64_t cap, int64_t* len) {
  return guarded([&] {
    if (!plan || !name || !len) return fail(RPA_ERR_INVALID_ARG, "null plan, name or len");
    const int32_t* src = nullptr;
    int64_t n = 0;
    std::vector<int32_t> tmp;
    std::string nm(name);
    // "own:<table>" reads the own part of a split plan
    if (nm.compare(0, 4, "own:") == 0) {
      if (!plan->own_part) return fail(RPA_ERR_INVALID_ARG, "not a split plan: " + nm);
      plan = plan->own_part.get();
      nm = nm.substr(4);
    }
    const int32_t* blob = plan->blob.data();
    if (nm == "items") {
      for (int k = 0; k < rpa::KC_COUNT; ++k)
        tmp.insert(tmp.end(), blob + plan->off_items[k],
                   blob + plan->off_items[k] + (int64_t)plan->n_items[k] * rpa::IT_WORDS);
      src = tmp.data();
      n = (int64_t)tmp.size();
    } else if (nm == "splits") {
      src = blob + plan->off_split;
      n = (int64_t)plan->batch_size * rpa::SP_WORDS;
    } else if (nm == "append") {
      src = blob + plan->off_append;
      n = (int64_t)plan->total_q * 2;
    } else if (nm == "wg_prefill" || nm == "wg_mla" || nm == "wg_decode") {
      const int k = nm == "wg_prefill" ? rpa::KC_PREFILL
                                       : (nm == "wg_mla" ? rpa::KC_MLA : rpa::KC_DECODE);
      src = blob + plan->off_wg[k];
      n = plan->n_items[k] > 0 ? (int64_t)plan->n_wgs[k] + 1 : 0;
    } else if (nm == "merge_rows") {
      src = blob + plan->off_merge;
      n = plan->n_merge_rows;
    } else if (nm == "merge_info") {
      src = blob + plan->off_merge_info;
      n = (int64_t)plan->n_merge_rows * 4;
    } else if (nm == "summary") {
      int32_t total = 0;
      for (int k = 0; k < rpa::KC_COUNT; ++k) total += plan->n_items[k];
      tmp = {plan->batch_size, plan->total_q, total, (int32_t)plan->partial_rows,
             plan->n_items[0], plan->n_items[1], plan->n_items[2], plan->n_items[3]};
      src = tmp.data();
      n = (int64_t)tmp.size();
    } else {
      return fail(RPA_ERR_INVALID_ARG, "unknown table name: " + nm);
    }
    *len = n;
    if (dst && cap > 0)
      std::memcpy(dst, src, (size_t)std::min<int64_t>(cap, n) * sizeof(int32_t));
    return RPA_OK;
  });
}
