// Host launchers of the HIP kernels (internal).  Each returns the HIP status
// of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include "rpa_internal.h"

namespace rpa {

// Size of the static device scratch used by rpa_batch_attention_noalloc.
constexpr size_t kStaticScratchBytes = RPA_STATIC_SCRATCH_BYTES;

// Device address of this device's static scratch (looked up once per device,
// with that device current).
hipError_t static_scratch(void** out);

hipError_t launch_append(const DevPlan& p, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, Strides ks, Strides vs, hipStream_t stream);

hipError_t launch_generic(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream);

hipError_t launch_decode(const DevPlan& p, const void* q, const void* k_cache, const void* v_cache,
                         Strides ks, Strides vs, void* o, float* lse, hipStream_t stream);

hipError_t launch_prefill(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream);

// One prefill launch over the items of two plans (the two parts of a split
// execution), each with its own pools: workgroups 0 .. p0.n_wgs - 1 run p0's
// lists, the next p1.n_wgs run p1's.
hipError_t launch_prefill2(const DevPlan& p0, const void* k0, const void* v0, Strides ks0,
                           Strides vs0, const DevPlan& p1, const void* k1, const void* v1,
                           Strides ks1, Strides vs1, const void* q, void* o, float* lse,
                           hipStream_t stream);

hipError_t launch_mla(const DevPlan& p, const void* q, const void* kv_cache, Strides ks, void* o,
                      float* lse, hipStream_t stream);

// Folds the split pieces of every row in p.merge_rows into o / lse.
hipError_t launch_merge_rows(const DevPlan& p, void* o, float* lse, hipStream_t stream);

// Copy of head ranges of pages between pools or buffers (strides in bytes).
// Page pairs with an id outside [0, pool pages) are skipped.
hipError_t launch_page_copy(const void* src, Strides src_b, const int32_t* src_pages,
                            int32_t src_pool_pages, void* dst, Strides dst_b,
                            const int32_t* dst_pages, int32_t dst_pool_pages, int32_t num_pages,
                            int32_t src_h0, int32_t dst_h0, int32_t num_heads, int32_t page_size,
                            int32_t row_bytes, hipStream_t stream);

// Standalone two-state merge.
hipError_t launch_merge_state(const void* o_a, const float* lse_a, const void* o_b,
                              const float* lse_b, void* o, float* lse, int64_t rows, int32_t heads,
                              int32_t dim, int32_t dtype, hipStream_t stream);

}  // namespace rpa
