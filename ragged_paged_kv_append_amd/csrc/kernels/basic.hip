// KV append, generic attention and the log-sum-exp merges (gfx950).
//
// KV append: every new token's K/V row is copied into its page slot; the
// disaggregation post (KV Messenger section) has each layer append its new
// KV entries before the attention that reads them, and pages use the HND
// layout (sharded-transfer section).
//
// Generic attention: one wavefront per query row, one lane per key in blocks
// of 64 keys, online softmax across blocks.  It serves every dtype, head
// dimension and page size; the MFMA kernels take the bf16 shapes.
//
// Merge: the online-softmax merge of the chunked-prefill post (section
// "correctness") folds the split pieces of a row.

#include "common.h"
#include "../launch.h"

namespace rpa {

// ----------------------------------------------------------------------------
// KV append
// ----------------------------------------------------------------------------

// One workgroup per new token: its page and slot are one scalar load, and its
// threads copy the token's K rows (all KV heads, contiguous in k_new) and then
// its V rows, 16 bytes per thread and step.  A plain copy: the stored bits
// move unchanged.  kc_div / vc_div: 16-byte chunks per K / V row.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(DevPlan p, const T* __restrict__ k_new,
                                                     const T* __restrict__ v_new,
                                                     T* __restrict__ k_cache,
                                                     T* __restrict__ v_cache, Strides ks,
                                                     Strides vs, int32_t kc_div, int32_t vc_div) {
  constexpr int kVec = 16 / sizeof(T);
  const int64_t i = blockIdx.x;  // new token (global row)
  const int64_t page = p.append[2 * i];
  const int64_t slot = p.append[2 * i + 1];
  const int32_t H = p.num_kv_heads;
  const int32_t kn = H * kc_div;             // K chunks of the token
  const int32_t vn = v_new ? H * vc_div : 0;  // V chunks
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new + i * H * p.head_dim_qk);
  for (int32_t c = threadIdx.x; c < kn; c += blockDim.x) {
    const int32_t h = c / kc_div, ch = c - h * kc_div;
    *reinterpret_cast<uint4*>(k_cache + page * ks.page + h * ks.head + slot * ks.token +
                              ch * kVec) = ksrc[c];
  }
  if (vn == 0) return;
  const uint4* vsrc = reinterpret_cast<const uint4*>(v_new + i * H * p.head_dim_v);
  for (int32_t c = threadIdx.x; c < vn; c += blockDim.x) {
    const int32_t h = c / vc_div, ch = c - h * vc_div;
    *reinterpret_cast<uint4*>(v_cache + page * vs.page + h * vs.head + slot * vs.token +
                              ch * kVec) = vsrc[c];
  }
}

hipError_t launch_append(const DevPlan& p, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, Strides ks, Strides vs, hipStream_t stream) {
  const int vec = p.dtype == RPA_DTYPE_BF16 ? 8 : 4;
  if (p.total_q == 0) return hipSuccess;
  const int32_t kc = p.head_dim_qk / vec, vc = v_new ? p.head_dim_v / vec : 1;
  const int32_t chunks = p.num_kv_heads * (kc + (v_new ? vc : 0));
  const int bs = chunks >= 256 ? 256 : (chunks + 63) / 64 * 64;
  if (p.dtype == RPA_DTYPE_BF16) {
    hipLaunchKernelGGL(append_kernel<bf16_t>, dim3((unsigned)p.total_q), dim3(bs), 0, stream, p,
                       static_cast<const bf16_t*>(k_new), static_cast<const bf16_t*>(v_new),
                       static_cast<bf16_t*>(k_cache), static_cast<bf16_t*>(v_cache), ks, vs, kc,
                       vc);
  } else {
    hipLaunchKernelGGL(append_kernel<float>, dim3((unsigned)p.total_q), dim3(bs), 0, stream, p,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), ks, vs, kc, vc);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Generic attention
// ----------------------------------------------------------------------------

// Writes one row's result: the final output when the request is not split,
// else the float32 partial of piece s (normalized like the output).
template <typename T>
__device__ __forceinline__ void write_row(const DevPlan& p, int32_t r, int32_t i, int32_t t,
                                          int32_t h, int32_t s, int32_t n, float lse_nat,
                                          const float* vals, int32_t d0, int32_t count,
                                          int32_t stride, T* o, float* lse, bool write_lse) {
  const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
  if (S == 1) {
    T* orow = o + ((int64_t)i * p.num_qo_heads + h) * p.head_dim_v;
    for (int32_t c = 0; c < count; ++c) orow[d0 + c * stride] = from_f32<T>(vals[c]);
    if (write_lse && lse) lse[(int64_t)i * p.num_qo_heads + h] = lse_nat;
  } else {
    const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
    float* orow = p.part_o + (prow * p.num_qo_heads + h) * p.head_dim_v;
    for (int32_t c = 0; c < count; ++c) orow[d0 + c * stride] = vals[c];
    if (write_lse) p.part_lse[prow * p.num_qo_heads + h] = lse_nat;
  }
}

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void generic_kernel(DevPlan p, const T* __restrict__ q,
                                                      const T* __restrict__ kc,
                                                      const T* __restrict__ vc, Strides ks,
                                                      Strides vs, T* __restrict__ o,
                                                      float* __restrict__ lse) {
  constexpr int kWaves = 4;
  constexpr int kCols = (DV + 63) / 64;
  __shared__ float qs[kWaves][DQK];
  const int32_t* it = p.items[KC_GENERIC] + (int64_t)blockIdx.x * IT_WORDS;
  const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], row0 = it[IT_ROW0], row1 = it[IT_ROW1];
  const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t G = p.group;
  const int32_t q0 = p.qo_indptr[r];
  const int32_t n = p.qo_indptr[r + 1] - q0;
  const int32_t L = p.kv_len[r];
  const int32_t cached = L - n;

  // Stage the query rows of all waves in LDS (float32).
  for (int w = 0; w < kWaves; ++w) {
    const int32_t row = row0 + w;
    if (row < row1) {
      const int32_t t = row / G, h = g * G + row % G;
      const T* qrow = q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * DQK;
      for (int d = threadIdx.x; d < DQK; d += blockDim.x) qs[w][d] = to_f32<T>(qrow[d]);
    }
  }
  __syncthreads();
  const int32_t row = row0 + wave;
  if (row >= row1) return;  // no block-level barrier after this point
  const int32_t t = row / G, h = g * G + row % G;
  const int32_t i = q0 + t;
  // A request with a tree mask sees every key up to L - 1, filtered among the
  // new tokens by its 64-bit mask row.
  const bool tree = p.tree_mask != nullptr && p.tree_req[r] != 0;
  const uint64_t tmask = tree ? ((uint64_t)p.tree_mask[2 * (int64_t)i + 1] << 32) |
                                    p.tree_mask[2 * (int64_t)i]
                              : 0ull;
  const int32_t pmax = (p.causal && !tree) ? cached + t : L - 1;
  const int32_t kend = min(k1, pmax + 1);
  const int32_t* pages = p.page_indices + p.page_indptr[r];
  const float sc = p.sm_scale * kLog2e;  // scores kept in log2 units

  float m = -INFINITY, l = 0.f;
  float acc[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) acc[c] = 0.f;

  for (int32_t kb = k0; kb < kend; kb += 64) {
    const int32_t key = kb + lane;
    const bool valid = key < kend && !(tree && key >= cached &&
                                       !((tmask >> (uint32_t)(key - cached)) & 1ull));
    float sv = -INFINITY;
    int64_t voff = 0;
    if (valid) {
      const int64_t page = pages[key >> p.page_shift];
      const int64_t slot = key & (p.page_size - 1);
      const T* krow = kc + page * ks.page + (int64_t)g * ks.head + slot * ks.token;
      voff = page * vs.page + (int64_t)g * vs.head + slot * vs.token;
      float dot = 0.f;
#pragma unroll 4
      for (int d = 0; d < DQK; d += 8) {
        float kv[8];
        load8(krow + d, kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qs[wave][d + e], kv[e], dot);
      }
      sv = dot * sc;
    }
    const float mb = wave_max(sv);
    const float m_new = fmaxf(m, mb);
    const float pr = valid ? exp2f(sv - m_new) : 0.f;
    const float alpha = exp2f(m - m_new);  // 0 on the first block (m = -inf)
    l = l * alpha + wave_sum(pr);
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[c] *= alpha;
    const int32_t nk = min(64, kend - kb);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(pr, j, 64);
      const int64_t vo = __shfl(voff, j, 64);
      const T* vrow = vc + vo;
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const int d = lane + 64 * c;
        if (d < DV) acc[c] = fmaf(pj, to_f32<T>(vrow[d]), acc[c]);
      }
    }
    m = m_new;
  }

  float vals[kCols];
  float lse_nat = -INFINITY;
  if (l > 0.f) {
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < kCols; ++c) vals[c] = acc[c] * inv;
    lse_nat = (m + log2f(l)) * kLn2;
  } else {
#pragma unroll
    for (int c = 0; c < kCols; ++c) vals[c] = 0.f;
  }
  const int count = (DV - lane + 63) / 64;
  write_row<T>(p, r, i, t, h, s, n, lse_nat, vals, lane, count, 64, o, lse, lane == 0);
}

template <typename T>
static hipError_t launch_generic_t(const DevPlan& p, const T* q, const T* kc, const T* vc,
                                   Strides ks, Strides vs, T* o, float* lse, hipStream_t stream) {
  const dim3 grid(p.n_items[KC_GENERIC]), block(256);
  if (p.head_dim_qk == 64)
    hipLaunchKernelGGL((generic_kernel<T, 64, 64>), grid, block, 0, stream, p, q, kc, vc, ks, vs,
                       o, lse);
  else if (p.head_dim_qk == 128)
    hipLaunchKernelGGL((generic_kernel<T, 128, 128>), grid, block, 0, stream, p, q, kc, vc, ks,
                       vs, o, lse);
  else
    hipLaunchKernelGGL((generic_kernel<T, 576, 512>), grid, block, 0, stream, p, q, kc, vc, ks,
                       vs, o, lse);
  return hipGetLastError();
}

hipError_t launch_generic(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream) {
  if (p.dtype == RPA_DTYPE_BF16)
    return launch_generic_t<bf16_t>(p, static_cast<const bf16_t*>(q),
                                    static_cast<const bf16_t*>(k_cache),
                                    static_cast<const bf16_t*>(v_cache), ks, vs,
                                    static_cast<bf16_t*>(o), lse, stream);
  return launch_generic_t<float>(p, static_cast<const float*>(q),
                                 static_cast<const float*>(k_cache),
                                 static_cast<const float*>(v_cache), ks, vs,
                                 static_cast<float*>(o), lse, stream);
}

// ----------------------------------------------------------------------------
// Merge of split pieces
// ----------------------------------------------------------------------------

// Block (x, y) merges row p.merge_rows[x]; a thread owns 8 consecutive output
// elements of one head (task y * blockDim.x + thread of the row's H * d_v / 8).
// The plan gives each merge row its first partial row, the stride between its
// pieces and how many pieces hold a key the row sees, so the partial loads
// depend on one table load only.  The pieces are read eight at a time, with
// a running maximum, so their loads are in flight together.
template <typename T>
__global__ __launch_bounds__(256) void merge_rows_kernel(DevPlan p, T* __restrict__ o,
                                                         float* __restrict__ lse) {
  constexpr int kGroup = 8;
  const int32_t DV = p.head_dim_v;
  const int32_t per_head = DV / 8;
  const int32_t H = p.num_qo_heads;
  const int32_t x = blockIdx.y * blockDim.x + threadIdx.x;
  if (x >= H * per_head) return;
  const int32_t i = p.merge_rows[blockIdx.x];
  const int4 info = *reinterpret_cast<const int4*>(p.merge_info + 4 * (int64_t)blockIdx.x);
  const int64_t prow0 = info.x;
  const int32_t n = info.y;
  const int32_t S_eff = info.z;  // 0: no key, an empty state
  const int32_t h = x / per_head;
  const int32_t d0 = (x - h * per_head) * 8;
  float m = -INFINITY;  // running maximum of the pieces' lse
  float tot = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int32_t s0 = 0; s0 < S_eff; s0 += kGroup) {
    float ls[kGroup];
    float v[kGroup][8];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (s0 + u < S_eff) {
        const int64_t prow = prow0 + (int64_t)(s0 + u) * n;
        ls[u] = p.part_lse[prow * H + h];
        load8(p.part_o + (prow * H + h) * DV + d0, v[u]);
      } else {
        ls[u] = -INFINITY;
      }
    }
    float mg = m;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) mg = fmaxf(mg, ls[u]);
    if (mg == -INFINITY) continue;  // nothing seen yet
    const float a = (m == -INFINITY) ? 0.f : __expf(m - mg);
    tot *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (s0 + u < S_eff && ls[u] != -INFINITY) {
        const float w = __expf(ls[u] - mg);
        tot += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
    m = mg;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8(o + ((int64_t)i * H + h) * DV + d0, acc);
  if (lse && d0 == 0) lse[(int64_t)i * H + h] = tot > 0.f ? m + __logf(tot) : -INFINITY;
}

hipError_t launch_merge_rows(const DevPlan& p, void* o, float* lse, hipStream_t stream) {
  const int tasks = p.num_qo_heads * (p.head_dim_v / 8);
  const int bs = tasks >= 256 ? 256 : (tasks + 63) / 64 * 64;
  const dim3 grid(p.n_merge_rows, (tasks + bs - 1) / bs), block(bs);
  if (p.dtype == RPA_DTYPE_BF16)
    hipLaunchKernelGGL(merge_rows_kernel<bf16_t>, grid, block, 0, stream, p,
                       static_cast<bf16_t*>(o), lse);
  else
    hipLaunchKernelGGL(merge_rows_kernel<float>, grid, block, 0, stream, p, static_cast<float*>(o),
                       lse);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Standalone two-state merge
// ----------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void merge_state_kernel(const T* o_a, const float* lse_a,
                                                          const T* o_b, const float* lse_b,
                                                          T* o, float* lse, int64_t rows,
                                                          int32_t heads, int32_t dim) {
  const int32_t per_head = dim / 8;
  const int64_t total = rows * heads * per_head;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rh = x / per_head;  // row * heads + head
    const int32_t d0 = (int32_t)(x - rh * per_head) * 8;
    const float la = lse_a[rh], lb = lse_b[rh];
    const float mx = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, out_lse = -INFINITY;
    if (mx != -INFINITY) {
      const float ea = la == -INFINITY ? 0.f : __expf(la - mx);
      const float eb = lb == -INFINITY ? 0.f : __expf(lb - mx);
      const float tot = ea + eb;
      wa = ea / tot;
      wb = eb / tot;
      out_lse = mx + __logf(tot);
    }
    float va[8], vb[8], vo[8];
    load8(o_a + rh * dim + d0, va);
    load8(o_b + rh * dim + d0, vb);
#pragma unroll
    for (int e = 0; e < 8; ++e) vo[e] = wa * va[e] + wb * vb[e];
    store8(o + rh * dim + d0, vo);
    if (lse && d0 == 0) lse[rh] = out_lse;
  }
}

hipError_t launch_merge_state(const void* o_a, const float* lse_a, const void* o_b,
                              const float* lse_b, void* o, float* lse, int64_t rows, int32_t heads,
                              int32_t dim, int32_t dtype, hipStream_t stream) {
  const int64_t total = rows * heads * (dim / 8);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (dtype == RPA_DTYPE_BF16)
    hipLaunchKernelGGL(merge_state_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(o_a), lse_a, static_cast<const bf16_t*>(o_b),
                       lse_b, static_cast<bf16_t*>(o), lse, rows, heads, dim);
  else
    hipLaunchKernelGGL(merge_state_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(o_a), lse_a, static_cast<const float*>(o_b),
                       lse_b, static_cast<float*>(o), lse, rows, heads, dim);
  return hipGetLastError();
}

}  // namespace rpa
