// Prefill-chunk attention (bf16, head dim 128, page size a multiple of 16):
// the MFMA-bound kernel.
//
// Prefill is compute bound ("Disaggregated prefill and decode", performance
// section), and a chunk of C new tokens attends to the cached prefix (a
// rectangle) and causally to itself (a triangle), as in the chunked-prefill
// post (sections "core-idea" and "correctness").
//
// One workgroup of four wavefronts takes a work item: request r, KV head g,
// up to 128 query rows (row = token * G + head-in-group, so the G query heads
// sharing a KV head sit in one tile and share its K/V loads), keys [k0, k1).
// Each wavefront owns 32 rows.  Keys stream in tiles of 64 through LDS:
//   S^T[key][row] = K[key][:] . Q[row][:]        mfma 32x32x16 bf16, A operand
//       read from LDS with ds_read_b128, Q resident in registers;
//   online softmax on S^T (each lane holds 16 keys of one row per 32-key block);
//   O^T[d][row] += V^T[d][key] . P^T[key][row]   mfma 32x32x16 bf16; the S^T
//       accumulators are already the P^T operand, and V^T is read from the
//       row-major V tile with the transposing LDS read.
// The next tile is loaded from HBM into registers while the current one is
// computed.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kKT = 64;        // keys per tile
constexpr int kKRow = 136;     // K tile row stride in LDS (elements): conflict-free b128 reads
constexpr int kVRow = 144;     // V tile row stride: conflict-free transposing reads
constexpr float kMinusBig = -1.0e30f;

}  // namespace

__global__ __launch_bounds__(256, 2) void prefill_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ kc,
                                                      const bf16_t* __restrict__ vc, Strides ks,
                                                      Strides vs, bf16_t* __restrict__ o,
                                                      float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) bf16_t klds[kKT * kKRow];
  __shared__ __attribute__((aligned(16))) bf16_t vlds[kKT * kVRow];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31;   // query row of this lane within the wave (S^T / O^T column)
  const int half = lane >> 5;  // k-slot group of the 32x32x16 operands

  const int32_t* it = p.items[KC_PREFILL] + (int64_t)blockIdx.x * IT_WORDS;
  const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], row0 = it[IT_ROW0], row1 = it[IT_ROW1];
  const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
  const int32_t G = p.group;
  const int32_t q0 = p.qo_indptr[r];
  const int32_t n = p.qo_indptr[r + 1] - q0;
  const int32_t L = p.kv_len[r];
  const int32_t cached = L - n;
  auto key_end = [&](int32_t row) {  // one past the last key row `row` may see in this item
    return min(k1, (p.causal ? cached + row / G : L - 1) + 1);
  };

  const int32_t row = row0 + wave * 32 + col;
  const bool row_ok = row < row1;
  const int32_t t = row_ok ? row / G : 0;
  const int32_t h = g * G + (row_ok ? row % G : 0);
  const int32_t kend_row = row_ok ? key_end(row) : k0;
  const int32_t kend = key_end(row1 - 1);
  const int32_t wrow0 = row0 + wave * 32;
  const bool wave_has_rows = wrow0 < row1;
  const int32_t kend_wmin = wave_has_rows ? key_end(wrow0) : k0;
  const int32_t kend_wmax = wave_has_rows ? key_end(min(row1, wrow0 + 32) - 1) : k0;

  // Q operand of the S^T products: qf[i] = Q[row][16 i + 8 half .. + 8).
  u32x4_t qf[8];
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kD + 8 * half;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qf[i] = row_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * i) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // Loader role: thread tid moves key tid / 4 of a tile, elements 32 (tid % 4) .. + 32.
  const int lkey = tid >> 2, lq = tid & 3;
  const int32_t* pages = p.page_indices + p.page_indptr[r];
  // Keys past k1 are loaded from the item's last key (always a valid slot) and
  // stored as zeros, so that 0 * value can never be NaN.  The zeroing happens
  // when the registers are written to LDS, a whole tile after the load was
  // issued, and page ids are fetched one tile ahead of the K/V loads, so that
  // nothing waits for a load in flight.
  u32x4_t kr0, kr1, kr2, kr3, vr0, vr1, vr2, vr3;
  const int64_t k_off = (int64_t)g * ks.head + 32 * lq;
  const int64_t v_off = (int64_t)g * vs.head + 32 * lq;
  auto page_of = [&](int32_t kb) {
    const int32_t key = min(kb + lkey, k1 - 1);
    return pages[key >> p.page_shift];
  };
#define RPA_LOAD_TILE(kb, pg_id)                                                              \
  do {                                                                                       \
    const int32_t kk_ = min((kb) + lkey, k1 - 1);                                            \
    const int64_t slot_ = kk_ & (p.page_size - 1);                                           \
    const u32x4_t* kp_ = reinterpret_cast<const u32x4_t*>(kc + (int64_t)(pg_id) * ks.page +   \
                                                          k_off + slot_ * ks.token);         \
    const u32x4_t* vp_ = reinterpret_cast<const u32x4_t*>(vc + (int64_t)(pg_id) * vs.page +   \
                                                          v_off + slot_ * vs.token);         \
    kr0 = kp_[0]; kr1 = kp_[1]; kr2 = kp_[2]; kr3 = kp_[3];                                  \
    vr0 = vp_[0]; vr1 = vp_[1]; vr2 = vp_[2]; vr3 = vp_[3];                                  \
  } while (0)

  const float sc = p.sm_scale * kLog2e;
  float m = kMinusBig;  // running row max, log2 units
  float lsum = 0.f;     // this lane's share of the running row sum
  f32x16_t oacc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;

  // Transposing-read source address of this lane inside a 16-key V chunk:
  // row 4 half + (lane % 16) / 4, column 16 (col / 16) + 4 (lane % 4).
  const int tr_row = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * (col >> 4) + 4 * (lane & 3);

  const int32_t ntiles = (kend - k0 + kKT - 1) / kKT;
  int32_t page_next = 0;
  if (ntiles > 0) {
    RPA_LOAD_TILE(k0, page_of(k0));
    if (ntiles > 1) page_next = page_of(k0 + kKT);
  }
  for (int32_t tile = 0; tile < ntiles; ++tile) {
    const int32_t kb = k0 + tile * kKT;
    __syncthreads();  // every wave is done reading the previous tile
    {
      const bool ok = kb + lkey < k1;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      u32x4_t* kd = reinterpret_cast<u32x4_t*>(&klds[lkey * kKRow + 32 * lq]);
      u32x4_t* vd = reinterpret_cast<u32x4_t*>(&vlds[lkey * kVRow + 32 * lq]);
      kd[0] = ok ? kr0 : z; kd[1] = ok ? kr1 : z; kd[2] = ok ? kr2 : z; kd[3] = ok ? kr3 : z;
      vd[0] = ok ? vr0 : z; vd[1] = ok ? vr1 : z; vd[2] = ok ? vr2 : z; vd[3] = ok ? vr3 : z;
    }
    if (tile + 1 < ntiles) {
      RPA_LOAD_TILE(kb + kKT, page_next);
      if (tile + 2 < ntiles) page_next = page_of(kb + 2 * kKT);
    }
    __syncthreads();  // tile visible
    if (!wave_has_rows || kb >= kend_wmax) continue;

    // S^T for the two 32-key blocks of the tile.
    f32x16_t sacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[b2][i] = 0.f;
      const bf16_t* krow = &klds[(32 * b2 + col) * kKRow + 8 * half];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + 16 * i);
        sacc[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[i]),
                                                           sacc[b2], 0, 0, 0);
      }
    }
    // Scale, mask and row max.  Element i of block b2 is key
    // kb + 32 b2 + 8 (i / 4) + 4 half + i % 4 of row `col`.
    const bool full = kb + kKT <= kend_wmin;  // every key of the tile visible to every row
    float mx = kMinusBig;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = sacc[b2][i] * sc;
        if (!full) {
          const int32_t key = kb + 32 * b2 + 8 * (i >> 2) + 4 * half + (i & 3);
          v = key < kend_row ? v : kMinusBig;
        }
        sacc[b2][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = sacc[b2][i];
        const float e = (full || v > 0.5f * kMinusBig) ? __builtin_amdgcn_exp2f(v - m_new) : 0.f;
        sacc[b2][i] = e;
        psum += e;
      }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) oacc[nb] *= alpha;

    // O^T += V^T P^T over the four 16-key chunks of the tile.
#pragma unroll
    for (int kc16 = 0; kc16 < 4; ++kc16) {
      const int b2 = kc16 >> 1, hb = kc16 & 1;
      u32x4_t pb;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pb[e] = pack_bf16x2(sacc[b2][8 * hb + 2 * e], sacc[b2][8 * hb + 2 * e + 1]);
      // key of k-slot (half, e) in this chunk: 16 kc16 + 8 (e / 4) + 4 half + e % 4
      const bf16_t* vsrc = &vlds[(16 * kc16 + tr_row) * kVRow + tr_col];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const s16x4_t lo = lds_read_tr16(vsrc + 32 * nb);
        const s16x4_t hi = lds_read_tr16(vsrc + 8 * kVRow + 32 * nb);
        const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
        const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t va = {lo2[0], lo2[1], hi2[0], hi2[1]};
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), oacc[nb],
                                                           0, 0, 0);
      }
    }
  }
#undef RPA_LOAD_TILE

  // Finish: the row sum is split over the two halves of the wave.
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (!row_ok) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse_nat = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  const int32_t i_tok = q0 + t;
  const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
  // Lane holds O^T[d][row] for d = 32 nb + 8 b + 4 half + j (element 4 b + j of block nb).
  if (S == 1) {
    bf16_t* orow = o + ((int64_t)i_tok * p.num_qo_heads + h) * kD + 4 * half;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t lo = pack_bf16x2(oacc[nb][4 * b] * inv, oacc[nb][4 * b + 1] * inv);
        const uint32_t hi = pack_bf16x2(oacc[nb][4 * b + 2] * inv, oacc[nb][4 * b + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * nb + 8 * b) = make_uint2(lo, hi);
      }
    if (half == 0 && lse) lse[(int64_t)i_tok * p.num_qo_heads + h] = lse_nat;
  } else {
    const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
    float* orow = p.part_o + (prow * p.num_qo_heads + h) * kD + 4 * half;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<float4*>(orow + 32 * nb + 8 * b) =
            make_float4(oacc[nb][4 * b] * inv, oacc[nb][4 * b + 1] * inv,
                        oacc[nb][4 * b + 2] * inv, oacc[nb][4 * b + 3] * inv);
    if (half == 0) p.part_lse[prow * p.num_qo_heads + h] = lse_nat;
  }
}

hipError_t launch_prefill(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream) {
  hipLaunchKernelGGL(prefill_kernel, dim3(p.n_items[KC_PREFILL]), dim3(256), 0, stream, p,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                     static_cast<const bf16_t*>(v_cache), ks, vs, static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
