// Absorbed latent attention (bf16, one latent KV head, key dim 576 = 512 latent
// + 64 rope, value = the first 512 latent dims, page size a multiple of 16).
//
// "Disaggregated prefill and decode" (deployment section) describes the
// latent cache: every KV head is compressed into one latent vector per token,
// so all query heads read the same cache rows.  With 128 query heads and two
// query tokens per request (MTP verify, "Accelerating Sonar through
// speculation"), each latent row is used by 256 query rows: the work is bound
// by the matrix cores, not by HBM.
//
// One workgroup (four wavefronts) takes 64 query rows (row = token * G +
// head) and a key range.  Keys stream in tiles of 32 latent rows (36 KiB)
// through LDS, read once from HBM and used for both products:
//   S phase: wavefront w computes S^T for rows 16 w .. 16 w + 15 over the
//     tile (mfma 16x16x32 bf16, 18 steps over the 576 dims, Q of its rows
//     resident in registers), runs the online softmax for those rows and
//     writes P (bf16) and the rescale factors to LDS;
//   PV phase: wavefront w owns value dims 128 w .. 128 w + 127 of all 64 rows
//     and accumulates O^T[d][row] += V^T[d][key] P^T[key][row] (mfma
//     32x32x16 bf16), V^T read from the same latent tile with the transposing
//     LDS read.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kRows = 64;    // query rows per workgroup
constexpr int kKT = 32;      // keys per tile
constexpr int kKRow = 584;   // latent tile row stride in LDS (elements)
constexpr int kPRow = 36;    // P tile row stride in LDS (elements), [row][key]
constexpr int kChunks = kDQK / 8;  // 16-byte chunks per latent row
constexpr float kMinusBig = -1.0e30f;

}  // namespace

__global__ __launch_bounds__(256) void mla_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                  const bf16_t* __restrict__ kvc, Strides ks,
                                                  bf16_t* __restrict__ o,
                                                  float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) bf16_t klds[kKT * kKRow];
  __shared__ __attribute__((aligned(16))) bf16_t plds[kRows * kPRow];
  __shared__ float alds[kRows];
  __shared__ float mlds[kRows];
  __shared__ float llds[kRows];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  const int32_t* it = p.items[KC_MLA] + (int64_t)blockIdx.x * IT_WORDS;
  const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], row0 = it[IT_ROW0], row1 = it[IT_ROW1];
  const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
  const int32_t G = p.group;
  const int32_t q0 = p.qo_indptr[r];
  const int32_t n = p.qo_indptr[r + 1] - q0;
  const int32_t L = p.kv_len[r];
  const int32_t cached = L - n;
  auto key_end = [&](int32_t row) {
    return min(k1, (p.causal ? cached + row / G : L - 1) + 1);
  };
  const int32_t kend = key_end(row1 - 1);

  // ---- S-phase role: rows 16 wave + (lane % 16) -------------------------------------
  const int scol = lane & 15, sgrp = lane >> 4;
  const int32_t srow = row0 + 16 * wave + scol;
  const bool srow_ok = srow < row1;
  const int32_t st = srow_ok ? srow / G : 0;
  const int32_t sh = g * G + (srow_ok ? srow % G : 0);
  const int32_t kend_row = srow_ok ? key_end(srow) : k0;
  u32x4_t qf[kDQK / 32];  // qf[j] = Q[srow][32 j + 8 sgrp .. + 8)
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + st) * p.num_qo_heads + sh) * kDQK + 8 * sgrp;
#pragma unroll
    for (int j = 0; j < kDQK / 32; ++j)
      qf[j] = srow_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const float sc = p.sm_scale * kLog2e;
  float m = kMinusBig, lsum = 0.f;

  // ---- PV-phase role: value dims 128 wave .. + 127, all rows -------------------------
  const int pcol = lane & 31, phalf = lane >> 5;
  f32x16_t oacc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[nb][rb][i] = 0.f;
  const int tr_row = 4 * phalf + ((lane & 15) >> 2);
  const int tr_col = 128 * wave + 16 * (pcol >> 4) + 4 * (lane & 3);

  const int32_t* pages = p.page_indices + p.page_indptr[r];
  const int32_t ntiles = (kend - k0 + kKT - 1) / kKT;
  for (int32_t tile = 0; tile < ntiles; ++tile) {
    const int32_t kb = k0 + tile * kKT;
    __syncthreads();  // previous tile and P fully consumed
    // Latent tile: 32 rows x 72 chunks of 16 bytes; keys past k1 become zeros.
#pragma unroll
    for (int j = 0; j < (kKT * kChunks) / 256; ++j) {
      const int c = tid + 256 * j;
      const int key = c / kChunks, ch = c - key * kChunks;
      const int32_t kk = kb + key;
      const bool ok = kk < k1;
      const int32_t kkc = ok ? kk : k1 - 1;
      const int64_t page = pages[kkc >> p.page_shift];
      const int64_t slot = kkc & (p.page_size - 1);
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(kvc + page * ks.page + (int64_t)g * ks.head +
                                                    slot * ks.token + 8 * ch);
      if (!ok) v = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(&klds[key * kKRow + 8 * ch]) = v;
    }
    __syncthreads();

    // S phase.  sacc[b][i] = S^T[key 16 b + 4 sgrp + i][row scol].
    f32x4_t sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const bf16_t* krow = &klds[(16 * b + scol) * kKRow + 8 * sgrp];
#pragma unroll
      for (int j = 0; j < kDQK / 32; ++j) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + 32 * j);
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[j]), sacc[b],
                                                          0, 0, 0);
      }
    }
    float mx = kMinusBig;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t key = kb + 16 * b + 4 * sgrp + i;
        const float v = key < kend_row ? sacc[b][i] * sc : kMinusBig;
        sacc[b][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = sacc[b][i] > 0.5f * kMinusBig ? __builtin_amdgcn_exp2f(sacc[b][i] - m_new) : 0.f;
        psum += e[i];
      }
      *reinterpret_cast<uint2*>(&plds[(16 * wave + scol) * kPRow + 16 * b + 4 * sgrp]) =
          make_uint2(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]));
    }
    lsum = lsum * alpha + psum;
    m = m_new;
    if (sgrp == 0) alds[16 * wave + scol] = alpha;
    __syncthreads();

    // PV phase.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float a = alds[32 * rb + pcol];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) oacc[nb][rb] *= a;
    }
#pragma unroll
    for (int kc16 = 0; kc16 < 2; ++kc16) {
      // P^T operand: row 32 rb + pcol, keys 16 kc16 + 8 (e / 4) + 4 phalf + e % 4.
      u32x4_t pb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16_t* prow = &plds[(32 * rb + pcol) * kPRow + 16 * kc16 + 4 * phalf];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(prow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(prow + 8);
        pb[rb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
      const bf16_t* vsrc = &klds[(16 * kc16 + tr_row) * kKRow + tr_col];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, lds_read_tr16(vsrc + 32 * nb));
        const u32x2_t hi = __builtin_bit_cast(u32x2_t, lds_read_tr16(vsrc + 8 * kKRow + 32 * nb));
        const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          oacc[nb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb[rb]),
                                                                 oacc[nb][rb], 0, 0, 0);
      }
    }
  }

  // Row statistics from the S-phase owners, then every wave stores its dims.
  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  __syncthreads();
  if (sgrp == 0) {
    mlds[16 * wave + scol] = m;
    llds[16 * wave + scol] = ltot;
  }
  const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
  if (sgrp == 0 && srow_ok) {
    const float lse_nat = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
    if (S == 1) {
      if (lse) lse[(int64_t)(q0 + st) * p.num_qo_heads + sh] = lse_nat;
    } else {
      const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + st;
      p.part_lse[prow * p.num_qo_heads + sh] = lse_nat;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int lrow = 32 * rb + pcol;
    const int32_t row = row0 + lrow;
    if (row >= row1) continue;
    const int32_t t = row / G, h = g * G + row % G;
    const float lt = llds[lrow];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // Lane holds O^T[d][row] for d = 128 wave + 32 nb + 8 b + 4 phalf + j.
    if (S == 1) {
      bf16_t* orow = o + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kDV + 128 * wave + 4 * phalf;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x16_t& a = oacc[nb][rb];
          *reinterpret_cast<uint2*>(orow + 32 * nb + 8 * b) =
              make_uint2(pack_bf16x2(a[4 * b] * inv, a[4 * b + 1] * inv),
                         pack_bf16x2(a[4 * b + 2] * inv, a[4 * b + 3] * inv));
        }
    } else {
      const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
      float* orow = p.part_o + (prow * p.num_qo_heads + h) * kDV + 128 * wave + 4 * phalf;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x16_t& a = oacc[nb][rb];
          *reinterpret_cast<float4*>(orow + 32 * nb + 8 * b) =
              make_float4(a[4 * b] * inv, a[4 * b + 1] * inv, a[4 * b + 2] * inv,
                          a[4 * b + 3] * inv);
        }
    }
  }
}

hipError_t launch_mla(const DevPlan& p, const void* q, const void* kv_cache, Strides ks, void* o,
                      float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(mla_kernel, dim3(p.n_items[KC_MLA]), dim3(256), 0, stream, p,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kv_cache), ks,
                     static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
