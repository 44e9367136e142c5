// Decode / speculative-verify attention (bf16, head dim 128, page size a
// multiple of 16): the HBM-streaming kernel.
//
// The disaggregation post (prefill/decode performance section) notes that
// decode is memory bound: a few query rows per KV head read the whole KV
// range.  One wavefront takes one work item: request r, KV head g, all of its
// n_r * G query rows (at most 16: decode rows and verify rows of n + 1 draft
// tokens, "Accelerating Sonar through speculation"), keys [k0, k1).  The item
// streams its keys in tiles of 16 tokens (one page head slice for P = 16, a
// quarter page for P = 64), so every tile is one contiguous 4 KiB run of K and
// one of V in the HND layout.
//
// Per tile, with 16x16 MFMA tiles and query rows padded to 16:
//   S^T[key][row] = K[key][:] . Q[row][:]      4 x mfma 16x16x32 bf16; the K
//       tile goes from HBM straight into the A operand (each lane loads 64
//       contiguous bytes of one key row);
//   online softmax on S^T: each lane holds 4 keys of one query row;
//   O^T[d][row] += V^T[d][keys] . P^T[keys][row]   8 x mfma 16x16x16 bf16; the
//       S^T accumulator layout is exactly the B operand layout of P^T, so P
//       never moves between lanes; V goes through LDS to be read per column.
// The next tile's K and V are loaded while the current one is computed.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kTile = 16;
// LDS row stride of a V tile (bf16): 288 bytes keeps rows 16-byte aligned and
// puts rows 4g .. 4g+3 (read together by one transposing read) in distinct banks.
constexpr int kVRow = 144;
constexpr float kMinusBig = -1.0e30f;

struct Frag64 {  // 64 contiguous bytes of one row: 32 bf16
  u32x4_t v[4];
};

__device__ __forceinline__ void load_frag(const bf16_t* p, Frag64& f) {
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) f.v[k] = __builtin_nontemporal_load(s + k);
}

}  // namespace

__global__ __launch_bounds__(64) void decode_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                    const bf16_t* __restrict__ kc,
                                                    const bf16_t* __restrict__ vc, Strides ks,
                                                    Strides vs, bf16_t* __restrict__ o,
                                                    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) bf16_t vlds[2][kTile * kVRow];
  const int lane = threadIdx.x;
  const int col = lane & 15;  // query row of S^T / P^T / O^T columns; key row of the K operand
  const int grp = lane >> 4;  // which 32-element quarter of a row this lane loads

  const int32_t* it = p.items[KC_DECODE] + (int64_t)blockIdx.x * IT_WORDS;
  const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], rows = it[IT_ROW1];
  const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
  const int32_t G = p.group;
  const int32_t q0 = p.qo_indptr[r];
  const int32_t n = p.qo_indptr[r + 1] - q0;
  const int32_t L = p.kv_len[r];
  const int32_t cached = L - n;

  // This lane's query row (as a column of S^T).
  const bool row_ok = col < rows;
  const int32_t t = row_ok ? col / G : 0;
  const int32_t h = g * G + (row_ok ? col % G : 0);
  const int32_t kend_row = row_ok ? min(k1, (p.causal ? cached + t : L - 1) + 1) : k0;
  const int32_t t_last = (rows - 1) / G;
  const int32_t kend = min(k1, (p.causal ? cached + t_last : L - 1) + 1);

  Frag64 qf;
  if (row_ok) {
    load_frag(q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kD + 32 * grp, qf);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) qf.v[k] = u32x4_t{0u, 0u, 0u, 0u};
  }

  const int32_t* pages = p.page_indices + p.page_indptr[r];
  const int64_t k_head = (int64_t)g * ks.head + (int64_t)col * ks.token + 32 * grp;
  const int64_t v_head = (int64_t)g * vs.head + (int64_t)col * vs.token + 32 * grp;
  auto k_ptr = [&](int32_t kb) {
    const int64_t page = pages[kb >> p.page_shift];
    return kc + page * ks.page + (int64_t)(kb & (p.page_size - 1)) * ks.token + k_head;
  };
  auto v_ptr = [&](int32_t kb) {
    const int64_t page = pages[kb >> p.page_shift];
    return vc + page * vs.page + (int64_t)(kb & (p.page_size - 1)) * vs.token + v_head;
  };

  const float sc = p.sm_scale * kLog2e;
  float m = kMinusBig;  // running max of this row, log2 units
  float lsum = 0.f;     // this lane's share of the running sum (its 4 keys per tile)
  f32x4_t acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t ntiles = (kend - k0 + kTile - 1) / kTile;
  Frag64 kf, vf, kf_next, vf_next;
  if (ntiles > 0) {
    load_frag(k_ptr(k0), kf);
    load_frag(v_ptr(k0), vf);
  }
  for (int32_t tile = 0; tile < ntiles; ++tile) {
    const int32_t kb = k0 + tile * kTile;
    if (tile + 1 < ntiles) {
      load_frag(k_ptr(kb + kTile), kf_next);
      load_frag(v_ptr(kb + kTile), vf_next);
    }
    // Stage V in LDS; keys past k1 (outside the item, possibly unwritten
    // slots) become zeros so that 0 * value can never be NaN.
    {
      bf16_t* dst = &vlds[tile & 1][col * kVRow + 32 * grp];
      const bool key_ok = kb + col < k1;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<u32x4_t*>(dst + 8 * k) = key_ok ? vf.v[k] : u32x4_t{0u, 0u, 0u, 0u};
    }
    // S^T = K . Q^T
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf.v[k]), as_bf16x8(qf.v[k]), sacc,
                                                     0, 0, 0);
    // Online softmax for query row `col`; this lane holds keys kb + 4*grp + e.
    float sv[4];
    float mx = kMinusBig;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = kb + 4 * grp + e < kend_row;
      sv[e] = ok ? sacc[e] * sc : kMinusBig;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float pv[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] = sv[e] > 0.5f * kMinusBig ? __builtin_amdgcn_exp2f(sv[e] - m_new) : 0.f;
      psum += pv[e];
    }
    lsum = lsum * alpha + psum;
    m = m_new;
    s16x4_t pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[e] = (short)f32_to_bf16(pv[e]);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[nb] *= alpha;

    __syncthreads();  // V tile visible to every lane of the wave
    // V^T operand of block nb: lane (d = 16 nb + col, group grp) needs
    // V[4 grp + e][d], e = 0..3.  With the transposing read, lane i of the
    // group supplies row 4 grp + i / 4, columns 16 nb + 4 (i % 4) .. + 3.
    const bf16_t* vt = &vlds[tile & 1][(4 * grp + (col >> 2)) * kVRow + 4 * (col & 3)];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const s16x4_t va = lds_read_tr16(vt + 16 * nb);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[nb], 0, 0, 0);
    }
    if (tile + 1 < ntiles) {
      kf = kf_next;
      vf = vf_next;
    }
  }

  // Row sum over the four lane groups, then normalise and store.
  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (!row_ok) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse_nat = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  const int32_t i = q0 + t;
  const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
  if (S == 1) {
    bf16_t* orow = o + ((int64_t)i * p.num_qo_heads + h) * kD + 4 * grp;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[nb][0] * inv) |
                          ((uint32_t)f32_to_bf16(acc[nb][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[nb][2] * inv) |
                          ((uint32_t)f32_to_bf16(acc[nb][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * nb) = make_uint2(lo, hi);
    }
    if (grp == 0 && lse) lse[(int64_t)i * p.num_qo_heads + h] = lse_nat;
  } else {
    const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
    float* orow = p.part_o + (prow * p.num_qo_heads + h) * kD + 4 * grp;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<float4*>(orow + 16 * nb) =
          make_float4(acc[nb][0] * inv, acc[nb][1] * inv, acc[nb][2] * inv, acc[nb][3] * inv);
    if (grp == 0) p.part_lse[prow * p.num_qo_heads + h] = lse_nat;
  }
}

hipError_t launch_decode(const DevPlan& p, const void* q, const void* k_cache, const void* v_cache,
                         Strides ks, Strides vs, void* o, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3(p.n_items[KC_DECODE]), dim3(64), 0, stream, p,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                     static_cast<const bf16_t*>(v_cache), ks, vs, static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
