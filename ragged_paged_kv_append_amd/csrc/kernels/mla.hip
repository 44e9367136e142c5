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
// One workgroup of eight wavefronts (two per SIMD) takes a work item of up
// to 128 query rows (row = token * G + head) and a key range; the planner
// packs the items onto one resident workgroup per compute unit, longest
// first.  Keys stream
// in tiles of 32 latent rows (36 KiB) through a three-slot LDS ring fed by the
// gfx950 global-to-LDS DMA (the next two tiles land while the current one is
// computed), each tile read from HBM once per item and used for both
// products.  In a latent row, 16-byte chunk c sits at position
// c ^ (row % 8), which keeps both LDS read patterns below conflict free.
//
// Per tile j:
//   S phase: wave w computes S^T for rows 16 w .. 16 w + 15 over the tile
//     (mfma 16x16x32 bf16, 18 steps over the 576 dims, Q of its rows resident
//     in registers), runs the online softmax for those rows and writes P (bf16)
//     and the per-row rescale factors into LDS;
//   PV phase: wave w owns value dims 64 w .. 64 w + 63 of all 128 rows and
//     accumulates O^T[d][row] += V^T[d][key] P^T[key][row] (mfma 32x32x16
//     bf16), V^T read from the latent tile with the transposing LDS read.
// A barrier separates the phases, and one more starts each tile.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kRows = 128;       // query rows per item
constexpr int kWaves = 8;
constexpr int kKT = 32;          // keys per tile
constexpr int kRowBytes = kDQK * 2;            // 1152
constexpr int kChunks = kDQK / 8;              // 72 chunks of 16 bytes per latent row
constexpr int kTileBytes = kKT * kRowBytes;    // 36864
constexpr int kSlots = 3;
constexpr int kDmaInst = kTileBytes / 1024;    // 36 DMA instructions of 1 KiB per tile
constexpr int kPRow = 36;                      // P row stride in LDS (bf16): 72 bytes
constexpr int kPBytes = kRows * kPRow * 2;     // 9216
constexpr float kMinusBig = -1.0e30f;
constexpr float kRescaleSlack = 8.f;           // log2 units

typedef __attribute__((address_space(3))) const bf16_t* lds_cptr_t;

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One global-to-LDS DMA instruction (gfx950 global_load_lds_dwordx4): every
// lane copies 16 bytes from `src` to LDS byte address lds + 16 * lane.  It is
// issued from inline assembly so that the compiler does not track it: left to
// itself the compiler makes every later LDS read wait for all DMA in flight,
// while the kernel waits for exactly the tile it needs (explicit vmcnt counts,
// which operations the compiler adds can only make stricter).  M0, which
// carries the LDS address, is saved and restored around the instruction.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Two transposing reads (low and high key halves, + 8 rows) at one address,
// with their own LDS wait (see the decode kernel: the compiler would
// otherwise drain the DMA stream before them).
__device__ __forceinline__ void read_vt2(uint32_t a, s16x4_t& lo, s16x4_t& hi) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(a), "n"(8 * kRowBytes)
      : "memory");
}

// The lane index as a value the compiler cannot see through: addresses
// derived from it are recomputed where they are used instead of being hoisted
// out of the tile loop (registers are fully used by Q and the O accumulators,
// and hoisted values would be spilled to scratch, whose reloads would also
// wait for the DMA stream).
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

}  // namespace

__global__ __launch_bounds__(512, 1) void mla_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                     const bf16_t* __restrict__ kvc, Strides ks,
                                                     bf16_t* __restrict__ o,
                                                     float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots][kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16_t plds[1][kRows * kPRow];
  __shared__ float alds[1][kRows];   // per-row rescale factor of the tile's P
  __shared__ float mlds[kRows];      // final row max (log2 units)
  __shared__ float llds[kRows];      // final row sum
  // Page ids of the current item's keys (the planner keeps an item within
  // MLA_MAX_KEYS keys, i.e. at most MLA_MAX_KEYS / 16 pages).
  __shared__ int32_t pglds[MLA_MAX_KEYS / 16];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)ring;

  // ---- S-phase role: rows 16 wave + scol ------------------------------------------
  const int scol = lane & 15, sgrp = lane >> 4;
  // K operand of step j (dims 32 j .. 32 j + 31) for key row scol of a
  // 16-key block: chunk 4 j + sgrp, at position (4 j + sgrp) ^ (scol % 8).
  // With j = 2 m + jj that is 8 m + ((4 jj + sgrp) ^ (scol % 8)).
  uint32_t k_rd[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
    k_rd[jj] = scol * kRowBytes + 16 * ((4 * jj + sgrp) ^ (scol & 7));
  // ---- PV-phase role: value dims 64 wave .. + 63, all rows ------------------------
  const int pcol = lane & 31, phalf = lane >> 5;
  const int tr_row = 4 * phalf + ((lane & 15) >> 2);  // (+ 8 for the high half)
  // Element column of block nb: 64 wave + 32 nb + 16 (pcol / 16) + 4 (lane % 4);
  // its chunk is 8 wave + 4 nb + tr_c.
  const int tr_c = 2 * (pcol >> 4) + ((lane & 3) >> 1);
  // ---- DMA role: instructions wave, wave + 8, ... of the tile's 36 -----------------
  // Instruction d moves chunks 64 d .. 64 d + 63 of the tile (72 chunks per
  // key row); lane L carries chunk 64 d + L into its LDS position, fetching
  // the global chunk (position) ^ (row % 8).
  const int n_dma = (kDmaInst - wave + kWaves - 1) / kWaves;  // 5 or 4

  const int32_t wb0 = p.wg_indptr[KC_MLA][blockIdx.x];
  const int32_t wb1 = p.wg_indptr[KC_MLA][blockIdx.x + 1];
  for (int32_t idx = wb0; idx < wb1; ++idx) {
    const int32_t* it = p.items[KC_MLA] + (int64_t)idx * IT_WORDS;
    const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], row0 = it[IT_ROW0], row1 = it[IT_ROW1];
    const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
    const int32_t G = p.group;
    const int32_t q0 = p.qo_indptr[r];
    const int32_t n = p.qo_indptr[r + 1] - q0;
    const int32_t L = p.kv_len[r];
    const int32_t cached = L - n;
    auto key_end = [&](int32_t row) __attribute__((always_inline)) {
      return min(k1, (p.causal ? cached + row / G : L - 1) + 1);
    };
    const int32_t kend = key_end(row1 - 1);
    const int32_t ntiles = (kend - k0 + kKT - 1) / kKT;

    const int32_t* pages = p.page_indices + p.page_indptr[r];
    const char* kvb = reinterpret_cast<const char*>(kvc + (int64_t)g * ks.head);
    // The item's page ids go to LDS once (coalesced), so a tile's DMA looks
    // them up there instead of waiting on a scalar load per tile.
    const int32_t pg0 = k0 >> p.page_shift;
    const int32_t npg = ((max(k1, k0 + 1) - 1) >> p.page_shift) - pg0 + 1;
    // DMA of the tile at key kb into ring slot `slot`.  Keys past k1 are
    // fetched from the item's last key (finite values; they are masked).  A
    // tile spans at most two pages (page size >= 16, tiles 32-aligned).
    // Row addresses are formed from two wave-uniform bases (keys kb and
    // kb + 16: the second half of a tile is in the same page for page sizes
    // >= 32, in the next one for 16) plus a 32-bit per-lane offset.
    struct DmaPlan {
      const char* base_a;
      const char* base_b;
      uint32_t rlim;  // last row of the tile that exists
      uint32_t lds;   // LDS byte address of the ring slot
    };
    auto dma_plan = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const int32_t klast = k1 - 1;
      const int32_t pa = __builtin_amdgcn_readfirstlane(
          pglds[(min(kb, klast) >> p.page_shift) - pg0]);
      const int32_t pb = __builtin_amdgcn_readfirstlane(
          pglds[(min(kb + 16, klast) >> p.page_shift) - pg0]);
      DmaPlan d;
      d.base_a = kvb + 2 * ((int64_t)pa * ks.page + (int64_t)(kb & (p.page_size - 1)) * ks.token);
      d.base_b =
          kvb + 2 * ((int64_t)pb * ks.page + (int64_t)((kb + 16) & (p.page_size - 1)) * ks.token);
      d.rlim = (uint32_t)(klast - kb);
      d.lds = ring_lds + slot * kTileBytes;
      return d;
    };
    // DMA instruction x (of this wave's n_dma) of a tile.
    auto dma_one = [&](const DmaPlan& d, int x) __attribute__((always_inline)) {
      const uint32_t tok2 = 2u * (uint32_t)ks.token;
      const uint32_t c = 64u * (wave + kWaves * x) + (uint32_t)opaque_lane(lane);  // < 2304
      const uint32_t kr = c / kChunks, cc = c - kr * kChunks;
      const uint32_t kq = min(kr, d.rlim);  // rows past the last key repeat it
      const uint32_t off = (kq & 15u) * tok2 + 16u * (cc ^ (kr & 7u));
      dma16((kq >= 16u ? d.base_b : d.base_a) + off,
            __builtin_amdgcn_readfirstlane(d.lds + 1024 * (wave + kWaves * x)));
    };
    auto issue = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const DmaPlan d = dma_plan(kb, slot);
#pragma unroll
      for (int x = 0; x < 5; ++x)
        if (x < n_dma) dma_one(d, x);
    };

    // S-phase rows of this wave.
    const int32_t srow = row0 + 16 * wave + scol;
    const bool srow_ok = srow < row1;
    const int32_t st = srow_ok ? srow / G : 0;
    const int32_t sh = g * G + (srow_ok ? srow % G : 0);
    const int32_t kend_row = srow_ok ? key_end(srow) : k0;
    const bool s_active_wave = row0 + 16 * wave < row1;
    const int32_t kend_wmin = s_active_wave ? key_end(row0 + 16 * wave) : k0;
    const int32_t kend_wmax = s_active_wave ? key_end(min(row1, row0 + 16 * wave + 16) - 1) : k0;
    const float sc = p.sm_scale * kLog2e;
    float m = kMinusBig, lsum = 0.f;

    f32x16_t oacc[2][4];  // [nb][rb]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][rb][i] = 0.f;

    barrier();  // the previous item's waves are done with the ring, P area and page table
    for (int32_t i = tid; i < npg; i += 64 * kWaves) pglds[i] = pages[pg0 + i];
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    barrier();  // the page table is in LDS
    if (ntiles > 0) issue(k0, 0);
    if (ntiles > 1) issue(k0 + kKT, 1);

    // Q operand: qf[j] = Q[srow][32 j + 8 sgrp .. + 8), loaded while the first
    // tiles are in flight.
    u32x4_t qf[kDQK / 32];
    {
      const bf16_t* qrow = q + ((int64_t)(q0 + st) * p.num_qo_heads + sh) * kDQK + 8 * sgrp;
#pragma unroll
      for (int j = 0; j < kDQK / 32; ++j)
        qf[j] = srow_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * j) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kDQK / 32; ++j) asm volatile("" ::"v"(qf[j]));
    }

    // S phase of the tile at key kb in `slot`: P and rescale factors into
    // P buffer `pbuf`.
    // With dma, this wave's DMA instructions of the tile at dkb (ring slot
    // dslot) are spread over the products, one after every second step.
    auto s_phase = [&](int32_t kb, int slot, int pbuf, bool dma, int32_t dkb, int dslot)
        __attribute__((always_inline)) {
      const bool active = s_active_wave && kb < kend_wmax;
      f32x4_t sacc[2];  // sacc[b][i] = S^T[key kb + 16 b + 4 sgrp + i][row scol]
#pragma unroll
      for (int b = 0; b < 2; ++b) sacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float alpha = 1.f;
      DmaPlan dp{};
      if (dma) dp = dma_plan(dkb, dslot);
      if (!active && dma) {
#pragma unroll
        for (int x = 0; x < 5; ++x)
          if (x < n_dma) dma_one(dp, x);
      }
      if (active) {
        const char* kt = reinterpret_cast<const char*>(&ring[slot][0]);
#pragma unroll
        for (int j = 0; j < kDQK / 32; ++j) {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kt + 16 * b * kRowBytes +
                                                                k_rd[j & 1] + 128 * (j >> 1));
            sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[j]),
                                                              sacc[b], 0, 0, 0);
          }
          if ((j & 1) && dma && (j >> 1) < n_dma) dma_one(dp, j >> 1);
          // Keep the compiler from hoisting all 36 K-operand reads: registers
          // are fully used by Q and the O accumulators.
          if (j & 1) __builtin_amdgcn_sched_barrier(0);
        }
        const bool full = kb + kKT <= kend_wmin;
        float mx = kMinusBig;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = sacc[b][i];
            if (!full) v = (kb + 16 * b + 4 * sgrp + i < kend_row) ? v : kMinusBig;
            sacc[b][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mt = mx > 0.5f * kMinusBig ? mx * sc : kMinusBig;
        if (mt > m + kRescaleSlack) {
          alpha = __builtin_amdgcn_exp2f(m - mt);
          lsum *= alpha;
          m = mt;
        }
        const float neg_m = -m;
        float psum = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = sacc[b][i];
            const float x =
                v > 0.5f * kMinusBig ? __builtin_amdgcn_exp2f(__builtin_fmaf(v, sc, neg_m)) : 0.f;
            sacc[b][i] = x;
            psum += x;
          }
        lsum += psum;
      }
      // P[row][key 16 b + 4 sgrp + i] and the row's rescale factor.
      bf16_t* prow = &plds[pbuf][(16 * wave + scol) * kPRow + 4 * sgrp];
#pragma unroll
      for (int b = 0; b < 2; ++b)
        *reinterpret_cast<uint2*>(prow + 16 * b) =
            make_uint2(pack_bf16x2(sacc[b][0], sacc[b][1]), pack_bf16x2(sacc[b][2], sacc[b][3]));
      if (sgrp == 0) alds[pbuf][16 * wave + scol] = alpha;
    };

    // PV phase of the tile in `slot` with P buffer `pbuf`.
    auto pv_phase = [&](int slot, int pbuf) __attribute__((always_inline)) {
      const int ln = opaque_lane(lane);
      const int pcol = ln & 31, phalf = ln >> 5;
      const int tr_row = 4 * phalf + ((ln & 15) >> 2);
      const int tr_c = 2 * (pcol >> 4) + ((ln & 3) >> 1);
      // Rescale the rows whose reference max was raised with this tile.
      float a[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[rb] = alds[pbuf][32 * rb + pcol];
      if (__ballot(a[0] != 1.f || a[1] != 1.f || a[2] != 1.f || a[3] != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) oacc[nb][rb] *= a[rb];
      }
      const uint32_t slot_lds = ring_lds + slot * kTileBytes;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4_t va[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          s16x4_t lo, hi;
          const int R = 16 * kc + tr_row;
          read_vt2(slot_lds + R * kRowBytes + 16 * ((8 * wave + 4 * nb + tr_c) ^ (R & 7)) +
                       8 * (ln & 1),
                   lo, hi);
          const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
          va[nb] = u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
        }
        // P^T operand of row block rb: row 32 rb + pcol, keys
        // 16 kc + 8 (e / 4) + 4 phalf + e % 4.
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const bf16_t* prow = &plds[pbuf][(32 * rb + pcol) * kPRow + 16 * kc + 4 * phalf];
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(prow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(prow + 8);
          const u32x4_t pbv = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            oacc[nb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[nb]),
                                                                   as_bf16x8(pbv), oacc[nb][rb],
                                                                   0, 0, 0);
        }
      }
    };

    // Step j: [wait for tile j] barrier [DMA of tile j + 2] [S of tile j]
    // barrier [PV of tile j].  The first barrier publishes tile j and frees
    // the ring slot of tile j - 1 and the P area; the second publishes P.
    // Two tiles (72 KiB) are in flight while one is computed.
    for (int32_t tile = 0, slot = 0; tile < ntiles; ++tile, slot = (slot == kSlots - 1) ? 0 : slot + 1) {
      if (tile + 1 < ntiles) {
        if (n_dma == 5) wait_vmem<5>(); else wait_vmem<4>();  // tile j + 1 may be in flight
      } else {
        wait_vmem<0>();
      }
      barrier();
      s_phase(k0 + tile * kKT, slot, 0, tile + 2 < ntiles, k0 + (tile + 2) * kKT,
              slot == 0 ? kSlots - 1 : slot - 1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's P is in LDS
      barrier();
      pv_phase(slot, 0);
    }

    // Row statistics from the S-phase owners, then every wave stores its dims.
    float ltot = lsum + __shfl_xor(lsum, 16, 64);
    ltot += __shfl_xor(ltot, 32, 64);
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
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int lrow = 32 * rb + pcol;
      const int32_t row = row0 + lrow;
      if (row >= row1) continue;
      const int32_t t = row / G, h = g * G + row % G;
      const float lt = llds[lrow];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      // Lane holds O^T[d][row] for d = 64 wave + 32 nb + 8 b + 4 phalf + j.
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x16_t& acc = oacc[nb][rb];
        if (S == 1) {
          bf16_t* orow = o + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kDV + 64 * wave + 32 * nb +
                         4 * phalf;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            *reinterpret_cast<uint2*>(orow + 8 * b) =
                make_uint2(pack_bf16x2(acc[4 * b] * inv, acc[4 * b + 1] * inv),
                           pack_bf16x2(acc[4 * b + 2] * inv, acc[4 * b + 3] * inv));
        } else {
          const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
          float* orow = p.part_o + (prow * p.num_qo_heads + h) * kDV + 64 * wave + 32 * nb + 4 * phalf;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            *reinterpret_cast<float4*>(orow + 8 * b) =
                make_float4(acc[4 * b] * inv, acc[4 * b + 1] * inv, acc[4 * b + 2] * inv,
                            acc[4 * b + 3] * inv);
        }
      }
    }
  }
}

hipError_t launch_mla(const DevPlan& p, const void* q, const void* kv_cache, Strides ks, void* o,
                      float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(mla_kernel, dim3(p.n_wgs[KC_MLA]), dim3(64 * kWaves), 0, stream, p,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kv_cache), ks,
                     static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
