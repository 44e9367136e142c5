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
// One workgroup of four wavefronts (one per SIMD, so each wave has the whole
// 512-entry register file: Q of its rows in VGPRs, its O accumulators in
// AGPRs) takes a work item of up to 128 query rows (row = token * G + head)
// and a key range; the planner packs the items onto one resident workgroup
// per compute unit, longest first.  Keys stream in tiles of 32 latent rows
// through a two-slot LDS ring fed by the gfx950 global-to-LDS DMA (the next
// tile lands while the current one is computed), each tile read from HBM
// once per item and used for both products.  A latent row takes 73 chunks of
// 16 bytes in LDS (72 of data and one of padding), which keeps the K-operand
// reads (16 rows, one chunk each) and the transposing V reads conflict free.
//
// Per tile j:
//   S phase: wave w computes S^T for rows 32 w .. 32 w + 31 over the tile as
//     four independent 16x16 blocks (mfma 16x16x32 bf16, 18 steps over the
//     576 dims, K operands read three steps ahead), runs the softmax for
//     those rows against their reference max (moved only far above it: see
//     the tile loop) and writes P (bf16) into LDS;
//   PV phase: wave w owns value dims 128 w .. 128 w + 127 of all 128 rows and
//     accumulates O^T[d][row] += V^T[d][key] P^T[key][row] (mfma 32x32x16
//     bf16), V^T read from the latent tile with the transposing LDS read.
// Each wave's share of the DMA of tile j + 1 is issued one instruction at a
// time between the first S products.
// A barrier separates the phases, and one more starts each tile.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kRows = 128;       // query rows per item
constexpr int kWaves = 4;
constexpr int kKT = 32;          // keys per tile
constexpr int kChunks = kDQK / 8;              // 72 data chunks of 16 bytes per latent row
constexpr int kRowChunks = kChunks + 1;        // 73 with the padding chunk
constexpr int kRowBytes = 16 * kRowChunks;     // 1168
constexpr int kDmaInst = (kKT * kRowChunks + 63) / 64;  // 37 DMA instructions of 1 KiB per tile
constexpr int kTileBytes = 1024 * kDmaInst;    // 37888 (the last instruction's tail is slack)
constexpr int kSlots = 2;
constexpr int kSteps = kDQK / 32;              // 18 steps of 32 dims per S tile
constexpr int kAhead = 3;                      // steps of K-operand reads in flight
constexpr int kPRow = 36;                      // P row stride in LDS (bf16): 72 bytes
constexpr float kMinusBig = -1.0e30f;
// A row's reference max only moves when a tile beats it by more than this
// (log2 units); P then stays below 2^64 and O below 2^79 |V|max (keys per item
// <= 2^15), far inside fp32 range.
constexpr float kRestartSlack = 64.f;

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
// carries the LDS address, is saved and restored around the instruction; the
// DMA reads M0 one wait state after the write that sets it.  No non-temporal
// hint: the workgroup paired on the same XCD reads the same lines from L2.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// The same DMA with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// offset (the saddr form: no per-lane address arithmetic).  The base usually
// comes straight from v_readfirstlane, and a memory instruction reads an SGPR
// that a VALU instruction wrote only five wait states later: s_nop 4 first.
__device__ __forceinline__ void dma16_base(const void* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// The lane index as a value the compiler cannot see through: addresses
// derived from it are recomputed where they are used instead of being hoisted
// out of the tile loop and kept in registers for the whole item.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// The S products are issued from inline assembly so that their accumulators
// stay in VGPRs (the compiler puts every matrix-core result of a kernel that
// uses AGPRs into AGPRs, and the O accumulators already fill them).  A chain
// of products on one accumulator needs no wait states between its links;
// s_wait_products covers the results' latency before any other instruction
// touches the accumulators.
__device__ __forceinline__ void mfma16_first(f32x4_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16(f32x4_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void s_wait_products(f32x4_t (&acc)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_kernel(
    DevPlan p, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kvc, Strides ks,
    bf16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots][kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16_t plds[kRows * kPRow];
  __shared__ int32_t restart;     // set when a tile moved a row's reference max
  __shared__ float llds[kRows];   // final row sum
  // Page ids of the current item's keys (the planner keeps an item within
  // MLA_MAX_KEYS keys, i.e. at most MLA_MAX_KEYS / 16 pages).
  __shared__ int32_t pglds[MLA_MAX_KEYS / 16];
  // Per-thread byte offsets (from the tile's first key) of this thread's DMA
  // chunks, x = 0..9, for a tile of 32 keys in one page.
  __shared__ uint32_t doff[10][64 * kWaves];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t ring_lds =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)ring;

  // ---- S-phase role: rows 32 wave + 16 rb + kq, keys 16 kb + 4 kg + i -------------
  const int kq = lane & 15, kg = lane >> 4;
  // ---- PV-phase role: value dims 128 wave .. + 127, all rows -----------------------
  const int pcol = lane & 31, phalf = lane >> 5;
  // ---- DMA role: instructions wave, wave + 4, ... of the tile's 37 -----------------
  // Instruction d fills LDS chunk positions 64 d .. 64 d + 63 of the slot;
  // position c is chunk c % 73 of key row c / 73 (chunk 72 is padding and
  // takes a copy of chunk 71; positions past the 32 rows are slack).
  const int n_dma = (kDmaInst - wave + kWaves - 1) / kWaves;  // 10 or 9
  {
    const uint32_t tok2 = 2u * (uint32_t)ks.token;
#pragma unroll
    for (int x = 0; x < 10; ++x) {
      const uint32_t c = 64u * (wave + kWaves * x) + (uint32_t)lane;
      const uint32_t kr = c / kRowChunks, cc = min(c - kr * kRowChunks, (uint32_t)kChunks - 1);
      doff[x][tid] = kr < (uint32_t)kKT ? kr * tok2 + 16u * cc : 0u;
    }
  }

  const int32_t wb0 = p.wg_indptr[KC_MLA][blockIdx.x];
  const int32_t wb1 = p.wg_indptr[KC_MLA][blockIdx.x + 1];
  // References kept when an item starts over (see the tile loop).
  float m_keep[2] = {kMinusBig, kMinusBig};
  bool again = false;
  for (int32_t idx = wb0; idx < wb1;) {
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
    // tile spans at most two pages (page size >= 16, tiles 32-aligned): row
    // addresses are formed from two wave-uniform bases (keys kb and kb + 16:
    // the second half of a tile is in the same page for page sizes >= 32, in
    // the next one for 16) plus a 32-bit per-lane offset.
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
      const uint32_t c = 64u * (wave + kWaves * x) + (uint32_t)opaque_lane(lane);  // < 2368
      const uint32_t kr = c / kRowChunks, cc = min(c - kr * kRowChunks, (uint32_t)kChunks - 1);
      const uint32_t kq = min(kr, d.rlim);  // rows past the last key (or the slot) repeat it
      const uint32_t off = (kq & 15u) * tok2 + 16u * cc;
      dma16((kq >= 16u ? d.base_b : d.base_a) + off,
            __builtin_amdgcn_readfirstlane(d.lds + 1024 * (wave + kWaves * x)));
    };
    auto issue = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const DmaPlan d = dma_plan(kb, slot);
#pragma unroll
      for (int x = 0; x < 10; ++x)
        if (x < n_dma) dma_one(d, x);
    };

    // S-phase rows of this lane (rb = 0, 1).
    int32_t st[2], sh[2], kend_row[2];
    bool srow_ok[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int32_t srow = row0 + 32 * wave + 16 * rb + kq;
      srow_ok[rb] = srow < row1;
      st[rb] = srow_ok[rb] ? srow / G : 0;
      sh[rb] = g * G + (srow_ok[rb] ? srow % G : 0);
      kend_row[rb] = srow_ok[rb] ? key_end(srow) : k0;
    }
    const bool s_active_wave = row0 + 32 * wave < row1;
    const int32_t kend_wmin = s_active_wave ? key_end(row0 + 32 * wave) : k0;
    const int32_t kend_wmax = s_active_wave ? key_end(min(row1, row0 + 32 * wave + 32) - 1) : k0;
    const float sc = p.sm_scale * kLog2e;
    float m[2] = {again ? m_keep[0] : kMinusBig, again ? m_keep[1] : kMinusBig};
    float lsum[2] = {0.f, 0.f};

    f32x16_t oacc[4][4];  // [nb][rb]: O^T[dims 128 wave + 32 nb ..][rows 32 rb ..]
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][rb][i] = 0.f;

    barrier();  // the previous item's waves are done with the ring, P area and page table
    for (int32_t i = tid; i < npg; i += 64 * kWaves) pglds[i] = pages[pg0 + i];
    if (tid == 0) restart = 0;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    barrier();  // the page table is in LDS
    if (ntiles > 0) issue(k0, 0);

    // Q operand: qf[rb][j] = Q[row 32 wave + 16 rb + kq][32 j + 8 kg .. + 8),
    // loaded while the first tiles are in flight.
    u32x4_t qf[2][kSteps];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bf16_t* qrow =
          q + ((int64_t)(q0 + st[rb]) * p.num_qo_heads + sh[rb]) * kDQK + 8 * kg;
#pragma unroll
      for (int j = 0; j < kSteps; ++j)
        qf[rb][j] = srow_ok[rb] ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * j)
                                : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < kSteps; ++j) asm volatile("" ::"v"(qf[rb][j]));

    // DMA of the next tile, one instruction after each of the first S steps.
    // Issuing it stalls the wave while many transfers are outstanding, so the
    // ring holds two slots and keeps one tile in flight, which covers the
    // memory latency.  A tile of 32 existing keys in one page (page size
    // >= 32) takes the table offsets and one SGPR base; other tiles clamp rows
    // per lane.
    bool dma_on = false, dma_fast = false;
    int32_t dma_kb = 0;
    int32_t dma_pid = 0;
    uint32_t dma_off = 0, dma_lds = 0;
    const char* dma_base = nullptr;
    DmaPlan dma_dp{};
    auto dma_begin = [&](bool on, int32_t kb, int slot) __attribute__((always_inline)) {
      dma_on = on;
      dma_kb = kb;
      dma_fast = on && p.page_size >= 2 * 16 && kb + kKT <= k1;
      if (on && !dma_fast) dma_dp = dma_plan(kb, slot);
      if (dma_fast) {
        dma_pid = pglds[(kb >> p.page_shift) - pg0];
        dma_off = doff[0][tid];
      }
      dma_lds = ring_lds + slot * kTileBytes + 1024 * wave;
    };
    auto dma_x = [&](int x) __attribute__((always_inline)) {
      if (!dma_on || x >= n_dma) return;
      if (dma_fast) {
        if (x == 0)
          dma_base = kvb + 2 * ((int64_t)__builtin_amdgcn_readfirstlane(dma_pid) * ks.page +
                                (int64_t)(dma_kb & (p.page_size - 1)) * ks.token);
        // (readfirstlane returns int: widen through uint32_t, not by sign)
        const uint64_t b = reinterpret_cast<uint64_t>(dma_base);
        const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
        const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
        const uint64_t bu = ((uint64_t)b_hi << 32) | (uint64_t)b_lo;
        dma16_base(reinterpret_cast<const void*>(bu), dma_off,
                   __builtin_amdgcn_readfirstlane(dma_lds + 1024 * kWaves * x));
        if (x + 1 < 10) dma_off = doff[x + 1][tid];
      } else {
        dma_one(dma_dp, x);
      }
    };

    // S phase of the tile at key kb in `slot`, with this wave's DMA of the
    // next tile between its first products.
    auto s_phase = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const bool active = s_active_wave && kb < kend_wmax;
      // sacc[kb][rb][i] = S^T[key kb + 16 kb + 4 kg + i][row 16 rb + kq]
      f32x4_t sacc[2][2];
      bool moved = false;
      if (!active) {
#pragma unroll
        for (int x = 0; x < 10; ++x) dma_x(x);
      }
      if (active) {
        // K operand of step j, key block b: key 16 b + kq, chunk 4 j + kg.
        const uint32_t krd = ring_lds + slot * kTileBytes +
                             (uint32_t)(opaque_lane(lane) & 15) * kRowBytes + 16u * kg;
        typedef __attribute__((address_space(3))) const u32x4_t* lds_u32x4_t;
        auto kread = [&](int j, int b) __attribute__((always_inline)) {
          return *reinterpret_cast<lds_u32x4_t>((uintptr_t)(krd + 16 * b * kRowBytes + 64 * j));
        };
        u32x4_t kbuf[kAhead][2];
#pragma unroll
        for (int j = 0; j < kAhead; ++j)
#pragma unroll
          for (int b = 0; b < 2; ++b) kbuf[j][b] = kread(j, b);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
          const u32x4_t a0 = kbuf[j % kAhead][0], a1 = kbuf[j % kAhead][1];
          if (j + kAhead < kSteps) {
#pragma unroll
            for (int b = 0; b < 2; ++b) kbuf[j % kAhead][b] = kread(j + kAhead, b);
          }
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            if (j == 0) {
              mfma16_first(sacc[0][rb], a0, qf[rb][0]);
              mfma16_first(sacc[1][rb], a1, qf[rb][0]);
            } else {
              mfma16(sacc[0][rb], a0, qf[rb][j]);
              mfma16(sacc[1][rb], a1, qf[rb][j]);
            }
          }
          if (j < 10) dma_x(j);
          __builtin_amdgcn_sched_barrier(0);
        }
        s_wait_products(sacc);
        if (kb + kKT > kend_wmin) {
          asm volatile("" ::: "memory");  // a real (uniform) branch, not selects
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sacc[b][rb][i] =
                    (kb + 16 * b + 4 * kg + i < kend_row[rb]) ? sacc[b][rb][i] : kMinusBig;
        }
        // This lane's largest score of each row.  The row's largest (a
        // reduction over the four lane groups kg) is needed only when some
        // lane's own would move its row's reference, which after a row's
        // first tile is rare: a wave-uniform branch skips the reduction.
        float mxl[2];
        bool up = false;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float mx = kMinusBig;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[b][rb][i]);
          mxl[rb] = mx;
          up |= (mx > 0.5f * kMinusBig ? mx * sc : kMinusBig) > m[rb] + kRestartSlack;
        }
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float mx = max_halves(max_rows16(mxl[rb]));
            const float mt = mx > 0.5f * kMinusBig ? mx * sc : kMinusBig;
            if (mt > m[rb] + kRestartSlack) {
              // While the row has seen no key its O and sum are still zero:
              // the first reference costs nothing.
              if (m[rb] > 0.5f * kMinusBig) moved = true;
              m[rb] = mt;
            }
          }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // Masked scores sit at kMinusBig: against a finite reference their
          // exponent is hugely negative (P = 0); a row with no key yet takes
          // reference 0 here, which gives the same.
          const float neg_m = m[rb] > 0.5f * kMinusBig ? -m[rb] : 0.f;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sacc[b][rb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][rb][i], sc, neg_m));
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) sacc[b][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      // P[row][key 16 b + 4 kg + i] in bf16; the row sums add the fp32 P
      // with plain adds (v_dot2 would hold up the matrix pipe).
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        bf16_t* prow = &plds[(32 * wave + 16 * rb + kq) * kPRow + 4 * kg];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t u0 = pack_bf16x2(sacc[b][rb][0], sacc[b][rb][1]);
          const uint32_t u1 = pack_bf16x2(sacc[b][rb][2], sacc[b][rb][3]);
          *reinterpret_cast<uint2*>(prow + 16 * b) = make_uint2(u0, u1);
          lsum[rb] += (sacc[b][rb][0] + sacc[b][rb][1]) + (sacc[b][rb][2] + sacc[b][rb][3]);
        }
      }
      if (moved) restart = 1;
    };

    // PV products of the tile in `slot`, operands read from inline assembly
    // with explicit waits (the compiler's own waits stop the products after
    // every few reads): the V^T operands of the first 16-key half are read
    // before the barrier that publishes P (pv_first), then P of that half and
    // both operands of the second half, and the first half's products run
    // while the second half's reads land (pv_rest).
    const int pv_ln = opaque_lane(lane);
    const int pv_pc = pv_ln & 31, pv_ph = pv_ln >> 5;
    // Transposing read: lane ln reads row 4 ph + (ln % 16) / 4 (+ 8 for the
    // high half) of a 16-key block, 4 value dims at element column
    // 32 nb + 16 (pc / 16) + 4 (ln % 4) of the wave's 128.
    const int pv_tr_row = 4 * pv_ph + ((pv_ln & 15) >> 2);
    const uint32_t pv_vt0 = ring_lds + (uint32_t)pv_tr_row * kRowBytes +
                            2u * (128 * wave + 16 * (pv_pc >> 4) + 4 * (pv_ln & 3));
    // P^T operand of row block rb: row 32 rb + pc, keys
    // 16 kc + 8 (e / 4) + 4 ph + e % 4 (two 8-byte reads, 16 bytes apart).
    const uint32_t pv_pt = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)
                               &plds[pv_pc * kPRow + 4 * pv_ph];
    auto read_vt = [&](u32x4_t& d, uint32_t vt, int kc, int nb) __attribute__((always_inline)) {
      u32x2_t lo, hi;
      asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
                   : "=&v"(lo), "=&v"(hi)
                   : "v"(vt), "i"(16 * kc * kRowBytes + 64 * nb),
                     "i"(16 * kc * kRowBytes + 64 * nb + 8 * kRowBytes)
                   : "memory");
      d = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
    auto read_pt = [&](u32x4_t& d, int kc, int rb) __attribute__((always_inline)) {
      u32x2_t lo, hi;
      asm volatile("ds_read_b64 %0, %2 offset:%3\n\tds_read_b64 %1, %2 offset:%4"
                   : "=&v"(lo), "=&v"(hi)
                   : "v"(pv_pt), "i"(2 * (32 * rb * kPRow + 16 * kc)),
                     "i"(2 * (32 * rb * kPRow + 16 * kc + 8))
                   : "memory");
      d = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4_t pv_va[2][4], pv_pb[2][4];
    auto pv_first = [&](int slot) __attribute__((always_inline)) {
      const uint32_t vt = (uint32_t)opaque_lane((int)(pv_vt0 + slot * kTileBytes));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) read_vt(pv_va[0][nb], vt, 0, nb);
    };
    auto pv_rest = [&](int slot) __attribute__((always_inline)) {
      const uint32_t vt = (uint32_t)opaque_lane((int)(pv_vt0 + slot * kTileBytes));
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) read_pt(pv_pb[0][rb], 0, rb);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) read_vt(pv_va[1][nb], vt, 1, nb);
      // the first half's operands are in (LDS operations complete in order)
      asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) read_pt(pv_pb[1][rb], 1, rb);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        if (kc == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+a"(oacc[nb][rb])
                         : "v"(pv_va[kc][nb]), "v"(pv_pb[kc][rb]));
      }
    };

    // Step j: [wait for tile j] barrier [S of tile j, DMA of tile j + 1]
    // barrier [PV of tile j].  The first barrier publishes tile j and frees
    // the ring slot of tile j - 1 and the P area; the second publishes P.
    //
    // O is never rescaled: P is taken against a per-row reference that moves
    // only when a tile beats it by more than kRestartSlack.  When that happens
    // the whole workgroup finishes the pass and then does the item over with
    // the new references (which no tile can beat again by that much).
    // This keeps O touched by the matrix cores alone, in AGPRs.
    bool restarted = false;
    for (int32_t tile = 0, slot = 0; tile < ntiles;) {
      wait_vmem<0>();  // this wave's share of tile j has landed
      barrier();
      dma_begin(tile + 1 < ntiles, k0 + (tile + 1) * kKT, slot ^ 1);
      s_phase(k0 + tile * kKT, slot);
      pv_first(slot);
      // this wave's P is in LDS (its stores precede the eight V^T reads)
      asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
      barrier();
      pv_rest(slot);
      ++tile;
      slot ^= 1;
    }
    // Every wave set the flag, if at all, before a barrier of the loop.
    restarted = __builtin_amdgcn_readfirstlane(restart) != 0;

    if (restarted) {
      // The item start's barrier orders this behind every wave's DMA and
      // read of the flag; the flag is cleared there.
      m_keep[0] = m[0];
      m_keep[1] = m[1];
      again = true;
      continue;
    }
    again = false;
    ++idx;

    // Row statistics from the S-phase owners, then every wave stores its dims.
    const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float ltot = lsum[rb] + __shfl_xor(lsum[rb], 16, 64);
      ltot += __shfl_xor(ltot, 32, 64);
      if (kg == 0) llds[32 * wave + 16 * rb + kq] = ltot;
      if (kg == 0 && srow_ok[rb]) {
        const float lse_nat = ltot > 0.f ? (m[rb] + log2f(ltot)) * kLn2 : -INFINITY;
        if (S == 1) {
          if (lse) lse[(int64_t)(q0 + st[rb]) * p.num_qo_heads + sh[rb]] = lse_nat;
        } else {
          const int64_t prow =
              (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + st[rb];
          p.part_lse[prow * p.num_qo_heads + sh[rb]] = lse_nat;
        }
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
      // Lane holds O^T[d][row] for d = 128 wave + 32 nb + 8 b + 4 phalf + j.
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const f32x16_t& acc = oacc[nb][rb];
        // The output row (bf16), or the float32 row of piece s's partial.
        const int64_t col = (int64_t)h * kDV + 128 * wave + 32 * nb + 4 * phalf;
        if (S == 1) {
          bf16_t* orow = o + (int64_t)(q0 + t) * p.num_qo_heads * kDV + col;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            *reinterpret_cast<uint2*>(orow + 8 * b) =
                make_uint2(pack_bf16x2(acc[4 * b] * inv, acc[4 * b + 1] * inv),
                           pack_bf16x2(acc[4 * b + 2] * inv, acc[4 * b + 3] * inv));
        } else {
          const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
          float* orow = p.part_o + prow * p.num_qo_heads * kDV + col;
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
