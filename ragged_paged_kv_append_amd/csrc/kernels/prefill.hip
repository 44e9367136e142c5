// Prefill-chunk attention (bf16, head dim 128, page size a multiple of 16):
// the MFMA-bound kernel.
//
// Prefill is compute bound ("Disaggregated prefill and decode", performance
// section), and a chunk of C new tokens attends to the cached prefix (a
// rectangle) and causally to itself (a triangle), as in the chunked-prefill
// post (sections "core-idea" and "correctness").
//
// One workgroup of eight wavefronts takes a work item: request r, KV head g,
// up to 256 query rows (row = token * G + head-in-group, so the G query heads
// sharing a KV head sit in one tile and share its K/V loads), keys [k0, k1).
// Each wavefront owns 32 rows.  The planner packs the items onto one resident
// workgroup per compute unit, longest first; a workgroup runs its list.
//
// K/V tiles of 64 keys (16 KiB each) move from HBM/L2 into a three-slot LDS
// ring with the gfx950 global-to-LDS DMA; tiles j + 1 and j + 2 are in flight
// while tile j is computed, and one barrier per tile both publishes the
// landed tile and frees the slot the next DMA overwrites.  Rows are stored with their 16-byte
// chunks permuted (K: chunk c of key row k at c ^ (k % 16); V: at
// c ^ 4 (k % 4)) so both LDS read patterns below are bank-conflict free.
//
//   S^T[key][row] = K[key][:] . Q[row][:]        mfma 32x32x16 bf16, A operand
//       read from LDS with ds_read_b128, Q resident in registers;
//   online softmax on S^T (each lane holds 16 keys of one row per 32-key
//       block), in log2 units with the scale folded into one FMA before the
//       exp2.  The running max is raised only when a tile's max exceeds it by
//       more than 8 (a factor of 256), so the O rescale is almost never run;
//       the result is the same softmax, normalised by the same running sum.
//       Only tiles that straddle a row's last visible key are masked;
//   O^T[d][row] += V^T[d][key] . P^T[key][row]   mfma 32x32x16 bf16; the S^T
//       accumulators are already the P^T operand, and V^T is read from the
//       row-major V tile with the transposing LDS read.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kKT = 64;                  // keys per tile
constexpr int kTileElems = kKT * kD;     // 16 KiB of bf16
constexpr int kTileBytes = kTileElems * 2;
constexpr int kSlotBytes = 2 * kTileBytes;  // K tile + V tile
constexpr int kSlots = 3;                   // ring depth
constexpr int kWaves = 8;
constexpr int kDmaRows = kKT / kWaves;      // key rows each wave moves per tile
constexpr float kMinusBig = -1.0e30f;
constexpr float kRescaleSlack = 8.f;     // log2 units
constexpr int kNonTemporal = 2;          // DMA cache policy: streaming

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const bf16_t* lds_cptr_t;

// Workgroup barrier without the memory fences of __syncthreads: the only
// cross-wave traffic is the DMA into the ring, whose completion each wave
// establishes with its own vmcnt wait before the barrier, and LDS reads whose
// values the wave has already consumed.  The fences would make the compiler
// drain the DMA stream at every barrier.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Blocking scalar load of one page id (scalar cache; waits only for LDS and
// scalar operations, never for the DMA in flight).
__device__ __forceinline__ int32_t load_scalar(const int32_t* ptr) {
  // The address is wave-uniform; readfirstlane puts it in scalar registers
  // even where the compiler holds it in vector registers.
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int32_t* sp = reinterpret_cast<const int32_t*>(lo | (hi << 32));
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sp) : "memory");
  return v;
}

// Position of 16-byte chunk c of row k inside a tile row.
__device__ __forceinline__ int k_pos(int c, int k) { return c ^ (k & 15); }
__device__ __forceinline__ int v_pos(int c, int k) { return c ^ (4 * (k & 3)); }

// Four transposing reads of one 16-key V chunk: two 32-dim blocks (base a0
// and a1: LDS byte addresses of the blocks for chunk 0 of the slot), low and
// high key halves (+ 8 rows = + 2048 bytes); kOff adds the chunk.  One asm
// block with its own LDS wait: the compiler cannot tell these reads from the
// DMA in flight and would otherwise drain it first.
template <int kOff>
__device__ __forceinline__ void read_vt4(uint32_t a0, uint32_t a1, s16x4_t (&v)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a0), "v"(a1), "n"(kOff), "n"(kOff + 2048)
      : "memory");
}

template <int kSlot>
struct SlotTag {
  static constexpr int value = kSlot;
};

}  // namespace

__global__ __launch_bounds__(512, 1) void prefill_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ kc,
                                                      const bf16_t* __restrict__ vc, Strides ks,
                                                      Strides vs, bf16_t* __restrict__ o,
                                                      float* __restrict__ lse) {
  // ring[slot][0] = K tile, ring[slot][1] = V tile; rows of 128 bf16.
  __shared__ __attribute__((aligned(1024))) bf16_t ring[kSlots][2][kTileElems];
  const int tid = threadIdx.x;
  // The wave index is uniform within a wave; readfirstlane tells the compiler,
  // so everything derived from it stays in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31;   // query row of this lane within the wave (S^T / O^T column)
  const int half = lane >> 5;  // k-slot group of the 32x32x16 operands

  // ---- per-lane constants, shared by every item of this workgroup ----------
  // LDS byte offsets (from the ring) of this lane's K operand reads: mfma i of
  // a 32-key block reads chunk 2 i + half of key row col (+ 32 b2).
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_cptr_t)ring;
  uint32_t k_rd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) k_rd[i] = col * 256 + 16 * k_pos(2 * i + half, col);
  // Transposing-read source of this lane inside a 16-key V chunk: row
  // 4 half + (lane % 16) / 4 (+ 8 for the high half), element column
  // 32 nb + 16 (col / 16) + 4 (lane % 4).
  const int tr_row = 4 * half + ((lane & 15) >> 2);
  const int tr_chunk = 2 * (col >> 4) + ((lane & 3) >> 1);
  uint32_t v_rd[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    v_rd[nb] = kTileBytes + tr_row * 256 + 16 * v_pos(4 * nb + tr_chunk, tr_row) + 8 * (lane & 1);
  // DMA role: wave w moves key rows 8 w .. 8 w + 7 of every tile (a run of
  // keys inside one page for any page size >= 16); instruction i carries rows
  // 8 w + 4 i + lane / 16, and lane % 16 is the 16-byte position in the row.
  // dma_k[i] / dma_v[i]: element offset of that chunk from the row group's
  // first key (the chunk placed at position lane % 16 is (lane % 16) ^ perm).
  // (Byte offsets, unsigned, so that each DMA address is a scalar base plus a
  // 32-bit lane offset.)
  uint32_t dma_k[2], dma_v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = 4 * i + (lane >> 4);          // row within the wave's 8-row group
    const int trow = 8 * (wave & 1) + rr;        // the row's index mod 16
    dma_k[i] = 2u * (uint32_t)(rr * ks.token + 8 * k_pos(lane & 15, trow));
    dma_v[i] = 2u * (uint32_t)(rr * vs.token + 8 * v_pos(lane & 15, trow));
  }

  const int32_t wb0 = p.wg_indptr[KC_PREFILL][blockIdx.x];
  const int32_t wb1 = p.wg_indptr[KC_PREFILL][blockIdx.x + 1];
  for (int32_t idx = wb0; idx < wb1; ++idx) {
    const int32_t* it = p.items[KC_PREFILL] + (int64_t)idx * IT_WORDS;
    const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], row0 = it[IT_ROW0], row1 = it[IT_ROW1];
    const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
    const int32_t G = p.group;
    const int32_t q0 = p.qo_indptr[r];
    const int32_t n = p.qo_indptr[r + 1] - q0;
    const int32_t L = p.kv_len[r];
    const int32_t cached = L - n;
    auto key_end = [&](int32_t row) __attribute__((always_inline)) {  // one past the last key row `row` may see in this item
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

    u32x4_t qf[8];  // Q operand, loaded once the first tiles are in flight
    const int32_t* pages = p.page_indices + p.page_indptr[r];
    const int64_t k_head = (int64_t)g * ks.head;
    const int64_t v_head = (int64_t)g * vs.head;
    // Starts the DMA of the tile at key kb into ring slot `sl`.  Keys past k1
    // are fetched from the item's last key (a written slot of the same page),
    // so masked keys hold finite values.
    auto issue = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const int32_t gkey = min(kb + kDmaRows * wave, k1 - 1);  // first key of this wave's rows
      const int32_t rmax = k1 - 1 - gkey;                      // rows past it that exist
      const int64_t page = load_scalar(pages + (gkey >> p.page_shift));
      const int64_t in_page = gkey & (p.page_size - 1);
      const bf16_t* kg = kc + page * ks.page + k_head + in_page * ks.token;
      const bf16_t* vg = vc + page * vs.page + v_head + in_page * vs.token;
      bf16_t* kl = &ring[slot][0][kDmaRows * wave * kD];
      bf16_t* vl = &ring[slot][1][kDmaRows * wave * kD];
      const char* kgb = reinterpret_cast<const char*>(kg);
      const char* vgb = reinterpret_cast<const char*>(vg);
      if (rmax >= kDmaRows - 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          __builtin_amdgcn_global_load_lds(kgb + dma_k[i], (lds_void_t*)(kl + 4 * i * kD), 16, 0,
                                           kNonTemporal);
          __builtin_amdgcn_global_load_lds(vgb + dma_v[i], (lds_void_t*)(vl + 4 * i * kD), 16, 0,
                                           kNonTemporal);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rr = 4 * i + (lane >> 4);
          const uint32_t back = (uint32_t)(rr - min(rr, rmax));  // rows clamped onto the last key
          __builtin_amdgcn_global_load_lds(kgb + (dma_k[i] - 2u * back * (uint32_t)ks.token),
                                           (lds_void_t*)(kl + 4 * i * kD), 16, 0, kNonTemporal);
          __builtin_amdgcn_global_load_lds(vgb + (dma_v[i] - 2u * back * (uint32_t)vs.token),
                                           (lds_void_t*)(vl + 4 * i * kD), 16, 0, kNonTemporal);
        }
      }
    };

    const float sc = p.sm_scale * kLog2e;
    float m = kMinusBig;  // running reference max of this row, log2 units
    float lsum = 0.f;     // this lane's share of the running row sum
    f32x16_t oacc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;

    // S^T of the tile in ring slot `sl` into sacc (two 32-key blocks).
    f32x16_t sacc[2];
    auto qk = [&](int slot) __attribute__((always_inline)) {
      const char* kt = reinterpret_cast<const char*>(&ring[slot][0][0]);
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b2][i] = 0.f;
      // The two blocks' products alternate, so consecutive MFMAs never wait on
      // each other, and only two K operands are live at a time.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(kt + k_rd[i]);
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(kt + k_rd[i] + 8192);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qf[i]),
                                                          sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qf[i]),
                                                          sacc[1], 0, 0, 0);
      }
    };

    // Online softmax of sacc (the tile at key kb), then O^T += V^T P^T with
    // the V tile of ring slot `sl`.
    auto softmax_pv = [&](int32_t kb, int slot) __attribute__((always_inline)) {
      const uint32_t slot_lds = ring_lds + slot * kSlotBytes;
      // Element i of block b2 is key kb + 32 b2 + 8 (i / 4) + 4 half + i % 4 of row `col`.
      const bool full = kb + kKT <= kend_wmin;  // every key of the tile visible to every row
      float mx = kMinusBig;
      if (full) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[b2][i]);
      } else {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t key = kb + 32 * b2 + 8 * (i >> 2) + 4 * half + (i & 3);
            sacc[b2][i] = key < kend_row ? sacc[b2][i] : kMinusBig;
            mx = fmaxf(mx, sacc[b2][i]);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Raise the reference max only when the tile's max exceeds it by more
      // than the slack; rows of the wave that need it are rescaled together.
      const float mt = mx > 0.5f * kMinusBig ? mx * sc : kMinusBig;
      const bool raise = mt > m + kRescaleSlack;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        lsum *= alpha;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) oacc[nb] *= alpha;
        m = m_new;
      }
      const float neg_m = -m;
      float psum = 0.f;
      if (full) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b2][i], sc, neg_m));
            sacc[b2][i] = e;
            psum += e;
          }
      } else {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float v = sacc[b2][i];
            const float e =
                v > 0.5f * kMinusBig ? __builtin_amdgcn_exp2f(__builtin_fmaf(v, sc, neg_m)) : 0.f;
            sacc[b2][i] = e;
            psum += e;
          }
      }
      lsum += psum;

      // O^T += V^T P^T over the four 16-key chunks of the tile.
      auto pv_chunk = [&](auto kct) __attribute__((always_inline)) {
        constexpr int kc16 = decltype(kct)::value;
        constexpr int b2 = kc16 >> 1, hb = kc16 & 1;
        u32x4_t pb;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pb[e] = pack_bf16x2(sacc[b2][8 * hb + 2 * e], sacc[b2][8 * hb + 2 * e + 1]);
        // key of k-slot (half, e) in this chunk: 16 kc16 + 8 (e / 4) + 4 half + e % 4
#pragma unroll
        for (int np = 0; np < 2; ++np) {
          s16x4_t vr[4];
          read_vt4<kc16 * 16 * 256>(slot_lds + v_rd[2 * np], slot_lds + v_rd[2 * np + 1], vr);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int nb = 2 * np + j;
            const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, vr[2 * j]);
            const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, vr[2 * j + 1]);
            const u32x4_t va = {lo2[0], lo2[1], hi2[0], hi2[1]};
            oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb),
                                                               oacc[nb], 0, 0, 0);
          }
        }
      };
      pv_chunk(SlotTag<0>{});
      pv_chunk(SlotTag<1>{});
      pv_chunk(SlotTag<2>{});
      pv_chunk(SlotTag<3>{});
    };

    // One step: wait for the tile (the next tile's DMA may still be in flight:
    // each wave issues 4 instructions per tile), start the DMA of the tile two
    // ahead into the slot freed by the previous tile, compute.
    const int32_t ntiles = (kend - k0 + kKT - 1) / kKT;
    auto step = [&](int32_t tile, int slot) __attribute__((always_inline)) {
      const int32_t kb = k0 + tile * kKT;
      if (tile + 1 < ntiles)
        wait_vmem<4>();  // this wave's part of the tile has landed
      else
        wait_vmem<0>();
      barrier();  // every part has landed, and every wave is done with tile - 1
      if (tile + 2 < ntiles) issue(kb + 2 * kKT, slot == 0 ? 2 : slot - 1);
      if (wave_has_rows && kb < kend_wmax) {
        qk(slot);
        softmax_pv(kb, slot);
      }
    };

    barrier();  // the previous item's waves are done with the ring
    if (ntiles > 0) issue(k0, 0);
    if (ntiles > 1) issue(k0 + kKT, 1);

    // Q operand of the S^T products: qf[i] = Q[row][16 i + 8 half .. + 8),
    // loaded while the first tiles are in flight.
    {
      const bf16_t* qrow = q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kD + 8 * half;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qf[i] = row_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * i) : u32x4_t{0u, 0u, 0u, 0u};
      // Complete the Q loads here: from now on the DMA owns the counter.
      asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
                   "v"(qf[6]), "v"(qf[7]));
    }
    for (int32_t tile = 0, slot = 0; tile < ntiles; ++tile, slot = (slot == kSlots - 1) ? 0 : slot + 1)
      step(tile, slot);

    // Finish: the row sum is split over the two halves of the wave.
    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (row_ok) {
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
  }
}

hipError_t launch_prefill(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream) {
  hipLaunchKernelGGL(prefill_kernel, dim3(p.n_wgs[KC_PREFILL]), dim3(64 * kWaves), 0, stream, p,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                     static_cast<const bf16_t*>(v_cache), ks, vs, static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
