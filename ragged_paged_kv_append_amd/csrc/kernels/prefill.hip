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
// K/V tiles of 64 keys (16 KiB each) move from HBM/L2 into a four-slot LDS
// ring with the gfx950 global-to-LDS DMA, issued four tiles ahead of the step
// that uses them.  The V tile is transposed once per workgroup into a V^T
// buffer (rows = head dims, keys in the order the PV product consumes them),
// so that the per-wave PV operands are plain 16-byte LDS reads: the
// transposing LDS read is four times slower than a 16-byte read, and each
// wave would otherwise transpose the whole tile for itself.  K rows keep
// chunk c at c ^ (k % 16), V rows at c ^ 4 (k % 4), V^T rows at
// c ^ ((d / 2) % 8): every LDS read pattern below is bank-conflict free.
//
// Per wavefront, tile j goes through a matrix phase and a softmax phase:
//   M(j): S^T_j[key][row] = K_j[key][:] . Q[row][:] and
//         O^T[d][row] += V^T_{j-1}[d][key] . P^T_{j-1}[key][row]
//         (mfma 32x32x16 bf16; K and V^T from LDS, Q resident in registers,
//         the S^T accumulators laid out as the P^T operand);
//   V(j): mask (only tiles that straddle a row's last visible key), row max,
//         P_j = exp2(S_j * scale * log2 e - m) rounded to bf16, row sum of the
//         rounded P.  The running max is raised only when a tile's max
//         exceeds it by more than 8 (a factor of 256, log2 units), so the O
//         rescale is almost never run.
// The two wavefronts that share a SIMD (w and w + 4) belong to two groups
// that run these phases half a step apart, one group's M beside the other
// group's V, with a workgroup barrier between slots; each phase's inputs and
// outputs are pinned to its slot so that the compiler cannot move work
// across the barriers.  The page ids of a work item's tiles are loaded once
// per item, one tile per lane.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kKT = 64;                     // keys per tile
constexpr int kTileBytes = kKT * kD * 2;    // 16 KiB
constexpr int kSlotBytes = 2 * kTileBytes;  // K tile + V tile
constexpr int kSlots = 4;                   // ring depth
// Tiles in flight ahead of the one being computed.  Two cover the memory
// latency; more outstanding DMA only makes each issue stall longer.
constexpr int kLookahead = 2;
constexpr int kWaves = 8;
constexpr int kDmaRows = kKT / (kWaves / 2);  // key rows each DMA wave moves per tile (16)
constexpr int kDmaInst = 2 * kDmaRows / 4;    // its DMA instructions per tile, K and V (8)
constexpr float kMinusBig = -1.0e30f;
constexpr float kRescaleSlack = 8.f;        // log2 units

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Hides x's value from the optimizer, so that addresses derived from it are
// formed where they are used instead of being hoisted and kept live.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 16-byte LDS read at byte address a.
__device__ __forceinline__ u32x4_t lds_ld16(uint32_t a) {
  return *reinterpret_cast<const lds_u32x4*>((uintptr_t)a);
}

// Workgroup barrier.  Cross-wave data are the DMA'd ring tiles (each wave
// waits for its own part with vmcnt before the barrier) and the V^T writes
// (covered here by the LDS count); no memory fence, which would make the
// compiler drain the DMA in flight.
// The scheduling barriers keep the compiler from moving register-only work
// (exponentials, products) across it, which would undo the phase split below.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One global-to-LDS DMA instruction (gfx950 global_load_lds_dwordx4): every
// lane copies 16 bytes from `src` to LDS byte address lds + 16 * lane.  It is
// issued from inline assembly so that the compiler does not track it: left to
// itself the compiler makes later LDS reads wait for all DMA in flight, while
// the kernel waits for exactly the tile it needs (explicit vmcnt counts,
// which operations the compiler adds can only make stricter).  M0, which
// carries the LDS address, is saved and restored around the instruction; the
// DMA reads M0 one wait state after the write that sets it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Positions of 16-byte chunk c inside a K row (key k), a V row (key k) and a
// V^T row (head dim d).
__device__ __forceinline__ int k_pos(int c, int k) { return c ^ (k & 15); }
__device__ __forceinline__ int v_pos(int c, int k) { return c ^ (4 * (k & 3)); }
__device__ __forceinline__ int vt_pos(int c, int d) { return c ^ ((d >> 1) & 7); }

}  // namespace

__global__ __launch_bounds__(512, 1) void prefill_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ kc,
                                                      const bf16_t* __restrict__ vc, Strides ks,
                                                      Strides vs, bf16_t* __restrict__ o,
                                                      float* __restrict__ lse) {
  // ring[slot]: K tile, then V tile (rows of 128 bf16).  vt[b]: V^T of a tile,
  // 128 rows (head dims) of 64 keys; in a row, 16-byte chunk 2 c + hh holds
  // the keys 16 c + 4 hh + (0..3) and 16 c + 8 + 4 hh + (0..3).
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots][kSlotBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vt[2][kTileBytes];
  const int tid = threadIdx.x;
  // The wave index is uniform within a wave; readfirstlane tells the compiler,
  // so everything derived from it stays in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31;   // query row of this lane within the wave (S^T / O^T column)
  const int half = lane >> 5;  // k-slot group of the 32x32x16 operands
  const uint32_t ring_lds =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)ring;
  const uint32_t vt_lds =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)vt;

  // ---- per-lane constants, shared by every item of this workgroup ----------
  // Buffer bases are multiples of 1024, so the XORs below, which touch bits
  // 4..7 only, commute with adding them.
  // K operand of mfma i of a 32-key block: chunk 2 i + half of key row col,
  // at k_rd ^ 32 i (+ 32 rows = + 8192 bytes for the second block).
  const uint32_t k_rd = col * 256 + 16 * k_pos(half, col);
  // V^T operand of 16-key chunk kc16 and 32-dim block nb: chunk 2 kc16 + half
  // of V^T row 32 nb + col, at vt_rd ^ 32 kc16 (+ 4096 bytes per nb).
  const uint32_t vt_rd = col * 128 + 16 * vt_pos(half, col);
  // Transpose role: instruction i = 2 ih + il of wave w handles unit
  // u = 16 w + 4 i + lane / 16, i.e. keys 4 (u / 8) .. + 3 and head dims
  // 16 (u % 8) .. + 15.  Lane c + 4 e of a 16-lane group reads key row
  // 4 (u / 8) + e, dims 16 (u % 8) + 4 c .. + 3; the transposing read hands
  // lane l of the group V^T[16 (u % 8) + l][4 keys], written as 8 bytes of
  // V^T row 16 (u % 8) + l.  The source of instruction i is
  // (tr_src ^ 128 il) + 1024 ih, its destination (tr_dst ^ 16 ih) + 8192 il.
  uint32_t tr_src, tr_dst;
  {
    const int u = 16 * wave + (lane >> 4);
    const int kq = u >> 3, cb = u & 7;
    const int l16 = lane & 15, c = l16 & 3, e = l16 >> 2;
    const int R = 4 * kq + e;                       // key row read by this lane
    tr_src = kTileBytes + R * 256 + 16 * v_pos(2 * cb + (c >> 1), R) + 8 * (c & 1);
    const int dd = 16 * cb + l16;                   // V^T row written by this lane
    const int kc16 = kq >> 2, q4 = kq & 3;          // 16-key chunk and 4-key group in it
    tr_dst = dd * 128 + 16 * vt_pos(2 * kc16 + (q4 & 1), dd) + 8 * (q4 >> 1);
  }
  // DMA role (waves of the first group only, so that the DMA issue, which
  // stalls the issuing wave while many transfers are outstanding, sits among
  // that wave's matrix products): wave w < 4 moves key rows 16 w .. 16 w + 15
  // of every tile (a run of keys inside one page for any page size >= 16);
  // instruction i carries rows 16 w + 4 i + lane / 16 and lane % 16 is the
  // 16-byte position in the row, which holds chunk (lane % 16) ^ perm.  Byte
  // offsets from the first key of the wave's rows.
  // The offsets are recomputed at each instruction (a few vector operations
  // beside the matrix products) rather than held in registers.
  const bool dma_wave = wave < kWaves / 2;

  // Both V^T buffers start as zeros, so that the first PV product of an item
  // (P = 0) never meets a non-finite value.
#pragma unroll
  for (int i = 0; i < 2 * kTileBytes / (16 * 64 * kWaves); ++i)
    *reinterpret_cast<lds_u32x4*>((uintptr_t)(vt_lds + 16 * (tid + 64 * kWaves * i))) =
        u32x4_t{0u, 0u, 0u, 0u};

  const int32_t wb0 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_PREFILL][blockIdx.x]);
  const int32_t wb1 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_PREFILL][blockIdx.x + 1]);
  for (int32_t idx = wb0; idx < wb1; ++idx) {
    // Item fields and request lengths are wave-uniform: readfirstlane keeps
    // them, and the loop control derived from them, in scalar registers.
    auto uni = [](int32_t x) __attribute__((always_inline)) {
      return __builtin_amdgcn_readfirstlane(x);
    };
    const int32_t* it = p.items[KC_PREFILL] + (int64_t)idx * IT_WORDS;
    const int32_t r = uni(it[IT_REQ]), g = uni(it[IT_KVHEAD]);
    const int32_t row0 = uni(it[IT_ROW0]), row1 = uni(it[IT_ROW1]);
    const int32_t k0 = uni(it[IT_K0]), k1 = uni(it[IT_K1]), s = uni(it[IT_SPLIT]);
    const int32_t G = p.group;
    const int32_t q0 = uni(p.qo_indptr[r]);
    const int32_t n = uni(p.qo_indptr[r + 1]) - q0;
    const int32_t L = uni(p.kv_len[r]);
    const int32_t S = uni(p.split[r * SP_WORDS + SP_COUNT]);     // pieces of this request
    const int32_t part0 = uni(p.split[r * SP_WORDS + SP_BASE]);  // its first partial row
    const int32_t cached = L - n;
    // A request with a tree mask sees every key up to L - 1, filtered among
    // the new tokens by its 64-bit mask row.
    const bool tree = p.tree_mask != nullptr && uni(p.tree_req[r]) != 0;
    const bool causal = p.causal && !tree;
    auto key_end = [&](int32_t row) __attribute__((always_inline)) {
      return min(k1, (causal ? cached + row / G : L - 1) + 1);
    };

    const int32_t row = row0 + wave * 32 + col;
    const bool row_ok = row < row1;
    const int32_t t = row_ok ? row / G : 0;
    const int32_t h = g * G + (row_ok ? row % G : 0);
    const int32_t kend_row = row_ok ? key_end(row) : k0;
    const int32_t kend = uni(key_end(row1 - 1));
    const int32_t wrow0 = row0 + wave * 32;
    const bool wave_has_rows = wrow0 < row1;
    const int32_t kend_wmin = uni(wave_has_rows ? key_end(wrow0) : k0);
    // Tiles from mask_from on need the element mask.
    const int32_t mask_from = tree ? min(kend_wmin, max(cached, k0)) : kend_wmin;
    const uint64_t tmask = (tree && row_ok)
                               ? ((uint64_t)p.tree_mask[2 * (int64_t)(q0 + t) + 1] << 32) |
                                     p.tree_mask[2 * (int64_t)(q0 + t)]
                               : 0ull;
    const int32_t ntiles = (kend - k0 + kKT - 1) / kKT;

    u32x4_t qf[8];  // Q operand, loaded once the first tiles are in flight
    const int32_t* pages = p.page_indices + p.page_indptr[r];
    const char* kbase = reinterpret_cast<const char*>(kc + (int64_t)g * ks.head);
    const char* vbase = reinterpret_cast<const char*>(vc + (int64_t)g * vs.head);
    if (idx > wb0) wait_vmem<0>();  // the previous item's output stores
    // Page id of the first key row this wave moves for tile T, in lane T % 64
    // of pid[T / 64] (the planner keeps an item within 128 tiles).  Rows past
    // k1 are clamped onto the item's last key.
    int32_t pid[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t gkey = min(k0 + (lane + 64 * c) * kKT + kDmaRows * wave, k1 - 1);
      pid[c] = dma_wave && (c == 0 || ntiles > 64) ? pages[gkey >> p.page_shift] : 0;
    }
    // DMA of tile T into ring slot `slot` by a wave of the first group: 4 K
    // and 4 V instructions, x = 0..7.  Keys past k1 are fetched from the
    // item's last key (a written slot of the same page), so masked keys hold
    // finite values.
    struct DmaTile {
      const char* kg;
      const char* vg;
      uint32_t kl;
      int32_t rmax;  // rows past the first that exist
    };
    auto dma_setup = [&](int32_t T, int slot) __attribute__((always_inline)) {
      const int32_t gkey = min(k0 + T * kKT + kDmaRows * wave, k1 - 1);  // first key of this wave's rows
      const int64_t page = T < 64 ? __builtin_amdgcn_readlane(pid[0], T)
                                  : __builtin_amdgcn_readlane(pid[1], T - 64);
      const int64_t in_page = gkey & (p.page_size - 1);
      DmaTile d;
      d.kg = kbase + 2 * (page * ks.page + in_page * ks.token);
      d.vg = vbase + 2 * (page * vs.page + in_page * vs.token);
      d.kl = __builtin_amdgcn_readfirstlane(ring_lds + slot * kSlotBytes + kDmaRows * wave * 256);
      d.rmax = k1 - 1 - gkey;
      return d;
    };
    auto dma_x = [&](const DmaTile& d, int x) __attribute__((always_inline)) {
      const int i = x & 3;
      const bool v = x >= 4;
      const int ln = (int)opaque((uint32_t)lane);
      const int rr = 4 * i + (ln >> 4);  // row within the wave's 16 rows (= its index mod 16)
      const int row = min(rr, d.rmax);   // rows past the last key repeat it
      const uint32_t off =
          v ? 2u * (uint32_t)(row * vs.token + 8 * v_pos(ln & 15, rr))
            : 2u * (uint32_t)(row * ks.token + 8 * k_pos(ln & 15, rr));
      dma16((v ? d.vg : d.kg) + off, d.kl + (v ? kTileBytes : 0) + 1024 * i);
    };
    auto issue = [&](int32_t T, int slot) __attribute__((always_inline)) {
      const DmaTile d = dma_setup(T, slot);
#pragma unroll
      for (int x = 0; x < kDmaInst; ++x) dma_x(d, x);
    };

    // Transpose of the V tile in ring slot `slot` into vt[buf]: this wave's
    // four transposing reads, then its four writes.
    auto transpose_read = [&](int slot, s16x4_t (&v)[4]) __attribute__((always_inline)) {
      const uint32_t src = opaque(ring_lds + slot * kSlotBytes + tr_src);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(uintptr_t)((src ^ (128u * (i & 1))) + 1024u * (i >> 1)));
    };
    auto transpose_write = [&](int buf, const s16x4_t (&v)[4]) __attribute__((always_inline)) {
      const uint32_t dst = opaque(vt_lds + buf * kTileBytes + tr_dst);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(
            (uintptr_t)((dst ^ (16u * (i >> 1))) + 8192u * (i & 1))) = v[i];
    };
    auto transpose = [&](int slot, int buf) __attribute__((always_inline)) {
      s16x4_t v[4];
      transpose_read(slot, v);
      transpose_write(buf, v);
    };

    // Waits until this wave's part of tile `tile` has landed, when tiles up
    // to `last` have been issued: each wave issues kDmaInst instructions per
    // tile, in tile order.
    auto wait_tile = [&](int32_t tile, int32_t last) __attribute__((always_inline)) {
      const int32_t later = last - tile;  // tiles issued after it
      if (later >= 3) wait_vmem<3 * kDmaInst>();
      else if (later == 2) wait_vmem<2 * kDmaInst>();
      else if (later == 1) wait_vmem<kDmaInst>();
      else wait_vmem<0>();
    };

    const float sc = p.sm_scale * kLog2e;
    float m = kMinusBig;  // running reference max of this row, log2 units
    float lsum = 0.f;     // this lane's share of the running row sum
    f32x16_t oacc[4];     // O^T: element 4 b + j of block nb is head dim 32 nb + 8 b + 4 half + j
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
    f32x16_t sacc[2];  // S^T of the current tile, two 32-key blocks
    u32x4_t pb[4];     // P^T of the previous tile, bf16 pairs, one 16-key chunk each
#pragma unroll
    for (int c = 0; c < 4; ++c) pb[c] = u32x4_t{0u, 0u, 0u, 0u};

    // K operand i of block b2 of the tile in ring slot `slot`.
    auto kld = [&](uint32_t kt, int i, int b2) __attribute__((always_inline)) {
      return lds_ld16((kt ^ (32u * i)) + 8192u * b2);
    };
    // V^T operand of 16-key chunk kc16 and 32-dim block nb.
    auto vld = [&](uint32_t vtb, int kc16, int nb) __attribute__((always_inline)) {
      return lds_ld16((vtb ^ (32u * kc16)) + 4096u * nb);
    };

    // Matrix phase M(j): S^T_j = K_j Q^T into sacc, and
    // O^T += V^T_{j-1} P^T_{j-1}.  The products of the two contractions
    // alternate, with their LDS operands read one step ahead.  At j = 0, P is
    // zero (and V^T finite); at j = ntiles, the S product reads a stale ring
    // slot and its result is not used.
    // With refill, this (first-group) wave's DMA of tile j + kLookahead into
    // its ring slot goes between the products, one instruction per step.
    auto mphase = [&](int32_t j, bool refill) __attribute__((always_inline)) {
      DmaTile rd{};
      if (refill) rd = dma_setup(j + kLookahead, (j + kLookahead) & (kSlots - 1));
      const uint32_t kt = opaque(ring_lds + (j & (kSlots - 1)) * kSlotBytes + k_rd);
      const uint32_t vtb = opaque(vt_lds + ((j - 1) & 1) * kTileBytes + vt_rd);
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b2][i] = 0.f;
      // step i: S products i of both blocks, PV products (kc16 = i / 2,
      // nb = 2 (i % 2) + 0, 1).  The operands of step i are read two steps
      // ahead; the scheduling barrier at the end of each step keeps the
      // compiler from sinking the reads next to their products.
      constexpr int kAhead = 2;
      u32x4_t ka[kAhead + 1][2], va[kAhead + 1][2];
      auto fetch = [&](int i) __attribute__((always_inline)) {
        const int b = i % (kAhead + 1);
        ka[b][0] = kld(kt, i, 0);
        ka[b][1] = kld(kt, i, 1);
        va[b][0] = vld(vtb, i >> 1, 2 * (i & 1));
        va[b][1] = vld(vtb, i >> 1, 2 * (i & 1) + 1);
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) fetch(i);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = i % (kAhead + 1), c = i & 1;
        if (i + kAhead < 8) fetch(i + kAhead);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[b][0]), as_bf16x8(qf[i]),
                                                          sacc[0], 0, 0, 0);
        oacc[2 * c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(va[b][0]), as_bf16x8(pb[i >> 1]), oacc[2 * c], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[b][1]), as_bf16x8(qf[i]),
                                                          sacc[1], 0, 0, 0);
        oacc[2 * c + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(va[b][1]), as_bf16x8(pb[i >> 1]), oacc[2 * c + 1], 0, 0, 0);
        if (refill) dma_x(rd, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Softmax phase V(j): mask (tiles that straddle a row's last visible key),
    // row max, lazy rescale, P^T_j = exp2(S^T_j * scale * log2 e - m) as bf16
    // pairs, and the row sum of the rounded P.
    // Element i of S^T block b2 of the tile at kb is key
    // kb + 32 b2 + 8 (i / 4) + 4 half + i % 4 of row `col`.
    auto vphase = [&](int32_t j) __attribute__((always_inline)) {
      // S enters here and P leaves at the end through empty asm statements:
      // the phase's arithmetic stays between the barriers that delimit it.
      asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]));
      const int32_t kb = k0 + j * kKT;
      if (kb + kKT > mask_from) {
        // Two uniform branches, each one compare and one select per element
        // (plus the bit test for trees), with no per-element control flow.
        const int32_t lim = kend_row - kb - 4 * half;
        if (!tree) {
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int idx = 32 * b2 + 8 * (i >> 2) + (i & 3);
              sacc[b2][i] = idx < lim ? sacc[b2][i] : kMinusBig;
            }
        } else {
          const int32_t rel = kb + 4 * half - cached;  // new-token index of element offset 0
          const uint32_t tlo = (uint32_t)tmask, thi = (uint32_t)(tmask >> 32);
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int idx = 32 * b2 + 8 * (i >> 2) + (i & 3);
              const int32_t bi = rel + idx;  // < 0: a cached key, always visible
              const uint32_t word = bi >= 32 ? thi : tlo;
              const bool in_tree = bi < 0 || ((word >> (bi & 31)) & 1u) != 0;
              sacc[b2][i] = (idx < lim) & in_tree ? sacc[b2][i] : kMinusBig;
            }
        }
      }
      // Row max as a tree (independent operations for the scheduler).
      float mx8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        mx8[k] = fmaxf(fmaxf(sacc[k >> 2][4 * (k & 3)], sacc[k >> 2][4 * (k & 3) + 1]),
                       fmaxf(sacc[k >> 2][4 * (k & 3) + 2], sacc[k >> 2][4 * (k & 3) + 3]));
      float mx = fmaxf(fmaxf(fmaxf(mx8[0], mx8[1]), fmaxf(mx8[2], mx8[3])),
                       fmaxf(fmaxf(mx8[4], mx8[5]), fmaxf(mx8[6], mx8[7])));
      mx = max_halves(mx);
      // The reference max is raised only when this tile's max exceeds it by
      // more than kRescaleSlack; O and the row sum are rescaled then.
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
      // A row with no visible key so far has m = kMinusBig; its masked
      // entries (kMinusBig) then still map to exp2 = 0.
      const float neg_m = m > 0.5f * kMinusBig ? -m : 0.f;
      // P in place of S, each stage over all 32 entries so that the
      // exponentials do not wait on one another's inputs.
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b2][i] = __builtin_fmaf(sacc[b2][i], sc, neg_m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b2][i] = __builtin_amdgcn_exp2f(sacc[b2][i]);
      __builtin_amdgcn_sched_barrier(0);
      // word w = k-slot pair e = w % 4 of 16-key chunk kc16 = w / 4; the row
      // sum is taken over the fp32 P, in four partial sums, with plain adds:
      // v_dot2 would serialise against the other wave's matrix products on
      // this SIMD, the adds overlap them.
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int kc16 = w >> 2, e = w & 3, b2 = kc16 >> 1, hb = kc16 & 1;
        const float x0 = sacc[b2][8 * hb + 2 * e], x1 = sacc[b2][8 * hb + 2 * e + 1];
        pb[kc16][e] = pack_bf16x2(x0, x1);
        ps[e] += x0 + x1;
      }
      lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(lsum));
    };

    // This wave's eighth of the V transpose of tile j (ring slot j % kSlots
    // into vt[j % 2]).
    auto transpose_part = [&](int32_t j) __attribute__((always_inline)) {
      transpose(j & (kSlots - 1), j & 1);
    };

    // The page ids are complete before the first DMA is issued (the DMA
    // addresses need them); the empty asm statement marks them as such.
    asm volatile("" : "+v"(pid[0]), "+v"(pid[1]));
    barrier();  // the previous item's waves are done with the ring and vt
    if (dma_wave) {
#pragma unroll
      for (int j = 0; j < kLookahead; ++j)
        if (j < ntiles) issue(j, j);
    }

    // Q operand of the S^T products: qf[i] = Q[row][16 i + 8 half .. + 8),
    // loaded while the first tiles are in flight.  The empty asm statement
    // makes the compiler complete these loads here (its wait also covers the
    // first tiles, whose latency the Q loads now share); a load still pending
    // in its view would make it wait for every untracked DMA in flight at
    // the first use inside the loop.
    {
      const bf16_t* qrow = q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kD + 8 * half;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qf[i] = row_ok ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * i) : u32x4_t{0u, 0u, 0u, 0u};
      asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]),
                   "+v"(qf[5]), "+v"(qf[6]), "+v"(qf[7]));
    }

    // Two groups of four wavefronts (one of each per SIMD) run the phases
    // M(0) V(0) M(1) V(1) ... M(ntiles) half a step apart, so that one
    // group's products overlap the other group's softmax.  Slot 2 j: group 0
    // runs M(j), group 1 runs V(j - 1); slot 2 j + 1: group 0 runs V(j),
    // group 1 runs M(j).  Each slot begins with a workgroup barrier.
    //   K_j and V^T_{j-1} are read in slots 2 j and 2 j + 1;
    //   V_j is transposed into vt[j % 2] in slots 2 j (group 1) and 2 j + 1
    //   (group 0), each wave its eighth, in the slot of its softmax phase;
    //   tile j + kLookahead is loaded into ring slot (j + kLookahead) % kSlots
    //   in slot 2 j (the tile that slot held was last read in slot 2 j - 3).
    // Waits for tile j before slot 2 j: tiles up to j + kLookahead - 1 have
    // been issued by then.  Only the first group issues DMA; the second sees
    // each tile through the barrier that follows the first group's wait.
    auto wait_for = [&](int32_t j) __attribute__((always_inline)) {
      if (j < ntiles) wait_tile(j, min(j + kLookahead - 1, ntiles - 1));
    };
    // In slot 2 j the first group loads tile j + kLookahead (inside its
    // matrix phase).
    auto refill_due = [&](int32_t j) __attribute__((always_inline)) {
      return j + kLookahead < ntiles;
    };
    if (wave < kWaves / 2) {
      for (int32_t j = 0; j <= ntiles; ++j) {
        wait_for(j);
        barrier();  // slot 2 j
        mphase(j, refill_due(j));
        barrier();  // slot 2 j + 1
        if (j < ntiles) {
          vphase(j);
          transpose_part(j);
        }
      }
    } else {
      for (int32_t j = 0; j <= ntiles; ++j) {
        barrier();  // slot 2 j
        if (j >= 1) vphase(j - 1);
        if (j < ntiles) transpose_part(j);
        barrier();  // slot 2 j + 1
        mphase(j, false);
      }
    }

    // Finish: the row sum is split over the two halves of the wave.
    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (row_ok) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      const float lse_nat = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
      const int32_t i_tok = q0 + t;
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
        const int64_t prow = (int64_t)part0 + (int64_t)s * n + t;
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
