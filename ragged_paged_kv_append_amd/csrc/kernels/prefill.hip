// Prefill-chunk attention (bf16, head dim 128, page size a multiple of 16):
// the MFMA-bound kernel.
//
// Prefill is compute bound ("Disaggregated prefill and decode", performance
// section), and a chunk of C new tokens attends to the cached prefix (a
// rectangle) and causally to itself (a triangle), as in the chunked-prefill
// post (sections "core-idea" and "correctness").
//
// One workgroup of eight wavefronts, two per SIMD, takes a work item: request
// r, KV head g, up to 256 query rows (row = token * G + head-in-group, so the
// G query heads sharing a KV head sit in one tile and share its K/V loads),
// keys [k0, k1).  Each wavefront owns one 32-row block and half the register
// file of its SIMD: Q of its rows and the O^T accumulators in AGPRs, the S^T
// accumulators in VGPRs.  (The code also builds with four wavefronts of two
// blocks each, one per SIMD; two per SIMD let one wave's products run while
// the other waits on its DMA issue or its LDS reads.)  The planner packs the
// items onto one resident workgroup per compute unit, longest first; a
// workgroup runs its list.
//
// K/V tiles of 64 keys (16 KiB each) move from HBM/L2 into a four-slot LDS
// ring with the gfx950 global-to-LDS DMA, two tiles ahead; each wave moves 8
// key rows of every tile.  K rows keep 16-byte chunk c at c ^ (k % 16), V rows
// at c ^ 4 (k % 4), so the K-operand reads and the transposing V reads are
// bank-conflict free.
//
// The products run in steps of 32 keys.  Step h of a wavefront issues
//   - the S^T products of step h + 1: S^T[key][row] = K[key][:] . Q[row][:]
//     (mfma 32x32x16 bf16, 16 products, K from LDS, Q resident);
//   - the PV products of step h - 1: O^T[d][row] += V^T[d][key] P^T[key][row]
//     (16 products; V^T comes straight from the V rows through the
//     transposing LDS read, P^T from registers: the S^T accumulator layout is
//     the P^T operand layout);
// and, between those products, the vector work of step h: P = exp2(S') rounded
// to bf16.  The row sums of P come from the matrix core too: two small
// products per step multiply the P^T operands by a 0/1 selector (mfma_sum).
// The products of one step do not depend on its vector work, so a wavefront
// keeps its SIMD's matrix core busy while it runs the softmax in the gaps,
// and the SIMD's second wavefront fills what the first leaves idle.
//
// The mask comes out of the matrix core with S: the first product of each
// S^T chain accumulates onto a block that holds 0, or -1e30 for a masked
// (key, row) pair (the causal diagonal, a tree mask, keys past the item).
// The vector pipe, which sets the pace next to the matrix core, then spends
// one fma (S' = S * scale * log2 e - m), one exp and half a conversion per
// score.  (Q is not scaled instead: rounding Q * scale to bf16 moves large
// scores by whole units.)
//
// O is never rescaled.  P is taken against a fixed per-row reference m (0 on
// the first pass): the scores only have to stay within about 2^64 of it,
// above and below, for P, the sums and O to stay well inside the float range
// without losing precision.  The row sum s checks this without a running
// max: s is at least the row's largest P and at most the number of keys
// times it.  A row with s outside [2^-64, 2^64] makes the workgroup finish
// the item and do it over once with reference m + log2 s (its sum is then
// 1).  Only a row whose s is 0 or not finite (every P under- or overflowed,
// or a tree row that may see no key of the item) needs its largest score:
// the item is then done over keeping each row's largest score, and once more
// with it as the reference of the rows that left the window.  This keeps O
// touched by the matrix cores alone, so it stays in AGPRs.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kRB = 256 / kWaves / 32;      // 32-row blocks per wave
constexpr int kWaveRows = 32 * kRB;         // query rows per wave
constexpr int kDmaRows = 64 / kWaves;       // key rows each wave moves per tile
constexpr int kDmaHalf = kDmaRows / 4;      // its DMA instructions per K (or V) share
constexpr int kKT = 64;                     // keys per ring tile
constexpr int kStep = 32;                   // keys per softmax step
constexpr int kTileBytes = kKT * kD * 2;    // 16 KiB: the K (or V) rows of a tile
constexpr int kSlotBytes = 2 * kTileBytes;  // K tile, then V tile
constexpr int kSlots = 4;
constexpr int kDmaInst = 2 * kDmaHalf;       // per wave and tile
constexpr float kMinusBig = -1.0e30f;
constexpr float kWindow = 64.f;             // log2 units around the reference
// Passes over an item: the first (reference 0, checked by the row sums), a
// final one (references set by a check, not checked again) and one that
// keeps each row's largest scaled score (reference 0, checked by it).
constexpr int kFirst = 0, kFinal = 1, kTrack = 2;

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Hides x's value from the optimizer, so that addresses derived from it are
// formed where they are used instead of being hoisted and kept live.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ u32x4_t lds_ld16(uint32_t a) {
  return *reinterpret_cast<const lds_u32x4*>((uintptr_t)a);
}

// Transposing read of four 16-bit elements (see common.h).
__device__ __forceinline__ u32x2_t lds_tr8(uint32_t a) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a));
}

// Workgroup barrier.  The data shared between waves are the DMA'd ring tiles
// (each wave waits for its own part with vmcnt before the barrier).  The
// scheduling barriers keep the compiler from moving work across it.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One global-to-LDS DMA instruction (gfx950 global_load_lds_dwordx4, saddr
// form) for the lanes in `lanes`: each copies 16 bytes from base + off to LDS
// byte address lds + 16 * lane; the other lanes move nothing, and what their
// LDS bytes held stays.  It is issued from inline assembly so that the
// compiler does not track it: left to itself the compiler makes later LDS
// reads wait for all DMA in flight, while the kernel waits for exactly the
// tiles it needs (explicit vmcnt counts).  EXEC and M0 (the LDS address) are
// saved and restored around the instruction; the DMA reads M0 one wait state
// after the write that sets it, and a memory instruction reads an SGPR that a
// vector instruction (v_readlane, v_readfirstlane) wrote only five wait
// states later: the first instruction of a tile waits (NOP), the others use
// scalar values formed by scalar instructions.
#define RPA_DMA16_BODY                \
  "s_mov_b64 %1, exec\n\t"             \
  "s_mov_b64 exec, %5\n\t"             \
  "s_mov_b32 %0, m0\n\t"               \
  "s_mov_b32 m0, %4\n\t"               \
  "s_nop 0\n\t"                        \
  "global_load_lds_dwordx4 %2, %3\n\t" \
  "s_mov_b32 m0, %0\n\t"               \
  "s_mov_b64 exec, %1"
template <bool NOP>
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds,
                                      uint64_t lanes) {
  uint32_t saved_m0;
  uint64_t saved_exec;
  if (NOP) {
    asm volatile("s_nop 4\n\t" RPA_DMA16_BODY
                 : "=&s"(saved_m0), "=&s"(saved_exec)
                 : "v"(off), "s"(base), "s"(lds), "s"(lanes)
                 : "memory");
  } else {
    asm volatile(RPA_DMA16_BODY
                 : "=&s"(saved_m0), "=&s"(saved_exec)
                 : "v"(off), "s"(base), "s"(lds), "s"(lanes)
                 : "memory");
  }
}
#undef RPA_DMA16_BODY

// The S^T products are issued from inline assembly so that their
// accumulators stay in VGPRs, where the softmax reads them (the compiler
// puts every matrix-core result of a kernel that uses AGPRs into AGPRs, and
// the O^T accumulators fill them).  A chain of products on one accumulator
// needs no wait states between its links.  The results are read by vector
// instructions only one step later, after the 16 PV products of the step
// that produced them.
// Q, the B operand, stays in AGPRs (the matrix cores read either file).  The
// first product of a chain starts from the block c (0, or -1e30 where
// masked).
__device__ __forceinline__ void mfma_s_first(f32x16_t& d, const u32x4_t& a, const u32x4_t& b,
                                             const f32x16_t& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void mfma_s(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Operand reads from LDS, from inline assembly: the compiler neither waits
// for them nor reuses their registers early; the kernel waits explicitly.
// A K operand: one 16-byte read.
__device__ __forceinline__ void ds_k(u32x4_t& d, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(a) : "memory");
}
// A V^T operand: two transposing reads, key rows r .. r + 3 and r + 8 .. r + 11.
__device__ __forceinline__ void ds_vt(u32x4_t& d, uint32_t a) {
  u32x2_t lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:2048"
               : "=&v"(lo), "=&v"(hi)
               : "v"(a)
               : "memory");
  d = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}
template <int N>
__device__ __forceinline__ void wait_lds() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// wait_lds with a count known after unrolling (n in 0..15).
__device__ __forceinline__ void wait_lds_n(int n) {
  switch (n) {
    case 0: wait_lds<0>(); break;
    case 1: wait_lds<1>(); break;
    case 2: wait_lds<2>(); break;
    case 3: wait_lds<3>(); break;
    case 4: wait_lds<4>(); break;
    case 5: wait_lds<5>(); break;
    case 6: wait_lds<6>(); break;
    case 7: wait_lds<7>(); break;
    case 8: wait_lds<8>(); break;
    case 9: wait_lds<9>(); break;
    case 10: wait_lds<10>(); break;
    case 11: wait_lds<11>(); break;
    case 12: wait_lds<12>(); break;
    case 13: wait_lds<13>(); break;
    case 14: wait_lds<14>(); break;
    default: wait_lds<15>(); break;
  }
}

// LDS reads issued in slot s of a step (see the operand schedule below).
constexpr int reads_in_slot(int s) {
  return s == 0 ? 2 : (s % 2 != 0 ? 0 : (s <= 16 ? 1 : 2));
}
// Reads issued in the five slots before slot u (of this or the previous step).
constexpr int reads_before(int u) {
  int n = 0;
  for (int d = 1; d <= 5; ++d) n += reads_in_slot(((u - d) % 32 + 32) % 32);
  return n < 15 ? n : 15;
}

// Softmax schedule of a step (see the main loop): exps of elements 0, 1 in
// slot 0, 2, 3 in slot 1 and e >= 4 in slot e - 2; the bf16 pack of pair p
// in slot 2 (p = 0), 3 (p = 1) or 2 p + 1 (p >= 2).
constexpr int exp_count(int s) {
  return kRB == 1 ? ((s & 1) == 0 ? 1 : 0) : (s < 2 ? 2 : (s <= 29 ? 1 : 0));
}
constexpr int exp_first(int s) { return kRB == 1 ? s / 2 : ((s < 2 ? 2 * s : s + 2) & 31); }
constexpr int pack_pair(int s) {
  return kRB == 1 ? ((s & 3) == 3 ? s / 4 : -1)
                  : (s == 2 ? 0 : (s == 3 ? 1 : ((s >= 5 && (s & 1)) ? (s - 1) / 2 : -1)));
}

// The PV products, also from inline assembly (accumulators in AGPRs), so that
// their order against the S^T products and the softmax is the program order.
__device__ __forceinline__ void mfma_pv(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// Row sums of P on the matrix core: a 16x16x32 product D[m][n] += A[m][k]
// B[k][n] whose B operand is a P^T operand of the PV products.  In the
// 16x16x32 layout lane l holds B[8 (l / 16) + 0..7][l % 16] and
// D[4 (l / 16) + 0..3][l % 16]; its eight P values are those of row l % 32.
// With A[m][k] = 1 where ((k / 8) & 1) == ((m / 4) & 1), else 0 (the
// selector), output block m / 4 = q sums the lanes 16 g + n with g = q
// (mod 2), which hold row n + 16 (q & 1): each lane's four results are the
// sum over the operand's 16 keys of its own row l % 32.
__device__ __forceinline__ void mfma_sum(f32x4_t& d, const u32x4_t& sel, const u32x4_t& p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "a"(sel), "v"(p));
}

// A plan and the pools its items read.
struct PrefillPart {
  DevPlan p;
  const bf16_t* kc;
  const bf16_t* vc;
  Strides ks, vs;
};

}  // namespace

// Workgroups 0 .. wgs0 - 1 run part0's workgroup lists, the rest part1's
// (wgs0 = the grid for a single plan).
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void prefill_kernel(PrefillPart part0, PrefillPart part1, int32_t wgs0,
                    const bf16_t* __restrict__ q, bf16_t* __restrict__ o,
                    float* __restrict__ lse) {
  const int32_t bid = (int32_t)__builtin_amdgcn_workgroup_id_x();
  const bool second = bid >= wgs0;
  const PrefillPart& pt = second ? part1 : part0;
  const DevPlan& p = pt.p;
  const bf16_t* __restrict__ kc = pt.kc;
  const bf16_t* __restrict__ vc = pt.vc;
  const Strides ks = pt.ks, vs = pt.vs;
  const int32_t wg = bid - (second ? wgs0 : 0);
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kSlots][kSlotBytes];
  __shared__ int32_t restart;  // set when a row needs a final pass with a new reference
  __shared__ int32_t retrack;  // set when a row needs the pass that keeps its max
  const int tid = threadIdx.x;
  // The wave index is uniform within a wave; readfirstlane tells the compiler,
  // so everything derived from it stays in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31;   // row of this lane within a 32-row block
  const int half = lane >> 5;  // k-slot group of the 32x32x16 operands
  const uint32_t ring_lds =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)ring;

  // ---- per-lane LDS offsets, shared by every item ------------------------------
  // The ring base is a multiple of 1024, so the XORs below, which touch bits
  // 5..7 only, commute with adding it.
  // K operand of step i of a 32-key half: chunk 2 i + half of key row col, at
  // k_rd ^ 32 i (+ 8192 for the second half of the tile).
  const uint32_t k_rd = col * 256 + 16 * (half ^ (col & 15));
  // V^T operand (d block nb, 16-key chunk kc) by two transposing reads: lane
  // reads key row 4 half + (lane % 16) / 4 (+ 8 for the second read) and four
  // dims 32 nb + 16 (col / 16) + 4 (lane % 4) .. + 3, which gives it
  // V^T[d = 32 nb + col][keys 4 half + 0..3 (, 8 + 4 half + 0..3)].  With the
  // V swizzle the dims sit at byte v_rd ^ 64 nb of the row (+ 4096 kc).
  const int q4 = (lane & 15) >> 2;
  const uint32_t v_rd = 256u * (4 * half + q4) + 64u * q4 + 32u * (col >> 4) + 8u * (lane & 3);

  // DMA lanes: instruction i of a wave's share of a tile carries its key rows
  // 4 i + lane / 16 (of 16), lane % 16 being the swizzled 16-byte position:
  // K row rr keeps chunk c at c ^ (rr % 16), V rows keep it at c ^ 4 (rr % 4).
  // The instruction's first row is in its scalar base; a lane adds its row
  // within the four (lane / 16) and its chunk.
  const int l4 = lane >> 4, p16 = lane & 15;
  const uint32_t ktok = 2u * (uint32_t)ks.token, vtok = 2u * (uint32_t)vs.token;
  const uint32_t k_lrow = (uint32_t)l4 * ktok;
  const uint32_t xk = 16u * (uint32_t)(p16 ^ l4);  // K chunk of instruction 0 (^ 64 i)
  // (^ 16 (r % 16) for this wave's first row r of a tile)
  const uint32_t kx_wave = 16u * (uint32_t)((kDmaRows * wave) & 15);
  const uint32_t dv_off = (uint32_t)l4 * vtok + 16u * (uint32_t)(p16 ^ (4 * l4));

  const int32_t wb0 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_PREFILL][wg]);
  const int32_t wb1 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_PREFILL][wg + 1]);
  // Zero the ring once (while the item list loads): the PV products of an
  // item's first step multiply a zero P by whatever the slot of the tile
  // before it holds, and key rows past an item keep an older tile's values;
  // both must be finite.
  for (int i = tid; i < kSlots * kSlotBytes / 16; i += 64 * kWaves)
    *reinterpret_cast<lds_u32x4*>((uintptr_t)(ring_lds + 16 * i)) = u32x4_t{0u, 0u, 0u, 0u};
  if (tid == 0) {
    restart = 0;
    retrack = 0;
  }
  // The selector of mfma_sum: lane l holds A[l % 16][8 (l / 16) + 0..7],
  // bf16 ones where ((l / 16) & 1) == ((l / 4) & 1), else zeros.
  u32x4_t sel_ones;
  {
    const uint32_t v = (((lane >> 4) ^ (lane >> 2)) & 1) ? 0u : 0x3F803F80u;
    sel_ones = u32x4_t{v, v, v, v};
  }
  asm volatile("" : "+a"(sel_ones));
  float m_keep[2] = {0.f, 0.f};  // references for the final pass of an item
  int pass = kFirst;
  for (int32_t idx = wb0; idx < wb1;) {
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
    // (read with the other per-request values: where it is used, the load
    // would add a level of memory latency before the first tile)
    const int32_t pg_base = uni(p.page_indptr[r]);
    const int32_t cached = L - n;
    // A request with a tree mask sees every key up to L - 1, filtered among
    // the new tokens by its 64-bit mask row.
    const bool tree = p.tree_mask != nullptr && uni(p.tree_req[r]) != 0;
    const bool causal = p.causal && !tree;
    auto key_end = [&](int32_t row) __attribute__((always_inline)) {
      return min(k1, (causal ? cached + row / G : L - 1) + 1);
    };

    // This lane's rows: kWaveRows wave + 32 rb + col of the item's tile.
    bool row_ok[2];
    int32_t t_of[2], h_of[2], kend_row[2];
    uint32_t tm_lo[2], tm_hi[2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int32_t row = row0 + kWaveRows * wave + 32 * rb + col;
      row_ok[rb] = row < row1;
      t_of[rb] = row_ok[rb] ? row / G : 0;
      h_of[rb] = g * G + (row_ok[rb] ? row % G : 0);
      kend_row[rb] = row_ok[rb] ? key_end(row) : k0;
      tm_lo[rb] = tm_hi[rb] = 0u;
      if (tree && row_ok[rb]) {
        tm_lo[rb] = p.tree_mask[2 * (int64_t)(q0 + t_of[rb])];
        tm_hi[rb] = p.tree_mask[2 * (int64_t)(q0 + t_of[rb]) + 1];
      }
    }
    const int32_t kend = uni(key_end(row1 - 1));
    const int32_t wrow0 = row0 + kWaveRows * wave;
    const int32_t kend_wmin = uni(wrow0 < row1 ? key_end(wrow0) : k0);
    // Steps that start at or past mask_from need the element mask.
    const int32_t mask_from = tree ? min(kend_wmin, max(cached, k0)) : kend_wmin;
    const int32_t nsteps = (kend - k0 + kStep - 1) / kStep;
    const int32_t ntiles = (nsteps + 1) / 2;

    const int32_t* pages = p.page_indices + pg_base;
    const char* kbase = reinterpret_cast<const char*>(kc + (int64_t)g * ks.head);
    const char* vbase = reinterpret_cast<const char*>(vc + (int64_t)g * vs.head);
    // Page id of the first key row this wave moves for tile T, in lane T (the
    // planner keeps an item within 64 tiles), clamped to the item's last key.
    int32_t pid = pages[min(k0 + lane * kKT + kDmaRows * wave, k1 - 1) >> p.page_shift];
    // DMA of tile T into ring slot T % 4: this wave's kDmaRows key rows from
    // kDmaRows wave (one page: pages hold a multiple of 16 keys), instructions
    // x < kDmaHalf for K, the next kDmaHalf for V, each 4 rows of 256 bytes.
    // Rows at or past k1 are not moved: their ring bytes keep an older tile's
    // finite values, which the mask hides.  A tile past the item moves nothing.  No branches.
    struct DmaTile {
      const char* kg;
      const char* vg;
      uint32_t lds;
      int32_t rmax;  // rows past the first that exist (< 0: none)
    };
    auto dma_setup = [&](int32_t T) __attribute__((always_inline)) {
      const int32_t gkey = k0 + T * kKT + kDmaRows * wave;
      const int64_t page = __builtin_amdgcn_readlane(pid, T);
      const int64_t in_page = min(gkey, k1 - 1) & (p.page_size - 1);
      DmaTile d;
      d.kg = kbase + 2 * (page * ks.page + in_page * ks.token);
      d.vg = vbase + 2 * (page * vs.page + in_page * vs.token);
      d.lds = __builtin_amdgcn_readfirstlane(ring_lds + (T & (kSlots - 1)) * kSlotBytes +
                                             kDmaRows * wave * 256);
      d.rmax = k1 - 1 - gkey;
      return d;
    };
    auto dma_x = [&](const DmaTile& d, int x) __attribute__((always_inline)) {
      const int i = x % kDmaHalf;
      const bool v = x >= kDmaHalf;
      // lanes of rows 4 i .. 4 i + 3 that exist: 16 per row
      const int32_t nr = min(max(d.rmax - 4 * i + 1, 0), 4);
      const uint64_t lanes = nr >= 4 ? ~0ull : ((1ull << (16 * nr)) - 1ull);
      const char* b = v ? d.vg + (int64_t)(4 * i) * vtok : d.kg + (int64_t)(4 * i) * ktok;
      const uint32_t off = v ? dv_off : k_lrow + (xk ^ (64u * i) ^ kx_wave);
      if (i == 0) dma16<true>(b, opaque(off), d.lds + (v ? kTileBytes : 0), lanes);
      else dma16<false>(b, opaque(off), d.lds + (v ? kTileBytes : 0) + 1024 * i, lanes);
    };

    const float sc = p.sm_scale * kLog2e;
    // The reference of each row: 0 in the first and kTrack passes.  Rows past
    // the item take one far above any score, so that their P are 0: one
    // overflowing P of any row would turn the sums of the rows that share its
    // mfma_sum product into NaN (inf times a zero of the selector).
    float m[2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      m[rb] = !row_ok[rb] ? -kMinusBig : (pass == kFinal ? m_keep[rb] : 0.f);
    f32x4_t ssum[2];  // the row's sum of P (all four elements), from mfma_sum
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) ssum[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float rmax[2] = {kMinusBig, kMinusBig};  // this lane's largest raw score of each row (kTrack)
    f32x16_t oacc[4][2];  // [nb][rb]: element i is O^T[32 nb + 8 (i/4) + 4 half + i%4][row]
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][rb][i] = 0.f;
    // S^T of two steps (by parity), -1e30 where masked: element i of [par][rb] is key
    // kb + 8 (i/4) + 4 half + i%4 of row 32 rb + col.
    f32x16_t sacc[2][2];
    // P^T of two steps (by parity), bf16 pairs: [par][rb][kc] holds the keys
    // 16 kc + 8 (e/4) + 4 half + e%4, e = 0..7, of the step.
    u32x4_t pb[2][2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < 2; ++c) pb[a][b][c] = u32x4_t{0u, 0u, 0u, 0u};
    // Start blocks of the S^T chains: 0, or -1e30 where the key is masked
    // for the row (set before the products of a step that needs the mask,
    // put back to 0 after it).
    f32x16_t cinit[2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) cinit[rb][i] = 0.f;
    // Vector writes of cinit, then a product reads it: wait states.
    auto cinit_ready = [&]() __attribute__((always_inline)) {
      if constexpr (kRB == 2)
        asm volatile("s_nop 4" : "+v"(cinit[0]), "+v"(cinit[1]));
      else
        asm volatile("s_nop 4" : "+v"(cinit[0]));
    };
    // Mask of the step whose keys start at kb, into cinit.
    auto set_mask = [&](int32_t kb) __attribute__((always_inline)) {
      if (!tree) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int32_t lim = kend_row[rb] - kb - 4 * half;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int e = 8 * (i >> 2) + (i & 3);
            cinit[rb][i] = e < lim ? 0.f : kMinusBig;
          }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          const int32_t lim = kend_row[rb] - kb - 4 * half;
          const int32_t rel = kb + 4 * half - cached;  // new-token index of offset 0
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int e = 8 * (i >> 2) + (i & 3);
            const int32_t bi = rel + e;  // < 0: a cached key, always visible
            const uint32_t word = bi >= 32 ? tm_hi[rb] : tm_lo[rb];
            // bitwise, not short-circuit: no per-element branch
            const bool vis = (e < lim) & ((bi < 0) | (((word >> (bi & 31)) & 1u) != 0));
            cinit[rb][i] = vis ? 0.f : kMinusBig;
          }
        }
      }
    };
    auto clear_mask = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) cinit[rb][i] = 0.f;
    };
    // Steps whose keys start at or past this need the mask.
    const int32_t mask_kb = mask_from - kStep + 1;

    // Page ids and tree-mask rows complete first: the compiler's own wait for
    // them drains every vector-memory operation, so it must come before the
    // untracked loads (Q, the DMA) are issued.
    asm volatile("" : "+v"(pid));
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) asm volatile("" : "+v"(tm_lo[rb]), "+v"(tm_hi[rb]));
    // Q operand of the S^T products: qf[rb][i] = Q[row 32 rb + col][16 i + 8 half .. + 8),
    // loaded into AGPRs from inline assembly, so that its latency overlaps
    // that of the first tiles (the previous item's last products read qf long
    // before its stores).  Rows past the item read a valid row of the request
    // (t_of = 0): their results are never stored.
    u32x4_t qf[2][8];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const bf16_t* qrow =
          q + ((int64_t)(q0 + t_of[rb]) * p.num_qo_heads + h_of[rb]) * kD + 8 * half;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        asm volatile("global_load_dwordx4 %0, %1, off"
                     : "=a"(qf[rb][i])
                     : "v"(qrow + 16 * i)
                     : "memory");
    }
    barrier();  // the previous item's waves are done with the ring
    // Tiles 0 and 1: the products start once Q and tile 0 are in (vector-memory
    // loads complete in order), while tile 1 lands.
    {
      const DmaTile d = dma_setup(0);
#pragma unroll
      for (int x = 0; x < kDmaInst; ++x) dma_x(d, x);
    }
    {
      const DmaTile d = dma_setup(1);
#pragma unroll
      for (int x = 0; x < kDmaInst; ++x) dma_x(d, x);
    }
    wait_vmem<kDmaInst>();  // Q and tile 0 are in; tile 1 may still be in flight
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+a"(qf[rb][i]));
    if (k0 >= mask_kb) set_mask(k0);
    cinit_ready();
    barrier();  // tile 0 is in the ring (tile 1 is waited for in step 0)

    // K operands of step h (ring slot of tile h / 2, its half h % 2), three
    // steps ahead of the products that use them.
    auto kaddr = [&](int32_t h) __attribute__((always_inline)) {
      return opaque(ring_lds + ((h >> 1) & (kSlots - 1)) * kSlotBytes + 8192u * (h & 1) + k_rd);
    };
    auto vaddr = [&](int32_t h) __attribute__((always_inline)) {
      return opaque(ring_lds + ((h >> 1) & (kSlots - 1)) * kSlotBytes + kTileBytes +
                    8192u * (h & 1) + v_rd);
    };
    // ---- operand rings -----------------------------------------------------------
    // Step u uses K operand i (of step u + 1) in slots 2 i, 2 i + 1, from
    // kr[i % 4], and V^T operand j = 4 kc + nb (of step u - 1) in slots
    // 16 + 2 j, 17 + 2 j, from vr[j % 4].  Reads, each issued after its slot's
    // product: slot 0 V^T (u - 1, 3); slots 2..8 K (u + 1, 4..7); slots 10..16
    // K (u + 2, 0..3); slots 18..24 V^T (u - 1, 4..7); slots 26..30 V^T
    // (u, 0..2).  Every operand is read at least six slots before its first
    // product; no ring register is overwritten before a product after its
    // last reader has issued (a product reads its sources during its
    // passes).  LDS reads complete in order, so before a product the wave
    // waits until no more are outstanding than were issued in the five slots
    // before it.
    u32x4_t kr[4], vr[4];
    // Step -1: the S^T products of step 0 alone (K of tile 0, first half).
    {
      const uint32_t ka = kaddr(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) ds_k(kr[i], ka ^ (32u * i));
      wait_lds<0>();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i == 4 || i == 5) wait_lds<2>();
        if (i == 6) wait_lds<1>();
        if (i == 7) wait_lds<0>();
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if (i == 0) mfma_s_first(sacc[0][rb], kr[0], qf[rb][0], cinit[rb]);
          else mfma_s(sacc[0][rb], kr[i % 4], qf[rb][i]);
        }
        // operand i + 3 into the register of operand i - 1 (one pair ago)
        if (i >= 1 && i + 3 < 8) ds_k(kr[(i + 3) % 4], ka ^ (32u * (i + 3)));
      }
      // The softmax of step 0 reads these accumulators next: wait states for
      // the products' latency (the compiler adds none after inline assembly);
      // they also let the last product read its operand before kr is reused.
      if constexpr (kRB == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sacc[0][0]), "+v"(sacc[0][1]));
      else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sacc[0][0]));
      // K operands 0..3 of step 1 (tile 0, second half) for the first step;
      // the V^T operands of step -1 only meet P = 0, so zeros do.
      const uint32_t kn = kaddr(1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ds_k(kr[i], kn ^ (32u * i));
        vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
      wait_lds<0>();
    }

    // Main loop: tile T holds steps 2 T (parity 0) and 2 T + 1 (parity 1).
    // Step h issues the S^T products of step h + 1 in its slots 0..15 and the
    // PV products of step h - 1 in slots 16..31, with the softmax of step h
    // spread over the slots.  In the parity-0 step of tile T, after slot 9,
    // the wave waits for its DMA of tile T + 1 and all waves meet at a
    // barrier: tile T + 1 is then in the ring (its K rows are read from slot
    // 10 on), and every wave is past step 2 T - 1, so the slot of tile T - 2
    // (whose last V^T reads were in step 2 T - 2) is free for tile T + 2,
    // which is loaded after the barrier, half in each step.  A step past the
    // last one only computes unused products from finite ring contents.
    bool masked = k0 >= mask_kb;  // cinit holds the mask of the step being computed
    const bool track_pass = __builtin_amdgcn_readfirstlane(pass) == kTrack;  // (scalar)
    for (int32_t T = 0; T < ntiles; ++T) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int32_t h = 2 * T + par;
        const uint32_t ka_next = kaddr(h + 1);   // K of step h + 1
        const uint32_t ka_next2 = kaddr(h + 2);  // K of step h + 2
        const uint32_t va_prev = vaddr(h - 1);   // V of step h - 1
        const uint32_t va_cur = vaddr(h);        // V of step h
        f32x16_t(&sc_in)[2] = sacc[par];        // S^T of step h
        f32x16_t(&sc_out)[2] = sacc[par ^ 1];   // S^T of step h + 1
        u32x4_t(&p_out)[2][2] = pb[par];        // P^T of step h
        u32x4_t(&p_in)[2][2] = pb[par ^ 1];     // P^T of step h - 1
        DmaTile dd{};
        // The start blocks of step h + 1: uniform branches, taken only near
        // the diagonal and past the item's keys.
        {
          const int32_t kb1 = k0 + kStep * (h + 1);
          if (kb1 >= mask_kb) {
            set_mask(kb1);
            masked = true;
          } else if (masked) {
            clear_mask();
            masked = false;
          }
          cinit_ready();
        }
        __builtin_amdgcn_sched_barrier(0);

        // Each slot: one matrix product, then a share of the softmax, the
        // operand reads and the DMA.  The empty asm statements at the end of a
        // slot pin what the slot computed: without them the compiler sinks the
        // pure arithmetic to its first use, all of it behind the products.
#pragma unroll
        for (int sl = 0; sl < 32; ++sl) {
          // ---- matrix product of this slot -------------------------------------
          // (an odd slot's product reuses the operand of the slot before it)
          if ((sl & 1) == 0) wait_lds_n(reads_before(sl));
          if (sl < 16) {
            const int i = sl >> 1, rb = sl & 1;
            if (rb < kRB) {
              if (i == 0) mfma_s_first(sc_out[rb], kr[0], qf[rb][0], cinit[rb]);
              else mfma_s(sc_out[rb], kr[i % 4], qf[rb][i]);
            }
          } else {
            const int j = (sl - 16) >> 1, rb = (sl - 16) & 1;  // operand j = 4 kc + nb
            if (rb < kRB) mfma_pv(oacc[j & 3][rb], vr[j % 4], p_in[rb][j >> 2]);
            // the row sums of step h - 1: kc 0 in slot 17, kc 1 in slot 25
            if (sl == 17 || sl == 25) {
#pragma unroll
              for (int rs = 0; rs < kRB; ++rs)
                mfma_sum(ssum[rs], sel_ones, p_in[rs][(sl - 17) / 8]);
            }
          }
          // ---- kTrack passes: each row's largest raw score of step h -----------
          // (the scale is positive, so it gives the largest S'; masked scores
          // stay near kMinusBig).  A uniform branch, before the first exp of
          // the step overwrites its score.
          if (sl == 0 && track_pass) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              float a = rmax[rb];
#pragma unroll
              for (int i = 0; i < 16; i += 2) a = fmaxf(a, fmaxf(sc_in[rb][i], sc_in[rb][i + 1]));
              rmax[rb] = a;
            }
          }
          // ---- operand reads of this slot --------------------------------------
          if (sl == 0) {
            ds_vt(vr[3], va_prev ^ (64u * 3));  // V^T (h - 1, 3): kc 0, nb 3
          } else if (sl >= 2 && sl <= 8 && (sl & 1) == 0) {
            const int i = sl / 2 + 3;  // K (h + 1, 4..7)
            ds_k(kr[i % 4], ka_next ^ (32u * i));
          } else if (sl >= 10 && sl <= 16 && (sl & 1) == 0) {
            const int i = (sl - 10) / 2;  // K (h + 2, 0..3)
            ds_k(kr[i], ka_next2 ^ (32u * i));
          } else if (sl >= 18 && sl <= 24 && (sl & 1) == 0) {
            const int j = (sl - 18) / 2 + 4;  // V^T (h - 1, 4..7): kc 1
            ds_vt(vr[j % 4], (va_prev ^ (64u * (j & 3))) + 4096u);
          } else if (sl >= 26 && (sl & 1) == 0) {
            const int j = (sl - 26) / 2;  // V^T (h, 0..2): kc 0
            ds_vt(vr[j], va_cur ^ (64u * j));
          }
          // ---- softmax of step h -----------------------------------------------
          // Spread over the 32 slots: S' = S * scale * log2 e - m and
          // P = exp2(S') for one element per even slot (with two 32-row
          // blocks: elements 0..3 in slots 0 and 1 and element e >= 4 in slot
          // e - 2); the bf16 pair of P two slots after its exps.
          {
            const int ne = exp_count(sl), e0 = exp_first(sl);
            auto soft_one = [&](int e) __attribute__((always_inline)) {
              const int rb = (e >> 4) & 1, i = e & 15;
              if (rb >= kRB) return;
              const float x = __builtin_fmaf(sc_in[rb][i], sc, -m[rb]);
              sc_in[rb][i] = __builtin_amdgcn_exp2f(x);
            };
            if (ne >= 1) soft_one(e0);
            if (ne >= 2) soft_one(e0 + 1);
            const int pp = pack_pair(sl);
            if (pp >= 0) {
              // bf16 pairs of P (their row sums come from mfma_sum)
              const int rb = (pp >> 3) & 1, kcc = (pp >> 2) & 1, e = pp & 3;
              if (rb < kRB) {
                const float x0 = sc_in[rb][8 * kcc + 2 * e], x1 = sc_in[rb][8 * kcc + 2 * e + 1];
                p_out[rb][kcc][e] = pack_bf16x2(x0, x1);
              }
            }
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              asm volatile("" : "+v"(sc_in[rb]));
              asm volatile("" : "+v"(p_out[rb][0]), "+v"(p_out[rb][1]));
            }
          }
          // ---- DMA of tile T + 2: slots 22, 25, 28, 31 of both steps -------------
          if (sl >= 22 && (sl - 22) % 3 == 0 && (sl - 22) / 3 < kDmaInst / 2) {
            const int idx = (sl - 22) / 3;
            const int x = (kDmaInst / 2) * par + idx;
            if (idx == 0) dd = dma_setup(T + 2);
            dma_x(dd, x);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (sl == 9 && par == 0) {
            // Tile T + 1 (this wave's DMA, then everyone's) is in the ring, and
            // every wave is past step 2 T - 1: the slot of tile T - 2 is free.
            wait_vmem<0>();
            barrier();
          }
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          asm volatile("" : "+v"(p_out[rb][0]), "+v"(p_out[rb][1]));
        if (par == 0 && h + 1 >= nsteps) break;
      }
    }
    // The PV products of the last step: V^T operands 0..2 were read by it,
    // the others are read here.
    {
      const int32_t hl = nsteps - 1;
      const uint32_t va_last = vaddr(hl);
      u32x4_t ve[5];
#pragma unroll
      for (int j = 3; j < 8; ++j) ds_vt(ve[j - 3], (va_last ^ (64u * (j & 3))) + 4096u * (j >> 2));
      wait_lds<0>();
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        if ((hl & 1) != par) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4_t va = j < 3 ? vr[j] : ve[j - 3];
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) mfma_pv(oacc[j & 3][rb], va, pb[par][rb][j >> 2]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          mfma_sum(ssum[rb], sel_ones, pb[par][rb][0]);
          mfma_sum(ssum[rb], sel_ones, pb[par][rb][1]);
        }
      }
      // Vector reads of O^T and the sums follow: wait states for the
      // products' latency.
      if constexpr (kRB == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(oacc[0][0]), "+a"(oacc[0][1]), "+a"(oacc[1][0]), "+a"(oacc[1][1]),
                       "+a"(oacc[2][0]), "+a"(oacc[2][1]), "+a"(oacc[3][0]), "+a"(oacc[3][1]),
                       "+a"(ssum[0]), "+a"(ssum[1]));
      else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(oacc[0][0]), "+a"(oacc[1][0]), "+a"(oacc[2][0]), "+a"(oacc[3][0]),
                       "+a"(ssum[0]));
    }

    // Did the item's rows stay in the window around their references?
    //   kFirst: by the row sums.  A row with s in [2^-64, 2^64] did; one with
    //   s finite and positive outside it gets reference m + log2 s for a final
    //   pass; one with s = 0 that has keys (every P underflowed; a tree row
    //   may have none), or with s not finite, needs the kTrack pass.  Rows
    //   past the causal limit of the item's keys have none.
    //   kTrack: by the largest S'.  A masked score leaves the products near
    //   kMinusBig, so its S' is near kMinusBig * scale - m: a row with no key
    //   in the item stays below half of that and did not leave the window;
    //   a row that did gets its largest scaled score as reference.
    //   kFinal: not checked.
    bool shift = false, track = false;
    if (pass == kTrack) {
      const float no_key = 0.5f * kMinusBig * sc;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float x = max_halves(rmax[rb]) * sc - m[rb];  // largest S' of the row
        const bool out = row_ok[rb] && x > no_key - m[rb] && (x > kWindow || x < -kWindow);
        shift |= out;
        m_keep[rb] = out ? m[rb] + x : m[rb];
      }
    } else if (pass == kFirst) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float sum = ssum[rb][0];
        const bool inside = sum >= 0x1p-64f && sum <= 0x1p64f;  // (false for NaN)
        const bool no_key = !tree && kend_row[rb] <= k0;
        const bool finite_pos = sum > 0.f && sum < INFINITY;
        const bool bad = row_ok[rb] && !inside && !(sum == 0.f && no_key);
        shift |= bad && finite_pos;
        track |= bad && !finite_pos;
        m_keep[rb] = bad && finite_pos ? m[rb] + log2f(sum) : m[rb];
      }
    }
    if (track) retrack = 1;
    if (shift) restart = 1;
    // Finish, before the workgroup learns whether the item is done over (a
    // pass that is done over stores its rows again, later in program order),
    // so that the stores overlap the wait for the other waves.  Every lane
    // holds its row's sum (ssum).  Lane l holds O^T[d][row] for d = 32 nb +
    // 8 b + 4 half + j (element 4 b + j of block nb); lanes l and l ^ 32 hold
    // the same row.  Output rows (bf16): one swap between the halves per pair
    // of b gives each lane eight consecutive dims (half 0 those of the even b,
    // half 1 those of the odd b), stored as 16 bytes.  Partial rows of a split
    // piece (float32): each lane's four consecutive dims are 16 bytes already.
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const float ltot = ssum[rb][0];
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      const float lse_nat = ltot > 0.f ? (m[rb] + log2f(ltot)) * kLn2 : -INFINITY;
      const int32_t i_tok = q0 + t_of[rb];
      const int32_t hh = h_of[rb];
      if (S == 1) {
        uint4 out[4][2];  // [nb][pair of b]
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            uint32_t w[2][2];  // [b of the pair][lo, hi]
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int b = 2 * pr + u;
              w[u][0] = pack_bf16x2(oacc[nb][rb][4 * b] * inv, oacc[nb][rb][4 * b + 1] * inv);
              w[u][1] =
                  pack_bf16x2(oacc[nb][rb][4 * b + 2] * inv, oacc[nb][rb][4 * b + 3] * inv);
            }
            const auto lo = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
            const auto hi = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
            out[nb][pr] = make_uint4(lo[0], hi[0], lo[1], hi[1]);
          }
        if (!row_ok[rb]) continue;
        bf16_t* orow = o + ((int64_t)i_tok * p.num_qo_heads + hh) * kD + 8 * half;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int pr = 0; pr < 2; ++pr)
            *reinterpret_cast<uint4*>(orow + 32 * nb + 16 * pr) = out[nb][pr];
        if (half == 0 && lse) lse[(int64_t)i_tok * p.num_qo_heads + hh] = lse_nat;
      } else {
        if (!row_ok[rb]) continue;
        const int64_t prow = (int64_t)part0 + (int64_t)s * n + t_of[rb];
        float* orow = p.part_o + (prow * p.num_qo_heads + hh) * kD + 4 * half;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            *reinterpret_cast<float4*>(orow + 32 * nb + 8 * b) =
                make_float4(oacc[nb][rb][4 * b] * inv, oacc[nb][rb][4 * b + 1] * inv,
                            oacc[nb][rb][4 * b + 2] * inv, oacc[nb][rb][4 * b + 3] * inv);
        if (half == 0) p.part_lse[prow * p.num_qo_heads + hh] = lse_nat;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    const bool do_track = __builtin_amdgcn_readfirstlane(retrack) != 0;
    const bool do_final = __builtin_amdgcn_readfirstlane(restart) != 0;
    barrier();  // every wave has read the flags
    if (do_track || do_final) {
      if (tid == 0) {  // ordered before any new write by the item's barriers
        restart = 0;
        retrack = 0;
      }
      pass = do_track ? kTrack : kFinal;
      continue;
    }
    pass = kFirst;
    ++idx;
  }
}

hipError_t launch_prefill(const DevPlan& p, const void* q, const void* k_cache,
                          const void* v_cache, Strides ks, Strides vs, void* o, float* lse,
                          hipStream_t stream) {
  const PrefillPart part{p, static_cast<const bf16_t*>(k_cache),
                         static_cast<const bf16_t*>(v_cache), ks, vs};
  hipLaunchKernelGGL(prefill_kernel, dim3(p.n_wgs[KC_PREFILL]), dim3(64 * kWaves), 0, stream,
                     part, part, p.n_wgs[KC_PREFILL], static_cast<const bf16_t*>(q),
                     static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_prefill2(const DevPlan& p0, const void* k0, const void* v0, Strides ks0,
                           Strides vs0, const DevPlan& p1, const void* k1, const void* v1,
                           Strides ks1, Strides vs1, const void* q, void* o, float* lse,
                           hipStream_t stream) {
  const PrefillPart a{p0, static_cast<const bf16_t*>(k0), static_cast<const bf16_t*>(v0), ks0,
                      vs0};
  const PrefillPart b{p1, static_cast<const bf16_t*>(k1), static_cast<const bf16_t*>(v1), ks1,
                      vs1};
  const int32_t w0 = p0.n_wgs[KC_PREFILL], w1 = p1.n_wgs[KC_PREFILL];
  hipLaunchKernelGGL(prefill_kernel, dim3(w0 + w1), dim3(64 * kWaves), 0, stream, a, b, w0,
                     static_cast<const bf16_t*>(q), static_cast<bf16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace rpa
