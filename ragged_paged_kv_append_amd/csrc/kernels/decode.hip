// Decode / speculative-verify attention (bf16, head dim 128, page size a
// multiple of 16): the HBM-streaming kernel.
//
// The disaggregation post (prefill/decode performance section) notes that
// decode is memory bound: a few query rows per KV head read the whole KV
// range.  A one-wave workgroup runs its list of work items, in turn; an item
// is request r, KV head g, all of its n_r * G query rows (at most 16: decode
// rows and verify rows of n + 1 draft tokens, "Accelerating Sonar through
// speculation"), keys [k0, k1).  The item streams its keys in tiles of 16
// tokens (one page head slice for P = 16, a quarter page for P = 64), so every
// tile is one contiguous 4 KiB run of K and one of V in the HND layout.
//
// Streaming: tiles move from HBM into a ring of kStages LDS slots with the
// gfx950 global-to-LDS DMA (global_load_lds_dwordx4, 1 KiB per instruction),
// issued kStages - 1 tiles ahead of the tile being computed.  The waits on
// the DMA are explicit vmcnt counts, so kStages - 1 tiles (24 KiB per wave)
// stay in flight through the whole loop without holding any registers.
// Within a slot, the 16-byte chunk c of row j sits at position c ^ j of the
// row, so the K-operand reads and the transposing V reads are free of bank
// conflicts.
//
// Per tile, with 16x16 MFMA tiles and query rows padded to 16:
//   S^T[key][row] = K[key][:] . Q[row][:]      4 x mfma 16x16x32 bf16, K read
//       from the slot (each lane: 64 bytes of one key row), Q in registers;
//   online softmax on S^T: each lane holds 4 keys of one query row;
//   O^T[d][row] += V^T[d][keys] . P^T[keys][row]   8 x mfma 16x16x16 bf16; the
//       S^T accumulator layout is exactly the B operand layout of P^T, so P
//       never moves between lanes; V^T comes from the slot through the
//       transposing LDS read.
// Keys past the item's end are fetched from its last key (a written slot of
// the same page), so the masked tail multiplies finite values by zero.


#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

constexpr int kD = 128;
constexpr int kTile = 16;    // keys per tile
constexpr int kTileElems = kTile * kD;
constexpr float kMinusBig = -1.0e30f;
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr int kNonTemporal = 2;  // cache-policy bit of the DMA loads: streaming data

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Waits for every LDS operation of this wave.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void_t;

// Blocking scalar load of one page id.  The page table is read through the
// scalar cache and the wait covers only LDS/scalar operations, never the DMA
// stream in flight.
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

// The eight transposing reads of a V tile (blocks nb = 0..7 of 16 value dims)
// for the lane whose row is `vrow`: block nb sits in chunk (2 nb + vhalf) ^ vrow.
// Written as one asm block with its own LDS wait: the compiler cannot tell
// these reads from the in-flight DMA and would otherwise drain the whole DMA
// stream before them.
__device__ __forceinline__ void read_vt(const bf16_t* row_base, int vrow, int vhalf,
                                        s16x4_t (&va)[8]) {
  typedef __attribute__((address_space(3))) const bf16_t* lds_ptr_t;
  uint32_t a[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    a[nb] = (uint32_t)(uintptr_t)(lds_ptr_t)(row_base + 8 * ((2 * nb + vhalf) ^ vrow));
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(va[0]), "=&v"(va[1]), "=&v"(va[2]), "=&v"(va[3]), "=&v"(va[4]), "=&v"(va[5]),
        "=&v"(va[6]), "=&v"(va[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// O^T += V^T P^T for the eight 16-dim blocks, issued from inline assembly so
// that the accumulators are VGPR operands: left to the compiler they live in
// AGPRs and are copied to VGPRs and back around every tile (the lazy rescale
// reads them with vector instructions), about a hundred extra instructions
// per tile.  The compiler does not see these as matrix instructions, so the
// wait states it would add are written here: two before the first product
// (P, and maybe a copy of an accumulator, were just written by vector
// instructions) and 24 after the last, more than any product needs before a
// vector instruction reads or overwrites its registers (the compiler may
// copy the accumulators right after this block).
__device__ __forceinline__ void pv_products(f32x4_t (&acc)[8], const s16x4_t (&va)[8],
                                            s16x4_t pb) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x16_bf16 %0, %8, %16, %0\n\t"
      "v_mfma_f32_16x16x16_bf16 %1, %9, %16, %1\n\t"
      "v_mfma_f32_16x16x16_bf16 %2, %10, %16, %2\n\t"
      "v_mfma_f32_16x16x16_bf16 %3, %11, %16, %3\n\t"
      "v_mfma_f32_16x16x16_bf16 %4, %12, %16, %4\n\t"
      "v_mfma_f32_16x16x16_bf16 %5, %13, %16, %5\n\t"
      "v_mfma_f32_16x16x16_bf16 %6, %14, %16, %6\n\t"
      "v_mfma_f32_16x16x16_bf16 %7, %15, %16, %7\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
        "+v"(acc[6]), "+v"(acc[7])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]),
        "v"(va[7]), "v"(pb));
}

}  // namespace

// kStages: LDS ring depth in tiles (8 KiB each); kStages - 1 tiles are in flight.
template <int kStages>
__global__ __launch_bounds__(64) void decode_kernel(DevPlan p, const bf16_t* __restrict__ q,
                                                    const bf16_t* __restrict__ kc,
                                                    const bf16_t* __restrict__ vc, Strides ks,
                                                    Strides vs, bf16_t* __restrict__ o,
                                                    float* __restrict__ lse) {
  // ring[slot][0] = K tile, ring[slot][1] = V tile, rows of 128 bf16.
  __shared__ __attribute__((aligned(1024))) bf16_t ring[kStages][2][kTileElems];
  const int lane = threadIdx.x;
  const int col = lane & 15;  // query row of S^T / P^T / O^T columns; key row of the K operand
  const int grp = lane >> 4;  // which 32-element quarter of a row this lane reads

  // This workgroup's items (its wg_indptr range), in turn.
  const int32_t wb0 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_DECODE][blockIdx.x]);
  const int32_t wb1 = __builtin_amdgcn_readfirstlane(p.wg_indptr[KC_DECODE][blockIdx.x + 1]);
  for (int32_t idx = wb0; idx < wb1; ++idx) {
  const int32_t* it = p.items[KC_DECODE] + (int64_t)idx * IT_WORDS;
  const int32_t r = it[IT_REQ], g = it[IT_KVHEAD], rows = it[IT_ROW1];
  const int32_t k0 = it[IT_K0], k1 = it[IT_K1], s = it[IT_SPLIT];
  const int32_t G = p.group;
  const int32_t q0 = p.qo_indptr[r];
  const int32_t n = p.qo_indptr[r + 1] - q0;
  const int32_t L = p.kv_len[r];
  const int32_t cached = L - n;

  // A request with a tree mask sees every key up to L - 1, filtered among
  // the new tokens by its mask row (at most 16 new tokens here).
  const bool tree = p.tree_mask != nullptr && p.tree_req[r] != 0;
  const bool causal = p.causal && !tree;

  // This lane's query row (as a column of S^T).
  const bool row_ok = col < rows;
  const int32_t t = row_ok ? col / G : 0;
  const int32_t h = g * G + (row_ok ? col % G : 0);
  const int32_t kend_row = row_ok ? min(k1, (causal ? cached + t : L - 1) + 1) : k0;
  const int32_t t_last = (rows - 1) / G;
  const int32_t kend = min(k1, (causal ? cached + t_last : L - 1) + 1);
  // Last key (exclusive) of the item's first row: tiles below it need no
  // mask, except that a tree mask filters the new tokens (keys >= cached).
  const int32_t kend_first = min(k1, (causal ? cached : L - 1) + 1);
  const int32_t mask_from = tree ? min(kend_first, cached) : kend_first;
  const uint32_t tmask = (tree && row_ok) ? p.tree_mask[2 * (int64_t)(q0 + t)] : 0u;

  // Q operand: qf[j] = Q[row][32 grp + 8 j .. + 8), the dims of chunk 4 grp + j.
  u32x4_t qf[4];
  {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        q + ((int64_t)(q0 + t) * p.num_qo_heads + h) * kD + 32 * grp);
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[j] = row_ok ? qp[j] : u32x4_t{0u, 0u, 0u, 0u};
    // Use Q here so that its load completes before the DMA stream starts: the
    // loop below then owns the vector-memory counter.
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]));
  }

  const int32_t* pages = p.page_indices + p.page_indptr[r];
  // The item's first 256 page ids, one per lane of pidv[c] (page pg0 + 64 c +
  // lane), loaded with Q before the DMA stream starts: a tile then takes its
  // page id with v_readlane instead of a scalar load and wait.  Pages past
  // the first 256 (items longer than 4096 keys at page size 16) use the
  // scalar load.
  const int32_t pg0 = k0 >> p.page_shift;
  const int32_t npg_req = p.page_indptr[r + 1] - p.page_indptr[r];
  int32_t pidv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int32_t pi = pg0 + 64 * c + lane;
    pidv[c] = pi < npg_req ? pages[pi] : 0;
  }
  asm volatile("" ::"v"(pidv[0]), "v"(pidv[1]), "v"(pidv[2]), "v"(pidv[3]));
  // DMA role: instruction i of a tile moves rows 4 (i % 4) + lane / 16, chunk
  // (lane % 16) ^ row into LDS position lane % 16 of that row.
  const int drow = lane >> 4;
  const int64_t k_head = (int64_t)g * ks.head;
  const int64_t v_head = (int64_t)g * vs.head;
  auto page_of = [&](int32_t kb) __attribute__((always_inline)) -> int64_t {
    const int32_t i = (kb >> p.page_shift) - pg0;  // wave-uniform
    if (i < 64) return __builtin_amdgcn_readlane(pidv[0], i);
    if (i < 128) return __builtin_amdgcn_readlane(pidv[1], i - 64);
    if (i < 192) return __builtin_amdgcn_readlane(pidv[2], i - 128);
    if (i < 256) return __builtin_amdgcn_readlane(pidv[3], i - 192);
    return load_scalar(pages + (kb >> p.page_shift));
  };
  // Byte offsets, from the tile's first key, of this lane's four K and four V
  // chunks: the same for every tile that lies inside its page and the item,
  // whose DMA then needs only a wave-uniform base per tile.
  uint32_t koff[4], voffs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + drow;
    const uint32_t chunk = (uint32_t)((lane & 15) ^ row);
    koff[i] = (uint32_t)row * 2u * (uint32_t)ks.token + 16u * chunk;
    voffs[i] = (uint32_t)row * 2u * (uint32_t)vs.token + 16u * chunk;
  }
  auto issue = [&](int32_t kb, int slot) {
    const int64_t page = page_of(kb);
    const bf16_t* kpage = kc + page * ks.page + k_head;
    const bf16_t* vpage = vc + page * vs.page + v_head;
    if (kb + kTile <= k1) {
      const int64_t in_page = kb & (p.page_size - 1);
      const char* kbase = reinterpret_cast<const char*>(kpage + in_page * ks.token);
      const char* vbase = reinterpret_cast<const char*>(vpage + in_page * vs.token);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_global_load_lds(kbase + koff[i], (lds_void_t*)&ring[slot][0][512 * i], 16,
                                         0, kNonTemporal);
        __builtin_amdgcn_global_load_lds(vbase + voffs[i], (lds_void_t*)&ring[slot][1][512 * i],
                                         16, 0, kNonTemporal);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + drow;
      const int32_t key = min(kb + row, k1 - 1);
      const int64_t slot_in_page = key & (p.page_size - 1);
      const int chunk = (lane & 15) ^ row;
      __builtin_amdgcn_global_load_lds(kpage + slot_in_page * ks.token + 8 * chunk,
                                       (lds_void_t*)&ring[slot][0][512 * i], 16, 0,
                                       kNonTemporal);
      __builtin_amdgcn_global_load_lds(vpage + slot_in_page * vs.token + 8 * chunk,
                                       (lds_void_t*)&ring[slot][1][512 * i], 16, 0,
                                       kNonTemporal);
    }
  };

  const float sc = p.sm_scale * kLog2e;
  float m = kMinusBig;  // running max of this row, log2 units
  float lsum = 0.f;     // this lane's share of the running sum (its 4 keys per tile)
  f32x4_t acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Transposing-read address of this lane inside a V tile: row 4 grp + col / 4,
  // element column 16 nb + 4 (col % 4), i.e. chunk 2 nb + (col % 4) / 2.
  const int vrow = 4 * grp + (col >> 2);
  const int vhalf = (col >> 1) & 1;
  const int voff = 4 * (col & 1);

  const int32_t ntiles = (kend - k0 + kTile - 1) / kTile;
  // The previous item's output stores count in the same vector-memory counter
  // and may complete after later loads, which would let the counted waits
  // below pass early: drain them before this item's DMA stream starts.
  if (idx > wb0) wait_vmem<0>();
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < ntiles) issue(k0 + j * kTile, j);

  for (int32_t tile = 0; tile < ntiles; ++tile) {
    const int32_t kb = k0 + tile * kTile;
    const int slot = tile % kStages;
    if (tile + kStages - 1 < ntiles) {
      wait_lds();  // the slot about to be refilled was read by the previous tile
      issue(kb + (kStages - 1) * kTile, (tile + kStages - 1) % kStages);
      wait_vmem<8 * (kStages - 1)>();  // this tile's 8 DMA instructions are done
    } else {
      wait_vmem<0>();
    }
    const bf16_t* kt = ring[slot][0];
    const bf16_t* vt = ring[slot][1];

    // S^T = K . Q^T
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(kt + col * kD + 8 * ((4 * grp + j) ^ col));
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[j]), sacc, 0, 0,
                                                     0);
    }
    // Online softmax for query row `col`; this lane holds keys kb + 4*grp + e.
    // Only a tile that reaches past some row's last key, or holds new tokens
    // of a tree-masked request, needs the mask: one compare and one select
    // per key (plus the bit test for trees), with no per-key branches.
    float sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = sacc[e] * sc;
    if (kb + kTile > mask_from) {
      if (!tree) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = kb + 4 * grp + e < kend_row ? sv[e] : kMinusBig;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t key = kb + 4 * grp + e;
          const int32_t u = key - cached;  // new-token index (< 0: a cached key)
          const bool in_tree = u < 0 || ((tmask >> (uint32_t)(u & 31)) & 1u) != 0;
          sv[e] = (key < kend_row) & in_tree ? sv[e] : kMinusBig;
        }
      }
    }
    // The reference max moves only when the tile beats it by more than the
    // slack (P then stays below 2^8), so O is rescaled on few tiles.  The
    // row's largest score (a reduction over the four lanes of the row) is
    // needed only when some lane's own beats its reference: a wave-uniform
    // vote skips the reduction on the other tiles.
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      mx = max_halves(max_rows16(mx));
      if (mx > m + kRescaleSlack) {
        if (m > 0.5f * kMinusBig) alpha = __builtin_amdgcn_exp2f(m - mx);
        m = mx;
      }
    }
    // Masked keys sit at kMinusBig; a row with no key yet takes reference 0,
    // so they still come out as 0.
    const float neg_m = m > 0.5f * kMinusBig ? -m : 0.f;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(sv[e] + neg_m);
    const u32x2_t pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
    // Plain adds for the row sum: v_dot2 would serialise against the matrix
    // products of the other waves on this SIMD.
    lsum = lsum * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, pw);
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[nb] *= alpha;
    }

    // O^T += V^T P^T, V^T of block nb through the transposing read.
    s16x4_t va[8];
    read_vt(vt + vrow * kD + voff, vrow, vhalf, va);
    pv_products(acc, va, pb);
  }

  // Row sum over the four lane groups, then normalise and store.
  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (row_ok) {
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse_nat = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  const int32_t i = q0 + t;
  const int32_t S = p.split[r * SP_WORDS + SP_COUNT];
  // The output row (bf16), or the float32 row of piece s's partial.
  const int64_t prow = (int64_t)p.split[r * SP_WORDS + SP_BASE] + (int64_t)s * n + t;
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
  } else {
    float* orow = p.part_o + (prow * p.num_qo_heads + h) * kD + 4 * grp;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<float4*>(orow + 16 * nb) =
          make_float4(acc[nb][0] * inv, acc[nb][1] * inv, acc[nb][2] * inv, acc[nb][3] * inv);
  }
  if (grp == 0) {
    if (S == 1) {
      if (lse) lse[(int64_t)i * p.num_qo_heads + h] = lse_nat;
    } else {
      p.part_lse[prow * p.num_qo_heads + h] = lse_nat;
    }
  }
  }  // row_ok
  }  // items
}

hipError_t launch_decode(const DevPlan& p, const void* q, const void* k_cache, const void* v_cache,
                         Strides ks, Strides vs, void* o, float* lse, hipStream_t stream) {
  // Ring depth: the planner's choice (3 tiles, 24 KiB of LDS per wave, six
  // waves per CU, for one item per workgroup; 2 tiles, 16 KiB, for the cut
  // lists it sizes for eight resident waves per CU).
  const dim3 grid(p.n_wgs[KC_DECODE]), block(64);
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kk = static_cast<const bf16_t*>(k_cache);
  const bf16_t* vv = static_cast<const bf16_t*>(v_cache);
  bf16_t* oo = static_cast<bf16_t*>(o);
  if (p.dec_stages == 2)
    hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, p, qq, kk, vv, ks, vs, oo, lse);
  else
    hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, p, qq, kk, vv, ks, vs, oo, lse);
  return hipGetLastError();
}

}  // namespace rpa
