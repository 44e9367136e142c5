// Page copies between paged pools and transfer buffers (gfx950).
//
// "Disaggregated prefill and decode" (Perplexity), sharded-transfer section:
// when the prefill and decode nodes shard the KV cache differently, pages are
// split or reconstructed by the ratio of the shards (a decoder rebuilds a
// full page from the halves sent by two prefill devices), and the HND layout
// keeps one head range of a page contiguous so that it moves as one write.
// The chunked-prefill post (prefix-cache section) reuses cached prefix
// blocks; a shared, partly filled tail block has to be copied before two
// requests append to it.  All of these are one operation here: copy heads
// [src_head0, src_head0 + num_heads) of page src_pages[i] of one pool into
// heads [dst_head0, ...) of page dst_pages[i] of another (or the same) pool,
// every slot and every element, with arbitrary strides on both sides, so an
// HND pool, an NHD buffer or a packed shard buffer are all just strides.
//
// One thread moves 16 bytes; block (i, y) copies part of page pair i.  A
// plain copy: the bits move unchanged.  HBM bound: 2 bytes of traffic per
// byte copied.

#include "common.h"
#include "../launch.h"

namespace rpa {

namespace {

__global__ __launch_bounds__(256) void page_copy_kernel(
    const char* __restrict__ src, Strides src_b, const int32_t* src_pages, int32_t src_pool_pages,
    char* __restrict__ dst, Strides dst_b, const int32_t* dst_pages, int32_t dst_pool_pages,
    int32_t src_h0, int32_t dst_h0, int32_t num_heads, int32_t page_size, int32_t row_chunks) {
  const int32_t i = blockIdx.x;
  const int64_t sp = src_pages ? src_pages[i] : i;
  const int64_t dp = dst_pages ? dst_pages[i] : i;
  // Device-side page ids are not seen by the host: a pair with an id outside
  // its pool is skipped rather than read or written out of bounds.
  if (sp < 0 || sp >= src_pool_pages || dp < 0 || dp >= dst_pool_pages) return;
  const int32_t per_head = page_size * row_chunks;
  const int32_t total = num_heads * per_head;
  const char* s0 = src + sp * src_b.page + (int64_t)src_h0 * src_b.head;
  char* d0 = dst + dp * dst_b.page + (int64_t)dst_h0 * dst_b.head;
  for (int32_t c = blockIdx.y * blockDim.x + threadIdx.x; c < total;
       c += gridDim.y * blockDim.x) {
    const int32_t hh = c / per_head;
    const int32_t rem = c - hh * per_head;
    const int32_t slot = rem / row_chunks;
    const int32_t ch = rem - slot * row_chunks;
    const uint4 v = *reinterpret_cast<const uint4*>(s0 + hh * src_b.head + slot * src_b.token +
                                                    16 * ch);
    *reinterpret_cast<uint4*>(d0 + hh * dst_b.head + slot * dst_b.token + 16 * ch) = v;
  }
}

}  // namespace

hipError_t launch_page_copy(const void* src, Strides src_b, const int32_t* src_pages,
                            int32_t src_pool_pages, void* dst, Strides dst_b,
                            const int32_t* dst_pages, int32_t dst_pool_pages, int32_t num_pages,
                            int32_t src_h0, int32_t dst_h0, int32_t num_heads, int32_t page_size,
                            int32_t row_bytes, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  const int32_t row_chunks = row_bytes / 16;
  const int64_t per_page = (int64_t)num_heads * page_size * row_chunks;
  const int64_t ys = std::min<int64_t>((per_page + 255) / 256, 64);
  hipLaunchKernelGGL(page_copy_kernel, dim3((unsigned)num_pages, (unsigned)ys), dim3(256), 0,
                     stream, static_cast<const char*>(src), src_b, src_pages, src_pool_pages,
                     static_cast<char*>(dst), dst_b, dst_pages, dst_pool_pages, src_h0, dst_h0,
                     num_heads, page_size, row_chunks);
  return hipGetLastError();
}

}  // namespace rpa
