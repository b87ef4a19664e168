// Append one token's K and V row per (sequence, KV head) into the paged
// pools: the "decode one new token at a time" step of the RetrievalAttention
// slides' setting frame ("One question: how can decoding read less KV?").
#include "ra_internal.h"

namespace ra {

// One 32-lane block per (b, g): lanes 0..15 copy the K row, 16..31 the V row,
// 16 bytes each.
__global__ __launch_bounds__(32) void kv_append_kernel(ra_kv_layer kv,
                                                       const uint16_t* k_new,
                                                       const uint16_t* v_new,
                                                       const int32_t* pos) {
  const int bg = blockIdx.x;
  const int b = bg / kv.H_kv;
  const int g = bg - b * kv.H_kv;
  const int lane = threadIdx.x;
  const int ps = pos[b];
  if (ps < 0 || ps >= kv.max_pages * kPage) return;
  const int pg = kv.block_table[(size_t)b * kv.max_pages + ps / kPage];
  if ((unsigned)pg >= (unsigned)kv.num_pages) return;
  const int part = lane >> 4;  // 0: K, 1: V
  const int c = lane & 15;
  const uint16_t* src = (part ? v_new : k_new) + (size_t)bg * kHeadDim + c * 8;
  uint16_t* dst = (part ? kv.v_pool : kv.k_pool) +
                  (((size_t)pg * kv.H_kv + g) * kPage + (ps & (kPage - 1))) *
                      kHeadDim +
                  c * 8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

hipError_t launch_kv_append(const ra_kv_layer& kv, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* pos,
                            int32_t B, hipStream_t s) {
  const unsigned blocks = unsigned(B) * unsigned(kv.H_kv);
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(32), 0, s, kv, k_new,
                     v_new, pos);
  return hipGetLastError();
}

}  // namespace ra
