// Gather of the kept contraction slice, A[:, I], into a K-contiguous bf16
// panel padded with zeros to the GEMM tile depth.
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach (Formula Level):
// only the kept columns of the activation take part in the product.  Each
// lane owns one output position t (so a wave reads 64 consecutive kept
// indices, which lie close together because the index list is ascending)
// and the 8 rows of a row block reuse the same indices held in registers.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kPackT = 2048;   // output positions per workgroup (8 per lane)
constexpr int kPackRows = 8;   // rows per workgroup

template <bool BF16>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ src, int64_t src_hs, int64_t src_rs,
                                                   int src_group, const int32_t* __restrict__ idx, int64_t idx_hs,
                                                   int k, int k_pad, int rows, uint16_t* __restrict__ out,
                                                   int64_t out_hs) {
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * kPackT;
  const int r0 = blockIdx.y * kPackRows;
  const int32_t* ib = idx + (size_t)b * idx_hs;
  int cols[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = t0 + e * 256 + threadIdx.x;
    cols[e] = t < k ? ib[t] : -1;
  }
  const size_t sbase = (size_t)(b / src_group) * src_hs;
  uint16_t* ob = out + (size_t)b * out_hs;
  for (int rr = 0; rr < kPackRows; ++rr) {
    const int r = r0 + rr;
    if (r >= rows) break;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = 0;
      if (cols[e] >= 0) {
        const size_t off = sbase + (size_t)r * src_rs + cols[e];
        v[e] = BF16 ? ((const uint16_t*)src)[off] : f32_to_bf16(((const float*)src)[off]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + e * 256 + threadIdx.x;
      if (t < k_pad) ob[(size_t)r * k_pad + t] = v[e];
    }
  }
}

}  // namespace

hipError_t launch_pack(const void* src, bool src_bf16, int64_t src_hs, int64_t src_rs, int src_group,
                       const int32_t* idx, int64_t idx_hs, int k, int k_pad, int batch, int rows, uint16_t* out,
                       int64_t out_hs, hipStream_t s) {
  dim3 grid((k_pad + kPackT - 1) / kPackT, (rows + kPackRows - 1) / kPackRows, batch);
  if (src_bf16)
    pack_kernel<true><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows, out, out_hs);
  else
    pack_kernel<false><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows, out, out_hs);
  return hipGetLastError();
}

}  // namespace rmm
