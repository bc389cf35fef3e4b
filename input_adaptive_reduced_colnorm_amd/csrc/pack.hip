// Gather of the kept contraction slice, A[:, I], into a K-contiguous bf16
// panel padded with zeros to the GEMM tile depth.
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach (Formula Level):
// only the kept columns of the activation take part in the product.  Each
// lane owns output positions t (so a wave reads 64 consecutive kept
// indices, which lie close together because the index list is ascending);
// the 8 rows of a row block reuse the same indices held in registers, all 64
// gathers of a lane are in flight together, and the values pass through LDS
// so that the panel is written with 16-byte stores.  k_pad is a multiple of
// 8, so every 16-byte piece lies inside the padded row.

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
  // the gathered values of all rows go through LDS so that every lane
  // writes whole 16-byte pieces of an output row
  __shared__ __attribute__((aligned(16))) uint16_t s_out[kPackRows][kPackT];
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
  uint16_t v[kPackRows][8];
#pragma unroll
  for (int rr = 0; rr < kPackRows; ++rr) {
    const int r = min(r0 + rr, rows - 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[rr][e] = 0;
      if (cols[e] >= 0) {
        const size_t off = sbase + (size_t)r * src_rs + cols[e];
        v[rr][e] = BF16 ? ((const uint16_t*)src)[off] : f32_to_bf16(((const float*)src)[off]);
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kPackRows; ++rr)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_out[rr][e * 256 + threadIdx.x] = v[rr][e];
  __syncthreads();
  uint16_t* ob = out + (size_t)b * out_hs;
  const int t = t0 + threadIdx.x * 8;
  if (t < k_pad) {
#pragma unroll
    for (int rr = 0; rr < kPackRows; ++rr) {
      const int r = r0 + rr;
      if (r >= rows) break;
      *(i32x4*)(ob + (size_t)r * k_pad + t) = *(const i32x4*)&s_out[rr][threadIdx.x * 8];
    }
  }
}

// Narrow rows (k_pad <= 256, e.g. the head features of attention): each lane
// owns one 16-byte piece (8 kept positions) of an output row, so k_pad / 8
// lanes cover a row and a workgroup covers 256 / (k_pad / 8) rows per pass.
constexpr int kNarrowMax = 256;
constexpr int kNarrowPasses = 8;

template <bool BF16>
__global__ __launch_bounds__(256) void pack_narrow_kernel(const void* __restrict__ src, int64_t src_hs,
                                                          int64_t src_rs, int src_group,
                                                          const int32_t* __restrict__ idx, int64_t idx_hs, int k,
                                                          int k_pad, int rows, uint16_t* __restrict__ out,
                                                          int64_t out_hs) {
  const int b = blockIdx.y;
  const int cpr = k_pad >> 3;                 // pieces per row, at most 32
  const int rstep = 256 / cpr;                // rows per pass
  if ((int)threadIdx.x >= rstep * cpr) return;
  const int piece = threadIdx.x % cpr;
  const int32_t* ib = idx + (size_t)b * idx_hs;
  int cols[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = piece * 8 + e;
    cols[e] = t < k ? ib[t] : -1;
  }
  const size_t sbase = (size_t)(b / src_group) * src_hs;
  uint16_t* ob = out + (size_t)b * out_hs;
  const int r0 = blockIdx.x * rstep * kNarrowPasses + threadIdx.x / cpr;
#pragma unroll
  for (int pass = 0; pass < kNarrowPasses; ++pass) {
    const int r = r0 + pass * rstep;
    if (r >= rows) break;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (cols[e] >= 0) {
        const size_t off = sbase + (size_t)r * src_rs + cols[e];
        const uint32_t h = BF16 ? ((const uint16_t*)src)[off] : f32_to_bf16(((const float*)src)[off]);
        w[e >> 1] |= h << (16 * (e & 1));
      }
    }
    *(i32x4*)(ob + (size_t)r * k_pad + piece * 8) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  }
}

}  // namespace

hipError_t launch_pack(const void* src, bool src_bf16, int64_t src_hs, int64_t src_rs, int src_group,
                       const int32_t* idx, int64_t idx_hs, int k, int k_pad, int batch, int rows, uint16_t* out,
                       int64_t out_hs, hipStream_t s) {
  if (k_pad <= kNarrowMax) {
    const int rows_per_wg = 256 / (k_pad / 8) * kNarrowPasses;
    dim3 grid((rows + rows_per_wg - 1) / rows_per_wg, batch);
    if (src_bf16)
      pack_narrow_kernel<true><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows, out,
                                                    out_hs);
    else
      pack_narrow_kernel<false><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows,
                                                     out, out_hs);
    return hipGetLastError();
  }
  dim3 grid((k_pad + kPackT - 1) / kPackT, (rows + kPackRows - 1) / kPackRows, batch);
  if (src_bf16)
    pack_kernel<true><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows, out, out_hs);
  else
    pack_kernel<false><<<grid, 256, 0, s>>>(src, src_hs, src_rs, src_group, idx, idx_hs, k, k_pad, rows, out, out_hs);
  return hipGetLastError();
}

}  // namespace rmm
