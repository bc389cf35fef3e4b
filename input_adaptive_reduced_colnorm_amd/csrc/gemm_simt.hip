// Reduced product on the vector ALUs, for fp32 inputs and for operands whose
// strides or alignment rule out the 16-byte matrix-core loaders.
//
// Computes C[b][i][j] = sum over t < k of A(b, i, col(t)) * B(b / group,
// row(t), j), where col(t) = row(t) = I[t] (the kept contraction indices of
// "Algorithm Deep-Dive: RMM", Core Approach) or t when no index is given.
// Every operand is addressed through explicit strides, so the same kernel
// covers X W (linear), Q K^T (per head, K read through its kv head) and P V.
// fp32 multiply-add with fp32 accumulation, 64 x 64 output tiles.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int TS = 64, TK = 16;

template <bool ABF, bool BBF, bool CBF>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const SimtArgs g) {
  __shared__ float As[TK][TS + 4];
  __shared__ float Bs[TK][TS + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int b = blockIdx.z;
  const int m0 = blockIdx.y * TS, n0 = blockIdx.x * TS;
  const char* Ab = (const char*)g.A + (size_t)b * g.a_bs * (ABF ? 2 : 4);
  const char* Bb = (const char*)g.B + (size_t)(b / g.b_group) * g.b_bs * (BBF ? 2 : 4);
  const int32_t* ib = g.idx ? g.idx + (size_t)b * g.idx_bs : nullptr;

  auto ld = [](const char* base, size_t off, bool bf) -> float {
    return bf ? bf16_to_f32(((const uint16_t*)base)[off]) : ((const float*)base)[off];
  };

  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.k; k0 += TK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int i = e >> 4, kk = e & 15;
      const int t = k0 + kk;
      float v = 0.f;
      if (m0 + i < g.M && t < g.k) {
        const int64_t col = ib ? ib[t] : t;   // -1: an index that contributes nothing
        if (col >= 0) v = ld(Ab, (size_t)((int64_t)(m0 + i) * g.a_rs + col * g.a_cs), ABF);
      }
      As[kk][i] = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int kk = e >> 6, j = e & 63;
      const int t = k0 + kk;
      float v = 0.f;
      if (n0 + j < g.N && t < g.k) {
        const int64_t row = ib ? ib[t] : t;
        if (row >= 0) v = ld(Bb, (size_t)(row * g.b_ts + (int64_t)(n0 + j) * g.b_js), BBF);
      }
      Bs[kk][j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = As[kk][ty * 4 + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx * 4 + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
  char* Cb = (char*)g.C + (size_t)b * g.c_bs * (CBF ? 2 : 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = m0 + ty * 4 + r;
    if (i >= g.M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = n0 + tx * 4 + c;
      if (j >= g.N) continue;
      const size_t off = (size_t)i * g.ldc + j;
      const float y = g.causal && (int64_t)j > (int64_t)i + g.causal_off ? -INFINITY : acc[r][c];
      if (CBF)
        ((uint16_t*)Cb)[off] = f32_to_bf16(y);
      else
        ((float*)Cb)[off] = y;
    }
  }
}

template <bool ABF, bool BBF>
void run_simt(const SimtArgs& g, dim3 grid, hipStream_t s) {
  if (g.c_bf16)
    gemm_simt_kernel<ABF, BBF, true><<<grid, 256, 0, s>>>(g);
  else
    gemm_simt_kernel<ABF, BBF, false><<<grid, 256, 0, s>>>(g);
}

}  // namespace

hipError_t launch_gemm_simt(const SimtArgs& g, hipStream_t s) {
  dim3 grid((g.N + TS - 1) / TS, (g.M + TS - 1) / TS, g.batch);
  if (g.a_bf16) {
    if (g.b_bf16)
      run_simt<true, true>(g, grid, s);
    else
      run_simt<true, false>(g, grid, s);
  } else {
    if (g.b_bf16)
      run_simt<false, true>(g, grid, s);
    else
      run_simt<false, false>(g, grid, s);
  }
  return hipGetLastError();
}

}  // namespace rmm
