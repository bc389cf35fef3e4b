// Decode-shaped reduced product (n <= 16 rows of A): a bandwidth-bound
// GEMV that streams only the kept rows B[I, :].
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach: the product runs
// over the kept contraction indices only; with a handful of rows in A the
// cost is reading B, so reading ceil(rho d) of its d rows is the saving.
// Engineering Notes on the same page: prefill and decode are tuned apart.
//
// Layout: a 512-thread workgroup owns a 64-column strip (128 bytes of every
// kept row of B) and all kept rows: 8 lanes span the strip with 16-byte
// loads, 64 row lanes stride the kept rows, and each lane keeps a batch of
// 16 rows (8 for 16-row A) in flight while it multiplies the previous batch.  The kept
// row list is staged in LDS first.  The 64 row-lane partial sums of each
// output are folded in a fixed order (shuffles, then LDS), so the result is
// bitwise reproducible and no workgroup waits on another.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kThreads = 512;
constexpr int kCols = 64;                     // output columns per workgroup
constexpr int kLanesPerRow = kCols / 8;       // 16-byte lanes per row segment
constexpr int kRowLanes = kThreads / kLanesPerRow;
constexpr int kMaxKept = 16384;               // kept rows staged in LDS

template <int NR>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvArgs g) {
  constexpr int kBatch = NR >= 16 ? 8 : 16;   // kept rows in flight per lane
  __shared__ int32_t s_rows[kMaxKept];
  __shared__ float red[kThreads / 64][NR][kCols];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = tid % kLanesPerRow, rl = tid / kLanesPerRow;
  const int c = blockIdx.x * kCols + cl * 8;
  const bool col_ok = c < g.m;
  const int k = g.k;

  for (int i = tid; i < k; i += kThreads) s_rows[i] = g.idx[i];
  __syncthreads();

  float acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  auto load_batch = [&](int base, i32x4 (&bv)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = base + kRowLanes * u;
      if (t < k && col_ok)
        bv[u] = __builtin_nontemporal_load((const i32x4*)(g.B + (size_t)s_rows[t] * g.ldb + c));
      else
        bv[u] = i32x4{0, 0, 0, 0};
    }
  };
  auto fma_batch = [&](int base, const i32x4 (&bv)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = base + kRowLanes * u;
      if (t >= k) break;
      float a[NR];
      const f32x4* ap = (const f32x4*)(g.a_t + (size_t)t * 16);
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        const f32x4 v = ap[q];
        a[4 * q] = v[0];
        a[4 * q + 1] = v[1];
        a[4 * q + 2] = v[2];
        a[4 * q + 3] = v[3];
      }
      float bf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t bits = (uint32_t)bv[u][w];
        bf[2 * w] = __uint_as_float(bits << 16);
        bf[2 * w + 1] = __uint_as_float(bits & 0xffff0000u);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(a[r], bf[e], acc[r][e]);
    }
  };

  constexpr int STEP = kRowLanes * kBatch;
  i32x4 b0[kBatch], b1[kBatch];
  int base = rl;
  if (base < k) load_batch(base, b0);
  while (base < k) {
    const int next = base + STEP;
    if (next < k) load_batch(next, b1);
    fma_batch(base, b0);
    if (next >= k) break;
    const int next2 = next + STEP;
    if (next2 < k) load_batch(next2, b0);
    fma_batch(next, b1);
    base = next2;
  }

  // fold the 8 row lanes of each wave (lane bits 3..5), then the 8 waves
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[r][e];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[r][e] = v;
    }
  if (lane < kLanesPerRow) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][r][cl * 8 + e] = acc[r][e];
  }
  __syncthreads();
  for (int i = tid; i < g.n * kCols; i += kThreads) {
    const int r = i / kCols, cc = i % kCols;
    const int col = blockIdx.x * kCols + cc;
    if (col >= g.m) continue;
    float v = red[0][r][cc];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v += red[w][r][cc];
    const size_t off = (size_t)r * g.ldy + col;
    if (g.y_bf16)
      ((uint16_t*)g.Y)[off] = f32_to_bf16(v);
    else
      ((float*)g.Y)[off] = v;
  }
}

}  // namespace

int gemv_max_kept() { return kMaxKept; }

hipError_t launch_gemv(const GemvArgs& g, hipStream_t s) {
  dim3 grid((g.m + kCols - 1) / kCols);
  if (g.n <= 4)
    gemv_kernel<4><<<grid, kThreads, 0, s>>>(g);
  else if (g.n <= 8)
    gemv_kernel<8><<<grid, kThreads, 0, s>>>(g);
  else
    gemv_kernel<16><<<grid, kThreads, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace rmm
