// Decode-shaped reduced product (n <= 16 rows of A): a bandwidth-bound
// GEMV that streams only the kept rows B[I, :].
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach: the product runs
// over the kept contraction indices only; with a handful of rows in A the
// cost is reading B, so reading ceil(rho d) of its d rows is the saving.
// Engineering Notes on the same page: prefill and decode are tuned apart.
//
// Layout: a workgroup owns a 128-column strip and a contiguous split of the
// kept rows; 16 lanes cover the strip with 16-byte loads and 16 row lanes
// stride the rows, four rows in flight per lane.  Partial sums are combined
// in a fixed order: across row lanes (shuffles, then LDS), then across
// splits by whichever workgroup of a strip finishes last (integer ticket),
// so the result is bitwise reproducible.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kCols = 128;
constexpr int kRowLanes = 16;
constexpr int kUnroll = 4;

template <int NR>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvArgs g) {
  __shared__ float red[4][NR][kCols];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = tid & 15, rg = tid >> 4;
  const int strip = blockIdx.x, split = blockIdx.y;
  const int c = strip * kCols + cl * 8;
  const bool col_ok = c < g.m;
  const int t_begin = split * g.rows_per_split;
  const int t_end = min(g.k, t_begin + g.rows_per_split);

  float acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  for (int t = t_begin + rg; t < t_end; t += kRowLanes * kUnroll) {
    int rows[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kRowLanes * u;
      rows[u] = tt < t_end ? g.idx[tt] : -1;
    }
    i32x4 bv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (rows[u] >= 0 && col_ok)
        bv[u] = __builtin_nontemporal_load((const i32x4*)(g.B + (size_t)rows[u] * g.ldb + c));
      else
        bv[u] = i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tt = t + kRowLanes * u;
      if (tt >= t_end) break;
      float a[NR];
      const f32x4* ap = (const f32x4*)(g.a_t + (size_t)tt * 16);
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        f32x4 v = ap[q];
        a[4 * q] = v[0];
        a[4 * q + 1] = v[1];
        a[4 * q + 2] = v[2];
        a[4 * q + 3] = v[3];
      }
      float bf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t bits = (uint32_t)bv[u][w];
        bf[2 * w] = __uint_as_float(bits << 16);
        bf[2 * w + 1] = __uint_as_float(bits & 0xffff0000u);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(a[r], bf[e], acc[r][e]);
    }
  }

  // fold the four row lanes of each wave (lanes differing in bits 4 and 5)
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[r][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[r][e] = v;
    }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][r][cl * 8 + e] = acc[r][e];
  }
  __syncthreads();
  float* part = g.partial + (size_t)split * 16 * g.m;
  for (int i = tid; i < NR * kCols; i += 256) {
    const int r = i / kCols, cc = i % kCols;
    const int col = strip * kCols + cc;
    const float v = ((red[0][r][cc] + red[1][r][cc]) + red[2][r][cc]) + red[3][r][cc];
    if (col < g.m) part[(size_t)r * g.m + col] = v;
  }
  // ticket: the last workgroup of this strip sums the splits in order
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t prev = __hip_atomic_fetch_add(&g.counters[strip], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)(gridDim.y - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int i = tid; i < g.n * kCols; i += 256) {
    const int r = i / kCols, cc = i % kCols;
    const int col = strip * kCols + cc;
    if (col >= g.m) continue;
    float v = 0.f;
    for (int sp = 0; sp < (int)gridDim.y; ++sp)
      v += __builtin_nontemporal_load(g.partial + ((size_t)sp * 16 + r) * g.m + col);
    const size_t off = (size_t)r * g.ldy + col;
    if (g.y_bf16)
      ((uint16_t*)g.Y)[off] = f32_to_bf16(v);
    else
      ((float*)g.Y)[off] = v;
  }
  if (tid == 0) g.counters[strip] = 0;
}

}  // namespace

int gemv_splits(int k, int n, int m) {
  const int nr = n <= 4 ? 4 : (n <= 8 ? 8 : 16);
  int s = k / (32 * nr);
  const int strips = (m + kCols - 1) / kCols;
  // keep at least a few hundred workgroups in flight
  while (s < 64 && (long)s * strips < 512 && s * 64 < k) ++s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

hipError_t launch_gemv(const GemvArgs& g, hipStream_t s) {
  dim3 grid((g.m + kCols - 1) / kCols, g.splits);
  if (g.n <= 4)
    gemv_kernel<4><<<grid, 256, 0, s>>>(g);
  else if (g.n <= 8)
    gemv_kernel<8><<<grid, 256, 0, s>>>(g);
  else
    gemv_kernel<16><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace rmm
