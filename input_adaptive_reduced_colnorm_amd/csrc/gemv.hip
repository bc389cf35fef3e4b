// Decode-shaped reduced product (n <= 16 rows of A): a bandwidth-bound
// GEMV that streams only the kept rows B[I, :].
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach: the product runs
// over the kept contraction indices only; with a handful of rows in A the
// cost is reading B, so reading ceil(rho d) of its d rows is the saving.
// Engineering Notes on the same page: prefill and decode are tuned apart.
//
// Layout: the kept rows are split into `splits` slices and the columns into
// 64-column strips (128 bytes of every kept row); one 256-thread workgroup
// owns a (slice, strip) pair, so several hundred workgroups keep every CU's
// memory pipeline busy.  8 lanes span a strip with 16-byte loads and 32 row
// lanes stride the slice, each with a batch of 8 kept rows in flight while
// it multiplies the previous batch.  The slice's kept-row list and its
// activations A[:, I] (fp32) are staged in LDS first, straight from A.
// Each workgroup folds its 32 row lanes in a fixed order and writes a
// partial sum per slice; a second kernel adds the slices in slice order, so
// the result is bitwise reproducible and no workgroup waits on another.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;                     // output columns per workgroup
constexpr int kLanesPerRow = kCols / 8;       // 16-byte lanes per row segment
constexpr int kRowLanes = kThreads / kLanesPerRow;
constexpr int kMaxSlice = 512;                // kept rows per workgroup (LDS staged)
constexpr int kBatch = 8;                     // kept rows in flight per lane
constexpr int kTargetGroups = 640;            // workgroups aimed for (256 CUs)

template <int NR, bool A_BF16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs g) {
  __shared__ __attribute__((aligned(16))) float s_a[kMaxSlice][NR];
  __shared__ int32_t s_rows[kMaxSlice];
  __shared__ float red[kThreads / 64][NR][kCols];
  {
    // batch member (attention head): shift every operand to its slice
    const int bz = blockIdx.z;
    g.A = (const char*)g.A + (size_t)bz * g.a_bs * (A_BF16 ? 2 : 4);
    g.B += (size_t)(bz / g.b_group) * g.b_bs;
    if (g.idx) g.idx += (size_t)bz * g.idx_bs;
    g.Y = (char*)g.Y + (size_t)bz * g.y_bs * (g.y_bf16 ? 2 : 4);
    g.partial += (size_t)bz * g.splits * g.n * g.m;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = tid % kLanesPerRow, rl = tid / kLanesPerRow;
  const int slice = (g.k + g.splits - 1) / g.splits;
  const int t0 = blockIdx.y * slice;
  const int L = max(0, min(g.k, t0 + slice) - t0);

  // ---- stage the slice: kept rows and the matching activations.  Each
  //      lane owns up to two kept rows; all their index and activation loads
  //      are issued before any is used ----
  constexpr int PER = kMaxSlice / kThreads;
  int rows[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kThreads;
    rows[u] = i < L ? (g.idx ? g.idx[t0 + i] : t0 + i) : 0;
  }
  float av[PER][NR];
#pragma unroll
  for (int u = 0; u < PER; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      av[u][r] = 0.f;
      if (tid + u * kThreads < L && r < g.n && rows[u] >= 0) {   // -1: contributes nothing
        const size_t off = (size_t)r * g.lda + rows[u];
        av[u][r] = A_BF16 ? bf16_to_f32(((const uint16_t*)g.A)[off]) : ((const float*)g.A)[off];
      }
    }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kThreads;
    if (i < L) {
      s_rows[i] = rows[u];
      if (!g.idx && g.idx_out && blockIdx.x == 0) g.idx_out[t0 + i] = t0 + i;
#pragma unroll
      for (int q = 0; q < NR / 4; ++q)
        *(f32x4*)&s_a[i][4 * q] = f32x4{av[u][4 * q], av[u][4 * q + 1], av[u][4 * q + 2], av[u][4 * q + 3]};
    }
  }
  __syncthreads();

  const int c = blockIdx.x * kCols + cl * 8;
  const bool col_ok = c < g.m;   // m is a multiple of 8
  float acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  auto load_batch = [&](int base, i32x4 (&bv)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int tl = base + kRowLanes * u;
      if (tl < L && col_ok && s_rows[tl] >= 0)
        bv[u] = __builtin_nontemporal_load((const i32x4*)(g.B + (size_t)s_rows[tl] * g.ldb + c));
      else
        bv[u] = i32x4{0, 0, 0, 0};
    }
  };
  auto fma_batch = [&](int base, const i32x4 (&bv)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int tl = base + kRowLanes * u;
      if (tl >= L) break;
      float a[NR];
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        const f32x4 v = *(const f32x4*)&s_a[tl][4 * q];
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
  if (base < L) load_batch(base, b0);
  while (base < L) {
    const int next = base + STEP;
    if (next < L) load_batch(next, b1);
    fma_batch(base, b0);
    if (next >= L) break;
    const int next2 = next + STEP;
    if (next2 < L) load_batch(next2, b0);
    fma_batch(next, b1);
    base = next2;
  }

  // fold the 8 row lanes of each wave (lane bits 3..5), then the 4 waves
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
  const bool direct = g.splits == 1;
  float* part = g.partial + (size_t)blockIdx.y * g.n * g.m;
  for (int i = tid; i < g.n * kCols; i += kThreads) {
    const int r = i / kCols, cc = i % kCols;
    const int col = blockIdx.x * kCols + cc;
    if (col >= g.m) continue;
    float v = red[0][r][cc];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v += red[w][r][cc];
    if (direct) {
      const size_t off = (size_t)r * g.ldy + col;
      if (g.y_bf16)
        ((uint16_t*)g.Y)[off] = f32_to_bf16(v);
      else
        ((float*)g.Y)[off] = v;
    } else {
      part[(size_t)r * g.m + col] = v;
    }
  }
}

// Y[r][c] = sum over slices s = 0, 1, ... of partial[s][r][c], in slice order.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const GemvArgs g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= g.n * g.m) return;
  const int bz = blockIdx.y;
  const int r = i / g.m, col = i % g.m;
  const float* part = g.partial + (size_t)bz * g.splits * g.n * g.m;
  float v = 0.f;
  for (int s = 0; s < g.splits; ++s) v += part[(size_t)s * g.n * g.m + i];
  const size_t off = (size_t)bz * g.y_bs + (size_t)r * g.ldy + col;
  if (g.y_bf16)
    ((uint16_t*)g.Y)[off] = f32_to_bf16(v);
  else
    ((float*)g.Y)[off] = v;
}

template <int NR>
void launch_nr(const GemvArgs& g, dim3 grid, hipStream_t s) {
  if (g.a_bf16)
    gemv_kernel<NR, true><<<grid, kThreads, 0, s>>>(g);
  else
    gemv_kernel<NR, false><<<grid, kThreads, 0, s>>>(g);
}

}  // namespace

int gemv_splits(int k, int m, int batch) {
  const int strips = (m + kCols - 1) / kCols;
  int splits = (kTargetGroups + strips * batch - 1) / (strips * batch);
  const int min_splits = (k + kMaxSlice - 1) / kMaxSlice;
  if (splits < min_splits) splits = min_splits;
  // at least 64 kept rows per slice
  const int max_splits = (k + 63) / 64;
  if (splits > max_splits) splits = max_splits > min_splits ? max_splits : min_splits;
  return splits < 1 ? 1 : splits;
}

hipError_t launch_gemv(const GemvArgs& g, hipStream_t s) {
  dim3 grid((g.m + kCols - 1) / kCols, g.splits, g.batch);
  if (g.n <= 4)
    launch_nr<4>(g, grid, s);
  else if (g.n <= 8)
    launch_nr<8>(g, grid, s);
  else
    launch_nr<16>(g, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.splits == 1) return e;
  gemv_reduce_kernel<<<dim3((g.n * g.m + 255) / 256, g.batch), 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace rmm
