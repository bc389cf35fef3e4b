// Row softmax of (scaled) attention logits that also emits the column energies of
// the probabilities it writes, so that the PV product can select key
// positions without reading P a second time.
//
// kaelemshawn.blog, section on where RMM cuts inside the Transformer: for
// PV the contraction axis is the key positions and the importance of key j
// is the L2 norm of column j of P over the query rows; hackcv.com, Core
// Approach: the scores are column L2 norms.  Producing them in the pass
// that already writes P removes the scoring pass over P.
//
// One 256-thread workgroup takes R consecutive query rows of one head: a
// thread owns the key positions j = tid + 256 c, keeps each row in
// registers, reduces the row maximum and the exponential sum over the
// workgroup in a fixed order, writes P, and accumulates P^2 per column.
// The per-workgroup column sums go to partial[h][row block][tk]; a second
// kernel adds the row blocks in order (with a single row block per head the
// sums are written as the energies directly).  Everything is deterministic.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // red is reused row after row
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// fixed-order sum: a butterfly inside each wave, then the 4 waves in order
__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

template <int C>
__global__ __launch_bounds__(kThreads) void softmax_energy_kernel(const float* __restrict__ L, int64_t l_hs,
                                                                  int64_t l_ts, float* __restrict__ P, int64_t p_hs,
                                                                  int64_t p_ts, int tq, int tk, int rows_per_block,
                                                                  float scale, float* __restrict__ partial) {
  __shared__ float red[kThreads / 64];
  const int head = blockIdx.y;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(tq, r0 + rows_per_block);
  const float* Lh = L + (size_t)head * l_hs;
  float* Ph = P + (size_t)head * p_hs;
  float e2[C];
#pragma unroll
  for (int c = 0; c < C; ++c) e2[c] = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float* lr = Lh + (size_t)r * l_ts;
    float x[C];
    float mx = -INFINITY;
    // every load of the row is issued before any is used (a use inside the
    // guarded load would wait for each load in turn); -inf stays -inf
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + kThreads * c;
      x[c] = j < tk ? lr[j] : -INFINITY;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      x[c] *= scale;
      mx = fmaxf(mx, x[c]);
    }
    mx = block_max(mx, red);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + kThreads * c;
      x[c] = j < tk ? expf(x[c] - mx) : 0.f;
      sum += x[c];
    }
    sum = block_sum(sum, red);
    const float inv = 1.f / sum;
    float* pr = Ph + (size_t)r * p_ts;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + kThreads * c;
      if (j < tk) {
        const float p = x[c] * inv;
        pr[j] = p;
        e2[c] = fmaf(p, p, e2[c]);
      }
    }
  }
  float* part = partial + ((size_t)head * gridDim.x + blockIdx.x) * tk;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = threadIdx.x + kThreads * c;
    if (j < tk) part[j] = e2[c];
  }
}

// q[h][j] = sum over row blocks b = 0, 1, ... of partial[h][b][j], in order.
__global__ __launch_bounds__(256) void energy_reduce_kernel(const float* __restrict__ partial, int blocks, int tk,
                                                            float* __restrict__ q) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int head = blockIdx.y;
  if (j >= tk) return;
  const float* ph = partial + (size_t)head * blocks * tk + j;
  float v = 0.f;
  for (int b = 0; b < blocks; ++b) v += ph[(size_t)b * tk];
  q[(size_t)head * tk + j] = v;
}

}  // namespace

int softmax_max_keys() { return 64 * kThreads; }

int softmax_row_blocks(int heads, int tq) {
  // about 2048 workgroups in all, at least 4 rows each
  int rpb = (int)(((long)heads * tq + 2047) / 2048);
  if (rpb < 4) rpb = 4;
  return (tq + rpb - 1) / rpb;
}

hipError_t launch_softmax_energy(const float* L, int64_t l_hs, int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts,
                                 int heads, int tq, int tk, int blocks, float scale, float* partial, float* q,
                                 hipStream_t s) {
  const int rpb = (tq + blocks - 1) / blocks;
  dim3 grid(blocks, heads);
  // one row block per head (decode): its column sums are the energies, laid
  // out [h][1][tk] = [h][tk], so they go straight to q
  if (blocks == 1) partial = q;
  const int C = (tk + kThreads - 1) / kThreads;
  if (C <= 8)
    softmax_energy_kernel<8><<<grid, kThreads, 0, s>>>(L, l_hs, l_ts, P, p_hs, p_ts, tq, tk, rpb, scale, partial);
  else if (C <= 32)
    softmax_energy_kernel<32><<<grid, kThreads, 0, s>>>(L, l_hs, l_ts, P, p_hs, p_ts, tq, tk, rpb, scale, partial);
  else
    softmax_energy_kernel<64><<<grid, kThreads, 0, s>>>(L, l_hs, l_ts, P, p_hs, p_ts, tq, tk, rpb, scale, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || blocks == 1) return e;
  dim3 g2((tk + 255) / 256, heads);
  energy_reduce_kernel<<<g2, 256, 0, s>>>(partial, blocks, tk, q);
  return hipGetLastError();
}

}  // namespace rmm
