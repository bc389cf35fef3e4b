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
#include "select_block.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Wave reduction in a fixed order on the DPP cross-lane paths (no LDS round
// trip): xor 1 and xor 2 inside each quad, then each lane with its mirror in
// the half-row and in the row, so every lane of a row of 16 holds the row's
// result; the four rows are then combined as (r0 op r1) op (r2 op r3).
template <typename F>
__device__ __forceinline__ float wave_reduce(float v, F op) {
  v = op(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  v = op(v, dpp_move<0x140>(v));   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return op(op(r0, r1), op(r2, r3));
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // red is reused row after row
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// fixed-order sum: wave_reduce inside each wave, then the waves in order
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_reduce(v, [](float a, float b) { return a + b; });
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) t += red[w];
  return t;
}

// Softmax of rows [r0, r1) of one head by NT threads, adding each key's
// P^2 into e2[c] (key tid + NT c).
template <int C, int NT = kThreads>
__device__ __forceinline__ void softmax_rows(const float* __restrict__ Lh, int64_t l_ts, float* __restrict__ Ph,
                                             int64_t p_ts, int r0, int r1, int tk, float scale, float* red,
                                             float (&e2)[C]) {
  for (int r = r0; r < r1; ++r) {
    const float* lr = Lh + (size_t)r * l_ts;
    float x[C];
    float mx = -INFINITY;
    // every load of the row is issued before any is used (a use inside the
    // guarded load would wait for each load in turn); -inf stays -inf
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + NT * c;
      x[c] = j < tk ? lr[j] : -INFINITY;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      x[c] *= scale;
      mx = fmaxf(mx, x[c]);
    }
    mx = block_max<NT>(mx, red);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + NT * c;
      x[c] = j < tk ? expf(x[c] - mx) : 0.f;
      sum += x[c];
    }
    sum = block_sum<NT>(sum, red);
    const float inv = 1.f / sum;
    float* pr = Ph + (size_t)r * p_ts;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = threadIdx.x + NT * c;
      if (j < tk) {
        const float p = x[c] * inv;
        pr[j] = p;
        e2[c] = fmaf(p, p, e2[c]);
      }
    }
  }
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
  float e2[C];
#pragma unroll
  for (int c = 0; c < C; ++c) e2[c] = 0.f;
  softmax_rows<C>(L + (size_t)head * l_hs, l_ts, P + (size_t)head * p_hs, p_ts, r0, r1, tk, scale, red, e2);
  float* part = partial + ((size_t)head * gridDim.x + blockIdx.x) * tk;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = threadIdx.x + kThreads * c;
    if (j < tk) part[j] = e2[c];
  }
}

// Decode: one workgroup holds every query row of its head, so its column
// sums are the head's final energies; it also ranks them (the block TopK of
// select_block.h, the keys passing through LDS into a contiguous chunk per
// thread so that the kept list comes out ascending) and writes the head's
// kept list.  1024 threads, so that the ranking holds at most 8 keys per
// thread (with 32 keys per thread on 256 threads it took longer than the
// separate TopK launch it replaces).  The softmax sums run over 16 waves,
// so P may differ from rmm_softmax_energy's in the last bit.
constexpr int kSelNT = 1024;

template <int C>
__global__ __launch_bounds__(kSelNT) void softmax_select_kernel(const float* __restrict__ L, int64_t l_hs,
                                                                int64_t l_ts, float* __restrict__ P, int64_t p_hs,
                                                                int64_t p_ts, int tq, int tk, float scale,
                                                                float* __restrict__ energy, int k,
                                                                int32_t* __restrict__ idx) {
  __shared__ float red[kSelNT / 64];
  __shared__ uint32_t s_keys[kSelNT * C];
  __shared__ sel::Shared<kSelNT / 64> sh;
  const int head = blockIdx.x;
  float e2[C];
#pragma unroll
  for (int c = 0; c < C; ++c) e2[c] = 0.f;
  softmax_rows<C, kSelNT>(L + (size_t)head * l_hs, l_ts, P + (size_t)head * p_hs, p_ts, 0, tq, tk, scale, red,
                          e2);
  float* eh = energy + (size_t)head * tk;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = threadIdx.x + kSelNT * c;
    if (j < tk) {
      eh[j] = e2[c];
      s_keys[j] = __float_as_uint(e2[c]);   // energies are >= 0: bit order is value order
    }
  }
  lds_barrier();
  sel::KeyChunk<C> kc;
  const int chunk = (tk + kSelNT - 1) / kSelNT;   // <= C
  kc.j0 = min(tk, (int)threadIdx.x * chunk);
  kc.cnt = min(chunk, tk - kc.j0);
#pragma unroll
  for (int i = 0; i < C; ++i) kc.key[i] = i < kc.cnt ? s_keys[kc.j0 + i] : 0u;
  int32_t* out = idx + (size_t)head * k;
  sel::select_ascending<kSelNT, C>(kc, k, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
    if (take) out[pos] = j;
  });
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

int softmax_select_max_keys() { return 8 * kSelNT; }

hipError_t launch_softmax_select(const float* L, int64_t l_hs, int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts,
                                 int heads, int tq, int tk, float scale, float* energy, int k, int32_t* idx,
                                 hipStream_t s) {
  if (tk > softmax_select_max_keys() || k < 1 || k > tk) return hipErrorInvalidValue;
  if (tk <= 4 * kSelNT)
    softmax_select_kernel<4><<<heads, kSelNT, 0, s>>>(L, l_hs, l_ts, P, p_hs, p_ts, tq, tk, scale, energy, k, idx);
  else
    softmax_select_kernel<8><<<heads, kSelNT, 0, s>>>(L, l_hs, l_ts, P, p_hs, p_ts, tq, tk, scale, energy, k, idx);
  return hipGetLastError();
}

}  // namespace rmm
