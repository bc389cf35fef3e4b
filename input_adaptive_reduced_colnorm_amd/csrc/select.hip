// Selection stage of RMM on gfx950: column energies and TopK.
//
// Scores follow "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach
// (Formula Level): the importance of contraction index j is the L2 norm of
// column j of the activation matrix over all of its rows, and the ceil(rho d)
// largest are kept.  The kernels rank by the fp32 sum of squares, which
// orders the columns exactly as the norm does; equal keys go to the lower
// index and the kept set is emitted in ascending order.  Reductions run in a
// fixed order and the only atomics are integer LDS histogram counts, so the
// result is bitwise reproducible.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeyCap = 15360;  // keys held in LDS (60 KiB); larger d uses global scratch

// ---------------------------------------------------------------------------
// Column energy sweep.  One workgroup covers a 128-byte column strip (64 bf16
// or 32 fp32 columns) over one row split: 8 lanes span the strip with 16-byte
// loads, 32 row lanes stride the rows, then the 32 row sums of each column
// are added in a fixed order.
// ---------------------------------------------------------------------------
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void colnorm_kernel(const void* __restrict__ A_, int64_t hs, int64_t lda,
                                                      int n, int d, int rows_per_split, int splits,
                                                      float* __restrict__ partial) {
  constexpr int VPT = BF16 ? 8 : 4;  // values per 16-byte load
  constexpr int CB = 8 * VPT;        // columns per workgroup
  __shared__ float red[32][CB + 1];

  const int tid = threadIdx.x;
  const int tr = tid >> 3, tc = tid & 7;
  const int head = blockIdx.z;
  const int col0 = blockIdx.x * CB + tc * VPT;
  const int r_begin = blockIdx.y * rows_per_split;
  const int r_end = min(n, r_begin + rows_per_split);

  float acc[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) acc[v] = 0.f;

  if (VEC && col0 + VPT <= d) {
    const char* base = (const char*)A_ + (size_t)head * hs * (BF16 ? 2 : 4) + (size_t)col0 * (BF16 ? 2 : 4);
    const size_t row_bytes = (size_t)lda * (BF16 ? 2 : 4);
    int r = r_begin + tr;
    for (; r + 96 < r_end; r += 128) {
      i32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *(const i32x4*)(base + (size_t)(r + 32 * u) * row_bytes);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t bits = (uint32_t)x[u][w];
          if (BF16) {
            float lo = __uint_as_float(bits << 16), hi = __uint_as_float(bits & 0xffff0000u);
            acc[2 * w] = fmaf(lo, lo, acc[2 * w]);
            acc[2 * w + 1] = fmaf(hi, hi, acc[2 * w + 1]);
          } else {
            float f = __uint_as_float(bits);
            acc[w] = fmaf(f, f, acc[w]);
          }
        }
      }
    }
    for (; r < r_end; r += 32) {
      i32x4 x = *(const i32x4*)(base + (size_t)r * row_bytes);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t bits = (uint32_t)x[w];
        if (BF16) {
          float lo = __uint_as_float(bits << 16), hi = __uint_as_float(bits & 0xffff0000u);
          acc[2 * w] = fmaf(lo, lo, acc[2 * w]);
          acc[2 * w + 1] = fmaf(hi, hi, acc[2 * w + 1]);
        } else {
          float f = __uint_as_float(bits);
          acc[w] = fmaf(f, f, acc[w]);
        }
      }
    }
  } else {
    for (int r = r_begin + tr; r < r_end; r += 32) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        if (col0 + v < d) {
          size_t off = (size_t)head * hs + (size_t)r * lda + col0 + v;
          float f = BF16 ? bf16_to_f32(((const uint16_t*)A_)[off]) : ((const float*)A_)[off];
          acc[v] = fmaf(f, f, acc[v]);
        }
      }
    }
  }

#pragma unroll
  for (int v = 0; v < VPT; ++v) red[tr][tc * VPT + v] = acc[v];
  __syncthreads();
  if (tid < CB) {
    float s = 0.f;
#pragma unroll 8
    for (int t = 0; t < 32; ++t) s += red[t][tid];
    const int col = blockIdx.x * CB + tid;
    if (col < d) partial[((size_t)head * splits + blockIdx.y) * d + col] = s;
  }
}

// ---------------------------------------------------------------------------
// Block-wide helpers for 1024-thread selection workgroups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

struct SelShared {
  uint32_t hist[256];
  uint32_t misc[4];
  uint32_t wave_tot[kSelWaves][2];
};

// Finds the k-th largest key: on return *T is its value and *rem the number
// of keys equal to T that belong to the kept set (the lowest-indexed ones).
// Four MSB-first 8-bit radix passes with integer LDS histograms.
__device__ void radix_threshold(const uint32_t* keys, int d, int k, SelShared& sh, uint32_t* T, uint32_t* rem_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < d; j += kSelThreads) {
      uint32_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns buckets 255-4l .. 252-4l, scanned from the top
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = sh.hist[255 - 4 * tid - i];
        sum += c[i];
      }
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
      if (excl < rem && rem <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + c[i] >= rem) {
            sh.misc[0] = 255u - 4u * tid - i;
            sh.misc[1] = rem - cum;
            break;
          }
          cum += c[i];
        }
      }
    }
    __syncthreads();
    const uint32_t b = sh.misc[0];
    rem = sh.misc[1];
    prefix |= b << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  *T = prefix;
  *rem_out = rem;
}

// Ordered compaction: every thread owns a contiguous index chunk; a block
// scan of (#greater, #equal) fixes each thread's output position, so the kept
// indices come out ascending.  emit(pos, j) is called once per kept index.
template <typename Emit>
__device__ void compact_ascending(const uint32_t* keys, int d, uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int chunk = (d + kSelThreads - 1) / kSelThreads;
  const int j0 = min(d, tid * chunk), j1 = min(d, j0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    uint32_t key = keys[j];
    n_gt += key > T;
    n_eq += key == T;
  }
  const uint32_t i_gt = wave_incl_scan(n_gt), i_eq = wave_incl_scan(n_eq);
  if (lane == 63) {
    sh.wave_tot[wave][0] = i_gt;
    sh.wave_tot[wave][1] = i_eq;
  }
  __syncthreads();
  uint32_t p_gt = i_gt - n_gt, p_eq = i_eq - n_eq;
  for (int w = 0; w < wave; ++w) {
    p_gt += sh.wave_tot[w][0];
    p_eq += sh.wave_tot[w][1];
  }
  uint32_t pos = p_gt + min(p_eq, rem);
  uint32_t eq_seen = p_eq;
  for (int j = j0; j < j1; ++j) {
    uint32_t key = keys[j];
    bool take = key > T;
    if (key == T) {
      take = eq_seen < rem;
      ++eq_seen;
    }
    if (take) emit(pos++, j);
  }
}

template <bool LDS_KEYS>
__global__ __launch_bounds__(kSelThreads) void topk_kernel(const float* __restrict__ partial, int splits, int d, int k,
                                                           int32_t* __restrict__ idx, int64_t idx_hs,
                                                           float* __restrict__ scores, int64_t scores_hs,
                                                           uint32_t* __restrict__ gkeys) {
  __shared__ uint32_t s_keys[LDS_KEYS ? kKeyCap : 1];
  __shared__ SelShared sh;
  const int head = blockIdx.x;
  const float* P = partial + (size_t)head * splits * d;
  uint32_t* keys = LDS_KEYS ? s_keys : gkeys + (size_t)head * d;
  for (int j = threadIdx.x; j < d; j += kSelThreads) {
    float q = 0.f;
    for (int s = 0; s < splits; ++s) q += P[(size_t)s * d + j];
    keys[j] = __float_as_uint(q);
    if (scores) scores[(size_t)head * scores_hs + j] = sqrtf(q);
  }
  if (!LDS_KEYS) __threadfence_block();
  __syncthreads();
  uint32_t T, rem;
  radix_threshold(keys, d, k, sh, &T, &rem);
  int32_t* out = idx + (size_t)head * idx_hs;
  compact_ascending(keys, d, T, rem, sh, [&](uint32_t pos, int j) { out[pos] = j; });
}

__global__ void iota_kernel(int32_t* idx, int64_t idx_hs, int d) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < d) idx[(size_t)blockIdx.y * idx_hs + j] = j;
}

// ---------------------------------------------------------------------------
// Decode selection (n <= 16 rows): one workgroup computes the energies,
// selects, and writes a_t[t][r] = A[r][idx[t]] (fp32, rows padded to 16),
// so the GEMV streams only kept rows of B.
// ---------------------------------------------------------------------------
template <bool BF16, bool LDS_KEYS>
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(const void* __restrict__ A_, int64_t lda, int n, int d,
                                                                    int k, int k_pad, int all, int32_t* __restrict__ idx,
                                                                    float* __restrict__ scores, float* __restrict__ a_t,
                                                                    uint32_t* __restrict__ gkeys,
                                                                    uint32_t* __restrict__ counters, int n_counters) {
  __shared__ uint32_t s_keys[LDS_KEYS ? kKeyCap : 1];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  auto load = [&](int r, int j) -> float {
    size_t off = (size_t)r * lda + j;
    return BF16 ? bf16_to_f32(((const uint16_t*)A_)[off]) : ((const float*)A_)[off];
  };
  for (int i = tid; i < n_counters; i += kSelThreads) counters[i] = 0;
  uint32_t* keys = LDS_KEYS ? s_keys : gkeys;
  const bool need_keys = !all || scores != nullptr;
  if (need_keys) {
    for (int j = tid; j < d; j += kSelThreads) {
      float q = 0.f;
      for (int r = 0; r < n; ++r) {
        float f = load(r, j);
        q = fmaf(f, f, q);
      }
      keys[j] = __float_as_uint(q);
      if (scores) scores[j] = sqrtf(q);
    }
  }
  for (int t = k + tid; t < k_pad; t += kSelThreads) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a_t[(size_t)t * 16 + r] = 0.f;
  }
  if (all) {
    for (int t = tid; t < k; t += kSelThreads) {
      idx[t] = t;
#pragma unroll
      for (int r = 0; r < 16; ++r) a_t[(size_t)t * 16 + r] = r < n ? load(r, t) : 0.f;
    }
    return;
  }
  if (!LDS_KEYS) __threadfence_block();
  __syncthreads();
  uint32_t T, rem;
  radix_threshold(keys, d, k, sh, &T, &rem);
  compact_ascending(keys, d, T, rem, sh, [&](uint32_t pos, int j) {
    idx[pos] = j;
    f32x4* dst = (f32x4*)(a_t + (size_t)pos * 16);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int r = 4 * q4 + e;
        v[e] = r < n ? load(r, j) : 0.f;
      }
      dst[q4] = v;
    }
  });
}

}  // namespace

int colnorm_splits(int heads, int n, int d, bool elt_bf16) {
  const int cb = elt_bf16 ? 64 : 32;
  const long col_blocks = (long)((d + cb - 1) / cb) * heads;
  long s = (1024 + col_blocks - 1) / col_blocks;
  long max_by_rows = (n + 127) / 128;
  if (s > max_by_rows) s = max_by_rows;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_colnorm(const void* A, bool elt_bf16, int64_t head_stride, int64_t lda, int heads, int n, int d,
                          int splits, float* partial, hipStream_t s) {
  const int cb = elt_bf16 ? 64 : 32;
  const int rows_per_split = (n + splits - 1) / splits;
  dim3 grid((d + cb - 1) / cb, splits, heads);
  const size_t elt = elt_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)A % 16 == 0) && ((lda * elt) % 16 == 0) && ((head_stride * elt) % 16 == 0);
  if (elt_bf16) {
    if (vec)
      colnorm_kernel<true, true><<<grid, 256, 0, s>>>(A, head_stride, lda, n, d, rows_per_split, splits, partial);
    else
      colnorm_kernel<true, false><<<grid, 256, 0, s>>>(A, head_stride, lda, n, d, rows_per_split, splits, partial);
  } else {
    if (vec)
      colnorm_kernel<false, true><<<grid, 256, 0, s>>>(A, head_stride, lda, n, d, rows_per_split, splits, partial);
    else
      colnorm_kernel<false, false><<<grid, 256, 0, s>>>(A, head_stride, lda, n, d, rows_per_split, splits, partial);
  }
  return hipGetLastError();
}

int topk_lds_capacity() { return kKeyCap; }

hipError_t launch_topk(const float* partial, int heads, int splits, int d, int k, int32_t* idx, int64_t idx_hs,
                       float* scores, int64_t scores_hs, uint32_t* gkeys, hipStream_t s) {
  if (d <= kKeyCap)
    topk_kernel<true><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, scores, scores_hs, nullptr);
  else
    topk_kernel<false><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, scores, scores_hs, gkeys);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* idx, int64_t idx_hs, int heads, int d, hipStream_t s) {
  dim3 grid((d + 255) / 256, heads);
  iota_kernel<<<grid, 256, 0, s>>>(idx, idx_hs, d);
  return hipGetLastError();
}

hipError_t launch_decode_select(const void* A, bool a_bf16, int64_t lda, int n, int d, int k, int k_pad, bool all,
                                int32_t* idx, float* scores, float* a_t, uint32_t* gkeys, uint32_t* counters,
                                int n_counters, hipStream_t s) {
  const int all_i = all ? 1 : 0;
  if (d <= kKeyCap) {
    if (a_bf16)
      decode_select_kernel<true, true><<<1, kSelThreads, 0, s>>>(A, lda, n, d, k, k_pad, all_i, idx, scores, a_t,
                                                                  nullptr, counters, n_counters);
    else
      decode_select_kernel<false, true><<<1, kSelThreads, 0, s>>>(A, lda, n, d, k, k_pad, all_i, idx, scores, a_t,
                                                                   nullptr, counters, n_counters);
  } else {
    if (a_bf16)
      decode_select_kernel<true, false><<<1, kSelThreads, 0, s>>>(A, lda, n, d, k, k_pad, all_i, idx, scores, a_t,
                                                                   gkeys, counters, n_counters);
    else
      decode_select_kernel<false, false><<<1, kSelThreads, 0, s>>>(A, lda, n, d, k, k_pad, all_i, idx, scores, a_t,
                                                                    gkeys, counters, n_counters);
  }
  return hipGetLastError();
}

}  // namespace rmm
