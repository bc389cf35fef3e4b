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

#include <type_traits>

#include "rmm_device.h"
#include "rmm_internal.h"
#include "select_block.h"

namespace rmm {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeyCap = 15360;  // keys held in LDS (60 KiB); larger d uses global scratch

// ---------------------------------------------------------------------------
// Column energy sweep.  One workgroup covers a 256-byte column strip (128
// bf16 or 64 fp32 columns) over one row split: 16 lanes span the strip with
// 16-byte loads, 16 row lanes stride the rows with 8 rows in flight each,
// then the 16 row sums of each column are added in a fixed order.  (Strips
// of 128 bytes streamed about 4.6 TB/s here, 256-byte strips about 5.2.)
// ---------------------------------------------------------------------------
constexpr int kCnLanes = 16;               // lanes across a strip
constexpr int kCnRowLanes = 256 / kCnLanes;
constexpr int kCnInFlight = 8;             // rows loaded per lane before use

template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void colnorm_kernel(const void* __restrict__ A_, int64_t hs, int64_t lda,
                                                      int n, int d, int rows_per_split, int splits,
                                                      float* __restrict__ partial) {
  constexpr int VPT = BF16 ? 8 : 4;  // values per 16-byte load
  constexpr int CB = kCnLanes * VPT; // columns per workgroup
  constexpr int RL = kCnRowLanes, U = kCnInFlight;
  __shared__ float red[RL][CB + 1];

  const int tid = threadIdx.x;
  const int tr = tid / kCnLanes, tc = tid % kCnLanes;
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
    for (int r = r_begin + tr; r < r_end; r += RL * U) {
      i32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = r + RL * u < r_end ? *(const i32x4*)(base + (size_t)(r + RL * u) * row_bytes) : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t bits = (uint32_t)x[u][w];
          if (BF16) {
            const float lo = __uint_as_float(bits << 16), hi = __uint_as_float(bits & 0xffff0000u);
            acc[2 * w] = fmaf(lo, lo, acc[2 * w]);
            acc[2 * w + 1] = fmaf(hi, hi, acc[2 * w + 1]);
          } else {
            const float f = __uint_as_float(bits);
            acc[w] = fmaf(f, f, acc[w]);
          }
        }
      }
    }
  } else {
    for (int r = r_begin + tr; r < r_end; r += RL) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        if (col0 + v < d) {
          const size_t off = (size_t)head * hs + (size_t)r * lda + col0 + v;
          const float f = BF16 ? bf16_to_f32(((const uint16_t*)A_)[off]) : ((const float*)A_)[off];
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
#pragma unroll
    for (int t = 0; t < RL; ++t) s += red[t][tid];
    const int col = blockIdx.x * CB + tid;
    if (col < d) partial[((size_t)head * splits + blockIdx.y) * d + col] = s;
  }
}

// ---------------------------------------------------------------------------
// Selection workgroups of 1024 threads (the block helpers: select_block.h).
// ---------------------------------------------------------------------------
using sel::hist_add;
using sel::kHistBins;
using sel::KeyChunk;
using SelShared = sel::Shared<kSelWaves>;

// most keys per thread held in registers (a multiple of 4, so that a
// thread's chunk is whole 16-byte groups of split partials)
constexpr int kChunk = ((kKeyCap + kSelThreads - 1) / kSelThreads + 3) / 4 * 4;

// Keys per thread for a key count d held in LDS: the radix passes run one
// unrolled histogram step per register slot, so the slot count follows d.
__host__ __device__ constexpr int chunk_for(int d) { return d <= 4096 ? 4 : (d <= 8192 ? 8 : kChunk); }

// Retained fraction of the energy: sum of the kept keys over the sum of all
// keys (each thread's keys in index order, then a butterfly inside each
// wave, then the waves in order; fp64 sums of the fp32 keys).
__device__ void write_retained(double kept, double total, SelShared& sh, float* out) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kept += __shfl_xor(kept, o, 64);
    total += __shfl_xor(total, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sh.energy[wave][0] = kept;
    sh.energy[wave][1] = total;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double k = 0.0, t = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      k += sh.energy[w][0];
      t += sh.energy[w][1];
    }
    *out = t > 0.0 ? (float)(k / t) : 1.0f;
  }
}

__device__ __forceinline__ void block_incl_scan2(uint32_t& a, uint32_t& b, SelShared& sh) {
  sel::block_incl_scan2<kSelThreads>(a, b, sh);
}

template <int CH>
__device__ __forceinline__ void load_chunk(const uint32_t* keys, int d, KeyChunk<CH>& kc) {
  const int chunk = (d + kSelThreads - 1) / kSelThreads;   // <= CH
  kc.j0 = min(d, (int)threadIdx.x * chunk);
  kc.cnt = min(chunk, d - kc.j0);
#pragma unroll
  for (int i = 0; i < CH; ++i) kc.key[i] = i < kc.cnt ? keys[kc.j0 + i] : 0u;
}

template <int CH>
__device__ __forceinline__ void radix_threshold(const KeyChunk<CH>& kc, int k, SelShared& sh, uint32_t* T,
                                                uint32_t* rem_out) {
  sel::radix_threshold<kSelThreads, CH>(kc, k, sh, T, rem_out);
}

template <int CH, typename Emit>
__device__ __forceinline__ void compact_ascending(const KeyChunk<CH>& kc, uint32_t T, uint32_t rem, SelShared& sh,
                                                  Emit emit) {
  sel::compact_ascending<kSelThreads, CH>(kc, T, rem, sh, emit);
}

// Same selection for key arrays too large for the register chunks (d above
// the LDS key capacity): keys stay in global scratch and are re-read.
__device__ __forceinline__ void radix_threshold_big(const uint32_t* keys, int d, int k, SelShared& sh, uint32_t* T, uint32_t* rem_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)k;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t nb = pass == 2 ? 1024u : 2048u;
    for (int i = tid; i < (int)nb; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < d; j0 += kSelThreads) {
      const int j = j0 + tid;
      const uint32_t key = j < d ? keys[j] : 0u;
      hist_add(sh.hist, j < d && (key & mask) == prefix, (key >> shift) & (nb - 1));
    }
    __syncthreads();
    uint32_t c0, c1 = 0;
    int b0, b1 = -1;
    if (nb == 2048u) {
      b0 = (int)nb - 1 - 2 * tid;
      b1 = b0 - 1;
      c0 = sh.hist[b0];
      c1 = sh.hist[b1];
    } else {
      b0 = (int)nb - 1 - tid;
      c0 = sh.hist[b0];
    }
    uint32_t incl = c0 + c1, dummy = 0;
    block_incl_scan2(incl, dummy, sh);
    const uint32_t excl = incl - (c0 + c1);
    if (excl < rem && rem <= incl) {
      if (excl + c0 >= rem) {
        sh.misc[0] = (uint32_t)b0;
        sh.misc[1] = rem - excl;
      } else {
        sh.misc[0] = (uint32_t)b1;
        sh.misc[1] = rem - excl - c0;
      }
    }
    __syncthreads();
    const uint32_t b = sh.misc[0];
    rem = sh.misc[1];
    prefix |= b << shift;
    mask |= (nb - 1) << shift;
    __syncthreads();
  }
  *T = prefix;
  *rem_out = rem;
}

template <typename Emit>
__device__ __forceinline__ void compact_ascending_big(const uint32_t* keys, int d, uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  const int chunk = (d + kSelThreads - 1) / kSelThreads;
  const int j0 = min(d, (int)threadIdx.x * chunk), j1 = min(d, j0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    n_gt += key > T;
    n_eq += key == T;
  }
  uint32_t i_gt = n_gt, i_eq = n_eq;
  block_incl_scan2(i_gt, i_eq, sh);
  uint32_t pos = (i_gt - n_gt) + min(i_eq - n_eq, rem);
  uint32_t eq_seen = i_eq - n_eq;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    bool take = key > T;
    if (key == T) {
      take = eq_seen < rem;
      ++eq_seen;
    }
    emit(take, pos, j, key);
    pos += take;
  }
}

// The keys of one thread's contiguous chunk of columns, summed over the
// split partials in split order straight into registers: the chunk is a
// whole number of 16-byte groups when d % 4 == 0 (c = ceil(d / 1024)
// rounded up to 4, at most CH), else single columns (c = ceil(d / 1024)).
// Two splits' loads are issued before either is added.
template <int CH>
__device__ __forceinline__ void sum_chunk(const float* P, int splits, int d, KeyChunk<CH>& kc, float* scores) {
  const bool vec = d % 4 == 0;
  int c = (d + kSelThreads - 1) / kSelThreads;
  if (vec) c = (c + 3) / 4 * 4;
  kc.j0 = min(d, (int)threadIdx.x * c);
  kc.cnt = min(c, d - kc.j0);
  float q[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) q[i] = 0.f;
  if (vec) {
    constexpr int V = CH / 4;
    for (int s0 = 0; s0 < splits; s0 += 2) {
      f32x4 v[2][V];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < V; ++u)
          v[t][u] = (s0 + t < splits && 4 * u < kc.cnt)
                        ? *(const f32x4*)(P + (size_t)(s0 + t) * d + kc.j0 + 4 * u)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (s0 + t < splits)
#pragma unroll
          for (int u = 0; u < V; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) q[4 * u + e] += v[t][u][e];
    }
  } else {
    for (int s0 = 0; s0 < splits; ++s0) {
      float v[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) v[i] = i < kc.cnt ? P[(size_t)s0 * d + kc.j0 + i] : 0.f;
#pragma unroll
      for (int i = 0; i < CH; ++i) q[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    kc.key[i] = i < kc.cnt ? __float_as_uint(q[i]) : 0u;
    if (scores && i < kc.cnt) scores[kc.j0 + i] = sqrtf(q[i]);
  }
}

// CH: keys per thread in registers (chunk_for(d)), or 0 for keys in global
// scratch (d above the LDS key capacity).
template <int CH>
__global__ __launch_bounds__(kSelThreads) void topk_kernel(const float* __restrict__ partial, int splits, int d, int k,
                                                           int32_t* __restrict__ idx, int64_t idx_hs,
                                                           int32_t* __restrict__ pad, int64_t pad_hs, int k_pad,
                                                           float* __restrict__ scores, int64_t scores_hs,
                                                           int32_t* __restrict__ mask, int64_t mask_hs,
                                                           float* __restrict__ retained,
                                                           uint32_t* __restrict__ gkeys) {
  constexpr bool LDS_KEYS = CH > 0;
  __shared__ uint32_t s_keys[LDS_KEYS ? kKeyCap : 1];
  __shared__ __attribute__((aligned(16))) int32_t s_out[LDS_KEYS ? kKeyCap : 1];
  __shared__ SelShared sh;
  const int head = blockIdx.x;
  const float* P = partial + (size_t)head * splits * d;
  uint32_t* keys = LDS_KEYS ? s_keys : gkeys + (size_t)head * d;
  KeyChunk<LDS_KEYS ? CH : 1> kc;
  if constexpr (LDS_KEYS) {
    sum_chunk(P, splits, d, kc, scores ? scores + (size_t)head * scores_hs : nullptr);
  } else {
    for (int j = threadIdx.x; j < d; j += kSelThreads) {
      float q = 0.f;
      for (int s = 0; s < splits; ++s) q += P[(size_t)s * d + j];
      keys[j] = __float_as_uint(q);
      if (scores) scores[(size_t)head * scores_hs + j] = sqrtf(q);
    }
    __threadfence_block();
    __syncthreads();
  }
  int32_t* out = idx + (size_t)head * idx_hs;
  int32_t* po = pad ? pad + (size_t)head * pad_hs : nullptr;
  if (po)
    for (int t = k + threadIdx.x; t < k_pad; t += kSelThreads) po[t] = -1;
  int32_t* mo = mask ? mask + (size_t)head * mask_hs : nullptr;
  double e_kept = 0.0, e_all = 0.0;
  auto emit = [&](bool take, uint32_t pos, int j, uint32_t key) {
    if (take) {
      out[pos] = j;
      if (po) po[pos] = j;
    }
    if (mo) mo[j] = take ? j : -1;
    const double q = (double)__uint_as_float(key);
    e_all += q;
    e_kept += take ? q : 0.0;   // no branch: both sums stay in registers
  };
  uint32_t T, rem;
  if constexpr (LDS_KEYS) {
    // the keys live in registers; the kept list is assembled in LDS and
    // written out coalesced, and s_keys takes the keep flags
    if (retained || mo) {
      sel::select_ascending<kSelThreads, CH>(kc, k, sh, [&](bool take, uint32_t pos, int j, uint32_t key) {
        if (take) s_out[pos] = j;
        s_keys[j] = take;
        const double q = (double)__uint_as_float(key);
        e_all += q;
        e_kept += take ? q : 0.0;
      });
    } else {
      sel::select_ascending<kSelThreads, CH>(kc, k, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
        if (take) s_out[pos] = j;
      });
    }
    __syncthreads();
    int t_done = 0;
    if ((((uintptr_t)out | (uintptr_t)(po ? po : out)) & 15) == 0) {
      // 16-byte pieces of the list, then the tail
      const int k4 = k / 4;
      for (int t4 = threadIdx.x; t4 < k4; t4 += kSelThreads) {
        const i32x4 v = *(const i32x4*)(s_out + 4 * t4);
        *(i32x4*)(out + 4 * t4) = v;
        if (po) *(i32x4*)(po + 4 * t4) = v;
      }
      t_done = 4 * k4;
    }
    for (int t = t_done + threadIdx.x; t < k; t += kSelThreads) {
      const int j = s_out[t];
      out[t] = j;
      if (po) po[t] = j;
    }
    if (mo)
      for (int j = threadIdx.x; j < d; j += kSelThreads) mo[j] = s_keys[j] ? j : -1;
  } else {
    radix_threshold_big(keys, d, k, sh, &T, &rem);
    compact_ascending_big(keys, d, T, rem, sh, emit);
  }
  if (retained) write_retained(e_kept, e_all, sh, retained + head);
}

// Small selections (d <= 256, e.g. the head features of attention): one
// 256-thread workgroup per head; thread j ranks its key against all d keys
// (higher key first, lower index first among equal keys), keeps it when the
// rank is below k, and writes it at the count of kept columns before it.
constexpr int kSmallD = 256;

__global__ __launch_bounds__(kSmallD) void topk_small_kernel(const float* __restrict__ partial, int splits, int d,
                                                             int k, int32_t* __restrict__ idx, int64_t idx_hs,
                                                             int32_t* __restrict__ pad, int64_t pad_hs, int k_pad,
                                                             float* __restrict__ scores, int64_t scores_hs,
                                                             int32_t* __restrict__ mask, int64_t mask_hs,
                                                             float* __restrict__ retained) {
  __shared__ __attribute__((aligned(16))) uint64_t s_ck[kSmallD];
  __shared__ int s_wave[kSmallD / 64];
  __shared__ double s_energy[kSmallD / 64][2];
  const int head = blockIdx.x;
  const int j = threadIdx.x;
  const float* P = partial + (size_t)head * splits * d;
  float q = 0.f;
  if (j < d) {
    // the loads of up to 16 splits (the scoring pass makes at most 16) are
    // issued together, then added in split order (the order topk_kernel uses)
    for (int s0 = 0; s0 < splits; s0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = s0 + u < splits ? P[(size_t)(s0 + u) * d + j] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < splits) q += v[u];
    }
    if (scores) scores[(size_t)head * scores_hs + j] = sqrtf(q);
  }
  // composite key (energy bits, 0xFFFF - j): a larger composite outranks
  // (higher energy, or equal energy and lower index), so one 64-bit compare
  // per pair ranks it; two composites per 16-byte LDS read
  const uint64_t ck = ((uint64_t)__float_as_uint(q) << 32) | (uint32_t)(0xFFFF - j);
  s_ck[j] = ck;
  __syncthreads();
  int rank = 0;
#pragma unroll 8
  for (int i2 = 0; i2 < (d + 1) / 2; ++i2) {
    const u64x2 v = *(const u64x2*)(s_ck + 2 * i2);
    rank += (int)(v[0] > ck) + ((int)(2 * i2 + 1 < d) & (int)(v[1] > ck));
  }
  const bool keep = j < d && rank < k;
  const uint64_t ballot = __ballot(keep);
  const int lane = j & 63, wave = j >> 6;
  const int before = __popcll(ballot & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(ballot);
  __syncthreads();
  int pos = before;
  for (int w = 0; w < wave; ++w) pos += s_wave[w];
  int32_t* out = idx + (size_t)head * idx_hs;
  int32_t* po = pad ? pad + (size_t)head * pad_hs : nullptr;
  if (keep) {
    out[pos] = j;
    if (po) po[pos] = j;
  }
  if (mask && j < d) mask[(size_t)head * mask_hs + j] = keep ? j : -1;
  if (po)
    for (int t = k + j; t < k_pad; t += kSmallD) po[t] = -1;
  if (retained) {
    // kept and total energy: butterfly inside each wave, then the waves in order
    double kept = keep ? (double)q : 0.0, total = j < d ? (double)q : 0.0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kept += __shfl_xor(kept, o, 64);
      total += __shfl_xor(total, o, 64);
    }
    if (lane == 0) {
      s_energy[wave][0] = kept;
      s_energy[wave][1] = total;
    }
    __syncthreads();
    if (j == 0) {
      double k2 = 0.0, t2 = 0.0;
      for (int w = 0; w < kSmallD / 64; ++w) {
        k2 += s_energy[w][0];
        t2 += s_energy[w][1];
      }
      retained[head] = t2 > 0.0 ? (float)(k2 / t2) : 1.0f;
    }
  }
}

// Caller-supplied index list -> the padded form the loaders read: entries
// outside [0, d) and the tail past k become -1 (a column / row that
// contributes nothing).
__global__ void pad_index_kernel(const int32_t* __restrict__ idx, int64_t idx_hs, int k, int d,
                                 int32_t* __restrict__ pad, int64_t pad_hs, int k_pad) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= k_pad) return;
  const int b = blockIdx.y;
  int v = -1;
  if (t < k) {
    const int j = idx[(size_t)b * idx_hs + t];
    v = (j >= 0 && j < d) ? j : -1;
  }
  pad[(size_t)b * pad_hs + t] = v;
}

__global__ void iota_kernel(int32_t* idx, int64_t idx_hs, int d, int32_t* pad, int64_t pad_hs, int k_pad) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < d) idx[(size_t)blockIdx.y * idx_hs + j] = j;
  if (pad && j < k_pad) pad[(size_t)blockIdx.y * pad_hs + j] = j < d ? j : -1;
}

// ---------------------------------------------------------------------------
// Decode selection (n <= 16 rows): one workgroup computes the energies over
// the n rows and selects into idx; the GEMV then reads A[:, I] itself.
// ---------------------------------------------------------------------------
template <bool BF16, int CH>
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(const void* __restrict__ A_, int64_t lda, int n,
                                                                    int d, int k, int32_t* __restrict__ idx,
                                                                    float* __restrict__ scores,
                                                                    uint32_t* __restrict__ gkeys) {
  constexpr bool LDS_KEYS = CH > 0;
  __shared__ uint32_t s_keys[LDS_KEYS ? kKeyCap : 1];
  __shared__ int32_t s_out[LDS_KEYS ? kKeyCap : 1];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  uint32_t* keys = LDS_KEYS ? s_keys : gkeys;
  constexpr int VPT = BF16 ? 8 : 4;   // columns per 16-byte load
  const bool vec = ((uintptr_t)A_ % 16 == 0) && (lda % VPT == 0) && (d % VPT == 0);
  if (vec) {
    // a thread takes VPT adjacent columns and issues the 16-byte loads of
    // all n rows before summing them (rows in ascending order)
    for (int c = tid; c < d / VPT; c += kSelThreads) {
      i32x4 x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        x[r] = r < n ? *(const i32x4*)((const char*)A_ + ((size_t)r * lda + (size_t)c * VPT) * (BF16 ? 2 : 4))
                     : i32x4{0, 0, 0, 0};
      float q[VPT];
#pragma unroll
      for (int e = 0; e < VPT; ++e) q[e] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < n) {
#pragma unroll
          for (int e = 0; e < VPT; ++e) {
            const uint32_t w = (uint32_t)x[r][BF16 ? e >> 1 : e];
            const float f = BF16 ? __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)) : __uint_as_float(w);
            q[e] = fmaf(f, f, q[e]);
          }
        }
#pragma unroll
      for (int e = 0; e < VPT; ++e) {
        keys[c * VPT + e] = __float_as_uint(q[e]);
        if (scores) scores[c * VPT + e] = sqrtf(q[e]);
      }
    }
  } else {
    // all 16 row loads of a column are issued before they are summed (rows
    // in ascending order)
    auto load = [&](int r, int j) -> float {
      const size_t off = (size_t)r * lda + j;
      return BF16 ? bf16_to_f32(((const uint16_t*)A_)[off]) : ((const float*)A_)[off];
    };
#pragma unroll 2
    for (int j = tid; j < d; j += kSelThreads) {
      float f[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) f[r] = r < n ? load(r, j) : 0.f;
      float q = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < n) q = fmaf(f[r], f[r], q);
      keys[j] = __float_as_uint(q);
      if (scores) scores[j] = sqrtf(q);
    }
  }
  if (!LDS_KEYS) __threadfence_block();
  __syncthreads();
  uint32_t T, rem;
  if constexpr (LDS_KEYS) {
    KeyChunk<CH> kc;
    load_chunk(keys, d, kc);
    sel::select_ascending<kSelThreads, CH>(kc, k, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
      if (take) s_out[pos] = j;
    });
    __syncthreads();
    for (int t = tid; t < k; t += kSelThreads) idx[t] = s_out[t];
  } else {
    radix_threshold_big(keys, d, k, sh, &T, &rem);
    compact_ascending_big(keys, d, T, rem, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
      if (take) idx[pos] = j;
    });
  }
}

// ---------------------------------------------------------------------------
// Selection fused with the gather of the kept columns (the prefill products).
// One 1024-thread workgroup per compute unit: each sums the split partials
// and ranks the keys as topk_kernel does, so that every workgroup holds the
// same ascending kept list, as 16-bit column indices in LDS padded to k_pad
// with the index z of a zero slot.  It then streams its rows of A, every
// G-th row from its own index (G workgroups), so that each workgroup's rows
// were swept by the column-energy pass at all stages of that pass (the rows
// it read first are the likeliest to have left the Infinity Cache, and a
// contiguous block of them made a few workgroups 1.5-2x slower than the
// rest, since they all have the same number of rows): each row goes whole from HBM into an LDS row buffer by direct 16-byte
// loads (D rows in flight, the first D issued before the ranking so that
// they land while it runs), and each lane gathers 8 consecutive kept
// positions from LDS and writes them as one 16-byte piece of the
// K-contiguous panel.  Whole-row loads avoid the address rate of 2-byte
// global gathers, and the ranking repeated per workgroup (several
// microseconds, while the first rows stream in) replaces a single-workgroup
// launch that the whole chip waited for.  Needs d <= kKeyCap, d % 8 == 0, lda % 8 == 0 and A 16-byte
// aligned (select_pack_fits).
//
// Row buffers: NB = D + 1, row i in buffer i % NB, so the buffer refilled
// for row i + D held row i - 1, which every thread finished reading before
// the barrier of row i.  The ranking's scratch lies in buffer D (and past
// it), which first receives a row after the ranking.  Rows past the last
// one are loaded through an empty buffer resource (no memory access, zeros),
// so every wave issues the same loads per row and the waits count them.
// ---------------------------------------------------------------------------
constexpr int kSpGroups = 256;   // workgroups: one per compute unit

__host__ __device__ constexpr int sp_row_cap(int pr) { return (pr == 1 ? 8192 : kKeyCap) + 8; }

// CH: keys per thread; PR: 16-byte pieces of a row per thread (rows and
// kept lists of up to PR * 8192 entries); D: rows in flight.  RANK = false
// gathers by a caller's list instead (`given`, k entries in any order,
// entries outside [0, d) read as zeros; k_pad may exceed d): no ranking, no
// idx output, and pad[t] is the entry or -1.
template <int CH, int PR, int D, bool RANK>
__global__ __launch_bounds__(kSelThreads) void select_pack_kernel(const float* __restrict__ partial, int splits,
                                                                  const int32_t* __restrict__ given,
                                                                  const uint16_t* __restrict__ A, int64_t lda, int n,
                                                                  int d, int k, int k_pad,
                                                                  int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ pad,
                                                                  uint16_t* __restrict__ out) {
  constexpr int NB = D + 1;
  constexpr int RC = sp_row_cap(PR);   // elements per row buffer (16-byte multiple)
  constexpr int LC = RC - 8;           // kept list capacity
  constexpr size_t kRowsBytes = (size_t)NB * RC * 2;
  constexpr size_t kSelEnd = (size_t)D * RC * 2 + sizeof(SelShared);
  constexpr size_t kStage = kRowsBytes > kSelEnd ? kRowsBytes : kSelEnd;
  static_assert(RC % 8 == 0, "row buffers must stay 16-byte aligned");
  __shared__ __attribute__((aligned(16))) uint16_t s_stage[kStage / 2];
  __shared__ __attribute__((aligned(16))) uint16_t s_list[LC];
  SelShared& sh = *reinterpret_cast<SelShared*>(s_stage + (size_t)D * RC);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, w0 = blockIdx.x;
  const int nr = (n - w0 + G - 1) / G;          // rows w0, w0 + G, ... below n (at least one)
  const int pieces = d >> 3;                    // 16-byte pieces of a row
  const int z = (pieces + 63) / 64 * 512;       // zero slot: past every wave's load span
  // this wave's loads per row: load p covers pieces [1024 p + 64 wave, + 64)
  int nload = 0;
#pragma unroll
  for (int p = 0; p < PR; ++p) nload += 1024 * p + 64 * wave < pieces;

  const uint32_t stage0 = lds_addr(s_stage);
  auto fetch = [&](int i) {
    const i32x4 r = rsrc_words(A + ((size_t)w0 + (size_t)min(i, nr - 1) * G) * lda, i < nr ? (uint32_t)d * 2u : 0u);
    const uint32_t row = stage0 + (uint32_t)((i % NB) * RC * 2);
#pragma unroll
    for (int p = 0; p < PR; ++p)
      if (1024 * p + 64 * wave < pieces)
        load_lds16_async(r, row + 16u * (uint32_t)(1024 * p + 64 * wave), 16u * (uint32_t)(1024 * p + tid));
  };

  if constexpr (RANK) {
    KeyChunk<CH> kc;
    sum_chunk(partial, splits, d, kc, nullptr);
#pragma unroll
    for (int i = 0; i < D; ++i) fetch(i);
    sel::select_ascending<kSelThreads, CH>(kc, k, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
      if (take) s_list[pos] = (uint16_t)j;
    });
    for (int t = k + tid; t < k_pad; t += kSelThreads) s_list[t] = (uint16_t)z;
  } else {
    // the list first: a wait the compiler places for these loads after the
    // untracked row loads would also wait for the rows
    for (int t = tid; t < k_pad; t += kSelThreads) {
      const int j = t < k ? given[t] : -1;
      s_list[t] = (uint16_t)((unsigned)j < (unsigned)d ? j : z);
    }
#pragma unroll
    for (int i = 0; i < D; ++i) fetch(i);
  }
  lds_barrier();

  // the kept list and its copy padded with -1, spread over the workgroups
  for (int t = blockIdx.x * kSelThreads + tid; t < k_pad; t += gridDim.x * kSelThreads) {
    const int j = s_list[t];
    if constexpr (RANK) {
      if (t < k) idx[t] = j;
      pad[t] = t < k ? j : -1;
    } else {
      pad[t] = j == z ? -1 : j;
    }
  }
  if (tid < 8 * NB) s_stage[(size_t)(tid >> 3) * RC + z + (tid & 7)] = 0;
  // this thread's output pieces g = tid + 1024 p: kept positions [8g, 8g + 8)
  uint32_t cw[PR][4];
#pragma unroll
  for (int p = 0; p < PR; ++p) {
    const int g = tid + p * kSelThreads;
    const i32x4 v = 8 * g < k_pad ? *(const i32x4*)(s_list + 8 * g) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) cw[p][e] = (uint32_t)v[e];
  }

  for (int i = 0; i < nr; ++i) {
    // row i's loads are followed by those of rows i + 1 .. i + D - 1
    if (nload == PR)
      wait_vmcnt<(D - 1) * PR>();
    else if (PR == 2 && nload == 1)
      wait_vmcnt<D - 1>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    fetch(i + D);
    const uint16_t* buf = s_stage + (size_t)(i % NB) * RC;
#pragma unroll
    for (int p = 0; p < PR; ++p) {
      const int g = tid + p * kSelThreads;
      if (8 * g < k_pad) {
        i32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (int)((uint32_t)buf[cw[p][e] & 0xffffu] | ((uint32_t)buf[cw[p][e] >> 16] << 16));
        *(i32x4*)(out + ((size_t)w0 + (size_t)i * G) * k_pad + 8 * g) = w;
      }
    }
  }
  // no direct load may still be writing LDS when the workgroup ends
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Per-head feature selection fused with the gather of Q and K (QK^T with
// heads of at most 256 features, rows of whole 16-byte pieces).  A
// workgroup of 256 threads owns 32 KB of rows (16384 / dh rows) of one
// query head's Q, or of its kv head's K: it sums the head's split partials,
// sends its rows from the buffer straight into LDS (untracked direct loads,
// issued before the ranking so that they land while it runs), ranks the
// features as topk_small_kernel does (each thread counts the composite keys
// that outrank its own), and writes the kept features of each row as
// 16-byte pieces of the K-contiguous panels.  The first Q workgroup of each head
// writes its ascending kept list.  Four workgroups share a compute unit
// (35 KB of LDS each), so one's ranking overlaps another's loads.
// ---------------------------------------------------------------------------
constexpr int kQkElems = 16384;   // row elements per workgroup (32 KB of bf16)

__global__ __launch_bounds__(kSmallD) void qk_select_pack_kernel(
    const float* __restrict__ partial, int splits, const uint16_t* __restrict__ Q, int64_t q_hs, int64_t q_ts,
    const uint16_t* __restrict__ K, int64_t k_hs, int64_t k_ts, int group, int tq, int tk, int dh, int k, int k_pad,
    int32_t* __restrict__ idx, uint16_t* __restrict__ qp, uint16_t* __restrict__ kp) {
  __shared__ __attribute__((aligned(16))) uint16_t s_rows[kQkElems];   // row r at r * dh
  __shared__ __attribute__((aligned(16))) uint16_t s_list[kSmallD];
  __shared__ __attribute__((aligned(16))) uint64_t s_ck[kSmallD];
  __shared__ int s_wave[kSmallD / 64];
  const int h = blockIdx.y;
  const int j = threadIdx.x;
  const int lane = j & 63;
  const int wave = __builtin_amdgcn_readfirstlane(j >> 6);
  const int rb_rows = kQkElems / dh;   // rows per workgroup
  const int qblocks = (tq + rb_rows - 1) / rb_rows;
  const bool is_q = (int)blockIdx.x < qblocks;
  const int r0 = (is_q ? (int)blockIdx.x : (int)blockIdx.x - qblocks) * rb_rows;
  const int nr = min(rb_rows, (is_q ? tq : tk) - r0);
  const int64_t ts = is_q ? q_ts : k_ts;
  const uint16_t* src = (is_q ? Q + (size_t)h * q_hs : K + (size_t)(h / group) * k_hs) + (size_t)r0 * ts;
  const int pieces = dh >> 3;   // 16-byte pieces of a row

  // the head's energies, summed over the splits in split order
  float q = 0.f;
  if (j < dh) {
    const float* P = partial + (size_t)h * splits * dh;
    for (int s0 = 0; s0 < splits; s0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = s0 + u < splits ? P[(size_t)(s0 + u) * dh + j] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < splits) q += v[u];
    }
  }

  // the block's rows: piece i = row * pieces + c lands at LDS byte 16 i;
  // wave w sends pieces [64 (w + 4 t), + 64) for t = 0, 1, ...
  const int npieces = nr * pieces;
  const i32x4 rs = rsrc_words(src, (uint32_t)(((size_t)(nr - 1) * ts + dh) * 2));
  const uint32_t rows0 = lds_addr(s_rows);
  for (int base = 64 * wave; base < npieces; base += 256) {
    const int i = base + lane;
    const int row = i / pieces, c = i - row * pieces;
    const uint32_t off = i < npieces ? (uint32_t)(((size_t)row * ts + 8 * c) * 2) : kOobOffset;
    load_lds16_async(rs, rows0 + 16u * (uint32_t)base, off);
  }

  // rank: composite key (energy bits, 0xFFFF - j), a larger one outranks
  const uint64_t ck = ((uint64_t)__float_as_uint(q) << 32) | (uint32_t)(0xFFFF - j);
  s_ck[j] = ck;
  lds_barrier();
  // dh is a multiple of 8 here (whole 16-byte pieces), so the pairs cover
  // exactly the dh keys and the count needs no bound test (a uniform test
  // in the loop would put a scalar step between every compare and its add)
  int rank = 0;
#pragma unroll 8
  for (int i2 = 0; i2 < dh / 2; ++i2) {
    const u64x2 v = *(const u64x2*)(s_ck + 2 * i2);
    rank += (int)(v[0] > ck) + (int)(v[1] > ck);
  }
  const bool keep = j < dh && rank < k;
  const uint64_t ballot = __ballot(keep);
  if (lane == 0) s_wave[wave] = __popcll(ballot);
  lds_barrier();
  int pos = __popcll(ballot & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) pos += s_wave[w];
  if (keep) s_list[pos] = (uint16_t)j;
  if (j >= k && j < k_pad) s_list[j] = 0xFFFF;   // padding: reads as zero
  if (keep && is_q && blockIdx.x == 0) idx[(size_t)h * k + pos] = j;
  wait_vmcnt<0>();
  lds_barrier();

  // gather: output piece g = row * (k_pad / 8) + p holds kept positions
  // [8 p, 8 p + 8) of that row; the threads step through the pieces by a
  // multiple of k_pad / 8, so each keeps one p (and its 8 column indices)
  const int opr = k_pad >> 3;
  const int gstride = kSmallD / opr * opr;
  uint16_t* dst = (is_q ? qp + (size_t)h * tq * k_pad : kp + (size_t)h * tk * k_pad) + (size_t)r0 * k_pad;
  const int p = j % opr;
  // padding positions read column 0 and are masked to zero afterwards, so
  // every LDS read is unconditional and a row's 8 reads issue together
  uint32_t col[8], keep_mask[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t c = s_list[8 * p + e];
    col[e] = c == 0xFFFFu ? 0u : c;
    keep_mask[e] = c == 0xFFFFu ? 0u : 0xFFFFu;
  }
  for (int g = j < gstride ? j : nr * opr; g < nr * opr; g += gstride) {
    const int row = g / opr;
    const uint16_t* rb = s_rows + row * dh;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (uint32_t)rb[col[e]] & keep_mask[e];
    i32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (int)(v[2 * e] | (v[2 * e + 1] << 16));
    *(i32x4*)(dst + (size_t)row * k_pad + 8 * p) = w;
  }
}

}  // namespace

bool qk_select_pack_fits(const void* Q, const void* K, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts,
                         int64_t dh) {
  return dh <= kSmallD && dh % 8 == 0 && (uintptr_t)Q % 16 == 0 && (uintptr_t)K % 16 == 0 && q_hs % 8 == 0 &&
         q_ts % 8 == 0 && k_hs % 8 == 0 && k_ts % 8 == 0;
}

hipError_t launch_qk_select_pack(const float* partial, int splits, const uint16_t* Q, int64_t q_hs, int64_t q_ts,
                                 const uint16_t* K, int64_t k_hs, int64_t k_ts, int hq, int group, int tq, int tk,
                                 int dh, int k, int k_pad, int32_t* idx, uint16_t* qp, uint16_t* kp, hipStream_t s) {
  const int rb_rows = kQkElems / dh;
  const int blocks = (tq + rb_rows - 1) / rb_rows + (tk + rb_rows - 1) / rb_rows;
  qk_select_pack_kernel<<<dim3(blocks, hq), kSmallD, 0, s>>>(partial, splits, Q, q_hs, q_ts, K, k_hs, k_ts, group,
                                                            tq, tk, dh, k, k_pad, idx, qp, kp);
  return hipGetLastError();
}

int colnorm_splits(int heads, int n, int d, bool elt_bf16) {
  const int cb = kCnLanes * (elt_bf16 ? 8 : 4);
  const long col_blocks = (long)((d + cb - 1) / cb) * heads;
  // The sweep lasts as long as its busiest CU: the split count is the one
  // that spreads the workgroups most evenly over the 256 CUs (average over
  // maximum per CU), among those giving at least 1.5 workgroups per CU (so
  // that enough loads are in flight), the fewest on a tie.  Every split adds
  // d partials that the selection reads back, so wide rows take at most 8
  // (mlp_down: 4 splits, 448 workgroups, sweep 24.5 against 27.9 us with 5,
  // and the fused selection also faster); the short feature rows of
  // attention heads up to 32.
  const long max_by_rows = (n + 127) / 128;
  long smax = d <= 256 ? 32 : 8;
  if (smax > max_by_rows) smax = max_by_rows;
  if (smax < 1) smax = 1;
  long best = smax;
  double best_eff = -1.0;
  for (long sp = 1; sp <= smax; ++sp) {
    const long groups = col_blocks * sp;
    if (groups * 2 < 3L * 256 && sp < smax) continue;
    const long per_cu = (groups + 255) / 256;
    const double eff = (double)groups / (256.0 * (double)per_cu);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = sp;
    }
  }
  return (int)best;
}

hipError_t launch_colnorm(const void* A, bool elt_bf16, int64_t head_stride, int64_t lda, int heads, int n, int d,
                          int splits, float* partial, hipStream_t s) {
  const int cb = kCnLanes * (elt_bf16 ? 8 : 4);
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
                       int32_t* pad, int64_t pad_hs, int k_pad, float* scores, int64_t scores_hs, uint32_t* gkeys,
                       hipStream_t s, int32_t* mask, int64_t mask_hs, float* retained) {
  if (d <= kSmallD)
    topk_small_kernel<<<heads, kSmallD, 0, s>>>(partial, splits, d, k, idx, idx_hs, pad, pad_hs, k_pad, scores,
                                                scores_hs, mask, mask_hs, retained);
  else if (d <= 4096)
    topk_kernel<chunk_for(4096)><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, pad, pad_hs, k_pad,
                                                               scores, scores_hs, mask, mask_hs, retained, nullptr);
  else if (d <= 8192)
    topk_kernel<chunk_for(8192)><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, pad, pad_hs, k_pad,
                                                               scores, scores_hs, mask, mask_hs, retained, nullptr);
  else if (d <= kKeyCap)
    topk_kernel<kChunk><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, pad, pad_hs, k_pad, scores,
                                                      scores_hs, mask, mask_hs, retained, nullptr);
  else
    topk_kernel<0><<<heads, kSelThreads, 0, s>>>(partial, splits, d, k, idx, idx_hs, pad, pad_hs, k_pad, scores,
                                                 scores_hs, mask, mask_hs, retained, gkeys);
  return hipGetLastError();
}

bool select_pack_fits(const void* A, int64_t lda, int64_t d) {
  return d <= kKeyCap && d % 8 == 0 && lda % 8 == 0 && (uintptr_t)A % 16 == 0;
}

hipError_t launch_select_pack(const float* partial, int splits, const uint16_t* A, int64_t lda, int n, int d, int k,
                              int k_pad, int32_t* idx, int32_t* pad, uint16_t* out, hipStream_t s) {
  const int grid = n < kSpGroups ? n : kSpGroups;
  if (d <= 4096)
    select_pack_kernel<chunk_for(4096), 1, 5, true><<<grid, kSelThreads, 0, s>>>(
        partial, splits, nullptr, A, lda, n, d, k, k_pad, idx, pad, out);
  else if (d <= 8192)
    select_pack_kernel<chunk_for(8192), 1, 5, true><<<grid, kSelThreads, 0, s>>>(
        partial, splits, nullptr, A, lda, n, d, k, k_pad, idx, pad, out);
  else
    select_pack_kernel<kChunk, 2, 3, true><<<grid, kSelThreads, 0, s>>>(
        partial, splits, nullptr, A, lda, n, d, k, k_pad, idx, pad, out);
  return hipGetLastError();
}

bool gather_pack_fits(const void* A, int64_t lda, int64_t d, int64_t k_pad) {
  return select_pack_fits(A, lda, d) && k_pad <= kKeyCap;
}

hipError_t launch_gather_pack(const int32_t* given, int k, const uint16_t* A, int64_t lda, int n, int d, int k_pad,
                              int32_t* pad, uint16_t* out, hipStream_t s) {
  const int grid = n < kSpGroups ? n : kSpGroups;
  if (d <= 8192 && k_pad <= 8192)
    select_pack_kernel<4, 1, 5, false><<<grid, kSelThreads, 0, s>>>(nullptr, 0, given, A, lda, n, d, k, k_pad,
                                                                     nullptr, pad, out);
  else
    select_pack_kernel<4, 2, 3, false><<<grid, kSelThreads, 0, s>>>(nullptr, 0, given, A, lda, n, d, k, k_pad,
                                                                     nullptr, pad, out);
  return hipGetLastError();
}

hipError_t launch_pad_index(const int32_t* idx, int k, int d, int32_t* pad, int k_pad, hipStream_t s, int heads,
                            int64_t idx_hs, int64_t pad_hs) {
  pad_index_kernel<<<dim3((k_pad + 255) / 256, heads), 256, 0, s>>>(idx, idx_hs, k, d, pad, pad_hs, k_pad);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* idx, int64_t idx_hs, int heads, int d, int32_t* pad, int64_t pad_hs, int k_pad,
                       hipStream_t s) {
  const int span = pad && k_pad > d ? k_pad : d;
  dim3 grid((span + 255) / 256, heads);
  iota_kernel<<<grid, 256, 0, s>>>(idx, idx_hs, d, pad, pad_hs, k_pad);
  return hipGetLastError();
}

hipError_t launch_decode_select(const void* A, bool a_bf16, int64_t lda, int n, int d, int k, int32_t* idx,
                                float* scores, uint32_t* gkeys, hipStream_t s) {
  const int ch = d <= kKeyCap ? chunk_for(d) : 0;
  auto go = [&](auto bf, auto chv) {
    decode_select_kernel<decltype(bf)::value, decltype(chv)::value>
        <<<1, kSelThreads, 0, s>>>(A, lda, n, d, k, idx, scores, decltype(chv)::value > 0 ? nullptr : gkeys);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using C4 = std::integral_constant<int, chunk_for(4096)>;
  using C8 = std::integral_constant<int, chunk_for(8192)>;
  using CM = std::integral_constant<int, kChunk>;
  using C0 = std::integral_constant<int, 0>;
  if (a_bf16) {
    if (ch == chunk_for(4096)) go(T_{}, C4{});
    else if (ch == chunk_for(8192)) go(T_{}, C8{});
    else if (ch == kChunk) go(T_{}, CM{});
    else go(T_{}, C0{});
  } else {
    if (ch == chunk_for(4096)) go(F_{}, C4{});
    else if (ch == chunk_for(8192)) go(F_{}, C8{});
    else if (ch == kChunk) go(F_{}, CM{});
    else go(F_{}, C0{});
  }
  return hipGetLastError();
}

}  // namespace rmm
