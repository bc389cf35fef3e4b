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
// Block-wide helpers for 1024-thread selection workgroups.
// ---------------------------------------------------------------------------
// Wave-wide inclusive scans on the DPP cross-lane paths (no LDS round
// trip): shifts by 1, 2, 4 and 8 lanes inside each row of 16, then the
// totals of rows 0 and 2 broadcast into rows 1 and 3 (row_bcast:15) and the
// total of rows 0-1 into rows 2-3 (row_bcast:31).  Lanes whose source is
// outside the pattern take `id`, the identity of the operation.
template <typename F>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x, uint32_t id, F op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));   // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));   // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));   // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));   // row_shr:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));   // row_bcast:15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  return wave_scan_dpp(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

constexpr int kHistBins = 2048;  // 11-bit radix digits
constexpr uint32_t kFoldAbove = 2048;   // bucket size from which a radix pass folds equal digits
constexpr int kChunk = (kKeyCap + kSelThreads - 1) / kSelThreads;  // most keys per thread held in registers

// Keys per thread for a key count d held in LDS: the radix passes run one
// unrolled histogram step per register slot, so the slot count follows d.
__host__ __device__ constexpr int chunk_for(int d) { return d <= 4096 ? 4 : (d <= 8192 ? 8 : kChunk); }

struct SelShared {
  uint32_t hist[3 * kHistBins];   // one histogram per radix pass
  uint32_t misc[4];
  uint32_t wave_tot[kSelWaves][2];
  uint32_t wave_nz[kSelWaves];
  double energy[kSelWaves][2];
};

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

// Block-wide inclusive scan of two counters (1024 threads, fixed order).
__device__ __forceinline__ void block_incl_scan2(uint32_t& a, uint32_t& b, SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if (lane == 63) {
    sh.wave_tot[wave][0] = a;
    sh.wave_tot[wave][1] = b;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t ta = sh.wave_tot[w][0], tb = sh.wave_tot[w][1];
    if (w < wave) {
      pa += ta;
      pb += tb;
    }
  }
  a += pa;
  b += pb;
}

// The keys of one thread: a contiguous index chunk [j0, j0 + cnt), kept in
// registers across all radix passes and the compaction.
template <int CH>
struct KeyChunk {
  uint32_t key[CH];
  int j0, cnt;
};

template <int CH>
__device__ __forceinline__ void load_chunk(const uint32_t* keys, int d, KeyChunk<CH>& kc) {
  const int chunk = (d + kSelThreads - 1) / kSelThreads;   // <= CH
  kc.j0 = min(d, (int)threadIdx.x * chunk);
  kc.cnt = min(chunk, d - kc.j0);
#pragma unroll
  for (int i = 0; i < CH; ++i) kc.key[i] = i < kc.cnt ? keys[kc.j0 + i] : 0u;
}

// Histogram increments.  hist_add_lane: one LDS atomic per active lane, the
// cheapest form while the lanes' digits are spread over many bins.
// hist_add: the lanes that share the first active lane's digit are folded
// into one atomic, for buckets where ties are likely (a run of equal keys
// sends every lane of a wave to one address, and per-lane atomics on one
// address serialize); it costs about twice the instructions per key.
__device__ __forceinline__ void hist_add_lane(uint32_t* hist, bool m, uint32_t dig) {
  if (m) atomicAdd(&hist[dig], 1u);
}

__device__ __forceinline__ void hist_add(uint32_t* hist, bool m, uint32_t dig) {
  const uint64_t act = __ballot(m);
  if (act == 0) return;
  const int first = __ffsll((unsigned long long)act) - 1;
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dig, first);
  const uint64_t same = __ballot(m && dig == d0);
  if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
  if (m && dig != d0) atomicAdd(&hist[dig], 1u);
}

// Finds the k-th largest key: on return *T is its value and *rem the number
// of keys equal to T that belong to the kept set (the lowest-indexed ones;
// 0xffffffff means every key equal to T is kept).  MSB-first radix passes
// with integer LDS histograms of up to 11-bit digits, over the offsets
// key - kmin of the nonzero keys: the first digit starts at the top bit of
// kmax - kmin, so the first histogram spreads over 1024-2048 buckets
// whatever the keys' magnitude (fp32 energies of a few octaves would share
// their sign and upper exponent bits and crowd a few dozen buckets).  All
// histograms are cleared up front, and the passes stop as soon as the
// bucket holding the k-th key is kept whole.  Zero keys (energies that are
// exactly zero or underflowed, often thousands of ties) stay out of the
// histograms: when k exceeds the nonzero count the answer is T = 0 at once,
// otherwise no zero key can be kept.  The first pass adds one atomic per
// lane; a later pass folds equal digits only when the bucket it refines
// holds more than kFoldAbove keys (a bucket that large makes ties likely).
template <int CH>
__device__ __forceinline__ void radix_threshold(const KeyChunk<CH>& kc, int k, SelShared& sh, uint32_t* T, uint32_t* rem_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t k_min = 0xffffffffu, k_max = 0u, nz = 0u;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    const bool live = i < kc.cnt && key != 0u;
    k_min = min(k_min, live ? key : 0xffffffffu);
    k_max = max(k_max, live ? key : 0u);
    nz += live;
  }
  k_min = (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_scan_dpp(k_min, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }), 63);
  k_max = (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_scan_dpp(k_max, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }), 63);
  nz = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(nz), 63);
  for (int i = tid; i < 3 * kHistBins; i += kSelThreads) sh.hist[i] = 0;
  if (lane == 0) {
    sh.wave_tot[wave][0] = k_min;
    sh.wave_tot[wave][1] = k_max;
    sh.wave_nz[wave] = nz;
  }
  __syncthreads();
  k_min = 0xffffffffu;
  k_max = 0u;
  nz = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    k_min = min(k_min, sh.wave_tot[w][0]);
    k_max = max(k_max, sh.wave_tot[w][1]);
    nz += sh.wave_nz[w];
  }
  // every wave has read wave_tot before any of them returns early: the
  // compaction's block scan writes wave_tot next, and a wave that is still
  // reading here would otherwise take a scan total for kmin (all nonzero
  // keys equal, or k above the nonzero count, both skip the radix passes)
  __syncthreads();
  if ((uint32_t)k > nz) {
    // every nonzero key is kept, and the lowest-indexed zeros fill up to k
    *T = 0u;
    *rem_out = (uint32_t)k - nz;
    return;
  }
  // from here k <= nz, so kmin <= kmax are keys; offsets lie in [0, span]
  const uint32_t span = k_max - k_min;
  int hi = span ? 32 - __clz(span) : 0;      // offset bits still to resolve
  uint32_t mask = hi == 32 ? 0u : ~((1u << hi) - 1u);
  uint32_t prefix = 0u;                      // resolved offset bits
  uint32_t rem = (uint32_t)k;
  bool fold = false;
  for (int pass = 0; hi > 0; ++pass) {
    const int w = hi < 11 ? hi : 11;
    const int shift = hi - w;
    const uint32_t nb = 1u << w;
    uint32_t* hist = sh.hist + pass * kHistBins;
    if (fold) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const uint32_t key = kc.key[i], off = key - k_min;
        hist_add(hist, i < kc.cnt && key != 0u && (off & mask) == prefix, (off >> shift) & (nb - 1));
      }
    } else {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const uint32_t key = kc.key[i], off = key - k_min;
        hist_add_lane(hist, i < kc.cnt && key != 0u && (off & mask) == prefix, (off >> shift) & (nb - 1));
      }
    }
    __syncthreads();
    // thread t owns the buckets nb-1-2t and nb-2-2t, counted from the top
    const int b0 = (int)nb - 1 - 2 * tid, b1 = b0 - 1;
    const uint32_t c0 = b0 >= 0 ? hist[b0] : 0u, c1 = b1 >= 0 ? hist[b1] : 0u;
    uint32_t incl = c0 + c1, dummy = 0;
    block_incl_scan2(incl, dummy, sh);
    const uint32_t excl = incl - (c0 + c1);
    if (excl < rem && rem <= incl) {
      if (excl + c0 >= rem) {
        sh.misc[0] = (uint32_t)b0;
        sh.misc[1] = rem - excl;
        sh.misc[2] = c0;
      } else {
        sh.misc[0] = (uint32_t)b1;
        sh.misc[1] = rem - excl - c0;
        sh.misc[2] = c1;
      }
    }
    __syncthreads();
    const uint32_t b = sh.misc[0], cnt = sh.misc[2];
    rem = sh.misc[1];
    prefix |= b << shift;
    mask |= (nb - 1) << shift;
    hi = shift;
    fold = cnt > kFoldAbove;
    if (cnt == rem) {
      // every key of this bucket is kept: keep all keys >= its lowest value
      // (at least kmin, so no zero key)
      *T = k_min + prefix;
      *rem_out = 0xffffffffu;
      return;
    }
  }
  *T = k_min + prefix;
  *rem_out = rem;
}

// Ordered compaction: every thread owns a contiguous index chunk; a block
// scan of (#greater, #equal) fixes each thread's output position, so the kept
// indices come out ascending.  emit(take, pos, j, key) is called once for
// every index j of the chunk, in order; pos is the output position when take.
template <int CH, typename Emit>
__device__ __forceinline__ void compact_ascending(const KeyChunk<CH>& kc, uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < kc.cnt) {
      n_gt += kc.key[i] > T;
      n_eq += kc.key[i] == T;
    }
  }
  uint32_t i_gt = n_gt, i_eq = n_eq;
  block_incl_scan2(i_gt, i_eq, sh);
  uint32_t pos = (i_gt - n_gt) + min(i_eq - n_eq, rem);
  uint32_t eq_seen = i_eq - n_eq;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < kc.cnt) {
      const uint32_t key = kc.key[i];
      bool take = key > T;
      if (key == T) {
        take = eq_seen < rem;
        ++eq_seen;
      }
      emit(take, pos, kc.j0 + i, key);
      pos += take;
    }
  }
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
  __shared__ int32_t s_out[LDS_KEYS ? kKeyCap : 1];
  __shared__ SelShared sh;
  const int head = blockIdx.x;
  const float* P = partial + (size_t)head * splits * d;
  uint32_t* keys = LDS_KEYS ? s_keys : gkeys + (size_t)head * d;
  if constexpr (LDS_KEYS) {
    if (d % 4 == 0) {
      // 4 columns per 16-byte load; a thread takes up to four 4-column
      // groups at once and issues the loads of all of them for up to six
      // splits before adding any (each column in split order)
      constexpr int G = 4, S = 6;
      const int d4 = d / 4;
      const f32x4* P4 = (const f32x4*)P;
      for (int jb = threadIdx.x; jb < d4; jb += G * kSelThreads) {
        f32x4 q[G];
#pragma unroll
        for (int u = 0; u < G; ++u) q[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < splits; s0 += S) {
          f32x4 v[G][S];
#pragma unroll
          for (int u = 0; u < G; ++u)
#pragma unroll
            for (int t = 0; t < S; ++t) {
              const int j4 = jb + u * kSelThreads;
              v[u][t] = (s0 + t < splits && j4 < d4) ? P4[(size_t)(s0 + t) * d4 + j4] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
          for (int u = 0; u < G; ++u)
#pragma unroll
            for (int t = 0; t < S; ++t)
              if (s0 + t < splits) {
                q[u][0] += v[u][t][0];
                q[u][1] += v[u][t][1];
                q[u][2] += v[u][t][2];
                q[u][3] += v[u][t][3];
              }
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const int j4 = jb + u * kSelThreads;
          if (j4 < d4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              keys[4 * j4 + e] = __float_as_uint(q[u][e]);
              if (scores) scores[(size_t)head * scores_hs + 4 * j4 + e] = sqrtf(q[u][e]);
            }
          }
        }
      }
    } else {
      // each thread owns columns tid + 1024 c; the loads of four splits are
      // issued together before they are added (in split order)
      constexpr int NC = CH > 0 ? CH : 1;
      float q[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) q[c] = 0.f;
      for (int s0 = 0; s0 < splits; s0 += 4) {
        float v[4][NC];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int j = threadIdx.x + c * kSelThreads;
            v[u][c] = (s0 + u < splits && j < d) ? P[(size_t)(s0 + u) * d + j] : 0.f;
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < splits)
#pragma unroll
            for (int c = 0; c < NC; ++c) q[c] += v[u][c];
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int j = threadIdx.x + c * kSelThreads;
        if (j < d) {
          keys[j] = __float_as_uint(q[c]);
          if (scores) scores[(size_t)head * scores_hs + j] = sqrtf(q[c]);
        }
      }
    }
  } else {
    for (int j = threadIdx.x; j < d; j += kSelThreads) {
      float q = 0.f;
      for (int s = 0; s < splits; ++s) q += P[(size_t)s * d + j];
      keys[j] = __float_as_uint(q);
      if (scores) scores[(size_t)head * scores_hs + j] = sqrtf(q);
    }
  }
  if (!LDS_KEYS) __threadfence_block();
  __syncthreads();
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
    // the kept list is assembled in LDS and written out coalesced; the keys
    // now live in registers, so s_keys takes the keep flags
    KeyChunk<CH> kc;
    load_chunk(keys, d, kc);
    radix_threshold(kc, k, sh, &T, &rem);
    if (retained || mo) {
      compact_ascending(kc, T, rem, sh, [&](bool take, uint32_t pos, int j, uint32_t key) {
        if (take) s_out[pos] = j;
        s_keys[j] = take;
        const double q = (double)__uint_as_float(key);
        e_all += q;
        e_kept += take ? q : 0.0;
      });
    } else {
      compact_ascending(kc, T, rem, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
        if (take) s_out[pos] = j;
      });
    }
    __syncthreads();
    for (int t = threadIdx.x; t < k; t += kSelThreads) {
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
__global__ void pad_index_kernel(const int32_t* __restrict__ idx, int k, int d, int32_t* __restrict__ pad, int k_pad) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= k_pad) return;
  int v = -1;
  if (t < k) {
    const int j = idx[t];
    v = (j >= 0 && j < d) ? j : -1;
  }
  pad[t] = v;
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
    radix_threshold(kc, k, sh, &T, &rem);
    compact_ascending(kc, T, rem, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
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

}  // namespace

int colnorm_splits(int heads, int n, int d, bool elt_bf16) {
  const int cb = kCnLanes * (elt_bf16 ? 8 : 4);
  const long col_blocks = (long)((d + cb - 1) / cb) * heads;
  // about 560 workgroups: more splits stream A a little faster (5.2 -> 5.4
  // TB/s at 1800 groups) but cost the selection more than they save
  long s = (560 + col_blocks - 1) / col_blocks;
  long max_by_rows = (n + 127) / 128;
  if (s > max_by_rows) s = max_by_rows;
  // the selection re-reads splits x d partials in one workgroup: few
  // splits for wide rows, more for the short feature rows of attention heads
  const long max_splits = d <= 256 ? 32 : 16;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  return (int)s;
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

hipError_t launch_pad_index(const int32_t* idx, int k, int d, int32_t* pad, int k_pad, hipStream_t s) {
  pad_index_kernel<<<(k_pad + 255) / 256, 256, 0, s>>>(idx, k, d, pad, k_pad);
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
