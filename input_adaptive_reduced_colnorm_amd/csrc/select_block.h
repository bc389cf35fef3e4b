// Block-wide TopK helpers for a workgroup of NT threads (NT a multiple of
// 64, at most 1024): the radix search for the k-th largest key and the
// ordered compaction of the kept indices.  Shared by the TopK kernels (1024
// threads) and the decode GEMV, whose 256-thread workgroups rank the
// columns of A themselves.
//
// Keys are the fp32 bit patterns of non-negative energies (so their integer
// order is their value order); the k largest are kept, equal keys going to
// the lower index, and the kept indices come out ascending ("Algorithm
// Deep-Dive: RMM" (hackcv.com), Core Approach: TopK by the column norm).
// Only integer LDS atomics are used, so the result is reproducible.  The
// helpers exchange data through LDS alone, so their barriers are LDS-only
// (lds_barrier): loads the caller has in flight (a prefetch) keep flying.
#pragma once

#include "rmm_device.h"

namespace rmm {
namespace sel {

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

constexpr int kHistBins = 2048;         // 11-bit radix digits
constexpr uint32_t kFoldAbove = 2048;   // bucket size from which a radix pass folds equal digits

constexpr int kBucketBins = 4096;       // one 12-bit digit (bucket search)
constexpr int kMaxCand = 128;           // keys of the k-th key's bucket ranked exactly

template <int NW>
struct alignas(16) Shared {
  uint32_t hist[3 * kHistBins];   // one histogram per radix pass (the bucket search uses the first 4096)
  uint32_t misc[4];
  uint32_t wave_tot[NW][2];
  uint32_t wave_nz[NW];
  double energy[NW][2];
  uint32_t cand_n;
  uint2 cand[kMaxCand];           // (key, index) of the k-th key's bucket
};

// Block-wide inclusive scan of two counters (NT threads, fixed order).
template <int NT>
__device__ __forceinline__ void block_incl_scan2(uint32_t& a, uint32_t& b, Shared<NT / 64>& sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if (lane == 63) {
    sh.wave_tot[wave][0] = a;
    sh.wave_tot[wave][1] = b;
  }
  lds_barrier();
  uint32_t pa = 0, pb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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
// Each thread owns kHistBins / NT consecutive buckets (counted from the
// top) for the scan that locates the k-th key.
template <int NT, int CH>
__device__ __forceinline__ void radix_threshold(const KeyChunk<CH>& kc, int k, Shared<NT / 64>& sh, uint32_t* T,
                                                uint32_t* rem_out) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kHistBins / NT;
  static_assert(BPT * NT == kHistBins, "thread count must divide the histogram");
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
  for (int i = tid; i < 3 * kHistBins; i += NT) sh.hist[i] = 0;
  if (lane == 0) {
    sh.wave_tot[wave][0] = k_min;
    sh.wave_tot[wave][1] = k_max;
    sh.wave_nz[wave] = nz;
  }
  lds_barrier();
  k_min = 0xffffffffu;
  k_max = 0u;
  nz = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    k_min = min(k_min, sh.wave_tot[w][0]);
    k_max = max(k_max, sh.wave_tot[w][1]);
    nz += sh.wave_nz[w];
  }
  // every wave has read wave_tot before any of them returns early: the
  // compaction's block scan writes wave_tot next, and a wave that is still
  // reading here would otherwise take a scan total for kmin (all nonzero
  // keys equal, or k above the nonzero count, both skip the radix passes)
  lds_barrier();
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
    lds_barrier();
    // thread t owns the buckets nb-1-BPT t .. nb-BPT-BPT t, counted from the top
    const int top = (int)nb - 1 - BPT * tid;
    uint32_t c[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = top - i >= 0 ? hist[top - i] : 0u;
      sum += c[i];
    }
    uint32_t incl = sum, dummy = 0;
    block_incl_scan2<NT>(incl, dummy, sh);
    const uint32_t excl = incl - sum;
    if (excl < rem && rem <= incl) {
      uint32_t run = excl;
      bool found = false;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        if (!found && run + c[i] >= rem) {
          sh.misc[0] = (uint32_t)(top - i);
          sh.misc[1] = rem - run;
          sh.misc[2] = c[i];
          found = true;
        }
        run += c[i];
      }
    }
    lds_barrier();
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

// Threshold in one histogram pass where it can be (the usual case): the
// kept set is every key with (key, -index) >= (T, -jT) in lexicographic
// order, i.e. the keys above T and, among the keys equal to T, those with
// index <= jT.  Steps: the nonzero keys' range [kmin, kmax] and count
// (wave DPP reductions, one barrier, which also covers the histogram
// clear); one 12-bit histogram of key - kmin shifted so the range fills
// the 4096 buckets; a block scan over the buckets from the top finds the
// bucket b holding the k-th largest key and how many of its keys are kept
// (rem); if that is all of them the threshold is b's lower edge, otherwise
// the bucket's keys (at most kMaxCand) are gathered and ranked exactly by
// (key desc, index asc) and the one of rank rem - 1 is the threshold.
// Returns false, having decided nothing, when k exceeds the nonzero count
// or the bucket is larger than kMaxCand (runs of equal keys): the caller
// then runs radix_threshold and compact_ascending.  The bucket ranking is
// order independent, so the result does not depend on the order in which
// the gathered keys land in LDS.
template <int NT, int CH>
__device__ __forceinline__ bool bucket_threshold(const KeyChunk<CH>& kc, int k, Shared<NT / 64>& sh, uint32_t* T,
                                                 int* jT) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kBucketBins / NT;   // buckets per thread (16 or 4)
  static_assert(BPT * NT == kBucketBins && BPT % 4 == 0, "thread count must divide the buckets by 4s");
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
  for (int i = tid; i < kBucketBins / 4; i += NT) ((uint4*)sh.hist)[i] = uint4{0u, 0u, 0u, 0u};
  if (tid == 0) sh.cand_n = 0u;
  if (lane == 0) {
    sh.wave_tot[wave][0] = k_min;
    sh.wave_tot[wave][1] = k_max;
    sh.wave_nz[wave] = nz;
  }
  lds_barrier();
  k_min = 0xffffffffu;
  k_max = 0u;
  nz = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    k_min = min(k_min, sh.wave_tot[w][0]);
    k_max = max(k_max, sh.wave_tot[w][1]);
    nz += sh.wave_nz[w];
  }
  lds_barrier();   // wave_tot is rewritten below
  if ((uint32_t)k > nz) return false;   // zero keys are kept: the radix path handles them
  const uint32_t span = k_max - k_min;
  const int bits = span ? 32 - __clz(span) : 0;
  const int shift = bits > 12 ? bits - 12 : 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    if (i < kc.cnt && key != 0u) atomicAdd(&sh.hist[(key - k_min) >> shift], 1u);
  }
  lds_barrier();
  // thread t owns buckets 4095 - BPT t down to 4096 - BPT (t + 1), read as
  // 16-byte groups (ascending in memory, so the top bucket is the last word)
  const int lo = kBucketBins - BPT * (tid + 1);
  uint32_t c[BPT], sum = 0;
#pragma unroll
  for (int q = 0; q < BPT / 4; ++q) {
    const uint4 v = ((const uint4*)sh.hist)[lo / 4 + q];
    c[4 * q] = v.x;
    c[4 * q + 1] = v.y;
    c[4 * q + 2] = v.z;
    c[4 * q + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += c[i];
  uint32_t incl = sum, dummy = 0;
  block_incl_scan2<NT>(incl, dummy, sh);
  const uint32_t excl = incl - sum;
  if (excl < (uint32_t)k && (uint32_t)k <= incl) {
    uint32_t run = excl;
    bool found = false;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {   // from this thread's top bucket down
      if (!found && run + c[i] >= (uint32_t)k) {
        sh.misc[0] = (uint32_t)(lo + i);
        sh.misc[1] = (uint32_t)k - run;
        sh.misc[2] = c[i];
        found = true;
      }
      run += c[i];
    }
  }
  lds_barrier();
  const uint32_t b = sh.misc[0], rem = sh.misc[1], cnt = sh.misc[2];
  if (cnt == rem) {
    // the whole bucket is kept: every key at or above its lower edge
    *T = k_min + (b << shift);
    *jT = 0x7fffffff;
    return true;
  }
  if (cnt > (uint32_t)kMaxCand) return false;
  // gather the bucket's keys (slots in arrival order), then rank them
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    if (i < kc.cnt && key != 0u && ((key - k_min) >> shift) == b) {
      const uint32_t slot = atomicAdd(&sh.cand_n, 1u);
      sh.cand[slot] = uint2{key, (uint32_t)(kc.j0 + i)};
    }
  }
  lds_barrier();
  if (tid < (int)cnt) {
    const uint2 me = sh.cand[tid];
    uint32_t rank = 0;
    for (uint32_t m = 0; m < cnt; ++m) {
      const uint2 o = sh.cand[m];
      rank += (o.x > me.x) || (o.x == me.x && o.y < me.y);
    }
    if (rank == rem - 1) {
      sh.misc[0] = me.x;
      sh.misc[1] = me.y;
    }
  }
  lds_barrier();
  *T = sh.misc[0];
  *jT = (int)sh.misc[1];
  return true;
}

// Ordered compaction against a composite threshold (bucket_threshold): a
// key is kept when key > T, or key == T and its index <= jT.  A block scan
// of the per-thread kept counts fixes each thread's output position, so the
// kept indices come out ascending; emit(take, pos, j, key) is called once
// for every index j of the chunk, in order.
template <int NT, int CH, typename Emit>
__device__ __forceinline__ void compact_composite(const KeyChunk<CH>& kc, uint32_t T, int jT, Shared<NT / 64>& sh,
                                                  Emit emit) {
  uint32_t n_take = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    n_take += i < kc.cnt && (key > T || (key == T && kc.j0 + i <= jT));
  }
  uint32_t incl = n_take, dummy = 0;
  block_incl_scan2<NT>(incl, dummy, sh);
  uint32_t pos = incl - n_take;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < kc.cnt) {
      const uint32_t key = kc.key[i];
      const bool take = key > T || (key == T && kc.j0 + i <= jT);
      emit(take, pos, kc.j0 + i, key);
      pos += take;
    }
  }
}

// The kept indices whose output positions fall in [lo, hi), for a caller
// that needs only one window of the ascending list: fn(pos, j) for each.  A
// thread whose kept run misses the window does nothing after the scan.
template <int NT, int CH, typename Fn>
__device__ __forceinline__ void compact_window(const KeyChunk<CH>& kc, uint32_t T, int jT, Shared<NT / 64>& sh,
                                               uint32_t lo, uint32_t hi, Fn fn) {
  uint32_t n_take = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    n_take += i < kc.cnt && (key > T || (key == T && kc.j0 + i <= jT));
  }
  uint32_t incl = n_take, dummy = 0;
  block_incl_scan2<NT>(incl, dummy, sh);
  uint32_t pos = incl - n_take;
  if (pos >= hi || incl <= lo) return;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t key = kc.key[i];
    const bool take = i < kc.cnt && (key > T || (key == T && kc.j0 + i <= jT));
    if (take && pos >= lo && pos < hi) fn(pos, kc.j0 + i);
    pos += take;
  }
}

// Threshold and ordered compaction: the bucket search where it decides,
// else the radix search (zero keys kept, or long runs of equal keys).
template <int NT, int CH, typename Emit>
__device__ __forceinline__ void select_ascending(const KeyChunk<CH>& kc, int k, Shared<NT / 64>& sh, Emit emit) {
  uint32_t T;
  int jT;
  if (bucket_threshold<NT, CH>(kc, k, sh, &T, &jT)) {
    compact_composite<NT, CH>(kc, T, jT, sh, emit);
  } else {
    uint32_t rem;
    radix_threshold<NT, CH>(kc, k, sh, &T, &rem);
    compact_ascending<NT, CH>(kc, T, rem, sh, emit);
  }
}

// Which indices are kept, without their list positions: fn(j) for every
// kept index j of the chunk.  Where the bucket search decides, each thread
// tests its own keys against the composite threshold and no block scan
// runs; otherwise the radix search and the ordered compaction run as in
// select_ascending.
template <int NT, int CH, typename Fn>
__device__ __forceinline__ void select_kept(const KeyChunk<CH>& kc, int k, Shared<NT / 64>& sh, Fn fn) {
  uint32_t T;
  int jT;
  if (bucket_threshold<NT, CH>(kc, k, sh, &T, &jT)) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t key = kc.key[i];
      if (i < kc.cnt && (key > T || (key == T && kc.j0 + i <= jT))) fn(kc.j0 + i);
    }
  } else {
    uint32_t rem;
    radix_threshold<NT, CH>(kc, k, sh, &T, &rem);
    compact_ascending<NT, CH>(kc, T, rem, sh, [&](bool take, uint32_t, int j, uint32_t) {
      if (take) fn(j);
    });
  }
}

// One window [lo, hi) of the ascending kept list (see compact_window).
template <int NT, int CH, typename Fn>
__device__ __forceinline__ void select_window(const KeyChunk<CH>& kc, int k, Shared<NT / 64>& sh, uint32_t lo,
                                              uint32_t hi, Fn fn) {
  uint32_t T;
  int jT;
  if (bucket_threshold<NT, CH>(kc, k, sh, &T, &jT)) {
    compact_window<NT, CH>(kc, T, jT, sh, lo, hi, fn);
  } else {
    uint32_t rem;
    radix_threshold<NT, CH>(kc, k, sh, &T, &rem);
    compact_ascending<NT, CH>(kc, T, rem, sh, [&](bool take, uint32_t pos, int j, uint32_t) {
      if (take && pos >= lo && pos < hi) fn(pos, j);
    });
  }
}

// Ordered compaction: every thread owns a contiguous index chunk; a block
// scan of (#greater, #equal) fixes each thread's output position, so the kept
// indices come out ascending.  emit(take, pos, j, key) is called once for
// every index j of the chunk, in order; pos is the output position when take.
template <int NT, int CH, typename Emit>
__device__ __forceinline__ void compact_ascending(const KeyChunk<CH>& kc, uint32_t T, uint32_t rem,
                                                  Shared<NT / 64>& sh, Emit emit) {
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < kc.cnt) {
      n_gt += kc.key[i] > T;
      n_eq += kc.key[i] == T;
    }
  }
  uint32_t i_gt = n_gt, i_eq = n_eq;
  block_incl_scan2<NT>(i_gt, i_eq, sh);
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

}  // namespace sel
}  // namespace rmm
