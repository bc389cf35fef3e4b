// Decode-shaped reduced QK^T: a few query rows per head (tq <= 16) against
// a key cache, S[h][r][t] = sum over f in I_h of Q[h][r][f] K[g(h)][t][f],
// with the selection of I_h done in the same kernel.
//
// hackcv.com, Component mapping: QK^T contracts over the head feature
// dimension, selection runs on Q per head and K gathers the same feature
// dims on its GQA head; hackcv.com, Engineering Notes: decode is tuned apart
// from prefill.  At decode the cost is reading the key cache, so the
// product is written as a streaming pass over K: one workgroup takes a block
// of tokens of one kv head and all the query heads of its group; each lane
// holds, for its 8 consecutive features, the query values of every (head,
// row) of the group with the unselected features set to zero, and every K
// row is read once with 16-byte loads.  The partial dot products of the
// lanes that span a row are folded in a fixed order on the DPP cross-lane
// paths, all of a pass's tokens at once.  The kept
// features of a head (at most 256, from at most 8 query rows) are ranked by
// every workgroup in its prologue (one wave per head, ballot counts, no LDS
// traffic), while the workgroup's first key rows are already in flight, so
// the decode step needs no separate scoring and TopK launches.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;
constexpr int kTokSteps = 8;   // token rows in flight per lane

// Workgroup barrier that waits for this wave's LDS operations only, not for
// its global loads in flight (__syncthreads' release fence would wait for
// those too).
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum of a token's partial dot products over its LPT lanes, on the DPP
// cross-lane paths (no LDS round trip): xor 1 and xor 2 inside each quad,
// then each lane with its mirror in the half-row (lane i with 7 - i) and in
// the row (i with 15 - i).  Every lane of a quad holds the same quad sum
// after the first two steps, so lane 0 adds the same pairs in the same order
// as a butterfly over xor 1, 2, 4 and 8; LPT = 32 adds the other row of 16
// through a cross-lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int LPT>
__device__ __forceinline__ float fold_lanes(float v) {
  v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);   // row_half_mirror
  if constexpr (LPT >= 16) v += dpp_move<0x140>(v);   // row_mirror
  if constexpr (LPT >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

template <int G, int LPT>
__global__ __launch_bounds__(kThreads) void qk_decode_kernel(const QkDecodeArgs a) {
  constexpr int TPW = 64 / LPT;                 // tokens per wave step
  constexpr int TPB = TPW * (kThreads / 64);    // tokens per workgroup step
  __shared__ float qm[G][256];
  const int g = blockIdx.y;
  const int group = a.hq / a.hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT;                    // which 8 features
  const int tw = lane / LPT;                     // token within the wave step
  // the first key rows are requested before the query loads and the ranking,
  // so that their fetch overlaps the prologue
  const uint16_t* Kg = (const uint16_t*)a.K + (size_t)g * a.k_hs;
  const int t_begin = blockIdx.x * a.tok_per_block;
  const int t_end = min(a.tk, t_begin + a.tok_per_block);
  const int t_first = t_begin + wave * TPW + tw;
  i32x4 kv[kTokSteps];
  // loads outside any branch (out-of-range lanes read a clamped in-range
  // row and drop the value), so that the waits before each use count exactly
  // the loads issued after it
  auto load_k = [&](int t0) {
#pragma unroll
    for (int u = 0; u < kTokSteps; ++u) {
      const int t = t0 + u * TPB;
      const bool ok = t < t_end && sub * 8 < a.dh;
      const size_t off = ok ? (size_t)t * a.k_ts + sub * 8 : (size_t)t_begin * a.k_ts;
      const i32x4 v = *(const i32x4*)(Kg + off);
      kv[u] = ok ? v : i32x4{0, 0, 0, 0};
    }
  };
  // ---- every feature of the group's query rows: qm[(h - g*group)*tq + r][f],
  //      thread tid loading feature tid of each row.  The query loads go
  //      out first and the first key rows right after them: loads complete in
  //      issue order, so the query values can be waited for while the key
  //      rows stay in flight through the ranking (the barriers wait for LDS
  //      only) ----
  uint16_t qv[G];
#pragma unroll
  for (int row = 0; row < G; ++row) {   // row = local head * tq + r
    const bool ok = row < group * a.tq && tid < a.dh;
    const int hl = ok ? row / a.tq : 0, r = ok ? row % a.tq : 0;
    const size_t off = ok ? (size_t)(g * group + hl) * a.q_hs + (size_t)r * a.q_ts + tid : 0;
    const uint16_t v = ((const uint16_t*)a.Q)[off];
    qv[row] = ok ? v : (uint16_t)0;
  }
  load_k(t_first);
#pragma unroll
  for (int row = 0; row < G; ++row) qm[row][tid] = bf16_to_f32(qv[row]);
  lds_sync();
  // ---- the kept features of each query head of the group, from the column
  //      energies of its tq rows (row order; with bf16 Q every square is exact
  //      in fp32, so these keys equal the scoring pass's).  Each feature gets
  //      the composite key (energy bits, 0xFFFF - j): a larger composite
  //      outranks (higher energy, or equal energy and lower index).  One wave
  //      per head finds the energy of the k-th largest composite with 32-bit
  //      compares and ballot counts, keeps the features above it and, among
  //      those equal to it, the lowest indices up to k places; it zeroes the
  //      others in qm, and the workgroups of the first token block write the
  //      ascending lists ----
  for (int hl = wave; hl < group; hl += kThreads / 64) {
    int32_t* out = a.idx_out + (size_t)(g * group + hl) * a.k;
    if (!a.select) {
      if (blockIdx.x == 0)
        for (int j = lane; j < a.dh; j += 64) out[j] = j;
      continue;
    }
    constexpr int NCH = LPT / 8;   // feature j = lane + 64 c, c < NCH (dh <= 8 LPT)
    uint32_t e[NCH];               // energy bits; 0 on lanes past dh
    uint64_t live[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = lane + 64 * c;
      float key = 0.f;
      if (j < a.dh)
        for (int r = 0; r < a.tq; ++r) key = fmaf(qm[hl * a.tq + r][j], qm[hl * a.tq + r][j], key);
      e[c] = j < a.dh ? __float_as_uint(key) : 0u;
      live[c] = __ballot(j < a.dh);
    }
    // Th: the energy bits of the k-th largest composite, built from the top
    // bit down (a bit stays set while at least k features reach the
    // candidate; the candidate is never 0, so lanes past dh never count)
    uint32_t Th = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = Th | (1u << b);
      int n = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) n += __popcll(__ballot(e[c] >= cand));
      if (n >= a.k) Th = cand;
    }
    // every feature above Th is kept; the other places go to the lowest
    // indices among the features equal to Th
    int above = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) above += __popcll(__ballot(e[c] > Th));
    const int eq_places = a.k - above;
    const uint64_t lt = (1ull << lane) - 1ull;
    int base = 0, eq_before = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = lane + 64 * c;
      const bool lv = j < a.dh;
      const uint64_t eqm = __ballot(e[c] == Th) & live[c];
      const bool keep =
          a.k > 0 && lv && (e[c] > Th || (e[c] == Th && eq_before + __popcll(eqm & lt) < eq_places));
      const uint64_t kept = __ballot(keep);
      if (keep && blockIdx.x == 0) out[base + __popcll(kept & lt)] = j;
      base += __popcll(kept);
      eq_before += __popcll(eqm);
      if (lv && !keep)
        for (int r = 0; r < a.tq; ++r) qm[hl * a.tq + r][j] = 0.f;
    }
  }
  lds_sync();
  float q[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[j][e] = qm[j][sub * 8 + e];
  // the S row of each (head, query row) of the group, and the last key
  // position it sees under the causal mask
  size_t srow[G];
  int tmax[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int hl = j / a.tq, r = j % a.tq;
    srow[j] = ((size_t)(g * group + hl) * a.tq + r) * a.tk;
    tmax[j] = a.causal ? r + a.tk - a.tq : a.tk;
  }
  // all dot products of the token steps first, then their lane folds, then
  // the stores, so that no product waits on another's fold or store
  for (int t0 = t_first; t0 < t_end; t0 += TPB * kTokSteps) {
    if (t0 != t_first) load_k(t0);
    float sv[kTokSteps][G];
#pragma unroll
    for (int u = 0; u < kTokSteps; ++u) {
      float kf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t bits = (uint32_t)kv[u][w];
        kf[2 * w] = __uint_as_float(bits << 16);
        kf[2 * w + 1] = __uint_as_float(bits & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float v = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v = fmaf(q[j][e], kf[e], v);
        sv[u][j] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < kTokSteps; ++u)
#pragma unroll
      for (int j = 0; j < G; ++j) sv[u][j] = fold_lanes<LPT>(sv[u][j]);
    if (sub == 0) {
#pragma unroll
      for (int u = 0; u < kTokSteps; ++u) {
        const int t = t0 + u * TPB;
#pragma unroll
        for (int j = 0; j < G; ++j) {
          if (t < t_end && j < group * a.tq) {
            const float v = t > tmax[j] ? -INFINITY : sv[u][j];
            if (a.s_bf16)
              ((uint16_t*)a.S)[srow[j] + t] = f32_to_bf16(v);
            else
              ((float*)a.S)[srow[j] + t] = v;
          }
        }
      }
    }
  }
}

template <int G>
hipError_t launch_g(const QkDecodeArgs& a, dim3 grid, hipStream_t s) {
  const int lpt = a.dh / 8;
  if (lpt <= 8)
    qk_decode_kernel<G, 8><<<grid, kThreads, 0, s>>>(a);
  else if (lpt <= 16)
    qk_decode_kernel<G, 16><<<grid, kThreads, 0, s>>>(a);
  else
    qk_decode_kernel<G, 32><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool qk_decode_fits(int group, int tq, int dh) { return group * tq <= 8 && dh % 8 == 0 && dh <= 256; }

hipError_t launch_qk_decode(QkDecodeArgs a, hipStream_t s) {
  if (!a.q_bf16) return hipErrorInvalidValue;   // the kernel reads bf16 queries
  // about 512 workgroups in all, at least 64 tokens each
  int tpb = (int)(((long)a.tk * a.hkv + 511) / 512);
  tpb = tpb < 64 ? 64 : (tpb + 63) / 64 * 64;
  a.tok_per_block = tpb;
  dim3 grid((a.tk + tpb - 1) / tpb, a.hkv);
  const int G = (a.hq / a.hkv) * a.tq;
  if (G <= 1) return launch_g<1>(a, grid, s);
  if (G <= 2) return launch_g<2>(a, grid, s);
  if (G <= 4) return launch_g<4>(a, grid, s);
  return launch_g<8>(a, grid, s);
}

}  // namespace rmm
