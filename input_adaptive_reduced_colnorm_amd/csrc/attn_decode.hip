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
// lanes that span a row are folded with a fixed butterfly.  The kept
// features of a head (at most 256, from at most 8 query rows) are ranked by
// every workgroup in its prologue, so the decode step needs no separate
// scoring and TopK launches.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;
constexpr int kTokSteps = 8;   // token rows in flight per lane

template <int G, int LPT>
__global__ __launch_bounds__(kThreads) void qk_decode_kernel(const QkDecodeArgs a) {
  constexpr int TPW = 64 / LPT;                 // tokens per wave step
  constexpr int TPB = TPW * (kThreads / 64);    // tokens per workgroup step
  __shared__ float qm[G][256];
  __shared__ __attribute__((aligned(16))) uint64_t s_ck[kThreads];
  __shared__ int s_cnt[kThreads / 64];
  const int g = blockIdx.y;
  const int group = a.hq / a.hkv;
  const int tid = threadIdx.x;
  // ---- every feature of the group's query rows: qm[(h - g*group)*tq + r][f] ----
  for (int i = tid; i < G * 256; i += kThreads) {
    const int row = i / 256, f = i % 256;   // row = local head * tq + r
    float v = 0.f;
    if (row < group * a.tq && f < a.dh) {
      const int hl = row / a.tq, r = row % a.tq;
      const size_t off = (size_t)(g * group + hl) * a.q_hs + (size_t)r * a.q_ts + f;
      v = a.q_bf16 ? bf16_to_f32(((const uint16_t*)a.Q)[off]) : ((const float*)a.Q)[off];
    }
    qm[row][f] = v;
  }
  __syncthreads();
  // ---- the kept features of each query head of the group, from the column
  //      energies of its tq rows (row order; with bf16 Q every square is exact
  //      in fp32, so these keys equal the scoring pass's).  Each feature gets
  //      the composite key (energy bits, 0xFFFF - j): a larger composite
  //      outranks (higher energy, or equal energy and lower index), so one
  //      64-bit compare per pair ranks it, and feature j is kept when fewer
  //      than k composites exceed its own.  With dh <= 128 two heads are
  //      ranked at once.  Dropped features are zeroed in qm; the workgroups
  //      of the first token block write the ascending lists ----
  const int hp_n = a.dh <= 128 ? 2 : 1;                 // heads per pass
  const int tph = kThreads / hp_n;                      // threads per head
  const int hsub = tid / tph, jf = tid % tph;           // head within the pass, feature
  const int lane_ = tid & 63, wave_ = tid >> 6;
  for (int h0 = 0; h0 < group; h0 += hp_n) {
    const int hl = h0 + hsub;
    const bool live = hl < group && jf < a.dh;
    int32_t* out = a.idx_out + (size_t)(g * group + (hl < group ? hl : 0)) * a.k;
    if (!a.select) {
      if (blockIdx.x == 0 && live) out[jf] = jf;
      continue;
    }
    float key = 0.f;
    if (live)
      for (int r = 0; r < a.tq; ++r) key = fmaf(qm[hl * a.tq + r][jf], qm[hl * a.tq + r][jf], key);
    const uint64_t ck = ((uint64_t)__float_as_uint(key) << 32) | (uint32_t)(0xFFFF - jf);
    s_ck[tid] = ck;
    __syncthreads();
    // two composites per 16-byte LDS read, many reads in flight (dh % 8 == 0)
    const uint64_t* row = s_ck + hsub * tph;
    int rank = 0;
#pragma unroll 8
    for (int i2 = 0; i2 < a.dh / 2; ++i2) {
      const u64x2 v = *(const u64x2*)(row + 2 * i2);
      rank += (int)(v[0] > ck) + (int)(v[1] > ck);
    }
    const bool keep = live && rank < a.k;
    const uint64_t kept = __ballot(keep);
    if (lane_ == 0) s_cnt[wave_] = __popcll(kept);
    __syncthreads();
    int pos = __popcll(kept & ((1ull << lane_) - 1ull));
    for (int w = hsub * (tph / 64); w < wave_; ++w) pos += s_cnt[w];
    if (keep && blockIdx.x == 0) out[pos] = jf;
    if (live && !keep)
      for (int r = 0; r < a.tq; ++r) qm[hl * a.tq + r][jf] = 0.f;
    __syncthreads();   // s_ck and s_cnt are reused by the next pass
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT;                    // which 8 features
  const int tw = lane / LPT;                     // token within the wave step
  float q[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[j][e] = qm[j][sub * 8 + e];
  const uint16_t* Kg = (const uint16_t*)a.K + (size_t)g * a.k_hs;
  const int t_begin = blockIdx.x * a.tok_per_block;
  const int t_end = min(a.tk, t_begin + a.tok_per_block);
  for (int t0 = t_begin + wave * TPW + tw; t0 < t_end; t0 += TPB * kTokSteps) {
    i32x4 kv[kTokSteps];
#pragma unroll
    for (int u = 0; u < kTokSteps; ++u) {
      const int t = t0 + u * TPB;
      kv[u] = (t < t_end && sub * 8 < a.dh) ? *(const i32x4*)(Kg + (size_t)t * a.k_ts + sub * 8) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kTokSteps; ++u) {
      const int t = t0 + u * TPB;
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
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) v += __shfl_xor(v, o, 64);
        if (sub == 0 && t < t_end && j < group * a.tq) {
          const int hl = j / a.tq, r = j % a.tq;
          const size_t off = ((size_t)(g * group + hl) * a.tq + r) * a.tk + t;
          if (a.causal && t > r + a.tk - a.tq) v = -INFINITY;
          if (a.s_bf16)
            ((uint16_t*)a.S)[off] = f32_to_bf16(v);
          else
            ((float*)a.S)[off] = v;
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
