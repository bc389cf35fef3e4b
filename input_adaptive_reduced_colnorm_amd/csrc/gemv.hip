// Decode-shaped reduced product (n <= 16 rows of A): a bandwidth-bound
// GEMV that streams only the kept rows B[I, :].
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach: the product runs
// over the kept contraction indices only; with a handful of rows in A the
// cost is reading B, so reading ceil(rho d) of its d rows is the saving.
// Engineering Notes on the same page: prefill and decode are tuned apart.
//
// The multiply-adds run on the matrix cores: with fp32 FMAs on the vector
// ALUs every 16 bytes of B cost n x 8 FMAs, which at n = 8 is as long as
// streaming B itself and does not overlap with it.  Here one wave covers a
// 128-column strip: lane l loads 8 consecutive kept rows (8 (l / 16) ..)
// of the 8 columns 8 (l % 16) .. with 16-byte loads, transposes the 8x8
// block in registers, and feeds eight v_mfma_f32_16x16x32_bf16 (MFMA j
// takes the columns 8 c + j of the strip, c = l % 16, over 32 kept rows);
// the activations A[:, I] of the slice (n <= 16 rows, zero padded to 16)
// sit in LDS as bf16 and are the other operand.  Roofline: HBM; the matrix
// cores only take the arithmetic off the vector ALUs.
//
// Work split: the kept rows are cut into `splits` slices of at most 512
// (a multiple of 32) and the columns into 128-column strips; a 256-thread
// workgroup owns a (strip, slice) pair and its 4 waves take the slice's
// 32-row chunks round robin.  Vector loads retire in order, so a wave first
// loads every kept-row index it needs, then the activations it stages, and
// only then all of its B rows: no wait for an index or an activation also
// waits for B.  The waves are added in a fixed order in LDS; several slices
// write partial sums that a second kernel adds in slice order, so the
// result is bitwise reproducible.  int8 weights (a scale per output column,
// applied to the finished sum) are read with 8-byte loads and widened to
// bf16 in registers before the same transpose.

#include <type_traits>

#include "rmm_device.h"
#include "rmm_internal.h"
#include "select_block.h"

namespace rmm {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCols = 128;                    // output columns per workgroup (one wave's strip)
constexpr int kChunk = 32;                    // kept rows per MFMA step
constexpr int kChunksPerWave = 4;
constexpr int kMaxSlice = kWaves * kChunksPerWave * kChunk;   // 512 kept rows per workgroup
constexpr int kTargetGroups = 480;            // workgroups aimed for (256 CUs; measured best near 1.9 per CU)

__device__ __forceinline__ int slice_rows(int k, int splits) {
  return ((k + splits - 1) / splits + kChunk - 1) / kChunk * kChunk;
}

// The kept set ranked inside the GEMV (CH > 0): every workgroup computes
// the column energies of all of A (n <= 16 rows, read from L2 after the
// first touch) with the same fixed-order fp32 sums as the selection kernel,
// finds the k-th largest (energy, lowest index) key with the block radix
// search, and compacts the kept indices that fall in its own slice of the
// ascending list into LDS; the workgroups of the first column strip also
// write their slice of the list to idx_out.  This replaces the selection
// launch in front of the GEMV and the round trip of the list through memory.
// Thread t ranks the columns [t c, t c + c), c = ceil(d / 256) <= CH.
template <int CH, int NR, bool A_BF16>
__device__ __forceinline__ void rank_columns(const GemvArgs& g, sel::KeyChunk<CH>& kc) {
  const int tid = threadIdx.x;
  const int chunk = (g.d + kThreads - 1) / kThreads;
  kc.j0 = min(g.d, tid * chunk);
  kc.cnt = min(chunk, g.d - kc.j0);
  float q[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) q[i] = 0.f;
  const bool vec = A_BF16 && ((uintptr_t)g.A % 16 == 0) && (g.lda % 8 == 0) && (chunk % 8 == 0);
  if (vec) {
    // 16-byte loads; the loads of 8 rows are issued before they are used,
    // rows are added in ascending order
    constexpr int V = CH / 8;
    const char* base = (const char*)g.A + (size_t)kc.j0 * 2;
    for (int r0 = 0; r0 < NR; r0 += 8) {
      i32x4 x[8][V];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const bool ok = r0 + r < g.n && 8 * v < kc.cnt;
          x[r][v] = ok ? *(const i32x4*)(base + ((size_t)(r0 + r) * g.lda + 8 * v) * 2) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r0 + r < g.n) {
#pragma unroll
          for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t w = (uint32_t)x[r][v][e >> 1];
              const float f = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
              q[8 * v + e] = fmaf(f, f, q[8 * v + e]);
            }
        }
      }
    }
  } else {
    for (int r = 0; r < g.n; ++r) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (i < kc.cnt) {
          const size_t off = (size_t)r * g.lda + kc.j0 + i;
          const float f = A_BF16 ? bf16_to_f32(((const uint16_t*)g.A)[off]) : ((const float*)g.A)[off];
          q[i] = fmaf(f, f, q[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) kc.key[i] = __float_as_uint(q[i]);
}

template <int NR, bool A_BF16, bool B_I8, int CH = 0>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs g) {
  constexpr int BE = B_I8 ? 1 : 2;   // bytes per B element
  constexpr bool SEL = CH > 0;
  __shared__ __attribute__((aligned(16))) uint16_t s_a[16][kMaxSlice + 8];   // bf16 activations, row r, kept row t
  __shared__ float red[kWaves][16][kCols];
  __shared__ sel::Shared<SEL ? kWaves : 1> ssh;
  __shared__ int32_t s_list[SEL ? kMaxSlice : 1];
  {
    // batch member (attention head): shift every operand to its slice
    const int bz = blockIdx.z;
    g.A = (const char*)g.A + (size_t)bz * g.a_bs * (A_BF16 ? 2 : 4);
    g.B = (const char*)g.B + (size_t)(bz / g.b_group) * g.b_bs * BE;
    if (g.idx) g.idx += (size_t)bz * g.idx_bs;
    if (g.idx_out) g.idx_out += (size_t)bz * g.idx_bs;
    g.Y = (char*)g.Y + (size_t)bz * g.y_bs * (g.y_bf16 ? 2 : 4);
    g.partial += (size_t)bz * g.splits * g.n * g.m;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int slice = slice_rows(g.k, g.splits);
  const int t0 = blockIdx.y * slice;
  const int L = max(0, min(g.k, t0 + slice) - t0);
  const int rb = lane >> 4, cg = lane & 15;
  const int c = blockIdx.x * kCols + cg * 8;
  const bool col_ok = c < g.m;   // m is a multiple of 8
  const bool write_list = g.idx_out && blockIdx.x == 0;

  if constexpr (SEL) {
    // ---- rank every column of A and keep this slice of the ascending list ----
    sel::KeyChunk<CH> kc;
    rank_columns<CH, NR, A_BF16>(g, kc);
    int32_t* out = g.idx_out;
    sel::select_window<kThreads, CH>(kc, g.k, ssh, (uint32_t)t0, (uint32_t)(t0 + L), [&](uint32_t pos, int j) {
      s_list[pos - t0] = j;
      if (write_list) out[pos] = j;
    });
    __syncthreads();
  } else if (write_list) {
    // the identity list (rho = 1): the first strip's workgroups write it
    for (int i = tid; i < L; i += kThreads) g.idx_out[t0 + i] = t0 + i;
  }
  // a caller's list entry outside [0, d) (d > 0: the row count of B) reads
  // as a zero row
  auto kept = [&](int t) -> int {
    if constexpr (SEL) {
      return s_list[t];
    } else {
      if (!g.idx) return t0 + t;
      const int j = g.idx[t0 + t];
      return g.d > 0 && (unsigned)j >= (unsigned)g.d ? -1 : j;
    }
  };

  // ---- load order matters: vector loads retire in order, so a wait for a
  //      load also waits for every load issued before it.  First every
  //      kept-row index this thread needs: its B rows (chunk q covers slice
  //      rows (wave + 4 q) * 32 .., the lane its 8 rows 8 rb ..) and the up
  //      to two rows it stages.  A row of -1, or past the slice, is invalid ----
  int row[kChunksPerWave][8];
#pragma unroll
  for (int q = 0; q < kChunksPerWave; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = (wave + kWaves * q) * kChunk + 8 * rb + e;
      row[q][e] = t < L ? kept(t) : -1;
    }
  constexpr int PER = kMaxSlice / kThreads;
  const int L32 = (L + kChunk - 1) / kChunk * kChunk;
  int srow[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kThreads;
    srow[u] = i < L ? kept(i) : -1;
  }
  // ---- then the activations to stage and every B row, all unconditional
  //      (an invalid row reads row 0 and is zeroed where it is used), so the
  //      staging below waits for its own loads only ----
  using Act = typename std::conditional<A_BF16, uint16_t, float>::type;
  Act av[PER][NR];
#pragma unroll
  for (int u = 0; u < PER; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int rr = r < g.n ? r : 0;
      const int col = srow[u] >= 0 ? srow[u] : 0;
      av[u][r] = ((const Act*)g.A)[(size_t)rr * g.lda + col];
    }
  __builtin_amdgcn_sched_barrier(0);   // keep every activation load ahead of the B loads
  typedef typename RowPiece<B_I8>::type R;
  R bv[kChunksPerWave][8];
  const int cc0 = col_ok ? c : 0;
#pragma unroll
  for (int q = 0; q < kChunksPerWave; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int rw = row[q][e] >= 0 ? row[q][e] : 0;
      bv[q][e] = __builtin_nontemporal_load((const R*)((const char*)g.B + ((size_t)rw * g.ldb + cc0) * BE));
    }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kThreads;
    if (i < L32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uint16_t v = 0;
        if (r < NR && r < g.n && srow[u] >= 0) {
          if constexpr (A_BF16)
            v = av[u][r < NR ? r : 0];
          else
            v = f32_to_bf16(av[u][r < NR ? r : 0]);
        }
        s_a[r][i] = v;
      }
    }
  }
  __syncthreads();

  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kChunksPerWave; ++q) {
    const int tb = (wave + kWaves * q) * kChunk;
    if (tb >= L) break;   // uniform across the wave
    // A operand: row l % 16 of A, kept rows tb + 8 (l / 16) ..
    const bf16x8 af = *(const bf16x8*)&s_a[cg][tb + 8 * rb];
    i32x4 rows8[8], tr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (row[q][e] < 0 || !col_ok)
        rows8[e] = i32x4{0, 0, 0, 0};
      else if constexpr (B_I8)
        rows8[e] = i8x8_to_bf16x8(bv[q][e]);
      else
        rows8[e] = bv[q][e];
    }
    transpose8x8(rows8, tr);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, tr[j]), acc[j], 0, 0, 0);
  }

  // ---- lane l, register v of acc[j]: row 4 (l / 16) + v, column
  //      8 (l % 16) + j of the strip.  Waves are added in order ----
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * rb + v;
    if (r < g.n) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave][r][cg * 8 + j] = acc[j][v];
    }
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
    for (int w = 1; w < kWaves; ++w) v += red[w][r][cc];
    if (direct) {
      const size_t off = (size_t)r * g.ldy + col;
      if (g.col_scale) v *= g.col_scale[col];
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
  // the loads of 16 slices are issued before they are added (in order)
  float v = 0.f;
  for (int s0 = 0; s0 < g.splits; s0 += 16) {
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = s0 + t < g.splits ? part[(size_t)(s0 + t) * g.n * g.m + i] : 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (s0 + t < g.splits) v += x[t];
  }
  if (g.col_scale) v *= g.col_scale[col];
  const size_t off = (size_t)bz * g.y_bs + (size_t)r * g.ldy + col;
  if (g.y_bf16)
    ((uint16_t*)g.Y)[off] = f32_to_bf16(v);
  else
    ((float*)g.Y)[off] = v;
}

}  // namespace

// Upper bound of gemv_splits(k, m, batch) over every k <= kmax: the split
// count before whole-chunk slicing is at most the larger of the target
// count and the minimum that keeps slices within kMaxSlice, and slicing only
// lowers it.
int gemv_splits_bound(int kmax, int m, int batch) {
  const int strips = (m + kCols - 1) / kCols;
  const int by_target = (kTargetGroups + strips * batch - 1) / (strips * batch);
  const int by_slice = (kmax + kMaxSlice - 1) / kMaxSlice;
  const int s = by_target > by_slice ? by_target : by_slice;
  return s < 1 ? 1 : s;
}

int gemv_splits(int k, int m, int batch) {
  const int strips = (m + kCols - 1) / kCols;
  int splits = (kTargetGroups + strips * batch - 1) / (strips * batch);
  const int min_splits = (k + kMaxSlice - 1) / kMaxSlice;
  if (splits < min_splits) splits = min_splits;
  // at least one 32-row chunk per wave
  const int max_splits = (k + kWaves * kChunk - 1) / (kWaves * kChunk);
  if (splits > max_splits) splits = max_splits > min_splits ? max_splits : min_splits;
  if (splits < 1) splits = 1;
  // slices are whole chunks: drop splits that would be empty
  const int slice = ((k + splits - 1) / splits + kChunk - 1) / kChunk * kChunk;
  return (k + slice - 1) / slice;
}

template <int NR, int CH>
void launch_nr_ch(const GemvArgs& g, dim3 grid, hipStream_t s) {
  if (g.b_i8)
    gemv_kernel<NR, true, true, CH><<<grid, kThreads, 0, s>>>(g);   // int8 weights take bf16 activations
  else if (g.a_bf16)
    gemv_kernel<NR, true, false, CH><<<grid, kThreads, 0, s>>>(g);
  else
    gemv_kernel<NR, false, false, CH><<<grid, kThreads, 0, s>>>(g);
}

template <int NR>
void launch_nr(const GemvArgs& g, dim3 grid, hipStream_t s) {
  if (!g.select)
    launch_nr_ch<NR, 0>(g, grid, s);
  else if (g.d <= 16 * kThreads)
    launch_nr_ch<NR, 16>(g, grid, s);
  else
    launch_nr_ch<NR, 32>(g, grid, s);
}

int gemv_select_max_d() { return 32 * kThreads; }

hipError_t launch_gemv(const GemvArgs& g, hipStream_t s) {
  if (g.n > 16 || (g.b_i8 && !g.a_bf16)) return hipErrorInvalidValue;
  if (g.select && (g.batch != 1 || g.d > gemv_select_max_d() || g.d < g.k || g.idx)) return hipErrorInvalidValue;
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
