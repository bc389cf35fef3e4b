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
// Work split: the rows are cut into `splits` slices of at most 512 (a
// multiple of 32; slices of a given or the identity list, or of the source
// rows of B where the kernel ranks A itself, see gemv_rank_kernel) and the
// columns into 128-column strips; a 256-thread
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
constexpr int kSliceStride = kMaxSlice + 8;   // LDS row of staged activations
constexpr int kHeadChunks = 1;                // ranking GEMV: chunks per wave requested before the ranking

__host__ __device__ __forceinline__ int slice_rows(int k, int splits) {
  return ((k + splits - 1) / splits + kChunk - 1) / kChunk * kChunk;
}

// One 32-row MFMA step of a wave: the A operand (row l % 16 of the slice's
// activations, kept rows 8 (l / 16) ..) from LDS, the lane's 8 B row pieces
// (zeroed where `valid` is clear or the columns lie past m) transposed into
// the eight column operands.
template <bool B_I8>
__device__ __forceinline__ void mfma_step(const bf16x8 af, const typename RowPiece<B_I8>::type (&bv)[8],
                                          uint32_t valid, f32x4 (&acc)[8]) {
  i32x4 rows8[8], tr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!((valid >> e) & 1u))
      rows8[e] = i32x4{0, 0, 0, 0};
    else if constexpr (B_I8)
      rows8[e] = i8x8_to_bf16x8(bv[e]);
    else
      rows8[e] = bv[e];
  }
  transpose8x8(rows8, tr);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, tr[j]), acc[j], 0, 0, 0);
}

// The workgroup's result: lane l, register v of acc[j] holds row 4 (l / 16)
// + v, column 8 (l % 16) + j of the strip.  The waves are added in order in
// LDS; one slice writes Y directly, several write their partial sums.
__device__ __forceinline__ void store_strip(const GemvArgs& g, const f32x4 (&acc)[8], float (&red)[kWaves][16][kCols]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = lane >> 4, cg = lane & 15;
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

// Product over a given list (idx; entries outside [0, d) read as zero rows
// when d > 0) or over the identity list (idx null: rows t0 .. of B, the
// list also written to idx_out by the first strip's workgroups).  The
// kept rows are cut into `splits` slices of the list.
template <int NR, bool A_BF16, bool B_I8>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs g) {
  constexpr int BE = B_I8 ? 1 : 2;   // bytes per B element
  __shared__ __attribute__((aligned(16))) uint16_t s_a[16][kSliceStride];   // bf16 activations, row r, kept row t
  __shared__ float red[kWaves][16][kCols];
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

  if (g.idx_out && blockIdx.x == 0) {
    // the identity list (rho = 1): the first strip's workgroups write it
    for (int i = tid; i < L; i += kThreads) g.idx_out[t0 + i] = t0 + i;
  }
  // ---- load order matters: vector loads retire in order, so a wait for a
  //      load also waits for every load issued before it.  First every
  //      kept-row index this thread needs: its B rows (chunk q covers slice
  //      rows (wave + 4 q) * 32 .., the lane its 8 rows 8 rb ..) and the up
  //      to two rows it stages.  The list loads are unconditional (positions
  //      past the slice read its last entry) and issued together, so one
  //      wait covers them all; then positions past the slice and entries
  //      outside [0, d) become -1 (invalid) ----
  constexpr int PER = kMaxSlice / kThreads;
  const int L32 = (L + kChunk - 1) / kChunk * kChunk;
  int row[kChunksPerWave][8];
  int srow[PER];
  if (g.idx && L > 0) {
    const int32_t* ip = g.idx + t0;
#pragma unroll
    for (int q = 0; q < kChunksPerWave; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (wave + kWaves * q) * kChunk + 8 * rb + e;
        row[q][e] = ip[t < L ? t : L - 1];
      }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kThreads;
      srow[u] = ip[i < L ? i : L - 1];
    }
    auto check = [&](int t, int j) {
      return t < L && !(g.d > 0 && (unsigned)j >= (unsigned)g.d) ? j : -1;
    };
#pragma unroll
    for (int q = 0; q < kChunksPerWave; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) row[q][e] = check((wave + kWaves * q) * kChunk + 8 * rb + e, row[q][e]);
#pragma unroll
    for (int u = 0; u < PER; ++u) srow[u] = check(tid + u * kThreads, srow[u]);
  } else {
#pragma unroll
    for (int q = 0; q < kChunksPerWave; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (wave + kWaves * q) * kChunk + 8 * rb + e;
        row[q][e] = t < L ? t0 + t : -1;
      }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kThreads;
      srow[u] = i < L ? t0 + i : -1;
    }
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
    uint32_t valid = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) valid |= (uint32_t)(row[q][e] >= 0 && col_ok) << e;
    mfma_step<B_I8>(*(const bf16x8*)&s_a[cg][tb + 8 * rb], bv[q], valid, acc);
  }
  store_strip(g, acc, red);
}

// ---------------------------------------------------------------------------
// The kept set ranked inside the GEMV (rho < 1, d <= 8192 columns, one
// product per launch).  Every workgroup computes the column energies of all
// of A (n <= 16 rows, read from L2 after the first touch) with the same
// fixed-order fp32 sums as the selection kernel and finds the k-th largest
// (energy, lowest index) key with the block search.  The slices here are
// ranges of source rows of B, not of the kept list: workgroup (strip,
// slice) owns rows [r0, r0 + S).  Ranking takes several microseconds, and a
// workgroup that waited for it before requesting B would leave HBM idle
// meanwhile; so the first kHeadChunks 32-row chunks of each wave (the
// slice's first 128 source rows) are requested before the ranking,
// whatever their fate, and a dropped row among them is zeroed on both
// operands; after the ranking only the kept rows of the rest of the slice
// are requested.  The loads of A for the energies go out first, the head's
// B rows right after them, so the energies wait for A alone.  The
// workgroup stages the activations of its own source rows from those same
// A loads.  The first strip's workgroups write their rows' positions of the
// ascending list to idx_out at the end.
// Thread t ranks the columns [t c, t c + c), c = ceil(d / 256) <= CH.
// `issue` is called once the last batch of A's loads is in flight (on the
// element-load path, after all of A); `src[r][o]` receives the bf16 value
// A[r][r0 + o] for the slice's columns.
template <int CH, int NR, bool A_BF16, typename Issue>
__device__ __forceinline__ void rank_columns(const GemvArgs& g, sel::KeyChunk<CH>& kc,
                                             uint16_t (&src)[16][kSliceStride], int r0, int Ls, Issue issue) {
  const int tid = threadIdx.x;
  const int chunk = (g.d + kThreads - 1) / kThreads;
  kc.j0 = min(g.d, tid * chunk);
  kc.cnt = min(chunk, g.d - kc.j0);
  // does this thread's chunk hold columns of the slice?
  const bool mine = kc.j0 < r0 + Ls && kc.j0 + kc.cnt > r0;
  float q[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) q[i] = 0.f;
  const bool vec = A_BF16 && ((uintptr_t)g.A % 16 == 0) && (g.lda % 8 == 0) && (chunk % 8 == 0);
  if (vec) {
    // 16-byte loads in batches of RB rows (16 loads per lane in flight),
    // each batch issued before it is used; rows are added in ascending order
    constexpr int V = CH / 8;
    constexpr int RB = 16 / V < NR ? 16 / V : NR;
    const char* base = (const char*)g.A + (size_t)kc.j0 * 2;
    auto load_batch = [&](int rb0, i32x4 (&x)[RB][V]) {
      // unconditional (a masked lane reads the start of A), so that the
      // energies can wait for these loads alone
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const bool ok = rb0 + r < g.n && 8 * v < kc.cnt;
          const char* pa = ok ? base + ((size_t)(rb0 + r) * g.lda + 8 * v) * 2 : (const char*)g.A;
          const i32x4 t = *(const i32x4*)pa;
          x[r][v] = ok ? t : i32x4{0, 0, 0, 0};
        }
    };
    auto fold_batch = [&](int rb0, const i32x4 (&x)[RB][V]) {
      // the slice's columns go to LDS as whole 16-byte groups (o is a
      // multiple of 8; past Ls they are never read)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int o = kc.j0 + 8 * v - r0;
          if (mine && rb0 + r < g.n && 8 * v < kc.cnt && (unsigned)o < (unsigned)Ls)
            *(i32x4*)&src[rb0 + r][o] = x[r][v];
        }
      // every row is folded (a row past n is zero and adds +0 exactly): a
      // fold under a branch would let the compiler sink its loads below the
      // head's, and the energies would wait for B
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = (uint32_t)x[r][v][e >> 1];
            const float f = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            q[8 * v + e] = fmaf(f, f, q[8 * v + e]);
          }
    };
    // batches of RB rows (16 loads of 16 bytes per lane in flight), rows
    // added in ascending order; the head goes out after the last batch's
    // loads, so that its energies wait for A alone
#pragma unroll 1
    for (int rb0 = 0; rb0 + RB < NR; rb0 += RB) {
      i32x4 x[RB][V];
      load_batch(rb0, x);
      fold_batch(rb0, x);
    }
    {
      i32x4 x[RB][V];
      load_batch(NR - RB, x);
      __builtin_amdgcn_sched_barrier(0);
      issue();
      __builtin_amdgcn_sched_barrier(0);
      fold_batch(NR - RB, x);
    }
  } else {
    // element loads, a row's CH loads in flight together (unconditional: a
    // masked lane reads the start of A); the head goes out after them
    for (int r = 0; r < g.n; ++r) {
      float f[CH];
      uint16_t h[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const size_t off = i < kc.cnt ? (size_t)r * g.lda + kc.j0 + i : 0;
        if constexpr (A_BF16) {
          h[i] = ((const uint16_t*)g.A)[off];
          f[i] = bf16_to_f32(h[i]);
        } else {
          f[i] = ((const float*)g.A)[off];
          h[i] = 0;
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (i < kc.cnt) {
          q[i] = fmaf(f[i], f[i], q[i]);
          const int o = kc.j0 + i - r0;
          if (mine && (unsigned)o < (unsigned)Ls) src[r][o] = A_BF16 ? h[i] : f32_to_bf16(f[i]);
        }
      }
    }
    issue();
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) kc.key[i] = __float_as_uint(q[i]);
}

// LDS of the ranking GEMV: the block search's scratch and the slice's
// activations are dead once the slice's rows are listed, so the wave sums
// at the end reuse their space.
struct RankStage {
  sel::Shared<kWaves> ssh;
  alignas(16) uint16_t src[16][kSliceStride];   // bf16 A[r][r0 + o] for the slice's source rows
};
union RankLds {
  RankStage st;
  float red[kWaves][16][kCols];
};

template <int NR, bool A_BF16, bool B_I8, int CH>
__global__ __launch_bounds__(kThreads, 2) void gemv_rank_kernel(GemvArgs g) {
  constexpr int BE = B_I8 ? 1 : 2;
  constexpr int HC = kHeadChunks;           // head chunks per wave
  constexpr int HR = HC * kWaves * kChunk;  // head rows of the slice (128)
  constexpr uint16_t kNone = 0xffff;   // s_pos of a dropped row (list positions are < k <= 8192)
  __shared__ __attribute__((aligned(16))) uint16_t s_a[16][kSliceStride];   // activations by MFMA position
  __shared__ __attribute__((aligned(16))) RankLds u;
  __shared__ __attribute__((aligned(16))) uint16_t s_pos[kMaxSlice];    // list position of source row r0 + o (first strip; 0 marks a kept row elsewhere)
  __shared__ __attribute__((aligned(16))) uint16_t s_rest[kMaxSlice];   // kept offsets o >= HR, ascending
  __shared__ uint32_t s_cnt;                                              // kept rows past the head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = slice_rows(g.d, g.splits);
  const int r0 = blockIdx.y * S;
  const int Ls = max(0, min(g.d, r0 + S) - r0);
  const int rb = lane >> 4, cg = lane & 15;
  const int c = blockIdx.x * kCols + cg * 8;
  const bool col_ok = c < g.m;   // m is a multiple of 8
  const int cc0 = col_ok ? c : 0;
  typedef typename RowPiece<B_I8>::type R;
  R bv[kChunksPerWave][8];

  // head: chunk q < HC of this wave holds the source offsets
  // (wave + 4 q) * 32 + 8 rb + e; offsets past the slice read row 0 and are
  // zeroed below
  auto issue_head = [&]() {
#pragma unroll
    for (int q = 0; q < HC; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = (wave + kWaves * q) * kChunk + 8 * rb + e;
        const int rw = o < Ls ? r0 + o : 0;
        bv[q][e] = __builtin_nontemporal_load((const R*)((const char*)g.B + ((size_t)rw * g.ldb + cc0) * BE));
      }
  };
  for (int i = tid; i < kMaxSlice; i += kThreads) {
    s_pos[i] = kNone;
    s_rest[i] = kNone;   // past the kept rows the list reads as "none"
  }
  sel::KeyChunk<CH> kc;
  rank_columns<CH, NR, A_BF16>(g, kc, u.st.src, r0, Ls, issue_head);
  // the ranking's barriers order the s_pos clear and the src stores before
  // anything below reads them.  Only the workgroups that write idx (the
  // first strip) need list positions; the others mark their kept rows
  // (position 0) and skip the ordered compaction's block scan
  if (g.idx_out && blockIdx.x == 0) {
    sel::select_ascending<kThreads, CH>(kc, g.k, u.st.ssh, [&](bool take, uint32_t pos, int j, uint32_t) {
      const int o = j - r0;
      if (take && (unsigned)o < (unsigned)Ls) s_pos[o] = (uint16_t)pos;
    });
  } else {
    sel::select_kept<kThreads, CH>(kc, g.k, u.st.ssh, [&](int j) {
      const int o = j - r0;
      if ((unsigned)o < (unsigned)Ls) s_pos[o] = 0;
    });
  }
  lds_barrier();

  // ---- the kept offsets past the head, in order (two per thread), from
  //      index 0 of their own list so that 8 of them are one 16-byte read ----
  {
    // both entries in one aligned read (o0 is even; past the array the
    // offsets are past Ls too and the read is masked)
    const int o0 = HR + 2 * tid;
    const uint32_t pp = *(const uint32_t*)&s_pos[o0 < kMaxSlice ? o0 : 0];
    const bool k0 = o0 < Ls && (pp & 0xffffu) != kNone;
    const bool k1 = o0 + 1 < Ls && (pp >> 16) != kNone;
    const uint32_t n_r = (uint32_t)k0 + (uint32_t)k1;
    uint32_t inc = n_r, unused = 0;
    sel::block_incl_scan2<kThreads>(inc, unused, u.st.ssh);
    uint32_t p = inc - n_r;
    if (k0) s_rest[p++] = (uint16_t)o0;
    if (k1) s_rest[p] = (uint16_t)(o0 + 1);
    if (tid == kThreads - 1) s_cnt = inc;
  }
  lds_barrier();
  const int Lr = (int)s_cnt;   // kept rows after the head

  // ---- rest: rest chunk i = wave + 4 (q - HC) takes rest entries 32 i ..;
  //      the lane's 8 entries in one read, loads unconditional as in
  //      gemv_kernel ----
  int rrow[kChunksPerWave][8];
#pragma unroll
  for (int q = HC; q < kChunksPerWave; ++q) {
    const i32x4 w = *(const i32x4*)&s_rest[(wave + kWaves * (q - HC)) * kChunk + 8 * rb];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t o = ((uint32_t)w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      rrow[q][e] = o != kNone ? r0 + (int)o : -1;
    }
  }
#pragma unroll
  for (int q = HC; q < kChunksPerWave; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int rw = rrow[q][e] >= 0 ? rrow[q][e] : 0;
      bv[q][e] = __builtin_nontemporal_load((const R*)((const char*)g.B + ((size_t)rw * g.ldb + cc0) * BE));
    }

  // ---- activations by MFMA position, 8 positions of one row per item: the
  //      head's source offsets (dropped rows and offsets past the slice
  //      zero), then the rest's kept rows, zero padded to a chunk; rows past
  //      n zero ----
  const int groups = (HR + (Lr + kChunk - 1) / kChunk * kChunk) / 8;
  for (int w = tid; w < 16 * groups; w += kThreads) {
    const int r = w / groups, t0 = 8 * (w - r * groups);
    i32x4 v = i32x4{0, 0, 0, 0};
    if (r < g.n) {
      if (t0 < HR) {
        const i32x4 a = *(const i32x4*)&u.st.src[r][t0];
        const i32x4 pw = *(const i32x4*)&s_pos[t0];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t m = (((uint32_t)pw[h] & 0xffffu) != kNone ? 0x0000ffffu : 0u) |
                             (((uint32_t)pw[h] >> 16) != kNone ? 0xffff0000u : 0u);
          v[h] = (int)((uint32_t)a[h] & m);
        }
      } else {
        // past the kept rows the list holds kNone: those positions read
        // offset 0 and are masked, so the 8 reads issue unconditionally
        const i32x4 ow = *(const i32x4*)&s_rest[t0 - HR];
        uint32_t e[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t o = ((uint32_t)ow[h >> 1] >> (16 * (h & 1))) & 0xffffu;
          e[h] = (uint32_t)u.st.src[r][o != kNone ? o : 0u] & (o != kNone ? 0xffffu : 0u);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) v[h] = (int)(e[2 * h] | (e[2 * h + 1] << 16));
      }
    }
    *(i32x4*)&s_a[r][t0] = v;
  }
  lds_barrier();

  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kChunksPerWave; ++q) {
    uint32_t valid = 0;
    int tb;
    if (q < HC) {
      tb = (wave + kWaves * q) * kChunk;
      if (tb >= Ls) continue;   // uniform across the wave
      const i32x4 pw = *(const i32x4*)&s_pos[tb + 8 * rb];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t pe = ((uint32_t)pw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        valid |= (uint32_t)(tb + 8 * rb + e < Ls && pe != kNone && col_ok) << e;
      }
    } else {
      const int ti = (wave + kWaves * (q - HC)) * kChunk;
      if (ti >= Lr) continue;   // uniform across the wave
      tb = HR + ti;
#pragma unroll
      for (int e = 0; e < 8; ++e) valid |= (uint32_t)(rrow[q][e] >= 0 && col_ok) << e;
    }
    mfma_step<B_I8>(*(const bf16x8*)&s_a[cg][tb + 8 * rb], bv[q], valid, acc);
  }
  // the sums overwrite the ranking's LDS: its last readers (the staging
  // above) are behind the barrier before the products
  store_strip(g, acc, u.red);

  if (g.idx_out && blockIdx.x == 0) {
    for (int o = tid; o < Ls; o += kThreads)
      if (s_pos[o] != kNone) g.idx_out[s_pos[o]] = r0 + o;
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
void launch_rank(const GemvArgs& g, dim3 grid, hipStream_t s) {
  if (g.b_i8)
    gemv_rank_kernel<NR, true, true, CH><<<grid, kThreads, 0, s>>>(g);   // int8 weights take bf16 activations
  else if (g.a_bf16)
    gemv_rank_kernel<NR, true, false, CH><<<grid, kThreads, 0, s>>>(g);
  else
    gemv_rank_kernel<NR, false, false, CH><<<grid, kThreads, 0, s>>>(g);
}

template <int NR>
void launch_nr(const GemvArgs& g, dim3 grid, hipStream_t s) {
  if (!g.select) {
    if (g.b_i8)
      gemv_kernel<NR, true, true><<<grid, kThreads, 0, s>>>(g);
    else if (g.a_bf16)
      gemv_kernel<NR, true, false><<<grid, kThreads, 0, s>>>(g);
    else
      gemv_kernel<NR, false, false><<<grid, kThreads, 0, s>>>(g);
  } else if (g.d <= 16 * kThreads) {
    launch_rank<NR, 16>(g, grid, s);
  } else {
    launch_rank<NR, 32>(g, grid, s);
  }
}

int gemv_select_max_d() { return 32 * kThreads; }

hipError_t launch_gemv(const GemvArgs& g, hipStream_t s) {
  if (g.n > 16 || (g.b_i8 && !g.a_bf16)) return hipErrorInvalidValue;
  if (g.select && (g.batch != 1 || g.d > gemv_select_max_d() || g.d < g.k || g.idx)) return hipErrorInvalidValue;
  // slices: of the source rows (select) or of the list, at most kMaxSlice
  // rows each, and the grid must cover them
  const int rows = g.select ? g.d : g.k;
  const int slice = slice_rows(rows, g.splits);
  if (g.splits < 1 || slice > kMaxSlice || (int64_t)slice * g.splits < rows) return hipErrorInvalidValue;
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
