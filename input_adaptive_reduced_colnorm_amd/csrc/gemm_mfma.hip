// Reduced product Y = A[:, I] * B[I, :] on gfx950 matrix cores.
//
// "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach (Formula Level):
// the reduced product multiplies densely over the kept contraction slice
// only, with the weights unchanged.  Here A arrives already packed to the
// kept columns (K contiguous, zero padded to the tile depth), and the kept
// rows of B are gathered by index inside the tile loader, so the contraction
// runs over ceil(rho d) indices and nothing else.  The same kernel with the
// identity index is the rho = 1 dense baseline.
//
// Tiling: BM x BN x 64 per workgroup.  Large products use 256 x 256 tiles
// over 8 waves (2 x 4, two waves per SIMD so that one wave's MFMAs cover the
// other's LDS traffic and barrier); small ones 128 x 128 over 4 waves (2 x 2).
// Each wave owns a block of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16.  The loads of K tile kt + 2 are issued while
// tile kt is multiplied; one barrier per K tile.  With K-major B (the linear
// products) bf16 A goes straight from the buffer into a ring of three LDS
// stages and the k16 steps run as a software pipeline with a pinned
// instruction order (see the main loop); otherwise both operands pass
// through registers into two LDS stages.  LDS rows are 128 bytes (64 bf16
// along K) with an XOR swizzle of the 16-byte chunks.
// B tiles that are K-major in memory (weights, V) are transposed in
// registers in 8x8 blocks (v_perm) before they reach LDS; int8 weights are
// loaded 8 bytes at a time and widened to bf16 just before that transpose,
// their per-column scale applied in the epilogue.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int BK = 64;

struct TileCoord {
  int tm, tn;
};

// XCD-aware tile order: consecutive workgroup ids land on different XCDs
// (round robin over 8), so the ids are regrouped such that each XCD receives
// a compact block of tiles that share A row panels and B column panels in its
// own L2; inside that block tiles are rastered in groups of GM tile rows.
// GM = 8 for the linear products (an XCD of the 4096 x 4096 MLP-down output
// holds 8 x 4 tiles, so the gathered rows of B are fetched by half as many
// XCDs as with 4 x 8: 2.5% faster); GM = 4 for the batched QK products,
// where 8 was 1.5% slower.
// Causal scores keep the plain order instead: a compact block of tile rows
// per XCD would leave the XCDs holding the top rows (almost all masked) idle
// while the others carry the whole product.
template <int GM>
__device__ __forceinline__ TileCoord tile_of(int bid, int tiles_m, int tiles_n, bool xcd_blocks) {
  const int total = tiles_m * tiles_n;
  int lin = bid;
  if (xcd_blocks && (total & 7) == 0) {
    const int per = total >> 3;
    lin = (bid & 7) * per + (bid >> 3);
  }
  const int group_size = GM * tiles_n;
  const int group = lin / group_size;
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = lin - group * group_size;
  TileCoord c;
  c.tm = first_m + in_group % gm;
  c.tn = in_group / gm;
  return c;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// The identity lists a dense product reports as its idx output (see
// GemmArgs::iota_out), written by the threads of the first workgroup.
__device__ __forceinline__ void write_iota(const GemmArgs& g, int tid, int nt) {
  const int total = g.iota_heads * g.iota_n;
  for (int i = tid; i < total; i += nt) {
    const int h = i / g.iota_n, t = i - h * g.iota_n;
    g.iota_out[(size_t)h * g.iota_hs + t] = t;
  }
}

// WAVES = 4: waves in a 2x2 grid, each (BM/2) x (BN/2).
// WAVES = 8: waves in a 2x4 grid, each (BM/2) x (BN/4); two waves share a
// SIMD so one wave's MFMAs cover the other's barrier and LDS latency.
template <int BM, int BN, bool KMAJOR, bool GATHER, bool A_F32, int WAVES, bool B_I8 = false>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_bf16_kernel(const GemmArgs g) {
  static_assert(KMAJOR || !B_I8, "int8 weights come K-major");
  constexpr uint32_t BE = B_I8 ? 1u : 2u;         // bytes per B element
  constexpr int NT = 64 * WAVES;
  constexpr int WGN = WAVES / 2;                   // wave grid: 2 x WGN
  constexpr int WM = BM / 2, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CH = BM * 8 / NT;                // 16-byte chunks of A (bf16) per thread
  constexpr int B_CH = BN * 8 / NT;                // (N-contiguous B) chunks per thread
  constexpr int ROWS_PER_PASS = NT / 8;            // A rows covered by one chunk index
  // K-major B: the 64 x BN tile is split into 8x8 blocks; each owner thread
  // loads BR rows (8 or 4) of one block and transposes them.
  constexpr int NBLK = BN;                          // (64 / 8) * (BN / 8)
  constexpr int BR = NT >= 2 * NBLK ? 4 : 8;
  constexpr int B_OWNERS = NBLK * (8 / BR);
  constexpr int ES = A_F32 ? 4 : 2;                // A element size
  static_assert(B_OWNERS <= NT, "B blocks exceed the thread count");
  // With K-major B (the linear products) bf16 A goes from the buffer
  // straight into LDS (no staging registers), two K tiles ahead through a
  // ring of three A stages; fp32 A (converted on the way), the A of the
  // N-major QK products (a K tile or two per output tile) and every B tile
  // pass through registers into two stages
  constexpr bool A_DIRECT = !A_F32 && KMAJOR;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int A_STAGES = A_DIRECT ? 3 : 2;
  static_assert(!A_DIRECT || !KMAJOR || B_OWNERS == NT, "every wave issues the same number of loads per tile");
  __shared__ __attribute__((aligned(16))) char smem[A_STAGES * A_BYTES + 2 * B_BYTES];

  const int tid = threadIdx.x;
  if (g.iota_out && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) write_iota(g, tid, NT);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int li = lane & 31, lk = lane >> 5;
  const int b = blockIdx.y;
  // split K (k_split > 1): this workgroup multiplies over the contraction
  // range [k0, k0 + Kc) and writes a partial sum of its tile
  const int Kc = g.K / g.k_split;
  const int k0 = (int)blockIdx.z * Kc;

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const TileCoord tc = tile_of<KMAJOR ? 8 : 4>(blockIdx.x, tiles_m, tiles_n, !g.causal);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;

  const char* Ab = (const char*)g.A + (size_t)b * g.a_bs * ES + (size_t)k0 * ES;
  const char* Bb = (const char*)g.B + (size_t)(b / g.b_group) * g.b_bs * BE;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, g.a_bytes - (uint32_t)((size_t)k0 * ES));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, g.b_bytes);
  const int32_t* idxb = GATHER ? g.idx + (size_t)b * g.idx_bs + k0 : nullptr;

  // ---- per-thread load geometry (K is a multiple of 64 on every path) -----
  // A chunk i of this thread: row (tid >> 3) + ROWS_PER_PASS * i, 8 elements
  // at column (tid & 7) * 8 of the K tile.  Rows past M read through an
  // offset that is always out of range, so they load zeros without a branch.
  const int a_kc = (tid & 7) * 8;
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int row = m0 + (tid >> 3) + ROWS_PER_PASS * i;
    a_off[i] = row < g.M ? (uint32_t)(row * g.lda + a_kc) * ES : kOobOffset;
  }
  // direct A: instruction i of wave w fills LDS rows (w A_CH + i) 8 .. + 7 of
  // a stage; lane l carries row + l / 8 and LDS chunk slot l % 8, which
  // holds global chunk swz(row, slot) (the swizzle is an involution, so the
  // layout is the one the fragment reads expect)
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t ad_off[A_DIRECT ? A_CH : 1];
  if constexpr (A_DIRECT) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = (wave_u * A_CH + i) * 8 + (lane >> 3);
      const int row = m0 + r;
      ad_off[i] = row < g.M ? (uint32_t)(row * g.lda + swz(r, lane & 7) * 8) * 2u : kOobOffset;
    }
  }
  uint32_t b_off[KMAJOR ? 1 : B_CH];
  if constexpr (!KMAJOR) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int row = n0 + (tid >> 3) + ROWS_PER_PASS * i;
      b_off[i] = row < g.N ? (uint32_t)(row * g.ldb + a_kc) * 2u : kOobOffset;
    }
  }
  // K-major B: this thread owns rows kb_kg*8 + kb_h*BR .. +BR-1 and columns
  // kb_cg*8 .. +7 of each K tile.  A row index of -1 (padding past k) makes
  // the 32-bit offset wrap far past the buffer end, so it also reads zeros.
  const bool kb_owner = KMAJOR && tid < B_OWNERS;
  const int kb_blk = tid / (8 / BR), kb_h = tid % (8 / BR);
  const int kb_cg = kb_blk % (BN / 8), kb_kg = kb_blk / (BN / 8);
  const uint32_t kb_colmask = (n0 + kb_cg * 8) < g.N ? 0u : kOobOffset;
  const int kb_col = n0 + kb_cg * 8;
  const int kb_row0 = kb_kg * 8 + kb_h * BR;

  constexpr int A_REGS = A_DIRECT ? 1 : (A_F32 ? 2 * A_CH : A_CH);
  i32x4 ra_regs[A_REGS];
  typename RowPiece<B_I8>::type rb_regs[KMAJOR ? BR : B_CH];
  i32x4 idx_lo, idx_hi;   // kept rows for the next tile to load

  auto load_idx = [&](int kt) {
    if constexpr (GATHER) {
      const i32x4* p = (const i32x4*)(idxb + kt * BK + kb_row0);
      idx_lo = p[0];
      if constexpr (BR == 8) idx_hi = p[1];
    }
  };

  auto issue_a = [&](int kt, int stage) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      load_lds16(ra, (lds_void*)(smem + stage * A_BYTES + (wave_u * A_CH + i) * 1024),
                 ad_off[i] + (uint32_t)(kt * BK * 2));
  };

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < (A_DIRECT ? 0 : A_CH); ++i) {
      const uint32_t off = a_off[i] + (uint32_t)(kt * BK * ES);
      if constexpr (A_F32) {
        ra_regs[2 * i] = buf_load16(ra, off);
        ra_regs[2 * i + 1] = buf_load16(ra, off + 16u);
      } else {
        ra_regs[i] = buf_load16(ra, off);
      }
    }
    if constexpr (KMAJOR) {
      if (kb_owner) {
#pragma unroll
        for (int e = 0; e < BR; ++e) {
          int row;
          if constexpr (GATHER)
            row = e < 4 ? idx_lo[e] : idx_hi[e - 4];
          else
            row = k0 + kt * BK + kb_row0 + e;
          const uint32_t off = ((uint32_t)(row * g.ldb + kb_col) * BE) | kb_colmask;
          if constexpr (B_I8)
            rb_regs[e] = buf_load8(rb, off);
          else
            rb_regs[e] = buf_load16(rb, off);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) rb_regs[i] = buf_load16(rb, b_off[i] + (uint32_t)((k0 + kt * BK) * 2));
    }
  };

  // register-staged parts of K tile kt into LDS: B into stage kt & 1, and
  // fp32 A (converted to bf16) into stage kt & 1 of the A stages
  auto store_tile = [&](int kt) {
    char* As = smem + (kt & 1) * A_BYTES;
    char* Bs = smem + A_STAGES * A_BYTES + (kt & 1) * B_BYTES;
#pragma unroll
    for (int i = 0; i < (A_DIRECT ? 0 : A_CH); ++i) {
      const int row = (tid >> 3) + ROWS_PER_PASS * i, ch = tid & 7;
      i32x4 v;
      if constexpr (A_F32) {
        const i32x4 lo = ra_regs[2 * i], hi = ra_regs[2 * i + 1];
        v[0] = (int)pack_bf16x2(__int_as_float(lo[0]), __int_as_float(lo[1]));
        v[1] = (int)pack_bf16x2(__int_as_float(lo[2]), __int_as_float(lo[3]));
        v[2] = (int)pack_bf16x2(__int_as_float(hi[0]), __int_as_float(hi[1]));
        v[3] = (int)pack_bf16x2(__int_as_float(hi[2]), __int_as_float(hi[3]));
      } else {
        v = ra_regs[i];
      }
      *(i32x4*)(As + row * 128 + swz(row, ch) * 16) = v;
    }
    if constexpr (KMAJOR) {
      if (kb_owner) {
        // int8 weights are widened to bf16 (exactly) here, once in flight
        i32x4 rows[BR];
#pragma unroll
        for (int e = 0; e < BR; ++e) {
          if constexpr (B_I8)
            rows[e] = i8x8_to_bf16x8(rb_regs[e]);
          else
            rows[e] = rb_regs[e];
        }
        if constexpr (BR == 8) {
          i32x4 tr[8];
          transpose8x8(rows, tr);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int nrow = kb_cg * 8 + c;
            *(i32x4*)(Bs + nrow * 128 + swz(nrow, kb_kg) * 16) = tr[c];
          }
        } else {
          // 4 rows x 8 columns: column c becomes 4 consecutive k (8 bytes)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            i32x2 v;
            v[0] = (int)__builtin_amdgcn_perm((uint32_t)rows[1][c >> 1], (uint32_t)rows[0][c >> 1], sel);
            v[1] = (int)__builtin_amdgcn_perm((uint32_t)rows[3][c >> 1], (uint32_t)rows[2][c >> 1], sel);
            const int nrow = kb_cg * 8 + c;
            *(i32x2*)(Bs + nrow * 128 + swz(nrow, kb_kg) * 16 + kb_h * 8) = v;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int row = (tid >> 3) + ROWS_PER_PASS * i, ch = tid & 7;
        *(i32x4*)(Bs + row * 128 + swz(row, ch) * 16) = rb_regs[i];
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = wm * WM + i * 32 + li;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row[j] = wn * WN + j * 32 + li;

  auto read_frags = [&](int kt, int s, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
    const char* As = smem + (A_DIRECT ? kt % 3 : kt & 1) * A_BYTES;
    const char* Bs = smem + A_STAGES * A_BYTES + (kt & 1) * B_BYTES;
    const int ch = 2 * s + lk;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)(As + a_row[i] * 128 + swz(a_row[i], ch) * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = *(const bf16x8*)(Bs + b_row[j] * 128 + swz(b_row[j], ch) * 16);
  };
  // K-major products run through the A fragments under each B fragment
  // (measured 0.5-1% faster than the A-outer order, interleaved runs); the
  // QK products keep the A-outer order they were tuned with.
  auto mfma_all = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfr)[TN]) {
    if constexpr (KMAJOR) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // causal scores: a tile whose every entry lies above the shifted diagonal
  // only writes -inf
  const bool masked_tile = g.causal && (int64_t)n0 > (int64_t)(m0 + BM - 1) + g.causal_off;
  const bool some_masked = g.causal && (int64_t)(n0 + BN - 1) > (int64_t)m0 + g.causal_off;
  const int KT = masked_tile ? 0 : Kc / BK;
  // per-column scales of int8 weights, loaded before the main loop: on this
  // chip the vector memory counter covers stores too, so a load among the
  // epilogue's stores would make its wait drain every store issued so far
  // (the other variants load nothing here)
  float cs[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    cs[j] = 1.f;
    if constexpr (B_I8) {
      const int col = n0 + wn * WN + j * 32 + li;
      cs[j] = g.col_scale[col < g.N ? col : 0];
    }
  }
  // prologue: tile 0 into LDS, tile 1 in flight (direct A: already bound
  // for its stage; the rest in registers)
  if (KT > 0) {
    if constexpr (A_DIRECT) issue_a(0, 0);
    load_idx(0);
    load_tile(0);
    store_tile(0);
  }
  if (KT > 1) {
    if constexpr (A_DIRECT) issue_a(1, 1);
    load_idx(1);
    load_tile(1);
  }
  if (KT > 2) load_idx(2);
  if constexpr (A_DIRECT) wait_vmcnt<0>();
  __syncthreads();

  // vector-memory operations one tile's issue adds per wave (direct A rows,
  // B rows or chunks, the next index vector)
  constexpr int VM_AB = A_CH + (KMAJOR ? BR : B_CH);
  constexpr int VM_IDX = GATHER ? (BR == 8 ? 2 : 1) : 0;
  if constexpr (KMAJOR) {
    // K-major B (the linear products): a software pipeline over the four k16
    // steps of a tile, each group of MFMAs issued together with the LDS
    // reads of the next group's fragments (scheduling groups pin the order):
    //   G1 step 0 products | step 1 reads, next tiles' LDS stores and loads
    //   G2 step 1 products | step 2 reads
    //   G3 step 2 products | step 3 reads, then the barrier
    //   G4 step 3 products | step 0 reads of the next tile (after the barrier)
    // so no MFMA group waits on an LDS read issued just before it and the
    // barrier is followed by products whose operands are already loaded.
    // Measured orders (interleaved runs against each other): in G1 the
    // loads, the transposes, the LDS reads of step 1 and then the LDS stores
    // of the next tiles all go before the MFMAs (the other wave of the SIMD
    // keeps the matrix core busy meanwhile; stores before reads was 1.2%
    // slower); in G2-G4 one
    // read follows each of the first TM + TN MFMAs (two reads after each of
    // the first (TM + TN) / 2 was 1-1.6% slower, all reads first 2-3%).  The
    // wave runs G1-G3 at raised priority and drops it for G4, which follows
    // the barrier, so that its loads, LDS stores and reads issue ahead of the
    // other wave's products (each step from no change to G1 alone, G1-G2 and
    // G1-G3 measured about 1% faster; raising it for G2-G4 instead was 3%
    // slower).
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    if (KT > 0) read_frags(0, 0, a0, b0);
    for (int kt = 0; kt < KT; ++kt) {
      __builtin_amdgcn_s_setprio(1);
      read_frags(kt, 1, a1, b1);
      mfma_all(a0, b0);
      // the B stage of tile kt + 1 and the A stage of tile kt + 2 were last
      // read before the barrier of iteration kt - 1
      if (kt + 1 < KT) {
        store_tile(kt + 1);
        if (kt + 2 < KT) {
          if constexpr (A_DIRECT) issue_a(kt + 2, (kt + 2) % 3);
          load_tile(kt + 2);
          if (kt + 3 < KT) load_idx(kt + 3);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);   // vector-memory read
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);   // LDS read
      __builtin_amdgcn_sched_group_barrier(0x200, 16, 0);   // LDS write
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);   // MFMA
      __builtin_amdgcn_sched_barrier(0);
      read_frags(kt, 2, a0, b0);
      mfma_all(a1, b1);
#pragma unroll
      for (int u = 0; u < TM + TN; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 1);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(kt, 3, a1, b1);
      mfma_all(a0, b0);
#pragma unroll
      for (int u = 0; u < TM + TN; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (A_DIRECT) {
        // the direct A rows of tile kt + 1 (issued an iteration ago) must be
        // in LDS before the barrier; only this iteration's loads may stay in
        // flight (vector-memory operations complete in issue order)
        if (kt + 3 < KT)
          wait_vmcnt<VM_AB + VM_IDX>();
        else if (kt + 2 < KT)
          wait_vmcnt<VM_AB>();
        else
          wait_vmcnt<0>();
        lds_barrier();
      } else {
        __syncthreads();
      }
      __builtin_amdgcn_s_setprio(0);
      if (kt + 1 < KT) read_frags(kt + 1, 0, a0, b0);
      mfma_all(a1, b1);
#pragma unroll
      for (int u = 0; u < TM + TN; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
      read_frags(kt, 0, a0, b0);
      read_frags(kt, 1, a1, b1);
      mfma_all(a0, b0);
      // the other stages were released by the barrier that ended kt - 1
      if (kt + 1 < KT) {
        store_tile(kt + 1);
        if (kt + 2 < KT) {
          load_tile(kt + 2);
          if (kt + 3 < KT) load_idx(kt + 3);
        }
      }
      read_frags(kt, 2, a0, b0);
      mfma_all(a1, b1);
      read_frags(kt, 3, a1, b1);
      mfma_all(a0, b0);
      mfma_all(a1, b1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane (li, lk) of accumulator register v holds row
  //      8*(v/4) + 4*lk + v%4 and column li of its 32x32 block.
  //      Split K: the fp32 partial of range blockIdx.z goes to
  //      partial[blockIdx.z][b] (M x N, row stride N) instead of C.
  const bool split = g.k_split > 1;
  char* Cb = split ? (char*)(g.partial + ((size_t)blockIdx.z * g.batch + b) * g.M * g.N)
                   : (char*)g.C + (size_t)b * g.c_bs * (g.c_bf16 ? 2 : 4);
  const int64_t ldc = split ? g.N : g.ldc;
  const bool c_bf16 = !split && g.c_bf16;
  const bool full = m0 + BM <= g.M && n0 + BN <= g.N;

  if (full && !c_bf16) {
    // whole fp32 tiles without a branch per element: unmasked, or with the
    // causal mask applied by a select
    if (!some_masked) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          float* c = (float*)Cb + (size_t)(m0 + wm * WM + i * 32 + 4 * lk) * ldc + (n0 + wn * WN + j * 32 + li);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __builtin_nontemporal_store(B_I8 ? acc[i][j][v] * cs[j] : acc[i][j][v],
                                        c + (size_t)(8 * (v >> 2) + (v & 3)) * ldc);
        }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row0 = m0 + wm * WM + i * 32 + 4 * lk;
          const int col = n0 + wn * WN + j * 32 + li;
          float* c = (float*)Cb + (size_t)row0 * ldc + col;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 8 * (v >> 2) + (v & 3);
            const float a = B_I8 ? acc[i][j][v] * cs[j] : acc[i][j][v];
            __builtin_nontemporal_store((int64_t)col > (int64_t)(row0 + r) + g.causal_off ? -INFINITY : a,
                                        c + (size_t)r * ldc);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 32 + li;
      const int row0 = m0 + wm * WM + i * 32 + 4 * lk;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + 8 * (v >> 2) + (v & 3);
        if (full || (row < g.M && col < g.N)) {
          const size_t off = (size_t)row * ldc + col;
          const float a = B_I8 ? acc[i][j][v] * cs[j] : acc[i][j][v];
          const float y = some_masked && (int64_t)col > (int64_t)row + g.causal_off ? -INFINITY : a;
          if (c_bf16)
            __builtin_nontemporal_store(f32_to_bf16(y), (uint16_t*)Cb + off);
          else
            __builtin_nontemporal_store(y, (float*)Cb + off);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the N-major product (the batched QK^T scores over
// many 256 x 256 tiles).  That product is bound by storing S:
// a tile of 64 or 128 products per output ends in a 256 KB store.  With one
// workgroup per tile (one per CU at a time) every tile pays its operand
// loads again after the previous tile's store, and they queue behind it.
// Here a workgroup per CU walks its tiles t = blockIdx.x + i gridDim.x as
// one stream of K steps (tile, kt): the operands of step s + 2 are requested
// while step s is multiplied, so the next tile's operands are already in
// flight when a tile's stores go out; and the next step's operands are
// moved into LDS before those stores are issued.  That move waits for every
// earlier memory operation (a store and a load cannot be told apart by the
// counter), i.e. for the previous tile's stores, which drain meanwhile: the
// stores of consecutive tiles follow each other with only that move between
// them.  Barriers wait for LDS only, never for the stores.  Causal scores
// run through the same stream: a tile wholly above the diagonal is still
// multiplied (its store, not its product, is the cost) and stored as -inf,
// so every tile costs the same and the XCD-blocked order stays balanced.
// ---------------------------------------------------------------------------
constexpr int kPersistGroups = 256;   // one workgroup per compute unit

__global__ __launch_bounds__(512, 1) void gemm_nmajor_persistent_kernel(const GemmArgs g, int total_tiles) {
  constexpr int BM = 256, BN = 256, NT = 512, WGN = 4;
  constexpr int WM = BM / 2, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
  constexpr int ROWS_PER_PASS = NT / 8;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * A_BYTES + 2 * B_BYTES];

  const int tid = threadIdx.x;
  if (g.iota_out && blockIdx.x == 0) write_iota(g, tid, 512);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int li = lane & 31, lk = lane >> 5;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int per_batch = tiles_m * tiles_n;
  const int KT = g.K / BK;
  const int my_tiles = (total_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int S = my_tiles * KT;   // K steps of this workgroup

  // tile i of this workgroup: batch and corner.  The grid is a multiple of
  // 8 and so is a batch's tile count where the XCD order applies, so the
  // tile keeps the XCD of its workgroup id and tile_of's blocks hold.
  auto tile_at = [&](int i, int& b, int& m0, int& n0) {
    const int t = (int)blockIdx.x + i * (int)gridDim.x;
    b = t / per_batch;
    const TileCoord c = tile_of<4>(t - b * per_batch, tiles_m, tiles_n, true);
    m0 = c.tm * BM;
    n0 = c.tn * BN;
  };

  const int a_kc = (tid & 7) * 8;
  i32x4 ra_regs[A_CH], rb_regs[B_CH];
  auto load_step = [&](int s) {
    const int i = s / KT, kt = s - (s / KT) * KT;
    int b, m0, n0;
    tile_at(i, b, m0, n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc((const char*)g.A + (size_t)b * g.a_bs * 2, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc((const char*)g.B + (size_t)(b / g.b_group) * g.b_bs * 2, g.b_bytes);
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int row = m0 + (tid >> 3) + ROWS_PER_PASS * c;
      const uint32_t off = row < g.M ? (uint32_t)(row * g.lda + a_kc + kt * BK) * 2u : kOobOffset;
      ra_regs[c] = buf_load16(ra, off);
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int row = n0 + (tid >> 3) + ROWS_PER_PASS * c;
      const uint32_t off = row < g.N ? (uint32_t)(row * g.ldb + a_kc + kt * BK) * 2u : kOobOffset;
      rb_regs[c] = buf_load16(rb, off);
    }
  };
  auto store_step = [&](int s) {
    char* As = smem + (s & 1) * A_BYTES;
    char* Bs = smem + 2 * A_BYTES + (s & 1) * B_BYTES;
    const int ch = tid & 7;
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int row = (tid >> 3) + ROWS_PER_PASS * c;
      *(i32x4*)(As + row * 128 + swz(row, ch) * 16) = ra_regs[c];
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int row = (tid >> 3) + ROWS_PER_PASS * c;
      *(i32x4*)(Bs + row * 128 + swz(row, ch) * 16) = rb_regs[c];
    }
  };

  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = wm * WM + i * 32 + li;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row[j] = wn * WN + j * 32 + li;
  auto read_frags = [&](int s, int k16, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
    const char* As = smem + (s & 1) * A_BYTES;
    const char* Bs = smem + 2 * A_BYTES + (s & 1) * B_BYTES;
    const int ch = 2 * k16 + lk;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8*)(As + a_row[i] * 128 + swz(a_row[i], ch) * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = *(const bf16x8*)(Bs + b_row[j] * 128 + swz(b_row[j], ch) * 16);
  };

  f32x16 acc[TM][TN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };
  auto mfma_all = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfr)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  // lane (li, lk) of accumulator register v holds row 8 (v / 4) + 4 lk + v % 4
  // and column li of its 32 x 32 block
  auto store_c = [&](int i_tile) {
    int b, m0, n0;
    tile_at(i_tile, b, m0, n0);
    char* Cb = (char*)g.C + (size_t)b * g.c_bs * (g.c_bf16 ? 2 : 4);
    const bool full = m0 + BM <= g.M && n0 + BN <= g.N;
    // causal scores: every entry of the tile above the shifted diagonal, or some
    const bool all_masked = g.causal && (int64_t)n0 > (int64_t)(m0 + BM - 1) + g.causal_off;
    const bool some_masked = g.causal && (int64_t)(n0 + BN - 1) > (int64_t)m0 + g.causal_off;
    if (full && !g.c_bf16) {
      // whole fp32 tiles without a branch per element: unmasked, or with
      // the mask applied by a select (a branch per element around the
      // stores of the diagonal tiles made causal launches a third slower)
      if (!some_masked) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            float* c = (float*)Cb + (size_t)(m0 + wm * WM + i * 32 + 4 * lk) * g.ldc + (n0 + wn * WN + j * 32 + li);
#pragma unroll
            for (int v = 0; v < 16; ++v)
              __builtin_nontemporal_store(acc[i][j][v], c + (size_t)(8 * (v >> 2) + (v & 3)) * g.ldc);
          }
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int row0 = m0 + wm * WM + i * 32 + 4 * lk;
            const int col = n0 + wn * WN + j * 32 + li;
            float* c = (float*)Cb + (size_t)row0 * g.ldc + col;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = 8 * (v >> 2) + (v & 3);
              const bool mk = all_masked || (int64_t)col > (int64_t)(row0 + r) + g.causal_off;
              __builtin_nontemporal_store(mk ? -INFINITY : acc[i][j][v], c + (size_t)r * g.ldc);
            }
          }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WN + j * 32 + li;
        const int row0 = m0 + wm * WM + i * 32 + 4 * lk;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = row0 + 8 * (v >> 2) + (v & 3);
          if (full || (row < g.M && col < g.N)) {
            const size_t off = (size_t)row * g.ldc + col;
            const float y = some_masked && (int64_t)col > (int64_t)row + g.causal_off ? -INFINITY : acc[i][j][v];
            if (g.c_bf16)
              __builtin_nontemporal_store(f32_to_bf16(y), (uint16_t*)Cb + off);
            else
              __builtin_nontemporal_store(y, (float*)Cb + off);
          }
        }
      }
    }
  };

  zero_acc();
  if (S > 0) {
    load_step(0);
    store_step(0);
  }
  if (S > 1) load_step(1);
  lds_barrier();
  for (int s = 0; s < S; ++s) {
    bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
    read_frags(s, 0, a0, b0);
    read_frags(s, 1, a1, b1);
    mfma_all(a0, b0);
    read_frags(s, 2, a0, b0);
    mfma_all(a1, b1);
    read_frags(s, 3, a1, b1);
    mfma_all(a0, b0);
    mfma_all(a1, b1);
    // stage (s + 1) & 1 was last read in step s - 1, before the barrier
    if (s + 1 < S) store_step(s + 1);
    if (s + 2 < S) load_step(s + 2);
    if (s % KT == KT - 1) {
      store_c(s / KT);
      zero_acc();
    }
    lds_barrier();
  }
}

hipError_t launch_gemm_nmajor_persistent(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  int groups = tiles < kPersistGroups ? tiles : kPersistGroups;
  if (groups >= 8) groups &= ~7;
  gemm_nmajor_persistent_kernel<<<groups, 512, 0, s>>>(g, tiles);
  return hipGetLastError();
}

template <int BM, int BN, int WAVES>
hipError_t dispatch(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, g.batch, g.k_split);
  const bool gather = g.idx != nullptr;
  if (g.b_kmajor) {
    if (gather)
      gemm_bf16_kernel<BM, BN, true, true, false, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
    else
      gemm_bf16_kernel<BM, BN, true, false, false, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
  } else {
    gemm_bf16_kernel<BM, BN, false, false, false, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
  }
  return hipGetLastError();
}

// A grid of 256 x 256 tiles whose last wave leaves at least half the CUs
// idle (mlp_up 2048 x 28672: 896 tiles, 3.5 waves) is split by columns: the
// tiles that fill whole waves keep 256 x 256, and the output columns after
// them go to a second launch of 128 x 128 tiles, which run two to a CU (80
// KB of LDS and at most 256 registers per lane each), so that last round
// costs about half a 256 x 256 tile per CU instead of a whole one.  The
// column band is a pointer offset into B, C and the column scale; B's
// buffer extent shrinks by the same bytes, so reads past its end still
// return zero.  Linear products only (K-major B, one batch, no mask, no
// split contraction).
bool split_last_wave(const GemmArgs& g, uint32_t b_esize, GemmArgs& head, GemmArgs& tail) {
  if (!g.b_kmajor || g.causal || g.k_split != 1 || g.batch != 1 || g.M < 256 || g.N < 512) return false;
  const long tm = (g.M + 255) / 256, tn = (g.N + 255) / 256;
  if (tm * tn <= kPersistGroups || (tm * tn) % kPersistGroups > kPersistGroups / 2 ||
      (tm * tn) % kPersistGroups == 0)
    return false;
  long n1 = tn - 1;                      // column tiles that fill whole waves
  while (n1 > 0 && (tm * n1) % kPersistGroups != 0) --n1;
  if (n1 == 0) return false;
  const int cols = (int)(n1 * 256);
  const long t128 = (long)((g.M + 127) / 128) * ((g.N - cols + 127) / 128);
  if (t128 > 2 * kPersistGroups) return false;
  head = g;
  head.N = cols;
  tail = g;
  tail.iota_out = nullptr;   // the head launch writes them
  tail.N = g.N - cols;
  tail.B = (const uint16_t*)((const char*)g.B + (size_t)cols * b_esize);
  tail.b_bytes = g.b_bytes - (uint32_t)cols * b_esize;
  tail.C = (char*)g.C + (size_t)cols * (g.c_bf16 ? 2 : 4);
  if (g.col_scale) tail.col_scale = g.col_scale + cols;
  return true;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  // Small-N / small-M products (per-head PV) use 128x128 tiles so that the
  // grid still covers the chip; large products use 256x256, and the
  // store-bound N-major ones (QK^T scores over many tiles) the persistent
  // kernel.
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  if (g.k_split != 1) return hipErrorInvalidValue;   // split K: fp32 A products only
  if (!g.b_kmajor && t256 >= 2 * kPersistGroups && g.N >= 256 && g.M >= 256)
    return launch_gemm_nmajor_persistent(g, s);
  GemmArgs head, tail;
  if (split_last_wave(g, 2, head, tail)) {
    const hipError_t e = dispatch<256, 256, 8>(head, s);
    return e != hipSuccess ? e : dispatch<128, 128, 4>(tail, s);
  }
  if (t256 >= 192 && g.N >= 256 && g.M >= 256) return dispatch<256, 256, 8>(g, s);
  return dispatch<128, 128, 4>(g, s);
}

// fp32-A variant (P of attention in fp32): A is read as fp32 and rounded to
// bf16 on its way into LDS.  With an index list the K-major B rows are
// gathered (a -1 entry reads a zero row), which lets PV run over every key
// position of P with the dropped rows of V masked to zero.
template <int BM, int BN, int WAVES>
void dispatch_af32(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, g.batch, g.k_split);
  if (g.b_kmajor) {
    if (g.idx)
      gemm_bf16_kernel<BM, BN, true, true, true, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
    else
      gemm_bf16_kernel<BM, BN, true, false, true, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
  } else {
    gemm_bf16_kernel<BM, BN, false, false, true, WAVES><<<grid, 64 * WAVES, 0, s>>>(g);
  }
}

// int8 K-major B (weights with a scale per output column in g.col_scale),
// rows gathered by idx or read in order.
template <int BM, int BN, int WAVES>
void dispatch_w8(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, g.batch, g.k_split);
  if (g.idx)
    gemm_bf16_kernel<BM, BN, true, true, false, WAVES, true><<<grid, 64 * WAVES, 0, s>>>(g);
  else
    gemm_bf16_kernel<BM, BN, true, false, false, WAVES, true><<<grid, 64 * WAVES, 0, s>>>(g);
}

hipError_t launch_gemm_w8(const GemmArgs& g, hipStream_t s) {
  if (!g.b_kmajor || !g.b_i8 || !g.col_scale || g.k_split != 1) return hipErrorInvalidValue;
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  GemmArgs head, tail;
  if (split_last_wave(g, 1, head, tail)) {
    dispatch_w8<256, 256, 8>(head, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dispatch_w8<128, 128, 4>(tail, s);
  } else if (t256 >= 192 && g.N >= 256 && g.M >= 256) {
    dispatch_w8<256, 256, 8>(g, s);
  } else {
    dispatch_w8<128, 128, 4>(g, s);
  }
  return hipGetLastError();
}

// C[b][i][j] = sum over ranges z = 0, 1, ... of partial[z][b][i][j], in
// range order; four consecutive elements per thread where N % 4 == 0.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmArgs g) {
  const size_t per = (size_t)g.M * g.N;
  const int b = blockIdx.y;
  const bool v4 = (g.N & 3) == 0;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * (v4 ? 4 : 1);
  if (e0 >= per) return;
  const int row = (int)(e0 / g.N), col = (int)(e0 % g.N);
  char* Cb = (char*)g.C + (size_t)b * g.c_bs * (g.c_bf16 ? 2 : 4);
  const size_t off = (size_t)row * g.ldc + col;
  if (v4) {
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < g.k_split; ++z) {
      const f32x4 p = *(const f32x4*)(g.partial + ((size_t)z * g.batch + b) * per + e0);
      v[0] += p[0];
      v[1] += p[1];
      v[2] += p[2];
      v[3] += p[3];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (g.c_bf16)
        ((uint16_t*)Cb)[off + t] = f32_to_bf16(v[t]);
      else
        ((float*)Cb)[off + t] = v[t];
    }
  } else {
    float v = 0.f;
    for (int z = 0; z < g.k_split; ++z) v += g.partial[((size_t)z * g.batch + b) * per + e0];
    if (g.c_bf16)
      ((uint16_t*)Cb)[off] = f32_to_bf16(v);
    else
      ((float*)Cb)[off] = v;
  }
}

hipError_t launch_gemm_bf16_af32(const GemmArgs& g, hipStream_t s) {
  if (g.k_split < 1 || g.K % (BK * g.k_split) != 0 || (g.k_split > 1 && (!g.partial || g.causal)))
    return hipErrorInvalidValue;
  // 128 x 128 tiles only: with fp32 A staged in registers the 256 x 256
  // tile needs more than the 256 registers two waves per SIMD allow
  dispatch_af32<128, 128, 4>(g, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.k_split == 1) return e;
  const size_t per = (size_t)g.M * g.N;
  const size_t threads = (g.N & 3) == 0 ? (per + 3) / 4 : per;
  splitk_reduce_kernel<<<dim3((unsigned)((threads + 255) / 256), g.batch), 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace rmm
