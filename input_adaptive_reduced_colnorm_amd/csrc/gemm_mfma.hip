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
// Tiling: BM x BN x 64 per workgroup of 4 waves (2 x 2), each wave owning a
// (BM/2) x (BN/2) block of 32x32 accumulators fed by v_mfma_f32_32x32x16_bf16.
// Global -> register prefetch of the next K tile overlaps the MFMAs of the
// current one; LDS is double buffered with one barrier per K tile.  LDS rows
// are 128 bytes (64 bf16 along K) with an XOR swizzle of the 16-byte chunks.
// B tiles that are K-major in memory (weights, V) are transposed in
// registers in 8x8 blocks (v_perm) before they reach LDS.

#include "rmm_device.h"
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;

struct TileCoord {
  int tm, tn;
};

// XCD-aware tile order: consecutive workgroup ids land on different XCDs
// (round robin over 8), so the ids are regrouped such that each XCD receives
// a compact block of tiles that share A row panels and B column panels in its
// own L2; inside that block tiles are rastered in groups of 4 tile rows.
__device__ __forceinline__ TileCoord tile_of(int bid, int tiles_m, int tiles_n) {
  const int total = tiles_m * tiles_n;
  int lin = bid;
  if ((total & 7) == 0) {
    const int per = total >> 3;
    lin = (bid & 7) * per + (bid >> 3);
  }
  constexpr int GM = 4;
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

// 8x8 transpose of bf16 held as 8 rows x 4 dwords: out[c] holds column c
// (8 values along the former rows) as 4 dwords.
__device__ __forceinline__ void transpose8x8(const i32x4 (&in)[8], i32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t lo = (uint32_t)in[2 * p][c >> 1];
      uint32_t hi = (uint32_t)in[2 * p + 1][c >> 1];
      out[c][p] = (int)__builtin_amdgcn_perm(hi, lo, sel);
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <int BM, int BN, bool KMAJOR, bool GATHER, bool A_F32, int NBUF>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CH = BM * 8 / kThreads;          // 16-byte chunks of A per thread
  constexpr int B_CH = BN * 8 / kThreads;          // (N-contiguous B) chunks per thread
  constexpr int B_BLK_THREADS = BN;                // (K-major B) threads owning one 8x8 block
  constexpr int STAGE = (BM + BN) * 128;           // bytes per LDS stage
  __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;
  const int b = blockIdx.y;

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;

  const char* Ab = (const char*)g.A + (size_t)b * g.a_bs * (A_F32 ? 4 : 2);
  const char* Bb = (const char*)g.B + (size_t)(b / g.b_group) * g.b_bs * 2;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, g.b_bytes);
  const int32_t* idxb = GATHER ? g.idx + (size_t)b * g.idx_bs : nullptr;

  // ---- per-thread load geometry -------------------------------------------
  uint32_t a_row_off[A_CH];
  int a_kc[A_CH];
  bool a_row_ok[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = i * kThreads + tid;
    const int row = c >> 3;
    a_kc[i] = (c & 7) * 8;
    a_row_ok[i] = (m0 + row) < g.M;
    a_row_off[i] = (uint32_t)((int64_t)(m0 + row) * g.lda * (A_F32 ? 4 : 2));
  }
  uint32_t b_row_off[KMAJOR ? 1 : B_CH];
  int b_kc[KMAJOR ? 1 : B_CH];
  bool b_row_ok[KMAJOR ? 1 : B_CH];
  if constexpr (!KMAJOR) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = i * kThreads + tid;
      const int row = c >> 3;
      b_kc[i] = (c & 7) * 8;
      b_row_ok[i] = (n0 + row) < g.N;
      b_row_off[i] = (uint32_t)((int64_t)(n0 + row) * g.ldb * 2);
    }
  }
  const bool kb_owner = KMAJOR && tid < B_BLK_THREADS;
  const int kb_cg = tid % (BN / 8), kb_kg = tid / (BN / 8);
  const bool kb_col_ok = (n0 + kb_cg * 8) < g.N;

  constexpr int A_REGS = A_F32 ? 2 * A_CH : A_CH;
  i32x4 ra_regs[A_REGS];
  i32x4 rb_regs[KMAJOR ? 8 : B_CH];
  int rows_next[8];  // gathered B rows for the tile being loaded

  auto load_rows = [&](int kt, int (&rows)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = kt * BK + kb_kg * 8 + e;
      if constexpr (GATHER) {
        rows[e] = t < g.k_valid ? idxb[t] : -1;
      } else {
        rows[e] = t < g.K ? t : -1;
      }
    }
  };

  auto load_tile = [&](int kt, const int (&rows)[8]) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int gk = kt * BK + a_kc[i];
      const bool ok = a_row_ok[i] && gk < g.K;
      if constexpr (A_F32) {
        const uint32_t off = ok ? a_row_off[i] + (uint32_t)gk * 4u : kOobOffset;
        ra_regs[2 * i] = buf_load16(ra, off);
        ra_regs[2 * i + 1] = buf_load16(ra, ok ? off + 16u : kOobOffset);
      } else {
        const uint32_t off = ok ? a_row_off[i] + (uint32_t)gk * 2u : kOobOffset;
        ra_regs[i] = buf_load16(ra, off);
      }
    }
    if constexpr (KMAJOR) {
      if (kb_owner) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = rows[e] >= 0 && kb_col_ok;
          const uint32_t off =
              ok ? (uint32_t)((int64_t)rows[e] * g.ldb * 2 + (int64_t)(n0 + kb_cg * 8) * 2) : kOobOffset;
          rb_regs[e] = buf_load16(rb, off);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int gk = kt * BK + b_kc[i];
        const bool ok = b_row_ok[i] && gk < g.K;
        rb_regs[i] = buf_load16(rb, ok ? b_row_off[i] + (uint32_t)gk * 2u : kOobOffset);
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* As = smem + buf * STAGE;
    char* Bs = As + BM * 128;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = i * kThreads + tid;
      const int row = c >> 3, ch = c & 7;
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
        i32x4 tr[8];
        transpose8x8(rb_regs, tr);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int nrow = kb_cg * 8 + c;
          *(i32x4*)(Bs + nrow * 128 + swz(nrow, kb_kg) * 16) = tr[c];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = i * kThreads + tid;
        const int row = c >> 3, ch = c & 7;
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

  auto compute = [&](int buf) {
    const char* As = smem + buf * STAGE;
    const char* Bs = As + BM * 128;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 af[TM], bfr[TN];
      const int ch = 2 * s + lk;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + li;
        af[i] = *(const bf16x8*)(As + row * 128 + swz(row, ch) * 16);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int nrow = wn * WN + j * 32 + li;
        bfr[j] = *(const bf16x8*)(Bs + nrow * 128 + swz(nrow, ch) * 16);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int KT = (g.K + BK - 1) / BK;
  int rows_cur[8];
  if constexpr (KMAJOR) load_rows(0, rows_cur);
  load_tile(0, rows_cur);
  if constexpr (KMAJOR) {
    if (KT > 1) load_rows(1, rows_next);
  }
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = NBUF == 1 ? 0 : (kt & 1);
    const bool more = kt + 1 < KT;
    int rows_after[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rows_after[e] = -1;
    if (more) {
      load_tile(kt + 1, rows_next);
      if constexpr (KMAJOR) {
        if (kt + 2 < KT) load_rows(kt + 2, rows_after);
      }
    }
    compute(cur);
    if (more) {
      if (NBUF == 1) __syncthreads();
      store_tile(NBUF == 1 ? 0 : (cur ^ 1));
      if constexpr (KMAJOR) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rows_next[e] = rows_after[e];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane (li, lk) of accumulator register v holds row
  //      8*(v/4) + 4*lk + v%4 and column li of its 32x32 block.
  char* Cb = (char*)g.C + (size_t)b * g.c_bs * (g.c_bf16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 32 + li;
      if (col >= g.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
        if (row < g.M) {
          const size_t off = (size_t)row * g.ldc + col;
          if (g.c_bf16)
            __builtin_nontemporal_store(f32_to_bf16(acc[i][j][v]), (uint16_t*)Cb + off);
          else
            __builtin_nontemporal_store(acc[i][j][v], (float*)Cb + off);
        }
      }
    }
  }
}

template <int BM, int BN, int NBUF>
hipError_t dispatch(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, g.batch);
  const bool gather = g.idx != nullptr;
  if (g.b_kmajor) {
    if (gather)
      gemm_bf16_kernel<BM, BN, true, true, false, NBUF><<<grid, kThreads, 0, s>>>(g);
    else
      gemm_bf16_kernel<BM, BN, true, false, false, NBUF><<<grid, kThreads, 0, s>>>(g);
  } else {
    gemm_bf16_kernel<BM, BN, false, false, false, NBUF><<<grid, kThreads, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  // Small-N / small-M products (per-head PV) use 128x128 tiles so that the
  // grid still covers the chip; large products use 256x256.
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  const int KT = (g.K + BK - 1) / BK;
  if (t256 >= 192 && g.N >= 256 && g.M >= 256) {
    if (KT == 1) return dispatch<256, 256, 1>(g, s);
    return dispatch<256, 256, 2>(g, s);
  }
  if (KT == 1) return dispatch<128, 128, 1>(g, s);
  return dispatch<128, 128, 2>(g, s);
}

// Dense fp32-A variant (P of attention in fp32, rho = 1): A is read as fp32
// and rounded to bf16 on its way into LDS.
hipError_t launch_gemm_bf16_af32(const GemmArgs& g, hipStream_t s) {
  const int KT = (g.K + BK - 1) / BK;
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  if (t256 >= 192 && g.N >= 256 && g.M >= 256) {
    const int tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
    dim3 grid(tiles, g.batch);
    if (g.b_kmajor)
      gemm_bf16_kernel<256, 256, true, false, true, 2><<<grid, kThreads, 0, s>>>(g);
    else
      gemm_bf16_kernel<256, 256, false, false, true, 2><<<grid, kThreads, 0, s>>>(g);
  } else {
    const int tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    dim3 grid(tiles, g.batch);
    if (g.b_kmajor)
      gemm_bf16_kernel<128, 128, true, false, true, 2><<<grid, kThreads, 0, s>>>(g);
    else
      gemm_bf16_kernel<128, 128, false, false, true, 2><<<grid, kThreads, 0, s>>>(g);
  }
  (void)KT;
  return hipGetLastError();
}

}  // namespace rmm
