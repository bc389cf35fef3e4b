// C ABI of librmm: argument checks, path planning, workspace carving and
// kernel dispatch.  Every check runs before the first launch.

#include <algorithm>
#include <math.h>
#include <mutex>
#include <string.h>

#include "rmm.h"
#include "rmm_internal.h"

using namespace rmm;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxOperandBytes = ((int64_t)1 << 31) - 1;
constexpr int kDecodeRows = 16;
constexpr int kKTile = 64;

bool rho_ok(double rho) { return isfinite(rho) && rho > 0.0 && rho <= 1.0; }

int64_t k_of(double rho, int64_t d) {
  if (!rho_ok(rho) || d < 1 || d >= kMaxDim) return -1;
  const double x = rho * (double)d;
  const double r = nearbyint(x);
  int64_t k;
  if (fabs(x - r) <= 1e-9 * (x > 1.0 ? x : 1.0))
    k = (int64_t)r;
  else
    k = (int64_t)ceil(x);
  if (k < 1) k = 1;
  if (k > d) k = d;
  return k;
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
bool dim_ok(int64_t x) { return x >= 1 && x < kMaxDim; }
bool dtype_ok(int dt) { return dt == RMM_FP32 || dt == RMM_BF16; }
size_t elt_size(int dt) { return dt == RMM_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Byte span [lo, hi) touched by a strided 3-D operand.
struct Span {
  uintptr_t lo, hi;
};
Span span3(const void* p, int64_t heads, int64_t hs, int64_t rows, int64_t rs, int64_t cols, size_t elt) {
  const int64_t last = (heads - 1) * hs + (rows - 1) * rs + (cols - 1);
  Span s;
  s.lo = (uintptr_t)p;
  s.hi = (uintptr_t)p + (uintptr_t)((last + 1) * (int64_t)elt);
  return s;
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Workspace carving: 256-byte aligned regions laid out in call order.
struct Carve {
  size_t used = 0;
  size_t take(size_t bytes) {
    const size_t off = used;
    used += (bytes + 255) / 256 * 256;
    return off;
  }
};

hipError_t clear_error() { return hipGetLastError(); }

#define RMM_LAUNCH(expr)                           \
  do {                                             \
    if ((expr) != hipSuccess) return RMM_ERR_HIP;  \
  } while (0)

// ---------------------------------------------------------------------------
// selection plan (shared by select / matmul / qk / pv)
// ---------------------------------------------------------------------------
struct SelPlan {
  int splits = 0;
  size_t off_partial = 0, off_gkeys = 0;
  bool gkeys = false;
};

void plan_select(Carve& cv, SelPlan& sp, int heads, int64_t n, int64_t d, bool bf16) {
  sp.splits = colnorm_splits(heads, (int)n, (int)d, bf16);
  sp.off_partial = cv.take((size_t)heads * sp.splits * d * 4);
  sp.gkeys = d > topk_lds_capacity();
  if (sp.gkeys) sp.off_gkeys = cv.take((size_t)heads * d * 4);
}

// Records stage event i when the caller asked for stage timing.
struct Marks {
  void* const* ev;
  hipStream_t s;
  hipError_t mark(int i) const { return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; }
};
hipError_t mark_of(const Marks* mk, int i) { return mk->mark(i); }

hipError_t run_select(const SelPlan& sp, char* ws, const void* A, bool bf16, int64_t hs, int64_t lda, int heads,
                      int64_t n, int64_t d, int64_t k, int32_t* idx, int64_t idx_hs, float* scores, hipStream_t s,
                      const Marks* mk = nullptr, int32_t* pad = nullptr, int64_t k_pad = 0) {
  float* partial = (float*)(ws + sp.off_partial);
  hipError_t e = launch_colnorm(A, bf16, hs, lda, heads, (int)n, (int)d, sp.splits, partial, s);
  if (e != hipSuccess) return e;
  if (mk && (e = mark_of(mk, 1)) != hipSuccess) return e;
  return launch_topk(partial, heads, sp.splits, (int)d, (int)k, idx, idx_hs, pad, k_pad, (int)k_pad, scores, d,
                     sp.gkeys ? (uint32_t*)(ws + sp.off_gkeys) : nullptr, s);
}

// Energies, then the selection and the gather of the kept columns in one
// launch (single bf16 matrix, shapes that select_pack_fits accepts).  Stage
// events 2 and 3 both close the fused launch.
hipError_t run_select_pack(const SelPlan& sp, char* ws, const void* A, int64_t lda, int64_t n, int64_t d, int64_t k,
                           int64_t k_pad, int32_t* idx, int32_t* ipad, uint16_t* pk, hipStream_t s, const Marks& mk) {
  float* partial = (float*)(ws + sp.off_partial);
  hipError_t e = launch_colnorm(A, true, 0, lda, 1, (int)n, (int)d, sp.splits, partial, s);
  if (e == hipSuccess) e = mk.mark(1);
  if (e == hipSuccess)
    e = launch_select_pack(partial, sp.splits, (const uint16_t*)A, lda, (int)n, (int)d, (int)k, (int)k_pad, idx, ipad,
                           pk, s);
  if (e == hipSuccess) e = mk.mark(2);
  if (e == hipSuccess) e = mk.mark(3);
  return e;
}

// ---------------------------------------------------------------------------
// matmul plan
// ---------------------------------------------------------------------------
enum class MatPath { kSimt, kDecode, kMfmaDirect, kMfmaPacked };

struct MatPlan {
  MatPath path;
  int64_t k = 0, k_pad = 0;
  bool all = false;
  SelPlan sel;
  bool use_sel = false;
  size_t off_pack = 0, off_ipad = 0, off_part = 0, off_dkeys = 0;
  int gemv_splits = 1;
  size_t total = 0;
};

MatPlan plan_matmul(int64_t n, int64_t d, int64_t m, int64_t lda, int64_t ldb, int dtype, double rho,
                    bool a_ptr_ok, bool b_ptr_ok) {
  MatPlan p;
  Carve cv;
  p.k = k_of(rho, d);
  p.all = p.k == d;
  p.k_pad = round_up(p.k, kKTile);
  const bool bf16 = dtype == RMM_BF16;
  const bool b_vec = bf16 && b_ptr_ok && ldb % 8 == 0 && m % 8 == 0;
  if (!bf16 || !b_vec) {
    p.path = MatPath::kSimt;
    if (!p.all) {
      plan_select(cv, p.sel, 1, n, d, bf16);
      p.use_sel = true;
    }
  } else if (n <= kDecodeRows) {
    p.path = MatPath::kDecode;
    if (!p.all && d > topk_lds_capacity()) p.off_dkeys = cv.take((size_t)d * 4);
    // a GEMV that ranks A itself slices the d source rows of B, otherwise
    // the k rows of the list
    const bool rank = !p.all && d <= gemv_select_max_d();
    p.gemv_splits = gemv_splits((int)(rank ? d : p.k), (int)m);
    if (p.gemv_splits > 1) p.off_part = cv.take((size_t)p.gemv_splits * n * m * 4);
  } else {
    const bool a_direct = p.all && a_ptr_ok && lda % 8 == 0 && d % kKTile == 0;
    if (a_direct) {
      p.path = MatPath::kMfmaDirect;
    } else {
      p.path = MatPath::kMfmaPacked;
      if (!p.all) {
        plan_select(cv, p.sel, 1, n, d, true);
        p.use_sel = true;
      }
      p.off_ipad = cv.take((size_t)p.k_pad * 4);
      p.off_pack = cv.take((size_t)n * p.k_pad * 2);
    }
  }
  p.total = cv.used;
  return p;
}

}  // namespace

extern "C" {

int64_t rmm_k(double rho, int64_t d) { return k_of(rho, d); }

const char* rmm_status_str(int status) {
  switch (status) {
    case RMM_OK: return "RMM_OK";
    case RMM_ERR_NULL: return "RMM_ERR_NULL: a required pointer is NULL";
    case RMM_ERR_RHO: return "RMM_ERR_RHO: rho must be finite and in (0, 1]";
    case RMM_ERR_SHAPE: return "RMM_ERR_SHAPE: invalid dimension, stride or size";
    case RMM_ERR_DTYPE: return "RMM_ERR_DTYPE: unsupported dtype";
    case RMM_ERR_ALIGN: return "RMM_ERR_ALIGN: pointer not aligned to its element size";
    case RMM_ERR_WORKSPACE: return "RMM_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case RMM_ERR_HIP: return "RMM_ERR_HIP: a kernel launch failed";
    case RMM_ERR_ALIAS: return "RMM_ERR_ALIAS: an output overlaps another argument";
    default: return "unknown rmm status";
  }
}

// ------------------------------- select ------------------------------------

size_t rmm_select_workspace(int64_t n, int64_t d, int dtype) {
  if (!dim_ok(n) || !dim_ok(d) || !dtype_ok(dtype)) return 0;
  Carve cv;
  SelPlan sp;
  plan_select(cv, sp, 1, n, d, dtype == RMM_BF16);
  return cv.used;
}

namespace {

rmm_status_t select_impl(const void* A, int dtype, int64_t n, int64_t d, int64_t lda, double rho, int32_t* idx,
                         float* scores, float* retained, void* workspace, size_t workspace_bytes, void* stream) {
  if (!A || !idx) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (!dtype_ok(dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(n) || !dim_ok(d) || lda < d || lda >= kMaxDim) return RMM_ERR_SHAPE;
  const size_t elt = elt_size(dtype);
  if (!aligned(A, elt) || !aligned(idx, 4) || (scores && !aligned(scores, 4))) return RMM_ERR_ALIGN;
  if (retained && !aligned(retained, 4)) return RMM_ERR_ALIGN;
  const int64_t k = k_of(rho, d);
  const bool all = k == d;
  Carve cv;
  SelPlan sp;
  const bool need_sel = !all || scores != nullptr || retained != nullptr;
  if (need_sel) plan_select(cv, sp, 1, n, d, dtype == RMM_BF16);
  if (cv.used > 0 && (!workspace || workspace_bytes < cv.used || !aligned(workspace, 256))) return RMM_ERR_WORKSPACE;
  const Span sa = span3(A, 1, 0, n, lda, d, elt);
  const Span si = span3(idx, 1, 0, 1, k, k, 4);
  if (overlap(si, sa)) return RMM_ERR_ALIAS;
  if (scores) {
    const Span ss = span3(scores, 1, 0, 1, d, d, 4);
    if (overlap(ss, sa) || overlap(ss, si)) return RMM_ERR_ALIAS;
  }
  if (retained) {
    const Span sr = span3(retained, 1, 0, 1, 1, 1, 4);
    if (overlap(sr, sa) || overlap(sr, si) || (scores && overlap(sr, span3(scores, 1, 0, 1, d, d, 4))))
      return RMM_ERR_ALIAS;
  }
  if (cv.used > 0) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)cv.used, (int64_t)cv.used, 1);
    if (overlap(sw, sa) || overlap(sw, si) || (scores && overlap(sw, span3(scores, 1, 0, 1, d, d, 4))))
      return RMM_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  clear_error();
  if (need_sel) {
    float* partial = (float*)((char*)workspace + sp.off_partial);
    RMM_LAUNCH(launch_colnorm(A, dtype == RMM_BF16, 0, lda, 1, (int)n, (int)d, sp.splits, partial, s));
    RMM_LAUNCH(launch_topk(partial, 1, sp.splits, (int)d, (int)k, idx, k, nullptr, 0, 0, scores, d,
                           sp.gkeys ? (uint32_t*)((char*)workspace + sp.off_gkeys) : nullptr, s, nullptr, 0,
                           retained));
  } else {
    RMM_LAUNCH(launch_iota(idx, k, 1, (int)d, nullptr, 0, 0, s));
  }
  return RMM_OK;
}

}  // namespace

rmm_status_t rmm_select(const void* A, int dtype, int64_t n, int64_t d, int64_t lda, double rho, int32_t* idx,
                        float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(A, dtype, n, d, lda, rho, idx, scores, nullptr, workspace, workspace_bytes, stream);
}

rmm_status_t rmm_select_retained(const void* A, int dtype, int64_t n, int64_t d, int64_t lda, double rho,
                                 int32_t* idx, float* scores, float* retained, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!retained) return RMM_ERR_NULL;
  return select_impl(A, dtype, n, d, lda, rho, idx, scores, retained, workspace, workspace_bytes, stream);
}

// ------------------------------- matmul ------------------------------------

size_t rmm_matmul_workspace(int64_t n, int64_t d, int64_t m, int64_t lda, int dtype, double rho) {
  if (!dim_ok(n) || !dim_ok(d) || !dim_ok(m) || lda < d || !dtype_ok(dtype) || !rho_ok(rho)) return 0;
  // Upper bound over the paths the call may take: neither the alignment of
  // A (rho = 1 reads a 16-byte aligned A in place, anything else is packed)
  // nor the layout of B is known here.
  size_t best = 0;
  for (int a_ok = 0; a_ok < 2; ++a_ok)
    for (int b_ok = 0; b_ok < 2; ++b_ok) {
      const MatPlan p = plan_matmul(n, d, m, lda, b_ok ? m : m + 1, dtype, rho, a_ok != 0, b_ok != 0);
      best = p.total > best ? p.total : best;
    }
  return best;
}

namespace {

// ------------------------ scratch of the no-alloc call ----------------------
// A file-scope device array, one copy per GPU the library runs on (held until
// the process ends), stands in for the caller's workspace in
// rmm_matmul_noalloc.  Its host-side name is not a device address: host code
// only uses the per-device address hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
static rmm_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RMM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RMM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RMM_OK;
}

// use_scratch: the workspace is the current device's scratch array instead
// of (workspace, workspace_bytes); a call that needs more than it holds is
// refused with RMM_ERR_WORKSPACE before anything is queued.
rmm_status_t matmul_impl(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                         int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* stage_events, bool use_scratch = false) {
  if (!A || !B || !idx || !Y) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (!dtype_ok(dtype) || !dtype_ok(y_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(n) || !dim_ok(d) || !dim_ok(m) || lda < d || ldb < m || ldy < m || lda >= kMaxDim ||
      ldb >= kMaxDim || ldy >= kMaxDim)
    return RMM_ERR_SHAPE;
  const size_t elt = elt_size(dtype);
  if (!aligned(A, elt) || !aligned(B, elt) || !aligned(idx, 4) || !aligned(Y, elt_size(y_dtype)))
    return RMM_ERR_ALIGN;
  const MatPlan p = plan_matmul(n, d, m, lda, ldb, dtype, rho, aligned(A, 16), aligned(B, 16));
  if (use_scratch) {
    if (p.total > kScratchBytes) return RMM_ERR_WORKSPACE;
  } else if (p.total > 0 && (!workspace || workspace_bytes < p.total || !aligned(workspace, 256))) {
    return RMM_ERR_WORKSPACE;
  }
  const Span sa = span3(A, 1, 0, n, lda, d, elt), sb = span3(B, 1, 0, d, ldb, m, elt);
  const Span si = span3(idx, 1, 0, 1, p.k, p.k, 4), sy = span3(Y, 1, 0, n, ldy, m, elt_size(y_dtype));
  if (overlap(si, sa) || overlap(si, sb) || overlap(sy, sa) || overlap(sy, sb) || overlap(sy, si))
    return RMM_ERR_ALIAS;
  if (p.total > 0 && !use_scratch) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
    if (overlap(sw, sa) || overlap(sw, sb) || overlap(sw, si) || overlap(sw, sy)) return RMM_ERR_ALIAS;
  }
  if (p.path == MatPath::kMfmaDirect || p.path == MatPath::kMfmaPacked) {
    const int64_t b_bytes = ((d - 1) * ldb + m) * 2;
    const int64_t a_bytes = p.path == MatPath::kMfmaDirect ? ((n - 1) * lda + d) * 2 : n * p.k_pad * 2;
    if (b_bytes > kMaxOperandBytes || a_bytes > kMaxOperandBytes) return RMM_ERR_SHAPE;
  }
  if (use_scratch && p.total > 0) {
    // every argument is valid: only now look up this device's scratch
    const rmm_status_t st = scratch_of_current_device(&workspace);
    if (st != RMM_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool bf16 = dtype == RMM_BF16;
  const Marks mk{stage_events, s};
  clear_error();
  RMM_LAUNCH(mk.mark(0));
  switch (p.path) {
    case MatPath::kSimt: {
      if (p.use_sel) {
        RMM_LAUNCH(run_select(p.sel, ws, A, bf16, 0, lda, 1, n, d, p.k, idx, p.k, nullptr, s, &mk));
      } else {
        RMM_LAUNCH(launch_iota(idx, p.k, 1, (int)d, nullptr, 0, 0, s));
        RMM_LAUNCH(mk.mark(1));
      }
      RMM_LAUNCH(mk.mark(2));
      RMM_LAUNCH(mk.mark(3));
      SimtArgs g{};
      g.A = A; g.a_bf16 = bf16; g.a_bs = 0; g.a_rs = lda; g.a_cs = 1;
      g.B = B; g.b_bf16 = bf16; g.b_bs = 0; g.b_ts = ldb; g.b_js = 1; g.b_group = 1;
      g.idx = p.all ? nullptr : idx; g.idx_bs = 0;
      g.C = Y; g.c_bf16 = y_dtype == RMM_BF16; g.c_bs = 0; g.ldc = ldy;
      g.M = (int)n; g.N = (int)m; g.k = (int)p.k; g.batch = 1;
      RMM_LAUNCH(launch_gemm_simt(g, s));
      break;
    }
    case MatPath::kDecode: {
      // rho < 1: the GEMV ranks the columns of A itself (up to
      // gemv_select_max_d() columns; wider rows take one selection kernel
      // first); rho = 1: the identity list, written by the GEMV
      const bool fused = !p.all && d <= gemv_select_max_d();
      if (!p.all && !fused)
        RMM_LAUNCH(launch_decode_select(A, bf16, lda, (int)n, (int)d, (int)p.k, idx, nullptr,
                                        d > topk_lds_capacity() ? (uint32_t*)(ws + p.off_dkeys) : nullptr, s));
      RMM_LAUNCH(mk.mark(1));
      RMM_LAUNCH(mk.mark(2));
      RMM_LAUNCH(mk.mark(3));
      GemvArgs g{};
      g.A = A; g.a_bf16 = bf16; g.lda = lda;
      g.B = (const uint16_t*)B; g.ldb = ldb;
      g.idx = p.all || fused ? nullptr : idx;
      g.select = fused; g.d = (int)d;
      g.idx_out = p.all || fused ? idx : nullptr;
      g.k = (int)p.k; g.n = (int)n; g.m = (int)m;
      g.partial = (float*)(ws + p.off_part); g.splits = p.gemv_splits;
      g.Y = Y; g.y_bf16 = y_dtype == RMM_BF16; g.ldy = ldy;
      RMM_LAUNCH(launch_gemv(g, s));
      break;
    }
    case MatPath::kMfmaDirect: {
      // every column kept: the GEMM's first workgroup writes the identity list
      RMM_LAUNCH(mk.mark(1));
      RMM_LAUNCH(mk.mark(2));
      RMM_LAUNCH(mk.mark(3));
      GemmArgs g{};
      g.A = (const uint16_t*)A; g.a_bs = 0; g.lda = lda;
      g.B = (const uint16_t*)B; g.b_bs = 0; g.ldb = ldb; g.b_group = 1;
      g.idx = nullptr; g.idx_bs = 0;
      g.C = Y; g.c_bs = 0; g.ldc = ldy; g.c_bf16 = y_dtype == RMM_BF16;
      g.M = (int)n; g.N = (int)m; g.K = (int)d; g.batch = 1; g.b_kmajor = true;
      g.a_bytes = (uint32_t)(((n - 1) * lda + d) * 2);
      g.b_bytes = (uint32_t)(((d - 1) * ldb + m) * 2);
      g.iota_out = idx; g.iota_heads = 1; g.iota_n = (int)d; g.iota_hs = 0;
      RMM_LAUNCH(launch_gemm_bf16(g, s));
      break;
    }
    case MatPath::kMfmaPacked: {
      int32_t* ipad = (int32_t*)(ws + p.off_ipad);
      uint16_t* pk = (uint16_t*)(ws + p.off_pack);
      if (p.use_sel && select_pack_fits(A, lda, d)) {
        RMM_LAUNCH(run_select_pack(p.sel, ws, A, lda, n, d, p.k, p.k_pad, idx, ipad, pk, s, mk));
      } else {
        if (p.use_sel) {
          RMM_LAUNCH(run_select(p.sel, ws, A, true, 0, lda, 1, n, d, p.k, idx, p.k, nullptr, s, &mk, ipad, p.k_pad));
        } else {
          RMM_LAUNCH(launch_iota(idx, p.k, 1, (int)d, ipad, 0, (int)p.k_pad, s));
          RMM_LAUNCH(mk.mark(1));
        }
        RMM_LAUNCH(mk.mark(2));
        RMM_LAUNCH(launch_pack(A, true, 0, lda, 1, idx, p.k, (int)p.k, (int)p.k_pad, 1, (int)n, pk, 0, s));
        RMM_LAUNCH(mk.mark(3));
      }
      GemmArgs g{};
      g.A = pk; g.a_bs = 0; g.lda = p.k_pad;
      g.B = (const uint16_t*)B; g.b_bs = 0; g.ldb = ldb; g.b_group = 1;
      g.idx = ipad; g.idx_bs = 0;
      g.C = Y; g.c_bs = 0; g.ldc = ldy; g.c_bf16 = y_dtype == RMM_BF16;
      g.M = (int)n; g.N = (int)m; g.K = (int)p.k_pad; g.batch = 1; g.b_kmajor = true;
      g.a_bytes = (uint32_t)(n * p.k_pad * 2);
      g.b_bytes = (uint32_t)(((d - 1) * ldb + m) * 2);
      RMM_LAUNCH(launch_gemm_bf16(g, s));
      break;
    }
  }
  RMM_LAUNCH(mk.mark(4));
  return RMM_OK;
}

}  // namespace

rmm_status_t rmm_matmul(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                        int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return matmul_impl(A, B, dtype, n, d, m, lda, ldb, rho, idx, Y, y_dtype, ldy, workspace, workspace_bytes, stream,
                     nullptr);
}

rmm_status_t rmm_matmul_noalloc(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                                int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy, void* stream) {
  return matmul_impl(A, B, dtype, n, d, m, lda, ldb, rho, idx, Y, y_dtype, ldy, nullptr, 0, stream, nullptr, true);
}

rmm_status_t rmm_matmul_timed(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                              int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy,
                              void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (!stage_events) return RMM_ERR_NULL;
  for (int i = 0; i < 5; ++i)
    if (!stage_events[i]) return RMM_ERR_NULL;
  return matmul_impl(A, B, dtype, n, d, m, lda, ldb, rho, idx, Y, y_dtype, ldy, workspace, workspace_bytes, stream,
                     stage_events);
}

// ------------------------------ matmul_w8 -----------------------------------

size_t rmm_matmul_w8_workspace(int64_t n, int64_t d, int64_t m, int64_t lda, double rho) {
  if (!dim_ok(n) || !dim_ok(d) || !dim_ok(m) || lda < d || !rho_ok(rho)) return 0;
  // the A side decides the path; B is always vector-loadable here
  MatPlan a = plan_matmul(n, d, m, lda, m, RMM_BF16, rho, true, true);
  MatPlan b = plan_matmul(n, d, m, lda, m, RMM_BF16, rho, false, true);
  return a.total > b.total ? a.total : b.total;
}

namespace {

rmm_status_t matmul_w8_impl(const void* A, int a_dtype, const int8_t* Bq, const float* scale, int64_t n, int64_t d,
                            int64_t m, int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype,
                            int64_t ldy, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* stage_events) {
  if (!A || !Bq || !scale || !idx || !Y) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (a_dtype != RMM_BF16 || !dtype_ok(y_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(n) || !dim_ok(d) || !dim_ok(m) || lda < d || ldb < m || ldy < m || lda >= kMaxDim ||
      ldb >= kMaxDim || ldy >= kMaxDim || m % 8 != 0 || ldb % 8 != 0)
    return RMM_ERR_SHAPE;
  if (!aligned(A, 2) || !aligned(Bq, 8) || !aligned(scale, 4) || !aligned(idx, 4) ||
      !aligned(Y, elt_size(y_dtype)))
    return RMM_ERR_ALIGN;
  const MatPlan p = plan_matmul(n, d, m, lda, ldb, RMM_BF16, rho, aligned(A, 16), true);
  if (p.path == MatPath::kSimt) return RMM_ERR_SHAPE;   // not reachable: B is vector-loadable
  if (p.total > 0 && (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)))
    return RMM_ERR_WORKSPACE;
  const Span sa = span3(A, 1, 0, n, lda, d, 2), sb = span3(Bq, 1, 0, d, ldb, m, 1);
  const Span sc = span3(scale, 1, 0, 1, m, m, 4);
  const Span si = span3(idx, 1, 0, 1, p.k, p.k, 4), sy = span3(Y, 1, 0, n, ldy, m, elt_size(y_dtype));
  if (overlap(si, sa) || overlap(si, sb) || overlap(si, sc) || overlap(sy, sa) || overlap(sy, sb) ||
      overlap(sy, sc) || overlap(sy, si))
    return RMM_ERR_ALIAS;
  if (p.total > 0) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
    if (overlap(sw, sa) || overlap(sw, sb) || overlap(sw, sc) || overlap(sw, si) || overlap(sw, sy))
      return RMM_ERR_ALIAS;
  }
  const int64_t b_bytes = (d - 1) * ldb + m;
  if (p.path != MatPath::kDecode) {
    const int64_t a_bytes = p.path == MatPath::kMfmaDirect ? ((n - 1) * lda + d) * 2 : n * p.k_pad * 2;
    if (b_bytes > kMaxOperandBytes || a_bytes > kMaxOperandBytes) return RMM_ERR_SHAPE;
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const Marks mk{stage_events, s};
  clear_error();
  RMM_LAUNCH(mk.mark(0));
  if (p.path == MatPath::kDecode) {
    const bool fused = !p.all && d <= gemv_select_max_d();
    if (!p.all && !fused)
      RMM_LAUNCH(launch_decode_select(A, true, lda, (int)n, (int)d, (int)p.k, idx, nullptr,
                                      d > topk_lds_capacity() ? (uint32_t*)(ws + p.off_dkeys) : nullptr, s));
    RMM_LAUNCH(mk.mark(1));
    RMM_LAUNCH(mk.mark(2));
    RMM_LAUNCH(mk.mark(3));
    GemvArgs g{};
    g.A = A; g.a_bf16 = true; g.lda = lda;
    g.B = Bq; g.ldb = ldb; g.b_i8 = true; g.col_scale = scale;
    g.idx = p.all || fused ? nullptr : idx;
    g.select = fused; g.d = (int)d;
    g.idx_out = p.all || fused ? idx : nullptr;
    g.k = (int)p.k; g.n = (int)n; g.m = (int)m;
    g.partial = (float*)(ws + p.off_part); g.splits = p.gemv_splits;
    g.Y = Y; g.y_bf16 = y_dtype == RMM_BF16; g.ldy = ldy;
    RMM_LAUNCH(launch_gemv(g, s));
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  GemmArgs g{};
  g.B = (const uint16_t*)(const void*)Bq; g.b_bs = 0; g.ldb = ldb; g.b_group = 1; g.b_i8 = true;
  g.b_bytes = (uint32_t)b_bytes;
  g.col_scale = scale;
  g.C = Y; g.c_bs = 0; g.ldc = ldy; g.c_bf16 = y_dtype == RMM_BF16;
  g.M = (int)n; g.N = (int)m; g.batch = 1; g.b_kmajor = true;
  if (p.path == MatPath::kMfmaDirect) {
    // every column kept: the GEMM's first workgroup writes the identity list
    RMM_LAUNCH(mk.mark(1));
    RMM_LAUNCH(mk.mark(2));
    RMM_LAUNCH(mk.mark(3));
    g.A = (const uint16_t*)A; g.a_bs = 0; g.lda = lda;
    g.idx = nullptr; g.idx_bs = 0;
    g.K = (int)d;
    g.a_bytes = (uint32_t)(((n - 1) * lda + d) * 2);
    g.iota_out = idx; g.iota_heads = 1; g.iota_n = (int)d; g.iota_hs = 0;
  } else {
    int32_t* ipad = (int32_t*)(ws + p.off_ipad);
    uint16_t* pk = (uint16_t*)(ws + p.off_pack);
    if (p.use_sel && select_pack_fits(A, lda, d)) {
      RMM_LAUNCH(run_select_pack(p.sel, ws, A, lda, n, d, p.k, p.k_pad, idx, ipad, pk, s, mk));
    } else {
      if (p.use_sel) {
        RMM_LAUNCH(run_select(p.sel, ws, A, true, 0, lda, 1, n, d, p.k, idx, p.k, nullptr, s, &mk, ipad, p.k_pad));
      } else {
        RMM_LAUNCH(launch_iota(idx, p.k, 1, (int)d, ipad, 0, (int)p.k_pad, s));
        RMM_LAUNCH(mk.mark(1));
      }
      RMM_LAUNCH(mk.mark(2));
      RMM_LAUNCH(launch_pack(A, true, 0, lda, 1, idx, p.k, (int)p.k, (int)p.k_pad, 1, (int)n, pk, 0, s));
      RMM_LAUNCH(mk.mark(3));
    }
    g.A = pk; g.a_bs = 0; g.lda = p.k_pad;
    g.idx = ipad; g.idx_bs = 0;
    g.K = (int)p.k_pad;
    g.a_bytes = (uint32_t)(n * p.k_pad * 2);
  }
  RMM_LAUNCH(launch_gemm_w8(g, s));
  RMM_LAUNCH(mk.mark(4));
  return RMM_OK;
}

}  // namespace

rmm_status_t rmm_matmul_w8(const void* A, int a_dtype, const int8_t* Bq, const float* scale, int64_t n, int64_t d,
                           int64_t m, int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype,
                           int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return matmul_w8_impl(A, a_dtype, Bq, scale, n, d, m, lda, ldb, rho, idx, Y, y_dtype, ldy, workspace,
                        workspace_bytes, stream, nullptr);
}

rmm_status_t rmm_matmul_w8_timed(const void* A, int a_dtype, const int8_t* Bq, const float* scale, int64_t n,
                                 int64_t d, int64_t m, int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y,
                                 int y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events) {
  if (!stage_events) return RMM_ERR_NULL;
  for (int i = 0; i < 5; ++i)
    if (!stage_events[i]) return RMM_ERR_NULL;
  return matmul_w8_impl(A, a_dtype, Bq, scale, n, d, m, lda, ldb, rho, idx, Y, y_dtype, ldy, workspace,
                        workspace_bytes, stream, stage_events);
}

// ----------------------------- matmul_idx -----------------------------------

namespace {

struct IdxPlan {
  MatPath path = MatPath::kSimt;
  int64_t k_pad = 0;
  int gemv_splits = 1;
  size_t off_ipad = 0, off_pack = 0, off_part = 0, total = 0;
};

IdxPlan plan_matmul_idx(int64_t n, int64_t k, int64_t m, int64_t ldb, int dtype, bool b_ptr_ok) {
  IdxPlan p;
  Carve cv;
  p.k_pad = round_up(k, kKTile);
  p.off_ipad = cv.take((size_t)p.k_pad * 4);
  const bool bf16 = dtype == RMM_BF16;
  const bool b_vec = bf16 && b_ptr_ok && ldb % 8 == 0 && m % 8 == 0;
  if (!b_vec) {
    p.path = MatPath::kSimt;
  } else if (n <= kDecodeRows) {
    p.path = MatPath::kDecode;
    p.gemv_splits = gemv_splits((int)k, (int)m);
    if (p.gemv_splits > 1) p.off_part = cv.take((size_t)p.gemv_splits * n * m * 4);
  } else {
    p.path = MatPath::kMfmaPacked;
    p.off_pack = cv.take((size_t)n * p.k_pad * 2);
  }
  p.total = cv.used;
  return p;
}

}  // namespace

size_t rmm_matmul_idx_workspace(int64_t n, int64_t k, int64_t m, int dtype) {
  if (!dim_ok(n) || !dim_ok(k) || !dim_ok(m) || !dtype_ok(dtype)) return 0;
  const size_t a = plan_matmul_idx(n, k, m, m, dtype, true).total;
  const size_t b = plan_matmul_idx(n, k, m, m, dtype, false).total;
  return a > b ? a : b;
}

rmm_status_t rmm_matmul_idx(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                            int64_t ldb, const int32_t* idx, int64_t k, void* Y, int y_dtype, int64_t ldy,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!A || !B || !idx || !Y) return RMM_ERR_NULL;
  if (!dtype_ok(dtype) || !dtype_ok(y_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(n) || !dim_ok(d) || !dim_ok(m) || !dim_ok(k) || lda < d || ldb < m || ldy < m || lda >= kMaxDim ||
      ldb >= kMaxDim || ldy >= kMaxDim)
    return RMM_ERR_SHAPE;
  const size_t elt = elt_size(dtype);
  if (!aligned(A, elt) || !aligned(B, elt) || !aligned(idx, 4) || !aligned(Y, elt_size(y_dtype)))
    return RMM_ERR_ALIGN;
  const IdxPlan p = plan_matmul_idx(n, k, m, ldb, dtype, aligned(B, 16));
  if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return RMM_ERR_WORKSPACE;
  const Span sa = span3(A, 1, 0, n, lda, d, elt), sb = span3(B, 1, 0, d, ldb, m, elt);
  const Span si = span3(idx, 1, 0, 1, k, k, 4), sy = span3(Y, 1, 0, n, ldy, m, elt_size(y_dtype));
  const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
  if (overlap(sy, sa) || overlap(sy, sb) || overlap(sy, si) || overlap(sw, sa) || overlap(sw, sb) ||
      overlap(sw, si) || overlap(sw, sy))
    return RMM_ERR_ALIAS;
  if (p.path == MatPath::kMfmaPacked &&
      (((d - 1) * ldb + m) * 2 > kMaxOperandBytes || n * p.k_pad * 2 > kMaxOperandBytes))
    return RMM_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool bf16 = dtype == RMM_BF16;
  int32_t* ipad = (int32_t*)(ws + p.off_ipad);
  clear_error();
  const bool gather = p.path == MatPath::kMfmaPacked && bf16 && gather_pack_fits(A, lda, d, p.k_pad);
  if (!gather) RMM_LAUNCH(launch_pad_index(idx, (int)k, (int)d, ipad, (int)p.k_pad, s));
  switch (p.path) {
    case MatPath::kSimt: {
      SimtArgs g{};
      g.A = A; g.a_bf16 = bf16; g.a_bs = 0; g.a_rs = lda; g.a_cs = 1;
      g.B = B; g.b_bf16 = bf16; g.b_bs = 0; g.b_ts = ldb; g.b_js = 1; g.b_group = 1;
      g.idx = ipad; g.idx_bs = 0;
      g.C = Y; g.c_bf16 = y_dtype == RMM_BF16; g.c_bs = 0; g.ldc = ldy;
      g.M = (int)n; g.N = (int)m; g.k = (int)k; g.batch = 1;
      RMM_LAUNCH(launch_gemm_simt(g, s));
      break;
    }
    case MatPath::kDecode: {
      GemvArgs g{};
      g.A = A; g.a_bf16 = bf16; g.lda = lda;
      g.B = (const uint16_t*)B; g.ldb = ldb;
      g.idx = ipad;
      g.k = (int)k; g.n = (int)n; g.m = (int)m;
      g.partial = (float*)(ws + p.off_part); g.splits = p.gemv_splits;
      g.Y = Y; g.y_bf16 = y_dtype == RMM_BF16; g.ldy = ldy;
      RMM_LAUNCH(launch_gemv(g, s));
      break;
    }
    default: {
      uint16_t* pk = (uint16_t*)(ws + p.off_pack);
      if (gather)
        RMM_LAUNCH(launch_gather_pack(idx, (int)k, (const uint16_t*)A, lda, (int)n, (int)d, (int)p.k_pad, ipad, pk,
                                      s));
      else
        RMM_LAUNCH(launch_pack(A, true, 0, lda, 1, ipad, 0, (int)p.k_pad, (int)p.k_pad, 1, (int)n, pk, 0, s));
      GemmArgs g{};
      g.A = pk; g.a_bs = 0; g.lda = p.k_pad;
      g.B = (const uint16_t*)B; g.b_bs = 0; g.ldb = ldb; g.b_group = 1;
      g.idx = ipad; g.idx_bs = 0;
      g.C = Y; g.c_bs = 0; g.ldc = ldy; g.c_bf16 = y_dtype == RMM_BF16;
      g.M = (int)n; g.N = (int)m; g.K = (int)p.k_pad; g.batch = 1; g.b_kmajor = true;
      g.a_bytes = (uint32_t)(n * p.k_pad * 2);
      g.b_bytes = (uint32_t)(((d - 1) * ldb + m) * 2);
      RMM_LAUNCH(launch_gemm_bf16(g, s));
      break;
    }
  }
  return RMM_OK;
}

// --------------------------------- qk ---------------------------------------

namespace {

struct QkPlan {
  int64_t k = 0, k_pad = 0;
  bool all = false, mfma = false, direct = false, use_sel = false;
  SelPlan sel;
  size_t off_q = 0, off_k = 0, total = 0;
};

QkPlan plan_qk(int64_t hq, int64_t tq, int64_t tk, int64_t dh, int dtype, double rho, bool direct_ok) {
  QkPlan p;
  Carve cv;
  p.k = k_of(rho, dh);
  p.all = p.k == dh;
  p.k_pad = round_up(p.k, kKTile);
  p.mfma = dtype == RMM_BF16;
  if (!p.all) {
    plan_select(cv, p.sel, (int)hq, tq, dh, dtype == RMM_BF16);
    p.use_sel = true;
  }
  if (p.mfma) {
    p.direct = p.all && direct_ok;
    if (!p.direct) {
      p.off_q = cv.take((size_t)hq * tq * p.k_pad * 2);
      p.off_k = cv.take((size_t)hq * tk * p.k_pad * 2);
    }
  }
  p.total = cv.used;
  return p;
}

}  // namespace

size_t rmm_qk_workspace(int64_t hq, int64_t tq, int64_t tk, int64_t dh, int dtype, double rho) {
  if (!dim_ok(hq) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dh) || !dtype_ok(dtype) || !rho_ok(rho)) return 0;
  return plan_qk(hq, tq, tk, dh, dtype, rho, false).total;
}

namespace {

rmm_status_t qk_impl(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                     int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho, int32_t* idx,
                     void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream,
                     void* const* stage_events, bool causal) {
  if (!Q || !K || !idx || !S) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (!dtype_ok(dtype) || !dtype_ok(s_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(hq) || !dim_ok(hkv) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dh) || hq % hkv != 0) return RMM_ERR_SHAPE;
  if (q_ts < dh || k_ts < dh || q_hs < 0 || k_hs < 0 || (hq > 1 && q_hs < 1) || (hkv > 1 && k_hs < 1))
    return RMM_ERR_SHAPE;
  if (hq * tq >= kMaxDim || (double)hq * tq * tk >= 9.0e18) return RMM_ERR_SHAPE;
  if (causal && tq > tk) return RMM_ERR_SHAPE;   // the queries are the last tq of the tk positions
  const size_t elt = elt_size(dtype);
  if (!aligned(Q, elt) || !aligned(K, elt) || !aligned(idx, 4) || !aligned(S, elt_size(s_dtype)))
    return RMM_ERR_ALIGN;
  const bool direct_ok = dtype == RMM_BF16 && aligned(Q, 16) && aligned(K, 16) && q_ts % 8 == 0 &&
                         k_ts % 8 == 0 && q_hs % 8 == 0 && k_hs % 8 == 0 && dh % kKTile == 0 &&
                         ((tq - 1) * q_ts + dh) * 2 <= kMaxOperandBytes && ((tk - 1) * k_ts + dh) * 2 <= kMaxOperandBytes;
  const QkPlan p = plan_qk(hq, tq, tk, dh, dtype, rho, direct_ok);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)))
    return RMM_ERR_WORKSPACE;
  if (p.mfma && !p.direct && (tq * p.k_pad * 2 > kMaxOperandBytes || tk * p.k_pad * 2 > kMaxOperandBytes))
    return RMM_ERR_SHAPE;
  const Span sq = span3(Q, hq, q_hs, tq, q_ts, dh, elt), sk = span3(K, hkv, k_hs, tk, k_ts, dh, elt);
  const Span si = span3(idx, 1, 0, hq, p.k, p.k, 4);
  const Span ss = span3(S, hq, tq * tk, tq, tk, tk, elt_size(s_dtype));
  if (overlap(si, sq) || overlap(si, sk) || overlap(ss, sq) || overlap(ss, sk) || overlap(ss, si))
    return RMM_ERR_ALIAS;
  if (p.total > 0) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
    if (overlap(sw, sq) || overlap(sw, sk) || overlap(sw, si) || overlap(sw, ss)) return RMM_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool bf16 = dtype == RMM_BF16;
  const int group = (int)(hq / hkv);
  const Marks mk{stage_events, s};
  clear_error();
  RMM_LAUNCH(mk.mark(0));
  if (p.mfma && tq <= kDecodeRows && qk_decode_fits(group, (int)tq, (int)dh) && aligned(K, 16) && k_ts % 8 == 0 &&
      k_hs % 8 == 0) {
    // decode-shaped: one kernel selects the features (bf16 Q, so its keys
    // equal the scoring pass's) and streams the key cache once
    RMM_LAUNCH(mk.mark(1));
    RMM_LAUNCH(mk.mark(2));
    QkDecodeArgs a{};
    a.Q = Q; a.q_bf16 = true; a.q_hs = q_hs; a.q_ts = q_ts;
    a.K = (const uint16_t*)K; a.k_hs = k_hs; a.k_ts = k_ts;
    a.idx_out = idx; a.k = (int)p.k; a.select = !p.all;
    a.hq = (int)hq; a.hkv = (int)hkv; a.tq = (int)tq; a.tk = (int)tk; a.dh = (int)dh;
    a.S = S; a.s_bf16 = s_dtype == RMM_BF16;
    a.causal = causal;
    RMM_LAUNCH(mk.mark(3));
    RMM_LAUNCH(launch_qk_decode(a, s));
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  // bf16 heads of whole 16-byte pieces: the features are ranked and Q and
  // K gathered in one launch after the energy sweep
  const bool fused = p.mfma && p.use_sel && !p.direct && qk_select_pack_fits(Q, K, q_hs, q_ts, k_hs, k_ts, dh);
  if (fused) {
    float* partial = (float*)(ws + p.sel.off_partial);
    RMM_LAUNCH(launch_colnorm(Q, true, q_hs, q_ts, (int)hq, (int)tq, (int)dh, p.sel.splits, partial, s));
    RMM_LAUNCH(mk.mark(1));
    RMM_LAUNCH(launch_qk_select_pack(partial, p.sel.splits, (const uint16_t*)Q, q_hs, q_ts, (const uint16_t*)K, k_hs,
                                     k_ts, (int)hq, group, (int)tq, (int)tk, (int)dh, (int)p.k, (int)p.k_pad, idx,
                                     (uint16_t*)(ws + p.off_q), (uint16_t*)(ws + p.off_k), s));
  } else if (p.use_sel) {
    RMM_LAUNCH(run_select(p.sel, ws, Q, bf16, q_hs, q_ts, (int)hq, tq, dh, p.k, idx, p.k, nullptr, s, &mk));
  } else {
    // every feature kept: the matrix-core product on Q and K in place writes
    // the identity lists itself; the other paths read them (pack, SIMT)
    if (!p.mfma || !p.direct) RMM_LAUNCH(launch_iota(idx, p.k, (int)hq, (int)dh, nullptr, 0, 0, s));
    RMM_LAUNCH(mk.mark(1));
  }
  RMM_LAUNCH(mk.mark(2));
  if (!p.mfma) {
    SimtArgs g{};
    g.A = Q; g.a_bf16 = false; g.a_bs = q_hs; g.a_rs = q_ts; g.a_cs = 1;
    g.B = K; g.b_bf16 = false; g.b_bs = k_hs; g.b_ts = 1; g.b_js = k_ts; g.b_group = group;
    g.idx = p.all ? nullptr : idx; g.idx_bs = p.k;
    g.C = S; g.c_bf16 = s_dtype == RMM_BF16; g.c_bs = tq * tk; g.ldc = tk;
    g.M = (int)tq; g.N = (int)tk; g.k = (int)p.k; g.batch = (int)hq;
    g.causal = causal; g.causal_off = tk - tq;
    RMM_LAUNCH(mk.mark(3));
    RMM_LAUNCH(launch_gemm_simt(g, s));
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  GemmArgs g{};
  if (p.direct) {
    g.A = (const uint16_t*)Q; g.a_bs = q_hs; g.lda = q_ts;
    g.B = (const uint16_t*)K; g.b_bs = k_hs; g.ldb = k_ts; g.b_group = group;
    g.K = (int)dh;
    if (!p.use_sel) {
      g.iota_out = idx; g.iota_heads = (int)hq; g.iota_n = (int)dh; g.iota_hs = p.k;
    }
    g.a_bytes = (uint32_t)(((tq - 1) * q_ts + dh) * 2);
    g.b_bytes = (uint32_t)(((tk - 1) * k_ts + dh) * 2);
  } else {
    uint16_t* qp = (uint16_t*)(ws + p.off_q);
    uint16_t* kp = (uint16_t*)(ws + p.off_k);
    if (!fused) {
      RMM_LAUNCH(launch_pack(Q, true, q_hs, q_ts, 1, idx, p.k, (int)p.k, (int)p.k_pad, (int)hq, (int)tq, qp,
                             tq * p.k_pad, s));
      RMM_LAUNCH(launch_pack(K, true, k_hs, k_ts, group, idx, p.k, (int)p.k, (int)p.k_pad, (int)hq, (int)tk, kp,
                             tk * p.k_pad, s));
    }
    g.A = qp; g.a_bs = tq * p.k_pad; g.lda = p.k_pad;
    g.B = kp; g.b_bs = tk * p.k_pad; g.ldb = p.k_pad; g.b_group = 1;
    g.K = (int)p.k_pad;
    g.a_bytes = (uint32_t)(tq * p.k_pad * 2);
    g.b_bytes = (uint32_t)(tk * p.k_pad * 2);
  }
  g.idx = nullptr; g.idx_bs = 0;
  g.C = S; g.c_bs = tq * tk; g.ldc = tk; g.c_bf16 = s_dtype == RMM_BF16;
  g.M = (int)tq; g.N = (int)tk; g.batch = (int)hq; g.b_kmajor = false;
  g.causal = causal; g.causal_off = tk - tq;
  RMM_LAUNCH(mk.mark(3));
  RMM_LAUNCH(launch_gemm_bf16(g, s));
  RMM_LAUNCH(mk.mark(4));
  return RMM_OK;
}

bool events_ok(void* const* ev) {
  if (!ev) return false;
  for (int i = 0; i < 5; ++i)
    if (!ev[i]) return false;
  return true;
}

}  // namespace

rmm_status_t rmm_qk(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                    int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho, int32_t* idx,
                    void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return qk_impl(Q, K, dtype, hq, hkv, tq, tk, dh, q_hs, q_ts, k_hs, k_ts, rho, idx, S, s_dtype, workspace,
                 workspace_bytes, stream, nullptr, false);
}

rmm_status_t rmm_qk_causal(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                           int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho,
                           int32_t* idx, void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return qk_impl(Q, K, dtype, hq, hkv, tq, tk, dh, q_hs, q_ts, k_hs, k_ts, rho, idx, S, s_dtype, workspace,
                 workspace_bytes, stream, nullptr, true);
}

rmm_status_t rmm_qk_timed(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                          int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho, int32_t* idx,
                          void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* stage_events) {
  if (!events_ok(stage_events)) return RMM_ERR_NULL;
  return qk_impl(Q, K, dtype, hq, hkv, tq, tk, dh, q_hs, q_ts, k_hs, k_ts, rho, idx, S, s_dtype, workspace,
                 workspace_bytes, stream, stage_events, false);
}

// --------------------------------- pv ---------------------------------------

namespace {

struct PvPlan {
  int64_t k = 0, k_pad = 0;
  bool all = false, mfma = false, direct = false, masked = false, use_sel = false;
  bool decode = false;   // tq <= 16: per-head GEMV over the kept rows of V
  int gemv_splits = 1;
  int k_split = 1;       // fp32 P read in place: contraction ranges of the product
  SelPlan sel;
  size_t off_p = 0, off_ipad = 0, off_mask = 0, off_gpart = 0, off_kpart = 0, total = 0;
};

// PV reads P once for the column energies whatever the path; the product
// then either packs the kept columns of P (a second read of P that touches
// every sector anyway once more than about one column in eight is kept) or
// runs over all key positions of P in place with the dropped rows of V read
// as zeros.  The second form ("masked") is used when at least one key in
// eight is kept and P can be read in place; both compute the same sum
// over the kept positions.
PvPlan plan_pv(int64_t h, int64_t tq, int64_t tk, int64_t dv, int p_dtype, int v_dtype, double rho, bool v_ok,
               bool direct_ok, bool has_energy = false) {
  PvPlan p;
  Carve cv;
  p.k = k_of(rho, tk);
  p.all = p.k == tk;
  p.k_pad = round_up(p.k, kKTile);
  p.mfma = v_dtype == RMM_BF16 && v_ok;
  if (!p.all) {
    if (has_energy) {
      // energies come from the caller: only TopK's key scratch (large tk)
      p.sel.splits = 1;
      p.sel.gkeys = tk > topk_lds_capacity();
      if (p.sel.gkeys) p.sel.off_gkeys = cv.take((size_t)h * tk * 4);
    } else {
      plan_select(cv, p.sel, (int)h, tq, tk, p_dtype == RMM_BF16);
    }
    p.use_sel = true;
  }
  if (p.mfma && tq <= kDecodeRows) {
    // decode-shaped: a GEMV per head that reads only the kept rows of V
    p.decode = true;
    p.gemv_splits = gemv_splits((int)p.k, (int)dv, (int)h);
    if (p.gemv_splits > 1) p.off_gpart = cv.take((size_t)p.gemv_splits * h * tq * dv * 4);
  } else if (p.mfma) {
    p.direct = p.all && direct_ok;
    p.masked = !p.all && direct_ok && p.k * 8 >= tk;
    if (p.masked) {
      p.off_mask = cv.take((size_t)h * tk * 4);
    } else if (!p.direct) {
      p.off_ipad = cv.take((size_t)h * p.k_pad * 4);
      p.off_p = cv.take((size_t)h * tq * p.k_pad * 2);
    }
    if ((p.direct || p.masked) && p_dtype == RMM_FP32) {
      // reading fp32 P in place is the whole cost: with fewer than two
      // 128 x 128 tiles per CU the contraction is split into ranges (at
      // least two K tiles each) so that twice the loads are in flight; the
      // partial sums (at most the size of the packed P the other path uses)
      // are added in range order
      const int64_t tiles = ((tq + 127) / 128) * ((dv + 127) / 128) * h;
      int ks = 1;
      while (ks < 4 && tiles * ks < 2 * 256 && tk % (kKTile * 2 * ks) == 0 && tk / (2 * ks) >= 2 * kKTile &&
             2 * ks * dv * 2 <= tk)
        ks *= 2;
      p.k_split = ks;
      if (ks > 1) p.off_kpart = cv.take((size_t)ks * h * tq * dv * 4);
    }
  }
  p.total = cv.used;
  return p;
}

}  // namespace

size_t rmm_pv_workspace(int64_t h, int64_t tq, int64_t tk, int64_t dv, int p_dtype, int v_dtype, double rho) {
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dv) || !dtype_ok(p_dtype) || !dtype_ok(v_dtype) ||
      !rho_ok(rho))
    return 0;
  // upper bound over the paths the call may take (alignment is not known here)
  const size_t a = plan_pv(h, tq, tk, dv, p_dtype, v_dtype, rho, true, false).total;
  const size_t b = plan_pv(h, tq, tk, dv, p_dtype, v_dtype, rho, true, true).total;
  return a > b ? a : b;
}

namespace {

rmm_status_t pv_impl(const void* P, int p_dtype, const void* V, int v_dtype, int64_t h, int64_t hkv, int64_t tq,
                     int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs, int64_t v_ts, double rho,
                     int32_t* idx, void* O, int o_dtype, void* workspace, size_t workspace_bytes, void* stream,
                     void* const* stage_events, const float* energy = nullptr) {
  if (!P || !V || !idx || !O) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (!dtype_ok(p_dtype) || !dtype_ok(v_dtype) || !dtype_ok(o_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(h) || !dim_ok(hkv) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dv) || h % hkv != 0) return RMM_ERR_SHAPE;
  if (p_ts < tk || v_ts < dv || p_hs < 0 || v_hs < 0 || (h > 1 && p_hs < 1) || (hkv > 1 && v_hs < 1))
    return RMM_ERR_SHAPE;
  if (h * tq >= kMaxDim) return RMM_ERR_SHAPE;
  const size_t pe = elt_size(p_dtype), ve = elt_size(v_dtype);
  if (!aligned(P, pe) || !aligned(V, ve) || !aligned(idx, 4) || !aligned(O, elt_size(o_dtype))) return RMM_ERR_ALIGN;
  const bool v_ok = v_dtype == RMM_BF16 && aligned(V, 16) && v_ts % 8 == 0 && v_hs % 8 == 0 && dv % 8 == 0 &&
                    ((tk - 1) * v_ts + dv) * 2 <= kMaxOperandBytes;
  const bool p_f32 = p_dtype == RMM_FP32;
  const bool direct_ok = aligned(P, 16) && tk % kKTile == 0 && p_hs % (p_f32 ? 4 : 8) == 0 && p_ts % (p_f32 ? 4 : 8) == 0 &&
                         ((tq - 1) * p_ts + tk) * (int64_t)pe <= kMaxOperandBytes;
  const PvPlan p = plan_pv(h, tq, tk, dv, p_dtype, v_dtype, rho, v_ok, direct_ok, energy != nullptr);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)))
    return RMM_ERR_WORKSPACE;
  if (p.mfma && !p.decode && !p.direct && !p.masked && tq * p.k_pad * 2 > kMaxOperandBytes) return RMM_ERR_SHAPE;
  const Span sp = span3(P, h, p_hs, tq, p_ts, tk, pe), sv = span3(V, hkv, v_hs, tk, v_ts, dv, ve);
  const Span si = span3(idx, 1, 0, h, p.k, p.k, 4);
  const Span so = span3(O, h, tq * dv, tq, dv, dv, elt_size(o_dtype));
  if (overlap(si, sp) || overlap(si, sv) || overlap(so, sp) || overlap(so, sv) || overlap(so, si))
    return RMM_ERR_ALIAS;
  if (p.total > 0) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
    if (overlap(sw, sp) || overlap(sw, sv) || overlap(sw, si) || overlap(sw, so)) return RMM_ERR_ALIAS;
    if (energy && overlap(sw, span3(energy, 1, 0, h, tk, tk, 4))) return RMM_ERR_ALIAS;
  }
  if (energy && (overlap(span3(energy, 1, 0, h, tk, tk, 4), si) || overlap(span3(energy, 1, 0, h, tk, tk, 4), so)))
    return RMM_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int group = (int)(h / hkv);
  const Marks mk{stage_events, s};
  clear_error();
  RMM_LAUNCH(mk.mark(0));
  const bool packed = p.mfma && !p.decode && !p.direct && !p.masked;
  int32_t* ipad = packed ? (int32_t*)(ws + p.off_ipad) : nullptr;
  int32_t* kmask = p.masked ? (int32_t*)(ws + p.off_mask) : nullptr;
  uint16_t* pp = packed ? (uint16_t*)(ws + p.off_p) : nullptr;
  // decode at rho = 1: the GEMV writes the identity lists (no iota launch)
  const bool gemv_lists = p.decode && p.all;
  if (p.use_sel) {
    const float* partial = energy;
    if (!energy) {
      float* part = (float*)(ws + p.sel.off_partial);
      RMM_LAUNCH(launch_colnorm(P, !p_f32, p_hs, p_ts, (int)h, (int)tq, (int)tk, p.sel.splits, part, s));
      partial = part;
    }
    RMM_LAUNCH(mk.mark(1));
    RMM_LAUNCH(launch_topk(partial, (int)h, p.sel.splits, (int)tk, (int)p.k, idx, p.k, ipad, p.k_pad,
                           ipad ? (int)p.k_pad : 0, nullptr, tk,
                           p.sel.gkeys ? (uint32_t*)(ws + p.sel.off_gkeys) : nullptr, s, kmask, tk));
  } else if (!gemv_lists) {
    RMM_LAUNCH(launch_iota(idx, p.k, (int)h, (int)tk, ipad, ipad ? p.k_pad : 0, ipad ? (int)p.k_pad : 0, s));
    RMM_LAUNCH(mk.mark(1));
  } else {
    RMM_LAUNCH(mk.mark(1));
  }
  RMM_LAUNCH(mk.mark(2));
  if (pp)
    RMM_LAUNCH(launch_pack(P, !p_f32, p_hs, p_ts, 1, idx, p.k, (int)p.k, (int)p.k_pad, (int)h, (int)tq, pp,
                           tq * p.k_pad, s));
  if (!p.mfma) {
    SimtArgs g{};
    g.A = P; g.a_bf16 = !p_f32; g.a_bs = p_hs; g.a_rs = p_ts; g.a_cs = 1;
    g.B = V; g.b_bf16 = v_dtype == RMM_BF16; g.b_bs = v_hs; g.b_ts = v_ts; g.b_js = 1; g.b_group = group;
    g.idx = p.all ? nullptr : idx; g.idx_bs = p.k;
    g.C = O; g.c_bf16 = o_dtype == RMM_BF16; g.c_bs = tq * dv; g.ldc = dv;
    g.M = (int)tq; g.N = (int)dv; g.k = (int)p.k; g.batch = (int)h;
    RMM_LAUNCH(mk.mark(3));
    RMM_LAUNCH(launch_gemm_simt(g, s));
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  if (p.decode) {
    GemvArgs g{};
    g.A = P; g.a_bf16 = !p_f32; g.lda = p_ts; g.a_bs = p_hs;
    g.B = (const uint16_t*)V; g.ldb = v_ts; g.b_bs = v_hs; g.b_group = group;
    g.idx = p.all ? nullptr : idx; g.idx_bs = p.k;
    g.idx_out = gemv_lists ? idx : nullptr;
    g.k = (int)p.k; g.n = (int)tq; g.m = (int)dv;
    g.partial = (float*)(ws + p.off_gpart); g.splits = p.gemv_splits;
    g.Y = O; g.y_bf16 = o_dtype == RMM_BF16; g.ldy = dv; g.y_bs = tq * dv;
    g.batch = (int)h;
    RMM_LAUNCH(mk.mark(3));
    RMM_LAUNCH(launch_gemv(g, s));
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  GemmArgs g{};
  g.B = (const uint16_t*)V; g.b_bs = v_hs; g.ldb = v_ts; g.b_group = group;
  g.b_bytes = (uint32_t)(((tk - 1) * v_ts + dv) * 2);
  g.C = O; g.c_bs = tq * dv; g.ldc = dv; g.c_bf16 = o_dtype == RMM_BF16;
  g.M = (int)tq; g.N = (int)dv; g.batch = (int)h; g.b_kmajor = true;
  if (p.direct || p.masked) {
    g.A = (const uint16_t*)P; g.a_bs = p_hs; g.lda = p_ts;
    g.a_bytes = (uint32_t)(((tq - 1) * p_ts + tk) * pe);
    g.idx = kmask; g.idx_bs = p.masked ? tk : 0; g.K = (int)tk;
    RMM_LAUNCH(mk.mark(3));
    if (p_f32) {
      g.k_split = p.k_split;
      g.partial = (float*)(ws + p.off_kpart);
      RMM_LAUNCH(launch_gemm_bf16_af32(g, s));
    } else {
      RMM_LAUNCH(launch_gemm_bf16(g, s));
    }
    RMM_LAUNCH(mk.mark(4));
    return RMM_OK;
  }
  g.A = pp; g.a_bs = tq * p.k_pad; g.lda = p.k_pad;
  g.a_bytes = (uint32_t)(tq * p.k_pad * 2);
  g.idx = ipad; g.idx_bs = p.k_pad; g.K = (int)p.k_pad;
  RMM_LAUNCH(mk.mark(3));
  RMM_LAUNCH(launch_gemm_bf16(g, s));
  RMM_LAUNCH(mk.mark(4));
  return RMM_OK;
}

}  // namespace

rmm_status_t rmm_pv(const void* P, int p_dtype, const void* V, int v_dtype, int64_t h, int64_t hkv, int64_t tq,
                    int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs, int64_t v_ts, double rho,
                    int32_t* idx, void* O, int o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return pv_impl(P, p_dtype, V, v_dtype, h, hkv, tq, tk, dv, p_hs, p_ts, v_hs, v_ts, rho, idx, O, o_dtype, workspace,
                 workspace_bytes, stream, nullptr);
}

size_t rmm_pv_energy_workspace(int64_t h, int64_t tq, int64_t tk, int64_t dv, int p_dtype, int v_dtype, double rho) {
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dv) || !dtype_ok(p_dtype) || !dtype_ok(v_dtype) ||
      !rho_ok(rho))
    return 0;
  const size_t a = plan_pv(h, tq, tk, dv, p_dtype, v_dtype, rho, true, false, true).total;
  const size_t b = plan_pv(h, tq, tk, dv, p_dtype, v_dtype, rho, true, true, true).total;
  return a > b ? a : b;
}

rmm_status_t rmm_pv_energy(const void* P, int p_dtype, const void* V, int v_dtype, const float* energy, int64_t h,
                           int64_t hkv, int64_t tq, int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs,
                           int64_t v_ts, double rho, int32_t* idx, void* O, int o_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!energy) return RMM_ERR_NULL;
  if (!aligned(energy, 4)) return RMM_ERR_ALIGN;
  return pv_impl(P, p_dtype, V, v_dtype, h, hkv, tq, tk, dv, p_hs, p_ts, v_hs, v_ts, rho, idx, O, o_dtype, workspace,
                 workspace_bytes, stream, nullptr, energy);
}

size_t rmm_softmax_energy_workspace(int64_t h, int64_t tq, int64_t tk) {
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || tk > softmax_max_keys()) return 0;
  return (size_t)h * softmax_row_blocks((int)h, (int)tq) * tk * 4;
}

rmm_status_t rmm_softmax_energy(const float* L, float scale, int64_t h, int64_t tq, int64_t tk, int64_t l_hs,
                                int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts, float* energy, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!L || !P || !energy) return RMM_ERR_NULL;
  if (!(scale > 0.f) || !(scale < INFINITY)) return RMM_ERR_SHAPE;
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || tk > softmax_max_keys() || l_ts < tk || p_ts < tk || l_hs < 0 ||
      p_hs < 0 || (h > 1 && (l_hs < 1 || p_hs < 1)) || h * tq >= kMaxDim)
    return RMM_ERR_SHAPE;
  if (!aligned(L, 4) || !aligned(P, 4) || !aligned(energy, 4)) return RMM_ERR_ALIGN;
  const size_t need = rmm_softmax_energy_workspace(h, tq, tk);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return RMM_ERR_WORKSPACE;
  const Span sl = span3(L, h, l_hs, tq, l_ts, tk, 4), sp = span3(P, h, p_hs, tq, p_ts, tk, 4);
  const Span se = span3(energy, 1, 0, h, tk, tk, 4);
  const Span sw = span3(workspace, 1, 0, 1, (int64_t)need, (int64_t)need, 1);
  if (overlap(sp, sl) || overlap(se, sl) || overlap(se, sp) || overlap(sw, sl) || overlap(sw, sp) || overlap(sw, se))
    return RMM_ERR_ALIAS;
  clear_error();
  RMM_LAUNCH(launch_softmax_energy(L, l_hs, l_ts, P, p_hs, p_ts, (int)h, (int)tq, (int)tk,
                                   softmax_row_blocks((int)h, (int)tq), scale, (float*)workspace, energy,
                                   (hipStream_t)stream));
  return RMM_OK;
}

// ------------------------- softmax with selection ----------------------------

namespace {

// one workgroup per head (decode) ranks inside the softmax pass; otherwise
// the softmax pass, then TopK over its energies
bool softmax_select_fused(int64_t h, int64_t tq, int64_t tk) {
  return softmax_row_blocks((int)h, (int)tq) == 1 && tk <= softmax_select_max_keys();
}

struct SmSelPlan {
  size_t off_part = 0, off_gkeys = 0, total = 0;
  bool fused = false, gkeys = false;
};

SmSelPlan plan_softmax_select(int64_t h, int64_t tq, int64_t tk) {
  SmSelPlan p;
  Carve cv;
  p.fused = softmax_select_fused(h, tq, tk);
  if (!p.fused) {
    p.off_part = cv.take((size_t)h * softmax_row_blocks((int)h, (int)tq) * tk * 4);
    p.gkeys = tk > topk_lds_capacity();
    if (p.gkeys) p.off_gkeys = cv.take((size_t)h * tk * 4);
  }
  p.total = cv.used;
  return p;
}

}  // namespace

size_t rmm_softmax_select_workspace(int64_t h, int64_t tq, int64_t tk) {
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || tk > softmax_max_keys()) return 0;
  return plan_softmax_select(h, tq, tk).total;
}

rmm_status_t rmm_softmax_select(const float* L, float scale, int64_t h, int64_t tq, int64_t tk, int64_t l_hs,
                                int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts, float* energy, double rho,
                                int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (!L || !P || !energy || !idx) return RMM_ERR_NULL;
  if (!rho_ok(rho)) return RMM_ERR_RHO;
  if (!(scale > 0.f) || !(scale < INFINITY)) return RMM_ERR_SHAPE;
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(tk) || tk > softmax_max_keys() || l_ts < tk || p_ts < tk || l_hs < 0 ||
      p_hs < 0 || (h > 1 && (l_hs < 1 || p_hs < 1)) || h * tq >= kMaxDim)
    return RMM_ERR_SHAPE;
  if (!aligned(L, 4) || !aligned(P, 4) || !aligned(energy, 4) || !aligned(idx, 4)) return RMM_ERR_ALIGN;
  const SmSelPlan p = plan_softmax_select(h, tq, tk);
  if (p.total > 0 && (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)))
    return RMM_ERR_WORKSPACE;
  const int64_t k = k_of(rho, tk);
  const Span sl = span3(L, h, l_hs, tq, l_ts, tk, 4), sp = span3(P, h, p_hs, tq, p_ts, tk, 4);
  const Span se = span3(energy, 1, 0, h, tk, tk, 4), si = span3(idx, 1, 0, h, k, k, 4);
  if (overlap(sp, sl) || overlap(se, sl) || overlap(se, sp) || overlap(si, sl) || overlap(si, sp) ||
      overlap(si, se))
    return RMM_ERR_ALIAS;
  if (p.total > 0) {
    const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
    if (overlap(sw, sl) || overlap(sw, sp) || overlap(sw, se) || overlap(sw, si)) return RMM_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  clear_error();
  if (p.fused) {
    RMM_LAUNCH(launch_softmax_select(L, l_hs, l_ts, P, p_hs, p_ts, (int)h, (int)tq, (int)tk, scale, energy, (int)k,
                                     idx, s));
    return RMM_OK;
  }
  RMM_LAUNCH(launch_softmax_energy(L, l_hs, l_ts, P, p_hs, p_ts, (int)h, (int)tq, (int)tk,
                                   softmax_row_blocks((int)h, (int)tq), scale, (float*)(ws + p.off_part), energy, s));
  RMM_LAUNCH(launch_topk(energy, (int)h, 1, (int)tk, (int)k, idx, k, nullptr, 0, 0, nullptr, tk,
                         p.gkeys ? (uint32_t*)(ws + p.off_gkeys) : nullptr, s));
  return RMM_OK;
}

// ------------------------------ pv over given lists ------------------------------

namespace {

struct PvIdxPlan {
  int64_t k_pad = 0;
  bool mfma = false, decode = false;
  int gemv_splits = 1;
  size_t off_ipad = 0, off_p = 0, off_gpart = 0, total = 0;
};

PvIdxPlan plan_pv_idx(int64_t h, int64_t tq, int64_t k, int64_t dv, int v_dtype, bool v_ok) {
  PvIdxPlan p;
  Carve cv;
  p.k_pad = round_up(k, kKTile);
  p.off_ipad = cv.take((size_t)h * p.k_pad * 4);
  p.mfma = v_dtype == RMM_BF16 && v_ok;
  if (p.mfma && tq <= kDecodeRows) {
    p.decode = true;
    p.gemv_splits = gemv_splits((int)k, (int)dv, (int)h);
    if (p.gemv_splits > 1) p.off_gpart = cv.take((size_t)p.gemv_splits * h * tq * dv * 4);
  } else if (p.mfma) {
    p.off_p = cv.take((size_t)h * tq * p.k_pad * 2);
  }
  p.total = cv.used;
  return p;
}

}  // namespace

size_t rmm_pv_idx_workspace(int64_t h, int64_t tq, int64_t k, int64_t dv, int v_dtype) {
  if (!dim_ok(h) || !dim_ok(tq) || !dim_ok(k) || !dim_ok(dv) || !dtype_ok(v_dtype)) return 0;
  const size_t a = plan_pv_idx(h, tq, k, dv, v_dtype, true).total;
  const size_t b = plan_pv_idx(h, tq, k, dv, v_dtype, false).total;
  return a > b ? a : b;
}

rmm_status_t rmm_pv_idx(const void* P, int p_dtype, const void* V, int v_dtype, const int32_t* idx, int64_t k,
                        int64_t h, int64_t hkv, int64_t tq, int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts,
                        int64_t v_hs, int64_t v_ts, void* O, int o_dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!P || !V || !idx || !O) return RMM_ERR_NULL;
  if (!dtype_ok(p_dtype) || !dtype_ok(v_dtype) || !dtype_ok(o_dtype)) return RMM_ERR_DTYPE;
  if (!dim_ok(h) || !dim_ok(hkv) || !dim_ok(tq) || !dim_ok(tk) || !dim_ok(dv) || !dim_ok(k) || h % hkv != 0)
    return RMM_ERR_SHAPE;
  if (p_ts < tk || v_ts < dv || p_hs < 0 || v_hs < 0 || (h > 1 && p_hs < 1) || (hkv > 1 && v_hs < 1))
    return RMM_ERR_SHAPE;
  if (h * tq >= kMaxDim) return RMM_ERR_SHAPE;
  const size_t pe = elt_size(p_dtype), ve = elt_size(v_dtype);
  if (!aligned(P, pe) || !aligned(V, ve) || !aligned(idx, 4) || !aligned(O, elt_size(o_dtype))) return RMM_ERR_ALIGN;
  const bool v_ok = v_dtype == RMM_BF16 && aligned(V, 16) && v_ts % 8 == 0 && v_hs % 8 == 0 && dv % 8 == 0 &&
                    ((tk - 1) * v_ts + dv) * 2 <= kMaxOperandBytes;
  const PvIdxPlan p = plan_pv_idx(h, tq, k, dv, v_dtype, v_ok);
  if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return RMM_ERR_WORKSPACE;
  if (p.mfma && !p.decode && tq * p.k_pad * 2 > kMaxOperandBytes) return RMM_ERR_SHAPE;
  const Span sp = span3(P, h, p_hs, tq, p_ts, tk, pe), sv = span3(V, hkv, v_hs, tk, v_ts, dv, ve);
  const Span si = span3(idx, 1, 0, h, k, k, 4);
  const Span so = span3(O, h, tq * dv, tq, dv, dv, elt_size(o_dtype));
  const Span sw = span3(workspace, 1, 0, 1, (int64_t)p.total, (int64_t)p.total, 1);
  if (overlap(so, sp) || overlap(so, sv) || overlap(so, si) || overlap(sw, sp) || overlap(sw, sv) ||
      overlap(sw, si) || overlap(sw, so))
    return RMM_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int group = (int)(h / hkv);
  int32_t* ipad = (int32_t*)(ws + p.off_ipad);
  clear_error();
  // entries outside [0, tk) become -1 (a zero row), the lists padded to
  // k_pad; the GEMV (decode) takes the lists as they are and drops such
  // entries itself
  if (!p.decode) RMM_LAUNCH(launch_pad_index(idx, (int)k, (int)tk, ipad, (int)p.k_pad, s, (int)h, k, p.k_pad));
  if (!p.mfma) {
    SimtArgs g{};
    g.A = P; g.a_bf16 = p_dtype == RMM_BF16; g.a_bs = p_hs; g.a_rs = p_ts; g.a_cs = 1;
    g.B = V; g.b_bf16 = v_dtype == RMM_BF16; g.b_bs = v_hs; g.b_ts = v_ts; g.b_js = 1; g.b_group = group;
    g.idx = ipad; g.idx_bs = p.k_pad;
    g.C = O; g.c_bf16 = o_dtype == RMM_BF16; g.c_bs = tq * dv; g.ldc = dv;
    g.M = (int)tq; g.N = (int)dv; g.k = (int)k; g.batch = (int)h;
    RMM_LAUNCH(launch_gemm_simt(g, s));
    return RMM_OK;
  }
  if (p.decode) {
    GemvArgs g{};
    g.A = P; g.a_bf16 = p_dtype == RMM_BF16; g.lda = p_ts; g.a_bs = p_hs;
    g.B = (const uint16_t*)V; g.ldb = v_ts; g.b_bs = v_hs; g.b_group = group;
    g.idx = idx; g.idx_bs = k; g.d = (int)tk;
    g.k = (int)k; g.n = (int)tq; g.m = (int)dv;
    g.partial = (float*)(ws + p.off_gpart); g.splits = p.gemv_splits;
    g.Y = O; g.y_bf16 = o_dtype == RMM_BF16; g.ldy = dv; g.y_bs = tq * dv;
    g.batch = (int)h;
    RMM_LAUNCH(launch_gemv(g, s));
    return RMM_OK;
  }
  uint16_t* pp = (uint16_t*)(ws + p.off_p);
  RMM_LAUNCH(launch_pack(P, p_dtype == RMM_BF16, p_hs, p_ts, 1, ipad, p.k_pad, (int)p.k_pad, (int)p.k_pad, (int)h,
                         (int)tq, pp, tq * p.k_pad, s));
  GemmArgs g{};
  g.A = pp; g.a_bs = tq * p.k_pad; g.lda = p.k_pad;
  g.a_bytes = (uint32_t)(tq * p.k_pad * 2);
  g.B = (const uint16_t*)V; g.b_bs = v_hs; g.ldb = v_ts; g.b_group = group;
  g.b_bytes = (uint32_t)(((tk - 1) * v_ts + dv) * 2);
  g.idx = ipad; g.idx_bs = p.k_pad;
  g.C = O; g.c_bs = tq * dv; g.ldc = dv; g.c_bf16 = o_dtype == RMM_BF16;
  g.M = (int)tq; g.N = (int)dv; g.K = (int)p.k_pad; g.batch = (int)h; g.b_kmajor = true;
  RMM_LAUNCH(launch_gemm_bf16(g, s));
  return RMM_OK;
}

// ------------------------- generic workspace query ---------------------------
//
// One bound per operation, over every rho in (0, 1], every dtype and
// every alignment or layout the operation accepts: the sum of the largest
// size each workspace region of the operation's paths can take (each
// carved region is rounded up to 256 bytes).

namespace {

size_t region(size_t bytes) { return (bytes + 255) / 256 * 256; }

// column-energy partials and the TopK key scratch of a selection over
// `heads` matrices of n rows x d columns, either input dtype
size_t select_bound(int64_t heads, int64_t n, int64_t d) {
  const int s16 = colnorm_splits((int)heads, (int)n, (int)d, true);
  const int s32 = colnorm_splits((int)heads, (int)n, (int)d, false);
  const size_t splits = (size_t)(s16 > s32 ? s16 : s32);
  return region((size_t)heads * splits * d * 4) + region((size_t)heads * d * 4);
}

// linear product (n x d) (d x m): selection, padded index list, packed A,
// decode key scratch and slice partials
size_t matmul_bound(int64_t n, int64_t d, int64_t m) {
  const size_t k_pad = (size_t)round_up(d, kKTile);
  size_t b = select_bound(1, n, d) + region(k_pad * 4) + region((size_t)n * k_pad * 2) + region((size_t)d * 4);
  if (n <= kDecodeRows) b += region((size_t)gemv_splits_bound((int)d, (int)m) * n * m * 4);
  return b;
}

}  // namespace

size_t rmm_workspace_bytes(int op, int64_t n_or_heads, int64_t d, int64_t m) {
  const int64_t h = n_or_heads;
  switch (op) {
    case RMM_OP_SELECT:
      if (!dim_ok(h) || !dim_ok(d)) return 0;
      return select_bound(1, h, d);
    case RMM_OP_MATMUL:
    case RMM_OP_MATMUL_W8:
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m)) return 0;
      return matmul_bound(h, d, m);
    case RMM_OP_MATMUL_IDX: {
      // d is the length of the index list here
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m)) return 0;
      const size_t k_pad = (size_t)round_up(d, kKTile);
      size_t b = region(k_pad * 4) + region((size_t)h * k_pad * 2);
      if (h <= kDecodeRows) b += region((size_t)gemv_splits_bound((int)d, (int)m) * h * m * 4);
      return b;
    }
    case RMM_OP_QK: {
      // d = head dim; m bounds both tq and tk
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m)) return 0;
      const size_t k_pad = (size_t)round_up(d, kKTile);
      return select_bound(h, m, d) + region((size_t)h * m * k_pad * 2) + region((size_t)h * m * k_pad * 2);
    }
    case RMM_OP_PV:
    case RMM_OP_PV_ENERGY: {
      // d = key positions tk (the contraction); m bounds both tq and dv
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m)) return 0;
      const size_t k_pad = (size_t)round_up(d, kKTile);
      const int64_t rows = m < kDecodeRows ? m : kDecodeRows;   // the GEMV path takes tq <= 16
      return select_bound(h, m, d) + region((size_t)h * d * 4) + region((size_t)h * k_pad * 4) +
             region((size_t)h * m * k_pad * 2) +
             // dv <= m is not known: the slice count is largest for one strip
             region((size_t)gemv_splits_bound((int)d, 1, (int)h) * h * rows * m * 4);
    }
    case RMM_OP_SOFTMAX_ENERGY:
      // d = key positions tk, m = query rows tq
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m) || d > softmax_max_keys()) return 0;
      return rmm_softmax_energy_workspace(h, m, d);
    case RMM_OP_SOFTMAX_SELECT:
      // d = key positions tk, m = query rows tq (no rho dependence)
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m) || d > softmax_max_keys()) return 0;
      return rmm_softmax_select_workspace(h, m, d);
    case RMM_OP_PV_IDX: {
      // d = length of each head's list, m bounds both tq and dv
      if (!dim_ok(h) || !dim_ok(d) || !dim_ok(m)) return 0;
      const size_t k_pad = (size_t)round_up(d, kKTile);
      const int64_t rows = m < kDecodeRows ? m : kDecodeRows;
      return region((size_t)h * k_pad * 4) + region((size_t)h * m * k_pad * 2) +
             region((size_t)gemv_splits_bound((int)d, 1, (int)h) * h * rows * m * 4);
    }
    default:
      return 0;
  }
}

rmm_status_t rmm_pv_timed(const void* P, int p_dtype, const void* V, int v_dtype, int64_t h, int64_t hkv, int64_t tq,
                          int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs, int64_t v_ts, double rho,
                          int32_t* idx, void* O, int o_dtype, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* stage_events) {
  if (!events_ok(stage_events)) return RMM_ERR_NULL;
  return pv_impl(P, p_dtype, V, v_dtype, h, hkv, tq, tk, dv, p_hs, p_ts, v_hs, v_ts, rho, idx, O, o_dtype, workspace,
                 workspace_bytes, stream, stage_events);
}

}  // extern "C"
