// Host side of the C interface in include/tp.h: argument checks (all before
// any HIP call), shard views (pointer + stride arithmetic, no data movement),
// kernel choice, workspace planning and launches on the caller's stream.
//
// The shard views follow the "Tensor Parallelism" topic page
// (chipfoundryservices.com): "Column-Wise Parallelism" (W = [W_1, ..., W_N],
// shard i computes X W_i) and "Row-Wise Parallelism" (W stacked by rows, X
// split to match, partial products summed). Shard s owns the s-th contiguous
// block of the split dimension; the split must be even.
#include <cmath>
#include <cstring>
#include <mutex>

#include "tp.h"
#include "tp_internal.h"

namespace {

using tp::CombineDesc;
using tp::GemmDesc;

int64_t elt_size(int32_t dtype) { return dtype == TP_BF16 ? 2 : 4; }
bool valid_dtype(int32_t dtype) { return dtype == TP_F32 || dtype == TP_BF16; }

// Address range [lo, hi) touched by `nblocks` blocks of [brows, bcols] with row
// stride ld and block stride `stride` (elements).
struct Range {
  uintptr_t lo = 0, hi = 0;
};

Range range_of(const void* ptr, int32_t dtype, int64_t nblocks, int64_t stride, int64_t brows, int64_t bcols,
               int64_t ld) {
  Range r;
  if (nblocks <= 0 || brows <= 0 || bcols <= 0) return r;
  const int64_t elems = (nblocks - 1) * stride + (brows - 1) * ld + bcols;
  r.lo = reinterpret_cast<uintptr_t>(ptr);
  r.hi = r.lo + (uintptr_t)(elems * elt_size(dtype));
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  if (a.hi <= a.lo || b.hi <= b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Sizes beyond these would overflow the kernels' 32-bit tile and grid arithmetic.
constexpr int64_t kMaxDim = (1ll << 31) - 1;
// One 256-thread workgroup per token row; a launch holds fewer than 2^32 work-items.
constexpr int64_t kMaxLnRows = (1ll << 24) - 1;

// Checks one matrix holding `nblocks` blocks of [brows, bcols]:
//   shard_stride == 0 -> the blocks are slices of one matrix whose rows need
//                        `row_len` elements (ld >= row_len);
//   shard_stride  > 0 -> each block has row stride ld >= bcols and the blocks
//                        must not overlap.
tp_status check_matrix(const tp_matrix* m, int64_t nblocks, int64_t brows, int64_t bcols, int64_t row_len,
                       bool need_ptr = true) {
  if (!m) return TP_ERR_NULL;
  if (!valid_dtype(m->dtype)) return TP_ERR_DTYPE;
  if (m->rows < 0 || m->cols < 0) return TP_ERR_SHAPE;
  if (m->rows > kMaxDim || m->cols > kMaxDim) return TP_ERR_TOO_LARGE;
  if (m->ld < 0 || m->shard_stride < 0) return TP_ERR_STRIDE;
  const bool empty = nblocks <= 0 || brows <= 0 || bcols <= 0;
  if (m->shard_stride == 0) {
    if (!empty && m->ld < row_len) return TP_ERR_STRIDE;
  } else {
    if (!empty && m->ld < bcols) return TP_ERR_STRIDE;
    if (!empty && nblocks > 1 && m->shard_stride < (brows - 1) * m->ld + bcols) return TP_ERR_STRIDE;
  }
  if (need_ptr && !empty && !m->ptr) return TP_ERR_NULL;
  return TP_OK;
}

tp_status hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

// Runs one batched product with the best kernel the operands allow.
hipError_t run_gemm(const GemmDesc& d, hipStream_t stream) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  if (d.in_bf16 && d.M <= tp::kSkinnyMaxRows && tp::gemm_skinny_supported(d))
    return tp::launch_gemm_skinny(d, 1, nullptr, stream);
  if (tp::gemm_mfma_supported(d)) return tp::launch_gemm_mfma(d, stream);
  return tp::launch_gemm_generic(d, stream);
}

struct ColPlan {
  GemmDesc g;
  Range x, w, y;
};

// Column-parallel views: Y_j = act(X W_{s0+j}).
tp_status plan_col(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns, int32_t act,
                   const tp_matrix* Y, ColPlan* out, bool need_ptr = true) {
  if (!X || !W || !Y) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W->dtype) || !valid_dtype(Y->dtype)) return TP_ERR_DTYPE;
  if (X->dtype != W->dtype) return TP_ERR_DTYPE;
  if (act != TP_ACT_NONE && act != TP_ACT_GELU) return TP_ERR_SHAPE;
  if (X->rows < 0 || X->cols < 0 || W->rows < 0 || W->cols < 0 || Y->rows < 0 || Y->cols < 0) return TP_ERR_SHAPE;
  if (N < 1 || W->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, K = X->cols, width = W->cols / N;
  if (W->rows != K) return TP_ERR_SHAPE;
  if (Y->rows != M || Y->cols != (int64_t)ns * width) return TP_ERR_SHAPE;
  if (X->shard_stride != 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(X, 1, M, K, K, need_ptr)) != TP_OK) return st;
  if ((st = check_matrix(W, ns, K, width, W->cols, need_ptr)) != TP_OK) return st;
  if ((st = check_matrix(Y, ns, M, width, Y->cols, need_ptr)) != TP_OK) return st;

  GemmDesc g;
  std::memset(&g, 0, sizeof(g));
  g.in_bf16 = X->dtype == TP_BF16;
  g.out_kind = Y->dtype == TP_BF16 ? tp::OUT_BF16 : tp::OUT_F32;
  g.act = act;
  g.M = M;
  g.K = K;
  g.A = X->ptr;
  g.lda = X->ld;
  g.sA = 0;
  const int64_t we = elt_size(W->dtype);
  const char* wbase = static_cast<const char*>(W->ptr);
  if (W->shard_stride == 0) wbase += (int64_t)s0 * width * we;
  else wbase += (int64_t)s0 * W->shard_stride * we;
  g.B = wbase;
  g.ldb = W->ld;
  g.C = Y->ptr;
  g.ldc = Y->ld;
  if (W->shard_stride == 0 && Y->shard_stride == 0) {
    // Contiguous column shards are one product over ns * width columns: every
    // output element is still the dot product of its own shard.
    g.N = (int64_t)ns * width;
    g.batch = 1;
  } else {
    g.N = width;
    g.batch = ns;
    g.sB = W->shard_stride == 0 ? width : W->shard_stride;
    g.sC = Y->shard_stride == 0 ? width : Y->shard_stride;
  }
  out->g = g;
  out->x = range_of(X->ptr, X->dtype, 1, 0, M, K, X->ld);
  out->w = W->shard_stride == 0 ? range_of(wbase, W->dtype, 1, 0, K, (int64_t)ns * width, W->ld)
                                : range_of(wbase, W->dtype, ns, W->shard_stride, K, width, W->ld);
  out->y = Y->shard_stride == 0 ? range_of(Y->ptr, Y->dtype, 1, 0, M, Y->cols, Y->ld)
                                : range_of(Y->ptr, Y->dtype, ns, Y->shard_stride, M, width, Y->ld);
  if (overlaps(out->y, out->x) || overlaps(out->y, out->w)) return TP_ERR_ALIAS;
  return TP_OK;
}

struct RowPlan {
  GemmDesc g;
  Range x, w, p;
};

// Row-parallel views: P_j = X_{s0+j} W_{s0+j}.
tp_status plan_row(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns, const tp_matrix* P,
                   RowPlan* out) {
  if (!X || !W || !P) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W->dtype) || !valid_dtype(P->dtype)) return TP_ERR_DTYPE;
  if (X->dtype != W->dtype || P->dtype != TP_F32) return TP_ERR_DTYPE;
  if (X->rows < 0 || X->cols < 0 || W->rows < 0 || W->cols < 0 || P->rows < 0 || P->cols < 0) return TP_ERR_SHAPE;
  if (N < 1 || X->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, K = X->cols, kb = K / N, Nout = W->cols;
  if (W->rows != K) return TP_ERR_SHAPE;
  if (P->rows != M || P->cols != Nout) return TP_ERR_SHAPE;
  if (ns > 1 && P->shard_stride == 0 && M > 0 && Nout > 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(X, ns, M, kb, K)) != TP_OK) return st;
  if ((st = check_matrix(W, ns, kb, Nout, Nout)) != TP_OK) return st;
  if ((st = check_matrix(P, ns, M, Nout, Nout)) != TP_OK) return st;

  GemmDesc g;
  std::memset(&g, 0, sizeof(g));
  g.in_bf16 = X->dtype == TP_BF16;
  g.out_kind = tp::OUT_F32;
  g.act = tp::ACT_NONE;
  g.M = M;
  g.N = Nout;
  g.K = kb;
  g.batch = ns;
  const int64_t e = elt_size(X->dtype);
  g.sA = X->shard_stride == 0 ? kb : X->shard_stride;
  g.sB = W->shard_stride == 0 ? kb * W->ld : W->shard_stride;
  g.sC = P->shard_stride;
  const char* xbase = static_cast<const char*>(X->ptr) + (int64_t)s0 * g.sA * e;
  const char* wbase = static_cast<const char*>(W->ptr) + (int64_t)s0 * g.sB * e;
  g.A = xbase;
  g.lda = X->ld;
  g.B = wbase;
  g.ldb = W->ld;
  g.C = P->ptr;
  g.ldc = P->ld;
  out->g = g;
  out->x = X->shard_stride == 0 ? range_of(xbase, X->dtype, 1, 0, M, (int64_t)ns * kb, X->ld)
                                : range_of(xbase, X->dtype, ns, X->shard_stride, M, kb, X->ld);
  out->w = W->shard_stride == 0 ? range_of(wbase, W->dtype, 1, 0, (int64_t)ns * kb, Nout, W->ld)
                                : range_of(wbase, W->dtype, ns, W->shard_stride, kb, Nout, W->ld);
  out->p = range_of(P->ptr, P->dtype, ns, P->shard_stride, M, Nout, P->ld);
  if (overlaps(out->p, out->x) || overlaps(out->p, out->w)) return TP_ERR_ALIAS;
  return TP_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ns consecutive blocks of one tp_matrix: block j starts `step` elements after
// block j-1 (a column or row slice of one matrix when shard_stride is 0,
// shard-major blocks otherwise), the first at block index `first`.
struct Blocks {
  const char* base;
  int64_t ld, step;
  int32_t dtype;
};

Blocks col_blocks(const tp_matrix* m, int64_t first, int64_t bcols) {
  Blocks b;
  b.ld = m->ld;
  b.step = m->shard_stride == 0 ? bcols : m->shard_stride;
  b.dtype = m->dtype;
  b.base = static_cast<const char*>(m->ptr) + first * b.step * elt_size(m->dtype);
  return b;
}

Blocks row_blocks(const tp_matrix* m, int64_t first, int64_t brows) {
  Blocks b;
  b.ld = m->ld;
  b.step = m->shard_stride == 0 ? brows * m->ld : m->shard_stride;
  b.dtype = m->dtype;
  b.base = static_cast<const char*>(m->ptr) + first * b.step * elt_size(m->dtype);
  return b;
}

Range blocks_range(const Blocks& b, int64_t ns, int64_t brows, int64_t bcols) {
  return range_of(b.base, b.dtype, ns, b.step, brows, bcols, b.ld);
}

// A batched product over ns shards: C_j = op(A_j) op(B_j), block j of each
// operand `step` elements after block j-1.
GemmDesc product(const Blocks& a, bool a_trans, const Blocks& b, bool b_trans, const Blocks& c, int64_t M,
                 int64_t N, int64_t K, int64_t batch, bool in_bf16) {
  GemmDesc g;
  std::memset(&g, 0, sizeof(g));
  g.A = a.base;
  g.lda = a.ld;
  g.sA = a.step;
  g.a_trans = a_trans;
  g.B = b.base;
  g.ldb = b.ld;
  g.sB = b.step;
  g.b_trans = b_trans;
  g.C = const_cast<char*>(c.base);
  g.ldc = c.ld;
  g.sC = c.step;
  g.M = M;
  g.N = N;
  g.K = K;
  g.batch = (int32_t)batch;
  g.in_bf16 = in_bf16;
  g.out_kind = c.dtype == TP_BF16 ? tp::OUT_BF16 : tp::OUT_F32;
  g.act = tp::ACT_NONE;
  return g;
}

Blocks whole(const tp_matrix* m) {
  Blocks b;
  b.base = static_cast<const char*>(m->ptr);
  b.ld = m->ld;
  b.step = 0;
  b.dtype = m->dtype;
  return b;
}

Blocks buffer_blocks(void* ptr, int32_t dtype, int64_t ld, int64_t step) {
  Blocks b;
  b.base = static_cast<const char*>(ptr);
  b.ld = ld;
  b.step = step;
  b.dtype = dtype;
  return b;
}

}  // namespace

// Scratch memory of tp_mlp_noalloc: a file-scope device array, so that entry
// point needs no allocation. Every GPU the library runs on holds its own copy
// (kScratchBytes each) from the loading of the library's code object until the
// process ends. In host code `scratch` is only a stand-in for the symbol; its
// device address on each GPU comes from hipGetSymbolAddress and is the only
// form ever handed to kernels.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
}  // namespace
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxScratchDevices];  // device address of `scratch` per device, resolved once

// The address of the current device's copy of `scratch`, looked up on the
// first call made with that device current.
tp_status current_device_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TP_ERR_HIP;
  if (dev >= kMaxScratchDevices) return TP_ERR_TOO_LARGE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TP_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return TP_OK;
}
}  // namespace

extern "C" {

tp_status tp_col_linear(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns, int32_t act,
                        const tp_matrix* Y, void* stream) {
  ColPlan plan;
  const tp_status st = plan_col(X, W, N, s0, ns, act, Y, &plan);
  if (st != TP_OK) return st;
  return hip_status(run_gemm(plan.g, static_cast<hipStream_t>(stream)));
}

tp_status tp_row_linear(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns,
                        const tp_matrix* P, void* stream) {
  RowPlan plan;
  const tp_status st = plan_row(X, W, N, s0, ns, P, &plan);
  if (st != TP_OK) return st;
  return hip_status(run_gemm(plan.g, static_cast<hipStream_t>(stream)));
}

tp_status tp_reduce_partials(const tp_matrix* P, int32_t n, int32_t axis, const tp_matrix* Y, void* stream) {
  if (!P || !Y) return TP_ERR_NULL;
  if (!valid_dtype(P->dtype) || !valid_dtype(Y->dtype)) return TP_ERR_DTYPE;
  if (axis != TP_SPLIT_ROWS && axis != TP_SPLIT_COLS && axis != TP_SPLIT_TOKENS) return TP_ERR_SHAPE;
  if (axis == TP_SPLIT_ROWS && P->dtype != TP_F32) return TP_ERR_DTYPE;
  if (n < 1) return TP_ERR_INDIVISIBLE;
  if (P->rows < 0 || P->cols < 0 || Y->rows < 0 || Y->cols < 0) return TP_ERR_SHAPE;
  const int64_t R = P->rows, C = P->cols;
  const int64_t ycols = axis == TP_SPLIT_COLS ? (int64_t)n * C : C;
  const int64_t yrows = axis == TP_SPLIT_TOKENS ? (int64_t)n * R : R;
  if (Y->rows != yrows || Y->cols != ycols) return TP_ERR_SHAPE;
  if (yrows > kMaxDim || ycols > kMaxDim) return TP_ERR_TOO_LARGE;
  if (Y->shard_stride != 0) return TP_ERR_STRIDE;
  if (n > 1 && P->shard_stride == 0 && R > 0 && C > 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(P, n, R, C, C)) != TP_OK) return st;
  if ((st = check_matrix(Y, 1, yrows, ycols, ycols)) != TP_OK) return st;
  if (overlaps(range_of(Y->ptr, Y->dtype, 1, 0, yrows, ycols, Y->ld),
               range_of(P->ptr, P->dtype, n, P->shard_stride, R, C, P->ld)))
    return TP_ERR_ALIAS;
  CombineDesc d;
  std::memset(&d, 0, sizeof(d));
  d.P = P->ptr;
  d.Y = Y->ptr;
  d.rows = R;
  d.cols = C;
  d.ldp = P->ld;
  d.sP = P->shard_stride;
  d.ldy = Y->ld;
  d.n = n;
  d.p_bf16 = P->dtype == TP_BF16;
  d.y_bf16 = Y->dtype == TP_BF16;
  d.concat = axis == TP_SPLIT_COLS ? 1 : axis == TP_SPLIT_TOKENS ? 2 : 0;
  return hip_status(tp::launch_combine(d, static_cast<hipStream_t>(stream)));
}

tp_status tp_sp_layernorm(const tp_matrix* P, int32_t n, const tp_matrix* R, const uint8_t* keep, float p_drop,
                          const float* gamma, const float* beta, float eps, int32_t N, int32_t s0, int32_t ns,
                          const tp_matrix* X1, const tp_matrix* Y, void* stream) {
  if (!P || !Y) return TP_ERR_NULL;
  if (P->dtype != TP_F32 || !valid_dtype(Y->dtype)) return TP_ERR_DTYPE;
  if (R && !valid_dtype(R->dtype)) return TP_ERR_DTYPE;
  if (X1 && X1->dtype != TP_F32) return TP_ERR_DTYPE;
  if (P->rows < 0 || P->cols < 0 || Y->rows < 0 || Y->cols < 0) return TP_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_ERR_SHAPE;
  if (keep && !(p_drop >= 0.0f && p_drop < 1.0f)) return TP_ERR_SHAPE;
  if (n < 1 || N < 1) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = P->rows, D = P->cols;
  if (M % N != 0) return TP_ERR_INDIVISIBLE;
  const int64_t T = M / N, rows = (int64_t)ns * T;
  if (Y->rows != rows || Y->cols != D) return TP_ERR_SHAPE;
  if (R && (R->rows != rows || R->cols != D)) return TP_ERR_SHAPE;
  if (X1 && (X1->rows != rows || X1->cols != D)) return TP_ERR_SHAPE;
  if (n > 1 && P->shard_stride == 0 && M > 0 && D > 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(P, n, M, D, D)) != TP_OK) return st;
  if ((st = check_matrix(Y, ns, T, D, D)) != TP_OK) return st;
  if (R && (st = check_matrix(R, ns, T, D, D)) != TP_OK) return st;
  if (X1 && (st = check_matrix(X1, ns, T, D, D)) != TP_OK) return st;
  if (rows == 0 || D == 0) return TP_OK;
  if (!gamma || !beta) return TP_ERR_NULL;
  if (rows > kMaxLnRows) return TP_ERR_TOO_LARGE;
  const Blocks pb = row_blocks(P, 0, M), yb = row_blocks(Y, 0, T);
  const Range ry = blocks_range(yb, ns, T, D);
  Range inputs[5] = {blocks_range(pb, n, M, D)};
  Blocks rb{}, xb{};
  if (R) {
    rb = row_blocks(R, 0, T);
    inputs[1] = blocks_range(rb, ns, T, D);
  }
  if (keep) {
    inputs[2].lo = reinterpret_cast<uintptr_t>(keep);
    inputs[2].hi = inputs[2].lo + (uintptr_t)(rows * D);
  }
  inputs[3].lo = reinterpret_cast<uintptr_t>(gamma);
  inputs[3].hi = inputs[3].lo + (uintptr_t)(D * 4);
  inputs[4].lo = reinterpret_cast<uintptr_t>(beta);
  inputs[4].hi = inputs[4].lo + (uintptr_t)(D * 4);
  Range rx;
  if (X1) {
    xb = row_blocks(X1, 0, T);
    rx = blocks_range(xb, ns, T, D);
    if (overlaps(rx, ry)) return TP_ERR_ALIAS;
  }
  for (const Range& in : inputs)
    if (overlaps(ry, in) || overlaps(rx, in)) return TP_ERR_ALIAS;
  tp::LnDesc d;
  std::memset(&d, 0, sizeof(d));
  // the partials' rows of the executed tokens, block t at t * shard_stride
  d.P = reinterpret_cast<const float*>(pb.base) + (int64_t)s0 * T * P->ld;
  d.ldp = P->ld;
  d.sP = P->shard_stride;
  d.n = n;
  if (R) {
    d.R = rb.base;
    d.ldr = rb.ld;
    d.sR = rb.step;
    d.r_bf16 = R->dtype == TP_BF16;
  }
  d.keep = keep;
  d.keep_scale = keep ? 1.0f / (1.0f - p_drop) : 1.0f;
  d.gamma = gamma;
  d.beta = beta;
  d.eps = eps;
  if (X1) {
    d.X1 = reinterpret_cast<float*>(const_cast<char*>(xb.base));
    d.ldx1 = xb.ld;
    d.sX1 = xb.step;
  }
  d.Y = const_cast<char*>(yb.base);
  d.ldy = yb.ld;
  d.sY = yb.step;
  d.y_bf16 = Y->dtype == TP_BF16;
  d.rows_per_shard = T;
  d.rows = rows;
  d.cols = D;
  return hip_status(tp::launch_sp_layernorm(d, static_cast<hipStream_t>(stream)));
}

tp_status tp_mlp(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, int32_t N, int32_t s0, int32_t ns,
                 int32_t act, void* workspace, size_t* workspace_bytes, const tp_matrix* Y, void* stream) {
  if (!X || !W1 || !W2 || !Y || !workspace_bytes) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W1->dtype) || !valid_dtype(W2->dtype) || !valid_dtype(Y->dtype))
    return TP_ERR_DTYPE;
  if (X->dtype != W1->dtype || X->dtype != W2->dtype || Y->dtype != TP_F32) return TP_ERR_DTYPE;
  if (act != TP_ACT_NONE && act != TP_ACT_GELU) return TP_ERR_SHAPE;
  if (X->rows < 0 || X->cols < 0 || W1->rows < 0 || W1->cols < 0 || W2->rows < 0 || W2->cols < 0 ||
      Y->rows < 0 || Y->cols < 0)
    return TP_ERR_SHAPE;
  if (N < 1 || W1->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, d = X->cols, F = W1->cols, width = F / N, Dout = W2->cols;
  if (W1->rows != d || W2->rows != F || Y->rows != M || Y->cols != Dout) return TP_ERR_SHAPE;
  if (X->shard_stride != 0 || Y->shard_stride != 0) return TP_ERR_STRIDE;
  // A size query (workspace == NULL) checks shapes, dtypes and strides only.
  const bool query = workspace == nullptr;
  tp_status st;
  if ((st = check_matrix(X, 1, M, d, d, !query)) != TP_OK) return st;
  if ((st = check_matrix(W1, ns, d, width, F, !query)) != TP_OK) return st;
  if ((st = check_matrix(W2, ns, width, Dout, Dout, !query)) != TP_OK) return st;
  if ((st = check_matrix(Y, 1, M, Dout, Dout, !query)) != TP_OK) return st;

  const bool bf16 = X->dtype == TP_BF16;
  const int32_t hdt = bf16 ? TP_BF16 : TP_F32;
  const int64_t hcols = (int64_t)ns * width;

  // Workspace: H [M, ns * width] (bf16 for bf16 inputs), then the fp32
  // partials [ns][M][Dout] when more than one shard runs, then the skinny
  // kernel's K-chunk sums when that kernel takes the first product.
  size_t off_h = 0;
  size_t bytes_h = align_up((size_t)(M * hcols * elt_size(hdt)), 256);
  size_t off_p = bytes_h;
  size_t bytes_p = ns > 1 ? align_up((size_t)ns * M * Dout * sizeof(float), 256) : 0;
  size_t off_k = off_p + bytes_p;

  // First product: H = act(X W1_s), columns of shard s at (s - s0) * width.
  tp_matrix H;
  std::memset(&H, 0, sizeof(H));
  H.dtype = hdt;
  H.rows = M;
  H.cols = hcols;
  H.ld = hcols;
  H.shard_stride = 0;
  ColPlan c1;
  H.ptr = query ? nullptr : static_cast<char*>(workspace) + off_h;
  st = plan_col(X, W1, N, s0, ns, act, &H, &c1, !query);
  if (st == TP_ERR_ALIAS && query) st = TP_OK;  // addresses are not known in a size query
  if (st != TP_OK) return st;

  int ksplit = 1;
  const bool skinny1 = bf16 && M <= tp::kSkinnyMaxRows && tp::gemm_skinny_supported(c1.g);
  if (skinny1) ksplit = tp::skinny_ksplit(c1.g);
  const size_t bytes_k = skinny1 ? align_up(tp::skinny_partial_bytes(c1.g, ksplit), 256) : 0;
  const size_t need = off_k + bytes_k;
  if (query) {
    *workspace_bytes = need > 0 ? need : 256;
    return TP_OK;
  }
  if (*workspace_bytes < need) return TP_ERR_WORKSPACE;

  // Second product: P_j = H[:, j * width ...] W2_{s0+j}; with one shard it writes Y directly.
  tp_matrix Hrow = H;
  Hrow.cols = (int64_t)ns * width;  // logical K of the row split over the executed shards
  tp_matrix Pm;
  std::memset(&Pm, 0, sizeof(Pm));
  Pm.dtype = TP_F32;
  Pm.rows = M;
  Pm.cols = Dout;
  if (ns > 1) {
    Pm.ptr = static_cast<char*>(workspace) + off_p;
    Pm.ld = Dout;
    Pm.shard_stride = M * Dout;
  } else {
    Pm.ptr = Y->ptr;
    Pm.ld = Y->ld;
    Pm.shard_stride = 0;
  }
  // The executed shards of W2 viewed as a row split of ns blocks, starting at block s0.
  tp_matrix W2v = *W2;
  if (W2->shard_stride == 0) W2v.ptr = static_cast<char*>(W2->ptr) + (int64_t)s0 * width * W2->ld * elt_size(W2->dtype);
  else W2v.ptr = static_cast<char*>(W2->ptr) + (int64_t)s0 * W2->shard_stride * elt_size(W2->dtype);
  W2v.rows = (int64_t)ns * width;
  RowPlan r2;
  if ((st = plan_row(&Hrow, &W2v, ns, 0, ns, &Pm, &r2)) != TP_OK) return st;

  const Range ws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  const Range xr = range_of(X->ptr, X->dtype, 1, 0, M, d, X->ld);
  const Range yr = range_of(Y->ptr, Y->dtype, 1, 0, M, Dout, Y->ld);
  if (overlaps(ws, xr) || overlaps(ws, c1.w) || overlaps(ws, r2.w) || overlaps(ws, yr)) return TP_ERR_ALIAS;
  if (overlaps(yr, xr) || overlaps(yr, c1.w) || overlaps(yr, r2.w)) return TP_ERR_ALIAS;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  float* part = skinny1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + off_k) : nullptr;
  // When the first product leaves K-chunk sums and the second is skinny too,
  // the second adds the sums (ascending), applies the activation and rounds
  // to bf16 as it loads its token fragments: the H it multiplies is bitwise
  // the one the finishing pass would have stored, without that pass. The
  // sums are laid out [chunk][z1][M][N1] for the first product's batch z1;
  // the second product's A_z is H's columns z sA .. z sA + K - 1.
  tp::ChunkedA ca;
  std::memset(&ca, 0, sizeof(ca));
  bool chunked_a = false;
  if (skinny1 && ksplit > 1 && r2.g.in_bf16 && !r2.g.a_trans && r2.g.A == c1.g.C && r2.g.lda == c1.g.ldc &&
      r2.g.M == c1.g.M && c1.g.out_kind == tp::OUT_BF16) {
    ca.part = part;
    ca.ksplit = ksplit;
    ca.act = c1.g.act;
    ca.ld = c1.g.N;
    ca.cs = (int64_t)c1.g.batch * c1.g.M * c1.g.N;
    if (c1.g.batch == r2.g.batch && c1.g.N == r2.g.K && r2.g.sA == c1.g.sC) {
      ca.sz = c1.g.M * c1.g.N;  // shard z's sums are their own block
      chunked_a = true;
    } else if (c1.g.batch == 1 && (int64_t)(r2.g.batch - 1) * r2.g.sA + r2.g.K <= c1.g.N) {
      ca.sz = r2.g.sA;  // one block holding every shard's columns
      chunked_a = true;
    }
    chunked_a = chunked_a && r2.g.M <= tp::kSkinnyMaxRows && tp::gemm_skinny_chunked_a_supported(r2.g, ca);
  }
  if (skinny1) {
    e = tp::launch_gemm_skinny(c1.g, ksplit, part, s);
    if (e == hipSuccess && ksplit > 1 && !chunked_a) e = tp::launch_skinny_finish(c1.g, ksplit, part, s);
  } else {
    e = run_gemm(c1.g, s);
  }
  if (e != hipSuccess) return TP_ERR_HIP;
  e = chunked_a ? tp::launch_gemm_skinny_chunked_a(r2.g, ca, s) : run_gemm(r2.g, s);
  if (e != hipSuccess) return TP_ERR_HIP;
  if (ns > 1) {
    CombineDesc cd;
    std::memset(&cd, 0, sizeof(cd));
    cd.P = Pm.ptr;
    cd.Y = Y->ptr;
    cd.rows = M;
    cd.cols = Dout;
    cd.ldp = Dout;
    cd.sP = Pm.shard_stride;
    cd.ldy = Y->ld;
    cd.n = ns;
    if ((e = tp::launch_combine(cd, s)) != hipSuccess) return TP_ERR_HIP;
  }
  return TP_OK;
}

tp_status tp_mlp_noalloc(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, int32_t N, int32_t s0,
                         int32_t ns, int32_t act, const tp_matrix* Y, void* stream) {
  // Shapes, dtypes and strides first (the size query enqueues nothing and needs no pointers).
  size_t need = 0;
  tp_status st = tp_mlp(X, W1, W2, N, s0, ns, act, nullptr, &need, Y, stream);
  if (st != TP_OK) return st;
  if (need > kScratchBytes) return TP_ERR_TOO_LARGE;
  void* ws = nullptr;
  if ((st = current_device_scratch(&ws)) != TP_OK) return st;
  size_t have = kScratchBytes;
  return tp_mlp(X, W1, W2, N, s0, ns, act, ws, &have, Y, stream);
}

size_t tp_mlp_noalloc_max_scratch(void) { return kScratchBytes; }

tp_status tp_col_linear_backward(const tp_matrix* X, const tp_matrix* W, const tp_matrix* dY, int32_t N,
                                 int32_t s0, int32_t ns, const tp_matrix* dXp, const tp_matrix* dW,
                                 void* stream) {
  if (!X || !W || !dY || (!dXp && !dW)) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W->dtype) || !valid_dtype(dY->dtype)) return TP_ERR_DTYPE;
  if (X->dtype != W->dtype || X->dtype != dY->dtype) return TP_ERR_DTYPE;
  if (dXp && dXp->dtype != TP_F32) return TP_ERR_DTYPE;
  if (dW && !valid_dtype(dW->dtype)) return TP_ERR_DTYPE;
  if (X->rows < 0 || X->cols < 0 || W->rows < 0 || W->cols < 0 || dY->rows < 0 || dY->cols < 0) return TP_ERR_SHAPE;
  if (N < 1 || W->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, K = X->cols, width = W->cols / N;
  if (W->rows != K || dY->rows != M || dY->cols != (int64_t)ns * width) return TP_ERR_SHAPE;
  if (dXp && (dXp->rows != M || dXp->cols != K)) return TP_ERR_SHAPE;
  if (dW && (dW->rows != K || dW->cols != (int64_t)ns * width)) return TP_ERR_SHAPE;
  if (X->shard_stride != 0) return TP_ERR_STRIDE;
  if (dXp && ns > 1 && dXp->shard_stride == 0 && M > 0 && K > 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(X, 1, M, K, K)) != TP_OK) return st;
  if ((st = check_matrix(W, ns, K, width, W->cols)) != TP_OK) return st;
  if ((st = check_matrix(dY, ns, M, width, dY->cols)) != TP_OK) return st;
  if (dXp && (st = check_matrix(dXp, ns, M, K, K)) != TP_OK) return st;
  if (dW && (st = check_matrix(dW, ns, K, width, dW->cols)) != TP_OK) return st;

  const bool bf16 = X->dtype == TP_BF16;
  const Blocks wb = col_blocks(W, s0, width), yb = col_blocks(dY, 0, width);
  const Range xr = range_of(X->ptr, X->dtype, 1, 0, M, K, X->ld);
  const Range wr = blocks_range(wb, ns, K, width), yr = blocks_range(yb, ns, M, width);
  Range pr, gr;
  if (dXp) {
    pr = range_of(dXp->ptr, dXp->dtype, ns, dXp->shard_stride, M, K, dXp->ld);
    if (overlaps(pr, xr) || overlaps(pr, wr) || overlaps(pr, yr)) return TP_ERR_ALIAS;
  }
  if (dW) {
    gr = blocks_range(col_blocks(dW, 0, width), ns, K, width);
    if (overlaps(gr, xr) || overlaps(gr, wr) || overlaps(gr, yr) || overlaps(gr, pr)) return TP_ERR_ALIAS;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dXp) {
    // P_j = dY_j W_s^T: W_s stored [K, width] is the transposed right operand
    const Blocks pb = buffer_blocks(dXp->ptr, TP_F32, dXp->ld, dXp->shard_stride);
    const GemmDesc g = product(yb, false, wb, true, pb, M, K, width, ns, bf16);
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  if (dW) {
    // dW_j = X^T dY_j: X stored [M, K] is the transposed left operand
    const Blocks gb = col_blocks(dW, 0, width);
    GemmDesc g = product(whole(X), true, yb, false, gb, K, width, M, ns, bf16);
    if (dY->shard_stride == 0 && dW->shard_stride == 0) {
      g.N = (int64_t)ns * width;  // side-by-side shards form one product
      g.batch = 1;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  return TP_OK;
}

tp_status tp_row_linear_backward(const tp_matrix* X, const tp_matrix* W, const tp_matrix* dY, int32_t N,
                                 int32_t s0, int32_t ns, const tp_matrix* dX, const tp_matrix* dW,
                                 void* stream) {
  if (!X || !W || !dY || (!dX && !dW)) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W->dtype) || !valid_dtype(dY->dtype)) return TP_ERR_DTYPE;
  if (X->dtype != W->dtype || X->dtype != dY->dtype) return TP_ERR_DTYPE;
  if ((dX && !valid_dtype(dX->dtype)) || (dW && !valid_dtype(dW->dtype))) return TP_ERR_DTYPE;
  if (X->rows < 0 || X->cols < 0 || W->rows < 0 || W->cols < 0 || dY->rows < 0 || dY->cols < 0) return TP_ERR_SHAPE;
  if (N < 1 || X->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, K = X->cols, kb = K / N, Nout = W->cols;
  if (W->rows != K || dY->rows != M || dY->cols != Nout) return TP_ERR_SHAPE;
  if (dX && (dX->rows != M || dX->cols != (int64_t)ns * kb)) return TP_ERR_SHAPE;
  if (dW && (dW->rows != (int64_t)ns * kb || dW->cols != Nout)) return TP_ERR_SHAPE;
  if (dY->shard_stride != 0) return TP_ERR_STRIDE;
  tp_status st;
  if ((st = check_matrix(X, ns, M, kb, K)) != TP_OK) return st;
  if ((st = check_matrix(W, ns, kb, Nout, Nout)) != TP_OK) return st;
  if ((st = check_matrix(dY, 1, M, Nout, Nout)) != TP_OK) return st;
  if (dX && (st = check_matrix(dX, ns, M, kb, dX->cols)) != TP_OK) return st;
  if (dW && (st = check_matrix(dW, ns, kb, Nout, Nout)) != TP_OK) return st;

  const bool bf16 = X->dtype == TP_BF16;
  const Blocks xb = col_blocks(X, s0, kb), wb = row_blocks(W, s0, kb);
  const Range xr = blocks_range(xb, ns, M, kb), wr = blocks_range(wb, ns, kb, Nout);
  const Range yr = range_of(dY->ptr, dY->dtype, 1, 0, M, Nout, dY->ld);
  Range ar, gr;
  if (dX) {
    ar = blocks_range(col_blocks(dX, 0, kb), ns, M, kb);
    if (overlaps(ar, xr) || overlaps(ar, wr) || overlaps(ar, yr)) return TP_ERR_ALIAS;
  }
  if (dW) {
    gr = blocks_range(row_blocks(dW, 0, kb), ns, kb, Nout);
    if (overlaps(gr, xr) || overlaps(gr, wr) || overlaps(gr, yr) || overlaps(gr, ar)) return TP_ERR_ALIAS;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dX) {
    // dX_j = dY W_s^T: W_s stored [kb, Nout] is the transposed right operand
    GemmDesc g = product(whole(dY), false, wb, true, col_blocks(dX, 0, kb), M, kb, Nout, ns, bf16);
    if (W->shard_stride == 0 && dX->shard_stride == 0) {
      g.N = (int64_t)ns * kb;  // consecutive row blocks of W give side-by-side blocks of dX
      g.batch = 1;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  if (dW) {
    // dW_j = X_s^T dY: X_s stored [M, kb] is the transposed left operand
    GemmDesc g = product(xb, true, whole(dY), false, row_blocks(dW, 0, kb), kb, Nout, M, ns, bf16);
    if (X->shard_stride == 0 && dW->shard_stride == 0) {
      g.M = (int64_t)ns * kb;  // side-by-side column blocks of X give stacked row blocks of dW
      g.batch = 1;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  return TP_OK;
}

tp_status tp_mlp_backward(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, const tp_matrix* dY,
                          int32_t N, int32_t s0, int32_t ns, int32_t act, void* workspace,
                          size_t* workspace_bytes, const tp_matrix* dX, const tp_matrix* dW1,
                          const tp_matrix* dW2, void* stream) {
  if (!X || !W1 || !W2 || !dY || !workspace_bytes || (!dX && !dW1 && !dW2)) return TP_ERR_NULL;
  if (!valid_dtype(X->dtype) || !valid_dtype(W1->dtype) || !valid_dtype(W2->dtype) || !valid_dtype(dY->dtype))
    return TP_ERR_DTYPE;
  if (X->dtype != W1->dtype || X->dtype != W2->dtype || X->dtype != dY->dtype) return TP_ERR_DTYPE;
  if (dX && dX->dtype != TP_F32) return TP_ERR_DTYPE;
  if ((dW1 && !valid_dtype(dW1->dtype)) || (dW2 && !valid_dtype(dW2->dtype))) return TP_ERR_DTYPE;
  if (act != TP_ACT_NONE && act != TP_ACT_GELU) return TP_ERR_SHAPE;
  if (X->rows < 0 || X->cols < 0 || W1->rows < 0 || W1->cols < 0 || W2->rows < 0 || W2->cols < 0 ||
      dY->rows < 0 || dY->cols < 0)
    return TP_ERR_SHAPE;
  if (N < 1 || W1->cols % N != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int64_t M = X->rows, d = X->cols, F = W1->cols, width = F / N, Dout = W2->cols;
  const int64_t hcols = (int64_t)ns * width;
  if (W1->rows != d || W2->rows != F || dY->rows != M || dY->cols != Dout) return TP_ERR_SHAPE;
  if (dX && (dX->rows != M || dX->cols != d)) return TP_ERR_SHAPE;
  if (dW1 && (dW1->rows != d || dW1->cols != hcols)) return TP_ERR_SHAPE;
  if (dW2 && (dW2->rows != hcols || dW2->cols != Dout)) return TP_ERR_SHAPE;
  if (X->shard_stride != 0 || dY->shard_stride != 0 || (dX && dX->shard_stride != 0)) return TP_ERR_STRIDE;
  const bool query = workspace == nullptr;
  tp_status st;
  if ((st = check_matrix(X, 1, M, d, d, !query)) != TP_OK) return st;
  if ((st = check_matrix(W1, ns, d, width, F, !query)) != TP_OK) return st;
  if ((st = check_matrix(W2, ns, width, Dout, Dout, !query)) != TP_OK) return st;
  if ((st = check_matrix(dY, 1, M, Dout, Dout, !query)) != TP_OK) return st;
  if (dX && (st = check_matrix(dX, 1, M, d, d, !query)) != TP_OK) return st;
  if (dW1 && (st = check_matrix(dW1, ns, d, width, hcols, !query)) != TP_OK) return st;
  if (dW2 && (st = check_matrix(dW2, ns, width, Dout, Dout, !query)) != TP_OK) return st;

  // Workspace, each part 256-byte aligned: Z (GeLU only), H, dZ (when dX or
  // dW1 is wanted), all [M, ns * width] in the input dtype with shard j at
  // column j * width; then the fp32 partials of dX [ns][M][d] when ns > 1.
  const bool bf16 = X->dtype == TP_BF16;
  const int32_t hdt = bf16 ? TP_BF16 : TP_F32;
  const bool gelu = act == TP_ACT_GELU;
  const bool need_dz = dX || dW1;
  const size_t bytes_hc = align_up((size_t)(M * hcols * elt_size(hdt)), 256);
  const size_t off_z = 0;
  const size_t off_h = off_z + (gelu ? bytes_hc : 0);
  const size_t off_dz = off_h + bytes_hc;
  const size_t off_p = off_dz + (need_dz ? bytes_hc : 0);
  const size_t bytes_p = dX && ns > 1 ? align_up((size_t)ns * M * d * sizeof(float), 256) : 0;
  const size_t need = off_p + bytes_p;
  if (query) {
    *workspace_bytes = need > 0 ? need : 256;
    return TP_OK;
  }
  if (*workspace_bytes < need) return TP_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  const Blocks w1b = col_blocks(W1, s0, width), w2b = row_blocks(W2, s0, width);
  const Range xr = range_of(X->ptr, X->dtype, 1, 0, M, d, X->ld);
  const Range yr = range_of(dY->ptr, dY->dtype, 1, 0, M, Dout, dY->ld);
  const Range w1r = blocks_range(w1b, ns, d, width), w2r = blocks_range(w2b, ns, width, Dout);
  const Range wsr{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + need};
  Range outs[3];
  int nout = 0;
  if (dX) outs[nout++] = range_of(dX->ptr, dX->dtype, 1, 0, M, d, dX->ld);
  if (dW1) outs[nout++] = blocks_range(col_blocks(dW1, 0, width), ns, d, width);
  if (dW2) outs[nout++] = blocks_range(row_blocks(dW2, 0, width), ns, width, Dout);
  if (overlaps(wsr, xr) || overlaps(wsr, yr) || overlaps(wsr, w1r) || overlaps(wsr, w2r)) return TP_ERR_ALIAS;
  for (int i = 0; i < nout; ++i) {
    if (overlaps(outs[i], xr) || overlaps(outs[i], yr) || overlaps(outs[i], w1r) || overlaps(outs[i], w2r) ||
        overlaps(outs[i], wsr))
      return TP_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return TP_ERR_ALIAS;
  }

  const hipStream_t s = static_cast<hipStream_t>(stream);
  // Shard j of Z, H and dZ: columns j * width of an [M, hcols] buffer.
  const Blocks zb = buffer_blocks(ws + off_z, hdt, hcols, width);
  const Blocks hb = buffer_blocks(ws + off_h, hdt, hcols, width);
  const Blocks dzb = buffer_blocks(ws + off_dz, hdt, hcols, width);
  const bool w1_contig = W1->shard_stride == 0, w2_contig = W2->shard_stride == 0;

  // 1. Recompute H_j = act(X W1_j), keeping Z_j for the GeLU derivative.
  {
    GemmDesc g = product(whole(X), false, w1b, false, hb, M, width, d, ns, bf16);
    g.sA = 0;
    if (w1_contig) {
      g.N = hcols;
      g.batch = 1;
    }
    if (gelu) {
      g.act = tp::ACT_GELU_SAVE;
      g.aux = ws + off_z;
      g.ldx = hcols;
      g.sX = g.batch > 1 ? width : 0;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  // 2. dZ_j = (dY W2_j^T) * act'(Z_j).
  if (need_dz) {
    GemmDesc g = product(whole(dY), false, w2b, true, dzb, M, width, Dout, ns, bf16);
    if (w2_contig) {
      g.N = hcols;
      g.batch = 1;
    }
    if (gelu) {
      g.act = tp::ACT_DGELU;
      g.aux = ws + off_z;
      g.ldx = hcols;
      g.sX = g.batch > 1 ? width : 0;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  // 3. dW2_j = H_j^T dY.
  if (dW2) {
    GemmDesc g = product(hb, true, whole(dY), false, row_blocks(dW2, 0, width), width, Dout, M, ns, bf16);
    if (dW2->shard_stride == 0) {
      g.M = hcols;
      g.batch = 1;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  // 4. dX = sum_j dZ_j W1_j^T: fp32 partials, then the fixed-order sum.
  if (dX) {
    const Blocks pb = ns > 1 ? buffer_blocks(ws + off_p, TP_F32, d, M * d) : buffer_blocks(dX->ptr, TP_F32, dX->ld, 0);
    const GemmDesc g = product(dzb, false, w1b, true, pb, M, d, width, ns, bf16);
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
    if (ns > 1) {
      CombineDesc cd;
      std::memset(&cd, 0, sizeof(cd));
      cd.P = ws + off_p;
      cd.Y = dX->ptr;
      cd.rows = M;
      cd.cols = d;
      cd.ldp = d;
      cd.sP = M * d;
      cd.ldy = dX->ld;
      cd.n = ns;
      if (tp::launch_combine(cd, s) != hipSuccess) return TP_ERR_HIP;
    }
  }
  // 5. dW1_j = X^T dZ_j.
  if (dW1) {
    GemmDesc g = product(whole(X), true, dzb, false, col_blocks(dW1, 0, width), d, width, M, ns, bf16);
    if (dW1->shard_stride == 0) {
      g.N = hcols;
      g.batch = 1;
    }
    if (run_gemm(g, s) != hipSuccess) return TP_ERR_HIP;
  }
  return TP_OK;
}

tp_status tp_attention(const tp_matrix* QKV, int32_t N, int32_t s0, int32_t ns, int32_t heads, int32_t kv_heads,
                       int32_t head_dim, int64_t seq_len, int32_t causal, const tp_matrix* A, void* stream) {
  if (!QKV || !A) return TP_ERR_NULL;
  if (!valid_dtype(QKV->dtype) || !valid_dtype(A->dtype)) return TP_ERR_DTYPE;
  if (QKV->dtype != A->dtype) return TP_ERR_DTYPE;
  if (QKV->rows < 0 || QKV->cols < 0 || A->rows < 0 || A->cols < 0) return TP_ERR_SHAPE;
  if (heads < 1 || kv_heads < 1 || head_dim < 1 || seq_len < 1 || (causal != 0 && causal != 1)) return TP_ERR_SHAPE;
  if (heads % kv_heads != 0) return TP_ERR_SHAPE;
  if (N < 1 || heads % N != 0) return TP_ERR_INDIVISIBLE;
  // key/value heads are split evenly, or (fewer than shards) replicated evenly
  if (kv_heads >= N ? kv_heads % N != 0 : N % kv_heads != 0) return TP_ERR_INDIVISIBLE;
  if (s0 < 0 || ns < 1 || (int64_t)s0 + ns > N) return TP_ERR_SHARD_RANGE;
  const int32_t hq = heads / N, hkv = kv_heads >= N ? kv_heads / N : 1;
  if (hq % hkv != 0) return TP_ERR_INDIVISIBLE;
  const int64_t M = QKV->rows;
  const int64_t blk = (int64_t)(hq + 2 * hkv) * head_dim, oblk = (int64_t)hq * head_dim;
  if (QKV->cols != (int64_t)ns * blk || A->rows != M || A->cols != (int64_t)ns * oblk) return TP_ERR_SHAPE;
  if (M % seq_len != 0) return TP_ERR_SHAPE;
  // the launch grid has one row per executed head and one layer per sequence
  if ((int64_t)hq * ns > 65535 || M / seq_len > 65535) return TP_ERR_TOO_LARGE;
  tp_status st;
  if ((st = check_matrix(QKV, ns, M, blk, QKV->cols)) != TP_OK) return st;
  if ((st = check_matrix(A, ns, M, oblk, A->cols)) != TP_OK) return st;
  const Blocks qb = col_blocks(QKV, 0, blk), ab = col_blocks(A, 0, oblk);
  if (overlaps(blocks_range(ab, ns, M, oblk), blocks_range(qb, ns, M, blk))) return TP_ERR_ALIAS;
  tp::AttnDesc a;
  std::memset(&a, 0, sizeof(a));
  a.qkv = qb.base;
  a.ld_qkv = qb.ld;
  a.s_qkv = qb.step;
  a.out = const_cast<char*>(ab.base);
  a.ld_out = ab.ld;
  a.s_out = ab.step;
  a.tokens = M;
  a.seq_len = seq_len;
  a.hq = hq;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.shards = ns;
  a.causal = causal;
  a.in_bf16 = QKV->dtype == TP_BF16;
  a.scale = 1.0f / std::sqrt((float)head_dim);
  if (M == 0) return TP_OK;
  if (!tp::attention_mfma_supported(a) && !tp::attention_generic_supported(a)) return TP_ERR_TOO_LARGE;
  return hip_status(tp::launch_attention(a, static_cast<hipStream_t>(stream)));
}

const char* tp_status_string(int32_t status) {
  switch (status) {
    case TP_OK: return "TP_OK";
    case TP_ERR_NULL: return "TP_ERR_NULL: a descriptor, data pointer or out-parameter is NULL";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unsupported or mismatched dtype";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE: shapes do not chain or a size is negative";
    case TP_ERR_INDIVISIBLE: return "TP_ERR_INDIVISIBLE: the shard count must be >= 1 and divide the split dimension";
    case TP_ERR_SHARD_RANGE: return "TP_ERR_SHARD_RANGE: need 0 <= s0, 1 <= ns, s0 + ns <= N";
    case TP_ERR_STRIDE: return "TP_ERR_STRIDE: leading dimension or shard stride too small";
    case TP_ERR_ALIAS: return "TP_ERR_ALIAS: an output overlaps an input";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_HIP: return "TP_ERR_HIP: a HIP launch failed";
    case TP_ERR_TOO_LARGE: return "TP_ERR_TOO_LARGE: a size exceeds the kernels' limits";
    default: return "unknown tp_status";
  }
}

int32_t tp_version(void) { return (1 << 16) | 1; }  // 1.1: sequence-parallel LayerNorm, token stacking

}  // extern "C"
