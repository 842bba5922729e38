// Element-guarded GEMM for any dtype (fp32 or bf16 inputs), alignment and shape:
// C_z = act(op(A_z) op(B_z)) with fp32 multiply-add in ascending k for every
// output; either operand may be stored transposed.
//
// It serves the exact fp32 path (integer-valued inputs give exact results, as
// in the worked example of the "Tensor Parallelism" entry of the AI Glossary,
// aiforbusinessandlife.com, section "Worked example") and bf16 operands whose
// strides or pointers do not meet the 16-byte needs of the matrix-core kernels.
#include "tp_internal.h"

namespace tp {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <typename T>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
  return (float)static_cast<const T*>(p)[i];
}

template <typename T, int OUT, int ACT>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmDesc d, int tiles_n) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t z = blockIdx.y;
  const int64_t m0 = (int64_t)tm * TM, n0 = (int64_t)tn * TN;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t abase = z * d.sA, bbase = z * d.sB;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int64_t k0 = 0; k0 < d.K; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / TK, kk = e % TK;  // A tile: 64 rows x 16 k
      const int64_t gm = m0 + r, gk = k0 + kk;
      const int64_t ai = d.a_trans ? gk * d.lda + gm : gm * d.lda + gk;
      As[kk][r] = (gm < d.M && gk < d.K) ? ld_elem<T>(d.A, abase + ai) : 0.f;
      const int kb = e / TN, c = e % TN;  // B tile: 16 k x 64 columns
      const int64_t gkb = k0 + kb, gn = n0 + c;
      const int64_t bi = d.b_trans ? gn * d.ldb + gkb : gkb * d.ldb + gn;
      Bs[kb][c] = (gkb < d.K && gn < d.N) ? ld_elem<T>(d.B, bbase + bi) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gm = m0 + ty + 16 * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = n0 + tx + 16 * j;
      if (gm < d.M && gn < d.N) {
        float v = acc[i][j];
        const int64_t xo = z * d.sX + gm * d.ldx + gn;  // the side matrix has the input dtype
        if (ACT == ACT_GELU_SAVE) static_cast<T*>(d.aux)[xo] = (T)v;
        if (ACT == ACT_GELU || ACT == ACT_GELU_SAVE) v = gelu(v);
        if (ACT == ACT_DGELU) v *= gelu_grad((float)static_cast<const T*>(d.aux)[xo]);
        const int64_t off = z * d.sC + gm * d.ldc + gn;
        if (OUT == OUT_F32) static_cast<float*>(d.C)[off] = v;
        else static_cast<__bf16*>(d.C)[off] = (__bf16)v;
      }
    }
  }
}

template <typename T, int OUT>
hipError_t launch_act(const GemmDesc& d, dim3 grid, int tiles_n, hipStream_t s) {
  const dim3 block(256);
  switch (d.act) {
    case ACT_NONE: gemm_generic_kernel<T, OUT, ACT_NONE><<<grid, block, 0, s>>>(d, tiles_n); break;
    case ACT_GELU: gemm_generic_kernel<T, OUT, ACT_GELU><<<grid, block, 0, s>>>(d, tiles_n); break;
    case ACT_GELU_SAVE: gemm_generic_kernel<T, OUT, ACT_GELU_SAVE><<<grid, block, 0, s>>>(d, tiles_n); break;
    case ACT_DGELU: gemm_generic_kernel<T, OUT, ACT_DGELU><<<grid, block, 0, s>>>(d, tiles_n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const GemmDesc& d, dim3 grid, int tiles_n, hipStream_t s) {
  return d.out_kind == OUT_F32 ? launch_act<T, OUT_F32>(d, grid, tiles_n, s)
                               : launch_act<T, OUT_BF16>(d, grid, tiles_n, s);
}

}  // namespace

hipError_t launch_gemm_generic(const GemmDesc& d, hipStream_t stream) {
  const int64_t tiles_m = (d.M + TM - 1) / TM, tiles_n = (d.N + TN - 1) / TN;
  if (tiles_m * tiles_n <= 0 || d.batch <= 0) return hipSuccess;
  if (tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
  // the batch index is the grid's second dimension: more than 65535 entries go in several launches
  const int64_t in_elt = d.in_bf16 ? 2 : 4, out_elt = d.out_kind == OUT_F32 ? 4 : 2;
  for (int64_t z0 = 0; z0 < d.batch; z0 += 65535) {
    GemmDesc c = d;
    c.batch = (int32_t)(d.batch - z0 < 65535 ? d.batch - z0 : 65535);
    c.A = static_cast<const char*>(d.A) + z0 * d.sA * in_elt;
    c.B = static_cast<const char*>(d.B) + z0 * d.sB * in_elt;
    c.C = static_cast<char*>(d.C) + z0 * d.sC * out_elt;
    if (d.aux) c.aux = static_cast<char*>(d.aux) + z0 * d.sX * in_elt;
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)c.batch);
    const hipError_t e = d.in_bf16 ? launch_typed<__bf16>(c, grid, (int)tiles_n, stream)
                                   : launch_typed<float>(c, grid, (int)tiles_n, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tp
