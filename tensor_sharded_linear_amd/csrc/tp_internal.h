// Internal launch descriptors shared by the host dispatcher and the HIP kernels.
// Nothing here is part of the public interface (include/tp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1 };
// Epilogue applied to the fp32 accumulator v of output (m, n):
//   ACT_NONE       C = v
//   ACT_GELU       C = GeLU(v)
//   ACT_GELU_SAVE  C = GeLU(v) and aux = v (bf16): the forward of the MLP's
//                  first product, keeping the pre-activation for the backward
//   ACT_DGELU      C = v * GeLU'(aux[m][n]) with aux bf16: the backward of GeLU
enum ActKind : int { ACT_NONE = 0, ACT_GELU = 1, ACT_GELU_SAVE = 2, ACT_DGELU = 3 };

// A batch of `batch` independent products C_z = act(op(A_z) * op(B_z)),
// z = 0..batch-1, with op(A_z) [M, K], op(B_z) [K, N] and C_z [M, N] (row
// stride ldc); A_z = A + z * sA elements and likewise for B, C and aux.
// Storage is row-major: A_z is [M, K] with row stride lda, or [K, M] when
// a_trans; B_z is [K, N] with row stride ldb, or [N, K] when b_trans. The
// backward products use the transposed forms: dX = dY W^T (b_trans) and
// dW = X^T dY (a_trans). For the sharded layers z is the shard index within
// the executed range.
struct GemmDesc {
  const void* A;
  const void* B;
  void* C;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  int64_t M, N, K;
  int32_t batch;
  int32_t in_bf16;   // 1: A and B are bf16, 0: fp32
  int32_t out_kind;  // OutKind
  int32_t act;       // ActKind
  int32_t a_trans;   // 1: A stored [K, M]
  int32_t b_trans;   // 1: B stored [N, K]
  void* aux;         // [M, N] per z in the input dtype (row stride ldx, z stride sX):
                     // ACT_GELU_SAVE output, ACT_DGELU input
  int64_t ldx, sX;
};

// Sum or concatenation of n fp32 / bf16 blocks [rows, cols] (see tp_reduce_partials).
struct CombineDesc {
  const void* P;
  void* Y;
  int64_t rows, cols;
  int64_t ldp, sP;  // row stride and block stride of P, elements
  int64_t ldy;
  int32_t n;
  int32_t p_bf16;    // P dtype (COLS mode only)
  int32_t y_bf16;    // Y dtype
  int32_t concat;    // 0: Y = sum; 1: Y = [P_0 | ... | P_{n-1}]; 2: Y = the blocks stacked by rows
};

// GeLU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, applied to the fp32
// accumulators of the column-parallel product before its single rounding.
// erf follows Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (|error| <= 1.5e-7): for u = |x| / sqrt 2 and t = 1 / (1 + p u),
// 1 - erf(u) = q = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2). Then
// Phi(x) = 1 - q / 2 for x >= 0 and q / 2 for x < 0, which also avoids the
// cancellation of 1 + erf at negative x. One reciprocal and one exp2 on the
// transcendental unit, the rest fused multiply-adds: about half the work of
// the library erff, which matters because the whole output tile of the
// column-parallel product passes through it. In fp32 the result is within
// 4.3e-7 of the exact GeLU at every x, no further than the form
// 0.5 x (1 + erf) is with a correctly rounded fp32 erf (4.5e-7).
__device__ __forceinline__ float gelu(float x) {
  const float u = __builtin_fabsf(x) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, u, 1.0f));
  float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  p *= t;
  // exp(-u^2) = exp(-x^2 / 2) = 2^(-x^2 log2(e) / 2)
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170368f);
  const float hq = 0.5f * p * e;
  return x * (x >= 0.0f ? 1.0f - hq : hq);
}

// Derivative of the GeLU above: GeLU'(x) = Phi(x) + x phi(x), phi the standard
// normal density exp(-x^2 / 2) / sqrt(2 pi); Phi and exp(-x^2 / 2) come from
// the same Abramowitz & Stegun evaluation.
__device__ __forceinline__ float gelu_grad(float x) {
  const float u = __builtin_fabsf(x) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, u, 1.0f));
  float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170368f);
  const float hq = 0.5f * p * e;
  const float cdf = x >= 0.0f ? 1.0f - hq : hq;
  return __builtin_fmaf(x * 0.39894228040143267794f, e, cdf);
}

// Large-tile bf16 matrix-core GEMM. Requirements checked by the caller
// (gemm_mfma_supported): bf16 inputs, K, N, lda, ldb, sA, sB multiples of 8
// (and M when a_trans), 16-byte aligned A and B.
bool gemm_mfma_supported(const GemmDesc& d);
hipError_t launch_gemm_mfma(const GemmDesc& d, hipStream_t stream);

// Skinny bf16 GEMM for few rows (M <= kSkinnyMaxRows): streams B once with
// every CU busy. ksplit > 1 writes fp32 partial sums of K-chunks to `part`
// (layout [ksplit][batch][M][N]) that a combine pass finishes.
constexpr int kSkinnyMaxRows = 32;
bool gemm_skinny_supported(const GemmDesc& d);
int skinny_ksplit(const GemmDesc& d);
size_t skinny_partial_bytes(const GemmDesc& d, int ksplit);
hipError_t launch_gemm_skinny(const GemmDesc& d, int ksplit, float* part, hipStream_t stream);
// C_z = act(sum_c part[c][z]) for the ksplit chunk sums written above.
hipError_t launch_skinny_finish(const GemmDesc& d, int ksplit, const float* part, hipStream_t stream);
// The next skinny product reading such chunk sums directly as its A operand:
// C_z = A'_z B_z with A'_z(m, k) = bf16(act(sum_c part[c cs + z sz + m ld + k])),
// c in ascending order, exactly what launch_skinny_finish would have stored
// for A. Taken for kChunkedA chunks, M <= 16, fp32 output and no epilogue
// activation of its own (d.A is not read).
constexpr int kChunkedA = 2;
struct ChunkedA {
  const float* part;
  int64_t cs, sz, ld;  // chunk, batch and row strides of part, elements
  int32_t ksplit;
  int32_t act;         // ACT_NONE or ACT_GELU
};
bool gemm_skinny_chunked_a_supported(const GemmDesc& d, const ChunkedA& a);
hipError_t launch_gemm_skinny_chunked_a(const GemmDesc& d, const ChunkedA& a, hipStream_t stream);

// Element-guarded GEMM for any dtype, alignment and shape.
hipError_t launch_gemm_generic(const GemmDesc& d, hipStream_t stream);

hipError_t launch_combine(const CombineDesc& d, hipStream_t stream);

// Sequence-parallel LayerNorm over token rows (see tp_sp_layernorm). Row i of
// the executed token rows (token shard j = i / rows_per_shard, row
// r = i % rows_per_shard within it): x = R_j[r] + keep[i] * sum_{t<n} P_t[i]
// * keep_scale (keep and R optional), X1_j[r] = x (optional), Y_j[r] =
// (x - mean) / sqrt(var + eps) * gamma + beta. P_t[i] is P + t * sP + i * ldp;
// the per-shard matrices R, X1 and Y hold shard j at j * s elements.
struct LnDesc {
  const float* P;
  int64_t ldp, sP;
  int32_t n;
  const void* R;
  int64_t ldr, sR;
  int32_t r_bf16;
  const uint8_t* keep;  // [rows, cols] 0/1 bytes, row stride cols
  float keep_scale;     // 1 / (1 - p)
  const float* gamma;
  const float* beta;
  float eps;
  float* X1;
  int64_t ldx1, sX1;
  void* Y;
  int64_t ldy, sY;
  int32_t y_bf16;
  int64_t rows_per_shard;
  int64_t rows, cols;
};
hipError_t launch_sp_layernorm(const LnDesc& d, hipStream_t stream);

// Attention over the heads of `shards` executed shards (see tp_attention):
// shard j's QKV block [tokens, (hq + 2 hkv) head_dim] starts s_qkv elements
// after block j-1 (row stride ld_qkv) and its output block [tokens, hq
// head_dim] s_out elements after block j-1 (row stride ld_out).
struct AttnDesc {
  const void* qkv;
  void* out;
  int64_t ld_qkv, s_qkv;
  int64_t ld_out, s_out;
  int64_t tokens, seq_len;
  int32_t hq, hkv, head_dim, shards;
  int32_t causal, in_bf16;
  float scale;  // applied to the scores: 1 / sqrt(head_dim)
};
bool attention_mfma_supported(const AttnDesc& a);
bool attention_generic_supported(const AttnDesc& a);
hipError_t launch_attention(const AttnDesc& a, hipStream_t stream);

}  // namespace tp
