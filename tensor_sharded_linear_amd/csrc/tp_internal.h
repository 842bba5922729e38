// Internal launch descriptors shared by the host dispatcher and the HIP kernels.
// Nothing here is part of the public interface (include/tp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1 };
enum ActKind : int { ACT_NONE = 0, ACT_GELU = 1 };

// A batch of `batch` independent products C_z = act(A_z * B_z), z = 0..batch-1,
// each A_z [M, K] (row stride lda), B_z [K, N] (row stride ldb), C_z [M, N]
// (row stride ldc), with A_z = A + z * sA elements and likewise for B and C.
// For the sharded layers z is the shard index within the executed range.
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
  int32_t concat;    // 1: Y = [P_0 | ... | P_{n-1}], 0: Y = sum
};

// Large-tile bf16 matrix-core GEMM. Requirements checked by the caller
// (gemm_mfma_supported): bf16 inputs, K, N, lda, ldb, sA, sB multiples of 8,
// 16-byte aligned A and B.
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

// Element-guarded GEMM for any dtype, alignment and shape.
hipError_t launch_gemm_generic(const GemmDesc& d, hipStream_t stream);

hipError_t launch_combine(const CombineDesc& d, hipStream_t stream);

}  // namespace tp
