// Large-tile bf16 GEMM on the gfx950 matrix cores: C_z = act(A_z B_z), fp32 accumulate.
//
// This is the per-shard dense product of the sharded linear layer ("Tensor
// Parallelism" topic page, chipfoundryservices.com, sections "Column-Wise
// Parallelism" and "Row-Wise Parallelism": each shard multiplies its input by
// its block of W). All shards of one call form one launch: either one wide
// product (column shards stored side by side) or a batch indexed by shard.
//
// Tile 256 x 256 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave owns a
// 128 x 128 block of C held as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators.
// A (row-major, K contiguous) and B (row-major, N contiguous, the pages'
// [in, out] weight) are staged through LDS in two buffers. A fragments are
// read with ds_read_b128; B fragments need K-contiguous lanes, which gfx950
// provides directly with the LDS transpose read ds_read_b64_tr_b16.
// Global loads use buffer resources so that rows past M and K read as zero.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int A_TILE = BM * BK;  // elements per LDS stage
constexpr int B_TILE = BK * BN;
constexpr int GROUP_M = 8;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

struct Params {
  GemmDesc d;
  int tiles_m, tiles_n, total;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

// Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
// range of logical tiles so the tiles that share A rows and B columns share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  int x, i;
  if (bid < (q << 3)) {
    x = bid & 7;
    i = bid >> 3;
  } else {
    x = bid - (q << 3);
    i = q;
  }
  return x * q + min(x, r) + i;
}

// LDS swizzles (16-byte chunk granularity) that keep the fragment reads free
// of bank conflicts: A rows are 64 elements = 8 chunks; B rows 256 elements = 32 chunks.
__device__ __forceinline__ int swz_a(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_b(int krow) { return ((krow & 1) * 6) ^ (((krow >> 1) & 1) * 12); }

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

template <int OUT, int ACT>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_mfma_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (A_TILE + B_TILE)];
  __bf16* As = smem;                // [2][BM][BK]
  __bf16* Bs = smem + 2 * A_TILE;   // [2][BK][BN]

  const GemmDesc& d = p.d;
  const int logical = xcd_remap(blockIdx.x, p.total);
  const int per_batch = p.tiles_m * p.tiles_n;
  const int z = logical / per_batch;
  const int u = logical - z * per_batch;
  const int in_group = GROUP_M * p.tiles_n;
  const int g = u / in_group;
  const int first_m = g * GROUP_M;
  const int gm = min(p.tiles_m - first_m, GROUP_M);
  const int ug = u - g * in_group;
  const int tm = first_m + ug % gm;
  const int tn = ug / gm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t M = d.M, N = d.N, K = d.K;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t lda = d.lda, ldb = d.ldb;

  const __bf16* Az = static_cast<const __bf16*>(d.A) + z * d.sA + m0 * lda;
  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB + n0;

  // Global chunk assignment (16 bytes = 8 elements per chunk).
  // A: chunk c = tid + 256 i -> row (tid >> 3) + 32 i, k-chunk tid & 7.
  // B: chunk c = tid + 256 i -> k-row (tid >> 5) + 8 i, n-chunk tid & 31.
  const int a_row0 = tid >> 3, a_kc = tid & 7;
  const int b_row0 = tid >> 5, b_nc = tid & 31;
  uint32_t a_voff[8], b_voff[8];
  int a_lds[8], b_lds[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ar = a_row0 + 32 * i;
    a_voff[i] = (uint32_t)(ar * lda * 2 + a_kc * 16);
    a_lds[i] = ar * BK + ((a_kc ^ swz_a(ar)) << 3);
    const int br = b_row0 + 8 * i;
    b_voff[i] = (uint32_t)(br * ldb * 2 + b_nc * 16);
    b_lds[i] = br * BN + ((b_nc ^ swz_b(br)) << 3);
  }

  const int KT = (int)((K + BK - 1) / BK);
  u32x4 ra[8], rb[8];

  auto load_tile = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(Az + k0, ((M - m0 - 1) * lda + (K - k0)) * 2);
    const __amdgpu_buffer_rsrc_t brsrc = make_rsrc(Bz + k0 * ldb, ((K - k0 - 1) * ldb + (N - n0)) * 2);
    const bool a_ok = k0 + a_kc * 8 < K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_voff[i], 0, 0);
      ra[i] = a_ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[i] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, b_voff[i], 0, 0);
  };
  auto store_tile = [&](int buf) {
    __bf16* a = As + buf * A_TILE;
    __bf16* b = Bs + buf * B_TILE;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(a + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(b + b_lds[i]) = rb[i];
  };

  // Per-lane fragment addressing.
  // A fragment (32 rows x 16 k): lane holds row (lane & 31), k-chunk 2 kk + (lane >> 5).
  // B fragment via transpose reads: lane (G = lane >> 4, j = lane & 15) supplies
  // k-row 8 (G >> 1) + 4 t + (j >> 2) and columns 16 (G & 1) + 4 (j & 3) .. + 3
  // of the 32-column block; it receives 4 k-values of column 16 (G & 1) + j.
  const int a_r = lane & 31, a_h = lane >> 5;
  const int G = lane >> 4, j16 = lane & 15;
  const int b_kr = 8 * (G >> 1) + (j16 >> 2);
  const int b_col = 16 * (G & 1) + 4 * (j16 & 3);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;

  if (KT > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const __bf16* a = As + cur * A_TILE;
    const __bf16* b = Bs + cur * B_TILE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int im = 0; im < 4; ++im) {
        const int row = wm * 128 + im * 32 + a_r;
        const int kc = kk * 2 + a_h;
        af[im] = *reinterpret_cast<const bf16x8*>(a + row * BK + ((kc ^ swz_a(row)) << 3));
      }
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const int col = wn * 128 + jn * 32 + b_col;
        bf16x4 lo, hi;
        {
          const int kr = kk * 16 + b_kr;
          const int off = kr * BN + ((((col >> 3) ^ swz_b(kr))) << 3) + (col & 4);
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(b + off));
        }
        {
          const int kr = kk * 16 + b_kr + 4;
          const int off = kr * BN + ((((col >> 3) ^ swz_b(kr))) << 3) + (col & 4);
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(b + off));
        }
        bfr[jn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int im = 0; im < 4; ++im)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
          acc[im][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[im], bfr[jn], acc[im][jn], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator element e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32 of its 32 x 32 block.
  const int64_t ldc = d.ldc;
#pragma unroll
  for (int im = 0; im < 4; ++im) {
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int64_t col = n0 + wn * 128 + jn * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + im * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        float v = acc[im][jn][e];
        if (ACT == ACT_GELU) v = gelu_erf(v);
        if (row < M && col < N) {
          if (OUT == OUT_F32) {
            static_cast<float*>(d.C)[z * d.sC + row * ldc + col] = v;
          } else {
            static_cast<__bf16*>(d.C)[z * d.sC + row * ldc + col] = (__bf16)v;
          }
        }
      }
    }
  }
}

}  // namespace

bool gemm_mfma_supported(const GemmDesc& d) {
  if (!d.in_bf16) return false;
  if ((d.K & 7) || (d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  // 32-bit in-tile offsets: 256 rows of A and 64 rows of B from the tile origin.
  if ((int64_t)BM * d.lda * 2 >= (1ll << 31) || (int64_t)BK * d.ldb * 2 >= (1ll << 31)) return false;
  return true;
}

hipError_t launch_gemm_mfma(const GemmDesc& d, hipStream_t stream) {
  Params p;
  p.d = d;
  p.tiles_m = (int)((d.M + BM - 1) / BM);
  p.tiles_n = (int)((d.N + BN - 1) / BN);
  const int64_t total = (int64_t)p.tiles_m * p.tiles_n * d.batch;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  p.total = (int)total;
  dim3 grid((unsigned)total), block(NTHREADS);
  if (d.out_kind == OUT_F32) {
    if (d.act == ACT_GELU) gemm_bf16_mfma_kernel<OUT_F32, ACT_GELU><<<grid, block, 0, stream>>>(p);
    else gemm_bf16_mfma_kernel<OUT_F32, ACT_NONE><<<grid, block, 0, stream>>>(p);
  } else {
    if (d.act == ACT_GELU) gemm_bf16_mfma_kernel<OUT_BF16, ACT_GELU><<<grid, block, 0, stream>>>(p);
    else gemm_bf16_mfma_kernel<OUT_BF16, ACT_NONE><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace tp
