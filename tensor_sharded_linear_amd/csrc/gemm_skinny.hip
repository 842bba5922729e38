// Skinny bf16 GEMM for a few rows (decode-shaped tensor-parallel layers):
// C_z = act(A_z B_z) with M <= 32, fp32 accumulate, on the gfx950 matrix cores.
//
// With so few rows the product is bound by streaming B (the weight shard)
// from HBM once. Each workgroup owns 64 columns of one shard and a chunk of
// K; its four waves take interleaved 32-row slices of every 128-row block,
// multiply them with v_mfma_f32_16x16x32_bf16 (16 rows of A per tile), and
// the four wave results are added in a fixed order at the end. B blocks are
// staged through LDS and read back K-contiguous with ds_read_b64_tr_b16.
// Splitting K over workgroups (ksplit > 1) keeps every CU streaming when a
// shard has few column tiles; the chunk sums are then finished by
// skinny_finish_kernel in ascending chunk order.
//
// The sharded layers follow the "Tensor Parallelism" topic page
// (chipfoundryservices.com), sections "Column-Wise Parallelism" and
// "Row-Wise Parallelism"; the serving use of the decode shape is the
// "Three practical examples" item on model serving of the AI Glossary entry.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int SBN = 64;    // columns per workgroup
constexpr int SBK = 128;   // k-rows per block (4 waves x 32)
constexpr int NTHREADS = 256;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

struct SkParams {
  GemmDesc d;
  int64_t kchunk;
  float* part;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: the four rows read by one
// 16-lane transpose group, and rows eight apart, land in distinct bank groups.
__device__ __forceinline__ int swz(int r) { return 2 * ((r & 3) ^ ((r >> 3) & 1)); }

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

template <int MT, int OUT, int ACT, bool PARTIAL>
__global__ __launch_bounds__(NTHREADS) void gemm_skinny_kernel(SkParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * SBK * SBN];  // 32 KB
  const GemmDesc& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * SBN;
  const int z = blockIdx.y;
  const int c = blockIdx.z;
  const int64_t M = d.M, N = d.N, K = d.K, lda = d.lda, ldb = d.ldb;
  const int64_t kbeg = (int64_t)c * p.kchunk;
  const int64_t kend = min(K, kbeg + p.kchunk);
  const int nblocks = kend > kbeg ? (int)((kend - kbeg + SBK - 1) / SBK) : 0;

  const __bf16* Az = static_cast<const __bf16*>(d.A) + z * d.sA;
  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB + n0;
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(Az, ((M - 1) * lda + K) * 2);

  // B chunk assignment: chunk tid + 256 i -> k-row (tid >> 3) + 32 i, n-chunk tid & 7.
  const int b_row0 = tid >> 3, b_nc = tid & 7;
  uint32_t b_voff[4];
  int b_lds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = b_row0 + 32 * i;
    b_voff[i] = (uint32_t)(r * ldb * 2 + b_nc * 16);
    b_lds[i] = r * SBN + ((b_nc ^ swz(r)) << 3);
  }
  // A fragment: lane holds row (lane & 15) + 16 mt, 8 k-values at 8 (lane >> 4).
  const int a_m = lane & 15, a_k = 8 * (lane >> 4);
  // B fragment via transpose reads: 16-lane group G = lane >> 4 takes k-rows
  // 8 G + 4 t .. + 3 of the wave's 32-row slice; lane j = lane & 15 supplies
  // row + (j >> 2), columns 4 (j & 3) .. + 3 and receives column j.
  const int G = lane >> 4, j16 = lane & 15;
  const int tr_row = 32 * wave + 8 * G + (j16 >> 2);
  const int tr_col = 4 * (j16 & 3);

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[mt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 rb[4];
  auto load_b = [&](int blk) {
    const int64_t k0 = kbeg + (int64_t)blk * SBK;
    const __amdgpu_buffer_rsrc_t brsrc = make_rsrc(Bz + k0 * ldb, ((K - k0 - 1) * ldb + (N - n0)) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, b_voff[i], 0, 0);
  };

  if (nblocks > 0) load_b(0);
  for (int blk = 0; blk < nblocks; ++blk) {
    __bf16* buf = smem + (blk & 1) * (SBK * SBN);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(buf + b_lds[i]) = rb[i];
    if (blk + 1 < nblocks) load_b(blk + 1);
    const int64_t ka = kbeg + (int64_t)blk * SBK + 32 * wave + a_k;
    bf16x8 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t off = (uint32_t)(((a_m + 16 * mt) * lda + ka) * 2);
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0, 0);
      af[mt] = __builtin_bit_cast(bf16x8, ka < K ? v : u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 16 * s + tr_col;
      const int r0 = tr_row, r1 = tr_row + 4;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_t*)(buf + r0 * SBN + (((col >> 3) ^ swz(r0)) << 3) + (col & 4)));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_t*)(buf + r1 * SBN + (((col >> 3) ^ swz(r1)) << 3) + (col & 4)));
      const bf16x8 bfr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr, acc[mt][s], 0, 0, 0);
    }
  }

  // Add the four waves' partial sums in wave order through LDS.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [4][MT * 16][64]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * MT * 16 + mt * 16 + 4 * (lane >> 4) + i) * SBN + 16 * s + (lane & 15)] = acc[mt][s][i];
  __syncthreads();
  const int col = tid & 63;
  const int64_t gn = n0 + col;
#pragma unroll
  for (int rr = 0; rr < MT * 4; ++rr) {
    const int row = (tid >> 6) + 4 * rr;
    float v = red[(0 * MT * 16 + row) * SBN + col];
    v += red[(1 * MT * 16 + row) * SBN + col];
    v += red[(2 * MT * 16 + row) * SBN + col];
    v += red[(3 * MT * 16 + row) * SBN + col];
    if (row < M && gn < N) {
      if (PARTIAL) {
        p.part[(((int64_t)c * d.batch + z) * M + row) * N + gn] = v;
      } else {
        if (ACT == ACT_GELU) v = gelu_erf(v);
        const int64_t off = z * d.sC + row * d.ldc + gn;
        if (OUT == OUT_F32) static_cast<float*>(d.C)[off] = v;
        else static_cast<__bf16*>(d.C)[off] = (__bf16)v;
      }
    }
  }
}

template <int OUT, int ACT>
__global__ __launch_bounds__(256) void skinny_finish_kernel(GemmDesc d, int ksplit, const float* part) {
  const int64_t per = d.M * d.N;
  const int64_t total = per * d.batch;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t z = idx / per, rem = idx - z * per;
    const int64_t m = rem / d.N, n = rem - m * d.N;
    float v = part[idx];
    for (int c = 1; c < ksplit; ++c) v += part[(int64_t)c * total + idx];
    if (ACT == ACT_GELU) v = gelu_erf(v);
    const int64_t off = z * d.sC + m * d.ldc + n;
    if (OUT == OUT_F32) static_cast<float*>(d.C)[off] = v;
    else static_cast<__bf16*>(d.C)[off] = (__bf16)v;
  }
}

template <int MT, bool PARTIAL>
void launch_mt(const SkParams& p, dim3 grid, hipStream_t s) {
  const dim3 block(NTHREADS);
  if (PARTIAL) {
    gemm_skinny_kernel<MT, OUT_F32, ACT_NONE, true><<<grid, block, 0, s>>>(p);
    return;
  }
  if (p.d.out_kind == OUT_F32) {
    if (p.d.act == ACT_GELU) gemm_skinny_kernel<MT, OUT_F32, ACT_GELU, false><<<grid, block, 0, s>>>(p);
    else gemm_skinny_kernel<MT, OUT_F32, ACT_NONE, false><<<grid, block, 0, s>>>(p);
  } else {
    if (p.d.act == ACT_GELU) gemm_skinny_kernel<MT, OUT_BF16, ACT_GELU, false><<<grid, block, 0, s>>>(p);
    else gemm_skinny_kernel<MT, OUT_BF16, ACT_NONE, false><<<grid, block, 0, s>>>(p);
  }
}

int64_t chunk_for(int64_t K, int ksplit) {
  int64_t kc = (K + ksplit - 1) / ksplit;
  kc = (kc + SBK - 1) / SBK * SBK;
  return kc > 0 ? kc : SBK;
}

}  // namespace

bool gemm_skinny_supported(const GemmDesc& d) {
  if (!d.in_bf16 || d.M < 1 || d.M > kSkinnyMaxRows) return false;
  if ((d.K & 7) || (d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  if ((int64_t)SBK * d.ldb * 2 >= (1ll << 31)) return false;
  if (((d.M - 1) * d.lda + d.K) * 2 >= (1ll << 31)) return false;
  if (d.batch > 65535 || (d.N + SBN - 1) / SBN > 0x7fffffff) return false;
  return true;
}

int skinny_ksplit(const GemmDesc& d) {
  const int64_t tiles = (d.N + SBN - 1) / SBN * d.batch;
  const int64_t target = 1024;  // about four workgroups per CU
  int64_t ks = tiles >= target ? 1 : (target + tiles - 1) / tiles;
  const int64_t max_ks = (d.K + SBK - 1) / SBK;
  if (ks > max_ks) ks = max_ks;
  if (ks > 64) ks = 64;
  if (ks < 1) ks = 1;
  // the chunk is rounded up to whole blocks; recount the chunks actually needed
  const int64_t kc = chunk_for(d.K, (int)ks);
  ks = d.K > 0 ? (d.K + kc - 1) / kc : 1;
  return (int)ks;
}

size_t skinny_partial_bytes(const GemmDesc& d, int ksplit) {
  return ksplit > 1 ? (size_t)ksplit * d.batch * d.M * d.N * sizeof(float) : 0;
}

hipError_t launch_gemm_skinny(const GemmDesc& d, int ksplit, float* part, hipStream_t stream) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  SkParams p;
  p.d = d;
  p.kchunk = chunk_for(d.K, ksplit);
  p.part = part;
  const dim3 grid((unsigned)((d.N + SBN - 1) / SBN), (unsigned)d.batch, (unsigned)(ksplit > 1 ? ksplit : 1));
  const bool partial = ksplit > 1;
  if (d.M <= 16) {
    if (partial) launch_mt<1, true>(p, grid, stream);
    else launch_mt<1, false>(p, grid, stream);
  } else {
    if (partial) launch_mt<2, true>(p, grid, stream);
    else launch_mt<2, false>(p, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_skinny_finish(const GemmDesc& d, int ksplit, const float* part, hipStream_t stream) {
  const int64_t total = d.M * d.N * d.batch;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid((unsigned)blocks), block(256);
  if (d.out_kind == OUT_F32) {
    if (d.act == ACT_GELU) skinny_finish_kernel<OUT_F32, ACT_GELU><<<grid, block, 0, stream>>>(d, ksplit, part);
    else skinny_finish_kernel<OUT_F32, ACT_NONE><<<grid, block, 0, stream>>>(d, ksplit, part);
  } else {
    if (d.act == ACT_GELU) skinny_finish_kernel<OUT_BF16, ACT_GELU><<<grid, block, 0, stream>>>(d, ksplit, part);
    else skinny_finish_kernel<OUT_BF16, ACT_NONE><<<grid, block, 0, stream>>>(d, ksplit, part);
  }
  return hipGetLastError();
}

}  // namespace tp
