// Large-tile bf16 GEMM on the gfx950 matrix cores: C_z = act(A_z B_z), fp32 accumulate.
//
// This is the per-shard dense product of the sharded linear layer ("Tensor
// Parallelism" topic page, chipfoundryservices.com, sections "Column-Wise
// Parallelism" and "Row-Wise Parallelism": each shard multiplies its input by
// its block of W). All shards of one call form one launch: either one wide
// product (column shards stored side by side) or a batch indexed by shard.
//
// Tile 256 x 256 x 64, 512 threads = 8 waves in a 2 x 4 grid (two waves per
// SIMD); each wave owns a 128 x 64 block of C held as 4 x 2
// v_mfma_f32_32x32x16_bf16 accumulators.
// A (row-major, K contiguous) and B (row-major, N contiguous: the pages'
// [in, out] weight) go from HBM straight into LDS with buffer loads in LDS
// mode (no register staging), two stages deep. A fragments are read with
// ds_read_b128; B fragments need K-contiguous lanes, which gfx950 provides
// with the LDS transpose read ds_read_b64_tr_b16. The fragments of the next
// 16-wide k step are read while the matrix cores work on the current one.
// Rows past M or K, and K chunks past K, read as zero through the buffer
// range check.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
#define TP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512, NWAVES = NTHREADS / 64;
constexpr int WM = 128, WN = 64;          // wave tile
constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 fragments per wave
constexpr int A_BYTES = BM * BK * 2;  // one LDS stage of A: 32 KB
constexpr int B_BYTES = BK * BN * 2;  // one LDS stage of B: 32 KB
constexpr int GROUP_M = 4;  // tile rows per group: 32 resident tiles form a 4 x 8 block per XCD
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every range used here
constexpr int kStoreNT = 2;                   // buffer-store cache policy: nontemporal

struct Params {
  GemmDesc d;
  int tiles_m, tiles_n, total;
};

// A buffer resource over `bytes` bytes from `base` (both uniform across the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(n),
                                           kRsrcWord3);
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

// XOR swizzles of 16-byte chunks that keep the fragment reads free of bank
// conflicts: A rows hold 64 elements (8 chunks), B rows 256 elements (32 chunks).
__device__ __forceinline__ int swz_a(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_b(int krow) { return ((krow & 1) * 6) ^ (((krow >> 1) & 1) * 12); }

template <int OUT, int ACT>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_mfma_kernel(Params p) {
  // Two stages of A and B, each its own array so the compiler can tell the
  // stage being filled by LDS-mode loads from the stage being read.
  __shared__ __attribute__((aligned(1024))) char sA0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[B_BYTES];

  const GemmDesc& d = p.d;
  const int logical = xcd_remap(blockIdx.x, p.total);
  const int per_batch = p.tiles_m * p.tiles_n;
  const int zz = logical / per_batch;
  const int u = logical - zz * per_batch;
  const int in_group = GROUP_M * p.tiles_n;
  const int g = u / in_group;
  const int first_m = g * GROUP_M;
  const int gm = min(p.tiles_m - first_m, GROUP_M);
  const int ug = u - g * in_group;
  // the tile coordinates are uniform; keep them (and all that derives from them) in scalar registers
  const int tm = __builtin_amdgcn_readfirstlane(first_m + ug % gm);
  const int tn = __builtin_amdgcn_readfirstlane(ug / gm);
  const int z = __builtin_amdgcn_readfirstlane(zz);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t M = d.M, N = d.N, K = d.K;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t lda = d.lda, ldb = d.ldb;
  const int rows_here = (int)min<int64_t>(M - m0, BM);

  const __bf16* Az = static_cast<const __bf16*>(d.A) + z * d.sA + m0 * lda;
  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB + n0;

  // LDS-mode loads: a stage of A (or B) is 32 regions of 1 KB; wave w fills
  // regions w + 8 i (i = 0..3) with one instruction each, and lane l lands at
  // region + 16 l, so each lane fetches the global chunk that the swizzle
  // places in that slot.
  //   A region r: rows 8r .. 8r+7; lane l -> row + (l >> 3), slot l & 7,
  //     k-chunk (l & 7) ^ swz_a(row) = (l & 7) ^ (l >> 3) ^ w, the same for every i.
  //   B region r: k-rows 2r, 2r+1; lane l -> k-row + (l >> 5), slot l & 31,
  //     n-chunk (l & 31) ^ swz_b(k-row), the same for every i.
  // The lane-dependent part of each offset goes in the vector offset, the
  // uniform row part in the scalar offset.
  const int a_kc = (lane & 7) ^ (lane >> 3) ^ wave;
  const uint32_t a_voff = (uint32_t)((lane >> 3) * lda * 2 + a_kc * 16);
  const uint32_t a_srow = (uint32_t)(8 * lda * 2);   // bytes per region (8 rows) of A
  const int b_rb = 2 * wave + (lane >> 5);
  const uint32_t b_voff = (uint32_t)((lane >> 5) * ldb * 2 + (((lane & 31) ^ swz_b(b_rb)) * 16));
  const uint32_t b_srow = (uint32_t)(2 * ldb * 2);   // bytes per region (2 k-rows) of B

  const int K32 = (int)K;
  const int KT = (K32 + BK - 1) / BK;

  auto issue_loads = [&](int kt, char* sa, char* sb) {
    const int k0 = kt * BK;
    const int krem = K32 - k0;
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(Az + k0, ((int64_t)(rows_here - 1) * lda + krem) * 2);
    const __amdgpu_buffer_rsrc_t brsrc =
        make_rsrc(Bz + (int64_t)k0 * ldb, ((int64_t)(min(krem, BK) - 1) * ldb + (N - n0)) * 2);
    char* abase = sa + wave * 1024;
    char* bbase = sb + wave * 1024;
    // k-chunks at or past K read as zero through an out-of-range offset
    const uint32_t ao = a_kc * 8 < krem ? a_voff : kOOB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, TP_LDS(abase + i * 8192), 16, ao,
                                               (wave + 8 * i) * a_srow, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, TP_LDS(bbase + i * 8192), 16, b_voff,
                                               (wave + 8 * i) * b_srow, 0, 0);
  };

  // Fragment addressing.
  // A fragment (32 rows x 16 k): lane holds row (lane & 31), k-chunk 2 kk + (lane >> 5).
  // B fragment via transpose reads: lane (G = lane >> 4, j = lane & 15) supplies
  // k-row 8 (G >> 1) + 4 t + (j >> 2) and columns 16 (G & 1) + 4 (j & 3) .. + 3
  // of a 32-column block; it receives 4 k-values of column 16 (G & 1) + j.
  int a_off[FM];
#pragma unroll
  for (int im = 0; im < FM; ++im) {
    const int row = wm * WM + im * 32 + (lane & 31);
    a_off[im] = row * 128;
  }
  const int a_h = lane >> 5;
  const int a_sw0 = swz_a(wm * WM + (lane & 31));  // rows differ by multiples of 32 below
  const int G = lane >> 4, j16 = lane & 15;
  const int b_kr = 8 * (G >> 1) + (j16 >> 2);
  const int b_sw = swz_b(b_kr);  // k-rows used with this lane differ by multiples of 4
  int b_off[FN];
#pragma unroll
  for (int jn = 0; jn < FN; ++jn) {
    const int col = wn * WN + jn * 32 + 16 * (G & 1) + 4 * (j16 & 3);
    b_off[jn] = b_kr * 512 + ((((col >> 3) ^ b_sw)) << 4) + (col & 4) * 2;
  }

  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const char* a, const char* b, int kk, int slot) {
#pragma unroll
    for (int im = 0; im < FM; ++im) {
      // rows of fragment im differ from row (wm*128 + lane&31) by 32 im: swz_a changes by (4 im) & 7
      const int sw = a_sw0 ^ ((4 * im) & 7);
      const int kc = kk * 2 + a_h;
      fa[slot][im] = *reinterpret_cast<const bf16x8*>(a + a_off[im] + ((kc ^ sw) << 4));
    }
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const char* bp = b + b_off[jn] + kk * 16 * 512;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(bp));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(bp + 4 * 512));
      fb[slot][jn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;

  // One k-tile: start the next tile's loads into the other stage, multiply the
  // current stage 16 k at a time while reading the next fragments, then wait
  // for the next stage at the barrier and read its first fragments.
  auto iteration = [&](int kt, const char* ca, const char* cb, char* na, char* nb) {
    if (kt + 1 < KT) issue_loads(kt + 1, na, nb);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read_frags(ca, cb, kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int im = 0; im < FM; ++im)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn)
          acc[im][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][im], fb[kk & 1][jn], acc[im][jn], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < KT) read_frags(na, nb, 0, 0);
  };

  if (KT > 0) {
    issue_loads(0, sA0, sB0);
    __syncthreads();
    read_frags(sA0, sB0, 0, 0);
  }
  for (int kt = 0; kt < KT; kt += 2) {
    iteration(kt, sA0, sB0, sA1, sB1);
    if (kt + 1 < KT) iteration(kt + 1, sA1, sB1, sA0, sB0);
  }

  // Epilogue: accumulator element e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32 of its 32 x 32 block. Stores go through a buffer resource
  // over this tile's rows of C: rows past M fall outside it and are dropped;
  // columns past N are masked per lane. The row part of every offset is
  // uniform and travels in the scalar offset.
  const int64_t ldc = d.ldc;
  constexpr int ES = OUT == OUT_F32 ? 4 : 2;
  char* Ct = static_cast<char*>(d.C) + (z * d.sC + m0 * ldc + n0) * ES;
  const __amdgpu_buffer_rsrc_t crsrc = make_rsrc(Ct, ((int64_t)(rows_here - 1) * ldc + (N - n0)) * ES);
  const uint32_t row_bytes = (uint32_t)(ldc * ES);
#pragma unroll
  for (int im = 0; im < FM; ++im) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const int col = wn * WN + jn * 32 + (lane & 31);
      const int row0 = wm * WM + im * 32 + 4 * (lane >> 5);
      const uint32_t voff = (n0 + col < N) ? (uint32_t)(row0 * row_bytes + col * ES) : kOOB;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[im][jn][e];
        if (ACT == ACT_GELU) v = gelu(v);
        const uint32_t srow = (uint32_t)(8 * (e >> 2) + (e & 3)) * row_bytes;
        if (OUT == OUT_F32)  // fp32 partials are streamed out (nontemporal): measured 12-15% faster
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), crsrc, voff, srow, kStoreNT);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), crsrc, voff, srow, 0);
      }
    }
  }
}

}  // namespace

bool gemm_mfma_supported(const GemmDesc& d) {
  if (!d.in_bf16) return false;
  if ((d.K & 7) || (d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  // 31-bit in-tile offsets: 256 rows of A and 64 rows of B from the tile origin.
  if ((int64_t)BM * d.lda * 2 >= (1ll << 31) || (int64_t)BK * d.ldb * 2 >= (1ll << 31)) return false;
  // and 256 rows of C
  if ((int64_t)BM * d.ldc * (d.out_kind == OUT_F32 ? 4 : 2) >= (1ll << 31)) return false;
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
