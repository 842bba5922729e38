// Large-tile bf16 GEMM on the gfx950 matrix cores: C_z = act(op(A_z) op(B_z)),
// fp32 accumulate.
//
// This is the per-shard dense product of the sharded linear layer ("Tensor
// Parallelism" topic page, chipfoundryservices.com, sections "Column-Wise
// Parallelism" and "Row-Wise Parallelism": each shard multiplies its input by
// its block of W). All shards of one call form one launch: either one wide
// product (column shards stored side by side) or a batch indexed by shard.
// The same kernel serves the backward products of those layers (section
// "Megatron-LM Tensor Parallelism", identity operators whose backward is the
// all-reduce): dX = dY W^T takes B transposed, dW = X^T dY takes A transposed.
//
// Tile 256 x 256 x 64, 512 threads = 8 waves in a 2 x 4 grid (two waves per
// SIMD); each wave owns a 128 x 64 block of C held as 4 x 2
// v_mfma_f32_32x32x16_bf16 accumulators.
// Each operand tile goes from HBM straight into LDS with buffer loads in LDS
// mode (no register staging), two stages deep, in one of two layouts chosen by
// how the operand is stored:
//   K-rows: 256 rows (of M or N) x 64 k, 128-byte rows (A as [M, K], B as
//     [N, K]); fragments are read with ds_read_b128.
//   MN-rows: 64 k-rows x 256 (of M or N), 512-byte rows (A as [K, M], B as
//     [K, N], the pages' [in, out] weight); fragments need K-contiguous lanes,
//     which gfx950 provides with the LDS transpose read ds_read_b64_tr_b16.
// The fragments of the next 16-wide k step are read while the matrix cores
// work on the current one. Rows past M, N or K and k chunks past K read as
// zero through the buffer range check.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
#define TP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int WM = 128, WN = 64;          // wave tile
constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 fragments per wave
constexpr int TILE_BYTES = 256 * BK * 2;   // one LDS stage of one operand: 32 KB
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
// conflicts: K-rows tiles hold 8 chunks per row, MN-rows tiles 32.
__device__ __forceinline__ int swz_k(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_mn(int krow) { return ((krow & 1) * 6) ^ (((krow >> 1) & 1) * 12); }

// One operand of the product: where its tile comes from and how it is laid out.
// KROWS: the operand is stored with k contiguous (A [M, K] or B [N, K]).
template <bool KROWS>
struct Operand {
  const __bf16* tile;  // element (row/col origin of the tile, k = 0) of this batch entry
  int64_t ld;          // row stride of the stored matrix, elements
  int extent;          // rows (KROWS) or columns (MN-rows) of the tile inside the matrix
  uint32_t voff, srow;
  int kc;              // KROWS: the k chunk this lane loads

  __device__ __forceinline__ void init(int lane, int wave) {
    if (KROWS) {
      // region r (1 KB) = rows 8r .. 8r+7; lane l -> row + (l >> 3), slot l & 7,
      // k-chunk (l & 7) ^ swz_k(row) = (l & 7) ^ (l >> 3) ^ w for regions w + 8 i
      kc = (lane & 7) ^ (lane >> 3) ^ wave;
      voff = (uint32_t)((lane >> 3) * ld * 2 + kc * 16);
      srow = (uint32_t)(8 * ld * 2);
    } else {
      // region r = k-rows 2r, 2r+1; lane l -> k-row + (l >> 5), slot l & 31,
      // chunk (l & 31) ^ swz_mn(k-row), the same for regions w + 8 i
      kc = 0;
      voff = (uint32_t)((lane >> 5) * ld * 2 + (((lane & 31) ^ swz_mn(2 * wave + (lane >> 5))) * 16));
      srow = (uint32_t)(2 * ld * 2);
    }
  }

  // LDS-mode loads of k-tile [k0, k0 + 64) into one stage: wave w fills regions
  // w + 8 i (i = 0..3), one instruction each; lane l lands at region + 16 l.
  __device__ __forceinline__ void load(int k0, int krem, char* stage, int wave) const {
    char* base = stage + wave * 1024;
    if (KROWS) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(tile + k0, ((int64_t)(extent - 1) * ld + krem) * 2);
      const uint32_t o = kc * 8 < krem ? voff : kOOB;  // k chunks at or past K read as zero
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, TP_LDS(base + i * 8192), 16, o, (wave + 8 * i) * srow, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(tile + (int64_t)k0 * ld, ((int64_t)(min(krem, BK) - 1) * ld + extent) * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, TP_LDS(base + i * 8192), 16, voff, (wave + 8 * i) * srow, 0, 0);
    }
  }
};

// Fragment reads of F 32-wide blocks starting at row/col `pos` of the tile.
// Either layout yields the lane format both MFMA operands use: lane l holds
// row/col (l & 31) of the block and k values 8 (l >> 5) .. + 7 of the k step.
template <bool KROWS, int F>
struct Frags {
  int off[F];
  int sw;
  __device__ __forceinline__ void init(int lane, int pos) {
    if (KROWS) {
      // rows of block f differ from row pos + (lane & 31) by 32 f: swz_k changes by (4 f) & 7
#pragma unroll
      for (int f = 0; f < F; ++f) off[f] = (pos + f * 32 + (lane & 31)) * 128;
      sw = swz_k(pos + (lane & 31));
    } else {
      // transpose reads: lane (G = lane >> 4, j = lane & 15) supplies k-row
      // 8 (G >> 1) + 4 t + (j >> 2) and columns 16 (G & 1) + 4 (j & 3) .. + 3 of a
      // 32-wide block, and receives 4 k values of column 16 (G & 1) + j
      const int G = lane >> 4, j16 = lane & 15;
      const int kr = 8 * (G >> 1) + (j16 >> 2);
      sw = swz_mn(kr);  // k-rows used with this lane differ by multiples of 4
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int col = pos + f * 32 + 16 * (G & 1) + 4 * (j16 & 3);
        off[f] = kr * 512 + (((col >> 3) ^ sw) << 4) + (col & 4) * 2;
      }
    }
  }
  __device__ __forceinline__ void read(const char* stage, int kk, int lane, bf16x8 (&out)[F]) const {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      if (KROWS) {
        const int kc = kk * 2 + (lane >> 5);
        out[f] = *reinterpret_cast<const bf16x8*>(stage + off[f] + ((kc ^ sw ^ ((4 * f) & 7)) << 4));
      } else {
        const char* p = stage + off[f] + kk * 16 * 512;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4 * 512));
        out[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }
};

template <int OUT, int ACT, bool AT, bool BT, bool WEAVE>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_mfma_kernel(Params p) {
  // Two stages of A and B, each its own array so the compiler can tell the
  // stage being filled by LDS-mode loads from the stage being read.
  __shared__ __attribute__((aligned(1024))) char sA0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[TILE_BYTES];
  constexpr bool A_KROWS = !AT, B_KROWS = BT;

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
  const int rows_here = (int)min<int64_t>(M - m0, BM);
  const int cols_here = (int)min<int64_t>(N - n0, BN);

  Operand<A_KROWS> opa;
  Operand<B_KROWS> opb;
  opa.ld = d.lda;
  opb.ld = d.ldb;
  const __bf16* Az = static_cast<const __bf16*>(d.A) + z * d.sA;
  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB;
  // K-rows tiles start at row m0 (n0); MN-rows tiles at column m0 (n0) of k-row 0.
  opa.tile = A_KROWS ? Az + m0 * d.lda : Az + m0;
  opb.tile = B_KROWS ? Bz + n0 * d.ldb : Bz + n0;
  // MN-rows extents run to the end of the row, so the columns past M (N) of a
  // partial tile read the next row's values; they only reach rows (columns) of
  // C that the epilogue drops.
  opa.extent = A_KROWS ? rows_here : (int)(M - m0);
  opb.extent = B_KROWS ? cols_here : (int)(N - n0);
  opa.init(lane, wave);
  opb.init(lane, wave);

  const int K32 = (int)K;
  const int KT = (K32 + BK - 1) / BK;
  auto issue_loads = [&](int kt, char* sa, char* sb) {
    const int k0 = kt * BK;
    opa.load(k0, K32 - k0, sa, wave);
    opb.load(k0, K32 - k0, sb, wave);
  };

  Frags<A_KROWS, FM> ra;
  Frags<B_KROWS, FN> rb;
  // LDS reads per 16-wide k step: one b128 per K-rows fragment, two transpose reads per MN-rows one
  constexpr int kReads = (A_KROWS ? FM : 2 * FM) + (B_KROWS ? FN : 2 * FN);
  ra.init(lane, wm * WM);
  rb.init(lane, wn * WN);
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const char* a, const char* b, int kk, int slot) {
    ra.read(a, kk, lane, fa[slot]);
    rb.read(b, kk, lane, fb[slot]);
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
      // WEAVE: interleave the next step's fragment reads with this step's
      // MFMAs, two MFMAs at a time, so every read has MFMAs to hide behind
      // (left alone, the compiler issues each read right before the MFMA that
      // needs it). Measured 3-6% faster for K up to 6144, 1-3% slower for
      // K of 8192 and more, where the kernels run long enough for the
      // engine clock to settle lower under the busier matrix cores.
      if (WEAVE && kk + 1 < BK / 16) {
        constexpr int r0 = kReads / 4, r1 = kReads * 2 / 4 - r0, r2 = kReads * 3 / 4 - r0 - r1;
        constexpr int r3 = kReads - r0 - r1 - r2, m = FM * FN / 4;
        __builtin_amdgcn_sched_group_barrier(0x100, r0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, r1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, r2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, r3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
      }
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
  // uniform and travels in the scalar offset. The bf16 side matrix (the saved
  // pre-activation, or the one the GeLU derivative is taken of) has the same
  // shape and is addressed the same way.
  const int64_t ldc = d.ldc;
  constexpr int ES = OUT == OUT_F32 ? 4 : 2;
  char* Ct = static_cast<char*>(d.C) + (z * d.sC + m0 * ldc + n0) * ES;
  const __amdgpu_buffer_rsrc_t crsrc = make_rsrc(Ct, ((int64_t)(rows_here - 1) * ldc + (N - n0)) * ES);
  const uint32_t row_bytes = (uint32_t)(ldc * ES);
  constexpr bool HAS_AUX = ACT == ACT_GELU_SAVE || ACT == ACT_DGELU;
  __amdgpu_buffer_rsrc_t xrsrc = crsrc;
  uint32_t xrow_bytes = 0;
  if (HAS_AUX) {
    char* Xt = static_cast<char*>(d.aux) + (z * d.sX + m0 * d.ldx + n0) * 2;
    xrsrc = make_rsrc(Xt, ((int64_t)(rows_here - 1) * d.ldx + (N - n0)) * 2);
    xrow_bytes = (uint32_t)(d.ldx * 2);
  }
#pragma unroll
  for (int im = 0; im < FM; ++im) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
      const int col = wn * WN + jn * 32 + (lane & 31);
      const int row0 = wm * WM + im * 32 + 4 * (lane >> 5);
      const bool in = n0 + col < N;
      const uint32_t voff = in ? (uint32_t)(row0 * row_bytes + col * ES) : kOOB;
      const uint32_t xoff = in ? (uint32_t)(row0 * xrow_bytes + col * 2) : kOOB;
      unsigned short zb[16];
      if (ACT == ACT_DGELU) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          zb[e] = __builtin_amdgcn_raw_buffer_load_b16(xrsrc, xoff, (uint32_t)(8 * (e >> 2) + (e & 3)) * xrow_bytes, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = acc[im][jn][e];
        const int erow = 8 * (e >> 2) + (e & 3);
        if (ACT == ACT_GELU_SAVE)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), xrsrc, xoff,
                                                (uint32_t)erow * xrow_bytes, 0);
        if (ACT == ACT_GELU || ACT == ACT_GELU_SAVE) v = gelu(v);
        if (ACT == ACT_DGELU) v *= gelu_grad((float)__builtin_bit_cast(__bf16, zb[e]));
        const uint32_t srow = (uint32_t)erow * row_bytes;
        if (OUT == OUT_F32)  // fp32 results (partials) are streamed out (nontemporal): measured 6-15% faster
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), crsrc, voff, srow, kStoreNT);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), crsrc, voff, srow, 0);
      }
    }
  }
}

constexpr int64_t kWeaveMaxK = 6144;

template <int OUT, int ACT, bool AT, bool BT>
void launch_one(const Params& p, hipStream_t s) {
  if (p.d.K <= kWeaveMaxK)
    gemm_bf16_mfma_kernel<OUT, ACT, AT, BT, true><<<dim3((unsigned)p.total), dim3(NTHREADS), 0, s>>>(p);
  else
    gemm_bf16_mfma_kernel<OUT, ACT, AT, BT, false><<<dim3((unsigned)p.total), dim3(NTHREADS), 0, s>>>(p);
}

}  // namespace

bool gemm_mfma_supported(const GemmDesc& d) {
  if (!d.in_bf16) return false;
  if ((d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  // K-rows tiles load k in chunks of 8 (their k tail is masked per chunk);
  // MN-rows tiles load along M or N in chunks of 8 (their k tail is masked per row)
  const bool krows = !d.a_trans || d.b_trans;
  if (krows && (d.K & 7)) return false;
  if (d.a_trans && (d.M & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  // 31-bit in-tile offsets: 256 rows of a K-rows tile and 64 k-rows of an MN-rows tile from the tile origin.
  const int64_t a_rows = d.a_trans ? BK : BM, b_rows = d.b_trans ? BN : BK;
  if (a_rows * d.lda * 2 >= (1ll << 31) || b_rows * d.ldb * 2 >= (1ll << 31)) return false;
  // and 256 rows of C (and of the side matrix)
  if ((int64_t)BM * d.ldc * (d.out_kind == OUT_F32 ? 4 : 2) >= (1ll << 31)) return false;
  if ((d.act == ACT_GELU_SAVE || d.act == ACT_DGELU) && (int64_t)BM * d.ldx * 2 >= (1ll << 31)) return false;
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
  const bool f32 = d.out_kind == OUT_F32;
  if (!d.a_trans && !d.b_trans) {
    // forward products
    if (d.act == ACT_GELU_SAVE) {
      if (f32) return hipErrorInvalidValue;
      launch_one<OUT_BF16, ACT_GELU_SAVE, false, false>(p, stream);
    } else if (d.act == ACT_GELU) {
      if (f32) launch_one<OUT_F32, ACT_GELU, false, false>(p, stream);
      else launch_one<OUT_BF16, ACT_GELU, false, false>(p, stream);
    } else if (d.act == ACT_NONE) {
      if (f32) launch_one<OUT_F32, ACT_NONE, false, false>(p, stream);
      else launch_one<OUT_BF16, ACT_NONE, false, false>(p, stream);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (!d.a_trans && d.b_trans) {
    // dX = dY W^T, optionally times GeLU'(pre-activation)
    if (d.act == ACT_DGELU) {
      if (f32) launch_one<OUT_F32, ACT_DGELU, false, true>(p, stream);
      else launch_one<OUT_BF16, ACT_DGELU, false, true>(p, stream);
    } else if (d.act == ACT_NONE) {
      if (f32) launch_one<OUT_F32, ACT_NONE, false, true>(p, stream);
      else launch_one<OUT_BF16, ACT_NONE, false, true>(p, stream);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (d.a_trans && !d.b_trans) {
    // dW = X^T dY
    if (d.act != ACT_NONE) return hipErrorInvalidValue;
    if (f32) launch_one<OUT_F32, ACT_NONE, true, false>(p, stream);
    else launch_one<OUT_BF16, ACT_NONE, true, false>(p, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tp
