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
// SIMD); each wave owns a 128 x 64 block of C held as 8 x 4
// v_mfma_f32_16x16x32_bf16 accumulators. Under the socket's power cap this
// shape sustains more than the 32 x 32 x 16 one (2.06 against 1.79 PFLOP/s of
// bare MFMAs on random data, the same cycles per flop on one wave): it moves
// half the accumulator bytes per flop.
// Each operand tile goes from HBM straight into LDS with buffer loads in LDS
// mode (no register staging), two stages deep, in one of two layouts chosen by
// how the operand is stored:
//   K-rows: 256 rows (of M or N) x 64 k, 128-byte rows (A as [M, K], B as
//     [N, K]); fragments are read with ds_read_b128.
//   MN-rows: 64 k-rows x 256 (of M or N), 512-byte rows (A as [K, M], B as
//     [K, N], the pages' [in, out] weight); fragments need K-contiguous lanes,
//     which gfx950 provides with the LDS transpose read ds_read_b64_tr_b16.
// The two waves of each SIMD run a ping-pong schedule: one issues an
// uninterrupted cluster of MFMAs while the other reads the next k-tile's
// fragments and issues loads (see Sched). Rows past M, N or K and k chunks
// past K read as zero through the buffer range check.
#include <cstdlib>
#include <cstring>

#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
#define TP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int WM = 128, WN = 64;          // wave tile
constexpr int FM = WM / 16, FN = WN / 16;  // 16 x 16 blocks per wave
constexpr int KS = 32;                     // k per MFMA (v_mfma_f32_16x16x32_bf16)
constexpr int TILE_BYTES = 256 * BK * 2;   // one LDS stage of one operand: 32 KB
constexpr int GROUP_M = 4;  // tile rows per group: 32 resident tiles form a 4 x 8 block per XCD (see group_m)
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every range used here
constexpr int kStoreNT = 2;                   // buffer-store cache policy: nontemporal

struct Params {
  GemmDesc d;
  int tiles_m, tiles_n, total;
  int vec;      // C (and the side matrix) take 16-byte (fp32) / 8-byte (bf16) stores
  int group_m;  // tile rows per group (GROUP_M, or 2 for long K)
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
// conflicts: K-rows tiles hold 8 chunks per row, MN-rows tiles 32. The LDS
// serves a 16-byte read to lanes 8i .. 8i + 7 together with lanes 32 + 8i ..
// 32 + 8i + 7, and an 8-byte transpose read to 32 consecutive lanes (bank
// conflict counters: zero with these layouts). In an MN-rows tile the four
// k-rows one transpose read takes (k-row bits 0-1) and the two 16-lane groups
// served together (k-rows 16 apart, bit 4) land on distinct slots.
__device__ __forceinline__ int swz_k(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_mn(int krow) {
  return ((krow & 1) * 6) ^ (((krow >> 1) & 1) * 12) ^ (((krow >> 4) & 1) * 2);
}

// The 8-wide k chunk of a 32-deep k step that lane group G = lane / 16 holds
// in both MFMA operands. Any assignment gives the same product; this one puts
// chunks c and c ^ 1 (not c and c ^ 2) on the lanes a 16-byte read serves
// together, which the K-rows swizzle separates.
__device__ __forceinline__ int kgroup_chunk(int G) { return ((G & 1) << 1) | (G >> 1); }

// One operand of the product: where its tile comes from and how it is laid out.
// KROWS: the operand is stored with k contiguous (A [M, K] or B [N, K]).
template <bool KROWS>
struct Operand {
  const __bf16* tile;  // element (row/col origin of the tile, k = 0) of this batch entry
  int64_t ld;          // row stride of the stored matrix, elements
  int extent;          // rows (KROWS) or columns (MN-rows) of the tile inside the matrix
  uint32_t voff, srow;
  uint32_t voff_odd;   // MN-rows: the offset for regions w + 8 i with i odd
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
      // chunk (l & 31) ^ swz_mn(k-row); for regions w + 8 i the k-row is
      // 2 w + 16 i + (l >> 5), whose swizzle bits depend on i only through i % 2
      kc = 0;
      voff = (uint32_t)((lane >> 5) * ld * 2 + (((lane & 31) ^ swz_mn(2 * wave + (lane >> 5))) * 16));
      voff_odd = (uint32_t)((lane >> 5) * ld * 2 + (((lane & 31) ^ swz_mn(2 * wave + 16 + (lane >> 5))) * 16));
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
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, TP_LDS(base + i * 8192), 16, (i & 1) ? voff_odd : voff,
                                                 (wave + 8 * i) * srow, 0, 0);
    }
  }
};

// Fragment reads of F 16-wide blocks starting at row/col `pos` of the tile,
// for the 32-deep k step kk of the tile. Either layout yields the lane format
// both MFMA operands use: lane l holds row/col (l & 15) of the block and the
// k values of chunk kgroup_chunk(l >> 4) of the k step.
template <bool KROWS, int F>
struct Frags {
  int off[F];
  __device__ __forceinline__ void init(int lane, int pos) {
    if (KROWS) {
      // row pos + 16 f + (l & 15), k chunk 4 kk + kgroup_chunk(l >> 4); kk only flips bit 2 of the chunk
      const int kg = kgroup_chunk(lane >> 4);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int row = pos + f * 16 + (lane & 15);
        off[f] = row * 128 + ((kg ^ swz_k(row)) << 4);
      }
    } else {
      // transpose reads: lane (G = lane >> 4, j = lane & 15) supplies k-row
      // 32 kk + 8 kgroup_chunk(G) + 4 t + (j >> 2) and columns 4 (j & 3) .. + 3
      // of a 16-wide block, and receives 4 k values of column j; t and kk leave
      // the k-row bits the swizzle uses unchanged
      const int G = lane >> 4, j16 = lane & 15;
      const int kr = 8 * kgroup_chunk(G) + (j16 >> 2);
      const int sw = swz_mn(kr);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int col = pos + f * 16 + 4 * (j16 & 3);
        off[f] = kr * 512 + (((col >> 3) ^ sw) << 4) + (col & 4) * 2;
      }
    }
  }
  __device__ __forceinline__ void read(const char* stage, int kk, int lane, bf16x8 (&out)[F]) const {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      if (KROWS) {
        out[f] = *reinterpret_cast<const bf16x8*>(stage + (off[f] ^ (kk << 6)));
      } else {
        const char* p = stage + off[f] + kk * KS * 512;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4 * 512));
        out[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }
};

// Tile owned by this workgroup: workgroups are dealt to XCDs contiguously
// (xcd_remap), then grouped group_m tile rows tall within each batch entry.
struct TileCoord {
  int tm, tn, z;
};
__device__ __forceinline__ TileCoord tile_coord(const Params& p) {
  const int logical = xcd_remap(blockIdx.x, p.total);
  const int per_batch = p.tiles_m * p.tiles_n;
  const int zz = logical / per_batch;
  const int u = logical - zz * per_batch;
  const int in_group = p.group_m * p.tiles_n;
  const int g = u / in_group;
  const int first_m = g * p.group_m;
  const int gm = min(p.tiles_m - first_m, p.group_m);
  const int ug = u - g * in_group;
  // the tile coordinates are uniform; keep them (and all that derives from them) in scalar registers
  TileCoord t;
  t.tm = __builtin_amdgcn_readfirstlane(first_m + ug % gm);
  t.tn = __builtin_amdgcn_readfirstlane(ug / gm);
  t.z = __builtin_amdgcn_readfirstlane(zz);
  return t;
}

typedef f32x4 AccTile[FM][FN];
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Epilogue through LDS. Accumulator element e of lane l is row 4 (l / 16) + e,
// column l % 16 of its 16 x 16 block; stored as it is, every store instruction
// would write 64-byte pieces of 4 rows. Instead each wave parks 64 of its 128
// rows in a private 16 KB patch of the (by then idle) LDS stages and reads
// them back as 4 consecutive columns per lane, so that each store writes 4
// rows of 64 contiguous columns. The activation, the side matrix and the
// conversion are applied on the way out. Stores go through a buffer resource
// over this tile's rows of C: rows past M fall outside it and are dropped;
// columns past N are masked per lane (N is a multiple of 8, so a lane's 4
// columns are all in or all out). `vec`: C (and the side matrix) allow
// 16-byte (fp32) or 8-byte (bf16) stores; else each value is stored alone.
template <int OUT, int ACT>
__device__ __forceinline__ void store_tile(const GemmDesc& d, const AccTile& acc, int64_t m0, int64_t n0, int z,
                                           int lane, int wm, int wn, float* patch, bool vec) {
  const int64_t N = d.N;
  const int rows_here = (int)min<int64_t>(d.M - m0, BM);
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
  const int g = lane >> 4, j = lane & 15;
  const int col = wn * WN + 4 * j;  // this lane's 4 columns on the way out
  const bool in = n0 + col < N;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // park rows 64 half .. + 63 of the wave's block: [64][64] fp32, the 16-column
    // groups of row r XOR-swizzled by (r / 4) % 4 so both directions are conflict-free
#pragma unroll
    for (int rb = 0; rb < FM / 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < FN; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rb * 16 + 4 * g + e;
          patch[row * 64 + ((cb ^ g) << 4) + j] = acc[half * (FM / 2) + rb][cb][e];
        }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + g;  // (row / 4) % 4 = i % 4
      f32x4 v = *reinterpret_cast<const f32x4*>(patch + row * 64 + ((4 * j) ^ (16 * (i & 3))));
      const int trow = wm * WM + half * 64 + row;  // row within the tile
      const uint32_t voff = in ? (uint32_t)(trow * row_bytes + col * ES) : kOOB;
      const uint32_t xoff = in ? (uint32_t)(trow * xrow_bytes + col * 2) : kOOB;
      if (ACT == ACT_GELU_SAVE) {
        if (vec) {
          u32x2 h;
          h[0] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[0]) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[1]) << 16);
          h[1] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[2]) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(h, xrsrc, xoff, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v[e]), xrsrc, xoff, 2 * e, 0);
        }
      }
      if (ACT == ACT_DGELU) {
        unsigned short zb[4];
        if (vec) {
          const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(xrsrc, xoff, 0, 0);
          zb[0] = (unsigned short)h[0];
          zb[1] = (unsigned short)(h[0] >> 16);
          zb[2] = (unsigned short)h[1];
          zb[3] = (unsigned short)(h[1] >> 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) zb[e] = __builtin_amdgcn_raw_buffer_load_b16(xrsrc, xoff, 2 * e, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= gelu_grad((float)__builtin_bit_cast(__bf16, zb[e]));
      }
      if (ACT == ACT_GELU || ACT == ACT_GELU_SAVE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu(v[e]);
      }
      if (OUT == OUT_F32) {  // fp32 results (partials) are streamed out (nontemporal): measured 6-15% faster
        if (vec) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), crsrc, voff, 0, kStoreNT);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ve = v[e];  // a bit cast of v[e] itself was compiled as one of v[0]
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ve), crsrc, voff, 4 * e, kStoreNT);
          }
        }
      } else {
        if (vec) {
          u32x2 h;
          h[0] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[0]) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[1]) << 16);
          h[1] = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[2]) |
                 ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(h, crsrc, voff, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v[e]), crsrc, voff, 2 * e, 0);
        }
      }
    }
  }
}

// Main-loop schedules.
//   SCHED_PLAIN: every wave reads the next 32-deep k step's fragments while
//     its matrix cores work on the current one; one barrier per k-tile.
//   SCHED_WEAVE: the same, with the reads and MFMAs interleaved two MFMAs at
//     a time by scheduling-group barriers.
//   SCHED_PINGPONG: the two waves that share a SIMD (waves w and w + 4) run
//     one phase apart. In a memory phase a wave reads all fragments of one
//     k-tile from LDS into registers and issues its share of the HBM->LDS
//     loads; in a compute phase it issues the k-tile's 64 MFMAs from
//     registers with nothing in between. Barriers separate the phases, so at
//     any time one wave of each SIMD feeds the matrix cores and the other
//     moves data.
// The launches use SCHED_PINGPONG; the other two remain for timing
// comparisons (TP_GEMM_SCHED).
enum Sched : int { SCHED_PLAIN = 0, SCHED_WEAVE = 1, SCHED_PINGPONG = 2 };

// s_waitcnt immediates (vmcnt, expcnt, lgkmcnt fields of the gfx9 encoding; a field at its
// maximum does not wait).
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// A workgroup barrier that no instruction is scheduled across and no memory
// access is moved across; waits for outstanding loads are explicit.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int OUT, int ACT, bool AT, bool BT, int SCHED>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_mfma_kernel(Params p) {
  // Two stages of A and B, each its own array so the compiler can tell the
  // stage being filled by LDS-mode loads from the stage being read.
  __shared__ __attribute__((aligned(1024))) char sA0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[TILE_BYTES];
  constexpr bool A_KROWS = !AT, B_KROWS = BT;

  const GemmDesc& d = p.d;
  const TileCoord tc = tile_coord(p);
  const int tm = tc.tm, tn = tc.tn, z = tc.z;

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
  // LDS reads per 32-deep k step: one b128 per K-rows fragment, two transpose reads per MN-rows one
  constexpr int kReads = (A_KROWS ? FM : 2 * FM) + (B_KROWS ? FN : 2 * FN);
  ra.init(lane, wm * WM);
  rb.init(lane, wn * WN);
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const char* a, const char* b, int kk, int slot) {
    ra.read(a, kk, lane, fa[slot]);
    rb.read(b, kk, lane, fb[slot]);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][jn][e] = 0.f;

  if constexpr (SCHED == SCHED_PINGPONG) {
    // Phases are numbered by the barriers between them. Group 0 (waves 0..3)
    // runs memory(i) in phase 2i and compute(i) in phase 2i + 1; group 1
    // (waves 4..7) runs them one phase later. k-tile i lives in stage i % 2,
    // read in phases 2i and 2i + 1, so the stage is free from phase 2i + 2,
    // when both groups issue their loads of k-tile i + 2 into it (group 0 in
    // memory(i + 1), group 1 in compute(i)); each wave waits for its own
    // loads at the end of the next phase, before the barrier after which
    // k-tile i + 2 is first read.
    const int grp = wave >> 2;
    bf16x8 ta[BK / KS][FM], tb[BK / KS][FN];
    auto read_tile = [&](const char* a, const char* b) {
#pragma unroll
      for (int kk = 0; kk < BK / KS; ++kk) {
        ra.read(a, kk, lane, ta[kk]);
        rb.read(b, kk, lane, tb[kk]);
      }
    };
    auto mma_tile = [&]() {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < BK / KS; ++kk)
#pragma unroll
        for (int im = 0; im < FM; ++im)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn)
            acc[im][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[kk][im], tb[kk][jn], acc[im][jn], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    };
    // group 0, k-tile i from stage (ca, cb); the other stage (na, nb) receives k-tile i + 1
    auto step0 = [&](int i, const char* ca, const char* cb, char* na, char* nb) {
      read_tile(ca, cb);
      if (i + 1 < KT) issue_loads(i + 1, na, nb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      phase_barrier();
      mma_tile();
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      phase_barrier();
    };
    // group 1, k-tile i from stage (ca, cb), which receives k-tile i + 2 during the compute phase
    auto step1 = [&](int i, char* ca, char* cb) {
      read_tile(ca, cb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      phase_barrier();
      if (i + 2 < KT) issue_loads(i + 2, ca, cb);
      mma_tile();
      phase_barrier();
    };
    if (KT > 0) {
      issue_loads(0, sA0, sB0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      phase_barrier();
      if (grp == 0) {
        for (int kt = 0; kt < KT; kt += 2) {
          step0(kt, sA0, sB0, sA1, sB1);
          if (kt + 1 < KT) step0(kt + 1, sA1, sB1, sA0, sB0);
        }
        phase_barrier();  // group 1's first barrier has no partner in the loop above
      } else {
        if (KT > 1) issue_loads(1, sA1, sB1);
        phase_barrier();  // group 1 starts one phase behind group 0
        for (int kt = 0; kt < KT; kt += 2) {
          step1(kt, sA0, sB0);
          if (kt + 1 < KT) step1(kt + 1, sA1, sB1);
        }
      }
    }
  } else {
  // One k-tile: start the next tile's loads into the other stage, multiply the
  // current stage 32 k at a time while reading the next fragments, then wait
  // for the next stage at the barrier and read its first fragments.
  auto iteration = [&](int kt, const char* ca, const char* cb, char* na, char* nb) {
    if (kt + 1 < KT) issue_loads(kt + 1, na, nb);
#pragma unroll
    for (int kk = 0; kk < BK / KS; ++kk) {
      if (kk + 1 < BK / KS) read_frags(ca, cb, kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int im = 0; im < FM; ++im)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn)
          acc[im][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kk & 1][im], fb[kk & 1][jn], acc[im][jn], 0, 0, 0);
      // WEAVE: interleave the next step's fragment reads with this step's
      // MFMAs, two MFMAs at a time, so every read has MFMAs to hide behind
      // (left alone, the compiler issues each read right before the MFMA that
      // needs it). Measured 3-6% faster for K up to 6144, 1-3% slower for
      // K of 8192 and more, where the kernels run long enough for the
      // engine clock to settle lower under the busier matrix cores.
      if (SCHED == SCHED_WEAVE && kk + 1 < BK / KS) {
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
  }  // SCHED_PLAIN, SCHED_WEAVE

  // the stages are free once every wave is past its last fragment read
  __syncthreads();
  char* stage_of_wave = (wave >> 1) == 0 ? sA0 : (wave >> 1) == 1 ? sA1 : (wave >> 1) == 2 ? sB0 : sB1;
  store_tile<OUT, ACT>(d, acc, m0, n0, z, lane, wm, wn, reinterpret_cast<float*>(stage_of_wave + (wave & 1) * 16384),
                       p.vec);
}

// Schedule override for timing comparisons of the same product: TP_GEMM_SCHED = plain | weave | pingpong.
int sched_override() {
  static const int v = [] {
    const char* e = std::getenv("TP_GEMM_SCHED");
    if (!e) return -1;
    if (!std::strcmp(e, "plain")) return (int)SCHED_PLAIN;
    if (!std::strcmp(e, "weave")) return (int)SCHED_WEAVE;
    if (!std::strcmp(e, "pingpong")) return (int)SCHED_PINGPONG;
    return -1;
  }();
  return v;
}

template <int OUT, int ACT, bool AT, bool BT>
void launch_one(const Params& p, hipStream_t s) {
  // Measured on the MLP and attention-projection shapes (same process, one
  // box): with the 16 x 16 x 32 MFMAs the ping-pong schedule is the fastest
  // at every K, 3-7% ahead of the previous 32 x 32 x 16 kernels; the woven
  // and plain schedules trail it by 5-20%.
  int sched = SCHED_PINGPONG;
  if (sched_override() >= 0) sched = sched_override();
  const dim3 grid((unsigned)p.total), block(NTHREADS);
  if (sched == SCHED_PINGPONG) {
    gemm_bf16_mfma_kernel<OUT, ACT, AT, BT, SCHED_PINGPONG><<<grid, block, 0, s>>>(p);
    return;
  }
  if (sched == SCHED_WEAVE)
    gemm_bf16_mfma_kernel<OUT, ACT, AT, BT, SCHED_WEAVE><<<grid, block, 0, s>>>(p);
  else
    gemm_bf16_mfma_kernel<OUT, ACT, AT, BT, SCHED_PLAIN><<<grid, block, 0, s>>>(p);
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
  // The 256 resident tiles stream K-long slabs: with groups 4 tile rows tall,
  // 8 XCDs x 4 A row slabs + 8 shared B column slabs = 40 slabs of 512 K bytes.
  // Past about 200 MB those no longer stay in the 256 MB memory-side cache
  // from one wave of tiles to the next; groups 2 rows tall stream 32 slabs, at
  // the price of 50% more L2 fetches per k-tile (measured: K = 12288 gains 2%,
  // K = 8192 and 6144 lose 2-3% with the shorter groups).
  p.group_m = (int64_t)40 * d.K * 512 > ((int64_t)200 << 20) ? 2 : GROUP_M;
  {
    const int64_t es = d.out_kind == OUT_F32 ? 4 : 2;
    bool v = (reinterpret_cast<uintptr_t>(d.C) % (4 * es)) == 0 && d.ldc % 4 == 0 && d.sC % 4 == 0;
    if (d.act == ACT_GELU_SAVE || d.act == ACT_DGELU)
      v = v && (reinterpret_cast<uintptr_t>(d.aux) % 8) == 0 && d.ldx % 4 == 0 && d.sX % 4 == 0;
    p.vec = v ? 1 : 0;
  }
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
