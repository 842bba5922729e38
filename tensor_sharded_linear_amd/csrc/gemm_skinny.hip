// Skinny bf16 GEMM for a few rows (decode-shaped tensor-parallel layers):
// C_z = act(A_z B_z) with M <= 32, fp32 accumulate, on the gfx950 matrix cores.
//
// With so few rows the product is bound by streaming B (the weight shard)
// from HBM exactly once, so the kernel is built for bytes in flight and high
// occupancy, with no workgroup barrier in its main loop. A workgroup of 8
// waves owns SBN = 128 or 256 columns of one shard (and a chunk of K when K is
// split); each wave walks every 8th 32-row slice of that chunk on its own. A
// slice of B (32 x SBN bf16, 8 or 16 KB) comes into registers with 16-byte
// nontemporal buffer loads, one or two slices ahead, goes through the wave's
// private patch of LDS so that
// ds_read_b64_tr_b16 can hand out K-contiguous fragments, and meets the A
// fragment (the 16 or 32 token rows, loaded straight from global memory) in
// v_mfma_f32_16x16x32_bf16 with the token rows as the M dimension. At the end
// the 8 waves' sums are added in wave order through LDS. Splitting K over
// workgroups (ksplit > 1) leaves fp32 chunk sums that skinny_finish_kernel
// adds in ascending chunk order.
//
// The sharded layers follow the "Tensor Parallelism" topic page
// (chipfoundryservices.com), sections "Column-Wise Parallelism" and
// "Row-Wise Parallelism"; the decode shape is the model-serving case of the
// "Three practical examples" of the AI Glossary's "Tensor Parallelism" entry.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int SLICE = 32;      // k-rows per wave step
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int SBK = SLICE * NWAVES;  // K-chunks are multiples of this
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kStream = 2;  // buffer-load cache policy: nontemporal (the weights are read once)

// Column-tile geometry. Wider tiles read longer contiguous pieces of each
// weight row per request wave, which keeps HBM pages open longer: on the
// decode shapes each doubling of the width up to 256 measured 6-13% faster,
// as long as there are enough tiles to give most CUs one.
template <int SBN>
struct Tile {
  static_assert(SBN == 128 || SBN == 256, "tile width");
  static constexpr int CPR = SBN / 8;             // 16-byte chunks per B row
  static constexpr int LPL = SLICE * CPR / 64;    // B loads per lane per slice
  static constexpr int NSUB = SBN / 16;           // 16-column MFMA subtiles
  static constexpr int UNROLL = 256 / SBN;        // slices of loads in flight per wave
  static constexpr int PATCH = SLICE * SBN * 2;   // LDS per wave
};

struct SkParams {
  GemmDesc d;
  int64_t kchunk;
  float* part;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(n),
                                           kRsrcWord3);
}

// Chunk swizzle of a B row in LDS: chunk c of k-row r sits in slot c ^ swz_w(r).
// The rows are 256 or 512 bytes, a whole number of 256-byte bank windows, so
// without it the four k-rows one transpose group reads would hit the same
// banks; with it they take 32-byte slots 0, 2, 4, 6 apart, and the k-rows 8
// further on (the next 16-lane group) move to the other half of the window.
__device__ __forceinline__ int swz_w(int r) { return (2 * (r & 3)) ^ (8 * ((r >> 3) & 1)); }

template <int SBN, int MT, int OUT, int ACT, bool PARTIAL>
__global__ __launch_bounds__(NTHREADS) void gemm_skinny_kernel(SkParams p) {
  using T = Tile<SBN>;
  constexpr int LPL = T::LPL, NSUB = T::NSUB, UNROLL = T::UNROLL, PATCH = T::PATCH, CPR = T::CPR;
  // one staging patch per wave; reused for the cross-wave sum, 64 columns at a time
  constexpr int RED_BYTES = NWAVES * MT * 16 * 64 * 4;
  constexpr int LDS_BYTES = NWAVES * PATCH > RED_BYTES ? NWAVES * PATCH : RED_BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const GemmDesc& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* patch = lds + wave * PATCH;
  const int64_t n0 = (int64_t)blockIdx.x * SBN;
  const int z = blockIdx.y;
  const int c = blockIdx.z;
  const int64_t M = d.M, N = d.N, K = d.K, lda = d.lda, ldb = d.ldb;
  const int64_t kbeg = (int64_t)c * p.kchunk;
  const int64_t kend = min(K, kbeg + p.kchunk);
  const int nslices = kend > kbeg ? (int)((kend - kbeg + SLICE - 1) / SLICE) : 0;
  const int nsteps = nslices > wave ? (nslices - wave + NWAVES - 1) / NWAVES : 0;  // slices wave, wave + 8, ...

  const __bf16* Az = static_cast<const __bf16*>(d.A) + z * d.sA;
  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB + n0;
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(Az, ((M - 1) * lda + K) * 2);

  // B slice loads: chunk q = lane + 64 i -> k-row q / CPR, column chunk q % CPR.
  uint32_t w_voff[LPL];
  int w_lds[LPL];
#pragma unroll
  for (int i = 0; i < LPL; ++i) {
    const int q = lane + 64 * i;
    const int row = q / CPR, ch = q % CPR;
    w_voff[i] = (uint32_t)(row * ldb * 2 + ch * 16);
    w_lds[i] = row * (SBN * 2) + ((ch ^ swz_w(row)) << 4);
  }
  // A fragment: lane holds row (lane & 15) + 16 mt, 8 k-values at 8 (lane >> 4) of the slice.
  uint32_t x_voff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) x_voff[mt] = (uint32_t)((((lane & 15) + 16 * mt) * lda + 8 * (lane >> 4)) * 2);
  const int x_k = 8 * (lane >> 4);
  // B fragment via transpose reads: 16-lane group G = lane >> 4 takes k-rows
  // 8 G + 4 t .. + 3 of the slice; lane j = lane & 15 supplies row + (j >> 2),
  // columns 4 (j & 3) .. + 3 of a 16-column subtile and receives column j.
  const int G = lane >> 4, j16 = lane & 15;
  int tr_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * G + 4 * t + (j16 >> 2);
    tr_off[t] = row * (SBN * 2) + ((((j16 & 3) >> 1) ^ swz_w(row)) << 4) + (j16 & 1) * 8;
  }

  f32x4 acc[MT][NSUB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[mt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < nsteps; s0 += UNROLL) {
    u32x4 wv[UNROLL][LPL], xv[UNROLL][MT];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (s0 + u < nsteps) {
        const int64_t k0 = kbeg + (int64_t)(wave + NWAVES * (s0 + u)) * SLICE;
        const int64_t krem = K - k0;
        const __amdgpu_buffer_rsrc_t wr =
            make_rsrc(Bz + k0 * ldb, ((min<int64_t>(krem, SLICE) - 1) * ldb + (N - n0)) * 2);
#pragma unroll
        for (int i = 0; i < LPL; ++i) wv[u][i] = __builtin_amdgcn_raw_buffer_load_b128(wr, w_voff[i], 0, kStream);
        const uint32_t kk = (uint32_t)(k0 * 2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)  // k-chunks at or past K read as zero
          xv[u][mt] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, x_k < krem ? x_voff[mt] + kk : kOOB, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (s0 + u < nsteps) {
#pragma unroll
        for (int i = 0; i < LPL; ++i) *reinterpret_cast<u32x4*>(patch + w_lds[i]) = wv[u][i];
#pragma unroll
        for (int sub = 0; sub < NSUB; ++sub) {
          // subtile sub adds 2 sub to the chunk index; the swizzle is an XOR
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(patch + (tr_off[0] ^ ((2 * sub) << 4))));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(patch + (tr_off[1] ^ ((2 * sub) << 4))));
          const bf16x8 bfr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[u][mt]), bfr,
                                                                   acc[mt][sub], 0, 0, 0);
        }
      }
    }
  }

  // Add the 8 waves' sums in wave order through LDS, 64 columns at a time.
  float* red = reinterpret_cast<float*>(lds);  // [8][MT * 16][64]
#pragma unroll
  for (int cb = 0; cb < SBN / 64; ++cb) {
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(wave * MT * 16 + mt * 16 + 4 * (lane >> 4) + i) * 64 + 16 * sub + (lane & 15)] = acc[mt][cb * 4 + sub][i];
    __syncthreads();
    const int col = tid & 63;
    const int64_t gn = n0 + cb * 64 + col;
    for (int row = tid >> 6; row < MT * 16; row += NWAVES) {
      float v = red[row * 64 + col];
#pragma unroll
      for (int w = 1; w < NWAVES; ++w) v += red[(w * MT * 16 + row) * 64 + col];
      if (row < M && gn < N) {
        if (PARTIAL) {
          p.part[(((int64_t)c * d.batch + z) * M + row) * N + gn] = v;
        } else {
          if (ACT == ACT_GELU) v = gelu(v);
          const int64_t off = z * d.sC + row * d.ldc + gn;
          if (OUT == OUT_F32) static_cast<float*>(d.C)[off] = v;
          else static_cast<__bf16*>(d.C)[off] = (__bf16)v;
        }
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
    if (ACT == ACT_GELU) v = gelu(v);
    const int64_t off = z * d.sC + m * d.ldc + n;
    if (OUT == OUT_F32) static_cast<float*>(d.C)[off] = v;
    else static_cast<__bf16*>(d.C)[off] = (__bf16)v;
  }
}

template <int SBN, int MT, bool PARTIAL>
void launch_mt(const SkParams& p, dim3 grid, hipStream_t s) {
  const dim3 block(NTHREADS);
  if (PARTIAL) {
    gemm_skinny_kernel<SBN, MT, OUT_F32, ACT_NONE, true><<<grid, block, 0, s>>>(p);
    return;
  }
  if (p.d.out_kind == OUT_F32) {
    if (p.d.act == ACT_GELU) gemm_skinny_kernel<SBN, MT, OUT_F32, ACT_GELU, false><<<grid, block, 0, s>>>(p);
    else gemm_skinny_kernel<SBN, MT, OUT_F32, ACT_NONE, false><<<grid, block, 0, s>>>(p);
  } else {
    if (p.d.act == ACT_GELU) gemm_skinny_kernel<SBN, MT, OUT_BF16, ACT_GELU, false><<<grid, block, 0, s>>>(p);
    else gemm_skinny_kernel<SBN, MT, OUT_BF16, ACT_NONE, false><<<grid, block, 0, s>>>(p);
  }
}

// Tile width: 256 columns when that still gives most CUs a workgroup; 128
// otherwise, and always for 17..32 rows (twice the accumulators).
int tile_width(const GemmDesc& d) {
  if (d.M > 16) return 128;
  return (d.N + 255) / 256 * d.batch >= 192 ? 256 : 128;
}

int64_t chunk_for(int64_t K, int ksplit) {
  int64_t kc = (K + ksplit - 1) / ksplit;
  kc = (kc + SBK - 1) / SBK * SBK;
  return kc > 0 ? kc : SBK;
}

}  // namespace

bool gemm_skinny_supported(const GemmDesc& d) {
  if (!d.in_bf16 || d.M < 1 || d.M > kSkinnyMaxRows) return false;
  if (d.a_trans || d.b_trans || (d.act != ACT_NONE && d.act != ACT_GELU)) return false;
  if ((d.K & 7) || (d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  if ((int64_t)SBK * d.ldb * 2 >= (1ll << 31)) return false;
  if (((d.M - 1) * d.lda + d.K) * 2 >= (1ll << 31)) return false;
  if (d.batch > 65535 || (d.N + 127) / 128 > 0x7fffffff) return false;
  return true;
}

int skinny_ksplit(const GemmDesc& d) {
  // Split K only when the column tiles leave many CUs idle: the chunk sums
  // cost a write, a read and a second launch, which measured slower than
  // one workgroup on each of 7 of every 8 CUs.
  const int sbn = tile_width(d);
  const int64_t tiles = (d.N + sbn - 1) / sbn * d.batch;
  int64_t ks = tiles >= 160 ? 1 : 256 / (tiles > 0 ? tiles : 1);
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
  const int sbn = tile_width(d);
  const dim3 grid((unsigned)((d.N + sbn - 1) / sbn), (unsigned)d.batch, (unsigned)(ksplit > 1 ? ksplit : 1));
  const bool partial = ksplit > 1;
  if (d.M > 16) {
    if (partial) launch_mt<128, 2, true>(p, grid, stream);
    else launch_mt<128, 2, false>(p, grid, stream);
  } else if (sbn == 256) {
    if (partial) launch_mt<256, 1, true>(p, grid, stream);
    else launch_mt<256, 1, false>(p, grid, stream);
  } else {
    if (partial) launch_mt<128, 1, true>(p, grid, stream);
    else launch_mt<128, 1, false>(p, grid, stream);
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
