// Skinny bf16 GEMM for a few rows (decode-shaped tensor-parallel layers):
// C_z = act(A_z B_z) with M <= 32, fp32 accumulate, on the gfx950 matrix cores.
//
// With so few rows the product is bound by streaming B (the weight shard)
// from HBM exactly once, so the kernel is built for bytes in flight, with no
// workgroup barrier in its main loop. A workgroup of 4 waves owns SBN = 128
// or 256 columns of one shard (and a chunk of K when K is split); each wave
// walks every 4th 32-row slice of that chunk on its own. A slice of B
// (32 x SBN bf16, 8 or 16 KB) goes straight from HBM into one of the wave's
// own LDS buffers with 16-byte nontemporal LDS-mode buffer loads, 4 (128
// columns) or 2 (256 columns) slices ahead, so that ds_read_b64_tr_b16 can
// hand out K-contiguous fragments, and meets the A fragment (the 16 or 32
// token rows, loaded straight from global memory) in
// v_mfma_f32_16x16x32_bf16 with the token rows as the M dimension. At the end
// the 4 waves' sums are added in wave order through LDS. Splitting K over
// workgroups (ksplit > 1) leaves fp32 chunk sums that skinny_finish_kernel
// adds in ascending chunk order, or that the next skinny product adds, in the
// same order and with the same activation and rounding, as it loads them for
// its token fragments (the MLP's second product: no pass in between).
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
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int SLICE = 32;      // k-rows per wave step
constexpr int SBK_MAX = 256;   // K-chunks are whole multiples of 256 rows (of SLICE x waves = 128)
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kStream = 2;  // buffer-load cache policy: nontemporal (the weights are read once)
#define TP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Column-tile geometry. Wider tiles read longer contiguous pieces of each
// weight row per request wave, which keeps HBM pages open longer: on the
// decode shapes each doubling of the width up to 256 measured 6-13% faster,
// as long as there are enough tiles to give most CUs one. 4 waves, each with
// NBUF slice buffers: 4 x 8 KB for 128 columns, 2 x 16 KB for 256, so 128 KB
// of LDS and one workgroup per CU either way. Measured on the decode shapes,
// 4 waves beat 8 waves with 2 slices each (128 columns) and 2 waves with 4
// slices each (256 columns).
template <int SBN>
struct Tile {
  static_assert(SBN == 128 || SBN == 256, "tile width");
  static constexpr int CPR = SBN / 8;                 // 16-byte chunks per B row
  static constexpr int NSUB = SBN / 16;               // 16-column MFMA subtiles
  static constexpr int SLICE_BYTES = SLICE * SBN * 2;  // 8 or 16 KB
  static constexpr int DMA = SLICE_BYTES / 1024;       // 1 KB LDS-mode loads per slice
  static constexpr int RPD = 1024 / (SBN * 2);         // B rows per such load
  static constexpr int NW = 4;                         // waves per workgroup
  static constexpr int NBUF = SBN == 128 ? 4 : 2;      // slices of each wave in LDS, in flight together
  static constexpr int SBK = SLICE * NW;               // K-chunk granule
};

struct SkParams {
  GemmDesc d;
  int64_t kchunk;
  float* part;
  // Chunked A (AK > 0): A_z(m, k) = bf16(act_a(sum_c apart[c a_cs + z a_sz + m a_ld + k])),
  // the c summed in ascending order: the unfinished first product of an MLP.
  const float* apart;
  int64_t a_cs, a_sz, a_ld;
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

// s_waitcnt immediates (vmcnt field of the gfx9 encoding; expcnt and lgkmcnt at their maximum)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;

// AK = 0: A is bf16 (d.A, row stride lda), grid (tiles, batch, chunks).
// AK > 0: A is AK fp32 chunk sums in p.apart, finished on load with ACTA;
// the grid is one-dimensional with the batch index fastest, so that with 8
// shards every XCD works on one shard and reads only that shard's sums.
template <int SBN, int MT, int OUT, int ACT, bool PARTIAL, int AK = 0, int ACTA = ACT_NONE>
__global__ __launch_bounds__(Tile<SBN>::NW * 64) void gemm_skinny_kernel(SkParams p) {
  using T = Tile<SBN>;
  constexpr int NSUB = T::NSUB, CPR = T::CPR, DMA = T::DMA, RPD = T::RPD, NW = T::NW;
  constexpr int SLICE_BYTES = T::SLICE_BYTES;
  constexpr int NBUF = T::NBUF;
  // NBUF slice buffers per wave, each buffer index its own array so the
  // compiler can tell the buffers being filled by LDS-mode loads from the one
  // being read; the first also takes the cross-wave sum at the end
  // (NW x MT x 16 x 64 floats).
  static_assert(NW * MT * 16 * 64 * 4 <= NW * SLICE_BYTES, "reduction space");
  __shared__ __attribute__((aligned(1024))) char lds0[NW * SLICE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds1[NW * SLICE_BYTES];
  const GemmDesc& d = p.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* buf0 = lds0 + wave * SLICE_BYTES;
  char* buf1 = lds1 + wave * SLICE_BYTES;
  const int tile = AK > 0 ? (int)(blockIdx.x / (unsigned)d.batch) : (int)blockIdx.x;
  const int z = AK > 0 ? (int)(blockIdx.x % (unsigned)d.batch) : (int)blockIdx.y;
  const int64_t n0 = (int64_t)tile * SBN;
  const int c = AK > 0 ? 0 : (int)blockIdx.z;
  const int64_t M = d.M, N = d.N, K = d.K, lda = d.lda, ldb = d.ldb;
  const int64_t kbeg = (int64_t)c * p.kchunk;
  const int64_t kend = min(K, kbeg + p.kchunk);
  const int nslices = kend > kbeg ? (int)((kend - kbeg + SLICE - 1) / SLICE) : 0;
  const int nsteps = nslices > wave ? (nslices - wave + NW - 1) / NW : 0;  // slices wave, wave + NW, ...

  const __bf16* Bz = static_cast<const __bf16*>(d.B) + z * d.sB + n0;
  // A: one range (bf16 rows of stride lda), or one per chunk sum (fp32 rows
  // of stride a_ld >= K): rows past M fall outside either way and read as zero.
  constexpr int NA = AK > 0 ? AK : 1;
  constexpr int ESZ = AK > 0 ? 4 : 2;
  const int64_t alda = AK > 0 ? p.a_ld : lda;
  __amdgpu_buffer_rsrc_t arsrc[NA];
  if constexpr (AK > 0) {
#pragma unroll
    for (int q = 0; q < AK; ++q)
      arsrc[q] = make_rsrc(p.apart + q * p.a_cs + z * p.a_sz, ((M - 1) * p.a_ld + K) * 4);
  } else {
    arsrc[0] = make_rsrc(static_cast<const __bf16*>(d.A) + z * d.sA, ((M - 1) * lda + K) * 2);
  }

  // LDS-mode load i of a slice writes 1 KB at buffer offset 1024 i, lane l at
  // +16 l: B row RPD i + l / CPR, slot l % CPR, so the lane fetches the chunk
  // that slot holds under the swizzle.
  uint32_t dma_voff[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int row = RPD * i + lane / CPR, slot = lane % CPR;
    dma_voff[i] = (uint32_t)(row * ldb * 2 + ((slot ^ swz_w(row)) << 4));
  }
  // captured through a pointer: the host compile pass rejects a lambda that
  // captures a local array of template-dependent size
  const uint32_t* const dvo = dma_voff;
  // A fragment: lane holds row (lane & 15) + 16 mt, 8 k-values at 8 (lane >> 4)
  // of the slice: one 16-byte load of bf16, or two per chunk sum of fp32.
  constexpr int XL = AK > 0 ? 2 * AK : 1;  // A loads per slice and row block
  uint32_t x_voff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) x_voff[mt] = (uint32_t)((((lane & 15) + 16 * mt) * alda + 8 * (lane >> 4)) * ESZ);
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

  // Slice i of this wave (k-rows kbeg + (wave + NW i) * 32 ..): B into LDS
  // buffer `buf`, the token fragment into x. Rows past K fall outside the
  // range and read as zero, like k chunks of A at or past K; a slice past the
  // wave's share (i >= nsteps) takes an empty range and reads as zero whole.
  u32x4 xv[NBUF][MT][XL];
  auto issue = [&](int i, char* buf, u32x4 (&x)[MT][XL]) {
    const bool valid = i < nsteps;
    const int64_t k0 = kbeg + (int64_t)(wave + NW * i) * SLICE;
    const int64_t krem = K - k0;
    const int64_t bytes = valid ? ((min<int64_t>(krem, SLICE) - 1) * ldb + (N - n0)) * 2 : 0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(Bz + (valid ? k0 : 0) * ldb, bytes);
#pragma unroll
    for (int q = 0; q < DMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, TP_LDS(buf + q * 1024), 16, dvo[q], 0, 0, kStream);
    const uint32_t kk = (uint32_t)(k0 * ESZ);
    const bool xin = valid && x_k < krem;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int l = 0; l < XL; ++l)
        x[mt][l] = __builtin_amdgcn_raw_buffer_load_b128(arsrc[l / 2], xin ? x_voff[mt] + kk + 16 * (l & 1) : kOOB, 0, 0);
  };
  auto consume = [&](const char* buf, const u32x4 (&x)[MT][XL]) {
    // token fragments: bf16 as loaded, or the chunk sums added in ascending
    // order, activated and rounded to bf16 (what the finishing pass would store)
    bf16x8 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (AK > 0) {
        f32x8 v = __builtin_shufflevector(__builtin_bit_cast(f32x4, x[mt][0]), __builtin_bit_cast(f32x4, x[mt][1]),
                                          0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int q = 1; q < AK; ++q)
          v += __builtin_shufflevector(__builtin_bit_cast(f32x4, x[mt][2 * q]),
                                       __builtin_bit_cast(f32x4, x[mt][2 * q + 1]), 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (ACTA == ACT_GELU) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu(v[e]);
        }
        af[mt] = __builtin_convertvector(v, bf16x8);
      } else {
        af[mt] = __builtin_bit_cast(bf16x8, x[mt][0]);
      }
    }
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      // subtile sub adds 2 sub to the chunk index; the swizzle is an XOR
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(buf + (tr_off[0] ^ ((2 * sub) << 4))));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(buf + (tr_off[1] ^ ((2 * sub) << 4))));
      const bf16x8 bfr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr, acc[mt][sub], 0, 0, 0);
    }
  };

  // NBUF slices in flight per wave: a slice's buffer is refilled with the
  // slice NBUF ahead as soon as its reads have returned, so the next NBUF - 1
  // slices' loads are always on their way while one is multiplied. Loads
  // complete in issue order: waiting until only the later slices' loads
  // remain means this one has landed. No barrier: every buffer belongs to
  // one wave. Issues and multiplications take no branch (past the share they
  // move zeros), which keeps the compiler's own tracking of the LDS-mode
  // loads exact.
  constexpr int kPerSlice = DMA + MT * XL;  // loads per slice issue
  static_assert(NBUF == 2 || NBUF == 4, "ring depth");
  static_assert((NBUF - 1) * kPerSlice <= 63, "vmcnt range");
  if constexpr (NBUF == 4) {
    __shared__ __attribute__((aligned(1024))) char lds2[NW * SLICE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds3[NW * SLICE_BYTES];
    char* buf2 = lds2 + wave * SLICE_BYTES;
    char* buf3 = lds3 + wave * SLICE_BYTES;
    issue(0, buf0, xv[0]);
    issue(1, buf1, xv[1]);
    issue(2, buf2, xv[2]);
    issue(3, buf3, xv[3]);
    for (int i = 0; i < nsteps; i += 4) {
      __builtin_amdgcn_s_waitcnt(wait_vm(3 * kPerSlice));
      consume(buf0, xv[0]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 4, buf0, xv[0]);
      __builtin_amdgcn_s_waitcnt(wait_vm(3 * kPerSlice));
      consume(buf1, xv[1]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 5, buf1, xv[1]);
      __builtin_amdgcn_s_waitcnt(wait_vm(3 * kPerSlice));
      consume(buf2, xv[2]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 6, buf2, xv[2]);
      __builtin_amdgcn_s_waitcnt(wait_vm(3 * kPerSlice));
      consume(buf3, xv[3]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 7, buf3, xv[3]);
    }
  } else {
    issue(0, buf0, xv[0]);
    issue(1, buf1, xv[1]);
    for (int i = 0; i < nsteps; i += 2) {
      __builtin_amdgcn_s_waitcnt(wait_vm(kPerSlice));
      consume(buf0, xv[0]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 2, buf0, xv[0]);
      __builtin_amdgcn_s_waitcnt(wait_vm(kPerSlice));
      consume(buf1, xv[1]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue(i + 3, buf1, xv[1]);
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));  // the last issues may still be writing their zeros

  // Add the NW waves' sums in wave order through LDS, 64 columns at a time.
  float* red = reinterpret_cast<float*>(lds0);  // [NW][MT * 16][64]
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
    for (int row = tid >> 6; row < MT * 16; row += NW) {
      float v = red[row * 64 + col];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[(w * MT * 16 + row) * 64 + col];
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
  const dim3 block(Tile<SBN>::NW * 64);
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

// Tile width: 256 columns when that still gives most CUs a workgroup. When
// the caller has room for K-chunk sums, also 256 columns with K split in two
// when the 256-column tiles number 96..128, so that the split gives 192..256
// workgroups: on the decode shape (112 such tiles) that ran about 1% faster
// than 128-column tiles unsplit, the chunk-sum pass included. 128 otherwise,
// and always for 17..32 rows (twice the accumulators).
int tile_width(const GemmDesc& d, bool may_split) {
  if (d.M > 16) return 128;
  const int64_t t256 = (d.N + 255) / 256 * d.batch;
  if (t256 >= 192) return 256;
  if (may_split && t256 >= 96 && t256 <= 128) return 256;
  return 128;
}

int64_t chunk_for(int64_t K, int ksplit) {
  // a multiple of both tile widths' granules, so the split does not depend on the width
  int64_t kc = (K + ksplit - 1) / ksplit;
  kc = (kc + SBK_MAX - 1) / SBK_MAX * SBK_MAX;
  return kc > 0 ? kc : SBK_MAX;
}

}  // namespace

bool gemm_skinny_supported(const GemmDesc& d) {
  if (!d.in_bf16 || d.M < 1 || d.M > kSkinnyMaxRows) return false;
  if (d.a_trans || d.b_trans || (d.act != ACT_NONE && d.act != ACT_GELU)) return false;
  if ((d.K & 7) || (d.N & 7) || (d.lda & 7) || (d.ldb & 7) || (d.sA & 7) || (d.sB & 7)) return false;
  if ((reinterpret_cast<uintptr_t>(d.A) & 15) || (reinterpret_cast<uintptr_t>(d.B) & 15)) return false;
  if ((int64_t)SLICE * d.ldb * 2 >= (1ll << 31)) return false;
  if (((d.M - 1) * d.lda + d.K) * 2 >= (1ll << 31)) return false;
  if (d.batch > 65535 || (d.N + 127) / 128 > 0x7fffffff) return false;
  return true;
}

int skinny_ksplit(const GemmDesc& d) {
  // Split K only when the column tiles of the chosen width leave many CUs
  // idle (fewer than 160 tiles): the chunk sums cost a write, a read and a
  // second launch.
  const int sbn = tile_width(d, true);
  const int64_t tiles = (d.N + sbn - 1) / sbn * d.batch;
  int64_t ks = tiles >= 160 ? 1 : 256 / (tiles > 0 ? tiles : 1);
  const int64_t max_ks = (d.K + SBK_MAX - 1) / SBK_MAX;
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
  p.apart = nullptr;
  p.a_cs = p.a_sz = p.a_ld = 0;
  const int sbn = tile_width(d, ksplit > 1);  // the width skinny_ksplit assumed when it split K
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

bool gemm_skinny_chunked_a_supported(const GemmDesc& d, const ChunkedA& a) {
  if (a.ksplit != kChunkedA || (a.act != ACT_NONE && a.act != ACT_GELU)) return false;
  if (d.M > 16 || d.out_kind != OUT_F32 || d.act != ACT_NONE || !gemm_skinny_supported(d)) return false;
  if (a.ld < d.K || (a.ld & 3) || (a.sz & 3) || (a.cs & 3) || (reinterpret_cast<uintptr_t>(a.part) & 15)) return false;
  if ((16 * a.ld + d.K) * 4 >= (1ll << 31)) return false;  // 32-bit ranges and offsets of all 16 fragment rows
  return (d.N + 127) / 128 * d.batch <= 0x7fffffff;
}

hipError_t launch_gemm_skinny_chunked_a(const GemmDesc& d, const ChunkedA& a, hipStream_t stream) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  if (!gemm_skinny_chunked_a_supported(d, a)) return hipErrorInvalidValue;
  const int act_a = a.act;
  SkParams p;
  p.d = d;
  p.kchunk = d.K;
  p.part = nullptr;
  p.apart = a.part;
  p.a_cs = a.cs;
  p.a_sz = a.sz;
  p.a_ld = a.ld;
  const int sbn = tile_width(d, false);
  const dim3 grid((unsigned)((d.N + sbn - 1) / sbn * d.batch)), block(Tile<128>::NW * 64);
  constexpr int AK = kChunkedA;
  if (sbn == 256) {
    if (act_a == ACT_GELU) gemm_skinny_kernel<256, 1, OUT_F32, ACT_NONE, false, AK, ACT_GELU><<<grid, block, 0, stream>>>(p);
    else gemm_skinny_kernel<256, 1, OUT_F32, ACT_NONE, false, AK, ACT_NONE><<<grid, block, 0, stream>>>(p);
  } else {
    if (act_a == ACT_GELU) gemm_skinny_kernel<128, 1, OUT_F32, ACT_NONE, false, AK, ACT_GELU><<<grid, block, 0, stream>>>(p);
    else gemm_skinny_kernel<128, 1, OUT_F32, ACT_NONE, false, AK, ACT_NONE><<<grid, block, 0, stream>>>(p);
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
