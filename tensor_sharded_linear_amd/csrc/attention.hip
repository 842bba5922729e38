// Attention per head subset on one GPU: for every executed shard and each of
// its query heads h, O_h = softmax(Q_h K_g^T / sqrt(d)) V_g over the tokens of
// each sequence (causal: token i sees tokens 0..i of its sequence), with
// g = h / (hq / hkv) the key/value head the query head reads.
//
// This is the step between the column-parallel QKV projection and the
// row-parallel output projection ([TP-topic] "Tensor Parallelism" topic page,
// chipfoundryservices.com: the figure's panel "Attention Head Parallelism",
// heads split evenly and computed independently, shared key/value heads
// replicated under grouped-query attention; section "Megatron-LM Tensor
// Parallelism", attention layer splitting). A shard's block of the QKV
// output holds its query heads, then its key heads, then its value heads,
// each head_dim columns wide; its output block holds its query heads.
//
// The matrix-core kernel (bf16, head_dim 64 or 128) runs one workgroup of 4
// waves per (128-query block, head, sequence). Each wave owns 32 queries and
// walks the key blocks of 64 with an online softmax, so the scores never
// leave registers:
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows): each lane then
//     holds one query's scores for half the keys, so the row max and sum
//     need one exchange with the lane 32 apart;
//   O^T += V^T P^T: the probabilities go straight from the S^T accumulators
//     into the B operand. The contraction order over a block's keys is free,
//     so it is chosen to match where the accumulators hold them, and the V^T
//     operand is read with ds_read_b64_tr_b16 in that same key order. Each
//     probability enters this product as a bf16 pair (rounded value and
//     rounded remainder, two MFMAs), so P keeps about 16 significant bits
//     instead of bf16's 8, and the softmax normalizer is the fp32 sum of the
//     probabilities themselves.
// K and V tiles come into LDS with LDS-mode buffer loads, two stages deep,
// shared by the 4 waves. Key blocks that every query of the workgroup sees
// run first, with no mask and no branch around their loads; the blocks on the
// causal diagonal or at the sequence tail follow with the mask. Under the
// causal mask a workgroup takes a long query block and then the matching
// short one (x and qblocks - 1 - x), so all workgroups carry about the same
// work. Everything else (fp32 inputs, other head sizes, unaligned strides)
// takes an element-wise fallback kernel.
#include "tp_internal.h"

namespace tp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
#define TP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BQ = 128;   // queries per workgroup (32 per wave)
constexpr int BKV = 64;   // keys per block
constexpr int NTHREADS = 256;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, __builtin_amdgcn_readfirstlane(n),
                                           kRsrcWord3);
}

// Work item of one workgroup: query block qb of head hx (executed-shard head
// index, shard j = hx / hq) of sequence b.
struct AttnParams {
  AttnDesc a;
  int qblocks;  // query blocks per sequence
};

// LDS tile of one K or V block: 64 rows (keys) of DH bf16, 16-byte chunks
// swizzled per row. K: slot = chunk ^ (row % 16), so 16 consecutive keys at
// the same chunk (one b128 read phase) hit 16 distinct slots. V: slot =
// chunk ^ (4 * (row % 4)), so the 4 consecutive keys of a transpose read and
// the two 16-column halves a read pairs up fall on distinct slots.
// max(v of lane l, v of lane l ^ 32): the two halves of the wave are exchanged in registers
// (v_permlane32_swap: the upper half of one copy trades places with the lower half of the other,
// so each lane ends up holding both values of its pair).
// The two halves are copied out of the returned pair before the bit casts: a
// bit cast applied to an element of a vector value was compiled as a cast of
// element 0.
__device__ __forceinline__ float pair_max(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned lo = r[0], hi = r[1];
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

template <int DH>
__device__ __forceinline__ int k_slot(int row, int chunk) { return chunk ^ (row & (DH / 8 - 1)); }
template <int DH>
__device__ __forceinline__ int v_slot(int row, int chunk) { return chunk ^ ((4 * (row & 3)) & (DH / 8 - 1)); }

template <int DH, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2) void attention_mfma_kernel(AttnParams p) {
  constexpr int CPR = DH / 8;              // 16-byte chunks per row
  constexpr int TILE = BKV * DH * 2;       // bytes of one K or V tile
  constexpr int ROWS_PER_REGION = 1024 / (DH * 2);
  constexpr int REGIONS = TILE / 1024;     // 1 KB regions per tile
  constexpr int RPW = REGIONS / 4;         // regions per wave
  constexpr int DT = DH / 32;              // 32-wide d tiles of O^T
  constexpr int KS = DH / 16;              // 16-wide d steps of S^T
  __shared__ __attribute__((aligned(1024))) char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE];

  const AttnDesc& a = p.a;
  // Causal: workgroup x takes query block qblocks - 1 - x (long) and then x
  // (short), so every workgroup has about the same number of key blocks.
  const int npass = CAUSAL && (int)blockIdx.x != p.qblocks - 1 - (int)blockIdx.x ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qb = __builtin_amdgcn_readfirstlane(
        CAUSAL ? (pass == 0 ? p.qblocks - 1 - (int)blockIdx.x : (int)blockIdx.x) : (int)blockIdx.x);
    const int hx = __builtin_amdgcn_readfirstlane((int)blockIdx.y);
    const int b = __builtin_amdgcn_readfirstlane((int)blockIdx.z);
    const int shard = hx / a.hq, h = hx - shard * a.hq;
    const int kvh = h / (a.hq / a.hkv);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t L = a.seq_len;
    const int64_t row0 = (int64_t)b * L;
    const int q0 = qb * BQ;
    const int qw = q0 + wave * 32;                      // first query of this wave
    const int nkeys = CAUSAL ? (int)min<int64_t>(L, q0 + BQ) : (int)L;
    const int nkb = (nkeys + BKV - 1) / BKV;

    const __bf16* blk = static_cast<const __bf16*>(a.qkv) + shard * a.s_qkv + row0 * a.ld_qkv;
    const __bf16* Qh = blk + h * DH;
    const __bf16* Kh = blk + (a.hq + kvh) * DH;
    const __bf16* Vh = blk + (a.hq + a.hkv + kvh) * DH;
    const int64_t ldq = a.ld_qkv;

    // Q^T fragments (B operand of S^T = K Q^T): lane holds query qw + (lane & 31),
    // d values 16 ks + 8 (lane >> 5) .. + 7; queries past the sequence read as zero.
    bf16x8 qf[KS];
    {
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(Qh, ((L - 1) * ldq + DH) * 2);
      const int q = qw + (lane & 31);
      const uint32_t base = q < L ? (uint32_t)((int64_t)q * ldq * 2 + (lane >> 5) * 16) : kOOB;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, base == kOOB ? kOOB : base + ks * 32, 0, 0));
    }

    // LDS-mode loads of key block kb: wave w fills regions w + 4 i; in a region
    // lane l lands at row l / CPR, slot l % CPR and fetches the chunk that slot holds.
    const int lrow = lane / CPR, lslot = lane % CPR;
    auto issue = [&](int kb, char* sk, char* sv) {
      const int k0 = kb * BKV;
      const int64_t krem = L - k0;
      const int rows = krem < BKV ? (int)krem : BKV;
      const int64_t bytes = (int64_t)(((uint32_t)(rows - 1) * (uint32_t)ldq + DH) * 2u);
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kh + (int64_t)k0 * ldq, bytes);
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vh + (int64_t)k0 * ldq, bytes);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int region = wave + 4 * i;
        const int row = region * ROWS_PER_REGION + lrow;
        const uint32_t kvoff = (uint32_t)(lrow * ldq * 2 + k_slot<DH>(row, lslot) * 16);
        const uint32_t vvoff = (uint32_t)(lrow * ldq * 2 + v_slot<DH>(row, lslot) * 16);
        const uint32_t soff = (uint32_t)(region * ROWS_PER_REGION * ldq * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, TP_LDS(sk + wave * 1024 + i * 4096), 16, kvoff, soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, TP_LDS(sv + wave * 1024 + i * 4096), 16, vvoff, soff, 0, 0);
      }
    };

    // V^T fragment addressing (transpose reads): lane (G = lane >> 4, j = lane & 15)
    // supplies key row base + (j >> 2) and d columns 32 dt + 16 (G & 1) + 4 (j & 3)
    // .. + 3, and receives d = 32 dt + (lane & 31) for 4 keys.
    const int G = lane >> 4, j16 = lane & 15;
    const int hh = lane >> 5;  // which half of the keys this lane's S^T values cover

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = a.scale * kLog2e;
    const int myq = qw + (lane & 31);

    // One key block. Full blocks (every key visible to every query of the
    // workgroup) take no mask and no skip, so the main loop over them has no
    // branch around its loads; the few blocks on the diagonal or at the
    // sequence tail come after it.
    auto block = [&](int kb, const char* sk, const char* sv, bool edge) {
      const int k0 = kb * BKV;
      if (edge && CAUSAL && k0 > qw + 31) return;  // every key of the block is past every query of this wave
      // S^T for 64 keys: tile kt covers keys 32 kt .. 32 kt + 31 of the block.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int chunk = 2 * ks + hh;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int row = 32 * kt + (lane & 31);
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sk + row * DH * 2 + (k_slot<DH>(row, chunk) << 4));
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kt], 0, 0, 0);
        }
      }
      // Mask (element e of tile kt is key k0 + 32 kt + 8 (e / 4) + 4 hh + e % 4) only
      // where a key may lie past a query of this wave or past the sequence; the
      // test is uniform across the wave, so other blocks skip it entirely.
      const bool diag = CAUSAL && k0 + BKV - 1 > qw;
      if (edge && (diag || k0 + BKV > L)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (key >= L || (CAUSAL && key > myq)) s[kt][e] = -INFINITY;
          }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, s[kt][e]);
      const float mblk = pair_max(mloc);
      // Scores stay unscaled; the running max m is in score units and the scale
      // c = log2(e) / sqrt(d) enters each exponent through one fused multiply-add.
      // The reference m only moves when some query of the wave would otherwise
      // see a probability above 2^8 (or on the first block): the softmax is
      // unchanged by the choice of reference, so the rescale of O and l (and
      // its exponential) is skipped for most blocks. Every query sees key 0 in
      // the first block, so m is finite from then on.
      const bool move = m_run == -INFINITY || (mblk - m_run) * c > 8.0f;
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float m_new = fmaxf(m_run, mblk);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t] *= alpha;
      }
      const float mc = m_run * c;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], c, -mc));
      float lsum = 0.f;
      // The two waves that share a SIMD come from different workgroups and run
      // unsynchronized; while this wave feeds the value product it takes issue
      // priority, so the other wave's softmax work fills the MFMA gaps rather
      // than delaying the MFMAs (measured 1-3% faster than equal priority;
      // raising it around the score MFMAs as well gained nothing).
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      // O^T += V^T P^T, 16 keys per step; step t takes elements 8 (t % 2) .. + 7 of tile t / 2,
      // i.e. keys 16 t + 8 (i / 4) + 4 hh + i % 4 for i = 0..7 (the k order of this step).
      // Each fp32 probability p is carried as two bf16 values, hi = bf16(p) and
      // lo = bf16(p - hi), and both are multiplied with V: hi + lo holds p to
      // about 2^-17 of itself, so the weights that reach V are the fp32
      // probabilities and the normalizer is their fp32 sum.
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 pf, pl;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {  // two probabilities per conversion instruction
          const f32x2 pv = {s[t >> 1][8 * (t & 1) + i], s[t >> 1][8 * (t & 1) + i + 1]};
          const bf16x2 hi = __builtin_convertvector(pv, bf16x2);
          const bf16x2 lo = __builtin_convertvector(pv - __builtin_convertvector(hi, f32x2), bf16x2);
          pf[i] = hi[0];
          pf[i + 1] = hi[1];
          pl[i] = lo[0];
          pl[i + 1] = lo[1];
          lsum += pv[0];
          lsum += pv[1];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x4 half[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int row = 16 * t + 8 * r + 4 * (G >> 1) + (j16 >> 2);
            const int byte = (32 * dt + 16 * (G & 1) + 4 * (j16 & 3)) * 2;
            const int chunk = byte >> 4;
            const char* ptr = sv + row * DH * 2 + (v_slot<DH>(row, chunk) << 4) + (byte & 8);
            half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)ptr);
          }
          const bf16x8 vf = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[dt], 0, 0, 0);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl, o[dt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      l_run += lsum;
    };

    // blocks whose keys every query of the workgroup sees, and are inside the sequence
    const int nfull = CAUSAL ? q0 / BKV : (int)(L / BKV);
    if (nkb > 0) {
      issue(0, sK0, sV0);
      __syncthreads();
    }
    int kb = 0;
    for (; kb + 1 < nfull; kb += 2) {
      issue(kb + 1, sK1, sV1);
      block(kb, sK0, sV0, false);
      __syncthreads();
      if (kb + 2 < nkb) issue(kb + 2, sK0, sV0);
      block(kb + 1, sK1, sV1, false);
      __syncthreads();
    }
    if (kb < nfull) {
      if (kb + 1 < nkb) issue(kb + 1, sK1, sV1);
      block(kb, sK0, sV0, false);
      __syncthreads();
      ++kb;
    }
    for (; kb < nkb; ++kb) {
      if (kb & 1) {
        if (kb + 1 < nkb) issue(kb + 1, sK0, sV0);
        block(kb, sK1, sV1, true);
      } else {
        if (kb + 1 < nkb) issue(kb + 1, sK1, sV1);
        block(kb, sK0, sV0, true);
      }
      __syncthreads();
    }

    // O = O^T / l: lane holds query myq; element e of tile dt is d = 32 dt + 8 (e / 4) + 4 hh + e % 4,
    // so each group of 4 elements is 4 consecutive d (8 bytes).
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    char* ob = static_cast<char*>(a.out) + (shard * a.s_out + row0 * a.ld_out + h * DH) * 2;
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(ob, ((L - 1) * a.ld_out + DH) * 2);
    const uint32_t obase = myq < L ? (uint32_t)((int64_t)myq * a.ld_out * 2) : kOOB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hh;
        unsigned short hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = __builtin_bit_cast(unsigned short, (__bf16)(o[dt][4 * g4 + i] * inv));
        const u32x2 w = {(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(w, orr, obase == kOOB ? kOOB : obase + d0 * 2, 0, 0);
      }
    __syncthreads();  // the next pass refills the K/V buffers
  }
}

// Element-wise fallback: one workgroup of 64 threads per (query, head, shard).
// Scores of the visible keys go to LDS (float), then the max, the sum and the
// weighted sum of values, all in fp32 in ascending key order per thread.
constexpr int kFallbackMaxKeys = 8192;

template <typename T>
__global__ __launch_bounds__(64) void attention_generic_kernel(AttnDesc a) {
  __shared__ float sc[kFallbackMaxKeys];
  __shared__ float red[64];
  const int64_t row = blockIdx.x;  // token index in [0, M)
  const int hx = blockIdx.y;
  const int shard = hx / a.hq, h = hx - shard * a.hq;
  const int kvh = h / (a.hq / a.hkv);
  const int tid = threadIdx.x;
  const int64_t L = a.seq_len;
  const int64_t b = row / L, i = row - b * L;
  const int64_t nk = a.causal ? i + 1 : L;
  const int dh = a.head_dim;
  const T* blk = static_cast<const T*>(a.qkv) + shard * a.s_qkv + b * L * a.ld_qkv;
  const T* q = blk + i * a.ld_qkv + h * dh;
  const T* K = blk + (a.hq + kvh) * dh;
  const T* V = blk + (a.hq + a.hkv + kvh) * dh;
  float mx = -INFINITY;
  for (int64_t j = tid; j < nk; j += 64) {
    float acc = 0.f;
    for (int t = 0; t < dh; ++t) acc = fmaf((float)q[t], (float)K[j * a.ld_qkv + t], acc);
    acc *= a.scale;
    sc[j] = acc;
    mx = fmaxf(mx, acc);
  }
  red[tid] = mx;
  __syncthreads();
  for (int s = 32; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int64_t j = tid; j < nk; j += 64) {
    const float e = expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  red[tid] = sum;
  __syncthreads();
  for (int s = 32; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  T* out = static_cast<T*>(a.out) + shard * a.s_out + row * a.ld_out + h * dh;
  for (int t = tid; t < dh; t += 64) {
    float acc = 0.f;
    for (int64_t j = 0; j < nk; ++j) acc = fmaf(sc[j], (float)V[j * a.ld_qkv + t], acc);
    out[t] = (T)(acc * inv);
  }
}

}  // namespace

bool attention_mfma_supported(const AttnDesc& a) {
  if (!a.in_bf16 || (a.head_dim != 64 && a.head_dim != 128)) return false;
  if ((a.ld_qkv & 7) || (a.s_qkv & 7) || (a.ld_out & 3) || (a.s_out & 3)) return false;
  if ((reinterpret_cast<uintptr_t>(a.qkv) & 15) || (reinterpret_cast<uintptr_t>(a.out) & 7)) return false;
  // 31-bit buffer offsets within one sequence
  if (a.seq_len * a.ld_qkv * 2 >= (1ll << 31) || a.seq_len * a.ld_out * 2 >= (1ll << 31)) return false;
  return true;
}

bool attention_generic_supported(const AttnDesc& a) { return a.seq_len <= kFallbackMaxKeys; }

hipError_t launch_attention(const AttnDesc& a, hipStream_t stream) {
  const int64_t heads = (int64_t)a.hq * a.shards;
  const int64_t seqs = a.seq_len > 0 ? a.tokens / a.seq_len : 0;
  if (heads <= 0 || seqs <= 0) return hipSuccess;
  if (heads > 65535 || seqs > 65535) return hipErrorInvalidValue;
  if (attention_mfma_supported(a)) {
    AttnParams p;
    p.a = a;
    p.qblocks = (int)((a.seq_len + BQ - 1) / BQ);
    const unsigned gx = a.causal ? (unsigned)((p.qblocks + 1) / 2) : (unsigned)p.qblocks;
    const dim3 grid(gx, (unsigned)heads, (unsigned)seqs), block(NTHREADS);
    if (a.head_dim == 128) {
      if (a.causal) attention_mfma_kernel<128, true><<<grid, block, 0, stream>>>(p);
      else attention_mfma_kernel<128, false><<<grid, block, 0, stream>>>(p);
    } else {
      if (a.causal) attention_mfma_kernel<64, true><<<grid, block, 0, stream>>>(p);
      else attention_mfma_kernel<64, false><<<grid, block, 0, stream>>>(p);
    }
    return hipGetLastError();
  }
  if (!attention_generic_supported(a)) return hipErrorInvalidValue;
  if (a.tokens > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.tokens, (unsigned)heads), block(64);
  if (a.in_bf16) attention_generic_kernel<__bf16><<<grid, block, 0, stream>>>(a);
  else attention_generic_kernel<float><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace tp
