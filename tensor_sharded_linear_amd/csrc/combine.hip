// Combining shard outputs on one GPU.
//
// Sum (the local form of the all-reduce): Y = P_0 + P_1 + ... + P_{n-1} in
// fp32, added in ascending shard order so that every run gives the same bits.
// Concatenation (the local form of the all-gather): Y = [P_0 | ... | P_{n-1}],
// or the blocks stacked by rows (token shards gathered back in order, the
// all-gather of sequence parallelism).
// The rule for choosing between them is the one of the "Tensor Parallelism"
// entry of the AI Glossary (aiforbusinessandlife.com), "Check your
// understanding": partial results for the same output coordinates are added,
// results for different coordinates are concatenated; the collectives are
// those of the "Tensor Parallelism" topic page (chipfoundryservices.com),
// "Tensor Parallelism Fundamentals".
//
// Both are bound by HBM traffic: every lane streams 16-byte vectors.
#include "tp_internal.h"

namespace tp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t grid_threads() { return (int64_t)gridDim.x * blockDim.x; }
__device__ __forceinline__ int64_t thread_index() { return (int64_t)blockIdx.x * blockDim.x + threadIdx.x; }

template <bool YBF16>
__global__ __launch_bounds__(256) void sum_vec4_kernel(CombineDesc d) {
  const int64_t c4 = d.cols >> 2;
  const int64_t total = d.rows * c4;
  const float* P = static_cast<const float*>(d.P);
  const int n = d.n;
  for (int64_t i = thread_index(); i < total; i += grid_threads()) {
    const int64_t r = i / c4, c = (i - r * c4) << 2;
    const f32x4* src = reinterpret_cast<const f32x4*>(P + r * d.ldp + c);
    const int64_t step = d.sP >> 2;  // shard stride in 16-byte vectors
    // The partials are read once: nontemporal loads, four shards in flight at
    // a time, added strictly in ascending shard order.
    f32x4 acc = __builtin_nontemporal_load(src);
    int j = 1;
    for (; j + 4 <= n; j += 4) {
      const f32x4 a = __builtin_nontemporal_load(src + (int64_t)j * step);
      const f32x4 b = __builtin_nontemporal_load(src + (int64_t)(j + 1) * step);
      const f32x4 e = __builtin_nontemporal_load(src + (int64_t)(j + 2) * step);
      const f32x4 f = __builtin_nontemporal_load(src + (int64_t)(j + 3) * step);
      acc += a;
      acc += b;
      acc += e;
      acc += f;
    }
    for (; j < n; ++j) acc += __builtin_nontemporal_load(src + (int64_t)j * step);
    if (YBF16) {
      bf16x4 h;
      h[0] = (__bf16)acc[0]; h[1] = (__bf16)acc[1]; h[2] = (__bf16)acc[2]; h[3] = (__bf16)acc[3];
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(d.Y) + r * d.ldy + c) = h;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(d.Y) + r * d.ldy + c) = acc;
    }
  }
}

template <bool YBF16>
__global__ __launch_bounds__(256) void sum_scalar_kernel(CombineDesc d) {
  const int64_t total = d.rows * d.cols;
  const float* P = static_cast<const float*>(d.P);
  for (int64_t i = thread_index(); i < total; i += grid_threads()) {
    const int64_t r = i / d.cols, c = i - r * d.cols;
    const float* src = P + r * d.ldp + c;
    float acc = src[0];
    for (int j = 1; j < d.n; ++j) acc += src[(int64_t)j * d.sP];
    if (YBF16) static_cast<__bf16*>(d.Y)[r * d.ldy + c] = (__bf16)acc;
    else static_cast<float*>(d.Y)[r * d.ldy + c] = acc;
  }
}

template <bool PBF16, bool YBF16>
__global__ __launch_bounds__(256) void concat_kernel(CombineDesc d) {
  const int64_t per = d.rows * d.cols;
  const int64_t total = per * d.n;
  for (int64_t i = thread_index(); i < total; i += grid_threads()) {
    const int64_t j = i / per, rem = i - j * per;
    const int64_t r = rem / d.cols, c = rem - r * d.cols;
    const int64_t src = j * d.sP + r * d.ldp + c;
    const float v = PBF16 ? (float)static_cast<const __bf16*>(d.P)[src] : static_cast<const float*>(d.P)[src];
    // concat 1: blocks side by side (columns); 2: stacked (rows)
    const int64_t dst = d.concat == 2 ? (j * d.rows + r) * d.ldy + c : r * d.ldy + j * d.cols + c;
    if (YBF16) static_cast<__bf16*>(d.Y)[dst] = (__bf16)v;
    else static_cast<float*>(d.Y)[dst] = v;
  }
}

// The same gather four elements per lane (8 or 16 bytes each way) for aligned
// layouts: lanes run along a row of one block, workgroups over column chunks,
// rows and blocks, so no index needs a division.
template <bool PBF16, bool YBF16>
__global__ __launch_bounds__(256) void concat_vec4_kernel(CombineDesc d) {
  const int64_t c4 = d.cols >> 2;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= c4) return;
  for (int64_t j = blockIdx.z; j < d.n; j += gridDim.z)
    for (int64_t r = blockIdx.y; r < d.rows; r += gridDim.y) {
      const int64_t src = j * d.sP + r * d.ldp + 4 * c;
      f32x4 v;
      if (PBF16) {
        const bf16x4 h = __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(d.P) + src));
        v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
      } else {
        v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(d.P) + src));
      }
      const int64_t dst = d.concat == 2 ? (j * d.rows + r) * d.ldy + 4 * c : r * d.ldy + j * d.cols + 4 * c;
      if (YBF16) {
        bf16x4 h;
        h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(d.Y) + dst) = h;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(d.Y) + dst) = v;
      }
    }
}

dim3 grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // 32 workgroups per CU, grid-stride beyond
  if (blocks < 1) blocks = 1;
  return dim3((unsigned)blocks);
}

}  // namespace

hipError_t launch_combine(const CombineDesc& d, hipStream_t stream) {
  if (d.rows <= 0 || d.cols <= 0 || d.n <= 0) return hipSuccess;
  const dim3 block(256);
  if (d.concat) {
    const int64_t pe = d.p_bf16 ? 2 : 4, ye = d.y_bf16 ? 2 : 4;
    const bool vec = (d.cols % 4 == 0) && (d.ldp % 4 == 0) && (d.sP % 4 == 0) && (d.ldy % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(d.P) % (4 * pe) == 0) &&
                     (reinterpret_cast<uintptr_t>(d.Y) % (4 * ye) == 0);
    if (vec) {
      // about 32 workgroups per CU in all: rows and blocks beyond the grid are looped over
      const int64_t cx = (d.cols / 4 + 255) / 256;
      const int64_t budget = 8192;
      int64_t gy = (budget + cx - 1) / cx;
      gy = gy < d.rows ? gy : d.rows;
      gy = gy < 65535 ? gy : 65535;
      int64_t gz = budget / (cx * gy);
      gz = gz < 1 ? 1 : gz;
      gz = gz < d.n ? gz : d.n;
      gz = gz < 65535 ? gz : 65535;
      const dim3 grid((unsigned)cx, (unsigned)gy, (unsigned)gz);
      if (d.p_bf16) {
        if (d.y_bf16) concat_vec4_kernel<true, true><<<grid, block, 0, stream>>>(d);
        else concat_vec4_kernel<true, false><<<grid, block, 0, stream>>>(d);
      } else {
        if (d.y_bf16) concat_vec4_kernel<false, true><<<grid, block, 0, stream>>>(d);
        else concat_vec4_kernel<false, false><<<grid, block, 0, stream>>>(d);
      }
      return hipGetLastError();
    }
    const dim3 grid = grid_for(d.rows * d.cols * d.n);
    if (d.p_bf16) {
      if (d.y_bf16) concat_kernel<true, true><<<grid, block, 0, stream>>>(d);
      else concat_kernel<true, false><<<grid, block, 0, stream>>>(d);
    } else {
      if (d.y_bf16) concat_kernel<false, true><<<grid, block, 0, stream>>>(d);
      else concat_kernel<false, false><<<grid, block, 0, stream>>>(d);
    }
    return hipGetLastError();
  }
  const bool vec = (d.cols % 4 == 0) && (d.ldp % 4 == 0) && (d.sP % 4 == 0) && (d.ldy % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(d.P) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(d.Y) % (d.y_bf16 ? 8 : 16) == 0);
  if (vec) {
    const dim3 grid = grid_for(d.rows * (d.cols / 4));
    if (d.y_bf16) sum_vec4_kernel<true><<<grid, block, 0, stream>>>(d);
    else sum_vec4_kernel<false><<<grid, block, 0, stream>>>(d);
  } else {
    const dim3 grid = grid_for(d.rows * d.cols);
    if (d.y_bf16) sum_scalar_kernel<true><<<grid, block, 0, stream>>>(d);
    else sum_scalar_kernel<false><<<grid, block, 0, stream>>>(d);
  }
  return hipGetLastError();
}

}  // namespace tp
