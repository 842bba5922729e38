// Sequence-parallel layer boundary on one GPU: the reduce-scatter of the
// row-parallel partials, dropout, the residual add and LayerNorm, fused in one
// pass over each token row of the executed token shards ([TP-topic] "Tensor
// Parallelism" topic page, chipfoundryservices.com, section "Sequence
// Parallelism Extension": the tokens are split over the shards for LayerNorm
// and Dropout, each shard handling its own subset of tokens).
//
// One workgroup of 256 threads per token row; each thread keeps its share of
// the row in registers as float4 vectors, so the partials are read once
// (nontemporal, added in ascending shard order) and the statistics take two
// passes over registers: the mean, then the mean squared deviation (biased
// variance). Bound by HBM traffic.
#include "tp_internal.h"

namespace tp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;

// Sum of v over the workgroup (every thread receives it).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read from the previous reduction
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int V4, bool RBF16, bool YBF16>
__global__ __launch_bounds__(NT) void sp_layernorm_kernel(LnDesc d) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;  // executed token row
  const int64_t j = i / d.rows_per_shard, r = i - j * d.rows_per_shard;
  const int tid = threadIdx.x;
  const int64_t c4 = d.cols >> 2;
  f32x4 x[V4];
  // reduce-scatter: this token's partials, ascending shard order
#pragma unroll
  for (int v = 0; v < V4; ++v) {
    const int64_t q = tid + (int64_t)NT * v;
    x[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (q < c4) {
      const f32x4* src = reinterpret_cast<const f32x4*>(d.P + i * d.ldp) + q;
      const int64_t step = d.sP >> 2;
      f32x4 acc = __builtin_nontemporal_load(src);
      for (int t = 1; t < d.n; ++t) acc += __builtin_nontemporal_load(src + t * step);
      if (d.keep) {
        const uint32_t k = *reinterpret_cast<const uint32_t*>(d.keep + i * d.cols + 4 * q);
        acc[0] *= (float)(k & 0xff) * d.keep_scale;
        acc[1] *= (float)((k >> 8) & 0xff) * d.keep_scale;
        acc[2] *= (float)((k >> 16) & 0xff) * d.keep_scale;
        acc[3] *= (float)(k >> 24) * d.keep_scale;
      }
      if (d.R) {
        if (RBF16) {
          const bf16x4 rv = *(reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(d.R) + j * d.sR + r * d.ldr) + q);
          acc[0] += (float)rv[0];
          acc[1] += (float)rv[1];
          acc[2] += (float)rv[2];
          acc[3] += (float)rv[3];
        } else {
          acc += *(reinterpret_cast<const f32x4*>(static_cast<const float*>(d.R) + j * d.sR + r * d.ldr) + q);
        }
      }
      x[v] = acc;
      if (d.X1) *(reinterpret_cast<f32x4*>(d.X1 + j * d.sX1 + r * d.ldx1) + q) = acc;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < V4; ++v) s += (x[v][0] + x[v][1]) + (x[v][2] + x[v][3]);
  const float mean = block_sum(s, red) / (float)d.cols;
  float s2 = 0.f;
#pragma unroll
  for (int v = 0; v < V4; ++v) {
    if (tid + (int64_t)NT * v < c4) {
      const f32x4 dv = x[v] - mean;
      s2 += (dv[0] * dv[0] + dv[1] * dv[1]) + (dv[2] * dv[2] + dv[3] * dv[3]);
    }
  }
  const float var = block_sum(s2, red) / (float)d.cols;
  const float rstd = 1.0f / __builtin_sqrtf(var + d.eps);
#pragma unroll
  for (int v = 0; v < V4; ++v) {
    const int64_t q = tid + (int64_t)NT * v;
    if (q < c4) {
      const f32x4 g = reinterpret_cast<const f32x4*>(d.gamma)[q];
      const f32x4 b = reinterpret_cast<const f32x4*>(d.beta)[q];
      const f32x4 y = (x[v] - mean) * rstd * g + b;
      if (YBF16) {
        bf16x4 h;
        h[0] = (__bf16)y[0];
        h[1] = (__bf16)y[1];
        h[2] = (__bf16)y[2];
        h[3] = (__bf16)y[3];
        *(reinterpret_cast<bf16x4*>(static_cast<__bf16*>(d.Y) + j * d.sY + r * d.ldy) + q) = h;
      } else {
        *(reinterpret_cast<f32x4*>(static_cast<float*>(d.Y) + j * d.sY + r * d.ldy) + q) = y;
      }
    }
  }
}

// Any width or alignment: the row is recomputed from memory for each pass.
template <bool RBF16, bool YBF16>
__global__ __launch_bounds__(NT) void sp_layernorm_scalar_kernel(LnDesc d) {
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const int64_t j = i / d.rows_per_shard, r = i - j * d.rows_per_shard;
  const int tid = threadIdx.x;
  auto value = [&](int64_t c) {
    float acc = d.P[i * d.ldp + c];
    for (int t = 1; t < d.n; ++t) acc += d.P[t * d.sP + i * d.ldp + c];
    if (d.keep) acc *= (float)d.keep[i * d.cols + c] * d.keep_scale;
    if (d.R) {
      const int64_t o = j * d.sR + r * d.ldr + c;
      acc += RBF16 ? (float)static_cast<const __bf16*>(d.R)[o] : static_cast<const float*>(d.R)[o];
    }
    return acc;
  };
  float s = 0.f;
  for (int64_t c = tid; c < d.cols; c += NT) {
    const float v = value(c);
    s += v;
    if (d.X1) d.X1[j * d.sX1 + r * d.ldx1 + c] = v;
  }
  const float mean = block_sum(s, red) / (float)d.cols;
  float s2 = 0.f;
  for (int64_t c = tid; c < d.cols; c += NT) {
    const float dv = value(c) - mean;
    s2 += dv * dv;
  }
  const float var = block_sum(s2, red) / (float)d.cols;
  const float rstd = 1.0f / __builtin_sqrtf(var + d.eps);
  for (int64_t c = tid; c < d.cols; c += NT) {
    const float y = (value(c) - mean) * rstd * d.gamma[c] + d.beta[c];
    const int64_t o = j * d.sY + r * d.ldy + c;
    if (YBF16) static_cast<__bf16*>(d.Y)[o] = (__bf16)y;
    else static_cast<float*>(d.Y)[o] = y;
  }
}

template <int V4>
void launch_v4(const LnDesc& d, hipStream_t s) {
  const dim3 grid((unsigned)d.rows), block(NT);
  if (d.r_bf16) {
    if (d.y_bf16) sp_layernorm_kernel<V4, true, true><<<grid, block, 0, s>>>(d);
    else sp_layernorm_kernel<V4, true, false><<<grid, block, 0, s>>>(d);
  } else {
    if (d.y_bf16) sp_layernorm_kernel<V4, false, true><<<grid, block, 0, s>>>(d);
    else sp_layernorm_kernel<V4, false, false><<<grid, block, 0, s>>>(d);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_sp_layernorm(const LnDesc& d, hipStream_t stream) {
  if (d.rows <= 0 || d.cols <= 0) return hipSuccess;
  if (d.rows >= (1ll << 24)) return hipErrorInvalidValue;  // 256 * rows work-items must stay below 2^32
  const int64_t c4 = (d.cols + 3) / 4;
  const bool vec = d.cols % 4 == 0 && d.ldp % 4 == 0 && d.sP % 4 == 0 && aligned16(d.P) && aligned16(d.gamma) &&
                   aligned16(d.beta) && d.ldy % 4 == 0 && d.sY % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(d.Y) & (d.y_bf16 ? 7 : 15)) == 0 &&
                   (!d.X1 || (d.ldx1 % 4 == 0 && d.sX1 % 4 == 0 && aligned16(d.X1))) &&
                   (!d.R || (d.ldr % 4 == 0 && d.sR % 4 == 0 &&
                             (reinterpret_cast<uintptr_t>(d.R) & (d.r_bf16 ? 7 : 15)) == 0)) &&
                   (!d.keep || (reinterpret_cast<uintptr_t>(d.keep) & 3) == 0);
  if (vec && c4 <= 16 * NT) {
    const int64_t per = (c4 + NT - 1) / NT;
    if (per <= 1) launch_v4<1>(d, stream);
    else if (per <= 2) launch_v4<2>(d, stream);
    else if (per <= 4) launch_v4<4>(d, stream);
    else if (per <= 8) launch_v4<8>(d, stream);
    else launch_v4<16>(d, stream);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)d.rows), block(NT);
  if (d.r_bf16) {
    if (d.y_bf16) sp_layernorm_scalar_kernel<true, true><<<grid, block, 0, stream>>>(d);
    else sp_layernorm_scalar_kernel<true, false><<<grid, block, 0, stream>>>(d);
  } else {
    if (d.y_bf16) sp_layernorm_scalar_kernel<false, true><<<grid, block, 0, stream>>>(d);
    else sp_layernorm_scalar_kernel<false, false><<<grid, block, 0, stream>>>(d);
  }
  return hipGetLastError();
}

}  // namespace tp
