// AdamW for the parameters Muon does not take (embeddings, output head,
// norms, biases): one launch updates every tensor of a parameter group.
//
//   m <- beta1*m + (1-beta1)*g,  v <- beta2*v + (1-beta2)*g^2
//   theta <- (1 - lr*wd)*theta - lr * (m*c1) / (sqrt(v*c2) + eps)
//
// with the bias corrections c1 = 1/(1-beta1^t), c2 = 1/(1-beta2^t) computed
// on the host ("LLM Optimizers: From SGD and AdamW to SOAP, Muon, and
// Scalable Training", sections 5 and 6).  Arithmetic is fp32; a bf16
// parameter is rounded once to nearest even.
//
// Work split: every tensor is cut into chunks of kChunk elements; the
// caller's chunk table (prefix sums of the per-tensor chunk counts) maps a
// workgroup to its tensor by binary search.  Each workgroup streams one
// chunk with 16-byte accesses (8 elements per thread step, every load of the
// chunk issued before the first store); a partial last chunk finishes
// element by element.  Every access is bounded by the tensor's own numel,
// whatever the chunk table holds.

#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kAdamWChunk / kThreads;  // 16
constexpr int kVec = 8;
static_assert(kPerThread % kVec == 0, "whole 16-byte groups per thread");

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16); }

__device__ __forceinline__ void load8(const char* p, int bf16, float* v) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
      v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ void store8(char* p, int bf16, const float* v) {
  if (bf16) {
    uint4 u;
    u.x = to_bf16(v[0]) | (static_cast<uint32_t>(to_bf16(v[1])) << 16);
    u.y = to_bf16(v[2]) | (static_cast<uint32_t>(to_bf16(v[3])) << 16);
    u.z = to_bf16(v[4]) | (static_cast<uint32_t>(to_bf16(v[5])) << 16);
    u.w = to_bf16(v[6]) | (static_cast<uint32_t>(to_bf16(v[7])) << 16);
    *reinterpret_cast<uint4*>(p) = u;
  } else {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

struct Step {
  float b1, omb1, b2, omb2, c1, c2, lr, eps, decay;
  __device__ __forceinline__ void operator()(float& p, float g, float& m, float& v) const {
    m = b1 * m + omb1 * g;
    v = b2 * v + omb2 * g * g;
    p = decay * p - lr * (m * c1) / (sqrtf(v * c2) + eps);
  }
};

__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamWArgs a) {
  // tensor of this chunk: the last i with chunk_offsets[i] <= blockIdx.x
  const int64_t chunk = blockIdx.x;
  int64_t lo = 0, hi = a.count - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (a.chunk_offsets[mid] <= chunk) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  const int64_t t = lo;
  const int64_t numel = a.numels[t];
  const int64_t start = (chunk - a.chunk_offsets[t]) * kAdamWChunk;
  if (start < 0 || start >= numel) return;  // an inconsistent chunk table: nothing to do here
  const int64_t len = numel - start < kAdamWChunk ? numel - start : kAdamWChunk;
  const int ps = a.param_bf16 ? 2 : 4;
  const int gs = a.grad_bf16 ? 2 : 4;
  char* P = static_cast<char*>(a.params[t]) + start * ps;
  const char* G = static_cast<const char*>(a.grads[t]) + start * gs;
  float* M = a.exp_avg[t] + start;
  float* V = a.exp_avg_sq[t] + start;
  const Step op{a.beta1, 1.0f - a.beta1, a.beta2, 1.0f - a.beta2, a.c1, a.c2, a.lr, a.eps, a.decay};

  if (len == kAdamWChunk) {
    float p[kPerThread / kVec][kVec], g[kPerThread / kVec][kVec], m[kPerThread / kVec][kVec],
        v[kPerThread / kVec][kVec];
#pragma unroll
    for (int u = 0; u < kPerThread / kVec; ++u) {
      const int e = (u * kThreads + threadIdx.x) * kVec;
      load8(P + e * ps, a.param_bf16, p[u]);
      load8(G + e * gs, a.grad_bf16, g[u]);
      load8(reinterpret_cast<const char*>(M + e), 0, m[u]);
      load8(reinterpret_cast<const char*>(V + e), 0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kPerThread / kVec; ++u) {
      const int e = (u * kThreads + threadIdx.x) * kVec;
#pragma unroll
      for (int k = 0; k < kVec; ++k) op(p[u][k], g[u][k], m[u][k], v[u][k]);
      store8(P + e * ps, a.param_bf16, p[u]);
      store8(reinterpret_cast<char*>(M + e), 0, m[u]);
      store8(reinterpret_cast<char*>(V + e), 0, v[u]);
    }
  } else {
    for (int e = threadIdx.x; e < len; e += kThreads) {
      float p = a.param_bf16 ? from_bf16(reinterpret_cast<const uint16_t*>(P)[e]) : reinterpret_cast<const float*>(P)[e];
      const float g = a.grad_bf16 ? from_bf16(reinterpret_cast<const uint16_t*>(G)[e]) : reinterpret_cast<const float*>(G)[e];
      float m = M[e], v = V[e];
      op(p, g, m, v);
      if (a.param_bf16) {
        reinterpret_cast<uint16_t*>(P)[e] = to_bf16(p);
      } else {
        reinterpret_cast<float*>(P)[e] = p;
      }
      M[e] = m;
      V[e] = v;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamWArgs& a, int64_t total_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned>(total_chunks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muon
