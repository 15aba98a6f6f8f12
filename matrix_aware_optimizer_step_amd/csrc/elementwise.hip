// HBM-bound kernels of the Muon step on gfx950:
//
//   momentum_kernel   M <- beta*M + (1-beta)*G and the Nesterov blend N
//                     ("Reading notes on SOAP, Muon and higher-order
//                     optimizers", section 1; "LLM Optimizers: From SGD and
//                     AdamW to SOAP, Muon, and Scalable Training", section
//                     11.3), with per-workgroup partial sums of N^2 for the
//                     Frobenius norm of section 11.4;
//   finalize_kernel   one fixed-order fp64 reduction of those partials per
//                     matrix (deterministic; no float atomics);
//   apply_kernel      W <- (1 - lr*wd)*W - lr*s*O (section 11.5);
//   pack_kernel       N / (||N||_F + eps) into the padded Newton-Schulz
//                     buffers: X (the wide orientation), X^T where the
//                     update reads it, the low part of X for bf16 compute,
//                     through an LDS tile transpose so that reads and writes
//                     stay coalesced;
//   copy_out_kernel   the zero-step output, N / (||N||_F + eps).
//
// The streaming kernels move 16 bytes per lane per access (8 bf16 or 4+4
// fp32 values per thread step), reduce with wave64 shuffles and one LDS
// exchange per workgroup, and address rows through a multiply-high division
// so that matrices with ld > cols (row blocks of a larger weight) need no
// separate path.

#include "lo8.h"
#include "muon_internal.h"

namespace muon {

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.l = l;
  // m = floor(2^32 * (2^l - d) / d) + 1
  f.m = static_cast<uint32_t>(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  return f;
}

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;        // elements per thread step
constexpr int kUnroll = 4;     // thread steps per workgroup pass
constexpr int kElemsPerBlock = kThreads * kVec * kUnroll;  // 8192

__device__ __forceinline__ uint32_t fdiv(const FastDiv& f, uint32_t n) {
  const uint64_t t = static_cast<uint64_t>(__umulhi(n, f.m)) + n;
  return static_cast<uint32_t>(t >> f.l);
}

__device__ __forceinline__ char* mat_ptr(const MatBatch& m, int64_t i) {
  return m.ptrs ? static_cast<char*>(m.ptrs[i]) : m.base + i * m.stride_bytes;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// Load 8 consecutive values of a bf16 or f32 matrix as fp32.
__device__ __forceinline__ void load8(const char* p, int dtype, float* v) {
  if (dtype) {
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

__device__ __forceinline__ void store8(char* p, int dtype, const float* v) {
  if (dtype) {
    uint4 u;
    u.x = bf16_pair(v[0], v[1]);
    u.y = bf16_pair(v[2], v[3]);
    u.z = bf16_pair(v[4], v[5]);
    u.w = bf16_pair(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
  } else {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Four consecutive values (8 bytes of bf16 or 16 of f32, aligned) as fp32.
__device__ __forceinline__ void load4(const char* p, int dtype, float* v) {
  if (dtype) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __builtin_bit_cast(float, u.x << 16);
    v[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
    v[2] = __builtin_bit_cast(float, u.y << 16);
    v[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}

__device__ __forceinline__ void store4(char* p, int dtype, const float* v) {
  if (dtype) {
    uint2 u;
    u.x = bf16_pair(v[0], v[1]);
    u.y = bf16_pair(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__device__ __forceinline__ float load1(const char* p, int dtype) {
  return dtype ? bf16_to_f32(*reinterpret_cast<const uint16_t*>(p)) : *reinterpret_cast<const float*>(p);
}
__device__ __forceinline__ void store1(char* p, int dtype, float v) {
  if (dtype) {
    *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
  } else {
    *reinterpret_cast<float*>(p) = v;
  }
}

// Workgroup sum of one float per thread; result valid in thread 0.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) s += red[i];
  }
  return s;
}

// ------------------------------------------------------------ momentum

// Block `blk` of matrix `mat`: the kernels below differ only in how a
// workgroup finds its (matrix, block) and its group's arguments.
template <bool VEC>
__device__ __forceinline__ void momentum_block(const MomentumArgs& a, int64_t mat, uint32_t blk, float* red) {
  const char* g = mat_ptr(a.G, mat);
  char* m = mat_ptr(a.M, mat);
  char* n = a.has_n ? mat_ptr(a.N, mat) : nullptr;
  const int gs = a.G.dtype ? 2 : 4;
  const int ns = a.N.dtype ? 2 : 4;
  const uint32_t total = static_cast<uint32_t>(a.rows) * static_cast<uint32_t>(a.cols);
  const float beta = a.beta;
  const float omb = 1.0f - a.beta;
  float ss = 0.0f;
  const uint32_t base = blk * kElemsPerBlock;
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = base + (u * kThreads + threadIdx.x) * kVec;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        float gv[kVec], mv[kVec], nv[kVec];
        load8(g + (r * a.G.ld + c) * gs, a.G.dtype, gv);
        float* mp = reinterpret_cast<float*>(m + (r * a.M.ld + c) * 4);
        load8(reinterpret_cast<const char*>(mp), 0, mv);
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          mv[k] = beta * mv[k] + omb * gv[k];
          nv[k] = a.nesterov ? omb * gv[k] + beta * mv[k] : mv[k];
          ss += nv[k] * nv[k];
        }
        store8(reinterpret_cast<char*>(mp), 0, mv);
        if (n) store8(n + (r * a.N.ld + c) * ns, a.N.dtype, nv);
      }
    }
  } else {
    for (int u = 0; u < kUnroll * kVec; ++u) {
      const uint32_t e = base + u * kThreads + threadIdx.x;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        const float gv = load1(g + (r * a.G.ld + c) * gs, a.G.dtype);
        float* mp = reinterpret_cast<float*>(m + (r * a.M.ld + c) * 4);
        const float mv = beta * *mp + omb * gv;
        const float nv = a.nesterov ? omb * gv + beta * mv : mv;
        ss += nv * nv;
        *mp = mv;
        if (n) store1(n + (r * a.N.ld + c) * ns, a.N.dtype, nv);
      }
    }
  }
  const float s = block_sum(ss, red);
  if (threadIdx.x == 0) a.partials[mat * a.blocks_per_mat + blk] = s;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const MomentumArgs a) {
  __shared__ float red[kThreads / 64];
  momentum_block<VEC>(a, blockIdx.y, blockIdx.x, red);
}

// The group that workgroup b of a flat grouped grid belongs to.
__device__ __forceinline__ int group_of(const int64_t* first, int ngroups, int64_t b) {
  int g = 0;
  while (g + 1 < ngroups && b >= first[g + 1]) ++g;
  return g;
}

__global__ __launch_bounds__(kThreads) void momentum_grouped_kernel(const MomentumGroups G) {
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.x;
  const int gi = group_of(G.first, G.ngroups, b);
  const MomentumArgs& a = G.g[gi];
  const int64_t local = b - G.first[gi];
  const int64_t mat = local / a.blocks_per_mat;
  const uint32_t blk = static_cast<uint32_t>(local - mat * a.blocks_per_mat);
  if (G.vec[gi]) {
    momentum_block<true>(a, mat, blk, red);
  } else {
    momentum_block<false>(a, mat, blk, red);
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void sumsq_partials_kernel(const SumsqArgs a) {
  __shared__ float red[kThreads / 64];
  const int64_t mat = blockIdx.y;
  const char* x = mat_ptr(a.X, mat);
  const int xs = a.X.dtype ? 2 : 4;
  const uint32_t total = static_cast<uint32_t>(a.rows) * static_cast<uint32_t>(a.cols);
  float ss = 0.0f;
  const uint32_t base = static_cast<uint32_t>(blockIdx.x) * kElemsPerBlock;
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = base + (u * kThreads + threadIdx.x) * kVec;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        float v[kVec];
        load8(x + (r * a.X.ld + c) * xs, a.X.dtype, v);
#pragma unroll
        for (int k = 0; k < kVec; ++k) ss += v[k] * v[k];
      }
    }
  } else {
    for (int u = 0; u < kUnroll * kVec; ++u) {
      const uint32_t e = base + u * kThreads + threadIdx.x;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        const float v = load1(x + (r * a.X.ld + c) * xs, a.X.dtype);
        ss += v * v;
      }
    }
  }
  const float s = block_sum(ss, red);
  if (threadIdx.x == 0) a.partials[mat * a.blocks_per_mat + blockIdx.x] = s;
}

// One workgroup per matrix: fixed-order fp64 sum of its `per` partials.
__device__ __forceinline__ void finalize_one(const float* p, int per, float* out, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < per; i += kThreads) s += static_cast<double>(p[i]);
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = static_cast<float>(red[0]);
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(const float* partials, int per, float* sumsq) {
  __shared__ double red[kThreads];
  const int64_t mat = blockIdx.x;
  finalize_one(partials + mat * per, per, sumsq + mat, red);
}

__global__ __launch_bounds__(kThreads) void finalize_grouped_kernel(const FinalizeGroups G) {
  __shared__ double red[kThreads];
  const int64_t b = blockIdx.x;  // one matrix of one group
  const int gi = group_of(G.first, G.ngroups, b);
  const int64_t mat = b - G.first[gi];
  finalize_one(G.partials[gi] + mat * G.per[gi], G.per[gi], G.sumsq[gi] + mat, red);
}

// ------------------------------------------------------------ apply

template <bool VEC>
__device__ __forceinline__ void apply_block(const ApplyArgs& a, int64_t mat, uint32_t blk) {
  char* w = mat_ptr(a.W, mat);
  const char* o = mat_ptr(a.O, mat);
  const int ws = a.W.dtype ? 2 : 4;
  const int os = a.O.dtype ? 2 : 4;
  const uint32_t total = static_cast<uint32_t>(a.rows) * static_cast<uint32_t>(a.cols);
  const uint32_t base = blk * kElemsPerBlock;
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = base + (u * kThreads + threadIdx.x) * kVec;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        char* wp = w + (r * a.W.ld + c) * ws;
        float wv[kVec], ov[kVec];
        load8(wp, a.W.dtype, wv);
        load8(o + (r * a.O.ld + c) * os, a.O.dtype, ov);
#pragma unroll
        for (int k = 0; k < kVec; ++k) wv[k] = a.decay * wv[k] - a.step * ov[k];
        store8(wp, a.W.dtype, wv);
      }
    }
  } else {
    for (int u = 0; u < kUnroll * kVec; ++u) {
      const uint32_t e = base + u * kThreads + threadIdx.x;
      if (e < total) {
        const uint32_t r = fdiv(a.cdiv, e);
        const uint32_t c = e - r * a.cols;
        char* wp = w + (r * a.W.ld + c) * ws;
        const float v = a.decay * load1(wp, a.W.dtype) - a.step * load1(o + (r * a.O.ld + c) * os, a.O.dtype);
        store1(wp, a.W.dtype, v);
      }
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void apply_kernel(const ApplyArgs a) {
  apply_block<VEC>(a, blockIdx.y, blockIdx.x);
}

__global__ __launch_bounds__(kThreads) void apply_grouped_kernel(const ApplyGroups G) {
  const int64_t b = blockIdx.x;
  const int gi = group_of(G.first, G.ngroups, b);
  const ApplyArgs& a = G.g[gi];
  const int64_t per = G.blocks_per_mat[gi];
  const int64_t local = b - G.first[gi];
  const int64_t mat = local / per;
  const uint32_t blk = static_cast<uint32_t>(local - mat * per);
  if (G.vec[gi]) {
    apply_block<true>(a, mat, blk);
  } else {
    apply_block<false>(a, mat, blk);
  }
}

// ------------------------------------------------------------ pack

constexpr int kTile = 64;

// The low part of a 64 x 64 tile of X staged in `tile` (stored orientation;
// X is its transpose when tall): thread t encodes lane (t % 64) of the
// update kernel's 32x32 block (t / 64) of this tile, as pack_kernel does.
__device__ __forceinline__ void store_low_part(const float (*tile)[kTile + 1], bool tall, uint32_t r0, uint32_t c0,
                                               int8_t* Lo, uint8_t* LoE, int bm, int tiles_n) {
  const uint32_t i0 = tall ? c0 : r0;
  const uint32_t j0 = tall ? r0 : c0;
  const int b = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hf = lane >> 5, jl = (b & 1) * 32 + (lane & 31);
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int il = (b >> 1) * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
    x[r] = tall ? tile[jl][il] : tile[il][jl];
  }
  const Lo8 c = lo8_encode(x);
  int8_t* run = Lo + lo_index(i0, j0, bm, tiles_n);
  *reinterpret_cast<uint4*>(run + (b * 64 + lane) * 16) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
  LoE[lo_exp_index(i0 + (b >> 1) * 32 + 4 * hf, j0 + (b & 1) * 32 + (lane & 31), bm, tiles_n)] =
      static_cast<uint8_t>(c.e);
}

// grid: (Pc/64, Pr/64, count).  Each workgroup moves one 64x64 tile of the
// padded stored-orientation extent.  Global accesses are 4-element pieces:
// 16 threads cover a 64-element row (N rows read, S rows written) or a
// 64-element column of the tile (T rows written).  With the 65-float LDS
// row stride both the row writes and the 4-row column reads of a wave hit
// 64 distinct banks.
__global__ __launch_bounds__(kThreads) void pack_kernel(const PackArgs a) {
  __shared__ float tile[kTile][kTile + 1];
  const int64_t mat = blockIdx.z;
  const int r0 = blockIdx.y * kTile;
  const int c0 = blockIdx.x * kTile;
  const char* n = mat_ptr(a.N, mat);
  const int nsz = a.N.dtype ? 2 : 4;
  const float ssq = a.sumsq[mat];
  const float scale = 1.0f / (sqrtf(ssq) + a.eps);
  const int q = threadIdx.x & 15;   // 4-element piece of a 64-element row
  const int rq = threadIdx.x >> 4;  // 0..15
  const int esz = a.compute ? 2 : 4;
  // read rows of N (zero outside m x n), write rows of S (if wanted)
  char* S = a.S ? a.S + mat * a.s_mat : nullptr;
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int rr = rq + 16 * k;
    const int r = r0 + rr;
    const int c = c0 + 4 * q;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r < a.rows) {
      const char* np = n + (static_cast<int64_t>(r) * a.N.ld + c) * nsz;
      if (a.nvec && c + 3 < a.cols) {
        load4(np, a.N.dtype, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < a.cols) v[e] = load1(np + e * nsz, a.N.dtype);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] *= scale;
      tile[rr][4 * q + e] = v[e];
    }
    if (S) store4(S + (static_cast<int64_t>(r) * a.Pc + c) * esz, a.compute, v);
  }
  __syncthreads();
  // The low part of X in the update kernel's accumulator order: this 64 x 64
  // tile of X is four consecutive 32x32 blocks of one wave there.
  if (a.Lo) store_low_part(tile, a.tall != 0, r0, c0, a.Lo + mat * a.lo_mat, a.LoE + mat * a.loe_mat, a.lo_bm,
                           a.lo_tiles_n);
  // write rows of T = columns of the tile (if wanted)
  if (!a.T) return;
  char* T = a.T + mat * a.t_mat;
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int cc = rq + 16 * k;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = tile[4 * q + e][cc];
    store4(T + (static_cast<int64_t>(c0 + cc) * a.Pr + r0 + 4 * q) * esz, a.compute, v);
  }
}

// ------------------------------------------------------------ momentum + pack

// Flat grid over the groups' tiles: workgroup b is 64 x 64 tile t of the
// padded stored extent of matrix `mat`.  Reads G and M once, writes M once,
// and writes N (not yet divided by its norm: the first Newton-Schulz step
// applies that scale) straight into the Newton-Schulz buffers, so N never
// makes a round trip through memory.  Global accesses are 4-element pieces,
// 16 threads per 64-element row; the tile transposes through LDS for X^T
// and the low part, as in pack_kernel.
__global__ __launch_bounds__(kThreads) void momentum_pack_kernel(const MomentumPackGroups P) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ float red[kThreads / 64];
  const int64_t b = blockIdx.x;
  const int gi = group_of(P.first, P.ngroups, b);
  const MomentumPackArgs& a = P.g[gi];
  const int64_t local = b - P.first[gi];
  const int64_t mat = local / a.tiles_per_mat;
  const int t = static_cast<int>(local - mat * a.tiles_per_mat);
  const int tr = t / a.tiles_c;
  const int r0 = tr * kTile;
  const int c0 = (t - tr * a.tiles_c) * kTile;
  const char* g = mat_ptr(a.G, mat);
  char* m = mat_ptr(a.M, mat);
  const int gsz = a.G.dtype ? 2 : 4;
  const float beta = a.beta;
  const float omb = 1.0f - a.beta;
  const int q = threadIdx.x & 15;   // 4-element piece of a 64-element row
  const int rq = threadIdx.x >> 4;  // 0..15
  const int esz = a.compute ? 2 : 4;
  char* S = a.S ? a.S + mat * a.s_mat : nullptr;
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int rr = rq + 16 * k;
    const int r = r0 + rr;
    const int c = c0 + 4 * q;
    float nv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r < a.rows) {
      const char* gp = g + (static_cast<int64_t>(r) * a.G.ld + c) * gsz;
      float* mp = reinterpret_cast<float*>(m + (static_cast<int64_t>(r) * a.M.ld + c) * 4);
      if (a.vec && c + 3 < a.cols) {
        float gv[4], mv[4];
        load4(gp, a.G.dtype, gv);
        load4(reinterpret_cast<const char*>(mp), 0, mv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = beta * mv[e] + omb * gv[e];
          nv[e] = a.nesterov ? omb * gv[e] + beta * mv[e] : mv[e];
        }
        store4(reinterpret_cast<char*>(mp), 0, mv);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < a.cols) {
            const float gv = load1(gp + e * gsz, a.G.dtype);
            const float mv = beta * mp[e] + omb * gv;
            nv[e] = a.nesterov ? omb * gv + beta * mv : mv;
            mp[e] = mv;
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss += nv[e] * nv[e];
      tile[rr][4 * q + e] = nv[e];
    }
    if (S) store4(S + (static_cast<int64_t>(r) * a.Pc + c) * esz, a.compute, nv);
  }
  // block_sum's barrier also makes the whole tile visible in LDS
  const float part = block_sum(ss, red);
  if (threadIdx.x == 0) a.partials[mat * a.tiles_per_mat + t] = part;
  if (a.Lo) store_low_part(tile, a.tall != 0, r0, c0, a.Lo + mat * a.lo_mat, a.LoE + mat * a.loe_mat, a.lo_bm,
                           a.lo_tiles_n);
  if (!a.T) return;
  char* T = a.T + mat * a.t_mat;
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int cc = rq + 16 * k;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = tile[4 * q + e][cc];
    store4(T + (static_cast<int64_t>(c0 + cc) * a.Pr + r0 + 4 * q) * esz, a.compute, v);
  }
}

// grid: (ceil(cols/64), ceil(rows/64), count) over the stored output.
__global__ __launch_bounds__(kThreads) void copy_out_kernel(const CopyOutArgs a) {
  const int64_t mat = blockIdx.z;
  const char* n = mat_ptr(a.N, mat);
  char* o = mat_ptr(a.out, mat);
  const int nsz = a.N.dtype ? 2 : 4;
  const int osz = a.out.dtype ? 2 : 4;
  const float scale = 1.0f / (sqrtf(a.sumsq[mat]) + a.eps);
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;
  for (int rr = ty; rr < kTile; rr += 4) {
    const int r = blockIdx.y * kTile + rr;
    const int c = blockIdx.x * kTile + tx;
    if (r < a.rows && c < a.cols) {
      const float v = scale * load1(n + (static_cast<int64_t>(r) * a.N.ld + c) * nsz, a.N.dtype);
      store1(o + (static_cast<int64_t>(r) * a.out.ld + c) * osz, a.out.dtype, v);
    }
  }
}

// ------------------------------------------------------------ split Gram

// One workgroup per 64x64 block of a computed tile (tile row <= tile
// column) of one matrix: adds the S slices' partial sums in a fixed order,
// scales (step 0 of the packed path), stores the block, and for a tile off
// the diagonal also its mirror, transposed through LDS.  Thread t sums 16
// consecutive elements of row t/4 of the block (float4 reads of each slice).
__global__ __launch_bounds__(256) void gram_reduce_kernel(const GramReduce R) {
  __shared__ float tr[64][65];
  const int64_t b = blockIdx.x;
  int gi = 0;
  while (gi + 1 < R.ngroups && b >= R.first[gi + 1]) ++gi;
  const GramReduceGroup& g = R.g[gi];
  const int T = g.Mp / g.tile;
  const int nb = g.tile / 64;                                            // 64-blocks per tile side
  const int64_t per = static_cast<int64_t>(T) * (T + 1) / 2 * nb * nb;  // workgroups per matrix
  const int64_t local = b - R.first[gi];
  const int64_t mat = local / per;
  const int r = static_cast<int>(local - mat * per);
  const int sub = r % (nb * nb);
  int tt = r / (nb * nb);
  int ti = 0;
  while (tt >= T - ti) {
    tt -= T - ti;
    ++ti;
  }
  const int tj = ti + tt;
  const int r0 = ti * g.tile + (sub / nb) * 64;
  const int c0 = tj * g.tile + (sub % nb) * 64;
  const int row = threadIdx.x >> 2;
  const int cq = (threadIdx.x & 3) * 16;
  const float* part = reinterpret_cast<const float*>(reinterpret_cast<const char*>(g.part) + mat * g.part_mat) +
                      static_cast<int64_t>(r0 + row) * g.Mp + c0 + cq;
  const int64_t slice = static_cast<int64_t>(g.Mp) * g.Mp;
  float scale = 1.0f;
  if (g.xs_sumsq != nullptr) {
    const float xs = 1.0f / (sqrtf(g.xs_sumsq[mat]) + g.xs_eps);
    scale = xs * xs;
  }
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = 0.0f;
  for (int s = 0; s < g.splits; ++s) {  // fixed order
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(part + s * slice + 4 * q);
      v[4 * q] += x.x;
      v[4 * q + 1] += x.y;
      v[4 * q + 2] += x.z;
      v[4 * q + 3] += x.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] *= scale;
  char* A = g.A + mat * g.a_mat;
  const int es = g.compute ? 2 : 4;  // compute 1 = bf16, as the dtype of store8
  auto put16 = [&](int i, int j, const float* w) {  // 16 consecutive elements of row i from column j
    char* p = A + (static_cast<int64_t>(i) * g.Mp + j) * es;
    store8(p, g.compute, w);
    store8(p + 8 * es, g.compute, w + 8);
  };
  put16(r0 + row, c0 + cq, v);
  if (ti == tj) return;  // a diagonal tile's partial sums hold both of its halves
#pragma unroll
  for (int e = 0; e < 16; ++e) tr[row][cq + e] = v[e];
  __syncthreads();
  float w[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) w[e] = tr[cq + e][row];  // mirror row c0 + row, columns r0 + cq ..
  put16(c0 + row, r0 + cq, w);
}

}  // namespace

int elementwise_blocks_per_matrix(int64_t rows, int64_t cols) {
  return static_cast<int>((rows * cols + kElemsPerBlock - 1) / kElemsPerBlock);
}

hipError_t launch_momentum(const MomentumArgs& a, int64_t count, bool vec, hipStream_t stream) {
  dim3 grid(a.blocks_per_mat, static_cast<unsigned>(count));
  if (vec) {
    hipLaunchKernelGGL(momentum_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(momentum_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_sumsq_partials(const SumsqArgs& a, int64_t count, bool vec, hipStream_t stream) {
  dim3 grid(a.blocks_per_mat, static_cast<unsigned>(count));
  if (vec) {
    hipLaunchKernelGGL(sumsq_partials_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sumsq_partials_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_sumsq_finalize(const float* partials, int per, float* sumsq, int64_t count,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(finalize_kernel, dim3(static_cast<unsigned>(count)), dim3(kThreads), 0, stream,
                     partials, per, sumsq);
  return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& a, int64_t count, bool vec, hipStream_t stream) {
  const int per = elementwise_blocks_per_matrix(a.rows, a.cols);
  dim3 grid(per, static_cast<unsigned>(count));
  if (vec) {
    hipLaunchKernelGGL(apply_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(apply_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_momentum_grouped(const MomentumGroups& a, hipStream_t stream) {
  hipLaunchKernelGGL(momentum_grouped_kernel, dim3(static_cast<unsigned>(a.first[a.ngroups])), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_sumsq_finalize_grouped(const FinalizeGroups& a, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_grouped_kernel, dim3(static_cast<unsigned>(a.first[a.ngroups])), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_apply_grouped(const ApplyGroups& a, hipStream_t stream) {
  hipLaunchKernelGGL(apply_grouped_kernel, dim3(static_cast<unsigned>(a.first[a.ngroups])), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, int64_t count, hipStream_t stream) {
  dim3 grid(a.Pc / kTile, a.Pr / kTile, static_cast<unsigned>(count));
  hipLaunchKernelGGL(pack_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_momentum_pack_grouped(const MomentumPackGroups& a, hipStream_t stream) {
  hipLaunchKernelGGL(momentum_pack_kernel, dim3(static_cast<unsigned>(a.first[a.ngroups])), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_out(const CopyOutArgs& a, int64_t count, hipStream_t stream) {
  dim3 grid((a.cols + kTile - 1) / kTile, (a.rows + kTile - 1) / kTile, static_cast<unsigned>(count));
  hipLaunchKernelGGL(copy_out_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gram_reduce(const GramReduce& a, hipStream_t stream) {
  if (a.first[a.ngroups] <= 0) return hipSuccess;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(static_cast<unsigned>(a.first[a.ngroups])), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muon
