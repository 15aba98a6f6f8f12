// SOAP kernels of libmuon355: Adam run in the eigenbasis of Shampoo's row
// and column statistics ("LLM Optimizers: From SGD and AdamW to SOAP, Muon,
// and Scalable Training", sections 11.1-11.2; "初探优化器（一）：从SGD到
// SOAP-Muon", section 6.2).
//
//   sgemm_kernel      C = alpha*op(A)*op(B) + beta*C in fp32 on the fp32 MFMA
//                     (v_mfma_f32_32x32x2_f32): the statistics G G^T and
//                     G^T G, the rotations Q_L^T G Q_R and Q_L D Q_R^T, the
//                     power-iteration product S Q and the QR's block updates.
//   qr_panel_*        one 16-column panel of a Householder QR (the basis
//                     refresh): reflectors, their block factor T, and the
//                     signs that make R's diagonal non-negative; held in
//                     registers up to 4096 rows, else worked in memory.
//   rot_adam_kernel   Adam's moments and direction in the rotated basis.
//
// Everything here computes in fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>

#include "muon_internal.h"

namespace muon {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kT = kSgemmTile;      // 128 x 128 output tile
constexpr int kBK = kSgemmBK;       // 32-deep k-slices
constexpr int kPitch = kT + 4;      // LDS row pitch in floats
constexpr int kThreads = 256;       // 4 waves, 2 x 2, each 64 x 64

__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float load1(const char* p, int32_t dtype, int64_t idx) {
  return dtype ? bf16f(reinterpret_cast<const uint16_t*>(p)[idx]) : reinterpret_cast<const float*>(p)[idx];
}

// Four consecutive elements of memory row `row` (of `rows`), columns
// col .. col+3 (of `cols`), zero outside.
__device__ __forceinline__ void load_run(const char* p, const SgemmOperand& o, int row, int col, int rows,
                                         int cols, float* v) {
  if (row >= rows) {
    v[0] = v[1] = v[2] = v[3] = 0.f;
    return;
  }
  const int64_t idx = static_cast<int64_t>(row) * o.ld + col;
  if (o.vec && col + 3 < cols) {
    if (o.dtype) {
      const uint2 u = *reinterpret_cast<const uint2*>(p + idx * 2);
      v[0] = bf16f(u.x & 0xffffu);
      v[1] = bf16f(u.x >> 16);
      v[2] = bf16f(u.y & 0xffffu);
      v[3] = bf16f(u.y >> 16);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(p + idx * 4);
      v[0] = f.x;
      v[1] = f.y;
      v[2] = f.z;
      v[3] = f.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (col + e < cols) ? load1(p, o.dtype, idx + e) : 0.f;
  }
}

// One OUT (outer) x kBK (reduction) slice of an operand into registers,
// OUT*kBK/1024 runs of four per thread (threads beyond the runs idle): outer
// rows o0.. (of `outer`), reduction k0.. (below klim).
template <int OUT>
__device__ __forceinline__ void load_slice(const char* p, const SgemmOperand& o, int outer, int klim, int o0,
                                           int k0, float* r) {
  constexpr int kRuns = OUT * kBK / 4;
  constexpr int kG = (kRuns + kThreads - 1) / kThreads;
  constexpr int kRPR = kBK / 4;  // runs per row of a k-contiguous operand
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int t = threadIdx.x + kThreads * g;
    if (kRuns % kThreads != 0 && t >= kRuns) continue;
    if (o.kcontig)
      load_run(p, o, o0 + t / kRPR, k0 + 4 * (t % kRPR), outer, klim, r + 4 * g);
    else
      load_run(p, o, k0 + t / (OUT / 4), o0 + 4 * (t % (OUT / 4)), klim, outer, r + 4 * g);
  }
}

// The slice into LDS as S[k][outer] (pitch OUT + 4).  For OUT = 128 the
// scattered form (kcontig, eight runs per row) touches each bank at most
// twice per wave: address mod 64 is 16*(t%8) + 4e + t/8 for lanes t.
template <int OUT>
__device__ __forceinline__ void store_slice(float* S, const SgemmOperand& o, const float* r) {
  constexpr int kRuns = OUT * kBK / 4;
  constexpr int kG = (kRuns + kThreads - 1) / kThreads;
  constexpr int kRPR = kBK / 4;  // runs per row of a k-contiguous operand
  constexpr int kP = OUT + 4;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int t = threadIdx.x + kThreads * g;
    if (kRuns % kThreads != 0 && t >= kRuns) continue;
    if (o.kcontig) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[(4 * (t % kRPR) + e) * kP + t / kRPR] = r[4 * g + e];
    } else {
      *reinterpret_cast<float4*>(S + (t / (OUT / 4)) * kP + 4 * (t % (OUT / 4))) =
          make_float4(r[4 * g], r[4 * g + 1], r[4 * g + 2], r[4 * g + 3]);
    }
  }
}

// Fast path, for operands whose every 4-element run along the contiguous
// index is aligned and inside the row (leading dimension and both extents
// multiples of 4): element type and orientation are template arguments and
// each run is one vector load from clamped indices, zeroed by a select when
// out of range.  No branch separates a load from its use, so the loads of
// the next slice stay in flight during the products.
template <bool BF16>
__device__ __forceinline__ void load4_fast(const char* p, int64_t idx, float* v) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(p + idx * 2);
    v[0] = bf16f(u.x & 0xffffu);
    v[1] = bf16f(u.x >> 16);
    v[2] = bf16f(u.y & 0xffffu);
    v[3] = bf16f(u.y >> 16);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p + idx * 4);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

template <int OUT, bool BF16, bool KC>
__device__ __forceinline__ void load_slice_fast(const char* p, int64_t ld, int outer, int klim, int o0, int k0,
                                                float* r) {
  constexpr int kRuns = OUT * kBK / 4;
  constexpr int kG = (kRuns + kThreads - 1) / kThreads;
  constexpr int kRPR = kBK / 4;  // runs per row of a k-contiguous operand
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int t = threadIdx.x + kThreads * g;
    if (kRuns % kThreads != 0 && t >= kRuns) continue;
    const int row = KC ? o0 + t / kRPR : k0 + t / (OUT / 4);
    const int col = KC ? k0 + 4 * (t % kRPR) : o0 + 4 * (t % (OUT / 4));
    const int rows = KC ? outer : klim, cols = KC ? klim : outer;
    const bool in = row < rows && col < cols;
    float v[4];
    load4_fast<BF16>(p, static_cast<int64_t>(min(row, rows - 1)) * ld + min(col, cols - 4), v);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * g + e] = in ? v[e] : 0.f;
  }
}

template <int OUT, bool KC>
__device__ __forceinline__ void store_slice_fast(float* S, const float* r) {
  constexpr int kRuns = OUT * kBK / 4;
  constexpr int kG = (kRuns + kThreads - 1) / kThreads;
  constexpr int kRPR = kBK / 4;  // runs per row of a k-contiguous operand
  constexpr int kP = OUT + 4;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int t = threadIdx.x + kThreads * g;
    if (kRuns % kThreads != 0 && t >= kRuns) continue;
    if constexpr (KC) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[(4 * (t % kRPR) + e) * kP + t / kRPR] = r[4 * g + e];
    } else {
      *reinterpret_cast<float4*>(S + (t / (OUT / 4)) * kP + 4 * (t % (OUT / 4))) =
          make_float4(r[4 * g], r[4 * g + 1], r[4 * g + 2], r[4 * g + 3]);
    }
  }
}

// Operand configuration of the fast path: bit 0 A bf16, bit 1 A kcontig,
// bit 2 B bf16, bit 3 B kcontig; -1 = the generic path.
template <int CFG>
struct FastCfg {
  static constexpr bool kOn = CFG >= 0;
  static constexpr bool kAB = CFG >= 0 && (CFG & 1), kAK = CFG >= 0 && (CFG & 2);
  static constexpr bool kBB = CFG >= 0 && (CFG & 4), kBK = CFG >= 0 && (CFG & 8);
};

__device__ __forceinline__ const char* entry(const SgemmOperand& o, int b) {
  const char* p = o.ptrs ? static_cast<const char*>(o.ptrs[b]) : o.base + static_cast<int64_t>(b) * o.stride;
  return p + o.off;
}

// TM x 128 output tile, four waves: TM = 128 as 2 x 2 waves of 64 x 64,
// TM = 32 (products with at most 32 rows) as 1 x 4 waves of 32 x 32.  At
// least three workgroups per CU (accumulators in VGPRs, no AGPRs): a third
// wave per SIMD covers the LDS reads before each step's products.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Tile (ti, tj) of batch entry and split z = bi * splits + sp.
template <int TM, int CFG>
__device__ __forceinline__ void sgemm_tile(const SgemmArgs& a, int ti, int tj, int z) {
  using F = FastCfg<CFG>;
  constexpr int WM = TM >= 64 ? 2 : 1, WN = 4 / WM;
  constexpr int FI = TM / WM / 32, FJ = kT / WN / 32;
  constexpr int kPA = TM + 4;
  const int bi = z / a.splits, sp = z % a.splits;
  const int kbeg = sp * a.ksplit;
  const int kend = min(a.K, kbeg + a.ksplit);
  const char* pa = entry(a.a, bi);
  const char* pb = entry(a.b, bi);
  char* pc = (a.c_ptrs ? static_cast<char*>(a.c_ptrs[bi]) : a.c + static_cast<int64_t>(bi) * a.c_stride) + a.c_off +
             static_cast<int64_t>(sp) * a.c_split;

  __shared__ float As[kBK * kPA];
  __shared__ float Bs[kBK * kPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;
  const int i0 = ti * TM, j0 = tj * kT;

  f32x16_t acc[FI][FJ];
#pragma unroll
  for (int x = 0; x < FI; ++x)
#pragma unroll
    for (int y = 0; y < FJ; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  float ra[(TM * kBK / 4 + kThreads - 1) / kThreads * 4], rb[(kT * kBK / 4 + kThreads - 1) / kThreads * 4];
  // The fast path's address arguments, taken into scalar registers once: read
  // from the argument block at a runtime offset (the product-list kernel),
  // the compiler would otherwise reload them every slice, and the wait for
  // those loads also waits for the slice's LDS stores.
  const int64_t lda = uniform64(a.a.ld), ldb = uniform64(a.b.ld);
  const int Mu = __builtin_amdgcn_readfirstlane(a.M), Nu = __builtin_amdgcn_readfirstlane(a.N);
  auto load = [&](int k0) {
    if constexpr (F::kOn) {
      load_slice_fast<TM, F::kAB, F::kAK>(pa, lda, Mu, kend, i0, k0, ra);
      load_slice_fast<kT, F::kBB, F::kBK>(pb, ldb, Nu, kend, j0, k0, rb);
    } else {
      load_slice<TM>(pa, a.a, a.M, kend, i0, k0, ra);
      load_slice<kT>(pb, a.b, a.N, kend, j0, k0, rb);
    }
  };
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kBK) {
    if constexpr (F::kOn) {
      store_slice_fast<TM, F::kAK>(As, ra);
      store_slice_fast<kT, F::kBK>(Bs, rb);
    } else {
      store_slice<TM>(As, a.a, ra);
      store_slice<kT>(Bs, a.b, rb);
    }
    __syncthreads();
    if (k0 + kBK < kend) load(k0 + kBK);  // next slice in flight during the products
#pragma unroll
    for (int kk = 0; kk < kBK / 2; ++kk) {
      // lane: A[i = l32][k = half] and B[k = half][j = l32] of each 32 x 2 step
      float av[FI], bv[FJ];
#pragma unroll
      for (int x = 0; x < FI; ++x) av[x] = As[(2 * kk + half) * kPA + wm * (TM / WM) + x * 32 + l32];
#pragma unroll
      for (int y = 0; y < FJ; ++y) bv[y] = Bs[(2 * kk + half) * kPitch + wn * (kT / WN) + y * 32 + l32];
#pragma unroll
      for (int x = 0; x < FI; ++x)
#pragma unroll
        for (int y = 0; y < FJ; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }

  // accumulator r of lane: row 8*(r/4) + 4*half + r%4, column l32 of its block
  float* C = reinterpret_cast<float*>(pc);
  const bool diag = a.sym && ti == tj;
#pragma unroll
  for (int fi = 0; fi < FI; ++fi)
#pragma unroll
    for (int fj = 0; fj < FJ; ++fj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + wm * (TM / WM) + fi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int j = j0 + wn * (kT / WN) + fj * 32 + l32;
        if (i >= a.M || j >= a.N || (diag && i > j)) continue;
        float* cij = C + static_cast<int64_t>(i) * a.ldc + j;
        float v = a.alpha * acc[fi][fj][r];
        if (a.beta != 0.f) v += a.beta * *cij;
        *cij = v;
        if (a.sym && i != j) C[static_cast<int64_t>(j) * a.ldc + i] = v;
      }
}

// Tile t of one matrix's grid: row-major over T x tn tiles, or for a
// symmetric product over the upper triangle only, row by row.  (A full grid
// whose lower half returns at once ran the remaining tiles at half their
// rate.)
__device__ __forceinline__ void tile_coords(const SgemmArgs& a, int t, int tn, int* ti, int* tj) {
  if (a.sym) {
    const int T = (a.N + kT - 1) / kT;
    int r = 0;
    while (t >= T - r) {
      t -= T - r;
      ++r;
    }
    *ti = r;
    *tj = r + t;
  } else {
    *ti = t / tn;
    *tj = t % tn;
  }
}

// One product: blockIdx.x = tile of the matrix grid, blockIdx.z = batch
// entry and split.
template <int TM, int CFG>
__global__ __launch_bounds__(kThreads, 3) void sgemm_kernel(SgemmArgs a) {
  int ti = blockIdx.y, tj = blockIdx.x;
  if (a.sym) tile_coords(a, blockIdx.x, 0, &ti, &tj);
  sgemm_tile<TM, CFG>(a, ti, tj, blockIdx.z);
}

// Several products in one launch (128-row tiles): product p owns the linear
// workgroups [tile_end[p-1], tile_end[p]), batch entry and split major, tile
// minor.
template <int CFG>
__global__ __launch_bounds__(kThreads, 3) void sgemm_list_kernel(SgemmList l) {
  int p = 0;
  while (p + 1 < l.n && static_cast<int>(blockIdx.x) >= l.tile_end[p]) ++p;
  const SgemmArgs& a = l.g[p];
  const int q = blockIdx.x - (p ? l.tile_end[p - 1] : 0);
  const int tn = (a.N + kT - 1) / kT;
  const int per = a.sym ? tn * (tn + 1) / 2 : tn * ((a.M + kT - 1) / kT);
  int ti, tj;
  tile_coords(a, q % per, tn, &ti, &tj);
  sgemm_tile<kT, CFG>(a, ti, tj, q / per);
}

// --------------------------------------------------------------- QR panel

constexpr int kQrThreads = 512;
constexpr int kQrWaves = kQrThreads / 64;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Workgroup sums of 32 per-thread values, left in tot[0..31].  Inside each
// wave a reduce-scatter halves the values at every exchange (xor 32, 16, 8,
// 4, 2), so lane l ends with value l >> 1, completed by the xor-1 exchange.
__device__ __forceinline__ void block_sum32(float* w, float* part, float* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int h = 16; h >= 1; h >>= 1) {
    const bool up = (lane & (2 * h)) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? w[i] : w[i + h];
      const float keep = up ? w[i + h] : w[i];
      w[i] = keep + __shfl_xor(send, 2 * h);
    }
  }
  w[0] += __shfl_xor(w[0], 1);
  if ((lane & 1) == 0) part[wave * 32 + (lane >> 1)] = w[0];
  __syncthreads();
  if (threadIdx.x < 32) {
    float s = 0.f;
    for (int q = 0; q < kQrWaves; ++q) s += part[q * 32 + threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
}

// Columns c0 .. c0+nb-1 of A (rows c0 .. n-1), one column at a time
// (LAPACK's dlarfg / dlarft conventions):
//   x = A[c:, c], alpha = x_0, s = |x_1:|^2; s = 0: no reflection (tau 0,
//   beta = alpha); else beta = -sign(alpha) |x|, tau = (beta - alpha)/beta,
//   v = x / (alpha - beta) with v_0 = 1, so (I - tau v v^T) x = beta e_0;
//   every later panel column y <- y - tau v (v^T y);
//   T[0:j, j] = -tau_j T[0:j, 0:j] (V[:, 0:j]^T v_j), T[j][j] = tau_j.
// The panel is first copied, column-major, into its slot of the reflector
// buffer, P[q][r] = A[c0 + r][c0 + q] at V + q*n + r, and reduced there:
// lanes take consecutive rows, so every column access of a wave is one
// contiguous run.  Column j of the slot ends as the explicit reflector
// (zeros above its unit diagonal).  Row r of a column step belongs to
// thread (r - j) mod kQrThreads in every phase that writes it; the barrier
// ending each column orders the next column's reads.  A is only read: R is
// not needed, only the signs of its diagonal.
__global__ __launch_bounds__(kQrThreads) void qr_panel_kernel(QrPanelArgs a) {
  const int64_t b = blockIdx.x;
  const float* A = a.A + b * a.a_mat;
  float* P = a.V + b * a.v_mat;
  float* TrT = a.TrepT + b * a.tT_mat;
  float* TrQ = a.TrepQ + b * a.tQ_mat;
  float* sg = a.sgn + b * a.s_mat;
  float* tg = a.tau + b * a.s_mat;
  const int n = a.n, c0 = a.c0, h = n - c0;
  const int nb = min(kQrPanel, h);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float tile[kQrWaves][32][33];
  __shared__ float part[kQrWaves * 32];
  __shared__ float tot[32];
  __shared__ float Ts[kQrPanel][kQrPanel + 1];
  __shared__ float par[3];

  // copy in: each wave moves 32 rows at a time through its own LDS tile
  // (row reads of 128 bytes, column writes of 128 bytes)
  for (int r0 = 32 * wave; r0 < h; r0 += 32 * kQrWaves) {
    for (int i = 0; i < 16; ++i) {
      const int rr = 2 * i + (lane >> 5), q = lane & 31, r = r0 + rr;
      tile[wave][rr][q] = (r < h && q < nb) ? A[static_cast<int64_t>(c0 + r) * n + c0 + q] : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    for (int q2 = 0; q2 < 32; q2 += 2) {
      const int q = q2 + (lane >> 5), rr = lane & 31, r = r0 + rr;
      if (r < h && q < nb) P[static_cast<int64_t>(q) * n + r] = tile[wave][rr][q];
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  for (int j = 0; j < nb; ++j) {
    float* pj = P + static_cast<int64_t>(j) * n;
    float s = 0.f;
    for (int r = j + 1 + tid; r < h; r += kQrThreads) {
      const float x = pj[r];
      s += x * x;
    }
    s = wave_sum(s);
    if (lane == 0) part[wave] = s;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int q = 0; q < kQrWaves; ++q) t += part[q];
      const float alpha = pj[j];
      float beta = alpha, tau = 0.f, scale = 0.f;
      if (t > 0.f) {
        const float nrm = sqrtf(alpha * alpha + t);
        beta = alpha >= 0.f ? -nrm : nrm;
        tau = (beta - alpha) / beta;
        scale = 1.f / (alpha - beta);
      }
      par[1] = tau;
      par[2] = scale;
      sg[c0 + j] = beta < 0.f ? -1.f : 1.f;
      tg[c0 + j] = tau;
      Ts[j][j] = tau;
    }
    __syncthreads();
    const float tau = par[1], scale = par[2];

    // v below the diagonal, in place; dot products of v with the panel's
    // columns: the earlier reflectors (q < j) and the columns still to be
    // reduced (q > j)
    float w[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) w[q] = 0.f;
    for (int r = j + tid; r < h; r += kQrThreads) {
      float vr = 1.f;
      if (r > j) {
        vr = pj[r] * scale;
        pj[r] = vr;
      }
#pragma unroll
      for (int q = 0; q < 32; ++q)
        if (q < nb && q != j) w[q] += vr * P[static_cast<int64_t>(q) * n + r];
    }
    block_sum32(w, part, tot);

    if (tid < j) {
      float t = 0.f;
      for (int k = tid; k < j; ++k) t += Ts[tid][k] * tot[k];
      Ts[tid][j] = -tau * t;
    }
    if (j + 1 < nb) {
      for (int r = j + tid; r < h; r += kQrThreads) {
        const float vr = r > j ? pj[r] : 1.f;
        for (int q = j + 1; q < nb; ++q) P[static_cast<int64_t>(q) * n + r] -= tau * tot[q] * vr;
      }
    }
    // explicit reflector: unit diagonal, zeros above it (R is not kept)
    for (int r = tid; r <= j; r += kQrThreads) pj[r] = r == j ? 1.f : 0.f;
    __syncthreads();
  }

  // rows of the outer block above the panel: zero in these columns
  for (int r = tid; r < a.zpre; r += blockDim.x)
    for (int q = 0; q < nb; ++q) P[static_cast<int64_t>(q) * n - a.zpre + r] = 0.f;
  // T below its diagonal is zero; repeated copies for the split products
  for (int e = tid; e < nb * nb; e += kQrThreads) {
    const int i = e / nb, k = e % nb;
    const float t = k >= i ? Ts[i][k] : 0.f;     // T[i][k]
    const float tt = i >= k ? Ts[k][i] : 0.f;    // T^T[i][k]
    for (int s2 = 0; s2 < a.reps_t; ++s2) TrT[static_cast<int64_t>(i) * nb * a.reps_t + s2 * nb + k] = tt;
    for (int s2 = 0; s2 < a.reps_q; ++s2) TrQ[static_cast<int64_t>(i) * nb * a.reps_q + s2 * nb + k] = t;
  }
}

// The same panel step with the panel held in registers: 512 threads, row
// r = tid + 512 k (k < 8) in x[k][0..15], so a panel of up to 4096 rows
// costs no memory traffic between its load and the store of the
// reflectors; a column step is two workgroup reductions.
constexpr int kRegThreads = 512;
constexpr int kRegRows = 8;
constexpr int kRegWaves = kRegThreads / 64;

// Workgroup sums of 16 per-thread values into tot[0..15]: reduce-scatter
// inside each wave (xor 32, 16, 8, 4 leave value lane >> 2 in each group of
// four lanes, completed by xor 2 and 1).
__device__ __forceinline__ void block_sum16(float* w, float* part, float* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int h = 8; h >= 1; h >>= 1) {
    const bool up = (lane & (4 * h)) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? w[i] : w[i + h];
      const float keep = up ? w[i + h] : w[i];
      w[i] = keep + __shfl_xor(send, 4 * h);
    }
  }
  w[0] += __shfl_xor(w[0], 2);
  w[0] += __shfl_xor(w[0], 1);
  if ((lane & 3) == 0) part[wave * 16 + (lane >> 2)] = w[0];
  __syncthreads();
  if (threadIdx.x < 16) {
    float s = 0.f;
    for (int q = 0; q < kRegWaves; ++q) s += part[q * 16 + threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kRegThreads) void qr_panel_reg_kernel(QrPanelArgs a) {
  const int64_t b = blockIdx.x;
  const float* A = a.A + b * a.a_mat;
  float* P = a.V + b * a.v_mat;
  float* TrT = a.TrepT + b * a.tT_mat;
  float* TrQ = a.TrepQ + b * a.tQ_mat;
  float* sg = a.sgn + b * a.s_mat;
  float* tg = a.tau + b * a.s_mat;
  const int n = a.n, c0 = a.c0, h = n - c0;
  const int nb = min(kQrPanel, h);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float part[kRegWaves * 16];
  __shared__ float partn[kRegWaves];  // norm partials: apart from part, which the dot products reuse
  __shared__ float tot[16];
  __shared__ float Ts[kQrPanel][kQrPanel + 1];
  __shared__ float sgs[kQrPanel];
  __shared__ float par[1];

  // one panel row per 16-float vector; 16-byte loads where every row of
  // the panel starts 16-byte aligned
  f32x16_t x[kRegRows];
  const bool vec = nb == kQrPanel && n % 4 == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
#pragma unroll
  for (int k = 0; k < kRegRows; ++k) {
    const int r = tid + kRegThreads * k;
    const float* row = A + static_cast<int64_t>(c0 + (r < h ? r : 0)) * n + c0;
    if (vec) {
#pragma unroll
      for (int q = 0; q < kQrPanel; q += 4) {
        const float4 v = r < h ? *reinterpret_cast<const float4*>(row + q) : make_float4(0.f, 0.f, 0.f, 0.f);
        x[k][q] = v.x;
        x[k][q + 1] = v.y;
        x[k][q + 2] = v.z;
        x[k][q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kQrPanel; ++q) x[k][q] = (r < h && q < nb) ? row[q < nb ? q : 0] : 0.f;
    }
  }

  // Each row's 16 values are one vector; column j (uniform over the
  // workgroup) is read and written by a register-relative move.  Three
  // barriers per column: every thread forms the reflector's factors from the
  // wave partials itself, and the next column's writes go to LDS words that
  // this column has finished reading before its last barrier.
  for (int j = 0; j < nb; ++j) {
    float s = 0.f;
    float vk[kRegRows];
#pragma unroll
    for (int k = 0; k < kRegRows; ++k) {
      const int r = tid + kRegThreads * k;
      const float c = x[k][j];
      vk[k] = c;
      s += (r > j && r < h) ? c * c : 0.f;
      if (k == 0 && tid == j) par[0] = c;  // alpha: row j is thread j's first row (j < 16)
    }
    s = wave_sum(s);
    if (lane == 0) partn[wave] = s;
    __syncthreads();
    float t2 = 0.f;
#pragma unroll
    for (int q = 0; q < kRegWaves; ++q) t2 += partn[q];
    const float alpha = par[0];
    float beta = alpha, tau = 0.f, scale = 0.f;
    if (t2 > 0.f) {
      const float nrm = sqrtf(alpha * alpha + t2);
      beta = alpha >= 0.f ? -nrm : nrm;
      tau = (beta - alpha) / beta;
      scale = 1.f / (alpha - beta);
    }
    if (tid == 0) {  // to global memory after the loop: a barrier waits for pending stores
      sgs[j] = beta < 0.f ? -1.f : 1.f;
      Ts[j][j] = tau;
    }

    // v (1 on the diagonal, x * scale below, 0 above) replaces column j
    // below the diagonal; w = v^T x for every column (w[j] is not used)
    float w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = 0.f;
#pragma unroll
    for (int k = 0; k < kRegRows; ++k) {
      const int r = tid + kRegThreads * k;
      const bool below = r > j && r < h;
      vk[k] = below ? vk[k] * scale : (r == j ? 1.f : 0.f);
      if (below) x[k][j] = vk[k];
#pragma unroll
      for (int q = 0; q < kQrPanel; ++q) w[q] += vk[k] * x[k][q];
    }
    block_sum16(w, part, tot);

    if (tid < j) {
      float t = 0.f;
      for (int k = tid; k < j; ++k) t += Ts[tid][k] * tot[k];
      Ts[tid][j] = -tau * t;
    }
    // columns right of j: x_q -= tau (v^T x_q) v
    float cq[kQrPanel];
#pragma unroll
    for (int q = 0; q < kQrPanel; ++q) cq[q] = q > j ? tau * tot[q] : 0.f;
#pragma unroll
    for (int k = 0; k < kRegRows; ++k)
#pragma unroll
      for (int q = 0; q < kQrPanel; ++q) x[k][q] = q > j ? x[k][q] - cq[q] * vk[k] : x[k][q];
  }
  __syncthreads();
  if (tid < nb) {
    sg[c0 + tid] = sgs[tid];
    tg[c0 + tid] = Ts[tid][tid];
  }

  // explicit reflectors, column-major in the slot (coalesced across lanes)
#pragma unroll
  for (int k = 0; k < kRegRows; ++k) {
    const int r = tid + kRegThreads * k;
    if (r < h) {
#pragma unroll
      for (int q = 0; q < kQrPanel; ++q)
        if (q < nb) P[static_cast<int64_t>(q) * n + r] = r > q ? x[k][q] : (r == q ? 1.f : 0.f);
    }
  }
  // rows of the outer block above the panel: zero in these columns
  for (int r = tid; r < a.zpre; r += blockDim.x)
    for (int q = 0; q < nb; ++q) P[static_cast<int64_t>(q) * n - a.zpre + r] = 0.f;
  for (int e = tid; e < nb * nb; e += kRegThreads) {
    const int i = e / nb, k = e % nb;
    const float t = k >= i ? Ts[i][k] : 0.f;
    const float tt = i >= k ? Ts[k][i] : 0.f;
    for (int s2 = 0; s2 < a.reps_t; ++s2) TrT[static_cast<int64_t>(i) * nb * a.reps_t + s2 * nb + k] = tt;
    for (int s2 = 0; s2 < a.reps_q; ++s2) TrQ[static_cast<int64_t>(i) * nb * a.reps_q + s2 * nb + k] = t;
  }
}

// Block factor of an outer block from the Gram matrix of its reflectors
// (LAPACK's dlarft recurrence T[0:j, j] = -tau_j T[0:j, 0:j] Y[0:j, j],
// taken 16 columns at a time).  First every 16 x 16 diagonal block by the
// scalar recurrence, all blocks at once; then block column J from the
// finished columns to its left: T[0:16J, J] = -(T[0:16J, 0:16J] Y[0:16J, J]) T_JJ,
// two small products spread over the workgroup.  Y, T and the intermediate
// product live in LDS; one workgroup per matrix.
constexpr int kTfThreads = 256;
constexpr int kTfB = 16;
__global__ __launch_bounds__(kTfThreads) void qr_tfactor_kernel(QrTArgs a) {
  const int64_t b = blockIdx.x;
  const float* Y = a.Y + b * a.y_mat;
  const float* tau = a.tau + b * a.s_mat;
  float* TrT = a.TrepT + b * a.tT_mat;
  float* TrQ = a.TrepQ + b * a.tQ_mat;
  const int bw = a.bw, tid = threadIdx.x;
  const int nblk = (bw + kTfB - 1) / kTfB;
  __shared__ float Ys[kQrOuter][kQrOuter + 1];
  __shared__ float T[kQrOuter][kQrOuter + 1];
  __shared__ float X[kQrOuter - kTfB][kTfB + 1];
  for (int e = tid; e < bw * bw; e += kTfThreads) {
    Ys[e / bw][e % bw] = Y[e];
    T[e / bw][e % bw] = 0.f;
  }
  __syncthreads();
  // diagonal blocks: thread (J, i) owns row 16J + i of block J
  {
    const int J = tid / kTfB, i = tid % kTfB, r = kTfB * J + i;
    const bool own = J < nblk && r < bw;
    const int jb = J < nblk ? min(kTfB, bw - kTfB * J) : 0;
    for (int j = 0; j < kTfB; ++j) {
      if (own && j < jb) {
        const int c = kTfB * J + j;
        if (i < j) {
          float t = 0.f;
          for (int k = i; k < j; ++k) t += T[r][kTfB * J + k] * Ys[kTfB * J + k][c];
          T[r][c] = -tau[c] * t;
        } else if (i == j) {
          T[r][c] = tau[c];
        }
      }
      __syncthreads();
    }
  }
  // off-diagonal block columns, left to right
  for (int J = 1; J < nblk; ++J) {
    const int c0 = kTfB * J, jb = min(kTfB, bw - c0);
    for (int e = tid; e < c0 * jb; e += kTfThreads) {
      const int i = e / jb, c = e % jb;
      float t = 0.f;
      for (int k = i; k < c0; ++k) t += T[i][k] * Ys[k][c0 + c];
      X[i][c] = t;
    }
    __syncthreads();
    for (int e = tid; e < c0 * jb; e += kTfThreads) {
      const int i = e / jb, c = e % jb;
      float t = 0.f;
      for (int k = 0; k <= c; ++k) t += X[i][k] * T[c0 + k][c0 + c];
      T[i][c0 + c] = -t;
    }
    __syncthreads();
  }
  for (int e = tid; e < bw * bw; e += kTfThreads) {
    const int i = e / bw, k = e % bw;
    const float t = k >= i ? T[i][k] : 0.f;
    const float tt = i >= k ? T[k][i] : 0.f;
    for (int s2 = 0; s2 < a.reps_t; ++s2) TrT[static_cast<int64_t>(i) * bw * a.reps_t + s2 * bw + k] = tt;
    for (int s2 = 0; s2 < a.reps_q; ++s2) TrQ[static_cast<int64_t>(i) * bw * a.reps_q + s2 * bw + k] = t;
  }
}

// ----------------------------------------------------------- elementwise

__global__ void eye_kernel(float* Q, int64_t q_mat, int32_t n) {
  const int64_t b = blockIdx.y;
  const int64_t nn = static_cast<int64_t>(n) * n;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < nn;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    Q[b * q_mat + e] = (e / n == e % n) ? 1.f : 0.f;
}

__device__ __forceinline__ char* mat_entry(const MatBatch& m, int64_t b) {
  return m.ptrs ? static_cast<char*>(m.ptrs[b]) : m.base + b * m.stride_bytes;
}

constexpr int kRowChunk = 1024;  // columns per workgroup in the row-wise kernels

__global__ __launch_bounds__(256) void sign_copy_kernel(const float* src, int64_t src_mat, const float* sgn,
                                                        int64_t s_mat, MatBatch dst, int32_t n) {
  const int64_t b = blockIdx.y;
  const int chunks = (n + kRowChunk - 1) / kRowChunk;
  const int r = blockIdx.x / chunks, cc = blockIdx.x % chunks;
  const float* srow = src + b * src_mat + static_cast<int64_t>(r) * n;
  const float* sg = sgn + b * s_mat;
  float* drow = reinterpret_cast<float*>(mat_entry(dst, b)) + static_cast<int64_t>(r) * dst.ld;
  for (int j = cc * kRowChunk + threadIdx.x; j < min(n, (cc + 1) * kRowChunk); j += blockDim.x)
    drow[j] = srow[j] * sg[j];
}

__global__ __launch_bounds__(256) void gather_kernel(MatBatch src, float* dst, int64_t d_mat, int32_t rows,
                                                     int32_t cols) {
  const int64_t b = blockIdx.y;
  const int chunks = (cols + kRowChunk - 1) / kRowChunk;
  const int r = blockIdx.x / chunks, cc = blockIdx.x % chunks;
  const float* srow = reinterpret_cast<const float*>(mat_entry(src, b)) + static_cast<int64_t>(r) * src.ld;
  float* drow = dst + b * d_mat + static_cast<int64_t>(r) * cols;
  for (int j = cc * kRowChunk + threadIdx.x; j < min(cols, (cc + 1) * kRowChunk); j += blockDim.x)
    drow[j] = srow[j];
}

// [GUIDE] 11.1 in the rotated basis; epsilon after the square root.
__global__ __launch_bounds__(256) void rot_adam_kernel(RotAdamArgs a) {
  const int64_t b = blockIdx.y;
  const int chunks = (a.cols + kRowChunk - 1) / kRowChunk;
  const int r = blockIdx.x / chunks, cc = blockIdx.x % chunks;
  const char* grow = mat_entry(a.G, b) + static_cast<int64_t>(r) * a.G.ld * (a.G.dtype ? 2 : 4);
  float* mrow = reinterpret_cast<float*>(mat_entry(a.M, b)) + static_cast<int64_t>(r) * a.M.ld;
  float* vrow = reinterpret_cast<float*>(mat_entry(a.V, b)) + static_cast<int64_t>(r) * a.V.ld;
  float* orow = reinterpret_cast<float*>(mat_entry(a.out, b)) + static_cast<int64_t>(r) * a.out.ld;
  for (int j = cc * kRowChunk + threadIdx.x; j < min(a.cols, (cc + 1) * kRowChunk); j += blockDim.x) {
    const float g = load1(grow, a.G.dtype, j);
    const float m = a.beta1 * mrow[j] + (1.f - a.beta1) * g;
    const float v = a.beta2 * vrow[j] + (1.f - a.beta2) * g * g;
    mrow[j] = m;
    vrow[j] = v;
    orow[j] = (a.c1 * m) / (sqrtf(a.c2 * v) + a.eps);
  }
}

}  // namespace

namespace {

template <int TM, int CFG>
void launch_cfg(const SgemmArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((sgemm_kernel<TM, CFG>), grid, dim3(kThreads), 0, stream, a);
}

template <int TM, int CFG = 0>
void launch_fast(int cfg, const SgemmArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (CFG < 16) {
    if (cfg == CFG)
      launch_cfg<TM, CFG>(a, grid, stream);
    else
      launch_fast<TM, CFG + 1>(cfg, a, grid, stream);
  }
}

template <int CFG = -1>
void launch_list(int cfg, const SgemmList& l, int tiles, hipStream_t stream) {
  if constexpr (CFG < 16) {
    if (cfg == CFG)
      hipLaunchKernelGGL((sgemm_list_kernel<CFG>), dim3(tiles), dim3(kThreads), 0, stream, l);
    else
      launch_list<CFG + 1>(cfg, l, tiles, stream);
  }
}

// The fast path needs every 4-element run aligned and inside its row: both
// operands' vector flag, and K plus each operand's outer extent along its
// contiguous index a multiple of 4.
int fast_cfg(const SgemmArgs& a) {
  const bool ok = a.a.vec && a.b.vec && a.K % 4 == 0 && (a.a.kcontig || a.M % 4 == 0) &&
                  (a.b.kcontig || a.N % 4 == 0) && !a.a.ptrs && !a.b.ptrs;
  if (!ok) return -1;
  return (a.a.dtype ? 1 : 0) | (a.a.kcontig ? 2 : 0) | (a.b.dtype ? 4 : 0) | (a.b.kcontig ? 8 : 0);
}

}  // namespace

hipError_t launch_sgemm(const SgemmArgs& a, hipStream_t stream) {
  const int cfg = fast_cfg(a);
  if (a.M <= 32 && !a.sym) {
    const dim3 grid((a.N + kT - 1) / kT, (a.M + 31) / 32, a.count * a.splits);
    if (cfg >= 0)
      launch_fast<32>(cfg, a, grid, stream);
    else
      launch_cfg<32, -1>(a, grid, stream);
  } else {
    const int T = (a.N + kT - 1) / kT;  // a symmetric product has M = N
    const dim3 grid(a.sym ? T * (T + 1) / 2 : T, a.sym ? 1 : (a.M + kT - 1) / kT, a.count * a.splits);
    if (cfg >= 0)
      launch_fast<kT>(cfg, a, grid, stream);
    else
      launch_cfg<kT, -1>(a, grid, stream);
  }
  return hipGetLastError();
}

int64_t sgemm_list_tiles(const SgemmArgs& a) {
  const int64_t tn = (a.N + kT - 1) / kT;
  const int64_t per = a.sym ? tn * (tn + 1) / 2 : tn * ((a.M + kT - 1) / kT);
  return per * a.count * a.splits;
}

hipError_t launch_sgemm_list(const SgemmArgs* gs, int n, hipStream_t stream) {
  // Products that take the 32-row tiles, and products with a fast-path
  // configuration of their own, launch apart; the rest go in lists of at
  // most kSgemmMaxList, longest reduction first.
  bool done[kSgemmMaxList * 2] = {};
  if (n < 1 || n > kSgemmMaxList * 2) return hipErrorInvalidValue;
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const int cfg = fast_cfg(gs[i]);
    if (gs[i].M <= 32 && !gs[i].sym) {
      done[i] = true;
      const hipError_t e = launch_sgemm(gs[i], stream);
      if (e != hipSuccess) return e;
      continue;
    }
    int idx[kSgemmMaxList * 2], m = 0;
    for (int j = i; j < n; ++j)
      if (!done[j] && !(gs[j].M <= 32 && !gs[j].sym) && fast_cfg(gs[j]) == cfg) idx[m++] = j;
    std::sort(idx, idx + m, [&](int x, int y) { return gs[x].ksplit > gs[y].ksplit || (gs[x].ksplit == gs[y].ksplit && x < y); });
    for (int b = 0; b < m; b += kSgemmMaxList) {
      SgemmList l;
      std::memset(&l, 0, sizeof(l));
      int64_t tiles = 0;
      l.n = std::min(kSgemmMaxList, m - b);
      for (int k = 0; k < l.n; ++k) {
        l.g[k] = gs[idx[b + k]];
        done[idx[b + k]] = true;
        tiles += sgemm_list_tiles(l.g[k]);
        if (tiles > INT32_MAX) return hipErrorInvalidValue;
        l.tile_end[k] = static_cast<int32_t>(tiles);
      }
      if (tiles > 0) launch_list(cfg, l, static_cast<int>(tiles), stream);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_qr_panel(const QrPanelArgs& a, int64_t count, hipStream_t stream) {
  if (a.n - a.c0 <= kRegThreads * kRegRows)
    hipLaunchKernelGGL(qr_panel_reg_kernel, dim3(count), dim3(kRegThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(qr_panel_kernel, dim3(count), dim3(kQrThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qr_tfactor(const QrTArgs& a, int64_t count, hipStream_t stream) {
  hipLaunchKernelGGL(qr_tfactor_kernel, dim3(count), dim3(kTfThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_eye(float* Q, int64_t q_mat, int32_t n, int64_t count, hipStream_t stream) {
  const int64_t nn = static_cast<int64_t>(n) * n;
  const int blocks = static_cast<int>(std::min<int64_t>((nn + 255) / 256, 4096));
  hipLaunchKernelGGL(eye_kernel, dim3(blocks, count), dim3(256), 0, stream, Q, q_mat, n);
  return hipGetLastError();
}

hipError_t launch_sign_copy(const float* src, int64_t src_mat, const float* sgn, int64_t s_mat,
                            const MatBatch& dst, int32_t n, int64_t count, hipStream_t stream) {
  const int chunks = (n + kRowChunk - 1) / kRowChunk;
  hipLaunchKernelGGL(sign_copy_kernel, dim3(n * chunks, count), dim3(256), 0, stream, src, src_mat, sgn, s_mat,
                     dst, n);
  return hipGetLastError();
}

hipError_t launch_gather(const MatBatch& src, float* dst, int64_t d_mat, int32_t rows, int32_t cols,
                         int64_t count, hipStream_t stream) {
  const int chunks = (cols + kRowChunk - 1) / kRowChunk;
  hipLaunchKernelGGL(gather_kernel, dim3(rows * chunks, count), dim3(256), 0, stream, src, dst, d_mat, rows,
                     cols);
  return hipGetLastError();
}

hipError_t launch_rot_adam(const RotAdamArgs& a, int64_t count, hipStream_t stream) {
  const int chunks = (a.cols + kRowChunk - 1) / kRowChunk;
  hipLaunchKernelGGL(rot_adam_kernel, dim3(a.rows * chunks, count), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muon
