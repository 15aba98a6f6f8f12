// Newton-Schulz GEMM stages on CDNA4 matrix cores (gfx950).
//
// Every product of the iteration ("LLM Optimizers: From SGD and AdamW to
// SOAP, Muon, and Scalable Training", section 11.4; "Matrix optimizers:
// K-FAC, Shampoo and Muon", Lemma 3) is written as an NT product
// C = P * Q^T whose operands are both contiguous along the reduction index:
//
//   Gram    A = X X^T         P = Q = X            (symmetric: upper tiles)
//   poly    B = b A + c A A   P = Q = A  (A = A^T) (symmetric: upper tiles)
//   update  X' = a X + B X    P = B, Q = X^T       (X^T kept alongside X)
//
// so one kernel template serves all three, with the stage's epilogue fused.
//
// Tiling: a workgroup computes a BM x BM output tile (BM = 256 with eight
// wave64s in a 2x4 grid, each owning 128x64; BM = 128 with four wave64s in a
// 2x2 grid, each owning 64x64) out of 32x32 MFMA blocks with fp32
// accumulators.  Operand tiles are staged through
// LDS in 128-byte rows (one k-tile: 64 bf16 or 32 fp32 per row), double
// buffered, with the 16-byte chunks of each row XOR-swizzled by the row index
// so that the MFMA fragment reads of 32 consecutive rows spread over all
// banks.  Global loads for k-tile t+1 are issued before the MFMAs of k-tile t.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (one 16-byte chunk = 8 k values per
// lane).  fp32 path: v_mfma_f32_32x32x2_f32, four per 16-byte chunk.  In both
// the same lane/element -> k assignment is used for the two operands, so the
// product does not depend on the hardware's internal k order.

#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t Chunk __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static void mma(f32x16_t& acc, const Chunk& a, const Chunk& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static float load(const char* p) {
    return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  }
  __device__ __forceinline__ static void store(char* p, float v) {
    *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
  }
  // four consecutive elements
  __device__ __forceinline__ static void store4(char* p, float v0, float v1, float v2, float v3) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16(v0)) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16(v2)) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  // Bit-cast the whole chunk, then index it: bit-casting a single component
  // of an ext_vector (v.y) is miscompiled to read component x.
  __device__ __forceinline__ static void mma(f32x16_t& acc, const Chunk& a, const Chunk& b) {
    const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
    const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static float load(const char* p) {
    return *reinterpret_cast<const float*>(p);
  }
  __device__ __forceinline__ static void store(char* p, float v) {
    *reinterpret_cast<float*>(p) = v;
  }
  __device__ __forceinline__ static void store4(char* p, float v0, float v1, float v2, float v3) {
    *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
  }
};

__device__ __forceinline__ char* user_ptr(const MatBatch& m, int mat) {
  return m.ptrs ? static_cast<char*>(m.ptrs[mat]) : m.base + static_cast<int64_t>(mat) * m.stride_bytes;
}

__device__ __forceinline__ void store_user(const MatBatch& u, char* base, int64_t r, int64_t c, float v) {
  char* p = base + (r * u.ld + c) * (u.dtype ? 2 : 4);
  if (u.dtype) {
    *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
  } else {
    *reinterpret_cast<float*>(p) = v;
  }
}

constexpr int kRowBytes = 128;  // one k-tile row in LDS: 8 chunks of 16 bytes

// BM x BM output tile per workgroup; WGM x WGN waves, each owning a
// (BM/WGM) x (BM/WGN) sub-tile of 32x32 MFMA blocks.
template <typename T, int BM, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN)
void ns_gemm_kernel(const GemmLaunch L) {
  constexpr int NT = 64 * WGM * WGN;     // threads
  constexpr int WTM = BM / WGM;          // wave sub-tile rows
  constexpr int WTN = BM / WGN;          // wave sub-tile cols
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int CH = Elem<T>::kPerChunk;  // elements per 16-byte chunk
  constexpr int BK = 8 * CH;             // elements per k-tile
  constexpr int RPP = NT / 8;            // tile rows loaded per pass
  constexpr int LOADS = BM / RPP;        // chunks per thread per operand
  constexpr int OPB = BM * kRowBytes;    // bytes of one operand tile
  static_assert(LOADS * RPP == BM, "tile rows must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * OPB];

  // ---- which tile of which matrix of which group
  const int t = blockIdx.x;
  int gi = 0;
  while (gi + 1 < L.ngroups && t >= L.g[gi + 1].tile_begin) ++gi;
  const GemmGroup& G = L.g[gi];
  const int lt = t - G.tile_begin;
  const int mat = lt / G.tiles_per_mat;
  int tt = lt - mat * G.tiles_per_mat;
  int ti, tj;
  if (G.sym) {
    ti = 0;
    while (tt >= G.tiles_n - ti) {
      tt -= G.tiles_n - ti;
      ++ti;
    }
    tj = ti + tt;
  } else {
    ti = tt / G.tiles_n;
    tj = tt - ti * G.tiles_n;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN;
  const int wn = wave - wm * WGN;

  const int ldp = G.ldp;
  const int ldq = G.ldq;
  const int lrow = tid >> 3;  // 0..RPP-1
  const int lch = tid & 7;    // chunk within the row
  const char* Pl = G.P + mat * G.p_mat +
                   (static_cast<int64_t>(ti * BM + lrow) * ldp + lch * CH) * sizeof(T);
  const char* Ql = G.Q + mat * G.q_mat +
                   (static_cast<int64_t>(tj * BM + lrow) * ldq + lch * CH) * sizeof(T);
  const int64_t pstep = static_cast<int64_t>(RPP) * ldp * sizeof(T);
  const int64_t qstep = static_cast<int64_t>(RPP) * ldq * sizeof(T);
  int soff[LOADS];
#pragma unroll
  for (int r = 0; r < LOADS; ++r) {
    const int row = lrow + RPP * r;
    soff[r] = row * kRowBytes + ((lch ^ (row & 7)) << 4);
  }

  Chunk pr[LOADS], qr[LOADS];
#pragma unroll
  for (int r = 0; r < LOADS; ++r) {
    pr[r] = *reinterpret_cast<const Chunk*>(Pl + r * pstep);
    qr[r] = *reinterpret_cast<const Chunk*>(Ql + r * qstep);
  }
#pragma unroll
  for (int r = 0; r < LOADS; ++r) {
    *reinterpret_cast<Chunk*>(smem + soff[r]) = pr[r];
    *reinterpret_cast<Chunk*>(smem + OPB + soff[r]) = qr[r];
  }
  __syncthreads();

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int frow = lane & 31;
  const int half = lane >> 5;
  const int nk = G.K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t kb = static_cast<int64_t>(kt + 1) * BK * sizeof(T);
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        pr[r] = *reinterpret_cast<const Chunk*>(Pl + kb + r * pstep);
        qr[r] = *reinterpret_cast<const Chunk*>(Ql + kb + r * qstep);
      }
    }
    const char* sp = smem + (kt & 1) * 2 * OPB;
    const char* sq = sp + OPB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + half;
      Chunk af[FM], bfr[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int ra = wm * WTM + f * 32 + frow;
        af[f] = *reinterpret_cast<const Chunk*>(sp + ra * kRowBytes + ((ch ^ (ra & 7)) << 4));
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int rb = wn * WTN + f * 32 + frow;
        bfr[f] = *reinterpret_cast<const Chunk*>(sq + rb * kRowBytes + ((ch ^ (rb & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Elem<T>::mma(acc[i][j], af[i], bfr[j]);
    }
    if (more) {
      char* dp = smem + ((kt + 1) & 1) * 2 * OPB;
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        *reinterpret_cast<Chunk*>(dp + soff[r]) = pr[r];
        *reinterpret_cast<Chunk*>(dp + OPB + soff[r]) = qr[r];
      }
    }
    __syncthreads();
  }

  // ---- epilogue.  acc[fi][fj][4q+e] holds C[i][j] with
  //   i = ti*BM + wm*WTM + fi*32 + 8q + 4*half + e
  //   j = tj*BM + wn*WTN + fj*32 + lane%32
  const int i_base = ti * BM + wm * WTM + 4 * half;
  const int j_base = tj * BM + wn * WTN + frow;

  if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) {
    char* Om = G.O0 + mat * G.o0_mat;
    const int ldo = G.ldo0;
    const char* Em = (EPI == EPI_POLY) ? G.E0 + mat * G.e0_mat : nullptr;
    const int lde = G.lde0;
    const bool mirror = (ti != tj);
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i0 = i_base + fi * 32 + 8 * q;
          const int j = j_base + fj * 32;
          float v0 = acc[fi][fj][4 * q + 0];
          float v1 = acc[fi][fj][4 * q + 1];
          float v2 = acc[fi][fj][4 * q + 2];
          float v3 = acc[fi][fj][4 * q + 3];
          if constexpr (EPI == EPI_POLY) {
            const char* e = Em + (static_cast<int64_t>(i0) * lde + j) * sizeof(T);
            const int64_t rs = static_cast<int64_t>(lde) * sizeof(T);
            v0 = L.b * Elem<T>::load(e) + L.c * v0;
            v1 = L.b * Elem<T>::load(e + rs) + L.c * v1;
            v2 = L.b * Elem<T>::load(e + 2 * rs) + L.c * v2;
            v3 = L.b * Elem<T>::load(e + 3 * rs) + L.c * v3;
          }
          // C[j][i0..i0+3] = C[i0..i0+3][j] by symmetry: one contiguous store
          Elem<T>::store4(Om + (static_cast<int64_t>(j) * ldo + i0) * sizeof(T), v0, v1, v2, v3);
          if (mirror) {
            char* o = Om + (static_cast<int64_t>(i0) * ldo + j) * sizeof(T);
            const int64_t rs = static_cast<int64_t>(ldo) * sizeof(T);
            Elem<T>::store(o, v0);
            Elem<T>::store(o + rs, v1);
            Elem<T>::store(o + 2 * rs, v2);
            Elem<T>::store(o + 3 * rs, v3);
          }
        }
  } else if constexpr (EPI == EPI_UPDATE) {
    const float* Em = reinterpret_cast<const float*>(G.E0 + mat * G.e0_mat);  // fp32 X
    const int lde = G.lde0;
    float* O0m = reinterpret_cast<float*>(G.O0 + mat * G.o0_mat);           // fp32 X'
    const int ldo0 = G.ldo0;
    uint16_t* O1m = G.O1 ? reinterpret_cast<uint16_t*>(G.O1 + mat * G.o1_mat) : nullptr;
    const int ldo1 = G.ldo1;
    char* OTm = G.OT + mat * G.ot_mat;                                      // X'^T
    const int ldot = G.ldot;
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i0 = i_base + fi * 32 + 8 * q;
          const int j = j_base + fj * 32;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = L.a * Em[static_cast<int64_t>(i0 + e) * lde + j] + acc[fi][fj][4 * q + e];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            O0m[static_cast<int64_t>(i0 + e) * ldo0 + j] = v[e];
            if (O1m) O1m[static_cast<int64_t>(i0 + e) * ldo1 + j] = f32_to_bf16(v[e]);
          }
          Elem<T>::store4(OTm + (static_cast<int64_t>(j) * ldot + i0) * sizeof(T), v[0], v[1], v[2], v[3]);
        }
  } else {  // EPI_FINAL: a*X + B*X into the caller's output, clipped to ms x ns
    const float* Em = reinterpret_cast<const float*>(G.E0 + mat * G.e0_mat);
    const int lde = G.lde0;
    char* U = user_ptr(G.user, mat);
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i0 = i_base + fi * 32 + 8 * q;
          const int j = j_base + fj * 32;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float v = L.a * Em[static_cast<int64_t>(i) * lde + j] + acc[fi][fj][4 * q + e];
            if (i < G.ms && j < G.ns) {
              if (G.tall) {
                store_user(G.user, U, j, i, v);
              } else {
                store_user(G.user, U, i, j, v);
              }
            }
          }
        }
  }
}

template <typename T, int BM, int WGM, int WGN>
hipError_t launch_t(int epi, const GemmLaunch& L, hipStream_t stream) {
  dim3 grid(L.total_tiles), block(64 * WGM * WGN);
  switch (epi) {
    case EPI_GRAM:
      hipLaunchKernelGGL((ns_gemm_kernel<T, BM, WGM, WGN, EPI_GRAM>), grid, block, 0, stream, L);
      break;
    case EPI_POLY:
      hipLaunchKernelGGL((ns_gemm_kernel<T, BM, WGM, WGN, EPI_POLY>), grid, block, 0, stream, L);
      break;
    case EPI_UPDATE:
      hipLaunchKernelGGL((ns_gemm_kernel<T, BM, WGM, WGN, EPI_UPDATE>), grid, block, 0, stream, L);
      break;
    default:
      hipLaunchKernelGGL((ns_gemm_kernel<T, BM, WGM, WGN, EPI_FINAL>), grid, block, 0, stream, L);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_gemm(int compute, int tile, int epi, const GemmLaunch& L, hipStream_t stream) {
  if (L.total_tiles <= 0) return hipSuccess;
  if (compute == 1) {
    return tile == 256 ? launch_t<uint16_t, 256, 2, 4>(epi, L, stream)
                       : launch_t<uint16_t, 128, 2, 2>(epi, L, stream);
  }
  return tile == 256 ? launch_t<float, 256, 2, 4>(epi, L, stream)
                     : launch_t<float, 128, 2, 2>(epi, L, stream);
}

}  // namespace muon
