// Newton-Schulz GEMM stages on CDNA4 matrix cores (gfx950).
//
// Every product of the iteration ("LLM Optimizers: From SGD and AdamW to
// SOAP, Muon, and Scalable Training", section 11.4; "Matrix optimizers:
// K-FAC, Shampoo and Muon", Lemma 3) is written as an NT product
// C = P * Q^T whose operands are both contiguous along the reduction index:
//
//   Gram    A = X X^T         P = Q = X            (symmetric: upper tiles)
//   poly    B = b A + c A A   P = Q = A  (A = A^T) (symmetric: upper tiles)
//   update  X' = a X + B X    P = B, Q = X^T       (fp32: X^T kept alongside X)
//
// so one kernel template serves all three, with the stage's epilogue fused.
// With bf16 compute the update instead reads X itself as a k-major second
// operand (row k of X holds the tile's columns contiguously) through LDS
// transpose reads, and no X^T is kept.
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

#include "lo8.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t Chunk __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  In each group of 16 lanes,
// lane j names an 8-byte piece P[j] (four 16-bit values); lane i receives
// P[4e + i/4][i%4] as its value e (checked by an in-bounds probe).  So when
// lane j points at row k0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major
// 16-bit tile, lane i receives column c0 + i of rows k0 .. k0+3.
__device__ __forceinline__ u32x2_t lds_read_tr(const char* p) {
  const i16x4_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

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
  static constexpr int kMfmaPerChunk = 1;
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
  // eight consecutive elements (16 bytes)
  __device__ __forceinline__ static void store8(char* p, const float4& a, const float4& b) {
    uint4 u;
    u.x = bf16_pair(a.x, a.y);
    u.y = bf16_pair(a.z, a.w);
    u.z = bf16_pair(b.x, b.y);
    u.w = bf16_pair(b.z, b.w);
    *reinterpret_cast<uint4*>(p) = u;
  }
  // four consecutive elements
  __device__ __forceinline__ static void store4(char* p, float v0, float v1, float v2, float v3) {
    uint2 u;
    u.x = bf16_pair(v0, v1);
    u.y = bf16_pair(v2, v3);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kMfmaPerChunk = 4;
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
  __device__ __forceinline__ static void store8(char* p, const float4& a, const float4& b) {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
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

// The parameter update folded into the last step ("LLM Optimizers: From SGD
// and AdamW to SOAP, Muon, and Scalable Training", section 11.5 update
// equation): W <- decay * W - step * O on the caller's weight, read and
// written in its own dtype, fp32 arithmetic as in the separate apply call.
__device__ __forceinline__ void apply_user(const MatBatch& u, char* base, int64_t r, int64_t c, float v, float decay,
                                           float step) {
  char* p = base + (r * u.ld + c) * (u.dtype ? 2 : 4);
  if (u.dtype) {
    const float w = bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
    *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(decay * w - step * v);
  } else {
    float* q = reinterpret_cast<float*>(p);
    *q = decay * *q - step * v;
  }
}
// ... eight consecutive elements (16-byte aligned)
__device__ __forceinline__ void apply8(char* p, int dtype, float decay, float step, const float4& a,
                                       const float4& b) {
  const float o[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float w[8];
  if (dtype) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[2 * k] = bf16_to_f32(static_cast<uint16_t>(q[k]));
      w[2 * k + 1] = bf16_to_f32(static_cast<uint16_t>(q[k] >> 16));
    }
  } else {
    const float4 x0 = reinterpret_cast<const float4*>(p)[0];
    const float4 x1 = reinterpret_cast<const float4*>(p)[1];
    w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
    w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = decay * w[e] - step * o[e];
  const float4 y0 = make_float4(w[0], w[1], w[2], w[3]), y1 = make_float4(w[4], w[5], w[6], w[7]);
  if (dtype) {
    Elem<uint16_t>::store8(p, y0, y1);
  } else {
    Elem<float>::store8(p, y0, y1);
  }
}

// Physical 16-byte slot of logical chunk c in an LDS row of RC chunks.  A
// ds_read_b128 from 16 consecutive rows at one logical chunk is one cycle of
// the 64-bank (256-byte) gfx950 LDS when the 16 slots are distinct modulo
// 256 bytes: rows sharing a 256-byte phase (row mod 16/RC) get different
// chunks.  SWZ = 0 is the 32-bank pattern (8 consecutive rows distinct).
template <int SWZ, int RC>
__device__ __forceinline__ int swizzle(int row, int c) {
  constexpr int kPhase = 16 / RC;  // rows per 256 bytes
  return SWZ ? (c ^ ((row / kPhase) & (RC - 1))) : (c ^ (row & (RC - 1)));
}

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's
// 16 bytes at base + off land at LDS address l + 16 i.  Issued as inline asm:
// after the intrinsic form the compiler puts a wait for every outstanding
// vector load (vmcnt 0) in front of each later ds_read_b64_tr_b16, which
// would make the k-major update wait for the next k-tile's copy in every
// k-tile.  The kernel orders these copies itself (barrier_keep_vm); nothing
// reads a register written by them.
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, char* l) {
  const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(l)));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(la))
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14,
  // expcnt (7) in bits 6:4 and lgkmcnt (15) in bits 11:8 left unconstrained.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that keeps later-issued DMA loads in flight: wait for
// this wave's LDS reads (lgkmcnt 0) and for all but the newest N vector
// loads, then s_barrier.  (__syncthreads() would wait for every load.)
template <int N>
__device__ __forceinline__ void barrier_keep_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
}

// BM x BM output tile per workgroup; WGM x WGN waves, each owning a
// (BM/WGM) x (BM/WGN) sub-tile of 32x32 MFMA blocks.
//   RC:     16-byte chunks per LDS row (k-tile = RC*16 bytes of k).
//   STAGES: LDS ring depth; k-tile t+STAGES-1 is in flight while t is used.
//   SWZ:    LDS swizzle (see swizzle()).
//   DMA:    1 = operand tiles go global -> LDS with global_load_lds_dwordx4
//           (no staging registers); 0 = through VGPRs (two stages only).
//   XCD:    1 = renumber workgroups so each of the 8 XCDs (which receive
//           workgroup ids round-robin) works on a contiguous tile range of
//           every group.
//   SCHED:  0 = compiler schedule; 1 = pin the order of MFMAs and the next
//           substep's LDS reads.
//   GM:     tiles of a non-symmetric product are numbered in groups of GM
//           tile rows, column by column inside a group, so that workgroups
//           running together (one XCD's range under XCD = 1) share GM row
//           blocks of P and a few column blocks of Q in L2.
//   QN:     1 = the bf16 update's second operand is X itself, k-major (read
//           through LDS transpose reads); 0 = it is X^T, n-major.
template <typename T, int BM, int WGM, int WGN, int EPI, int RC = 4, int STAGES = 4, int SWZ = 1, int DMA = 1,
          int XCD = 0, int SCHED = 0, int GM = 1, int BN = BM, int QN = 0, int AP = 0>
__global__ __launch_bounds__(64 * WGM * WGN, 2)  // at least two waves per SIMD
void ns_gemm_kernel(const GemmLaunch L) {
  constexpr int NW = WGM * WGN;          // waves
  constexpr int NT = 64 * NW;            // threads
  constexpr int WTM = BM / WGM;          // wave sub-tile rows
  constexpr int WTN = BN / WGN;          // wave sub-tile cols
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int CH = Elem<T>::kPerChunk;  // elements per 16-byte chunk
  constexpr int ROWB = RC * 16;          // bytes per LDS row
  constexpr int BK = RC * CH;            // elements per k-tile
  constexpr int SUB = RC / 2;            // MFMA substeps per k-tile (2 chunks each)
  constexpr int RPP = NT / RC;           // tile rows per register-path pass
  constexpr int LOADS = BM / RPP;        // P chunks per thread (register path)
  constexpr int LOADSQ = BN / RPP;       // Q chunks per thread (register path)
  constexpr int RPI = 64 / RC;           // rows per DMA instruction (64 lanes x 16 bytes)
  constexpr int IPW = BM / (RPI * NW);   // P DMA instructions per wave
  constexpr int IPWQ = BN / (RPI * NW);  // Q DMA instructions per wave
  constexpr int OPB = BM * ROWB;         // bytes of the P tile (the Q tile follows)
  constexpr int STB = (BM + BN) * ROWB;  // bytes of one stage
  static_assert(DMA || STAGES == 2, "the register path is double-buffered");
  // bf16 update: Q is X, k-major; a k-tile of it is BK rows of QROWB bytes,
  // 16-byte chunks XOR-swizzled in groups of four by (row % 4), so that the
  // transpose reads of 4 consecutive rows x 64 bytes hit all 64 banks once.
  constexpr bool kQN = QN && (EPI == EPI_UPDATE || EPI == EPI_FINAL) && sizeof(T) == 2;
  static_assert(kQN || sizeof(T) == 4 || !(EPI == EPI_UPDATE || EPI == EPI_FINAL), "the bf16 update reads X k-major");
  constexpr int QROWB = BN * 2;
  constexpr int QRC = QROWB / 16;
  static_assert(!kQN || (DMA && QRC >= 16 && BK * QROWB == BN * ROWB), "k-major Q tile: same bytes as n-major");
  static_assert(LOADS * RPP == BM && LOADSQ * RPP == BN, "tile rows must split evenly over the threads");
  static_assert(IPW * RPI * NW == BM && IPWQ * RPI * NW == BN, "tile rows must split evenly over the waves");
  constexpr int EPI_BYTES = NW * 64 * 68 * 4;  // transposed-store staging
  constexpr int SMEM = STAGES * STB > EPI_BYTES ? STAGES * STB : EPI_BYTES;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  // Tiles t = blockIdx.x, + gridDim.x, ...: one tile per workgroup when the
  // grid covers the launch, several in turn when the host chose a persistent
  // grid (a multiple of 8, so every tile of a workgroup is on its XCD).
  // ---- which tile of which matrix of which group
  constexpr int R = BM / BN;  // column tiles per row tile
  static_assert(R * BN == BM, "BN must divide BM");
  auto decode = [&](int t, int& gi, int& mat, int& slice, int& ti, int& tj) {
    gi = 0;
    while (gi + 1 < L.ngroups && t >= L.g[gi + 1].tile_begin) ++gi;
    const GemmGroup& G = L.g[gi];
    int lt = t - G.tile_begin;  // position within the group
    if (XCD) {
      // Workgroup ids reach the 8 XCDs round-robin.  Inside each group, the
      // positions that land on one XCD are renumbered to one contiguous range
      // of the group's tiles: every XCD keeps a proportional share of every
      // group (groups of unequal tile cost stay balanced across XCDs) and
      // neighbouring tiles on an XCD share its L2.
      const int n = G.tiles_per_mat * G.count;
      const int f = (t - G.tile_begin) & 7;  // first in-group position on this XCD
      int start = 0;
      for (int e = 0; e < f; ++e) start += (n - e + 7) >> 3;  // positions on XCDs ranked before
      lt = start + ((lt - f) >> 3);
    }
    mat = lt / G.tiles_per_mat;
    int tt = lt - mat * G.tiles_per_mat;
    slice = 0;  // split Gram: slice of the reduction this tile sums
    if (G.splits > 1) {
      slice = tt % G.splits;
      tt /= G.splits;
    }
    if (G.sym) {
      // upper tiles only: row tile ti keeps column tiles tj >= R*ti
      ti = 0;
      while (tt >= G.tiles_n - R * ti) {
        tt -= G.tiles_n - R * ti;
        ++ti;
      }
      tj = R * ti + tt;
    } else if (GM == 1) {
      ti = tt / G.tiles_n;
      tj = tt - ti * G.tiles_n;
    } else {
      const int span = GM * G.tiles_n;          // tiles in one full group of GM rows
      const int grp = tt / span;
      const int in = tt - grp * span;
      const int rows = min(GM, G.tiles_m - grp * GM);  // the last group may be shorter
      tj = in / rows;
      ti = grp * GM + (in - tj * rows);
    }
  };

  // bf16 update on a persistent grid: the next tile's first k-tile is copied
  // into stage 0 during this tile's epilogue (which then stages in bf16 above
  // stage 0), so that its latency is off the next tile's prologue
  constexpr bool kXPF = EPI == EPI_UPDATE && sizeof(T) == 2 && DMA && STAGES == 2;
  bool pf = false;  // this tile's first k-tile is already on its way
  for (int t = blockIdx.x; t < L.total_tiles; t += gridDim.x) {
    if (t != static_cast<int>(blockIdx.x)) {  // the previous tile is done with LDS
      if constexpr (kXPF) {
        barrier_keep_vm<63>();  // (its stores and the prefetch are waited for in the prologue)
      } else {
        __syncthreads();
      }
    }
    int gi, mat, slice, ti, tj;
    decode(t, gi, mat, slice, ti, tj);
    const GemmGroup& G = L.g[gi];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN;
    const int wn = wave - wm * WGN;

    const int ldp = G.ldp;
    const int ldq = G.ldq;
    const int ksl = G.splits > 1 ? G.K / G.splits : G.K;  // reduction length of this tile
    const int64_t k0 = static_cast<int64_t>(slice) * ksl * sizeof(T);  // (the split Gram is never k-major)
    const char* Pt = G.P + mat * G.p_mat + static_cast<int64_t>(ti) * BM * ldp * sizeof(T) + k0;
    // a k-major Q starts at the tile's first column, an n-major one at its first row
    const char* Qt = G.Q + mat * G.q_mat + static_cast<int64_t>(tj) * BN * (kQN ? 1 : ldq) * sizeof(T) + k0;
    const int nk = ksl / BK;
    // A diagonal tile of a symmetric product multiplies a block of rows by
    // itself: its Q tile is the P tile already in LDS, so only P is loaded.
    // Not on a persistent grid: there the workgroups walk their tiles nearly
    // in step and share k-tiles in L2, and diagonal tiles finishing early
    // break that (measured slower on the 32-layer dense set, faster with one
    // workgroup per tile).
    const bool same_pq = R == 1 && G.sym && ti == tj && G.P == G.Q && G.p_mat == G.q_mat && ldp == ldq && !kQN &&
                         static_cast<int>(gridDim.x) == L.total_tiles;

    // ---- operand staging
    uint32_t dofs_p[DMA ? IPW : 1], dofs_q[DMA ? IPWQ : 1];  // DMA: lane byte offsets within the tile
    int soff[DMA ? 1 : LOADS];                               // register path: LDS slot offsets
    Chunk pr[DMA ? 1 : LOADS], qr[DMA ? 1 : LOADSQ];
    const char* Pl = nullptr;
    const char* Ql = nullptr;
    int64_t pstep = 0, qstep = 0;
    if constexpr (DMA) {
#pragma unroll
      for (int r = 0; r < IPW; ++r) {
        const int row = (wave * IPW + r) * RPI + lane / RC;
        const int c = swizzle<SWZ, RC>(row, lane % RC);
        dofs_p[r] = static_cast<uint32_t>((row * ldp + c * CH) * static_cast<int>(sizeof(T)));
      }
#pragma unroll
      for (int r = 0; r < IPWQ; ++r) {
        if constexpr (kQN) {
          const int slot = (wave * IPWQ + r) * 64 + lane;  // 16-byte slot of the k-tile in LDS
          const int row = slot / QRC;                      // k
          const int c = (slot % QRC) ^ ((row & 3) << 2);   // logical chunk: columns 8c .. 8c+7
          dofs_q[r] = static_cast<uint32_t>(row * ldq * 2 + c * 16);
        } else {
          const int row = (wave * IPWQ + r) * RPI + lane / RC;
          const int c = swizzle<SWZ, RC>(row, lane % RC);
          dofs_q[r] = static_cast<uint32_t>((row * ldq + c * CH) * static_cast<int>(sizeof(T)));
        }
      }
    } else {
      const int lrow = tid / RC;
      const int lch = tid % RC;
      Pl = Pt + (static_cast<int64_t>(lrow) * ldp + lch * CH) * sizeof(T);
      Ql = Qt + (static_cast<int64_t>(lrow) * ldq + lch * CH) * sizeof(T);
      pstep = static_cast<int64_t>(RPP) * ldp * sizeof(T);
      qstep = static_cast<int64_t>(RPP) * ldq * sizeof(T);
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        const int row = lrow + RPP * r;
        soff[r] = row * ROWB + (swizzle<SWZ, RC>(row, lch) << 4);
      }
    }

    // DMA: issue k-tile kt into LDS stage st (lands asynchronously; vmcnt).
    // (dma_issue_at: the same for the tile whose operands start at P0, Q0)
    auto dma_issue_at = [&](const char* P0, const char* Q0, int kt, int st) {
      const int64_t kb = static_cast<int64_t>(kt) * BK * sizeof(T);
      const char* pk = P0 + kb;
      const char* qk = Q0 + (kQN ? static_cast<int64_t>(kt) * BK * ldq * static_cast<int64_t>(sizeof(T)) : kb);
      char* lp = smem + st * STB + wave * IPW * 1024;
      char* lq = smem + st * STB + OPB + wave * IPWQ * 1024;
#pragma unroll
      for (int r = 0; r < IPW; ++r) lds_dma16(pk, dofs_p[r], lp + r * 1024);
      if (!same_pq) {
#pragma unroll
        for (int r = 0; r < IPWQ; ++r) lds_dma16(qk, dofs_q[r], lq + r * 1024);
      }
    };
    auto dma_issue = [&](int kt, int st) { dma_issue_at(Pt, Qt, kt, st); };
    auto reg_load = [&](int kt) {
      const int64_t kb = static_cast<int64_t>(kt) * BK * sizeof(T);
#pragma unroll
      for (int r = 0; r < LOADS; ++r) pr[r] = *reinterpret_cast<const Chunk*>(Pl + kb + r * pstep);
#pragma unroll
      for (int r = 0; r < LOADSQ; ++r) qr[r] = *reinterpret_cast<const Chunk*>(Ql + kb + r * qstep);
    };
    auto reg_store = [&](int st) {
      char* dp = smem + st * STB;
#pragma unroll
      for (int r = 0; r < LOADS; ++r) *reinterpret_cast<Chunk*>(dp + soff[r]) = pr[r];
#pragma unroll
      for (int r = 0; r < LOADSQ; ++r) *reinterpret_cast<Chunk*>(dp + OPB + soff[r]) = qr[r];
    };

    // ---- accumulators (fp32, from zero: the update's a*X term is added later,
    // its bf16 high part when the main loop reaches the k-tiles that hold it
    // and the rest in the epilogue, so the running sum's early roundings are
    // at the scale of the product itself)
    const int frow = lane & 31;
    const int half = lane >> 5;
    const int i_base = ti * BM + wm * WTM + 4 * half;  // acc[fi][fj][4q+e]: row i_base + fi*32 + 8q + e
    const int j_base = tj * BN + wn * WTN + frow;      //                    col j_base + fj*32
    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr int kPerTile = IPW + IPWQ;  // DMA instructions per wave per k-tile
    static_assert(SUB % 2 == 0, "fragment double buffer assumes an even substep count");
    if constexpr (DMA) {
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk && !(kXPF && pf)) dma_issue(s, s);
      if (nk >= STAGES - 1) {
        barrier_keep_vm<(STAGES - 2) * kPerTile>();  // k-tile 0 has landed
      } else {
        barrier_keep_vm<0>();
      }
      pf = false;
    } else {
      reg_load(0);
      reg_store(0);
      __syncthreads();
    }

    int fa_off[FM], fb_off[FN], fa_row[FM], fb_row[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      fa_row[f] = wm * WTM + f * 32 + frow;
      fa_off[f] = fa_row[f] * ROWB;
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      fb_row[f] = wn * WTN + f * 32 + frow;
      fb_off[f] = (same_pq ? 0 : OPB) + fb_row[f] * ROWB;
    }
    // k-major Q: lane j of a 16-lane group points at row (j/4) of a group of
    // four and at columns 4*(j%4) .. +3 of its 16-column half of block f;
    // rows of one read are congruent mod 4 to j/4, which fixes the swizzle
    int qn_off[kQN ? FN : 1];
    if constexpr (kQN) {
      const int j = lane & 15;
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int col = wn * WTN + f * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
        qn_off[f] = (j >> 2) * QROWB + (((col >> 3) ^ ((j >> 2) << 2)) << 4) + (col & 7) * 2;
      }
    }

    // Main loop.  Fragments of substep s+1 are read while the MFMAs of
    // substep s run; at the last substep of k-tile kt the wave waits for its
    // own DMA of k-tile kt+1, joins the barrier, and reads k-tile kt+1's first
    // fragments before issuing kt's last MFMAs, so the barrier and the LDS
    // latency overlap matrix work.  The barrier also retires every read of
    // k-tile kt's stage, which the DMA issued next iteration overwrites.
    Chunk af[2][FM], bfr[2][FN];
    auto frags = [&](const char* sb, int s, Chunk* a, Chunk* b) {
      const int ch = 2 * s + half;
#pragma unroll
      for (int f = 0; f < FM; ++f)
        a[f] = *reinterpret_cast<const Chunk*>(sb + fa_off[f] + (swizzle<SWZ, RC>(fa_row[f], ch) << 4));
      if constexpr (kQN) {
        // k = 16s + 8*half + 0..7 of column l%32: two transpose reads
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const char* q = sb + OPB + qn_off[f] + (8 * half + 16 * s) * QROWB;
          const u32x2_t lo = lds_read_tr(q);
          const u32x2_t hi = lds_read_tr(q + 4 * QROWB);
          b[f] = Chunk{lo.x, lo.y, hi.x, hi.y};
        }
      } else {
#pragma unroll
        for (int f = 0; f < FN; ++f)
          b[f] = *reinterpret_cast<const Chunk*>(sb + fb_off[f] + (swizzle<SWZ, RC>(fb_row[f], ch) << 4));
      }
    };
    frags(smem, 0, af[0], bfr[0]);
    // bf16 update: the high part of a*X enters from the operand tiles (below),
    // the epilogue adds only the low part.  k-tile kt_x0 + hh of Q (X,
    // k-major) holds rows [hh*BK, (hh+1)*BK) of this wave's sub-tile, i.e.
    // kFPK of its 32-row blocks, at the wave's columns.
    constexpr bool kAddXInLoop = (EPI == EPI_UPDATE || EPI == EPI_FINAL) && sizeof(T) == 2;
    constexpr int kFPK = BK / 32;
    constexpr int kNH = WTM / BK;
    static_assert(!kAddXInLoop || (kNH * BK == WTM && kFPK * 32 == BK && RC == 2 * kFPK * 2),
                  "wave rows must split into whole k-tiles of whole 32-row blocks");
    static_assert(!(EPI == EPI_POLY && sizeof(T) == 2) || (kNH * BK == WTM && kFPK * 32 == BK && RC == 4 * kFPK),
                  "the polynomial's in-loop term assumes whole k-tiles of whole 32-row blocks");
    const int kt_x0 = (ti * BM + wm * WTM) / BK;
    // Step 0 from a packed, unnormalized input N (the momentum kernel wrote
    // N itself): X_0 = xs*N with xs = 1/(||N|| + eps).  The Gram is then xs^2
    // times its product, the polynomial takes xs*b and xs*c (B_0 is stored
    // already multiplied by xs) and the update xs*a, so that
    // X_1 = xs*a*N + (xs*B_0)*N.  Otherwise xs = 1 and these are the
    // coefficients themselves.
    // (The Gram needs xs only in its epilogue: computed there, it holds no
    // register through the main loop, where the Gram uses all 256.)
    auto scale_of = [&]() { return G.xs_sumsq != nullptr ? 1.0f / (sqrtf(G.xs_sumsq[mat]) + G.xs_eps) : 1.0f; };
    const float xs = EPI == EPI_GRAM ? 1.0f : scale_of();
    const float at = L.a * xs;
    const float bt = L.b * xs;
    const float ct = L.c * xs;
    // bf16 polynomial with c != 0: B = c * (A*A + (b/c) * A), and (b/c) * A
    // enters the accumulator from the operand tiles, as the update's a * X
    // does: A is symmetric, so the second operand's k-tiles that cover this
    // wave's rows hold A[j][i] = A[i][j] for its output elements.  The
    // epilogue then only scales by c and loads nothing.
    const float bc = ct != 0.0f ? bt / ct : 0.0f;
    const bool poly_in_loop = EPI == EPI_POLY && sizeof(T) == 2 && ct != 0.0f && __builtin_isfinite(bc);
    int st = 0;  // stage holding k-tile kt
    for (int kt = 0; kt < nk; ++kt) {
      const bool issue = DMA ? (kt + STAGES - 1 < nk) : (kt + 1 < nk);
      if (issue) {
        if constexpr (DMA) {
          int sn = st + STAGES - 1;
          if (sn >= STAGES) sn -= STAGES;
          dma_issue(kt + STAGES - 1, sn);
        } else {
          reg_load(kt + 1);
        }
      }
      const char* sb = smem + st * STB;
      const int stn = (st + 1 == STAGES) ? 0 : st + 1;
      if constexpr (EPI == EPI_POLY && sizeof(T) == 2 && !kQN) {
        // row j of the second operand's k-tile, k = i: chunk 4f + q holds
        // k = 32f + 8q .. +7 of it, and this lane's four rows start 4*half in
#pragma unroll
        for (int hh = 0; hh < kNH; ++hh) {
          if (poly_in_loop && kt == kt_x0 + hh) {  // uniform over the wave
#pragma unroll
            for (int f = 0; f < kFPK; ++f)
#pragma unroll
              for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int fi = hh * kFPK + f;
                  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(
                      sb + fb_off[fj] + (swizzle<SWZ, RC>(fb_row[fj], 4 * f + q) << 4) + 8 * half);
                  acc[fi][fj][4 * q + 0] += bc * bf16_to_f32(static_cast<uint16_t>(v.x));
                  acc[fi][fj][4 * q + 1] += bc * bf16_to_f32(static_cast<uint16_t>(v.x >> 16));
                  acc[fi][fj][4 * q + 2] += bc * bf16_to_f32(static_cast<uint16_t>(v.y));
                  acc[fi][fj][4 * q + 3] += bc * bf16_to_f32(static_cast<uint16_t>(v.y >> 16));
                }
          }
        }
      }
      if constexpr (kAddXInLoop) {
        // a * X[i][j] = a * Q[k = i][j]: the k-tiles that cover this wave's
        // rows hold the bf16 high part of X for its output elements.
#pragma unroll
        for (int hh = 0; hh < kNH; ++hh) {
          if (kt == kt_x0 + hh) {  // uniform over the wave
#pragma unroll
            for (int f = 0; f < kFPK; ++f)
#pragma unroll
              for (int fj = 0; fj < FN; ++fj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  // rows f*32 + 8q + 4*half + 0..3 of the k-tile, column l%32 of block fj
                  const int fi = hh * kFPK + f;
                  const u32x2_t v = lds_read_tr(sb + OPB + qn_off[fj] + (f * 32 + 8 * q + 4 * half) * QROWB);
                  acc[fi][fj][4 * q + 0] += at * bf16_to_f32(static_cast<uint16_t>(v.x));
                  acc[fi][fj][4 * q + 1] += at * bf16_to_f32(static_cast<uint16_t>(v.x >> 16));
                  acc[fi][fj][4 * q + 2] += at * bf16_to_f32(static_cast<uint16_t>(v.y));
                  acc[fi][fj][4 * q + 3] += at * bf16_to_f32(static_cast<uint16_t>(v.y >> 16));
                }
          }
        }
      }
      auto mma_range = [&](int cur, int q0, int q1) {
#pragma unroll
        for (int q = q0; q < q1; ++q) Elem<T>::mma(acc[q / FN][q % FN], af[cur][q / FN], bfr[cur][q % FN]);
      };
      constexpr int NQ = FM * FN;
      constexpr int kMf = Elem<T>::kMfmaPerChunk;
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int cur = s & 1;  // SUB is even: k-tile kt+1 starts in buffer 0 again
        if (s + 1 < SUB) {
          frags(sb, s + 1, af[cur ^ 1], bfr[cur ^ 1]);
          mma_range(cur, 0, NQ);
          if constexpr (SCHED == 1) {
            // two MFMAs (their operands' wait comes first), the next substep's
            // reads, then the remaining MFMAs
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * kMf, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, (NQ - 2) * kMf, 0);
          }
        } else {
          // Half of the last substep's MFMAs go before the barrier so the MFMA
          // pipe stays busy while the wave waits in it.  The barrier and the
          // next k-tile's first reads are unconditional, also after the last
          // k-tile (the reads are then unused but in bounds): a branch would
          // merge two different counts of outstanding LDS reads and force a
          // full lgkmcnt wait.
          mma_range(cur, 0, NQ / 2);
          if constexpr (DMA) {
            if (kt + STAGES - 1 < nk) {
              barrier_keep_vm<(STAGES - 2) * kPerTile>();  // k-tile kt+1 has landed for this wave
            } else {
              barrier_keep_vm<0>();
            }
          } else {
            if (issue) reg_store(stn);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS stores done
            __builtin_amdgcn_s_barrier();
          }
          frags(smem + stn * STB, 0, af[cur ^ 1], bfr[cur ^ 1]);
          mma_range(cur, NQ / 2, NQ);
          if constexpr (SCHED == 1) {
            __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, (NQ - NQ / 2) * kMf, 0);
          }
        }
      }
      st = stn;
    }
    // ---- epilogue.  acc[fi][fj][4q+e] holds C[i][j] with
    //   i = ti*BM + wm*WTM + fi*32 + 8q + 4*half + e
    //   j = tj*BM + wn*WTN + fj*32 + lane%32
    // Each value is finished in registers.  Gram and polynomial tiles, and
    // the fp32 update, store row-major straight from the MFMA layout (32
    // lanes cover 32 consecutive columns of one row); the bf16 low part of X'
    // leaves in its own accumulator-order layout.  Everything else (X'^T, the
    // mirror tile of a symmetric product, the bf16 high part of X', the last
    // step's output) is staged per wave through LDS in 64-row halves,
    // column-major with a 68-float stride (conflict-free for the 16-byte
    // writes of 4 rows and the 16-byte reads of 8 rows), and leaves as 16-byte
    // pieces of 128-byte row segments.
    const int gi0 = ti * BM + wm * WTM;  // first row of this wave's sub-tile
    const int gj0 = tj * BN + wn * WTN;  // first column

    // split Gram: the tile stores its fp32 partial sums, unscaled and
    // unmirrored, into its slice; gram_reduce adds the slices, scales and mirrors
    const bool split = EPI == EPI_GRAM && G.splits > 1;
    if constexpr (EPI == EPI_GRAM) {  // A_0 = xs^2 N N^T (see xs above)
      const float xg = split ? 1.0f : scale_of();
      const float x2 = xg * xg;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= x2;
    }

    // 1. finish the values, one 32x32 block at a time, and store what leaves
    //    from registers.  The epilogue operand (X, or A for the polynomial)
    //    of the next PF blocks can be loaded ahead; PF = 0 measured best (more
    //    only adds register pressure).
    constexpr int NB = FM * FN;  // 32x32 blocks per wave
    constexpr int PF = 0;        // blocks loaded ahead (more only adds register pressure)
    constexpr bool kHasE = (EPI != EPI_GRAM);
    float ebuf[kHasE ? PF + 1 : 1][16];
    // bf16 update: the low part of X is kept in this kernel's accumulator
    // order (lo_index(), lo_exp_index()): a lane's 16 codes of a block are 16
    // contiguous bytes and its exponents of all NB blocks NB contiguous bytes,
    // so everything is loaded here in one round and the new low part leaves
    // the same way.
    constexpr bool kLoNative = (EPI == EPI_UPDATE || EPI == EPI_FINAL) && sizeof(T) == 2;
    static_assert(!kLoNative || (BN == BM && WGM == 2 && WGN == BM / 64 && WTN == 64 && NB % 4 == 0),
                  "the low part's layout assumes this tile shape (see lo_index)");
    uint4 lo_pre[kLoNative ? NB : 1];
    uint32_t lo_exp[kLoNative ? NB / 4 : 1];
    const uint32_t tile_wave = static_cast<uint32_t>(ti * G.tiles_n + tj) * NW + wave;
    const uint32_t lo_off = tile_wave * NB * 1024u + static_cast<uint32_t>(lane) * 16u;  // bytes, block 0
    const uint32_t lo_eoff = (tile_wave * 64u + static_cast<uint32_t>(lane)) * NB;
    if constexpr (kLoNative) {
      const char* El = G.E1 + mat * G.e1_mat;
#pragma unroll
      for (int b = 0; b < NB; ++b) lo_pre[b] = *reinterpret_cast<const uint4*>(El + lo_off + b * 1024u);
      const uint32_t* Ee = reinterpret_cast<const uint32_t*>(G.LoE + mat * G.loe_mat + lo_eoff);
#pragma unroll
      for (int k = 0; k < NB / 4; ++k) lo_exp[k] = Ee[k];
    }
    auto eload = [&](int blk, float* e) {
      const int fi = blk / FN, fj = blk % FN;
      const int j = j_base + fj * 32;
      if constexpr (EPI == EPI_POLY) {
        const char* Em = G.E0 + mat * G.e0_mat;
        const uint32_t lde = G.lde0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
          e[r] = Elem<T>::load(Em + (i * lde + j) * static_cast<uint32_t>(sizeof(T)));
        }
      } else if constexpr (EPI == EPI_UPDATE || EPI == EPI_FINAL) {
        // X: fp32, or bf16 high part + bf16 low part (per-matrix byte offsets fit in 32 bits)
        const char* Em = G.E0 + mat * G.e0_mat;
        const uint32_t lde = G.lde0;
        if constexpr (sizeof(T) == 2) {  // the high part was added in the main loop
          // the codes; their step is folded into the coefficient a below
          const uint32_t w[4] = {lo_pre[blk].x, lo_pre[blk].y, lo_pre[blk].z, lo_pre[blk].w};
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = lo8_code(w, r);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
            e[r] = *reinterpret_cast<const float*>(Em + (i * lde + j) * 4u);
          }
        }
      }
    };
    if constexpr (kHasE) {
      if (!poly_in_loop) {
#pragma unroll
        for (int b = 0; b < PF && b < NB; ++b) eload(b, ebuf[b]);
      }
    }
    uint32_t new_exp[kLoNative ? NB / 4 : 1];
    uint32_t hiw[kXPF ? NB : 1][8];  // bf16 update: the high part of X', pairs of rows
#pragma unroll
    for (int k = 0; k < (kLoNative ? NB / 4 : 1); ++k) new_exp[k] = 0;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int fi = blk / FN, fj = blk % FN;
      const int j = j_base + fj * 32;
      if constexpr (kHasE) {
        if (blk + PF < NB && !poly_in_loop) eload(blk + PF, ebuf[(blk + PF) % (PF + 1)]);
        const float* e = ebuf[blk % (PF + 1)];
        if constexpr (EPI == EPI_POLY) {
          if (poly_in_loop) {  // b/c * A is already in the accumulator
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fi][fj][r] = ct * acc[fi][fj][r];
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fi][fj][r] = bt * e[r] + ct * acc[fi][fj][r];
          }
        } else {
          // a * Xlo: with bf16 compute e holds the low part's codes, and
          // a * step is exact (a power-of-two step)
          float ae = at;
          if constexpr (kLoNative) ae = at * lo8_step((lo_exp[blk >> 2] >> (8 * (blk & 3))) & 0xffu);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[fi][fj][r] = ae * e[r] + acc[fi][fj][r];
        }
      }
      if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) {
        const uint32_t ldo = G.ldo0;
        if (split) {  // (a slice holds at most 3840^2 floats: 32-bit offsets)
          char* Pm = reinterpret_cast<char*>(G.part) + mat * G.part_mat +
                     static_cast<int64_t>(slice) * ldo * ldo * static_cast<int64_t>(sizeof(float));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
            *reinterpret_cast<float*>(Pm + (i * ldo + j) * 4u) = acc[fi][fj][r];
          }
        } else {
          char* Om = G.O0 + mat * G.o0_mat;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
            Elem<T>::store(Om + (i * ldo + j) * static_cast<uint32_t>(sizeof(T)), acc[fi][fj][r]);
          }
        }
      } else if constexpr (EPI == EPI_UPDATE) {
        char* O0m = G.O0 + mat * G.o0_mat;  // X' (fp32) or its bf16 low part
        const uint32_t ldo0 = G.ldo0;
        if constexpr (sizeof(T) == 2) {
          // the high part leaves from the LDS staging below, as row segments;
          // the low part's codes here, its exponents after the last block
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = acc[fi][fj][r];
          const Lo8 c = lo8_encode(x, kXPF ? hiw[blk] : nullptr);
          *reinterpret_cast<uint4*>(O0m + lo_off + blk * 1024u) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
          new_exp[blk >> 2] |= c.e << (8 * (blk & 3));
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
            *reinterpret_cast<float*>(O0m + (i * ldo0 + j) * 4u) = acc[fi][fj][r];
          }
        }
      } else if constexpr (sizeof(T) == 4) {  // EPI_FINAL, fp32 compute: caller output in the NS orientation
        if (!G.tall) {
          char* U = user_ptr(G.user, mat);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = i_base + fi * 32 + 8 * (r >> 2) + (r & 3);
            if (i >= G.ms || j >= G.ns) continue;
            if constexpr (AP) {
              apply_user(G.user, U, i, j, acc[fi][fj][r], G.ap_decay, G.ap_step);
            } else {
              store_user(G.user, U, i, j, acc[fi][fj][r]);
            }
          }
        }
      }  // EPI_FINAL, bf16 compute: the caller's output leaves from the LDS staging below
    }
    if constexpr (kLoNative && EPI == EPI_UPDATE) {
      uint32_t* Eo = reinterpret_cast<uint32_t*>(G.LoE + mat * G.loe_mat + lo_eoff);  // in place
#pragma unroll
      for (int k = 0; k < NB / 4; ++k) Eo[k] = new_exp[k];
    }

    if constexpr (kXPF) {
      // The next tile of this workgroup, if it is in the same group (same
      // operand strides): its first k-tile goes into stage 0 now, under this
      // epilogue's stores.  No wave reads stage 0 any more: the last k-tile's
      // barrier retired every read that matters (what follows it only
      // prefetches fragments that are never used).  Issued after the last
      // load this epilogue waits for: the compiler's counted waits do not see
      // these copies, and vector memory operations complete in issue order.
      const int tn = t + static_cast<int>(gridDim.x);
      if (tn < L.total_tiles) {
        int gn, mn, sn, tin, tjn;
        decode(tn, gn, mn, sn, tin, tjn);
        if (gn == gi) {
          dma_issue_at(G.P + mn * G.p_mat + static_cast<int64_t>(tin) * BM * ldp * sizeof(T),
                       G.Q + mn * G.q_mat + static_cast<int64_t>(tjn) * BN * sizeof(T), 0, 0);
          pf = true;
        }
      }
    }

    // 3. transposed stores through LDS
    bool transposed;
    if constexpr (EPI == EPI_UPDATE) {
      transposed = true;
    } else if constexpr (EPI == EPI_FINAL) {
      transposed = sizeof(T) == 2 || G.tall != 0;  // bf16: staged either way (row or column segments)
    } else {
      transposed = !split && tj >= R * (ti + 1);  // the mirror of a tile off the diagonal block
    }
    if (!transposed) continue;  // uniform over the workgroup
    static_assert(WTN == 64 && WTM % 64 == 0, "transposed staging works on 64 x 64 wave blocks");
    constexpr int ES = 68;  // floats per staged column
    // every wave is done with the operand stages.  The bf16 update needs no
    // barrier here: each wave stages into its own part of the ring above
    // stage 0, and after the last k-tile's barrier the other waves read only
    // fragments they never use (the next tile's copy is in stage 0).
    if constexpr (!kXPF) __syncthreads();
    float* wl = reinterpret_cast<float*>(smem) + wave * 64 * ES;
    constexpr int ES2 = 68;  // bf16 update: bf16 values per staged column
    char* wl2 = smem + STB + wave * 64 * ES2 * 2;
    static_assert(!kXPF || STB + NW * 64 * ES2 * 2 <= SMEM, "bf16 staging above stage 0");
    char* OTm;
    int64_t ldot;
    if constexpr (EPI == EPI_UPDATE) {
      OTm = G.OT + mat * G.ot_mat;
      ldot = G.ldot;
    } else if constexpr (EPI == EPI_FINAL) {
      OTm = user_ptr(G.user, mat);
      ldot = G.user.ld;
    } else {
      OTm = G.O0 + mat * G.o0_mat;
      ldot = G.ldo0;
    }
#pragma unroll
    for (int h = 0; h < WTM / 64; ++h) {
      if constexpr (kXPF) {
        // the high part of X', already bf16 (from the encoder): column-major
        // in LDS, 4 rows of one column per 8-byte write, then read back as
        // 4-row x 8-column pieces and stored as 16-byte row segments.  A
        // half-wave reads columns c and c + 16 (68-element columns put them
        // 32 banks apart); its writes cover the 64 banks once.
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int fj = 0; fj < FN; ++fj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int blk = (2 * h + f) * FN + fj;
              *reinterpret_cast<u32x2_t*>(wl2 + ((fj * 32 + frow) * ES2 + f * 32 + 8 * q + 4 * half) * 2) =
                  u32x2_t{hiw[blk][2 * q], hiw[blk][2 * q + 1]};
            }
        char* O1m = G.O1 + mat * G.o1_mat;
        const uint32_t ldo1 = G.ldo1;
        const int rg = lane & 15;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int c0 = 8 * it + 16 * ((lane >> 4) & 1) + 32 * (lane >> 5);
          u32x2_t x[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = *reinterpret_cast<const u32x2_t*>(wl2 + ((c0 + t) * ES2 + 4 * rg) * 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t a = e < 2 ? x[2 * k].x : x[2 * k].y, b = e < 2 ? x[2 * k + 1].x : x[2 * k + 1].y;
              w[k] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            const uint32_t row = gi0 + h * 64 + 4 * rg + e;
            *reinterpret_cast<uint4*>(O1m + (row * ldo1 + gj0 + c0) * 2u) = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      } else {
      // registers -> LDS column-major: 4 consecutive rows of one column per write
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = f * 32 + 8 * q + 4 * half;
            const int c = fj * 32 + frow;
            const int fi = 2 * h + f;
            *reinterpret_cast<float4*>(wl + c * ES + r) =
                make_float4(acc[fi][fj][4 * q], acc[fi][fj][4 * q + 1], acc[fi][fj][4 * q + 2], acc[fi][fj][4 * q + 3]);
          }
      }
      if constexpr (EPI == EPI_UPDATE && sizeof(T) == 2 && !kXPF) {
        // the high part of X' row-major: lanes read 4-row x 8-column pieces of
        // the staged half (16 lanes cover 256 consecutive bytes of LDS) and
        // store 16-byte row segments
        char* O1m = G.O1 + mat * G.o1_mat;
        const uint32_t ldo1 = G.ldo1;
        const int rg = lane & 15;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int c0 = 8 * (lane >> 4) + 32 * it;
          float4 x[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = *reinterpret_cast<const float4*>(wl + (c0 + t) * ES + 4 * rg);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = e == 0 ? x[t].x : e == 1 ? x[t].y : e == 2 ? x[t].z : x[t].w;
            const uint32_t row = gi0 + h * 64 + 4 * rg + e;
            Elem<T>::store8(O1m + (row * ldo1 + gj0 + c0) * 2u, make_float4(v[0], v[1], v[2], v[3]),
                            make_float4(v[4], v[5], v[6], v[7]));
          }
        }
      }
      if constexpr (EPI == EPI_FINAL) {
        // the caller's output: 8-element segments, 16-byte (bf16) or 32-byte
        // (fp32) stores where a segment is whole and the rows are 16-byte
        // aligned, element by element at the ragged edges
        const int es = G.user.dtype ? 2 : 4;
        const bool vec = ((reinterpret_cast<uintptr_t>(OTm) | static_cast<uintptr_t>(ldot * es)) & 15) == 0;
        auto put8 = [&](int orow, int ocol, int rows, int cols, const float4& x0, const float4& x1) {
          if (orow >= rows) return;
          if (vec && ocol + 8 <= cols) {
            char* p = OTm + (static_cast<int64_t>(orow) * ldot + ocol) * es;
            if constexpr (AP) {
              apply8(p, G.user.dtype, G.ap_decay, G.ap_step, x0, x1);
            } else if (G.user.dtype) {
              Elem<uint16_t>::store8(p, x0, x1);
            } else {
              Elem<float>::store8(p, x0, x1);
            }
          } else {
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (ocol + e >= cols) continue;
              if constexpr (AP) {
                apply_user(G.user, OTm, orow, ocol + e, xv[e], G.ap_decay, G.ap_step);
              } else {
                store_user(G.user, OTm, orow, ocol + e, xv[e]);
              }
            }
          }
        };
        // bf16 weights in 16-byte segments and the wave's staged 64 x 64
        // block inside the matrix (no bounds checks): each segment's old
        // weights are loaded one segment ahead, so that a load is in flight
        // while the previous segment is computed and stored.  (put8 below
        // loads and stores one segment after the other: the compiler cannot
        // move a load above the previous segment's store to the same array.)
        const bool wpipe = AP && G.user.dtype && vec && gi0 + h * 64 + 64 <= G.ms && gj0 + 64 <= G.ns;
        auto wl16 = [&](int orow, int ocol) {
          return *reinterpret_cast<const uint4*>(OTm + (static_cast<int64_t>(orow) * ldot + ocol) * 2);
        };
        auto wput16 = [&](int orow, int ocol, const uint4& wq, const float4& x0, const float4& x1) {
          const uint32_t q[4] = {wq.x, wq.y, wq.z, wq.w};
          const float o[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          float w[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            w[2 * k] = bf16_to_f32(static_cast<uint16_t>(q[k]));
            w[2 * k + 1] = bf16_to_f32(static_cast<uint16_t>(q[k] >> 16));
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = G.ap_decay * w[e] - G.ap_step * o[e];
          Elem<uint16_t>::store8(OTm + (static_cast<int64_t>(orow) * ldot + ocol) * 2,
                                 make_float4(w[0], w[1], w[2], w[3]), make_float4(w[4], w[5], w[6], w[7]));
        };
        if (wpipe && !G.tall) {
          const int rg = lane & 15;
          uint4 wa = wl16(gi0 + h * 64 + 4 * rg, gj0 + 8 * (lane >> 4)), wb = wa;
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const int c0 = 8 * (lane >> 4) + 32 * it;
            float4 x[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = *reinterpret_cast<const float4*>(wl + (c0 + t) * ES + 4 * rg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int sn = 4 * it + e + 1;
              if (sn < 8) wb = wl16(gi0 + h * 64 + 4 * rg + (sn & 3), gj0 + 8 * (lane >> 4) + 32 * (sn >> 2));
              float v[8];
#pragma unroll
              for (int t = 0; t < 8; ++t) v[t] = e == 0 ? x[t].x : e == 1 ? x[t].y : e == 2 ? x[t].z : x[t].w;
              wput16(gi0 + h * 64 + 4 * rg + e, gj0 + c0, wa, make_float4(v[0], v[1], v[2], v[3]),
                     make_float4(v[4], v[5], v[6], v[7]));
              wa = wb;
            }
          }
        } else if (wpipe) {
          const int rc = (lane & 7) * 8;
          uint4 wa = wl16(gj0 + (lane >> 3), gi0 + h * 64 + rc), wb = wa;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (k + 1 < 8) wb = wl16(gj0 + (lane >> 3) + 8 * (k + 1), gi0 + h * 64 + rc);
            const int c = (lane >> 3) + 8 * k;
            const float4 x0 = *reinterpret_cast<const float4*>(wl + c * ES + rc);
            const float4 x1 = *reinterpret_cast<const float4*>(wl + c * ES + rc + 4);
            wput16(gj0 + c, gi0 + h * 64 + rc, wa, x0, x1);
            wa = wb;
          }
        } else if (!G.tall) {
          // rows of X are rows of the output: 4-row x 8-column pieces
          const int rg = lane & 15;
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const int c0 = 8 * (lane >> 4) + 32 * it;
            float4 x[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] = *reinterpret_cast<const float4*>(wl + (c0 + t) * ES + 4 * rg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v[8];
#pragma unroll
              for (int t = 0; t < 8; ++t) v[t] = e == 0 ? x[t].x : e == 1 ? x[t].y : e == 2 ? x[t].z : x[t].w;
              put8(gi0 + h * 64 + 4 * rg + e, gj0 + c0, G.ms, G.ns, make_float4(v[0], v[1], v[2], v[3]),
                   make_float4(v[4], v[5], v[6], v[7]));
            }
          }
        } else {
          // columns of X are rows of the output: 8 lanes per 64-element row segment
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int c = (lane >> 3) + 8 * k;
            const int rc = (lane & 7) * 8;
            const float4 x0 = *reinterpret_cast<const float4*>(wl + c * ES + rc);
            const float4 x1 = *reinterpret_cast<const float4*>(wl + c * ES + rc + 4);
            put8(gj0 + c, gi0 + h * 64 + rc, G.ns, G.ms, x0, x1);
          }
        }
      } else if constexpr (!kQN) {  // the bf16 update writes no X'^T
        // LDS -> global: 8 lanes write one 8 x 8-element row segment of the output
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = (lane >> 3) + 8 * k;
          const int rc = (lane & 7) * 8;
          const float4 x0 = *reinterpret_cast<const float4*>(wl + c * ES + rc);
          const float4 x1 = *reinterpret_cast<const float4*>(wl + c * ES + rc + 4);
          const int orow = gj0 + c;            // output row = this tile's column
          const int ocol = gi0 + h * 64 + rc;  // output column = this tile's row
          Elem<T>::store8(OTm + (static_cast<uint32_t>(orow) * static_cast<uint32_t>(ldot) + ocol) *
                                    static_cast<uint32_t>(sizeof(T)), x0, x1);
        }
      }
    }
  }  // tiles
}

// Workgroups of a tile size that are resident on the current device at once
// (one 256-tile or two 128-tile workgroups per CU: LDS bound), rounded down
// to a multiple of the 8 XCDs; 0 if the device cannot be queried.
int resident_workgroups(int tile) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return (cus[dev] * (tile == 256 ? 1 : 2)) & ~7;
}

// Launches with many tiles per resident workgroup run on a persistent grid
// (each workgroup takes tiles t, t + grid, ... of the longest-first order,
// which keeps the rounds balanced and saves a workgroup launch and retire
// per tile); short launches keep one workgroup per tile, so the hardware's
// dynamic dispatch balances tiles of unequal cost.
// Chosen by measurement on MI355X over the 8B-dense matrix shapes: 64-element
// k-tiles moved by LDS DMA through a two-stage ring, the 64-bank swizzle,
// XCD-contiguous tile ranges and groups of four tile rows for the
// non-symmetric product.
template <typename T, int BM, int WGM, int WGN, int EPI, int QN = 0, int AP = 0>
void launch_one(const GemmLaunch& L, hipStream_t stream) {
  constexpr int RC = 8, STAGES = 2, SWZ = 1, DMA = 1, XCD = 1, SCHED = 0, GM = 4;
  const int cap = resident_workgroups(BM);
  const int grid = (cap >= 8 && L.total_tiles >= 4 * cap) ? cap : L.total_tiles;
  hipLaunchKernelGGL((ns_gemm_kernel<T, BM, WGM, WGN, EPI, RC, STAGES, SWZ, DMA, XCD, SCHED, GM, BM, QN, AP>),
                     dim3(grid), dim3(64 * WGM * WGN), 0, stream, L);
}

template <typename T, int BM, int WGM, int WGN>
hipError_t launch_t(int epi, const GemmLaunch& L, hipStream_t stream) {
  switch (epi) {
    case EPI_GRAM: launch_one<T, BM, WGM, WGN, EPI_GRAM>(L, stream); break;
    case EPI_POLY: launch_one<T, BM, WGM, WGN, EPI_POLY>(L, stream); break;
    // the bf16 update reads X k-major, the fp32 update X^T
    case EPI_UPDATE: launch_one<T, BM, WGM, WGN, EPI_UPDATE, sizeof(T) == 2>(L, stream); break;
    default:  // the last step writes O, or (ap) applies the update to W
      if (L.g[0].ap) {
        launch_one<T, BM, WGM, WGN, EPI_FINAL, sizeof(T) == 2, 1>(L, stream);
      } else {
        launch_one<T, BM, WGM, WGN, EPI_FINAL, sizeof(T) == 2>(L, stream);
      }
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_gemm(int compute, int tile, int epi, bool kmajor, const GemmLaunch& L, hipStream_t stream) {
  if (L.total_tiles <= 0) return hipSuccess;
  // the update's second operand: X k-major with bf16 compute, X^T with fp32
  if ((epi == EPI_UPDATE || epi == EPI_FINAL) && kmajor != (compute == 1)) return hipErrorInvalidValue;
  if (compute == 1) {
    return tile == 256 ? launch_t<uint16_t, 256, 2, 4>(epi, L, stream) : launch_t<uint16_t, 128, 2, 2>(epi, L, stream);
  }
  return tile == 256 ? launch_t<float, 256, 2, 4>(epi, L, stream) : launch_t<float, 128, 2, 2>(epi, L, stream);
}

}  // namespace muon
