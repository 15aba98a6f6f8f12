// Internal declarations shared by the libmuon355 kernels and its C-ABI layer.
// Nothing here is part of the public interface (include/muon355.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace muon {

constexpr int kMaxGroups = 8;

// One batch of same-shape matrices in device memory, as seen by a kernel.
struct MatBatch {
  char* base;            // matrix i at base + i*stride_bytes when ptrs == nullptr
  int64_t stride_bytes;
  void* const* ptrs;     // device array of per-matrix pointers, or nullptr
  int64_t ld;            // leading dimension in elements
  int32_t dtype;         // 0 = f32, 1 = bf16
  int32_t pad_;
};

// Fast unsigned 32-bit division by a runtime-constant divisor
// (round-up multiply-high method of Granlund and Montgomery).
struct FastDiv {
  uint32_t d, m, l;
};
FastDiv make_fastdiv(uint32_t d);

// ---------------------------------------------------------------- GEMM stage

enum Epi : int { EPI_GRAM = 0, EPI_POLY = 1, EPI_UPDATE = 2, EPI_FINAL = 3 };

// One group of same-shape products C = P * Q^T with the stage's epilogue.
// P has rows i contiguous along the reduction index k; Q has rows j
// contiguous along k, except in the bf16 update and last step, where Q is X
// itself stored k-major (row k, columns j contiguous; ldq is its row pitch).
struct GemmGroup {
  const char* P; int64_t p_mat;  // bytes between matrices
  const char* Q; int64_t q_mat;
  int32_t ldp, ldq;              // elements
  int32_t K;                     // reduction length, a multiple of the k-tile
  int32_t tiles_m, tiles_n;      // tile grid of one matrix
  int32_t sym;                   // 1: only tiles with ti <= tj, mirrored on store
  int32_t count;
  int32_t tiles_per_mat;
  int32_t tile_begin;            // first linear tile of this group in the launch
  // epilogue operands (row-major, i x j orientation unless noted)
  // X itself is held as fp32 (fp32 compute) or, with bf16 compute, as a
  // bf16 high part (the MFMA operand) plus a bf16 low part (the rounding
  // residual), about 16 significant bits together.
  const char* E0; int64_t e0_mat; int32_t lde0;  // POLY: A; UPDATE/FINAL, fp32 compute: X
  int32_t pad0_;
  const char* E1; int64_t e1_mat; int32_t lde1;  // UPDATE/FINAL, bf16 compute: low part of X, int8
                                                 // codes in the lo_index() layout (the high part is
                                                 // Q, added from the operand tiles)
  int32_t pad5_;
  uint8_t* LoE; int64_t loe_mat;                 // ... and its exponents (lo_exp_index()), read and
                                                 // rewritten in place by the update
  char* O0; int64_t o0_mat; int32_t ldo0;        // GRAM/POLY: A or B; UPDATE: next X (fp32) or its low
                                                 // part's codes (lo_index() layout, in place)
  int32_t pad1_;
  char* O1; int64_t o1_mat; int32_t ldo1;        // UPDATE, bf16 compute: high part of the next X
  int32_t pad2_;
  char* OT; int64_t ot_mat; int32_t ldot;        // UPDATE, fp32 compute: X^T (next)
  int32_t pad3_;
  // FINAL: the caller's output in its stored orientation
  MatBatch user;
  int32_t tall;                  // 1: user output is X^T
  int32_t ms, ns;                // true (unpadded) Newton-Schulz shape
  // FINAL with the parameter update folded in (ap = 1): `user` is the weight
  // W, and the epilogue writes W <- ap_decay * W - ap_step * O in place of O
  int32_t ap;
  float ap_decay, ap_step;
  int32_t pad7_;
  // Step 0 from an unnormalized packed input (the momentum kernel wrote
  // N itself): with xs = 1/(sqrt(xs_sumsq[mat]) + xs_eps), the Gram's
  // products are multiplied by xs^2, the polynomial uses xs*b and xs*c and
  // the update xs*a; null: xs = 1.
  float xs_eps;
  const float* xs_sumsq;
  // Gram with the reduction split in `splits` slices (1: not split): each
  // tile of each slice stores its fp32 partial sums, unscaled and not
  // mirrored, at part + mat*part_mat + slice*ldo0*ldo0*4 (row-major, ldo0 =
  // the padded order), and gram_reduce adds the slices.
  int32_t splits;
  int32_t pad6_;
  float* part; int64_t part_mat;  // bytes per matrix
};

// A = scale * (sum over the slices of the split Gram's partials), for every
// element of the padded order-Mp matrices of up to kMaxGroups groups; an
// element below the diagonal tile row reads the mirrored partial (only tiles
// with ti <= tj were computed).  scale = xs^2 of step 0 of the packed input,
// else 1.  Workgroup b of the flat grid handles 1024 elements of group g
// (first[g] <= b < first[g+1]).
struct GramReduceGroup {
  const float* part; int64_t part_mat;  // bytes per matrix
  char* A; int64_t a_mat;               // bytes per matrix; row-major, ld Mp
  const float* xs_sumsq;                // null: scale 1
  float xs_eps;
  int32_t Mp, tile, splits, compute;
  int32_t pad_;
};
struct GramReduce {
  int32_t ngroups;
  int32_t pad_;
  int64_t first[kMaxGroups + 1];
  GramReduceGroup g[kMaxGroups];
};
hipError_t launch_gram_reduce(const GramReduce& a, hipStream_t stream);

// The low part of X (bf16 compute): the residual X - bf16(X), kept as int8
// codes in multiples of a step shared by the 16 values one lane holds in one
// 32x32 MFMA block.  step = 2^(E - 142), with E the biased exponent of the
// largest |bf16(X)| of those 16: 1/256 of that value's bf16 spacing, so
// every residual (at most half a spacing) is a code in [-127, 127]; E < 16
// (values below 2^-111) keeps a zero residual.  With the high part that is
// about 16 significant bits (device helpers in lo8.h).  Only the update
// kernel reads and writes it (plus the pack kernel, which writes its first
// value), so it is kept in the update kernel's accumulator order: a bm x bm
// output tile is split over 2 x (bm/64) waves of (bm/2) x 64 elements, each
// wave's sub-tile into 32x32 MFMA blocks, and each block into 64 lanes x 16
// values (lane = 32*half + column, value r <-> row 8*(r/4) + 4*half + r%4).
// One lane's 16 codes of a block are 16 contiguous bytes; the code of element
// (i, j) of the padded Newton-Schulz matrix with `tiles_n` tile columns is
// at byte:
__host__ __device__ inline uint32_t lo_index(uint32_t i, uint32_t j, uint32_t bm, uint32_t tiles_n) {
  const uint32_t wgn = bm / 64, wtm = bm / 2, nb = (wtm / 32) * 2;
  const uint32_t ti = i / bm, tj = j / bm, il = i % bm, jl = j % bm;
  const uint32_t wave = (il / wtm) * wgn + jl / 64;
  const uint32_t ii = il % wtm, jj = jl % 64;
  const uint32_t blk = (ii / 32) * 2 + jj / 32;
  const uint32_t rb = ii % 32;
  const uint32_t lane = ((rb % 8) / 4) * 32 + jj % 32;
  const uint32_t r = 4 * (rb / 8) + rb % 4;
  return (((ti * tiles_n + tj) * (2 * wgn) + wave) * nb + blk) * 1024u + lane * 16u + r;
}

// One exponent byte per lane and block, a lane's exponents of all its
// blocks contiguous (one 8- or 4-byte access); the exponent that element
// (i, j)'s code uses is at byte:
__host__ __device__ inline uint32_t lo_exp_index(uint32_t i, uint32_t j, uint32_t bm, uint32_t tiles_n) {
  const uint32_t wgn = bm / 64, wtm = bm / 2, nb = (wtm / 32) * 2;
  const uint32_t ti = i / bm, tj = j / bm, il = i % bm, jl = j % bm;
  const uint32_t wave = (il / wtm) * wgn + jl / 64;
  const uint32_t ii = il % wtm, jj = jl % 64;
  const uint32_t blk = (ii / 32) * 2 + jj / 32;
  const uint32_t lane = (((ii % 32) % 8) / 4) * 32 + jj % 32;
  return (((ti * tiles_n + tj) * (2 * wgn) + wave) * 64u + lane) * nb + blk;
}

// Bytes of the low part per element of the padded matrix: one code, and one
// exponent per 16 codes.
constexpr int kLoExpPerCodes = 16;

struct GemmLaunch {
  int32_t ngroups;
  int32_t total_tiles;
  float a, b, c;
  int32_t pad_;
  GemmGroup g[kMaxGroups];
};

// Launch one stage for all groups (all with the same tile size `tile`).
// compute: 0 = f32, 1 = bf16.  kmajor (bf16 update and last step only): the
// second operand of every group is X itself, k-major; otherwise X^T.
hipError_t launch_ns_gemm(int compute, int tile, int epi, bool kmajor, const GemmLaunch& L,
                          hipStream_t stream);

// ------------------------------------------------------------ elementwise

struct MomentumArgs {
  MatBatch G, M, N;      // N.base == nullptr && N.ptrs == nullptr: N is M
  float* partials;       // [count * blocks_per_mat]
  int32_t blocks_per_mat;
  int32_t rows, cols;
  FastDiv cdiv;          // division by cols
  float beta;
  int32_t nesterov;
  int32_t has_n;
};
hipError_t launch_momentum(const MomentumArgs& a, int64_t count, bool vec,
                           hipStream_t stream);

struct SumsqArgs {
  MatBatch X;
  float* partials;
  int32_t blocks_per_mat;
  int32_t rows, cols;
  FastDiv cdiv;
};
hipError_t launch_sumsq_partials(const SumsqArgs& a, int64_t count, bool vec,
                                 hipStream_t stream);

// sumsq[i] = sum of partials[i*per .. i*per+per) in fp64, fixed order.
hipError_t launch_sumsq_finalize(const float* partials, int per, float* sumsq,
                                 int64_t count, hipStream_t stream);

struct ApplyArgs {
  MatBatch W, O;
  int32_t rows, cols;
  FastDiv cdiv;
  float decay;           // 1 - lr*wd
  float step;            // lr * s
};
hipError_t launch_apply(const ApplyArgs& a, int64_t count, bool vec,
                        hipStream_t stream);

// Several groups (shape classes) in one launch over a flat grid: workgroup b
// belongs to the group g with first[g] <= b < first[g+1]; inside it, the
// momentum and apply kernels take block (b - first[g]) % blocks_per_mat of
// matrix (b - first[g]) / blocks_per_mat, and the finalize kernel matrix
// b - first[g].  vec[g]: the group's rows allow 16-byte accesses.
struct MomentumGroups {
  int32_t ngroups;
  int32_t vec[kMaxGroups];
  int32_t pad_;
  int64_t first[kMaxGroups + 1];
  MomentumArgs g[kMaxGroups];
};
hipError_t launch_momentum_grouped(const MomentumGroups& a, hipStream_t stream);

// The static device scratch array of the allocation-free entry point on the
// current device: its address (looked up once per device) and size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

struct FinalizeGroups {
  int32_t ngroups;
  int32_t per[kMaxGroups];  // partials per matrix
  int32_t pad_;
  int64_t first[kMaxGroups + 1];
  const float* partials[kMaxGroups];
  float* sumsq[kMaxGroups];
};
hipError_t launch_sumsq_finalize_grouped(const FinalizeGroups& a, hipStream_t stream);

struct ApplyGroups {
  int32_t ngroups;
  int32_t vec[kMaxGroups];
  int32_t blocks_per_mat[kMaxGroups];
  int32_t pad_;
  int64_t first[kMaxGroups + 1];
  ApplyArgs g[kMaxGroups];
};
hipError_t launch_apply_grouped(const ApplyGroups& a, hipStream_t stream);

// Copy the caller's N (stored m x n) into the padded Newton-Schulz buffers,
// scaled by 1/(sqrt(sumsq)+eps):  S[r][c] (stored orientation, Pr x Pc)
// and/or T[c][r] (Pc x Pr), each written when non-null, zero outside m x n,
// in the compute type; with bf16 compute and Lo != null also the low part of
// X (= S if !tall, T if tall): codes and exponents of value - bf16(value).
struct PackArgs {
  MatBatch N;
  const float* sumsq;
  float eps;
  int32_t rows, cols;      // m, n
  int32_t Pr, Pc;          // padded
  int32_t compute;         // element type of S and T
  int32_t tall;
  int32_t nvec;            // N's rows and matrices start on 4-element boundaries (aligned)
  int32_t pad_;
  char* S; int64_t s_mat;  // stored orientation (bytes per matrix); null: not written
  char* T; int64_t t_mat;  // its transpose; null: not written
  int8_t* Lo; int64_t lo_mat;     // low part's codes (lo_index()), bytes per matrix
  uint8_t* LoE; int64_t loe_mat;  // and exponents (lo_exp_index()), bytes per matrix
  int32_t lo_bm, lo_tiles_n;      // update tile size and tile columns of X
};
hipError_t launch_pack(const PackArgs& a, int64_t count, hipStream_t stream);

// Momentum fused with the packing of the Newton-Schulz input: per 64x64
// tile of the padded stored extent of one matrix, M <- beta*M + (1-beta)*G,
// the Nesterov blend N (the same arithmetic as momentum_kernel), one partial
// sum of N^2 per tile, and N itself (not yet normalized) into the padded
// buffers as PackArgs describes them (S, T, Lo, LoE).
struct MomentumPackArgs {
  MatBatch G, M;
  float beta;
  int32_t nesterov;
  int32_t rows, cols;      // stored m, n
  int32_t Pr, Pc;          // padded
  int32_t compute, tall;
  int32_t vec;             // G's and M's rows and matrices start on 4-element boundaries
  int32_t tiles_c;         // Pc / 64
  int32_t tiles_per_mat;   // (Pr / 64) * (Pc / 64)
  int32_t lo_bm, lo_tiles_n;
  int32_t pad_;
  float* partials;         // [count * tiles_per_mat]
  char* S; int64_t s_mat;
  char* T; int64_t t_mat;
  int8_t* Lo; int64_t lo_mat;
  uint8_t* LoE; int64_t loe_mat;
};
struct MomentumPackGroups {
  int32_t ngroups;
  int32_t pad_;
  int64_t first[kMaxGroups + 1];  // first workgroup of each group (one per tile)
  MomentumPackArgs g[kMaxGroups];
};
hipError_t launch_momentum_pack_grouped(const MomentumPackGroups& a, hipStream_t stream);

// Zero-step output: out = N / (sqrt(sumsq) + eps), both in the stored
// orientation.
struct CopyOutArgs {
  MatBatch N;
  const float* sumsq;
  float eps;
  MatBatch out;
  int32_t rows, cols;      // stored m, n
};
hipError_t launch_copy_out(const CopyOutArgs& a, int64_t count, hipStream_t stream);

// ------------------------------------------------------------ AdamW

constexpr int64_t kAdamWChunk = 4096;  // elements per workgroup; MUON_ADAMW_CHUNK

struct AdamWArgs {
  int64_t count;                  // tensors
  void* const* params;            // device arrays of `count` pointers
  const void* const* grads;
  float* const* exp_avg;
  float* const* exp_avg_sq;
  const int64_t* numels;          // device [count]
  const int64_t* chunk_offsets;   // device [count + 1]
  int32_t param_bf16, grad_bf16;
  float beta1, beta2, eps;
  float c1, c2;                   // 1/(1-beta1^t), 1/(1-beta2^t)
  float lr, decay;                // decay = 1 - lr*wd
};
hipError_t launch_adamw(const AdamWArgs& a, int64_t total_chunks, hipStream_t stream);

// ------------------------------------------------------------ SOAP

// One operand of the fp32 product C = alpha*op(A)*op(B) + beta*C, as the
// kernel reads it: batch entry b starts at (ptrs ? ptrs[b] : base + b*stride)
// + off.  kcontig: the reduction index is the contiguous one in memory (A
// stored M x K, or B stored N x K); otherwise the outer index is (A stored
// K x M, B stored K x N).  vec: every 4-element run along the contiguous
// index that starts on a multiple of 4 is aligned for one vector load.
struct SgemmOperand {
  const char* base;
  int64_t stride;          // bytes between batch entries
  const void* const* ptrs;
  int64_t off;             // bytes
  int64_t ld;              // elements
  int32_t dtype;           // 0 = f32, 1 = bf16
  int32_t kcontig;
  int32_t vec;
  int32_t pad_;
};

// C is fp32.  With splits > 1, split s of batch entry b sums the reduction
// range [s*ksplit, min(K, (s+1)*ksplit)) into C_b + s*c_split (beta = 0).
// sym: op(A)*op(B) is symmetric (M == N); only tiles ti <= tj are computed
// and each value is stored at (i, j) and (j, i), so C stays exactly
// symmetric (and beta*C reads only the upper triangle).
struct SgemmArgs {
  SgemmOperand a, b;
  char* c;
  int64_t c_stride;
  void* const* c_ptrs;
  int64_t c_off;
  int64_t ldc;
  int64_t c_split;
  int32_t M, N, K, ksplit;
  int32_t splits, count;
  float alpha, beta;
  int32_t sym;
  int32_t pad_;
};
constexpr int kSgemmTile = 128;
constexpr int kSgemmBK = 32;
hipError_t launch_sgemm(const SgemmArgs& a, hipStream_t stream);

// Up to kSgemmMaxList products in one launch; tile_end[p] = the workgroups of
// products 0..p (each: tiles of one matrix x count x splits).
constexpr int kSgemmMaxList = 8;
struct SgemmList {
  SgemmArgs g[kSgemmMaxList];
  int32_t tile_end[kSgemmMaxList];
  int32_t n;
  int32_t pad_;
};
// Enqueues n (at most 2 * kSgemmMaxList) independent products; the result of
// each is what launch_sgemm gives for it, bit for bit.
hipError_t launch_sgemm_list(const SgemmArgs* gs, int n, hipStream_t stream);

// Householder QR, one 16-column panel of `count` n x n matrices (row-major,
// ld n): columns c0 .. c0+nb-1 (nb = min(16, n - c0)), rows c0 .. n-1, of A
// (read only) are reduced in the panel's slot of the reflector buffer,
// column-major with absolute rows: V points at row c0 of the slot's first
// column (column q at V + q*n, row c0 + r at offset r), and the zpre rows
// above it (up to the enclosing outer block's first row) are zeroed.  The
// slot ends holding the explicit reflectors (unit diagonal, zeros above
// it); tau[c0 + j] gets each reflector's factor and sgn[c0 + j] the sign of
// R's diagonal entry (+1 for zero).  The block factor T of
// H_c0 ... H_(c0+nb-1) = I - V T V^T (nb x nb, upper triangular) is written
// repeated side by side for the split-K products: TrepT (nb x nb*reps_t,
// row-major) holds [T^T ... T^T], TrepQ (nb x nb*reps_q) holds [T ... T]
// (reps_q may be 0).
constexpr int kQrPanel = 16;
constexpr int kQrOuter = 128;   // outer block: the trailing matrix is updated once per 128 columns
struct QrPanelArgs {
  const float* A; int64_t a_mat;  // floats per matrix
  float* V; int64_t v_mat;
  float* TrepT; int64_t tT_mat;
  float* TrepQ; int64_t tQ_mat;
  float* sgn; float* tau; int64_t s_mat;
  int32_t n, c0, reps_t, reps_q;
  int32_t zpre;
  int32_t pad_;
};
hipError_t launch_qr_panel(const QrPanelArgs& a, int64_t count, hipStream_t stream);

// Block factor of an outer block of bw (<= 128) reflectors from their Gram
// matrix Y = V^T V (bw x bw, ld bw) and factors tau: T[j][j] = tau_j,
// T[0:j, j] = -tau_j T[0:j, 0:j] Y[0:j, j]; written as TrepT / TrepQ like
// the panel's (bw x bw*reps).
struct QrTArgs {
  const float* Y; int64_t y_mat;
  const float* tau; int64_t s_mat;
  float* TrepT; int64_t tT_mat;
  float* TrepQ; int64_t tQ_mat;
  int32_t bw, reps_t, reps_q;
  int32_t pad_;
};
hipError_t launch_qr_tfactor(const QrTArgs& a, int64_t count, hipStream_t stream);

// dst[b][i][j] = src(b)[i][j] for `count` rows x cols f32 matrices (dst
// contiguous, d_mat floats per matrix).
hipError_t launch_gather(const MatBatch& src, float* dst, int64_t d_mat, int32_t rows, int32_t cols,
                         int64_t count, hipStream_t stream);

// Q[i][j] = (i == j) for `count` n x n matrices (ld n).
hipError_t launch_eye(float* Q, int64_t q_mat, int32_t n, int64_t count, hipStream_t stream);

// dst[i][j] = src[i][j] * sgn[j] (src ld n, dst a caller batch, f32).
hipError_t launch_sign_copy(const float* src, int64_t src_mat, const float* sgn, int64_t s_mat,
                            const MatBatch& dst, int32_t n, int64_t count, hipStream_t stream);

// Adam in the rotated basis, elementwise over `count` rows x cols matrices:
//   M <- b1 M + (1-b1) g,  V <- b2 V + (1-b2) g^2,
//   out = (c1 M) / (sqrt(c2 V) + eps),
// g read from G (f32 or bf16), M, V in place (f32), out f32.
struct RotAdamArgs {
  MatBatch G, M, V, out;
  int32_t rows, cols;
  float beta1, beta2, eps, c1, c2;
  int32_t pad_;
};
hipError_t launch_rot_adam(const RotAdamArgs& a, int64_t count, hipStream_t stream);

}  // namespace muon
