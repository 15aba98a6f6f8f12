// Host stand-ins for the kernel launchers of libmuon355, for building the
// C-ABI layer (abi.cpp) on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing is enqueued and no device address is
// dereferenced: every launch the C-ABI layer builds is checked instead, each
// workspace operand against the workspace the caller passed (count x the
// per-matrix stride plus the operand's full extent for its tile grid).
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include <algorithm>

#include "muon_internal.h"

namespace {

const char* g_lo = nullptr;
const char* g_hi = nullptr;
long g_launches = 0;

[[noreturn]] void die(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::fprintf(stderr, "launch check failed: ");
  std::vfprintf(stderr, fmt, ap);
  std::fprintf(stderr, "\n");
  va_end(ap);
  std::abort();
}

// [p, p + (count-1)*mat + extent) inside the workspace
void in_ws(const void* p, int64_t count, int64_t mat, int64_t extent, const char* what) {
  if (!p) die("%s is NULL", what);
  if (count < 1 || mat < 0 || extent <= 0) die("%s: count %lld, stride %lld, extent %lld", what, (long long)count,
                                                (long long)mat, (long long)extent);
  const char* c = static_cast<const char*>(p);
  const int64_t end = (count - 1) * mat + extent;
  if (c < g_lo || end > g_hi - c) die("%s: [%p, +%lld) outside the workspace [%p, %p)", what, p, (long long)end, g_lo, g_hi);
}

}  // namespace

extern "C" void stub_set_workspace(const void* base, size_t bytes) {
  g_lo = static_cast<const char*>(base);
  g_hi = g_lo + bytes;
}
extern "C" long stub_launches() { return g_launches; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
extern "C" hipError_t hipGetLastError() { return hipSuccess; }

namespace muon {

FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) die("division by zero columns");
  FastDiv f{};
  f.d = d;
  return f;
}

int elementwise_blocks_per_matrix(int64_t rows, int64_t cols) { return static_cast<int>((rows * cols + 8191) / 8192); }

hipError_t launch_momentum(const MomentumArgs& a, int64_t count, bool, hipStream_t) {
  ++g_launches;
  in_ws(a.partials, 1, 0, count * a.blocks_per_mat * 4, "momentum partials");
  return hipSuccess;
}

hipError_t launch_momentum_grouped(const MomentumGroups& a, hipStream_t) {
  ++g_launches;
  if (a.ngroups < 1 || a.ngroups > kMaxGroups || a.first[0] != 0) die("momentum groups: %d", a.ngroups);
  for (int g = 0; g < a.ngroups; ++g) {
    const int64_t n = a.first[g + 1] - a.first[g];
    if (n <= 0 || n % a.g[g].blocks_per_mat) die("momentum group %d: %lld blocks", g, (long long)n);
    in_ws(a.g[g].partials, 1, 0, n * 4, "grouped momentum partials");
  }
  return hipSuccess;
}

// The static scratch of the allocation-free entry point: a fake device
// range of MUON_NOALLOC_SCRATCH_BYTES; the launches that follow are checked
// against it as against a caller's workspace.
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static const uintptr_t kScratch = uintptr_t{0x7f0000000000};
  *ptr = reinterpret_cast<void*>(kScratch);
  *bytes = size_t{8} << 20;
  stub_set_workspace(*ptr, *bytes);
  return hipSuccess;
}

hipError_t launch_sumsq_partials(const SumsqArgs& a, int64_t count, bool, hipStream_t) {
  ++g_launches;
  in_ws(a.partials, 1, 0, count * a.blocks_per_mat * 4, "sum-of-squares partials");
  return hipSuccess;
}

hipError_t launch_sumsq_finalize(const float* partials, int per, float* sumsq, int64_t count, hipStream_t) {
  ++g_launches;
  if (!sumsq || per < 1) die("finalize: sumsq %p, per %d", static_cast<void*>(sumsq), per);
  in_ws(partials, 1, 0, count * per * 4, "finalize partials");
  return hipSuccess;
}

hipError_t launch_sumsq_finalize_grouped(const FinalizeGroups& a, hipStream_t) {
  ++g_launches;
  for (int g = 0; g < a.ngroups; ++g)
    in_ws(a.partials[g], 1, 0, (a.first[g + 1] - a.first[g]) * a.per[g] * 4, "grouped finalize partials");
  return hipSuccess;
}

hipError_t launch_apply(const ApplyArgs&, int64_t count, bool, hipStream_t) {
  ++g_launches;
  if (count < 1) die("apply count %lld", (long long)count);
  return hipSuccess;
}

hipError_t launch_apply_grouped(const ApplyGroups& a, hipStream_t) {
  ++g_launches;
  for (int g = 0; g < a.ngroups; ++g)
    if (a.first[g + 1] - a.first[g] <= 0) die("apply group %d empty", g);
  return hipSuccess;
}

hipError_t launch_pack(const PackArgs& a, int64_t count, hipStream_t) {
  ++g_launches;
  const int es = a.compute ? 2 : 4;
  const int64_t n = static_cast<int64_t>(a.Pr) * a.Pc;
  if (a.Pr % 64 || a.Pc % 64) die("pack: padded shape %d x %d", a.Pr, a.Pc);
  if (!a.S && !a.T) die("pack writes nothing");
  if (a.S) in_ws(a.S, count, a.s_mat, n * es, "pack S");
  if (a.T) in_ws(a.T, count, a.t_mat, n * es, "pack T");
  if (a.Lo) {
    in_ws(a.Lo, count, a.lo_mat, n, "pack low-part codes");
    in_ws(a.LoE, count, a.loe_mat, n / kLoExpPerCodes, "pack low-part exponents");
  }
  return hipSuccess;
}

hipError_t launch_gram_reduce(const GramReduce& a, hipStream_t) {
  ++g_launches;
  if (a.ngroups < 1 || a.ngroups > kMaxGroups || a.first[0] != 0) die("gram reduce groups: %d", a.ngroups);
  for (int g = 0; g < a.ngroups; ++g) {
    const GramReduceGroup& r = a.g[g];
    const int64_t mm = static_cast<int64_t>(r.Mp) * r.Mp;
    const int64_t n = a.first[g + 1] - a.first[g];
    if ((r.tile != 128 && r.tile != 256) || r.Mp % r.tile) die("gram reduce %d: order %d, tile %d", g, r.Mp, r.tile);
    const int64_t T = r.Mp / r.tile, nb = r.tile / 64, per = T * (T + 1) / 2 * nb * nb;
    if (n <= 0 || n % per) die("gram reduce %d: order %d, %lld blocks", g, r.Mp, (long long)n);
    const int64_t count = n / per;
    in_ws(r.part, count, r.part_mat, r.splits * mm * 4, "gram reduce partials");
    in_ws(r.A, count, r.a_mat, mm * (r.compute ? 2 : 4), "gram reduce output");
  }
  return hipSuccess;
}

hipError_t launch_momentum_pack_grouped(const MomentumPackGroups& a, hipStream_t) {
  ++g_launches;
  if (a.ngroups < 1 || a.ngroups > kMaxGroups || a.first[0] != 0) die("momentum pack groups: %d", a.ngroups);
  for (int g = 0; g < a.ngroups; ++g) {
    const MomentumPackArgs& p = a.g[g];
    const int64_t n = a.first[g + 1] - a.first[g];
    if (p.Pr % 64 || p.Pc % 64 || p.Pr < p.rows || p.Pc < p.cols) die("momentum pack %d: padded %d x %d", g, p.Pr, p.Pc);
    if (p.tiles_c != p.Pc / 64 || p.tiles_per_mat != (p.Pr / 64) * p.tiles_c) die("momentum pack %d: tile grid", g);
    if (n <= 0 || n % p.tiles_per_mat) die("momentum pack group %d: %lld tiles", g, (long long)n);
    const int64_t count = n / p.tiles_per_mat;
    const int64_t elems = static_cast<int64_t>(p.Pr) * p.Pc;
    const int es = p.compute ? 2 : 4;
    in_ws(p.partials, 1, 0, n * 4, "momentum pack partials");
    if (!p.S && !p.T) die("momentum pack %d writes no X", g);
    if (p.S) in_ws(p.S, count, p.s_mat, elems * es, "momentum pack S");
    if (p.T) in_ws(p.T, count, p.t_mat, elems * es, "momentum pack T");
    if (p.compute != (p.Lo != nullptr)) die("momentum pack %d: low part with compute %d", g, p.compute);
    if (p.Lo) {
      in_ws(p.Lo, count, p.lo_mat, elems, "momentum pack low-part codes");
      in_ws(p.LoE, count, p.loe_mat, elems / kLoExpPerCodes, "momentum pack low-part exponents");
    }
  }
  return hipSuccess;
}

hipError_t launch_copy_out(const CopyOutArgs& a, int64_t count, hipStream_t) {
  ++g_launches;
  if (count < 1 || a.rows < 1 || a.cols < 1) die("copy_out shape");
  return hipSuccess;
}

hipError_t launch_adamw(const AdamWArgs& a, int64_t total_chunks, hipStream_t) {
  ++g_launches;
  if (total_chunks < 1 || a.count < 1) die("adamw: %lld chunks", (long long)total_chunks);
  return hipSuccess;
}

hipError_t launch_ns_gemm(int compute, int tile, int epi, bool kmajor, const GemmLaunch& L, hipStream_t) {
  ++g_launches;
  const int64_t es = compute ? 2 : 4;
  if (tile != 128 && tile != 256) die("tile %d", tile);
  if ((epi == EPI_UPDATE || epi == EPI_FINAL) && kmajor != (compute == 1)) die("update layout %d for compute %d", kmajor, compute);
  if (L.ngroups < 1 || L.ngroups > kMaxGroups) die("ngroups %d", L.ngroups);
  int64_t begin = 0;
  for (int g = 0; g < L.ngroups; ++g) {
    const GemmGroup& G = L.g[g];
    if (G.tile_begin != begin) die("group %d starts at tile %d, expected %lld", g, G.tile_begin, (long long)begin);
    const int64_t rows = static_cast<int64_t>(G.tiles_m) * tile, cols = static_cast<int64_t>(G.tiles_n) * tile;
    const int64_t want = G.sym ? static_cast<int64_t>(G.tiles_m) * (G.tiles_m + 1) / 2 : static_cast<int64_t>(G.tiles_m) * G.tiles_n;
    const int splits = G.splits > 1 ? G.splits : 1;
    if (splits > 1 && (epi != EPI_GRAM || !G.sym)) die("group %d: split reduction outside the Gram", g);
    if (G.tiles_per_mat != want * splits)
      die("group %d: %d tiles per matrix, expected %lld", g, G.tiles_per_mat, (long long)(want * splits));
    if (splits > 1) {
      if (G.K % (splits * 64) != 0) die("group %d: K %d in %d slices", g, G.K, splits);
      in_ws(G.part, G.count, G.part_mat, splits * rows * rows * 4, "split Gram partials");
    }
    if (G.K < 64 || G.K % 64) die("group %d: K %d", g, G.K);
    if (G.ms < 1 || G.ms > rows) die("group %d: short side %d beyond %lld padded rows", g, G.ms, (long long)rows);
    if (epi >= EPI_UPDATE && (G.ns < G.ms || G.ns > cols)) die("group %d: long side %d, %lld padded columns", g, G.ns, (long long)cols);
    begin += static_cast<int64_t>(G.tiles_per_mat) * G.count;
    // operands: P rows i with K contiguous; Q rows j with K contiguous, or k-major (K rows of cols)
    in_ws(G.P, G.count, G.p_mat, ((rows - 1) * G.ldp + G.K) * es, "P");
    if (kmajor && epi >= EPI_UPDATE && compute) {
      in_ws(G.Q, G.count, G.q_mat, ((G.K - 1) * static_cast<int64_t>(G.ldq) + cols) * es, "Q (k-major)");
    } else {
      in_ws(G.Q, G.count, G.q_mat, ((cols - 1) * G.ldq + G.K) * es, "Q");
    }
    if (epi == EPI_GRAM || epi == EPI_POLY) {
      if (G.tiles_m != G.tiles_n || !G.sym) die("symmetric stage with a %d x %d grid", G.tiles_m, G.tiles_n);
      if (epi == EPI_POLY) in_ws(G.E0, G.count, G.e0_mat, ((rows - 1) * G.lde0 + cols) * es, "poly A");
      in_ws(G.O0, G.count, G.o0_mat, ((rows - 1) * G.ldo0 + cols) * es, "Gram/poly output");
    } else if (compute) {
      in_ws(G.E1, G.count, G.e1_mat, rows * cols, "low-part codes in");
      in_ws(G.LoE, G.count, G.loe_mat, rows * cols / kLoExpPerCodes, "low-part exponents");
      if (epi == EPI_UPDATE) {
        in_ws(G.O0, G.count, G.o0_mat, rows * cols, "low-part codes out");
        in_ws(G.O1, G.count, G.o1_mat, ((rows - 1) * G.ldo1 + cols) * 2, "high part out");
        if (kmajor != (G.OT == nullptr)) die("X'^T output %p with kmajor %d", static_cast<void*>(G.OT), kmajor);
        if (G.OT) in_ws(G.OT, G.count, G.ot_mat, ((cols - 1) * G.ldot + rows) * 2, "X'^T out");
      }
    } else {
      in_ws(G.E0, G.count, G.e0_mat, ((rows - 1) * G.lde0 + cols) * 4, "X in");
      if (epi == EPI_UPDATE) {
        in_ws(G.O0, G.count, G.o0_mat, ((rows - 1) * G.ldo0 + cols) * 4, "X out");
        in_ws(G.OT, G.count, G.ot_mat, ((cols - 1) * G.ldot + rows) * 4, "X^T out");
      }
    }
  }
  if (begin != L.total_tiles) die("%lld tiles in groups, launch says %d", (long long)begin, L.total_tiles);
  return hipSuccess;
}

}  // namespace muon

// ------------------------------------------------------------------ SOAP

namespace {

using muon::MatBatch;
using muon::SgemmOperand;

bool in_workspace(const void* p) {
  const char* c = static_cast<const char*>(p);
  return c >= g_lo && c < g_hi;
}

// A product operand that lives in the workspace: every batch entry's rows x
// cols (memory orientation) inside it.  Caller memory is not checked.
void check_operand(const SgemmOperand& o, int64_t outer, int64_t K, int64_t count, const char* what) {
  if (o.ptrs || !in_workspace(o.base)) return;
  const int64_t es = o.dtype ? 2 : 4;
  const int64_t rows = o.kcontig ? outer : K, cols = o.kcontig ? K : outer;
  if (o.ld < cols) die("%s: ld %lld < %lld columns", what, (long long)o.ld, (long long)cols);
  if (o.vec && (o.ld % 4 || (reinterpret_cast<uintptr_t>(o.base) + o.off) % (4 * es) || o.stride % (4 * es)))
    die("%s: vector loads on a misaligned operand", what);
  in_ws(o.base + o.off, count, o.stride, ((rows - 1) * o.ld + cols) * es, what);
}

void check_batch_ws(const MatBatch& m, int64_t rows, int64_t cols, int64_t count, const char* what) {
  if (m.ptrs || !in_workspace(m.base)) return;
  if (m.ld < cols) die("%s: ld %lld < %lld", what, (long long)m.ld, (long long)cols);
  in_ws(m.base, count, m.stride_bytes, ((rows - 1) * m.ld + cols) * (m.dtype ? 2 : 4), what);
}

}  // namespace

namespace muon {

hipError_t launch_sgemm(const SgemmArgs& a, hipStream_t) {
  ++g_launches;
  if (a.M < 1 || a.N < 1 || a.K < 1 || a.count < 1 || a.splits < 1) die("sgemm %d x %d x %d", a.M, a.N, a.K);
  if (int64_t{a.count} * a.splits > 65535) die("sgemm: %d x %d batch entries", a.count, a.splits);
  if (a.splits > 1) {
    if (a.ksplit % kSgemmBK || int64_t{a.splits - 1} * a.ksplit >= a.K || int64_t{a.splits} * a.ksplit < a.K)
      die("sgemm: %d splits of %d do not tile K = %d", a.splits, a.ksplit, a.K);
    if (a.beta != 0.f) die("sgemm: split partials with beta != 0");
    if (a.sym) die("sgemm: symmetric split");
  } else if (a.ksplit < a.K) {
    die("sgemm: ksplit %d < K %d", a.ksplit, a.K);
  }
  if (a.sym && a.M != a.N) die("sgemm: symmetric %d x %d", a.M, a.N);
  check_operand(a.a, a.M, a.K, a.count, "sgemm A");
  check_operand(a.b, a.N, a.K, a.count, "sgemm B");
  if (!a.c_ptrs && in_workspace(a.c)) {
    if (a.ldc < a.N) die("sgemm C: ldc %lld < %d", (long long)a.ldc, a.N);
    const int64_t extent = ((int64_t{a.M} - 1) * a.ldc + a.N) * 4;
    if (a.splits > 1 && a.c_split < extent) die("sgemm C: split partials overlap");
    in_ws(a.c + a.c_off, a.count, a.c_stride, (int64_t{a.splits} - 1) * a.c_split + extent, "sgemm C");
  }
  return hipSuccess;
}

hipError_t launch_sgemm_list(const SgemmArgs* gs, int n, hipStream_t s) {
  if (n < 1 || n > 2 * kSgemmMaxList) die("sgemm list of %d products", n);
  for (int i = 0; i < n; ++i) {
    const hipError_t e = launch_sgemm(gs[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_qr_panel(const QrPanelArgs& a, int64_t count, hipStream_t) {
  ++g_launches;
  if (a.n < 1 || a.c0 < 0 || a.c0 >= a.n || a.c0 % kQrPanel) die("qr panel: n %d, c0 %d", a.n, a.c0);
  if (a.reps_t < 1 || a.reps_t > 16 || a.reps_q < 0 || a.reps_q > 16) die("qr panel reps %d %d", a.reps_t, a.reps_q);
  if (a.zpre < 0 || a.zpre > a.c0 || a.zpre >= kQrOuter) die("qr panel: %d rows above", a.zpre);
  const int64_t n = a.n, h = n - a.c0, nb = std::min<int64_t>(kQrPanel, h);
  in_ws(a.A, count, a.a_mat * 4, n * n * 4, "qr A");
  in_ws(a.V - a.zpre, count, a.v_mat * 4, ((nb - 1) * n + a.zpre + h) * 4, "qr reflector slot");
  in_ws(a.TrepT, count, a.tT_mat * 4, nb * nb * a.reps_t * 4, "qr T^T copies");
  if (a.reps_q > 0) in_ws(a.TrepQ, count, a.tQ_mat * 4, nb * nb * a.reps_q * 4, "qr T copies");
  in_ws(a.sgn, count, a.s_mat * 4, n * 4, "qr signs");
  in_ws(a.tau, count, a.s_mat * 4, n * 4, "qr factors");
  return hipSuccess;
}

hipError_t launch_qr_tfactor(const QrTArgs& a, int64_t count, hipStream_t) {
  ++g_launches;
  if (a.bw < 1 || a.bw > kQrOuter || a.reps_t < 1 || a.reps_t > 16 || a.reps_q < 1 || a.reps_q > 16)
    die("qr block factor: width %d, reps %d %d", a.bw, a.reps_t, a.reps_q);
  const int64_t bw = a.bw;
  in_ws(a.Y, count, a.y_mat * 4, bw * bw * 4, "qr block gram");
  in_ws(a.tau, count, a.s_mat * 4, bw * 4, "qr block factors");
  in_ws(a.TrepT, count, a.tT_mat * 4, bw * bw * a.reps_t * 4, "qr block T^T copies");
  in_ws(a.TrepQ, count, a.tQ_mat * 4, bw * bw * a.reps_q * 4, "qr block T copies");
  return hipSuccess;
}

hipError_t launch_eye(float* Q, int64_t q_mat, int32_t n, int64_t count, hipStream_t) {
  ++g_launches;
  in_ws(Q, count, q_mat * 4, int64_t{n} * n * 4, "identity");
  return hipSuccess;
}

hipError_t launch_sign_copy(const float* src, int64_t src_mat, const float* sgn, int64_t s_mat, const MatBatch& dst,
                            int32_t n, int64_t count, hipStream_t) {
  ++g_launches;
  in_ws(src, count, src_mat * 4, int64_t{n} * n * 4, "sign copy source");
  in_ws(sgn, count, s_mat * 4, int64_t{n} * 4, "sign copy signs");
  if (dst.dtype != 0 || dst.ld < n) die("sign copy destination");
  return hipSuccess;
}

hipError_t launch_gather(const MatBatch& src, float* dst, int64_t d_mat, int32_t rows, int32_t cols, int64_t count,
                         hipStream_t) {
  ++g_launches;
  if (src.dtype != 0 || src.ld < cols) die("gather source");
  in_ws(dst, count, d_mat * 4, int64_t{rows} * cols * 4, "gather destination");
  return hipSuccess;
}

hipError_t launch_rot_adam(const RotAdamArgs& a, int64_t count, hipStream_t) {
  ++g_launches;
  if (a.rows < 1 || a.cols < 1) die("rotated adam %d x %d", a.rows, a.cols);
  check_batch_ws(a.G, a.rows, a.cols, count, "rotated adam G");
  check_batch_ws(a.M, a.rows, a.cols, count, "rotated adam M");
  check_batch_ws(a.V, a.rows, a.cols, count, "rotated adam V");
  check_batch_ws(a.out, a.rows, a.cols, count, "rotated adam out");
  if (a.out.dtype != 0 || a.M.dtype != 0 || a.V.dtype != 0) die("rotated adam state dtypes");
  return hipSuccess;
}

}  // namespace muon
