// C-ABI layer of libmuon355: argument validation, workspace planning and the
// host loop that enqueues the Newton-Schulz stages.  Declarations and their
// contracts are in include/muon355.h.

#include "../../include/muon355.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "muon_internal.h"

namespace muon {
int elementwise_blocks_per_matrix(int64_t rows, int64_t cols);
}

namespace {

using namespace muon;

thread_local char g_last_error[512] = "";

muon_status_t fail(muon_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
muon_status_t fail(muon_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Prefix the current error detail with the group it belongs to.
muon_status_t in_group(muon_status_t st, int g) {
  if (st == MUON_OK) return st;
  char tmp[sizeof(g_last_error)];
  snprintf(tmp, sizeof(tmp), "group %d: %.480s", g, g_last_error);
  memcpy(g_last_error, tmp, sizeof(tmp));
  return st;
}

muon_status_t ok() {
  g_last_error[0] = '\0';
  return MUON_OK;
}

constexpr int64_t kAlign = 256;
static_assert(kAdamWChunk == MUON_ADAMW_CHUNK, "chunk size of the AdamW tensor list");
constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;
constexpr int64_t kSplitGramWorkgroups = 512;  // see gram_splits

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// A group whose Gram has few tiles (the 96 per-head 128 x 4096 blocks are 96
// tiles; the GPU holds 512 of that size at once) splits its reduction in
// slices: up to kSplitGramWorkgroups workgroups, each slice at least 512 deep
// and a whole number of 64-deep k-tiles.  Decided per group from its own
// shape and count only, so a group's results do not depend on the groups it
// is launched with.
int gram_splits(int64_t count, int64_t T, int64_t Np) {
  const int64_t tiles = count * T * (T + 1) / 2;
  int S = 1;
  if (tiles > 128) return S;
  while (S < 8 && tiles * S * 2 <= kSplitGramWorkgroups && Np % (S * 2 * 64) == 0 && Np / (S * 2) >= 512) S *= 2;
  return S;
}
int esize(int32_t dtype) { return dtype == MUON_BF16 ? 2 : 4; }

muon_status_t check_batch(const muon_batch_t* b, const char* name, bool allow_bf16) {
  if (!b) return fail(MUON_ERR_INVALID_VALUE, "%s: descriptor is NULL", name);
  if (b->dtype != MUON_F32 && b->dtype != MUON_BF16)
    return fail(MUON_ERR_INVALID_VALUE, "%s: dtype %d is not MUON_F32 or MUON_BF16", name, b->dtype);
  if (b->dtype == MUON_BF16 && !allow_bf16)
    return fail(MUON_ERR_UNSUPPORTED, "%s: must be MUON_F32", name);
  if (b->reserved != 0) return fail(MUON_ERR_INVALID_VALUE, "%s: reserved field must be 0", name);
  if (b->count < 1 || b->count > 65535)
    return fail(MUON_ERR_INVALID_VALUE, "%s: count %lld outside [1, 65535]", name, (long long)b->count);
  if (b->rows < 1 || b->cols < 1)
    return fail(MUON_ERR_INVALID_VALUE, "%s: rows and cols must be >= 1 (got %lld x %lld)", name,
                (long long)b->rows, (long long)b->cols);
  if (b->rows > kMaxElems / b->cols)
    return fail(MUON_ERR_UNSUPPORTED, "%s: %lld x %lld has more than 2^31-1 elements", name,
                (long long)b->rows, (long long)b->cols);
  if (b->ld < b->cols)
    return fail(MUON_ERR_INVALID_VALUE, "%s: ld %lld < cols %lld", name, (long long)b->ld, (long long)b->cols);
  if (!b->ptrs && !b->base) return fail(MUON_ERR_INVALID_VALUE, "%s: both ptrs and base are NULL", name);
  if (!b->ptrs && b->count > 1 && b->stride < (b->rows - 1) * b->ld + b->cols)
    return fail(MUON_ERR_INVALID_VALUE, "%s: stride %lld overlaps consecutive matrices", name,
                (long long)b->stride);
  if (!b->ptrs && (reinterpret_cast<uintptr_t>(b->base) % esize(b->dtype)) != 0)
    return fail(MUON_ERR_INVALID_VALUE, "%s: base is not aligned to its element size", name);
  return MUON_OK;
}

bool same_shape(const muon_batch_t* a, const muon_batch_t* b) {
  return a->count == b->count && a->rows == b->rows && a->cols == b->cols;
}

MatBatch to_mat(const muon_batch_t* b) {
  MatBatch m;
  m.base = static_cast<char*>(b->base);
  m.stride_bytes = b->stride * esize(b->dtype);
  m.ptrs = b->ptrs;
  m.ld = b->ld;
  m.dtype = b->dtype;
  m.pad_ = 0;
  return m;
}

// 16-byte vector path possible: rows of 8 elements start on 16-byte boundaries.
// Four-element loads (8 bytes of bf16, 16 of f32): every row and matrix
// starts on a 4-element boundary of a suitably aligned base (the entries of
// a pointer array are documented 16-byte aligned).
bool vec4_ok(const muon_batch_t* b) {
  if (b->ld % 4 != 0) return false;
  if (b->ptrs) return true;
  return reinterpret_cast<uintptr_t>(b->base) % (4 * esize(b->dtype)) == 0 && (b->count == 1 || b->stride % 4 == 0);
}

bool vec_ok(const muon_batch_t* b) {
  if (b->cols % 8 != 0 || b->ld % 8 != 0) return false;
  if (b->ptrs) return true;  // documented: every pointer 16-byte aligned
  if (reinterpret_cast<uintptr_t>(b->base) % 16 != 0) return false;
  return (b->stride * esize(b->dtype)) % 16 == 0 || b->count == 1;
}

bool finite(float x) { return std::isfinite(x); }

muon_status_t launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MUON_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return MUON_OK;
}

// With MUON355_DEBUG_SYNC=1 in the environment every entry point waits for
// the work it enqueued and reports a failed kernel as MUON_ERR_LAUNCH naming
// the call.  A debugging aid only: otherwise the library never synchronizes.
muon_status_t done(hipStream_t s, const char* what) {
  const char* v = std::getenv("MUON355_DEBUG_SYNC");
  if (v && v[0] == '1' && v[1] == '\0') {
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(MUON_ERR_LAUNCH, "%s (debug sync): %s", what, hipGetErrorString(e));
  }
  return ok();
}

// ------------------------------------------------------------ NS workspace plan

struct GroupPlan {
  int64_t count;
  int32_t rows, cols;   // stored shape
  int32_t ms, ns;       // Newton-Schulz shape (ms <= ns)
  int32_t tall;
  int32_t tile;
  int32_t Mp, Np;       // padded NS shape
  int32_t Pr, Pc;       // padded stored shape
  int32_t kmajor;       // bf16 update reads X itself, k-major (no X^T kept)
  // byte offsets into the workspace
  int64_t xlo, xloe, xc[2], xt[2], a, b, sumsq, partials;  // xlo, xloe: low part of X, codes and
                                                            // exponents (bf16 compute)
  int32_t blocks_per_mat;
  int32_t pack_tiles;   // 64 x 64 tiles of the padded stored extent
  int32_t gram_splits;  // the Gram's reduction in this many slices (1: not split)
  int64_t part;         // byte offset of the split Gram's partial sums
};

struct Plan {
  std::vector<GroupPlan> g;
  int64_t bytes = 0;
};

// packed: the momentum kernel writes N into the buffers (momentum_pack_kernel),
// with one partial sum of squares per 64 x 64 tile of the padded stored extent.
bool make_plan(int ngroups, const int64_t* counts, const int64_t* rows, const int64_t* cols,
               int32_t compute, const bool* need_sumsq, Plan* plan, bool packed = false) {
  if (ngroups < 1 || ngroups > kMaxGroups) return false;
  if (compute != MUON_F32 && compute != MUON_BF16) return false;
  const int64_t es = compute == MUON_BF16 ? 2 : 4;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  plan->g.clear();
  // With bf16 compute the update reads X itself, k-major through LDS
  // transpose reads, and X^T is never written (on MI355X this beat reading a
  // kept X^T at every reduction length measured, 128 to 4096 deep: the saved
  // X'^T stores and transposed staging outweigh the transpose reads).  The
  // fp32 update reads X^T.
  for (int i = 0; i < ngroups; ++i) {
    if (counts[i] < 1 || counts[i] > 65535 || rows[i] < 1 || cols[i] < 1) return false;
    if (rows[i] > kMaxElems / cols[i]) return false;
    GroupPlan p{};
    p.count = counts[i];
    p.rows = static_cast<int32_t>(rows[i]);
    p.cols = static_cast<int32_t>(cols[i]);
    p.tall = rows[i] > cols[i];
    p.ms = static_cast<int32_t>(p.tall ? cols[i] : rows[i]);
    p.ns = static_cast<int32_t>(p.tall ? rows[i] : cols[i]);
    p.tile = p.ms <= 128 ? 128 : 256;
    p.Mp = static_cast<int32_t>(align_up(p.ms, p.tile));
    p.Np = static_cast<int32_t>(align_up(p.ns, p.tile));
    p.kmajor = compute == MUON_BF16;
    // per-matrix byte offsets inside the GEMM kernels are 32-bit: an fp32
    // padded matrix must stay below 4 GiB
    if (static_cast<int64_t>(p.Mp) * p.Np > (int64_t{1} << 30)) return false;
    p.Pr = p.tall ? p.Np : p.Mp;
    p.Pc = p.tall ? p.Mp : p.Np;
    const int64_t mn = static_cast<int64_t>(p.Mp) * p.Np;
    const int64_t mm = static_cast<int64_t>(p.Mp) * p.Mp;
    p.xlo = compute == MUON_BF16 ? take(p.count * mn) : -1;
    p.xloe = compute == MUON_BF16 ? take(p.count * mn / kLoExpPerCodes) : -1;
    p.xc[0] = take(p.count * mn * es);
    p.xc[1] = take(p.count * mn * es);
    // X^T only where the update reads it
    p.xt[0] = p.kmajor ? -1 : take(p.count * mn * es);
    p.xt[1] = p.kmajor ? -1 : take(p.count * mn * es);
    p.a = take(p.count * mm * es);
    p.b = take(p.count * mm * es);
    p.gram_splits = gram_splits(p.count, p.Mp / p.tile, p.Np);
    p.part = p.gram_splits > 1 ? take(p.count * p.gram_splits * mm * 4) : -1;
    p.blocks_per_mat = elementwise_blocks_per_matrix(p.rows, p.cols);
    p.pack_tiles = (p.Pr / 64) * (p.Pc / 64);
    if (packed) {
      p.sumsq = -1;
      p.partials = take(p.count * p.pack_tiles * 4);
    } else if (need_sumsq == nullptr || need_sumsq[i]) {
      p.sumsq = take(p.count * 4);
      p.partials = take(p.count * p.blocks_per_mat * 4);
    } else {
      p.sumsq = p.partials = -1;
    }
    plan->g.push_back(p);
  }
  plan->bytes = off;
  return true;
}

GemmGroup base_group(const GroupPlan& p, int tiles_per_mat, int tiles_m, int tiles_n, int sym) {
  GemmGroup G;
  std::memset(&G, 0, sizeof(G));
  G.count = static_cast<int32_t>(p.count);
  G.tiles_per_mat = tiles_per_mat;
  G.tiles_m = tiles_m;
  G.tiles_n = tiles_n;
  G.sym = sym;
  G.ms = p.ms;
  G.ns = p.ns;
  G.tall = p.tall;
  return G;
}

// packed: there is no `ins`; the momentum kernel has written N (not yet
// normalized) into the workspace and the sums of squares into sumsqs, and
// step 0 applies the scale.
muon_status_t run_orthogonalize(int ngroups, const muon_batch_t* ins, const float* const* sumsqs,
                                const muon_batch_t* outs, int steps, float a, float b, float c,
                                float eps, int32_t compute, void* workspace, size_t ws_bytes,
                                hipStream_t stream, bool packed = false, const float* ap_decay = nullptr,
                                const float* ap_step = nullptr) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (compute != MUON_F32 && compute != MUON_BF16)
    return fail(MUON_ERR_INVALID_VALUE, "compute %d is not MUON_F32 or MUON_BF16", compute);
  if (steps < 0) return fail(MUON_ERR_INVALID_VALUE, "steps %d < 0", steps);
  if (!finite(a) || !finite(b) || !finite(c)) return fail(MUON_ERR_INVALID_VALUE, "coefficients must be finite");
  if (!finite(eps) || eps < 0.0f) return fail(MUON_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  if ((!packed && !ins) || !outs) return fail(MUON_ERR_INVALID_VALUE, "ins/outs is NULL");
  if (packed && steps < 1) return fail(MUON_ERR_INVALID_VALUE, "the packed form needs steps >= 1");
  if (packed && !sumsqs) return fail(MUON_ERR_INVALID_VALUE, "sumsqs is NULL");
  std::vector<int64_t> counts(ngroups), rows(ngroups), cols(ngroups);
  bool need[kMaxGroups];
  for (int g = 0; g < ngroups; ++g) {
    muon_status_t st;
    if (!packed) {
      st = check_batch(&ins[g], "in", true);
      if (st != MUON_OK) return st;
    }
    st = check_batch(&outs[g], "out", true);
    if (st != MUON_OK) return st;
    if (!packed && !same_shape(&ins[g], &outs[g]))
      return fail(MUON_ERR_INVALID_VALUE, "in and out shapes differ (group %d)", g);
    if (packed && !sumsqs[g]) return fail(MUON_ERR_INVALID_VALUE, "sumsqs[%d] is NULL", g);
    counts[g] = outs[g].count;
    rows[g] = outs[g].rows;
    cols[g] = outs[g].cols;
    need[g] = !packed && (sumsqs == nullptr || sumsqs[g] == nullptr);
  }
  Plan plan;
  if (!make_plan(ngroups, counts.data(), rows.data(), cols.data(), compute, need, &plan, packed))
    return fail(MUON_ERR_UNSUPPORTED, "a padded Newton-Schulz shape exceeds 2^30 elements");
  if (!workspace || ws_bytes < static_cast<size_t>(plan.bytes))
    return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes given, %lld needed", ws_bytes, (long long)plan.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MUON_ERR_WORKSPACE, "workspace must be 16-byte aligned");

  char* ws = static_cast<char*>(workspace);
  const int64_t es = compute == MUON_BF16 ? 2 : 4;
  hipError_t e;

  // 1. sums of squares that the caller did not provide
  std::vector<const float*> ssq(ngroups);
  for (int g = 0; g < ngroups; ++g) {
    const GroupPlan& p = plan.g[g];
    if (!need[g]) {
      ssq[g] = sumsqs[g];
      continue;
    }
    SumsqArgs sa;
    sa.X = to_mat(&ins[g]);
    sa.partials = reinterpret_cast<float*>(ws + p.partials);
    sa.blocks_per_mat = p.blocks_per_mat;
    sa.rows = p.rows;
    sa.cols = p.cols;
    sa.cdiv = make_fastdiv(static_cast<uint32_t>(p.cols));
    if ((e = launch_sumsq_partials(sa, p.count, vec_ok(&ins[g]), stream)) != hipSuccess)
      return launch_status(e, "sumsq partials");
    float* out = reinterpret_cast<float*>(ws + p.sumsq);
    if ((e = launch_sumsq_finalize(sa.partials, p.blocks_per_mat, out, p.count, stream)) != hipSuccess)
      return launch_status(e, "sumsq finalize");
    ssq[g] = out;
  }

  if (steps == 0) {  // X_0 itself, straight from N
    for (int g = 0; g < ngroups; ++g) {
      const GroupPlan& p = plan.g[g];
      CopyOutArgs ca;
      ca.N = to_mat(&ins[g]);
      ca.sumsq = ssq[g];
      ca.eps = eps;
      ca.out = to_mat(&outs[g]);
      ca.rows = p.rows;
      ca.cols = p.cols;
      if ((e = launch_copy_out(ca, p.count, stream)) != hipSuccess) return launch_status(e, "copy out");
    }
    return done(stream, "run_orthogonalize");
  }

  // 2. X_0 = N / (||N|| + eps) into the padded buffers (X, and X^T where the
  // update reads it); the packed form has N there already
  for (int g = 0; g < ngroups && !packed; ++g) {
    const GroupPlan& p = plan.g[g];
    const int64_t mn = static_cast<int64_t>(p.Mp) * p.Np;
    PackArgs pa;
    pa.N = to_mat(&ins[g]);
    pa.sumsq = ssq[g];
    pa.eps = eps;
    pa.rows = p.rows;
    pa.cols = p.cols;
    pa.Pr = p.Pr;
    pa.Pc = p.Pc;
    pa.compute = compute;
    pa.tall = p.tall;
    pa.nvec = vec4_ok(&ins[g]);
    pa.pad_ = 0;
    // S: the stored orientation, T: its transpose; X is whichever is wide.
    // A k-major group keeps no X^T.
    pa.S = p.tall ? (p.kmajor ? nullptr : ws + p.xt[0]) : ws + p.xc[0];
    pa.T = p.tall ? ws + p.xc[0] : (p.kmajor ? nullptr : ws + p.xt[0]);
    pa.s_mat = pa.t_mat = mn * es;
    pa.Lo = compute == MUON_BF16 ? reinterpret_cast<int8_t*>(ws + p.xlo) : nullptr;
    pa.lo_mat = mn;
    pa.LoE = compute == MUON_BF16 ? reinterpret_cast<uint8_t*>(ws + p.xloe) : nullptr;
    pa.loe_mat = mn / kLoExpPerCodes;
    pa.lo_bm = p.tile;
    pa.lo_tiles_n = p.Np / p.tile;
    if ((e = launch_pack(pa, p.count, stream)) != hipSuccess) return launch_status(e, "pack");
  }

  // 3. the K-step loop: Gram, polynomial, update; one launch per stage and
  // tile class
  for (int k = 0; k < steps; ++k) {
    const int cur = k & 1;
    const int nxt = cur ^ 1;
    const bool last = k + 1 == steps;
    for (int stage = 0; stage < 3; ++stage) {
      for (int tile : {256, 128}) {
        GemmLaunch L;
        std::memset(&L, 0, sizeof(L));
        L.a = a;
        L.b = b;
        L.c = c;
        int total = 0;
        for (int g = 0; g < ngroups; ++g) {
          const GroupPlan& p = plan.g[g];
          if (p.tile != tile) continue;
          const int T = p.Mp / tile;
          const int64_t mn = static_cast<int64_t>(p.Mp) * p.Np;
          const int64_t mm = static_cast<int64_t>(p.Mp) * p.Mp;
          GemmGroup G;
          if (stage == 0) {  // A = X X^T
            G = base_group(p, T * (T + 1) / 2 * p.gram_splits, T, T, 1);
            G.P = G.Q = ws + p.xc[cur];
            G.p_mat = G.q_mat = mn * es;
            G.ldp = G.ldq = p.Np;
            G.K = p.Np;
            G.O0 = ws + p.a;
            G.o0_mat = mm * es;
            G.ldo0 = p.Mp;
            G.splits = p.gram_splits;
            if (p.gram_splits > 1) {
              G.part = reinterpret_cast<float*>(ws + p.part);
              G.part_mat = p.gram_splits * mm * 4;
            }
          } else if (stage == 1) {  // B = b A + c A A
            G = base_group(p, T * (T + 1) / 2, T, T, 1);
            G.P = G.Q = ws + p.a;
            G.p_mat = G.q_mat = mm * es;
            G.ldp = G.ldq = p.Mp;
            G.K = p.Mp;
            G.E0 = ws + p.a;
            G.e0_mat = mm * es;
            G.lde0 = p.Mp;
            G.O0 = ws + p.b;
            G.o0_mat = mm * es;
            G.ldo0 = p.Mp;
          } else {  // X' = a X + B X
            const int Tn = p.Np / tile;
            G = base_group(p, T * Tn, T, Tn, 0);
            G.P = ws + p.b;
            G.p_mat = mm * es;
            G.ldp = p.Mp;
            // second operand: X^T, or X itself read k-major (a k-major bf16 class)
            G.Q = ws + (p.kmajor ? p.xc[cur] : p.xt[cur]);
            G.q_mat = mn * es;
            G.ldq = p.kmajor ? p.Np : p.Mp;
            G.K = p.Mp;
            // a*X: X in fp32, or with bf16 compute its low part (the high
            // part is the Q operand, which the kernel adds from LDS)
            if (compute == MUON_BF16) {
              G.E1 = ws + p.xlo;
              G.e1_mat = mn;
              G.LoE = reinterpret_cast<uint8_t*>(ws + p.xloe);
              G.loe_mat = mn / kLoExpPerCodes;
              G.lde1 = p.Np;
            } else {
              G.E0 = ws + p.xc[cur];
              G.e0_mat = mn * 4;
              G.lde0 = p.Np;
            }
            if (last) {
              G.user = to_mat(&outs[g]);
              if (ap_decay != nullptr) {  // outs are the weights: W <- decay*W - step*O
                G.ap = 1;
                G.ap_decay = ap_decay[g];
                G.ap_step = ap_step[g];
              }
            } else if (compute == MUON_BF16) {
              // the low part is rewritten in place: each element is read
              // and written by the same lane of the same tile
              G.O0 = ws + p.xlo;
              G.o0_mat = mn;
              G.ldo0 = p.Np;
              G.O1 = ws + p.xc[nxt];
              G.o1_mat = mn * 2;
              G.ldo1 = p.Np;
            } else {
              G.O0 = ws + p.xc[nxt];
              G.o0_mat = mn * 4;
              G.ldo0 = p.Np;
            }
            if (!last && !p.kmajor) {
              G.OT = ws + p.xt[nxt];
              G.ot_mat = mn * es;
              G.ldot = p.Mp;
            }
          }
          if (packed && k == 0) {  // X_0 = N / (||N|| + eps), applied in step 0's three stages
            G.xs_sumsq = ssq[g];
            G.xs_eps = eps;
          }
          L.g[L.ngroups++] = G;
        }
        if (L.ngroups == 0) continue;
        // Longest tiles first (reduction length decides a tile's cost), so
        // the short ones fill in at the end of the launch.
        std::stable_sort(L.g, L.g + L.ngroups, [](const GemmGroup& x, const GemmGroup& y) { return x.K > y.K; });
        for (int q = 0; q < L.ngroups; ++q) {
          L.g[q].tile_begin = total;
          total += L.g[q].tiles_per_mat * L.g[q].count;
        }
        L.total_tiles = total;
        const int epi = stage == 0 ? EPI_GRAM : stage == 1 ? EPI_POLY : (last ? EPI_FINAL : EPI_UPDATE);
        if ((e = launch_ns_gemm(compute, tile, epi, compute == MUON_BF16, L, stream)) != hipSuccess)
          return launch_status(e, "newton-schulz gemm");
        if (stage == 0) {  // add the slices of split Grams
          GramReduce R;
          std::memset(&R, 0, sizeof(R));
          for (int g = 0; g < ngroups; ++g) {
            const GroupPlan& p = plan.g[g];
            if (p.tile != tile || p.gram_splits < 2) continue;
            const int64_t mm = static_cast<int64_t>(p.Mp) * p.Mp;
            GramReduceGroup& r = R.g[R.ngroups];
            r.part = reinterpret_cast<const float*>(ws + p.part);
            r.part_mat = p.gram_splits * mm * 4;
            r.A = ws + p.a;
            r.a_mat = mm * es;
            r.xs_sumsq = packed && k == 0 ? ssq[g] : nullptr;
            r.xs_eps = eps;
            r.Mp = p.Mp;
            r.tile = tile;
            r.splits = p.gram_splits;
            r.compute = compute;
            const int64_t T = p.Mp / tile, nb = tile / 64;  // 64x64 blocks of the computed tiles
            R.first[R.ngroups + 1] = R.first[R.ngroups] + p.count * (T * (T + 1) / 2 * nb * nb);
            ++R.ngroups;
          }
          if (R.ngroups > 0 && (e = launch_gram_reduce(R, stream)) != hipSuccess)
            return launch_status(e, "split gram reduce");
        }
      }
    }
  }
  return done(stream, "run_orthogonalize");
}

}  // namespace

extern "C" {

int muon_abi_version(void) { return MUON355_ABI_VERSION; }

const char* muon_last_error(void) { return g_last_error; }

muon_status_t muon_adamw(const muon_tensor_list_t* t, int64_t step, float lr, float beta1, float beta2,
                         float eps, float weight_decay, void* stream) {
  if (!t) return fail(MUON_ERR_INVALID_VALUE, "tensor list is NULL");
  if (t->count < 1) return fail(MUON_ERR_INVALID_VALUE, "count %lld < 1", (long long)t->count);
  if (t->total_chunks < 1 || t->total_chunks > kMaxElems)
    return fail(MUON_ERR_INVALID_VALUE, "total_chunks %lld outside [1, 2^31-1]", (long long)t->total_chunks);
  if (!t->params || !t->grads || !t->exp_avg || !t->exp_avg_sq || !t->numels || !t->chunk_offsets)
    return fail(MUON_ERR_INVALID_VALUE, "a device array of the tensor list is NULL");
  if ((t->param_dtype != MUON_F32 && t->param_dtype != MUON_BF16) ||
      (t->grad_dtype != MUON_F32 && t->grad_dtype != MUON_BF16))
    return fail(MUON_ERR_INVALID_VALUE, "param_dtype/grad_dtype must be MUON_F32 or MUON_BF16");
  if (step < 1) return fail(MUON_ERR_INVALID_VALUE, "step %lld < 1", (long long)step);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(MUON_ERR_INVALID_VALUE, "betas must lie in [0, 1)");
  if (!finite(eps) || eps < 0.0f) return fail(MUON_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  if (!finite(lr) || !finite(weight_decay)) return fail(MUON_ERR_INVALID_VALUE, "lr and weight_decay must be finite");
  AdamWArgs a;
  a.count = t->count;
  a.params = t->params;
  a.grads = t->grads;
  a.exp_avg = t->exp_avg;
  a.exp_avg_sq = t->exp_avg_sq;
  a.numels = t->numels;
  a.chunk_offsets = t->chunk_offsets;
  a.param_bf16 = t->param_dtype == MUON_BF16;
  a.grad_bf16 = t->grad_dtype == MUON_BF16;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  // bias corrections in double: 1 - beta^t loses nothing for small t
  a.c1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step))));
  a.c2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step))));
  a.lr = lr;
  a.decay = static_cast<float>(1.0 - static_cast<double>(lr) * weight_decay);
  const hipError_t e = launch_adamw(a, t->total_chunks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return launch_status(e, "adamw");
  return done(static_cast<hipStream_t>(stream), "muon_adamw");
}

const char* muon_status_string(muon_status_t s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_VALUE: return "MUON_ERR_INVALID_VALUE";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_LAUNCH: return "MUON_ERR_LAUNCH";
  }
  return "unknown muon_status_t";
}

size_t muon_momentum_workspace(int64_t count, int64_t rows, int64_t cols) {
  if (count < 1 || rows < 1 || cols < 1 || rows > kMaxElems / cols) return 0;
  return static_cast<size_t>(align_up(count * elementwise_blocks_per_matrix(rows, cols) * 4, kAlign));
}

}  // extern "C"

namespace {

// Checks of one momentum batch; fills the kernel arguments (partials left
// for the caller) and whether 16-byte accesses apply.
muon_status_t prepare_momentum(const muon_batch_t* grad, const muon_batch_t* mom, const muon_batch_t* nout,
                               float* sumsq, float beta, int nesterov, MomentumArgs* a, bool* vec) {
  muon_status_t st;
  if ((st = check_batch(grad, "grad", true)) != MUON_OK) return st;
  if ((st = check_batch(mom, "mom", false)) != MUON_OK) return st;
  if (!same_shape(grad, mom)) return fail(MUON_ERR_INVALID_VALUE, "grad and mom shapes differ");
  if (nout) {
    if ((st = check_batch(nout, "nout", true)) != MUON_OK) return st;
    if (!same_shape(grad, nout)) return fail(MUON_ERR_INVALID_VALUE, "grad and nout shapes differ");
  } else if (nesterov) {
    return fail(MUON_ERR_INVALID_VALUE, "nout may be NULL only without Nesterov");
  }
  if (!sumsq) return fail(MUON_ERR_INVALID_VALUE, "sumsq is NULL");
  if (!(beta >= 0.0f && beta < 1.0f)) return fail(MUON_ERR_INVALID_VALUE, "beta must lie in [0, 1)");
  if (nesterov != 0 && nesterov != 1) return fail(MUON_ERR_INVALID_VALUE, "nesterov must be 0 or 1");
  std::memset(a, 0, sizeof(*a));
  a->G = to_mat(grad);
  a->M = to_mat(mom);
  if (nout) a->N = to_mat(nout);
  a->has_n = nout != nullptr;
  a->blocks_per_mat = elementwise_blocks_per_matrix(grad->rows, grad->cols);
  a->rows = static_cast<int32_t>(grad->rows);
  a->cols = static_cast<int32_t>(grad->cols);
  a->cdiv = make_fastdiv(static_cast<uint32_t>(grad->cols));
  a->beta = beta;
  a->nesterov = nesterov;
  *vec = vec_ok(grad) && vec_ok(mom) && (!nout || vec_ok(nout));
  return MUON_OK;
}

muon_status_t check_workspace(void* workspace, size_t ws_bytes, size_t need) {
  if (!workspace || ws_bytes < need)
    return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MUON_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  return MUON_OK;
}

// Checks of one apply batch; fills the kernel arguments.
// The update's factors for an m x n weight: decay = 1 - lr*weight_decay and
// step = lr * s, s from the scale mode ("LLM Optimizers…" section 11.5).
muon_status_t apply_factors(int64_t rows, int64_t cols, float lr, float weight_decay, int32_t mode, float coeff,
                            float* decay, float* step) {
  if (!finite(lr) || !finite(weight_decay) || !finite(coeff))
    return fail(MUON_ERR_INVALID_VALUE, "lr, weight_decay and coeff must be finite");
  const double m = static_cast<double>(rows);
  const double n = static_cast<double>(cols);
  double s;
  switch (mode) {
    case MUON_SCALE_MATCH_RMS: s = static_cast<double>(coeff) * std::sqrt(m > n ? m : n); break;
    case MUON_SCALE_ORIGINAL: s = std::sqrt(m / n > 1.0 ? m / n : 1.0); break;
    case MUON_SCALE_NONE: s = 1.0; break;
    default: return fail(MUON_ERR_INVALID_VALUE, "unknown scale mode %d", mode);
  }
  *decay = static_cast<float>(1.0 - static_cast<double>(lr) * weight_decay);
  *step = static_cast<float>(static_cast<double>(lr) * s);
  return MUON_OK;
}

muon_status_t prepare_apply(const muon_batch_t* weight, const muon_batch_t* ortho, float lr, float weight_decay,
                            int32_t mode, float coeff, ApplyArgs* a, bool* vec) {
  muon_status_t st;
  if ((st = check_batch(weight, "weight", true)) != MUON_OK) return st;
  if ((st = check_batch(ortho, "ortho", true)) != MUON_OK) return st;
  if (!same_shape(weight, ortho)) return fail(MUON_ERR_INVALID_VALUE, "weight and ortho shapes differ");
  float decay, step;
  if ((st = apply_factors(weight->rows, weight->cols, lr, weight_decay, mode, coeff, &decay, &step)) != MUON_OK)
    return st;
  std::memset(a, 0, sizeof(*a));
  a->W = to_mat(weight);
  a->O = to_mat(ortho);
  a->rows = static_cast<int32_t>(weight->rows);
  a->cols = static_cast<int32_t>(weight->cols);
  a->cdiv = make_fastdiv(static_cast<uint32_t>(weight->cols));
  a->decay = decay;
  a->step = step;
  *vec = vec_ok(weight) && vec_ok(ortho);
  return MUON_OK;
}

}  // namespace

extern "C" {

muon_status_t muon_momentum(const muon_batch_t* grad, const muon_batch_t* mom, const muon_batch_t* nout,
                            float* sumsq, float beta, int nesterov, void* workspace, size_t ws_bytes,
                            void* stream) {
  muon_status_t st;
  MomentumArgs a;
  bool vec;
  if ((st = prepare_momentum(grad, mom, nout, sumsq, beta, nesterov, &a, &vec)) != MUON_OK) return st;
  if ((st = check_workspace(workspace, ws_bytes, muon_momentum_workspace(grad->count, grad->rows, grad->cols))) !=
      MUON_OK)
    return st;
  a.partials = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_momentum(a, grad->count, vec, s);
  if (e != hipSuccess) return launch_status(e, "momentum");
  e = launch_sumsq_finalize(a.partials, a.blocks_per_mat, sumsq, grad->count, s);
  if (e != hipSuccess) return launch_status(e, "sumsq finalize");
  return done(s, "muon_momentum");
}

size_t muon_momentum_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows,
                                       const int64_t* cols) {
  if (ngroups < 1 || ngroups > kMaxGroups || !counts || !rows || !cols) return 0;
  size_t total = 0;
  for (int g = 0; g < ngroups; ++g) {
    const size_t w = muon_momentum_workspace(counts[g], rows[g], cols[g]);
    if (w == 0) return 0;
    total += w;
  }
  return total;
}

}  // extern "C"

namespace {

// muon_momentum_grouped and its allocation-free form.  With noalloc the
// workspace arguments are ignored and the partials go to the library's
// static scratch array of the current device, after every check has passed.
muon_status_t momentum_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* moms,
                               const muon_batch_t* nouts, float* const* sumsqs, float beta, int nesterov,
                               void* workspace, size_t ws_bytes, bool noalloc, void* stream, const char* name) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!grads || !moms || !sumsqs) return fail(MUON_ERR_INVALID_VALUE, "grads, moms and sumsqs must not be NULL");
  MomentumGroups G;
  FinalizeGroups F;
  std::memset(&G, 0, sizeof(G));
  std::memset(&F, 0, sizeof(F));
  G.ngroups = F.ngroups = ngroups;
  int64_t counts[kMaxGroups], rows[kMaxGroups], cols[kMaxGroups];
  muon_status_t st;
  for (int g = 0; g < ngroups; ++g) {
    bool vec;
    st = prepare_momentum(&grads[g], &moms[g], nouts ? &nouts[g] : nullptr, sumsqs[g], beta, nesterov, &G.g[g],
                          &vec);
    if (st != MUON_OK) return in_group(st, g);
    G.vec[g] = vec;
    counts[g] = grads[g].count;
    rows[g] = grads[g].rows;
    cols[g] = grads[g].cols;
  }
  const size_t need = muon_momentum_grouped_workspace(ngroups, counts, rows, cols);
  if (noalloc) {
    if (need > MUON_NOALLOC_SCRATCH_BYTES)
      return fail(MUON_ERR_WORKSPACE, "%s: %zu bytes of partial sums needed, the static scratch holds %zu", name,
                  need, static_cast<size_t>(MUON_NOALLOC_SCRATCH_BYTES));
  } else if ((st = check_workspace(workspace, ws_bytes, need)) != MUON_OK) {
    return st;
  }
  char* ws = static_cast<char*>(workspace);
  for (int g = 0; g < ngroups; ++g) {
    const int64_t blocks = counts[g] * G.g[g].blocks_per_mat;
    G.first[g + 1] = G.first[g] + blocks;
  }
  if (G.first[ngroups] > INT32_MAX)
    return fail(MUON_ERR_UNSUPPORTED, "%lld workgroups exceed one launch", (long long)G.first[ngroups]);
  if (noalloc) {
    size_t have = 0;
    void* p = nullptr;
    const hipError_t e = noalloc_scratch(&p, &have);
    if (e != hipSuccess) return launch_status(e, "static scratch lookup");
    if (need > have) return fail(MUON_ERR_WORKSPACE, "%s: static scratch of %zu bytes too small", name, have);
    ws = static_cast<char*>(p);
  }
  for (int g = 0; g < ngroups; ++g) {
    G.g[g].partials = reinterpret_cast<float*>(ws);
    ws += muon_momentum_workspace(counts[g], rows[g], cols[g]);
    F.first[g + 1] = F.first[g] + counts[g];
    F.per[g] = G.g[g].blocks_per_mat;
    F.partials[g] = G.g[g].partials;
    F.sumsq[g] = sumsqs[g];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_momentum_grouped(G, s);
  if (e != hipSuccess) return launch_status(e, "momentum");
  e = launch_sumsq_finalize_grouped(F, s);
  if (e != hipSuccess) return launch_status(e, "sumsq finalize");
  return done(s, name);
}

}  // namespace

extern "C" {

muon_status_t muon_momentum_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* moms,
                                    const muon_batch_t* nouts, float* const* sumsqs, float beta, int nesterov,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return momentum_grouped(ngroups, grads, moms, nouts, sumsqs, beta, nesterov, workspace, ws_bytes, false, stream,
                          "muon_momentum_grouped");
}

muon_status_t muon_momentum_grouped_noalloc(int ngroups, const muon_batch_t* grads, const muon_batch_t* moms,
                                            const muon_batch_t* nouts, float* const* sumsqs, float beta,
                                            int nesterov, void* stream) {
  return momentum_grouped(ngroups, grads, moms, nouts, sumsqs, beta, nesterov, nullptr, 0, true, stream,
                          "muon_momentum_grouped_noalloc");
}

size_t muon_orthogonalize_workspace(int64_t count, int64_t rows, int64_t cols, int32_t compute) {
  Plan plan;
  bool need = true;
  if (!make_plan(1, &count, &rows, &cols, compute, &need, &plan)) return 0;
  return static_cast<size_t>(plan.bytes);
}

size_t muon_orthogonalize_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows,
                                            const int64_t* cols, int32_t compute) {
  if (!counts || !rows || !cols) return 0;
  Plan plan;
  if (!make_plan(ngroups, counts, rows, cols, compute, nullptr, &plan)) return 0;
  return static_cast<size_t>(plan.bytes);
}

muon_status_t muon_orthogonalize(const muon_batch_t* in, const float* sumsq, const muon_batch_t* out, int steps,
                                 float a, float b, float c, float eps, int32_t compute, void* workspace,
                                 size_t ws_bytes, void* stream) {
  const float* s[1] = {sumsq};
  return run_orthogonalize(1, in, s, out, steps, a, b, c, eps, compute, workspace, ws_bytes,
                           static_cast<hipStream_t>(stream));
}

muon_status_t muon_orthogonalize_grouped(int ngroups, const muon_batch_t* ins, const float* const* sumsqs,
                                         const muon_batch_t* outs, int steps, float a, float b, float c,
                                         float eps, int32_t compute, void* workspace, size_t ws_bytes,
                                         void* stream) {
  return run_orthogonalize(ngroups, ins, sumsqs, outs, steps, a, b, c, eps, compute, workspace, ws_bytes,
                           static_cast<hipStream_t>(stream));
}

size_t muon_packed_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows, const int64_t* cols,
                                     int32_t compute) {
  if (!counts || !rows || !cols) return 0;
  Plan plan;
  if (!make_plan(ngroups, counts, rows, cols, compute, nullptr, &plan, true)) return 0;
  return static_cast<size_t>(plan.bytes);
}

muon_status_t muon_momentum_packed_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* moms,
                                           float* const* sumsqs, float beta, int nesterov, int32_t compute,
                                           void* workspace, size_t ws_bytes, void* stream) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!grads || !moms || !sumsqs) return fail(MUON_ERR_INVALID_VALUE, "grads, moms and sumsqs must not be NULL");
  if (compute != MUON_F32 && compute != MUON_BF16)
    return fail(MUON_ERR_INVALID_VALUE, "compute %d is not MUON_F32 or MUON_BF16", compute);
  int64_t counts[kMaxGroups], rows[kMaxGroups], cols[kMaxGroups];
  MomentumArgs ma[kMaxGroups];
  muon_status_t st;
  for (int g = 0; g < ngroups; ++g) {
    bool vec;
    // the checks of muon_momentum without N (the packed buffers take its place)
    st = prepare_momentum(&grads[g], &moms[g], nullptr, sumsqs[g], beta, 0, &ma[g], &vec);
    if (st != MUON_OK) return in_group(st, g);
    if (nesterov != 0 && nesterov != 1) return fail(MUON_ERR_INVALID_VALUE, "nesterov must be 0 or 1");
    counts[g] = grads[g].count;
    rows[g] = grads[g].rows;
    cols[g] = grads[g].cols;
  }
  Plan plan;
  if (!make_plan(ngroups, counts, rows, cols, compute, nullptr, &plan, true))
    return fail(MUON_ERR_UNSUPPORTED, "a padded Newton-Schulz shape exceeds 2^30 elements");
  if ((st = check_workspace(workspace, ws_bytes, static_cast<size_t>(plan.bytes))) != MUON_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const int64_t es = compute == MUON_BF16 ? 2 : 4;
  MomentumPackGroups P;
  FinalizeGroups F;
  std::memset(&P, 0, sizeof(P));
  std::memset(&F, 0, sizeof(F));
  P.ngroups = F.ngroups = ngroups;
  for (int g = 0; g < ngroups; ++g) {
    const GroupPlan& p = plan.g[g];
    const int64_t mn = static_cast<int64_t>(p.Mp) * p.Np;
    MomentumPackArgs& a = P.g[g];
    a.G = to_mat(&grads[g]);
    a.M = to_mat(&moms[g]);
    a.beta = beta;
    a.nesterov = nesterov;
    a.rows = p.rows;
    a.cols = p.cols;
    a.Pr = p.Pr;
    a.Pc = p.Pc;
    a.compute = compute;
    a.tall = p.tall;
    a.vec = vec4_ok(&grads[g]) && vec4_ok(&moms[g]);
    a.tiles_c = p.Pc / 64;
    a.tiles_per_mat = p.pack_tiles;
    a.lo_bm = p.tile;
    a.lo_tiles_n = p.Np / p.tile;
    a.partials = reinterpret_cast<float*>(ws + p.partials);
    // the same buffers as the pack step of run_orthogonalize: X is whichever
    // orientation is wide, X^T only where the update reads it
    a.S = p.tall ? (p.kmajor ? nullptr : ws + p.xt[0]) : ws + p.xc[0];
    a.T = p.tall ? ws + p.xc[0] : (p.kmajor ? nullptr : ws + p.xt[0]);
    a.s_mat = a.t_mat = mn * es;
    a.Lo = compute == MUON_BF16 ? reinterpret_cast<int8_t*>(ws + p.xlo) : nullptr;
    a.lo_mat = mn;
    a.LoE = compute == MUON_BF16 ? reinterpret_cast<uint8_t*>(ws + p.xloe) : nullptr;
    a.loe_mat = mn / kLoExpPerCodes;
    P.first[g + 1] = P.first[g] + counts[g] * p.pack_tiles;
    F.first[g + 1] = F.first[g] + counts[g];
    F.per[g] = p.pack_tiles;
    F.partials[g] = a.partials;
    F.sumsq[g] = sumsqs[g];
  }
  if (P.first[ngroups] > INT32_MAX)
    return fail(MUON_ERR_UNSUPPORTED, "%lld workgroups exceed one launch", (long long)P.first[ngroups]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_momentum_pack_grouped(P, s);
  if (e != hipSuccess) return launch_status(e, "momentum pack");
  e = launch_sumsq_finalize_grouped(F, s);
  if (e != hipSuccess) return launch_status(e, "sumsq finalize");
  return done(s, "muon_momentum_packed_grouped");
}

muon_status_t muon_orthogonalize_packed_grouped(int ngroups, const float* const* sumsqs, const muon_batch_t* outs,
                                                int steps, float a, float b, float c, float eps, int32_t compute,
                                                void* workspace, size_t ws_bytes, void* stream) {
  return run_orthogonalize(ngroups, nullptr, sumsqs, outs, steps, a, b, c, eps, compute, workspace, ws_bytes,
                           static_cast<hipStream_t>(stream), true);
}

muon_status_t muon_orthogonalize_apply_packed_grouped(int ngroups, const float* const* sumsqs,
                                                      const muon_batch_t* weights, int steps, float a, float b,
                                                      float c, float eps, float lr, float weight_decay, int32_t mode,
                                                      float coeff, int32_t compute, void* workspace, size_t ws_bytes,
                                                      void* stream) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!weights) return fail(MUON_ERR_INVALID_VALUE, "weights is NULL");
  float decay[kMaxGroups], step[kMaxGroups];
  for (int g = 0; g < ngroups; ++g) {
    muon_status_t st = check_batch(&weights[g], "weight", true);
    if (st == MUON_OK)
      st = apply_factors(weights[g].rows, weights[g].cols, lr, weight_decay, mode, coeff, &decay[g], &step[g]);
    if (st != MUON_OK) return in_group(st, g);
  }
  return run_orthogonalize(ngroups, nullptr, sumsqs, weights, steps, a, b, c, eps, compute, workspace, ws_bytes,
                           static_cast<hipStream_t>(stream), true, decay, step);
}

muon_status_t muon_apply(const muon_batch_t* weight, const muon_batch_t* ortho, float lr, float weight_decay,
                         int32_t mode, float coeff, void* stream) {
  muon_status_t st;
  ApplyArgs a;
  bool vec;
  if ((st = prepare_apply(weight, ortho, lr, weight_decay, mode, coeff, &a, &vec)) != MUON_OK) return st;
  hipError_t e = launch_apply(a, weight->count, vec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return launch_status(e, "apply");
  return done(static_cast<hipStream_t>(stream), "muon_apply");
}

muon_status_t muon_apply_grouped(int ngroups, const muon_batch_t* weights, const muon_batch_t* orthos, float lr,
                                 float weight_decay, int32_t mode, float coeff, void* stream) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!weights || !orthos) return fail(MUON_ERR_INVALID_VALUE, "weights and orthos must not be NULL");
  ApplyGroups G;
  std::memset(&G, 0, sizeof(G));
  G.ngroups = ngroups;
  for (int g = 0; g < ngroups; ++g) {
    bool vec;
    const muon_status_t st = prepare_apply(&weights[g], &orthos[g], lr, weight_decay, mode, coeff, &G.g[g], &vec);
    if (st != MUON_OK) return in_group(st, g);
    G.vec[g] = vec;
    G.blocks_per_mat[g] = elementwise_blocks_per_matrix(weights[g].rows, weights[g].cols);
    G.first[g + 1] = G.first[g] + weights[g].count * G.blocks_per_mat[g];
  }
  if (G.first[ngroups] > INT32_MAX)
    return fail(MUON_ERR_UNSUPPORTED, "%lld workgroups exceed one launch", (long long)G.first[ngroups]);
  hipError_t e = launch_apply_grouped(G, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return launch_status(e, "apply");
  return done(static_cast<hipStream_t>(stream), "muon_apply_grouped");
}

}  // extern "C"

// ------------------------------------------------------------------ SOAP
//
// Adam in the eigenbasis of Shampoo's statistics ("LLM Optimizers: From SGD
// and AdamW to SOAP, Muon, and Scalable Training", sections 11.1-11.2;
// "初探优化器（一）：从SGD到SOAP-Muon", section 6.2), on the fp32 products,
// the blocked Householder QR and the rotated-Adam kernel of soap.hip.

namespace {

constexpr int64_t kQrMaxDim = 32768;
constexpr int kMaxSplits = 16;

int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }

// Floats of one panel's reflector slot: kQrPanel columns of n rows,
// column-major with column pitch n and absolute row indices.  The slots of
// one matrix are contiguous, so the reflectors of an outer block form one
// (block width) x n matrix with leading dimension n.
int64_t qr_vslot(int64_t n) { return int64_t{kQrPanel} * n; }

// Per-matrix float offsets of the QR scratch for an n x n factorization.
struct QrLayout {
  int64_t V, Q, W, W2, TT, TQ, Y, sgn, tau, total;
};

QrLayout qr_layout(int64_t n) {
  const int64_t panels = (n + kQrPanel - 1) / kQrPanel;
  const int64_t blocks = (n + kQrOuter - 1) / kQrOuter;
  QrLayout L;
  int64_t o = 0;
  L.V = o;   o += round64(panels * qr_vslot(n));
  L.Q = o;   o += round64(n * n);
  L.W = o;   o += round64(int64_t{kMaxSplits} * kQrOuter * n);
  L.W2 = o;  o += round64(int64_t{kQrOuter} * n);
  L.TT = o;  o += round64(int64_t{kQrOuter} * kQrOuter * kMaxSplits);
  L.TQ = o;  o += blocks * round64(int64_t{kQrOuter} * kQrOuter * kMaxSplits);
  L.Y = o;   o += round64(int64_t{kQrOuter} * kQrOuter);
  L.sgn = o; o += round64(n);
  L.tau = o; o += round64(n);
  L.total = o;
  return L;
}

// Split-K plan for a reduction of length K over `tiles` output tiles of
// `count` matrices: enough splits for about 512 workgroups, each split at
// least 64 deep, a multiple of the k-slice depth.
int plan_splits(int64_t K, int64_t tiles, int64_t count, int* ksplit) {
  int64_t want = (512 + tiles * count - 1) / (tiles * count);
  want = std::min<int64_t>(want, kMaxSplits);
  want = std::min<int64_t>(want, std::max<int64_t>(1, K / 64));
  want = std::min<int64_t>(want, std::max<int64_t>(1, 65535 / count));
  want = std::max<int64_t>(want, 1);
  int64_t ks = (K + want - 1) / want;
  ks = (ks + kSgemmBK - 1) / kSgemmBK * kSgemmBK;
  *ksplit = static_cast<int>(std::max<int64_t>(ks, 1));
  return static_cast<int>(std::max<int64_t>(1, (K + *ksplit - 1) / *ksplit));
}

SgemmOperand op_batch(const muon_batch_t* b, bool kcontig) {
  SgemmOperand o;
  std::memset(&o, 0, sizeof(o));
  o.base = static_cast<const char*>(b->base);
  o.stride = b->stride * esize(b->dtype);
  o.ptrs = b->ptrs;
  o.ld = b->ld;
  o.dtype = b->dtype == MUON_BF16 ? 1 : 0;
  o.kcontig = kcontig;
  o.vec = vec4_ok(b);
  return o;
}

SgemmOperand op_ws(const float* base, int64_t mat, int64_t ld, bool kcontig, int64_t off = 0) {
  SgemmOperand o;
  std::memset(&o, 0, sizeof(o));
  o.base = reinterpret_cast<const char*>(base);
  o.stride = mat * 4;
  o.off = off * 4;
  o.ld = ld;
  o.kcontig = kcontig;
  o.vec = ld % 4 == 0 && off % 4 == 0 && mat % 4 == 0;
  return o;
}

struct COut {
  char* c;
  int64_t stride;
  void* const* ptrs;
  int64_t off;
  int64_t ld;
};

COut out_batch(const muon_batch_t* b) {
  return COut{static_cast<char*>(b->base), b->stride * 4, b->ptrs, 0, b->ld};
}

COut out_ws(float* base, int64_t mat, int64_t ld, int64_t off = 0) {
  return COut{reinterpret_cast<char*>(base), mat * 4, nullptr, off * 4, ld};
}

SgemmArgs gemm_args(const SgemmOperand& A, const SgemmOperand& B, const COut& C, int64_t M, int64_t N, int64_t K,
                    int64_t count, float alpha, float beta, bool sym, int splits = 1, int ksplit = 0,
                    int64_t c_split_floats = 0) {
  SgemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.a = A;
  g.b = B;
  g.c = C.c;
  g.c_stride = C.stride;
  g.c_ptrs = C.ptrs;
  g.c_off = C.off;
  g.ldc = C.ld;
  g.c_split = c_split_floats * 4;
  g.M = static_cast<int32_t>(M);
  g.N = static_cast<int32_t>(N);
  g.K = static_cast<int32_t>(K);
  g.splits = splits;
  g.ksplit = splits > 1 ? ksplit : static_cast<int32_t>(std::max<int64_t>(K, 1));
  g.count = static_cast<int32_t>(count);
  g.alpha = alpha;
  g.beta = beta;
  g.sym = sym;
  return g;
}

hipError_t gemm(const SgemmOperand& A, const SgemmOperand& B, const COut& C, int64_t M, int64_t N, int64_t K,
                int64_t count, float alpha, float beta, bool sym, hipStream_t s, int splits = 1, int ksplit = 0,
                int64_t c_split_floats = 0) {
  if (M == 0 || N == 0) return hipSuccess;
  return launch_sgemm(gemm_args(A, B, C, M, N, K, count, alpha, beta, sym, splits, ksplit, c_split_floats), s);
}

#define SOAP_TRY(expr, what)                                  \
  do {                                                        \
    const hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return launch_status(e_, what);     \
  } while (0)

// Where a batched QR's Q factors go: matrices first .. first+count-1 of the
// batch into the caller's batch q.
struct QrOut {
  const muon_batch_t* q;
  int64_t first, count;
};

// Q factor (R's diagonal made non-negative) of the n x n matrices in P
// (contiguous, p_mat floats apart; overwritten), written to the outputs.
// Two-level blocked Householder QR in the compact WY form I - V T V^T:
//  - each 128-column outer block is reduced 16 columns at a time by the
//    panel kernel, each panel's reflectors applied at once to the rest of
//    the block (W = V^T A_blk, W2 = T^T W, A_blk -= V W2);
//  - the block's factor T comes from the Gram matrix of its reflectors, and
//    the trailing matrix is updated once per block: W = V^T A_t (split over
//    the reduction), W2 = [T^T ... T^T] [W_0; ...], A_t -= V W2;
//  - Q is formed from the identity, last block first: Q_t -= V (T (V^T Q_t)).
// V is kept transposed (rows are reflectors), so V^T X is the product of the
// k-contiguous operand V with X.
muon_status_t qr_enqueue(float* P, int64_t p_mat, int64_t n, int64_t count, float* ws, const QrOut* outs, int nouts,
                         hipStream_t s) {
  const QrLayout L = qr_layout(n);
  const int64_t vslot = qr_vslot(n);
  const int64_t tslot = round64(int64_t{kQrOuter} * kQrOuter * kMaxSplits);
  auto ntiles = [](int64_t x) { return (x + kSgemmTile - 1) / kSgemmTile; };
  for (int64_t c0o = 0; c0o < n; c0o += kQrOuter) {
    const int64_t bw = std::min<int64_t>(kQrOuter, n - c0o), ho = n - c0o, nto = ho - bw;
    float* Vo = ws + L.V + (c0o / kQrPanel) * vslot;  // the block's reflectors, bw x n
    for (int64_t c1 = c0o; c1 < c0o + bw; c1 += kQrPanel) {
      const int64_t nb = std::min<int64_t>(kQrPanel, n - c1), h = n - c1, w = c0o + bw - c1 - nb;
      int ks = 0;
      const int si = w > 0 ? plan_splits(h, ntiles(w), count, &ks) : 1;
      float* Vp = ws + L.V + (c1 / kQrPanel) * vslot;
      QrPanelArgs a;
      std::memset(&a, 0, sizeof(a));
      a.A = P;
      a.a_mat = p_mat;
      a.V = Vp + c1;
      a.v_mat = L.total;
      a.TrepT = ws + L.TT;
      a.tT_mat = L.total;
      a.TrepQ = ws + L.TT;  // not written: reps_q = 0
      a.tQ_mat = L.total;
      a.sgn = ws + L.sgn;
      a.tau = ws + L.tau;
      a.s_mat = L.total;
      a.n = static_cast<int32_t>(n);
      a.c0 = static_cast<int32_t>(c1);
      a.reps_t = si;
      a.reps_q = 0;
      a.zpre = static_cast<int32_t>(c1 - c0o);
      SOAP_TRY(launch_qr_panel(a, count, s), "qr panel");
      if (w > 0) {
        const int64_t ao = c1 * n + c1 + nb;
        SOAP_TRY(gemm(op_ws(Vp, L.total, n, true, c1), op_ws(P, p_mat, n, false, ao), out_ws(ws + L.W, L.total, w), nb,
                      w, h, count, 1.f, 0.f, false, s, si, ks, nb * w),
                 "qr panel update product");
        SOAP_TRY(gemm(op_ws(ws + L.TT, L.total, nb * si, true), op_ws(ws + L.W, L.total, w, false),
                      out_ws(ws + L.W2, L.total, w), nb, w, nb * si, count, 1.f, 0.f, false, s),
                 "qr panel update factor");
        SOAP_TRY(gemm(op_ws(Vp, L.total, n, false, c1), op_ws(ws + L.W2, L.total, w, false),
                      out_ws(P, p_mat, n, ao), h, w, nb, count, -1.f, 1.f, false, s),
                 "qr panel update");
      }
    }
    int ks_o = 0, ks_q = 0;
    const int so = nto > 0 ? plan_splits(ho, ntiles(nto), count, &ks_o) : 1;
    const int sq = plan_splits(ho, ntiles(ho), count, &ks_q);
    SOAP_TRY(gemm(op_ws(Vo, L.total, n, true, c0o), op_ws(Vo, L.total, n, true, c0o), out_ws(ws + L.Y, L.total, bw),
                  bw, bw, ho, count, 1.f, 0.f, true, s),
             "qr block gram");
    QrTArgs t;
    std::memset(&t, 0, sizeof(t));
    t.Y = ws + L.Y;
    t.y_mat = L.total;
    t.tau = ws + L.tau + c0o;
    t.s_mat = L.total;
    t.TrepT = ws + L.TT;
    t.tT_mat = L.total;
    t.TrepQ = ws + L.TQ + (c0o / kQrOuter) * tslot;
    t.tQ_mat = L.total;
    t.bw = static_cast<int32_t>(bw);
    t.reps_t = so;
    t.reps_q = sq;
    SOAP_TRY(launch_qr_tfactor(t, count, s), "qr block factor");
    if (nto > 0) {
      const int64_t ao = c0o * n + c0o + bw;
      SOAP_TRY(gemm(op_ws(Vo, L.total, n, true, c0o), op_ws(P, p_mat, n, false, ao), out_ws(ws + L.W, L.total, nto),
                    bw, nto, ho, count, 1.f, 0.f, false, s, so, ks_o, bw * nto),
               "qr trailing product");
      SOAP_TRY(gemm(op_ws(ws + L.TT, L.total, bw * so, true), op_ws(ws + L.W, L.total, nto, false),
                    out_ws(ws + L.W2, L.total, nto), bw, nto, bw * so, count, 1.f, 0.f, false, s),
               "qr trailing factor");
      SOAP_TRY(gemm(op_ws(Vo, L.total, n, false, c0o), op_ws(ws + L.W2, L.total, nto, false),
                    out_ws(P, p_mat, n, ao), ho, nto, bw, count, -1.f, 1.f, false, s),
               "qr trailing update");
    }
  }
  SOAP_TRY(launch_eye(ws + L.Q, L.total, static_cast<int32_t>(n), count, s), "qr identity");
  for (int64_t c0o = (n - 1) / kQrOuter * kQrOuter; c0o >= 0; c0o -= kQrOuter) {
    const int64_t bw = std::min<int64_t>(kQrOuter, n - c0o), ho = n - c0o;
    int ks_q = 0;
    const int sq = plan_splits(ho, ntiles(ho), count, &ks_q);
    const int64_t qo = c0o * n + c0o;
    float* Vo = ws + L.V + (c0o / kQrPanel) * vslot;
    SOAP_TRY(gemm(op_ws(Vo, L.total, n, true, c0o), op_ws(ws + L.Q, L.total, n, false, qo),
                  out_ws(ws + L.W, L.total, ho), bw, ho, ho, count, 1.f, 0.f, false, s, sq, ks_q, bw * ho),
             "qr formation product");
    SOAP_TRY(gemm(op_ws(ws + L.TQ + (c0o / kQrOuter) * tslot, L.total, bw * sq, true),
                  op_ws(ws + L.W, L.total, ho, false), out_ws(ws + L.W2, L.total, ho), bw, ho, bw * sq, count, 1.f,
                  0.f, false, s),
             "qr formation factor");
    SOAP_TRY(gemm(op_ws(Vo, L.total, n, false, c0o), op_ws(ws + L.W2, L.total, ho, false),
                  out_ws(ws + L.Q, L.total, n, qo), ho, ho, bw, count, -1.f, 1.f, false, s),
             "qr formation update");
  }
  for (int o = 0; o < nouts; ++o)
    SOAP_TRY(launch_sign_copy(ws + L.Q + outs[o].first * L.total, L.total, ws + L.sgn + outs[o].first * L.total,
                              L.total, to_mat(outs[o].q), static_cast<int32_t>(n), outs[o].count, s),
             "qr signs");
  return MUON_OK;
}

muon_status_t check_f32(const muon_batch_t* b, const char* name, int64_t count, int64_t rows, int64_t cols) {
  muon_status_t st;
  if ((st = check_batch(b, name, false)) != MUON_OK) return st;
  if (b->count != count || b->rows != rows || b->cols != cols)
    return fail(MUON_ERR_INVALID_VALUE, "%s: %lld x (%lld x %lld) given, %lld x (%lld x %lld) expected", name,
                (long long)b->count, (long long)b->rows, (long long)b->cols, (long long)count, (long long)rows,
                (long long)cols);
  return MUON_OK;
}

size_t qr_bytes(int64_t count, int64_t n) {
  return static_cast<size_t>(count * (round64(n * n) + qr_layout(n).total) * 4);
}

// soap_statistics and soap_statistics_grouped: every group is checked before
// anything is enqueued; `grouped` names the group in error messages.
muon_status_t statistics(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* Ls,
                         const muon_batch_t* const* Rs, float beta_s, void* stream, bool grouped) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!grads || !Ls || !Rs) return fail(MUON_ERR_INVALID_VALUE, "the per-group arrays must not be NULL");
  if (!(beta_s >= 0.f && beta_s < 1.f)) return fail(MUON_ERR_INVALID_VALUE, "beta_s %g outside [0, 1)", beta_s);
  auto tag = [&](muon_status_t st, int g) { return grouped ? in_group(st, g) : st; };
  muon_status_t st;
  for (int g = 0; g < ngroups; ++g) {
    const muon_batch_t* grad = &grads[g];
    if ((st = check_batch(grad, "grad", true)) != MUON_OK) return tag(st, g);
    const int64_t c = grad->count, m = grad->rows, n = grad->cols;
    if (Ls[g] && (st = check_f32(Ls[g], "L", c, m, m)) != MUON_OK) return tag(st, g);
    if (Rs[g] && (st = check_f32(Rs[g], "R", c, n, n)) != MUON_OK) return tag(st, g);
  }
  // L <- b L + (1-b) G G^T, R <- b R + (1-b) G^T G, upper tiles mirrored;
  // all of them in as few launches as their operand layouts allow
  SgemmArgs gs[2 * kMaxGroups];
  int np = 0;
  for (int g = 0; g < ngroups; ++g) {
    const muon_batch_t* grad = &grads[g];
    const int64_t c = grad->count, m = grad->rows, n = grad->cols;
    if (Ls[g])
      gs[np++] = gemm_args(op_batch(grad, true), op_batch(grad, true), out_batch(Ls[g]), m, m, n, c, 1.f - beta_s,
                           beta_s, true);
    if (Rs[g])
      gs[np++] = gemm_args(op_batch(grad, false), op_batch(grad, false), out_batch(Rs[g]), n, n, m, c, 1.f - beta_s,
                           beta_s, true);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (np > 0) SOAP_TRY(launch_sgemm_list(gs, np, s), "statistics");
  return done(s, grouped ? "soap_statistics_grouped" : "soap_statistics");
}


// soap_precondition and soap_precondition_grouped.  Per group, with
// temporaries w1, w2 (m x n each) at the group's place in the workspace:
//   Gbar = QL^T G QR (a side without a basis skipped), Dbar = Adam's
//   direction in the rotated basis, D = QL Dbar QR^T.
// Every rotation stage launches the products of all groups together.
muon_status_t precondition(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* QLs,
                           const muon_batch_t* const* QRs, const muon_batch_t* mbars, const muon_batch_t* vbars,
                           const muon_batch_t* dirs, int64_t step, float beta1, float beta2, float eps,
                           void* workspace, size_t ws_bytes, void* stream, bool grouped) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!grads || !QLs || !QRs || !mbars || !vbars || !dirs)
    return fail(MUON_ERR_INVALID_VALUE, "the per-group arrays must not be NULL");
  auto tag = [&](muon_status_t st, int g) { return grouped ? in_group(st, g) : st; };
  muon_status_t st;
  int64_t counts[kMaxGroups], rows[kMaxGroups], cols[kMaxGroups];
  for (int g = 0; g < ngroups; ++g) {
    const muon_batch_t* grad = &grads[g];
    if ((st = check_batch(grad, "grad", true)) != MUON_OK) return tag(st, g);
    const int64_t c = grad->count, m = grad->rows, n = grad->cols;
    if (QLs[g] && (st = check_f32(QLs[g], "QL", c, m, m)) != MUON_OK) return tag(st, g);
    if (QRs[g] && (st = check_f32(QRs[g], "QR", c, n, n)) != MUON_OK) return tag(st, g);
    if ((st = check_f32(&mbars[g], "mbar", c, m, n)) != MUON_OK) return tag(st, g);
    if ((st = check_f32(&vbars[g], "vbar", c, m, n)) != MUON_OK) return tag(st, g);
    if ((st = check_f32(&dirs[g], "dir", c, m, n)) != MUON_OK) return tag(st, g);
    counts[g] = c;
    rows[g] = m;
    cols[g] = n;
  }
  if (step < 1) return fail(MUON_ERR_INVALID_VALUE, "step %lld < 1", (long long)step);
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f))
    return fail(MUON_ERR_INVALID_VALUE, "betas must lie in [0, 1)");
  if (!(finite(eps) && eps >= 0.f)) return fail(MUON_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  const size_t need = soap_precondition_grouped_workspace(ngroups, counts, rows, cols);
  if (need == 0) return fail(MUON_ERR_UNSUPPORTED, "sizes outside the supported range");
  if ((st = check_workspace(workspace, ws_bytes, need)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  float* w1[kMaxGroups];
  float* w2[kMaxGroups];
  int64_t wm[kMaxGroups];
  float* cur = static_cast<float*>(workspace);
  for (int g = 0; g < ngroups; ++g) {
    wm[g] = round64(rows[g] * cols[g]);
    w1[g] = cur;
    w2[g] = cur + counts[g] * wm[g];
    cur += 2 * counts[g] * wm[g];
  }
  SgemmArgs gs[kMaxGroups];
  int np = 0;
  auto flush = [&](const char* what) -> muon_status_t {
    if (np > 0) {
      const hipError_t e = launch_sgemm_list(gs, np, s);
      np = 0;
      if (e != hipSuccess) return launch_status(e, what);
    }
    return MUON_OK;
  };
  // Gbar: the left rotation (or the right one alone) ...
  for (int g = 0; g < ngroups; ++g) {
    const muon_batch_t* grad = &grads[g];
    const int64_t c = counts[g], m = rows[g], n = cols[g];
    if (QLs[g])
      gs[np++] = gemm_args(op_batch(QLs[g], false), op_batch(grad, false), out_ws(QRs[g] ? w1[g] : w2[g], wm[g], n),
                           m, n, m, c, 1.f, 0.f, false);
    else if (QRs[g])
      gs[np++] = gemm_args(op_batch(grad, true), op_batch(QRs[g], false), out_ws(w2[g], wm[g], n), m, n, n, c, 1.f,
                           0.f, false);
  }
  if ((st = flush("rotate in")) != MUON_OK) return st;
  // ... then the right rotation of the two-sided groups
  for (int g = 0; g < ngroups; ++g)
    if (QLs[g] && QRs[g])
      gs[np++] = gemm_args(op_ws(w1[g], wm[g], cols[g], true), op_batch(QRs[g], false), out_ws(w2[g], wm[g], cols[g]),
                           rows[g], cols[g], cols[g], counts[g], 1.f, 0.f, false);
  if ((st = flush("rotate in, right")) != MUON_OK) return st;
  // Adam in the rotated basis: Dbar into w2 (in place over Gbar), or into
  // dir when both bases are the identity
  const float c1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step))));
  const float c2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step))));
  for (int g = 0; g < ngroups; ++g) {
    const bool rot = QLs[g] || QRs[g];
    const MatBatch tmp{reinterpret_cast<char*>(w2[g]), wm[g] * 4, nullptr, cols[g], MUON_F32, 0};
    RotAdamArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    ra.G = rot ? tmp : to_mat(&grads[g]);
    ra.M = to_mat(&mbars[g]);
    ra.V = to_mat(&vbars[g]);
    ra.out = rot ? tmp : to_mat(&dirs[g]);
    ra.rows = static_cast<int32_t>(rows[g]);
    ra.cols = static_cast<int32_t>(cols[g]);
    ra.beta1 = beta1;
    ra.beta2 = beta2;
    ra.eps = eps;
    ra.c1 = c1;
    ra.c2 = c2;
    SOAP_TRY(launch_rot_adam(ra, counts[g], s), "rotated adam");
  }
  // D = QL Dbar QR^T: the left rotation back (or the right one alone) ...
  for (int g = 0; g < ngroups; ++g) {
    const int64_t c = counts[g], m = rows[g], n = cols[g];
    if (QLs[g])
      gs[np++] = gemm_args(op_batch(QLs[g], true), op_ws(w2[g], wm[g], n, false),
                           QRs[g] ? out_ws(w1[g], wm[g], n) : out_batch(&dirs[g]), m, n, m, c, 1.f, 0.f, false);
    else if (QRs[g])
      gs[np++] = gemm_args(op_ws(w2[g], wm[g], n, true), op_batch(QRs[g], true), out_batch(&dirs[g]), m, n, n, c,
                           1.f, 0.f, false);
  }
  if ((st = flush("rotate back")) != MUON_OK) return st;
  // ... then the right rotation back of the two-sided groups
  for (int g = 0; g < ngroups; ++g)
    if (QLs[g] && QRs[g])
      gs[np++] = gemm_args(op_ws(w1[g], wm[g], cols[g], true), op_batch(QRs[g], true), out_batch(&dirs[g]), rows[g],
                           cols[g], cols[g], counts[g], 1.f, 0.f, false);
  if ((st = flush("rotate back, right")) != MUON_OK) return st;
  return done(s, grouped ? "soap_precondition_grouped" : "soap_precondition");
}

}  // namespace

extern "C" {

size_t soap_qr_workspace(int64_t count, int64_t n) {
  if (count < 1 || count > 65535 || n < 1 || n > kQrMaxDim) return 0;
  return qr_bytes(count, n);
}

muon_status_t soap_qr(const muon_batch_t* a, const muon_batch_t* q, void* workspace, size_t ws_bytes,
                      void* stream) {
  muon_status_t st;
  if ((st = check_batch(a, "a", false)) != MUON_OK) return st;
  if (a->rows != a->cols) return fail(MUON_ERR_INVALID_VALUE, "a: must be square");
  if (a->rows > kQrMaxDim) return fail(MUON_ERR_UNSUPPORTED, "a: order above %lld", (long long)kQrMaxDim);
  if ((st = check_f32(q, "q", a->count, a->rows, a->cols)) != MUON_OK) return st;
  const int64_t n = a->rows;
  if ((st = check_workspace(workspace, ws_bytes, soap_qr_workspace(a->count, n))) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* P = static_cast<float*>(workspace);
  float* ws = P + a->count * round64(n * n);
  SOAP_TRY(launch_gather(to_mat(a), P, round64(n * n), static_cast<int32_t>(n), static_cast<int32_t>(n), a->count,
                         s),
           "qr input");
  const QrOut out{q, 0, a->count};
  if ((st = qr_enqueue(P, round64(n * n), n, a->count, ws, &out, 1, s)) != MUON_OK) return st;
  return done(s, "soap_qr");
}

muon_status_t soap_statistics(const muon_batch_t* grad, const muon_batch_t* L, const muon_batch_t* R, float beta_s,
                              void* stream) {
  if (!grad) return fail(MUON_ERR_INVALID_VALUE, "grad: descriptor is NULL");
  return statistics(1, grad, &L, &R, beta_s, stream, false);
}

muon_status_t soap_statistics_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* Ls,
                                      const muon_batch_t* const* Rs, float beta_s, void* stream) {
  return statistics(ngroups, grads, Ls, Rs, beta_s, stream, true);
}

size_t soap_refresh_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows, const int64_t* cols,
                                      const int* with_l, const int* with_r) {
  if (ngroups < 1 || ngroups > kMaxGroups || !counts || !rows || !cols || !with_l || !with_r) return 0;
  int64_t tmp = 0;
  std::vector<std::pair<int64_t, int64_t>> dims;  // (order, matrices of that order)
  for (int g = 0; g < ngroups; ++g) {
    const int64_t c = counts[g], m = rows[g], n = cols[g];
    if (c < 1 || c > 65535 || m < 1 || n < 1 || m > kMaxElems / n) return 0;
    if ((with_l[g] && m > kQrMaxDim) || (with_r[g] && n > kQrMaxDim)) return 0;
    tmp += 2 * c * round64(m * n);
    for (int side = 0; side < 2; ++side) {
      if (!(side ? with_r[g] : with_l[g])) continue;
      const int64_t d = side ? n : m;
      auto it = std::find_if(dims.begin(), dims.end(), [d](const std::pair<int64_t, int64_t>& x) { return x.first == d; });
      if (it == dims.end()) dims.emplace_back(d, c); else it->second += c;
    }
  }
  size_t side = 0;
  for (const auto& d : dims) {
    if (d.second > 65535) return 0;
    side = std::max(side, qr_bytes(d.second, d.first));
  }
  return side + static_cast<size_t>(tmp * 4);
}

size_t soap_refresh_workspace(int64_t count, int64_t rows, int64_t cols, int with_l, int with_r) {
  return soap_refresh_grouped_workspace(1, &count, &rows, &cols, &with_l, &with_r);
}

muon_status_t soap_refresh_grouped(int ngroups, const muon_batch_t* const* Ls, const muon_batch_t* const* Rs,
                                   const muon_batch_t* const* QLs, const muon_batch_t* const* QRs,
                                   const muon_batch_t* mbars, void* workspace, size_t ws_bytes, void* stream) {
  if (ngroups < 1 || ngroups > kMaxGroups)
    return fail(MUON_ERR_INVALID_VALUE, "ngroups %d outside [1, %d]", ngroups, kMaxGroups);
  if (!Ls || !Rs || !QLs || !QRs || !mbars)
    return fail(MUON_ERR_INVALID_VALUE, "the per-group arrays must not be NULL");
  muon_status_t st;
  int64_t counts[kMaxGroups], rows[kMaxGroups], cols[kMaxGroups];
  int wl[kMaxGroups], wr[kMaxGroups];
  for (int g = 0; g < ngroups; ++g) {
    const muon_batch_t* mb = &mbars[g];
    if ((st = check_batch(mb, "mbar", false)) != MUON_OK) return in_group(st, g);
    const int64_t c = mb->count, m = mb->rows, n = mb->cols;
    if (!Ls[g] != !QLs[g] || !Rs[g] != !QRs[g])
      return in_group(fail(MUON_ERR_INVALID_VALUE, "a statistic and its basis come together"), g);
    if (Ls[g] && ((st = check_f32(Ls[g], "L", c, m, m)) != MUON_OK || (st = check_f32(QLs[g], "QL", c, m, m)) != MUON_OK))
      return in_group(st, g);
    if (Rs[g] && ((st = check_f32(Rs[g], "R", c, n, n)) != MUON_OK || (st = check_f32(QRs[g], "QR", c, n, n)) != MUON_OK))
      return in_group(st, g);
    counts[g] = c;
    rows[g] = m;
    cols[g] = n;
    wl[g] = Ls[g] != nullptr;
    wr[g] = Rs[g] != nullptr;
  }
  const size_t need = soap_refresh_grouped_workspace(ngroups, counts, rows, cols, wl, wr);
  if (need == 0) return fail(MUON_ERR_UNSUPPORTED, "refresh sizes outside the supported range");
  if ((st = check_workspace(workspace, ws_bytes, need)) != MUON_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // two m x n temporaries per group for the first moment, then the region
  // of the QR batch of each distinct order, reused order after order
  float* t1[kMaxGroups];
  float* t2[kMaxGroups];
  float* cur = static_cast<float*>(workspace);
  for (int g = 0; g < ngroups; ++g) {
    const int64_t tm = round64(rows[g] * cols[g]);
    t1[g] = cur;
    t2[g] = cur + counts[g] * tm;
    cur += 2 * counts[g] * tm;
  }
  float* region = cur;
  std::vector<int64_t> orders;
  for (int g = 0; g < ngroups; ++g) {
    if (wl[g] && std::find(orders.begin(), orders.end(), rows[g]) == orders.end()) orders.push_back(rows[g]);
    if (wr[g] && std::find(orders.begin(), orders.end(), cols[g]) == orders.end()) orders.push_back(cols[g]);
  }
  for (const int64_t d : orders) {
    const int64_t pm = round64(d * d);
    int64_t total = 0;
    for (int g = 0; g < ngroups; ++g) total += counts[g] * ((wl[g] && rows[g] == d) + (wr[g] && cols[g] == d));
    float* P = region;
    float* qws = P + total * pm;
    QrOut outs[2 * kMaxGroups];
    int nouts = 0;
    int64_t first = 0;
    // power-iteration products and the first moment in the old bases:
    // t1 = QL_old mbar, or mbar QR_old^T, or (both sides of this order) t2 = QL_old mbar QR_old^T.
    // A group with one side whose other axis is longer (ql / qr) instead
    // keeps mbar (t1) and the old basis (t2), and carries mbar through the
    // small product C = QL_new^T QL_old (or QR_old^T QR_new) after the QR:
    // 2 d^3 + 2 m n d flops instead of 4 m n d.
    int64_t slot[kMaxGroups];
    for (int g = 0; g < ngroups; ++g) {
      const int64_t c = counts[g], m = rows[g], n = cols[g], tm = round64(m * n);
      const bool l = wl[g] && m == d, r = wr[g] && n == d;
      const bool ql = l && !wr[g] && n > m, qr = r && !wl[g] && m > n;
      if (ql || qr) {
        SOAP_TRY(launch_gather(to_mat(&mbars[g]), t1[g], tm, static_cast<int32_t>(m), static_cast<int32_t>(n), c, s),
                 "refresh moment copy");
        SOAP_TRY(launch_gather(to_mat(ql ? QLs[g] : QRs[g]), t2[g], tm, static_cast<int32_t>(d),
                               static_cast<int32_t>(d), c, s),
                 "refresh old basis copy");
      }
      if (l) {
        SOAP_TRY(gemm(op_batch(Ls[g], true), op_batch(QLs[g], false), out_ws(P + first * pm, pm, m), m, m, m, c, 1.f,
                      0.f, false, s),
                 "refresh power step L");
        outs[nouts++] = QrOut{QLs[g], first, c};
        slot[g] = first;
        first += c;
        if (!ql)
          SOAP_TRY(gemm(op_batch(QLs[g], true), op_batch(&mbars[g], false), out_ws(t1[g], tm, n), m, n, m, c, 1.f,
                        0.f, false, s),
                   "refresh moment L");
      }
      if (r) {
        SOAP_TRY(gemm(op_batch(Rs[g], true), op_batch(QRs[g], false), out_ws(P + first * pm, pm, n), n, n, n, c, 1.f,
                      0.f, false, s),
                 "refresh power step R");
        outs[nouts++] = QrOut{QRs[g], first, c};
        slot[g] = first;
        first += c;
        if (!qr) {
          const SgemmOperand src = l ? op_ws(t1[g], tm, n, true) : op_batch(&mbars[g], true);
          SOAP_TRY(gemm(src, op_batch(QRs[g], true), out_ws(l ? t2[g] : t1[g], tm, n), m, n, n, c, 1.f, 0.f, false,
                        s),
                   "refresh moment R");
        }
      }
    }
    if ((st = qr_enqueue(P, pm, d, total, qws, outs, nouts, s)) != MUON_OK) return st;
    // the first moment into the new bases
    for (int g = 0; g < ngroups; ++g) {
      const int64_t c = counts[g], m = rows[g], n = cols[g], tm = round64(m * n);
      const bool l = wl[g] && m == d, r = wr[g] && n == d;
      if (l && r) {
        SOAP_TRY(gemm(op_batch(QLs[g], false), op_ws(t2[g], tm, n, false), out_ws(t1[g], tm, n), m, n, m, c, 1.f, 0.f,
                      false, s),
                 "refresh moment L'");
        SOAP_TRY(gemm(op_ws(t1[g], tm, n, true), op_batch(QRs[g], false), out_batch(&mbars[g]), m, n, n, c, 1.f, 0.f,
                      false, s),
                 "refresh moment R'");
      } else if (l && !wr[g] && n > m) {
        // C = QL_new^T QL_old in the group's QR input slot (free after the QR), then mbar = C t1
        float* C = P + slot[g] * pm;
        SOAP_TRY(gemm(op_batch(QLs[g], false), op_ws(t2[g], tm, m, false), out_ws(C, pm, m), m, m, m, c, 1.f, 0.f,
                      false, s),
                 "refresh basis change L");
        SOAP_TRY(gemm(op_ws(C, pm, m, true), op_ws(t1[g], tm, n, false), out_batch(&mbars[g]), m, n, m, c, 1.f, 0.f,
                      false, s),
                 "refresh moment L'");
      } else if (l) {
        SOAP_TRY(gemm(op_batch(QLs[g], false), op_ws(t1[g], tm, n, false), out_batch(&mbars[g]), m, n, m, c, 1.f, 0.f,
                      false, s),
                 "refresh moment L'");
      } else if (r && !wl[g] && m > n) {
        // C = QR_old^T QR_new in the group's QR input slot, then mbar = t1 C
        float* C = P + slot[g] * pm;
        SOAP_TRY(gemm(op_ws(t2[g], tm, n, false), op_batch(QRs[g], false), out_ws(C, pm, n), n, n, n, c, 1.f, 0.f,
                      false, s),
                 "refresh basis change R");
        SOAP_TRY(gemm(op_ws(t1[g], tm, n, true), op_ws(C, pm, n, false), out_batch(&mbars[g]), m, n, n, c, 1.f, 0.f,
                      false, s),
                 "refresh moment R'");
      } else if (r) {
        SOAP_TRY(gemm(op_ws(t1[g], tm, n, true), op_batch(QRs[g], false), out_batch(&mbars[g]), m, n, n, c, 1.f, 0.f,
                      false, s),
                 "refresh moment R'");
      }
    }
  }
  return done(s, "soap_refresh_grouped");
}

muon_status_t soap_refresh(const muon_batch_t* L, const muon_batch_t* R, const muon_batch_t* QL,
                           const muon_batch_t* QR, const muon_batch_t* mbar, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (!mbar) return fail(MUON_ERR_INVALID_VALUE, "mbar: descriptor is NULL");
  return soap_refresh_grouped(1, &L, &R, &QL, &QR, mbar, workspace, ws_bytes, stream);
}

size_t soap_precondition_workspace(int64_t count, int64_t rows, int64_t cols) {
  return soap_precondition_grouped_workspace(1, &count, &rows, &cols);
}

size_t soap_precondition_grouped_workspace(int ngroups, const int64_t* counts, const int64_t* rows,
                                           const int64_t* cols) {
  if (ngroups < 1 || ngroups > kMaxGroups || !counts || !rows || !cols) return 0;
  int64_t total = 0;
  for (int g = 0; g < ngroups; ++g) {
    const int64_t c = counts[g], m = rows[g], n = cols[g];
    if (c < 1 || c > 65535 || m < 1 || n < 1 || m > kMaxElems / n) return 0;
    total += 2 * c * round64(m * n);
  }
  return static_cast<size_t>(total * 4);
}

muon_status_t soap_precondition(const muon_batch_t* grad, const muon_batch_t* QL, const muon_batch_t* QR,
                                const muon_batch_t* mbar, const muon_batch_t* vbar, const muon_batch_t* dir,
                                int64_t step, float beta1, float beta2, float eps, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (!grad || !mbar || !vbar || !dir) return fail(MUON_ERR_INVALID_VALUE, "a required descriptor is NULL");
  return precondition(1, grad, &QL, &QR, mbar, vbar, dir, step, beta1, beta2, eps, workspace, ws_bytes, stream,
                      false);
}

muon_status_t soap_precondition_grouped(int ngroups, const muon_batch_t* grads, const muon_batch_t* const* QLs,
                                        const muon_batch_t* const* QRs, const muon_batch_t* mbars,
                                        const muon_batch_t* vbars, const muon_batch_t* dirs, int64_t step,
                                        float beta1, float beta2, float eps, void* workspace, size_t ws_bytes,
                                        void* stream) {
  return precondition(ngroups, grads, QLs, QRs, mbars, vbars, dirs, step, beta1, beta2, eps, workspace, ws_bytes,
                      stream, true);
}

}  // extern "C"
