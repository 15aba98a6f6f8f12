// Drives every entry point of the C-ABI layer through valid and invalid
// arguments on the CPU (with the stub launchers: nothing reaches a GPU).
// Device addresses are fake and never dereferenced.  Exits non-zero on the
// first unexpected status; the sanitizers abort on any memory or UB error.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "muon355.h"

extern "C" void stub_set_workspace(const void* base, size_t bytes);
extern "C" long stub_launches();

namespace {

int g_fail = 0;
char* const kDev = reinterpret_cast<char*>(uintptr_t{1} << 40);  // fake, 16-byte aligned, never read
char* const kWs = reinterpret_cast<char*>(uintptr_t{1} << 44);

void expect(muon_status_t got, muon_status_t want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, muon_last_error());
    g_fail = 1;
  }
}

muon_batch_t batch(int64_t count, int64_t rows, int64_t cols, int32_t dtype, char* base = kDev) {
  return muon_batch_t{nullptr, base, rows * cols, count, rows, cols, cols, dtype, 0};
}

void orthogonalize_cases() {
  struct Case { int64_t count, rows, cols; int32_t compute; int steps; };
  const Case cases[] = {{1, 256, 128, MUON_F32, 5},   {3, 300, 700, MUON_BF16, 5}, {2, 900, 256, MUON_BF16, 5},
                        {1, 4096, 14336, MUON_BF16, 5}, {384, 768, 2048, MUON_BF16, 5}, {96, 128, 4096, MUON_BF16, 5},
                        {1, 1, 64, MUON_BF16, 5},      {1, 64, 1, MUON_F32, 5},      {2, 700, 520, MUON_F32, 12},
                        {1, 300, 300, MUON_BF16, 0},   {1, 2100, 2200, MUON_BF16, 1}, {1, 129, 900, MUON_F32, 3}};
  for (const Case& c : cases) {
    const size_t need = muon_orthogonalize_workspace(c.count, c.rows, c.cols, c.compute);
    if (need == 0) { std::fprintf(stderr, "workspace query 0\n"); g_fail = 1; continue; }
    stub_set_workspace(kWs, need);
    muon_batch_t in = batch(c.count, c.rows, c.cols, c.compute == MUON_BF16 ? MUON_F32 : MUON_F32);
    muon_batch_t out = batch(c.count, c.rows, c.cols, MUON_BF16);
    expect(muon_orthogonalize(&in, nullptr, &out, c.steps, 3.4445f, -4.775f, 2.0315f, 1e-7f, c.compute, kWs, need,
                              nullptr), MUON_OK, "orthogonalize");
    expect(muon_orthogonalize(&in, nullptr, &out, c.steps, 3.4445f, -4.775f, 2.0315f, 1e-7f, c.compute, kWs, need - 1,
                              nullptr), MUON_ERR_WORKSPACE, "orthogonalize, short workspace");
  }
  // grouped, both tile classes, wide and tall; bf16 (X read k-major) and fp32 (X^T kept)
  const int64_t counts[] = {2, 1, 96, 3, 1}, rows[] = {4096, 14336, 128, 520, 2300}, cols[] = {4096, 4096, 4096, 700, 2050};
  for (int32_t compute : {MUON_BF16, MUON_F32}) {
    const size_t need = muon_orthogonalize_grouped_workspace(5, counts, rows, cols, compute);
    stub_set_workspace(kWs, need);
    std::vector<muon_batch_t> ins, outs;
    for (int g = 0; g < 5; ++g) {
      ins.push_back(batch(counts[g], rows[g], cols[g], MUON_F32));
      outs.push_back(batch(counts[g], rows[g], cols[g], MUON_BF16));
    }
    expect(muon_orthogonalize_grouped(5, ins.data(), nullptr, outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f, compute,
                                      kWs, need, nullptr), MUON_OK, "orthogonalize_grouped");
    ins[3].cols = 701;
    expect(muon_orthogonalize_grouped(5, ins.data(), nullptr, outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f, compute,
                                      kWs, need, nullptr), MUON_ERR_INVALID_VALUE, "orthogonalize_grouped, shapes");
  }
  // the packed pair: momentum into the Newton-Schulz buffers, then the iteration from them
  for (int32_t compute : {MUON_BF16, MUON_F32}) {
    const size_t need = muon_packed_grouped_workspace(5, counts, rows, cols, compute);
    stub_set_workspace(kWs, need);
    std::vector<muon_batch_t> gs, ms, outs;
    std::vector<float*> sums;
    for (int g = 0; g < 5; ++g) {
      gs.push_back(batch(counts[g], rows[g], cols[g], MUON_BF16));
      ms.push_back(batch(counts[g], rows[g], cols[g], MUON_F32));
      outs.push_back(batch(counts[g], rows[g], cols[g], MUON_BF16));
      sums.push_back(reinterpret_cast<float*>(kDev));
    }
    expect(muon_momentum_packed_grouped(5, gs.data(), ms.data(), sums.data(), 0.95f, 1, compute, kWs, need, nullptr),
           MUON_OK, "momentum_packed_grouped");
    expect(muon_momentum_packed_grouped(5, gs.data(), ms.data(), sums.data(), 0.95f, 1, compute, kWs, need - 1,
                                        nullptr), MUON_ERR_WORKSPACE, "momentum_packed_grouped, short workspace");
    expect(muon_orthogonalize_packed_grouped(5, sums.data(), outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f, compute,
                                             kWs, need, nullptr), MUON_OK, "orthogonalize_packed_grouped");
    expect(muon_orthogonalize_packed_grouped(5, sums.data(), outs.data(), 0, 3.4445f, -4.775f, 2.0315f, 1e-7f, compute,
                                             kWs, need, nullptr), MUON_ERR_INVALID_VALUE, "orthogonalize_packed, K 0");
    // ... with the update folded into the last step: the outputs are the weights
    expect(muon_orthogonalize_apply_packed_grouped(5, sums.data(), outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f,
                                                   1e-3f, 0.1f, MUON_SCALE_MATCH_RMS, 0.2f, compute, kWs, need,
                                                   nullptr), MUON_OK, "orthogonalize_apply_packed_grouped");
    expect(muon_orthogonalize_apply_packed_grouped(5, sums.data(), outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f,
                                                   1e-3f, 0.1f, 9, 0.2f, compute, kWs, need, nullptr),
           MUON_ERR_INVALID_VALUE, "orthogonalize_apply_packed_grouped, mode");
    expect(muon_orthogonalize_packed_grouped(5, nullptr, outs.data(), 5, 3.4445f, -4.775f, 2.0315f, 1e-7f, compute,
                                             kWs, need, nullptr), MUON_ERR_INVALID_VALUE, "orthogonalize_packed, sums");
  }
  expect(muon_orthogonalize_workspace(1, 65536, 65536, MUON_F32) == 0 ? MUON_OK : MUON_ERR_LAUNCH, MUON_OK,
         "padded-size limit");
  expect(muon_orthogonalize_workspace(int64_t{1} << 40, 64, 64, MUON_BF16) == 0 ? MUON_OK : MUON_ERR_LAUNCH, MUON_OK,
         "count limit");
}

void momentum_and_apply_cases() {
  muon_batch_t g = batch(2, 300, 700, MUON_BF16), m = batch(2, 300, 700, MUON_F32), n = batch(2, 300, 700, MUON_F32);
  float* sumsq = reinterpret_cast<float*>(kDev);
  size_t need = muon_momentum_workspace(2, 300, 700);
  stub_set_workspace(kWs, need);
  expect(muon_momentum(&g, &m, &n, sumsq, 0.95f, 1, kWs, need, nullptr), MUON_OK, "momentum");
  expect(muon_momentum(&g, &m, nullptr, sumsq, 0.95f, 0, kWs, need, nullptr), MUON_OK, "momentum without N");
  expect(muon_momentum(&g, &m, &n, sumsq, 1.0f, 1, kWs, need, nullptr), MUON_ERR_INVALID_VALUE, "momentum beta 1");
  expect(muon_momentum(&g, &m, &n, sumsq, 0.95f, 1, kWs, need - 4, nullptr), MUON_ERR_WORKSPACE, "momentum workspace");
  const int64_t counts[] = {2, 1, 96}, rows[] = {4096, 14336, 128}, cols[] = {4096, 4096, 4096};
  std::vector<muon_batch_t> gs, ms, ns, ws, os;
  std::vector<float*> sums;
  for (int i = 0; i < 3; ++i) {
    gs.push_back(batch(counts[i], rows[i], cols[i], MUON_BF16));
    ms.push_back(batch(counts[i], rows[i], cols[i], MUON_F32));
    ns.push_back(batch(counts[i], rows[i], cols[i], MUON_F32));
    ws.push_back(batch(counts[i], rows[i], cols[i], MUON_BF16));
    os.push_back(batch(counts[i], rows[i], cols[i], MUON_BF16));
    sums.push_back(sumsq);
  }
  need = muon_momentum_grouped_workspace(3, counts, rows, cols);
  stub_set_workspace(kWs, need);
  expect(muon_momentum_grouped(3, gs.data(), ms.data(), ns.data(), sums.data(), 0.95f, 1, kWs, need, nullptr), MUON_OK,
         "momentum_grouped");
  expect(muon_momentum_grouped(3, gs.data(), ms.data(), ns.data(), sums.data(), 0.95f, 1, kWs, need - 1, nullptr),
         MUON_ERR_WORKSPACE, "momentum_grouped workspace");
  expect(muon_momentum_grouped_noalloc(3, gs.data(), ms.data(), ns.data(), sums.data(), 0.95f, 1, nullptr), MUON_OK,
         "momentum_grouped_noalloc");
  {
    // 17 matrices of 2^30 elements need 8.5 MiB of partial sums: over the static scratch
    muon_batch_t big = batch(17, 32768, 32768, MUON_F32);
    float* s17[1] = {sumsq};
    expect(muon_momentum_grouped_noalloc(1, &big, &big, &big, s17, 0.95f, 1, nullptr), MUON_ERR_WORKSPACE,
           "momentum_grouped_noalloc over the scratch");
  }
  expect(muon_apply(&ws[0], &os[0], 3e-4f, 0.1f, MUON_SCALE_MATCH_RMS, 0.2f, nullptr), MUON_OK, "apply");
  expect(muon_apply_grouped(3, ws.data(), os.data(), 3e-4f, 0.1f, MUON_SCALE_ORIGINAL, 0.2f, nullptr), MUON_OK,
         "apply_grouped");
  expect(muon_apply_grouped(9, ws.data(), os.data(), 3e-4f, 0.1f, 0, 0.2f, nullptr), MUON_ERR_INVALID_VALUE,
         "apply_grouped, 9 groups");
  muon_tensor_list_t t{2, 3, reinterpret_cast<void* const*>(kDev), reinterpret_cast<const void* const*>(kDev),
                       reinterpret_cast<float* const*>(kDev), reinterpret_cast<float* const*>(kDev),
                       reinterpret_cast<const int64_t*>(kDev), reinterpret_cast<const int64_t*>(kDev), MUON_BF16,
                       MUON_BF16};
  expect(muon_adamw(&t, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, nullptr), MUON_OK, "adamw");
  expect(muon_adamw(&t, 0, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, nullptr), MUON_ERR_INVALID_VALUE, "adamw step 0");
}


void soap_cases() {
  struct Case { int64_t count, m, n; bool l, r; };
  const Case cases[] = {{2, 4096, 4096, true, true},   {2, 1024, 4096, true, true}, {2, 14336, 4096, false, true},
                        {1, 4096, 14336, true, false}, {3, 130, 70, true, true},    {1, 1, 33, true, true},
                        {4, 33, 200, true, true},      {2, 40, 50, false, false}};
  for (const Case& c : cases) {
    muon_batch_t g = batch(c.count, c.m, c.n, MUON_BF16);
    muon_batch_t Ls = batch(c.count, c.m, c.m, MUON_F32), QL = batch(c.count, c.m, c.m, MUON_F32);
    muon_batch_t Rs = batch(c.count, c.n, c.n, MUON_F32), QR = batch(c.count, c.n, c.n, MUON_F32);
    muon_batch_t mb = batch(c.count, c.m, c.n, MUON_F32), vb = batch(c.count, c.m, c.n, MUON_F32);
    muon_batch_t d = batch(c.count, c.m, c.n, MUON_F32);
    const muon_batch_t* pL = c.l ? &Ls : nullptr;
    const muon_batch_t* pR = c.r ? &Rs : nullptr;
    const muon_batch_t* pQL = c.l ? &QL : nullptr;
    const muon_batch_t* pQR = c.r ? &QR : nullptr;
    expect(soap_statistics(&g, pL, pR, 0.9f, nullptr), MUON_OK, "soap_statistics");
    size_t need = soap_refresh_workspace(c.count, c.m, c.n, c.l, c.r);
    stub_set_workspace(kWs, need);
    if (c.l || c.r) {
      expect(soap_refresh(pL, pR, pQL, pQR, &mb, kWs, need, nullptr), MUON_OK, "soap_refresh");
      expect(soap_refresh(pL, pR, pQL, pQR, &mb, kWs, need - 1, nullptr), MUON_ERR_WORKSPACE,
             "soap_refresh, short workspace");
    }
    need = soap_precondition_workspace(c.count, c.m, c.n);
    stub_set_workspace(kWs, need);
    expect(soap_precondition(&g, pQL, pQR, &mb, &vb, &d, 3, 0.9f, 0.999f, 1e-8f, kWs, need, nullptr), MUON_OK,
           "soap_precondition");
    expect(soap_precondition(&g, pQL, pQR, &mb, &vb, &d, 0, 0.9f, 0.999f, 1e-8f, kWs, need, nullptr),
           MUON_ERR_INVALID_VALUE, "soap_precondition, step 0");
  }
  {  // the 8B-style layer's groups in one grouped refresh, as the benchmark runs it
    const int64_t counts[] = {2, 2, 2, 1}, rows[] = {4096, 1024, 14336, 4096}, cols[] = {4096, 4096, 4096, 14336};
    const int wl[] = {1, 1, 0, 1}, wr[] = {1, 1, 1, 0};
    std::vector<muon_batch_t> L, R, QL, QR, mb;
    for (int g = 0; g < 4; ++g) {
      L.push_back(batch(counts[g], rows[g], rows[g], MUON_F32));
      QL.push_back(batch(counts[g], rows[g], rows[g], MUON_F32));
      R.push_back(batch(counts[g], cols[g], cols[g], MUON_F32));
      QR.push_back(batch(counts[g], cols[g], cols[g], MUON_F32));
      mb.push_back(batch(counts[g], rows[g], cols[g], MUON_F32));
    }
    const muon_batch_t* pl[4];
    const muon_batch_t* pr[4];
    const muon_batch_t* pql[4];
    const muon_batch_t* pqr[4];
    for (int g = 0; g < 4; ++g) {
      pl[g] = wl[g] ? &L[g] : nullptr;
      pql[g] = wl[g] ? &QL[g] : nullptr;
      pr[g] = wr[g] ? &R[g] : nullptr;
      pqr[g] = wr[g] ? &QR[g] : nullptr;
    }
    std::vector<muon_batch_t> grads;
    for (int g = 0; g < 4; ++g) grads.push_back(batch(counts[g], rows[g], cols[g], MUON_BF16));
    expect(soap_statistics_grouped(4, grads.data(), pl, pr, 0.9f, nullptr), MUON_OK, "soap_statistics_grouped");
    expect(soap_statistics_grouped(9, grads.data(), pl, pr, 0.9f, nullptr), MUON_ERR_INVALID_VALUE,
           "soap_statistics_grouped, 9 groups");
    {
      std::vector<muon_batch_t> vb, dirs;
      for (int g = 0; g < 4; ++g) {
        vb.push_back(batch(counts[g], rows[g], cols[g], MUON_F32));
        dirs.push_back(batch(counts[g], rows[g], cols[g], MUON_F32));
      }
      const size_t pneed = soap_precondition_grouped_workspace(4, counts, rows, cols);
      stub_set_workspace(kWs, pneed);
      expect(soap_precondition_grouped(4, grads.data(), pql, pqr, mb.data(), vb.data(), dirs.data(), 2, 0.9f, 0.999f,
                                       1e-8f, kWs, pneed, nullptr),
             MUON_OK, "soap_precondition_grouped");
      expect(soap_precondition_grouped(4, grads.data(), pql, pqr, mb.data(), vb.data(), dirs.data(), 2, 0.9f, 0.999f,
                                       1e-8f, kWs, pneed - 1, nullptr),
             MUON_ERR_WORKSPACE, "soap_precondition_grouped, short workspace");
    }
    const size_t need = soap_refresh_grouped_workspace(4, counts, rows, cols, wl, wr);
    stub_set_workspace(kWs, need);
    expect(soap_refresh_grouped(4, pl, pr, pql, pqr, mb.data(), kWs, need, nullptr), MUON_OK, "soap_refresh_grouped");
    expect(soap_refresh_grouped(4, pl, pr, pql, pqr, mb.data(), kWs, need - 1, nullptr), MUON_ERR_WORKSPACE,
           "soap_refresh_grouped, short workspace");
  }
  for (int64_t n : {1, 5, 16, 17, 33, 100, 257, 300, 1024, 4096, 4200}) {
    for (int64_t count : {1, 3}) {
      const size_t need = soap_qr_workspace(count, n);
      stub_set_workspace(kWs, need);
      muon_batch_t a = batch(count, n, n, MUON_F32), q = batch(count, n, n, MUON_F32);
      expect(soap_qr(&a, &q, kWs, need, nullptr), MUON_OK, "soap_qr");
    }
  }
}

}  // namespace

int main() {
  orthogonalize_cases();
  momentum_and_apply_cases();
  soap_cases();
  if (g_fail) return 1;
  std::printf("ok: %ld launches checked\n", stub_launches());
  return 0;
}
