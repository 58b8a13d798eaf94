// A C++ caller of libbsa.so through include/bsa.h alone (no Python, no
// torch): device buffers from hipMalloc, plain pointers and sizes.
//
// Forward: a dense causal varlen problem whose V is all ones, so every row's
// output is a softmax-weighted mean of ones, 1 up to the rounding of P and of
// the fp16 output (|O - 1| <= 2e-3), and every lse is finite (each causal row
// keeps its diagonal key).  Backward with dO = 0: D = rowsum(dO o O) = 0 and
// dP = dO V^T = 0, so dS = 0 and dQ = dK = dV = 0 exactly.  Also the error
// paths of the descriptor checks.  Prints "abi_check: ok" and exits 0.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bsa.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("abi_check: FAILED %s\n", what);
    ++failures;
  }
}

bool hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::printf("abi_check: HIP error %s at %s\n", hipGetErrorString(e), what);
    return false;
  }
  return true;
}

uint16_t half_bits(float x) {
  _Float16 h = (_Float16)x;
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

float half_value(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}

}  // namespace

int main() {
  const int B = 2, N1 = 4, N2 = 2, D = 64;
  const int64_t cu_host[3] = {0, 300, 470};  // sequence lengths 300 and 170, queries = keys
  const int64_t T = cu_host[B];

  bsa_problem_t p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.dtype = BSA_DTYPE_F16;
  p.batch = B;
  p.num_heads_q = N1;
  p.num_heads_kv = N2;
  p.head_dim = D;
  p.total_q = T;
  p.total_kv = T;
  p.max_seqlen_q = 300;
  p.max_seqlen_kv = 300;
  p.block_x = 128;
  p.block_y = 128;
  p.sparse_kind = BSA_SPARSE_NONE;
  p.sparse_heads = N1;
  p.mask_type = BSA_MASK_CAUSAL;
  p.kv_layout = BSA_KV_TND;
  p.scale = 0.0;

  size_t fwd_bytes = 0, bwd_bytes = 0;
  expect(bsa_get_workspace_size(&p, &fwd_bytes, &bwd_bytes) == BSA_OK, "workspace size query");
  expect(fwd_bytes > 0 && bwd_bytes >= fwd_bytes, "workspace sizes");

  // inputs: q, k pseudo-random (a fixed linear congruential sequence), v = 1, dout = 0
  const size_t nq = (size_t)T * N1 * D, nk = (size_t)T * N2 * D;
  std::vector<uint16_t> hq(nq), hk(nk), hv(nk, half_bits(1.f)), hz(nq, 0);
  uint32_t s = 12345u;
  auto rnd = [&s]() {
    s = s * 1664525u + 1013904223u;
    return ((s >> 8) & 0xFFFF) / 32768.f - 1.f;
  };
  for (auto& x : hq) x = half_bits(rnd());
  for (auto& x : hk) x = half_bits(rnd());

  void *q, *k, *v, *out, *dout, *dq, *dk, *dv, *ws;
  float* lse;
  int64_t* cu;
  bool ok = hip_ok(hipMalloc(&q, nq * 2), "malloc q") && hip_ok(hipMalloc(&k, nk * 2), "malloc k") &&
            hip_ok(hipMalloc(&v, nk * 2), "malloc v") && hip_ok(hipMalloc(&out, nq * 2), "malloc out") &&
            hip_ok(hipMalloc(&dout, nq * 2), "malloc dout") && hip_ok(hipMalloc(&dq, nq * 2), "malloc dq") &&
            hip_ok(hipMalloc(&dk, nk * 2), "malloc dk") && hip_ok(hipMalloc(&dv, nk * 2), "malloc dv") &&
            hip_ok(hipMalloc((void**)&lse, (size_t)T * N1 * 4), "malloc lse") &&
            hip_ok(hipMalloc((void**)&cu, sizeof(cu_host)), "malloc cu") &&
            hip_ok(hipMalloc(&ws, bwd_bytes), "malloc workspace");
  if (!ok) return 1;
  ok = hip_ok(hipMemcpy(q, hq.data(), nq * 2, hipMemcpyHostToDevice), "copy q") &&
       hip_ok(hipMemcpy(k, hk.data(), nk * 2, hipMemcpyHostToDevice), "copy k") &&
       hip_ok(hipMemcpy(v, hv.data(), nk * 2, hipMemcpyHostToDevice), "copy v") &&
       hip_ok(hipMemcpy(dout, hz.data(), nq * 2, hipMemcpyHostToDevice), "copy dout") &&
       hip_ok(hipMemcpy(cu, cu_host, sizeof(cu_host), hipMemcpyHostToDevice), "copy cu");
  if (!ok) return 1;

  // descriptor checks: a missing pointer, a wrong struct size
  expect(bsa_fwd(&p, nullptr, k, v, cu, cu, nullptr, nullptr, nullptr, nullptr, out, lse, ws, bwd_bytes, nullptr) ==
             BSA_ERR_PARAM_NULLPTR,
         "null q rejected");
  bsa_problem_t bad = p;
  bad.struct_size = sizeof(p) - 8;
  expect(bsa_fwd(&bad, q, k, v, cu, cu, nullptr, nullptr, nullptr, nullptr, out, lse, ws, bwd_bytes, nullptr) ==
             BSA_ERR_PARAM_INVALID,
         "wrong struct size rejected");
  expect(bsa_fwd(&p, q, k, v, cu, cu, nullptr, nullptr, nullptr, nullptr, out, lse, ws, fwd_bytes - 1, nullptr) ==
             BSA_ERR_PARAM_INVALID,
         "short workspace rejected");
  expect(std::strlen(bsa_status_string(BSA_ERR_INNER)) > 0, "status string");

  // value check: sequence 0 longer than max_seqlen_q / _kv is rejected before
  // any other work, with its bits in header slot 6; consistent values pass
  const int64_t cu_bad_host[3] = {0, 320, 470};
  int64_t* cu_bad;
  if (!hip_ok(hipMalloc((void**)&cu_bad, sizeof(cu_bad_host)), "malloc cu_bad") ||
      !hip_ok(hipMemcpy(cu_bad, cu_bad_host, sizeof(cu_bad_host), hipMemcpyHostToDevice), "copy cu_bad"))
    return 1;
  bsa_problem_t pc = p;
  pc.flags = BSA_FLAG_CHECK_VALUES;
  expect(bsa_fwd(&pc, q, k, v, cu_bad, cu_bad, nullptr, nullptr, nullptr, nullptr, out, lse, ws, bwd_bytes,
                 nullptr) == BSA_ERR_PARAM_INVALID,
         "value check rejects a sequence past max_seqlen");
  bsa_index_view_t view;
  expect(bsa_index_view(&pc, 0, &view) == BSA_OK, "index view");
  int32_t word = 0;
  hip_ok(hipMemcpy(&word, static_cast<char*>(ws) + view.off_header + 6 * sizeof(int32_t), sizeof(word),
                   hipMemcpyDeviceToHost),
         "copy check word");
  expect(word == (BSA_CHECK_SQ_LONG | BSA_CHECK_SKV_LONG), "check word names both long sequences");
  expect(bsa_fwd(&pc, q, k, v, cu, cu, nullptr, nullptr, nullptr, nullptr, out, lse, ws, bwd_bytes, nullptr) ==
             BSA_OK,
         "value check passes consistent values");
  hipFree(cu_bad);

  // forward: O = 1, lse finite
  expect(bsa_fwd(&p, q, k, v, cu, cu, nullptr, nullptr, nullptr, nullptr, out, lse, ws, bwd_bytes, nullptr) == BSA_OK,
         "bsa_fwd");
  if (!hip_ok(hipDeviceSynchronize(), "forward")) return 1;
  std::vector<uint16_t> ho(nq);
  std::vector<float> hl((size_t)T * N1);
  hip_ok(hipMemcpy(ho.data(), out, nq * 2, hipMemcpyDeviceToHost), "copy out");
  hip_ok(hipMemcpy(hl.data(), lse, hl.size() * 4, hipMemcpyDeviceToHost), "copy lse");
  double worst = 0.0;
  for (uint16_t x : ho) worst = std::fmax(worst, std::fabs((double)half_value(x) - 1.0));
  bool lse_finite = true;
  for (float x : hl) lse_finite = lse_finite && std::isfinite(x);
  expect(worst <= 2e-3, "O == 1 with V = 1");
  expect(lse_finite, "lse finite on causal rows");

  // backward with dO = 0: all gradients exactly zero
  expect(bsa_bwd(&p, q, k, v, out, dout, lse, cu, cu, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, ws, bwd_bytes,
                 nullptr) == BSA_OK,
         "bsa_bwd");
  if (!hip_ok(hipDeviceSynchronize(), "backward")) return 1;
  std::vector<uint16_t> g(nq);
  bool zero = true;
  hip_ok(hipMemcpy(g.data(), dq, nq * 2, hipMemcpyDeviceToHost), "copy dq");
  for (uint16_t x : g) zero = zero && (x & 0x7FFF) == 0;
  g.resize(nk);
  for (void* t : {dk, dv}) {
    hip_ok(hipMemcpy(g.data(), t, nk * 2, hipMemcpyDeviceToHost), "copy dk / dv");
    for (uint16_t x : g) zero = zero && (x & 0x7FFF) == 0;
  }
  expect(zero, "dQ = dK = dV = 0 with dO = 0");

  for (void* t : {q, k, v, out, dout, dq, dk, dv, ws}) hipFree(t);
  hipFree(lse);
  hipFree(cu);
  std::printf("abi_check: %s (max |O - 1| = %.3g)\n", failures ? "FAILED" : "ok", worst);
  return failures ? 1 : 0;
}
