// host_checks.cpp -- drives the host-only code of libqgemv.so (every qg_check_*
// twin, every workspace query, qg_tiled_bytes) and every oracle function on
// small inputs, in a build with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_sanitizers.py builds and runs it on the CPU; no
// GPU is touched: the check twins launch nothing).  Exit status 0 and no
// sanitizer report mean the argument checks, the plan arithmetic and the
// oracle's loops stay in bounds and free of undefined behaviour over the
// shapes below, valid and invalid.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/qgemv.h"
#include "../../oracle/oracle.h"

namespace {

// fake, distinct, 256-byte aligned device addresses far apart: the check
// twins compare and align them but never dereference them
template <typename T>
T* fake(int i) {
  return reinterpret_cast<T*>((uintptr_t)0x10'0000'0000ull * (uintptr_t)(i + 1));
}
void* const kWs = fake<void>(11);
const size_t kWsBytes = (size_t)1 << 30;

int g_calls = 0;
void note(qg_status) { ++g_calls; }

void checks() {
  const int Ms[] = {-1, 0, 1, 3, 8, 9};
  const int Ns[] = {-5, 0, 1, 16, 17, 3072, 151936, 1 << 30};
  const int Ks[] = {-64, 0, 32, 64, 192, 512, 1024, 2560, 9088, 9216, 12800, 1 << 29};
  for (int M : Ms)
    for (int N : Ns)
      for (int K : Ks) {
        note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                                    fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                                    fake<uint16_t>(4), M, N, K, nullptr, 0));
        note(qg_check_qgemv_affine8(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                                    fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_qgemv_q4k(fake<uint16_t>(0), fake<uint8_t>(1), fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_qgemv_q6k(fake<uint16_t>(0), fake<uint8_t>(1), fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_qgemv_affine4_tiled(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2),
                                          fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_affine4_tile_pack(fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3), fake<uint32_t>(5),
                                        fake<uint16_t>(6), N, K));
        for (int had : {0, 2, 3, 64, 1024, 8192})
          note(qg_check_qgemv_affine4_rht(fake<uint16_t>(0), fake<int8_t>(7), had, fake<uint32_t>(1),
                                          fake<uint16_t>(2), fake<uint16_t>(3), fake<uint16_t>(4), M, N, K, kWs,
                                          kWsBytes));
        note(qg_check_rmsnorm_gateup_swiglu(fake<uint16_t>(0), fake<uint16_t>(7), 1e-6f, fake<uint32_t>(1),
                                            fake<uint16_t>(2), fake<uint16_t>(3), fake<uint16_t>(4), M, N, K, kWs,
                                            kWsBytes));
        note(qg_check_rmsnorm_gateup_swiglu_tiled(fake<uint16_t>(0), fake<uint16_t>(7), 1e-6f, fake<uint32_t>(1),
                                                  fake<uint16_t>(2), fake<uint16_t>(4), M, N, K, kWs, kWsBytes));
        note(qg_check_lmhead_argmax(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                                    fake<float>(4), fake<int32_t>(5), fake<int32_t>(6), fake<int32_t>(7), M, N, K,
                                    kWs, kWsBytes));
        note(qg_check_lmhead_argmax_tiled(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), nullptr,
                                          fake<int32_t>(5), nullptr, nullptr, M, N, K, kWs, kWsBytes));
        for (int k : {0, 1, 8, 64, 65})
          note(qg_check_lmhead_topk(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                                    (k & 1) ? fake<float>(4) : nullptr, fake<int32_t>(5), fake<float>(6), M, N, K,
                                    k, kWs, kWsBytes));
        for (int k : {0, 1, 8, 64, 65})
          note(qg_check_lmhead_topk_tiled(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2),
                                          (k & 1) ? fake<float>(4) : nullptr, fake<int32_t>(5), fake<float>(6), M,
                                          N, K, k, kWs, kWsBytes));
        note(qg_check_mlp_block_affine4_tiled(fake<uint16_t>(0), fake<uint16_t>(1), 1e-6f, fake<uint32_t>(2),
                                              fake<uint16_t>(3), fake<uint32_t>(4), fake<uint16_t>(5),
                                              fake<uint16_t>(6), fake<uint16_t>(7), M, K, N, kWs, kWsBytes));
        for (int L : {0, 1, 28, 5000})
          note(qg_check_mlp_stack_affine4_tiled(fake<uint16_t>(0), fake<uint16_t>(1), 1e-6f, fake<uint32_t>(2),
                                                fake<uint16_t>(3), fake<uint32_t>(4), fake<uint16_t>(5),
                                                fake<uint16_t>(6), fake<uint16_t>(7), L, M, K, N, kWs, kWsBytes));
        // workspace queries
        volatile size_t q = 0;
        q += qgemv_affine4_workspace(M, N, K) + qgemv_affine8_workspace(M, N, K) + qgemv_q4k_workspace(M, N, K) +
             qgemv_q6k_workspace(M, N, K) + qgemv_affine4_tiled_workspace(M, N, K) +
             qgemv_affine4_rht_workspace(M, N, K) + rmsnorm_gateup_swiglu_workspace(M, N, K) +
             rmsnorm_gateup_swiglu_tiled_workspace(M, N, K) + lmhead_argmax_workspace(M, N, K) +
             lmhead_argmax_tiled_workspace(M, N, K) + lmhead_topk_workspace(M, N, K, 8, 0) +
             lmhead_topk_workspace(M, N, K, 64, 1) + lmhead_topk_tiled_workspace(M, N, K, 8, 0) +
             lmhead_topk_tiled_workspace(M, N, K, 64, 1) + mlp_block_affine4_tiled_workspace(M, K, N) +
             mlp_stack_affine4_tiled_workspace(M, K, N) + qg_affine4_valu_workspace(M, N, K);
        size_t sb = 0;
        q += qg_tiled_bytes(N, K, &sb) + sb;
        (void)q;
      }
  // MoE: (top_k, E, D, I)
  for (int top_k : {0, 1, 8, 64, 65})
    for (int E : {0, 1, 8, 128, 1024, 1025})
      for (int D : {0, 256, 2048, 2049})
        for (int I : {0, 256, 768, 1000}) {
          note(qg_check_moe_expert_qgemv(fake<uint16_t>(0), fake<float>(1), top_k, fake<uint8_t>(2),
                                         fake<uint8_t>(3), fake<uint16_t>(4), fake<int32_t>(5), fake<float>(6), E,
                                         D, I, kWs, kWsBytes));
          volatile size_t q = moe_expert_qgemv_workspace(top_k, E, D, I);
          (void)q;
        }
  // null pointers, misaligned pointers, aliasing outputs
  note(qg_check_qgemv_affine4(nullptr, fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3), fake<uint16_t>(4),
                              8, 3072, 1024, kWs, kWsBytes));
  note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1) + 1, fake<uint16_t>(2), fake<uint16_t>(3),
                              fake<uint16_t>(4), 8, 3072, 1024, kWs, kWsBytes));
  note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                              reinterpret_cast<uint16_t*>(fake<uint32_t>(1)) + 8, 8, 3072, 1024, kWs, kWsBytes));
  note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                              fake<uint16_t>(4), 8, 2560, 12800, reinterpret_cast<char*>(kWs) + 8, kWsBytes));
  note(qg_check_qgemv_affine4(fake<uint16_t>(0), fake<uint32_t>(1), fake<uint16_t>(2), fake<uint16_t>(3),
                              fake<uint16_t>(4), 8, 2560, 12800, kWs, 16));
  for (int s = -6; s <= 2; ++s) (void)qg_status_string((qg_status)s);
  (void)qg_last_error();
}

// oracle functions on small inputs (random bits in the byte formats)
template <typename T>
std::vector<T> rnd(std::mt19937& g, size_t n, uint32_t mask = 0xFFFFFFFFu) {
  std::vector<T> v(n);
  for (auto& e : v) e = (T)(g() & mask);
  return v;
}

std::vector<uint16_t> bf16s(std::mt19937& g, size_t n) {
  std::normal_distribution<float> d(0.f, 1.f);
  std::vector<uint16_t> v(n);
  for (auto& e : v) {
    float f = d(g);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    e = (uint16_t)(u >> 16);
  }
  return v;
}

int oracles() {
  std::mt19937 g(7);
  int bad = 0;
  const int M = 3, N = 20, K = 512, I = 256, E = 4, top_k = 2, D = 256, V = 300;
  auto x = bf16s(g, (size_t)M * K);
  auto gamma = bf16s(g, K);
  auto codes = rnd<uint32_t>(g, (size_t)N * K / 8);
  auto codes8 = rnd<uint32_t>(g, (size_t)N * K / 4);
  std::vector<uint16_t> sc((size_t)N * K / 64, 0x3C00), bi((size_t)N * K / 64, 0x3D00);
  std::vector<double> y((size_t)M * N), w((size_t)N * K);
  bad |= oracle_dequant_affine4(codes.data(), sc.data(), bi.data(), N, K, 0, N, w.data());
  bad |= oracle_qgemv_affine4(x.data(), codes.data(), sc.data(), bi.data(), M, N, K, y.data());
  std::vector<double> xd((size_t)M * K, 0.5);
  bad |= oracle_qgemv_affine4_f64x(xd.data(), codes.data(), sc.data(), bi.data(), M, N, K, y.data());
  bad |= oracle_dequant_affine8(codes8.data(), sc.data(), bi.data(), N, K, 0, N, w.data());
  bad |= oracle_qgemv_affine8(x.data(), codes8.data(), sc.data(), bi.data(), M, N, K, y.data());
  auto q4 = rnd<uint8_t>(g, (size_t)N * (K / 256) * 144, 0xFF);
  auto q6 = rnd<uint8_t>(g, (size_t)N * (K / 256) * 210, 0xFF);
  bad |= oracle_dequant_q4k(q4.data(), N, K, 0, N, w.data());
  bad |= oracle_qgemv_q4k(x.data(), q4.data(), M, N, K, y.data());
  bad |= oracle_dequant_q6k(q6.data(), N, K, 0, N, w.data());
  bad |= oracle_qgemv_q6k(x.data(), q6.data(), M, N, K, y.data());
  std::vector<double> xn((size_t)M * K);
  bad |= oracle_rmsnorm(x.data(), gamma.data(), 1e-6, M, K, xn.data());
  auto cgu = rnd<uint32_t>(g, (size_t)2 * I * K / 8);
  std::vector<uint16_t> sgu((size_t)2 * I * K / 64, 0x3C00), bgu((size_t)2 * I * K / 64, 0x3D00);
  std::vector<double> h((size_t)M * I);
  bad |= oracle_rmsnorm_gateup_swiglu(x.data(), gamma.data(), 1e-6, cgu.data(), sgu.data(), bgu.data(), M, I, K,
                                      h.data());
  auto cd = rnd<uint32_t>(g, (size_t)K * I / 8);
  std::vector<uint16_t> sd((size_t)K * I / 64, 0x3C00), bd((size_t)K * I / 64, 0x3D00);
  std::vector<double> yb((size_t)M * K);
  bad |= oracle_mlp_block(x.data(), gamma.data(), 1e-6, cgu.data(), sgu.data(), bgu.data(), cd.data(), sd.data(),
                          bd.data(), M, I, K, yb.data());
  auto wgu = rnd<uint8_t>(g, (size_t)E * 2 * I * (D / 256) * 144, 0xFF);
  auto wdn = rnd<uint8_t>(g, (size_t)E * D * (I / 256) * 144, 0xFF);
  std::vector<float> logits = {0.5f, -1.f, 2.f, 0.5f};
  std::vector<double> ym(D), p(top_k);
  std::vector<int32_t> ids(top_k);
  bad |= oracle_moe(x.data(), logits.data(), top_k, wgu.data(), wdn.data(), E, D, I, ym.data(), ids.data(),
                    p.data());
  auto cv = rnd<uint32_t>(g, (size_t)V * K / 8);
  std::vector<uint16_t> sv((size_t)V * K / 64, 0x3C00), bv((size_t)V * K / 64, 0x3D00);
  std::vector<double> lg((size_t)M * V), gap(M);
  std::vector<int32_t> lid(M), draft = {1, 2, 3};
  int32_t acc = 0;
  bad |= oracle_lmhead(x.data(), cv.data(), sv.data(), bv.data(), M, V, K, lg.data(), lid.data(), gap.data(),
                       draft.data(), &acc);
  std::vector<int32_t> tid((size_t)M * 64);
  std::vector<double> tv((size_t)M * 64);
  bad |= oracle_lmhead_topk(x.data(), cv.data(), sv.data(), bv.data(), M, V, K, 64, tid.data(), tv.data());
  std::vector<int8_t> signs(K);
  for (auto& s : signs) s = (g() & 1) ? 1 : -1;
  std::vector<double> xr((size_t)M * K);
  bad |= oracle_rht(x.data(), signs.data(), 128, M, K, xr.data());
  bad |= oracle_qgemv_affine4_rht(x.data(), signs.data(), 512, codes.data(), sc.data(), bi.data(), M, N, K,
                                  y.data());
  // rejected arguments return an error without touching memory
  if (oracle_qgemv_affine4(x.data(), codes.data(), sc.data(), bi.data(), 0, N, K, y.data()) == 0) bad = 1;
  if (oracle_moe(x.data(), logits.data(), 5, wgu.data(), wdn.data(), E, D, I, ym.data(), ids.data(), p.data()) == 0)
    bad = 1;
  for (double v : {0.0, -0.0, 1.0, 3.0e38, 1e-45, -2.5, 1e300})
    (void)o_f64_to_bf16_rne(v);
  for (int b = 0; b < 65536; b += 97) {
    (void)o_bf16_to_f64((uint16_t)b);
    (void)o_f16_to_f64((uint16_t)b);
  }
  return bad;
}

}  // namespace

int main() {
  checks();
  const int bad = oracles();
  std::printf("host checks: %d check calls, oracle status %d\n", g_calls, bad);
  return bad ? 1 : 0;
}
