// abi.hip -- the C ABI of libqgemv.so (declared in include/qgemv.h):
// argument checks (shared by every entry point and its host-only qg_check_
// twin), the caller-owned workspace (size queries and checks), the work
// decomposition (split-K, tiles per wave) and dispatch to the kernel
// launchers.  Nothing here allocates, frees or synchronises on the call path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <tuple>
#include <mutex>
#include <utility>

#include "../../include/qgemv.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

qg_status fail(qg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

void clear_err() { g_err[0] = '\0'; }

struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
};

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

qg_status check_ptr(const Buf& b, size_t align, const char* fn) {
  if (b.bytes == 0) return QG_OK;
  if (!b.p) return fail(QG_EINVAL, "%s: %s is null", fn, b.name);
  if (!aligned(b.p, align)) return fail(QG_EINVAL, "%s: %s must be %zu-byte aligned", fn, b.name, align);
  return QG_OK;
}

bool overlaps(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes, b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

qg_status check_alias(const Buf* outs, int nout, const Buf* ins, int nin, const char* fn) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j]))
        return fail(QG_EALIAS, "%s: output %s overlaps input %s", fn, outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(QG_EALIAS, "%s: output %s overlaps output %s", fn, outs[i].name, outs[j].name);
  }
  return QG_OK;
}

// Every input and output buffer of a call, for the workspace overlap check.
struct BufList {
  Buf b[16];
  int n = 0;
};
void collect(BufList* all, const Buf* outs, int nout, const Buf* ins, int nin) {
  if (!all) return;
  for (int i = 0; i < nout && all->n < 16; ++i) all->b[all->n++] = outs[i];
  for (int i = 0; i < nin && all->n < 16; ++i) all->b[all->n++] = ins[i];
}

constexpr size_t kLdsBudget = 163840;      // bytes of LDS one workgroup may use (all of a gfx950 CU's)
constexpr size_t kQ4kLdsBudget = 65536;    // staged-slice bound of the Q4_K projection (keeps 2+ workgroups per CU)
// Share (percent) of the resident workgroup slots an affine projection fills, per mode.
// Gate/up with 4-wave workgroups (M >= 5) fills three of a CU's four slots: on
// the 2560 -> 2 x 12,800 block 13.6-13.7 us at M = 8 against 14.3 at 100%, and
// 14.6-14.9 / 14.8-14.9 / 14.6-14.7 at 50 / 60 / 85% (the same number of
// workgroups on every CU matters more than the count); its 8- and 16-wave
// workgroups fill every slot (one or two per CU).
#ifndef QG_FILL_GATEUP
#define QG_FILL_GATEUP 100
#endif
#ifndef QG_FILL_GATEUP4
#define QG_FILL_GATEUP4 75
#endif
#ifndef QG_FILL_PLAIN
#define QG_FILL_PLAIN 75
#endif
#ifndef QG_FILL_OTHER
#define QG_FILL_OTHER 50
#endif
constexpr int kTargetWaves = 2048;         // enough (tile, slice) pieces to cover HBM latency on 256 CUs
constexpr int kMaxWavesInFlight = 4096;    // beyond this, waves stream several tiles
constexpr int kMaxUnsplitSteps = 4;        // batches of loads per tile a plain projection takes unsplit

// LDS of the affine kernels per 128-k chunk of the staged slice (operand
// entries for PL activation planes, group sums, sums of x^2) and fixed (the
// zero region read by empty operand slots, 64*PL*M entries of 16 bytes, and
// the per-wave argmax keys).
size_t affine_lds_per_chunk(int M, int PL) { return (size_t)256 * M * PL + 64 + (size_t)8 * M; }
size_t affine_lds_fixed(int M, int PL) { return (size_t)1024 * PL * M + (size_t)kWaves * 64; }
size_t q4k_lds_per_sb(int M) { return (size_t)512 * M + 256; }
size_t q6k_lds_per_sb(int M) { return (size_t)512 * M + 512; }  // operands + 16 scale-block sums x 8 rows

// The LM head splits K when M staged rows of it exceed the LDS budget
// (partial sums then go through the workspace); this bounds K all the same.
constexpr int kLmMaxK = 1 << 18;

struct Plan {
  int S, cps, tpw, rgroups;
};

// Split-K and tiles-per-wave choice shared by the projection kernels.
Plan plan_split(int ntiles, int nchunks, int cps_max, bool allow_split, int target = kTargetWaves) {
  Plan pl{};
  const int s_min = (nchunks + cps_max - 1) / cps_max;
  int S = s_min;
  if (allow_split && (long long)ntiles * S < target) {
    const int want = (target + ntiles - 1) / std::max(ntiles, 1);
    S = std::max(s_min, std::min(want, std::max(1, nchunks / 2)));
  }
  if (!allow_split) S = 1;
  pl.cps = (nchunks + S - 1) / S;
  pl.S = (nchunks + pl.cps - 1) / pl.cps;
  const long long waves = (long long)ntiles * pl.S;
  pl.tpw = (int)std::min<long long>(8, std::max<long long>(1, waves / kMaxWavesInFlight));
  pl.rgroups = (ntiles + kWaves * pl.tpw - 1) / (kWaves * pl.tpw);
  return pl;
}

// ---------------------------------------------------------- workspace --
// Scratch memory comes from the caller (ws, ws_bytes): the library never
// allocates, frees or synchronises.  Layout of a workspace:
//   [0, kWsHeader)  state words (the LM head's running maxima and arrival
//                   counter, the persistent block's barrier counters and
//                   failure flags) that must be zero before the first call;
//                   every call that uses them leaves them zero again (so one
//                   workspace can serve every entry point and every shape,
//                   one call at a time);
//   [kWsHeader, ...) per-call scratch (split-K partial sums, top-k
//                   candidates, RHT planes, MoE routing and expert
//                   activations); written before it is read within a call.
// A call that needs neither returns 0 from its size query and accepts ws = NULL.
constexpr size_t kWsAlign = 256;
constexpr int kMaxCus = 256;  // workspace sizes are computed for this many compute units (gfx950)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Total workspace bytes for `scratch` bytes of per-call scratch (0 if none is needed).
size_t ws_total(size_t scratch, bool state = false) {
  if (scratch == 0 && !state) return 0;
  return kWsHeader + align_up(scratch, kWsAlign);
}

// Checks the caller's workspace against the `need` bytes the plan requires:
// present, 256-byte aligned, large enough, and overlapping no input or output.
qg_status check_ws(const char* fn, const void* ws, size_t ws_bytes, size_t need, const Buf* others, int nothers) {
  if (need == 0) return QG_OK;
  if (!ws) return fail(QG_EINVAL, "%s: needs a workspace of %zu bytes (ws is null)", fn, need);
  if (!aligned(ws, kWsAlign)) return fail(QG_EINVAL, "%s: ws must be %zu-byte aligned", fn, kWsAlign);
  if (ws_bytes < need) return fail(QG_EINVAL, "%s: ws_bytes=%zu, needs %zu", fn, ws_bytes, need);
  const Buf w = {ws, ws_bytes, "ws"};
  for (int i = 0; i < nothers; ++i)
    if (overlaps(w, others[i])) return fail(QG_EALIAS, "%s: ws overlaps %s", fn, others[i].name);
  return QG_OK;
}

int g_cus[64] = {0};  // compute units per device, filled by check_device

// The kernels are gfx950 code objects; refuse other devices by name.
qg_status check_device() {
  static std::mutex mu;
  static int ok[64] = {0};  // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(QG_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(QG_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  if (ok[dev] < 0) return fail(QG_EUNSUPPORTED, "device %d is not gfx950 (MI355X); no kernels for it", dev);
  return QG_OK;
}

// Compute units of the current device (set by check_device), at most kMaxCus.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || g_cus[dev] <= 0) return kMaxCus;
  return std::min(g_cus[dev], kMaxCus);
}

// Workgroups per K slice for the persistent affine kernel: `fill_pct` percent
// of the device's resident workgroup slots (`waves` waves per workgroup, 16
// waves per CU at 128 registers per lane, fewer workgroups if the staged slice
// limits LDS occupancy), and no more workgroups than it takes to give every
// wave a tile.
int affine_rgroups(int ntiles, int S, size_t lds, int waves, int fill_pct, int cus) {
  const size_t lds_cu = 160 * 1024;
  const int max_occ = std::max(1, 16 / waves);
  const int occ = (int)std::max<size_t>(1, std::min<size_t>((size_t)max_occ, lds_cu / std::max<size_t>(lds, 1)));
  const long long slots = (long long)cus * occ * fill_pct / 100;
  const long long per_slice = std::max<long long>(1, slots / S);
  const long long max_r = std::max<long long>(1, (ntiles + waves - 1) / waves);
  return (int)std::min(per_slice, max_r);
}

// Waves per workgroup of the affine kernel.  Gate/up stages the slice's two
// activation planes once per workgroup; with few activation rows its waves
// run short, and wider workgroups (one staged copy shared by more waves, the
// same plan and tile order, bit-identical results) measured faster on the
// 2560 -> 2 x 12,800 block: 11.8 vs 12.5 us at M = 1 (16 waves), 12.3 vs
// 13.1 at M = 2 and 13.1 vs 13.8 at M = 4 (8 waves); at M = 8, 4 waves.
int affine_waves(int mode, int M) {
  if (mode != QG_MODE_GATEUP) return kWaves;
  return M == 1 ? 16 : (M <= 4 ? 8 : kWaves);
}

qg_status launched(int err, const char* fn) {
  if (err != 0) return fail(QG_EHIP, "%s: launch failed: %s", fn, hipGetErrorString((hipError_t)err));
  clear_err();
  return QG_OK;
}

// ------------------------------------------------------------ checks --
qg_status check_affine_common(const char* fn, int M, int N, int K) {
  if (M < 1 || M > 8) return fail(QG_EINVAL, "%s: M=%d must be in 1..8", fn, M);
  if (N < 0) return fail(QG_EINVAL, "%s: N=%d must be >= 0", fn, N);
  if (K <= 0 || K % 64 != 0) return fail(QG_EINVAL, "%s: K=%d must be a positive multiple of 64", fn, K);
  if ((long long)N * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: N=%d too large", fn, N);
  return QG_OK;
}

qg_status do_check_qgemv_affine4(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, BufList* all = nullptr) {
  const char* fn = "qgemv_affine4";
  qg_status st = check_affine_common(fn, M, N, K);
  if (st) return st;
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"},
                    {codes, n * k / 2, "codes"},
                    {scales, n * (k / 64) * 2, "scales"},
                    {biases, n * (k / 64) * 2, "biases"}};
  const Buf out[] = {{y, (size_t)M * n * 2, "y"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 4);
  return check_alias(out, 1, in, 4, fn);
}

qg_status do_check_qgemv_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, BufList* all = nullptr) {
  const char* fn = "qgemv_affine8";
  qg_status st = check_affine_common(fn, M, N, K);
  if (st) return st;
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"},
                    {codes, n * k, "codes"},
                    {scales, n * (k / 64) * 2, "scales"},
                    {biases, n * (k / 64) * 2, "biases"}};
  const Buf out[] = {{y, (size_t)M * n * 2, "y"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 4);
  return check_alias(out, 1, in, 4, fn);
}

qg_status do_check_qgemv_q4k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K, BufList* all = nullptr) {
  const char* fn = "qgemv_q4k";
  if (M < 1 || M > 8) return fail(QG_EINVAL, "%s: M=%d must be in 1..8", fn, M);
  if (N < 0) return fail(QG_EINVAL, "%s: N=%d must be >= 0", fn, N);
  if (K <= 0 || K % 256 != 0) return fail(QG_EINVAL, "%s: K=%d must be a positive multiple of 256", fn, K);
  if ((long long)N * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: N=%d too large", fn, N);
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"}, {blocks, n * (k / 256) * 144, "blocks"}};
  const Buf out[] = {{y, (size_t)M * n * 2, "y"}};
  qg_status st;
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 2);
  return check_alias(out, 1, in, 2, fn);
}

qg_status do_check_qgemv_q6k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K, BufList* all = nullptr) {
  const char* fn = "qgemv_q6k";
  if (M < 1 || M > 8) return fail(QG_EINVAL, "%s: M=%d must be in 1..8", fn, M);
  if (N < 0) return fail(QG_EINVAL, "%s: N=%d must be >= 0", fn, N);
  if (K <= 0 || K % 256 != 0) return fail(QG_EINVAL, "%s: K=%d must be a positive multiple of 256", fn, K);
  if ((long long)N * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: N=%d too large", fn, N);
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"}, {blocks, n * (k / 256) * 210, "blocks"}};
  const Buf out[] = {{y, (size_t)M * n * 2, "y"}};
  qg_status st;
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 2, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 2);
  return check_alias(out, 1, in, 2, fn);
}

qg_status do_check_gateup(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes,
                          const uint16_t* scales, const uint16_t* biases, uint16_t* h, int M, int I, int K, BufList* all = nullptr) {
  const char* fn = "rmsnorm_gateup_swiglu";
  qg_status st = check_affine_common(fn, M, I, K);
  if (st) return st;
  if (!(eps > 0.0f) || eps != eps || eps > 3.0e38f) return fail(QG_EINVAL, "%s: eps must be positive and finite", fn);
  if ((long long)I * 2 * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: I=%d too large", fn, I);
  const size_t i2 = (size_t)2 * I, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"},
                    {gamma, k * 2, "gamma"},
                    {codes, i2 * k / 2, "codes_gu"},
                    {scales, i2 * (k / 64) * 2, "scales_gu"},
                    {biases, i2 * (k / 64) * 2, "biases_gu"}};
  const Buf out[] = {{h, (size_t)M * I * 2, "h"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 16, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(in[4], 2, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 5);
  return check_alias(out, 1, in, 5, fn);
}

qg_status do_check_moe(const uint16_t* x, const float* logits, int top_k, const uint8_t* w_gu,
                       const uint8_t* w_down, uint16_t* y, int32_t* out_ids, float* out_w, int E, int D, int I, BufList* all = nullptr) {
  const char* fn = "moe_expert_qgemv";
  if (E < 1 || E > 1024) return fail(QG_EINVAL, "%s: E=%d must be in 1..1024", fn, E);
  if (top_k < 1 || top_k > E) return fail(QG_EINVAL, "%s: top_k=%d must be in 1..E", fn, top_k);
  if (top_k > 64) return fail(QG_EUNSUPPORTED, "%s: top_k=%d above 64", fn, top_k);
  if (D <= 0 || D % 256 != 0) return fail(QG_EINVAL, "%s: D=%d must be a positive multiple of 256", fn, D);
  if (I <= 0 || I % 256 != 0) return fail(QG_EINVAL, "%s: I=%d must be a positive multiple of 256", fn, I);
  if (16 + (size_t)(D / 256) * 768 > kLdsBudget)
    return fail(QG_EUNSUPPORTED, "%s: D=%d too large for the staged activation", fn, D);
  if (16 + (size_t)top_k * (I / 256) * 768 > kLdsBudget)
    return fail(QG_EUNSUPPORTED, "%s: top_k*I/256=%d too large for the staged expert activations", fn,
                top_k * (I / 256));
  const size_t e = (size_t)E, d = (size_t)D, i = (size_t)I;
  const Buf in[] = {{x, d * 2, "x"},
                    {logits, e * 4, "router_logits"},
                    {w_gu, e * 2 * i * (d / 256) * 144, "w_gu"},
                    {w_down, e * d * (i / 256) * 144, "w_down"}};
  const Buf out[] = {{y, d * 2, "y"}, {out_ids, out_ids ? (size_t)top_k * 4 : 0, "out_ids"},
                     {out_w, out_w ? (size_t)top_k * 4 : 0, "out_w"}};
  qg_status st;
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 4, fn)) || (st = check_ptr(in[2], 16, fn)) ||
      (st = check_ptr(in[3], 16, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  if (out_ids && (st = check_ptr(out[1], 4, fn))) return st;
  if (out_w && (st = check_ptr(out[2], 4, fn))) return st;
  collect(all, out, 3, in, 4);
  return check_alias(out, 3, in, 4, fn);
}

qg_status do_check_lmhead(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                          float* logits, int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V,
                          int K, BufList* all = nullptr) {
  const char* fn = "lmhead_argmax";
  qg_status st = check_affine_common(fn, M, V, K);
  if (st) return st;
  if (V < 1) return fail(QG_EINVAL, "%s: V=%d must be >= 1", fn, V);
  if (K > kLmMaxK) return fail(QG_EUNSUPPORTED, "%s: K=%d above %d", fn, K, kLmMaxK);
  const size_t v = (size_t)V, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"},
                    {codes, v * k / 2, "codes"},
                    {scales, v * (k / 64) * 2, "scales"},
                    {biases, v * (k / 64) * 2, "biases"},
                    {draft, draft ? (size_t)M * 4 : 0, "draft"}};
  const Buf out[] = {{logits, logits ? (size_t)M * v * 4 : 0, "logits"},
                     {ids, (size_t)M * 4, "ids"},
                     {accepted, accepted ? (size_t)4 : (size_t)0, "accepted"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(out[1], 4, fn)))
    return st;
  if (draft && (st = check_ptr(in[4], 4, fn))) return st;
  if (logits && (st = check_ptr(out[0], 4, fn))) return st;
  if (accepted && (st = check_ptr(out[2], 4, fn))) return st;
  collect(all, out, 3, in, 5);
  return check_alias(out, 3, in, 5, fn);
}

qg_status do_check_lmhead_topk(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, float* logits, int32_t* ids, float* vals, int M, int V, int K,
                               int k, BufList* all = nullptr) {
  const char* fn = "lmhead_topk";
  qg_status st = check_affine_common(fn, M, V, K);
  if (st) return st;
  if (V < 1) return fail(QG_EINVAL, "%s: V=%d must be >= 1", fn, V);
  if (k < 1 || k > V) return fail(QG_EINVAL, "%s: k=%d must be in 1..V", fn, k);
  if (k > kTopkMax) return fail(QG_EUNSUPPORTED, "%s: k=%d above %d", fn, k, kTopkMax);
  if (K > kLmMaxK) return fail(QG_EUNSUPPORTED, "%s: K=%d above %d", fn, K, kLmMaxK);
  const size_t v = (size_t)V, kk = (size_t)K;
  const Buf in[] = {{x, (size_t)M * kk * 2, "x"},
                    {codes, v * kk / 2, "codes"},
                    {scales, v * (kk / 64) * 2, "scales"},
                    {biases, v * (kk / 64) * 2, "biases"}};
  const Buf out[] = {{logits, logits ? (size_t)M * v * 4 : 0, "logits"},
                     {ids, (size_t)M * k * 4, "ids"},
                     {vals, vals ? (size_t)M * k * 4 : (size_t)0, "vals"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(out[1], 4, fn)))
    return st;
  if (logits && (st = check_ptr(out[0], 4, fn))) return st;
  if (vals && (st = check_ptr(out[2], 4, fn))) return st;
  collect(all, out, 3, in, 4);
  return check_alias(out, 3, in, 4, fn);
}

qg_status do_check_qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had, const uint32_t* codes,
                                     const uint16_t* scales, const uint16_t* biases, uint16_t* y, int M, int N,
                                     int K, BufList* all = nullptr) {
  const char* fn = "qgemv_affine4_rht";
  qg_status st = check_affine_common(fn, M, N, K);
  if (st) return st;
  if (had < 2 || had > kRhtMax || (had & (had - 1)) != 0)
    return fail(QG_EINVAL, "%s: had=%d must be a power of two in 2..%d", fn, had, kRhtMax);
  if (K % had != 0) return fail(QG_EINVAL, "%s: had=%d must divide K=%d", fn, had, K);
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{x, (size_t)M * k * 2, "x"},
                    {codes, n * k / 2, "codes"},
                    {scales, n * (k / 64) * 2, "scales"},
                    {biases, n * (k / 64) * 2, "biases"},
                    {signs, k, "signs"}};
  const Buf out[] = {{y, (size_t)M * n * 2, "y"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(in[3], 2, fn)) || (st = check_ptr(in[4], 1, fn)) || (st = check_ptr(out[0], 2, fn)))
    return st;
  collect(all, out, 1, in, 5);
  return check_alias(out, 1, in, 5, fn);
}

// Sizes of the tile-order layout of an [N][K] affine-4 matrix.
size_t tiled_codes_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((size_t)K / 128) * 1024; }
size_t tiled_sb_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((size_t)K / 512) * 512; }

qg_status do_check_tile_pack(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             uint32_t* codes_t, uint16_t* sb_t, int N, int K) {
  const char* fn = "affine4_tile_pack";
  if (N < 1) return fail(QG_EINVAL, "%s: N=%d must be >= 1", fn, N);
  if (K <= 0 || K % 512 != 0) return fail(QG_EINVAL, "%s: K=%d must be a positive multiple of 512", fn, K);
  if ((long long)N * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: N=%d too large", fn, N);
  const size_t n = (size_t)N, k = (size_t)K;
  const Buf in[] = {{codes, n * k / 2, "codes"}, {scales, n * (k / 64) * 2, "scales"},
                    {biases, n * (k / 64) * 2, "biases"}};
  const Buf out[] = {{codes_t, tiled_codes_bytes(N, K), "codes_t"}, {sb_t, tiled_sb_bytes(N, K), "sb_t"}};
  qg_status st;
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 2, fn)) || (st = check_ptr(in[2], 2, fn)) ||
      (st = check_ptr(out[0], 16, fn)) || (st = check_ptr(out[1], 16, fn)))
    return st;
  return check_alias(out, 2, in, 3, fn);
}

qg_status do_check_tiled(const char* fn, const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, int M,
                         int N, int K, const Buf* outs, int nout, BufList* all = nullptr) {
  qg_status st = check_affine_common(fn, M, N, K);
  if (st) return st;
  if (K % 512 != 0) return fail(QG_EINVAL, "%s: K=%d must be a multiple of 512 (tile-order layout)", fn, K);
  const Buf in[] = {{x, (size_t)M * K * 2, "x"}, {codes_t, tiled_codes_bytes(N, K), "codes_t"},
                    {sb_t, tiled_sb_bytes(N, K), "sb_t"}};
  if ((st = check_ptr(in[0], 16, fn)) || (st = check_ptr(in[1], 16, fn)) || (st = check_ptr(in[2], 16, fn)))
    return st;
  collect(all, outs, nout, in, 3);
  return check_alias(outs, nout, in, 3, fn);
}

qg_status do_check_qgemv_affine4_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, uint16_t* y,
                                       int M, int N, int K, BufList* all) {
  const char* fn = "qgemv_affine4_tiled";
  const Buf out[] = {{y, (size_t)M * N * 2, "y"}};
  qg_status st = do_check_tiled(fn, x, codes_t, sb_t, M, N, K, out, 1, all);
  if (st) return st;
  return check_ptr(out[0], 2, fn);
}

qg_status do_check_lmhead_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, float* logits,
                                int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V, int K,
                                BufList* all) {
  const char* fn = "lmhead_argmax_tiled";
  if (V < 1) return fail(QG_EINVAL, "%s: V=%d must be >= 1", fn, V);
  if (K > kLmMaxK) return fail(QG_EUNSUPPORTED, "%s: K=%d above %d", fn, K, kLmMaxK);
  const Buf out[] = {{logits, logits ? (size_t)M * V * 4 : 0, "logits"},
                     {ids, (size_t)M * 4, "ids"},
                     {accepted, accepted ? (size_t)4 : (size_t)0, "accepted"}};
  qg_status st = do_check_tiled(fn, x, codes_t, sb_t, M, V, K, out, 3, all);
  if (st) return st;
  if ((st = check_ptr(out[1], 4, fn))) return st;
  if (logits && (st = check_ptr(out[0], 4, fn))) return st;
  if (accepted && (st = check_ptr(out[2], 4, fn))) return st;
  const Buf dr = {draft, draft ? (size_t)M * 4 : 0, "draft"};
  if (draft && (st = check_ptr(dr, 4, fn))) return st;
  collect(all, nullptr, 0, &dr, 1);
  return check_alias(out, 3, &dr, 1, fn);
}

qg_status do_check_lmhead_topk_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t,
                                     float* logits, int32_t* ids, float* vals, int M, int V, int K, int k,
                                     BufList* all) {
  const char* fn = "lmhead_topk_tiled";
  if (V < 1) return fail(QG_EINVAL, "%s: V=%d must be >= 1", fn, V);
  if (k < 1 || k > V) return fail(QG_EINVAL, "%s: k=%d must be in 1..V", fn, k);
  if (k > kTopkMax) return fail(QG_EUNSUPPORTED, "%s: k=%d above %d", fn, k, kTopkMax);
  if (K > kLmMaxK) return fail(QG_EUNSUPPORTED, "%s: K=%d above %d", fn, K, kLmMaxK);
  const Buf out[] = {{logits, logits ? (size_t)M * V * 4 : 0, "logits"},
                     {ids, (size_t)M * k * 4, "ids"},
                     {vals, vals ? (size_t)M * k * 4 : (size_t)0, "vals"}};
  qg_status st = do_check_tiled(fn, x, codes_t, sb_t, M, V, K, out, 3, all);
  if (st) return st;
  if ((st = check_ptr(out[1], 4, fn))) return st;
  if (logits && (st = check_ptr(out[0], 4, fn))) return st;
  if (vals && (st = check_ptr(out[2], 4, fn))) return st;
  return QG_OK;
}

qg_status do_check_gateup_tiled(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes_t,
                                const uint16_t* sb_t, uint16_t* h, int M, int I, int K, BufList* all) {
  const char* fn = "rmsnorm_gateup_swiglu_tiled";
  if (I < 1 || (long long)I * 2 * 16 > 0x7FFFFFFFLL) return fail(QG_EINVAL, "%s: I=%d out of range", fn, I);
  if (!(eps > 0.0f) || eps != eps || eps > 3.0e38f) return fail(QG_EINVAL, "%s: eps must be positive and finite", fn);
  const Buf out[] = {{h, (size_t)M * I * 2, "h"}};
  qg_status st = do_check_tiled(fn, x, codes_t, sb_t, M, 2 * I, K, out, 1, all);
  if (st) return st;
  const Buf gm = {gamma, (size_t)K * 2, "gamma"};
  if ((st = check_ptr(gm, 16, fn)) || (st = check_ptr(out[0], 2, fn))) return st;
  collect(all, nullptr, 0, &gm, 1);
  return check_alias(out, 1, &gm, 1, fn);
}

// --------------------------------------------------------- dispatch --
// Split plan of an affine projection (a.M, a.N, a.K and a.tiled set): fills
// G, nchunks, ntiles, waves, S, cps and wide, *lds (bytes of LDS per
// workgroup) and rgroups (workgroups per slice on `cus` compute units).  The
// persistent MLP block uses the same plans, so its results equal those of the
// separate entry points.
//
// The K split is chosen with the LDS footprint of an 8-row call, so that a
// call's slices -- and with them the order in which partial sums are added --
// do not depend on M: row i of an M-row call equals, bit for bit, the 1-row
// call on row i (TensorFold page, section "핵심 메커니즘 2 — 정확 디코딩").
qg_status plan_affine(int mode, QgAffineArgs& a, const char* fn, size_t* lds_out, int cus) {
  const int G = a.K / 64;
  a.G = G;
  a.nchunks = (G + 1) / 2;
  a.ntiles = (a.N + 15) / 16;
  a.waves = affine_waves(mode, a.M);
  const int PL = (mode == QG_MODE_GATEUP || mode == QG_MODE_PLANES) ? 2 : 1;
  const size_t per = affine_lds_per_chunk(a.M, PL);
  const bool split_ok = (mode != QG_MODE_LMHEAD);
  const int Ms = split_ok ? 8 : a.M;  // rows the slice length is sized for
  const int cps_max = (int)std::min<size_t>(
      (size_t)a.nchunks, (kLdsBudget - affine_lds_fixed(Ms, PL)) / affine_lds_per_chunk(Ms, PL));
  // the LM head keeps K in one slice whenever its M staged rows fit, and
  // splits K beyond that (in as few slices as fit)
  if (mode == QG_MODE_LMHEAD && a.K > kLmMaxK) return fail(QG_EUNSUPPORTED, "%s: K=%d above %d", fn, a.K, kLmMaxK);
  const bool lm_split = (mode == QG_MODE_LMHEAD) && a.nchunks > cps_max;
  // A split costs a follow-up kernel (a few microseconds); a plain projection
  // is split only when a tile has more than kMaxUnsplitSteps batches of
  // loads (or the slice would not fit on chip).  Gate/up always ends in the
  // pairing reduce, so it may always split.
  const int steps_per_tile = (a.nchunks + 3) / 4;
  const bool allow_split = split_ok && (mode == QG_MODE_GATEUP || steps_per_tile > kMaxUnsplitSteps ||
                                        a.nchunks > cps_max);
  // Pieces to aim for and share of the resident workgroup slots to fill, per
  // mode (measured on the decode shapes): gate/up, whose staging is the
  // costliest, prefers many short slices, on three quarters of the slots with
  // 4-wave workgroups and on every slot with wider ones; plain projections run
  // best on three quarters of the slots, the LM head and the other modes on
  // half, with two or more tiles per wave.
#ifndef QG_TARGET_GATEUP
#define QG_TARGET_GATEUP (4 * kTargetWaves)
#endif
#ifndef QG_TARGET_OTHER
#define QG_TARGET_OTHER (2 * kTargetWaves)
#endif
  const int target = (mode == QG_MODE_GATEUP) ? QG_TARGET_GATEUP : QG_TARGET_OTHER;
  const int fill_pct = (mode == QG_MODE_GATEUP) ? (a.waves == kWaves ? QG_FILL_GATEUP4 : QG_FILL_GATEUP)
                                                : (mode == QG_MODE_PLAIN ? QG_FILL_PLAIN : QG_FILL_OTHER);
  Plan pl = lm_split ? plan_split(a.ntiles, a.nchunks, std::max(cps_max, 1), true, 0)
                     : plan_split(a.ntiles, a.nchunks, std::max(cps_max, 1), allow_split, target);
  // slices start on a batch boundary (4 chunks) when that keeps them within LDS
  const int batch = 4;
  if (pl.S > 1) {
    const int cps_b = (pl.cps + batch - 1) / batch * batch;
    if (cps_b <= cps_max) {
      pl.cps = cps_b;
      pl.S = (a.nchunks + pl.cps - 1) / pl.cps;
    }
  }
  a.S = pl.S;
  a.cps = pl.cps;
  {
    const size_t vec = (size_t)2 * batch * 2;  // bytes of one batch's scales of one row
    a.wide = (a.G % (2 * batch) == 0) && (a.S == 1 || a.cps % batch == 0) &&
             ((uintptr_t)a.scales % vec == 0) && ((uintptr_t)a.biases % vec == 0);
  }
  if (a.tiled && !a.wide)
    return fail(QG_EUNSUPPORTED, "%s: no K split of whole 512-k batches fits for K=%d", fn, a.K);
  *lds_out = (size_t)a.cps * per + affine_lds_fixed(a.M, PL);
  a.rgroups = affine_rgroups(a.ntiles, a.S, *lds_out, a.waves, fill_pct, cus);
  return QG_OK;
}

// One affine call: its mode, launch arguments, plan and scratch layout
// (offsets from the start of the scratch region, kWsHeader into ws).
struct AffineCall {
  int mode = QG_MODE_PLAIN;
  QgAffineArgs a{};
  size_t lds = 0;
  size_t reserve = 0;  // leading scratch of the entry point (the RHT planes)
  size_t off_part = 0, off_ssq = 0, off_cand = 0, off_surv = 0, off_lg = 0, scratch = 0;
};

// The greedy LM head merges its workgroups' maxima in the workspace header
// and finishes in its last workgroup (no second kernel); the top-k readout
// stores them in its scratch for the selection kernel instead.
bool lm_fused(const AffineCall& c) { return c.mode == QG_MODE_LMHEAD && c.a.topk == 0; }

qg_status affine_layout(AffineCall& c, const char* fn, int cus) {
  // the top-k readout is planned for kMaxCus compute units whatever the device:
  // its scratch (one key per workgroup and row, the kept keys) depends on the plan
  const bool topk = c.mode == QG_MODE_LMHEAD && c.a.topk > 0;
  qg_status st = plan_affine(c.mode, c.a, fn, &c.lds, topk ? kMaxCus : cus);
  if (st) return st;
  QgAffineArgs& a = c.a;
  size_t off = align_up(c.reserve, kWsAlign);
  const bool partials = a.S > 1 || c.mode == QG_MODE_GATEUP;
  c.off_part = off;
  off += partials ? align_up((size_t)a.S * a.M * a.N * 4, kWsAlign) : 0;
  c.off_ssq = off;
  off += (c.mode == QG_MODE_GATEUP) ? align_up((size_t)a.S * 8 * 4, kWsAlign) : 0;
  c.off_cand = c.off_surv = c.off_lg = off;
  if (topk) {
    // each workgroup's largest key per row; the kept keys past the LDS list
    // (at most min(k, workgroups) workgroups' keys); the logits when the
    // caller keeps none
    // one candidate row per workgroup of a slice (with K split, k_topk_reduce
    // forms them over the same tiles after adding the slices)
    const int nwg = a.rgroups;
    if (nwg > kTopkMaxWg)
      return fail(QG_EUNSUPPORTED, "%s: %d workgroups exceed the top-k selection's %d", fn, nwg, kTopkMaxWg);
    a.topk_tpw = (a.ntiles + a.rgroups * a.waves - 1) / (a.rgroups * a.waves);
    const long long keep = (long long)std::min(a.topk, nwg) * 16 * a.waves * a.topk_tpw;
    if (keep > 0x7FFFFFFFLL) return fail(QG_EUNSUPPORTED, "%s: V=%d too large for the top-k selection", fn, a.N);
    off += align_up((size_t)a.M * nwg * 8, kWsAlign);
    c.off_surv = off;
    off += align_up((size_t)a.M * (size_t)keep * 8, kWsAlign);
    c.off_lg = off;
    off += a.logits ? 0 : align_up((size_t)a.M * a.N * 4, kWsAlign);
  }
  c.scratch = off;
  return QG_OK;
}

// Shared by an entry point and its host-only twin: the plan for kMaxCus
// compute units (the largest scratch any device needs) and the workspace check.
qg_status affine_prepare(AffineCall& c, const char* fn, const void* ws, size_t ws_bytes, const BufList& bl) {
  qg_status st = affine_layout(c, fn, kMaxCus);
  if (st) return st;
  return check_ws(fn, ws, ws_bytes, ws_total(c.scratch, lm_fused(c)), bl.b, bl.n);
}

// Workspace bytes of an affine call of this shape (0 if it needs none or the
// shape has no plan; the entry point reports the latter).
size_t affine_query(AffineCall c, const char* fn) {
  if (c.a.M < 1 || c.a.M > 8 || c.a.N < 1 || c.a.K < 64 || c.a.K % 64) return 0;
  if (affine_layout(c, fn, kMaxCus)) return 0;
  return ws_total(c.scratch, lm_fused(c));
}

// After the checks: the plan's workgroup count for this device (the K split
// and so the scratch needed are unchanged), the scratch pointers, and the
// launch.  `pre` (if
// set) enqueues work that the projection reads (the RHT planes) and may
// change the arguments.
qg_status affine_launch(AffineCall c, const char* fn, void* ws, hipStream_t stream,
                        const std::function<int(unsigned char*, QgAffineArgs&)>& pre = nullptr) {
  qg_status st = affine_layout(c, fn, device_cus());
  if (st) return st;
  unsigned char* base = ws ? static_cast<unsigned char*>(ws) + kWsHeader : nullptr;
  if (pre) {
    const int err = pre(base, c.a);
    if (err) return fail(QG_EHIP, "%s: launch failed: %s", fn, hipGetErrorString((hipError_t)err));
  }
  if (lm_fused(c)) {
    if (!ws) return fail(QG_EINVAL, "%s: the greedy readout needs its workspace header", fn);
    c.a.state = static_cast<unsigned char*>(ws);
  }
  if (base) {
    c.a.part = reinterpret_cast<float*>(base + c.off_part);
    c.a.ssq_part = reinterpret_cast<float*>(base + c.off_ssq);
    c.a.cand = reinterpret_cast<unsigned long long*>(base + c.off_cand);
    c.a.surv = reinterpret_cast<unsigned long long*>(base + c.off_surv);
    // the top-k readout reads the logits back (from the scratch when the caller keeps none)
    if (c.a.topk > 0 && !c.a.logits) c.a.logits = reinterpret_cast<float*>(base + c.off_lg);
  }
  return launched(qg_launch_affine(c.mode, c.a, c.lds, stream), fn);
}

// ------------------------------------------------------------ Q4_K / Q6_K --
struct Q4kCall {
  QgQ4kArgs a{};
  size_t lds = 0, scratch = 0;
};

// Split plan of a Q4_K (bpb = 144) or Q6_K (bpb = 210) projection; the slice
// length is sized for 8 rows, so the split does not depend on M.
void q4k_layout(Q4kCall& c, int bpb) {
  QgQ4kArgs& a = c.a;
  a.nchunks = a.K / 256;
  a.ntiles = (a.N + 15) / 16;
  a.waves = kWaves;
  const size_t per8 = bpb == 144 ? q4k_lds_per_sb(8) : q6k_lds_per_sb(8);
  const size_t per = bpb == 144 ? q4k_lds_per_sb(a.M) : q6k_lds_per_sb(a.M);
  const int cps_max = (int)std::max<size_t>(1, std::min<size_t>((size_t)a.nchunks, (kQ4kLdsBudget - 16) / per8));
  // Both formats split for 4096 (tile, slice) pieces.  On 2560 x 12,800, 25
  // slices of two superblocks took 10.7-10.8 / 12.45 us (Q4_K) and 20.4 / 21.3
  // us (Q6_K) at M = 1 / 8, against 11.5 / 12.9 and 22.5 / 23.15 us with 13
  // slices of four (2048 pieces); 50 slices measured the same as 25 (Q4_K).
  Plan pl = plan_split(a.ntiles, a.nchunks, cps_max, true, 2 * kTargetWaves);
  a.S = pl.S;
  a.cps = pl.cps;
  a.tpw = pl.tpw;
  a.rgroups = pl.rgroups;
  c.lds = 16 + (size_t)a.cps * per;
  c.scratch = (a.S > 1) ? align_up((size_t)a.S * a.M * a.N * 4, kWsAlign) : 0;
}

// ------------------------------------------------------------------ MoE --
constexpr size_t kMoeRouteBytes = 512;  // selected ids [64] then their weights [64]
size_t moe_scratch(int top_k, int I) { return kMoeRouteBytes + align_up((size_t)top_k * I * 2, kWsAlign); }

// Measurement aid: a plain streaming read of a buffer (each workgroup reads
// consecutive 4-KB pieces, eight 16-byte non-temporal loads per lane in
// flight, grid-stride), so the HBM read rate of the device can be reported
// beside the kernels'.  The xor of the data goes to *sink only if it equals a
// value no buffer of ours produces, so the loads are kept.
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ p, size_t n16, unsigned* sink) {
  typedef unsigned u4v __attribute__((ext_vector_type(4)));
  uint32_t acc = 0;
  const size_t per = (size_t)8 * 256;
  for (size_t b = (size_t)blockIdx.x * per; b < n16; b += (size_t)gridDim.x * per) {
    u4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t i = std::min(b + (size_t)u * 256 + threadIdx.x, n16 - 1);
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p + i));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

// ------------------------------------------------ persistent MLP block --
constexpr int kMlpSpinLimit = 200000;  // polls of one wait before a workgroup gives up (tens of ms)

// The persistent MLP stack: L layers of stacked tile-order weights; gamma
// [L][D]; h [M][I] (scratch output, the last layer's h); ys [L][M][D] (layer
// l's output, layer l + 1's input).  L = 1 is mlp_block_affine4_tiled.
constexpr int kMaxLayers = 4096;

qg_status do_check_mlp(const char* fn, const uint16_t* x, const uint16_t* gamma, float eps,
                       const uint32_t* gu_codes_t, const uint16_t* gu_sb_t, const uint32_t* dn_codes_t,
                       const uint16_t* dn_sb_t, uint16_t* h, uint16_t* ys, int L, int M, int D, int I,
                       BufList* all = nullptr) {
  if (L < 1 || L > kMaxLayers) return fail(QG_EINVAL, "%s: L=%d must be in 1..%d", fn, L, kMaxLayers);
  if (M < 1 || M > 8) return fail(QG_EINVAL, "%s: M=%d must be in 1..8", fn, M);
  if (D <= 0 || D % 512 != 0) return fail(QG_EINVAL, "%s: D=%d must be a positive multiple of 512", fn, D);
  if (I <= 0 || I % 512 != 0) return fail(QG_EINVAL, "%s: I=%d must be a positive multiple of 512", fn, I);
  if ((long long)I * 2 * 16 > 0x7FFFFFFFLL || (long long)D * 16 > 0x7FFFFFFFLL)
    return fail(QG_EINVAL, "%s: D=%d or I=%d too large", fn, D, I);
  if (!(eps > 0.0f) || eps != eps || eps > 3.0e38f) return fail(QG_EINVAL, "%s: eps must be positive and finite", fn);
  const size_t l = (size_t)L;
  const Buf in[] = {{x, (size_t)M * D * 2, "x"},
                    {gamma, l * D * 2, "gamma"},
                    {gu_codes_t, l * tiled_codes_bytes(2 * I, D), "gu_codes_t"},
                    {gu_sb_t, l * tiled_sb_bytes(2 * I, D), "gu_sb_t"},
                    {dn_codes_t, l * tiled_codes_bytes(D, I), "dn_codes_t"},
                    {dn_sb_t, l * tiled_sb_bytes(D, I), "dn_sb_t"}};
  const Buf out[] = {{h, (size_t)M * I * 2, "h"}, {ys, l * M * D * 2, L > 1 ? "ys" : "y"}};
  qg_status st;
  for (const Buf& b : in)
    if ((st = check_ptr(b, 16, fn))) return st;
  if ((st = check_ptr(out[0], 16, fn)) || (st = check_ptr(out[1], 4, fn))) return st;
  collect(all, out, 2, in, 6);
  return check_alias(out, 2, in, 6, fn);
}

struct MlpCall {
  AffineCall gu, dn;  // gate/up (y = h) and down (x = h) plans
  size_t lds = 0, off_part_a = 0, off_ssq_a = 0, off_part_c = 0, scratch = 0;
};

qg_status mlp_layout(MlpCall& c, const char* fn, int cus) {
  qg_status st;
  if ((st = affine_layout(c.gu, fn, cus)) || (st = affine_layout(c.dn, fn, cus))) return st;
  c.lds = std::max(c.gu.lds, c.dn.lds);
  const QgAffineArgs &pa = c.gu.a, &pc = c.dn.a;
  c.off_part_a = 0;
  c.off_ssq_a = align_up((size_t)pa.S * pa.M * pa.N * 4, kWsAlign);
  c.off_part_c = c.off_ssq_a + align_up((size_t)pa.S * 8 * 4, kWsAlign);
  c.scratch = c.off_part_c + align_up((size_t)pc.S * pc.M * pc.N * 4, kWsAlign);
  return QG_OK;
}

void mlp_fill(MlpCall& c, const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* gu_codes_t,
              const uint16_t* gu_sb_t, const uint32_t* dn_codes_t, const uint16_t* dn_sb_t, uint16_t* h, uint16_t* y,
              int M, int D, int I) {
  QgAffineArgs& pa = c.gu.a;
  QgAffineArgs& pc = c.dn.a;
  c.gu.mode = QG_MODE_GATEUP;
  c.dn.mode = QG_MODE_PLAIN;
  pa.x = x;
  pa.gamma = gamma;
  pa.eps = eps;
  pa.codes = gu_codes_t;
  pa.scales = gu_sb_t;
  pa.biases = gu_sb_t;
  pa.tiled = 1;
  pa.y = h;
  pa.M = M;
  pa.N = 2 * I;
  pa.K = D;
  pc.x = h;
  pc.codes = dn_codes_t;
  pc.scales = dn_sb_t;
  pc.biases = dn_sb_t;
  pc.tiled = 1;
  pc.y = y;
  pc.M = M;
  pc.N = D;
  pc.K = I;
}

// Resident workgroups of the persistent kernel for M rows at this LDS size on
// the current device, rounded down to the barrier's 32 groups (0 if none).
int mlp_grid(int M, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_tuple(dev, M, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, qg_mlp_kernel(M), 256, lds) != hipSuccess) occ = 0;
  const int grid = occ < 1 ? 0 : device_cus() * std::min(occ, 4) / 32 * 32;
  cache[key] = grid;
  return grid;
}

}  // namespace

extern "C" {

qg_status qg_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  clear_err();
  if (!buf || !sink) return fail(QG_EINVAL, "qg_stream_read: null pointer");
  if (bytes < 16 || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4))
    return fail(QG_EINVAL, "qg_stream_read: bytes must be a positive multiple of 16 and buf 16-byte aligned");
  qg_status st;
  if ((st = check_device())) return st;
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>(8192, (n16 + 2047) / 2048);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, static_cast<const uint4*>(buf), n16,
                     sink);
  return launched((int)hipGetLastError(), "qg_stream_read");
}

const char* qg_status_string(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument (shape, null pointer, alignment or workspace size)";
    case QG_EALIAS: return "an output or the workspace overlaps an input or another output";
    case QG_EUNSUPPORTED: return "valid request with no kernel instance";
    case QG_EHIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

const char* qg_last_error(void) { return g_err; }

size_t qg_workspace_header_bytes(void) { return kWsHeader; }

// ------------------------------------------- mlp_block / mlp_stack_affine4 --
static qg_status prep_mlp(const char* fn, const uint16_t* x, const uint16_t* gamma, float eps,
                          const uint32_t* gu_codes_t, const uint16_t* gu_sb_t, const uint32_t* dn_codes_t,
                          const uint16_t* dn_sb_t, uint16_t* h, uint16_t* ys, int L, int M, int D, int I,
                          const void* ws, size_t ws_bytes, MlpCall& c) {
  BufList bl;
  qg_status st = do_check_mlp(fn, x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, ys, L, M, D, I, &bl);
  if (st) return st;
  mlp_fill(c, x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, ys, M, D, I);
  if ((st = mlp_layout(c, fn, kMaxCus))) return st;
  return check_ws(fn, ws, ws_bytes, ws_total(c.scratch, true), bl.b, bl.n);
}

static size_t mlp_query(int M, int D, int I) {
  if (M < 1 || M > 8 || D <= 0 || D % 512 || I <= 0 || I % 512) return 0;
  if ((long long)I * 2 * 16 > 0x7FFFFFFFLL || (long long)D * 16 > 0x7FFFFFFFLL) return 0;
  MlpCall c;
  mlp_fill(c, nullptr, nullptr, 1e-6f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, D, I);
  if (mlp_layout(c, "mlp_stack_affine4_tiled", kMaxCus)) return 0;
  return ws_total(c.scratch, true);
}

static qg_status run_mlp(const char* fn, const uint16_t* x, const uint16_t* gamma, float eps,
                         const uint32_t* gu_codes_t, const uint16_t* gu_sb_t, const uint32_t* dn_codes_t,
                         const uint16_t* dn_sb_t, uint16_t* h, uint16_t* ys, int L, int M, int D, int I, void* ws,
                         size_t ws_bytes, void* stream) {
  clear_err();
  MlpCall c;
  qg_status st = prep_mlp(fn, x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, ys, L, M, D, I, ws, ws_bytes,
                          c);
  if (st) return st;
  if ((st = check_device())) return st;
  if ((st = mlp_layout(c, fn, device_cus()))) return st;
  const int P = mlp_grid(M, c.lds);
  if (P < 32) return fail(QG_EUNSUPPORTED, "%s: fewer than 32 workgroups can be resident", fn);
  // every job of a phase gets its own resident workgroup when the plan allows
  QgAffineArgs pa = c.gu.a, pc = c.dn.a;
  pa.rgroups = std::max(1, std::min(P / pa.S, (pa.ntiles + kWaves - 1) / kWaves));
  pc.rgroups = std::max(1, std::min(P / pc.S, (pc.ntiles + kWaves - 1) / kWaves));
  unsigned char* base = static_cast<unsigned char*>(ws) + kWsHeader;
  pa.part = reinterpret_cast<float*>(base + c.off_part_a);
  pa.ssq_part = reinterpret_cast<float*>(base + c.off_ssq_a);
  pc.part = reinterpret_cast<float*>(base + c.off_part_c);
  QgMlpStack stk{};
  stk.L = L;
  stk.gu_codes = tiled_codes_bytes(2 * I, D) / 4;
  stk.gu_sb = tiled_sb_bytes(2 * I, D) / 2;
  stk.dn_codes = tiled_codes_bytes(D, I) / 4;
  stk.dn_sb = tiled_sb_bytes(D, I) / 2;
  stk.gamma = (size_t)D;
  stk.y = (size_t)M * D;
  return launched(qg_launch_mlp(pa, pc, stk, static_cast<unsigned char*>(ws), kMlpSpinLimit, P, c.lds,
                                (hipStream_t)stream),
                  fn);
}

size_t mlp_block_affine4_tiled_workspace(int M, int D, int I) { return mlp_query(M, D, I); }
size_t mlp_stack_affine4_tiled_workspace(int M, int D, int I) { return mlp_query(M, D, I); }

qg_status qg_check_mlp_block_affine4_tiled(const uint16_t* x, const uint16_t* gamma, float eps,
                                           const uint32_t* gu_codes_t, const uint16_t* gu_sb_t,
                                           const uint32_t* dn_codes_t, const uint16_t* dn_sb_t, uint16_t* h,
                                           uint16_t* y, int M, int D, int I, const void* ws, size_t ws_bytes) {
  clear_err();
  MlpCall c;
  return prep_mlp("mlp_block_affine4_tiled", x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, y, 1, M, D,
                  I, ws, ws_bytes, c);
}

qg_status mlp_block_affine4_tiled(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* gu_codes_t,
                                  const uint16_t* gu_sb_t, const uint32_t* dn_codes_t, const uint16_t* dn_sb_t,
                                  uint16_t* h, uint16_t* y, int M, int D, int I, void* ws, size_t ws_bytes,
                                  void* stream) {
  return run_mlp("mlp_block_affine4_tiled", x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, y, 1, M, D, I,
                 ws, ws_bytes, stream);
}

qg_status qg_check_mlp_stack_affine4_tiled(const uint16_t* x, const uint16_t* gamma, float eps,
                                           const uint32_t* gu_codes_t, const uint16_t* gu_sb_t,
                                           const uint32_t* dn_codes_t, const uint16_t* dn_sb_t, uint16_t* h,
                                           uint16_t* ys, int L, int M, int D, int I, const void* ws,
                                           size_t ws_bytes) {
  clear_err();
  MlpCall c;
  return prep_mlp("mlp_stack_affine4_tiled", x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, ys, L, M, D,
                  I, ws, ws_bytes, c);
}

qg_status mlp_stack_affine4_tiled(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* gu_codes_t,
                                  const uint16_t* gu_sb_t, const uint32_t* dn_codes_t, const uint16_t* dn_sb_t,
                                  uint16_t* h, uint16_t* ys, int L, int M, int D, int I, void* ws, size_t ws_bytes,
                                  void* stream) {
  return run_mlp("mlp_stack_affine4_tiled", x, gamma, eps, gu_codes_t, gu_sb_t, dn_codes_t, dn_sb_t, h, ys, L, M, D,
                 I, ws, ws_bytes, stream);
}

int32_t mlp_block_affine4_tiled_failures(void* ws, void* stream) {
  clear_err();
  if (!ws) return -1;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return -1;
  uint32_t v = 0, zero = 0;
  unsigned char* cnt = static_cast<unsigned char*>(ws) + 20;
  if (hipMemcpy(&v, cnt, 4, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  if (v && hipMemcpy(cnt, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return -1;
  return (int32_t)v;
}

// ------------------------------------------------------------ qgemv_affine4 --
static qg_status prep_qgemv_affine4(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* biases, uint16_t* y, int M, int N, int K, const void* ws,
                                    size_t ws_bytes, AffineCall& c, const char* fn = "qgemv_affine4") {
  BufList bl;
  qg_status st = do_check_qgemv_affine4(x, codes, scales, biases, y, M, N, K, &bl);
  if (st || N == 0) return st;
  c.mode = QG_MODE_PLAIN;
  QgAffineArgs& a = c.a;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return affine_prepare(c, fn, ws, ws_bytes, bl);
}

size_t qgemv_affine4_workspace(int M, int N, int K) {
  AffineCall c;
  c.a.M = M;
  c.a.N = N;
  c.a.K = K;
  return affine_query(c, "qgemv_affine4");
}

qg_status qg_check_qgemv_affine4(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, const void* ws,
                                 size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_qgemv_affine4(x, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
}

qg_status qgemv_affine4(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                        uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_qgemv_affine4(x, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "qgemv_affine4", ws, (hipStream_t)stream);
}

// The same projection with the products on the vector ALU (measurement aid):
// qgemv_affine4's plan, arguments and workspace.
size_t qg_affine4_valu_workspace(int M, int N, int K) { return qgemv_affine4_workspace(M, N, K); }

qg_status qg_affine4_valu(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                          uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "qg_affine4_valu";
  clear_err();
  AffineCall c;
  qg_status st = prep_qgemv_affine4(x, codes, scales, biases, y, M, N, K, ws, ws_bytes, c, fn);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  if ((st = affine_layout(c, fn, device_cus()))) return st;
  if (qg_valu_lds_bytes(c.a.M, c.a.cps) > c.lds) return fail(QG_EUNSUPPORTED, "%s: slice does not fit", fn);
  if (ws) c.a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kWsHeader + c.off_part);
  return launched(qg_launch_affine_valu(c.a, (hipStream_t)stream), fn);
}

// ------------------------------------------------------------ qgemv_affine8 --
static qg_status prep_qgemv_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* biases, uint16_t* y, int M, int N, int K, const void* ws,
                                    size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_qgemv_affine8(x, codes, scales, biases, y, M, N, K, &bl);
  if (st || N == 0) return st;
  c.mode = QG_MODE_PLAIN8;
  QgAffineArgs& a = c.a;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return affine_prepare(c, "qgemv_affine8", ws, ws_bytes, bl);
}

size_t qgemv_affine8_workspace(int M, int N, int K) {
  AffineCall c;
  c.mode = QG_MODE_PLAIN8;
  c.a.M = M;
  c.a.N = N;
  c.a.K = K;
  return affine_query(c, "qgemv_affine8");
}

qg_status qg_check_qgemv_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* biases, uint16_t* y, int M, int N, int K, const void* ws,
                                 size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_qgemv_affine8(x, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
}

qg_status qgemv_affine8(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                        uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_qgemv_affine8(x, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "qgemv_affine8", ws, (hipStream_t)stream);
}

// -------------------------------------------------------- qgemv_affine4_rht --
static qg_status prep_rht(const uint16_t* x, const int8_t* signs, int had, const uint32_t* codes,
                          const uint16_t* scales, const uint16_t* biases, uint16_t* y, int M, int N, int K,
                          const void* ws, size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_qgemv_affine4_rht(x, signs, had, codes, scales, biases, y, M, N, K, &bl);
  if (st || N == 0) return st;
  c.mode = QG_MODE_PLANES;
  QgAffineArgs& a = c.a;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  c.reserve = 2 * align_up((size_t)M * K * 2, kWsAlign);  // the transformed rows: hi and lo bf16 planes
  return affine_prepare(c, "qgemv_affine4_rht", ws, ws_bytes, bl);
}

size_t qgemv_affine4_rht_workspace(int M, int N, int K) {
  if (M < 1 || M > 8 || K < 64 || K % 64) return 0;
  AffineCall c;
  c.mode = QG_MODE_PLANES;
  c.a.M = M;
  c.a.N = N;
  c.a.K = K;
  c.reserve = 2 * align_up((size_t)M * K * 2, kWsAlign);
  return N < 1 ? 0 : affine_query(c, "qgemv_affine4_rht");
}

qg_status qg_check_qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had, const uint32_t* codes,
                                     const uint16_t* scales, const uint16_t* biases, uint16_t* y, int M, int N, int K,
                                     const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_rht(x, signs, had, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
}

qg_status qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, uint16_t* y, int M, int N, int K,
                            void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_rht(x, signs, had, codes, scales, biases, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const size_t plane_al = align_up((size_t)M * K * 2, kWsAlign);
  return affine_launch(c, "qgemv_affine4_rht", ws, s, [&](unsigned char* base, QgAffineArgs& args) {
    uint16_t* hi = reinterpret_cast<uint16_t*>(base);
    uint16_t* lo = reinterpret_cast<uint16_t*>(base + plane_al);
    args.x = hi;
    args.x_lo = lo;
    return qg_launch_rht(x, signs, had, M, K, hi, lo, s);
  });
}

// --------------------------------------------------------------- tile order --
size_t qg_tiled_bytes(int N, int K, size_t* sb_bytes) {
  if (N < 1 || K <= 0 || K % 512 != 0) {
    if (sb_bytes) *sb_bytes = 0;
    return 0;
  }
  if (sb_bytes) *sb_bytes = tiled_sb_bytes(N, K);
  return tiled_codes_bytes(N, K);
}

qg_status qg_check_affine4_tile_pack(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                                     uint32_t* codes_t, uint16_t* sb_t, int N, int K) {
  clear_err();
  return do_check_tile_pack(codes, scales, biases, codes_t, sb_t, N, K);
}

qg_status affine4_tile_pack(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, uint32_t* codes_t,
                            uint16_t* sb_t, int N, int K, void* stream) {
  clear_err();
  qg_status st = do_check_tile_pack(codes, scales, biases, codes_t, sb_t, N, K);
  if (st) return st;
  if ((st = check_device())) return st;
  return launched(qg_launch_tile_pack(codes, scales, biases, codes_t, sb_t, N, K, (hipStream_t)stream),
                  "affine4_tile_pack");
}

static qg_status prep_affine4_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, uint16_t* y,
                                    int M, int N, int K, const void* ws, size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_qgemv_affine4_tiled(x, codes_t, sb_t, y, M, N, K, &bl);
  if (st || N == 0) return st;
  c.mode = QG_MODE_PLAIN;
  QgAffineArgs& a = c.a;
  a.x = x;
  a.codes = codes_t;
  a.scales = sb_t;
  a.biases = sb_t;
  a.tiled = 1;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return affine_prepare(c, "qgemv_affine4_tiled", ws, ws_bytes, bl);
}

size_t qgemv_affine4_tiled_workspace(int M, int N, int K) {
  if (K % 512) return 0;
  AffineCall c;
  c.a.tiled = 1;
  c.a.M = M;
  c.a.N = N;
  c.a.K = K;
  return affine_query(c, "qgemv_affine4_tiled");
}

qg_status qg_check_qgemv_affine4_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, uint16_t* y,
                                       int M, int N, int K, const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_affine4_tiled(x, codes_t, sb_t, y, M, N, K, ws, ws_bytes, c);
}

qg_status qgemv_affine4_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, uint16_t* y, int M,
                              int N, int K, void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_affine4_tiled(x, codes_t, sb_t, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "qgemv_affine4_tiled", ws, (hipStream_t)stream);
}

// ---------------------------------------------------- rmsnorm_gateup_swiglu --
static void fill_gateup(AffineCall& c, const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes,
                        const uint16_t* scales, const uint16_t* biases, uint16_t* h, int M, int I, int K, int tiled) {
  c.mode = QG_MODE_GATEUP;
  QgAffineArgs& a = c.a;
  a.x = x;
  a.gamma = gamma;
  a.eps = eps;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.tiled = tiled;
  a.y = h;
  a.M = M;
  a.N = 2 * I;  // gate rows then up rows, one matrix for the projection kernel
  a.K = K;
}

static qg_status prep_gateup(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes,
                             const uint16_t* scales, const uint16_t* biases, uint16_t* h, int M, int I, int K,
                             const void* ws, size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_gateup(x, gamma, eps, codes, scales, biases, h, M, I, K, &bl);
  if (st || I == 0) return st;
  fill_gateup(c, x, gamma, eps, codes, scales, biases, h, M, I, K, 0);
  return affine_prepare(c, "rmsnorm_gateup_swiglu", ws, ws_bytes, bl);
}

static qg_status prep_gateup_tiled(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes_t,
                                   const uint16_t* sb_t, uint16_t* h, int M, int I, int K, const void* ws,
                                   size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_gateup_tiled(x, gamma, eps, codes_t, sb_t, h, M, I, K, &bl);
  if (st) return st;
  fill_gateup(c, x, gamma, eps, codes_t, sb_t, sb_t, h, M, I, K, 1);
  return affine_prepare(c, "rmsnorm_gateup_swiglu_tiled", ws, ws_bytes, bl);
}

// I in range for the fused [2I][K] matrix (2I rows of 16-row tiles in an int)
static bool gateup_rows_ok(int I) { return I >= 1 && (long long)I * 2 * 16 <= 0x7FFFFFFFLL; }

size_t rmsnorm_gateup_swiglu_workspace(int M, int I, int K) {
  if (!gateup_rows_ok(I)) return 0;
  AffineCall c;
  fill_gateup(c, nullptr, nullptr, 1e-6f, nullptr, nullptr, nullptr, nullptr, M, I, K, 0);
  return affine_query(c, "rmsnorm_gateup_swiglu");
}

size_t rmsnorm_gateup_swiglu_tiled_workspace(int M, int I, int K) {
  if (K % 512 || !gateup_rows_ok(I)) return 0;
  AffineCall c;
  fill_gateup(c, nullptr, nullptr, 1e-6f, nullptr, nullptr, nullptr, nullptr, M, I, K, 1);
  return affine_query(c, "rmsnorm_gateup_swiglu_tiled");
}

qg_status qg_check_rmsnorm_gateup_swiglu(const uint16_t* x, const uint16_t* gamma, float eps,
                                         const uint32_t* codes_gu, const uint16_t* scales_gu,
                                         const uint16_t* biases_gu, uint16_t* h, int M, int I, int K, const void* ws,
                                         size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_gateup(x, gamma, eps, codes_gu, scales_gu, biases_gu, h, M, I, K, ws, ws_bytes, c);
}

qg_status rmsnorm_gateup_swiglu(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes_gu,
                                const uint16_t* scales_gu, const uint16_t* biases_gu, uint16_t* h, int M, int I,
                                int K, void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_gateup(x, gamma, eps, codes_gu, scales_gu, biases_gu, h, M, I, K, ws, ws_bytes, c);
  if (st || I == 0) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "rmsnorm_gateup_swiglu", ws, (hipStream_t)stream);
}

qg_status qg_check_rmsnorm_gateup_swiglu_tiled(const uint16_t* x, const uint16_t* gamma, float eps,
                                               const uint32_t* codes_t, const uint16_t* sb_t, uint16_t* h, int M,
                                               int I, int K, const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_gateup_tiled(x, gamma, eps, codes_t, sb_t, h, M, I, K, ws, ws_bytes, c);
}

qg_status rmsnorm_gateup_swiglu_tiled(const uint16_t* x, const uint16_t* gamma, float eps, const uint32_t* codes_t,
                                      const uint16_t* sb_t, uint16_t* h, int M, int I, int K, void* ws,
                                      size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_gateup_tiled(x, gamma, eps, codes_t, sb_t, h, M, I, K, ws, ws_bytes, c);
  if (st) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "rmsnorm_gateup_swiglu_tiled", ws, (hipStream_t)stream);
}

// ------------------------------------------------------------- lmhead_argmax --
static void fill_lmhead(AffineCall& c, const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                        const uint16_t* biases, float* logits, int32_t* ids, const int32_t* draft, int32_t* accepted,
                        int M, int V, int K, int tiled) {
  c.mode = QG_MODE_LMHEAD;
  QgAffineArgs& a = c.a;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  a.biases = biases;
  a.tiled = tiled;
  a.logits = logits;
  a.ids = ids;
  a.draft = draft;
  a.accepted = accepted;
  a.M = M;
  a.N = V;
  a.K = K;
}

static qg_status prep_lmhead(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                             float* logits, int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V,
                             int K, const void* ws, size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_lmhead(x, codes, scales, biases, logits, ids, draft, accepted, M, V, K, &bl);
  if (st) return st;
  fill_lmhead(c, x, codes, scales, biases, logits, ids, draft, accepted, M, V, K, 0);
  return affine_prepare(c, "lmhead_argmax", ws, ws_bytes, bl);
}

static qg_status prep_lmhead_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, float* logits,
                                   int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V, int K,
                                   const void* ws, size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_lmhead_tiled(x, codes_t, sb_t, logits, ids, draft, accepted, M, V, K, &bl);
  if (st) return st;
  fill_lmhead(c, x, codes_t, sb_t, sb_t, logits, ids, draft, accepted, M, V, K, 1);
  return affine_prepare(c, "lmhead_argmax_tiled", ws, ws_bytes, bl);
}

size_t lmhead_argmax_workspace(int M, int V, int K) {
  AffineCall c;
  fill_lmhead(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, V, K, 0);
  return affine_query(c, "lmhead_argmax");
}

size_t lmhead_argmax_tiled_workspace(int M, int V, int K) {
  if (K % 512) return 0;
  AffineCall c;
  fill_lmhead(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, V, K, 1);
  return affine_query(c, "lmhead_argmax_tiled");
}

qg_status qg_check_lmhead_argmax(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* biases, float* logits, int32_t* ids, const int32_t* draft,
                                 int32_t* accepted, int M, int V, int K, const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_lmhead(x, codes, scales, biases, logits, ids, draft, accepted, M, V, K, ws, ws_bytes, c);
}

qg_status lmhead_argmax(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                        float* logits, int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V, int K,
                        void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_lmhead(x, codes, scales, biases, logits, ids, draft, accepted, M, V, K, ws, ws_bytes, c);
  if (st) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "lmhead_argmax", ws, (hipStream_t)stream);
}

// ----------------------------------------------------- lmhead_argmax_static --
// lmhead_argmax for callers that cannot allocate device memory: the scratch
// it needs (the workspace header: every row's running (logit, index) maximum
// and the workgroups' arrival counter) is this file-scope device array, one
// copy per GPU, zero when the library is loaded and left at zero by every
// call.  Its device address is looked up once per device (hipGetSymbolAddress
// with that device current) and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = kWsHeader;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {nullptr};

static qg_status static_scratch(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QG_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(QG_EUNSUPPORTED, "%s: device index %d out of range", fn, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QG_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}

qg_status lmhead_argmax_static(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, float* logits, int32_t* ids, const int32_t* draft,
                               int32_t* accepted, int M, int V, int K, void* stream) {
  const char* fn = "lmhead_argmax_static";
  clear_err();
  const size_t need = lmhead_argmax_workspace(M, V, K);
  if (need > kStaticScratchBytes)
    return fail(QG_EUNSUPPORTED, "%s: M=%d V=%d K=%d needs %zu bytes of scratch, the static array holds %zu", fn, M,
                V, K, need, kStaticScratchBytes);
  qg_status st;
  if ((st = check_device())) return st;
  void* ptr = nullptr;
  if ((st = static_scratch(fn, &ptr))) return st;
  AffineCall c;
  st = prep_lmhead(x, codes, scales, biases, logits, ids, draft, accepted, M, V, K, ptr, kStaticScratchBytes, c);
  if (st) return st;
  return affine_launch(c, fn, ptr, (hipStream_t)stream);
}

qg_status qg_check_lmhead_argmax_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t,
                                       float* logits, int32_t* ids, const int32_t* draft, int32_t* accepted, int M,
                                       int V, int K, const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_lmhead_tiled(x, codes_t, sb_t, logits, ids, draft, accepted, M, V, K, ws, ws_bytes, c);
}

qg_status lmhead_argmax_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, float* logits,
                              int32_t* ids, const int32_t* draft, int32_t* accepted, int M, int V, int K, void* ws,
                              size_t ws_bytes, void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_lmhead_tiled(x, codes_t, sb_t, logits, ids, draft, accepted, M, V, K, ws, ws_bytes, c);
  if (st) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "lmhead_argmax_tiled", ws, (hipStream_t)stream);
}

// --------------------------------------------------------------- lmhead_topk --
static qg_status prep_topk(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                           float* logits, int32_t* ids, float* vals, int M, int V, int K, int k, const void* ws,
                           size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_lmhead_topk(x, codes, scales, biases, logits, ids, vals, M, V, K, k, &bl);
  if (st) return st;
  fill_lmhead(c, x, codes, scales, biases, logits, ids, nullptr, nullptr, M, V, K, 0);
  c.a.topk = k;
  c.a.topk_vals = vals;
  return affine_prepare(c, "lmhead_topk", ws, ws_bytes, bl);
}

size_t lmhead_topk_workspace(int M, int V, int K, int k, int logits_kept) {
  if (k < 1 || k > kTopkMax) return 0;
  AffineCall c;
  fill_lmhead(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, V, K, 0);
  c.a.topk = k;
  c.a.logits = logits_kept ? reinterpret_cast<float*>(kWsAlign) : nullptr;  // only its presence matters here
  return affine_query(c, "lmhead_topk");
}

qg_status qg_check_lmhead_topk(const uint16_t* x, const uint32_t* codes, const uint16_t* scales,
                               const uint16_t* biases, float* logits, int32_t* ids, float* vals, int M, int V, int K,
                               int k, const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_topk(x, codes, scales, biases, logits, ids, vals, M, V, K, k, ws, ws_bytes, c);
}

qg_status lmhead_topk(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                      float* logits, int32_t* ids, float* vals, int M, int V, int K, int k, void* ws, size_t ws_bytes,
                      void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_topk(x, codes, scales, biases, logits, ids, vals, M, V, K, k, ws, ws_bytes, c);
  if (st) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "lmhead_topk", ws, (hipStream_t)stream);
}

static qg_status prep_topk_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, float* logits,
                                 int32_t* ids, float* vals, int M, int V, int K, int k, const void* ws,
                                 size_t ws_bytes, AffineCall& c) {
  BufList bl;
  qg_status st = do_check_lmhead_topk_tiled(x, codes_t, sb_t, logits, ids, vals, M, V, K, k, &bl);
  if (st) return st;
  fill_lmhead(c, x, codes_t, sb_t, sb_t, logits, ids, nullptr, nullptr, M, V, K, 1);
  c.a.topk = k;
  c.a.topk_vals = vals;
  return affine_prepare(c, "lmhead_topk_tiled", ws, ws_bytes, bl);
}

size_t lmhead_topk_tiled_workspace(int M, int V, int K, int k, int logits_kept) {
  if (k < 1 || k > kTopkMax || K % 512) return 0;
  AffineCall c;
  fill_lmhead(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, V, K, 1);
  c.a.topk = k;
  c.a.logits = logits_kept ? reinterpret_cast<float*>(kWsAlign) : nullptr;  // only its presence matters here
  return affine_query(c, "lmhead_topk_tiled");
}

qg_status qg_check_lmhead_topk_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t,
                                     float* logits, int32_t* ids, float* vals, int M, int V, int K, int k,
                                     const void* ws, size_t ws_bytes) {
  clear_err();
  AffineCall c;
  return prep_topk_tiled(x, codes_t, sb_t, logits, ids, vals, M, V, K, k, ws, ws_bytes, c);
}

qg_status lmhead_topk_tiled(const uint16_t* x, const uint32_t* codes_t, const uint16_t* sb_t, float* logits,
                            int32_t* ids, float* vals, int M, int V, int K, int k, void* ws, size_t ws_bytes,
                            void* stream) {
  clear_err();
  AffineCall c;
  qg_status st = prep_topk_tiled(x, codes_t, sb_t, logits, ids, vals, M, V, K, k, ws, ws_bytes, c);
  if (st) return st;
  if ((st = check_device())) return st;
  return affine_launch(c, "lmhead_topk_tiled", ws, (hipStream_t)stream);
}

// ------------------------------------------------------- qgemv_q4k / q6k --
static qg_status prep_q4k(int bpb, const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K,
                          const void* ws, size_t ws_bytes, Q4kCall& c) {
  const char* fn = bpb == 144 ? "qgemv_q4k" : "qgemv_q6k";
  BufList bl;
  qg_status st = bpb == 144 ? do_check_qgemv_q4k(x, blocks, y, M, N, K, &bl)
                            : do_check_qgemv_q6k(x, blocks, y, M, N, K, &bl);
  if (st || N == 0) return st;
  QgQ4kArgs& a = c.a;
  a.x = x;
  a.blocks = blocks;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  q4k_layout(c, bpb);
  return check_ws(fn, ws, ws_bytes, ws_total(c.scratch), bl.b, bl.n);
}

static size_t q4k_query(int bpb, int M, int N, int K) {
  if (M < 1 || M > 8 || N < 1 || K < 256 || K % 256) return 0;
  Q4kCall c;
  c.a.M = M;
  c.a.N = N;
  c.a.K = K;
  q4k_layout(c, bpb);
  return ws_total(c.scratch);
}

size_t qgemv_q4k_workspace(int M, int N, int K) { return q4k_query(144, M, N, K); }
size_t qgemv_q6k_workspace(int M, int N, int K) { return q4k_query(210, M, N, K); }

qg_status qg_check_qgemv_q4k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K,
                             const void* ws, size_t ws_bytes) {
  clear_err();
  Q4kCall c;
  return prep_q4k(144, x, blocks, y, M, N, K, ws, ws_bytes, c);
}

qg_status qg_check_qgemv_q6k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K,
                             const void* ws, size_t ws_bytes) {
  clear_err();
  Q4kCall c;
  return prep_q4k(210, x, blocks, y, M, N, K, ws, ws_bytes, c);
}

qg_status qgemv_q4k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K, void* ws,
                    size_t ws_bytes, void* stream) {
  clear_err();
  Q4kCall c;
  qg_status st = prep_q4k(144, x, blocks, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  if (ws) c.a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kWsHeader);
  return launched(qg_launch_q4k(c.a, c.lds, (hipStream_t)stream), "qgemv_q4k");
}

qg_status qgemv_q6k(const uint16_t* x, const uint8_t* blocks, uint16_t* y, int M, int N, int K, void* ws,
                    size_t ws_bytes, void* stream) {
  clear_err();
  Q4kCall c;
  qg_status st = prep_q4k(210, x, blocks, y, M, N, K, ws, ws_bytes, c);
  if (st || N == 0) return st;
  if ((st = check_device())) return st;
  if (ws) c.a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kWsHeader);
  return launched(qg_launch_q6k(c.a, c.lds, (hipStream_t)stream), "qgemv_q6k");
}

// --------------------------------------------------------- moe_expert_qgemv --
static qg_status prep_moe(const uint16_t* x, const float* logits, int top_k, const uint8_t* w_gu,
                          const uint8_t* w_down, uint16_t* y, int32_t* out_ids, float* out_w, int E, int D, int I,
                          const void* ws, size_t ws_bytes) {
  BufList bl;
  qg_status st = do_check_moe(x, logits, top_k, w_gu, w_down, y, out_ids, out_w, E, D, I, &bl);
  if (st) return st;
  return check_ws("moe_expert_qgemv", ws, ws_bytes, ws_total(moe_scratch(top_k, I)), bl.b, bl.n);
}

size_t moe_expert_qgemv_workspace(int top_k, int E, int D, int I) {
  if (top_k < 1 || top_k > 64 || top_k > E || I < 256 || I % 256 || D < 256 || D % 256) return 0;
  return ws_total(moe_scratch(top_k, I));
}

qg_status qg_check_moe_expert_qgemv(const uint16_t* x, const float* router_logits, int top_k, const uint8_t* w_gu,
                                    const uint8_t* w_down, uint16_t* y, int32_t* out_ids, float* out_w, int E, int D,
                                    int I, const void* ws, size_t ws_bytes) {
  clear_err();
  return prep_moe(x, router_logits, top_k, w_gu, w_down, y, out_ids, out_w, E, D, I, ws, ws_bytes);
}

qg_status moe_expert_qgemv(const uint16_t* x, const float* router_logits, int top_k, const uint8_t* w_gu,
                           const uint8_t* w_down, uint16_t* y, int32_t* out_ids, float* out_w, int E, int D, int I,
                           void* ws, size_t ws_bytes, void* stream) {
  clear_err();
  qg_status st = prep_moe(x, router_logits, top_k, w_gu, w_down, y, out_ids, out_w, E, D, I, ws, ws_bytes);
  if (st) return st;
  if ((st = check_device())) return st;
  unsigned char* base = static_cast<unsigned char*>(ws) + kWsHeader;
  QgMoeArgs a{};
  a.x = x;
  a.logits = router_logits;
  a.top_k = top_k;
  a.w_gu = w_gu;
  a.w_down = w_down;
  a.y = y;
  a.out_ids = out_ids;
  a.out_w = out_w;
  a.route_ids = reinterpret_cast<int32_t*>(base);   // 64 entries
  a.route_w = reinterpret_cast<float*>(base + 256);  // 64 entries
  a.h = reinterpret_cast<uint16_t*>(base + kMoeRouteBytes);
  a.E = E;
  a.D = D;
  a.I = I;
  return launched(qg_launch_moe(a, (hipStream_t)stream), "moe_expert_qgemv");
}

}  // extern "C"
