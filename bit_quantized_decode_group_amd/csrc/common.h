// common.h -- device helpers and launch descriptors shared by the gfx950
// kernels of libqgemv.so.  Internal to the library.
//
// Operand scheme used by every projection kernel
// ----------------------------------------------
// The reduction runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
//   A (16 x 32)  = activation rows (one MFMA row per activation row m < M),
//   B (32 x 16)  = 16 weight rows n of the current tile,
//   C (16 x 16)  = fp32 partial sums.
// Lane l of a wave holds A row l%16, B column l%16 and k-slots 8*(l/16)..+7 of
// both operands; it receives C rows 4*(l/16)..+3 of column l%16.
//
// Exact operands: a 4-bit code q becomes the bf16 bit pattern 0x4300|q, which
// is exactly 128+q, so no dequantised weight is ever rounded.  The activation
// is bf16 already.  The offset and the per-group affine are applied to the
// fp32 group sums afterwards:  sum_k x*(s*q+b) = s*D + (b-128*s)*sum_k x,
// with D = sum_k x*(128+q) coming from the MFMA.
//
// Two scale groups per MFMA: decode activations have M <= 8 rows but the MFMA
// has 16.  Rows 0..7 carry group g and rows 8..15 carry group g+1; the k-slots
// of lanes 0..31 (l/16 in {0,1}) hold codes of group g and those of lanes
// 32..63 codes of group g+1, and the activation row of the other group is zero
// in those slots.  After the MFMAs of one "chunk" (two groups), lanes 0..31
// hold group g's sums and lanes 32..63 group g+1's, so every lane applies one
// scale and one bias; the two halves are added once per tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 16-byte load of weight bytes, each read exactly once.  NT: a non-temporal
// (streaming) load, which does not keep the line in the caches it passes
// through.  Measured on MI355X: a plain streaming read reaches 6.8-6.9 TB/s
// with non-temporal loads against 6.0-6.1 TB/s with ordinary ones, and the
// long LM-head stream gains from them; kernels whose waves live for a few
// steps only (the split projections, the MoE) lose (their first loads wait
// longer), so they use ordinary loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld_weights(const void* ptr) {
  u32x4_t v;
  if constexpr (NT)
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  else
    v = *reinterpret_cast<const u32x4_t*>(ptr);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same 16-byte weight load through a buffer resource (raw, untyped:
// stride 0, gfx9's third descriptor word) over `bytes` bytes from `base`.  A
// buffer load whose offset lies past the resource's size reads no memory and
// returns zero, so a resource of zero bytes turns the load into one that is
// still issued (the compiler's count of loads in flight stays exact) but moves
// nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <bool NT>
__device__ __forceinline__ uint4 ld_weights(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// v + (the value of lane l ^ 32) for lanes 0..31, on the VALU (gfx950's
// v_permlane32_swap exchanges the wave's two 32-lane halves) instead of an
// LDS permute.  Each result is one addition of the same two values, so it
// equals v + __shfl_xor(v, 32) bit for bit.
__device__ __forceinline__ float add_upper_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v + (the value of lane l ^ 16), on the VALU (v_permlane16_swap exchanges
// the odd and even 16-lane rows); equal to v + __shfl_xor(v, 16) bit for bit.
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v + (the value of lane l ^ 8): a rotation by 8 inside each 16-lane row (DPP
// row_ror:8) is the lane l ^ 8; equal to v + __shfl_xor(v, 8) bit for bit.
__device__ __forceinline__ float add_xor8(float v) {
  const int r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false);
  return v + __int_as_float(r);
}

// The value of lane lane ^ S (S = 1, 2, 8: DPP quad permutes and a rotation
// by 8 in each row of 16; S = 4: a swizzle).
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (S == 4) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);
  } else {
    static_assert(S == 1 || S == 2 || S == 8, "lane distance");
    constexpr int ctrl = S == 1 ? 0xB1 : S == 2 ? 0x4E : 0x128;  // quad_perm [1,0,3,2], [2,3,0,1]; row_ror:8
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
  }
}

// v summed over the P neighbouring lanes of its group (P a power of two <= 64,
// uniform); distances 16 and 32 go through the permlane swaps, which return
// this lane's value and its partner's in either order.
__device__ __forceinline__ uint32_t group_sum(uint32_t v, unsigned P) {
  if (P > 1) v += lane_xor<1>(v);
  if (P > 2) v += lane_xor<2>(v);
  if (P > 4) v += lane_xor<4>(v);
  if (P > 8) v += lane_xor<8>(v);
  if (P > 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = r[0] + r[1];
  }
  if (P > 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = r[0] + r[1];
  }
  return v;
}

// Two fp32 values as bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32),
// `lo` in the low half; the same bits as f32_to_bf16_bits for every non-NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// a.lo*b.lo + a.hi*b.hi + c for two packed bf16 pairs (v_dot2_f32_bf16): the
// products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The index of the calling wave in its workgroup, as a scalar (wave-uniform
// values derived from it, such as tile and step counters and the address
// arithmetic built on them, then stay on the scalar unit).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN, overflow -> inf.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The unpack constants, materialised once in vector registers: an and-or of
// three vector operands is one instruction (v_and_or_b32), while with both
// constants as literals or scalars it splits into two (a VOP3 instruction
// reads at most one scalar or literal operand).  Non-volatile, so the
// compiler hoists it.
struct UnpackK {
  uint32_t mask, one28;
};
__device__ __forceinline__ UnpackK unpack_constants() {
  UnpackK k;
  asm("v_mov_b32 %0, %1" : "=v"(k.mask) : "i"(0x000F000F));
  asm("v_mov_b32 %0, %1" : "=v"(k.one28) : "i"(0x43004300));
  return k;
}

// Eight affine codes of one little-endian word (code i at bits 4i..4i+3) as
// eight bf16 values 128+q (0x4300 | q).  Element 2j (low half of dword j) is
// code j and element 2j+1 (high half) is code j+4, so MFMA k-slot s holds
// code s/2 + 4*(s%2).
__device__ __forceinline__ uint4 unpack_affine_word(uint32_t w, const UnpackK& k) {
  uint4 r;
  r.x = (w & k.mask) | k.one28;
  r.y = ((w >> 4) & k.mask) | k.one28;
  r.z = ((w >> 8) & k.mask) | k.one28;
  r.w = ((w >> 12) & k.mask) | k.one28;
  return r;
}

// Eight affine 8-bit codes (bytes of w0 = codes 0..3, w1 = codes 4..7, least
// significant byte first) as eight bf16 values q: a byte converts to fp32
// exactly and its upper half is the exact bf16 (q has at most 8 significant
// bits).  As in unpack_affine_word, dword j holds code j (low half) and code
// j+4 (high half).
__device__ __forceinline__ uint32_t bf16_pair_of_floats(float lo, float hi) {
  // bytes 2,3 of lo, then bytes 2,3 of hi (v_perm_b32: selectors 0..3 pick the
  // second operand's bytes, 4..7 the first's)
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ uint4 unpack_affine8_pair(uint32_t w0, uint32_t w1) {
  uint4 r;
  r.x = bf16_pair_of_floats((float)(w0 & 0xFFu), (float)(w1 & 0xFFu));
  r.y = bf16_pair_of_floats((float)((w0 >> 8) & 0xFFu), (float)((w1 >> 8) & 0xFFu));
  r.z = bf16_pair_of_floats((float)((w0 >> 16) & 0xFFu), (float)((w1 >> 16) & 0xFFu));
  r.w = bf16_pair_of_floats((float)(w0 >> 24), (float)(w1 >> 24));
  return r;
}

// Eight Q4_K codes from eight consecutive code bytes (w0 = bytes 0..3, w1 =
// bytes 4..7): the low nibbles when sh == 0, the high nibbles when sh == 4.
// Slot s holds the code of byte {0,2,1,3,4,6,5,7}[s].
__device__ __forceinline__ uint4 unpack_q4k_bytes(uint32_t w0, uint32_t w1, uint32_t sh, const UnpackK& k) {
  const uint32_t m = k.mask, one28 = k.one28;
  uint4 r;
  r.x = ((w0 >> sh) & m) | one28;
  r.y = ((w0 >> (sh + 8u)) & m) | one28;
  r.z = ((w1 >> sh) & m) | one28;
  r.w = ((w1 >> (sh + 8u)) & m) | one28;
  return r;
}

// Order-preserving key of (logit, index) for a max-reduction: a larger value
// wins, then a lower index; any NaN beats every number (the first NaN wins);
// -0 and +0 compare equal.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  uint32_t fk;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) fk = 0xFFFFFFFFu;
  else if ((u & 0x7FFFFFFFu) == 0u) fk = 0x80000000u;
  else fk = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)fk << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

// The logit of an argmax_key: the exact value for every number (-0 comes back
// as +0), a quiet NaN for a NaN.
__device__ __forceinline__ float key_logit(unsigned long long key) {
  const uint32_t fk = (uint32_t)(key >> 32);
  if (fk == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((fk & 0x80000000u) ? (fk & 0x7FFFFFFFu) : ~fk);
}

}  // namespace qg

// ------------------------------------------------------ workspace header ---
// The first kWsHeader bytes of a caller's workspace hold state that is zero
// before a call and that the call leaves at zero (its last workgroup resets
// it); the per-call scratch follows.  Offsets within the header:
constexpr size_t kWsHeader = 16384;
constexpr size_t kHdrMlpBarrier = 0;      // persistent MLP block: grid barrier (qg_mlp_state_bytes())
// LM head, greedy finish: the workgroups form kLmGroups groups (blockIdx.x mod
// kLmGroups) so that no address takes more than a group's share of the atomics.
constexpr int kLmGroups = 8;
constexpr size_t kHdrLmSlots = 8704;       // per group g and row m, at (g * 8 + m) * kHdrLmSlotStride: the
constexpr size_t kHdrLmSlotStride = 64;    //   largest (logit, index) key of the group's workgroups so far
constexpr size_t kHdrLmGroupCount = 12800; // per group, at g * 64: its workgroups that have merged their keys
constexpr size_t kHdrLmCount = 13312;      // groups whose workgroups have all merged

// ----------------------------------------------------------- host side ---
// Launch descriptors filled by the ABI layer (abi.hip) and consumed by the
// launchers in affine4.hip / q4k.hip.

enum QgAffineMode { QG_MODE_PLAIN = 0, QG_MODE_GATEUP = 1, QG_MODE_LMHEAD = 2, QG_MODE_PLANES = 3, QG_MODE_PLAIN8 = 4 };
// QG_MODE_PLANES: Y = (X_hi + X_lo) . dequant(W)^T with X given as two bf16
// planes (the transformed input of the RHT projection), epilogue as PLAIN.
// QG_MODE_PLAIN8: Y = X . dequant(W)^T with 8-bit affine codes ([N][K/4]
// words), epilogue as PLAIN.

struct QgAffineArgs {
  const uint16_t* x;
  const uint16_t* x_lo;  // PLANES: the low plane of X [M][K]
  const uint16_t* gamma;
  float eps;
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  uint16_t* y;  // PLAIN: Y [M][N]; GATEUP: h [M][N] with N = I
  float* logits;
  int32_t* ids;
  const int32_t* draft;
  int32_t* accepted;
  float* part;                // [S][NB][M][N] split-K partials (NB = 2 for gate and up)
  float* ssq_part;            // [S][8] per-slice sums of x^2 (GATEUP with S > 1)
  unsigned char* state;       // workspace header (zero between calls): the LM head's running maxima
                              // and arrival counter when its finalize is fused into the projection
  int M, N, K, G;
  int nchunks, S, cps, ntiles;
  int rgroups;  // workgroups per K slice; workgroup r owns tiles [r*ntiles/rgroups, (r+1)*ntiles/rgroups)
  int waves;    // waves per workgroup
  int wide;     // scales/biases of a whole batch can be loaded as one aligned vector per row
  int tiled;    // codes / scales hold the tile-order layout (see affine4.hip); biases unused
  // top-k readout (LM head mode with topk > 0): the projection stores the
  // logits and each workgroup's largest key of every row; k_topk_select
  // (topk.hip) then finds the k largest keys of each row
  int topk;
  float* topk_vals;          // [M][topk] (nullable)
  unsigned long long* cand;  // [M][workgroups] each workgroup's largest key of the row
  unsigned long long* surv;  // [M][min(topk, workgroups) * 16 * waves * topk_tpw] selected keys past the LDS list
  int topk_tpw;              // tiles per wave of the projection's plan
};

struct QgQ4kArgs {
  const uint16_t* x;
  const uint8_t* blocks;
  uint16_t* y;
  float* part;  // [S][M][N] split-K partials
  int M, N, K;
  int nchunks, S, cps, ntiles, tpw, rgroups, waves;
};

struct QgMoeArgs {
  const uint16_t* x;
  const float* logits;
  int top_k;
  const uint8_t* w_gu;
  const uint8_t* w_down;
  uint16_t* y;
  int32_t* out_ids;
  float* out_w;
  int32_t* route_ids;  // [top_k] workspace: selected experts in ascending order
  float* route_w;      // [top_k] workspace: their routing weights
  uint16_t* h;         // [top_k][I] bf16 workspace
  int E, D, I;
};

// Launchers return a hipError_t value (0 on success).
int qg_launch_affine(int mode, const QgAffineArgs& a, size_t lds_bytes, hipStream_t stream);
int qg_launch_q4k(const QgQ4kArgs& a, size_t lds_bytes, hipStream_t stream);
// k_split_reduce of a plain projection (adds the S slices' partial sums in
// slice order and stores bf16 Y), for kernels that share qgemv_affine4's plan.
int qg_launch_split_reduce_plain(const QgAffineArgs& a, hipStream_t stream);
// valu.hip: the affine-4 projection with vector-ALU dot products (measurement
// aid); LDS bytes it needs for a slice of cps chunks.
int qg_launch_affine_valu(const QgAffineArgs& a, hipStream_t stream);
size_t qg_valu_lds_bytes(int M, int cps);
// GGUF Q6_K projection (q6k.hip): QgQ4kArgs with blocks of 210 bytes, the
// split plan in superblocks; k_q4k_reduce adds the slices when S > 1.
int qg_launch_q6k(const QgQ4kArgs& a, size_t lds_bytes, hipStream_t stream);
int qg_launch_q4k_reduce(const QgQ4kArgs& a, hipStream_t stream);
int qg_launch_moe(const QgMoeArgs& a, hipStream_t stream);
// Repack canonical affine-4 weights [N][K] (K % 512 == 0) into the tile-order
// layout the tiled kernels read.
int qg_launch_tile_pack(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, uint32_t* codes_t,
                        uint16_t* sb_t, int N, int K, hipStream_t stream);
// The persistent MLP block (mlp.hip): pa = gate/up plan (y = h), pc = down
// plan (x = h); state: qg_mlp_state_bytes() bytes, zero when the launch starts
// and left zero by it (the grid barrier's counters; failure flag of the launch
// at byte 16, count of failed launches at byte 20); grid a multiple of 32,
// every workgroup resident (cooperative launch).
size_t qg_mlp_state_bytes();
// A stack of L MLP blocks in one launch: strides (in elements) from one
// layer's tile-order weights, gamma and output to the next layer's.
struct QgMlpStack {
  int L;
  size_t gu_codes, gu_sb, dn_codes, dn_sb, gamma, y;
};
int qg_launch_mlp(const QgAffineArgs& pa, const QgAffineArgs& pc, const QgMlpStack& stack, unsigned char* state,
                  int spin_limit, int grid, size_t lds, hipStream_t stream);
const void* qg_mlp_kernel(int M);  // the kernel instance for M rows (occupancy queries)
// Input randomised Hadamard transform: x [M][K] bf16 and signs [K] to the hi
// and lo bf16 planes of (1/sqrt(had)) H_had diag(s) x, blockwise along K.
constexpr int kRhtMax = 4096;  // largest transform block
int qg_launch_rht(const uint16_t* x, const int8_t* signs, int had, int M, int K, uint16_t* hi, uint16_t* lo,
                  hipStream_t stream);
constexpr int kWaves = 4;  // waves per workgroup of the projection kernels
// Top-k selection after the LM-head projection (topk.hip).
constexpr int kTopkMax = 64;         // largest k
constexpr int kTopkMaxWg = 512;      // projection workgroups whose row maxima one wave ranks (8 per lane)
constexpr int kTopkSurvLds = 2048;   // selected keys a row keeps in LDS (the rest go to QgAffineArgs::surv)
int qg_launch_topk(const QgAffineArgs& a, int nwg, hipStream_t stream);
