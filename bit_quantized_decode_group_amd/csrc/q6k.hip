// q6k.hip -- gfx950 projection kernel for GGUF Q6_K weights (256-weight
// superblocks of 210 bytes: 128 bytes of low nibbles, 64 bytes of 2-bit high
// parts, sixteen int8 scales, fp16 d), consumed as stored (runNburn page,
// section "GGUF를 그대로 진실의 원본으로 둡니다": Q4_K_M files mix Q6_K in).
//
//   k_q6k   Y = X . dequant(W)^T, split-K partial sums added by k_q4k_reduce
//
// Weight o of a superblock (half h = o/128, quarter j = (o%128)/32, l = o%32)
// takes its low four bits from ql[64h + 32(j%2) + l] (low nibble for j < 2,
// high nibble otherwise) and its high two bits from bits 2j, 2j+1 of
// qh[32h + l]; u = low | high << 4 is 0..63 and w = d * sc[o/16] * (u - 32).
//
// Operands (see common.h for the MFMA scheme): u becomes the bf16 pattern
// 0x4300 | u = 128 + u (exact), so per 16-weight scale block the MFMA gives
// D = sum x*(128+u) and the epilogue applies d*sc*(D - 160*sum x).  One MFMA
// covers 32 k = two scale blocks: lanes 0..31 (kb = 0, 1) carry block 2i,
// lanes 32..63 block 2i+1, and rows 0..7 / 8..15 of the activation operand
// the matching rows.  Lane (n, kb) of MFMA i takes weights 32i + 8kb .. +7 of
// row n in natural order; v_perm_b32 with a register of 0x43 bytes turns two
// code bytes into two operand halves in one instruction.
//
// A 210-byte superblock is 2-byte aligned at best; the per-lane 8- and
// 16-byte loads are unaligned vector loads, which gfx950 serves from global
// memory.
#include "common.h"

namespace qg {

constexpr int kQ6kBlock = 210;

// Loads of one superblock for one lane: the four 8-byte ql runs it needs
// (half h, quarter parity), the two 8-byte qh runs (per half), the 16 scales
// and d.
struct Q6kBuf {
  uint2 ql[4];  // index 2h + (j % 2)
  uint2 qh[2];  // index h
  uint4 sc;
  uint32_t d;
};

__device__ __forceinline__ void q6k_load(Q6kBuf& b, const uint8_t* bp, int kb) {
#pragma unroll
  for (int c = 0; c < 4; ++c) __builtin_memcpy(&b.ql[c], bp + 64 * (c >> 1) + 32 * (c & 1) + 8 * kb, 8);
#pragma unroll
  for (int h = 0; h < 2; ++h) __builtin_memcpy(&b.qh[h], bp + 128 + 32 * h + 8 * kb, 8);
  __builtin_memcpy(&b.sc, bp + 192, 16);
  uint16_t d;
  __builtin_memcpy(&d, bp + 208, 2);
  b.d = d;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// Stage activation rows [M][slice of nsb superblocks from sb0] into LDS:
// entry ((sbl*8 + i)*4 + kb)*M + m holds x[m][256(sb0+sbl) + 32i + 8kb + s],
// s = 0..7 in natural order; sx[(sbl*16 + sub)*8 + m] is the fp32 sum of the
// 16 values of scale block sub (zero for rows m >= M).
template <int M>
__device__ __forceinline__ void stage_q6k_x(const uint16_t* x, int K, uint4* xs, float* sx, int sb0, int nsb) {
  for (int pi = threadIdx.x; pi < nsb * 16 * 8; pi += blockDim.x) {
    const int m = pi & 7, sub = (pi >> 3) & 15, sbl = pi >> 7;
    float sum = 0.f;
    if (m < M) {
      const size_t k0 = (size_t)256 * (sb0 + sbl) + 16 * sub;
      const uint4 a = *reinterpret_cast<const uint4*>(x + (size_t)m * K + k0);
      const uint4 b = *reinterpret_cast<const uint4*>(x + (size_t)m * K + k0 + 8);
      const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) sum += bf16_bits_to_f32(v[t] & 0xFFFFu) + bf16_bits_to_f32(v[t] >> 16);
      const int i = sub >> 1, kb0 = 2 * (sub & 1);
      xs[((sbl * 8 + i) * 4 + kb0) * M + m] = a;
      xs[((sbl * 8 + i) * 4 + kb0 + 1) * M + m] = b;
    }
    sx[(sbl * 16 + sub) * 8 + m] = sum;
  }
}

template <int M>
__global__ void __launch_bounds__(256) k_q6k(QgQ4kArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S, rg = blockIdx.x / p.S;
  const int sb0 = slice * p.cps;
  const int nsb = min(p.cps, p.nchunks - sb0);
  uint4* lds = reinterpret_cast<uint4*>(smem);  // [0] zero entry, then the staged slice
  uint4* xs = lds + 1;
  float* sx = reinterpret_cast<float*>(xs + nsb * 32 * M);
  const int nb_row = p.K / 256;
  const int kb = lane >> 4, half = lane >> 5, rho = lane & 15;
  const bool a_act = ((rho >> 3) == (kb >> 1)) && ((rho & 7) < M);
  const float* sx_base = sx + half * 8 + 4 * (kb & 1);
  uint32_t k43;
  asm("v_mov_b32 %0, %1" : "=v"(k43) : "i"(0x43434343));
  auto row_blocks = [&](int tile) {
    const int row = min(tile * 16 + (lane & 15), p.N - 1);
    return p.blocks + ((size_t)row * nb_row + sb0) * kQ6kBlock;
  };
  // the first tile's first superblock is in flight while the slice is staged
  const int tile0 = min((rg * W) * p.tpw + wave, p.ntiles - 1);
  Q6kBuf cur;
  q6k_load(cur, row_blocks(tile0), kb);
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x == 0) lds[0] = make_uint4(0u, 0u, 0u, 0u);
  stage_q6k_x<M>(p.x, p.K, xs, sx, sb0, nsb);
  __syncthreads();

  for (int it = 0; it < p.tpw; ++it) {
    const int tile = (rg * W) * p.tpw + wave + it * W;
    if (tile >= p.ntiles) break;
    const uint8_t* rb = row_blocks(tile);
    if (it > 0) q6k_load(cur, rb, kb);
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sbl = 0; sbl < nsb; ++sbl) {
      Q6kBuf nxt;
      q6k_load(nxt, rb + (size_t)min(sbl + 1, nsb - 1) * kQ6kBlock, kb);
      __builtin_amdgcn_sched_barrier(0);
      const float d = f16_to_f32(cur.d);
      const uint32_t scw[4] = {cur.sc.x, cur.sc.y, cur.sc.z, cur.sc.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int h = i >> 2, j = i & 3;
        const uint2 q = cur.ql[2 * h + (j & 1)];
        const uint2 qh = cur.qh[h];
        const uint32_t lo0 = (j < 2 ? q.x : q.x >> 4) & 0x0F0F0F0Fu;
        const uint32_t lo1 = (j < 2 ? q.y : q.y >> 4) & 0x0F0F0F0Fu;
        const uint32_t hi0 = (j < 3 ? qh.x << (4 - 2 * j) : qh.x >> 2) & 0x30303030u;
        const uint32_t hi1 = (j < 3 ? qh.y << (4 - 2 * j) : qh.y >> 2) & 0x30303030u;
        const uint32_t u0 = lo0 | hi0, u1 = lo1 | hi1;  // code bytes 0..3 and 4..7, values 0..63
        const uint4 bw = make_uint4(__builtin_amdgcn_perm(k43, u0, 0x04010400u), __builtin_amdgcn_perm(k43, u0, 0x04030402u),
                                    __builtin_amdgcn_perm(k43, u1, 0x04010400u), __builtin_amdgcn_perm(k43, u1, 0x04030402u));
        const uint4 a = lds[a_act ? 1u + (uint32_t)(((sbl * 8 + i) * 4 + kb) * M + (rho & 7)) : 0u];
        const f32x4_t C = mfma_bf16(a, bw, f32x4_t{0.f, 0.f, 0.f, 0.f});
        const int sub = 2 * i + half;  // scale block of this lane's sums
        const int scb = (int)(int8_t)((scw[sub >> 2] >> (8 * (sub & 3))) & 0xFFu);
        const float f = d * (float)scb;  // exact in fp32
        const float bt = 160.0f * f;     // exact
        const float4 sxv = *reinterpret_cast<const float4*>(sx_base + (sbl * 16 + 2 * i) * 8);
        acc[0] = fmaf(f, C[0], fmaf(-bt, sxv.x, acc[0]));
        acc[1] = fmaf(f, C[1], fmaf(-bt, sxv.y, acc[1]));
        acc[2] = fmaf(f, C[2], fmaf(-bt, sxv.z, acc[2]));
        acc[3] = fmaf(f, C[3], fmaf(-bt, sxv.w, acc[3]));
      }
      cur = nxt;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], 32);
    const int row = tile * 16 + (lane & 15);
    const int mbase = 4 * (lane >> 4);
    if (lane < 32 && row < p.N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (mbase + r < M) {
          if (p.S == 1)
            p.y[(size_t)(mbase + r) * p.N + row] = f32_to_bf16_bits(acc[r]);
          else  // this slice's sums; k_q4k_reduce adds the slices in order
            p.part[((size_t)slice * M + mbase + r) * p.N + row] = acc[r];
        }
      }
    }
  }
}

template <int M>
static int launch_q6k_m(const QgQ4kArgs& a, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_q6k<M>), dim3((unsigned)(a.S * a.rgroups)), dim3((unsigned)(64 * a.waves)), lds, st, a);
  int err = (int)hipGetLastError();
  if (err || a.S == 1) return err;
  return qg_launch_q4k_reduce(a, st);
}

}  // namespace qg

int qg_launch_q6k(const QgQ4kArgs& a, size_t lds, hipStream_t st) {
  switch (a.M) {
    case 1: return qg::launch_q6k_m<1>(a, lds, st);
    case 2: return qg::launch_q6k_m<2>(a, lds, st);
    case 3: return qg::launch_q6k_m<3>(a, lds, st);
    case 4: return qg::launch_q6k_m<4>(a, lds, st);
    case 5: return qg::launch_q6k_m<5>(a, lds, st);
    case 6: return qg::launch_q6k_m<6>(a, lds, st);
    case 7: return qg::launch_q6k_m<7>(a, lds, st);
    case 8: return qg::launch_q6k_m<8>(a, lds, st);
    default: return (int)hipErrorInvalidValue;
  }
}
