// affine_stage.h -- activation staging shared by the affine projection
// kernels (affine4.hip) and the persistent MLP-block kernel (mlp.hip).
// Internal to the library.
#pragma once
#include "common.h"

namespace qg {

// Activation staging: X[:, slice] -> LDS in MFMA operand order.  Entry
// (((c*4 + t)*4 + kb)*PL + plane)*M + m of xs holds, for activation row m,
// the eight values at k = 128c + 32kb + 8t + nib(s), s = 0..7 with
// nib(s) = s/2 + 4*(s%2) (the code order unpack_affine_word produces).
// sx[(2c + par)*8 + m] holds the fp32 sum of the 64 staged values (all planes)
// of group 2c+par, the value the offset and the bias are folded against
// (zero for rows m >= M).  GATEUP keeps the per-(row, group) sum of x^2 in ssq
// for the RMS.
//
// One wave stages one scale group at a time: lane (m, h, t) = (lane & 7,
// (lane >> 3) & 1, lane >> 4) takes the eight values of row m at
// k = 64g + 32h + 8t, so the eight lanes of a row write consecutive entries
// and the group sum is a butterfly over the lanes of that row.  A round
// gives each wave stage_groups(MODE) groups; all of a round's loads are
// issued before any is used.  Gate/up also loads gamma, and its short K
// slices need one round of two groups per wave, which keeps it within 128
// registers per lane.
__host__ __device__ constexpr int stage_groups(int mode) {
  return (mode == QG_MODE_GATEUP || mode == QG_MODE_PLANES) ? 2 : 4;
}
// activation planes staged per value: (hi, lo) for gate/up and the RHT input
__host__ __device__ constexpr int planes(int mode) { return (mode == QG_MODE_GATEUP || mode == QG_MODE_PLANES) ? 2 : 1; }

template <int MODE>
struct StageIn {
  uint4 x[stage_groups(MODE)];
  uint4 gm[planes(MODE) == 2 ? stage_groups(MODE) : 1];  // gamma (GATEUP) or the lo plane (PLANES)
};

// COH: X was written by other workgroups of the same launch (agent-scope
// stores), so it is read with agent-scope loads.
__device__ __forceinline__ uint4 load_u4_coherent(const uint16_t* ptr) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(ptr);
  return make_uint4(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int M, int MODE, bool COH = false>
__device__ __forceinline__ void stage_load(const QgAffineArgs& p, int c0, int nc, int round, StageIn<MODE>& in) {
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  const int m = min(lane & 7, M - 1), h = (lane >> 3) & 1, t = lane >> 4;
  const int glmax = 2 * nc - 1;
  constexpr int SG = stage_groups(MODE);
#pragma unroll
  for (int j = 0; j < SG; ++j) {
    // clamped in-bounds addresses; stage_store discards what it does not need
    const int gl = min((round * SG + j) * W + wave, glmax);
    const int g = min(2 * c0 + gl, p.G - 1);
    const size_t k0 = (size_t)g * 64 + 32 * h + 8 * t;
    if constexpr (COH)
      in.x[j] = load_u4_coherent(p.x + (size_t)m * p.K + k0);
    else
      in.x[j] = *reinterpret_cast<const uint4*>(p.x + (size_t)m * p.K + k0);
    if constexpr (MODE == QG_MODE_GATEUP) in.gm[j] = *reinterpret_cast<const uint4*>(p.gamma + k0);
    if constexpr (MODE == QG_MODE_PLANES) in.gm[j] = *reinterpret_cast<const uint4*>(p.x_lo + (size_t)m * p.K + k0);
  }
}

template <int M, int MODE>
__device__ __forceinline__ void stage_store(const QgAffineArgs& p, uint4* xs, float* sx, float* ssq, int c0, int nc,
                                            int round, const StageIn<MODE>& in) {
  constexpr int PL = planes(MODE);
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  const int m = lane & 7, h = (lane >> 3) & 1, t = lane >> 4;
  const int ngl = 2 * nc;
  constexpr int SG = stage_groups(MODE);
#pragma unroll
  for (int j = 0; j < SG; ++j) {
    const int gl = (round * SG + j) * W + wave;
    if (gl >= ngl) break;  // uniform across the wave
    const int g = 2 * c0 + gl;
    const bool live = (m < M) && (g < p.G);
    const uint32_t raw[4] = {live ? in.x[j].x : 0u, live ? in.x[j].y : 0u, live ? in.x[j].z : 0u,
                             live ? in.x[j].w : 0u};
    uint32_t v[PL][4];  // value i of the eight at dword i/2, half i%2
    float sum = 0.f, sq = 0.f;
    if constexpr (MODE == QG_MODE_GATEUP) {
      const uint32_t gg[4] = {in.gm[j].x, in.gm[j].y, in.gm[j].z, in.gm[j].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float x0 = bf16_bits_to_f32(raw[d] & 0xFFFFu), x1 = bf16_bits_to_f32(raw[d] >> 16);
        sq = fmaf(x0, x0, sq);
        sq = fmaf(x1, x1, sq);
        const float p0 = x0 * bf16_bits_to_f32(gg[d] & 0xFFFFu);  // exact in fp32
        const float p1 = x1 * bf16_bits_to_f32(gg[d] >> 16);
        const uint32_t hh = pack_bf16x2(p0, p1);
        v[0][d] = hh;
        // the remainders are exact bf16 values
        v[PL - 1][d] = pack_bf16x2(p0 - __uint_as_float(hh << 16), p1 - __uint_as_float(hh & 0xFFFF0000u));
      }
    } else if constexpr (MODE == QG_MODE_PLANES) {
      const uint32_t lo[4] = {live ? in.gm[j].x : 0u, live ? in.gm[j].y : 0u, live ? in.gm[j].z : 0u,
                              live ? in.gm[j].w : 0u};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[0][d] = raw[d];
        v[PL - 1][d] = lo[d];
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) v[0][d] = raw[d];
    }
    const int c = gl >> 1, kb = 2 * (gl & 1) + h;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
#pragma unroll
      for (int d = 0; d < 4; ++d) sum += bf16_bits_to_f32(v[pl][d] & 0xFFFFu) + bf16_bits_to_f32(v[pl][d] >> 16);
      // operand dword e holds values e and e + 4
      const uint4 e = make_uint4((v[pl][0] & 0xFFFFu) | (v[pl][2] << 16), (v[pl][0] >> 16) | (v[pl][2] & 0xFFFF0000u),
                                 (v[pl][1] & 0xFFFFu) | (v[pl][3] << 16), (v[pl][1] >> 16) | (v[pl][3] & 0xFFFF0000u));
      if (m < M) xs[(((c * 4 + t) * 4 + kb) * PL + pl) * M + m] = e;
    }
    // sum over the eight lanes of row m, lanes l ^ 8, l ^ 16, l ^ 32 in turn
    // (every lane ends with the same value), on the VALU
    sum = add_upper_half(add_xor16(add_xor8(sum)));
    if constexpr (MODE == QG_MODE_GATEUP) sq = add_upper_half(add_xor16(add_xor8(sq)));
    if (lane < 8) {
      sx[gl * 8 + m] = sum;
      if (MODE == QG_MODE_GATEUP && m < M) ssq[m * ngl + gl] = sq;
    }
  }
}

}  // namespace qg
