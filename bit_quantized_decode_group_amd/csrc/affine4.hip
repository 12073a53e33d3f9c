// affine4.hip -- gfx950 kernels for MLX-style affine 4-bit weights (group 64,
// bf16 scale and bias per group).
//
// One kernel template covers the three affine operations of the decode step:
//   QG_MODE_PLAIN   Y = X . dequant(W)^T                      (qgemv_affine4)
//   QG_MODE_GATEUP  h = silu(xn.Wg^T) * (xn.Wu^T), xn = RMSNorm(x)
//                   (rmsnorm_gateup_swiglu: norm fused into the projection,
//                   gate and up computed together -- Husky page, section
//                   "MSI의 네 가지 구현 요소")
//   QG_MODE_LMHEAD  logits = X . dequant(W)^T, greedy argmax per row and the
//                   accepted draft prefix, all on the device (uzu page: untied
//                   readout; Husky page: next token handed over on the GPU)
//
// Work decomposition
//   * A "tile" is 16 consecutive weight rows (one MFMA B operand width).
//   * A "chunk" is 128 consecutive k (two scale groups): per lane one 16-byte
//     load of codes (4 words = 32 codes) and one scale+bias per lane.
//   * The K axis is cut into S slices of `cps` chunks (split-K across
//     workgroups, used when there are few tiles); each workgroup owns one
//     slice and a run of tiles, stages its slice of X once in LDS, and its
//     waves stream whole tiles.  With S > 1 the last workgroup to finish a
//     tile (per-tile arrival counter) adds the S fp32 partials in slice order,
//     so the result does not depend on timing.
//   * Weight bytes are read exactly once; X is read once per workgroup.
//
// Per chunk and lane: codes word t (t = 0..3) of lane l covers
//   k = 128*c + 32*(l/16) + 8*t + i, i = 0..7,
// lanes 0..31 therefore carry group 2c and lanes 32..63 group 2c+1, which is
// exactly the split of C rows described in common.h.
#include "common.h"

namespace qg {

constexpr int kAffineChunkK = 128;
constexpr int kBatch = 8;  // chunks whose loads are issued together

// Activation staging: X[:, slice] -> LDS in MFMA operand order.
// LDS entry ((c*4 + t)*4 + kb)*M + m holds, for activation row m, the eight
// values at k = 128c + 32kb + 8t + nib(s), s = 0..7 with nib(s) = s/2 + 4*(s%2)
// (the code order unpack_affine_word produces).  sx[(2c + par)*8 + m] holds
// the fp32 sum of the 64 staged values of group 2c+par (the value the offset
// and bias are folded against).  GATEUP stages bf16(x*gamma) and keeps the
// per-(row, group) sum of x^2 for the RMS.
template <int M, int MODE>
__device__ __forceinline__ void stage_affine_x(const QgAffineArgs& p, uint4* xs, float* sx, float* ssq,
                                               int c0, int nc) {
  const int ngl = 2 * nc;
  for (int pi = threadIdx.x; pi < M * ngl; pi += blockDim.x) {
    const int m = pi / ngl;
    const int gl = pi - m * ngl;
    const int g = 2 * c0 + gl;
    uint32_t v[32];
    float sum = 0.f, sq = 0.f;
    if (g < p.G) {
      const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)m * p.K + (size_t)g * 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 t = src[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
      if (MODE == QG_MODE_GATEUP) {
        const uint4* gsrc = reinterpret_cast<const uint4*>(p.gamma + (size_t)g * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 t = gsrc[i];
          const uint32_t gg[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t xv = v[4 * i + j];
            const float x0 = bf16_bits_to_f32(xv & 0xFFFFu), x1 = bf16_bits_to_f32(xv >> 16);
            const float g0 = bf16_bits_to_f32(gg[j] & 0xFFFFu), g1 = bf16_bits_to_f32(gg[j] >> 16);
            sq = fmaf(x0, x0, sq);
            sq = fmaf(x1, x1, sq);
            // x*gamma of two bf16 values is exact in fp32; one rounding to bf16
            v[4 * i + j] = (uint32_t)f32_to_bf16_bits(x0 * g0) | ((uint32_t)f32_to_bf16_bits(x1 * g1) << 16);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        sum += bf16_bits_to_f32(v[i] & 0xFFFFu);
        sum += bf16_bits_to_f32(v[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0u;
    }
    const int c = gl >> 1, par = gl & 1;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int base = 32 * kb2 + 8 * t;  // k within the group, even
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int klo = base + j, khi = base + j + 4;
          const uint32_t lo = (klo & 1) ? (v[klo >> 1] >> 16) : (v[klo >> 1] & 0xFFFFu);
          const uint32_t hi = (khi & 1) ? (v[khi >> 1] >> 16) : (v[khi >> 1] & 0xFFFFu);
          e[j] = lo | (hi << 16);
        }
        xs[((c * 4 + t) * 4 + (2 * par + kb2)) * M + m] = make_uint4(e[0], e[1], e[2], e[3]);
      }
    }
    sx[gl * 8 + m] = sum;
    if (MODE == QG_MODE_GATEUP) ssq[m * ngl + gl] = sq;
  }
  if (M < 8) {
    for (int pi = threadIdx.x; pi < ngl * (8 - M); pi += blockDim.x) {
      const int gl = pi / (8 - M), m = M + pi % (8 - M);
      sx[gl * 8 + m] = 0.f;
    }
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t lo2 = (uint32_t)__shfl_xor((int)lo, mask), hi2 = (uint32_t)__shfl_xor((int)hi, mask);
  return ((unsigned long long)hi2 << 32) | lo2;
}

template <int M, int MODE>
__global__ void __launch_bounds__(256) k_affine(QgAffineArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NB = (MODE == QG_MODE_GATEUP) ? 2 : 1;  // weight tiles per unit (gate, up)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S;
  const int rg = blockIdx.x / p.S;
  const int c0 = slice * p.cps;
  const int nc = min(p.cps, p.nchunks - c0);

  uint4* xs = reinterpret_cast<uint4*>(smem);
  float* sx = reinterpret_cast<float*>(xs + nc * 16 * M);
  float* ssq = sx + nc * 16;       // GATEUP: [M][2nc]
  float* rinv = ssq + M * 2 * nc;  // GATEUP: [8]
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(rinv + 8);  // LMHEAD: [W][8]
  __shared__ int s_last;
  __shared__ int s_ids[8];

  if (MODE == QG_MODE_LMHEAD) {
    for (int i = threadIdx.x; i < W * 8; i += blockDim.x) wkeys[i] = 0ull;
  }
  stage_affine_x<M, MODE>(p, xs, sx, ssq, c0, nc);
  __syncthreads();
  if (MODE == QG_MODE_GATEUP) {
    if (threadIdx.x < M) {
      float t = 0.f;
      for (int gl = 0; gl < 2 * nc; ++gl) t += ssq[threadIdx.x * 2 * nc + gl];
      rinv[threadIdx.x] = 1.0f / sqrtf(t / (float)p.K + p.eps);
    }
    __syncthreads();
  }

  const int nl = lane & 15;
  const int kb = lane >> 4;
  const int half = lane >> 5;  // scale group parity of this lane (B and C layouts agree)
  const int rho = lane & 15;
  const bool a_act = ((rho >> 3) == (kb >> 1)) && ((rho & 7) < M);
  const uint4* a_base = xs + kb * M + (rho & 7);
  const float* sx_base = sx + half * 8 + 4 * (kb & 1);
  const size_t wrow_words = (size_t)p.K / 8;

  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};

  for (int it = 0; it < p.tpw; ++it) {
    const int tile = (rg * W) * p.tpw + wave + it * W;
    if (tile >= p.ntiles) break;
    const int row = tile * 16 + nl;
    const bool row_ok = row < p.N;
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int cb = 0; cb < nc; cb += kBatch) {
      uint4 q[NB][kBatch];
      uint32_t sb[NB][kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int cl = cb + u;
        const int cg = c0 + cl;
        const int g = 2 * cg + half;
        const bool ok = row_ok && (cl < nc) && (g < p.G);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const size_t r = (size_t)row + (size_t)b * p.N;  // up rows follow the I gate rows
          q[b][u] = make_uint4(0u, 0u, 0u, 0u);
          sb[b][u] = 0u;
          if (ok) {
            q[b][u] = *reinterpret_cast<const uint4*>(p.codes + r * wrow_words + (size_t)cg * 16 + kb * 4);
            sb[b][u] = (uint32_t)p.scales[r * p.G + g] | ((uint32_t)p.biases[r * p.G + g] << 16);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int cl = cb + u;
        if (cl >= nc) break;
        uint4 a[4];
        const uint4* ap = a_base + (size_t)cl * 16 * M;
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = a_act ? ap[t * 4 * M] : make_uint4(0u, 0u, 0u, 0u);
        const float4 sxv = *reinterpret_cast<const float4*>(sx_base + cl * 16);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4_t C = {0.f, 0.f, 0.f, 0.f};
          C = mfma_bf16(a[0], unpack_affine_word(q[b][u].x), C);
          C = mfma_bf16(a[1], unpack_affine_word(q[b][u].y), C);
          C = mfma_bf16(a[2], unpack_affine_word(q[b][u].z), C);
          C = mfma_bf16(a[3], unpack_affine_word(q[b][u].w), C);
          const float sv = bf16_bits_to_f32(sb[b][u] & 0xFFFFu);
          const float bv = bf16_bits_to_f32(sb[b][u] >> 16);
          const float cbias = fmaf(-128.0f, sv, bv);
          acc[b][0] = fmaf(sv, C[0], fmaf(cbias, sxv.x, acc[b][0]));
          acc[b][1] = fmaf(sv, C[1], fmaf(cbias, sxv.y, acc[b][1]));
          acc[b][2] = fmaf(sv, C[2], fmaf(cbias, sxv.z, acc[b][2]));
          acc[b][3] = fmaf(sv, C[3], fmaf(cbias, sxv.w, acc[b][3]));
        }
      }
    }
    // lanes l and l^32 hold the two scale groups of every chunk: add them
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[b][r] += __shfl_xor(acc[b][r], 32);

    const bool out_lane = (lane < 32) && row_ok;
    const int mbase = 4 * (lane >> 4);  // valid for lanes < 32

    if (MODE == QG_MODE_GATEUP) {
      if (out_lane) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) {
            const float gv = acc[0][r] * rinv[m];
            const float uv = acc[NB - 1][r] * rinv[m];
            const float h = gv / (1.0f + __expf(-gv)) * uv;
            p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(h);
          }
        }
      }
    } else if (MODE == QG_MODE_LMHEAD) {
      if (out_lane) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) {
            if (p.logits) p.logits[(size_t)m * p.N + row] = acc[0][r];
            const unsigned long long key = argmax_key(acc[0][r], (uint32_t)row);
            best[r] = key > best[r] ? key : best[r];
          }
        }
      }
    } else if (p.S == 1) {
      if (out_lane) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(acc[0][r]);
        }
      }
    } else {
      if (out_lane) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) p.part[((size_t)slice * M + m) * p.N + row] = acc[0][r];
        }
      }
      __threadfence();  // release this slice's partials (device scope)
      uint32_t prev = 0u;
      if (lane == 0) prev = atomicAdd(&p.tile_cnt[tile], 1u);
      prev = (uint32_t)__shfl((int)prev, 0);
      if (prev == (uint32_t)(p.S - 1)) {
        __threadfence();  // acquire the other slices' partials
        if (out_lane) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = mbase + r;
            if (m < M) {
              float t = 0.f;
              for (int s2 = 0; s2 < p.S; ++s2) t += p.part[((size_t)s2 * M + m) * p.N + row];
              p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(t);
            }
          }
        }
        if (lane == 0) atomicExch(&p.tile_cnt[tile], 0u);  // leave the counter at zero
      }
    }
  }

  if (MODE == QG_MODE_LMHEAD) {
    // wave: lanes 0..15 share rows m = 0..3, lanes 16..31 rows 4..7
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const unsigned long long o = shfl_xor_u64(best[r], off);
        best[r] = o > best[r] ? o : best[r];
      }
    if (lane == 0 || lane == 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        if (m < M) wkeys[wave * 8 + m] = best[r];
      }
    }
    __syncthreads();
    if (threadIdx.x < M) {
      unsigned long long v = 0ull;
      for (int w = 0; w < W; ++w) v = wkeys[w * 8 + threadIdx.x] > v ? wkeys[w * 8 + threadIdx.x] : v;
      if (v) atomicMax(&p.keys[threadIdx.x], v);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(p.done_cnt, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (s_last) {
      __threadfence();
      if (threadIdx.x < M) {
        const unsigned long long k = atomicMax(&p.keys[threadIdx.x], 0ull);  // read
        const int id = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        p.ids[threadIdx.x] = id;
        s_ids[threadIdx.x] = id;
        atomicExch(&p.keys[threadIdx.x], 0ull);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        if (p.accepted) {
          int a = 0;
          if (p.draft)
            while (a < M && s_ids[a] == p.draft[a]) ++a;
          *p.accepted = a;
        }
        atomicExch(p.done_cnt, 0u);
      }
    }
  }
}

template <int M>
static int launch_affine_m(int mode, const QgAffineArgs& a, size_t lds, hipStream_t st) {
  const dim3 grid((unsigned)(a.S * a.rgroups)), block((unsigned)(64 * a.waves));
  switch (mode) {
    case QG_MODE_PLAIN:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLAIN>), grid, block, lds, st, a);
      break;
    case QG_MODE_GATEUP:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_GATEUP>), grid, block, lds, st, a);
      break;
    default:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_LMHEAD>), grid, block, lds, st, a);
      break;
  }
  return (int)hipGetLastError();
}

}  // namespace qg

int qg_launch_affine(int mode, const QgAffineArgs& a, size_t lds, hipStream_t st) {
  switch (a.M) {
    case 1: return qg::launch_affine_m<1>(mode, a, lds, st);
    case 2: return qg::launch_affine_m<2>(mode, a, lds, st);
    case 3: return qg::launch_affine_m<3>(mode, a, lds, st);
    case 4: return qg::launch_affine_m<4>(mode, a, lds, st);
    case 5: return qg::launch_affine_m<5>(mode, a, lds, st);
    case 6: return qg::launch_affine_m<6>(mode, a, lds, st);
    case 7: return qg::launch_affine_m<7>(mode, a, lds, st);
    case 8: return qg::launch_affine_m<8>(mode, a, lds, st);
    default: return (int)hipErrorInvalidValue;
  }
}
