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
//   * A "tile" is 16 consecutive weight rows (one MFMA B operand width); in
//     GATEUP a unit is the gate tile rows n.. and the up tile rows I+n.. .
//   * A "chunk" is 128 consecutive k (two scale groups): per lane one 16-byte
//     load of codes (4 words = 32 codes) and one scale+bias per lane.
//   * The K axis is cut into S slices of `cps` chunks (split-K across
//     workgroups, used when there are few tiles or when the staged activations
//     would not fit); each workgroup owns one slice and a run of tiles, stages
//     its slice of X once in LDS, and its waves stream whole tiles.  With
//     S > 1 every slice stores fp32 partial sums and k_split_reduce, launched
//     next on the same stream, adds them in slice order and applies the
//     epilogue: no atomics, no cross-workgroup fences, and the result does not
//     depend on timing.
//   * The LM head stores one (logit, index) key per row and workgroup;
//     k_lmhead_finalize takes the maximum over workgroups and writes the ids
//     and the accepted count.
//   * Weight bytes are read exactly once; X is read once per workgroup.
//
// Per chunk and lane: codes word t (t = 0..3) of lane l covers
//   k = 128*c + 32*(l/16) + 8*t + i, i = 0..7,
// lanes 0..31 therefore carry group 2c and lanes 32..63 group 2c+1, which is
// exactly the split of C rows described in common.h.
//
// GATEUP operands stay exact: x*gamma of two bf16 values is exact in fp32 and
// has at most 16 significant bits, so it is the sum of hi = bf16(x*gamma) and
// lo = x*gamma - hi, both exact bf16 values.  Each MFMA step runs on the hi
// plane and then the lo plane with the same unpacked weights.
#include "common.h"

namespace qg {

__device__ __forceinline__ uint32_t half_of(const uint32_t* v, int k) {
  return (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xFFFFu);
}

// Activation staging: X[:, slice] -> LDS in MFMA operand order.
// xs[0] is a zero entry (read by lanes whose operand slots are empty); entry
// 1 + (((c*4 + t)*4 + kb)*PL + plane)*M + m holds, for activation row m,
// the eight values at k = 128c + 32kb + 8t + nib(s), s = 0..7 with
// nib(s) = s/2 + 4*(s%2) (the code order unpack_affine_word produces).
// sx[(2c + par)*8 + m] holds the fp32 sum of the 64 staged values (all planes)
// of group 2c+par, the value the offset and the bias are folded against.
// GATEUP keeps the per-(row, group) sum of x^2 in ssq for the RMS.
template <int M, int MODE>
__device__ __forceinline__ void stage_affine_x(const QgAffineArgs& p, uint4* xs, float* sx, float* ssq,
                                               int c0, int nc) {
  constexpr int PL = (MODE == QG_MODE_GATEUP) ? 2 : 1;
  const int ngl = 2 * nc;
  for (int pi = threadIdx.x; pi < M * ngl; pi += blockDim.x) {
    const int m = pi / ngl;
    const int gl = pi - m * ngl;
    const int g = 2 * c0 + gl;
    const bool live = g < p.G;
    const int c = gl >> 1, par = gl & 1;
    float sum = 0.f, sq = 0.f;
    // the group's 64 values in two halves of 32 (lanes kb = 2*par and 2*par+1)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      uint32_t v[PL][16];
      if (live) {
        const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)m * p.K + (size_t)g * 64 + 32 * kb2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 t = src[i];
          v[0][4 * i] = t.x; v[0][4 * i + 1] = t.y; v[0][4 * i + 2] = t.z; v[0][4 * i + 3] = t.w;
        }
        if constexpr (MODE == QG_MODE_GATEUP) {
          const uint4* gsrc = reinterpret_cast<const uint4*>(p.gamma + (size_t)g * 64 + 32 * kb2);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 t = gsrc[i];
            const uint32_t gg[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t xv = v[0][4 * i + j];
              const float x0 = bf16_bits_to_f32(xv & 0xFFFFu), x1 = bf16_bits_to_f32(xv >> 16);
              sq = fmaf(x0, x0, sq);
              sq = fmaf(x1, x1, sq);
              const float p0 = x0 * bf16_bits_to_f32(gg[j] & 0xFFFFu);  // exact in fp32
              const float p1 = x1 * bf16_bits_to_f32(gg[j] >> 16);
              const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
              const uint32_t l0 = f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));  // exact remainder
              const uint32_t l1 = f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
              v[0][4 * i + j] = h0 | (h1 << 16);
              v[PL - 1][4 * i + j] = l0 | (l1 << 16);
            }
          }
        }
#pragma unroll
        for (int pl = 0; pl < PL; ++pl)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sum += bf16_bits_to_f32(v[pl][i] & 0xFFFFu);
            sum += bf16_bits_to_f32(v[pl][i] >> 16);
          }
      } else {
#pragma unroll
        for (int pl = 0; pl < PL; ++pl)
#pragma unroll
          for (int i = 0; i < 16; ++i) v[pl][i] = 0u;
      }
      const int kb = 2 * par + kb2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
          uint32_t e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            e[j] = half_of(v[pl], 8 * t + j) | (half_of(v[pl], 8 * t + j + 4) << 16);
          xs[1 + (((c * 4 + t) * 4 + kb) * PL + pl) * M + m] = make_uint4(e[0], e[1], e[2], e[3]);
        }
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

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// WIDE: every batch of every slice lies inside the row and the scale/bias rows
// are aligned for one vector load per batch (the host checks G, the slice
// length and the pointers); the loop body then has no data-dependent branch
// around its loads, so the loads of the next step stay in flight while the
// current one is computed.
template <int M, int MODE, bool WIDE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == QG_MODE_GATEUP ? 3 : 4, 8)))
k_affine(QgAffineArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NB = (MODE == QG_MODE_GATEUP) ? 2 : 1;     // weight tiles per unit (gate, up)
  constexpr int PL = (MODE == QG_MODE_GATEUP) ? 2 : 1;     // activation planes (hi, lo)
  constexpr int BATCH = (MODE == QG_MODE_GATEUP) ? 2 : 4;  // chunks whose loads are issued together
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S;
  const int rg = blockIdx.x / p.S;
  const int c0 = slice * p.cps;
  const int nc = min(p.cps, p.nchunks - c0);
  // this workgroup's tiles [t_begin, t_end); wave w takes t_begin + w, t_begin + w + W, ...
  const int t_begin = (int)(((long long)rg * p.ntiles) / p.rgroups);
  const int t_end = (int)(((long long)(rg + 1) * p.ntiles) / p.rgroups);
  const int ntw = (t_end - t_begin > wave) ? (t_end - t_begin - wave + W - 1) / W : 0;
  const int nbt = (nc + BATCH - 1) / BATCH;  // batches per tile
  const int nsteps = ntw * nbt;              // this wave's (tile, batch) steps

  uint4* xs = reinterpret_cast<uint4*>(smem);
  float* sx = reinterpret_cast<float*>(xs + 1 + nc * 16 * M * PL);
  float* ssq = sx + nc * 16;       // GATEUP: [M][2nc]
  float* rinv = ssq + M * 2 * nc;  // GATEUP: [8]
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(rinv + 8);  // LMHEAD: [W][8]

  const int nl = lane & 15;
  const int kb = lane >> 4;
  const int half = lane >> 5;  // scale group parity of this lane (B and C layouts agree)
  const int rho = lane & 15;
  const bool a_act = ((rho >> 3) == (kb >> 1)) && ((rho & 7) < M);
  // operand entry of this lane for (chunk cl, step t, plane pl): 1 + a_lane + (cl*16 + t*4)*PL*M + pl*M,
  // or the zero entry for lanes whose slots carry the other group / a padding row
  const uint32_t a_lane = 1u + (uint32_t)(kb * PL * M + (rho & 7));
  const uint32_t a_mask = a_act ? 0xFFFFFFFFu : 0u;
  const float* sx_base = sx + half * 8 + 4 * (kb & 1);
  const size_t wrow_words = (size_t)p.K / 8;
  const uint32_t wmax = (uint32_t)(wrow_words - 4);  // last in-row 16-byte load
  const int mbase = 4 * (lane >> 4);                 // activation row of C element 0 (lanes < 32)

  // ---- loads of one (tile, batch) step: unconditional, at clamped in-bounds addresses.
  // sw / bw dword u holds the bf16 scales / biases of groups 2(c0+cb+u) (low half) and
  // 2(c0+cb+u)+1 (high half); lane l uses the half of its group parity.  A batch
  // whose 2*BATCH groups are all inside the row loads them as one vector per row.
  struct Buf {
    uint4 q[NB][BATCH];
    uint32_t sw[NB][BATCH], bw[NB][BATCH];
  };
  auto load_step = [&](Buf& bf, int st) {
    const int ti = st / nbt;
    const int cb = (st - ti * nbt) * BATCH;
    const int row = (t_begin + wave + ti * W) * 16 + nl;
    const size_t row_c = (size_t)min(row, p.N - 1);
    const int gb = 2 * (c0 + cb);  // first scale group of the batch
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int cg = WIDE ? c0 + cb + u : c0 + min(cb + u, nc - 1);
      const uint32_t wo = min((uint32_t)(cg * 16 + kb * 4), wmax);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const size_t r = row_c + (size_t)b * p.N;  // up rows follow the I gate rows
        bf.q[b][u] = *reinterpret_cast<const uint4*>(p.codes + r * wrow_words + wo);
      }
    }
    if constexpr (WIDE) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const size_t off = (row_c + (size_t)b * p.N) * p.G + gb;
        if constexpr (BATCH == 4) {
          const uint4 sv = *reinterpret_cast<const uint4*>(p.scales + off);
          const uint4 bv = *reinterpret_cast<const uint4*>(p.biases + off);
          bf.sw[b][0] = sv.x; bf.sw[b][1] = sv.y; bf.sw[b][2] = sv.z; bf.sw[b][3] = sv.w;
          bf.bw[b][0] = bv.x; bf.bw[b][1] = bv.y; bf.bw[b][2] = bv.z; bf.bw[b][3] = bv.w;
        } else {
          const uint2 sv = *reinterpret_cast<const uint2*>(p.scales + off);
          const uint2 bv = *reinterpret_cast<const uint2*>(p.biases + off);
          bf.sw[b][0] = sv.x; bf.sw[b][1] = sv.y;
          bf.bw[b][0] = bv.x; bf.bw[b][1] = bv.y;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int g = min(gb + 2 * u + half, p.G - 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const size_t r = row_c + (size_t)b * p.N;
          bf.sw[b][u] = (uint32_t)p.scales[r * p.G + g] << (16 * half);
          bf.bw[b][u] = (uint32_t)p.biases[r * p.G + g] << (16 * half);
        }
      }
    }
  };

  f32x4_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};

  // ---- end of a tile: add the two group halves, then store / publish
  auto finish_tile = [&](int tile) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[b][r] += __shfl_xor(acc[b][r], 32);
    const int row = tile * 16 + nl;
    if ((lane < 32) && row < p.N) {
      if (p.S > 1) {
        // split-K: this slice's sums; k_split_reduce finishes the tile
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mbase + r < M) p.part[(((size_t)slice * NB + b) * M + mbase + r) * p.N + row] = acc[b][r];
      } else if (MODE == QG_MODE_GATEUP) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) {
            const float ri = rinv[m];
            p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(silu_mul(acc[0][r] * ri, acc[NB - 1][r] * ri));
          }
        }
      } else if (MODE == QG_MODE_LMHEAD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) {
            if (p.logits) p.logits[(size_t)m * p.N + row] = acc[0][r];
            const unsigned long long key = argmax_key(acc[0][r], (uint32_t)row);
            best[r] = key > best[r] ? key : best[r];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(acc[0][r]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // ---- compute one (tile, batch) step: independent MFMA chains per chunk, then the group epilogues
  auto compute_step = [&](const Buf& bf, int st) {
    const int ti = st / nbt;
    const int bi = st - ti * nbt;
    const int cb = bi * BATCH;
    f32x4_t C[NB][BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) C[b][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (WIDE || cb + u < nc) {
          uint4 a[PL];
#pragma unroll
          for (int pl = 0; pl < PL; ++pl)
            a[pl] = xs[(a_lane + (uint32_t)(((cb + u) * 16 + t * 4) * PL * M + pl * M)) & a_mask];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const uint32_t w = t == 0 ? bf.q[b][u].x : t == 1 ? bf.q[b][u].y : t == 2 ? bf.q[b][u].z : bf.q[b][u].w;
            const uint4 bw = unpack_affine_word(w);
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) C[b][u] = mfma_bf16(a[pl], bw, C[b][u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (WIDE || cb + u < nc) {
        const float4 sxv = *reinterpret_cast<const float4*>(sx_base + (cb + u) * 16);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float sc = __uint_as_float((bf.sw[b][u] >> (16 * half)) << 16);
          const float cbias = fmaf(-128.0f, sc, __uint_as_float((bf.bw[b][u] >> (16 * half)) << 16));
          acc[b][0] = fmaf(sc, C[b][u][0], fmaf(cbias, sxv.x, acc[b][0]));
          acc[b][1] = fmaf(sc, C[b][u][1], fmaf(cbias, sxv.y, acc[b][1]));
          acc[b][2] = fmaf(sc, C[b][u][2], fmaf(cbias, sxv.z, acc[b][2]));
          acc[b][3] = fmaf(sc, C[b][u][3], fmaf(cbias, sxv.w, acc[b][3]));
        }
      }
    }
    if (bi == nbt - 1) finish_tile(t_begin + wave + ti * W);
  };

  // ---- prologue: first weight loads in flight while the activations are staged
  // every load_step takes a step index clamped to [0, last]: a wave without
  // work, or the odd step after the last one, reloads an in-bounds step
  const int last = max(nsteps - 1, 0);
  Buf bufA, bufB;
  load_step(bufA, 0);
  if (threadIdx.x == 0) xs[0] = make_uint4(0u, 0u, 0u, 0u);
  if (MODE == QG_MODE_LMHEAD) {
    for (int i = threadIdx.x; i < W * 8; i += blockDim.x) wkeys[i] = 0ull;
  }
  stage_affine_x<M, MODE>(p, xs, sx, ssq, c0, nc);
  __syncthreads();
  if (MODE == QG_MODE_GATEUP) {
    if (threadIdx.x < M) {
      float t = 0.f;
      for (int gl = 0; gl < 2 * nc; ++gl) t += ssq[threadIdx.x * 2 * nc + gl];
      if (p.S == 1) {
        rinv[threadIdx.x] = 1.0f / sqrtf(t / (float)p.K + p.eps);
      } else if (rg == 0) {
        p.ssq_part[(size_t)slice * 8 + threadIdx.x] = t;  // this slice's sum of x^2, for k_split_reduce
      }
    }
    __syncthreads();
  }

  // ---- main loop: two steps per iteration, loads of the next step ahead of the compute
  // (the scheduling barriers keep the compiler from sinking the loads below
  // the computation that waits for the previous step's data)
  for (int st = 0; st < nsteps; st += 2) {
    load_step(bufB, min(st + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    compute_step(bufA, st);
    load_step(bufA, min(st + 2, last));
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nsteps) compute_step(bufB, st + 1);
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
      p.keys[(size_t)blockIdx.x * 8 + threadIdx.x] = v;  // this workgroup's best (logit, index) of row m
    }
  }
}

// Split-K epilogue: one thread per output (m, n); the S slices' partial sums are
// added in slice order, then the mode's epilogue (bf16 store, or RMS scaling and
// SwiGLU for gate/up).  Loads are issued eight slices at a time.
template <int MODE>
__global__ void __launch_bounds__(256) k_split_reduce(QgAffineArgs p) {
  constexpr int NB = (MODE == QG_MODE_GATEUP) ? 2 : 1;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)p.M * p.N;
  if (idx >= total) return;
  const int m = (int)(idx / (size_t)p.N);
  float t[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    t[b] = 0.f;
    for (int s0 = 0; s0 < p.S; s0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p.part[((size_t)min(s0 + j, p.S - 1) * NB + b) * total + idx];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < p.S) t[b] += v[j];
    }
  }
  if (MODE == QG_MODE_GATEUP) {
    float ss = 0.f;
    for (int s2 = 0; s2 < p.S; ++s2) ss += p.ssq_part[(size_t)s2 * 8 + m];
    const float ri = 1.0f / sqrtf(ss / (float)p.K + p.eps);
    p.y[idx] = f32_to_bf16_bits(silu_mul(t[0] * ri, t[NB - 1] * ri));
  } else {
    p.y[idx] = f32_to_bf16_bits(t[0]);
  }
}

// Greedy verify: maximum key over all workgroups per row (order-independent),
// then the ids and the number of leading rows that match the draft.  One
// workgroup; each thread reads whole 64-byte key records of several workgroups.
__global__ void __launch_bounds__(256) k_lmhead_finalize(QgAffineArgs p, int nwg) {
  __shared__ unsigned long long red[4][8];
  __shared__ int s_ids[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = 0ull;
#pragma unroll 4
  for (int w = threadIdx.x; w < nwg; w += blockDim.x) {
    const ulonglong2* kp = reinterpret_cast<const ulonglong2*>(p.keys + (size_t)w * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const ulonglong2 k = kp[j];
      v[2 * j] = k.x > v[2 * j] ? k.x : v[2 * j];
      v[2 * j + 1] = k.y > v[2 * j + 1] ? k.y : v[2 * j + 1];
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = shfl_xor_u64(v[m], off);
      v[m] = o > v[m] ? o : v[m];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < 8; ++m) red[wave][m] = v[m];
  }
  __syncthreads();
  if ((int)threadIdx.x < p.M) {
    unsigned long long b = 0ull;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) b = red[w][threadIdx.x] > b ? red[w][threadIdx.x] : b;
    const int id = (int)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
    p.ids[threadIdx.x] = id;
    s_ids[threadIdx.x] = id;
  }
  __syncthreads();
  if (threadIdx.x == 0 && p.accepted) {
    int a = 0;
    if (p.draft)
      while (a < p.M && s_ids[a] == p.draft[a]) ++a;
    *p.accepted = a;
  }
}

template <int M, bool WIDE>
static void launch_main(int mode, const QgAffineArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
  switch (mode) {
    case QG_MODE_PLAIN:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLAIN, WIDE>), grid, block, lds, st, a);
      break;
    case QG_MODE_GATEUP:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_GATEUP, WIDE>), grid, block, lds, st, a);
      break;
    default:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_LMHEAD, WIDE>), grid, block, lds, st, a);
      break;
  }
}

template <int M>
static int launch_affine_m(int mode, const QgAffineArgs& a, size_t lds, hipStream_t st) {
  const dim3 grid((unsigned)(a.S * a.rgroups)), block((unsigned)(64 * a.waves));
  if (a.wide)
    launch_main<M, true>(mode, a, grid, block, lds, st);
  else
    launch_main<M, false>(mode, a, grid, block, lds, st);
  int err = (int)hipGetLastError();
  if (err) return err;
  if (mode == QG_MODE_LMHEAD) {
    hipLaunchKernelGGL(k_lmhead_finalize, dim3(1), dim3(256), 0, st, a, (int)grid.x);
  } else if (a.S > 1) {
    const unsigned nblk = (unsigned)(((size_t)a.M * a.N + 255) / 256);
    if (mode == QG_MODE_GATEUP)
      hipLaunchKernelGGL(k_split_reduce<QG_MODE_GATEUP>, dim3(nblk), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_split_reduce<QG_MODE_PLAIN>, dim3(nblk), dim3(256), 0, st, a);
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
