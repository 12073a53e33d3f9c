// affine4.hip -- gfx950 kernels for MLX-style affine 4-bit weights (group 64,
// bf16 scale and bias per group).
//
// One kernel template covers the three affine operations of the decode step:
//   QG_MODE_PLAIN   Y = X . dequant(W)^T                      (qgemv_affine4)
//   QG_MODE_GATEUP  h = silu(xn.Wg^T) * (xn.Wu^T), xn = RMSNorm(x)
//                   (rmsnorm_gateup_swiglu: norm fused into the projection,
//                   gate and up computed together -- Husky page, section
//                   "MSI의 네 가지 구현 요소")
//   QG_MODE_PLAIN8  Y = X . dequant8(W)^T for 8-bit affine codes   (qgemv_affine8;
//                   uzu page: MLX 4- and 8-bit weights)
//   QG_MODE_LMHEAD  logits = X . dequant(W)^T, greedy argmax per row and the
//                   accepted draft prefix, all on the device (uzu page: untied
//                   readout; Husky page: next token handed over on the GPU)
//
// Work decomposition
//   * A "tile" is 16 consecutive weight rows (one MFMA B operand width).  In
//     GATEUP the 2I rows of the gate and up projections form one matrix; its
//     tiles are independent and k_split_reduce pairs gate row n with up row
//     I+n.
//   * A "chunk" is 128 consecutive k (two scale groups): per lane one 16-byte
//     load of codes (4 words = 32 codes) and one scale+bias per lane.
//   * The K axis is cut into S slices of `cps` chunks (split-K across
//     workgroups, used when there are few tiles or when the staged activations
//     would not fit); each workgroup owns one slice and a share of its tiles, stages
//     its slice of X once in LDS, and its waves stream whole tiles.  With
//     S > 1 (and always in GATEUP) every slice stores fp32 partial sums and
//     k_split_reduce, launched next on the same stream, adds them in slice
//     order and applies the epilogue: no atomics, no cross-workgroup fences,
//     and the result does not depend on timing.
//   * The LM head merges each workgroup's best (logit, index) key per row into
//     a running maximum in the workspace header; the last workgroup writes the
//     ids and the accepted count (lmhead_merge_finish).  For the top-k
//     readout it stores the logits and each workgroup's best key per row
//     instead, and k_topk_select (topk.hip) follows.
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
#include <algorithm>

#include "affine_stage.h"

namespace qg {

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t lo2 = (uint32_t)__shfl_xor((int)lo, mask), hi2 = (uint32_t)__shfl_xor((int)hi, mask);
  return ((unsigned long long)hi2 << 32) | lo2;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Greedy verify fused into the LM-head projection.  Every workgroup has
// merged its best key of each row into its group's slot for the row in the
// workspace header (an agent-scope maximum, applied at the device's coherence
// point; blockIdx.x mod kLmGroups picks the group, so each slot takes a
// group's share of the atomics instead of every workgroup's); once those
// atomics have completed it counts itself into its group, and the group's
// last workgroup counts the group in.  The workgroup that completes the last
// group finds every row's maximum across the group slots, writes the ids and
// the number of leading rows that match the draft, and sets the slots and
// counters back to zero for the next call.
template <int M>
__device__ __forceinline__ void lmhead_merge_finish(const QgAffineArgs& p) {
  static_assert(kLmGroups == 8, "one lane per (group, row) below");
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's maximum has been applied
  __syncthreads();
  const unsigned g = blockIdx.x & (kLmGroups - 1);
  const unsigned ngroups = min((unsigned)kLmGroups, gridDim.x);
  if (threadIdx.x == 0) {
    unsigned* gcnt = reinterpret_cast<unsigned*>(p.state + kHdrLmGroupCount + (size_t)g * 64);
    unsigned* cnt = reinterpret_cast<unsigned*>(p.state + kHdrLmCount);
    const unsigned in_group = (gridDim.x - g + kLmGroups - 1) / kLmGroups;
    int l = 0;
    if (__hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_group - 1)
      l = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1;
    last = l;
  }
  __syncthreads();
  if (!last || threadIdx.x >= 64) return;
  const int lane = threadIdx.x, gl = lane >> 3, m = lane & 7;  // lane = group * 8 + row
  unsigned long long* slot =
      reinterpret_cast<unsigned long long*>(p.state + kHdrLmSlots + (size_t)lane * kHdrLmSlotStride);
  unsigned long long key = 0ull;
  if (m < M && (unsigned)gl < ngroups) {
    key = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {  // the maximum over the groups, in every lane of the row
    const unsigned long long o = shfl_xor_u64(key, off);
    key = o > key ? o : key;
  }
  const int id = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
  const bool row = lane < M;  // lanes 0..M-1: group 0's lanes carry the rows' results
  const int draft = (p.draft && row) ? p.draft[lane] : -1;
  if (row) p.ids[lane] = id;
  if (lane < kLmGroups)
    __hip_atomic_store(reinterpret_cast<unsigned*>(p.state + kHdrLmGroupCount + (size_t)lane * 64), 0u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long match = __ballot(row && p.draft && id == draft);
  if (lane == 0) {
    if (p.accepted) *p.accepted = (int)__builtin_ctzll(~match);
    __hip_atomic_store(reinterpret_cast<unsigned*>(p.state + kHdrLmCount), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// WIDE: every batch of every slice lies inside the row and the scale/bias rows
// are aligned for one vector load per batch (the host checks G, the slice
// length and the pointers); the loop body then has no data-dependent branch
// around its loads.
//
// Each wave keeps a ring of R steps of weight loads in flight: the loads of
// step st + R are issued as soon as step st has been computed.  The LM head's
// waves stream several tiles each and keep two steps in flight; the split
// projections' waves live for a few steps and run best with one (measured:
// the extra registers and waits cost more than the overlap gains there).
// Every mode keeps within 128 registers per lane (4 waves per SIMD).
// Workgroups have p.waves waves: four, except gate/up at M < 5, which runs
// 8 or 16 (one staged copy of the slice shared by more waves).
// TK (LM head only): the top-k readout's projection, which stores each
// workgroup's largest key of every row instead of the greedy finish.
template <int M, int MODE, bool WIDE, bool TILED = false, bool TK = false>
__global__ void __launch_bounds__(MODE == QG_MODE_GATEUP ? 1024 : 256) __attribute__((amdgpu_waves_per_eu(4, 8)))
k_affine(QgAffineArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int PL = planes(MODE);  // activation planes (hi, lo)
  constexpr int BATCH = 4;                              // chunks whose loads are issued together
#ifndef QG_R_SPLIT
#define QG_R_SPLIT 1
#endif
  constexpr int R = (MODE == QG_MODE_LMHEAD) ? 2 : QG_R_SPLIT;  // steps of weight loads in flight per wave
  constexpr int CW = (MODE == QG_MODE_PLAIN8) ? 2 : 1;  // 16-byte code loads per lane and chunk
  constexpr bool NTL = (MODE == QG_MODE_LMHEAD);        // non-temporal weight loads (the long LM-head stream)
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S;
  const int rg = blockIdx.x / p.S;
  const int c0 = slice * p.cps;
  const int nc = min(p.cps, p.nchunks - c0);
  // the slice's tiles are dealt round-robin to its rgroups*W waves: wave gw
  // takes tiles gw, gw + nw, ... (neighbouring waves read neighbouring tiles)
  const int gw = rg * W + wave, nw = p.rgroups * W;
  const int ntw = gw < p.ntiles ? (p.ntiles - gw + nw - 1) / nw : 0;
  const int nbt = (nc + BATCH - 1) / BATCH;  // batches per tile
  const int nsteps = ntw * nbt;              // this wave's (tile, batch) steps

  // LDS: a zero region of ZR entries, then the staged slice (xs), its group
  // sums (sx), sums of squares (ssq) and the LM head's per-wave keys.  Lanes
  // whose operand slots carry the other scale group (or a padding row) read
  // the zero region: one select per step instead of a mask per read, and
  // every read of a step is an immediate offset from one base.
  constexpr int ZR = 64 * PL * M;  // spans the operand offsets of one step
  uint4* zr = reinterpret_cast<uint4*>(smem);
  uint4* xs = zr + ZR;
  float* sx = reinterpret_cast<float*>(xs + nc * 16 * M * PL);
  float* ssq = sx + nc * 16;  // GATEUP: [M][2nc]
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(ssq + M * 2 * nc);  // LMHEAD: [W][8]

  const int nl = lane & 15;
  const int kb = lane >> 4;
  const int half = lane >> 5;  // scale group parity of this lane (B and C layouts agree)
  const int rho = lane & 15;
  const bool a_act = ((rho >> 3) == (kb >> 1)) && ((rho & 7) < M);
  // operand entry of this lane for (chunk cl, step t, plane pl): a_lane + (cl*16 + t*4)*PL*M + pl*M of xs
  const uint32_t a_lane = (uint32_t)(ZR + kb * PL * M + (rho & 7));
  const float* sx_base = sx + half * 8 + 4 * (kb & 1);
  const size_t wrow_words = (size_t)p.K / (CW == 2 ? 4 : 8);
  const uint32_t wmax = (uint32_t)(wrow_words - 4 * CW);  // last in-row load (CW 16-byte pieces)
  const int mbase = 4 * (lane >> 4);                 // activation row of C element 0 (lanes < 32)
  const UnpackK uk = unpack_constants();

  // ---- loads of one (tile, batch) step: unconditional, at clamped in-bounds addresses.
  // sw / bw dword u holds the bf16 scales / biases of groups 2(c0+cb+u) (low half) and
  // 2(c0+cb+u)+1 (high half); lane l uses the half of its group parity.
  struct Buf {
    uint4 q[BATCH * CW];
    uint32_t sw[BATCH], bw[BATCH];
  };
  // a step st = ti * nbt + bi (tile ti of the wave's, batch bi of the tile)
  auto load_step = [&](Buf& bf, int st, int ti, int bi) {
    const int cb = bi * BATCH;
    const int row = (gw + ti * nw) * 16 + nl;
    const size_t row_c = (size_t)min(row, p.N - 1);
    const int gb = 2 * (c0 + cb);  // first scale group of the batch
    if constexpr (TILED) {
      // tile order: every load of the wave reads 1 KB (codes) or 256 bytes
      // (scales, biases) of consecutive memory, through a resource based at
      // the step's own bytes.  A step past the wave's last (ring refills at
      // the end, a wave without work) gets resources of zero bytes: the loads
      // are issued, so every wait of the loop leaves the next step's loads in
      // flight, but they read nothing.
      const bool real = st < nsteps;  // uniform
      const size_t tile = (size_t)min(gw + ti * nw, p.ntiles - 1);
      const char* cbase = reinterpret_cast<const char*>(p.codes) + (tile * p.nchunks + c0 + cb) * 1024;
      const auto rc = weight_rsrc(cbase, real ? BATCH * 1024 : 0);
#pragma unroll
      for (int u = 0; u < BATCH; ++u) bf.q[u] = ld_weights<NTL>(rc, lane * 16 + u * 1024);  // 1-KB immediate offsets
      // one 16-byte record per (row, group parity): dword u = (scale, bias) of group 2(c0+cb+u) + half
      const char* rec = reinterpret_cast<const char*>(p.scales) + (tile * (p.nchunks / BATCH) + (c0 + cb) / BATCH) * 512;
      const uint4 sv = ld_weights<NTL>(weight_rsrc(rec, real ? 512 : 0), half * 256 + nl * 16);
      bf.sw[0] = sv.x; bf.sw[1] = sv.y; bf.sw[2] = sv.z; bf.sw[3] = sv.w;
      return;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int cg = WIDE ? c0 + cb + u : c0 + min(cb + u, nc - 1);
      if constexpr (CW == 2) {
        // 8-bit: lane kb's 32 codes of chunk cg are bytes 32kb..32kb+31 of the chunk's 128
        const uint32_t wo = min((uint32_t)(cg * 32 + kb * 8), wmax);
        bf.q[2 * u] = ld_weights<NTL>(p.codes + row_c * wrow_words + wo);
        bf.q[2 * u + 1] = ld_weights<NTL>(p.codes + row_c * wrow_words + wo + 4);
      } else {
        const uint32_t wo = min((uint32_t)(cg * 16 + kb * 4), wmax);
        bf.q[u] = ld_weights<NTL>(p.codes + row_c * wrow_words + wo);
      }
    }
    if constexpr (WIDE) {
      const size_t off = row_c * p.G + gb;
      const uint4 sv = ld_weights<NTL>(p.scales + off);
      const uint4 bv = ld_weights<NTL>(p.biases + off);
      bf.sw[0] = sv.x; bf.sw[1] = sv.y; bf.sw[2] = sv.z; bf.sw[3] = sv.w;
      bf.bw[0] = bv.x; bf.bw[1] = bv.y; bf.bw[2] = bv.z; bf.bw[3] = bv.w;
    } else {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int g = min(gb + 2 * u + half, p.G - 1);
        bf.sw[u] = (uint32_t)p.scales[row_c * p.G + g] << (16 * half);
        bf.bw[u] = (uint32_t)p.biases[row_c * p.G + g] << (16 * half);
      }
    }
  };

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};

  // ---- end of a tile: add the two group halves, then store / publish
  auto finish_tile = [&](int tile) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = add_upper_half(acc[r]);
    const int row = tile * 16 + nl;
    if ((lane < 32) && row < p.N) {
      if (MODE == QG_MODE_GATEUP || p.S > 1) {
        // this slice's sums; k_split_reduce finishes the row (and pairs gate with up)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mbase + r < M) p.part[((size_t)slice * M + mbase + r) * p.N + row] = acc[r];
      } else if (MODE == QG_MODE_LMHEAD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (M == 8 || m < M) {  // lanes < 32 hold rows 0..7
            if (p.logits) p.logits[(size_t)m * p.N + row] = acc[r];
            const unsigned long long key = argmax_key(acc[r], (uint32_t)row);
            best[r] = key > best[r] ? key : best[r];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + r;
          if (m < M) p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(acc[r]);
        }
      }
    }
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // ---- compute one (tile, batch) step: independent MFMA chains per chunk, then the group epilogues
  auto compute_step = [&](const Buf& bf, int ti, int bi) {
    const int cb = bi * BATCH;
    const uint32_t a_base = a_act ? a_lane + (uint32_t)(cb * 16 * PL * M) : 0u;  // entry in zr[]
    f32x4_t C[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) C[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (WIDE || cb + u < nc) {
          uint4 bw;
          if constexpr (CW == 2) {  // MFMA t takes codes 8t..8t+7 of the lane's 32: words 2t and 2t+1
            const uint4& qq = bf.q[2 * u + (t >> 1)];
            bw = unpack_affine8_pair((t & 1) ? qq.z : qq.x, (t & 1) ? qq.w : qq.y);
          } else {
            const uint32_t w = t == 0 ? bf.q[u].x : t == 1 ? bf.q[u].y : t == 2 ? bf.q[u].z : bf.q[u].w;
            bw = unpack_affine_word(w, uk);
          }
#pragma unroll
          for (int pl = 0; pl < PL; ++pl) {
            const uint4 a = zr[a_base + (uint32_t)((u * 16 + t * 4) * PL * M + pl * M)];
            C[u] = mfma_bf16(a, bw, C[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (WIDE || cb + u < nc) {
        const float4 sxv = *reinterpret_cast<const float4*>(sx_base + (cb + u) * 16);
        float sc, cbias;
        if constexpr (TILED) {  // (scale, bias) of this lane's group in one dword
          sc = __uint_as_float(bf.sw[u] << 16);
          cbias = fmaf(-128.0f, sc, __uint_as_float(bf.sw[u] & 0xFFFF0000u));
        } else if constexpr (CW == 2) {  // 8-bit operands carry q itself: no offset to fold
          sc = __uint_as_float((bf.sw[u] >> (16 * half)) << 16);
          cbias = __uint_as_float((bf.bw[u] >> (16 * half)) << 16);
        } else {
          sc = __uint_as_float((bf.sw[u] >> (16 * half)) << 16);
          cbias = fmaf(-128.0f, sc, __uint_as_float((bf.bw[u] >> (16 * half)) << 16));
        }
        acc[0] = fmaf(sc, C[u][0], fmaf(cbias, sxv.x, acc[0]));
        acc[1] = fmaf(sc, C[u][1], fmaf(cbias, sxv.y, acc[1]));
        acc[2] = fmaf(sc, C[u][2], fmaf(cbias, sxv.z, acc[2]));
        acc[3] = fmaf(sc, C[u][3], fmaf(cbias, sxv.w, acc[3]));
      }
    }
    if (bi == nbt - 1) finish_tile(gw + ti * nw);
  };

  // ---- prologue: the activation loads go out first and the first R weight
  // steps right after them, so staging waits only for the former.  A ring
  // slot past the wave's last step reads nothing (see load_step).
  Buf ring[R];
  StageIn<MODE> sin;
  stage_load<M, MODE>(p, c0, nc, 0, sin);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (TILED || r < nsteps) load_step(ring[r], r, r / nbt, r % nbt);
  __builtin_amdgcn_sched_barrier(0);
  for (int i = threadIdx.x; i < ZR; i += blockDim.x) zr[i] = make_uint4(0u, 0u, 0u, 0u);
  if (MODE == QG_MODE_LMHEAD) {
    for (int i = threadIdx.x; i < W * 8; i += blockDim.x) wkeys[i] = 0ull;
  }
  stage_store<M, MODE>(p, xs, sx, ssq, c0, nc, 0, sin);
  const int rounds = (2 * nc + stage_groups(MODE) * W - 1) / (stage_groups(MODE) * W);
  if (rounds > 1) {
    for (int r = 1; r < rounds; ++r) {
      stage_load<M, MODE>(p, c0, nc, r, sin);
      stage_store<M, MODE>(p, xs, sx, ssq, c0, nc, r, sin);
    }
    // the last round's loads past the slice's last group are never read; wait
    // for them here (the reads above have already waited for the weight
    // loads), or the main loop would wait for every load in flight each step
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  __syncthreads();
  if (MODE == QG_MODE_GATEUP && rg == 0 && threadIdx.x < M) {
    float t = 0.f;
    for (int gl = 0; gl < 2 * nc; ++gl) t += ssq[threadIdx.x * 2 * nc + gl];
    p.ssq_part[(size_t)slice * 8 + threadIdx.x] = t;  // this slice's sum of x^2, for k_split_reduce
  }

  // ---- main loop: compute step st from ring slot st % R, then refill the
  // slot with step st + R if there is one (the scheduling barriers keep the
  // compiler from moving loads across the computation that waits for older
  // ones).  Reloading an in-bounds step instead of skipping costs HBM bytes:
  // the weight loads are non-temporal (LM head), so the repeat misses L2.
  // (tile, batch) of the step computed next and of the step loaded next,
  // advanced one step at a time instead of divided out of st
  int cti = 0, cbi = 0, lti = R / nbt, lbi = R % nbt;
  for (int st = 0; st < nsteps; st += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (st + r < nsteps) compute_step(ring[r], cti, cbi);
      if (++cbi == nbt) {  // uniform: the next step computed starts a tile
        cbi = 0;
        ++cti;
      }
      // nothing is reloaded past the last step: the tiled loads read zero
      // bytes there, the row-major ones are skipped (a uniform branch)
      if (TILED || st + r + R < nsteps) load_step(ring[r], st + r + R, lti, lbi);
      if (++lbi == nbt) {
        lbi = 0;
        ++lti;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the workgroup's largest key of each row: merged into the greedy readout's
  // running maxima (then its finish), or stored for the top-k selection.  With
  // K split (S > 1) the slices store partial sums and k_lmhead_reduce does this.
  if (MODE == QG_MODE_LMHEAD && (TK || p.state) && p.S == 1) {
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
      if constexpr (TK) {
        p.cand[(size_t)threadIdx.x * gridDim.x + blockIdx.x] = v;  // 0: the workgroup had no tile
      } else {
        // merged into the group's running maximum of the row (order-independent)
        const size_t slot = ((size_t)(blockIdx.x & (kLmGroups - 1)) * 8 + threadIdx.x) * kHdrLmSlotStride;
        __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(p.state + kHdrLmSlots + slot), v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if constexpr (!TK) lmhead_merge_finish<M>(p);
  }
}

// Split-K epilogue: one thread per output (m, n); the S slices' partial sums
// ([S][M][N] fp32) are added in slice order, then the mode's epilogue: a bf16
// store, or for gate/up (N = 2I: gate rows 0..I-1, up rows I..2I-1) the RMS
// scaling and SwiGLU of the gate and up sums of row n.
template <int MODE>
__global__ void __launch_bounds__(256) k_split_reduce(QgAffineArgs p) {
  constexpr int NB = (MODE == QG_MODE_GATEUP) ? 2 : 1;
  const int NO = p.N / NB;  // outputs per row
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)p.M * NO) return;
  const int m = (int)(idx / (size_t)NO);
  const int n = (int)(idx - (size_t)m * NO);
  const size_t stride = (size_t)p.M * p.N;  // one slice
  const size_t base = (size_t)m * p.N + n;
  // all loads of up to SC slices (gate, up and the sums of squares together) are
  // issued before any is added, so a call waits for one round of load latency per
  // SC slices instead of one per 8 slices and per operand; the additions keep
  // slice order
  constexpr int SC = (MODE == QG_MODE_GATEUP) ? 16 : 32;
  float t[NB], ss = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) t[b] = 0.f;
  for (int s0 = 0; s0 < p.S; s0 += SC) {
    float v[NB][SC], q[SC];
#pragma unroll
    for (int j = 0; j < SC; ++j) {
      if (s0 + j < p.S) {  // uniform across the launch
#pragma unroll
        for (int b = 0; b < NB; ++b) v[b][j] = p.part[(size_t)(s0 + j) * stride + base + (size_t)b * NO];
        if (MODE == QG_MODE_GATEUP) q[j] = p.ssq_part[(size_t)(s0 + j) * 8 + m];
      }
    }
#pragma unroll
    for (int j = 0; j < SC; ++j) {
      if (s0 + j < p.S) {
#pragma unroll
        for (int b = 0; b < NB; ++b) t[b] += v[b][j];
        if (MODE == QG_MODE_GATEUP) ss += q[j];
      }
    }
  }
  if (MODE == QG_MODE_GATEUP) {
    const float ri = 1.0f / sqrtf(ss / (float)p.K + p.eps);
    p.y[idx] = f32_to_bf16_bits(silu_mul(t[0] * ri, t[NB - 1] * ri));
  } else {
    p.y[idx] = f32_to_bf16_bits(t[0]);
  }
}

// Greedy LM head with K split over S slices (K beyond what one slice's M
// staged rows hold in LDS): thread n adds the slices' partial sums of output
// n of every row in slice order (the same additions as k_split_reduce), stores
// the logits if asked, and takes each row's (logit, index) key; the
// workgroup's largest key of each row is merged into the greedy readout's
// running maxima, then the greedy finish runs as in the unsplit projection.
template <int M>
__global__ void __launch_bounds__(256) k_lmhead_reduce(QgAffineArgs p) {
  __shared__ unsigned long long wk[4][8];  // per wave and row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)p.M * p.N;  // one slice
  unsigned long long best[M];
#pragma unroll
  for (int m = 0; m < M; ++m) best[m] = 0ull;
  if (n < p.N) {
    float t[M];
#pragma unroll
    for (int m = 0; m < M; ++m) t[m] = 0.f;
    for (int s = 0; s < p.S; ++s) {
      float v[M];
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] = p.part[(size_t)s * stride + (size_t)m * p.N + n];
#pragma unroll
      for (int m = 0; m < M; ++m) t[m] += v[m];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (p.logits) p.logits[(size_t)m * p.N + n] = t[m];
      best[m] = argmax_key(t[m], (uint32_t)n);
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = shfl_xor_u64(best[m], off);
      best[m] = o > best[m] ? o : best[m];
    }
    if (lane == 0) wk[wave][m] = best[m];
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    unsigned long long v = 0ull;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) v = wk[w][threadIdx.x] > v ? wk[w][threadIdx.x] : v;
    const size_t slot = ((size_t)(blockIdx.x & (kLmGroups - 1)) * 8 + threadIdx.x) * kHdrLmSlotStride;
    __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(p.state + kHdrLmSlots + slot), v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  lmhead_merge_finish<M>(p);
}

// Top-k readout with K split over S slices: workgroup g covers the tiles the
// projection's workgroup g streams when K is not split (tiles 4g + w + t*nw
// for wave w, t < topk_tpw).  Lane (mg, n) of a wave adds the slices' partial
// sums of output n of rows mg and mg + 4 in slice order, stores the logits
// (the selection reads them back) and keeps each row's largest (logit, index)
// key; cand[m][g] gets the workgroup's largest key of row m, as the unsplit
// projection leaves it for k_topk_select.
template <int M>
__global__ void __launch_bounds__(256) k_topk_reduce(QgAffineArgs p) {
  static_assert(kWaves == 4, "the selection reads the tiles of four waves per workgroup");
  __shared__ unsigned long long wk[kWaves][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = p.rgroups * kWaves, gw = blockIdx.x * kWaves + wave;
  const size_t stride = (size_t)p.M * p.N;  // one slice
  const int nl = lane & 15, mg = lane >> 4;   // output of the tile; rows mg and mg + 4
  unsigned long long best[2] = {0ull, 0ull};
  for (int t = 0; t < p.topk_tpw; ++t) {
    const int tile = gw + t * nw;
    const int n = tile * 16 + nl;
    if (tile < p.ntiles && n < p.N) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = mg + 4 * j;
        if (m < M) {
          float v = 0.f;
          for (int s = 0; s < p.S; ++s) v += p.part[(size_t)s * stride + (size_t)m * p.N + n];
          p.logits[(size_t)m * p.N + n] = v;
          const unsigned long long key = argmax_key(v, (uint32_t)n);
          best[j] = key > best[j] ? key : best[j];
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {  // within the 16 lanes of one row group
      const unsigned long long o = shfl_xor_u64(best[j], off);
      best[j] = o > best[j] ? o : best[j];
    }
    if (nl == 0 && mg + 4 * j < M) wk[wave][mg + 4 * j] = best[j];
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    unsigned long long v = 0ull;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v = wk[w][threadIdx.x] > v ? wk[w][threadIdx.x] : v;
    p.cand[(size_t)threadIdx.x * gridDim.x + blockIdx.x] = v;  // 0: the workgroup had no output
  }
}

template <int M, bool WIDE>
static void launch_main(int mode, const QgAffineArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
  if (a.tiled) {  // tile-order weights: plain projection, gate/up and LM head
    if (mode == QG_MODE_LMHEAD && a.topk > 0)
      hipLaunchKernelGGL((k_affine<M, QG_MODE_LMHEAD, true, true, true>), grid, block, lds, st, a);
    else if (mode == QG_MODE_LMHEAD)
      hipLaunchKernelGGL((k_affine<M, QG_MODE_LMHEAD, true, true>), grid, block, lds, st, a);
    else if (mode == QG_MODE_GATEUP)
      hipLaunchKernelGGL((k_affine<M, QG_MODE_GATEUP, true, true>), grid, block, lds, st, a);
    else
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLAIN, true, true>), grid, block, lds, st, a);
    return;
  }
  switch (mode) {
    case QG_MODE_PLAIN:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLAIN, WIDE>), grid, block, lds, st, a);
      break;
    case QG_MODE_GATEUP:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_GATEUP, WIDE>), grid, block, lds, st, a);
      break;
    case QG_MODE_PLANES:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLANES, WIDE>), grid, block, lds, st, a);
      break;
    case QG_MODE_PLAIN8:
      hipLaunchKernelGGL((k_affine<M, QG_MODE_PLAIN8, WIDE>), grid, block, lds, st, a);
      break;
    default:
      if (a.topk > 0)
        hipLaunchKernelGGL((k_affine<M, QG_MODE_LMHEAD, WIDE, false, true>), grid, block, lds, st, a);
      else
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
  if (mode == QG_MODE_LMHEAD && a.topk > 0) {
    if (a.S > 1) {  // K split: add the slices and form the candidate rows first
      hipLaunchKernelGGL(k_topk_reduce<M>, dim3((unsigned)a.rgroups), dim3(64 * kWaves), 0, st, a);
      if ((err = (int)hipGetLastError())) return err;
      return qg_launch_topk(a, a.rgroups, st);
    }
    return qg_launch_topk(a, (int)grid.x, st);
  } else if (mode == QG_MODE_LMHEAD && a.S > 1) {
    hipLaunchKernelGGL(k_lmhead_reduce<M>, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, st, a);
  } else if (a.S > 1 || mode == QG_MODE_GATEUP) {
    const size_t outs = (size_t)a.M * (mode == QG_MODE_GATEUP ? a.N / 2 : a.N);
    const unsigned nblk = (unsigned)((outs + 255) / 256);
    if (mode == QG_MODE_GATEUP)
      hipLaunchKernelGGL(k_split_reduce<QG_MODE_GATEUP>, dim3(nblk), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_split_reduce<QG_MODE_PLAIN>, dim3(nblk), dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

// Tile-order layout of affine-4 weights (K % 512 == 0; Husky page, section
// "MSI의 네 가지 구현 요소": weights laid out in the order the kernel reads
// them).  For 16-row tile t, 128-k chunk c and lane l = 16*kb + n of a wave:
//   codes_t[((t*C + c)*64 + l)*4 + w] = codes[(16t + n)*(K/8) + 16c + 4kb + w]
// (C = K/128 chunks; w = 0..3), i.e. the 16 bytes lane l loads for chunk c,
// so a load of the whole wave reads 1 KB of consecutive memory; and for
// batch b of 8 groups, group parity h and u = 0..3:
//   sb_t[(((t*B + b)*2 + h)*16 + n)*8 + 2u]     = scales[(16t + n)*G + 8b + 2u + h]
//   sb_t[(((t*B + b)*2 + h)*16 + n)*8 + 2u + 1] = biases[(16t + n)*G + 8b + 2u + h]
// (B = K/512 batches, G = K/64 groups): the 16 bytes a lane of parity h needs
// for one step.  Rows past N are zero.
__global__ void __launch_bounds__(256) k_tile_pack(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                                   const uint16_t* __restrict__ biases, uint32_t* __restrict__ codes_t,
                                                   uint16_t* __restrict__ sb_t, int N, int K) {
  const int C = K / 128, B = K / 512, G = K / 64;
  const int ntiles = (N + 15) / 16;
  const size_t ncode = (size_t)ntiles * C * 64;  // 16-byte pieces of codes_t
  const size_t nsb = (size_t)ntiles * B * 2 * 16;  // 16-byte pieces of sb_t
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < ncode + nsb; i += (size_t)gridDim.x * blockDim.x) {
    if (i < ncode) {
      const int l = (int)(i % 64), n = l & 15, kb = l >> 4;
      const size_t tc = i / 64;
      const int c = (int)(tc % C), t = (int)(tc / C);
      const int row = 16 * t + n;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < N) v = *reinterpret_cast<const uint4*>(codes + (size_t)row * (K / 8) + 16 * c + 4 * kb);
      *reinterpret_cast<uint4*>(codes_t + i * 4) = v;
    } else {
      const size_t q = i - ncode;
      const int n = (int)(q % 16), h = (int)((q / 16) % 2);
      const size_t tb = q / 32;
      const int b = (int)(tb % B), t = (int)(tb / B);
      const int row = 16 * t + n;
      const size_t g0 = (size_t)row * G + 8 * b + h;
      uint16_t* dst = sb_t + q * 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[2 * u] = row < N ? scales[g0 + 2 * u] : (uint16_t)0;
        dst[2 * u + 1] = row < N ? biases[g0 + 2 * u] : (uint16_t)0;
      }
    }
  }
}

}  // namespace qg

int qg_launch_split_reduce_plain(const QgAffineArgs& a, hipStream_t st) {
  const unsigned nblk = (unsigned)(((size_t)a.M * a.N + 255) / 256);
  hipLaunchKernelGGL(qg::k_split_reduce<QG_MODE_PLAIN>, dim3(nblk), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

int qg_launch_tile_pack(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, uint32_t* codes_t,
                        uint16_t* sb_t, int N, int K, hipStream_t st) {
  const size_t pieces = (size_t)((N + 15) / 16) * ((size_t)K / 128 * 64 + (size_t)K / 512 * 32);
  const unsigned grid = (unsigned)std::min<size_t>(65535, (pieces + 255) / 256);
  hipLaunchKernelGGL(qg::k_tile_pack, dim3(grid), dim3(256), 0, st, codes, scales, biases, codes_t, sb_t, N, K);
  return (int)hipGetLastError();
}

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
