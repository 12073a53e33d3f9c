// mlp.hip -- the MLP block of one decode step in a single persistent launch
// (Husky page, section "MSI의 네 가지 구현 요소": one dispatch for the layer's
// MLP; the same page notes that a single dispatch pays off only when the
// weight reads of one projection overlap the tail of the previous one):
//
//   phase A  gate/up split-K partial sums of RMSNorm(x) . [Wg; Wu]^T
//   phase B  per (row, output pair): sum of the slices, RMS scale, SwiGLU -> h
//   phase C  down split-K partial sums of h . Wd^T
//   phase D  sum of the slices -> y
//
// Weights are in the tile-order layout (affine4.hip).  Every workgroup of the
// launch is resident at once (the host sizes the grid from the occupancy of
// this kernel), and the phases are separated by a grid barrier.  Before the
// first barrier each workgroup issues the weight loads of its first phase-C
// job, so that the down projection's weights stream in while phase B and the
// barriers run.
//
// The same kernel runs a stack of L blocks, block l + 1 taking block l's
// output as its input (the page's next step: one dispatch spanning layers).
// A fifth barrier separates the blocks; before waiting on it each workgroup
// issues the loads of its first gate/up step of the next block, whose
// weights do not depend on the block that is finishing.
//
// Data handed from one workgroup to another within the launch (partial sums,
// sums of squares, h) is written with agent-scope stores and read with
// agent-scope loads; the barrier waits for each thread's stores to complete
// before it counts the workgroup as arrived.  The slices are added in slice
// order with the same arithmetic as k_split_reduce, so h and y are identical
// to those of the separate entry points run with the same split.
#include <algorithm>

#include "affine_stage.h"

namespace qg {

namespace {

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two-level grid barrier.  The grid is split into kBarGroups groups of equal
// size; a workgroup adds one to its group's counter, the last arrival of a
// group adds one to the top counter, and the last group to arrive writes the
// barrier's sequence number into every group's release word.  Each workgroup
// then polls its own group's release word, so no single address is polled by
// the whole grid (a hot address slows every load that maps to its memory
// channel).  Arrival and wait are separate so that a workgroup can issue
// loads that do not depend on the other workgroups in between (waiting for
// the stores to complete, vmcnt(0), would also wait for such loads).  The wait
// is bounded: after spin_limit polls the workgroup records the failure and
// goes on.  The state lives in the caller's workspace, is zero when a launch
// starts, and the last workgroup to leave the launch sets it back to zero.
//
// Barrier state (bytes): [0, 8) top counter, [16, 20) failure flag of this
// launch, [20, 24) failed launches not yet reported, [32, 40) exit counter;
// group g at 256 * (g + 1): [0, 8) arrival counter, [8, 16) release word.
constexpr int kBarGroups = 32;

__device__ __forceinline__ void barrier_arrive(unsigned char* bar, unsigned long long* target_lds) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned gs = gridDim.x / kBarGroups;
    const unsigned g = blockIdx.x / gs;
    unsigned long long* gc = reinterpret_cast<unsigned long long*>(bar + 256 * (g + 1));
    const unsigned long long a = __hip_atomic_fetch_add(gc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long k = a / gs;  // sequence number of this barrier on this state
    *target_lds = k + 1;
    if (a % gs == gs - 1) {  // the group is complete
      unsigned long long* top = reinterpret_cast<unsigned long long*>(bar);
      const unsigned long long t = __hip_atomic_fetch_add(top, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t % kBarGroups == kBarGroups - 1) {  // every group is complete: release them all
        for (int q = 0; q < kBarGroups; ++q)
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(bar + 256 * (q + 1) + 8), k + 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__device__ __forceinline__ void barrier_wait(unsigned char* bar, const unsigned long long* target_lds,
                                             int spin_limit) {
  if (threadIdx.x == 0) {
    const unsigned gs = gridDim.x / kBarGroups;
    const unsigned g = blockIdx.x / gs;
    const unsigned long long* rel = reinterpret_cast<const unsigned long long*>(bar + 256 * (g + 1) + 8);
    const unsigned long long target = *target_lds;
    int it = 0;
    while (__hip_atomic_load(rel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it >= spin_limit) {
        __hip_atomic_store(reinterpret_cast<unsigned*>(bar + 16), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// One step of tile-order loads: four 128-k chunks of codes (16 bytes per
// lane each) and the (scale, bias) record of this lane's group parity.
struct TBuf {
  uint4 q[4];
  uint4 sb;
};

// A job is one (K slice, row group) of a split plan, as one workgroup of the
// separate projection kernel would run it.  The host guarantees that cps and
// K/128 are multiples of 4 (every slice is whole batches).
struct Job {
  int slice, rg, c0, nc, gw, nw, ntw, nbt, nsteps;
};

__device__ __forceinline__ Job job_of(const QgAffineArgs& p, int job) {
  Job j;
  const int W = blockDim.x >> 6, wave = wave_id();
  j.slice = job % p.S;
  j.rg = job / p.S;
  j.c0 = j.slice * p.cps;
  j.nc = min(p.cps, p.nchunks - j.c0);  // a multiple of 4 (K % 512 == 0)
  j.gw = j.rg * W + wave;
  j.nw = p.rgroups * W;
  j.ntw = j.gw < p.ntiles ? (p.ntiles - j.gw + j.nw - 1) / j.nw : 0;
  j.nbt = j.nc / 4;
  j.nsteps = j.ntw * j.nbt;
  return j;
}

// Loads of step st of the job (clamped to an in-bounds tile: a wave without
// work reloads a real one and discards it).
__device__ __forceinline__ void load_tstep(const QgAffineArgs& p, const Job& j, int st, TBuf& b) {
  const int lane = threadIdx.x & 63, nl = lane & 15, half = lane >> 5;
  const int ti = st / j.nbt;
  const int cb = (st - ti * j.nbt) * 4;
  const size_t tile = (size_t)min(j.gw + ti * j.nw, p.ntiles - 1);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    b.q[u] = ld_weights<false>(p.codes + ((tile * p.nchunks + j.c0 + cb + u) * 64 + lane) * 4);
  const uint16_t* rec = p.scales + ((tile * (p.nchunks / 4) + (j.c0 + cb) / 4) * 2 + half) * 128 + nl * 8;
  b.sb = ld_weights<false>(rec);
}

// Stage the job's slice of X, run its steps (the first R from `pre` when
// given), and store each finished tile's partial sums of this slice with
// agent-scope stores.  MODE is QG_MODE_GATEUP (X = the block input, hi/lo
// planes of x*gamma, sums of x^2 per slice) or QG_MODE_PLAIN (X = h, written
// by phase B of this launch, read with agent-scope loads).
template <int M, int MODE, int R>
__device__ void run_job(const QgAffineArgs& p, int job, unsigned char* smem, TBuf (&ring)[R], bool preloaded) {
  constexpr int PL = planes(MODE);
  // X was written earlier in this launch (h by phase B; a layer's input by the
  // previous layer's phase D), so it is read with agent-scope loads
  constexpr bool COH_X = true;
  const Job j = job_of(p, job);
  const int nc = j.nc;
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  constexpr int ZR = 64 * PL * M;
  uint4* zr = reinterpret_cast<uint4*>(smem);
  uint4* xs = zr + ZR;
  float* sx = reinterpret_cast<float*>(xs + nc * 16 * M * PL);
  float* ssq = sx + nc * 16;

  const int nl = lane & 15, kb = lane >> 4, half = lane >> 5, rho = lane & 15;
  const bool a_act = ((rho >> 3) == (kb >> 1)) && ((rho & 7) < M);
  const uint32_t a_lane = (uint32_t)(ZR + kb * PL * M + (rho & 7));
  const float* sx_base = sx + half * 8 + 4 * (kb & 1);
  const int mbase = 4 * (lane >> 4);
  const UnpackK uk = unpack_constants();
  const int last = max(j.nsteps - 1, 0);

  StageIn<MODE> sin;
  stage_load<M, MODE, COH_X>(p, j.c0, nc, 0, sin);
  __builtin_amdgcn_sched_barrier(0);
  if (!preloaded) {
#pragma unroll
    for (int r = 0; r < R; ++r) load_tstep(p, j, min(r, last), ring[r]);
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int i = threadIdx.x; i < ZR; i += blockDim.x) zr[i] = make_uint4(0u, 0u, 0u, 0u);
  stage_store<M, MODE>(p, xs, sx, ssq, j.c0, nc, 0, sin);
  const int rounds = (2 * nc + stage_groups(MODE) * W - 1) / (stage_groups(MODE) * W);
  for (int r = 1; r < rounds; ++r) {
    stage_load<M, MODE, COH_X>(p, j.c0, nc, r, sin);
    stage_store<M, MODE>(p, xs, sx, ssq, j.c0, nc, r, sin);
  }
  __syncthreads();
  if (MODE == QG_MODE_GATEUP && j.rg == 0 && threadIdx.x < M) {
    float t = 0.f;
    for (int gl = 0; gl < 2 * nc; ++gl) t += ssq[threadIdx.x * 2 * nc + gl];
    st_coh(p.ssq_part + (size_t)j.slice * 8 + threadIdx.x, t);
  }

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int st0 = 0; st0 < j.nsteps; st0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int st = st0 + r;
      if (st < j.nsteps) {
        const TBuf& b = ring[r];
        const int ti = st / j.nbt;
        const int bi = st - ti * j.nbt;
        const int cb = bi * 4;
        const uint32_t a_base = a_act ? a_lane + (uint32_t)(cb * 16 * PL * M) : 0u;
        f32x4_t C[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) C[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t w = t == 0 ? b.q[u].x : t == 1 ? b.q[u].y : t == 2 ? b.q[u].z : b.q[u].w;
            const uint4 bw = unpack_affine_word(w, uk);
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
              const uint4 a = zr[a_base + (uint32_t)((u * 16 + t * 4) * PL * M + pl * M)];
              C[u] = mfma_bf16(a, bw, C[u]);
            }
          }
        }
        const uint32_t sbw[4] = {b.sb.x, b.sb.y, b.sb.z, b.sb.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 sxv = *reinterpret_cast<const float4*>(sx_base + (cb + u) * 16);
          const float sc = __uint_as_float(sbw[u] << 16);
          const float cbias = fmaf(-128.0f, sc, __uint_as_float(sbw[u] & 0xFFFF0000u));
          acc[0] = fmaf(sc, C[u][0], fmaf(cbias, sxv.x, acc[0]));
          acc[1] = fmaf(sc, C[u][1], fmaf(cbias, sxv.y, acc[1]));
          acc[2] = fmaf(sc, C[u][2], fmaf(cbias, sxv.z, acc[2]));
          acc[3] = fmaf(sc, C[u][3], fmaf(cbias, sxv.w, acc[3]));
        }
        if (bi == j.nbt - 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += __shfl_xor(acc[q], 32);
          const int row = (j.gw + ti * j.nw) * 16 + nl;
          if (lane < 32 && row < p.N) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (mbase + q < M) st_coh(p.part + ((size_t)j.slice * M + mbase + q) * p.N + row, acc[q]);
          }
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
      load_tstep(p, j, min(st + R, last), ring[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();  // the next job re-stages LDS
}

__device__ __forceinline__ float silu_mul_f(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Sum over the S slices of part[s*stride + off], in slice order; the loads of
// eight slices are issued together (agent-scope loads wait one by one when
// each is used right away).
__device__ __forceinline__ float sum_slices(const float* part, size_t stride, size_t off, int S) {
  float t = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld_coh(part + (size_t)min(s0 + j, S - 1) * stride + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) t += v[j];
  }
  return t;
}

// Phase B: outputs n, n+1 of row m (the same arithmetic as k_split_reduce for gate/up).
__device__ __forceinline__ void gateup_pair(const QgAffineArgs& p, int m, int n, uint32_t* h) {
  const int I = p.N / 2;
  const size_t stride = (size_t)p.M * p.N;
  const size_t base = (size_t)m * p.N + n;
  float t[2][2];
  if (p.S <= 8) {  // every load of the item in flight at once
    float v[2][2][8], w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t so = (size_t)min(j, p.S - 1) * stride + base;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int b = 0; b < 2; ++b) v[e][b][j] = ld_coh(p.part + so + e + (size_t)b * I);
      w[j] = ld_coh(p.ssq_part + (size_t)min(j, p.S - 1) * 8 + m);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < p.S) acc += v[e][b][j];
        t[e][b] = acc;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < p.S) ss += w[j];
    const float ri = 1.0f / sqrtf(ss / (float)p.K + p.eps);
    const uint32_t h0 = f32_to_bf16_bits(silu_mul_f(t[0][0] * ri, t[0][1] * ri));
    const uint32_t h1 = f32_to_bf16_bits(silu_mul_f(t[1][0] * ri, t[1][1] * ri));
    st_coh(h + ((size_t)m * I + n) / 2, h0 | (h1 << 16));
    return;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int b = 0; b < 2; ++b) t[e][b] = sum_slices(p.part, stride, base + e + (size_t)b * I, p.S);
  const float ss = sum_slices(p.ssq_part, 8, (size_t)m, p.S);
  const float ri = 1.0f / sqrtf(ss / (float)p.K + p.eps);
  const uint32_t h0 = f32_to_bf16_bits(silu_mul_f(t[0][0] * ri, t[0][1] * ri));
  const uint32_t h1 = f32_to_bf16_bits(silu_mul_f(t[1][0] * ri, t[1][1] * ri));
  st_coh(h + ((size_t)m * I + n) / 2, h0 | (h1 << 16));
}

}  // namespace

// grid: one workgroup per resident slot (a multiple of kBarGroups); pa
// (gate/up) and pc (down) carry the split plans and layer 0's pointers; st
// gives the number of layers and the strides from one layer's weights,
// gamma and output to the next's; pc.x is h; bar: the barrier state
// (kBarGroups + 1 slots of 256 bytes).  Layer l reads its input from layer
// l - 1's output (layer 0: pa.x) and writes its output to pc.y + l * y_stride.
template <int M>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
    k_mlp_block(QgAffineArgs pa0, QgAffineArgs pc0, QgMlpStack st, unsigned char* bar, int spin_limit) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int R = 2;  // down-projection steps in flight per wave (prefetched before the barriers)
  const int P = gridDim.x;
  __shared__ unsigned long long target;
  const int ja = pa0.S * pa0.rgroups, jc = pc0.S * pc0.rgroups;
  // the first gate/up job's weights of the next layer go out before the barrier
  // that precedes its phase A (layer 0: at the start)
  TBuf ring_a[1];
  bool a_pre = false;
  for (int l = 0; l < st.L; ++l) {
    QgAffineArgs pa = pa0, pc = pc0;
    pa.codes += (size_t)l * st.gu_codes;
    pa.scales += (size_t)l * st.gu_sb;
    pa.biases = pa.scales;
    pa.gamma += (size_t)l * st.gamma;
    if (l > 0) pa.x = pc0.y + (size_t)(l - 1) * st.y;
    pc.codes += (size_t)l * st.dn_codes;
    pc.scales += (size_t)l * st.dn_sb;
    pc.biases = pc.scales;
    pc.y += (size_t)l * st.y;
    // phase A (one step in flight, as the separate gate/up kernel)
    for (int job = blockIdx.x; job < ja; job += P) {
      run_job<M, QG_MODE_GATEUP, 1>(pa, job, smem, ring_a, a_pre && job == (int)blockIdx.x);
    }
    a_pre = false;
    barrier_arrive(bar, &target);
    // the first phase-C job's weights go out while the barriers and phase B run
    TBuf pre[R];
    if ((int)blockIdx.x < jc) {
      const Job j = job_of(pc, blockIdx.x);
#pragma unroll
      for (int r = 0; r < R; ++r) load_tstep(pc, j, min(r, max(j.nsteps - 1, 0)), pre[r]);
    }
    barrier_wait(bar, &target, spin_limit);
    // phase B
    {
      const int I = pa.N / 2;
      const int npairs = pa.M * (I / 2);
      uint32_t* h = reinterpret_cast<uint32_t*>(pa.y);
      for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < npairs; i += P * blockDim.x) {
        const int m = i / (I / 2);
        gateup_pair(pa, m, 2 * (i - m * (I / 2)), h);
      }
    }
    barrier_arrive(bar, &target);
    barrier_wait(bar, &target, spin_limit);
    // phase C
    for (int job = blockIdx.x; job < jc; job += P) run_job<M, QG_MODE_PLAIN, R>(pc, job, smem, pre, job == (int)blockIdx.x);
    barrier_arrive(bar, &target);
    barrier_wait(bar, &target, spin_limit);
    // phase D (the same arithmetic as k_split_reduce for a plain projection);
    // agent-scope stores: the next layer's phase A and a failed launch's NaN
    // fill below read or overwrite them from other workgroups
    {
      const int n_out = pc.M * pc.N;
      const size_t stride = (size_t)pc.M * pc.N;
      for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_out; i += P * blockDim.x)
        __hip_atomic_store(pc.y + i, f32_to_bf16_bits(sum_slices(pc.part, stride, (size_t)i, pc.S)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (l + 1 < st.L) {
      barrier_arrive(bar, &target);
      // the next layer's first gate/up weights (they do not depend on this layer's output)
      if ((int)blockIdx.x < ja) {
        QgAffineArgs pn = pa0;
        pn.codes += (size_t)(l + 1) * st.gu_codes;
        pn.scales += (size_t)(l + 1) * st.gu_sb;
        load_tstep(pn, job_of(pn, blockIdx.x), 0, ring_a[0]);
        a_pre = true;
      }
      barrier_wait(bar, &target, spin_limit);
    }
  }
  // exit: the last workgroup to leave (every other one has passed its last
  // wait and its stores have completed) fills h and y with NaN if a wait of
  // this launch gave up, counts the failure, and sets the barrier state back
  // to zero for the next launch on this workspace
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int last_out;
  if (threadIdx.x == 0) {
    const unsigned long long a = __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(bar + 32), 1ull,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_out = (a == (unsigned long long)gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last_out) return;
  const unsigned failed = __hip_atomic_load(reinterpret_cast<unsigned*>(bar + 16), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  if (failed) {
    const uint16_t qnan = 0x7FC0;
    for (size_t i = threadIdx.x; i < (size_t)st.L * st.y; i += blockDim.x)
      __hip_atomic_store(pc0.y + i, qnan, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < pa0.M * (pa0.N / 2); i += blockDim.x)
      __hip_atomic_store(pa0.y + i, qnan, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < kBarGroups) {
    unsigned long long* g = reinterpret_cast<unsigned long long*>(bar + 256 * (threadIdx.x + 1));
    __hip_atomic_store(g, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(g + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) {
    if (failed) __hip_atomic_fetch_add(reinterpret_cast<unsigned*>(bar + 20), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<unsigned*>(bar + 16), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(bar), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(bar + 32), 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace qg

namespace {
// A cooperative launch: the runtime refuses a grid whose workgroups cannot
// all be resident at once, instead of letting the grid barrier wait for
// workgroups that are not running.
template <int M>
int launch_mlp_m(QgAffineArgs pa, QgAffineArgs pc, QgMlpStack stk, unsigned char* bar, int spin_limit, int grid,
                 size_t lds, hipStream_t st) {
  void* args[] = {&pa, &pc, &stk, &bar, &spin_limit};
  return (int)hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&qg::k_mlp_block<M>), dim3((unsigned)grid),
                                         dim3(256), args, (unsigned)lds, st);
}
}  // namespace

const void* qg_mlp_kernel(int M) {
  switch (M) {
    case 1: return reinterpret_cast<const void*>(&qg::k_mlp_block<1>);
    case 2: return reinterpret_cast<const void*>(&qg::k_mlp_block<2>);
    case 3: return reinterpret_cast<const void*>(&qg::k_mlp_block<3>);
    case 4: return reinterpret_cast<const void*>(&qg::k_mlp_block<4>);
    case 5: return reinterpret_cast<const void*>(&qg::k_mlp_block<5>);
    case 6: return reinterpret_cast<const void*>(&qg::k_mlp_block<6>);
    case 7: return reinterpret_cast<const void*>(&qg::k_mlp_block<7>);
    case 8: return reinterpret_cast<const void*>(&qg::k_mlp_block<8>);
    default: return nullptr;
  }
}

size_t qg_mlp_state_bytes() { return (size_t)256 * (qg::kBarGroups + 1); }

int qg_launch_mlp(const QgAffineArgs& pa, const QgAffineArgs& pc, const QgMlpStack& stk, unsigned char* bar,
                  int spin_limit, int grid, size_t lds, hipStream_t st) {
  if (grid % qg::kBarGroups != 0) return (int)hipErrorInvalidValue;
  switch (pa.M) {
    case 1: return launch_mlp_m<1>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 2: return launch_mlp_m<2>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 3: return launch_mlp_m<3>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 4: return launch_mlp_m<4>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 5: return launch_mlp_m<5>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 6: return launch_mlp_m<6>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 7: return launch_mlp_m<7>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    case 8: return launch_mlp_m<8>(pa, pc, stk, bar, spin_limit, grid, lds, st);
    default: return (int)hipErrorInvalidValue;
  }
}
