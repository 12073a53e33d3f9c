// valu.hip -- measurement aid: the affine-4 projection with the M-row
// products on the vector ALU (v_dot2_f32_bf16) instead of MFMA, on the same
// plan (K slices, workgroups, waves, tiles), the same staged activations and
// the same split-K reduce as qgemv_affine4's kernel, so the two differ only
// in how the products are formed.  Not on the decode path: it exists to
// compare the matrix cores with packed vector arithmetic at M = 1..8.
//
// Lane l = 16*kb + n of a wave owns row n of its 16-row tile and, per 128-k
// chunk c, the 32 codes of word t = 0..3 at k = 128c + 32kb + 8t + i (the
// canonical layout's 16 bytes at codes[row][16c + 4kb ..]).  For each word
// it unpacks the codes as bf16 pairs 128+q (unpack_affine_word: dword j holds
// codes j and j+4), reads the staged activations of every row m (the entry
// holds the same pairs of x) and accumulates D[m] = sum x*(128+q) with four
// v_dot2_f32_bf16 per row.  Per chunk it folds its group's scale s and bias
// b: acc[m] += s*D[m], and the lane with kb even adds (b - 128 s) * (group
// sum of x) once per group.  At the end of a tile the four lanes of a row
// (kb = 0..3) add their sums with two butterflies.
#include "affine_stage.h"

namespace qg {

constexpr int kValuBatch = 4;  // chunks whose loads are issued together

struct ValuBuf {
  uint4 q[kValuBatch];
  uint32_t s[kValuBatch], b[kValuBatch];  // bf16 bits of this lane's group scale and bias per chunk
};

template <int M>
__global__ void __launch_bounds__(256) k_affine_valu(QgAffineArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S, rg = blockIdx.x / p.S;
  const int c0 = slice * p.cps;
  const int nc = min(p.cps, p.nchunks - c0);
  const int gw = rg * W + wave, nw = p.rgroups * W;
  const int ntw = gw < p.ntiles ? (p.ntiles - gw + nw - 1) / nw : 0;
  const int nbt = (nc + kValuBatch - 1) / kValuBatch;
  const int nsteps = ntw * nbt;
  uint4* xs = reinterpret_cast<uint4*>(smem);                // [nc*16][M] staged entries
  float* sx = reinterpret_cast<float*>(xs + (size_t)nc * 16 * M);  // [2*nc][8] group sums
  const int n = lane & 15, kb = lane >> 4, par = kb >> 1;
  const size_t K8 = (size_t)(p.K / 8);

  // loads of step st (tile, batch of chunks); chunks past the slice or groups
  // past the row load nothing and contribute zero
  // (with p.wide every batch lies inside the row, and its eight scales and
  // eight biases are one aligned 16-byte load each, as in k_affine)
  auto load_step = [&](ValuBuf& bf, int st) {
    const int tile = gw + (st / nbt) * nw, bi = st % nbt;
    const int row = min(tile * 16 + n, p.N - 1);
    if (p.wide) {
      const size_t g0 = (size_t)row * p.G + 2 * (c0 + bi * kValuBatch);
      const uint4 sv = *reinterpret_cast<const uint4*>(p.scales + g0);
      const uint4 bv = *reinterpret_cast<const uint4*>(p.biases + g0);
      const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int u = 0; u < kValuBatch; ++u) {
        const int cl = bi * kValuBatch + u;
        bf.q[u] = *reinterpret_cast<const uint4*>(p.codes + (size_t)row * K8 + (size_t)(c0 + cl) * 16 + 4 * kb);
        bf.s[u] = par ? (sw[u] >> 16) : (sw[u] & 0xFFFFu);  // group 2(c0+cl)+par is element 2u+par
        bf.b[u] = par ? (bw[u] >> 16) : (bw[u] & 0xFFFFu);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kValuBatch; ++u) {
      const int cl = bi * kValuBatch + u;
      const int g = 2 * (c0 + cl) + par;
      const bool ok = (cl < nc) && (g < p.G);
      bf.q[u] = ok ? *reinterpret_cast<const uint4*>(p.codes + (size_t)row * K8 + (size_t)(c0 + cl) * 16 + 4 * kb)
                   : make_uint4(0u, 0u, 0u, 0u);
      bf.s[u] = ok ? p.scales[(size_t)row * p.G + g] : 0u;
      bf.b[u] = ok ? p.biases[(size_t)row * p.G + g] : 0u;
    }
  };

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  const UnpackK uk = unpack_constants();

  auto compute_step = [&](const ValuBuf& bf, int st) {
    const int tile = gw + (st / nbt) * nw, bi = st % nbt;
#pragma unroll
    for (int u = 0; u < kValuBatch; ++u) {
      const int cl = bi * kValuBatch + u;
      if (cl >= nc) break;  // uniform across the wave
      float D[M];
#pragma unroll
      for (int m = 0; m < M; ++m) D[m] = 0.f;
      const uint32_t w[4] = {bf.q[u].x, bf.q[u].y, bf.q[u].z, bf.q[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 wv = unpack_affine_word(w[t], uk);
        const uint4* xe = xs + (size_t)((cl * 4 + t) * 4 + kb) * M;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint4 xv = xe[m];
          D[m] = dot2_bf16(xv.x, wv.x, D[m]);
          D[m] = dot2_bf16(xv.y, wv.y, D[m]);
          D[m] = dot2_bf16(xv.z, wv.z, D[m]);
          D[m] = dot2_bf16(xv.w, wv.w, D[m]);
        }
      }
      const float s = bf16_bits_to_f32(bf.s[u]);
      // the group's offset and bias term, added by one of its two lanes
      const float off = (kb & 1) ? 0.f : fmaf(-128.f, s, bf16_bits_to_f32(bf.b[u]));
      const float* sg = sx + (2 * cl + par) * 8;
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = fmaf(s, D[m], fmaf(off, sg[m], acc[m]));
    }
    if (bi == nbt - 1) {  // tile done: add the four lanes of each row, store, reset
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m] += __shfl_xor(acc[m], 16);
        acc[m] += __shfl_xor(acc[m], 32);
      }
      const int row = tile * 16 + n;
      if (kb == 0 && row < p.N) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          if (p.S == 1)
            p.y[(size_t)m * p.N + row] = f32_to_bf16_bits(acc[m]);
          else  // this slice's sums; k_split_reduce adds the slices in order
            p.part[((size_t)slice * M + m) * p.N + row] = acc[m];
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.f;
    }
  };

  // stage the slice (activation loads first, then the first weight step)
  const int last = max(nsteps - 1, 0);
  ValuBuf bufA, bufB;
  StageIn<QG_MODE_PLAIN> sin;
  stage_load<M, QG_MODE_PLAIN>(p, c0, nc, 0, sin);
  __builtin_amdgcn_sched_barrier(0);
  load_step(bufA, 0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<M, QG_MODE_PLAIN>(p, xs, sx, nullptr, c0, nc, 0, sin);
  const int rounds = (2 * nc + stage_groups(QG_MODE_PLAIN) * W - 1) / (stage_groups(QG_MODE_PLAIN) * W);
  for (int r = 1; r < rounds; ++r) {
    stage_load<M, QG_MODE_PLAIN>(p, c0, nc, r, sin);
    stage_store<M, QG_MODE_PLAIN>(p, xs, sx, nullptr, c0, nc, r, sin);
  }
  __syncthreads();

  // two buffers: the loads of the next step are in flight while one is computed
  for (int st = 0; st < nsteps; st += 2) {
    load_step(bufB, min(st + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    compute_step(bufA, st);
    load_step(bufA, min(st + 2, last));
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nsteps) compute_step(bufB, st + 1);
  }
}

template <int M>
static int launch_valu_m(const QgAffineArgs& a, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_affine_valu<M>), dim3((unsigned)(a.S * a.rgroups)), dim3((unsigned)(64 * a.waves)), lds, st, a);
  const int err = (int)hipGetLastError();
  if (err || a.S == 1) return err;
  return qg_launch_split_reduce_plain(a, st);
}

}  // namespace qg

size_t qg_valu_lds_bytes(int M, int cps) { return (size_t)cps * (256 * (size_t)M + 64); }

int qg_launch_affine_valu(const QgAffineArgs& a, hipStream_t st) {
  const size_t lds = qg_valu_lds_bytes(a.M, a.cps);
  switch (a.M) {
    case 1: return qg::launch_valu_m<1>(a, lds, st);
    case 2: return qg::launch_valu_m<2>(a, lds, st);
    case 3: return qg::launch_valu_m<3>(a, lds, st);
    case 4: return qg::launch_valu_m<4>(a, lds, st);
    case 5: return qg::launch_valu_m<5>(a, lds, st);
    case 6: return qg::launch_valu_m<6>(a, lds, st);
    case 7: return qg::launch_valu_m<7>(a, lds, st);
    case 8: return qg::launch_valu_m<8>(a, lds, st);
    default: return (int)hipErrorInvalidValue;
  }
}
