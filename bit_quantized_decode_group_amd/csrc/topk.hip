// topk.hip -- top-k readout of the LM head (uzu page, section "내부 동작 3:
// DFlash + Weaver": the target's readout rows give candidate pools of their
// best tokens).  Runs after the LM-head projection has stored the fp32 logits
// [M][V]; two kernels on the caller's stream:
//   k_topk_block   one workgroup per (row, block of kTopkBlock logits): the
//                  block's logits become (logit, index) keys and its k largest
//                  keys are written out;
//   k_topk_merge   one workgroup per row: the k largest of the blocks'
//                  candidates, written as ids (and their logits).
// Keys are argmax_key (common.h): a larger logit first, equal logits by lower
// index, a NaN above every number (NaNs by lower index).  The keys of a row
// are distinct, so "the k largest keys" is one well-defined set in one order,
// and the result does not depend on scheduling.  A row's k largest keys are
// among its blocks' k largest, so the merge sees all of them.
//
// Selection (both kernels): radix select of the k-th largest key, eight bits
// at a time from the top (an LDS histogram of the next digit among the keys
// that share the bits chosen so far, then the digit where the count from the
// top reaches k); it stops as soon as the chosen digit's bucket holds exactly
// the keys still needed.  The selected keys (at most 64) are gathered and
// sorted by one wave with a bitonic network over its 64 lanes.
#include "common.h"

namespace qg {

struct TopkSmem {
  unsigned hist[256];
  unsigned long long list[kTopkMax];
  unsigned long long prefix, mask;
  unsigned need, count, done;
};

__device__ __forceinline__ unsigned long long shfl_xor_key(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m), hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// The k largest of the workgroup's keys (KPT per thread; 0 marks an empty
// slot and is below every key), largest first, into out[0..k).  Every thread
// of the workgroup calls it.
template <int KPT, bool AGG_FIRST>
__device__ void select_topk(const unsigned long long (&key)[KPT], int k, unsigned long long* out, TopkSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) {
    sm.prefix = 0ull;
    sm.mask = 0ull;
    sm.need = (unsigned)k;
    sm.count = 0u;
    sm.done = 0u;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) sm.hist[i] = 0u;
    __syncthreads();
    const unsigned long long prefix = sm.prefix, mask = sm.mask;
    if (sm.done) break;  // uniform: read after the barrier
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      // empty slots are not counted; with AGG_FIRST the first pass (sign and
      // top exponent bits of candidates that are already the largest of
      // their blocks: a handful of distinct digits) counts the keys of a wave
      // that share a digit with one atomic
      unsigned d = (key[j] != 0ull && (key[j] & mask) == prefix) ? (unsigned)((key[j] >> shift) & 255u) : 256u;
      if (AGG_FIRST && shift == 56) {
        unsigned long long pending = __ballot(d != 256u);
        while (pending) {
          const int leader = __builtin_ctzll(pending);
          const unsigned dl = (unsigned)__builtin_amdgcn_readlane((int)d, leader);
          const unsigned long long same = __ballot(d == dl);
          if (lane == leader) atomicAdd(&sm.hist[dl], (unsigned)__builtin_popcountll(same));
          pending &= ~same;
          if (d == dl) d = 256u;
        }
      } else if (d != 256u) {
        atomicAdd(&sm.hist[d], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l..4l+3; counts from the top (bin 255) down
      const unsigned b0 = sm.hist[4 * lane], b1 = sm.hist[4 * lane + 1], b2 = sm.hist[4 * lane + 2],
                     b3 = sm.hist[4 * lane + 3];
      const unsigned s = b0 + b1 + b2 + b3;
      unsigned suf = s;  // sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = (unsigned)__shfl_down((int)suf, off);
        if (lane + off < 64) suf += o;
      }
      const unsigned need = sm.need;
      const unsigned above = suf - s;  // keys in bins above this lane's
      if (above < need && need <= suf) {
        unsigned acc = above, d = 0u, cnt = 0u;
        const unsigned bins[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (acc < need && need <= acc + bins[q] && cnt == 0u) {
            d = (unsigned)(4 * lane + q);
            cnt = bins[q];
            sm.need = need - acc;
          }
          if (cnt == 0u) acc += bins[q];
        }
        sm.prefix = prefix | ((unsigned long long)d << shift);
        sm.mask = mask | (255ull << shift);
        if (cnt == need - acc) sm.done = 1u;  // the bucket holds exactly the keys still needed
      }
    }
    __syncthreads();
  }
  // selected: the resolved high bits at or above the threshold's
  const unsigned long long prefix = sm.prefix, mask = sm.mask;
  if (tid < kTopkMax) sm.list[tid] = 0ull;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (key[j] != 0ull && (key[j] & mask) >= prefix) {
      const unsigned pos = atomicAdd(&sm.count, 1u);
      if (pos < (unsigned)kTopkMax) sm.list[pos] = key[j];
    }
  }
  __syncthreads();
  if (tid < 64) {  // one wave sorts the (at most 64) selected keys, largest first
    unsigned long long v = sm.list[lane];
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const unsigned long long o = shfl_xor_key(v, stride);
        const bool lower = (lane & stride) == 0;   // this lane holds the pair's first element
        const bool desc = (lane & size) == 0;      // the run this pair belongs to ends up descending
        const bool take_max = (lower == desc);
        v = take_max ? (o > v ? o : v) : (o < v ? o : v);
      }
    }
    if (lane < k) out[lane] = v;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) k_topk_block(QgAffineArgs p, int nblk) {
  __shared__ TopkSmem sm;
  constexpr int KPT = kTopkBlock / 256;
  const int m = blockIdx.y, b = blockIdx.x;
  const int v0 = b * kTopkBlock;
  const float* row = p.logits + (size_t)m * p.N;
  unsigned long long key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int v = v0 + (int)threadIdx.x + 256 * j;
    key[j] = v < p.N ? argmax_key(row[v], (uint32_t)v) : 0ull;
  }
  select_topk<KPT, false>(key, p.topk, p.cand + ((size_t)m * nblk + b) * p.topk, sm);
}

__global__ void __launch_bounds__(1024) k_topk_merge(QgAffineArgs p, int nblk) {
  __shared__ TopkSmem sm;
  __shared__ unsigned long long best[kTopkMax];
  constexpr int KPT = kTopkMergeMax / 1024;
  const int m = blockIdx.x;
  const int n = nblk * p.topk;
  const unsigned long long* in = p.cand + (size_t)m * n;
  unsigned long long key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = (int)threadIdx.x + 1024 * j;
    key[j] = i < n ? in[i] : 0ull;
  }
  select_topk<KPT, true>(key, p.topk, best, sm);
  for (int j = threadIdx.x; j < p.topk; j += blockDim.x) {
    const int id = (int)(0xFFFFFFFFu - (uint32_t)(best[j] & 0xFFFFFFFFull));
    p.ids[(size_t)m * p.topk + j] = id;
    // every selected key is a real logit's (the row has at least k of them),
    // so id is in range; the clamp only keeps the read inside the row
    if (p.topk_vals) p.topk_vals[(size_t)m * p.topk + j] = p.logits[(size_t)m * p.N + min(max(id, 0), p.N - 1)];
  }
}

}  // namespace qg

int qg_launch_topk(const QgAffineArgs& a, hipStream_t st) {
  const int nblk = (a.N + kTopkBlock - 1) / kTopkBlock;
  hipLaunchKernelGGL(qg::k_topk_block, dim3((unsigned)nblk, (unsigned)a.M), dim3(256), 0, st, a, nblk);
  int err = (int)hipGetLastError();
  if (err) return err;
  hipLaunchKernelGGL(qg::k_topk_merge, dim3((unsigned)a.M), dim3(1024), 0, st, a, nblk);
  return (int)hipGetLastError();
}
