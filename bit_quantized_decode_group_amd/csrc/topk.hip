// topk.hip -- top-k readout of the LM head (uzu page, section "내부 동작 3:
// DFlash + Weaver": the target's readout rows give candidate pools of their
// best tokens).  Runs after the LM-head projection on the caller's stream.
//
// Keys are argmax_key (common.h): a larger logit first, equal logits by lower
// index, a NaN above every number (NaNs by lower index).  The keys of a row
// are distinct, so "the k largest keys" is one well-defined set in one order,
// and the result does not depend on scheduling.
//
// The projection has stored the fp32 logits [M][V] and, per row, the largest
// key of each of its workgroups (the greedy readout's per-workgroup maxima).
// k_topk_select, one workgroup per row, then:
//   1. ranks the workgroup maxima: T is the k-th largest of them (or 1, the
//      smallest key, with at most k workgroups holding keys).  k distinct keys
//      are >= T, so every key of the row's top k is >= T, and a key >= T lies
//      in a workgroup whose maximum is >= T: exactly the k workgroups ranked
//      first (or all of them).
//   2. reads the logits of those workgroups' tiles only (k * 16 * waves *
//      tiles-per-wave logits, against V for the whole row) and keeps the keys
//      >= T: for logits without heavy ties near the top, about k of them.
//   3. ranks the kept keys (each key's count of larger kept keys is its
//      place) and writes the first k as ids (and logits).  Up to 1024 kept
//      keys are ranked directly; more (heavy ties, or a few workgroups holding
//      the whole row) are first cut to the k largest by a radix selection,
//      the slow but general path.
#include "common.h"

namespace qg {

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

// The largest key of the wave, in every lane.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long v) {
  auto step = [](unsigned long long x, auto xor_fn) {
    const unsigned long long o = ((unsigned long long)xor_fn((uint32_t)(x >> 32)) << 32) | xor_fn((uint32_t)x);
    return max_u64(x, o);
  };
  v = step(v, [](uint32_t u) { return lane_xor<1>(u); });
  v = step(v, [](uint32_t u) { return lane_xor<2>(u); });
  v = step(v, [](uint32_t u) { return lane_xor<4>(u); });
  v = step(v, [](uint32_t u) { return lane_xor<8>(u); });
  {
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = max_u64(((unsigned long long)h[0] << 32) | l[0], ((unsigned long long)h[1] << 32) | l[1]);
  }
  {
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = max_u64(((unsigned long long)h[0] << 32) | l[0], ((unsigned long long)h[1] << 32) | l[1]);
  }
  return v;
}

// The k-th largest of the wave's nonzero keys (one per lane, distinct, more
// than k of them), two bits per round from the top: the counts of keys that
// carry the bits chosen so far and then 11, 10 or 01 decide both bits.
// Exactly k keys are >= the result.
__device__ __forceinline__ unsigned long long wave_kth_largest_1(unsigned long long v, unsigned k) {
  unsigned long long prefix = 0ull, mask = 0ull;
  unsigned need = k;
  for (int b = 62; b >= 0; b -= 2) {
    const unsigned long long hm = mask | (3ull << b);
    const unsigned long long key = v & hm;
    const unsigned c3 = (unsigned)__popcll(__ballot(key == (prefix | (3ull << b))));
    const unsigned c2 = (unsigned)__popcll(__ballot(key == (prefix | (2ull << b))));
    const unsigned c1 = (unsigned)__popcll(__ballot(key == (prefix | (1ull << b))));
    mask = hm;
    if (c3 >= need) {
      prefix |= 3ull << b;
      if (c3 == need) break;
    } else if (c3 + c2 >= need) {
      need -= c3;
      prefix |= 2ull << b;
      if (c2 == need) break;
    } else if (c3 + c2 + c1 >= need) {
      need -= c3 + c2;
      prefix |= 1ull << b;
      if (c1 == need) break;
    } else {
      need -= c3 + c2 + c1;  // the next two bits are 00
    }
  }
  return prefix;
}

__device__ __forceinline__ unsigned lane_rank(unsigned long long ballot) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
}

struct SelectSmem {
  unsigned long long kept[kTopkSurvLds];  // keys >= T; more spill to p.surv
  unsigned long long cmax[kTopkMaxWg];    // workgroup maxima at or above the first bound
  int cwg[kTopkMaxWg];                    // their workgroups
  unsigned hist[256];
  unsigned long long top[kTopkMax];
  int wsel[kTopkMax];  // the workgroups ranked first, largest maximum first
  unsigned long long lb[kTopkMaxWg / 64];
  unsigned nzw[kTopkMaxWg / 64];
  unsigned long long thr, prefix, mask;
  unsigned nsel, ncand, count, need, done, ntop;
};

// Rank of a key among keys[0..n) (the count of larger keys; keys distinct),
// n <= 1024, all 1024 threads: P = 1024 / (n rounded up to a power of two)
// neighbouring threads (at most 64) share key i = tid / P, each counting
// every P-th key, and add their counts.  The first thread of each group
// (lead) gets i < n: the key, its index and its rank.
struct Ranked {
  unsigned long long key;
  unsigned idx, rank;
  bool lead;
};
__device__ __forceinline__ Ranked rank_of(const unsigned long long* keys, unsigned n) {
  unsigned np = 1;
  while (np < n) np <<= 1;
  const unsigned P = min(64u, max(1u, 1024u / np));
  const unsigned i = threadIdx.x / P, r0 = threadIdx.x & (P - 1);
  const unsigned long long key = i < n ? keys[i] : 0ull;
  unsigned rank = 0, j = r0;
  for (; j + 7 * P < n; j += 8 * P) {  // eight LDS reads in flight
    unsigned long long v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = keys[j + u * P];
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += v[u] > key ? 1u : 0u;
  }
  for (; j < n; j += P) rank += keys[j] > key ? 1u : 0u;
  rank = group_sum(rank, P);
  return Ranked{key, i, rank, r0 == 0 && i < n};
}

// The k largest of the n kept keys (n > 1024) into sm.top, in no order: a
// radix selection of the k-th largest key, eight bits at a time from the top
// (an LDS histogram of the next digit among the keys that share the bits
// chosen so far, then the digit where the count from the top reaches the keys
// still needed); it stops once the chosen digit's bucket holds exactly the
// keys still needed.  Every thread calls it.
__device__ void select_kept(SelectSmem& sm, const unsigned long long* spill, unsigned n, unsigned k) {
  const int tid = threadIdx.x, lane = tid & 63;
  auto key_at = [&](unsigned i) { return i < (unsigned)kTopkSurvLds ? sm.kept[i] : spill[i]; };
  if (tid == 0) {
    sm.prefix = 0ull;
    sm.mask = 0ull;
    sm.need = k;
    sm.done = 0u;
    sm.ntop = 0u;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) sm.hist[i] = 0u;
    __syncthreads();
    const unsigned long long prefix = sm.prefix, mask = sm.mask;
    if (sm.done) break;  // uniform: read after the barrier
    for (unsigned i = tid; i < n; i += blockDim.x) {
      const unsigned long long key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(unsigned)((key >> shift) & 255u)], 1u);
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
          }
          if (cnt == 0u) acc += bins[q];
        }
        sm.need = need - acc;
        sm.prefix = prefix | ((unsigned long long)d << shift);
        sm.mask = mask | (255ull << shift);
        if (cnt == need - acc) sm.done = 1u;  // the bucket holds exactly the keys still needed
      }
    }
    __syncthreads();
  }
  const unsigned long long prefix = sm.prefix, mask = sm.mask;
  for (unsigned i = tid; i < n; i += blockDim.x) {
    const unsigned long long key = key_at(i);
    if ((key & mask) >= prefix) {
      const unsigned pos = atomicAdd(&sm.ntop, 1u);
      if (pos < (unsigned)kTopkMax) sm.top[pos] = key;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(1024) k_topk_select(QgAffineArgs p, int nwg) {
  __shared__ SelectSmem sm;
  constexpr int NW1 = kTopkMaxWg / 64;  // waves holding the workgroup maxima
  static_assert(kWaves == 4, "a workgroup's four waves streamed four neighbouring tiles per step");
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwave = (int)(blockDim.x >> 6);
  const unsigned k = (unsigned)p.topk;
  const int tpw = p.topk_tpw, nw = p.rgroups * kWaves;
  const size_t stride = (size_t)min((int)k, nwg) * 16 * kWaves * tpw;
  unsigned long long* spill = p.surv + (size_t)m * stride;

  // 1. T, the k-th largest workgroup maximum, and the k workgroups holding
  //    the largest.  A first bound: each of the NW1 waves finds the
  //    ceil(k/NW1)-th largest of its 64 maxima (or 1 when it holds fewer);
  //    at least k maxima reach the smallest of those.  The maxima at or above
  //    it are then ranked among themselves.
  const unsigned long long mx = tid < nwg ? p.cand[(size_t)m * nwg + tid] : 0ull;
  if (wave < NW1) {
    const unsigned kw = (k + NW1 - 1) / NW1;
    const unsigned nz = (unsigned)__popcll(__ballot(mx != 0ull));
    const unsigned long long lb = nz <= kw ? 1ull : kw == 1 ? wave_max_key(mx) : wave_kth_largest_1(mx, kw);
    if (lane == 0) {
      sm.lb[wave] = lb;
      sm.nzw[wave] = nz;
    }
  }
  if (tid == 0) {
    sm.ncand = 0u;
    sm.count = 0u;
  }
  __syncthreads();
  unsigned long long L = sm.lb[0];
  unsigned nz = sm.nzw[0];
#pragma unroll
  for (int w = 1; w < NW1; ++w) {
    L = sm.lb[w] < L ? sm.lb[w] : L;
    nz += sm.nzw[w];
  }
  if (nz <= k) L = 1ull;  // every workgroup with a key is selected
  if (wave < NW1) {
    const bool c = mx >= L;  // L >= 1: no empty maximum
    const unsigned long long b = __ballot(c);
    if (b) {
      unsigned base = 0;
      if (lane == 0) base = atomicAdd(&sm.ncand, (unsigned)__popcll(b));
      base = (unsigned)__builtin_amdgcn_readfirstlane((int)base);
      if (c) {
        const unsigned pos = base + lane_rank(b);
        sm.cmax[pos] = mx;
        sm.cwg[pos] = tid;
      }
    }
  }
  __syncthreads();
  {
    const unsigned nc = sm.ncand;
    const Ranked r = rank_of(sm.cmax, nc);
    if (r.lead && r.rank < k) {
      sm.wsel[r.rank] = sm.cwg[r.idx];
      if (r.rank == k - 1 && nc > k) sm.thr = r.key;
    }
    if (tid == 0) {
      sm.nsel = min(nc, k);
      if (nc <= k) sm.thr = 1ull;  // at most k workgroups hold keys: all of them, every key
    }
  }
  __syncthreads();

  // 2. the keys >= T in those workgroups' tiles.  At step t the four waves of
  //    workgroup g streamed tiles 4g .. 4g+3 + t*nw: 64 neighbouring logits,
  //    a unit.  Units are dealt eight per wave load (lanes 8u..8u+7 read unit
  //    u's logits, eight each), QB loads in flight per wave.  A logit below
  //    T's value cannot give a key >= T: a load none of whose logits reach it
  //    is dropped after one compare per logit; in the rest, each component
  //    some lane may keep builds its keys and appends the ones >= T (one LDS
  //    atomic per wave and component).
  constexpr int QB = 4;
  const unsigned long long T = sm.thr;
  const float Tf = key_logit(T);  // NaN when T is a NaN key or 1: then no logit is dropped early
  const int nsel = (int)sm.nsel;
  const int nunits = nsel * tpw, nops = (nunits + 7) >> 3;
  const float rtpw = 1.0f / (float)tpw;
  const float* lg = p.logits + (size_t)m * p.N;
  const bool vec = (p.N % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.logits) & 15u) == 0);
  for (int o0 = wave; o0 < nops; o0 += QB * nwave) {
    float f[QB][8];
    int vb[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int o = o0 + q * nwave;  // uniform across the wave
      vb[q] = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[q][j] = 0.f;
      if (o < nops) {
        const int uu = 8 * o + (lane >> 3);
        if (uu < nunits) {
          const int sel = (int)(((float)uu + 0.5f) * rtpw), t = uu - sel * tpw;
          const int v0 = (sm.wsel[sel] * kWaves + t * nw) * 16 + (lane & 7) * 8;
          if (v0 < p.N) vb[q] = v0;
        }
        if (vb[q] >= 0) {
          if (vec) {  // N % 4 == 0: a quad that starts in the row ends in it
            const float4 a = *reinterpret_cast<const float4*>(lg + vb[q]);
            f[q][0] = a.x; f[q][1] = a.y; f[q][2] = a.z; f[q][3] = a.w;
            if (vb[q] + 4 < p.N) {
              const float4 b = *reinterpret_cast<const float4*>(lg + vb[q] + 4);
              f[q][4] = b.x; f[q][5] = b.y; f[q][6] = b.z; f[q][7] = b.w;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (vb[q] + j < p.N) f[q][j] = lg[vb[q] + j];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (o0 + q * nwave >= nops) break;  // uniform
      unsigned long long any = 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j) any |= __ballot(!(f[q][j] < Tf));
      if (!any) continue;  // uniform: no key of the load reaches T
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool c = vb[q] >= 0 && vb[q] + j < p.N && !(f[q][j] < Tf);
        if (!__ballot(c)) continue;  // uniform
        const unsigned long long key = c ? argmax_key(f[q][j], (uint32_t)(vb[q] + j)) : 0ull;
        const bool keep = key >= T;  // T >= 1: no empty key
        const unsigned long long b = __ballot(keep);
        if (!b) continue;
        unsigned base = 0;
        if (lane == 0) base = atomicAdd(&sm.count, (unsigned)__popcll(b));
        base = (unsigned)__builtin_amdgcn_readfirstlane((int)base);
        if (keep) {
          const unsigned pos = base + lane_rank(b);
          if (pos < (unsigned)kTopkSurvLds)
            sm.kept[pos] = key;
          else
            spill[pos] = key;
        }
      }
    }
  }
  __syncthreads();

  // 3. the k largest, in order: up to 1024 kept keys are ranked directly;
  //    more are first cut to the k largest by the radix selection
  static_assert(kTopkSurvLds >= 1024, "up to 1024 kept keys are ranked in LDS");
  const unsigned n = sm.count;
  const unsigned long long* keys = sm.kept;
  unsigned nk = n;
  if (n > 1024) {
    __threadfence_block();  // the spilled keys are read back by other threads
    __syncthreads();
    select_kept(sm, spill, n, k);
    keys = sm.top;
    nk = k;
  }
  const Ranked r = rank_of(keys, nk);
  if (r.lead && r.rank < k) {
    p.ids[(size_t)m * k + r.rank] = (int)(0xFFFFFFFFu - (uint32_t)(r.key & 0xFFFFFFFFull));
    if (p.topk_vals) p.topk_vals[(size_t)m * k + r.rank] = key_logit(r.key);
  }
}

}  // namespace qg

// nwg: the projection's workgroups (rows of cand)
int qg_launch_topk(const QgAffineArgs& a, int nwg, hipStream_t st) {
  hipLaunchKernelGGL(qg::k_topk_select, dim3((unsigned)a.M), dim3(1024), 0, st, a, nwg);
  return (int)hipGetLastError();
}
