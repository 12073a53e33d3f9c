// q4k.hip -- gfx950 kernels for GGUF Q4_K weights (256-weight superblocks,
// eight 32-weight sub-blocks with 6-bit scales and mins, fp16 d and dmin),
// consumed as stored (runNburn page, section "GGUF를 그대로 진실의 원본으로 둡니다").
//
//   k_q4k          Y = X . dequant(W)^T                          (qgemv_q4k)
//   k_moe_gateup   route, then h_e = silu(G_e x) * (U_e x) for every selected
//                  expert e, into a bf16 workspace (with the routing)
//   k_moe_down     y = sum_e p_e Down_e h_e over the selected experts in
//                  ascending expert order
//   (uzu page: MixtureOfExperts with a routing function; runNburn page: the
//   engine never alters routing or quantisation semantics -- the selected set
//   and weights are the plain top-k / softmax of the given logits.)
//
// Operand mapping (see common.h for the MFMA scheme).  A Q4_K "chunk" is 64
// consecutive weights = 32 code bytes = sub-blocks 2c (low nibbles) and 2c+1
// (high nibbles).  Lane l (row l%16, kb = l/16) loads 16 consecutive code
// bytes from each half of the block: bytes 64p + 16kb .. +15 (p = 0, 1), i.e.
// lanes kb = 0, 1 hold chunk 2p and lanes kb = 2, 3 chunk 2p+1 -- one
// 16-byte load per half instead of four 8-byte ones.  MFMA (p, t, n) takes the
// nibbles n (0 low, 1 high) of bytes 8t..8t+7 of every lane's 16: C rows 0..7
// then sum sub-block j = 4p + n (chunk 2p) and rows 8..15 sub-block j + 2
// (chunk 2p+1), and lane l's C values belong to sub-block 4p + n + 2*(l/32).
// Slot s of a lane holds code byte {0,2,1,3,4,6,5,7}[s] of its eight bytes.
#include "common.h"

namespace qg {

constexpr int kSbBatch = 2;  // superblocks whose loads are issued together (default)

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Stage activation rows [M][K-slice of nsb superblocks starting at sb0] into
// LDS in operand order.  Entry ((((sbl*2 + p)*2 + t)*2 + n)*4 + kb)*M + m
// holds, for superblock sbl of the slice, the eight activations of row m at
// k = 256*sbl + 64c + 32n + 16(kb%2) + 8t + byte(s) with c = 2p + kb/2 (the
// operand of MFMA (p, t, n) for lane kb); sx[jl*8 + m] is the fp32 sum of
// sub-block jl's 32 staged values.  Source rows are bf16 (T = uint16_t) or
// fp32 rounded to bf16 (T = float).
// One staged piece: the 32 bf16 values (as 16 dword pairs in v) of sub-block
// jl of row m of a region, into that region's operand entries and sub-block sums.
template <int M>
__device__ __forceinline__ void stage_q4k_piece(const uint4 (&hv)[4], uint4* rxs, float* rsx, int jl, int m) {
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i] = hv[i].x; v[4 * i + 1] = hv[i].y; v[4 * i + 2] = hv[i].z; v[4 * i + 3] = hv[i].w;
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sum += bf16_bits_to_f32(v[i] & 0xFFFFu);
    sum += bf16_bits_to_f32(v[i] >> 16);
  }
  const int sbl = jl >> 3, c = (jl >> 1) & 3, nb = jl & 1, pp = c >> 1;
  constexpr int kByte[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int kbn = 2 * (c & 1) + (g >> 1), t = g & 1;
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int klo = 8 * g + kByte[2 * j], khi = 8 * g + kByte[2 * j + 1];
      const uint32_t lo = (klo & 1) ? (v[klo >> 1] >> 16) : (v[klo >> 1] & 0xFFFFu);
      const uint32_t hi = (khi & 1) ? (v[khi >> 1] >> 16) : (v[khi >> 1] & 0xFFFFu);
      e[j] = lo | (hi << 16);
    }
    rxs[((((sbl * 2 + pp) * 2 + t) * 2 + nb) * 4 + kbn) * M + m] = make_uint4(e[0], e[1], e[2], e[3]);
  }
  rsx[jl * 8 + m] = sum;
}

template <int M, typename T>
__device__ __forceinline__ void stage_q4k_x(const T* src, size_t ld, int K, uint4* xs, float* sx, int sb0,
                                            int nsb, int tid, int nthr, int regions = 1) {
  // `regions` > 1 stages that many independent M-row activations (source rows
  // r*M.., region r at xs + r*nsb*32*M and sx + r*nsb*64)
  const int nj = 8 * nsb;
  for (int pi = tid; pi < regions * M * nj; pi += nthr) {
    const int reg = pi / (M * nj);
    const int m = (pi - reg * M * nj) / nj;
    const int jl = pi - reg * M * nj - m * nj;
    const size_t k0 = (size_t)(sb0 * 8 + jl) * 32;
    const size_t srow = (size_t)reg * M + m;
    uint4 hv[4] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u),
                   make_uint4(0u, 0u, 0u, 0u)};  // 32 bf16 values, pairs
    if (k0 < (size_t)K) {
      if constexpr (sizeof(T) == 2) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src + srow * ld + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = s4[i];
      } else {
        const float4* s4 = reinterpret_cast<const float4*>(src + srow * ld + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 a = s4[2 * i], b = s4[2 * i + 1];
          hv[i] = make_uint4((uint32_t)f32_to_bf16_bits(a.x) | ((uint32_t)f32_to_bf16_bits(a.y) << 16),
                             (uint32_t)f32_to_bf16_bits(a.z) | ((uint32_t)f32_to_bf16_bits(a.w) << 16),
                             (uint32_t)f32_to_bf16_bits(b.x) | ((uint32_t)f32_to_bf16_bits(b.y) << 16),
                             (uint32_t)f32_to_bf16_bits(b.z) | ((uint32_t)f32_to_bf16_bits(b.w) << 16));
        }
      }
    }
    stage_q4k_piece<M>(hv, xs + (size_t)reg * nsb * 32 * M, sx + (size_t)reg * nsb * 64, jl, m);
  }
  if (M < 8) {
    for (int pi = tid; pi < regions * nj * (8 - M); pi += nthr)
      sx[(pi / (8 - M)) * 8 + M + pi % (8 - M)] = 0.f;
  }
}

// Loads of one batch of SB superblocks for NB tiles: each block's 16-byte
// header and this lane's 16 code bytes of each half of the block.
template <int NB, int SB = kSbBatch>
struct Q4kBuf {
  uint4 hdr[NB][SB];
  uint4 cq[NB][SB][2];
};

// Issues the loads of the batch starting at superblock sb (clamped to the
// last of nsb, so every address is in bounds; the caller clamps the row).
template <int NB, int SB>
__device__ __forceinline__ void q4k_load(Q4kBuf<NB, SB>& bf, const uint8_t* const (&blk)[NB], int sb, int nsb, int kb) {
#pragma unroll
  for (int u = 0; u < SB; ++u) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint8_t* bp = blk[b] + (size_t)min(sb + u, nsb - 1) * 144;
      bf.hdr[b][u] = ld_weights<false>(bp);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) bf.cq[b][u][hh] = ld_weights<false>(bp + 16 + 64 * hh + 16 * kb);
    }
  }
}

// Accumulate one lane's share of a 16-row tile over nsb superblocks of K into
// acc[b] for NB tiles whose (row, superblock 0) blocks start at blk[b].  `cur`
// holds the loads of the first batch (issued by the caller, so they can be in
// flight while the activations are staged); each batch's successor, if any,
// is loaded before the batch is used.  xs / sx are this slice's staged activations,
// read from lds[region + entry]; lds[0] is a zero entry that lanes whose
// slots carry the other sub-block (or a padding row) read instead.
template <int M, int NB, int SB = kSbBatch>
__device__ __forceinline__ void q4k_tile(f32x4_t (&acc)[NB], const uint8_t* const (&blk)[NB], int nsb,
                                         const uint4* lds, uint32_t region, const float* sx, int lane,
                                         Q4kBuf<NB, SB> cur) {
  const int kb = lane >> 4;
  const int half = lane >> 5;
  const int rho = lane & 15;
  // A rows 0..7 take k-slots of lanes kb = 0, 1 and rows 8..15 those of kb = 2, 3
  const uint32_t amask = (((rho >> 3) == (kb >> 1)) && ((rho & 7) < M)) ? 0xFFFFFFFFu : 0u;
  const uint32_t a_lane = region + (uint32_t)(kb * M + (rho & 7));
  const float* sx_base = sx + half * 16 + 4 * (kb & 1);  // + 8*(8*sbl + 4p + n): sub-block 4p + n + 2*half
  const UnpackK uk = unpack_constants();

  auto compute = [&](const Q4kBuf<NB, SB>& cur, int sb) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int sbl = sb + u;
      if (sbl >= nsb) break;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 h = cur.hdr[b][u];
        const float d = f16_bits_to_f32(h.x & 0xFFFFu);
        const float dmin = f16_bits_to_f32(h.x >> 16);
        const uint32_t Y = h.y >> (16 * half), Z = h.z >> (16 * half), Wd = h.w >> (16 * half);
        // six-bit scale / min of sub-block j = 4p + n + 2*half, q = 2p + n (public
        // Q4_K packing: j < 4 in the low six bits of bytes j, j+4; j >= 4 from
        // byte j+4's nibbles and the top two bits of bytes j-4, j)
        const uint32_t sc[4] = {Y & 63u, (Y >> 8) & 63u, (Wd & 15u) | ((Y >> 2) & 0x30u),
                                ((Wd >> 8) & 15u) | ((Y >> 10) & 0x30u)};
        const uint32_t mn[4] = {Z & 63u, (Z >> 8) & 63u, ((Wd >> 4) & 15u) | ((Z >> 2) & 0x30u),
                                ((Wd >> 12) & 15u) | ((Z >> 10) & 0x30u)};
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // c = 2p + n
          const int pp = c >> 1, nb = c & 1;
          const uint32_t ai = a_lane + (uint32_t)((((sbl * 2 + pp) * 2) * 2 + nb) * 4 * M);
          const uint4 a0 = lds[ai & amask];                  // t = 0
          const uint4 a1 = lds[(ai + 8 * M) & amask];        // t = 1: eight entries on (two n x four kb)
          const uint4 q = cur.cq[b][u][pp];
          f32x4_t C = {0.f, 0.f, 0.f, 0.f};
          C = mfma_bf16(a0, unpack_q4k_bytes(q.x, q.y, 4u * (uint32_t)nb, uk), C);
          C = mfma_bf16(a1, unpack_q4k_bytes(q.z, q.w, 4u * (uint32_t)nb, uk), C);
          const float4 sxv = *reinterpret_cast<const float4*>(sx_base + (8 * sbl + 4 * pp + nb) * 8);
          const float a = d * (float)sc[c];                 // exact in fp32
          const float bt = fmaf(dmin, (float)mn[c], 128.0f * a);
          acc[b][0] = fmaf(a, C[0], fmaf(-bt, sxv.x, acc[b][0]));
          acc[b][1] = fmaf(a, C[1], fmaf(-bt, sxv.y, acc[b][1]));
          acc[b][2] = fmaf(a, C[2], fmaf(-bt, sxv.z, acc[b][2]));
          acc[b][3] = fmaf(a, C[3], fmaf(-bt, sxv.w, acc[b][3]));
        }
      }
    }
  };
  // every batch but the last has a successor to load first; the loop body has
  // no branch around its loads
  int sb = 0;
  for (; sb + SB < nsb; sb += SB) {
    Q4kBuf<NB, SB> nxt;
    q4k_load<NB, SB>(nxt, blk, sb + SB, nsb, kb);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, sb);
    cur = nxt;
  }
  compute(cur, sb);
}

// ------------------------------------------------------------ qgemv_q4k --
template <int M>
__global__ void __launch_bounds__(256) k_q4k(QgQ4kArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = wave_id(), W = blockDim.x >> 6;
  const int slice = blockIdx.x % p.S, rg = blockIdx.x / p.S;
  const int sb0 = slice * p.cps;
  const int nsb = min(p.cps, p.nchunks - sb0);  // here a "chunk" of the split is one superblock
  uint4* lds = reinterpret_cast<uint4*>(smem);  // [0] zero entry, then the staged slice
  float* sx = reinterpret_cast<float*>(lds + 1 + nsb * 32 * M);
  const int nb_row = p.K / 256;
  auto tile_blocks = [&](int it, bool& row_ok) {
    const int tile = min((rg * W) * p.tpw + wave + it * W, p.ntiles - 1);
    const int row = tile * 16 + (lane & 15);
    row_ok = row < p.N;
    return p.blocks + ((size_t)(row_ok ? row : 0) * nb_row + sb0) * 144;
  };
  // the first tile's first weight batch is in flight while the slice is staged
  bool ok0;
  const uint8_t* blk0[1] = {tile_blocks(0, ok0)};
  (void)ok0;
  Q4kBuf<1> first;
  q4k_load<1>(first, blk0, 0, nsb, lane >> 4);
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x == 0) lds[0] = make_uint4(0u, 0u, 0u, 0u);
  stage_q4k_x<M, uint16_t>(p.x, (size_t)p.K, p.K, lds + 1, sx, sb0, nsb, threadIdx.x, blockDim.x);
  __syncthreads();

  for (int it = 0; it < p.tpw; ++it) {
    const int tile = (rg * W) * p.tpw + wave + it * W;
    if (tile >= p.ntiles) break;
    const int row = tile * 16 + (lane & 15);
    bool row_ok;
    const uint8_t* blk[1] = {tile_blocks(it, row_ok)};
    if (it > 0) q4k_load<1>(first, blk, 0, nsb, lane >> 4);
    f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
    q4k_tile<M, 1>(acc, blk, nsb, lds, 1u, sx, lane, first);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[0][r] += __shfl_xor(acc[0][r], 32);
    const bool out_lane = (lane < 32) && row_ok;
    const int mbase = 4 * (lane >> 4);
    if (!out_lane) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (mbase + r < M) {
        if (p.S == 1)
          p.y[(size_t)(mbase + r) * p.N + row] = f32_to_bf16_bits(acc[0][r]);
        else  // this slice's sums; k_q4k_reduce adds the slices in order
          p.part[((size_t)slice * M + mbase + r) * p.N + row] = acc[0][r];
      }
    }
  }
}

// Split-K epilogue: one thread per output, slices added in slice order; the
// loads of up to 32 slices are issued before any is added (one round of load
// latency per 32 slices).
__global__ void __launch_bounds__(256) k_q4k_reduce(QgQ4kArgs p) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)p.M * p.N;
  if (idx >= total) return;
  constexpr int SC = 32;
  float t = 0.f;
  for (int s0 = 0; s0 < p.S; s0 += SC) {
    float v[SC];
#pragma unroll
    for (int j = 0; j < SC; ++j)
      if (s0 + j < p.S) v[j] = p.part[(size_t)(s0 + j) * total + idx];  // uniform across the launch
#pragma unroll
    for (int j = 0; j < SC; ++j)
      if (s0 + j < p.S) t += v[j];
  }
  p.y[idx] = f32_to_bf16_bits(t);
}

// ---------------------------------------------------------------- routing --
// All threads of the workgroup select the top_k largest logits by rank.  Each
// expert gets the 64-bit key argmax_key(logit, e) (larger logit first, then
// lower index; keys are unique), and the rank of expert e is the number of
// keys above its own, so expert e is selected iff its rank < top_k.  Results
// in LDS: sel[] / pw[] in rank order with the softmax weights over the
// selected logits, asc[] / pasc[] the same sorted by expert index.  Every
// workgroup runs the same code on the same logits and gets the same bytes.
// (NaN logits are unsupported; they still give a valid permutation.)
//
// route_load reads the logits into registers (up to four per thread, so
// E <= 4 * blockDim; other loads can be issued while they are in flight),
// route_store puts them and their keys into LDS (keys[] has two zero entries
// past E), route_rank starts with a barrier, ranks and ends with a barrier.
// When the workgroup has threads to spare, each expert's count is split over
// up to four key ranges (partial counts in LDS, added in range order).
struct RouteIn {
  float v[4];
};
constexpr int kRouteMaxThreads = 256;  // workgroup size route_rank is used with

__device__ __forceinline__ void route_load(const float* logits, int E, RouteIn& in) {
#pragma unroll
  for (int i = 0; i < 4; ++i) in.v[i] = logits[min((int)(threadIdx.x + i * blockDim.x), E - 1)];
}

__device__ __forceinline__ void route_store(const RouteIn& in, int E, float* lg, unsigned long long* keys) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + i * blockDim.x;
    if (e < E) {
      lg[e] = in.v[i];
      keys[e] = argmax_key(in.v[i], (uint32_t)e);
    }
  }
  if (threadIdx.x < 2) keys[E + threadIdx.x] = 0ull;  // below every key
}

__device__ void route_rank(int E, int top_k, const float* lg, const unsigned long long* keys, int* sel, float* pw,
                           int* asc, float* pasc) {
  __shared__ int rpart[kRouteMaxThreads];
  __syncthreads();
  const int P = min(4, max(1, (int)blockDim.x / E));  // key ranges per expert (E * P <= blockDim when P > 1)
  const int chunk = ((E + 2 * P - 1) / (2 * P)) * 2;  // even: pairs stay inside keys[0 .. E+1]
  for (int idx = threadIdx.x; idx < E * P; idx += blockDim.x) {
    const int e = idx % E, part = idx / E;
    const unsigned long long ke = keys[e];
    const int j1 = min((part + 1) * chunk, E);
    int rank = 0;
#pragma unroll 8
    for (int j = part * chunk; j < j1; j += 2) {
      const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(keys + j);
      rank += (kk.x > ke ? 1 : 0) + (kk.y > ke ? 1 : 0);
    }
    if (P == 1) {
      if (rank < top_k) sel[rank] = e;
    } else {
      rpart[idx] = rank;
    }
  }
  if (P > 1) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int rank = 0;
      for (int q = 0; q < P; ++q) rank += rpart[q * E + e];
      if (rank < top_k) sel[rank] = e;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // one wave: softmax over the selected logits, then the ascending order
    const int t = threadIdx.x;
    const float lmax = lg[sel[0]];
    const float ex = t < top_k ? expf(lg[sel[t]] - lmax) : 0.f;
    float z = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    if (t < top_k) {
      const float w = ex / z;
      pw[t] = w;
      const int e = sel[t];
      int pos = 0;  // position of expert e among the selected, by expert index
      for (int s2 = 0; s2 < top_k; ++s2) pos += (sel[s2] < e) ? 1 : 0;
      asc[pos] = e;
      pasc[pos] = w;
    }
  }
  __syncthreads();
}

// ----------------------------------------------------------- MoE gate/up --
// One workgroup per (selected expert slot, 16-row tile of I); its four waves
// split the D/256 superblocks and add their partial sums in wave order.
// Workgroup 0 also hands the routing to k_moe_down (workspace) and to the
// caller (out_ids / out_w).  h is stored in bf16, the precision k_moe_down
// consumes it in.
constexpr int kMoeWaves = 4;
static_assert(64 * kMoeWaves <= kRouteMaxThreads, "route_rank's partial counts are sized for this workgroup");

__global__ void __launch_bounds__(256) k_moe_gateup(QgMoeArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int sel[64], asc[64];
  __shared__ float pw[64], pasc[64];
  __shared__ float lg[1024];
  __shared__ __align__(16) unsigned long long keys[1026];
  __shared__ f32x4_t red[kMoeWaves][2][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int tiles = (p.I + 15) / 16;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int nsb = p.D / 256;
  uint4* lds = reinterpret_cast<uint4*>(smem);  // [0] zero entry, then the staged token
  float* sx = reinterpret_cast<float*>(lds + 1 + nsb * 32);

  RouteIn rin;
  route_load(p.logits, p.E, rin);
  if (threadIdx.x == 0) lds[0] = make_uint4(0u, 0u, 0u, 0u);
  stage_q4k_x<1, uint16_t>(p.x, (size_t)p.D, p.D, lds + 1, sx, 0, nsb, threadIdx.x, blockDim.x);
  route_store(rin, p.E, lg, keys);
  route_rank(p.E, p.top_k, lg, keys, sel, pw, asc, pasc);
  if (blockIdx.x == 0 && (int)threadIdx.x < p.top_k) {
    p.route_ids[threadIdx.x] = asc[threadIdx.x];
    p.route_w[threadIdx.x] = pasc[threadIdx.x];
    if (p.out_ids) p.out_ids[threadIdx.x] = sel[threadIdx.x];
    if (p.out_w) p.out_w[threadIdx.x] = pw[threadIdx.x];
  }

  const int e = min(max(asc[slot], 0), p.E - 1);  // always in range; clamped for memory safety
  const int row = tile * 16 + (lane & 15);
  const bool row_ok = row < p.I;
  // this wave's superblocks: [sb_lo, sb_hi)
  const int per = (nsb + kMoeWaves - 1) / kMoeWaves;
  const int sb_lo = min(nsb, wave * per), sb_hi = min(nsb, sb_lo + per);
  const size_t expert_bytes = (size_t)2 * p.I * nsb * 144;
  const uint8_t* base = p.w_gu + (size_t)e * expert_bytes;
  const int r0 = row_ok ? row : 0;
  const int sbc = min(sb_lo, nsb - 1);  // in-bounds base for a wave without superblocks
  const uint8_t* blk[2] = {base + ((size_t)r0 * nsb + sbc) * 144, base + ((size_t)(p.I + r0) * nsb + sbc) * 144};
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  if (sb_hi > sb_lo) {
    Q4kBuf<2> first;
    q4k_load<2>(first, blk, 0, sb_hi - sb_lo, lane >> 4);
    q4k_tile<1, 2>(acc, blk, sb_hi - sb_lo, lds, 1u + (uint32_t)sb_lo * 32u, sx + sb_lo * 64, lane, first);
  }
  red[wave][0][lane] = acc[0];
  red[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave == 0) {
    f32x4_t g = red[0][0][lane], u = red[0][1][lane];
    for (int w = 1; w < kMoeWaves; ++w) {
      g += red[w][0][lane];
      u += red[w][1][lane];
    }
    const float gv = g[0] + __shfl_xor(g[0], 32);  // M = 1: row 0 lives in element 0 of lanes 0..15
    const float uv = u[0] + __shfl_xor(u[0], 32);
    if (lane < 16 && row_ok) p.h[(size_t)slot * p.I + row] = f32_to_bf16_bits(gv / (1.0f + __expf(-gv)) * uv);
  }
}

// ------------------------------------------------------------- MoE down --
// One workgroup per 16-row tile of D.  Wave w handles the selected experts
// w, w+W, ... (ascending expert order, as handed over by k_moe_gateup); each
// expert's sum is scaled by its routing weight; the waves' totals are added
// in wave order.  Each wave's first weight batch is in flight while the
// experts' activations are staged.
constexpr int kMoeDownWaves = 8;
constexpr int kMoeDownBatch = 3;  // superblocks per load batch (I = 768: one batch per expert)

__global__ void __launch_bounds__(512) k_moe_down(QgMoeArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ f32x4_t red[kMoeDownWaves][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int W = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int nsb = p.I / 256;
  const size_t xs_per = (size_t)nsb * 32;  // uint4 entries per expert (M = 1)
  uint4* lds = reinterpret_cast<uint4*>(smem);  // [0] zero entry, then one staged region per expert
  float* sx = reinterpret_cast<float*>(lds + 1 + xs_per * p.top_k);

  const int row = tile * 16 + (lane & 15);
  const bool row_ok = row < p.D;
  const int r0 = row_ok ? row : 0;
  const size_t expert_bytes = (size_t)p.D * nsb * 144;
  auto expert_blocks = [&](int s) {
    const int e = min(max(p.route_ids[s], 0), p.E - 1);
    return p.w_down + (size_t)e * expert_bytes + (size_t)r0 * nsb * 144;
  };
  const int s0 = min(wave, p.top_k - 1);
  const uint8_t* blk0[1] = {expert_blocks(s0)};
  Q4kBuf<1, kMoeDownBatch> first;
  if (threadIdx.x == 0) lds[0] = make_uint4(0u, 0u, 0u, 0u);
  // the selected experts' activations, one row per expert slot.  When each
  // thread stages at most one piece, its loads go out before the first weight
  // batch (loads complete in order per wave, so staging then waits for h
  // alone, while the weights are still in flight)
  const int pieces = p.top_k * 8 * nsb;
  if (pieces <= (int)blockDim.x) {  // uniform
    const int pi = threadIdx.x;
    uint4 hv[4];
    const int reg = pi / (8 * nsb), jl = pi - reg * 8 * nsb;
    const bool live = pi < pieces;
    const uint4* src = reinterpret_cast<const uint4*>(p.h + (size_t)min(reg, p.top_k - 1) * p.I + (size_t)jl * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = src[i];
    q4k_load<1>(first, blk0, 0, nsb, lane >> 4);
    __builtin_amdgcn_sched_barrier(0);
    if (live) {
      float* rsx = sx + (size_t)reg * nsb * 64;
      stage_q4k_piece<1>(hv, lds + 1 + xs_per * reg, rsx, jl, 0);
#pragma unroll
      for (int r = 1; r < 8; ++r) rsx[jl * 8 + r] = 0.f;  // rows past M = 1, as stage_q4k_x leaves them
    }
  } else {
    q4k_load<1>(first, blk0, 0, nsb, lane >> 4);
    __builtin_amdgcn_sched_barrier(0);
    stage_q4k_x<1, uint16_t>(p.h, (size_t)p.I, p.I, lds + 1, sx, 0, nsb, threadIdx.x, blockDim.x, p.top_k);
  }
  const float pe0 = p.route_w[s0];  // used after the MFMAs
  __syncthreads();

  f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
  for (int s = wave; s < p.top_k; s += W) {
    const uint8_t* blk[1] = {expert_blocks(s)};
    if (s != wave) q4k_load<1>(first, blk, 0, nsb, lane >> 4);
    f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
    q4k_tile<1, 1>(acc, blk, nsb, lds, 1u + (uint32_t)(xs_per * s), sx + (size_t)s * nsb * 64, lane, first);
    const float pe = (s == wave) ? pe0 : p.route_w[s];
    tot[0] = fmaf(pe, acc[0][0], tot[0]);
    tot[1] = fmaf(pe, acc[0][1], tot[1]);
    tot[2] = fmaf(pe, acc[0][2], tot[2]);
    tot[3] = fmaf(pe, acc[0][3], tot[3]);
  }
  red[wave][lane] = tot;
  __syncthreads();
  if (wave == 0) {
    f32x4_t t = red[0][lane];
    for (int w = 1; w < W; ++w) t += red[w][lane];
    const float yv = t[0] + __shfl_xor(t[0], 32);
    if (lane < 16 && row_ok) p.y[row] = f32_to_bf16_bits(yv);
  }
}

template <int M>
static int launch_q4k_m(const QgQ4kArgs& a, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_q4k<M>), dim3((unsigned)(a.S * a.rgroups)), dim3((unsigned)(64 * a.waves)), lds, st, a);
  int err = (int)hipGetLastError();
  if (err || a.S == 1) return err;
  hipLaunchKernelGGL(k_q4k_reduce, dim3((unsigned)(((size_t)a.M * a.N + 255) / 256)), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace qg

int qg_launch_q4k_reduce(const QgQ4kArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(qg::k_q4k_reduce, dim3((unsigned)(((size_t)a.M * a.N + 255) / 256)), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

int qg_launch_q4k(const QgQ4kArgs& a, size_t lds, hipStream_t st) {
  switch (a.M) {
    case 1: return qg::launch_q4k_m<1>(a, lds, st);
    case 2: return qg::launch_q4k_m<2>(a, lds, st);
    case 3: return qg::launch_q4k_m<3>(a, lds, st);
    case 4: return qg::launch_q4k_m<4>(a, lds, st);
    case 5: return qg::launch_q4k_m<5>(a, lds, st);
    case 6: return qg::launch_q4k_m<6>(a, lds, st);
    case 7: return qg::launch_q4k_m<7>(a, lds, st);
    case 8: return qg::launch_q4k_m<8>(a, lds, st);
    default: return (int)hipErrorInvalidValue;
  }
}

int qg_launch_moe(const QgMoeArgs& a, hipStream_t st) {
  const int nsb_d = a.D / 256, nsb_i = a.I / 256;
  const size_t lds_gu = 16 + (size_t)nsb_d * 32 * 16 + (size_t)nsb_d * 64 * 4;
  const int tiles_i = (a.I + 15) / 16;
  hipLaunchKernelGGL(qg::k_moe_gateup, dim3((unsigned)(a.top_k * tiles_i)), dim3(64 * qg::kMoeWaves), lds_gu, st,
                     a);
  int err = (int)hipGetLastError();
  if (err) return err;
  const size_t lds_dn = 16 + (size_t)a.top_k * ((size_t)nsb_i * 32 * 16 + (size_t)nsb_i * 64 * 4);
  const int waves = a.top_k < qg::kMoeDownWaves ? a.top_k : qg::kMoeDownWaves;
  hipLaunchKernelGGL(qg::k_moe_down, dim3((unsigned)((a.D + 15) / 16)), dim3(64 * waves), lds_dn, st, a);
  return (int)hipGetLastError();
}
