/*
 * oracle.h -- plain fp64 CPU reference for the 4-bit quantized decode projections.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or constant with the GPU library: it has its own bf16 /
 * fp16 decoders, its own nibble and 6-bit-field unpackers and its own loops.
 *
 * Every function computes the plain definition of one step of the decode
 * projection, in double precision, in ascending index order:
 *   O0  bf16 / fp16 bit patterns -> exact doubles
 *   O1  MLX-style affine 4-bit dequantisation, group 64
 *   O2  GGUF Q4_K superblock dequantisation (256 weights, 8 sub-blocks of 32)
 *   O3  Y[m][n] = sum_k X[m][k] * W[n][k]
 *   O4  RMSNorm
 *   O5  SiLU / SwiGLU
 *   O6  RMSNorm -> gate+up -> SwiGLU (-> down)
 *   O7  MoE: top-k routing, softmax over the selected logits, weighted sum of
 *       the selected experts' SwiGLU MLPs
 *   O8  LM-head readout, greedy argmax, accepted draft prefix
 *   O9  LM-head top-k readout (candidate pools)
 *   O10 input randomised Hadamard transform (blockwise, Sylvester order)
 *   O11 affine-4 projection of the transformed input
 *   O12 MLX-style affine 8-bit dequantisation, group 64
 *   O13 Y = X . W^T on affine-8 weights
 *   O14 GGUF Q6_K superblock dequantisation (256 weights, 16 int8 scales)
 *   O15 Y = X . W^T on Q6_K weights
 *
 * Sources (the four pages the method is taken from):
 *   [uzu]        "trymirai/uzu ... deep dive" (blog.123qwe.co.kr), section
 *                "내부 동작 1: 모델은 설정으로 조립된다" -- weight_matrix row names MLX 4/8-bit
 *                quantized weights; linear row names the untied readout; mlp row
 *                names dense and routed-expert MLPs.
 *   [runNburn]   "runNburn 로컬 LLM 추론 엔진을 만든 이유" (coderred.com), sections
 *                "GGUF를 그대로 진실의 원본으로 둡니다" (GGUF Q4_K_M consumed as stored)
 *                and "하드웨어가 달라도 모델 의미는 바꾸지 않습니다" (routing and
 *                quantisation semantics are never altered).
 *   [TensorFold] "ashhart/TensorFold 1.2.7 ... deep dive" (blog.123qwe.co.kr),
 *                section "핵심 메커니즘 3 — 커널 계약" (a float64 reference per kernel)
 *                and the box-measurement table (4-bit, group 64).
 *   [Husky]      "Husky - MLX보다 최대 4.5배 빠른 추론 엔진" (molayo1419.me), section
 *                "MSI의 네 가지 구현 요소" (norm fused into the projection, gate and up
 *                computed together, 4-bit unpack) and "8행 투영 커널 개선" (8-row
 *                verify projection).
 * The pages do not define the bit layouts; the readings used here are listed
 * at each function (affine4: low nibble first, 8 codes per little-endian
 * 32-bit word; Q4_K: the public GGUF 144-byte block).
 *
 * Conventions: all arrays are row-major; bf16 and fp16 values are passed as
 * their 16-bit patterns; every function returns 0 on success and -1 on a bad
 * argument (nothing is written then).
 */
#ifndef QG_ORACLE_H
#define QG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* O0: exact decoders and the round-to-nearest-even encoder used by tests. */
/* Threads of the all-cores build (liboracle_mt.so) for the calls that follow;
 * returns the count in effect (always 1 in the single-threaded build). */
int oracle_set_threads(int n);

double o_bf16_to_f64(uint16_t h);
double o_f16_to_f64(uint16_t h);
uint16_t o_f64_to_bf16_rne(double v);

/* O1: rows [n0, n0+nr) of an affine-4 matrix W[N][K] -> w[nr][K].
 * codes: uint32 [N][K/8], scales/biases: bf16 [N][K/64]. K % 64 == 0. */
int oracle_dequant_affine4(const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, int64_t N, int64_t K,
                           int64_t n0, int64_t nr, double* w);

/* O2: rows [n0, n0+nr) of a Q4_K matrix (blocks: [N][K/256][144] bytes). */
int oracle_dequant_q4k(const uint8_t* blocks, int64_t N, int64_t K,
                       int64_t n0, int64_t nr, double* w);

/* O3 on quantised weights; x is bf16 [M][K], y is fp64 [M][N]. */
int oracle_qgemv_affine4(const uint16_t* x, const uint32_t* codes,
                         const uint16_t* scales, const uint16_t* biases,
                         int M, int64_t N, int64_t K, double* y);
int oracle_qgemv_q4k(const uint16_t* x, const uint8_t* blocks, int M,
                     int64_t N, int64_t K, double* y);
/* O3 with an fp64 activation (used where the activation is itself an oracle
 * intermediate, e.g. the SwiGLU output feeding the down projection). */
int oracle_qgemv_affine4_f64x(const double* x, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* biases,
                              int M, int64_t N, int64_t K, double* y);

/* O4: xn[m][k] = x[m][k] * gamma[k] / sqrt(mean_k x[m][k]^2 + eps). */
int oracle_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps, int M,
                   int64_t K, double* xn);

/* O5 */
double oracle_silu(double g);

/* O4 + O3 + O5: h[m][i] = silu(g) * u with g = row i and u = row I+i of the
 * fused gate/up matrix [2I][K] applied to rmsnorm(x). */
int oracle_rmsnorm_gateup_swiglu(const uint16_t* x, const uint16_t* gamma,
                                 double eps, const uint32_t* codes_gu,
                                 const uint16_t* scales_gu,
                                 const uint16_t* biases_gu, int M, int64_t I,
                                 int64_t K, double* h);

/* O6: y = Down . swiglu(GU . rmsnorm(x)); down matrix is [D][I] with D = K. */
int oracle_mlp_block(const uint16_t* x, const uint16_t* gamma, double eps,
                     const uint32_t* codes_gu, const uint16_t* scales_gu,
                     const uint16_t* biases_gu, const uint32_t* codes_d,
                     const uint16_t* scales_d, const uint16_t* biases_d, int M,
                     int64_t I, int64_t K, double* y);

/* O7: one token x bf16 [D]; logits fp32 [E]; experts stored as Q4_K:
 *   w_gu   [E][2I][D/256][144]  (rows 0..I-1 gate, I..2I-1 up)
 *   w_down [E][D][I/256][144]
 * Outputs y fp64 [D], ids int32 [top_k] (descending logit, ties -> lower
 * index), p fp64 [top_k] (softmax over the selected logits). */
int oracle_moe(const uint16_t* x, const float* logits, int top_k,
               const uint8_t* w_gu, const uint8_t* w_down, int E, int64_t D,
               int64_t I, double* y, int32_t* ids, double* p);

/* O8: logits[m][v] (nullable) = x[m] . w[v]; ids[m] = lowest index of the
 * maximum (a NaN counts as the maximum, first NaN wins); gap[m] (nullable) =
 * max - second largest logit of row m; accepted (nullable) = number of
 * leading rows whose id equals draft[row] (draft nullable -> 0). */
int oracle_lmhead(const uint16_t* x, const uint32_t* codes,
                  const uint16_t* scales, const uint16_t* biases, int M,
                  int64_t V, int64_t K, double* logits, int32_t* ids,
                  double* gap, const int32_t* draft, int32_t* accepted);

/* O9: top-k readout (uzu page, "내부 동작 3: DFlash + Weaver 트리형 투기
 * 디코딩": every preview row yields a candidate pool of its top tokens).
 * For each row m, ids[m][0..k-1] are the indices of the k largest logits
 * x[m] . w[v] in order: larger logit first, equal logits by lower index, a
 * NaN logit above every number (NaNs by lower index).  vals[m][j]
 * (nullable) is the logit of ids[m][j].  1 <= k <= V. */
int oracle_lmhead_topk(const uint16_t* x, const uint32_t* codes,
                       const uint16_t* scales, const uint16_t* biases, int M,
                       int64_t V, int64_t K, int k, int32_t* ids,
                       double* vals);

/* O10: input randomised Hadamard transform (uzu page, section "내부 동작 1",
 * linear row: an input-side random Hadamard transform that spreads the
 * quantisation error; the Metal kernel list names a hadamard_transform).
 * For each row m and each block b of `had` consecutive k (had a power of two
 * dividing K):
 *   xr[m][b*had + i] = (1/sqrt(had)) * sum_j H[i][j] * s[b*had + j] * x[m][b*had + j]
 * with H[i][j] = (-1)^popcount(i & j) (Sylvester order) and s[k] = -1 where
 * signs[k] < 0, else +1.  x is bf16 [M][K]; xr fp64 [M][K]. */
int oracle_rht(const uint16_t* x, const int8_t* signs, int had, int M,
               int64_t K, double* xr);

/* O11: y = dequant(W) . RHT(x) (O10 then O3 on the fp64 transformed rows). */
int oracle_qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had,
                             const uint32_t* codes, const uint16_t* scales,
                             const uint16_t* biases, int M, int64_t N,
                             int64_t K, double* y);

/* O12: rows [n0, n0+nr) of an affine-8 matrix W[N][K] -> w[nr][K].
 * codes: uint32 [N][K/4] (code k in byte k%4 of word k/4, least significant
 * byte first), scales/biases: bf16 [N][K/64]. K % 64 == 0. */
int oracle_dequant_affine8(const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, int64_t N, int64_t K,
                           int64_t n0, int64_t nr, double* w);

/* O13: O3 on affine-8 weights; x bf16 [M][K], y fp64 [M][N]. */
int oracle_qgemv_affine8(const uint16_t* x, const uint32_t* codes,
                         const uint16_t* scales, const uint16_t* biases,
                         int M, int64_t N, int64_t K, double* y);

/* O14: rows [n0, n0+nr) of a Q6_K matrix (blocks: [N][K/256][210] bytes:
 * ql 128, qh 64, int8 scales 16, fp16 d). K % 256 == 0. */
int oracle_dequant_q6k(const uint8_t* blocks, int64_t N, int64_t K, int64_t n0,
                       int64_t nr, double* w);

/* O15: O3 on Q6_K weights; x bf16 [M][K], y fp64 [M][N]. */
int oracle_qgemv_q6k(const uint16_t* x, const uint8_t* blocks, int M, int64_t N,
                     int64_t K, double* y);

#ifdef __cplusplus
}
#endif
#endif
