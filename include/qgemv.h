/*
 * qgemv.h -- C ABI of libqgemv.so: 4-bit quantized decode projections on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the weight projection of one LLM decode step,
 *     Y[M][N] = X[M][K] . dequant(W)[N][K]^T,
 * with M = 1 for a plain decode step and M <= 8 for a speculative verify block
 * that scores the current token and up to seven drafted tokens in one read of
 * the weights (Husky page "Husky - MLX보다 최대 4.5배 빠른 추론 엔진", sections
 * "일반 글쓰기의 한계와 편집 가속 원리" (an 8-token block verified per step) and
 * "8행 투영 커널 개선..." (the 8-row projection kernel)).
 *
 * Weight formats
 *   affine4  MLX-style 4-bit weights with one bf16 scale and one bf16 bias per
 *            group of 64 consecutive weights along K (uzu deep-dive page,
 *            section "내부 동작 1", weight_matrix row: MLX 4/8-bit; TensorFold
 *            deep-dive page, box-measurement table: "4-bit group 64").
 *            codes  : uint32 [N][K/8]; code of weight k of row n is bits
 *                     4*(k%8) .. 4*(k%8)+3 of word k/8 (low nibble first).
 *            scales : bf16 [N][K/64];  biases : bf16 [N][K/64].
 *            w[n][k] = scale[n][k/64] * code + bias[n][k/64].
 *   q4k      GGUF Q4_K superblocks, consumed as stored (runNburn page, section
 *            "GGUF를 그대로 진실의 원본으로 둡니다").  blocks: uint8 [N][K/256][144]:
 *            fp16 d, fp16 dmin, 12 bytes of eight 6-bit scales sc_j and eight
 *            6-bit mins m_j, then 128 bytes of codes; weight o of a block is in
 *            sub-block j = o/32 and equals d*sc_j*q - dmin*m_j.  The byte layout
 *            is the public GGUF one (the pages only name the format).
 *
 * Common conventions
 *   * bf16 and fp16 values are passed as uint16_t bit patterns.
 *   * Every pointer is caller-owned device memory (hipMalloc / torch CUDA
 *     tensors), except the workspace, which is also caller-owned device
 *     memory (see below).  X, codes and Q4_K blocks must be 16-byte aligned; float and
 *     int32 buffers 4-byte aligned; other bf16 buffers 2-byte aligned.
 *   * `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work and return; results are ready when the stream is synchronised.
 *   * Every argument is checked before anything is launched; a call that fails
 *     its checks writes nothing (the refuse-before-touching-weights and
 *     explicit-error conventions of the TensorFold and runNburn pages).
 *     Outputs may not overlap any input or each other (QG_EALIAS).
 *   * Workspace.  Entry points that need device scratch (split-K partial
 *     sums, per-workgroup argmax keys, top-k candidates, the RHT's transformed
 *     rows, MoE routing and expert activations, a grid barrier's counters)
 *     take it from the caller as (ws, ws_bytes): the library never allocates,
 *     frees or synchronises on a call.  <entry>_workspace(...) returns the
 *     bytes a call of that shape needs (host-only, no GPU access); 0 means
 *     none, and ws may then be NULL.  The size is the same on every gfx950
 *     device.  ws must be 256-byte aligned, at least that large, and may not
 *     overlap any input or output (QG_EALIAS).  A workspace must be zeroed
 *     once (e.g. hipMemset) before its first use: its first
 *     qg_workspace_header_bytes() bytes hold state that some entry points
 *     need to find at zero and always leave at zero, so one workspace can
 *     serve every entry point and every shape, one call at a time.  The
 *     contents carry no results between calls.  Calls that may run at the
 *     same time (different streams, or graphs replayed concurrently) need
 *     different workspaces.  With that, calls are stateless: any number of
 *     host threads may issue calls, and the calls can be captured into a HIP
 *     graph on any stream, also as the stream's first work.
 *   * A call may enqueue more than one kernel (a split-K reduction follows
 *     its main kernel on the same stream).
 *   * Floating point: fp32 accumulation; bf16 outputs rounded to nearest even.
 *     Results are deterministic: the same inputs give the same bytes on every
 *     call (fixed reduction order, no atomics).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qg_status;
#define QG_OK 0
#define QG_EINVAL (-1)        /* bad shape, null pointer or misalignment        */
#define QG_EALIAS (-2)        /* an output overlaps an input or another output  */
#define QG_EUNSUPPORTED (-3)  /* valid request with no kernel instance          */
#define QG_EHIP (-4)          /* HIP runtime or launch error                    */

/* Static description of a status code. */
const char* qg_status_string(qg_status status);
/* Detail of the most recent failure on the calling thread ("" if none). */
const char* qg_last_error(void);
/* Bytes at the start of every workspace that hold zero-initialised state. */
size_t qg_workspace_header_bytes(void);

/*
 * qgemv_affine4 -- Y = X . dequant(W)^T for affine4 weights.
 *   x      bf16 [M][K]           activations
 *   codes  uint32 [N][K/8]; scales, biases bf16 [N][K/64]
 *   y      bf16 [M][N]           output
 *   1 <= M <= 8; N >= 0 (N = 0 does nothing); K > 0, K % 64 == 0.
 *   ws: split-K partial sums when K is long enough to be split:
 *   qgemv_affine4_workspace(M, N, K) bytes (0 when it is not split).
 */
qg_status qgemv_affine4(const uint16_t* x, const uint32_t* codes,
                        const uint16_t* scales, const uint16_t* biases,
                        uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes,
                        void* stream);
size_t qgemv_affine4_workspace(int M, int N, int K);

/*
 * qgemv_affine4_rht -- the projection of an input-side randomised Hadamard
 * transform (uzu page, section "내부 동작 1", linear row: an input-side random
 * Hadamard transform spreads the quantisation error; the weights were
 * quantised in the rotated basis):
 *   xr[m][b*had + i] = (1/sqrt(had)) sum_j H[i][j] s[b*had + j] x[m][b*had + j]
 *   Y = xr . dequant(W)^T
 *   H[i][j] = (-1)^popcount(i & j) (Sylvester order); s[k] = -1 where
 *   signs[k] < 0, else +1 (the random signs are an input).
 *   x bf16 [M][K]; signs int8 [K]; codes uint32 [N][K/8]; scales, biases
 *   bf16 [N][K/64]; y bf16 [M][N].  had: a power of two, 2 <= had <= 4096,
 *   dividing K; other shape rules as qgemv_affine4.  The transform runs in
 *   fp32 and reaches the projection as two bf16 planes (16 significant bits).
 *   A call enqueues the transform and the projection (and a split-K reduce).
 */
qg_status qgemv_affine4_rht(const uint16_t* x, const int8_t* signs, int had,
                            const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* biases, uint16_t* y, int M, int N,
                            int K, void* ws, size_t ws_bytes,
                            void* stream);
size_t qgemv_affine4_rht_workspace(int M, int N, int K);

/*
 * qgemv_affine8 -- Y = X . dequant8(W)^T for MLX-style affine 8-bit weights
 * (uzu page, section "내부 동작 1: 모델은 설정으로 조립된다": the weight_matrix
 * row names MLX 4- and 8-bit quantized weights).  Code k of row n is byte k%4
 * (least significant first) of codes[n][k/4], an unsigned value 0..255; the
 * weight is scale * code + bias with the bf16 scale and bias of group k/64.
 *   x      bf16 [M][K]
 *   codes  uint32 [N][K/4] (16-byte aligned); scales, biases bf16 [N][K/64]
 *   y      bf16 [M][N]
 *   1 <= M <= 8; N >= 0 (N = 0 does nothing); K > 0, K % 64 == 0.
 *   Errors as qgemv_affine4.
 */
qg_status qgemv_affine8(const uint16_t* x, const uint32_t* codes,
                        const uint16_t* scales, const uint16_t* biases,
                        uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes,
                        void* stream);
size_t qgemv_affine8_workspace(int M, int N, int K);

/*
 * mlp_block_affine4_tiled -- the whole MLP block in one persistent launch
 * (Husky page, section "MSI의 네 가지 구현 요소": one dispatch per layer MLP,
 * useful when one projection's weight reads overlap the tail of the previous):
 *   h = silu(xn . Wg^T) * (xn . Wu^T), xn = RMSNorm(x)  (as rmsnorm_gateup_swiglu)
 *   y = h . Wd^T                                          (as qgemv_affine4)
 *   x       bf16 [M][D]; gamma bf16 [D]; eps > 0
 *   gu_codes_t, gu_sb_t  tile-order copy of the [2I][D] gate-then-up matrix
 *   dn_codes_t, dn_sb_t  tile-order copy of the [D][I] down matrix
 *   h       bf16 [M][I] output (16-byte aligned); y bf16 [M][D] output
 *   1 <= M <= 8; D % 512 == 0; I % 512 == 0.
 * h and y are bit-identical to rmsnorm_gateup_swiglu_tiled followed by
 * qgemv_affine4_tiled (same K splits, same summation order).  The launch is
 * cooperative (the runtime refuses it, QG_EHIP, rather than start more
 * workgroups than can be resident at once); it keeps one workgroup per
 * resident slot and separates its phases (gate/up, h, down, y) with grid
 * barriers whose counters live in the workspace header (zero when the call
 * starts; the last workgroup to leave sets them back to zero).  Waits are
 * bounded: should one give up, the call still ends, h and y are filled with
 * NaN, and mlp_block_affine4_tiled_failures counts the call; the workspace is
 * reusable as it is.  The workspace also holds the split-K partial sums.
 */
qg_status mlp_block_affine4_tiled(const uint16_t* x, const uint16_t* gamma,
                                  float eps, const uint32_t* gu_codes_t,
                                  const uint16_t* gu_sb_t,
                                  const uint32_t* dn_codes_t,
                                  const uint16_t* dn_sb_t, uint16_t* h,
                                  uint16_t* y, int M, int D, int I,
                                  void* ws, size_t ws_bytes,
                                  void* stream);
size_t mlp_block_affine4_tiled_workspace(int M, int D, int I);
/*
 * mlp_stack_affine4_tiled -- L MLP blocks in a row in one persistent launch,
 * layer l's output being layer l + 1's input (Husky page, section "전체 단계
 * 메가커널의 실험과 다음 과제": one dispatch for several layers pays off when
 * the weight reads of the next layer overlap the tail of the previous one):
 *   x_0 = x;  x_{l+1} = y_l = MLP_l(x_l) (as mlp_block_affine4_tiled)
 *   x       bf16 [M][D]; gamma bf16 [L][D]; eps > 0
 *   gu_codes_t, gu_sb_t  L stacked tile-order copies of the [2I][D]
 *                        gate-then-up matrices (qg_tiled_bytes(2I, D) and its
 *                        sb_bytes per layer)
 *   dn_codes_t, dn_sb_t  L stacked tile-order copies of the [D][I] down matrices
 *   h       bf16 [M][I] (16-byte aligned): the last layer's SwiGLU output
 *   ys      bf16 [L][M][D]: every layer's output (ys[L-1] is the stack's)
 *   1 <= L <= 4096; other rules as mlp_block_affine4_tiled, whose results each
 *   layer reproduces bit for bit.  Before the barrier that precedes a layer's
 *   gate/up phase, every workgroup issues the loads of its first gate/up
 *   weights (they do not depend on the previous layer's output).
 *   ws: mlp_stack_affine4_tiled_workspace(M, D, I) bytes (the same as one block).
 */
qg_status mlp_stack_affine4_tiled(const uint16_t* x, const uint16_t* gamma,
                                  float eps, const uint32_t* gu_codes_t,
                                  const uint16_t* gu_sb_t,
                                  const uint32_t* dn_codes_t,
                                  const uint16_t* dn_sb_t, uint16_t* h,
                                  uint16_t* ys, int L, int M, int D, int I,
                                  void* ws, size_t ws_bytes, void* stream);
size_t mlp_stack_affine4_tiled_workspace(int M, int D, int I);
qg_status qg_check_mlp_stack_affine4_tiled(
    const uint16_t* x, const uint16_t* gamma, float eps,
    const uint32_t* gu_codes_t, const uint16_t* gu_sb_t,
    const uint32_t* dn_codes_t, const uint16_t* dn_sb_t, uint16_t* h,
    uint16_t* ys, int L, int M, int D, int I, const void* ws, size_t ws_bytes);

/* Diagnostic, not for the decode path: synchronises `stream`, returns how many
 * mlp_block_affine4_tiled calls on workspace `ws` had a barrier wait give up
 * since the last query (0: none; -1: HIP error) and resets that count. */
int32_t mlp_block_affine4_tiled_failures(void* ws, void* stream);

/*
 * qgemv_q6k -- Y = X . dequant(W)^T for GGUF Q6_K weights as stored (runNburn
 * page, section "GGUF를 그대로 진실의 원본으로 둡니다": Q4_K_M files mix Q6_K
 * in).  Reading of the public 210-byte block of 256 weights: bytes 0..127 ql
 * (low 4 bits), 128..191 qh (high 2 bits), 192..207 sixteen int8 scales (one
 * per 16 weights), 208..209 fp16 d; weight o (h = o/128, j = (o%128)/32,
 * l = o%32) has low bits = low (j < 2) or high nibble of ql[64h + 32(j%2) + l],
 * high bits = bits 2j..2j+1 of qh[32h + l], q = (low | high << 4) - 32, and
 * value d * sc[o/16] * q.
 *   x      bf16 [M][K] (16-byte aligned)
 *   blocks uint8 [N][K/256][210] (2-byte aligned)
 *   y      bf16 [M][N]
 *   1 <= M <= 8; N >= 0 (N = 0 does nothing); K > 0, K % 256 == 0.
 */
qg_status qgemv_q6k(const uint16_t* x, const uint8_t* blocks, uint16_t* y,
                    int M, int N, int K, void* ws, size_t ws_bytes,
                    void* stream);
size_t qgemv_q6k_workspace(int M, int N, int K);

/*
 * Tile-order layout of affine4 weights (Husky page, section "MSI의 네 가지 구현
 * 요소": weights stored in the order the projection kernel reads them), for
 * K % 512 == 0.  With T = ceil(N/16) 16-row tiles, C = K/128 chunks, B = K/512
 * batches and G = K/64 groups:
 *   codes_t uint32 [T][C][64][4]:
 *     codes_t[t][c][16*kb + n][w] = codes[16t + n][16c + 4kb + w]
 *   sb_t bf16 [T][B][2][16][4][2]:
 *     sb_t[t][b][h][n][u][0] = scales[16t + n][8b + 2u + h],
 *     sb_t[t][b][h][n][u][1] = biases[16t + n][8b + 2u + h]
 * (kb = 0..3, n = 0..15, w = 0..3, h = 0..1, u = 0..3; rows past N are zero:
 * the (scale, bias) pairs of the even, then the odd groups).  The same
 * bytes as the canonical layout, reordered so that every load of a wave
 * reads consecutive memory.  The tiled entry points compute exactly what
 * their canonical twins compute, in the same order (bit-identical results).
 *
 * qg_tiled_bytes -- bytes of codes_t for [N][K] (0 if K % 512 != 0 or N < 1);
 *   *sb_bytes (nullable) receives the bytes of sb_t.
 * affine4_tile_pack -- writes codes_t and sb_t from the canonical arrays
 *   (device memory, 16-byte aligned outputs); N >= 1, K % 512 == 0.
 * qgemv_affine4_tiled -- qgemv_affine4 on tile-order weights.
 * lmhead_argmax_tiled -- lmhead_argmax on tile-order weights.
 * rmsnorm_gateup_swiglu_tiled -- rmsnorm_gateup_swiglu with codes_t / sb_t the
 *   tile-order copy of the whole [2I][K] gate-then-up matrix (N = 2I).
 */
size_t qg_tiled_bytes(int N, int K, size_t* sb_bytes);
qg_status affine4_tile_pack(const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* biases, uint32_t* codes_t,
                            uint16_t* sb_t, int N, int K, void* stream);
qg_status qgemv_affine4_tiled(const uint16_t* x, const uint32_t* codes_t,
                              const uint16_t* sb_t, uint16_t* y, int M, int N,
                              int K, void* ws, size_t ws_bytes,
                              void* stream);
size_t qgemv_affine4_tiled_workspace(int M, int N, int K);
qg_status lmhead_argmax_tiled(const uint16_t* x, const uint32_t* codes_t,
                              const uint16_t* sb_t, float* logits,
                              int32_t* ids, const int32_t* draft,
                              int32_t* accepted, int M, int V, int K,
                              void* ws, size_t ws_bytes,
                              void* stream);
size_t lmhead_argmax_tiled_workspace(int M, int V, int K);
qg_status rmsnorm_gateup_swiglu_tiled(const uint16_t* x, const uint16_t* gamma,
                                      float eps, const uint32_t* codes_t,
                                      const uint16_t* sb_t, uint16_t* h, int M,
                                      int I, int K, void* ws, size_t ws_bytes,
                                      void* stream);
size_t rmsnorm_gateup_swiglu_tiled_workspace(int M, int I, int K);

/*
 * qgemv_q4k -- Y = X . dequant(W)^T for Q4_K weights.
 *   x bf16 [M][K]; blocks uint8 [N][K/256][144]; y bf16 [M][N].
 *   1 <= M <= 8; N >= 0; K > 0, K % 256 == 0.
 */
qg_status qgemv_q4k(const uint16_t* x, const uint8_t* blocks, uint16_t* y,
                    int M, int N, int K, void* ws, size_t ws_bytes,
                    void* stream);
size_t qgemv_q4k_workspace(int M, int N, int K);

/*
 * rmsnorm_gateup_swiglu -- the front half of a dense SwiGLU MLP with the norm
 * fused into the projection and gate and up computed together (Husky page,
 * section "MSI의 네 가지 구현 요소"):
 *   xn[m][k] = x[m][k] * gamma[k] / sqrt(mean_k x[m][k]^2 + eps)
 *   g = xn . Wg^T, u = xn . Wu^T, h[m][i] = silu(g[m][i]) * u[m][i]
 *   x bf16 [M][K]; gamma bf16 [K]; eps > 0 (finite)
 *   codes_gu uint32 [2I][K/8], scales_gu / biases_gu bf16 [2I][K/64]:
 *     rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
 *   h bf16 [M][I].   1 <= M <= 8; I >= 0; K > 0, K % 64 == 0.
 */
qg_status rmsnorm_gateup_swiglu(const uint16_t* x, const uint16_t* gamma,
                                float eps, const uint32_t* codes_gu,
                                const uint16_t* scales_gu,
                                const uint16_t* biases_gu, uint16_t* h, int M,
                                int I, int K, void* ws, size_t ws_bytes,
                                void* stream);
size_t rmsnorm_gateup_swiglu_workspace(int M, int I, int K);

/*
 * moe_expert_qgemv -- one decode token through a routed-expert SwiGLU MLP
 * stored in Q4_K (uzu page: MixtureOfExperts with a routing function; runNburn
 * page: routing and quantisation semantics are never altered):
 *   S = the top_k largest router logits (ties -> lower expert index),
 *   p_e = softmax over the selected logits only,
 *   y = sum_{e in S} p_e * Down_e . swiglu(GU_e . x), summed in ascending e.
 *   x bf16 [D]; router_logits fp32 [E];
 *   w_gu   uint8 [E][2I][D/256][144]  (rows 0..I-1 gate, I..2I-1 up)
 *   w_down uint8 [E][D][I/256][144]
 *   y bf16 [D]; out_ids int32 [top_k] (nullable; selected experts, largest
 *   logit first); out_w fp32 [top_k] (nullable; their weights, same order).
 *   1 <= top_k <= E <= 1024, top_k <= 64; D, I > 0 and multiples of 256.
 *   NaN router logits are not supported.
 *   ws: the routing (selected experts and weights) and the expert
 *   activations h [top_k][I] (bf16) pass from the gate/up kernel to the down
 *   kernel through it: moe_expert_qgemv_workspace(top_k, E, D, I) bytes.
 */
qg_status moe_expert_qgemv(const uint16_t* x, const float* router_logits,
                           int top_k, const uint8_t* w_gu,
                           const uint8_t* w_down, uint16_t* y,
                           int32_t* out_ids, float* out_w, int E, int D, int I,
                           void* ws, size_t ws_bytes,
                           void* stream);
size_t moe_expert_qgemv_workspace(int top_k, int E, int D, int I);

/*
 * lmhead_argmax -- untied LM-head readout with greedy verify (uzu page,
 * linear row: untied_readout; DFlash + Weaver section: the target scores the
 * proposal and keeps the longest accepted path; Husky page: the next token is
 * handed over on the GPU):
 *   logits[m][v] = x[m] . dequant(W)[v]      (fp32; stored only if non-null)
 *   ids[m]       = lowest v with the largest logit (a NaN logit counts as the
 *                  largest; the first NaN wins)
 *   accepted     = number of leading rows m with ids[m] == draft[m]
 *                  (written only if non-null; 0 if draft is null)
 *   x bf16 [M][K]; codes uint32 [V][K/8]; scales, biases bf16 [V][K/64];
 *   logits fp32 [M][V] (nullable); ids int32 [M]; draft int32 [M] (nullable);
 *   accepted int32 [1] (nullable).   1 <= M <= 8; V >= 1; K % 64 == 0;
 *   K <= 262144 (else QG_EUNSUPPORTED).
 *   ws (lmhead_argmax_workspace(M, V, K) bytes): when all of x fits on chip,
 *   ceil(K/128) * (264*M + 64) + 1024*M + 256 <= 163840 bytes (M = 8:
 *   K <= 9088; M = 1: K <= 63360), the header only: every workgroup merges
 *   its best (logit, index) of each row into a running maximum there, and
 *   the last one to finish writes ids and accepted and sets the maximum back
 *   to zero -- one kernel per call.  Beyond that K is split into the fewest
 *   slices that fit, each slice's fp32 partial sums [S][M][V] go to the
 *   workspace after the header, and a second kernel adds them in slice order
 *   and then merges and finishes as above (the summation order then differs
 *   from a call with fewer rows whose x still fits in one slice).
 */
qg_status lmhead_argmax(const uint16_t* x, const uint32_t* codes,
                        const uint16_t* scales, const uint16_t* biases,
                        float* logits, int32_t* ids, const int32_t* draft,
                        int32_t* accepted, int M, int V, int K, void* ws, size_t ws_bytes,
                        void* stream);
size_t lmhead_argmax_workspace(int M, int V, int K);

/*
 * lmhead_argmax_static -- lmhead_argmax for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, checks, kernel and results, minus the
 * workspace.  Its scratch (the 16 KB workspace header: the running maxima and
 * the arrival counter) is a static device array of the library, one per GPU,
 * holding at most 16384 bytes (larger needs are refused with
 * QG_EUNSUPPORTED); the call allocates nothing.  The array is zero when the
 * library is loaded and every call leaves it at zero.  All calls on one GPU
 * share it: calls that may overlap in time on one GPU (different streams,
 * graphs replayed concurrently) race on it and give undefined ids.
 */
qg_status lmhead_argmax_static(const uint16_t* x, const uint32_t* codes,
                               const uint16_t* scales, const uint16_t* biases,
                               float* logits, int32_t* ids, const int32_t* draft,
                               int32_t* accepted, int M, int V, int K,
                               void* stream);

/*
 * lmhead_topk -- top-k readout of the untied LM head (uzu page, section
 * "내부 동작 3: DFlash + Weaver": the target's readout of each draft position
 * yields a pool of its best candidate tokens):
 *   logits[m][v] = x[m] . dequant(W)[v]           (fp32)
 *   ids[m][0..k-1] = indices of the k largest logits of row m, larger logit
 *                    first, equal logits by lower index, a NaN logit above
 *                    every number (NaNs by lower index)
 *   vals[m][j]     = logits[m][ids[m][j]]           (written only if non-null)
 *   x bf16 [M][K]; codes uint32 [V][K/8]; scales, biases bf16 [V][K/64];
 *   logits fp32 [M][V] (nullable: if null they are kept in the workspace,
 *   which then needs 4*M*V more bytes: pass logits_kept = 0 to the size
 *   query); ids int32 [M][k]; vals fp32 [M][k] (nullable).
 *   1 <= M <= 8; 1 <= k <= min(64, V); K as for lmhead_argmax.
 *   A call enqueues two kernels: the projection, which stores the logits and
 *   each of its workgroups' largest logit per row, and a selection kernel,
 *   one workgroup per row.  (With K split as for lmhead_argmax, a third
 *   kernel between them adds the slices' partial sums, stores the logits and
 *   forms the same per-workgroup maxima over the same tiles.)  The k-th largest of those maxima bounds the
 *   row's k-th largest logit from below, so only the k workgroups ranked
 *   first can hold the top k; the selection reads their logits alone and
 *   sorts the ones at or above the bound.  vals come from the selection
 *   keys: a -0 logit is returned as +0, a NaN as a quiet NaN.
 */
qg_status lmhead_topk(const uint16_t* x, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases,
                      float* logits, int32_t* ids, float* vals, int M, int V,
                      int K, int k, void* ws, size_t ws_bytes,
                      void* stream);
size_t lmhead_topk_workspace(int M, int V, int K, int k, int logits_kept);

/*
 * lmhead_topk_tiled -- lmhead_topk on the tile-order copy of W (codes_t, sb_t
 * from affine4_tile_pack, K % 512 == 0); the same results.
 */
qg_status lmhead_topk_tiled(const uint16_t* x, const uint32_t* codes_t,
                            const uint16_t* sb_t, float* logits, int32_t* ids,
                            float* vals, int M, int V, int K, int k, void* ws,
                            size_t ws_bytes, void* stream);
size_t lmhead_topk_tiled_workspace(int M, int V, int K, int k, int logits_kept);

/*
 * qg_stream_read -- measurement aid, not part of the decode path: one plain
 * streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a positive
 * multiple of 16) on `stream`, for reporting the device's HBM read rate
 * beside the kernels' (a pure-stream reference, as the Husky page's
 * "측정 환경과 검증 조건" section compares a step with a plain weight read).
 * *sink (4-byte aligned) is written only in a case that does not occur for
 * real data; it keeps the loads from being optimised away.
 */
qg_status qg_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                         void* stream);

/*
 * qg_affine4_valu -- measurement aid, not part of the decode path: the same
 * projection as qgemv_affine4 (same arguments, layout, checks and errors;
 * same K-slice / workgroup plan and the same split-K reduce), with the M-row
 * products formed on the vector ALU (v_dot2_f32_bf16 on bf16 activation
 * pairs and the exact bf16 values 128+q of the codes) instead of on the
 * matrix cores.  It exists so the two ways of computing the products can be
 * timed against each other on identical work at M = 1..8; its results agree
 * with qgemv_affine4's within fp32 summation order.
 */
qg_status qg_affine4_valu(const uint16_t* x, const uint32_t* codes,
                          const uint16_t* scales, const uint16_t* biases,
                          uint16_t* y, int M, int N, int K, void* ws, size_t ws_bytes,
                          void* stream);
size_t qg_affine4_valu_workspace(int M, int N, int K);

/*
 * Host-only twins of the entry points above: the same argument checks, no
 * GPU access, no launch.  They return what the entry point would return
 * before launching anything.
 */
qg_status qg_check_qgemv_affine4(const uint16_t* x, const uint32_t* codes,
                                 const uint16_t* scales, const uint16_t* biases,
                                 uint16_t* y, int M, int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_mlp_block_affine4_tiled(
    const uint16_t* x, const uint16_t* gamma, float eps,
    const uint32_t* gu_codes_t, const uint16_t* gu_sb_t,
    const uint32_t* dn_codes_t, const uint16_t* dn_sb_t, uint16_t* h,
    uint16_t* y, int M, int D, int I, const void* ws, size_t ws_bytes);
qg_status qg_check_qgemv_q6k(const uint16_t* x, const uint8_t* blocks,
                             uint16_t* y, int M, int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_qgemv_affine8(const uint16_t* x, const uint32_t* codes,
                                 const uint16_t* scales, const uint16_t* biases,
                                 uint16_t* y, int M, int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_qgemv_affine4_rht(const uint16_t* x, const int8_t* signs,
                                     int had, const uint32_t* codes,
                                     const uint16_t* scales,
                                     const uint16_t* biases, uint16_t* y, int M,
                                     int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_affine4_tile_pack(const uint32_t* codes,
                                     const uint16_t* scales,
                                     const uint16_t* biases, uint32_t* codes_t,
                                     uint16_t* sb_t, int N, int K);
qg_status qg_check_qgemv_affine4_tiled(const uint16_t* x,
                                       const uint32_t* codes_t,
                                       const uint16_t* sb_t, uint16_t* y, int M,
                                       int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_lmhead_argmax_tiled(const uint16_t* x,
                                       const uint32_t* codes_t,
                                       const uint16_t* sb_t, float* logits,
                                       int32_t* ids, const int32_t* draft,
                                       int32_t* accepted, int M, int V, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_rmsnorm_gateup_swiglu_tiled(const uint16_t* x,
                                               const uint16_t* gamma, float eps,
                                               const uint32_t* codes_t,
                                               const uint16_t* sb_t,
                                               uint16_t* h, int M, int I,
                                               int K, const void* ws, size_t ws_bytes);
qg_status qg_check_qgemv_q4k(const uint16_t* x, const uint8_t* blocks,
                             uint16_t* y, int M, int N, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_rmsnorm_gateup_swiglu(const uint16_t* x,
                                         const uint16_t* gamma, float eps,
                                         const uint32_t* codes_gu,
                                         const uint16_t* scales_gu,
                                         const uint16_t* biases_gu, uint16_t* h,
                                         int M, int I, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_moe_expert_qgemv(const uint16_t* x,
                                    const float* router_logits, int top_k,
                                    const uint8_t* w_gu, const uint8_t* w_down,
                                    uint16_t* y, int32_t* out_ids, float* out_w,
                                    int E, int D, int I, const void* ws, size_t ws_bytes);
qg_status qg_check_lmhead_argmax(const uint16_t* x, const uint32_t* codes,
                                 const uint16_t* scales, const uint16_t* biases,
                                 float* logits, int32_t* ids,
                                 const int32_t* draft, int32_t* accepted, int M,
                                 int V, int K, const void* ws, size_t ws_bytes);
qg_status qg_check_lmhead_topk(const uint16_t* x, const uint32_t* codes,
                               const uint16_t* scales, const uint16_t* biases,
                               float* logits, int32_t* ids, float* vals, int M,
                               int V, int K, int k, const void* ws, size_t ws_bytes);
qg_status qg_check_lmhead_topk_tiled(const uint16_t* x, const uint32_t* codes_t,
                                     const uint16_t* sb_t, float* logits,
                                     int32_t* ids, float* vals, int M, int V,
                                     int K, int k, const void* ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
