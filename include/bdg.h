/*
 * bdg.h - C ABI of libbdg, sparse-MoE expert decode over low-bit packed
 * weights on AMD Instinct MI355X (gfx950).
 *
 * The operation is one decode step of a mixture-of-experts layer (or a stack
 * of them) at small M: router top-k, then for each chosen expert a fused
 * dequant-GEMV over its packed gate_up weights, SwiGLU, a fused dequant-GEMV
 * over its packed down weights, and the router-weighted combine.  It is the
 * expert path of the pages:
 *   - "Sovereign gpt-oss-20B (MXFP4) on Apple Silicon": MXFP4 experts, the
 *     MXFP4 dequant-GEMV kernel (section 1), per token a router and 4
 *     sequential experts x 2 GEMVs per layer (section 3 Results), and the
 *     un-built lever of running the K active experts together (section 5);
 *   - "Single-stream int4 decode of a 30B MoE on Apple Silicon": packed int4
 *     weights dequantized on chip (sections 1 and 6);
 *   - "Amortizing the per-token host-sync setup tax in fused all-layer q4
 *     decode on Apple M1 Ultra": per-session setup tables rebuilt only on a
 *     geometry change (section 3), GPU-side top-k;
 *   - the TinyTitan project-tracker history, entries D108/D110 (fused int4
 *     dequant-inside-matmul, 16-byte row loads) and D114 (a layer's experts
 *     in one submission).
 * Beside it: a dense packed GEMV (qgemv), the large-M expert products on the
 * MX-scaled matrix cores, and the decode attention of a gpt-oss layer
 * (attn_rope_table, attn_decode).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must be device memory (hipMalloc /
 *     torch CUDA tensors); the caller owns every weight, input and output
 *     buffer and must keep them alive while work that uses them is queued.
 *     The library never frees or copies caller weights.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Calls only enqueue work on it and never synchronise, except
 *     moe_plan_create / moe_plan_destroy, which may allocate, free and
 *     synchronise, moe_expert_decode_profiled (it reads its timing events),
 *     and moe_expert_decode when a new key evicts a cached graph (it waits
 *     for that graph's last launch).
 *   - Return value: BDG_OK (0) or a negative BDG_E_* status.  Argument
 *     errors are found on the host before anything is enqueued, and leave
 *     outputs untouched.  Faults inside kernels surface at the caller's next
 *     synchronisation of the stream.
 *   - Layout (PLAIN, the interchange layout): row-major, K contiguous.
 *       MXFP4: codes [n][k/2] bytes, two FP4 E2M1 codes per byte, the low
 *              nibble holds the even K index; scales [n][k/32] E8M0 bytes,
 *              one per 32 contiguous K-elements of a row (OCP MX v1.0).
 *       INT4G: codes [n][k/2] bytes (unsigned q, low nibble = even k);
 *              scales [n][k/group] fp16; zeros [n][ceil(k/group/2)] bytes,
 *              two unsigned zero points per byte along the group axis, low
 *              nibble = even group.  w = (q - z) * s.
 *     Code rows are k/2 bytes; code bases and expert strides must be
 *     16-byte aligned (BDG_E_ALIGN otherwise).
 *   - Numerics: dequantized weights are exact (bit-exact with the IEEE fp32
 *     product, subnormals kept); dot products accumulate in fp32 in a fixed
 *     order, so repeated calls give identical bits.
 */
#ifndef BDG_H
#define BDG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define BDG_OK 0
#define BDG_E_INVALID -1     /* bad shape, dtype, flag, count or NULL pointer */
#define BDG_E_ALIGN -2       /* a code buffer or stride is not 16-byte aligned */
#define BDG_E_UNSUPPORTED -3 /* valid request outside what the kernels cover */
#define BDG_E_HIP -4         /* a HIP runtime call or kernel launch failed */
#define BDG_E_NOMEM -5       /* device allocation failed */
#define BDG_E_TOO_LARGE -6   /* request exceeds the static scratch of an allocation-free entry point */
#define BDG_E_WAIT -7        /* a bounded wait inside a kernel gave up (its outputs were made NaN) */

/* ---- activation dtypes ---- */
#define BDG_F32 0
#define BDG_BF16 1

/* ---- weight formats ---- */
#define BDG_FMT_MXFP4 0
#define BDG_FMT_INT4G 1

/* Limits of the kernels (BDG_E_UNSUPPORTED beyond them). */
#define BDG_MAX_K 8192       /* reduction length of one GEMV row */
#define BDG_MAX_M 16         /* tokens per call */
#define BDG_MAX_EXPERTS 1024
#define BDG_MAX_TOPK 32

/* A packed low-bit matrix [n][k] in the PLAIN layout, optionally one of a
 * batch of experts laid out at fixed byte strides.  One matrix (one expert)
 * holds at most 2^32 code bytes (n * k / 2; BDG_E_UNSUPPORTED beyond). */
typedef struct bdg_qmat {
  int32_t fmt;     /* BDG_FMT_MXFP4 or BDG_FMT_INT4G */
  int32_t group;   /* MXFP4: 32; INT4G: group size, a multiple of 32 */
  int64_t n;       /* rows (outputs) */
  int64_t k;       /* columns (reduction), a multiple of 32 and of group */
  const void* codes;   /* device, [n][k/2] bytes */
  const void* scales;  /* device, MXFP4 [n][k/32] bytes, INT4G [n][k/group] fp16 */
  const void* zeros;   /* device, INT4G [n][ceil(k/group/2)] bytes; NULL for MXFP4 */
  int64_t expert_stride_codes;   /* bytes from expert e to e+1 (0 if single) */
  int64_t expert_stride_scales;
  int64_t expert_stride_zeros;
  /* optional, MXFP4 only, for the MX matrix-core products (mx_gemm,
   * moe_prefill_mx): device, 16-byte aligned, the stage-major copy of
   * `scales` that mx_stage_scales writes ([E][k/128][n] 32-bit words).
   * NULL: those calls stage a copy into their workspace on every call.
   * The decode paths ignore it. */
  const void* mx_scale_words;
} bdg_qmat;

/* mxfp4_dequant - decode an MXFP4 matrix to fp32 (or bf16).
 * Defines the weight values every other call multiplies with: element
 * (r, c) = E2M1(code) * 2^(e - 127), E8M0 e = 255 giving NaN (OCP MX v1.0;
 * the MXFP4 reader of the gpt-oss page, section 3, is bit-exact).
 * codes [n][k/2], scales [n][k/32] as in the PLAIN layout; out [n][k] of
 * out_dtype (BDG_F32: bit-exact IEEE product, subnormals kept, +-inf on
 * overflow; BDG_BF16: that value rounded to nearest even, produced by
 * gfx950's scaled FP4 -> bf16 conversion, the one the matrix-core decode
 * path (BDG_MOE_MFMA) uses).  k % 32 == 0. */
int mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                  void* out, int32_t out_dtype, void* stream);

/* int4g_dequant - decode a group-quantized int4 matrix to fp32:
 * out[r][c] = (q - z) * s (on-chip int4 dequantisation of the 30B int4
 * page, section 6; fused-kernel identity of tracker entry D108).  Exact.
 * codes [n][k/2], scales_f16 [n][k/group], zeros [n][ceil(k/group/2)],
 * out [n][k] fp32; group % 32 == 0, k % group == 0. */
int int4g_dequant(const uint8_t* codes, const uint16_t* scales_f16, const uint8_t* zeros,
                  int64_t n, int64_t k, int32_t group, float* out, void* stream);

/* qgemv - fused dequant-GEMV: y[t][r] = sum_c W[r][c] * x[t][c] for t < m
 * (the MXFP4 dequant-GEMV of the gpt-oss page, section 1, with 16-byte
 * coalesced loads and on-chip dequant, section 4).  W is read packed, never
 * materialised.  x [m][k] of x_dtype (BDG_F32 or BDG_BF16), device;
 * y [m][n] fp32, device; x 16-byte aligned.  1 <= m <= BDG_MAX_M,
 * k <= BDG_MAX_K.  W's expert strides are ignored (expert 0). */
int qgemv(const bdg_qmat* w, const void* x, int32_t x_dtype, int32_t m, float* y,
          void* stream);

/* moe_router_topk - router GEMV + top-k + softmax over the chosen k.
 * logits[t][e] = sum_h W_r[e][h] * xin[t][h] (+ b_r[e]), computed in fp32;
 * idx[t][0..k) = the k largest logits in descending order, ties to the
 * lower expert index; wts[t][j] = exp(l_j - l_0) / sum_j' exp(l_j' - l_0).
 * xin = x, or RMSNorm(x) = x / sqrt(mean(x^2) + eps) (unit gain) when flags
 * has BDG_ROUTER_RMSNORM.  The GPU top-k of the host-sync page, section 3.
 * x [m][h] of x_dtype, w_r [e][h] fp32, b_r [e] fp32 or NULL; idx [m][k]
 * int32, wts [m][k] fp32, logits [m][e] fp32 or NULL - all device; x and
 * w_r 16-byte aligned, h % 4 == 0. */
#define BDG_ROUTER_RMSNORM 1
int moe_router_topk(const void* x, int32_t x_dtype, const float* w_r, const float* b_r,
                    int32_t m, int32_t h, int32_t e, int32_t topk, int32_t flags,
                    float norm_eps, int32_t* idx, float* wts, float* logits, void* stream);

/* ---- MoE decode plans ---- */

/* Per-layer weights: router [E][H] fp32 (+ optional bias [E]); gate_up is a
 * batch of E experts of [2I][H] (rows 0..I-1 are the gate g, rows I..2I-1
 * the up projection u); down is a batch of E experts of [I -> H], i.e.
 * [H][I].  All device pointers owned by the caller. */
typedef struct bdg_layer_desc {
  const float* w_router;
  const float* b_router;   /* NULL: no bias */
  bdg_qmat gate_up;
  bdg_qmat down;
} bdg_layer_desc;

/* flags for bdg_moe_desc.flags.  Every choice of the plan is made here, at
 * create time, from the descriptor alone (no environment variables): the
 * per-session setup of the host-sync page (section 3) is keyed on the
 * geometry, and a change needs a new plan. */
#define BDG_MOE_STACK 1      /* x <- x + MoE(RMSNorm(x)) per layer; else bare layers: x <- MoE(x) */
#define BDG_MOE_NO_GRAPH 2   /* launch the per-token kernels directly instead of replaying a graph
                                (same kernels, same results; for A/B checks) */
#define BDG_MOE_ROUTE_EVERY_LAYER 4  /* route every layer of an m = 1 stack with its own router
                                        kernel instead of from partial sums written by the
                                        previous layer's down kernel (same selection rule;
                                        logits differ only in fp32 summation order) */
#define BDG_MOE_PER_TOKEN 8  /* steps of m > 1 tokens run the per-token kernels (each pick reads
                                its expert) instead of the grouped kernels (each distinct
                                expert read once per step); same results bit for bit */
#define BDG_MOE_FUSED_LAYER 16  /* m = 1 steps run each layer as one kernel that streams the down
                                   weights into LDS behind the gate_up weights and exchanges h
                                   through a grid barrier, instead of two kernels (gate_up +
                                   SwiGLU, then down + combine); same results bit for bit.
                                   Slower on MI355X (measured); kept for A/B measurement */
#define BDG_MOE_MFMA 32  /* MXFP4 steps of m > 1 run each layer's grouped gate_up and down on the
                            matrix cores (v_mfma_f32_32x32x16_bf16): weights decoded once to
                            bf16 with the block scale, activations as bf16 hi + lo parts, fp32
                            accumulation; within the fp32 tolerance of the exact result, not
                            bit for bit with the VALU kernels.  Needs hidden and inter
                            multiples of 64 (else ignored) */
#define BDG_MOE_ROUTE_KERNEL 64  /* steps that run per-token kernels: every layer that needs its own
                                    router (the first layer; later layers with more than 64 experts,
                                    or BDG_MOE_ROUTE_EVERY_LAYER) launches the router kernel before
                                    gate_up.  By default such a layer routes inside its gate_up
                                    launch instead: the launch's first blocks take one router row
                                    per wave and publish the sums, every block waits for them (a
                                    bounded wait, see wait_polls); the first layer reads the
                                    caller's x there.  Same routing and results bit for bit, one
                                    launch per such layer fewer.  Self-routing needs hidden <= 3072,
                                    n_experts <= 256 and 4 * ceil(n_experts / 4) <= 24 *
                                    ceil(top_k * inter / 24); other shapes launch the router
                                    kernel */

typedef struct bdg_moe_desc {
  int32_t n_layers;
  int32_t hidden;      /* H */
  int32_t inter;       /* I */
  int32_t n_experts;   /* E */
  int32_t top_k;       /* k */
  int32_t fmt;         /* BDG_FMT_MXFP4 or BDG_FMT_INT4G (all layers alike) */
  int32_t group;       /* 32 for MXFP4; int4 group size */
  int32_t flags;       /* BDG_MOE_* */
  float norm_eps;      /* RMSNorm eps (stack only), e.g. 1e-5 */
  int32_t max_m;       /* largest m a decode call will pass, <= BDG_MAX_M */
  const bdg_layer_desc* layers;   /* n_layers entries; copied at create */
  int32_t wait_polls;  /* bound of the in-kernel waits (the fused kernel's grid barrier, a
                          self-routing gate_up's wait for the router sums), in polls of about
                          a microsecond: 0 = the default (2^20, about a second); a negative
                          value makes every wait give up at once (exercises the failure path) */
} bdg_moe_desc;

typedef struct bdg_plan bdg_plan;

/* moe_plan_create - validate a model geometry once and build what every
 * decode step reuses: the per-layer weight addresses (baked into each
 * captured kernel launch), the workspace (residual, routing partial sums,
 * intermediate activations),
 * and a cache of captured per-token HIP graphs.  The session-keyed setup
 * cache of the host-sync page (section 3): nothing of this is rebuilt per
 * token; a change of any weight pointer, shape or flag needs a new plan.
 * Allocates device memory, zero-fills the routing partial sums (padding
 * past the slices the kernels write must read as 0) and waits for the
 * device; synchronous.  *out receives the plan; BDG_E_HIP if the fill
 * fails. */
int moe_plan_create(const bdg_moe_desc* d, bdg_plan** out);

/* moe_plan_destroy - free a plan and everything it allocated (the end of
 * the session whose setup moe_plan_create built; host-sync page, section 3).
 * Waits for the device to finish queued work first, since captured graphs
 * and the workspace may still be in use.  NULL is accepted.  Returns BDG_OK. */
int moe_plan_destroy(bdg_plan* p);

/* moe_plan_check - report and clear the plan's fault word: BDG_E_WAIT if,
 * since the last check, a bounded wait inside the fused per-layer kernel or
 * a self-routing gate_up gave up (the blocks that gave up wrote NaN outputs,
 * so the step's y holds NaN), else BDG_OK.  Such a wait holds a block until
 * every block of the layer has published its h (fused kernel) or until the
 * launch's router rows are published (self-routing); it gives up only when
 * blocks of the grid could not run (the device shared with other work for
 * about a second) or when wait_polls is negative.  Waits for the plan's work
 * queued on `stream` (synchronous). */
int moe_plan_check(bdg_plan* p, void* stream);

/* moe_expert_decode - one decode step of m tokens through every layer of
 * the plan: per layer the router, top-k + softmax, the chosen experts'
 * gate_up dequant-GEMV + SwiGLU and down dequant-GEMV, and the weighted
 * combine (the per-token expert path of the gpt-oss page, section 3, with
 * the k experts of a layer run together as its section 5 proposes and the
 * tracker's entry D114 does; the all-layer decode of one submission per
 * token of the host-sync page, section 3).  x [m][H] of x_dtype (device) is the input hidden state; y [m][H]
 * fp32 (device) receives the output: for a stack, the residual stream after
 * the last layer; for a bare layer, the combine sum_j w_j * down_j(h_j).
 * Optional device traces (NULL to skip): topk_trace [L][m][k] int32 with
 * each layer's chosen experts, wts_trace [L][m][k] fp32 with their weights,
 * resid_trace [L][m][H] fp32 with each layer's input residual (stack) or
 * input (bare layer).  The per-token path is replayed from a captured HIP
 * graph keyed on (x, y, traces, m, x_dtype), captured at the first call with
 * that key (a cache of 8 graphs, least recently used evicted).  The first
 * call with a new key captures and instantiates (host work, no device
 * synchronisation); when that evicts a cached graph, the call first waits
 * on the host for the evicted graph's last launch to finish (an event
 * recorded on whichever stream launched it), then destroys it.  Other calls
 * only enqueue.  x, y and resid_trace must be 16-byte aligned.  m > max_m is
 * BDG_E_INVALID.  A plan is not re-entrant: calls on one plan must not run
 * concurrently (they share its workspace). */
int moe_expert_decode(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                      int32_t* topk_trace, float* wts_trace, float* resid_trace, void* stream);

/* moe_experts_routed - the expert part of one layer with caller-fixed
 * routing: y[t] = sum_j wts[t][j] * FFN_{idx[t][j]}(x[t]) (no router, no
 * norm, no residual): the "4 sequential experts x 2 GEMVs" of the gpt-oss
 * page (section 3) for routing the caller fixes, e.g. duplicate or skewed
 * picks.  Runs the same grouped gate_up/SwiGLU and down kernels
 * as moe_expert_decode.  x [m][H] of x_dtype, idx [m][k] int32 in [0, E),
 * wts [m][k] fp32, y [m][H] fp32, all device.  Expert ids are not range
 * checked on the host (they live on the device): out-of-range ids are
 * clamped to E-1 by the kernels. */
int moe_experts_routed(bdg_plan* p, int32_t layer, const void* x, int32_t x_dtype, int32_t m,
                       const int32_t* idx, const float* wts, float* y, void* stream);

/* ---- large-M product on the MX-scaled matrix cores ---- */

/* mxfp8_quantize - quantize activations x [m][k] (x_dtype BDG_F32 or
 * BDG_BF16, device, 16-byte aligned) to MXFP8: codes [m][k] FP8 E4M3 bytes
 * (device, 4-byte aligned) and scales [m][k/32] E8M0 bytes (device), one
 * per 32 contiguous elements of a row.  OCP MX v1.0 conversion, the reading
 * for the fp8 / grouped-expert GEMM that the host-sync page (section 5) and
 * the gpt-oss page (section 5) leave beyond their decode path: scale
 * 2^X with X = floor(log2 max|x|) - 8 (clamped to >= -127; an all-zero
 * block gives X = -127), elements x / 2^X rounded to nearest, ties to even,
 * saturating at +-448; a block holding a NaN or infinity gets scale 255 and
 * codes 0x7F.  k % 32 == 0. */
int mxfp8_quantize(const void* x, int32_t x_dtype, int64_t m, int64_t k, uint8_t* codes, uint8_t* scales,
                   void* stream);

/* mx_scale_words_bytes - bytes of the stage-major scale copy of n_experts
 * MXFP4 matrices like w (n_experts * ceil(k/128) * n 32-bit words), -1 for
 * invalid arguments. */
int64_t mx_scale_words_bytes(const bdg_qmat* w, int32_t n_experts);

/* mx_stage_scales - write the stage-major copy of the E8M0 scales of
 * n_experts MXFP4 matrices (w->scales at w->expert_stride_scales) into out
 * (device, 16-byte aligned, at least mx_scale_words_bytes(w, n_experts)
 * bytes): word [e][s][r] = row r's bytes of K blocks 4s .. 4s+3 (byte q =
 * block 4s + q, 127 past k).  One stage's scales of consecutive rows then
 * sit in consecutive words - a block row range's scales of a K stage are
 * one contiguous run for the MX products' copies to LDS, where the [n][k/32]
 * layout spreads them over a cache line per row.  A weight-layout step,
 * done once per matrix: point w->mx_scale_words at out afterwards (and
 * stage again if the scales change). */
int mx_stage_scales(const bdg_qmat* w, int32_t n_experts, void* out, int64_t out_bytes, void* stream);

/* mx_gemm_workspace - bytes of device workspace mx_gemm needs for an n x k
 * weight matrix and m tokens (-1 for invalid arguments): the stage-major
 * copies of both operands' scale bytes, [k/128][n] and [k/128][m] 32-bit
 * words (word [s][r] = row r's E8M0 bytes of K blocks 4s .. 4s+3), each
 * part 256-byte aligned. */
int64_t mx_gemm_workspace(int64_t n, int64_t k, int64_t m);

/* mx_gemm - y[t][r] = sum_c W[r][c] * xq[t][c] for t < m: MXFP4 weights W
 * (bdg_qmat, BDG_FMT_MXFP4, PLAIN layout, expert strides ignored) times
 * MXFP8 activations (x_codes [m][k], x_scales [m][k/32] from
 * mxfp8_quantize; x_codes 16-byte aligned), on the MX-scaled MFMA with fp32
 * accumulation; y [m][n] fp32, device.  workspace: device, 16-byte
 * aligned, at least mx_gemm_workspace(n, k, m) bytes, owned by the caller
 * (the call allocates nothing; it rewrites the workspace, and stages w's
 * scale words into it unless w->mx_scale_words is set).  The instruction
 * sums its products at reduced internal precision, so results agree with
 * the exact product to about 1e-4 of sum |W||xq| (not bit for bit).  Any
 * m >= 1, n >= 1 with n * k / 2 and m * k below 2^32 (BDG_E_UNSUPPORTED
 * beyond). */
int mx_gemm(const bdg_qmat* w, const uint8_t* x_codes, const uint8_t* x_scales, int64_t m, float* y,
            void* workspace, int64_t workspace_bytes, void* stream);

/* moe_prefill_mx_workspace - bytes of device workspace moe_prefill_mx needs
 * for m tokens of a layer of the given shape (-1 for invalid arguments).
 * Layout (each part starting 256-byte aligned, in this order; P = m * top_k):
 * activation codes [m][H] and scales [m][H/32] (MXFP8), row_off and
 * tile_off [E+1] int32, row_src [P] int32 (token of each grouped row),
 * pick_row [P] int32 (grouped row of pick t*k + j), h codes [P][I] (MXFP8),
 * then stage-major scale words (32-bit word [s][r] = row r's E8M0 bytes of
 * K blocks 4s .. 4s+3, 127 past K): the grouped activations' [H/128][P],
 * h's [I/128][P], the gate_up weights' [E][H/128][2I] and the down
 * weights' [E][I/128][H] (divisions rounded up), then down outputs [P][H]
 * fp32. */
int64_t moe_prefill_mx_workspace(int64_t m, int32_t hidden, int32_t inter, int32_t n_experts, int32_t top_k);

/* moe_prefill_mx - one bare MoE layer (no norm, no residual) over m tokens
 * at once on the MX-scaled matrix cores: the grouped-expert GEMM the
 * gpt-oss page leaves untried (section 5).  Router logits of x (fp32),
 * top-k + softmax as moe_router_topk (written to topk_idx [m][k] int32 and
 * topk_w [m][k] fp32); x quantized to MXFP8 (mxfp8_quantize); picks grouped
 * by expert; per expert [g; u] = W_gu . xq on the matrix cores, h = silu(g) *
 * u quantized to MXFP8 along the intermediate axis in the same kernel,
 * d = W_d . hq; y[t] = sum_j topk_w[t][j] d_{t,j} in slot order.  layer:
 * MXFP4 gate_up [E][2I][H] and down [E][H][I] at expert strides, router
 * w_router [E][H] fp32 (+ b_router); x [m][H] (BDG_F32 / BDG_BF16), y [m][H]
 * fp32, all device and 16-byte aligned; workspace: device memory of at least
 * moe_prefill_mx_workspace(...) bytes, owned by the caller (the call
 * allocates nothing; a weight matrix whose mx_scale_words is set is not
 * staged again).  Results agree with the exact MX arithmetic to about
 * 1e-3 of sum |W_d| |hq| (the matrix cores' reduced-precision sums, and the
 * rare rounding-boundary flips of hq that they cause). */
int moe_prefill_mx(const bdg_layer_desc* layer, int32_t n_experts, int32_t top_k, const void* x, int32_t x_dtype,
                   int64_t m, float* y, int32_t* topk_idx, float* topk_w, void* workspace,
                   int64_t workspace_bytes, void* stream);

/* ---- decode attention (gpt-oss layer) ---- */

/* Rotary embedding parameters, YaRN form (Peng, Quesnelle, Fan, Shippole
 * 2023) - the gpt-oss page reproduces its inverse frequencies and
 * attention scaling ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
 * section 3).  gpt-oss: theta 150000, factor 32, beta_fast 32, beta_slow 1,
 * orig_ctx 4096, truncate 0. */
typedef struct bdg_rope {
  double theta;       /* rotary base */
  double factor;      /* YaRN scale s; <= 1 gives plain rotary frequencies */
  double beta_fast;   /* rotation count over orig_ctx above which a frequency is kept */
  double beta_slow;   /* rotation count below which a frequency is divided by s */
  int32_t orig_ctx;   /* original context length L */
  int32_t truncate;   /* 1: round the two ramp ends outward to whole indices */
} bdg_rope;

/* attn_rope_table - the rotary table for positions 0 .. n_pos-1, computed
 * once per session: table [n_pos][head_dim] fp32 (device) holds
 * cos(p f_i) a in column i and sin(p f_i) a in column head_dim/2 + i, where
 * f_i is the YaRN inverse frequency of pair i and a the attention scaling
 * 0.1 ln s + 1 (1 when s <= 1), both rounded to fp32 first; the angle p f_i
 * is exact (float64) and each entry is rounded once to fp32.  Base
 * frequencies are theta^(-2i/d); between the indices where a pair turns
 * beta_fast and beta_slow times over orig_ctx the weight of the base
 * frequency falls linearly in the index from 1 to 0, the rest going to
 * f_i / s.  Optional outputs (device, nullable): inv_freq [head_dim/2] and
 * attn_scale [1].  head_dim even; n_pos <= 2^31. */
int attn_rope_table(const bdg_rope* rope, int32_t head_dim, int64_t n_pos, float* table, float* inv_freq,
                    float* attn_scale, void* stream);

/* attn_decode_workspace - bytes of device workspace attn_decode needs for
 * calls of m tokens whose longest key range (window, or pos0 + m) is at most
 * max_keys (-1 for shapes attn_decode does not take): the split partials
 * [m][n_kv_heads][splits <= 64][8][66] fp32 (max, sum, 64 weighted values)
 * of the attention over the cached keys. */
int64_t attn_decode_workspace(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t m,
                              int64_t max_keys);

/* attn_decode - one attention step of m new tokens at positions pos0 ..
 * pos0 + m - 1 (a decode token, or a short causal chunk), the attention of a
 * gpt-oss layer with learned per-head sinks ("Sovereign gpt-oss-20B (MXFP4)
 * on Apple Silicon", sections 1 and 4) and a sliding window (section 3).
 *   q [m][n_heads][64], k and v [m][n_kv_heads][64]: fp32 projections of
 *     the new tokens, before the rotation (device).
 *   k_cache, v_cache [n_kv_heads][cache_cap][64] of cache_dtype (BDG_BF16 or
 *     BDG_F32, device): positions < pos0 hold earlier tokens; the call
 *     stores the new tokens' rotated keys and values at pos0 .. pos0 + m - 1
 *     (rotation in fp32 with each product and sum rounded on its own, then
 *     round-to-nearest-even to the cache dtype).
 *   rope_table [table_rows][64] from attn_rope_table (device).
 *   Query head h uses KV head h / 8 (n_heads = 8 n_kv_heads) and its rotated
 *     query; token t (position p = pos0 + t) attends keys j with
 *     max(0, p - window + 1) <= j <= p (window 0: 0 <= j <= p):
 *     o = sum_j e^(s_j) v_j / (sum_j e^(s_j) + e^(sinks[h])),
 *     s_j = sm_scale (q . k_j); sinks [n_heads] fp32 (device) or NULL for none.
 *   o [m][n_heads][64] fp32 (device).
 *   workspace: attn_decode_workspace(...) bytes of device memory, 16-byte
 *     aligned, owned by the caller (no initial contents needed).  Calls that
 *     share a workspace must not overlap in time.
 * Two kernels: the attention over the cached keys, split across blocks;
 * then per (token, KV head) the keys of the call itself, the merge of the
 * splits and the sink, and the append of the token's key and value.
 * Scores, softmax and sums are fp32 (within a stated bound of the exact
 * result, not bit for bit); the stored cache entries are exact.  All device
 * pointers 16-byte aligned.  head_dim 64, 8 query heads per KV head and
 * m <= 64 only (BDG_E_UNSUPPORTED otherwise); pos0 + m <= cache_cap and
 * <= table_rows.
 * Inputs must be finite. */
int attn_decode(const float* q, const float* k, const float* v, void* k_cache, void* v_cache, int32_t cache_dtype,
                int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t m, int64_t pos0,
                const float* rope_table, int64_t table_rows, float sm_scale, const float* sinks, int32_t window,
                float* o, void* workspace, int64_t workspace_bytes, void* stream);

/* attn_decode_noalloc - attn_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * (bit for bit) as attn_decode, without the workspace: the split partials
 * live in a static device array of BDG_ATTN_SCRATCH_BYTES per GPU, owned by
 * the library and held until the process ends (its device address is looked
 * up once per device, at that device's first call).  The call itself
 * allocates and frees nothing.  A call whose attn_decode_workspace(...)
 * exceeds BDG_ATTN_SCRATCH_BYTES returns BDG_E_TOO_LARGE before any launch
 * (with 8 KV heads: m <= 7 tokens).  Nothing in the array needs initial
 * contents; every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (other streams, other threads) race: order
 * them. */
#define BDG_ATTN_SCRATCH_BYTES (8 * 1024 * 1024)
int attn_decode_noalloc(const float* q, const float* k, const float* v, void* k_cache, void* v_cache,
                        int32_t cache_dtype, int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads,
                        int32_t head_dim, int32_t m, int64_t pos0, const float* rope_table, int64_t table_rows,
                        float sm_scale, const float* sinks, int32_t window, float* o, void* stream);

/* ---- measurement aids ---- */

/* moe_expert_decode_profiled - one decode step exactly as moe_expert_decode
 * computes it (same kernels, same grids), launched directly rather than from
 * a graph, each kernel with a start and a stop event that take the
 * dispatch's own start and end times.  Adds each kernel's duration (ms) to
 * kernel_ms[kind] and 1 to kernel_count[kind]; kind 0 = route (router
 * GEMV + sum of squares, and for steps of m > 1 the previous layer's
 * combine), 1 = gate_up (top-k + grouped gate_up GEMV + SwiGLU), 2 = down
 * (grouped down GEMV; combine + residual when m = 1), 3 = the final combine
 * of an m > 1 step, 4 = the fused per-layer kernel; host arrays of at
 * least 5.
 * Synchronises on the last event before returning.  Used by the benchmark
 * for per-kernel roofline figures. */
int moe_expert_decode_profiled(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                               double* kernel_ms, int64_t* kernel_count, void* stream);

/* moe_expert_decode_timeline - one single-token decode step exactly as
 * moe_expert_decode computes it on the fused per-layer path (launched
 * directly, not from a graph), with each block of each layer kernel
 * stamping the GPU's 100 MHz clock at its phase boundaries: routing done,
 * gate_up loads issued, down codes issued, h computed, h stored, barrier
 * passed, h staged, down rows done, end (see LayerStamp in the sources).
 * stamps (host) receives [n_layers][blocks][16] uint64 (0 = not reached);
 * returns the count written, or a negative status (BDG_E_UNSUPPORTED when
 * the plan does not use the fused kernel).  Synchronous; allocates a stamp
 * buffer in the plan on first use.  For measuring where a layer's time
 * goes. */
int64_t moe_expert_decode_timeline(bdg_plan* p, const void* x, int32_t x_dtype, float* y, uint64_t* stamps,
                                   int64_t max_stamps, void* stream);

/* bdg_stream_read - read `bytes` (a multiple of 16) of device memory with
 * 16-byte coalesced loads and write one fp32 checksum per workgroup into
 * sink [n_blocks] (device).  n_blocks <= 0 picks the default grid.  Used to
 * measure the achievable HBM read rate next to the decode path. */
int bdg_stream_read(const void* buf, int64_t bytes, float* sink, int32_t n_blocks, void* stream);

/* bdg_stream_copy - copy `bytes` (a multiple of 16) device to device with
 * 16-byte loads/stores; a kernel of known traffic for calibrating counters. */
int bdg_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* bdg_strerror - static text for a status code (any int; unknown codes get
 * a generic text).  Host only, never fails; the text is owned by the
 * library. */
const char* bdg_strerror(int32_t status);

/* bdg_version - library version string. */
const char* bdg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BDG_H */
