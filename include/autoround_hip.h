/*
 * autoround_hip.h - C ABI of the MI355X (gfx950) AutoRound per-Linear tuning library.
 *
 * AutoRound tunes, per weight group, a rounding offset V in [-0.5, 0.5] and two
 * clip factors (alpha on the group minimum, beta on the group maximum) by
 * SignSGD so that the fake-quantized weight Ŵ = s*(clamp(rint(W/s + V) + zp) - zp)
 * reproduces the layer output X·Wᵀ on calibration tokens; the final integer codes
 * are then packed into 32-bit words.
 *
 * Sources (page title, section):
 *   [LLMC]  "[llm-compressor] AutoRound: 부호 경사 하강법으로 라운딩 최적화":
 *           paper-core equations (RTN, learnable offset, SignSGD), constructor
 *           parameter table, the per-module tuning loop, _fake_quantize_with_offset.
 *   [INTEL] "Introducing AutoRound: Intel's Advanced Quantization for LLMs and VLMs":
 *           section 2 (rounding and clipping range tuned jointly), section 4
 *           (zero iterations = RTN; 8/4/3/2-bit).
 *   [SGL]   "[SGLang] AutoRound: 자동 라운딩 최적화 양자화": "1. AutoRoundConfig"
 *           (bits {2,3,4,8}, sym, pack_factor = Fraction(32, bits)), "설계 근거"
 *           (GPTQ/AWQ packing reuse).
 *
 * Conventions for every entry point:
 *   - Every array pointer is a caller-owned DEVICE pointer (hipMalloc / torch),
 *     row-major and contiguous, 16-byte aligned. The library never allocates
 *     device memory; scratch space comes in through (ws, ws_bytes).
 *   - `stream` is a hipStream_t (NULL = default stream). All device work is
 *     enqueued asynchronously on it, except where an entry point says it blocks.
 *   - Arguments are validated before anything is enqueued; on any error status
 *     nothing has been written. No C++ exception crosses this interface.
 *   - Shapes: W is [N, K] (N out features, K in features, torch Linear layout).
 *     K must be a multiple of 8 and of group_size; G = K / group_size groups per
 *     row (group_size = -1: one group of K per row). group_size must be a
 *     multiple of 8. N >= 1 and K >= 8, except where an entry point accepts N*K = 0.
 *   - bf16 data is passed as uint16 bit patterns.
 */
#ifndef AUTOROUND_HIP_H
#define AUTOROUND_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AR_OK = 0,
  AR_ERR_INVALID_ARG = 1,   /* null pointer, bad hyper-parameter, misaligned pointer */
  AR_ERR_UNSUPPORTED = 2,   /* bits not in {2,3,4,8} (16 = "leave unquantized"), bad dtype */
  AR_ERR_SHAPE = 3,         /* size constraint violated */
  AR_ERR_WORKSPACE = 4,     /* ws_bytes smaller than the *_workspace_size result */
  AR_ERR_NONFINITE = 5,     /* check_finite set and an input holds NaN or Inf */
  AR_ERR_HIP = 6            /* a HIP runtime call or kernel launch failed */
} ar_status;

typedef enum { AR_F32 = 0, AR_BF16 = 1 } ar_dtype;

/* Tuning hyper-parameters; names as on the [LLMC] constructor parameter table. */
typedef struct {
  int32_t bits;          /* {2,3,4,8}: [SGL] 1. AutoRoundConfig SUPPORTED_BITS            */
  int32_t group_size;    /* input channels per group; -1 = whole row                      */
  int32_t sym;           /* 0: asymmetric (zero-point from the range), 1: symmetric        */
  int32_t nsamples;      /* calibration samples ([LLMC] default 128)                       */
  int32_t seqlen;        /* tokens per sample ([LLMC] default 2048)                        */
  int32_t batch_samples; /* samples per SignSGD step; nsamples % batch_samples == 0        */
  int32_t iters;         /* SignSGD steps ([LLMC] default 200); 0 = RTN ([INTEL] sec. 4)   */
  float lr;              /* offset step ([LLMC] default 0.005)                             */
  float minmax_lr;       /* clip-factor step; < 0 means "unset" = lr ([LLMC] minmax_lr)    */
  float minmax_shrink;   /* initial alpha = beta ([LLMC] minmax_shrink, default 1.0)       */
  float clip_lo;         /* alpha/beta lower clamp (default 0.5)                           */
  float clip_hi;         /* alpha/beta upper clamp (default 1.0)                           */
  int32_t init_scale;    /* initial alpha = beta ([LLMC] tuning loop: "Min-Max or MSE"):
                            0: minmax_shrink (Min-Max); 1: MSE, per group the shrink p of
                            the grid p_j = float32(1 - j/mse_grid) inside [clip_lo, clip_hi]
                            whose round-to-nearest quantization has the smallest sum of
                            squared weight errors (float32 errors, float64 sum, first
                            minimum on ties)                                              */
  int32_t mse_grid;      /* grid steps per unit shrink for init_scale = 1 (default 100)   */
  int32_t check_finite;  /* 0 (default): no check. A NaN or Inf in the data then makes
                            the loss of every step that reads it NaN: such a step is
                            never taken as the best (the comparison is a strict <), and
                            its non-finite gradients move nothing (sgn(NaN) = 0), so the
                            returned state stays finite. The [LLMC] tuning loop reads
                            each batch loss on the host; this loop does not.
                            1: the tuning entry points (ar_tune_step, ar_tune_linear and
                            their Gram and no-allocation forms) first scan their inputs
                            (W, X, Y; the step also V, alpha, beta) on the device and
                            return AR_ERR_NONFINITE, with no output written, when any
                            element is NaN or infinite. The call then blocks until the
                            scan's result is on the host, so it cannot be captured in a
                            HIP graph. ar_tune_block passes it to each Linear's tuning. */
} ar_config;

/* Per-kernel device time of one ar_tune_linear call, measured with HIP events
   recorded on the call's stream around the kernels of every sample_every-th
   SignSGD step (milliseconds, summed over the timed steps). */
typedef struct {
  int32_t sample_every;  /* input: time steps i with i % sample_every == 0 (<= 1: every step) */
  double fwd_gemm_ms;    /* Y' = X_b·Ŵᵀ with the residual / dY / R² epilogue               */
  double wgrad_gemm_ms;  /* G = (2/(T_b·N))·dYᵀ·X_b, with the loss reduction and best-loss
                            decision in its prologue                                        */
  double ste_update_ms;  /* straight-through fold + SignSGD update + next fake-quant         */
  int64_t steps;         /* output: number of SignSGD steps timed                          */
} ar_kernel_times;

/* Fill *cfg with the [LLMC] defaults: bits 4, group_size 128, asym, nsamples 128,
   seqlen 2048, batch_samples 8, iters 200, lr 0.005, minmax_lr unset (-1),
   minmax_shrink 1.0, clip range [0.5, 1.0], Min-Max initial scale (mse_grid 100).
   Returns AR_ERR_INVALID_ARG on NULL. */
ar_status ar_config_default(ar_config* cfg);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ar_status_string(int32_t status);

/* Bytes of device workspace ar_tune_linear needs for this problem (X is
   [nsamples*seqlen, K] bf16, Y is [nsamples*seqlen, N] of dtype ydt). */
ar_status ar_workspace_size(const ar_config* cfg, int64_t N, int64_t K, int32_t ydt,
                            size_t* bytes);

/* Bytes of device workspace ar_tune_step needs for a minibatch of Tb tokens. */
ar_status ar_step_workspace_size(const ar_config* cfg, int64_t N, int64_t K, int64_t Tb,
                                 int32_t ydt, size_t* bytes);

/* Initial clip factors of every group ([LLMC] tuning loop, initial scale):
   alpha = beta = minmax_shrink (init_scale 0) or the MSE shrink (init_scale 1).
   alpha, beta [N, G] float32, required. N*K = 0 is a no-op. */
ar_status ar_init_clip(const ar_config* cfg, int32_t wdt, const void* W, int64_t N, int64_t K,
                       float* alpha, float* beta, void* stream);

/* Round-to-nearest quantization ([LLMC] paper-core RTN equation): V = 0 and
   the initial clip factors of ar_init_clip; group min/max from W ([LLMC] tuning
   loop, initial scale).
   W      [N, K] of dtype wdt (AR_F32 or AR_BF16)
   codes  [N, K] uint8 in [0, 2^bits-1]        (nullable)
   scale  [N, G] float32                       (nullable)
   zp     [N, G] uint8 zero-points              (nullable)
   Wq     [N, K] of dtype wdt, s*(code - zp)    (nullable)
   N*K = 0 is a no-op. */
ar_status ar_rtn_quant(const ar_config* cfg, int32_t wdt, const void* W, int64_t N, int64_t K,
                       uint8_t* codes, float* scale, uint8_t* zp, void* Wq, void* stream);

/* Fake-quantization with learnable offset and clip factors ([LLMC] paper-core
   offset equation and _fake_quantize_with_offset; [INTEL] sec. 2 clip range):
   per group lo = min(alpha*wmin, 0), hi = max(beta*wmax, 0), s = (hi-lo)/maxq,
   zp = clamp(rint(-lo/s), 0, maxq)  (sym: s = 2*max(|alpha*wmin|, |beta*wmax|)/maxq,
   zp = 2^(bits-1)); per element code = clamp(rint(W/s + V) + zp, 0, maxq),
   Ŵ = s*(code - zp). A zero-range group uses s = 1. All float32, rint = half-even.
   V [N, K] float32; alpha, beta [N, G] float32.
   Wq_bf16 [N, K] bf16 Ŵ (nullable); codes, scale, zp as in ar_rtn_quant (nullable).
   N*K = 0 is a no-op. */
ar_status ar_fakequant_fwd(const ar_config* cfg, int32_t wdt, const void* W, int64_t N,
                           int64_t K, const float* V, const float* alpha, const float* beta,
                           uint16_t* Wq_bf16, uint8_t* codes, float* scale, uint8_t* zp,
                           void* stream);

/* Tuning state of one Linear, all device pointers owned by the caller. */
typedef struct {
  const void* W;       /* [N, K] weight, dtype wdt          */
  int32_t wdt;         /* AR_F32 or AR_BF16                  */
  int64_t N, K;
  float* V;            /* [N, K] offsets, updated in place   */
  float* alpha;        /* [N, G] min clip factors, in place  */
  float* beta;         /* [N, G] max clip factors, in place  */
  float* best_V;       /* [N, K] best-state snapshot   (nullable: no snapshot; the four
                          best_* pointers are all set or all NULL) */
  float* best_alpha;   /* [N, G]                              */
  float* best_beta;    /* [N, G]                              */
  float* best_loss;    /* device scalar; caller initialises it to +inf */
} ar_state;

/* One SignSGD iteration on one minibatch ([LLMC] tuning loop; [LLMC] SignSGD
   equation). From the current state: Ŵ (bf16 operand), Y' = Xb·Ŵᵀ (bf16 MFMA,
   float32 accumulation), R = Y' - Yb, loss = sum(R²)/(Tb·N) -> loss_out[0];
   dY = bf16(R); G = (2/(Tb·N))·dYᵀ·Xb; straight-through fold to dL/dV, dL/dalpha,
   dL/dbeta. If best_* are set and loss < *best_loss, the current (pre-update)
   state is copied to best_* and *best_loss = loss. If apply_update != 0:
   V <- clamp(V - lr·sgn(dL/dV), -0.5, 0.5), alpha/beta <- clamp(· - minmax_lr·sgn, clip_lo, clip_hi).
   Xb [Tb, K] bf16; Yb [Tb, N] of dtype ydt; Tb > 0, Tb % 8 == 0.
   loss_out: device float (required). gV [N, K], galpha/gbeta [N, G] float32:
   pre-update gradients (nullable). ws: ar_step_workspace_size bytes. */
ar_status ar_tune_step(const ar_config* cfg, const ar_state* state, const uint16_t* Xb,
                       const void* Yb, int32_t ydt, int64_t Tb, float* loss_out, float* gV,
                       float* galpha, float* gbeta, int32_t apply_update, void* ws,
                       size_t ws_bytes, void* stream);

/* ar_tune_step for callers that cannot allocate device memory (code under HIP
   graph capture, tight loops, harnesses that forbid allocation): the same
   arguments without (ws, ws_bytes), and the same kernels, results and errors.
   Its scratch is a fixed array of AR_NOALLOC_SCRATCH_BYTES in each GPU's
   memory, set up on the first call on that device (the device current at the
   call, which must be the stream's) and held until the process ends. A problem
   whose ar_step_workspace_size exceeds AR_NOALLOC_SCRATCH_BYTES returns
   AR_ERR_WORKSPACE before anything is enqueued. The call makes no device
   allocation. Every call on one GPU shares that GPU's array: calls that may
   overlap on one GPU (other streams, other host threads) race and must be
   serialised by the caller. Each call writes every part of the array it reads
   before reading it, so what an earlier call left there does not matter. */
#define AR_NOALLOC_SCRATCH_BYTES ((size_t)64 * 1024 * 1024)
ar_status ar_tune_step_noalloc(const ar_config* cfg, const ar_state* state, const uint16_t* Xb,
                               const void* Yb, int32_t ydt, int64_t Tb, float* loss_out,
                               float* gV, float* galpha, float* gbeta, int32_t apply_update,
                               void* stream);

/* The whole per-Linear tuning loop ([LLMC] tuning loop with best-loss snapshot):
   V = 0, alpha and beta from ar_init_clip; step i uses minibatch b = i mod
   (nsamples/batch_samples), i.e. rows [b*Tb, (b+1)*Tb) of X and Y with
   Tb = batch_samples*seqlen; after cfg->iters steps the state with the lowest
   loss (strictly lower than all before it, evaluated before its update) is
   restored and quantized. iters = 0 gives RTN ([INTEL] section 4).
   W [N, K] wdt; X [nsamples*seqlen, K] bf16; Y [nsamples*seqlen, N] ydt.
   Outputs: codes [N, K] uint8, scale [N, G] float32, zp [N, G] uint8 (required);
   Wq [N, K] wdt (nullable); V_out [N, K], alpha_out/beta_out [N, G] float32 final
   (restored) state (nullable); losses [iters] float32 per-step loss (nullable).
   ws: ar_workspace_size bytes. times: when non-NULL, per-kernel device times of
   every times->sample_every-th step are measured with HIP events and, with
   iters > 0, the call blocks until the stream has drained (iters = 0 leaves the
   times at zero and does not block). */
ar_status ar_tune_linear(const ar_config* cfg, int32_t wdt, const void* W, int64_t N, int64_t K,
                         const uint16_t* X, const void* Y, int32_t ydt, uint8_t* codes,
                         float* scale, uint8_t* zp, void* Wq, float* V_out, float* alpha_out,
                         float* beta_out, float* losses, void* ws, size_t ws_bytes,
                         ar_kernel_times* times, void* stream);

/* ---- W{2,3,4,8} x bf16 product on the packed format ------------------------
   Y = X·bf16(Ŵ)ᵀ with Ŵ = s·(q - zp) read from ar_pack's format ([SGL] "설계
   근거": AutoRound checkpoints reuse GPTQ/AWQ packing; [LLMC]
   _fake_quantize_with_offset for the dequantisation): the deployment side of the
   tuned codes. The bf16 Ŵ is the operand the tuning loop's forward product uses.
   X [M, K] bf16 row-major; qweight [K*bits/32, N] int32 and qzeros
   [G, N*bits/32] int32 as ar_pack writes them (qzeros NULL: symmetric grid,
   zp = 2^(bits-1)); scale [N, G] float32 (ar_tune_linear's layout); Y [M, N]
   row-major, ydt AR_F32 or AR_BF16. float32 accumulation. group_size as in
   ar_config (-1: whole row); K*bits % 32 == 0, K % group = 0, group % 8 == 0;
   with qzeros N*bits % 32 == 0. M <= 16 streams the packed words once,
   dequantizing each code once for all M rows (split-K, slices summed in a fixed
   order); larger M dequantizes once into a blocked bf16 operand and runs the
   MFMA product. M = 0 or N = 0 is a no-op. The workspace size depends on bits,
   group_size and the shape (the split-K slice length follows the group size);
   ar_dequant_gemm_workspace_size validates them as ar_dequant_gemm does. */
ar_status ar_dequant_gemm_workspace_size(int32_t bits, int32_t group_size, int64_t M, int64_t N,
                                         int64_t K, size_t* bytes);
ar_status ar_dequant_gemm(int32_t bits, int32_t group_size, const uint16_t* X, int64_t M,
                          int64_t K, const int32_t* qweight, const int32_t* qzeros,
                          const float* scale, int64_t N, void* Y, int32_t ydt, void* ws,
                          size_t ws_bytes, void* stream);

/* ---- Sequential block-wise tuning with quantized inputs --------------------
   [LLMC] tuning loop (each Linear of a subgraph tuned in turn on its captured
   inputs and targets), parameter table and "enable_quanted_input 모드" (the
   previous layers' quantized output as input), design point 3 (layer by
   layer). The pages do not show the block; a Llama-style decoder block is
   used: a = RMSNorm(h); q, k, v = a·W{q,k,v}ᵀ; rotate-half rotary embedding
   on q and k (theta rope_theta, position = token index within its sequence);
   causal softmax(q·kᵀ/sqrt(Dh))·v per sequence and head; h1 = h + attn·Woᵀ;
   m = RMSNorm(h1); z = SiLU(m·Wgᵀ)·(m·Wuᵀ); out = h1 + z·Wdᵀ. bf16
   activations between operations. */
typedef struct {
  int64_t hidden;       /* D                                  */
  int64_t heads;        /* H; head_dim D/H must be 64 or 128  */
  int64_t inter;        /* F (MLP width)                      */
  int64_t seqlen;       /* tokens per calibration sequence    */
  int64_t nsamples;     /* calibration sequences              */
  float rms_eps;
  float rope_theta;
} ar_block_dims;

typedef struct {        /* bf16 [out, in] row-major; norms bf16 [D] */
  const uint16_t *Wq, *Wk, *Wv, *Wo, *Wg, *Wu, *Wd;
  const uint16_t *norm_attn, *norm_mlp;
} ar_block_weights;

/* Per Linear, in the order q, k, v, o, gate, up, down: codes [N, K] uint8,
   scale [N, G] float32, zp [N, G] uint8, Wq [N, K] bf16 (all required),
   losses [iters] float32 (nullable). out_fp / out_q [M, D] bf16: the block
   output with the original / the tuned weights (nullable). */
typedef struct {
  uint8_t* codes[7];
  float* scale[7];
  uint8_t* zp[7];
  uint16_t* Wq[7];
  float* losses[7];
  uint16_t* out_fp;
  uint16_t* out_q;
} ar_block_outputs;

/* Workspace bytes for ar_block_forward (cfg NULL) or ar_tune_block (cfg set;
   cfg->nsamples * cfg->seqlen must equal the block's token count). */
ar_status ar_block_workspace_size(const ar_config* cfg, const ar_block_dims* dims, size_t* bytes);

/* The block's forward on h [nsamples*seqlen, D] bf16 -> out (same shape). */
ar_status ar_block_forward(const ar_block_dims* dims, const ar_block_weights* w,
                           const uint16_t* h, uint16_t* out, void* ws, size_t ws_bytes,
                           void* stream);

/* The block's attention step alone: out = causal softmax(q·kᵀ/sqrt(Dh))·v per
   sequence (dims->seqlen consecutive rows) and head (dims->heads column groups
   of Dh = hidden/heads, 64 or 128), with q and k already rotated. q, k, v, out
   [nsamples·seqlen, hidden] bf16 row-major, 16-byte aligned; float32
   accumulation and softmax, bf16 output. No workspace. */
ar_status ar_attention(const ar_block_dims* dims, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, uint16_t* out, void* stream);

/* Tune the block's seven Linears in order q, k, v, o, gate, up, down, each with
   ar_tune_linear on target Y = its full-precision output (the block with the
   original weights on h) and input X = its input in the quantized pipeline
   (quanted_input != 0: the block on h_q with the Linears tuned so far replaced
   by their bf16 Ŵ; h_q NULL means h) or in the full-precision pipeline
   (quanted_input = 0). cfg as for ar_tune_linear with nsamples*seqlen = the
   block's tokens. Blocks until the host has enqueued all work. */
ar_status ar_tune_block(const ar_config* cfg, const ar_block_dims* dims,
                        const ar_block_weights* w, const uint16_t* h, const uint16_t* h_q,
                        int32_t quanted_input, const ar_block_outputs* outs, void* ws,
                        size_t ws_bytes, void* stream);

/* ---- Per-layer configuration ([SGL] "2. 레이어별 개별 설정", "3. 정규식 기반
   레이어 매칭", "4. FusedMoE와 Fused QKV 처리"). Host-only calls: strings and
   arrays are host memory, nothing touches the GPU. -------------------------- */

/* One per-layer rule. The key is an exact layer name, or a pattern when it
   contains any of the characters * + ? ^ $ ( ) [ ] { } | \ (ECMAScript regular
   expression, matched against the whole name). */
typedef struct {
  const char* key;
  int32_t bits;         /* < 0: not set                      */
  int32_t group_size;   /* 0: not set (-1 is "whole row")    */
  int32_t sym;          /* < 0: not set, else 0 / 1          */
} ar_layer_rule;

typedef struct {
  int32_t bits;         /* 16: leave the layer unquantized   */
  int32_t group_size;
  int32_t sym;
} ar_layer_qconfig;

/* Config of layer `name`. quantized = 0 marks a layer outside the quantized
   set: with no rule, or an exact-name rule leaving fields unset, it gets
   bits 16, group_size -1, sym 1. Order: exact key, then the first pattern key
   that fully matches (keys that do not compile are skipped; unset fields from
   *defaults), then the fallback. AR_ERR_INVALID_ARG on NULL arguments. */
ar_status ar_resolve_layer_config(const ar_layer_rule* rules, int32_t nrules,
                                  const ar_layer_qconfig* defaults, int32_t quantized,
                                  const char* name, ar_layer_qconfig* out);

/* Config of a fused layer: every sub-layer must resolve to the same config,
   else AR_ERR_INVALID_ARG. With sub_names set (nsub > 0) the sub-layers are
   sub_names (a fused q/k/v-style layer). With sub_names NULL (nsub = 0) they
   are the rule keys that start with layer_name (a fused expert layer); with
   no such key, layer_name itself. sub_names set with nsub = 0 (an empty
   sub-layer list) is AR_ERR_INVALID_ARG, as is sub_names NULL with nsub > 0. */
ar_status ar_resolve_fused_config(const ar_layer_rule* rules, int32_t nrules,
                                  const ar_layer_qconfig* defaults, int32_t quantized,
                                  const char* layer_name, const char* const* sub_names,
                                  int32_t nsub, ar_layer_qconfig* out);

/* ---- Gram form (same-input Linears) --------------------------------------
   For one Linear the quantized and the reference outputs see the same tokens,
   so the minibatch loss and its gradient depend on the tokens only through
   H = Xbᵀ·Xb (the Hessian weight of the layer objective, ADMM-Q page "1. 문제
   공식화"), Cn = (Xb·Wᵀ - Yb)ᵀ·Xb and e2 = |Xb·Wᵀ - Yb|²: with D = bf16(Ŵ) - W,
     sum(R²) = Σ D∘(D·H) + 2·Σ D∘Cn + e2,   dL/dŴ = (2/(Tb·N))·(D·H + Cn).
   This is the [LLMC] output-reconstruction loss with the residual kept
   unrounded (the token form rounds dY to bf16), at 2·N·K·3K product FLOP per
   step instead of 4·Tb·K·N: D·H runs as bf16 MFMA on a hi/lo split
   (D_hi·H_hi + D_hi·H_lo + D_lo·H_hi, float32 accumulation). The statistics
   are computed once per minibatch (three products of the minibatch's tokens).
   Everything else (quantizer, straight-through fold, SignSGD, snapshot,
   finalisation) is the token form's. */

/* Bytes of device workspace for ar_tune_linear_gram (wdt: dtype of W). */
ar_status ar_gram_workspace_size(const ar_config* cfg, int32_t wdt, int64_t N, int64_t K,
                                 int32_t ydt, size_t* bytes);

/* Bytes of device workspace for ar_tune_step_gram with a minibatch of Tb tokens. */
ar_status ar_gram_step_workspace_size(const ar_config* cfg, int32_t wdt, int64_t N, int64_t K,
                                      int64_t Tb, int32_t ydt, size_t* bytes);

/* ar_tune_step in the Gram form: same arguments, state semantics and outputs
   (loss_out = sum(R²)/(Tb·N) with R unrounded; gradients from D·H + Cn). The
   minibatch's statistics are computed inside the call. ws:
   ar_gram_step_workspace_size bytes. */
ar_status ar_tune_step_gram(const ar_config* cfg, const ar_state* state, const uint16_t* Xb,
                            const void* Yb, int32_t ydt, int64_t Tb, float* loss_out, float* gV,
                            float* galpha, float* gbeta, int32_t apply_update, void* ws,
                            size_t ws_bytes, void* stream);

/* ar_tune_linear in the Gram form: same arguments and outputs. ws:
   ar_gram_workspace_size bytes (the per-minibatch H and Cn live there: nb·(6·K·K
   + 4·N·K) bytes for nb = nsamples/batch_samples minibatches). With times,
   fwd_gemm_ms is the product D·H, ste_update_ms the update kernel and
   wgrad_gemm_ms is 0. */
ar_status ar_tune_linear_gram(const ar_config* cfg, int32_t wdt, const void* W, int64_t N,
                              int64_t K, const uint16_t* X, const void* Y, int32_t ydt,
                              uint8_t* codes, float* scale, uint8_t* zp, void* Wq, float* V_out,
                              float* alpha_out, float* beta_out, float* losses, void* ws,
                              size_t ws_bytes, ar_kernel_times* times, void* stream);

/* Pack codes into 32-bit words ([SGL] pack_factor = Fraction(32, bits); GPTQ-style
   layout): code (n, k) occupies bits [k*bits, (k+1)*bits) of the bit string of
   column n, least significant bit first, so word w of column n is
   qweight[w, n] (a 3-bit code that straddles two words is split, low bits first).
   codes [N, K] uint8 -> qweight [K*bits/32, N] int32.
   zp [N, G] uint8 -> qzeros [G, N*bits/32] int32, same scheme along N (zp and
   qzeros nullable together). Requires K*bits % 32 == 0, and N*bits % 32 == 0
   when zp is given. N*K = 0 is a no-op. */
ar_status ar_pack(int32_t bits, const uint8_t* codes, const uint8_t* zp, int64_t N, int64_t K,
                  int64_t G, int32_t* qweight, int32_t* qzeros, void* stream);

/* Inverse of ar_pack (same shapes and constraints). */
ar_status ar_unpack(int32_t bits, const int32_t* qweight, const int32_t* qzeros, int64_t N,
                    int64_t K, int64_t G, uint8_t* codes, uint8_t* zp, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AUTOROUND_HIP_H */
