/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert-layer library, libmoe.so.
 *
 * One call runs the whole expert layer of a sparse LLM on the GPU:
 *
 *   1. router scores  l[t][e] = sum_i x[t][i] * router_w[e][i], in fp32
 *      ("Muse Spark Open を段階的に分解する" (animemo.app), section ⑧: one
 *      matrix product per token, kept in FP32 because a wrong choice is
 *      costly);
 *   2. top-k experts per token, ordered by score (descending) then expert id
 *      (ascending), weights = softmax over the k chosen scores (section ⑧:
 *      top 8 of 256, no shared expert; section ⑨: outputs weighted by the
 *      router's scores, weights of a token summing to one);
 *   3. grouping of the token slots by expert, a stable counting sort by
 *      (expert, token) (section ⑫: each expert's tokens are gathered and
 *      computed together);
 *   4. per expert, a SwiGLU FFN h = silu(x W_gate^T) * (x W_up^T),
 *      o = h W_down^T on block-scaled 4-bit weights (section ⑨: gate, up and
 *      down matrices; section ⑪: 4-bit values sharing a scale per block,
 *      expanded to BF16 for the multiply);
 *   5. RMS normalisation of every expert output over d, eps inside the
 *      square root, no learned gain (section ⑨: each expert's output is
 *      normalised before the weighted sum);
 *   6. y[t] = sum_j w[t][j] * norm(o[t][j]) and the gated residual
 *      s_out = alpha * x + beta * y with per-dimension alpha, beta
 *      (section ③: s <- alpha*s + beta*(.)), rounded to bf16 (nearest even).
 *
 * All pointers passed to moe_layer_forward are DEVICE pointers on the
 * current HIP device unless stated otherwise; the caller allocates and owns
 * them, including the workspace.  The library allocates no device memory,
 * keeps no pointer to the caller's buffers after returning, and queues all
 * work asynchronously on
 * `stream` (a hipStream_t; NULL = the null stream).  Buffers must stay valid
 * until that work completes.  Calls on distinct workspaces are independent.
 *
 * Status codes: every entry point returns MOE_OK (0) or a negative MOE_ERR_*
 * code and never aborts, prints or throws.  Argument errors are detected
 * before anything is queued.  Faults inside kernels surface as errors of a
 * later HIP synchronisation on the stream.  Weight contents are not checked:
 * an E8M0 scale byte of 0xFF (NaN) gives undefined results.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,      /* a required pointer is NULL                        */
    MOE_ERR_SHAPE = -2,     /* T < 0, d not a positive multiple of 256, F not a
                               positive multiple of 128, E < 1 or E > 1024, k not
                               in [1, E], eps < 0 or not finite, or sizes that
                               overflow int32 indexing                           */
    MOE_ERR_WORKSPACE = -3, /* workspace_bytes below moe_layer_workspace_size()  */
    MOE_ERR_ARCH = -4,      /* current device is not gfx950                      */
    MOE_ERR_HIP = -5,       /* a HIP runtime call or kernel launch failed        */
    MOE_ERR_ALIGN = -6,     /* a device pointer is not 16-byte aligned           */
    MOE_ERR_SCRATCH = -7    /* moe_layer_forward_noalloc: the sizes need more
                               than MOE_STATIC_SCRATCH_BYTES of scratch          */
};

typedef struct moe_dims {
    int32_t T;   /* tokens in this call (0 = no-op)                 */
    int32_t d;   /* token width (hidden size)                       */
    int32_t E;   /* experts                                         */
    int32_t F;   /* expert FFN width                                */
    float eps;   /* RMSNorm epsilon, added to the mean square (1e-6) */
} moe_dims_t;

/* Stages of one forward call, in queue order. */
enum {
    MOE_STAGE_ROUTER = 0,  /* router scores                          */
    MOE_STAGE_TOPK = 1,    /* top-k and softmax weights              */
    MOE_STAGE_GROUP = 2,   /* counting sort by expert, tile list     */
    MOE_STAGE_GEMM1 = 3,   /* gate/up projections + SwiGLU           */
    MOE_STAGE_GEMM2 = 4,   /* down projection + row sums of squares  */
    MOE_STAGE_COMBINE = 5, /* RMSNorm, weighted sum, gated residual  */
    MOE_NUM_STAGES = 6
};

/*
 * Optional copies of the routing decisions (device pointers, any may be
 * NULL; pass NULL for the whole struct in production):
 *   ids     int32 [T][k]  chosen experts, best first
 *   weights fp32  [T][k]  softmax weights, same order
 *   offsets int32 [E+1]   segment start of each expert; offsets[E] = T*k
 *   perm    int32 [T*k]   slot id t*k+j at each grouped position
 *   inv     int32 [T*k]   grouped position of each slot (inverse of perm)
 * and optional timing events (hipEvent_t handles created by the caller, any
 * may be NULL): stage_begin[s] / stage_end[s] are recorded on the stream
 * right before the first and right after the last kernel of stage s.  The
 * gate/up stage is a single kernel and its two events are recorded by that
 * kernel's own dispatch, so they bracket exactly its execution.  With very
 * few tokens (T*k <= 16, E <= 256, d a multiple of 2048) the gate/up kernel does
 * the top-k and the grouping itself, in its prologue: the top-k and group
 * stages then launch nothing, their events bracket no work, and the gate/up
 * events include the routing.
 *   xn      bf16  [T][d]  moe_block_forward only: the normalised rows x_n
 *                         the router and the experts read (ignored by the
 *                         other entry points)
 */
typedef struct moe_debug {
    int32_t *ids;
    float *weights;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv;
    void *stage_begin[MOE_NUM_STAGES];
    void *stage_end[MOE_NUM_STAGES];
    void *xn;
} moe_debug_t;

/*
 * Bytes of device workspace moe_layer_forward needs for these sizes and k.
 * Returns 0 when the sizes are invalid (see MOE_ERR_SHAPE).  The value only
 * depends on (T, d, E, F, k); it grows linearly with T (the largest parts
 * are the grouped intermediates: T*k*F*2 + T*k*d*2 bytes).
 */
size_t moe_layer_workspace_size(const moe_dims_t *dims, int32_t k);

/*
 * Natural MXFP4 expert weights (the input of moe_pack_weights):
 *   codes  uint8, expert e at byte offset e*(3*d*F/2):
 *            gate [F][d/2] | up [F][d/2] | down [d][F/2]
 *          each row holds its K elements as FP4 E2M1 codes, two per byte:
 *          element 2b in the low nibble of byte b, 2b+1 in the high nibble
 *          (sign bit 3, exponent bits 2..1 bias 1, mantissa bit 0)
 *   scales uint8 E8M0, expert e at byte offset e*(3*d*F/32):
 *            gate [F][d/32] | up [F][d/32] | down [d][F/32]
 *          scale byte s multiplies a block of 32 consecutive elements of one
 *          row by 2^(s-127)
 *
 * Rearranges natural weights of E experts (dims->E, d, F; T and eps are not
 * used) into the packed layout moe_layer_forward reads: the same bytes, with
 * each 128-element K chunk of 256 consecutive weight rows stored as one
 * contiguous 16 KB tile ("Muse Spark Open を段階的に分解する", section ⑬:
 * at decode batch sizes the layer time is the read of the expert weights, so
 * the format is chosen for that read).  Exact layout, per expert:
 *   W1 = gate and up, K = d: tiles (nt, kc), nt < F/128, kc < d/128, at byte
 *        (nt*(d/128) + kc)*16384; tile row r (0..255) is feature
 *        f = nt*128 + (r/128)*64 + (r%64) of the up matrix if (r/64) is odd,
 *        else of the gate matrix;
 *   W2 = down, K = F: at byte d*F, tiles (nt, kc), nt < d/256, kc < F/128,
 *        tile row r is output row nt*256 + r;
 *   a tile row is 64 bytes: the codes of K elements 128kc..128kc+127 as four
 *   16-byte blocks of 32 elements, block b stored in slot
 *   b ^ ((r >> 1) & 3);
 *   scales: the same tiles, 1024 bytes each (W2 at byte d*F/16): tile row r
 *   holds the 4 E8M0 bytes of its blocks 4kc..4kc+3 in order.
 * Device pointers, 16-byte aligned, packed buffers of the same sizes as the
 * natural ones and not overlapping them.  Asynchronous on `stream`; weights
 * are packed once and reused by every layer call.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (d, F, E rules of moe_layer_forward),
 * MOE_ERR_ALIGN, MOE_ERR_ARCH, MOE_ERR_HIP.
 */
int moe_pack_weights(const moe_dims_t *dims, const uint8_t *codes, const uint8_t *scales,
                     uint8_t *codes_packed, uint8_t *scales_packed, void *stream);

/*
 * The expert layer, steps 1-6 above.
 *
 *   x               bf16 [T][d], row-major (bf16 = upper 16 bits of fp32)
 *   router_w        fp32 [E][d], row-major
 *   expert_w_packed uint8 [E][3*d*F/2]: the codes in the packed layout
 *                   written by moe_pack_weights
 *   scales          uint8 [E][3*d*F/32]: the E8M0 scales in the packed layout
 *   alpha, beta     fp32 [d]
 *   k               experts per token, 1 <= k <= E
 *   s_out           bf16 [T][d]; may be the same buffer as x (in place)
 *   workspace       device scratch of workspace_bytes, 256-byte aligned
 *   stream          hipStream_t to queue on
 *   debug           optional routing copies (see moe_debug_t) or NULL
 *
 * Every device pointer must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *
 * Deterministic: the same inputs and launch give bitwise identical outputs
 * (no floating-point atomics, fixed reduction orders).
 */
int moe_layer_forward(const moe_dims_t *dims, const void *x, const float *router_w,
                      const uint8_t *expert_w_packed, const uint8_t *scales,
                      const float *alpha, const float *beta, int32_t k, void *s_out,
                      void *workspace, size_t workspace_bytes, void *stream,
                      const moe_debug_t *debug);

/*
 * For callers that cannot allocate device memory at all -- code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc: moe_layer_forward without the workspace argument.  Its
 * intermediate buffers live in a static device array of the library
 * (MOE_STATIC_SCRATCH_BYTES, 32 MiB, 256-byte aligned), one per GPU, part of
 * the library's device code and held until the process ends; the call
 * itself allocates nothing.  32 MiB holds every call whose
 * moe_layer_workspace_size(dims, k) is at most that size: at d = 8192,
 * E = 256, k = 8, F = 2048 up to T = 128 tokens.  Larger sizes return
 * MOE_ERR_SCRATCH before anything is queued.
 *
 * Arguments, errors, determinism and output as moe_layer_forward.  Every
 * call on one GPU uses that GPU's single array, and no kernel reads scratch
 * it has not written in the same call, so consecutive calls on one stream
 * are independent; calls that can overlap on one GPU (two streams, two host
 * threads) race on the array and give undefined results: serialise them.
 */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)

int moe_layer_forward_noalloc(const moe_dims_t *dims, const void *x, const float *router_w,
                              const uint8_t *expert_w_packed, const uint8_t *scales,
                              const float *alpha, const float *beta, int32_t k, void *s_out,
                              void *stream, const moe_debug_t *debug);

/*
 * The 16-block weight format ("Muse Spark Open を段階的に分解する"
 * (animemo.app), section ⑪: the released expert weights share one small
 * scale per 16 values, about 4.5 bits per value).  The pages do not give the
 * scale's encoding; here, as in the published NVFP4 format, it is one FP8
 * E4M3 byte per 16 values (sign bit 7, exponent bits 6..3 with bias 7,
 * mantissa bits 2..0, exponent 0 subnormal: 2^-6 * m/8; the byte 0x7F or
 * 0xFF is NaN and gives undefined results) plus one fp32 scale per matrix.
 * Element value = E2M1 code * E4M3 block scale * matrix scale.
 *
 * Natural layout (the input of moe_pack_weights_nvfp4):
 *   codes    exactly as for moe_pack_weights (expert e at e*(3*d*F/2));
 *   scales16 uint8 E4M3, expert e at byte offset e*(3*d*F/16):
 *              gate [F][d/16] | up [F][d/16] | down [d][F/16]
 *            byte j of a row scales its elements 16j .. 16j+15.
 * Per expert: 3dF/2 + 3dF/16 bytes + 12 (the three matrix scales): at
 * d = 8192, F = 2048 that is 28,311,564 bytes, the page's 28.3 MB.
 *
 * Rearranges E experts' natural weights into the packed layout that
 * moe_layer_forward_nvfp4 reads: the code tiles exactly as
 * moe_pack_weights writes them, and scale tiles of 256 rows x 8 bytes per
 * 128-element K chunk (2048 bytes; W1 tiles (nt, kc) at
 * (nt*(d/128) + kc)*2048, W2's from byte d*F/8 of the expert): tile row r
 * holds the 8 E4M3 bytes of its 16-blocks 8kc .. 8kc+7, in order, and is
 * the same weight row as row r of the code tile.  Device pointers, 16-byte
 * aligned, packed buffers of the natural sizes, not overlapping the inputs.
 * Asynchronous on `stream`.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (d, F, E rules of moe_layer_forward),
 * MOE_ERR_ALIGN, MOE_ERR_ARCH, MOE_ERR_HIP.
 */
int moe_pack_weights_nvfp4(const moe_dims_t *dims, const uint8_t *codes, const uint8_t *scales16,
                           uint8_t *codes_packed, uint8_t *scales_packed, void *stream);

/*
 * The expert layer (steps 1-6 above) on weights in the 16-block format:
 * arguments as moe_layer_forward, with
 *   expert_w_packed, scales16  the packed codes and scale tiles written by
 *                   moe_pack_weights_nvfp4
 *   gscale          fp32 [E][3]: the matrix scales of each expert's gate,
 *                   up and down matrices (device pointer)
 * and the same workspace size (moe_layer_workspace_size).  The pages' own
 * design widens the 4-bit weights for the multiply (section ⑪); here they
 * are widened exactly to fp16 in registers and multiplied with fp16
 * activations (each row of x and of the SwiGLU output carried with its own
 * power-of-two scale; exact except elements below 2^-32 of their row's
 * largest) on the fp16 MFMA with fp32 accumulation.  Deterministic.
 */
int moe_layer_forward_nvfp4(const moe_dims_t *dims, const void *x, const float *router_w,
                            const uint8_t *expert_w_packed, const uint8_t *scales16,
                            const float *gscale, const float *alpha, const float *beta,
                            int32_t k, void *s_out, void *workspace, size_t workspace_bytes,
                            void *stream, const moe_debug_t *debug);

/*
 * Expands `rows` rows of K MXFP4 elements in the natural layout (one matrix
 * of the moe_pack_weights input: codes [rows][K/2], scales [rows][K/32],
 * device pointers) into bf16 out [rows][K] (device), with the conversion the
 * few-token expert kernels use ("Muse Spark Open を段階的に分解する", section ⑪: 4-bit values
 * are expanded to BF16 before the multiply).  Exact for every code and
 * scale bytes 1..252; above that the largest codes exceed the bf16 range and
 * give +-inf.  K must be a positive multiple of 32.
 */
int moe_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t K,
                      void *out_bf16, void *stream);

/*
 * Latent-width variant ("Muse Spark Open を段階的に分解する", section ⑨: the
 * chosen experts do not take the token at its full width; a matrix shared by
 * them narrows it first (8,192 -> 4,096 on the page), each chosen expert
 * runs gate / up / down at that width, and the normalised, router-weighted
 * sum is widened back by a second shared matrix before the gated residual):
 *
 *   1-3. routing and grouping as moe_layer_forward, on the full-width x;
 *   N.   z = x W_narrow^T (bf16 out, fp32 accumulation);
 *   4-5. the experts of moe_layer_forward on z, at width d;
 *   W.   y = sum_j w[t][j] * norm(o[t][j]) rounded to bf16, then
 *        f = y W_widen^T (fp32 accumulation);
 *   6.   s_out = alpha * x + beta * f at width D, rounded to bf16.
 *
 * Reading: the shared matrices are bf16 (the pages give a 4-bit format for
 * the expert weights only, section ⑪); z and y are carried in bf16 like
 * every other activation between kernels.
 *
 *   dims->T, E, F, eps as moe_dims_t; D the token width, d the experts'
 *   width (d takes moe_dims_t's d rules: a positive multiple of 256; D the
 *   same).
 *   x               bf16 [T][D]
 *   router_w        fp32 [E][D]
 *   w_narrow        bf16 [d][D]: z[j] = sum_i w_narrow[j][i] * x[i]
 *   expert_w_packed uint8 [E][3*d*F/2], scales uint8 [E][3*d*F/32]: the
 *                   experts at width d, packed by moe_pack_weights (dims d, F)
 *   w_widen         bf16 [D][d]: f[i] = sum_j w_widen[i][j] * y[j]
 *   alpha, beta     fp32 [D]
 *   s_out           bf16 [T][D]; may be the same buffer as x
 *   workspace       moe_latent_workspace_size bytes, 256-byte aligned
 *   stream, debug   as moe_layer_forward (debug copies and stage events
 *                   refer to the routing and expert stages)
 *
 * The two shared-matrix products run in the library's own kernels (bf16
 * MFMA, fp32 accumulation: a weight-streaming kernel for T <= 8, LDS-tiled
 * 256 x 256 tiles otherwise).  Allocates nothing; same status codes and
 * determinism as moe_layer_forward.
 */
typedef struct moe_latent_dims {
    int32_t T;   /* tokens in this call (0 = no-op)            */
    int32_t D;   /* token width                                */
    int32_t d;   /* experts' width                             */
    int32_t E;   /* experts                                    */
    int32_t F;   /* expert FFN width                           */
    float eps;   /* RMSNorm epsilon (1e-6)                     */
} moe_latent_dims_t;

size_t moe_latent_workspace_size(const moe_latent_dims_t *dims, int32_t k);

int moe_latent_forward(const moe_latent_dims_t *dims, const void *x, const float *router_w,
                       const void *w_narrow, const uint8_t *expert_w_packed,
                       const uint8_t *scales, const void *w_widen, const float *alpha,
                       const float *beta, int32_t k, void *s_out, void *workspace,
                       size_t workspace_bytes, void *stream, const moe_debug_t *debug);

/*
 * The MoE block with its stream norms ("Muse Spark Open を段階的に分解する",
 * section ③: the block reads a normalised copy of the residual stream s,
 * its output is normalised again and mixed in by the gate
 * s <- alpha * s + beta * norm(output)):
 *
 *   P.   x_n = bf16(s * r_s * gamma_pre), r_s = 1/sqrt(mean(s^2) + eps);
 *   1-5. moe_layer_forward's steps on x_n (routing, experts, per-expert norms);
 *   6.   y = sum_j w[t][j] * norm(o[t][j]) (fp32), and
 *        s_out = bf16(alpha * s + beta * y * r_y * gamma_post),
 *        r_y = 1/sqrt(mean(y^2) + eps).
 *
 * Reading: both norms are RMSNorm over d with a learned per-dimension gain
 * and the layer's eps; x_n is handed to the router and the experts in bf16.
 *
 *   dims, k, router_w, expert_w_packed, scales, alpha, beta, s_out,
 *   stream, debug   as moe_layer_forward (x is the stream s)
 *   gamma_pre       fp32 [d], the gain of the norm in front of the block
 *   gamma_post      fp32 [d], the gain of the norm on the block's output
 *   workspace       moe_block_workspace_size bytes, 256-byte aligned
 *
 * Allocates nothing; same status codes and determinism as moe_layer_forward.
 */
size_t moe_block_workspace_size(const moe_dims_t *dims, int32_t k);

int moe_block_forward(const moe_dims_t *dims, const void *x, const float *gamma_pre,
                      const float *router_w, const uint8_t *expert_w_packed, const uint8_t *scales,
                      const float *gamma_post, const float *alpha, const float *beta, int32_t k,
                      void *s_out, void *workspace, size_t workspace_bytes, void *stream,
                      const moe_debug_t *debug);

/* Static, human-readable text for a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
