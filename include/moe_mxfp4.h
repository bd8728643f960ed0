/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer with MXFP4
 * expert weights.
 *
 * The layer (txtmix.com article "DeepSeek V4 Flash 单卡 MI300X", §1, §3 and §9;
 * aihot.vn README translation, section "Định tuyến MXFP4") routes each of T
 * tokens to k of E experts, builds the token x expert bit matrix, groups the
 * (token, expert) slots by expert, runs every expert's two-layer FFN on its
 * rows, and sums each token's k expert outputs with the routing weights:
 *
 *   moe_route              -> topk_ids, topk_weights
 *   moe_build_bitmatrix    -> bitmatrix
 *   moe_expert_offsets     -> counts, offsets, gather, scatter
 *   moe_grouped_ffn_mxfp4  -> y_sorted   (W1 gate|up, clamped SwiGLU, W2)
 *   moe_combine            -> y
 * moe_route_and_group runs the first three as one call (one launch for small T);
 * moe_forward_mxfp4 runs all five.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer (memory the GPU can read or
 *     write) owned by the caller; the library keeps no reference after return.
 *   - Every call only enqueues work on `stream` (a hipStream_t passed as void*;
 *     NULL means the null stream) and returns without synchronising.  Calls
 *     never allocate device memory; scratch memory is the caller's workspace.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns an error code and enqueues nothing.  A launch failure
 *     returns MOE_ERR_HIP.  A fault inside a kernel surfaces at the caller's
 *     next synchronisation, as for any asynchronous GPU work.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics anywhere).
 *   - The library holds no state; calls are reentrant.  Two calls that share
 *     an output or workspace buffer must not run concurrently.
 *   - Sizes: T >= 0 tokens, E experts (1..1024), k experts per token (1..8,
 *     k <= E), hidden size H and expert intermediate size I (multiples of 128,
 *     at most 65536).  T*k must fit in int32, and for the FFN each of T*H,
 *     T*k*I and T*k*H bf16 values must fit in 3.5 GiB.
 *   - Row-major layouts throughout; "bf16" buffers hold bfloat16 bit patterns.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* negative T, k < 1, k > E, null pointer, ... */
  MOE_ERR_UNSUPPORTED = 2,        /* E > 1024, k > 8, H or I not a multiple of 128 or above
                                     65536, H = I = 65536 (one expert's W1 codes would reach
                                     4 GiB), T*k > INT32_MAX, activations above 3.5 GiB */
  MOE_ERR_MISALIGNED = 3,         /* a buffer is not aligned as its call requires */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4,
  MOE_ERR_HIP = 5                 /* the HIP runtime rejected a launch */
} moe_status;

/*
 * moe_route -- top-k selection over router logits and the routing weights.
 *
 * Defined by the routing step of the txtmix.com article, §3 ("fast DeepSeek
 * routing": each token picks its top-6 of 256 experts, §1).  Per token t:
 * topk_ids[t][0..k-1] are the k experts with the largest logits, listed by
 * logit descending; equal logits are ordered by expert index ascending, so the
 * lower index wins a tie at the boundary, and -0.0 counts as equal to +0.0.
 * topk_weights[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k chosen
 * logits (softmax over the selection), in fp32.
 *
 *   logits        fp32  [T][E]   must be finite (NaN order is unspecified)
 *   topk_ids      int32 [T][k]   out
 *   topk_weights  fp32  [T][k]   out
 * T = 0 enqueues nothing.  logits must be 4-byte aligned.
 */
moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_build_bitmatrix -- the token x expert routing bit matrix.
 *
 * The txtmix.com article, §3, and the aihot.vn README translation, section
 * "Định tuyến MXFP4": the kernel's lanes are padded past the logical block of
 * (token, slot) entries that each wavefront owns, and those padding lanes must
 * be masked by the logical block size as well as by the global bound; masking
 * them by the global bound alone lets them inject entries that are not theirs.
 * Output: bit (e % 32) of word (e / 32) of row t is set iff expert e is among
 * topk_ids[t][*]; every other bit (including bits for e >= E in the last word)
 * is zero.  Every word of every row is written, so the buffer needs no clearing.
 *
 *   topk_ids   int32  [T][k]           expert ids in [0, E), distinct per row
 *                                      (ids outside [0, E) are ignored)
 *   bitmatrix  uint32 [T][(E+31)/32]   out
 * T = 0 enqueues nothing.
 */
moe_status moe_build_bitmatrix(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k,
                               uint32_t* bitmatrix, void* stream);

/*
 * moe_expert_offsets -- expert histogram, exclusive prefix sum, and the
 * gather / scatter permutations between token order and expert-major order.
 *
 * The grouped-expert step that the deployment's README (mynewscn.com
 * translation) assigns to the Triton OGS kernels: rows are grouped by expert
 * before the expert products.
 *   counts[e]    number of tokens that chose expert e (bit matrix column sum)
 *   offsets[e]   sum of counts[0..e-1]; offsets[E] = T*k
 *   gather[p]    slot id t*k + j of the p-th row in expert-major order: experts
 *                ascending, tokens ascending within an expert
 *   scatter[s]   the position p with gather[p] == s (inverse permutation)
 *
 *   bitmatrix  uint32 [T][(E+31)/32]   as written by moe_build_bitmatrix
 *   topk_ids   int32  [T][k]           the ids the bit matrix was built from
 *   counts     int32  [E]      out
 *   offsets    int32  [E+1]    out
 *   gather     int32  [T*k]    out
 *   scatter    int32  [T*k]    out
 *   ws         workspace of at least moe_workspace_bytes(T, E, k, H, I) bytes
 *              (any H, I), 16-byte aligned; contents on entry are ignored.
 * T = 0 writes zeros to counts and offsets.
 */
moe_status moe_expert_offsets(const uint32_t* bitmatrix, const int32_t* topk_ids, int64_t T,
                              int32_t E, int32_t k, int32_t* counts, int32_t* offsets,
                              int32_t* gather, int32_t* scatter, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * moe_grouped_ffn_mxfp4 -- every expert's FFN on its rows, in expert-major order.
 *
 * MXFP4 weights (txtmix.com article, §1 and §3): 4-bit E2M1 elements with one
 * E8M0 scale per 32 consecutive elements along the reduction dimension (OCP MX
 * v1.0; element value E2M1(code) * 2^(s - 127), s = 255 decodes to NaN).  In a
 * packed row, element 2i is the low nibble of byte i and element 2i+1 the high
 * nibble.  The clamped SwiGLU is the txtmix.com article, §9: the gate is capped
 * at +limit and the up projection clamped to [-limit, +limit] before the
 * product (limit 10 for the checkpoint the pages run).
 *
 * For expert e and each row p in [offsets[e], offsets[e+1]), with token
 * t = gather[p] / k:
 *   g = x[t] . W1[e][i],  u = x[t] . W1[e][I+i]          (i < I; fp32 accumulation)
 *   h[p][i] = SiLU(min(g, limit)) * clamp(u, -limit, limit),  SiLU(z) = z / (1 + e^-z)
 *   y_sorted[p][n] = h[p] . W2[e][n]                      (n < H; fp32 accumulation)
 * h is held in the workspace as bf16; y_sorted is written as bf16.  A limit
 * <= 0 or not finite disables the clamp.
 *
 *   x         bf16  [T][H]            16-byte aligned
 *   w1        uint8 [E][2I][H/2]      W1 codes; rows 0..I-1 gate, I..2I-1 up; 16-byte aligned
 *   w1_scale  uint8 [E][2I][H/32]     E8M0 scales of W1; 16-byte aligned
 *   w2        uint8 [E][H][I/2]       W2 codes; 16-byte aligned
 *   w2_scale  uint8 [E][H][I/32]      E8M0 scales of W2; 16-byte aligned
 *   counts, offsets, gather           as written by moe_expert_offsets
 *   y_sorted  bf16  [T*k][H]          out; 16-byte aligned
 *   ws        workspace of at least moe_workspace_bytes(T, E, k, H, I) bytes,
 *             16-byte aligned; contents on entry are ignored.
 * T = 0 enqueues nothing.
 */
moe_status moe_grouped_ffn_mxfp4(const uint16_t* x, int64_t T, int32_t H, int32_t I,
                                 int32_t E, int32_t k, const uint8_t* w1,
                                 const uint8_t* w1_scale, const uint8_t* w2,
                                 const uint8_t* w2_scale, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* gather,
                                 float swiglu_limit, uint16_t* y_sorted, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * moe_combine -- weighted sum of each token's k expert outputs, back in token order.
 *
 * y[t][n] = sum over j = 0..k-1 of topk_weights[t][j] * y_sorted[scatter[t*k+j]][n],
 * accumulated in fp32 in j order and rounded once to bf16 (nearest, ties to even).
 *
 *   y_sorted      bf16  [T*k][H]   16-byte aligned
 *   topk_weights  fp32  [T][k]
 *   scatter       int32 [T*k]      as written by moe_expert_offsets
 *   y             bf16  [T][H]     out; 16-byte aligned
 * H must be a positive multiple of 8.  T = 0 enqueues nothing.
 */
moe_status moe_combine(const uint16_t* y_sorted, const float* topk_weights,
                       const int32_t* scatter, int64_t T, int32_t H, int32_t k, uint16_t* y,
                       void* stream);

/*
 * moe_route_and_group -- the routing front-end in one call: exactly the outputs of
 * moe_route, moe_build_bitmatrix and moe_expert_offsets on the same arguments
 * (see those calls for each output's definition, layout and citation).
 *
 * For T <= 64 the three steps run as one kernel launch (one workgroup; the
 * bit matrix is built in LDS under the same logical-block mask); for larger T
 * the routing kernel also writes each token's bit-matrix row (one wavefront
 * per token: lane w writes word w), then the expert-offsets kernels of the
 * separate call run.  ws is the
 * workspace of moe_expert_offsets.  T = 0 writes zeros to counts and offsets.
 */
moe_status moe_route_and_group(const float* logits, int64_t T, int32_t E, int32_t k,
                               int32_t* topk_ids, float* topk_weights, uint32_t* bitmatrix,
                               int32_t* counts, int32_t* offsets, int32_t* gather,
                               int32_t* scatter, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_mxfp4 -- the whole layer in one call: exactly the outputs of
 * moe_route_and_group, moe_grouped_ffn_mxfp4 and moe_combine on the same
 * arguments (see those calls for each output's definition, layout, alignment
 * and citation).  The FFN's row-tile plan is written by the routing side where
 * it holds the counts in one workgroup -- the one-launch front-end for T <= 64,
 * the expert-offsets kernel for 64 < T <= 512, the expert-offsets scan above --
 * which saves the FFN its plan launch.  On the decode GEMV path (T*k < E, H and
 * I each 2048 or 4096) the W2 launch also computes y, with the combine's
 * arithmetic (fp32 sum in slot order, one bf16 rounding), which saves the combine
 * launch; the outputs are the same bits.  ws is the workspace of those calls
 * (moe_workspace_bytes).  T = 0 writes zeros to counts and offsets and nothing
 * else.
 */
moe_status moe_forward_mxfp4(const float* logits, const uint16_t* x, int64_t T, int32_t H,
                             int32_t I, int32_t E, int32_t k, const uint8_t* w1,
                             const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                             float swiglu_limit, int32_t* topk_ids, float* topk_weights,
                             uint32_t* bitmatrix, int32_t* counts, int32_t* offsets,
                             int32_t* gather, int32_t* scatter, uint16_t* y_sorted, uint16_t* y,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_mxfp4_noalloc -- moe_forward_mxfp4 for callers that cannot
 * allocate device memory: code under HIP stream capture, tight serving loops,
 * harnesses that forbid the allocator.  Same arguments, outputs, checks and
 * kernels as moe_forward_mxfp4, minus the workspace: the library uses its own
 * static device scratch of MOE_NOALLOC_SCRATCH_BYTES instead (one copy per GPU,
 * held until the process ends; the call itself allocates nothing).
 *   - Sizes whose moe_workspace_bytes(T, E, k, H, I) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE_TOO_SMALL and enqueue
 *     nothing (at E = 256, k = 6, H = 4096, I = 2048: up to T = 4032 tokens).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (no kernel needs it cleared).  Calls that overlap on one
 *     GPU (other streams, other threads) race; serialise them.
 *   - The first call on a GPU looks up the scratch's device address there (a
 *     HIP symbol query, no allocation); MOE_ERR_HIP if that fails.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

moe_status moe_forward_mxfp4_noalloc(const float* logits, const uint16_t* x, int64_t T,
                                     int32_t H, int32_t I, int32_t E, int32_t k,
                                     const uint8_t* w1, const uint8_t* w1_scale,
                                     const uint8_t* w2, const uint8_t* w2_scale,
                                     float swiglu_limit, int32_t* topk_ids, float* topk_weights,
                                     uint32_t* bitmatrix, int32_t* counts, int32_t* offsets,
                                     int32_t* gather, int32_t* scatter, uint16_t* y_sorted,
                                     uint16_t* y, void* stream);

/*
 * Workspace bytes that moe_expert_offsets and moe_grouped_ffn_mxfp4 need for
 * these sizes (one buffer of this size serves both calls, used one at a time,
 * and moe_route_and_group and moe_forward_mxfp4).
 * Returns 0 for invalid sizes.  Pure host function.
 */
size_t moe_workspace_bytes(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/* A static, human-readable name for a status code.  Pure host function. */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
