/*
 * dap.h -- C ABI of libdap: draft-guided mixed-precision block-sparse attention on MI355X (gfx950).
 *
 * The method is DraftAttention2 ("DraftAttention2: Fast Video Diffusion with Low-Resolution-Guided
 * Mixed-Precision Attention"; newx.sg paper card, Abstract; pchao.org blog, section 方法概览 and the
 * Figure 2 / Figure 3 captions).  One attention layer is four stream-ordered calls:
 *
 *   dap_prepare    reorder video tokens into compact spatial regions with padding, avg/max-pool
 *                  Q and K per region, quantise Q/K (per-block INT8; the 4-bit level as
 *                  per-32-channel MXFP4 or, per fp4_format, NVFP4) and reorder + transpose + pack
 *                  V (bf16 and per-channel FP8 e4m3)
 *                  -- blog section 方法概览 bullets 2 and 4, Figure 3 caption (a) and (b).
 *   dap_draft_rank build the lambda-mixed draft attention map from the pooled descriptors, rank all
 *                  region pairs of each head and assign 16-bit / 8-bit / 4-bit / skip by quota
 *                  -- blog section 方法概览 bullets 1 and 2; paper card AI Summary (shared sort).
 *   dap_attention  attention over the kept blocks in precision order 16 -> 8 -> 4, one kernel
 *                  whose phases update the same running max, running sum and output
 *                  accumulator of each query row -- paper card Abstract; blog section 方法概览
 *                  bullet 4.
 *   dap_restore    put the output back in the original token order, dropping padding
 *                  -- pith.science, DraftAttention abstract (reorder, attend, restore).
 *
 * Conventions
 *   Tensors Q, K, V, out: bf16, [batch, heads, N, D] contiguous, token n = (t*H + y)*W + x.
 *   Regions: region_h rows x region_w columns of one frame; the grid is padded at high y / high x
 *   to multiples of the region size; pad slots are zero and are masked as keys.
 *   Quotas: basis points (1/100 %) of the Nb*Nb region pairs of each (batch, head), in the order
 *   skip, 4-bit, 8-bit, 16-bit; the skip entry is informational (skip = the remainder).  Cut ranks
 *   are cumulative from the top with round-half-up: c16 = round(P*q16), c8 = round(P*(q16+q8)),
 *   c4 = round(P*(q16+q8+q4)) in integer arithmetic, P = Nb*Nb.
 *   Ranking order: draft score descending, then pair index qb*Nb + kb ascending.
 *   Block-map codes: 0 = skip, 1 = 4-bit, 2 = 8-bit, 3 = 16-bit.
 *
 * Memory and ownership
 *   The caller owns every buffer: inputs, output and one workspace of dap_workspace_bytes() bytes.
 *   All pointers passed to the four calls are device pointers (map_out / scores_out too) and must
 *   be 256-byte aligned.  The library allocates nothing and, apart from the static scratch array
 *   of dap_prepare_static_scratch, keeps no global state; calls on different workspaces may run
 *   concurrently.  Work is enqueued on `stream` (0 = null stream)
 *   and the calls return without synchronising; buffers must stay alive until the enqueued work
 *   completes.  The four calls must be issued in the order prepare -> draft_rank -> attention ->
 *   restore on one workspace, in stream order.  The workspace carries a stage word (see
 *   dap_layout.off_stage) that enforces this: dap_prepare sets DAP_STAGE_PREPARED; dap_draft_rank
 *   moves a prepared (or later) workspace to DAP_STAGE_RANKED; dap_attention runs only on a
 *   ranked (or attended) workspace and moves it to DAP_STAGE_ATTENDED; dap_restore copies the
 *   attention output only from an attended workspace.  A call that finds the wrong stage, or a
 *   stage written under another configuration, still returns DAP_OK (the check runs on the
 *   device, in stream order), writes zeros instead of its result (attention: the packed output;
 *   restore: out) and leaves the stage at DAP_STAGE_BROKEN until the next dap_prepare.  The
 *   caller can read the two stage words after synchronising.  dap_draft_rank on an unprepared
 *   workspace ranks whatever the pooled sections hold (its map_out / scores_out copies are then
 *   meaningless) and marks the stage broken.
 *
 * Errors
 *   Host-side validation runs before any HIP call and returns DAP_E_INVALID (null pointer, bad
 *   size, lambda outside [0, 1], negative quota or quota sum above 10000, misaligned pointer,
 *   fp4_format neither DAP_FP4_MXFP4 nor DAP_FP4_NVFP4),
 *   DAP_E_UNSUPPORTED (head_dim not 64/128, region size not 16/64/128 tokens, more than 4096
 *   regions per head) or DAP_E_WORKSPACE (ws_bytes too small).  A failed kernel launch returns
 *   DAP_E_HIP.  Device faults surface at the caller's next synchronisation.  Non-finite inputs
 *   are outside the contract.
 */
#ifndef DAP_H_
#define DAP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DAP_ABI_VERSION 2

/* Stage word values (first 32-bit word of the stage section); the second word is a tag of the
 * configuration that wrote it. */
#define DAP_STAGE_PREPARED 0xDA900001u
#define DAP_STAGE_RANKED 0xDA900002u
#define DAP_STAGE_ATTENDED 0xDA900003u
#define DAP_STAGE_BROKEN 0xDA9000FFu

/* 4-bit operand formats (dap_config.fp4_format). */
#define DAP_FP4_MXFP4 0 /* OCP MXFP4: E2M1 codes, one E8M0 power-of-two scale per 32 channels */
#define DAP_FP4_NVFP4 1 /* E2M1 codes, one E4M3 scale per 16 channels over one fp32 scale per
                          (head, tensor) */

typedef enum {
  DAP_OK = 0,
  DAP_E_INVALID = 1,
  DAP_E_UNSUPPORTED = 2,
  DAP_E_WORKSPACE = 3,
  DAP_E_HIP = 4,
  DAP_E_SCRATCH_LIMIT = 5 /* dap_prepare_static_scratch: batch*heads*head_dim above 65536 */
} dap_status;

typedef struct {
  int32_t batch;        /* >= 1 */
  int32_t heads;        /* >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t T, H, W;      /* latent grid, each >= 1 */
  int32_t region_h;     /* region rows (height) */
  int32_t region_w;     /* region columns (width); region_h*region_w in {16, 64, 128} */
  double lambda;        /* draft-map mix weight of the max-pooled map, in [0, 1] */
  int32_t quota_bp[4];  /* skip, 4-bit, 8-bit, 16-bit, basis points */
  int32_t fp4_format;   /* DAP_FP4_MXFP4 or DAP_FP4_NVFP4 */
} dap_config;

/* Derived sizes and the byte offsets of every workspace section (all 256-byte aligned).
 * Section layouts (bh = batch*heads index, b / qb / kb = region block, p = packed row):
 *   q_bf16, k_bf16  [bh][Np][D] bf16, packed rows p = b*B + iy*region_w + ix
 *   vt_bf16         [bh][Nb][D][B] bf16: V transposed per block, keys of each 16-key chunk stored
 *                   in the order 0-3, 8-11, 4-7, 12-15 (the order the matrix-core operand takes)
 *   q_i8, k_i8      [bh][Np][D] int8 codes;  q_i8_scale, k_i8_scale [bh][Nb] fp32
 *   q_fp4, k_fp4    [bh][Np][D/2] E2M1 codes, two per byte, even channel in the low nibble
 *   q_e8m0, k_e8m0  [bh][Np][D/32] E8M0 exponents (value 2^(byte-127)) per 32-channel group
 *                   (fp4_format MXFP4; with NVFP4, q_fp4 / k_fp4 hold the NVFP4 E2M1 codes)
 *   q_nv_scale, k_nv_scale  [bh][Np][D/16] e4m3fn group scales of NVFP4 (empty for MXFP4)
 *   q_nv_bf16, k_nv_bf16    [bh][Np][D] bf16: NVFP4 values without the tensor scale (E2M1 value x
 *                   group scale, exact in bf16), the operands of the 4-bit Q K^T (empty for MXFP4)
 *   nv_tscale       [bh][2] fp32 NVFP4 tensor scales of Q and K (empty for MXFP4)
 *   qk_amax         [2][bh][D] uint32 (fp32 bits): per-channel maxima of |Q| and |K|, scratch of
 *                   the NVFP4 tensor scale (empty for MXFP4)
 *   vt_fp8          [bh][Nb][D][kp8] e4m3fn codes of V transposed per block, kp8 = B rounded up to
 *                   64; inside each 64-key chunk position 32*g + j holds key
 *                   32*(j/16) + 8*((j%16)/4) + 4*g + j%4; unused positions are 0
 *   v_scale         [bh][D] fp32 per-channel FP8 scale;  v_amax [bh][D] uint32 (fp32 bits)
 *   q_avg, q_max, k_avg, k_max   [bh][Nb][D] fp64 pooled descriptors
 *   scores          [bh][Nb][Nb] fp64 mixed draft map;  lmax [bh][Nb][Nb] fp64 scratch
 *   rank_state, rank_hist        ranking scratch
 *   map             [bh][Nb][Nb] uint8 block map
 *   lists           [bh][Nb][Nb] uint16: per query block, key blocks of level 16, then 8, then 4,
 *                   each ascending
 *   counts          [bh][Nb][4] int32: n16, n8, n4, 0
 *   zeros           256 zero bytes (source of the all-zero key rows a 16-token block pads to)
 *   order           [8][bh * ceil(Nb/8)] uint32 (bh << 16 | qb): attention work order, one slice per
 *                   accelerator die (XCD); each head's rows are ranked by cost and dealt to the
 *                   dies in snake order
 *   out             [bh][Np][D] bf16 attention output in packed order
 *   stage           2 x uint32: stage word (DAP_STAGE_*) and configuration tag */
typedef struct {
  int32_t Hp, Wp, nby, nbx, Nb, B, Np, kp8, bh, D;
  int64_t pairs, c16, c8, c4;
  uint64_t off_q_bf16, off_k_bf16, off_vt_bf16;
  uint64_t off_q_i8, off_k_i8, off_q_i8_scale, off_k_i8_scale;
  uint64_t off_q_fp4, off_k_fp4, off_q_e8m0, off_k_e8m0;
  uint64_t off_vt_fp8, off_v_scale, off_v_amax;
  uint64_t off_q_avg, off_q_max, off_k_avg, off_k_max;
  uint64_t off_scores, off_lmax, off_rank_state, off_rank_hist;
  uint64_t off_map, off_lists, off_counts, off_out, off_zeros, off_order;
  uint64_t off_stage;
  uint64_t off_q_nv_scale, off_k_nv_scale, off_q_nv_bf16, off_k_nv_bf16, off_nv_tscale, off_qk_amax;
  uint64_t total_bytes;
} dap_layout;

/* DAP_ABI_VERSION of the loaded library. */
size_t dap_abi_version(void);

/* Pure host.  *bytes = workspace size for cfg.  Errors: DAP_E_INVALID / DAP_E_UNSUPPORTED. */
dap_status dap_workspace_bytes(const dap_config* cfg, size_t* bytes);

/* Pure host.  Fills *out with derived sizes and section offsets (see dap_layout). */
dap_status dap_workspace_layout(const dap_config* cfg, dap_layout* out);

/* Region reorder + pad, avg/max pooling, INT8 and 4-bit (MXFP4, or NVFP4 per fp4_format)
 * quantisation of Q and K, V reorder, transpose and pack (bf16 and FP8).  q, k, v: device bf16
 * [batch, heads, N, D]; read only.  Formats of a precision whose quota is 0 are not written.
 * NVFP4 (pchao.org blog, section 方法概览 bullet 2, the pages' example 4-bit format): one fp32
 * tensor scale t = amax/2688 per (batch, head, tensor), E4M3 scales per 16 channels
 * s = E4M3(a_16 / 6t), codes E2M1(|x| x 1/(s t)), every step in fp32; the 4-bit Q K^T then runs
 * on the exactly dequantised bf16 values E2M1 x s and applies t_q t_k with the softmax scale
 * (gfx950's scaled matrix-core instructions take power-of-two scales per 32 channels only). */
dap_status dap_prepare(const dap_config* cfg, const void* q, const void* k, const void* v,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dap_prepare with its scratch -- the per-channel maxima
 * of |V| and, when fp4_format is NVFP4, of |Q| and |K|, batch*heads*head_dim 32-bit words each --
 * held in a static device array of the library (3 x 65536 words, 768 KiB, one copy per device,
 * kept until the process ends) instead of the workspace's v_amax and qk_amax sections, which it
 * leaves untouched.  Same arguments, results and errors as dap_prepare, plus DAP_E_SCRATCH_LIMIT
 * when batch*heads*head_dim exceeds 65536.  It allocates
 * nothing: the array's device address is looked up once per device (hipGetSymbolAddress) on the
 * first call made with that device current; `stream` must belong to the current device.  All
 * calls on one device share the array and each clears it before use, so calls that can overlap
 * on one device (other streams, other host threads) race and must be serialised by the caller. */
dap_status dap_prepare_static_scratch(const dap_config* cfg, const void* q, const void* k,
                                      const void* v, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* Draft map (pooled Q K^T / sqrt(D), row softmax over key regions, (1-lambda)*avg + lambda*max),
 * per-head ranking and 4-level block map with per-row key-block lists.  map_out (uint8
 * [batch, heads, Nb, Nb]) and scores_out (fp64, same shape) are optional device copies. */
dap_status dap_draft_rank(const dap_config* cfg, void* ws, size_t ws_bytes, uint8_t* map_out,
                          double* scores_out, hipStream_t stream);

/* Mixed-precision block-sparse attention over the block map; writes the packed output section
 * of the workspace.  16-bit blocks: bf16 Q K^T and bf16 P V; 8-bit: INT8 Q K^T and FP8 e4m3 P V;
 * 4-bit: MXFP4 Q K^T (NVFP4: its exact values contracted in bf16, the tensor scales folded into
 * the softmax scale) and FP8 e4m3 P V.  Phases run 16 -> 8 -> 4, key blocks ascending within a
 * phase, one running-max update per key block; a query block with no kept pair outputs 0. */
dap_status dap_attention(const dap_config* cfg, void* ws, size_t ws_bytes, hipStream_t stream);

/* Diagnostic for profiling the attention kernel: dap_attention (same output, same stage
 * transition, same errors) run by a second instance of its kernel that reads the shader clock
 * (s_memtime) around each part of the key-block loop.  Per precision phase p (0: 16-bit, 1: 8-bit,
 * 2: MXFP4 4-bit, 3: NVFP4 4-bit) it adds, summed over waves, into clocks[8 p + i]:
 *   i = 0  cycles from the start of a key block until its K tile has landed (the wait, and the
 *          bias / scale stores and, for blocks below 128 tokens, the K stores into LDS)
 *       1  in the first barrier
 *       2  in Q K^T, the softmax statistics and the rescale of the output accumulator
 *       3  waiting for the V tile (for blocks below 128 tokens, also storing it into LDS)
 *       4  in the second barrier
 *       5  in P V and the next K tile's load issue
 *       6  wave-blocks counted (one wave of 32 queries against one key block)
 * and clocks[7] the summed lifetimes of the waves, in the same cycles.  clocks: device uint64_t[32],
 * 8-byte aligned, added to (zero it first); DAP_E_INVALID if null or misaligned.  Reading the clock
 * makes this run a few per cent slower than dap_attention. */
dap_status dap_attention_section_clocks(const dap_config* cfg, void* ws, size_t ws_bytes,
                                        uint64_t* clocks, hipStream_t stream);

/* Packed output -> out (device bf16 [batch, heads, N, D]) in the original token order. */
dap_status dap_restore(const dap_config* cfg, const void* ws, size_t ws_bytes, void* out,
                       hipStream_t stream);

/* Static string for a status code. */
const char* dap_status_string(dap_status s);

#ifdef __cplusplus
}
#endif

#endif /* DAP_H_ */
