/*
 * sdpa.h - C ABI of the MI355X (gfx950) memory-efficient scaled-dot-product
 * attention library: a forward that also writes the per-row logsumexp, and a
 * tiled backward that returns dQ, dK and dV at O(L) device memory.
 *
 * What the operations compute
 * ---------------------------
 * For query head h (kv head g = h / group), query row i and key j:
 *   S_ij  = scale * <Q[h,i], K[g,j]>
 *   P_ij  = exp(S_ij - lse_i) on allowed pairs, exactly 0 elsewhere
 *   lse_i = log(sum over allowed j of exp(S_ij))   (natural log)
 *   O[h,i] = sum_j P_ij V[g,j]
 * and the backward is the gradient of sum(dO * O) with respect to Q, K, V,
 * summed over the q-heads of each kv group for dK and dV.
 *
 * The forward also stores each row's logsumexp; the backward rebuilds P from
 * the scores and that stored value one tile at a time, never visits tiles that
 * lie wholly outside the mask's band (above the causal diagonal, behind or,
 * for a two-sided window, ahead of the window), and masks
 * single elements only in the tiles the band's edges cross: page "Lab 028 lab
 * detail: Off NVIDIA, you fix the platform yourself", sections "2026-10-21"
 * ("What the code says") and "What I changed, in plain terms" (items 1, 3,
 * 4). GQA maps q-head h to kv head h / group: page "MiniCPM5 Decode
 * Megakernel - end-to-end build plan (handoff)", section 4.1, stage 5 of the
 * per-layer list.
 *
 * Rows and keys
 * -------------
 * There are Lq query rows and Lk keys; the queries are the LAST Lq of the Lk
 * key positions, so row i's diagonal is key i + off, off = Lk - Lq (the
 * pages' diag_off; Lq == Lk gives off = 0). Masks (allowed pairs (i, j),
 * 0 <= i < Lq, 0 <= j < Lk; d = i + off - j):
 *   SDPA_MASK_NONE           every pair
 *   SDPA_MASK_CAUSAL         d >= 0
 *   SDPA_MASK_CAUSAL_WINDOW  0 <= d < window   (window counts the diagonal:
 *                            window 1 = the diagonal key only; window >= Lk
 *                            is identical to causal)
 *   SDPA_MASK_WINDOW         -window < d < window   (both sides of the
 *                            diagonal, no causal mask: 2 window - 1 keys;
 *                            window >= Lq + Lk is identical to no mask)
 * The non-causal window and queries that are a suffix of the keys are the
 * variants of the same page, "What I changed, in plain terms", items 3-5.
 * A row with no allowed key (Lq > Lk under a causal mask, or Lk == 0) gets
 * O = 0, lse = -inf and dQ = 0, and adds nothing to dK/dV.
 *
 * Layout and ownership
 * --------------------
 * Every tensor pointer is a DEVICE pointer owned by the caller. Tensors are
 * contiguous row-major (the *_ex entry points take any batch / head / row
 * strides instead): Q, O, dO, dQ [B, Hq, Lq, D]; K, V, dK, dV
 * [B, Hq/group, Lk, D]; lse [B, Hq, Lq] float32. Element type: bfloat16
 * (SDPA_BF16), float16 (SDPA_F16) or float32 (SDPA_F32) for Q, K, V, O, dO,
 * dQ, dK, dV; lse is always float32. The 16-bit types run on the matrix
 * cores with fp32 accumulation, S, dP and the softmax state in fp32, and P and
 * dS rounded to the input type as operands; float32 runs in fp32 throughout. Pointers of non-empty tensors must be non-null and 16-byte
 * aligned (pointers of tensors with no elements are not read). Outputs must
 * not alias inputs. The library never allocates device memory: the
 * backward's scratch space is the caller's `workspace` buffer.
 *
 * Execution and errors
 * --------------------
 * Work is enqueued on `stream` (0 = the null stream) and the call returns
 * after the enqueue. There is no global state; calls are thread-safe. All
 * argument checks happen before any launch: on error nothing is launched and
 * no output is touched. Empty problems are valid: B, Hq, Lq or Lk may be 0
 * (the forward then launches nothing when there are no rows; the backward
 * writes zero dK/dV when there are keys but no rows). There is no silent
 * fallback to another algorithm: unsupported combinations return
 * SDPA_ERR_UNSUPPORTED.
 */
#ifndef SDPA_H
#define SDPA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_INVALID_ARG = -1, /* null pointer, negative size, Hq % group != 0,
                                window < 1 with a window mask, scale not
                                finite or <= 0, unknown enum, misaligned ptr */
  SDPA_ERR_UNSUPPORTED = -2, /* valid but not built: D not in {64,128,256,512};
                                Lq + Lk > 2^30; B or Hq > 65535 */
  SDPA_ERR_WORKSPACE = -3,   /* workspace null or smaller than required */
  SDPA_ERR_LAUNCH = -4,      /* the HIP runtime reported a launch error */
  SDPA_ERR_SCRATCH_LIMIT = -5 /* sdpa_bwd_noalloc: the problem needs more
                                scratch than its fixed array holds */
};

enum sdpa_dtype { SDPA_BF16 = 0, SDPA_F32 = 1, SDPA_F16 = 2 };

enum sdpa_mask {
  SDPA_MASK_NONE = 0,
  SDPA_MASK_CAUSAL = 1,
  SDPA_MASK_CAUSAL_WINDOW = 2,
  SDPA_MASK_WINDOW = 3 /* two-sided, not causal */
};

/* Forward. Reads q, k, v; writes o (input dtype, fully overwritten for every
 * row i < Lq) and lse (float32, natural log, one value per query row).
 * `window` is ignored unless mask is SDPA_MASK_CAUSAL_WINDOW or
 * SDPA_MASK_WINDOW. */
int sdpa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                 int32_t dtype, int32_t mask, int32_t window, float scale,
                 hipStream_t stream);

/* Element strides of one tensor seen as [B, H, L, D]: batch, head and row
 * (sequence position). The D elements of a row must be contiguous. */
typedef struct {
  int64_t b, h, l;
} sdpa_strides;

/* Extensions of the *_ex entry points; a NULL extension pointer, or zeroed
 * fields, mean none of them.
 *
 * strides: NULL (every tensor contiguous [B, H, L, D]) or 4 entries for the
 *   forward (q, k, v, o) / 8 for the backward (q, k, v, o, dO, dq, dk, dv), in
 *   that order, for tensors in any layout (e.g. [B, L, H, D] projection
 *   outputs, views into a fused QKV buffer). lse stays contiguous [B, Hq, Lq].
 *   Each stride must be >= 0 and a multiple of 16 bytes' worth of elements,
 *   each row stride at least D and below 2^23 (else SDPA_ERR_INVALID_ARG). K
 *   and V must have the same row stride, and in the backward Q and dO too
 *   (else SDPA_ERR_UNSUPPORTED): true of [B, L, H, D] tensors of one shape and
 *   of views into one fused QKV buffer. Output rows must not overlap.
 * sinks: NULL or a DEVICE array of Hq float32 logits, one per query head,
 *   16-byte aligned: sink h joins every row's softmax normalizer as one more
 *   score with a zero value row, lse_i = log(exp(sinks[h]) + sum_j exp(S_ij)),
 *   so it takes probability mass without adding to O (the pages list sinks
 *   among the backward's parameters: page "Lab 028 lab detail: Off NVIDIA,
 *   you fix the platform yourself", "What I changed, in plain terms", item 2).
 *   -INFINITY is no sink; a row with no allowed key gets lse = sinks[h] and
 *   O = 0. The backward needs the forward's sinks (and its lse).
 * dsinks: backward only, set exactly when sinks is: a DEVICE array of Hq
 *   float32 that receives d sinks[h] = -sum over batches and rows of
 *   exp(sinks[h] - lse_i) Delta_i, Delta_i = <dO_i, O_i> (fully overwritten,
 *   reduced in a fixed order); else SDPA_ERR_INVALID_ARG.
 * cut_row, cut_key_lo, cut_key_hi: a block-sparse cut on top of the mask:
 *   rows i >= cut_row do not see keys cut_key_lo <= j < cut_key_hi
 *   (cut_key_lo == cut_key_hi: no cut; else 0 <= cut_row <= Lq and
 *   0 <= cut_key_lo <= cut_key_hi <= Lk, or SDPA_ERR_INVALID_ARG). With the
 *   sequence [prompt; chosen; rejected], causal mask, cut_row = cut_key_hi =
 *   start of rejected and cut_key_lo = start of chosen, this is the
 *   prefix-sharing mask: the rejected rows never see the chosen tokens, and
 *   one pass equals the two passes [prompt; chosen] and [prompt; rejected]
 *   (page "Training - design (ORPO, flash-CCE head, prefix sharing,
 *   segmented backward)", section 5.4).
 * cut_logical: 0 or 1 (else SDPA_ERR_INVALID_ARG; ignored without a cut).
 *   1: the mask's distances for rows i >= cut_row count positions without
 *   the cut keys: a key j < cut_key_lo sits at j + (cut_key_hi - cut_key_lo)
 *   (the same section's window cut at logical positions, where each
 *   response restarts right after the prompt). With a window, the prefix-
 *   sharing pass then equals the two windowed branch passes; without one
 *   (causal, cut_row >= cut_key_hi) it changes nothing. */
typedef struct {
  const sdpa_strides* strides;
  const float* sinks;
  float* dsinks;
  int32_t cut_row, cut_key_lo, cut_key_hi;
  int32_t cut_logical;
} sdpa_ext;

/* sdpa_fwd_lse with extensions (strided tensors, sinks, block-sparse cut). */
int sdpa_fwd_lse_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                    int32_t dtype, int32_t mask, int32_t window, float scale,
                    const sdpa_ext* ext, hipStream_t stream);

/* Bytes of workspace with which sdpa_fwd_lse_ws splits the key range of each
 * query tile over 2 or 4 workgroups (0: it would not split). The split
 * applies to 16-bit calls whose query tiles (128 rows, 64 at D = 512, per
 * batch and q-head) number at most 128, so that the GPU's 256 CUs would
 * otherwise sit partly idle: 2 shares, or 4 when they number at most 64,
 * while the longest query tile still spans two key tiles (64 keys, 32 at
 * D = 512) per share. Each workgroup keeps the online softmax over its own key range
 * and writes fp32 partial rows (unnormalised O, used max, row sum); a combine
 * pass merges them into O and lse. nseg * B * Hq * Lq * (D + 2) float32, so
 * linear in Lq. Returns 0 for invalid arguments. (A throughput choice, not
 * part of the pages' method; the result equals the unsplit call's up to fp32
 * rounding of the merge.) */
size_t sdpa_fwd_workspace_bytes(int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                                int32_t dtype, int32_t mask, int32_t window);

/* sdpa_fwd_lse with a caller-provided device workspace (non-null and 16-byte
 * aligned when workspace_bytes > 0, else SDPA_ERR_WORKSPACE; null with
 * workspace_bytes 0 is sdpa_fwd_lse): with at least
 * sdpa_fwd_workspace_bytes(...) bytes the split above runs, otherwise the
 * call is sdpa_fwd_lse's. Contiguous tensors only (the strided, sink and cut
 * forms are sdpa_fwd_lse_ex's). The workspace's contents on entry do not
 * matter and are clobbered; calls that share it must be stream-ordered. */
int sdpa_fwd_lse_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes,
                    int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                    int32_t dtype, int32_t mask, int32_t window, float scale, hipStream_t stream);

/* Bytes of caller-provided workspace sdpa_bwd needs for this shape: the row
 * terms Delta_i = <dO_i, O_i>, one float32 per query row ([B, Hq, Lq]),
 * rounded up to 256 bytes. Linear in Lq. Returns 0 for empty shapes and for
 * invalid arguments. */
size_t sdpa_bwd_workspace_bytes(int32_t B, int32_t Hq, int32_t Lq, int32_t D, int32_t dtype);

/* Bytes of workspace with which sdpa_bwd / sdpa_bwd_ex run their fastest
 * plan for this shape and mask (mask and window as for sdpa_fwd_lse): the
 * bytes above, plus the larger of
 *  - the small-problem split: for 16-bit inputs with D <= 256 whose key
 *    blocks (128 keys per kv head and batch) number fewer than 256, fp32
 *    shares of dK and dV (2 * n * B * (Hq/group) * Lk * D floats, n in
 *    {2, 4, 8}) that the query range of each key block is split over, summed
 *    afterwards in a fixed order;
 *  - the dS band buffer: for 16-bit inputs at D = 256 with at least 256 key
 *    blocks, when every block of 128 query rows sees keys in at most
 *    nkb <= 36 tiles of 64 (a band at most 9 D = 2304 keys wide: sliding
 *    windows up to about 2150 keys, the two-sided window up to about 1080),
 *    B * Hq * ceil(Lq / 128) * nkb tiles of
 *    64 x 128 16-bit values. The dK/dV pass then also writes dS for the band
 *    and dQ = scale * dS K is formed from it, instead of a dQ pass that
 *    recomputes the scores (page "Lab 028 lab detail: Off NVIDIA, you fix the
 *    platform yourself", section "What I changed, in plain terms", item 5(a):
 *    dQ summed over the key tiles). At most 9 times the bytes of q, and
 *    linear in Lq at a fixed window; used only while the part of one kv
 *    head's q-heads (group * ceil(Lq / 128) * nkb tiles) stays under 2 GiB;
 *  - when there is no band buffer, the dQ pass's key-range split: the same
 *    split and condition as sdpa_fwd_workspace_bytes, with fp32 dQ partials
 *    (nseg * B * Hq * Lq * D float32) summed by a combine pass; they share
 *    their memory with the dK/dV shares, which are written after that pass.
 * All of them apply to calls with contiguous tensors and no cut, and only when the
 * workspace given holds them; with sdpa_bwd_workspace_bytes(...) bytes the
 * results are the same up to fp32 summation order. Returns 0 for empty
 * shapes and invalid arguments. (Both are throughput choices, not part of
 * the pages' method.) */
size_t sdpa_bwd_workspace_bytes_ex(int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                                   int32_t dtype, int32_t mask, int32_t window);

/* Backward. Reads q, k, v, o, dO and lse as written by sdpa_fwd_lse for the
 * same arguments; writes dq [B, Hq, Lq, D] and dk, dv [B, Hq/group, Lk, D] in
 * the input dtype, every element fully overwritten (keys no query attends get
 * exact zeros). `workspace` is device memory of at least
 * sdpa_bwd_workspace_bytes(...) bytes (it may be null when that is 0); its
 * contents on entry do not matter and are clobbered. Calls that share a
 * workspace must be stream-ordered. */
int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
             int32_t dtype, int32_t mask, int32_t window, float scale,
             hipStream_t stream);

/* sdpa_bwd with extensions: the same sdpa_ext as the forward (with dsinks
 * when there are sinks, and the cut and mask the forward used). */
int sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes,
                int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                int32_t dtype, int32_t mask, int32_t window, float scale,
                const sdpa_ext* ext, hipStream_t stream);

/* Measurement variant of sdpa_bwd: identical arguments and results, plus an
 * array of four caller-created HIP events (or null: same as sdpa_bwd; a null
 * entry: SDPA_ERR_INVALID_ARG). They are recorded on `stream` before the
 * first kernel and after each of the backward's three passes, so
 * hipEventElapsedTime between neighbours gives each pass's duration:
 *   events[0] -> [1]: the dQ pass (which also forms Delta), or, with the dS
 *                     band buffer, the Delta pass;
 *   events[1] -> [2]: the key-stationary dK/dV pass (with its share reduce
 *                     when split; with the band buffer it also writes dS);
 *   events[2] -> [3]: with the band buffer the dQ = scale dS K pass, else
 *                     nothing.
 * (float32: [0] -> [1] the dQ kernel, [1] -> [2] the dK/dV kernel.) The
 * events stay owned by the caller. */
int sdpa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                   int32_t dtype, int32_t mask, int32_t window, float scale,
                   hipStream_t stream, const hipEvent_t* events);

/* Size of the fixed scratch array behind sdpa_bwd_noalloc (64 MiB). */
#define SDPA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Backward that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments as sdpa_bwd minus
 * the workspace, same results: its scratch is a fixed device array of
 * SDPA_NOALLOC_SCRATCH_BYTES per GPU, held by the library until the process
 * ends (its address is looked up on the first call on each device, with that
 * device current; the stream must belong to the current device). Problems
 * whose Delta rows (4 * B * Hq * Lq bytes) exceed it return
 * SDPA_ERR_SCRATCH_LIMIT before anything is launched; the small-problem split
 * and the dS band buffer (see sdpa_bwd_workspace_bytes_ex) are used only when
 * they fit as well. Nothing in the array needs clearing between calls (every
 * pass writes what a later pass reads). All calls on one GPU share the array:
 * calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race and must not be issued; stream-ordered calls are
 * safe. No hipMalloc, hipFree or allocating library call is made. */
int sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     int32_t B, int32_t Hq, int32_t group, int32_t Lq, int32_t Lk, int32_t D,
                     int32_t dtype, int32_t mask, int32_t window, float scale,
                     hipStream_t stream);

/* Static description of a status code. */
const char* sdpa_status_string(int status);

/* ABI version of this header (major * 100 + minor): 500. */
int sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H */
