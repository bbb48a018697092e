/*
 * rl_moe -- routed-expert MoE FFN stage of prompt ingestion on 1.8-2.3-bit block-quantized
 * experts, for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * Operation (Red Lite dev75, "Prompt ingestion" and "Decode"; dev72, "2-row verify"):
 * every token t was routed to k experts; column j of topk_ids/topk_w is the token's j-th
 * selection.  For each token-expert pair (t, j) with expert e = topk_ids[t][j]:
 *     g = Wg_e x_t,   u = Wu_e x_t,   h = silu(g) * u,   y_{t,j} = Wd_e h
 * and the layer output is the weighted sum of the expert outputs taken in selection order:
 *     out_t = sum_{j=0..k-1} topk_w[t][j] * y_{t,j}
 * (the MoE tail of dev75 sums in the row's selection order; the 2-row verify of dev72 keeps
 * every row's own selection order).  Shared experts and the residual are not part of it.
 *
 * Pointer kinds: [dev] device memory, [host] host memory.  Every device buffer is owned by
 * the caller and must stay valid until the stream has passed the call.  The library keeps no
 * mutable device state of its own between calls (per-call tables live in the caller's
 * workspace or in kernel arguments), so calls on different streams need different workspaces.
 * `stream` is a hipStream_t (NULL = the default stream).
 *
 * Errors: a negative status is returned synchronously, before anything is launched, and
 * `out` is then untouched.  An expert id outside [0, E) is only seen on the device: it sets
 * bit 0 of the workspace status flags (read with rl_moe_status after the stream is synced);
 * such a token's output is then unspecified, every other token's is still correct.  The
 * per-pair down outputs y wait for the ordered combine in fp16 under a power-of-two scale per
 * (pair, 64 columns) chosen from their own largest value, so every finite y is kept with fp16's
 * 11 significant bits relative to that maximum (none overflows).
 */
#ifndef RL_MOE_H
#define RL_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RL_OK 0
#define RL_EINVAL (-1)     /* a required pointer is NULL, or qtype / code unknown */
#define RL_ESHAPE (-2)     /* a size is outside the supported set (see each call) */
#define RL_EWORKSPACE (-3) /* workspace NULL, too small, or not 256-byte aligned */
#define RL_EHIP (-4)       /* the HIP runtime reported an error at launch */
#define RL_EQTYPE (-5)     /* the host descriptor copy names an unknown block type */
#define RL_ETOOBIG (-6)    /* the call needs more than a fixed-size resource holds (the no-allocation
                              * scratch buffer, or an expert cache's slots) */

/* Block types.  Both use 256-value blocks that tile a matrix flattened row-major; rows are
 * output features, the input dimension is contiguous.
 *   Q2B (74 B/block): fp16 d | 16 4-bit sub-scales (16 values each, low nibble first) |
 *                     2-bit codes q, value = d * s * (q - 1.5)
 *   T1  (57 B/block): fp16 d | 24-bit word of 8 3-bit sub-scales (32 values each) |
 *                     base-3 digits five per byte, least significant first,
 *                     value = d * s * (digit - 1); digit bytes are 0..242. */
#define RL_QTYPE_Q2B 1
#define RL_QTYPE_T1 2

/* One expert: its block type and the byte offsets of its gate [I x H], up [I x H] and
 * down [H x I] matrices inside the arena. */
typedef struct rl_expert_desc {
    int32_t qtype;
    int32_t reserved;
    uint64_t gate_off;
    uint64_t up_off;
    uint64_t down_off;
} rl_expert_desc;

/* The experts of one layer.  arena [dev]: packed blocks, 4-byte aligned, its allocation a
 * whole number of dwords; arena_bytes its size: every matrix of every expert must lie inside it
 * (offset a multiple of 4, offset + matrix bytes <= arena_bytes; RL_EINVAL otherwise).  desc
 * [dev]: E descriptors (read by the kernels).  desc_host [host]: the same E descriptors (read by
 * the host to decide which type-specialised kernels to launch and to check the offsets); the two
 * copies must agree.  E in [1, 1024].  H (hidden) a multiple of 256 in [256, 8192].  I (expert
 * intermediate) a multiple of 64 in [64, 4096] that is either a multiple of 256 or one of
 * 64 / 128.  Matrix bytes: H * I / 256 blocks of 74 (Q2B) or 57 (T1) bytes.  A T1 digit byte
 * holds five base-3 digits, so it is at most 242; the kernels do not check it (a larger byte
 * decodes as five zero weights), so arenas are to be validated once when they are loaded (the
 * Python binding does so for arenas it copies from host memory). */
typedef struct rl_expert_blobs {
    const void* arena;
    const rl_expert_desc* desc;
    const rl_expert_desc* desc_host;
    int32_t E, H, I;
    uint64_t arena_bytes;
} rl_expert_blobs;

/* Bytes of workspace that rl_moe_prefill / rl_moe_decode / rl_moe_gate_up need for up to
 * T_max tokens with k selections each.  0 if the sizes are outside the supported set, which
 * besides the ranges above requires T * k <= 2^24 and that the kernels' 32-bit buffer offsets
 * cannot wrap: T * 2 * H and T * k * 2 * I bytes (the activation rows of the gate/up and down
 * GEMMs) at most 2^31 - 2^16. */
size_t rl_moe_workspace_bytes(int32_t T_max, int32_t k, int32_t E, int32_t H, int32_t I);

/* Routed-expert layer for T tokens (prompt ingestion).
 *   x        [dev] bf16 bits [T][H]
 *   topk_ids [dev] int32 [T][k], column j = j-th selection (the summation order)
 *   topk_w   [dev] float [T][k]
 *   experts  [host] struct, see above
 *   out      [dev] float [T][H], overwritten
 *   T >= 0 (T = 0 launches nothing), k in [1, 16]
 *   workspace [dev], 256-byte aligned, ws_bytes >= rl_moe_workspace_bytes(T, k, E, H, I).
 * Alignment (RL_EINVAL otherwise): x and out 16-byte aligned, topk_ids and topk_w 4-byte
 * aligned, experts->desc 8-byte aligned (rows of any T-row slice of such buffers stay aligned).
 * Launches: pair grouping, one fused dequant + gate/up + SwiGLU kernel per block type
 * present, one fused dequant + down kernel per type, the ordered combine (in selection order,
 * so out does not depend on the order in which experts finish).  Asynchronous. */
int rl_moe_prefill(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                   const rl_expert_blobs* experts, float* out, int32_t T, int32_t k,
                   void* workspace, size_t ws_bytes, void* stream);

/* The MoE block around the routed experts (dev75 "Prompt ingestion": the prefill profile lists
 * the shared expert beside the routed ones; the block's output joins the residual stream):
 *     out_t = ((sum_{j=0..k-1} topk_w[t][j] * y_{t,j}) + shared_gate[t] * s_t) + residual[t]
 * in that order, where s_t = Wd_s (silu(Wg_s x_t) * (Wu_s x_t)) is the shared expert: descriptor
 * `shared_expert` of experts (a dense SwiGLU FFN of the same shapes and block formats as the
 * routed experts; topk_ids may name it too).  The shared expert runs as one more pair of every
 * token, through the same grouping, GEMMs and ordered combine, summed after the routed pairs.
 *   shared_expert  in [0, E) (RL_EINVAL otherwise)
 *   shared_gate    [dev] float [T]: the per-token weight of the shared expert (the caller's gate,
 *                  e.g. a sigmoid of a projection of x), 4-byte aligned
 *   residual       [dev] float [T][H] or NULL (no residual), 16-byte aligned
 *   k in [0, 15] (k = 0: the shared expert alone; topk_ids / topk_w may then be NULL)
 *   workspace      at least rl_moe_workspace_bytes(T, k + 1, E, H, I) bytes
 * Other arguments, errors and launches as rl_moe_prefill. */
int rl_moe_prefill_block(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                         const rl_expert_blobs* experts, int32_t shared_expert, const float* shared_gate,
                         const float* residual, float* out, int32_t T, int32_t k, void* workspace,
                         size_t ws_bytes, void* stream);

/* The router and the layer in one call: every token's k experts are chosen among experts
 * [0, n_route) from its fp32 logits exactly as rl_moe_route chooses them (its kernel, launched
 * first on the stream) and written to topk_ids / topk_w; then the layer (with shared_expert >= 0
 * the MoE block, as
 * rl_moe_prefill_block; shared_expert < 0: the routed experts only, shared_gate and residual
 * ignored) runs on them.
 *   logits    [dev] float [T][n_route], 4-byte aligned, finite
 *   topk_ids  [dev] int32 [T][k], topk_w [dev] float [T][k]: outputs (the routing), 4-byte aligned
 *   n_route in [1, E]; k in [1, min(16, n_route)], at most 15 with a shared expert
 *   workspace at least rl_moe_workspace_bytes(T, k (+1 with a shared expert), E, H, I) bytes
 * Other arguments and errors as rl_moe_prefill / rl_moe_prefill_block. */
int rl_moe_prefill_from_logits(const uint16_t* x, const float* logits, int32_t n_route,
                               const rl_expert_blobs* experts, int32_t shared_expert, const float* shared_gate,
                               const float* residual, float* out, int32_t* topk_ids, float* topk_w, int32_t T,
                               int32_t k, void* workspace, size_t ws_bytes, void* stream);

/* Measurement hook: rl_moe_prefill with RL_TIMED_EVENTS events (events [host] array of
 * hipEvent_t, created by the caller) recorded on `stream`: 0 before the grouping kernels (whose
 * first launch also splits x for the T1 path), 1 after them, 2 after the gate/up kernel(s), 3
 * after the split of h for the T1 down path, 4 after the down kernel(s), 5 after the combine (an
 * event whose kernel a layer does not use is recorded at the same place as the one before it),
 * so that the caller can time each kernel on the stream the kernels run on.  Otherwise
 * identical to rl_moe_prefill; RL_EINVAL if an event is NULL. */
#define RL_TIMED_EVENTS 6
int rl_moe_prefill_timed(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                         const rl_expert_blobs* experts, float* out, int32_t T, int32_t k,
                         void* workspace, size_t ws_bytes, void* stream, void* const* events);

/* rl_moe_prefill for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): no workspace argument; the library
 * uses a static device buffer of RL_NOALLOC_SCRATCH_BYTES (40 MiB) that each GPU it runs on holds
 * until the process ends, in place of the workspace.  The call itself allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine); its first call on a device looks up that
 * device's copy of the buffer (hipGetSymbolAddress, once per device).  Sizes whose workspace
 * (rl_moe_workspace_bytes) exceeds the buffer are RL_ETOOBIG before any launch: 40 MiB holds a
 * 512-token call of a 512-expert, top-10, H 2048, I 512 layer.  Every call on one GPU shares its
 * buffer: calls that may overlap on one GPU (other streams, other threads) race and must not be
 * made; a call sets up everything it reads from the buffer, so consecutive calls are
 * independent.  The status flags (rl_moe_status) live in the buffer: read them with
 * rl_moe_noalloc_status.  Other arguments, results and errors as rl_moe_prefill. */
#define RL_NOALLOC_SCRATCH_BYTES (40u << 20)
int rl_moe_prefill_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                           const rl_expert_blobs* experts, float* out, int32_t T, int32_t k, void* stream);

/* Status flags of the last rl_moe_prefill_noalloc on the current device (after the stream is
 * synced), as rl_moe_status; RL_EHIP if the buffer was never used on this device. */
int rl_moe_noalloc_status(int32_t* flags_out);

/* The same layer for 1 or 2 rows (decode and 2-row verify; dev75 "Decode", dev72 "2-row
 * verify"): matrix-vector kernels, gate/up + SwiGLU then down + the ordered combine in one
 * dispatch.  T (= rows) must be 1 or 2.  Each row's result is bit-identical to a call with
 * that row alone.  Arguments as rl_moe_prefill; additionally H and I must be multiples of 256
 * whose D/16 columns per lane (16 lanes per row) make few strips of 64, 32 or 16 columns (the
 * largest that divides D/16): H at most 8 strips (any multiple of 1024 up to 8192,
 * 512 x odd up to 3584, 256 x odd up to 1792), I at most 4 (multiples of 1024 up to 4096, 256,
 * 512, 768, 1536); other sizes return RL_ESHAPE. */
int rl_moe_decode(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                  const rl_expert_blobs* experts, float* out, int32_t T, int32_t k,
                  void* workspace, size_t ws_bytes, void* stream);

/* rl_moe_prefill_block for 1 or 2 rows on the matrix-vector kernels (decode and 2-row verify):
 * the shared expert's pair follows each row's routed pairs in its ordered sum, then the residual.
 * Arguments as rl_moe_prefill_block; T and the dimensions as rl_moe_decode.  Each row's result
 * is bit-identical to a call with that row alone. */
int rl_moe_decode_block(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        const rl_expert_blobs* experts, int32_t shared_expert, const float* shared_gate,
                        const float* residual, float* out, int32_t T, int32_t k, void* workspace,
                        size_t ws_bytes, void* stream);

/* Pair grouping alone (parity hook for the first step of rl_moe_prefill).  Pairs (t, j) are
 * ordered by (expert, token, slot):
 *   offsets  [dev] int32 [E+1], exclusive prefix sum of the per-expert pair counts
 *   pair_src [dev] int32 [T*k], t*k + j of the pair at each sorted position
 *   inv      [dev] int32 [T*k], sorted position of pair (t, j); -1 for an invalid id
 *   workspace [dev], 256-byte aligned, at least rl_moe_workspace_bytes(T, k, E, 256, 64)
 *            bytes; an id outside [0, E) sets bit 0 of the status flags (rl_moe_status).
 * T*k <= 2^24, E in [1, 1024]. */
int rl_moe_group_pairs(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                       int32_t* pair_src, int32_t* inv, void* workspace, size_t ws_bytes, void* stream);

/* Block decode alone (parity hook for the in-kernel weight decode): n_values (a multiple of
 * 256) consecutive values of `blocks` [dev] (any byte address) as float d * s * c into out [dev].
 * `decoder` picks which of the library's device decoders runs, exactly as the kernels run it:
 *   RL_DEC_STRIP        the full-table strip decoder of the down kernel for I < 256 (64-value
 *                       strips; operand table with every sub-scale, here in bf16)
 *   RL_DEC_MFMA_GATEUP  the MFMA operand decoder of the gate/up GEMMs (T1: fp8 operands, digit
 *                       selector and fp8 scale tables built on the device; Q2B: bf16 operands);
 *                       value k of a block is written where its operand byte / half stands for
 *   RL_DEC_MFMA_DOWN    the same for the down GEMMs (T1: identical to gate/up; Q2B: fp16 operands)
 *   RL_DEC_ROWS_GATEUP  the decoder of the 1-2 row gate/up kernel: unit operands (bf16) from the
 *                       s = 1 row of the value table, times the strip's sub-scale, times the block
 *                       scale; block b is cut into strips of 64, 32 or 16 values by b % 3 (the
 *                       three strip widths those kernels use)
 *   RL_DEC_ROWS_DOWN    the same with the fp16 unit operands of the 1-2 row down kernel
 * Every such product is exact in fp32, so any correct decode is bit-identical to the format's
 * definition.  RL_EINVAL for an unknown qtype or decoder; RL_ESHAPE if the blocks span more than
 * 2^32 - 16 bytes. */
#define RL_DEC_STRIP 0
#define RL_DEC_MFMA_GATEUP 1
#define RL_DEC_MFMA_DOWN 2
#define RL_DEC_ROWS_GATEUP 3
#define RL_DEC_ROWS_DOWN 4
int rl_moe_dequant(int32_t qtype, int32_t decoder, const void* blocks, int64_t n_values, float* out, void* stream);

/* Grouping + fused dequant/gate/up/SwiGLU alone (parity hook): the launches rl_moe_prefill makes
 * before its down GEMM, with h left where the down GEMM would read it, rows in sorted-pair order
 * (row = sorted position of the pair, as rl_moe_group_pairs orders them):
 *   h16_out [dev] fp16 bits [T*k][I]: the rows of Q2B experts, and of T1 experts when the layer's
 *           T1 gate/up writes fp16 h (I > 512 or I < 256)
 *   h8_out  [dev] bytes [T*k][2*I], hsc_out [dev] uint32 [T*k]: the rows of T1 experts when I is
 *           a multiple of 256 and at most 512.  Then gate/up writes h already split for the fp8
 *           down GEMM: row r holds, for each 256-column block kb, lane group g (0..3) and half hh,
 *           32 bytes hi then 32 bytes lo at byte 512*kb + 256*hh + 64*g (+32 for lo); byte p of
 *           them stands for h column 256*kb + m(g, 32*hh + p), m(g, j) = 60g + j for j < 60, else
 *           240 + 4g + (j - 60); hi and lo are e4m3; byte 2*kb + (g >> 1) of hsc_out[r] is the
 *           E8M0 scale e of that block's lane groups {g, g^1}: h = (hi + lo) * 2^(e - 127).
 * Rows of the other kind are left untouched.  h8_out / hsc_out may be NULL when no row uses
 * them (RL_EINVAL if they are needed); h16_out likewise.  Other arguments as rl_moe_prefill. */
int rl_moe_gate_up(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                   const rl_expert_blobs* experts, uint16_t* h16_out, uint8_t* h8_out, uint32_t* hsc_out,
                   int32_t T, int32_t k, void* workspace, size_t ws_bytes, void* stream);

/* Router, the step before the layer (the MoE routing that the pages take as given; dev72
 * "2-row verify" keeps each row's selection order): for every token t, softmax over the E
 * experts of logits[t], the k most probable experts in descending order, ties to the lower
 * id, and their probabilities renormalised to sum to one (summed in selection order):
 *   logits   [dev] float [T][E]
 *   topk_ids [dev] int32 [T][k], overwritten; column j = the j-th selection
 *   topk_w   [dev] float [T][k], overwritten; p_j / sum_{j'} p_{j'}
 * The probability is strictly increasing in the logit, so the selection compares the fp32
 * logits themselves (decisions exact); the weights are computed in fp32 as
 * exp(l_j - max) / sum_{j' in selection order} exp(l_j' - max).  Logits are finite.
 * T >= 0 (T = 0 launches nothing), E in [1, 1024], k in [1, 16] and k <= E (RL_ESHAPE
 * otherwise); RL_EINVAL if a pointer is NULL or not 4-byte aligned with T > 0.  One kernel,
 * asynchronous. */
int rl_moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                 void* stream);

/* Bounded expert cache (dev72 "The 2-row verify with a bounded expert cache"): the layer's experts
 * stay in host memory and a fixed number of device slots hold the ones the next call needs.  A
 * prepare makes every expert of a request resident at once -- for a 2-row verify, the union of
 * both rows' selections, so that no row's experts are evicted while the other row is in flight --
 * and evicts, for the request's missing experts, the least recently requested experts outside
 * it (free slots first, lowest index first).  Each row then runs with its own selection order
 * (rl_moe_decode / rl_moe_decode_block on the view the prepare returns), bit-identical to a run on
 * the whole resident arena.  The cache object is host memory owned by the library (create /
 * destroy); the slots and the device descriptor table are the caller's device memory.  A cache is
 * used by one host thread at a time. */
typedef struct rl_cache rl_cache;

/* Bytes of one slot: the three matrices of an expert of either block type, each 256-byte
 * aligned; 0 for unsupported H / I. */
uint64_t rl_cache_slot_bytes(int32_t H, int32_t I);

/* host_arena [host]: the layer's packed experts, host_arena_bytes long, laid out per host_desc
 * [host] (E descriptors, offsets into host_arena; copied by the call).  Pinned host memory
 * (hipHostMalloc) lets the copies of prepare run asynchronously; it must stay valid and unchanged
 * for the cache's lifetime.  slots [dev]: n_slots * rl_cache_slot_bytes(H, I) bytes, 256-byte
 * aligned, n_slots in [1, E]; dev_desc [dev]: E descriptors, 8-byte aligned, which the cache keeps
 * naming each expert's slot (experts not resident name slot 0 and must not be routed to).  With
 * slots = NULL (and dev_desc NULL) the cache only plans: residency, hits, misses and evictions are
 * tracked, nothing is copied.  Synchronises the NULL stream once (the initial table).  *out
 * receives the cache; RL_ESHAPE / RL_EINVAL / RL_EQTYPE as the layer calls define them. */
int rl_cache_create(const void* host_arena, uint64_t host_arena_bytes, const rl_expert_desc* host_desc, int32_t E,
                    int32_t H, int32_t I, void* slots, int32_t n_slots, rl_expert_desc* dev_desc, rl_cache** out);

/* Make the experts ids [host] (n ids, duplicates allowed) resident together.  Missing experts are
 * copied from the host arena into their slots and the changed descriptors written to dev_desc, all
 * enqueued on `stream` (calls that use the view must follow on that stream); the descriptor
 * entries travel in kernel arguments, so later prepares never change what an earlier enqueued
 * call reads.  blobs [host] (may be NULL) receives the device view: arena = slots, desc = dev_desc,
 * desc_host = the cache's host copy of the table (valid until the next prepare or destroy), E, H,
 * I, arena_bytes.  RL_ETOOBIG if the request names more distinct experts than there are slots
 * (nothing changes); RL_EINVAL for an id outside [0, E); RL_EHIP if a copy could not be enqueued
 * (the cache must then be destroyed). */
int rl_cache_prepare(rl_cache* cache, const int32_t* ids, int32_t n, rl_expert_blobs* blobs, void* stream);

/* stats [host] int64 [4]: prepares, hits, misses (experts copied in), evictions. */
int rl_cache_stats(const rl_cache* cache, int64_t* stats);

/* Slot holding expert e, or -1 if it is not resident. */
int32_t rl_cache_slot_of(const rl_cache* cache, int32_t e);

void rl_cache_destroy(rl_cache* cache);

/* Device status flags of the last call that used `workspace` [dev]; the caller must have
 * synchronised the stream.  flags_out [host] int32 [4].  Blocking copy. */
int rl_moe_status(const void* workspace, int32_t* flags_out);

/* Text of a status code. */
const char* rl_moe_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* RL_MOE_H */
