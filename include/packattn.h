/*
 * packattn.h -- C ABI of libpackattn.so: packed segment-id masked attention
 * (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Several variable-length episodes are packed into one
 * sequence; every token carries a segment id.  A query attends only to keys
 * with the same id, and a negative id (padding frames past an episode's valid
 * frames get -1) removes the token both as query and as key
 * ("Furniture packing, variable length" report, implementation part;
 * "LingBot-VA packing" report, section 2.1).  Rows with no allowed key come
 * out as exact zeros with LSE = -inf, never NaN ("LingBot-VA packing" report,
 * section 3.1 table).  The mask is built once, as per-tile block sparsity, and
 * shared by forward and backward; a forward of another shape between the two
 * must not silently corrupt the backward (same report, section 2.2), so both
 * passes take the mask descriptor explicitly and check it.
 *
 * Conventions for every entry point:
 *   - returns an int32 status: PA_OK (0) or a negative PA_ERR_* code;
 *   - never allocates device memory, never synchronizes the device; all work
 *     is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *   - every device buffer is owned by the caller; the library keeps no state
 *     between calls and is safe to call from several host threads;
 *   - argument errors are detected on the host before anything is launched;
 *     a failed launch returns PA_ERR_HIP;
 *   - tensors are contiguous row-major: q, o, dout, dq are [nq][heads][head_dim],
 *     k, v, dk, dv are [nkv][heads][head_dim]; lse is [heads][nq] fp32.
 *     Pointers to tensors must be 16-byte aligned.
 */
#ifndef PACKATTN_H
#define PACKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,          /* a required pointer is NULL                          */
  PA_ERR_SHAPE = -2,         /* a size is out of range                              */
  PA_ERR_DTYPE = -3,         /* unknown pa_dtype                                    */
  PA_ERR_HEADDIM = -4,       /* head_dim not supported (64 or 128)                  */
  PA_ERR_MASK_MISMATCH = -5, /* mask descriptor does not fit this call              */
  PA_ERR_WORKSPACE = -6,     /* caller storage / workspace too small                */
  PA_ERR_HIP = -7,           /* a HIP launch failed                                 */
  PA_ERR_ALIGN = -8          /* a tensor pointer is not 16-byte aligned             */
};

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_str(int32_t status);

/*
 * seq_ids_from_valid_frames -- per-token segment ids of a frame-padded pack
 * ("LingBot-VA packing" report, section 2.1: frames at or past
 * valid_frames[b] get -1, the other tokens of episode b get b).
 *
 *   valid_frames      device int32[B]; entries are clamped to [0, frames_padded]
 *   B                 number of episodes, >= 0 (0 writes nothing)
 *   frames_padded     padded frame count per episode, >= 1
 *   tokens_per_frame  tokens per frame, >= 1
 *   seq_id            device int32[B * frames_padded * tokens_per_frame], written;
 *                     token order is episode, then frame, then token
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, or more than 2^31-1 tokens).
 */
int32_t seq_ids_from_valid_frames(const int32_t* valid_frames, int32_t B, int32_t frames_padded,
                                  int32_t tokens_per_frame, int32_t* seq_id, void* stream);

/*
 * Unpadded packing ("LingBot-VA attention profiling" report, conclusion and
 * next steps: concatenate several episodes along the sequence axis, each token
 * tagged with its document id; "LingBot-VA packing" report, section 1: fill
 * the per-GPU token budget of about 68k tokens).
 *
 * plan_token_packs -- HOST function: assigns episodes, in the given order, to
 *   packs of at most `budget` tokens, next-fit (a pack is closed when the next
 *   episode would overflow it; that episode opens the next pack).
 *     lengths  host int32[B], tokens per episode, each in [0, budget]
 *     pack_of  host int32[B], written: pack index of each episode (0, 1, ...)
 *     n_packs  host int32, written: number of packs (0 when B = 0)
 *   Errors: PA_ERR_SHAPE (B < 0, budget < 1, a length outside [0, budget]),
 *           PA_ERR_NULL.
 *
 * seq_ids_from_lengths -- ids of one unpadded pack: episode e (0-based, in
 *   order) takes the next max(lengths[e], 0) tokens and gives them id e;
 *   positions past the last episode get -1; tokens past n_tokens are cut.
 *     lengths   device int32[B], B in [0, 8192]
 *     n_tokens  length of the id buffer (a fixed shape; >= 0)
 *     seq_id    device int32[n_tokens], written
 *     offsets   device int32[B + 1] or NULL; if given, written with each
 *               episode's first token (clamped to n_tokens) and, last, the
 *               number of tokens that carry an id
 *   Errors: PA_ERR_SHAPE, PA_ERR_NULL, PA_ERR_HIP.
 */
int32_t plan_token_packs(const int32_t* lengths, int32_t B, int64_t budget, int32_t* pack_of,
                         int32_t* n_packs);
int32_t seq_ids_from_lengths(const int32_t* lengths, int32_t B, int32_t n_tokens,
                             int32_t* seq_id, int32_t* offsets, void* stream);

/*
 * Block mask: the per-tile sparsity of the same-id predicate
 * ("LingBot-VA packing" report, sections 1 and 2.2: a block mask built from the
 * seq ids; blocks without an allowed pair are skipped).
 *
 * The query axis is cut into nq_tiles = ceil(nq/block_q) tiles and the key axis
 * into nkv_tiles = ceil(nkv/block_kv) tiles; the last tile of an axis may be
 * short.  tile_class[i*nkv_tiles + j] is 0 (empty: no allowed pair), 2 (full:
 * all block_q*block_kv positions are allowed pairs; a short tile never is) or
 * 1 (partial).  The CSR lists hold the non-empty tiles in ascending order:
 * key tiles of query tile i are q_cols[q_ptr[i] .. q_ptr[i+1]), query tiles of
 * key tile j are kv_rows[kv_ptr[j] .. kv_ptr[j+1]).  q_order / kv_order list
 * the tiles by decreasing list length (ties by ascending index); the attention
 * kernels use them to start the longest work first.
 *
 * Pair lists: the query tiles at positions 2w and 2w + 1 of q_order form pair
 * w (w < ceil(nq_tiles / 2); the last pair of an odd count has one tile).
 * pair_ent[pair_off[w] .. pair_off[w] + pair_len[w]) lists, ascending, every
 * key tile kt that either tile of the pair has an allowed pair with, as
 * kt | class(first, kt) << 16 | class(second, kt) << 24 (class 0 for a tile
 * outside that tile's list, and for a missing second tile).  pair_off[w] is
 * the exclusive prefix sum over pairs of the two tiles' list lengths (room for
 * the union; pair_off[last + 1] is the total).  The paired attention kernels
 * walk these lists, so they visit exactly the key tiles with work.
 *
 * All pointers in the descriptor point into the caller's `storage` buffer; the
 * descriptor itself is host memory, filled by build_block_mask.
 */
typedef struct pa_block_mask {
  int32_t nq, nkv, block_q, block_kv, nq_tiles, nkv_tiles;
  uint8_t* tile_class; /* device [nq_tiles * nkv_tiles]                         */
  int32_t* q_ptr;      /* device [nq_tiles + 1]                                 */
  int32_t* q_cols;     /* device, capacity nq_tiles * nkv_tiles                 */
  int32_t* kv_ptr;     /* device [nkv_tiles + 1]                                */
  int32_t* kv_rows;    /* device, capacity nq_tiles * nkv_tiles                 */
  int32_t* q_order;    /* device [nq_tiles]                                     */
  int32_t* kv_order;   /* device [nkv_tiles]                                    */
  int32_t* pair_off;   /* device [ceil(nq_tiles / 2) + 1]                       */
  int32_t* pair_len;   /* device [ceil(nq_tiles / 2)]                           */
  int32_t* pair_ent;   /* device, capacity nq_tiles * nkv_tiles                 */
} pa_block_mask;

/* Bytes of device storage build_block_mask needs for these sizes, or 0 if the
 * sizes are invalid (nq, nkv >= 1; block sizes 16..1024; at most 16384 tiles
 * per axis). */
size_t build_block_mask_bytes(int32_t nq, int32_t nkv, int32_t block_q, int32_t block_kv);

/*
 *   q_seq_id, kv_seq_id  device int32[nq], int32[nkv]; any negative id is padding;
 *                        ids need not be sorted or contiguous
 *   block_q, block_kv    tile sizes, 16..1024
 *   storage, bytes       caller device buffer of >= build_block_mask_bytes(...),
 *                        256-byte aligned; its contents are overwritten
 *   out                  host descriptor, filled on success
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_WORKSPACE, PA_ERR_ALIGN, PA_ERR_HIP.
 */
int32_t build_block_mask(const int32_t* q_seq_id, int32_t nq, const int32_t* kv_seq_id,
                         int32_t nkv, int32_t block_q, int32_t block_kv, void* storage,
                         size_t bytes, pa_block_mask* out, void* stream);

/*
 * attn_packed_fwd -- O = softmax(scale * Q K^T, masked) V per head, over the
 * allowed pairs only, and LSE = log sum exp of the allowed scaled scores
 * (natural log, fp32).  Rows with no allowed key: O = 0, LSE = -inf.
 * Work per query tile runs only over its non-empty key tiles; the elementwise
 * mask is applied only on partial tiles.
 * Passages: the forward template of the masked attention kernel that runs on
 * the packed pack ("LingBot-VA attention profiling" report, kernel profile:
 * FlexAttention forward); the same-id predicate ("LingBot-VA attention
 * profiling" report, next steps; "Furniture packing, variable length" report,
 * implementation part: -1 removed as query and as key); fully masked padding
 * rows must come out without NaN ("LingBot-VA packing" report, section 3.1
 * table); packed output equals each episode run alone (same report, section
 * 2.2).
 *
 *   dtype      PA_BF16 (bf16 in/out, fp32 accumulation; head_dim 64 or 128;
 *              the mask must use 128 x 128 tiles) or PA_F32 (fp32 throughout;
 *              head_dim 64 or 128; mask tiles of 32, 64 or 128 per axis)
 *   nq, nkv    tokens on each side, >= 1; heads >= 1
 *   scale      score scale (1/sqrt(head_dim) is the usual choice)
 *   q, k, v    device tensors of `dtype`
 *   q_seq_id, kv_seq_id  the ids the mask was built from
 *   mask       descriptor from build_block_mask for (nq, nkv)
 *   o          device [nq][heads][head_dim] of `dtype`, written
 *   lse        device fp32 [heads][nq], written
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_HEADDIM,
 *         PA_ERR_MASK_MISMATCH, PA_ERR_ALIGN, PA_ERR_HIP.
 */
int32_t attn_packed_fwd(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads, int32_t head_dim,
                        float scale, const void* q, const void* k, const void* v,
                        const int32_t* q_seq_id, const int32_t* kv_seq_id,
                        const pa_block_mask* mask, void* o, float* lse, void* stream);

/* Workspace bytes attn_packed_bwd needs (fp32 Delta = rowsum(dO*O) and the LSE in
 * log2 units, each [heads][nq]), or 0 for invalid sizes.  These row terms are
 * the standard softmax-gradient quantities of the backward template the pages
 * run ("LingBot-VA attention profiling" report, kernel profile: FlexAttention
 * backward). */
size_t attn_packed_bwd_workspace_bytes(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                       int32_t head_dim);

/*
 * attn_packed_bwd -- gradients of attn_packed_fwd for upstream gradient dout:
 *   P = exp(scale*QK^T - LSE) on allowed pairs (0 elsewhere and on -inf rows),
 *   Delta = rowsum(dout * o), dS = P * (dout V^T - Delta),
 *   dq = scale dS K, dk = scale dS^T Q, dv = P^T dout.
 * Rows of dq with no allowed key, and rows of dk/dv that no query selects, are
 * exact zeros.
 * Passages: the backward template of the masked attention kernel
 * ("LingBot-VA attention profiling" report, kernel profile: FlexAttention
 * backward); gradients must stay finite on a pack with padding frames and the
 * packed gradients match per-episode runs ("LingBot-VA packing" report,
 * section 3.1 table and section 2.2); the mask shared by forward and backward
 * must match the call (same report, section 2.2: a forward of another shape in
 * between broke the backward), hence PA_ERR_MASK_MISMATCH.
 * Arguments as for attn_packed_fwd, plus
 *   o, lse      the forward's outputs
 *   dout        device [nq][heads][head_dim] of `dtype`
 *   dq, dk, dv  device outputs of `dtype`, written (all rows)
 *   workspace   device buffer of >= attn_packed_bwd_workspace_bytes(...),
 *               256-byte aligned, overwritten
 * Errors: as attn_packed_fwd, plus PA_ERR_WORKSPACE.
 */
int32_t attn_packed_bwd(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads, int32_t head_dim,
                        float scale, const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, const int32_t* q_seq_id,
                        const int32_t* kv_seq_id, const pa_block_mask* mask, void* dq, void* dk,
                        void* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages attn_packed_bwd runs, callable one by one (same kernels,
 * same results; for callers that time or overlap the stages), and the row
 * terms alone.  `workspace` is a device buffer of >=
 * attn_packed_bwd_workspace_bytes(...) bytes, 256-byte aligned.
 *
 * attn_packed_bwd_preprocess -- the row terms of the softmax gradient alone,
 *   into the workspace: Delta[h][i] = sum_d dout[i][h][d] * o[i][h][d] (fp32)
 *   and the forward's LSE in log2 units (+inf on rows without an allowed key,
 *   so that P = 0 there).  attn_packed_bwd does not need it (its dQ stage
 *   computes the same terms); it serves callers that want them alone.
 *   Errors: PA_ERR_DTYPE, PA_ERR_HEADDIM, PA_ERR_SHAPE, PA_ERR_NULL, PA_ERR_ALIGN,
 *           PA_ERR_WORKSPACE, PA_ERR_HIP.
 * attn_packed_bwd_dq -- the row terms (written to the workspace, as by the
 *   preprocess; with bf16 and 128-wide heads the dQ kernel computes them from
 *   o and dout itself, otherwise the preprocess kernel runs first) and
 *   dq = scale * dS K, query tile by query tile.
 * attn_packed_bwd_dkdv -- dk = scale * dS^T Q and dv = P^T dout, one workgroup
 *   per key tile; reads the row terms a dQ stage (or the preprocess) on the
 *   same inputs wrote into the workspace.
 *   Both: arguments and errors as attn_packed_bwd.
 */
int32_t attn_packed_bwd_preprocess(int32_t dtype, int32_t nq, int32_t heads, int32_t head_dim,
                                   const void* o, const void* dout, const float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);
int32_t attn_packed_bwd_dq(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                           int32_t head_dim, float scale, const void* q, const void* k,
                           const void* v, const void* o, const void* dout, const float* lse,
                           void* workspace, size_t workspace_bytes,
                           const int32_t* q_seq_id, const int32_t* kv_seq_id,
                           const pa_block_mask* mask, void* dq, void* stream);
int32_t attn_packed_bwd_dkdv(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                             int32_t head_dim, float scale, const void* q, const void* k,
                             const void* v, const void* dout, const float* lse,
                             const void* workspace, size_t workspace_bytes,
                             const int32_t* q_seq_id, const int32_t* kv_seq_id,
                             const pa_block_mask* mask, void* dk, void* dv, void* stream);

/*
 * attn_packed_bwd_noalloc -- attn_packed_bwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and the same results, bit for bit,
 * but the workspace (Delta and LSE2, 8 bytes per head and query) lives in a
 * fixed array inside the library, one per device, held until the process ends.
 * The entry point calls no hipMalloc, hipFree or allocating routine; on the
 * first call made on a device it looks up that device's array address once.
 *   Arguments, layouts and ownership as for attn_packed_bwd, without the
 *   workspace.  Sizes: 8 * heads * nq (rounded up to 256) must not exceed
 *   attn_packed_bwd_noalloc_max_bytes() (64 MiB: heads * nq <= 8,388,608),
 *   else PA_ERR_WORKSPACE before any launch.
 *   The array keeps the last call's contents; every value a call reads was
 *   written by that call first, so no clearing is needed.  All calls on one
 *   device share the array: calls that overlap in time on one device (other
 *   streams, other host threads) race and must be serialised by the caller.
 * Errors: as attn_packed_bwd; PA_ERR_HIP also if the array's address cannot be
 * looked up.
 */
size_t attn_packed_bwd_noalloc_max_bytes(void);
int32_t attn_packed_bwd_noalloc(int32_t dtype, int32_t nq, int32_t nkv, int32_t heads,
                                int32_t head_dim, float scale, const void* q, const void* k,
                                const void* v, const void* o, const void* dout, const float* lse,
                                const int32_t* q_seq_id, const int32_t* kv_seq_id,
                                const pa_block_mask* mask, void* dq, void* dk, void* dv,
                                void* stream);

/*
 * pa_test_set_handover_spin_limit -- test hook, not for production callers.
 * In the bf16 dK/dV kernel for 128-wide heads, the two waves that share a SIMD
 * hand the probabilities P over through LDS, and the writer waits (bounded) for
 * the reader's release of the previous P.  A wait that runs out makes that
 * wave write NaN into its dv rows instead of values, so a broken hand-over
 * shows in the output.  This sets the bound, in polls of about 64 cycles, for
 * launches made after the call in this process (host state, not thread-safe);
 * a negative limit restores the default (2^20).  Returns the previous bound.
 * With a limit of 0 every wait after a tile's first step runs out at once
 * (no poll is made), which lets a test see the NaN path without any kernel
 * waiting long.
 */
int32_t pa_test_set_handover_spin_limit(int32_t limit);

/*
 * pa_handover_failures -- how many dK/dV waves on the current device ran out
 * of their bounded hand-over wait (see above) since the library was loaded or
 * the count was last reset; each such wave wrote NaN into its dv rows.  For
 * monitoring a training job: a nonzero count means the gradients of those
 * launches are not to be used.  Synchronous (a device-to-host copy on the null
 * stream, so it waits for the device's earlier work); reset != 0 sets the
 * count back to 0 after reading it.  Returns the count (>= 0), or PA_ERR_HIP.
 */
int32_t pa_handover_failures(int32_t reset);

/*
 * Frame-valid masked squared-error loss ("LingBot-VA packing" report, section
 * 2.1, compute_loss: on a padded pack the latent and action losses are averaged
 * over valid frames only).  A token is valid iff its seq id is >= 0:
 *   L = sum over valid rows i and channels c of (pred[i][c] - target[i][c])^2,
 *       divided by (n_valid * C);  L = 0 when no row is valid;
 *   dL/dpred = 2 (pred - target) / (n_valid * C) on valid rows, exact 0 on
 *       padding rows.
 * Sums run in fp32 in a fixed order: results are bitwise reproducible.
 *
 *   dtype        PA_F32 or PA_BF16 (pred, target and dpred share it)
 *   n, C         rows (tokens) >= 0 and channels, C a multiple of 8, n*C <= 2^36;
 *                n = 0 reads nothing (pred, target, seq_id, dpred may be NULL)
 *                and gives stats {0, 0, 0, 0}
 *   pred, target device [n][C], 16-byte aligned
 *   seq_id       device int32[n]
 *   stats        device fp32[4], written: {loss, sum of squared errors over
 *                valid rows, n_valid (exact below 2^24), 2/(n_valid*C) or 0}
 *   upstream     dL_total/dL, multiplies the gradient (1 for a plain loss)
 *   dpred        device [n][C] of dtype, written (all rows), 16-byte aligned
 *   workspace    device buffer of >= masked_mse_workspace_bytes(n) bytes (8 KiB
 *                for any n; 0 means n < 0), 256-byte aligned, overwritten
 * masked_mse_fwd      loss only: writes stats.
 * masked_mse_bwd      gradient only, from the stats of a finished
 *                     masked_mse_fwd on the same inputs (stats[3] is read);
 *                     the same bits as masked_mse_fwd_bwd's dpred.
 * masked_mse_fwd_bwd  both in one pass over pred and target (counts the valid
 *                     rows from the ids first); writes stats and dpred.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_ALIGN,
 *         PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
size_t masked_mse_workspace_bytes(int32_t n);
int32_t masked_mse_fwd(int32_t dtype, int32_t n, int32_t C, const void* pred, const void* target,
                       const int32_t* seq_id, float* stats, void* workspace,
                       size_t workspace_bytes, void* stream);
int32_t masked_mse_bwd(int32_t dtype, int32_t n, int32_t C, const void* pred, const void* target,
                       const int32_t* seq_id, const float* stats, float upstream, void* dpred,
                       void* stream);
int32_t masked_mse_fwd_bwd(int32_t dtype, int32_t n, int32_t C, const void* pred,
                           const void* target, const int32_t* seq_id, float upstream,
                           float* stats, void* dpred, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * AdaLN on a packed sequence (AdaptiveLoad summary, section 2B: LayerNorm and
 * modulation fused into one pass with the row statistics kept on chip; the
 * backward reduces the modulation gradients over the sequence with feature
 * tiles, each thread owning fixed feature columns down a tile of rows).
 *
 *   xhat = (x - mean) / sqrt(var + eps)        (per row over D, biased variance)
 *   y    = xhat * (1 + scale[s]) + shift[s]    (s = segment of the row)
 *   dx   = rstd * (g - mean_D(g) - xhat * mean_D(g * xhat)),  g = dy * (1 + scale[s])
 *   d_scale[s] = sum over valid rows of s of dy * xhat,  d_shift[s] = sum of dy
 *
 * Segments: segment s (0 <= s < n_seg) is rows seg_offsets[s] .. seg_offsets[s+1]-1
 * (episodes stored back to back, e.g. the offsets seq_ids_from_lengths
 * returns, or b * frames_padded * tokens_per_frame for a frame-padded pack).
 * The offsets are read clamped into [0, n] and made non-decreasing.  A row is
 * valid iff it lies in a segment and seq_id >= 0; invalid rows give y = 0,
 * dx = 0, mean = rstd = 0 and add nothing to d_shift / d_scale.  Results are
 * bitwise reproducible (every sum has a fixed order).
 *
 *   dtype         PA_F32 or PA_BF16: x, y, dy, dx (modulation and statistics are fp32)
 *   n, D          rows >= 0 and features, D a multiple of 8 in [8, 4096]
 *   n_seg         segments, 0 .. 2048
 *   eps           >= 0, added to the variance (1e-6 is the usual choice)
 *   x, y, dy, dx  device [n][D] of dtype, 16-byte aligned
 *   seq_id        device int32[n]
 *   seg_offsets   device int32[n_seg + 1]
 *   shift, scale  device fp32 [n_seg][D], 16-byte aligned
 *   mean, rstd    device fp32 [n]: written by adaln_fwd, read by adaln_bwd
 *   d_shift, d_scale  device fp32 [n_seg][D], written (all rows), 16-byte aligned
 *   workspace     device buffer of >= adaln_bwd_workspace_bytes(n, D, n_seg)
 *                 bytes, 256-byte aligned, overwritten (per-tile partial sums)
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_ALIGN,
 *         PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
int32_t adaln_fwd(int32_t dtype, int32_t n, int32_t D, int32_t n_seg, float eps, const void* x,
                  const int32_t* seq_id, const int32_t* seg_offsets, const float* shift,
                  const float* scale, void* y, float* mean, float* rstd, void* stream);
size_t adaln_bwd_workspace_bytes(int32_t n, int32_t D, int32_t n_seg);
int32_t adaln_bwd(int32_t dtype, int32_t n, int32_t D, int32_t n_seg, const void* x,
                  const void* dy, const int32_t* seq_id, const int32_t* seg_offsets,
                  const float* scale, const float* mean, const float* rstd, void* dx,
                  float* d_shift, float* d_scale, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Batch planning -- HOST functions (host pointers; no device work).
 *
 * length_bucket_batches: one rank's batches for one epoch ("LingBot-VA packing"
 * report, section 2.1, LengthBucketBatchSampler and the pad collate):
 *   1. the episodes 0 .. n-1 are shuffled (Fisher-Yates driven by SplitMix64
 *      seeded with seed + epoch; j = high 64 bits of next() * (i + 1));
 *   2. the list is padded to a multiple of world_size by repeating it from
 *      its start; rank r takes positions r, r + world_size, ... (every rank
 *      gets the same count, length_bucket_rank_size(n, world_size));
 *   3. the rank's list is cut into pools of pool_size episodes, each pool is
 *      sorted by frames (ascending, stable) and cut into batches: batch_size
 *      episodes (the pool's last batch may be short), or, with batch_size = 0,
 *      greedily under the dual constraint below (a batch grows while its size
 *      is within dual_constraint_batch of its padded sequence length
 *      round_up(max frames, pad_multiple) * tokens_per_frame);
 *   4. the batch order is shuffled, continuing the same generator.
 *   frames        host int32[n], latent frames per episode (>= 0)
 *   episodes      host int32[length_bucket_rank_size(n, W)], written: the
 *                 episodes of all batches, batch after batch
 *   batch_ptr     host int32[that + 1], written: batch b is
 *                 episodes[batch_ptr[b] .. batch_ptr[b+1])
 *   batch_frames  host int32[that], written: padded frames of each batch,
 *                 round_up(max frames, pad_multiple)
 *   n_batches     host int32, written
 *   Errors: PA_ERR_SHAPE (n < 0, pool_size < 1, pad_multiple < 1, batch_size < 0,
 *           rank outside [0, world_size), a negative frame count, bad dual
 *           parameters), PA_ERR_NULL (NULL outputs, or dual NULL with batch_size 0).
 *
 * dual_constraint_batch: AdaptiveLoad summary, section 2A: the batch size of a
 *   bucket of sequence length S, max(1, min(floor(m_mem / S), floor(m_comp / S^p))),
 *   from B * S <= m_mem (memory, linear) and B * S^p <= m_comp (compute).
 *   Returns the batch size (>= 1) or PA_ERR_SHAPE for non-positive S, m_mem, m_comp.
 *
 * fit_step_cost: fits step time t ~ a + b * B * S^p to m >= 2 measured shapes
 *   (same section: the step-cost model behind p and m_comp) by least squares in
 *   t: for each p the best a, b are a straight-line fit, and p in [p_lo, p_hi]
 *   minimises the residual (golden-section search).  out = {a, b, p}.
 *   Errors: PA_ERR_SHAPE (m < 2, empty range, a non-positive B or S), PA_ERR_NULL.
 */
typedef struct pa_dual_constraint {
  double m_mem;             /* token budget per batch (memory constraint)        */
  double m_comp;            /* compute budget: B * S^p <= m_comp                  */
  double p;                 /* cost exponent                                      */
  int32_t tokens_per_frame; /* sequence length S = padded frames * this          */
} pa_dual_constraint;

size_t length_bucket_rank_size(int32_t n, int32_t world_size);
int32_t length_bucket_batches(const int32_t* frames, int32_t n, uint64_t seed, int32_t epoch,
                              int32_t pool_size, int32_t pad_multiple, int32_t batch_size,
                              const pa_dual_constraint* dual, int32_t rank, int32_t world_size,
                              int32_t* episodes, int32_t* batch_ptr, int32_t* batch_frames,
                              int32_t* n_batches);
int32_t dual_constraint_batch(double seq_len, double m_mem, double m_comp, double p);
int32_t fit_step_cost(const double* B, const double* S, const double* t, int32_t m, double p_lo,
                      double p_hi, double* out);

#ifdef __cplusplus
}
#endif

#endif /* PACKATTN_H */
