/*
 * attn.h -- C ABI of the fused attention forward for MI355X (gfx950).
 *
 * The operation (the plain definition the library reproduces, computed tile by
 * tile so that no N x N score matrix ever reaches device memory):
 *
 *     O   = softmax( mods( scale * Q K^T ) under mask ) V
 *     LSE = log( sum_j exp( mods( scale * q_i . k_j ) ) )      over allowed j
 *
 * Sources: "FlashAttention-3 : une attention plus rapide et plus precise grace
 * a l'asynchronisme et a la basse precision" (fr.news.hada.io), section
 * "Rappel du fonctionnement de FlashAttention" (blocks move from HBM to SRAM,
 * attention is computed per block, tiling plus softmax rescaling is exact);
 * "Les kernels d'attention rapide et la fusion d'operateurs accelerent les
 * modeles d'IA", section "Attention de type FlashAttention et attention
 * paginee" (the full score matrix is never stored); "FlexAttention de PyTorch
 * avec FlashAttention-4 change la donne", opening section (score and mask
 * modifiers: soft-capping, ALiBi, sliding window, document masking) and
 * section "Limitations actuelles" (block sparsity; no silent fallback here).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or retains them, and never synchronises the host.
 * - Tensors are contiguous, row-major, BHSD: Q and O are [B][Hq][Nq][d], K and
 *   V are [B][Hkv][Nk][d], LSE is [B][Hq][Nq] float32 (natural log).
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   All work is enqueued on it; every call is safe to capture into a HIP graph.
 * - Return value: ATTN_OK or a negative attn_status. Arguments are validated
 *   before any HIP call; an invalid call has no side effect. Faults during
 *   kernel execution surface, as for any stream API, at the caller's next
 *   synchronisation.
 * - No call keeps mutable global state; calls are thread-safe.
 *
 * Debug aids (environment variables, read once per process):
 * - ATTN_CHECK=1 checks preconditions on device data before launching:
 *   doc_ids non-decreasing (attn_fwd with ATTN_MASK_DOC), cu_seqlens starting
 *   at 0, non-decreasing and ending at total (attn_fwd_varlen), seq_lens
 *   within max_blocks * block_size (attn_decode_paged); a violation returns
 *   ATTN_ERR_INVALID_ARG and launches nothing. The data is copied to the host
 *   and the stream synchronised: not for use under graph capture.
 * - ATTN_LOG=1 prints each call's arguments to stderr and, for attn_fwd, the
 *   grid and the forward's tile counts (blocks of 32 query rows by 64-key
 *   tiles: empty = skipped, partial = element mask, full = no mask code) and
 *   the skipped fraction. With ATTN_MASK_DOC it copies doc_ids to the host
 *   and synchronises the stream, as ATTN_CHECK does.
 */
#ifndef TILED_ATTN_H
#define TILED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1,   /* NULL required pointer, bad size, bad flag, non-finite scalar */
    ATTN_ERR_UNSUPPORTED = -2,   /* a valid request this build does not implement (no fallback) */
    ATTN_ERR_HIP = -3            /* a HIP runtime call or kernel launch failed */
} attn_status;

typedef enum {
    ATTN_F32 = 0,        /* Q, K, V, O float32 */
    ATTN_BF16 = 1,       /* Q, K, V, O bfloat16 */
    ATTN_FP8_E4M3 = 2    /* Q, K, V are buffers written by attn_fp8_prepare; O is bfloat16 */
} attn_dtype;

/* mask_kind bit flags */
enum {
    ATTN_MASK_NONE = 0,
    ATTN_MASK_CAUSAL = 1,   /* key j allowed for query i iff j <= i + (Nk - Nq)               */
    ATTN_MASK_WINDOW = 2,   /* with CAUSAL only: also (i + Nk - Nq) - j < window (W keys)      */
    ATTN_MASK_DOC = 4       /* doc_ids[b][i] == doc_ids[b][j]; needs Nq == Nk; with/without CAUSAL */
};

/*
 * attn_fwd -- fused attention forward.
 *
 * q, k, v    : input tensors (layouts above); element type from `dtype`.
 * o          : output [B][Hq][Nq][d]; float32 for ATTN_F32, bfloat16 otherwise.
 * lse        : float32 [B][Hq][Nq] natural-log log-sum-exp of the modified
 *              scores of each row, or NULL to skip it. A row with no allowed key
 *              gets O = 0 and LSE = -inf.
 * B, Hq, Hkv : batch, query heads, key/value heads; Hq % Hkv == 0 and query head
 *              h reads key/value head h / (Hq / Hkv) (grouped-query attention).
 * Nq, Nk     : query and key lengths, >= 1.
 * d          : head dimension: 64 or 128 (128 only for ATTN_FP8_E4M3).
 * scale      : finite multiplier of q . k (usually 1/sqrt(d)).
 * mask_kind  : ATTN_MASK_* flags.  window: width W >= 1, read only with WINDOW.
 * doc_ids    : device int32 [B][Nk], non-decreasing along each row (packed
 *              documents); required iff ATTN_MASK_DOC. A decreasing sequence
 *              is a precondition violation (attn_block_mask_build flags it).
 * softcap    : 0 for none, else > 0: s <- softcap * tanh(s / softcap), applied
 *              to s = scale * q . k before the ALiBi bias.
 * alibi_slopes: device float32 [Hq] or NULL: s <- s - slope[h] * (i - j).
 * dtype      : attn_dtype.
 * Errors     : ATTN_ERR_INVALID_ARG for NULL q/k/v/o, dims < 1, Hq % Hkv != 0,
 *              non-finite scale, softcap < 0 or non-finite, unknown mask bits,
 *              WINDOW with window < 1, DOC without doc_ids, unknown dtype;
 *              ATTN_ERR_UNSUPPORTED for d not in {64, 128}, WINDOW without
 *              CAUSAL, DOC with Nq != Nk, fp8 with d != 128, Nq != Nk, a
 *              mask, soft-cap or ALiBi; ATTN_ERR_HIP if the launch fails.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int mask_kind, int window, const int32_t* doc_ids,
             float softcap, const float* alibi_slopes, int dtype, void* stream);

/*
 * attn_fwd_varlen -- the same forward over a packed batch of variable-length
 * sequences ("FlashAttention-3 : ...", section "Optimisations restantes et
 * integration future": variable-length sequences). Sequence s owns tokens
 * [cu_seqlens[s], cu_seqlens[s + 1]) of the packed dimension and attends only
 * within itself: the document mask of "FlexAttention de PyTorch avec
 * FlashAttention-4 change la donne" (opening section) over the concatenation.
 *
 * q, o       : [Hq][total][d]; k, v: [Hkv][total][d]; lse: float32 [Hq][total]
 *              or NULL. Element types and O / LSE conventions as attn_fwd.
 * cu_seqlens : device int32 [num_seqs + 1]: cu_seqlens[0] = 0, non-decreasing,
 *              cu_seqlens[num_seqs] = total (empty sequences allowed). Tokens
 *              past cu_seqlens[num_seqs] would form one more sequence: a
 *              precondition violation, not detected (the offsets live on the
 *              device).
 * mask_kind  : ATTN_MASK_NONE, or ATTN_MASK_CAUSAL (j <= i within a sequence),
 *              optionally | ATTN_MASK_WINDOW (with window W as in attn_fwd).
 * softcap, alibi_slopes, scale, d, Hq, Hkv: as attn_fwd (ALiBi distances are
 *              within a sequence).
 * workspace  : device int32 [total], caller-owned scratch, overwritten before
 *              the forward runs (the library allocates nothing); must not
 *              alias another argument. ATTN_BF16, when ceil(total / 256) +
 *              num_seqs <= total, num_seqs <= 4096 and total <= 4096 * 256:
 *              each sequence is tiled on its own, and the first
 *              ceil(total / 256) + num_seqs entries receive the list of its
 *              256-row query tiles (first packed row of each tile;
 *              sequences by tile count descending, lower index first, each
 *              sequence's tiles from its last to its first; -1 past the last
 *              tile). Otherwise, and for
 *              ATTN_F32: each token's sequence index, and the document-mask
 *              forward over the concatenation. The two paths group keys
 *              into tiles differently, so their results agree up to rounding.
 * dtype      : ATTN_F32 or ATTN_BF16.
 * Errors     : ATTN_ERR_INVALID_ARG for NULL q/k/v/o/cu_seqlens/workspace,
 *              num_seqs < 1, total < 1, mask bits other than CAUSAL / WINDOW,
 *              and every attn_fwd argument error; ATTN_ERR_UNSUPPORTED for
 *              ATTN_FP8_E4M3 and attn_fwd's unsupported cases. Every check runs
 *              before the first HIP call.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int total, int Hq, int Hkv, int d,
                    float scale, int mask_kind, int window, float softcap,
                    const float* alibi_slopes, int32_t* workspace, int dtype, void* stream);

/*
 * fp8 incoherent-processing prepare step ("FlashAttention-3 : ...", section
 * "Basse precision FP8 et incoherent processing": Q and K are multiplied by a
 * Hadamard transform with random signs, per head, in O(d log d), to spread
 * outliers before fp8 quantisation).
 *
 * Packed buffer format (one per tensor), for H heads and N tokens, with
 * Np = N rounded up to a multiple of 128 and P = B*H*Np*d (one code plane):
 *   bytes [0, P)       e4m3 (OCP, max 448) value codes c1;
 *                      Q and K: [B][H][Np][d] (rows rotated: x D H);
 *                      V:       [B][H][d][Np] (transposed, not rotated);
 *                      padding rows / columns hold 0.
 *   bytes [P, 2P)      Q and K only: e4m3 residual codes c2, same layout;
 *                      c2 = e4m3(x / scale - value(c1)) on the same scale, so
 *                      x ~ scale * (value(c1) + value(c2)) to about 2^-7
 *                      relative. Not read or written for V.
 *   then, at byte offset 2P, float32 scales [B][H][Np/128]: one per tile of
 *   128 tokens of one head (scale = tile amax / 448, 1 for an all-zero
 *   tile); codes are rounded to nearest even and c1 saturates at +-448.
 * The forward scores a (query, key) pair with the three products
 * c1.c1' + c1.c2' + c2.c1' of its rows (the c2.c2' term is left out): one
 * e4m3 code alone misses the 5e-2 relative-RMS accuracy bar on inputs with
 * x20 outlier channels (the rounding error of Q and K dominates there).
 * attn_fp8_buffer_bytes gives the size of one such buffer (0 on bad sizes).
 *
 * q, k, v : device bfloat16 BHSD inputs, Q [B][Hq][N][d], K/V [B][Hkv][N][d].
 * signs   : device int8 [d] of +-1 (the random diagonal D), shared by all heads;
 *           NULL quantises Q and K without the rotation (for comparisons).
 * q8, k8, v8 : device buffers of attn_fp8_buffer_bytes(B, Hq|Hkv, N, d) bytes.
 * d must be 128. Errors as for attn_fwd.
 */
size_t attn_fp8_buffer_bytes(int B, int H, int N, int d);
int attn_fp8_prepare(const void* q, const void* k, const void* v,
                     int B, int Hq, int Hkv, int N, int d, const int8_t* signs,
                     void* q8, void* k8, void* v8, void* stream);

/*
 * attn_fp8_prepare_rope -- the same prepare step with the rotary position
 * embedding of Q and K fused in front of the Hadamard rotation (same page and
 * section: the Hadamard transform is memory-bound and can be fused with a
 * preceding memory-bound step such as the rotary embedding at no extra cost).
 * For token t and pair i < d/2, (x_i, x_{i+d/2}) becomes
 *   (x_i * rope_cos[t][i] - x_{i+d/2} * rope_sin[t][i],
 *    x_i * rope_sin[t][i] + x_{i+d/2} * rope_cos[t][i]);
 * then signs, Hadamard and quantisation exactly as attn_fp8_prepare. V is
 * neither turned nor rotated.
 *
 * rope_cos, rope_sin : device float32 [N][d/2], caller-owned (usually
 *   cos / sin of t * base^(-2i/d)); token t of every batch row and head uses
 *   row t. Errors: ATTN_ERR_INVALID_ARG for NULL tables, otherwise as
 *   attn_fp8_prepare.
 */
int attn_fp8_prepare_rope(const void* q, const void* k, const void* v,
                          int B, int Hq, int Hkv, int N, int d, const int8_t* signs,
                          const float* rope_cos, const float* rope_sin,
                          void* q8, void* k8, void* v8, void* stream);

/*
 * Block mask builder ("FlexAttention de PyTorch ...", section "Limitations
 * actuelles": block sparsity).  Classifies every (query tile, key tile) pair of
 * a block_m x block_n tiling of the Nq x Nk score matrix of batch row b:
 *   0 = empty (no allowed pair: skipped), 1 = partial (needs the element mask),
 *   2 = full (every pair allowed: no mask code).
 * Output buffer of attn_block_mask_bytes(...) bytes, laid out as
 *   int8  kind[B][nQt][nKt]                     (nQt = ceil(Nq/block_m), nKt = ceil(Nk/block_n))
 *   int32 counts[B][nQt][3]   at byte offset round_up(B*nQt*nKt, 16): empty, partial, full
 *   int32 flags               after counts: bit 0 set iff some doc_ids row decreases
 * block_m, block_n in [1, 4096]. Same mask semantics and errors as attn_fwd.
 */
size_t attn_block_mask_bytes(int B, int Nq, int Nk, int block_m, int block_n);
int attn_block_mask_build(int B, int Nq, int Nk, int mask_kind, int window,
                          const int32_t* doc_ids, int block_m, int block_n,
                          void* out, void* stream);

/*
 * attn_fwd_tile_kinds -- the bf16 forward's own tile schedule, for inspection
 * (same page and section: block sparsity). The forward gives each wave 32
 * query rows and walks 64-key tiles; this writes, for every (batch row, block
 * of 32 rows, key tile), the kind the forward kernel assigns through the same
 * device functions: 0 = empty (skipped), 1 = partial (element mask), 2 = full
 * (no mask code). It equals attn_block_mask_build's table at block_m = 32,
 * block_n = 64, except that a ragged last key tile (Nk % 64 != 0) whose
 * existing pairs are all allowed is partial here (the kernel masks the
 * missing keys).
 * out : device int8 [B][ceil(Nq/32)][ceil(Nk/64)], attn_fwd_tile_kinds_bytes
 *       bytes (0 on bad sizes). Mask arguments and errors as attn_fwd.
 */
size_t attn_fwd_tile_kinds_bytes(int B, int Nq, int Nk);
int attn_fwd_tile_kinds(int B, int Nq, int Nk, int mask_kind, int window,
                        const int32_t* doc_ids, int8_t* out, void* stream);

/*
 * attn_decode_paged -- one new token per sequence attending to its whole
 * key/value cache, stored in fixed-size blocks addressed through a block table
 * ("Les kernels d'attention rapide et la fusion d'operateurs accelerent les
 * modeles d'IA", section "Attention de type FlashAttention et attention
 * paginee": the kernel translates every logical position through the table).
 * Computes, per sequence b and query head h (grouped as in attn_fwd),
 *   O[b][h] = softmax_j(scale * q[b][h] . k_j) v_j,  LSE[b][h] = log sum_j exp(...)
 * over the seq_lens[b] keys of sequence b (no mask: the new token is the last
 * position). The keys are split into num_splits ranges computed independently
 * and merged exactly: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *
 * q          : bfloat16 [B][Hq][d]; o: bfloat16 [B][Hq][d]; lse: float32 [B][Hq]
 *              or NULL (a sequence of length 0 gets O = 0, LSE = -inf).
 * k_cache, v_cache : bfloat16 [num_blocks][Hkv][block_size][d]; token i of
 *              sequence b is row i % block_size of physical block
 *              block_table[b][i / block_size].
 * block_table: device int32 [B][max_blocks]; seq_lens: device int32 [B], each in
 *              [0, max_blocks * block_size]; the entries used must name valid
 *              blocks (device data: a precondition, not checked).
 * num_splits : 1..256; with more than one, workspace is device float32 of
 *              attn_decode_workspace_floats(B, Hq, d, num_splits) entries
 *              (caller-owned scratch, overwritten: the splits' partial outputs
 *              and LSEs, and the order in which the sequences are launched,
 *              longest first); NULL is allowed with 1.
 * Supported  : dtype ATTN_BF16, d = 128, block_size = 16, Hq / Hkv <= 32.
 * Errors     : ATTN_ERR_INVALID_ARG for NULL q/k_cache/v_cache/block_table/
 *              seq_lens/o, sizes < 1, Hq % Hkv != 0, non-finite scale,
 *              num_splits outside 1..256, a missing workspace, unknown dtype;
 *              ATTN_ERR_UNSUPPORTED otherwise outside the supported set.
 */
size_t attn_decode_workspace_floats(int B, int Hq, int d, int num_splits);
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int d, int block_size, int max_blocks, float scale,
                      int num_splits, float* workspace, int dtype, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without `workspace`,
 * the same kernels and results. The split outputs, LSEs and launch order live
 * in a fixed device array of the library, 16 MiB (4 * 2^20 floats) per GPU,
 * held until the process ends. attn_decode_workspace_floats(B, Hq, d,
 * num_splits) must not exceed 4 * 2^20, else ATTN_ERR_INVALID_ARG (nothing
 * launched). Calls that overlap in time on one GPU (different streams) share
 * the array and race: serialise them. The call allocates nothing and makes
 * no allocating runtime call; the array's device address is looked up once
 * per device. Errors otherwise as attn_decode_paged.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int d, int block_size, int max_blocks, float scale,
                              int num_splits, int dtype, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd (no modifiers) for an output gradient dO.
 * With P_ij = exp(scale q_i . k_j - LSE_i) recomputed from the forward's LSE
 * and D_i = sum_c dO_ic O_ic:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV summed over the query heads of each key/value head. Exact and
 * deterministic ("FlashAttention-2 (FR)", section "Performance et efficacite";
 * "FlexAttention de PyTorch avec FlashAttention-4 change la donne", section
 * "Limitations actuelles", names the non-deterministic backward this avoids):
 * no gradient is accumulated with atomics.
 *
 * q, o, dout, dq : bfloat16 [B][Hq][N][d]; k, v, dk, dv: bfloat16 [B][Hkv][N][d];
 * lse        : float32 [B][Hq][N], the forward's natural-log LSE of the same call.
 * workspace  : device float32 [B][Hq][N], caller-owned scratch (D), overwritten.
 * mask_kind  : ATTN_MASK_NONE or ATTN_MASK_CAUSAL (Nq = Nk = N).
 * Supported  : dtype ATTN_BF16, d = 128. Errors: ATTN_ERR_INVALID_ARG for a NULL
 *              pointer, sizes < 1, Hq % Hkv != 0, non-finite scale, unknown mask
 *              bits or dtype; ATTN_ERR_UNSUPPORTED for other dtypes, d != 128,
 *              WINDOW or DOC masks.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* workspace,
             int B, int Hq, int Hkv, int N, int d, float scale, int mask_kind, int dtype, void* stream);

/* Static, human-readable text for an attn_status value (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TILED_ATTN_H */
