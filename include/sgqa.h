/*
 * sgqa.h -- C ABI of the blockwise Sparse GQA hot path for AMD MI355X (gfx950).
 *
 * Source of the method: "Inside Step 5 Preview" (StepFun blog), section "Sparse GQA":
 *   - paragraph "Reducing indexer's cost": the index keys of B adjacent historical positions are
 *     compressed into one block representation (B = 8), which cuts indexer + top-k cost by B;
 *   - paragraph "Efficient implementation of sparse attention": during prefill the top-k results
 *     of adjacent tokens are unioned so that overlapping work is grouped;
 *   - paragraph "Trade-off between top-k and block size": k = 4096 tokens = k/B = 512 blocks;
 *   - Figure 3 caption: the index keys are shared, every KV group selects its own history, and the
 *     main path reads the original K/V of the selected blocks plus the causally visible positions
 *     of the query's own (current) block.
 * The pages leave the indexer's form open. This library fixes it as:
 *   block key      kbar[b] = bf16_rne( mean_{j<B} ki[b*B + j] )            (complete blocks only)
 *   block score    s(i,g,b) = sum_h w[g,h] * max(0, <qi[i,g,h,:], kbar[b]>)  for b < c(i) = floor(i/B)
 *   selection      Sel(i,g) = first min(k/B, c(i)) blocks in the order (s descending, b ascending)
 *   attended set   Sel(i,g) plus the own block c(i), causally masked at token level (j <= i)
 *   prefill union  U(t,g) = union over the queries i of tile t = floor(i/Tq) of Sel(i,g) + {c(i)};
 *                  every query of the tile attends over U(t,g), causally masked.
 *
 * Conventions for every call
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16_t).
 *   - Every tensor pointer is DEVICE memory owned by the caller; it must be 16-byte aligned and
 *     the tensor dense (row-major, innermost dimension last, no padding).
 *   - The library never allocates, frees or keeps a pointer after a call returns. Scratch memory
 *     comes only from the caller's workspace `ws` of `ws_bytes`, sized by sgqa_workspace_size.
 *   - Calls are asynchronous on `stream` (a hipStream_t; 0 = the null stream). Nothing is copied
 *     between host and device and nothing synchronizes the device.
 *   - Arguments are validated on the host BEFORE anything is enqueued, and every kernel's launch
 *     attributes are set once per device before its first launch: any nonzero status other than
 *     SGQA_ERR_HIP means no work was launched. SGQA_ERR_HIP (the runtime refused a launch) may
 *     leave the earlier kernels of a multi-kernel call (prefill, decode) enqueued. A fault inside
 *     a kernel surfaces at the caller's next synchronization.
 *   - Results are deterministic: the same inputs give the same bits (no floating-point atomics).
 *   - Calls keep no state beyond per-device facts filled once (thread-safe) on first use, and the
 *     backward's second stream and events (sgqa_attend_bwd); calls on different streams or host
 *     threads may run concurrently if their outputs and workspaces do not overlap.
 *   - v1 limits: head_dim == 128, idx_heads == 4, idx_dim == 64, block a power of two <= 64,
 *     topk_tokens a positive multiple of block with topk_tokens/block <= 2048, n_q_heads a multiple
 *     of n_kv_heads, n_q_heads/n_kv_heads <= 16, n_tokens >= 1, union_tile >= 1.
 *     Any other value returns SGQA_ERR_SHAPE.
 */
#ifndef SGQA_H
#define SGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGQA_ABI_VERSION 1

typedef uint16_t sgqa_bf16;   /* raw bfloat16 bits */
typedef void* sgqa_stream;    /* a hipStream_t */

/* Status codes returned by every call. */
enum {
  SGQA_OK = 0,
  SGQA_ERR_NULL = 1,       /* a required pointer is NULL */
  SGQA_ERR_SHAPE = 2,      /* unsupported or inconsistent sizes (see v1 limits) */
  SGQA_ERR_ALIGN = 3,      /* a tensor pointer is not 16-byte aligned */
  SGQA_ERR_WORKSPACE = 4,  /* workspace missing or smaller than sgqa_workspace_size */
  SGQA_ERR_DEVICE = 5,     /* the current device is not a gfx950 GPU, or no device */
  SGQA_ERR_HIP = 6,        /* the HIP runtime reported an error while launching */
  SGQA_ERR_SCRATCH = 7     /* sgqa_decode_noalloc: the call needs more scratch than the library holds */
};

/* Operation selectors for sgqa_workspace_size. */
enum {
  SGQA_OP_COMPRESS = 0,
  SGQA_OP_INDEX_TOPK = 1,
  SGQA_OP_UNION = 2,
  SGQA_OP_ATTEND = 3,
  SGQA_OP_PREFILL = 4,
  SGQA_OP_DECODE = 5,
  SGQA_OP_ATTEND_MASKED = 6,
  SGQA_OP_PREFILL_MASKED = 7,
  SGQA_OP_ATTEND_BWD = 8
};

/* Sizes of one call. Symbols: N tokens, S sequences, Hq query heads, G KV groups (KV heads),
 * r = Hq/G query heads per group, D head dim, H_I indexer heads, d_I indexer dim, B block,
 * k selected tokens, K_B = k/B selected blocks, Tq union tile, NB = floor(N/B) complete blocks,
 * NBc = ceil(N/B) blocks, T = ceil(N/Tq) tiles, W = ceil(NBc/32) mask words. */
typedef struct sgqa_params {
  int32_t n_tokens;      /* prefill: N. decode: L, the cached context length INCLUDING the query token */
  int32_t n_seqs;        /* prefill: must be 1 (compress accepts S >= 1). decode: S */
  int32_t n_q_heads;     /* Hq */
  int32_t n_kv_heads;    /* G */
  int32_t head_dim;      /* D (v1: 128) */
  int32_t idx_heads;     /* H_I (v1: 4) */
  int32_t idx_dim;       /* d_I (v1: 64) */
  int32_t block;         /* B (power of two, 1..64) */
  int32_t topk_tokens;   /* k (multiple of B) */
  int32_t union_tile;    /* Tq (>= 1; 1 = no union, every query keeps its own selection) */
  float softmax_scale;   /* sigma; <= 0 selects 1/sqrt(D) */
} sgqa_params;

/* ABI version of the loaded library (SGQA_ABI_VERSION). Host only. */
int sgqa_abi_version(void);

/* Static text for a status code. Host only; never NULL. */
const char* sgqa_status_string(int status);

/* Bytes of workspace that operation `op` (SGQA_OP_*) needs for `p`, written to *bytes.
 * Host only: touches no device. Returns SGQA_ERR_NULL / SGQA_ERR_SHAPE like the operation would. */
int sgqa_workspace_size(const sgqa_params* p, int op, size_t* bytes);

/* Block compression ("Inside Step 5 Preview", Sparse GQA, paragraph "Reducing indexer's cost",
 * and Figure 3: one shared set of index keys is merged block by block into block keys).
 *   idx_k  [S][N][d_I]        bf16   shared index keys of every token
 *   blk_k  [S][floor(N/B)][d_I] bf16 out: blk_k[s][b][d] = bf16_rne(sum_{j<B} idx_k[s][b*B+j][d] / B),
 *                                    summed in fp64 in ascending j and rounded once (nearest even;
 *                                    NaN -> 0x7FC0). A trailing partial block is not compressed (it
 *                                    can only ever be a query's own block).
 * Uses p->n_seqs, n_tokens, idx_dim, block; blk_k may be NULL when N < B. No workspace. */
int sgqa_compress(const sgqa_params* p, const sgqa_bf16* idx_k, sgqa_bf16* blk_k, sgqa_stream stream);

/* Indexer scores and per-query top-k ("Reducing indexer's cost"; Figure 3: the selection is
 * made separately for every KV group; "Trade-off between top-k and block size" for k/B).
 *   idx_q  [N][G][H_I][d_I]  bf16   per-group indexer queries
 *   idx_w  [G][H_I]          fp32   per-group indexer head weights
 *   blk_k  [floor(N/B)][d_I] bf16   block keys from sgqa_compress
 *   topk   [G][N][K_B]       int32  out: Sel(i,g), ascending block ids, padded with -1 after
 *                                   min(K_B, c(i)) entries. The own block c(i) is NOT stored.
 * Scores are fp32 (products of bf16 accumulated in fp32 on the matrix cores); -0 counts as +0;
 * ties go to the lower block id. No workspace (pass NULL/0). */
int sgqa_index_topk(const sgqa_params* p, const sgqa_bf16* idx_q, const float* idx_w,
                    const sgqa_bf16* blk_k, int32_t* topk, void* ws, size_t ws_bytes,
                    sgqa_stream stream);

/* Tile union of adjacent queries' selections (Sparse GQA, paragraph "Efficient implementation
 * of sparse attention": prefill groups the overlapping selections of neighbouring tokens).
 *   topk   [G][N][K_B]  int32   from sgqa_index_topk
 *   umask  [G][T][W]    uint32  out: bit (b % 32) of word b/32 is set iff block b is in U(t,g)
 *   ucount [G][T]       int32   out: |U(t,g)| (popcount of the row)
 * Tiles are aligned at token 0; the last tile may be partial. No workspace. */
int sgqa_union(const sgqa_params* p, const int32_t* topk, uint32_t* umask, int32_t* ucount,
               sgqa_stream stream);

/* Fused selection and union (same sources as sgqa_index_topk and sgqa_union): the per-query
 * selections go straight into the tile-union bitmask, so the [G][N][K_B] topk array is never
 * written (it is the largest intermediate of the prefill: 2 GiB at N = 131072, G = 8, K_B = 512).
 *   idx_q, idx_w, blk_k  as in sgqa_index_topk
 *   umask, ucount        out, as in sgqa_union; bit-identical to sgqa_index_topk + sgqa_union
 * No workspace (pass NULL/0). */
int sgqa_index_union(const sgqa_params* p, const sgqa_bf16* idx_q, const float* idx_w,
                     const sgqa_bf16* blk_k, uint32_t* umask, int32_t* ucount, void* ws, size_t ws_bytes,
                     sgqa_stream stream);

/* Gathered-block causal GQA attention over the tile unions (Figure 3: the attention main path
 * loads the uncompressed K/V of the chosen history blocks and, for the query's own block, only
 * the positions the causal mask lets it see).
 *   q      [N][Hq][D]  bf16
 *   k, v   [G][N][D]   bf16  (head-major: one block of one group is B*D contiguous elements)
 *   umask, ucount          from sgqa_union
 *   out    [N][Hq][D]  bf16  out: for head h, group g = h / r, tile t = floor(i/Tq):
 *          out[i][h] = sum_{j in J} softmax_j(sigma * <q[i][h], k[g][j]>) v[g][j],
 *          J = { j <= i : floor(j/B) in U(t,g) }; fp32 softmax and accumulation, bf16 RNE output.
 * No workspace (pass NULL/0). */
int sgqa_attend(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out, void* ws,
                size_t ws_bytes, sgqa_stream stream);

/* Whole prefill layer path on one stream: compress -> fused index/union (sgqa_index_union) ->
 * attend, with blk_k, umask and ucount kept in the workspace (layouts as above; no topk). Arguments
 * as in the single calls; out [N][Hq][D] bf16, bit-identical to the single calls
 * compress -> index_topk -> union -> attend. Workspace: sgqa_workspace_size(p, SGQA_OP_PREFILL). */
int sgqa_prefill(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                 const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* idx_k,
                 sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream);

/* Single-token decode over a cache: the same selection for the last position and no union,
 * since the pages introduce the union only for prefill ("Efficient implementation of sparse
 * attention").
 * For every sequence s the query sits at position i = L-1 of its cache; candidates are the
 * blocks b < c = floor((L-1)/B); the attended tokens are those of Sel(s,g) plus the own-block
 * tokens c*B .. L-1.
 *   q          [S][Hq][D]          bf16
 *   k_cache,
 *   v_cache    [S][G][L][D]        bf16
 *   blk_k      [S][floor(L/B)][d_I] bf16  block keys of the cached index keys (sgqa_compress)
 *   idx_q      [S][G][H_I][d_I]    bf16
 *   idx_w      [G][H_I]            fp32
 *   topk_out   [S][G][K_B]         int32  optional (NULL = not written): Sel, ascending, -1 pad
 *   out        [S][Hq][D]          bf16
 * Workspace: sgqa_workspace_size(p, SGQA_OP_DECODE). */
int sgqa_decode(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache,
                const sgqa_bf16* v_cache, const sgqa_bf16* blk_k, const sgqa_bf16* idx_q,
                const float* idx_w, int32_t* topk_out, sgqa_bf16* out, void* ws, size_t ws_bytes,
                sgqa_stream stream);

/* ---------------------------------------------------------------- decode without allocation
 * For callers that cannot allocate device memory around a call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments, result and errors as
 * sgqa_decode, minus the workspace: the scratch (selection, scores, segment lists) lives in a buffer
 * of SGQA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it is loaded on, until the
 * process ends. The output is bit-identical to sgqa_decode's.
 *   - Sizes whose decode workspace (sgqa_workspace_size(p, SGQA_OP_DECODE)) exceeds
 *     SGQA_NOALLOC_SCRATCH_BYTES return SGQA_ERR_SCRATCH before anything is enqueued (e.g. the
 *     32 x 262144-token decode needs ~33 MiB and fits; S * G * ceil(c / 512) * 512 * 4 bytes of scores
 *     must stay below the limit, c = floor((L-1)/B)).
 *   - The call allocates nothing and frees nothing (no hipMalloc/hipFree, no allocating routine).
 *   - Every call on one GPU shares that GPU's buffer, which keeps the last call's contents: calls that
 *     overlap in time on one GPU (different streams, or host threads without ordering) RACE on it and
 *     must be ordered by the caller. Its kernels overwrite every scratch entry before reading it, so
 *     nothing needs clearing between calls. */
#define SGQA_NOALLOC_SCRATCH_BYTES (64u << 20)
int sgqa_decode_noalloc(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache,
                        const sgqa_bf16* v_cache, const sgqa_bf16* blk_k, const sgqa_bf16* idx_q,
                        const float* idx_w, int32_t* topk_out, sgqa_bf16* out, sgqa_stream stream);

/* ---------------------------------------------------------------- incremental / varlen decode
 * The decode call above takes one context length L = n_tokens for every sequence and dense caches.
 * A serving loop needs per-sequence lengths, caches that grow one token per step, and paged K/V
 * storage. The method is unchanged: the selection of sequence s runs at its own last position
 * L_s - 1 over its blocks b < floor((L_s - 1)/B), exactly as in sgqa_decode.
 */

/* Paged K/V cache. The pools hold pages of `page_tokens` consecutive positions of one sequence for
 * every group: pool layout [n_pages][G][page_tokens][D] bf16. Position t of sequence s lives in pool
 * page table[s * max_pages + t / page_tokens]. page_tokens must be a power of two and a multiple of
 * B (a block never straddles two pages); max_pages * page_tokens >= p->n_tokens (the capacity);
 * n_pages * G * page_tokens < 2^31 (pool rows are indexed in 32 bits). table is DEVICE memory [S][max_pages] int32. The table entries of positions < L_s must lie in
 * [0, n_pages): the kernels clamp other values, so a bad table yields wrong results but never an
 * access outside the pools (sgqa_append skips the K/V write of a token whose entry is out of range). */
typedef struct sgqa_pages {
  const int32_t* table;
  int32_t max_pages;
  int32_t page_tokens;
  int32_t n_pages;
} sgqa_pages;

/* Decode with per-sequence context lengths ("Inside Step 5 Preview", Sparse GQA, Figure 3 and the
 * paragraph "Reducing indexer's cost": the same selection and attended set as sgqa_decode, each
 * sequence at its own last position).
 *   p->n_tokens   capacity C of the per-sequence caches (positions 0 .. C-1)
 *   seq_lens      [S] int32 DEVICE: L_s, the context length of sequence s including its query
 *                 token, 1 <= L_s <= C (values outside are clamped into [1, C])
 *   k_cache, v_cache  pages == NULL: dense [S][G][C][D]; else the pools described by *pages
 *   blk_k         [S][floor(C/B)][d_I]: block keys of the complete blocks of every sequence (from
 *                 sgqa_compress or sgqa_append); blocks at or past floor((L_s-1)/B) are not read
 *   q, idx_q, idx_w, topk_out, out   as in sgqa_decode
 * Workspace: sgqa_workspace_size(p, SGQA_OP_DECODE). With every L_s = C and dense caches the result
 * is bit-identical to sgqa_decode. */
int sgqa_decode_varlen(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache,
                       const sgqa_bf16* v_cache, const sgqa_pages* pages, const sgqa_bf16* blk_k,
                       const sgqa_bf16* idx_q, const float* idx_w, const int32_t* seq_lens, int32_t* topk_out,
                       sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream);

/* Append one token to every sequence's caches (the cache side of incremental decode; block keys as
 * in sgqa_compress, "Reducing indexer's cost").
 *   positions     [S] int32 DEVICE: position j_s of the new token of sequence s (usually its old
 *                 length); sequences with j_s outside [0, p->n_tokens) are left untouched
 *   k_new, v_new  [S][G][D] bf16: the token's K and V rows -> k_cache / v_cache at position j_s
 *                 (dense [S][G][C][D], or the page of *pages)
 *   idx_k_new     [S][d_I] bf16: the token's shared index key -> idx_k_cache [S][C][d_I]
 *   blk_k         [S][floor(C/B)][d_I]: when j_s % B == B-1 the new token completes block j_s / B,
 *                 and its block key is written with the arithmetic of sgqa_compress (bit-identical)
 * Uses p->n_seqs, n_tokens (= C), n_kv_heads, head_dim, idx_dim, block. No workspace. The previous
 * B-1 index keys of a completing block must already be in idx_k_cache (earlier calls or a prefill
 * copy on the same stream). */
int sgqa_append(const sgqa_params* p, const sgqa_bf16* k_new, const sgqa_bf16* v_new, const sgqa_bf16* idx_k_new,
                const int32_t* positions, sgqa_bf16* k_cache, sgqa_bf16* v_cache, const sgqa_pages* pages,
                sgqa_bf16* idx_k_cache, sgqa_bf16* blk_k, sgqa_stream stream);

/* ---------------------------------------------------------------- FP8 K/V cache decode
 * The pages serve the model with an FP8 K/V cache to raise the effective cache capacity ("Inside
 * Step 5 Preview", Agentic RL, High-Throughput and Low-Redundancy Infrastructure). The selection is
 * unchanged (the index keys and block keys stay bf16); only the gather of the attended K/V rows
 * reads 1-byte codes, which halves the bytes of the decode's dominant kernel.
 *
 * Decode as sgqa_decode_varlen with FP8 E4M3 K/V caches:
 *   k_cache, v_cache  uint8 OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *                 the all-ones exponent with all-ones mantissa is NaN, there is no infinity), same
 *                 layouts as the bf16 caches: dense [S][G][C][D], or the pools of *pages
 *                 ([n_pages][G][page_tokens][D], one byte per element)
 *   kv_scale      [S][G][2] fp32 DEVICE: the key and value scale of (sequence s, group g); the
 *                 attended rows are code value * scale (NaN codes propagate into the output)
 *   seq_lens      [S] int32 DEVICE, or NULL: every sequence at the full capacity C = p->n_tokens
 *   pages         NULL for dense caches
 *   q, blk_k, idx_q, idx_w, topk_out, out   as in sgqa_decode
 * Every E4M3 value is exact in bf16 and the scales are applied in fp32 (the key scale inside the
 * softmax exponent, the value scale to the normalised output), so the result is that of the decode
 * over the dequantised rows up to fp32 rounding order. kv_scale == NULL -> SGQA_ERR_NULL.
 * Workspace: sgqa_workspace_size(p, SGQA_OP_DECODE). */
int sgqa_decode_fp8(const sgqa_params* p, const sgqa_bf16* q, const uint8_t* k_cache, const uint8_t* v_cache,
                    const float* kv_scale, const sgqa_pages* pages, const sgqa_bf16* blk_k,
                    const sgqa_bf16* idx_q, const float* idx_w, const int32_t* seq_lens, int32_t* topk_out,
                    sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream);

/* ---------------------------------------------------------------- training: attention gradient
 * Sparse GQA is used in training ("Inside Step 5 Preview", Sparse GQA, and the training sections):
 * the gradient below is that of sgqa_attend for fixed selections (the selection and the indexer get
 * no gradient; the pages leave the indexer's training signal open).
 *
 * Forward of sgqa_attend that also returns, for every row, the base-2 log-sum-exp of its scaled
 * logits: lse[i][h] = log2( sum_{j in J} 2^(sigma * log2(e) * <q[i][h], k[g][j]>) ). Same arguments
 * and result as sgqa_attend otherwise; lse [N][Hq] fp32 DEVICE. No workspace. */
int sgqa_attend_fwd(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                    const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out, float* lse, void* ws,
                    size_t ws_bytes, sgqa_stream stream);

/* Gradient of sgqa_attend for an upstream gradient dout [N][Hq][D] bf16, given the forward's out and
 * lse (sgqa_attend_fwd). With p the row's softmax over J and delta_i = <dout_i, out_i>:
 *   dv[g][j] = sum over rows (i, h of g) with j in J of p_ij dout[i][h]
 *   dk[g][j] = sigma * sum over those rows of p_ij (<dout[i][h], v[g][j]> - delta_i) q[i][h]
 *   dq[i][h] = sigma * sum_{j in J} p_ij (<dout[i][h], v[g][j]> - delta_i) k[g][j]
 * dq [N][Hq][D], dk, dv [G][N][D] bf16 out (fp32 sums, one bf16 rounding; keys no row attends get 0).
 * Deterministic: every sum has a fixed order (no floating-point atomics). Workspace:
 * sgqa_workspace_size(p, SGQA_OP_ATTEND_BWD): the deltas and, for dk/dv, an fp32 accumulator
 * [G][N][2D], the per-(tile, group) plan tables and work items, and the fp32 partial rows of the
 * batches of tiles (two buffers of at most 2 GiB; about 5.1 GiB in all at N = 131072, G = 8). dk/dv
 * are summed tile by tile (every key's partial rows in ascending tile order) unless that needs more
 * than 2048 batches (the longest contexts), where a key-major kernel sums every key in one place;
 * both give the same sums up to fp32 rounding order. The tile-by-tile sums of a batch run on a
 * second stream, beside the next batch's products on `stream`: the first such call on a device
 * creates that stream (default priority, non-blocking) and four events, kept until the process
 * ends; the call makes `stream` wait for that work before its last kernel, so the results are
 * ordered on `stream` as for any other call, and the call holds a lock while it enqueues (calls on
 * one device share the events). Two environment variables, read by the host code at each
 * call and meant for tests, select the design: SGQA_BWD_PATH=key forces the key-major kernel,
 * SGQA_BWD_BATCH_ROWS=<n> caps a batch at n partial rows (never below twice the largest tile's
 * rows); sgqa_workspace_size and sgqa_attend_bwd size the workspace for the design they select at
 * that moment (a smaller workspace than the call needs -> SGQA_ERR_WORKSPACE). Shapes as sgqa_attend, and
 * min(Tq, N) * r * (r - 1) < 2^32 with r = Hq / G (otherwise SGQA_ERR_SHAPE). */
int sgqa_attend_bwd(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                    const uint32_t* umask, const int32_t* ucount, const sgqa_bf16* out, const float* lse,
                    const sgqa_bf16* dout, sgqa_bf16* dq, sgqa_bf16* dk, sgqa_bf16* dv, void* ws,
                    size_t ws_bytes, sgqa_stream stream);

/* ---------------------------------------------------------------- masked-union variant
 * The pages group the top-k results of adjacent prefill tokens so that overlapping K/V reads are
 * done together ("Efficient implementation of sparse attention"). The calls above read that as:
 * every query of a tile attends over the tile's union. The variant below reads it as scheduling
 * only: the union decides which blocks are gathered, and every query still attends exactly its own
 * selection plus its own block (Figure 3 caption), causally masked -- the result then does not
 * depend on Tq (it equals the union reading at Tq = 1).
 *
 * Attention over the tile unions with every Q row restricted to its own query's set.
 *   q, k, v, umask, ucount, out   as in sgqa_attend
 *   topk   [G][N][K_B] int32  the selections (sgqa_index_topk)
 *   out[i][h] = sum_{j in J} softmax_j(sigma * <q[i][h], k[g][j]>) v[g][j],
 *          J = { j <= i : floor(j/B) in Sel(i,g) or floor(j/B) = floor(i/B) }
 * Shapes: the per-chunk membership table must fit: (64/B) * ceil((256/r + 1)/32) <= 64 words
 * (B = 8 needs r >= 2; B = 1 needs r >= 8); otherwise SGQA_ERR_SHAPE.
 * Workspace: sgqa_workspace_size(p, SGQA_OP_ATTEND_MASKED) (per-query selection bitmaps). */
int sgqa_attend_masked(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                       const int32_t* topk, const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out,
                       void* ws, size_t ws_bytes, sgqa_stream stream);

/* Whole prefill path of the variant: compress -> index_topk -> union -> masked attention, with
 * blk_k, topk, umask, ucount and the selection bitmaps in the workspace. Arguments as in
 * sgqa_prefill. Workspace: sgqa_workspace_size(p, SGQA_OP_PREFILL_MASKED). */
int sgqa_prefill_masked(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                        const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* idx_k,
                        sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* SGQA_H */
