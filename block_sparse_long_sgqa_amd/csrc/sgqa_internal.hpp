// sgqa_internal.hpp -- launch functions shared between the kernel files and the C-ABI layer of
// libsgqa. Every launcher only enqueues work on `stream` and returns hipGetLastError(); argument
// validation happens in sgqa_api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sgqa {

// A paged K/V cache: pools [n_pages][G][page_tokens][D], position t of sequence s in pool page
// table[s * max_pages + t / page_tokens] (page_tokens a power of two, a multiple of B). table ==
// nullptr means dense per-sequence caches [S][G][capacity][D].
struct PageTable {
  const int32_t* table = nullptr;
  int max_pages = 0;
  int page_tokens = 0;
  int n_pages = 0;
};

// Append one token per sequence to the decode caches (see sgqa_append): K/V at position pos[s]
// (dense or paged), the index key into idx_cache [S][cap][d_I], and the block key into
// kbar [S][cap/B][d_I] when the token completes its block. pos[s] outside [0, cap) skips s.
hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, const uint16_t* idx_new, const int32_t* pos,
                         uint16_t* kc, uint16_t* vc, const PageTable& pages, uint16_t* idx_cache, uint16_t* kbar,
                         int n_seqs, int cap, int n_groups, int idx_dim, int block, hipStream_t stream);

// Block compression: ki [S][N][dI] -> kbar [S][N/B][dI].
hipError_t launch_compress(const uint16_t* ki, uint16_t* kbar, int n_seqs, int n_tokens, int idx_dim, int block,
                           hipStream_t stream);

// Per-query block top-k for a prefill: qi [N][G][4][64], w [G][4], kbar [N/B][64] -> topk [G][N][kb].
hipError_t launch_index_topk(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, int n_tokens,
                             int n_groups, int block, int kb, hipStream_t stream);

// Tile union: topk [G][N][kb] -> umask [G][T][W], ucount [G][T].
// Fused index -> union: the selections go straight into the (zeroed here) tile-union mask, then
// its popcounts; topk is never written.
hipError_t launch_index_union(const uint16_t* qi, const float* w, const uint16_t* kbar, uint32_t* umask,
                              int32_t* ucount, int n_tokens, int n_groups, int block, int kb, int tile,
                              hipStream_t stream);
hipError_t launch_fill_zero(uint32_t* dst, long long n, hipStream_t stream);
hipError_t launch_mask_count(const uint32_t* umask, int32_t* ucount, long long n_rows, int n_words,
                             hipStream_t stream);
// Per-query selection bitmaps selbits [G][N][W] from topk (for the masked-union attention).
hipError_t launch_sel_bitmap(const int32_t* topk, uint32_t* selbits, int n_tokens, int n_groups, int block, int kb,
                             hipStream_t stream);
// Masked-union attention: gathers by the union, keeps per Q row only its query's selection
// (selbits from launch_sel_bitmap) and own block.
hipError_t launch_attend_masked(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                                const uint32_t* selbits, uint16_t* out, int n_tokens, int n_q_heads, int n_groups,
                                int block, int tile, float scale, hipStream_t stream);
// Table bits per thread of the masked attention (1, 2 or 4); 0 = shape not supported.
int attend_masked_loads(int n_q_heads, int n_groups, int block);
hipError_t launch_union(const int32_t* topk, uint32_t* umask, int32_t* ucount, int n_tokens, int n_groups, int block,
                        int kb, int tile, hipStream_t stream);

// Gathered-block prefill attention over the tile unions.
// lse (optional, [N][Hq] fp32): base-2 log-sum-exp of every row's scaled logits, for the backward.
hipError_t launch_attend(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                         const int32_t* ucount, uint16_t* out, int n_tokens, int n_q_heads, int n_groups, int block,
                         int tile, float scale, hipStream_t stream, float* lse = nullptr);

// Workspace of the backward (attend_bwd_plan(...).bytes) and how dk/dv are computed: key-major
// (one kernel) or tile-major (per-tile partial rows in batches, then an ordered sum). The
// environment variable SGQA_BWD_PATH=key forces the key-major kernel; SGQA_BWD_BATCH_ROWS=n lowers
// the partial rows per batch (at least twice the largest union's rows).
struct BwdPlan {
  bool tile_major = false;
  int n_pairs = 0, n_batches = 0;
  long long cap_rows = 0, hstep = 0;
  size_t o_acc = 0, o_nblk = 0, o_ebase = 0, o_ipref = 0, o_bstart = 0, o_pre = 0, o_items = 0, o_part = 0;
  size_t bytes = 0;  // whole workspace (the deltas first)
};
BwdPlan attend_bwd_plan(int n_tokens, int n_q_heads, int n_groups, int block, int tile);

// Backward of launch_attend given its output and lse: dq [N][Hq][D], dk/dv [G][N][D] (bf16), from
// dout [N][Hq][D]; ws holds attend_bwd_plan(...).bytes (the deltas <dout, out> per row first).
hipError_t launch_attend_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                             const uint16_t* out, const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                             uint16_t* dv, void* ws, int n_tokens, int n_q_heads, int n_groups, int block,
                             int tile, float scale, hipStream_t stream);
size_t attend_bwd_lds_dq(int n_tokens, int block);

// Decode selection: K-bar cache [S][L/B][64], qi [S][G][4][64] -> sel [S][G][kb] (and topk_out if not
// null). lens (device, nullable): per-sequence context lengths (clamped to [1, n_tokens]); null =
// n_tokens for every sequence. Uses decode_select_ws_bytes() of workspace.
size_t decode_select_ws_bytes(int n_seqs, int n_tokens, int n_groups, int block, int kb);
hipError_t launch_decode_select(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* sel,
                                int32_t* topk_out, void* ws, int n_seqs, int n_tokens, int n_groups, int block, int kb,
                                const int32_t* lens, hipStream_t stream);

// Decode attention over Sel + own block, one workgroup per (sequence, group), straight into
// out [S][Hq][D] (no workspace).
hipError_t launch_decode_attend(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* sel,
                                uint16_t* out, int n_seqs, int ctx, int n_q_heads, int n_groups, int block, int kb,
                                float scale, const int32_t* lens, const PageTable& pages, hipStream_t stream);

// LDS a launch needs (validation rejects shapes that do not fit before anything is enqueued).
size_t index_topk_lds_min(int kb);
size_t decode_attend_lds(int kb);
size_t decode_attend_f8_lds(int kb);

// Decode attention over FP8 E4M3 K/V caches (uint8 codes, same layouts as the bf16 caches) with
// kv_scale [S][G][2] fp32 (key scale, value scale).
hipError_t launch_decode_attend_f8(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* kv_scale,
                                   const int32_t* sel, uint16_t* out, int n_seqs, int ctx, int n_q_heads,
                                   int n_groups, int block, int kb, float scale, const int32_t* lens,
                                   const PageTable& pages, hipStream_t stream);
size_t attend_lds_bytes_for(int n_tokens, int block);
constexpr size_t kGfx950LdsBytes = 160 * 1024;

// Largest dynamic LDS allocation one workgroup may use on the current device (bytes).
int max_lds_per_block();
// Compute units of the current device.
int device_cu_count();

// Once per device, before any launch: let every kernel that takes dynamic LDS use all that is left
// beside its static LDS (lds_max = the device's limit per workgroup). One function per kernel file.
hipError_t allow_full_lds(const void* fn, int lds_max);
hipError_t prepare_kernels(int lds_max);
hipError_t prepare_index_topk_kernels(int lds_max);
hipError_t prepare_union_kernels(int lds_max);
hipError_t prepare_attend_kernels(int lds_max);
hipError_t prepare_attend_bwd_kernels(int lds_max);

}  // namespace sgqa
