// attend.hip -- gathered-block causal GQA flash attention (prefill over tile unions, decode split-K).
//
// "Inside Step 5 Preview", section Sparse GQA, Figure 3: the attention main path loads the original
// (uncompressed) K/V of the selected history blocks and, in the query's own block, only the
// causally visible positions. Paragraph "Efficient implementation of sparse attention": during
// prefill the union over a tile of adjacent queries is attended by every query of the tile, which
// turns many small per-token gathers into one dense matrix-core workload per (tile, KV group).
//
// For head h of group g = h / r and query i in tile t:
//   out[i][h] = sum_{j in J} softmax_j(sigma * <q[i][h], k[g][j]>) v[g][j],
//   J = { j <= i : floor(j/B) in U(t,g) }           (decode: U = Sel + own block, i = L-1)
//
// gfx950 design
//  * Workgroup = the Q rows (query, head) of one (tile, group) pair that share the same K/V
//    stream; every wave owns QT tiles of 32 Q rows (QT = 2 in prefill: 64 rows per wave, so each
//    K/V byte read from LDS feeds twice the matrix-core work).
//  * The union bitmask is expanded once into an ascending block list in LDS. K/V are gathered in
//    chunks of 64 keys (64/B blocks; one B = 8 block is 2 KiB contiguous per tensor) through
//    registers into double-buffered, XOR-swizzled LDS tiles.
//  * Scores are computed transposed, S^T = K Q^T (32x32x16 bf16 MFMA, fp32 accumulate), so a lane
//    holds 32 keys of a single Q row: the online-softmax max/sum need one cross-lane exchange.
//  * O^T += V^T P^T: P comes straight from the score registers (cvt to bf16); the V^T operand is
//    read from the row-major V tile with ds_read_b64_tr_b16 (two 4x16 transposing reads per
//    operand), in the key order the score registers already have.
//  * fp32 online softmax in the exp2 domain; causal / tail masking only on the chunks that need it.
//  * Launch order is XCD-aware: consecutive workgroup ids go to different XCDs, so the
//    (tile, group) pairs are dealt round-robin over the 8 XCDs and all parts of one pair (same K/V
//    stream) land on the same XCD's L2; with G = 8 every XCD serves one KV group.
#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 128;
constexpr int kKeys = 64;            // keys per chunk
constexpr int kTileBytes = kKeys * kD * 2;  // 16 KiB per tensor per chunk
constexpr int kStageBytes = 2 * kTileBytes + kKeys * 4;  // K, V, token table
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMinit = -1.0e30f;

__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
// Byte offset of the 16-byte piece `c` (0..15) of key row `row` in a K or V tile.
__device__ __forceinline__ int kv_off(int row, int c) { return row * 256 + ((c ^ swz(row)) << 4); }

template <int QT>
struct AttnState {
  f32x16 o[QT][4];  // O^T tiles: [d-tile][32 d x 32 rows], column = this lane's row
  float m[QT];      // running max (log2 domain)
  float l[QT];      // running denominator
};

template <int QT>
__device__ __forceinline__ void state_init(AttnState<QT>& st) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[qt][dt][j] = 0.0f;
    st.m[qt] = kMinit;
    st.l[qt] = 0.0f;
  }
}

// One 64-key chunk for the QT Q tiles of this wave.
//   kt/vt: K and V tiles (row-major, swizzled); tok: token ids of the 64 keys (INT_MAX = invalid)
//   row_pos[qt]: query position of this lane's Q row in tile qt (for the causal mask)
template <int QT>
__device__ __forceinline__ void attn_chunk(const uint8_t* kt_lds, const uint8_t* vt_lds, const int* tok,
                                           const bf16x8 (&qreg)[QT][8], AttnState<QT>& st, float scale_log2,
                                           bool masked, const int (&row_pos)[QT]) {
  const int l = lane_id();
  const int hi = l >> 5;
  f32x16 s[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[qt][kt][j] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_lds + kv_off(kt * 32 + (l & 31), 2 * ks + hi));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma32(a, qreg[qt][ks], s[qt][kt]);
    }
  }

  bf16x8 pb[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = s[qt][kt][j] * scale_log2;
        if (masked) {
          const int key = kt * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
          if (tok[key] > row_pos[qt]) x = kNegInf;
        }
        s[qt][kt][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(st.m[qt], mx);
    const float alpha = exp2f(st.m[qt] - m_new);
    float sum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = exp2f(s[qt][kt][j] - m_new);
        s[qt][kt][j] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 32, 64);
    st.l[qt] = st.l[qt] * alpha + sum;
    st.m[qt] = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[qt][dt][j] *= alpha;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[qt][ss][e] = (__bf16)s[qt][ss >> 1][8 * (ss & 1) + e];
  }

  // V^T operand: lane group (l / 16) -> d half (dgrp) and key half (khalf); two transposing
  // reads each give 4 keys of this lane's d.
  const int grp = l >> 4;
  const int dgrp = grp & 1, khalf = grp >> 1, s16 = l & 15;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d0 = dt * 32 + 16 * dgrp + 4 * (s16 & 3);
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      i16x4 r2[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 16 * ss + 8 * r + 4 * khalf + (s16 >> 2);
        const int off = row * 256 + (((d0 >> 3) ^ swz(row)) << 4) + ((d0 & 7) << 1);
        r2[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt_lds + off));
      }
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 cat = __builtin_shufflevector(r2[0], r2[1], 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma32(a, pb[qt][ss], st.o[qt][dt]);
    }
  }
}

// Register staging of one chunk: NT threads copy 64 K rows and 64 V rows (16-byte pieces).
template <int NT>
struct ChunkRegs {
  static constexpr int kPer = (kKeys * 16 + NT - 1) / NT;
  u32x4 k[kPer];
  u32x4 v[kPer];
  int tok_mine;
};

// tok_of(key) -> token id or -1 (invalid). kbase/vbase: rows of this (sequence, group).
template <int NT, typename TokFn>
__device__ __forceinline__ void chunk_load(ChunkRegs<NT>& cr, const uint16_t* kbase, const uint16_t* vbase,
                                           TokFn tok_of) {
#pragma unroll
  for (int x = 0; x < ChunkRegs<NT>::kPer; ++x) {
    const int p = threadIdx.x + x * NT;
    const int row = p >> 4, c = p & 15;
    int tk = -1;
    if (p < kKeys * 16) tk = tok_of(row);
    if (tk >= 0) {
      cr.k[x] = *reinterpret_cast<const u32x4*>(kbase + (long long)tk * kD + c * 8);
      cr.v[x] = *reinterpret_cast<const u32x4*>(vbase + (long long)tk * kD + c * 8);
    } else {
      cr.k[x] = u32x4{0u, 0u, 0u, 0u};
      cr.v[x] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  cr.tok_mine = (threadIdx.x < kKeys) ? tok_of((int)threadIdx.x) : -1;
}

template <int NT>
__device__ __forceinline__ void chunk_store(const ChunkRegs<NT>& cr, uint8_t* stage) {
#pragma unroll
  for (int x = 0; x < ChunkRegs<NT>::kPer; ++x) {
    const int p = threadIdx.x + x * NT;
    if (p < kKeys * 16) {
      const int row = p >> 4, c = p & 15;
      *reinterpret_cast<u32x4*>(stage + kv_off(row, c)) = cr.k[x];
      *reinterpret_cast<u32x4*>(stage + kTileBytes + kv_off(row, c)) = cr.v[x];
    }
  }
  if (threadIdx.x < kKeys) {
    int* tok = reinterpret_cast<int*>(stage + 2 * kTileBytes);
    tok[threadIdx.x] = cr.tok_mine >= 0 ? cr.tok_mine : 0x7FFFFFFF;
  }
}

// Block-wide exclusive scan of one value per thread (NT threads); returns the exclusive prefix and
// writes the total to *total. `scratch` holds NT/64 + 1 ints of LDS.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int l = lane_id(), wave = threadIdx.x >> 6;
  const int incl = (int)wave_prefix_sum((uint32_t)v);
  if (l == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int x = 0; x < NT / 64; ++x) {
    const int s = scratch[x];
    if (x < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

}  // namespace

// ------------------------------------------------------------------------------------ prefill

template <int WAVES, int QT>
__global__ __launch_bounds__(WAVES * 64) void k_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint32_t* __restrict__ umask,
                                                       uint16_t* __restrict__ out, int n_tokens, int n_q_heads,
                                                       int n_groups, int block, int tile, float scale_log2,
                                                       int n_words, int parts, int n_pairs) {
  constexpr int NT = WAVES * 64;
  constexpr int kRowsWg = WAVES * 32 * QT;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;                                            // 2 x kStageBytes
  int* scan = reinterpret_cast<int*>(smem + 2 * kStageBytes);       // WAVES + 1 ints (padded to 16)
  uint16_t* list = reinterpret_cast<uint16_t*>(smem + 2 * kStageBytes + 16 * ((WAVES + 4) / 4));

  // XCD-aware decode of the workgroup id into (pair, part).
  const int x = blockIdx.x;
  const int slot = x >> 3, xcd = x & 7;
  const int pair = (slot / parts) * 8 + xcd;
  const int part = slot % parts;
  if (pair >= n_pairs) return;
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int t = n_tiles - 1 - pair / n_groups;  // heaviest tiles first
  const int g = pair % n_groups;
  const int r = n_q_heads / n_groups;

  const int l = lane_id(), wave = threadIdx.x >> 6;
  const int i0 = t * tile;
  const int tile_rows = ((i0 + tile <= n_tokens) ? tile : n_tokens - i0) * r;
  const int row0 = part * kRowsWg;
  if (row0 >= tile_rows) return;
  const int row_last = (row0 + kRowsWg <= tile_rows ? row0 + kRowsWg : tile_rows) - 1;
  const int i_lo = i0 + row0 / r, i_hi = i0 + row_last / r;
  const int c_hi = i_hi / block;  // no block above the last query's own block is visible

  // Expand U(t,g) restricted to blocks <= c_hi into the ascending list.
  int n_list;
  {
    const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
    const int n_w = c_hi / 32 + 1;
    const int per = (n_w + NT - 1) / NT;
    const int w0 = threadIdx.x * per;
    int cnt = 0;
    for (int e = 0; e < per; ++e) {
      const int wd = w0 + e;
      if (wd < n_w) {
        uint32_t m = mrow[wd];
        if (wd == n_w - 1 && (c_hi & 31) != 31) m &= (2u << (c_hi & 31)) - 1u;
        cnt += __popc(m);
      }
    }
    int total;
    int pos = block_exclusive_scan<NT>(cnt, scan, &total);
    for (int e = 0; e < per; ++e) {
      const int wd = w0 + e;
      if (wd < n_w) {
        uint32_t m = mrow[wd];
        if (wd == n_w - 1 && (c_hi & 31) != 31) m &= (2u << (c_hi & 31)) - 1u;
        while (m) {
          const int b = __ffs(m) - 1;
          m &= m - 1u;
          list[pos++] = (uint16_t)(wd * 32 + b);
        }
      }
    }
    n_list = total;
    __syncthreads();
  }

  // Q operand (B of S^T): lane column = Q row (l % 32) of tile qt; 8 k-steps of 16 dims.
  bf16x8 qreg[QT][8];
  int row_pos[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row0 + (wave * QT + qt) * 32 + (l & 31);
    const bool valid = row < tile_rows;
    const int i = i0 + (valid ? row / r : 0);
    const int h = g * r + (valid ? row % r : 0);
    row_pos[qt] = valid ? i : -1;
    const uint16_t* src = q + ((long long)i * n_q_heads + h) * kD + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (valid) {
        qreg[qt][ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[qt][ks][e] = (__bf16)0.0f;
      }
    }
  }

  AttnState<QT> st;
  state_init(st);

  const uint16_t* kbase = k + (long long)g * n_tokens * kD;
  const uint16_t* vbase = v + (long long)g * n_tokens * kD;
  const int n_keys = n_list * block;
  const int n_chunks = (n_keys + kKeys - 1) / kKeys;
  // Smallest query of this wave (masking is needed once a chunk reaches past it).
  int wave_i_min = 0x7FFFFFFF;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row0 + (wave * QT + qt) * 32;
    if (row < tile_rows) wave_i_min = min(wave_i_min, i0 + row / r);
  }
  (void)i_lo;

  auto tok_at = [&](int chunk, int key) -> int {
    const int kp = chunk * kKeys + key;
    if (kp >= n_keys) return -1;
    const int tk = (int)list[kp / block] * block + (kp % block);
    return tk < n_tokens ? tk : -1;
  };

  ChunkRegs<NT> cr;
  if (n_chunks > 0) {
    chunk_load<NT>(cr, kbase, vbase, [&](int key) { return tok_at(0, key); });
    chunk_store<NT>(cr, stage);
  }
  __syncthreads();
  for (int n = 0; n < n_chunks; ++n) {
    const int buf = n & 1;
    const bool has_next = n + 1 < n_chunks;
    if (has_next) chunk_load<NT>(cr, kbase, vbase, [&](int key) { return tok_at(n + 1, key); });
    const uint8_t* sb = stage + buf * kStageBytes;
    const int* tok = reinterpret_cast<const int*>(sb + 2 * kTileBytes);
    // The chunk's last valid key has the largest token; mask only if it can exceed a query.
    const int last_kp = min((n + 1) * kKeys, n_keys) - 1;
    const int last_tok = (int)list[last_kp / block] * block + (last_kp % block);
    const bool masked = ((n + 1) * kKeys > n_keys) || (last_tok > wave_i_min);
    if (wave_i_min != 0x7FFFFFFF)
      attn_chunk<QT>(sb, sb + kTileBytes, tok, qreg, st, scale_log2, masked, row_pos);
    if (has_next) chunk_store<NT>(cr, stage + (buf ^ 1) * kStageBytes);
    __syncthreads();
  }

  // out[i][h][d] = O^T[d][row] / l
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row0 + (wave * QT + qt) * 32 + (l & 31);
    if (row >= tile_rows) continue;
    const int i = i0 + row / r, h = g * r + row % r;
    const float inv = 1.0f / st.l[qt];
    uint16_t* dst = out + ((long long)i * n_q_heads + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + 8 * a + 4 * (l >> 5);
        uint2 pk;
        pk.x = pack_bf16x2(st.o[qt][dt][4 * a] * inv, st.o[qt][dt][4 * a + 1] * inv);
        pk.y = pack_bf16x2(st.o[qt][dt][4 * a + 2] * inv, st.o[qt][dt][4 * a + 3] * inv);
        *reinterpret_cast<uint2*>(dst + d) = pk;
      }
  }
}

namespace {
constexpr int kPrefillWaves = 4;
constexpr int kPrefillQT = 2;

size_t attend_lds_bytes(int waves, int list_cap) {
  return (size_t)2 * kStageBytes + 16 * ((waves + 4) / 4) + (size_t)list_cap * 2;
}
}  // namespace

size_t attend_lds_bytes_for(int n_tokens, int block) {
  const int nbc = (n_tokens + block - 1) / block;
  return attend_lds_bytes(kPrefillWaves, (nbc + 7) / 8 * 8);
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                         const int32_t* ucount, uint16_t* out, int n_tokens, int n_q_heads, int n_groups, int block,
                         int tile, float scale, hipStream_t stream) {
  (void)ucount;
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int nbc = (n_tokens + block - 1) / block;
  const int n_words = (nbc + 31) / 32;
  const int r = n_q_heads / n_groups;
  const int rows_wg = kPrefillWaves * 32 * kPrefillQT;
  const int tile_rows = (tile < n_tokens ? tile : n_tokens) * r;
  const int parts = (tile_rows + rows_wg - 1) / rows_wg;
  const int n_pairs = n_tiles * n_groups;
  if (n_pairs == 0) return hipSuccess;
  const int list_cap = (nbc + 7) / 8 * 8;
  const size_t lds = attend_lds_bytes(kPrefillWaves, list_cap);
  if (lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  const long long grid = (long long)((n_pairs + 7) / 8) * 8 * parts;
  const float scale_log2 = scale * 1.4426950408889634f;
  auto kern = k_attend<kPrefillWaves, kPrefillQT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPrefillWaves * 64), lds, stream, q, k, v, umask, out, n_tokens,
                     n_q_heads, n_groups, block, tile, scale_log2, n_words, parts, n_pairs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ decode

// Split-K decode attention. Workgroup (one wave) = (sequence s, group g, split p): the Q rows are
// the r heads of group g (one 32-row tile, r <= 32 valid); its keys are list entries
// [p*per, (p+1)*per) of Sel(s,g) + {own block}. Writes unnormalised partial O, max and sum.
__global__ __launch_bounds__(64) void k_decode_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                      const uint16_t* __restrict__ vc,
                                                      const int32_t* __restrict__ sel, float* __restrict__ part_o,
                                                      float* __restrict__ part_ml, int n_seqs, int ctx, int n_q_heads,
                                                      int n_groups, int block, int kb, int n_split, int per_split,
                                                      float scale_log2) {
  constexpr int NT = 64;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;
  int* blocks = reinterpret_cast<int*>(smem + 2 * kStageBytes);  // per_split entries

  const int p = blockIdx.x % n_split;
  const int sg = blockIdx.x / n_split;
  const int s = sg / n_groups, g = sg % n_groups;
  const int r = n_q_heads / n_groups;
  const int l = lane_id();
  const int i_q = ctx - 1;
  const int own = i_q / block;

  // Entries of this split: Sel entries (ascending, -1 padded) then the own block.
  const int32_t* srow = sel + ((long long)s * n_groups + g) * kb;
  int n_sel = 0;
  for (int e = l; e < kb; e += 64) n_sel += srow[e] >= 0 ? 1 : 0;
  for (int off = 32; off >= 1; off >>= 1) n_sel += __shfl_xor(n_sel, off, 64);
  const int n_ent = n_sel + 1;
  const int e0 = p * per_split;
  const int e1 = min(n_ent, e0 + per_split);
  const int n_here = max(0, e1 - e0);
  for (int e = l; e < n_here; e += 64) blocks[e] = (e0 + e < n_sel) ? srow[e0 + e] : own;
  __syncthreads();

  bf16x8 qreg[1][8];
  int row_pos[1];
  {
    const int hh = l & 31;
    const bool valid = hh < r;
    row_pos[0] = valid ? i_q : -1;
    const uint16_t* src = q + ((long long)s * n_q_heads + g * r + (valid ? hh : 0)) * kD + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (valid) {
        qreg[0][ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[0][ks][e] = (__bf16)0.0f;
      }
    }
  }
  AttnState<1> st;
  state_init(st);
  const long long seq_off = ((long long)s * n_groups + g) * ctx * kD;
  const uint16_t* kbase = kc + seq_off;
  const uint16_t* vbase = vc + seq_off;
  const int n_keys = n_here * block;
  const int n_chunks = (n_keys + kKeys - 1) / kKeys;
  auto tok_at = [&](int chunk, int key) -> int {
    const int kp = chunk * kKeys + key;
    if (kp >= n_keys) return -1;
    const int tk = blocks[kp / block] * block + (kp % block);
    return tk < ctx ? tk : -1;
  };
  ChunkRegs<NT> cr;
  if (n_chunks > 0) {
    chunk_load<NT>(cr, kbase, vbase, [&](int key) { return tok_at(0, key); });
    chunk_store<NT>(cr, stage);
  }
  __syncthreads();
  for (int n = 0; n < n_chunks; ++n) {
    const int buf = n & 1;
    const bool has_next = n + 1 < n_chunks;
    if (has_next) chunk_load<NT>(cr, kbase, vbase, [&](int key) { return tok_at(n + 1, key); });
    const uint8_t* sb = stage + buf * kStageBytes;
    const int* tok = reinterpret_cast<const int*>(sb + 2 * kTileBytes);
    attn_chunk<1>(sb, sb + kTileBytes, tok, qreg, st, scale_log2, true, row_pos);
    if (has_next) chunk_store<NT>(cr, stage + (buf ^ 1) * kStageBytes);
    __syncthreads();
  }
  // Partials: part_o [S][G][n_split][r][D], part_ml [S][G][n_split][r][2]
  const int hh = l & 31;
  if (hh < r) {
    const long long pr = (((long long)s * n_groups + g) * n_split + p) * r + hh;
    float* dst = part_o + pr * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + 8 * a + 4 * (l >> 5);
        *reinterpret_cast<float4*>(dst + d) =
            make_float4(st.o[0][dt][4 * a], st.o[0][dt][4 * a + 1], st.o[0][dt][4 * a + 2], st.o[0][dt][4 * a + 3]);
      }
    if (l < 32) {
      part_ml[pr * 2 + 0] = st.m[0];
      part_ml[pr * 2 + 1] = st.l[0];
    }
  }
}

// Fixed-order combine of the split partials: one workgroup (128 threads = D) per (s, head).
__global__ __launch_bounds__(128) void k_decode_combine(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml, uint16_t* __restrict__ out,
                                                        int n_q_heads, int n_groups, int n_split) {
  const int sh = blockIdx.x;
  const int s = sh / n_q_heads, h = sh % n_q_heads;
  const int r = n_q_heads / n_groups;
  const int g = h / r, hh = h % r;
  const int d = threadIdx.x;
  float m = kMinit;
  for (int p = 0; p < n_split; ++p) {
    const long long pr = (((long long)s * n_groups + g) * n_split + p) * r + hh;
    m = fmaxf(m, part_ml[pr * 2]);
  }
  float acc = 0.0f, den = 0.0f;
  for (int p = 0; p < n_split; ++p) {
    const long long pr = (((long long)s * n_groups + g) * n_split + p) * r + hh;
    const float wgt = exp2f(part_ml[pr * 2] - m);
    den += part_ml[pr * 2 + 1] * wgt;
    acc += part_o[pr * kD + d] * wgt;
  }
  out[((long long)s * n_q_heads + h) * kD + d] = (uint16_t)f32_to_bf16_bits(acc / den);
}

size_t decode_attend_part_bytes(int n_seqs, int n_q_heads, int n_split) {
  return (size_t)n_seqs * n_q_heads * n_split * (kD + 2) * sizeof(float);
}

int decode_split_count(int kb) {
  // Entries (<= kb + 1) per split: about 32 blocks each.
  const int n = (kb + 1 + 31) / 32;
  return n < 1 ? 1 : n;
}

hipError_t launch_decode_attend(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* sel,
                                void* part_ws, uint16_t* out, int n_seqs, int ctx, int n_q_heads, int n_groups,
                                int block, int kb, float scale, hipStream_t stream) {
  const int n_split = decode_split_count(kb);
  const int per_split = (kb + 1 + n_split - 1) / n_split;
  float* part_o = reinterpret_cast<float*>(part_ws);
  float* part_ml = part_o + (size_t)n_seqs * n_q_heads * n_split * kD;
  const size_t lds = (size_t)2 * kStageBytes + (size_t)per_split * 4;
  if (lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  if (lds > 65536) {
    hipError_t e =
        hipFuncSetAttribute((const void*)k_decode_attend, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const long long grid = (long long)n_seqs * n_groups * n_split;
  hipLaunchKernelGGL(k_decode_attend, dim3((unsigned)grid), dim3(64), lds, stream, q, kc, vc, sel, part_o, part_ml,
                     n_seqs, ctx, n_q_heads, n_groups, block, kb, n_split, per_split, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_combine, dim3((unsigned)(n_seqs * n_q_heads)), dim3(kD), 0, stream, part_o, part_ml, out,
                     n_q_heads, n_groups, n_split);
  return hipGetLastError();
}

}  // namespace sgqa
