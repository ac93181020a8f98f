// index_topk.hip -- indexer scores on the matrix cores fused with an exact per-row top-k.
//
// "Inside Step 5 Preview", section Sparse GQA: paragraph "Reducing indexer's cost" (block-level
// indexer, top-k over blocks), Figure 3 (every KV group selects on its own, over shared block
// keys) and paragraph "Trade-off between top-k and block size" (K_B = k / B blocks).
//
// A "row" is one (query i, group g) pair; its candidates are the blocks b < c(i) = floor(i/B) and
//   s(i,g,b) = sum_h w[g][h] * max(0, <qi[i][g][h], kbar[b]>)          (fp32)
// Sel(i,g) = the first min(K_B, c(i)) candidates in the order (s descending, b ascending).
//
// Design (gfx950)
//  * A workgroup owns 4*WAVES rows (4 per wave): one group, consecutive queries. One 16x16x32
//    bf16 MFMA takes A = (4 rows x 4 indexer heads) x 32 dims and B = 32 dims x 16 blocks; after the two K-steps
//    of d_I = 64 every lane holds the 4 head dots of one (row, block) pair and forms the score
//    locally (ReLU, weights, head sum): no cross-lane traffic, no score matrix in memory.
//  * Block keys stream through LDS in chunks of 128 blocks, gathered with global_load_lds into
//    double-buffered 144-byte rows (16 B of padding spread the MFMA operand reads over all banks);
//    each chunk feeds every row of the workgroup.
//  * Exact selection without a score matrix, in three streaming passes over the candidates:
//    pass 0 lists a strided sample of each row's keys (all of them when few) -- a complete list
//    gives the K_B-th key at once, a sample the key range where it must lie; pass 1 counts the
//    keys of that range into 256 power-of-two buckets per row (LDS atomics) and moves to the
//    bucket holding the K_B-th key, repeating on a finer scale while that bucket is wide and
//    crowded; pass 2 emits, in ascending block order, every candidate above the bucket plus the
//    bucket's members -- the first `take` of them when the bucket is one key (lowest ids win
//    ties), or all of them flagged, with their keys listed, when it is wider; the flagged ones are
//    then settled by an exact select over the listed keys. Scores are recomputed in every pass
//    (the stream of block keys through LDS is cheap next to storing them).
//  * Decode selection (one query, many candidates) is shaped differently and lives on its own.
#include <type_traits>

#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kChunk = 128;                        // candidate blocks per stage
constexpr int kKRowBytes = 144;                    // 128 B block key + 16 B pad
constexpr int kKSlots = kKRowBytes / 16;           // 9 slots of 16 B per row, the last is padding
constexpr int kStageBytes = kChunk * kKRowBytes;   // 18432 B
constexpr int kStageInsts = kChunk * kKSlots / 64;  // 18 wave-wide 16-byte loads per stage
constexpr int kListPad = 16;                       // words between row regions (spreads LDS banks)
constexpr int kSideCap = 192;                      // bucket members listed per row in the emit pass

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts; rows are lanes 16q..16q+15).
__device__ __forceinline__ uint32_t row16_prefix(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  return v;
}

// The value of the last lane of each 16-lane row, for every lane of the row (four lane reads
// instead of an LDS permute).
__device__ __forceinline__ uint32_t row16_total(uint32_t incl) {
  const uint32_t t0 = __builtin_amdgcn_readlane(incl, 15), t1 = __builtin_amdgcn_readlane(incl, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(incl, 47), t3 = __builtin_amdgcn_readlane(incl, 63);
  const int q = lane_id() >> 4;
  return q == 0 ? t0 : (q == 1 ? t1 : (q == 2 ? t2 : t3));
}

// A key list in registers: lane l holds entries l, l + 64, ... (P per lane; absent entries are 0,
// which no finite score maps to).
template <int P>
struct KeyRegs {
  uint32_t k[P];
};

template <int P>
__device__ __forceinline__ void keys_load(KeyRegs<P>& r, const uint32_t* keys, int n) {
  const int l = lane_id();
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int e = j * 64 + l;
    r.k[j] = e < n ? keys[e] : 0u;
  }
}

template <int P>
__device__ __forceinline__ int keys_count_ge(const KeyRegs<P>& r, uint32_t t) {  // t >= 1
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) cnt += popc64(ballot(r.k[j] >= t));
  return cnt;
}

// The K-th largest of the n listed keys (1 <= K <= n <= 64 P) and the number of keys above it.
// Histogram select over [min, max] of the list: every round splits the live key range into 256
// equal power-of-two buckets, counts the keys of each bucket with LDS atomics into hist (256 words
// owned by this wave; LDS operations of one wave complete in order, so no barrier is needed),
// and keeps the bucket where the running count from the top reaches K.
template <int P>
__device__ __forceinline__ uint32_t keys_kth_largest(const KeyRegs<P>& r, int K, int* n_above, uint32_t* hist) {
  const int l = lane_id();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    if (r.k[j]) mn = min(mn, r.k[j]);
    mx = max(mx, r.k[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  }
  if (mx == 0u || K < 1) {  // no keys listed: nothing to select (callers never ask for this)
    *n_above = 0;
    return 0u;
  }
  // Invariant: count(>= lo) >= K > count(>= hi) = c_hi.
  uint64_t lo = mn, hi = (uint64_t)mx + 1;
  uint32_t c_hi = 0;
  while (hi - lo > 1) {
    const int bits = 64 - __clzll((long long)(hi - lo - 1));
    const int shift = bits > 8 ? bits - 8 : 0;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(hist + 4 * l) = z;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const uint32_t x = r.k[j];
      if (x >= lo && x < hi) atomicAdd(&hist[(uint32_t)((x - lo) >> shift)], 1u);
    }
    const u32x4 hv = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
    const uint32_t above = wave_suffix_sum(local) - local + c_hi;  // count(>= bucket 4l + 4)
    const uint32_t s3 = above + hv[3], s2 = s3 + hv[2], s1 = s2 + hv[1], s0 = s1 + hv[0];
    const uint64_t m = ballot(s0 >= (uint32_t)K);  // lanes 0 .. l*, never empty while n >= K
    if (m == 0) break;                              // fewer than K keys listed: keep lo
    const int ls = 63 - __clzll((long long)m);
    const int j = s3 >= (uint32_t)K ? 3 : (s2 >= (uint32_t)K ? 2 : (s1 >= (uint32_t)K ? 1 : 0));
    const uint32_t s_next = j == 3 ? above : (j == 2 ? s3 : (j == 1 ? s2 : s1));
    const int bsel = readlane(4 * l + j, ls);
    c_hi = readlane(s_next, ls);
    lo += (uint64_t)bsel << shift;
    const uint64_t nhi = lo + (1ull << shift);
    hi = nhi < hi ? nhi : hi;
  }
  *n_above = (int)c_hi;
  return (uint32_t)lo;
}

}  // namespace

// A workgroup owns the rows (i, g) of one group g and 4*WAVES consecutive queries i (the heaviest
// query ranges are launched first); candidates [0, c(i)); output the ascending ids into
// topk [G][N][K_B] (-1 padded).
//
// LDS: the double-buffered stage, then per row a region A of kb + kSideCap words (the sample keys
// of pass 0, later the row's output list) and a region B of 256 words (the histogram of pass 1,
// the scratch of a list select, later the keys of the threshold bucket's members), kListPad words
// apart.
//
// UNION: instead of writing topk, every selected id and the row's own block are ORed into the
// tile-union bitmask umask [G][T][W] (bit b % 32 of word b / 32 of row (g, floor(i / tile))), which
// the caller has zeroed: the fused index -> union path that never materialises topk.
template <int WAVES, int P, bool UNION>
__global__ __launch_bounds__(WAVES * 64) void k_select(const uint16_t* __restrict__ qi, const float* __restrict__ w,
                                                       const uint16_t* __restrict__ kbar,
                                                       int32_t* __restrict__ topk, int n_tokens, int n_groups,
                                                       int block, int kb, uint32_t* __restrict__ umask, int tile,
                                                       int n_tiles, int n_words) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;                                                        // 2 x kStageBytes
  const int out_cap = (kb + 3) / 4 * 4 + kSideCap;                             // region A words
  const int rstride = out_cap + 256 + kListPad;                                // words per row
  uint32_t* rows_lds = reinterpret_cast<uint32_t*>(smem + 2 * kStageBytes);

  constexpr int kRowsPerWg = WAVES * 4;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int quarter = l >> 4;
  const int l16 = l & 15;

  // Workgroup = (group g, queries i0 .. i0 + 4*WAVES - 1), the heaviest query ranges first; the
  // row of lane quarter q of wave w is query i0 + 4w + q.
  const long long wg = (long long)gridDim.x - 1 - blockIdx.x;
  const int g_wg = (int)(wg % n_groups);
  const int i0 = (int)(wg / n_groups) * kRowsPerWg;
  const int i_last = min(i0 + kRowsPerWg, n_tokens) - 1;
  const int lo = 0;
  const int hi_all = i_last / block;  // the last row has the most candidates
  const int n_blocks = n_tokens / block;

  const int i_o = i0 + wave * 4 + quarter;
  const bool valid_o = i_o < n_tokens;
  const int g_o = g_wg;
  const int hi_lane = valid_o ? i_o / block : 0;
  const int n_cand = max(0, hi_lane - lo);  // candidates of this lane's row

  // The union mask row of (i, g).
  auto mask_row = [&](int i, int g) -> uint32_t* {
    return umask + ((long long)g * n_tiles + i / tile) * n_words;
  };
  if (hi_all <= kb) {
    // Every row has at most K_B candidates: all of them are selected.
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + wave * 4 + q, g = g_wg;
      if (i >= n_tokens) break;
      const int c = i / block;
      if constexpr (UNION) {  // blocks 0 .. c: the selection and the own block, a word at a time
        uint32_t* m = mask_row(i, g);
        for (int wd = l; wd <= (c >> 5); wd += 64) {
          const int hi_bit = c - 32 * wd;  // bits 0 .. hi_bit of this word
          atomicOr(&m[wd], hi_bit >= 31 ? 0xFFFFFFFFu : ((2u << hi_bit) - 1u));
        }
      } else {
        int32_t* out = topk + ((long long)g * n_tokens + i) * kb;
        for (int e = l; e < kb; e += 64) out[e] = e < c ? e : -1;
      }
    }
    return;
  }

  // A operand: row (l16 / 4) of this wave, head (l16 % 4), dims 8*quarter + 32*ks.
  bf16x8 a_op[2];
  {
    const int ia = i0 + wave * 4 + (l16 >> 2);
    const int head = l16 & 3;
    if (ia < n_tokens) {
      const uint16_t* src = qi + (((long long)ia * n_groups + g_wg) * kIdxHeads + head) * kIdxDim + 8 * quarter;
      a_op[0] = *reinterpret_cast<const bf16x8*>(src);
      a_op[1] = *reinterpret_cast<const bf16x8*>(src + 32);
    } else {
      for (int e = 0; e < 8; ++e) {
        a_op[0][e] = (__bf16)0.0f;
        a_op[1][e] = (__bf16)0.0f;
      }
    }
  }
  float w4[4];
  for (int j = 0; j < 4; ++j) w4[j] = w[g_o * kIdxHeads + j];

  // Stage issue: 18 wave-wide loads of 64 slots; slot s = stage row s / 9, piece s % 9 (piece 8 =
  // pad). Stage row R = 16 ct + j holds candidate v0 + kTiles j + ct, so that tile ct (rows 16 ct ..
  // 16 ct + 15, read by lanes j = l % 16) gives lane j the candidates kTiles j .. kTiles j + 7 of
  // the chunk in ascending order over the tiles. Candidate v is block lo + v * stride + off. The
  // (row, piece) of this lane's slots do not change from chunk to chunk.
  constexpr int kTiles = kChunk / 16;
  constexpr int kIssuePerWave = (kStageInsts + WAVES - 1) / WAVES;
  int is_row[kIssuePerWave], is_piece[kIssuePerWave];
#pragma unroll
  for (int x = 0; x < kIssuePerWave; ++x) {
    const int slot = (wave + x * WAVES) * 64 + l;
    is_row[x] = slot / kKSlots;
    const int piece = slot - is_row[x] * kKSlots;
    is_piece[x] = piece == kKSlots - 1 ? 0 : piece;
  }
  auto issue = [&](int v0, int buf, int stride, int off, int n_virt) {
#pragma unroll
    for (int x = 0; x < kIssuePerWave; ++x) {
      const int ii = wave + x * WAVES;
      if (ii < kStageInsts) {
        const int v = v0 + (is_row[x] & 15) * kTiles + (is_row[x] >> 4);
        int b = lo + v * stride + off;
        if (v >= n_virt || b >= n_blocks) b = 0;  // beyond the candidates: any valid key (never used)
        __builtin_amdgcn_global_load_lds((const void*)(kbar + (long long)b * kIdxDim + is_piece[x] * 8),
                                         (lds_void*)(stage + buf * kStageBytes + ii * 1024), 16, 0, 0);
      }
    }
  };
  const int boff = l16 * kKRowBytes + quarter * 16;  // B operand: row l16 of a 16-block tile
  // Scores of one staged chunk: all operand reads first, then all products, then the per-lane
  // ReLU / weight / head sum, so that LDS and matrix-core latencies overlap across the 8 tiles.
  auto chunk_scores = [&](const uint8_t* sb, float (&sc)[kTiles]) {
    bf16x8 b_lo[kTiles], b_hi[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const uint8_t* p = sb + ct * 16 * kKRowBytes + boff;
      b_lo[ct] = *reinterpret_cast<const bf16x8*>(p);
      b_hi[ct] = *reinterpret_cast<const bf16x8*>(p + 64);
    }
    f32x4 acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      acc[ct] = mfma16(a_op[0], b_lo[ct], z);
    }
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = mfma16(a_op[1], b_hi[ct], acc[ct]);
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) s += w4[j] * __builtin_amdgcn_fmed3f(acc[ct][j], 0.0f, 3.402823466e38f);  // ReLU
      sc[ct] = s;
    }
  };
  // Smallest candidate bound over this wave's rows: chunks entirely below it need no checks.
  int hi_wave = hi_lane;
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) hi_wave = min(hi_wave, __shfl_xor(hi_wave, off, 64));
  // Streams candidates v in [0, n_virt) (block lo + v * stride + off) through the double-buffered
  // stage. For every chunk, body(sc, v_first, full) gets this lane's 8 scores, for candidates
  // v_first .. v_first + 7 (ascending), and whether every candidate of the wave's rows in the chunk
  // is valid (a compile-time tag); after() runs once per chunk.
  auto stream = [&](int n_virt, int stride, int off, auto&& body, auto&& after) {
    const int n_ch = (n_virt + kChunk - 1) / kChunk;
    if (n_ch > 0) issue(0, 0, stride, off, n_virt);
    for (int n = 0; n < n_ch; ++n) {
      wait_vm();
      __syncthreads();
      if (n + 1 < n_ch) issue((n + 1) * kChunk, (n + 1) & 1, stride, off, n_virt);
      float sc[kTiles];
      chunk_scores(stage + (n & 1) * kStageBytes, sc);
      const int v_end = (n + 1) * kChunk;
      const int v_first = n * kChunk + l16 * kTiles;
      if (v_end <= n_virt && lo + (v_end - 1) * stride + off < hi_wave)
        body(sc, v_first, std::true_type());
      else
        body(sc, v_first, std::false_type());
      after();
    }
    __syncthreads();  // the stage buffers are free again
  };
  // Validity of this lane's candidate v_first + ct.
  auto valid_at = [&](int v, int n_virt, int stride, int off) -> bool {
    return v < n_virt && lo + v * stride + off < hi_lane;
  };
  const int n_all = hi_all - lo;

  uint32_t* my_a = rows_lds + (size_t)(wave * 4 + quarter) * rstride;  // this lane's row: region A
  uint32_t* my_b = my_a + out_cap;                                       // region B
  auto row_a = [&](int q) { return rows_lds + (size_t)(wave * 4 + q) * rstride; };
  auto row_b = [&](int q) { return rows_lds + (size_t)(wave * 4 + q) * rstride + out_cap; };

  // ------------------------------------------------------------------ pass 0: sample
  // Every row's candidates, or a strided sample of them when there are more than sample_cap, go
  // into region A. A complete list gives the exact K_B-th key at once; a sample gives the range
  // for the histogram of pass 1.
  const int sample_cap = min(512, out_cap) / 64 * 64;
  const int stride = n_all > sample_cap ? (n_all + sample_cap - 1) / sample_cap : 1;
  const int s_off = stride / 2;
  const int s_virt = (n_all - s_off + stride - 1) / stride;
  int n_cnt = 0;  // keys listed for this lane's row (uniform over the quarter)
  auto append_all = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
    constexpr bool kFull = decltype(full_t)::value;
    uint32_t pm = 0;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct)
      pm |= (kFull || valid_at(v_first + ct, s_virt, stride, s_off)) ? (1u << ct) : 0u;
    if (!ballot(pm != 0u)) return;
    const uint32_t cnt = __popc(pm);
    const uint32_t incl = row16_prefix(cnt);
    const uint32_t total = row16_total(incl);
    uint32_t pos = n_cnt + incl - cnt;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct)
      if (pm & (1u << ct)) my_a[pos++] = score_key(sc[ct]);
    n_cnt += total;
  };
  auto nothing = [&]() {};

  // Row state (uniform over the row's 16 lanes). Modes: every candidate selected; ties (keys above
  // t_hi selected, the first `take` keys equal to t_lo = t_hi in block order too); bucket (keys
  // above t_hi selected, keys in [t_lo, t_hi] listed for an exact select after the emit pass);
  // histogram (the threshold bucket is not narrow enough yet).
  enum { kAll = 0, kTies = 1, kBucket = 2, kHist = 3 };
  int mode = kAll;
  uint32_t t_lo = 1u, t_hi = 0u;
  int take = 0;                 // kTies: equal keys to take; kBucket / kHist: keys still to select
  uint32_t h_lo = 0u, h_hi = 0xFFFFFFFFu;  // kHist: keys in [h_lo, h_hi] are bucketed ...
  int h_shift = 0;              // ... into bucket (key - h_lo) >> h_shift
  bool h_open = false;          // ... except that with an open range bucket 255 takes every key above

  stream(s_virt, stride, s_off, append_all, nothing);
  lds_wait();
  for (int q = 0; q < 4; ++q) {
    const int nq = readlane(n_cnt, 16 * q);
    const int cq = readlane(n_cand, 16 * q);
    if (cq <= kb) continue;  // every candidate is selected
    uint32_t* ka = row_a(q);
    KeyRegs<8> r;
    keys_load(r, ka, nq);
    if (stride == 1) {  // complete list: the exact K_B-th key and its ties
      int above;
      const uint32_t tau = keys_kth_largest(r, kb, &above, row_b(q));
      if (quarter == q) {
        mode = kTies;
        t_lo = t_hi = tau;
        take = kb - above;
      }
    } else {
      // Histogram range: from the sample key with about 4 K_B candidates expected at or above it
      // (the lowest sample key if that is more than the sample) up to the largest sample key.
      int ks = (int)(((long long)4 * kb * nq + cq - 1) / cq);
      ks = ks < 1 ? 1 : (ks > nq ? nq : ks);
      int above;
      const uint32_t lo_k = keys_kth_largest(r, ks, &above, row_b(q));
      uint32_t mx = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, r.k[j]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
      const uint64_t width = (uint64_t)mx - lo_k + 1;
      const int bits = 64 - __clzll((long long)(width - 1 | 1));
      if (quarter == q) {
        mode = kHist;
        take = kb;
        h_lo = lo_k;
        h_hi = 0xFFFFFFFFu;
        h_open = true;
        h_shift = bits > 8 ? bits - 8 : 0;
      }
    }
  }

  // ------------------------------------------------------------------ pass 1: histograms
  // Rows still in histogram mode count their keys in [h_lo, h_hi] per bucket (LDS atomics into
  // region B), then move to the bucket that holds their K_B-th key: a one-key bucket gives the
  // exact threshold (ties mode), a bucket of at most kSideCap keys is listed in the emit pass
  // (bucket mode), a larger one is histogrammed again on a 256 times finer scale.
  __shared__ int any_hist;
  for (;;) {
    if (threadIdx.x == 0) any_hist = 0;
    __syncthreads();
    if (ballot(mode == kHist) && l == 0) any_hist = 1;
    __syncthreads();
    if (!any_hist) break;
    if (mode == kHist) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(my_b + 64 * j + 4 * l16) = z;
    }
    const bool hist_row = mode == kHist;
    auto count = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
      constexpr bool kFull = decltype(full_t)::value;
      if (!ballot(hist_row)) return;
#pragma unroll
      for (int ct = 0; ct < kTiles; ++ct) {
        const uint32_t key = score_key(sc[ct]);
        const bool ok = hist_row && (kFull || valid_at(v_first + ct, n_all, 1, 0)) && key >= h_lo && key <= h_hi;
        if (ok) {
          uint32_t bk = (key - h_lo) >> h_shift;
          bk = bk > 255u ? 255u : bk;
          atomicAdd(&my_b[bk], 1u);
        }
      }
    };
    stream(n_all, 1, 0, count, nothing);
    lds_wait();
    for (int q = 0; q < 4; ++q) {
      if (readlane((int)(mode == kHist), 16 * q) == 0) continue;
      const int need = readlane(take, 16 * q);
      const uint32_t lo_q = readlane(h_lo, 16 * q), hi_q = readlane(h_hi, 16 * q);
      const int sh_q = readlane(h_shift, 16 * q);
      const bool open_q = readlane((int)h_open, 16 * q) != 0;
      const u32x4 hv = *reinterpret_cast<const u32x4*>(row_b(q) + 4 * l);
      const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
      const uint32_t above = wave_suffix_sum(local) - local;  // keys in buckets >= 4l + 4
      const uint32_t s3 = above + hv[3], s2 = s3 + hv[2], s1 = s2 + hv[1], s0 = s1 + hv[0];
      const uint64_t m = ballot(s0 >= (uint32_t)need);
      if (m == 0) {
        // Fewer than `need` keys in the range. On the first histogram the sampled lower end was too
        // high: count every key >= 1 on a coarse scale next time. When that range already held
        // every key >= 1, the remaining keys are 0 (only a NaN score maps there): the K_B-th key is
        // 0 and the first (need - count) of them in block order complete the selection.
        const bool full_range = lo_q == 1u && hi_q == 0xFFFFFFFFu && !open_q;
        const int in_range = (int)readlane(s0, 0);
        if (quarter == q) {
          if (full_range) {
            mode = kTies;
            t_lo = t_hi = 0u;
            take = need - in_range;
          } else {
            h_lo = 1u;
            h_hi = 0xFFFFFFFFu;
            h_open = false;
            h_shift = 24;
          }
        }
        continue;
      }
      const int ls = 63 - __clzll((long long)m);
      const int j = s3 >= (uint32_t)need ? 3 : (s2 >= (uint32_t)need ? 2 : (s1 >= (uint32_t)need ? 1 : 0));
      const uint32_t s_next = j == 3 ? above : (j == 2 ? s3 : (j == 1 ? s2 : s1));
      const uint32_t in_b = j == 3 ? hv[3] : (j == 2 ? hv[2] : (j == 1 ? hv[1] : hv[0]));
      const int bsel = readlane(4 * l + j, ls);
      const int need2 = need - (int)readlane(s_next, ls);  // keys still to select inside the bucket
      const int cnt_b = (int)readlane(in_b, ls);
      const uint64_t b_lo = (uint64_t)lo_q + ((uint64_t)bsel << sh_q);
      uint64_t b_hi = (open_q && bsel == 255) ? 0xFFFFFFFFull : b_lo + (1ull << sh_q) - 1;
      if (b_hi > hi_q) b_hi = hi_q;
      if (quarter == q) {
        take = need2;
        if (b_hi == b_lo) {
          mode = kTies;
          t_lo = t_hi = (uint32_t)b_lo;
        } else if (cnt_b <= kSideCap) {
          mode = kBucket;
          t_lo = (uint32_t)b_lo;
          t_hi = (uint32_t)b_hi;
        } else {
          const uint64_t width = b_hi - b_lo + 1;
          const int bits = 64 - __clzll((long long)(width - 1));
          h_lo = (uint32_t)b_lo;
          h_hi = (uint32_t)b_hi;
          h_open = false;
          h_shift = bits > 8 ? bits - 8 : 0;
        }
      }
    }
  }

  // ------------------------------------------------------------------ pass 2: emit in order
  // In block order, every candidate above t_hi, and the candidates in [t_lo, t_hi]: in ties mode the
  // first `take` of them, in bucket mode all of them, flagged (bit 31) in the output list with their
  // keys listed in region B, to be decided once the bucket's exact threshold is known.
  const bool all_row = mode == kAll;
  const bool bucket_row = mode == kBucket;
  int n_out = 0, t_seen = 0, n_side = 0;  // uniform over the quarter
  int32_t* out_a = reinterpret_cast<int32_t*>(my_a);
  auto emit = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
    constexpr bool kFull = decltype(full_t)::value;
    uint32_t gm = 0, em = 0;
    uint32_t keys[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const bool ok = kFull || valid_at(v_first + ct, n_all, 1, 0);
      keys[ct] = score_key(sc[ct]);
      gm |= (ok && (all_row || keys[ct] > t_hi)) ? (1u << ct) : 0u;
      em |= (ok && !all_row && keys[ct] >= t_lo && keys[ct] <= t_hi) ? (1u << ct) : 0u;
    }
    if (!ballot((gm | em) != 0u)) return;
    const uint32_t ng = __popc(gm), ne = __popc(em);
    const uint32_t incl = row16_prefix(ng | (ne << 16));  // row totals <= 128 each
    const uint32_t total = row16_total(incl);
    const int g_before = (int)((incl & 0xFFFFu) - ng), e_before = (int)((incl >> 16) - ne);
    const int rem = bucket_row ? 0x7FFFFFFF : max(0, take - t_seen);  // members still to take
    // This lane takes its first min(ne, rem - e_before) members (all of them in bucket mode).
    const int k_take = min((int)ne, max(0, rem - e_before));
    uint32_t et = 0u;
    for (uint32_t t = em, j = 0; j < (uint32_t)k_take; ++j) {
      et |= t & (0u - t);
      t &= t - 1u;
    }
    uint32_t sm = gm | et;
    int pos = n_out + g_before + min(e_before, rem);
    int side = n_side + e_before;
    // Taken candidates in ascending order; the loop runs as often as the busiest lane takes one.
    while (sm) {
      const int ct = __builtin_ctz(sm);
      sm &= sm - 1u;
      const bool flag = bucket_row && ((em >> ct) & 1u);
      out_a[pos++] = (lo + v_first + ct) | (flag ? (int)0x80000000u : 0);
      if (flag) {
        uint32_t key = keys[0];
#pragma unroll
        for (int j = 1; j < kTiles; ++j) key = ct == j ? keys[j] : key;
        my_b[side++] = key;
      }
    }
    const int tot_e = (int)(total >> 16);
    n_out += (int)(total & 0xFFFFu) + min(tot_e, rem);
    t_seen += tot_e;
    n_side += bucket_row ? tot_e : 0;
  };
  stream(n_all, 1, 0, emit, nothing);
  lds_wait();

  // ------------------------------------------------------------------ output
  // Bucket rows: the exact threshold tau among the listed bucket keys (binary search on the key,
  // counting with ballots), then the flagged entries with key > tau and the first (need - above)
  // with key == tau stay. Every row is written out in order, -1 padded.
  // Union output: the tiles this workgroup's queries fall in are ORed together in LDS (the stage
  // buffers are free now) and each non-zero word is then ORed into umask once; when they do not fit,
  // every bit goes to umask directly.
  const int t0 = i0 / tile, n_wt = i_last / tile - t0 + 1;
  const bool lds_union = UNION && (long long)n_wt * n_words * 4 <= 2LL * kStageBytes;
  uint32_t* umask_lds = reinterpret_cast<uint32_t*>(stage);
  if (lds_union) {
    for (int x = threadIdx.x; x < n_wt * n_words; x += blockDim.x) umask_lds[x] = 0u;
    __syncthreads();
  }
  for (int q = 0; q < 4; ++q) {
    const int i = i0 + wave * 4 + q, g = g_wg;
    if (i >= n_tokens) break;
    int32_t* out = UNION ? nullptr : topk + ((long long)g * n_tokens + i) * kb;
    uint32_t* mrow = !UNION ? nullptr : (lds_union ? umask_lds + (i / tile - t0) * n_words : mask_row(i, g));
    auto put_bit = [&](int b) { atomicOr(&mrow[b >> 5], 1u << (b & 31)); };
    if (UNION && l == 0) put_bit(i / block);  // the own block
    const int32_t* list = reinterpret_cast<const int32_t*>(row_a(q));
    const int nq = readlane(n_out, 16 * q);
    if (readlane((int)bucket_row, 16 * q) == 0) {
      if constexpr (UNION) {
        for (int e = l; e < nq; e += 64) put_bit(list[e]);
      } else {
        for (int e = l; e < kb; e += 64) out[e] = e < nq ? list[e] : -1;
      }
      continue;
    }
    const uint32_t* sk = row_b(q);
    const int ns = readlane(n_side, 16 * q);
    const int need = readlane(take, 16 * q);
    KeyRegs<kSideCap / 64> r;
    keys_load(r, sk, ns);
    // tau = the largest t with count(keys >= t) >= need.
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = tau | (1u << bit);
      if (keys_count_ge(r, t) >= need) tau = t;
    }
    const int ties = need - keys_count_ge(r, tau + 1u);  // tau < 2^32 - 1: a listed key is above it
    int wr = 0, j_side = 0, t_cnt = 0;
    for (int e0 = 0; e0 < nq; e0 += 64) {
      const int e = e0 + l;
      const int32_t v = e < nq ? list[e] : 0;
      const bool flagged = e < nq && v < 0;
      const uint64_t fm = ballot(flagged);
      const int js = j_side + popc64(fm & lanemask_lt());
      const uint32_t key = flagged ? sk[js] : 0u;
      const bool tie = flagged && key == tau;
      const uint64_t tm = ballot(tie);
      const int tr = t_cnt + popc64(tm & lanemask_lt());
      const bool keep = e < nq && (!flagged || key > tau || (tie && tr < ties));
      const uint64_t km = ballot(keep);
      if (keep) {
        if constexpr (UNION)
          put_bit(v & 0x7FFFFFFF);
        else
          out[wr + popc64(km & lanemask_lt())] = v & 0x7FFFFFFF;
      }
      wr += popc64(km);
      j_side += popc64(fm);
      t_cnt += popc64(tm);
    }
    if constexpr (!UNION)
      for (int e = wr + l; e < kb; e += 64) out[e] = -1;
  }
  if (lds_union) {
    __syncthreads();
    for (int x = threadIdx.x; x < n_wt * n_words; x += blockDim.x) {
      const uint32_t m = umask_lds[x];
      if (m) atomicOr(mask_row((t0 + x / n_words) * tile, g_wg) + x % n_words, m);
    }
  }
}

namespace {

// Stage buffers and the per-row regions.
size_t select_lds_bytes(int waves, int kb) {
  return (size_t)2 * kStageBytes + (size_t)waves * 4 * ((kb + 3) / 4 * 4 + kSideCap + 256 + kListPad) * 4;
}

int prefill_waves(int kb, size_t lds_budget) {
  for (int wv = 8; wv >= 1; wv >>= 1)
    if (select_lds_bytes(wv, kb) + 256 <= lds_budget) return wv;  // 256 B: static LDS
  return 0;
}

}  // namespace

size_t index_topk_lds_min(int kb) { return select_lds_bytes(1, kb) + 256; }

namespace {

// One launch of k_select; topk (UNION = false) or the zeroed umask (UNION = true) receives the
// selections.
template <bool UNION>
hipError_t launch_select(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, uint32_t* umask,
                         int n_tokens, int n_groups, int block, int kb, int tile, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_groups;
  if (n_rows == 0) return hipSuccess;
  const int waves = prefill_waves(kb, (size_t)max_lds_per_block());
  if (waves == 0) return hipErrorInvalidValue;
  const size_t lds = select_lds_bytes(waves, kb);
  const long long grid = (long long)n_groups * ((n_tokens + waves * 4 - 1) / (waves * 4));
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int n_words = ((n_tokens + block - 1) / block + 31) / 32;
#define SGQA_TOPK_CASE(WV)                                                                                       \
  if (waves == WV) {                                                                                             \
    hipLaunchKernelGGL((k_select<WV, 8, UNION>), dim3((unsigned)grid), dim3(WV * 64), lds, stream, qi, w, kbar,  \
                       topk, n_tokens, n_groups, block, kb, umask, tile, n_tiles, n_words);                      \
    return hipGetLastError();                                                                                    \
  }
  SGQA_TOPK_CASE(8)
  SGQA_TOPK_CASE(4)
  SGQA_TOPK_CASE(2)
  SGQA_TOPK_CASE(1)
#undef SGQA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t prepare_index_topk_kernels(int lds_max) {
  const void* fns[] = {(const void*)k_select<8, 8, false>, (const void*)k_select<4, 8, false>,
                       (const void*)k_select<2, 8, false>, (const void*)k_select<1, 8, false>,
                       (const void*)k_select<8, 8, true>,  (const void*)k_select<4, 8, true>,
                       (const void*)k_select<2, 8, true>,  (const void*)k_select<1, 8, true>};
  for (const void* fn : fns) {
    const hipError_t e = allow_full_lds(fn, lds_max);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_index_topk(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, int n_tokens,
                             int n_groups, int block, int kb, hipStream_t stream) {
  return launch_select<false>(qi, w, kbar, topk, nullptr, n_tokens, n_groups, block, kb, 1, stream);
}

hipError_t launch_index_union(const uint16_t* qi, const float* w, const uint16_t* kbar, uint32_t* umask,
                              int32_t* ucount, int n_tokens, int n_groups, int block, int kb, int tile,
                              hipStream_t stream) {
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int n_words = ((n_tokens + block - 1) / block + 31) / 32;
  hipError_t e = launch_fill_zero(umask, (long long)n_groups * n_tiles * n_words, stream);
  if (e == hipSuccess) e = launch_select<true>(qi, w, kbar, nullptr, umask, n_tokens, n_groups, block, kb, tile, stream);
  if (e == hipSuccess) e = launch_mask_count(umask, ucount, (long long)n_groups * n_tiles, n_words, stream);
  return e;
}

}  // namespace sgqa
