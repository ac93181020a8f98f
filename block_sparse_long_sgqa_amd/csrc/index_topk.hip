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
//  * A workgroup owns 4*WAVES consecutive rows (4 per wave). One 16x16x32 bf16 MFMA takes
//    A = (4 rows x 4 indexer heads) x 32 dims and B = 32 dims x 16 blocks; after the two K-steps
//    of d_I = 64 every lane holds the 4 head dots of one (row, block) pair and forms the score
//    locally (ReLU, weights, head sum): no cross-lane traffic, no score matrix in memory.
//  * Block keys stream through LDS in chunks of 128 blocks, gathered with global_load_lds into
//    double-buffered 144-byte rows (16 B of padding spread the MFMA operand reads over all banks);
//    each chunk feeds every row of the workgroup.
//  * Pass 1 finds, per row, the exact K_B-th largest score tau and how many candidates equal to
//    tau belong to the selection. Each row keeps in LDS only the keys of candidates scoring above
//    an acceptance threshold; when the list could overflow it is trimmed to the multiset of its
//    K_B largest keys and the threshold rises to the new K_B-th key (a rejected candidate is
//    already beaten by K_B others). The K-th largest key is found by binary search over the
//    order-preserving 32-bit key, counting with wave ballots (no atomics).
//  * Pass 2 recomputes the scores and emits, in ascending block order, every candidate with
//    s > tau plus the lowest-id candidates with s == tau (ballot + popcount compaction).
//  * Decode selection (one query, many candidates) is shaped differently and lives on its own.
#include <type_traits>

#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
#ifndef SGQA_TOPK_CHUNK
#define SGQA_TOPK_CHUNK 128
#endif
#ifndef SGQA_TOPK_WGS_PER_CU
#define SGQA_TOPK_WGS_PER_CU 1
#endif
constexpr int kChunk = SGQA_TOPK_CHUNK;            // candidate blocks per stage
constexpr int kKRowBytes = 144;                    // 128 B block key + 16 B pad
constexpr int kKSlots = kKRowBytes / 16;           // 9 slots of 16 B per row, the last is padding
constexpr int kStageBytes = kChunk * kKRowBytes;   // 18432 B
constexpr int kStageInsts = kChunk * kKSlots / 64;  // 18 wave-wide 16-byte loads per stage
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kListPad = 16;                       // words between row lists (spreads LDS banks)

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

// Inverse of score_key (canonical +0).
__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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

template <int P>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t* keys, int n, int K, int* n_above,
                                                     uint32_t* hist) {
  KeyRegs<P> r;
  keys_load(r, keys, n);
  return keys_kth_largest(r, K, n_above, hist);
}

// Trim a key list to the multiset of its K largest keys (K < n); returns the K-th largest key.
template <int P>
__device__ __forceinline__ uint32_t wave_trim_keys(uint32_t* keys, int n, int K, uint32_t* hist) {
  KeyRegs<P> r;
  keys_load(r, keys, n);
  int above;
  const uint32_t tau = keys_kth_largest(r, K, &above, hist);
  const int l = lane_id();
  const uint64_t lt = lanemask_lt();
  int wr = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const bool keep = r.k[j] > tau;
    const uint64_t m = ballot(keep);
    if (keep) keys[wr + popc64(m & lt)] = r.k[j];
    wr += popc64(m);
  }
  for (int e = wr + l; e < K; e += 64) keys[e] = tau;  // the tied keys that stay
  lds_wait();
  (void)above;
  return tau;
}

}  // namespace

// Row = (i, g) flattened as i*G + g (largest rows first); candidates [0, c(i)); output the
// ascending ids into topk [G][N][K_B] (-1 padded).
template <int WAVES, int P>
__global__ __launch_bounds__(WAVES * 64) void k_select(const uint16_t* __restrict__ qi, const float* __restrict__ w,
                                                       const uint16_t* __restrict__ kbar,
                                                       int32_t* __restrict__ topk, int n_tokens, int n_groups,
                                                       int block, int kb, int cap) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;                                                        // 2 x kStageBytes
  uint32_t* keys_all = reinterpret_cast<uint32_t*>(smem + 2 * kStageBytes);     // 4*WAVES x cap
  const int lstride = cap + kListPad;                                          // words per row list
  uint32_t* hist = keys_all + (size_t)WAVES * 4 * lstride + (threadIdx.x >> 6) * 256;  // this wave's 256 words

  constexpr int kRowsPerWg = WAVES * 4;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int quarter = l >> 4;
  const int l16 = l & 15;

  const long long wg = (long long)gridDim.x - 1 - blockIdx.x;  // largest rows first
  const long long r0 = wg * kRowsPerWg;
  const long long n_rows = (long long)n_tokens * n_groups;
  const long long r_last = (r0 + kRowsPerWg - 1 < n_rows) ? r0 + kRowsPerWg - 1 : n_rows - 1;
  const int lo = 0;
  const int hi_all = (int)(r_last / n_groups) / block;  // the last row has the most candidates
  const int n_blocks = n_tokens / block;

  auto row_group = [&](long long row) -> int { return (int)(row % n_groups); };
  auto row_qi = [&](long long row) -> long long { return row; };
  auto row_hi = [&](long long row) -> int { return (int)(row / n_groups) / block; };

  // The row whose scores this lane produces: row `quarter` of the wave.
  const long long row_o = r0 + wave * 4 + quarter;
  const bool valid_o = row_o < n_rows;
  const int g_o = valid_o ? row_group(row_o) : 0;
  const int hi_lane = valid_o ? row_hi(row_o) : 0;
  const int n_cand = max(0, hi_lane - lo);  // candidates of this lane's row

  if (hi_all <= kb) {
    // Every row has at most K_B candidates: all of them are selected.
    for (int q = 0; q < 4; ++q) {
      const long long row = r0 + wave * 4 + q;
      if (row >= n_rows) break;
      const int i = (int)(row / n_groups), g = (int)(row % n_groups);
      const int c = i / block;
      int32_t* out = topk + ((long long)g * n_tokens + i) * kb;
      for (int e = l; e < kb; e += 64) out[e] = e < c ? e : -1;
    }
    return;
  }

  // A operand: row (l16 / 4) of this wave, head (l16 % 4), dims 8*quarter + 32*ks.
  bf16x8 a_op[2];
  {
    const long long row_a = r0 + wave * 4 + (l16 >> 2);
    const int head = l16 & 3;
    if (row_a < n_rows) {
      const uint16_t* src = qi + (row_qi(row_a) * kIdxHeads + head) * kIdxDim + 8 * quarter;
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

  uint32_t* my_keys = keys_all + (size_t)(wave * 4 + quarter) * lstride;
  int n_cnt = 0;            // keys in this lane's row list (uniform over the quarter)
  float accept = kNegInf;   // scores >= accept are kept
  // Keys of the scores >= accept join the row's list (any order); positions from a prefix count
  // over the row's 16 lanes.
  int s_n_virt = 0, s_stride = 1, s_off = 0;  // the current stream's candidate mapping
  auto append = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
    constexpr bool kFull = decltype(full_t)::value;
    uint32_t pm = 0;  // bit ct: candidate v_first + ct passes
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const bool ok = kFull || valid_at(v_first + ct, s_n_virt, s_stride, s_off);
      pm |= (ok && sc[ct] >= accept) ? (1u << ct) : 0u;
    }
    if (!ballot(pm != 0u)) return;
    const uint32_t cnt = __popc(pm);
    const uint32_t incl = row16_prefix(cnt);
    const uint32_t total = __shfl(incl, l | 15, 64);
    uint32_t pos = n_cnt + incl - cnt;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct)
      if (pm & (1u << ct)) my_keys[pos++] = score_key(sc[ct]);
    n_cnt += total;
  };
  auto trim_full = [&]() {  // trim the rows whose list could overflow on the next chunk
    const uint64_t need_m = ballot(n_cnt + kChunk > cap);
    if (need_m) {
      lds_wait();
      for (int q = 0; q < 4; ++q) {
        if ((need_m >> (16 * q)) & 1ull) {
          const int nq = readlane(n_cnt, 16 * q);
          const uint32_t tau = wave_trim_keys<P>(keys_all + (size_t)(wave * 4 + q) * lstride, nq, kb, hist);
          if (quarter == q) {
            n_cnt = kb;
            accept = key_to_score(tau);
          }
        }
      }
    }
  };
  auto nothing = [&]() {};

  // ------------------------------------------------------------------ pass 0: starting threshold
  // A strided sample of every row's candidates gives a conservative estimate of the K_B-th score:
  // the sample quantile at which about 2*K_B candidates are expected above. It only sets where
  // pass 1 starts keeping keys; a row whose estimate turns out too high is rescanned from -inf.
  const int sample_max = min(512, cap - kChunk);
  const int stride = n_all > 2 * kb ? (n_all + sample_max - 1) / sample_max : 0;
  if (stride > 1) {
    const int n_virt = (n_all - stride / 2 + stride - 1) / stride;
    s_n_virt = n_virt;
    s_stride = stride;
    s_off = stride / 2;
    stream(n_virt, stride, stride / 2, append, nothing);
    lds_wait();
    float est = kNegInf;
    for (int q = 0; q < 4; ++q) {
      const int nq = readlane(n_cnt, 16 * q);     // samples of row q
      const int cq = readlane(n_cand, 16 * q);    // candidates of row q
      const int ks = cq > 0 ? (int)(((long long)2 * kb * nq + cq - 1) / cq) : 0;
      if (cq > 2 * kb && ks >= 1 && ks < nq) {
        int above;
        const uint32_t t = wave_kth_largest<P>(keys_all + (size_t)(wave * 4 + q) * lstride, nq, ks, &above, hist);
        if (quarter == q) est = key_to_score(t);
      }
    }
    accept = est;
    n_cnt = 0;
  }

  // ------------------------------------------------------------------ pass 1: tau and ties
  s_n_virt = n_all;
  s_stride = 1;
  s_off = 0;
  stream(n_all, 1, 0, append, trim_full);
  lds_wait();
  // A row whose starting threshold was above its K_B-th score kept fewer than K_B keys: rescan
  // those rows from -inf (the other rows keep their lists and take nothing new).
  {
    __shared__ int redo;
    if (threadIdx.x == 0) redo = 0;
    __syncthreads();
    const bool failed = n_cand > kb && n_cnt < kb;
    if (ballot(failed) && l == 0) redo = 1;
    __syncthreads();
    if (redo) {
      if (failed) {
        n_cnt = 0;
        accept = kNegInf;
      } else {
        accept = __builtin_huge_valf();
      }
      stream(n_all, 1, 0, append, trim_full);
      lds_wait();
    }
  }
  // Exact threshold per row: select everything when the row has at most K_B candidates.
  float tau_f = kNegInf;
  int ties = 0;
  for (int q = 0; q < 4; ++q) {
    const int nq = readlane(n_cnt, 16 * q);
    const int cq = readlane(n_cand, 16 * q);
    if (cq > kb) {
      int above;
      const uint32_t tau = wave_kth_largest<P>(keys_all + (size_t)(wave * 4 + q) * lstride, nq, kb, &above, hist);
      if (quarter == q) {
        tau_f = key_to_score(tau);
        ties = kb - above;
      }
    }
  }

  // ------------------------------------------------------------------ pass 2: emit in order
  int n_out = 0, t_seen = 0;  // uniform over the quarter
  // The selection is staged in the row's (now unused) key list and written out at the end: global
  // stores inside the loop would make every chunk's vmcnt wait for them as well.
  int32_t* out_row = valid_o ? topk + ((long long)g_o * n_tokens + row_o / n_groups) * kb : nullptr;
  int32_t* sel_lds = reinterpret_cast<int32_t*>(my_keys);
  // Candidates above tau, and the first `ties` equal to tau, in ascending block order: this lane's
  // 8 candidates follow those of lanes with a lower l % 16 in the same row.
  auto emit = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
    constexpr bool kFull = decltype(full_t)::value;
    uint32_t gm = 0, em = 0;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const bool ok = kFull || valid_at(v_first + ct, n_all, 1, 0);
      gm |= (ok && sc[ct] > tau_f) ? (1u << ct) : 0u;
      em |= (ok && sc[ct] == tau_f) ? (1u << ct) : 0u;
    }
    if (!ballot((gm | em) != 0u)) return;
    const uint32_t ng = __popc(gm), ne = __popc(em);
    const uint32_t incl = row16_prefix(ng | (ne << 16));  // row totals <= 128 each
    const uint32_t total = __shfl(incl, l | 15, 64);
    const int g_before = (int)((incl & 0xFFFFu) - ng), e_before = (int)((incl >> 16) - ne);
    const int rem = max(0, ties - t_seen);  // ties still to take
    int pos = n_out + g_before + min(e_before, rem);
    int e_rank = e_before;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      if (gm & (1u << ct)) {
        sel_lds[pos++] = lo + v_first + ct;
      } else if (em & (1u << ct)) {
        if (e_rank < rem) sel_lds[pos++] = lo + v_first + ct;
        ++e_rank;
      }
    }
    n_out += (int)(total & 0xFFFFu) + min((int)(total >> 16), rem);
    t_seen += (int)(total >> 16);
  };
  stream(n_all, 1, 0, emit, nothing);
  lds_wait();
  if (valid_o)
    for (int e = l16; e < kb; e += 16) out_row[e] = e < n_out ? sel_lds[e] : -1;
}

namespace {

// Stage buffers, the rows' key lists and one 256-word histogram per wave.
size_t select_lds_bytes(int waves, int cap) {
  return (size_t)2 * kStageBytes + (size_t)waves * 4 * (cap + kListPad) * 4 + (size_t)waves * 1024;
}

// Largest list capacity (multiple of 64) that fits `waves` in the LDS budget, capped at a size
// where trims are rare; 0 below the minimum (K_B plus one chunk of appends plus slack).
int select_cap(int waves, int kb, size_t lds_budget) {
  const long long avail = (long long)lds_budget - 2LL * kStageBytes - 256 - waves * 1024LL;  // 256 B: static LDS
  if (avail <= 0) return 0;
  int cap = (int)(avail / ((long long)waves * 4 * 4) - kListPad) / 64 * 64;
  const int need = kb + kChunk + 64;
  const int enough = ((4 * kb + kChunk > need ? 4 * kb + kChunk : need) + 63) / 64 * 64;
  if (cap > enough) cap = enough;
  if (cap > 4096) cap = 4096;  // trims hold at most 64 keys per lane in registers
  // Prefer the smaller register footprint when it still leaves room for K_B + a chunk or more.
  if (cap > 1024 && 1024 >= 2 * kb + kChunk) cap = 1024;
  if (cap > 2048 && 2048 >= 2 * kb + kChunk) cap = 2048;
  return cap >= need ? cap : 0;
}

// Keys per lane a trim holds in registers for a list capacity.
int keys_per_lane(int cap) { return cap <= 1024 ? 16 : (cap <= 2048 ? 32 : 64); }

int prefill_waves(int kb, size_t lds_budget) {
  for (int wv = 8; wv >= 1; wv >>= 1)
    if (select_cap(wv, kb, lds_budget) > 0) return wv;
  return 0;
}

}  // namespace

size_t index_topk_lds_min(int kb) {
  const int cap = select_cap(1, kb, kGfx950LdsBytes);
  return cap > 0 ? select_lds_bytes(1, cap) : kGfx950LdsBytes + 1;
}

hipError_t launch_index_topk(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, int n_tokens,
                             int n_groups, int block, int kb, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_groups;
  if (n_rows == 0) return hipSuccess;
  const size_t budget = (size_t)max_lds_per_block() / SGQA_TOPK_WGS_PER_CU;
#ifdef SGQA_TOPK_WAVES
  const int waves = select_cap(SGQA_TOPK_WAVES, kb, budget) > 0 ? SGQA_TOPK_WAVES : 0;
#else
  const int waves = prefill_waves(kb, budget);
#endif
  if (waves == 0) return hipErrorInvalidValue;
  const int cap = select_cap(waves, kb, budget);
  const size_t lds = select_lds_bytes(waves, cap);
  const long long grid = (n_rows + waves * 4 - 1) / (waves * 4);
  const int pk = keys_per_lane(cap);
#define SGQA_TOPK_CASE(WV, PK)                                                                                   \
  if (waves == WV && pk == PK) {                                                                                 \
    hipError_t e = hipFuncSetAttribute((const void*)k_select<WV, PK>,                                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                    \
    if (e != hipSuccess) return e;                                                                               \
    hipLaunchKernelGGL((k_select<WV, PK>), dim3((unsigned)grid), dim3(WV * 64), lds, stream, qi, w, kbar,       \
                       topk, n_tokens, n_groups, block, kb, cap);                                                 \
    return hipGetLastError();                                                                                    \
  }
  SGQA_TOPK_CASE(8, 16)
  SGQA_TOPK_CASE(4, 16)
  SGQA_TOPK_CASE(4, 32)
  SGQA_TOPK_CASE(2, 16)
  SGQA_TOPK_CASE(2, 32)
  SGQA_TOPK_CASE(2, 64)
  SGQA_TOPK_CASE(1, 16)
  SGQA_TOPK_CASE(1, 32)
  SGQA_TOPK_CASE(1, 64)
#undef SGQA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace sgqa
