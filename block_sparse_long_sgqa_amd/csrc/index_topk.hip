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
// Design (gfx950):
//  * A workgroup owns WAVES*4 consecutive rows; every wave owns 4 rows. One 16x16x32 bf16 MFMA
//    takes A = (4 rows x 4 indexer heads) x 32 dims and B = 32 dims x 16 blocks, so after the two
//    K-steps of d_I = 64 each lane holds the 4 head dots of one (row, block) pair and forms the
//    score locally (ReLU, weights, head sum) -- no cross-lane traffic.
//  * Block keys stream through LDS in chunks of 64 blocks (8 KiB, double buffered, XOR-swizzled
//    16-byte pieces); each chunk is shared by all rows of the workgroup.
//  * Selection never materialises the score matrix. Every row keeps, in LDS, a list of (key, id)
//    candidates in ascending id order plus an acceptance threshold. New scores above the threshold
//    are appended in id order (ballot + popcount compaction). When the list could overflow, the
//    wave trims it to exactly the top K_B by an exact radix select on the order-preserving 32-bit
//    key (4 passes of 8-bit digits, LDS histogram) and keeps ties at the threshold by lowest id; the
//    trim raises the threshold to the new K_B-th key. A rejected candidate is already beaten by K_B
//    others (higher key, or equal key and lower id), so the final list is the exact selection.
#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kChunk = 64;                       // candidate blocks per stage
constexpr int kStageBytes = kChunk * kIdxDim * 2;  // 8 KiB

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Byte offset of 16-byte piece `c` (0..7) of block-key row `row` inside one stage buffer.
__device__ __forceinline__ int stage_off(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

// Exact top-K of a row list (n > K entries, ascending ids) kept in LDS; the whole wave cooperates.
// Returns the threshold key tau: afterwards the list holds exactly K entries in ascending id order,
// all keys > tau plus the lowest-id entries with key == tau.
__device__ __forceinline__ uint32_t wave_trim(uint32_t* keys, uint32_t* ids, int n, int K, uint32_t* hist) {
  const int l = lane_id();
  uint32_t prefix = 0;
  uint32_t kk = (uint32_t)K;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int x = l; x < 256; x += 64) hist[x] = 0u;
    lds_wait();
    const uint32_t hi_mask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int e = l; e < n; e += 64) {
      const uint32_t k = keys[e];
      if (((k ^ prefix) & hi_mask) == 0u) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    lds_wait();
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const uint32_t local = h[0] + h[1] + h[2] + h[3];
    const uint32_t suf = wave_suffix_sum(local);  // keys in bins >= 4l
    const uint64_t ge = ballot(suf >= kk);
    const int ls = 63 - __clzll((long long)ge);
    uint32_t above = suf - local;  // keys in bins > 4l+3
    int digit = 4 * l;
    if (above + h[3] >= kk) {
      digit = 4 * l + 3;
    } else if (above + h[3] + h[2] >= kk) {
      digit = 4 * l + 2;
      above += h[3];
    } else if (above + h[3] + h[2] + h[1] >= kk) {
      digit = 4 * l + 1;
      above += h[3] + h[2];
    } else {
      above += h[3] + h[2] + h[1];
    }
    digit = readlane(digit, ls);
    above = readlane(above, ls);
    kk -= above;
    prefix |= ((uint32_t)digit) << shift;
    lds_wait();
  }
  const uint32_t tau = prefix;
  const int r = (int)kk;  // entries equal to tau that stay
  int wr = 0, ties = 0;
  const uint64_t lt = lanemask_lt();
  for (int base = 0; base < n; base += 64) {
    const int e = base + l;
    const bool v = e < n;
    const uint32_t k = v ? keys[e] : 0u;
    const uint32_t id = v ? ids[e] : 0u;
    const bool gt = v && k > tau;
    const bool eq = v && k == tau;
    const uint64_t em = ballot(eq);
    const int trank = ties + popc64(em & lt);
    const bool keep = gt || (eq && trank < r);
    const uint64_t km = ballot(keep);
    const int pos = wr + popc64(km & lt);
    if (keep) {
      keys[pos] = k;
      ids[pos] = id;
    }
    wr += popc64(km);
    ties += popc64(em);
  }
  lds_wait();
  return tau;
}

}  // namespace

// Row parameters of the two uses of the selection kernel.
//  PREFILL: row = (i, g) flattened as i*G + g (largest rows first); candidates [0, c(i)); output
//           the final ascending ids into topk [G][N][K_B].
//  DECODE:  workgroup = (sequence s, candidate slice ch); row = group g; candidates
//           [ch*slice, min(c, (ch+1)*slice)) with c = floor((L-1)/B); output the slice's exact local
//           top-K_B as (key, id) lists plus counts. The global selection is the top-K_B of the
//           concatenated slice lists (k_select_merge): a candidate in the global top-K_B is beaten
//           by fewer than K_B others overall, hence inside its slice too.
template <int WAVES, bool DECODE>
__global__ __launch_bounds__(WAVES * 64) void k_select(const uint16_t* __restrict__ qi, const float* __restrict__ w,
                                                       const uint16_t* __restrict__ kbar_all,
                                                       int32_t* __restrict__ topk, uint32_t* __restrict__ part_keys,
                                                       uint32_t* __restrict__ part_ids,
                                                       int32_t* __restrict__ part_cnt, int n_tokens, int n_groups,
                                                       int block, int kb, int cap, int n_slices, int slice_len) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;                                                       // 2 x 8 KiB
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(smem + 2 * kStageBytes);    // WAVES x 256
  uint32_t* keys_all = hist_all + WAVES * 256;                                 // WAVES*4 x cap
  uint32_t* ids_all = keys_all + (size_t)WAVES * 4 * cap;                      // WAVES*4 x cap

  constexpr int kRowsPerWg = WAVES * 4;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int quarter = l >> 4;
  const int l16 = l & 15;

  // Rows of this workgroup.
  long long r0, n_rows;
  int seq = 0, slice = 0, lo = 0, hi_all = 0;
  const uint16_t* kbar = kbar_all;
  if (DECODE) {
    seq = blockIdx.x / n_slices;
    slice = blockIdx.x % n_slices;
    r0 = 0;
    n_rows = n_groups;
    const int c = (n_tokens - 1) / block;
    lo = slice * slice_len;
    hi_all = min(c, lo + slice_len);
    kbar = kbar_all + (long long)seq * (n_tokens / block) * kIdxDim;
  } else {
    const long long wg = (long long)gridDim.x - 1 - blockIdx.x;  // largest rows first
    r0 = wg * kRowsPerWg;
    n_rows = (long long)n_tokens * n_groups;
    const long long r_last = (r0 + kRowsPerWg - 1 < n_rows) ? r0 + kRowsPerWg - 1 : n_rows - 1;
    hi_all = (int)(r_last / n_groups) / block;  // the last row has the most candidates
  }
  const int n_blocks = n_tokens / block;
  uint32_t* hist = hist_all + wave * 256;

  auto row_group = [&](long long row) -> int { return DECODE ? (int)row : (int)(row % n_groups); };
  auto row_qi = [&](long long row) -> long long {  // row index into qi [..][G][H_I][d_I]
    return DECODE ? (long long)seq * n_groups + row : row;
  };
  auto row_hi = [&](long long row) -> int {  // exclusive candidate bound of a row
    return DECODE ? hi_all : (int)(row / n_groups) / block;
  };

  // The row whose scores this lane produces (result rows 4*quarter .. +3 = row `quarter`, 4 heads).
  const long long row_o = r0 + wave * 4 + quarter;
  const bool valid_o = row_o < n_rows;
  const int g_o = valid_o ? row_group(row_o) : 0;
  const int hi_lane = valid_o ? row_hi(row_o) : 0;

  if (!DECODE && hi_all <= kb) {
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

  uint32_t* my_keys = keys_all + (size_t)(wave * 4 + quarter) * cap;
  uint32_t* my_ids = ids_all + (size_t)(wave * 4 + quarter) * cap;
  int n_cnt = 0;           // entries in this lane's row list (uniform over the quarter)
  uint32_t accept = 0u;    // keys >= accept are appended

  // Stage loader: the workgroup copies 64 block keys (512 pieces of 16 B) into a stage buffer.
  constexpr int kPieces = kChunk * 8;
  constexpr int kPerThread = (kPieces + WAVES * 64 - 1) / (WAVES * 64);
  u32x4 pre[kPerThread];
  auto load_chunk = [&](int b0) {
#pragma unroll
    for (int x = 0; x < kPerThread; ++x) {
      const int p = threadIdx.x + x * WAVES * 64;
      const int row = p >> 3, c = p & 7;
      const int b = b0 + row;
      if (p < kPieces && b < n_blocks)
        pre[x] = *reinterpret_cast<const u32x4*>(kbar + (long long)b * kIdxDim + c * 8);
      else
        pre[x] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int x = 0; x < kPerThread; ++x) {
      const int p = threadIdx.x + x * WAVES * 64;
      if (p < kPieces) *reinterpret_cast<u32x4*>(stage + buf * kStageBytes + stage_off(p >> 3, p & 7)) = pre[x];
    }
  };

  if (lo < hi_all) {
    load_chunk(lo);
    store_chunk(0);
  }
  __syncthreads();

  int buf = 0;
  for (int b0 = lo; b0 < hi_all; b0 += kChunk) {
    const bool has_next = b0 + kChunk < hi_all;
    if (has_next) load_chunk(b0 + kChunk);
    const uint8_t* sb = stage + buf * kStageBytes;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int row = ct * 16 + l16;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const bf16x8 b_lo = *reinterpret_cast<const bf16x8*>(sb + stage_off(row, quarter));
      const bf16x8 b_hi = *reinterpret_cast<const bf16x8*>(sb + stage_off(row, 4 + quarter));
      acc = mfma16(a_op[0], b_lo, acc);
      acc = mfma16(a_op[1], b_hi, acc);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) s += w4[j] * fmaxf(acc[j], 0.0f);
      const uint32_t key = score_key(s);
      const int b = b0 + row;
      const bool pass = (b < hi_lane) && (key >= accept);
      const uint64_t m = ballot(pass);
      const uint32_t m16 = (uint32_t)(m >> (16 * quarter)) & 0xFFFFu;
      const int pos = n_cnt + __popc(m16 & ((1u << l16) - 1u));
      if (pass) {
        my_keys[pos] = key;
        my_ids[pos] = (uint32_t)b;
      }
      n_cnt += __popc(m16);
    }
    // Trim rows whose list could overflow on the next chunk.
    const bool need = n_cnt + kChunk > cap;
    const uint64_t need_m = ballot(need);
    if (need_m) {
      lds_wait();
      for (int q = 0; q < 4; ++q) {
        if ((need_m >> (16 * q)) & 1ull) {
          const int nq = readlane(n_cnt, 16 * q);
          const uint32_t tau = wave_trim(keys_all + (size_t)(wave * 4 + q) * cap,
                                         ids_all + (size_t)(wave * 4 + q) * cap, nq, kb, hist);
          if (quarter == q) {
            n_cnt = kb;
            accept = tau + 1u;
          }
        }
      }
    }
    if (has_next) store_chunk(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // Final: exactly min(K_B, candidates) entries per row, ascending ids.
  lds_wait();
  for (int q = 0; q < 4; ++q) {
    const long long row = r0 + wave * 4 + q;
    if (row >= n_rows) break;
    int nq = readlane(n_cnt, 16 * q);
    uint32_t* kq = keys_all + (size_t)(wave * 4 + q) * cap;
    uint32_t* iq = ids_all + (size_t)(wave * 4 + q) * cap;
    if (nq > kb) {
      wave_trim(kq, iq, nq, kb, hist);
      nq = kb;
    }
    if (DECODE) {
      const long long base = (((long long)seq * n_slices + slice) * n_groups + row) * kb;
      for (int e = l; e < nq; e += 64) {
        part_keys[base + e] = kq[e];
        part_ids[base + e] = iq[e];
      }
      if (l == 0) part_cnt[((long long)seq * n_slices + slice) * n_groups + row] = nq;
    } else {
      const int i = (int)(row / n_groups), g = (int)(row % n_groups);
      int32_t* out = topk + ((long long)g * n_tokens + i) * kb;
      for (int e = l; e < kb; e += 64) out[e] = e < nq ? (int32_t)iq[e] : -1;
    }
  }
}

// Decode merge: one wave per (sequence, group) streams the slice lists (ascending ids) through the
// same accept / trim list and writes Sel ascending, -1 padded, to sel (and to topk_out if given).
__global__ __launch_bounds__(64) void k_select_merge(const uint32_t* __restrict__ part_keys,
                                                     const uint32_t* __restrict__ part_ids,
                                                     const int32_t* __restrict__ part_cnt, int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ topk_out, int n_groups, int kb, int cap,
                                                     int n_slices) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);
  uint32_t* keys = hist + 256;
  uint32_t* ids = keys + cap;
  const int s = blockIdx.x / n_groups, g = blockIdx.x % n_groups;
  const int l = lane_id();
  const uint64_t lt = lanemask_lt();
  int n = 0;
  uint32_t accept = 0u;
  for (int ch = 0; ch < n_slices; ++ch) {
    const long long pr = ((long long)s * n_slices + ch) * n_groups + g;
    const int cnt = part_cnt[pr];
    for (int base = 0; base < cnt; base += 64) {
      const int e = base + l;
      const bool v = e < cnt;
      const uint32_t key = v ? part_keys[pr * kb + e] : 0u;
      const uint32_t id = v ? part_ids[pr * kb + e] : 0u;
      const bool pass = v && key >= accept;
      const uint64_t m = ballot(pass);
      if (pass) {
        const int pos = n + popc64(m & lt);
        keys[pos] = key;
        ids[pos] = id;
      }
      n += popc64(m);
      if (n + 64 > cap) {
        lds_wait();
        accept = wave_trim(keys, ids, n, kb, hist) + 1u;
        n = kb;
      }
    }
  }
  lds_wait();
  if (n > kb) {
    wave_trim(keys, ids, n, kb, hist);
    n = kb;
  }
  int32_t* dst = sel + ((long long)s * n_groups + g) * kb;
  int32_t* dst2 = topk_out ? topk_out + ((long long)s * n_groups + g) * kb : nullptr;
  for (int e = l; e < kb; e += 64) {
    const int32_t val = e < n ? (int32_t)ids[e] : -1;
    dst[e] = val;
    if (dst2) dst2[e] = val;
  }
}

namespace {

int topk_cap(int kb) {
  int extra = kb > 128 ? kb : 128;
  int cap = kb + extra;
  return (cap + 63) / 64 * 64;
}

size_t topk_lds_bytes(int waves, int cap) {
  return (size_t)2 * kStageBytes + (size_t)waves * 256 * 4 + (size_t)waves * 4 * cap * 8;
}

}  // namespace

hipError_t launch_index_topk(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, int n_tokens,
                             int n_groups, int block, int kb, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_groups;
  if (n_rows == 0) return hipSuccess;
  const int cap = topk_cap(kb);
  const int lds_max = max_lds_per_block();
  int waves = 4;
  while (waves > 1 && topk_lds_bytes(waves, cap) > (size_t)lds_max) waves >>= 1;
  const size_t lds = topk_lds_bytes(waves, cap);
  if (lds > (size_t)lds_max) return hipErrorInvalidValue;
  const long long grid = (n_rows + waves * 4 - 1) / (waves * 4);
#define SGQA_TOPK_CASE(WV)                                                                                       \
  case WV: {                                                                                                     \
    hipError_t e = hipFuncSetAttribute((const void*)k_select<WV, false>,                                         \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                    \
    if (e != hipSuccess) return e;                                                                               \
    hipLaunchKernelGGL((k_select<WV, false>), dim3((unsigned)grid), dim3(WV * 64), lds, stream, qi, w, kbar,     \
                       topk, nullptr, nullptr, nullptr, n_tokens, n_groups, block, kb, cap, 0, 0);               \
    break;                                                                                                       \
  }
  switch (waves) {
    SGQA_TOPK_CASE(4)
    SGQA_TOPK_CASE(2)
    SGQA_TOPK_CASE(1)
    default:
      return hipErrorInvalidValue;
  }
#undef SGQA_TOPK_CASE
  return hipGetLastError();
}

size_t index_topk_lds_min(int kb) { return topk_lds_bytes(1, topk_cap(kb)); }

size_t decode_select_lds(int n_groups, int kb) { return topk_lds_bytes((n_groups + 3) / 4, topk_cap(kb)); }

int decode_slice_len() { return 1024; }

int decode_slice_count(int n_tokens, int block) {
  const int c = (n_tokens - 1) / block;
  const int n = (c + decode_slice_len() - 1) / decode_slice_len();
  return n < 1 ? 1 : n;
}

size_t decode_select_ws_bytes(int n_seqs, int n_tokens, int n_groups, int block, int kb) {
  const size_t n_sl = (size_t)decode_slice_count(n_tokens, block);
  return (size_t)n_seqs * n_sl * n_groups * ((size_t)kb * 8 + 4);
}

hipError_t launch_decode_select(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* sel,
                                int32_t* topk_out, void* ws, int n_seqs, int n_tokens, int n_groups, int block, int kb,
                                hipStream_t stream) {
  const int n_slices = decode_slice_count(n_tokens, block);
  const size_t n_lists = (size_t)n_seqs * n_slices * n_groups;
  uint32_t* part_keys = reinterpret_cast<uint32_t*>(ws);
  uint32_t* part_ids = part_keys + n_lists * kb;
  int32_t* part_cnt = reinterpret_cast<int32_t*>(part_ids + n_lists * kb);
  const int cap = topk_cap(kb);
  const int waves = (n_groups + 3) / 4;
  const size_t lds = topk_lds_bytes(waves, cap);
  const int lds_max = max_lds_per_block();
  if (lds > (size_t)lds_max) return hipErrorInvalidValue;
  const long long grid = (long long)n_seqs * n_slices;
#define SGQA_DSEL_CASE(WV)                                                                                       \
  case WV: {                                                                                                     \
    hipError_t e = hipFuncSetAttribute((const void*)k_select<WV, true>,                                          \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                    \
    if (e != hipSuccess) return e;                                                                               \
    hipLaunchKernelGGL((k_select<WV, true>), dim3((unsigned)grid), dim3(WV * 64), lds, stream, qi, w, kbar,      \
                       nullptr, part_keys, part_ids, part_cnt, n_tokens, n_groups, block, kb, cap, n_slices,     \
                       decode_slice_len());                                                                      \
    break;                                                                                                       \
  }
  switch (waves) {
    SGQA_DSEL_CASE(1)
    SGQA_DSEL_CASE(2)
    SGQA_DSEL_CASE(3)
    SGQA_DSEL_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef SGQA_DSEL_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t mlds = (size_t)(256 + 2 * cap) * 4;
  if (mlds > 65536) {
    e = hipFuncSetAttribute((const void*)k_select_merge, hipFuncAttributeMaxDynamicSharedMemorySize, (int)mlds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_select_merge, dim3((unsigned)(n_seqs * n_groups)), dim3(64), mlds, stream, part_keys, part_ids,
                     part_cnt, sel, topk_out, n_groups, kb, cap, n_slices);
  return hipGetLastError();
}

}  // namespace sgqa
