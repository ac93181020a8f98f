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
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// The K-th largest of the n listed keys (1 <= K <= n <= 64 P) and the number of keys above it,
// by binary search over the 32-bit key between the list's minimum and maximum.
template <int P>
__device__ __forceinline__ uint32_t keys_kth_largest(const KeyRegs<P>& r, int K, int* n_above) {
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
  // Largest t in [mn, mx] with count(>= t) >= K; count(>= mn) = n >= K holds throughout.
  uint32_t lo = mn, hi = mx;
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
    if (keys_count_ge(r, mid) >= K)
      lo = mid;
    else
      hi = mid - 1;
  }
  *n_above = (lo == 0xFFFFFFFFu) ? 0 : keys_count_ge(r, lo + 1);
  return lo;
}

template <int P>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t* keys, int n, int K, int* n_above) {
  KeyRegs<P> r;
  keys_load(r, keys, n);
  return keys_kth_largest(r, K, n_above);
}

// Trim a key list to the multiset of its K largest keys (K < n); returns the K-th largest key.
template <int P>
__device__ __forceinline__ uint32_t wave_trim_keys(uint32_t* keys, int n, int K) {
  KeyRegs<P> r;
  keys_load(r, keys, n);
  int above;
  const uint32_t tau = keys_kth_largest(r, K, &above);
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

  constexpr int kRowsPerWg = WAVES * 4;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int quarter = l >> 4;
  const int l16 = l & 15;
  const uint32_t lt16 = (1u << l16) - 1u;

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

  // Stage issue: 18 wave-wide loads of 64 slots; slot s = row s / 9, piece s % 9 (piece 8 = pad).
  // Row r of the stage holds candidate block lo + (v0 + r) * stride + off.
  auto issue = [&](int v0, int buf, int stride, int off, int n_virt) {
    for (int ii = wave; ii < kStageInsts; ii += WAVES) {
      const int slot = ii * 64 + l;
      const int row = slot / kKSlots;
      int piece = slot - row * kKSlots;
      if (piece == kKSlots - 1) piece = 0;
      const int v = v0 + row;
      int b = lo + v * stride + off;
      if (v >= n_virt || b >= n_blocks) b = 0;  // beyond the candidates: any valid key (never used)
      __builtin_amdgcn_global_load_lds((const void*)(kbar + (long long)b * kIdxDim + piece * 8),
                                       (lds_void*)(stage + buf * kStageBytes + ii * 1024), 16, 0, 0);
    }
  };
  const int boff = l16 * kKRowBytes + quarter * 16;  // B operand: row l16 of a 16-block tile
  auto score_of = [&](const uint8_t* sb, int ct) -> float {
    const uint8_t* p = sb + ct * 16 * kKRowBytes + boff;
    const bf16x8 b_lo = *reinterpret_cast<const bf16x8*>(p);
    const bf16x8 b_hi = *reinterpret_cast<const bf16x8*>(p + 64);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mfma16(a_op[0], b_lo, acc);
    acc = mfma16(a_op[1], b_hi, acc);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += w4[j] * __builtin_amdgcn_fmed3f(acc[j], 0.0f, 3.402823466e38f);  // ReLU
    return s;
  };
  // Streams candidates v in [0, n_virt) (block lo + v * stride + off) through the double-buffered
  // stage; body(score, block, valid) runs for every (row, candidate) pair of this lane, after(..)
  // once per chunk.
  auto stream = [&](int n_virt, int stride, int off, auto&& body, auto&& after) {
    const int n_ch = (n_virt + kChunk - 1) / kChunk;
    if (n_ch > 0) issue(0, 0, stride, off, n_virt);
    for (int n = 0; n < n_ch; ++n) {
      wait_vm();
      __syncthreads();
      if (n + 1 < n_ch) issue((n + 1) * kChunk, (n + 1) & 1, stride, off, n_virt);
      const uint8_t* sb = stage + (n & 1) * kStageBytes;
#pragma unroll 2
      for (int ct = 0; ct < kChunk / 16; ++ct) {
        const float sc = score_of(sb, ct);
        const int v = n * kChunk + ct * 16 + l16;
        const int b = lo + v * stride + off;
        body(sc, b, v < n_virt && b < hi_lane);
      }
      after();
    }
    __syncthreads();  // the stage buffers are free again
  };
  const int n_all = hi_all - lo;

  uint32_t* my_keys = keys_all + (size_t)(wave * 4 + quarter) * cap;
  int n_cnt = 0;            // keys in this lane's row list (uniform over the quarter)
  float accept = kNegInf;   // scores >= accept are kept
  auto append = [&](float sc, int b, bool valid) {
    const bool pass = valid && sc >= accept;
    const uint64_t m = ballot(pass);
    if (m) {
      const uint32_t m16 = (uint32_t)(m >> (16 * quarter)) & 0xFFFFu;
      if (pass) my_keys[n_cnt + __popc(m16 & lt16)] = score_key(sc);
      n_cnt += __popc(m16);
    }
  };
  auto trim_full = [&]() {  // trim the rows whose list could overflow on the next chunk
    const uint64_t need_m = ballot(n_cnt + kChunk > cap);
    if (need_m) {
      lds_wait();
      for (int q = 0; q < 4; ++q) {
        if ((need_m >> (16 * q)) & 1ull) {
          const int nq = readlane(n_cnt, 16 * q);
          const uint32_t tau = wave_trim_keys<P>(keys_all + (size_t)(wave * 4 + q) * cap, nq, kb);
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
    stream(n_virt, stride, stride / 2, append, nothing);
    lds_wait();
    float est = kNegInf;
    for (int q = 0; q < 4; ++q) {
      const int nq = readlane(n_cnt, 16 * q);     // samples of row q
      const int cq = readlane(n_cand, 16 * q);    // candidates of row q
      const int ks = cq > 0 ? (int)(((long long)2 * kb * nq + cq - 1) / cq) : 0;
      if (cq > 2 * kb && ks >= 1 && ks < nq) {
        int above;
        const uint32_t t = wave_kth_largest<P>(keys_all + (size_t)(wave * 4 + q) * cap, nq, ks, &above);
        if (quarter == q) est = key_to_score(t);
      }
    }
    accept = est;
    n_cnt = 0;
  }

  // ------------------------------------------------------------------ pass 1: tau and ties
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
      const uint32_t tau = wave_kth_largest<P>(keys_all + (size_t)(wave * 4 + q) * cap, nq, kb, &above);
      if (quarter == q) {
        tau_f = key_to_score(tau);
        ties = kb - above;
      }
    }
  }

  // ------------------------------------------------------------------ pass 2: emit in order
  int n_out = 0, t_seen = 0;  // uniform over the quarter
  int32_t* out_row = valid_o ? topk + ((long long)g_o * n_tokens + row_o / n_groups) * kb : nullptr;
  auto emit = [&](float sc, int b, bool valid) {
    const bool gt = valid && sc > tau_f;
    const bool eq = valid && sc == tau_f;
    const uint32_t em16 = (uint32_t)(ballot(eq) >> (16 * quarter)) & 0xFFFFu;
    const bool keep = gt || (eq && t_seen + __popc(em16 & lt16) < ties);
    const uint32_t km16 = (uint32_t)(ballot(keep) >> (16 * quarter)) & 0xFFFFu;
    if (keep) {
      const int pos = n_out + __popc(km16 & lt16);
      out_row[pos] = b;
    }
    n_out += __popc(km16);
    t_seen += __popc(em16);
  };
  stream(n_all, 1, 0, emit, nothing);
  // Padding / counts.
  if (valid_o)
    for (int e = n_out + l16; e < kb; e += 16) out_row[e] = -1;
}

namespace {

size_t select_lds_bytes(int waves, int cap) { return (size_t)2 * kStageBytes + (size_t)waves * 4 * cap * 4; }

// Largest list capacity (multiple of 64) that fits `waves` in the LDS budget, capped at a size
// where trims are rare; 0 below the minimum (K_B plus one chunk of appends plus slack).
int select_cap(int waves, int kb, size_t lds_budget) {
  const long long avail = (long long)lds_budget - 2LL * kStageBytes - 256;  // 256 B: static LDS
  if (avail <= 0) return 0;
  int cap = (int)(avail / ((long long)waves * 4 * 4)) / 64 * 64;
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
  const size_t budget = (size_t)max_lds_per_block();
  const int waves = prefill_waves(kb, budget);
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
