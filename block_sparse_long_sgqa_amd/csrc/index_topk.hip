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
//    bf16 MFMA takes A = (4 rows x 4 indexer heads) x 32 dims and B = 32 dims x 16 blocks; after
//    the two K-steps of d_I = 64 every lane holds the 4 head dots of one (row, block) pair and
//    forms the score locally (ReLU, weights, head sum): no cross-lane traffic, no score matrix.
//  * Block keys stream through LDS in chunks of 64 blocks, staged through registers into
//    double-buffered 144-byte rows (16 B of padding spread the MFMA operand reads over all banks);
//    each chunk feeds every row of the workgroup, and every wave reads its operands a chunk ahead
//    of its products. Lane j of a row sees candidates 4j .. 4j+3 of a chunk, so ascending block
//    order is lane-major. (Loading the operands straight from the L2 cache into every wave's
//    registers, with no stage and no barrier, measured 1.5x slower: the shared stage divides the
//    L2 traffic by the number of waves.)
//  * The selection is VALU work, and one wave per SIMD issues VALU at half the rate of two. The
//    first shape has four waves (16 rows) per workgroup in at most 80 KiB of LDS, so two
//    workgroups share a CU (two waves per SIMD): while the waves of one wait at a chunk barrier
//    for a wave that is cutting its buffer, the other's keep the SIMDs busy. The 64-block chunk
//    keeps the LDS that small.
//  * Exact selection in ONE streaming pass over the candidates, with a buffer per row in LDS of
//    C >= K_B + 64 entries (order key, block id; room for K_B plus one chunk's appends), filled in
//    ascending block order:
//    - a strided sample of at most 576 candidates per row (the same blocks for the whole
//      workgroup) gives a threshold tau0 with, by a margin of two standard deviations of the
//      sample quantile, at least K_B candidates at or above it in most rows; rows with at most C
//      candidates take every candidate instead;
//    - the pass appends every candidate whose fp32 score is not below the row's threshold (one
//      compare per candidate; the order key is formed only for appended ones). A chunk that
//      would overflow a buffer first cuts it: to the entries at or above a key bound t that
//      leaves between K_B and K_B + 32 of them (t at or below the K_B-th key, usually found by a
//      few probes), or, when ties make that impossible, to exactly its K_B best
//      entries (key descending, among equal keys the earliest = lowest block ids) with t the
//      K_B-th key; the row's threshold becomes "strictly above t": every candidate at or below
//      it has K_B better ones already, so it cannot enter the final top-K_B;
//    - a row whose sampled threshold let fewer than min(K_B, c) candidates through (a two-sigma
//      event) runs the pass again taking every candidate: the result is exact either way, and the
//      margin only trades the appends and cuts of the pass against the rare second pass;
//    - each buffer is finally cut to exactly its K_B best and written out (still in ascending
//      order).
//    A cut searches the key values for its bound with the whole wave: every probe counts the
//    keys at or above a value with ballots (no LDS, no atomics); then it compacts the buffer in
//    place with ballot prefix counts.
//  * Decode selection (one query, many candidates) is shaped differently and lives on its own.
#include <math.h>

#include <type_traits>

#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {


constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kChunk = 64;                         // candidate blocks per stage
constexpr int kKRowBytes = 144;                    // 128 B block key + 16 B pad
constexpr int kStageBytes = kChunk * kKRowBytes;   // 9216 B
constexpr int kSampleCap = 576;                    // sampled candidates per row (512: 1-2 % slower; 640: mixed)
// A cut in the middle of the stream keeps between K_B and K_B + kCutSlack entries (at most C - kChunk,
// so that a chunk's appends still fit): a bound found in a few probes (an exact cut, which resolves
// ties at the K_B-th key, costs about twice as much).
constexpr int kCutSlack = 32;
constexpr int kStaticLds = 256;                    // bound on the kernel's static LDS
constexpr int kRowPad = 16;                        // pad entries after every row buffer
// Width of the sample margin: tau0 has at least ks = (mean + kSampleSigmas * sd + 1) sample keys
// at or above it, mean and sd those of the number of sample keys at or above the true K_B-th key
// (and at most ks + ks / 8 + 1: any such value bounds the threshold as safely, and the search for
// one stops after a few probes). Measured at 128K (32K, 32K with independent queries): 3 sigma
// 22.0 ms (2.67, 2.68), 2.5 21.2 (2.56, 2.57), 2 20.6 (2.49, 2.51), 1.5 20.0 (2.43, 2.53), 1 20.1
// (2.60, 2.83), 0.5 22.5 (3.04, 3.44): below ~2 the second passes cost more than the appends saved.
constexpr float kSampleSigmas = 2.0f;

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The value of the last lane of each 16-lane row, for every lane of the row (one DPP broadcast
// of lane 15 within each row, row_newbcast:15).
__device__ __forceinline__ uint32_t row16_total(uint32_t incl) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x15F, 0xF, 0xF, false);
}

// Sum over the lanes above this one (exclusive suffix sum), and the wave total.
__device__ __forceinline__ uint32_t wave_suffix_excl(uint32_t v, uint32_t* total) {
  const uint32_t incl = row16_prefix(v);
  const uint32_t r0 = __builtin_amdgcn_readlane((int)incl, 15), r1 = __builtin_amdgcn_readlane((int)incl, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)incl, 47), r3 = __builtin_amdgcn_readlane((int)incl, 63);
  const int q = lane_id() >> 4;
  const uint32_t before = (q > 0 ? r0 : 0u) + (q > 1 ? r1 : 0u) + (q > 2 ? r2 : 0u);
  *total = r0 + r1 + r2 + r3;
  return *total - (before + incl);
}

// The fp32 bits / value whose order key (score_key) is k.
__device__ __forceinline__ uint32_t key_bits(uint32_t k) { return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k; }
__device__ __forceinline__ float key_to_float(uint32_t k) { return __uint_as_float(key_bits(k)); }

// Order key of a buffered score (its raw fp32 bits): score_key, with the one bit pattern that
// maps to 0 (a NaN) moved to 1, so that 0 can mark an absent entry; and back to fp32 bits.
__device__ __forceinline__ uint32_t kept_key(uint32_t raw) {
  const uint32_t k = score_key(__uint_as_float(raw));
  return k > 1u ? k : 1u;
}

// Row threshold for "order key >= t" as an fp32 value thr: a score s passes iff !(s < thr) (NaN
// scores always pass and are ordered by their keys later). Keys above that of +inf give +inf
// (such candidates are dropped by the next cut).
__device__ __forceinline__ float threshold_of(uint32_t t) {
  return t > 0xFF800000u ? __builtin_inff() : key_to_float(t);
}

// Cuts one row's buffer (fp32 score bits kb_, ids ib_; n entries in ascending block order) to its
// K best entries -- keys descending, among equal keys the earliest -- in place and in order, with
// the whole wave. Requires n > K >= 1 and n <= 64 P. Returns the K-th key.
// With cap > K (a cut in the middle of the stream) it may instead keep every entry whose key is at
// least a bound t at or below the K-th key, when between K and cap entries are that large: every
// dropped entry still has K better ones, which is all a later exact cut needs. Returns t then.
// Either way, a candidate arriving later with a key at or below the returned value has K better
// entries before it, and *n_kept gets the number of entries kept.
template <int P, typename IdT>
__device__ __forceinline__ uint32_t cut_to(uint32_t* kb_, IdT* ib_, int n, int K, int cap = 0, int* n_kept = nullptr) {
  const int l = lane_id();
  uint32_t k[P], id[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {  // every entry slot is inside the buffer: load all, then mask
    k[j] = kb_[j * 64 + l];
    id[j] = (uint32_t)ib_[j * 64 + l];
  }
#pragma unroll
  for (int j = 0; j < P; ++j) k[j] = j * 64 + l < n ? kept_key(k[j]) : 0u;
  int above, n_at;
  const uint32_t tau = kth_largest(k, K, &above, cap, &n_at);
  const bool loose = n_at <= cap;  // keep every key >= tau
  if (n_kept) *n_kept = loose ? n_at : K;
  const uint64_t lt = lanemask_lt();
  const int need = K - above;  // without the loose bound: entries equal to tau that stay, the first ones
  int wpos = 0, tseen = 0;
#pragma unroll
  for (int j0 = 0; j0 < P; j0 += kMaskGroup) {
    uint64_t km[kMaskGroup];  // the keep masks of a group of entries, then their writes
#pragma unroll
    for (int j = 0; j < kMaskGroup; ++j) {
      if (j0 + j >= P) {
        km[j] = 0ull;
      } else if (loose) {
        km[j] = ballot(k[j0 + j] >= tau);
      } else {
        const bool eq = k[j0 + j] == tau;  // absent entries are 0 < tau
        const uint64_t em = ballot(eq);
        km[j] = ballot(k[j0 + j] > tau || (eq && tseen + popc64(em & lt) < need));
        tseen += popc64(em);
      }
    }
#pragma unroll
    for (int j = 0; j < kMaskGroup; ++j) {
      if (j0 + j < P && ((km[j] >> l) & 1u)) {
        const int dst = wpos + popc64(km[j] & lt);
        kb_[dst] = key_bits(k[j0 + j]);
        ib_[dst] = (IdT)id[j0 + j];
      }
      wpos += popc64(km[j]);
    }
  }
  return tau;
}

// The keys of a list of fp32 score bits in registers (for the sample threshold): lane l holds
// entries l, l + 64, ...; every slot up to 64 P must be readable.
template <int P>
__device__ __forceinline__ void keys_load(uint32_t (&k)[P], const uint32_t* bits, int n) {
  const int l = lane_id();
#pragma unroll
  for (int j = 0; j < P; ++j) k[j] = bits[j * 64 + l];
#pragma unroll
  for (int j = 0; j < P; ++j) k[j] = j * 64 + l < n ? kept_key(k[j]) : 0u;
}

}  // namespace

// A workgroup owns the rows (i, g) of one group g and 4*WAVES consecutive queries i (the heaviest
// query ranges are launched first); candidates [0, c(i)); output the ascending ids into
// topk [G][N][K_B] (-1 padded).
//
// LDS: the double-buffered stage, then per row a buffer of C = 64 P
// fp32 score bits and, after all rows' scores, their block ids (IdT: uint16 when every block id
// fits, else int32). Each row buffer is followed by kRowPad pad entries: lane j of the row writes
// the candidates it does not keep to pad entry j, so the append needs no branch.
//
// UNION: instead of writing topk, every selected id and the row's own block are ORed into the
// tile-union bitmask umask [G][T][W] (bit b % 32 of word b / 32 of row (g, floor(i / tile))), which
// the caller has zeroed: the fused index -> union path that never materialises topk.
//
// Shapes whose LDS lets two workgroups share a CU get the register budget of two waves per SIMD
// (which also keeps the products' results in VGPRs).
template <int WAVES, int P, typename IdT>
constexpr int kSelectLds = 2 * kStageBytes + WAVES * 4 * (64 * P + kRowPad) * (4 + (int)sizeof(IdT));
template <int WAVES, int P, typename IdT>
constexpr int kSelectWavesPerSimd = kSelectLds<WAVES, P, IdT> + kStaticLds <= kGfx950LdsBytes / 2 ? 2 : 1;

template <int WAVES, int P, typename IdT, bool UNION>
__global__ __launch_bounds__(WAVES * 64, (kSelectWavesPerSimd<WAVES, P, IdT>)) void k_select(
    const uint16_t* __restrict__ qi, const float* __restrict__ w, const uint16_t* __restrict__ kbar,
    int32_t* __restrict__ topk, int n_tokens, int n_groups, int block, int kb, uint32_t* __restrict__ umask, int tile,
    int n_tiles, int n_words) {
  constexpr int C = 64 * P;
  constexpr int CS = C + kRowPad;  // row stride in entries
  static_assert(C >= kSampleCap, "a row buffer holds the sample");
  constexpr int kRowsPerWg = WAVES * 4;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;  // 2 x kStageBytes
  uint32_t* keys_lds = reinterpret_cast<uint32_t*>(smem + 2 * kStageBytes);
  IdT* ids_lds = reinterpret_cast<IdT*>(keys_lds + kRowsPerWg * CS);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
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
  // Wait for these loads here, where the compiler sees it: otherwise it assumes them in flight at
  // every stream step and waits for the next chunk's loads before the first product.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // Stage fill: 16 wave-wide 16-byte loads per chunk; slot s = stage row s / 8, piece s % 8. Stage
  // row R = 16 ct + j holds candidate v0 + kTiles j + ct, so that tile ct (rows 16 ct .. 16 ct + 15,
  // read by lanes j = l % 16) gives lane j the candidates kTiles j .. kTiles j + 7 of the chunk in
  // ascending order over the tiles. Candidate v is block lo + v * stride + off. The (row, piece) of
  // this lane's slots do not change from chunk to chunk. The next chunk's keys are loaded into
  // registers at the start of a step and written to its stage buffer at the end: an LDS-direct load
  // would hold the issuing wave, and with them in flight every LDS read would wait for all of them.
  constexpr int kTiles = kChunk / 16;
  constexpr int kFillLoads = kChunk * 8 / 64;
  constexpr int kFillPerWave = (kFillLoads + WAVES - 1) / WAVES;
  int fl_v[kFillPerWave], fl_piece[kFillPerWave], fl_lds[kFillPerWave];
#pragma unroll
  for (int x = 0; x < kFillPerWave; ++x) {
    const int slot = (wave + x * WAVES) * 64 + l;
    const int row = slot >> 3;
    fl_piece[x] = slot & 7;
    fl_v[x] = (row & 15) * kTiles + (row >> 4);
    fl_lds[x] = row * kKRowBytes + fl_piece[x] * 16;
  }
  u32x4 fill[kFillPerWave];
  auto fetch = [&](int v0, int stride, int off, int n_virt) {
    // Whole chunk inside the candidates and the block keys: no per-slot checks.
    const bool whole = v0 + kChunk <= n_virt && lo + (v0 + kChunk - 1) * stride + off < n_blocks;
#pragma unroll
    for (int x = 0; x < kFillPerWave; ++x) {
      if (wave + x * WAVES < kFillLoads) {
        const int v = v0 + fl_v[x];
        int b = lo + v * stride + off;
        if (!whole && (v >= n_virt || b >= n_blocks)) b = 0;  // beyond the candidates: any valid key
        fill[x] = *reinterpret_cast<const u32x4*>(kbar + (uint32_t)(b * kIdxDim + fl_piece[x] * 8));
      }
    }
  };
  auto deposit = [&](int buf) {
#pragma unroll
    for (int x = 0; x < kFillPerWave; ++x)
      if (wave + x * WAVES < kFillLoads) *reinterpret_cast<u32x4*>(stage + buf * kStageBytes + fl_lds[x]) = fill[x];
  };
  const int boff = l16 * kKRowBytes + quarter * 16;  // B operand: row l16 of a 16-block tile
  // B operands of one staged chunk (every tile, both K-steps), read into registers a chunk ahead
  // of their products: all waves read the whole stage right after a barrier, and this way that
  // burst overlaps the previous chunk's selection work instead of delaying the products.
  auto read_b = [&](const uint8_t* sb, bf16x8 (&b_lo)[kTiles], bf16x8 (&b_hi)[kTiles]) {
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const uint8_t* p = sb + ct * 16 * kKRowBytes + boff;
      b_lo[ct] = *reinterpret_cast<const bf16x8*>(p);
      b_hi[ct] = *reinterpret_cast<const bf16x8*>(p + 64);
    }
  };
  // Scores of one chunk: all products; then, while their results are computed, the operands of
  // the next chunk are read into the same registers (next(), possibly nothing); then the per-lane
  // ReLU / weight / head sum.
  auto chunk_scores = [&](bf16x8 (&b_lo)[kTiles], bf16x8 (&b_hi)[kTiles], float (&sc)[kTiles], auto&& next) {
    f32x4 acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      acc[ct] = mfma16(a_op[0], b_lo[ct], z);
    }
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = mfma16(a_op[1], b_hi[ct], acc[ct]);
    next();
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
  hi_wave = __builtin_amdgcn_readfirstlane(hi_wave);  // equal in every lane: a scalar branch below
  // Streams candidates v in [0, n_virt) (block lo + v * stride + off) through the double-buffered
  // stage, two chunks ahead of the products: at the start of step n the B operands of chunk n are
  // in registers and chunk n+1 is in buffer (n+1) % 2; the step loads chunk n+2's keys into
  // registers, issues chunk n's products, reads chunk n+1's operands into the operand registers
  // and, after the selection work, writes chunk n+2 to buffer n % 2, whose operand reads (issued
  // in step n-1) were waited for before the barrier that ended step n-1. The barrier at the end of
  // the step publishes chunk n+2. For every chunk, body(sc, v_first,
  // full) gets this lane's scores, for candidates v_first .. v_first + kTiles - 1 (ascending), and
  // whether every candidate of the wave's rows in the chunk is valid (a compile-time tag); after()
  // runs once per chunk.
  auto stream = [&](int n_virt, int stride, int off, auto&& body, auto&& after) {
    const int n_ch = (n_virt + kChunk - 1) / kChunk;
    if (n_ch <= 0) return;
    bf16x8 b_lo[kTiles], b_hi[kTiles];
    fetch(0, stride, off, n_virt);
    deposit(0);
    if (n_ch > 1) {
      fetch(kChunk, stride, off, n_virt);
      deposit(1);
    }
    __syncthreads();  // chunks 0 and 1 are staged
    read_b(stage, b_lo, b_hi);
    __syncthreads();  // every wave holds chunk 0's operands: buffer 0 may be refilled
    for (int n = 0; n < n_ch; ++n) {
      if (n + 2 < n_ch) fetch((n + 2) * kChunk, stride, off, n_virt);
      float sc[kTiles];
      chunk_scores(b_lo, b_hi, sc, [&]() {
        if (n + 1 < n_ch) read_b(stage + ((n + 1) & 1) * kStageBytes, b_lo, b_hi);
      });
      const int v_end = (n + 1) * kChunk;
      const int v_first = n * kChunk + l16 * kTiles;
      if (v_end <= n_virt && lo + (v_end - 1) * stride + off < hi_wave)
        body(sc, v_first, std::true_type());
      else
        body(sc, v_first, std::false_type());
      after();
      if (n + 2 < n_ch) deposit(n & 1);
      __syncthreads();  // chunk n+2 is staged; chunk n+1's operands are in registers
    }
  };
  // Validity of this lane's candidate v_first + ct.
  auto valid_at = [&](int v, int n_virt, int stride, int off) -> bool {
    return v < n_virt && lo + v * stride + off < hi_lane;
  };
  const int n_all = hi_all - lo;

  uint32_t* my_k = keys_lds + (size_t)(wave * 4 + quarter) * CS;  // this lane's row buffer
  IdT* my_i = ids_lds + (size_t)(wave * 4 + quarter) * CS;
  auto row_k = [&](int q) { return keys_lds + (size_t)(wave * 4 + q) * CS; };
  auto row_i = [&](int q) { return ids_lds + (size_t)(wave * 4 + q) * CS; };
  const uint32_t pad_pos = C + l16;  // this lane's pad entry
  auto nothing = [&]() {};

  // Row state, uniform over the row's 16 lanes: the threshold (a score s passes iff !(s < thr)),
  // the number of buffered entries, and whether the row takes part in the current pass.
  float thr = -__builtin_inff();
  int n_cnt = 0;
  bool active = true;

  // ------------------------------------------------------------------ sample
  // A strided sample of the candidates (the same blocks for every row of the workgroup) goes into
  // the row buffers; for every row with more than C candidates its keys give the threshold tau0.
  if (n_all > C) {
    const int sample_cap = kSampleCap;
    const int stride = (n_all + sample_cap - 1) / sample_cap;
    const int s_off = stride / 2;
    const int s_virt = (n_all - s_off + stride - 1) / stride;
    auto append_sample = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
      constexpr bool kFull = decltype(full_t)::value;
      bool f[kTiles];
      uint32_t cnt = 0;
#pragma unroll
      for (int ct = 0; ct < kTiles; ++ct) {
        f[ct] = kFull | valid_at(v_first + ct, s_virt, stride, s_off);
        cnt += f[ct] ? 1u : 0u;
      }
      const uint32_t incl = row16_prefix(cnt);
      uint32_t pos = n_cnt + incl - cnt;
#pragma unroll
      for (int ct = 0; ct < kTiles; ++ct) {
        my_k[f[ct] ? pos : pad_pos] = __float_as_uint(sc[ct]);
        pos += f[ct] ? 1u : 0u;
      }
      n_cnt += row16_total(incl);
    };
    stream(s_virt, stride, s_off, append_sample, nothing);
    lds_wait();

    for (int q = 0; q < 4; ++q) {
      const int cq = readlane(n_cand, 16 * q);
      if (cq <= C) continue;  // the row takes every candidate
      const int nq = readlane(n_cnt, 16 * q);
      const float p = (float)kb / (float)cq;
      const float mean = (float)nq * p;
      const int ks = (int)ceilf(mean + kSampleSigmas * sqrtf(mean * (1.0f - p))) + 1;
      if (ks >= nq) continue;  // the sample cannot bound the threshold: take every candidate
      uint32_t sk[kSampleCap / 64];
      keys_load(sk, row_k(q), nq);
      int unused;
      const uint32_t tau0 = kth_largest(sk, ks, &unused, ks + ks / 8 + 1);
      if (quarter == q) thr = threshold_of(tau0);
    }
    n_cnt = 0;
  }

  // ------------------------------------------------------------------ the pass
  // Every candidate that passes its row's threshold is appended, in ascending block order. A
  // chunk that would overflow a row's buffer first cuts it to at most min(K_B + kCutSlack, C -
  // kChunk) entries that include its K_B best, and raises the row's threshold past the cut's bound.
  // At most C - kChunk entries after a cut leave room for the chunk's appends (C >= K_B + kChunk).
  const int cut_cap = min(kb + kCutSlack, C - kChunk);
  auto append = [&](const float (&sc)[kTiles], int v_first, auto full_t) {
    constexpr bool kFull = decltype(full_t)::value;
    bool f[kTiles];
    uint32_t cnt = 0;
    auto filter = [&]() {
      cnt = 0;
#pragma unroll
      for (int ct = 0; ct < kTiles; ++ct) {
        f[ct] = active & (kFull | (v_first + ct < n_cand)) & !(sc[ct] < thr);  // no branches
        cnt += f[ct] ? 1u : 0u;
      }
    };
    filter();
    uint32_t incl = row16_prefix(cnt);
    int tot = (int)row16_total(incl);
    if (ballot(n_cnt + tot > C)) {
      lds_wait();
      for (int q = 0; q < 4; ++q) {
        if (readlane((int)(n_cnt + tot > C), 16 * q) == 0) continue;
        int kept;
        const uint32_t tau = cut_to<P, IdT>(row_k(q), row_i(q), readlane(n_cnt, 16 * q), kb, cut_cap, &kept);
        if (quarter == q) {
          n_cnt = kept;
          thr = tau == 0xFFFFFFFFu ? __builtin_inff() : threshold_of(tau + 1u);
        }
      }
      filter();
      incl = row16_prefix(cnt);
      tot = (int)row16_total(incl);
    }
    // Kept candidates go to consecutive entries, the others to this lane's pad entry.
    uint32_t pos = n_cnt + incl - cnt;
    const uint32_t id0 = (uint32_t)(lo + v_first);
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
      const uint32_t e = f[ct] ? pos : pad_pos;
      my_k[e] = __float_as_uint(sc[ct]);
      my_i[e] = (IdT)(id0 + ct);
      pos += f[ct] ? 1u : 0u;
    }
    n_cnt += tot;
  };
  stream(n_all, 1, 0, append, nothing);

  // A row whose sampled threshold let too few candidates through takes every candidate again.
  __shared__ int any_redo;
  if (threadIdx.x == 0) any_redo = 0;
  __syncthreads();
  const bool redo = valid_o && n_cnt < min(kb, n_cand);
  if (ballot(redo) && l == 0) any_redo = 1;
  __syncthreads();
  if (any_redo) {
    active = redo;
    if (redo) {
      thr = -__builtin_inff();
      n_cnt = 0;
    }
    stream(n_all, 1, 0, append, nothing);
  }

  // ------------------------------------------------------------------ output
  // Every buffer is cut to its K_B best and written out in order (-1 padded), or its ids and the
  // row's own block are ORed into the union mask. Union output: the tiles this workgroup's queries
  // fall in are ORed together in LDS (the stage buffers are free now) and each non-zero word is
  // then ORed into umask once; when they do not fit, every bit goes to umask directly.
  lds_wait();
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
    int nq = readlane(n_cnt, 16 * q);
    if (nq > kb) {
      cut_to<P, IdT>(row_k(q), row_i(q), nq, kb);
      nq = kb;
      lds_wait();
    }
    const IdT* list = row_i(q);
    if constexpr (UNION) {
      uint32_t* mrow = lds_union ? umask_lds + (i / tile - t0) * n_words : mask_row(i, g);
      auto put_bit = [&](int b) { atomicOr(&mrow[b >> 5], 1u << (b & 31)); };
      if (l == 0) put_bit(i / block);  // the own block
      for (int e = l; e < nq; e += 64) put_bit((int)list[e]);
    } else {
      int32_t* out = topk + ((long long)g * n_tokens + i) * kb;
      for (int e = l; e < kb; e += 64) out[e] = e < nq ? (int32_t)list[e] : -1;
    }
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

// The shapes a launch can take: WAVES waves of 4 rows, buffers of 64 P entries, 16- or 32-bit ids.
// Each fits the gfx950 LDS with the stage; the first whose buffer holds K_B plus one chunk of
// appends (K_B + kChunk entries) is used. The selection is VALU work, which one wave per SIMD
// issues at half the rate of two: the first shape fits two workgroups on a CU (32-bit ids leave no
// shape that does).
struct SelectShape {
  int waves, p;
  bool id32;
};
constexpr SelectShape kShapes[] = {{4, 10, false}, {4, 20, false}, {2, 40, false}, {4, 14, true}, {1, 60, true}};

size_t select_lds_bytes(const SelectShape& s) {
  return (size_t)2 * kStageBytes +
         (size_t)s.waves * 4 * (64 * s.p + kRowPad) * (4 + (s.id32 ? 4 : 2));
}

// The shape for K_B blocks out of n_blocks complete blocks, or null when none fits.
const SelectShape* select_shape(int kb, int n_blocks) {
  const bool id32 = n_blocks > 65536;
  for (const SelectShape& s : kShapes)
    if (s.id32 == id32 && 64 * s.p >= kb + kChunk && select_lds_bytes(s) + kStaticLds <= kGfx950LdsBytes) return &s;
  return nullptr;
}

}  // namespace

size_t index_topk_lds_min(int kb) {
  // Selection is possible for this K_B at every sequence length (both id widths).
  const SelectShape* a = select_shape(kb, 1);
  const SelectShape* b = select_shape(kb, 1 << 30);
  if (!a || !b) return kGfx950LdsBytes + 1;
  return select_lds_bytes(*a) + kStaticLds;
}

namespace {

// One launch of k_select; topk (UNION = false) or the zeroed umask (UNION = true) receives the
// selections.
template <bool UNION>
hipError_t launch_select(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* topk, uint32_t* umask,
                         int n_tokens, int n_groups, int block, int kb, int tile, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_groups;
  if (n_rows == 0) return hipSuccess;
  const SelectShape* s = select_shape(kb, n_tokens / block);
  if (!s) return hipErrorInvalidValue;
  const size_t lds = select_lds_bytes(*s);
  if (lds + kStaticLds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  const int rows_wg = s->waves * 4;
  const long long grid = (long long)n_groups * ((n_tokens + rows_wg - 1) / rows_wg);
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int n_words = ((n_tokens + block - 1) / block + 31) / 32;
#define SGQA_SELECT_CASE(WV, PP, IDT)                                                                            \
  if (s->waves == WV && s->p == PP && s->id32 == std::is_same<IDT, int32_t>::value) {                          \
    hipLaunchKernelGGL((k_select<WV, PP, IDT, UNION>), dim3((unsigned)grid), dim3(WV * 64), lds, stream, qi, w, \
                       kbar, topk, n_tokens, n_groups, block, kb, umask, tile, n_tiles, n_words);                \
    return hipGetLastError();                                                                                    \
  }
  SGQA_SELECT_CASE(4, 10, uint16_t)
  SGQA_SELECT_CASE(4, 20, uint16_t)
  SGQA_SELECT_CASE(2, 40, uint16_t)
  SGQA_SELECT_CASE(4, 14, int32_t)
  SGQA_SELECT_CASE(1, 60, int32_t)
#undef SGQA_SELECT_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t prepare_index_topk_kernels(int lds_max) {
  const void* fns[] = {(const void*)k_select<4, 10, uint16_t, false>, (const void*)k_select<4, 10, uint16_t, true>,
                       (const void*)k_select<4, 20, uint16_t, false>, (const void*)k_select<2, 40, uint16_t, false>,
                       (const void*)k_select<4, 14, int32_t, false>,  (const void*)k_select<1, 60, int32_t, false>,
                       (const void*)k_select<4, 20, uint16_t, true>,  (const void*)k_select<2, 40, uint16_t, true>,
                       (const void*)k_select<4, 14, int32_t, true>,   (const void*)k_select<1, 60, int32_t, true>};
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
