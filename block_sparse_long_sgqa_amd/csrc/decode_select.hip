// decode_select.hip -- block selection of single-token decode: indexer scores of every candidate
// block on the matrix cores, then an exact top-K_B per (sequence, group) with one workgroup each.
//
// "Inside Step 5 Preview", section Sparse GQA: paragraph "Reducing indexer's cost" (block-level
// indexer scores, top-k over blocks), Figure 3 (each KV group selects on its own over the shared
// block keys), paragraph "Trade-off between top-k and block size" (K_B = k / B).
//
// The query of sequence s sits at position L-1; its candidates are the blocks b < c = floor((L-1)/B)
// and, per group g,
//   s(g,b) = sum_h w[g][h] * max(0, <qi[s][g][h], kbar[s][b]>)            (fp32)
//   Sel(s,g) = the first min(K_B, c) candidates in the order (s descending, b ascending).
//
// Design (gfx950). A decode step has few queries and many candidates, so the work is shaped the
// other way round from prefill: the block keys of all sequences are read once, at HBM rate.
//  * k_dscore: one 32x32x16 bf16 MFMA takes A = the 32 (group, head) rows of 8 groups' indexer
//    queries and B = 16 dims x 32 blocks. After the 4 K-steps of d_I = 64 each lane holds the four
//    head dots of 4 groups for one block, and forms their scores in registers (ReLU, weights,
//    head sum). Scores leave as order-preserving 32-bit keys (0 = no candidate) in one row per
//    (sequence, group). The K dimension is permuted (lane half h takes dims 32h..32h+31), the same
//    way in A and B, so every lane reads 64 contiguous bytes of a block key.
//  * k_dpick: one 1024-thread workgroup per (row, segment of up to 32768 keys), P <= 32 keys per
//    thread in registers, thread t holding entries tP..tP+P-1 (ascending block ids). The K_B-th
//    largest key tau is found exactly by histogram rounds (256 buckets of a power-of-two width per
//    round, LDS atomics, one wave scans the counts from the top), first over the per-thread maxima,
//    whose K_B-th largest bounds tau from below, then over the keys between that bound and the
//    maximum. One scan of the per-entry flags (above tau, equal to tau) gives every selected entry
//    its output slot, in ascending id: everything above tau and the lowest ids equal to tau.
//  * Longer rows (c > 32768) are reduced segment by segment: a segment's own top-K_B list always
//    contains every entry of the row's top-K_B that falls in it, so picking again over the
//    concatenated (key, id) lists gives the same set; levels repeat until one segment is left.
#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kScoreBlocksPerWave = 128;                    // 4 MFMA tiles of 32 blocks
constexpr int kScoreWaves = 4;
constexpr int kScoreBlocksPerWg = kScoreBlocksPerWave * kScoreWaves;  // 512
constexpr int kPickThreads = 1024;
constexpr int kPickWaves = kPickThreads / 64;
constexpr int kSegMax = kPickThreads * 32;                  // 32768 keys per pick workgroup
constexpr int kCandCap = 8192;                              // keys listed for the exact rounds

// Key row stride of the score buffer: whole score workgroups, so the pick may read up to it.
long long score_stride(int c) { return ((long long)(c > 0 ? c : 0) + kScoreBlocksPerWg - 1) / kScoreBlocksPerWg * kScoreBlocksPerWg; }

// Candidates of sequence s: c = floor((L_s - 1) / B) with L_s = lens[s] clamped to [1, cap], or
// L_s = cap for every sequence when lens is null.
__device__ __forceinline__ int seq_candidates(const int32_t* lens, int s, int cap, int block) {
  int len = lens ? lens[s] : cap;
  len = len < 1 ? 1 : (len > cap ? cap : len);
  return (len - 1) / block;
}

// Grid: (sequence, 512-block range). Rows of the output: keys[(s * G + g) * stride + b].
__global__ __launch_bounds__(256) void k_dscore(const uint16_t* __restrict__ qi, const float* __restrict__ w,
                                                const uint16_t* __restrict__ kbar_all, uint32_t* __restrict__ keys,
                                                int n_groups, long long kbar_rows, const int32_t* __restrict__ lens,
                                                int cap, int block, long long stride, int wg_per_seq) {
  const int s = blockIdx.x / wg_per_seq;
  const int c = seq_candidates(lens, s, cap, block);
  const int part = blockIdx.x % wg_per_seq;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int half = l >> 5;
  const int b_base = part * kScoreBlocksPerWg + wave * kScoreBlocksPerWave;
  const uint16_t* kbar = kbar_all + (long long)s * kbar_rows * kIdxDim;

  // B operands of the wave's 4 tiles: lane (l & 31) of tile t is block b_base + 32 t + (l & 31),
  // dims 32*half .. 32*half + 31 as four 16-byte pieces (one per K-step). Blocks >= c read block 0.
  bf16x8 bop[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int b = b_base + 32 * t + (l & 31);
    const uint16_t* src = kbar + (long long)(b < c ? b : 0) * kIdxDim + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bop[t][ks] = *reinterpret_cast<const bf16x8*>(src + 8 * ks);
  }

  for (int g0 = 0; g0 < n_groups; g0 += 8) {
    // A operand: row (l & 31) = (group g0 + row/4, head row%4); missing groups are zero rows.
    const int ga = g0 + ((l & 31) >> 2), ha = l & 3;
    bf16x8 aop[4];
    if (ga < n_groups) {
      const uint16_t* src = qi + (((long long)s * n_groups + ga) * kIdxHeads + ha) * kIdxDim + 32 * half;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) aop[ks] = *reinterpret_cast<const bf16x8*>(src + 8 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) aop[ks][e] = (__bf16)0.0f;
    }
    // Output register j of lane l: block column (l & 31), row 8 (j/4) + 4 half + j%4, i.e. group
    // g0 + 2 (j/4) + half, head j%4.
    float w4[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = g0 + 2 * q + half;
#pragma unroll
      for (int h = 0; h < 4; ++h) w4[q][h] = g < n_groups ? w[g * kIdxHeads + h] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16 acc;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32(aop[ks], bop[t][ks], acc);
      const int b = b_base + 32 * t + (l & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = g0 + 2 * q + half;
        float sc = 0.0f;
#pragma unroll
        for (int h = 0; h < 4; ++h) sc += w4[q][h] * __builtin_amdgcn_fmed3f(acc[4 * q + h], 0.0f, 3.402823466e38f);
        if (g < n_groups) keys[((long long)s * n_groups + g) * stride + b] = b < c ? score_key(sc) : 0u;
      }
    }
  }
}

// ------------------------------------------------------------------------------ pick helpers

constexpr int kBuckets = 256;

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return wave_sum_dpp(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_max_dpp(v); }

// Sum / maximum over the 16 lanes of each row (DPP row shifts: lane 15 of the row ends up with
// the total), read from lane 15.
__device__ __forceinline__ uint32_t lanes16_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
}

__device__ __forceinline__ uint32_t lanes16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
}

// Workgroup reduction of wave-uniform values: two sums and two maxima, one barrier. Lanes 0..15
// of every wave read the 16 wave partials and reduce them across the row.
__device__ __forceinline__ void block_reduce(uint32_t (*red)[4], uint32_t a, uint32_t b, uint32_t mx0, uint32_t mx1,
                                             uint32_t (&out)[4]) {
  const int l = lane_id();
  if (l == 0) {
    const u32x4 v = {a, b, mx0, mx1};
    *reinterpret_cast<u32x4*>(red[threadIdx.x >> 6]) = v;
  }
  __syncthreads();
  u32x4 v = {0u, 0u, 0u, 0u};
  if (l < kPickWaves) v = *reinterpret_cast<const u32x4*>(red[l]);
  out[0] = lanes16_sum(v[0]);
  out[1] = lanes16_sum(v[1]);
  out[2] = lanes16_max(v[2]);
  out[3] = lanes16_max(v[3]);
}

// Histogram select of the kb-th largest value of a multiset spread over the workgroup's threads.
// for_each(f) calls f(x) for every value x this thread holds (0 = absent). Requires
// count(>= lo) >= kb > count(>= hi) = c_hi. Every round splits [lo, hi) into 256 equal power-of-two
// buckets, counts the values of each (LDS atomics), and keeps the bucket where the running count
// from the top reaches kb. Returns tau, the largest t with count(>= t) >= kb, and writes
// count(>= tau + 1) to gt. `round` carries the parity of the histogram buffers across calls: the
// buffer a round fills was cleared during the round before (both are clear at the start).
template <typename ForEach>
__device__ __forceinline__ uint32_t bucket_select(uint64_t lo, uint64_t hi, uint32_t c_hi, uint32_t kb,
                                                  uint32_t (*hist)[kBuckets], uint32_t* bc, int& round,
                                                  ForEach for_each, uint32_t& gt) {
  const int l = lane_id();
  while (hi - lo > 1) {
    const uint64_t span = hi - lo;
    const int bits = 64 - __clzll((long long)(span - 1));  // ceil(log2(span))
    const int shift = bits > 8 ? bits - 8 : 0;
    uint32_t* h = hist[round & 1];
    if (threadIdx.x < kBuckets) hist[(round + 1) & 1][threadIdx.x] = 0u;
    for_each([&](uint32_t x) {
      if (x >= lo && x < hi) atomicAdd(&h[(uint32_t)((x - lo) >> shift)], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      // Lane l holds buckets 4l..4l+3; S(b) = c_hi + (values in buckets >= b) = count(>= lo + b << shift).
      const u32x4 hv = *reinterpret_cast<const u32x4*>(h + 4 * l);
      const uint32_t local = hv[0] + hv[1] + hv[2] + hv[3];
      const uint32_t above = wave_suffix_sum(local) - local + c_hi;  // S(4l + 4)
      const uint32_t s3 = above + hv[3], s2 = s3 + hv[2], s1 = s2 + hv[1], s0 = s1 + hv[0];
      const uint64_t m = ballot(s0 >= kb);  // S is non-increasing: lanes 0 .. l* (never empty)
      if (m == 0 && l == 0) {                 // count(>= lo) < kb cannot happen; end the search
        bc[0] = 0u;
        bc[1] = kb;
      }
      if (m != 0 && l == 63 - __clzll((long long)m)) {
        const int j = s3 >= kb ? 3 : (s2 >= kb ? 2 : (s1 >= kb ? 1 : 0));
        bc[0] = (uint32_t)(4 * l + j);
        bc[1] = j == 3 ? above : (j == 2 ? s3 : (j == 1 ? s2 : s1));  // S(b + 1)
      }
    }
    __syncthreads();
    const uint64_t nlo = lo + ((uint64_t)bc[0] << shift);
    const uint64_t nhi = nlo + (1ull << shift);
    const bool stop = bc[1] >= kb;  // only from the impossible case above
    c_hi = stop ? 0u : bc[1];
    lo = nlo;
    hi = stop ? lo + 1 : (nhi < hi ? nhi : hi);
    ++round;
  }
  gt = c_hi;
  return (uint32_t)lo;
}

// Exact top-K_B of one segment of one row. keys: row r, segment sg holds entries
// [sg * seg_len, min(n, (sg + 1) * seg_len)) at keys + r * row_stride + sg * seg_len (padding up to
// the next multiple of 4 is readable). ids: the entries' block ids (same indexing), or null when the
// id is the entry index. Output either the final selection (sel, topk_out: [row][kb]) or, with
// out_keys, the segment's list (out_keys / out_ids: [row][n_seg][out_stride], key 0 / id -1 padding
// from the list's length up to out_stride, a multiple of 4 so that lists stay 16-byte aligned).
//
// tau is bounded from below first: the K_B-th largest of the per-thread maxima v has at least K_B
// keys at or above it, so tau >= v, and few keys lie in [v, max] (typically a small multiple of
// K_B), which keeps the histogram rounds over the keys cheap and their buckets spread.
// lens (first level only): row r = s * G + g has seq_candidates(lens, s, cap, block) entries instead
// of n.
template <int P>
__global__ __launch_bounds__(kPickThreads) void k_dpick(const uint32_t* __restrict__ keys, long long row_stride,
                                                        const int32_t* __restrict__ ids, int n, int seg_len,
                                                        int n_seg, int kb, int out_stride,
                                                        const int32_t* __restrict__ lens, int n_groups, int cap,
                                                        int block,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ topk_out,
                                                        uint32_t* __restrict__ out_keys,
                                                        int32_t* __restrict__ out_ids) {
  __shared__ __align__(16) uint32_t red[kPickWaves][4];
  __shared__ __align__(16) uint32_t hist[2][kBuckets];
  __shared__ uint32_t scan_tot[kPickWaves];
  __shared__ uint32_t bc[2];
  __shared__ uint32_t cand[kCandCap];  // the keys >= the lower bound of tau
  const long long row = blockIdx.x / n_seg;
  const int sg = blockIdx.x % n_seg;
  const int t = threadIdx.x, wave = t >> 6, l = lane_id();
  const long long base = row * row_stride + (long long)sg * seg_len;
  const int n_row = lens ? seq_candidates(lens, (int)(row / n_groups), cap, block) : n;
  const int len = max(0, min(seg_len, n_row - sg * seg_len));
  const int e0 = t * P;

  uint32_t k[P];
  // Block ids of the entries (later levels), loaded with the keys: the output loop below must not
  // load, or every one of its stores would wait for the earlier ones (one counter tracks both).
  int32_t idv[P];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const int e = e0 + 4 * q;
    u32x4 v = {0u, 0u, 0u, 0u}, vi = {0u, 0u, 0u, 0u};
    if (e < len) v = *reinterpret_cast<const u32x4*>(keys + base + e);
    if (ids && e < len) vi = *reinterpret_cast<const u32x4*>(ids + base + e);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      k[4 * q + x] = (e + x < len) ? v[x] : 0u;
      idv[4 * q + x] = (int32_t)vi[x];
    }
  }
  if (t < kBuckets) {
    hist[0][t] = 0u;
    hist[1][t] = 0u;
  }

  uint32_t my_max = 0, my_valid = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    my_max = max(my_max, k[j]);
    my_valid += k[j] != 0u ? 1u : 0u;
  }
  uint32_t r4[4];
  block_reduce(red, wave_sum_u32(my_valid), (uint32_t)popc64(ballot(my_max != 0u)), wave_max_u32(my_max),
               wave_max_u32(~my_max), r4);
  const uint32_t n_valid = r4[0];          // keys present
  const uint32_t n_thr = r4[1];            // threads holding at least one key
  const uint64_t hi0 = (uint64_t)r4[2] + 1;  // count(>= hi0) = 0
  const uint32_t min_max = ~r4[3];         // smallest per-thread maximum

  uint32_t tau = 0;      // selected: keys > tau, and the first need_eq keys == tau (id order)
  uint32_t need_eq = 0;
  if (n_valid > (uint32_t)kb) {
    int round = 0;
    uint64_t v = 1;
    uint32_t unused;
    if (kb <= kPickThreads && n_thr >= (uint32_t)kb)
      v = bucket_select(min_max > 0u ? min_max : 1u, hi0, 0u, (uint32_t)kb, hist, bc, round,
                        [&](auto&& f) { f(my_max); }, unused);
    // The keys >= v (typically one to three times K_B) are gathered into an LDS list at
    // prefix-scan positions, so that the rounds visit only them instead of every thread's P keys;
    // a row with more than kCandCap of them keeps the keys in registers.
    uint32_t my_c = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) my_c += k[j] >= v ? 1u : 0u;
    const uint32_t cincl = wave_prefix_sum(my_c);
    if (l == 63) scan_tot[wave] = cincl;
    __syncthreads();
    uint32_t cpos = cincl - my_c, c_all = 0;
    for (int wv = 0; wv < kPickWaves; ++wv) {
      const uint32_t x = scan_tot[wv];
      if (wv < wave) cpos += x;
      c_all += x;
    }
    const bool listed = c_all <= (uint32_t)kCandCap;
    if (listed && my_c != 0u) {
#pragma unroll
      for (int j = 0; j < P; ++j)
        if (k[j] >= v) cand[cpos++] = k[j];
    }
    __syncthreads();  // the list is complete and every read of scan_tot above is done
    uint32_t gt_total;
    if (listed)
      tau = bucket_select(v, hi0, 0u, (uint32_t)kb, hist, bc, round,
                          [&](auto&& f) {
                            for (uint32_t x = (uint32_t)t; x < c_all; x += kPickThreads) f(cand[x]);
                          },
                          gt_total);
    else
      tau = bucket_select(v, hi0, 0u, (uint32_t)kb, hist, bc, round,
                          [&](auto&& f) {
#pragma unroll
                            for (int j = 0; j < P; ++j) f(k[j]);
                          },
                          gt_total);
    need_eq = (uint32_t)kb - gt_total;
  }

  // Output slot of an entry = (# above tau before it) + min(# equal to tau before it, need_eq),
  // counted in ascending id order.
  // This thread's entries above tau and equal to tau, as bit masks (bit j = entry e0 + j).
  static_assert(P <= 32, "entry masks are 32-bit");
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    gtm |= (k[j] > tau ? 1u : 0u) << j;
    eqm |= ((k[j] == tau && tau != 0u) ? 1u : 0u) << j;
  }
  const uint32_t my_gt = (uint32_t)__popc(gtm), my_eq = (uint32_t)__popc(eqm);
  // Per-wave totals fit 16 bits (at most 64 P = 2048), so the wave scan runs on packed pairs.
  const uint32_t incl = wave_prefix_sum(my_gt | (my_eq << 16));
  uint32_t gt_pre = (incl & 0xFFFFu) - my_gt;
  uint32_t eq_pre = (incl >> 16) - my_eq;
  if (l == 63) scan_tot[wave] = incl;
  __syncthreads();
  uint32_t gt_all = 0, eq_all = 0;
  for (int wv = 0; wv < kPickWaves; ++wv) {
    const uint32_t x = scan_tot[wv];
    if (wv < wave) {
      gt_pre += x & 0xFFFFu;
      eq_pre += x >> 16;
    }
    gt_all += x & 0xFFFFu;
    eq_all += x >> 16;
  }
  const uint32_t n_sel = gt_all + min(eq_all, need_eq);

  const bool final_out = out_keys == nullptr;
  int32_t* sel_row = final_out ? sel + row * kb : nullptr;
  int32_t* top_row = (final_out && topk_out) ? topk_out + row * kb : nullptr;
  uint32_t* lk = final_out ? nullptr : out_keys + (row * n_seg + sg) * out_stride;
  int32_t* li = final_out ? nullptr : out_ids + (row * n_seg + sg) * out_stride;
  const int id_base = sg * seg_len;
  if (my_gt + my_eq != 0u && !ids && final_out) {
    // The final selection with entry ids = entry positions: walk only the taken entries (all above
    // tau, and the equal ones while fewer than need_eq equal entries precede them), slots from the
    // masks.
    const uint32_t eq_room = need_eq > eq_pre ? need_eq - eq_pre : 0u;
    uint32_t eq_take = eqm;
    if (my_eq > eq_room) {  // keep the lowest eq_room equal entries (eq_room < 32 here)
      uint32_t rest = eqm;
      for (uint32_t c = 0; c < eq_room; ++c) rest &= rest - 1u;
      eq_take = eqm & ~rest;
    }
    uint32_t m = gtm | eq_take;
    while (m) {
      const int j = __ffs(m) - 1;
      m &= m - 1u;
      const uint32_t below = (1u << j) - 1u;
      const uint32_t slot = gt_pre + (uint32_t)__popc(gtm & below) + min(eq_pre + (uint32_t)__popc(eqm & below), need_eq);
      const int32_t id = id_base + e0 + j;
      sel_row[slot] = id;
      if (top_row) top_row[slot] = id;
    }
  } else if (my_gt + my_eq != 0u) {
    // Segment lists (keys and ids out) and later levels (ids from the previous level's lists,
    // loaded with the keys).
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const uint32_t kx = k[j];
      bool take = false;
      uint32_t slot = 0;
      if (kx > tau) {
        take = true;
        slot = gt_pre + min(eq_pre, need_eq);
        ++gt_pre;
      } else if (kx == tau && tau != 0u) {
        take = eq_pre < need_eq;
        slot = gt_pre + eq_pre;
        ++eq_pre;
      }
      if (take) {
        const int e = e0 + j;
        const int32_t id = ids ? idv[j] : id_base + e;
        if (final_out) {
          sel_row[slot] = id;
          if (top_row) top_row[slot] = id;
        } else {
          lk[slot] = kx;
          li[slot] = id;
        }
      }
    }
  }
  for (int p = (int)n_sel + t; p < out_stride; p += kPickThreads) {
    if (final_out) {
      sel_row[p] = -1;
      if (top_row) top_row[p] = -1;
    } else {
      lk[p] = 0u;
      li[p] = -1;
    }
  }
}

int pick_p(int n) {
  if (n <= kPickThreads * 8) return 8;
  if (n <= kPickThreads * 16) return 16;
  return 32;
}

int list_stride(int kb) { return (kb + 3) / 4 * 4; }

hipError_t launch_pick(const uint32_t* keys, long long row_stride, const int32_t* ids, int n, int n_rows, int kb,
                       int32_t* sel, int32_t* topk_out, uint32_t* out_keys, int32_t* out_ids, const int32_t* lens,
                       int n_groups, int cap, int block, hipStream_t stream) {
  int seg_len, n_seg, p;
  if (n <= kSegMax) {
    p = pick_p(n);
    seg_len = kPickThreads * p;
    n_seg = 1;
  } else {
    p = 32;
    seg_len = kSegMax;
    n_seg = (n + kSegMax - 1) / kSegMax;
  }
  const dim3 grid((unsigned)((long long)n_rows * n_seg));
#define SGQA_PICK_CASE(PP)                                                                                   \
  if (p == PP) {                                                                                             \
    hipLaunchKernelGGL(k_dpick<PP>, grid, dim3(kPickThreads), 0, stream, keys, row_stride, ids, n, seg_len,  \
                       n_seg, kb, out_keys ? list_stride(kb) : kb, lens, n_groups, cap, block, sel, topk_out, out_keys, out_ids);                                         \
    return hipGetLastError();                                                                                \
  }
  SGQA_PICK_CASE(8)
  SGQA_PICK_CASE(16)
  SGQA_PICK_CASE(32)
#undef SGQA_PICK_CASE
  return hipErrorInvalidValue;
}

struct SelectLayout {
  uint32_t* keys;          // [S*G][stride]
  uint32_t* list_keys[2];  // ping-pong segment lists [S*G][n_seg][kb]
  int32_t* list_ids[2];
  size_t bytes;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

SelectLayout select_layout(void* ws, int n_seqs, int n_tokens, int n_groups, int block, int kb) {
  const int c = (n_tokens - 1) / block;
  const size_t rows = (size_t)n_seqs * n_groups;
  const size_t key_bytes = round256(rows * (size_t)score_stride(c) * 4);
  const size_t n_seg = c > kSegMax ? (size_t)((c + kSegMax - 1) / kSegMax) : 0;
  const size_t list_bytes = round256(rows * n_seg * (size_t)list_stride(kb) * 4);
  SelectLayout lay;
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  size_t off = 0;
  lay.keys = reinterpret_cast<uint32_t*>(b ? b + off : nullptr);
  off += key_bytes;
  for (int x = 0; x < 2; ++x) {
    lay.list_keys[x] = reinterpret_cast<uint32_t*>(b ? b + off : nullptr);
    off += list_bytes;
    lay.list_ids[x] = reinterpret_cast<int32_t*>(b ? b + off : nullptr);
    off += list_bytes;
  }
  lay.bytes = off;
  return lay;
}

}  // namespace

size_t decode_select_ws_bytes(int n_seqs, int n_tokens, int n_groups, int block, int kb) {
  return select_layout(nullptr, n_seqs, n_tokens, n_groups, block, kb).bytes;
}

hipError_t launch_decode_select(const uint16_t* qi, const float* w, const uint16_t* kbar, int32_t* sel,
                                int32_t* topk_out, void* ws, int n_seqs, int n_tokens, int n_groups, int block, int kb,
                                const int32_t* lens, hipStream_t stream) {
  const int c = (n_tokens - 1) / block;
  const int n_rows = n_seqs * n_groups;
  if (n_rows == 0) return hipSuccess;
  const SelectLayout lay = select_layout(ws, n_seqs, n_tokens, n_groups, block, kb);
  const long long stride = score_stride(c);
  if (c > 0) {
    const int wg_per_seq = (int)(stride / kScoreBlocksPerWg);
    hipLaunchKernelGGL(k_dscore, dim3((unsigned)((long long)n_seqs * wg_per_seq)), dim3(kScoreWaves * 64), 0, stream,
                       qi, w, kbar, lay.keys, n_groups, (long long)(n_tokens / block), lens, n_tokens, block, stride,
                       wg_per_seq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Reduce the rows segment by segment until one segment holds them, then pick the selection.
  const uint32_t* keys = lay.keys;
  const int32_t* ids = nullptr;
  long long row_stride = stride;
  int n = c;
  int level = 0;
  const int32_t* lv_lens = lens;  // only the first level has per-sequence lengths
  while (n > kSegMax) {
    const int n_seg = (n + kSegMax - 1) / kSegMax;
    uint32_t* ok = lay.list_keys[level & 1];
    int32_t* oi = lay.list_ids[level & 1];
    hipError_t e = launch_pick(keys, row_stride, ids, n, n_rows, kb, nullptr, nullptr, ok, oi, lv_lens, n_groups,
                               n_tokens, block, stream);
    if (e != hipSuccess) return e;
    keys = ok;
    ids = oi;
    n = n_seg * list_stride(kb);
    row_stride = (long long)n_seg * list_stride(kb);
    lv_lens = nullptr;
    ++level;
  }
  return launch_pick(keys, row_stride, ids, n, n_rows, kb, sel, topk_out, nullptr, nullptr, lv_lens, n_groups, n_tokens,
                     block, stream);
}

}  // namespace sgqa
