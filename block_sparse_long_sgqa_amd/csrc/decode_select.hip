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
//  * k_dpick: one 1024-thread workgroup per (row, segment of up to 65536 keys), P <= 64 keys per
//    thread in registers, thread t holding entries tP..tP+P-1 (ascending block ids). The K_B-th
//    largest key tau is found exactly by a 4-way search over the 32-bit key range (three
//    thresholds per workgroup barrier, counted with wave ballots). One scan of the per-thread
//    counts (above tau, equal to tau) gives every selected entry its output slot, in ascending id:
//    everything above tau and the lowest ids equal to tau.
//  * Longer rows (c > 65536) are reduced segment by segment: a segment's own top-K_B list always
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
constexpr int kSegMax = kPickThreads * 64;                  // 65536 keys per pick workgroup

// Key row stride of the score buffer: whole score workgroups, so the pick may read up to it.
long long score_stride(int c) { return ((long long)(c > 0 ? c : 0) + kScoreBlocksPerWg - 1) / kScoreBlocksPerWg * kScoreBlocksPerWg; }

// Grid: (sequence, 512-block range). Rows of the output: keys[(s * G + g) * stride + b].
__global__ __launch_bounds__(256) void k_dscore(const uint16_t* __restrict__ qi, const float* __restrict__ w,
                                                const uint16_t* __restrict__ kbar_all, uint32_t* __restrict__ keys,
                                                int n_groups, long long kbar_rows, int c, long long stride,
                                                int wg_per_seq) {
  const int s = blockIdx.x / wg_per_seq;
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

// Exact top-K_B of one segment of one row. keys: row r, segment sg holds entries
// [sg * seg_len, min(n, (sg + 1) * seg_len)) at keys + r * row_stride + sg * seg_len (padding up to
// the next multiple of 4 is readable). ids: the entries' block ids (same indexing), or null when the
// id is the entry index. Output either the final selection (sel, topk_out: [row][kb]) or, with
// out_keys, the segment's list (out_keys / out_ids: [row][n_seg][out_stride], key 0 / id -1 padding
// from the list's length up to out_stride, a multiple of 4 so that lists stay 16-byte aligned).
template <int P>
__global__ __launch_bounds__(kPickThreads) void k_dpick(const uint32_t* __restrict__ keys, long long row_stride,
                                                        const int32_t* __restrict__ ids, int n, int seg_len,
                                                        int n_seg, int kb, int out_stride,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ topk_out,
                                                        uint32_t* __restrict__ out_keys,
                                                        int32_t* __restrict__ out_ids) {
  __shared__ uint32_t red[2][kPickWaves][4];
  __shared__ uint32_t scan_tot[kPickWaves];
  const long long row = blockIdx.x / n_seg;
  const int sg = blockIdx.x % n_seg;
  const int t = threadIdx.x, wave = t >> 6, l = lane_id();
  const long long base = row * row_stride + (long long)sg * seg_len;
  const int len = min(seg_len, n - sg * seg_len);
  const int e0 = t * P;

  uint32_t k[P];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const int e = e0 + 4 * q;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (e < len) v = *reinterpret_cast<const u32x4*>(keys + base + e);
#pragma unroll
    for (int x = 0; x < 4; ++x) k[4 * q + x] = (e + x < len) ? v[x] : 0u;
  }

  // Block-wide counts of keys >= each of three thresholds (threshold 0 counts nothing useful and
  // is never asked for). One barrier per call: the two buffers alternate.
  int call = 0;
  auto count3 = [&](uint32_t a, uint32_t b, uint32_t cth, uint32_t (&out)[3]) {
    uint32_t ca = 0, cb = 0, cc = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      ca += popc64(ballot(k[j] >= a));
      cb += popc64(ballot(k[j] >= b));
      cc += popc64(ballot(k[j] >= cth));
    }
    const int buf = call & 1;
    ++call;
    if (l == 0) {
      red[buf][wave][0] = ca;
      red[buf][wave][1] = cb;
      red[buf][wave][2] = cc;
    }
    __syncthreads();
    out[0] = out[1] = out[2] = 0;
#pragma unroll
    for (int wv = 0; wv < kPickWaves; ++wv) {
      out[0] += red[buf][wv][0];
      out[1] += red[buf][wv][1];
      out[2] += red[buf][wv][2];
    }
  };

  uint32_t cnt[3];
  count3(1u, 1u, 1u, cnt);
  const uint32_t n_valid = cnt[0];
  uint32_t tau = 0;     // selected: keys > tau, and the first need_eq keys == tau (id order)
  uint32_t need_eq = 0;
  if (n_valid > (uint32_t)kb) {
    // Invariant: count(>= lo) >= kb > count(>= hi); the answer is lo once hi = lo + 1.
    uint64_t lo = 1, hi = 1ull << 32;
    while (hi - lo > 1) {
      const uint64_t d = hi - lo;
      const uint64_t m1 = lo + d / 4, m2 = lo + d / 2, m3 = lo + (3 * d) / 4;
      count3((uint32_t)m1, (uint32_t)m2, (uint32_t)m3, cnt);
      if (cnt[2] >= (uint32_t)kb) {
        lo = m3;
      } else if (cnt[1] >= (uint32_t)kb) {
        lo = m2;
        hi = m3;
      } else if (cnt[0] >= (uint32_t)kb) {
        lo = m1;
        hi = m2;
      } else {
        hi = m1;
      }
    }
    tau = (uint32_t)lo;
    uint32_t gt_total = 0;
    if (tau != 0xFFFFFFFFu) {
      count3(tau + 1, tau + 1, tau + 1, cnt);
      gt_total = cnt[0];
    }
    need_eq = (uint32_t)kb - gt_total;
  }

  // Output slot of an entry = (# above tau before it) + min(# equal to tau before it, need_eq).
  uint32_t my_gt = 0, my_eq = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    my_gt += k[j] > tau ? 1u : 0u;
    my_eq += (k[j] == tau && tau != 0u) ? 1u : 0u;
  }
  // Per-wave totals fit 16 bits (at most 64 P = 4096), so the wave scan runs on packed pairs.
  const uint32_t incl = wave_prefix_sum(my_gt | (my_eq << 16));
  uint32_t gt_pre = (incl & 0xFFFFu) - my_gt;
  uint32_t eq_pre = (incl >> 16) - my_eq;
  if (l == 63) scan_tot[wave] = incl;
  __syncthreads();
  uint32_t gt_all = 0, eq_all = 0;
  for (int wv = 0; wv < kPickWaves; ++wv) {
    const uint32_t v = scan_tot[wv];
    if (wv < wave) {
      gt_pre += v & 0xFFFFu;
      eq_pre += v >> 16;
    }
    gt_all += v & 0xFFFFu;
    eq_all += v >> 16;
  }
  const uint32_t n_sel = gt_all + min(eq_all, need_eq);

  const bool final_out = out_keys == nullptr;
  int32_t* sel_row = final_out ? sel + row * kb : nullptr;
  int32_t* top_row = (final_out && topk_out) ? topk_out + row * kb : nullptr;
  uint32_t* lk = final_out ? nullptr : out_keys + (row * n_seg + sg) * out_stride;
  int32_t* li = final_out ? nullptr : out_ids + (row * n_seg + sg) * out_stride;
  const int id_base = sg * seg_len;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const uint32_t kj = k[j];
    bool take = false;
    uint32_t pos = 0;
    if (kj > tau) {
      take = true;
      pos = gt_pre + min(eq_pre, need_eq);
      ++gt_pre;
    } else if (kj == tau && tau != 0u) {
      take = eq_pre < need_eq;
      pos = gt_pre + eq_pre;
      ++eq_pre;
    }
    if (take) {
      const int e = e0 + j;
      const int32_t id = ids ? ids[base + e] : id_base + e;
      if (final_out) {
        sel_row[pos] = id;
        if (top_row) top_row[pos] = id;
      } else {
        lk[pos] = kj;
        li[pos] = id;
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
  if (n <= kPickThreads * 32) return 32;
  return 64;
}

int list_stride(int kb) { return (kb + 3) / 4 * 4; }

hipError_t launch_pick(const uint32_t* keys, long long row_stride, const int32_t* ids, int n, int n_rows, int kb,
                       int32_t* sel, int32_t* topk_out, uint32_t* out_keys, int32_t* out_ids, hipStream_t stream) {
  int seg_len, n_seg, p;
  if (n <= kSegMax) {
    p = pick_p(n);
    seg_len = kPickThreads * p;
    n_seg = 1;
  } else {
    p = 64;
    seg_len = kSegMax;
    n_seg = (n + kSegMax - 1) / kSegMax;
  }
  const dim3 grid((unsigned)((long long)n_rows * n_seg));
#define SGQA_PICK_CASE(PP)                                                                                   \
  if (p == PP) {                                                                                             \
    hipLaunchKernelGGL(k_dpick<PP>, grid, dim3(kPickThreads), 0, stream, keys, row_stride, ids, n, seg_len,  \
                       n_seg, kb, out_keys ? list_stride(kb) : kb, sel, topk_out, out_keys, out_ids);                                         \
    return hipGetLastError();                                                                                \
  }
  SGQA_PICK_CASE(8)
  SGQA_PICK_CASE(16)
  SGQA_PICK_CASE(32)
  SGQA_PICK_CASE(64)
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
                                hipStream_t stream) {
  const int c = (n_tokens - 1) / block;
  const int n_rows = n_seqs * n_groups;
  if (n_rows == 0) return hipSuccess;
  const SelectLayout lay = select_layout(ws, n_seqs, n_tokens, n_groups, block, kb);
  const long long stride = score_stride(c);
  if (c > 0) {
    const int wg_per_seq = (int)(stride / kScoreBlocksPerWg);
    hipLaunchKernelGGL(k_dscore, dim3((unsigned)((long long)n_seqs * wg_per_seq)), dim3(kScoreWaves * 64), 0, stream,
                       qi, w, kbar, lay.keys, n_groups, (long long)(n_tokens / block), c, stride, wg_per_seq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Reduce the rows segment by segment until one segment holds them, then pick the selection.
  const uint32_t* keys = lay.keys;
  const int32_t* ids = nullptr;
  long long row_stride = stride;
  int n = c;
  int level = 0;
  while (n > kSegMax) {
    const int n_seg = (n + kSegMax - 1) / kSegMax;
    uint32_t* ok = lay.list_keys[level & 1];
    int32_t* oi = lay.list_ids[level & 1];
    hipError_t e = launch_pick(keys, row_stride, ids, n, n_rows, kb, nullptr, nullptr, ok, oi, stream);
    if (e != hipSuccess) return e;
    keys = ok;
    ids = oi;
    n = n_seg * list_stride(kb);
    row_stride = (long long)n_seg * list_stride(kb);
    ++level;
  }
  return launch_pick(keys, row_stride, ids, n, n_rows, kb, sel, topk_out, nullptr, nullptr, stream);
}

}  // namespace sgqa
