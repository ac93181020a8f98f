// attend_bwd.hip -- gradient of the gathered-block causal GQA attention over the tile unions.
//
// "Inside Step 5 Preview", section Sparse GQA: the model is trained with this attention (the
// selection itself gets no gradient here: the pages leave the indexer's training signal open). For
// a row (query i, head h of group g) with token set J (as in the forward) and softmax p over J:
//   dv_j += p_j dout_i,  dp_j = <dout_i, v_j>,  ds_j = p_j (dp_j - delta_i),  delta_i = <dout_i, out_i>
//   dq_i = sigma sum_j ds_j k_j,  dk_j += sigma ds_j q_i
// p is recomputed from the forward's base-2 log-sum-exp. Every sum has a fixed order (no
// floating-point atomics), so the result is deterministic.
//
// gfx950 design
//  * delta: one pass over dout and out.
//  * dq: the forward's workgroup = (tile, group, part) of 32-row Q tiles, streaming the tile union in
//    64-key chunks gathered into LDS; per chunk S^T = K Q^T and dP^T = V dO^T (A operands from
//    padded K and V tiles, Q and dO in registers), dS^T in the score registers, then
//    dQ^T += K^T dS^T with K^T read transposed (ds_read_b64_tr_b16) from a second, swizzled copy of
//    the K tile -- the forward's O^T += V^T P^T with V replaced by K.
//  * dk, dv, tile-major (what runs unless the context is too long for its batches): a work item is
//    128 keys of one tile union, four waves of 32 keys (K and V as persistent B operands); the
//    tile's Q and dO rows stream once through shared LDS row tiles in 32-row groups, and every wave
//    pipelines the groups (S and dP of the next group on the matrix cores while the vector ALU forms
//    P and dS of the current one, then dV^T += dO^T P and dK^T += Q^T dS with transposed reads). Each
//    item writes fp32 partial rows per key, summed per key in ascending tile order by a second
//    kernel that runs on a second stream, beside the products of the next batch of tiles (see the
//    tile-major section below).
//  * dk, dv, key-major (the longest contexts): every key's sum runs over its rows in one place. A
//    wave owns 32 consecutive keys of one group and walks the tiles whose union holds one of its
//    blocks; per 32-row group of such a tile, Q and dO rows are gathered into the wave's swizzled
//    LDS tiles (double-buffered, one group ahead), with the same products.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attn_common.hpp"

namespace sgqa {

namespace {

constexpr int kBwdWaves = 4;  // dk/dv workgroup (one wave per SIMD)
constexpr int kDqWaves = 8;                 // dq workgroup (two waves per SIMD, as the forward)
// dq stage: padded K tile, padded V tile, swizzled K tile.
constexpr int kDqKs = 2 * kKTileBytes;                          // swizzled K tile offset
constexpr int kDqStageBytes = kDqKs + kVTileBytes;              // one stage

// Two 4x16 transposing reads at `a0` and 8 rows below: the A operand of a (d x rows) product whose
// B operand is packed from score registers (see the forward's O^T += V^T P^T).
__device__ __forceinline__ bf16x8 tr_read(const uint8_t* a0) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * 256));
  const i16x8 cat = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, cat);
}

}  // namespace

// delta[r] = <dout[r], out[r]> over the D = 128 elements of every row r of [N * Hq] (fp32).
__global__ __launch_bounds__(256) void k_bwd_delta(const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout,
                                                   float* __restrict__ delta, long long n_rows) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);  // 16 lanes per row
  const int part = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < n_rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(out + row * kD + 8 * part);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * kD + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < n_rows && part == 0) delta[row] = acc;
}

// ------------------------------------------------------------------------------------ dq

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_bwd_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint32_t* __restrict__ umask,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ delta,
                                                       const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
                                                       int n_tokens, int n_q_heads, int n_groups, int block,
                                                       int block_shift, int tile, float scale, float scale_log2,
                                                       int n_words, int parts, int n_pairs, int list_cap) {
  constexpr int NT = WAVES * 64;
  constexpr int kRowsWg = WAVES * 32;
  // The two stages and the token tables are variables of their own (see the forward kernel: the
  // compiler then does not make the reads of one stage wait for the gathers into the other).
  static_assert(WAVES + 1 <= 16, "scan words");
  __shared__ __align__(16) uint8_t stage0[kDqStageBytes];
  __shared__ __align__(16) uint8_t stage1[kDqStageBytes];
  __shared__ __align__(16) int toks[4 * kKeys];  // token tables of chunks n % 4
  __shared__ int scan[16];
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* list = reinterpret_cast<uint32_t*>(smem);  // one segment of the block list

  const int x = blockIdx.x;
  const int slot = x >> 3, xcd = x & 7;
  const int pair = (slot / parts) * 8 + xcd;
  const int part = slot % parts;
  if (pair >= n_pairs) return;
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int t = n_tiles - 1 - pair / n_groups;
  const int g = pair % n_groups;
  const int r = n_q_heads / n_groups;
  const int l = lane_id(), wave = threadIdx.x >> 6;
  const int i0 = t * tile;
  const int tile_rows = ((i0 + tile <= n_tokens) ? tile : n_tokens - i0) * r;
  const int row0 = part * kRowsWg;
  if (row0 >= tile_rows) return;
  const int row_last = (row0 + kRowsWg <= tile_rows ? row0 + kRowsWg : tile_rows) - 1;
  const int c_hi = (i0 + row_last / r) / block;

  // U(t,g) restricted to blocks <= c_hi: a window of list_cap entries from rank win_lo, moved on
  // at the end of a step when the next token table needs an entry past it (as in the forward).
  const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
  int win_lo = 0, n_list = 0;
  union_list_fill<NT>(mrow, c_hi, list, 0, list_cap, scan, &n_list);
  __syncthreads();

  // This lane's Q row (column l % 32 of the wave's tile): Q and dO as B operands, lse and delta.
  const int row = row0 + wave * 32 + (l & 31);
  const bool valid = row < tile_rows;
  const int i = i0 + (valid ? row / r : 0);
  const int h = g * r + (valid ? row % r : 0);
  const int row_pos = valid ? i : -1;
  bf16x8 qreg[8], dreg[8];
  {
    const long long base = ((long long)i * n_q_heads + h) * kD + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (valid) {
        qreg[ks] = *reinterpret_cast<const bf16x8*>(q + base + 16 * ks);
        dreg[ks] = *reinterpret_cast<const bf16x8*>(dout + base + 16 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qreg[ks][e] = (__bf16)0.0f;
          dreg[ks][e] = (__bf16)0.0f;
        }
      }
    }
  }
  const float row_lse = valid ? lse[(long long)i * n_q_heads + h] : 0.0f;
  const float row_delta = valid ? delta[(long long)i * n_q_heads + h] : 0.0f;

  f32x16 acc[4];  // dQ^T tiles [d-tile][32 d x 32 rows], column = this lane's row
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[dt][j] = 0.0f;

  const uint16_t* kbase = k + (long long)g * n_tokens * kD;
  const uint16_t* vbase = v + (long long)g * n_tokens * kD;
  const int n_keys = n_list * block;
  const int n_chunks = (n_keys + kKeys - 1) / kKeys;
  auto tok_at = [&](int chunk, int key) -> int {
    const int kp = chunk * kKeys + key;
    if (kp >= n_keys) return -1;
    const int tk = ((int)list[(kp >> block_shift) - win_lo] << block_shift) + (kp & (block - 1));
    return tk < n_tokens ? tk : -1;
  };
  // Gather of one chunk into a stage, staged through registers: 16 K and 16 V wave-wide 16-byte
  // loads (1 KiB each), four per wave (load xi of a wave is load wave + xi * WAVES; 0 .. 15 are K).
  // Load i, lane l holds row (64 i + l) / 16, piece (64 i + l) % 16 of its tensor; a K slice is
  // stored twice, into the padded K tile and into the swizzled one (physical piece v_phys(row, p)
  // holds logical piece p), a V slice into the padded V tile. The loads fly while the current chunk
  // is computed (LDS-direct loads would hold up the issuing wave and keep the compiler from
  // overlapping the operand reads). The rows' tokens come from the chunk's token table (written two
  // chunks ahead by the first wave), all read before the first load.
  constexpr int kDqLoads = 2 * kKeys * kD * 2 / 1024;  // 32
  constexpr int kPer = kDqLoads / WAVES;
  constexpr int kKPer = kPer / 2;
  static_assert(kDqLoads % WAVES == 0 && kPer % 2 == 0, "K and V loads split evenly over the waves");
  u32x4 stg[kPer];
  auto load_chunk = [&](int n) __attribute__((always_inline)) {
    const int* tab = toks + (n & 3) * kKeys;
    int tkn[kPer];
#pragma unroll
    for (int xi = 0; xi < kPer; ++xi) {
      const int ii = wave + xi * WAVES;
      const int sl = (xi < kKPer ? ii : ii - kDqLoads / 2) * 64 + l;
      const int t = tab[sl >> 4];
      tkn[xi] = t == 0x7FFFFFFF ? 0 : t;
    }
#pragma unroll
    for (int xi = 0; xi < kPer; ++xi) {
      const int ii = wave + xi * WAVES;
      const int sl = (xi < kKPer ? ii : ii - kDqLoads / 2) * 64 + l;
      stg[xi] = *reinterpret_cast<const u32x4*>((xi < kKPer ? kbase : vbase) + (long long)tkn[xi] * kD + (sl & 15) * 8);
    }
  };
  auto store_chunk = [&](uint8_t* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int xi = 0; xi < kPer; ++xi) {
      const int ii = wave + xi * WAVES;
      const int sl = (xi < kKPer ? ii : ii - kDqLoads / 2) * 64 + l;
      const int row = sl >> 4, piece = sl & 15;
      if (xi < kKPer) {
        *reinterpret_cast<u32x4*>(sb + row * kKRowBytes + 16 * piece) = stg[xi];
        *reinterpret_cast<u32x4*>(sb + kDqKs + row * 256 + 16 * v_phys(row, piece)) = stg[xi];
      } else {
        *reinterpret_cast<u32x4*>(sb + kKTileBytes + row * kKRowBytes + 16 * piece) = stg[xi];
      }
    }
  };
  auto write_tokens = [&](int c) __attribute__((always_inline)) {  // token table of chunk c
    if (threadIdx.x < kKeys && c < n_chunks) {
      const int tk = tok_at(c, (int)threadIdx.x);
      toks[(c & 3) * kKeys + threadIdx.x] = tk >= 0 ? tk : 0x7FFFFFFF;
    }
  };

  const LaneOffsets lo = lane_offsets(kDqKs);
  const int hi = l >> 5;
  auto chunk = [&](const uint8_t* sb, const int* tok) __attribute__((always_inline)) {
    // S^T = K Q^T and dP^T = V dO^T.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[kt][j] = 0.0f;
        dp[kt][j] = 0.0f;
      }
    const uint8_t* kp = sb + lo.k;
    const uint8_t* vp = sb + kKTileBytes + lo.k;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp + kt * 32 * kKRowBytes + ks * 32);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vp + kt * 32 * kKRowBytes + ks * 32);
        s[kt] = mfma32(ka, qreg[ks], s[kt]);
        dp[kt] = mfma32(va, dreg[ks], dp[kt]);
      }
    }
    // dS^T = P^T (dP^T - delta), P^T from the forward's log-sum-exp; masked keys give 0.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int4 t4 = *reinterpret_cast<const int4*>(tok + kt * 32 + 8 * a + 4 * hi);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int tk = c == 0 ? t4.x : (c == 1 ? t4.y : (c == 2 ? t4.z : t4.w));
          const int j = 4 * a + c;
          const float p = tk <= row_pos ? fast_exp2(__builtin_fmaf(s[kt][j], scale_log2, -row_lse)) : 0.0f;
          s[kt][j] = p * (dp[kt][j] - row_delta);
        }
      }
    bf16x8 pb[4];
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[ss][e] = (__bf16)s[ss >> 1][8 * (ss & 1) + e];
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int dt = step >> 2, ss = step & 3;
      acc[dt] = mfma32(tr_read(sb + lo.v[dt] + (16 * ss) * 256), pb[ss], acc[dt]);
    }
  };

  // Step n: start the gather of chunk n + 1 and write the token table of chunk n + 2, compute chunk
  // n, wait for the gather, sync. P = n % 2 picks the stages at compile time.
  auto step = [&](auto parity, int n) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    if (n + 1 < n_chunks) load_chunk(n + 1);
    write_tokens(n + 2);
    chunk(P ? stage1 : stage0, toks + (n & 3) * kKeys);
    if (n + 1 < n_chunks) store_chunk(P ? stage0 : stage1);
    __syncthreads();
    // Step n + 1 writes the token table of chunk n + 3: move the window to start at chunk n + 2
    // when chunk n + 3 reaches past it.
    if (n + 3 < n_chunks && (((n + 4) * kKeys - 1) >> block_shift) >= win_lo + list_cap) {
      int unused;
      win_lo = ((n + 2) * kKeys) >> block_shift;
      union_list_fill<NT>(mrow, c_hi, list, win_lo, list_cap, scan, &unused);
      __syncthreads();
    }
  };
  write_tokens(0);
  write_tokens(1);
  __syncthreads();
  if (n_chunks > 0) {
    load_chunk(0);
    store_chunk(stage0);
  }
  __syncthreads();
  // Every global load so far (Q, dO, lse, delta, chunk 0) has landed, as a wait the compiler sees:
  // otherwise it takes them as in flight inside the loop and waits for the staged loads as well.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  for (int n = 0; n < n_chunks; n += 2) {
    step(std::integral_constant<int, 0>(), n);
    if (n + 1 < n_chunks) step(std::integral_constant<int, 1>(), n + 1);
  }

  // dq[i][h][d] = sigma * dQ^T[d][row]
  if (valid) {
    uint16_t* dst = dq + ((long long)i * n_q_heads + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + 8 * a + 4 * hi;
        uint2 pk;
        pk.x = pack_bf16x2(acc[dt][4 * a] * scale, acc[dt][4 * a + 1] * scale);
        pk.y = pack_bf16x2(acc[dt][4 * a + 2] * scale, acc[dt][4 * a + 3] * scale);
        *reinterpret_cast<uint2*>(dst + d) = pk;
      }
  }
}

// ------------------------------------------------------------------------------------ dk, dv

namespace {
constexpr int kTileWin = 256;                  // tiles listed per scan window
constexpr int kRowTileBytes = 32 * 256;        // 32 rows x 128 bf16, pieces swizzled by rt_phys
constexpr int kRgBytes = 2 * kRowTileBytes;    // Q rows, then dO rows

// Row tiles are read both ways: row-wise, 16 bytes per lane (the A operands of S = Q K^T and
// dP = dO V^T: 16 lanes read one logical piece of 16 consecutive rows), and transposed (two 4x16
// transposing reads, as for the forward's V tile: 32 lanes read 4 logical pieces of 4 consecutive
// rows). Physical piece of logical piece p in row `row`: XOR with 4 (row % 4) + (row / 4) % 4,
// which gives each read phase of either kind 16 distinct pieces, i.e. all 64 banks once (the
// forward's V swizzle, XOR with 4 (row % 4) alone, leaves the row-wise reads 4-way conflicted). The
// swizzle repeats every 16 rows.
__device__ __forceinline__ int rt_phys(int row, int p) { return p ^ (((row & 3) << 2) | ((row >> 2) & 3)); }

// Per-lane byte offsets of the transposed reads of a row tile: d-tile dt, rows r (v0) and r + 8
// (v1) of the lane's read (see lane_offsets for the forward's V tile); + 16 ss rows for the
// second half of the 32 rows (the swizzle repeats every 16 rows).
struct RowTileOffsets {
  int v0[4], v1[4];
};
__device__ __forceinline__ RowTileOffsets row_tile_offsets() {
  const int l = lane_id(), grp = l >> 4, s16 = l & 15;
  const int row = 4 * (grp >> 1) + (s16 >> 2);
  RowTileOffsets o;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int piece = 4 * dt + 2 * (grp & 1) + ((s16 & 3) >> 1);
    o.v0[dt] = row * 256 + 16 * rt_phys(row, piece) + 8 * (s16 & 1);
    o.v1[dt] = (row + 8) * 256 + 16 * rt_phys(row + 8, piece) + 8 * (s16 & 1);
  }
  return o;
}

// The two transposing reads of a row tile (at a0 + v0 and a0 + v1): a bf16x8 A operand.
__device__ __forceinline__ bf16x8 rt_tr_read(const uint8_t* a0, int v0, int v1) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + v0));
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + v1));
  const i16x8 cat = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, cat);
}
}  // namespace

// One 32-row group against a wave's 32 keys (lane l holds key column l % 32): from the group's Q and
// dO rows in `b` (swizzled row-major, Q then dO), its rows' lse and delta (lsde) and queries (qrow,
// -1 past the tile), accumulates dV^T += dO^T P and dK^T += Q^T dS (unscaled) for the keys; `take`:
// this lane's key is attended by the group's rows (causality is tested here).
__device__ __forceinline__ void dkdv_rows(const uint8_t* b, const float* lsde, const int* qrow, bool take, int key,
                                          const bf16x8 (&kb)[8], const bf16x8 (&vb)[8], f32x16 (&adk)[4],
                                          f32x16 (&adv)[4], const RowTileOffsets& lo, float scale_log2) {
  const int l = lane_id(), hi = l >> 5;
  const uint8_t* dob = b + kRowTileBytes;
  // S = Q K^T, dP = dO V^T: A operands row (l % 32), logical piece 2 ks + (l / 32).
  f32x16 s, dp;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    s[j] = 0.0f;
    dp[j] = 0.0f;
  }
  // The operands of step ks + 2 are read while the products of step ks run.
  const int arow = l & 31;
  auto off_of = [&](int ks) { return arow * 256 + 16 * rt_phys(arow, 2 * ks + hi); };
  bf16x8 qa[3], da[3];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    qa[ks] = *reinterpret_cast<const bf16x8*>(b + off_of(ks));
    da[ks] = *reinterpret_cast<const bf16x8*>(dob + off_of(ks));
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks + 2 < 8) {
      qa[(ks + 2) % 3] = *reinterpret_cast<const bf16x8*>(b + off_of(ks + 2));
      da[(ks + 2) % 3] = *reinterpret_cast<const bf16x8*>(dob + off_of(ks + 2));
    }
    s = mfma32(qa[ks % 3], kb[ks], s);
    dp = mfma32(da[ks % 3], vb[ks], dp);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Rows of score j: 8 (j / 4) + 4 hi + (j % 4).
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int4 qi4 = *reinterpret_cast<const int4*>(qrow + 8 * a + 4 * hi);
    const float4 ls4 = *reinterpret_cast<const float4*>(lsde + 8 * a + 4 * hi);
    const float4 de4 = *reinterpret_cast<const float4*>(lsde + 32 + 8 * a + 4 * hi);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qi = c == 0 ? qi4.x : (c == 1 ? qi4.y : (c == 2 ? qi4.z : qi4.w));
      const float ls = c == 0 ? ls4.x : (c == 1 ? ls4.y : (c == 2 ? ls4.z : ls4.w));
      const float de = c == 0 ? de4.x : (c == 1 ? de4.y : (c == 2 ? de4.z : de4.w));
      const int j = 4 * a + c;
      const bool ok = take && key <= qi;  // qi = -1 for rows past the tile
      const float p = ok ? fast_exp2(__builtin_fmaf(s[j], scale_log2, -ls)) : 0.0f;
      s[j] = p;
      dp[j] = p * (dp[j] - de);
    }
  }
  bf16x8 pp[2], pd[2];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pp[ss][e] = (__bf16)s[8 * ss + e];
      pd[ss][e] = (__bf16)dp[8 * ss + e];
    }
  // dV^T += dO^T P, dK^T += Q^T dS; step = 2 dt + ss, operands read two steps ahead.
  auto tr_op = [&](const uint8_t* base, int step) {
    return rt_tr_read(base + (16 * (step & 1)) * 256, lo.v0[step >> 1], lo.v1[step >> 1]);
  };
  bf16x8 oa[3], qt[3];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    oa[st] = tr_op(dob, st);
    qt[st] = tr_op(b, st);
  }
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    if (st + 2 < 8) {
      oa[(st + 2) % 3] = tr_op(dob, st + 2);
      qt[(st + 2) % 3] = tr_op(b, st + 2);
    }
    const int dt = st >> 1, ss = st & 1;
    adv[dt] = mfma32(oa[st % 3], pp[ss], adv[dt]);
    adk[dt] = mfma32(qt[st % 3], pd[ss], adk[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(kBwdWaves * 64) void k_bwd_dkdv(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const uint32_t* __restrict__ umask,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ delta,
                                                             const uint16_t* __restrict__ dout,
                                                             uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                             int n_tokens, int n_q_heads, int n_groups, int block,
                                                             int block_shift, int tile, float scale,
                                                             float scale_log2, int n_words) {
  // Per wave: two row-group buffers (Q and dO rows; each row's query, lse and delta), the tile
  // window. Every buffer is a variable of its own, so the compiler can tell the gathers into one
  // from the reads of the other and waits only for the loads a read needs.
  __shared__ __align__(16) uint8_t rows0[kBwdWaves][kRgBytes];
  __shared__ __align__(16) uint8_t rows1[kBwdWaves][kRgBytes];
  __shared__ __align__(16) float lsde0[kBwdWaves][64];  // lse of the 32 rows, then delta
  __shared__ __align__(16) float lsde1[kBwdWaves][64];
  __shared__ __align__(16) int qrow0[kBwdWaves][32];    // query of each row (-1 past the tile)
  __shared__ __align__(16) int qrow1[kBwdWaves][32];
  __shared__ int win_tile_all[kBwdWaves][kTileWin];
  __shared__ uint32_t win_bits_all[kBwdWaves][kTileWin];
  const int wave = threadIdx.x >> 6, l = lane_id(), hi = l >> 5;
  int* win_tile = win_tile_all[wave];
  uint32_t* win_bits = win_bits_all[wave];

  const int chunks_per_g = (n_tokens + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  const int g = blockIdx.x / chunks_per_g;
  const int j0 = ((blockIdx.x % chunks_per_g) * kBwdWaves + wave) * 32;  // this wave's keys j0 .. j0 + 31
  if (j0 >= n_tokens) return;  // wave-uniform; the waves never synchronise with each other
  const int r = n_q_heads / n_groups;
  // x / r for the row indices of a tile, 0 <= x < tile * r: the high word of x * ceil(2^32 / r),
  // exact while x * (r - 1) < 2^32 (checked on the host for x = tile * r).
  const uint32_t r_magic = r > 1 ? (uint32_t)((0x100000000ull + (uint32_t)r - 1u) / (uint32_t)r) : 0u;
  auto div_r = [&](int x) -> int { return r > 1 ? (int)__umulhi((uint32_t)x, r_magic) : x; };
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int key = j0 + (l & 31);
  const bool key_ok = key < n_tokens;

  // K^T and V^T B operands of this lane's key (column l % 32), dims 16 ks + 8 (l / 32) .. + 7.
  bf16x8 kb[8], vb[8];
  {
    const long long base = ((long long)g * n_tokens + (key_ok ? key : 0)) * kD + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kb[ks] = *reinterpret_cast<const bf16x8*>(k + base + 16 * ks);
      vb[ks] = *reinterpret_cast<const bf16x8*>(v + base + 16 * ks);
    }
    // Wait for them here (vmcnt(0), a wait the compiler sees): otherwise it cannot tell how many
    // loads were issued after them on the way into the loop and waits for all at every product.
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  f32x16 adk[4], adv[4];  // dK^T, dV^T tiles [d-tile][32 d x 32 keys], column = this lane's key
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      adk[dt][j] = 0.0f;
      adv[dt][j] = 0.0f;
    }

  // The wave's blocks b0 .. b0 + nblk - 1 lie in one mask word (32 keys, j0 a multiple of 32).
  const int b0 = j0 >> block_shift;
  const int nblk = block >= 32 ? 1 : 32 >> block_shift;
  const uint32_t wmask = nblk >= 32 ? 0xFFFFFFFFu : (((1u << nblk) - 1u) << (b0 & 31));
  const int my_blk = (key >> block_shift) - b0;  // this lane's block within the wave's blocks
  const RowTileOffsets lo = row_tile_offsets();

  // Row group `rg` of tile `t`: Q and dO rows into buffer `buf` (swizzled row-major, 8 + 8
  // wave-wide loads), and each row's query, lse and delta.
  auto rg_rows = [&](int t) -> int {
    const int i0 = t * tile;
    return ((i0 + tile <= n_tokens) ? tile : n_tokens - i0) * r;
  };
  // Row group `rg` of tile `t`: its Q and dO rows (swizzled row-major like the forward's V tile)
  // and each row's query, lse and delta are loaded into registers while the previous group is
  // computed, then stored into the group's buffer. (LDS-direct loads hold the single wave of the
  // SIMD up for ~120 cycles each; these loads do not.)
  // Row rho of a tile's rows lies (rho / r) * Hq + rho % r rows past the tile's first row of group
  // g. When r divides 32 this splits into a part per row group and a part per row within the group
  // (fixed for each lane), so the per-item address work is one add per row.
  const bool r_div32 = (32 % r) == 0;
  int frow[8];
#pragma unroll
  for (int ti = 0; ti < 8; ++ti) {
    const int rw = 4 * ti + (l >> 4);
    frow[ti] = (rw / r) * n_q_heads + rw % r;
  }
  const int lrow = l & 31;
  const int frow_l = (lrow / r) * n_q_heads + lrow % r, fq_l = lrow / r;
  auto load_rg = [&](int t, int rg, u32x4 (&sq)[8], u32x4 (&sd)[8], float& ls, float& de, int& qi)
                     __attribute__((always_inline)) {
    const int nrows = rg_rows(t);
    const long long tbase = (long long)(t * tile) * n_q_heads + g * r;  // row 0 of the tile, group g
    long long gbase = 0;                                              // row rg * 32 (r | 32)
    if (r_div32) gbase = tbase + (long long)(rg * (32 / r)) * n_q_heads;
    {
      const int rho = rg * 32 + lrow;
      long long rix;
      int qq;
      if (r_div32) {
        qq = rg * (32 / r) + fq_l;
        rix = rho < nrows ? gbase + frow_l : tbase;
      } else {
        const int rr = rho < nrows ? rho : 0;
        qq = div_r(rr);
        rix = tbase + (long long)qq * n_q_heads + (rr - qq * r);
      }
      ls = lse[rix];
      de = delta[rix];
      qi = rho < nrows ? t * tile + qq : -1;
    }
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
      const int rw = 4 * ti + (l >> 4);
      const int rho = rg * 32 + rw;
      long long src_row;
      if (r_div32) {
        src_row = rho < nrows ? gbase + frow[ti] : tbase;
      } else {
        const int rr = rho < nrows ? rho : 0;
        const int qq = div_r(rr);
        src_row = tbase + (long long)qq * n_q_heads + (rr - qq * r);
      }
      const int piece = rt_phys(rw, l & 15);
      sq[ti] = *reinterpret_cast<const u32x4*>(q + src_row * kD + piece * 8);
      sd[ti] = *reinterpret_cast<const u32x4*>(dout + src_row * kD + piece * 8);
    }
  };
  auto store_rg = [&](uint8_t* b, float* lsde, int* qrow, const u32x4 (&sq)[8], const u32x4 (&sd)[8], float ls,
                      float de, int qi) __attribute__((always_inline)) {
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
      *reinterpret_cast<u32x4*>(b + ti * 1024 + 16 * l) = sq[ti];
      *reinterpret_cast<u32x4*>(b + kRowTileBytes + ti * 1024 + 16 * l) = sd[ti];
    }
    if (l < 32) {
      lsde[l] = ls;
      lsde[32 + l] = de;
      qrow[l] = qi;
    }
  };
  // One row group from buffer `buf`: member = this lane's key block is in the tile's union.
  auto compute_rg = [&](const uint8_t* b, const float* lsde, const int* qrow, bool member)
                        __attribute__((always_inline)) {
    dkdv_rows(b, lsde, qrow, member && key_ok, key, kb, vb, adk, adv, lo, scale_log2);
  };

  // Work items: the row groups of the tiles t >= the first one holding a query >= j0 whose union
  // holds one of the wave's blocks (listed a window of kTileWin tiles at a time), that reach a
  // query >= j0. The tiles are walked from the last one down: the waves that start together then
  // read the same tiles' rows at about the same time, which the caches can serve more than once.
  const int t_first = j0 / tile;
  int tw = n_tiles, n_win = 0, e_win = 0, rg_next = 0;  // tw: the next window ends below tile tw
  int cur_t = 0, cur_nrows = 0;  // the window entry e_win (read when e_win moves)
  uint32_t cur_bits = 0u;
  bool cur_stale = true;
  auto next_item = [&](int& it_t, int& it_rg, uint32_t& it_bits) __attribute__((always_inline)) -> bool {
    while (true) {
      if (e_win >= n_win) {
        if (tw <= t_first) return false;
        const int w_lo = tw - kTileWin > t_first ? tw - kTileWin : t_first;
        n_win = 0;
        for (int x0 = 0; x0 < tw - w_lo; x0 += 64) {
          const int t = tw - 1 - (x0 + l);  // descending
          uint32_t bits = 0u;
          if (t >= w_lo) bits = umask[((long long)g * n_tiles + t) * n_words + (b0 >> 5)] & wmask;
          const uint64_t m = ballot(bits != 0u);
          if (bits) {
            const int pos = n_win + popc64(m & lanemask_lt());
            win_tile[pos] = t;
            win_bits[pos] = bits;
          }
          n_win += popc64(m);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        tw = w_lo;
        e_win = 0;
        rg_next = 0;
        cur_stale = true;
        continue;
      }
      if (cur_stale) {
        cur_t = win_tile[e_win];
        cur_bits = win_bits[e_win];
        cur_nrows = rg_rows(cur_t);
        cur_stale = false;
      }
      if (rg_next * 32 >= cur_nrows) {
        ++e_win;
        rg_next = 0;
        cur_stale = true;
        continue;
      }
      const int rg = rg_next++;
      const int last_q = cur_t * tile + div_r(min(rg * 32 + 31, cur_nrows - 1));
      if (last_q < j0) continue;  // every key of the wave is past every query of the group
      it_t = cur_t;
      it_rg = rg;
      it_bits = cur_bits;
      return true;
    }
  };
  auto is_member = [&](uint32_t bits) -> bool { return ((bits >> ((b0 & 31) + my_blk)) & 1u) != 0u; };
  // Software pipeline over two buffers: the next item's rows are loaded while an item is computed.
  uint8_t* rb0 = rows0[wave];
  uint8_t* rb1 = rows1[wave];
  float* ld0 = lsde0[wave];
  float* ld1 = lsde1[wave];
  int* qr0 = qrow0[wave];
  int* qr1 = qrow1[wave];
  int ta, rga, tb, rgb;
  uint32_t bitsa, bitsb;
  u32x4 sq[8], sd[8];
  float sls, sde;
  int sqi;
  bool ha = next_item(ta, rga, bitsa);
  if (ha) {
    load_rg(ta, rga, sq, sd, sls, sde, sqi);
    store_rg(rb0, ld0, qr0, sq, sd, sls, sde, sqi);
  }
  while (ha) {
    const bool hb = next_item(tb, rgb, bitsb);
    if (hb) load_rg(tb, rgb, sq, sd, sls, sde, sqi);
    compute_rg(rb0, ld0, qr0, is_member(bitsa));
    if (!hb) break;
    store_rg(rb1, ld1, qr1, sq, sd, sls, sde, sqi);
    ha = next_item(ta, rga, bitsa);
    if (ha) load_rg(ta, rga, sq, sd, sls, sde, sqi);
    compute_rg(rb1, ld1, qr1, is_member(bitsb));
    if (ha) store_rg(rb0, ld0, qr0, sq, sd, sls, sde, sqi);
  }

  // dk[g][key][d] = sigma * dK^T[d][key], dv[g][key][d] = dV^T[d][key].
  if (key_ok) {
    const long long base = ((long long)g * n_tokens + key) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + 8 * a + 4 * hi;
        uint2 pk;
        pk.x = pack_bf16x2(adk[dt][4 * a] * scale, adk[dt][4 * a + 1] * scale);
        pk.y = pack_bf16x2(adk[dt][4 * a + 2] * scale, adk[dt][4 * a + 3] * scale);
        *reinterpret_cast<uint2*>(dk + base + d) = pk;
        pk.x = pack_bf16x2(adv[dt][4 * a], adv[dt][4 * a + 1]);
        pk.y = pack_bf16x2(adv[dt][4 * a + 2], adv[dt][4 * a + 3]);
        *reinterpret_cast<uint2*>(dv + base + d) = pk;
      }
  }
}

// ------------------------------------------------------------------------------------ dk, dv: tile-major
//
// The same sums, organised by tile: a work item is 128 consecutive entries of one union U(t,g) (the
// union's blocks in ascending order, B tokens each), four waves of 32 keys; it streams the tile's
// Q and dO rows once through a shared LDS double buffer, and every row's Q/dO slice serves all 128
// keys. An item writes its keys' unscaled dK^T and dV^T columns (fp32) as one partial row per key;
// a second kernel adds, for every key, the partial rows of the tiles that hold it in ascending tile
// order, so the result does not depend on the scheduling. Partial rows are Σ_t |U(t,g)| B per
// group, data dependent and up to the whole causal triangle, so the (tile, group) pairs are taken
// in batches of at most a fixed number of rows: a planning pass on the device numbers the pairs'
// rows and items, and batch b holds the pairs whose first row lies in [b H, (b + 1) H) with H the
// batch size minus the largest pair; the host launches the worst-case number of batches, and the
// kernels of an empty batch return at once. The partial rows alternate between two buffers: the
// sums of batch b (bound by HBM) run on a second stream while the products of batch b + 1 (bound
// by the matrix cores and LDS, one wave per SIMD) fill the other buffer, the two kernels sharing
// the CUs.

namespace {
constexpr int kTmWaves = 4;
constexpr int kTmKeys = kTmWaves * 32;      // union entries per work item
constexpr int kTmRowFloats = 2 * kD;        // partial row: dK^T column, then dV^T column
constexpr long long kTmCapRows = 1LL << 21; // partial rows per batch buffer (2 GiB; two buffers)
constexpr int kTmReduceLds = 96 * 1024;     // LDS reserved (unused) by a reduce workgroup
constexpr int kTmMaxBatches = 2048;         // more batches than this: the key-major kernel runs
constexpr int kTmPlanThreads = 1024;
struct TmItem {
  uint32_t pair, word;  // (tile, group) pair t * G + g; mask word holding the item's first block
};

// Word w of a tile's union mask restricted to the blocks <= c_hi (the tile's causal range).
__device__ __forceinline__ uint32_t tm_word(const uint32_t* mrow, int w, int c_hi) {
  const int wl = c_hi >> 5;
  if (w > wl) return 0u;
  uint32_t m = mrow[w];
  if (w == wl && (c_hi & 31) != 31) m &= (2u << (c_hi & 31)) - 1u;
  return m;
}

// Last block of tile t's causal range.
__device__ __forceinline__ int tm_chi(int t, int n_tokens, int tile, int block_shift) {
  const long long end = min((long long)n_tokens, (long long)(t + 1) * tile);
  return (int)((end - 1) >> block_shift);
}

// Block-wide exclusive scan of a 64-bit value per thread (NT threads; scratch: NT/64 entries).
template <int NT>
__device__ __forceinline__ unsigned long long block_scan_u64(unsigned long long v, unsigned long long* scratch,
                                                             unsigned long long* total) {
  const int l = lane_id(), wave = threadIdx.x >> 6;
  unsigned long long incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(incl, off, 64);
    if (l >= off) incl += o;
  }
  if (l == 63) scratch[wave] = incl;
  __syncthreads();
  unsigned long long before = 0, all = 0;
  for (int x = 0; x < NT / 64; ++x) {
    const unsigned long long s = scratch[x];
    if (x < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}
}  // namespace

// Per (tile, group) pair: pre[pair][w] = set bits of the causal union words before w (the rank of
// the word's first block), nblk[pair] = the union's size. One workgroup per pair.
__global__ __launch_bounds__(256) void k_tm_prefix(const uint32_t* __restrict__ umask, uint32_t* __restrict__ pre,
                                                   uint32_t* __restrict__ nblk, int n_tokens, int n_groups, int tile,
                                                   int block_shift, int n_tiles, int n_words) {
  __shared__ int scan[4];
  const int pair = blockIdx.x;
  const int t = pair / n_groups, g = pair - t * n_groups;
  const int c_hi = tm_chi(t, n_tokens, tile, block_shift);
  const int n_w = (c_hi >> 5) + 1;
  const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
  uint32_t* prow = pre + (long long)pair * n_words;
  int base = 0;
  for (int w0 = 0; w0 < n_w; w0 += 256) {
    const int w = w0 + (int)threadIdx.x;
    const int c = w < n_w ? __popc(tm_word(mrow, w, c_hi)) : 0;
    int all;
    const int ex = block_exclusive_scan<256>(c, scan, &all);
    if (w < n_w) prow[w] = (uint32_t)(base + ex);
    base += all;
  }
  if (threadIdx.x == 0) nblk[pair] = (uint32_t)base;
}

// The plan (one workgroup): over the pairs in order t * G + g, ebase = exclusive prefix of the
// partial rows (nblk * B), ipref = exclusive prefix of the items (ceil(nblk / blocks per item)),
// both with the totals appended; bstart[b] = first pair of batch b (pairs whose ebase lies in
// [b * hstep, (b + 1) * hstep)), bstart[n_batches] = n_pairs.
__global__ __launch_bounds__(kTmPlanThreads) void k_tm_plan(const uint32_t* __restrict__ nblk,
                                                            unsigned long long* __restrict__ ebase,
                                                            uint32_t* __restrict__ ipref, int* __restrict__ bstart,
                                                            int n_pairs, int block_shift, long long hstep,
                                                            int n_batches) {
  __shared__ unsigned long long scan[kTmPlanThreads / 64];
  const int per = (n_pairs + kTmPlanThreads - 1) / kTmPlanThreads;
  const int p0 = (int)threadIdx.x * per;
  const int p1 = min(n_pairs, p0 + per);
  const int nbi = kTmKeys >> block_shift;
  unsigned long long rows = 0, items = 0;
  for (int p = p0; p < p1; ++p) {
    rows += (unsigned long long)nblk[p] << block_shift;
    items += (nblk[p] + nbi - 1) / nbi;
  }
  unsigned long long all_rows, all_items;
  unsigned long long er = block_scan_u64<kTmPlanThreads>(rows, scan, &all_rows);
  unsigned long long ei = block_scan_u64<kTmPlanThreads>(items, scan, &all_items);
  if (p0 >= n_pairs) return;
  const unsigned long long h = (unsigned long long)hstep;
  // (The host sizes n_batches so that every batch index stays below it; the clamp keeps the writes
  // inside bstart whatever the mask holds.)
  long long b_prev = p0 == 0 ? -1 : (long long)((er - ((unsigned long long)nblk[p0 - 1] << block_shift)) / h);
  b_prev = min(b_prev, (long long)n_batches - 1);
  for (int p = p0; p < p1; ++p) {
    ebase[p] = er;
    ipref[p] = (uint32_t)ei;
    const long long b = min((long long)(er / h), (long long)n_batches - 1);
    for (long long x = b_prev + 1; x <= b; ++x) bstart[x] = p;
    b_prev = b;
    er += (unsigned long long)nblk[p] << block_shift;
    ei += (nblk[p] + nbi - 1) / nbi;
  }
  if (p1 == n_pairs) {
    ebase[n_pairs] = all_rows;
    ipref[n_pairs] = (uint32_t)all_items;
    for (long long x = b_prev + 1; x <= n_batches; ++x) bstart[x] = n_pairs;
  }
}

// Work items of every pair: items[ipref[pair] + kr] = {pair, word holding block rank kr * (128 / B)}.
__global__ __launch_bounds__(256) void k_tm_items(const uint32_t* __restrict__ umask,
                                                  const uint32_t* __restrict__ pre,
                                                  const uint32_t* __restrict__ ipref, TmItem* __restrict__ items,
                                                  int n_tokens, int n_groups, int tile, int block_shift, int n_tiles,
                                                  int n_words) {
  const int pair = blockIdx.x;
  const int t = pair / n_groups, g = pair - t * n_groups;
  const int c_hi = tm_chi(t, n_tokens, tile, block_shift);
  const int n_w = (c_hi >> 5) + 1;
  const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
  const uint32_t* prow = pre + (long long)pair * n_words;
  const uint32_t base = ipref[pair];
  const int nbi = kTmKeys >> block_shift;
  for (int w = (int)threadIdx.x; w < n_w; w += 256) {
    const int c = __popc(tm_word(mrow, w, c_hi));
    if (c == 0) continue;
    const int p = (int)prow[w];
    for (int kr = (p + nbi - 1) / nbi; kr * nbi < p + c; ++kr) items[base + kr] = TmItem{(uint32_t)pair, (uint32_t)w};
  }
}

// One step of the tile-major row-group pipeline for a wave's 32 keys (lane l holds key column l % 32):
// S = Q K^T and dP = dO V^T of the NEXT row group (buffer bn) go to the matrix cores while the vector
// ALU turns the current group's S and dP (registers s, dp) into P and dS, one score element after
// each product, so that one wave keeps both busy; then dV^T += dO^T P and dK^T += Q^T dS (unscaled)
// of the current group (buffer bc, its rows' lse and delta in lsde, queries in qrow, -1 past the
// tile). On return s, dp hold the next group's S and dP. The arithmetic of every element is that of
// dkdv_rows.
__device__ __forceinline__ void tm_pipe(const uint8_t* bn, const uint8_t* bc, const float* lsde, const int* qrow,
                                        bool take, int key, const bf16x8 (&kb)[8], const bf16x8 (&vb)[8],
                                        f32x16 (&adk)[4], f32x16 (&adv)[4], const RowTileOffsets& lo,
                                        float scale_log2, f32x16& s, f32x16& dp) {
  const int l = lane_id(), hi = l >> 5;
  // Rows of score j: 8 (j / 4) + 4 hi + (j % 4).
  int4 qi4[4];
  float4 ls4[4], de4[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    qi4[a] = *reinterpret_cast<const int4*>(qrow + 8 * a + 4 * hi);
    ls4[a] = *reinterpret_cast<const float4*>(lsde + 8 * a + 4 * hi);
    de4[a] = *reinterpret_cast<const float4*>(lsde + 32 + 8 * a + 4 * hi);
  }
  auto elem = [&](int j) __attribute__((always_inline)) {
    const int a = j >> 2, c = j & 3;
    const int qi = c == 0 ? qi4[a].x : (c == 1 ? qi4[a].y : (c == 2 ? qi4[a].z : qi4[a].w));
    const float ls = c == 0 ? ls4[a].x : (c == 1 ? ls4[a].y : (c == 2 ? ls4[a].z : ls4[a].w));
    const float de = c == 0 ? de4[a].x : (c == 1 ? de4[a].y : (c == 2 ? de4[a].z : de4[a].w));
    const bool ok = take && key <= qi;
    const float p = ok ? fast_exp2(__builtin_fmaf(s[j], scale_log2, -ls)) : 0.0f;
    s[j] = p;
    dp[j] = p * (dp[j] - de);
  };
  f32x16 s2, dp2;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    s2[j] = 0.0f;
    dp2[j] = 0.0f;
  }
  const uint8_t* dobn = bn + kRowTileBytes;
  const int arow = l & 31;
  auto off_of = [&](int ks) { return arow * 256 + 16 * rt_phys(arow, 2 * ks + hi); };
  bf16x8 qa[3], da[3];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    qa[ks] = *reinterpret_cast<const bf16x8*>(bn + off_of(ks));
    da[ks] = *reinterpret_cast<const bf16x8*>(dobn + off_of(ks));
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks + 2 < 8) {
      qa[(ks + 2) % 3] = *reinterpret_cast<const bf16x8*>(bn + off_of(ks + 2));
      da[(ks + 2) % 3] = *reinterpret_cast<const bf16x8*>(dobn + off_of(ks + 2));
    }
    s2 = mfma32(qa[ks % 3], kb[ks], s2);
    elem(2 * ks);
    dp2 = mfma32(da[ks % 3], vb[ks], dp2);
    elem(2 * ks + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 pp[2], pd[2];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pp[ss][e] = (__bf16)s[8 * ss + e];
      pd[ss][e] = (__bf16)dp[8 * ss + e];
    }
  // dV^T += dO^T P, dK^T += Q^T dS; step = 2 dt + ss, operands read two steps ahead.
  const uint8_t* dobc = bc + kRowTileBytes;
  auto tr_op = [&](const uint8_t* base, int step) {
    return rt_tr_read(base + (16 * (step & 1)) * 256, lo.v0[step >> 1], lo.v1[step >> 1]);
  };
  bf16x8 oa[3], qt[3];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    oa[st] = tr_op(dobc, st);
    qt[st] = tr_op(bc, st);
  }
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    if (st + 2 < 8) {
      oa[(st + 2) % 3] = tr_op(dobc, st + 2);
      qt[(st + 2) % 3] = tr_op(bc, st + 2);
    }
    const int dt = st >> 1, ss = st & 1;
    adv[dt] = mfma32(oa[st % 3], pp[ss], adv[dt]);
    adk[dt] = mfma32(qt[st % 3], pd[ss], adk[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
  s = s2;
  dp = dp2;
}

// S and dP of the first row group (buffer b) for tm_pipe.
__device__ __forceinline__ void tm_first(const uint8_t* b, const bf16x8 (&kb)[8], const bf16x8 (&vb)[8], f32x16& s,
                                         f32x16& dp) {
  const int l = lane_id(), hi = l >> 5, arow = l & 31;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    s[j] = 0.0f;
    dp[j] = 0.0f;
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int off = arow * 256 + 16 * rt_phys(arow, 2 * ks + hi);
    s = mfma32(*reinterpret_cast<const bf16x8*>(b + off), kb[ks], s);
    dp = mfma32(*reinterpret_cast<const bf16x8*>(b + kRowTileBytes + off), vb[ks], dp);
  }
}

// Work items of batch `batch`: every key's partial row of the item's tile (see above). A
// persistent grid (a multiple of 8 workgroups): XCD x takes the x-th eighth of the batch's items,
// so the items of one pair, which read the same rows, share an L2.
__global__ __launch_bounds__(kTmWaves * 64) void k_tm_dkdv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint32_t* __restrict__ umask, const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, const uint32_t* __restrict__ pre, const unsigned long long* __restrict__ ebase,
    const uint32_t* __restrict__ ipref, const int* __restrict__ bstart, const TmItem* __restrict__ items,
    float* __restrict__ part, int batch, int n_tokens, int n_q_heads, int n_groups, int block, int block_shift,
    int tile, float scale_log2, int n_tiles, int n_words) {
  __shared__ __align__(16) uint8_t rows0[kRgBytes];  // row groups rg % 3 == 0, 1, 2
  __shared__ __align__(16) uint8_t rows1[kRgBytes];
  __shared__ __align__(16) uint8_t rows2[kRgBytes];
  __shared__ __align__(16) float lsde0[64];  // lse of the 32 rows, then delta
  __shared__ __align__(16) float lsde1[64];
  __shared__ __align__(16) float lsde2[64];
  __shared__ __align__(16) int qrow0[32];    // query of each row (-1 past the tile)
  __shared__ __align__(16) int qrow1[32];
  __shared__ __align__(16) int qrow2[32];
  __shared__ uint32_t blist[kTmKeys];        // the item's blocks
  const int wave = threadIdx.x >> 6, l = lane_id(), hi = l >> 5;
  const int ps = bstart[batch], pe = bstart[batch + 1];
  if (ps >= pe) return;
  // The previous batch's reduction shares the SIMDs (one wave each): these waves issue first.
  __builtin_amdgcn_s_setprio(2);
  const uint32_t it0 = ipref[ps];
  const uint32_t n_items = ipref[pe] - it0;
  const unsigned long long e0 = ebase[ps];
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, n_slot = gridDim.x >> 3;
  const uint32_t i_lo = (uint32_t)(((unsigned long long)n_items * xcd) >> 3);
  const uint32_t i_hi = (uint32_t)(((unsigned long long)n_items * (xcd + 1)) >> 3);

  const int r = n_q_heads / n_groups;
  // x / r for the row indices of a tile, as in k_bwd_dkdv (checked on the host).
  const uint32_t r_magic = r > 1 ? (uint32_t)((0x100000000ull + (uint32_t)r - 1u) / (uint32_t)r) : 0u;
  auto div_r = [&](int x) -> int { return r > 1 ? (int)__umulhi((uint32_t)x, r_magic) : x; };
  const int nbi = kTmKeys >> block_shift;
  const RowTileOffsets lo = row_tile_offsets();
  const bool r_div32 = (32 % r) == 0;
  // This thread's share of a row group: 1-KiB slices ti = 2 wave, 2 wave + 1 of the Q and dO tiles
  // (slice ti, lane l: row 4 ti + l / 16, physical piece l % 16, as in k_bwd_dkdv).
  int frow[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int rw = 4 * (2 * wave + x) + (l >> 4);
    frow[x] = (rw / r) * n_q_heads + rw % r;
  }
  const int lrow = l & 31;
  const int frow_l = (lrow / r) * n_q_heads + lrow % r, fq_l = lrow / r;

  for (uint32_t ii = i_lo + slot; ii < i_hi; ii += n_slot) {
    const uint32_t it = it0 + ii;
    const TmItem item = items[it];
    const int pair = (int)item.pair;
    const int t = pair / n_groups, g = pair - t * n_groups;
    const int kr = (int)(it - ipref[pair]);
    const unsigned long long eb = ebase[pair];
    const int nblk = (int)((ebase[pair + 1] - eb) >> block_shift);
    const int r0 = kr * nbi;
    const int n_r = min(nbi, nblk - r0);
    const int i0 = t * tile;
    const int c_hi = tm_chi(t, n_tokens, tile, block_shift);
    const int nrows = (min(n_tokens, i0 + tile) - i0) * r;
    const int n_rg = (nrows + 31) >> 5;

    // Row group rg of the tile into registers (clamped to the last group: the loads past the end
    // are repeats, never stored where they are read).
    const long long tbase = (long long)i0 * n_q_heads + g * r;
    auto load_rg = [&](int rg, u32x4 (&sq)[2], u32x4 (&sd)[2], float& ls, float& de, int& qi)
                       __attribute__((always_inline)) {
      rg = min(rg, n_rg - 1);
      long long gbase = 0;
      if (r_div32) gbase = tbase + (long long)(rg * (32 / r)) * n_q_heads;
      if (wave == 0) {
        const int rho = rg * 32 + lrow;
        long long rix;
        int qq;
        if (r_div32) {
          qq = rg * (32 / r) + fq_l;
          rix = rho < nrows ? gbase + frow_l : tbase;
        } else {
          const int rr = rho < nrows ? rho : 0;
          qq = div_r(rr);
          rix = tbase + (long long)qq * n_q_heads + (rr - qq * r);
        }
        ls = lse[rix];
        de = delta[rix];
        qi = rho < nrows ? i0 + qq : -1;
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int rw = 4 * (2 * wave + x) + (l >> 4);
        const int rho = rg * 32 + rw;
        long long src_row;
        if (r_div32) {
          src_row = rho < nrows ? gbase + frow[x] : tbase;
        } else {
          const int rr = rho < nrows ? rho : 0;
          const int qq = div_r(rr);
          src_row = tbase + (long long)qq * n_q_heads + (rr - qq * r);
        }
        const int piece = rt_phys(rw, l & 15);
        sq[x] = *reinterpret_cast<const u32x4*>(q + src_row * kD + piece * 8);
        sd[x] = *reinterpret_cast<const u32x4*>(dout + src_row * kD + piece * 8);
      }
    };
    auto store_rg = [&](uint8_t* b, float* lsde, int* qrow, const u32x4 (&sq)[2], const u32x4 (&sd)[2], float ls,
                        float de, int qi) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int ti = 2 * wave + x;
        *reinterpret_cast<u32x4*>(b + ti * 1024 + 16 * l) = sq[x];
        *reinterpret_cast<u32x4*>(b + kRowTileBytes + ti * 1024 + 16 * l) = sd[x];
      }
      if (wave == 0 && l < 32) {
        lsde[l] = ls;
        lsde[32 + l] = de;
        qrow[l] = qi;
      }
    };
    u32x4 sqa[2], sda[2], sqb[2], sdb[2];
    float lsa = 0.0f, dea = 0.0f, lsb = 0.0f, deb = 0.0f;
    int qia = -1, qib = -1;
    load_rg(0, sqa, sda, lsa, dea, qia);
    load_rg(1, sqb, sdb, lsb, deb, qib);

    // The item's blocks (ranks r0 .. r0 + n_r - 1 of the union) into blist: lane l of wave 0 takes
    // mask word item.word + l (+ 64 per round) and lists the item's ranks that fall in it.
    if (wave == 0) {
      const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
      const uint32_t* prow = pre + (long long)pair * n_words;
      const int n_w = (c_hi >> 5) + 1;
      for (int w = (int)item.word + l;; w += 64) {
        const bool in = w < n_w;
        uint32_t m = in ? tm_word(mrow, w, c_hi) : 0u;
        const int p = in ? (int)prow[w] : nblk;
        const int c = __popc(m);
        const int rlo = max(p, r0), rhi = min(p + c, r0 + n_r);
        for (int s = p; s < rlo; ++s) m &= m - 1u;
        for (int rr = rlo; rr < rhi; ++rr) {
          blist[rr - r0] = (uint32_t)(w * 32 + __ffs(m) - 1);
          m &= m - 1u;
        }
        if (__shfl(p + c, 63, 64) >= r0 + n_r) break;
      }
    }
    store_rg(rows0, lsde0, qrow0, sqa, sda, lsa, dea, qia);
    store_rg(rows1, lsde1, qrow1, sqb, sdb, lsb, deb, qib);
    load_rg(2, sqa, sda, lsa, dea, qia);
    __syncthreads();

    // This lane's key: entry kr * 128 + 32 wave + l % 32 of the union.
    const int e = wave * 32 + (l & 31);
    bool key_ok = (e >> block_shift) < n_r;
    int key = key_ok ? (int)blist[e >> block_shift] * block + (e & (block - 1)) : 0;
    key_ok = key_ok && key < n_tokens;
    if (!key_ok) key = 0;
    // Keys ascend with the entry, so lane 0 holds the wave's first key (none valid if it is not).
    const bool wave_keys = __builtin_amdgcn_readfirstlane((int)key_ok) != 0;

    bf16x8 kb[8], vb[8];
    {
      const long long base = ((long long)g * n_tokens + key) * kD + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        kb[ks] = *reinterpret_cast<const bf16x8*>(k + base + 16 * ks);
        vb[ks] = *reinterpret_cast<const bf16x8*>(v + base + 16 * ks);
      }
    }
    f32x16 adk[4], adv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        adk[dt][j] = 0.0f;
        adv[dt][j] = 0.0f;
      }

    // Step rg (B = rg % 3): groups rg and rg + 1 are in buffers B and B + 1 (mod 3), group rg + 2 in
    // register set a, and s, dp hold S and dP of group rg. The step stores group rg + 2 into buffer
    // B + 2 (read last in step rg - 1), loads group rg + 3, and runs tm_pipe: P and dS of group rg
    // with S and dP of group rg + 1, then dV and dK of group rg. Every step issues the same loads and
    // stores (groups past the tile repeat the last one and are never computed).
    f32x16 s, dp;
    if (wave_keys) tm_first(rows0, kb, vb, s, dp);
    auto step = [&](auto phase, int rg) __attribute__((always_inline)) {
      constexpr int B = decltype(phase)::value;
      // Buffers of groups rg (B), rg + 1 and rg + 2, selected at compile time.
      auto buf = [&](auto which) __attribute__((always_inline)) -> uint8_t* {
        constexpr int X = decltype(which)::value;
        return X == 0 ? rows0 : (X == 1 ? rows1 : rows2);
      };
      auto lsde_of = [&](auto which) __attribute__((always_inline)) -> float* {
        constexpr int X = decltype(which)::value;
        return X == 0 ? lsde0 : (X == 1 ? lsde1 : lsde2);
      };
      auto qrow_of = [&](auto which) __attribute__((always_inline)) -> int* {
        constexpr int X = decltype(which)::value;
        return X == 0 ? qrow0 : (X == 1 ? qrow1 : qrow2);
      };
      using Cur = std::integral_constant<int, B>;
      using Next = std::integral_constant<int, (B + 1) % 3>;
      using Free = std::integral_constant<int, (B + 2) % 3>;
      store_rg(buf(Free()), lsde_of(Free()), qrow_of(Free()), sqa, sda, lsa, dea, qia);
      load_rg(rg + 3, sqa, sda, lsa, dea, qia);
      if (wave_keys && rg < n_rg)
        tm_pipe(buf(Next()), buf(Cur()), lsde_of(Cur()), qrow_of(Cur()), key_ok, key, kb, vb, adk, adv, lo,
                scale_log2, s, dp);
      __syncthreads();
    };
    for (int rg = 0; rg < n_rg; rg += 3) {
      step(std::integral_constant<int, 0>(), rg);
      step(std::integral_constant<int, 1>(), rg + 1);
      step(std::integral_constant<int, 2>(), rg + 2);
    }

    // Partial row of this key: unscaled dK^T column (128 floats), then dV^T column.
    if (key_ok) {
      float* dst = part + ((eb - e0) + (unsigned long long)(kr * kTmKeys + e)) * kTmRowFloats;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = dt * 32 + 8 * a + 4 * hi;
          *reinterpret_cast<f32x4*>(dst + d) =
              f32x4{adk[dt][4 * a], adk[dt][4 * a + 1], adk[dt][4 * a + 2], adk[dt][4 * a + 3]};
          *reinterpret_cast<f32x4*>(dst + kD + d) =
              f32x4{adv[dt][4 * a], adv[dt][4 * a + 1], adv[dt][4 * a + 2], adv[dt][4 * a + 3]};
        }
    }
  }
}

// acc[g][j] += the partial rows of key j from the batch's tiles, in ascending tile order. This
// kernel runs on a second stream beside the dk/dv kernel of the next batch, whose workgroup holds
// one wave per SIMD at 424 registers, so it is built to share a CU with it: at most 88 registers a
// lane, one workgroup per CU (a grid of one per CU, and a dynamic-LDS reservation of
// kTmReduceLds that leaves no room for a second one but room for the dk/dv workgroup), persistent
// over 32-key chunks. Wave w owns keys j0 + 8 w .. j0 + 8 w + 7 (one block for B = 8; for any B
// their blocks lie in one mask word), lane l their floats 4 l .. 4 l + 3. The tiles' membership
// words for the wave's keys come 64 tiles at a time, one per lane, and the wave walks only the
// tiles whose union holds one of its keys. Partial rows are read once: non-temporal loads.
__global__ __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(88))) void k_tm_reduce(
    const uint32_t* __restrict__ umask, const uint32_t* __restrict__ pre, const unsigned long long* __restrict__ ebase,
    const int* __restrict__ bstart, const float* __restrict__ part, float* __restrict__ acc, int batch, int n_tokens,
    int n_groups, int block_shift, int tile, int n_tiles, int n_words) {
  const int ps = bstart[batch], pe = bstart[batch + 1];
  if (ps >= pe) return;
  const unsigned long long e0 = ebase[ps];
  // The wave index as a uniform value: keys, rows and row addresses stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), l = lane_id();
  const uint32_t lofs = 4u * (uint32_t)l;
  const int cpg = (n_tokens + 31) >> 5;
  const int n_chunks = cpg * n_groups;
  for (int c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const int g = c / cpg;
    const int k0 = ((c - g * cpg) << 5) + 8 * wave;
    if (k0 >= n_tokens) continue;
    // Tiles of this group in the batch (pairs t * G + g in [ps, pe)) that reach key k0.
    const int t_lo = max(ps - g <= 0 ? 0 : (ps - g + n_groups - 1) / n_groups, k0 / tile);
    const int t_hi = pe - g <= 0 ? 0 : (pe - g + n_groups - 1) / n_groups;
    if (t_lo >= t_hi) continue;
    const int k_end = min(k0 + 8, n_tokens), n_keys = k_end - k0;
    // Rows as a uniform pointer plus this lane's 32-bit float offset (scalar-base addressing).
    float* const arow = acc + ((long long)g * n_tokens + k0) * kTmRowFloats;
    const int b_first = k0 >> block_shift, b_last = (k_end - 1) >> block_shift;
    const int wa = b_first >> 5;
    const uint32_t wmask =
        ((b_last & 31) == 31 ? ~0u : (2u << (b_last & 31)) - 1u) & ~((1u << (b_first & 31)) - 1u);
    bool started = false;
    f32x4 a[8];
    for (int tb = t_lo; tb < t_hi; tb += 64) {
      const int tl = tb + l;
      uint32_t w_l = 0u;
      if (tl < t_hi)
        w_l = tm_word(umask + ((long long)g * n_tiles + tl) * n_words, wa, tm_chi(tl, n_tokens, tile, block_shift));
      uint64_t hit = ballot((w_l & wmask) != 0u);
      if (hit == 0) continue;
      uint32_t p_l = 0u;
      unsigned long long base_l = 0;
      if (w_l & wmask) {
        const int pair = tl * n_groups + g;
        p_l = pre[(long long)pair * n_words + wa];
        base_l = ebase[pair] - e0;
      }
      if (!started) {
        started = true;
#pragma unroll
        for (int m = 0; m < 8; ++m)
          a[m] = m < n_keys ? *reinterpret_cast<const f32x4*>(arow + (lofs + 256u * m)) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      while (hit) {
        const int x = __builtin_ctzll(hit);
        hit &= hit - 1;
        const uint32_t w_t = __builtin_amdgcn_readlane(w_l, x), p_t = __builtin_amdgcn_readlane(p_l, x);
        const unsigned long long base_t =
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(base_l >> 32), x) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((uint32_t)base_l, x);
        f32x4 xs[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int key = k0 + m;
          const int bit = (key >> block_shift) & 31;
          const bool member = key < n_tokens && ((w_t >> bit) & 1u);
          const uint32_t rank = p_t + __popc(w_t & ((1u << bit) - 1u));
          const unsigned long long row =
              member ? base_t + ((unsigned long long)rank << block_shift) + (key & ((1 << block_shift) - 1)) : 0ull;
          const float* prow = part + row * kTmRowFloats;  // uniform
          xs[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(prow + lofs));
          if (!member) xs[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) a[m] += xs[m];
      }
    }
    if (started) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (m < n_keys) *reinterpret_cast<f32x4*>(arow + (lofs + 256u * m)) = a[m];
    }
  }
}

// dk = bf16(sigma * acc dK part), dv = bf16(acc dV part); 8 floats per thread.
__global__ __launch_bounds__(256) void k_tm_final(const float* __restrict__ acc, uint16_t* __restrict__ dk,
                                                  uint16_t* __restrict__ dv, long long n_rows, float scale) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = x >> 5;
  const int part = (int)(x & 31);
  if (row >= n_rows) return;
  const float* src = acc + row * kTmRowFloats + part * 8;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
  const float s = part < 16 ? scale : 1.0f;
  uint4 pk;
  pk.x = pack_bf16x2(a[0] * s, a[1] * s);
  pk.y = pack_bf16x2(a[2] * s, a[3] * s);
  pk.z = pack_bf16x2(b[0] * s, b[1] * s);
  pk.w = pack_bf16x2(b[2] * s, b[3] * s);
  uint16_t* dst = (part < 16 ? dk : dv) + row * kD + (part & 15) * 8;
  *reinterpret_cast<uint4*>(dst) = pk;
}

__global__ __launch_bounds__(256) void k_tm_zero(f32x4* __restrict__ p, long long n4) {
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n4; x += (long long)gridDim.x * 256)
    p[x] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// ------------------------------------------------------------------------------------ launch

// Static LDS of the dq kernel (two stages, four token tables, scan words) and its dynamic part (the
// block list).
constexpr size_t kDqStaticBytes = 2 * (size_t)kDqStageBytes + 4 * kKeys * 4 + 64;
// One segment of the block list (32-bit ids), as in the forward; a multiple of a chunk's entries.
constexpr int kDqListCap = 12288;
static_assert(kDqStaticBytes + 4 * kDqListCap <= kGfx950LdsBytes, "list segment fits the LDS");
int dq_list_cap(int n_tokens, int block) {
  const long long nbc = ((long long)n_tokens + block - 1) / block;
  const long long cap = (nbc + 63) / 64 * 64;
  return cap < kDqListCap ? (int)cap : kDqListCap;
}
size_t attend_bwd_dq_list_bytes(int n_tokens, int block) { return (size_t)dq_list_cap(n_tokens, block) * 4; }
size_t attend_bwd_lds_dq(int n_tokens, int block) {
  return kDqStaticBytes + attend_bwd_dq_list_bytes(n_tokens, block);
}

// Workspace plan of the backward: delta first; with the tile-major dk/dv also the fp32 gradient
// accumulator [G][N][256], the pair tables, the work items and the partial rows of one batch.
BwdPlan attend_bwd_plan(int n_tokens, int n_q_heads, int n_groups, int block, int tile) {
  BwdPlan pl;
  auto rup = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.bytes = rup((size_t)n_tokens * n_q_heads * 4);
  const char* path = getenv("SGQA_BWD_PATH");
  if (path && strcmp(path, "key") == 0) return pl;
  const int shift = __builtin_ctz(block);
  const long long n_tiles = ((long long)n_tokens + tile - 1) / tile;
  const long long nbc = ((long long)n_tokens + block - 1) / block;
  const long long n_words = (nbc + 31) / 32;
  const long long nbi = kTmKeys / block;
  long long rows_bound = 0, items_bound = 0;
  for (long long t = 0; t < n_tiles; ++t) {
    const long long end = (t + 1) * tile < n_tokens ? (t + 1) * tile : n_tokens;
    const long long nb = ((end - 1) >> shift) + 1;
    rows_bound += (long long)n_groups * (nb << shift);
    items_bound += (long long)n_groups * ((nb + nbi - 1) / nbi);
  }
  const long long unit_max = nbc << shift;  // the last tile's union at most
  long long cap = kTmCapRows;
  if (const char* e = getenv("SGQA_BWD_BATCH_ROWS")) {
    const long long x = atoll(e);
    if (x > 0 && x < cap) cap = x;
  }
  if (cap < 2 * unit_max) cap = 2 * unit_max;
  long long hstep, n_batches;
  if (cap >= rows_bound) {
    cap = rows_bound;
    hstep = rows_bound;
    n_batches = 1;
  } else {
    hstep = cap - unit_max;
    n_batches = (rows_bound - 1) / hstep + 1;
  }
  const long long n_pairs = n_tiles * n_groups;
  if (n_batches > kTmMaxBatches || items_bound >= (1LL << 32) || n_pairs >= (1LL << 31)) return pl;
  pl.tile_major = true;
  pl.n_pairs = (int)n_pairs;
  pl.n_batches = (int)n_batches;
  pl.hstep = hstep;
  pl.cap_rows = cap;
  size_t off = pl.bytes;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += rup(b);
    return o;
  };
  pl.o_acc = take((size_t)n_groups * n_tokens * kTmRowFloats * 4);
  pl.o_nblk = take((size_t)n_pairs * 4);
  pl.o_ebase = take((size_t)(n_pairs + 1) * 8);
  pl.o_ipref = take((size_t)(n_pairs + 1) * 4);
  pl.o_bstart = take((size_t)(n_batches + 1) * 4);
  pl.o_pre = take((size_t)n_pairs * n_words * 4);
  pl.o_items = take((size_t)items_bound * sizeof(TmItem));
  // Batch b's partial rows go to buffer b % 2: the reduction of batch b runs while the dk/dv kernel
  // fills the other buffer with batch b + 1.
  pl.o_part = take((size_t)(n_batches > 1 ? 2 : 1) * cap * kTmRowFloats * 4);
  pl.bytes = off;
  return pl;
}

namespace {
// The second stream of the tile-major backward on one device (the reductions run there, beside the
// dk/dv kernel on the caller's stream) and the events that order the two, created by the first
// backward on the device and kept until the process ends. The events are shared by the calls on
// the device, so a call holds `mu` while it enqueues its batches.
struct BwdStreams {
  std::once_flag once;
  hipError_t status = hipErrorNotInitialized;
  hipStream_t side = nullptr;
  hipEvent_t dkdv_done[2] = {nullptr, nullptr}, reduce_done[2] = {nullptr, nullptr};
  std::mutex mu;
};
constexpr int kBwdMaxDevices = 64;
BwdStreams g_bwd_streams[kBwdMaxDevices];

BwdStreams* bwd_streams() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kBwdMaxDevices) return nullptr;
  BwdStreams& b = g_bwd_streams[dev];
  std::call_once(b.once, [&b] {
    hipError_t e = hipStreamCreateWithFlags(&b.side, hipStreamNonBlocking);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&b.dkdv_done[i], hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&b.reduce_done[i], hipEventDisableTiming);
    b.status = e;
  });
  return &b;
}
}  // namespace

hipError_t launch_attend_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                             const uint16_t* out, const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                             uint16_t* dv, void* ws, int n_tokens, int n_q_heads, int n_groups, int block,
                             int tile, float scale, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_q_heads;
  if (n_rows == 0) return hipSuccess;
  {  // the dk/dv kernels divide row indices by r with a multiply-high (see k_bwd_dkdv)
    const long long rr = n_q_heads / n_groups;
    const long long tr = (long long)(tile < n_tokens ? tile : n_tokens) * rr;
    if (tr * (rr - 1) >= (1LL << 32)) return hipErrorInvalidValue;
  }
  const BwdPlan pl = attend_bwd_plan(n_tokens, n_q_heads, n_groups, block, tile);
  BwdStreams* bs = nullptr;
  if (pl.tile_major) {  // set up before the first launch, so that a failure launches nothing
    bs = bwd_streams();
    if (!bs) return hipErrorInvalidDevice;
    if (bs->status != hipSuccess) return bs->status;
    if (kTmReduceLds > max_lds_per_block()) return hipErrorInvalidValue;
  }
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* delta = reinterpret_cast<float*>(wsb);
  hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), 0, stream, out, dout, delta,
                     n_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int nbc = (n_tokens + block - 1) / block;
  const int n_words = (nbc + 31) / 32;
  const int r = n_q_heads / n_groups;
  const int shift = __builtin_ctz(block);
  const float scale_log2 = scale * 1.4426950408889634f;
  {
    const int rows_wg = kDqWaves * 32;
    const int tile_rows = (tile < n_tokens ? tile : n_tokens) * r;
    const int parts = (tile_rows + rows_wg - 1) / rows_wg;
    const int n_pairs = n_tiles * n_groups;
    if (attend_bwd_lds_dq(n_tokens, block) > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
    const size_t lds = attend_bwd_dq_list_bytes(n_tokens, block);
    const long long grid = (long long)((n_pairs + 7) / 8) * 8 * parts;
    auto kern = k_bwd_dq<kDqWaves>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDqWaves * 64), lds, stream, q, k, v, umask, lse, delta,
                       dout, dq, n_tokens, n_q_heads, n_groups, block, shift, tile, scale, scale_log2, n_words,
                       parts, n_pairs, dq_list_cap(n_tokens, block));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!pl.tile_major) {
    const int chunks_per_g = (n_tokens + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    hipLaunchKernelGGL(k_bwd_dkdv, dim3((unsigned)(chunks_per_g * n_groups)), dim3(kBwdWaves * 64), 0, stream, q,
                       k, v, umask, lse, delta, dout, dk, dv, n_tokens, n_q_heads, n_groups, block, shift, tile,
                       scale, scale_log2, n_words);
    return hipGetLastError();
  }
  float* acc = reinterpret_cast<float*>(wsb + pl.o_acc);
  uint32_t* nblk = reinterpret_cast<uint32_t*>(wsb + pl.o_nblk);
  unsigned long long* ebase = reinterpret_cast<unsigned long long*>(wsb + pl.o_ebase);
  uint32_t* ipref = reinterpret_cast<uint32_t*>(wsb + pl.o_ipref);
  int* bstart = reinterpret_cast<int*>(wsb + pl.o_bstart);
  uint32_t* pre = reinterpret_cast<uint32_t*>(wsb + pl.o_pre);
  TmItem* items = reinterpret_cast<TmItem*>(wsb + pl.o_items);
  float* part = reinterpret_cast<float*>(wsb + pl.o_part);
  const long long acc_rows = (long long)n_groups * n_tokens;
  hipLaunchKernelGGL(k_tm_zero, dim3(2048), dim3(256), 0, stream, reinterpret_cast<f32x4*>(acc),
                     acc_rows * kTmRowFloats / 4);
  hipLaunchKernelGGL(k_tm_prefix, dim3((unsigned)pl.n_pairs), dim3(256), 0, stream, umask, pre, nblk, n_tokens,
                     n_groups, tile, shift, n_tiles, n_words);
  hipLaunchKernelGGL(k_tm_plan, dim3(1), dim3(kTmPlanThreads), 0, stream, nblk, ebase, ipref, bstart, pl.n_pairs,
                     shift, pl.hstep, pl.n_batches);
  hipLaunchKernelGGL(k_tm_items, dim3((unsigned)pl.n_pairs), dim3(256), 0, stream, umask, pre, ipref, items,
                     n_tokens, n_groups, tile, shift, n_tiles, n_words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cu = device_cu_count();
  const unsigned main_grid = (unsigned)((cu + 7) / 8 * 8);
  const long long n_chunks = (long long)n_groups * ((n_tokens + 31) / 32);
  const unsigned red_grid = (unsigned)(n_chunks < cu ? n_chunks : cu);
  // Batch b: dk/dv on the caller's stream into buffer b % 2 (after the reduction of batch b - 2 has
  // read it), then its reduction on the side stream (after that dk/dv); the side stream keeps the
  // reductions in batch order, and the caller's stream waits for the last one.
  {
    std::lock_guard<std::mutex> lock(bs->mu);
    for (int b = 0; b < pl.n_batches; ++b) {
      float* pb = part + (size_t)(b & 1) * (size_t)pl.cap_rows * kTmRowFloats;
      if (b >= 2 && (e = hipStreamWaitEvent(stream, bs->reduce_done[b & 1], 0)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_tm_dkdv, dim3(main_grid), dim3(kTmWaves * 64), 0, stream, q, k, v, umask, lse, delta,
                         dout, pre, ebase, ipref, bstart, items, pb, b, n_tokens, n_q_heads, n_groups, block, shift,
                         tile, scale_log2, n_tiles, n_words);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(bs->dkdv_done[b & 1], stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(bs->side, bs->dkdv_done[b & 1], 0)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_tm_reduce, dim3(red_grid), dim3(256), kTmReduceLds, bs->side, umask, pre, ebase, bstart,
                         pb, acc, b, n_tokens, n_groups, shift, tile, n_tiles, n_words);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(bs->reduce_done[b & 1], bs->side)) != hipSuccess) return e;
    }
    e = hipStreamWaitEvent(stream, bs->reduce_done[(pl.n_batches - 1) & 1], 0);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_tm_final, dim3((unsigned)((acc_rows * 32 + 255) / 256)), dim3(256), 0, stream, acc, dk, dv,
                     acc_rows, scale);
  return hipGetLastError();
}

hipError_t prepare_attend_bwd_kernels(int lds_max) {
  hipError_t e = allow_full_lds((const void*)k_bwd_dq<kDqWaves>, lds_max);
  if (e == hipSuccess && kTmReduceLds <= lds_max)
    e = hipFuncSetAttribute((const void*)k_tm_reduce, hipFuncAttributeMaxDynamicSharedMemorySize, kTmReduceLds);
  return e;
}

}  // namespace sgqa
