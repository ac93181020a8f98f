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
//  * dk, dv: key-major, so that every key's sum runs over its rows in one place. A wave owns 32
//    consecutive keys of one group (their K and V as persistent B operands) and walks the tiles
//    whose union holds one of its blocks; per 32-row group of such a tile, Q and dO rows are
//    gathered into the wave's swizzled LDS tiles (double-buffered, one group ahead), S = Q K^T and
//    dP = dO V^T give P and dS with the keys in the lane columns, and dV^T += dO^T P,
//    dK^T += Q^T dS take dO^T and Q^T transposed from LDS.
#ifndef SGQA_BWD_WAVES
#define SGQA_BWD_WAVES 4
#endif

#include "attn_common.hpp"

namespace sgqa {

namespace {

constexpr int kBwdWaves = SGQA_BWD_WAVES;  // dk/dv workgroup (one wave per SIMD)
constexpr int kDqWaves = 8;                 // dq workgroup (two waves per SIMD, as the forward)
// dq stage: padded K tile, padded V tile, swizzled K tile, token table.
constexpr int kDqKs = 2 * kKTileBytes;                          // swizzled K tile offset
constexpr int kDqTok = kDqKs + kVTileBytes;                     // token table offset
constexpr int kDqStageBytes = kDqTok + kKeys * 4;
constexpr int kDqInsts = 2 * kKTileInsts + kVTileInsts;         // 17 + 17 + 16 wave-wide loads

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
                                                       int n_words, int parts, int n_pairs) {
  constexpr int NT = WAVES * 64;
  constexpr int kRowsWg = WAVES * 32;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;                                             // 2 x kDqStageBytes
  int* scan = reinterpret_cast<int*>(smem + 2 * kDqStageBytes);      // WAVES ints (padded to 16)
  uint16_t* list = reinterpret_cast<uint16_t*>(smem + 2 * kDqStageBytes + 16 * ((WAVES + 4) / 4));

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

  // U(t,g) restricted to blocks <= c_hi, as an ascending list (as in the forward).
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
    const int tk = ((int)list[kp >> block_shift] << block_shift) + (kp & (block - 1));
    return tk < n_tokens ? tk : -1;
  };
  // Gather of one chunk: padded K (instructions 0..16), padded V (17..33), swizzled K (34..49).
  auto issue = [&](int n, uint8_t* sb) {
    for (int inst = wave; inst < kDqInsts; inst += WAVES) {
      int tile_id, ti;
      if (inst < kKTileInsts) {
        tile_id = 0;
        ti = inst;
      } else if (inst < 2 * kKTileInsts) {
        tile_id = 1;
        ti = inst - kKTileInsts;
      } else {
        tile_id = 2;
        ti = inst - 2 * kKTileInsts;
      }
      const int sl = ti * 64 + l;
      int rw, piece;
      if (tile_id < 2) {
        rw = sl / kKSlotsPerRow;
        piece = sl - rw * kKSlotsPerRow;
        if (piece == 16) piece = 0;  // padding slot: any in-bounds data
      } else {
        rw = sl >> 4;
        piece = v_phys(rw, sl & 15);
      }
      int tkn = tok_at(n, rw);
      if (tkn < 0) tkn = 0;
      const uint16_t* src = (tile_id == 1 ? vbase : kbase) + (long long)tkn * kD + piece * 8;
      uint8_t* dst = sb + (tile_id == 0 ? 0 : (tile_id == 1 ? kKTileBytes : kDqKs)) + ti * 1024;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst, 16, 0, 0);
    }
    if (threadIdx.x < kKeys) {
      const int tk = tok_at(n, (int)threadIdx.x);
      reinterpret_cast<int*>(sb + kDqTok)[threadIdx.x] = tk >= 0 ? tk : 0x7FFFFFFF;
    }
  };

  const LaneOffsets lo = lane_offsets(kDqKs);
  const int hi = l >> 5;
  auto chunk = [&](const uint8_t* sb) {
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
    const int* tok = reinterpret_cast<const int*>(sb + kDqTok);
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

  if (n_chunks > 0) issue(0, stage);
  wait_vm();
  __syncthreads();
  for (int n = 0; n < n_chunks; ++n) {
    const int buf = n & 1;
    if (n + 1 < n_chunks) issue(n + 1, stage + (buf ^ 1) * kDqStageBytes);
    chunk(stage + buf * kDqStageBytes);
    wait_vm();
    __syncthreads();
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
constexpr int kRowTileBytes = 32 * 256;        // 32 rows x 128 bf16, swizzled like the forward's V tile
// Per wave: two buffers of (Q rows, dO rows, query / lse / delta of each row), then the tile window.
constexpr int kRgBytes = 2 * kRowTileBytes + 3 * 32 * 4;
constexpr int kWaveBytes = 2 * kRgBytes + kTileWin * 8;
}  // namespace

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
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, l = lane_id(), hi = l >> 5;
  uint8_t* wbase = smem + wave * kWaveBytes;
  int* win_tile = reinterpret_cast<int*>(wbase + 2 * kRgBytes);
  uint32_t* win_bits = reinterpret_cast<uint32_t*>(win_tile + kTileWin);

  const int chunks_per_g = (n_tokens + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  const int g = blockIdx.x / chunks_per_g;
  const int j0 = ((blockIdx.x % chunks_per_g) * kBwdWaves + wave) * 32;  // this wave's keys j0 .. j0 + 31
  if (j0 >= n_tokens) return;  // wave-uniform; the waves never synchronise with each other
  const int r = n_q_heads / n_groups;
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
  const LaneOffsets lo = lane_offsets(0);

  // Row group `rg` of tile `t`: Q and dO rows into buffer `buf` (swizzled row-major, 8 + 8
  // wave-wide loads), and each row's query, lse and delta.
  auto rg_rows = [&](int t) -> int {
    const int i0 = t * tile;
    return ((i0 + tile <= n_tokens) ? tile : n_tokens - i0) * r;
  };
  auto issue_rg = [&](int t, int rg, int buf) {
    uint8_t* b = wbase + buf * kRgBytes;
    const int nrows = rg_rows(t);
    // The row values first: their wait (before the LDS writes below) then leaves the 16 row loads
    // of this group in flight.
    int qi = -1;
    float ls = 0.0f, de = 0.0f;
    if (l < 32) {
      const int rho = rg * 32 + l;
      if (rho < nrows) {
        qi = t * tile + rho / r;
        const long long rix = (long long)qi * n_q_heads + g * r + rho % r;
        ls = lse[rix];
        de = delta[rix];
      }
    }
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
      const int rw = 4 * ti + (l >> 4);
      const int rho = rg * 32 + rw;
      const int rr = rho < nrows ? rho : 0;
      const long long src_row = (long long)(t * tile + rr / r) * n_q_heads + g * r + rr % r;
      const int piece = v_phys(rw, l & 15);
      __builtin_amdgcn_global_load_lds((const void*)(q + src_row * kD + piece * 8), (lds_void*)(b + ti * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dout + src_row * kD + piece * 8),
                                       (lds_void*)(b + kRowTileBytes + ti * 1024), 16, 0, 0);
    }
    if (l < 32) {
      int* meta = reinterpret_cast<int*>(b + 2 * kRowTileBytes);
      meta[l] = qi;
      reinterpret_cast<float*>(meta + 32)[l] = ls;
      reinterpret_cast<float*>(meta + 64)[l] = de;
    }
  };
  // One row group from buffer `buf`: member = this lane's key block is in the tile's union.
  auto compute_rg = [&](int buf, bool member) {
    const uint8_t* b = wbase + buf * kRgBytes;
    const uint8_t* dob = b + kRowTileBytes;
    const int* meta = reinterpret_cast<const int*>(b + 2 * kRowTileBytes);
    // S = Q K^T, dP = dO V^T: A operands row (l % 32), logical piece 2 ks + (l / 32).
    f32x16 s, dp;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s[j] = 0.0f;
      dp[j] = 0.0f;
    }
    const int arow = l & 31;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int off = arow * 256 + 16 * v_phys(arow, 2 * ks + hi);
      s = mfma32(*reinterpret_cast<const bf16x8*>(b + off), kb[ks], s);
      dp = mfma32(*reinterpret_cast<const bf16x8*>(dob + off), vb[ks], dp);
    }
    // Rows of score j: 8 (j / 4) + 4 hi + (j % 4).
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int4 qi4 = *reinterpret_cast<const int4*>(meta + 8 * a + 4 * hi);
      const float4 ls4 = *reinterpret_cast<const float4*>(meta + 32 + 8 * a + 4 * hi);
      const float4 de4 = *reinterpret_cast<const float4*>(meta + 64 + 8 * a + 4 * hi);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int qi = c == 0 ? qi4.x : (c == 1 ? qi4.y : (c == 2 ? qi4.z : qi4.w));
        const float ls = c == 0 ? ls4.x : (c == 1 ? ls4.y : (c == 2 ? ls4.z : ls4.w));
        const float de = c == 0 ? de4.x : (c == 1 ? de4.y : (c == 2 ? de4.z : de4.w));
        const int j = 4 * a + c;
        const bool ok = member && key_ok && key <= qi;  // qi = -1 for rows past the tile
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
    // dV^T += dO^T P, dK^T += Q^T dS.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        adv[dt] = mfma32(tr_read(dob + lo.v[dt] + (16 * ss) * 256), pp[ss], adv[dt]);
        adk[dt] = mfma32(tr_read(b + lo.v[dt] + (16 * ss) * 256), pd[ss], adk[dt]);
      }
  };

  // Walk the tiles t >= the first one holding a query >= j0, a window of kTileWin at a time; list
  // those whose union holds one of the wave's blocks, then their row groups that reach a query >= j0.
  const int t_first = j0 / tile;
  int pend_t = -1, pend_rg = 0, pend_buf = 0;
  uint32_t pend_bits = 0u;
  for (int tw = t_first; tw < n_tiles; tw += kTileWin) {
    int n_win = 0;
    for (int t0 = tw; t0 < tw + kTileWin && t0 < n_tiles; t0 += 64) {
      const int t = t0 + l;
      uint32_t bits = 0u;
      if (t < n_tiles && t < tw + kTileWin)
        bits = umask[((long long)g * n_tiles + t) * n_words + (b0 >> 5)] & wmask;
      const uint64_t m = ballot(bits != 0u);
      if (bits) {
        const int pos = n_win + popc64(m & lanemask_lt());
        win_tile[pos] = t;
        win_bits[pos] = bits;
      }
      n_win += popc64(m);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int e = 0; e < n_win; ++e) {
      const int t = win_tile[e];
      const uint32_t bits = win_bits[e];
      const int nrows = rg_rows(t);
      for (int rg = 0; rg * 32 < nrows; ++rg) {
        const int last_q = t * tile + min(rg * 32 + 31, nrows - 1) / r;
        if (last_q < j0) continue;  // every key of the wave is past every query of the group
        // Software pipeline: issue this group, then compute the pending one.
        const int buf = pend_t < 0 ? 0 : pend_buf ^ 1;
        issue_rg(t, rg, buf);
        if (pend_t >= 0) {
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // the pending group's 16 loads landed
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          compute_rg(pend_buf, ((pend_bits >> ((b0 & 31) + my_blk)) & 1u) != 0u);
        }
        pend_t = t;
        pend_rg = rg;
        pend_buf = buf;
        pend_bits = bits;
      }
    }
  }
  if (pend_t >= 0) {
    wait_vm();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    compute_rg(pend_buf, ((pend_bits >> ((b0 & 31) + my_blk)) & 1u) != 0u);
  }
  (void)pend_rg;

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

// ------------------------------------------------------------------------------------ launch

size_t attend_bwd_lds_dq(int n_tokens, int block) {
  const int nbc = (n_tokens + block - 1) / block;
  return (size_t)2 * kDqStageBytes + 16 * ((kDqWaves + 4) / 4) + (size_t)((nbc + 7) / 8 * 8) * 2;
}

hipError_t launch_attend_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                             const uint16_t* out, const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk,
                             uint16_t* dv, float* delta, int n_tokens, int n_q_heads, int n_groups, int block,
                             int tile, float scale, hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_q_heads;
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), 0, stream, out, dout, delta,
                     n_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int nbc = (n_tokens + block - 1) / block;
  const int n_words = (nbc + 31) / 32;
  const int r = n_q_heads / n_groups;
  const float scale_log2 = scale * 1.4426950408889634f;
  {
    const int rows_wg = kDqWaves * 32;
    const int tile_rows = (tile < n_tokens ? tile : n_tokens) * r;
    const int parts = (tile_rows + rows_wg - 1) / rows_wg;
    const int n_pairs = n_tiles * n_groups;
    const size_t lds = attend_bwd_lds_dq(n_tokens, block);
    if (lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
    const long long grid = (long long)((n_pairs + 7) / 8) * 8 * parts;
    auto kern = k_bwd_dq<kDqWaves>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDqWaves * 64), lds, stream, q, k, v, umask, lse, delta,
                       dout, dq, n_tokens, n_q_heads, n_groups, block, __builtin_ctz(block), tile, scale,
                       scale_log2, n_words, parts, n_pairs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int chunks_per_g = (n_tokens + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    const size_t lds = (size_t)kBwdWaves * kWaveBytes;
    e = hipFuncSetAttribute((const void*)k_bwd_dkdv, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_dkdv, dim3((unsigned)(chunks_per_g * n_groups)), dim3(kBwdWaves * 64), lds, stream, q,
                       k, v, umask, lse, delta, dout, dk, dv, n_tokens, n_q_heads, n_groups, block,
                       __builtin_ctz(block), tile, scale, scale_log2, n_words);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sgqa
