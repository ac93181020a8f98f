// attend.hip -- gathered-block causal GQA flash attention (prefill over tile unions, decode over Sel + own block).
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

#include "attn_common.hpp"


namespace sgqa {

namespace {
// Prefill LDS held in separate variables (two K tiles, two V tiles, four token tables, two
// membership tables, the scan words): with one variable per tile the compiler can tell the
// gathers into one tile from the reads of the other and does not make the reads wait for them.
constexpr int kAttnStaticBytes = 2 * kKTileBytes + 2 * kVTileBytes + 4 * kKeys * 4 + 2 * kSelTableWords * 4 + 64;
}  // namespace


// ------------------------------------------------------------------------------------ prefill

// SEL: the masked-union variant. The union still decides which blocks are gathered, but every Q row
// keeps only the keys of its own query's selection (selbits [G][N][W], bit b of row (g, i) = b in
// Sel(i,g)) and of its own block. Per chunk, the workgroup builds a membership table (one bit per
// (block entry of the chunk, query of the workgroup)) next to the token table, one chunk ahead like
// the K/V gather: the selbits words are loaded before the chunk's gather is issued and turned into
// table words (wave ballots) after the current chunk's products. SEL_LOADS (0 = no masking) is the
// number of table bits each thread computes per chunk.
template <int WAVES, int QT, int SEL_LOADS>
__global__ __launch_bounds__(WAVES * 64) void k_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint32_t* __restrict__ umask,
                                                       uint16_t* __restrict__ out, int n_tokens, int n_q_heads,
                                                       int n_groups, int block, int block_shift, int tile,
                                                       float scale_log2, int n_words, int parts, int n_pairs,
                                                       const uint32_t* __restrict__ selbits,
                                                       float* __restrict__ lse, int list_cap) {
  constexpr int NT = WAVES * 64;
  constexpr int kRowsWg = WAVES * 32 * QT;
  static_assert(WAVES + 1 <= 16, "scan words");
  __shared__ __align__(16) uint8_t k_tile0[kKTileBytes];  // K tiles of the even / odd chunks
  __shared__ __align__(16) uint8_t k_tile1[kKTileBytes];
  __shared__ __align__(16) uint8_t v_tile0[kVTileBytes];  // V tiles of the even / odd chunks
  __shared__ __align__(16) uint8_t v_tile1[kVTileBytes];
  __shared__ __align__(16) int toks[4 * kKeys];                // token tables of chunks n % 4
  __shared__ __align__(16) uint32_t mtabs[2 * kSelTableWords];  // membership tables of chunks n % 2
  __shared__ int scan[16];
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* list = reinterpret_cast<uint32_t*>(smem);  // one segment of the block list

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

  // U(t,g) restricted to blocks <= c_hi as an ascending list of block ids. LDS holds a window of
  // list_cap consecutive entries starting at rank win_lo; the window moves on at the end of a step
  // when the next token table would need an entry past it (only unions longer than list_cap).
  const uint32_t* mrow = umask + ((long long)g * n_tiles + t) * n_words;
  int win_lo = 0, n_list = 0;
  union_list_fill<NT>(mrow, c_hi, list, 0, list_cap, scan, &n_list);
  __syncthreads();

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
  static_assert(WAVES % 2 == 0, "two wave groups");
  // Smallest query of this wave (masking is needed once a chunk reaches past it).
  int wave_i_min = 0x7FFFFFFF;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row0 + (wave * QT + qt) * 32;
    if (row < tile_rows) wave_i_min = min(wave_i_min, i0 + row / r);
  }
  (void)i_lo;

  // Token of key `key` of chunk `chunk` (-1 past the list or the sequence).
  auto tok_at = [&](int chunk, int key) __attribute__((always_inline)) -> int {
    const int kp = chunk * kKeys + key;
    if (kp >= n_keys) return -1;
    const int tk = ((int)list[(kp >> block_shift) - win_lo] << block_shift) + (kp & (block - 1));
    return tk < n_tokens ? tk : -1;
  };

  // Gathers. Loop step n fetches the K tile of chunk n + 1 and the V tile of chunk n. Each lane
  // takes the tokens of its rows from the chunks' token tables, which the first wave writes two steps
  // ahead; invalid keys read row 0 of the group (finite data, masked out through the token table).
  //  * Plain variant, register-staged: in the first half of the step every wave loads its share of
  //    the 16 + 16 wave-wide 16-byte loads (1 KiB each) into registers, and after the mid-step barrier
  //    it writes them to the tiles. Group 1 (softmax first) issues its loads at the start of the
  //    step; group 0 issues one after every second k-step of its score products, so that the 32 loads
  //    of a step do not reach the memory unit in one burst (2-4 % faster than all at the start; group
  //    1 spreading its own loads over its second-half products, or issuing all of them from the
  //    softmax group, measured slower). Unlike LDS-direct loads they do not hold up the issuing wave,
  //    and the compiler has no LDS write in flight to wait for before the operand reads. K load i,
  //    lane l fills row (64 i + l) / 16, piece (64 i + l) % 16 (the padding piece of a K row is never
  //    written); V load i, lane l fills V slot 64 i + l of the tile gather layout.
  //  * Masked variant: LDS-direct loads (tile gather layout, 17 + 16 instructions) in one burst at the
  //    start of the step; it holds the membership state in registers and has none to stage with.
  constexpr bool kStaged = SEL_LOADS == 0;
  constexpr int kKInsts = kStaged ? kKeys * kD * 2 / 1024 : kKTileInsts;
  constexpr int kInsts = kKInsts + kVTileInsts;
  constexpr int kPer = (kInsts + WAVES - 1) / WAVES;  // loads per wave: load xi is load wave + xi * WAVES
  // Staged: loads 0 .. kKPer - 1 of every wave are K loads, the rest V loads.
  constexpr int kKPer = kKInsts / WAVES;
  static_assert(!kStaged || (kKInsts % WAVES == 0 && kInsts % WAVES == 0), "staged loads split evenly");
  auto slot_of = [&](int ii, int& row, int& piece) __attribute__((always_inline)) {
    const bool is_v = ii >= kKInsts;
    const int sl = (is_v ? ii - kKInsts : ii) * 64 + l;
    if (is_v) {
      row = sl >> 4;
      piece = v_phys(row, sl & 15);
    } else if (kStaged) {
      row = sl >> 4;
      piece = sl & 15;
    } else {
      row = sl / kKSlotsPerRow;
      piece = sl - row * kKSlotsPerRow;
      if (piece == 16) piece = 0;  // padding slot: any in-bounds data
    }
  };
  auto load_on = [&](int ii, bool k_on, bool v_on) __attribute__((always_inline)) -> bool {
    return ii < kInsts && (ii >= kKInsts ? v_on : k_on);
  };
  // Tokens of this wave's loads of step n (all table reads before the first load). Without a chunk
  // n + 1 (k_on false) the K loads take token 0 (the staged variant loads and stores them anyway:
  // that K tile is never read).
  auto gather_tokens = [&](int n, int (&tq)[kPer], bool k_on) __attribute__((always_inline)) {
#pragma unroll
    for (int xi = 0; xi < kPer; ++xi) {
      const int ii = wave + xi * WAVES;
      int row, piece;
      slot_of(ii, row, piece);
      const bool is_v = ii >= kKInsts;
      const int t = (is_v ? toks + (n & 3) * kKeys : toks + ((n + 1) & 3) * kKeys)[row & (kKeys - 1)];
      tq[xi] = (t == 0x7FFFFFFF || !(is_v || k_on)) ? 0 : t;
    }
  };
  auto src_of = [&](int ii, int tk) __attribute__((always_inline)) -> const uint16_t* {
    int row, piece;
    slot_of(ii, row, piece);
    return (ii >= kKInsts ? vbase : kbase) + piece * 8 + (long long)tk * kD;
  };
  // Masked variant: load xi of this wave for step n, K rows of chunk n + 1 into kdst (if k_on), V
  // rows of chunk n into vdst (if v_on), LDS-direct.
  auto gather_one = [&](int xi, const int (&tq)[kPer], uint8_t* kdst, uint8_t* vdst, bool k_on,
                        bool v_on) __attribute__((always_inline)) {
    const int ii = wave + xi * WAVES;
    if (load_on(ii, k_on, v_on)) {
      const bool is_v = ii >= kKInsts;
      uint8_t* dst = (is_v ? vdst : kdst) + (is_v ? ii - kKInsts : ii) * 1024;
      __builtin_amdgcn_global_load_lds((const void*)src_of(ii, tq[xi]), (lds_void*)dst, 16, 0, 0);
    }
  };
  // Plain variant: the same loads into registers, and their stores into the tiles (unconditional, so
  // that the compiler keeps the stores together after the barrier).
  auto stage_load = [&](int xi, const int (&tq)[kPer], u32x4& d) __attribute__((always_inline)) {
    d = *reinterpret_cast<const u32x4*>(src_of(wave + xi * WAVES, tq[xi]));
  };
  auto stage_store = [&](int xi, const u32x4& d, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const int ii = wave + xi * WAVES;
    const bool is_v = xi >= kKPer;
    const int sl = (is_v ? ii - kKInsts : ii) * 64 + l;
    uint8_t* dst = is_v ? vdst + 16 * sl : kdst + (sl >> 4) * kKRowBytes + 16 * (sl & 15);
    *reinterpret_cast<u32x4*>(dst) = d;
  };
  auto write_tokens = [&](int c) __attribute__((always_inline)) {  // token table of chunk c
    if (threadIdx.x < kKeys && c < n_chunks) {
      const int tk = tok_at(c, (int)threadIdx.x);
      toks[(c & 3) * kKeys + threadIdx.x] = tk >= 0 ? tk : 0x7FFFFFFF;
    }
  };
  // A chunk needs the causal / tail mask when its last key lies above this wave's first query or
  // past the list (tokens ascend with the chunk index): its token table's last entry says so.
  auto needs_mask = [&](int n) -> bool { return toks[(n & 3) * kKeys + kKeys - 1] > wave_i_min; };

  // SEL: queries of this workgroup, membership table words per block entry, this lane's query index.
  const int nq = i_hi - i_lo + 1, nqw = (nq + 31) >> 5;
  const int ents = kKeys >> block_shift;  // block entries per chunk (block <= 64)
  const int pairs = ents * nqw * 32;      // <= SEL_LOADS per thread (chosen on the host)
  int ql[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) ql[qt] = row_pos[qt] < 0 ? 0 : min(max(row_pos[qt] - i_lo, 0), nq - 1);
  constexpr bool SEL = SEL_LOADS > 0;
  constexpr int kLoads = SEL ? SEL_LOADS : 1;
  // Operand reads in flight ahead of the products (fewer in the masked variant, which holds the
  // membership state in registers).
  constexpr int kKAhead = SEL ? 2 : kKReadsAhead;
  constexpr int kVAhead = SEL ? 2 : kVReadsAhead;
  uint32_t sel_word[kLoads];  // the selbits word of this thread's table bit j, loaded a chunk ahead
  // Table bit pp: block entry e of chunk n, query qq of the workgroup.
  auto sel_pair = [&](int n, int pp, int& b, int& i) __attribute__((always_inline)) -> bool {
    const int e = pp / (nqw * 32), qq = ((pp >> 5) % nqw) * 32 + (pp & 31);
    const int ent = n * ents + e;
    i = i_lo + qq;
    const bool ok = pp < pairs && qq < nq && ent < n_list && i < n_tokens;
    b = ok ? (int)list[ent - win_lo] : 0;
    return ok;
  };
  auto sel_load = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      int b, i;
      const bool ok = sel_pair(n, (int)threadIdx.x + j * (WAVES * 64), b, i);
      sel_word[j] = ok ? selbits[((long long)g * n_tokens + i) * n_words + (b >> 5)] : 0u;
    }
  };
  auto sel_store = [&](int n) __attribute__((always_inline)) {
    uint32_t* mt = mtabs + (n & 1) * kSelTableWords;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (j * (WAVES * 64) + (int)(threadIdx.x & ~63) < pairs) {  // wave-uniform
        const int pp = (int)threadIdx.x + j * (WAVES * 64);
        int b, i;
        const bool ok = sel_pair(n, pp, b, i);
        const bool bit = ok && (((sel_word[j] >> (b & 31)) & 1u) || b == (i >> block_shift));
        const uint64_t bl = ballot(bit);
        if ((l & 31) == 0 && pp < pairs) mt[pp >> 5] = (uint32_t)(bl >> (l & 32));
      }
    }
  };

  // Two wave groups take turns on each SIMD (wave w and wave w + WAVES / 2 share one): while one
  // group runs the matrix-core products of a chunk, the other runs the softmax of its previous
  // chunk. Step n starts the gathers of K(n + 1) and V(n). Half-period 2n: group 0 computes S(n) and
  // P(n - 1) V(n - 1), group 1 runs the softmax of chunk n - 1. Then the staged gathers are written
  // to the tiles. Half-period 2n + 1: group 0 the softmax of chunk n, group 1 S(n) and
  // P(n - 1) V(n - 1); the membership table of chunk n + 1 is built; then the workgroup syncs (the
  // LDS-direct gathers are waited for first). A K tile is read up to
  // half-period 2n + 1, a V tile up to 2n + 3, a token table (written in step n - 2) up to 2n + 2
  // and a membership table from 2n + 1 to 2n + 2: two K, two V, four token and two membership
  // slots suffice.
  const LaneOffsets lo = lane_offsets(0);
  const bool has_rows = wave_i_min != 0x7FFFFFFF;
  const int grp = wave / (WAVES / 2);
  f32x16 s[QT][2];
  bf16x8 pb[QT][4];
  auto softmax = [&](int n) __attribute__((always_inline)) {
    if (!has_rows || n < 0 || n >= n_chunks) return;
    const int* tk = toks + (n & 3) * kKeys;
    if constexpr (SEL) {
      chunk_softmax<QT, 1, true>(s, tk, st, scale_log2, true, row_pos, pb, mtabs + (n & 1) * kSelTableWords, nqw,
                                 ql, block_shift);
    } else {
      if (needs_mask(n))
        chunk_softmax<QT, 1>(s, tk, st, scale_log2, true, row_pos, pb);
      else
        chunk_softmax<QT, 0>(s, tk, st, scale_log2, false, row_pos, pb);
    }
  };
  // One loop step n; P = n % 2 picks the tiles (compile-time, so that every access names its tile).
  auto step = [&](auto parity, int n) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    uint8_t* k_cur = P ? k_tile1 : k_tile0;   // K(n)
    uint8_t* k_next = P ? k_tile0 : k_tile1;  // K(n + 1)
    uint8_t* v_cur = P ? v_tile1 : v_tile0;   // V(n)
    uint8_t* v_prev = P ? v_tile0 : v_tile1;  // V(n - 1)
    const bool k_on = n + 1 < n_chunks, v_on = n < n_chunks;
    int tq[kPer];                    // tokens of this wave's gathers of step n
    u32x4 stg[kStaged ? kPer : 1];  // staged gathers of step n
    // S(n) and P(n - 1) V(n - 1) at raised wave priority. Staged variant: group 0 issues its gathers
    // of the step here (a wave without rows issues them at once; in group 1 that repeats loads it
    // has already stored, which is harmless and keeps the compiler's counter waits out of the
    // products).
    auto products = [&]() __attribute__((always_inline)) {
      if (!has_rows) {
        if (kStaged && n < n_chunks)
#pragma unroll
          for (int xi = 0; xi < kPer; ++xi) stage_load(xi, tq, stg[xi]);
        return;
      }
      __builtin_amdgcn_s_setprio(1);
      if (n < n_chunks) {
        auto hook = [&](int ks) __attribute__((always_inline)) {
          if (kStaged && grp == 0 && (ks & 1) == 0 && (ks >> 1) < kPer) stage_load(ks >> 1, tq, stg[ks >> 1]);
        };
        score_products<QT, decltype(hook), kKAhead>(k_cur, lo, qreg, s, hook);
      }
      if (n >= 1) pv_products<QT, kVAhead>(v_prev, lo, pb, st);
      __builtin_amdgcn_s_setprio(0);
    };
    if constexpr (SEL)
      if (n + 1 < n_chunks) sel_load(n + 1);
    if (n < n_chunks) {
      gather_tokens(n, tq, k_on);
      if (!kStaged || grp == 1)
#pragma unroll
        for (int xi = 0; xi < kPer; ++xi) {
          if constexpr (kStaged)
            stage_load(xi, tq, stg[xi]);
          else
            gather_one(xi, tq, k_next, v_cur, k_on, v_on);
        }
    }
    if (grp == 0) {
      products();
      write_tokens(n + 2);
    } else {
      softmax(n - 1);
    }
    __builtin_amdgcn_s_barrier();
    if constexpr (kStaged)
      if (n < n_chunks)
#pragma unroll
        for (int xi = 0; xi < kPer; ++xi) stage_store(xi, stg[xi], k_next, v_cur);
    if (grp == 0)
      softmax(n);
    else
      products();
    if constexpr (SEL)
      if (n + 1 < n_chunks) sel_store(n + 1);
    if constexpr (!kStaged) wait_vm();
    __syncthreads();
    // Step n + 1 writes the token table of chunk n + 3 and builds the membership table of chunk
    // n + 2: move the window to start at chunk n + 2 when chunk n + 3 reaches past it.
    if (n + 3 < n_chunks && (((n + 4) * kKeys - 1) >> block_shift) >= win_lo + list_cap) {
      int unused;
      win_lo = ((n + 2) * kKeys) >> block_shift;
      union_list_fill<NT>(mrow, c_hi, list, win_lo, list_cap, scan, &unused);
      __syncthreads();
    }
  };
  if (n_chunks > 0) {
    if constexpr (SEL) sel_load(0);
    write_tokens(0);
    write_tokens(1);
    __syncthreads();
    {  // the K tile of chunk 0
      int tq[kPer];
      gather_tokens(-1, tq, true);
      if constexpr (kStaged) {  // the K loads only
        u32x4 stg[kKPer > 0 ? kKPer : 1];
#pragma unroll
        for (int xi = 0; xi < kKPer; ++xi) stage_load(xi, tq, stg[xi]);
#pragma unroll
        for (int xi = 0; xi < kKPer; ++xi) stage_store(xi, stg[xi], k_tile0, v_tile0);
      } else {
#pragma unroll
        for (int xi = 0; xi < kPer; ++xi) gather_one(xi, tq, k_tile0, v_tile0, true, false);
        wait_vm();
      }
    }
    if constexpr (SEL) sel_store(0);
    __syncthreads();
  }
  // Every global load so far (Q operands, the prologue) has landed, as a wait the compiler sees:
  // otherwise it assumes them in flight at the loop head and waits for all loads (the staged
  // gathers included) before the first operand of every step.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  const int n_steps = n_chunks + (n_chunks > 0);
  for (int n = 0; n < n_steps; n += 2) {
    step(std::integral_constant<int, 0>(), n);
    if (n + 1 < n_steps) step(std::integral_constant<int, 1>(), n + 1);
  }

  // out[i][h][d] = O^T[d][row] / l
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l_all = st.l[qt] + __shfl_xor(st.l[qt], 32, 64);
    const int row = row0 + (wave * QT + qt) * 32 + (l & 31);
    if (row >= tile_rows) continue;
    const int i = i0 + row / r, h = g * r + row % r;
    const float inv = 1.0f / l_all;
    // Base-2 log-sum-exp of the row's scaled logits (for the backward pass).
    if (lse && l < 32) lse[(long long)i * n_q_heads + h] = st.m[qt] + __log2f(l_all);
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
constexpr int kPrefillWaves = 8;
constexpr int kPrefillQT = 1;

// Dynamic LDS of the prefill kernel: one segment of the block list, 32-bit ids. The segment holds
// the whole union whenever N / B <= kAttnListCap (every B = 8 sequence up to 128K tokens); longer
// unions are attended segment by segment. The cap is a multiple of the block entries of a chunk.
constexpr int kAttnListCap = 16384;
static_assert(kAttnStaticBytes + 4 * kAttnListCap <= kGfx950LdsBytes, "list segment fits the LDS");
int attend_list_cap(int n_tokens, int block) {
  const long long nbc = ((long long)n_tokens + block - 1) / block;
  const long long cap = (nbc + 63) / 64 * 64;
  return cap < kAttnListCap ? (int)cap : kAttnListCap;
}
size_t attend_lds_bytes(int list_cap) { return (size_t)list_cap * 4; }
}  // namespace

size_t attend_lds_bytes_for(int n_tokens, int block) {
  return kAttnStaticBytes + attend_lds_bytes(attend_list_cap(n_tokens, block));
}

namespace {

template <int SEL_LOADS>
hipError_t launch_attend_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                              const uint32_t* selbits, uint16_t* out, int n_tokens, int n_q_heads, int n_groups,
                              int block, int tile, float scale, hipStream_t stream, float* lse = nullptr) {
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int nbc = (n_tokens + block - 1) / block;
  const int n_words = (nbc + 31) / 32;
  const int r = n_q_heads / n_groups;
  const int rows_wg = kPrefillWaves * 32 * kPrefillQT;
  const int tile_rows = (tile < n_tokens ? tile : n_tokens) * r;
  const int parts = (tile_rows + rows_wg - 1) / rows_wg;
  const int n_pairs = n_tiles * n_groups;
  if (n_pairs == 0) return hipSuccess;
  if (SEL_LOADS > 0 && attend_masked_loads(n_q_heads, n_groups, block) > SEL_LOADS) return hipErrorInvalidValue;
  const int list_cap = attend_list_cap(n_tokens, block);
  const size_t lds = attend_lds_bytes(list_cap);
  if (kAttnStaticBytes + lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  const long long grid = (long long)((n_pairs + 7) / 8) * 8 * parts;
  const float scale_log2 = scale * 1.4426950408889634f;
  auto kern = k_attend<kPrefillWaves, kPrefillQT, SEL_LOADS>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPrefillWaves * 64), lds, stream, q, k, v, umask, out, n_tokens,
                     n_q_heads, n_groups, block, __builtin_ctz(block), tile, scale_log2, n_words, parts, n_pairs,
                     selbits, lse, list_cap);
  return hipGetLastError();
}

}  // namespace

// The membership table of a chunk has (64 / B) block entries times ceil(queries / 32) words, at most
// kSelTableWords; a workgroup spans at most ceil(rows / r) + 1 queries. Returns the table bits per
// thread (1, 2 or 4), or 0 when the table does not fit.
int attend_masked_loads(int n_q_heads, int n_groups, int block) {
  const int r = n_q_heads / n_groups;
  const int rows_wg = kPrefillWaves * 32 * kPrefillQT;
  const int span = (rows_wg + r - 1) / r + 1;
  const int words = (kKeys / block) * ((span + 31) / 32);
  if (words > kSelTableWords) return 0;
  const int loads = (words * 32 + kPrefillWaves * 64 - 1) / (kPrefillWaves * 64);
  return loads <= 1 ? 1 : (loads <= 2 ? 2 : 4);
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                         const int32_t* ucount, uint16_t* out, int n_tokens, int n_q_heads, int n_groups, int block,
                         int tile, float scale, hipStream_t stream, float* lse) {
  (void)ucount;
  return launch_attend_impl<0>(q, k, v, umask, nullptr, out, n_tokens, n_q_heads, n_groups, block, tile, scale,
                               stream, lse);
}

hipError_t launch_attend_masked(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint32_t* umask,
                                const uint32_t* selbits, uint16_t* out, int n_tokens, int n_q_heads, int n_groups,
                                int block, int tile, float scale, hipStream_t stream) {
  const int loads = attend_masked_loads(n_q_heads, n_groups, block);
  if (loads == 1)
    return launch_attend_impl<1>(q, k, v, umask, selbits, out, n_tokens, n_q_heads, n_groups, block, tile, scale,
                                 stream);
  if (loads == 2)
    return launch_attend_impl<2>(q, k, v, umask, selbits, out, n_tokens, n_q_heads, n_groups, block, tile, scale,
                                 stream);
  if (loads == 4)
    return launch_attend_impl<4>(q, k, v, umask, selbits, out, n_tokens, n_q_heads, n_groups, block, tile, scale,
                                 stream);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------ decode

constexpr int kDecVStage = kVTileBytes + kKeys * 4;  // decode: V tile + token table of a chunk

// Decode gather of one wave: the V tile of one chunk (16 wave-wide global_load_lds, tile gather
// layout) and its token table.
// off_of(key) is the element offset (from `base`) of the row of key `key` of the chunk.
template <typename TokFn, typename OffFn>
__device__ __forceinline__ void v_issue_wave(uint8_t* vst, const uint16_t* base, OffFn off_of, TokFn tok_of) {
  const int l = lane_id();
#pragma unroll
  for (int ti = 0; ti < kVTileInsts; ++ti) {
    const int slot = ti * 64 + l;
    const int row = slot >> 4;
    const int piece = v_phys(row, slot & 15);
    __builtin_amdgcn_global_load_lds((const void*)(base + off_of(row) + piece * 8), (lds_void*)(vst + ti * 1024), 16,
                                     0, 0);
  }
  const int t = tok_of(l);
  reinterpret_cast<int*>(vst + kVTileBytes)[l] = t >= 0 ? t : 0x7FFFFFFF;
}

// The K operands of one chunk straight from global memory into registers: the A operand of
// S^T = K Q^T for key tile kt and step ks is key row 32 kt + (l % 32), elements 16 ks + 8 (l / 32)
// .. +7, i.e. 16 contiguous bytes of one cached key.
template <typename OffFn>
__device__ __forceinline__ void k_load_regs(bf16x8 (&kreg)[16], const uint16_t* base, OffFn off_of) {
  const int l = lane_id();
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const uint16_t* src = base + off_of(32 * kt + (l & 31)) + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kreg[ks * 2 + kt] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }
}

// Attended block list of one (sequence s, group g) into LDS: blocks[0 .. n_sel-1] = Sel(s,g)
// (ascending), blocks[n_sel] = the own block; paged caches also get prow[e], the pool row of the
// first token of entry e (a block lies inside one page, the page size being a multiple of B). The
// selection holds exactly n_sel = min(K_B, c) valid entries, c = floor((ctx-1)/B) candidate blocks,
// so no pass over the list is needed to count them, and every thread issues all of its list loads
// (and the length load) before the first wait. Entries are clamped to [0, own], so even a corrupt
// list never addresses outside the caches or the page table. Ends with a barrier.
template <bool PAGED>
__device__ __forceinline__ void load_decode_list(const int32_t* __restrict__ srow, int kb, int ctx, int block_shift,
                                                 int* blocks, int* prow, const int32_t* __restrict__ table_row,
                                                 int page_shift, int n_pages, int n_groups, int g, int& n_sel_out) {
  const int own = (ctx - 1) >> block_shift;
  const int n_sel = own < kb ? own : kb;
  n_sel_out = n_sel;
  for (int e0 = threadIdx.x; e0 <= kb; e0 += 4 * blockDim.x) {
    int b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * blockDim.x;
      b[u] = e < kb ? srow[e] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * blockDim.x;
      const int v = e < n_sel ? b[u] : own;
      b[u] = v < 0 ? 0 : (v > own ? own : v);
    }
    int pg[4];
    if (PAGED) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pg[u] = e0 + u * (int)blockDim.x <= n_sel ? table_row[(b[u] << block_shift) >> page_shift] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * blockDim.x;
      if (e <= n_sel) {
        blocks[e] = b[u];
        if (PAGED) {
          const int p = pg[u] < 0 ? 0 : (pg[u] >= n_pages ? n_pages - 1 : pg[u]);
          const int tb = b[u] << block_shift;
          prow[e] = ((p * n_groups + g) << page_shift) + (tb & ((1 << page_shift) - 1));
        }
      }
    }
  }
  __syncthreads();
}

// Decode attention: one workgroup of 4 waves per (sequence s, group g). The attended blocks are
// Sel(s,g) (ascending) plus the own block; wave w handles chunks w, w+4, ... Decode is a gather at
// HBM rate, so the loop is built to keep bytes in flight: the K operands of a chunk go straight
// into registers (issued as soon as the previous chunk's score products have read theirs), and
// the V tiles, which need the transposing LDS reads, are double-buffered per wave. Each wave keeps
// its own online-softmax state for the r heads (one 32-row tile, r <= 32 rows used); the four
// states are merged in LDS into the bf16 output.
//
// Caches: dense [S][G][cap][D] per sequence (PAGED = false), or pools [n_pages][G][page][D] with the
// position t of sequence s in page table[s * max_pages + t / page] (PAGED = true; page = 1 << page_shift,
// a multiple of B, so a block never straddles two pages; entries outside [0, n_pages) are clamped, so
// a bad table reads wrong data but never outside the pool). The context length of sequence s is
// lens[s] clamped to [1, cap] (cap for every sequence when lens is null).
template <bool PAGED>
__global__ __launch_bounds__(256) void k_decode_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                       const uint16_t* __restrict__ vc,
                                                       const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
                                                       int cap, int n_q_heads, int n_groups, int block,
                                                       int block_shift, int kb, float scale_log2,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ table, int max_pages,
                                                       int page_shift, int n_pages) {
  constexpr int kWavesD = 4;
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6;
  uint8_t* vbuf[2] = {smem + wave * 2 * kDecVStage, smem + wave * 2 * kDecVStage + kDecVStage};
  int* blocks = reinterpret_cast<int*>(smem + kWavesD * 2 * kDecVStage);  // kb + 1 entries
  int* prow = blocks + (kb + 1);  // paged: pool row of each entry's first token (kb + 1 entries)

  const int s = blockIdx.x / n_groups, g = blockIdx.x % n_groups;
  const int r = n_q_heads / n_groups;
  const int l = lane_id();
  int ctx = lens ? lens[s] : cap;
  ctx = ctx < 1 ? 1 : (ctx > cap ? cap : ctx);
  const int i_q = ctx - 1;

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
  int n_sel;
  load_decode_list<PAGED>(sel + ((long long)s * n_groups + g) * kb, kb, ctx, block_shift, blocks, prow,
                          PAGED ? table + (long long)s * max_pages : nullptr, page_shift, n_pages, n_groups, g, n_sel);
  AttnState<1> st;
  state_init(st);
  const long long seq_off = PAGED ? 0 : ((long long)s * n_groups + g) * cap * kD;
  const int n_keys = (n_sel + 1) * block;
  // Element offset of the cache row of key `key` of chunk c (keys past the list or past the context
  // read row 0; the token table masks them).
  auto off_in = [&](int c) {
    return [&, c](int key) -> long long {
      const int kp = c * kKeys + key;
      if (kp >= n_keys) return seq_off;
      const int e = kp >> block_shift, j = kp & (block - 1);
      if (PAGED) return ((long long)prow[e] + j) * kD;  // a block lies inside its page
      const int tk = (blocks[e] << block_shift) + j;  // own-block rows past ctx may lie past cap: masked,
      return seq_off + (long long)(tk < ctx ? tk : 0) * kD;  // so read row 0 instead
    };
  };
  const int n_chunks = (n_keys + kKeys - 1) / kKeys;
  const LaneOffsets lo = lane_offsets(0);
  auto tok_in = [&](int c) {
    return [&, c](int key) -> int {
      const int kp = c * kKeys + key;
      if (kp >= n_keys) return -1;
      const int tk = (blocks[kp >> block_shift] << block_shift) + (kp & (block - 1));
      return tk < ctx ? tk : -1;
    };
  };
  bf16x8 kreg[16];
  if (wave < n_chunks) {
    v_issue_wave(vbuf[0], vc, off_in(wave), tok_in(wave));
    k_load_regs(kreg, kc, off_in(wave));
  }
  int i = 0;
  for (int c = wave; c < n_chunks; c += kWavesD, ++i) {
    const int cn = c + kWavesD;
    if (cn < n_chunks) {
      v_issue_wave(vbuf[(i + 1) & 1], vc, off_in(cn), tok_in(cn));
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // V and K of chunk c landed; V of cn flies
    } else {
      wait_vm();
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // Only the last chunk holds the own block (and the padding past the list): the Sel blocks are
    // all below it, hence visible to the query.
    attn_chunk<1, 2, true>(vbuf[i & 1], lo, qreg, st, scale_log2, c == n_chunks - 1, row_pos, kreg, [&]() {
      if (cn < n_chunks) k_load_regs(kreg, kc, off_in(cn));
    });
  }

  // Merge the four wave states: O^T tiles to LDS (reusing the wave's buffers), then 256 threads
  // combine r x 128 outputs.
  const float l_all = st.l[0] + __shfl_xor(st.l[0], 32, 64);
  float* o_lds = reinterpret_cast<float*>(vbuf[0]);  // [32 rows][128]
  float* ml_lds = reinterpret_cast<float*>(blocks) + 2 * (kb + 1);  // [4][32][2]
  __syncthreads();  // every wave is done with its buffers
  {
    const int row = l & 31;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int d = dt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3);
        o_lds[row * kD + d] = st.o[0][dt][j];
      }
    if (l < 32) {
      ml_lds[(wave * 32 + row) * 2 + 0] = st.m[0];
      ml_lds[(wave * 32 + row) * 2 + 1] = l_all;
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < r * kD; x += blockDim.x) {
    const int row = x / kD, d = x % kD;
    float m = -1.0e30f;
    for (int w = 0; w < kWavesD; ++w) m = fmaxf(m, ml_lds[(w * 32 + row) * 2]);
    float num = 0.0f, den = 0.0f;
    for (int w = 0; w < kWavesD; ++w) {
      const float f = fast_exp2(ml_lds[(w * 32 + row) * 2] - m);
      den += ml_lds[(w * 32 + row) * 2 + 1] * f;
      num += reinterpret_cast<const float*>(smem + w * 2 * kDecVStage)[row * kD + d] * f;
    }
    out[((long long)s * n_q_heads + g * r + row) * kD + d] = (uint16_t)f32_to_bf16_bits(num / den);
  }
}

// ---------------------------------------------------------------------- decode over FP8 K/V caches

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled (register arrays indexed by i stay
// in registers).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// The K/V caches hold OCP FP8 E4M3 codes with one scale per (sequence, group) for K and one for V
// (kv_scale [S][G][2]); every E4M3 value is exact in bf16, so the codes are converted to bf16 and fed
// to the same matrix-core chunk as the bf16 path, the key scale folded into the softmax exponent
// scale and the value scale into the final normalisation. One 4-wave workgroup per (sequence, group)
// as in k_decode_attend; per wave and chunk the K and V codes of the NEXT chunk are gathered into
// registers while the current chunk computes: K straight into MFMA operands (the head dimension is
// permuted so that lane half h holds dims 64h .. 64h + 63, contiguous in the cache row; Q is loaded
// with the same permutation), V converted and written into the wave's bf16 V tile (row-major,
// swizzled as in the tile gather layout) for the transposing reads.
template <bool PAGED, int DEPTH>
__global__ __launch_bounds__(256) void k_decode_attend_f8(const uint16_t* __restrict__ q,
                                                          const uint8_t* __restrict__ kc,
                                                          const uint8_t* __restrict__ vc,
                                                          const float* __restrict__ kv_scale,
                                                          const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
                                                          int cap, int n_q_heads, int n_groups, int block,
                                                          int block_shift, int kb, float scale_log2,
                                                          const int32_t* __restrict__ lens,
                                                          const int32_t* __restrict__ table, int max_pages,
                                                          int page_shift, int n_pages) {
  constexpr int kWavesD = 4;
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6;
  uint8_t* vt = smem + wave * kDecVStage;  // this wave's bf16 V tile + token table
  int* blocks = reinterpret_cast<int*>(smem + kWavesD * kDecVStage);  // kb + 1 entries
  int* prow = blocks + (kb + 1);

  const int s = blockIdx.x / n_groups, g = blockIdx.x % n_groups;
  const int r = n_q_heads / n_groups;
  const int l = lane_id(), h = l >> 5;
  int ctx = lens ? lens[s] : cap;
  ctx = ctx < 1 ? 1 : (ctx > cap ? cap : ctx);
  const int i_q = ctx - 1;
  const float k_scale = kv_scale[((long long)s * n_groups + g) * 2 + 0];
  const float v_scale = kv_scale[((long long)s * n_groups + g) * 2 + 1];

  // Q (B operand of S^T) with the permuted head dimension: step ks, lane half h -> dims 64h + 8ks.
  bf16x8 qreg[1][8];
  int row_pos[1];
  {
    const int hh = l & 31;
    const bool valid = hh < r;
    row_pos[0] = valid ? i_q : -1;
    const uint16_t* src = q + ((long long)s * n_q_heads + g * r + (valid ? hh : 0)) * kD + 64 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (valid) {
        qreg[0][ks] = *reinterpret_cast<const bf16x8*>(src + 8 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[0][ks][e] = (__bf16)0.0f;
      }
    }
  }
  int n_sel;
  load_decode_list<PAGED>(sel + ((long long)s * n_groups + g) * kb, kb, ctx, block_shift, blocks, prow,
                          PAGED ? table + (long long)s * max_pages : nullptr, page_shift, n_pages, n_groups, g, n_sel);
  AttnState<1> st;
  state_init(st);
  const long long seq_off = PAGED ? 0 : ((long long)s * n_groups + g) * cap * kD;
  const int n_keys = (n_sel + 1) * block;
  const int n_chunks = (n_keys + kKeys - 1) / kKeys;
  const LaneOffsets lo = lane_offsets(0);
  // Byte offset of the cache row of key `key` of chunk c; keys past the list or the context (and
  // chunks past the last) read row 0, which the token table masks. Branch-free, so every gather
  // issues the same loads.
  auto off_of = [&](int c, int key) -> long long {
    const int kp = c * kKeys + key;
    const bool in = kp < n_keys;
    const int e = in ? kp >> block_shift : 0, j = kp & (block - 1);
    if (PAGED) return in ? ((long long)prow[e] + j) * kD : 0;
    const int tk = (blocks[e] << block_shift) + j;
    return seq_off + (long long)(in && tk < ctx ? tk : 0) * kD;
  };
  auto tok_of = [&](int c, int key) -> int {
    const int kp = c * kKeys + key;
    if (kp >= n_keys) return -1;
    const int tk = (blocks[kp >> block_shift] << block_shift) + (kp & (block - 1));
    return tk < ctx ? tk : -1;
  };
  // Gathers of one chunk into register set d: K, key row 32 kt + (l % 32), bytes 64h .. 64h + 63
  // (4 x 16 B); V, row 8w + l / 8 for w < 8, bytes 16 (l % 8) .. + 15. DEPTH sets are in flight,
  // the chunks c + 4, c + 8, ... of this wave; the compiler's counter waits release each set.
  u32x4 k8[DEPTH][2][4];
  u32x4 v8[DEPTH][8];
  auto gather = [&](auto dd, int c) {
    constexpr int d = decltype(dd)::value;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint8_t* src = kc + off_of(c, 32 * kt + (l & 31)) + 64 * h;
#pragma unroll
      for (int j = 0; j < 4; ++j) k8[d][kt][j] = *reinterpret_cast<const u32x4*>(src + 16 * j);
    }
#pragma unroll
    for (int w = 0; w < 8; ++w)
      v8[d][w] = *reinterpret_cast<const u32x4*>(vc + off_of(c, 8 * w + (l >> 3)) + 16 * (l & 7));
  };
  auto cvt8 = [](uint32_t w0, uint32_t w1) -> bf16x8 {  // 8 codes (little-endian) -> 8 bf16
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    bf16x8 o;
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
    o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
    return o;
  };
  bf16x8 kreg[16];
  const float sl2 = scale_log2 * k_scale;
  // One chunk from register set d: V codes -> bf16 V tile (the tile gather layout of the V
  // tile) and the token table, K codes -> MFMA operands; then set d is refilled with chunk
  // c + 4 DEPTH (always issued, past the end it reads row 0, so that the number of loads between
  // a set's issue and its use is the same on every path and the counter waits stay partial).
  auto step = [&](auto dd, int c) {
    constexpr int d = decltype(dd)::value;
    const bool live = c < n_chunks;  // wave-uniform
    if (live) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int row = 8 * w + (l >> 3), piece = 2 * (l & 7);
        *reinterpret_cast<bf16x8*>(vt + row * 256 + 16 * v_phys(row, piece)) = cvt8(v8[d][w].x, v8[d][w].y);
        *reinterpret_cast<bf16x8*>(vt + row * 256 + 16 * v_phys(row, piece + 1)) = cvt8(v8[d][w].z, v8[d][w].w);
      }
      const int t = tok_of(c, l);
      reinterpret_cast<int*>(vt + kVTileBytes)[l] = t >= 0 ? t : 0x7FFFFFFF;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kreg[(2 * j) * 2 + kt] = cvt8(k8[d][kt][j].x, k8[d][kt][j].y);
          kreg[(2 * j + 1) * 2 + kt] = cvt8(k8[d][kt][j].z, k8[d][kt][j].w);
        }
    }
    gather(dd, c + DEPTH * kWavesD);
    if (live) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      attn_chunk<1, 2, true>(vt, lo, qreg, st, sl2, c == n_chunks - 1, row_pos, kreg);
    }
  };
  if (wave < n_chunks) {
    static_for<DEPTH>([&](auto dd) { gather(dd, wave + decltype(dd)::value * kWavesD); });
    for (int c0 = wave; c0 < n_chunks; c0 += DEPTH * kWavesD)
      static_for<DEPTH>([&](auto dd) { step(dd, c0 + decltype(dd)::value * kWavesD); });
  }

  // Merge the four wave states (as in k_decode_attend), the value scale applied once at the end.
  const float l_all = st.l[0] + __shfl_xor(st.l[0], 32, 64);
  float* o_lds = reinterpret_cast<float*>(vt);  // [32 rows][128]
  float* ml_lds = reinterpret_cast<float*>(blocks) + 2 * (kb + 1);  // [4][32][2]
  __syncthreads();
  {
    const int row = l & 31;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int d = dt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3);
        o_lds[row * kD + d] = st.o[0][dt][j];
      }
    if (l < 32) {
      ml_lds[(wave * 32 + row) * 2 + 0] = st.m[0];
      ml_lds[(wave * 32 + row) * 2 + 1] = l_all;
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < r * kD; x += blockDim.x) {
    const int row = x / kD, d = x % kD;
    float m = -1.0e30f;
    for (int w = 0; w < kWavesD; ++w) m = fmaxf(m, ml_lds[(w * 32 + row) * 2]);
    float num = 0.0f, den = 0.0f;
    for (int w = 0; w < kWavesD; ++w) {
      const float f = fast_exp2(ml_lds[(w * 32 + row) * 2] - m);
      den += ml_lds[(w * 32 + row) * 2 + 1] * f;
      num += reinterpret_cast<const float*>(smem + w * kDecVStage)[row * kD + d] * f;
    }
    out[((long long)s * n_q_heads + g * r + row) * kD + d] = (uint16_t)f32_to_bf16_bits(num / den * v_scale);
  }
}

// Chunks of FP8 codes in flight per wave (register sets of 32 VGPRs each). One set already keeps
// the gather at the rate of a bare gather loop: a second one measured no faster.
constexpr int kF8Depth = 1;

size_t decode_attend_f8_lds(int kb) { return (size_t)4 * kDecVStage + (size_t)2 * (kb + 1) * 4 + 4 * 32 * 2 * 4; }

hipError_t launch_decode_attend_f8(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* kv_scale,
                                   const int32_t* sel, uint16_t* out, int n_seqs, int ctx, int n_q_heads,
                                   int n_groups, int block, int kb, float scale, const int32_t* lens,
                                   const PageTable& pages, hipStream_t stream) {
  const size_t lds = decode_attend_f8_lds(kb);
  if (lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(n_seqs * n_groups));
  if (pages.table)
    hipLaunchKernelGGL((k_decode_attend_f8<true, kF8Depth>), grid, dim3(256), lds, stream, q, kc, vc, kv_scale, sel,
                       out, ctx, n_q_heads, n_groups, block, __builtin_ctz(block), kb, scale_log2, lens, pages.table,
                       pages.max_pages, __builtin_ctz(pages.page_tokens), pages.n_pages);
  else
    hipLaunchKernelGGL((k_decode_attend_f8<false, kF8Depth>), grid, dim3(256), lds, stream, q, kc, vc, kv_scale, sel,
                       out, ctx, n_q_heads, n_groups, block, __builtin_ctz(block), kb, scale_log2, lens, nullptr, 0,
                       0, 0);
  return hipGetLastError();
}

// Four waves' double-buffered V stages, the entry list and the paged rows (2 x (kb + 1) ints), and the
// merge's (max, sum) pairs.
size_t decode_attend_lds(int kb) { return (size_t)4 * 2 * kDecVStage + (size_t)2 * (kb + 1) * 4 + 4 * 32 * 2 * 4; }

hipError_t launch_decode_attend(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* sel,
                                uint16_t* out, int n_seqs, int ctx, int n_q_heads, int n_groups, int block, int kb,
                                float scale, const int32_t* lens, const PageTable& pages, hipStream_t stream) {
  const size_t lds = decode_attend_lds(kb);
  if (lds > (size_t)max_lds_per_block()) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(n_seqs * n_groups));
  if (pages.table)
    hipLaunchKernelGGL(k_decode_attend<true>, grid, dim3(256), lds, stream, q, kc, vc, sel, out, ctx, n_q_heads,
                       n_groups, block, __builtin_ctz(block), kb, scale_log2, lens, pages.table, pages.max_pages,
                       __builtin_ctz(pages.page_tokens), pages.n_pages);
  else
    hipLaunchKernelGGL(k_decode_attend<false>, grid, dim3(256), lds, stream, q, kc, vc, sel, out, ctx, n_q_heads,
                       n_groups, block, __builtin_ctz(block), kb, scale_log2, lens, nullptr, 0, 0, 0);
  return hipGetLastError();
}

hipError_t prepare_attend_kernels(int lds_max) {
  const void* fns[] = {(const void*)k_attend<kPrefillWaves, kPrefillQT, 0>,
                       (const void*)k_attend<kPrefillWaves, kPrefillQT, 1>,
                       (const void*)k_attend<kPrefillWaves, kPrefillQT, 2>,
                       (const void*)k_attend<kPrefillWaves, kPrefillQT, 4>,
                       (const void*)k_decode_attend<true>,
                       (const void*)k_decode_attend<false>,
                       (const void*)k_decode_attend_f8<true, kF8Depth>,
                       (const void*)k_decode_attend_f8<false, kF8Depth>};
  for (const void* fn : fns) {
    const hipError_t e = allow_full_lds(fn, lds_max);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sgqa
