// attn_common.hpp -- device helpers shared by the forward and backward gathered-block attention
// kernels: tile geometry, the MFMA chunk of the online-softmax forward, LDS layouts and gathers.
// Everything lives in an unnamed namespace: each translation unit gets its own copy.
#pragma once

#include <type_traits>

#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"


namespace sgqa {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;
constexpr int kKeys = 64;                          // keys per chunk
constexpr int kKRowBytes = 272;                    // K row: 256 B + 16 B pad (bank spread for 16-B reads)
constexpr int kKSlotsPerRow = kKRowBytes / 16;     // 17 slots of 16 B, the last one is padding
constexpr int kKTileBytes = kKeys * kKRowBytes;    // 17408 B
constexpr int kKTileInsts = kKeys * kKSlotsPerRow / 64;  // 17 wave-wide 16-byte loads fill the K tile
constexpr int kVTileBytes = kKeys * 256;           // V rows unpadded; 16-B pieces XOR-swizzled by row
constexpr int kVTileInsts = kVTileBytes / 1024;    // 16
constexpr int kSelTableWords = 64;                 // masked variant: membership words of a chunk
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kKReadsAhead = 3;   // K-operand steps read ahead of the score products
constexpr int kVReadsAhead = 4;   // V-operand steps read ahead of the value products
constexpr float kLazyLog2 = 8.0f;  // the running maximum moves only when a row's grows by more
constexpr float kMinit = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int QT>
struct AttnState {
  f32x16 o[QT][4];  // O^T tiles: [d-tile][32 d x 32 rows], column = this lane's row
  float m[QT];      // running max (log2 domain), identical in lanes l and l^32
  float l[QT];      // this lane's part of the running denominator (lanes l and l^32 hold halves)
};

template <int QT>
__device__ __forceinline__ void state_init(AttnState<QT>& st) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[qt][dt][j] = 0.0f;
    st.m[qt] = kMinit;
    st.l[qt] = 0.0f;
  }
}

// Physical 16-byte piece of logical piece p in V row `row`: XOR with 4 * (row % 4). A transposing
// read phase (32 lanes) touches 4 consecutive rows x 4 consecutive pieces; the swizzle spreads them
// over all 16 piece positions, i.e. all 64 banks once.
__device__ __forceinline__ int v_phys(int row, int p) { return p ^ ((row & 3) << 2); }

// Per-lane LDS byte offsets inside a stage (constant over the chunks).
struct LaneOffsets {
  int k;     // K A-operand: key row (l % 32), 16-byte piece (l / 32); + kt * 32 rows + ks * 32 B
  int v[4];  // V transposing read for d-tile dt: row 4 * khalf + (s16 / 4), d 32 dt + 16 dgrp + 4 (s16 % 4)
  int tok;   // the chunk's token table
};

// v_tile: byte offset of the V tile inside a stage (the token table follows it).
__device__ __forceinline__ LaneOffsets lane_offsets(int v_tile = kKTileBytes) {
  const int l = lane_id();
  LaneOffsets o;
  o.k = (l & 31) * kKRowBytes + (l >> 5) * 16;
  const int grp = l >> 4, s16 = l & 15;
  const int row = 4 * (grp >> 1) + (s16 >> 2);  // + 16 ss + 8 r (multiples of 4: same swizzle)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int piece = 4 * dt + 2 * (grp & 1) + ((s16 & 3) >> 1);
    o.v[dt] = v_tile + row * 256 + 16 * v_phys(row, piece) + 8 * (s16 & 1);
  }
  o.tok = v_tile + kVTileBytes;
  return o;
}

struct NoOp {
  __device__ void operator()() const {}
};
struct NoHook {
  __device__ void operator()(int) const {}
};

// S^T = K Q^T for the 64 keys of a K tile (ktile + lo.k is this lane's first operand): the K
// operands of step ks+2 are read while the MFMAs of step ks run.
// hook(ks) runs after the products of step ks (other work to spread between them).
template <int QT, typename Hook = NoHook, int PF = kKReadsAhead>
__device__ __forceinline__ void score_products(const uint8_t* ktile, const LaneOffsets& lo,
                                               const bf16x8 (&qreg)[QT][8], f32x16 (&s)[QT][2],
                                               Hook hook = Hook()) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[qt][kt][j] = 0.0f;
  const uint8_t* kp = ktile + lo.k;
  bf16x8 ka[PF + 1][2];
#pragma unroll
  for (int ks = 0; ks < PF; ++ks) {
    ka[ks][0] = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
    ka[ks][1] = *reinterpret_cast<const bf16x8*>(kp + 32 * kKRowBytes + ks * 32);
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks + PF < 8) {
      ka[(ks + PF) % (PF + 1)][0] = *reinterpret_cast<const bf16x8*>(kp + (ks + PF) * 32);
      ka[(ks + PF) % (PF + 1)][1] = *reinterpret_cast<const bf16x8*>(kp + 32 * kKRowBytes + (ks + PF) * 32);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma32(ka[ks % (PF + 1)][kt], qreg[qt][ks], s[qt][kt]);
    __builtin_amdgcn_sched_barrier(0);
    hook(ks);
  }
}

// Online softmax of one chunk's scores s (S^T tiles: lane column = Q row, 32 keys per tile) into
// the bf16 probabilities pb (the B operands of the V products); rescales the running state.
//   tok: the chunk's token table (INT_MAX = invalid key); row_pos[qt]: query position of this
//        lane's Q row in tile qt (for the causal mask)
//   MASK: 0 = no key of the chunk can be masked, 1 = apply the mask, 2 = decided by masked_rt.
//   SEL (with MASK = 1): a key also needs its block to be a member of the Q row's own set: the
//        word mt[e * nqw + ql / 32] of the chunk's membership table holds, for block entry
//        e = key >> bs of the chunk, one bit per query of the workgroup; ql[qt] is this lane's
//        query index within the workgroup.
// The running maximum only moves when some row's maximum grows by more than kLazyLog2 (log2
// units): most chunks then skip the rescale of O. The probabilities stay below 2^kLazyLog2, which
// fp32 sums and bf16 operands carry with the same relative precision as values below 1, and the
// final normalisation uses the same maximum, so the result is unchanged up to rounding.
template <int QT, int MASK = 2, bool SEL = false>
__device__ __forceinline__ void chunk_softmax(f32x16 (&s)[QT][2], const int* tok, AttnState<QT>& st,
                                              float scale_log2, bool masked_rt, const int (&row_pos)[QT],
                                              bf16x8 (&pb)[QT][4], const uint32_t* mt = nullptr, int nqw = 0,
                                              const int* ql = nullptr, int bs = 0) {
  const bool masked = MASK == 2 ? masked_rt : MASK == 1;
  const int hi = lane_id() >> 5;

  // Tokens of this lane's keys: key kt*32 + 8*a + 4*hi + (0..3), four consecutive ints.
  int4 tk[2][4];
  if (masked) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int a = 0; a < 4; ++a) tk[kt][a] = *reinterpret_cast<const int4*>(tok + kt * 32 + 8 * a + 4 * hi);
  }

  // SEL: keys outside the row's set get the invalid token, so the causal test masks them too.
  if constexpr (SEL) {
    static_assert(QT == 1, "the membership folds into the token table of the single Q tile");
    const uint32_t* col = mt + (ql[0] >> 5);
    const int sh = ql[0] & 31;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int key = kt * 32 + 8 * a + 4 * hi;
        int4& t4 = tk[kt][a];
        if (bs >= 2) {  // the four keys share one block
          if (!((col[(key >> bs) * nqw] >> sh) & 1u)) t4 = make_int4(0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF);
        } else {
          if (!((col[(key >> bs) * nqw] >> sh) & 1u)) t4.x = 0x7FFFFFFF;
          if (!((col[((key + 1) >> bs) * nqw] >> sh) & 1u)) t4.y = 0x7FFFFFFF;
          if (!((col[((key + 2) >> bs) * nqw] >> sh) & 1u)) t4.z = 0x7FFFFFFF;
          if (!((col[((key + 3) >> bs) * nqw] >> sh) & 1u)) t4.w = 0x7FFFFFFF;
        }
      }
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = s[qt][kt][j];
        if (masked) {
          const int4 t4 = tk[kt][j >> 2];
          const int t = (j & 3) == 0 ? t4.x : (j & 3) == 1 ? t4.y : (j & 3) == 2 ? t4.z : t4.w;
          if (t > row_pos[qt]) x = kNegInf;
        }
        s[qt][kt][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_of_halves(mx);
    const float m_new = fmaxf(st.m[qt], mx * scale_log2);
    if (ballot(m_new > st.m[qt] + kLazyLog2)) {
      const float alpha = fast_exp2(st.m[qt] - m_new);
      st.l[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) st.o[qt][dt][j] *= alpha;
      st.m[qt] = m_new;
    }
    const float m_use = st.m[qt];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[qt][kt][j] = fast_exp2(__builtin_fmaf(s[qt][kt][j], scale_log2, -m_use));
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[qt][ss][e] = (__bf16)s[qt][ss >> 1][8 * (ss & 1) + e];
    float sum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += s[qt][kt][j];
    st.l[qt] += sum;
  }
}

// O^T += V^T P^T. The V^T operand of lane l (row d, 8 keys) comes from two transposing reads, each
// returning 4 keys of this lane's d, in the key order the score registers already have; vbase +
// lo.v[dt] addresses this lane's first read of d-tile dt.
template <int QT, int PF = kVReadsAhead>
__device__ __forceinline__ void pv_products(const uint8_t* vbase, const LaneOffsets& lo, const bf16x8 (&pb)[QT][4],
                                            AttnState<QT>& st) {
  auto vread = [&](int step) -> bf16x8 {
    const int dt = step >> 2, ss = step & 3;
    const uint8_t* a0 = vbase + lo.v[dt] + (16 * ss) * 256;
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * 256));
    const i16x8 cat = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, cat);
  };
  bf16x8 va[PF + 1];
#pragma unroll
  for (int step = 0; step < PF; ++step) va[step] = vread(step);
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    if (step + PF < 16) va[(step + PF) % (PF + 1)] = vread(step + PF);
    const int dt = step >> 2, ss = step & 3;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) st.o[qt][dt] = mfma32(va[step % (PF + 1)], pb[qt][ss], st.o[qt][dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 64-key chunk for the QT Q tiles of this wave, all phases in order.
//   stage: K tile, V tile, token table at the offsets of lo
//   KREG: the K operands come from kreg[ks * 2 + kt] (registers) instead of the K tile; after()
//         runs once the score products have consumed them.
//   MASK, SEL and the membership arguments: as for chunk_softmax.
template <int QT, int MASK = 2, bool KREG = false, typename After = NoOp, bool SEL = false>
__device__ __forceinline__ void attn_chunk(const uint8_t* stage, const LaneOffsets& lo, const bf16x8 (&qreg)[QT][8],
                                           AttnState<QT>& st, float scale_log2, bool masked_rt,
                                           const int (&row_pos)[QT], const bf16x8* kreg = nullptr,
                                           After after = After(), const uint32_t* mt = nullptr, int nqw = 0,
                                           const int* ql = nullptr, int bs = 0) {
  f32x16 s[QT][2];
  if constexpr (KREG) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[qt][kt][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma32(kreg[ks * 2 + kt], qreg[qt][ks], s[qt][kt]);
  } else {
    score_products<QT>(stage, lo, qreg, s);
  }
  after();
  const int* tok = reinterpret_cast<const int*>(stage + (KREG ? lo.tok : kKTileBytes + kVTileBytes));
  bf16x8 pb[QT][4];
  chunk_softmax<QT, MASK, SEL>(s, tok, st, scale_log2, masked_rt, row_pos, pb, mt, nqw, ql, bs);
  pv_products<QT>(stage, lo, pb, st);
}

// Tile gather layout. A chunk's 64 keys are gathered straight from global memory into the K and V
// tiles (global_load_lds: every wave-wide instruction fills 64 consecutive 16-byte slots). K: slot s
// of the tile is row s / 17, piece s % 17 (piece 16 is padding). V: slot s is row s / 16, physical
// piece s % 16, holding logical piece v_phys(row, s % 16). Invalid keys read row 0 of the group
// (finite data, always masked out through the token table).

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Block-wide exclusive scan of one value per thread (NT threads); returns the exclusive prefix and
// writes the total to *total. `scratch` holds NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int l = lane_id(), wave = threadIdx.x >> 6;
  const int incl = (int)wave_prefix_sum((uint32_t)v);
  if (l == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int x = 0; x < NT / 64; ++x) {
    const int s = scratch[x];
    if (x < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// The union U(t,g) restricted to blocks <= c_hi, handed out as ascending lists of absolute block
// ids in segments of at most `cap` entries, so that the LDS list has a fixed size however long the
// sequence is (a tile's union can hold tens of thousands of blocks at a 1M-token context).
// union_list_fill writes the ids of ranks [lo, lo + cap) (rank = position in the whole ascending
// list) to list[0 ..), sets *total to the size of the whole list (wave-uniform) and returns how
// many ids it wrote. Every thread owns consecutive words of the mask row and finds the rank of
// its first set bit with a workgroup scan on each call, so nothing per thread is kept between
// segments. The caller syncs the workgroup before the list is read, and after the last read
// before the next fill.
template <int NT>
__device__ __forceinline__ int union_list_fill(const uint32_t* mrow, int c_hi, uint32_t* list, int lo, int cap,
                                               int* scan, int* total) {
  const int n_w = c_hi / 32 + 1;
  const int per = (n_w + NT - 1) / NT;
  const int w0 = (int)threadIdx.x * per;
  auto word = [&](int wd) __attribute__((always_inline)) -> uint32_t {
    uint32_t m = mrow[wd];
    if (wd == n_w - 1 && (c_hi & 31) != 31) m &= (2u << (c_hi & 31)) - 1u;
    return m;
  };
  int cnt = 0;
  for (int e = 0; e < per; ++e) {
    const int wd = w0 + e;
    if (wd < n_w) cnt += __popc(word(wd));
  }
  int all;
  int rank = block_exclusive_scan<NT>(cnt, scan, &all);
  all = __builtin_amdgcn_readfirstlane(all);
  *total = all;
  const int hi = lo + cap;
  for (int e = 0; e < per && rank < hi; ++e) {
    const int wd = w0 + e;
    if (wd >= n_w) break;
    uint32_t m = word(wd);
    const int c = __popc(m);
    if (rank + c <= lo) {
      rank += c;
      continue;
    }
    while (m && rank < hi) {
      const int b = __ffs(m) - 1;
      m &= m - 1u;
      if (rank >= lo) list[rank - lo] = (uint32_t)(wd * 32 + b);
      ++rank;
    }
  }
  const int left = all - lo;
  return left < cap ? left : cap;
}

}  // namespace

}  // namespace sgqa
