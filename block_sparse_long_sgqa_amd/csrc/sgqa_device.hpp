// sgqa_device.hpp -- device-side building blocks shared by the gfx950 kernels of libsgqa.
//
// Only the HIP library includes this file. It fixes the register layouts of the two bf16 matrix
// instructions used here (CDNA4 v_mfma_f32_16x16x32_bf16 and v_mfma_f32_32x32x16_bf16, wave64):
//
//   16x16x32: A operand lane l holds row (l % 16), 8 consecutive k starting at 8 * (l / 16);
//             B operand lane l holds column (l % 16), the same 8 k;
//             result lane l holds column (l % 16), rows 4 * (l / 16) + 0..3.
//   32x32x16: A operand lane l holds row (l % 32), 8 consecutive k starting at 8 * (l / 32);
//             B operand lane l holds column (l % 32), the same 8 k;
//             result register j of lane l holds column (l % 32), row 8 * (j / 4) + 4 * (l / 32) + j % 4.
//
// Only the row/column placement matters for correctness: A and B always use the same k order, so
// any consistent permutation of k inside a step gives the same contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (lowered to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// fp64 -> bf16 bits, rounded once to nearest even, from the bit pattern of x: the 52-bit fraction
// is cut to 7 bits with round-half-even on the 45 dropped bits (a carry moves into the exponent);
// values below the smallest normal bf16 (2^-126) are multiples of 2^-133, rounded as the integer
// rint(|x| * 2^133), whose bits are the subnormal encoding (128 gives the smallest normal). Results
// past the largest finite bf16 become infinity; NaN gives the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  const int dexp = (int)(a >> 52);
  if (dexp == 0x7FF) return (a << 12) != 0 ? 0x7FC0u : (sign | 0x7F80u);
  if (dexp < 1023 - 126) {  // below 2^-126 (zero and double subnormals included)
    const double n = rint(ldexp(__longlong_as_double((long long)a), 133));
    return sign | (uint32_t)n;
  }
  uint64_t q = a >> 45;  // sign-free exponent and the top 7 fraction bits
  const uint64_t rem = a & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rem > half || (rem == half && (q & 1u))) ++q;
  const int fexp = (int)(q >> 7) - 1023 + 127;
  if (fexp >= 255) return sign | 0x7F80u;
  return sign | ((uint32_t)fexp << 7) | (uint32_t)(q & 0x7Fu);
}

// Order-preserving unsigned key of an fp32 score: a larger score gives a larger key; -0 and +0 map
// to the same key. (Non-negative floats get the top bit set; negative floats are bit-inverted.)
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

template <typename T>
__device__ __forceinline__ T readlane(T v, int l) {
  return __shfl(v, l, 64);
}

// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts; rows are lanes 16q..16q+15;
// lanes shifted in from outside the row contribute 0).
__device__ __forceinline__ uint32_t row16_prefix(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  return v;
}

// Inclusive prefix sum across the 64 lanes: the row prefix sums plus the totals of the rows
// before (three lane reads) -- no LDS permutes.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  const uint32_t incl = row16_prefix(v);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)incl, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)incl, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)incl, 47);
  const int q = lane_id() >> 4;
  return incl + (q > 0 ? r0 : 0u) + (q > 1 ? r1 : 0u) + (q > 2 ? r2 : 0u);
}

// Inclusive suffix sum across the 64 lanes: lane l gets sum_{l' >= l} v[l'].
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const uint32_t incl = wave_prefix_sum(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl + v;
}

// Wave-wide sum / maximum of a per-lane value, in every lane: a DPP reduction inside each 16-lane
// row and four lane reads.
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  const uint32_t incl = row16_prefix(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 15) + (uint32_t)__builtin_amdgcn_readlane((int)incl, 31) +
         (uint32_t)__builtin_amdgcn_readlane((int)incl, 47) + (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}

// max(x of lane l, x of lane l ^ 32) in every lane, through one v_permlane32_swap (a register swap
// of the two wave halves) instead of an LDS permute.
__device__ __forceinline__ float max_of_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------- k-th largest key of a wave's list

// Number of listed keys at or above t (lane l holds entries j * 64 + l), the same in every lane:
// ballot counts, no LDS.
constexpr int kMaskGroup = 8;  // ballot masks held at once (2 SGPRs each)

template <int P>
__device__ __forceinline__ int count_ge(const uint32_t (&k)[P], uint32_t t) {
  int c = 0;
#pragma unroll
  for (int j0 = 0; j0 < P; j0 += kMaskGroup) {
    // A group of comparisons first, each into its own mask, so that they issue back to back.
    uint64_t m[kMaskGroup];
#pragma unroll
    for (int j = 0; j < kMaskGroup; ++j) m[j] = j0 + j < P ? ballot(k[j0 + j] >= t) : 0ull;
#pragma unroll
    for (int j = 0; j < kMaskGroup; ++j) c += popc64(m[j]);
  }
  return c;
}

// The K-th largest listed key (lane l holds entries j * 64 + l; absent ones are 0): the largest t
// with count(>= t) >= K (1 <= K <= keys present); *n_above gets count(> t).
// With cap >= K the search may stop early at a value t with K <= count(>= t) <= cap (then t is a
// bound at or below the K-th largest key, not the key itself); *n_at gets count(>= t) of the
// returned t when it is known to be at most cap, else a value above cap.
// Search over key values: it keeps lo < hi with count(>= lo) >= K > count(>= hi) and probes a
// value between them, alternately where the count, interpolated linearly between the bounds,
// reaches the target (K, or the middle of [K, cap]) and the midpoint, so it ends within 64 probes
// (typically a handful). When count(>= lo) is exactly K, the answer is the smallest key at or
// above lo.
template <int P>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&k)[P], int K, int* n_above, int cap = 0,
                                                int* n_at = nullptr) {
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    mn = min(mn, k[j] ? k[j] : 0xFFFFFFFFu);
    mx = max(mx, k[j]);
  }
  mn = wave_min_dpp(mn);
  mx = wave_max_dpp(mx);
  // Invariant: lo <= hm, count(>= lo) = c_lo >= K > count(>= hm + 1) = c_hi (keys are nonzero, so
  // lo >= 1 and every span below fits 32 bits).
  uint32_t lo = mn, hm = mx;
  int c_lo = count_ge(k, lo), c_hi = 0;
  const int target = cap >= K ? (K + cap) / 2 : K;
  for (int step = 0;; ++step) {
    if (c_lo <= cap) break;  // a bound: K <= count(>= lo) <= cap
    if (c_lo == K) {         // the K entries at or above lo: the K-th largest is the smallest of them
      uint32_t m = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < P; ++j) m = k[j] >= lo ? min(m, k[j]) : m;
      lo = wave_min_dpp(m);
      c_hi = lo == 0xFFFFFFFFu ? 0 : count_ge(k, lo + 1u);
      break;
    }
    if (hm <= lo) break;  // count(>= lo) >= K > count(>= lo + 1) = c_hi: lo is the K-th key
    const uint32_t span = hm - lo;  // probes lie in [lo + 1, hm]
    uint32_t d;
    if (step & 1) {
      d = span / 2;
    } else {
      const float f = (float)(c_lo - target) * __builtin_amdgcn_rcpf((float)(c_lo - c_hi));
      d = (uint32_t)(f * (float)span);
    }
    d = __builtin_amdgcn_readfirstlane(d);
    const uint32_t t = lo + max(1u, min(d, span));
    const int c = count_ge(k, t);
    if (c >= K) {
      lo = t;
      c_lo = c;
    } else {
      hm = t - 1u;
      c_hi = c;
    }
  }
  *n_above = c_hi;
  if (n_at) *n_at = c_lo;
  return lo;
}

}  // namespace sgqa
