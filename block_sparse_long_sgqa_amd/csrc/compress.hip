// compress.hip -- block compression of the shared index keys.
//
// "Inside Step 5 Preview", section Sparse GQA, paragraph "Reducing indexer's cost" and Figure 3:
// the index keys of B adjacent positions are merged into one block key. Here the merge is the
// mean, rounded once to bf16: kbar[s][b][d] = bf16_rne((sum_{j<B} ki[s][b*B+j][d]) * (1/B)),
// summed in fp64 in ascending j (1/B is a power of two, so the scaling is exact). The fp64 sum of
// up to 64 bf16 values is exact unless their exponents span more than ~40 binades, so the block
// key is the exact mean rounded once.
//
// HBM-bound: every thread owns 8 consecutive dims (16 B) of one block and streams the B rows of
// that block; 8 lanes cover one 128-byte row, so each wave reads 8 blocks' rows with full 128-byte
// segments and writes 8 whole 128-byte block keys.
#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

template <int BLOCK>
__global__ __launch_bounds__(256) void k_compress(const uint16_t* __restrict__ ki, uint16_t* __restrict__ kbar,
                                                  int n_tokens, int n_blocks, int idx_dim, int dyn_block,
                                                  long long n_items) {
  const int block = BLOCK > 0 ? BLOCK : dyn_block;
  const int chunks = idx_dim >> 3;  // 16-byte pieces per row
  const double inv = 1.0 / (double)block;
  for (long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x; item < n_items;
       item += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(item % chunks);
    const long long sb = item / chunks;  // s * n_blocks + b
    const long long s = sb / n_blocks;
    const long long b = sb - s * n_blocks;
    const uint16_t* src = ki + ((s * n_tokens + b * block) * idx_dim + c * 8);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    if (BLOCK > 0) {
      u32x4 rows[BLOCK > 0 ? BLOCK : 1];
#pragma unroll
      for (int j = 0; j < BLOCK; ++j) rows[j] = *reinterpret_cast<const u32x4*>(src + (long long)j * idx_dim);
#pragma unroll
      for (int j = 0; j < BLOCK; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)bf16_bits_to_f32(rows[j][e] & 0xFFFFu);
          acc[2 * e + 1] += (double)bf16_bits_to_f32(rows[j][e] >> 16);
        }
      }
    } else {
      for (int j = 0; j < block; ++j) {
        u32x4 r = *reinterpret_cast<const u32x4*>(src + (long long)j * idx_dim);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)bf16_bits_to_f32(r[e] & 0xFFFFu);
          acc[2 * e + 1] += (double)bf16_bits_to_f32(r[e] >> 16);
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = f64_to_bf16_bits(acc[2 * e] * inv) | (f64_to_bf16_bits(acc[2 * e + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(kbar + (sb * idx_dim + c * 8)) = o;
  }
}

hipError_t launch_compress(const uint16_t* ki, uint16_t* kbar, int n_seqs, int n_tokens, int idx_dim, int block,
                           hipStream_t stream) {
  const int n_blocks = n_tokens / block;
  const long long n_items = (long long)n_seqs * n_blocks * (idx_dim / 8);
  if (n_items == 0) return hipSuccess;
  const int threads = 256;
  long long grid = (n_items + threads - 1) / threads;
  if (grid > 1 << 20) grid = 1 << 20;
#define SGQA_COMPRESS_CASE(BV)                                                                             \
  case BV:                                                                                                 \
    hipLaunchKernelGGL(k_compress<BV>, dim3((unsigned)grid), dim3(threads), 0, stream, ki, kbar, n_tokens, \
                       n_blocks, idx_dim, block, n_items);                                                 \
    break;
  switch (block) {
    SGQA_COMPRESS_CASE(1)
    SGQA_COMPRESS_CASE(2)
    SGQA_COMPRESS_CASE(4)
    SGQA_COMPRESS_CASE(8)
    SGQA_COMPRESS_CASE(16)
    default:
      hipLaunchKernelGGL(k_compress<0>, dim3((unsigned)grid), dim3(threads), 0, stream, ki, kbar, n_tokens, n_blocks,
                         idx_dim, block, n_items);
  }
#undef SGQA_COMPRESS_CASE
  return hipGetLastError();
}

// Incremental decode: append the token at position j = pos[s] of every sequence s (one workgroup per
// sequence). K/V rows go to the dense cache [S][G][cap][D] or to the pool page table[s][j / page]
// ([n_pages][G][page][D]; a page entry outside [0, n_pages) skips the K/V write); the index key goes to
// idx_cache [S][cap][d_I]; when j closes a block (j % B == B - 1) the block key of block j / B is
// formed with the arithmetic of k_compress (fp64 sum of the B keys in ascending position, times
// 1/B, one rounding to bf16), the new key taken from registers rather than re-read.
__global__ __launch_bounds__(256) void k_append(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                                const uint16_t* __restrict__ idx_new, const int32_t* __restrict__ pos,
                                                uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                                                const int32_t* __restrict__ table, int max_pages, int page_shift,
                                                int n_pages, uint16_t* __restrict__ idx_cache,
                                                uint16_t* __restrict__ kbar, int cap, int n_groups, int idx_dim,
                                                int block) {
  constexpr int kD = 128;
  const int s = blockIdx.x;
  const int j = pos[s];
  if (j < 0 || j >= cap) return;
  const int t = threadIdx.x;
  long long pg = -1;
  if (table) {
    pg = table[(long long)s * max_pages + (j >> page_shift)];
    if (pg >= n_pages) pg = -1;
  }
  const bool write_kv = !table || pg >= 0;
  if (write_kv) {
    for (int x = t; x < n_groups * (kD / 8); x += blockDim.x) {
      const int g = x / (kD / 8), pc = x % (kD / 8);
      const long long row = table ? (((pg * n_groups + g) << page_shift) + (j & ((1 << page_shift) - 1)))
                                  : (((long long)s * n_groups + g) * cap + j);
      const long long src = ((long long)s * n_groups + g) * kD + pc * 8;
      *reinterpret_cast<u32x4*>(kc + row * kD + pc * 8) = *reinterpret_cast<const u32x4*>(k_new + src);
      *reinterpret_cast<u32x4*>(vc + row * kD + pc * 8) = *reinterpret_cast<const u32x4*>(v_new + src);
    }
  }
  const int chunks = idx_dim / 8;
  if (t < chunks) {
    const u32x4 nv = *reinterpret_cast<const u32x4*>(idx_new + (long long)s * idx_dim + t * 8);
    *reinterpret_cast<u32x4*>(idx_cache + ((long long)s * cap + j) * idx_dim + t * 8) = nv;
    if (j % block == block - 1) {
      double acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0;
      for (int r = j - block + 1; r < j; ++r) {
        const u32x4 rv = *reinterpret_cast<const u32x4*>(idx_cache + ((long long)s * cap + r) * idx_dim + t * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)bf16_bits_to_f32(rv[e] & 0xFFFFu);
          acc[2 * e + 1] += (double)bf16_bits_to_f32(rv[e] >> 16);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_bits_to_f32(nv[e] & 0xFFFFu);
        acc[2 * e + 1] += (double)bf16_bits_to_f32(nv[e] >> 16);
      }
      const double inv = 1.0 / (double)block;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = f64_to_bf16_bits(acc[2 * e] * inv) | (f64_to_bf16_bits(acc[2 * e + 1] * inv) << 16);
      const long long nb = cap / block;
      *reinterpret_cast<u32x4*>(kbar + ((long long)s * nb + j / block) * idx_dim + t * 8) = o;
    }
  }
}

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, const uint16_t* idx_new, const int32_t* pos,
                         uint16_t* kc, uint16_t* vc, const PageTable& pages, uint16_t* idx_cache, uint16_t* kbar,
                         int n_seqs, int cap, int n_groups, int idx_dim, int block, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  const int page_shift = pages.table ? __builtin_ctz(pages.page_tokens) : 0;
  hipLaunchKernelGGL(k_append, dim3((unsigned)n_seqs), dim3(256), 0, stream, k_new, v_new, idx_new, pos, kc, vc,
                     pages.table, pages.max_pages, page_shift, pages.n_pages, idx_cache, kbar, cap, n_groups, idx_dim,
                     block);
  return hipGetLastError();
}

}  // namespace sgqa
