// union.hip -- union of the selections of adjacent prefill queries.
//
// "Inside Step 5 Preview", section Sparse GQA, paragraph "Efficient implementation of sparse
// attention": during prefill the top-k results of neighbouring tokens are merged so that their
// largely overlapping K/V reads are done once for the group. Here the group is an aligned tile of
// Tq queries, per KV group g:
//   U(t,g) = union over i in tile t of Sel(i,g) and the own block floor(i/B)
// stored as a bitmask over ceil(N/B) blocks (bit b%32 of word b/32) plus its popcount.
//
// One workgroup per (g, t). The tile's selections are one contiguous [Tq][K_B] slab of the topk
// array, read with 16-byte loads; each thread folds the ids of one load that fall into the same
// 32-block word together and ORs them into the LDS bitmask. The mask and its popcount are then
// written once. HBM-bound (the slab is read exactly once).
#include "sgqa_device.hpp"
#include "sgqa_internal.hpp"

namespace sgqa {

__global__ __launch_bounds__(256) void k_union(const int32_t* __restrict__ topk, uint32_t* __restrict__ umask,
                                               int32_t* __restrict__ ucount, int n_tokens, int n_tiles, int block,
                                               int kb, int tile, int n_words, int vec4, int nbc) {
  extern __shared__ __align__(16) uint32_t mask[];
  __shared__ uint32_t wave_sums[4];
  const int t = blockIdx.x % n_tiles;
  const int g = blockIdx.x / n_tiles;
  for (int x = threadIdx.x; x < n_words; x += blockDim.x) mask[x] = 0u;
  __syncthreads();

  const int i0 = t * tile;
  const int i1 = (i0 + tile < n_tokens) ? i0 + tile : n_tokens;
  const long long base = ((long long)g * n_tokens + i0) * kb;
  const long long count = (long long)(i1 - i0) * kb;

  uint32_t cur_word = 0xFFFFFFFFu, cur_bits = 0u;
  auto add = [&](int b) {
    if (b < 0 || b >= nbc) return;  // -1 padding; ids outside the mask are ignored
    const uint32_t wd = (uint32_t)b >> 5;
    if (wd != cur_word) {
      if (cur_bits) atomicOr(&mask[cur_word], cur_bits);
      cur_word = wd;
      cur_bits = 0u;
    }
    cur_bits |= 1u << (b & 31);
  };
  if (vec4) {
    const int4* src = reinterpret_cast<const int4*>(topk + base);
    const long long n4 = count >> 2;
    for (long long x = threadIdx.x; x < n4; x += blockDim.x) {
      const int4 v = src[x];
      add(v.x);
      add(v.y);
      add(v.z);
      add(v.w);
    }
  } else {
    for (long long x = threadIdx.x; x < count; x += blockDim.x) add(topk[base + x]);
  }
  if (cur_bits) atomicOr(&mask[cur_word], cur_bits);
  // The own block of every query of the tile is always attended.
  for (int i = i0 + (int)threadIdx.x; i < i1; i += blockDim.x) {
    const int b = i / block;
    atomicOr(&mask[b >> 5], 1u << (b & 31));
  }
  __syncthreads();

  uint32_t* dst = umask + ((long long)g * n_tiles + t) * n_words;
  uint32_t pc = 0;
  for (int x = threadIdx.x; x < n_words; x += blockDim.x) {
    const uint32_t m = mask[x];
    dst[x] = m;
    pc += __popc(m);
  }
  for (int off = 32; off >= 1; off >>= 1) pc += __shfl_xor(pc, off, 64);
  if (lane_id() == 0) wave_sums[threadIdx.x >> 6] = pc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t total = 0;
    for (int x = 0; x < (int)(blockDim.x >> 6); ++x) total += wave_sums[x];
    ucount[(long long)g * n_tiles + t] = (int32_t)total;
  }
}

hipError_t prepare_union_kernels(int lds_max) { return allow_full_lds((const void*)k_union, lds_max); }

hipError_t launch_union(const int32_t* topk, uint32_t* umask, int32_t* ucount, int n_tokens, int n_groups, int block,
                        int kb, int tile, hipStream_t stream) {
  const int n_tiles = (n_tokens + tile - 1) / tile;
  const int nbc = (n_tokens + block - 1) / block;
  const int n_words = (nbc + 31) / 32;
  const long long grid = (long long)n_tiles * n_groups;
  if (grid == 0) return hipSuccess;
  const size_t lds = (size_t)n_words * 4;
  const int vec4 = (kb % 4 == 0) ? 1 : 0;
  hipLaunchKernelGGL(k_union, dim3((unsigned)grid), dim3(256), lds, stream, topk, umask, ucount, n_tokens, n_tiles,
                     block, kb, tile, n_words, vec4, nbc);
  return hipGetLastError();
}

// Zero n words (a kernel rather than a memset node, so that the fused path can be captured in a
// graph).
__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ dst, long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += stride) dst[x] = 0u;
}

hipError_t launch_fill_zero(uint32_t* dst, long long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)grid), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

// ucount[r] = popcount of mask row r (n_words words); one workgroup per row.
__global__ __launch_bounds__(256) void k_mask_count(const uint32_t* __restrict__ umask, int32_t* __restrict__ ucount,
                                                    int n_words) {
  __shared__ uint32_t wave_sums[4];
  const uint32_t* src = umask + (long long)blockIdx.x * n_words;
  uint32_t pc = 0;
  for (int x = threadIdx.x; x < n_words; x += blockDim.x) pc += __popc(src[x]);
  for (int off = 32; off >= 1; off >>= 1) pc += __shfl_xor(pc, off, 64);
  if (lane_id() == 0) wave_sums[threadIdx.x >> 6] = pc;
  __syncthreads();
  if (threadIdx.x == 0) ucount[blockIdx.x] = (int32_t)(wave_sums[0] + wave_sums[1] + wave_sums[2] + wave_sums[3]);
}

hipError_t launch_mask_count(const uint32_t* umask, int32_t* ucount, long long n_rows, int n_words,
                             hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mask_count, dim3((unsigned)n_rows), dim3(256), 0, stream, umask, ucount, n_words);
  return hipGetLastError();
}

// Per-query selection bitmaps for the masked-union attention: selbits [G][N][W], bit b % 32 of
// word b / 32 of row (g, i) set iff b is in Sel(i,g) (the own block is not included). One wave per
// row; the row is assembled in LDS in windows of 512 words and written with coalesced stores.
__global__ __launch_bounds__(256) void k_sel_bitmap(const int32_t* __restrict__ topk, uint32_t* __restrict__ selbits,
                                                    long long n_rows, int kb, int n_words) {
  constexpr int kWin = 512;
  __shared__ uint32_t win[4][kWin];
  const int wave = threadIdx.x >> 6, l = lane_id();
  const long long row = (long long)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // wave-uniform; no barrier below
  const int32_t* sel = topk + row * kb;
  uint32_t* dst = selbits + row * n_words;
  uint32_t* w = win[wave];
  for (int w0 = 0; w0 < n_words; w0 += kWin) {
    for (int x = l; x < kWin; x += 64) w[x] = 0u;
    for (int e = l; e < kb; e += 64) {
      const int b = sel[e];
      const int wd = (b >> 5) - w0;
      if (b >= 0 && wd >= 0 && wd < kWin) atomicOr(&w[wd], 1u << (b & 31));
    }
    const int n = n_words - w0 < kWin ? n_words - w0 : kWin;
    for (int x = l; x < n; x += 64) dst[w0 + x] = w[x];
  }
}

hipError_t launch_sel_bitmap(const int32_t* topk, uint32_t* selbits, int n_tokens, int n_groups, int block, int kb,
                             hipStream_t stream) {
  const long long n_rows = (long long)n_tokens * n_groups;
  if (n_rows == 0) return hipSuccess;
  const int n_words = ((n_tokens + block - 1) / block + 31) / 32;
  hipLaunchKernelGGL(k_sel_bitmap, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream, topk, selbits, n_rows,
                     kb, n_words);
  return hipGetLastError();
}

}  // namespace sgqa
