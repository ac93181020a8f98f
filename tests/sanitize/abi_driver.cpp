// abi_driver.cpp -- drives the host side of the C ABI (include/sgqa.h) through its validation
// paths, for a build of the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py). Every entry point is called with parameter sets that it must reject
// before any device work: NULL parameters or tensors, unsupported and extreme sizes (up to
// INT32_MAX, where a size computation in 32-bit arithmetic would overflow), misaligned tensors and
// short workspaces. No call here is valid in full, so none can reach a launch, with or without a
// GPU. sgqa_workspace_size is also asked for every operation over the same parameter sets.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sgqa.h"

namespace {

int failures = 0;

void expect_rejected(int st, const char* what, int line) {
  const bool ok = st == SGQA_ERR_NULL || st == SGQA_ERR_SHAPE || st == SGQA_ERR_ALIGN || st == SGQA_ERR_WORKSPACE ||
                  st == SGQA_ERR_DEVICE || st == SGQA_ERR_SCRATCH;
  if (!ok) {
    std::fprintf(stderr, "line %d: %s returned %d (%s), expected a validation error\n", line, what, st,
                 sgqa_status_string(st));
    ++failures;
  }
}
#define REJECT(call) expect_rejected((call), #call, __LINE__)

sgqa_params base() {
  sgqa_params p;
  std::memset(&p, 0, sizeof(p));
  p.n_tokens = 32768;
  p.n_seqs = 1;
  p.n_q_heads = 64;
  p.n_kv_heads = 8;
  p.head_dim = 128;
  p.idx_heads = 4;
  p.idx_dim = 64;
  p.block = 8;
  p.topk_tokens = 4096;
  p.union_tile = 64;
  p.softmax_scale = 0.0f;
  return p;
}

// Parameter sets: the base with one field changed (valid and invalid values, extremes included).
std::vector<sgqa_params> param_sets() {
  std::vector<sgqa_params> out;
  const int32_t vals[] = {INT32_MIN, -1, 0, 1, 2, 3, 7, 8, 9, 63, 64, 65, 128, 4096, 65536, 1 << 20, 1 << 28,
                          INT32_MAX - 64, INT32_MAX};
  for (int field = 0; field < 10; ++field) {
    for (int32_t v : vals) {
      sgqa_params p = base();
      int32_t* f[] = {&p.n_tokens, &p.n_seqs,  &p.n_q_heads, &p.n_kv_heads,  &p.head_dim,
                      &p.idx_heads, &p.idx_dim, &p.block,     &p.topk_tokens, &p.union_tile};
      *f[field] = v;
      out.push_back(p);
    }
  }
  // Extremes together.
  sgqa_params p = base();
  p.n_tokens = INT32_MAX;
  p.block = 64;
  p.topk_tokens = 64 * 2048;
  p.union_tile = INT32_MAX;
  out.push_back(p);
  p = base();
  p.n_tokens = INT32_MAX;
  p.n_seqs = INT32_MAX;
  out.push_back(p);
  p = base();
  p.n_tokens = 1 << 30;
  p.block = 1;
  p.topk_tokens = 2048;
  p.union_tile = 1;
  out.push_back(p);
  return out;
}

}  // namespace

int main() {
  if (sgqa_abi_version() != SGQA_ABI_VERSION) {
    std::fprintf(stderr, "ABI version mismatch\n");
    return 1;
  }
  for (int s = -3; s < 12; ++s)
    if (!sgqa_status_string(s)) ++failures;

  // Tensors: one aligned host buffer stands for every pointer (never dereferenced by a rejected call).
  alignas(64) static unsigned char buf[256];
  void* a = buf;
  void* mis = buf + 2;
  const size_t huge = (size_t)1 << 40;
  uint16_t* b16 = static_cast<uint16_t*>(a);
  float* f32 = static_cast<float*>(a);
  int32_t* i32 = static_cast<int32_t*>(a);
  uint32_t* u32 = static_cast<uint32_t*>(a);
  uint8_t* u8 = static_cast<uint8_t*>(a);
  sgqa_pages pages = {i32, 4, 64, 8};

  size_t bytes = 0;
  REJECT(sgqa_workspace_size(nullptr, SGQA_OP_PREFILL, &bytes));
  sgqa_params p0 = base();
  REJECT(sgqa_workspace_size(&p0, SGQA_OP_PREFILL, nullptr));
  REJECT(sgqa_workspace_size(&p0, 99, &bytes));
  REJECT(sgqa_workspace_size(&p0, -1, &bytes));

  const std::vector<sgqa_params> sets = param_sets();
  for (const sgqa_params& p : sets) {
    for (int op = 0; op <= SGQA_OP_ATTEND_BWD; ++op) {
      const int st = sgqa_workspace_size(&p, op, &bytes);
      if (st != SGQA_OK && st != SGQA_ERR_SHAPE) {
        std::fprintf(stderr, "workspace_size(op %d) returned %d\n", op, st);
        ++failures;
      }
    }
  }

  // NULL parameters.
  REJECT(sgqa_compress(nullptr, b16, b16, nullptr));
  REJECT(sgqa_index_topk(nullptr, b16, f32, b16, i32, a, huge, nullptr));
  REJECT(sgqa_union(nullptr, i32, u32, i32, nullptr));
  REJECT(sgqa_index_union(nullptr, b16, f32, b16, u32, i32, a, huge, nullptr));
  REJECT(sgqa_attend(nullptr, b16, b16, b16, u32, i32, b16, a, huge, nullptr));
  REJECT(sgqa_prefill(nullptr, b16, b16, b16, b16, f32, b16, b16, a, huge, nullptr));
  REJECT(sgqa_decode(nullptr, b16, b16, b16, b16, b16, f32, i32, b16, a, huge, nullptr));
  REJECT(sgqa_decode_noalloc(nullptr, b16, b16, b16, b16, b16, f32, i32, b16, nullptr));
  REJECT(sgqa_decode_varlen(nullptr, b16, b16, b16, nullptr, b16, b16, f32, i32, i32, b16, a, huge, nullptr));
  REJECT(sgqa_append(nullptr, b16, b16, b16, i32, b16, b16, nullptr, b16, b16, nullptr));
  REJECT(sgqa_decode_fp8(nullptr, b16, u8, u8, f32, nullptr, b16, b16, f32, i32, i32, b16, a, huge, nullptr));
  REJECT(sgqa_attend_fwd(nullptr, b16, b16, b16, u32, i32, b16, f32, a, huge, nullptr));
  REJECT(sgqa_attend_bwd(nullptr, b16, b16, b16, u32, i32, b16, f32, b16, b16, b16, b16, a, huge, nullptr));
  REJECT(sgqa_attend_masked(nullptr, b16, b16, b16, i32, u32, i32, b16, a, huge, nullptr));
  REJECT(sgqa_prefill_masked(nullptr, b16, b16, b16, b16, f32, b16, b16, a, huge, nullptr));

  // Every entry point over every parameter set, each call with one defect besides: a NULL tensor, a
  // misaligned tensor, a short workspace, or (for the unsupported sets) nothing else.
  for (const sgqa_params& p0s : sets) {
    for (int defect = 0; defect < 4; ++defect) {
      const sgqa_params* p = &p0s;
      // defect 0: the parameter set alone (must be unsupported to be rejected: skip supported ones)
      if (defect == 0) {
        size_t w = 0;
        if (sgqa_workspace_size(p, SGQA_OP_PREFILL, &w) == SGQA_OK) continue;
      }
      uint16_t* t = defect == 1 ? nullptr : (defect == 2 ? static_cast<uint16_t*>(mis) : b16);
      void* ws = defect == 3 ? a : a;
      const size_t wsb = defect == 3 ? 16 : huge;
      if (defect == 3) {
        // Only the calls that take a workspace are meaningful here; shapes that need none would
        // pass: run them with a NULL output tensor as well, so that every call stays invalid.
        REJECT(sgqa_index_topk(p, b16, f32, b16, nullptr, ws, wsb, nullptr));
        REJECT(sgqa_index_union(p, b16, f32, b16, u32, nullptr, ws, wsb, nullptr));
        REJECT(sgqa_attend(p, b16, b16, b16, u32, i32, nullptr, ws, wsb, nullptr));
        REJECT(sgqa_prefill(p, b16, b16, b16, b16, f32, b16, b16, ws, wsb, nullptr));
        REJECT(sgqa_decode(p, b16, b16, b16, b16, b16, f32, i32, b16, ws, wsb, nullptr));
        REJECT(sgqa_decode_varlen(p, b16, b16, b16, &pages, b16, b16, f32, i32, i32, b16, ws, wsb, nullptr));
        REJECT(sgqa_decode_fp8(p, b16, u8, u8, f32, &pages, b16, b16, f32, i32, i32, b16, ws, wsb, nullptr));
        REJECT(sgqa_attend_fwd(p, b16, b16, b16, u32, i32, b16, nullptr, ws, wsb, nullptr));
        REJECT(sgqa_attend_bwd(p, b16, b16, b16, u32, i32, b16, f32, b16, b16, b16, b16, ws, wsb, nullptr));
        REJECT(sgqa_attend_masked(p, b16, b16, b16, i32, u32, i32, b16, ws, wsb, nullptr));
        REJECT(sgqa_prefill_masked(p, b16, b16, b16, b16, f32, b16, b16, ws, wsb, nullptr));
        continue;
      }
      REJECT(sgqa_compress(p, t, b16, nullptr));
      REJECT(sgqa_index_topk(p, t, f32, b16, i32, ws, wsb, nullptr));
      REJECT(sgqa_union(p, defect == 0 ? i32 : nullptr, u32, i32, nullptr));
      REJECT(sgqa_index_union(p, t, f32, b16, u32, i32, ws, wsb, nullptr));
      REJECT(sgqa_attend(p, t, b16, b16, u32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_prefill(p, t, b16, b16, b16, f32, b16, b16, ws, wsb, nullptr));
      REJECT(sgqa_decode(p, t, b16, b16, b16, b16, f32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_decode_noalloc(p, t, b16, b16, b16, b16, f32, i32, b16, nullptr));
      REJECT(sgqa_decode_varlen(p, t, b16, b16, &pages, b16, b16, f32, i32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_decode_varlen(p, t, b16, b16, nullptr, b16, b16, f32, i32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_append(p, t, b16, b16, i32, b16, b16, &pages, b16, b16, nullptr));
      REJECT(sgqa_append(p, t, b16, b16, i32, b16, b16, nullptr, b16, b16, nullptr));
      REJECT(sgqa_decode_fp8(p, t, u8, u8, f32, &pages, b16, b16, f32, i32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_attend_fwd(p, t, b16, b16, u32, i32, b16, f32, ws, wsb, nullptr));
      REJECT(sgqa_attend_bwd(p, t, b16, b16, u32, i32, b16, f32, b16, b16, b16, b16, ws, wsb, nullptr));
      REJECT(sgqa_attend_masked(p, t, b16, b16, i32, u32, i32, b16, ws, wsb, nullptr));
      REJECT(sgqa_prefill_masked(p, t, b16, b16, b16, f32, b16, b16, ws, wsb, nullptr));
    }
  }
  // Page tables that do not fit the cache (checked on the host).
  sgqa_params d = base();
  d.n_tokens = 4096;
  d.n_seqs = 2;
  d.union_tile = 1;
  const sgqa_pages bad_pages[] = {{i32, 4, 48, 8}, {i32, 4, 4, 8}, {i32, 1, 64, 8}, {i32, 64, 64, 0},
                                  {nullptr, 64, 64, 8}, {i32, -1, 64, 8}, {i32, INT32_MAX, 64, INT32_MAX}};
  for (const sgqa_pages& pg : bad_pages) {
    REJECT(sgqa_decode_varlen(&d, b16, b16, b16, &pg, b16, b16, f32, i32, i32, b16, a, huge, nullptr));
    REJECT(sgqa_append(&d, b16, b16, b16, i32, b16, b16, &pg, b16, b16, nullptr));
    REJECT(sgqa_decode_fp8(&d, b16, u8, u8, f32, &pg, b16, b16, f32, i32, i32, b16, a, huge, nullptr));
  }
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("abi driver: %zu parameter sets, every call rejected cleanly\n", sets.size());
  return 0;
}
