// sgqa_api.hip -- the C ABI of libsgqa (declared in include/sgqa.h): host-side validation,
// workspace carving and kernel launches. Nothing here allocates, copies or synchronizes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/sgqa.h"
#include "sgqa_internal.hpp"

namespace sgqa {

namespace {

constexpr int kMaxDevices = 64;

// Scratch of sgqa_decode_noalloc: one copy per GPU, allocated when the library's code object loads
// on that GPU. Host code never passes `scratch` itself to a kernel (on the host it is only a stand-in
// for the symbol); it uses the device address resolved per device in device_state().
static __device__ __align__(256) uint8_t scratch[SGQA_NOALLOC_SCRATCH_BYTES];

// Facts about one device, filled once (std::call_once) on the first call that runs with it current:
// whether it is a gfx950, its LDS limit per workgroup, and the dynamic-LDS attribute of every
// kernel (set here, before any launch, so that a call never fails between two of its launches).
struct DeviceState {
  std::once_flag once;
  int status = SGQA_ERR_DEVICE;
  int lds_max = 65536;
  int cu_count = 256;
  void* scratch = nullptr;  // this device's address of `scratch` (null if it could not be resolved)
};
DeviceState g_device[kMaxDevices];

int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return (dev >= 0 && dev < kMaxDevices) ? dev : -1;
}

DeviceState* device_state() {
  const int dev = current_device();
  if (dev < 0) return nullptr;
  DeviceState& d = g_device[dev];
  std::call_once(d.once, [&d, dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
    d.lds_max = v;
    if (prop.multiProcessorCount > 0) d.cu_count = prop.multiProcessorCount;
    d.status = prepare_kernels(v) == hipSuccess ? SGQA_OK : SGQA_ERR_HIP;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) d.scratch = ptr;
  });
  return &d;
}

// SGQA_OK when the current device is a gfx950 whose kernels are set up, else the status to return.
int device_ready() {
  const DeviceState* d = device_state();
  return d ? d->status : SGQA_ERR_DEVICE;
}

}  // namespace

int max_lds_per_block() {
  const DeviceState* d = device_state();
  return d ? d->lds_max : 65536;
}

int device_cu_count() {
  const DeviceState* d = device_state();
  return d ? d->cu_count : 256;
}

hipError_t allow_full_lds(const void* fn, int lds_max) {
  hipFuncAttributes a;
  hipError_t e = hipFuncGetAttributes(&a, fn);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max - (int)a.sharedSizeBytes);
}

hipError_t prepare_kernels(int lds_max) {
  hipError_t e = prepare_index_topk_kernels(lds_max);
  if (e == hipSuccess) e = prepare_union_kernels(lds_max);
  if (e == hipSuccess) e = prepare_attend_kernels(lds_max);
  if (e == hipSuccess) e = prepare_attend_bwd_kernels(lds_max);
  return e;
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

size_t round_up(size_t x) { return (x + 255) / 256 * 256; }

bool is_pow2_le64(int b) { return b >= 1 && b <= 64 && (b & (b - 1)) == 0; }

int kb_of(const sgqa_params* p) { return p->topk_tokens / p->block; }

float scale_of(const sgqa_params* p) {
  return p->softmax_scale > 0.0f ? p->softmax_scale : (float)(1.0 / sqrt((double)p->head_dim));
}

// Checks shared by the calls; `need` selects which groups of fields matter.
enum { NEED_INDEX = 1, NEED_ATTN = 2, NEED_SELECT = 4, NEED_UNION = 8, NEED_LIST = 16, NEED_DECODE = 32,
       NEED_MASKED = 64, NEED_BWD = 128 };

int check_params(const sgqa_params* p, int need, bool prefill) {
  if (!p) return SGQA_ERR_NULL;
  if (p->n_tokens < 1 || p->n_seqs < 1) return SGQA_ERR_SHAPE;
  if (prefill && p->n_seqs != 1) return SGQA_ERR_SHAPE;
  if (!is_pow2_le64(p->block)) return SGQA_ERR_SHAPE;
  if (need & NEED_INDEX) {
    if (p->idx_dim != 64) return SGQA_ERR_SHAPE;
  }
  if (need & (NEED_SELECT | NEED_ATTN | NEED_UNION)) {
    if (p->n_kv_heads < 1) return SGQA_ERR_SHAPE;
    if (p->topk_tokens < p->block || p->topk_tokens % p->block != 0) return SGQA_ERR_SHAPE;
    if (kb_of(p) > 2048) return SGQA_ERR_SHAPE;
  }
  // Head counts first: the checks below derive r = Hq / G from them.
  if (need & NEED_ATTN) {
    if (p->head_dim != 128) return SGQA_ERR_SHAPE;
    if (p->n_q_heads < 1 || p->n_q_heads % p->n_kv_heads != 0) return SGQA_ERR_SHAPE;
    if (p->n_q_heads / p->n_kv_heads > 16) return SGQA_ERR_SHAPE;
  }
  if (need & NEED_SELECT) {
    if (p->idx_heads != 4 || p->idx_dim != 64) return SGQA_ERR_SHAPE;
    if (p->n_kv_heads > 16) return SGQA_ERR_SHAPE;
    if (index_topk_lds_min(kb_of(p)) > kGfx950LdsBytes) return SGQA_ERR_SHAPE;
  }
  if (need & NEED_BWD) {
    if (attend_bwd_lds_dq(p->n_tokens, p->block) > kGfx950LdsBytes) return SGQA_ERR_SHAPE;
    const long long r = p->n_kv_heads > 0 ? p->n_q_heads / p->n_kv_heads : 1;
    const long long tile = p->union_tile < p->n_tokens ? p->union_tile : p->n_tokens;
    if (tile * r * (r - 1) >= (1LL << 32)) return SGQA_ERR_SHAPE;  // row-index division in dk/dv
  }
  if (need & NEED_MASKED) {
    if (attend_masked_loads(p->n_q_heads, p->n_kv_heads, p->block) == 0) return SGQA_ERR_SHAPE;
  }
  if (need & NEED_DECODE) {
    if (decode_attend_lds(kb_of(p)) > kGfx950LdsBytes) return SGQA_ERR_SHAPE;
  }
  if (need & NEED_UNION) {
    if (p->union_tile < 1) return SGQA_ERR_SHAPE;
  }
  if (need & NEED_LIST) {
    // Prefill attention walks the tile's block list in fixed-size LDS segments (any length).
    if (attend_lds_bytes_for(p->n_tokens, p->block) > kGfx950LdsBytes) return SGQA_ERR_SHAPE;
  }
  return SGQA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? SGQA_OK : SGQA_ERR_HIP; }

struct PrefillWs {
  uint16_t* kbar;
  int32_t* topk;
  uint32_t* umask;
  int32_t* ucount;
  uint32_t* selbits;
  size_t bytes;
};

// Bytes of the per-query selection bitmaps [G][N][W] of the masked-union attention.
size_t selbits_bytes(const sgqa_params* p) {
  const long long nbc = ((long long)p->n_tokens + p->block - 1) / p->block;
  return round_up((size_t)p->n_kv_heads * p->n_tokens * ((nbc + 31) / 32) * 4);
}

// Prefill workspace: kbar, [topk (masked variant only)], umask, ucount, [selbits (masked variant)].
PrefillWs prefill_layout(const sgqa_params* p, void* ws, bool with_topk) {
  const long long N = p->n_tokens, G = p->n_kv_heads;
  const long long NB = N / p->block, T = (N + p->union_tile - 1) / p->union_tile;
  const long long nbc = (N + p->block - 1) / p->block, W = (nbc + 31) / 32;
  size_t off = 0;
  PrefillWs l;
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  l.kbar = reinterpret_cast<uint16_t*>(b ? b + off : nullptr);
  off += round_up((size_t)NB * p->idx_dim * 2);
  l.topk = reinterpret_cast<int32_t*>(b && with_topk ? b + off : nullptr);
  if (with_topk) off += round_up((size_t)G * N * kb_of(p) * 4);
  l.umask = reinterpret_cast<uint32_t*>(b ? b + off : nullptr);
  off += round_up((size_t)G * T * W * 4);
  l.ucount = reinterpret_cast<int32_t*>(b ? b + off : nullptr);
  off += round_up((size_t)G * T * 4);
  l.selbits = reinterpret_cast<uint32_t*>(b && with_topk ? b + off : nullptr);
  if (with_topk) off += selbits_bytes(p);
  l.bytes = off;
  return l;
}

struct DecodeWs {
  int32_t* sel;
  void* select_ws;
  size_t bytes;
};

DecodeWs decode_layout(const sgqa_params* p, void* ws) {
  const int kb = kb_of(p);
  size_t off = 0;
  DecodeWs l;
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  l.sel = reinterpret_cast<int32_t*>(b ? b + off : nullptr);
  off += round_up((size_t)p->n_seqs * p->n_kv_heads * kb * 4);
  l.select_ws = b ? b + off : nullptr;
  off += round_up(decode_select_ws_bytes(p->n_seqs, p->n_tokens, p->n_kv_heads, p->block, kb));
  l.bytes = off;
  return l;
}

}  // namespace

}  // namespace sgqa

using namespace sgqa;

extern "C" {

int sgqa_abi_version(void) { return SGQA_ABI_VERSION; }

const char* sgqa_status_string(int status) {
  switch (status) {
    case SGQA_OK:
      return "ok";
    case SGQA_ERR_NULL:
      return "a required pointer is NULL";
    case SGQA_ERR_SHAPE:
      return "unsupported or inconsistent sizes";
    case SGQA_ERR_ALIGN:
      return "a tensor pointer is not 16-byte aligned";
    case SGQA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case SGQA_ERR_DEVICE:
      return "the current device is not a gfx950 GPU";
    case SGQA_ERR_HIP:
      return "the HIP runtime reported an error while launching";
    case SGQA_ERR_SCRATCH:
      return "the call needs more scratch than the library's static buffer holds (SGQA_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown status";
  }
}

int sgqa_workspace_size(const sgqa_params* p, int op, size_t* bytes) {
  if (!bytes || !p) return SGQA_ERR_NULL;
  int st = SGQA_OK;
  switch (op) {
    case SGQA_OP_COMPRESS:
      st = check_params(p, NEED_INDEX, false);
      if (st == SGQA_OK) *bytes = 0;
      return st;
    case SGQA_OP_INDEX_TOPK:
      st = check_params(p, NEED_SELECT, true);
      if (st == SGQA_OK) *bytes = 0;
      return st;
    case SGQA_OP_UNION:
      st = check_params(p, NEED_UNION, true);
      if (st == SGQA_OK) *bytes = 0;
      return st;
    case SGQA_OP_ATTEND:
      st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST, true);
      if (st == SGQA_OK) *bytes = 0;
      return st;
    case SGQA_OP_PREFILL:
      st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_UNION | NEED_ATTN | NEED_LIST, true);
      if (st == SGQA_OK) *bytes = prefill_layout(p, nullptr, false).bytes;
      return st;
    case SGQA_OP_DECODE:
      st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_DECODE | NEED_ATTN, false);
      if (st == SGQA_OK) *bytes = decode_layout(p, nullptr).bytes;
      return st;
    case SGQA_OP_ATTEND_BWD:
      st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST | NEED_BWD, true);
      if (st == SGQA_OK)
        *bytes = attend_bwd_plan(p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block, p->union_tile).bytes;
      return st;
    case SGQA_OP_ATTEND_MASKED:
      st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST | NEED_MASKED, true);
      if (st == SGQA_OK) *bytes = selbits_bytes(p);
      return st;
    case SGQA_OP_PREFILL_MASKED:
      st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_UNION | NEED_ATTN | NEED_LIST | NEED_MASKED, true);
      if (st == SGQA_OK) *bytes = prefill_layout(p, nullptr, true).bytes;
      return st;
    default:
      return SGQA_ERR_SHAPE;
  }
}

int sgqa_compress(const sgqa_params* p, const sgqa_bf16* idx_k, sgqa_bf16* blk_k, sgqa_stream stream) {
  int st = check_params(p, NEED_INDEX, false);
  if (st) return st;
  if (!idx_k || (!blk_k && p->n_tokens >= p->block)) return SGQA_ERR_NULL;  // N < B: nothing to write
  if (!aligned16(idx_k) || !aligned16(blk_k)) return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_compress(idx_k, blk_k, p->n_seqs, p->n_tokens, p->idx_dim, p->block, (hipStream_t)stream));
}

int sgqa_index_topk(const sgqa_params* p, const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* blk_k,
                    int32_t* topk, void* ws, size_t ws_bytes, sgqa_stream stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_params(p, NEED_SELECT, true);
  if (st) return st;
  if (!idx_q || !idx_w || !topk || (!blk_k && p->n_tokens >= p->block)) return SGQA_ERR_NULL;
  if (!aligned16(idx_q) || !aligned16(idx_w) || !aligned16(blk_k) || !aligned16(topk)) return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_index_topk(idx_q, idx_w, blk_k, topk, p->n_tokens, p->n_kv_heads, p->block, kb_of(p),
                                     (hipStream_t)stream));
}

int sgqa_union(const sgqa_params* p, const int32_t* topk, uint32_t* umask, int32_t* ucount, sgqa_stream stream) {
  int st = check_params(p, NEED_UNION, true);
  if (st) return st;
  if (!topk || !umask || !ucount) return SGQA_ERR_NULL;
  if (!aligned16(topk) || !aligned16(umask) || !aligned16(ucount)) return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_union(topk, umask, ucount, p->n_tokens, p->n_kv_heads, p->block, kb_of(p), p->union_tile,
                                (hipStream_t)stream));
}

int sgqa_index_union(const sgqa_params* p, const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* blk_k,
                     uint32_t* umask, int32_t* ucount, void* ws, size_t ws_bytes, sgqa_stream stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_params(p, NEED_SELECT | NEED_UNION, true);
  if (st) return st;
  if (!idx_q || !idx_w || !umask || !ucount || (!blk_k && p->n_tokens >= p->block)) return SGQA_ERR_NULL;
  if (!aligned16(idx_q) || !aligned16(idx_w) || !aligned16(blk_k) || !aligned16(umask) || !aligned16(ucount))
    return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_index_union(idx_q, idx_w, blk_k, umask, ucount, p->n_tokens, p->n_kv_heads, p->block,
                                      kb_of(p), p->union_tile, (hipStream_t)stream));
}

int sgqa_attend(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out, void* ws, size_t ws_bytes,
                sgqa_stream stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST, true);
  if (st) return st;
  if (!q || !k || !v || !umask || !ucount || !out) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(umask) || !aligned16(ucount) || !aligned16(out))
    return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_attend(q, k, v, umask, ucount, out, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block,
                                 p->union_tile, scale_of(p), (hipStream_t)stream));
}

int sgqa_attend_fwd(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                    const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out, float* lse, void* ws,
                    size_t ws_bytes, sgqa_stream stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST, true);
  if (st) return st;
  if (!q || !k || !v || !umask || !ucount || !out || !lse) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(umask) || !aligned16(ucount) || !aligned16(out) ||
      !aligned16(lse))
    return SGQA_ERR_ALIGN;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_attend(q, k, v, umask, ucount, out, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block,
                                 p->union_tile, scale_of(p), (hipStream_t)stream, lse));
}

int sgqa_attend_bwd(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                    const uint32_t* umask, const int32_t* ucount, const sgqa_bf16* out, const float* lse,
                    const sgqa_bf16* dout, sgqa_bf16* dq, sgqa_bf16* dk, sgqa_bf16* dv, void* ws, size_t ws_bytes,
                    sgqa_stream stream) {
  int st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST | NEED_BWD, true);
  if (st) return st;
  if (!q || !k || !v || !umask || !ucount || !out || !lse || !dout || !dq || !dk || !dv) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(umask) || !aligned16(ucount) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ws))
    return SGQA_ERR_ALIGN;
  if (!ws || ws_bytes < attend_bwd_plan(p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block, p->union_tile).bytes)
    return SGQA_ERR_WORKSPACE;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_attend_bwd(q, k, v, umask, out, lse, dout, dq, dk, dv, ws,
                                     p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block, p->union_tile, scale_of(p),
                                     (hipStream_t)stream));
}

int sgqa_attend_masked(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                       const int32_t* topk, const uint32_t* umask, const int32_t* ucount, sgqa_bf16* out, void* ws,
                       size_t ws_bytes, sgqa_stream stream) {
  int st = check_params(p, NEED_ATTN | NEED_UNION | NEED_LIST | NEED_MASKED, true);
  if (st) return st;
  if (!q || !k || !v || !topk || !umask || !ucount || !out) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(topk) || !aligned16(umask) ||
      !aligned16(ucount) || !aligned16(out) || !aligned16(ws))
    return SGQA_ERR_ALIGN;
  if (!ws || ws_bytes < selbits_bytes(p)) return SGQA_ERR_WORKSPACE;
  if ((st = device_ready()) != SGQA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* selbits = static_cast<uint32_t*>(ws);
  hipError_t e = launch_sel_bitmap(topk, selbits, p->n_tokens, p->n_kv_heads, p->block, kb_of(p), s);
  if (e == hipSuccess)
    e = launch_attend_masked(q, k, v, umask, selbits, out, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block,
                             p->union_tile, scale_of(p), s);
  return status_of(e);
}

int sgqa_prefill_masked(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                        const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* idx_k, sgqa_bf16* out, void* ws,
                        size_t ws_bytes, sgqa_stream stream) {
  int st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_UNION | NEED_ATTN | NEED_LIST | NEED_MASKED, true);
  if (st) return st;
  if (!q || !k || !v || !idx_q || !idx_w || !idx_k || !out) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx_q) || !aligned16(idx_w) ||
      !aligned16(idx_k) || !aligned16(out) || !aligned16(ws))
    return SGQA_ERR_ALIGN;
  const PrefillWs l = prefill_layout(p, ws, true);
  if (!ws || ws_bytes < l.bytes) return SGQA_ERR_WORKSPACE;
  if ((st = device_ready()) != SGQA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_compress(idx_k, l.kbar, 1, p->n_tokens, p->idx_dim, p->block, s);
  if (e == hipSuccess)
    e = launch_index_topk(idx_q, idx_w, l.kbar, l.topk, p->n_tokens, p->n_kv_heads, p->block, kb_of(p), s);
  if (e == hipSuccess)
    e = launch_union(l.topk, l.umask, l.ucount, p->n_tokens, p->n_kv_heads, p->block, kb_of(p), p->union_tile, s);
  if (e == hipSuccess) e = launch_sel_bitmap(l.topk, l.selbits, p->n_tokens, p->n_kv_heads, p->block, kb_of(p), s);
  if (e == hipSuccess)
    e = launch_attend_masked(q, k, v, l.umask, l.selbits, out, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block,
                             p->union_tile, scale_of(p), s);
  return status_of(e);
}

int sgqa_prefill(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k, const sgqa_bf16* v,
                 const sgqa_bf16* idx_q, const float* idx_w, const sgqa_bf16* idx_k, sgqa_bf16* out, void* ws,
                 size_t ws_bytes, sgqa_stream stream) {
  int st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_UNION | NEED_ATTN | NEED_LIST, true);
  if (st) return st;
  if (!q || !k || !v || !idx_q || !idx_w || !idx_k || !out) return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx_q) || !aligned16(idx_w) ||
      !aligned16(idx_k) || !aligned16(out) || !aligned16(ws))
    return SGQA_ERR_ALIGN;
  const PrefillWs l = prefill_layout(p, ws, false);
  if (!ws || ws_bytes < l.bytes) return SGQA_ERR_WORKSPACE;
  if ((st = device_ready()) != SGQA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_compress(idx_k, l.kbar, 1, p->n_tokens, p->idx_dim, p->block, s);
  if (e == hipSuccess)
    e = launch_index_union(idx_q, idx_w, l.kbar, l.umask, l.ucount, p->n_tokens, p->n_kv_heads, p->block, kb_of(p),
                           p->union_tile, s);
  if (e == hipSuccess)
    e = launch_attend(q, k, v, l.umask, l.ucount, out, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block,
                      p->union_tile, scale_of(p), s);
  return status_of(e);
}

namespace {

// Checks of a paged-cache descriptor (null = dense caches); on success fills `out`.
int check_pages(const sgqa_params* p, const sgqa_pages* pg, PageTable* out) {
  *out = PageTable();
  if (!pg) return SGQA_OK;
  if (!pg->table) return SGQA_ERR_NULL;
  if (!aligned16(pg->table)) return SGQA_ERR_ALIGN;
  const int pt = pg->page_tokens;
  if (pt < p->block || (pt & (pt - 1)) != 0) return SGQA_ERR_SHAPE;
  if (pg->max_pages < 1 || (long long)pg->max_pages * pt < p->n_tokens || pg->n_pages < 1) return SGQA_ERR_SHAPE;
  if ((long long)pg->n_pages * p->n_kv_heads * pt > 0x7FFFFFFFLL) return SGQA_ERR_SHAPE;  // pool rows index in int32
  out->table = pg->table;
  out->max_pages = pg->max_pages;
  out->page_tokens = pt;
  out->n_pages = pg->n_pages;
  return SGQA_OK;
}

// Shared body of sgqa_decode, sgqa_decode_varlen and sgqa_decode_fp8 (kv_scale != nullptr: the caches
// hold FP8 E4M3 codes).
int decode_impl(const sgqa_params* p, const sgqa_bf16* q, const void* k_cache, const void* v_cache,
                const float* kv_scale, const sgqa_pages* pages, const sgqa_bf16* blk_k, const sgqa_bf16* idx_q,
                const float* idx_w, const int32_t* seq_lens, int32_t* topk_out, sgqa_bf16* out, void* ws,
                size_t ws_bytes, sgqa_stream stream) {
  const bool fp8 = kv_scale != nullptr;
  int st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_DECODE | NEED_ATTN, false);
  if (st) return st;
  if (fp8 && decode_attend_f8_lds(kb_of(p)) > kGfx950LdsBytes) return SGQA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !idx_q || !idx_w || !out || (!blk_k && p->n_tokens > p->block))
    return SGQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(blk_k) || !aligned16(idx_q) ||
      !aligned16(idx_w) || !aligned16(topk_out) || !aligned16(out) || !aligned16(ws) || !aligned16(seq_lens) ||
      !aligned16(kv_scale))
    return SGQA_ERR_ALIGN;
  PageTable pt;
  st = check_pages(p, pages, &pt);
  if (st) return st;
  const DecodeWs l = decode_layout(p, ws);
  if (!ws || ws_bytes < l.bytes) return SGQA_ERR_WORKSPACE;
  if ((st = device_ready()) != SGQA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int kb = kb_of(p);
  hipError_t e = launch_decode_select(idx_q, idx_w, blk_k, l.sel, topk_out, l.select_ws, p->n_seqs, p->n_tokens,
                                      p->n_kv_heads, p->block, kb, seq_lens, s);
  if (e == hipSuccess && fp8)
    e = launch_decode_attend_f8(q, static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache),
                                kv_scale, l.sel, out, p->n_seqs, p->n_tokens, p->n_q_heads, p->n_kv_heads,
                                p->block, kb, scale_of(p), seq_lens, pt, s);
  else if (e == hipSuccess)
    e = launch_decode_attend(q, static_cast<const sgqa_bf16*>(k_cache), static_cast<const sgqa_bf16*>(v_cache),
                             l.sel, out, p->n_seqs, p->n_tokens, p->n_q_heads, p->n_kv_heads, p->block, kb,
                             scale_of(p), seq_lens, pt, s);
  return status_of(e);
}

}  // namespace

int sgqa_decode(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache, const sgqa_bf16* v_cache,
                const sgqa_bf16* blk_k, const sgqa_bf16* idx_q, const float* idx_w, int32_t* topk_out,
                sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream) {
  return decode_impl(p, q, k_cache, v_cache, nullptr, nullptr, blk_k, idx_q, idx_w, nullptr, topk_out, out, ws,
                     ws_bytes, stream);
}

int sgqa_decode_noalloc(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache,
                        const sgqa_bf16* v_cache, const sgqa_bf16* blk_k, const sgqa_bf16* idx_q, const float* idx_w,
                        int32_t* topk_out, sgqa_bf16* out, sgqa_stream stream) {
  int st = check_params(p, NEED_INDEX | NEED_SELECT | NEED_DECODE | NEED_ATTN, false);
  if (st) return st;
  if (decode_layout(p, nullptr).bytes > (size_t)SGQA_NOALLOC_SCRATCH_BYTES) return SGQA_ERR_SCRATCH;
  if ((st = device_ready()) != SGQA_OK) return st;
  void* ws = device_state()->scratch;
  if (!ws) return SGQA_ERR_HIP;
  return decode_impl(p, q, k_cache, v_cache, nullptr, nullptr, blk_k, idx_q, idx_w, nullptr, topk_out, out, ws,
                     (size_t)SGQA_NOALLOC_SCRATCH_BYTES, stream);
}

int sgqa_decode_varlen(const sgqa_params* p, const sgqa_bf16* q, const sgqa_bf16* k_cache,
                       const sgqa_bf16* v_cache, const sgqa_pages* pages, const sgqa_bf16* blk_k,
                       const sgqa_bf16* idx_q, const float* idx_w, const int32_t* seq_lens, int32_t* topk_out,
                       sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream) {
  if (!seq_lens) return SGQA_ERR_NULL;
  return decode_impl(p, q, k_cache, v_cache, nullptr, pages, blk_k, idx_q, idx_w, seq_lens, topk_out, out, ws,
                     ws_bytes, stream);
}

int sgqa_decode_fp8(const sgqa_params* p, const sgqa_bf16* q, const uint8_t* k_cache, const uint8_t* v_cache,
                    const float* kv_scale, const sgqa_pages* pages, const sgqa_bf16* blk_k,
                    const sgqa_bf16* idx_q, const float* idx_w, const int32_t* seq_lens, int32_t* topk_out,
                    sgqa_bf16* out, void* ws, size_t ws_bytes, sgqa_stream stream) {
  if (!kv_scale) return SGQA_ERR_NULL;
  return decode_impl(p, q, k_cache, v_cache, kv_scale, pages, blk_k, idx_q, idx_w, seq_lens, topk_out, out, ws,
                     ws_bytes, stream);
}

int sgqa_append(const sgqa_params* p, const sgqa_bf16* k_new, const sgqa_bf16* v_new, const sgqa_bf16* idx_k_new,
                const int32_t* positions, sgqa_bf16* k_cache, sgqa_bf16* v_cache, const sgqa_pages* pages,
                sgqa_bf16* idx_k_cache, sgqa_bf16* blk_k, sgqa_stream stream) {
  int st = check_params(p, NEED_INDEX, false);
  if (st) return st;
  if (p->head_dim != 128 || p->n_kv_heads < 1) return SGQA_ERR_SHAPE;
  if (!k_new || !v_new || !idx_k_new || !positions || !k_cache || !v_cache || !idx_k_cache ||
      (!blk_k && p->n_tokens >= p->block))
    return SGQA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(idx_k_new) || !aligned16(positions) ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(idx_k_cache) || !aligned16(blk_k))
    return SGQA_ERR_ALIGN;
  PageTable pt;
  st = check_pages(p, pages, &pt);
  if (st) return st;
  if ((st = device_ready()) != SGQA_OK) return st;
  return status_of(launch_append(k_new, v_new, idx_k_new, positions, k_cache, v_cache, pt, idx_k_cache, blk_k,
                                 p->n_seqs, p->n_tokens, p->n_kv_heads, p->idx_dim, p->block, (hipStream_t)stream));
}

}  // extern "C"
