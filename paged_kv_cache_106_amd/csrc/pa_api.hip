// pa_api.hip -- libpa's C ABI for the device entry points: host-side argument
// checks, workspace layout and kernel dispatch.  No device memory is
// allocated here and no stream is synchronised.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;

constexpr int32_t kMaxPartition = 1024;
constexpr int32_t kMaxGrid = 65535;        // grid y / z limit

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int log2_exact(int32_t v) {
  int k = 0;
  while ((1 << k) < v) ++k;
  return (1 << k) == v ? k : -1;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Workspace {
  size_t acc_off, max_off, sum_off, total;
};

Workspace workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                           int64_t num_parts) {
  const size_t rows = static_cast<size_t>(num_seqs * num_q_heads * num_parts);
  Workspace w{};
  w.acc_off = 0;
  w.max_off = round_up(rows * static_cast<size_t>(head_dim) * sizeof(float), 256);
  w.sum_off = w.max_off + round_up(rows * sizeof(float), 256);
  w.total = w.sum_off + round_up(rows * sizeof(float), 256);
  return w;
}

int (*attn_launcher(pa_dtype dtype, int32_t head_dim, bool q8 = false))(
    int, const AttnParams&, hipStream_t, hipEvent_t, hipEvent_t) {
  if (q8) {
    if (dtype == PA_F16) return head_dim == 64 ? launch_attn_q8_f16_d64 : launch_attn_q8_f16_d128;
    return head_dim == 64 ? launch_attn_q8_bf16_d64 : launch_attn_q8_bf16_d128;
  }
  if (dtype == PA_F16) return head_dim == 64 ? launch_attn_f16_d64 : launch_attn_f16_d128;
  return head_dim == 64 ? launch_attn_bf16_d64 : launch_attn_bf16_d128;
}

// The INT8 scale arrays of a decode: present and 4-byte aligned.
pa_status check_scales(const float* key_scale, const float* value_scale, int32_t num_seqs,
                       AttnParams* p) {
  if (num_seqs > 0) {
    if (!key_scale || !value_scale) return fail(PA_ERR_INVALID_ARG, "NULL scale array");
    if (!aligned(key_scale, 4) || !aligned(value_scale, 4))
      return fail(PA_ERR_INVALID_ARG, "scale arrays must be 4-byte aligned");
  }
  p->k_scale = key_scale;
  p->v_scale = value_scale;
  return PA_OK;
}

// Shared checks of pa_decode / pa_decode_partitioned; fills p on success.
pa_status check_decode(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_context_len, float scale, pa_dtype dtype, AttnParams* p) {
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be 16 or 32");
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (max_context_len < 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len outside [0, max_blocks_per_seq * block_size]");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size overflows int32");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (num_seqs > kMaxGrid) return fail(PA_ERR_UNSUPPORTED, "num_seqs above 65535");
  if (static_cast<int64_t>(num_seqs) * num_q_heads > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_q_heads overflows int32");
  if (num_seqs > 0) {
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
      return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
        !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
      return fail(PA_ERR_INVALID_ARG, "device buffers must be 16-byte aligned (metadata 4-byte)");
  }
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t chunks = (group + 7) / 8;
  const int32_t gt = (group + chunks - 1) / chunks;
  if (static_cast<int64_t>(num_kv_heads) * chunks > kMaxGrid)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * head chunks above 65535");

  *p = AttnParams{};
  p->out = out;
  p->q = query;
  p->k_cache = key_cache;
  p->v_cache = value_cache;
  p->block_tables = block_tables;
  p->context_lens = context_lens;
  p->block_stride = static_cast<int64_t>(block_size) * num_kv_heads * head_dim;
  p->mb = max_blocks_per_seq;
  p->num_seqs = num_seqs;
  p->num_q_heads = num_q_heads;
  p->num_kv_heads = num_kv_heads;
  p->group = group;
  p->heads_per_wg = gt;
  p->head_chunks = chunks;
  p->work_items = nullptr;
  p->num_work_items = 0;
  p->block_size = block_size;
  p->log2_block_size = log2_exact(block_size);
  p->num_blocks = num_blocks;
  p->scale_log2 = scale * 1.4426950408889634f;
  return PA_OK;
}

// With nothing to launch, the caller's events still mark this point of the
// stream, so waiting on them behaves as after a launch.
pa_status mark_events(hipEvent_t start, hipEvent_t stop, hipStream_t stream, const char* what) {
  for (hipEvent_t e : {start, stop}) {
    if (e && hipEventRecord(e, stream) != hipSuccess) {
      g_last_error = std::string(what) + ": hipEventRecord failed";
      return PA_ERR_HIP;
    }
  }
  return PA_OK;
}

pa_status launched(int err, const char* what) {
  if (err != 0) {
    std::string msg = std::string(what) + ": " + hipGetErrorString(static_cast<hipError_t>(err));
    g_last_error = msg;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace

pa_status fail(pa_status st, const char* msg) {
  g_last_error = msg;
  return st;
}

// The split-context decode after the shared checks (16-bit or INT8 pools).
pa_status partitioned(AttnParams& p, bool q8, pa_dtype dtype, int32_t head_dim,
                      int32_t block_size, int32_t max_context_len, int32_t partition_size,
                      const int32_t* work_items, int32_t num_work_items, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t start_event,
                      hipEvent_t stop_event, const char* what);

void clear_error() { g_last_error.clear(); }

}  // namespace pa

using pa::fail;

extern "C" {

const char* pa_last_error(void) { return pa::g_last_error.c_str(); }

const char* pa_version(void) { return "libpa 0.1 (gfx950)"; }

pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  pa::clear_error();
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads, head_dim, block_size, num_blocks must be positive");
  if (head_dim % 8 != 0) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!pa::aligned(key, 16) || !pa::aligned(value, 16) || !pa::aligned(key_cache, 16) ||
      !pa::aligned(value_cache, 16) || !pa::aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "device buffers must be 16-byte aligned (slots 8-byte)");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;   // elements per token
  const int64_t chunks_per_tok = row / 8;
  if (chunks_per_tok > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "token row too large");
  const int64_t num_chunks = static_cast<int64_t>(num_tokens) * chunks_per_tok;
  if ((num_chunks + 255) / 256 > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  return pa::launched(pa::launch_cache_write(key, value, key_cache, value_cache, slot_mapping,
                                             num_tokens, static_cast<int32_t>(chunks_per_tok),
                                             num_slots, stream),
                      "pa_reshape_and_cache");
}

namespace {
// Device address of pinned host memory (NULL stays NULL); fails for memory
// the device cannot read.
bool device_view(const void* host, const void** dev) {
  if (!host) {
    *dev = nullptr;
    return true;
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host), 0) != hipSuccess || !d) {
    (void)hipGetLastError();   // leave no sticky error for the next call
    return false;
  }
  *dev = d;
  return true;
}
}  // namespace

pa_status pa_write_step(const int64_t* staged_slots, const int32_t* staged_lens,
                        const int32_t* staged_items, int32_t num_items, int64_t* slot_mapping,
                        int32_t* context_lens, int32_t* work_items, int32_t* block_tables,
                        int32_t max_blocks_per_seq, const void* key, const void* value,
                        void* key_cache, void* value_cache, int32_t num_seqs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, hipStream_t stream, hipEvent_t done_event) {
  pa::clear_error();
  if (num_seqs < 0 || num_items < 0) return fail(PA_ERR_INVALID_ARG, "negative count");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq must be positive");
  if (head_dim % 8 != 0) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (num_seqs == 0 && num_items == 0)
    return pa::mark_events(nullptr, done_event, stream, "pa_write_step");
  if (num_seqs > 0 && (!staged_slots || !staged_lens || !slot_mapping || !context_lens ||
                       !block_tables || !key || !value || !key_cache || !value_cache))
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (num_items > 0 && (!staged_items || !work_items))
    return fail(PA_ERR_INVALID_ARG, "NULL work list");
  if (!pa::aligned(staged_slots, 8) || !pa::aligned(staged_lens, 4) ||
      !pa::aligned(staged_items, 8) || !pa::aligned(slot_mapping, 8) ||
      !pa::aligned(context_lens, 4) || !pa::aligned(work_items, 8) ||
      !pa::aligned(block_tables, 4) || !pa::aligned(key, 16) || !pa::aligned(value, 16) ||
      !pa::aligned(key_cache, 16) || !pa::aligned(value_cache, 16))
    return fail(PA_ERR_INVALID_ARG,
                "misaligned buffer (K/V 16 bytes, slots and work list 8, lengths and tables 4)");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  const int64_t chunks_per_tok = row / 8;
  if (chunks_per_tok > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "token row too large");
  const int64_t num_chunks = static_cast<int64_t>(num_seqs) * chunks_per_tok;
  if ((num_chunks + 255) / 256 + (static_cast<int64_t>(num_items) + 255) / 256 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  const void *ds, *dl, *di;
  if (!device_view(staged_slots, &ds) || !device_view(staged_lens, &dl) ||
      !device_view(staged_items, &di))
    return fail(PA_ERR_INVALID_ARG,
                "staged arrays must be pinned host memory the device can read (hipHostMalloc)");
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  return pa::launched(
      pa::launch_write_step(static_cast<const int64_t*>(ds), static_cast<const int32_t*>(dl),
                            static_cast<const int32_t*>(di), num_items, slot_mapping,
                            context_lens, work_items, block_tables, max_blocks_per_seq,
                            block_size, key, value, key_cache, value_cache, num_seqs,
                            static_cast<int32_t>(chunks_per_tok), num_slots, stream,
                            done_event),
      "pa_write_step");
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_context_len, float scale, pa_dtype dtype,
                    hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event) {
  pa::clear_error();
  pa::AttnParams p;
  const pa_status st = pa::check_decode(out, query, key_cache, value_cache, block_tables,
                                        max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, num_blocks,
                                        max_context_len, scale, dtype, &p);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return pa::mark_events(start_event, stop_event, stream, "pa_decode");
  p.chunk = pa::kSingleChunk;
  return pa::launched(pa::attn_launcher(dtype, head_dim)(0, p, stream, start_event, stop_event),
                      "pa_decode");
}

pa_status pa_decode_int8(void* out, const void* query, const int8_t* key_cache,
                         const int8_t* value_cache, const float* key_scale,
                         const float* value_scale, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_context_len, float scale, pa_dtype dtype, hipStream_t stream,
                         hipEvent_t start_event, hipEvent_t stop_event) {
  pa::clear_error();
  pa::AttnParams p;
  pa_status st = pa::check_decode(out, query, key_cache, value_cache, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                  num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                  scale, dtype, &p);
  if (st == PA_OK) st = pa::check_scales(key_scale, value_scale, num_seqs, &p);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return pa::mark_events(start_event, stop_event, stream, "pa_decode_int8");
  p.chunk = pa::kSingleChunk;
  return pa::launched(
      pa::attn_launcher(dtype, head_dim, true)(0, p, stream, start_event, stop_event),
      "pa_decode_int8");
}

size_t pa_decode_partitioned_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_context_len,
                                            int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size <= 0)
    return 0;
  const int64_t parts = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
  return pa::workspace_layout(num_seqs, num_q_heads, head_dim, parts).total;
}

pa_status pa_decode_partitioned(void* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, pa_dtype dtype,
                                int32_t partition_size, const int32_t* work_items,
                                int32_t num_work_items, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, hipEvent_t start_event,
                                hipEvent_t stop_event) {
  pa::clear_error();
  pa::AttnParams p;
  const pa_status st = pa::check_decode(out, query, key_cache, value_cache, block_tables,
                                        max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, num_blocks,
                                        max_context_len, scale, dtype, &p);
  if (st != PA_OK) return st;
  return pa::partitioned(p, false, dtype, head_dim, block_size, max_context_len, partition_size,
                         work_items, num_work_items, workspace, workspace_bytes, stream,
                         start_event, stop_event, "pa_decode_partitioned");
}

pa_status pa_decode_partitioned_int8(
    void* out, const void* query, const int8_t* key_cache, const int8_t* value_cache,
    const float* key_scale, const float* value_scale, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_context_len, float scale, pa_dtype dtype,
    int32_t partition_size, const int32_t* work_items, int32_t num_work_items, void* workspace,
    size_t workspace_bytes, hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event) {
  pa::clear_error();
  pa::AttnParams p;
  pa_status st = pa::check_decode(out, query, key_cache, value_cache, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                  num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                  scale, dtype, &p);
  if (st == PA_OK) st = pa::check_scales(key_scale, value_scale, num_seqs, &p);
  if (st != PA_OK) return st;
  return pa::partitioned(p, true, dtype, head_dim, block_size, max_context_len, partition_size,
                         work_items, num_work_items, workspace, workspace_bytes, stream,
                         start_event, stop_event, "pa_decode_partitioned_int8");
}

}  // extern "C"

// ---- the split-context decode with no allocation anywhere ------------------
// Its workspace is this file-scope array: one copy per GPU, created when the
// code object is loaded on that GPU and held until the process ends.  In
// host code `scratch` names a host-side stand-in; the array's device address
// comes from hipGetSymbolAddress, once per device, with that device current.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device; NULL with the
// error set when it cannot be found.
void* scratch_of_current_device(const char* what) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    pa::g_last_error = std::string(what) + ": no usable current device";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      pa::g_last_error = std::string(what) + ": hipGetSymbolAddress(scratch) failed: " +
                         hipGetErrorString(e);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t pa_decode_partitioned_noalloc_max_workspace(void) { return kScratchBytes; }

pa_status pa_decode_partitioned_noalloc(void* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks,
                                        int32_t max_context_len, float scale, pa_dtype dtype,
                                        int32_t partition_size, const int32_t* work_items,
                                        int32_t num_work_items, hipStream_t stream,
                                        hipEvent_t start_event, hipEvent_t stop_event) {
  pa::clear_error();
  const char* what = "pa_decode_partitioned_noalloc";
  pa::AttnParams p;
  const pa_status st = pa::check_decode(out, query, key_cache, value_cache, block_tables,
                                        max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                        num_kv_heads, head_dim, block_size, num_blocks,
                                        max_context_len, scale, dtype, &p);
  if (st != PA_OK) return st;
  if (num_seqs > 0 && partition_size > 0) {
    const size_t need = pa_decode_partitioned_workspace_size(
        num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
    if (need > kScratchBytes)
      return fail(PA_ERR_INVALID_ARG,
                  "pa_decode_partitioned_noalloc: the split workspace this call needs "
                  "(num_seqs x num_q_heads x ceil(max_context_len / partition_size) x "
                  "(head_dim + 2) x 4 bytes, each part 256-byte aligned) exceeds the 64 MiB "
                  "scratch array; use pa_decode_partitioned with a caller workspace");
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    int sdev = -1, cur = -1;
    if (stream && (hipStreamGetDevice(stream, &sdev) != hipSuccess ||
                   hipGetDevice(&cur) != hipSuccess || sdev != cur)) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID_ARG,
                  "pa_decode_partitioned_noalloc: the stream must belong to the current device");
    }
    ws = scratch_of_current_device(what);
    if (!ws) return PA_ERR_HIP;
  }
  return pa::partitioned(p, false, dtype, head_dim, block_size, max_context_len, partition_size,
                         work_items, num_work_items, ws, kScratchBytes, stream, start_event,
                         stop_event, what);
}

}  // extern "C"

namespace pa {

pa_status partitioned(AttnParams& p, bool q8, pa_dtype dtype, int32_t head_dim,
                      int32_t block_size, int32_t max_context_len, int32_t partition_size,
                      const int32_t* work_items, int32_t num_work_items, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t start_event,
                      hipEvent_t stop_event, const char* what) {
  const int32_t num_seqs = p.num_seqs, num_q_heads = p.num_q_heads;
  if (partition_size < block_size || partition_size > pa::kMaxPartition ||
      partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG,
                "partition_size must be a multiple of block_size in [block_size, 1024]");
  if (num_work_items < 0 || (num_work_items > 0 && !work_items) ||
      (work_items && !pa::aligned(work_items, 4)))
    return fail(PA_ERR_INVALID_ARG, "work_items must be NULL or a 4-byte aligned device array");
  // a list names every partition to compute; an empty one would leave every
  // sequence's partials unwritten before the merge reads them
  if (work_items && num_work_items == 0 && num_seqs > 0)
    return fail(PA_ERR_INVALID_ARG,
                "an empty work list names no partition: pass NULL for the full grid");
  // the merge reads 64 partitions of one (sequence, head) through one buffer
  // resource of 64 workspace rows of num_q_heads * head_dim floats
  if (static_cast<int64_t>(num_q_heads) * head_dim * 4 * 64 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_q_heads * head_dim must stay below 2^23 for the merge");
  if ((static_cast<int64_t>(num_work_items) + 7) * p.num_kv_heads * p.head_chunks > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_work_items * num_kv_heads * head chunks overflows int32");
  if (num_seqs == 0) return pa::mark_events(start_event, stop_event, stream, what);
  const int64_t parts = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
  if (parts >= pa::kMaxGrid) return fail(PA_ERR_UNSUPPORTED, "more than 65534 partitions");
  const pa::Workspace w = pa::workspace_layout(num_seqs, num_q_heads, head_dim, parts);
  if (!workspace || !pa::aligned(workspace, 16))
    return fail(PA_ERR_INVALID_ARG, "workspace must be a 16-byte aligned device buffer");
  if (workspace_bytes < w.total) return fail(PA_ERR_INVALID_ARG, "workspace too small");
  char* ws = static_cast<char*>(workspace);
  p.part_acc = reinterpret_cast<float*>(ws + w.acc_off);
  p.part_max = reinterpret_cast<float*>(ws + w.max_off);
  p.part_sum = reinterpret_cast<float*>(ws + w.sum_off);
  p.chunk = partition_size;
  p.num_parts = static_cast<int32_t>(parts);
  p.grid_parts = static_cast<int32_t>(parts | 1);
  p.work_items = num_work_items > 0 ? work_items : nullptr;
  p.num_work_items = num_work_items;
  auto launch = pa::attn_launcher(dtype, head_dim, q8);
  const bool any = work_items ? true : parts > 0;
  if (any) {
    const bool mfma = q8 && p.group >= pa::kQ8MfmaMinGroup;
    const pa_status s1 = pa::launched(
        mfma ? pa::launch_attn_q8_mfma_split(dtype, head_dim, p, stream, start_event, nullptr)
             : launch(1, p, stream, start_event, nullptr),
        what);
    if (s1 != PA_OK) return s1;
  }
  return pa::launched(launch(2, p, stream, any ? nullptr : start_event, stop_event), what);
}

}  // namespace pa

extern "C" {

pa_status pa_update_block_tables(int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, const int64_t* slot_mapping,
                                 int32_t num_seqs, int32_t block_size, int32_t num_blocks,
                                 hipStream_t stream) {
  pa::clear_error();
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad size");
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!pa::aligned(block_tables, 4) || !pa::aligned(context_lens, 4) ||
      !pa::aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned device buffer");
  return pa::launched(pa::launch_update_tables(block_tables, max_blocks_per_seq, context_lens,
                                               slot_mapping, num_seqs, block_size,
                                               static_cast<int64_t>(num_blocks) * block_size,
                                               stream),
                      "pa_update_block_tables");
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         hipStream_t stream) {
  pa::clear_error();
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad size");
  if (head_dim % 8 != 0) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > pa::kMaxGrid) return fail(PA_ERR_UNSUPPORTED, "more than 65535 pairs");
  if (!key_cache || !value_cache || !block_pairs) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (!pa::aligned(key_cache, 16) || !pa::aligned(value_cache, 16) || !pa::aligned(block_pairs, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned device buffer");
  const int64_t chunks_per_block = static_cast<int64_t>(block_size) * num_kv_heads * head_dim / 8;
  return pa::launched(pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs,
                                             chunks_per_block, num_blocks, stream),
                      "pa_copy_blocks");
}


pa_status pa_reshape_and_cache_int8(const void* key, const void* value, int8_t* key_cache,
                                    int8_t* value_cache, float* key_scale, float* value_scale,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  pa::clear_error();
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads, block_size, num_blocks must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !key_scale || !value_scale || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!pa::aligned(key, 16) || !pa::aligned(value, 16) || !pa::aligned(key_cache, 8) ||
      !pa::aligned(value_cache, 8) || !pa::aligned(key_scale, 4) ||
      !pa::aligned(value_scale, 4) || !pa::aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG,
                "misaligned buffer (K/V 16 bytes, codes and slots 8, scales 4)");
  const int64_t chunks_per_tok = static_cast<int64_t>(num_kv_heads) * head_dim / 8;
  if (chunks_per_tok > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "token row too large");
  const int64_t num_chunks = static_cast<int64_t>(num_tokens) * chunks_per_tok;
  if ((num_chunks + 255) / 256 > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  return pa::launched(
      pa::launch_cache_write_q8(key, value, key_cache, value_cache, key_scale, value_scale,
                                slot_mapping, num_tokens, head_dim,
                                static_cast<int32_t>(chunks_per_tok),
                                static_cast<int64_t>(num_blocks) * block_size, block_size,
                                dtype == PA_BF16 ? 1 : 0, stream),
      "pa_reshape_and_cache_int8");
}

pa_status pa_write_step_int8(const int64_t* staged_slots, const int32_t* staged_lens,
                             const int32_t* staged_items, int32_t num_items,
                             int64_t* slot_mapping, int32_t* context_lens, int32_t* work_items,
                             int32_t* block_tables, int32_t max_blocks_per_seq, const void* key,
                             const void* value, int8_t* key_cache, int8_t* value_cache,
                             float* key_scale, float* value_scale, int32_t num_seqs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, pa_dtype dtype, hipStream_t stream,
                             hipEvent_t done_event) {
  pa::clear_error();
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_seqs < 0 || num_items < 0) return fail(PA_ERR_INVALID_ARG, "negative count");
  if (num_kv_heads <= 0 || block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG,
                "num_kv_heads, block_size, num_blocks, max_blocks_per_seq must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_seqs == 0 && num_items == 0)
    return pa::mark_events(nullptr, done_event, stream, "pa_write_step_int8");
  if (num_seqs > 0 && (!staged_slots || !staged_lens || !slot_mapping || !context_lens ||
                       !block_tables || !key || !value || !key_cache || !value_cache ||
                       !key_scale || !value_scale))
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (num_items > 0 && (!staged_items || !work_items))
    return fail(PA_ERR_INVALID_ARG, "NULL work list");
  if (!pa::aligned(staged_slots, 8) || !pa::aligned(staged_lens, 4) ||
      !pa::aligned(staged_items, 8) || !pa::aligned(slot_mapping, 8) ||
      !pa::aligned(context_lens, 4) || !pa::aligned(work_items, 8) ||
      !pa::aligned(block_tables, 4) || !pa::aligned(key, 16) || !pa::aligned(value, 16) ||
      !pa::aligned(key_cache, 8) || !pa::aligned(value_cache, 8) ||
      !pa::aligned(key_scale, 4) || !pa::aligned(value_scale, 4))
    return fail(PA_ERR_INVALID_ARG,
                "misaligned buffer (K/V 16 bytes; codes, slots and work list 8; lengths, tables "
                "and scales 4)");
  const int64_t chunks_per_tok = static_cast<int64_t>(num_kv_heads) * head_dim / 8;
  if (chunks_per_tok > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "token row too large");
  const int64_t num_chunks = static_cast<int64_t>(num_seqs) * chunks_per_tok;
  if ((num_chunks + 255) / 256 + (static_cast<int64_t>(num_items) + 255) / 256 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  const void *ds, *dl, *di;
  if (!device_view(staged_slots, &ds) || !device_view(staged_lens, &dl) ||
      !device_view(staged_items, &di))
    return fail(PA_ERR_INVALID_ARG,
                "staged arrays must be pinned host memory the device can read (hipHostMalloc)");
  return pa::launched(
      pa::launch_write_step_q8(static_cast<const int64_t*>(ds), static_cast<const int32_t*>(dl),
                               static_cast<const int32_t*>(di), num_items, slot_mapping,
                               context_lens, work_items, block_tables, max_blocks_per_seq,
                               block_size, key, value, key_cache, value_cache, key_scale,
                               value_scale, num_seqs, head_dim,
                               static_cast<int32_t>(chunks_per_tok),
                               static_cast<int64_t>(num_blocks) * block_size,
                               dtype == PA_BF16 ? 1 : 0, stream, done_event),
      "pa_write_step_int8");
}

pa_status pa_copy_blocks_int8(int8_t* key_cache, int8_t* value_cache, float* key_scale,
                              float* value_scale, const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, hipStream_t stream) {
  pa::clear_error();
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad size");
  if (head_dim % 16 != 0 || (static_cast<int64_t>(num_kv_heads) * block_size) % 4 != 0)
    return fail(PA_ERR_UNSUPPORTED,
                "head_dim must be a multiple of 16 and num_kv_heads * block_size of 4");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > pa::kMaxGrid) return fail(PA_ERR_UNSUPPORTED, "more than 65535 pairs");
  if (!key_cache || !value_cache || !key_scale || !value_scale || !block_pairs)
    return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (!pa::aligned(key_cache, 16) || !pa::aligned(value_cache, 16) ||
      !pa::aligned(key_scale, 16) || !pa::aligned(value_scale, 16) ||
      !pa::aligned(block_pairs, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned device buffer (pools and scales 16 bytes)");
  const int64_t code_chunks = static_cast<int64_t>(block_size) * num_kv_heads * head_dim / 16;
  const int64_t scale_chunks = static_cast<int64_t>(num_kv_heads) * block_size / 4;
  const pa_status st =
      pa::launched(pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs,
                                          code_chunks, num_blocks, stream),
                   "pa_copy_blocks_int8 (codes)");
  if (st != PA_OK) return st;
  return pa::launched(pa::launch_copy_blocks(key_scale, value_scale, block_pairs, num_pairs,
                                             scale_chunks, num_blocks, stream),
                      "pa_copy_blocks_int8 (scales)");
}
}  // extern "C"
