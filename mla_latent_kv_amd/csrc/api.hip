// C ABI of the MLA decode library (declared in include/mla_decode.h):
// argument validation, workspace sizing and the launch sequences
// plan -> absorb -> attention -> merge (decode) and product -> finish (cache
// append), all on the caller's stream.
#include <math.h>
#include <algorithm>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/mla_decode.h"
#include "common.h"

struct mla_decode_ctx {
  mla_decode_config cfg;
  int device;
  int n_cu;
  float scale;
  int split_target;   // 0 = default for the device
};

namespace {
int split_target_of(const mla_decode_ctx* c, int q_tokens) {
  return c->split_target > 0 ? c->split_target : mla::default_split_target(c->n_cu, q_tokens);
}
}  // namespace

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kMaxNaiveLen = 1 << 20;   // tokens per sequence on the naive path

#ifdef MLA_DEBUG_CHECKS
// Debug build: the preconditions of mla_decode_check_inputs on host copies of
// the lengths and the block table, before any launch (synchronises `stream`).
int debug_check(const int32_t* seq_lens, const int32_t* block_table, int batch, int q_tokens, int mbps,
                int max_seq_len, int64_t num_blocks, hipStream_t stream) {
  std::vector<int32_t> lens, table;
  try {
    lens.resize((size_t)batch);
    table.resize((size_t)batch * (size_t)mbps);
  } catch (const std::bad_alloc&) {
    return MLA_ERR_INVALID_ARG;
  }
  if (hipMemcpyAsync(lens.data(), seq_lens, lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipMemcpyAsync(table.data(), block_table, table.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MLA_ERR_HIP;
  return mla_decode_check_inputs(lens.data(), table.data(), batch, q_tokens, mbps, max_seq_len, num_blocks,
                                 nullptr);
}
#define MLA_DEBUG_CHECK(...)                              \
  do {                                                    \
    const int st_ = debug_check(__VA_ARGS__);             \
    if (st_ != MLA_OK) {                                  \
      if (prev != ctx->device) (void)hipSetDevice(prev);  \
      return st_;                                         \
    }                                                     \
  } while (0)
#else
#define MLA_DEBUG_CHECK(...) \
  do {                       \
  } while (0)
#endif

}  // namespace

extern "C" {

const char* mla_decode_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration or device";
    case MLA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_PRECONDITION: return "inputs break a documented precondition";
    default: return "unknown status";
  }
}

int mla_decode_init(const mla_decode_config* cfg, int hip_device, mla_decode_ctx** out) {
  if (!cfg || !out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg->num_heads != mla::kHeads || cfg->d_nope != mla::kDNope || cfg->d_rope != mla::kDRope ||
      cfg->d_latent != mla::kDLat || cfg->d_v != mla::kDV || cfg->block_size != mla::kBlock)
    return MLA_ERR_UNSUPPORTED;
  if (cfg->max_q_tokens < 1 || cfg->max_q_tokens > 2) return MLA_ERR_UNSUPPORTED;
  if (!(cfg->softmax_scale == cfg->softmax_scale)) return MLA_ERR_INVALID_ARG;   // NaN
  if (cfg->split_target < 0 || cfg->split_target > mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess) return MLA_ERR_HIP;
  if (hip_device < 0 || hip_device >= n_dev) return MLA_ERR_INVALID_ARG;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return MLA_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MLA_ERR_UNSUPPORTED;
  mla_decode_ctx* c = new (std::nothrow) mla_decode_ctx;
  if (!c) return MLA_ERR_INVALID_ARG;
  c->cfg = *cfg;
  c->device = hip_device;
  c->n_cu = prop.multiProcessorCount;
  c->split_target = cfg->split_target;
  c->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                      : 1.0f / sqrtf((float)(cfg->d_nope + cfg->d_rope));
  *out = c;
  return MLA_OK;
}

int mla_decode_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                              int32_t max_seq_len, size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || batch > mla::kMaxBatch || max_seq_len < 1)
    return MLA_ERR_INVALID_ARG;
  if (q_tokens < 1 || q_tokens > ctx->cfg.max_q_tokens) return MLA_ERR_INVALID_ARG;
  const mla::Layout L =
      mla::make_layout(batch, q_tokens, max_seq_len, split_target_of(ctx, q_tokens));
  *bytes = L.total;
  return MLA_OK;
}

namespace {

// one_round: the allocation-free variant's plan (one round of at most one
// work item per slot, which needs batch <= split target)
int run_impl(const mla_decode_ctx* ctx, const mla_decode_args* a, void* workspace,
             size_t workspace_bytes, void* stream_handle, void* const* events, bool one_round = false) {
  if (!ctx || !a) return MLA_ERR_INVALID_ARG;
  if (!a->q_nope || !a->q_pe || !a->w_uk || !a->w_uv || !a->kv_cache || !a->block_table ||
      !a->seq_lens || !a->out)
    return MLA_ERR_INVALID_ARG;
  if (a->batch < 1 || a->batch > mla::kMaxBatch || a->q_tokens < 1 || a->q_tokens > ctx->cfg.max_q_tokens ||
      a->num_blocks < 1 || a->max_blocks_per_seq < 1 || a->max_seq_len < 1)
    return MLA_ERR_INVALID_ARG;
  if ((long long)a->max_blocks_per_seq * mla::kBlock < a->max_seq_len) return MLA_ERR_INVALID_ARG;
  if (!aligned16(a->q_nope) || !aligned16(a->q_pe) || !aligned16(a->w_uk) ||
      !aligned16(a->w_uv) || !aligned16(a->kv_cache) || !aligned16(a->block_table) ||
      !aligned16(a->seq_lens) || !aligned16(a->out))
    return MLA_ERR_MISALIGNED;
  const int target = split_target_of(ctx, a->q_tokens);
  if (one_round && a->batch > target) return MLA_ERR_WORKSPACE;
  const mla::Layout L = mla::make_layout(a->batch, a->q_tokens, a->max_seq_len, target, one_round);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < L.total)
    return MLA_ERR_WORKSPACE;

  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  MLA_DEBUG_CHECK(a->seq_lens, a->block_table, a->batch, a->q_tokens, a->max_blocks_per_seq, a->max_seq_len,
                  a->num_blocks, stream);

  char* ws = (char*)workspace;
  mla::WorkItem* work = (mla::WorkItem*)(ws + L.work);
  mla::SeqInfo* seqinfo = (mla::SeqInfo*)(ws + L.seqinfo);
  int* meta = (int*)(ws + L.meta);
  _Float16* q_abs = (_Float16*)(ws + L.qabs);
  _Float16* part_o = (_Float16*)(ws + L.part_o);
  float* part_lse = (float*)(ws + L.part_lse);
  const int max_len = (int)((long long)a->max_blocks_per_seq * mla::kBlock < a->max_seq_len
                                ? (long long)a->max_blocks_per_seq * mla::kBlock
                                : a->max_seq_len);

  auto mark = [&](int i) -> bool {
    return !events || !events[i] || hipEventRecord((hipEvent_t)events[i], stream) == hipSuccess;
  };
  int status = MLA_OK;
  if (!mark(0) || !mark(1) ||
      mla::launch_prep(a->seq_lens, a->block_table, a->max_blocks_per_seq, a->num_blocks, a->batch, max_len, target, one_round ? 1 : mla::kPlanWaves, L.positions,
                       L.depth, L.max_chunks, work,
                       seqinfo, meta,
                       (const uint16_t*)a->q_nope, (const uint16_t*)a->w_uk, q_abs, L.rows,
                       (int*)(ws + L.range), stream) != hipSuccess) {
    status = MLA_ERR_HIP;
  } else {
    mla::AttnArgs aa;
    aa.cache = (const uint16_t*)a->kv_cache;
    aa.block_table = a->block_table;
    aa.q_pe = (const uint16_t*)a->q_pe;
    aa.q_abs = q_abs;
    aa.work = work;
    aa.seqinfo = seqinfo;
    aa.meta = meta;
    aa.part_o = part_o;
    aa.part_lse = part_lse;
    aa.num_blocks = a->num_blocks;
    aa.max_blocks_per_seq = a->max_blocks_per_seq;
    aa.q_tokens = a->q_tokens;
    aa.max_chunks = L.max_chunks;
    aa.positions = L.positions;
    aa.depth = L.depth;
    aa.scale_log2 = ctx->scale * 1.4426950408889634f / mla::kQScale;
    if (!mark(2) || mla::launch_attn(aa, stream) != hipSuccess || !mark(3) ||
        mla::launch_merge(part_o, part_lse, seqinfo, (const uint16_t*)a->w_uv, a->out, a->batch,
                          a->q_tokens, L.max_chunks, stream) != hipSuccess ||
        !mark(4))
      status = MLA_ERR_HIP;
  }
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

}  // namespace

int mla_decode_run(const mla_decode_ctx* ctx, const mla_decode_args* a, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return run_impl(ctx, a, workspace, workspace_bytes, stream, nullptr);
}

int mla_decode_run_profiled(const mla_decode_ctx* ctx, const mla_decode_args* a,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const events[5]) {
  return run_impl(ctx, a, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

// ---- allocation-free decode: the workspace lives in a file-scope device
// array. In host code `scratch` names a host-side stand-in, not the device
// array: its device address is looked up once per device (with that device
// current) and only that address is used.
namespace {
constexpr size_t kScratchBytes = (size_t)66 << 20;   // 66 MiB per GPU
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of `scratch` on the current device `dev`; nullptr on failure
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int mla_decode_run_noalloc(const mla_decode_ctx* ctx, const mla_decode_args* a, void* stream) {
  if (!ctx || !a) return MLA_ERR_INVALID_ARG;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  void* ws = scratch_address(ctx->device);
  if (prev != ctx->device) (void)hipSetDevice(prev);
  if (!ws) return MLA_ERR_HIP;
  // run_impl rejects a batch above the split target and a layout past the
  // array (MLA_ERR_WORKSPACE) before anything is launched
  return run_impl(ctx, a, ws, kScratchBytes, stream, nullptr, true);
}

int mla_decode_range_flags(const mla_decode_ctx* ctx, const void* workspace, size_t workspace_bytes,
                           void* stream_handle, int32_t* flags) {
  if (!ctx || !flags) return MLA_ERR_INVALID_ARG;
  const size_t need = sizeof(int) * mla::kAbsorbGroups;
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  int host[mla::kAbsorbGroups];
  hipStream_t stream = (hipStream_t)stream_handle;
  int status = MLA_OK;
  if (hipMemcpyAsync(host, workspace, need, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    status = MLA_ERR_HIP;
  } else {
    int any = 0;
    for (int i = 0; i < mla::kAbsorbGroups; ++i) any |= host[i] != 0;
    *flags = any ? MLA_RANGE_QABS : 0;
  }
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_cache_append_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                    size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || batch > mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  if (q_tokens < 1 || q_tokens > ctx->cfg.max_q_tokens) return MLA_ERR_INVALID_ARG;
  *bytes = mla::append_workspace_bytes(batch * q_tokens);
  return MLA_OK;
}

int mla_cache_append(const mla_decode_ctx* ctx, const mla_append_args* a, void* workspace,
                     size_t workspace_bytes, void* stream_handle) {
  if (!ctx || !a) return MLA_ERR_INVALID_ARG;
  if (!a->hidden || !a->w_kv || !a->kv_cache || !a->block_table || !a->seq_lens) return MLA_ERR_INVALID_ARG;
  if (a->batch < 1 || a->batch > mla::kMaxBatch || a->q_tokens < 1 ||
      a->q_tokens > ctx->cfg.max_q_tokens || a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return MLA_ERR_INVALID_ARG;
  if (!(a->rope_base == a->rope_base)) return MLA_ERR_INVALID_ARG;   // NaN
  if (!aligned16(a->hidden) || !aligned16(a->w_kv) || !aligned16(a->kv_cache) ||
      !aligned16(a->block_table) || !aligned16(a->seq_lens))
    return MLA_ERR_MISALIGNED;
  const size_t need = mla::append_workspace_bytes(a->batch * a->q_tokens);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return MLA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  MLA_DEBUG_CHECK(a->seq_lens, a->block_table, a->batch, a->q_tokens, a->max_blocks_per_seq,
                  (int)std::min<long long>((long long)mla::kBlock * a->max_blocks_per_seq, 0x7fffffff),
                  a->num_blocks, stream);
  const double base = a->rope_base > 0.f ? (double)a->rope_base : 10000.0;
  const int status =
      mla::launch_append((const uint16_t*)a->hidden, (const uint16_t*)a->w_kv, (uint16_t*)a->kv_cache,
                         a->block_table, a->seq_lens, a->num_blocks, a->max_blocks_per_seq, a->batch,
                         a->q_tokens, base, workspace, stream) == hipSuccess
          ? MLA_OK
          : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_query_project_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                     size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || batch > mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  if (q_tokens < 1 || q_tokens > ctx->cfg.max_q_tokens) return MLA_ERR_INVALID_ARG;
  *bytes = mla::qproj_workspace_bytes(batch * q_tokens);
  return MLA_OK;
}

int mla_query_project(const mla_decode_ctx* ctx, const mla_query_args* a, void* workspace,
                      size_t workspace_bytes, void* stream_handle) {
  if (!ctx || !a || !a->hidden || !a->w_dq || !a->w_uq || !a->seq_lens || !a->q_nope || !a->q_pe)
    return MLA_ERR_INVALID_ARG;
  if (a->batch < 1 || a->batch > mla::kMaxBatch || a->q_tokens < 1 ||
      a->q_tokens > ctx->cfg.max_q_tokens)
    return MLA_ERR_INVALID_ARG;
  if (!(a->rope_base == a->rope_base)) return MLA_ERR_INVALID_ARG;   // NaN
  if (!aligned16(a->hidden) || !aligned16(a->w_dq) || !aligned16(a->w_uq) ||
      !aligned16(a->seq_lens) || !aligned16(a->q_nope) || !aligned16(a->q_pe))
    return MLA_ERR_MISALIGNED;
  const size_t need = mla::qproj_workspace_bytes(a->batch * a->q_tokens);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  const double base = a->rope_base > 0.f ? (double)a->rope_base : 10000.0;
  const int status =
      mla::launch_qproj((const uint16_t*)a->hidden, (const uint16_t*)a->w_dq,
                        (const uint16_t*)a->w_uq, a->seq_lens, (uint16_t*)a->q_nope,
                        (uint16_t*)a->q_pe, a->batch, a->q_tokens, base, workspace, stream) == hipSuccess
          ? MLA_OK
          : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_project_new_tokens_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                          size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || batch > mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  if (q_tokens < 1 || q_tokens > ctx->cfg.max_q_tokens) return MLA_ERR_INVALID_ARG;
  *bytes = mla::prologue_workspace_bytes(batch * q_tokens);
  return MLA_OK;
}

int mla_project_new_tokens(const mla_decode_ctx* ctx, const mla_prologue_args* a, void* workspace,
                           size_t workspace_bytes, void* stream_handle) {
  if (!ctx || !a || !a->hidden || !a->w_dq || !a->w_uq || !a->w_kv || !a->kv_cache || !a->block_table ||
      !a->seq_lens || !a->q_nope || !a->q_pe)
    return MLA_ERR_INVALID_ARG;
  if (a->batch < 1 || a->batch > mla::kMaxBatch || a->q_tokens < 1 || a->q_tokens > ctx->cfg.max_q_tokens ||
      a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return MLA_ERR_INVALID_ARG;
  if (!(a->rope_base == a->rope_base)) return MLA_ERR_INVALID_ARG;   // NaN
  if (!aligned16(a->hidden) || !aligned16(a->w_dq) || !aligned16(a->w_uq) || !aligned16(a->w_kv) ||
      !aligned16(a->kv_cache) || !aligned16(a->block_table) || !aligned16(a->seq_lens) || !aligned16(a->q_nope) ||
      !aligned16(a->q_pe))
    return MLA_ERR_MISALIGNED;
  const size_t need = mla::prologue_workspace_bytes(a->batch * a->q_tokens);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  const double base = a->rope_base > 0.f ? (double)a->rope_base : 10000.0;
  const int status =
      mla::launch_prologue((const uint16_t*)a->hidden, (const uint16_t*)a->w_dq, (const uint16_t*)a->w_uq,
                           (const uint16_t*)a->w_kv, (uint16_t*)a->kv_cache, a->block_table, a->seq_lens,
                           a->num_blocks, a->max_blocks_per_seq, (uint16_t*)a->q_nope, (uint16_t*)a->q_pe,
                           a->batch, a->q_tokens, base, workspace, stream) == hipSuccess
          ? MLA_OK
          : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_output_project_workspace_size(const mla_decode_ctx* ctx, int32_t rows, size_t* bytes) {
  if (!ctx || !bytes || rows < 1 || rows > 2 * mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  *bytes = mla::oproj_workspace_bytes(rows);
  return MLA_OK;
}

int mla_output_project(const mla_decode_ctx* ctx, const mla_oproj_args* a, void* workspace,
                       size_t workspace_bytes, void* stream_handle) {
  if (!ctx || !a || !a->x || !a->w_o || !a->y) return MLA_ERR_INVALID_ARG;
  if (a->rows < 1 || a->rows > 2 * mla::kMaxBatch) return MLA_ERR_INVALID_ARG;
  if (!aligned16(a->x) || !aligned16(a->w_o) || !aligned16(a->y)) return MLA_ERR_MISALIGNED;
  const size_t need = mla::oproj_workspace_bytes(a->rows);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  const int status =
      mla::launch_oproj(a->x, (const uint16_t*)a->w_o, a->y, a->rows, workspace, stream) == hipSuccess
          ? MLA_OK
          : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_pack_weight(const mla_decode_ctx* ctx, const void* w, void* packed, int32_t n, int32_t k,
                    void* stream_handle) {
  if (!ctx || !w || !packed) return MLA_ERR_INVALID_ARG;
  if (n < 32 || k < 16 || n % 32 || k % 16 || (long long)n * k > (1LL << 33)) return MLA_ERR_INVALID_ARG;
  const uintptr_t wb = (uintptr_t)w, pb = (uintptr_t)packed, nb = (uintptr_t)n * (uintptr_t)k * 2u;
  if (wb < pb + nb && pb < wb + nb) return MLA_ERR_INVALID_ARG;   // overlapping buffers
  if (!aligned16(w) || !aligned16(packed)) return MLA_ERR_MISALIGNED;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  const int status =
      mla::launch_pack_weight((const uint16_t*)w, (uint16_t*)packed, n, k, stream) == hipSuccess ? MLA_OK
                                                                                                 : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

int mla_naive_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t max_seq_len, size_t* bytes) {
  if (!ctx || !bytes || batch < 1 || batch > mla::kMaxBatch || max_seq_len < 1 || max_seq_len > kMaxNaiveLen)
    return MLA_ERR_INVALID_ARG;
  *bytes = mla::naive_workspace_bytes(batch, max_seq_len);
  return MLA_OK;
}

int mla_naive_run(const mla_decode_ctx* ctx, const mla_naive_args* a, void* workspace, size_t workspace_bytes,
                  void* stream_handle) {
  if (!ctx || !a || !a->q_nope || !a->q_pe || !a->w_uk || !a->w_uv || !a->kv_cache || !a->block_table ||
      !a->seq_lens || !a->out)
    return MLA_ERR_INVALID_ARG;
  if (a->batch < 1 || a->batch > mla::kMaxBatch || a->max_seq_len < 1 || a->max_seq_len > kMaxNaiveLen ||
      a->q_tokens < 1 || a->q_tokens > a->max_seq_len || a->num_blocks < 1 || a->max_blocks_per_seq < 1 ||
      (long long)a->max_blocks_per_seq * mla::kBlock < a->max_seq_len)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(a->q_nope) || !aligned16(a->q_pe) || !aligned16(a->w_uk) || !aligned16(a->w_uv) ||
      !aligned16(a->kv_cache) || !aligned16(a->block_table) || !aligned16(a->seq_lens) || !aligned16(a->out))
    return MLA_ERR_MISALIGNED;
  const size_t need = mla::naive_workspace_bytes(a->batch, a->max_seq_len);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_handle;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
  if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return MLA_ERR_HIP;
  MLA_DEBUG_CHECK(a->seq_lens, a->block_table, a->batch, a->q_tokens, a->max_blocks_per_seq, a->max_seq_len,
                  a->num_blocks, stream);
  const int status =
      mla::launch_naive((const uint16_t*)a->q_nope, (const uint16_t*)a->q_pe, (const uint16_t*)a->w_uk,
                        (const uint16_t*)a->w_uv, (const uint16_t*)a->kv_cache, a->block_table, a->seq_lens, a->out,
                        a->num_blocks, a->batch, a->q_tokens, a->max_blocks_per_seq, a->max_seq_len,
                        ctx->scale, workspace, stream) == hipSuccess
          ? MLA_OK
          : MLA_ERR_HIP;
  if (prev != ctx->device) (void)hipSetDevice(prev);
  return status;
}

void mla_decode_destroy(mla_decode_ctx* ctx) { delete ctx; }

}  // extern "C"
