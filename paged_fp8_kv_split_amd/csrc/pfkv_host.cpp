// C ABI of libpfkv (declared in include/pfkv.h): argument validation, the
// segment-count heuristic, device-property caching and the two launches.
//
// The call mirrors mtp_verify_attn_fwd(...) / mtp_verify_attn_fwd_asm(...) and
// mtp_verify_attn_num_segments() of aiter PR #5190 ("gfx950 assembly MTP-verify
// attention for head_dim 256 fp8 paged KV"), section Modifications; what is
// accepted follows its section Supported (gfx950, head_dim 256, page 16, e4m3
// per-tensor K/V, bf16 Q, GQA 16 or 8; this library adds GQA 4 and 32) with
// q_len 1..4 per sequence as in SGLang PR #37465, Modifications. Unsupported
// shapes return PFKV_UNSUPPORTED so that a caller can fall back, as the SGLang
// entry points do.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pfkv.h"
#include "pfkv_internal.h"
#include "pfkv_prefill.h"
#include "prefill_config.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

struct DeviceProps {
  bool valid = false;
  std::string arch;
  int num_cus = 0;
};

std::mutex g_props_mu;
std::vector<DeviceProps> g_props;

int cached_props(int device, DeviceProps* out) {
  std::lock_guard<std::mutex> lock(g_props_mu);
  if (device < 0) return fail(PFKV_INVALID, "negative device index");
  if ((size_t)device >= g_props.size()) g_props.resize(device + 1);
  DeviceProps& d = g_props[device];
  if (!d.valid) {
    hipDeviceProp_t prop;
    const hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PFKV_LAUNCH, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    }
    d.arch = prop.gcnArchName;
    d.num_cus = prop.multiProcessorCount;
    d.valid = true;
  }
  *out = d;
  return PFKV_OK;
}

// Debug mode (PFKV_DEBUG=1 in the environment, or pfkv_set_debug): a checking
// kernel validates the device-side inputs before every main-kernel launch. It
// synchronizes the stream and keeps a 16-byte status buffer per device, so it
// is not for graph capture.
std::mutex g_debug_mu;
int g_debug = -1;   // -1: not read from the environment yet
std::vector<int32_t*> g_debug_status;

bool debug_enabled() {
  std::lock_guard<std::mutex> lock(g_debug_mu);
  if (g_debug < 0) {
    const char* e = std::getenv("PFKV_DEBUG");
    g_debug = (e != nullptr && std::strcmp(e, "1") == 0) ? 1 : 0;
  }
  return g_debug == 1;
}

int debug_check(const pfkv_args* a, void* stream) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  int32_t* status = nullptr;
  if (e == hipSuccess) {
    std::lock_guard<std::mutex> lock(g_debug_mu);
    if ((size_t)device >= g_debug_status.size()) g_debug_status.resize(device + 1, nullptr);
    if (g_debug_status[device] == nullptr) e = hipMalloc((void**)&g_debug_status[device], 4 * sizeof(int32_t));
    status = g_debug_status[device];
  }
  const int32_t init[4] = {0, INT32_MAX, 0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(status, init, sizeof(init), hipMemcpyHostToDevice, (hipStream_t)stream);
  pfkv::CheckParams c;
  c.cu_seqlens_q = a->cu_seqlens_q;
  c.seq_lens = a->seq_lens;
  c.block_tables = a->block_tables;
  c.block_table_stride = a->block_table_stride;
  c.num_seqs = a->num_seqs;
  c.total_q = a->total_q;
  c.max_q_len = a->max_q_len > 0 ? a->max_q_len : pfkv::kDefaultMaxQLen;
  c.page_size = a->page_size;
  c.max_pages_per_seq = a->max_pages_per_seq;
  c.num_pages = a->num_pages;
  if (e == hipSuccess) e = pfkv::launch_precondition_check(c, status, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  int32_t got[4] = {0, 0, 0, 0};
  if (e == hipSuccess) e = hipMemcpy(got, status, sizeof(got), hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("debug check: ") + hipGetErrorString(e));
  }
  if (got[0] == 0) return PFKV_OK;
  std::string msg = "debug check: sequence " + std::to_string(got[1]) + " (value " + std::to_string(got[2]) + "):";
  if (got[0] & 1) msg += " cu_seqlens_q does not start at 0, decreases, or does not end at total_q;";
  if (got[0] & 2) msg += " more query tokens than max_q_len;";
  if (got[0] & 4) msg += " seq_len below its query tokens or above page_size * max_pages_per_seq;";
  if (got[0] & 8) msg += " block-table entry outside [0, num_pages);";
  return fail(PFKV_INVALID, msg);
}

bool is_gfx950(const char* arch) {
  return std::strncmp(arch, "gfx950", 6) == 0 && (arch[6] == '\0' || arch[6] == ':');
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Pointers already found to be device memory of a device, per thread: the
// last kCheckedSlots distinct (pointer, device) pairs. A serving loop that
// passes the same buffers every call then makes no pointer queries (each costs
// about a microsecond on the host). A buffer freed after a call and passed
// again is not queried again; freed memory is the caller's error either way.
constexpr int kCheckedSlots = 32;
struct CheckedPointer {
  const void* ptr;
  int device;
};
thread_local CheckedPointer g_checked[kCheckedSlots];
thread_local int g_checked_next = 0;

bool already_checked(const void* ptr, int device) {
  for (int i = 0; i < kCheckedSlots; ++i)
    if (g_checked[i].ptr == ptr && g_checked[i].device == device && ptr != nullptr) return true;
  return false;
}

int check_device_pointer(const void* ptr, int device, const char* name) {
  if (already_checked(ptr, device)) return PFKV_OK;
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_DEVICE, std::string(name) + " is not memory known to HIP");
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(PFKV_DEVICE, std::string(name) + " is not device memory");
  if (attr.device != device)
    return fail(PFKV_DEVICE, std::string(name) + " belongs to device " + std::to_string(attr.device) +
                                 ", not the current device " + std::to_string(device));
  g_checked[g_checked_next] = CheckedPointer{ptr, device};
  g_checked_next = (g_checked_next + 1) % kCheckedSlots;
  return PFKV_OK;
}

// Split of a sequence's query heads and tokens over work-groups (blockIdx.z):
// kv_split = 2 when 32 query heads share a KV head; q_split = 2 when 16 query
// heads per work-group meet more than 4 query tokens (a work-group stacks at
// most kMaxRows = 64 query rows).
int kv_split_of(const pfkv_args* a) { return a->num_q_heads / a->num_kv_heads == 32 ? 2 : 1; }
int q_per_wg_of(const pfkv_args* a) {
  const int group = a->num_q_heads / a->num_kv_heads;
  return std::min(pfkv::kMaxRows / (group == 32 ? 16 : group), pfkv::kMaxQLen);
}
int q_split_of(const pfkv_args* a) {
  const int max_q_len = a->max_q_len > 0 ? a->max_q_len : pfkv::kDefaultMaxQLen;
  return (max_q_len + q_per_wg_of(a) - 1) / q_per_wg_of(a);
}
// merge groups (blockIdx.z values) per sequence
uint64_t merge_groups_per_seq(const pfkv_args* a) {
  return (uint64_t)a->num_kv_heads * kv_split_of(a) * q_split_of(a);
}

}  // namespace

extern "C" {

const char* pfkv_last_error(void) { return g_last_error.c_str(); }

int pfkv_num_segments(int num_cus, int num_seqs, int num_kv_heads) {
  if (num_cus <= 0 || num_seqs <= 0 || num_kv_heads <= 0) return 0;
  const long long per = (long long)num_seqs * num_kv_heads;
  long long s = num_cus / per;
  if (s < 1) s = 1;
  if (s > pfkv::kMaxSegments) s = pfkv::kMaxSegments;
  return (int)s;
}

uint64_t pfkv_workspace_bytes(int num_segments, int total_q, int num_q_heads) {
  if (num_segments <= 0 || total_q <= 0 || num_q_heads <= 0) return 0;
  return (uint64_t)num_segments * (uint64_t)total_q * (uint64_t)num_q_heads * pfkv::kPartialBytes;
}

int pfkv_partials_row_major(int precision, int head_dim, int page_size, int num_segments) {
  // the instantiations that write row-major partials: 16-bit arithmetic, head
  // dim 256, pages of 16 tokens or more
  const bool pages = page_size == 16 || page_size == 32 || page_size == 64;
  return precision == PFKV_PRECISION_16BIT && head_dim == 256 && pages && num_segments > pfkv::kRowMajorAbove &&
                 num_segments <= pfkv::kMaxBalancedSegments
             ? 1
             : 0;
}

uint64_t pfkv_merge_sync_bytes(int num_seqs, int num_q_heads) {
  // merge groups per sequence: num_kv_heads * kv_split * q_split <= num_q_heads / 4
  if (num_seqs <= 0 || num_q_heads <= 0) return 0;
  const uint64_t groups = (uint64_t)num_seqs * (uint64_t)((num_q_heads + 3) / 4);
  return groups * pfkv::kMergeSyncWords * 4;
}

int pfkv_check_args(const pfkv_args* a, const char* arch, int num_cus) {
  g_last_error.clear();
  if (a == nullptr) return fail(PFKV_INVALID, "args is NULL");
  if (arch == nullptr) return fail(PFKV_INVALID, "arch is NULL");
  if (num_cus <= 0) return fail(PFKV_INVALID, "num_cus must be positive");

  const struct { const void* p; const char* name; } ptrs[] = {
      {a->q, "q"}, {a->k_cache, "k_cache"}, {a->v_cache, "v_cache"}, {a->block_tables, "block_tables"},
      {a->seq_lens, "seq_lens"}, {a->cu_seqlens_q, "cu_seqlens_q"}, {a->k_descale, "k_descale"},
      {a->v_descale, "v_descale"}, {a->workspace, "workspace"}, {a->out, "out"}};
  for (const auto& x : ptrs)
    if (x.p == nullptr) return fail(PFKV_INVALID, std::string(x.name) + " is NULL");

  if (a->num_seqs < 1 || a->num_seqs > (1 << 20)) return fail(PFKV_INVALID, "num_seqs must be in [1, 2^20]");
  if (a->total_q < 1) return fail(PFKV_INVALID, "total_q must be >= 1");
  if (a->balance_segments != 0 && a->balance_segments != 1) return fail(PFKV_INVALID, "balance_segments must be 0 or 1");
  if (a->balance_segments && (a->num_segments < 2 || a->num_seqs > 1024))
    return fail(PFKV_INVALID, "balanced segments need num_segments (the cap) >= 2 and num_seqs <= 1024");
  if (a->max_q_len < 0 || a->max_q_len > pfkv::kMaxQLen)
    return fail(PFKV_INVALID, "max_q_len must be in [0, 8] (0 = 4)");
  const int max_q_len = a->max_q_len > 0 ? a->max_q_len : pfkv::kDefaultMaxQLen;
  if ((int64_t)a->total_q > (int64_t)max_q_len * a->num_seqs)
    return fail(PFKV_INVALID, "total_q exceeds max_q_len query tokens per sequence");
  if (a->num_q_heads < 1 || a->num_kv_heads < 1) return fail(PFKV_INVALID, "head counts must be positive");
  if (a->num_kv_heads > 4096) return fail(PFKV_INVALID, "num_kv_heads must be <= 4096");
  if (a->num_q_heads % a->num_kv_heads != 0) return fail(PFKV_INVALID, "num_q_heads % num_kv_heads != 0");
  if (a->num_pages < 1) return fail(PFKV_INVALID, "num_pages must be >= 1");
  if (a->max_pages_per_seq < 1) return fail(PFKV_INVALID, "max_pages_per_seq must be >= 1");
  if (a->max_pages_per_seq > (1 << 26)) return fail(PFKV_INVALID, "max_pages_per_seq must be <= 2^26");
  if (a->block_table_stride < a->max_pages_per_seq)
    return fail(PFKV_INVALID, "block_table_stride < max_pages_per_seq");
  if (a->num_segments < 1 || a->num_segments > (a->balance_segments == 1 ? pfkv::kMaxBalancedSegments : pfkv::kMaxSegments))
    return fail(PFKV_INVALID, "num_segments must be in [1, 64] (a cap of up to 128 with balanced segments)");
  if (a->precision != PFKV_PRECISION_16BIT && a->precision != PFKV_PRECISION_FP8_P &&
      a->precision != PFKV_PRECISION_FP8)
    return fail(PFKV_INVALID, "precision must be one of PFKV_PRECISION_16BIT, _FP8_P, _FP8");
  if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f))
    return fail(PFKV_INVALID, "softmax_scale must be finite and positive");
  if (!std::isfinite(a->softcap) || a->softcap < 0.f)
    return fail(PFKV_INVALID, "softcap must be finite and >= 0 (0 = off)");
  if (a->q_stride_token <= 0 || a->q_stride_head <= 0 || a->out_stride_token <= 0 || a->out_stride_head <= 0)
    return fail(PFKV_INVALID, "q / out strides must be positive");
  if (a->q_stride_token % 8 || a->q_stride_head % 8 || !aligned(a->q, 16))
    return fail(PFKV_INVALID, "q rows must be 16-byte aligned (strides multiple of 8 elements)");
  {
    // the main kernel addresses a work-group's Q rows (its query tokens, at most
    // max_q_len, times its query heads) with 32-bit byte offsets
    const int64_t group = a->num_q_heads / a->num_kv_heads;
    const int64_t tokens = max_q_len;
    const int64_t span = ((tokens - 1) * a->q_stride_token + (group - 1) * a->q_stride_head + a->head_dim) * 2;
    if (span >= ((int64_t)1 << 32)) return fail(PFKV_INVALID, "q strides too large (a KV head's rows span >= 4 GiB)");
  }
  if (a->out_stride_token % 4 || a->out_stride_head % 4 || !aligned(a->out, 8))
    return fail(PFKV_INVALID, "out rows must be 8-byte aligned (strides multiple of 4 elements)");
  if (!aligned(a->workspace, 16)) return fail(PFKV_INVALID, "workspace must be 16-byte aligned");
  if (!aligned(a->k_cache, 16) || !aligned(a->v_cache, 16))
    return fail(PFKV_INVALID, "k_cache / v_cache must be 16-byte aligned");
  if (!aligned(a->block_tables, 4) || !aligned(a->seq_lens, 4) || !aligned(a->cu_seqlens_q, 4) ||
      !aligned(a->k_descale, 4) || !aligned(a->v_descale, 4) || !aligned(a->lse, 4) || !aligned(a->sinks, 4))
    return fail(PFKV_INVALID, "int32 / fp32 arguments must be 4-byte aligned");
  const uint64_t need = pfkv_workspace_bytes(a->num_segments, a->total_q, a->num_q_heads);
  if (a->workspace_size < need)
    return fail(PFKV_INVALID, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                  std::to_string(a->workspace_size));
  if (a->merge_sync != nullptr) {
    if (!aligned(a->merge_sync, 256)) return fail(PFKV_INVALID, "merge_sync must be 256-byte aligned");
    const uint64_t need_sync = (uint64_t)a->num_seqs * merge_groups_per_seq(a) * pfkv::kMergeSyncWords * 4;
    if (a->merge_sync_size < need_sync)
      return fail(PFKV_INVALID, "merge_sync too small: need " + std::to_string(need_sync) + " bytes, got " +
                                    std::to_string(a->merge_sync_size));
  }
  if (a->merge_wait_us > 100000) return fail(PFKV_INVALID, "merge_wait_us must be <= 100000");

  // Supported envelope of the kernels.
  if (!is_gfx950(arch)) return fail(PFKV_UNSUPPORTED, std::string("device is ") + arch + ", kernels are gfx950");
  if (a->head_dim != 256 && a->head_dim != 128) return fail(PFKV_UNSUPPORTED, "head_dim must be 256 or 128");
  if (a->page_size != 1 && a->page_size != 16 && a->page_size != 32 && a->page_size != 64)
    return fail(PFKV_UNSUPPORTED, "page_size must be 1, 16, 32 or 64");
  if (a->page_size > 1) {
    if ((int64_t)a->max_pages_per_seq * (a->page_size / pfkv::kPageSize) > (1 << 26))
      return fail(PFKV_INVALID, "max_pages_per_seq * page_size / 16 must be <= 2^26");
    if ((int64_t)a->num_pages * (a->page_size / pfkv::kPageSize) > INT32_MAX)
      return fail(PFKV_INVALID, "num_pages * page_size / 16 must fit in int32");
  }
  const int group = a->num_q_heads / a->num_kv_heads;
  if (group != 32 && group != 16 && group != 8 && group != 4)
    return fail(PFKV_UNSUPPORTED, "query heads per KV head must be 32, 16, 8 or 4, got " + std::to_string(group));
  return PFKV_OK;
}

int pfkv_device_info(int device, char* arch, int arch_len, int* num_cus) {
  g_last_error.clear();
  DeviceProps d;
  const int st = cached_props(device, &d);
  if (st != PFKV_OK) return st;
  if (arch != nullptr && arch_len > 0) {
    std::strncpy(arch, d.arch.c_str(), (size_t)arch_len - 1);
    arch[arch_len - 1] = '\0';
  }
  if (num_cus != nullptr) *num_cus = d.num_cus;
  return PFKV_OK;
}

}  // extern "C"

namespace {

// Validation shared by the launch entry points; fills the kernel params.
// library_workspace: the workspace is the library's own device array (the
// allocation-free entry point), which is not memory HIP's pointer query knows.
int prepare(const pfkv_args* a, pfkv::MainParams* mp, pfkv::ReduceParams* rp, bool library_workspace = false) {
  g_last_error.clear();
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
  }
  DeviceProps d;
  int st = cached_props(device, &d);
  if (st != PFKV_OK) return st;
  st = pfkv_check_args(a, d.arch.c_str(), d.num_cus);
  if (st != PFKV_OK) return st;
  const struct { const void* p; const char* name; } ptrs[] = {
      {a->q, "q"}, {a->k_cache, "k_cache"}, {a->v_cache, "v_cache"}, {a->block_tables, "block_tables"},
      {a->seq_lens, "seq_lens"}, {a->cu_seqlens_q, "cu_seqlens_q"}, {a->k_descale, "k_descale"},
      {a->v_descale, "v_descale"}, {a->workspace, "workspace"}, {a->out, "out"}};
  for (const auto& x : ptrs) {
    if (library_workspace && x.p == a->workspace) continue;
    st = check_device_pointer(x.p, device, x.name);
    if (st != PFKV_OK) return st;
  }
  if (a->lse != nullptr) {
    st = check_device_pointer(a->lse, device, "lse");
    if (st != PFKV_OK) return st;
  }
  if (a->sinks != nullptr) {
    st = check_device_pointer(a->sinks, device, "sinks");
    if (st != PFKV_OK) return st;
  }

  const int group = a->num_q_heads / a->num_kv_heads;
  const uint64_t part_rows = (uint64_t)a->num_segments * a->total_q * a->num_q_heads;
  uint16_t* ws_o = (uint16_t*)a->workspace;
  float* ws_ml = (float*)(ws_o + part_rows * pfkv::kHeadDim);

  *mp = pfkv::MainParams();
  *rp = pfkv::ReduceParams();
  pfkv::MainParams& m = *mp;
  m.q = (const uint16_t*)a->q;
  m.q_stride_token = a->q_stride_token;
  m.q_stride_head = a->q_stride_head;
  m.k_cache = (const uint8_t*)a->k_cache;
  m.v_cache = (const uint8_t*)a->v_cache;
  m.block_tables = a->block_tables;
  m.block_table_stride = a->block_table_stride;
  m.seq_lens = a->seq_lens;
  m.cu_seqlens_q = a->cu_seqlens_q;
  m.k_descale = a->k_descale;
  m.ws_o = ws_o;
  m.ws_ml = ws_ml;
  m.out = (uint16_t*)a->out;
  m.out_stride_token = a->out_stride_token;
  m.out_stride_head = a->out_stride_head;
  m.v_descale = a->v_descale;
  m.lse = a->lse;
  m.sinks = a->sinks;
  m.window_left = a->window_keys > 0 ? a->window_keys - 1 : -1;
  m.softcap = a->softcap;
  m.direct = a->num_segments == 1 ? 1 : 0;
  m.kv_split = kv_split_of(a);
  m.q_per_wg = q_per_wg_of(a);
  m.q_split = q_split_of(a);
  m.precision = a->precision;
  m.head_dim = a->head_dim;
  m.num_seqs = a->num_seqs;
  m.total_q = a->total_q;
  m.num_q_heads = a->num_q_heads;
  m.num_kv_heads = a->num_kv_heads;
  m.num_pages = a->num_pages;
  m.page_ratio_log2 = a->page_size == 64 ? 2 : (a->page_size == 32 ? 1 : 0);
  m.token_pages = a->page_size == 1 ? 1 : 0;
  m.max_seq_len = a->max_pages_per_seq * a->page_size;   // <= 2^30 (checked)
  m.num_segments = a->num_segments;
  m.balance = a->balance_segments;
  m.num_slots = 0;
  if (m.balance) {
    // about one work-group per CU: slots x (work-groups per slot along z)
    const int per_slot = a->num_kv_heads * m.kv_split * m.q_split;
    m.num_slots = std::max(a->num_seqs, std::max(1, d.num_cus / per_slot));
  }
  m.score_scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634073599);
  m.ws_row_major = pfkv_partials_row_major(a->precision, a->head_dim, a->page_size, a->num_segments);
  m.merge_sync = nullptr;
  if (a->merge_sync != nullptr) {
    st = check_device_pointer(a->merge_sync, device, "merge_sync");
    if (st != PFKV_OK) return st;
    // every work-group of the grid resident at once (one per CU), so that the
    // waits of a group normally end by its last arrival, not by the time limit
    // (and o partials under 2^31 bytes, the reach of the merge's buffer loads)
    const uint64_t wgs = (uint64_t)a->num_segments * a->num_seqs * merge_groups_per_seq(a);
    if (a->precision == PFKV_PRECISION_16BIT && a->head_dim == 256 && a->page_size >= 16 && !m.balance &&
        a->num_segments >= 2 && wgs <= (uint64_t)d.num_cus && part_rows * pfkv::kHeadDim * 2 < (1ull << 31)) {
      m.merge_sync = (uint32_t*)a->merge_sync;
      m.merge_wait_ticks = a->merge_wait_us == 0 ? pfkv::kMergeWaitTicksDefault
                                                 : (a->merge_wait_us < 0 ? 0u : (uint32_t)a->merge_wait_us * 100u);
    }
  }

  rp->ws_o = ws_o;
  rp->ws_ml = ws_ml;
  rp->v_descale = a->v_descale;
  rp->out = (uint16_t*)a->out;
  rp->out_stride_token = a->out_stride_token;
  rp->out_stride_head = a->out_stride_head;
  rp->lse = a->lse;
  rp->sinks = a->sinks;
  rp->total_q = a->total_q;
  rp->num_q_heads = a->num_q_heads;
  rp->num_segments = a->num_segments;
  rp->head_dim = a->head_dim;
  rp->balance = m.balance;
  rp->num_slots = m.num_slots;
  rp->num_seqs = a->num_seqs;
  rp->window_left = m.window_left;
  rp->max_seq_len = m.max_seq_len;
  rp->seq_lens = a->seq_lens;
  rp->cu_seqlens_q = a->cu_seqlens_q;
  rp->ws_row_major = m.ws_row_major;
  (void)group;
  return PFKV_OK;
}

int launch_main(const pfkv::MainParams& mp, int group, void* stream) {
  // 32 query heads per KV head: two work-groups of 16 per KV head (mp.kv_split)
  const hipError_t e = pfkv::launch_splitkv_main(mp, group == 32 ? 16 : group, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("split-KV main kernel launch: ") + hipGetErrorString(e));
  }
  return PFKV_OK;
}

int launch_reduce(const pfkv::ReduceParams& rp, void* stream) {
  const hipError_t e = pfkv::launch_segment_reduce(rp, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("segment reduce launch: ") + hipGetErrorString(e));
  }
  return PFKV_OK;
}

}  // namespace

namespace pfkv {

// The verify call on a workspace the library owns (ws, ws_bytes): the same
// validation and launches as pfkv_verify_attn_fwd, without the debug check
// (which allocates and synchronizes).
int verify_attn_library_workspace(const pfkv_args* a, void* ws, uint64_t ws_bytes, void* stream) {
  if (a == nullptr) return fail(PFKV_INVALID, "args is NULL");
  pfkv_args b = *a;
  b.workspace = ws;
  b.workspace_size = ws_bytes;
  pfkv::MainParams mp;
  pfkv::ReduceParams rp;
  int st = prepare(&b, &mp, &rp, /*library_workspace=*/true);
  if (st == PFKV_OK) st = launch_main(mp, b.num_q_heads / b.num_kv_heads, stream);
  if (st == PFKV_OK && !mp.direct && mp.merge_sync == nullptr) st = launch_reduce(rp, stream);
  return st;
}

int set_error(int status, const char* msg) { return fail(status, msg); }

}  // namespace pfkv

extern "C" {

int pfkv_set_debug(int on) {
  const int prev = debug_enabled() ? 1 : 0;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  g_debug = on ? 1 : 0;
  return prev;
}

int pfkv_verify_attn_fwd(const pfkv_args* a, void* stream) {
  pfkv::MainParams mp;
  pfkv::ReduceParams rp;
  int st = prepare(a, &mp, &rp);
  if (st == PFKV_OK && debug_enabled()) st = debug_check(a, stream);
  if (st == PFKV_OK) st = launch_main(mp, a->num_q_heads / a->num_kv_heads, stream);
  // one segment, or the merge inside the main launch: out is final
  if (st == PFKV_OK && !mp.direct && mp.merge_sync == nullptr) st = launch_reduce(rp, stream);
  return st;
}

int pfkv_splitkv_main(const pfkv_args* a, void* stream) {
  pfkv::MainParams mp;
  pfkv::ReduceParams rp;
  int st = prepare(a, &mp, &rp);
  mp.merge_sync = nullptr;   // this stage writes the partials only
  if (st == PFKV_OK && debug_enabled()) st = debug_check(a, stream);
  if (st == PFKV_OK) st = launch_main(mp, a->num_q_heads / a->num_kv_heads, stream);
  return st;
}

int pfkv_segment_reduce(const pfkv_args* a, void* stream) {
  pfkv::MainParams mp;
  pfkv::ReduceParams rp;
  int st = prepare(a, &mp, &rp);
  if (st == PFKV_OK && !mp.direct) st = launch_reduce(rp, stream);
  return st;
}

int pfkv_stream_read(const void* buf, uint64_t bytes, int variant, const int32_t* page_order, int64_t num_pages,
                     void* sink, void* stream) {
  g_last_error.clear();
  if (buf == nullptr || sink == nullptr) return fail(PFKV_INVALID, "buf and sink must be non-NULL");
  if (variant < 0 || variant > 3) return fail(PFKV_INVALID, "variant must be 0, 1, 2 or 3");
  if (bytes == 0 || bytes % 4096) return fail(PFKV_INVALID, "bytes must be a positive multiple of 4096");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(PFKV_INVALID, "buf must be 16-byte aligned");
  const bool ordered = variant == 2 || variant == 3;
  if (ordered && (page_order == nullptr || num_pages < 1))
    return fail(PFKV_INVALID, "variants 2 and 3 need a page order");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) {
    int st = check_device_pointer(buf, device, "buf");
    if (st == PFKV_OK) st = check_device_pointer(sink, device, "sink");
    if (st == PFKV_OK && ordered) st = check_device_pointer(page_order, device, "page_order");
    if (st != PFKV_OK) return st;
    e = pfkv::launch_stream_read(buf, bytes, variant, page_order, num_pages, (uint32_t*)sink,
                                 (hipStream_t)stream);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("stream read: ") + hipGetErrorString(e));
  }
  return PFKV_OK;
}

// ---------------------------------------------------------------- prefill
// The second workload (include/pfkv_prefill.h): fp8 varlen prefill attention
// as aiter PR #7375 ("gfx1250 fp8 varlen FMHA") specifies it in its sections
// Summary and Changes (e4m3 q/k/v with single-element fp32 descales on the
// device, qk head dim 192 / v head dim 128, packed THD rows, optional lse
// [Hq, total_q], causal aligned to the bottom right).

int pfkv_prefill_check_args(const pfkv_prefill_args* a, const char* arch, int num_cus) {
  g_last_error.clear();
  if (a == nullptr) return fail(PFKV_INVALID, "args is NULL");
  if (arch == nullptr) return fail(PFKV_INVALID, "arch is NULL");
  if (num_cus <= 0) return fail(PFKV_INVALID, "num_cus must be positive");
  const struct {
    const void* p;
    const char* name;
  } ptrs[] = {{a->q, "q"}, {a->k, "k"}, {a->v, "v"}, {a->out, "out"}, {a->cu_seqlens_q, "cu_seqlens_q"},
              {a->cu_seqlens_k, "cu_seqlens_k"}, {a->q_descale, "q_descale"}, {a->k_descale, "k_descale"},
              {a->v_descale, "v_descale"}};
  for (const auto& x : ptrs)
    if (x.p == nullptr) return fail(PFKV_INVALID, std::string(x.name) + " is NULL");
  if (a->num_seqs < 1 || a->num_seqs > 65535) return fail(PFKV_INVALID, "num_seqs must be in [1, 65535]");
  if (a->total_q < 1) return fail(PFKV_INVALID, "total_q must be >= 1");
  if (a->total_k < 0) return fail(PFKV_INVALID, "total_k must be >= 0");
  if (a->num_q_heads < 1 || a->num_q_heads > 65535 || a->num_kv_heads < 1)
    return fail(PFKV_INVALID, "head counts must be positive (num_q_heads <= 65535)");
  if (a->num_q_heads % a->num_kv_heads != 0) return fail(PFKV_INVALID, "num_q_heads % num_kv_heads != 0");
  if (a->max_seqlen_q < 1 || a->max_seqlen_q > (1 << 30)) return fail(PFKV_INVALID, "max_seqlen_q must be in [1, 2^30]");
  // the kernel numbers a sequence's (query tile, head) work-groups in 32 bits
  const int64_t tiles = ((int64_t)a->max_seqlen_q + pfkv::kPrefillTileRows - 1) / pfkv::kPrefillTileRows;
  if (tiles * a->num_q_heads > INT32_MAX)
    return fail(PFKV_INVALID, "ceil(max_seqlen_q / 256) * num_q_heads must be below 2^31");
  if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f))
    return fail(PFKV_INVALID, "softmax_scale must be finite and positive");
  const int64_t byte_strides[] = {a->q_stride_token, a->q_stride_head, a->k_stride_token,
                                  a->k_stride_head,  a->v_stride_token, a->v_stride_head};
  for (int64_t st : byte_strides)
    if (st <= 0 || st % 16) return fail(PFKV_INVALID, "q / k / v strides must be positive multiples of 16 bytes");
  if (a->out_stride_token <= 0 || a->out_stride_head <= 0 || a->out_stride_token % 4 || a->out_stride_head % 4)
    return fail(PFKV_INVALID, "out strides must be positive multiples of 4 elements");
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16))
    return fail(PFKV_INVALID, "q / k / v must be 16-byte aligned");
  if (!aligned(a->out, 8)) return fail(PFKV_INVALID, "out must be 8-byte aligned");
  if (!aligned(a->cu_seqlens_q, 4) || !aligned(a->cu_seqlens_k, 4) || !aligned(a->q_descale, 4) ||
      !aligned(a->k_descale, 4) || !aligned(a->v_descale, 4) || !aligned(a->lse, 4))
    return fail(PFKV_INVALID, "int32 / fp32 arguments must be 4-byte aligned");
  if (!is_gfx950(arch)) return fail(PFKV_UNSUPPORTED, std::string("device is ") + arch + ", kernels are gfx950");
  if (a->head_dim_qk != 192 || a->head_dim_v != 128)
    return fail(PFKV_UNSUPPORTED, "head dims must be 192 (q, k) and 128 (v)");
  return PFKV_OK;
}

int pfkv_prefill_fwd(const pfkv_prefill_args* a, void* stream) {
  g_last_error.clear();
  if (a == nullptr) return fail(PFKV_INVALID, "args is NULL");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("hipGetDevice: ") + hipGetErrorString(e));
  }
  DeviceProps d;
  int st = cached_props(device, &d);
  if (st != PFKV_OK) return st;
  st = pfkv_prefill_check_args(a, d.arch.c_str(), d.num_cus);
  if (st != PFKV_OK) return st;
  const struct {
    const void* p;
    const char* name;
  } ptrs[] = {{a->q, "q"}, {a->k, "k"}, {a->v, "v"}, {a->out, "out"}, {a->cu_seqlens_q, "cu_seqlens_q"},
              {a->cu_seqlens_k, "cu_seqlens_k"}, {a->q_descale, "q_descale"}, {a->k_descale, "k_descale"},
              {a->v_descale, "v_descale"}, {a->lse, "lse"}};
  for (const auto& x : ptrs) {
    if (x.p == nullptr) continue;   // only lse may be NULL here
    st = check_device_pointer(x.p, device, x.name);
    if (st != PFKV_OK) return st;
  }
  pfkv::PrefillParams p;
  p.q = (const uint8_t*)a->q;
  p.q_stride_token = a->q_stride_token;
  p.q_stride_head = a->q_stride_head;
  p.k = (const uint8_t*)a->k;
  p.k_stride_token = a->k_stride_token;
  p.k_stride_head = a->k_stride_head;
  p.v = (const uint8_t*)a->v;
  p.v_stride_token = a->v_stride_token;
  p.v_stride_head = a->v_stride_head;
  p.out = (uint16_t*)a->out;
  p.out_stride_token = a->out_stride_token;
  p.out_stride_head = a->out_stride_head;
  p.lse = a->lse;
  p.cu_seqlens_q = a->cu_seqlens_q;
  p.cu_seqlens_k = a->cu_seqlens_k;
  p.q_descale = a->q_descale;
  p.k_descale = a->k_descale;
  p.v_descale = a->v_descale;
  p.num_seqs = a->num_seqs;
  p.total_q = a->total_q;
  p.total_k = a->total_k;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.max_seqlen_q = a->max_seqlen_q;
  p.scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634073599);
  p.causal = a->causal != 0 ? 1 : 0;
  e = pfkv::launch_prefill(p, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PFKV_LAUNCH, std::string("prefill launch: ") + hipGetErrorString(e));
  }
  return PFKV_OK;
}

}  // extern "C"
