// C-ABI layer of libmla355: descriptor validation (host only, before any HIP call),
// per-(device, stream) workspace, and kernel launches.  See include/mla355.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/mla355.h"
#include "mla_kernels.h"

namespace {

thread_local char g_msg[512] = "";

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

mla_status ok() {
  g_msg[0] = 0;
  return MLA_OK;
}

size_t dtype_size(int32_t d) {
  switch (d) {
    case MLA_DTYPE_BF16: return 2;
    case MLA_DTYPE_FP8_E4M3: return 1;
    case MLA_DTYPE_F32:
    case MLA_DTYPE_I32:
    case MLA_DTYPE_U32: return 4;
    default: return 0;
  }
}

// Checks a descriptor: non-null, dtype, rank, inner stride 1, outer strides and base
// 16-byte aligned when `aligned16`.
mla_status check_tensor(const mla_tensor* t, const char* name, int32_t dtype, int32_t ndim,
                        bool aligned16) {
  if (!t) return fail(MLA_ERR_NULL_ARG, "%s: descriptor is NULL", name);
  if (t->dtype != dtype) return fail(MLA_ERR_DTYPE, "%s: dtype %d, expected %d", name, t->dtype, dtype);
  if (t->ndim != ndim) return fail(MLA_ERR_SHAPE, "%s: rank %d, expected %d", name, t->ndim, ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(MLA_ERR_SHAPE, "%s: negative extent in dim %d", name, i);
  bool empty = false;
  for (int i = 0; i < ndim; ++i) empty |= t->shape[i] == 0;
  if (!t->data && !empty) return fail(MLA_ERR_NULL_ARG, "%s: data pointer is NULL", name);
  if (empty) return MLA_OK;  // no element is ever addressed: strides and alignment do not matter
  if (t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1)
    return fail(MLA_ERR_SHAPE, "%s: innermost dimension must be contiguous", name);
  const size_t es = dtype_size(dtype);
  if (aligned16) {
    if ((uintptr_t)t->data % 16) return fail(MLA_ERR_ALIGNMENT, "%s: base pointer not 16-byte aligned", name);
    for (int i = 0; i < ndim - 1; ++i)
      if (t->shape[i] > 1 && ((size_t)t->stride[i] * es) % 16)
        return fail(MLA_ERR_ALIGNMENT, "%s: stride of dim %d not a multiple of 16 bytes", name, i);
  } else if ((uintptr_t)t->data % es) {
    return fail(MLA_ERR_ALIGNMENT, "%s: base pointer not element aligned", name);
  }
  for (int i = 0; i < ndim - 1; ++i)
    if (t->shape[i] > 1 && t->stride[i] < 0) return fail(MLA_ERR_SHAPE, "%s: negative stride", name);
  return MLA_OK;
}

mla_status check_1d(const mla_tensor* t, const char* name, int32_t dtype, int64_t n) {
  mla_status s = check_tensor(t, name, dtype, 1, false);
  if (s != MLA_OK) return s;
  if (t->shape[0] != n) return fail(MLA_ERR_SHAPE, "%s: length %lld, expected %lld", name, (long long)t->shape[0], (long long)n);
  return MLA_OK;
}

bool supported_heads(int64_t h) { return h == 16 || h == 32 || h == 64 || h == 128; }

// ---------------------------------------------------------------------------------------
// workspace: one grow-only buffer per (device, stream)
// ---------------------------------------------------------------------------------------
constexpr size_t kZeroRowBytes = 4096;  // the zero row (>= 1152 bytes) and the error word
constexpr size_t kErrOffset = mla::kHdrErrOffset;
constexpr size_t kHeaderBytes = kZeroRowBytes;
constexpr int64_t kMaxRows = (int64_t)1 << 24;

struct Workspace {
  void* base = nullptr;
  size_t bytes = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;
// Outgrown workspaces, kept until mla_shutdown: a graph captured earlier may still hold
// their addresses, so they are never freed while the library is in use.
std::vector<std::pair<int, void*>> g_ws_retired;
std::map<int, int> g_cu_count;

int current_device() {
  int d = 0;
  (void)hipGetDevice(&d);
  return d;
}

int cu_count(int device) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto it = g_cu_count.find(device);
  if (it != g_cu_count.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) n = 256;
  g_cu_count[device] = n;
  return n;
}

mla_status grow_workspace(int device, void* stream, size_t need, bool capturing, void** out_base) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& w = g_ws[{device, stream}];
  need += kHeaderBytes;
  if (w.bytes >= need) {
    *out_base = w.base;
    return MLA_OK;
  }
  if (capturing)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed while the stream is capturing; reserve it first", need);
  size_t bytes = need + need / 4;  // headroom so slowly growing calls do not reallocate
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) return fail(MLA_ERR_WORKSPACE, "hipMalloc(%zu) failed", bytes);
  // the zero row and the error word must start cleared; the rest needs no initial value
  const float one = 1.f;
  if (hipMemset(p, 0, kHeaderBytes) != hipSuccess ||
      hipMemcpy((char*)p + mla::kSparseOneOffset, &one, sizeof(one), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(MLA_ERR_HIP, "initialising the workspace header failed");
  }
  if (w.base) {
    // The old buffer is retired, not freed (graphs captured on this stream may still
    // replay into it).  Its error word carries over once the stream's work has finished.
    uint32_t flags = 0;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
        hipMemcpy(&flags, (char*)w.base + kErrOffset, 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy((char*)p + kErrOffset, &flags, 4, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(p);
      return fail(MLA_ERR_HIP, "could not move the device error word to the grown workspace");
    }
    g_ws_retired.emplace_back(device, w.base);
  }
  w.base = p;
  w.bytes = bytes;
  *out_base = p;
  return MLA_OK;
}

mla_status stream_capturing(void* stream, bool* capturing) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &st) != hipSuccess)
    return fail(MLA_ERR_HIP, "hipStreamIsCapturing failed");
  *capturing = st != hipStreamCaptureStatusNone;
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The most pieces the balanced split of the decode kernels (mla_plan.h) cuts one query row
// into, for `batch` rows of `keys` visible keys each over `grid` work-groups.  Row parts
// (batch <= grid): the smallest S with batch * ceil(nt / S) <= grid tiles per part, nt the
// row's 32-key tiles, so ceil(nt / S) parts; stream (batch > grid): runs of
// ceil(batch * nt / grid) tiles over the concatenated rows, the most runs one row meets.
int32_t balanced_parts_per_row(int64_t batch, int64_t keys, int grid) {
  const int64_t nt = (keys + 31) / 32;
  if (batch <= grid) {
    const int64_t per_row = grid / batch;  // parts every row may have
    const int64_t S = (nt + per_row - 1) / per_row;
    return (int32_t)((nt + S - 1) / S);
  }
  const int64_t W = (batch * nt + grid - 1) / grid;
  int64_t most = 1;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t first = b * nt / W, last = ((b + 1) * nt - 1) / W;
    if (last - first + 1 > most) most = last - first + 1;
  }
  return (int32_t)most;
}

// ---------------------------------------------------------------------------------------
// optional kernel timing: a ring of event pairs created when timing is enabled, so that
// no call creates an event (event creation on the call path would delay the host enough
// for the GPU to drain its queue, and the gaps would be timed as kernel time)
// ---------------------------------------------------------------------------------------
constexpr int kProfileSlots = 4096;
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<mla::KernelTimer> g_prof_ring;  // created by mla_profile_enable
std::vector<char> g_prof_live;              // slot i was recorded by a launch
int64_t g_prof_used = 0;                    // slots handed out since the last read
int64_t g_prof_dropped = 0;                 // launches past the ring's capacity (not timed)

// Reserves the next timer of the ring (copied into *slot, its index in *index), or
// returns null when timing is off or the ring is full.
mla::KernelTimer* profile_timer(mla::KernelTimer* slot, int64_t* index) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_ring.empty()) return nullptr;
  if (g_prof_used >= (int64_t)g_prof_ring.size()) {
    ++g_prof_dropped;
    return nullptr;
  }
  *index = g_prof_used++;
  *slot = g_prof_ring[(size_t)*index];
  g_prof_live[(size_t)*index] = 0;
  return slot;
}

void profile_keep(mla::KernelTimer* t, int64_t index, bool launched) {
  if (!t || !launched) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (index >= 0 && index < (int64_t)g_prof_live.size()) g_prof_live[(size_t)index] = 1;
}

void profile_destroy_ring() {
  for (auto& t : g_prof_ring) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_prof_ring.clear();
  g_prof_live.clear();
  g_prof_used = 0;
  g_prof_dropped = 0;
}

// Past the header: the split rows' parts (bf16), their log2-sum-exps and the split table.
struct DecodeLayout {
  size_t part_o, part_lse, meta, total;
};

DecodeLayout decode_layout(int64_t T, int32_t H, int32_t nparts, int32_t grid) {
  const size_t slots = mla::decode_slots(T, nparts, grid);
  DecodeLayout L;
  L.part_o = 0;
  L.part_lse = align256(slots * (size_t)H * 512 * sizeof(uint16_t));
  L.meta = L.part_lse + align256(slots * (size_t)H * sizeof(float));
  L.total = L.meta + align256((2 + 2 * (size_t)T) * sizeof(int32_t));
  return L;
}

// ---------------------------------------------------------------------------------------
// No-allocation variant: the dense decode's workspace in a fixed array of device memory
// (per GPU, for the life of the process), for callers that cannot allocate (graph
// capture, serving loops that forbid hipMalloc).  Its layout is the stream workspace's:
// the header (zero row, error word) and then the split parts.  The limit covers the
// balanced split of up to 128 heads over up to 256 compute units (512 part slots of
// 128 x 512 bf16) and the split table of up to 2^16 query rows.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = ((size_t)65 << 20) + ((size_t)1 << 19);  // 65.5 MiB
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void scratch_header_init(uint8_t* base) {
  // the zero row and the error word start cleared
  for (int i = threadIdx.x; i < (int)(kHeaderBytes / 16); i += blockDim.x)
    reinterpret_cast<uint4*>(base)[i] = make_uint4(0, 0, 0, 0);
}

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device address of `scratch` on each device
std::map<int, bool> g_scratch_ready; // header cleared (by a call outside capture)

// The device address of this device's scratch array, its header cleared before any work
// the caller queues next on `stream`.
mla_status scratch_base(int device, void* stream, bool capturing, void** base) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(device);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
    it = g_scratch_ptr.emplace(device, ptr).first;
  }
  if (!g_scratch_ready[device]) {
    // a kernel, not a memset: the clear may be captured into a graph
    hipLaunchKernelGGL(scratch_header_init, dim3(1), dim3(256), 0, (hipStream_t)stream, (uint8_t*)it->second);
    if (hipGetLastError() != hipSuccess) return fail(MLA_ERR_HIP, "clearing the scratch header failed");
    if (!capturing) {
      if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return fail(MLA_ERR_HIP, "clearing the scratch header failed");
      g_scratch_ready[device] = true;
    }
  }
  *base = it->second;
  return MLA_OK;
}

}  // namespace

namespace mla {
size_t decode_workspace_bytes(int64_t T, int32_t H, int32_t nparts, int32_t grid) {
  return decode_layout(T, H, nparts, grid).total;
}
}  // namespace mla

extern "C" {

const char* mla_version(void) { return "libmla355 0.1 (gfx950)"; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "null argument";
    case MLA_ERR_SHAPE: return "shape mismatch";
    case MLA_ERR_DTYPE: return "wrong element type";
    case MLA_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace unavailable";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_VALUE: return "scalar argument out of range";
  }
  return "unknown status";
}

const char* mla_last_error_message(void) { return g_msg; }

// The indexer's workspace past the header: the keys [T, keys_row], then the run tables
// [T, hist_row].
struct IndexerLayout {
  int64_t keys_row, hist_row;
  size_t key_bytes, total;
};
static IndexerLayout indexer_layout(int64_t T, int64_t max_pages, int64_t PS) {
  IndexerLayout L;
  L.keys_row = (max_pages * PS + 1) & ~(int64_t)1;  // even: every key slice starts 16-byte aligned
  L.hist_row = 512 * ((L.keys_row + mla::kIdxSlice - 1) / mla::kIdxSlice);
  L.key_bytes = (size_t)(T * L.keys_row) * sizeof(uint64_t);
  L.total = L.key_bytes + (size_t)(T * L.hist_row) * sizeof(uint32_t);
  return L;
}

size_t mla_indexer_workspace_bytes(int64_t total_q, int32_t max_pages, int32_t page_size) {
  if (total_q < 0 || max_pages < 0 || page_size < 0) return 0;
  return indexer_layout(total_q, max_pages, page_size).total + kHeaderBytes;
}

size_t mla_decode_workspace_bytes(int64_t total_q, int32_t num_heads, int32_t num_partitions, int32_t device) {
  const int dev = device < 0 ? current_device() : device;
  const int grid = cu_count(dev);
  return decode_layout(total_q, num_heads, num_partitions > 0 ? num_partitions : 0, grid).total + kHeaderBytes;
}

mla_status mla_reserve_workspace(int32_t device, void* stream, size_t bytes) {
  const int dev = device < 0 ? current_device() : device;
  bool cap = false;
  mla_status s = stream_capturing(stream, &cap);
  if (s != MLA_OK) return s;
  if (cap) return fail(MLA_ERR_WORKSPACE, "cannot reserve workspace while the stream is capturing");
  void* base = nullptr;
  const size_t need = bytes > kHeaderBytes ? bytes - kHeaderBytes : 0;
  s = grow_workspace(dev, stream, need, false, &base);
  return s == MLA_OK ? ok() : s;
}

mla_status mla_check_device_errors(int32_t device, void* stream, uint32_t* flags) {
  if (!flags) return fail(MLA_ERR_NULL_ARG, "flags is NULL");
  *flags = 0;
  const int dev = device < 0 ? current_device() : device;
  // the stream's workspace and, when the no-allocation decode has run on this device, the
  // scratch array's header
  std::vector<void*> words;
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws.find({dev, stream});
    if (it != g_ws.end()) words.push_back((char*)it->second.base + kErrOffset);
  }
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end() && g_scratch_ready[dev]) words.push_back((char*)it->second + kErrOffset);
  }
  if (words.empty()) return ok();
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return fail(MLA_ERR_HIP, "reading the device error word failed");
  const uint32_t zero = 0;
  for (void* w : words) {
    uint32_t v = 0;
    if (hipMemcpy(&v, w, 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(w, &zero, 4, hipMemcpyHostToDevice) != hipSuccess)
      return fail(MLA_ERR_HIP, "reading the device error word failed");
    *flags |= v;
  }
  return ok();
}

size_t mla_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

mla_status mla_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  if (g_prof_on && g_prof_ring.empty()) {
    std::vector<mla::KernelTimer> ring;
    ring.reserve(kProfileSlots);
    for (int i = 0; i < kProfileSlots; ++i) {
      mla::KernelTimer t;
      if (hipEventCreate(&t.start) != hipSuccess) break;
      if (hipEventCreate(&t.stop) != hipSuccess) {
        (void)hipEventDestroy(t.start);
        break;
      }
      ring.push_back(t);
    }
    if ((int)ring.size() != kProfileSlots) {
      for (auto& t : ring) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
      }
      g_prof_on = false;
      return fail(MLA_ERR_HIP, "creating the timing events failed");
    }
    g_prof_ring.swap(ring);
    g_prof_live.assign(kProfileSlots, 0);
  }
  g_prof_used = 0;
  g_prof_dropped = 0;
  return ok();
}

mla_status mla_profile_read_each(double* ms_each, int64_t capacity, int64_t* launches) {
  if (!launches || (capacity > 0 && !ms_each)) return fail(MLA_ERR_NULL_ARG, "output pointers are NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  bool bad = false;
  int64_t n = 0;
  for (int64_t i = 0; i < g_prof_used; ++i) {
    if (!g_prof_live[(size_t)i]) continue;  // a slot whose launch failed
    const auto& t = g_prof_ring[(size_t)i];
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
      bad = true;
    if (n < capacity) ms_each[n] = ms;
    ++n;
  }
  *launches = n;
  const int64_t dropped = g_prof_dropped;
  g_prof_used = 0;
  g_prof_dropped = 0;
  if (bad) return fail(MLA_ERR_HIP, "reading kernel timing events failed");
  if (dropped > 0) return fail(MLA_ERR_WORKSPACE, "%lld launches past the %d timing slots were not timed",
                               (long long)dropped, kProfileSlots);
  return ok();
}

mla_status mla_profile_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(MLA_ERR_NULL_ARG, "output pointers are NULL");
  std::vector<double> each(kProfileSlots);
  const mla_status s = mla_profile_read_each(each.data(), (int64_t)each.size(), launches);
  double sum = 0.0;
  for (int64_t i = 0; i < *launches && i < (int64_t)each.size(); ++i) sum += each[(size_t)i];
  *total_ms = sum;
  return s;
}

void mla_shutdown(void) {
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    profile_destroy_ring();
    g_prof_on = false;
  }
  std::lock_guard<std::mutex> lk(g_ws_mu);
  std::vector<std::pair<int, void*>> all = g_ws_retired;
  for (auto& kv : g_ws)
    if (kv.second.base) all.emplace_back(kv.first.first, kv.second.base);
  for (auto& dp : all) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(dp.first);
    (void)hipDeviceSynchronize();
    (void)hipFree(dp.second);
    (void)hipSetDevice(cur);
  }
  g_ws.clear();
  g_ws_retired.clear();
}

int32_t mla_decode_num_partitions(int64_t batch, int64_t num_heads, int64_t max_pages, int32_t page_size) {
  if (batch < 1 || batch > kMaxRows || !supported_heads(num_heads) || max_pages < 1 || page_size < 1 ||
      max_pages * page_size > (int64_t)1 << 30)
    return 0;
  return balanced_parts_per_row(batch, max_pages * page_size, cu_count(current_device()));
}

}  // extern "C"

namespace {

// The dense decode; fixed_ws selects the scratch array instead of the stream workspace.
mla_status decode_impl(const mla_tensor* q, const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                       const mla_tensor* cache_lens, const mla_tensor* latent_cache, float scale, int32_t mask,
                       int32_t local_window_size, int32_t num_partitions, mla_tensor* out, void* stream,
                       bool fixed_ws) {
  mla_status s;
  if ((s = check_tensor(q, "q", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  const int64_t T = q->shape[0], H = q->shape[1];
  if (q->shape[2] != 576) return fail(MLA_ERR_SHAPE, "q: head width %lld, expected 576", (long long)q->shape[2]);
  if ((s = check_tensor(input_row_offsets, "input_row_offsets", MLA_DTYPE_U32, 1, false)) != MLA_OK) return s;
  const int64_t B = input_row_offsets->shape[0] - 1;
  if (B < 1) return fail(MLA_ERR_SHAPE, "input_row_offsets: needs batch + 1 >= 2 entries");
  if ((s = check_tensor(page_table, "page_table", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  if (page_table->shape[0] != B) return fail(MLA_ERR_SHAPE, "page_table: %lld rows, expected batch %lld", (long long)page_table->shape[0], (long long)B);
  if ((s = check_1d(cache_lens, "cache_lens", MLA_DTYPE_I32, B)) != MLA_OK) return s;
  if ((s = check_tensor(latent_cache, "latent_cache", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (latent_cache->shape[2] != 576) return fail(MLA_ERR_SHAPE, "latent_cache: row width %lld, expected 576", (long long)latent_cache->shape[2]);
  const int64_t PS = latent_cache->shape[1];
  if (PS < 1) return fail(MLA_ERR_SHAPE, "latent_cache: page size must be >= 1");
  if (latent_cache->shape[0] > 0 && latent_cache->shape[1] > 1 && latent_cache->stride[1] != 576)
    return fail(MLA_ERR_SHAPE, "latent_cache: rows of a page must be contiguous (stride 576)");
  if (latent_cache->shape[0] > 1 && latent_cache->stride[0] < PS * 576)
    return fail(MLA_ERR_SHAPE, "latent_cache: pages overlap (page stride below page_size * 576)");
  if ((s = check_tensor(out, "out", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (out->shape[0] != T || out->shape[1] != H || out->shape[2] != 512)
    return fail(MLA_ERR_SHAPE, "out: shape must be [%lld, %lld, 512]", (long long)T, (long long)H);
  if (!supported_heads(H)) return fail(MLA_ERR_UNSUPPORTED, "num_heads %lld not in {16, 32, 64, 128}", (long long)H);
  if (mask < MLA_MASK_NULL || mask > MLA_MASK_SLIDING_WINDOW_CAUSAL) return fail(MLA_ERR_VALUE, "mask %d unknown", mask);
  if (mask == MLA_MASK_SLIDING_WINDOW_CAUSAL && local_window_size <= 0)
    return fail(MLA_ERR_VALUE, "sliding-window mask needs local_window_size > 0");
  if (!std::isfinite(scale)) return fail(MLA_ERR_VALUE, "scale must be finite");
  if (num_partitions > 4096) return fail(MLA_ERR_VALUE, "num_partitions %d above 4096", num_partitions);
  if (page_table->shape[1] * PS > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "max_pages * page_size above 2^30");
  if (T > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 query rows");
  if (T == 0) return ok();

  const int dev = current_device();
  const int grid = cu_count(dev);
  const int32_t nparts = num_partitions > 0 ? num_partitions : 0;
  const DecodeLayout L = decode_layout(T, (int32_t)H, nparts, grid);
  if (fixed_ws && L.total + kHeaderBytes > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "the call needs %zu bytes of workspace, above the %zu-byte scratch array",
                L.total + kHeaderBytes, kScratchBytes);
  bool cap = false;
  if ((s = stream_capturing(stream, &cap)) != MLA_OK) return s;
  void* ws = nullptr;
  if (fixed_ws) {
    if ((s = scratch_base(dev, stream, cap, &ws)) != MLA_OK) return s;
  } else if ((s = grow_workspace(dev, stream, L.total, cap, &ws)) != MLA_OK) {
    return s;
  }
  char* w = (char*)ws + kHeaderBytes;

  mla::DecodeArgs a{};
  a.q = (const uint16_t*)q->data;
  a.q_tok = q->stride[0];
  a.q_head = q->stride[1];
  a.offsets = (const uint32_t*)input_row_offsets->data;
  a.page_table = (const int32_t*)page_table->data;
  a.pt_row = page_table->stride[0];
  a.cache_lens = (const int32_t*)cache_lens->data;
  a.cache = (const uint8_t*)latent_cache->data;
  a.page_bytes = latent_cache->stride[0] * 2;
  a.num_pages = latent_cache->shape[0];
  a.B = (int32_t)B;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.PS = (int32_t)PS;
  a.max_pages = (int32_t)page_table->shape[1];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = mask;
  a.window = local_window_size;
  a.nparts = nparts;
  a.grid = grid;
  a.out = (uint16_t*)out->data;
  a.o_tok = out->stride[0];
  a.o_head = out->stride[1];
  a.part_o = (uint16_t*)(w + L.part_o);
  a.part_lse = (float*)(w + L.part_lse);
  a.row_meta = (int32_t*)(w + L.meta);
  a.zero_row = (const uint8_t*)ws;
  a.err = (uint32_t*)((char*)ws + kErrOffset);
  mla::KernelTimer tslot;
  int64_t tindex = -1;
  mla::KernelTimer* timer = profile_timer(&tslot, &tindex);
  const hipError_t e = mla::launch_decode(a, (hipStream_t)stream, timer);
  profile_keep(timer, tindex, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_decode_paged(const mla_tensor* q, const mla_tensor* input_row_offsets,
                            const mla_tensor* page_table, const mla_tensor* cache_lens,
                            const mla_tensor* latent_cache, float scale, int32_t mask,
                            int32_t local_window_size, int32_t num_partitions, mla_tensor* out,
                            void* stream) {
  return decode_impl(q, input_row_offsets, page_table, cache_lens, latent_cache, scale, mask, local_window_size,
                     num_partitions, out, stream, false);
}

mla_status mla_decode_paged_noalloc(const mla_tensor* q, const mla_tensor* input_row_offsets,
                                    const mla_tensor* page_table, const mla_tensor* cache_lens,
                                    const mla_tensor* latent_cache, float scale, int32_t mask,
                                    int32_t local_window_size, int32_t num_partitions, mla_tensor* out,
                                    void* stream) {
  return decode_impl(q, input_row_offsets, page_table, cache_lens, latent_cache, scale, mask, local_window_size,
                     num_partitions, out, stream, true);
}

}  // extern "C"

namespace {

// The sparse decode with its optional parts: sink logits and a second stream (null = none).
mla_status sparse_impl(const mla_tensor* q, const mla_tensor* q_scale, const mla_tensor* input_row_offsets,
                       const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                       const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                       const mla_tensor* attn_sink, const mla_tensor* extra_cache,
                       const mla_tensor* extra_cache_scale, const mla_tensor* extra_d_indices,
                       const mla_tensor* extra_topk_lengths, float scale, int32_t num_partitions,
                       mla_tensor* out, void* stream, bool shared = false) {
  mla_status s;
  if (!q) return fail(MLA_ERR_NULL_ARG, "q: descriptor is NULL");
  const bool q_bf16 = q->dtype == MLA_DTYPE_BF16;
  if ((s = check_tensor(q, "q", q_bf16 ? MLA_DTYPE_BF16 : MLA_DTYPE_FP8_E4M3, 3, true)) != MLA_OK) return s;
  const int64_t T = q->shape[0], H = q->shape[1];
  if (!latent_cache) return fail(MLA_ERR_NULL_ARG, "latent_cache: descriptor is NULL");
  // the row width picks the layout: 576 all e4m3, 640 rope-aware (q and cache alike)
  const int64_t RW = latent_cache->ndim == 3 && latent_cache->shape[2] == 640 ? 640 : 576;
  if (q->shape[2] != RW)
    return fail(MLA_ERR_SHAPE, "q: head width %lld, expected %lld (the cache's row width)", (long long)q->shape[2], (long long)RW);
  if (RW == 640 && q_bf16) return fail(MLA_ERR_VALUE, "the rope-aware layout needs an fp8 q");
  if (q_scale) {
    if (q_bf16) return fail(MLA_ERR_VALUE, "q_scale must be NULL when q is bf16");
    if ((s = check_1d(q_scale, "q_scale", MLA_DTYPE_F32, T)) != MLA_OK) return s;
  }
  if ((s = check_tensor(input_row_offsets, "input_row_offsets", MLA_DTYPE_U32, 1, false)) != MLA_OK) return s;
  if (input_row_offsets->shape[0] < 2) return fail(MLA_ERR_SHAPE, "input_row_offsets: needs batch + 1 >= 2 entries");
  // the rows of d_indices / topk_lengths: one per query row, or one per sequence (shared)
  const int64_t B = input_row_offsets->shape[0] - 1;
  const int64_t LR = shared ? B : T;
  if (shared && B > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 sequences");
  if (latent_cache->dtype == MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "sparse decode reads an fp8 e4m3 cache; a bf16 cache is not supported");
  if ((s = check_tensor(latent_cache, "latent_cache", MLA_DTYPE_FP8_E4M3, 3, true)) != MLA_OK) return s;
  if (latent_cache->shape[2] != RW) return fail(MLA_ERR_SHAPE, "latent_cache: row width %lld, expected 576 or 640", (long long)latent_cache->shape[2]);
  const int64_t NP = latent_cache->shape[0], PS = latent_cache->shape[1];
  if (PS < 1) return fail(MLA_ERR_SHAPE, "latent_cache: page size must be >= 1");
  if (NP > 0 && PS > 1 && latent_cache->stride[1] != RW)
    return fail(MLA_ERR_SHAPE, "latent_cache: rows of a page must be contiguous (stride %lld)", (long long)RW);
  if (NP > 1 && latent_cache->stride[0] < PS * RW)
    return fail(MLA_ERR_SHAPE, "latent_cache: pages overlap (page stride below page_size * %lld)", (long long)RW);
  if (NP * PS > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 cache rows");
  if (cache_scale) {
    if ((s = check_tensor(cache_scale, "cache_scale", MLA_DTYPE_F32, 2, false)) != MLA_OK) return s;
    if (cache_scale->shape[0] != NP || cache_scale->shape[1] != PS)
      return fail(MLA_ERR_SHAPE, "cache_scale: shape must be [%lld, %lld]", (long long)NP, (long long)PS);
  }
  if ((s = check_tensor(d_indices, "d_indices", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  if (d_indices->shape[0] != LR) return fail(MLA_ERR_SHAPE, "d_indices: %lld rows, expected %lld", (long long)d_indices->shape[0], (long long)LR);
  if (d_indices->shape[1] > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "d_indices: too many columns");
  if (LR > 1 && d_indices->stride[0] < d_indices->shape[1])
    return fail(MLA_ERR_SHAPE, "d_indices: row stride below the row length");
  if ((s = check_1d(topk_lengths, "topk_lengths", MLA_DTYPE_I32, LR)) != MLA_OK) return s;
  if ((s = check_tensor(out, "out", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (out->shape[0] != T || out->shape[1] != H || out->shape[2] != 512)
    return fail(MLA_ERR_SHAPE, "out: shape must be [%lld, %lld, 512]", (long long)T, (long long)H);
  if (!supported_heads(H)) return fail(MLA_ERR_UNSUPPORTED, "num_heads %lld not in {16, 32, 64, 128}", (long long)H);
  if (attn_sink && (s = check_1d(attn_sink, "attn_sink", MLA_DTYPE_F32, H)) != MLA_OK) return s;
  // the second stream: all four descriptors or none of its index parts
  const bool xtra = extra_d_indices != nullptr || extra_topk_lengths != nullptr || extra_cache != nullptr;
  if (RW == 640 && (xtra || attn_sink || extra_cache_scale))
    return fail(MLA_ERR_UNSUPPORTED, "the rope-aware layout is not supported with a sink or a second stream");
  int64_t XNP = 0, XPS = 0;
  if (xtra) {
    if (!extra_d_indices || !extra_topk_lengths || !extra_cache)
      return fail(MLA_ERR_NULL_ARG, "the extra stream needs extra_cache, extra_d_indices and extra_topk_lengths");
    if ((s = check_tensor(extra_cache, "extra_cache", MLA_DTYPE_FP8_E4M3, 3, true)) != MLA_OK) return s;
    if (extra_cache->shape[2] != 576)
      return fail(MLA_ERR_SHAPE, "extra_cache: row width %lld, expected 576", (long long)extra_cache->shape[2]);
    XNP = extra_cache->shape[0];
    XPS = extra_cache->shape[1];
    if (XPS < 1) return fail(MLA_ERR_SHAPE, "extra_cache: page size must be >= 1");
    if (XNP > 0 && XPS > 1 && extra_cache->stride[1] != 576)
      return fail(MLA_ERR_SHAPE, "extra_cache: rows of a page must be contiguous (stride 576)");
    if (XNP > 1 && extra_cache->stride[0] < XPS * 576)
      return fail(MLA_ERR_SHAPE, "extra_cache: pages overlap (page stride below page_size * 576)");
    if (extra_cache_scale) {
      if ((s = check_tensor(extra_cache_scale, "extra_cache_scale", MLA_DTYPE_F32, 2, false)) != MLA_OK) return s;
      if (extra_cache_scale->shape[0] != XNP || extra_cache_scale->shape[1] != XPS)
        return fail(MLA_ERR_SHAPE, "extra_cache_scale: shape must be [%lld, %lld]", (long long)XNP, (long long)XPS);
    }
    if ((s = check_tensor(extra_d_indices, "extra_d_indices", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
    if (extra_d_indices->shape[0] != T)
      return fail(MLA_ERR_SHAPE, "extra_d_indices: %lld rows, expected %lld", (long long)extra_d_indices->shape[0], (long long)T);
    if (extra_d_indices->shape[1] > INT32_MAX / 2 || d_indices->shape[1] > INT32_MAX / 2)
      return fail(MLA_ERR_UNSUPPORTED, "index lists too wide for two streams");
    if (T > 1 && extra_d_indices->stride[0] < extra_d_indices->shape[1])
      return fail(MLA_ERR_SHAPE, "extra_d_indices: row stride below the row length");
    if ((s = check_1d(extra_topk_lengths, "extra_topk_lengths", MLA_DTYPE_I32, T)) != MLA_OK) return s;
    if (NP * PS >= (int64_t)mla::kExtraRowBit || XNP * XPS >= (int64_t)mla::kExtraRowBit)
      return fail(MLA_ERR_UNSUPPORTED, "with an extra stream each pool holds fewer than 2^30 rows");
  } else if (extra_cache_scale) {
    return fail(MLA_ERR_VALUE, "extra_cache_scale given without an extra stream");
  }
  if (!std::isfinite(scale)) return fail(MLA_ERR_VALUE, "scale must be finite");
  if (num_partitions > 4096) return fail(MLA_ERR_VALUE, "num_partitions %d above 4096", num_partitions);
  if (T > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 query rows");
  if (T == 0) return ok();

  bool cap = false;
  if ((s = stream_capturing(stream, &cap)) != MLA_OK) return s;
  const int dev = current_device();
  const int grid = cu_count(dev);
  const int32_t nparts = num_partitions > 0 ? num_partitions : 0;
  const DecodeLayout L = decode_layout(T, (int32_t)H, nparts, grid);
  void* ws = nullptr;
  if ((s = grow_workspace(dev, stream, L.total, cap, &ws)) != MLA_OK) return s;
  char* w = (char*)ws + kHeaderBytes;

  mla::SparseArgs a{};
  a.q = (const uint8_t*)q->data;
  a.q_tok = q->stride[0];
  a.q_head = q->stride[1];
  a.q_scale = q_scale ? (const float*)q_scale->data : nullptr;
  a.cache = (const uint8_t*)latent_cache->data;
  a.page_bytes = latent_cache->stride[0];
  a.cache_scale = cache_scale ? (const float*)cache_scale->data : nullptr;
  a.cs_page = cache_scale ? cache_scale->stride[0] : 0;
  a.num_rows = NP * PS;
  a.PS = (int32_t)PS;
  a.flat = a.page_bytes == PS * RW && (cache_scale == nullptr || a.cs_page == PS) ? 1 : 0;
  a.rope = RW == 640 ? 1 : 0;
  a.shared = shared ? 1 : 0;
  if (shared) {
    a.offsets = (const uint32_t*)input_row_offsets->data;
    a.B = (int32_t)B;
  }
  a.idx = (const int32_t*)d_indices->data;
  a.idx_row = d_indices->stride[0];
  a.idx_cols = (int32_t)d_indices->shape[1];
  a.topk = (const int32_t*)topk_lengths->data;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.q_bf16 = q_bf16 ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.nparts = nparts;
  a.grid = grid;
  a.out = (uint16_t*)out->data;
  a.o_tok = out->stride[0];
  a.o_head = out->stride[1];
  a.part_o = (uint16_t*)(w + L.part_o);
  a.part_lse = (float*)(w + L.part_lse);
  a.row_meta = (int32_t*)(w + L.meta);
  a.zero_row = (const uint8_t*)ws;
  a.err = (uint32_t*)((char*)ws + kErrOffset);
  a.sink = attn_sink ? (const float*)attn_sink->data : nullptr;
  if (xtra) {
    a.flat = 0;  // rows of both pools go through the per-row address path
    a.xidx = (const int32_t*)extra_d_indices->data;
    a.xidx_row = extra_d_indices->stride[0];
    a.xidx_cols = (int32_t)extra_d_indices->shape[1];
    a.xtopk = (const int32_t*)extra_topk_lengths->data;
    a.xcache = (const uint8_t*)extra_cache->data;
    a.xpage_bytes = extra_cache->stride[0];
    a.xcache_scale = extra_cache_scale ? (const float*)extra_cache_scale->data : nullptr;
    a.xcs_page = extra_cache_scale ? extra_cache_scale->stride[0] : 0;
    a.xnum_rows = XNP * XPS;
    a.xPS = (int32_t)XPS;
  }
  mla::KernelTimer tslot;
  int64_t tindex = -1;
  mla::KernelTimer* timer = profile_timer(&tslot, &tindex);
  const hipError_t e = mla::launch_sparse(a, (hipStream_t)stream, timer);
  profile_keep(timer, tindex, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "sparse decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_decode_paged_sparse(const mla_tensor* q, const mla_tensor* q_scale,
                                   const mla_tensor* input_row_offsets,
                                   const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                   const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                   float scale, int32_t num_partitions, mla_tensor* out,
                                   void* stream) {
  return sparse_impl(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, nullptr,
                     nullptr, nullptr, nullptr, nullptr, scale, num_partitions, out, stream);
}

mla_status mla_decode_paged_sparse_shared(const mla_tensor* q, const mla_tensor* q_scale,
                                          const mla_tensor* input_row_offsets,
                                          const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                          const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                          float scale, int32_t num_partitions, mla_tensor* out,
                                          void* stream) {
  return sparse_impl(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, nullptr,
                     nullptr, nullptr, nullptr, nullptr, scale, num_partitions, out, stream, true);
}

mla_status mla_decode_paged_sparse_ext(const mla_tensor* q, const mla_tensor* q_scale,
                                       const mla_tensor* input_row_offsets,
                                       const mla_tensor* latent_cache, const mla_tensor* cache_scale,
                                       const mla_tensor* d_indices, const mla_tensor* topk_lengths,
                                       const mla_tensor* attn_sink, const mla_tensor* extra_cache,
                                       const mla_tensor* extra_cache_scale,
                                       const mla_tensor* extra_d_indices,
                                       const mla_tensor* extra_topk_lengths, float scale,
                                       int32_t num_partitions, mla_tensor* out, void* stream) {
  return sparse_impl(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, attn_sink,
                     extra_cache, extra_cache_scale, extra_d_indices, extra_topk_lengths, scale, num_partitions,
                     out, stream);
}

mla_status mla_decode_paged_fp8(const mla_tensor* q, const mla_tensor* q_scale,
                                const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                                const mla_tensor* cache_lens, const mla_tensor* latent_cache,
                                const mla_tensor* cache_scale, float scale, int32_t mask,
                                int32_t local_window_size, int32_t num_partitions, mla_tensor* out,
                                void* stream) {
  mla_status s;
  if ((s = check_tensor(q, "q", MLA_DTYPE_FP8_E4M3, 3, true)) != MLA_OK) return s;
  const int64_t T = q->shape[0], H = q->shape[1];
  if (!latent_cache) return fail(MLA_ERR_NULL_ARG, "latent_cache: descriptor is NULL");
  // the row width picks the layout: 576 all e4m3, 640 rope-aware (q and cache alike)
  const int64_t RW = latent_cache->ndim == 3 && latent_cache->shape[2] == 640 ? 640 : 576;
  if (q->shape[2] != RW)
    return fail(MLA_ERR_SHAPE, "q: head width %lld, expected %lld (the cache's row width)", (long long)q->shape[2], (long long)RW);
  if (q_scale && (s = check_1d(q_scale, "q_scale", MLA_DTYPE_F32, T)) != MLA_OK) return s;
  if ((s = check_tensor(input_row_offsets, "input_row_offsets", MLA_DTYPE_U32, 1, false)) != MLA_OK) return s;
  const int64_t B = input_row_offsets->shape[0] - 1;
  if (B < 1) return fail(MLA_ERR_SHAPE, "input_row_offsets: needs batch + 1 >= 2 entries");
  if ((s = check_tensor(page_table, "page_table", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  if (page_table->shape[0] != B) return fail(MLA_ERR_SHAPE, "page_table: %lld rows, expected batch %lld", (long long)page_table->shape[0], (long long)B);
  if ((s = check_1d(cache_lens, "cache_lens", MLA_DTYPE_I32, B)) != MLA_OK) return s;
  if ((s = check_tensor(latent_cache, "latent_cache", MLA_DTYPE_FP8_E4M3, 3, true)) != MLA_OK) return s;
  if (latent_cache->shape[2] != RW) return fail(MLA_ERR_SHAPE, "latent_cache: row width %lld, expected 576 or 640", (long long)latent_cache->shape[2]);
  const int64_t NP = latent_cache->shape[0], PS = latent_cache->shape[1];
  if (PS < 1) return fail(MLA_ERR_SHAPE, "latent_cache: page size must be >= 1");
  if (NP > 0 && PS > 1 && latent_cache->stride[1] != RW)
    return fail(MLA_ERR_SHAPE, "latent_cache: rows of a page must be contiguous (stride %lld)", (long long)RW);
  if (NP > 1 && latent_cache->stride[0] < PS * RW)
    return fail(MLA_ERR_SHAPE, "latent_cache: pages overlap (page stride below page_size * %lld)", (long long)RW);
  if (NP * PS > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 cache rows");
  if (cache_scale) {
    if ((s = check_tensor(cache_scale, "cache_scale", MLA_DTYPE_F32, 2, false)) != MLA_OK) return s;
    if (cache_scale->shape[0] != NP || cache_scale->shape[1] != PS)
      return fail(MLA_ERR_SHAPE, "cache_scale: shape must be [%lld, %lld]", (long long)NP, (long long)PS);
  }
  if ((s = check_tensor(out, "out", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (out->shape[0] != T || out->shape[1] != H || out->shape[2] != 512)
    return fail(MLA_ERR_SHAPE, "out: shape must be [%lld, %lld, 512]", (long long)T, (long long)H);
  if (!supported_heads(H)) return fail(MLA_ERR_UNSUPPORTED, "num_heads %lld not in {16, 32, 64, 128}", (long long)H);
  if (mask < MLA_MASK_NULL || mask > MLA_MASK_SLIDING_WINDOW_CAUSAL) return fail(MLA_ERR_VALUE, "mask %d unknown", mask);
  if (mask == MLA_MASK_SLIDING_WINDOW_CAUSAL && local_window_size <= 0)
    return fail(MLA_ERR_VALUE, "sliding-window mask needs local_window_size > 0");
  if (!std::isfinite(scale)) return fail(MLA_ERR_VALUE, "scale must be finite");
  if (num_partitions > 4096) return fail(MLA_ERR_VALUE, "num_partitions %d above 4096", num_partitions);
  if (page_table->shape[1] * PS > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "max_pages * page_size above 2^30");
  if (T > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 query rows");
  if (T == 0) return ok();

  bool cap = false;
  if ((s = stream_capturing(stream, &cap)) != MLA_OK) return s;
  const int dev = current_device();
  const int grid = cu_count(dev);
  const int32_t nparts = num_partitions > 0 ? num_partitions : 0;
  const DecodeLayout L = decode_layout(T, (int32_t)H, nparts, grid);
  void* ws = nullptr;
  if ((s = grow_workspace(dev, stream, L.total, cap, &ws)) != MLA_OK) return s;
  char* w = (char*)ws + kHeaderBytes;

  mla::SparseArgs a{};
  a.q = (const uint8_t*)q->data;
  a.q_tok = q->stride[0];
  a.q_head = q->stride[1];
  a.q_scale = q_scale ? (const float*)q_scale->data : nullptr;
  a.cache = (const uint8_t*)latent_cache->data;
  a.page_bytes = latent_cache->stride[0];
  a.cache_scale = cache_scale ? (const float*)cache_scale->data : nullptr;
  a.cs_page = cache_scale ? cache_scale->stride[0] : 0;
  a.num_rows = NP * PS;
  a.PS = (int32_t)PS;
  a.flat = a.page_bytes == PS * RW && (cache_scale == nullptr || a.cs_page == PS) ? 1 : 0;
  a.rope = RW == 640 ? 1 : 0;
  a.dense = 1;
  a.offsets = (const uint32_t*)input_row_offsets->data;
  a.page_table = (const int32_t*)page_table->data;
  a.pt_row = page_table->stride[0];
  a.cache_lens = (const int32_t*)cache_lens->data;
  a.B = (int32_t)B;
  a.max_pages = (int32_t)page_table->shape[1];
  a.mask = mask;
  a.window = local_window_size;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.q_bf16 = 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.nparts = nparts;
  a.grid = grid;
  a.out = (uint16_t*)out->data;
  a.o_tok = out->stride[0];
  a.o_head = out->stride[1];
  a.part_o = (uint16_t*)(w + L.part_o);
  a.part_lse = (float*)(w + L.part_lse);
  a.row_meta = (int32_t*)(w + L.meta);
  a.zero_row = (const uint8_t*)ws;
  a.err = (uint32_t*)((char*)ws + kErrOffset);
  mla::KernelTimer tslot;
  int64_t tindex = -1;
  mla::KernelTimer* timer = profile_timer(&tslot, &tindex);
  const hipError_t e = mla::launch_sparse(a, (hipStream_t)stream, timer);
  profile_keep(timer, tindex, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "fp8 decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_indexer_paged_fp8(const mla_tensor* q, const mla_tensor* q_s,
                                 const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                                 const mla_tensor* cache_lens, const mla_tensor* k_cache,
                                 const mla_tensor* k_scale, int32_t mask, int32_t local_window_size,
                                 mla_tensor* out_indices, void* stream) {
  mla_status s;
  if ((s = check_tensor(q, "q", MLA_DTYPE_FP8_E4M3, 3, false)) != MLA_OK) return s;
  const int64_t T = q->shape[0], NH = q->shape[1], D = q->shape[2];
  if (q->stride[2] != 1) return fail(MLA_ERR_SHAPE, "q: the head width must be contiguous");
  if (D < 16 || D > mla::kIdxMaxDepth || D % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "indexer head width %lld: a multiple of 16 up to %d", (long long)D, mla::kIdxMaxDepth);
  if (NH < 1) return fail(MLA_ERR_SHAPE, "q: needs at least one head");
  if ((s = check_tensor(q_s, "q_s", MLA_DTYPE_F32, 2, false)) != MLA_OK) return s;
  if (q_s->shape[0] != T || q_s->shape[1] != NH || q_s->stride[1] != 1)
    return fail(MLA_ERR_SHAPE, "q_s: shape must be [%lld, %lld], heads contiguous", (long long)T, (long long)NH);
  if ((s = check_tensor(input_row_offsets, "input_row_offsets", MLA_DTYPE_U32, 1, false)) != MLA_OK) return s;
  const int64_t B = input_row_offsets->shape[0] - 1;
  if (B < 1) return fail(MLA_ERR_SHAPE, "input_row_offsets: needs batch + 1 >= 2 entries");
  if ((s = check_tensor(page_table, "page_table", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  if (page_table->shape[0] != B) return fail(MLA_ERR_SHAPE, "page_table: %lld rows, expected batch %lld", (long long)page_table->shape[0], (long long)B);
  if ((s = check_1d(cache_lens, "cache_lens", MLA_DTYPE_I32, B)) != MLA_OK) return s;
  if ((s = check_tensor(k_cache, "k_cache", MLA_DTYPE_FP8_E4M3, 3, false)) != MLA_OK) return s;
  const int64_t NP = k_cache->shape[0], PS = k_cache->shape[1];
  if (k_cache->shape[2] != D) return fail(MLA_ERR_SHAPE, "k_cache: row width %lld, expected %lld", (long long)k_cache->shape[2], (long long)D);
  if (PS < 1) return fail(MLA_ERR_SHAPE, "k_cache: page size must be >= 1");
  if (k_cache->stride[2] != 1 || (NP > 0 && PS > 1 && k_cache->stride[1] != D))
    return fail(MLA_ERR_SHAPE, "k_cache: rows of a page must be contiguous");
  if (NP > 1 && k_cache->stride[0] < PS * D) return fail(MLA_ERR_SHAPE, "k_cache: pages overlap");
  if (k_cache->stride[0] % 16 != 0 || (uintptr_t)k_cache->data % 16 != 0)
    return fail(MLA_ERR_ALIGNMENT, "k_cache: base and page stride must be multiples of 16 bytes");
  if (NP * PS > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 cache rows");
  if (k_scale) {
    if ((s = check_tensor(k_scale, "k_scale", MLA_DTYPE_F32, 2, false)) != MLA_OK) return s;
    if (k_scale->shape[0] != NP || k_scale->shape[1] != PS || (PS > 1 && k_scale->stride[1] != 1))
      return fail(MLA_ERR_SHAPE, "k_scale: shape must be [%lld, %lld], rows contiguous", (long long)NP, (long long)PS);
  }
  if ((s = check_tensor(out_indices, "out_indices", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  const int64_t K = out_indices->shape[1];
  if (out_indices->shape[0] != T || out_indices->stride[1] != 1 || (T > 1 && out_indices->stride[0] < K))
    return fail(MLA_ERR_SHAPE, "out_indices: shape must be [%lld, top_k], rows contiguous", (long long)T);
  if (K < 1 || K > mla::kIdxMaxTopK) return fail(MLA_ERR_UNSUPPORTED, "top_k %lld not in [1, %d]", (long long)K, mla::kIdxMaxTopK);
  if (page_table->shape[1] * PS > mla::kIdxMaxKeys)
    return fail(MLA_ERR_UNSUPPORTED, "max_pages * page_size above %d rows per sequence", mla::kIdxMaxKeys);
  if (mask < MLA_MASK_NULL || mask > MLA_MASK_SLIDING_WINDOW_CAUSAL) return fail(MLA_ERR_VALUE, "mask %d unknown", mask);
  if (mask == MLA_MASK_SLIDING_WINDOW_CAUSAL && local_window_size <= 0)
    return fail(MLA_ERR_VALUE, "sliding-window mask needs local_window_size > 0");
  if (T > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 query rows");
  if (T == 0) return ok();

  bool cap = false;
  if ((s = stream_capturing(stream, &cap)) != MLA_OK) return s;
  void* ws = nullptr;
  const IndexerLayout L = indexer_layout(T, page_table->shape[1], PS);
  if ((s = grow_workspace(current_device(), stream, L.total, cap, &ws)) != MLA_OK) return s;
  mla::IndexerArgs a{};
  a.keys = (uint64_t*)((char*)ws + kHeaderBytes);
  a.keys_row = L.keys_row;
  a.slice_hist = (uint32_t*)((char*)ws + kHeaderBytes + L.key_bytes);
  a.hist_row = L.hist_row;
  a.zero_row = (const uint8_t*)ws;  // the header's zero row
  a.q = (const uint8_t*)q->data;
  a.q_tok = q->stride[0];
  a.q_head = q->stride[1];
  a.q_s = (const float*)q_s->data;
  a.qs_tok = q_s->stride[0];
  a.offsets = (const uint32_t*)input_row_offsets->data;
  a.page_table = (const int32_t*)page_table->data;
  a.pt_row = page_table->stride[0];
  a.cache_lens = (const int32_t*)cache_lens->data;
  a.k = (const uint8_t*)k_cache->data;
  a.page_bytes = k_cache->stride[0];
  a.num_pages = NP;
  a.k_s = k_scale ? (const float*)k_scale->data : nullptr;
  a.ks_page = k_scale ? k_scale->stride[0] : 0;
  a.B = (int32_t)B;
  a.T = (int32_t)T;
  a.NH = (int32_t)NH;
  a.depth = (int32_t)D;
  a.PS = (int32_t)PS;
  a.max_pages = (int32_t)page_table->shape[1];
  a.mask = mask;
  a.window = local_window_size;
  a.top_k = (int32_t)K;
  a.out = (int32_t*)out_indices->data;
  a.out_row = out_indices->stride[0];
  a.err = (uint32_t*)((char*)ws + kErrOffset);
  mla::KernelTimer tslot;
  int64_t tindex = -1;
  mla::KernelTimer* timer = profile_timer(&tslot, &tindex);
  const hipError_t e = mla::launch_indexer(a, (hipStream_t)stream, timer);
  profile_keep(timer, tindex, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "indexer launch failed: %s", hipGetErrorString(e));
  return ok();
}

mla_status mla_prefill_paged(const mla_tensor* q, const mla_tensor* k, const mla_tensor* v,
                             const mla_tensor* buffer_row_offsets, const mla_tensor* cache_offsets,
                             const mla_tensor* input_row_offsets, const mla_tensor* page_table,
                             const mla_tensor* cache_lens, const mla_tensor* latent_cache,
                             float scale, int32_t mask, mla_tensor* out, void* stream) {
  mla_status s;
  if ((s = check_tensor(q, "q", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  const int64_t Tq = q->shape[0], H = q->shape[1];
  if (q->shape[2] != 192) return fail(MLA_ERR_SHAPE, "q: head width %lld, expected 192", (long long)q->shape[2]);
  if ((s = check_tensor(k, "k", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if ((s = check_tensor(v, "v", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  const int64_t Tk = k->shape[0];
  if (k->shape[1] != H || k->shape[2] != 128) return fail(MLA_ERR_SHAPE, "k: shape must be [Tk, %lld, 128]", (long long)H);
  if (v->shape[0] != Tk || v->shape[1] != H || v->shape[2] != 128)
    return fail(MLA_ERR_SHAPE, "v: shape must be [%lld, %lld, 128]", (long long)Tk, (long long)H);
  if ((s = check_tensor(input_row_offsets, "input_row_offsets", MLA_DTYPE_U32, 1, false)) != MLA_OK) return s;
  const int64_t B = input_row_offsets->shape[0] - 1;
  if (B < 1) return fail(MLA_ERR_SHAPE, "input_row_offsets: needs batch + 1 >= 2 entries");
  if ((s = check_1d(buffer_row_offsets, "buffer_row_offsets", MLA_DTYPE_U32, B + 1)) != MLA_OK) return s;
  if ((s = check_1d(cache_offsets, "cache_offsets", MLA_DTYPE_U32, B)) != MLA_OK) return s;
  if ((s = check_tensor(page_table, "page_table", MLA_DTYPE_I32, 2, false)) != MLA_OK) return s;
  if (page_table->shape[0] != B) return fail(MLA_ERR_SHAPE, "page_table: %lld rows, expected batch %lld", (long long)page_table->shape[0], (long long)B);
  if ((s = check_1d(cache_lens, "cache_lens", MLA_DTYPE_I32, B)) != MLA_OK) return s;
  if ((s = check_tensor(latent_cache, "latent_cache", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (latent_cache->shape[2] != 576) return fail(MLA_ERR_SHAPE, "latent_cache: row width %lld, expected 576", (long long)latent_cache->shape[2]);
  const int64_t PS = latent_cache->shape[1];
  if (PS < 1) return fail(MLA_ERR_SHAPE, "latent_cache: page size must be >= 1");
  if (latent_cache->shape[0] > 0 && PS > 1 && latent_cache->stride[1] != 576)
    return fail(MLA_ERR_SHAPE, "latent_cache: rows of a page must be contiguous (stride 576)");
  if ((s = check_tensor(out, "out", MLA_DTYPE_BF16, 3, true)) != MLA_OK) return s;
  if (out->shape[0] != Tq || out->shape[1] != H || out->shape[2] != 128)
    return fail(MLA_ERR_SHAPE, "out: shape must be [%lld, %lld, 128]", (long long)Tq, (long long)H);
  if (H < 1 || H > 1024) return fail(MLA_ERR_UNSUPPORTED, "num_heads %lld not in [1, 1024]", (long long)H);
  if (mask == MLA_MASK_SLIDING_WINDOW_CAUSAL) return fail(MLA_ERR_UNSUPPORTED, "prefill takes the causal or the null mask");
  if (mask != MLA_MASK_NULL && mask != MLA_MASK_CAUSAL) return fail(MLA_ERR_VALUE, "mask %d unknown", mask);
  if (!std::isfinite(scale)) return fail(MLA_ERR_VALUE, "scale must be finite");
  if (Tq > kMaxRows || Tk > kMaxRows) return fail(MLA_ERR_UNSUPPORTED, "more than 2^24 query or key rows");
  if (page_table->shape[1] * PS > (int64_t)1 << 40) return fail(MLA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  if (((Tq + 127) / 128 + B) * H > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "too many work-groups");
  if (Tq == 0) return ok();

  mla::PrefillArgs a{};
  a.q = (const uint16_t*)q->data;
  a.q_tok = q->stride[0];
  a.q_head = q->stride[1];
  a.k = (const uint16_t*)k->data;
  a.k_tok = k->stride[0];
  a.k_head = k->stride[1];
  a.v = (const uint16_t*)v->data;
  a.v_tok = v->stride[0];
  a.v_head = v->stride[1];
  a.buf_off = (const uint32_t*)buffer_row_offsets->data;
  a.cache_off = (const uint32_t*)cache_offsets->data;
  a.in_off = (const uint32_t*)input_row_offsets->data;
  a.page_table = (const int32_t*)page_table->data;
  a.pt_row = page_table->stride[0];
  a.cache_lens = (const int32_t*)cache_lens->data;
  a.cache = (const uint8_t*)latent_cache->data;
  a.page_bytes = latent_cache->stride[0] * 2;
  a.num_pages = latent_cache->shape[0];
  a.B = (int32_t)B;
  a.Tq = (int32_t)Tq;
  a.Tk = (int32_t)Tk;
  a.H = (int32_t)H;
  a.PS = (int32_t)PS;
  a.max_pages = (int32_t)page_table->shape[1];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = mask;
  a.out = (uint16_t*)out->data;
  a.o_tok = out->stride[0];
  a.o_head = out->stride[1];
  // the error word and the zero row live in the stream's workspace (allocated on first use)
  bool cap = false;
  if ((s = stream_capturing(stream, &cap)) != MLA_OK) return s;
  void* ws = nullptr;
  if ((s = grow_workspace(current_device(), stream, 0, cap, &ws)) != MLA_OK) return s;
  a.zero_row = (const uint8_t*)ws;
  a.err = (uint32_t*)((char*)ws + kErrOffset);
  mla::KernelTimer tslot;
  int64_t tindex = -1;
  mla::KernelTimer* timer = profile_timer(&tslot, &tindex);
  const hipError_t e = mla::launch_prefill(a, (hipStream_t)stream, timer);
  profile_keep(timer, tindex, e == hipSuccess);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
