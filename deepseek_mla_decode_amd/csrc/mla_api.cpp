// mla_api.cpp -- host side of the MLA decode C ABI: argument validation,
// workspace layout, the host twin of the split planner, launches and timing.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mla_decode.h"
#include "mla_kernels.h"
#include "plan_rule.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MLA_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_num_cus[kMaxDevices];

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout: [plan ints][partial lse fp32][partial rows fp16][fp32 copies of wide rows].
struct Layout {
  size_t num_splits, split_offset, work, part_lse, part16, part32, total;
};

Layout layout(const mla_desc* d, int32_t max_work) {
  Layout L;
  const size_t B = (size_t)d->batch, H = (size_t)d->heads, W = (size_t)max_work;
  L.num_splits = 0;
  L.split_offset = L.num_splits + B * 4;
  L.work = L.split_offset + (B + 1) * 4;
  L.part_lse = round_up(L.work + 4 * W * 4, 256);
  L.part16 = round_up(L.part_lse + W * H * 4, 256);
  L.part32 = round_up(L.part16 + W * H * 512 * 2, 256);
  L.total = round_up(L.part32 + W * H * 512 * 4, 256);
  return L;
}

int check_desc(const mla_desc* d) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", d->batch);
  if (d->heads < 1) return fail(MLA_ERR_INVALID_ARG, "heads %d < 1", d->heads);
  if (d->d_latent != MLA_D_LATENT || d->d_rope != MLA_D_ROPE)
    return fail(MLA_ERR_UNSUPPORTED, "dims %d/%d: only 512 latent + 64 rope are supported", d->d_latent,
                d->d_rope);
  if (d->dtype != MLA_DTYPE_F16 && d->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->kv_dtype != MLA_KV_AS_DTYPE && d->kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "kv_dtype %d not supported", d->kv_dtype);
  if (d->kv_dtype == MLA_KV_FP8_E4M3) {
    if (!std::isfinite(d->kv_scale) || !(d->kv_scale > 0.f))
      return fail(MLA_ERR_INVALID_ARG, "kv_scale of an FP8 cache must be finite and positive");
  } else if (d->kv_scale != 0.f && d->kv_scale != 1.f) {
    return fail(MLA_ERR_INVALID_ARG, "kv_scale %g given for a 16-bit cache (only an FP8 cache is scaled)",
                (double)d->kv_scale);
  }
  if (d->seqlen_q < 0) return fail(MLA_ERR_INVALID_ARG, "seqlen_q %d < 0", d->seqlen_q);
  if (d->seqlen_q > mla::kMaxSeqlenQ)
    return fail(MLA_ERR_UNSUPPORTED, "seqlen_q %d above %d", d->seqlen_q, mla::kMaxSeqlenQ);
  if (d->seqlen_q > 1 && d->heads % d->seqlen_q != 0)
    return fail(MLA_ERR_INVALID_ARG, "heads %d (query rows) is not a multiple of seqlen_q %d", d->heads,
                d->seqlen_q);
  return MLA_OK;
}

int32_t seqlen_q_of(const mla_desc* d) { return d->seqlen_q < 1 ? 1 : d->seqlen_q; }

int check_num_split(int32_t num_split) {
  if (num_split < 0 || num_split > MLA_MAX_SPLITS)
    return fail(MLA_ERR_INVALID_ARG, "num_split %d outside [0, %d]", num_split, MLA_MAX_SPLITS);
  return MLA_OK;
}

int max_work_of(const mla_desc* d, int32_t num_split, int32_t num_cus, int32_t* out) {
  if (num_cus < 1) return fail(MLA_ERR_INVALID_ARG, "num_cus %d < 1", num_cus);
  const int64_t w = mla::max_splits(d->batch, d->heads, num_split, num_cus, seqlen_q_of(d));
  if (w > (int64_t)INT32_MAX / 4) return fail(MLA_ERR_INVALID_ARG, "too many work items (%lld)", (long long)w);
  *out = (int32_t)w;
  return MLA_OK;
}

// ---- timing ----------------------------------------------------------------
constexpr int kMaxTimed = 4096;
constexpr int kEventsPerCall = 4;
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_events;  // 4 per call: split, combine (start, stop)
std::vector<uint8_t> g_combined;   // per call: whether a combine ran (and its events were recorded)
int g_timed = 0;

// A timed call's events (copies of the handles, so that another thread
// growing the pool cannot invalidate them) and its index.
struct TimingSlot {
  int index;
  hipEvent_t ev[kEventsPerCall];
};

bool timing_slot(TimingSlot* s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || g_timed >= kMaxTimed) return false;
  const size_t need = kEventsPerCall * (size_t)(g_timed + 1);
  while (g_events.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return false;
    g_events.push_back(e);
  }
  if (g_combined.size() < (size_t)g_timed + 1) g_combined.resize((size_t)g_timed + 1);
  g_combined[g_timed] = 0;
  s->index = g_timed;
  for (int k = 0; k < kEventsPerCall; ++k) s->ev[k] = g_events[kEventsPerCall * (size_t)g_timed + k];
  ++g_timed;
  return true;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_last_error.c_str(); }

int mla_num_cus(int device, int32_t* num_cus_out) {
  if (!num_cus_out) return fail(MLA_ERR_INVALID_ARG, "num_cus_out is NULL");
  if (device < 0 || device >= kMaxDevices) return fail(MLA_ERR_INVALID_ARG, "device %d out of range", device);
  int32_t v = g_num_cus[device].load(std::memory_order_relaxed);
  if (v <= 0) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess || n <= 0)
      return fail(MLA_ERR_HIP, "hipDeviceGetAttribute(multiProcessorCount): %s", hipGetErrorString(e));
    v = n;
    g_num_cus[device].store(v, std::memory_order_relaxed);
  }
  *num_cus_out = v;
  return ok();
}

int mla_max_work(const mla_desc* desc, int32_t num_split, int32_t num_cus, int32_t* max_work_out) {
  int st;
  if ((st = check_desc(desc)) != MLA_OK) return st;
  if ((st = check_num_split(num_split)) != MLA_OK) return st;
  if (!max_work_out) return fail(MLA_ERR_INVALID_ARG, "max_work_out is NULL");
  if ((st = max_work_of(desc, num_split, num_cus, max_work_out)) != MLA_OK) return st;
  return ok();
}

int mla_workspace_size(const mla_desc* desc, int32_t num_split, int32_t num_cus, size_t* bytes_out) {
  int st;
  if ((st = check_desc(desc)) != MLA_OK) return st;
  if ((st = check_num_split(num_split)) != MLA_OK) return st;
  if (!bytes_out) return fail(MLA_ERR_INVALID_ARG, "bytes_out is NULL");
  int32_t w;
  if ((st = max_work_of(desc, num_split, num_cus, &w)) != MLA_OK) return st;
  *bytes_out = layout(desc, w).total;
  return ok();
}

int mla_plan_host(const int32_t* cache_seqlens, int32_t batch, int32_t heads, int32_t seqlen_q,
                  int32_t num_split, int32_t num_cus, int32_t* num_splits, int32_t* split_offset, int32_t* work,
                  int32_t max_work) {
  int st;
  if (batch < 0 || heads < 1 || num_cus < 1) return fail(MLA_ERR_INVALID_ARG, "bad batch/heads/num_cus");
  if (seqlen_q < 0 || seqlen_q > mla::kMaxSeqlenQ) return fail(MLA_ERR_INVALID_ARG, "bad seqlen_q %d", seqlen_q);
  if (seqlen_q < 1) seqlen_q = 1;
  if ((st = check_num_split(num_split)) != MLA_OK) return st;
  if (batch > 0 && (!cache_seqlens || !num_splits || !work)) return fail(MLA_ERR_INVALID_ARG, "NULL array");
  if (!split_offset) return fail(MLA_ERR_INVALID_ARG, "NULL split_offset");
  const int32_t cap_rows = INT32_MAX;
  const int32_t tail = mla::tail_splits(seqlen_q);
  // Blocks of each sequence's prefix (the rows every query token sees).
  std::vector<int32_t> nb(batch);
  int32_t mx = 0;
  for (int b = 0; b < batch; ++b) {
    nb[b] = mla::num_blocks(mla::prefix_len(mla::clamp_len(cache_seqlens[b], cap_rows), seqlen_q));
    mx = nb[b] > mx ? nb[b] : mx;
  }
  int32_t t = 1;
  if (num_split == 0) {
    const int64_t cap = mla::planner_cap(batch, heads, num_cus, seqlen_q);
    int32_t lo = 1, hi = mx > 1 ? mx : 1;
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      int64_t cnt = 0;
      for (int b = 0; b < batch; ++b) cnt += mla::splits_for_budget(nb[b], mid);
      if (cnt <= cap) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }
  auto prefix_splits = [&](int b) { return num_split > 0 ? num_split : mla::splits_for_budget(nb[b], t); };
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) total += prefix_splits(b) + tail;
  if (total > max_work) return fail(MLA_ERR_INVALID_ARG, "plan needs %lld work items > max_work %d",
                                    (long long)total, max_work);
  int32_t off = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t L = mla::clamp_len(cache_seqlens[b], cap_rows);
    const int32_t sp = prefix_splits(b), s = sp + tail;
    num_splits[b] = s;
    split_offset[b] = off;
    for (int32_t k = 0; k < s; ++k) {
      int32_t r0, r1;
      mla::seq_split_range(L, seqlen_q, sp, k, &r0, &r1);
      int32_t* w = work + 4 * (size_t)(off + k);
      w[0] = b;
      w[1] = k;
      w[2] = r0;
      w[3] = r1;
    }
    off += s;
  }
  split_offset[batch] = off;
  return ok();
}

int mla_plan_device(const int32_t* cache_seqlens, int32_t batch, int32_t heads, int32_t seqlen_q,
                    int32_t num_split, int32_t num_cus, int32_t* num_splits, int32_t* split_offset, int32_t* work,
                    int32_t max_work, hipStream_t stream) {
  int st;
  if (batch < 0 || heads < 1 || num_cus < 1) return fail(MLA_ERR_INVALID_ARG, "bad batch/heads/num_cus");
  if (seqlen_q < 0 || seqlen_q > mla::kMaxSeqlenQ) return fail(MLA_ERR_INVALID_ARG, "bad seqlen_q %d", seqlen_q);
  if (seqlen_q < 1) seqlen_q = 1;
  if ((st = check_num_split(num_split)) != MLA_OK) return st;
  if (batch > 0 && (!cache_seqlens || !num_splits || !work)) return fail(MLA_ERR_INVALID_ARG, "NULL array");
  if (!split_offset) return fail(MLA_ERR_INVALID_ARG, "NULL split_offset");
  const int64_t need = mla::max_splits(batch, heads, num_split, num_cus, seqlen_q);
  if (need > max_work) return fail(MLA_ERR_INVALID_ARG, "max_work %d < %lld", max_work, (long long)need);
  mla::PlanParams p{};
  p.seqlens = cache_seqlens;
  p.num_splits = num_splits;
  p.split_offset = split_offset;
  p.work = work;
  p.batch = batch;
  p.heads = heads;
  p.num_split = num_split;
  p.num_cus = num_cus;
  p.seqlen_q = seqlen_q;
  p.row_cap = INT32_MAX;
  hipError_t e = mla::launch_plan(p, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

// A plan made beforehand (mla_decode_planned): device arrays as
// mla_plan_device writes them, and the capacity they were made with.
struct GivenPlan {
  const int32_t* num_splits = nullptr;
  const int32_t* split_offset = nullptr;
  const int32_t* work = nullptr;
  int32_t max_work = 0;
};

// mla_decode, mla_decode_noalloc and mla_decode_planned.  noalloc: the
// workspace is this device's static scratch array (workspace /
// workspace_bytes are ignored); nothing here allocates (no events either).
// plan: non-null for mla_decode_planned (num_split is 0 then).
static int decode_impl(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
                       const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                       int32_t num_split, void* out, float* lse, const mla_desc* d, void* workspace,
                       size_t workspace_bytes, bool noalloc, hipStream_t stream, const GivenPlan* plan = nullptr) {
  int st;
  if ((st = check_desc(d)) != MLA_OK) return st;
  if ((st = check_num_split(num_split)) != MLA_OK) return st;
  if (plan) {
    if (!plan->num_splits || !plan->split_offset || !plan->work) return fail(MLA_ERR_INVALID_ARG, "NULL plan array");
    if (plan->max_work < 1) return fail(MLA_ERR_INVALID_ARG, "plan capacity max_work %d < 1", plan->max_work);
    if (!aligned(plan->num_splits, 4) || !aligned(plan->split_offset, 4) || !aligned(plan->work, 16))
      return fail(MLA_ERR_INVALID_ARG, "plan arrays must be 4-byte aligned (work 16-byte aligned)");
  }
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
  if (d->batch == 0) return ok();
  if (!q_nope || !q_pe || !kv_latent || !k_pe || !cache_seqlens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "NULL data pointer");
  // Element strides that keep rows 16-byte aligned: 8 16-bit elements, 16
  // bytes of an FP8 cache.
  const bool kv8 = d->kv_dtype == MLA_KV_FP8_E4M3;
  const int64_t strides[] = {d->q_nope_sb, d->q_nope_sh, d->q_pe_sb, d->q_pe_sh, d->kv_sb,
                             d->kv_sr,     d->kpe_sb,    d->kpe_sr,  d->out_sb,  d->out_sh};
  for (int i = 0; i < 10; ++i) {
    const int64_t s = strides[i];
    const int64_t unit = kv8 && i >= 4 && i < 8 ? 16 : 8;
    if (s < 0) return fail(MLA_ERR_INVALID_ARG, "negative stride %lld", (long long)s);
    if (s % unit)
      return fail(MLA_ERR_UNSUPPORTED, "stride %lld is not a multiple of %lld elements", (long long)s,
                  (long long)unit);
  }
  if (d->kv_sr >= MLA_MAX_ROW_STRIDE || d->kpe_sr >= MLA_MAX_ROW_STRIDE || d->q_nope_sh >= MLA_MAX_ROW_STRIDE ||
      d->q_pe_sh >= MLA_MAX_ROW_STRIDE)
    return fail(MLA_ERR_UNSUPPORTED, "cache row and query head strides must be below %d elements",
                MLA_MAX_ROW_STRIDE);
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(kv_latent, 16) || !aligned(k_pe, 16) ||
      !aligned(out, 16))
    return fail(MLA_ERR_UNSUPPORTED, "q/cache/out pointers must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cache_seqlens, 4) || (block_table && !aligned(block_table, 4)))
    return fail(MLA_ERR_INVALID_ARG, "lse/cache_seqlens/block_table must be 4-byte aligned");
  const bool paged = block_table != nullptr;
  int32_t row_cap;
  if (paged) {
    if (d->page_block_size < 32 || d->page_block_size % 32)
      return fail(MLA_ERR_UNSUPPORTED, "page_block_size %d must be a positive multiple of 32", d->page_block_size);
    if (d->block_table_stride < 1) return fail(MLA_ERR_INVALID_ARG, "block_table_stride < 1");
    if (d->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages < 1");
    const int64_t cap = (int64_t)d->block_table_stride * d->page_block_size;
    row_cap = cap > INT32_MAX ? INT32_MAX : (int32_t)cap;
  } else {
    if (d->max_seqlen < 0) return fail(MLA_ERR_INVALID_ARG, "max_seqlen < 0");
    row_cap = d->max_seqlen;
  }

  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int32_t num_cus = 0;
  if ((st = mla_num_cus(device, &num_cus)) != MLA_OK) return st;
  int32_t max_work;
  if (plan) max_work = plan->max_work;
  else if ((st = max_work_of(d, num_split, num_cus, &max_work)) != MLA_OK) return st;
  const Layout L = layout(d, max_work);
  if (noalloc) {
    if ((e = mla::noalloc_scratch(&workspace, &workspace_bytes)) != hipSuccess)
      return fail(MLA_ERR_HIP, "no-allocation scratch: %s", hipGetErrorString(e));
    if (L.total > workspace_bytes)
      return fail(MLA_ERR_WORKSPACE, "this problem needs %zu bytes of workspace, beyond the %zu bytes of the "
                  "no-allocation scratch (MLA_NOALLOC_SCRATCH_BYTES)", L.total, workspace_bytes);
  }
  if (!workspace || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? workspace_bytes : 0, L.total);
  if (!aligned(workspace, 256)) return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  char* ws = static_cast<char*>(workspace);
  int32_t* num_splits = reinterpret_cast<int32_t*>(ws + L.num_splits);
  int32_t* split_offset = reinterpret_cast<int32_t*>(ws + L.split_offset);
  int32_t* work = reinterpret_cast<int32_t*>(ws + L.work);
  float* part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  uint16_t* part16 = reinterpret_cast<uint16_t*>(ws + L.part16);
  float* part32 = reinterpret_cast<float*>(ws + L.part32);

  // In planner mode the split kernel plans for itself (no planner launch).
  mla::SplitParams sp{};
  sp.q_nope = static_cast<const uint16_t*>(q_nope);
  sp.q_pe = static_cast<const uint16_t*>(q_pe);
  sp.kv = kv_latent;
  sp.kpe = k_pe;
  sp.block_table = block_table;
  sp.seqlens = cache_seqlens;
  // With a plan made beforehand the kernels read (never write) the caller's
  // arrays; the workspace's plan region then goes unused.
  sp.num_splits = plan ? const_cast<int32_t*>(plan->num_splits) : num_splits;
  sp.split_offset = plan ? const_cast<int32_t*>(plan->split_offset) : split_offset;
  sp.work = plan ? const_cast<int32_t*>(plan->work) : work;

  sp.out = static_cast<uint16_t*>(out);
  sp.lse = lse;
  sp.part16 = part16;
  sp.part32 = part32;
  sp.part_lse = part_lse;
  sp.q_nope_sb = d->q_nope_sb;
  sp.q_nope_sh = d->q_nope_sh;
  sp.q_pe_sb = d->q_pe_sb;
  sp.q_pe_sh = d->q_pe_sh;
  sp.kv_sb = d->kv_sb;
  sp.kv_sr = d->kv_sr;
  sp.kpe_sb = d->kpe_sb;
  sp.kpe_sr = d->kpe_sr;
  sp.out_sb = d->out_sb;
  sp.out_sh = d->out_sh;
  // Forced mode: splits per sequence, the tail included.
  const int32_t seqlen_q = seqlen_q_of(d);
  const int32_t per_seq = num_split > 0 ? num_split + mla::tail_splits(seqlen_q) : 0;
  sp.num_split = plan ? mla::kPlanGiven : per_seq;
  sp.seqlen_q = seqlen_q;
  sp.heads_per_token = d->heads / seqlen_q;
  sp.batch = d->batch;
  sp.heads = d->heads;
  sp.page_size = paged ? d->page_block_size : 1;
  sp.bt_stride = paged ? d->block_table_stride : 0;
  sp.num_pages = paged ? d->num_pages : 0;
  sp.row_cap = row_cap;
  sp.num_cus = plan ? max_work : num_cus;
  // An FP8 cache's scale multiplies every score (folded into c) and the
  // output (out_scale); the products use the stored values.
  sp.scale_log2 = kv8 ? (float)((double)softmax_scale * (double)d->kv_scale * 1.4426950408889634)
                      : softmax_scale * 1.4426950408889634f;
  sp.out_scale = kv8 ? d->kv_scale : 1.f;
  // Timing (when enabled): each launch is timed from its dispatch packet.
  // Not in the no-allocation form (creating events may allocate).
  TimingSlot ts;
  hipEvent_t* ev = !noalloc && timing_slot(&ts) ? ts.ev : nullptr;
  if ((e = mla::launch_split(sp, d->dtype, paged, kv8, max_work, mla::head_groups(d->heads), stream,
                             ev ? ev[0] : nullptr, ev ? ev[1] : nullptr)) != hipSuccess)
    return fail(MLA_ERR_HIP, "split launch: %s", hipGetErrorString(e));

  if (per_seq != 1) {
    mla::CombineParams cp{};
    cp.part16 = part16;
    cp.part32 = part32;
    cp.part_lse = part_lse;
    cp.split_offset = sp.split_offset;
    cp.max_work = max_work;
    cp.out = static_cast<uint16_t*>(out);
    cp.lse = lse;
    cp.out_sb = d->out_sb;
    cp.out_sh = d->out_sh;
    cp.num_split = per_seq;
    cp.heads = d->heads;
    // Splits per sequence on average: forced, or at most max_work / B.
    const int mean_splits = per_seq > 0 ? per_seq : (max_work + d->batch - 1) / (d->batch > 0 ? d->batch : 1);
    if ((e = mla::launch_combine(cp, d->dtype, d->batch, mean_splits, stream, ev ? ev[2] : nullptr,
                                 ev ? ev[3] : nullptr)) != hipSuccess)
      return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    if (ev) {
      std::lock_guard<std::mutex> lk(g_tmu);
      g_combined[ts.index] = 1;
    }
  }
  return ok();
}

int mla_decode(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
               const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
               int32_t num_split, void* out, float* lse, const mla_desc* d, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale, num_split, out, lse,
                     d, workspace, workspace_bytes, false, stream);
}

int mla_decode_noalloc(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
                       const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                       int32_t num_split, void* out, float* lse, const mla_desc* d, hipStream_t stream) {
  return decode_impl(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale, num_split, out, lse,
                     d, nullptr, 0, true, stream);
}

int mla_decode_planned(const void* q_nope, const void* q_pe, const void* kv_latent, const void* k_pe,
                       const int32_t* block_table, const int32_t* cache_seqlens, float softmax_scale,
                       const int32_t* num_splits, const int32_t* split_offset, const int32_t* work,
                       int32_t max_work, void* out, float* lse, const mla_desc* d, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  GivenPlan plan;
  plan.num_splits = num_splits;
  plan.split_offset = split_offset;
  plan.work = work;
  plan.max_work = max_work;
  return decode_impl(q_nope, q_pe, kv_latent, k_pe, block_table, cache_seqlens, softmax_scale, 0, out, lse, d,
                     workspace, workspace_bytes, false, stream, &plan);
}

int mla_check_block_table(const int32_t* block_table, const int32_t* cache_seqlens, const mla_desc* d,
                          int32_t* bad, hipStream_t stream) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", d->batch);
  if (d->batch == 0) return ok();
  if (!block_table || !cache_seqlens || !bad) return fail(MLA_ERR_INVALID_ARG, "NULL array");
  if (!aligned(block_table, 4) || !aligned(cache_seqlens, 4) || !aligned(bad, 4))
    return fail(MLA_ERR_INVALID_ARG, "arrays must be 4-byte aligned");
  if (d->page_block_size < 32 || d->page_block_size % 32)
    return fail(MLA_ERR_UNSUPPORTED, "page_block_size %d must be a positive multiple of 32", d->page_block_size);
  if (d->block_table_stride < 1) return fail(MLA_ERR_INVALID_ARG, "block_table_stride < 1");
  if (d->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages < 1");
  mla::BlockCheckParams p{};
  p.block_table = block_table;
  p.seqlens = cache_seqlens;
  p.bad = bad;
  p.page_size = d->page_block_size;
  p.bt_stride = d->block_table_stride;
  p.num_pages = d->num_pages;
  const int64_t cap = (int64_t)d->block_table_stride * d->page_block_size;
  p.row_cap = cap > INT32_MAX ? INT32_MAX : (int32_t)cap;
  hipError_t e = mla::launch_check_block_table(p, d->batch, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "block-table check launch: %s", hipGetErrorString(e));
  return ok();
}

int mla_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  g_timed = 0;
  return ok();
}

int mla_timing_read(float* split_ms, float* combine_ms, int32_t* calls) {
  if (!split_ms || !combine_ms || !calls) return fail(MLA_ERR_INVALID_ARG, "NULL output");
  std::lock_guard<std::mutex> lk(g_tmu);
  double acc[2] = {0, 0};
  for (int i = 0; i < g_timed; ++i) {
    hipEvent_t* ev = &g_events[kEventsPerCall * (size_t)i];
    const int launches = g_combined[i] ? 2 : 1;
    hipError_t e = hipEventSynchronize(ev[2 * launches - 1]);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    for (int k = 0; k < launches; ++k) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]);
      if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
      acc[k] += ms;
    }
  }
  *split_ms = (float)acc[0];
  *combine_ms = (float)acc[1];
  *calls = g_timed;
  g_timed = 0;
  return ok();
}

}  // extern "C"
