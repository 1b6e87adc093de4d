// pa_api.cpp - the C ABI declared in include/pa.h: host-side argument checks,
// split planning and kernel launches.  No allocation, no synchronisation.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>

#include "pa_kernels.h"
#include "pa_prefill.h"
#include "pa_rope.h"

namespace {

constexpr int32_t kMaxPartitionTokens = 2048;  // a split holds at most 128 pages
constexpr int32_t kTargetItems = 192;          // automatic choice: about this many large items per call
constexpr size_t kAlign = 256;

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
inline size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_dims(int32_t Hq, int32_t Hkv, int32_t D) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return PA_ERR_SHAPE;
  if (Hq != pa::kQHeads || Hkv != pa::kKvHeads || D != pa::kHeadDim) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

struct Plan {
  int32_t part_pages;  // 0: automatic (decided on the device from the batch)
  int32_t S;           // upper bound of any sequence's split count = partial rows per (b, h)
  size_t off_m, off_l, off_c, off_q, bytes;
};

// With partition_tokens > 0 a sequence of L tokens has ceil(L / partition_tokens)
// splits, independent of the rest of the batch.  With 0 the kernel picks the
// split size from the batch's total pages (at least 4 pages per split for
// batches of up to 64 sequences, 8 above).
int make_plan(int32_t B, int32_t max_blocks, int32_t partition_tokens, Plan* p) {
  if (partition_tokens < 0 || partition_tokens % pa::kPageTokens != 0) return PA_ERR_SHAPE;
  int32_t min_pages;
  if (partition_tokens == 0) {
    p->part_pages = 0;
    min_pages = pa::auto_split_min_pages(B);
  } else {
    const int32_t pt = partition_tokens > kMaxPartitionTokens ? kMaxPartitionTokens : partition_tokens;
    p->part_pages = pt / pa::kPageTokens;
    min_pages = p->part_pages;
  }
  p->S = (max_blocks + min_pages - 1) / min_pages;
  if (p->S < 1) p->S = 1;
  // part_o [B][Hq][S][D], part_m [B][Hq][S], part_l [B][Hq][S] (only when a
  // sequence can have several splits), counters int32 [B][Hkv], queue int32 [2]
  const size_t rows = p->S > 1 ? (size_t)B * pa::kQHeads * p->S : 0;
  p->off_m = round_up(rows * pa::kHeadDim * sizeof(float));
  p->off_l = p->off_m + round_up(rows * sizeof(float));
  p->off_c = p->off_l + round_up(rows * sizeof(float));
  p->off_q = p->off_c + round_up((size_t)B * pa::kKvHeads * sizeof(int32_t));
  p->bytes = p->off_q + kAlign;
  return PA_OK;
}

// Compute units of the current device (256 on MI355X).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  return 256;
}

// Workgroups the decode grid gets: an upper bound of the number of work items
// of a batch with one page count, capped at what the GPU holds at once (2
// workgroups per CU while the plan's LDS fits beside the page ring, else 1).
// Items beyond the workgroups that take them (a larger batch, or mixed
// lengths, which plan smaller items; batches of long items use one workgroup
// per CU) are handed out by the queue.

int decode_grid(int32_t B, int32_t max_blocks, const Plan& p) {
  uint64_t items;
  if (p.part_pages > 0) {
    items = (uint64_t)B * p.S;
  } else {
    // sum_b ceil(np_b / pp) < B + total/pp, and total/pp is at most kTargetItems
    // unless pp is capped at 128 pages, when it is at most ceil(B * max_blocks / 128)
    const uint64_t capped = ((uint64_t)B * (uint64_t)max_blocks + 127) / 128;
    const uint64_t bound = (uint64_t)B + (capped > (uint64_t)kTargetItems ? capped : (uint64_t)kTargetItems);
    const uint64_t all = (uint64_t)B * p.S;
    items = bound < all ? bound : all;
  }
  const int cus = device_cus();
  const int per_cu = pa::decode_lds_bytes(B) <= 80 * 1024 ? 2 : 1;
  const uint64_t cap = (uint64_t)cus * per_cu;
  return (int)(items < cap ? items : cap);
}

// Grid of a planned decode launch: every item can have a workgroup of its own,
// up to two workgroups per CU (the page ring leaves room for two), and no more
// workgroups than a plan deals to.  The plan is dealt for this grid.
int planned_grid(int32_t B, int32_t max_blocks, int32_t part_pages) {
  const size_t items = pa::plan_max_items(B, max_blocks, part_pages);
  size_t cap = 2 * (size_t)device_cus();
  if (cap > (size_t)pa::kPlanMaxBins) cap = pa::kPlanMaxBins;
  return (int)(items < cap ? items : cap);
}

// Bytes of a plan: the header and one 16-byte slot per item, plus the empty
// slots of a last round (fewer than one grid).
size_t plan_buffer_bytes(int32_t B, int32_t max_blocks, int32_t part_pages) {
  return pa::kPlanHeaderBytes + (pa::plan_max_items(B, max_blocks, part_pages) + pa::kPlanMaxBins) * 16;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size or value is out of range";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: only Hq=32, Hkv=8, D=64 are built";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: an array pointer is not 16-byte aligned";
    case PA_ERR_REJECTED: return "PA_ERR_REJECTED: the request's page budget exceeds the whole pool";
    case PA_ERR_BUDGET: return "PA_ERR_BUDGET: growth beyond the request's reserved prefix";
    case PA_ERR_STATE: return "PA_ERR_STATE: the request is not active";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more workspace than the fixed scratch array of "
             "pa_append_decode_noalloc holds (use pa_append_decode with a workspace)";
    default: return "unknown pa status";
  }
}

int32_t pa_default_partition_tokens(void) { return 0; }

int pa_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
              const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t B,
              int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream) {
  if (B < 0 || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT || num_pages <= 0 ||
      num_pages > INT32_MAX)
    return PA_ERR_SHAPE;
  if (Hkv <= 0 || D <= 0) return PA_ERR_SHAPE;
  if (Hkv != pa::kKvHeads || D != pa::kHeadDim) return PA_ERR_UNSUPPORTED;
  if (B == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens) return PA_ERR_NULL;
  if (misaligned(k_new) || misaligned(v_new) || misaligned(k_pool) || misaligned(v_pool))
    return PA_ERR_ALIGN;
  if (pa::launch_append(k_new, v_new, k_pool, v_pool, block_table, max_blocks, seq_lens, B,
                        stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

int pa_rope_append(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const float* cos_sin,
                   int32_t max_pos, uint16_t* q_out, uint16_t* k_pool, uint16_t* v_pool,
                   const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                   int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream) {
  if (B < 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT || max_pos <= 0 ||
      num_pages <= 0 || num_pages > INT32_MAX)
    return PA_ERR_SHAPE;
  const int dims = check_dims(Hq, Hkv, D);
  if (dims != PA_OK) return dims;
  if (B == 0) return PA_OK;
  if (!q || !k_new || !v_new || !cos_sin || !q_out || !k_pool || !v_pool || !block_table || !seq_lens)
    return PA_ERR_NULL;
  if (misaligned(q) || misaligned(k_new) || misaligned(v_new) || misaligned(cos_sin) || misaligned(q_out) ||
      misaligned(k_pool) || misaligned(v_pool))
    return PA_ERR_ALIGN;
  pa::RopeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cos_sin = cos_sin;
  a.q_out = q_out;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.max_pos = max_pos;
  a.num_pages = (int)num_pages;
  if (pa::launch_rope_append(a, stream) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

int pa_fill(const uint16_t* k_src, const uint16_t* v_src, uint16_t* k_pool, uint16_t* v_pool,
            const int32_t* block_table, int32_t max_blocks, const int32_t* start, const int32_t* cu_tokens,
            int32_t B, int64_t T, int32_t Hkv, int32_t D, int64_t num_pages, hipStream_t stream) {
  if (B < 0 || B > PA_MAX_FILL_BATCH || T < 0 || T > INT32_MAX - 16 || max_blocks <= 0 ||
      max_blocks > PA_MAX_BLOCKS_LIMIT || num_pages <= 0 || num_pages > INT32_MAX)
    return PA_ERR_SHAPE;
  if (Hkv <= 0 || D <= 0) return PA_ERR_SHAPE;
  if (Hkv != pa::kKvHeads || D != pa::kHeadDim) return PA_ERR_UNSUPPORTED;
  if (B == 0 || T == 0) return PA_OK;
  if (!k_src || !v_src || !k_pool || !v_pool || !block_table || !cu_tokens) return PA_ERR_NULL;
  if (misaligned(k_src) || misaligned(v_src) || misaligned(k_pool) || misaligned(v_pool)) return PA_ERR_ALIGN;
  pa::FillArgs a;
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.start = start;
  a.cu_tokens = cu_tokens;
  a.B = B;
  a.max_blocks = max_blocks;
  a.T = (int)T;
  a.num_pages = (int)num_pages;
  if (pa::launch_fill(a, stream) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

int pa_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu_tokens, int32_t B,
               int64_t T, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t weights, float* out,
               hipStream_t stream) {
  if (B <= 0 || B > PA_MAX_PREFILL_BATCH || T < 0 || T > PA_MAX_PREFILL_ROWS) return PA_ERR_SHAPE;
  if (weights != PA_PREFILL_WEIGHTS_BF16X2 && weights != PA_PREFILL_WEIGHTS_FP16) return PA_ERR_SHAPE;
  const int dims = check_dims(Hq, Hkv, D);
  if (dims != PA_OK) return dims;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (T == 0) return PA_OK;
  if (!q || !k || !v || !cu_tokens || !out) return PA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return PA_ERR_ALIGN;
  pa::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_tokens = cu_tokens;
  a.B = B;
  a.T = (int)T;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.fp16_weights = weights == PA_PREFILL_WEIGHTS_FP16;
  a.out = out;
  if (pa::launch_prefill(a, stream) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_blocks,
                                 int32_t partition_tokens) {
  if (B <= 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT) return 0;
  if (check_dims(Hq, pa::kKvHeads, D) != PA_OK) return 0;
  Plan p;
  if (make_plan(B, max_blocks, partition_tokens, &p) != PA_OK) return 0;
  return p.bytes;
}

size_t pa_decode_plan_bytes(int32_t B, int32_t max_blocks, int32_t partition_tokens) {
  if (B <= 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT) return 0;
  Plan p;
  if (make_plan(B, max_blocks, partition_tokens, &p) != PA_OK) return 0;
  return plan_buffer_bytes(B, max_blocks, p.part_pages);
}

int pa_decode_plan(const int32_t* seq_lens, int32_t B, int32_t max_blocks, int32_t partition_tokens, void* plan,
                   size_t plan_bytes, hipStream_t stream) {
  if (B < 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT) return PA_ERR_SHAPE;
  Plan p;
  const int pst = make_plan(B > 0 ? B : 1, max_blocks, partition_tokens, &p);
  if (pst != PA_OK) return pst;
  if (B == 0) return PA_OK;
  if (!seq_lens || !plan) return PA_ERR_NULL;
  if (misaligned(plan)) return PA_ERR_ALIGN;
  if (plan_bytes < plan_buffer_bytes(B, max_blocks, p.part_pages)) return PA_ERR_WORKSPACE;
  if (pa::launch_plan(seq_lens, B, max_blocks, p.part_pages, device_cus(), planned_grid(B, max_blocks, p.part_pages),
                      static_cast<int*>(plan), stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // extern "C"

namespace {

// Shared by pa_decode and pa_append_decode: checks, split plan, one launch.
int run_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
               const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, float scale,
               float* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages,
               int32_t partition_tokens, void* workspace, size_t workspace_bytes,
               const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool_w, uint16_t* v_pool_w,
               bool fused_append, const float* cos_sin, int32_t max_pos, hipStream_t stream,
               bool clear_counters = false, bool planned = false, const void* plan_buf = nullptr,
               size_t plan_bytes = 0) {
  const bool rope = cos_sin != nullptr || max_pos != 0;
  if (B < 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT ||
      num_pages <= 0 || num_pages > INT32_MAX || !isfinite(scale))
    return PA_ERR_SHAPE;
  const int dims = check_dims(Hq, Hkv, D);
  if (dims != PA_OK) return dims;
  Plan plan;
  const int pst = make_plan(B > 0 ? B : 1, max_blocks, partition_tokens, &plan);
  if (pst != PA_OK) return pst;
  if (B == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_table || (!seq_lens && !planned) || !out) return PA_ERR_NULL;
  if (planned) {  // the plan carries the lengths
    if (!plan_buf) return PA_ERR_NULL;
    if (misaligned(plan_buf)) return PA_ERR_ALIGN;
    if (plan_bytes < plan_buffer_bytes(B, max_blocks, plan.part_pages)) return PA_ERR_WORKSPACE;
  }
  if (fused_append && (!k_new || !v_new)) return PA_ERR_NULL;
  if (misaligned(q) || misaligned(k_pool) || misaligned(v_pool) || misaligned(out))
    return PA_ERR_ALIGN;
  if (fused_append && (misaligned(k_new) || misaligned(v_new))) return PA_ERR_ALIGN;
  if (rope) {  // the table covers every position the block table can address
    if ((int64_t)max_pos < (int64_t)max_blocks * pa::kPageTokens) return PA_ERR_SHAPE;
    if (!cos_sin) return PA_ERR_NULL;
    if (misaligned(cos_sin)) return PA_ERR_ALIGN;
  }
  if (!workspace || workspace_bytes < plan.bytes) return PA_ERR_WORKSPACE;
  if (misaligned(workspace)) return PA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  pa::DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool_w = k_pool_w;
  a.v_pool_w = v_pool_w;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_o = plan.S > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_m = plan.S > 1 ? reinterpret_cast<float*>(ws + plan.off_m) : nullptr;
  a.part_l = plan.S > 1 ? reinterpret_cast<float*>(ws + plan.off_l) : nullptr;
  a.counters = reinterpret_cast<int*>(ws + plan.off_c);
  a.B = B;
  a.max_blocks = max_blocks;
  a.part_pages = plan.part_pages;
  a.S = plan.S;
  a.scale_log2 = scale * 1.4426950408889634f;
  // the plan when every sequence fills its table row
  a.guess_pp = plan.part_pages > 0 ? plan.part_pages : pa::auto_split_pages((long long)B * max_blocks, B);
  a.guess_ns = (max_blocks + a.guess_pp - 1) / a.guess_pp;
  a.guess_magic = a.guess_ns > 1 ? (uint32_t)(((1ull << 32) + a.guess_ns - 1) / a.guess_ns) : 0u;
  const int grid = planned ? planned_grid(B, max_blocks, plan.part_pages) : decode_grid(B, max_blocks, plan);
  // batches of long items run one workgroup per CU (the kernel decides from the lengths)
  a.narrow = device_cus();
  // the kernel uses the queue only when the plan has more items than the grid
  a.queue = reinterpret_cast<int*>(ws + plan.off_q);
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.plan = static_cast<const int*>(plan_buf);
  // the counters and the queue, which the kernel needs at zero (contiguous)
  if (clear_counters &&
      pa::launch_clear(a.counters, (int)((plan.off_q - plan.off_c) / sizeof(int)) + 2, stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  const hipError_t err = planned ? pa::launch_decode_planned(a, grid, fused_append, rope, stream)
                                 : pa::launch_decode(a, grid, fused_append, rope, stream);
  if (err != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free decode.  The workspace of pa_append_decode_noalloc is this
// file-scope device array: every GPU the library runs on holds its own copy
// (PA_NOALLOC_SCRATCH_BYTES) from the first use until the process ends.  Host
// code never passes the array's name to a kernel (on the host it only names a
// stand-in); it passes the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device and kept here.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// Device address of this device's scratch array, or nullptr if it cannot be found.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* found = nullptr;
  if (hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)) != hipSuccess || !found) return nullptr;
  g_scratch_ptr[dev].store(found, std::memory_order_release);  // a racing lookup stores the same address
  return found;
}

}  // namespace

extern "C" {

int pa_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
              const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, float scale,
              float* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  return run_decode(q, k_pool, v_pool, block_table, max_blocks, seq_lens, scale, out, B, Hq, Hkv, D,
                    num_pages, partition_tokens, workspace, workspace_bytes, nullptr, nullptr,
                    nullptr, nullptr, false, nullptr, 0, stream);
}

int pa_append_decode(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                     uint16_t* v_pool, const uint16_t* q, const int32_t* block_table,
                     int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                     int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(q, k_pool, v_pool, block_table, max_blocks, seq_lens, scale, out, B, Hq, Hkv, D,
                    num_pages, partition_tokens, workspace, workspace_bytes, k_new, v_new, k_pool,
                    v_pool, true, nullptr, 0, stream);
}

int pa_rope_append_decode(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool, uint16_t* v_pool,
                          const uint16_t* q, const float* cos_sin, int32_t max_pos, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (max_pos <= 0) return PA_ERR_SHAPE;
  return run_decode(q, k_pool, v_pool, block_table, max_blocks, seq_lens, scale, out, B, Hq, Hkv, D,
                    num_pages, partition_tokens, workspace, workspace_bytes, k_new, v_new, k_pool,
                    v_pool, true, cos_sin, max_pos, stream);
}

int pa_append_decode_noalloc(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                             uint16_t* v_pool, const uint16_t* q, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, float scale, float* out, int32_t B,
                             int32_t Hq, int32_t Hkv, int32_t D, int64_t num_pages, int32_t partition_tokens,
                             hipStream_t stream) {
  // sizes first, so that an oversized call is refused before the device is touched
  if (B < 0 || B > pa::kMaxDecodeBatch || max_blocks <= 0 || max_blocks > PA_MAX_BLOCKS_LIMIT)
    return PA_ERR_SHAPE;
  const int dims = check_dims(Hq, Hkv, D);
  if (dims != PA_OK) return dims;
  Plan plan;
  const int pst = make_plan(B > 0 ? B : 1, max_blocks, partition_tokens, &plan);
  if (pst != PA_OK) return pst;
  if (plan.bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  if (B == 0) return PA_OK;
  void* ws = scratch_on_current_device();
  if (!ws) return PA_ERR_LAUNCH;
  return run_decode(q, k_pool, v_pool, block_table, max_blocks, seq_lens, scale, out, B, Hq, Hkv, D, num_pages,
                    partition_tokens, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, k_new, v_new, k_pool, v_pool, true,
                    nullptr, 0, stream, /*clear_counters=*/true);
}

int pa_decode_planned(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const float* cos_sin,
                      int32_t max_pos, uint16_t* k_pool, uint16_t* v_pool, const int32_t* block_table,
                      int32_t max_blocks, float scale, float* out, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                      int64_t num_pages, int32_t partition_tokens, const void* plan, size_t plan_bytes,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool append = k_new != nullptr || v_new != nullptr;
  if (cos_sin && !append) return PA_ERR_NULL;  // RoPE rotates the key it appends
  if (cos_sin && max_pos <= 0) return PA_ERR_SHAPE;
  return run_decode(q, k_pool, v_pool, block_table, max_blocks, nullptr, scale, out, B, Hq, Hkv, D, num_pages,
                    partition_tokens, workspace, workspace_bytes, k_new, v_new, append ? k_pool : nullptr,
                    append ? v_pool : nullptr, append, cos_sin, cos_sin ? max_pos : 0, stream,
                    /*clear_counters=*/false, /*planned=*/true, plan, plan_bytes);
}

int pa_merge(const float* part_o, const float* part_m, const float* part_l,
             const int32_t* seq_lens, int32_t partition_tokens, float* out, int32_t B, int32_t Hq,
             int32_t D, int32_t S, hipStream_t stream) {
  if (B < 0 || S <= 0 || S > PA_MAX_BLOCKS_LIMIT) return PA_ERR_SHAPE;
  const int dims = check_dims(Hq, pa::kKvHeads, D);
  if (dims != PA_OK) return dims;
  if (seq_lens && (partition_tokens <= 0 || partition_tokens % pa::kPageTokens != 0))
    return PA_ERR_SHAPE;
  if (B == 0) return PA_OK;
  if (!part_o || !part_m || !part_l || !out) return PA_ERR_NULL;
  if (misaligned(part_o) || misaligned(out)) return PA_ERR_ALIGN;
  pa::MergeArgs m;
  m.B = B;
  m.part_o = part_o;
  m.part_m = part_m;
  m.part_l = part_l;
  m.seq_lens = seq_lens;
  m.out = out;
  // the splits pa_decode makes: partition_tokens above 2048 act as 2048 there
  m.part_tokens = seq_lens ? (partition_tokens > kMaxPartitionTokens ? kMaxPartitionTokens : partition_tokens) : 0;
  m.S = S;
  m.skip_single = 0;
  if ((uint64_t)B * pa::kQHeads * 16 >= (1ull << 32)) return PA_ERR_SHAPE;
  if (pa::launch_merge(m, stream) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // extern "C"
