// C-ABI shim of libgqa_decode: argument checks, workspace sizing, launch
// planning and dispatch. Every check runs on the host before anything is
// enqueued, so each error path is reachable without a GPU.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "gqa_decode.h"
#include "gqa_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return GQA_OK;
}

constexpr int kMaxBatch = 65535;
constexpr int kMaxHeads = 4096;
constexpr int kMaxTokens = 64;  // new tokens per sequence of a multi-token call
constexpr int kMaxLen = 1 << 28;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDefaultCUs = 256;  // MI355X, used when no device can be queried
// Empty schedule units ahead of each segment (lead units; see plan_decode).
constexpr int kSegmentLead8 = 2;       // eight-wave matrix kernel (up to 16 heads per KV head)
constexpr int kSegmentLead8Short = 3;  // ... when no segment is longer than kShortSegmentUnits
constexpr int kShortSegmentUnits = 24;
constexpr int kSegmentLead32 = 3;      // four-wave kernel, 17-32 heads
constexpr int kSegmentLead64 = 5;      // four-wave kernel, 33-64 heads
constexpr int kMaxSegmentLead = 5;
constexpr int kLeadMinUnits = 8;       // four-wave kernels: lead units only from this many units per workgroup
constexpr int kStreamLeadTiles = 6;    // one-block stream kernel: empty tiles ahead of each segment
constexpr int kStreamSplitMinTiles = 5;  // stream kernel, second-launch merge: tiles per workgroup at least

bool supported_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

// Compute units of the current device (cached per device, relaxed atomics:
// concurrent first calls store the same value; kDefaultCUs if the runtime
// cannot say).
int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  const int known = cached[dev].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = kDefaultCUs;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct Plan {
  int path;
  int gblk;
  int nhb;
  int workgroups;
  bool merge_kernel;  // shared segments merged by a second launch
  bool merge_spread;  // (stream kernel) shared segments merged at the end of the launch, a slice of heads by each part
  int seg_lead;       // empty schedule units ahead of each segment (tiles for the stream kernel)
  bool stream;        // the one-block stream kernel (decode_stream.hip)
};

// Largest head block any path may use for G heads per KV head (workspace sizing).
int gblk_bound(int G) {
  const int m = G < gqa::kMatrixMaxGroup ? G : gqa::kMatrixMaxGroup;
  const int v = gqa::vector_heads_per_block(G);
  return m > v ? m : v;
}

// Shared shape checks of the decode entry points (pointers are checked by the
// callers). Fills plan on success. workgroups: 0 = one per resident slot of
// the device (compute units x workgroups that fit per unit, at most two).
int plan_decode(int b, int h, int g, int d_k, int d_v, int cap, int max_len, int dtype, int path,
                int workgroups, Plan* plan, bool fused = false, bool paged = false, bool causal = false) {
  if (b <= 0 || b > kMaxBatch) return fail(GQA_ERR_ARG, "b=%d must be in [1, %d]", b, kMaxBatch);
  if (h <= 0 || h > kMaxHeads) return fail(GQA_ERR_ARG, "h=%d must be in [1, %d]", h, kMaxHeads);
  if (g <= 0) return fail(GQA_ERR_ARG, "g=%d must be positive", g);
  if (d_k <= 0 || d_v <= 0) return fail(GQA_ERR_ARG, "d_k=%d, d_v=%d must be positive", d_k, d_v);
  if (cap <= 0) return fail(GQA_ERR_ARG, "cap=%d must be positive", cap);
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (h % g != 0)
    return fail(GQA_ERR_GROUPS, "h=%d query heads cannot be split into g=%d equal groups", h, g);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "dtype=%d is not GQA_DTYPE_F32 or GQA_DTYPE_BF16", dtype);
  if (d_k != d_v || !supported_head_dim(d_k))
    return fail(GQA_ERR_UNSUPPORTED, "head dims d_k=%d, d_v=%d: need d_k == d_v in {16,32,64,128,256}",
                d_k, d_v);
  if (max_len > cap) return fail(GQA_ERR_CAPACITY, "max_len=%d exceeds cap=%d", max_len, cap);
  if (max_len > kMaxLen) return fail(GQA_ERR_UNSUPPORTED, "max_len=%d exceeds %d", max_len, kMaxLen);
  const int merge_flags = GQA_MERGE_INLINE | GQA_MERGE_KERNEL | GQA_MERGE_SPREAD;
  const int merge_req = path & merge_flags;
  const int path_req = path & ~merge_flags;
  if ((path_req != GQA_PATH_AUTO && path_req != GQA_PATH_VECTOR && path_req != GQA_PATH_MATRIX) ||
      (merge_req & (merge_req - 1)) != 0)
    return fail(GQA_ERR_UNSUPPORTED, "path=%d is not a GQA_PATH_* value, optionally with one GQA_MERGE_* flag",
                path);
  path = path_req;
  if (workgroups < 0 || workgroups > gqa::kMaxWorkgroups)
    return fail(GQA_ERR_UNSUPPORTED, "workgroups=%d must be in [0, %d]", workgroups, gqa::kMaxWorkgroups);

  const int G = h / g;
  const bool matrix_ok = dtype == GQA_DTYPE_BF16 && d_k == 128 && G <= gqa::kMatrixMaxGroup;
  if (path == GQA_PATH_MATRIX && !matrix_ok)
    return fail(GQA_ERR_UNSUPPORTED, "matrix path needs bf16, d=128 and at most 64 heads per KV head");
  int chosen = path;
  // Matrix cores pay once a K/V row serves three or more query heads; below
  // that the vector path keeps up with HBM on its own.
  if (chosen == GQA_PATH_AUTO) chosen = (matrix_ok && G >= 3) ? GQA_PATH_MATRIX : GQA_PATH_VECTOR;

  plan->path = chosen;
  if (chosen == GQA_PATH_MATRIX) {
    plan->gblk = G;
    plan->nhb = 1;
  } else {
    plan->gblk = gqa::vector_heads_per_block(G);
    plan->nhb = (G + plan->gblk - 1) / plan->gblk;
  }
  // At most 64 (virtual) heads per KV head and 64 sequences: the stream
  // kernel (tile-granular schedule, waves finishing pieces on their own).
  plan->stream = chosen == GQA_PATH_MATRIX && G <= gqa::kStreamMaxGroup && b <= gqa::kStreamMaxBatch;
  const int waves = plan->stream ? 8
                    : chosen == GQA_PATH_MATRIX ? gqa::matrix_waves(G) : gqa::vector_waves(dtype, d_k, plan->gblk);
  const int unit_len = plan->stream ? gqa::kTile : gqa::kTile * gqa::kUnitTiles;
  const long long segments = (long long)b * g * plan->nhb;
  // lengths <= max_len; kMaxSegmentLead: empty units ahead of each segment (at most)
  const long long units_plain = segments * ((max_len + unit_len - 1) / unit_len);
  const long long units_bound = units_plain + segments * (plan->stream ? kStreamLeadTiles : kMaxSegmentLead);
  const bool auto_grid = workgroups == 0;
  if (auto_grid) {
    // Up to eight waves per compute unit (two 4-wave workgroups or one
    // 8-wave one keep enough loads in flight), never more than fit at once, so
    // the persistent grid runs in a single round.
    int fit = plan->stream ? gqa::stream_workgroups_per_cu(fused, paged, G)
              : chosen == GQA_PATH_MATRIX ? gqa::matrix_workgroups_per_cu(G, fused, paged, causal)
                                          : gqa::vector_workgroups_per_cu(dtype, d_k, plan->gblk, fused, paged, causal);
    if (fit <= 0) fit = 2;  // no device to ask: assume the common case
    const int per_cu_max = 8 / waves;
    const int per_cu = fit < per_cu_max ? fit : per_cu_max;
    long long n = (long long)device_cus() * per_cu;
    if (n > units_bound) n = units_bound;
    if (n < 1) n = 1;
    if (n > gqa::kMaxWorkgroups) n = gqa::kMaxWorkgroups;
    workgroups = int(n);
  }
  // Merging a shared segment inside the decode kernel falls to the one
  // workgroup that arrives last, which reads all the segment's partial states
  // alone at the very end; past 64 KiB of them per segment a second launch
  // that merges with one workgroup per (segment, head) is faster. With 33-64
  // heads the stream kernel merges with two waves of 32 heads each; there
  // the limit is 48 KiB per wave, i.e. three parts (measured inline against
  // the second launch: three parts, the eight-token Llama-3-70B step 93 us
  // against 101, b = 64, h = 128, g = 2 at 2,048 positions 47 against 56;
  // four parts, b = 40, h = 64, g = 2, two tokens, 45.5 against 44; five
  // parts, b = 64, h = 64, g = 1, 45 against 36.5).
  plan->merge_spread = false;
  if (merge_req == GQA_MERGE_SPREAD) {
    if (!plan->stream || paged || causal)
      return fail(GQA_ERR_UNSUPPORTED,
                  "GQA_MERGE_SPREAD needs the stream kernel (bf16, d = 128, 3-64 heads per KV head, b <= 64) "
                  "on a contiguous cache with one query token per sequence");
    plan->merge_kernel = false;
    plan->merge_spread = true;
  } else if (merge_req == GQA_MERGE_KERNEL) {
    plan->merge_kernel = true;
  } else if (merge_req == GQA_MERGE_INLINE) {
    plan->merge_kernel = false;
  } else {
    const long long slots_per_segment = workgroups / (segments > 0 ? segments : 1) + 1;
    const long long per_head = slots_per_segment * d_v * 4;  // partial-state bytes per head
    plan->merge_kernel = plan->stream && plan->gblk > 32 ? per_head * 32 > 48 * 1024
                                                        : per_head * plan->gblk > 64 * 1024;
  }
  if (auto_grid && plan->stream && plan->merge_kernel) {
    // Merged by the second launch, a split segment costs one partial state
    // per part; where the parts would hold only a few tiles, fewer and longer
    // ones are faster: at least kStreamSplitMinTiles tiles (schedule units,
    // lead tiles included) per workgroup. MQA step, b = 8, h = 32, L = 4097
    // (1,080 units): 17.35 us at 256 workgroups, 16.7 at 224, 16.8 at 192,
    // 17.0 at 160; one long sequence per KV head (b = 4, L = 32769, 16 units
    // per workgroup at 256) is fastest on the whole chip and unchanged.
    const long long by_work = (units_bound + kStreamSplitMinTiles - 1) / kStreamSplitMinTiles;
    if (workgroups > by_work) workgroups = int(by_work > 0 ? by_work : 1);
  }
  if (auto_grid && !plan->merge_kernel && !plan->merge_spread) {
    // Inline merges: for large head groups keep at least G/2 tiles per
    // workgroup (at most 4 KiB of partial state per 16 KiB tile of K/V) so
    // that the single-workgroup merges stay small.
    const int min_tiles = plan->gblk / 2;
    const int min_units = plan->stream ? (min_tiles > 1 ? min_tiles : 1)
                          : min_tiles > gqa::kUnitTiles ? (min_tiles + gqa::kUnitTiles - 1) / gqa::kUnitTiles : 1;
    const long long by_work = (units_bound + min_units - 1) / min_units;
    if (workgroups > by_work) workgroups = int(by_work > 0 ? by_work : 1);
  }
  plan->workgroups = workgroups;
  // Lead units: empty units ahead of each segment in the schedule, so that a
  // range starting just before a segment skips them instead of opening a
  // piece of a unit or two there (each piece costs a query load, a merge of
  // the waves and a publish). On the matrix path, where ranges are long
  // against that cost, they pay off; measured best: 2 for the eight-wave
  // kernel (3 where segments are short, at most 24 units: the Qwen2.5-7B
  // shape at 2049 positions, -1.4 %; the Llama-3-70B shape, up to 64 units,
  // is 1.2 % slower with 3), 3 and 5 for the four-wave 32- and 64-head ones,
  // whose pieces cost more to merge and publish (4 and 8 new tokens per sequence on the
  // Llama-3-70B shape: -7 % and -14 %). Where a workgroup's range is a few
  // units (MQA, one long sequence per KV head) they only add imbalance, and
  // the vector path was measured neutral or slower.
  plan->seg_lead = 0;
  if (plan->stream) {
    plan->seg_lead = kStreamLeadTiles;
  } else if (chosen == GQA_PATH_MATRIX) {
    if (waves == 8) {
      const long long seg_units = (max_len + unit_len - 1) / unit_len;  // the longest segment
      plan->seg_lead = seg_units <= kShortSegmentUnits ? kSegmentLead8Short : kSegmentLead8;
    } else if (units_plain >= (long long)kLeadMinUnits * workgroups) {
      plan->seg_lead = G <= 32 ? kSegmentLead32 : kSegmentLead64;
    }
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

const char* gqa_last_error(void) { return g_last_error.c_str(); }

int gqa_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  int32_t* lens, int b, int g, int d_k, int d_v, int cap, int max_len,
                  int dtype, void* stream) {
  if (!k_cache || !v_cache || !k_new || !v_new || !lens)
    return fail(GQA_ERR_ARG, "gqa_kv_append: null pointer argument");
  if (b <= 0 || b > kMaxBatch) return fail(GQA_ERR_ARG, "b=%d must be in [1, %d]", b, kMaxBatch);
  if (g <= 0 || d_k <= 0 || d_v <= 0 || cap <= 0)
    return fail(GQA_ERR_ARG, "g=%d, d_k=%d, d_v=%d, cap=%d must be positive", g, d_k, d_v, cap);
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "dtype=%d is not GQA_DTYPE_F32 or GQA_DTYPE_BF16", dtype);
  if ((long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs cap > %d, cap=%d", max_len, max_len, cap);
  gqa::AppendParams p{k_cache, v_cache, k_new, v_new, lens, g, d_k, d_v, cap, gqa::PagedLayout{nullptr, 0, 0, 0}, 1};
  const hipError_t e = gqa::launch_append(p, b, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_kv_append launch: %s", hipGetErrorString(e));
  return ok();
}

size_t gqa_decode_workspace_size(int b, int h, int g, int d_k, int d_v, int max_len, int dtype) {
  if (b <= 0 || b > kMaxBatch || h <= 0 || h > kMaxHeads || g <= 0 || h % g != 0 || d_k <= 0 ||
      d_v <= 0 || max_len < 0 || max_len > kMaxLen || (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16))
    return 0;
  return gqa::workspace_layout(b, h, gblk_bound(h / g), d_v).total;
}

int gqa_decode_plan(int b, int h, int g, int d_k, int d_v, int cap, int max_len, int dtype,
                    int path, int workgroups, int* chosen_path, int* chosen_workgroups) {
  Plan plan;
  const int rc = plan_decode(b, h, g, d_k, d_v, cap, max_len, dtype, path, workgroups, &plan);
  if (rc != GQA_OK) return rc;
  if (chosen_path)
    *chosen_path = plan.path |
                   (plan.merge_spread ? GQA_MERGE_SPREAD : plan.merge_kernel ? GQA_MERGE_KERNEL : GQA_MERGE_INLINE) |
                   (plan.stream ? GQA_PLAN_STREAM : 0);
  if (chosen_workgroups) *chosen_workgroups = plan.workgroups;
  return ok();
}

}  // extern "C"

namespace {

// Checks and launch parameters of the attention and fused-step entry points
// (nothing is enqueued). max_len_att is the bound of the attended lengths
// (the appended token included).
int decode_prepare(const char* fn, void* out, const void* q, void* k_cache, void* v_cache, int32_t* lens,
                   const void* k_new, const void* v_new, int b, int h, int g, int d_k, int d_v, int cap,
                   int max_len_att, float scale, int dtype, void* workspace, size_t workspace_bytes, int path,
                   int workgroups, int fused, gqa::DecodeParams* pp, Plan* planp,
                   const gqa::PagedLayout* paged = nullptr, bool causal = false, bool slots_by_grid = false) {
  Plan& plan = *planp;
  const int rc = plan_decode(b, h, g, d_k, d_v, cap, max_len_att, dtype, path, workgroups, &plan, fused != 0,
                             paged != nullptr, causal);
  if (rc != GQA_OK) return rc;
  // Partial slots for every possible grid (the caller's workspace serves any
  // call of this shape), or only for the planned grid (the static scratch).
  const gqa::WorkspaceLayout ws = gqa::workspace_layout(b, h, gblk_bound(h / g), d_v,
                                                        slots_by_grid ? plan.workgroups : gqa::kMaxWorkgroups);
  if (!workspace) return fail(GQA_ERR_WORKSPACE, "%s: workspace is null (%zu bytes needed)", fn, ws.total);
  const size_t usable = workspace_bytes & ~size_t(255);
  if (usable < ws.total)
    return fail(GQA_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, ws.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(GQA_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);

  gqa::DecodeParams& p = *pp;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.lens = lens;
  p.k_new = k_new;
  p.v_new = v_new;
  char* wsb = static_cast<char*>(workspace);
  p.seg_info = reinterpret_cast<int2*>(wsb);
  p.ws_slots = reinterpret_cast<float*>(wsb + ws.info_bytes);
  p.ws_stamp = reinterpret_cast<int*>(wsb + usable - gqa::kStampBytes);
  p.ws_done = reinterpret_cast<int*>(wsb + usable - gqa::kStampBytes - gqa::kDoneBytes);
  p.ws_cnt = reinterpret_cast<int*>(wsb + usable - gqa::kStampBytes - gqa::kDoneBytes - ws.cnt_bytes);
  p.cnt_stride = int(gqa::counter_stride(b, h));
  p.merge_kernel = plan.merge_kernel ? 1 : 0;
  p.merge_spread = plan.merge_spread ? 1 : 0;
  p.b = b;
  p.h = h;
  p.g = g;
  p.G = h / g;
  p.d = d_k;
  p.cap = cap;
  p.max_len = max_len_att;
  p.fused = fused;
  p.gblk = plan.gblk;
  p.nhb = plan.nhb;
  p.ngroups = g * plan.nhb;
  p.slot_floats = gqa::slot_floats_for(plan.gblk, d_v);
  p.workgroups = plan.workgroups;
  p.seg_lead = plan.seg_lead;
  p.scale_log2 = scale * kLog2e;
  p.pg = paged ? *paged : gqa::PagedLayout{nullptr, 0, 0, 0};
  p.n_tok = 1;

  return GQA_OK;
}

int decode_launch(const char* fn, const gqa::DecodeParams& p, const Plan& plan, int dtype, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = plan.stream ? gqa::launch_decode_stream(p, st)
                 : plan.path == GQA_PATH_MATRIX ? gqa::launch_decode_matrix(p, st)
                                                : gqa::launch_decode_vector(p, dtype, st);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  if (plan.merge_kernel) {
    e = gqa::launch_merge_partials(p, dtype, st);
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s merge launch: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

// Shared body of the attention and fused-step entry points. max_len_att is
// the bound of the attended lengths (the appended token included).
int decode_common(const char* fn, void* out, const void* q, void* k_cache, void* v_cache, int32_t* lens,
                  const void* k_new, const void* v_new, int b, int h, int g, int d_k, int d_v, int cap,
                  int max_len_att, float scale, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream, int path, int workgroups, int fused) {
  gqa::DecodeParams p;
  Plan plan;
  const int rc = decode_prepare(fn, out, q, k_cache, v_cache, lens, k_new, v_new, b, h, g, d_k, d_v, cap,
                                max_len_att, scale, dtype, workspace, workspace_bytes, path, workgroups, fused,
                                &p, &plan);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// Checks of one linear projection (rows x n_in times n_out x n_in, bf16).
int linear_check(const char* fn, int rows, int n_in, int n_out, int dtype) {
  if (dtype != GQA_DTYPE_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: projections need bf16 (dtype=%d)", fn, dtype);
  if (rows <= 0 || rows > gqa::kLinearMaxRows)
    return fail(GQA_ERR_UNSUPPORTED, "%s: rows=%d must be in [1, %d]", fn, rows, gqa::kLinearMaxRows);
  if (n_in <= 0 || n_out <= 0) return fail(GQA_ERR_ARG, "%s: n_in=%d, n_out=%d must be positive", fn, n_in, n_out);
  if (n_in % 8 != 0) return fail(GQA_ERR_UNSUPPORTED, "%s: n_in=%d must be a multiple of 8", fn, n_in);
  return GQA_OK;
}

void linear_segment(gqa::LinearParams& lp, const void* w, void* y, int n_out) {
  const int s = lp.nseg++;
  lp.w[s] = static_cast<const uint16_t*>(w);
  lp.y[s] = static_cast<uint16_t*>(y);
  lp.n_out[s] = n_out;
  lp.blocks[s] = (n_out + 15) / 16;
}

}  // namespace

extern "C" {

int gqa_decode_attention_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                            int max_len, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream, int path, int workgroups) {
  if (!out || !q || !k_cache || !v_cache || !lens)
    return fail(GQA_ERR_ARG, "gqa_decode_attention: null pointer argument");
  // The attention kernels only read the caches and lens when not fused.
  return decode_common("gqa_decode_attention", out, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                       const_cast<int32_t*>(lens), nullptr, nullptr, b, h, g, d_k, d_v, cap, max_len, scale,
                       dtype, workspace, workspace_bytes, stream, path, workgroups, 0);
}

int gqa_decode_step_ex(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                       int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream, int path, int workgroups) {
  if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !lens)
    return fail(GQA_ERR_ARG, "gqa_decode_step: null pointer argument");
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (cap > 0 && (long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs cap > %d, cap=%d", max_len, max_len, cap);
  if (max_len == INT32_MAX) return fail(GQA_ERR_CAPACITY, "max_len=%d too large", max_len);
  return decode_common("gqa_decode_step", out, q, k_cache, v_cache, lens, k_new, v_new, b, h, g, d_k, d_v, cap,
                       max_len + 1, scale, dtype, workspace, workspace_bytes, stream, path, workgroups, 1);
}

int gqa_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap, int max_len,
                    float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return gqa_decode_step_ex(out, q, k_new, v_new, k_cache, v_cache, lens, b, h, g, d_k, d_v, cap, max_len, scale,
                            dtype, workspace, workspace_bytes, stream, GQA_PATH_AUTO, 0);
}

size_t gqa_packed_weight_bytes(int n_out, int n_in) {
  if (n_out <= 0 || n_in <= 0) return 0;
  return gqa::packed_weight_bytes(n_out, n_in);
}

int gqa_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if (!src || !sink) return fail(GQA_ERR_ARG, "gqa_read_bandwidth: null pointer argument");
  if (workgroups < 1 || workgroups > gqa::kMaxWorkgroups)
    return fail(GQA_ERR_ARG, "gqa_read_bandwidth: workgroups=%d must be in [1, %d]", workgroups, gqa::kMaxWorkgroups);
  if (bytes % 16 != 0 || !aligned16(src))
    return fail(GQA_ERR_ARG, "gqa_read_bandwidth: src must be 16-byte aligned and bytes=%zu a multiple of 16", bytes);
  // one workgroup's range is addressed with 32-bit offsets
  const size_t chunks_per_wg = (bytes / 16 + size_t(workgroups) - 1) / size_t(workgroups);
  if (chunks_per_wg > size_t(INT32_MAX) / 16)
    return fail(GQA_ERR_ARG, "gqa_read_bandwidth: %zu bytes over %d workgroups exceed 2 GiB per workgroup", bytes,
                workgroups);
  const hipError_t e = gqa::launch_read_bandwidth(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_read_bandwidth launch: %s", hipGetErrorString(e));
  return ok();
}

int gqa_fold_kv_heads(void* dst, const void* src, const int32_t* lens, int b, int g_src, int g_dst, int cap_src,
                      int cap_dst, int d, int max_rows, int dtype, void* stream) {
  if (!dst || !src) return fail(GQA_ERR_ARG, "gqa_fold_kv_heads: null pointer argument");
  if (b <= 0 || b > kMaxBatch || g_src <= 0 || g_dst <= 0 || g_dst > 65535 || cap_src <= 0 || cap_dst <= 0 ||
      d <= 0 || max_rows < 0)
    return fail(GQA_ERR_ARG, "gqa_fold_kv_heads: b=%d, g_src=%d, g_dst=%d, cap_src=%d, cap_dst=%d, d=%d, max_rows=%d",
                b, g_src, g_dst, cap_src, cap_dst, d, max_rows);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "gqa_fold_kv_heads: dtype=%d", dtype);
  if (g_src % g_dst != 0)
    return fail(GQA_ERR_GROUPS, "gqa_fold_kv_heads: g_src=%d is not a multiple of g_dst=%d", g_src, g_dst);
  if (d % 8 != 0) return fail(GQA_ERR_UNSUPPORTED, "gqa_fold_kv_heads: d=%d must be a multiple of 8", d);
  if (max_rows > cap_src || max_rows > cap_dst)
    return fail(GQA_ERR_CAPACITY, "gqa_fold_kv_heads: max_rows=%d exceeds cap_src=%d or cap_dst=%d", max_rows,
                cap_src, cap_dst);
  if ((long long)max_rows * d / 2048 >= (1LL << 31))
    return fail(GQA_ERR_ARG, "gqa_fold_kv_heads: max_rows * d too large");
  if (!aligned16(dst) || !aligned16(src)) return fail(GQA_ERR_ARG, "gqa_fold_kv_heads: dst and src must be 16-byte aligned");
  const size_t es = dtype == GQA_DTYPE_F32 ? 4 : 2;
  const size_t src_bytes = size_t(b) * g_src * size_t(cap_src) * d * es;
  const size_t dst_bytes = size_t(b) * g_dst * size_t(cap_dst) * d * es;
  const char* sp = static_cast<const char*>(src);
  const char* dp = static_cast<const char*>(dst);
  if (dp < sp + src_bytes && sp < dp + dst_bytes)
    return fail(GQA_ERR_ARG, "gqa_fold_kv_heads: dst and src overlap");
  if (max_rows == 0) return ok();
  const gqa::FoldParams p{dst, src, lens, g_src, g_dst, cap_src, cap_dst, d, max_rows};
  const hipError_t e = gqa::launch_fold(p, b, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_fold_kv_heads launch: %s", hipGetErrorString(e));
  return ok();
}

int gqa_pack_weight(void* dst, const void* src, int n_out, int n_in, int dtype, void* stream) {
  if (!dst || !src) return fail(GQA_ERR_ARG, "gqa_pack_weight: null pointer argument");
  if (n_out <= 0 || n_in <= 0) return fail(GQA_ERR_ARG, "gqa_pack_weight: n_out=%d, n_in=%d", n_out, n_in);
  if (dtype != GQA_DTYPE_BF16) return fail(GQA_ERR_UNSUPPORTED, "gqa_pack_weight: bf16 only (dtype=%d)", dtype);
  if (!aligned16(dst)) return fail(GQA_ERR_ARG, "gqa_pack_weight: dst must be 16-byte aligned");
  const hipError_t e = gqa::launch_pack_weight(dst, src, n_out, n_in, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_pack_weight launch: %s", hipGetErrorString(e));
  return ok();
}

int gqa_linear(void* y, const void* x, const void* w, int rows, int n_in, int n_out, int dtype, void* stream) {
  if (!y || !x || !w) return fail(GQA_ERR_ARG, "gqa_linear: null pointer argument");
  const int rc = linear_check("gqa_linear", rows, n_in, n_out, dtype);
  if (rc != GQA_OK) return rc;
  if (!aligned16(x) || !aligned16(w)) return fail(GQA_ERR_ARG, "gqa_linear: x and w must be 16-byte aligned");
  gqa::LinearParams lp{};
  lp.x = static_cast<const uint16_t*>(x);
  lp.rows = rows;
  lp.n_in = n_in;
  linear_segment(lp, w, y, n_out);
  const hipError_t e = gqa::launch_linear(lp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_linear launch: %s", hipGetErrorString(e));
  return ok();
}

int gqa_decode_layer(void* y, const void* x, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                     void* q, void* k_new, void* v_new, void* attn, void* k_cache, void* v_cache, int32_t* lens,
                     int b, int h, int g, int d_model, int d_k, int d_v, int cap, int max_len, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!y || !x || !w_q || !w_k || !w_v || !w_o || !q || !k_new || !v_new || !attn || !k_cache || !v_cache || !lens)
    return fail(GQA_ERR_ARG, "gqa_decode_layer: null pointer argument");
  if (d_model <= 0) return fail(GQA_ERR_ARG, "gqa_decode_layer: d_model=%d must be positive", d_model);
  if (h <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 || (long long)h * d_v > (1 << 30))
    return fail(GQA_ERR_ARG, "gqa_decode_layer: h=%d, g=%d, d_k=%d, d_v=%d", h, g, d_k, d_v);
  int rc = linear_check("gqa_decode_layer", b, d_model, 1, dtype);
  if (rc != GQA_OK) return rc;
  rc = linear_check("gqa_decode_layer", b, h * d_v, d_model, dtype);
  if (rc != GQA_OK) return rc;
  for (const void* ptr : {x, w_q, w_k, w_v, w_o, static_cast<const void*>(attn)})
    if (!aligned16(ptr)) return fail(GQA_ERR_ARG, "gqa_decode_layer: x, weights and attn must be 16-byte aligned");
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (cap > 0 && (long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs cap > %d, cap=%d", max_len, max_len, cap);
  if (max_len == INT32_MAX) return fail(GQA_ERR_CAPACITY, "max_len=%d too large", max_len);
  gqa::DecodeParams p;
  Plan plan;
  rc = decode_prepare("gqa_decode_layer", attn, q, k_cache, v_cache, lens, k_new, v_new, b, h, g, d_k, d_v, cap,
                      max_len + 1, scale, dtype, workspace, workspace_bytes, GQA_PATH_AUTO, 0, 1, &p, &plan);
  if (rc != GQA_OK) return rc;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  gqa::LinearParams qkv{};
  qkv.x = static_cast<const uint16_t*>(x);
  qkv.rows = b;
  qkv.n_in = d_model;
  linear_segment(qkv, w_q, q, h * d_k);
  linear_segment(qkv, w_k, k_new, g * d_k);
  linear_segment(qkv, w_v, v_new, g * d_v);
  hipError_t e = gqa::launch_linear(qkv, st);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_decode_layer projection launch: %s", hipGetErrorString(e));
  rc = decode_launch("gqa_decode_layer", p, plan, dtype, stream);
  if (rc != GQA_OK) return rc;
  gqa::LinearParams out{};
  out.x = static_cast<const uint16_t*>(attn);
  out.rows = b;
  out.n_in = h * d_v;
  linear_segment(out, w_o, y, d_model);
  e = gqa::launch_linear(out, st);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_decode_layer output projection launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Checks of a paged layout; fills pg and the positions one sequence can hold.
int paged_check(const char* fn, const int32_t* table, int b, int block_size, int max_blocks, int num_blocks,
                gqa::PagedLayout* pg, int* cap) {
  if (!table) return fail(GQA_ERR_ARG, "%s: block_table is null", fn);
  if (max_blocks <= 0 || num_blocks <= 0)
    return fail(GQA_ERR_ARG, "%s: max_blocks=%d, num_blocks=%d must be positive", fn, max_blocks, num_blocks);
  if (block_size < gqa::kTile || block_size > (1 << 20) || (block_size & (block_size - 1)) != 0)
    return fail(GQA_ERR_UNSUPPORTED, "%s: block_size=%d must be a power of two in [%d, 2^20]", fn, block_size,
                gqa::kTile);
  if (b > 0 && (long long)b * max_blocks >= (1LL << 31))
    return fail(GQA_ERR_ARG, "%s: the block table (b=%d x max_blocks=%d) is too large", fn, b, max_blocks);
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  *pg = gqa::PagedLayout{table, max_blocks, lg, num_blocks};
  const long long c = (long long)max_blocks * block_size;
  *cap = c > INT32_MAX ? INT32_MAX : int(c);
  return GQA_OK;
}

// Checks and launch parameters of a multi-token attention (nothing enqueued).
// The n tokens of a KV group are its n * G virtual heads: planned and laid
// out as a one-token call with n * h heads, then addressed through head_row.
// fused: the step's n appended rows are stored by the attention launch
// itself (k_new, v_new; the stream kernel only).
int multi_prepare(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* lens, int b, int n, int h, int g, int d_k, int d_v, int cap, int max_len, float scale,
                  int dtype, void* workspace, size_t workspace_bytes, gqa::DecodeParams* p, Plan* plan,
                  const gqa::PagedLayout* pg = nullptr, const void* k_new = nullptr, const void* v_new = nullptr,
                  bool fused = false) {
  if (!out || !q || !k_cache || !v_cache || !lens) return fail(GQA_ERR_ARG, "%s: null pointer argument", fn);
  if (n <= 0 || n > kMaxTokens) return fail(GQA_ERR_ARG, "%s: n=%d must be in [1, %d]", fn, n, kMaxTokens);
  if (h <= 0 || g <= 0 || (long long)n * h > kMaxHeads)
    return fail(GQA_ERR_ARG, "%s: h=%d, g=%d, n=%d (n * h at most %d)", fn, h, g, n, kMaxHeads);
  if (h % g != 0) return fail(GQA_ERR_GROUPS, "h=%d query heads cannot be split into g=%d equal groups", h, g);
  // planned like a one-token call with n * h heads: the matrix path when it
  // applies (bf16, d = 128, n * h/g in [3, 64]), else the vector path
  const int rc = decode_prepare(fn, out, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                const_cast<int32_t*>(lens), k_new, v_new, b, n * h, g, d_k, d_v, cap, max_len,
                                scale, dtype, workspace, workspace_bytes, GQA_PATH_AUTO, 0, fused ? n : 0, p, plan, pg,
                                n > 1);
  if (rc != GQA_OK) return rc;
  p->h = h;
  p->G = h / g;
  p->n_tok = n;
  return GQA_OK;
}

// Checks and launch of a multi-token append; cap is the positions a
// sequence can hold (max_blocks * block_size when pg is set).
int append_multi(const char* fn, void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t* lens,
                 int b, int n, int g, int d_k, int d_v, int cap, int max_len, int dtype, void* stream,
                 const gqa::PagedLayout& pg) {
  if (!k_cache || !v_cache || !k_new || !v_new || !lens) return fail(GQA_ERR_ARG, "%s: null pointer argument", fn);
  if (b <= 0 || b > kMaxBatch) return fail(GQA_ERR_ARG, "b=%d must be in [1, %d]", b, kMaxBatch);
  if (n <= 0 || n > kMaxTokens) return fail(GQA_ERR_ARG, "n=%d must be in [1, %d]", n, kMaxTokens);
  if (g <= 0 || d_k <= 0 || d_v <= 0 || cap <= 0)
    return fail(GQA_ERR_ARG, "g=%d, d_k=%d, d_v=%d, cap=%d must be positive", g, d_k, d_v, cap);
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "dtype=%d is not GQA_DTYPE_F32 or GQA_DTYPE_BF16", dtype);
  if ((long long)max_len + n > cap)
    return fail(GQA_ERR_CAPACITY, "%s: appending %d tokens to max_len=%d needs room for %lld positions, have %d", fn,
                n, max_len, (long long)max_len + n, cap);
  gqa::AppendParams p{k_cache, v_cache, k_new, v_new, lens, g, d_k, d_v, cap, pg, n};
  const hipError_t e = gqa::launch_append(p, b, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int gqa_kv_append_paged(void* k_pool, void* v_pool, const void* k_new, const void* v_new, int32_t* lens,
                        const int32_t* block_table, int b, int g, int d_k, int d_v, int block_size, int max_blocks,
                        int num_blocks, int max_len, int dtype, void* stream) {
  if (!k_pool || !v_pool || !k_new || !v_new || !lens)
    return fail(GQA_ERR_ARG, "gqa_kv_append_paged: null pointer argument");
  if (b <= 0 || b > kMaxBatch) return fail(GQA_ERR_ARG, "b=%d must be in [1, %d]", b, kMaxBatch);
  if (g <= 0 || d_k <= 0 || d_v <= 0) return fail(GQA_ERR_ARG, "g=%d, d_k=%d, d_v=%d must be positive", g, d_k, d_v);
  gqa::PagedLayout pg;
  int cap = 0;
  int rc = paged_check("gqa_kv_append_paged", block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "dtype=%d is not GQA_DTYPE_F32 or GQA_DTYPE_BF16", dtype);
  if ((long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs max_blocks * block_size > %d, have %d", max_len,
                max_len, cap);
  gqa::AppendParams p{k_pool, v_pool, k_new, v_new, lens, g, d_k, d_v, cap, pg, 1};
  const hipError_t e = gqa::launch_append(p, b, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "gqa_kv_append_paged launch: %s", hipGetErrorString(e));
  return ok();
}

int gqa_decode_attention_paged(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* lens, const int32_t* block_table, int b, int h, int g, int d_k,
                               int d_v, int block_size, int max_blocks, int num_blocks, int max_len, float scale,
                               int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_pool || !v_pool || !lens)
    return fail(GQA_ERR_ARG, "gqa_decode_attention_paged: null pointer argument");
  gqa::PagedLayout pg;
  int cap = 0;
  int rc = paged_check("gqa_decode_attention_paged", block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  gqa::DecodeParams p;
  Plan plan;
  rc = decode_prepare("gqa_decode_attention_paged", out, q, const_cast<void*>(k_pool), const_cast<void*>(v_pool),
                      const_cast<int32_t*>(lens), nullptr, nullptr, b, h, g, d_k, d_v, cap, max_len, scale, dtype,
                      workspace, workspace_bytes, GQA_PATH_AUTO, 0, 0, &p, &plan, &pg);
  if (rc != GQA_OK) return rc;
  return decode_launch("gqa_decode_attention_paged", p, plan, dtype, stream);
}

int gqa_decode_step_paged(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, int32_t* lens, const int32_t* block_table, int b, int h, int g, int d_k,
                          int d_v, int block_size, int max_blocks, int num_blocks, int max_len, float scale,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_new || !v_new || !k_pool || !v_pool || !lens)
    return fail(GQA_ERR_ARG, "gqa_decode_step_paged: null pointer argument");
  gqa::PagedLayout pg;
  int cap = 0;
  int rc = paged_check("gqa_decode_step_paged", block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if ((long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs max_blocks * block_size > %d, have %d", max_len,
                max_len, cap);
  if (max_len == INT32_MAX) return fail(GQA_ERR_CAPACITY, "max_len=%d too large", max_len);
  gqa::DecodeParams p;
  Plan plan;
  rc = decode_prepare("gqa_decode_step_paged", out, q, k_pool, v_pool, lens, k_new, v_new, b, h, g, d_k, d_v, cap,
                      max_len + 1, scale, dtype, workspace, workspace_bytes, GQA_PATH_AUTO, 0, 1, &p, &plan, &pg);
  if (rc != GQA_OK) return rc;
  return decode_launch("gqa_decode_step_paged", p, plan, dtype, stream);
}

size_t gqa_decode_multi_workspace_size(int b, int n, int h, int g, int d_k, int d_v, int dtype) {
  if (n <= 0 || n > kMaxTokens || h <= 0 || (long long)n * h > kMaxHeads) return 0;
  return gqa_decode_workspace_size(b, n * h, g, d_k, d_v, 0, dtype);
}

int gqa_kv_append_multi(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t* lens, int b,
                        int n, int g, int d_k, int d_v, int cap, int max_len, int dtype, void* stream) {
  return append_multi("gqa_kv_append_multi", k_cache, v_cache, k_new, v_new, lens, b, n, g, d_k, d_v, cap, max_len,
                      dtype, stream, gqa::PagedLayout{nullptr, 0, 0, 0});
}

int gqa_decode_attention_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* lens, int b, int n, int h, int g, int d_k, int d_v, int cap,
                               int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const char* fn = "gqa_decode_attention_multi";
  gqa::DecodeParams p;
  Plan plan;
  const int rc = multi_prepare(fn, out, q, k_cache, v_cache, lens, b, n, h, g, d_k, d_v, cap, max_len, scale, dtype,
                               workspace, workspace_bytes, &p, &plan);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

int gqa_decode_step_multi(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, int32_t* lens, int b, int n, int h, int g, int d_k, int d_v, int cap,
                          int max_len, float scale, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const char* fn = "gqa_decode_step_multi";
  if (!k_new || !v_new) return fail(GQA_ERR_ARG, "%s: null pointer argument", fn);
  if (max_len < 0 || max_len > INT32_MAX - kMaxTokens) return fail(GQA_ERR_ARG, "%s: max_len=%d out of range", fn, max_len);
  // every check of both launches runs before the first is enqueued
  gqa::DecodeParams p;
  Plan plan;
  int rc = multi_prepare(fn, out, q, k_cache, v_cache, lens, b, n, h, g, d_k, d_v, cap, max_len + n, scale, dtype,
                         workspace, workspace_bytes, &p, &plan);
  if (rc != GQA_OK) return rc;
  if (plan.stream) {  // one launch: the tiles holding the new positions store the new rows first
    rc = multi_prepare(fn, out, q, k_cache, v_cache, lens, b, n, h, g, d_k, d_v, cap, max_len + n, scale, dtype,
                       workspace, workspace_bytes, &p, &plan, nullptr, k_new, v_new, true);
    if (rc != GQA_OK) return rc;
    return decode_launch(fn, p, plan, dtype, stream);
  }
  rc = gqa_kv_append_multi(k_cache, v_cache, k_new, v_new, lens, b, n, g, d_k, d_v, cap, max_len, dtype, stream);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

int gqa_kv_append_multi_paged(void* k_pool, void* v_pool, const void* k_new, const void* v_new, int32_t* lens,
                              const int32_t* block_table, int b, int n, int g, int d_k, int d_v, int block_size,
                              int max_blocks, int num_blocks, int max_len, int dtype, void* stream) {
  const char* fn = "gqa_kv_append_multi_paged";
  gqa::PagedLayout pg;
  int cap = 0;
  const int rc = paged_check(fn, block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  return append_multi(fn, k_pool, v_pool, k_new, v_new, lens, b, n, g, d_k, d_v, cap, max_len, dtype, stream, pg);
}

int gqa_decode_attention_multi_paged(void* out, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* lens, const int32_t* block_table, int b, int n, int h, int g,
                                     int d_k, int d_v, int block_size, int max_blocks, int num_blocks, int max_len,
                                     float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gqa_decode_attention_multi_paged";
  gqa::PagedLayout pg;
  int cap = 0;
  int rc = paged_check(fn, block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  gqa::DecodeParams p;
  Plan plan;
  rc = multi_prepare(fn, out, q, k_pool, v_pool, lens, b, n, h, g, d_k, d_v, cap, max_len, scale, dtype, workspace,
                     workspace_bytes, &p, &plan, &pg);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

int gqa_decode_step_multi_paged(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                void* v_pool, int32_t* lens, const int32_t* block_table, int b, int n, int h, int g,
                                int d_k, int d_v, int block_size, int max_blocks, int num_blocks, int max_len,
                                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gqa_decode_step_multi_paged";
  if (!k_new || !v_new) return fail(GQA_ERR_ARG, "%s: null pointer argument", fn);
  if (max_len < 0 || max_len > INT32_MAX - kMaxTokens) return fail(GQA_ERR_ARG, "%s: max_len=%d out of range", fn, max_len);
  gqa::PagedLayout pg;
  int cap = 0;
  int rc = paged_check(fn, block_table, b, block_size, max_blocks, num_blocks, &pg, &cap);
  if (rc != GQA_OK) return rc;
  // every check of both launches runs before the first is enqueued
  gqa::DecodeParams p;
  Plan plan;
  rc = multi_prepare(fn, out, q, k_pool, v_pool, lens, b, n, h, g, d_k, d_v, cap, max_len + n, scale, dtype,
                     workspace, workspace_bytes, &p, &plan, &pg);
  if (rc != GQA_OK) return rc;
  if (plan.stream) {  // one launch, as in gqa_decode_step_multi
    rc = multi_prepare(fn, out, q, k_pool, v_pool, lens, b, n, h, g, d_k, d_v, cap, max_len + n, scale, dtype,
                       workspace, workspace_bytes, &p, &plan, &pg, k_new, v_new, true);
    if (rc != GQA_OK) return rc;
    return decode_launch(fn, p, plan, dtype, stream);
  }
  rc = append_multi(fn, k_pool, v_pool, k_new, v_new, lens, b, n, g, d_k, d_v, cap, max_len, dtype, stream, pg);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

int gqa_decode_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap,
                         int max_len, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return gqa_decode_attention_ex(out, q, k_cache, v_cache, lens, b, h, g, d_k, d_v, cap, max_len,
                                 scale, dtype, workspace, workspace_bytes, stream, GQA_PATH_AUTO, 0);
}

}  // extern "C"

// ----------------------------------------------------------- static scratch
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the fused
// step with its workspace in this file-scope device array instead of a
// caller buffer. Each GPU the library runs on holds its own copy (for the
// life of the process) at its own address, which is fetched once per device
// with hipGetSymbolAddress; host code uses that address, never the array's
// name (which on the host is only a stand-in). The counters the kernels need
// at zero are zero when the module is loaded and every call leaves them zero
// again; the partial states need no clearing. All calls on one GPU share
// the array, so calls that overlap on one GPU (different streams without
// synchronisation) race.
static constexpr size_t kStaticScratchBytes = size_t(8) << 20;  // 8 MiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of this device's scratch array (nullptr and an error
// message on failure). Concurrent first calls store the same address.
void* static_scratch(const char* fn) {
  static std::atomic<void*> addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(GQA_ERR_HIP, "%s: no usable current device (%s)", fn, hipGetErrorString(e));
    return nullptr;
  }
  void* known = addr[dev].load(std::memory_order_relaxed);
  if (known) return known;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    fail(GQA_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  addr[dev].store(ptr, std::memory_order_relaxed);
  return ptr;
}

}  // namespace

extern "C" {

int gqa_decode_step_static(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                           void* v_cache, int32_t* lens, int b, int h, int g, int d_k, int d_v, int cap, int max_len,
                           float scale, int dtype, void* stream) {
  const char* fn = "gqa_decode_step_static";
  if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !lens)
    return fail(GQA_ERR_ARG, "%s: null pointer argument", fn);
  if (max_len < 0) return fail(GQA_ERR_ARG, "max_len=%d must be >= 0", max_len);
  if (cap > 0 && (long long)max_len + 1 > cap)
    return fail(GQA_ERR_CAPACITY, "appending to max_len=%d needs cap > %d, cap=%d", max_len, max_len, cap);
  if (max_len == INT32_MAX) return fail(GQA_ERR_CAPACITY, "max_len=%d too large", max_len);
  // every shape check first (no device is needed for them), then the scratch
  // of the current device; the layout reserves partial slots for the planned
  // grid only, and a shape that needs more than the array holds is rejected
  Plan plan;
  int rc = plan_decode(b, h, g, d_k, d_v, cap, max_len + 1, dtype, GQA_PATH_AUTO, 0, &plan, true);
  if (rc != GQA_OK) return rc;
  const size_t need = gqa::workspace_layout(b, h, gblk_bound(h / g), d_v, plan.workgroups).total;
  if (need > kStaticScratchBytes)
    return fail(GQA_ERR_WORKSPACE, "%s: this shape needs %zu bytes of workspace, the static scratch holds %zu", fn,
                need, kStaticScratchBytes);
  void* ws = static_scratch(fn);
  if (!ws) return GQA_ERR_HIP;
  gqa::DecodeParams p;
  rc = decode_prepare(fn, out, q, k_cache, v_cache, lens, k_new, v_new, b, h, g, d_k, d_v, cap, max_len + 1, scale,
                      dtype, ws, kStaticScratchBytes, GQA_PATH_AUTO, 0, 1, &p, &plan, nullptr, false, true);
  if (rc != GQA_OK) return rc;
  return decode_launch(fn, p, plan, dtype, stream);
}

}  // extern "C"
