// C ABI of libmoefp8: host-side validation, workspace planning and the
// launch sequence of the expert layer. Nothing here allocates or
// synchronizes; every argument is checked before the first HIP call, so an
// invalid request returns an error with nothing enqueued.
#include <atomic>
#include <climits>
#include <mutex>

#include "../../include/moe_fp8.h"
#include "kernels.h"

static_assert(MOE_DECODE_MAX_PAIRS == moe::kDcMaxPairs && MOE_DECODE_FC2_ROW_BYTES == moe::kDcTokBytes &&
                  MOE_DECODE_FC2_MAX_SCALES == moe::kDcMaxScales &&
                  MOE_DECODE_LAYER_TOKEN_BYTES == moe::kF1TokBytesWide &&
                  MOE_DECODE_LAYER_MAX_SCALES == moe::kF1MaxScalesWide,
              "the header's decode limits are the kernels'");

namespace moe {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace moe

// Workspace of moe_forward_noalloc: one copy per device, held until the
// process ends. Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxTopk = 64;
constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup failed.
void* scratch_address() {
  static std::atomic<void*> cache[kMaxDevices];
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> g(lock);
  ptr = cache[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    cache[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

bool fmt_ok(int f) { return f == MOE_SCALE_FP32 || f == MOE_SCALE_FP32_POW2 || f == MOE_SCALE_UE8M0; }
bool act_ok(int a) {
  return a == MOE_ACT_SWIGLU || a == MOE_ACT_SWIGLU_CLAMP || a == MOE_ACT_SWIGLU_CLAMP_AFTER_SILU;
}
bool rounding_ok(int r) { return r == MOE_ROUND_DIVIDE || r == MOE_ROUND_RECIPROCAL; }
bool dim128(int32_t d) { return d > 0 && d % 128 == 0; }
// Limits of the GEMM kernels: k <= 32768 (per-tile weight scale table in
// LDS) and 32-bit byte offsets within one operand (a_rows * k and one
// expert's n * k below 2^32).
bool gemm_shape_ok(int64_t a_rows, int64_t n, int64_t k) {
  return k <= 32768 && a_rows * k < (int64_t{1} << 32) && n * k < (int64_t{1} << 32);
}
size_t scale_bytes(int fmt) { return fmt == MOE_SCALE_UE8M0 ? 1 : 4; }
moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Rows any routing of t_cap tokens can need: with n <= min(E, pairs) experts
// in use, sum_e ceil(c_e / A) <= floor((pairs + n * (A - 1)) / A).
int64_t min_row_cap64(int64_t t_cap, int64_t topk, int64_t num_experts, int64_t align_rows) {
  const int64_t pairs = t_cap * topk;
  const int64_t used = num_experts < pairs ? num_experts : pairs;
  return (pairs + used * (align_rows - 1)) / align_rows * align_rows;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" {

int32_t moe_min_row_cap(int32_t t_cap, int32_t topk, int32_t num_experts, int32_t align_rows) {
  if (t_cap < 0 || topk < 1 || num_experts < 1 || align_rows < 1) return -1;
  const int64_t v = min_row_cap64(t_cap, topk, num_experts, align_rows);
  return v > INT32_MAX ? -1 : static_cast<int32_t>(v);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_CAPACITY: return "capacity too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

moe_status moe_align(const int32_t* topk_ids, int32_t t_cap, const int32_t* t_live_dev,
                     int32_t topk, int32_t num_experts, int32_t expert_start, int32_t align_rows,
                     int32_t row_cap, int32_t* expert_counts, int32_t* expert_offsets,
                     int32_t* row_to_pair, int32_t* pair_to_row, void* stream) {
  if (t_cap < 0 || topk < 1 || topk > kMaxTopk || num_experts < 1 || align_rows < 1 || row_cap < 0)
    return MOE_ERR_INVALID_ARG;
  if (num_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(t_cap) * topk > INT32_MAX / 2) return MOE_ERR_INVALID_ARG;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (t_cap > 0 && (!topk_ids || !row_to_pair || !pair_to_row)) return MOE_ERR_INVALID_ARG;
  if (row_cap < min_row_cap64(t_cap, topk, num_experts, align_rows)) return MOE_ERR_CAPACITY;
  moe::AlignMode mode;
  mode.expert_start = expert_start;
  return from_hip(moe::launch_align(topk_ids, t_cap, t_live_dev, topk, num_experts, align_rows,
                                    expert_counts, expert_offsets, row_to_pair, pair_to_row, mode,
                                    as_stream(stream)));
}

moe_status moe_align_batched(const int32_t* topk_ids, int32_t t_cap, const int32_t* t_live_dev,
                             int32_t topk, int32_t num_experts, int32_t expert_start,
                             int32_t expert_cap, int32_t* masked_m, int32_t* row_to_pair,
                             int32_t* pair_to_row, int32_t* overflow, void* stream) {
  if (t_cap < 0 || topk < 1 || topk > kMaxTopk || num_experts < 1 || expert_cap < 1)
    return MOE_ERR_INVALID_ARG;
  if (num_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(t_cap) * topk > INT32_MAX / 2 ||
      static_cast<int64_t>(num_experts) * expert_cap > INT32_MAX / 2)
    return MOE_ERR_INVALID_ARG;
  if (!masked_m) return MOE_ERR_INVALID_ARG;
  if (t_cap > 0 && (!topk_ids || !row_to_pair || !pair_to_row)) return MOE_ERR_INVALID_ARG;
  moe::AlignMode mode;
  mode.expert_start = expert_start;
  mode.batch_cap = expert_cap;
  mode.overflow = overflow;
  // The fixed segments' endpoints e*cap are implicit: no offsets output.
  return from_hip(moe::launch_align(topk_ids, t_cap, t_live_dev, topk, num_experts, 1, masked_m,
                                    nullptr, row_to_pair, pair_to_row, mode, as_stream(stream)));
}

moe_status moe_act_quant(const uint16_t* x, int32_t t_cap, const int32_t* t_live_dev,
                         int32_t hidden, moe_scale_fmt fmt, moe_rounding rounding, uint8_t* xq,
                         void* xs, void* stream) {
  if (t_cap < 0 || !dim128(hidden) || !fmt_ok(fmt) || !rounding_ok(rounding))
    return MOE_ERR_INVALID_ARG;
  if (t_cap > 0 && (!x || !xq || !xs)) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(t_cap) * (hidden / 128) > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (t_cap == 0) return MOE_OK;
  return from_hip(moe::launch_act_quant(x, t_cap, t_live_dev, hidden, fmt, rounding, xq, xs,
                                        as_stream(stream)));
}

static moe_status gemm_checked(const moe::GemmArgs& g, void* stream) {
  if (!dim128(g.n) || !dim128(g.k) || !fmt_ok(g.fmt) || g.a_rows < 0 || g.a_row_div < 1 ||
      g.num_experts < 1 || g.row_cap < 0)
    return MOE_ERR_INVALID_ARG;
  if (g.num_experts > moe::kMaxExperts || !gemm_shape_ok(g.a_rows, g.n, g.k))
    return MOE_ERR_UNSUPPORTED;
  if (!g.counts || (!g.offsets && g.seg_cap == 0) || !g.w || !g.w_scales) return MOE_ERR_INVALID_ARG;
  if (g.row_cap > 0 && (!g.c || !g.a || !g.a_scales)) return MOE_ERR_INVALID_ARG;
  if (g.row_cap == 0) return MOE_OK;
  return from_hip(moe::launch_grouped_gemm(g, as_stream(stream)));
}

moe_status moe_grouped_gemm_fp8(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                const uint8_t* w, const float* w_scales,
                                const int32_t* expert_counts, const int32_t* expert_offsets,
                                int32_t num_experts, int32_t row_cap, int32_t max_rows_per_expert,
                                int32_t n, int32_t k, uint16_t* c, int32_t* tiles_visited,
                                void* stream) {
  if (max_rows_per_expert < 0) return MOE_ERR_INVALID_ARG;
  moe::GemmArgs g;
  g.a = a;
  g.a_scales = a_scales;
  g.fmt = fmt;
  g.a_rows = a_rows;
  g.a_row_map = a_row_map;
  g.a_row_div = a_row_div;
  g.w = w;
  g.w_scales = w_scales;
  g.counts = expert_counts;
  g.offsets = expert_offsets;
  g.num_experts = num_experts;
  g.row_cap = row_cap;
  g.max_rows_per_expert =
      (max_rows_per_expert == 0 || max_rows_per_expert > row_cap) ? row_cap : max_rows_per_expert;
  g.max_live_experts = row_cap < num_experts ? row_cap : num_experts;
  g.n = n;
  g.k = k;
  g.c = c;
  g.tiles_visited = tiles_visited;
  return gemm_checked(g, stream);
}

moe_status moe_grouped_gemm_fp8_masked(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                       int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                       const uint8_t* w, const float* w_scales,
                                       const int32_t* masked_m, int32_t num_experts,
                                       int32_t expert_cap, int32_t n, int32_t k, uint16_t* c,
                                       int32_t* tiles_visited, void* stream) {
  if (expert_cap < 1 || num_experts < 1) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_experts) * expert_cap > INT32_MAX / 2) return MOE_ERR_INVALID_ARG;
  const int32_t rows = num_experts * expert_cap;
  moe::GemmArgs g;
  g.a = a;
  g.a_scales = a_scales;
  g.fmt = fmt;
  g.a_rows = a_rows;
  g.a_row_map = a_row_map;
  g.a_row_div = a_row_div;
  g.w = w;
  g.w_scales = w_scales;
  g.counts = masked_m;
  g.offsets = nullptr;
  g.seg_cap = expert_cap;
  g.num_experts = num_experts;
  g.row_cap = rows;
  g.max_rows_per_expert = expert_cap;
  g.max_live_experts = num_experts;
  g.n = n;
  g.k = k;
  g.c = c;
  g.tiles_visited = tiles_visited;
  return gemm_checked(g, stream);
}

static moe_status gemm_w4_checked(const moe::W4Args& g, void* stream) {
  if (!dim128(g.n) || !dim128(g.k) || !fmt_ok(g.fmt) || g.a_rows < 0 || g.a_row_div < 1 ||
      g.num_experts < 1 || g.row_cap < 0 || g.seg_cap < 0)
    return MOE_ERR_INVALID_ARG;
  if (g.seg_cap > 0 && static_cast<int64_t>(g.seg_cap) * g.num_experts != g.row_cap)
    return MOE_ERR_INVALID_ARG;
  if (g.num_experts > moe::kMaxExperts || !gemm_shape_ok(g.a_rows, g.n, g.k))
    return MOE_ERR_UNSUPPORTED;
  if (!g.counts || (!g.offsets && g.seg_cap == 0) || !g.w || !g.w_scales) return MOE_ERR_INVALID_ARG;
  if (g.row_cap > 0 && (!g.c || !g.a || !g.a_scales || g.a_rows < 1)) return MOE_ERR_INVALID_ARG;
  if (g.row_cap == 0) return MOE_OK;
  return from_hip(moe::launch_grouped_gemm_w4(g, as_stream(stream)));
}

moe_status moe_grouped_gemm_mxfp4(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                  int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                  const uint8_t* w, const uint8_t* w_scales,
                                  const int32_t* expert_counts, const int32_t* expert_offsets,
                                  int32_t expert_cap, int32_t num_experts, int32_t row_cap,
                                  int32_t max_rows_per_expert, int32_t n, int32_t k, uint16_t* c,
                                  void* stream) {
  if (max_rows_per_expert < 0) return MOE_ERR_INVALID_ARG;
  moe::W4Args g;
  g.a = a;
  g.a_scales = a_scales;
  g.fmt = fmt;
  g.a_rows = a_rows;
  g.a_row_map = a_row_map;
  g.a_row_div = a_row_div;
  g.w = w;
  g.w_scales = w_scales;
  g.counts = expert_counts;
  g.offsets = expert_offsets;
  g.seg_cap = expert_cap;
  g.num_experts = num_experts;
  g.row_cap = row_cap;
  const int32_t seg = expert_cap > 0 ? expert_cap : row_cap;
  g.max_rows_per_expert = (max_rows_per_expert == 0 || max_rows_per_expert > seg) ? seg : max_rows_per_expert;
  g.n = n;
  g.k = k;
  g.c = c;
  return gemm_w4_checked(g, stream);
}

moe_status moe_silu_mul_quant(const uint16_t* gate_up, int32_t inter,
                              const int32_t* expert_counts, const int32_t* expert_offsets,
                              int32_t num_experts, int32_t row_cap, moe_act act,
                              float clamp_limit, moe_scale_fmt fmt, moe_rounding rounding,
                              uint8_t* hq, void* hs, void* stream) {
  if (!dim128(inter) || num_experts < 1 || row_cap < 0 || !fmt_ok(fmt) || !act_ok(act) ||
      !rounding_ok(rounding))
    return MOE_ERR_INVALID_ARG;
  if (act != MOE_ACT_SWIGLU && !(clamp_limit > 0.0f)) return MOE_ERR_INVALID_ARG;
  if (num_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;  // the kernel's LDS endpoint table
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (row_cap > 0 && (!gate_up || !hq || !hs)) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(row_cap) * (inter / 128) > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (row_cap == 0) return MOE_OK;
  return from_hip(moe::launch_silu_mul_quant(gate_up, inter, expert_counts, expert_offsets,
                                             num_experts, row_cap, act, clamp_limit, fmt,
                                             rounding, hq, hs, 0, as_stream(stream)));
}

moe_status moe_silu_mul_quant_masked(const uint16_t* gate_up, int32_t inter,
                                     const int32_t* masked_m, int32_t num_experts,
                                     int32_t expert_cap, moe_act act, float clamp_limit,
                                     moe_scale_fmt fmt, moe_rounding rounding, uint8_t* hq,
                                     void* hs, void* stream) {
  if (!dim128(inter) || num_experts < 1 || expert_cap < 1 || !fmt_ok(fmt) || !act_ok(act) ||
      !rounding_ok(rounding))
    return MOE_ERR_INVALID_ARG;
  if (num_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_ACT_SWIGLU && !(clamp_limit > 0.0f)) return MOE_ERR_INVALID_ARG;
  const int64_t rows = static_cast<int64_t>(num_experts) * expert_cap;
  if (rows > INT32_MAX / 2 || rows * (inter / 128) > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!masked_m || !gate_up || !hq || !hs) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_silu_mul_quant(gate_up, inter, masked_m, nullptr, num_experts,
                                             static_cast<int>(rows), act, clamp_limit, fmt,
                                             rounding, hq, hs, expert_cap, as_stream(stream)));
}

moe_status moe_topk_combine(const uint16_t* y, int32_t row_cap, const int32_t* pair_to_row,
                            const float* topk_w, int32_t t_cap, const int32_t* t_live_dev,
                            int32_t topk, int32_t hidden, uint16_t* out, void* stream) {
  if (row_cap < 0 || t_cap < 0 || topk < 1 || topk > kMaxTopk || !dim128(hidden))
    return MOE_ERR_INVALID_ARG;
  if (t_cap > 0 && (!pair_to_row || !topk_w || !out || (row_cap > 0 && !y)))
    return MOE_ERR_INVALID_ARG;
  if (t_cap == 0) return MOE_OK;
  return from_hip(moe::launch_topk_combine(y, row_cap, pair_to_row, topk_w, t_cap, t_live_dev,
                                           topk, hidden, out, as_stream(stream)));
}

moe_status moe_workspace_plan(const moe_problem* p, moe_workspace_layout* L) {
  if (!p || !L) return MOE_ERR_INVALID_ARG;
  if (p->num_experts < 1 || !dim128(p->hidden) || !dim128(p->inter) || p->topk < 1 ||
      p->topk > kMaxTopk || p->t_cap < 0 || p->align_rows < 1 || p->row_cap < 0 ||
      !fmt_ok(p->scale_fmt) || !act_ok(p->act) || !rounding_ok(p->rounding) ||
      (p->weight_fmt != MOE_WEIGHT_E4M3 && p->weight_fmt != MOE_WEIGHT_MXFP4))
    return MOE_ERR_INVALID_ARG;
  if (p->act != MOE_ACT_SWIGLU && !(p->clamp_limit > 0.0f)) return MOE_ERR_INVALID_ARG;
  if (p->num_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (p->expert_cap < 0) return MOE_ERR_INVALID_ARG;
  const bool batched = p->expert_cap > 0;
  // Rows: any aligned routing's need, or the batched layout's E * cap.
  const int64_t need = batched ? static_cast<int64_t>(p->num_experts) * p->expert_cap
                               : min_row_cap64(p->t_cap, p->topk, p->num_experts, p->align_rows);
  if (need > INT32_MAX / 2) return MOE_ERR_INVALID_ARG;
  const int64_t rc = p->row_cap == 0 ? need : p->row_cap;
  if (batched && rc != need) return MOE_ERR_INVALID_ARG;  // the batched layout fixes its rows
  if (rc < need) return MOE_ERR_CAPACITY;
  if (rc * (p->inter / 128) > INT32_MAX) return MOE_ERR_INVALID_ARG;  // as moe_silu_mul_quant
  if (!gemm_shape_ok(p->t_cap, 2 * static_cast<int64_t>(p->inter), p->hidden) ||
      !gemm_shape_ok(rc, p->hidden, p->inter))
    return MOE_ERR_UNSUPPORTED;
  const size_t E = p->num_experts, H = p->hidden, I = p->inter, T = p->t_cap;
  const size_t R = static_cast<size_t>(rc), P = T * p->topk, sb = scale_bytes(p->scale_fmt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->expert_counts = take(E * 4);
  L->expert_offsets = take((E + 1) * 4);
  L->row_to_pair = take(R * 4);
  L->pair_to_row = take(P * 4);
  L->xq = take(T * H);
  L->xs = take((H / 128) * T * sb);
  L->c1 = take(R * 2 * I * 2);
  L->hq = take(R * I);
  L->hs = take((I / 128) * R * sb);
  L->y = take(R * H * 2);
  // The decode path serves the aligned layout; MXFP4 weights take only its
  // one-launch layer, whose stages need H and I multiples of 256.
  const bool decode = !batched && moe::down_combine_fits(p->t_cap, p->topk, p->inter) &&
                      (p->weight_fmt == MOE_WEIGHT_E4M3 ||
                       moe::decode_layer_fits_fmt(p->t_cap, p->topk, p->hidden, p->inter, p->weight_fmt));
  L->act = decode ? take(R * I * 4) : 0;
  L->status = take(static_cast<size_t>(moe::kDlMaxGrid) * 4);
  L->overflow = take(4);
  L->total = off;
  if (!decode) L->act = L->status;
  L->row_cap = static_cast<int32_t>(rc);
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_problem* p) {
  moe_workspace_layout L;
  return moe_workspace_plan(p, &L) == MOE_OK ? L.total : 0;
}

namespace {

// FC2 and the top-k combine of the decode path, reading the workspace.
moe::DownCombineArgs down_combine_args(const moe_problem* p, const moe_tensors* t,
                                      const moe_workspace_layout& L, char* ws) {
  moe::DownCombineArgs d;
  d.act = reinterpret_cast<const float*>(ws + L.act);
  d.fmt = p->scale_fmt;
  d.w = t->w2;
  d.w_scales = t->w2_scales;
  d.counts = reinterpret_cast<const int32_t*>(ws + L.expert_counts);
  d.offsets = reinterpret_cast<const int32_t*>(ws + L.expert_offsets);
  d.row_to_pair = reinterpret_cast<const int32_t*>(ws + L.row_to_pair);
  d.pair_to_row = reinterpret_cast<const int32_t*>(ws + L.pair_to_row);
  d.topk_w = t->topk_w;
  d.t_live_dev = t->t_live_dev;
  d.num_experts = p->num_experts;
  d.row_cap = L.row_cap;
  d.t_cap = p->t_cap;
  d.topk = p->topk;
  d.hidden = p->hidden;
  d.inter = p->inter;
  d.hq = reinterpret_cast<uint8_t*>(ws + L.hq);
  d.hs = ws + L.hs;
  d.y = reinterpret_cast<uint16_t*>(ws + L.y);
  d.out = t->out;
  d.rounding = p->rounding;
  return d;
}

// Routing, activation quantization and FC1 of the decode path, writing the workspace.
moe::DecodeFc1Args fc1_decode_args(const moe_problem* p, const moe_tensors* t,
                                   const moe_workspace_layout& L, char* ws) {
  moe::DecodeFc1Args f;
  f.ids = t->topk_ids;
  f.t_live_dev = t->t_live_dev;
  f.t_cap = p->t_cap;
  f.topk = p->topk;
  f.num_experts = p->num_experts;
  f.align_rows = p->align_rows;
  f.row_cap = L.row_cap;
  f.expert_start = p->expert_start;
  f.x = t->x;
  f.hidden = p->hidden;
  f.inter = p->inter;
  f.fmt = p->scale_fmt;
  f.w = t->w1;
  f.w_scales = t->w1_scales;
  f.weight_fmt = p->weight_fmt;
  f.act = p->act;
  f.act_limit = p->clamp_limit;
  f.counts = reinterpret_cast<int32_t*>(ws + L.expert_counts);
  f.offsets = reinterpret_cast<int32_t*>(ws + L.expert_offsets);
  f.row_to_pair = reinterpret_cast<int32_t*>(ws + L.row_to_pair);
  f.pair_to_row = reinterpret_cast<int32_t*>(ws + L.pair_to_row);
  f.xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  f.xs = ws + L.xs;
  f.c1 = reinterpret_cast<uint16_t*>(ws + L.c1);
  f.act_out = reinterpret_cast<float*>(ws + L.act);
  f.rounding = p->rounding;
  return f;
}

}  // namespace

moe_status moe_fc1_decode(const moe_problem* p, const moe_tensors* t, void* workspace,
                          size_t workspace_bytes, void* stream) {
  moe_workspace_layout L;
  const moe_status st = moe_workspace_plan(p, &L);
  if (st != MOE_OK) return st;
  if (!(L.act < L.status) || p->weight_fmt != MOE_WEIGHT_E4M3 ||
      !moe::fc1_decode_fits(p->t_cap, p->topk, p->hidden, p->inter))
    return MOE_ERR_UNSUPPORTED;
  if (!t || !workspace) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return MOE_ERR_CAPACITY;
  if (!t->x || !t->topk_ids || !t->w1 || !t->w1_scales) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_fc1_decode(fc1_decode_args(p, t, L, static_cast<char*>(workspace)),
                                         as_stream(stream)));
}

moe_status moe_barrier_timeouts(uint32_t* count) {
  if (!count) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::decode_layer_timeouts(count));
}

int32_t moe_barrier_spin_limit(int32_t polls) {
  const int32_t old = moe::decode_layer_spin_limit();
  moe::set_decode_layer_spin_limit(polls);
  return old;
}

static moe_status forward_impl(const moe_problem* p, const moe_workspace_layout& L,
                               const moe_tensors* t, void* workspace, void* stream);

moe_status moe_forward(const moe_problem* p, const moe_tensors* t, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_workspace_layout L;
  const moe_status st = moe_workspace_plan(p, &L);
  if (st != MOE_OK) return st;
  if (!t || !workspace) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return MOE_ERR_CAPACITY;
  return forward_impl(p, L, t, workspace, stream);
}

moe_status moe_forward_noalloc(const moe_problem* p, const moe_tensors* t, void* stream) {
  moe_workspace_layout L;
  const moe_status st = moe_workspace_plan(p, &L);
  if (st != MOE_OK) return st;
  if (!t) return MOE_ERR_INVALID_ARG;
  if (L.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_CAPACITY;
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_HIP;
  return forward_impl(p, L, t, ws, stream);
}

static moe_status forward_impl(const moe_problem* p, const moe_workspace_layout& L,
                               const moe_tensors* t, void* workspace, void* stream) {
  if (!t || !workspace) return MOE_ERR_INVALID_ARG;
  if (p->t_cap > 0 && (!t->x || !t->topk_ids || !t->topk_w || !t->w1 || !t->w1_scales ||
                       !t->w2 || !t->w2_scales || !t->out))
    return MOE_ERR_INVALID_ARG;
  if (p->t_cap == 0) return MOE_OK;

  char* ws = static_cast<char*>(workspace);
  auto* counts = reinterpret_cast<int32_t*>(ws + L.expert_counts);
  auto* offsets = reinterpret_cast<int32_t*>(ws + L.expert_offsets);
  auto* r2p = reinterpret_cast<int32_t*>(ws + L.row_to_pair);
  auto* p2r = reinterpret_cast<int32_t*>(ws + L.pair_to_row);
  auto* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
  void* xs = ws + L.xs;
  auto* c1 = reinterpret_cast<uint16_t*>(ws + L.c1);
  auto* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
  void* hs = ws + L.hs;
  auto* y = reinterpret_cast<uint16_t*>(ws + L.y);
  const bool decode = L.act < L.status;  // fused decode path (the plan lays out act)
  auto* act = reinterpret_cast<float*>(ws + L.act);
  const hipStream_t s = as_stream(stream);
  const int R = L.row_cap;
  const int64_t pairs64 = static_cast<int64_t>(p->t_cap) * p->topk;
  const int pairs = static_cast<int>(pairs64);

  hipError_t e = hipSuccess;
  if (decode && moe::decode_layer_fits_fmt(p->t_cap, p->topk, p->hidden, p->inter, p->weight_fmt) &&
      moe::decode_layer_grid(moe::decode_layer_wide(p->t_cap, p->hidden)) > 0) {
    // The whole layer in one launch.
    moe::DecodeLayerArgs a;
    a.f1 = fc1_decode_args(p, t, L, ws);
    a.f2 = down_combine_args(p, t, L, ws);
    a.status = reinterpret_cast<int32_t*>(ws + L.status);
    a.spin_limit = moe::decode_layer_spin_limit();
    return from_hip(moe::launch_decode_layer(a, s));
  }
  if (decode && p->weight_fmt == MOE_WEIGHT_E4M3 && moe::fc1_decode_fits(p->t_cap, p->topk, p->hidden, p->inter)) {
    // Routing, activation quantization and FC1 with SiLU(gate) * up in one
    // launch, then FC2 with the combine.
    e = moe::launch_fc1_decode(fc1_decode_args(p, t, L, ws), s);
    if (e == hipSuccess) e = moe::launch_down_combine(down_combine_args(p, t, L, ws), s);
    return from_hip(e);
  }
  // Alignment and activation quantization share one launch (independent work).
  moe::AlignMode mode;
  mode.expert_start = p->expert_start;
  mode.batch_cap = p->expert_cap;
  mode.overflow = p->expert_cap > 0 ? reinterpret_cast<int32_t*>(ws + L.overflow) : nullptr;
  e = moe::launch_prep(t->topk_ids, p->t_cap, t->t_live_dev, p->topk, p->num_experts,
                       p->align_rows, counts, offsets, r2p, p2r, t->x, p->hidden, p->scale_fmt,
                       p->rounding, xq, xs, mode, s);

  if (p->weight_fmt == MOE_WEIGHT_MXFP4) {
    // FC1 and FC2 with MXFP4 weights; the rest as the general path.
    moe::W4Args w;
    w.fmt = p->scale_fmt;
    w.counts = counts;
    w.offsets = offsets;
    w.seg_cap = 0;  // the batched layout's offsets are e * cap, written by the alignment
    w.num_experts = p->num_experts;
    w.row_cap = R;
    w.max_rows_per_expert = pairs < R ? pairs : R;
    if (p->expert_cap > 0 && p->expert_cap < w.max_rows_per_expert) w.max_rows_per_expert = p->expert_cap;
    if (e == hipSuccess) {
      w.a = xq;
      w.a_scales = xs;
      w.a_rows = p->t_cap;
      w.a_row_map = r2p;
      w.a_row_div = p->topk;
      w.w = t->w1;
      w.w_scales = static_cast<const uint8_t*>(t->w1_scales);
      w.n = 2 * p->inter;
      w.k = p->hidden;
      w.c = c1;
      e = moe::launch_grouped_gemm_w4(w, s);
    }
    if (e == hipSuccess)
      e = moe::launch_silu_mul_quant(c1, p->inter, counts, offsets, p->num_experts, R, p->act,
                                     p->clamp_limit, p->scale_fmt, p->rounding, hq, hs, 0, s);
    if (e == hipSuccess) {
      w.a = hq;
      w.a_scales = hs;
      w.a_rows = R;
      w.a_row_map = nullptr;
      w.a_row_div = 1;
      w.w = t->w2;
      w.w_scales = static_cast<const uint8_t*>(t->w2_scales);
      w.n = p->hidden;
      w.k = p->inter;
      w.c = y;
      e = moe::launch_grouped_gemm_w4(w, s);
    }
    if (e == hipSuccess)
      e = moe::launch_topk_combine(y, R, p2r, t->topk_w, p->t_cap, t->t_live_dev, p->topk,
                                   p->hidden, t->out, s);
    return from_hip(e);
  }

  moe::GemmArgs g;
  g.fmt = p->scale_fmt;
  g.counts = counts;
  g.offsets = offsets;
  g.num_experts = p->num_experts;
  g.row_cap = R;
  g.max_rows_per_expert = pairs < R ? pairs : R;
  if (p->expert_cap > 0 && p->expert_cap < g.max_rows_per_expert) g.max_rows_per_expert = p->expert_cap;
  g.max_live_experts = pairs < p->num_experts ? pairs : p->num_experts;
  g.tiles_visited = nullptr;
  g.rounding = p->rounding;
  if (e == hipSuccess) {  // FC1: A rows gathered from the token-major quantized activations
    g.a = xq;
    g.a_scales = xs;
    g.a_rows = p->t_cap;
    g.a_row_map = r2p;
    g.a_row_div = p->topk;
    g.w = t->w1;
    g.w_scales = static_cast<const float*>(t->w1_scales);
    g.n = 2 * p->inter;
    g.k = p->hidden;
    g.c = c1;
    if (decode) {  // SiLU(gate) * up in FC1's epilogue
      g.act_out = act;
      g.act = p->act;
      g.act_limit = p->clamp_limit;
    }
    e = moe::launch_grouped_gemm(g, s);
    g.act_out = nullptr;
  }
  if (decode) {  // FC2 and the top-k combine in one launch
    if (e == hipSuccess) e = moe::launch_down_combine(down_combine_args(p, t, L, ws), s);
    return from_hip(e);
  }
  if (e == hipSuccess)
    e = moe::launch_silu_mul_quant(c1, p->inter, counts, offsets, p->num_experts, R, p->act,
                                   p->clamp_limit, p->scale_fmt, p->rounding, hq, hs, 0, s);
  if (e == hipSuccess) {  // FC2
    g.a = hq;
    g.a_scales = hs;
    g.a_rows = R;
    g.a_row_map = nullptr;
    g.a_row_div = 1;
    g.w = t->w2;
    g.w_scales = static_cast<const float*>(t->w2_scales);
    g.n = p->hidden;
    g.k = p->inter;
    g.c = y;
    e = moe::launch_grouped_gemm(g, s);
  }
  if (e == hipSuccess)
    e = moe::launch_topk_combine(y, R, p2r, t->topk_w, p->t_cap, t->t_live_dev, p->topk,
                                 p->hidden, t->out, s);
  return from_hip(e);
}

}  // extern "C"
