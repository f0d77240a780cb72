// Host runtime and C ABI of the weight-informed activation-sparse linear
// layer: argument validation, handle-owned device buffers, the host-side
// Phi^-1 for the statistical gate, launch planning and error mapping.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

#pragma clang fp contract(off)

namespace {

thread_local std::string g_last_error;

sl_status fail(sl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sl_status hip_fail(hipError_t e, const char* what) {
  const sl_status st = (e == hipErrorOutOfMemory) ? SL_ERR_OOM : SL_ERR_HIP;
  return fail(st, "%s: %s", what, hipGetErrorString(e));
}

#define SL_HIP(expr)                                \
  do {                                              \
    hipError_t e_ = (expr);                         \
    if (e_ != hipSuccess) return hip_fail(e_, #expr); \
  } while (0)

// Phi^-1(p), Wichura's AS241 (PPND16), Applied Statistics 37 (1988) 477-484:
// a rational approximation in r = 0.180625 - q^2 for |p - 1/2| <= 0.425, and in
// r = sqrt(-log(min(p, 1-p))) (shifted by 1.6 or 5) in the tails, evaluated
// in nested (Horner) form as published, in fp64, without fused multiply-add.
double as241(double p) {
  const double q = p - 0.5;
  if (fabs(q) <= 0.425) {
    const double r = 0.180625 - q * q;
    const double num =
        (((((((2.5090809287301226727e+3 * r + 3.3430575583588128105e+4) * r + 6.7265770927008700853e+4) * r +
             4.5921953931549871457e+4) * r + 1.3731693765509461125e+4) * r + 1.9715909503065514427e+3) * r +
          1.3314166789178437745e+2) * r + 3.3871328727963666080e+0) * q;
    const double den =
        ((((((5.2264952788528545610e+3 * r + 2.8729085735721942674e+4) * r + 3.9307895800092710610e+4) * r +
             2.1213794301586595867e+4) * r + 5.3941960214247511077e+3) * r + 6.8718700749205790830e+2) * r +
          4.2313330701600911252e+1) * r + 1.0;
    return num / den;
  }
  double r = (q <= 0.0) ? p : 1.0 - p;
  r = sqrt(-log(r));
  double num, den;
  if (r <= 5.0) {
    r = r - 1.6;
    num = (((((((7.74545014278341407640e-4 * r + 2.27238449892691845833e-2) * r + 2.41780725177450611770e-1) * r +
               1.27045825245236838258e+0) * r + 3.64784832476320460504e+0) * r + 5.76949722146069140550e+0) * r +
            4.63033784615654529590e+0) * r + 1.42343711074968357734e+0);
    den = (((((((1.05075007164441684324e-9 * r + 5.47593808499534494600e-4) * r + 1.51986665636164571966e-2) * r +
               1.48103976427480074590e-1) * r + 6.89767334985100004550e-1) * r + 1.67638483018380384940e+0) * r +
            2.05319162663775882187e+0) * r + 1.0);
  } else {
    r = r - 5.0;
    num = (((((((2.01033439929228813265e-7 * r + 2.71155556874348757815e-5) * r + 1.24266094738807843860e-3) * r +
               2.65321895265761230930e-2) * r + 2.96560571828504891230e-1) * r + 1.78482653991729133580e+0) * r +
            5.46378491116411436990e+0) * r + 6.65790464350110377720e+0);
    den = (((((((2.04426310338993978564e-15 * r + 1.42151175831644588870e-7) * r + 1.84631831751005468180e-5) * r +
               7.86869131145613259100e-4) * r + 1.48753612908506148525e-2) * r + 1.36929880922735805310e-1) * r +
            5.99832206555887937690e-1) * r + 1.0);
  }
  double x = num / den;
  if (q < 0.0) x = -x;
  return x;
}

size_t dtype_size(sl_dtype d) { return d == SL_BF16 ? 2 : 4; }

int vec_elems(sl_dtype d) { return d == SL_BF16 ? 8 : 4; }

// Upper bound on the splits any plan may use (chunks of >= 32 inputs).
int max_splits(int64_t n) { return (int)std::min<int64_t>(sl::kMaxSplits, (n + 31) / 32); }

// Expected number of kept inputs, used to size the split count.
int64_t expected_kept(const sl_linear* h, bool dense) {
  if (dense) return h->n;
  switch (h->gate) {
    case SL_GATE_TOPK: return h->K;
    case SL_GATE_STAT: return (int64_t)ceil(h->s_keep * (double)h->n);
    default: return h->n / 2;
  }
}

sl::Plan make_plan(const sl_linear* h, bool dense, sl_dtype ydt) {
  sl::Plan p;
  p.atomic = (ydt == SL_F32) && !h->deterministic;
  const int vec = vec_elems(h->wdt);
  int lpc;
  if (h->plan_rows > 0) {
    lpc = h->plan_rows / vec;
  } else if (h->m >= 8192) {
    lpc = 64;
  } else if (h->m >= 2048) {
    lpc = 32;
  } else {
    lpc = 16;
  }
  lpc = std::max(16, std::min(64, lpc));
  p.lpc = lpc;
  p.rows = lpc * vec;
  p.tiles = (int)((h->m + p.rows - 1) / p.rows);
  p.unroll = 4;
  const int64_t n = h->n;
  int splits;
  if (h->plan_splits > 0) {
    splits = h->plan_splits;
  } else {
    const int64_t kept = std::max<int64_t>(1, expected_kept(h, dense));
    splits = (int)std::max<int64_t>(1, 2048 / p.tiles);
    splits = (int)std::min<int64_t>(splits, std::max<int64_t>(1, kept / 24));
  }
  splits = std::min(splits, max_splits(n));
  splits = std::max<int>(splits, (int)((n + sl::kMaxChunk - 1) / sl::kMaxChunk));
  p.chunk = (int)((n + splits - 1) / splits);
  p.splits = (int)((n + p.chunk - 1) / p.chunk);
  return p;
}

// Union (B > 1) product: 256-row tiles; input chunks of 256..512 sized so that
// the workgroups fill the device's slots once (a second, partial wave of
// workgroups cost ~20 % on the Qwen-shaped layers).
int max_union_splits(int64_t n) { return (int)std::max<int64_t>(1, (n + sl::kUnionMinChunk - 1) / sl::kUnionMinChunk); }

sl::UnionPlan make_union_plan(const sl_linear* h, sl_dtype ydt) {
  sl::UnionPlan p;
  p.atomic = (ydt == SL_F32) && !h->deterministic;
  p.rows = (h->uplan_rows == 128 || h->uplan_rows == 256) ? h->uplan_rows : 256;
  p.tiles = (int)((h->m + p.rows - 1) / p.rows);
  const int64_t n = h->n;
  const int slots = std::max(1, h->cus) * sl::union_workgroups_per_cu(p.rows, ydt, p.atomic);
  int splits = (int)std::max<int64_t>(1, (h->uplan_wgs > 0 ? h->uplan_wgs : slots) / p.tiles);
  splits = std::min(splits, max_union_splits(n));
  splits = std::max<int>(splits, (int)((n + sl::kUnionMaxChunk - 1) / sl::kUnionMaxChunk));
  p.chunk = (int)((n + splits - 1) / splits);
  p.splits = (int)((n + p.chunk - 1) / p.chunk);
  p.spec = false;  // set per forward from the batch size (expected union density)
  return p;
}

// Expected union density 1 - (1 - f)^B of B independent tokens keeping a
// fraction f each; only steers the union product's speculative first loads.
bool union_spec(const sl_linear* h, int B, bool dense) {
  if (dense) return true;
  double f = 0.0;
  if (h->gate == SL_GATE_TOPK) f = h->n > 0 ? (double)h->K / (double)h->n : 0.0;
  else if (h->gate == SL_GATE_STAT) f = h->s_keep;
  else return false;  // fixed threshold: no prior on the kept fraction
  return 1.0 - std::pow(1.0 - f, (double)B) >= 0.98;
}

// Reports (and clears) a timed-out hand-off that an earlier fused forward of
// this handle recorded in its host-visible error word. Needs no
// synchronization: the kernel stores the word with system scope, so a
// forward that has completed is seen by the next call at the latest.
sl_status take_async_error(const sl_linear* h) {
  if (h->herr == nullptr) return SL_OK;
  const uint32_t e = __atomic_exchange_n(h->herr, 0u, __ATOMIC_ACQ_REL);
  if (e == 0) return SL_OK;
  return fail(SL_ERR_HIP,
              "fused forward: a %s wait timed out in an earlier call on this handle (that call's y is incomplete)",
              e == 1 ? "product workgroup's gate" : "gate workgroup's acknowledgement");
}

sl_status check_device(const sl_linear* h) {
  int dev = -1;
  SL_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(SL_ERR_ARG, "handle belongs to device %d, current device is %d", h->device, dev);
  return SL_OK;
}

void free_handle(sl_linear* h) {
  if (!h) return;
  (void)hipFree(h->Wt);
  (void)hipFree(h->c);
  (void)hipFree(h->gout);
  (void)hipFree(h->partials);
  (void)hipFree(h->ctr);
  (void)hipFree(h->upartials);
  (void)hipFree(h->uctr);
  (void)hipFree(h->fsync);
  if (h->herr) (void)hipHostFree(h->herr);
  delete h;
}

}  // namespace

extern "C" {

const char* sparse_linear_strerror(sl_status s) {
  switch (s) {
    case SL_OK: return "success";
    case SL_ERR_ARG: return "invalid argument";
    case SL_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case SL_ERR_OOM: return "device allocation failed";
    case SL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sparse_linear_last_error(void) { return g_last_error.c_str(); }

double sparse_linear_normal_quantile(double p) {
  if (!(p > 0.0 && p < 1.0)) return NAN;
  return as241(p);
}

sl_status sparse_linear_init(sl_handle* out, const void* W, sl_dtype w_dtype, sl_layout w_layout, int64_t m,
                             int64_t n, const float* c, sl_gate gate, int64_t K, double s_keep,
                             int32_t max_batch, void* stream) {
  try {
    g_last_error.clear();
    if (out == nullptr) return fail(SL_ERR_ARG, "out is NULL");
    if (W == nullptr) return fail(SL_ERR_ARG, "W is NULL");
    if (w_dtype != SL_F32 && w_dtype != SL_BF16) return fail(SL_ERR_ARG, "bad w_dtype %d", (int)w_dtype);
    if (w_layout != SL_W_ROWMAJOR_OUT_IN && w_layout != SL_W_COLMAJOR)
      return fail(SL_ERR_ARG, "bad w_layout %d", (int)w_layout);
    if (m < 1 || n < 1) return fail(SL_ERR_ARG, "m and n must be >= 1 (m=%lld n=%lld)", (long long)m, (long long)n);
    if (n > SL_MAX_N) return fail(SL_ERR_UNSUPPORTED, "n=%lld exceeds %d", (long long)n, SL_MAX_N);
    if (m > (1 << 21)) return fail(SL_ERR_UNSUPPORTED, "m=%lld exceeds 2^21", (long long)m);
    if (m % vec_elems(w_dtype) != 0)
      return fail(SL_ERR_UNSUPPORTED, "m=%lld must be a multiple of %d for this dtype", (long long)m,
                  vec_elems(w_dtype));
    if (max_batch < 1 || max_batch > SL_MAX_BATCH)
      return fail(SL_ERR_ARG, "max_batch=%d outside [1, %d]", (int)max_batch, SL_MAX_BATCH);
    switch (gate) {
      case SL_GATE_TOPK:
        if (K < 0 || K > n) return fail(SL_ERR_ARG, "K=%lld outside [0, n=%lld]", (long long)K, (long long)n);
        break;
      case SL_GATE_STAT:
        if (!(s_keep > 0.0 && s_keep < 1.0)) return fail(SL_ERR_ARG, "s_keep=%g outside (0, 1)", s_keep);
        break;
      case SL_GATE_FIXED:
        if (!(s_keep >= 0.0) || !isfinite(s_keep) || s_keep > 3.0e38)
          return fail(SL_ERR_ARG, "tau=%g must be finite and >= 0", s_keep);
        break;
      default:
        return fail(SL_ERR_ARG, "bad gate %d", (int)gate);
    }
    int dev = -1;
    SL_HIP(hipGetDevice(&dev));
    hipStream_t s = (hipStream_t)stream;
    {
      // set-up of the allocation-free FFN entry point: the static workspace's
      // address on this device (cached; a failure here is reported by that
      // entry point, which looks it up again)
      void* ws = nullptr;
      (void)sl::ffn_scratch(dev, &ws);
    }

    sl_linear* h = new (std::nothrow) sl_linear();
    if (!h) return fail(SL_ERR_OOM, "host allocation failed");
    h->device = dev;
    h->m = m;
    h->n = n;
    h->wdt = w_dtype;
    h->gate = gate;
    h->K = (gate == SL_GATE_TOPK) ? K : 0;
    h->s_keep = s_keep;
    h->max_batch = max_batch;
    if (gate == SL_GATE_STAT) h->z = as241(1.0 - s_keep);
    if (gate == SL_GATE_FIXED) h->tau = (float)s_keep;

    auto cleanup_fail = [&](hipError_t e, const char* what) {
      free_handle(h);
      return hip_fail(e, what);
    };
    hipError_t e;
    const size_t wbytes = (size_t)m * (size_t)n * dtype_size(w_dtype);
    if ((e = hipMalloc(&h->Wt, wbytes)) != hipSuccess) return cleanup_fail(e, "hipMalloc(W)");
    if ((e = hipMalloc(&h->c, (size_t)n * sizeof(float))) != hipSuccess) return cleanup_fail(e, "hipMalloc(c)");
    if ((e = hipMalloc(&h->gout, (size_t)max_batch * sizeof(sl::GateOut))) != hipSuccess)
      return cleanup_fail(e, "hipMalloc(gate)");
    const size_t part = (size_t)max_splits(n) * (size_t)m * sizeof(float);
    if ((e = hipMalloc(&h->partials, part)) != hipSuccess) return cleanup_fail(e, "hipMalloc(partials)");
    h->ctr_len = (m + 63) / 64 + 1;
    if ((e = hipMalloc(&h->ctr, (size_t)h->ctr_len * sizeof(uint32_t))) != hipSuccess)
      return cleanup_fail(e, "hipMalloc(counters)");
    if ((e = hipMemsetAsync(h->ctr, 0, (size_t)h->ctr_len * sizeof(uint32_t), s)) != hipSuccess)
      return cleanup_fail(e, "hipMemsetAsync(counters)");
    if ((e = hipMalloc(&h->fsync, sizeof(sl::FusedSync))) != hipSuccess) return cleanup_fail(e, "hipMalloc(sync)");
    if ((e = hipMemsetAsync(h->fsync, 0, sizeof(sl::FusedSync), s)) != hipSuccess)
      return cleanup_fail(e, "hipMemsetAsync(sync)");
    if ((e = hipHostMalloc((void**)&h->herr, 64, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess)
      return cleanup_fail(e, "hipHostMalloc(error word)");
    *h->herr = 0u;
    if ((e = hipHostGetDevicePointer((void**)&h->herr_dev, h->herr, 0)) != hipSuccess)
      return cleanup_fail(e, "hipHostGetDevicePointer(error word)");
    if ((e = hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return cleanup_fail(e, "hipDeviceGetAttribute(compute units)");

    if (max_batch > 1 && w_dtype == SL_BF16) {
      h->upart_len = (int64_t)max_union_splits(n) * max_batch * m;
      if ((e = hipMalloc(&h->upartials, (size_t)h->upart_len * sizeof(float))) != hipSuccess)
        return cleanup_fail(e, "hipMalloc(union partials)");
      const size_t uc = (size_t)((m + 127) / 128);  // tiles of >= 128 rows
      if ((e = hipMalloc(&h->uctr, uc * sizeof(uint32_t))) != hipSuccess)
        return cleanup_fail(e, "hipMalloc(union counters)");
      if ((e = hipMemsetAsync(h->uctr, 0, uc * sizeof(uint32_t), s)) != hipSuccess)
        return cleanup_fail(e, "hipMemsetAsync(union counters)");
    }
    if (w_layout == SL_W_ROWMAJOR_OUT_IN) {
      if ((e = sl::launch_repack(W, w_dtype, m, n, h->Wt, s)) != hipSuccess) return cleanup_fail(e, "repack");
    } else {
      if ((e = hipMemcpyAsync(h->Wt, W, wbytes, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "hipMemcpyAsync(W)");
    }
    if (c != nullptr) {
      if ((e = hipMemcpyAsync(h->c, c, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "hipMemcpyAsync(c)");
    } else {
      if ((e = sl::launch_norms(h->Wt, w_dtype, m, n, h->c, s)) != hipSuccess) return cleanup_fail(e, "norms");
    }
    {
      // Every slot starts as "keep nothing"; a fixed threshold is known now, so the
      // product kernel can run without a gate launch.
      std::vector<sl::GateOut> g0(max_batch);
      for (auto& g : g0) {
        g.kthr = 0xffffffffu;
        g.jlast = -1;
        g.count = 0;
        g.pad = 0;
        g.thresh = 0.0;
        if (gate == SL_GATE_FIXED) {
          uint32_t bits;
          memcpy(&bits, &h->tau, sizeof(bits));
          g.kthr = bits & 0x7fffffffu;
          g.thresh = (double)h->tau;
        }
      }
      if ((e = hipMemcpyAsync(h->gout, g0.data(), g0.size() * sizeof(sl::GateOut), hipMemcpyHostToDevice, s)) !=
          hipSuccess)
        return cleanup_fail(e, "hipMemcpyAsync(gate)");
      if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup_fail(e, "hipStreamSynchronize");
    }
    *out = h;
    return SL_OK;
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in init");
  }
}

static sl_status forward_impl(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                              uint8_t* mask_out, int32_t* count_out, double* thresh_out, void* stream,
                              bool dense, int stages) {
  g_last_error.clear();
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  if (x == nullptr || y == nullptr) return fail(SL_ERR_ARG, "x and y must be non-NULL");
  if (B < 1 || B > h->max_batch) return fail(SL_ERR_ARG, "B=%d outside [1, max_batch=%d]", (int)B, h->max_batch);
  if (y_dtype != SL_F32 && y_dtype != SL_BF16) return fail(SL_ERR_ARG, "bad y_dtype %d", (int)y_dtype);
  if (stages < 1 || stages > 3) return fail(SL_ERR_ARG, "stages=%d outside 1..3", stages);
  sl_status st = check_device(h);
  if (st != SL_OK) return st;
  if ((st = take_async_error(h)) != SL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const bool full = (stages & SL_STAGE_GATE) && (stages & SL_STAGE_PRODUCT);
  const bool gate_wanted = !dense && (stages & SL_STAGE_GATE) &&
                           (h->gate != SL_GATE_FIXED || mask_out || count_out || thresh_out);
  const size_t ysz = (y_dtype == SL_BF16) ? 2 : 4;

  if (B > 1 && h->wdt == SL_BF16) {
    // one matrix-core pass over the union of the B kept sets
    const sl::UnionPlan up = make_union_plan(h, y_dtype);
    const bool zero = up.atomic && up.splits > 1;
    if (gate_wanted)
      SL_HIP(sl::launch_gate(h, x, B, mask_out, count_out, thresh_out, (zero && full) ? (float*)y : nullptr, s));
    else if (zero && full)
      SL_HIP(sl::launch_zero((float*)y, (int64_t)B * h->m, s));
    if (stages & SL_STAGE_PRODUCT) {
      sl::UnionPlan ups = up;
      ups.spec = union_spec(h, B, dense);
      SL_HIP(sl::launch_union_product(h, ups, x, B, dense, y, y_dtype, s));
    }
    return SL_OK;
  }

  // one token at a time through the single-token product kernel (B == 1, or
  // fp32 weights, which the matrix-core path does not take)
  const sl::Plan plan = make_plan(h, dense, y_dtype);
  // With the atomic split reduction y must start at zero: the gate kernel
  // clears it, or a fill kernel does when no gate kernel runs. A product stage
  // run on its own adds onto y as it stands.
  const bool zero = plan.atomic && plan.splits > 1;
  const size_t xsz = (h->wdt == SL_BF16) ? 2 : 4;
  if (full && !dense && (gate_wanted || h->gate == SL_GATE_FIXED) && h->fused && sl::fused_supported(h, x)) {
    // gate and product of each token in one launch (with a fixed threshold
    // also when no gate output is wanted: one launch instead of fill + product)
    for (int b = 0; b < B; ++b)
      SL_HIP(sl::launch_fused(h, (const char*)x + (size_t)b * h->n * xsz, h->gout + b,
                              mask_out ? mask_out + (size_t)b * h->n : nullptr, count_out ? count_out + b : nullptr,
                              thresh_out ? thresh_out + b : nullptr, (char*)y + (size_t)b * h->m * ysz, y_dtype,
                              plan.atomic, s));
    return SL_OK;
  }
  if (gate_wanted)
    SL_HIP(sl::launch_gate(h, x, B, mask_out, count_out, thresh_out, (zero && full) ? (float*)y : nullptr, s));
  else if (zero && full)
    SL_HIP(sl::launch_zero((float*)y, (int64_t)B * h->m, s));
  if (stages & SL_STAGE_PRODUCT) {
    for (int b = 0; b < B; ++b)
      SL_HIP(sl::launch_product(h, plan, (const char*)x + (size_t)b * h->n * xsz, h->gout + b, dense,
                                (char*)y + (size_t)b * h->m * ysz, y_dtype, s));
  }
  return SL_OK;
}

sl_status sparse_linear_forward(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                                uint8_t* mask_out, int32_t* count_out, double* thresh_out, void* stream) {
  try {
    return forward_impl(h, x, B, y, y_dtype, mask_out, count_out, thresh_out, stream, false, 3);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward");
  }
}

static sl_status group_impl(const sl_handle* handles, int32_t count, const void* x, int32_t B, void* const* ys,
                            sl_dtype y_dtype, void* stream) {
  g_last_error.clear();
  if (handles == nullptr || ys == nullptr || x == nullptr) return fail(SL_ERR_ARG, "NULL argument");
  if (count < 1 || count > sl::kMaxGroupLinears)
    return fail(SL_ERR_ARG, "count=%d outside [1, %d]", (int)count, sl::kMaxGroupLinears);
  if (y_dtype != SL_F32 && y_dtype != SL_BF16) return fail(SL_ERR_ARG, "bad y_dtype %d", (int)y_dtype);
  if (B < 1) return fail(SL_ERR_ARG, "B=%d must be >= 1", (int)B);
  for (int l = 0; l < count; ++l) {
    const sl_linear* h = handles[l];
    if (h == nullptr || ys[l] == nullptr) return fail(SL_ERR_ARG, "handle or y %d is NULL", l);
    if (h->n != handles[0]->n || h->wdt != handles[0]->wdt)
      return fail(SL_ERR_ARG, "linear %d: n or weight dtype differs from linear 0", l);
    if (B > h->max_batch) return fail(SL_ERR_ARG, "linear %d: B=%d above its max_batch=%d", l, (int)B, h->max_batch);
    sl_status st = check_device(h);
    if (st != SL_OK) return st;
  }
  // one handle twice would make two linears of the launch share its
  // hand-off state and scratch
  for (int a = 0; a < count; ++a)
    for (int b = a + 1; b < count; ++b)
      if (handles[a] == handles[b]) return fail(SL_ERR_ARG, "linears %d and %d are the same handle", a, b);
  for (int l = 0; l < count; ++l) {
    sl_status st = take_async_error(handles[l]);
    if (st != SL_OK) return st;
  }
  const sl_linear* hs[sl::kMaxGroupLinears];
  for (int l = 0; l < count; ++l) hs[l] = handles[l];
  hipStream_t s = (hipStream_t)stream;
  if (B > 1) {
    // the linears' gates for the B tokens in one launch, then each linear's
    // matrix-core pass over the union of its B kept sets
    bool grouped = count > 1;
    for (int l = 0; l < count && grouped; ++l)
      grouped = hs[l]->wdt == SL_BF16 && hs[l]->gate == hs[0]->gate && hs[l]->gate != SL_GATE_FIXED;
    if (!grouped) {
      for (int l = 0; l < count; ++l) {
        sl_status st = forward_impl(handles[l], x, B, ys[l], y_dtype, nullptr, nullptr, nullptr, stream, false, 3);
        if (st != SL_OK) return st;
      }
      return SL_OK;
    }
    float* zy[sl::kMaxGroupLinears];
    for (int l = 0; l < count; ++l) {
      const sl::UnionPlan up = make_union_plan(hs[l], y_dtype);
      zy[l] = (up.atomic && up.splits > 1) ? (float*)ys[l] : nullptr;
    }
    SL_HIP(sl::launch_gate_group(hs, count, x, B, zy, s));
    for (int l = 0; l < count; ++l) {
      sl::UnionPlan up = make_union_plan(hs[l], y_dtype);
      up.spec = union_spec(hs[l], B, false);
      SL_HIP(sl::launch_union_product(hs[l], up, x, B, false, ys[l], y_dtype, s));
    }
    return SL_OK;
  }
  bool grouped = count > 1 && y_dtype == SL_F32;
  for (int l = 0; l < count && grouped; ++l) {
    const sl_linear* h = handles[l];
    grouped = h->fused && !h->deterministic && h->gate == handles[0]->gate && sl::fused_supported(h, x);
  }
  if (!grouped) {
    for (int l = 0; l < count; ++l) {
      sl_status st = forward_impl(handles[l], x, 1, ys[l], y_dtype, nullptr, nullptr, nullptr, stream, false, 3);
      if (st != SL_OK) return st;
    }
    return SL_OK;
  }
  float* yf[sl::kMaxGroupLinears];
  for (int l = 0; l < count; ++l) yf[l] = (float*)ys[l];
  SL_HIP(sl::launch_fused_group(hs, count, x, yf, s));
  return SL_OK;
}

sl_status sparse_linear_forward_group(const sl_handle* handles, int32_t count, const void* x, void* const* ys,
                                      sl_dtype y_dtype, void* stream) {
  try {
    return group_impl(handles, count, x, 1, ys, y_dtype, stream);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_group");
  }
}

sl_status sparse_linear_forward_group_batch(const sl_handle* handles, int32_t count, const void* x, int32_t B,
                                            void* const* ys, sl_dtype y_dtype, void* stream) {
  try {
    return group_impl(handles, count, x, B, ys, y_dtype, stream);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_group_batch");
  }
}

// FFN workspace: g and u (fp32 [m]) and h (bf16 [m]), each 256-byte aligned.
static int64_t ffn_piece(int64_t bytes) { return (bytes + 255) / 256 * 256; }
static int64_t ffn_bytes(int64_t m) { return 2 * ffn_piece(4 * m) + ffn_piece(2 * m); }

int64_t sparse_linear_ffn_workspace_bytes(sl_handle up) {
  if (up == nullptr) return 0;
  return ffn_bytes(up->m);
}

sl_status sparse_linear_forward_ffn(sl_handle gate, sl_handle up, sl_handle down, const void* x, void* y,
                                    sl_dtype y_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (gate == nullptr || up == nullptr || down == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
    if (gate == up || gate == down || up == down)
      return fail(SL_ERR_ARG, "gate, up and down must be three different handles");
    if (x == nullptr || y == nullptr || workspace == nullptr) return fail(SL_ERR_ARG, "NULL pointer");
    if (gate->m != up->m || gate->n != up->n || down->n != up->m)
      return fail(SL_ERR_ARG, "shapes: gate %lldx%lld, up %lldx%lld, down %lldx%lld do not chain", (long long)gate->m,
                  (long long)gate->n, (long long)up->m, (long long)up->n, (long long)down->m, (long long)down->n);
    if (gate->wdt != SL_BF16 || up->wdt != SL_BF16 || down->wdt != SL_BF16)
      return fail(SL_ERR_UNSUPPORTED, "the FFN chain takes bf16 weights");
    if (((uintptr_t)workspace % 256) != 0) return fail(SL_ERR_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < ffn_bytes(up->m))
      return fail(SL_ERR_ARG, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                  (long long)ffn_bytes(up->m));
    char* ws = (char*)workspace;
    float* g = (float*)ws;
    float* u = (float*)(ws + ffn_piece(4 * up->m));
    uint16_t* hb = (uint16_t*)(ws + 2 * ffn_piece(4 * up->m));
    const sl_handle gu[2] = {gate, up};
    void* const ys[2] = {g, u};
    sl_status st = sparse_linear_forward_group(gu, 2, x, ys, SL_F32, stream);
    if (st != SL_OK) return st;
    SL_HIP(sl::launch_silu_mul(g, u, hb, up->m, (hipStream_t)stream));
    return forward_impl(down, hb, 1, y, y_dtype, nullptr, nullptr, nullptr, stream, false, 3);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_ffn");
  }
}

sl_status sparse_linear_forward_ffn_noalloc(sl_handle gate, sl_handle up, sl_handle down, const void* x, void* y,
                                            sl_dtype y_dtype, void* stream) {
  try {
    g_last_error.clear();
    if (gate == nullptr || up == nullptr || down == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
    if (up->m > sl::kFfnScratchMaxM)
      return fail(SL_ERR_UNSUPPORTED, "intermediate width m=%lld exceeds the static workspace's %lld",
                  (long long)up->m, (long long)sl::kFfnScratchMaxM);
    sl_status st = check_device(up);
    if (st != SL_OK) return st;
    void* ws = nullptr;
    SL_HIP(sl::ffn_scratch(up->device, &ws));
    return sparse_linear_forward_ffn(gate, up, down, x, y, y_dtype, ws, (int64_t)sl::kFfnScratchBytes, stream);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_ffn_noalloc");
  }
}

sl_status sparse_linear_forward_dense(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                                      void* stream) {
  try {
    return forward_impl(h, x, B, y, y_dtype, nullptr, nullptr, nullptr, stream, true, 3);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_dense");
  }
}

sl_status sparse_linear_get_norms(sl_handle h, float* c_out, void* stream) {
  if (h == nullptr || c_out == nullptr) return fail(SL_ERR_ARG, "NULL argument");
  sl_status st = check_device(h);
  if (st != SL_OK) return st;
  SL_HIP(hipMemcpyAsync(c_out, h->c, (size_t)h->n * sizeof(float), hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return SL_OK;
}

sl_status sparse_linear_destroy(sl_handle h) {
  free_handle(h);
  return SL_OK;
}

sl_status sparse_linear_forward_stages(sl_handle h, const void* x, int32_t B, void* y, sl_dtype y_dtype,
                                       uint8_t* mask_out, int32_t* count_out, double* thresh_out,
                                       int32_t stages, void* stream) {
  try {
    return forward_impl(h, x, B, y, y_dtype, mask_out, count_out, thresh_out, stream, false, stages);
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in forward_stages");
  }
}

sl_status sparse_linear_set_union_plan(sl_handle h, int32_t rows_per_tile, int32_t workgroups) {
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  if (rows_per_tile != 0 && rows_per_tile != 128 && rows_per_tile != 256)
    return fail(SL_ERR_ARG, "rows_per_tile=%d must be 0, 128 or 256", (int)rows_per_tile);
  if (workgroups < 0) return fail(SL_ERR_ARG, "workgroups=%d must be >= 0", (int)workgroups);
  h->uplan_rows = rows_per_tile;
  h->uplan_wgs = workgroups;
  return SL_OK;
}

sl_status sparse_linear_set_fused(sl_handle h, int32_t on) {
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  h->fused = (on != 0);
  return SL_OK;
}

sl_status sparse_linear_sync_status(sl_handle h, void* stream) {
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  sl_status st = check_device(h);
  if (st != SL_OK) return st;
  SL_HIP(hipStreamSynchronize((hipStream_t)stream));
  return take_async_error(h);
}


sl_status sparse_linear_gather_ceiling(sl_handle h, const int32_t* idx, int32_t count, float* sink, void* stream) {
  try {
    g_last_error.clear();
    if (h == nullptr || idx == nullptr || sink == nullptr) return fail(SL_ERR_ARG, "NULL argument");
    if (count < 0 || count > h->n) return fail(SL_ERR_ARG, "count=%d outside [0, n=%lld]", (int)count, (long long)h->n);
    sl_status st = check_device(h);
    if (st != SL_OK) return st;
    if (count == 0) return SL_OK;
    SL_HIP(sl::launch_gather_ceiling(h, idx, count, sink, (hipStream_t)stream));
    return SL_OK;
  } catch (...) {
    return fail(SL_ERR_OOM, "unexpected host exception in gather_ceiling");
  }
}

sl_status sparse_linear_set_timeline(void* buf) {
  g_last_error.clear();
  const hipError_t e = sl::timeline_set(buf);
  if (e == hipErrorNotSupported)
    return fail(SL_ERR_UNSUPPORTED, "this library was built without the fused forward's timestamps");
  SL_HIP(e);
  return SL_OK;
}

sl_status sparse_linear_set_deterministic(sl_handle h, int32_t on) {
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  h->deterministic = (on != 0);
  return SL_OK;
}

sl_status sparse_linear_set_plan(sl_handle h, int32_t rows_per_tile, int32_t splits) {
  if (h == nullptr) return fail(SL_ERR_ARG, "handle is NULL");
  const int vec = vec_elems(h->wdt);
  if (rows_per_tile != 0) {
    const int lpc = rows_per_tile / vec;
    if (rows_per_tile % vec != 0 || (lpc != 16 && lpc != 32 && lpc != 64))
      return fail(SL_ERR_ARG, "rows_per_tile=%d must be 16, 32 or 64 times %d", (int)rows_per_tile, vec);
  }
  if (splits < 0 || splits > max_splits(h->n)) return fail(SL_ERR_ARG, "splits=%d outside [0, %d]", (int)splits, max_splits(h->n));
  h->plan_rows = rows_per_tile;
  h->plan_splits = splits;
  return SL_OK;
}

}  // extern "C"

// ------------------------------------------------------------ Double Sparsity
namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

sl_status ds_check_shape(int32_t batch, int32_t heads, int32_t max_seq, int32_t head_dim, int32_t r) {
  if (batch < 1 || heads < 1) return fail(SL_ERR_ARG, "batch=%d and heads=%d must be >= 1", (int)batch, (int)heads);
  if ((int64_t)batch * heads > INT32_MAX) return fail(SL_ERR_ARG, "batch * heads exceeds 2^31 - 1");
  if (max_seq < 1 || max_seq > DS_MAX_SEQ)
    return fail(SL_ERR_ARG, "max_seq=%d outside [1, %d]", (int)max_seq, DS_MAX_SEQ);
  if (head_dim != 64 && head_dim != 128)
    return fail(SL_ERR_UNSUPPORTED, "head_dim=%d: 64 and 128 are supported", (int)head_dim);
  if (r != 8 && r != 16 && r != 32) return fail(SL_ERR_UNSUPPORTED, "r=%d: 8, 16 and 32 are supported", (int)r);
  return SL_OK;
}

sl_status ds_device() {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return SL_OK;
}

}  // namespace

extern "C" {

sl_status ds_label_cache_update(const void* key, void* label, const int32_t* channels, const int32_t* start,
                                int32_t batch, int32_t heads, int32_t max_seq, int32_t head_dim, int32_t r,
                                int32_t span, void* stream) {
  try {
    g_last_error.clear();
    if (key == nullptr || label == nullptr || channels == nullptr)
      return fail(SL_ERR_ARG, "key, label and channels must not be NULL");
    const sl_status st = ds_check_shape(batch, heads, max_seq, head_dim, r);
    if (st != SL_OK) return st;
    if (span < 0) return fail(SL_ERR_ARG, "span=%d must be >= 0", (int)span);
    if (!aligned(label, 16)) return fail(SL_ERR_UNSUPPORTED, "label must be 16-byte aligned");
    if (!aligned(key, 2) || !aligned(channels, 4) || (start != nullptr && !aligned(start, 4)))
      return fail(SL_ERR_ARG, "key, channels or start misaligned for its element type");
    if (span == 0) return SL_OK;
    const sl_status sd = ds_device();
    if (sd != SL_OK) return sd;
    SL_HIP(sl::launch_ds_label((const uint16_t*)key, (uint16_t*)label, channels, start, batch, heads, max_seq,
                               head_dim, r, std::min<int32_t>(span, DS_MAX_SEQ), (hipStream_t)stream));
    return SL_OK;
  } catch (...) {
    return fail(SL_ERR_HIP, "unexpected exception");
  }
}

sl_status ds_decode_attention(const void* q, const void* key, const void* value, const void* label,
                              const int32_t* channels, const int32_t* seq_len, int32_t batch, int32_t heads,
                              int32_t max_seq, int32_t head_dim, int32_t r, int32_t k, float scale, float* out,
                              int32_t* tokens_out, void* stream) {
  try {
    g_last_error.clear();
    if (q == nullptr || key == nullptr || value == nullptr || channels == nullptr || seq_len == nullptr ||
        out == nullptr)
      return fail(SL_ERR_ARG, "q, key, value, channels, seq_len and out must not be NULL");
    const sl_status st = ds_check_shape(batch, heads, max_seq, head_dim, r);
    if (st != SL_OK) return st;
    if (k < 1) return fail(SL_ERR_ARG, "k=%d must be >= 1", (int)k);
    if (k < max_seq && k > DS_MAX_K)
      return fail(SL_ERR_UNSUPPORTED, "k=%d: at most %d kept tokens unless k >= max_seq", (int)k, DS_MAX_K);
    if (k < max_seq && label == nullptr) return fail(SL_ERR_ARG, "label must not be NULL when k < max_seq");
    if (tokens_out != nullptr && k > DS_MAX_SEQ)
      return fail(SL_ERR_ARG, "k=%d: tokens_out needs k <= %d", (int)k, DS_MAX_SEQ);
    if (!std::isfinite(scale)) return fail(SL_ERR_ARG, "scale must be finite");
    const size_t row_align = head_dim == 128 ? 16 : 8;
    if (!aligned(q, row_align) || !aligned(key, row_align) || !aligned(value, row_align))
      return fail(SL_ERR_UNSUPPORTED, "q, key and value must be %d-byte aligned", (int)row_align);
    if (label != nullptr && !aligned(label, 16)) return fail(SL_ERR_UNSUPPORTED, "label must be 16-byte aligned");
    if (!aligned(out, 4) || !aligned(channels, 4) || !aligned(seq_len, 4) ||
        (tokens_out != nullptr && !aligned(tokens_out, 4)))
      return fail(SL_ERR_ARG, "out, channels, seq_len or tokens_out misaligned for its element type");
    const sl_status sd = ds_device();
    if (sd != SL_OK) return sd;
    sl::DsDecodeParams p;
    p.q = (const uint16_t*)q;
    p.key = (const uint16_t*)key;
    p.value = (const uint16_t*)value;
    p.label = (const uint16_t*)label;
    p.channels = channels;
    p.seq_len = seq_len;
    p.heads = heads;
    p.max_seq = max_seq;
    p.k = k;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.out = out;
    p.tokens_out = tokens_out;
    SL_HIP(sl::launch_ds_decode(p, batch, head_dim, r, (hipStream_t)stream));
    return SL_OK;
  } catch (...) {
    return fail(SL_ERR_HIP, "unexpected exception");
  }
}

}  // extern "C"
