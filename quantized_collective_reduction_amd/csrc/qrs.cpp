// C-ABI host library: parameter checks, plans, and launches on the caller's
// stream. The contract of every entry point is documented in include/qrs.h.

#include "qrs.h"

#include <hip/hip_runtime_api.h>

#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "qrs_launch.h"

struct qrs_launch_s {
  hipStream_t stream;
  uint64_t n_parts;
  qrs::PreparedReduce** parts;  // n_parts launches, enqueued in this order
};

struct qrs_plan_s {
  int world_size;
  int64_t bs;
  int64_t rows;
  int64_t h;
  qrs::XFormat x_format;
  qrs::ScaleLayout scale_layout;
  qrs::OutFormat out_format;
};

namespace {

thread_local char g_last_error[512];

qrs_status fail(qrs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

qrs_status ok() {
  g_last_error[0] = '\0';
  return QRS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// The (x format, scale layout) pair selects one of the page's modes.
qrs_status check_mode(qrs_x_dtype x_dtype, qrs_scale_layout scale_layout) {
  if (x_dtype == QRS_X_HIFLOAT8)
    return fail(QRS_ERR_UNSUPPORTED, "HIFLOAT8 x is reserved: its encoding is not defined");
  if (x_dtype != QRS_X_INT8 && x_dtype != QRS_X_FP8_E4M3FN && x_dtype != QRS_X_FP8_E5M2)
    return fail(QRS_ERR_INVALID_ARG, "x_dtype %d is not a qrs_x_dtype", static_cast<int>(x_dtype));
  if (scale_layout != QRS_SCALE_F32_GROUP128 && scale_layout != QRS_SCALE_E8M0_BLOCK32)
    return fail(QRS_ERR_INVALID_ARG, "scale_layout %d is not a qrs_scale_layout", static_cast<int>(scale_layout));
  // MX mode (E8M0 scales) is defined for the FP8 formats only.
  if (scale_layout == QRS_SCALE_E8M0_BLOCK32 && x_dtype == QRS_X_INT8)
    return fail(QRS_ERR_INVALID_ARG, "INT8 x is paired with fp32 per-group scales only");
  return QRS_OK;
}

// Per-share algorithmic bytes above which qrs_run_all_shares launches each
// share separately (see there).
#ifndef QRS_SPLIT_SHARE_BYTES
#define QRS_SPLIT_SHARE_BYTES 300000000ull
#endif
constexpr uint64_t kSplitShareBytes = QRS_SPLIT_SHARE_BYTES;

// H is 128-aligned and in [1024, 8192].
bool valid_h(int64_t h) { return h >= 1024 && h <= 8192 && h % 128 == 0; }

qrs::XFormat to_x_format(qrs_x_dtype x) {
  return x == QRS_X_INT8 ? qrs::kXInt8 : x == QRS_X_FP8_E4M3FN ? qrs::kXE4M3FN : qrs::kXE5M2;
}

// HIP runs at most 2^32 - 1 work-items along a grid dimension, and every
// kernel gives a lane at least 8 elements. A call over more elements per
// share than one launch may cover (kMaxLaunchElems) therefore runs as
// consecutive launches over consecutive element ranges of each share (whole
// rows of a row-strided share). Each launch computes its elements exactly as
// one launch over the whole share would, so the results are the same bits.
// QRS_MAX_LAUNCH_ELEMS, read once per process, may lower the bound (a
// multiple of 4096 elements), which runs the same split at small sizes; any
// other value makes every call that launches fail with QRS_ERR_INVALID_ARG.
constexpr uint64_t kMaxLaunchElems = uint64_t{1} << 34;  // 2^31 lanes of 8 elements
constexpr uint64_t kMaxCopyBytes = uint64_t{1} << 35;    // 2^31 lanes of 16 bytes

uint64_t max_launch_elems() {
  static const uint64_t bound = [] {
    const char* s = std::getenv("QRS_MAX_LAUNCH_ELEMS");
    if (s == nullptr || *s == '\0') return kMaxLaunchElems;
    char* end = nullptr;
    errno = 0;
    const unsigned long long v = std::strtoull(s, &end, 10);
    if (errno != 0 || *end != '\0' || s[0] < '0' || s[0] > '9' || v < 4096 || v > kMaxLaunchElems || v % 4096 != 0)
      return uint64_t{0};
    return static_cast<uint64_t>(v);
  }();
  return bound;
}

qrs_status check_launch_bound() {
  if (max_launch_elems() == 0)
    return fail(QRS_ERR_INVALID_ARG, "QRS_MAX_LAUNCH_ELEMS must be a multiple of 4096 in [4096, 2^34]");
  return QRS_OK;
}

// Rows per launch of a row-strided share (at least one).
uint64_t part_rows(const qrs::ReduceLaunch& l, uint64_t m) {
  const uint64_t r = m / l.row_elems;
  return r != 0 ? r : 1;
}

uint64_t part_count(const qrs::ReduceLaunch& l, uint64_t m) {
  if (l.n_rows > 1) {
    const uint64_t r = part_rows(l, m);
    return (l.n_rows + r - 1) / r;
  }
  return (l.row_elems + m - 1) / m;
}

// Launch k of l's split. Contiguous shares (n_rows = 1, all shares of a
// group alike): elements [k m, k m + m) of every share, whose scales start
// k m / 32 bytes further on in both layouts (4 bytes per 128 elements, or 1
// per 32); the share strides stay. Row-strided shares: rows [k R, k R + R).
qrs::ReduceLaunch part_of(const qrs::ReduceLaunch& l, uint64_t m, uint64_t k) {
  qrs::ReduceLaunch q = l;
  const uint64_t ob = l.out_format == qrs::kOutF32 ? 4 : 2;
  uint64_t dx, ds, dout;
  if (l.n_rows > 1) {
    const uint64_t r = part_rows(l, m), r0 = k * r;
    q.n_rows = l.n_rows - r0 < r ? l.n_rows - r0 : r;
    dx = r0 * l.x_row_stride;
    ds = r0 * l.scale_row_stride;
    dout = r0 * l.out_row_stride;
  } else {
    const uint64_t e0 = k * m;
    q.row_elems = l.row_elems - e0 < m ? l.row_elems - e0 : m;
    dx = e0;
    ds = e0 / 32;
    dout = e0 * ob;
  }
  for (int r = 0; r < l.world_size; ++r) {
    q.x[r] = static_cast<const char*>(l.x[r]) + dx;
    q.scales[r] = static_cast<const char*>(l.scales[r]) + ds;
  }
  for (int j = 0; j < l.n_shares; ++j) q.out[j] = static_cast<char*>(l.out[j]) + dout;
  return q;
}

// Enqueues l as its launches, in order, after checking every one of them.
hipError_t launch_in_parts(const qrs::ReduceLaunch& l, hipStream_t stream) {
  const uint64_t m = max_launch_elems();
  if (m == 0) return hipErrorInvalidValue;  // callers report check_launch_bound() first
  const uint64_t parts = part_count(l, m);
  if (parts == 1) return qrs::launch_reduce(l, stream);
  for (uint64_t k = 0; k < parts; ++k) {
    qrs::LaunchShape shape;
    const hipError_t e = qrs::reduce_launch_shape(part_of(l, m, k), stream, &shape);
    if (e != hipSuccess) return e;
  }
  for (uint64_t k = 0; k < parts; ++k) {
    const hipError_t e = qrs::launch_reduce(part_of(l, m, k), stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* qrs_status_string(qrs_status status) {
  switch (status) {
    case QRS_OK: return "QRS_OK";
    case QRS_ERR_INVALID_ARG: return "QRS_ERR_INVALID_ARG";
    case QRS_ERR_UNSUPPORTED: return "QRS_ERR_UNSUPPORTED";
    case QRS_ERR_HIP: return "QRS_ERR_HIP";
    case QRS_ERR_OUT_OF_MEMORY: return "QRS_ERR_OUT_OF_MEMORY";
    default: break;
  }
  return "QRS_ERR_UNKNOWN";
}

const char* qrs_last_error(void) { return g_last_error; }

qrs_status qrs_plan(int world_size, int64_t bs, int64_t h, qrs_x_dtype x_dtype, qrs_scale_layout scale_layout,
                    qrs_out_dtype out_dtype, qrs_plan_t* plan_out, size_t* workspace_bytes_out) {
  if (plan_out) *plan_out = nullptr;
  if (!plan_out || !workspace_bytes_out) return fail(QRS_ERR_INVALID_ARG, "plan_out and workspace_bytes_out must be non-null");
  // Communicator size 2, 4 or 8.
  if (world_size != 2 && world_size != 4 && world_size != 8)
    return fail(QRS_ERR_INVALID_ARG, "world_size %d: must be 2, 4 or 8", world_size);
  // Empty input is not supported; the share has bs / W rows.
  if (bs <= 0) return fail(QRS_ERR_INVALID_ARG, "bs %lld: must be positive", static_cast<long long>(bs));
  if (bs % world_size != 0)
    return fail(QRS_ERR_INVALID_ARG, "bs %lld is not a multiple of world_size %d", static_cast<long long>(bs),
                world_size);
  // H is 128-aligned and in [1024, 8192].
  if (!valid_h(h))
    return fail(QRS_ERR_INVALID_ARG, "h %lld: must be a multiple of 128 in [1024, 8192]", static_cast<long long>(h));
  const int64_t rows = bs / world_size;
  // At most 2^40 elements per share (2^34 per launch: larger shares run as several launches).
  if (rows > (int64_t{1} << 40) / h) return fail(QRS_ERR_INVALID_ARG, "bs %lld too large", static_cast<long long>(bs));

  const qrs_status mode = check_mode(x_dtype, scale_layout);
  if (mode != QRS_OK) return mode;
  if (out_dtype != QRS_OUT_F32 && out_dtype != QRS_OUT_BF16 && out_dtype != QRS_OUT_F16)
    return fail(QRS_ERR_INVALID_ARG, "out_dtype %d is not a qrs_out_dtype", static_cast<int>(out_dtype));

  qrs_plan_s* p = new (std::nothrow) qrs_plan_s;
  if (!p) return fail(QRS_ERR_OUT_OF_MEMORY, "out of host memory");
  p->world_size = world_size;
  p->bs = bs;
  p->rows = rows;
  p->h = h;
  p->x_format = to_x_format(x_dtype);
  p->scale_layout = scale_layout == QRS_SCALE_F32_GROUP128 ? qrs::kScaleF32Group128 : qrs::kScaleE8M0Block32;
  p->out_format = out_dtype == QRS_OUT_F32 ? qrs::kOutF32 : out_dtype == QRS_OUT_BF16 ? qrs::kOutBF16 : qrs::kOutF16;
  *plan_out = p;
  *workspace_bytes_out = 0;
  return ok();
}

qrs_status qrs_plan_destroy(qrs_plan_t plan) {
  delete plan;
  return ok();
}

qrs_status qrs_plan_shape(qrs_plan_t plan, int64_t* rows_out, int64_t* h_out) {
  if (!plan) return fail(QRS_ERR_INVALID_ARG, "null plan");
  if (rows_out) *rows_out = plan->rows;
  if (h_out) *h_out = plan->h;
  return ok();
}

qrs_status qrs_slice_pitch(qrs_plan_t plan, int full_inputs, size_t* x_pitch_out, size_t* scale_pitch_out) {
  if (!plan) return fail(QRS_ERR_INVALID_ARG, "null plan");
  if (full_inputs != 0 && full_inputs != 1) return fail(QRS_ERR_INVALID_ARG, "full_inputs must be 0 or 1");
  const uint64_t rows = static_cast<uint64_t>(full_inputs ? plan->bs : plan->rows);
  const uint64_t x_bytes = rows * static_cast<uint64_t>(plan->h);
  const uint64_t s_bytes = plan->scale_layout == qrs::kScaleF32Group128 ? x_bytes / 128 * 4 : x_bytes / 32;
  // x: round up to 64 KiB, then stagger to 1.25 MiB modulo 4 MiB (the
  // residue the W read streams are fastest at, whatever the slice size).
  // Scales: round up to 4 KiB, then a 40 KiB stagger.
  auto round_up = [](uint64_t v, uint64_t a) { return (v + a - 1) / a * a; };
  const uint64_t period = uint64_t{4} << 20, residue = uint64_t{1280} << 10;
  const uint64_t x_base = round_up(x_bytes, 64 * 1024);
  if (x_pitch_out) *x_pitch_out = x_base + (residue + period - x_base % period) % period;
  if (scale_pitch_out) *scale_pitch_out = round_up(s_bytes, 4096) + 40 * 1024;
  return ok();
}

}  // extern "C"

namespace {

// The checks of qrs_run, and the launch they describe.
qrs_status share_launch(qrs_plan_t plan, const void* const* x_slices, const void* const* scale_slices, void* out,
                        qrs::ReduceLaunch* lp) {
  qrs::ReduceLaunch& l = *lp;
  if (!plan) return fail(QRS_ERR_INVALID_ARG, "null plan");
  if (!x_slices || !scale_slices || !out) return fail(QRS_ERR_INVALID_ARG, "null pointer array or output");
  const int W = plan->world_size;
  const uint64_t n = static_cast<uint64_t>(plan->rows) * static_cast<uint64_t>(plan->h);
  const bool f32_scales = plan->scale_layout == qrs::kScaleF32Group128;
  const uint64_t scale_bytes = f32_scales ? n / 128 * 4 : n / 32;
  const uint64_t out_bytes = n * (plan->out_format == qrs::kOutF32 ? 4 : 2);
  if (!aligned(out, 16)) return fail(QRS_ERR_INVALID_ARG, "out is not 16-byte aligned");

  std::memset(&l, 0, sizeof(l));
  l.world_size = W;
  l.x_format = plan->x_format;
  l.scale_layout = plan->scale_layout;
  l.out_format = plan->out_format;
  l.n_rows = 1;
  l.row_elems = n;
  l.n_shares = 1;
  l.out[0] = out;
  for (int r = 0; r < W; ++r) {
    if (!x_slices[r] || !scale_slices[r]) return fail(QRS_ERR_INVALID_ARG, "null slice pointer for rank %d", r);
    if (!aligned(x_slices[r], 16)) return fail(QRS_ERR_INVALID_ARG, "x slice of rank %d is not 16-byte aligned", r);
    if (f32_scales && !aligned(scale_slices[r], 4))
      return fail(QRS_ERR_INVALID_ARG, "fp32 scale slice of rank %d is not 4-byte aligned", r);
    if (overlaps(out, out_bytes, x_slices[r], n) || overlaps(out, out_bytes, scale_slices[r], scale_bytes))
      return fail(QRS_ERR_INVALID_ARG, "out overlaps an input slice of rank %d", r);
    l.x[r] = x_slices[r];
    l.scales[r] = scale_slices[r];
  }
  return QRS_OK;
}

}  // namespace

extern "C" {

qrs_status qrs_run(qrs_plan_t plan, const void* const* x_slices, const void* const* scale_slices, void* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  qrs::ReduceLaunch l;
  qrs_status st = share_launch(plan, x_slices, scale_slices, out, &l);
  if (st != QRS_OK) return st;
  st = check_launch_bound();
  if (st != QRS_OK) return st;
  const hipError_t e = launch_in_parts(l, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

qrs_status qrs_launch_create(qrs_plan_t plan, const void* const* x_slices, const void* const* scale_slices, void* out,
                             void* stream, qrs_launch_t* launch_out) {
  if (launch_out) *launch_out = nullptr;
  if (!launch_out) return fail(QRS_ERR_INVALID_ARG, "null launch_out");
  qrs::ReduceLaunch l;
  qrs_status st = share_launch(plan, x_slices, scale_slices, out, &l);
  if (st != QRS_OK) return st;
  st = check_launch_bound();
  if (st != QRS_OK) return st;
  const uint64_t m = max_launch_elems();
  qrs_launch_s* h = new (std::nothrow) qrs_launch_s;
  if (!h) return fail(QRS_ERR_OUT_OF_MEMORY, "out of host memory");
  h->stream = static_cast<hipStream_t>(stream);
  h->n_parts = part_count(l, m);
  h->parts = new (std::nothrow) qrs::PreparedReduce*[h->n_parts]();
  if (!h->parts) {
    delete h;
    return fail(QRS_ERR_OUT_OF_MEMORY, "out of host memory");
  }
  for (uint64_t k = 0; k < h->n_parts; ++k) {
    const hipError_t e = qrs::prepare_reduce_launch(part_of(l, m, k), h->stream, &h->parts[k]);
    if (e != hipSuccess) {
      qrs_launch_destroy(h);
      if (e == hipErrorOutOfMemory) return fail(QRS_ERR_OUT_OF_MEMORY, "out of host memory");
      return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
  }
  *launch_out = h;
  return ok();
}

qrs_status qrs_launch_enqueue(qrs_launch_t launch) {
  if (!launch) return fail(QRS_ERR_INVALID_ARG, "null launch");
  for (uint64_t k = 0; k < launch->n_parts; ++k) {
    const hipError_t e = qrs::enqueue_prepared_reduce(launch->parts[k], launch->stream);
    if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

qrs_status qrs_launch_destroy(qrs_launch_t launch) {
  if (launch) {
    for (uint64_t k = 0; k < launch->n_parts; ++k)
      if (launch->parts[k]) qrs::destroy_prepared_reduce(launch->parts[k]);
    delete[] launch->parts;
    delete launch;
  }
  return ok();
}

qrs_status qrs_run_launch_info(qrs_plan_t plan, void* stream, qrs_launch_info* info_out) {
  if (!plan || !info_out) return fail(QRS_ERR_INVALID_ARG, "null plan or info pointer");
  qrs::ReduceLaunch l;
  std::memset(&l, 0, sizeof(l));
  l.world_size = plan->world_size;
  l.x_format = plan->x_format;
  l.scale_layout = plan->scale_layout;
  l.out_format = plan->out_format;
  l.n_rows = 1;
  l.row_elems = static_cast<uint64_t>(plan->rows) * static_cast<uint64_t>(plan->h);
  l.n_shares = 1;
  const qrs_status st = check_launch_bound();
  if (st != QRS_OK) return st;
  const uint64_t m = max_launch_elems();
  qrs::LaunchShape shape;
  const hipError_t e = qrs::reduce_launch_shape(part_of(l, m, 0), static_cast<hipStream_t>(stream), &shape);
  if (e != hipSuccess) return fail(QRS_ERR_HIP, "launch shape: %s", hipGetErrorString(e));
  info_out->launches = static_cast<uint32_t>(part_count(l, m));  // at most 2^40 / 4096
  info_out->blocks = shape.blocks;
  info_out->threads_per_block = shape.threads_per_block;
  info_out->dynamic_lds_bytes = shape.dynamic_lds;
  info_out->blocks_per_cu_cap = shape.blocks_per_cu_cap;
  info_out->device_cus = shape.device.cus;
  info_out->device_lds_per_cu = shape.device.lds_per_cu;
  info_out->device_lds_per_block = shape.device.lds_per_block;
  return ok();
}

qrs_status qrs_run_all_shares(qrs_plan_t plan, const void* const* x_full, const void* const* scale_full,
                              void* const* out_shares, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!plan) return fail(QRS_ERR_INVALID_ARG, "null plan");
  if (!x_full || !scale_full || !out_shares) return fail(QRS_ERR_INVALID_ARG, "null pointer array");
  const int W = plan->world_size;
  const uint64_t n = static_cast<uint64_t>(plan->rows) * static_cast<uint64_t>(plan->h);  // per share
  const bool f32_scales = plan->scale_layout == qrs::kScaleF32Group128;
  const uint64_t share_scale_bytes = f32_scales ? n / 128 * 4 : n / 32;
  const uint64_t out_bytes = n * (plan->out_format == qrs::kOutF32 ? 4 : 2);
  const uint64_t full_x_bytes = n * W, full_scale_bytes = share_scale_bytes * W;

  qrs::ReduceLaunch l;
  std::memset(&l, 0, sizeof(l));
  l.world_size = W;
  l.x_format = plan->x_format;
  l.scale_layout = plan->scale_layout;
  l.out_format = plan->out_format;
  l.n_rows = 1;
  l.row_elems = n;
  l.n_shares = W;
  l.x_share_stride = n;  // row block j of rank r starts j * rows * H bytes into x_full[r]
  l.scale_share_stride = share_scale_bytes;
  for (int j = 0; j < W; ++j) {
    if (!out_shares[j]) return fail(QRS_ERR_INVALID_ARG, "null output for share %d", j);
    if (!aligned(out_shares[j], 16)) return fail(QRS_ERR_INVALID_ARG, "output of share %d is not 16-byte aligned", j);
    for (int k = 0; k < j; ++k)
      if (overlaps(out_shares[j], out_bytes, out_shares[k], out_bytes))
        return fail(QRS_ERR_INVALID_ARG, "outputs of shares %d and %d overlap", k, j);
    l.out[j] = out_shares[j];
  }
  for (int r = 0; r < W; ++r) {
    if (!x_full[r] || !scale_full[r]) return fail(QRS_ERR_INVALID_ARG, "null input pointer for rank %d", r);
    if (!aligned(x_full[r], 16)) return fail(QRS_ERR_INVALID_ARG, "x of rank %d is not 16-byte aligned", r);
    if (f32_scales && !aligned(scale_full[r], 4))
      return fail(QRS_ERR_INVALID_ARG, "fp32 scales of rank %d are not 4-byte aligned", r);
    for (int j = 0; j < W; ++j)
      if (overlaps(out_shares[j], out_bytes, x_full[r], full_x_bytes) ||
          overlaps(out_shares[j], out_bytes, scale_full[r], full_scale_bytes))
        return fail(QRS_ERR_INVALID_ARG, "output of share %d overlaps an input of rank %d", j, r);
    l.x[r] = x_full[r];
    l.scales[r] = scale_full[r];
  }
  // Large shares of the uncapped launches run as one launch each: past about
  // 300 MB of algorithmic bytes per share that measured faster than one
  // launch over all shares (514 MB per share with fp32 group scales: 640
  // against 671 us for the group; MX at W = 2: 156 against 173 us), while
  // smaller shares gain from sharing one launch's fixed cost (172 MB per
  // share: 207 against 223 us). Groups that run as capped 8-element pieces
  // (MX at W = 8) stay one launch at any size (514 MB per share: 607 against
  // 614 us). Both give the same bits.
  const uint64_t share_bytes = n * static_cast<uint64_t>(W) + share_scale_bytes * static_cast<uint64_t>(W) + out_bytes;
  const qrs_status st = check_launch_bound();
  if (st != QRS_OK) return st;
  hipError_t e = hipSuccess;
  if (share_bytes > kSplitShareBytes && !qrs::all_shares_take_one_capped_launch(l)) {
    qrs::ReduceLaunch one = l;
    one.n_shares = 1;
    for (int j = 0; j < W && e == hipSuccess; ++j) {
      for (int r = 0; r < W; ++r) {
        one.x[r] = static_cast<const char*>(x_full[r]) + static_cast<uint64_t>(j) * n;
        one.scales[r] = static_cast<const char*>(scale_full[r]) + static_cast<uint64_t>(j) * share_scale_bytes;
      }
      for (int k = 0; k < qrs::kMaxWorld; ++k) one.out[k] = nullptr;
      one.out[0] = out_shares[j];
      e = launch_in_parts(one, static_cast<hipStream_t>(stream));
    }
  } else {
    e = launch_in_parts(l, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

qrs_status qrs_run_strided(qrs_plan_t plan, const void* const* x_slices, int64_t x_row_stride,
                           const void* const* scale_slices, int64_t scale_row_stride, void* out,
                           int64_t out_row_stride, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!plan) return fail(QRS_ERR_INVALID_ARG, "null plan");
  if (!x_slices || !scale_slices || !out) return fail(QRS_ERR_INVALID_ARG, "null pointer array or output");
  const int W = plan->world_size;
  const int64_t rows = plan->rows, h = plan->h;
  const bool f32_scales = plan->scale_layout == qrs::kScaleF32Group128;
  const int64_t g = f32_scales ? 128 : 32;
  const int64_t sb = f32_scales ? 4 : 1;
  const int64_t ob = plan->out_format == qrs::kOutF32 ? 4 : 2;
  // Lower bounds first, so that every product below is of positive values.
  if (x_row_stride < h || x_row_stride % 16)
    return fail(QRS_ERR_INVALID_ARG, "x_row_stride %lld: must be >= h and a multiple of 16 bytes",
                static_cast<long long>(x_row_stride));
  if (scale_row_stride < h / g)
    return fail(QRS_ERR_INVALID_ARG, "scale_row_stride %lld: must be >= h / %lld", static_cast<long long>(scale_row_stride),
                static_cast<long long>(g));
  if (out_row_stride < h) return fail(QRS_ERR_INVALID_ARG, "out_row_stride %lld: must be >= h", static_cast<long long>(out_row_stride));
  // Every address the kernel forms must stay well inside 64 bits: bound the
  // byte extent of each tensor (rows - 1 strides plus one row) by 2^48.
  // Compare before multiplying so the check itself cannot overflow.
  const int64_t limit = int64_t{1} << 48;
  if (x_row_stride > limit / rows || scale_row_stride > limit / rows / sb || out_row_stride > limit / rows / ob)
    return fail(QRS_ERR_INVALID_ARG, "row stride too large for %lld rows", static_cast<long long>(rows));
  // The kernel forms each row's offset as a 32 x 32-bit product.
  const int64_t stride_limit = int64_t{1} << 32;
  if (rows >= stride_limit) return fail(QRS_ERR_INVALID_ARG, "%lld rows: must be below 2^32", static_cast<long long>(rows));
  if (x_row_stride >= stride_limit || scale_row_stride * sb >= stride_limit || out_row_stride * ob >= stride_limit)
    return fail(QRS_ERR_INVALID_ARG, "row strides must be below 4 GiB");
  if ((out_row_stride * ob) % 16)
    return fail(QRS_ERR_INVALID_ARG, "out_row_stride %lld: must span a multiple of 16 bytes",
                static_cast<long long>(out_row_stride));
  if (!aligned(out, 16)) return fail(QRS_ERR_INVALID_ARG, "out is not 16-byte aligned");
  // Extents actually addressed (last row ends at its h-th element).
  const uint64_t x_span = static_cast<uint64_t>((rows - 1) * x_row_stride + h);
  const uint64_t s_span = static_cast<uint64_t>(((rows - 1) * scale_row_stride + h / g) * sb);
  const uint64_t o_span = static_cast<uint64_t>(((rows - 1) * out_row_stride + h) * ob);
  if (s_span >= (uint64_t{1} << 32))
    return fail(QRS_ERR_INVALID_ARG, "the scale rows of one slice must span less than 4 GiB");

  qrs::ReduceLaunch l;
  std::memset(&l, 0, sizeof(l));
  l.world_size = W;
  l.x_format = plan->x_format;
  l.scale_layout = plan->scale_layout;
  l.out_format = plan->out_format;
  l.n_rows = static_cast<uint64_t>(rows);
  l.row_elems = static_cast<uint64_t>(h);
  l.x_row_stride = static_cast<uint64_t>(x_row_stride);
  l.scale_row_stride = static_cast<uint64_t>(scale_row_stride * sb);
  l.out_row_stride = static_cast<uint64_t>(out_row_stride * ob);
  l.n_shares = 1;
  l.out[0] = out;
  for (int r = 0; r < W; ++r) {
    if (!x_slices[r] || !scale_slices[r]) return fail(QRS_ERR_INVALID_ARG, "null slice pointer for rank %d", r);
    if (!aligned(x_slices[r], 16)) return fail(QRS_ERR_INVALID_ARG, "x slice of rank %d is not 16-byte aligned", r);
    if (f32_scales && !aligned(scale_slices[r], 4))
      return fail(QRS_ERR_INVALID_ARG, "fp32 scale slice of rank %d is not 4-byte aligned", r);
    if (overlaps(out, o_span, x_slices[r], x_span) || overlaps(out, o_span, scale_slices[r], s_span))
      return fail(QRS_ERR_INVALID_ARG, "out overlaps an input slice of rank %d", r);
    l.x[r] = x_slices[r];
    l.scales[r] = scale_slices[r];
  }
  const qrs_status st = check_launch_bound();
  if (st != QRS_OK) return st;
  const hipError_t e = launch_in_parts(l, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

qrs_status qrs_quantize(int64_t tokens, int64_t h, qrs_x_dtype x_dtype, qrs_scale_layout scale_layout,
                        const void* x_bf16, void* x_codes, void* scales, void* stream) {
  if (tokens <= 0) return fail(QRS_ERR_INVALID_ARG, "tokens %lld: must be positive", static_cast<long long>(tokens));
  if (!valid_h(h))
    return fail(QRS_ERR_INVALID_ARG, "h %lld: must be a multiple of 128 in [1024, 8192]", static_cast<long long>(h));
  if (tokens > (int64_t{1} << 40) / h)
    return fail(QRS_ERR_INVALID_ARG, "tokens %lld too large", static_cast<long long>(tokens));
  const qrs_status mode = check_mode(x_dtype, scale_layout);
  if (mode != QRS_OK) return mode;
  if (!x_bf16 || !x_codes || !scales) return fail(QRS_ERR_INVALID_ARG, "null pointer");
  const bool f32_scales = scale_layout == QRS_SCALE_F32_GROUP128;
  if (!aligned(x_bf16, 16)) return fail(QRS_ERR_INVALID_ARG, "input is not 16-byte aligned");
  if (!aligned(x_codes, 16)) return fail(QRS_ERR_INVALID_ARG, "codes output is not 16-byte aligned");
  if (f32_scales && !aligned(scales, 4)) return fail(QRS_ERR_INVALID_ARG, "fp32 scales are not 4-byte aligned");
  const uint64_t n = static_cast<uint64_t>(tokens) * static_cast<uint64_t>(h);
  const uint64_t scale_bytes = f32_scales ? n / 128 * 4 : n / 32;
  if (overlaps(x_bf16, 2 * n, x_codes, n) || overlaps(x_bf16, 2 * n, scales, scale_bytes) ||
      overlaps(x_codes, n, scales, scale_bytes))
    return fail(QRS_ERR_INVALID_ARG, "input, codes and scales must not overlap");
  const qrs_status st = check_launch_bound();
  if (st != QRS_OK) return st;
  // Consecutive launches of at most max_launch_elems() elements, as for the
  // reduce: groups never cross a launch's edge, whose scales start e0 / 32
  // bytes on in both layouts.
  const uint64_t m = max_launch_elems();
  for (uint64_t e0 = 0; e0 < n; e0 += m) {
    qrs::QuantizeLaunch l;
    l.x_format = to_x_format(x_dtype);
    l.scale_layout = f32_scales ? qrs::kScaleF32Group128 : qrs::kScaleE8M0Block32;
    l.n_elems = n - e0 < m ? n - e0 : m;
    l.in = static_cast<const char*>(x_bf16) + 2 * e0;
    l.codes = static_cast<char*>(x_codes) + e0;
    l.scales = static_cast<char*>(scales) + e0 / 32;
    const hipError_t e = qrs::launch_quantize(l, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

qrs_status qrs_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(QRS_ERR_INVALID_ARG, "null pointer");
  if (bytes == 0 || bytes % 16 != 0) return fail(QRS_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(QRS_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (overlaps(src, bytes, dst, bytes)) return fail(QRS_ERR_INVALID_ARG, "ranges overlap");
  for (uint64_t b0 = 0; b0 < bytes; b0 += kMaxCopyBytes) {
    const uint64_t nb = bytes - b0 < kMaxCopyBytes ? bytes - b0 : kMaxCopyBytes;
    const hipError_t e = qrs::launch_stream_copy(static_cast<const char*>(src) + b0, static_cast<char*>(dst) + b0, nb,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QRS_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"
