// Internal interface between the C-ABI host library (qrs.cpp) and the gfx950
// kernels (qrs_kernels.hip). Not installed; callers use include/qrs.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qrs {

constexpr int kMaxWorld = 8;

template <typename T>
struct same_type {
  using type = T;
};

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return the status
// of this launch itself. A triple-chevron launch returns nothing, and
// reading hipGetLastError after it would also report an earlier, unrelated
// failure of the calling thread as this launch's. Each argument takes the
// exact type of its kernel parameter, so the bytes handed to the runtime
// are the parameter's.
template <typename... Params>
inline hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                                typename same_type<Params>::type... args) {
  void* arg_ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, arg_ptrs, 0, stream);
}

// Element and scale formats as the kernels see them.
enum XFormat : int { kXInt8 = 0, kXE4M3FN = 1, kXE5M2 = 2 };
enum ScaleLayout : int { kScaleF32Group128 = 0, kScaleE8M0Block32 = 1 };
enum OutFormat : int { kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2 };

// One launch of the dequant + rank-ordered reduce. A share is n_rows rows of
// row_elems elements (a multiple of 128). Element c of row i of rank r's
// slice is byte i * x_row_stride + c of x[r]; its scale is element c / G of
// the row that starts i * scale_row_stride bytes into scales[r]; the output
// row starts i * out_row_stride bytes into the output. A contiguous share is
// the case n_rows = 1, row_elems = rows * H (G divides H, so the flat
// indexing is the same), strides unused.
//
// n_shares == 1: x[r] / scales[r] point at rank r's slice of this GPU's
// share, out[0] at the share's output.
// n_shares == W: x[r] / scales[r] point at rank r's whole [BS, H] input (and
// its scales) before the all-to-all; share j reads row block j of every
// rank, found x_share_stride / scale_share_stride bytes further on, and
// writes out[j].
struct ReduceLaunch {
  int world_size;          // 2, 4 or 8
  XFormat x_format;
  ScaleLayout scale_layout;
  OutFormat out_format;
  uint64_t n_rows;
  uint64_t row_elems;
  uint64_t x_row_stride;      // bytes, a multiple of 16
  uint64_t scale_row_stride;  // bytes
  uint64_t out_row_stride;    // bytes, a multiple of 16
  int n_shares;               // 1 or world_size
  uint64_t x_share_stride;      // bytes between consecutive shares' x row blocks
  uint64_t scale_share_stride;  // bytes between consecutive shares' scale row blocks
  const void* x[kMaxWorld];
  const void* scales[kMaxWorld];
  void* out[kMaxWorld];
};

// Returns hipErrorInvalidValue, launching nothing, for shapes outside the
// kernels' index ranges: 2^39 or more chunks of 16 elements in a share;
// for n_rows > 1 also rows or a row stride (in its units) of 2^32 or more,
// a scale slice spanning 4 GiB or more, or a row of fewer than 64 or more
// than 768 chunks. The caller keeps one launch at or below 2^34 elements per
// share (qrs.cpp splits larger shares into several launches): a HIP grid
// holds fewer than 2^32 work-items along a dimension, and a lane takes 8 or
// 16 elements.
hipError_t launch_reduce(const ReduceLaunch& l, hipStream_t stream);

// Whether an all-shares launch of this mode (n_shares = world_size) runs as
// 8-element pieces with a residency cap: such groups measured faster as one
// launch even where their shares are large.
bool all_shares_take_one_capped_launch(const ReduceLaunch& l);

// launch_reduce in two steps: prepare_reduce_launch chooses the kernel, grid,
// residency cap (for the device of `stream`) and arguments once and keeps
// them in *out (host memory; the same errors as launch_reduce, or
// hipErrorOutOfMemory); enqueue_prepared_reduce enqueues them on `stream`.
struct PreparedReduce;
hipError_t prepare_reduce_launch(const ReduceLaunch& l, hipStream_t stream, PreparedReduce** out);
hipError_t enqueue_prepared_reduce(const PreparedReduce* p, hipStream_t stream);
void destroy_prepared_reduce(PreparedReduce* p);

// The launch device's compute-unit count and LDS sizes in bytes, as
// hipDeviceGetAttribute reports them (multiprocessor count, shared memory per
// multiprocessor, shared memory per block) for the device of `stream` (the
// current device for the null stream). Read once per device and cached;
// false if they cannot be read.
struct DeviceShape {
  uint32_t cus;
  uint32_t lds_per_cu;
  uint32_t lds_per_block;
};
bool device_shape(hipStream_t stream, DeviceShape* out);

// What launch_reduce would enqueue for l on stream, without enqueuing it:
// work-groups, threads per work-group, the unused dynamic LDS that caps
// residency (0 = none), the cap in work-groups per CU (0 = none), and the
// device sizes the cap was derived from (zeros if they could not be read).
struct LaunchShape {
  uint64_t blocks;
  uint32_t threads_per_block;
  uint32_t dynamic_lds;
  uint32_t blocks_per_cu_cap;
  DeviceShape device;
};
hipError_t reduce_launch_shape(const ReduceLaunch& l, hipStream_t stream, LaunchShape* out);

// Producer-side quantization of n_elems bf16 values (a multiple of 128,
// row-major [tokens, H] with G dividing H, so groups never cross rows):
// codes (uint8, one per element) and scales (fp32 per 128 or E8M0 per 32).
struct QuantizeLaunch {
  XFormat x_format;
  ScaleLayout scale_layout;
  uint64_t n_elems;
  const void* in;  // bf16, 16-byte aligned
  void* codes;     // 8-byte aligned
  void* scales;    // 4-byte aligned for fp32
};

// At most 2^34 elements per launch, as for launch_reduce (qrs.cpp splits).
hipError_t launch_quantize(const QuantizeLaunch& l, hipStream_t stream);

// Plain 16-byte-per-lane device copy (bytes % 16 == 0, both pointers 16-byte
// aligned, at most 2^35 bytes per launch): the reference stream for bandwidth
// and traffic-counter calibration.
hipError_t launch_stream_copy(const void* src, void* dst, uint64_t bytes, hipStream_t stream);

}  // namespace qrs
