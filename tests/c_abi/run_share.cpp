// A C++ caller of the C ABI with no Python in the loop: reads a problem from
// a binary file, runs qrs_plan / qrs_run on its own HIP stream with hipMalloc'd
// buffers, and writes the output bytes to a file. It also runs the same share
// through a prepared launch (qrs_launch_create, two qrs_launch_enqueue) into a
// second buffer and exits with status 4 if those bytes differ.
//
// Input file layout (little endian): int32 W, int64 BS, int64 H, int32 x_dtype,
// int32 scale_layout, int32 out_dtype, then W x slices [BS/W, H] (uint8), then
// W scale slices (fp32 [BS/W, H/128] or uint8 [BS/W, H/32]).
//
// usage: run_share IN OUT
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qrs.h"

#define HIP_OK(e)                                                              \
  do {                                                                         \
    hipError_t err_ = (e);                                                     \
    if (err_ != hipSuccess) {                                                  \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(err_), __LINE__); \
      return 2;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 1;
  int32_t w, xd, sl, od;
  int64_t bs, h;
  if (std::fread(&w, 4, 1, f) != 1 || std::fread(&bs, 8, 1, f) != 1 || std::fread(&h, 8, 1, f) != 1 ||
      std::fread(&xd, 4, 1, f) != 1 || std::fread(&sl, 4, 1, f) != 1 || std::fread(&od, 4, 1, f) != 1)
    return 1;

  qrs_plan_t plan = nullptr;
  size_t ws = 0;
  qrs_status st = qrs_plan(w, bs, h, static_cast<qrs_x_dtype>(xd), static_cast<qrs_scale_layout>(sl),
                           static_cast<qrs_out_dtype>(od), &plan, &ws);
  if (st != QRS_OK) {
    std::fprintf(stderr, "qrs_plan: %s (%s)\n", qrs_status_string(st), qrs_last_error());
    return 3;
  }
  int64_t rows = 0;
  qrs_plan_shape(plan, &rows, nullptr);
  const size_t n = static_cast<size_t>(rows * h);
  const size_t sbytes = sl == QRS_SCALE_F32_GROUP128 ? n / 128 * 4 : n / 32;
  const size_t obytes = n * (od == QRS_OUT_F32 ? 4 : 2);

  std::vector<unsigned char> host(w * n + w * sbytes);
  if (std::fread(host.data(), 1, host.size(), f) != host.size()) return 1;
  std::fclose(f);

  std::vector<void*> dx(w), ds(w);
  for (int r = 0; r < w; ++r) {
    HIP_OK(hipMalloc(&dx[r], n));
    HIP_OK(hipMalloc(&ds[r], sbytes));
    HIP_OK(hipMemcpy(dx[r], host.data() + r * n, n, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(ds[r], host.data() + w * n + r * sbytes, sbytes, hipMemcpyHostToDevice));
  }
  void* dout = nullptr;
  HIP_OK(hipMalloc(&dout, obytes));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  st = qrs_run(plan, dx.data(), ds.data(), dout, nullptr, 0, stream);
  if (st != QRS_OK) {
    std::fprintf(stderr, "qrs_run: %s (%s)\n", qrs_status_string(st), qrs_last_error());
    return 3;
  }
  HIP_OK(hipStreamSynchronize(stream));
  std::vector<unsigned char> out(obytes);
  HIP_OK(hipMemcpy(out.data(), dout, obytes, hipMemcpyDeviceToHost));

  // The prepared launch of the same share, enqueued twice.
  void* dout2 = nullptr;
  HIP_OK(hipMalloc(&dout2, obytes));
  HIP_OK(hipMemset(dout2, 0xFF, obytes));
  qrs_launch_t launch = nullptr;
  st = qrs_launch_create(plan, dx.data(), ds.data(), dout2, stream, &launch);
  if (st != QRS_OK) {
    std::fprintf(stderr, "qrs_launch_create: %s (%s)\n", qrs_status_string(st), qrs_last_error());
    return 3;
  }
  for (int k = 0; k < 2; ++k) {
    st = qrs_launch_enqueue(launch);
    if (st != QRS_OK) {
      std::fprintf(stderr, "qrs_launch_enqueue: %s (%s)\n", qrs_status_string(st), qrs_last_error());
      return 3;
    }
  }
  HIP_OK(hipStreamSynchronize(stream));
  qrs_launch_destroy(launch);
  std::vector<unsigned char> out2(obytes);
  HIP_OK(hipMemcpy(out2.data(), dout2, obytes, hipMemcpyDeviceToHost));
  HIP_OK(hipFree(dout2));
  if (std::memcmp(out.data(), out2.data(), obytes) != 0) {
    std::fprintf(stderr, "prepared launch differs from qrs_run\n");
    return 4;
  }

  FILE* g = std::fopen(argv[2], "wb");
  if (!g || std::fwrite(out.data(), 1, obytes, g) != obytes) return 1;
  std::fclose(g);

  HIP_OK(hipStreamDestroy(stream));
  for (int r = 0; r < w; ++r) {
    HIP_OK(hipFree(dx[r]));
    HIP_OK(hipFree(ds[r]));
  }
  HIP_OK(hipFree(dout));
  qrs_plan_destroy(plan);
  return 0;
}
