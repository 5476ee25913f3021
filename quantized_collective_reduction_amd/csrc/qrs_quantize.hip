// gfx950 kernel for the producer side of the quantized reduce-scatter: bf16
// activations -> x codes + scales in one of the two modes the page
// "aclnnQuantReduceScatter" accepts (Constraints): per-token-per-group (128
// columns, fp32 scales; INT8, E4M3FN or E5M2 codes) or MX (32 elements, E8M0
// scales; E4M3FN or E5M2 codes).
//
// The page does not say how scales are chosen. MX follows the conversion of
// the OCP Microscaling v1.0 specification: shared exponent
// floor(log2(amax)) - emax of the element format, limited to the E8M0 range;
// elements divided by that power of two (exact) and rounded nearest-even,
// clamped to the largest normal. The per-group mode uses scale = amax / qmax
// and codes = RNE(clamp(v * (qmax / amax))), the scale kept at or above 2^-126
// (multiplier 2^126 there, so it never overflows). Zero blocks get E8M0 code 0
// (MX) and zero codes.
//
// A lane owns pieces of 8 consecutive elements (one 16-byte load of bf16, one
// 8-byte store of codes each), so every load and store instruction of a wave
// is contiguous. A group is G/8 consecutive lanes (16 for G = 128, 4 for
// G = 32); its absolute maximum is combined across those lanes with DPP lane
// moves. The kernel streams 3 bytes per element and is bound by HBM.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qrs_launch.h"

// One rounding per operation: never fuse.
#pragma clang fp contract(off)

namespace qrs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kElemsPerLane = 8;

// 8-element pieces per lane; piece j of a lane is block_first + j*kBlock +
// lane, so each load and store instruction of a wave stays contiguous.
#ifndef QRS_Q_PIECES
#define QRS_Q_PIECES 2
#endif
// Group maximum across lanes with DPP lane moves (1) or LDS permutes (0).
#ifndef QRS_Q_DPP
#define QRS_Q_DPP 1
#endif

template <int XF>
struct Fmt;
template <>
struct Fmt<kXInt8> {
  static constexpr float kMax = 127.0f;
};
template <>
struct Fmt<kXE4M3FN> {
  static constexpr float kMax = 448.0f;
  static constexpr int kEmax = 8;  // 448 = 1.75 * 2^8
};
template <>
struct Fmt<kXE5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr int kEmax = 15;  // 57344 = 1.75 * 2^15
};

// Four values already clamped to the format's range -> four codes in one
// 32-bit word (byte k = value k), nearest-even.
template <int XF>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  if constexpr (XF == kXInt8) {
    const uint32_t ia = static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(a))) & 0xFFu;
    const uint32_t ib = static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(b))) & 0xFFu;
    const uint32_t ic = static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(c))) & 0xFFu;
    const uint32_t id = static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(d))) & 0xFFu;
    return ia | (ib << 8) | (ic << 16) | (id << 24);
  } else if constexpr (XF == kXE4M3FN) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
  } else {
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
  }
}

__device__ __forceinline__ float clampf(float v, float lim) { return fminf(fmaxf(v, -lim), lim); }

// 2^k for k in [-127, 127] as an exact binary32 (2^-127 is subnormal).
__device__ __forceinline__ float exp2_int(int k) {
  const uint32_t bits = k >= -126 ? static_cast<uint32_t>(k + 127) << 23 : 0x00400000u;
  return __builtin_bit_cast(float, bits);
}

// Maximum of v over each aligned group of L consecutive lanes (L = 4 or 16);
// every lane of the group gets the result.
template <int L>
__device__ __forceinline__ float group_max(float v) {
#if QRS_Q_DPP
  // quad_perm [1,0,3,2] and [2,3,0,1] combine the lanes of each quad; for 16
  // lanes, row_half_mirror (lane i <-> 7-i) and row_mirror (i <-> 15-i) then
  // pair quads across the half row and the row.
  int b = __builtin_bit_cast(int, v);
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));
  b = __builtin_bit_cast(int, v);
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false)));
  if constexpr (L == 16) {
    b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x141, 0xF, 0xF, false)));
    b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x140, 0xF, 0xF, false)));
  }
  return v;
#else
#pragma unroll
  for (int m = 1; m < L; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
#endif
}

template <int XF, int SL>
__device__ __forceinline__ void quantize_piece(u32x2* __restrict__ codes, void* __restrict__ scales, uint64_t t,
                                               bool active, u32x4 w);

template <int XF, int SL>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const u32x4* __restrict__ in, u32x2* __restrict__ codes,
                                                          void* __restrict__ scales, uint64_t n_lanes) {
  constexpr int P = QRS_Q_PIECES;
  const uint64_t block_first = static_cast<uint64_t>(blockIdx.x) * (kBlock * P);
  // Every lane takes part in the group reductions; pieces past the end hold
  // zeros. n_lanes is a multiple of 16, so a group never straddles the end.
  u32x4 w[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const uint64_t t = block_first + static_cast<uint64_t>(j) * kBlock + threadIdx.x;
    w[j] = u32x4{0u, 0u, 0u, 0u};
    if (t < n_lanes) w[j] = __builtin_nontemporal_load(in + t);
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const uint64_t t = block_first + static_cast<uint64_t>(j) * kBlock + threadIdx.x;
    quantize_piece<XF, SL>(codes, scales, t, t < n_lanes, w[j]);
  }
}

// One 8-element piece: decode the bf16 pair words, combine the group
// maximum, pick the scale, encode, store (codes, and the scale from the
// group's first lane).
template <int XF, int SL>
__device__ __forceinline__ void quantize_piece(u32x2* __restrict__ codes, void* __restrict__ scales, uint64_t t,
                                               bool active, u32x4 w) {
  constexpr int G = SL == kScaleF32Group128 ? 128 : 32;
  constexpr int L = G / kElemsPerLane;  // lanes per group
  float v[kElemsPerLane];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __builtin_bit_cast(float, w[k] << 16);            // element 2k: low half
    v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);  // element 2k+1: high half
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kElemsPerLane; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = group_max<L>(amax);

  float mul;
  float group_scale = 0.0f;
  uint32_t scale_code = 0;
  constexpr float kMax = Fmt<XF>::kMax;
  if constexpr (SL == kScaleF32Group128) {
    constexpr float kMinScale = 0x1p-126f;
    group_scale = amax / kMax;
    const bool small = group_scale < kMinScale;  // includes amax == 0
    mul = small ? 0x1p126f : kMax / amax;
    group_scale = small ? kMinScale : group_scale;
  } else {
    int shared = -127;
    if (amax != 0.0f) {
      int e2;
      (void)frexpf(amax, &e2);  // amax = m * 2^e2, m in [0.5, 1): floor(log2(amax)) = e2 - 1
      shared = min(max(e2 - 1 - Fmt<XF>::kEmax, -127), 127);
    }
    scale_code = static_cast<uint32_t>(shared + 127);
    mul = exp2_int(-shared);  // dividing by the power-of-two scale is this exact product
  }

  float q[kElemsPerLane];
#pragma unroll
  for (int k = 0; k < kElemsPerLane; ++k) q[k] = clampf(v[k] * mul, kMax);
  const u32x2 out = {encode4<XF>(q[0], q[1], q[2], q[3]), encode4<XF>(q[4], q[5], q[6], q[7])};

  if (active) {
    __builtin_nontemporal_store(out, codes + t);
    if ((t & (L - 1)) == 0) {
      if constexpr (SL == kScaleF32Group128) {
        static_cast<float*>(scales)[t / L] = group_scale;
      } else {
        static_cast<uint8_t*>(scales)[t / L] = static_cast<uint8_t>(scale_code);
      }
    }
  }
}

template <int XF, int SL>
hipError_t launch_typed(const void* in, void* codes, void* scales, uint64_t n_elems, hipStream_t stream) {
  const uint64_t n_lanes = n_elems / kElemsPerLane;
  const uint64_t per_block = static_cast<uint64_t>(kBlock) * QRS_Q_PIECES;
  const uint64_t blocks = (n_lanes + per_block - 1) / per_block;
  if (blocks == 0 || blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  return launch_kernel(quantize_kernel<XF, SL>, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), stream,
                       static_cast<const u32x4*>(in), static_cast<u32x2*>(codes), scales, n_lanes);
}

}  // namespace

hipError_t launch_quantize(const QuantizeLaunch& l, hipStream_t stream) {
  if (l.n_elems % 128 != 0) return hipErrorInvalidValue;
  if (l.scale_layout == kScaleE8M0Block32) {
    switch (l.x_format) {
      case kXE4M3FN: return launch_typed<kXE4M3FN, kScaleE8M0Block32>(l.in, l.codes, l.scales, l.n_elems, stream);
      case kXE5M2: return launch_typed<kXE5M2, kScaleE8M0Block32>(l.in, l.codes, l.scales, l.n_elems, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (l.x_format) {
    case kXInt8: return launch_typed<kXInt8, kScaleF32Group128>(l.in, l.codes, l.scales, l.n_elems, stream);
    case kXE4M3FN: return launch_typed<kXE4M3FN, kScaleF32Group128>(l.in, l.codes, l.scales, l.n_elems, stream);
    case kXE5M2: return launch_typed<kXE5M2, kScaleF32Group128>(l.in, l.codes, l.scales, l.n_elems, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qrs
