// gfx950 kernels for one GPU's share of the quantized reduce-scatter.
//
// Page "aclnnQuantReduceScatter", Function description: the output is the
// reduction, over the data of the different ranks, of the exchanged scales
// times the exchanged quantized x. Here the exchange has already happened:
// W rank slices [rows, H] of x codes and their scales sit in HBM, and each
// output element is
//
//   p_r = fp32(decode(x_r) * decode(scale_r))      one rounding
//   acc = p_0, then acc = fp32(acc + p_r) for r = 1 .. W-1, in rank order
//   out = acc (fp32) or round-to-nearest-even(acc) (bf16, fp16)
//
// Modes (same page, Constraints): FP8 E4M3FN / E5M2 x with one E8M0 scale per
// 32 elements (MX), or INT8 / E4M3FN / E5M2 x with one fp32 scale per token
// and 128-column group.
//
// The work is a read-once stream with no reuse, so it is bound by HBM, not by
// arithmetic: no matrix cores. Each lane owns 16 consecutive elements of the
// flat [rows*H] range (a "chunk"). It issues one 16-byte load per rank for
// the codes plus one scale load per rank, decodes with the CDNA4 fp8/bf8
// conversion instructions (two elements per instruction), multiplies and
// adds in separate fp32 instructions (no contraction, so results match the
// definition bit for bit), converts with the packed round-to-nearest-even
// instructions, and writes 16-byte stores. MX modes with fp32 output decode
// and scale in one scaled conversion instead (exact, see product_pair).
// fp32 outputs go through LDS and 16-bit outputs with fp32 group scales
// through a cross-half lane swap, so that each store instruction writes one
// contiguous 1 KiB. MX modes with 16-bit outputs, and with fp32 outputs at
// W = 4 and 8, get the same from lanes that own 8 elements instead (a
// "piece": one 8-byte load per rank, one 16-byte store per 16-bit piece,
// two swapped ones per fp32 piece), in every launch form. Which variant
// each mode uses was chosen by measurement; the macros below select them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <new>

#include "qrs_launch.h"

// The definition has one rounding per product and per sum: never fuse.
#pragma clang fp contract(off)

// Threads per block.
#ifndef QRS_BLOCK
#define QRS_BLOCK 256
#endif
// Chunks of 16 elements per lane.
#ifndef QRS_CHUNKS_PER_LANE
#define QRS_CHUNKS_PER_LANE 1
#endif
// Streaming (non-temporal) hint on the x loads, read exactly once.
#ifndef QRS_NT_LOADS
#define QRS_NT_LOADS 1
#endif
// Streaming hint on the output stores, written exactly once.
#ifndef QRS_NT_STORES
#define QRS_NT_STORES 1
#endif
// Route each wave's output through LDS so that every store instruction of
// the wave writes one contiguous 1 KiB range. A lane's own 16 results are 64
// contiguous bytes in fp32, so without staging each store instruction writes
// 16 bytes every 64, and streaming stores of that shape run at half the
// bandwidth. In bf16 (32 bytes per lane) direct stores measured faster.
// 0: never stage, 1: stage fp32 output only, 2: always stage.
#ifndef QRS_STAGE_STORES
#define QRS_STAGE_STORES 1
#endif
// 16-bit outputs: where to pair each lane's two 16-byte pieces across the
// wave's halves (v_permlane32_swap) so that each store instruction writes
// one contiguous 1 KiB. 0: never; 1: with fp32 group scales only (measured
// faster there, slower in the MX modes); 2: always.
#ifndef QRS_SWAP_STORES
#define QRS_SWAP_STORES 1
#endif
// Block-to-XCD placement: the hardware hands consecutive block ids to the
// 8 XCDs in turn. With 1, block id b is renumbered so that XCD b % 8 walks
// one contiguous eighth of the element range (each XCD's L2 and TLB then
// see 1/8 of the pages). Needs a block count divisible by 8 to apply.
#ifndef QRS_XCD_REMAP
#define QRS_XCD_REMAP 0
#endif
// MX modes: where to decode and scale with the gfx950 scaled fp8 conversions
// (one instruction per two products) instead of decode, then multiply.
// 0: never; 1: fp32 outputs only (measured 0.6-0.7 % faster there, and 1.5-2 %
// slower with 16-bit outputs); 2: always.
#ifndef QRS_MX_SCALED_CVT
#define QRS_MX_SCALED_CVT 1
#endif
// MX scales with 16-bit outputs: lanes own 8-element pieces instead of
// 16-element chunks in the contiguous share, so that each lane's output is
// one 16-byte store and every store instruction of a wave writes one
// contiguous 1 KiB (no partial lines reach HBM). 1: on (measured faster at
// W = 2, 4 and 8 with its own residency cap, below); 0: chunks as above.
#ifndef QRS_MX16_PIECES
#define QRS_MX16_PIECES 1
#endif
// The same for MX scales with an fp32 output, from this world size up
// (0 = never). Each lane's 32 output bytes go out as two 16-byte stores
// after a trade across the half-waves, so each store instruction still
// writes 1 KiB contiguously. Measured against chunks (whole library, one
// box, 4 rounds, medians, outputs identical): at W = 8 the H = 5120 share
// -2.4 %, the H = 8192 share -3.8 %, row-strided -1.8 and -2.8 %, all
// shares -0.9 %; at W = 4 (6 blocks per CU) -1.7 and -0.6 %; at W = 2
// +1.7 % at best (6 blocks per CU).
#ifndef QRS_MX32_PIECES_MIN_WORLD
#define QRS_MX32_PIECES_MIN_WORLD 4
#endif
// The chunk kernel's row-strided blocks, renumbered in pairs per XCD like
// the piece kernel's (1) or in hardware order (0).
#ifndef QRS_ROWS_XCD_PAIRS
#define QRS_ROWS_XCD_PAIRS 0
#endif
// The piece kernel's row-strided form when scale rows do not start on
// 128-byte lines: 1 = each XCD takes runs of consecutive blocks that cover
// whole rows (so every row's scale lines are fetched into one L2); 0 = the
// pairs below.
#ifndef QRS_ROWS_XCD_GROUPS
#define QRS_ROWS_XCD_GROUPS 1
#endif
// The contiguous piece share: reduce_piece_flat_kernel, whose leading
// arguments the hardware preloads (1), or reduce_piece_kernel (0).
#ifndef QRS_PIECE_PRELOAD
#define QRS_PIECE_PRELOAD 1
#endif
// The piece kernel's blocks, renumbered so that the two that share each
// line of scales run on one XCD (see reduce_piece_kernel). 1: on; 0: off.
#ifndef QRS_PIECE_XCD_PAIRS
#define QRS_PIECE_XCD_PAIRS 1
#endif
// 1: block barrier around the LDS exchange; 0: wave-local ordering only.
#ifndef QRS_STAGE_BLOCK_SYNC
#define QRS_STAGE_BLOCK_SYNC 0
#endif
// Contiguous shares of at least three generations of capped blocks: blocks
// resident per CU (0 = no cap). Fewer waves in flight keep the HBM request
// queues shorter; measured faster on every such share shape tried (0.3-8 %),
// and slower on smaller grids, row-strided shares and all-shares launches,
// which stay uncapped. The cap is unused dynamic LDS: the launch device's
// LDS per CU (160 KiB on gfx950) divided among the blocks, with the CU count
// and LDS sizes read from the device.
#ifndef QRS_FLAT_BLOCKS_PER_CU
#define QRS_FLAT_BLOCKS_PER_CU 4
#endif

namespace qrs {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 16;  // elements per chunk: one 16-byte load of codes

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
#if QRS_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
#if QRS_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Decode two adjacent codes of a 32-bit word: bytes 0,1 (hi == false) or
// bytes 2,3 (hi == true). Every code maps exactly to an fp32 value; the fp8
// conversions are the gfx950 OCP E4M3 / E5M2 ones.
template <int XF>
__device__ __forceinline__ f32x2 decode_pair(uint32_t w, bool hi);

template <>
__device__ __forceinline__ f32x2 decode_pair<kXE4M3FN>(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

template <>
__device__ __forceinline__ f32x2 decode_pair<kXE5M2>(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_bf8(w, true) : __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
}

template <>
__device__ __forceinline__ f32x2 decode_pair<kXInt8>(uint32_t w, bool hi) {
  const uint32_t v = hi ? (w >> 16) : w;
  f32x2 r;
  r.x = static_cast<float>(static_cast<int8_t>(v & 0xFFu));
  r.y = static_cast<float>(static_cast<int8_t>((v >> 8) & 0xFFu));
  return r;
}

// E8M0 scale byte -> fp32: 2^(b-127). b = 0 is the fp32 subnormal 2^-127,
// b = 255 is NaN; otherwise the byte is the fp32 exponent field.
__device__ __forceinline__ float decode_e8m0(uint32_t b) {
  uint32_t bits = b << 23;
  bits = (b == 0u) ? 0x00400000u : bits;
  bits = (b == 255u) ? 0x7FC00000u : bits;
  return __builtin_bit_cast(float, bits);
}

// Whether a kernel instantiation uses the scaled conversions (MX scales,
// output type per QRS_MX_SCALED_CVT).
template <int SL, int OF>
constexpr bool kScaledCvt =
    SL == kScaleE8M0Block32 && (QRS_MX_SCALED_CVT == 2 || (QRS_MX_SCALED_CVT == 1 && OF == kOutF32));

// The scale operand of an MX chunk. For the scaled conversions (below) it is
// the E8M0 byte placed in an fp32 exponent field, which is the form those
// instructions read; otherwise the decoded scale.
template <bool SCALED>
__device__ __forceinline__ float mx_scale_operand(uint32_t b) {
  if constexpr (SCALED)
    return __builtin_bit_cast(float, b << 23);
  else
    return decode_e8m0(b);
}

template <int SL, bool SCALED>
__device__ __forceinline__ float load_scale(const void* base, uint64_t chunk) {
  if constexpr (SL == kScaleF32Group128) {
    // 128 elements = 8 chunks share one fp32 scale.
    return static_cast<const float*>(base)[chunk >> 3];
  } else {
    // 32 elements = 2 chunks share one E8M0 byte.
    return mx_scale_operand<SCALED>(static_cast<const uint8_t*>(base)[chunk >> 1]);
  }
}

// Byte offset, within a scale row, of the scale of chunk `chunk` of that row.
template <int SL>
__device__ __forceinline__ uint64_t scale_byte_offset(uint64_t chunk) {
  return SL == kScaleF32Group128 ? (chunk >> 3) * sizeof(float) : (chunk >> 1);
}

template <int SL, bool SCALED>
__device__ __forceinline__ float load_scale_at(const char* p) {
  if constexpr (SL == kScaleF32Group128) {
    return *reinterpret_cast<const float*>(p);
  } else {
    return mx_scale_operand<SCALED>(*reinterpret_cast<const uint8_t*>(p));
  }
}

// The products p = fp32(x * scale) of two adjacent codes of a 32-bit word
// (bytes 0,1 or 2,3) in MX mode (E8M0 scales, fp8 codes): gfx950's scaled
// conversions v_cvt_scalef32_pk_f32_fp8 / _bf8 decode and multiply by
// 2^(E8M0 - 127) in one instruction. An fp8 value times a power of two in
// [2^-127, 2^127] never needs rounding in binary32 (its lowest set bit stays
// at or above 2^-143), so the exact result is the IEEE product; on the
// device these instructions give that product, bit for bit, for every code
// and every E8M0 byte (2^-127 for byte 0, NaN for 255, overflow to
// infinity), which the GPU code-probe tests check.
template <int XF, bool SCALED>
__device__ __forceinline__ f32x2 product_pair(uint32_t w, float s, bool hi) {
  static_assert(SCALED && XF != kXInt8, "scaled conversions: MX scales with fp8 codes only");
  if constexpr (XF == kXE4M3FN)
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, s, true) : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, s, false);
  else
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, s, true) : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, s, false);
}

struct KernelArgs {
  const u32x4* x[kMaxWorld];
  const void* scales[kMaxWorld];
  void* out[kMaxWorld];  // one per share (blockIdx.y)
  // The share is n_rows rows of chunks_per_row chunks. Contiguous shares are
  // one row of all their chunks (row strides unused). Row-strided shares are
  // numbered as one flat range of total_chunks chunks, like contiguous ones;
  // each lane splits its chunk index into (row, column) by multiplication:
  // div_magic = ceil(2^64 / chunks_per_row) for the block's first chunk,
  // div_m20 = ceil(2^20 / chunks_per_row) for the lane's short offset from
  // it (both exact for the ranges the launch admits).
  uint64_t chunks_per_row;
  uint64_t total_chunks;
  uint64_t div_magic;
  uint32_t div_m20;
  uint32_t x_row_stride;      // in 16-byte units
  uint32_t scale_row_stride;  // in bytes
  uint32_t out_row_stride;    // in 16-byte units
  uint64_t x_share_stride;      // in 16-byte units
  uint64_t scale_share_stride;  // in bytes
  // Piece kernels: block ids below this (the grid's full groups of 16, or
  // of 8 * xcd_group) are renumbered in XCD pairs (or runs). Read from the
  // arguments, with the rest of them, rather than from the dispatch packet.
  uint32_t pair_limit;
  // Row-strided piece kernel: when nonzero, each XCD takes runs of
  // xcd_group consecutive blocks instead of pairs; xcd_group_magic =
  // ceil(2^32 / xcd_group) divides by it.
  uint32_t xcd_group;
  uint32_t xcd_group_magic;
};

// Orders a wave's LDS writes before its following LDS reads of other lanes'
// data (LDS instructions of one wave execute in order; this stops the
// compiler from moving the reads above the writes).
__device__ __forceinline__ void stage_sync() {
#if QRS_STAGE_BLOCK_SYNC
  __syncthreads();
#else
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#endif
}

// acc[0..15] = rank-ordered fold of the dequantized products of one chunk.
template <int W, int XF, bool SCALED>
__device__ __forceinline__ void fold_chunk(const u32x4 (&xv)[W], const float (&sv)[W], float (&acc)[kChunk]) {
  if constexpr (SCALED) {
    // Rank 0 starts the fold: acc = p_0.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2 lo = product_pair<XF, true>(xv[0][q], sv[0], false);
      const f32x2 hi = product_pair<XF, true>(xv[0][q], sv[0], true);
      acc[4 * q + 0] = lo.x;
      acc[4 * q + 1] = lo.y;
      acc[4 * q + 2] = hi.x;
      acc[4 * q + 3] = hi.y;
    }
    // Ranks 1..W-1 in order: acc = acc + p_r, each a separate rounding.
#pragma unroll
    for (int r = 1; r < W; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x2 lo = product_pair<XF, true>(xv[r][q], sv[r], false);
        const f32x2 hi = product_pair<XF, true>(xv[r][q], sv[r], true);
        acc[4 * q + 0] = acc[4 * q + 0] + lo.x;
        acc[4 * q + 1] = acc[4 * q + 1] + lo.y;
        acc[4 * q + 2] = acc[4 * q + 2] + hi.x;
        acc[4 * q + 3] = acc[4 * q + 3] + hi.y;
      }
    }
  } else {
    // The same fold with the decode and the rounded multiply written out.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = xv[0][q];
      const f32x2 lo = decode_pair<XF>(w, false);
      const f32x2 hi = decode_pair<XF>(w, true);
      acc[4 * q + 0] = lo.x * sv[0];
      acc[4 * q + 1] = lo.y * sv[0];
      acc[4 * q + 2] = hi.x * sv[0];
      acc[4 * q + 3] = hi.y * sv[0];
    }
#pragma unroll
    for (int r = 1; r < W; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = xv[r][q];
        const f32x2 lo = decode_pair<XF>(w, false);
        const f32x2 hi = decode_pair<XF>(w, true);
        const float p0 = lo.x * sv[r];
        const float p1 = lo.y * sv[r];
        const float p2 = hi.x * sv[r];
        const float p3 = hi.y * sv[r];
        acc[4 * q + 0] = acc[4 * q + 0] + p0;
        acc[4 * q + 1] = acc[4 * q + 1] + p1;
        acc[4 * q + 2] = acc[4 * q + 2] + p2;
        acc[4 * q + 3] = acc[4 * q + 3] + p3;
      }
    }
  }
}

// The chunk's output as 16-byte pieces: 4 for fp32, 2 for bf16 and fp16.
template <int OF>
struct OutPieces {
  static constexpr int kCount = OF == kOutF32 ? 4 : 2;
};

template <int OF>
__device__ __forceinline__ void pack_chunk(const float (&acc)[kChunk], u32x4 (&piece)[OutPieces<OF>::kCount]) {
  if constexpr (OF == kOutF32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      piece[q] = u32x4{__builtin_bit_cast(uint32_t, acc[4 * q + 0]), __builtin_bit_cast(uint32_t, acc[4 * q + 1]),
                       __builtin_bit_cast(uint32_t, acc[4 * q + 2]), __builtin_bit_cast(uint32_t, acc[4 * q + 3])};
    }
  } else {
    uint32_t packed[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f32x2 pr;
      pr.x = acc[2 * k];
      pr.y = acc[2 * k + 1];
      if constexpr (OF == kOutBF16) {
        // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN.
        packed[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
      } else {
        // v_cvt_pk_f16_f32: round to nearest even, overflow to infinity.
        packed[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2));
      }
    }
    piece[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    piece[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
  }
}

// Use every argument the contiguous kernels read (no instruction is
// emitted), so that their scalar loads issue together at the start of a
// wave and it waits once for them, instead of once for the bounds and
// again, after the bounds check, for the base pointers. Measured about 1 %
// faster on the W=8 H=8192 piece kernel, whose waves are short-lived, and
// about 0.35 % on the W=8 H=5120 share in 16-element chunks (the contiguous
// piece share now preloads its leading arguments instead; see
// reduce_piece_flat_kernel). One asm statement per group:
// separate statements let the scheduler put a wait between them.
template <int W>
__device__ __forceinline__ void pin_flat_args(const KernelArgs& a, uint64_t n, uint32_t m);
template <>
__device__ __forceinline__ void pin_flat_args<8>(const KernelArgs& a, uint64_t n, uint32_t m) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.x[4]), "s"(a.x[5]), "s"(a.x[6]),
               "s"(a.x[7]));
  asm volatile("" ::"s"(a.scales[0]), "s"(a.scales[1]), "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.scales[4]),
               "s"(a.scales[5]), "s"(a.scales[6]), "s"(a.scales[7]), "s"(a.out[0]), "s"(n), "s"(m));
}
template <>
__device__ __forceinline__ void pin_flat_args<4>(const KernelArgs& a, uint64_t n, uint32_t m) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.scales[0]), "s"(a.scales[1]),
               "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.out[0]), "s"(n), "s"(m));
}
template <>
__device__ __forceinline__ void pin_flat_args<2>(const KernelArgs& a, uint64_t n, uint32_t m) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.scales[0]), "s"(a.scales[1]), "s"(a.out[0]), "s"(n), "s"(m));
}

// The same for the piece kernel's row-strided form (row split and strides
// too; -1.7 % on the W=8 H=8192 strided share) and all-shares form (share
// strides; -0.4 % on the W=8 H=8192 group).
template <int W>
__device__ __forceinline__ void pin_rows_args(const KernelArgs& a);
template <>
__device__ __forceinline__ void pin_rows_args<8>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.x[4]), "s"(a.x[5]), "s"(a.x[6]),
               "s"(a.x[7]), "s"(a.out[0]), "s"(a.total_chunks), "s"(a.pair_limit), "s"(a.chunks_per_row),
               "s"(a.div_magic));
  asm volatile("" ::"s"(a.scales[0]), "s"(a.scales[1]), "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.scales[4]),
               "s"(a.scales[5]), "s"(a.scales[6]), "s"(a.scales[7]), "s"(a.x_row_stride), "s"(a.scale_row_stride),
               "s"(a.out_row_stride), "s"(a.xcd_group), "s"(a.xcd_group_magic));
}
template <>
__device__ __forceinline__ void pin_rows_args<4>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.scales[0]), "s"(a.scales[1]),
               "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.out[0]), "s"(a.total_chunks), "s"(a.pair_limit),
               "s"(a.chunks_per_row), "s"(a.div_magic), "s"(a.x_row_stride), "s"(a.scale_row_stride),
               "s"(a.out_row_stride), "s"(a.xcd_group), "s"(a.xcd_group_magic));
}
template <>
__device__ __forceinline__ void pin_rows_args<2>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.scales[0]), "s"(a.scales[1]), "s"(a.out[0]),
               "s"(a.total_chunks), "s"(a.pair_limit), "s"(a.chunks_per_row), "s"(a.div_magic), "s"(a.x_row_stride),
               "s"(a.scale_row_stride), "s"(a.out_row_stride), "s"(a.xcd_group), "s"(a.xcd_group_magic));
}
template <int W>
__device__ __forceinline__ void pin_shares_args(const KernelArgs& a);
template <>
__device__ __forceinline__ void pin_shares_args<8>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.x[4]), "s"(a.x[5]), "s"(a.x[6]),
               "s"(a.x[7]), "s"(a.total_chunks), "s"(a.pair_limit), "s"(a.x_share_stride), "s"(a.scale_share_stride));
  asm volatile("" ::"s"(a.scales[0]), "s"(a.scales[1]), "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.scales[4]),
               "s"(a.scales[5]), "s"(a.scales[6]), "s"(a.scales[7]));
}
template <>
__device__ __forceinline__ void pin_shares_args<4>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.x[2]), "s"(a.x[3]), "s"(a.scales[0]), "s"(a.scales[1]),
               "s"(a.scales[2]), "s"(a.scales[3]), "s"(a.total_chunks), "s"(a.pair_limit), "s"(a.x_share_stride),
               "s"(a.scale_share_stride));
}
template <>
__device__ __forceinline__ void pin_shares_args<2>(const KernelArgs& a) {
  asm volatile("" ::"s"(a.x[0]), "s"(a.x[1]), "s"(a.scales[0]), "s"(a.scales[1]), "s"(a.total_chunks),
               "s"(a.pair_limit), "s"(a.x_share_stride), "s"(a.scale_share_stride));
}

// Addressing of a launch: one contiguous share (no per-block offset
// arithmetic: the hot path), one share with row-strided slices and output,
// or all W shares of contiguous pre-all-to-all inputs (blockIdx.y = share).
// kAddrFlat32 is the contiguous share when every slice, scale slice and the
// output span less than 4 GiB: each lane then forms one 32-bit byte offset
// per tensor kind and every load and store takes the rank's base address
// from scalar registers (fewer vector instructions and registers).
enum Addr : int { kAddrFlat = 0, kAddrRows = 1, kAddrShares = 2, kAddrFlat32 = 3 };

template <int W, int XF, int SL, int OF, int ADDR>
__global__ __launch_bounds__(QRS_BLOCK) void reduce_kernel(KernelArgs a) {
  constexpr bool ROWS = ADDR == kAddrRows;
  constexpr bool SHARES = ADDR == kAddrShares;
  constexpr bool OFF32 = ADDR == kAddrFlat32;
  constexpr bool SCALED = kScaledCvt<SL, OF>;
  constexpr bool kStage = QRS_STAGE_STORES == 2 || (QRS_STAGE_STORES == 1 && OF == kOutF32);
  // Swapped stores need the whole wave active up to the stores: lanes past
  // the end then load the last chunk again and store nothing.
  constexpr bool kSwap = (QRS_SWAP_STORES == 2 || (QRS_SWAP_STORES == 1 && SL == kScaleF32Group128)) &&
                         !kStage && !ROWS && OutPieces<OF>::kCount == 2;
  constexpr int CH = QRS_CHUNKS_PER_LANE;
  constexpr int P = OutPieces<OF>::kCount;
  static_assert(!ROWS || CH <= 2, "row split assumes a lane's offset from its block's first chunk < 1024");
  if constexpr (OFF32) pin_flat_args<W>(a, a.chunks_per_row, 0u);
  uint32_t block_id = blockIdx.x;
#if QRS_XCD_REMAP
  if ((gridDim.x & 7u) == 0) block_id = (block_id & 7u) * (gridDim.x >> 3) + (block_id >> 3);
#endif
#if QRS_ROWS_XCD_PAIRS
  // Row-strided shares: scale rows need not start on a line, so consecutive
  // blocks can share one; pair them on one XCD as the piece kernel does.
  if constexpr (ROWS) {
    if (block_id < (gridDim.x & ~15u)) block_id = (block_id & ~15u) | ((block_id & 7u) << 1) | ((block_id >> 3) & 1u);
  }
#endif
  // First chunk of this block (uniform). Chunk j of this lane is
  // base + j*QRS_BLOCK: every load instruction of a wave covers one
  // contiguous range of chunks (for row-strided shares, one contiguous range
  // per row it touches).
  const uint64_t block_first = static_cast<uint64_t>(block_id) * (QRS_BLOCK * CH);
  const uint64_t base = block_first + threadIdx.x;
  const uint64_t n_chunks = ROWS ? a.total_chunks : a.chunks_per_row;
  // Row-strided shares: the row and column of the block's first chunk.
  [[maybe_unused]] const uint64_t cpr = a.chunks_per_row;
  [[maybe_unused]] const uint32_t row_b = ROWS ? static_cast<uint32_t>(__umul64hi(block_first, a.div_magic)) : 0u;
  [[maybe_unused]] const uint32_t col_b = ROWS ? static_cast<uint32_t>(block_first - row_b * cpr) : 0u;
  // Share handled by this block (one share unless the all-to-all is
  // emulated on this GPU): uniform offsets into every rank's input.
  const uint32_t share = SHARES ? blockIdx.y : 0u;
  const uint64_t x_off = SHARES ? share * a.x_share_stride : 0;
  const uint64_t s_off = SHARES ? share * a.scale_share_stride : 0;

  // Row-strided shares: chunk base + j*QRS_BLOCK sits at (row_b + dr,
  // col[j]); col[j] is the chunk's index within its row.
  [[maybe_unused]] uint32_t row_of[CH];
  [[maybe_unused]] uint32_t col_of[CH];
  u32x4 xv[CH][W];
  float sv[CH][W];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint64_t c_lane = base + static_cast<uint64_t>(j) * QRS_BLOCK;
    const uint64_t c = (kSwap && c_lane >= n_chunks) ? n_chunks - 1 : c_lane;
    if constexpr (ROWS) {
      const uint32_t t = col_b + threadIdx.x + j * QRS_BLOCK;
      const uint32_t dr = (t * a.div_m20) >> 20;
      row_of[j] = row_b + dr;
      col_of[j] = t - dr * static_cast<uint32_t>(cpr);
    }
    if (kSwap || c < n_chunks) {
      if constexpr (ROWS) {
        // One byte offset per lane for all ranks' codes and one for their
        // scales: a single 64-bit add per load.
        const uint64_t xb = (static_cast<uint64_t>(row_of[j]) * a.x_row_stride + col_of[j]) * sizeof(u32x4);
        // A scale slice spans less than 4 GiB (checked at launch): a 32-bit
        // offset, which also keeps the compiler from redoing the row product
        // for every rank.
        const uint32_t sb = row_of[j] * a.scale_row_stride + static_cast<uint32_t>(scale_byte_offset<SL>(col_of[j]));
#pragma unroll
        for (int r = 0; r < W; ++r)
          xv[j][r] = load_stream(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.x[r]) + xb));
#pragma unroll
        for (int r = 0; r < W; ++r) sv[j][r] = load_scale_at<SL, SCALED>(static_cast<const char*>(a.scales[r]) + sb);
      } else if constexpr (OFF32) {
        const uint32_t xb = static_cast<uint32_t>(c) * static_cast<uint32_t>(sizeof(u32x4));
        const uint32_t sb = static_cast<uint32_t>(scale_byte_offset<SL>(c));
#pragma unroll
        for (int r = 0; r < W; ++r)
          xv[j][r] = load_stream(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.x[r]) + xb));
#pragma unroll
        for (int r = 0; r < W; ++r) sv[j][r] = load_scale_at<SL, SCALED>(static_cast<const char*>(a.scales[r]) + sb);
      } else {
#pragma unroll
        for (int r = 0; r < W; ++r) xv[j][r] = load_stream(a.x[r] + x_off + c);
#pragma unroll
        for (int r = 0; r < W; ++r) sv[j][r] = load_scale<SL, SCALED>(static_cast<const char*>(a.scales[r]) + s_off, c);
      }
    }
  }

  u32x4* const out = static_cast<u32x4*>(a.out[share]);
  __shared__ u32x4 stage[kStage ? QRS_BLOCK * P : 1];
  [[maybe_unused]] const int lane = threadIdx.x & 63;
  [[maybe_unused]] u32x4* const wave_stage = stage + (kStage ? (threadIdx.x & ~63) * P : 0);

#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const uint64_t c = base + static_cast<uint64_t>(j) * QRS_BLOCK;
    u32x4 piece[P];
    if constexpr (kSwap) {
      float acc[kChunk];
      fold_chunk<W, XF, SCALED>(xv[j], sv[j], acc);
      pack_chunk<OF>(acc, piece);
    }
    if (!kSwap && c < n_chunks) {
      float acc[kChunk];
      fold_chunk<W, XF, SCALED>(xv[j], sv[j], acc);
      pack_chunk<OF>(acc, piece);
      if constexpr (!kStage) {
        const uint64_t oc = ROWS ? static_cast<uint64_t>(row_of[j]) * a.out_row_stride + col_of[j] * P : c * P;
#pragma unroll
        for (int q = 0; q < P; ++q) {
          if constexpr (OFF32)
            store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) +
                                                  static_cast<uint32_t>(oc + q) * static_cast<uint32_t>(sizeof(u32x4))),
                         piece[q]);
          else
            store_stream(out + oc + q, piece[q]);
        }
      }
    }
    if constexpr (kSwap) {
      // Lane l holds pieces 2l and 2l+1 of the wave's 128 (its chunk's two
      // halves). Swap the lower half-wave's second pieces with the upper
      // half-wave's first pieces: lane l < 32 then holds pieces 2l and
      // 2l+64, lane l >= 32 pieces 2l-63 and 2l+1, so the first store writes
      // pieces 0..63 and the second 64..127, each one contiguous 1 KiB.
      u32x4 lo = piece[0], hi = piece[1];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
        lo[d] = r[0];
        hi[d] = r[1];
      }
      const uint32_t lane_id = threadIdx.x & 63u;
      const uint64_t wave_first_chunk = block_first + static_cast<uint64_t>(j) * QRS_BLOCK + (threadIdx.x & ~63u);
      const uint32_t p_lo = lane_id < 32u ? 2u * lane_id : 2u * lane_id - 63u;
      const uint32_t p_hi = lane_id < 32u ? 2u * lane_id + 64u : 2u * lane_id + 1u;
      // Piece p belongs to chunk wave_first_chunk + p / 2.
      if (wave_first_chunk + p_lo / 2u < n_chunks) {
        if constexpr (OFF32)
          store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) +
                                                static_cast<uint32_t>(wave_first_chunk * 2 + p_lo) * 16u),
                       lo);
        else
          store_stream(out + wave_first_chunk * 2 + p_lo, lo);
      }
      if (wave_first_chunk + p_hi / 2u < n_chunks) {
        if constexpr (OFF32)
          store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) +
                                                static_cast<uint32_t>(wave_first_chunk * 2 + p_hi) * 16u),
                       hi);
        else
          store_stream(out + wave_first_chunk * 2 + p_hi, hi);
      }
    }
    if constexpr (kStage) {
      // The wave's 64 chunks are contiguous in the output row: write them to
      // LDS in output order, then let lane l store pieces l, l+64, ... of
      // that range, so each store instruction covers 64 consecutive pieces.
      if (j > 0) stage_sync();  // the previous round's reads are done
      if (c < n_chunks) {
#pragma unroll
        for (int q = 0; q < P; ++q) wave_stage[lane * P + q] = piece[q];
      }
      stage_sync();
      const uint64_t wave_first_chunk = block_first + static_cast<uint64_t>(j) * QRS_BLOCK + (threadIdx.x & ~63);
      u32x4 staged[P];
#pragma unroll
      for (int q = 0; q < P; ++q) staged[q] = wave_stage[q * 64 + lane];
      // Row-strided shares: row and column of the wave's first chunk; a
      // chunk d < 64 further on is at most one row later (a row has at
      // least 64 chunks).
      [[maybe_unused]] uint32_t wrow = 0;
      [[maybe_unused]] uint32_t wcol = 0;
      if constexpr (ROWS) {
        const uint32_t t = col_b + (threadIdx.x & ~63) + j * QRS_BLOCK;
        const uint32_t dr = (t * a.div_m20) >> 20;
        wrow = row_b + dr;
        wcol = t - dr * static_cast<uint32_t>(cpr);
      }
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int k = q * 64 + lane;  // piece k of the wave's range belongs to chunk k / P
        if (wave_first_chunk + k / P < n_chunks) {
          if constexpr (ROWS) {
            uint32_t col = wcol + k / P;
            const bool next = col >= static_cast<uint32_t>(cpr);
            col = next ? col - static_cast<uint32_t>(cpr) : col;
            const uint32_t orow = wrow + (next ? 1u : 0u);
            store_stream(out + static_cast<uint64_t>(orow) * a.out_row_stride + col * P + k % P, staged[q]);
          } else if constexpr (OFF32) {
            const uint32_t ob = static_cast<uint32_t>(wave_first_chunk * P + k) * static_cast<uint32_t>(sizeof(u32x4));
            store_stream(reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) + ob), staged[q]);
          } else {
            store_stream(out + wave_first_chunk * P + k, staged[q]);
          }
        }
      }
    }
  }
}

// acc[0..7] = rank-ordered fold of the dequantized products of one
// 8-element piece (decode, then one rounded multiply and one rounded add per
// rank, as in fold_chunk; with SCALED, each product one scaled conversion).
template <int W, int XF, bool SCALED>
__device__ __forceinline__ void fold_piece(const u32x2 (&xv)[W], const float (&sv)[W], float (&acc)[8]) {
  if constexpr (SCALED) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x2 lo = product_pair<XF, true>(xv[0][q], sv[0], false);
      const f32x2 hi = product_pair<XF, true>(xv[0][q], sv[0], true);
      acc[4 * q + 0] = lo.x;
      acc[4 * q + 1] = lo.y;
      acc[4 * q + 2] = hi.x;
      acc[4 * q + 3] = hi.y;
    }
#pragma unroll
    for (int r = 1; r < W; ++r) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x2 lo = product_pair<XF, true>(xv[r][q], sv[r], false);
        const f32x2 hi = product_pair<XF, true>(xv[r][q], sv[r], true);
        acc[4 * q + 0] = acc[4 * q + 0] + lo.x;
        acc[4 * q + 1] = acc[4 * q + 1] + lo.y;
        acc[4 * q + 2] = acc[4 * q + 2] + hi.x;
        acc[4 * q + 3] = acc[4 * q + 3] + hi.y;
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t w = xv[0][q];
    const f32x2 lo = decode_pair<XF>(w, false);
    const f32x2 hi = decode_pair<XF>(w, true);
    acc[4 * q + 0] = lo.x * sv[0];
    acc[4 * q + 1] = lo.y * sv[0];
    acc[4 * q + 2] = hi.x * sv[0];
    acc[4 * q + 3] = hi.y * sv[0];
  }
#pragma unroll
  for (int r = 1; r < W; ++r) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w = xv[r][q];
      const f32x2 lo = decode_pair<XF>(w, false);
      const f32x2 hi = decode_pair<XF>(w, true);
      const float p0 = lo.x * sv[r];
      const float p1 = lo.y * sv[r];
      const float p2 = hi.x * sv[r];
      const float p3 = hi.y * sv[r];
      acc[4 * q + 0] = acc[4 * q + 0] + p0;
      acc[4 * q + 1] = acc[4 * q + 1] + p1;
      acc[4 * q + 2] = acc[4 * q + 2] + p2;
      acc[4 * q + 3] = acc[4 * q + 3] + p3;
    }
  }
}

// Writes 16-byte unit u (of 128) of the fp32 output of the wave whose first
// piece is wave_first: unit u holds elements [4u, 4u + 4) of the wave's
// 512, half (u & 1) of piece wave_first + u / 2. Nothing past the share.
template <int ADDR>
__device__ __forceinline__ void store_piece_unit(const KernelArgs& a, uint64_t wave_first, uint32_t u,
                                                 uint64_t n_pieces, const u32x4& v) {
  const uint64_t q = wave_first + (u >> 1);
  if (q >= n_pieces) return;
  if constexpr (ADDR == kAddrFlat32) {
    store_stream(reinterpret_cast<u32x4*>(static_cast<char*>(a.out[0]) +
                                          (static_cast<uint32_t>(wave_first) * 2u + u) * 16u),
                 v);
  } else if constexpr (ADDR == kAddrShares) {
    store_stream(static_cast<u32x4*>(a.out[blockIdx.y]) + wave_first * 2 + u, v);
  } else {
    const uint64_t ppr = a.chunks_per_row * 2;
    const uint64_t row = __umul64hi(q, a.div_magic);
    const uint64_t col = q - row * ppr;
    store_stream(static_cast<u32x4*>(a.out[0]) + row * a.out_row_stride + col * 2 + (u & 1u), v);
  }
}

// Converts and stores one lane's folded piece. A 16-bit output is one
// 16-byte store at dst. An fp32 output is two 16-byte units: lane l holds
// units 2l and 2l + 1 of the wave's 128. Trading the lower half-wave's
// second units for the upper half-wave's first leaves lane l < 32 with
// units 2l and 2l + 64 and lane l >= 32 with units 2l - 63 and 2l + 1: the
// first store writes units 0..63, the second 64..127 (store_piece_unit).
template <int OF, int ADDR>
__device__ __forceinline__ void store_piece(const KernelArgs& a, const float (&acc)[8], u32x4* dst,
                                            uint64_t wave_first, uint64_t n_pieces) {
  if constexpr (OF == kOutF32) {
    u32x4 lo, hi;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, acc[d]),
                                                      __builtin_bit_cast(uint32_t, acc[4 + d]), false, false);
      lo[d] = r[0];
      hi[d] = r[1];
    }
    const uint32_t lane = threadIdx.x & 63u;
    store_piece_unit<ADDR>(a, wave_first, lane < 32u ? 2u * lane : 2u * lane - 63u, n_pieces, lo);
    store_piece_unit<ADDR>(a, wave_first, lane < 32u ? 2u * lane + 64u : 2u * lane + 1u, n_pieces, hi);
  } else {
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f32x2 pr;
      pr.x = acc[2 * k];
      pr.y = acc[2 * k + 1];
      if constexpr (OF == kOutBF16)
        packed[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));  // RNE
      else
        packed[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2));  // RNE
    }
    store_stream(dst, u32x4{packed[0], packed[1], packed[2], packed[3]});
  }
}

// Shares with MX scales: lane l of block b owns piece p = b * QRS_BLOCK + l
// of the share, elements [8p, 8p + 8). It loads 8 code bytes per rank (one
// 8-byte load; a wave's load covers 512 contiguous bytes of a row) and the
// piece's E8M0 byte (element 8p's block of 32), and folds. A 16-bit output
// is converted and written with one 16-byte store, so a wave's store covers
// 1 KiB of a row contiguously. An fp32 output is two 16-byte units per lane;
// the two halves of the wave trade units first, so that each of the wave's
// two stores covers 1 KiB contiguously as well. Addressing:
//   kAddrFlat32  one contiguous share, every slice, scale slice and the
//                output under 4 GiB (32-bit offsets on the scalar bases);
//   kAddrShares  all W shares of contiguous pre-all-to-all inputs: share
//                j = blockIdx.y reads row block j of every rank (64-bit
//                offsets) and writes out[j];
//   kAddrRows    one share with row-strided slices and output: piece p is
//                column p mod (H / 8) of row p div (H / 8), the division a
//                multiply by div_magic = ceil(2^64 / (H / 8)).
template <int W, int XF, int OF, int ADDR>
__global__ __launch_bounds__(QRS_BLOCK) void reduce_piece_kernel(KernelArgs a) {
  static_assert(XF != kXInt8, "MX scales with fp8 codes");
  constexpr bool F32 = OF == kOutF32;
  constexpr bool SCALED = kScaledCvt<kScaleE8M0Block32, OF>;
  static_assert(ADDR == kAddrFlat32 || ADDR == kAddrShares || ADDR == kAddrRows, "addressing");
  if constexpr (ADDR == kAddrFlat32) pin_flat_args<W>(a, a.total_chunks, a.pair_limit);
  if constexpr (ADDR == kAddrRows) pin_rows_args<W>(a);
  if constexpr (ADDR == kAddrShares) pin_shares_args<W>(a);
  const uint64_t n_pieces = a.total_chunks * 2;
  uint32_t b = blockIdx.x;
#if QRS_PIECE_XCD_PAIRS
  // A block covers 64 E8M0 bytes per rank, half a 128-byte line, so two
  // consecutive blocks share every scale line. The hardware hands block ids
  // to the XCDs in turn (linear id mod 8), so ids b and b + 8 run on one
  // XCD: within each full group of 16 ids (below pair_limit), id
  // 16g + 8h + x takes the pieces of block 16g + 2x + h, and each scale
  // line is fetched into one L2.
  if constexpr (ADDR == kAddrRows) {
    if (b < a.pair_limit) {
      if (a.xcd_group != 0) {
        // Runs: XCD x's k-th block (b = 8k + x) takes block
        // ((k div G) * 8 + x) * G + k mod G, G = xcd_group, so each XCD
        // walks G consecutive blocks at a time; G * 256 pieces cover whole
        // rows, so no scale row is split between two XCDs' runs.
        const uint32_t k = b >> 3;
        const uint32_t q = __umulhi(k, a.xcd_group_magic);
        b = ((q << 3) + (b & 7u)) * a.xcd_group + (k - q * a.xcd_group);
      } else {
        b = (b & ~15u) | ((b & 7u) << 1) | ((b >> 3) & 1u);
      }
    }
  } else if (b < a.pair_limit) {
    b = (b & ~15u) | ((b & 7u) << 1) | ((b >> 3) & 1u);
  }
#endif
  uint64_t p = static_cast<uint64_t>(b) * QRS_BLOCK + threadIdx.x;
  [[maybe_unused]] uint64_t wave_first = 0;
  if constexpr (F32) {
    // The trade of output units needs the whole wave: lanes past the end
    // load the last piece again and store nothing.
    wave_first = static_cast<uint64_t>(b) * QRS_BLOCK + (threadIdx.x & ~63u);
    if (wave_first >= n_pieces) return;
    p = p < n_pieces ? p : n_pieces - 1;
  } else {
    if (p >= n_pieces) return;
  }
  u32x2 xv[W];
  float sv[W];
  [[maybe_unused]] u32x4* dst = nullptr;
  if constexpr (ADDR == kAddrFlat32) {
    // 32-bit offsets on the scalar bases for the codes and the scale bytes.
    const uint32_t p32 = static_cast<uint32_t>(p);
    const uint32_t xb = p32 * 8u;
    const uint32_t sb = p32 >> 2;
#pragma unroll
    for (int r = 0; r < W; ++r)
      xv[r] = load_stream(reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(a.x[r]) + xb));
#pragma unroll
    for (int r = 0; r < W; ++r) sv[r] = mx_scale_operand<SCALED>(*(static_cast<const uint8_t*>(a.scales[r]) + sb));
    if constexpr (!F32) dst = reinterpret_cast<u32x4*>(static_cast<char*>(a.out[0]) + p32 * 16u);
  } else if constexpr (ADDR == kAddrShares) {
    const uint32_t share = blockIdx.y;
    const uint64_t xb = share * a.x_share_stride * sizeof(u32x4) + p * 8u;
    const uint64_t sb = share * a.scale_share_stride + (p >> 2);
#pragma unroll
    for (int r = 0; r < W; ++r)
      xv[r] = load_stream(reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(a.x[r]) + xb));
#pragma unroll
    for (int r = 0; r < W; ++r) sv[r] = mx_scale_operand<SCALED>(*(static_cast<const uint8_t*>(a.scales[r]) + sb));
    if constexpr (!F32) dst = static_cast<u32x4*>(a.out[share]) + p;
  } else {
    const uint64_t ppr = a.chunks_per_row * 2;  // pieces per row
    const uint64_t row = __umul64hi(p, a.div_magic);
    const uint32_t col = static_cast<uint32_t>(p - row * ppr);
    const uint64_t xb = row * a.x_row_stride * sizeof(u32x4) + col * 8u;
    // A scale slice spans less than 4 GiB (checked at launch).
    const uint32_t sb = static_cast<uint32_t>(row) * a.scale_row_stride + (col >> 2);
#pragma unroll
    for (int r = 0; r < W; ++r)
      xv[r] = load_stream(reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(a.x[r]) + xb));
#pragma unroll
    for (int r = 0; r < W; ++r) sv[r] = mx_scale_operand<SCALED>(*(static_cast<const uint8_t*>(a.scales[r]) + sb));
    if constexpr (!F32) dst = static_cast<u32x4*>(a.out[0]) + row * a.out_row_stride + col;
  }
  float acc[8];
  fold_piece<W, XF, SCALED>(xv, sv, acc);
  store_piece<OF, ADDR>(a, acc, dst, wave_first, n_pieces);
}

// The contiguous form of reduce_piece_kernel (kAddrFlat32) with its hottest
// arguments first: the piece count, the pairing bound and the W code bases
// lead the argument list, ahead of the rest in KernelArgs (whose x[] it does
// not read). The hardware preloads the first 14 dwords of a kernel's
// arguments into SGPRs when the compiler is asked to
// (-amdgpu-kernarg-preload-count), so a wave has n, the bound and x0..x5
// when it starts: it issues those ranks' code loads at once, and makes its
// one scalar round trip (x6, x7, the scale bases, the output) while they are
// in flight. Piece indices and byte offsets fit 32 bits: the output, the
// largest of the share's tensors, spans less than 4 GiB.
template <int W, int XF, int OF>
__global__ __launch_bounds__(QRS_BLOCK) void reduce_piece_flat_kernel(uint32_t n_pieces, uint32_t pair_limit,
                                                                     const u32x2* x0, const u32x2* x1,
                                                                     const u32x2* x2, const u32x2* x3,
                                                                     const u32x2* x4, const u32x2* x5,
                                                                     const u32x2* x6, const u32x2* x7, KernelArgs a) {
  static_assert(XF != kXInt8, "MX scales with fp8 codes");
  constexpr bool F32 = OF == kOutF32;
  constexpr bool SCALED = kScaledCvt<kScaleE8M0Block32, OF>;
  const u32x2* const xs[8] = {x0, x1, x2, x3, x4, x5, x6, x7};
  uint32_t b = blockIdx.x;
#if QRS_PIECE_XCD_PAIRS
  // Pairs per XCD, as in reduce_piece_kernel.
  if (b < pair_limit) b = (b & ~15u) | ((b & 7u) << 1) | ((b >> 3) & 1u);
#endif
  uint32_t p = b * QRS_BLOCK + threadIdx.x;
  [[maybe_unused]] uint32_t wave_first = 0;
  if constexpr (F32) {
    // The trade of output units needs the whole wave: lanes past the end
    // load the last piece again and store nothing.
    wave_first = b * QRS_BLOCK + (threadIdx.x & ~63u);
    if (wave_first >= n_pieces) return;
    p = p < n_pieces ? p : n_pieces - 1;
  } else {
    if (p >= n_pieces) return;
  }
  u32x2 xv[W];
  float sv[W];
  // The preloaded ranks' code loads first, kept ahead of everything that
  // waits for the scalar round trip (scheduling barriers: no instruction
  // moves across them).
  constexpr int kPre = W < 6 ? W : 6;
#pragma unroll
  for (int r = 0; r < kPre; ++r)
    xv[r] = load_stream(reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(xs[r]) + p * 8u));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = kPre; r < W; ++r)
    xv[r] = load_stream(reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(xs[r]) + p * 8u));
  uint32_t sb[W];
#pragma unroll
  for (int r = 0; r < W; ++r) sb[r] = *(static_cast<const uint8_t*>(a.scales[r]) + (p >> 2));
  // Every load issued before the first wait for data.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < W; ++r) sv[r] = mx_scale_operand<SCALED>(sb[r]);
  [[maybe_unused]] u32x4* dst = nullptr;
  if constexpr (!F32) dst = reinterpret_cast<u32x4*>(static_cast<char*>(a.out[0]) + p * 16u);
  float acc[8];
  fold_piece<W, XF, SCALED>(xv, sv, acc);
  store_piece<OF, kAddrFlat32>(a, acc, dst, wave_first, n_pieces);
}

// Whether a kernel instantiation takes the piece layout.
template <int W, int SL, int OF>
constexpr bool kPieceLayout =
    SL == kScaleE8M0Block32 &&
    (OF == kOutF32 ? (QRS_MX32_PIECES_MIN_WORLD > 0 && W >= QRS_MX32_PIECES_MIN_WORLD) : QRS_MX16_PIECES);

// Blocks resident per CU for the all-shares piece launch (0 = no cap), by
// world size. At W = 8 four (one box, 4 rounds, medians, against no cap:
// the H = 8192 MX group -1.3 % with bf16 out and -3.0 % with fp32 out; 5
// the same, 6 -0.1 / -2.2 %, 8 no change); at W = 4 none (4 to 6 blocks
// +4 to +16 %).
#ifndef QRS_PIECE_SHARES_BLOCKS_PER_CU_W8
#define QRS_PIECE_SHARES_BLOCKS_PER_CU_W8 4
#endif
#ifndef QRS_PIECE_SHARES_BLOCKS_PER_CU_W4
#define QRS_PIECE_SHARES_BLOCKS_PER_CU_W4 0
#endif
#ifndef QRS_PIECE_SHARES_BLOCKS_PER_CU_W2
#define QRS_PIECE_SHARES_BLOCKS_PER_CU_W2 0
#endif
template <int W>
constexpr uint32_t kPieceSharesBlocksPerCu =
    W >= 8 ? QRS_PIECE_SHARES_BLOCKS_PER_CU_W8
           : (W >= 4 ? QRS_PIECE_SHARES_BLOCKS_PER_CU_W4 : QRS_PIECE_SHARES_BLOCKS_PER_CU_W2);
// Blocks resident per CU for the piece kernel with a 16-bit output (0 = no
// cap), by world size.
// A lane keeps W 8-byte loads in flight: at W = 8 six blocks per CU
// measured best (W=8 shares with H = 8192 and 5120; 4 and 5 slower), at
// W = 2 and 4 full occupancy (capped at 4 or 6 blocks they ran 0-16 %
// slower).
#ifndef QRS_PIECE_BLOCKS_PER_CU_W8
#define QRS_PIECE_BLOCKS_PER_CU_W8 6
#endif
#ifndef QRS_PIECE_BLOCKS_PER_CU_W4
#define QRS_PIECE_BLOCKS_PER_CU_W4 0
#endif
#ifndef QRS_PIECE_BLOCKS_PER_CU_W2
#define QRS_PIECE_BLOCKS_PER_CU_W2 0
#endif
// With an fp32 output a lane also keeps 32 output bytes, and at W = 8 four
// blocks per CU measured best (5 the same within noise; 6 +1.5 %, 8 and
// no cap +3.3 % on the H = 5120 share); at W = 4 six (4 and 8 slower
// than chunks).
#ifndef QRS_PIECE32_BLOCKS_PER_CU_W8
#define QRS_PIECE32_BLOCKS_PER_CU_W8 4
#endif
#ifndef QRS_PIECE32_BLOCKS_PER_CU_W4
#define QRS_PIECE32_BLOCKS_PER_CU_W4 6
#endif
#ifndef QRS_PIECE32_BLOCKS_PER_CU_W2
#define QRS_PIECE32_BLOCKS_PER_CU_W2 0
#endif
template <int W, int OF>
constexpr uint32_t kPieceBlocksPerCu =
    OF == kOutF32
        ? (W >= 8 ? QRS_PIECE32_BLOCKS_PER_CU_W8 : (W >= 4 ? QRS_PIECE32_BLOCKS_PER_CU_W4 : QRS_PIECE32_BLOCKS_PER_CU_W2))
        : (W >= 8 ? QRS_PIECE_BLOCKS_PER_CU_W8 : (W >= 4 ? QRS_PIECE_BLOCKS_PER_CU_W4 : QRS_PIECE_BLOCKS_PER_CU_W2));

// One launch, chosen but not yet enqueued: the kernel instantiation, its
// grid, the dynamic LDS that caps residency, and the launch device's sizes
// (zeros when they were not read).
struct Prepared {
  const void* kernel = nullptr;
  dim3 grid;
  dim3 block;
  size_t lds = 0;
  uint32_t blocks_per_cu_cap = 0;
  DeviceShape device{};
  KernelArgs args{};
  // reduce_piece_flat_kernel: the leading arguments (piece count, pairing
  // bound; the code bases come from args.x).
  bool lead_args = false;
  uint32_t lead_n = 0;
  uint32_t lead_limit = 0;
};

hipError_t launch_prepared(const Prepared& p, hipStream_t stream) {
  KernelArgs a = p.args;
  if (p.lead_args) {
    uint32_t n = p.lead_n;
    uint32_t limit = p.lead_limit;
    const void* x[kMaxWorld];
    for (int r = 0; r < kMaxWorld; ++r) x[r] = a.x[r];
    void* arg_ptrs[] = {&n, &limit, &x[0], &x[1], &x[2], &x[3], &x[4], &x[5], &x[6], &x[7], &a};
    return hipLaunchKernel(p.kernel, p.grid, p.block, arg_ptrs, p.lds, stream);
  }
  void* arg_ptrs[] = {&a};
  return hipLaunchKernel(p.kernel, p.grid, p.block, arg_ptrs, p.lds, stream);
}

// Unused dynamic LDS that leaves room for only N blocks of Kernel per CU of
// the launch device. No cap for grids under three
// generations of such blocks, when the device's sizes or the kernel's static
// LDS cannot be read (the next launch asks again), or when one block may not
// allocate its share. One instantiation, and one cached static LDS size, per
// kernel.
template <auto Kernel>
void flat_cap(uint64_t blocks, uint64_t N, hipStream_t stream, Prepared* p) {
  // No device has fewer than 32 CUs per partition here: smaller grids are
  // never capped, and skip the device query.
  if (N == 0 || blocks < 3 * 32 * N) return;
  DeviceShape d;
  if (!device_shape(stream, &d)) return;
  p->device = d;
  if (blocks < 3 * static_cast<uint64_t>(d.cus) * N) return;
  static std::atomic<int64_t> cached_static_lds{-1};
  int64_t static_lds = cached_static_lds.load(std::memory_order_relaxed);
  if (static_lds < 0) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(Kernel)) != hipSuccess) return;
    static_lds = static_cast<int64_t>(attr.sharedSizeBytes);
    cached_static_lds.store(static_lds, std::memory_order_relaxed);
  }
  const uint64_t per_block = d.lds_per_cu / N;
  if (per_block > d.lds_per_block || per_block <= static_cast<uint64_t>(static_lds)) return;
  p->lds = per_block - static_cast<uint64_t>(static_lds);
  p->blocks_per_cu_cap = static_cast<uint32_t>(N);
}

template <int W, int XF, int SL, int OF>
hipError_t prepare_typed(const ReduceLaunch& l, hipStream_t stream, Prepared* p) {
  KernelArgs& a = p->args;
  for (int r = 0; r < kMaxWorld; ++r) {
    a.x[r] = r < W ? static_cast<const u32x4*>(l.x[r]) : nullptr;
    a.scales[r] = r < W ? l.scales[r] : nullptr;
    a.out[r] = r < l.n_shares ? l.out[r] : nullptr;
  }
  if (l.n_rows == 0 || l.row_elems == 0 || l.row_elems % 128) return hipErrorInvalidValue;
  if (l.x_row_stride % 16 || l.out_row_stride % 16 || l.x_share_stride % 16) return hipErrorInvalidValue;
  if (l.n_shares != 1 && l.n_shares != W) return hipErrorInvalidValue;
  a.chunks_per_row = l.row_elems / kChunk;
  const uint64_t per_block = static_cast<uint64_t>(QRS_BLOCK) * QRS_CHUNKS_PER_LANE;
  if (l.n_rows > (1ull << 40) / a.chunks_per_row) return hipErrorInvalidValue;
  a.total_chunks = a.chunks_per_row * l.n_rows;
  const uint64_t blocks = (a.total_chunks + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  // Row split constants. Exact when the chunk index is below 2^39 (block
  // count above) and when a lane's offset from its block's first row start,
  // below chunks_per_row + per_block, stays under 1024 with
  // chunks_per_row < 1024: the rounding excess of each product then stays
  // below 1 / chunks_per_row.
  if (l.n_rows > 1 && (a.chunks_per_row < 64 || a.chunks_per_row + per_block > 1024)) return hipErrorInvalidValue;
  a.div_magic = ~0ull / a.chunks_per_row + 1;
  a.div_m20 = static_cast<uint32_t>(((1ull << 20) + a.chunks_per_row - 1) / a.chunks_per_row);
  // Row-strided shares: rows and row strides below 2^32 (of their units),
  // so each row offset is one 32 x 32 -> 64-bit multiply.
  if (l.n_rows > 1 && (l.n_rows > 0xFFFFFFFFull || l.x_row_stride / 16 > 0xFFFFFFFFull ||
                       l.scale_row_stride > 0xFFFFFFFFull || l.out_row_stride / 16 > 0xFFFFFFFFull))
    return hipErrorInvalidValue;
  // ... and each scale slice spans less than 4 GiB (32-bit offsets).
  const uint64_t scale_row_bytes = l.row_elems / 32;  // both layouts: 1/32 byte per element
  if (l.n_rows > 1 && (l.n_rows - 1) * l.scale_row_stride + scale_row_bytes > 0xFFFFFFFFull)
    return hipErrorInvalidValue;
  a.x_row_stride = static_cast<uint32_t>(l.x_row_stride / 16);
  a.scale_row_stride = static_cast<uint32_t>(l.scale_row_stride);
  a.out_row_stride = static_cast<uint32_t>(l.out_row_stride / 16);
  a.x_share_stride = l.x_share_stride / 16;
  a.scale_share_stride = l.scale_share_stride;
  p->grid = dim3(static_cast<uint32_t>(blocks), l.n_shares);
  p->block = dim3(QRS_BLOCK);
  const uint64_t piece_blocks = (a.total_chunks * 2 + QRS_BLOCK - 1) / QRS_BLOCK;
  if (l.n_shares > 1) {
    if (l.n_rows != 1) return hipErrorInvalidValue;
    if constexpr (kPieceLayout<W, SL, OF>) {
      if (piece_blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
      p->grid = dim3(static_cast<uint32_t>(piece_blocks), l.n_shares);
      a.pair_limit = static_cast<uint32_t>(piece_blocks) & ~15u;
      constexpr auto kernel = reduce_piece_kernel<W, XF, OF, kAddrShares>;
      p->kernel = reinterpret_cast<const void*>(kernel);
      flat_cap<kernel>(piece_blocks * l.n_shares, kPieceSharesBlocksPerCu<W>, stream, p);
      return hipSuccess;
    }
    p->kernel = reinterpret_cast<const void*>(reduce_kernel<W, XF, SL, OF, kAddrShares>);
    return hipSuccess;
  }
  if (l.n_rows > 1) {
    if constexpr (kPieceLayout<W, SL, OF>) {
      if (piece_blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
      a.div_magic = ~0ull / (a.chunks_per_row * 2) + 1;  // rows of H / 8 pieces
      p->grid = dim3(static_cast<uint32_t>(piece_blocks));
      a.pair_limit = static_cast<uint32_t>(piece_blocks) & ~15u;
#if QRS_ROWS_XCD_GROUPS
      // Scale rows off 128-byte lines (a row's bytes, its stride or a rank's
      // base): lines are shared between ranks' rows and between rows, so
      // give each XCD runs of blocks covering whole rows (G = lcm(pieces per
      // row, 256) / 256 <= 64), unless the grid holds no full set of runs.
      bool misaligned = (l.row_elems / 32) % 128 != 0 || l.scale_row_stride % 128 != 0;
      for (int r = 0; r < W; ++r) misaligned |= reinterpret_cast<uintptr_t>(l.scales[r]) % 128 != 0;
      const uint64_t ppr = a.chunks_per_row * 2;
      uint64_t g = 256;
      for (uint64_t m = ppr; m != 0;) {  // g = gcd(ppr, 256)
        const uint64_t t = g % m;
        g = m;
        m = t;
      }
      const uint64_t run = ppr / g;  // lcm(ppr, 256) / 256
      // (The division by multiply-high is exact for k = b / 8 below 2^26.)
      if (misaligned && run >= 2 && run <= 64 && piece_blocks >= 8 * run && piece_blocks < (1ull << 29)) {
        a.xcd_group = static_cast<uint32_t>(run);
        a.xcd_group_magic = static_cast<uint32_t>(((1ull << 32) + run - 1) / run);
        a.pair_limit = static_cast<uint32_t>(piece_blocks / (8 * run) * (8 * run));
      }
#endif
      p->kernel = reinterpret_cast<const void*>(reduce_piece_kernel<W, XF, OF, kAddrRows>);
      return hipSuccess;
    }
    p->kernel = reinterpret_cast<const void*>(reduce_kernel<W, XF, SL, OF, kAddrRows>);
    return hipSuccess;
  }
  // The output is the largest of the share's tensors (at least 2 bytes per
  // element against 1 + 1/32 for a slice and its scales).
  if (a.chunks_per_row * OutPieces<OF>::kCount * sizeof(u32x4) < (1ull << 32)) {
    if constexpr (kPieceLayout<W, SL, OF>) {
      if (piece_blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
#if QRS_PIECE_PRELOAD
      constexpr auto kernel = reduce_piece_flat_kernel<W, XF, OF>;
      p->lead_args = true;
      p->lead_n = static_cast<uint32_t>(a.total_chunks * 2);  // below 2^28: the output is under 4 GiB
      p->lead_limit = static_cast<uint32_t>(piece_blocks) & ~15u;
#else
      constexpr auto kernel = reduce_piece_kernel<W, XF, OF, kAddrFlat32>;
#endif
      p->grid = dim3(static_cast<uint32_t>(piece_blocks));
      a.pair_limit = static_cast<uint32_t>(piece_blocks) & ~15u;
      p->kernel = reinterpret_cast<const void*>(kernel);
      flat_cap<kernel>(piece_blocks, kPieceBlocksPerCu<W, OF>, stream, p);
      return hipSuccess;
    }
    constexpr auto kernel = reduce_kernel<W, XF, SL, OF, kAddrFlat32>;
    p->kernel = reinterpret_cast<const void*>(kernel);
    flat_cap<kernel>(blocks, QRS_FLAT_BLOCKS_PER_CU, stream, p);
    return hipSuccess;
  }
  constexpr auto kernel = reduce_kernel<W, XF, SL, OF, kAddrFlat>;
  p->kernel = reinterpret_cast<const void*>(kernel);
  flat_cap<kernel>(blocks, QRS_FLAT_BLOCKS_PER_CU, stream, p);
  return hipSuccess;
}

template <int W, int XF, int SL>
hipError_t prepare_out(const ReduceLaunch& l, hipStream_t s, Prepared* p) {
  switch (l.out_format) {
    case kOutF32: return prepare_typed<W, XF, SL, kOutF32>(l, s, p);
    case kOutBF16: return prepare_typed<W, XF, SL, kOutBF16>(l, s, p);
    case kOutF16: return prepare_typed<W, XF, SL, kOutF16>(l, s, p);
  }
  return hipErrorInvalidValue;
}

template <int W>
hipError_t prepare_mode(const ReduceLaunch& l, hipStream_t s, Prepared* p) {
  if (l.scale_layout == kScaleE8M0Block32) {
    switch (l.x_format) {
      case kXE4M3FN: return prepare_out<W, kXE4M3FN, kScaleE8M0Block32>(l, s, p);
      case kXE5M2: return prepare_out<W, kXE5M2, kScaleE8M0Block32>(l, s, p);
      default: return hipErrorInvalidValue;  // INT8 has no MX mode
    }
  }
  switch (l.x_format) {
    case kXInt8: return prepare_out<W, kXInt8, kScaleF32Group128>(l, s, p);
    case kXE4M3FN: return prepare_out<W, kXE4M3FN, kScaleF32Group128>(l, s, p);
    case kXE5M2: return prepare_out<W, kXE5M2, kScaleF32Group128>(l, s, p);
  }
  return hipErrorInvalidValue;
}

hipError_t prepare_reduce(const ReduceLaunch& l, hipStream_t stream, Prepared* p) {
  switch (l.world_size) {
    case 2: return prepare_mode<2>(l, stream, p);
    case 4: return prepare_mode<4>(l, stream, p);
    case 8: return prepare_mode<8>(l, stream, p);
  }
  return hipErrorInvalidValue;
}

// Launch devices whose sizes are cached (device ordinal below this).
constexpr int kMaxDevices = 64;
// Per device: CUs in bits 0-15, LDS per CU in bits 16-39, LDS per block in
// bits 40-63; 0 until read.
std::atomic<uint64_t> g_device_shape[kMaxDevices];

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          uint64_t n) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) store_stream(dst + i, load_stream(src + i));
}

}  // namespace

bool device_shape(hipStream_t stream, DeviceShape* out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return false;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return false;
  }
  if (dev < 0 || dev >= kMaxDevices) return false;
  uint64_t packed = g_device_shape[dev].load(std::memory_order_relaxed);
  if (packed == 0) {
    int cus = 0, lds_cu = 0, lds_block = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return false;
    if (cus <= 0 || cus > 0xFFFF || lds_cu <= 0 || lds_cu > 0xFFFFFF || lds_block <= 0 || lds_block > 0xFFFFFF)
      return false;
    packed = static_cast<uint64_t>(cus) | static_cast<uint64_t>(lds_cu) << 16 | static_cast<uint64_t>(lds_block) << 40;
    g_device_shape[dev].store(packed, std::memory_order_relaxed);
  }
  out->cus = static_cast<uint32_t>(packed & 0xFFFF);
  out->lds_per_cu = static_cast<uint32_t>((packed >> 16) & 0xFFFFFF);
  out->lds_per_block = static_cast<uint32_t>(packed >> 40);
  return true;
}

namespace {
template <int W, int SL, int OF>
constexpr bool kSharesOneCappedLaunch = kPieceLayout<W, SL, OF> && kPieceSharesBlocksPerCu<W> > 0;

template <int W>
bool shares_one_capped_launch_w(const ReduceLaunch& l) {
  if (l.scale_layout != kScaleE8M0Block32) return false;
  switch (l.out_format) {
    case kOutF32: return kSharesOneCappedLaunch<W, kScaleE8M0Block32, kOutF32>;
    case kOutBF16: return kSharesOneCappedLaunch<W, kScaleE8M0Block32, kOutBF16>;
    case kOutF16: return kSharesOneCappedLaunch<W, kScaleE8M0Block32, kOutF16>;
  }
  return false;
}
}  // namespace

bool all_shares_take_one_capped_launch(const ReduceLaunch& l) {
  switch (l.world_size) {
    case 2: return shares_one_capped_launch_w<2>(l);
    case 4: return shares_one_capped_launch_w<4>(l);
    case 8: return shares_one_capped_launch_w<8>(l);
  }
  return false;
}

hipError_t launch_reduce(const ReduceLaunch& l, hipStream_t stream) {
  Prepared p;
  const hipError_t e = prepare_reduce(l, stream, &p);
  if (e != hipSuccess) return e;
  return launch_prepared(p, stream);
}

struct PreparedReduce {
  Prepared p;
};

hipError_t prepare_reduce_launch(const ReduceLaunch& l, hipStream_t stream, PreparedReduce** out) {
  *out = nullptr;
  PreparedReduce* q = new (std::nothrow) PreparedReduce;
  if (q == nullptr) return hipErrorOutOfMemory;
  const hipError_t e = prepare_reduce(l, stream, &q->p);
  if (e != hipSuccess) {
    delete q;
    return e;
  }
  *out = q;
  return hipSuccess;
}

hipError_t enqueue_prepared_reduce(const PreparedReduce* p, hipStream_t stream) { return launch_prepared(p->p, stream); }

void destroy_prepared_reduce(PreparedReduce* p) { delete p; }

hipError_t reduce_launch_shape(const ReduceLaunch& l, hipStream_t stream, LaunchShape* out) {
  Prepared p;
  const hipError_t e = prepare_reduce(l, stream, &p);
  if (e != hipSuccess) return e;
  out->blocks = static_cast<uint64_t>(p.grid.x) * p.grid.y * p.grid.z;
  out->threads_per_block = p.block.x * p.block.y * p.block.z;
  out->dynamic_lds = static_cast<uint32_t>(p.lds);
  out->blocks_per_cu_cap = p.blocks_per_cu_cap;
  out->device = p.device;
  if (out->device.cus == 0 && !device_shape(stream, &out->device)) out->device = DeviceShape{};
  return hipSuccess;
}

hipError_t launch_stream_copy(const void* src, void* dst, uint64_t bytes, hipStream_t stream) {
  const uint64_t n = bytes / 16;
  const uint64_t blocks = (n + 255) / 256;
  if (blocks == 0 || blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  return launch_kernel(stream_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
}

}  // namespace qrs
