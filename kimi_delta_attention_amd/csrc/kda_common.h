// kda_common.h -- small device helpers shared by the gfx950 KDA kernels:
// vector types, bf16 hi/lo splitting and the MFMA tile primitives.
//
// MFMA operand layouts used throughout (wave64, gfx950):
//   v_mfma_f32_16x16x32_bf16  A (16 x 32): lane l holds row l%16, k = 8*(l/16) .. +7
//                             B (32 x 16): lane l holds col l%16, k = 8*(l/16) .. +7
//                             C (16 x 16): lane l holds col l%16, rows 4*(l/16) .. +3
//   v_mfma_f32_16x16x4_f32    one fp32 per lane, k-slot = l/16; the fp32 path maps
//                             the 32-wide k block onto 8 such MFMAs so that MFMA i
//                             uses k = 8*(l/16) + i, i.e. the same per-lane k range
//                             as the bf16 form.
// Every operand of a 16x16 tile product is therefore one contiguous 8-element
// run of a k-contiguous LDS row: [M][K] for A operands, [N][K] for B operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// x = hi + lo with hi = RNE(x), lo = RNE(x - hi): the pair carries about 16
// significant bits, so a product of two split operands computed as
// hi*hi + hi*lo + lo*hi keeps fp32-level accuracy (the split-bf16 technique of
// Henry, Tang & Heinecke, ARITH 2019).
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_f32x8(const floatx8& a, const floatx8& b, floatx4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// Operand fragment for one 16x32 (A) or 32x16 (B) k-block.
template <bool F32> struct Frag;
template <> struct Frag<false> { bf16x8 hi, lo; };
template <> struct Frag<true> { floatx8 v; };

// Loads the fragment of row `row` (A: the tile row; B: the tile column) for the
// k-block starting at `k0` from a k-contiguous LDS array with leading dimension
// `ld` (elements).  `lo_off` is the element offset from the hi array to the lo
// array (bf16 path); `want_lo` skips the lo load when the product is single-pass.
template <bool F32> struct Lds;

template <> struct Lds<false> {
  typedef bf16 T;
  static __device__ __forceinline__ Frag<false> load(const bf16* base, int ld, int row, int k0,
                                                     int lo_off, bool want_lo) {
    const int lane = threadIdx.x & 63;
    const bf16* p = base + row * ld + k0 + 8 * (lane >> 4);
    Frag<false> f;
    f.hi = *reinterpret_cast<const bf16x8*>(p);
    if (want_lo) f.lo = *reinterpret_cast<const bf16x8*>(p + lo_off);
    else f.lo = bf16x8{};
    return f;
  }
  // Stores one value split into hi / lo.
  static __device__ __forceinline__ void store(bf16* base, int idx, int lo_off, float x) {
    bf16 h, l;
    split_bf16(x, h, l);
    base[idx] = h;
    base[idx + lo_off] = l;
  }
  static __device__ __forceinline__ void store_hi(bf16* base, int idx, float x) {
    base[idx] = (bf16)x;
  }
};

template <> struct Lds<true> {
  typedef float T;
  static __device__ __forceinline__ Frag<true> load(const float* base, int ld, int row, int k0,
                                                    int, bool) {
    const int lane = threadIdx.x & 63;
    const float* p = base + row * ld + k0 + 8 * (lane >> 4);
    Frag<true> f;
    f.v = *reinterpret_cast<const floatx8*>(p);
    return f;
  }
  static __device__ __forceinline__ void store(float* base, int idx, int, float x) {
    base[idx] = x;
  }
  static __device__ __forceinline__ void store_hi(float* base, int idx, float x) { base[idx] = x; }
};

// Precision of one tile product (bf16 path): how many bf16 passes it takes.
enum Pass { P_SINGLE = 0, P_SPLIT_A = 1, P_SPLIT_B = 2, P_SPLIT_AB = 3 };

template <int MODE>
__device__ __forceinline__ floatx4 mma(const Frag<false>& a, const Frag<false>& b, floatx4 c) {
  c = mfma_bf16(a.hi, b.hi, c);
  if (MODE == P_SPLIT_B || MODE == P_SPLIT_AB) c = mfma_bf16(a.hi, b.lo, c);
  if (MODE == P_SPLIT_A || MODE == P_SPLIT_AB) c = mfma_bf16(a.lo, b.hi, c);
  return c;
}

template <int MODE>
__device__ __forceinline__ floatx4 mma(const Frag<true>& a, const Frag<true>& b, floatx4 c) {
  return mfma_f32x8(a.v, b.v, c);
}

__device__ __forceinline__ bool wants_lo_a(int mode) { return mode == P_SPLIT_A || mode == P_SPLIT_AB; }
__device__ __forceinline__ bool wants_lo_b(int mode) { return mode == P_SPLIT_B || mode == P_SPLIT_AB; }

}  // namespace kda
