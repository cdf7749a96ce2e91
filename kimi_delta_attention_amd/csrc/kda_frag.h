// kda_frag.h -- register-fragment helpers of the gfx950 bf16 chunk kernels
// (prefill pass 1 / fused prefill in kda_prefill.hip, the state pass in
// kda_prefill_state.hip) and the layout of the per-chunk operand images that
// pass 1 writes and the state pass reads.
#pragma once
#include "kda_common.h"
#include "kda_layer.h"

namespace kda {
namespace frag {

constexpr int CH = 64;    // chunk
constexpr int BV = 64;    // value slice per workgroup

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

// Operand fragment (16 columns m0.., 8 k values per lane) of a row-major
// [k][m] LDS tile: lane l (j = l%16) gets column m0 + j at rows ra..ra+3 and
// rb..rb+3 (ra, rb chosen per 16-lane group).  Two transpose reads, each of which
// gives lane i of a 16-lane group element i%4 of the 8-byte words read by
// lanes i/4, i/4+4, i/4+8, i/4+12 of that group.
__device__ __forceinline__ bf16x8 frag_tr(const bf16* X, int ld, int m0, int ra, int rb, int j) {
  const bf16* pa = X + (ra + (j >> 2)) * ld + m0 + 4 * (j & 3);
  const bf16* pb = X + (rb + (j >> 2)) * ld + m0 + 4 * (j & 3);
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)pa);
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)pb);
  const short8v s = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, s);
}

// 16 contiguous bytes of a k-contiguous LDS row (g = lane / 16).
__device__ __forceinline__ bf16x8 frag_ld(const bf16* X, int ld, int row, int k0, int g) {
  return *reinterpret_cast<const bf16x8*>(X + row * ld + k0 + 8 * g);
}

// Inclusive product scan over the 16 lanes of each DPP row, for N values per
// lane: lane i of a row ends with x_0 * ... * x_i.  Each step is one
// v_mul_f32_dpp with row_shr:D and bound_ctrl off, which leaves lanes i < D
// unwritten (they keep x_i).  A step reads values written N instructions
// earlier, so only the first needs the 2 wait states of a VALU write -> DPP
// read.
template <int N>
__device__ __forceinline__ void row_scan_mul(float* x) {
  static_assert(N == 8 || N == 16, "scan width");
#define KDA_SCAN_STEP(D, i) "v_mul_f32_dpp %" #i ", %" #i ", %" #i " row_shr:" #D " row_mask:0xf bank_mask:0xf\n"
#define KDA_SCAN8(D) KDA_SCAN_STEP(D, 0) KDA_SCAN_STEP(D, 1) KDA_SCAN_STEP(D, 2) KDA_SCAN_STEP(D, 3) \
  KDA_SCAN_STEP(D, 4) KDA_SCAN_STEP(D, 5) KDA_SCAN_STEP(D, 6) KDA_SCAN_STEP(D, 7)
#define KDA_SCAN16(D) KDA_SCAN8(D) KDA_SCAN_STEP(D, 8) KDA_SCAN_STEP(D, 9) KDA_SCAN_STEP(D, 10) \
  KDA_SCAN_STEP(D, 11) KDA_SCAN_STEP(D, 12) KDA_SCAN_STEP(D, 13) KDA_SCAN_STEP(D, 14) KDA_SCAN_STEP(D, 15)
  if constexpr (N == 8) {
    __asm__("s_nop 1\n" KDA_SCAN8(1) KDA_SCAN8(2) KDA_SCAN8(4) KDA_SCAN8(8)
            : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
              "+v"(x[7]));
  } else {
    __asm__("s_nop 1\n" KDA_SCAN16(1) KDA_SCAN16(2) KDA_SCAN16(4) KDA_SCAN16(8)
            : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
              "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
              "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
  }
#undef KDA_SCAN16
#undef KDA_SCAN8
#undef KDA_SCAN_STEP
}

__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)x[e];
    hi[e] = h;
    lo[e] = (bf16)(x[e] - (float)h);
  }
}

__device__ __forceinline__ float bfv(unsigned int packed, int half) {
  return __builtin_bit_cast(float, half ? (packed & 0xffff0000u) : (packed << 16));
}

// Exclusive suffix product over the 16 lanes of each DPP row, for N values per
// lane: lane i ends with x_{i+1} * ... * x_15 (1 for lane 15).  A shift by one
// lane (lane 15 takes 1), then steps of v_mul_f32_dpp with row_shl:D and
// bound_ctrl off, which leave lanes i >= 16 - D unwritten.  Every factor is a
// product of decays <= 1, so nothing can overflow.
template <int N>
__device__ __forceinline__ void row_rscan_excl(float* x) {
  static_assert(N == 8, "suffix scan width");
#pragma unroll
  for (int e = 0; e < N; ++e)
    x[e] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x[e]),
                                                      0x101, 0xf, 0xf, false));  // row_shl:1
#define KDA_RSCAN_STEP(D, i) "v_mul_f32_dpp %" #i ", %" #i ", %" #i " row_shl:" #D " row_mask:0xf bank_mask:0xf\n"
#define KDA_RSCAN8(D) KDA_RSCAN_STEP(D, 0) KDA_RSCAN_STEP(D, 1) KDA_RSCAN_STEP(D, 2) KDA_RSCAN_STEP(D, 3) \
  KDA_RSCAN_STEP(D, 4) KDA_RSCAN_STEP(D, 5) KDA_RSCAN_STEP(D, 6) KDA_RSCAN_STEP(D, 7)
  __asm__("s_nop 1\n" KDA_RSCAN8(1) KDA_RSCAN8(2) KDA_RSCAN8(4) KDA_RSCAN8(8)
          : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
            "+v"(x[7]));
#undef KDA_RSCAN8
#undef KDA_RSCAN_STEP
}

// The diagonal 16-token tile of A and Mqk uses the factored decay
// (k_j / P_j) . (q_r P_r): exact as long as 1 / P_j stays in fp32 range.  A tile
// whose whole-tile decay E (its smallest P) falls below kTileMin in any key
// channel is computed instead by tile_exact_sums, and its other factors that
// divide by P (E / P_j for Ktil and the key side of later tiles) become the
// exclusive suffix products of the tile's decays.  K3's lower-bounded gate
// (log alpha >= -5 per token, "Kimi K3 的 KDA" section 6, "Kimi K3模型架构详解"
// section 3.4) never goes below it: e^(-80) > 2^(-116), so such tiles take the
// factored path, bitwise as before.
constexpr float kTileMin = 0x1p-116f;

// 1 in every lane if any of the tile's Dk whole-tile decays (E, a [Dk] row in
// LDS) is below kTileMin: a wave-uniform decision.
template <int DK>
__device__ __forceinline__ bool tile_flagged(const float* E, int lane) {
  bool low = false;
#pragma unroll
  for (int c = 0; c < DK; c += 64) low = low || E[c + lane] < kTileMin;
  return __builtin_amdgcn_ballot_w64(low) != 0;
}

// Exact decayed dot products inside one 16-token tile (the fallback of the
// factored diagonal tile).  This lane holds query token r = tr of the tile and,
// for NB 32-channel blocks, the 8 channels 32 kb + 16 h + 4 g + i (h, i < 2, 4):
// their decays al[b][4 h + i] and k, q packed two bf16 per word (kp, qp, as
// loaded).  For key token j of the tile,
//     R_c(r, j) = alpha_{j+1,c} ... alpha_{r,c}   (1 for j = r),
//     a(j) = sum_c k_rc k_jc R_c(r, j),   m(j) = sum_c q_rc k_jc R_c(r, j),
// summed over these blocks' channels of all four lane rows; R is a running
// product restarted after j (a 16-lane DPP scan), so no factor exceeds 1.
// Returns in A[i], M[i] the sums for j = 4 g + i, the accumulator layout of a
// 16 x 16 tile product with rows j and columns r (entries with j > r are not
// meaningful; the callers mask them).  Fixed order of every sum, so the two
// schedules that call it agree bitwise.
template <int NB>
__device__ __forceinline__ void tile_exact_sums(const float (*al)[8], const uint2v (*kp)[2],
                                                const uint2v (*qp)[2], int tr, int g,
                                                float (&A)[4], float (&M)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i] = 0.f;
    M[i] = 0.f;
  }
  const int row0 = 4 * 16 * g;  // ds_bpermute byte address of lane 16 g
  for (int j = 0; j < 16; ++j) {
    float pa = 0.f, pm = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = tr > j ? al[b][e] : 1.f;
      row_scan_mul<8>(x);
      unsigned kj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kj[u] = (unsigned)__builtin_amdgcn_ds_bpermute(row0 + 4 * j, (int)kp[b][u >> 1][u & 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = x[e] * bfv(kj[e >> 1], e & 1);
        pa = __builtin_fmaf(bfv(kp[b][e >> 2][(e & 3) >> 1], e & 1), t, pa);
        pm = __builtin_fmaf(bfv(qp[b][e >> 2][(e & 3) >> 1], e & 1), t, pm);
      }
    }
    pa = rows4_sum(pa);
    pm = rows4_sum(pm);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[i] = j == 4 * g + i ? pa : A[i];
      M[i] = j == 4 * g + i ? pm : M[i];
    }
  }
}


__device__ __forceinline__ void st_bf16x4(bf16* p, const float* x) {
  // 4 values -> one 8-byte LDS store
  short4v s;
#pragma unroll
  for (int e = 0; e < 4; ++e) s[e] = __builtin_bit_cast(short, (bf16)x[e]);
  *reinterpret_cast<short4v*>(p) = s;
}

__device__ __forceinline__ void st_split4(bf16* hi, int lo_off, const float* x) {
  short4v sh, sl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 h = (bf16)x[e];
    sh[e] = __builtin_bit_cast(short, h);
    sl[e] = __builtin_bit_cast(short, (bf16)(x[e] - (float)h));
  }
  *reinterpret_cast<short4v*>(hi) = sh;
  *reinterpret_cast<short4v*>(hi + lo_off) = sl;
}

// x = hi + lo for 4 values, each part packed two bf16 per 32-bit word.
__device__ __forceinline__ void split4_pack(const float* x, uint2v& hi, uint2v& lo) {
  unsigned int h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 hv = (bf16)x[e];
    h[e] = __builtin_bit_cast(unsigned short, hv);
    l[e] = __builtin_bit_cast(unsigned short, (bf16)(x[e] - (float)hv));
  }
  hi = uint2v{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  lo = uint2v{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
}

// a (rounded once) times b = bh + bl: the A operand W of W S when the gate
// decays (its single rounding then stays within the error budget; the B side,
// the state, does not)
__device__ __forceinline__ floatx4 mma_a1(const bf16x8& a, const bf16x8& bh, const bf16x8& bl,
                                          floatx4 c) {
  c = mfma_bf16(a, bh, c);
  c = mfma_bf16(a, bl, c);
  return c;
}

__device__ __forceinline__ floatx4 mma_ab(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bl, floatx4 c) {
  c = mfma_bf16(ah, bh, c);
  c = mfma_bf16(ah, bl, c);
  c = mfma_bf16(al, bh, c);
  return c;
}

// W S with W rounded once, or split where the rounding would build up: the
// products of mma_ab in the same order, the third (W's low part) only for a
// split chunk, so both schedules give bitwise the same results.
__device__ __forceinline__ floatx4 mma_w(bool split, const bf16x8& wh, const bf16x8& wl,
                                         const bf16x8& bh, const bf16x8& bl, floatx4 c) {
  c = mma_a1(wh, bh, bl, c);
  if (split) c = mfma_bf16(wl, bh, c);
  return c;
}

// The rounding of W (W S's left side) once to bf16 enters the state through
// Ktil^T P and decays with it: where every key channel keeps less than half of
// its state over the chunk (Gamma_C < 1/2), the error of a chunk is at most
// doubled by the chunks after it, but where some channel keeps more (slow
// decay, alpha = 1, the gate without decay) it accumulates over the sequence.
// Such chunks keep W split (hi + lo).  A wave-uniform decision from the
// chunk's Dk decays Gamma_C (a [Dk] row in LDS).
constexpr float kKeepSplitW = 0.5f;
template <int DK>
__device__ __forceinline__ bool w_split_chunk(const float* GC, int lane) {
  bool keep = false;
#pragma unroll
  for (int c = 0; c < DK; c += 64) keep = keep || GC[c + lane] >= kKeepSplitW;
  return __builtin_amdgcn_ballot_w64(keep) != 0;
}

// Per-chunk operand images written by the first pass of the two-pass prefill
// and read by the state pass.  Every image is a sequence of 1 KiB frames; a
// frame is one 16-byte register fragment per lane (lane l at byte 16 l), so a
// wave moves a frame with one fully coalesced 16-byte load or store per lane.
// Frames (w = token tile of the chunk, kb = 32-wide k block):
//   W  [w][kb < DK/32][hi, lo]   A operand of W S (row = token, k = channel
//                                position 32kb + 8g + 4h + i <-> channel
//                                32kb + 16h + 4g + i); the low part written
//                                only for a chunk that keeps W split
//                                (w_split_chunk)
//   Q  [w][kb < DK/32]           A operand of (Gamma*Q) S, same positions
//   QL [kb < DK/32]              low halves of tile 0's Gamma*Q, written and
//                                read only in a sequence's first chunk (there
//                                the read-out of the entry state is the least
//                                decayed and keeps Gamma*Q split)
//   M  [w][kb < 2][hi, lo]       A operand of Mqk P (k = token position)
//   K  [rt < DK/16][kb < 2][hi, lo]  A operand of Ktil^T P for state rows
//                                16rt..16rt+15 (k = token position)
//   T  [w][kb < 2][hi, lo]       A operand of U = T Diag(b) V (row = token r,
//                                k = token j in order); the frames of key
//                                blocks after the tile are zero and not written
//   V  [64 tokens][DV] bf16      the chunk's v rows, written only by the layer
//                                prefill (its v exists only inside the first
//                                pass); otherwise the state pass reads v itself
// followed by Gamma_C (DK floats) and a flag word (non-zero: W is split).
// U is not stored: the state pass forms it from T Diag(b) and v (12 KiB of
// T frames against 32 KiB of fp32 U at Dv = 128, and v is read once).
template <int DK, int DV>
struct Images {
  static constexpr int NKB = DK / 32, NCHT = DK / 16, NVT = DV / 16;
  static constexpr int W = 0;
  static constexpr int Q = W + 4 * NKB * 2;
  // Gamma*Q: the high halves of every tile, then the low halves of tile 0
  // (used in a sequence's first chunk only)
  static constexpr int QL = Q + 4 * NKB;
  static constexpr int M = QL + NKB;
  static constexpr int K = M + 4 * 2 * 2;
  static constexpr int TB = K + NCHT * 2 * 2;
  static constexpr int V = TB + 4 * 2 * 2;
  static constexpr int frames = V + DV / 8;  // 64 rows of DV bf16
  static constexpr size_t v_off = (size_t)V * 1024;
  static constexpr size_t g_off = (size_t)frames * 1024;
  static constexpr size_t f_off = g_off + DK * 4;
  static constexpr size_t bytes = (f_off + 4 + 255) / 256 * 256;
  static __device__ __forceinline__ int w_frame(int w, int kb, int part) { return W + (w * NKB + kb) * 2 + part; }
  static __device__ __forceinline__ int q_frame(int w, int kb) { return Q + w * NKB + kb; }
  static __device__ __forceinline__ int ql_frame(int kb) { return QL + kb; }
  static __device__ __forceinline__ int m_frame(int w, int kb, int part) { return M + (w * 2 + kb) * 2 + part; }
  static __device__ __forceinline__ int k_frame(int rt, int kb, int part) { return K + (rt * 2 + kb) * 2 + part; }
  static __device__ __forceinline__ int tb_frame(int w, int kb, int part) { return TB + (w * 2 + kb) * 2 + part; }
};

// 16-byte fragment of frame f of an image at `base`, lane `lane`.
template <typename T>
__device__ __forceinline__ T* frame_ptr(unsigned char* base, int f, int lane) {
  return reinterpret_cast<T*>(base + (size_t)f * 1024 + 16 * lane);
}
template <typename T>
__device__ __forceinline__ const T* frame_ptr(const unsigned char* base, int f, int lane) {
  return reinterpret_cast<const T*>(base + (size_t)f * 1024 + 16 * lane);
}

// Number of 64-token chunks, over all sequences in order, that start before
// packed token `tok`.  Dense: n_seq sequences of T tokens back to back (cu
// NULL).  Packed: sequence s spans tokens cu[s]..cu[s+1]-1 and its chunks are
// numbered from off[s] (the chunk table).  Chunk starts increase with the chunk
// index, so the chunks starting in [a, b) are chunks_before(a)..chunks_before(b)-1.
__device__ __forceinline__ int chunks_before(long long tok, const int32_t* cu, const int32_t* off,
                                             int n_seq, int T) {
  if (tok <= 0 || n_seq <= 0) return 0;
  if (!cu) {
    const int nch = (T + CH - 1) / CH;
    const long long s = tok / T;
    if (s >= n_seq) return n_seq * nch;
    const long long c = (tok - s * T + CH - 1) / CH;
    return (int)s * nch + (int)(c < nch ? c : nch);
  }
  if (tok >= cu[n_seq]) return off[n_seq];
  int lo = 0, hi = n_seq - 1;  // last sequence starting at or before tok
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  const int nch = off[lo + 1] - off[lo];
  long long c = (tok - cu[lo] + CH - 1) / CH;
  if (c < 0) c = 0;
  return off[lo] + (int)(c < nch ? c : nch);
}

// Streaming store of one fragment into an image: written once, read by the
// next kernel, so it bypasses the caches (non-temporal).
template <typename T>
__device__ __forceinline__ void put_frame(unsigned char* base, int f, int lane, const T& v) {
  __builtin_nontemporal_store(v, frame_ptr<T>(base, f, lane));
}

}  // namespace frag
}  // namespace kda
