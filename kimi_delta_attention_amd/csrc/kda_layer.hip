// kda_layer.hip -- the KDA layer's prologue (ShortConv + Swish + L2Norm, with
// the conv state) and epilogue (per-head RMSNorm and sigmoid output gate) as
// standalone kernels for prefill, dense or packed.  Both are HBM-bound
// elementwise passes over [tokens, H, D] rows; the per-row arithmetic is in
// kda_layer.h, shared with the fused decode kernel.
//
// Prologue: one wave walks a block of 64 packed tokens for one (head, tensor),
// carrying the three previous inputs of its channels in registers; at a
// sequence boundary it reloads them from that sequence's conv state (or
// zeros), and at a sequence's last token it writes the new conv state (the last
// three inputs).  Empty sequences get their state copied through.
// Epilogue: one wave per 8 consecutive (token, head) rows.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_layer.h"

namespace kda {
namespace {

constexpr int TB = 64;         // tokens per prologue wave
constexpr int ROWS_EPI = 8;    // rows per epilogue wave
constexpr int PF_ROWS = 8;     // prologue rows in flight per wave
static_assert(TB % PF_ROWS == 0, "whole groups of rows per block");

// The sequence holding packed token t: the last s with cu[s] <= t (t below
// cu[n_seq]; such an s has cu[s + 1] > t, so it is not empty).
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seq, long long t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <typename T, int CPL, bool NORM>
__device__ __forceinline__ void prologue_rows(const T* __restrict__ x, T* __restrict__ y,
                              const float* __restrict__ taps, const float* __restrict__ st_in,
                              float* __restrict__ st_out, int st_off, int SW,
                              const int32_t* __restrict__ cu, int n_seq, long long Tseq, int H,
                              int h, long long t0, long long t1, int lane, float eps) {
  constexpr int D = 64 * CPL;
  float w[CPL][4];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[c][j] = taps[((size_t)h * D + CPL * lane + c) * 4 + j];
  int s = cu ? seq_of(cu, n_seq, t0) : (int)(t0 / Tseq);
  long long start = cu ? cu[s] : (long long)s * Tseq;
  long long end = cu ? cu[s + 1] : start + Tseq;
  float hist[3][CPL];
  // the three inputs before token t of sequence s
  auto init_hist = [&](long long t) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const long long tj = t - 3 + j;
      if (tj >= start) {
        row_load<T, CPL>(x + ((size_t)tj * H + h) * D, lane, hist[j]);
      } else {
        const int sr = (int)(tj - start + 3);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          hist[j][c] = st_in ? st_in[(((size_t)s * 3 + sr) * H + h) * SW + st_off + CPL * lane + c]
                             : 0.f;
      }
    }
  };
  init_hist(t0);
  if (t1 - t0 == TB && t1 < end) {
    // A whole block inside one sequence that does not hold its last token
    // (no sequence change, no state row): PF_ROWS rows in flight per wave.
    // Slot i of the ring holds row t0 + PF_ROWS gi + i of group gi and is
    // refilled with the same slot's row of group gi + 1 once read; the group
    // is unrolled and every
    // step issues exactly one load and one store, so the slots are fixed
    // registers and a row is waited for only when it is used (a row past the
    // block re-reads its last row).
    T ring[PF_ROWS][CPL];  // as loaded: converted when used, so only the use waits
#pragma unroll
    for (int i = 0; i < PF_ROWS; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) ring[i][c] = x[((size_t)(t0 + i) * H + h) * D + CPL * lane + c];
    for (int gi = 0; gi < TB / PF_ROWS; ++gi) {
#pragma unroll
      for (int i = 0; i < PF_ROWS; ++i) {
        const long long t = t0 + PF_ROWS * gi + i;
        const long long tn = t + PF_ROWS < t1 ? t + PF_ROWS : t1 - 1;
        float xr[CPL], out[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) xr[c] = to_f(ring[i][c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) ring[i][c] = x[((size_t)tn * H + h) * D + CPL * lane + c];
        prologue_row<CPL, NORM>(hist, xr, w, eps, out);
        row_store<T, CPL>(y + ((size_t)t * H + h) * D, lane, out);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          hist[0][c] = hist[1][c];
          hist[1][c] = hist[2][c];
          hist[2][c] = xr[c];
        }
      }
    }
    return;
  }
  for (long long t = t0; t < t1; ++t) {
    if (t >= end) {  // next non-empty sequence
      do {
        ++s;
        start = end;
        end = cu ? cu[s + 1] : start + Tseq;
      } while (t >= end);
      init_hist(t);
    }
    float xr[CPL], out[CPL];
    row_load<T, CPL>(x + ((size_t)t * H + h) * D, lane, xr);
    prologue_row<CPL, NORM>(hist, xr, w, eps, out);
    row_store<T, CPL>(y + ((size_t)t * H + h) * D, lane, out);
    if (st_out && t == end - 1) {
      float* so = st_out + ((size_t)s * 3 * H + h) * SW + st_off + CPL * lane;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        so[c] = hist[1][c];
        so[(size_t)H * SW + c] = hist[2][c];
        so[(size_t)2 * H * SW + c] = xr[c];
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      hist[0][c] = hist[1][c];
      hist[1][c] = hist[2][c];
      hist[2][c] = xr[c];
    }
  }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void prologue_kernel(
    const T* __restrict__ xq, const T* __restrict__ xk, const T* __restrict__ xv, ConvArgs conv,
    const float* __restrict__ st_in, float* __restrict__ st_out, const int32_t* __restrict__ cu,
    int n_seq, long long Tseq, long long total, int H, T* __restrict__ q, T* __restrict__ k,
    T* __restrict__ v) {
  constexpr int SW = 2 * DK + DV;
  const int lane = threadIdx.x & 63;
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long n_blk = (total + TB - 1) / TB;
  const long long n_items = n_blk * H * 3;
  if (item < n_items) {
    const int ten = (int)(item % 3);
    const int h = (int)((item / 3) % H);
    const long long t0 = (item / (3 * H)) * TB;
    const long long t1 = t0 + TB < total ? t0 + TB : total;
    if (ten == 0)
      prologue_rows<T, DK / 64, true>(xq, q, conv.w[0], st_in, st_out, 0, SW, cu, n_seq, Tseq, H,
                                      h, t0, t1, lane, conv.eps);
    else if (ten == 1)
      prologue_rows<T, DK / 64, true>(xk, k, conv.w[1], st_in, st_out, DK, SW, cu, n_seq, Tseq,
                                      H, h, t0, t1, lane, conv.eps);
    else
      prologue_rows<T, DV / 64, false>(xv, v, conv.w[2], st_in, st_out, 2 * DK, SW, cu, n_seq,
                                       Tseq, H, h, t0, t1, lane, conv.eps);
    return;
  }
  // one wave per empty sequence hands its conv state through
  const long long s = item - n_items;
  if (!st_out || s >= n_seq) return;
  const long long len = cu ? (long long)cu[s + 1] - cu[s] : Tseq;
  if (len > 0) return;
  for (long long e = lane; e < (long long)3 * H * SW; e += 64)
    st_out[s * 3 * H * SW + e] = st_in ? st_in[s * 3 * H * SW + e] : 0.f;
}

// conv state out [n_seq][3][H][SW]: element (s, j, h, c) is input end - 3 + j
// of sequence s, from x when it lies in the sequence, else from the state
// handed in (row index shifted by the sequence's length) or zero.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_kernel(
    const T* __restrict__ xq, const T* __restrict__ xk, const T* __restrict__ xv,
    const float* __restrict__ st_in, float* __restrict__ st_out, const int32_t* __restrict__ cu,
    int n_seq, long long Tseq, int H, int Dk, int Dv) {
  const int SW = 2 * Dk + Dv;
  const long long n = (long long)n_seq * 3 * H * SW;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx % SW);
    const int h = (int)((idx / SW) % H);
    const int j = (int)((idx / ((long long)SW * H)) % 3);
    const long long s = idx / (3LL * SW * H);
    const long long start = cu ? (long long)cu[s] : s * Tseq;
    const long long end = cu ? (long long)cu[s + 1] : start + Tseq;
    const long long p = end - 3 + j;
    float val = 0.f;
    if (p >= start) {
      const T* x = c < Dk ? xq : c < 2 * Dk ? xk : xv;
      const int cc = c < Dk ? c : c < 2 * Dk ? c - Dk : c - 2 * Dk;
      const int D = c < 2 * Dk ? Dk : Dv;
      val = to_f(x[((size_t)p * H + h) * D + cc]);
    } else if (st_in) {
      val = st_in[((s * 3 + (p - start + 3)) * H + h) * SW + c];
    }
    st_out[idx] = val;
  }
}

template <typename TO, typename TG, typename TY, int CPL>
__global__ __launch_bounds__(256) void epilogue_kernel(const TO* __restrict__ o,
                                                       const TG* __restrict__ g,
                                                       const float* __restrict__ wn, float eps,
                                                       TY* __restrict__ y, long long rows) {
  constexpr int D = 64 * CPL;
  const int lane = threadIdx.x & 63;
  const long long r0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * ROWS_EPI;
  float w[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) w[c] = wn[CPL * lane + c];
  for (long long r = r0; r < r0 + ROWS_EPI && r < rows; ++r) {
    float ov[CPL], gv[CPL], out[CPL];
    row_load<TO, CPL>(o + (size_t)r * D, lane, ov);
    row_load<TG, CPL>(g + (size_t)r * D, lane, gv);
    epilogue_row<CPL>(ov, gv, w, eps, out);
    row_store<TY, CPL>(y + (size_t)r * D, lane, out);
  }
}

template <typename T, int DK, int DV>
hipError_t launch_pro_t(const PrologueArgs& a) {
  const long long n_blk = (a.total + TB - 1) / TB;
  const long long waves = n_blk * a.H * 3 + (a.st_out ? a.n_seq : 0);
  const long long grid = (waves + 3) / 4;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prologue_kernel<T, DK, DV>), dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)a.stream, (const T*)a.xq, (const T*)a.xk, (const T*)a.xv,
                     a.conv, a.st_in, a.st_out, a.cu_seqlens, a.n_seq, a.Tseq, a.total, a.H,
                     (T*)a.q, (T*)a.k, (T*)a.v);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pro_d(const PrologueArgs& a) {
  if (a.Dk == 128) return a.Dv == 128 ? launch_pro_t<T, 128, 128>(a) : launch_pro_t<T, 128, 64>(a);
  return a.Dv == 128 ? launch_pro_t<T, 64, 128>(a) : launch_pro_t<T, 64, 64>(a);
}

template <typename TO, typename TG, typename TY>
hipError_t launch_epi_t(const EpilogueArgs& a) {
  const long long rows = a.rows * a.H;
  const long long grid = (rows + 4 * ROWS_EPI - 1) / (4 * ROWS_EPI);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.Dv == 128)
    hipLaunchKernelGGL((epilogue_kernel<TO, TG, TY, 2>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)a.stream, (const TO*)a.o, (const TG*)a.g, a.w, a.eps,
                       (TY*)a.y, rows);
  else
    hipLaunchKernelGGL((epilogue_kernel<TO, TG, TY, 1>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)a.stream, (const TO*)a.o, (const TG*)a.g, a.w, a.eps,
                       (TY*)a.y, rows);
  return hipGetLastError();
}

template <typename TO, typename TG>
hipError_t launch_epi_g(const EpilogueArgs& a) {
  return a.y_bf16 ? launch_epi_t<TO, TG, bf16>(a) : launch_epi_t<TO, TG, float>(a);
}

template <typename TO>
hipError_t launch_epi_o(const EpilogueArgs& a) {
  return a.g_bf16 ? launch_epi_g<TO, bf16>(a) : launch_epi_g<TO, float>(a);
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a) {
  return a.bf16 ? launch_pro_d<bf16>(a) : launch_pro_d<float>(a);
}

hipError_t launch_epilogue(const EpilogueArgs& a) {
  return a.o_bf16 ? launch_epi_o<bf16>(a) : launch_epi_o<float>(a);
}

hipError_t launch_conv_state(const PrologueArgs& a) {
  if (!a.st_out || a.n_seq <= 0) return hipSuccess;
  const long long n = (long long)a.n_seq * 3 * a.H * (2 * a.Dk + a.Dv);
  long long grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (a.bf16)
    hipLaunchKernelGGL((conv_state_kernel<bf16>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)a.stream, (const bf16*)a.xq, (const bf16*)a.xk,
                       (const bf16*)a.xv, a.st_in, a.st_out, a.cu_seqlens, a.n_seq, a.Tseq, a.H,
                       a.Dk, a.Dv);
  else
    hipLaunchKernelGGL((conv_state_kernel<float>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)a.stream, (const float*)a.xq, (const float*)a.xk,
                       (const float*)a.xv, a.st_in, a.st_out, a.cu_seqlens, a.n_seq, a.Tseq, a.H,
                       a.Dk, a.Dv);
  return hipGetLastError();
}

}  // namespace kda
