// Backward of one ring step for the inputs the tuned bf16 kernels do not
// cover: float32 inputs, or head dimension 64.  Plain SIMT code in float32,
// for parity-scale problems (no tiling: each pair's two dot products are
// workgroup reductions).
//
// The same definition as attn_bwd_bf16.hip, with the forward's final
// log-sum-exp L of every query row (ringmaster's reverse ring, "Status", Ring
// row; the chain rule through the softmax):
//   P = exp(scale q.k - L),  dP = dO.v,  dS = P (dP - delta),
//   delta = rowsum(dO * O),  dQ += scale dS k,  dK += scale dS q,  dV += P dO,
// over each row's visible keys of the step (causal, window, packed
// sequences: key_lo(t) .. key_hi(t)).
//   * dQ: a workgroup of D threads (thread d holds column d) per (batch,
//     query row, query head) walks the visible keys of the step's key spans.
//   * dK and dV: a workgroup of D threads per (batch, key, kv head) walks the
//     rows of every query head of the group that see the key.
// No two workgroups write the same output element.
#include "attn_common.h"

namespace ra {
namespace {

using namespace dev;

template <typename T>
__device__ inline float ld(const T* p, long long i);
template <>
__device__ inline float ld<float>(const float* p, long long i) {
  return p[i];
}
template <>
__device__ inline float ld<uint16_t>(const uint16_t* p, long long i) {
  return __uint_as_float((unsigned)p[i] << 16);
}

// (a, b) summed over the workgroup's D threads (D = 64: one wave; 128: two,
// through LDS).  The leading barrier keeps the previous sums' readers ahead
// of this sum's writers.
template <int D>
__device__ inline void wg_sum2(float& a, float& b, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
  }
  if (D == 64) return;
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = a;
    red[2 * w + 1] = b;
  }
  __syncthreads();
  a = red[0] + red[2];
  b = red[1] + red[3];
}

// delta[row] = -sum_d dO[row, d] O[row, d] (stored negated), one thread per row
template <typename T, int D>
__global__ __launch_bounds__(256) void simt_delta_kernel(long long rows, const T* __restrict__ dout,
                                                         const float* __restrict__ o, float* __restrict__ delta) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc += ld<T>(dout, row * D + d) * o[row * D + d];
  delta[row] = -acc;
}

// grid: x = the step's listed query rows (span 0's, then span 1's), y = query
// head, z = batch
template <typename T, int D>
__global__ __launch_bounds__(D) void simt_dq_kernel(BwdParams bp) {
  const StepParams& p = bp.s;
  __shared__ float red[4];
  const int h = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const long long i = blockIdx.x;
  const int sp = i < p.qs_len[0] ? 0 : 1;
  const long long r_in = sp ? i - p.qs_len[0] : i;
  const long long t = (sp ? p.qs_start[1] : p.qs_start[0]) + r_in;
  const long long qrow = ((long long)b * p.Sq + (sp ? p.qs_off[1] : p.qs_off[0]) + r_in) * p.Hq + h;
  const int g = h / p.G;
  const float q = ld<T>((const T*)p.q, qrow * D + d);
  const float dov = ld<T>((const T*)bp.dout, qrow * D + d);
  const float lse = bp.lse[qrow], ndl = bp.delta[qrow];  // -delta
  const long long lo = key_lo(p, t), hi = key_hi(p, t);
  float acc = 0.f;
  for (int ks = 0; ks < p.nks; ++ks) {
    const long long k0 = p.ks_start[ks], j0 = max(lo, k0), j1 = min(hi, k0 + p.ks_len[ks] - 1);
    for (long long j = j0; j <= j1; ++j) {
      const long long krow = ((long long)b * p.Sk + p.ks_off[ks] + (j - k0)) * p.Hkv + g;
      const float k = ld<T>((const T*)p.k, krow * D + d), v = ld<T>((const T*)p.v, krow * D + d);
      float s = q * k, dp = dov * v;
      wg_sum2<D>(s, dp, red);
      const float pr = expf(p.scale * s - lse);
      acc += pr * (dp + ndl) * k;
    }
  }
  float* dst = bp.dq + qrow * D + d;
  *dst = (p.accum ? *dst : 0.f) + p.scale * acc;
}

// grid: x = the step's keys (span 0's, then span 1's), y = kv head, z = batch
template <typename T, int D>
__global__ __launch_bounds__(D) void simt_dkv_kernel(BwdParams bp) {
  const StepParams& p = bp.s;
  __shared__ float red[4];
  const int g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const long long i = blockIdx.x;
  const int ks = i < p.ks_len[0] ? 0 : 1;
  const long long k_in = ks ? i - p.ks_len[0] : i;
  const long long kj = (ks ? p.ks_start[1] : p.ks_start[0]) + k_in;
  const long long krow = ((long long)b * p.Sk + (ks ? p.ks_off[1] : p.ks_off[0]) + k_in) * p.Hkv + g;
  const float k = ld<T>((const T*)p.k, krow * D + d), v = ld<T>((const T*)p.v, krow * D + d);
  long long t0, t1;
  rows_seeing(p, kj, kj, t0, t1);
  float dk = 0.f, dv = 0.f;
  for (int hh = 0; hh < p.G; ++hh) {
    const int h = g * p.G + hh;
    for (int qs = 0; qs < p.nqs; ++qs) {
      const long long a0 = p.qs_start[qs], r0 = max(t0, a0), r1 = min(t1, a0 + p.qs_len[qs] - 1);
      for (long long t = r0; t <= r1; ++t) {
        const long long qrow = ((long long)b * p.Sq + p.qs_off[qs] + (t - a0)) * p.Hq + h;
        const float q = ld<T>((const T*)p.q, qrow * D + d), dov = ld<T>((const T*)bp.dout, qrow * D + d);
        float s = q * k, dp = dov * v;
        wg_sum2<D>(s, dp, red);
        const float pr = expf(p.scale * s - bp.lse[qrow]);
        dk += pr * (dp + bp.delta[qrow]) * q;  // the workspace holds -delta
        dv += pr * dov;
      }
    }
  }
  bp.dk[krow * D + d] += p.scale * dk;
  bp.dv[krow * D + d] += dv;
}

template <typename T, int D>
hipError_t launch_simt(const BwdParams& bp, hipStream_t s) {
  const StepParams& p = bp.s;
  const long long rows = p.qs_len[0] + p.qs_len[1], keys = p.ks_len[0] + p.ks_len[1];
  if (rows > 0)
    hipLaunchKernelGGL((simt_dq_kernel<T, D>), dim3((unsigned)rows, p.Hq, p.B), dim3(D), 0, s, bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || keys == 0) return e;
  hipLaunchKernelGGL((simt_dkv_kernel<T, D>), dim3((unsigned)keys, p.Hkv, p.B), dim3(D), 0, s, bp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_simt(const BwdParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 0 && D == 64) return launch_simt<float, 64>(p, s);
  if (dtype == 0 && D == 128) return launch_simt<float, 128>(p, s);
  if (dtype == 1 && D == 64) return launch_simt<uint16_t, 64>(p, s);
  if (dtype == 1 && D == 128) return launch_simt<uint16_t, 128>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_simt_delta(long long rows, int D, int dtype, const void* dout, const float* o, float* delta,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 255) / 256);
  if (dtype == 0 && D == 64)
    hipLaunchKernelGGL((simt_delta_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, rows, (const float*)dout, o,
                       delta);
  else if (dtype == 0 && D == 128)
    hipLaunchKernelGGL((simt_delta_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, rows, (const float*)dout, o,
                       delta);
  else if (dtype == 1 && D == 64)
    hipLaunchKernelGGL((simt_delta_kernel<uint16_t, 64>), dim3(blocks), dim3(256), 0, s, rows, (const uint16_t*)dout,
                       o, delta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ra
