// Bandwidth-bound kernels: the standalone log-sum-exp merge of two partial
// results, and the Ulysses sequence<->head regrouping.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();
// Units of 16 bytes per thread: two for the merge (loads of both issued
// before the stores), one for the permutations (measured best on MI355X).
constexpr int kMergeUnits = 2;
constexpr int kUpt = 1;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
// Every byte is read once and written once: non-temporal loads and stores
// keep the stream from displacing cached data (8-11% faster here).
template <typename T> __device__ inline T ldg(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T> __device__ inline void stg(T v, T* p) { __builtin_nontemporal_store(v, p); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Unsigned division by a run-time constant with a precomputed multiplier
// (round-up method of Granlund & Montgomery, "Division by invariant integers
// using multiplication", 1994): q = (umulhi(n, m) + n) >> s for n < 2^31.
struct FastDiv {
  uint32_t d, m, s;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}

__device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------------------
// Merge (DeDLOC guide, "3. Online Softmax Rescaling Across Decentralized
// Ranks"): with m = max(lse_a, lse_b), w = exp(lse - m):
//   o = (w_a o_a + w_b o_b) / (w_a + w_b), lse = m + ln(w_a + w_b),
// and (0, -inf) passes the other side through unchanged.  V = 4 (D a multiple
// of 4 kMergeUnits, 16-byte aligned rows): a thread handles kMergeUnits
// float4 of one row; otherwise V = 1, one float per thread.
template <int V>
__global__ __launch_bounds__(256) void lse_merge_kernel(uint32_t total, FastDiv per_row, int D,
                                                        const float* __restrict__ o_a,
                                                        const float* __restrict__ lse_a,
                                                        const float* __restrict__ o_b,
                                                        const float* __restrict__ lse_b,
                                                        float* o_out, float* lse_out) {
  // V == 4: tpr = per_row / kMergeUnits threads per row, thread c of a row
  // handles its units c, c + tpr, ... (the row's weights are computed once)
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  const uint32_t tpr = per_row.d / (V == 4 ? kMergeUnits : 1);
  const uint32_t row = V == 4 ? g / tpr : fdiv(g, per_row);
  const uint32_t c0 = g - row * tpr;
  if ((V == 4 ? row * per_row.d : g) >= total) return;
  const float la = lse_a[row], lb = lse_b[row];
  float ca, cb, lo;
  if (la == kNegInf && lb == kNegInf) {
    ca = 0.f; cb = 0.f; lo = kNegInf;
  } else if (la == kNegInf) {
    ca = 0.f; cb = 1.f; lo = lb;
  } else if (lb == kNegInf) {
    ca = 1.f; cb = 0.f; lo = la;
  } else {
    const float m = fmaxf(la, lb);
    const float wa = __builtin_amdgcn_exp2f((la - m) * kLog2e);
    const float wb = __builtin_amdgcn_exp2f((lb - m) * kLog2e);
    const float den = wa + wb;
    ca = wa / den;
    cb = wb / den;
    lo = m + __builtin_amdgcn_logf(den) * kLn2;
  }
  if (V == 4) {
    f32x4v a[kMergeUnits], bb[kMergeUnits];
#pragma unroll
    for (int k = 0; k < kMergeUnits; ++k) {
      const long long off = (long long)row * D + 4 * (c0 + tpr * k);
      a[k] = ldg((const f32x4v*)(o_a + off));
      bb[k] = ldg((const f32x4v*)(o_b + off));
    }
#pragma unroll
    for (int k = 0; k < kMergeUnits; ++k) {
      const long long off = (long long)row * D + 4 * (c0 + tpr * k);
      f32x4v r;
      if (cb == 0.f) r = ca == 0.f ? f32x4v{0.f, 0.f, 0.f, 0.f} : a[k];
      else if (ca == 0.f) r = bb[k];
      else r = ca * a[k] + cb * bb[k];
      stg(r, (f32x4v*)(o_out + off));
    }
    if (c0 == 0) lse_out[row] = lo;
  } else {
    const uint32_t col = g - row * per_row.d;
    const long long off = (long long)row * D + col;
    const float a = o_a[off], b = o_b[off];
    float r;
    if (cb == 0.f) r = ca == 0.f ? 0.f : a;
    else if (ca == 0.f) r = b;
    else r = ca * a + cb * b;
    o_out[off] = r;
    if (col == 0) lse_out[row] = lo;
  }
}

// ---------------------------------------------------------------------------
// Relayout ("Sequence Parallelism II: DeepSpeed Ulysses and All-to-All
// Attention"): destination j owns heads [j Hp, (j+1) Hp), Hp = H / P_u.  Each
// (token, destination) pair moves one contiguous run of Hp*D elements:
//   SEQ2HEAD: in run ((b s_loc + t) P_u + j)  -> out run ((j B + b) s_loc + t)
//   HEAD2SEQ: the reverse.
// Threads walk the OUTPUT in order (coalesced stores); each moves one W-byte
// unit of a run.  SEQ2HEAD's output is destination-major, so blocks taken in
// order would, for a long stretch, all read the same P_u-th of every token's
// row; with `spread` (the grid divided by P_u) block i takes output slot
// (i mod P_u) spread + i / P_u instead, so the blocks in flight read every
// part of the rows (measured 12% faster on [2, 8192, 16, 128], P_u = 8).
template <typename W>
__global__ __launch_bounds__(256) void relayout_kernel(int dir, uint32_t total, FastDiv upr,
                                                       FastDiv s_loc, FastDiv pu, FastDiv bdim, uint32_t spread,
                                                       const W* __restrict__ in, W* __restrict__ out) {
  uint32_t blk = blockIdx.x;
  if (spread) {
    const uint32_t q = fdiv(blk, pu);
    blk = (blk - q * pu.d) * spread + q;
  }
  const uint32_t base = blk * (256u * kUpt) + threadIdx.x;
  W v[kUpt];
#pragma unroll
  for (int k = 0; k < kUpt; ++k) {
    const uint32_t u = base + 256u * k;
    if (u >= total) continue;
    const uint32_t run = fdiv(u, upr);
    const uint32_t e = u - run * upr.d;
    uint32_t src_run;
    if (dir == 0) {
      const uint32_t jb = fdiv(run, s_loc);
      const uint32_t t = run - jb * s_loc.d;
      const uint32_t j = fdiv(jb, bdim);
      const uint32_t b = jb - j * bdim.d;
      src_run = ((b * s_loc.d) + t) * pu.d + j;
    } else {
      const uint32_t bt = fdiv(run, pu);
      const uint32_t j = run - bt * pu.d;
      const uint32_t b = fdiv(bt, s_loc);
      const uint32_t t = bt - b * s_loc.d;
      src_run = (j * bdim.d + b) * s_loc.d + t;
    }
    v[k] = ldg(in + (long long)src_run * upr.d + e);
  }
#pragma unroll
  for (int k = 0; k < kUpt; ++k) {
    const uint32_t u = base + 256u * k;
    if (u < total) stg(v[k], out + u);
  }
}

template <typename W>
hipError_t launch_relayout_w(int dir, uint32_t total, uint32_t units_per_run, int B,
                             long long s_loc, int P_u, const void* in, void* out, hipStream_t s) {
  const uint32_t blocks = (total + 256u * kUpt - 1) / (256u * kUpt);
  const uint32_t spread = (dir == 0 && blocks % (uint32_t)P_u == 0) ? blocks / (uint32_t)P_u : 0u;
  hipLaunchKernelGGL(relayout_kernel<W>, dim3(blocks), dim3(256), 0, s, dir, total,
                     make_fastdiv(units_per_run), make_fastdiv((uint32_t)s_loc),
                     make_fastdiv((uint32_t)P_u), make_fastdiv((uint32_t)B), spread, (const W*)in, (W*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Messages of the Ulysses all-to-all for several tensors at once (the fused
// exchange of ringmaster's Ulysses leg, one collective for K and V, and the
// receive side of "Sequence Parallelism II").  A piece is the message of one
// (source, destination) pair: the tensors' sections one after another, each
// [B, s_loc, run].  Grouping HEADS: tensor i is [B, s_loc, P_u, run_i] and
// piece j holds run j of every token.  Grouping SEQ: tensor i is
// [B, P_u, s_loc, run_i] (global token order, block u from source u) and
// piece u holds block u.  blockIdx.y picks the tensor; threads walk the
// destination in order (coalesced stores), one W-byte unit each; towards the
// pieces the blocks are spread over the destinations as in the relayout.
struct PieceSec {
  const char* src;       // tensor or pieces, by direction
  char* dst;
  uint32_t total;        // units of this tensor
  uint32_t sec;          // units before this section in a piece
  FastDiv run;           // units per run
};

struct PieceArgs {
  PieceSec s[kMaxPieceTensors];
  uint32_t piece;        // units per piece
  FastDiv s_loc, pu, bdim;
  int group, to_pieces;
  uint32_t spread;       // 0, or gridDim.x / P_u: block i takes slot (i mod P_u) spread + i / P_u
};

template <typename W>
__global__ __launch_bounds__(256) void pieces_kernel(PieceArgs a) {
  const PieceSec sc = a.s[blockIdx.y];
  uint32_t blk = blockIdx.x;
  if (a.spread) {
    const uint32_t q = fdiv(blk, a.pu);
    blk = (blk - q * a.pu.d) * a.spread + q;
  }
  const uint32_t base = blk * (256u * kUpt) + threadIdx.x;
  W v[kUpt];
  long long dsts[kUpt];
#pragma unroll
  for (int k = 0; k < kUpt; ++k) {
    const uint32_t u = base + 256u * k;
    if (u >= sc.total) continue;
    const uint32_t r = fdiv(u, sc.run);
    const uint32_t e = u - r * sc.run.d;
    uint32_t j, b, t;
    if (a.to_pieces) {
      const uint32_t jb = fdiv(r, a.s_loc);
      t = r - jb * a.s_loc.d;
      j = fdiv(jb, a.bdim);
      b = jb - j * a.bdim.d;
    } else if (a.group == 0) {
      const uint32_t bt = fdiv(r, a.pu);
      j = r - bt * a.pu.d;
      b = fdiv(bt, a.s_loc);
      t = bt - b * a.s_loc.d;
    } else {
      const uint32_t bj = fdiv(r, a.s_loc);
      t = r - bj * a.s_loc.d;
      b = fdiv(bj, a.pu);
      j = bj - b * a.pu.d;
    }
    const long long piece_u = (long long)j * a.piece + sc.sec + ((long long)b * a.s_loc.d + t) * sc.run.d + e;
    const long long tensor_r = a.group == 0 ? ((long long)b * a.s_loc.d + t) * a.pu.d + j
                                            : ((long long)b * a.pu.d + j) * a.s_loc.d + t;
    const long long tensor_u = tensor_r * sc.run.d + e;
    const long long src = a.to_pieces ? tensor_u : piece_u;
    dsts[k] = a.to_pieces ? piece_u : (long long)u;
    v[k] = ldg((const W*)sc.src + src);
  }
#pragma unroll
  for (int k = 0; k < kUpt; ++k) {
    const uint32_t u = base + 256u * k;
    if (u < sc.total) stg(v[k], (W*)sc.dst + dsts[k]);
  }
}

template <typename W>
hipError_t launch_pieces_w(const PieceArgs& a, int n, uint32_t max_total, hipStream_t s) {
  const dim3 grid((max_total + 256u * kUpt - 1) / (256u * kUpt), (unsigned)n);
  PieceArgs b = a;
  b.spread = (a.to_pieces && grid.x % a.pu.d == 0) ? grid.x / a.pu.d : 0u;
  hipLaunchKernelGGL(pieces_kernel<W>, grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(long long rows, int D, const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                            hipStream_t s) {
  const bool vec = (D % 4) == 0 && ((uintptr_t)o_a % 16) == 0 && ((uintptr_t)o_b % 16) == 0 &&
                   ((uintptr_t)o_out % 16) == 0;
  const bool vec4 = vec && (D / 4) % kMergeUnits == 0;
  const uint32_t per_row = vec4 ? (uint32_t)(D / 4) : (uint32_t)D;
  const uint32_t total = (uint32_t)(rows * per_row);
  const uint32_t threads = vec4 ? total / kMergeUnits : total;
  const uint32_t blocks = (threads + 255u) / 256u;
  if (vec4)
    hipLaunchKernelGGL(lse_merge_kernel<4>, dim3(blocks), dim3(256), 0, s, total,
                       make_fastdiv(per_row), D, o_a, lse_a, o_b, lse_b, o_out, lse_out);
  else
    hipLaunchKernelGGL(lse_merge_kernel<1>, dim3(blocks), dim3(256), 0, s, total,
                       make_fastdiv(per_row), D, o_a, lse_a, o_b, lse_b, o_out, lse_out);
  return hipGetLastError();
}

int relayout_unit(long long run_bytes, const void* in, const void* out) {
  const uintptr_t a = (uintptr_t)in | (uintptr_t)out;
  for (int w = 16; w > 1; w /= 2)
    if (run_bytes % w == 0 && a % w == 0) return w;
  return 1;
}

hipError_t launch_relayout(int dir, int elem_bytes, int B, long long s_loc, int H, int D, int P_u,
                           const void* in, void* out, hipStream_t s) {
  const long long run_bytes = (long long)(H / P_u) * D * elem_bytes;
  const long long runs = (long long)P_u * B * s_loc;
  const int w = relayout_unit(run_bytes, in, out);
  const uint32_t upr = (uint32_t)(run_bytes / w), total = (uint32_t)(runs * upr);
  switch (w) {
    case 16: return launch_relayout_w<u32x4>(dir, total, upr, B, s_loc, P_u, in, out, s);
    case 8: return launch_relayout_w<u32x2>(dir, total, upr, B, s_loc, P_u, in, out, s);
    case 4: return launch_relayout_w<uint32_t>(dir, total, upr, B, s_loc, P_u, in, out, s);
    case 2: return launch_relayout_w<uint16_t>(dir, total, upr, B, s_loc, P_u, in, out, s);
    default: return launch_relayout_w<uint8_t>(dir, total, upr, B, s_loc, P_u, in, out, s);
  }
}

hipError_t launch_pieces(int to_pieces, int group, int B, long long s_loc, int P_u, int n, void* const* tensors,
                         const long long* run_bytes, void* pieces, int unit, hipStream_t s) {
  PieceArgs a = {};
  long long sec = 0, piece = 0;
  for (int i = 0; i < n; ++i) piece += (long long)B * s_loc * run_bytes[i];
  uint32_t max_total = 0;
  for (int i = 0; i < n; ++i) {
    const uint32_t run = (uint32_t)(run_bytes[i] / unit);
    const uint32_t total = (uint32_t)((long long)P_u * B * s_loc * run);
    char* piece_base = (char*)pieces;
    a.s[i].src = to_pieces ? (const char*)tensors[i] : (const char*)piece_base;
    a.s[i].dst = to_pieces ? piece_base : (char*)tensors[i];
    a.s[i].total = total;
    a.s[i].sec = (uint32_t)(sec / unit);
    a.s[i].run = make_fastdiv(run);
    sec += (long long)B * s_loc * run_bytes[i];
    if (total > max_total) max_total = total;
  }
  a.piece = (uint32_t)(piece / unit);
  a.s_loc = make_fastdiv((uint32_t)s_loc);
  a.pu = make_fastdiv((uint32_t)P_u);
  a.bdim = make_fastdiv((uint32_t)B);
  a.group = group;
  a.to_pieces = to_pieces;
  if (max_total == 0) return hipSuccess;
  switch (unit) {
    case 16: return launch_pieces_w<u32x4>(a, n, max_total, s);
    case 8: return launch_pieces_w<u32x2>(a, n, max_total, s);
    case 4: return launch_pieces_w<uint32_t>(a, n, max_total, s);
    case 2: return launch_pieces_w<uint16_t>(a, n, max_total, s);
    default: return launch_pieces_w<uint8_t>(a, n, max_total, s);
  }
}

}  // namespace ra
