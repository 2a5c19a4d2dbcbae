// Device code shared by the attention step kernels: wave reductions, the key
// tile plan of a work item, the work-item decode and the epilogue that stores
// (INIT) or merges (ACCUM) a work item's normalised output and log-sum-exp.
//
// Accumulator layout used throughout: a 32x32 MFMA accumulator puts row
// 8(r/4) + 4(l/32) + r%4, column l%32 in register r of lane l.  The kernels
// compute transposed products, so a column is a query row and each lane owns
// one query of every 32-row block (lanes l and l+32 share it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

#define RA_LDS __attribute__((address_space(3)))

namespace ra {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The reference maximum of a row only moves when probabilities would exceed
// 2^kTau, so most tiles skip the rescale of O; the final division by the row
// sum makes the result independent of where the reference sits.
constexpr float kTau = 8.0f;
constexpr float kTauSum = 256.0f;  // 2^kTau
// A reference (in log2 units) for a row that has seen no visible key yet: any
// finite score is more than kTau above it, and exp2 of its distance to any
// such score is 0, while a masked score's exponent stays -inf (no inf - inf).
constexpr float kMbNone = -0x1p100f;

__device__ inline float max_halves(float x) {
  // v_permlane32_swap with both operands x: every lane sees x of lane ^ 32 in
  // one of the two results; max/sum of both is symmetric.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline u32x4 lds_load16(const RA_LDS char* base, unsigned off) {
  return *(const RA_LDS u32x4*)(base + off);
}

// ---------------------------------------------------------------------------
// Key tiles of one work item.  Tiles restart at each key span.  Within a span
// the tiles whose keys are all visible to every query row of the work item
// come first and run no mask code; the rest (on the causal diagonal, or cut
// short by the span's end) follow and are masked.  The order of the tiles does
// not change the result.
struct KTile {
  long long local0;  // first local key row
  long long glob0;   // its global position
  int count;         // rows that exist and may be visible (<= kBK)
};

struct TilePlan {
  // Per key span, in tiles of kBK keys counted from the span's first key:
  // unmasked tiles [fb, fb + nf), masked tiles below them [lb, lb + nlo)
  // (a sliding window's or a packed sequence's left edge) and above them
  // [hb, hb + nr) (the causal diagonal, a span's ragged end).
  int fb[2], nf[2], lb[2], nlo[2], hb[2], nr[2];
  long long hi[2];     // keys of the span visible to some row of the work item: [0, hi)
  long long off[2];    // first local row of each key span
  long long start[2];  // its global position
  int n_full, n;

  // Tile t in plan order, for plans without masked tiles below the unmasked
  // ones (no window, no packed sequences).  Only selects between the two
  // spans: no indexing by a run-time span number, which would re-read the
  // kernel arguments on every tile.
  __device__ KTile tile(int t) const {
    bool s1;
    long long kin;
    if (t < n_full) {
      s1 = t >= nf[0];
      kin = (long long)(s1 ? t - nf[0] : t) * kBK;
    } else {
      const int u = t - n_full;
      s1 = u >= nr[0];
      kin = (long long)(s1 ? nf[1] + u - nr[0] : nf[0] + u) * kBK;
    }
    KTile kt;
    kt.local0 = (s1 ? off[1] : off[0]) + kin;
    kt.glob0 = (s1 ? start[1] : start[0]) + kin;
    kt.count = (int)min((long long)kBK, (s1 ? hi[1] : hi[0]) - kin);
    return kt;
  }
};

// Packed sequences: boundaries cu[0] = 0 < cu[1] < ... < cu[nseg] (global
// positions).  Index of the sequence holding t.
__device__ inline int seg_of(const StepParams& p, long long t) {
  int lo = 0, hi = p.nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Keys visible to the query at global position t: [key_lo(t), key_hi(t)].
// Both are non-decreasing in t, so a run of rows r0..r1 sees keys
// [key_lo(r0), key_hi(r1)] and every one of them sees [key_lo(r1), key_hi(r0)].
__device__ inline long long key_lo(const StepParams& p, long long t) {
  long long lo = p.window > 0 ? t - p.window + 1 : 0;
  if (p.cu) lo = max(lo, p.cu[seg_of(p, t)]);
  return lo;
}
__device__ inline long long key_hi(const StepParams& p, long long t) {
  if (p.causal) return t;
  if (p.cu) return p.cu[seg_of(p, t) + 1] - 1;
  return 0x3fffffffffffffffLL;
}

// Rows that see some key of [k0, k1] (global positions):
// key_hi and key_lo never decrease along the rows, so they are the rows t
// with key_hi(t) >= k0 and key_lo(t) <= k1, one interval [t0, t1].
__device__ inline void rows_seeing(const StepParams& p, long long k0, long long k1, long long& t0, long long& t1) {
  t0 = p.causal ? k0 : (p.cu ? p.cu[seg_of(p, k0)] : 0);
  t1 = 0x3fffffffffffffffLL;
  if (p.window > 0) t1 = k1 + p.window - 1;
  if (p.cu) t1 = min(t1, p.cu[seg_of(p, k1) + 1] - 1);
}

__device__ inline TilePlan plan_tiles(const StepParams& p, long long qglob0, long long qglob_last) {
  TilePlan tp;
  tp.n_full = 0;
  tp.n = 0;
  const long long lo0 = key_lo(p, qglob0), lo1 = key_lo(p, qglob_last);
  const long long hi0 = key_hi(p, qglob0), hi1 = key_hi(p, qglob_last);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    long long v0 = 0, v1 = 0, f0 = 0, f1 = 0;
    if (s < p.nks) {
      const long long ks = p.ks_start[s], len = p.ks_len[s];
      v0 = min(max(lo0 - ks, 0LL), len);
      v1 = min(max(hi1 - ks + 1, 0LL), len);
      f0 = min(max(lo1 - ks, 0LL), len);
      f1 = min(max(hi0 - ks + 1, 0LL), len);
    }
    int fb = 0, nf = 0, lb = 0, nlo = 0, hb = 0, nr = 0;
    if (v1 > v0) {
      const int lt = (int)(v0 / kBK), ht = (int)((v1 + kBK - 1) / kBK);
      const int ff = (int)((f0 + kBK - 1) / kBK), fe = (int)(f1 / kBK);
      if (fe > ff) {
        fb = ff;
        nf = fe - ff;
        lb = lt;
        nlo = ff - lt;
        hb = fe;
        nr = ht - fe;
      } else {
        fb = lt;
        lb = lt;
        hb = lt;
        nr = ht - lt;
      }
    }
    tp.fb[s] = fb;
    tp.nf[s] = nf;
    tp.lb[s] = lb;
    tp.nlo[s] = nlo;
    tp.hb[s] = hb;
    tp.nr[s] = nr;
    tp.hi[s] = v1;
    tp.off[s] = p.ks_off[s];
    tp.start[s] = p.ks_start[s];
    tp.n_full += nf;
    tp.n += nf + nlo + nr;
  }
  return tp;
}

// Row order in which a wave feeds the 32 rows of an MFMA A operand: sigma
// swaps bits 2 and 3 of the row index.  Fed so, register r of lane l of the
// 32x32 accumulator holds row 16(r/8) + 8(l/32) + r%8, which puts rows
// 16h .. 16h+15 in registers 8h .. 8h+7 in natural order: the layout of the
// B operand of a 32x32x16 MFMA that reduces over those rows.
__device__ inline unsigned sigma(unsigned i) { return (i & ~12u) | ((i & 4u) << 1) | ((i & 8u) >> 1); }

// Word 3 of a buffer resource for raw, unswizzled 32-bit-addressed loads.  A
// record that ends with the last row a tile may see makes loads of rows past
// a span's ragged end return 0 and never leave the tensor.
constexpr int kRsrcWord3 = 0x00020000;

// Walks the key tiles of a work item in the order the tile plan fixes (the
// unmasked tiles of each span, then the masked ones), one scalar update per
// tile; only the first tile of a segment recomputes from the plan.
struct TileCursor {
  long long local0, glob0;  // first local row of the tile, its global position
  long long vis;            // rows of the span visible from local0 on
  int rem;                  // tiles left in the segment, this one included
  int seg;                  // 0, 1: unmasked tiles of span 0, 1; 2, 3: masked
                            // below them; 4, 5: masked above them

  __device__ int count() const { return (int)min((long long)kBK, vis); }
  __device__ bool masked() const { return seg >= 2; }

  __device__ bool enter(const TilePlan& tp, int j) {
    // selects only: a run-time index into the plan's arrays would put the
    // plan in scratch memory
    const bool s = j & 1;
    int n, t0;
    if (j < 2) {
      n = s ? tp.nf[1] : tp.nf[0];
      t0 = s ? tp.fb[1] : tp.fb[0];
    } else if (j < 4) {
      n = s ? tp.nlo[1] : tp.nlo[0];
      t0 = s ? tp.lb[1] : tp.lb[0];
    } else {
      n = s ? tp.nr[1] : tp.nr[0];
      t0 = s ? tp.hb[1] : tp.hb[0];
    }
    if (n == 0) return false;
    const long long kin = (long long)t0 * kBK;
    local0 = (s ? tp.off[1] : tp.off[0]) + kin;
    glob0 = (s ? tp.start[1] : tp.start[0]) + kin;
    vis = (s ? tp.hi[1] : tp.hi[0]) - kin;
    rem = n;
    seg = j;
    return true;
  }
  // The segment loops are unrolled so that every enter() sees a constant j:
  // with a run-time j the compiler turns the selects back into indexing.
  __device__ void first(const TilePlan& tp) {
#pragma unroll
    for (int j = 0; j < 6; ++j)
      if (enter(tp, j)) return;
  }
  __device__ void advance(const TilePlan& tp) {
    if (rem > 1) {
      --rem;
      local0 += kBK;
      glob0 += kBK;
      vis -= kBK;
      return;
    }
#pragma unroll
    for (int j = 1; j < 6; ++j)
      if (j > seg && enter(tp, j)) return;
  }
  // tile idx (< tp.n) of the plan order
  __device__ void seek(const TilePlan& tp, int idx) {
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      if (!enter(tp, j)) continue;
      if (idx < rem) {
        rem -= idx;
        local0 += (long long)idx * kBK;
        glob0 += (long long)idx * kBK;
        vis -= (long long)idx * kBK;
        return;
      }
      idx -= rem;
    }
  }
};

// ---------------------------------------------------------------------------
// Work item of a workgroup: BQ consecutive query rows of one (batch, query
// head).  XCD x (= block id mod 8, dispatch is round-robin over the 8 XCDs)
// takes a contiguous run of work items, ordered kv-head major so the query
// tiles that read one K/V head share that XCD's L2, heavier (later) query
// tiles first.
struct WorkItem {
  int b, g, h;
  int qrows;            // rows of the work item that exist (<= BQ)
  long long qlocal0;    // first local query row
  long long qglob0;     // its global position
};

template <int BQ>
__device__ inline bool decode_work(const StepParams& p, WorkItem& wi) {
  // Workgroup i runs on XCD i mod 8; XCD x takes items [x per_xcd,
  // (x+1) per_xcd) of the list (heads outer, then query tiles, heaviest end
  // first: the last tiles for causal rows, the first ones when the host finds
  // them heavier, as for a window over an earlier block), so
  // that a head's K/V stays in one L2.  When that range is whole heads (lpt),
  // the XCD walks it tile-major instead: the last (for causal rows the
  // heaviest) tile of every head first, which evens out the finish times of
  // its CUs on diagonal blocks.
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  int w = x * p.per_xcd + j;
  if (p.lpt) {
    const int nb = p.per_xcd / p.n_qtiles;  // heads per XCD
    w = (x * nb + j % nb) * p.n_qtiles + j / nb;
  }
  if (w >= p.n_work) return false;
  const int qt_rev = w % p.n_qtiles;
  int rest = w / p.n_qtiles;
  const int hh = rest % p.G;
  rest /= p.G;
  wi.g = rest % p.Hkv;
  wi.b = rest / p.Hkv;
  wi.h = wi.g * p.G + hh;
  const int qt = p.first_heavy ? qt_rev : p.n_qtiles - 1 - qt_rev;
  const int qs = qt < p.qt_span0 ? 0 : 1;
  const long long q_in = (long long)(qs ? qt - p.qt_span0 : qt) * BQ;
  wi.qrows = (int)min((long long)BQ, p.qs_len[qs] - q_in);
  wi.qlocal0 = p.qs_off[qs] + q_in;
  wi.qglob0 = p.qs_start[qs] + q_in;
  return true;
}

// INIT of a work item whose rows see no key of the block: the merge identity
// (O = 0, LSE = -inf).  ACCUM leaves such rows untouched.
template <int D, int THREADS>
__device__ inline void store_identity(const StepParams& p, const WorkItem& wi) {
  if (p.accum) return;
  for (int i = threadIdx.x; i < wi.qrows * (D / 4); i += THREADS) {
    const int r = i / (D / 4), c = i % (D / 4);
    const long long orr = ((long long)wi.b * p.Sq + wi.qlocal0 + r) * p.Hq + wi.h;
    *(float4*)(p.o + orr * D + 4 * c) = float4{0.f, 0.f, 0.f, 0.f};
    if (c == 0) p.lse[orr] = kNegInf;
  }
}

// Epilogue of 32-row block qb held by a wave: O^T accumulators oq[D/32][qb]
// (already complete over the block's keys), the reference maximum mb of the
// scores in log2 units (raw maximum times scale log2(e)) and this lane's
// share of the row sum.  INIT stores O / l and
// the LSE; ACCUM merges them into the (O, LSE) already in HBM (a stored LSE of
// -inf is the identity and is replaced); a row that saw no visible key stores
// the identity in INIT and is left alone in ACCUM.
template <int D, int NQB>
__device__ inline void finish_rows(const StepParams& p, const f32x16 (*oq)[NQB], int qb, float mb, float l_part,
                                   bool row_ok, long long orow, int lane) {
  const int dsub = 4 * (lane >> 5);
  const float l_tot = sum_halves(l_part);
  if (!row_ok) return;
  float* orow_ptr = p.o + orow * D;
  if (l_tot > 0.f) {
    const float inv = 1.f / l_tot;
    const float lse_s = (mb + __builtin_amdgcn_logf(l_tot)) * kLn2;
    float lse_r = kNegInf;
    if (p.accum) lse_r = p.lse[orow];
    if (lse_r == kNegInf) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& a = oq[db][qb];
          const float4 v = {a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv};
          *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = v;
        }
      if (lane < 32) p.lse[orow] = lse_s;
    } else {
      const float m = fmaxf(lse_r, lse_s);
      const float wr = __builtin_amdgcn_exp2f((lse_r - m) * kLog2e);
      const float wsum = __builtin_amdgcn_exp2f((lse_s - m) * kLog2e);
      const float den = wr + wsum;
      const float cr = wr / den;
      const float cs = wsum / den * inv;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& a = oq[db][qb];
          float* ptr = orow_ptr + 32 * db + 8 * j + dsub;
          const float4 r = *(const float4*)ptr;
          const float4 v = {cr * r.x + cs * a[4 * j], cr * r.y + cs * a[4 * j + 1], cr * r.z + cs * a[4 * j + 2],
                            cr * r.w + cs * a[4 * j + 3]};
          *(float4*)ptr = v;
        }
      if (lane < 32) p.lse[orow] = m + __builtin_amdgcn_logf(den) * kLn2;
    }
  } else if (!p.accum) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = float4{0.f, 0.f, 0.f, 0.f};
    if (lane < 32) p.lse[orow] = kNegInf;
  }
}

}  // namespace dev
}  // namespace ra
