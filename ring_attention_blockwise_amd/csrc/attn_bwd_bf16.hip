// Backward of one ring step of blockwise attention on gfx950, bf16 inputs,
// head dimension 128.
//
// What it computes: the gradient of sum(dO * O) for O = softmax(scale q K^T) V
// over the visible keys of the step's key/value block, with the forward's
// final log-sum-exp L of every query row: P = exp(scale q K^T - L) is then the
// exact softmax weight of the whole sequence, so each step's share is exact
// and the shares add up.  ringmaster's description asks for this backward on
// the p2p ring, flash style, with the ring run in reverse ("Status", Ring row;
// its note on the two Ring paths under "Why"); the formulas are the chain rule
// through the softmax:
//   dP = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O),
//   dQ += scale dS K,  dK += scale dS^T Q,  dV += P^T dO,
// with the G query heads of a group adding into their shared K/V head.
//
// The kernels; in none of them do two workgroups add into the same rows:
//   * dQ: a workgroup (4 waves) owns 128 query rows of one (batch, query
//     head), 32 per wave, and walks the step's key tiles like the forward
//     kernel: S^T = K Q^T and dP^T = V dO^T (K, V rows from LDS, Q^T and dO^T
//     in registers), then dQ^T += K^T dS^T with K^T gathered by transposing
//     LDS reads.
//   * dK and dV in one launch (the default): an eight-wave workgroup owns
//     128 keys of one (batch, kv head) and walks the query tiles (32 rows) of
//     every query head of the group that see them; waves w and w + 4 share
//     keys 32w .. 32w + 31, with K^T or V^T in registers for the whole item.
//     The four products of a (query tile, key tile) pair on this side (the
//     dQ kernel takes the other three) are split two and two between the two
//     waves of a SIMD: waves 0..3 form S = Q K^T and P (P to LDS as bf16) and
//     add dK^T += Q^T dS; waves 4..7 form dP - delta = dO V^T - delta (to LDS
//     as float32) and add dV^T += dO^T P, each using the other group's result
//     of the previous query tile, so the groups meet only at the one barrier
//     per tile.  One wave holding both accumulators
//     would need about 290 registers (one wave per SIMD); split over two
//     waves of a SIMD they fit.
//   * dV and dK, separate (two kernels of one template), for launches whose
//     key tiles would not give every CU a workgroup: the same walk, S formed
//     in both; eight-wave workgroups let two groups of four waves share a key
//     tile's query tiles, the second handing its partial sums to the first
//     through LDS.
// The softmax rows are spread over the accumulator registers in the dK/dV
// kernels, so the rows' L and delta come from LDS as 16 values per lane.
// Tiles are copied global -> LDS by buffer loads with the LDS bit.  One LDS
// layout serves both read patterns: chunk c of row r sits at c ^ csw(r), with
// csw(r) = 4 (r mod 4) + (r / 4) mod 4, which keeps the 16 rows of a row read
// and the 4 rows x 4 chunks of a transposing read in distinct banks.
#include "attn_common.h"

namespace ra {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kD = 128;

// Tag for the two instantiations of a tile body, with and without the
// per-row key-range select.
template <bool B>
struct KvbSel {
  static constexpr bool value = B;
};
constexpr int kThreads = 256;
constexpr int kRowB = 2 * kD;               // bytes of one bf16 row
constexpr int kTileB = 32 * kRowB;          // a 32-row tile
static_assert(kBK == 32, "32-row key tiles");

__device__ inline unsigned csw(unsigned r) { return ((r & 3u) << 2) | ((r >> 2) & 3u); }

// A-operand row read of unit u (16 columns): row_base ^ 32u, rows sigma(l%32).
__device__ inline unsigned row_base_sigma(unsigned lane) {
  const unsigned rho = sigma(lane & 31u);
  return rho * kRowB + 16u * (csw(rho) ^ (lane >> 5));
}
// B-operand row read of unit u: row l%32 in natural order.
__device__ inline unsigned row_base_plain(unsigned lane) {
  const unsigned r = lane & 31u;
  return r * kRowB + 16u * (csw(r) ^ (lane >> 5));
}
// Transposing reads: lane s of 16-lane group g reads row 8(g/2) + s/4 (b0)
// and the row 4 below (b1) at column 32 db + 16 (g%2) + 4 (s%4); block db is
// at b ^ 64 db and rows 16 further down at + 16 kRowB (csw repeats every 16).
__device__ inline void tr_bases(unsigned lane, unsigned& b0, unsigned& b1) {
  const unsigned g = lane >> 4, s = lane & 15u;
  const unsigned r = 8u * (g >> 1) + (s >> 2);
  const unsigned x = 2u * (g & 1u) + ((s & 3u) >> 1);
  const unsigned e = 8u * (s & 1u);
  b0 = r * kRowB + 16u * (x ^ csw(r)) + e;
  b1 = (r + 4u) * kRowB + 16u * (x ^ csw(r + 4u)) + e;
}
__device__ inline bf16x8 tr_read(RA_LDS char* tile, unsigned b0, unsigned b1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(tile + b0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(tile + b1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Tile offset (in the tensor) of the chunk a lane copies with DMA
// instruction i of wave w (2 instructions of 1 KiB per wave fill 32 rows).
__device__ inline unsigned dma_off(int w, int i, unsigned lane, unsigned row_bytes) {
  const unsigned slot = (unsigned)(w * 2 + i) * 64u + lane;
  const unsigned r = slot >> 4;
  return r * row_bytes + 16u * ((slot & 15u) ^ csw(r));
}

__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline float neg_inf_select(int d, float x) {
  // x if d >= 0, else -inf (sign bit of d, no compare masks)
  asm volatile("" : "+v"(d));
  const unsigned m = (unsigned)(d >> 31);
  return __uint_as_float((m & 0xff800000u) | (~m & __float_as_uint(x)));
}

// ===========================================================================
// dQ kernel
struct DqStage {
  const char* khead;
  const char* vhead;
  unsigned row_bytes;
  unsigned off[2];
  int wave;

  __device__ void init(const StepParams& p, const WorkItem& wi, int w, unsigned lane) {
    row_bytes = (unsigned)(p.Hkv * kRowB);
    const long long head = ((long long)wi.b * p.Sk * p.Hkv + wi.g) * (long long)kRowB;
    khead = (const char*)p.k + head;
    vhead = (const char*)p.v + head;
    wave = w;
    off[0] = dma_off(w, 0, lane, row_bytes);
    off[1] = dma_off(w, 1, lane, row_bytes);
  }
  __device__ void issue(const TileCursor& c, RA_LDS char* kdst, RA_LDS char* vdst) const {
    const long long o = c.local0 * (long long)row_bytes;
    const int nrec = (c.count() - 1) * (int)row_bytes + kRowB;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(khead + o), (short)0, nrec, kRsrcWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vhead + o), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (RA_LDS void*)(kdst + (wave * 2 + i) * 1024), 16, (int)off[i], 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (RA_LDS void*)(vdst + (wave * 2 + i) * 1024), 16, (int)off[i], 0,
                                               0, 0);
    }
  }
};

struct DqState {
  bf16x8 q[kD / 16];    // Q^T operand: Q[row][16u + 8(l/32) .. +7]
  bf16x8 d[kD / 16];    // dO^T operand, same layout
  f32x16 acc[kD / 32];  // dQ^T accumulators
  float lse2;           // L * log2(e) of the lane's row (+inf: the row has no weight)
  f32x16 ndl;           // -delta of the lane's row (the workspace's value) in
                        // every element: dP^T's starting value, so the chain
                        // yields dP - delta
};

template <int PAR, bool kExt>
__device__ inline void dq_tile(DqState& st, const BwdParams& bp, const TilePlan& tp, const WorkItem& wi,
                               const DqStage& stg, TileCursor& cur, int t, RA_LDS char* const* kbuf,
                               RA_LDS char* const* vbuf, const RA_LDS int* row_lo, const RA_LDS int* row_hi,
                               unsigned lane, int wave) {
  const StepParams& p = bp.s;
  const TileCursor ti = cur;
  // issue priority swapped every 32 tiles, in opposite phase for the two
  // workgroups sharing a CU, as in the forward step kernel (the older wave
  // would otherwise run ahead and finish long before the younger): -1.1%
  // on the 131k backward
  if ((((unsigned)t >> 5) ^ (blockIdx.x >> 8)) & 1u)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
  if (t + 1 < tp.n) {
    cur.advance(tp);
    stg.issue(cur, kbuf[PAR ^ 1], vbuf[PAR ^ 1]);
  }
  const unsigned rb = row_base_sigma(lane);
  // S^T = K Q^T and dP^T - delta = V dO^T - delta (the chain starts from -delta)
  f32x16 s = f32x16{}, dp = st.ndl;
#pragma unroll
  for (int u = 0; u < kD / 16; ++u) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(kbuf[PAR], rb ^ (32u * u)));
    const bf16x8 b = __builtin_bit_cast(bf16x8, lds_load16(vbuf[PAR], rb ^ (32u * u)));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.q[u], s, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, st.d[u], dp, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int L = (int)(lane >> 5);
  if (ti.masked()) {
    // key 16(r/8) + 8L + r%8 of the tile is visible to the lane's row iff it
    // is below lim
    const long long d0 = wi.qglob0 - ti.glob0 + 1;
    const int dc = p.causal ? (int)max(-1024LL, min(1024LL, d0)) : 1024;
    const int ri = 32 * wave + (int)(lane & 31u);
    int lim = min(ti.count(), max(0, dc + ri));
    // window, packed sequences: the row's key range [lo, hi] from LDS
    const int base = kExt ? (int)max(-(1LL << 30), min(1LL << 30, ti.glob0 - wi.qglob0)) : 0;
    if (kExt) lim = max(0, min(ti.count(), row_hi[ri] + 1 - base));
    const int lim_l = lim - 8 * L - 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = neg_inf_select(lim_l - (16 * (r >> 3) + (r & 7)), s[r]);
    if (kExt) {
      const int lo_l = 8 * L - max(-1, min(33, row_lo[ri] - base));
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = neg_inf_select(lo_l + (16 * (r >> 3) + (r & 7)), s[r]);
    }
  }
  // P^T = exp2(S^T sl2 - L log2 e); dS^T = P^T (dP^T - delta), rounded to bf16
  // (dp holds dP^T - delta already)
  bf16x8 dsb[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hf + e], p.sl2, -st.lse2));
      x[e] = pr * dp[8 * hf + e];
    }
    dsb[hf] = __builtin_convertvector(x, bf16x8);
  }
  __builtin_amdgcn_sched_barrier(0);
  // dQ^T += K^T dS^T
  unsigned b0, b1;
  tr_bases(lane, b0, b1);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
      const bf16x8 a = tr_read(kbuf[PAR], (b0 ^ (64u * db)) + 16u * kRowB * hf, (b1 ^ (64u * db)) + 16u * kRowB * hf);
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[hf], st.acc[db], 0, 0, 0);
    }
  wait_loads();
  __syncthreads();
}

template <bool kExt>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdParams bp) {
  const StepParams& p = bp.s;
  __shared__ __attribute__((aligned(16))) char k0_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char k1_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char v0_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char v1_raw[kTileB];
  RA_LDS char* const kbuf[2] = {(RA_LDS char*)k0_raw, (RA_LDS char*)k1_raw};
  RA_LDS char* const vbuf[2] = {(RA_LDS char*)v0_raw, (RA_LDS char*)v1_raw};
  __shared__ int lo_raw[kBwdRows], hi_raw[kBwdRows];
  const RA_LDS int* row_lo = (const RA_LDS int*)lo_raw;
  const RA_LDS int* row_hi = (const RA_LDS int*)hi_raw;
  const unsigned lane = threadIdx.x & 63u;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  WorkItem wi;
  if (!decode_work<kBwdRows>(p, wi)) return;
  const int row = 32 * wave + (int)(lane & 31u);
  const bool row_ok = row < wi.qrows;
  const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + row) * p.Hq + wi.h;  // (b, row, h)
  const int dsub = 4 * (int)(lane >> 5);
  const TilePlan tp = plan_tiles(p, wi.qglob0, wi.qglob0 + wi.qrows - 1);
  if (tp.n == 0) {
    if (!p.accum && row_ok) {
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) *(float4*)(bp.dq + orow * kD + 32 * db + 8 * j + dsub) = float4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }

  if (kExt) {
    // visible key range of each row of the work item, relative to its first
    // row (read after the barrier below)
    for (int r = threadIdx.x; r < kBwdRows; r += kThreads) {
      const long long tq = wi.qglob0 + r;
      lo_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_lo(p, tq) - wi.qglob0));
      hi_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_hi(p, tq) - wi.qglob0));
    }
  }

  DqStage stg;
  stg.init(p, wi, wave, lane);
  TileCursor cur;
  cur.first(tp);
  stg.issue(cur, kbuf[0], vbuf[0]);

  DqState st;
  {
    const uint16_t* qrow = (const uint16_t*)p.q + orow * kD;
    const uint16_t* drow = (const uint16_t*)bp.dout + orow * kD;
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      st.q[u] = row_ok ? *(const bf16x8*)(qrow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
      st.d[u] = row_ok ? *(const bf16x8*)(drow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
    }
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) st.acc[db] = f32x16{};
    const float l = row_ok ? bp.lse[orow] : kNegInf;
    st.lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    const float ndl = row_ok ? bp.delta[orow] : 0.f;  // the workspace holds -delta
#pragma unroll
    for (int e = 0; e < 16; ++e) st.ndl[e] = ndl;
  }
  wait_loads();
  __syncthreads();

  int t = 0;
  for (; t + 1 < tp.n; t += 2) {
    dq_tile<0, kExt>(st, bp, tp, wi, stg, cur, t, kbuf, vbuf, row_lo, row_hi, lane, wave);
    dq_tile<1, kExt>(st, bp, tp, wi, stg, cur, t + 1, kbuf, vbuf, row_lo, row_hi, lane, wave);
  }
  if (t < tp.n) dq_tile<0, kExt>(st, bp, tp, wi, stg, cur, t, kbuf, vbuf, row_lo, row_hi, lane, wave);

  if (!row_ok) return;
  float* dst = bp.dq + orow * kD;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16& a = st.acc[db];
      float4 v = {a[4 * j] * p.scale, a[4 * j + 1] * p.scale, a[4 * j + 2] * p.scale, a[4 * j + 3] * p.scale};
      float* ptr = dst + 32 * db + 8 * j + dsub;
      if (p.accum) {
        const float4 r = *(const float4*)ptr;
        v.x += r.x;
        v.y += r.y;
        v.z += r.z;
        v.w += r.w;
      }
      *(float4*)ptr = v;
    }
}

// ===========================================================================
// dK/dV kernel

// Query tiles (32 rows) of every head of the group that see a key tile: per
// query span, the tiles from the first row at or after the tile's first key
// (causal) to the span's end.
struct QPlan {
  int tbeg[2], tend[2];  // tile range per span
  int per_head;          // tiles per query head
  int n;                 // G * per_head
};

struct QCursor {
  int hh;       // query head within the group
  int span;     // 0 or 1
  int tile;     // tile index within the span
  __device__ void first(const QPlan& qp) {
    hh = 0;
    span = qp.tend[0] > qp.tbeg[0] ? 0 : 1;
    tile = span ? qp.tbeg[1] : qp.tbeg[0];
  }
  // tile `idx` of the list (heads outer, then spans, then tiles)
  __device__ void seek(const QPlan& qp, int idx) {
    hh = idx / qp.per_head;
    const int r = idx - hh * qp.per_head;
    const int n0 = qp.tend[0] - qp.tbeg[0];
    span = r < n0 ? 0 : 1;
    tile = span ? qp.tbeg[1] + (r - n0) : qp.tbeg[0] + r;
  }
  __device__ void advance(const QPlan& qp) {
    ++tile;
    const int end = span ? qp.tend[1] : qp.tend[0];
    if (tile < end) return;
    if (span == 0 && qp.tend[1] > qp.tbeg[1]) {
      span = 1;
      tile = qp.tbeg[1];
      return;
    }
    ++hh;
    span = qp.tend[0] > qp.tbeg[0] ? 0 : 1;
    tile = span ? qp.tbeg[1] : qp.tbeg[0];
  }
};

struct KvItem {
  int b, g;
  int kcount;            // keys of the item that exist (<= kBwdKeys)
  long long klocal0;     // first local key row
  long long kglob0;      // its global position
};

__device__ inline bool decode_kv(const BwdParams& bp, KvItem& it) {
  const StepParams& p = bp.s;
  const int w = (blockIdx.x & 7) * bp.per_xcd_kv + (blockIdx.x >> 3);
  if (w >= bp.n_kwork) return false;
  const int kt = w % bp.n_ktiles;  // earlier keys first: causal rows see them most
  const int rest = w / bp.n_ktiles;
  it.g = rest % p.Hkv;
  it.b = rest / p.Hkv;
  const int ks = kt < bp.kt_span0 ? 0 : 1;
  const long long k_in = (long long)(ks ? kt - bp.kt_span0 : kt) * kBwdKeys;
  it.kcount = (int)min((long long)kBwdKeys, p.ks_len[ks] - k_in);
  it.klocal0 = p.ks_off[ks] + k_in;
  it.kglob0 = p.ks_start[ks] + k_in;
  return true;
}

__device__ inline QPlan plan_q(const StepParams& p, long long kglob0, int kcount) {
  QPlan qp;
  qp.per_head = 0;
  long long t0, t1;
  rows_seeing(p, kglob0, kglob0 + kcount - 1, t0, t1);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    int b = 0, e = 0;
    if (s < p.nqs) {
      const long long len = p.qs_len[s];
      const long long first = max(0LL, t0 - p.qs_start[s]);
      const long long last = min(len - 1, t1 - p.qs_start[s]);
      if (first <= last) {
        b = (int)(first / 32);
        e = (int)(last / 32 + 1);
      }
    }
    qp.tbeg[s] = b;
    qp.tend[s] = e;
    qp.per_head += e - b;
  }
  qp.n = p.G * qp.per_head;
  return qp;
}

struct KvStage {
  const char* qbase;     // row 0 of (batch b, query head 0) in Q
  const char* dbase;     // same in dO
  const float* lbase;    // (b, row 0, head 0) in L
  const float* tbase;    // same in delta
  unsigned row_bytes;    // Hq * 2D
  unsigned off[2];
  int wave, Hq;

  __device__ void init(const BwdParams& bp, const KvItem& it, int w, unsigned lane) {
    const StepParams& p = bp.s;
    Hq = p.Hq;
    row_bytes = (unsigned)(p.Hq * kRowB);
    const long long base = (long long)it.b * p.Sq * p.Hq;
    qbase = (const char*)p.q + base * kRowB;
    dbase = (const char*)bp.dout + base * kRowB;
    lbase = bp.lse + base;
    tbase = bp.delta + base;
    wave = w;
    off[0] = dma_off(w, 0, lane, row_bytes);
    off[1] = dma_off(w, 1, lane, row_bytes);
  }
  // Query tile `c` of head h: 32 rows of Q and dO, and L, delta of the rows
  // (lanes 0..63 of one 4-byte copy each; rows past the tile's end read 0).
  template <bool kExt>
  __device__ void issue(const StepParams& p, const QPlan& qp, const QCursor& c, int g, unsigned lane,
                        RA_LDS char* qdst, RA_LDS char* ddst, RA_LDS char* ldst) const {
    (void)qp;
    const int h = g * p.G + c.hh;
    const long long qin = (long long)c.tile * 32;
    const long long local0 = (c.span ? p.qs_off[1] : p.qs_off[0]) + qin;
    const int count = (int)min(32LL, (c.span ? p.qs_len[1] : p.qs_len[0]) - qin);
    const long long o = local0 * (long long)row_bytes + (long long)h * kRowB;
    const int nrec = (count - 1) * (int)row_bytes + kRowB;
    const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(qbase + o), (short)0, nrec, kRsrcWord3);
    const auto rd = __builtin_amdgcn_make_buffer_rsrc((void*)(dbase + o), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (RA_LDS void*)(qdst + (wave * 2 + i) * 1024), 16, (int)off[i], 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (RA_LDS void*)(ddst + (wave * 2 + i) * 1024), 16, (int)off[i], 0,
                                               0, 0);
    }
    if (wave < 2) {
      // wave 0: L of rows 0..63 into ldst[0, 256); wave 1: delta into [256, 512)
      const float* src = (wave == 0 ? lbase : tbase) + local0 * Hq + h;
      const int nr = ((count - 1) * Hq + 1) * 4;
      const auto rl = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nr, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (RA_LDS void*)(ldst + wave * 256), 4,
                                               (int)(lane * (unsigned)Hq * 4u), 0, 0, 0);
    } else if (kExt && lane < 32) {
      // masks: key range [lo, hi] of each row, relative to the tile's first
      // row (wave 2: lo, wave 3: hi), at ldst[512, 768)
      const long long qg = (c.span ? p.qs_start[1] : p.qs_start[0]) + (long long)c.tile * 32;
      const long long v = wave == 2 ? key_lo(p, qg + lane) : key_hi(p, qg + lane);
      ((RA_LDS int*)(ldst + 512))[(wave - 2) * 32 + lane] = (int)max(-(1LL << 30), min(1LL << 30, v - qg));
    }
  }
};

// kDK = false: dV^T += dO^T P (needs S only); kDK = true: dK^T += Q^T dS
// (needs S and dP).  Two kernels instead of one keep each within 256
// registers, so two waves share every SIMD.
template <bool kDK>
struct KvState {
  bf16x8 k[kD / 16];               // K^T operand: K[key l%32][16u + 8(l/32) .. +7]
  bf16x8 v[kDK ? kD / 16 : 1];     // V^T operand, same layout (dP = dO V^T)
  f32x16 acc[kD / 32];             // dK^T or dV^T accumulators
};

// Tile t of the list from buffers CUR while tile t+1 is copied into NXT;
// te: end of this wave group's part of the list (tiles at or past it only
// keep the group in step with the other at the barrier).
template <int CUR, int NXT, bool kDK, bool kExt>
__device__ inline void kv_tile(KvState<kDK>& st, const BwdParams& bp, const QPlan& qp, const KvItem& it,
                               const KvStage& stg, QCursor& cur, int t, int te, RA_LDS char* const* qbuf,
                               RA_LDS char* const* dbuf, RA_LDS char* const* lbuf, unsigned lane, int wave) {
  const StepParams& p = bp.s;
  const QCursor ci = cur;
  if (t + 1 < te) {
    cur.advance(qp);
    stg.template issue<kExt>(p, qp, cur, it.g, lane, qbuf[NXT], dbuf[NXT], lbuf[NXT]);
  }
  // this wave's keys against the tile's rows
  const long long qin = (long long)ci.tile * 32;
  const long long qglob = (ci.span ? p.qs_start[1] : p.qs_start[0]) + qin;
  const int qcount = (int)min(32LL, (ci.span ? p.qs_len[1] : p.qs_len[0]) - qin);
  const long long kwg = it.kglob0 + 32 * wave;
  const bool has_keys = 32 * wave < it.kcount && t < te;
  const bool live = has_keys && (!p.causal || kwg <= qglob + qcount - 1);
  if (live) {
    const unsigned rb = row_base_sigma(lane);
    const int L = (int)(lane >> 5);
    const RA_LDS float* lt = (const RA_LDS float*)lbuf[CUR];
    // dP starts from the rows' -delta (staged with the tile; the workspace
    // holds -delta), so the chain yields dP - delta: register r of the lane
    // is row 16(r/8) + 8L + r%8
    f32x16 s = f32x16{}, dp = f32x16{};
    if (kDK) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 t0 = *(const RA_LDS f32x4*)(lt + 64 + 16 * hf + 8 * L);
        const f32x4 t1 = *(const RA_LDS f32x4*)(lt + 64 + 16 * hf + 8 * L + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[8 * hf + e] = t0[e], dp[8 * hf + 4 + e] = t1[e];
      }
    }
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(qbuf[CUR], rb ^ (32u * u)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.k[u], s, 0, 0, 0);
      if (kDK) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, lds_load16(dbuf[CUR], rb ^ (32u * u)));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, st.v[u], dp, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // rows of register r: 16(r/8) + 8L + r%8 of the tile
    const int key = (int)(lane & 31u);
    // window, packed sequences: row i sees key j iff lo_i <= j <= hi_i, the
    // row's range relative to the tile's first row (staged with the tile)
    const RA_LDS int* rt = (const RA_LDS int*)(lbuf[CUR] + 512);
    const int dk = kExt ? (int)max(-(1LL << 30), min(1LL << 30, kwg - qglob)) + key : 0;
    if (!kExt && p.causal && kwg + 31 > qglob) {
      // row i sees key j iff qglob + i >= kwg + j
      const int dd = (int)max(-1024LL, min(1024LL, qglob - kwg)) + 8 * L - key;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = neg_inf_select(dd + 16 * (r >> 3) + (r & 7), s[r]);
    }
    unsigned b0, b1;
    tr_bases(lane, b0, b1);
    // one 16-row half at a time: P (and dS) of rows 16hf .. 16hf+15, then the
    // product over those rows; kSel: with the per-row key-range select
    // (masks; not on tiles whose every row sees all the wave's keys)
    auto halves = [&](auto sel) {
      constexpr bool kSel = decltype(sel)::value;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 l0 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L);
        const f32x4 l1 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L + 4);
        const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        int lo[8], hi[8];
        if (kSel) {
          const i32x4 a0 = *(const RA_LDS i32x4*)(rt + 16 * hf + 8 * L);
          const i32x4 a1 = *(const RA_LDS i32x4*)(rt + 16 * hf + 8 * L + 4);
          const i32x4 c0 = *(const RA_LDS i32x4*)(rt + 32 + 16 * hf + 8 * L);
          const i32x4 c1 = *(const RA_LDS i32x4*)(rt + 32 + 16 * hf + 8 * L + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) lo[e] = a0[e], lo[e + 4] = a1[e], hi[e] = c0[e], hi[e + 4] = c1[e];
        }
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // No guard for rows past the tile's end: their Q, dO, L and delta
          // were staged as zeros, so P = 1 there multiplies zero rows (and dS
          // = 0).  L is finite on every real row (each row sees at least its
          // own key), so P needs no -inf case; under masks a key outside the
          // row's range gets exponent -inf.  A select, not a branch, before
          // exp2.
          float a = __builtin_fmaf(s[8 * hf + e], p.sl2, -lv[e] * kLog2e);
          if (kSel) a = (lo[e] <= dk && dk <= hi[e]) ? a : kNegInf;
          const float pr = __builtin_amdgcn_exp2f(a);
          x[e] = kDK ? pr * dp[8 * hf + e] : pr;
        }
        const bf16x8 xb = __builtin_convertvector(x, bf16x8);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < kD / 32; ++db) {
          const unsigned o0 = (b0 ^ (64u * db)) + 16u * kRowB * hf, o1 = (b1 ^ (64u * db)) + 16u * kRowB * hf;
          const bf16x8 a = tr_read(kDK ? qbuf[CUR] : dbuf[CUR], o0, o1);
          st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb, st.acc[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (kExt && !kDK) {
      // the ranges never move left along the rows: every row sees the wave's
      // keys (relative positions dk - key .. dk - key + 31) iff the last
      // row's lower end and the first row's upper end do.  (The dK kernel,
      // with dP's registers live as well, would spill with both bodies.)
      const int lo_last = __builtin_amdgcn_readfirstlane(rt[31]);
      const int hi_first = __builtin_amdgcn_readfirstlane(rt[32]);
      const int k0 = __builtin_amdgcn_readfirstlane(dk - key);
      if (lo_last <= k0 && k0 + 31 <= hi_first)
        halves(KvbSel<false>{});
      else
        halves(KvbSel<true>{});
    } else {
      halves(KvbSel<kExt>{});
    }
  }
  wait_loads();
  __syncthreads();
}

// One key tile's pass over its query tiles by one group of four waves (GRP),
// tiles [tb, te) of the list; returns the accumulators in st.
template <bool kDK, bool kExt>
__device__ __attribute__((always_inline)) inline void kv_pass(KvState<kDK>& st, const BwdParams& bp,
                                                               const QPlan& qp, const KvItem& it, int tb, int te,
                                                               int iters, RA_LDS char* const* qbuf,
                                                               RA_LDS char* const* dbuf, RA_LDS char* const* lbuf,
                                                               unsigned lane, int wave) {
  const StepParams& p = bp.s;
  KvStage stg;
  stg.init(bp, it, wave, lane);
  QCursor cur;
  cur.first(qp);
  if (tb > 0) cur.seek(qp, tb);
  if (tb < te) stg.template issue<kExt>(p, qp, cur, it.g, lane, qbuf[0], dbuf[0], lbuf[0]);
  wait_loads();
  __syncthreads();

  int i = 0;
  for (; i + 1 < iters; i += 2) {
    kv_tile<0, 1, kDK, kExt>(st, bp, qp, it, stg, cur, tb + i, te, qbuf, dbuf, lbuf, lane, wave);
    kv_tile<1, 0, kDK, kExt>(st, bp, qp, it, stg, cur, tb + i + 1, te, qbuf, dbuf, lbuf, lane, wave);
  }
  if (i < iters) kv_tile<0, 1, kDK, kExt>(st, bp, qp, it, stg, cur, tb + i, te, qbuf, dbuf, lbuf, lane, wave);
}

// kSplit = false: four waves (one workgroup) per key tile of 128 keys (the
// launcher uses the fused kernel below instead).
// kSplit = true: eight waves, two groups of four over the same 128 keys; group
// 0 takes the first half of the query-tile list and group 1 the rest, and
// group 1 hands its partial sums to group 0 through LDS at the end (a fixed
// order of additions, so results do not depend on timing).  For launches
// with few key tiles: one workgroup per CU still keeps two waves on every
// SIMD.
template <bool kDK, bool kExt, bool kSplit>
__global__ __launch_bounds__(kSplit ? 2 * kThreads : kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_kv_kernel(BwdParams bp) {
  const StepParams& p = bp.s;
  constexpr int kB2 = kSplit ? kTileB : 16;  // group 1's buffers
  __shared__ __attribute__((aligned(16))) char q0_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char q1_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char d0_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char d1_raw[kTileB];
  __shared__ __attribute__((aligned(16))) char l0_raw[768];  // L, delta, and with masks the rows' key ranges
  __shared__ __attribute__((aligned(16))) char l1_raw[768];
  __shared__ __attribute__((aligned(16))) char q2_raw[kB2];
  __shared__ __attribute__((aligned(16))) char q3_raw[kB2];
  __shared__ __attribute__((aligned(16))) char d2_raw[kB2];
  __shared__ __attribute__((aligned(16))) char d3_raw[kB2];
  __shared__ __attribute__((aligned(16))) char l2_raw[kSplit ? 768 : 16];
  __shared__ __attribute__((aligned(16))) char l3_raw[kSplit ? 768 : 16];
  const unsigned lane = threadIdx.x & 63u;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = kSplit ? wv >> 2 : 0;
  const int wave = wv & 3;  // the wave's 32 keys within the tile

  KvItem it;
  if (!decode_kv(bp, it)) return;
  const QPlan qp = plan_q(p, it.kglob0, it.kcount);
  if (qp.n == 0) return;

  // K^T (and V^T) operands of the wave's 32 keys into registers
  const unsigned krow_bytes = (unsigned)(p.Hkv * kRowB);
  const long long khead = ((long long)it.b * p.Sk * p.Hkv + it.g) * (long long)kRowB;
  KvState<kDK> st;
  {
    const int key = 32 * wave + (int)(lane & 31u);
    const bool kok = key < it.kcount;
    const long long ro = khead + (it.klocal0 + key) * (long long)krow_bytes;
    const uint16_t* krow = (const uint16_t*)((const char*)p.k + ro);
    const uint16_t* vrow = (const uint16_t*)((const char*)p.v + ro);
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      st.k[u] = kok ? *(const bf16x8*)(krow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
      if (kDK) st.v[kDK ? u : 0] = kok ? *(const bf16x8*)(vrow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
    }
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) st.acc[db] = f32x16{};
  }

  const int half = kSplit ? (qp.n + 1) / 2 : qp.n;
  if (grp == 0) {
    RA_LDS char* const qbuf[2] = {(RA_LDS char*)q0_raw, (RA_LDS char*)q1_raw};
    RA_LDS char* const dbuf[2] = {(RA_LDS char*)d0_raw, (RA_LDS char*)d1_raw};
    RA_LDS char* const lbuf[2] = {(RA_LDS char*)l0_raw, (RA_LDS char*)l1_raw};
    kv_pass<kDK, kExt>(st, bp, qp, it, 0, half, half, qbuf, dbuf, lbuf, lane, wave);
  } else {
    RA_LDS char* const qbuf[2] = {(RA_LDS char*)q2_raw, (RA_LDS char*)q3_raw};
    RA_LDS char* const dbuf[2] = {(RA_LDS char*)d2_raw, (RA_LDS char*)d3_raw};
    RA_LDS char* const lbuf[2] = {(RA_LDS char*)l2_raw, (RA_LDS char*)l3_raw};
    kv_pass<kDK, kExt>(st, bp, qp, it, half, qp.n, half, qbuf, dbuf, lbuf, lane, wave);
  }

  if (kSplit) {
    // group 1's sums into LDS (8 KB of each of two buffers per wave, the
    // staging buffers being idle after the last barrier), then group 0 adds
    // them; layout [4 registers][64 lanes] of float4, conflict-free
    // (selects, not a table indexed by the wave: LDS addresses cannot be
    // stored as data)
    RA_LDS f32x4* const x0 = (RA_LDS f32x4*)(wave == 0   ? (RA_LDS char*)q0_raw
                                              : wave == 1 ? (RA_LDS char*)q1_raw
                                              : wave == 2 ? (RA_LDS char*)d0_raw
                                                          : (RA_LDS char*)d1_raw);
    RA_LDS f32x4* const x1 = (RA_LDS f32x4*)(wave == 0   ? (RA_LDS char*)q2_raw
                                              : wave == 1 ? (RA_LDS char*)q3_raw
                                              : wave == 2 ? (RA_LDS char*)d2_raw
                                                          : (RA_LDS char*)d3_raw);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = {st.acc[db][4 * j], st.acc[db][4 * j + 1], st.acc[db][4 * j + 2], st.acc[db][4 * j + 3]};
          (db < 2 ? x0 : x1)[((db & 1) * 4 + j) * 64 + lane] = v;
        }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = (db < 2 ? x0 : x1)[((db & 1) * 4 + j) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) st.acc[db][4 * j + e] += v[e];
      }
  }

  // dK = scale dS^T Q or dV = P^T dO of the wave's keys, added to the tensor
  const int key = 32 * wave + (int)(lane & 31u);
  if (key >= it.kcount) return;
  const long long krow = ((long long)it.b * p.Sk + it.klocal0 + key) * p.Hkv + it.g;
  float* dst = (kDK ? bp.dk : bp.dv) + krow * kD;
  const float f = kDK ? p.scale : 1.f;
  const int dsub = 4 * (int)(lane >> 5);
#pragma unroll
  for (int db = 0; db < kD / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 32 * db + 8 * j + dsub;
      const f32x16& a = st.acc[db];
      float4 r = *(const float4*)(dst + c);
      r.x += a[4 * j] * f;
      r.y += a[4 * j + 1] * f;
      r.z += a[4 * j + 2] * f;
      r.w += a[4 * j + 3] * f;
      *(float4*)(dst + c) = r;
    }
}

// ===========================================================================
// dK and dV in one launch with the products split evenly between the two
// wave groups of a key tile (128 keys; waves w and w + 4 share keys 32w ..
// 32w + 31).  Iteration t of the query-tile list:
//   dK waves: S(t) = Q K^T, P(t) = exp2(S sl2 - L log2 e), P(t) to LDS as
//     bf16 (the dV product's operand) and kept in float32 registers; and,
//     for tile t - 1, dS = P (dP - delta) with dP - delta from the dV waves,
//     and dK^T += Q^T dS (when both tiles are live and unmasked, P(t)'s
//     vector work runs between these products).
//   dV waves: dP(t) - delta = dO V^T - delta (the product chain starts from
//     the staged -delta), to LDS as float32; then, for tile t - 1, dV^T +=
//     dO^T P with P from the dK waves.
// Each group stages its own operands of tile t + 1 (Q and L, or dO and
// -delta); one barrier ends every iteration, so nothing inside an iteration
// waits for the other group, and each SIMD runs one wave of each with 16
// products apiece.  Q, dO, L and -delta are staged in three stages (tile t
// is read in iterations t and t + 1), P and dP - delta in two.

// Copy through the buffer unit into LDS, lane i's kBytes (16 or 4) from byte
// voff of a record of nrec bytes at base to dst + kBytes * i, issued
// from inline assembly so that the compiler does not see an LDS write in
// flight: it cannot tell this kernel's staged buffers apart from the ones its
// waves are reading and would otherwise wait for every copy before those
// reads.  The kernel's own wait before each barrier covers the copies.  M0
// carries the LDS address and is restored before the block ends; the copy
// writes no register.  The resource words may come from v_readfirstlane, and a
// buffer instruction reading an SGPR that a vector instruction wrote needs
// five wait states, which the compiler does not insert for operands of inline
// assembly: the two moves and s_nop 2 give them.
template <int kBytes>
__device__ inline void kvb_copy(const void* base, int nrec, unsigned voff, RA_LDS void* dst) {
  const unsigned long long a = (unsigned long long)base;
  u32x4 r;
  r[0] = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  r[2] = (unsigned)__builtin_amdgcn_readfirstlane(nrec);
  r[3] = (unsigned)kRsrcWord3;
  const int m = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)dst);
  int saved;
  if constexpr (kBytes == 16)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 2\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(m), "s"(r)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 2\n\tbuffer_load_dword %1, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(m), "s"(r)
        : "memory");
}

// The query tile list of a key tile (heads outer, then spans, then tiles),
// with what staging and masking take of the current tile carried from tile to
// tile by additions; only a move to the other span or the next head goes back
// to the plan.  Q and dO share a layout, and so do L and -delta, so the one
// cursor serves both wave groups.
struct KvbCursor {
  int hh, span, tile;
  int left;          // rows of the span from the tile's first row on
  int qrel;          // (tile's first position) - kwg (the wave's first key), held in [-2^30, 2^30]
  long long xoff;    // bytes from (b, row 0, head 0) to the tile's first row, head h, in Q or dO;
                     // xoff / kRowB is the same row's offset in L or -delta

  __device__ int count() const { return min(32, left); }
  __device__ long long qglob(const StepParams& p) const {
    return (span ? p.qs_start[1] : p.qs_start[0]) + (long long)tile * 32;
  }
  __device__ void place(const StepParams& p, int g, unsigned row_bytes, long long kwg) {
    const long long qin = (long long)tile * 32;
    const long long local0 = (span ? p.qs_off[1] : p.qs_off[0]) + qin;
    const int h = g * p.G + hh;
    left = (int)((span ? p.qs_len[1] : p.qs_len[0]) - qin);
    xoff = local0 * row_bytes + (long long)h * kRowB;
    qrel = (int)max(-(1LL << 30), min(1LL << 30, qglob(p) - kwg));
  }
  __device__ void first(const StepParams& p, const QPlan& qp, int g, unsigned row_bytes, long long kwg) {
    hh = 0;
    span = qp.tend[0] > qp.tbeg[0] ? 0 : 1;
    tile = span ? qp.tbeg[1] : qp.tbeg[0];
    place(p, g, row_bytes, kwg);
  }
  __device__ void advance(const StepParams& p, const QPlan& qp, int g, unsigned row_bytes, long long kwg) {
    ++tile;
    if (tile < (span ? qp.tend[1] : qp.tend[0])) {
      left -= 32;
      xoff += 32LL * row_bytes;
      // exact while above -2^29 (a value held at 2^30 stays there: the rows
      // only move on); below, from the positions again
      if (qrel > -(1 << 29))
        qrel = min(qrel + 32, 1 << 30);
      else
        qrel = (int)max(-(1LL << 30), min(1LL << 30, qglob(p) - kwg));
      return;
    }
    if (span == 0 && qp.tend[1] > qp.tbeg[1]) {
      span = 1;
      tile = qp.tbeg[1];
    } else {
      ++hh;
      span = qp.tend[0] > qp.tbeg[0] ? 0 : 1;
      tile = span ? qp.tbeg[1] : qp.tbeg[0];
    }
    place(p, g, row_bytes, kwg);
  }
};

struct KvbStage {
  const char* xbase;     // row 0 of (batch b, query head 0) in Q (dK group) or dO (dV group)
  const float* sbase;    // (b, row 0, head 0) in L (dK group) or in -delta (dV group)
  unsigned row_bytes;    // Hq * 2D
  unsigned off[2];
  int wave, Hq;

  __device__ void init(const BwdParams& bp, const KvItem& it, int w, unsigned lane, bool dv) {
    const StepParams& p = bp.s;
    Hq = p.Hq;
    row_bytes = (unsigned)(p.Hq * kRowB);
    const long long base = (long long)it.b * p.Sq * p.Hq;
    xbase = (const char*)(dv ? bp.dout : p.q) + base * kRowB;
    sbase = (dv ? bp.delta : bp.lse) + base;
    wave = w;
    off[0] = dma_off(w, 0, lane, row_bytes);
    off[1] = dma_off(w, 1, lane, row_bytes);
  }
  // Staging of query tile c in pieces, so that a wave can place them between
  // the products of a chain: 1, with masks (dK group, waves 2 and 3) the
  // rows' key ranges to ldst[512, 768), first: with packed sequences they are
  // looked up in global memory, and the wait for that lookup then covers no
  // copy of this tile; 2 and 3, the wave's two 1 KB parts of the tile's 32
  // rows of the group's tensor; 4, (wave 0) the rows' L to ldst[0, 256) or
  // -delta to ldst[256, 512).  Rows past the tile's end read 0.
  template <bool kExt, bool kDV>
  __device__ void piece(int k, const StepParams& p, const KvbCursor& c, unsigned lane, RA_LDS char* xdst,
                        RA_LDS char* ldst) const {
    const int count = c.count();
    if (k == 1) {
      if (kExt && !kDV && wave >= 2 && lane < 32) {
        const long long qg = c.qglob(p);
        const long long v = wave == 2 ? key_lo(p, qg + lane) : key_hi(p, qg + lane);
        ((RA_LDS int*)(ldst + 512))[(wave - 2) * 32 + lane] = (int)max(-(1LL << 30), min(1LL << 30, v - qg));
      }
    } else if (k == 2 || k == 3) {
      const int nrec = (count - 1) * (int)row_bytes + kRowB;
      kvb_copy<16>(xbase + c.xoff, nrec, off[k - 2], xdst + (wave * 2 + k - 2) * 1024);
    } else if (k == 4 && wave == 0) {
      const float* src = sbase + (c.xoff >> 8);  // row offset: xoff / kRowB
      const int nr = ((count - 1) * Hq + 1) * 4;
      kvb_copy<4>(src, nr, lane * (unsigned)Hq * 4u, ldst + (kDV ? 256 : 0));
    }
  }
  template <bool kExt, bool kDV>
  __device__ void issue(const StepParams& p, const KvbCursor& c, unsigned lane, RA_LDS char* xdst,
                        RA_LDS char* ldst) const {
#pragma unroll
    for (int k = 1; k <= 4; ++k) piece<kExt, kDV>(k, p, c, lane, xdst, ldst);
  }
};

// The end of the prologue: the K^T or V^T operand registers and tile 0
// complete, then the barrier.  The wait is the compiler's own instruction, so
// it knows that the operand loads complete here and adds no wait for them
// inside the loop, where it would also wait for the copies in flight.
__device__ inline void kvb_begin() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Whether the wave's 32 keys meet query tile c at all (causal: its first key
// at or before the tile's last row).
__device__ inline bool kvb_live(const StepParams& p, const KvbCursor& c, bool has_keys) {
  return has_keys && (!p.causal || c.qrel + c.count() - 1 >= 0);
}

struct KvbDk {
  bf16x8 k[kD / 16];      // K^T operand: K[key l%32][16u + 8(l/32) .. +7]
  f32x16 acc[kD / 32];    // dK^T accumulators
  f32x16 pk[2];           // P, float32, of the tiles of even and odd t
  bool live_prev;
};

// Iteration t of the dK group; T6 = t mod 6 names the stages statically.
template <int T6, bool kExt>
__device__ inline void kvb_dk_iter(KvbDk& st, const BwdParams& bp, const QPlan& qp, const KvItem& it,
                                   const KvbStage& stg, KvbCursor& cur, int t, int n, RA_LDS char* const* qbuf,
                                   RA_LDS char* const* lbuf, RA_LDS char* const* pbuf, RA_LDS char* const* gbuf,
                                   unsigned lane, int wave, long long kwg, bool has_keys) {
  constexpr int CUR = T6 % 3, PRV = (T6 + 2) % 3, NXT = (T6 + 1) % 3, PC = T6 % 2, PP = (T6 + 1) % 2;
  const StepParams& p = bp.s;
  const KvbCursor ci = cur;
  const bool stage = t + 1 < n;
  // staging of tile t + 1 (piece 0: the cursor's advance), placed between
  // the dependent products of the score chain when the tile is live (with
  // masks, whose tiles carry more scalar work, all before it: between the
  // products it would not fit the scalar registers)
  auto piece = [&](int k) {
    if (!stage) return;
    if (k == 0)
      cur.advance(p, qp, it.g, stg.row_bytes, kwg);
    else
      stg.template piece<kExt, false>(k, p, cur, lane, qbuf[NXT], lbuf[NXT]);
  };
  const int L = (int)(lane >> 5);
  const bool live = t < n && kvb_live(p, ci, has_keys);
  f32x16& pk = st.pk[PC];  // tile t's P, read next iteration only if live
  if (kExt || !live) {
#pragma unroll
    for (int k = 0; k <= 4; ++k) piece(k);
  }
  if (live) {
    // every operand read issued before the product chain (the chain then
    // waits only for the read it needs next)
    const unsigned rb = row_base_sigma(lane);
    bf16x8 a[kD / 16];
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) a[u] = __builtin_bit_cast(bf16x8, lds_load16(qbuf[CUR], rb ^ (32u * u)));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{};
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], st.k[u], s, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (!kExt && u <= 4) piece(u);
      __builtin_amdgcn_sched_barrier(0);
    }
    // rows of register r: 16(r/8) + 8L + r%8 of the tile; the lane's key
    const int key = (int)(lane & 31u);
    const RA_LDS int* rt = (const RA_LDS int*)(lbuf[CUR] + 512);
    const int dk = kExt ? key - ci.qrel : 0;
    if (!kExt && p.causal && ci.qrel < 31) {
      // row i sees key j iff qglob + i >= kwg + j
      const int dd = max(-1024, min(1024, ci.qrel)) + 8 * L - key;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = neg_inf_select(dd + 16 * (r >> 3) + (r & 7), s[r]);
    }
    const RA_LDS float* lt = (const RA_LDS float*)lbuf[CUR];
    // P of the tile; kSel: with the per-row key-range select (masks; not
    // on tiles whose every row sees all the wave's keys)
    auto probabilities = [&](auto sel) {
      constexpr bool kSel = decltype(sel)::value;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 l0 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L);
        const f32x4 l1 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L + 4);
        const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        int lo[8], hi[8];
        if (kSel) {
          const i32x4 a0 = *(const RA_LDS i32x4*)(rt + 16 * hf + 8 * L);
          const i32x4 a1 = *(const RA_LDS i32x4*)(rt + 16 * hf + 8 * L + 4);
          const i32x4 c0 = *(const RA_LDS i32x4*)(rt + 32 + 16 * hf + 8 * L);
          const i32x4 c1 = *(const RA_LDS i32x4*)(rt + 32 + 16 * hf + 8 * L + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) lo[e] = a0[e], lo[e + 4] = a1[e], hi[e] = c0[e], hi[e + 4] = c1[e];
        }
        f32x8 xp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // rows past the tile's end were staged as zeros (P = 1 times zero
          // rows); L is finite on every real row; a key outside the row's
          // range gets exponent -inf (a select before exp2)
          float a = __builtin_fmaf(s[8 * hf + e], p.sl2, -lv[e] * kLog2e);
          if (kSel) a = (lo[e] <= dk && dk <= hi[e]) ? a : kNegInf;
          xp[e] = __builtin_amdgcn_exp2f(a);
          pk[8 * hf + e] = xp[e];
        }
        *(RA_LDS bf16x8*)(pbuf[PC] + (wave * 2 + hf) * 1024 + lane * 16) = __builtin_convertvector(xp, bf16x8);
      }
    };
    if constexpr (kExt) {
      // the ranges never move left along the rows, so every row sees the
      // wave's keys (relative positions -qrel .. 31 - qrel) iff the last
      // row's lower end and the first row's upper end do
      const int lo_last = __builtin_amdgcn_readfirstlane(rt[31]);
      const int hi_first = __builtin_amdgcn_readfirstlane(rt[32]);
      if (lo_last <= -ci.qrel && 31 - ci.qrel <= hi_first)
        probabilities(KvbSel<false>{});
      else
        probabilities(KvbSel<true>{});
    } else if (!(t > 0 && st.live_prev)) {
      probabilities(KvbSel<false>{});
    } else {
      // Both tiles live (unmasked kernel): tile t's P and tile t - 1's dK
      // products in one stretch.  Per 16-row half: the half's operand reads
      // (Q^T of tile t - 1, dP - delta, L), dS of tile t - 1, then its four
      // products with the half's exponentials between them (the scheduler
      // told one product, then seven vector instructions), so that the
      // products run while this wave works through P.
      const RA_LDS f32x4* g = (const RA_LDS f32x4*)(gbuf[PP] + wave * 4096) + lane;
      unsigned b0, b1;
      tr_bases(lane, b0, b1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 g0 = g[(2 * hf) * 64], g1 = g[(2 * hf + 1) * 64];
        const f32x4 l0 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L);
        const f32x4 l1 = *(const RA_LDS f32x4*)(lt + 16 * hf + 8 * L + 4);
        bf16x8 qt[kD / 32];
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
          qt[db] = tr_read(qbuf[PRV], (b0 ^ (64u * db)) + 16u * kRowB * hf, (b1 ^ (64u * db)) + 16u * kRowB * hf);
        __builtin_amdgcn_sched_barrier(0);
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = st.pk[PP][8 * hf + e] * g0[e];
          x[e + 4] = st.pk[PP][8 * hf + 4 + e] * g1[e];
        }
        const bf16x8 xb = __builtin_convertvector(x, bf16x8);
        __builtin_amdgcn_sched_barrier(0);
        const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        f32x8 xp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hf + e], p.sl2, -lv[e] * kLog2e));
          pk[8 * hf + e] = xp[e];
        }
        *(RA_LDS bf16x8*)(pbuf[PC] + (wave * 2 + hf) * 1024 + lane * 16) = __builtin_convertvector(xp, bf16x8);
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
          st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[db], xb, st.acc[db], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kD / 32; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (t > 0 && st.live_prev && (kExt || !live)) {
    // dS of tile t - 1 from its P (kept) and dP - delta (the dV waves'),
    // then dK^T += Q^T dS over its two 16-row halves
    const RA_LDS f32x4* g = (const RA_LDS f32x4*)(gbuf[PP] + wave * 4096) + lane;
    unsigned b0, b1;
    tr_bases(lane, b0, b1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 g0 = g[(2 * hf) * 64], g1 = g[(2 * hf + 1) * 64];
      bf16x8 qt[kD / 32];
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
        qt[db] = tr_read(qbuf[PRV], (b0 ^ (64u * db)) + 16u * kRowB * hf, (b1 ^ (64u * db)) + 16u * kRowB * hf);
      __builtin_amdgcn_sched_barrier(0);
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = st.pk[PP][8 * hf + e] * g0[e];
        x[e + 4] = st.pk[PP][8 * hf + 4 + e] * g1[e];
      }
      const bf16x8 xb = __builtin_convertvector(x, bf16x8);
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
        st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[db], xb, st.acc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  st.live_prev = live;
  if (t < n) {
    wait_loads();
    __syncthreads();
  }
}

struct KvbDv {
  bf16x8 v[kD / 16];      // V^T operand, the layout of K^T in KvbDk
  f32x16 acc[kD / 32];    // dV^T accumulators
  bool live_prev;
};

template <int T6, bool kExt>
__device__ inline void kvb_dv_iter(KvbDv& st, const BwdParams& bp, const QPlan& qp, const KvItem& it,
                                   const KvbStage& stg, KvbCursor& cur, int t, int n, RA_LDS char* const* dbuf,
                                   RA_LDS char* const* lbuf, RA_LDS char* const* pbuf, RA_LDS char* const* gbuf,
                                   unsigned lane, int wave, long long kwg, bool has_keys) {
  constexpr int CUR = T6 % 3, PRV = (T6 + 2) % 3, NXT = (T6 + 1) % 3, PC = T6 % 2, PP = (T6 + 1) % 2;
  const StepParams& p = bp.s;
  const KvbCursor ci = cur;
  const bool stage = t + 1 < n;
  // staging of tile t + 1, placed between the dependent products of the dP
  // chain when the tile is live (with masks, all before it)
  auto piece = [&](int k) {
    if (!stage) return;
    if (k == 0)
      cur.advance(p, qp, it.g, stg.row_bytes, kwg);
    else
      stg.template piece<kExt, true>(k, p, cur, lane, dbuf[NXT], lbuf[NXT]);
  };
  const bool live = t < n && kvb_live(p, ci, has_keys);
  if (kExt || !live) {
#pragma unroll
    for (int k = 0; k <= 4; ++k) piece(k);
  }
  if (live) {
    // dP - delta: the chain starts from the rows' -delta (register r of the
    // lane is row 16(r/8) + 8L + r%8)
    const int L = (int)(lane >> 5);
    const RA_LDS float* lt = (const RA_LDS float*)lbuf[CUR];
    f32x16 dp;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 t0 = *(const RA_LDS f32x4*)(lt + 64 + 16 * hf + 8 * L);
      const f32x4 t1 = *(const RA_LDS f32x4*)(lt + 64 + 16 * hf + 8 * L + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[8 * hf + e] = t0[e], dp[8 * hf + 4 + e] = t1[e];
    }
    const unsigned rb = row_base_sigma(lane);
    bf16x8 b[kD / 16];
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) b[u] = __builtin_bit_cast(bf16x8, lds_load16(dbuf[CUR], rb ^ (32u * u)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[u], st.v[u], dp, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (!kExt && u <= 4) piece(u);
      __builtin_amdgcn_sched_barrier(0);
    }
    RA_LDS f32x4* g = (RA_LDS f32x4*)(gbuf[PC] + wave * 4096) + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) g[k * 64] = f32x4{dp[4 * k], dp[4 * k + 1], dp[4 * k + 2], dp[4 * k + 3]};
  }
  __builtin_amdgcn_sched_barrier(0);
  if (t > 0 && st.live_prev) {
    // dV^T += dO^T P for tile t - 1, P from the dK waves
    unsigned b0, b1;
    tr_bases(lane, b0, b1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bf16x8 xb = *(const RA_LDS bf16x8*)(pbuf[PP] + (wave * 2 + hf) * 1024 + lane * 16);
      bf16x8 dt[kD / 32];
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
        dt[db] = tr_read(dbuf[PRV], (b0 ^ (64u * db)) + 16u * kRowB * hf, (b1 ^ (64u * db)) + 16u * kRowB * hf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
        st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dt[db], xb, st.acc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  st.live_prev = live;
  if (t < n) {
    wait_loads();
    __syncthreads();
  }
}

template <bool kExt>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_kvb_kernel(BwdParams bp) {
  const StepParams& p = bp.s;
  // One array with fixed offsets: the Q, dO and L / -delta stages (the
  // transposing and operand reads of every tile) below 64 KB, where a DS
  // instruction's 16-bit offset reaches them from a per-lane base; then P
  // (4 waves x 2 halves x 1 KB per stage) and dP - delta (4 waves x 4 KB).
  constexpr int kQ = 0, kDo = 3 * kTileB, kL = 6 * kTileB, kP = kL + 3 * 768, kG = kP + 2 * kTileB;
  static_assert(kL + 3 * 768 <= 65536, "staged tiles within reach of the DS offset");
  __shared__ __attribute__((aligned(16))) char lds_raw[kG + 2 * 4 * 4096];
  RA_LDS char* const lds = (RA_LDS char*)lds_raw;
  RA_LDS char* const lbuf[3] = {lds + kL, lds + kL + 768, lds + kL + 1536};
  RA_LDS char* const pbuf[2] = {lds + kP, lds + kP + kTileB};
  RA_LDS char* const gbuf[2] = {lds + kG, lds + kG + 4 * 4096};
  const unsigned lane = threadIdx.x & 63u;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wv & 3;  // the wave's 32 keys within the tile

  KvItem it;
  if (!decode_kv(bp, it)) return;
  const QPlan qp = plan_q(p, it.kglob0, it.kcount);
  if (qp.n == 0) return;
  const int n = qp.n;
  const int key = 32 * wave + (int)(lane & 31u);
  const long long krow = ((long long)it.b * p.Sk + it.klocal0 + key) * p.Hkv + it.g;
  const int dsub = 4 * (int)(lane >> 5);
  const long long kwg = it.kglob0 + 32 * wave;
  const bool has_keys = 32 * wave < it.kcount;
  const bool kok = key < it.kcount;
  const long long ro = ((long long)it.b * p.Sk * p.Hkv + it.g) * (long long)kRowB +
                       (it.klocal0 + key) * (long long)(p.Hkv * kRowB);
  const bool dv = wv >= 4;
  KvbStage stg;
  stg.init(bp, it, wave, lane, dv);
  KvbCursor cur;
  cur.first(p, qp, it.g, stg.row_bytes, kwg);

  if (!dv) {
    RA_LDS char* const qbuf[3] = {lds + kQ, lds + kQ + kTileB, lds + kQ + 2 * kTileB};
    KvbDk st;
    const uint16_t* kr = (const uint16_t*)((const char*)p.k + ro);
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) st.k[u] = kok ? *(const bf16x8*)(kr + 16 * u + 8 * (lane >> 5)) : bf16x8{};
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) st.acc[db] = f32x16{};
    st.live_prev = false;
    stg.template issue<kExt, false>(p, cur, lane, qbuf[0], lbuf[0]);
    kvb_begin();
    int t = 0;
    for (; t + 5 <= n; t += 6) {
      kvb_dk_iter<0, kExt>(st, bp, qp, it, stg, cur, t, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
      kvb_dk_iter<1, kExt>(st, bp, qp, it, stg, cur, t + 1, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
      kvb_dk_iter<2, kExt>(st, bp, qp, it, stg, cur, t + 2, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
      kvb_dk_iter<3, kExt>(st, bp, qp, it, stg, cur, t + 3, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
      kvb_dk_iter<4, kExt>(st, bp, qp, it, stg, cur, t + 4, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
      kvb_dk_iter<5, kExt>(st, bp, qp, it, stg, cur, t + 5, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    }
    // the rest of t = 0 .. n (at most six iterations, the last one t = n)
    if (t <= n) kvb_dk_iter<0, kExt>(st, bp, qp, it, stg, cur, t, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    if (t + 1 <= n)
      kvb_dk_iter<1, kExt>(st, bp, qp, it, stg, cur, t + 1, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    if (t + 2 <= n)
      kvb_dk_iter<2, kExt>(st, bp, qp, it, stg, cur, t + 2, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    if (t + 3 <= n)
      kvb_dk_iter<3, kExt>(st, bp, qp, it, stg, cur, t + 3, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    if (t + 4 <= n)
      kvb_dk_iter<4, kExt>(st, bp, qp, it, stg, cur, t + 4, n, qbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    if (!kok) return;
    float* dst = bp.dk + krow * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 32 * db + 8 * j + dsub;
        float4 r = *(const float4*)(dst + c);
        r.x += st.acc[db][4 * j] * p.scale;
        r.y += st.acc[db][4 * j + 1] * p.scale;
        r.z += st.acc[db][4 * j + 2] * p.scale;
        r.w += st.acc[db][4 * j + 3] * p.scale;
        *(float4*)(dst + c) = r;
      }
    return;
  }

  RA_LDS char* const dbuf[3] = {lds + kDo, lds + kDo + kTileB, lds + kDo + 2 * kTileB};
  KvbDv st;
  const uint16_t* vr = (const uint16_t*)((const char*)p.v + ro);
#pragma unroll
  for (int u = 0; u < kD / 16; ++u) st.v[u] = kok ? *(const bf16x8*)(vr + 16 * u + 8 * (lane >> 5)) : bf16x8{};
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) st.acc[db] = f32x16{};
  st.live_prev = false;
  stg.template issue<kExt, true>(p, cur, lane, dbuf[0], lbuf[0]);
  kvb_begin();
  int t = 0;
  for (; t + 5 <= n; t += 6) {
    kvb_dv_iter<0, kExt>(st, bp, qp, it, stg, cur, t, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    kvb_dv_iter<1, kExt>(st, bp, qp, it, stg, cur, t + 1, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    kvb_dv_iter<2, kExt>(st, bp, qp, it, stg, cur, t + 2, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    kvb_dv_iter<3, kExt>(st, bp, qp, it, stg, cur, t + 3, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    kvb_dv_iter<4, kExt>(st, bp, qp, it, stg, cur, t + 4, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
    kvb_dv_iter<5, kExt>(st, bp, qp, it, stg, cur, t + 5, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  }
  if (t <= n) kvb_dv_iter<0, kExt>(st, bp, qp, it, stg, cur, t, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  if (t + 1 <= n)
    kvb_dv_iter<1, kExt>(st, bp, qp, it, stg, cur, t + 1, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  if (t + 2 <= n)
    kvb_dv_iter<2, kExt>(st, bp, qp, it, stg, cur, t + 2, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  if (t + 3 <= n)
    kvb_dv_iter<3, kExt>(st, bp, qp, it, stg, cur, t + 3, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  if (t + 4 <= n)
    kvb_dv_iter<4, kExt>(st, bp, qp, it, stg, cur, t + 4, n, dbuf, lbuf, pbuf, gbuf, lane, wave, kwg, has_keys);
  if (!kok) return;
  float* dst = bp.dv + krow * kD;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 32 * db + 8 * j + dsub;
      float4 r = *(const float4*)(dst + c);
      r.x += st.acc[db][4 * j];
      r.y += st.acc[db][4 * j + 1];
      r.z += st.acc[db][4 * j + 2];
      r.w += st.acc[db][4 * j + 3];
      *(float4*)(dst + c) = r;
    }
}

// ===========================================================================
// delta = rowsum(dO * O): 16 lanes per row of 128, 8 elements per lane.
template <typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(long long rows, const T* __restrict__ dout,
                                                        const float* __restrict__ o, float* __restrict__ delta) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const float* orow = o + row * kD + 8 * part;
    const float4 o0 = *(const float4*)orow;
    const float4 o1 = *(const float4*)(orow + 4);
    float dv[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 d = *(const bf16x8*)((const uint16_t*)dout + row * kD + 8 * part);
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] = (float)d[e];
    } else {
      const float4 d0 = *(const float4*)((const float*)dout + row * kD + 8 * part);
      const float4 d1 = *(const float4*)((const float*)dout + row * kD + 8 * part + 4);
      dv[0] = d0.x, dv[1] = d0.y, dv[2] = d0.z, dv[3] = d0.w;
      dv[4] = d1.x, dv[5] = d1.y, dv[6] = d1.z, dv[7] = d1.w;
    }
    acc = dv[0] * o0.x + dv[1] * o0.y + dv[2] * o0.z + dv[3] * o0.w + dv[4] * o1.x + dv[5] * o1.y + dv[6] * o1.z +
          dv[7] * o1.w;
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  // stored negated: the products start their dP accumulation from it
  if (row < rows && part == 0) delta[row] = -acc;
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdParams& p, hipStream_t s) {
  const bool ext = p.s.mask_ext != 0;
  if (p.s.n_work > 0) {
    if (ext)
      hipLaunchKernelGGL(attn_bwd_dq_kernel<true>, dim3(8 * p.s.per_xcd), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_bwd_dq_kernel<false>, dim3(8 * p.s.per_xcd), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.n_kwork > 0) {
    const dim3 grid(8 * p.per_xcd_kv), blk(2 * kThreads);
    // split query tiles: the dV kernel, then the dK kernel; otherwise both
    // in one fused launch
    if (ext && p.kv_split) {
      hipLaunchKernelGGL((attn_bwd_kv_kernel<false, true, true>), grid, blk, 0, s, p);
      hipLaunchKernelGGL((attn_bwd_kv_kernel<true, true, true>), grid, blk, 0, s, p);
    } else if (ext) {
      hipLaunchKernelGGL(attn_bwd_kvb_kernel<true>, grid, blk, 0, s, p);
    } else if (p.kv_split) {
      hipLaunchKernelGGL((attn_bwd_kv_kernel<false, false, true>), grid, blk, 0, s, p);
      hipLaunchKernelGGL((attn_bwd_kv_kernel<true, false, true>), grid, blk, 0, s, p);
    } else {
      hipLaunchKernelGGL(attn_bwd_kvb_kernel<false>, grid, blk, 0, s, p);
    }
  }
  return hipGetLastError();
}

hipError_t launch_bwd_delta(long long rows, int D, int dtype, const void* dout, const float* o, float* delta,
                            hipStream_t s) {
  if (D != kD) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 15) / 16);
  if (dtype == 1)
    hipLaunchKernelGGL(bwd_delta_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, rows, (const uint16_t*)dout, o,
                       delta);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3(blocks), dim3(256), 0, s, rows, (const float*)dout, o, delta);
  return hipGetLastError();
}

}  // namespace ra
