// One ring step of blockwise attention on gfx950 for fp32 inputs, with the
// log-sum-exp merge fused into the epilogue.
//
// What it computes (DeDLOC guide, "Step 3" and "3. Online Softmax Rescaling
// Across Decentralized Ranks"; causal skipping from its "Best Practices" row
// "Causal Mask Handling"): for every query row of the rank's fixed block and
// the key/value block that arrived at this ring step, the partial output
// O = softmax(scale * q K^T) V over the visible keys and its log-sum-exp; in
// INIT mode that pair is stored, in ACCUM mode it is merged into the running
// (O, LSE) held in HBM.
//
// Work decomposition
//   * A workgroup (4 waves) owns 128 consecutive query rows of one (batch,
//     query head); wave w owns rows [32w, 32w + 32).
//   * Keys are processed in tiles of 32.  Tile t+1 is loaded into registers
//     at the start of iteration t and written to the other LDS buffer (two
//     each for K and V) at its end; the loop is unrolled by two so that every
//     LDS buffer is named statically.
//   * Only key tiles with at least one visible key are visited; tiles all of
//     whose keys every row of the work item sees run first and skip the mask.
//
// Per-wave math (32 queries x 32 keys per tile), on the fp32 32x32x2 MFMA
//   S^T = K Q^T: register r of lane l holds key 8(r/4) + 4(l/32) + r%4 of
//   query l%32.  O^T += V^T P^T: the MFMA pairs reduction index l/32 of
//   step j with key 8(j/4) + 4(l/32) + j%4, i.e. with accumulator register
//   j of the lane, so P^T needs no data movement; V is read from LDS as
//   scalars.  Softmax in base 2 with a lazily moved reference maximum.
#include "attn_common.h"

namespace ra {
namespace {

using namespace dev;

constexpr int kThreads = 256;  // 4 waves
static_assert(kBQ == 4 * 32, "workgroup rows");
static_assert(kBK == 32, "one 32x32 score block per tile");

template <int D>
struct Layout {
  // Tiles in LDS: 32 key rows of D floats, 16-byte chunks XOR-swizzled per
  // row so that both the operand reads and the tile fills hit distinct banks:
  //   K: chunk ^ (row mod chunks)   -- 32 rows, one element per lane
  //   V: chunk ^ (4 (row mod 4))    -- 32 columns of 4 rows
  static constexpr int kRowBytes = D * 4;
  static constexpr int kCPR = kRowBytes / 16;
  static constexpr int kTileBytes = kBK * kRowBytes;
  static constexpr int kPer = kBK * kCPR / kThreads;  // chunks per thread and tile
  __device__ static unsigned swz_k(unsigned row) { return row & (kCPR - 1); }
  __device__ static unsigned swz_v(unsigned row) { return (4u * (row & 3u)) & (kCPR - 1); }
  __device__ static float read(const RA_LDS char* t, unsigned row, unsigned d, unsigned swz) {
    return *(const RA_LDS float*)(t + row * kRowBytes + (((d >> 2) ^ swz) * 16) + (d & 3) * 4);
  }
};

// Staging of K and V tiles through registers.  Rows past `count` (only in a
// span's last tile) repeat the last real row: their keys are masked to -inf
// (K) and weighted by exactly 0 (V).
template <int D>
struct TileStage {
  typedef Layout<D> Ly;
  u32x4 k[Ly::kPer], v[Ly::kPer];
  unsigned row_bytes;  // global stride between key rows

  __device__ void init(const StepParams& p) { row_bytes = (unsigned)(p.Hkv * D * 4); }

  __device__ void load(const StepParams& p, const WorkItem& wi, const KTile& kt) {
    const long long base = (((long long)wi.b * p.Sk + kt.local0) * p.Hkv + wi.g) * (long long)(D * 4);
    const char* ks = (const char*)p.k + base;
    const char* vs = (const char*)p.v + base;
#pragma unroll
    for (int i = 0; i < Ly::kPer; ++i) {
      const unsigned idx = threadIdx.x + i * kThreads;
      const unsigned row = min(idx / Ly::kCPR, (unsigned)kt.count - 1u), c = idx % Ly::kCPR;
      const unsigned off = row * row_bytes + c * 16;
      k[i] = *(const u32x4*)(ks + off);
      v[i] = *(const u32x4*)(vs + off);
    }
  }

  __device__ void store(RA_LDS char* kdst, RA_LDS char* vdst) const {
#pragma unroll
    for (int i = 0; i < Ly::kPer; ++i) {
      const unsigned idx = threadIdx.x + i * kThreads;
      const unsigned row = idx / Ly::kCPR, c = idx % Ly::kCPR;
      *(RA_LDS u32x4*)(kdst + row * Ly::kRowBytes + ((c ^ Ly::swz_k(row)) * 16)) = k[i];
      *(RA_LDS u32x4*)(vdst + row * Ly::kRowBytes + ((c ^ Ly::swz_v(row)) * 16)) = v[i];
    }
  }
};

template <int D>
struct WaveState {
  float q[D / 2];    // Q^T operand of step u: Q[row][2u + l/32]
  f32x16 o[D / 32][1];
  float m_ref, l_part;
};

__device__ inline KTile ktile(const TileCursor& c) {
  KTile kt;
  kt.local0 = c.local0;
  kt.glob0 = c.glob0;
  kt.count = c.count();
  return kt;
}

// Tile t of the plan (cursor cur) from buffer PAR; the lane's row sees keys
// [row_lo, row_hi] (global positions).
template <int D, int PAR>
__device__ inline void step_tile(WaveState<D>& ws, const StepParams& p, const TilePlan& tp, TileStage<D>& st,
                                 const WorkItem& wi, TileCursor& cur, int t, RA_LDS char* const* kbuf,
                                 RA_LDS char* const* vbuf, long long row_lo, long long row_hi, int lane) {
  typedef Layout<D> Ly;
  const TileCursor ci = cur;
  const KTile ti = ktile(ci);
  const bool more = t + 1 < tp.n;
  if (more) {
    cur.advance(tp);
    st.load(p, wi, ktile(cur));
  }

  const int L = lane >> 5;
  f32x16 s = {};
  {
    const unsigned row = lane & 31;
#pragma unroll
    for (int u = 0; u < D / 2; ++u) {
      const float a = Ly::read(kbuf[PAR], row, 2 * u + L, Ly::swz_k(row));
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, ws.q[u], s, 0, 0, 0);
    }
  }
  if (ci.masked()) {  // masked tiles only (a uniform branch)
    // keys [lo, lim) of the tile: the causal diagonal, a span's ragged end,
    // a window's or a packed sequence's edges
    const int lim = (int)max(0LL, min((long long)ti.count, row_hi - ti.glob0 + 1));
    const int lo = (int)max(0LL, min((long long)kBK, row_lo - ti.glob0));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * L + (r & 3);
      if (key >= lim || key < lo) s[r] = kNegInf;
    }
  }
  float tmax = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = max_halves(tmax);
  const float m_new = fmaxf(ws.m_ref, tmax);
  // -inf reference: the difference is +inf and the maximum is taken;
  // both -inf: NaN compares false and nothing moves.
  const bool grow = (m_new - ws.m_ref) * p.sl2 > kTau;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float alpha = grow ? __builtin_amdgcn_exp2f((ws.m_ref - m_new) * p.sl2) : 1.f;
    if (grow) ws.m_ref = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) ws.o[db][0] *= alpha;
    ws.l_part *= alpha;
  }
  const float mb = ws.m_ref == kNegInf ? 0.f : ws.m_ref * p.sl2;
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.sl2, -mb));
    lsum += s[r];
  }
  ws.l_part += lsum;
  // materialise the row sum here: otherwise the adds sink into the next tile
  // and keep this tile's probabilities alive across it
  asm volatile("" : "+v"(ws.l_part));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const unsigned d = 32 * db + (lane & 31);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const unsigned row = 8 * (j >> 2) + 4 * L + (j & 3);
      const float a = Ly::read(vbuf[PAR], row, d, Ly::swz_v(row));
      ws.o[db][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[j], ws.o[db][0], 0, 0, 0);
    }
  }
  if (more) st.store(kbuf[PAR ^ 1], vbuf[PAR ^ 1]);
  __syncthreads();
}

// With D = 128 the fp32 operands and staging registers need more than the
// 256 registers two waves per SIMD leave, so that variant runs one wave per
// SIMD.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : 2)))
void attn_step_f32_kernel(StepParams p) {
  typedef Layout<D> Ly;
  __shared__ __attribute__((aligned(16))) char k0_raw[Ly::kTileBytes];
  __shared__ __attribute__((aligned(16))) char k1_raw[Ly::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v0_raw[Ly::kTileBytes];
  __shared__ __attribute__((aligned(16))) char v1_raw[Ly::kTileBytes];
  RA_LDS char* const kbuf[2] = {(RA_LDS char*)k0_raw, (RA_LDS char*)k1_raw};
  RA_LDS char* const vbuf[2] = {(RA_LDS char*)v0_raw, (RA_LDS char*)v1_raw};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  WorkItem wi;
  if (!decode_work<kBQ>(p, wi)) return;
  const TilePlan tp = plan_tiles(p, wi.qglob0, wi.qglob0 + wi.qrows - 1);
  if (tp.n == 0) {
    store_identity<D, kThreads>(p, wi);
    return;
  }

  const int wrow = 32 * wave + (lane & 31);
  const bool row_ok = wrow < wi.qrows;
  const long long qg = wi.qglob0 + wrow;
  // the row's visible keys (any position: past the work item's rows the
  // values are not used)
  const long long row_lo = key_lo(p, qg), row_hi = key_hi(p, qg);
  const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + wrow) * p.Hq + wi.h;  // (b, row, h)

  TileStage<D> st;
  st.init(p);
  TileCursor cur;
  cur.first(tp);
  st.load(p, wi, ktile(cur));
  WaveState<D> ws;
  {
    const float* qrow = (const float*)p.q + orow * D;
#pragma unroll
    for (int u = 0; u < D / 2; ++u) ws.q[u] = row_ok ? qrow[2 * u + (lane >> 5)] : 0.f;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) ws.o[db][0] = f32x16{};
  ws.m_ref = kNegInf;
  ws.l_part = 0.f;
  st.store(kbuf[0], vbuf[0]);
  __syncthreads();

  // unrolled by two so that buffers are named statically: iteration t uses
  // parity t mod 2
  int t = 0;
  for (; t + 1 < tp.n; t += 2) {
    step_tile<D, 0>(ws, p, tp, st, wi, cur, t, kbuf, vbuf, row_lo, row_hi, lane);
    step_tile<D, 1>(ws, p, tp, st, wi, cur, t + 1, kbuf, vbuf, row_lo, row_hi, lane);
  }
  if (t < tp.n) step_tile<D, 0>(ws, p, tp, st, wi, cur, t, kbuf, vbuf, row_lo, row_hi, lane);

  finish_rows<D, 1>(p, ws.o, 0, ws.m_ref * p.sl2, ws.l_part, row_ok, orow, lane);
}

template <int D>
hipError_t launch(const StepParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attn_step_f32_kernel<D>, dim3(8 * p.per_xcd), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_step_f32(const StepParams& p, int D, hipStream_t s) {
  if (D == 128) return launch<128>(p, s);
  if (D == 64) return launch<64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_step(const StepParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 0) return launch_attn_step_f32(p, D, s);
  if (dtype == 1) return launch_attn_step_bf16(p, D, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
