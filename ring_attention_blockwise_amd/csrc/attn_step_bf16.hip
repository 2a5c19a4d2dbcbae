// One ring step of blockwise attention on gfx950 for bf16 inputs, with the
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
//   * A workgroup (4 waves, one per SIMD) owns 256 consecutive query rows of
//     one (batch, query head); wave w owns rows [64w, 64w + 64) as two 32-row
//     blocks.  Every K or V operand a wave reads from LDS feeds the MFMAs of
//     both blocks, which halves the LDS read traffic per flop against 32 rows
//     per wave: LDS, not the matrix cores, is the tighter limit of this loop
//     otherwise.  Two workgroups share a CU, so each SIMD interleaves two
//     waves: while one runs its softmax on the vector ALUs, the other issues
//     MFMAs.
//   * Keys are processed in tiles of 32, double-buffered in LDS.  Both tiles
//     are copied global -> LDS by the load unit itself (buffer loads with the
//     LDS bit, 16 bytes per lane), so staging takes no registers and no LDS
//     store instructions.  Tile t+1 is started early in iteration t (after
//     the first four score products are issued) and waited for just before
//     the barrier that ends it, so its latency hides behind a tile of work.
//     The per-tile bookkeeping (which rows the next tile holds, where they
//     are) advances a small scalar cursor; the per-lane DMA offsets are
//     computed once per work item.
//   * Only key tiles with at least one visible key are visited; tiles all of
//     whose keys every row of the work item sees run first and skip the mask.
//   * Steps with fewer work items than two per CU (small rings) run a
//     second kernel: eight-wave workgroups whose two wave sets take the two
//     halves of an item's key tiles and merge their partial softmax sums
//     through LDS at the end, so every SIMD still interleaves two waves.
//
// Per-wave math (64 queries x 32 keys per tile)
//   S^T = K Q^T on 32x32x16 MFMAs.  Lane l feeds the K row sigma(l % 32),
//   sigma swapping bits 2 and 3 of the row index, which makes register r of
//   lane l hold key 16(r/8) + 8(l/32) + r%8 of query l%32.  Row max and row
//   sum are in-lane reductions plus one swap of the two lane halves.
//   O^T += V^T P^T on 32x32x16 MFMAs, 16 keys per MFMA: accumulator registers
//   8h .. 8h+7 of lane l, exponentiated and rounded to bf16, are the B
//   operand of keys 16h + [0, 16) in natural order; the A operand (8
//   consecutive keys of one column d of V per lane) comes from the row-major
//   V tile through two transposing LDS reads (ds_read_b64_tr_b16).
//   The softmax runs in base 2 (exp2 of scale*log2(e)-scaled scores) in fp32
//   with a lazily moved reference maximum.
#include "attn_common.h"

namespace ra {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kThreads = 256;  // 4 waves
constexpr int kQB = 2;         // 32-row query blocks per wave
constexpr int kBQBf16 = 4 * 32 * kQB;  // workgroup rows
static_assert(kBK == 32, "one 32x32 score block per query block and tile");

template <int D>
struct Layout {
  static constexpr int kRowBytes = 2 * D;   // a key row in HBM
  static constexpr int kCPR = kRowBytes / 16;
  // K tile in LDS: 32 rows of 2D bytes; 16-byte chunk c of row r sits at
  // chunk c ^ ksw(r), so the 16 rows one operand read touches per pass land
  // in distinct banks.
  static constexpr int kKStride = kRowBytes;
  static constexpr int kKTileBytes = kBK * kKStride;
  // V tile in LDS: 32 rows of 2D bytes; chunk c of row r sits at c ^ vsw(r),
  // which puts the 4 rows one transposing read touches per pass (64 bytes
  // each) in distinct banks.
  static constexpr int kVStride = kRowBytes;
  static constexpr int kVTileBytes = kBK * kVStride;
  // DMA: one instruction writes 64 consecutive 16-byte slots (1 KiB); each
  // wave copies kDma of them per tile for K and as many for V.
  static constexpr int kDma = kKTileBytes / 1024 / 4;
  static_assert(kKTileBytes % 4096 == 0, "K and V instructions split evenly over the 4 waves");

  __device__ static unsigned ksw(unsigned r) { return (kCPR == 16 ? r : r >> 1) & (kCPR - 1); }
  __device__ static unsigned vsw(unsigned r) { return (4u * ((r & 3u) >> (kCPR == 16 ? 0 : 1))) & (kCPR - 1); }
};

template <int D>
struct WaveState {
  bf16x8 q[kQB][D / 16];      // Q^T operands: Q[row][16u + 8(l/32) .. +7]
  f32x16 o[D / 32][kQB];      // O^T accumulators
  float mb[kQB];              // reference maximum times scale log2(e); kMbNone before any key
  float l_part[kQB];          // this lane's share of the row sum
};

// Per-thread addresses.  They are cheap to derive from the thread id, so each
// tile derives them again from a laundered copy of it instead of keeping them
// in registers across the loop; the four-wave kernel keeps one, the V read
// base, for the whole item (derived per tile it cost about 15 vector
// instructions of a tile's ~140; the key-split kernels, short of registers,
// still derive it per tile).
template <int D>
struct Lane {
  typedef Layout<D> Ly;
  unsigned lane, row_bytes;
  int wave;

  __device__ Lane(unsigned row_bytes_, int wave_) : row_bytes(row_bytes_), wave(wave_) {
    unsigned tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63u;
  }
  // K operand read of unit u: kb0() ^ 32u (row sigma(l % 32), chunk 2u + l/32)
  __device__ unsigned kb0() const {
    const unsigned rho = sigma(lane & 31u);
    return (rho * Ly::kKStride) | (16u * (Ly::ksw(rho) ^ (lane >> 5)));
  }
  // Transposing V reads.  In each 16-lane group g (lanes 16g + s) lane s
  // addresses key row r = 8(g/2) + s/4 (+16h for key half h, +4 for the
  // second read) at column d = 32db + 16(g%2) + 4(s%4); the read hands lane s
  // element s%4 of the chunk of lane 4j + s/4 as its element j, i.e. column
  // 32db + 16(g%2) + s of key rows +j: the A operand of the PV MFMA.
  // r mod 4 = s/4 whatever h, so vsw(r) is fixed per lane and the address of
  // block db is vb0() ^ 64 db plus a whole number of rows.
  __device__ unsigned vb0() const {
    const unsigned g = lane >> 4, s = lane & 15u;
    const unsigned r = 8u * (g >> 1) + (s >> 2);
    const unsigned x = 2u * (g & 1u) + ((s & 3u) >> 1);  // chunk of d within block 0
    return r * Ly::kVStride + 16u * (x ^ Ly::vsw(r)) + 2u * (4u * (s & 1u));
  }
  // Tile offset of the chunk this lane copies with DMA instruction i: slot s
  // of a tile holds row s / kCPR, chunk (s % kCPR) ^ sw(row).
  __device__ unsigned dma_offset(int i, bool v) const {
    const unsigned slot = (wave * Ly::kDma + i) * 64 + lane;
    const unsigned r = slot / Ly::kCPR;
    return r * row_bytes + 16u * ((slot % Ly::kCPR) ^ (v ? Ly::vsw(r) : Ly::ksw(r)));
  }
};

// DMA staging of K and V tiles for one work item.  kLazy: the lane's chunk
// offsets are derived again at each copy (from a laundered thread id) instead
// of being held in registers across the loop; the eight-wave kernel and the
// masked instantiations, whose loops carry a few more values, need those
// registers.
template <int D, bool kLazy>
struct Stager {
  typedef Layout<D> Ly;
  const char* khead;   // row 0 of this (batch, kv head) in K
  const char* vhead;
  unsigned row_bytes;
  unsigned ko[kLazy ? 1 : Ly::kDma], vo[kLazy ? 1 : Ly::kDma];  // this lane's chunk offsets in a tile
  int wave;

  __device__ void init(const StepParams& p, const WorkItem& wi, const Lane<D>& ln) {
    row_bytes = ln.row_bytes;
    const long long head = ((long long)wi.b * p.Sk * p.Hkv + wi.g) * (long long)(D * 2);
    khead = (const char*)p.k + head;
    vhead = (const char*)p.v + head;
    wave = ln.wave;
    if (!kLazy) {
#pragma unroll
      for (int i = 0; i < Ly::kDma; ++i) {
        ko[i] = ln.dma_offset(i, false);
        vo[i] = ln.dma_offset(i, true);
      }
    }
  }

  // Starts the copy of the tile at cursor c into kdst / vdst.  Rows past
  // `count` load as 0: masked keys for K, zero-weighted values for V.
  __device__ void issue(const TileCursor& c, RA_LDS char* kdst, RA_LDS char* vdst) const {
    const long long off = c.local0 * (long long)row_bytes;
    const int nrec = (c.count() - 1) * (int)row_bytes + 2 * D;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(khead + off), (short)0, nrec, kRsrcWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vhead + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < Ly::kDma; ++i) {
      RA_LDS char* kd = kdst + (wave * Ly::kDma + i) * 1024;
      RA_LDS char* vd = vdst + (wave * Ly::kDma + i) * 1024;
      unsigned kof, vof;
      if (kLazy) {
        const Lane<D> ln(row_bytes, wave);
        kof = ln.dma_offset(i, false);
        vof = ln.dma_offset(i, true);
      } else {
        kof = ko[i];
        vof = vo[i];
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (RA_LDS void*)kd, 16, (int)kof, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (RA_LDS void*)vd, 16, (int)vof, 0, 0, 0);
    }
  }
};

__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Iteration t.  PAR = t mod 2 names the LDS buffers statically: tile t is read
// from kbuf[PAR] / vbuf[PAR]; tile t+1 is started first, into kbuf[PAR ^ 1] /
// vbuf[PAR ^ 1].
// Tile t of the plan from buffer PAR while tile t+1 is copied into PAR ^ 1.
// te: end of this wave group's tiles (a tile at or past it only keeps the
// group in step with the other at the barrier); phase: 0 or 1, which of the
// two wave sets sharing each SIMD this is.
template <int D, int PAR, bool kExt, bool kKS>
__device__ inline void step_tile(WaveState<D>& ws, const StepParams& p, const TilePlan& tp, const WorkItem& wi,
                                 const Stager<D, kKS || kExt>& st, TileCursor& cur, int t, int te, unsigned phase,
                                 RA_LDS char* const* kbuf, RA_LDS char* const* vbuf, const RA_LDS int* row_lo,
                                 const RA_LDS int* row_hi, int lane, int wave, unsigned vb0) {
  if (kKS && t >= te) {
    __syncthreads();
    return;
  }
  const Lane<D> ln((unsigned)(p.Hkv * D * 2), wave);
  const TileCursor ti = cur;
  // the scores' first two K operands are read before the scalar work of the
  // next tile's cursor, which then covers their latency
  const unsigned kb0 = ln.kb0();
  const bf16x8 a0 = __builtin_bit_cast(bf16x8, lds_load16(kbuf[PAR], kb0));
  const bf16x8 a1 = __builtin_bit_cast(bf16x8, lds_load16(kbuf[PAR], kb0 ^ 32u));
  // Two wave sets share each SIMD (two workgroups of a CU, or the two groups
  // of an eight-wave workgroup); the wave arbiter favours the older, which
  // then finishes its (equal) work long before the younger.  Swapping the
  // issue priority every 64 tiles (32 in the key split, whose wave sets walk
  // fewer tiles), in opposite phase for the two (dispatch fills one slot on
  // each of the 256 CUs before the second), lets both progress at about the
  // same rate.  Measured on the 131k and 64k rings: a period of 64 or 128
  // tiles beats 32 by ~1% and 8 or 16 do not; 256 or no swap lose 3-4%.
  if ((((unsigned)t >> (kKS ? 5 : 6)) ^ (kKS ? phase : (blockIdx.x >> 8))) & 1u)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
  const bool more = t + 1 < (kKS ? te : tp.n);
  if (more) cur.advance(tp);

  // S^T = K Q^T; masked: (tiles past the unmasked ones only; a uniform
  // branch) the keys of the tile each row may not see are set to -inf: keys
  // below lim (the causal diagonal, a span's ragged end, a packed sequence's
  // end) and, with a window or packed sequences, from lo on are visible.  The
  // sign bit of each distance selects -inf with a bitfield insert (no compare
  // masks, which would take scalar registers).
  f32x16 s[kQB];
  const int L = lane >> 5;
  // (again, in the rare path below)
  auto scores = [&]() {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(kbuf[PAR], kb0 ^ (32u * u)));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.q[qb][u], s[qb], 0, 0, 0);
    }
  };
  auto mask = [&]() {
    if (!ti.masked()) return;
    const long long d0 = wi.qglob0 - ti.glob0 + 1;
    const int dc = p.causal ? (int)max(-1024LL, min(1024LL, d0)) : 1024;
    const int base = kExt ? (int)max(-(1LL << 30), min(1LL << 30, ti.glob0 - wi.qglob0)) : 0;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int ri = 64 * wave + 32 * qb + (lane & 31);
      int lim = min(ti.count(), max(0, dc + ri));
      if (kExt) lim = max(0, min(ti.count(), row_hi[ri] + 1 - base));
      // key of register r is 16(r/8) + r%8 + 8L: it is visible iff
      // lim - 8L - 1 - (16(r/8) + r%8) >= 0 and, with a lower end lo,
      // 16(r/8) + r%8 + 8L - lo >= 0; one sign test of the two ORed
      const int lim_l = lim - 8 * L - 1;
      const int lo_l = kExt ? 8 * L - max(-1, min(33, row_lo[ri] - base)) : 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int d = lim_l - (16 * (r >> 3) + (r & 7));
        if (kExt) d |= lo_l + (16 * (r >> 3) + (r & 7));
        asm volatile("" : "+v"(d));
        const unsigned m = (unsigned)(d >> 31);
        s[qb][r] = __uint_as_float((m & 0xff800000u) | (~m & __float_as_uint(s[qb][r])));
      }
    }
  };
  // The scores' first four products (the operands read above) go to the
  // matrix core before the next tile's copy instructions are issued, so the
  // copy's address setup and its four load instructions issue while those
  // products run (131k and 64k rings +0.5% and +0.8% against issuing the
  // copy first, same box).  The empty asm keeps the products above the
  // branch around the copy.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) s[qb] = f32x16{};
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u ? a1 : a0, ws.q[qb][u], s[qb], 0, 0, 0);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) asm volatile("" : "+v"(s[qb]));
  if (more) st.issue(cur, kbuf[PAR ^ 1], vbuf[PAR ^ 1]);
#pragma unroll
  for (int u = 2; u < D / 16; ++u) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(kbuf[PAR], kb0 ^ (32u * u)));
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ws.q[qb][u], s[qb], 0, 0, 0);
  }
  // Scheduling groups kept from the form that issued all sixteen products in
  // this block: they name four products more than the twelve left here, and
  // the scheduler places each later operand read just before its pair (one
  // read in flight).  A pattern that matches the block (read, then its two
  // products) was 0.3-0.6% slower, and reading one operand ahead gained
  // nothing: the other wave of the SIMD covers these LDS round trips.
#pragma unroll
  for (int u = 2; u < D / 16; ++u) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_sched_barrier(0);
  mask();

  // P = exp2(S sl2 - mb) against the row's current reference mb (log2
  // units), rounded to bf16 as the B operand of O^T += V^T P^T, and this
  // lane's share of the tile's row sum, which adds the rounded probabilities
  // (the weights the products apply) two at a time: v_dot2 with a pair of
  // ones.  A masked score gives 0.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pb[kQB][2];
  float lt[kQB];
  auto probabilities = [&](int qb) {
    lt[qb] = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * hf + e], p.sl2, -ws.mb[qb]));
      pb[qb][hf] = __builtin_convertvector(x, bf16x8);
      const u32x4 pw = __builtin_bit_cast(u32x4, pb[qb][hf]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the element goes through a scalar: a bit cast taken straight from
        // pw[e] compiles to element 0 for every e with this compiler
        const unsigned w = pw[e];
        lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, lt[qb], false);
      }
      // one 8-key group at a time keeps the exponentials' temporaries few
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  bool over = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    probabilities(qb);
    over |= !(lt[qb] <= kTauSum);
  }
  // A lane's tile sum bounds each of its probabilities, so while no sum
  // passes 2^kTau every P is at most 2^kTau and the reference stays (the
  // common case).  Otherwise (the first visible tile, where mb is still
  // kMbNone, or scores that grew) the scores are formed again from the K
  // tile, still in LDS (keeping them alive under the probabilities would
  // not fit the registers), the rows whose tile maximum lies more than kTau
  // above the reference move it there, O and l are rescaled, and the
  // probabilities are taken again.
  if (__builtin_amdgcn_ballot_w64(over)) {
    scores();
    mask();
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float t = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) t = fmaxf(t, s[qb][r]);
      const float mb = max_halves(t) * p.sl2;
      if (mb - ws.mb[qb] > kTau) {
        const float alpha = __builtin_amdgcn_exp2f(ws.mb[qb] - mb);
        ws.mb[qb] = mb;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) ws.o[db][qb] *= alpha;
        ws.l_part[qb] *= alpha;
      }
      probabilities(qb);
    }
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    ws.l_part[qb] += lt[qb];
    // materialise the row sum here: otherwise the sums sink into the next
    // tile and keep this tile's probabilities alive across it
    asm volatile("" : "+v"(ws.l_part[qb]));
  }

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned off = (vb0 ^ (64u * db)) + 16 * hf * Layout<D>::kVStride;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vbuf[PAR] + off));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vbuf[PAR] + off + 4 * Layout<D>::kVStride));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        ws.o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][hf], ws.o[db][qb], 0, 0, 0);
    }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
  for (int i = 2; i < 2 * (D / 32); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);

  wait_loads();
  __syncthreads();
}

// One wave set's pass over tiles [tb, te) of the plan (iters iterations, the
// same for both sets of an eight-wave workgroup): tile tb in flight while Q
// is read, then the tiles through buffers kbuf, vbuf.
template <int D, bool kExt, bool kKS>
__device__ __attribute__((always_inline)) inline void fwd_pass(WaveState<D>& ws, const StepParams& p,
                                                               const TilePlan& tp, const WorkItem& wi, int tb, int te,
                                                               int iters, unsigned phase, RA_LDS char* const* kbuf,
                                                               RA_LDS char* const* vbuf, const RA_LDS int* row_lo,
                                                               const RA_LDS int* row_hi, int lane, int wave) {
  Stager<D, kKS || kExt> st;
  st.init(p, wi, Lane<D>((unsigned)(p.Hkv * D * 2), wave));
  TileCursor cur;
  cur.first(tp);
  if (kKS && tb > 0) cur.seek(tp, tb);
  if (!kKS || tb < te) st.issue(cur, kbuf[0], vbuf[0]);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int wrow = 64 * wave + 32 * qb + (lane & 31);
    const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + wrow) * p.Hq + wi.h;  // (b, row, h)
    const uint16_t* qrow = (const uint16_t*)p.q + orow * D;
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
      ws.q[qb][u] = wrow < wi.qrows ? *(const bf16x8*)(qrow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) ws.o[db][qb] = f32x16{};
    ws.mb[qb] = kMbNone;
    ws.l_part[qb] = 0.f;
  }
  wait_loads();
  __syncthreads();

  // main loop, unrolled by two so that buffers are named statically:
  // iteration i uses parity i mod 2.
  const int tend = kKS ? tb + iters : tp.n;
  int t = kKS ? tb : 0;
  for (; t + 1 < tend; t += 2) {
    step_tile<D, 0, kExt, kKS>(ws, p, tp, wi, st, cur, t, te, phase, kbuf, vbuf, row_lo, row_hi, lane, wave,
                               Lane<D>((unsigned)(p.Hkv * D * 2), wave).vb0());
    step_tile<D, 1, kExt, kKS>(ws, p, tp, wi, st, cur, t + 1, te, phase, kbuf, vbuf, row_lo, row_hi, lane, wave,
                               Lane<D>((unsigned)(p.Hkv * D * 2), wave).vb0());
  }
  if (t < tend)
    step_tile<D, 0, kExt, kKS>(ws, p, tp, wi, st, cur, t, te, phase, kbuf, vbuf, row_lo, row_hi, lane, wave,
                               Lane<D>((unsigned)(p.Hkv * D * 2), wave).vb0());
}

// The kernel above: four waves (256 query rows, 64 per wave) walk every key
// tile of the work item; two workgroups per CU.  This one (kKS = true; the
// template keeps the shared code paths in step with it): eight waves, two sets of four over the same 256 rows, the
// first taking the first half of the item's key tiles and the second the
// rest; at the end the second hands its (O, m, l) to the first through LDS,
// which merges them (the softmax merge of two partial sums) and writes the
// rows.  For steps with fewer work items than two per CU: one workgroup per
// CU still keeps two waves on every SIMD.
template <int D, bool kExt>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16_kernel(StepParams p) {
  typedef Layout<D> Ly;
  __shared__ __attribute__((aligned(16))) char k0_raw[Ly::kKTileBytes];
  __shared__ __attribute__((aligned(16))) char k1_raw[Ly::kKTileBytes];
  __shared__ __attribute__((aligned(16))) char v0_raw[Ly::kVTileBytes];
  __shared__ __attribute__((aligned(16))) char v1_raw[Ly::kVTileBytes];
  RA_LDS char* const kbuf[2] = {(RA_LDS char*)k0_raw, (RA_LDS char*)k1_raw};
  RA_LDS char* const vbuf[2] = {(RA_LDS char*)v0_raw, (RA_LDS char*)v1_raw};
  __shared__ int lo_raw[kBQBf16], hi_raw[kBQBf16];
  const RA_LDS int* row_lo = (const RA_LDS int*)lo_raw;
  const RA_LDS int* row_hi = (const RA_LDS int*)hi_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  WorkItem wi;
  if (!decode_work<kBQBf16>(p, wi)) return;
  const TilePlan tp = plan_tiles(p, wi.qglob0, wi.qglob0 + wi.qrows - 1);
  if (tp.n == 0) {
    store_identity<D, kThreads>(p, wi);
    return;
  }

  if (kExt) {
    // visible key range of each row of the work item (window, packed
    // sequences), relative to the item's first row and clamped to +-2^30
    for (int r = threadIdx.x; r < kBQBf16; r += kThreads) {
      const long long t = wi.qglob0 + r;
      lo_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_lo(p, t) - wi.qglob0));
      hi_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_hi(p, t) - wi.qglob0));
    }
  }

  // prologue: tile 0 in flight while Q is read
  Stager<D, kExt> st;
  st.init(p, wi, Lane<D>((unsigned)(p.Hkv * D * 2), wave));
  TileCursor cur;
  cur.first(tp);
  st.issue(cur, kbuf[0], vbuf[0]);
  WaveState<D> ws;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int wrow = 64 * wave + 32 * qb + (lane & 31);
    const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + wrow) * p.Hq + wi.h;  // (b, row, h)
    const uint16_t* qrow = (const uint16_t*)p.q + orow * D;
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
      ws.q[qb][u] = wrow < wi.qrows ? *(const bf16x8*)(qrow + 16 * u + 8 * (lane >> 5)) : bf16x8{};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) ws.o[db][qb] = f32x16{};
    ws.mb[qb] = kMbNone;
    ws.l_part[qb] = 0.f;
  }
  wait_loads();
  __syncthreads();

  // main loop, unrolled by two so that buffers are named statically:
  // iteration t uses parity t mod 2.  The V read base stays in a register for
  // the whole item.
  const unsigned vb0 = Lane<D>((unsigned)(p.Hkv * D * 2), wave).vb0();
  int t = 0;
  for (; t + 1 < tp.n; t += 2) {
    step_tile<D, 0, kExt, false>(ws, p, tp, wi, st, cur, t, tp.n, 0u, kbuf, vbuf, row_lo, row_hi, lane, wave, vb0);
    step_tile<D, 1, kExt, false>(ws, p, tp, wi, st, cur, t + 1, tp.n, 0u, kbuf, vbuf, row_lo, row_hi, lane,
                                  wave, vb0);
  }
  if (t < tp.n)
    step_tile<D, 0, kExt, false>(ws, p, tp, wi, st, cur, t, tp.n, 0u, kbuf, vbuf, row_lo, row_hi, lane, wave, vb0);

#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int wrow = 64 * wave + 32 * qb + (lane & 31);
    const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + wrow) * p.Hq + wi.h;
    finish_rows<D, kQB>(p, ws.o, qb, ws.mb[qb], ws.l_part[qb], wrow < wi.qrows, orow, lane);
  }
}

template <int D, bool kExt, bool kKS>
__global__ __launch_bounds__(kKS ? 2 * kThreads : kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_step_bf16_ks_kernel(StepParams p) {
  typedef Layout<D> Ly;
  // the hand-over below puts 16 KB per wave and round into two tile buffers
  static_assert(!kKS || (D == 128 && Ly::kKTileBytes == 8192 && Ly::kVTileBytes == 8192), "kKS needs D = 128");
  constexpr int kT = kKS ? 2 * kThreads : kThreads;
  __shared__ __attribute__((aligned(16))) char k0_raw[Ly::kKTileBytes];
  __shared__ __attribute__((aligned(16))) char k1_raw[Ly::kKTileBytes];
  __shared__ __attribute__((aligned(16))) char v0_raw[Ly::kVTileBytes];
  __shared__ __attribute__((aligned(16))) char v1_raw[Ly::kVTileBytes];
  __shared__ __attribute__((aligned(16))) char k2_raw[kKS ? Ly::kKTileBytes : 16];
  __shared__ __attribute__((aligned(16))) char k3_raw[kKS ? Ly::kKTileBytes : 16];
  __shared__ __attribute__((aligned(16))) char v2_raw[kKS ? Ly::kVTileBytes : 16];
  __shared__ __attribute__((aligned(16))) char v3_raw[kKS ? Ly::kVTileBytes : 16];
  __shared__ __attribute__((aligned(16))) float xm_raw[kKS ? 4 * 64 * 2 * kQB : 4];
  __shared__ int lo_raw[kBQBf16], hi_raw[kBQBf16];
  const RA_LDS int* row_lo = (const RA_LDS int*)lo_raw;
  const RA_LDS int* row_hi = (const RA_LDS int*)hi_raw;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = kKS ? wv >> 2 : 0;
  const int wave = wv & 3;

  WorkItem wi;
  if (!decode_work<kBQBf16>(p, wi)) return;
  const TilePlan tp = plan_tiles(p, wi.qglob0, wi.qglob0 + wi.qrows - 1);
  if (tp.n == 0) {
    store_identity<D, kT>(p, wi);
    return;
  }

  if (kExt) {
    // visible key range of each row of the work item (window, packed
    // sequences), relative to the item's first row and clamped to +-2^30
    for (int r = threadIdx.x; r < kBQBf16; r += kT) {
      const long long t = wi.qglob0 + r;
      lo_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_lo(p, t) - wi.qglob0));
      hi_raw[r] = (int)max(-(1LL << 30), min(1LL << 30, key_hi(p, t) - wi.qglob0));
    }
  }

  WaveState<D> ws;
  const int half = kKS ? (tp.n + 1) / 2 : tp.n;
  if (grp == 0) {
    RA_LDS char* const kbuf[2] = {(RA_LDS char*)k0_raw, (RA_LDS char*)k1_raw};
    RA_LDS char* const vbuf[2] = {(RA_LDS char*)v0_raw, (RA_LDS char*)v1_raw};
    fwd_pass<D, kExt, kKS>(ws, p, tp, wi, 0, half, half, 0u, kbuf, vbuf, row_lo, row_hi, lane, wave);
  } else {
    RA_LDS char* const kbuf[2] = {(RA_LDS char*)k2_raw, (RA_LDS char*)k3_raw};
    RA_LDS char* const vbuf[2] = {(RA_LDS char*)v2_raw, (RA_LDS char*)v3_raw};
    fwd_pass<D, kExt, kKS>(ws, p, tp, wi, half, tp.n, half, 1u, kbuf, vbuf, row_lo, row_hi, lane, wave);
  }

  if (kKS) {
    // The second set's partial sums to the first: its (m, l) per row into
    // xm, its O in rounds of two 32-column blocks, 16 KB per wave per round,
    // through the idle tile buffers (two per wave).  Exponents relative to
    // each set's own reference m: O = a0 O0 + a1 O1, l = a0 l0 + a1 l1 with
    // a = exp2((m_set - m) sl2) for m = max(m0, m1) (a set that saw no key
    // has m = -inf and a = 0).
    RA_LDS float* const xm = (RA_LDS float*)xm_raw + (wave * 64 + lane) * 2 * kQB;
    float a0[kQB], a1[kQB];
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
      RA_LDS char* const xb0 = wave == 0   ? (RA_LDS char*)k0_raw
                               : wave == 1 ? (RA_LDS char*)v0_raw
                               : wave == 2 ? (RA_LDS char*)k2_raw
                                           : (RA_LDS char*)v2_raw;
      RA_LDS char* const xb1 = wave == 0   ? (RA_LDS char*)k1_raw
                               : wave == 1 ? (RA_LDS char*)v1_raw
                               : wave == 2 ? (RA_LDS char*)k3_raw
                                           : (RA_LDS char*)v3_raw;
      if (grp == 1) {
        if (r == 0) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            xm[qb] = ws.mb[qb];
            xm[kQB + qb] = ws.l_part[qb];
          }
        }
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x16& o = ws.o[2 * r + d2][qb];
              const f32x4 v = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
              const int slot = (d2 * kQB + qb) * 4 + j;  // 0 .. 15
              ((RA_LDS f32x4*)(slot < 8 ? xb0 : xb1))[(slot & 7) * 64 + lane] = v;
            }
      }
      __syncthreads();
      if (grp == 0) {
        if (r == 0) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            // a set that saw no key has kMbNone, far below the other's reference
            // (a = 0), or both have it and l = 0
            const float m0 = ws.mb[qb], m1 = xm[qb];
            const float m = fmaxf(m0, m1);
            a0[qb] = __builtin_amdgcn_exp2f(m0 - m);
            a1[qb] = __builtin_amdgcn_exp2f(m1 - m);
            ws.l_part[qb] = a0[qb] * ws.l_part[qb] + a1[qb] * xm[kQB + qb];
            ws.mb[qb] = m;
          }
        }
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int slot = (d2 * kQB + qb) * 4 + j;
              const f32x4 v = ((RA_LDS f32x4*)(slot < 8 ? xb0 : xb1))[(slot & 7) * 64 + lane];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                ws.o[2 * r + d2][qb][4 * j + e] = a0[qb] * ws.o[2 * r + d2][qb][4 * j + e] + a1[qb] * v[e];
            }
      }
      if (r + 1 < D / 64) __syncthreads();
    }
    if (grp == 1) return;
  }

#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int wrow = 64 * wave + 32 * qb + (lane & 31);
    const long long orow = ((long long)wi.b * p.Sq + wi.qlocal0 + wrow) * p.Hq + wi.h;
    finish_rows<D, kQB>(p, ws.o, qb, ws.mb[qb], ws.l_part[qb], wrow < wi.qrows, orow, lane);
  }
}

template <int D>
hipError_t launch(const StepParams& p, hipStream_t s) {
  const dim3 grid(8 * p.per_xcd);
  if constexpr (D == 128) {
    if (p.ksplit) {
      if (p.mask_ext)
        hipLaunchKernelGGL((attn_step_bf16_ks_kernel<D, true, true>), grid, dim3(2 * kThreads), 0, s, p);
      else
        hipLaunchKernelGGL((attn_step_bf16_ks_kernel<D, false, true>), grid, dim3(2 * kThreads), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.mask_ext) {
    hipLaunchKernelGGL((attn_step_bf16_kernel<D, true>), grid, dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((attn_step_bf16_kernel<D, false>), grid, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

int attn_step_rows_bf16() { return kBQBf16; }

hipError_t launch_attn_step_bf16(const StepParams& p, int D, hipStream_t s) {
  if (D == 128) return launch<128>(p, s);
  if (D == 64) return launch<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
