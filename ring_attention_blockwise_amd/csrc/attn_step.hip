// One ring step of blockwise attention on gfx950, with the log-sum-exp merge
// fused into the epilogue.
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
//   * A workgroup (4 waves, one per SIMD) owns 128 consecutive query rows of
//     one (batch, query head); wave w owns rows [32w, 32w + 32).  Two
//     workgroups share a CU, so each SIMD interleaves two waves: while one
//     runs its softmax on the vector ALUs, the other can issue MFMAs.
//   * Keys are processed in tiles of 32.  Tile t+1 is loaded into registers
//     at the start of iteration t and written to the other LDS buffer (two
//     each for K and V) at its end; the loop is unrolled by two so that every
//     LDS buffer is named statically.
//   * Only key tiles with at least one visible key are visited.  Tiles whose
//     keys every query row of the work item sees run first with no mask code;
//     tiles on the causal diagonal or cut short by the end of a span run last,
//     masked.
//   * Workgroups are ordered so that all query tiles reading the same K/V head
//     land on the same XCD (dispatch is round-robin over the 8 XCDs), which
//     keeps that head's K/V in one L2.
//
// Per-wave math (32 queries x 32 keys per tile)
//   S^T = K Q^T on MFMA 32x32 tiles: the accumulator of a 32x32 block puts one
//   query per lane (lane n and n+32 share query n) and 16 of its keys in that
//   lane's registers, so the row max and row sum of the online softmax are
//   in-lane reductions plus one lane swap across the two halves.
//   O^T += V^T P^T on MFMA: P^T is the exponentiated accumulator itself (bf16
//   rounded for the bf16 path), with the MFMA's reduction index mapped onto the
//   keys in the order the accumulator holds them.  The bf16 path stages V
//   transposed in LDS, keys permuted into that same order, so each V^T operand
//   is one 16-byte LDS read; the f32 path keeps V row-major and reads scalars.
//   The softmax runs in base 2 (exp2 of scale*log2(e)-scaled scores) in fp32.
//   The running maximum is only moved when it grows by more than 2^8 in the
//   exponent, so the O rescale is skipped on most tiles; probabilities stay
//   below 2^8 and the final division by the row sum makes the result exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

#define RA_LDS __attribute__((address_space(3)))

namespace ra {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kThreads = 256;              // 4 waves
constexpr int kQB = kBQ / 128;              // 32-row query blocks per wave
constexpr int kKB = kBK / 32;               // 32-key blocks per key tile
constexpr int kWavesPerSimd = kQB == 1 ? 2 : 1;  // register budget 256 or 512
static_assert(kBQ == 4 * 32 * kQB, "workgroup rows");
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Grow the reference maximum only when probabilities would exceed 2^kTau.
constexpr float kTau = 8.0f;

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
// LDS tile layout: 32 key rows of D elements, row-major, 16-byte chunks.  The
// chunk index is XOR-swizzled per row so that both the MFMA operand reads and
// the tile fills hit distinct banks:
//   K: chunk ^ (row mod chunks)      -- 32 rows, one chunk per lane
//   V: chunk ^ (4 (row mod 4))       -- transposing reads, 4 rows x 4 chunks
template <int CPR>
__device__ inline unsigned swz_k(unsigned row) { return row & (CPR - 1); }
template <int CPR>
__device__ inline unsigned swz_v(unsigned row) { return (4u * (row & 3u)) & (CPR - 1); }

// ---------------------------------------------------------------------------
// Element-type traits.  Both variants produce S^T and O^T in the 32x32 MFMA
// accumulator layout: lane l, register r holds row 8(r/4) + 4(l/32) + r%4 and
// column l%32.
template <int D_>
struct Bf16 {
  static constexpr int D = D_;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kCPR = kRowBytes / 16;  // 16-byte chunks per row
  typedef uint16_t Elem;
  struct QFrag { bf16x8 f[kQB][D / 16]; };

  // Q^T operand of block qb: lane l holds Q[query l%32][16 dc + 8 (l/32) .. +7].
  __device__ static void load_q(QFrag& q, int qb, const Elem* row, bool ok, int lane) {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      q.f[qb][dc] = ok ? *(const bf16x8*)(row + 16 * dc + 8 * (lane >> 5)) : bf16x8{};
  }

  // One K operand read of S^T block kb (keys 32kb..32kb+31 of the tile),
  // reduction over d in [16u, 16u+16), feeding the MFMA of every query block.
  static constexpr int kSUnits = D / 16;
  __device__ static void s_unit(f32x16* acc, const RA_LDS char* kt, int kb, int u, const QFrag& q, int lane) {
    const unsigned row = 32 * kb + (lane & 31);
    const unsigned c = 2 * u + (lane >> 5);
    const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(kt, row * kRowBytes + ((c ^ swz_k<kCPR>(row)) * 16)));
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      acc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.f[qb][u], acc[qb], 0, 0, 0);
  }

  // V is staged into LDS transposed: row d (64 bytes) holds the 32 keys of
  // the tile in the order the S^T accumulator holds them,
  //   pos(k) = 16 (k / 16) + 8 ((k / 4) % 2) + 4 ((k / 8) % 2) + k % 4,
  // i.e. bits 2 and 3 of k swapped.  The 8 keys one lane feeds to a P V MFMA
  // are then 16 contiguous bytes (one ds_read_b128).  The 16-byte chunk pos/8
  // of row d sits at chunk ^ (((d >> 2) ^ (d >> 4)) & 3), conflict-free for
  // both the reads (16 consecutive rows) and the writes (8 rows x 4 chunks).
  static_assert(kBK == 32, "V^T rows hold one 32-key tile");
  __device__ static unsigned vt_swz(unsigned d) { return ((d >> 2) ^ (d >> 4)) & 3u; }
  __device__ static unsigned vt_pos(unsigned k) {
    return (k & ~15u) | (((k >> 2) & 1u) << 3) | (((k >> 3) & 1u) << 2) | (k & 3u);
  }

  // Staging of one V tile: thread t takes keys 2m, 2m+1 (m = t % 16) at
  // d-chunk c = t / 16 (8 values of d), packs each (V[2m][d], V[2m+1][d])
  // into a dword and writes the 8 dwords to rows 8c .. 8c+7 of V^T.
  struct VStage {
    u32x4 ra, rb;
    unsigned goff;       // global byte offset of (row 2m, chunk c) in a full tile
    unsigned wbase[2];   // LDS byte offset for rows 8c + 4h, h = 0, 1
    bool active;

    __device__ void init(unsigned row_bytes) {
      const unsigned m = threadIdx.x % 16, c = threadIdx.x / 16;
      active = c < D / 8;
      goff = 2 * m * row_bytes + c * 16;
      const unsigned pos = vt_pos(2 * m);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned d = 8 * c + 4 * h;
        wbase[h] = d * 64 + (((pos >> 3) ^ vt_swz(d)) * 16) + (pos & 7) * 2;
      }
    }
    __device__ void load(const char* src, int count, unsigned row_bytes) {
      if (!active) return;
      const unsigned m = threadIdx.x % 16, c = threadIdx.x / 16;
      if (count == kBK) {
        ra = *(const u32x4*)(src + goff);
        rb = *(const u32x4*)(src + goff + row_bytes);
      } else {
        ra = *(const u32x4*)(src + min((int)(2 * m), count - 1) * row_bytes + c * 16);
        rb = *(const u32x4*)(src + min((int)(2 * m + 1), count - 1) * row_bytes + c * 16);
      }
    }
    __device__ void store(RA_LDS char* dst) const {
      if (!active) return;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned x = ra[j >> 1], y = rb[j >> 1];
        const unsigned w = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        *(RA_LDS unsigned*)(dst + wbase[j >> 2] + (j & 3) * 64) = w;
      }
    }
  };

  // O^T[db][qb] += V^T P^T over the 16 keys 32kb + 16hf + [0, 16) of the
  // tile.  The MFMA consumes accumulator registers 8hf..8hf+7 of S^T block kb
  // (already exponentiated, rounded to bf16 here), i.e. reduction index
  // 8(l/32)+e <-> key 32kb + 16hf + 8(e/4) + 4(l/32) + e%4; V^T row
  // 32db + l%32 holds exactly those keys at chunk 2hf + l/32.
  __device__ static void pv_group(f32x16 (*o)[kQB], const RA_LDS char* vt, const f32x16 (*p)[kQB], int kb,
                                  int hf, int lane) {
    bf16x8 pb[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[kb][qb][8 * hf + e];
      pb[qb] = __builtin_convertvector(x, bf16x8);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned d = 32 * db + (lane & 31);
      const unsigned chunk = 2 * (16 * kb + 8 * hf) / 8 + (lane >> 5);
      const bf16x8 a = __builtin_bit_cast(bf16x8, lds_load16(vt, d * 64 + ((chunk ^ vt_swz(d)) * 16)));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], o[db][qb], 0, 0, 0);
    }
  }
};

template <int D_>
struct F32 {
  static constexpr int D = D_;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kCPR = kRowBytes / 16;
  typedef float Elem;
  struct QFrag { float f[kQB][D / 2]; };

  // Q^T operand of the 32x32x2 f32 MFMA: lane l holds Q[query l%32][2u + l/32].
  __device__ static void load_q(QFrag& q, int qb, const Elem* row, bool ok, int lane) {
#pragma unroll
    for (int u = 0; u < D / 2; ++u) q.f[qb][u] = ok ? row[2 * u + (lane >> 5)] : 0.f;
  }

  __device__ static float lds_f(const RA_LDS char* t, unsigned row, unsigned d, unsigned swz) {
    return *(const RA_LDS float*)(t + row * kRowBytes + (((d >> 2) ^ swz) * 16) + (d & 3) * 4);
  }

  // One K operand of S^T block kb: reduction over d in {2u, 2u+1}.
  static constexpr int kSUnits = D / 2;
  __device__ static void s_unit(f32x16* acc, const RA_LDS char* kt, int kb, int u, const QFrag& q, int lane) {
    const unsigned row = 32 * kb + (lane & 31);
    const float a = lds_f(kt, row, 2 * u + (lane >> 5), swz_k<kCPR>(row));
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) acc[qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, q.f[qb][u], acc[qb], 0, 0, 0);
  }

  // V is staged row-major with the V swizzle (read back with scalar reads).
  struct VStage {
    static constexpr int kPer = kBK * kCPR / kThreads;
    u32x4 r[kPer];
    unsigned goff[kPer], woff[kPer];
    __device__ void init(unsigned row_bytes) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const unsigned idx = threadIdx.x + i * kThreads;
        const unsigned row = idx / kCPR, c = idx % kCPR;
        goff[i] = row * row_bytes + c * 16;
        woff[i] = row * kRowBytes + ((c ^ swz_v<kCPR>(row)) * 16);
      }
    }
    __device__ void load(const char* src, int count, unsigned row_bytes) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const unsigned idx = threadIdx.x + i * kThreads;
        const unsigned row = idx / kCPR, c = idx % kCPR;
        r[i] = *(const u32x4*)(src + (count == kBK ? goff[i] : min((int)row, count - 1) * row_bytes + c * 16));
      }
    }
    __device__ void store(RA_LDS char* dst) const {
#pragma unroll
      for (int i = 0; i < kPer; ++i) *(RA_LDS u32x4*)(dst + woff[i]) = r[i];
    }
  };

  // MFMA (kb, j) pairs reduction index l/32 with key 32kb + 8(j/4) + 4(l/32) + j%4,
  // which is the key accumulator register j of lane l holds; group hf covers
  // registers 8hf..8hf+7.
  __device__ static void pv_group(f32x16 (*o)[kQB], const RA_LDS char* vt, const f32x16 (*p)[kQB], int kb,
                                  int hf, int lane) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned d = 32 * db + (lane & 31);
#pragma unroll
      for (int j = 8 * hf; j < 8 * hf + 8; ++j) {
        const unsigned row = 32 * kb + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        const float a = lds_f(vt, row, d, swz_v<kCPR>(row));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[kb][qb][j], o[db][qb], 0, 0, 0);
      }
    }
  }
};

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
  bool masked;
};

struct TilePlan {
  int nf[2], nr[2];  // full and masked tiles per span
  long long hi[2];   // keys of the span visible to the work item's last row
  int n_full, n;

  __device__ KTile tile(const StepParams& p, int t) const {
    int s;
    long long kin;
    bool masked;
    if (t < n_full) {
      masked = false;
      s = t < nf[0] ? 0 : 1;
      kin = (long long)(s ? t - nf[0] : t) * kBK;
    } else {
      masked = true;
      const int u = t - n_full;
      s = u < nr[0] ? 0 : 1;
      kin = (long long)(nf[s] + (s ? u - nr[0] : u)) * kBK;
    }
    KTile kt;
    kt.local0 = p.ks_off[s] + kin;
    kt.glob0 = p.ks_start[s] + kin;
    kt.count = (int)min((long long)kBK, hi[s] - kin);
    kt.masked = masked;
    return kt;
  }
};

__device__ inline TilePlan plan_tiles(const StepParams& p, long long qglob0, long long qglob_last) {
  TilePlan tp;
  tp.n_full = 0;
  tp.n = 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    long long hi = 0, full = 0;
    if (s < p.nks) {
      hi = p.ks_len[s];
      full = hi;
      if (p.causal) {
        hi = min(hi, qglob_last + 1 - p.ks_start[s]);   // keys <= the last row
        full = min(hi, qglob0 + 1 - p.ks_start[s]);     // keys <= the first row
      }
      hi = max(hi, 0LL);
      full = max(full, 0LL);
    }
    tp.hi[s] = hi;
    tp.nf[s] = (int)(full / kBK);
    tp.nr[s] = (int)((hi - (long long)tp.nf[s] * kBK + kBK - 1) / kBK);
    tp.n_full += tp.nf[s];
    tp.n += tp.nf[s] + tp.nr[s];
  }
  return tp;
}

// ---------------------------------------------------------------------------
// Staging of K and V tiles through registers: each thread loads kPer 16-byte
// chunks of the K tile and of the V tile with ordinary global loads, and
// writes them to LDS (swizzled) after the tile being finished has been
// computed.  Routing the data through registers (rather than the LDS DMA path)
// lets the compiler see that the MFMA operand reads of one buffer do not depend
// on loads in flight for the other.  Rows past `count` (only in a span's last
// tile) repeat the last real row: their keys are masked to -inf (K) and
// weighted by exactly 0 (V).
template <class Tr>
struct TileStage {
  static constexpr int kPer = kBK * Tr::kCPR / kThreads;
  u32x4 k[kPer];
  unsigned goff[kPer];   // global byte offset of each K chunk in a full tile
  unsigned koff[kPer];   // its swizzled LDS byte offset
  unsigned row_bytes;    // global stride between key rows
  typename Tr::VStage vs;

  __device__ void init(const StepParams& p) {
    row_bytes = (unsigned)(p.Hkv * Tr::D * (int)sizeof(typename Tr::Elem));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const unsigned idx = threadIdx.x + i * kThreads;
      const unsigned row = idx / Tr::kCPR, c = idx % Tr::kCPR;
      goff[i] = row * row_bytes + c * 16;
      koff[i] = row * Tr::kRowBytes + ((c ^ swz_k<Tr::kCPR>(row)) * 16);
    }
    vs.init(row_bytes);
  }

  // Loads tile kt of K (is_v false) or V into the staging registers.
  __device__ void load(const StepParams& p, int b, int g, const KTile& kt, bool is_v) {
    const long long base = (((long long)b * p.Sk + kt.local0) * p.Hkv + g) * (long long)(Tr::D * sizeof(typename Tr::Elem));
    if (is_v) {
      vs.load((const char*)p.v + base, kt.count, row_bytes);
      return;
    }
    const char* src = (const char*)p.k + base;
    if (kt.count == kBK) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) k[i] = *(const u32x4*)(src + goff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const unsigned idx = threadIdx.x + i * kThreads;
        const unsigned row = idx / Tr::kCPR, c = idx % Tr::kCPR;
        k[i] = *(const u32x4*)(src + min((int)row, kt.count - 1) * row_bytes + c * 16);
      }
    }
  }

  __device__ void store_k(RA_LDS char* dst) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) *(RA_LDS u32x4*)(dst + koff[i]) = k[i];
  }
  __device__ void store_v(RA_LDS char* dst) const { vs.store(dst); }
};

// Per-wave state carried across key tiles.
template <class Tr>
struct WaveState {
  typename Tr::QFrag qf;
  f32x16 o[Tr::D / 32][kQB];  // O^T accumulators
  f32x16 s[kKB][kQB];         // S^T of the tile being finished
  float m_ref[kQB];           // reference maximum of the raw (unscaled) scores
  float l_part[kQB];          // this lane's share of the row sum
};

// Mask (masked tiles only), running maximum and, when it grows by more than
// 2^kTau, rescale of O and l.  Leaves in mb the exp2 offset of each block.
template <class Tr, bool kMasked>
__device__ inline void softmax_prep(WaveState<Tr>& ws, const StepParams& p, const KTile& ti, const long long* qg,
                                    int lane, float* mb) {
  constexpr int D = Tr::D;
  if (kMasked) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const bool vis = key < ti.count && (!p.causal || ti.glob0 + key <= qg[qb]);
          if (!vis) ws.s[kb][qb][r] = kNegInf;
        }
  }
  bool grow[kQB];
  bool any = false;
  float m_new[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, ws.s[kb][qb][r]);
    tmax = max_halves(tmax);
    m_new[qb] = fmaxf(ws.m_ref[qb], tmax);
    // -inf reference: the difference is +inf and the maximum is taken;
    // both -inf: NaN compares false and nothing moves.
    grow[qb] = (m_new[qb] - ws.m_ref[qb]) * p.sl2 > kTau;
    any |= grow[qb];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float alpha = grow[qb] ? __builtin_amdgcn_exp2f((ws.m_ref[qb] - m_new[qb]) * p.sl2) : 1.f;
      if (grow[qb]) ws.m_ref[qb] = m_new[qb];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) ws.o[db][qb] *= alpha;
      ws.l_part[qb] *= alpha;
    }
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) mb[qb] = ws.m_ref[qb] == kNegInf ? 0.f : ws.m_ref[qb] * p.sl2;
}

// Exponentials and O += V P for 16-key group grp of the tile in ws.s.
template <class Tr>
__device__ inline void softmax_pv_group(WaveState<Tr>& ws, const StepParams& p, int grp, const float* mb,
                                        float* lsum, const RA_LDS char* vt, int lane) {
  const int kb = grp >> 1, hf = grp & 1;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(ws.s[kb][qb][8 * hf + e], p.sl2, -mb[qb]));
      ws.s[kb][qb][8 * hf + e] = pr;
      lsum[qb] += pr;
    }
  Tr::pv_group(ws.o, vt, ws.s, kb, hf, lane);
}

// Iteration t.  PAR = t mod 2 names the buffers statically: tile t is read
// from kbuf[PAR] / vbuf[PAR]; tile t+1 is loaded into registers first and
// written to kbuf[PAR ^ 1] / vbuf[PAR ^ 1] at the end.
template <class Tr, int PAR, bool kMasked>
__device__ inline void step_tile(WaveState<Tr>& ws, const StepParams& p, const TilePlan& tp, TileStage<Tr>* st,
                                 int t, int b, int g, const long long* qg, RA_LDS char* const* kbuf,
                                 RA_LDS char* const* vbuf, int lane) {
  const KTile ti = tp.tile(p, t);
  const bool more = t + 1 < tp.n;
  if (more) {
    const KTile t1 = tp.tile(p, t + 1);
    st[0].load(p, b, g, t1, false);
    st[0].load(p, b, g, t1, true);
  }
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) ws.s[kb][qb] = f32x16{};
#pragma unroll
    for (int u = 0; u < Tr::kSUnits; ++u) Tr::s_unit(ws.s[kb], kbuf[PAR], kb, u, ws.qf, lane);
  }
  float mb[kQB], lsum[kQB];
  softmax_prep<Tr, kMasked>(ws, p, ti, qg, lane, mb);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) lsum[qb] = 0.f;
#pragma unroll
  for (int grp = 0; grp < 2 * kKB; ++grp)
    softmax_pv_group<Tr>(ws, p, grp, mb, lsum, vbuf[PAR], lane);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) ws.l_part[qb] += lsum[qb];
  if (more) {
    st[0].store_k(kbuf[PAR ^ 1]);
    st[0].store_v(vbuf[PAR ^ 1]);
  }
  __syncthreads();
}

template <class Tr>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
void attn_step_kernel(StepParams p) {
  constexpr int D = Tr::D;
  constexpr int kTileBytes = kBK * Tr::kRowBytes;
  // Two K and two V tile buffers, as distinct arrays.
  __shared__ __attribute__((aligned(16))) char k0_raw[kTileBytes];
  __shared__ __attribute__((aligned(16))) char k1_raw[kTileBytes];
  __shared__ __attribute__((aligned(16))) char v0_raw[kTileBytes];
  __shared__ __attribute__((aligned(16))) char v1_raw[kTileBytes];
  RA_LDS char* const kbuf[2] = {(RA_LDS char*)k0_raw, (RA_LDS char*)k1_raw};
  RA_LDS char* const vbuf[2] = {(RA_LDS char*)v0_raw, (RA_LDS char*)v1_raw};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // --- work item: XCD x (= block id mod 8) takes a contiguous run of work
  const int w = (blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (w >= p.n_work) return;
  const int qt_rev = w % p.n_qtiles;
  int rest = w / p.n_qtiles;
  const int hh = rest % p.G;
  rest /= p.G;
  const int g = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int h = g * p.G + hh;
  const int qt = p.n_qtiles - 1 - qt_rev;  // later (heavier) query tiles first
  const int qs = qt < p.qt_span0 ? 0 : 1;
  const long long q_in = (long long)(qs ? qt - p.qt_span0 : qt) * kBQ;
  const int qrows = (int)min((long long)kBQ, p.qs_len[qs] - q_in);
  const long long qlocal0 = p.qs_off[qs] + q_in;
  const long long qglob0 = p.qs_start[qs] + q_in;
  const long long qglob_last = qglob0 + qrows - 1;

  const TilePlan tp = plan_tiles(p, qglob0, qglob_last);

  if (tp.n == 0) {
    // INIT of rows that see no key of this block: the merge identity.
    if (!p.accum) {
      for (int i = threadIdx.x; i < qrows * (D / 4); i += kThreads) {
        const int r = i / (D / 4), c = i % (D / 4);
        const long long orr = ((long long)b * p.Sq + qlocal0 + r) * p.Hq + h;
        *(float4*)(p.o + orr * D + 4 * c) = float4{0.f, 0.f, 0.f, 0.f};
        if (c == 0) p.lse[orr] = kNegInf;
      }
    }
    return;
  }

  // This lane's query rows: row 32 kQB wave + 32 qb + lane % 32 of the work item.
  bool row_ok[kQB];
  long long qg[kQB], orow[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int wrow = 32 * kQB * wave + 32 * qb + (lane & 31);
    row_ok[qb] = wrow < qrows;
    qg[qb] = qglob0 + wrow;
    orow[qb] = ((long long)b * p.Sq + qlocal0 + wrow) * p.Hq + h;  // (b, row, h)
  }

  TileStage<Tr> st[1];
  st[0].init(p);

  // --- prologue: tile 0 in flight while Q is read
  st[0].load(p, b, g, tp.tile(p, 0), false);
  st[0].load(p, b, g, tp.tile(p, 0), true);
  WaveState<Tr> ws;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    Tr::load_q(ws.qf, qb, (const typename Tr::Elem*)p.q + orow[qb] * D, row_ok[qb], lane);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) ws.o[db][qb] = f32x16{};
    ws.m_ref[qb] = kNegInf;
    ws.l_part[qb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) ws.s[kb][qb] = f32x16{};
  }
  st[0].store_k(kbuf[0]);
  st[0].store_v(vbuf[0]);
  __syncthreads();

  // --- main loop: tiles every row sees, unrolled by two so that buffers
  // are named statically, then the masked tiles (no mask code runs on the
  // former).  Iteration t uses parity t mod 2 in both loops.
  int t = 0;
  for (; t + 1 < tp.n_full; t += 2) {
    step_tile<Tr, 0, false>(ws, p, tp, st, t, b, g, qg, kbuf, vbuf, lane);
    step_tile<Tr, 1, false>(ws, p, tp, st, t + 1, b, g, qg, kbuf, vbuf, lane);
  }
  if (t < tp.n_full) step_tile<Tr, 0, false>(ws, p, tp, st, t++, b, g, qg, kbuf, vbuf, lane);
  for (; t < tp.n; ++t) {
    if (t & 1)
      step_tile<Tr, 1, true>(ws, p, tp, st, t, b, g, qg, kbuf, vbuf, lane);
    else
      step_tile<Tr, 0, true>(ws, p, tp, st, t, b, g, qg, kbuf, vbuf, lane);
  }

  // --- epilogue: normalise, then store (INIT) or merge into HBM (ACCUM)
  const int dsub = 4 * (lane >> 5);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = sum_halves(ws.l_part[qb]);
    if (!row_ok[qb]) continue;
    float* orow_ptr = p.o + orow[qb] * D;
    if (l_tot > 0.f) {
      const float inv = 1.f / l_tot;
      const float lse_s = ws.m_ref[qb] * p.scale + __builtin_amdgcn_logf(l_tot) * kLn2;
      float lse_r = kNegInf;
      if (p.accum) lse_r = p.lse[orow[qb]];
      if (lse_r == kNegInf) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16& a = ws.o[db][qb];
            const float4 v = {a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv};
            *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = v;
          }
        if (lane < 32) p.lse[orow[qb]] = lse_s;
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
            const f32x16& a = ws.o[db][qb];
            float* ptr = orow_ptr + 32 * db + 8 * j + dsub;
            const float4 r = *(const float4*)ptr;
            const float4 v = {cr * r.x + cs * a[4 * j], cr * r.y + cs * a[4 * j + 1],
                              cr * r.z + cs * a[4 * j + 2], cr * r.w + cs * a[4 * j + 3]};
            *(float4*)ptr = v;
          }
        if (lane < 32) p.lse[orow[qb]] = m + __builtin_amdgcn_logf(den) * kLn2;
      }
    } else if (!p.accum) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = float4{0.f, 0.f, 0.f, 0.f};
      if (lane < 32) p.lse[orow[qb]] = kNegInf;
    }
  }
}

template <class Tr>
hipError_t launch(const StepParams& p, hipStream_t s) {
  const int grid = 8 * p.per_xcd;
  hipLaunchKernelGGL(attn_step_kernel<Tr>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_step(const StepParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 1 && D == 128) return launch<Bf16<128>>(p, s);
  if (dtype == 1 && D == 64) return launch<Bf16<64>>(p, s);
  if (dtype == 0 && D == 128) return launch<F32<128>>(p, s);
  if (dtype == 0 && D == 64) return launch<F32<64>>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
