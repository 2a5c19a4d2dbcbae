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
//   * A workgroup (4 waves) owns 128 consecutive query rows of one (batch,
//     query head); wave w owns rows [32w, 32w + 32).
//   * Keys are processed in tiles of 64, staged in LDS and double buffered:
//     tile t+1 is fetched into registers while tile t is computed, then stored
//     to the other LDS buffer.
//   * Only key tiles with at least one visible key are visited.  A tile that
//     straddles the causal diagonal, or is cut short by the end of a span, runs
//     the mask code; every other tile runs none.
//   * Workgroups are ordered so that all query tiles reading the same K/V head
//     land on the same XCD (dispatch is round-robin over the 8 XCDs), which
//     keeps that head's K/V in one L2.
//
// Per-wave math (32 queries x 64 keys per tile)
//   S^T = K Q^T on MFMA 32x32 tiles: the accumulator of a 32x32 block puts one
//   query per lane (lane n and n+32 share query n) and 16 of its keys in that
//   lane's registers, so the row max and row sum of the online softmax are
//   in-lane reductions plus one lane swap across the two halves.
//   O^T += V^T P^T on MFMA: P^T is the exponentiated accumulator itself (bf16
//   rounded for the bf16 path), with the MFMA's reduction index mapped onto the
//   keys in the order the accumulator holds them; V^T is read from row-major V
//   in LDS with the transposing LDS read (bf16) or scalar reads (f32).
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
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Grow the reference maximum only when probabilities would exceed 2^kTau.
constexpr float kTau = 8.0f;

__device__ inline float swap_halves(float x) {
  // v_permlane32_swap with both operands x: every lane sees x of lane ^ 32 in
  // one of the two results; max/sum of both is symmetric.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]) - x;
}

__device__ inline float max_halves(float x) {
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
__device__ inline void lds_store16(RA_LDS char* base, unsigned off, u32x4 v) {
  *(RA_LDS u32x4*)(base + off) = v;
}

// ---------------------------------------------------------------------------
// LDS tile layout: 64 key rows of D elements, row-major, 16-byte chunks.  The
// chunk index is XOR-swizzled per row so that both the MFMA operand reads and
// the tile stores hit distinct banks:
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
  struct QFrag { bf16x8 f[D / 16]; };

  // Q^T operand: lane l holds Q[query l%32][16 dc + 8 (l/32) .. +7].
  __device__ static void load_q(QFrag& q, const Elem* row, bool ok, int lane) {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      if (ok) {
        q.f[dc] = *(const bf16x8*)(row + 16 * dc + 8 * (lane >> 5));
      } else {
        q.f[dc] = bf16x8{};
      }
    }
  }

  // S^T block kb (keys 32kb..32kb+31 of the tile) = K Q^T.
  __device__ static f32x16 s_block(const RA_LDS char* kt, int kb, const QFrag& q, int lane) {
    f32x16 acc = {};
    const unsigned row = 32 * kb + (lane & 31);
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      const unsigned c = 2 * dc + (lane >> 5);
      u32x4 a = lds_load16(kt, row * kRowBytes + ((c ^ swz_k<kCPR>(row)) * 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), q.f[dc], acc, 0, 0, 0);
    }
    return acc;
  }

  // O^T[db] += V^T P^T for the 64 keys of the tile.  MFMA (kb, hf) consumes
  // accumulator registers 8hf..8hf+7 of S^T block kb, i.e. reduction index
  // 8(l/32)+e <-> key 32kb + 16hf + 8(e/4) + 4(l/32) + e%4; the V^T operand is
  // gathered with two transposing reads of 4 keys x 16 columns per lane group.
  __device__ static void pv(f32x16* o, const RA_LDS char* vt, const f32x16* p, int lane) {
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[kb][8 * hf + e];
        pb[kb][hf] = __builtin_convertvector(x, bf16x8);
      }
    }
    const int gi = lane >> 4, s = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned d = 32 * db + 16 * (gi & 1) + 4 * (s & 3);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const unsigned r1 = 32 * kb + 16 * hf + 4 * (gi >> 1) + (s >> 2);
          const unsigned r2 = r1 + 8;
          const unsigned o1 = r1 * kRowBytes + (((d >> 3) ^ swz_v<kCPR>(r1)) * 16) + (d & 7) * 2;
          const unsigned o2 = r2 * kRowBytes + (((d >> 3) ^ swz_v<kCPR>(r2)) * 16) + (d & 7) * 2;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vt + o1));
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS i16x4*)(vt + o2));
          typedef __attribute__((ext_vector_type(8))) short i16x8;
          i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[kb][hf], o[db], 0, 0, 0);
        }
      }
    }
  }
};

template <int D_>
struct F32 {
  static constexpr int D = D_;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kCPR = kRowBytes / 16;
  typedef float Elem;
  struct QFrag { float f[D / 2]; };

  // Q^T operand of the 32x32x2 f32 MFMA: lane l holds Q[query l%32][2kk + l/32].
  __device__ static void load_q(QFrag& q, const Elem* row, bool ok, int lane) {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) q.f[kk] = ok ? row[2 * kk + (lane >> 5)] : 0.f;
  }

  __device__ static float lds_f(const RA_LDS char* t, unsigned row, unsigned d, unsigned swz) {
    return *(const RA_LDS float*)(t + row * kRowBytes + (((d >> 2) ^ swz) * 16) + (d & 3) * 4);
  }

  __device__ static f32x16 s_block(const RA_LDS char* kt, int kb, const QFrag& q, int lane) {
    f32x16 acc = {};
    const unsigned row = 32 * kb + (lane & 31);
    const unsigned sw = swz_k<kCPR>(row);
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      float a = lds_f(kt, row, 2 * kk + (lane >> 5), sw);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, q.f[kk], acc, 0, 0, 0);
    }
    return acc;
  }

  // MFMA (kb, j) pairs reduction index l/32 with key 32kb + 8(j/4) + 4(l/32) + j%4,
  // which is the key accumulator register j of lane l holds.
  __device__ static void pv(f32x16* o, const RA_LDS char* vt, const f32x16* p, int lane) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned d = 32 * db + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const unsigned row = 32 * kb + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
          float a = lds_f(vt, row, d, swz_v<kCPR>(row));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[kb][j], o[db], 0, 0, 0);
        }
      }
    }
  }
};

// Key tile t of the step: which span, where it starts, how many rows are real.
struct KTile {
  long long local0;  // first local key row
  long long glob0;   // its global position
  int count;         // rows of the tile that exist and may be visible
};

__device__ inline KTile key_tile(const StepParams& p, const int* nt, const long long* khi, int t) {
  const int s = t < nt[0] ? 0 : 1;
  const long long kin = (long long)(t - (s ? nt[0] : 0)) * kBK;
  KTile kt;
  kt.local0 = p.ks_off[s] + kin;
  kt.glob0 = p.ks_start[s] + kin;
  kt.count = (int)min((long long)kBK, khi[s] - kin);
  return kt;
}

// Staging of one K/V tile through registers: each thread moves kPer 16-byte
// chunks of K and of V.  Rows past `count` are zero-filled.
template <class Tr>
struct Stage {
  static constexpr int kChunks = kBK * Tr::kCPR;
  static constexpr int kPer = kChunks / kThreads;
  u32x4 kreg[kPer], vreg[kPer];

  __device__ void load(const StepParams& p, int b, int g, const KTile& kt) {
    const typename Tr::Elem* kb = (const typename Tr::Elem*)p.k;
    const typename Tr::Elem* vb = (const typename Tr::Elem*)p.v;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int row = idx / Tr::kCPR, c = idx % Tr::kCPR;
      if (row < kt.count) {
        const long long off = (((long long)b * p.Sk + kt.local0 + row) * p.Hkv + g) * Tr::D;
        kreg[i] = *(const u32x4*)((const char*)(kb + off) + c * 16);
        vreg[i] = *(const u32x4*)((const char*)(vb + off) + c * 16);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ void store(RA_LDS char* kt, RA_LDS char* vt) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const unsigned row = idx / Tr::kCPR, c = idx % Tr::kCPR;
      lds_store16(kt, row * Tr::kRowBytes + ((c ^ swz_k<Tr::kCPR>(row)) * 16), kreg[i]);
      lds_store16(vt, row * Tr::kRowBytes + ((c ^ swz_v<Tr::kCPR>(row)) * 16), vreg[i]);
    }
  }
};

template <class Tr>
__global__ __launch_bounds__(256) void attn_step_kernel(StepParams p) {
  constexpr int D = Tr::D;
  constexpr int kTileBytes = kBK * Tr::kRowBytes;
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * kTileBytes];
  RA_LDS char* smem = (RA_LDS char*)smem_raw;

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

  // --- key tiles with at least one key visible to some row of the tile
  int nt[2] = {0, 0};
  long long khi[2] = {0, 0};
  for (int s = 0; s < p.nks; ++s) {
    long long hi = p.ks_len[s];
    if (p.causal) hi = min(hi, qglob_last + 1 - p.ks_start[s]);
    hi = max(hi, 0LL);
    khi[s] = hi;
    nt[s] = (int)((hi + kBK - 1) / kBK);
  }
  const int ntiles = nt[0] + nt[1];

  const int n = lane & 31;
  const int wrow = wave * 32 + n;
  const bool row_ok = wrow < qrows;
  const long long qg = qglob0 + wrow;
  const long long orow = ((long long)b * p.Sq + qlocal0 + wrow) * p.Hq + h;  // (b, row, h)

  if (ntiles == 0) {
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

  typename Tr::QFrag qf;
  Tr::load_q(qf, (const typename Tr::Elem*)p.q + orow * D, row_ok, lane);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_ref = kNegInf;  // reference maximum of the raw (unscaled) scores
  float l_part = 0.f;     // this lane's share of the row sum

  const bool wave_rows = wave * 32 < qrows;
  const long long wq0 = qglob0 + wave * 32;                    // wave's first query
  const long long wq1 = qglob0 + min(wave * 32 + 31, qrows - 1);  // and last

  Stage<Tr> st;
  st.load(p, b, g, key_tile(p, nt, khi, 0));
  st.store(smem, smem + kTileBytes);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const RA_LDS char* kt = smem + buf * 2 * kTileBytes;
    const RA_LDS char* vt = kt + kTileBytes;
    if (t + 1 < ntiles) st.load(p, b, g, key_tile(p, nt, khi, t + 1));

    const KTile ti = key_tile(p, nt, khi, t);
    const bool skip = !wave_rows || (p.causal && ti.glob0 > wq1);
    if (!skip) {
      f32x16 sacc[2];
      sacc[0] = Tr::s_block(kt, 0, qf, lane);
      sacc[1] = Tr::s_block(kt, 1, qf, lane);
      const bool need_mask = ti.count < kBK || (p.causal && ti.glob0 + kBK - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const bool vis = key < ti.count && (!p.causal || ti.glob0 + key <= qg);
            if (!vis) sacc[kb][r] = kNegInf;
          }
        }
      }
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kb][r]);
      }
      tmax = max_halves(tmax);
      const float m_new = fmaxf(m_ref, tmax);
      // -inf reference: the difference is +inf and the maximum is taken;
      // both -inf: NaN compares false and nothing moves.
      const bool grow = (m_new - m_ref) * p.sl2 > kTau;
      float alpha = 1.f;
      if (grow) {
        alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * p.sl2);
        m_ref = m_new;
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        l_part *= alpha;
      }
      const float mb = m_ref == kNegInf ? 0.f : m_ref * p.sl2;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.sl2, -mb));
          sacc[kb][r] = pr;
          lsum += pr;
        }
      }
      l_part += lsum;
      Tr::pv(oacc, vt, sacc, lane);
    }

    if (t + 1 < ntiles) {
      RA_LDS char* kn = smem + (buf ^ 1) * 2 * kTileBytes;
      st.store(kn, kn + kTileBytes);
    }
    __syncthreads();
  }

  // --- epilogue: normalise, then store (INIT) or merge into HBM (ACCUM)
  const float l_tot = sum_halves(l_part);
  if (!row_ok) return;
  float* orow_ptr = p.o + orow * D;
  const int dsub = 4 * (lane >> 5);
  if (l_tot > 0.f) {
    const float inv = 1.f / l_tot;
    const float lse_s = m_ref * p.scale + __builtin_amdgcn_logf(l_tot) * kLn2;
    float lse_r = kNegInf;
    if (p.accum) lse_r = p.lse[orow];
    if (lse_r == kNegInf) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float4 v = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                      oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
          *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = v;
        }
      }
      if (lane < 32) p.lse[orow] = lse_s;
    } else {
      const float m = fmaxf(lse_r, lse_s);
      const float wr = __builtin_amdgcn_exp2f((lse_r - m) * kLog2e);
      const float ws = __builtin_amdgcn_exp2f((lse_s - m) * kLog2e);
      const float den = wr + ws;
      const float cr = wr / den;
      const float cs = ws / den * inv;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* ptr = orow_ptr + 32 * db + 8 * j + dsub;
          const float4 r = *(const float4*)ptr;
          float4 v = {cr * r.x + cs * oacc[db][4 * j], cr * r.y + cs * oacc[db][4 * j + 1],
                      cr * r.z + cs * oacc[db][4 * j + 2], cr * r.w + cs * oacc[db][4 * j + 3]};
          *(float4*)ptr = v;
        }
      }
      if (lane < 32) p.lse[orow] = m + __builtin_amdgcn_logf(den) * kLn2;
    }
  } else if (!p.accum) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) *(float4*)(orow_ptr + 32 * db + 8 * j + dsub) = float4{0.f, 0.f, 0.f, 0.f};
    }
    if (lane < 32) p.lse[orow] = kNegInf;
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
