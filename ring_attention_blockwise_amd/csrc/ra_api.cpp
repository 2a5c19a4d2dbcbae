// C ABI of libra.so: argument checks, the host-side plan of a ring step, the
// rank driver, and the launches.  Every check runs before anything is
// enqueued, so a failing call leaves the caller's buffers untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "ra.h"
#include "ra_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return RA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Compute units of the current device, queried once per device.  0 if the
// query fails (no device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// ---------------------------------------------------------------------------
// Index maps.  Contiguous: rank r owns [r S/P, (r+1) S/P).  Zigzag: 2P chunks
// of c = S/(2P); rank r owns chunk r, then chunk 2P-1-r.  Ring: at step s rank
// r holds the shard of (r - s) mod P.
struct Spans {
  int n;
  ra_span s[2];
};

int check_ring(int32_t order, int64_t S, int32_t P, int32_t rank) {
  if (order != RA_ORDER_CONTIGUOUS && order != RA_ORDER_ZIGZAG)
    return fail(RA_E_INVAL, "order must be RA_ORDER_CONTIGUOUS or RA_ORDER_ZIGZAG (got %d)", order);
  if (P < 1) return fail(RA_E_INVAL, "P must be >= 1 (got %d)", P);
  if (S < 0) return fail(RA_E_INVAL, "S must be >= 0");
  if (rank < 0 || rank >= P) return fail(RA_E_INVAL, "rank %d outside [0, %d)", rank, P);
  const int64_t parts = order == RA_ORDER_ZIGZAG ? 2LL * P : (int64_t)P;
  if (S % parts != 0)
    return fail(RA_E_INVAL, "S = %lld is not divisible by %lld chunks", (long long)S, (long long)parts);
  return RA_OK;
}

Spans rank_spans(int32_t order, int64_t S, int32_t P, int32_t rank) {
  Spans sp;
  if (order == RA_ORDER_CONTIGUOUS) {
    const int64_t c = S / P;
    sp.n = 1;
    sp.s[0] = {rank * c, c};
  } else {
    const int64_t c = S / (2LL * P);
    sp.n = 2;
    sp.s[0] = {rank * c, c};
    sp.s[1] = {(2LL * P - 1 - rank) * c, c};
  }
  return sp;
}

int32_t ring_src(int32_t rank, int32_t step, int32_t P) { return ((rank - step) % P + P) % P; }

// Class of query positions [q0, q0+nq) against key positions [k0, k0+nk).
int32_t pair_class(int64_t q0, int64_t nq, int64_t k0, int64_t nk, bool causal) {
  if (nq <= 0 || nk <= 0) return RA_CLASS_SKIP;
  if (!causal) return RA_CLASS_FULL;
  if (k0 > q0 + nq - 1) return RA_CLASS_SKIP;
  if (k0 + nk - 1 <= q0) return RA_CLASS_FULL;
  return RA_CLASS_DIAG;
}

// Keys visible to the query at global position t under a mask: [key_lo(t),
// key_hi(t)], both non-decreasing in t.
int64_t seq_index(const ra_mask* m, int64_t t) {
  const int64_t* cu = m->cu_seqlens;
  int lo = 0, hi = m->n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
int64_t host_key_lo(const ra_mask* m, int64_t t) {
  int64_t lo = m->window > 0 ? t - m->window + 1 : 0;
  if (m->n_seqs > 0) lo = std::max(lo, m->cu_seqlens[seq_index(m, t)]);
  return lo;
}
int64_t host_key_hi(const ra_mask* m, bool causal, int64_t t) {
  if (causal) return t;
  if (m->n_seqs > 0) return m->cu_seqlens[seq_index(m, t) + 1] - 1;
  return INT64_MAX;
}
// Does some query of [q0, q0+nq) see some key of [k0, k0+nk)?
bool span_sees(int64_t q0, int64_t nq, int64_t k0, int64_t nk, bool causal, const ra_mask* m) {
  if (nq <= 0 || nk <= 0) return false;
  if (!m) return pair_class(q0, nq, k0, nk, causal) != RA_CLASS_SKIP;
  const int64_t lo = std::max(host_key_lo(m, q0), k0);
  const int64_t hi = std::min(host_key_hi(m, causal, q0 + nq - 1), k0 + nk - 1);
  return lo <= hi;
}

// Key tiles of kBwdKeys keys that some query row of the step sees (the
// dK/dV kernels' items with work, per batch entry and kv head).  A tile
// [k0, k1] is seen by the rows t with key_hi(t) >= k0 and key_lo(t) <= k1,
// one interval since both ends never decrease; the same test as the
// kernels' own plan.
int64_t kv_active(const ra::StepParams& p, const ra_mask* m) {
  const bool cu = m && m->n_seqs > 0;
  int64_t active = 0;
  for (int s = 0; s < p.nks; ++s) {
    const int64_t end = p.ks_start[s] + p.ks_len[s];
    for (int64_t k0 = p.ks_start[s]; k0 < end; k0 += ra::kBwdKeys) {
      const int64_t k1 = std::min(k0 + ra::kBwdKeys, end) - 1;
      const int64_t t0 = p.causal ? k0 : (cu ? m->cu_seqlens[seq_index(m, k0)] : 0);
      int64_t t1 = INT64_MAX;
      if (m && m->window > 0) t1 = k1 + m->window - 1;
      if (cu) t1 = std::min(t1, m->cu_seqlens[seq_index(m, k1) + 1] - 1);
      for (int q = 0; q < p.nqs; ++q) {
        const int64_t first = std::max((int64_t)0, t0 - (int64_t)p.qs_start[q]);
        const int64_t last = std::min((int64_t)p.qs_len[q] - 1, t1 - (int64_t)p.qs_start[q]);
        if (first <= last) {
          ++active;
          break;
        }
      }
    }
  }
  return active;
}

int check_mask(const ra_mask* m, int64_t S, bool causal) {
  if (!m) return RA_OK;
  if (m->window < 0) return fail(RA_E_INVAL, "window must be >= 0");
  if (m->window > 0 && !causal) return fail(RA_E_INVAL, "a window needs the causal mask");
  if (m->n_seqs < 0) return fail(RA_E_INVAL, "n_seqs must be >= 0");
  if (m->n_seqs > 0) {
    if (!m->cu_seqlens || !m->cu_seqlens_dev) return fail(RA_E_INVAL, "cu_seqlens (host and device) must be given");
    if (!aligned(m->cu_seqlens_dev, 8)) return fail(RA_E_INVAL, "cu_seqlens_dev must be 8-byte aligned");
    if (m->cu_seqlens[0] != 0 || m->cu_seqlens[m->n_seqs] != S)
      return fail(RA_E_INVAL, "cu_seqlens must run from 0 to S = %lld", (long long)S);
    for (int i = 0; i < m->n_seqs; ++i)
      if (m->cu_seqlens[i + 1] <= m->cu_seqlens[i]) return fail(RA_E_INVAL, "cu_seqlens must increase strictly");
  }
  return RA_OK;
}

// ---------------------------------------------------------------------------
int check_step(const ra_step_desc* d, const void* q, const void* k, const void* v, const float* o,
               const float* lse, uint32_t flags, bool check_ptrs = true) {
  if (!d) return fail(RA_E_INVAL, "descriptor is NULL");
  if (d->dtype != RA_DTYPE_F32 && d->dtype != RA_DTYPE_BF16)
    return fail(RA_E_UNSUPPORTED, "dtype %d not supported (RA_DTYPE_F32 or RA_DTYPE_BF16)", d->dtype);
  if (d->D != 64 && d->D != 128) return fail(RA_E_UNSUPPORTED, "head dimension %d not built (64 or 128)", d->D);
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1) return fail(RA_E_INVAL, "B, Hq, Hkv must be >= 1");
  if (d->Hq % d->Hkv) return fail(RA_E_INVAL, "Hq = %d is not a multiple of Hkv = %d", d->Hq, d->Hkv);
  if (d->Sq < 0 || d->Sk < 0) return fail(RA_E_INVAL, "Sq and Sk must be >= 0");
  if (flags != RA_STEP_INIT && flags != RA_STEP_ACCUM) return fail(RA_E_INVAL, "unknown flags 0x%x", flags);
  if (!(std::isfinite(d->scale) && d->scale > 0.f)) return fail(RA_E_INVAL, "scale must be finite and > 0");
  if (d->n_qspans < 1 || d->n_qspans > 2 || d->n_kspans < 1 || d->n_kspans > 2)
    return fail(RA_E_INVAL, "n_qspans and n_kspans must be 1 or 2");
  int64_t sq = 0, sk = 0;
  for (int i = 0; i < d->n_qspans; ++i) {
    if (d->qspans[i].len < 0 || d->qspans[i].start < 0) return fail(RA_E_INVAL, "query span %d is negative", i);
    sq += d->qspans[i].len;
  }
  for (int i = 0; i < d->n_kspans; ++i) {
    if (d->kspans[i].len < 0 || d->kspans[i].start < 0) return fail(RA_E_INVAL, "key span %d is negative", i);
    sk += d->kspans[i].len;
  }
  if (sq != d->Sq) return fail(RA_E_INVAL, "query spans sum to %lld, Sq = %lld", (long long)sq, (long long)d->Sq);
  if (sk != d->Sk) return fail(RA_E_INVAL, "key spans sum to %lld, Sk = %lld", (long long)sk, (long long)d->Sk);
  const int64_t qtiles = (d->qspans[0].len + ra::kBQ - 1) / ra::kBQ +
                         (d->n_qspans > 1 ? (d->qspans[1].len + ra::kBQ - 1) / ra::kBQ : 0);
  if ((int64_t)d->B * d->Hq * qtiles > (int64_t)1 << 30) return fail(RA_E_INVAL, "too many query tiles");
  if (!check_ptrs) return RA_OK;
  if (d->Sq > 0) {
    if (!q || !o || !lse) return fail(RA_E_INVAL, "q, o and lse must not be NULL");
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4))
      return fail(RA_E_INVAL, "q and o must be 16-byte aligned, lse 4-byte aligned");
  }
  if (d->Sq > 0 && d->Sk > 0) {
    if (!k || !v) return fail(RA_E_INVAL, "k and v must not be NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(RA_E_INVAL, "k and v must be 16-byte aligned");
  }
  return RA_OK;
}

// Builds the kernel parameters of one step.  Returns false when nothing has to
// be launched (empty rows, or ACCUM with every pair masked).
// Keys of the step's key spans that the query at global position t sees.
int64_t visible_keys(const ra::StepParams& p, const ra_mask* m, int64_t t) {
  const int64_t lo = m ? host_key_lo(m, t) : 0;
  const int64_t hi = m ? host_key_hi(m, p.causal != 0, t) : (p.causal ? t : INT64_MAX);
  int64_t n = 0;
  for (int s = 0; s < p.nks; ++s) {
    const int64_t a = std::max(lo, (int64_t)p.ks_start[s]);
    const int64_t b = std::min(hi, (int64_t)(p.ks_start[s] + p.ks_len[s] - 1));
    if (a <= b) n += b - a + 1;
  }
  return n;
}

// Work items per XCD, and whether each XCD's share is whole heads (then its
// items run heaviest tile first).
void set_grid(ra::StepParams* p) {
  p->per_xcd = (p->n_work + 7) / 8;
  p->lpt = (p->n_work % 8 == 0 && p->n_qtiles > 0 && p->per_xcd % p->n_qtiles == 0) ? 1 : 0;
}

bool build_params(const ra_step_desc* d, const void* q, const void* k, const void* v, float* o,
                  float* lse, bool accum, int n_cus, ra::StepParams* p, const ra_mask* m = nullptr) {
  if (d->Sq == 0) return false;
  p->q = q;
  p->k = k;
  p->v = v;
  p->o = o;
  p->lse = lse;
  p->B = d->B;
  p->Hq = d->Hq;
  p->Hkv = d->Hkv;
  p->G = d->Hq / d->Hkv;
  p->Sq = d->Sq;
  p->Sk = d->Sk;
  p->causal = d->causal ? 1 : 0;
  p->accum = accum ? 1 : 0;
  p->scale = d->scale;
  p->sl2 = (float)((double)d->scale * 1.4426950408889634);
  p->window = m ? m->window : 0;
  p->cu = m && m->n_seqs > 0 ? (const long long*)m->cu_seqlens_dev : nullptr;
  p->nseg = m ? m->n_seqs : 0;
  p->mask_ext = (p->window > 0 || p->cu) ? 1 : 0;
  p->nks = 0;
  int64_t off = 0;
  for (int i = 0; i < d->n_kspans; ++i) {
    if (d->kspans[i].len > 0) {
      p->ks_start[p->nks] = d->kspans[i].start;
      p->ks_len[p->nks] = d->kspans[i].len;
      p->ks_off[p->nks] = off;
      ++p->nks;
    }
    off += d->kspans[i].len;
  }
  p->nqs = 0;
  off = 0;
  for (int i = 0; i < d->n_qspans; ++i) {
    const ra_span qs = d->qspans[i];
    bool any = false;
    for (int j = 0; j < p->nks; ++j) any |= span_sees(qs.start, qs.len, p->ks_start[j], p->ks_len[j], p->causal, m);
    if (qs.len > 0 && (any || !accum)) {
      p->qs_start[p->nqs] = qs.start;
      p->qs_len[p->nqs] = qs.len;
      p->qs_off[p->nqs] = off;
      ++p->nqs;
    }
    off += qs.len;
  }
  if (p->nqs == 0) return false;
  {
    // which end of the query rows sees more keys: the first tile's or the
    // last tile's (each by its first and last row)
    const int bq = ra::step_rows(d->dtype);
    const int64_t f0 = p->qs_start[0], f1 = f0 + std::min((int64_t)bq, (int64_t)p->qs_len[0]) - 1;
    const int ls = p->nqs - 1;
    const int64_t l1 = p->qs_start[ls] + p->qs_len[ls] - 1, l0 = std::max((int64_t)p->qs_start[ls], l1 - bq + 1);
    const int64_t wf = visible_keys(*p, m, f0) + visible_keys(*p, m, f1);
    const int64_t wl = visible_keys(*p, m, l0) + visible_keys(*p, m, l1);
    p->first_heavy = wf > wl ? 1 : 0;
  }
  for (int i = p->nqs; i < 2; ++i) p->qs_start[i] = p->qs_len[i] = p->qs_off[i] = 0;
  for (int i = p->nks; i < 2; ++i) p->ks_start[i] = p->ks_len[i] = p->ks_off[i] = 0;
  // bf16, D = 128: eight-wave workgroups split each item's key tiles between
  // two wave sets when the query tiles with work give fewer than two
  // workgroups per CU, or fewer than four and very unequal ones (the
  // heaviest, by its first and last rows' visible keys, half again the
  // average: a diagonal or a window over an earlier block).
  p->ksplit = 0;
  if (d->dtype == RA_DTYPE_BF16 && d->D == 128) {
    const int bq = ra::step_rows(d->dtype);
    int64_t active = 0, total = 0, heaviest = 0;
    for (int i = 0; i < p->nqs; ++i)
      for (int64_t off = 0; off < p->qs_len[i]; off += bq) {
        const int64_t rows = std::min((int64_t)bq, (int64_t)p->qs_len[i] - off);
        const int64_t r0 = p->qs_start[i] + off;
        const int64_t w = visible_keys(*p, m, r0) + visible_keys(*p, m, r0 + rows - 1);
        if (w == 0) continue;
        ++active;
        total += w;
        heaviest = std::max(heaviest, w);
      }
    if (active > 0 && n_cus > 0) {
      const int64_t items = active * d->B * d->Hq;
      const bool unequal = 2 * heaviest * active >= 3 * total;
      p->ksplit = (items < 2 * (int64_t)n_cus || (items < 4 * (int64_t)n_cus && unequal)) ? 1 : 0;
    }
  }
  const int bq = ra::step_rows(d->dtype);
  p->qt_span0 = (int)((p->qs_len[0] + bq - 1) / bq);
  p->n_qtiles = p->qt_span0 + (int)((p->qs_len[1] + bq - 1) / bq);
  p->n_work = p->B * p->Hq * p->n_qtiles;
  set_grid(p);
  return true;
}

int launch_step(const ra::StepParams& p, int dtype, int D, void* stream) {
  hipError_t e = ra::launch_attn_step(p, dtype, D, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_E_HIP, "attention step launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

// The P steps of one rank's ring (forward or backward): validation once,
// then the parameters of each step.  The rank drivers launch from these, and
// ra_rank_launches reports them.
struct RankRing {
  const ra_rank_desc* d = nullptr;
  const ra_mask* m = nullptr;
  const void *q = nullptr, *k = nullptr, *v = nullptr;
  float *o = nullptr, *lse = nullptr;
  int64_t s_loc = 0, shard_elems = 0;
  size_t esz = 0;
  ra_step_desc sd;

  // o_ and lse_ are the forward's outputs (the backward passes dq and the
  // forward's lse, which it only reads: they are checked, never written here)
  int init(const ra_rank_desc* d_, const ra_mask* m_, const void* q_, const void* k_, const void* v_, float* o_,
           const float* lse_, bool check_ptrs) {
    d = d_;
    m = m_;
    q = q_;
    k = k_;
    v = v_;
    o = o_;
    lse = const_cast<float*>(lse_);
    if (!d) return fail(RA_E_INVAL, "descriptor is NULL");
    int rc = check_ring(d->order, d->S, d->P, d->rank);
    if (rc) return rc;
    rc = check_mask(m, d->S, d->causal != 0);
    if (rc) return rc;
    s_loc = d->S / d->P;
    esz = d->dtype == RA_DTYPE_BF16 ? 2 : 4;
    sd.dtype = d->dtype;
    sd.B = d->B;
    sd.Hq = d->Hq;
    sd.Hkv = d->Hkv;
    sd.D = d->D;
    sd.Sq = s_loc;
    sd.Sk = s_loc;
    sd.causal = d->causal;
    sd.scale = d->scale;
    const Spans qs = rank_spans(d->order, d->S, d->P, d->rank);
    sd.n_qspans = qs.n;
    for (int i = 0; i < 2; ++i) sd.qspans[i] = i < qs.n ? qs.s[i] : ra_span{0, 0};
    sd.n_kspans = qs.n;
    for (int i = 0; i < 2; ++i) sd.kspans[i] = sd.qspans[i];
    shard_elems = (int64_t)d->B * s_loc * d->Hkv * d->D;
    // every step's descriptor differs from this one only in its key spans
    return check_step(&sd, q, k, v, o, lse, RA_STEP_INIT, check_ptrs);
  }

  bool tuned() const { return d->dtype == RA_DTYPE_BF16 && d->D == 128; }

  // Key spans and shard pointers of step s.
  void at_step(int32_t s, const void** kp, const void** vp, int32_t* src) {
    *src = ring_src(d->rank, s, d->P);
    const Spans ks = rank_spans(d->order, d->S, d->P, *src);
    sd.n_kspans = ks.n;
    for (int i = 0; i < 2; ++i) sd.kspans[i] = i < ks.n ? ks.s[i] : ra_span{0, 0};
    *kp = k ? (const char*)k + (size_t)*src * shard_elems * esz : nullptr;
    *vp = v ? (const char*)v + (size_t)*src * shard_elems * esz : nullptr;
  }

  // Parameters of forward step s; false when the step launches nothing.
  bool forward_step(int32_t s, int n_cus, ra::StepParams* p) {
    if (s_loc == 0) return false;
    const void *kp, *vp;
    int32_t src;
    at_step(s, &kp, &vp, &src);
    return build_params(&sd, q, kp, vp, o, lse, s > 0, n_cus, p, m);
  }

  // Parameters of backward step s (o and lse of init() are dq and the
  // forward's lse); false when the step launches nothing.
  bool backward_step(int32_t s, int n_cus, const float* fwd_lse, const void* dout, const float* delta, float* dq,
                     float* dk_shards, float* dv_shards, ra::BwdParams* bp) {
    if (s_loc == 0) return false;
    const void *kp, *vp;
    int32_t src;
    at_step(s, &kp, &vp, &src);
    if (!build_params(&sd, q, kp, vp, nullptr, nullptr, s > 0, n_cus, &bp->s, m)) return false;
    // the dQ kernel's query tiles are kBwdRows rows
    bp->s.qt_span0 = (int)((bp->s.qs_len[0] + ra::kBwdRows - 1) / ra::kBwdRows);
    bp->s.n_qtiles = bp->s.qt_span0 + (int)((bp->s.qs_len[1] + ra::kBwdRows - 1) / ra::kBwdRows);
    bp->s.n_work = bp->s.B * bp->s.Hq * bp->s.n_qtiles;
    set_grid(&bp->s);
    bp->dout = dout;
    bp->lse = fwd_lse;
    bp->delta = delta;
    bp->dq = dq;
    bp->dk = dk_shards ? dk_shards + (size_t)src * shard_elems : nullptr;
    bp->dv = dv_shards ? dv_shards + (size_t)src * shard_elems : nullptr;
    // key tiles of kBwdKeys keys over the block's key spans, for the dK/dV kernel
    bp->kt_span0 = (int)((bp->s.ks_len[0] + ra::kBwdKeys - 1) / ra::kBwdKeys);
    bp->n_ktiles = bp->kt_span0 + (int)((bp->s.ks_len[1] + ra::kBwdKeys - 1) / ra::kBwdKeys);
    bp->n_kwork = bp->s.B * bp->s.Hkv * bp->n_ktiles;
    bp->per_xcd_kv = (bp->n_kwork + 7) / 8;
    // Two groups of waves share each key tile's query rows (eight-wave
    // workgroups, separate dV and dK kernels) only when the key tiles with
    // work would not give every CU a workgroup; otherwise the fused dK/dV
    // kernel.  Unequal tiles (causal and windowed diagonals) need no split:
    // each XCD takes one kv head's tiles heaviest first, with work falling
    // linearly along them, so the tiles dispatched second land on the CUs
    // whose first tiles were lightest (measured: split 2.74 ms against fused
    // 2.58 ms for the windowed 131k backward, 30.3 against 30.0 ms causal).
    bp->kv_split = ((int64_t)bp->s.B * bp->s.Hkv * kv_active(bp->s, m) <= n_cus) ? 1 : 0;
    return true;
  }
};

int check_backward_ptrs(const float* o, const void* dout, const float* dk_shards, const float* dv_shards,
                        const float* delta) {
  if (!o || !dout || !dk_shards || !dv_shards || !delta) return fail(RA_E_INVAL, "NULL pointer");
  if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(dk_shards, 16) || !aligned(dv_shards, 16) ||
      !aligned(delta, 4))
    return fail(RA_E_INVAL, "o, dout, dk_shards and dv_shards must be 16-byte aligned, delta 4-byte aligned");
  return RA_OK;
}

// Everything ra_rank_backward enqueues once its arguments are checked:
// -delta = -rowsum(dO * O) into `delta`, then per launched step the dQ and
// dK/dV kernels.
int run_backward(RankRing& ring, const float* o, const float* lse, const void* dout, float* dq, float* dk_shards,
                 float* dv_shards, float* delta, void* stream) {
  const ra_rank_desc* d = ring.d;
  const int n_cus = device_cus();
  if (n_cus <= 0) return fail(RA_E_HIP, "cannot query the device's compute units");
  const int64_t rows = (int64_t)d->B * ring.s_loc * d->Hq;
  hipError_t e = ring.tuned() ? ra::launch_bwd_delta(rows, d->D, 1, dout, o, delta, (hipStream_t)stream)
                              : ra::launch_simt_delta(rows, d->D, d->dtype, dout, o, delta, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_E_HIP, "delta launch failed: %s", hipGetErrorString(e));
  for (int32_t s = 0; s < d->P; ++s) {
    ra::BwdParams bp;
    if (!ring.backward_step(s, n_cus, lse, dout, delta, dq, dk_shards, dv_shards, &bp)) continue;
    e = ring.tuned() ? ra::launch_attn_bwd_bf16(bp, (hipStream_t)stream)
                     : ra::launch_attn_bwd_simt(bp, d->dtype, d->D, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RA_E_HIP, "backward launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

// Scratch of ra_rank_backward_noalloc: the backward's delta rows, one copy
// per device (every device the library runs on holds it until the process
// ends).  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol): scratch_ptr() resolves its device
// address once per device, with that device current, and that address is
// what the launches get.
constexpr int64_t kScratchRows = RA_NOALLOC_MAX_ROWS;
__device__ __align__(256) float scratch[kScratchRows];

float* scratch_ptr() {
  static std::mutex mu;
  static float* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = (float*)p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

int ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_last_error(void) { return g_err; }

int ra_plan(int32_t order, int64_t S, int32_t P, int32_t rank, int32_t step, int32_t causal, int32_t tile_q,
            int32_t tile_k, ra_plan_out* out) {
  if (!out) return fail(RA_E_INVAL, "out is NULL");
  int rc = check_ring(order, S, P, rank);
  if (rc) return rc;
  if (step < 0 || step >= P) return fail(RA_E_INVAL, "step %d outside [0, %d)", step, P);
  if (tile_q < 1 || tile_k < 1) return fail(RA_E_INVAL, "tile sizes must be >= 1");
  const int32_t src = ring_src(rank, step, P);
  const Spans qs = rank_spans(order, S, P, rank), ks = rank_spans(order, S, P, src);
  out->src = src;
  out->n_qspans = qs.n;
  out->n_kspans = ks.n;
  for (int i = 0; i < 2; ++i) {
    out->qspans[i] = i < qs.n ? qs.s[i] : ra_span{0, 0};
    out->kspans[i] = i < ks.n ? ks.s[i] : ra_span{0, 0};
    for (int j = 0; j < 2; ++j)
      out->pair_class[i][j] = (i < qs.n && j < ks.n)
                                  ? pair_class(qs.s[i].start, qs.s[i].len, ks.s[j].start, ks.s[j].len, causal != 0)
                                  : RA_CLASS_SKIP;
  }
  // Tile counts: per span pair, count tiles by class.  For a causal pair the
  // class of (query tile [a, a+tq), key tile [b, b+tk)) only depends on the
  // two ends, so each query tile's key tiles split into a FULL prefix, a DIAG
  // middle and a SKIP suffix; the loop is over query tiles only.
  int64_t nf = 0, nd = 0, ns = 0;
  for (int i = 0; i < qs.n; ++i) {
    for (int j = 0; j < ks.n; ++j) {
      const int64_t qa = qs.s[i].start, qn = qs.s[i].len, ka = ks.s[j].start, kn = ks.s[j].len;
      const int64_t nkt = (kn + tile_k - 1) / tile_k;
      for (int64_t a = 0; a < qn; a += tile_q) {
        const int64_t q0 = qa + a, q1 = qa + (a + tile_q < qn ? a + tile_q : qn);  // [q0, q1)
        if (!causal) {
          nf += nkt;
          continue;
        }
        // key tile t spans [ka + t tk, min(ka + (t+1) tk, ka + kn))
        int64_t full = 0, skip = 0;
        for (int64_t t = 0; t < nkt; ++t) {
          const int64_t k0 = ka + t * tile_k;
          const int64_t k1 = ka + ((t + 1) * tile_k < kn ? (t + 1) * tile_k : kn);
          const int32_t c = pair_class(q0, q1 - q0, k0, k1 - k0, true);
          if (c == RA_CLASS_FULL) {
            ++full;
          } else if (c == RA_CLASS_SKIP) {
            // key tiles only move right from here: the rest are SKIP too
            skip += nkt - t;
            break;
          }
        }
        nf += full;
        ns += skip;
        nd += nkt - full - skip;
      }
    }
  }
  out->tiles_full = nf;
  out->tiles_diag = nd;
  out->tiles_skip = ns;
  return ok();
}

int ra_step(const ra_step_desc* d, const void* q, const void* k, const void* v, float* o, float* lse,
            uint32_t flags, void* stream) {
  int rc = check_step(d, q, k, v, o, lse, flags);
  if (rc) return rc;
  ra::StepParams p;
  if (!build_params(d, q, k, v, o, lse, flags == RA_STEP_ACCUM, device_cus(), &p)) return ok();
  rc = launch_step(p, d->dtype, d->D, stream);
  return rc ? rc : ok();
}

int ra_rank_forward(const ra_rank_desc* d, const void* q_local, const void* k_shards, const void* v_shards,
                    float* o, float* lse, void* stream) {
  return ra_rank_forward_masked(d, nullptr, q_local, k_shards, v_shards, o, lse, stream);
}

int ra_rank_forward_masked(const ra_rank_desc* d, const ra_mask* m, const void* q_local, const void* k_shards,
                           const void* v_shards, float* o, float* lse, void* stream) {
  RankRing ring;
  int rc = ring.init(d, m, q_local, k_shards, v_shards, o, lse, true);
  if (rc) return rc;
  const int cus = device_cus();
  for (int32_t s = 0; s < d->P; ++s) {
    ra::StepParams p;
    if (!ring.forward_step(s, cus, &p)) continue;
    rc = launch_step(p, d->dtype, d->D, stream);
    if (rc) return rc;
  }
  return ok();
}

int ra_allgather_forward(const ra_rank_desc* d, const void* q_local, const void* k_global, const void* v_global,
                         float* o, float* lse, void* stream) {
  if (!d) return fail(RA_E_INVAL, "descriptor is NULL");
  int rc = check_ring(d->order, d->S, d->P, d->rank);
  if (rc) return rc;
  ra_step_desc sd;
  sd.dtype = d->dtype;
  sd.B = d->B;
  sd.Hq = d->Hq;
  sd.Hkv = d->Hkv;
  sd.D = d->D;
  sd.Sq = d->S / d->P;
  sd.Sk = d->S;
  sd.causal = d->causal;
  sd.scale = d->scale;
  const Spans qs = rank_spans(d->order, d->S, d->P, d->rank);
  sd.n_qspans = qs.n;
  for (int i = 0; i < 2; ++i) sd.qspans[i] = i < qs.n ? qs.s[i] : ra_span{0, 0};
  sd.n_kspans = 1;
  sd.kspans[0] = ra_span{0, d->S};
  sd.kspans[1] = ra_span{0, 0};
  rc = check_step(&sd, q_local, k_global, v_global, o, lse, RA_STEP_INIT);
  if (rc) return rc;
  ra::StepParams p;
  if (!build_params(&sd, q_local, k_global, v_global, o, lse, false, device_cus(), &p)) return ok();
  rc = launch_step(p, d->dtype, d->D, stream);
  if (rc) return rc;
  return ok();
}

int ra_rank_backward(const ra_rank_desc* d, const void* q_local, const void* k_shards, const void* v_shards,
                     const float* o, const float* lse, const void* dout, float* dq, float* dk_shards,
                     float* dv_shards, float* delta, void* stream) {
  return ra_rank_backward_masked(d, nullptr, q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards,
                                 delta, stream);
}

int ra_rank_backward_masked(const ra_rank_desc* d, const ra_mask* m, const void* q_local, const void* k_shards,
                            const void* v_shards, const float* o, const float* lse, const void* dout, float* dq,
                            float* dk_shards, float* dv_shards, float* delta, void* stream) {
  RankRing ring;
  int rc = ring.init(d, m, q_local, k_shards, v_shards, dq, lse, true);
  if (rc) return rc;
  if (ring.s_loc == 0) return ok();
  rc = check_backward_ptrs(o, dout, dk_shards, dv_shards, delta);
  if (rc) return rc;
  return run_backward(ring, o, lse, dout, dq, dk_shards, dv_shards, delta, stream);
}

int ra_rank_backward_noalloc(const ra_rank_desc* d, const void* q_local, const void* k_shards,
                             const void* v_shards, const float* o, const float* lse, const void* dout, float* dq,
                             float* dk_shards, float* dv_shards, void* stream) {
  RankRing ring;
  int rc = ring.init(d, nullptr, q_local, k_shards, v_shards, dq, lse, true);
  if (rc) return rc;
  if (ring.s_loc == 0) return ok();
  const int64_t rows = (int64_t)d->B * ring.s_loc * d->Hq;
  if (rows > kScratchRows)
    return fail(RA_E_INVAL, "B * S/P * Hq = %lld rows exceed the %lld rows of the library's scratch",
                (long long)rows, (long long)kScratchRows);
  float* delta = scratch_ptr();
  if (!delta) return fail(RA_E_HIP, "cannot resolve the scratch array's device address");
  rc = check_backward_ptrs(o, dout, dk_shards, dv_shards, delta);
  if (rc) return rc;
  return run_backward(ring, o, lse, dout, dq, dk_shards, dv_shards, delta, stream);
}

int ra_rank_launches(const ra_rank_desc* d, const ra_mask* m, int32_t backward, int32_t n_cus,
                     ra_launch_info* out) {
  if (!out) return fail(RA_E_INVAL, "out is NULL");
  if (backward != 0 && backward != 1) return fail(RA_E_INVAL, "backward must be 0 or 1");
  if (n_cus < 0) return fail(RA_E_INVAL, "n_cus must be >= 0");
  RankRing ring;
  int rc = ring.init(d, m, nullptr, nullptr, nullptr, nullptr, nullptr, false);
  if (rc) return rc;
  if (n_cus == 0) {
    n_cus = device_cus();
    if (n_cus <= 0) return fail(RA_E_HIP, "cannot query the device's compute units");
  }
  for (int32_t s = 0; s < d->P; ++s) {
    ra_launch_info& li = out[s];
    li = ra_launch_info{RA_KERNEL_NONE, 0, 0, 0, 0, 0};
    if (!backward) {
      ra::StepParams p;
      if (ring.s_loc == 0 || !ring.forward_step(s, n_cus, &p)) continue;
      li.kernel = d->dtype == RA_DTYPE_F32 ? RA_KERNEL_STEP_F32
                  : p.ksplit               ? RA_KERNEL_STEP_BF16_KSPLIT
                                           : RA_KERNEL_STEP_BF16;
      li.masked = p.mask_ext;
      li.items = p.n_work;
      li.grid = 8 * p.per_xcd;
      li.lpt = p.lpt;
      li.first_heavy = p.first_heavy;
    } else {
      ra::BwdParams bp;
      if (ring.s_loc == 0 || !ring.backward_step(s, n_cus, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &bp))
        continue;
      li.kernel = !ring.tuned() ? RA_KERNEL_BWD_SIMT : bp.kv_split ? RA_KERNEL_BWD_SPLIT : RA_KERNEL_BWD_FUSED;
      li.masked = bp.s.mask_ext;
      li.items = (int32_t)((int64_t)bp.s.B * bp.s.Hkv * kv_active(bp.s, m));
      li.grid = 8 * bp.s.per_xcd;
      li.lpt = bp.s.lpt;
      li.first_heavy = bp.s.first_heavy;
    }
  }
  return ok();
}

int ra_lse_merge(int64_t rows, int32_t D, const float* o_a, const float* lse_a, const float* o_b,
                 const float* lse_b, float* o_out, float* lse_out, void* stream) {
  if (rows < 0) return fail(RA_E_INVAL, "rows must be >= 0");
  if (D < 1 || D > 4096) return fail(RA_E_INVAL, "D = %d outside [1, 4096]", D);
  if (rows == 0) return ok();
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return fail(RA_E_INVAL, "NULL pointer");
  if (!aligned(o_a, 4) || !aligned(o_b, 4) || !aligned(o_out, 4) || !aligned(lse_a, 4) ||
      !aligned(lse_b, 4) || !aligned(lse_out, 4))
    return fail(RA_E_INVAL, "pointers must be 4-byte aligned");
  if (rows * (int64_t)D >= ((int64_t)1 << 31)) return fail(RA_E_INVAL, "rows * D must be < 2^31");
  hipError_t e = ra::launch_lse_merge(rows, D, o_a, lse_a, o_b, lse_b, o_out, lse_out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ra_ulysses_relayout(int32_t dir, int32_t elem_bytes, int32_t B, int64_t s_loc, int32_t H, int32_t D,
                        int32_t P_u, const void* in, void* out, void* stream) {
  if (dir != RA_SEQ2HEAD && dir != RA_HEAD2SEQ) return fail(RA_E_INVAL, "dir must be RA_SEQ2HEAD or RA_HEAD2SEQ");
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return fail(RA_E_INVAL, "elem_bytes must be 1, 2, 4 or 8");
  if (B < 0 || s_loc < 0 || H < 1 || D < 0 || P_u < 1) return fail(RA_E_INVAL, "bad shape");
  if (H % P_u) return fail(RA_E_INVAL, "H = %d is not divisible by P_u = %d", H, P_u);
  const int64_t bytes = (int64_t)B * s_loc * H * D * elem_bytes;
  if (bytes == 0) return ok();
  if (!in || !out) return fail(RA_E_INVAL, "NULL pointer");
  const uintptr_t i0 = (uintptr_t)in, o0 = (uintptr_t)out;
  if (i0 < o0 + (uintptr_t)bytes && o0 < i0 + (uintptr_t)bytes) return fail(RA_E_INVAL, "in and out overlap");
  const int64_t runs = (int64_t)P_u * B * s_loc;
  const int64_t run_bytes = (int64_t)(H / P_u) * D * elem_bytes;
  const int64_t units = runs * (run_bytes / ra::relayout_unit(run_bytes, in, out));
  if (runs >= ((int64_t)1 << 31) || units >= ((int64_t)1 << 31))
    return fail(RA_E_INVAL, "tensor too large for one relayout call (2^31 copy units)");
  hipError_t e = ra::launch_relayout(dir, elem_bytes, B, s_loc, H, D, P_u, in, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_E_HIP, "relayout launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ra_ulysses_pieces(int32_t to_pieces, int32_t group, int32_t B, int64_t s_loc, int32_t P_u, int32_t n,
                      void* const* tensors, const int64_t* run_bytes, void* pieces, void* stream) {
  if (to_pieces != 0 && to_pieces != 1) return fail(RA_E_INVAL, "to_pieces must be 0 or 1");
  if (group != RA_GROUP_HEADS && group != RA_GROUP_SEQ)
    return fail(RA_E_INVAL, "group must be RA_GROUP_HEADS or RA_GROUP_SEQ");
  if (n < 1 || n > ra::kMaxPieceTensors) return fail(RA_E_INVAL, "n = %d outside [1, %d]", n, ra::kMaxPieceTensors);
  if (B < 0 || s_loc < 0 || P_u < 1) return fail(RA_E_INVAL, "bad shape");
  if (!tensors || !run_bytes) return fail(RA_E_INVAL, "NULL tensor or run list");
  int64_t piece = 0;
  for (int i = 0; i < n; ++i) {
    if (run_bytes[i] < 1) return fail(RA_E_INVAL, "run_bytes[%d] must be >= 1", i);
    piece += (int64_t)B * s_loc * run_bytes[i];
  }
  if (piece == 0) return ok();
  if (!pieces) return fail(RA_E_INVAL, "NULL pieces");
  const uintptr_t p0 = (uintptr_t)pieces, p1 = p0 + (uintptr_t)(piece * P_u);
  uintptr_t align = p0 | (uintptr_t)piece;
  int64_t sec = 0;
  for (int i = 0; i < n; ++i) {
    if (!tensors[i]) return fail(RA_E_INVAL, "NULL tensor %d", i);
    const int64_t bytes = (int64_t)P_u * B * s_loc * run_bytes[i];
    const uintptr_t t0 = (uintptr_t)tensors[i], t1 = t0 + (uintptr_t)bytes;
    if (t0 < p1 && p0 < t1) return fail(RA_E_INVAL, "tensor %d overlaps the pieces", i);
    align |= t0 | (uintptr_t)run_bytes[i] | (uintptr_t)sec;
    sec += (int64_t)B * s_loc * run_bytes[i];
  }
  int unit = 16;
  while (unit > 1 && (align % (uintptr_t)unit)) unit /= 2;
  for (int i = 0; i < n; ++i)
    if ((int64_t)P_u * B * s_loc * (run_bytes[i] / unit) >= ((int64_t)1 << 31))
      return fail(RA_E_INVAL, "tensor %d too large for one call (2^31 units)", i);
  if (piece * P_u / unit >= ((int64_t)1 << 31)) return fail(RA_E_INVAL, "pieces too large for one call");
  hipError_t e = ra::launch_pieces(to_pieces, group, B, s_loc, P_u, n, tensors, (const long long*)run_bytes, pieces,
                                   unit, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_E_HIP, "pieces launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
