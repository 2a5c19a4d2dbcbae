// Internal interface between the C ABI (ra_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Query rows per workgroup of the f32 kernel (4 waves x 32 rows); keys per
// LDS tile of both kernels.  The bf16 kernel states its own workgroup rows.
constexpr int kBQ = 128;
constexpr int kBK = 32;

// Query rows per workgroup of the bf16 kernel (defined with it).
int attn_step_rows_bf16();

// Query rows per workgroup for dtype 0 = f32, 1 = bf16.
inline int step_rows(int dtype) { return dtype == 1 ? attn_step_rows_bf16() : kBQ; }

// Everything one launch of the attention step kernel needs.  Spans are the
// (at most two) query / key spans of the step in local row order; only query
// spans that have work are listed (in ACCUM mode a span that sees no key is
// dropped so its workgroups are never launched).
struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, G;        // G = Hq / Hkv
  long long Sq, Sk;         // rows of q / k (row strides of the batch dim)
  int causal, accum;
  float scale, sl2;         // sl2 = scale * log2(e)
  int nqs, nks;
  long long qs_start[2], qs_len[2], qs_off[2];
  long long ks_start[2], ks_len[2], ks_off[2];
  long long window;         // > 0: a query sees its `window` most recent keys (causal only)
  const long long* cu;      // packed sequences: boundaries cu[0..nseg] (device), or null
  int nseg;
  int mask_ext;             // window or packed sequences in use
  int qt_span0;             // query tiles in listed query span 0
  int n_qtiles;             // query tiles per (batch, head)
  int n_work;               // B * Hq * n_qtiles
  int per_xcd;              // ceil(n_work / 8)
  int lpt;                  // 1: each XCD's items are whole heads, walked heaviest tile first across them
  int first_heavy;          // 1: the first query tiles see the most keys (walk them first)
  int ksplit;               // bf16, D = 128: eight-wave workgroups splitting each item's key tiles
};

// dtype: 0 = f32, 1 = bf16; D in {64, 128}.  The work decomposition of p
// (n_qtiles, qt_span0) must use step_rows(dtype) rows per query tile.
hipError_t launch_attn_step(const StepParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_attn_step_f32(const StepParams& p, int D, hipStream_t s);
hipError_t launch_attn_step_bf16(const StepParams& p, int D, hipStream_t s);

// Backward of one ring step for bf16 inputs, D = 128: the dQ kernel (query
// tiles of kBwdRows rows, loops over the step's key tiles) and the dK/dV
// kernel (key tiles of kBwdKeys keys, loops over the query heads of their
// group and the visible query tiles).
constexpr int kBwdRows = 128;
constexpr int kBwdKeys = 128;

struct BwdParams {
  StepParams s;          // q, k, v, spans, shapes, causal, scale; s.accum: dQ INIT / ACCUM;
                         // s.n_qtiles, qt_span0, n_work, per_xcd: the dQ kernel's query tiles
  const void* dout;      // dO, the layout and dtype of q
  const float* lse;      // forward LSE (natural log), [B, Sq, Hq]
  const float* delta;    // rowsum(dO * O), [B, Sq, Hq]
  float* dq;             // [B, Sq, Hq, D]: written (INIT) or added to (ACCUM)
  float* dk;             // [B, Sk, Hkv, D]: added to
  float* dv;             // [B, Sk, Hkv, D]: added to
  int kt_span0;          // key tiles in listed key span 0
  int n_ktiles;          // key tiles per (batch, kv head)
  int n_kwork;           // B * Hkv * n_ktiles
  int per_xcd_kv;        // ceil(n_kwork / 8)
  int kv_split;          // 1: two groups of four waves per key tile (few key tiles with work)
};

hipError_t launch_attn_bwd_bf16(const BwdParams& p, hipStream_t s);
// The same step for float32 inputs (dtype 0) or D = 64: plain SIMT kernels.
hipError_t launch_attn_bwd_simt(const BwdParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_simt_delta(long long rows, int D, int dtype, const void* dout, const float* o, float* delta,
                             hipStream_t s);
// delta[row] = sum_d dO[row, d] * O[row, d] over rows of D elements; dO bf16
// (dtype 1) or f32 (dtype 0), O f32.
hipError_t launch_bwd_delta(long long rows, int D, int dtype, const void* dout, const float* o, float* delta,
                            hipStream_t s);

hipError_t launch_lse_merge(long long rows, int D, const float* o_a,
                            const float* lse_a, const float* o_b,
                            const float* lse_b, float* o_out, float* lse_out,
                            hipStream_t s);

// Bytes moved per thread by the relayout kernel for these runs and pointers.
int relayout_unit(long long run_bytes, const void* in, const void* out);

hipError_t launch_relayout(int dir, int elem_bytes, int B, long long s_loc,
                           int H, int D, int P_u, const void* in, void* out,
                           hipStream_t s);

// Multi-tensor Ulysses messages (at most kMaxPieceTensors tensors per call).
// to_pieces: tensors -> pieces, else pieces -> tensors; group 0: head blocks,
// 1: token blocks; unit: bytes moved per thread (divides every run, section
// and pointer).
constexpr int kMaxPieceTensors = 4;
hipError_t launch_pieces(int to_pieces, int group, int B, long long s_loc, int P_u, int n, void* const* tensors,
                         const long long* run_bytes, void* pieces, int unit, hipStream_t s);

}  // namespace ra
