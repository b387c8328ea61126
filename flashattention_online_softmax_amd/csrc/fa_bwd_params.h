// Backward parameters and launchers (fa_bwd.hip), apart from the forward's
// shared declarations so that the backward can change without touching the
// headers the forward kernels are built from.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

// Attention backward parameters (16-bit, D = 64 or 128). Strides in elements.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // [B, Hq, Sq] contiguous
  float* delta;       // [B, Hq, Sq] contiguous: dO . O per row (written)
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t dq_sb, dq_sh, dq_ss;
  const uint8_t* mask;  // NULL, or [B|1, Hq|1, Sq, Skv] bytes, non-zero = excluded
  int64_t m_sb, m_sh, m_ss;  // 0 for a broadcast dim
  const int32_t* seqlens_q;  // nullable [B]: rows i >= Lq_b have no keys
  const int32_t* seqlens_k;  // nullable [B]: keys j >= Lk_b are excluded
  const float* o_lo;   // nullable [B, Hq, Sq, Dv] fp32: O - rounded(O) of the forward
  int64_t ol_sb, ol_sh, ol_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  int32_t B, Hq, Hkv, G, Sq, Skv;
  float scale;
  float scale_log2;
  // Packed variable-length batches (nullable): batch b's query rows are rows
  // cu_q[b] .. cu_q[b+1]-1 of q, o, dout, dq (and of the [Tq, Hq] lse and
  // delta), its keys rows cu_k[b] .. cu_k[b+1]-1 of k, v, dk, dv; Sq and Skv
  // are then the longest lengths, Tq and Tk the tensors' row counts.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t Tq, Tk;
  // Nullable dS workspace in the input dtype, tile-major: for (batch b,
  // query head hq), 256-row block rb, 32-key tile kt and 32-row sub-block
  // sb, one contiguous 32 x 32 block, key-major (dS of key j, row i at
  // element 32 (j % 32) + 16 ((r >> 2) & 1) + 4 (r >> 3) + (r & 3), r = i %
  // 32: the order in which a lane holds its rows in the accumulator):
  //   block (((b Hq + hq) ds_nrb + rb) ds_nkt + kt) 8 + sb, 1024 elements
  // with ds_nrb = ceil(Sq / 256) and ds_nkt = ceil(Skv / 32). When set, the
  // dK/dV kernel stores dS there and dQ = scale dS K is formed from it
  // instead of recomputing S and dP; ds_qp = Sq rounded up to 32.
  uint16_t* ds;
  int32_t ds_nrb, ds_nkt, ds_qp;
  // Non-zero: store dS non-temporally (the blocks the sweep touches exceed
  // what the last-level cache would keep for the dQ kernel).
  int32_t ds_nt;
  // With ds: fp32 start values of the S and dP accumulators per 32-row tile,
  // after the dS region of the workspace: at ((b Hq + hq) ds_qp / 32 + t) 64,
  // 32 values -LSE / scale (+inf for rows without keys or past the batch),
  // then 32 values -Delta.
  float* ldrec;
};

// Elements (16-bit) of the backward's workspace for (B, Hq, Sq, Skv): the
// dS blocks, then the per-tile start values (two fp32 per row).
inline int64_t bwd_ds_blocks_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  return B * Hq * ((Sq + 255) / 256 * 256) * ((Skv + 31) / 32 * 32);
}
inline int64_t bwd_ds_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  return bwd_ds_blocks_elems(B, Hq, Sq, Skv) + B * Hq * ((Sq + 31) / 32 * 32) * 4;
}

hipError_t launch_bwd(Dt dt, int d, bool causal, bool mask, BwdParams& p, hipStream_t stream);
// The backward over packed variable-length batches (p.cu_q / p.cu_k set, no mask).
hipError_t launch_bwd_varlen(Dt dt, int d, bool causal, BwdParams& p, hipStream_t stream);

}  // namespace fa
