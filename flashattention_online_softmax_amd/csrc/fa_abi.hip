// C ABI of libfa.so: argument validation on the host, then dispatch to the
// gfx950 kernels on the caller's stream. See include/fa.h for the contract.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fa.h"
#include "fa_bwd_params.h"
#include "fa_internal.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

int64_t elem_size(int32_t dt) {
  switch (dt) {
    case FA_F32: return 4;
    case FA_F16: return 2;
    case FA_BF16: return 2;
    case FA_U8: return 1;
    case FA_I32: return 4;
    default: return 0;
  }
}

const char* dtype_name(int32_t dt) {
  switch (dt) {
    case FA_F32: return "f32";
    case FA_F16: return "f16";
    case FA_BF16: return "bf16";
    case FA_U8: return "u8";
    case FA_I32: return "i32";
    default: return "?";
  }
}

int64_t numel(const fa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Rank, extents >= 0, unit last stride (unless empty), non-null data when
// non-empty, and 16-byte alignment of the data pointer and of every row
// (rows_aligned) for vector loads.
fa_status check_tensor(const char* name, const fa_tensor* t, int ndim, bool rows_aligned) {
  if (!t) return fail(FA_ERR_NULL, "%s is NULL", name);
  if (t->ndim != ndim) return fail(FA_ERR_SHAPE, "%s must have rank %d, got %d", name, ndim, t->ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(FA_ERR_SHAPE, "%s has a negative extent", name);
  if (elem_size(t->dtype) == 0) return fail(FA_ERR_DTYPE, "%s has unknown dtype %d", name, t->dtype);
  if (numel(t) == 0) return FA_OK;
  if (!t->data) return fail(FA_ERR_NULL, "%s.data is NULL", name);
  if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1)
    return fail(FA_ERR_STRIDE, "%s: last dimension must be contiguous (stride %lld)", name,
                (long long)t->stride[ndim - 1]);
  for (int i = 0; i < ndim; ++i)
    if (t->stride[i] < 0) return fail(FA_ERR_STRIDE, "%s: negative stride", name);
  if (rows_aligned) {
    const int64_t es = elem_size(t->dtype);
    if (((uintptr_t)t->data) % 16 != 0) return fail(FA_ERR_STRIDE, "%s.data is not 16-byte aligned", name);
    for (int i = 0; i < ndim - 1; ++i)
      if (t->shape[i] > 1 && (t->stride[i] * es) % 16 != 0)
        return fail(FA_ERR_STRIDE, "%s: stride of dim %d is not a multiple of 16 bytes", name, i);
  }
  return FA_OK;
}

fa_status check_dtype(const char* name, const fa_tensor* t, int32_t want) {
  if (t->dtype != want)
    return fail(FA_ERR_DTYPE, "%s has dtype %s, expected %s", name, dtype_name(t->dtype), dtype_name(want));
  return FA_OK;
}

fa_status check_contiguous(const char* name, const fa_tensor* t) {
  if (numel(t) == 0) return FA_OK;
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] > 1 && t->stride[i] != expect)
      return fail(FA_ERR_STRIDE, "%s must be contiguous", name);
    expect *= t->shape[i];
  }
  return FA_OK;
}

// Optional int32 [B] sequence-length vector.
fa_status check_seqlens(const char* name, const fa_tensor* t, int64_t B) {
  if (!t) return FA_OK;
  fa_status s = check_tensor(name, t, 1, false);
  if (s != FA_OK) return s;
  if ((s = check_dtype(name, t, FA_I32)) != FA_OK) return s;
  if (t->shape[0] != B) return fail(FA_ERR_SHAPE, "%s must have %lld entries", name, (long long)B);
  return FA_OK;
}

// Optional fp32 rounding residual shaped like o (16-byte aligned rows).
fa_status check_o_lo(const fa_tensor* o_lo, const fa_tensor* o) {
  if (!o_lo) return FA_OK;
  fa_status s = check_tensor("o_lo", o_lo, o->ndim, true);
  if (s != FA_OK) return s;
  if ((s = check_dtype("o_lo", o_lo, FA_F32)) != FA_OK) return s;
  for (int i = 0; i < o->ndim; ++i)
    if (o_lo->shape[i] != o->shape[i]) return fail(FA_ERR_SHAPE, "o_lo must be shaped like o");
  if (o->dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "o_lo is for 16-bit outputs");
  return FA_OK;
}

// Bytes of stored dS beyond which the dK/dV kernel stores it non-temporally
// (measured on MI355X, causal bf16 D = 128: at 134 MB touched the cached
// stores let the dQ kernel read dS from the 256 MB last-level cache and win
// by 9%; at 269 MB they lose and the non-temporal ones win).
constexpr int64_t kDsCachedBytes = (int64_t)192 << 20;

// Optional dS workspace of the backward: rank 1, q's dtype, contiguous,
// 16-byte aligned, at least fa_bwd_ds_workspace_elems(B, Hq, Sq, Skv)
// elements. Sets p.ds, its block counts and the store kind when one is
// given (causal: half of the blocks are touched).
fa_status check_ds_work(const fa_tensor* ds, int32_t dtype, int64_t B, int64_t Hq, int64_t Sq, int64_t Skv,
                        bool causal, fa::BwdParams& p) {
  if (!ds || numel(ds) == 0) return FA_OK;
  fa_status s = check_tensor("ds_workspace", ds, 1, true);
  if (s != FA_OK) return s;
  if ((s = check_dtype("ds_workspace", ds, dtype)) != FA_OK) return s;
  const int64_t need = fa::bwd_ds_elems(B, Hq, Sq, Skv);
  if (ds->shape[0] < need)
    return fail(FA_ERR_SHAPE, "ds_workspace holds %lld elements, %lld needed", (long long)ds->shape[0],
                (long long)need);
  p.ds = (uint16_t*)ds->data;
  p.ds_nrb = (int32_t)((Sq + 255) / 256);
  p.ds_nkt = (int32_t)((Skv + 31) / 32);
  p.ds_qp = (int32_t)((Sq + 31) / 32 * 32);
  p.ldrec = (float*)(p.ds + fa::bwd_ds_blocks_elems(B, Hq, Sq, Skv));
  const int64_t touched = 2 * fa::bwd_ds_blocks_elems(B, Hq, Sq, Skv) / (causal ? 2 : 1);
  p.ds_nt = touched > kDsCachedBytes ? 1 : 0;
  return FA_OK;
}

fa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
}

bool fits_i32(int64_t x) { return x >= 0 && x <= 0x7fffffff; }

// The kernels work in the exp2 domain with c = scale * log2(e); c must be a
// normal positive float so that masked scores (-inf) stay -inf after scaling.
bool scale_ok(float scale) {
  return std::isfinite(scale) && scale * 1.4426950408889634f >= 1.17549435e-38f;
}

// Shared validation of q/k/v/o/lse for the BNSD entry points.
// Largest rescale threshold accepted (log2 units): p stays <= 2^10, far
// inside the fp16 range.
constexpr float kMaxRescaleThreshold = 10.f;

fa_status check_bnsd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* o,
                     const fa_tensor* lse, float scale, float rescale_threshold) {
  fa_status s;
  if ((s = check_tensor("q", q, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("k", k, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("v", v, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("o", o, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("lse", lse, 3, false)) != FA_OK) return s;
  if (q->dtype != FA_F32 && q->dtype != FA_F16 && q->dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "q dtype must be f32, f16 or bf16, got %s", dtype_name(q->dtype));
  if ((s = check_dtype("k", k, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("v", v, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("o", o, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("lse", lse, FA_F32)) != FA_OK) return s;
  const int64_t B = q->shape[0], Hq = q->shape[1], Sq = q->shape[2], D = q->shape[3];
  const int64_t Hkv = k->shape[1], Skv = k->shape[2];
  if (k->shape[0] != B || v->shape[0] != B) return fail(FA_ERR_SHAPE, "batch sizes of q, k, v differ");
  if (k->shape[3] != D) return fail(FA_ERR_SHAPE, "k head dim %lld != q head dim %lld", (long long)k->shape[3], (long long)D);
  if (v->shape[1] != Hkv || v->shape[2] != Skv) return fail(FA_ERR_SHAPE, "v must match k in heads and length");
  const int64_t Dv = v->shape[3];
  if (o->shape[0] != B || o->shape[1] != Hq || o->shape[2] != Sq || o->shape[3] != Dv)
    return fail(FA_ERR_SHAPE, "o must be [B, Hq, Sq, Dv]");
  if (lse->shape[0] != B || lse->shape[1] != Hq || lse->shape[2] != Sq)
    return fail(FA_ERR_SHAPE, "lse must be [B, Hq, Sq]");
  if ((s = check_contiguous("lse", lse)) != FA_OK) return s;
  if (Hkv == 0 && B * Hq * Sq > 0) return fail(FA_ERR_SHAPE, "k has no heads");
  if (Hkv > 0 && Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (!scale_ok(scale)) return fail(FA_ERR_VALUE, "scale must be finite and > 0");
  if (!(rescale_threshold >= 0.f && rescale_threshold <= kMaxRescaleThreshold))
    return fail(FA_ERR_VALUE, "rescale_threshold must be in [0, %g]", (double)kMaxRescaleThreshold);
  if (D != Dv) return fail(FA_ERR_UNSUPPORTED, "D (%lld) != Dv (%lld) is not supported", (long long)D, (long long)Dv);
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)D);
  if (!fits_i32(B * Hq * Sq) || !fits_i32(Skv) || !fits_i32(B * Hq))
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  // K/V tiles are fetched with 32-bit per-lane offsets from the tile start.
  if (k->stride[2] > (1 << 22) || v->stride[2] > (1 << 22))
    return fail(FA_ERR_UNSUPPORTED, "k/v row stride above 2^22 elements is not supported");
  return FA_OK;
}

void fill_common(fa::FwdParams& p, const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                 const fa_tensor* o, const fa_tensor* lse, float scale, float rescale_threshold) {
  memset(&p, 0, sizeof(p));
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.lse = (float*)lse->data;
  p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_ss = q->stride[2];
  p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_ss = k->stride[2];
  p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_ss = v->stride[2];
  p.o_sb = o->stride[0]; p.o_sh = o->stride[1]; p.o_ss = o->stride[2];
  p.B = (int32_t)q->shape[0];
  p.Hq = (int32_t)q->shape[1];
  p.Sq = (int32_t)q->shape[2];
  p.Hkv = (int32_t)k->shape[1];
  p.Skv = (int32_t)k->shape[2];
  p.G = p.Hkv > 0 ? p.Hq / p.Hkv : 1;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.rescale_thr = rescale_threshold;
  p.lse_sb = (int64_t)p.Hq * p.Sq;
  p.lse_sh = p.Sq;
  p.lse_ss = 1;
  p.n_splits = 1;
}

// Split-KV sizing shared by the entry points and the sizing helpers: the
// number of key ranges (the requested count, or with 0 the fewest that give
// every compute unit of an MI355X (256) one workgroup, at least 384 keys per
// range, at most 64 ranges), each a multiple of 192 keys (whole 64- and
// 96-key tiles); ranges past the keys are dropped. One round of the GPU
// measured 3-22% faster than two over six few-row shapes (the split-KV
// workload: 8 -> 4 ranges, 0.518 -> 0.501 ms): longer ranges amortise each
// workgroup's prologue and write fewer partial results.
constexpr int kSplitGranule = 192;
constexpr int kMaxSplits = 64;
constexpr int kSplitFillWorkgroups = 256;

int split_plan(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int requested, int* split_len) {
  if (B < 0 || Hq < 0 || Sq < 0 || Skv < 0 || requested < 0) return -1;
  int ns = requested;
  if (ns == 0) {
    const int64_t base = ((Sq + 255) / 256) * B * Hq;
    ns = base > 0 ? (int)std::min<int64_t>(kMaxSplits, (kSplitFillWorkgroups + base - 1) / base) : 1;
    ns = (int)std::min<int64_t>(ns, std::max<int64_t>(1, Skv / 384));
  }
  ns = std::max(1, std::min(ns, kMaxSplits));
  int64_t len = Skv > 0 ? (Skv + ns - 1) / ns : kSplitGranule;
  len = (len + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  if (split_len) *split_len = (int)len;
  return Skv > 0 ? (int)((Skv + len - 1) / len) : 1;
}

fa::Dt to_dt(int32_t d) { return d == FA_F32 ? fa::Dt::F32 : d == FA_F16 ? fa::Dt::F16 : fa::Dt::BF16; }

}  // namespace

extern "C" {

// The boolean mask forms shared by the forward and the backward: uint8
// [Sq, Skv] or [B|1, Hq|1, Sq, Skv]; a broadcast dim gets stride 0.
static fa_status parse_mask(const fa_tensor* mask, int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int64_t* sb,
                            int64_t* sh, int64_t* ss) {
  fa_status s;
  if (mask->ndim != 2 && mask->ndim != 4) return fail(FA_ERR_SHAPE, "mask must have rank 2 or 4");
  if ((s = check_tensor("mask", mask, mask->ndim, false)) != FA_OK) return s;
  if ((s = check_dtype("mask", mask, FA_U8)) != FA_OK) return s;
  if (mask->ndim == 2) {
    if (mask->shape[0] != Sq || mask->shape[1] != Skv) return fail(FA_ERR_SHAPE, "mask must be [Sq, Skv]");
    *sb = 0;
    *sh = 0;
    *ss = mask->stride[0];
  } else {
    if ((mask->shape[0] != B && mask->shape[0] != 1) || (mask->shape[1] != Hq && mask->shape[1] != 1) ||
        mask->shape[2] != Sq || mask->shape[3] != Skv)
      return fail(FA_ERR_SHAPE, "mask must be [B|1, Hq|1, Sq, Skv]");
    *sb = mask->shape[0] == 1 ? 0 : mask->stride[0];
    *sh = mask->shape[1] == 1 ? 0 : mask->stride[1];
    *ss = mask->stride[2];
  }
  return FA_OK;
}

fa_status fa_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* mask,
                 const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, int causal, float scale,
                 float rescale_threshold, const fa_tensor* o, const fa_tensor* o_lo, const fa_tensor* lse,
                 void* stream) {
  clear_error();
  fa_status s = check_bnsd(q, k, v, o, lse, scale, rescale_threshold);
  if (s != FA_OK) return s;
  if ((s = check_o_lo(o_lo, o)) != FA_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA_ERR_VALUE, "causal must be 0 or 1");
  const int64_t B = q->shape[0], Hq = q->shape[1], Sq = q->shape[2], Skv = k->shape[2];
  if ((s = check_seqlens("seqlens_q", seqlens_q, B)) != FA_OK) return s;
  if ((s = check_seqlens("seqlens_k", seqlens_k, B)) != FA_OK) return s;
  fa::FwdParams p;
  fill_common(p, q, k, v, o, lse, scale, rescale_threshold);
  if (mask) {
    if ((s = parse_mask(mask, B, Hq, Sq, Skv, &p.m_sb, &p.m_sh, &p.m_ss)) != FA_OK) return s;
    p.mask = (const uint8_t*)mask->data;
    p.mask_vec4 = (((uintptr_t)mask->data) % 4 == 0) && (p.m_sb % 4 == 0) && (p.m_sh % 4 == 0) &&
                  (p.m_ss % 4 == 0);
    p.mask_vec16 = (((uintptr_t)mask->data) % 16 == 0) && (p.m_sb % 16 == 0) && (p.m_sh % 16 == 0) &&
                   (p.m_ss % 16 == 0);
    // LDS-staged mask tiles: whole 16-byte chunks of every row up to Skv, and
    // 32-bit offsets for 32 rows of one (batch, head) slice.
    p.mask_lds = p.mask_vec16 && Skv % 16 == 0 && p.m_ss < (int64_t(1) << 26);
  }
  p.seqlens_q = seqlens_q ? (const int32_t*)seqlens_q->data : nullptr;
  p.seqlens_k = seqlens_k ? (const int32_t*)seqlens_k->data : nullptr;
  if (o_lo && numel(o_lo) > 0) {
    p.o_lo = (float*)o_lo->data;
    p.ol_sb = o_lo->stride[0];
    p.ol_sh = o_lo->stride[1];
    p.ol_ss = o_lo->stride[2];
  }
  if (B * Hq * Sq == 0) return FA_OK;
  const bool has_mask = mask && numel(mask) > 0;
  if (mask && !has_mask && Skv > 0) return fail(FA_ERR_SHAPE, "mask is empty");
  return hip_status(fa::launch_dense(to_dt(q->dtype), (int)q->shape[3], causal != 0, has_mask, false, p,
                                     (hipStream_t)stream));
}

fa_status fa_fwd_blocksparse(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                             const fa_tensor* block_idx, int block_q, int block_k,
                             const fa_tensor* seqlens, float scale, float rescale_threshold,
                             const fa_tensor* o, const fa_tensor* lse, void* stream) {
  clear_error();
  fa_status s = check_bnsd(q, k, v, o, lse, scale, rescale_threshold);
  if (s != FA_OK) return s;
  if (block_q != 128 || block_k != 128)
    return fail(FA_ERR_UNSUPPORTED, "block_q and block_k must be 128 (got %d, %d)", block_q, block_k);
  const int64_t B = q->shape[0], Hq = q->shape[1], Sq = q->shape[2], Hkv = k->shape[1];
  if ((s = check_seqlens("seqlens", seqlens, B)) != FA_OK) return s;
  if (!block_idx) return fail(FA_ERR_NULL, "block_idx is NULL");
  if (block_idx->ndim != 2 && block_idx->ndim != 4) return fail(FA_ERR_SHAPE, "block_idx must have rank 2 or 4");
  if ((s = check_tensor("block_idx", block_idx, block_idx->ndim, false)) != FA_OK) return s;
  if ((s = check_dtype("block_idx", block_idx, FA_I32)) != FA_OK) return s;
  fa::FwdParams p;
  fill_common(p, q, k, v, o, lse, scale, rescale_threshold);
  const int nd = block_idx->ndim;
  const int64_t nqb = block_idx->shape[nd - 2], max_sel = block_idx->shape[nd - 1];
  if (nqb < (Sq + block_q - 1) / block_q) return fail(FA_ERR_SHAPE, "block_idx has %lld query blocks, need %lld", (long long)nqb, (long long)((Sq + block_q - 1) / block_q));
  if (max_sel > 256) return fail(FA_ERR_UNSUPPORTED, "maxSel %lld > 256", (long long)max_sel);
  if (nd == 4) {
    if ((block_idx->shape[0] != B && block_idx->shape[0] != 1) || (block_idx->shape[1] != Hkv && block_idx->shape[1] != 1))
      return fail(FA_ERR_SHAPE, "block_idx must be [B|1, Hkv|1, nQB, maxSel]");
    p.bi_sb = block_idx->shape[0] == 1 ? 0 : block_idx->stride[0];
    p.bi_sh = block_idx->shape[1] == 1 ? 0 : block_idx->stride[1];
  }
  p.bi_sq = block_idx->stride[nd - 2];
  p.max_sel = (int32_t)max_sel;
  p.block_idx = (const int32_t*)block_idx->data;
  p.seqlens_q = seqlens ? (const int32_t*)seqlens->data : nullptr;
  p.seqlens_k = p.seqlens_q;
  if (B * Hq * Sq == 0) return FA_OK;
  if (max_sel > 0 && !block_idx->data) return fail(FA_ERR_NULL, "block_idx.data is NULL");
  return hip_status(fa::launch_dense(to_dt(q->dtype), (int)q->shape[3], false, false, true, p, (hipStream_t)stream));
}

fa_status fa_fwd_topk_gather(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                             const fa_tensor* idx, float scale, const fa_tensor* o,
                             const fa_tensor* o_lo, const fa_tensor* lse, void* stream) {
  clear_error();
  fa_status s;
  if ((s = check_tensor("q", q, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("k", k, 2, true)) != FA_OK) return s;
  if ((s = check_tensor("v", v, 2, true)) != FA_OK) return s;
  if ((s = check_tensor("idx", idx, 2, false)) != FA_OK) return s;
  if ((s = check_tensor("o", o, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("lse", lse, 2, false)) != FA_OK) return s;
  if (q->dtype != FA_F16 && q->dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "q dtype must be f16 or bf16, got %s", dtype_name(q->dtype));
  if ((s = check_dtype("k", k, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("v", v, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("o", o, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("idx", idx, FA_I32)) != FA_OK) return s;
  if ((s = check_dtype("lse", lse, FA_F32)) != FA_OK) return s;
  const int64_t T = q->shape[0], Hq = q->shape[1], Dqk = q->shape[2];
  const int64_t S = k->shape[0], Dv = v->shape[1], W = idx->shape[1];
  if (k->shape[1] != Dqk) return fail(FA_ERR_SHAPE, "k must be [S, Dqk]");
  if (v->shape[0] != S) return fail(FA_ERR_SHAPE, "v must have as many rows as k");
  if (idx->shape[0] != T) return fail(FA_ERR_SHAPE, "idx must be [T, W]");
  if (o->shape[0] != T || o->shape[1] != Hq || o->shape[2] != Dv) return fail(FA_ERR_SHAPE, "o must be [T, Hq, Dv]");
  if (lse->shape[0] != T || lse->shape[1] != Hq) return fail(FA_ERR_SHAPE, "lse must be [T, Hq]");
  if ((s = check_contiguous("lse", lse)) != FA_OK) return s;
  if (!scale_ok(scale)) return fail(FA_ERR_VALUE, "scale must be finite and > 0");
  if (Dqk != 576 || Dv != 512) return fail(FA_ERR_UNSUPPORTED, "only Dqk = 576, Dv = 512 is supported");
  if (W > 4096) return fail(FA_ERR_UNSUPPORTED, "W (%lld) > 4096", (long long)W);
  if (!fits_i32(T * Hq) || !fits_i32(S) || !fits_i32(W)) return fail(FA_ERR_UNSUPPORTED, "problem too large");
  // Bytes spanned by k and v (the gathers address them with 32-bit offsets).
  const int64_t k_bytes = S > 0 ? (S - 1) * k->stride[0] * 2 + Dqk * 2 : 0;
  const int64_t v_bytes = S > 0 ? (S - 1) * v->stride[0] * 2 + Dv * 2 : 0;
  if (k_bytes > 0xFFFFFFFFLL || v_bytes > 0xFFFFFFFFLL)
    return fail(FA_ERR_UNSUPPORTED, "k and v must each span less than 4 GiB");
  if ((s = check_o_lo(o_lo, o)) != FA_OK) return s;
  if (T * Hq == 0) return FA_OK;
  if (W > 0 && !idx->data) return fail(FA_ERR_NULL, "idx.data is NULL");
  fa::TopkParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.lse = (float*)lse->data;
  p.idx = (const int32_t*)idx->data;
  p.q_st = q->stride[0]; p.q_sh = q->stride[1];
  p.k_ss = k->stride[0]; p.v_ss = v->stride[0];
  p.o_st = o->stride[0]; p.o_sh = o->stride[1];
  if (o_lo && numel(o_lo) > 0) {
    p.o_lo = (float*)o_lo->data;
    p.ol_st = o_lo->stride[0];
    p.ol_sh = o_lo->stride[1];
  }
  p.idx_st = idx->stride[0];
  p.T = (int32_t)T; p.Hq = (int32_t)Hq; p.S = (int32_t)S; p.W = (int32_t)W;
  p.k_bytes = (uint32_t)k_bytes; p.v_bytes = (uint32_t)v_bytes;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(fa::launch_topk(to_dt(q->dtype), p, (hipStream_t)stream));
}

fa_status fa_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* mask,
                 const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, const fa_tensor* o,
                 const fa_tensor* o_lo, const fa_tensor* lse, const fa_tensor* dout, int causal, float scale,
                 const fa_tensor* delta, const fa_tensor* dq, const fa_tensor* dk,
                 const fa_tensor* dv, const fa_tensor* ds_workspace, void* stream) {
  clear_error();
  fa_status s = check_bnsd(q, k, v, o, lse, scale, 0.f);
  if (s != FA_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA_ERR_VALUE, "causal must be 0 or 1");
  if ((s = check_seqlens("seqlens_q", seqlens_q, q->shape[0])) != FA_OK) return s;
  if ((s = check_seqlens("seqlens_k", seqlens_k, q->shape[0])) != FA_OK) return s;
  if ((s = check_o_lo(o_lo, o)) != FA_OK) return s;
  if (q->dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the backward takes f16 or bf16");
  if (q->shape[3] != 64 && q->shape[3] != 128)
    return fail(FA_ERR_UNSUPPORTED, "the backward supports head dim 64 or 128 (got %lld)", (long long)q->shape[3]);
  if ((s = check_tensor("dout", dout, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("dq", dq, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("dk", dk, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("dv", dv, 4, true)) != FA_OK) return s;
  if ((s = check_tensor("delta", delta, 3, false)) != FA_OK) return s;
  if ((s = check_dtype("dout", dout, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("dq", dq, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("dk", dk, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("dv", dv, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("delta", delta, FA_F32)) != FA_OK) return s;
  // Q and dO tiles are fetched with 32-bit per-lane offsets from the tile start.
  if (q->stride[2] > (1 << 22) || dout->stride[2] > (1 << 22))
    return fail(FA_ERR_UNSUPPORTED, "q/dout row stride above 2^22 elements is not supported");
  for (int i = 0; i < 4; ++i) {
    if (dout->shape[i] != o->shape[i]) return fail(FA_ERR_SHAPE, "dout must be shaped like o");
    if (dq->shape[i] != q->shape[i]) return fail(FA_ERR_SHAPE, "dq must be shaped like q");
    if (dk->shape[i] != k->shape[i]) return fail(FA_ERR_SHAPE, "dk must be shaped like k");
    if (dv->shape[i] != v->shape[i]) return fail(FA_ERR_SHAPE, "dv must be shaped like v");
  }
  for (int i = 0; i < 3; ++i)
    if (delta->shape[i] != lse->shape[i]) return fail(FA_ERR_SHAPE, "delta must be [B, Hq, Sq]");
  if ((s = check_contiguous("delta", delta)) != FA_OK) return s;
  fa::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.dout = dout->data;
  p.lse = (const float*)lse->data;
  p.delta = (float*)delta->data;
  p.dq = dq->data;
  p.dk = dk->data;
  p.dv = dv->data;
  const fa_tensor* ts[8] = {q, k, v, o, dout, dq, dk, dv};
  int64_t* st[8][3] = {{&p.q_sb, &p.q_sh, &p.q_ss},    {&p.k_sb, &p.k_sh, &p.k_ss},
                       {&p.v_sb, &p.v_sh, &p.v_ss},    {&p.o_sb, &p.o_sh, &p.o_ss},
                       {&p.do_sb, &p.do_sh, &p.do_ss}, {&p.dq_sb, &p.dq_sh, &p.dq_ss},
                       {&p.dk_sb, &p.dk_sh, &p.dk_ss}, {&p.dv_sb, &p.dv_sh, &p.dv_ss}};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) *st[t][i] = ts[t]->stride[i];
  p.B = (int32_t)q->shape[0];
  p.Hq = (int32_t)q->shape[1];
  p.Hkv = (int32_t)k->shape[1];
  p.G = p.Hkv > 0 ? p.Hq / p.Hkv : 1;
  p.Sq = (int32_t)q->shape[2];
  p.Skv = (int32_t)k->shape[2];
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (mask) {
    if ((s = parse_mask(mask, p.B, p.Hq, p.Sq, p.Skv, &p.m_sb, &p.m_sh, &p.m_ss)) != FA_OK) return s;
    p.mask = (const uint8_t*)mask->data;
  }
  p.seqlens_q = seqlens_q ? (const int32_t*)seqlens_q->data : nullptr;
  p.seqlens_k = seqlens_k ? (const int32_t*)seqlens_k->data : nullptr;
  if (o_lo && numel(o_lo) > 0) {
    p.o_lo = (const float*)o_lo->data;
    p.ol_sb = o_lo->stride[0];
    p.ol_sh = o_lo->stride[1];
    p.ol_ss = o_lo->stride[2];
  }
  if ((s = check_ds_work(ds_workspace, q->dtype, p.B, p.Hq, p.Sq, p.Skv, causal != 0, p)) != FA_OK) return s;
  if ((int64_t)p.B * p.Hq * p.Sq == 0 && (int64_t)p.B * p.Hkv * p.Skv == 0) return FA_OK;
  const bool has_mask = mask && numel(mask) > 0;
  return hip_status(fa::launch_bwd(to_dt(q->dtype), (int)q->shape[3], causal != 0, has_mask, p, (hipStream_t)stream));
}

fa_status fa_bwd_varlen(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_seqlens_q,
                        const fa_tensor* cu_seqlens_k, int max_seqlen_q, int max_seqlen_k, const fa_tensor* o,
                        const fa_tensor* o_lo, const fa_tensor* lse, const fa_tensor* dout, int causal, float scale,
                        const fa_tensor* delta, const fa_tensor* dq, const fa_tensor* dk, const fa_tensor* dv,
                        const fa_tensor* ds_workspace, void* stream) {
  clear_error();
  fa_status s;
  const char* names3[9] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv", nullptr};
  const fa_tensor* ts3[8] = {q, k, v, o, dout, dq, dk, dv};
  for (int t = 0; t < 8; ++t)
    if ((s = check_tensor(names3[t], ts3[t], 3, true)) != FA_OK) return s;
  if ((s = check_tensor("lse", lse, 2, false)) != FA_OK) return s;
  if ((s = check_tensor("delta", delta, 2, false)) != FA_OK) return s;
  if ((s = check_tensor("cu_seqlens_q", cu_seqlens_q, 1, false)) != FA_OK) return s;
  if ((s = check_tensor("cu_seqlens_k", cu_seqlens_k, 1, false)) != FA_OK) return s;
  if (q->dtype != FA_F16 && q->dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "q dtype must be f16 or bf16, got %s", dtype_name(q->dtype));
  for (int t = 1; t < 8; ++t)
    if ((s = check_dtype(names3[t], ts3[t], q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("lse", lse, FA_F32)) != FA_OK) return s;
  if ((s = check_dtype("delta", delta, FA_F32)) != FA_OK) return s;
  if ((s = check_dtype("cu_seqlens_q", cu_seqlens_q, FA_I32)) != FA_OK) return s;
  if ((s = check_dtype("cu_seqlens_k", cu_seqlens_k, FA_I32)) != FA_OK) return s;
  const int64_t Tq = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t Tk = k->shape[0], Hkv = k->shape[1], Dv = v->shape[2];
  const int64_t nb = cu_seqlens_q->shape[0];
  if (nb < 1 || cu_seqlens_k->shape[0] != nb)
    return fail(FA_ERR_SHAPE, "cu_seqlens_q and cu_seqlens_k must both have B + 1 >= 1 entries");
  if (k->shape[2] != D) return fail(FA_ERR_SHAPE, "k head dim differs from q's");
  if (v->shape[0] != Tk || v->shape[1] != Hkv) return fail(FA_ERR_SHAPE, "v must match k in rows and heads");
  for (int i = 0; i < 3; ++i) {
    const int64_t ow = i == 2 ? Dv : q->shape[i];
    if (o->shape[i] != ow || dout->shape[i] != ow) return fail(FA_ERR_SHAPE, "o and dout must be [Tq, Hq, Dv]");
    if (dq->shape[i] != q->shape[i]) return fail(FA_ERR_SHAPE, "dq must be shaped like q");
    if (dk->shape[i] != k->shape[i]) return fail(FA_ERR_SHAPE, "dk must be shaped like k");
    if (dv->shape[i] != v->shape[i]) return fail(FA_ERR_SHAPE, "dv must be shaped like v");
  }
  if (lse->shape[0] != Tq || lse->shape[1] != Hq) return fail(FA_ERR_SHAPE, "lse must be [Tq, Hq]");
  if (delta->shape[0] != Tq || delta->shape[1] != Hq) return fail(FA_ERR_SHAPE, "delta must be [Tq, Hq]");
  if ((s = check_contiguous("lse", lse)) != FA_OK) return s;
  if ((s = check_contiguous("delta", delta)) != FA_OK) return s;
  if ((s = check_o_lo(o_lo, o)) != FA_OK) return s;
  if (Hkv == 0 && Tq * Hq > 0) return fail(FA_ERR_SHAPE, "k has no heads");
  if (Hkv > 0 && Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (causal != 0 && causal != 1) return fail(FA_ERR_VALUE, "causal must be 0 or 1");
  if (max_seqlen_q < 0 || max_seqlen_k < 0) return fail(FA_ERR_VALUE, "max_seqlen_q and max_seqlen_k must be >= 0");
  if (!scale_ok(scale)) return fail(FA_ERR_VALUE, "scale must be finite and > 0");
  if (D != Dv) return fail(FA_ERR_UNSUPPORTED, "D (%lld) != Dv (%lld) is not supported", (long long)D, (long long)Dv);
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "the backward supports head dim 64 or 128 (got %lld)", (long long)D);
  if (!fits_i32(Tq) || !fits_i32(Tk) || !fits_i32(nb * Hq) || !fits_i32(Tq * Hq))
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  // Tiles are fetched with 32-bit per-lane offsets from the tile start.
  for (int t = 0; t < 5; ++t)
    if (ts3[t]->stride[0] > (1 << 22))
      return fail(FA_ERR_UNSUPPORTED, "%s row stride above 2^22 elements is not supported", names3[t]);
  const int64_t B = nb - 1;
  fa::BwdParams p;
  memset(&p, 0, sizeof(p));
  if ((s = check_ds_work(ds_workspace, q->dtype, B, Hq, max_seqlen_q, max_seqlen_k, causal != 0, p)) != FA_OK)
    return s;
  // (With keys but no query rows the kernels still run: dk and dv are zero.)
  if (B * Hq == 0 || ((int64_t)max_seqlen_q == 0 && (int64_t)max_seqlen_k == 0)) return FA_OK;
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.dout = dout->data;
  p.lse = (const float*)lse->data;
  p.delta = (float*)delta->data;
  p.dq = dq->data;
  p.dk = dk->data;
  p.dv = dv->data;
  int64_t* st[8][2] = {{&p.q_sh, &p.q_ss},   {&p.k_sh, &p.k_ss},   {&p.v_sh, &p.v_ss},   {&p.o_sh, &p.o_ss},
                       {&p.do_sh, &p.do_ss}, {&p.dq_sh, &p.dq_ss}, {&p.dk_sh, &p.dk_ss}, {&p.dv_sh, &p.dv_ss}};
  for (int t = 0; t < 8; ++t) {
    *st[t][0] = ts3[t]->stride[1];
    *st[t][1] = ts3[t]->stride[0];
  }
  if (o_lo && numel(o_lo) > 0) {
    p.o_lo = (const float*)o_lo->data;
    p.ol_sh = o_lo->stride[1];
    p.ol_ss = o_lo->stride[0];
  }
  p.B = (int32_t)B;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.G = (int32_t)(Hq / Hkv);
  p.Sq = max_seqlen_q;
  p.Skv = max_seqlen_k;
  p.Tq = (int32_t)Tq;
  p.Tk = (int32_t)Tk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.cu_q = (const int32_t*)cu_seqlens_q->data;
  p.cu_k = (const int32_t*)cu_seqlens_k->data;
  return hip_status(fa::launch_bwd_varlen(to_dt(q->dtype), (int)D, causal != 0, p, (hipStream_t)stream));
}

fa_status fa_fwd_varlen(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_seqlens_q,
                        const fa_tensor* cu_seqlens_k, int max_seqlen_q, int causal, float scale,
                        float rescale_threshold, const fa_tensor* o, const fa_tensor* lse, void* stream) {
  clear_error();
  fa_status s;
  if ((s = check_tensor("q", q, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("k", k, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("v", v, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("o", o, 3, true)) != FA_OK) return s;
  if ((s = check_tensor("lse", lse, 2, false)) != FA_OK) return s;
  if ((s = check_tensor("cu_seqlens_q", cu_seqlens_q, 1, false)) != FA_OK) return s;
  if ((s = check_tensor("cu_seqlens_k", cu_seqlens_k, 1, false)) != FA_OK) return s;
  if (q->dtype != FA_F16 && q->dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "q dtype must be f16 or bf16, got %s", dtype_name(q->dtype));
  if ((s = check_dtype("k", k, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("v", v, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("o", o, q->dtype)) != FA_OK) return s;
  if ((s = check_dtype("lse", lse, FA_F32)) != FA_OK) return s;
  if ((s = check_dtype("cu_seqlens_q", cu_seqlens_q, FA_I32)) != FA_OK) return s;
  if ((s = check_dtype("cu_seqlens_k", cu_seqlens_k, FA_I32)) != FA_OK) return s;
  const int64_t Tq = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t Tk = k->shape[0], Hkv = k->shape[1], Dv = v->shape[2];
  const int64_t nb = cu_seqlens_q->shape[0];
  if (nb < 1 || cu_seqlens_k->shape[0] != nb)
    return fail(FA_ERR_SHAPE, "cu_seqlens_q and cu_seqlens_k must both have B + 1 >= 1 entries");
  if (k->shape[2] != D) return fail(FA_ERR_SHAPE, "k head dim differs from q's");
  if (v->shape[0] != Tk || v->shape[1] != Hkv) return fail(FA_ERR_SHAPE, "v must match k in rows and heads");
  if (o->shape[0] != Tq || o->shape[1] != Hq || o->shape[2] != Dv) return fail(FA_ERR_SHAPE, "o must be [Tq, Hq, Dv]");
  if (lse->shape[0] != Tq || lse->shape[1] != Hq) return fail(FA_ERR_SHAPE, "lse must be [Tq, Hq]");
  if ((s = check_contiguous("lse", lse)) != FA_OK) return s;
  if (Hkv == 0 && Tq * Hq > 0) return fail(FA_ERR_SHAPE, "k has no heads");
  if (Hkv > 0 && Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (causal != 0 && causal != 1) return fail(FA_ERR_VALUE, "causal must be 0 or 1");
  if (max_seqlen_q < 0) return fail(FA_ERR_VALUE, "max_seqlen_q must be >= 0");
  if (!scale_ok(scale)) return fail(FA_ERR_VALUE, "scale must be finite and > 0");
  if (!(rescale_threshold >= 0.f && rescale_threshold <= kMaxRescaleThreshold))
    return fail(FA_ERR_VALUE, "rescale_threshold must be in [0, %g]", (double)kMaxRescaleThreshold);
  if (D != Dv) return fail(FA_ERR_UNSUPPORTED, "D (%lld) != Dv (%lld) is not supported", (long long)D, (long long)Dv);
  if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)D);
  if (!fits_i32(Tq) || !fits_i32(Tk) || !fits_i32(nb * Hq) || !fits_i32(Tq * Hq))
    return fail(FA_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
  if (k->stride[0] > (1 << 22) || v->stride[0] > (1 << 22))
    return fail(FA_ERR_UNSUPPORTED, "k/v row stride above 2^22 elements is not supported");
  const int64_t B = nb - 1;
  if (B * Hq * (int64_t)max_seqlen_q == 0 || Tq == 0) return FA_OK;
  fa::FwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.lse = (float*)lse->data;
  p.q_sh = q->stride[1]; p.q_ss = q->stride[0];
  p.k_sh = k->stride[1]; p.k_ss = k->stride[0];
  p.v_sh = v->stride[1]; p.v_ss = v->stride[0];
  p.o_sh = o->stride[1]; p.o_ss = o->stride[0];
  p.lse_sh = lse->stride[1]; p.lse_ss = lse->stride[0];
  p.B = (int32_t)B;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.G = (int32_t)(Hq / Hkv);
  p.Sq = max_seqlen_q;
  p.Skv = (int32_t)Tk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.rescale_thr = rescale_threshold;
  p.n_splits = 1;
  p.cu_q = (const int32_t*)cu_seqlens_q->data;
  p.cu_k = (const int32_t*)cu_seqlens_k->data;
  return hip_status(fa::launch_varlen(to_dt(q->dtype), (int)D, causal != 0, p, (hipStream_t)stream));
}

int fa_fwd_splitkv_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int num_splits) {
  return split_plan(B, Hq, Sq, Skv, num_splits, nullptr);
}

int64_t fa_bwd_ds_workspace_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  if (B < 0 || Hq < 0 || Sq < 0 || Skv < 0) return -1;
  return fa::bwd_ds_elems(B, Hq, Sq, Skv);
}

int64_t fa_fwd_splitkv_workspace_elems(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int64_t Dv, int num_splits) {
  const int ns = split_plan(B, Hq, Sq, Skv, num_splits, nullptr);
  if (ns < 0 || Dv < 0) return -1;
  return ns > 1 ? (int64_t)ns * B * Hq * Sq * (Dv + 1) : 0;
}

// Shared body of the split-KV entry points: the partial results go to the
// caller's workspace tensor, or with static_scratch to the library's static
// device scratch (looked up only once a split is actually needed).
static fa_status splitkv_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* seqlens_q,
                              const fa_tensor* seqlens_k, int causal, float scale, float rescale_threshold,
                              int num_splits, const fa_tensor* workspace, bool static_scratch, const fa_tensor* o,
                              const fa_tensor* lse, void* stream);

fa_status fa_fwd_splitkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* seqlens_q,
                         const fa_tensor* seqlens_k, int causal, float scale, float rescale_threshold, int num_splits,
                         const fa_tensor* workspace, const fa_tensor* o, const fa_tensor* lse, void* stream) {
  clear_error();
  return splitkv_impl(q, k, v, seqlens_q, seqlens_k, causal, scale, rescale_threshold, num_splits, workspace,
                      false, o, lse, stream);
}

fa_status fa_fwd_splitkv_noalloc(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                                 const fa_tensor* seqlens_q, const fa_tensor* seqlens_k, int causal, float scale,
                                 float rescale_threshold, int num_splits, const fa_tensor* o, const fa_tensor* lse,
                                 void* stream) {
  clear_error();
  return splitkv_impl(q, k, v, seqlens_q, seqlens_k, causal, scale, rescale_threshold, num_splits, nullptr, true, o,
                      lse, stream);
}

static fa_status splitkv_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* seqlens_q,
                              const fa_tensor* seqlens_k, int causal, float scale, float rescale_threshold,
                              int num_splits, const fa_tensor* workspace, bool static_scratch, const fa_tensor* o,
                              const fa_tensor* lse, void* stream) {
  fa_status s = check_bnsd(q, k, v, o, lse, scale, rescale_threshold);
  if (s != FA_OK) return s;
  if (q->dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the split-KV forward takes f16 or bf16");
  if (causal != 0 && causal != 1) return fail(FA_ERR_VALUE, "causal must be 0 or 1");
  if (num_splits < 0 || num_splits > kMaxSplits) return fail(FA_ERR_VALUE, "num_splits must be in [0, %d]", kMaxSplits);
  const int64_t B = q->shape[0], Hq = q->shape[1], Sq = q->shape[2], Skv = k->shape[2], Dv = v->shape[3];
  if ((s = check_seqlens("seqlens_q", seqlens_q, B)) != FA_OK) return s;
  if ((s = check_seqlens("seqlens_k", seqlens_k, B)) != FA_OK) return s;
  fa::FwdParams p;
  fill_common(p, q, k, v, o, lse, scale, rescale_threshold);
  p.seqlens_q = seqlens_q ? (const int32_t*)seqlens_q->data : nullptr;
  p.seqlens_k = seqlens_k ? (const int32_t*)seqlens_k->data : nullptr;
  int split_len = 0;
  const int ns = split_plan(B, Hq, Sq, Skv, num_splits, &split_len);
  if (B * Hq * Sq == 0) return FA_OK;
  if (ns <= 1)  // one key range: the plain forward, no workspace
    return hip_status(fa::launch_dense(to_dt(q->dtype), (int)q->shape[3], causal != 0, false, false, p,
                                       (hipStream_t)stream));
  const int64_t need = (int64_t)ns * B * Hq * Sq * (Dv + 1);
  float* ws = nullptr;
  if (!static_scratch) {
    if ((s = check_tensor("workspace", workspace, 1, true)) != FA_OK) return s;
    if ((s = check_dtype("workspace", workspace, FA_F32)) != FA_OK) return s;
    if (workspace->shape[0] < need)
      return fail(FA_ERR_SHAPE, "workspace holds %lld floats, %d key ranges need %lld", (long long)workspace->shape[0],
                  ns, (long long)need);
    ws = (float*)workspace->data;
  } else {
    if (need > fa::kScratchFloats)
      return fail(FA_ERR_UNSUPPORTED,
                  "%d key ranges of %lld rows need %lld floats of partial results; the static scratch holds %lld "
                  "(use fewer ranges or fa_fwd_splitkv with a workspace)",
                  ns, (long long)(B * Hq * Sq), (long long)need, (long long)fa::kScratchFloats);
    if ((s = hip_status(fa::scratch_address(&ws))) != FA_OK) return s;
  }
  if (!fits_i32((int64_t)ns * B * Hq * ((Sq + 255) / 256)))  // one workgroup per (range, 256 rows, head)
    return fail(FA_ERR_UNSUPPORTED, "too many workgroups");
  p.n_splits = ns;
  p.split_len = split_len;
  p.part_o = ws;
  p.part_lse = p.part_o + (int64_t)ns * B * Hq * Sq * Dv;
  return hip_status(fa::launch_splitkv(to_dt(q->dtype), (int)q->shape[3], causal != 0, p, (hipStream_t)stream));
}

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_STRIDE: return "FA_ERR_STRIDE";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_VALUE: return "FA_ERR_VALUE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
  }
}

const char* fa_last_error(void) { return g_err; }

int fa_version(void) { return 400; }

}  // extern "C"
