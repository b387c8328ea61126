// Reference attention forward (and the gradients of the dense forward) in
// fp64 on the CPU.
//
// TEST INFRASTRUCTURE ONLY. This file is the oracle that the GPU path is
// checked against. It shares no code with the GPU library: no header, no
// helper, no table. Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load it.
//
// Every entry point computes, for each requested output row r, exactly the
// textbook definition of attention restricted to the row's key set K_r:
//
//   s_j  = scale * sum_d q_d * k_{j,d}                (j in K_r)
//   m    = max_j s_j                                   (stable softmax)
//   e_j  = exp(s_j - m),  l = sum_j e_j
//   O_r  = (sum_j e_j * v_j) / l,   LSE_r = m + ln l
//
// and O_r = 0, LSE_r = -inf when K_r is empty.
//
// Sources (titles of the pages this follows):
//   * "FlashAttention correctness verification" page: the standard attention
//     S = QK^T/sqrt(d), P = softmax(S), O = PV and its max-subtracted stable
//     softmax (section on standard vs. tiled attention, and the reference
//     implementation in the verifier class).
//   * Ascend FlashAttentionScore README: attention formula with a scale and a
//     boolean atten_mask where 1 excludes a position (formula and parameter
//     table).
//   * ops-transformer FlashAttentionScoreGrad pytest page, section 5.1: GQA as
//     a [B, Nkv, G, S, D] layout whose K/V group dimension is broadcast, i.e.
//     kv_head = q_head / G.
//   * PyPTO BSA README, sections 1 and 3: per-Q-block lists of KV blocks,
//     invalid slots contribute nothing, per-batch actual_seq_lengths mask the
//     tails and padded rows are zero.
//   * flash-attention SM100 sparse-MLA page, background section: each row
//     attends only to the W keys named by gather_kv_indices.
//
// All sums over keys run in ascending key index, whatever order the caller
// listed them in, so the result does not depend on the order of an index
// list. Duplicate valid indices are a precondition violation and are
// rejected (returned as an error) rather than given a meaning.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <thread>
#include <vector>

namespace {

enum OracleStatus : int {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = -1,        // null pointer or negative size
  ORACLE_ERR_INDEX = -2,      // index outside [0, S) / [0, nKB)
  ORACLE_ERR_DUPLICATE = -3,  // the same key (block) listed twice in one row
};

// One output row: softmax-weighted average of the value rows in `keys`.
// `keys` must be sorted ascending. k(j) / v(j) return row j of K / V.
template <class KRow, class VRow>
void attend_row(const double* q, int64_t D, int64_t Dv, const std::vector<int64_t>& keys,
                KRow k, VRow v, double scale, double* o, double* lse) {
  if (keys.empty()) {
    for (int64_t d = 0; d < Dv; ++d) o[d] = 0.0;
    *lse = -std::numeric_limits<double>::infinity();
    return;
  }
  std::vector<double> s(keys.size());
  for (size_t n = 0; n < keys.size(); ++n) {
    const double* kj = k(keys[n]);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * kj[d];
    s[n] = scale * dot;
  }
  double m = -std::numeric_limits<double>::infinity();
  for (double x : s) m = std::max(m, x);
  double l = 0.0;
  std::vector<double> acc(Dv, 0.0);
  for (size_t n = 0; n < keys.size(); ++n) {
    const double e = std::exp(s[n] - m);
    l += e;
    const double* vj = v(keys[n]);
    for (int64_t d = 0; d < Dv; ++d) acc[d] += e * vj[d];
  }
  for (int64_t d = 0; d < Dv; ++d) o[d] = acc[d] / l;
  *lse = m + std::log(l);
}

// Runs fn(r) for r in [0, n) on `nthreads` threads (0 = all hardware threads).
// fn returns an OracleStatus; the first non-OK status wins.
template <class Fn>
int parallel_rows(int64_t n, int nthreads, Fn fn) {
  if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
  nthreads = (int)std::min<int64_t>(nthreads, std::max<int64_t>(n, 1));
  std::vector<int> status(nthreads, ORACLE_OK);
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t) {
    pool.emplace_back([&, t] {
      for (int64_t r = t; r < n; r += nthreads) {
        int st = fn(r);
        if (st != ORACLE_OK) { status[t] = st; return; }
      }
    });
  }
  for (auto& th : pool) th.join();
  for (int st : status) if (st != ORACLE_OK) return st;
  return ORACLE_OK;
}

}  // namespace

extern "C" {

// Dense attention with optional causal mask, boolean mask, GQA and per-batch
// sequence lengths.
//
// q_rows  [nrows, D]: the query vector of each requested row.
// row_ids [nrows]   : flattened (b, hq, i) = (b * Hq + hq) * Sq + i.
// k [B, Hkv, Skv, D], v [B, Hkv, Skv, Dv]: contiguous.
// mask: nullable uint8; element (b, hq, i, j) at
//   mask[b*ms[0] + hq*ms[1] + i*ms[2] + j*ms[3]]; non-zero = excluded.
// seqlens_q / seqlens_k: nullable int32 [B]; rows i >= Lq_b have no keys,
//   keys j >= Lk_b are excluded. Without them Lq_b = Sq and Lk_b = Skv.
// causal: key j is excluded when j > i + (Lk_b - Lq_b) (bottom-right aligned).
// o [nrows, Dv], lse [nrows].
int oracle_attn_dense(const double* q_rows, const int64_t* row_ids, int64_t nrows,
                      const double* k, const double* v, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t Sq, int64_t Skv, int64_t D, int64_t Dv, const uint8_t* mask,
                      const int64_t* ms, const int32_t* seqlens_q, const int32_t* seqlens_k,
                      int causal, double scale, double* o, double* lse, int nthreads) {
  if (nrows < 0 || B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0)
    return ORACLE_ERR_ARG;
  if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
  if (nrows > 0 && (!q_rows || !row_ids || !o || !lse)) return ORACLE_ERR_ARG;
  if (mask && !ms) return ORACLE_ERR_ARG;
  const int64_t G = Hq / Hkv;
  return parallel_rows(nrows, nthreads, [&](int64_t r) -> int {
    const int64_t id = row_ids[r];
    if (id < 0 || id >= B * Hq * Sq) return ORACLE_ERR_INDEX;
    const int64_t i = id % Sq, bh = id / Sq, hq = bh % Hq, b = bh / Hq;
    const int64_t hkv = hq / G;
    const int64_t Lq = seqlens_q ? seqlens_q[b] : Sq;
    const int64_t Lk = seqlens_k ? seqlens_k[b] : Skv;
    std::vector<int64_t> keys;
    if (i < Lq) {
      for (int64_t j = 0; j < std::min(Lk, Skv); ++j) {
        if (causal && j > i + (Lk - Lq)) continue;
        if (mask && mask[b * ms[0] + hq * ms[1] + i * ms[2] + j * ms[3]] != 0) continue;
        keys.push_back(j);
      }
    }
    const double* kb = k + (b * Hkv + hkv) * Skv * D;
    const double* vb = v + (b * Hkv + hkv) * Skv * Dv;
    attend_row(q_rows + r * D, D, Dv, keys, [&](int64_t j) { return kb + j * D; },
               [&](int64_t j) { return vb + j * Dv; }, scale, o + r * Dv, lse + r);
    return ORACLE_OK;
  });
}

// Gradients of dense attention (same key sets as oracle_attn_dense) with
// respect to q, k and v, given the gradient dO of the output. Written out from
// the definitions, as on the ops-transformer FlashAttentionScoreGrad pytest
// page (section 5.2, the backward golden) and the PyPTO BSA README (section 1:
// dV carries no scale, dQ and dK carry scaleValue; GQA sums dK and dV over the
// query heads of a KV head):
//
//   P_ij  = exp(s_ij - LSE_i) over the row's key set (s = scale q.k)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
//   dQ_i  = scale sum_j dS_ij k_j,     dK_j = scale sum_i dS_ij q_i
//
// q [B,Hq,Sq,D], dout [B,Hq,Sq,Dv], k [B,Hkv,Skv,D], v [B,Hkv,Skv,Dv],
// dq like q, dk like k, dv like v: contiguous fp64. Rows with an empty key set
// contribute nothing. Runs one (b, kv head) per thread, so the dK / dV sums
// have one writer each.
int oracle_attn_dense_bwd(const double* q, const double* k, const double* v, const double* dout,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                          int64_t Dv, const uint8_t* mask, const int64_t* ms,
                          const int32_t* seqlens_q, const int32_t* seqlens_k, int causal,
                          double scale, double* dq, double* dk, double* dv, int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0) return ORACLE_ERR_ARG;
  if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
  if (B * Hq * Sq > 0 && (!q || !dout || !dq)) return ORACLE_ERR_ARG;
  if (B * Hkv * Skv > 0 && (!k || !v || !dk || !dv)) return ORACLE_ERR_ARG;
  if (mask && !ms) return ORACLE_ERR_ARG;
  const int64_t G = Hq / Hkv;
  return parallel_rows(B * Hkv, nthreads, [&](int64_t bk) -> int {
    const int64_t b = bk / Hkv, hkv = bk % Hkv;
    const double* kb = k + bk * Skv * D;
    const double* vb = v + bk * Skv * Dv;
    double* dkb = dk + bk * Skv * D;
    double* dvb = dv + bk * Skv * Dv;
    for (int64_t x = 0; x < Skv * D; ++x) dkb[x] = 0.0;
    for (int64_t x = 0; x < Skv * Dv; ++x) dvb[x] = 0.0;
    const int64_t Lq = seqlens_q ? seqlens_q[b] : Sq;
    const int64_t Lk = seqlens_k ? seqlens_k[b] : Skv;
    std::vector<int64_t> keys;
    std::vector<double> s, p, dp;
    for (int64_t hq = hkv * G; hq < (hkv + 1) * G; ++hq) {
      for (int64_t i = 0; i < Sq; ++i) {
        const int64_t row = (b * Hq + hq) * Sq + i;
        const double* qi = q + row * D;
        const double* doi = dout + row * Dv;
        double* dqi = dq + row * D;
        for (int64_t d = 0; d < D; ++d) dqi[d] = 0.0;
        keys.clear();
        if (i < Lq) {
          for (int64_t j = 0; j < std::min(Lk, Skv); ++j) {
            if (causal && j > i + (Lk - Lq)) continue;
            if (mask && mask[b * ms[0] + hq * ms[1] + i * ms[2] + j * ms[3]] != 0) continue;
            keys.push_back(j);
          }
        }
        if (keys.empty()) continue;
        const size_t n = keys.size();
        s.assign(n, 0.0);
        p.assign(n, 0.0);
        dp.assign(n, 0.0);
        double m = -std::numeric_limits<double>::infinity();
        for (size_t t = 0; t < n; ++t) {
          const double* kj = kb + keys[t] * D;
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d) dot += qi[d] * kj[d];
          s[t] = scale * dot;
          m = std::max(m, s[t]);
        }
        double l = 0.0;
        for (size_t t = 0; t < n; ++t) l += std::exp(s[t] - m);
        double delta = 0.0;  // sum_j P_ij dP_ij
        for (size_t t = 0; t < n; ++t) {
          p[t] = std::exp(s[t] - m) / l;
          const double* vj = vb + keys[t] * Dv;
          double dot = 0.0;
          for (int64_t d = 0; d < Dv; ++d) dot += doi[d] * vj[d];
          dp[t] = dot;
          delta += p[t] * dot;
        }
        for (size_t t = 0; t < n; ++t) {
          const int64_t j = keys[t];
          const double ds = p[t] * (dp[t] - delta);
          const double* kj = kb + j * D;
          for (int64_t d = 0; d < D; ++d) dqi[d] += scale * ds * kj[d];
          for (int64_t d = 0; d < D; ++d) dkb[j * D + d] += scale * ds * qi[d];
          for (int64_t d = 0; d < Dv; ++d) dvb[j * Dv + d] += p[t] * doi[d];
        }
      }
    }
    return ORACLE_OK;
  });
}

// First-order error scales of the gradients above, for per-element
// tolerances: the same key sets and the same P and dS, but every signed sum
// replaced by the sum of the magnitudes of its terms, plus the effect of an
// error in Delta_i = sum_j P_ij dP_ij of at most 2 E_i with
// E_i = sum_d |dO_id| sum_j P_ij |v_jd| (a gradient pipeline that forms
// Delta from a computed O whose error is bounded by the magnitudes of the
// terms of P V):
//
//   gv_j = sum_i P_ij |dO_i|
//   gk_j = scale sum_i (|dS_ij| + 2 P_ij E_i) |q_i|
//   gq_i = scale sum_j (|dS_ij| + 2 P_ij E_i) |k_j|
//
// (elementwise over d). If each rounded quantity carries a relative error of
// at most u, the error of dV, dK, dQ is at most u times these (to first
// order). Same argument conventions as oracle_attn_dense_bwd; outputs
// gq, gk, gv shaped like dq, dk, dv.
int oracle_attn_dense_bwd_bound(const double* q, const double* k, const double* v, const double* dout,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                int64_t Dv, const uint8_t* mask, const int64_t* ms,
                                const int32_t* seqlens_q, const int32_t* seqlens_k, int causal,
                                double scale, double* gq, double* gk, double* gv, int nthreads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0) return ORACLE_ERR_ARG;
  if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
  if (B * Hq * Sq > 0 && (!q || !dout || !gq)) return ORACLE_ERR_ARG;
  if (B * Hkv * Skv > 0 && (!k || !v || !gk || !gv)) return ORACLE_ERR_ARG;
  if (mask && !ms) return ORACLE_ERR_ARG;
  const int64_t G = Hq / Hkv;
  return parallel_rows(B * Hkv, nthreads, [&](int64_t bk) -> int {
    const int64_t b = bk / Hkv, hkv = bk % Hkv;
    const double* kb = k + bk * Skv * D;
    const double* vb = v + bk * Skv * Dv;
    double* gkb = gk + bk * Skv * D;
    double* gvb = gv + bk * Skv * Dv;
    for (int64_t x = 0; x < Skv * D; ++x) gkb[x] = 0.0;
    for (int64_t x = 0; x < Skv * Dv; ++x) gvb[x] = 0.0;
    const int64_t Lq = seqlens_q ? seqlens_q[b] : Sq;
    const int64_t Lk = seqlens_k ? seqlens_k[b] : Skv;
    std::vector<int64_t> keys;
    std::vector<double> s, p, dp, pv(Dv);
    for (int64_t hq = hkv * G; hq < (hkv + 1) * G; ++hq) {
      for (int64_t i = 0; i < Sq; ++i) {
        const int64_t row = (b * Hq + hq) * Sq + i;
        const double* qi = q + row * D;
        const double* doi = dout + row * Dv;
        double* gqi = gq + row * D;
        for (int64_t d = 0; d < D; ++d) gqi[d] = 0.0;
        keys.clear();
        if (i < Lq) {
          for (int64_t j = 0; j < std::min(Lk, Skv); ++j) {
            if (causal && j > i + (Lk - Lq)) continue;
            if (mask && mask[b * ms[0] + hq * ms[1] + i * ms[2] + j * ms[3]] != 0) continue;
            keys.push_back(j);
          }
        }
        if (keys.empty()) continue;
        const size_t n = keys.size();
        s.assign(n, 0.0);
        p.assign(n, 0.0);
        dp.assign(n, 0.0);
        double m = -std::numeric_limits<double>::infinity();
        for (size_t t = 0; t < n; ++t) {
          const double* kj = kb + keys[t] * D;
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d) dot += qi[d] * kj[d];
          s[t] = scale * dot;
          m = std::max(m, s[t]);
        }
        double l = 0.0;
        for (size_t t = 0; t < n; ++t) l += std::exp(s[t] - m);
        double delta = 0.0;
        for (int64_t d = 0; d < Dv; ++d) pv[d] = 0.0;
        for (size_t t = 0; t < n; ++t) {
          p[t] = std::exp(s[t] - m) / l;
          const double* vj = vb + keys[t] * Dv;
          double dot = 0.0;
          for (int64_t d = 0; d < Dv; ++d) {
            dot += doi[d] * vj[d];
            pv[d] += p[t] * std::fabs(vj[d]);
          }
          dp[t] = dot;
          delta += p[t] * dot;
        }
        double e = 0.0;  // E_i
        for (int64_t d = 0; d < Dv; ++d) e += std::fabs(doi[d]) * pv[d];
        for (size_t t = 0; t < n; ++t) {
          const int64_t j = keys[t];
          const double w = std::fabs(p[t] * (dp[t] - delta)) + 2.0 * p[t] * e;
          const double* kj = kb + j * D;
          for (int64_t d = 0; d < D; ++d) gqi[d] += scale * w * std::fabs(kj[d]);
          for (int64_t d = 0; d < D; ++d) gkb[j * D + d] += scale * w * std::fabs(qi[d]);
          for (int64_t d = 0; d < Dv; ++d) gvb[j * Dv + d] += p[t] * std::fabs(doi[d]);
        }
      }
    }
    return ORACLE_OK;
  });
}

// Block-sparse attention: row i of query block qb = i / block_q attends to the
// union of the KV blocks [block_k * idx, block_k * idx + block_k) listed in its
// block list, cut at the batch's sequence length.
//
// block_idx: int32, element (b, hkv, qb, s) at
//   block_idx[b*bs[0] + hkv*bs[1] + qb*bs[2] + s*bs[3]], s in [0, max_sel);
//   negative = unused slot (anywhere in the list).
// seqlens: nullable int32 [B]; applies to both queries and keys: rows i >= L_b
//   have no keys, keys j >= L_b are excluded.
int oracle_attn_blocksparse(const double* q_rows, const int64_t* row_ids, int64_t nrows,
                            const double* k, const double* v, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int64_t Dv,
                            const int32_t* block_idx, const int64_t* bs, int64_t max_sel,
                            int64_t block_q, int64_t block_k, const int32_t* seqlens,
                            double scale, double* o, double* lse, int nthreads) {
  if (nrows < 0 || B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0 ||
      max_sel < 0 || block_q <= 0 || block_k <= 0)
    return ORACLE_ERR_ARG;
  if (Hq % Hkv != 0) return ORACLE_ERR_ARG;
  if (nrows > 0 && (!q_rows || !row_ids || !o || !lse || !bs || (max_sel > 0 && !block_idx)))
    return ORACLE_ERR_ARG;
  const int64_t G = Hq / Hkv;
  const int64_t nkb = (Skv + block_k - 1) / block_k;
  return parallel_rows(nrows, nthreads, [&](int64_t r) -> int {
    const int64_t id = row_ids[r];
    if (id < 0 || id >= B * Hq * Sq) return ORACLE_ERR_INDEX;
    const int64_t i = id % Sq, bh = id / Sq, hq = bh % Hq, b = bh / Hq;
    const int64_t hkv = hq / G;
    const int64_t Lq = seqlens ? std::min<int64_t>(seqlens[b], Sq) : Sq;
    const int64_t Lk = seqlens ? std::min<int64_t>(seqlens[b], Skv) : Skv;
    const int64_t qb = i / block_q;
    std::vector<int64_t> blocks;
    for (int64_t s = 0; s < max_sel; ++s) {
      const int64_t x = block_idx[b * bs[0] + hkv * bs[1] + qb * bs[2] + s * bs[3]];
      if (x < 0) continue;
      if (x >= nkb) return ORACLE_ERR_INDEX;
      blocks.push_back(x);
    }
    std::sort(blocks.begin(), blocks.end());
    if (std::adjacent_find(blocks.begin(), blocks.end()) != blocks.end())
      return ORACLE_ERR_DUPLICATE;
    std::vector<int64_t> keys;
    if (i < Lq) {
      for (int64_t x : blocks)
        for (int64_t j = x * block_k; j < std::min((x + 1) * block_k, Lk); ++j) keys.push_back(j);
    }
    const double* kb = k + (b * Hkv + hkv) * Skv * D;
    const double* vb = v + (b * Hkv + hkv) * Skv * Dv;
    attend_row(q_rows + r * D, D, Dv, keys, [&](int64_t j) { return kb + j * D; },
               [&](int64_t j) { return vb + j * Dv; }, scale, o + r * Dv, lse + r);
    return ORACLE_OK;
  });
}

// Top-k gathered attention with one shared KV head: row (t, h) attends to the
// keys idx[t, 0..W) that are >= 0.
//
// q_rows [nrows, Dqk]; row_ids[r] = t * Hq + h.
// k [S, Dqk], v [S, Dv]: contiguous. idx [T, W] int32: contiguous.
int oracle_attn_topk(const double* q_rows, const int64_t* row_ids, int64_t nrows,
                     const double* k, const double* v, int64_t T, int64_t Hq, int64_t S,
                     int64_t Dqk, int64_t Dv, const int32_t* idx, int64_t W, double scale,
                     double* o, double* lse, int nthreads) {
  if (nrows < 0 || T < 0 || Hq <= 0 || S < 0 || Dqk <= 0 || Dv <= 0 || W < 0)
    return ORACLE_ERR_ARG;
  if (nrows > 0 && (!q_rows || !row_ids || !o || !lse || (W > 0 && !idx)))
    return ORACLE_ERR_ARG;
  return parallel_rows(nrows, nthreads, [&](int64_t r) -> int {
    const int64_t id = row_ids[r];
    if (id < 0 || id >= T * Hq) return ORACLE_ERR_INDEX;
    const int64_t t = id / Hq;
    std::vector<int64_t> keys;
    for (int64_t s = 0; s < W; ++s) {
      const int64_t j = idx[t * W + s];
      if (j < 0) continue;
      if (j >= S) return ORACLE_ERR_INDEX;
      keys.push_back(j);
    }
    std::sort(keys.begin(), keys.end());
    if (std::adjacent_find(keys.begin(), keys.end()) != keys.end()) return ORACLE_ERR_DUPLICATE;
    attend_row(q_rows + r * Dqk, Dqk, Dv, keys, [&](int64_t j) { return k + j * Dqk; },
               [&](int64_t j) { return v + j * Dv; }, scale, o + r * Dv, lse + r);
    return ORACLE_OK;
  });
}

int oracle_hardware_threads(void) { return (int)std::thread::hardware_concurrency(); }

}  // extern "C"
