// Internal interface between the C-ABI layer (fa_abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

// Parameters of the dense / block-sparse forward kernels. All strides are in
// elements. Shapes are already validated by the host layer.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* o_lo;             // nullable, fp32 like o: O - rounded(O)
  float* lse;              // [B, Hq, Sq] contiguous
  const uint8_t* mask;     // nullable; element (b, hq, i, j) at b*m_sb + hq*m_sh + i*m_ss + j
  const int32_t* seqlens_q;  // nullable [B]
  const int32_t* seqlens_k;  // nullable [B]
  const int32_t* block_idx;  // block-sparse only: (b, hkv, qb, slot) at b*bi_sb + hkv*bi_sh + qb*bi_sq + slot
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t ol_sb, ol_sh, ol_ss;
  int64_t m_sb, m_sh, m_ss;
  int64_t bi_sb, bi_sh, bi_sq;
  int32_t B, Hq, Hkv, G, Sq, Skv;
  int32_t max_sel;         // block-sparse slots per query block
  int32_t mask_vec4;       // 1: mask rows may be read 4 bytes at a time
  int32_t mask_vec16;      // 1: ... and 16 bytes at a time
  int32_t mask_lds;        // 1: ... and mask tiles may be copied to LDS in 16-byte chunks
  int32_t n_mblocks;       // query blocks per head
  int32_t n_hgroups;       // head groups per KV head (G / heads per workgroup)
  float scale;             // softmax scale (LSE is reported in these units)
  float scale_log2;        // scale * log2(e): scores enter exp2 through one FMA
  float rescale_thr;       // running-max rescale threshold, log2 units (0 = exact)
  // LSE element (b, hq, i) at lse[b * lse_sb + hq * lse_sh + i * lse_ss].
  int64_t lse_sb, lse_sh, lse_ss;
  // Packed variable-length (TND) layout: the query rows of batch b are rows
  // cu_q[b] .. cu_q[b+1]-1 of q, o and lse (Sq is the longest of them), its
  // keys rows cu_k[b] .. cu_k[b+1]-1 of k and v; the batch strides are 0.
  const int32_t* cu_q;
  const int32_t* cu_k;
  // Split-KV: the keys of a row block are cut into n_splits ranges of
  // split_len keys; each workgroup writes its range's normalised fp32 output
  // and LSE to part_o [n_splits, B*Hq*Sq, Dv] and part_lse [n_splits, B*Hq*Sq]
  // for the merge kernel.
  int32_t n_splits, split_len;
  float* part_o;
  float* part_lse;
};

// Inputs of the split-KV merge: the partial results above into O and LSE.
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;  // [B, Hq, Sq] contiguous
  int64_t o_sb, o_sh, o_ss;
  int32_t B, Hq, Sq, Dv, n_splits;
};

// Top-k gathered MLA forward parameters.
struct TopkParams {
  const void* q;     // [T, Hq, Dqk]
  const void* k;     // [S, Dqk]
  const void* v;     // [S, Dv]
  void* o;           // [T, Hq, Dv]
  float* o_lo;       // nullable [T, Hq, Dv] fp32: O - rounded(O)
  float* lse;        // [T, Hq]
  const int32_t* idx;  // [T, W]
  int64_t q_st, q_sh;
  int64_t k_ss, v_ss;
  int64_t o_st, o_sh;
  int64_t ol_st, ol_sh;
  int64_t idx_st;
  int32_t T, Hq, S, W;
  uint32_t k_bytes, v_bytes;  // bytes spanned by k and v
  int32_t n_htiles;  // head tiles per token
  float scale;
  float scale_log2;
};

// Kernel `name` of the run-time loaded code object (the 16-bit dense,
// block-sparse and top-k kernels) on the current device (loaded on first use).
hipError_t code_object_function(const char* name, hipFunction_t* fn);

// Launchers: enqueue on `stream`, return the HIP status of the launch.
hipError_t launch_dense(Dt dt, int D, bool causal, bool has_mask, bool sparse,
                        FwdParams& p, hipStream_t stream);
// Packed variable-length forward (p.cu_q / p.cu_k set; 16-bit, no mask).
hipError_t launch_varlen(Dt dt, int D, bool causal, FwdParams& p, hipStream_t stream);
// Split-KV forward (p.n_splits > 1, p.split_len, p.part_o / p.part_lse set)
// followed by the merge into p.o / p.lse.
hipError_t launch_splitkv(Dt dt, int D, bool causal, FwdParams& p, hipStream_t stream);
// The merge alone (fa_split.hip).
hipError_t launch_merge(Dt dt, const MergeParams& m, hipStream_t stream);

// Static device scratch of the allocation-free split-KV entry point (a
// file-scope array in fa_split.hip): 64 MiB of fp32 per GPU.
constexpr int64_t kScratchFloats = (int64_t)16 << 20;
constexpr int kMaxDevices = 64;
// Device address of the current device's copy of the scratch array (looked
// up once per device, with that device current).
hipError_t scratch_address(float** ptr);
hipError_t launch_topk(Dt dt, TopkParams& p, hipStream_t stream);

}  // namespace fa
