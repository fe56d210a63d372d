// Host-side interface between the C ABI (abi.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lla.h"

namespace lla {

// One decode read at loop t (lla_attend_decode after validation).
struct DecodeParams {
  const void* q;
  const void* zk;
  const void* zv;
  const int32_t* seq_lens;
  const void* Wk;
  const void* Wv;
  const void* mu_k;
  const void* mu_v;
  const void* k_self;
  const void* v_self;
  void* out;
  float* lse;
  float* ws;          // split partials [B][H][S][2 + r_v] (m, l, a[r_v]); unused when S == 1
  int32_t B, H, d, T, t, n_max, r_k, r_v;
  // Query rows: B rows per call; row i reads latent sequence i / rows_per_seq. For decode
  // rows_per_seq = 1 and the key count is seq_lens[seq]. For prefill (causal = 1) row i is chunk
  // row j = i % rows_per_seq and sees seq_lens[seq] + j + 1 latents. Counts clamp to [0, n_max].
  int32_t rows_per_seq;
  int32_t causal;
  int32_t variant;    // LLA_PER_HEAD or LLA_2D
  int32_t splits;     // S: token-range splits per (b, h), from decode_plan / prefill_plan
  int32_t chunk;      // tokens per split
  // Waves of one workgroup that share a (row, head, split): each takes chunk / wg_waves of the
  // split's tokens and the partials merge in LDS (streaming kernels; 0 or 1: one wave).
  int32_t wg_waves;
  // Rotary read (streaming): heads of one row per workgroup (0 or 1: one; else the compiled head
  // group), which share each batch's rotary rows through LDS. Excludes wg_waves > 1.
  int32_t wg_heads;
  float scale_log2;   // softmax scale * log2(e)
  size_t ws_bytes;    // bytes available at ws; launchers refuse a plan that does not fit
  // Gather-indexed read (lla_attend_decode_gather): row b attends the latents at
  // slots[b * budget + j], j < seq_lens[b] clamped to [0, budget] (all budget when seq_lens is
  // null); a slot outside [0, n_max) is skipped. slots == nullptr: the contiguous read above.
  const int32_t* slots;
  int32_t budget;
  // Decoupled rotary branch (lla_attend_decode_rope; d_rope == 0 without), formed inside the read
  // (streaming and LLA-2D MFMA kernels alike): q_rope [rows][H][d_rope] unrotated (rotated at the
  // row's key count N_b), k_rope [B][n_max][d_rope] rotated at each slot, k_rope_self [B][d_rope]
  // or NULL, RoFormer base.
  const void* q_rope;
  const void* k_rope;
  const void* k_rope_self;
  int32_t d_rope;
  double rope_base;
};

struct EncodeParams {
  const void* x;      // [B][C][T][H][d]
  const void* E;      // per-head [H][r][T*d]; 2D as per-head with H=1, d=H*d
  const void* mu;     // per-head [H][T*d] or NULL
  const int32_t* pos; // [B]
  void* z;            // [B][H][n_max][r]
  int32_t B, C, H, d, T, r, n_max;
};

// Rotary key write (lla_rope_write): k_rope[b][pos[b]+c] = rope(k_in[b][c], pos[b]+c).
struct RopeWriteParams {
  const void* k_in;    // bf16 [B][C][d_r]
  const int32_t* pos;  // [B]
  void* k_rope;        // bf16 [B][n_max][d_r]
  int32_t B, C, n_max, d_r;
  double base;
};

// Rebuild of one axis's loop-t K or V for the reconstruct-then-attend comparator (per head).
struct ReconParams {
  const void* z;       // bf16 latents [B][H][n_max][r]
  const void* W;       // bf16 [T][H][d][r]
  const void* mu;      // bf16 [H][T*d] or NULL
  const int32_t* seq_lens;
  void* x;             // bf16 out [B][H][n_max][d], rows < N_b written
  int32_t H, T, t, n_max, r;
};

// Quantisation of bf16 latent rows into a low-bit cache (lla_quantize_latents, one axis).
struct QuantParams {
  const void* src;     // bf16 [B][H][C][r] (LLA-2D: H = 1)
  void* dst;           // low-bit cache [B][H][n_max][Q8::row(r)] bytes
  const int32_t* pos;  // [B]
  int32_t B, C, H, r, n_max;
  bool int8;           // LLA_BF16_I8 codes (else LLA_BF16_Q8)
};

struct PrefillParams {
  const void* q;      // [B][C][H][d]
  const void* zk;
  const void* zv;
  const int32_t* ctx_lens;
  const void* Wk;
  const void* Wv;
  const void* mu_k;
  const void* mu_v;
  void* out;          // [B][C][H][d]
  void* ws;
  int32_t B, C, H, d, T, t, n_max, r_k, r_v, variant;
  int32_t splits, chunk;  // from prefill_plan
  int32_t wg_waves;       // streaming path: waves per (row, head, split), from prefill_plan
  float scale_log2;
  size_t ws_bytes;
  // Rotary branch (lla_attend_prefill_rope; d_rope == 0 without it): q_rope [B][C][H][d_rope]
  // unrotated, k_rope [B][n_max][d_rope] rotated at each slot, RoFormer base.
  const void* q_rope;
  const void* k_rope;
  int32_t d_rope;
  double rope_base;
};

// Token-split plan of one lla_attend_decode call. The C ABI computes it once per call, sizes the
// workspace from it and hands it to the launchers, which never re-plan.
// wg_waves (optional): waves per workgroup of the streaming kernels; without it the plan uses one.
void decode_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves = nullptr);
void valu_plan(const lla_desc& desc, int rows, int* splits, int* chunk, int* wg_waves = nullptr);
void prefill_plan(const lla_desc& desc, int B, int C, int* splits, int* chunk, int* wg_waves = nullptr);
// Workspace of one lla_attend_decode call under decode_plan.
size_t decode_workspace_bytes(const lla_desc& desc, int B);
// Workspace of the streaming decode kernels for `rows` query rows and a given split count.
size_t valu_workspace_bytes(const lla_desc& desc, int rows, int splits);
bool valu_supported(int variant, int dtype, int r_k, int r_v);
bool decode_uses_mfma2d(const lla_desc& desc);
// LLA-2D MFMA decode (decode2d.hip).
bool decode2d_mfma_supported(int dtype, int r_k, int r_v, int d_head);
void decode2d_plan(const lla_desc& desc, int B, int* splits, int* chunk);
// Workspace of the LLA-2D MFMA read; d_rope > 0 for the fused rotary branch.
size_t decode2d_workspace_bytes(const lla_desc& desc, int B, int splits, int d_rope = 0);
// dtype LLA_BF16, or LLA_BF16_Q8 / LLA_BF16_I8 rows (no rotary branch with those)
hipError_t launch_decode2d(const DecodeParams& p, int dtype, hipStream_t s);
size_t prefill_workspace_bytes(const lla_desc& desc, int B, int C);

// Launchers: return hipSuccess, or hipErrorNotSupported when no kernel is compiled for the
// requested (dtype, r_k, r_v); other errors come from the HIP launch.
hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s);
// Gather-indexed decode (streaming kernels, both variants): plan, workspace and launch.
void gather_plan(const lla_desc& desc, int B, int budget, int* splits, int* chunk);
size_t gather_workspace_bytes(const lla_desc& desc, int B, int budget);
hipError_t launch_decode_gather(const DecodeParams& p, int dtype, hipStream_t s);
hipError_t launch_encode(const EncodeParams& p, int dtype, hipStream_t s);
// both axes of one encode call (one launch where their plans match)
hipError_t launch_encode_kv(const EncodeParams& pk, const EncodeParams& pv, int dtype, hipStream_t s);
hipError_t launch_quantize(const QuantParams& pk, const QuantParams& pv, hipStream_t stream);
// Decoupled rotary branch (rope.hip, decode.hip).
hipError_t launch_rope_write(const RopeWriteParams& p, hipStream_t s);
bool rope_supported(const lla_desc& desc, int d_rope);
// The streaming read has instances with the rotary branch for (dtype, r_k, r_v) and d_rope.
bool rope_valu_supported(int dtype, int r_k, int r_v, int d_rope);
// Plan of one lla_attend_decode_rope call (decode_plan, or head groups for the streaming read).
void rope_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves, int* wg_heads);
size_t rope_workspace_bytes(const lla_desc& desc, int B);
hipError_t launch_decode_rope(const DecodeParams& p, int dtype, hipStream_t s);
// Reconstruct-then-attend comparator (reconstruct.hip).
bool reconstruct_supported(const lla_desc& desc);
void reconstruct_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves = nullptr);
size_t reconstruct_workspace_bytes(const lla_desc& desc, int B);
hipError_t launch_decode_reconstruct(const DecodeParams& p, const lla_desc& desc, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int dtype, hipStream_t s);

bool decode_supported(int variant, int dtype, int r_k, int r_v, int d_head);
bool encode_supported(int dtype, int r);
bool prefill_supported(int variant, int dtype, int r_k, int r_v);
bool prefill_rope_supported(const lla_desc& desc, int d_rope);

}  // namespace lla
