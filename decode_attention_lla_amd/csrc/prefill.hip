// Chunked-prefill attention over the latent cache.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Appendix A ("Decoding and
// caching") describes the latent-store decoder's prefill as two passes: the chunk's per-loop K/V
// are captured and encoded first, and attention then runs against the cache. Here the chunk's
// latents are already in slots ctx .. ctx+C-1, and chunk row j (position ctx + j) attends latents
// 0 .. ctx + j. The arithmetic per row is the absorbed decode of Section 7.
//
// Streaming path: every (row, head) is one query row of the absorbed split-K decode kernels, with
// its own causal key count. Rows of one sequence re-read the same latents, which mostly hit in
// cache for modest chunks.
#include "lla_internal.h"

namespace lla {

bool prefill_supported(int variant, int dtype, int r_k, int r_v) {
  return valu_supported(variant, dtype, r_k, r_v);
}

void prefill_plan(const lla_desc& desc, int B, int C, int* splits, int* chunk) {
  valu_plan(desc, B * C, splits, chunk);
}

size_t prefill_workspace_bytes(const lla_desc& desc, int B, int C) {
  int s, c;
  prefill_plan(desc, B, C, &s, &c);
  return valu_workspace_bytes(desc, B * C, s);
}

hipError_t launch_prefill(const PrefillParams& pp, int dtype, hipStream_t stream) {
  DecodeParams p{};
  p.q = pp.q;
  p.zk = pp.zk;
  p.zv = pp.zv;
  p.seq_lens = pp.ctx_lens;
  p.Wk = pp.Wk;
  p.Wv = pp.Wv;
  p.mu_k = pp.mu_k;
  p.mu_v = pp.mu_v;
  p.out = pp.out;
  p.ws = static_cast<float*>(pp.ws);
  p.B = pp.B * pp.C;
  p.H = pp.H;
  p.d = pp.d;
  p.T = pp.T;
  p.t = pp.t;
  p.n_max = pp.n_max;
  p.r_k = pp.r_k;
  p.r_v = pp.r_v;
  p.rows_per_seq = pp.C;
  p.causal = 1;
  p.variant = pp.variant;
  p.scale_log2 = pp.scale_log2;
  p.splits = pp.splits;  // planned by the caller with prefill_plan
  p.chunk = pp.chunk;
  p.ws_bytes = pp.ws_bytes;
  return launch_decode(p, dtype, stream);
}

}  // namespace lla
