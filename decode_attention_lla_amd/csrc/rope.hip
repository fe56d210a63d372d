// Decoupled rotary branch of the absorbed read: rotary key writes and rotary score pre-pass.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 7 ("Per-head LLA
// versus LLA-2D at inference"): RoPE cannot be absorbed into the latent path, so attention splits,
// as in MLA, into the NoPE latent content path and a small explicit rotary branch, which a looped
// model shares across recurrence steps for a token. Here one rotary key of width d_r is cached per
// token (shared by heads and loops), already rotated at its slot position; the rotation is
// RoFormer's (Su et al., 2021): channel pairs (2i, 2i+1) at position p turn by p * base^(-2i/d_r).
// Angles, sines and cosines are evaluated in float64: at positions near 2^18 a float32 angle is
// off by ~1e-2 rad.
//
// The rotary score of token i for head h, q_r(b,h) . k_r(b,i) with q_r rotated at the decoding
// position N_b, depends on the head only through q_r, and k_r is shared by all heads: one pre-pass
// per read forms every head's rotary scores (already in the base-2 softmax scale) reading each
// rotary key once, and the streaming decode kernel adds them to the latent scores.
#include <hip/hip_runtime.h>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}

// Rotate the pair (x0, x1) of channel pair i at position pos (float64 angle and trigonometry).
__device__ __forceinline__ void rotate_pair(float x0, float x1, int i, int d, double pos,
                                            double base, float* y0, float* y1) {
  const double theta = pow(base, -2.0 * i / d);
  double s, c;
  sincos(pos * theta, &s, &c);
  *y0 = static_cast<float>(x0 * c - x1 * s);
  *y1 = static_cast<float>(x0 * s + x1 * c);
}

// k_rope[b][pos[b] + c][:] = rotate(k_in[b][c][:], pos[b] + c); one thread per channel pair.
__global__ __launch_bounds__(256) void rope_write_kernel(RopeWriteParams p) {
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const int half = p.d_r / 2;
  const long total = static_cast<long>(p.B) * p.C * half;
  if (idx >= total) return;
  const int i = static_cast<int>(idx % half);
  const long bc = idx / half;
  const int c = static_cast<int>(bc % p.C);
  const int b = static_cast<int>(bc / p.C);
  const int slot = p.pos[b] + c;
  if (slot < 0 || slot >= p.n_max) return;
  const uint16_t* x = static_cast<const uint16_t*>(p.k_in) + bc * p.d_r;
  float y0, y1;
  rotate_pair(bf16_at(x, 2 * i), bf16_at(x, 2 * i + 1), i, p.d_r, slot, p.base, &y0, &y1);
  uint32_t* out = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.k_rope) +
                                              (static_cast<size_t>(b) * p.n_max + slot) * p.d_r);
  out[i] = f32x2_to_bf16x2(y0, y1);
}

constexpr int kTokTile = 256;

// sr[b][h][i] = scale_log2 * rope(q_rope[b][h], N_b) . k_rope[b][i] for i < N_b; the workgroup of
// tile 0 also writes sr_self[b][h] = scale_log2 * q_rope[b][h] . k_rope_self[b] (rotating both at
// N_b leaves their dot product unchanged). One thread per token, every head; DR = d_r.
template <int DR>
__global__ __launch_bounds__(kTokTile) void rope_scores_kernel(RopeScoreParams p) {
  extern __shared__ float q_s[];  // [H][d_r] rotated rotary queries, times scale_log2
  const int b = blockIdx.y;
  int nb = p.seq_lens != nullptr ? p.seq_lens[b] : p.n_max;
  nb = min(max(nb, 0), p.n_max);
  const int tok0 = blockIdx.x * kTokTile;
  constexpr int half = DR / 2;
  const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + static_cast<size_t>(b) * p.H * DR;
  if (blockIdx.x == 0 && p.k_rope_self != nullptr) {
    const uint16_t* ks = static_cast<const uint16_t*>(p.k_rope_self) + static_cast<size_t>(b) * DR;
    for (int h = threadIdx.x; h < p.H; h += kTokTile) {
      float acc = 0.f;
      for (int j = 0; j < DR; ++j) acc += bf16_at(qr, static_cast<size_t>(h) * DR + j) * bf16_at(ks, j);
      p.sr_self[static_cast<size_t>(b) * p.H + h] = acc * p.scale_log2;
    }
  }
  if (tok0 >= nb) return;  // workgroup-uniform, before the barrier
  for (int idx = threadIdx.x; idx < p.H * half; idx += kTokTile) {
    const int h = idx / half;
    const int i = idx - h * half;
    float y0, y1;
    rotate_pair(bf16_at(qr, static_cast<size_t>(h) * DR + 2 * i),
                bf16_at(qr, static_cast<size_t>(h) * DR + 2 * i + 1), i, DR, nb, p.base, &y0, &y1);
    q_s[h * DR + 2 * i] = y0 * p.scale_log2;
    q_s[h * DR + 2 * i + 1] = y1 * p.scale_log2;
  }
  __syncthreads();
  const int tok = tok0 + threadIdx.x;
  if (tok >= nb) return;
  const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k_rope) +
                                                   (static_cast<size_t>(b) * p.n_max + tok) * DR);
  float k[DR];
#pragma unroll
  for (int cch = 0; cch < DR / 8; ++cch) {
    const uint4 w = kr[cch];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[8 * cch + 2 * e] = bf16_lo(ws[e]);
      k[8 * cch + 2 * e + 1] = bf16_hi(ws[e]);
    }
  }
  float* out = p.sr + static_cast<size_t>(b) * p.H * p.n_max + tok;
  for (int h = 0; h < p.H; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < DR; ++j) acc += q_s[h * DR + j] * k[j];
    out[static_cast<size_t>(h) * p.n_max] = acc;
  }
}

}  // namespace

hipError_t launch_rope_write(const RopeWriteParams& p, hipStream_t stream) {
  const long total = static_cast<long>(p.B) * p.C * (p.d_r / 2);
  hipLaunchKernelGGL(rope_write_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

hipError_t launch_rope_scores(const RopeScoreParams& p, hipStream_t stream) {
  const dim3 grid((p.n_max + kTokTile - 1) / kTokTile, p.B);
  const size_t lds = static_cast<size_t>(p.H) * p.d_r * sizeof(float);
  switch (p.d_r) {
    case 32: hipLaunchKernelGGL(rope_scores_kernel<32>, grid, dim3(kTokTile), lds, stream, p); break;
    case 64: hipLaunchKernelGGL(rope_scores_kernel<64>, grid, dim3(kTokTile), lds, stream, p); break;
    case 128: hipLaunchKernelGGL(rope_scores_kernel<128>, grid, dim3(kTokTile), lds, stream, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace lla
