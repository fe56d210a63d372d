// Decoupled rotary branch of the absorbed read: rotary key writes.
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
// position N_b, is formed inside the decode reads (decode.hip: the streaming read dots each
// token's rotary key in the token's lane group; decode2d.hip: extra MFMA k-steps of the LLA-2D
// read); this file holds the rotary key writes.
#include <hip/hip_runtime.h>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
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

}  // namespace

hipError_t launch_rope_write(const RopeWriteParams& p, hipStream_t stream) {
  const long total = static_cast<long>(p.B) * p.C * (p.d_r / 2);
  hipLaunchKernelGGL(rope_write_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace lla
