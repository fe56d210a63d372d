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
// per read forms every head's rotary scores (already in the base-2 softmax scale) on MFMA, reading
// each rotary key once, and the streaming decode kernel adds them to the latent scores.
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

constexpr int kTokTile = 256;  // tokens per workgroup: 4 waves x 4 blocks of 16

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// sr[b][h][i] = scale_log2 * rope(q_rope[b][h], N_b) . k_rope[b][i] for i < N_b, on MFMA: per
// 16-token block, S (16 heads x 16 tokens) = Q_r (16 heads x d_r, A operand) . K_rope^T (d_r x
// 16 tokens, B operand straight from HBM, 16 bytes per lane along the key); each store then writes
// 16 consecutive tokens of a head's score row. The rotated, scaled queries
// are split into two bf16 parts (hi + lo) accumulated into the same result, so the queries keep
// ~16 mantissa bits. The workgroup of tile 0 also writes sr_self[b][h] = scale_log2 *
// q_rope[b][h] . k_rope_self[b] (rotating both at N_b leaves their dot product unchanged).
template <int DR>
__global__ __launch_bounds__(kTokTile) void rope_scores_kernel(RopeScoreParams p) {
  extern __shared__ float q_s[];  // [H][DR] rotated rotary queries times scale_log2
  constexpr int half = DR / 2;
  constexpr int KS = DR / 32;
  const int tiles = (p.n_max + kTokTile - 1) / kTokTile;  // one-dimensional grid: b * tiles + tile
  const int b = blockIdx.x / tiles;
  const int tile = blockIdx.x - b * tiles;
  int nb = p.seq_lens != nullptr ? uniform(p.seq_lens[b]) : p.n_max;
  nb = min(max(nb, 0), p.n_max);
  const int tok0 = tile * kTokTile;
  const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + static_cast<size_t>(b) * p.H * DR;
  if (tile == 0 && p.k_rope_self != nullptr) {
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

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k_rope) + static_cast<size_t>(b) * p.n_max * DR;
  float* sbase = p.sr + static_cast<size_t>(b) * p.H * p.sr_stride;
  for (int hg = 0; hg < p.H; hg += 16) {
    // A operand: lane (head hg + col, group g) holds q_r[head][32 ks + 8 g .. + 7], hi and lo
    uint4 qh[KS], ql[KS];
    const int head = hg + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int j = 32 * ks + 8 * g + 2 * e2;
        const float v0 = head < p.H ? q_s[head * DR + j] : 0.f;
        const float v1 = head < p.H ? q_s[head * DR + j + 1] : 0.f;
        hw[e2] = f32x2_to_bf16x2(v0, v1);
        lw[e2] = f32x2_to_bf16x2(v0 - bf16_lo(hw[e2]), v1 - bf16_hi(hw[e2]));
      }
      qh[ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      ql[ks] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    // every block's key operands are loaded before any is used (tokens past N_b read as zeros)
    constexpr int NB = kTokTile / 64;  // 16-token blocks per wave
    uint4 kb[NB][KS];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int row = tok0 + (4 * wave + blk) * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[blk][ks] = row < nb ? *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(row) * DR + 32 * ks + 8 * g)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int row = tok0 + (4 * wave + blk) * 16 + col;  // B operand column (token) of this lane
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = mfma16(qh[ks], kb[blk][ks], acc);
        acc = mfma16(ql[ks], kb[blk][ks], acc);
      }
      // C: lane (token row, group g) holds heads hg + 4 g + e
      if (row < nb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int hh = hg + 4 * g + e;
          // non-temporal: the scores are read once, by the next kernel; left dirty in the caches
          // they cost that read ~3% more
          if (hh < p.H) __builtin_nontemporal_store(acc[e], &sbase[static_cast<size_t>(hh) * p.sr_stride + row]);
        }
      }
    }
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
  const int64_t blocks = static_cast<int64_t>((p.n_max + kTokTile - 1) / kTokTile) * p.B;
  if (blocks >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const dim3 grid(static_cast<unsigned>(blocks));
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
