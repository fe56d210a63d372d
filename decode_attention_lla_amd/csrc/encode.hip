// Latent encode: z = E (x - mu) for finished tokens, written into the cache.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456, Section 3: Eq. 1 stacks the
// T per-loop vectors of one (token, head, axis) loop-major, x = [x_1; ...; x_T]; Eq. 2 encodes
// c = (x - mu) W_down, i.e. z = E (x - mu) with E = W_down^T of shape [r][T*d] (column form).
// LLA-2D uses the same arithmetic on the whole (loop, head, channel) stack; the host maps it onto
// this kernel as one "head" of width H*d.
//
// The input x is [B][C][T][H][d]: for fixed (b, c, h) the stack is T runs of d contiguous values,
// H*d apart. One workgroup of 256 threads handles NTOK consecutive tokens (b, c) of one head: it
// stages x - mu for those tokens in LDS as float32, then each wave produces whole latent rows,
// reading E once per row for all NTOK tokens.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8192;  // T*d (per-head) or T*H*d (2D) upper bound for the LDS stage

// kNtok tokens share each pass over E; the stage holds kNtok*K floats (at most 32 KiB).
template <class S, int kNtok>
__global__ __launch_bounds__(kThreads) void encode_valu_kernel(EncodeParams p) {
  extern __shared__ float xs[];  // [kNtok][K]
  const int K = p.T * p.d;
  const int h = blockIdx.y;
  const int n0 = blockIdx.x * kNtok;  // first flattened token (b, c)
  const int ntok_total = p.B * p.C;
  const int tid = threadIdx.x;

  for (int i = tid; i < kNtok * K; i += kThreads) {
    const int nt = i / K;
    const int k = i - nt * K;
    const int n = n0 + nt;
    float v = 0.f;
    if (n < ntok_total) {
      const int t = k / p.d;
      const int j = k - t * p.d;
      // x[b][c][t][h][j] with (b, c) flattened as n
      const size_t xi = ((static_cast<size_t>(n) * p.T + t) * p.H + h) * p.d + j;
      v = ld<S>(p.x, xi);
      if (p.mu != nullptr) v -= ld<S>(p.mu, static_cast<size_t>(h) * K + k);
    }
    xs[i] = v;
  }
  __syncthreads();

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const size_t ebase = static_cast<size_t>(h) * p.r * K;
  for (int r = wave; r < p.r; r += kThreads / 64) {
    float acc[kNtok];
#pragma unroll
    for (int nt = 0; nt < kNtok; ++nt) acc[nt] = 0.f;
    const size_t erow = ebase + static_cast<size_t>(r) * K;
    for (int k = lane; k < K; k += 64) {
      const float e = ld<S>(p.E, erow + k);
#pragma unroll
      for (int nt = 0; nt < kNtok; ++nt) acc[nt] += e * xs[nt * K + k];
    }
#pragma unroll
    for (int nt = 0; nt < kNtok; ++nt) acc[nt] = wave_sum(acc[nt]);
    if (lane < kNtok) {
      const int n = n0 + lane;
      float mine = acc[0];
#pragma unroll
      for (int nt = 1; nt < kNtok; ++nt)
        if (lane == nt) mine = acc[nt];
      if (n < ntok_total) {
        const int b = n / p.C;
        const int c = n - b * p.C;
        const int slot = p.pos[b] + c;
        if (slot >= 0 && slot < p.n_max)
          st<S>(p.z, ((static_cast<size_t>(b) * p.H + h) * p.n_max + slot) * p.r + r, mine);
      }
    }
  }
}

}  // namespace

bool encode_supported(int dtype, int r) {
  return (dtype == LLA_F32 || dtype == LLA_BF16) && r >= 1 && r <= 512;
}

hipError_t launch_encode(const EncodeParams& p, int dtype, hipStream_t stream) {
  const int K = p.T * p.d;
  if (K > kMaxK) return hipErrorNotSupported;
  const unsigned ntok = static_cast<unsigned>(p.B) * p.C;
  const int nt = K <= 1024 ? 8 : K <= 2048 ? 4 : K <= 4096 ? 2 : 1;
  dim3 grid((ntok + nt - 1) / nt, p.H);
  const size_t lds = static_cast<size_t>(nt) * K * sizeof(float);
  void (*fn)(EncodeParams) = nullptr;
  if (dtype == LLA_BF16)
    fn = nt == 8 ? encode_valu_kernel<BF16, 8> : nt == 4 ? encode_valu_kernel<BF16, 4>
       : nt == 2 ? encode_valu_kernel<BF16, 2> : encode_valu_kernel<BF16, 1>;
  else
    fn = nt == 8 ? encode_valu_kernel<F32, 8> : nt == 4 ? encode_valu_kernel<F32, 4>
       : nt == 2 ? encode_valu_kernel<F32, 2> : encode_valu_kernel<F32, 1>;
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace lla
