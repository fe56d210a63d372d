// Latent encode: z = E (x - mu) for finished tokens, written into the cache.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456, Section 3: Eq. 1 stacks the
// T per-loop vectors of one (token, head, axis) loop-major, x = [x_1; ...; x_T]; Eq. 2 encodes
// c = (x - mu) W_down, i.e. z = E (x - mu) with E = W_down^T of shape [r][T*d] (column form).
// LLA-2D uses the same arithmetic on the whole (loop, head, channel) stack; the host maps it onto
// this kernel as one "head" of width H*d.
//
// The input x is [B][C][T][H][d]: for fixed (b, c, h) the stack is T runs of d contiguous values,
// H*d apart.
//
// bf16 storage: a GEMM per head on MFMA, Z^T[token][r] = X[token][k] . E[r][k]^T with
// v_mfma_f32_16x16x32_bf16. Both operands are read straight from memory as 16-byte runs along k
// (a run of 8 never straddles two loops because d_head is a multiple of 8). A wave owns 32 tokens x
// 16*NT latent rows. For small token counts (decode) the four waves of a workgroup split K and
// reduce through LDS; for large ones (prefill chunks) they take four token tiles. E mu is computed
// by the same MFMA (mu as the only non-zero row of an A tile) and subtracted from the float32
// accumulators, so x - mu is never rounded.
//
// fp32 storage: one 256-thread workgroup handles NTOK tokens of one head: x - mu for those tokens
// is staged in LDS as float32 and each wave produces whole latent rows.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// NT: 16-column latent tiles per wave; MT: 16-token tiles per wave. KSPLIT 1: each of the 4 waves
// owns its own 16*MT tokens over the whole K; KSPLIT 4 or 8: that many waves share 16*MT tokens
// and split K, reducing through LDS (KSPLIT 8 runs 8-wave workgroups).
template <int NT, int MT, int KSPLIT>
__global__ __launch_bounds__(KSPLIT == 8 ? 512 : 256) void encode_mfma_kernel(EncodeParams p) {
  constexpr int U = 4;  // k-steps whose loads are issued together
  constexpr int NW = KSPLIT == 8 ? 8 : 4;  // waves per workgroup
  constexpr int TOK_WG = KSPLIT == 1 ? NW * 16 * MT : 16 * MT;
  constexpr int NACC = MT * NT * 4;
  __shared__ float red[KSPLIT == 1 ? 1 : KSPLIT - 1][64][NACC];
  __shared__ float emu_s[NW][16 * NT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int K = p.T * p.d;
  const int nk = (K + 31) / 32;
  const int ntok = p.B * p.C;
  const int h = blockIdx.z;
  const int r0 = blockIdx.y * 16 * NT;
  const int n_base = blockIdx.x * TOK_WG + (KSPLIT == 1 ? wave * 16 * MT : 0);
  const size_t HD = static_cast<size_t>(p.H) * p.d;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* E = static_cast<const uint16_t*>(p.E);

  // E mu for this lane's latent rows, summed over the waves' shares of K
  float emu[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) emu[nt] = 0.f;
  if (p.mu != nullptr) {
    const uint16_t* mu = static_cast<const uint16_t*>(p.mu) + static_cast<size_t>(h) * K;
    const int qw = (nk + NW - 1) / NW;
    floatx4_t am[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) am[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int ks = wave * qw; ks < min(nk, (wave + 1) * qw); ++ks) {
      const int kk = 32 * ks + 8 * g;
      const uint4 a = (col == 0 && kk < K) ? *reinterpret_cast<const uint4*>(mu + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = r0 + 16 * nt + col;
        const uint4 b = (r < p.r && kk < K) ? *reinterpret_cast<const uint4*>(E + (static_cast<size_t>(h) * p.r + r) * K + kk)
                                           : make_uint4(0, 0, 0, 0);
        am[nt] = mfma(a, b, am[nt]);
      }
    }
    if (g == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) emu_s[wave][16 * nt + col] = am[nt][0];  // row 0 of C
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      for (int w = 0; w < NW; ++w) emu[nt] += emu_s[w][16 * nt + col];
  }

  // token rows of the MT A tiles, latent rows of the NT B tiles
  const uint16_t* xrow[MT];
  bool nok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int n = n_base + 16 * mt + col;
    nok[mt] = n < ntok;
    xrow[mt] = x + static_cast<size_t>(nok[mt] ? n : 0) * p.T * HD + static_cast<size_t>(h) * p.d;
  }
  const uint16_t* erow[NT];
  bool rok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + col;
    rok[nt] = r < p.r;
    erow[nt] = E + (static_cast<size_t>(h) * p.r + (rok[nt] ? r : 0)) * K;
  }

  int kb = 0, ke = nk;
  if (KSPLIT > 1) {
    const int qs = (nk + KSPLIT - 1) / KSPLIT;
    kb = min(nk, wave * qs);
    ke = min(nk, kb + qs);
  }
  floatx4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int ks = kb; ks < ke; ks += U) {
    uint4 a[U][MT];
    uint4 b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = 32 * (ks + u) + 8 * g;
      const bool kok = (ks + u) < ke && kk < K;
      const int t = kok ? kk / p.d : 0;
      const int j = kk - t * p.d;
      const size_t xo = static_cast<size_t>(t) * HD + j;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[u][mt] = (kok && nok[mt]) ? *reinterpret_cast<const uint4*>(xrow[mt] + xo) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[u][nt] = (kok && rok[nt]) ? *reinterpret_cast<const uint4*>(erow[nt] + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma(a[u][mt], b[u][nt], acc[mt][nt]);
  }

  if (KSPLIT > 1) {
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[wave - 1][lane][(mt * NT + nt) * 4 + e] = acc[mt][nt][e];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mt][nt][e] += red[w][lane][(mt * NT + nt) * 4 + e];
  }

  // C layout: lane holds latent row r = r0 + 16 nt + col for tokens n_base + 16 mt + 4 g + e
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = n_base + 16 * mt + 4 * g + e;
      if (n >= ntok) continue;
      const int b = n / p.C;
      const int c = n - b * p.C;
      const int slot = p.pos[b] + c;
      if (slot < 0 || slot >= p.n_max) continue;
      uint16_t* z = static_cast<uint16_t*>(p.z) + ((static_cast<size_t>(b) * p.H + h) * p.n_max + slot) * p.r;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (rok[nt]) z[r0 + 16 * nt + col] = f32_to_bf16(acc[mt][nt][e] - emu[nt]);
    }
}

template <int MT, int KSPLIT>
hipError_t launch_encode_mfma(const EncodeParams& p, int nt_tiles, hipStream_t stream) {
  constexpr int NW = KSPLIT == 8 ? 8 : 4;
  constexpr int TOK_WG = KSPLIT == 1 ? NW * 16 * MT : 16 * MT;
  const unsigned ntok = static_cast<unsigned>(p.B) * p.C;
  dim3 grid((ntok + TOK_WG - 1) / TOK_WG, (p.r + 16 * nt_tiles - 1) / (16 * nt_tiles), p.H);
  dim3 block(64 * NW);
  if (nt_tiles == 1)
    hipLaunchKernelGGL((encode_mfma_kernel<1, MT, KSPLIT>), grid, block, 0, stream, p);
  else if (nt_tiles == 2)
    hipLaunchKernelGGL((encode_mfma_kernel<2, MT, KSPLIT>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((encode_mfma_kernel<4, MT, KSPLIT>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool encode_supported(int dtype, int r) {
  return (dtype == LLA_F32 || dtype == LLA_BF16) && r >= 1 && r <= 512;
}

hipError_t launch_encode(const EncodeParams& p, int dtype, hipStream_t stream) {
  const int K = p.T * p.d;
  if (dtype == LLA_BF16) {
    const int nt_tiles = p.r <= 16 ? 1 : p.r <= 32 ? 2 : 4;
    const long ntok = static_cast<long>(p.B) * p.C;
    const long wgs1 = (ntok + 127) / 128 * ((p.r + 16 * nt_tiles - 1) / (16 * nt_tiles)) * p.H;
    // few workgroups with whole-K waves would leave most of the chip idle: split K instead,
    // eight ways for decode-size token counts
    if (ntok <= 256) return launch_encode_mfma<1, 8>(p, nt_tiles, stream);
    return wgs1 < 1024 ? launch_encode_mfma<2, 4>(p, nt_tiles, stream)
                       : launch_encode_mfma<2, 1>(p, nt_tiles, stream);
  }
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
