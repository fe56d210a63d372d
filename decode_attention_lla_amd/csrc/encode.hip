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

// The parameters of one axis: the second (pv) for workgroups in the upper half of a two-axis grid.
// Field by field, so each stays a scalar.
__device__ __forceinline__ EncodeParams pick_axis(const EncodeParams& pk, const EncodeParams& pv, bool v) {
  EncodeParams p;
  p.x = v ? pv.x : pk.x;
  p.E = v ? pv.E : pk.E;
  p.mu = v ? pv.mu : pk.mu;
  p.pos = v ? pv.pos : pk.pos;
  p.z = v ? pv.z : pk.z;
  p.B = v ? pv.B : pk.B;
  p.C = v ? pv.C : pk.C;
  p.H = v ? pv.H : pk.H;
  p.d = v ? pv.d : pk.d;
  p.T = v ? pv.T : pk.T;
  p.r = v ? pv.r : pk.r;
  p.n_max = v ? pv.n_max : pk.n_max;
  return p;
}

// NT: 16-column latent tiles per wave; MT: 16-token tiles per wave. KSPLIT 1: each of the 4 waves
// owns its own 16*MT tokens over the whole K; KSPLIT 4 or 8: that many waves share 16*MT tokens
// and split K, reducing through LDS (KSPLIT 8 runs 8-wave workgroups). Grid y is the latent tiles
// of one axis (ytiles of them), or of both axes when the K and V encodes share a launch (pk's in
// the lower half, pv's in the upper half): a dependent launch costs a few microseconds on its own,
// as much as a decode-size encode's work.
template <int NT, int MT, int KSPLIT>
__global__ __launch_bounds__(KSPLIT == 8 ? 512 : 256) void encode_mfma_kernel(EncodeParams pk, EncodeParams pv,
                                                                            int ytiles) {
  const bool second = static_cast<int>(blockIdx.y) >= ytiles;
  const EncodeParams p = pick_axis(pk, pv, second);
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
  const int r0 = (static_cast<int>(blockIdx.y) - (second ? ytiles : 0)) * 16 * NT;
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

// pv: the second axis sharing the launch (same shape and rank as p), or null for p alone
template <int MT, int KSPLIT>
hipError_t launch_encode_mfma(const EncodeParams& p, const EncodeParams* pv, int nt_tiles, hipStream_t stream) {
  constexpr int NW = KSPLIT == 8 ? 8 : 4;
  constexpr int TOK_WG = KSPLIT == 1 ? NW * 16 * MT : 16 * MT;
  const unsigned ntok = static_cast<unsigned>(p.B) * p.C;
  const int ytiles = (p.r + 16 * nt_tiles - 1) / (16 * nt_tiles);
  dim3 grid((ntok + TOK_WG - 1) / TOK_WG, ytiles * (pv != nullptr ? 2 : 1), p.H);
  dim3 block(64 * NW);
  const EncodeParams& q = pv != nullptr ? *pv : p;
  if (nt_tiles == 1)
    hipLaunchKernelGGL((encode_mfma_kernel<1, MT, KSPLIT>), grid, block, 0, stream, p, q, ytiles);
  else if (nt_tiles == 2)
    hipLaunchKernelGGL((encode_mfma_kernel<2, MT, KSPLIT>), grid, block, 0, stream, p, q, ytiles);
  else
    hipLaunchKernelGGL((encode_mfma_kernel<4, MT, KSPLIT>), grid, block, 0, stream, p, q, ytiles);
  return hipGetLastError();
}

// ---- LDS-tiled GEMM for large token counts -----------------------------------------------------
// Z^T[token][r] = X[token][k] . E[r][k]^T as one dense product per head: a workgroup of 8 waves owns
// 256 tokens x TN latent rows and walks k in steps of 32. The X tile (256 x 32) and the E tile
// (TN x 32) of a step go straight from memory to LDS with global_load_lds into a 4-deep ring of
// named stages (one __shared__ object each, so the compiler tells the stage being read from those
// being filled). Tiles are stored as 64-byte rows whose 16-byte chunks are XOR-swizzled by
// (row / 4) mod 4: the MFMA operand reads (ds_read_b128, 16 rows x one chunk per 16 lanes) then
// touch every LDS bank once. Waves form a 4 x 2 grid of 64 x TN/2 tiles on
// v_mfma_f32_32x32x16_bf16 (A[i][k] at lane i + 32 (k / 8), element k % 8; B[k][j] likewise;
// C[i][j] at lane j + 32 ((i / 4) % 2), element 4 (i / 8) + i % 4). A 32-wide k chunk stays inside
// one loop t when d is a multiple of 32, so each lane's 16 bytes are contiguous in x.
constexpr int kGM = 256;     // tokens per workgroup
constexpr int kGK = 32;      // k per stage
constexpr int kGStages = 4;  // ring depth

template <int N>
struct GStage {
  static constexpr int value = N;
};

typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__device__ __forceinline__ floatx16_t mfma3232(uint4 a, uint4 b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int gswz(int row, int c) { return c ^ ((row >> 2) & 3); }

template <int TN>
__global__ __launch_bounds__(512) void encode_gemm_kernel(EncodeParams p) {
  constexpr int WN = TN / 2;           // latent rows per wave
  constexpr int MT = 2;                // 32-token tiles per wave (64 tokens)
  constexpr int NT = WN / 32;          // 32-row latent tiles per wave
  constexpr int A_BYTES = kGM * kGK * 2;
  constexpr int B_BYTES = TN * kGK * 2;
  constexpr int IA = A_BYTES / 1024;   // 1 KiB load instructions per stage
  constexpr int IB = B_BYTES / 1024;
  static_assert(IA % 8 == 0 && (IB % 8 == 0 || IB == 8), "loads spread evenly over 8 waves");
  constexpr int LA = IA / 8;
  constexpr int LB = IB / 8;
  constexpr int LPW = LA + LB;         // loads per wave and stage
  static_assert(2 * LPW < 16, "vmcnt encoding below");
  __shared__ __attribute__((aligned(16))) char a0[A_BYTES], a1[A_BYTES], a2[A_BYTES], a3[A_BYTES];
  __shared__ __attribute__((aligned(16))) char b0[B_BYTES], b1[B_BYTES], b2[B_BYTES], b3[B_BYTES];
  __shared__ float emu_s[TN];
  __shared__ int2 tok_s[kGM];  // (sequence, cache slot) of each token row; slot -1: not written
  auto astage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return a0; else if constexpr (st == 1) return a1;
    else if constexpr (st == 2) return a2; else return a3;
  };
  auto bstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return b0; else if constexpr (st == 1) return b1;
    else if constexpr (st == 2) return b2; else return b3;
  };

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave & 3;
  const int wn = wave >> 2;
  const int h = blockIdx.z;
  const int r0 = blockIdx.y * TN;
  const int n0 = blockIdx.x * kGM;
  const int ntok = p.B * p.C;
  const int K = p.T * p.d;
  const int nst = K / kGK;  // stages, a multiple of kGStages
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* E = static_cast<const uint16_t*>(p.E) + static_cast<size_t>(h) * p.r * K;

  if (tid < kGM) {
    const int n = n0 + tid;
    int2 ts = make_int2(0, -1);
    if (n < ntok) {
      const int b = n / p.C;
      const int slot = p.pos[b] + (n - b * p.C);
      if (slot >= 0 && slot < p.n_max) ts = make_int2(b, slot);
    }
    tok_s[tid] = ts;
  }
  // E mu for this workgroup's latent rows (only with centering): 16-row groups on
  // v_mfma_f32_16x16x32_bf16 with mu as row 0 of the A operand
  if (p.mu != nullptr) {
    const uint16_t* mu = static_cast<const uint16_t*>(p.mu) + static_cast<size_t>(h) * K;
    const int col = lane & 15;
    const int g = lane >> 4;
    for (int grp = wave; grp < TN / 16; grp += 8) {
      const int er = min(r0 + 16 * grp + col, p.r - 1);
      const uint16_t* erow = E + static_cast<size_t>(er) * K;
      // the loads of 8 steps are issued before their products (K is a multiple of 128 here), so
      // the walk over E's rows is not one memory round trip per step
      floatx4_t am = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < K; k += 32 * 8) {
        uint4 a[8], bb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kk = min(k + 32 * u, K - 32);
          a[u] = col == 0 ? *reinterpret_cast<const uint4*>(mu + kk + 8 * g) : make_uint4(0, 0, 0, 0);
          bb[u] = *reinterpret_cast<const uint4*>(erow + kk + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k + 32 * u < K) am = mfma(a[u], bb[u], am);
      }
      if (g == 0) emu_s[16 * grp + col] = am[0];  // row 0 of C: lane j, element 0
    }
  } else {
    for (int i = tid; i < TN; i += 512) emu_s[i] = 0.f;
  }
  __syncthreads();

  // Loads of stage `s` (k0 = s * kGK, clamped to the last stage for the spare fetches past the
  // end). Each lane's byte offset inside the workgroup's X rows and E rows never changes; the step
  // only moves the wave-uniform base. Keeping the per-lane offsets fixed keeps their registers from
  // being rewritten while a transfer that reads them may still be in flight (the compiler would
  // wait for every outstanding load before such a rewrite).
  const char* xw = reinterpret_cast<const char*>(x) +
                   (static_cast<size_t>(n0) * p.T * p.H + h) * p.d * 2;   // token n0, head h, k = 0
  const char* ew = reinterpret_cast<const char*>(E) + static_cast<size_t>(r0) * K * 2;
  uint32_t aoff[LA], boff[LB];
#pragma unroll
  for (int u = 0; u < LA; ++u) {
    const int unit = (wave + 8 * u) * 64 + lane;
    const int row = unit >> 2;
    const int n = min(n0 + row, ntok - 1) - n0;  // rows past the last token re-read it
    aoff[u] = (static_cast<uint32_t>(n) * p.T * p.H * p.d + 8 * gswz(row, unit & 3)) * 2;
  }
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    const int i = IB >= 8 ? wave + 8 * u : wave % IB;
    const int unit = i * 64 + lane;
    const int row = unit >> 2;
    const int er = min(r0 + row, p.r - 1) - r0;
    boff[u] = (static_cast<uint32_t>(er) * K + 8 * gswz(row, unit & 3)) * 2;
  }
  // the lane offset goes in voffset and the step's k offset in soffset, so the address registers
  // are never rewritten
  auto issue = [&](int s, char* ad, char* bd) {
    const int k0 = min(s, nst - 1) * kGK;
    const int t = k0 / p.d;
    const int j0 = k0 - t * p.d;
    const int xso = (t * p.H * p.d + j0) * 2;
    const int eso = k0 * 2;
#pragma unroll
    for (int u = 0; u < LA; ++u)
      buffer_lds16(xw, 0x7fffffff, (lptr_t)(ad + (wave + 8 * u) * 1024), aoff[u], xso);
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int i = IB >= 8 ? wave + 8 * u : wave % IB;
      buffer_lds16(ew, 0x7fffffff, (lptr_t)(bd + i * 1024), boff[u], eso);
    }
  };

  floatx16_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;

  // one stage: wait for this wave's loads of stage s (two stages may stay in flight) and for the
  // other waves, refill the stage computed last, then 2 k-steps of MT x NT MFMAs
  auto step = [&](auto S, int s) {
    constexpr int st = decltype(S)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * LPW));  // vmcnt(2 * LPW)
    lds_barrier();  // (lla_device.h) not a full fence: later stages stay in flight
    issue(s + 3, astage(GStage<(st + 3) % kGStages>{}), bstage(GStage<(st + 3) % kGStages>{}));
    const char* at = astage(S);
    const char* bt = bstage(S);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      uint4 av[MT], bv[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 64 * wm + 32 * mt + (lane & 31);
        av[mt] = *reinterpret_cast<const uint4*>(at + opaque(row * 64 + gswz(row, c) * 16));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int row = WN * wn + 32 * nt + (lane & 31);
        bv[nt] = *reinterpret_cast<const uint4*>(bt + opaque(row * 64 + gswz(row, c) * 16));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma3232(av[mt], bv[nt], acc[mt][nt]);
    }
  };

  issue(0, a0, b0);
  issue(1, a1, b1);
  issue(2, a2, b2);
  for (int s = 0; s < nst; s += kGStages) {
    step(GStage<0>{}, s);
    step(GStage<1>{}, s + 1);
    step(GStage<2>{}, s + 2);
    step(GStage<3>{}, s + 3);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // the spare fetches have landed before the wave ends

  // C layout: lane (j + 32 hh) element e holds token row 8 (e / 4) + 4 hh + e % 4, latent row j
  const int hh = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int2 ts = tok_s[64 * wm + 32 * mt + 8 * (e >> 2) + 4 * hh + (e & 3)];
      if (ts.y < 0) continue;
      uint16_t* z = static_cast<uint16_t*>(p.z) + ((static_cast<size_t>(ts.x) * p.H + h) * p.n_max + ts.y) * p.r;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int rl = WN * wn + 32 * nt + (lane & 31);
        if (r0 + rl < p.r) z[r0 + rl] = f32_to_bf16(acc[mt][nt][e] - emu_s[rl]);
      }
    }
}

template <int TN>
hipError_t launch_encode_gemm(const EncodeParams& p, hipStream_t stream) {
  const unsigned ntok = static_cast<unsigned>(p.B) * p.C;
  dim3 grid((ntok + kGM - 1) / kGM, (p.r + TN - 1) / TN, p.H);
  hipLaunchKernelGGL(encode_gemm_kernel<TN>, grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

// the tiled GEMM applies when a 32-wide k chunk stays inside one loop, the k extent is whole
// groups of four stages, the latent rank fills 128-row tiles and there are enough tokens
bool encode_gemm_ok(const EncodeParams& p) {
  const long ntok = static_cast<long>(p.B) * p.C;
  // byte offsets inside a workgroup's rows must fit the 31-bit buffer range
  const long stack = static_cast<long>(p.T) * p.H * p.d * 2;
  const long xspan = kGM * stack;
  const long espan = 256L * p.T * p.d * 2;
  return p.d % kGK == 0 && (p.T * p.d) % (kGK * kGStages) == 0 && p.r % 128 == 0 && ntok >= kGM &&
         xspan < 0x7fffffffL && espan < 0x7fffffffL;
}

}  // namespace

bool encode_supported(int dtype, int r) {
  return (dtype == LLA_F32 || dtype == LLA_BF16) && r >= 1 && r <= 512;
}

namespace {

// bf16 encode on the MFMA kernel for token counts below the tiled GEMM's (pv: a second axis of
// the same shape and rank in the same launch, or null)
hipError_t launch_encode_small(const EncodeParams& p, const EncodeParams* pv, hipStream_t stream) {
  int nt_tiles = p.r <= 16 ? 1 : p.r <= 32 ? 2 : 4;
  const long ntok = static_cast<long>(p.B) * p.C;
  // few workgroups with whole-K waves would leave most of the chip idle: split K instead,
  // eight ways for decode-size token counts, and narrow the latent tiles until the launch has a
  // workgroup per CU (fewer latent rows per workgroup re-read x more often, from L2)
  if (ntok <= 256) {
    auto wgs = [&](int nt) { return (ntok + 15) / 16 * ((p.r + 16 * nt - 1) / (16 * nt)) * p.H; };
    while (nt_tiles > 1 && wgs(nt_tiles) < 256) nt_tiles /= 2;
    return launch_encode_mfma<1, 8>(p, pv, nt_tiles, stream);
  }
  const long wgs1 = (ntok + 127) / 128 * ((p.r + 16 * nt_tiles - 1) / (16 * nt_tiles)) * p.H;
  return wgs1 < 1024 ? launch_encode_mfma<2, 4>(p, pv, nt_tiles, stream)
                     : launch_encode_mfma<2, 1>(p, pv, nt_tiles, stream);
}

}  // namespace

hipError_t launch_encode(const EncodeParams& p, int dtype, hipStream_t stream) {
  const int K = p.T * p.d;
  if (dtype == LLA_BF16) {
    if (encode_gemm_ok(p))
      return p.r % 256 == 0 ? launch_encode_gemm<256>(p, stream) : launch_encode_gemm<128>(p, stream);
    return launch_encode_small(p, nullptr, stream);
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

// Both axes of a token's encode (K then V). Where the two take the same decode-size MFMA plan
// (bf16, equal ranks, below the tiled GEMM's token counts) they share one launch, else each has its
// own.
hipError_t launch_encode_kv(const EncodeParams& pk, const EncodeParams& pv, int dtype, hipStream_t stream) {
  if (dtype == LLA_BF16 && pk.r == pv.r && !encode_gemm_ok(pk) && !encode_gemm_ok(pv))
    return launch_encode_small(pk, &pv, stream);
  const hipError_t e = launch_encode(pk, dtype, stream);
  if (e != hipSuccess) return e;
  return launch_encode(pv, dtype, stream);
}

}  // namespace lla
