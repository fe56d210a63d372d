// LLA-2D absorbed decode on bf16 MFMA.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 3, "The LLA-2D
// variant": one latent per token and layer rebuilds every head, so head h's loop-t key is rows
// h*d .. (h+1)*d-1 of W^K_t z^K. With the absorbed form of Section 7 every head scores the same
// latent with its own q~_h = W^K_t[h]^T q_h, and the V side accumulates sum_i p_hi z^V_i per head
// in latent space before one W^V_t[h] projection. Unlike per-head LLA this contraction is dense:
// 16 heads x r against every latent, so it runs on MFMA:
//
//   1. qproj2d_kernel: q~ (fp32, pre-scaled by scale*log2 e) and beta = q . mu^K_t per (b, h).
//   2. decode2d_partial_kernel: a workgroup owns (sequence b, token split, group of 16 heads);
//      each wave takes 16-token tiles. Scores S^T[token][head] = Z^K (16 x r_k) . Q~^T come from
//      v_mfma_f32_16x16x32_bf16 with q~ split into bf16 hi + lo parts (two MFMAs per k-step), so
//      the scores keep ~16 mantissa bits of q~. The accumulator layout puts head (lane % 16) and
//      four tokens in each lane, which is exactly the B-operand layout of
//      v_mfma_f32_16x16x16bf16_1k for P^T (tokens x heads): A^T[r][head] += Z^V^T (r x 16 tokens)
//      . P^T needs no data movement for P. Z^V is staged per wave in LDS (coalesced 16-byte
//      loads, rows padded so the transposed 16-bit reads are bank-conflict free). Online softmax
//      per head, rescaling only when the running max grows by more than 8 (base 2). The four
//      waves merge through LDS and the workgroup writes one (m, l, a[r_v]) partial per head.
//   3. combine2d_kernel: per (sequence, head); merges the split partials by log-sum-exp, adds the
//      optional self token, projects once through W^V_t[h], adds mu^V_t, normalises, writes o
//      and lse.
// Decoupled rotary branch (DR = d_rope > 0, Section 7): the rotary query rotated at the decoding
// position joins q~ as DR more contraction entries, and the tile's cached rotary keys (already
// rotated at their slots) join its K rows as DR/32 more MFMA k-steps, so the rotary scores are
// formed in the same accumulators; the self token's rotary score is q_rope . k_rope_self (rotating
// both at the same position leaves their dot product unchanged).
#include <type_traits>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

typedef const __attribute__((address_space(1))) void* gptr_t;  // global address space
typedef __attribute__((address_space(3))) void* lptr_t;         // LDS address space

constexpr float kLazy2d = 8.0f;

// XOR swizzle of the 16-byte chunks of V row `row` inside each aligned 8-chunk window. Every four
// consecutive rows land on four distinct chunk pairs (the transposed read below touches one
// adjacent pair in each of four consecutive rows per 16-lane group), and every eight consecutive
// rows on eight distinct chunks.
__device__ __forceinline__ int vswz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// A operand of v_mfma_f32_16x16x16bf16_1k holding Z^V^T[r0 + i][kb + k] (i, k < 16) from a
// row-major [key][RV] bf16 tile whose 16-byte chunks are XOR-swizzled by vswz(key). One
// ds_read_b64_tr_b16: in each 16-lane group q, source lane 4e + c points at the 8 bytes
// V[kb + 4q + e][r0 + 4c .. +3]; the transposed read hands lane i of the group element e =
// V[kb + 4q + e][r0 + i], which is the MFMA's A layout (row i, k = 4q + e). (Lane mapping of the
// instruction checked on the hardware.)
typedef __attribute__((address_space(3))) short4_t* lds_short4_ptr;
template <int RV>
__device__ __forceinline__ short4_t v_operand_tr(const char* vt, int kb, int r0, int lane) {
  const int q = lane >> 4;
  const int j = lane & 15;
  const int row = kb + 4 * q + (j >> 2);
  const int r = r0 + 4 * (j & 3);
  const int lc = r >> 3;
  const int pc = (lc & ~7) | ((lc & 7) ^ vswz(row));
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_ptr)(vt + row * RV * 2 + pc * 16 + (r & 7) * 2));
}

constexpr int kQB = 4;     // sequences per qproj / combine workgroup

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int seq_keys(const DecodeParams& p, int b) {
  int n = p.seq_lens != nullptr ? uniform(p.seq_lens[b]) : p.n_max;
  return min(max(n, 0), p.n_max);
}

// ---- 1. query absorption for every (b, h) ------------------------------------------------------
// grid H * ceil(B / kQB) (x), 256 threads. Wave w takes rows j in [32 w, 32 w + 32) of W^K_t[h]
// (d <= 128), lane l the CPL = RK / 64 columns l * CPL .. of each of those rows, so every load
// instruction reads one whole W^K row and a thread's 32 loads are all issued before its sums. Each
// thread forms its columns' partial q~ over its rows for kQB sequences; the four waves' partials
// meet in LDS.
// qt rows hold RK + DR floats: q~, then the rotated rotary query (both times scale * log2 e).
template <int CPL>
struct WSlice;  // CPL consecutive bf16 of a W^K row
template <>
struct WSlice<1> { using T = uint16_t; };
template <>
struct WSlice<2> { using T = uint32_t; };
template <>
struct WSlice<4> { using T = uint2; };
template <int CPL>
__device__ __forceinline__ float wslice_elem(const typename WSlice<CPL>::T& w, int e) {
  if constexpr (CPL == 1) return __uint_as_float(static_cast<uint32_t>(w) << 16);
  else if constexpr (CPL == 2) return e == 0 ? bf16_lo(w) : bf16_hi(w);
  else return e == 0 ? bf16_lo(w.x) : e == 1 ? bf16_hi(w.x) : e == 2 ? bf16_lo(w.y) : bf16_hi(w.y);
}

template <int RK, int DR>
__global__ __launch_bounds__(256) void qproj2d_kernel(DecodeParams p, float* qt, float* beta) {
  constexpr int QS = RK + DR;
  constexpr int CPL = RK / 64;
  constexpr int JQ = 32;  // rows of W^K per wave
  static_assert(CPL == 1 || CPL == 2 || CPL == 4, "r_k of 64, 128 or 256");
  using WT = typename WSlice<CPL>::T;
  __shared__ __attribute__((aligned(16))) float q_s[kQB][128];
  __shared__ float red_s[4][kQB][RK];
  const int h = blockIdx.x % p.H;  // one-dimensional grid: (block of kQB sequences) * H + head
  const int b0 = blockIdx.x / p.H * kQB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const size_t wrow = (static_cast<size_t>(p.t) * p.H + h) * p.d;  // rows of W^K_t for head h
  const WT* wsrc = reinterpret_cast<const WT*>(static_cast<const uint16_t*>(p.Wk) + wrow * RK) + lane;
  WT wv[JQ];
#pragma unroll
  for (int jj = 0; jj < JQ; ++jj) {
    const int j = wave * JQ + jj;
    wv[jj] = j < p.d ? wsrc[static_cast<size_t>(j) * 64] : WT{};
  }
  // q of the block's sequences, zero past d and past B
  for (int i = tid; i < kQB * 128; i += 256) {
    const int bb = i >> 7;
    const int j = i & 127;
    const int b = b0 + bb;
    q_s[bb][j] = (b < p.B && j < p.d) ? ld<BF16>(p.q, (static_cast<size_t>(b) * p.H + h) * p.d + j) : 0.f;
  }
  __syncthreads();
  float acc[kQB][CPL];
#pragma unroll
  for (int bb = 0; bb < kQB; ++bb)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[bb][e] = 0.f;
#pragma unroll
  for (int j4 = 0; j4 < JQ; j4 += 4) {
    float4 qv[kQB];
#pragma unroll
    for (int bb = 0; bb < kQB; ++bb) qv[bb] = *reinterpret_cast<const float4*>(&q_s[bb][wave * JQ + j4]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const float w = wslice_elem<CPL>(wv[j4 + u], e);
#pragma unroll
        for (int bb = 0; bb < kQB; ++bb)
          acc[bb][e] += w * (u == 0 ? qv[bb].x : u == 1 ? qv[bb].y : u == 2 ? qv[bb].z : qv[bb].w);
      }
  }
#pragma unroll
  for (int bb = 0; bb < kQB; ++bb)
#pragma unroll
    for (int e = 0; e < CPL; ++e) red_s[wave][bb][lane * CPL + e] = acc[bb][e];
  __syncthreads();
  for (int i = tid; i < kQB * RK; i += 256) {
    const int bb = i / RK;
    const int k = i - bb * RK;
    if (b0 + bb < p.B)
      qt[(static_cast<size_t>(b0 + bb) * p.H + h) * QS + k] =
          ((red_s[0][bb][k] + red_s[1][bb][k]) + (red_s[2][bb][k] + red_s[3][bb][k])) * p.scale_log2;
  }
  if constexpr (DR > 0) {
    // rotary query of each sequence rotated at its decoding position N_b (the sequence differs
    // across the threads here, so its length is read per thread)
    for (int i = tid; i < kQB * (DR / 2); i += 256) {
      const int bb = i / (DR / 2);
      const int pr = i - bb * (DR / 2);
      const int b = b0 + bb;
      if (b >= p.B) continue;
      int n = p.seq_lens != nullptr ? p.seq_lens[b] : p.n_max;
      n = min(max(n, 0), p.n_max);
      const size_t row = static_cast<size_t>(b) * p.H + h;
      float y0, y1;
      rotate_pair(ld<BF16>(p.q_rope, row * DR + 2 * pr), ld<BF16>(p.q_rope, row * DR + 2 * pr + 1), pr, DR,
                  n, p.rope_base, &y0, &y1);
      qt[row * QS + RK + 2 * pr] = y0 * p.scale_log2;
      qt[row * QS + RK + 2 * pr + 1] = y1 * p.scale_log2;
    }
  }
  // beta = scale*log2e * q . mu^K_t (2D mu is [T*H*d], loop t head h at (t*H + h)*d)
  for (int bb = wave; bb < kQB; bb += 4) {
    float part = 0.f;
    if (p.mu_k != nullptr)
      for (int j = lane; j < p.d; j += 64) part += q_s[bb][j] * ld<BF16>(p.mu_k, wrow + j);
    part = wave_sum(part);
    if (lane == 0 && b0 + bb < p.B) beta[static_cast<size_t>(b0 + bb) * p.H + h] = part * p.scale_log2;
  }
}

// ---- 2. MFMA latent stream ---------------------------------------------------------------------
// One workgroup of kW waves per (sequence, token split, 16-head group); wave w takes the 16-token
// tiles w, w + kW, ... of the split. Per tile:
//   * the next tile's K rows are loaded into registers and its V rows go straight to LDS with
//     global_load_lds (each lane's 16 bytes land at base + 16*lane), into the other half of the
//     wave's double-buffered ring, so both loads overlap the current tile's MFMAs;
//   * K is loaded as whole 128-byte lines (see k_lines_to_operands) with a non-temporal hint and
//     put into the MFMA operand layout when the tile is consumed;
//   * V rows are stored unpadded with 16-byte chunks XOR-swizzled by the row: chunk c of row rho
//     sits at (c & ~7) | ((c & 7) ^ vswz(rho)), so the transposed reads of the MFMA's V operand
//     (ds_read_b64_tr_b16, 16 rows x 32 bytes per read) spread evenly over the banks. The swizzle
//     is applied by choosing each lane's global source address;
//   * rows past the valid range are clamped to the last valid token (finite data times a zero
//     weight), so a partial tail tile needs no separate zeroing.
// K tiles are loaded as whole 128-byte lines. The pair of 32-wide k-steps (2m, 2m + 1) covers
// bytes [128 m, 128 m + 128) of each token row. In the first of its two loads lane (i, g) reads
// token i & 7 and in the second token 8 + (i & 7); the lane takes 16 bytes at 16 g of the line's
// first half when the token's half of the tile (token < 8 or not) matches the lane's half of its
// row of 16 (i < 8 or not), else of the second half. Each load then reads 8 whole lines, where
// the MFMA layout (token i at lane (i, g), one 64-byte half per load) would read 16 half lines.
// The A operand of step 2m (token i, first half) is a lane select between the two loads; that of
// step 2m + 1 (token i, second half) is the opposite select moved by 8 lanes within each row of
// 16 (DPP row_ror:8, lane i <-> i ^ 8).
__device__ __forceinline__ uint32_t row_ror8(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ void k_lines_to_operands(uint4& a, uint4& b, bool lo) {
  const uint4 x = lo ? a : b;
  const uint4 z = lo ? b : a;
  a = x;
  b = make_uint4(row_ror8(z.x), row_ror8(z.y), row_ror8(z.z), row_ror8(z.w));
}

template <int RK, int RV>
struct Cfg2d {
  static constexpr int kW = 8;                          // waves per workgroup
  static constexpr int kVTile = 16 * RV * 2;            // bytes of one 16-token V tile
  static constexpr int kPart = 16 * (2 + RV) * 4;       // one (m, l, a) partial for 16 heads
  static constexpr int kRing = kW * 2 * kVTile;         // all waves' double-buffered V rings
  static_assert(kRing >= 4 * kPart, "the final merge reuses the V rings");
};

// DR: width of the fused rotary branch (0 without): DR / 32 more k-steps whose A fragments are the
// tile's rotary key rows, loaded with its K rows.
template <int RK, int RV, int DR = 0>
__global__ __launch_bounds__(512) void decode2d_partial_kernel(DecodeParams p, const float* qt,
                                                               const float* beta, float* part) {
  using CF = Cfg2d<RK, RV>;
  constexpr int kW = CF::kW;
  constexpr int KS = RK / 32;
  constexpr int KT = KS + DR / 32;     // k-steps: the latent, then the rotary branch
  constexpr int QS = RK + DR;          // q~ row (qproj2d_kernel's layout)
  constexpr int RT = RV / 16;
  constexpr int CPR = RV / 8;          // 16-byte chunks per V row
  constexpr int VPL = CPR / 4;         // chunks per lane for a 16-row tile (16*CPR / 64)
  static_assert(RK % 64 == 0 && RV % 64 == 0 && DR % 32 == 0, "r_k, r_v multiples of 64, d_rope of 32");

  __shared__ __attribute__((aligned(16))) uint16_t qhi[16 * QS];
  __shared__ __attribute__((aligned(16))) uint16_t qlo[16 * QS];
  __shared__ float beta_s[16];
  __shared__ __attribute__((aligned(16))) char ring[CF::kRing];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int split = blockIdx.x % p.splits;  // grid x: b * splits + split; y: head group
  const int b = blockIdx.x / p.splits;
  const int h0 = blockIdx.y * 16;
  const int h = h0 + col;
  const bool hvalid = h < p.H;

  const int nb = seq_keys(p, b);
  const int tb = split * p.chunk;
  const int te = min(nb, tb + p.chunk);

  const char* zkb = static_cast<const char*>(p.zk) + static_cast<size_t>(b) * p.n_max * RK * 2;
  const char* zvb = static_cast<const char*>(p.zv) + static_cast<size_t>(b) * p.n_max * RV * 2;
  char* myring = ring + wave * 2 * CF::kVTile;

  const char* krb = DR > 0 ? static_cast<const char*>(p.k_rope) + static_cast<size_t>(b) * p.n_max * DR * 2 : nullptr;
  // issue the loads of the tile starting at tok0 (tok0 < te): V into ring half `buf`, K and the
  // rotary keys into kr
  auto issue = [&](int tok0, int buf, uint4 (&kr)[KT]) {
    const int last = te - 1;
    char* dst = myring + buf * CF::kVTile;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int f = i * 64 + lane;               // LDS slot of this lane
      const int row = f / CPR;
      const int pc = f - row * CPR;
      const int lc = (pc & ~7) | ((pc & 7) ^ vswz(row));
      const char* src = zvb + (static_cast<size_t>(min(tok0 + row, last)) * RV + lc * 8) * 2;
      // non-temporal: each instruction reads 1 KiB of whole rows that nothing reads again
      __builtin_amdgcn_global_load_lds((const gptr_t)src, (lptr_t)(dst + i * 1024), 16, 0, 2);
    }
    // whole 128-byte lines of tokens 0..7 (first load of a pair) and 8..15 (second)
    const char* ra = zkb + static_cast<size_t>(min(tok0 + (col & 7), last)) * RK * 2 + (col >= 8 ? 64 : 0) + 16 * g;
    const char* rb = zkb + static_cast<size_t>(min(tok0 + 8 + (col & 7), last)) * RK * 2 + (col < 8 ? 64 : 0) + 16 * g;
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) {
      kr[2 * m] = load_stream(ra + 128 * m);
      kr[2 * m + 1] = load_stream(rb + 128 * m);
    }
    if constexpr (DR > 0) {
      const char* rrow = krb + static_cast<size_t>(min(tok0 + col, last)) * DR * 2;
#pragma unroll
      for (int ks = 0; ks < DR / 32; ++ks)
        kr[KS + ks] = *reinterpret_cast<const uint4*>(rrow + (32 * ks + 8 * g) * 2);
    }
  };

  floatx4_t D[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) D[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;
  float l = 0.f;

  uint4 kc[KT];
  int tok0 = tb + wave * 16;
  int buf = 0;
  // the first tile is requested before q~ is staged, so the two latencies overlap
  if (tok0 < te) issue(tok0, 0, kc);
  for (int i = tid; i < 16 * QS; i += 64 * kW) {
    const int hh = i / QS;
    const int k = i - hh * QS;
    const float v = (h0 + hh < p.H) ? qt[(static_cast<size_t>(b) * p.H + h0 + hh) * QS + k] : 0.f;
    const uint16_t hi = f32_to_bf16(v);
    qhi[i] = hi;
    qlo[i] = f32_to_bf16(v - __uint_as_float(static_cast<uint32_t>(hi) << 16));
  }
  if (tid < 16) beta_s[tid] = (h0 + tid < p.H) ? beta[static_cast<size_t>(b) * p.H + h0 + tid] : 0.f;
  __syncthreads();

  const float bt = beta_s[col];
  for (; tok0 < te; tok0 += 16 * kW) {
    uint4 kn[KT];
    const bool more = tok0 + 16 * kW < te;
    if (more) issue(tok0 + 16 * kW, buf ^ 1, kn);
    // scores S^T[token tok0 + i][head h0 + j]: hi and lo parts of q~ in two independent chains
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) k_lines_to_operands(kc[2 * m], kc[2 * m + 1], col < 8);
    floatx4_t sh = {0.f, 0.f, 0.f, 0.f};
    floatx4_t sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KT; ++ks) {
      const uint4 bh = *reinterpret_cast<const uint4*>(&qhi[col * QS + 32 * ks + 8 * g]);
      const uint4 bl = *reinterpret_cast<const uint4*>(&qlo[col * QS + 32 * ks + 8 * g]);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, kc[ks]);
      sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bh), sh, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bl), sl, 0, 0, 0);
    }
    float sc[4];
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = hvalid && (tok0 + 4 * g + e) < te;
      sc[e] = ok ? (sh[e] + sl[e]) + bt : kNegInf;
      tmax = fmaxf(tmax, sc[e]);
    }
    tmax = max_over_groups(tmax);
    if (tmax > m + kLazy2d) {
      const float c = fast_exp2(m - tmax);
      l *= c;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) D[rt] *= c;
      m = tmax;
    }
    short4_t bp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = (sc[e] == kNegInf) ? 0.f : fast_exp2(sc[e] - m);
      l += pe;
      bp[e] = static_cast<short>(f32_to_bf16(pe));
    }
    // this tile's V must have landed in LDS: at most the next tile's loads may be outstanding
    if (more)
      __builtin_amdgcn_s_waitcnt((KT + VPL) >= 16 ? 0x4f70 | (((KT + VPL) - 16) & 15) : 0x0f70 | (KT + VPL));
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __asm__ volatile("" ::: "memory");
    const char* vt = myring + buf * CF::kVTile;
    // A^T[r][head] += Z^V^T[r][tokens 4g+e] . P^T[tokens][head]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      D[rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v_operand_tr<RV>(vt, 0, 16 * rt, lane), bp, D[rt], 0, 0, 0);
    // the ring half just read is refilled two tiles from now; finish the reads first
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < KT; ++i) kc[i] = kn[i];
    buf ^= 1;
  }
  l = sum_over_groups(l);

  // merge the waves through LDS (the V rings are free now): 8 -> 4 -> 2 -> 1
  __syncthreads();
  float* ps = reinterpret_cast<float*>(ring);
  constexpr int PS = 16 * (2 + RV);
  auto put = [&](float* dst) {
    if (g == 0) {
      dst[col * (2 + RV)] = m;
      dst[col * (2 + RV) + 1] = l;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[col * (2 + RV) + 2 + 16 * rt + 4 * g + e] = D[rt][e];
  };
  auto take = [&](const float* src) {
    const float mo = src[col * (2 + RV)];
    const float lo = src[col * (2 + RV) + 1];
    const float M = fmaxf(m, mo);
    const float fa = (m == kNegInf) ? 0.f : fast_exp2(m - M);
    const float fb = (mo == kNegInf) ? 0.f : fast_exp2(mo - M);
    l = l * fa + lo * fb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) D[rt][e] = D[rt][e] * fa + src[col * (2 + RV) + 2 + 16 * rt + 4 * g + e] * fb;
    m = M;
  };
#pragma unroll
  for (int half = kW / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) put(ps + (wave - half) * PS);
    __syncthreads();
    if (wave < half) take(ps + wave * PS);
    __syncthreads();
  }
  if (wave != 0 || !hvalid) return;
  // partial layout [B][H][S][2 + RV]
  float* w = part + ((static_cast<size_t>(b) * p.H + h) * p.splits + split) * (2 + RV);
  if (g == 0) {
    w[0] = m;
    w[1] = l;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) w[2 + 16 * rt + 4 * g + e] = D[rt][e];
}

// ---- 2b. MFMA latent stream with register-staged tiles -----------------------------------------
// The contraction of decode2d_partial_kernel (bf16 MFMA, q~ as hi + lo, same score layout and
// online softmax) with the tiles staged through registers instead of an LDS-DMA ring. Instantiated
// for low-bit rows (LS = Q8 or I8: LLA-2D rows of E4M3 or int8 codes with a float32 row scale, the
// low-bit layout of lla.h), whose codes must be converted before the MFMA; it also reads bf16 rows
// (LS = BF16), but there the LDS-DMA ring is faster (190 vs 222-231 us per read at B = 128,
// N = 8192, r = 256: the staged bf16 tiles need 256 registers and spill).
//   * Two register sets per wave hold the loads of the next two 16-token tiles; a tile's set is
//     refilled with the tile two ahead as soon as its registers have been consumed (after its V
//     rows are in LDS and its score MFMAs are issued), so every tile's loads have about one and a
//     half iterations to land. The loads are unconditional (rows past the split are clamped to its
//     last token and masked; a wave may run one wholly masked tile at its end).
//   * V: the wave writes the tile's rows to its own LDS tile in the XOR-swizzled layout of the ring
//     kernel, so the transposed operand reads are the same; written and read in one iteration.
//   * Low-bit rows: every code is exactly a bf16 value, so codes are converted to bf16 on the way
//     to the MFMA and the row scales stay outside the products -- the K scale multiplies the
//     token's score, the V scale its weight in P (the softmax denominator sums unscaled weights).
//     Inside each pair of 32-wide k-steps the contraction order is permuted so that a lane's
//     operands for both steps are one 16-byte run of its token's codes (lane (i, g) of step 2 m + hh
//     holds entries 64 m + 16 g + 8 hh .. + 7; q~ is read in the same order). Lanes 0..15 load
//     their token's two scales; the score layout (head per lane, four tokens) takes them by lane
//     shuffles.
template <class LS>
__device__ __forceinline__ float code_value(uint32_t w, int e);  // byte e (literal) of w as a float
template <>
__device__ __forceinline__ float code_value<Q8>(uint32_t w, int e) {
  switch (e) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), 3);
  }
}
template <>
__device__ __forceinline__ float code_value<I8>(uint32_t w, int e) {
  return static_cast<float>(static_cast<int8_t>(w >> (8 * e)));
}
// four codes (one word) -> four bf16 (two words), exactly
template <class LS>
__device__ __forceinline__ uint2 codes4_bf16(uint32_t w) {
  return make_uint2(f32x2_to_bf16x2(code_value<LS>(w, 0), code_value<LS>(w, 1)),
                    f32x2_to_bf16x2(code_value<LS>(w, 2), code_value<LS>(w, 3)));
}

template <class LS, int RK, int RV>
__global__ __launch_bounds__(512) void decode2d_staged_kernel(DecodeParams p, const float* qt,
                                                              const float* beta, float* part) {
  constexpr bool kLow = !std::is_same<LS, BF16>::value;
  constexpr int kW = 8;
  constexpr int KS = RK / 32;
  constexpr int NK = kLow ? KS / 2 : KS;        // 16-byte K loads per lane and tile
  constexpr int QS = RK;
  constexpr int RT = RV / 16;
  constexpr int RKB = kLow ? LS::row(RK) : RK * 2;  // bytes per cached row
  constexpr int RVB = kLow ? LS::row(RV) : RV * 2;
  constexpr int CPR = (kLow ? RV : 2 * RV) / 16;    // 16-byte chunks of a row's V codes or values
  constexpr int NV = CPR / 4;                       // V loads per lane and tile (16 * CPR / 64)
  constexpr int kVTile = 16 * RV * 2;               // bytes of one bf16 tile in LDS
  constexpr int kPart = 16 * (2 + RV) * 4;
  constexpr int kTiles = kW * kVTile > 4 * kPart ? kW * kVTile : 4 * kPart;  // the merge reuses it
  static_assert(RK % 64 == 0 && RV % 64 == 0, "r_k and r_v multiples of 64");

  __shared__ __attribute__((aligned(16))) uint16_t qhi[16 * QS];
  __shared__ __attribute__((aligned(16))) uint16_t qlo[16 * QS];
  __shared__ float beta_s[16];
  __shared__ __attribute__((aligned(16))) char tiles[kTiles];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int split = blockIdx.x % p.splits;  // grid x: b * splits + split; y: head group
  const int b = blockIdx.x / p.splits;
  const int h0 = blockIdx.y * 16;
  const int h = h0 + col;
  const bool hvalid = h < p.H;

  const int nb = seq_keys(p, b);
  const int tb = split * p.chunk;
  const int te = min(nb, tb + p.chunk);

  for (int i = tid; i < 16 * QS; i += 64 * kW) {
    const int hh = i / QS;
    const int k = i - hh * QS;
    const float v = (h0 + hh < p.H) ? qt[(static_cast<size_t>(b) * p.H + h0 + hh) * QS + k] : 0.f;
    const uint16_t hi = f32_to_bf16(v);
    qhi[i] = hi;
    qlo[i] = f32_to_bf16(v - __uint_as_float(static_cast<uint32_t>(hi) << 16));
  }
  if (tid < 16) beta_s[tid] = (h0 + tid < p.H) ? beta[static_cast<size_t>(b) * p.H + h0 + tid] : 0.f;
  __syncthreads();

  const float bt = beta_s[col];
  const char* zkb = static_cast<const char*>(p.zk) + static_cast<size_t>(b) * p.n_max * RKB;
  const char* zvb = static_cast<const char*>(p.zv) + static_cast<size_t>(b) * p.n_max * RVB;
  char* mytile = tiles + wave * kVTile;

  struct Set {
    uint4 k[NK];
    uint4 v[NV];
    float sk, sv;  // low-bit: the scales of token col of the tile
  };
  // the loads of the tile starting at tok0 (tok0 <= te - 1): K runs, V chunks, row scales
  auto issue = [&](int tok0, Set& st) {
    const int last = te - 1;
    const size_t krow = static_cast<size_t>(min(tok0 + col, last));
    const char* kr = zkb + krow * RKB;
#pragma unroll
    for (int i = 0; i < NK; ++i) st.k[i] = *reinterpret_cast<const uint4*>(kr + 64 * i + 16 * g);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = u * 64 + lane;
      const int row = c / CPR;
      st.v[u] = *reinterpret_cast<const uint4*>(zvb + static_cast<size_t>(min(tok0 + row, last)) * RVB +
                                                16 * (c - row * CPR));
    }
    if constexpr (kLow) {
      st.sk = *reinterpret_cast<const float*>(kr + RKB - 4);
      st.sv = *reinterpret_cast<const float*>(zvb + krow * RVB + RVB - 4);
    }
  };

  floatx4_t D[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) D[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;
  float l = 0.f;

  // one tile: its V rows into LDS, its scores, the refill of its set with tile tnext, then the
  // softmax and the P.V products
  auto run = [&](Set& st, int tok0, int tnext) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int c = u * 64 + lane;
      const int row = c / CPR;
      const int cc = c - row * CPR;
      if constexpr (kLow) {  // 16 codes -> bf16 chunks 2 cc and 2 cc + 1 of the row
        const uint2 a0 = codes4_bf16<LS>(st.v[u].x), a1 = codes4_bf16<LS>(st.v[u].y);
        const uint2 a2 = codes4_bf16<LS>(st.v[u].z), a3 = codes4_bf16<LS>(st.v[u].w);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int lc = 2 * cc + half;
          const int pc = (lc & ~7) | ((lc & 7) ^ vswz(row));
          *reinterpret_cast<uint4*>(mytile + row * RV * 2 + pc * 16) =
              half == 0 ? make_uint4(a0.x, a0.y, a1.x, a1.y) : make_uint4(a2.x, a2.y, a3.x, a3.y);
        }
      } else {
        const int pc = (cc & ~7) | ((cc & 7) ^ vswz(row));
        *reinterpret_cast<uint4*>(mytile + row * RV * 2 + pc * 16) = st.v[u];
      }
    }
    // scores S^T[token tok0 + i][head h0 + j], hi and lo parts of q~ in two chains
    floatx4_t sh = {0.f, 0.f, 0.f, 0.f};
    floatx4_t sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 a;
      int e0;
      if constexpr (kLow) {
        const uint4 w = st.k[ks >> 1];
        const uint2 k0 = codes4_bf16<LS>((ks & 1) ? w.z : w.x);
        const uint2 k1 = codes4_bf16<LS>((ks & 1) ? w.w : w.y);
        a = make_uint4(k0.x, k0.y, k1.x, k1.y);
        e0 = 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);
      } else {
        a = st.k[ks];
        e0 = 32 * ks + 8 * g;
      }
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
      const uint4 bh = *reinterpret_cast<const uint4*>(&qhi[col * QS + e0]);
      const uint4 bl = *reinterpret_cast<const uint4*>(&qlo[col * QS + e0]);
      sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bh), sh, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bl), sl, 0, 0, 0);
    }
    float sks[4], svs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // lane 4g + e holds token 4g + e's scales
      sks[e] = kLow ? __shfl(st.sk, 4 * g + e, 64) : 1.f;
      svs[e] = kLow ? __shfl(st.sv, 4 * g + e, 64) : 1.f;
    }
    issue(min(tnext, te - 1), st);
    float sc[4];
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = hvalid && (tok0 + 4 * g + e) < te;
      sc[e] = ok ? (sh[e] + sl[e]) * sks[e] + bt : kNegInf;
      tmax = fmaxf(tmax, sc[e]);
    }
    tmax = max_over_groups(tmax);
    if (tmax > m + kLazy2d) {
      const float c = fast_exp2(m - tmax);
      l *= c;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) D[rt] *= c;
      m = tmax;
    }
    short4_t bp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = (sc[e] == kNegInf) ? 0.f : fast_exp2(sc[e] - m);
      l += pe;
      bp[e] = static_cast<short>(f32_to_bf16(pe * svs[e]));
    }
    wave_lds_sync();  // the tile's bf16 rows are in LDS before the transposed reads
    // A^T[r][head] += Z^V^T[r][tokens 4g+e] . (P^T, times the V row scales)[tokens][head]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      D[rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v_operand_tr<RV>(mytile, 0, 16 * rt, lane), bp, D[rt], 0, 0, 0);
    wave_lds_sync();  // the reads are done before the next tile's rows are written
  };

  constexpr int kStep = 16 * kW;
  Set s0, s1;
  int tok0 = tb + wave * 16;
  if (tok0 < te) {
    issue(tok0, s0);
    issue(min(tok0 + kStep, te - 1), s1);
  }
  for (; tok0 < te; tok0 += 2 * kStep) {
    run(s0, tok0, tok0 + 2 * kStep);
    run(s1, tok0 + kStep, tok0 + 3 * kStep);  // wholly masked when past the split
  }
  l = sum_over_groups(l);

  // merge the waves through LDS (the tiles are free now): 8 -> 4 -> 2 -> 1
  __syncthreads();
  float* ps = reinterpret_cast<float*>(tiles);
  constexpr int PS = 16 * (2 + RV);
  auto put = [&](float* dst) {
    if (g == 0) {
      dst[col * (2 + RV)] = m;
      dst[col * (2 + RV) + 1] = l;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[col * (2 + RV) + 2 + 16 * rt + 4 * g + e] = D[rt][e];
  };
  auto take = [&](const float* src) {
    const float mo = src[col * (2 + RV)];
    const float lo = src[col * (2 + RV) + 1];
    const float M = fmaxf(m, mo);
    const float fa = (m == kNegInf) ? 0.f : fast_exp2(m - M);
    const float fb = (mo == kNegInf) ? 0.f : fast_exp2(mo - M);
    l = l * fa + lo * fb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) D[rt][e] = D[rt][e] * fa + src[col * (2 + RV) + 2 + 16 * rt + 4 * g + e] * fb;
    m = M;
  };
#pragma unroll
  for (int half = kW / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) put(ps + (wave - half) * PS);
    __syncthreads();
    if (wave < half) take(ps + wave * PS);
    __syncthreads();
  }
  if (wave != 0 || !hvalid) return;
  float* w = part + ((static_cast<size_t>(b) * p.H + h) * p.splits + split) * (2 + RV);
  if (g == 0) {
    w[0] = m;
    w[1] = l;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) w[2 + 16 * rt + 4 * g + e] = D[rt][e];
}

// ---- 3. merge splits, project once through W^V_t[h], finish ------------------------------------
// One 256-thread workgroup per (head, block of kQB sequences): W^V_t[h] is read once for the block.
// Thread (grp, sub) = (tid / 16, tid % 16) holds rows grp + 16 i (i < 8: d <= 128) of it, 16-byte
// chunks sub + 16 k of each, so each load instruction reads whole runs of four consecutive rows.
// Every load that does not depend on the merge (W^V, the first split partials of all kQB
// sequences, mu^V_t, the self values) is issued first; wave w merges sequences w, w + 4, ...
// (log-sum-exp over the splits, the self token), the merged latent sums go to LDS, each thread
// dots its row slices with them, 16 lanes sum each row, and lane sub writes row grp + 16 sub.
template <int RV>
__global__ __launch_bounds__(256) void combine2d_kernel(DecodeParams p, const float* part) {
  constexpr int CPR = RV / 8;            // 16-byte chunks of a W^V row
  constexpr int NC = (CPR + 15) / 16;    // chunks per thread and row
  constexpr int RPT = (RV + 255) / 256;  // latent entries per thread in the merge
  constexpr int kPre = 2;                // splits whose partial sums are loaded up front
  __shared__ __attribute__((aligned(16))) float a_s[kQB][RV];
  __shared__ float f_s[kQB][64];
  __shared__ float fin_s[kQB][4];  // f_lat, p_self, 1/den, l
  const int h = blockIdx.x % p.H;  // one-dimensional grid: (block of kQB sequences) * H + head
  const int b0 = blockIdx.x / p.H * kQB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int S_ = p.splits;
  const size_t wrow = (static_cast<size_t>(p.t) * p.H + h) * p.d;  // W^V_t rows of head h; mu offset

  // ---- issue: this thread's slices of W^V_t[h] ----
  const int grp = tid >> 4;
  const int sub = tid & 15;
  uint4 w[8][NC];
  {
    const uint4* wr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.Wv) + wrow * RV);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        const int j = grp + 16 * i;
        const int c = sub + 16 * k;
        w[i][k] = (j < p.d && c < CPR) ? wr[static_cast<size_t>(j) * CPR + c] : make_uint4(0, 0, 0, 0);
      }
  }
  const int jw = grp + 16 * sub;  // the row this thread writes (sub < 8)
  const bool jok = sub < 8 && jw < p.d;
  float mu_j = 0.f;
  if (jok && p.mu_v != nullptr) mu_j = ld<BF16>(p.mu_v, wrow + jw);
  float vself[kQB];  // this thread's row of each sequence's self value
#pragma unroll
  for (int bb = 0; bb < kQB; ++bb)
    vself[bb] = (jok && p.v_self != nullptr && b0 + bb < p.B)
                    ? ld<BF16>(p.v_self, (static_cast<size_t>(b0 + bb) * p.H + h) * p.d + jw) : 0.f;
  // split latent sums of the first kPre splits for every sequence of the block
  float pa[kQB][RPT][kPre];
#pragma unroll
  for (int bb = 0; bb < kQB; ++bb) {
    const bool bok = b0 + bb < p.B;
    const float* pw = part + ((static_cast<size_t>(bok ? b0 + bb : 0)) * p.H + h) * S_ * (2 + RV);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = tid + 256 * i;
#pragma unroll
      for (int s2 = 0; s2 < kPre; ++s2)
        pa[bb][i][s2] = (bok && r < RV && s2 < S_) ? pw[static_cast<size_t>(s2) * (2 + RV) + 2 + r] : 0.f;
    }
  }
  // wave w: split maxima and sums, self score, of sequences w, w + 4, ...
  for (int bb = wave; bb < kQB; bb += 4) {
    const int b = b0 + bb;
    if (b >= p.B) break;
    const size_t bh = static_cast<size_t>(b) * p.H + h;
    const float* pw = part + bh * S_ * (2 + RV);
    float ms = kNegInf, ls = 0.f, pt = 0.f;
    if (lane < S_) {
      ms = pw[static_cast<size_t>(lane) * (2 + RV)];
      ls = pw[static_cast<size_t>(lane) * (2 + RV) + 1];
    }
    if (p.k_self != nullptr)
      for (int jj = lane; jj < p.d; jj += 64) pt += ld<BF16>(p.q, bh * p.d + jj) * ld<BF16>(p.k_self, bh * p.d + jj);
    if (p.k_self != nullptr && p.d_rope > 0)  // the self key's rotary part (same position as q)
      for (int jj = lane; jj < p.d_rope; jj += 64)
        pt += ld<BF16>(p.q_rope, bh * p.d_rope + jj) * ld<BF16>(p.k_rope_self, static_cast<size_t>(b) * p.d_rope + jj);
    const float M = wave_max(ms);
    const float fs = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
    const float l = wave_sum(fs * ls);
    const float s_self = p.k_self != nullptr ? wave_sum(pt) * p.scale_log2 : kNegInf;
    f_s[bb][lane] = fs;
    const float M2 = fmaxf(M, s_self);
    const float f_lat = (M == kNegInf) ? 0.f : fast_exp2(M - M2);
    const float p_self = (s_self == kNegInf) ? 0.f : fast_exp2(s_self - M2);
    const float den = l * f_lat + p_self;
    if (lane == 0) {
      fin_s[bb][0] = f_lat;
      fin_s[bb][1] = p_self;
      fin_s[bb][2] = den > 0.f ? 1.0f / den : 0.f;
      fin_s[bb][3] = l;
      if (p.lse != nullptr) p.lse[bh] = den > 0.f ? (M2 + fast_log2(den)) * kLn2 : kNegInf;
    }
  }
  __syncthreads();
  // merged latent sums a = sum_s f_s a_s (f_s is 0 for splits >= S)
#pragma unroll
  for (int bb = 0; bb < kQB; ++bb) {
    if (b0 + bb >= p.B) break;
    const float* pw = part + ((static_cast<size_t>(b0 + bb)) * p.H + h) * S_ * (2 + RV);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = tid + 256 * i;
      if (r < RV) {
        float a = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kPre; ++s2) a += f_s[bb][s2] * pa[bb][i][s2];
        for (int s2 = kPre; s2 < S_; ++s2) a += f_s[bb][s2] * pw[static_cast<size_t>(s2) * (2 + RV) + 2 + r];
        a_s[bb][r] = a;
      }
    }
  }
  __syncthreads();
  // o[b][j] = (W^V_t[h] row j . a_b + l_b mu^V_t[j]) f_lat + p_self v_self[j], normalised
  for (int bb = 0; bb < kQB; ++bb) {
    const int b = b0 + bb;
    if (b >= p.B) break;
    float av[NC][8];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = min(sub + 16 * k, CPR - 1);  // chunks past the row hold zero weights
      const float4 x0 = *reinterpret_cast<const float4*>(&a_s[bb][8 * c]);
      const float4 x1 = *reinterpret_cast<const float4*>(&a_s[bb][8 * c + 4]);
      av[k][0] = x0.x; av[k][1] = x0.y; av[k][2] = x0.z; av[k][3] = x0.w;
      av[k][4] = x1.x; av[k][5] = x1.y; av[k][6] = x1.z; av[k][7] = x1.w;
    }
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        o += bf16_lo(w[i][k].x) * av[k][0] + bf16_hi(w[i][k].x) * av[k][1];
        o += bf16_lo(w[i][k].y) * av[k][2] + bf16_hi(w[i][k].y) * av[k][3];
        o += bf16_lo(w[i][k].z) * av[k][4] + bf16_hi(w[i][k].z) * av[k][5];
        o += bf16_lo(w[i][k].w) * av[k][6] + bf16_hi(w[i][k].w) * av[k][7];
      }
      o = group_sum<16>(o);
      if (sub == i) mine = o;
    }
    if (jok) {
      const size_t bh = static_cast<size_t>(b) * p.H + h;
      float o = mine + fin_s[bb][3] * mu_j;
      o *= fin_s[bb][0];
      o += fin_s[bb][1] * vself[bb];
      st<BF16>(p.out, bh * p.d + jw, o * fin_s[bb][2]);
    }
  }
}

// Rotary branch widths of the fused read, index 0 = none.
constexpr int kRopeWidths[4] = {0, 32, 64, 128};

struct Entry2d {
  int r_k, r_v;
  void (*qproj[4])(DecodeParams, float*, float*);                     // by kRopeWidths
  void (*partial[4])(DecodeParams, const float*, const float*, float*);
  void (*combine)(DecodeParams, const float*);
  void (*staged[2])(DecodeParams, const float*, const float*, float*);  // E4M3, int8 rows
};

template <int RK, int RV>
constexpr Entry2d entry2d() {
  return {RK, RV,
          {qproj2d_kernel<RK, 0>, qproj2d_kernel<RK, 32>, qproj2d_kernel<RK, 64>, qproj2d_kernel<RK, 128>},
          {decode2d_partial_kernel<RK, RV, 0>, decode2d_partial_kernel<RK, RV, 32>,
           decode2d_partial_kernel<RK, RV, 64>, decode2d_partial_kernel<RK, RV, 128>},
          combine2d_kernel<RV>,
          {decode2d_staged_kernel<Q8, RK, RV>, decode2d_staged_kernel<I8, RK, RV>}};
}

int rope_index(int d_rope) {
  for (int i = 0; i < 4; ++i)
    if (kRopeWidths[i] == d_rope) return i;
  return -1;
}

const Entry2d kTable2d[] = {
    entry2d<64, 64>(), entry2d<128, 128>(), entry2d<256, 256>(),
};

const Entry2d* find2d(int r_k, int r_v) {
  for (const Entry2d& e : kTable2d)
    if (e.r_k == r_k && e.r_v == r_v) return &e;
  return nullptr;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool decode2d_mfma_supported(int dtype, int r_k, int r_v, int d_head) {
  return (dtype == LLA_BF16 || dtype == LLA_BF16_Q8 || dtype == LLA_BF16_I8) && d_head <= 128 &&
         find2d(r_k, r_v) != nullptr;
}

void decode2d_plan(const lla_desc& desc, int B, int* splits, int* chunk) {
  const int hg = (desc.H + 15) / 16;
  const long wgs = static_cast<long>(B) * hg;
  // one full round of resident 8-wave workgroups: one per CU at r_v = 256 (LDS), two below
  const long target = 256L * (desc.r_v > 128 ? 1 : 2);
  int s = static_cast<int>((target + wgs - 1) / wgs);
  const int max_by_len = desc.n_max / 256 > 0 ? desc.n_max / 256 : 1;
  if (s > max_by_len) s = max_by_len;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int c = (desc.n_max + s - 1) / s;
  c = (c + 63) / 64 * 64;
  s = (desc.n_max + c - 1) / c;
  *splits = s;
  *chunk = c;
}

size_t decode2d_workspace_bytes(const lla_desc& desc, int B, int splits, int d_rope) {
  const size_t bh = static_cast<size_t>(B) * desc.H;
  return align256(bh * (desc.r_k + d_rope) * 4) + align256(bh * 4) + bh * splits * (2 + desc.r_v) * 4;
}

hipError_t launch_decode2d(const DecodeParams& p, int dtype, hipStream_t stream) {
  const Entry2d* e = find2d(p.r_k, p.r_v);
  const int ri = rope_index(p.d_rope);
  if (e == nullptr || p.d > 128 || ri < 0) return hipErrorNotSupported;
  const bool low = dtype == LLA_BF16_Q8 || dtype == LLA_BF16_I8;
  if (low && p.d_rope != 0) return hipErrorNotSupported;  // low-bit rows: no rotary branch here
  // splits and chunk were planned by the caller with decode2d_plan
  lla_desc d{};
  d.H = p.H;
  d.r_k = p.r_k;
  d.r_v = p.r_v;
  if (p.splits < 1 || p.splits > 64 || decode2d_workspace_bytes(d, p.B, p.splits, p.d_rope) > p.ws_bytes)
    return hipErrorInvalidValue;  // the plan does not fit the workspace: never launch
  const size_t bh = static_cast<size_t>(p.B) * p.H;
  char* ws = reinterpret_cast<char*>(p.ws);
  const size_t qt_bytes = align256(bh * (p.r_k + p.d_rope) * 4);
  float* qt = reinterpret_cast<float*>(ws);
  float* beta = reinterpret_cast<float*>(ws + qt_bytes);
  float* part = reinterpret_cast<float*>(ws + qt_bytes + align256(bh * 4));
  const unsigned qb = (p.B + kQB - 1) / kQB;
  hipLaunchKernelGGL(e->qproj[ri], dim3(p.H * qb), dim3(256), 0, stream, p, qt, beta);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto partial = low ? e->staged[dtype == LLA_BF16_I8 ? 1 : 0] : e->partial[ri];
  hipLaunchKernelGGL(partial, dim3(p.splits * p.B, (p.H + 15) / 16), dim3(64 * Cfg2d<64, 64>::kW), 0,
                     stream, p, qt, beta, part);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(e->combine, dim3(p.H * qb), dim3(256), 0, stream, p, part);
  return hipGetLastError();
}

}  // namespace lla
