// Chunked-prefill attention over the latent cache.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Appendix A ("Decoding and
// caching") describes the latent-store decoder's prefill as two passes: the chunk's per-loop K/V
// are captured and encoded first, and attention then runs against the cache. Here the chunk's
// latents are already in slots ctx .. ctx+C-1, and chunk row j (position ctx + j) attends latents
// 0 .. ctx + j. The arithmetic per row is the absorbed form of Section 7: scores q~ . z^K with
// q~ = W^K_t^T q (plus q . mu^K_t), softmax, latent-space sum of z^V, one W^V_t projection.
//
// MFMA path (bf16 storage, r_k and r_v in {64, 128, 256}, d_head a multiple of 32): a chunk of C
// rows against N_ctx + C latents is a dense contraction, so it runs as two kernels:
//   P0 transpose W^K_t[h] to [r_k][d] so the q~ projection reads 16-byte runs of d;
//   P1 causal flash attention over the latents: a workgroup of 8 waves owns 128 consecutive chunk
//      rows of one head; each wave first forms Q~ = scale*log2(e) * Q . W^K_t[h] of its 16 rows on
//      MFMA (kept as bf16 hi + lo in registers); 32-latent K and V tiles are fetched with buffer
//      LDS-DMA loads into a 4-deep ring of named LDS stages shared by the 8 waves; S^T = Z^K . Q~^T,
//      online softmax per row with a causal mask, then A^T += Z^V^T . P^T on
//      v_mfma_f32_16x16x32_bf16 with P taken straight from the S^T accumulators (two 16-key halves
//      form one K=32 step) and Z^V^T read with the transposing ds_read_b64_tr_b16; finally
//      O = A . W^V_t[h]^T (+ mu^V_t when the row saw any latent) on MFMA from the accumulators.
//      For r_k = r_v of 128 or 256 without the rotary branch, P1 runs as prefill_attn_ws_kernel:
//      the same arithmetic with score waves and product waves (see there), fewer LDS reads per MFMA.
// LLA-2D and per-head differ only in which latent sequence a head reads (b, or (b, h)) and in the
// factor and mu offsets.
//
// Streaming path (everything else): every (row, head) is one query row of the absorbed split-K
// decode kernels, with its own causal key count.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr float kLazyP = 8.0f;

typedef __attribute__((address_space(3))) short4_t* lds_short4_ptr;

// LDS layout of a V tile (kKeyTile keys x RV latent entries, bf16): 128-byte blocks of 4 keys x 16
// entries, row-major inside the block (16-byte unit = 8 entries of one key, units ordered key,
// half), blocks ordered key quad major. Byte offset of unit (key, 8-entry group r8):
// The entry block index is XORed with the key quad's parity: the two 16-lane groups of a 32-lane
// half of a transposed read take consecutive key quads, whose blocks would otherwise lie a multiple
// of 256 bytes apart, on the same LDS banks.
template <int RV>
__device__ __forceinline__ int v_unit_offset(int key, int r8) {
  constexpr int NRQ = RV / 16;  // entry blocks per key quad
  const int kq = key >> 2;
  return (kq * NRQ + ((r8 >> 1) ^ (kq & 1))) * 128 + ((key & 3) * 2 + (r8 & 1)) * 16;
}

// LDS placement of 16-byte chunk c of K tile row `row` (CPK chunks per row). A K operand read is a
// ds_read_b128 whose 16-lane groups take 16 consecutive rows at one chunk; it touches every LDS bank
// once when those 16 chunks fall in 16 distinct 16-byte slots of a 256-byte bank window: an XOR by
// the row inside 16-chunk windows for rows of >= 256 bytes, and by row / 2 for 128-byte rows.
template <int CPK>
__device__ __forceinline__ int k_chunk_slot(int row, int c) {
  if constexpr (CPK >= 16) return (c & ~15) | ((c & 15) ^ (row & 15));
  else return c ^ ((row >> 1) & 7);
}

// A operand of v_mfma_f32_16x16x16bf16_1k-style 4-key slices holding Z^V^T[r0 + i][kb + 4q + e]
// (16-lane group q, lane i of the group, element e < 4), r0 a multiple of 16, kb a multiple of 4.
// One ds_read_b64_tr_b16: source lane j = 4e + c of group q points at the 8 bytes
// V[kb + 4q + e][r0 + 4c .. + 3]; the transposed read hands lane i element e = V[kb + 4q + e][r0 + i].
// In the blocked layout the 16 source lanes of a group cover one whole 128-byte block in lane
// order, and the four groups cover four blocks of consecutive key quads. (Lane mapping of the
// instruction checked on the hardware.)
template <int RV>
__device__ __forceinline__ short4_t v_operand_tr(const char* vt, int kb, int r0, int lane) {
  const int q = lane >> 4;
  const int j = lane & 15;
  const char* blk = vt + v_unit_offset<RV>(kb + 4 * q, r0 >> 3);  // unit (key quad start, r0)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_ptr)(blk + 8 * j));
}

constexpr int kRowsWG = 128;  // chunk rows per attention workgroup (8 waves x 16)
constexpr int kKeyTile = 32;  // latents per K/V tile

__device__ __forceinline__ floatx4_t mfma32(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace segments of the MFMA path.
struct PrefillWs {
  uint16_t* wkt;   // [H][RK][d]: W^K_t[h] transposed, so the q~ projection reads 16-byte runs of d
};

size_t prefill_mfma_bytes(int B, int C, int H, int d, int rk, int rv) {
  (void)B;
  (void)C;
  (void)rv;
  return align256(static_cast<size_t>(H) * rk * d * 2);
}

PrefillWs carve(void* ws) {
  PrefillWs w;
  w.wkt = static_cast<uint16_t*>(ws);
  return w;
}

// offset of W_t restricted to head h (per-head [T][H][d][r], 2D [T][H*d][r]): (t*H + h)*d*r
__device__ __forceinline__ size_t wofs(const PrefillParams& p, int h, int r) {
  return (static_cast<size_t>(p.t) * p.H + h) * p.d * r;
}
// offset of mu_t restricted to head h (per-head [H][T*d], 2D [T*H*d])
__device__ __forceinline__ size_t mofs(const PrefillParams& p, int h) {
  return p.variant == LLA_2D ? (static_cast<size_t>(p.t) * p.H + h) * p.d
                             : (static_cast<size_t>(h) * p.T + p.t) * p.d;
}

// ---- P0: W^K_t[h] [d][RK] -> [RK][d] ------------------------------------------------------------
// One 32 x 32 tile per workgroup (grid: head, d / 32, RK / 32; d and RK are multiples of 32 on this
// path) through LDS, so the reads run along RK and the writes along d, 8 bytes per thread each.
template <int RK>
__global__ __launch_bounds__(256) void wk_transpose_kernel(PrefillParams p, uint16_t* wkt) {
  __shared__ uint16_t tile[32][32 + 4];
  const int h = blockIdx.x;
  const int j0 = blockIdx.y * 32;
  const int k0 = blockIdx.z * 32;
  const uint16_t* src = static_cast<const uint16_t*>(p.Wk) + wofs(p, h, RK);
  uint16_t* dst = wkt + static_cast<size_t>(h) * RK * p.d;
  const int t = threadIdx.x;
  {
    const int jj = t >> 3, kk = (t & 7) * 4;
    const uint2 v = *reinterpret_cast<const uint2*>(src + static_cast<size_t>(j0 + jj) * RK + k0 + kk);
    tile[jj][kk] = static_cast<uint16_t>(v.x);
    tile[jj][kk + 1] = static_cast<uint16_t>(v.x >> 16);
    tile[jj][kk + 2] = static_cast<uint16_t>(v.y);
    tile[jj][kk + 3] = static_cast<uint16_t>(v.y >> 16);
  }
  __syncthreads();
  {
    const int kk = t >> 3, jj = (t & 7) * 4;
    const uint2 v = make_uint2(tile[jj][kk] | (static_cast<uint32_t>(tile[jj + 1][kk]) << 16),
                               tile[jj + 2][kk] | (static_cast<uint32_t>(tile[jj + 3][kk]) << 16));
    *reinterpret_cast<uint2*>(dst + static_cast<size_t>(k0 + kk) * p.d + j0 + jj) = v;
  }
}

// Epilogue of the attention kernels: O = A . W^V_t[h]^T (+ mu^V_t when the row saw any latent),
// A = D / l, on MFMA as O^T[j][row] = W^V . A^T. The B operand of each 32-wide r chunk comes
// straight from the accumulator layout: lane (row + 16 g) holds r = 16 rt + 4 g + (0..3), so
// elements 0-3 take chunk half rt = 2 ks and elements 4-7 rt = 2 ks + 1 (the order of r inside a
// contraction is free); the A operand, rows j of W^V_t[h], is read in the same order as two 8-byte
// pieces. A is split into bf16 hi + lo parts, like q~.
__device__ __forceinline__ void a_hi_lo(const floatx4_t& d0, const floatx4_t& d1, float inv, uint4& hi,
                                        uint4& lo) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = d0[e] * inv;
    v[4 + e] = d1[e] * inv;
  }
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    hw[e2] = f32x2_to_bf16x2(v[2 * e2], v[2 * e2 + 1]);
    lw[e2] = f32x2_to_bf16x2(v[2 * e2] - bf16_lo(hw[e2]), v[2 * e2 + 1] - bf16_hi(hw[e2]));
  }
  hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

template <int RV>
__device__ __forceinline__ void project_rows(const PrefillParams& p, int h, size_t tok, bool rvalid, float l,
                                             const uint4 (&ahv)[RV / 32], const uint4 (&alv)[RV / 32], int col,
                                             int g) {
  const uint16_t* wv = static_cast<const uint16_t*>(p.Wv) + wofs(p, h, RV);
  const float wr = l > 0.f ? 1.f : 0.f;
  const size_t mo = mofs(p, h);
  uint16_t* orow = static_cast<uint16_t*>(p.out) + (tok * p.H + h) * p.d;
  for (int j0 = 0; j0 < p.d; j0 += 16) {
    // A operand rows: output channel j0 + col
    const uint16_t* wrow_j = wv + static_cast<size_t>(j0 + col) * RV + 4 * g;
    floatx4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RV / 32; ++ks) {
      const uint2 p0 = *reinterpret_cast<const uint2*>(wrow_j + 32 * ks);
      const uint2 p1 = *reinterpret_cast<const uint2*>(wrow_j + 32 * ks + 16);
      const uint4 aw = make_uint4(p0.x, p0.y, p1.x, p1.y);
      o = mfma32(aw, ahv[ks], o);
      o = mfma32(aw, alv[ks], o);
    }
    // C layout: lane (row + 16 g) holds channels j0 + 4 g + (0..3) of its row
    if (rvalid) {
      float r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r4[e] = o[e];
        if (p.mu_v != nullptr) r4[e] += wr * ld<BF16>(p.mu_v, mo + j0 + 4 * g + e);
      }
      *reinterpret_cast<uint2*>(orow + j0 + 4 * g) = make_uint2(f32x2_to_bf16x2(r4[0], r4[1]), f32x2_to_bf16x2(r4[2], r4[3]));
    }
  }
}

// Q~ = scale*log2e * W^K_t[h]^T q of a wave's 16 rows (this lane's row at chunk token `tok`),
// formed on MFMA as Q~^T[k][row] = W^K_t^T . Q^T over d. For each 32-wide k chunk ks two 16x16
// accumulator tiles take the k-values 32 ks + 8 m + (0..3) and 32 ks + 8 m + 4 + (0..3) as their rows
// 4 m + (0..3); lane (row + 16 g) then holds elements g of both, k = 32 ks + 8 g + (0..7): exactly the
// B-operand fragment of the score product. Rows of the transposed W^K are picked in that order.
// q~ is kept as bf16 hi + lo, so scores keep float32 accuracy.
template <int RK>
__device__ __forceinline__ void form_qtilde(const PrefillParams& p, const PrefillWs& w, int h, size_t tok,
                                            int col, int g, uint4 (&qh)[RK / 32], uint4 (&ql)[RK / 32]) {
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (tok * p.H + h) * p.d;
  const uint16_t* wkt = w.wkt + static_cast<size_t>(h) * RK * p.d;
  for (int ks = 0; ks < RK / 32; ++ks) {
    floatx4_t c0 = {0.f, 0.f, 0.f, 0.f};
    floatx4_t c1 = {0.f, 0.f, 0.f, 0.f};
    const int k0 = 32 * ks + 8 * (col >> 2) + (col & 3);  // tile row col of the first tile
    for (int dd = 0; dd < p.d; dd += 32) {
      const uint4 bq = *reinterpret_cast<const uint4*>(qrow + dd + 8 * g);
      const uint4 a0 = *reinterpret_cast<const uint4*>(wkt + static_cast<size_t>(k0) * p.d + dd + 8 * g);
      const uint4 a1 = *reinterpret_cast<const uint4*>(wkt + static_cast<size_t>(k0 + 4) * p.d + dd + 8 * g);
      c0 = mfma32(a0, bq, c0);
      c1 = mfma32(a1, bq, c1);
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = c0[e] * p.scale_log2;
      v[4 + e] = c1[e] * p.scale_log2;
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      hw[e2] = f32x2_to_bf16x2(v[2 * e2], v[2 * e2 + 1]);
      lw[e2] = f32x2_to_bf16x2(v[2 * e2] - bf16_lo(hw[e2]), v[2 * e2 + 1] - bf16_hi(hw[e2]));
    }
    qh[ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    ql[ks] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// Source byte offset, inside a K tile (kKeyTile rows of RK bf16), of the 16 bytes that land in LDS
// slot f (= 64 i + lane of the i-th 1 KiB load): chunk slots are XOR-placed by row (the slot map is
// an involution).
template <int RK>
__device__ __forceinline__ uint32_t k_tile_offset(int f) {
  constexpr int CPK = RK / 8;
  const int row = f / CPK;
  const int pc = f - row * CPK;
  return (row * RK + k_chunk_slot<CPK>(row, pc) * 8) * 2;
}

// Source byte offset, inside a V tile, of LDS unit U of the blocked V layout (see v_unit_offset):
// its (key, 8-entry group).
template <int RV>
__device__ __forceinline__ uint32_t v_tile_offset(int U) {
  constexpr int NRQ = RV / 16;
  const int block = U >> 3;
  const int kq = block / NRQ;
  const int rq = (block - kq * NRQ) ^ (kq & 1);  // inverse of the block XOR of v_unit_offset
  const int key = 4 * kq + ((U >> 1) & 3);
  const int r8 = 2 * rq + (U & 1);
  return (key * RV + r8 * 8) * 2;
}

// ---- P2: causal flash attention over the latents ----------------------------------------------
// 1D grid of RB*H*B workgroups (RB = ceil(C / 128) row blocks), 512 threads; wave w owns chunk
// rows j0 + 16 w .. + 15. Workgroups are dispatched round-robin over the 8 XCDs; when B is a
// multiple of 8 the id is remapped so that every workgroup of one sequence runs on the same XCD
// and its latents are shared through that XCD's L2.
// K/V tiles go through a kStages-deep LDS ring: tile i+kStages-1 is fetched while tile i is
// computed, one barrier per tile. Every wave issues the same number of loads per tile (small tiles
// repeat an instruction on two waves, writing identical bytes), so the vmcnt thresholds are
// compile-time constants. Each stage is its own __shared__ object and the tile loop is unrolled
// by the ring depth, so every LDS access names its stage statically: the compiler can then tell
// the stage being read from the stages still being filled by global_load_lds, and does not add a
// wait for all outstanding loads before each tile's first LDS read (it cannot prove that for
// offsets into one array). The explicit vmcnt waits below are what orders the ring.
constexpr int kStages = 4;

template <int N>
struct StageIdx {
  static constexpr int value = N;
};

template <int N>
__device__ __forceinline__ void wait_vm_tiles(int ahead) {
  // vmcnt(ahead * N) for ahead in 0..kStages-1, N loads per tile and wave
  switch (ahead) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14)); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0f70 | ((2 * N) & 15) | (((2 * N) >> 4) << 14)); break;
    default: __builtin_amdgcn_s_waitcnt(0x0f70 | ((3 * N) & 15) | (((3 * N) >> 4) << 14)); break;
  }
}

// DR > 0: the decoupled rotary branch. Each key also has a DR-wide rotary key (shared by heads,
// rotated at its slot) in a third tile per ring stage, each row a rotary query rotated at the row's
// position; KR = DR / 32 more contraction steps add q_r . k_r to the score accumulators.
template <int RK, int RV, int DR = 0>
__global__ __launch_bounds__(512) void prefill_attn_kernel(PrefillParams p, PrefillWs w) {
  constexpr int KS = RK / 32;
  constexpr int KR = DR / 32;
  constexpr int CPR = DR / 8;                 // 16-byte chunks per rotary row
  constexpr int RR_BYTES = DR > 0 ? kKeyTile * DR * 2 : 1024;
  constexpr int IR = RR_BYTES / 1024;
  constexpr int LR = DR > 0 ? (IR >= 8 ? IR / 8 : 1) : 0;  // rotary loads per wave and tile
  static_assert(DR == 0 || DR == 64 || DR == 128, "rotary rows of 8 or 16 chunks");
  constexpr int RT = RV / 16;
  constexpr int CPK = RK / 8;                 // 16-byte chunks per K row
  constexpr int NRQ = RV / 16;                // 16-entry blocks per key quad of a V tile
  constexpr int KT_BYTES = kKeyTile * RK * 2;
  constexpr int VT_BYTES = kKeyTile * RV * 2;
  constexpr int IK = KT_BYTES / 1024;         // 1 KiB global_load_lds instructions per K tile
  constexpr int IV = VT_BYTES / 1024;
  constexpr int LK = IK >= 8 ? IK / 8 : 1;    // K loads per wave and tile
  constexpr int LV = IV >= 8 ? IV / 8 : 1;
  static_assert(RK % 64 == 0 && RV % 64 == 0, "swizzle windows need 8 chunks per row");
  static_assert(IK % 8 == 0 || 8 % IK == 0, "K tile instructions spread evenly over 8 waves");
  static_assert(IV % 8 == 0 || 8 % IV == 0, "V tile instructions spread evenly over 8 waves");
  static_assert(3 * (LK + LV + LR) < 64, "vmcnt range");
  // one __shared__ object per ring stage, always named statically (see StageIdx)
  __shared__ __attribute__((aligned(16))) char kb0[KT_BYTES], kb1[KT_BYTES], kb2[KT_BYTES], kb3[KT_BYTES];
  __shared__ __attribute__((aligned(16))) char vb0[VT_BYTES], vb1[VT_BYTES], vb2[VT_BYTES], vb3[VT_BYTES];
  __shared__ __attribute__((aligned(16))) char rb0[DR > 0 ? RR_BYTES : 16], rb1[DR > 0 ? RR_BYTES : 16],
      rb2[DR > 0 ? RR_BYTES : 16], rb3[DR > 0 ? RR_BYTES : 16];
  static_assert(kStages == 4, "four named stages");
  auto kstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return kb0; else if constexpr (st == 1) return kb1;
    else if constexpr (st == 2) return kb2; else return kb3;
  };
  auto vstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return vb0; else if constexpr (st == 1) return vb1;
    else if constexpr (st == 2) return vb2; else return vb3;
  };
  auto rstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return rb0; else if constexpr (st == 1) return rb1;
    else if constexpr (st == 2) return rb2; else return rb3;
  };

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int RB = (p.C + kRowsWG - 1) / kRowsWG;
  const int NB = RB * p.H;                    // workgroups per sequence
  int b, k;
  if ((p.B & 7) == 0) {
    const int P = blockIdx.x;
    const int rest = P >> 3;
    k = rest % NB;
    b = (rest / NB) * 8 + (P & 7);
  } else {
    b = blockIdx.x / NB;
    k = blockIdx.x - b * NB;
  }
  const int h = k / RB;
  const int j0 = (k - h * RB) * kRowsWG;
  const int ctx = uniform(p.ctx_lens[b]);

  // this lane's query row (for scores and accumulators): chunk row jr
  const int jr = j0 + wave * 16 + col;
  const bool rvalid = jr < p.C;
  const int lim = rvalid ? min(ctx + jr, p.n_max - 1) : -1;  // last visible latent (inclusive)
  // last latent any row of this workgroup sees
  const int j_last = min(j0 + kRowsWG, p.C) - 1;
  const int kmax = min(ctx + j_last, p.n_max - 1);
  const int ntiles = kmax >= 0 ? kmax / kKeyTile + 1 : 0;

  const size_t lat = p.variant == LLA_2D ? static_cast<size_t>(b) * p.n_max
                                         : (static_cast<size_t>(b) * p.H + h) * p.n_max;
  const char* zk = static_cast<const char*>(p.zk) + lat * RK * 2;
  const char* zv = static_cast<const char*>(p.zv) + lat * RV * 2;

  // q~ of this wave's 16 rows (form_qtilde). The mu^K_t part of every score of a row,
  // scale*log2e * q . mu^K_t, is one constant per row: softmax does not depend on it and this path
  // returns no log-sum-exp, so it is never formed.
  const size_t tok = static_cast<size_t>(b) * p.C + (rvalid ? jr : 0);  // (b, chunk row) of this lane
  uint4 qh[KS], ql[KS];
  form_qtilde<RK>(p, w, h, tok, col, g, qh, ql);
  // Rotary query fragments (B operand of the extra steps, same element order as the rotary tile's
  // chunks): lane (row, g) holds channels 32 kr + 8 g .. + 7 of the row's rotary query, rotated at
  // the row's position ctx + jr (float64 angles), times scale*log2e, as bf16 hi + lo.
  uint4 qrh[KR > 0 ? KR : 1], qrl[KR > 0 ? KR : 1];
  if constexpr (DR > 0) {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + (tok * p.H + h) * DR;
    const double pos = static_cast<double>(ctx) + (rvalid ? jr : 0);
#pragma unroll
    for (int kr = 0; kr < KR; ++kr) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qr + 32 * kr + 8 * g);
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int i = 16 * kr + 4 * g + e2;  // channel pair (2i, 2i + 1)
        const double theta = pow(p.rope_base, -2.0 * i / DR);
        double sn, cs;
        sincos(pos * theta, &sn, &cs);
        const float x0 = bf16_lo(rw[e2]), x1 = bf16_hi(rw[e2]);
        const float y0 = static_cast<float>(x0 * cs - x1 * sn) * p.scale_log2;
        const float y1 = static_cast<float>(x0 * sn + x1 * cs) * p.scale_log2;
        hw[e2] = f32x2_to_bf16x2(y0, y1);
        lw[e2] = f32x2_to_bf16x2(y0 - bf16_lo(hw[e2]), y1 - bf16_hi(hw[e2]));
      }
      qrh[kr] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      qrl[kr] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }

  // Cooperative tile fetch into ring stage (kd, vd) as buffer loads over this sequence's latents
  // 0 .. kmax: each lane's byte offset inside a tile is fixed, the tile's position moves in the
  // wave-uniform offset, and latents past kmax (the tail of the last tile, the spare fetches past
  // the end) land as zeros. Keys past a row's limit are masked, so those zeros are never weighed.
  const int kbytes = (kmax + 1) * RK * 2;
  const int vbytes = (kmax + 1) * RV * 2;
  const int rbytes = (kmax + 1) * DR * 2;
  const char* zr = DR > 0 ? static_cast<const char*>(p.k_rope) + static_cast<size_t>(b) * p.n_max * DR * 2
                          : nullptr;
  uint32_t koff[LK], voff[LV], roff[LR > 0 ? LR : 1];
#pragma unroll
  for (int u = 0; u < LR; ++u) {
    const int i = IR >= 8 ? wave + 8 * u : wave % IR;
    const int f = i * 64 + lane;
    const int row = f / CPR;
    const int pc = f - row * CPR;
    roff[u] = (row * DR + k_chunk_slot<CPR>(row, pc) * 8) * 2;
  }
#pragma unroll
  for (int u = 0; u < LK; ++u) koff[u] = k_tile_offset<RK>((IK >= 8 ? wave + 8 * u : wave % IK) * 64 + lane);
#pragma unroll
  for (int u = 0; u < LV; ++u) voff[u] = v_tile_offset<RV>((IV >= 8 ? wave + 8 * u : wave % IV) * 64 + lane);
  auto issue = [&](int tile, char* kd, char* vd, char* rd) {
    const uint32_t key0 = tile * kKeyTile;
#pragma unroll
    for (int u = 0; u < LR; ++u) {
      const int i = IR >= 8 ? wave + 8 * u : wave % IR;
      buffer_lds16(zr, rbytes, (lptr_t)(rd + i * 1024), roff[u], key0 * DR * 2);
    }
#pragma unroll
    for (int u = 0; u < LK; ++u) {
      const int i = IK >= 8 ? wave + 8 * u : wave % IK;
      buffer_lds16(zk, kbytes, (lptr_t)(kd + i * 1024), koff[u], key0 * RK * 2);
    }
#pragma unroll
    for (int u = 0; u < LV; ++u) {
      const int i = IV >= 8 ? wave + 8 * u : wave % IV;
      buffer_lds16(zv, vbytes, (lptr_t)(vd + i * 1024), voff[u], key0 * RV * 2);
    }
  };

  floatx4_t D[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) D[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // Running maximum m of this row's scores (q~ . z in log2 units), kept as the offset bm = -m that
  // the score accumulators start from, so that they hold score - m directly. m starts at 0 and is
  // re-based on the first tile that shows the row any latent, whatever that tile's maximum; after
  // that only when the maximum grows by more than kLazyP. Until the first re-base every weight is
  // exp2(-inf) = 0, so l and D are still exactly 0 and need no rescale then.
  float bm = 0.f;
  bool based = false;
  float l = 0.f;
  // The wave's rows are j0 + 16 wave + (0 .. 15). When all of them are inside the chunk, the
  // smallest causal limit is that of the first row, and a tile wholly at or below it needs no mask.
  const int jw = j0 + wave * 16;
  const int wave_lim = (jw + 15 < p.C) ? min(ctx + jw, p.n_max - 1) : -1;

  // Tile `tile` lives in stage tile % kStages. The ring runs without conditions: the prologue
  // fetches three tiles, every step fetches tile + 3, and the loop runs whole groups of four steps
  // (rows past kmax are clamped, so fetches past the last tile re-read valid latents, and the
  // spare steps see only keys above every row's causal limit: their weights are 0). With no
  // conditional transfers the compiler can follow which stage each outstanding load fills and
  // adds no waits of its own; the explicit ones below keep exactly two tiles in flight.
  auto step = [&](auto S, int tile) {
    constexpr int st = decltype(S)::value;
    // this wave's loads of `tile` have landed (tiles + 1 and + 2 may still be in flight) ...
    wait_vm_tiles<LK + LV + LR>(kStages - 2);
    // ... and every other wave's; everyone has also finished computing tile - 1, whose stage is
    // refilled once this tile's score MFMAs are issued (requested right after the barrier, the
    // transfers contend with the score phase's K reads: 2-3% slower at r = 256)
    lds_barrier();  // (lla_device.h) not a full fence: later stages stay in flight
    const char* kt = kstage(S);
    const char* rt_ = rstage(S);
    const char* vt = vstage(S);
    const int key0 = tile * kKeyTile;
    float sc[2][4];
    float tmax = kNegInf;
    const bool masked = key0 + kKeyTile - 1 > wave_lim;  // wave-uniform
#pragma unroll
    for (int kt16 = 0; kt16 < 2; ++kt16) {
      // S^T[key 16*kt16 + i][row] - m: A = K rows (chunks at their slots), B = Q~^T fragments
      const int row = 16 * kt16 + col;
      // the hi and lo parts of q~ accumulate into one fp32 accumulator (one add fewer per score
      // than two chains summed at the end: 13.4 -> 12.3 ms per loop at r = 256)
      floatx4_t sh = {bm, bm, bm, bm};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 4 * ks + g;
        const int pc = k_chunk_slot<CPK>(row, c);
        const uint4 a = *reinterpret_cast<const uint4*>(kt + row * RK * 2 + pc * 16);
        sh = mfma32(a, qh[ks], sh);
        sh = mfma32(a, ql[ks], sh);
      }
#pragma unroll
      for (int kr = 0; kr < KR; ++kr) {
        const int pc = k_chunk_slot<CPR>(row, 4 * kr + g);
        const uint4 a = *reinterpret_cast<const uint4*>(rt_ + row * DR * 2 + pc * 16);
        sh = mfma32(a, qrh[kr], sh);
        sh = mfma32(a, qrl[kr], sh);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[kt16][e] = sh[e];
      if (masked) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key0 + 16 * kt16 + 4 * g + e > lim) sc[kt16][e] = kNegInf;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sc[kt16][e]);
    }
    issue(tile + kStages - 1, kstage(StageIdx<(st + kStages - 1) % kStages>{}),
          vstage(StageIdx<(st + kStages - 1) % kStages>{}),
          rstage(StageIdx<(st + kStages - 1) % kStages>{}));
    tmax = max_over_groups(tmax);
    if (tmax > kLazyP || (!based && tmax > kNegInf)) {
      if (based) {
        const float c = fast_exp2(-tmax);
        l *= c;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) D[rt] *= c;
      }
      based = true;
      bm -= tmax;
#pragma unroll
      for (int kt16 = 0; kt16 < 2; ++kt16)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kt16][e] -= tmax;
    }
    // P^T as the B operand of one K=32 step: the order of keys inside a contraction is free, so
    // lane group g's 8 entries are keys 4g .. 4g+3 (elements 0-3) and 16+4g .. 16+4g+3 (4-7),
    // exactly what the S^T accumulators hold; the A operand takes the same key order from two
    // transposed reads of the 16-key halves.
    float pe[2][4];
#pragma unroll
    for (int kt16 = 0; kt16 < 2; ++kt16)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[kt16][e] = fast_exp2(sc[kt16][e]);  // exp2(-inf) = 0 for masked keys
        l += pe[kt16][e];
      }
    const bf16x8_t pb = __builtin_bit_cast(
        bf16x8_t, make_uint4(f32x2_to_bf16x2(pe[0][0], pe[0][1]), f32x2_to_bf16x2(pe[0][2], pe[0][3]),
                             f32x2_to_bf16x2(pe[1][0], pe[1][1]), f32x2_to_bf16x2(pe[1][2], pe[1][3])));
    // the rotary fragments leave no room to hoist the P.V operand reads into the score phase
    if constexpr (DR > 0) __builtin_amdgcn_sched_barrier(0);
    // A^T[r][row] += Z^V^T[r][keys] . P^T
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const short4_t v0 = v_operand_tr<RV>(vt, 0, 16 * rt, lane);
      const short4_t v1 = v_operand_tr<RV>(vt, 16, 16 * rt, lane);
      D[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7)), pb, D[rt], 0, 0, 0);
    }
  };
  if (ntiles > 0) {
    // the Q~ loads land before any tile is requested, so the tile loop never has to
    // wait for them
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    issue(0, kb0, vb0, rb0);
    issue(1, kb1, vb1, rb1);
    issue(2, kb2, vb2, rb2);
    for (int tile = 0; tile < ntiles; tile += kStages) {
      step(StageIdx<0>{}, tile);
      step(StageIdx<1>{}, tile + 1);
      step(StageIdx<2>{}, tile + 2);
      step(StageIdx<3>{}, tile + 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the spare fetches have landed before the wave ends
  }
  l = sum_over_groups(l);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint4 ahv[RT / 2], alv[RT / 2];
#pragma unroll
  for (int ks = 0; ks < RT / 2; ++ks) a_hi_lo(D[2 * ks], D[2 * ks + 1], inv, ahv[ks], alv[ks]);
  project_rows<RV>(p, h, tok, rvalid, l, ahv, alv, col, g);
}
// ---- P2w: the attention kernel with specialised waves (r_k = r_v, no rotary branch) -----------
// Same workgroup rows (128 chunk rows of one head), tiles, scores, softmax and epilogue as
// prefill_attn_kernel (and the same results, bit for bit), with 16 waves in two roles:
//   * score waves 0..7 own rows j0 + 16 w .. + 15 as before, q~ in registers: at step t they form
//     the scores of tile t, the online softmax, and P^T(t) (the bf16 B-operand fragments) with each
//     row's accumulator rescale factor in a double-buffered LDS slot;
//   * product waves 8..15 own 64 rows (half p / 4) x RV / 4 latent entries (quarter p % 4,
//     p = w - 8): at step t they rescale and accumulate A^T += Z^V^T(t - 1) . P^T(t - 1) for four
//     row blocks, so each transposed V read feeds four MFMAs instead of one (the single-role kernel
//     reads a whole V tile per 16 rows). They also issue every tile load.
// Ring (4 stages each): at step t the score waves read K(t) (stage t % 4), the product waves read
// V(t - 1) (stage (t + 3) % 4), and K(t + 3) and V(t + 2) are requested into the stages read at
// step t - 1; the loads issued at step t - 3 have landed at step t. Four waves per SIMD, two of each
// role. At the end the product waves hand A over through the eight ring stages (one 64-row x RV / 4
// piece per stage, in the accumulator layout) and the score waves run the projection.
template <int RK, int RV>
__global__ __launch_bounds__(1024) void prefill_attn_ws_kernel(PrefillParams p, PrefillWs w) {
  static_assert(RK == RV, "the A hand-off fills the eight ring stages exactly");
  constexpr int KS = RK / 32;
  constexpr int RT = RV / 16;
  constexpr int RQ = RT / 4;                  // 16-entry blocks per product wave
  constexpr int CPK = RK / 8;
  constexpr int NRQ = RV / 16;
  constexpr int KT_BYTES = kKeyTile * RK * 2;
  constexpr int VT_BYTES = kKeyTile * RV * 2;
  constexpr int IK = KT_BYTES / 1024;
  constexpr int IV = VT_BYTES / 1024;
  constexpr int LK = IK >= 8 ? IK / 8 : 1;    // loads per product wave and tile
  constexpr int LV = IV >= 8 ? IV / 8 : 1;
  static_assert(RQ >= 1 && 4 * RQ * 64 * 16 == KT_BYTES, "one 64-row A piece per ring stage");
  static_assert(IK % 8 == 0 || 8 % IK == 0, "K tile instructions spread evenly over 8 waves");
  static_assert(IV % 8 == 0 || 8 % IV == 0, "V tile instructions spread evenly over 8 waves");
  static_assert(3 * (LK + LV) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char kb0[KT_BYTES], kb1[KT_BYTES], kb2[KT_BYTES], kb3[KT_BYTES];
  __shared__ __attribute__((aligned(16))) char vb0[VT_BYTES], vb1[VT_BYTES], vb2[VT_BYTES], vb3[VT_BYTES];
  __shared__ uint4 pt_s[2][8][64];    // P^T fragments of the 8 row blocks, by step parity
  __shared__ float cf_s[2][kRowsWG];  // accumulator rescale factor of each row, by step parity
  auto kstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return kb0; else if constexpr (st == 1) return kb1;
    else if constexpr (st == 2) return kb2; else return kb3;
  };
  auto vstage = [&](auto S) -> char* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return vb0; else if constexpr (st == 1) return vb1;
    else if constexpr (st == 2) return vb2; else return vb3;
  };
  // ring stage o of the A hand-off: 0..3 the K stages, 4..7 the V stages
  auto stage_obj = [&](int o) -> char* {
    return o == 0 ? kb0 : o == 1 ? kb1 : o == 2 ? kb2 : o == 3 ? kb3
         : o == 4 ? vb0 : o == 5 ? vb1 : o == 6 ? vb2 : vb3;
  };

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const bool scorer = wave < 8;
  const int RB = (p.C + kRowsWG - 1) / kRowsWG;
  const int NB = RB * p.H;
  int b, k;
  if ((p.B & 7) == 0) {
    const int P = blockIdx.x;
    const int rest = P >> 3;
    k = rest % NB;
    b = (rest / NB) * 8 + (P & 7);
  } else {
    b = blockIdx.x / NB;
    k = blockIdx.x - b * NB;
  }
  const int h = k / RB;
  const int j0 = (k - h * RB) * kRowsWG;
  const int ctx = uniform(p.ctx_lens[b]);
  const int j_last = min(j0 + kRowsWG, p.C) - 1;
  const int kmax = min(ctx + j_last, p.n_max - 1);
  const int ntiles = kmax >= 0 ? kmax / kKeyTile + 1 : 0;

  const size_t lat = p.variant == LLA_2D ? static_cast<size_t>(b) * p.n_max
                                         : (static_cast<size_t>(b) * p.H + h) * p.n_max;
  const char* zk = static_cast<const char*>(p.zk) + lat * RK * 2;
  const char* zv = static_cast<const char*>(p.zv) + lat * RV * 2;

  // step 0's products read the odd slot: P^T(-1) = 0 with factors 1 (published by step 0's barrier)
  for (int i = tid; i < 8 * 64; i += 1024) pt_s[1][i >> 6][i & 63] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < kRowsWG; i += 1024) cf_s[1][i] = 1.f;

  if (scorer) {
    // ---- score wave: chunk row jr of this lane (row block sw)
    const int sw = wave;
    const int jr = j0 + sw * 16 + col;
    const bool rvalid = jr < p.C;
    const int lim = rvalid ? min(ctx + jr, p.n_max - 1) : -1;
    const size_t tok = static_cast<size_t>(b) * p.C + (rvalid ? jr : 0);
    const int jw = j0 + sw * 16;
    const int wave_lim = (jw + 15 < p.C) ? min(ctx + jw, p.n_max - 1) : -1;
    uint4 qh[KS], ql[KS];
    form_qtilde<RK>(p, w, h, tok, col, g, qh, ql);
    // running maximum of the row as the accumulators' starting offset (see prefill_attn_kernel)
    float bm = 0.f;
    bool based = false;
    float l = 0.f;
    auto score_step = [&](auto S, int t) {
      constexpr int st = decltype(S)::value;
      lds_barrier();  // K(t) has landed; P^T(t - 2)'s slot has been read
      const char* kt = kstage(S);
      const int key0 = t * kKeyTile;
      float sc[2][4];
      float tmax = kNegInf;
      const bool masked = key0 + kKeyTile - 1 > wave_lim;  // wave-uniform
#pragma unroll
      for (int kt16 = 0; kt16 < 2; ++kt16) {
        const int row = 16 * kt16 + col;
        floatx4_t sh = {bm, bm, bm, bm};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int pc = k_chunk_slot<CPK>(row, 4 * ks + g);
          const uint4 a = *reinterpret_cast<const uint4*>(kt + row * RK * 2 + pc * 16);
          sh = mfma32(a, qh[ks], sh);
          sh = mfma32(a, ql[ks], sh);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kt16][e] = sh[e];
        if (masked) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key0 + 16 * kt16 + 4 * g + e > lim) sc[kt16][e] = kNegInf;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sc[kt16][e]);
      }
      tmax = max_over_groups(tmax);
      float c = 1.f;
      if (tmax > kLazyP || (!based && tmax > kNegInf)) {
        if (based) {
          c = fast_exp2(-tmax);
          l *= c;
        }
        based = true;
        bm -= tmax;
#pragma unroll
        for (int kt16 = 0; kt16 < 2; ++kt16)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[kt16][e] -= tmax;
      }
      float pe[2][4];
#pragma unroll
      for (int kt16 = 0; kt16 < 2; ++kt16)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[kt16][e] = fast_exp2(sc[kt16][e]);
          l += pe[kt16][e];
        }
      pt_s[st & 1][sw][lane] =
          make_uint4(f32x2_to_bf16x2(pe[0][0], pe[0][1]), f32x2_to_bf16x2(pe[0][2], pe[0][3]),
                     f32x2_to_bf16x2(pe[1][0], pe[1][1]), f32x2_to_bf16x2(pe[1][2], pe[1][3]));
      if (g == 0) cf_s[st & 1][sw * 16 + col] = c;
    };
    // one step more than the tiles (the product waves finish the last tile there), in whole
    // groups of four; both roles pass the same barriers
    if (ntiles > 0) {
      for (int t = 0; t <= ntiles; t += kStages) {
        score_step(StageIdx<0>{}, t);
        score_step(StageIdx<1>{}, t + 1);
        score_step(StageIdx<2>{}, t + 2);
        score_step(StageIdx<3>{}, t + 3);
      }
    }
    __syncthreads();  // the product waves are past the ring
    __syncthreads();  // A is in the ring stages
    l = sum_over_groups(l);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint4 ahv[RT / 2], alv[RT / 2];
#pragma unroll
    for (int ks = 0; ks < RT / 2; ++ks) {
      floatx4_t d2[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int rt = 2 * ks + v;
        const char* src = stage_obj(2 * (rt / RQ) + (sw >> 2));
        d2[v] = *reinterpret_cast<const floatx4_t*>(src + (((sw & 3) * RQ + rt % RQ) * 64 + lane) * 16);
      }
      a_hi_lo(d2[0], d2[1], inv, ahv[ks], alv[ks]);
    }
    project_rows<RV>(p, h, tok, rvalid, l, ahv, alv, col, g);
    return;
  }

  const int sw = wave - 8;  // product wave index: its load share
  // ---- product wave: rows 64 half .. + 63, latent entries 16 RQ quarter ..
  const int half = sw >> 2;
  const int quarter = sw & 3;
  const int kbytes = (kmax + 1) * RK * 2;
  const int vbytes = (kmax + 1) * RV * 2;
  uint32_t koff[LK], voff[LV];
#pragma unroll
  for (int u = 0; u < LK; ++u) koff[u] = k_tile_offset<RK>((IK >= 8 ? sw + 8 * u : sw % IK) * 64 + lane);
#pragma unroll
  for (int u = 0; u < LV; ++u) voff[u] = v_tile_offset<RV>((IV >= 8 ? sw + 8 * u : sw % IV) * 64 + lane);
  // K tile tk into kd, V tile tv into vd (tiles past kmax read as zeros)
  auto issue_k = [&](int tk, char* kd) {
#pragma unroll
    for (int u = 0; u < LK; ++u) {
      const int i = IK >= 8 ? sw + 8 * u : sw % IK;
      buffer_lds16(zk, kbytes, (lptr_t)(kd + i * 1024), koff[u], tk * kKeyTile * RK * 2);
    }
  };
  auto issue_v = [&](int tv, char* vd) {
#pragma unroll
    for (int u = 0; u < LV; ++u) {
      const int i = IV >= 8 ? sw + 8 * u : sw % IV;
      buffer_lds16(zv, vbytes, (lptr_t)(vd + i * 1024), voff[u], tv * kKeyTile * RV * 2);
    }
  };
  // lane offsets of the transposed V reads inside a stage (keys 0-15; keys 16-31 sit 4 NRQ 128-byte
  // blocks further); they pass through opaque() at every step so the compiler forms each stage's
  // addresses where they are used instead of keeping all of them live across the loop
  int vlo[RQ];
#pragma unroll
  for (int j = 0; j < RQ; ++j) vlo[j] = v_unit_offset<RV>(4 * g, 2 * (RQ * quarter + j)) + 8 * col;
  floatx4_t D[4][RQ];  // row block 4 half + i, latent block RQ quarter + j
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < RQ; ++j) D[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  auto product_step = [&](auto S, int t) {
    constexpr int st = decltype(S)::value;
    // this wave's loads of K(t) and V(t - 1) (step t - 3) have landed; the barrier publishes
    // everyone's, and P^T(t - 1), and frees the stages read at step t - 1
    wait_vm_tiles<LK + LV>(kStages - 2);
    lds_barrier();
    issue_k(t + kStages - 1, kstage(StageIdx<(st + kStages - 1) % kStages>{}));
    issue_v(t + kStages - 2, vstage(StageIdx<(st + kStages - 2) % kStages>{}));
    // A^T += Z^V^T(t - 1) . P^T(t - 1) for the four row blocks (P^T(-1) = 0, factors 1)
    const char* vt = vstage(StageIdx<(st + kStages - 1) % kStages>{});
    uint4 pb[4];
    float cv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = pt_s[(st + 1) & 1][4 * half + i][lane];
      cv[i] = cf_s[(st + 1) & 1][(4 * half + i) * 16 + col];
    }
    const bool rescale = cv[0] != 1.f || cv[1] != 1.f || cv[2] != 1.f || cv[3] != 1.f;
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < RQ; ++j) D[i][j] *= cv[i];
    }
#pragma unroll
    for (int j = 0; j < RQ; ++j) {
      // v_operand_tr<RV>(vt, 0 / 16, 16 (RQ quarter + j), lane), with the lane offset precomputed
      const char* va = vt + opaque(vlo[j]);
      const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_ptr)va);
      const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_ptr)(va + 4 * NRQ * 128));
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        D[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, pb[i]), D[i][j], 0, 0, 0);
      // one V block at a time: hoisting every block's reads ran the wave out of registers, and the
      // spilled load offsets were then reloaded (and waited for) at every step
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (ntiles > 0) {
    // the loads of steps -3 .. -1: K(0..2) with V(-1..1) (V(-1) a placeholder never read)
    issue_k(0, kb0);
    issue_v(0, vb3);
    issue_k(1, kb1);
    issue_v(0, vb0);
    issue_k(2, kb2);
    issue_v(1, vb1);
    for (int t = 0; t <= ntiles; t += kStages) {
      product_step(StageIdx<0>{}, t);
      product_step(StageIdx<1>{}, t + 1);
      product_step(StageIdx<2>{}, t + 2);
      product_step(StageIdx<3>{}, t + 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the spare fetches have landed
  }
  __syncthreads();  // every wave is past its last ring read
  // hand A over: row half `half` of quarter `quarter` goes to ring stage 2 quarter + half, in the
  // accumulator layout
  char* dst = stage_obj(2 * quarter + half);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < RQ; ++j) *reinterpret_cast<floatx4_t*>(dst + ((i * RQ + j) * 64 + lane) * 16) = D[i][j];
  __syncthreads();
}

struct EntryP {
  int r_k, r_v;
  void (*wkt)(PrefillParams, uint16_t*);
  void (*attn)(PrefillParams, PrefillWs);
  void (*attn_r64)(PrefillParams, PrefillWs);   // with a 64-wide rotary branch
  void (*attn_r128)(PrefillParams, PrefillWs);  // with a 128-wide rotary branch
  void (*attn_ws)(PrefillParams, PrefillWs);    // specialised waves (r_k = r_v, no rotary branch)
};

// the specialised-wave kernel where it is faster: r_k = r_v of 128 and 256 (10.2-10.8 vs 11.9-12.2 ms
// per LLA-2D loop at 256, 6.5-6.6 vs 7.2-7.3 at 128); at 64 the single-role kernel is (3.5 vs 4.9)
template <int RK, int RV>
constexpr void (*ws_kernel())(PrefillParams, PrefillWs) {
  if constexpr (RK == RV && RK >= 128) return prefill_attn_ws_kernel<RK, RV>;
  else return nullptr;
}

template <int RK, int RV>
constexpr EntryP entryP() {
  return {RK, RV, wk_transpose_kernel<RK>, prefill_attn_kernel<RK, RV>,
          prefill_attn_kernel<RK, RV, 64>, prefill_attn_kernel<RK, RV, 128>, ws_kernel<RK, RV>()};
}

const EntryP kTableP[] = {
    entryP<64, 64>(), entryP<128, 128>(), entryP<256, 256>(), entryP<64, 128>(), entryP<128, 256>(),
};

const EntryP* findP(int r_k, int r_v) {
  for (const EntryP& e : kTableP)
    if (e.r_k == r_k && e.r_v == r_v) return &e;
  return nullptr;
}

// The MFMA path fetches a sequence's latents through buffer descriptors with a 31-bit byte range.
bool mfma_prefill(int dtype, int r_k, int r_v, int d_head, int n_max) {
  return dtype == LLA_BF16 && d_head % 32 == 0 && findP(r_k, r_v) != nullptr &&
         static_cast<long>(n_max) * (r_k > r_v ? r_k : r_v) * 2 < 0x7fffffffL;
}

}  // namespace

// MFMA path: d_rope 64 or 128; streaming path (pairs without the MFMA prefill): the streaming
// read's rotary instances, each causal row a query with its own key count and position
bool prefill_rope_supported(const lla_desc& desc, int d_rope) {
  if (static_cast<long>(desc.n_max) * d_rope * 2 >= 0x7fffffffL) return false;
  if (mfma_prefill(desc.dtype, desc.r_k, desc.r_v, desc.d_head, desc.n_max))
    return d_rope == 64 || d_rope == 128;
  return rope_valu_supported(desc.dtype, desc.r_k, desc.r_v, d_rope);
}

bool prefill_supported(int variant, int dtype, int r_k, int r_v) {
  return valu_supported(variant, dtype, r_k, r_v) || (dtype == LLA_BF16 && findP(r_k, r_v) != nullptr);
}

void prefill_plan(const lla_desc& desc, int B, int C, int* splits, int* chunk, int* wg_waves) {
  if (mfma_prefill(desc.dtype, desc.r_k, desc.r_v, desc.d_head, desc.n_max)) {
    *splits = 1;
    *chunk = desc.n_max;
    if (wg_waves != nullptr) *wg_waves = 1;
    return;
  }
  valu_plan(desc, B * C, splits, chunk, wg_waves);
}

size_t prefill_workspace_bytes(const lla_desc& desc, int B, int C) {
  if (mfma_prefill(desc.dtype, desc.r_k, desc.r_v, desc.d_head, desc.n_max))
    return prefill_mfma_bytes(B, C, desc.H, desc.d_head, desc.r_k, desc.r_v);
  int s, c, nw;
  prefill_plan(desc, B, C, &s, &c, &nw);  // the plan the call runs
  return valu_workspace_bytes(desc, B * C, s);
}

hipError_t launch_prefill(const PrefillParams& pp, int dtype, hipStream_t stream) {
  if (mfma_prefill(dtype, pp.r_k, pp.r_v, pp.d, pp.n_max)) {
    const EntryP* e = findP(pp.r_k, pp.r_v);
    if (prefill_mfma_bytes(pp.B, pp.C, pp.H, pp.d, pp.r_k, pp.r_v) > pp.ws_bytes)
      return hipErrorInvalidValue;  // the plan does not fit the workspace: never launch
    const PrefillWs w = carve(pp.ws);
    hipLaunchKernelGGL(e->wkt, dim3(pp.H, pp.d / 32, pp.r_k / 32), dim3(256), 0, stream, pp, w.wkt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned nwg = static_cast<unsigned>((pp.C + kRowsWG - 1) / kRowsWG) * pp.H * pp.B;
    if (pp.d_rope == 0 && e->attn_ws != nullptr) {
      hipLaunchKernelGGL(e->attn_ws, dim3(nwg), dim3(1024), 0, stream, pp, w);
      return hipGetLastError();
    }
    auto attn = pp.d_rope == 64 ? e->attn_r64 : pp.d_rope == 128 ? e->attn_r128 : e->attn;
    hipLaunchKernelGGL(attn, dim3(nwg), dim3(512), 0, stream, pp, w);
    return hipGetLastError();
  }
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
  p.wg_waves = pp.wg_waves;
  p.ws_bytes = pp.ws_bytes;
  if (pp.d_rope > 0) {  // rotary branch: one wave per head (no head groups), the same plan
    p.q_rope = pp.q_rope;
    p.k_rope = pp.k_rope;
    p.d_rope = pp.d_rope;
    p.rope_base = pp.rope_base;
    return launch_decode_rope(p, dtype, stream);
  }
  return launch_decode(p, dtype, stream);
}

}  // namespace lla
