// Absorbed latent decode attention (per-head LLA, and LLA-2D on the VALU path).
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 3, Eq. 3 rebuilds
// loop t as k_t = W^K_t z^K + mu^K_t (column form). Section 7 ("Per-head LLA versus LLA-2D at
// inference") notes that the score is bilinear, so q . k_t = (W^K_t^T q) . z^K + q . mu^K_t, and
// that sum_i p_i W^V_t z^V_i = W^V_t sum_i p_i z^V_i. The kernels below therefore
//   1. form q~ = scale*log2(e) * W^K_t^T q and beta = scale*log2(e) * q . mu^K_t once per (b, h);
//   2. stream the bf16/fp32 latents of one (b, h, token range) from HBM, one token per LPT lanes,
//      computing base-2 scores q~ . z^K_i + beta with a per-lane online softmax;
//   3. accumulate sum_i 2^(s_i - m) z^V_i in r_v-wide fp32 registers (latent space);
//   4. merge lanes, then either write a split partial (m, l, a) or finish: merge the optional
//      self token, apply W^V_t once, add l * mu^V_t, normalise and store o and lse.
// The reconstructed K/V of cached tokens are never formed.
#include <algorithm>
#include <type_traits>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

// Largest growth of the running maximum tolerated before rescaling (base-2 units). Weights are
// at most 2^kLazy = 256 relative to the stored maximum, which float32 sums absorb without loss of
// range; skipping most rescales keeps the branch rare.
constexpr float kLazy = 8.0f;

// First latent row of sequence `seq` (head h): per-head cache [B][H][n_max][r], 2D [B][n_max][r].
__device__ __forceinline__ size_t latent_row(const DecodeParams& p, int seq, int h) {
  return p.variant == LLA_2D ? static_cast<size_t>(seq) * p.n_max
                             : (static_cast<size_t>(seq) * p.H + h) * p.n_max;
}

// Listed slots of a gather-indexed row, clamped to [0, budget].
__device__ __forceinline__ int gather_keys(const DecodeParams& p, int row) {
  const int n = p.seq_lens != nullptr ? uniform(p.seq_lens[row]) : p.budget;
  return min(max(n, 0), p.budget);
}

// Keys visible to query row `row` (see DecodeParams), clamped to [0, n_max].
__device__ __forceinline__ int row_keys(const DecodeParams& p, int row) {
  const int seq = row / p.rows_per_seq;
  int n = p.seq_lens != nullptr ? uniform(p.seq_lens[seq]) : p.n_max;
  if (p.causal) n += row - seq * p.rows_per_seq + 1;
  return min(max(n, 0), p.n_max);
}

// Position of query row `row` for the rotary branch: a decode row sits at its key count nb (after
// the cached keys); a causal (prefill) row j of a chunk at ctx + j, the slot of its own key.
__device__ __forceinline__ double row_position(const DecodeParams& p, int row, int nb) {
  if (!p.causal) return nb;
  const int seq = row / p.rows_per_seq;
  const int ctx = p.seq_lens != nullptr ? uniform(p.seq_lens[seq]) : p.n_max;
  return static_cast<double>(ctx) + (row - seq * p.rows_per_seq);
}

// Offset of mu_t restricted to head h: per-head [H][T*d] at (h, t*d); 2D [T*H*d] at t*H*d + h*d.
__device__ __forceinline__ size_t mu_offset(const DecodeParams& p, int h) {
  return p.variant == LLA_2D ? (static_cast<size_t>(p.t) * p.H + h) * p.d
                             : (static_cast<size_t>(h) * p.T + p.t) * p.d;
}

// W_t restricted to head h: per-head [T][H][d][r] at (t, h); 2D [T][H*d][r] at rows t*H*d + h*d.
// Both are element offset (t*H + h)*d*r.
__device__ __forceinline__ size_t w_offset(const DecodeParams& p, int h, int r) {
  return (static_cast<size_t>(p.t) * p.H + h) * p.d * r;
}

// Finish one (b, h): merge the latent part (M, l, a[] in LDS, base-2, relative to M) with the
// optional self token, apply W^V_t once, add mu^V_t, normalise, store. Runs on one wave.
template <class S>
__device__ void finish_unit(const DecodeParams& p, int b, int h, float M, float l,
                            const float* a_s, const float* q_s, int lane) {
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  float s_self = kNegInf;
  if (p.k_self != nullptr) {
    float part = 0.f;
    for (int j = lane; j < p.d; j += 64) part += q_s[j] * ld<S>(p.k_self, bh * p.d + j);
    // decoupled rotary branch: the self key's rotary part, q_rope . k_rope_self (both would be
    // rotated at the same position N_b, which leaves their dot product unchanged)
    if (p.d_rope > 0 && p.k_rope_self != nullptr) {
      const size_t seq = static_cast<size_t>(b) / p.rows_per_seq;
      for (int j = lane; j < p.d_rope; j += 64)
        part += ld<BF16>(p.q_rope, bh * p.d_rope + j) * ld<BF16>(p.k_rope_self, seq * p.d_rope + j);
    }
    s_self = wave_sum(part) * p.scale_log2;
  }
  const float M2 = fmaxf(M, s_self);
  const float f_lat = (M == kNegInf) ? 0.f : fast_exp2(M - M2);
  const float p_self = (s_self == kNegInf) ? 0.f : fast_exp2(s_self - M2);
  const float den = l * f_lat + p_self;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const size_t woff = w_offset(p, h, p.r_v);
  const size_t moff = mu_offset(p, h);
  constexpr int VE = 16 / S::kBytes;  // values per 16-byte piece of a W^V row
  for (int j = lane; j < p.d; j += 64) {
    float o = 0.f;
    const size_t row = woff + static_cast<size_t>(j) * p.r_v;
    // rows of r_v values start 16-byte aligned (r_v is a multiple of VE for every compiled pair):
    // each lane reads its row as whole 16-byte pieces, all issued before the sums
    const uint4* wr = reinterpret_cast<const uint4*>(static_cast<const char*>(p.Wv) + row * S::kBytes);
    int r = 0;
    for (; r + VE <= p.r_v; r += VE) {
      const uint4 w = wr[r / VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) o += frag_elem<S>(&w, e) * a_s[r + e];
    }
    for (; r < p.r_v; ++r) o += ld<S>(p.Wv, row + r) * a_s[r];
    if (p.mu_v != nullptr) o += l * ld<S>(p.mu_v, moff + j);
    o *= f_lat;
    if (p.v_self != nullptr) o += p_self * ld<S>(p.v_self, bh * p.d + j);
    st<S>(p.out, bh * p.d + j, o * inv);
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[bh] = den > 0.f ? (M2 + fast_log2(den)) * kLn2 : kNegInf;
}

// One wave per (b, h, split). LPT lanes share a token; each holds EK = RK/LPT K elements and
// EV = RV/LPT V elements. U tiles of 64/LPT tokens are loaded before any is consumed. With G the
// split ranges over the row's slot list instead of its first N latents: each token's slot is read
// first, and a slot outside [0, n_max) counts as masked. S is the storage of q, W, mu, the self
// token and out; LS that of the latent rows (S itself, or Q8 low-bit rows read whole by one lane:
// the K row scale multiplies the score, the V row scale the token's weight). With DR > 0 each
// token's score also gets its rotary part q_R . k_R (decoupled RoPE branch): q_R (the head's
// rotary query, rotated at the decoding position, scaled) is formed in the prologue, and each
// token's DR-wide rotary key, shared by every head of the sequence, is dotted in the token's lane
// group beside its latent slices. HG == 1: every wave loads the rotary rows of its tokens itself.
// HG > 1 (head groups): the HG waves of a workgroup are HG heads of one sequence over the same
// tokens; each batch's rotary rows are loaded once, an HG-th by each wave, and handed over in LDS,
// so the rows cross the L2 once per head group rather than once per head (a head past H is a
// placeholder wave: it loads its share of the rotary rows, reads no latents and writes nothing).
// A lane's S-byte row slice (whole words, S <= 32) of the row at byte offset row of a raw buffer,
// for lane sub of the LPT lanes that share the row. Up to 16 bytes: one load at S*sub. Longer
// slices are split: the first 16 bytes at 16*sub (into f[0]), the rest at 16*LPT + (S-16)*sub
// (into f[1]), so each of the two load instructions reads every row as one run without gaps.
template <int S, int AUX, int LPT>
__device__ __forceinline__ void load_slice(__amdgpu_buffer_rsrc_t rs, uint32_t row, int sub, uint4* f) {
  if constexpr (S <= 16) {
    f[0] = buffer_words<S / 4, AUX>(rs, row + S * sub);
  } else {
    f[0] = buffer_words<4, AUX>(rs, row + 16 * sub);
    f[1] = buffer_words<(S - 16) / 4, AUX>(rs, row + 16 * LPT + (S - 16) * sub);
  }
}
// The latent entry that element e of lane sub's slice holds (E elements per slice, E16 of them in
// the first 16 bytes; SPLIT: the slice is split as load_slice splits slices over 16 bytes).
template <bool SPLIT, int E, int E16, int LPT>
__device__ __forceinline__ int slice_entry(int sub, int e) {
  if constexpr (SPLIT) return e < E16 ? sub * E16 + e : LPT * E16 + sub * (E - E16) + (e - E16);
  return sub * E + e;
}

// Waves per workgroup of the streaming kernels (all on one (row, head, split)).
constexpr int kMaxWaves = 8;

// q~ = scale*log2(e) * W^K_t[h]^T q of one (row, head) into qt_s[RK], by the nw waves of the
// workgroup (q at element qoff of p.q). Each lane owns one 16-byte piece of the W^K rows (VE
// consecutive r) and a residue class of rows j, and loads those rows' q entries itself: every load
// it makes is issued before the sums and the whole slice arrives in one memory round trip (no
// wait for q to be staged first). Lanes sharing a piece add up in registers (DPP), the waves
// through LDS (red_s [kMaxWaves][RK]); the barrier before that also publishes what the caller
// wrote to LDS before the call.
template <class S, int RK>
__device__ __forceinline__ void absorb_query(const DecodeParams& p, int h, int nw, int wave, int lane,
                                             size_t qoff, float* red_s, float* qt_s) {
  constexpr int VE = 16 / S::kBytes;
  constexpr int NRB = RK / VE;  // 16-byte pieces per W^K row
  static_assert(RK % VE == 0 && NRB <= 64, "W^K rows of whole 16-byte pieces");
  constexpr int GL = NRB > 32 ? 1 : NRB > 16 ? 2 : NRB > 8 ? 4 : NRB > 4 ? 8 : NRB > 2 ? 16 : NRB > 1 ? 32 : 64;
  const int rb = lane / GL;
  const int jg = lane % GL;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  if (rb < NRB) {
    const uint4* wk = reinterpret_cast<const uint4*>(static_cast<const char*>(p.Wk) +
                                                     w_offset(p, h, RK) * S::kBytes) + rb;
    for (int j = wave * GL + jg; j < p.d; j += GL * nw) {
      const uint4 w = wk[static_cast<size_t>(j) * NRB];
      const float qj = ld<S>(p.q, qoff + j);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += frag_elem<S>(&w, e) * qj;
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = group_sum<GL>(acc[e]);
  if (rb < NRB && jg == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) red_s[wave * RK + rb * VE + e] = acc[e];
  }
  __syncthreads();
  for (int r = wave * 64 + lane; r < RK; r += 64 * nw) {
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += red_s[w * RK + r];
    qt_s[r] = v * p.scale_log2;
  }
}

template <class S, class LS, int RK, int RV, int LPT, int U, bool G, int DR = 0, int HG = 1>
__global__ __launch_bounds__(64 * kMaxWaves) void decode_partial_kernel(DecodeParams p) {
  constexpr bool R = DR > 0;
  constexpr bool kHG = HG > 1;
  static_assert(!kHG || (R && HG <= kMaxWaves), "head groups share rotary rows");
  constexpr int RPC = R ? DR / 8 : 1;          // 16-byte pieces of a rotary key row
  constexpr int NRP = (RPC + LPT - 1) / LPT;   // pieces per lane (piece sub + LPT * k)
  constexpr bool kQ8 = std::is_same<LS, Q8>::value || std::is_same<LS, I8>::value;  // low-bit rows
  constexpr int RKB = LS::row(RK);  // bytes per latent row
  constexpr int RVB = LS::row(RV);
  // A lane's slice of a row: RK / LPT elements, or for low-bit rows RKB / LPT byte slots (codes,
  // then the row's zero padding and, in the last lane of the token's group, its float32 scale).
  constexpr int EK = kQ8 ? RKB / LPT : RK / LPT;
  constexpr int EV = kQ8 ? RVB / LPT : RV / LPT;
  constexpr int TPW = 64 / LPT;
  constexpr int SK = EK * LS::kBytes;  // bytes of a lane's slice of a K row
  constexpr int SV = EV * LS::kBytes;
  // Buffer loads of whole-word slices of at most 32 bytes (one load of up to 16 bytes, a second
  // for the rest): the LPT lanes of a token then read its row as one run, and each load
  // instruction covers 64 / LPT consecutive rows without gaps (one load per slice) or leaves only
  // the second load's bytes for the next instruction; the contiguous read streams past the caches
  // (non-temporal). Low-bit slices follow the same map (a 112-byte r = 96 row: 4 lanes x 28 bytes).
  constexpr bool kOne = SK % 4 == 0 && SV % 4 == 0 && SK <= 32 && SV <= 32;
  constexpr int VK = kOne ? (SK + 15) / 16 : SK / 16;
  constexpr int VV = kOne ? (SV + 15) / 16 : SV / 16;
  static_assert(kQ8 ? (EK * LPT == RKB && EV * LPT == RVB) : (EK * LPT == RK && EV * LPT == RV),
                "rows must split evenly over lanes");
  static_assert(kOne || (VK * 16 == SK && VV * 16 == SV), "16-byte fragments");
  static_assert(!kQ8 || kOne || LPT == 1, "a low-bit row is one lane's, or one load per lane");
  constexpr int E16 = 16 / LS::kBytes;                // elements in a slice's first 16 bytes
  constexpr bool kSplitK = kOne && SK > 16;          // slices read by two loads (load_slice)
  constexpr bool kSplitV = kOne && SV > 16;

  // per (row, head): one copy, or one per wave of a head group
  __shared__ float q_a[HG][256];
  __shared__ float qt_a[HG][RK];
  __shared__ float qr_a[HG][R ? DR : 1];  // rotated rotary query times scale * log2(e)
  __shared__ float a_a[HG][RV];
  // the waves' partial sums of q~ (absorb_query), later their (m, l, a) partials (merge below)
  __shared__ float xs_s[(kMaxWaves * RK > (kMaxWaves - 1) * (2 + RV)) ? kMaxWaves * RK : (kMaxWaves - 1) * (2 + RV)];

  // nw waves share one (row, head, split): wave w streams the w-th of nw equal parts of the
  // split's tokens (the gather read keeps one wave: its slot list is staged per wave). A head
  // group's HG waves each take one head over the whole split.
  const int nw = G ? 1 : kHG ? HG : min(max(p.wg_waves, 1), kMaxWaves);
  const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int hw = kHG ? wave : 0;  // this wave's copy of the per-head LDS arrays
  float* const q_s = q_a[hw];
  float* const qt_s = qt_a[hw];
  float* const qr_s = qr_a[hw];
  float* const a_s = a_a[hw];
  // the prologue's work is divided over pn waves (a head group's waves each do their own)
  const int pw = kHG ? 0 : wave;
  const int pn = kHG ? 1 : nw;
  // Sequences whose heads share what they stream (the rotary keys; LLA-2D: the latents too) keep
  // all their workgroups on one XCD when B is a multiple of 8: workgroups are dispatched round-
  // robin over the 8 XCDs, so unit (x % 8) + 8 * k runs on XCD x % 8, and consecutive k there
  // are the heads and splits of one sequence, co-resident and sharing that XCD's L2.
  const int ng = kHG ? (p.H + HG - 1) / HG : p.H;  // head units of one row
  int unit = blockIdx.x;
  if ((R || p.variant == LLA_2D) && (p.B & 7) == 0) {
    const int per = ng * p.splits;  // units of one row
    const int k = unit >> 3;
    unit = ((k / per) * 8 + (unit & 7)) * per + k % per;
  }
  const int split = unit % p.splits;
  const int b = unit / p.splits / ng;
  int h = unit / p.splits % ng;
  if (kHG) h = h * HG + wave;
  const bool live = !kHG || h < p.H;  // a placeholder wave past H reads and writes no head
  if (kHG) h = min(h, p.H - 1);
  const int bh = b * p.H + h;

  const int nb = G ? gather_keys(p, b) : row_keys(p, b);
  // the split's keys [s0, s1); nw > 1 waves divide the keys the row actually has (not the planned
  // chunk) into parts of a multiple of 32 tokens, so no wave streams more than its share
  const int s0 = split * p.chunk;
  const int s1 = min(nb, s0 + p.chunk);
  const int cw = (kHG || nw == 1) ? p.chunk : (max(s1 - s0, 0) + 32 * nw - 1) / (32 * nw) * 32;
  const int tb = uniform(s0 + (kHG ? 0 : wave * cw));
  const int te = uniform(min(s1, tb + cw));

  // One-load rows stream two register batches ahead. The gather read first stages its split's
  // slot list in LDS (when it fits), so finding a row costs an LDS read rather than a memory round
  // trip in front of every batch; longer splits take the one-batch loop below.
  static_assert(!(G && R), "the rotary branch is read for contiguous rows only");
  constexpr int kSlotCap = 2048;
  __shared__ __attribute__((aligned(16))) int32_t slot_s[G ? kSlotCap : 4];
  const int32_t* srow = G ? p.slots + static_cast<size_t>(b) * p.budget : nullptr;
  const bool piped = kOne && (!G || te - tb <= kSlotCap);
  // every 16-byte load of the list is issued here (positions past the split read as zeros) and
  // written to LDS after the query absorption below, whose own loads then overlap the list's
  const int nsl = G && kOne && piped ? (max(te - tb, 0) + 255) / 256 : 0;  // 256 positions per load
  uint4 sl[G && kOne ? kSlotCap / 256 : 1];
  if constexpr (G && kOne) {
    const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(srow + tb, static_cast<uint32_t>(max(te - tb, 0)) * 4);
#pragma unroll
    for (int k = 0; k < kSlotCap / 256; ++k)
      if (k < nsl) sl[k] = buffer_words<4, 0>(rl, static_cast<uint32_t>(k * 64 + lane) * 16);
  }

  const int sub = lane % LPT;
  const int grp = lane / LPT;
  // low-bit slices: the bytes of each of this lane's words (load f, word k) that hold codes
  // (padding and the scale must never be converted as codes: a scale byte can be an E4M3 NaN
  // pattern); byte e of the slice holds row entry slice_entry(sub, e)
  uint32_t kmask[2][4], vmask[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t mk = 0, mv = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 16 * f + 4 * k + i;
        if (e < EK && slice_entry<kSplitK, EK, E16, LPT>(sub, e) < RK) mk |= 0xffu << (8 * i);
        if (e < EV && slice_entry<kSplitV, EV, E16, LPT>(sub, e) < RV) mv |= 0xffu << (8 * i);
      }
      kmask[f][k] = mk;
      vmask[f][k] = mv;
    }

  // --- 2-3. latent stream with online softmax -------------------------------------------------
  const size_t lrow = latent_row(p, b / p.rows_per_seq, h);
  const char* zkp = static_cast<const char*>(p.zk) + lrow * RKB + sub * SK;
  const char* zvp = static_cast<const char*>(p.zv) + lrow * RVB + sub * SV;
  // kOne: buffer descriptors over the rows this wave may read (the gather read: all n_max slots;
  // the contiguous read: its split [tb, te)); an offset at the end reads zeros
  const int row0 = G ? 0 : tb;
  const uint32_t nrows = static_cast<uint32_t>(uniform(G ? p.n_max : max(te - tb, 0)));
  const uint32_t nlat = live ? nrows : 0;  // a placeholder wave's latent loads all read zeros
  const __amdgpu_buffer_rsrc_t rsk = buffer_rsrc(static_cast<const char*>(p.zk) + (lrow + row0) * RKB, nlat * RKB);
  const __amdgpu_buffer_rsrc_t rsv = buffer_rsrc(static_cast<const char*>(p.zv) + (lrow + row0) * RVB, nlat * RVB);
  // non-temporal: rows are read once. For the gather read this pays when listed slots run in
  // order (a sink + window list: 248 -> 229 us at the capacity shape); a random list of 48-byte
  // rows reads ~5% slower than with ordinary loads.
  constexpr int kAux = 2;
  constexpr bool kPipe = kOne && !G;  // the contiguous buffer-load read (always two batches ahead)
  // the gather read's one-batch-ahead row lookup (below), where its registers keep the occupancy
  constexpr bool kAhead = G && kOne &&
                          (std::is_same<S, F32>::value || (kQ8 && RK >= 16) || (RK == 24 && RV == 24) ||
                           (RK == 96 && RV == 96));
  // Rotary keys (R): [B][n_max][DR] bf16, one row per token shared by every head of the sequence.
  // Lane `sub` of a token's group holds pieces sub + LPT * k of the row (16 bytes each); ordinary
  // loads, so the row stays in L2 for the sequence's other heads.
  static_assert(!R || kPipe, "the rotary branch takes the pipelined contiguous read");
  // registers of a batch's rotary loads: per tile NRP pieces (HG == 1), or the wave's share of
  // the batch's pieces, NSH per lane (HG > 1), which the batch's consume hands over in LDS
  constexpr int kStep = TPW * U;        // tokens per batch
  constexpr int PB = kStep * RPC;       // 16-byte rotary pieces of a batch
  constexpr int NSH = kHG ? (PB + 64 * HG - 1) / (64 * HG) : 1;
  constexpr int SRU = kHG ? 1 : U;
  constexpr int NSR = kHG ? NSH : R ? NRP : 1;
  // batch rotary tiles in LDS (HG > 1), two in turn: piece k of lane sub of tile u's token grp at
  // [k][u * 64 + lane], so each read instruction of the consume covers 1 KiB without gaps
  __shared__ uint4 rt_s[kHG ? 2 : 1][kHG ? NRP * kStep * LPT : 1];
  const __amdgpu_buffer_rsrc_t rss = buffer_rsrc(
      R ? static_cast<const char*>(p.k_rope) + (static_cast<size_t>(b / p.rows_per_seq) * p.n_max + row0) * DR * 2 : nullptr,
      R ? nrows * DR * 2 : 0);

  // --- 1. query absorption (prologue): q~ and beta, then (gather read) the slot list in LDS.
  // The contiguous read issues its first batch of latent loads before it (they do not depend on
  // q~), so the absorption's memory round trips overlap the stream's first one.
  float qt[EK];
  float qr[NRP][R ? 8 : 1];
  float beta = 0.f;
  auto prologue = [&]() {
    const size_t qoff = static_cast<size_t>(bh) * p.d;
    // q in LDS for the mu^K and self-key scores (read after the absorption's barrier)
    for (int j = pw * 64 + lane; j < p.d; j += 64 * pn) q_s[j] = ld<S>(p.q, qoff + j);
    absorb_query<S, RK>(p, h, pn, pw, lane, qoff, xs_s + (kHG ? wave * RK : 0), qt_s);
    if (p.mu_k != nullptr) {
      const size_t moff = mu_offset(p, h);
      float part = 0.f;
      for (int j = lane; j < p.d; j += 64) part += q_s[j] * ld<S>(p.mu_k, moff + j);
      beta = wave_sum(part) * p.scale_log2;
    }
    if constexpr (G && kOne) {
#pragma unroll
      for (int k = 0; k < kSlotCap / 256; ++k)
        if (k < nsl) *reinterpret_cast<uint4*>(&slot_s[(k * 64 + lane) * 4]) = sl[k];
    }
    if constexpr (R) {  // rotary query of this head rotated at the row's position
      const size_t qro = static_cast<size_t>(bh) * DR;
      const double rpos = row_position(p, b, nb);
      for (int i = pw * 64 + lane; i < DR / 2; i += 64 * pn) {
        float y0, y1;
        rotate_pair(ld<BF16>(p.q_rope, qro + 2 * i), ld<BF16>(p.q_rope, qro + 2 * i + 1), i, DR, rpos,
                    p.rope_base, &y0, &y1);
        qr_s[2 * i] = y0 * p.scale_log2;
        qr_s[2 * i + 1] = y1 * p.scale_log2;
      }
    }
    __syncthreads();  // q~ and the slot list are visible to every lane from here
#pragma unroll
    for (int e = 0; e < EK; ++e) {
      const int c = slice_entry<kSplitK, EK, E16, LPT>(sub, e);  // low-bit slots past the codes take a zero query weight
      qt[e] = (!kQ8 || c < RK) ? qt_s[min(c, RK - 1)] : 0.f;
    }
    if constexpr (R) {
#pragma unroll
      for (int k = 0; k < NRP; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = sub + LPT * k;
          qr[k][e] = c < RPC ? qr_s[c * 8 + e] : 0.f;
        }
    }
  };

  float m = kNegInf;
  float l = 0.f;
  float acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;

  // fold one batch of U tiles (ok: token inside the split and valid) into (m, l, acc)
  auto consume = [&](uint4 (&kr)[U][VK], uint4 (&vr)[U][VV], const bool (&ok)[U], uint4 (&srv)[SRU][NSR],
                     uint4* tile) {
    if constexpr (kHG) {  // hand this wave's share of the batch's rotary rows to the group
#pragma unroll
      for (int k = 0; k < NSH; ++k) {
        const int i = (wave + HG * k) * 64 + lane;  // piece c of the batch's row li
        const int li = i / RPC, c = i % RPC;
        if (PB % (64 * HG) == 0 || i < PB) tile[((c / LPT) * kStep + li) * LPT + c % LPT] = srv[0][k];
      }
      // every share is in LDS; the tile written here two batches ago has been read by all waves
      // (each passed the barrier of the batch in between only after its reads)
      lds_barrier();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sk = 1.f, sv = 1.f;  // low-bit row scales
      if constexpr (kQ8 && kOne) {
        // the scale is the last word of the group's last lane; a zero-padded group sum gives it
        // to every lane of the group exactly. Then the non-code bytes are cleared.
        // (a split slice ends in its second load)
        constexpr int FK = kSplitK ? 1 : 0, FV = kSplitV ? 1 : 0;
        constexpr int WK = (kSplitK ? SK - 16 : SK) / 4 - 1, WV = (kSplitV ? SV - 16 : SV) / 4 - 1;
        const uint4 kl = kr[u][FK], vl = vr[u][FV];
        const uint32_t kw = WK == 0 ? kl.x : WK == 1 ? kl.y : WK == 2 ? kl.z : kl.w;
        const uint32_t vw = WV == 0 ? vl.x : WV == 1 ? vl.y : WV == 2 ? vl.z : vl.w;
        sk = group_sum<LPT>(sub == LPT - 1 ? __uint_as_float(kw) : 0.f);
        sv = group_sum<LPT>(sub == LPT - 1 ? __uint_as_float(vw) : 0.f);
#pragma unroll
        for (int f = 0; f < VK; ++f)
          kr[u][f] = make_uint4(kr[u][f].x & kmask[f][0], kr[u][f].y & kmask[f][1], kr[u][f].z & kmask[f][2],
                                kr[u][f].w & kmask[f][3]);
#pragma unroll
        for (int f = 0; f < VV; ++f)
          vr[u][f] = make_uint4(vr[u][f].x & vmask[f][0], vr[u][f].y & vmask[f][1], vr[u][f].z & vmask[f][2],
                                vr[u][f].w & vmask[f][3]);
      } else if constexpr (kQ8) {
        // the last 16 bytes of a low-bit row hold padding the arithmetic never reads; without
        // this the compiler narrows their load and a row takes three partial loads, not two
        asm("" : "+v"(kr[u][VK - 1].x), "+v"(kr[u][VK - 1].y), "+v"(kr[u][VK - 1].z));
        asm("" : "+v"(vr[u][VV - 1].x), "+v"(vr[u][VV - 1].y), "+v"(vr[u][VV - 1].z));
        sk = q8_row_scale(kr[u], VK);
        sv = q8_row_scale(vr[u], VV);
      }
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e)
        if (!kQ8 || kOne || e < RK) sc += qt[e] * frag_elem<LS>(kr[u], e);
      if constexpr (R) {  // this lane's pieces of the token's rotary key
#pragma unroll
        for (int k = 0; k < NRP; ++k) {
          uint4 pc;
          if constexpr (kHG)
            pc = (sub + LPT * k < RPC) ? tile[(k * kStep + u * TPW) * LPT + lane] : make_uint4(0, 0, 0, 0);
          else
            pc = srv[u][k];
#pragma unroll
          for (int e = 0; e < 8; ++e) sc += qr[k][e] * frag_elem<BF16>(&pc, e);
        }
      }
      sc = group_sum<LPT>(sc);
      if (kQ8) sc *= sk;
      sc += beta;
      if (ok[u]) {
        if (sc > m + kLazy) {
          const float c = fast_exp2(m - sc);
          l *= c;
#pragma unroll
          for (int e = 0; e < EV; ++e) acc[e] *= c;
          m = sc;
        }
        const float pr = fast_exp2(sc - m);
        l += pr;
        const float pv = kQ8 ? pr * sv : pr;
#pragma unroll
        for (int e = 0; e < EV; ++e)
          if (!kQ8 || kOne || e < RV) acc[e] += pv * frag_elem<LS>(vr[u], e);
      }
    }
  };

  if (piped) {
   if constexpr (kOne) {
    // Two register batches in turn, the next batch's loads issued before the current one is
    // consumed, so a wave always has a batch in flight. Rows past the split (or, gathered, with
    // a slot outside the cache) read as zeros through the descriptor bound (no memory access)
    // and are masked; a batch wholly past the split costs only its masked arithmetic.
    // A gathered row comes from the staged list (nrows: past the split, or a slot outside the
    // cache). With kAhead the gather read looks a batch's rows up one batch before its loads are
    // issued, so the LDS read's latency overlaps the batch consumed in between instead of delaying
    // the issue (sink + window list at the capacity shape: 210-212 -> 203-206 us); it costs 2 U
    // registers, so it is kept where the kernel's occupancy stays the same.
    auto gathered_row = [&](int tok) -> uint32_t {
      const int s = tok < te ? slot_s[min(tok - tb, kSlotCap - 1)] : -1;
      return static_cast<unsigned>(s) < static_cast<unsigned>(p.n_max) ? static_cast<uint32_t>(s) : nrows;
    };
    auto lookup = [&](int t0, uint32_t (&rr)[U]) {
      if constexpr (kAhead) {
#pragma unroll
        for (int u = 0; u < U; ++u) rr[u] = gathered_row(t0 + u * TPW + grp);
      }
    };
    auto issue = [&](int t0, const uint32_t (&rrs)[U], uint4 (&kr)[U][VK], uint4 (&vr)[U][VV],
                     uint4 (&srv)[SRU][NSR]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        uint32_t rr;
        if constexpr (kAhead) rr = rrs[u];
        else if constexpr (G) rr = gathered_row(tok);
        else rr = static_cast<uint32_t>(min(tok, te) - row0);
        load_slice<SK, kAux, LPT>(rsk, rr * RKB, sub, kr[u]);
        load_slice<SV, kAux, LPT>(rsv, rr * RVB, sub, vr[u]);
        if constexpr (!kHG) {
#pragma unroll
          for (int k = 0; k < NSR; ++k) {
            const int c = sub + LPT * k;
            srv[u][k] = (R && c < RPC) ? buffer_words<4, 0>(rss, rr * (DR * 2) + c * 16) : make_uint4(0, 0, 0, 0);
          }
        }
      }
      if constexpr (kHG) {  // this wave's share: 1 KiB runs of the batch's rows (zeros past te)
#pragma unroll
        for (int k = 0; k < NSH; ++k) {
          const int i = (wave + HG * k) * 64 + lane;
          const int li = i / RPC, c = i % RPC;
          const uint32_t rr = static_cast<uint32_t>(min(t0 + li, te) - row0);
          srv[0][k] = (PB % (64 * HG) == 0 || i < PB) ? buffer_words<4, 0>(rss, rr * (DR * 2) + c * 16)
                                                      : make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto mask = [&](int t0, const uint32_t (&rrs)[U], bool (&ok)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        if constexpr (kAhead) {
          ok[u] = rrs[u] != nrows;
        } else {
          ok[u] = tok < te;
          if constexpr (G)
            ok[u] = ok[u] && static_cast<unsigned>(slot_s[min(tok - tb, kSlotCap - 1)]) < static_cast<unsigned>(p.n_max);
        }
      }
    };
    uint4 ka[U][VK], va[U][VV], kb[U][VK], vb[U][VV];
    uint4 sa[SRU][NSR], sb[SRU][NSR];
    uint32_t ra[U], rb[U];  // kAhead: the looked-up rows of the batches in ka and kb
    bool ok[U];
    if constexpr (G) {  // the first rows' slots come from the list the prologue stages
      prologue();
      lookup(tb, ra);
      if (tb < te) issue(tb, ra, ka, va, sa);
    } else {
      if (tb < te) issue(tb, ra, ka, va, sa);
      prologue();
    }
    lookup(tb + kStep, rb);
    for (int t0 = tb; t0 < te; t0 += 2 * kStep) {
      issue(t0 + kStep, rb, kb, vb, sb);
      mask(t0, ra, ok);
      lookup(t0 + 2 * kStep, ra);
      consume(ka, va, ok, sa, rt_s[0]);
      // no early exit here: with one exit at the bottom the compiler's wait before the loop top
      // leaves the batch just issued in flight (an exit here made it drain every load)
      issue(t0 + 2 * kStep, ra, ka, va, sa);
      mask(t0 + kStep, rb, ok);
      lookup(t0 + 3 * kStep, rb);
      consume(kb, vb, ok, sb, rt_s[kHG ? 1 : 0]);
    }
   }
  } else if constexpr (!kPipe) {  // the contiguous one-load read always takes the loop above
    prologue();
    for (int t0 = tb; t0 < te; t0 += TPW * U) {
      uint4 kr[U][VK];
      uint4 vr[U][VV];
      bool ok[U];
      int slot[U];
      uint4 srv[SRU][NSR];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        ok[u] = tok < te;
        slot[u] = tok;
        if (G) {
          slot[u] = ok[u] ? srow[tok] : 0;
          ok[u] = ok[u] && static_cast<unsigned>(slot[u]) < static_cast<unsigned>(p.n_max);
        }
#pragma unroll
        for (int k = 0; k < NSR; ++k) srv[u][k] = make_uint4(0, 0, 0, 0);  // no rotary branch here
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (kOne) {
          const uint32_t rr = ok[u] ? static_cast<uint32_t>(slot[u] - row0) : nrows;
          load_slice<SK, kAux, LPT>(rsk, rr * RKB, sub, kr[u]);
          load_slice<SV, kAux, LPT>(rsv, rr * RVB, sub, vr[u]);
        } else if (ok[u]) {
          const uint4* kp = reinterpret_cast<const uint4*>(zkp + static_cast<size_t>(slot[u]) * RKB);
          const uint4* vp = reinterpret_cast<const uint4*>(zvp + static_cast<size_t>(slot[u]) * RVB);
#pragma unroll
          for (int i = 0; i < VK; ++i) kr[u][i] = kp[i];
#pragma unroll
          for (int i = 0; i < VV; ++i) vr[u][i] = vp[i];
        } else {
#pragma unroll
          for (int i = 0; i < VK; ++i) kr[u][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < VV; ++i) vr[u][i] = make_uint4(0, 0, 0, 0);
        }
      }
      consume(kr, vr, ok, srv, rt_s[0]);
    }
  }

  // --- 4. merge lanes ---------------------------------------------------------------------------
  const float M = wave_max(m);
  const float f = (m == kNegInf) ? 0.f : fast_exp2(m - M);
  l *= f;
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] *= f;
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
    l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }

  // --- merge the workgroup's waves: waves 1.. hand (M, l, a) to wave 0 through LDS -----------
  float Mt = M;
  if (!kHG && nw > 1) {
    __syncthreads();  // every wave is past its last read of xs_s (absorb_query)
    if (wave > 0) {
      float* xw = xs_s + (wave - 1) * (2 + RV);
      if (lane == 0) {
        xw[0] = M;
        xw[1] = l;
      }
      if (lane < LPT) {
#pragma unroll
        for (int e = 0; e < EV; ++e)
          if (!kQ8 || slice_entry<kSplitV, EV, E16, LPT>(lane, e) < RV) xw[2 + slice_entry<kSplitV, EV, E16, LPT>(lane, e)] = acc[e];
      }
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < nw; ++w) Mt = fmaxf(Mt, xs_s[(w - 1) * (2 + RV)]);
      const float f0 = (M == kNegInf) ? 0.f : fast_exp2(M - Mt);
      l *= f0;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] *= f0;
      for (int w = 1; w < nw; ++w) {
        const float* xv = xs_s + (w - 1) * (2 + RV);
        const float fw = (xv[0] == kNegInf) ? 0.f : fast_exp2(xv[0] - Mt);
        l += fw * xv[1];
#pragma unroll
        for (int e = 0; e < EV; ++e)
          if (!kQ8 || slice_entry<kSplitV, EV, E16, LPT>(sub, e) < RV) acc[e] += fw * xv[2 + slice_entry<kSplitV, EV, E16, LPT>(sub, e)];
      }
    }
  }

  const bool out_wave = kHG ? live : wave == 0;  // the wave that holds the unit's merged partial
  if (p.splits > 1) {
    float* w = p.ws + (static_cast<size_t>(bh) * p.splits + split) * (2 + RV);
    if (out_wave && lane == 0) {
      w[0] = Mt;
      w[1] = l;
    }
    if (out_wave && lane < LPT) {
#pragma unroll
      for (int e = 0; e < EV; ++e)
        if (!kQ8 || slice_entry<kSplitV, EV, E16, LPT>(lane, e) < RV) w[2 + slice_entry<kSplitV, EV, E16, LPT>(lane, e)] = acc[e];
    }
    return;
  }
  if (out_wave && lane < LPT) {
#pragma unroll
    for (int e = 0; e < EV; ++e)
      if (!kQ8 || slice_entry<kSplitV, EV, E16, LPT>(lane, e) < RV) a_s[slice_entry<kSplitV, EV, E16, LPT>(lane, e)] = acc[e];
  }
  __syncthreads();
  if (out_wave) finish_unit<S>(p, b, h, Mt, l, a_s, q_s, lane);
}

// Log-sum-exp merge of the S split partials of one (b, h), then the same finish. 256 threads:
// the split maximum and weighted sum are block reductions, each thread merges one latent entry
// across every split (loads coalesced over entries), and wave 0 runs the finish. (With one wave
// per (b, h), a long context at B = 1 -- 16 units, 256 splits -- left the merge latency-bound.)
constexpr int kCombineThreads = 256;

template <class S>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeParams p) {
  __shared__ float q_s[256];
  __shared__ float a_s[512];
  __shared__ float f_s[256];
  __shared__ float red[kCombineThreads / 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int bh = blockIdx.x;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int S_ = p.splits;  // <= 256 (valu_plan)
  const int stride = 2 + p.r_v;
  const float* w = p.ws + static_cast<size_t>(bh) * S_ * stride;

  float mloc = kNegInf;
  for (int s = tid; s < S_; s += kCombineThreads) mloc = fmaxf(mloc, w[static_cast<size_t>(s) * stride]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kCombineThreads / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();  // red is reused below
  float lloc = 0.f;
  for (int s = tid; s < S_; s += kCombineThreads) {
    const float ms = w[static_cast<size_t>(s) * stride];
    const float fs = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
    f_s[s] = fs;
    lloc += fs * w[static_cast<size_t>(s) * stride + 1];
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[wave] = lloc;
  for (int j = tid; j < p.d; j += kCombineThreads) q_s[j] = ld<S>(p.q, static_cast<size_t>(bh) * p.d + j);
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) l += red[i];
  for (int r = tid; r < p.r_v; r += kCombineThreads) {
    float a = 0.f;
#pragma unroll 8
    for (int s = 0; s < S_; ++s) a += f_s[s] * w[static_cast<size_t>(s) * stride + 2 + r];
    a_s[r] = a;
  }
  __syncthreads();
  if (wave == 0) finish_unit<S>(p, b, h, M, l, a_s, q_s, lane);
}

using PartialFn = void (*)(DecodeParams);

template <class S, int RK, int RV, int LPT, int U>
PartialFn partial_fn() {
  return decode_partial_kernel<S, S, RK, RV, LPT, U, false>;
}
template <class S, int RK, int RV, int LPT, int U>
PartialFn gather_fn() {
  return decode_partial_kernel<S, S, RK, RV, LPT, U, true>;
}
// the contiguous read with the rotary branch, one instance per rotary width (32, 64, 128), one
// wave per head (w*) or head groups of kRopeGroup waves (g*); a wave's own rotary pieces take
// registers beside the latent slices, so fewer tiles are in flight per batch
constexpr int kRopeGroup = 8;
struct RopeFns {
  PartialFn w32, w64, w128;
  PartialFn g32, g64, g128;
};
template <class S, int RK, int RV, int LPT, int U>
RopeFns rope_fns() {
  constexpr int U2 = U > 2 ? U / 2 : 1;
  return {decode_partial_kernel<S, S, RK, RV, LPT, U, false, 32>,
          decode_partial_kernel<S, S, RK, RV, LPT, U, false, 64>,
          decode_partial_kernel<S, S, RK, RV, LPT, U2, false, 128>,
          decode_partial_kernel<S, S, RK, RV, LPT, U, false, 32, kRopeGroup>,
          decode_partial_kernel<S, S, RK, RV, LPT, U, false, 64, kRopeGroup>,
          decode_partial_kernel<S, S, RK, RV, LPT, U2, false, 128, kRopeGroup>};
}
template <class LS, int RK, int RV, int LPT, int U>
PartialFn q8_fn() {
  return decode_partial_kernel<BF16, LS, RK, RV, LPT, U, false>;
}
template <class LS, int RK, int RV, int LPT, int U>
PartialFn q8_gather_fn() {
  return decode_partial_kernel<BF16, LS, RK, RV, LPT, U, true>;
}

struct Entry {
  int dtype, r_k, r_v;
  PartialFn fn;   // contiguous read
  PartialFn gfn;  // gather-indexed read
  RopeFns rfn;    // contiguous read with the rotary branch (bf16 pairs only)
};

// Compiled (dtype, r_k, r_v) -> (lanes per token, tiles in flight). Lanes per token are chosen so
// that a lane's slice of a row is one load of at most 16 bytes wherever the rank allows it.
const Entry kTable[] = {
    {LLA_BF16, 8, 8, partial_fn<BF16, 8, 8, 1, 4>(), gather_fn<BF16, 8, 8, 1, 4>(),
     rope_fns<BF16, 8, 8, 4, 4>()},
    {LLA_BF16, 16, 16, partial_fn<BF16, 16, 16, 2, 4>(), gather_fn<BF16, 16, 16, 2, 4>(),
     rope_fns<BF16, 16, 16, 4, 4>()},
    {LLA_BF16, 24, 24, partial_fn<BF16, 24, 24, 4, 8>(), gather_fn<BF16, 24, 24, 4, 8>(),
     rope_fns<BF16, 24, 24, 4, 4>()},
    {LLA_BF16, 32, 32, partial_fn<BF16, 32, 32, 4, 4>(), gather_fn<BF16, 32, 32, 4, 8>(),
     rope_fns<BF16, 32, 32, 4, 4>()},
    {LLA_BF16, 64, 64, partial_fn<BF16, 64, 64, 8, 8>(), gather_fn<BF16, 64, 64, 8, 8>(),
     rope_fns<BF16, 64, 64, 8, 4>()},
    {LLA_BF16, 96, 96, partial_fn<BF16, 96, 96, 16, 8>(), gather_fn<BF16, 96, 96, 16, 8>(),
     rope_fns<BF16, 96, 96, 16, 4>()},
    {LLA_BF16, 128, 128, partial_fn<BF16, 128, 128, 16, 8>(), gather_fn<BF16, 128, 128, 16, 8>(),
     rope_fns<BF16, 128, 128, 16, 4>()},
    {LLA_BF16, 96, 160, partial_fn<BF16, 96, 160, 16, 8>(), gather_fn<BF16, 96, 160, 16, 8>(),
     rope_fns<BF16, 96, 160, 16, 4>()},
    {LLA_BF16, 256, 256, partial_fn<BF16, 256, 256, 32, 8>(), gather_fn<BF16, 256, 256, 32, 8>(),
     rope_fns<BF16, 256, 256, 32, 4>()},
    {LLA_F32, 8, 8, partial_fn<F32, 8, 8, 2, 4>(), gather_fn<F32, 8, 8, 2, 4>(), RopeFns{}},
    {LLA_F32, 16, 16, partial_fn<F32, 16, 16, 4, 4>(), gather_fn<F32, 16, 16, 4, 4>(), RopeFns{}},
    {LLA_F32, 24, 24, partial_fn<F32, 24, 24, 8, 4>(), gather_fn<F32, 24, 24, 8, 4>(), RopeFns{}},
    {LLA_F32, 32, 32, partial_fn<F32, 32, 32, 8, 4>(), gather_fn<F32, 32, 32, 8, 4>(), RopeFns{}},
    {LLA_F32, 64, 64, partial_fn<F32, 64, 64, 16, 4>(), gather_fn<F32, 64, 64, 16, 4>(), RopeFns{}},
    {LLA_F32, 96, 96, partial_fn<F32, 96, 96, 32, 4>(), gather_fn<F32, 96, 96, 32, 4>(), RopeFns{}},
    {LLA_F32, 128, 128, partial_fn<F32, 128, 128, 32, 4>(), gather_fn<F32, 128, 128, 32, 4>(), RopeFns{}},
    {LLA_F32, 96, 160, partial_fn<F32, 96, 160, 8, 1>(), gather_fn<F32, 96, 160, 8, 1>(), RopeFns{}},
    {LLA_F32, 256, 256, partial_fn<F32, 256, 256, 64, 4>(), gather_fn<F32, 256, 256, 64, 4>(), RopeFns{}},
    {LLA_BF16_Q8, 8, 8, q8_fn<Q8, 8, 8, 1, 4>(), q8_gather_fn<Q8, 8, 8, 1, 4>(), RopeFns{}},
    {LLA_BF16_Q8, 16, 16, q8_fn<Q8, 16, 16, 2, 4>(), q8_gather_fn<Q8, 16, 16, 2, 4>(), RopeFns{}},
    {LLA_BF16_Q8, 24, 24, q8_fn<Q8, 24, 24, 2, 4>(), q8_gather_fn<Q8, 24, 24, 2, 4>(), RopeFns{}},
    {LLA_BF16_Q8, 32, 32, q8_fn<Q8, 32, 32, 4, 8>(), q8_gather_fn<Q8, 32, 32, 4, 8>(), RopeFns{}},
    {LLA_BF16_Q8, 96, 96, q8_fn<Q8, 96, 96, 4, 2>(), q8_gather_fn<Q8, 96, 96, 4, 2>(), RopeFns{}},
    {LLA_BF16_I8, 8, 8, q8_fn<I8, 8, 8, 1, 4>(), q8_gather_fn<I8, 8, 8, 1, 4>(), RopeFns{}},
    {LLA_BF16_I8, 16, 16, q8_fn<I8, 16, 16, 2, 4>(), q8_gather_fn<I8, 16, 16, 2, 4>(), RopeFns{}},
    {LLA_BF16_I8, 24, 24, q8_fn<I8, 24, 24, 2, 4>(), q8_gather_fn<I8, 24, 24, 2, 4>(), RopeFns{}},
    {LLA_BF16_I8, 32, 32, q8_fn<I8, 32, 32, 4, 8>(), q8_gather_fn<I8, 32, 32, 4, 8>(), RopeFns{}},
    {LLA_BF16_I8, 96, 96, q8_fn<I8, 96, 96, 4, 2>(), q8_gather_fn<I8, 96, 96, 4, 2>(), RopeFns{}},
};

const Entry* find(int dtype, int r_k, int r_v) {
  for (const Entry& e : kTable)
    if (e.dtype == dtype && e.r_k == r_k && e.r_v == r_v) return &e;
  return nullptr;
}

}  // namespace

bool valu_supported(int variant, int dtype, int r_k, int r_v) {
  if (variant != LLA_PER_HEAD && variant != LLA_2D) return false;
  return find(dtype, r_k, r_v) != nullptr;
}

bool decode_supported(int variant, int dtype, int r_k, int r_v, int d_head) {
  return valu_supported(variant, dtype, r_k, r_v) ||
         (variant == LLA_2D && decode2d_mfma_supported(dtype, r_k, r_v, d_head));
}

bool decode_uses_mfma2d(const lla_desc& desc) {
  return desc.variant == LLA_2D && decode2d_mfma_supported(desc.dtype, desc.r_k, desc.r_v, desc.d_head);
}

void valu_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves) {
  // About 2048 waves per launch: one round for any of these kernels (each wave keeping two
  // batches of rows in flight). More waves than fit at once leave a last, partly filled round that
  // streams at a fraction of the bandwidth (4096 waves at 12 per CU: 410 us for the 262k-token
  // read). Few (row, head) units are therefore cut into parts of at least 256 tokens: first into
  // up to 8 waves of one workgroup, which merge in LDS (no workspace, no combine launch), then
  // into token splits merged by the combine kernel.
  const long units = static_cast<long>(B) * desc.H;
  const int target_waves = 2048;
  int want = static_cast<int>((target_waves + units - 1) / units);
  const int max_by_len = desc.n_max / 256 > 0 ? desc.n_max / 256 : 1;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  int nw = 1;
  if (wg_waves != nullptr) nw = want < kMaxWaves ? want : kMaxWaves;
  int s = (want + nw - 1) / nw;
  if (s > 256) s = 256;  // long contexts at small B*H: up to 256 splits fill the chip
  // tokens per split: a multiple of 128 for one wave, of 32 * nw for nw waves (each wave's part a
  // multiple of 32 tokens), so every batch but a part's last is full
  int c = (desc.n_max + s - 1) / s;
  c = nw == 1 ? (c + 127) / 128 * 128 : (c + 32 * nw - 1) / (32 * nw) * (32 * nw);
  s = (desc.n_max + c - 1) / c;
  *splits = s;
  *chunk = c;
  if (wg_waves != nullptr) *wg_waves = nw;
}

void decode_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves) {
  if (decode_uses_mfma2d(desc)) {
    decode2d_plan(desc, B, splits, chunk);
    if (wg_waves != nullptr) *wg_waves = 1;
  } else {
    valu_plan(desc, B, splits, chunk, wg_waves);
  }
}

size_t decode_workspace_bytes(const lla_desc& desc, int B) {
  int s, c, nw;
  decode_plan(desc, B, &s, &c, &nw);  // the plan the call runs
  if (decode_uses_mfma2d(desc)) return decode2d_workspace_bytes(desc, B, s);
  return valu_workspace_bytes(desc, B, s);
}

size_t valu_workspace_bytes(const lla_desc& desc, int rows, int splits) {
  if (splits <= 1) return 0;
  return static_cast<size_t>(rows) * desc.H * splits * (2 + desc.r_v) * sizeof(float);
}

namespace {

// Streaming partial kernel (contiguous or gather-indexed), then the split combine when S > 1.
hipError_t launch_valu(const DecodeParams& p, int dtype, PartialFn fn, hipStream_t stream) {
  if (p.splits > 1 &&
      static_cast<size_t>(p.B) * p.H * p.splits * (2 + p.r_v) * sizeof(float) > p.ws_bytes)
    return hipErrorInvalidValue;  // the plan does not fit the workspace: never launch
  const int hg = p.wg_heads > 1 ? p.wg_heads : 1;
  if (hg > 1 && (hg != kRopeGroup || p.d_rope == 0 || p.slots != nullptr || p.wg_waves > 1))
    return hipErrorInvalidValue;  // head groups: the compiled size, rotary read only
  const unsigned units = static_cast<unsigned>(p.B) * ((p.H + hg - 1) / hg) * p.splits;
  const int nw = hg > 1 ? hg : p.slots != nullptr ? 1 : std::min(std::max(p.wg_waves, 1), kMaxWaves);
  if (hg == 1 && p.chunk % (32 * nw) != 0) return hipErrorInvalidValue;  // waves take whole 32-token parts
  hipLaunchKernelGGL(fn, dim3(units), dim3(64 * nw), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  if (dtype == LLA_BF16 || dtype == LLA_BF16_Q8 || dtype == LLA_BF16_I8)
    hipLaunchKernelGGL(decode_combine_kernel<BF16>, dim3(p.B * p.H), dim3(kCombineThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_combine_kernel<F32>, dim3(p.B * p.H), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream) {
  // LLA-2D decode rows (one query per sequence) take the MFMA path when it is compiled
  if (p.variant == LLA_2D && p.rows_per_seq == 1 && !p.causal &&
      decode2d_mfma_supported(dtype, p.r_k, p.r_v, p.d))
    return launch_decode2d(p, dtype, stream);
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr) return hipErrorNotSupported;
  return launch_valu(p, dtype, e->fn, stream);
}

void gather_plan(const lla_desc& desc, int B, int budget, int* splits, int* chunk) {
  lla_desc g = desc;
  g.n_max = budget;  // splits range over list positions
  valu_plan(g, B, splits, chunk);
  // at most 2048 positions per split where 256 splits allow it: such a split's slot list is staged
  // in LDS by the kernel (a longer split is read without that staging)
  if (*chunk > 2048 && *splits < 256) {
    int s = (budget + 2047) / 2048;
    if (s > 256) s = 256;
    int c = (budget + s - 1) / s;
    c = (c + 127) / 128 * 128;
    *splits = (budget + c - 1) / c;
    *chunk = c;
  }
}

size_t gather_workspace_bytes(const lla_desc& desc, int B, int budget) {
  int s, c;
  gather_plan(desc, B, budget, &s, &c);
  return valu_workspace_bytes(desc, B, s);
}

bool rope_valu_supported(int dtype, int r_k, int r_v, int d_rope) {
  if (dtype != LLA_BF16 || !(d_rope == 32 || d_rope == 64 || d_rope == 128)) return false;
  const Entry* e = find(dtype, r_k, r_v);
  return e != nullptr && e->rfn.w64 != nullptr;
}

bool rope_supported(const lla_desc& desc, int d_rope) {
  if (desc.dtype != LLA_BF16 || !(d_rope == 32 || d_rope == 64 || d_rope == 128)) return false;
  // the LLA-2D MFMA read takes the branch as extra k-steps of its own contraction
  if (decode_uses_mfma2d(desc)) return true;
  const Entry* e = find(desc.dtype, desc.r_k, desc.r_v);
  return e != nullptr && e->rfn.w64 != nullptr;
}

// Head groups pay where the rotary rows, not the latents, set the L2 traffic, so whenever groups
// of kRopeGroup heads leave at most a quarter of the waves as placeholders (H = 8, 16, 40, 130 ...).
void rope_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves, int* wg_heads) {
  const int padded = (desc.H + kRopeGroup - 1) / kRopeGroup * kRopeGroup;
  if (!decode_uses_mfma2d(desc) && desc.H >= kRopeGroup && 4 * padded <= 5 * desc.H) {
    valu_plan(desc, B, splits, chunk);  // one wave per (row, head, split): no wave token parts
    *wg_waves = 1;
    *wg_heads = kRopeGroup;
    return;
  }
  decode_plan(desc, B, splits, chunk, wg_waves);
  *wg_heads = 1;
}

size_t rope_workspace_bytes(const lla_desc& desc, int B) {
  int s, c, nw, hg;
  rope_plan(desc, B, &s, &c, &nw, &hg);
  // LLA-2D on MFMA: the branch is fused into the read (q~ rows widened by up to 128 entries)
  if (decode_uses_mfma2d(desc)) return decode2d_workspace_bytes(desc, B, s, 128);
  // streaming read: the rotary scores are formed in the read; only its split partials
  return valu_workspace_bytes(desc, B, s);
}

hipError_t launch_decode_rope(const DecodeParams& p, int dtype, hipStream_t stream) {
  if (p.variant == LLA_2D && p.rows_per_seq == 1 && !p.causal &&
      decode2d_mfma_supported(dtype, p.r_k, p.r_v, p.d))
    return launch_decode2d(p, dtype, stream);  // rotary keys as extra MFMA k-steps of the read
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr) return hipErrorNotSupported;
  const bool grp = p.wg_heads > 1;
  const PartialFn fn = p.d_rope == 32 ? (grp ? e->rfn.g32 : e->rfn.w32)
                     : p.d_rope == 64 ? (grp ? e->rfn.g64 : e->rfn.w64)
                     : p.d_rope == 128 ? (grp ? e->rfn.g128 : e->rfn.w128) : nullptr;
  if (fn == nullptr) return hipErrorNotSupported;
  return launch_valu(p, dtype, fn, stream);
}

hipError_t launch_decode_gather(const DecodeParams& p, int dtype, hipStream_t stream) {
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr) return hipErrorNotSupported;
  if (p.slots == nullptr || p.budget <= 0 || p.rows_per_seq != 1 || p.causal)
    return hipErrorInvalidValue;
  return launch_valu(p, dtype, e->gfn, stream);
}

}  // namespace lla
