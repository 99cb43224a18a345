// Blockwise (flash) attention forward for prefill / encoder batches on gfx950.
//
// Method: the-ai.news, "Snelle attention-kernels en operatorfusie versnellen
// AI-modellen", section "FlashAttention-type aandacht en gepagineerde
// aandacht": queries, keys and values are processed per block; for each
// block a part of the scores is computed, the softmax statistics are updated
// and the output is accumulated on chip, so the T x T matrix is never stored.
// Tiling exists because on-chip memory is small ("讨论CUDA图形优化与推理加速",
// section on Flash Attention's role); ragged batches spend no compute on
// padding (ai-stack.site kernels update, "关键技术点" items 1-2).
//
// Per wavefront: 32 consecutive query rows of one (batch, query head). The
// workgroup streams the key/value rows of its kv head in tiles of BK keys
// through LDS (row-major, with a 16-byte-chunk XOR swizzle that keeps every
// LDS access below free of bank conflicts).
//
// Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16: keys on
// rows, the 32 queries of a wavefront on columns), so a lane holds 16 keys of
// one query per 32-key block: row max and row sum are in-lane reductions plus
// one exchange with lane l^32. After exp2 and rounding, the transposed scores
// are exactly the B operand of O^T += V^T P^T, so P never leaves registers.
// The V^T operand is read from the row-major V tile with ds_read_b64_tr_b16
// (gfx950's transposing LDS read: within 16 lanes, lane j receives element
// j + 16e of the concatenated 4-element chunks the lanes address). Q^T lives
// in registers for the whole key loop.
//
// Online softmax (base 2, x = s * scale * log2 e): per query the running max
// m, two running sums and the accumulator O^T. O is normalised by the sum of
// the probabilities after their rounding to the 16-bit input type, i.e. by the
// very weights the P.V product applies, so O is a weighted mean of value rows
// (a one-hot row returns its value row exactly); lse uses the fp32 sum of the
// unrounded probabilities. The max only moves when a tile's max exceeds it by
// more than kLazyRescale (in log2 units); otherwise p = 2^(x-m) is at most
// 2^kLazyRescale, which fp32 and the 16-bit P hold without loss of relative
// precision. O = O^T / l and lse = (m + log2 l) ln 2 are exact rearrangements
// of the same sums.
//
// Masking is a selection of -inf on the raw score (never an addition), and
// only on tiles that need it (the causal diagonal, the ragged / Tk tail).
// Value rows beyond the sequence are zero-filled in LDS so 0 * NaN cannot
// reach O. Causal tiles entirely above a wavefront's diagonal are skipped;
// causal workgroups are issued heaviest (last query tile) first, and the G
// query heads that share a kv head are placed on one XCD (one L2) together.
//
// Schedule: 4 wavefronts x 32 rows (128 query rows) per workgroup, two
// workgroups per CU (two wavefronts per SIMD, so one wavefront's MFMAs overlap
// the other's softmax), K/V tiles double-buffered in LDS with one barrier per
// tile: tile j+1 travels HBM -> LDS directly (buffer loads that write LDS)
// while tile j is consumed. LDS operand reads are issued ahead of the MFMAs
// that consume them (register double buffering). A step is one vector phase
// (tile j's exponentials) and one matrix phase (tile j's product, then tile
// j+1's scores); the two wavefronts of a SIMD overlap one's vector phase
// with the other's matrix phase.
//
// The FP8 form lags the P.V product by one tile: step j computes the scores
// of tile j+1 and the product of tile j-1 beside tile j's exponentials, over
// four-deep K/V rings in LDS whose loads stay in flight across barriers (the
// waits count tiles). Its 8-bit tiles keep the rings at 64 KiB per workgroup.
//
// FP8 form (contiguous E4M3 q, k, v; KV8 without PAGED): both products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), twice the bf16 rate.
// A lane's 32 contraction slots are 32 consecutive dims of its row for S^T,
// and for O^T += V^T P^T the lane's own 32 keys of the tile (the B operand P^T
// is the lane's 32 probabilities, rounded to E4M3 after scaling by 2^7; the
// A operand V^T is 4 ds_read_b64_tr_b8 in the same key order). Each tile's
// max is taken before its exponentials; the running max moves once it grows
// by more than 1 (log2), so p <= 2 and the scaled p stay <= 2^8; O is divided
// by the fp32 sum of the unrounded scaled p. Error
// of the rounding of P per output element (row i, column d): at most
// 2^-4 sum_j P_ij |v_jd| + 2^-17 max_j P_ij sum_j |v_jd| over the row's keys
// (2^-4 relative in E4M3's normal range, 2^-17 absolute below it).
//
// E4M3 form (chunked prefill over an FP8 cache, paged only): K/V tiles hold
// one byte per element; operand fragments are converted to the 16-bit type
// right after their LDS reads (exact), k_scale folds into the exponent factor
// and v_scale into the final normalisation. A K read takes 16 codes = the
// fragments of two k-steps (each k-step's 16 dims are split over the two lane
// halves in another order than in the 16-bit form, and Q's fragments follow
// the same order); a V^T fragment is one ds_read_b64_tr_b8 (8 keys of one
// column). K and V tiles use different swizzles, each conflict-free for its
// read pattern.
#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kLazyRescale = 8.0f;
// 16-bit products: bound on a lane's tile sum of p under the running max as it
// stands, past which the tile is redone after moving the max
constexpr float kOptimisticSum = 32768.0f;
// FP8 form: lazy margin of the running max and the matching scale 2^(8 - margin) of p
constexpr float kF8Margin = 1.0f;
constexpr float kF8PScaleLog2 = 8.0f - kF8Margin;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 16-byte chunk slot of (row, chunk c) inside an LDS row: c ^ f(row). LDS
// serves 256 bytes per cycle: 16 lanes of a 16-byte access, 32 lanes of an
// 8-byte one. The functions make every such lane group hit distinct banks for
// the K operand reads (16 consecutive rows, one chunk), the transposing V
// reads (32 lanes: 4 consecutive rows x 4 chunks) and the row-major tile
// writes. f depends only on row bits 0-3, which the offset hoisting relies on.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row >> 3) & 1) | (((row >> 2) & 1) << 1) | (((row >> 1) & 1) << 2);
}

// E4M3 tiles (rows of D bytes). K is read 16 bytes per lane at 16 rows x one
// chunk per 16 lanes: rows sharing the same 256-byte bank phase (equal parity
// at D = 128, equal row % 4 at D = 64) take distinct chunk swaps. V is read
// 8 bytes per lane (ds_read_b64_tr_b8) at rows {0-3, 8-11} (or {4-7, 12-15})
// x 4 chunk halves per 32 lanes; the swap (always even, whole 16-byte chunks
// stay together for the LDS-direct loads) is spread over row bits 1 and 3.
template <int D>
__device__ __forceinline__ int kswz8(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int vswz8(int row) {
  if constexpr (D == 128) return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
  else return 2 * ((row >> 3) & 1);
}
// the swizzle of a K (V = false) or V (V = true) tile
template <int D, bool KV8, bool V>
__device__ __forceinline__ int tswz(int row) {
  if constexpr (!KV8) return swz<D>(row);
  else if constexpr (V) return vswz8<D>(row);
  else return kswz8<D>(row);
}

template <int D, int BK, bool KV8 = false>
struct Shape {
  static constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;   // 32-row blocks of O^T
  static constexpr int KB = BK / 32;  // 32-key blocks of S^T
  static constexpr int PS = BK / 16;  // k-steps of O^T += V^T P^T
  static constexpr int RB = KV8 ? D : 2 * D;  // bytes per tile row
  static constexpr int C8 = RB / 16;  // 16-byte chunks per row
  static constexpr int TILE = BK * RB;
};

// Which (batch, head, query tile) this workgroup owns, and its bounds.
struct Geo {
  int b, hq, kvh, Lq, Lk, off, q_lo, nkt;
  const uint16_t* Qg;
  const uint16_t* Kg;
  const uint16_t* Vg;
  uint16_t* Og;
  float* Lg;
};

// Chunked prefill: keys the query tile's workgroup visits (its work), from
// the sequence's key count lk and row count lq; -1 for a tile past the rows.
template <int BQ, bool CAUSAL>
__device__ __forceinline__ int tile_work(int lk, int lq, int qt) {
  if (qt * BQ >= lq) return -1;
  return CAUSAL ? lk - lq + min((qt + 1) * BQ, lq) : lk;
}

// Chunked prefill, longest first: the rank-r (sequence, query tile) group in
// decreasing work (ties by sequence, then tile). The sequences of a chunked
// batch have different cached prefixes, so a fixed order leaves long groups
// for the end of the launch (about 7 % over the ideal makespan on the bench
// batch, against 2 % for this order, by a greedy-scheduling model). Lane l
// holds sequence l's counts (B <= 64); each lane ranks its groups against all
// others with the counts read by readlane, so the loop touches no memory.
template <int BQ, bool CAUSAL>
__device__ __forceinline__ void lpt_group(const PrefillArgs& a, int r, int& b, int& qt) {
  const int lane = threadIdx.x & 63;
  const int lk = lane < a.B ? min(a.ctx_lens[lane], a.max_blocks * 16) : 0;
  const int lq = lane < a.B ? (a.q_lens ? min(a.q_lens[lane], a.Tq) : a.Tq) : 0;
  const int ng = a.B * a.nqt;
  b = 0;
  qt = a.nqt;  // past the rows: exits (only for r >= ng, which the grid excludes)
  for (int g0 = 0; g0 < ng; g0 += 64) {  // wave-uniform
    const int gi = min(g0 + lane, ng - 1);
    const int bi = gi / a.nqt;
    const int wi = tile_work<BQ, CAUSAL>(__shfl(lk, bi), __shfl(lq, bi), gi % a.nqt);
    int rank = 0;
    for (int bj = 0; bj < a.B; ++bj) {
      const int lkj = __builtin_amdgcn_readlane(lk, bj);
      const int lqj = __builtin_amdgcn_readlane(lq, bj);
      for (int qj = 0; qj < a.nqt; ++qj) {
        const int wj = tile_work<BQ, CAUSAL>(lkj, lqj, qj);
        const int gj = bj * a.nqt + qj;
        rank += (wj > wi || (wj == wi && gj < gi)) ? 1 : 0;
      }
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(g0 + lane < ng && rank == r);
    if (hit) {
      const int gsel = __builtin_amdgcn_readfirstlane(g0 + (int)__builtin_ctzll(hit));
      b = gsel / a.nqt;
      qt = gsel % a.nqt;
      return;
    }
  }
}

template <int D, int BQ, int BK, bool CAUSAL, bool PAGED>
__device__ __forceinline__ Geo make_geo(const PrefillArgs& a) {
  Geo g;
  int id = blockIdx.x;
  if (a.xcd_remap) {  // members of a kv-head group land on one XCD (dispatch is round-robin over 8)
    const int x = id & 7, slot = id >> 3;
    id = ((slot / a.G) * 8 + x) * a.G + slot % a.G;
  }
  const int per = a.Hq * a.B;
  int qt = CAUSAL ? (a.nqt - 1 - id / per) : (id / per);
  const int rem = id % per;
  g.hq = rem % a.Hq;
  g.b = rem / a.Hq;
  if constexpr (PAGED) {
    if (a.lpt) {  // groups of Hq workgroups (one per query head) in decreasing work
      g.hq = id % a.Hq;
      lpt_group<BQ, CAUSAL>(a, id / a.Hq, g.b, qt);
    }
  }
  g.kvh = g.hq / a.G;
  if constexpr (PAGED) {
    // the newest Lq positions of a sequence of Lk cached tokens
    // (clamped to what the table and q can hold, which keeps every access in bounds)
    g.Lk = min(a.ctx_lens[g.b], a.max_blocks * 16);
    g.Lq = a.q_lens ? min(a.q_lens[g.b], a.Tq) : a.Tq;
    // (the stagers address the cache blocks themselves)
    g.Kg = nullptr;
    g.Vg = nullptr;
  } else {
    g.Lq = a.Tq;
    g.Lk = a.Tk;
    if (a.seq_lens) {
      g.Lq = a.seq_lens[g.b];
      g.Lk = g.Lq;
    }
    g.Kg = static_cast<const uint16_t*>(a.k) + (size_t)(g.b * a.Hkv + g.kvh) * a.Tk * D;
    g.Vg = static_cast<const uint16_t*>(a.v) + (size_t)(g.b * a.Hkv + g.kvh) * a.Tk * D;
  }
  g.off = g.Lk - g.Lq;  // bottom-right causal alignment
  g.q_lo = qt * BQ;
  g.Qg = static_cast<const uint16_t*>(a.q) + (size_t)(g.b * a.Hq + g.hq) * a.Tq * D;
  g.Og = static_cast<uint16_t*>(a.o) + (size_t)(g.b * a.Hq + g.hq) * a.Tq * D;
  g.Lg = a.lse ? a.lse + (size_t)(g.b * a.Hq + g.hq) * a.Tq : nullptr;
  int kend = g.Lk;  // exclusive key bound of the whole tile
  if (CAUSAL) kend = min(g.Lk, min(g.q_lo + BQ, g.Lq) + g.off);
  g.nkt = (g.q_lo < g.Lq && kend > 0) ? (kend + BK - 1) / BK : 0;
  return g;
}

// Per-wavefront accumulator state.
template <int D>
struct Acc {
  u32x4 qf[D / 16];    // Q^T fragments (B operand): lane holds Q[qrow][16s + 8h .. +8)
  f32x16 oacc[D / 32];
  float m, l, lr;      // running max (log2 units), fp32 sum, sum of the rounded p
};

// Column of the 8 dims lane half h holds in k-step s: 16s + 8h in the 16-bit
// form; in the E4M3 form k-steps 2p and 2p + 1 share one 32-dim group, lane
// half h holding dims 32p + 16h .. +16 (the first 8 in step 2p). In both,
// step s + D/32 holds the partner columns (+ D/2) of step s.
template <int D, bool KV8>
__device__ __forceinline__ int q_col(int s, int h) {
  return KV8 ? 32 * (s >> 1) + 16 * h + 8 * (s & 1) : 16 * s + 8 * h;
}

// The sign flip (qmode 1) and zeroing (qmode 2, and rows past the sequence)
// of Q's fragments, applied after load_q where Q is first used, so that Q's
// loads stay in flight behind the first tiles' loads until then.
template <class T, int D, bool F8>
__device__ __forceinline__ void q_modes(Acc<D>& st, const Geo& g, int qmode, int qrow) {
  const uint32_t flip = qmode == 1 ? (F8 ? 0x80808080u : 0x80008000u) : 0u;
  const bool zero = qmode == 2 || !(qrow < g.Lq);
#pragma unroll
  for (int s = 0; s < (F8 ? D / 32 : D / 16); ++s) st.qf[s] = zero ? u32x4{0, 0, 0, 0} : st.qf[s] ^ flip;
}

template <class T, int D, bool KV8, bool F8 = false>
__device__ __forceinline__ void load_q(Acc<D>& st, const Geo& g, int qrow, int h, const float* rope,
                                       int max_pos, const uint8_t* q8 = nullptr) {
  const bool live = qrow < g.Lq;
  if constexpr (F8) {
    // k-step p (64 dims): lane half h holds dims 64p + 32h .. +32 (32 codes)
    const uint8_t* src8 = q8 + (size_t)(live ? qrow : 0) * D + 32 * h;
#pragma unroll
    for (int p = 0; p < D / 64; ++p)
#pragma unroll
      for (int u = 0; u < 2; ++u) st.qf[2 * p + u] = *reinterpret_cast<const u32x4*>(src8 + 64 * p + 16 * u);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.oacc[i] = f32x16{};
    st.m = -__builtin_inff();
    st.l = 0.f;
    st.lr = 0.f;
    return;
  }
  const uint16_t* src = g.Qg + (size_t)(live ? qrow : 0) * D;
  u32x4 x[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) x[s] = *reinterpret_cast<const u32x4*>(src + q_col<D, KV8>(s, h));
  if (rope) {
    // rotary embedding at the row's position (Lk - Lq + row): fragment s < D/32
    // holds 8 columns of the first half, fragment s + D/32 their partners
    const float* tr = rope + (size_t)min(max(g.off + qrow, 0), max_pos - 1) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const int col = q_col<D, KV8>(s, h);
      float c[8], sn[8];
      *reinterpret_cast<f32x4*>(c) = *reinterpret_cast<const f32x4*>(tr + col);
      *reinterpret_cast<f32x4*>(c + 4) = *reinterpret_cast<const f32x4*>(tr + col + 4);
      *reinterpret_cast<f32x4*>(sn) = *reinterpret_cast<const f32x4*>(tr + D / 2 + col);
      *reinterpret_cast<f32x4*>(sn + 4) = *reinterpret_cast<const f32x4*>(tr + D / 2 + col + 4);
      rope8<T>(x[s], x[s + D / 32], c, sn);
    }
  }
#pragma unroll
  for (int s = 0; s < D / 16; ++s) st.qf[s] = x[s];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) st.oacc[i] = f32x16{};
  st.m = -__builtin_inff();
  st.l = 0.f;
  st.lr = 0.f;
}

// Per-lane LDS read offsets (identical for every tile). E4M3 tiles: one per
// read. 16-bit tiles: a base per operand, from which koff / voff derive each
// read's offset with one XOR (see make_offs), so the key loop holds 2
// registers instead of D/8.
template <int D, int BK>
struct Offs {
  int k[D / 16];
  int v[D / 32][2];
  int k0, v0;
};

template <int D, int BK, bool KV8, bool F8 = false>
__device__ __forceinline__ void make_offs(Offs<D, BK>& o, int lane) {
  using S = Shape<D, BK, KV8>;
  const int h = lane >> 5, c32 = lane & 31, g16 = lane >> 4, i16 = lane & 15;
  o.k0 = 0;
  o.v0 = 0;
  if constexpr (KV8) {
    if constexpr (F8) {
      // K: 64-dim step p from two 16-byte reads of row c32 at chunks 4p + 2h, +1
#pragma unroll
      for (int p = 0; p < D / 64; ++p)
#pragma unroll
        for (int u = 0; u < 2; ++u) o.k[2 * p + u] = c32 * S::RB + 16 * ((4 * p + 2 * h + u) ^ kswz8<D>(c32));
    } else {
      // K: k-steps 2p, 2p + 1 from one 16-byte read of row c32 at chunk 2p + h
#pragma unroll
      for (int p = 0; p < S::KS / 2; ++p) o.k[p] = c32 * S::RB + 16 * ((2 * p + h) ^ kswz8<D>(c32));
    }
    // V^T via ds_read_b64_tr_b8: in each 16-lane group, lane j receives byte
    // (j & 7) of the 8 bytes read by lanes 2e + (j >> 3). Element e of lane
    // half h is key 8(e >> 2) + 4h + (e & 3) of the k-step (P^T's order), so
    // lane i addresses that key for e = i >> 1 at columns
    // 32db + 16(g16 % 2) + 8(i & 1) .. +8 and receives column 32db + 16(g16 % 2) + i.
    const int e = i16 >> 1;
    const int row = 8 * (e >> 2) + 4 * h + (e & 3);  // plus 16s per k-step (keeps the swizzle)
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      o.v[db][0] = row * S::RB + 16 * ((2 * db + (g16 & 1)) ^ vswz8<D>(row)) + 8 * (i16 & 1);
      o.v[db][1] = o.v[db][0];
    }
    return;
  }
  // K operand of k-step s: row kb*32 + c32, chunk (2s + h) ^ swz(row); swz(row)
  // does not depend on kb because kb*32 is a multiple of 16. As 2s + h =
  // 2s ^ h, the chunk is (h ^ swz) ^ 2s: koff(s) = k0 ^ 32s (the row's bytes
  // start at a multiple of RB, above the chunk bits).
  o.k0 = c32 * S::RB + 16 * (h ^ swz<D>(c32));
  // V^T operand: k-step s covers keys 16s + 8r + 4h + (0..3) for element group
  // r = 0, 1; lane i of 16-lane group g addresses row (those keys' base) + i/4
  // at columns 32db + 16(g%2) + 4(i%4) and receives column 32db + 16(g%2) + i.
  // The swizzle of row 16s + 8r + vr depends only on r and the lane (16s + 8r
  // is a multiple of 8), so the offset is voff(db, r) + 16s * RB. The column's
  // chunk is 4db ^ (vc / 8), and swz(8r + vr) = swz(vr) ^ 2r (D = 128) or
  // ^ r (D = 64), so voff(db, r) = (v0 ^ 64db ^ XR r) + 8r RB, XR = 32 or 16.
  const int vr = 4 * h + (i16 >> 2);
  const int vc = 16 * (g16 & 1) + 4 * (i16 & 3);
  o.v0 = vr * S::RB + 16 * ((vc >> 3) ^ swz<D>(vr)) + 2 * (vc & 7);
}

template <int D, int BK, bool KV8>
__device__ __forceinline__ int koff(const Offs<D, BK>& o, int s) {
  return KV8 ? o.k[s] : (o.k0 ^ (32 * s));
}
template <int D, int BK, bool KV8>
__device__ __forceinline__ int voff(const Offs<D, BK>& o, int db, int r) {
  if constexpr (KV8) return o.v[db][r];
  return (o.v0 ^ (64 * db) ^ ((D == 128 ? 32 : 16) * r)) + 8 * 2 * D * r;
}

// S^T = K Q^T for one tile in LDS. The K fragments of k-step s+2 are read
// while the MFMAs of step s run (a three-deep register ring). No scheduling
// directives: callers add the pattern they want.
constexpr int kQkDepth = 2;

// fp8 x fp8 -> fp32, 32x32x64, unit block scales (E8M0 127 = 2^0)
__device__ __forceinline__ f32x16 mfma_f8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

template <class T, int D, int BK, bool KV8 = false, bool F8 = false>
__device__ __forceinline__ void tile_qk_plain(f32x16 (&sacc)[BK / 32], const char* Ks, const Offs<D, BK>& o,
                                              const Acc<D>& st) {
  using S = Shape<D, BK, KV8>;
  if constexpr (F8) {
    u32x4 fr[D / 64][S::KB][2];
#pragma unroll
    for (int p = 0; p < D / 64; ++p)
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) fr[p][kb][u] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * S::RB + o.k[2 * p + u]);
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int p = 0; p < D / 64; ++p)
        sacc[kb] = mfma_f8(fr[p][kb][0], fr[p][kb][1], st.qf[2 * p], st.qf[2 * p + 1], sacc[kb]);
    }
    return;
  }
  if constexpr (KV8) {
    // one 16-byte read per (key block, k-step pair) = the two steps' fragments
    // as 16 codes; the next pair's reads go out before this pair's MFMAs
    u32x4 raw[2][S::KB];
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) {
      sacc[kb] = f32x16{};
      raw[0][kb] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * S::RB + o.k[0]);
    }
#pragma unroll
    for (int p = 0; p < S::KS / 2; ++p) {
      if (p + 1 < S::KS / 2) {
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb)
          raw[(p + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * S::RB + o.k[p + 1]);
      }
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb) {
        const u32x4 r = raw[p & 1][kb];
        sacc[kb] = T::mfma32(e4m3x8<T>(u32x2{r[0], r[1]}), st.qf[2 * p], sacc[kb]);
        sacc[kb] = T::mfma32(e4m3x8<T>(u32x2{r[2], r[3]}), st.qf[2 * p + 1], sacc[kb]);
      }
    }
    return;
  }
  constexpr int DEPTH = kQkDepth;
  u32x4 fr[DEPTH + 1][S::KB];
#pragma unroll
  for (int kb = 0; kb < S::KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
      fr[s][kb] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * S::RB + koff<D, BK, false>(o, s));
#pragma unroll
  for (int s = 0; s < S::KS; ++s) {
    if (s + DEPTH < S::KS) {
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb)
        fr[(s + DEPTH) % (DEPTH + 1)][kb] =
            *reinterpret_cast<const u32x4*>(Ks + kb * 32 * S::RB + koff<D, BK, false>(o, s + DEPTH));
    }
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) sacc[kb] = T::mfma32(fr[s % (DEPTH + 1)][kb], st.qf[s], sacc[kb]);
  }
}

template <class T, int D, int BK, bool KV8 = false, bool F8 = false>
__device__ __forceinline__ void tile_qk(f32x16 (&sacc)[BK / 32], const char* Ks, const Offs<D, BK>& o,
                                        const Acc<D>& st) {
  using S = Shape<D, BK>;
  tile_qk_plain<T, D, BK, KV8, F8>(sacc, Ks, o, st);
  if constexpr (KV8) return;  // compiler-scheduled
  // schedule: the reads of step s+DEPTH go out before the MFMAs of step s
  __builtin_amdgcn_sched_group_barrier(0x100, kQkDepth * S::KB, 0);
#pragma unroll
  for (int s = 0; s < S::KS; ++s) {
    if (s + kQkDepth < S::KS) __builtin_amdgcn_sched_group_barrier(0x100, S::KB, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, S::KB, 0);
  }
}

// Two transposing reads give the 8-element V^T operand of one MFMA.
template <class T, int D, int BK, bool KV8 = false>
__device__ __forceinline__ u32x4 vt_frag(const char* Vs, const Offs<D, BK>& o, int db, int s) {
  using S = Shape<D, BK, KV8>;
  if constexpr (KV8) {
    const i32x2 v8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + 16 * s * S::RB + o.v[db][0]));
    return e4m3x8<T>(__builtin_bit_cast(u32x2, v8));
  }
  const i16x4 p0 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + 16 * s * S::RB + voff<D, BK, false>(o, db, 0)));
  const i16x4 p1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + 16 * s * S::RB + voff<D, BK, false>(o, db, 1)));
  const u32x2 a0 = __builtin_bit_cast(u32x2, p0);
  const u32x2 a1 = __builtin_bit_cast(u32x2, p1);
  return u32x4{a0[0], a0[1], a1[0], a1[1]};
}

// O^T += V^T P^T for one tile in LDS; fragments of k-step s+1 are read while
// the DB independent MFMAs of step s run.
template <class T, int D, int BK, bool KV8 = false, bool F8 = false>
__device__ __forceinline__ void tile_pv(Acc<D>& st, const u32x4 (&pf)[BK / 16], const char* Vs,
                                        const Offs<D, BK>& o) {
  using S = Shape<D, BK>;
  if constexpr (F8) {
    static_assert(BK == 64, "one 64-key product per tile");
    // V^T: the lane's 32 keys of the tile in P^T's byte order (4 transposing reads)
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      u32x2 v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                             (lds_i32x2*)(Vs + 16 * t * D + o.v[db][0])));
      st.oacc[db] = mfma_f8(u32x4{v[0][0], v[0][1], v[1][0], v[1][1]}, u32x4{v[2][0], v[2][1], v[3][0], v[3][1]},
                            pf[0], pf[1], st.oacc[db]);
    }
    return;
  }
  u32x4 fr[2][S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) fr[0][db] = vt_frag<T, D, BK, KV8>(Vs, o, db, 0);
#pragma unroll
  for (int s = 0; s < S::PS; ++s) {
    if (s + 1 < S::PS) {
#pragma unroll
      for (int db = 0; db < S::DB; ++db) fr[(s + 1) & 1][db] = vt_frag<T, D, BK, KV8>(Vs, o, db, s + 1);
    }
#pragma unroll
    for (int db = 0; db < S::DB; ++db) st.oacc[db] = T::mfma32(fr[s & 1][db], pf[s], st.oacc[db]);
  }
}

// Mask and online-softmax statistics for one tile of scores: the tile max,
// and the (lazy) rescale of the running sums and of O. Returns the max to
// subtract in the exponentials.
// Mask (diagonal and tail tiles only): keys past the row's last visible key
// become -inf.
template <int D, int BK, bool CAUSAL>
__device__ __forceinline__ void softmax_mask(f32x16 (&sacc)[BK / 32], const Geo& g, int k0, int qrow, int w_lo, int h) {
  using S = Shape<D, BK>;
  const bool need_mask = (k0 + BK > g.Lk) || (CAUSAL && k0 + BK - 1 > w_lo + g.off);
  if (need_mask) {
    const int lim = CAUSAL ? min(g.Lk - 1, qrow + g.off) : (g.Lk - 1);
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        sacc[kb][r] = key > lim ? -__builtin_inff() : sacc[kb][r];
      }
  }
}

// Tile max in log2 units (raw scores times cexp > 0; -inf stays -inf).
template <int D, int BK>
__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[BK / 32], float cexp) {
  using S = Shape<D, BK>;
  float mx = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  return half_swap_max(mx) * cexp;
}

// Lazy rescale: the running max moves to the tile max mx where that exceeds
// it by more than the margin (16-bit products: 8, so p <= 2^8; FP8 form: 1,
// so p <= 2 and the scaled p * 2^7 stay <= 2^8, inside E4M3's range). Callers
// take the wavefront-wide vote first; a lane whose max stays keeps alpha = 1.
template <int D, bool F8>
__device__ __forceinline__ bool max_grows(float mx, const Acc<D>& st) {
  return mx > st.m + (F8 ? kF8Margin : kLazyRescale);
}
template <int D, bool F8>
__device__ __forceinline__ void rescale(Acc<D>& st, float mx) {
  const bool grow = max_grows<D, F8>(mx, st);
  const float m_new = grow ? mx : st.m;
  const float alpha = grow ? fast_exp2(st.m - m_new) : 1.f;  // m = -inf -> 0
  st.m = m_new;
  st.l *= alpha;
  st.lr *= alpha;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) st.oacc[i] *= alpha;
}
template <int D>
__device__ __forceinline__ float max_to_subtract(const Acc<D>& st) {
  return st.m == -__builtin_inff() ? 0.f : st.m;
}

// p = 2^(s*c - m) for the lane's 16 scores of key block kb, their fp32
// partial sums and the P^T operand (no branches). 16-bit: two groups of 8
// (group 2 kb + hf), each with the sum of its rounded p, which the normaliser
// adds (the weights the P.V product applies). FP8 form: four groups of 4,
// p * 2^7 rounded to E4M3; byte 16 kb + r of the lane's P^T operand is key
// kb*32 + 8(r/4) + 4h + r%4, as in the scores' layout.
template <class T, int D, int BK, bool F8>
__device__ __forceinline__ void exp_block(const f32x16 (&sacc)[BK / 32], u32x4 (&pf)[BK / 16], int kb,
                                          float (&lsum)[BK / 8], float (&lrsum)[BK / 8], float msub, float cexp) {
  if constexpr (F8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = fast_exp2(__builtin_fmaf(sacc[kb][4 * w + e], cexp, kF8PScaleLog2 - msub));
      lsum[4 * kb + w] = (p[0] + p[1]) + (p[2] + p[3]);
      // the first conversion keeps the other half of its destination: pass
      // the register's old bits (overwritten by the second) rather than a
      // zero that would cost a move per word
      int r = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], (int)pf[kb][w], false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], r, true);
      pf[kb][w] = (uint32_t)r;
    }
    return;
  }
  // one partial sum per 8 probabilities keeps the dependency chains short, so
  // the work interleaves with the matrix instructions beside it
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int i = kb * 2 + hf;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(sacc[kb][8 * hf + e], cexp, -msub));
    lsum[i] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    const u32x4 pk = {T::pack2(p[0], p[1]), T::pack2(p[2], p[3]), T::pack2(p[4], p[5]), T::pack2(p[6], p[7])};
    lrsum[i] = T::sum2(pk[3], T::sum2(pk[2], T::sum2(pk[1], T::sum2(pk[0], 0.f))));
    pf[i] = pk;
  }
}

// Adds a tile's partial sums to the running sums (in a fixed order); returns
// the tile's fp32 sum.
template <int D, int BK, bool F8>
__device__ __forceinline__ float exp_finish(Acc<D>& st, const float (&lsum)[BK / 8], const float (&lrsum)[BK / 8]) {
  constexpr int NG = F8 ? BK / 8 : BK / 16;
  float ls = 0.f, lrs = 0.f;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    ls += lsum[i];
    if constexpr (!F8) lrs += lrsum[i];
  }
  st.l += ls;
  // FP8 form: O is divided by the sum of the unrounded scaled p
  st.lr = F8 ? st.l : st.lr + lrs;
  return ls;
}

// The exponentials of a whole tile; returns its fp32 sum.
template <class T, int D, int BK, bool F8 = false>
__device__ __forceinline__ float softmax_exp(const f32x16 (&sacc)[BK / 32], u32x4 (&pf)[BK / 16], Acc<D>& st,
                                             float msub, float cexp) {
  float lsum[BK / 8], lrsum[BK / 8];
#pragma unroll
  for (int kb = 0; kb < BK / 32; ++kb) exp_block<T, D, BK, F8>(sacc, pf, kb, lsum, lrsum, msub, cexp);
  return exp_finish<D, BK, F8>(st, lsum, lrsum);
}

// Tile max and lazy rescale; returns the max to subtract.
template <class T, int D, int BK, bool F8 = false>
__device__ __forceinline__ float softmax_max(const f32x16 (&sacc)[BK / 32], Acc<D>& st, float cexp) {
  const float mx = tile_max<D, BK>(sacc, cexp);
  if (__builtin_amdgcn_ballot_w64(max_grows<D, F8>(mx, st))) rescale<D, F8>(st, mx);
  return max_to_subtract(st);
}

// O = O^T / l, lse = (m + log2 l) ln 2; padding rows -> 0, -inf.
template <class T, int D>
__device__ __forceinline__ void epilogue(const Acc<D>& st, const Geo& g, int Tq, int qrow, int h,
                                         float vscale = 1.f, float lse_shift = 0.f) {
  const float l_tot = half_swap_sum(st.l);
  const float lr_tot = half_swap_sum(st.lr);
  if (qrow >= Tq) return;
  const bool has = qrow < g.Lq && l_tot > 0.f;
  const float inv = has ? vscale / lr_tot : 0.f;
  uint16_t* orow = g.Og + (size_t)qrow * D + 4 * h;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 pk = {T::pack2(st.oacc[db][4 * q4 + 0] * inv, st.oacc[db][4 * q4 + 1] * inv),
                  T::pack2(st.oacc[db][4 * q4 + 2] * inv, st.oacc[db][4 * q4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * q4) = pk;
    }
  if (g.Lg && h == 0) g.Lg[qrow] = has ? (st.m + fast_log2(l_tot) - lse_shift) * kLn2 : -__builtin_inff();
}

// Global -> LDS staging of K or V tiles (row-major, swizzled) with buffer
// loads that write LDS directly (no registers, no LDS store instructions).
// One such wavefront instruction fills 1 KiB of consecutive LDS: lane l writes
// bytes [16 l, 16 l + 16) after a wave-uniform base. So instruction n of a tile
// covers rows n*RPI .. n*RPI + RPI - 1, lane l the row n*RPI + l / C8 at slot
// p = l % C8, and the lane fetches the global chunk that the swizzle places in
// that slot, c = p ^ f(row). The descriptor starts at the tile's first row and
// covers only the rows below the sequence length: the hardware writes zeros
// for the rest (no branch, no access beyond the tensor).
constexpr int kBufferDword3 = 0x00020000;  // raw (untyped) buffer, 32-bit data

typedef __attribute__((address_space(3))) void lds_void;

template <int D, int BK, int THREADS, bool PAGED, bool KV8 = false, bool V = false>
struct Stager {
  using S = Shape<D, BK, KV8>;
  static constexpr int NW = THREADS / 64;
  static constexpr int RPI = 1024 / S::RB;      // rows per wavefront instruction
  static constexpr int CPT = BK / (RPI * NW);   // instructions per wavefront per tile
  static_assert(CPT >= 1 && BK % (RPI * NW) == 0, "staging shape");
  static_assert(16 % RPI == 0, "an instruction's rows lie in one cache block");
  static constexpr int EPT = BK / 16;         // cache blocks per tile (paged form)
  // paged form: wavefront w stages cache block w of each tile (its 16 rows in
  // CPT instructions), so one descriptor covers all its loads of the tile
  static_assert(!PAGED || EPT == NW, "paged staging: one cache block per wavefront");
  int voff[CPT];  // per-lane byte offset of the fetched chunk (within the tile, or within the cache block)
  int loff[CPT];  // wave-uniform LDS byte offset of the instruction within the tile
  int wblk;       // paged: the wave's cache block within a tile
  const char* base;
  size_t bstride;   // paged: bytes per physical block (all kv heads)
  const int* tbl;   // paged: the sequence's block-table row, in LDS

  __device__ __forceinline__ void init(const char* b, int tid, size_t block_stride = 0,
                                       const int* table = nullptr) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      // contiguous: instruction i of wave w covers rows (i*NW + w)*RPI ..;
      // paged: rows 16w + i*RPI .. (block w of the tile)
      const int r0 = PAGED ? 16 * w + i * RPI : (i * NW + w) * RPI;
      const int row = r0 + l / S::C8;
      const int chunk = 16 * ((l % S::C8) ^ tswz<D, KV8, V>(row));
      voff[i] = (PAGED ? row % 16 : row) * S::RB + chunk;
      loff[i] = r0 * S::RB;
    }
    wblk = w;
    base = b;
    bstride = block_stride;
    tbl = table;
  }
  // Paged form: the physical block ids of tile kt's cache blocks, read with
  // one LDS access (the same address in every lane) and made wave-uniform.
  __device__ __forceinline__ void entries(int kt, int (&e)[EPT]) const {
    if constexpr (PAGED) {
      static_assert(EPT == 4, "one 16-byte table read per tile");
      const int idx = min(kt * EPT, kMaxPagedPrefillBlocks - EPT);
      const u32x4 v = *reinterpret_cast<const u32x4*>(tbl + idx);
#pragma unroll
      for (int i = 0; i < EPT; ++i) e[i] = __builtin_amdgcn_readfirstlane((int)v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < EPT; ++i) e[i] = 0;
    }
    (void)kt;
  }
  // Issues the loads of tile kt into the LDS tile at `tile`; they complete
  // asynchronously (wait for the vector memory counter before reading).
  // e: the tile's physical blocks (paged form only).
  __device__ __forceinline__ void load(int kt, int Lk, char* tile, const int (&e)[EPT]) const {
    const int k0 = kt * BK;
    if constexpr (!PAGED) {
      // uniform by construction; readfirstlane tells the compiler so (a
      // descriptor in vector registers would need a loop per load)
      const int rows = __builtin_amdgcn_readfirstlane(min(max(Lk - k0, 0), BK));
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(base + (size_t)k0 * S::RB), (short)0, rows * S::RB, kBufferDword3);
#pragma unroll
      for (int i = 0; i < CPT; ++i) load_lds(rsrc, tile + loff[i], voff[i]);
      (void)e;
    } else {
      // the wave's cache block: its physical block, and only its rows below
      // Lk (a block past the sequence, or an unmapped one (id -1 in the LDS
      // table), gets none: nothing is read and the LDS rows receive zeros).
      // e[wblk], written as a mask-and-or over the candidates: as a select
      // chain the compiler turns it into an indexed load from a stack copy of
      // e (a scratch store and load per tile)
      int phys = 0;
#pragma unroll
      for (int j = 0; j < EPT; ++j) phys |= e[j] & -(int)(wblk == j);
      const int lb = k0 / 16 + wblk;
      const int rows = __builtin_amdgcn_readfirstlane(phys < 0 ? 0 : min(max(Lk - 16 * lb, 0), 16));
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(base + (size_t)(rows > 0 ? phys : 0) * bstride), (short)0, rows * S::RB, kBufferDword3);
#pragma unroll
      for (int i = 0; i < CPT; ++i) load_lds(rsrc, tile + loff[i], voff[i]);
    }
  }
  static __device__ __forceinline__ void* uniform_ptr(const char* ptr) {
    const uint64_t p = reinterpret_cast<uint64_t>(ptr);
    return reinterpret_cast<void*>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p));
  }
  // The host compilation pass of this file does not know the LDS-load
  // builtin (and would then drop the kernels' host stubs); the function is
  // only ever compiled for the device.
  static __device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t rsrc, char* dst, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    // The LDS address passes through an empty asm statement, which hides
    // which LDS array the load writes: the compiler then inserts no waits of
    // its own before LDS reads (its per-array tracking of these loads is
    // coarse across loop iterations and would wait for tiles the kernel
    // means to leave in flight). Every LDS read of a staged tile follows the
    // kernel's explicit wait and barrier.
    uint32_t lds = (uint32_t)(uintptr_t)(lds_void*)dst;
    asm volatile("" : "+s"(lds));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(uintptr_t)lds, 16, voffset, 0, 0, 0);
#else
    (void)rsrc;
    (void)dst;
    (void)voffset;
#endif
  }
};

// Waits until this wavefront's LDS-bound loads have landed, then synchronises
// the workgroup so that every wavefront's loads are visible.
__device__ __forceinline__ void staged_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// The end of a tile's arithmetic in the double-buffered key loop and its
// debug form (16-bit products: contiguous and paged 16-bit tiles, paged E4M3
// tiles): a lane whose 32 probabilities sum past 2^15 (or to inf / NaN: the
// first visible tile, where the running max is -inf) needs the running max
// moved first, so the tile's exponentials are redone after the lazy rescale
// (below that sum every p <= 2^15 stays inside fp16's range and the P operand
// keeps the relative precision of any other p); then O^T += V^T P^T.
template <class T, int D, int BK>
__device__ __forceinline__ void redo_tile(const f32x16 (&s_cur)[BK / 32], u32x4 (&pf)[BK / 16], Acc<D>& st, float ls,
                                          float l0, float lr0, float cexp) {
  if (__builtin_amdgcn_ballot_w64(!(ls <= kOptimisticSum))) {
    st.l = l0;
    st.lr = lr0;
    const float m2 = softmax_max<T, D, BK>(s_cur, st, cexp);
    softmax_exp<T, D, BK>(s_cur, pf, st, m2, cexp);
  }
}
template <class T, int D, int BK, bool KV8>
__device__ __forceinline__ void finish_tile(const f32x16 (&s_cur)[BK / 32], u32x4 (&pf)[BK / 16], Acc<D>& st,
                                            const Offs<D, BK>& o, const char* vcur, float ls, float l0, float lr0,
                                            float cexp) {
  redo_tile<T, D, BK>(s_cur, pf, st, ls, l0, lr0, cexp);
  __builtin_amdgcn_s_setprio(2);
  tile_pv<T, D, BK, KV8>(st, pf, vcur, o);
  __builtin_amdgcn_s_setprio(0);
}

// Issue order of the matrix phase of a 16-bit step (S of the next tile, then
// P.V of this one): the first 6 LDS reads (K fragments), then each MFMA
// followed by the next 2 reads during S and the next one during P.V (the
// reads run K, then V^T). Each MFMA's operand was then read several MFMAs
// earlier. Left to itself the compiler reads each pair of K fragments just
// before its two MFMAs, which then wait for the full LDS latency; ordered,
// the kernel measured 3-4 % faster.
template <int D, int BK>
__device__ __forceinline__ void matrix_phase_order() {
  constexpr int NPV = (D / 32) * (BK / 16), NQK = (D / 16) * (BK / 32);
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// One key step kt of the double-buffered loop (16-bit products). On entry
// the scores of tile kt (s_cur) are in registers, K of tile kt+1 and V of
// tile kt are in LDS. The step starts the loads of K_{kt+2} and V_{kt+1} into
// the buffers read one step earlier, then
//   * masks tile kt where needed (VALU);
//   * computes the exponentials, sums and packing of tile kt (VALU) under
//     the running max as it stands (no tile max on the way);
//   * computes S of tile kt+1 and accumulates O^T += V^T P^T for tile kt
//     (MFMA, at raised priority);
// and ends with the wait for its loads and a barrier.
template <class T, int D, int BK, bool CAUSAL, bool KV8, class KStg, class VStg>
__device__ __forceinline__ void pipe_step(int kt, const char* kcur, const char* vcur, char* kload, char* vload,
                                          f32x16 (&s_cur)[BK / 32], f32x16 (&s_nxt)[BK / 32],
                                          const KStg& ks, const VStg& vs,
                                          int (&ecar)[KStg::EPT], Acc<D>& st, const Offs<D, BK>& o_in,
                                          const Geo& g, bool wave_live, int w_last, int w_lo, int qrow, int h,
                                          float cexp) {
  using S = Shape<D, BK>;
  // 16-bit tiles: the offset bases pass through an empty asm statement, so the
  // per-read offsets derived from them are computed inside the step, where
  // they are used, instead of living in registers across the loop
  Offs<D, BK> o = o_in;
  if constexpr (!KV8) asm volatile("" : "+v"(o.k0), "+v"(o.v0));
  // (paged form) ecar: the physical blocks of tile kt+1, read one step earlier
  // for its K and reused now for its V
  if (kt + 2 < g.nkt) {
    int enew[KStg::EPT];
    ks.entries(kt + 2, enew);
    ks.load(kt + 2, g.Lk, kload, enew);
    if (kt + 1 < g.nkt) vs.load(kt + 1, g.Lk, vload, ecar);
#pragma unroll
    for (int i = 0; i < KStg::EPT; ++i) ecar[i] = enew[i];
  } else if (kt + 1 < g.nkt) {
    vs.load(kt + 1, g.Lk, vload, ecar);
  }
  // causal: tiles entirely above this wavefront's part of the diagonal are
  // skipped (monotone in kt, so the next tile's work implies this one's)
  const bool work = wave_live && (!CAUSAL || kt * BK <= w_last);
  if (work) {
    u32x4 pf[S::PS];
    softmax_mask<D, BK, CAUSAL>(s_cur, g, kt * BK, qrow, w_lo, h);
    const float l0 = st.l, lr0 = st.lr;
    const float msub = st.m;
    // this tile's exponentials first, then the next tile's scores and this
    // tile's product back to back at raised priority: one vector phase and
    // one matrix phase per step, which the two wavefronts of a SIMD overlap
    // with each other (faster than the next tile's scores before the
    // exponentials, and than an explicit MFMA/VALU interleave of the two)
    const float ls = softmax_exp<T, D, BK>(s_cur, pf, st, msub, cexp);
    redo_tile<T, D, BK>(s_cur, pf, st, ls, l0, lr0, cexp);
    __builtin_amdgcn_s_setprio(2);
    if constexpr (KV8) {
      tile_pv<T, D, BK, KV8>(st, pf, vcur, o);
      const bool work_next = kt + 1 < g.nkt && (!CAUSAL || (kt + 1) * BK <= w_last);
      if (work_next) tile_qk_plain<T, D, BK, KV8>(s_nxt, kcur, o, st);
    } else {
      // The next tile's scores are computed with every tile's product, also
      // past the last tile or above this wavefront's diagonal, where they are
      // never read (the buffer then holds an older tile or unwritten LDS: no
      // load is in flight into it). With no branch between them, both products
      // are one block of code whose LDS reads can be issued ahead. The scores
      // go first: the next step's exponentials wait for them, while P.V's
      // results are not read again until the next P.V, so its last MFMAs
      // overlap the wavefront's barrier and next vector phase.
      tile_qk_plain<T, D, BK, KV8>(s_nxt, kcur, o, st);
      tile_pv<T, D, BK, KV8>(st, pf, vcur, o);
      matrix_phase_order<D, BK>();
    }
    __builtin_amdgcn_s_setprio(0);
  }
  staged_barrier();
}

// The matrix and vector work of a lagged step (FP8 form): O^T +=
// V_{kt-1}^T P_{kt-1}^T (PREV) and S_{kt+1} = K_{kt+1} Q^T (NEXT) on the
// matrix cores, while the vector ALU computes tile kt's exponentials, sums and
// P^T operand. Neither product reads what the exponentials write, so the two
// units overlap (the compiler interleaves them).
template <class T, int D, int BK, bool KV8, bool F8, bool PREV, bool NEXT>
__device__ __forceinline__ void lag_body(const f32x16 (&s_cur)[BK / 32], f32x16 (&s_nxt)[BK / 32],
                                         u32x4 (&pcur)[BK / 16], const u32x4 (&pprev)[BK / 16], const char* kcur,
                                         const char* vprev, Acc<D>& st, const Offs<D, BK>& o, float msub,
                                         float cexp) {
  float lsum[BK / 8], lrsum[BK / 8];
  if constexpr (PREV) tile_pv<T, D, BK, KV8, F8>(st, pprev, vprev, o);
  exp_block<T, D, BK, F8>(s_cur, pcur, 0, lsum, lrsum, msub, cexp);
  if constexpr (NEXT) tile_qk_plain<T, D, BK, KV8, F8>(s_nxt, kcur, o, st);
  exp_block<T, D, BK, F8>(s_cur, pcur, 1, lsum, lrsum, msub, cexp);
  exp_finish<D, BK, F8>(st, lsum, lrsum);
}

// Waits until at most N tiles of this wavefront's loads (CPT instructions
// each) are in flight, then synchronises the workgroup (deep ring). The vector
// memory counter drains in issue order, so the older tiles have landed. The
// barrier is written without __syncthreads, whose fence would wait for every
// load; the LDS counter is drained so that no read of a buffer is still in
// flight when another wavefront's loads may refill it, and the memory clobber
// keeps the compiler's LDS accesses on their side of the barrier.
template <int N, int CPT>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N * CPT) : "memory");
}

// One key step kt of the lagged pipeline of the FP8 form, over four-deep K
// and V rings (K four tiles ahead of the scores that use it, V three ahead of
// its product). With the matrix products twice as fast as in 16 bits, the
// exponentials would otherwise dominate the step; the lag puts both products
// of a step beside them. (The 16-bit forms keep the double-buffered step
// above: holding the previous tile's P^T as well would take the registers
// their fragment prefetch needs at two wavefronts per SIMD, and a 16-bit ring
// would leave room for one workgroup per CU only.) On entry the scores of
// tile kt are in registers (s_cur), and so is the P^T operand of tile kt-1
// (pprev); LDS holds K_{kt+1} and V_{kt-1}. The step
//   * starts the loads of K_{kt+4} and V_{kt+2} into the buffers that held
//     K_kt and V_{kt-2} (read last in step kt-1, which ended with a barrier);
//     both are issued every step, also past the last tile (an empty
//     descriptor: nothing is read, the LDS rows receive zeros), so the number
//     of loads in flight at each wait is fixed;
//   * masks tile kt where needed and takes its max; if the running max moves,
//     tile kt-1's product (relative to the old max) is added to O first, then
//     O and the sums are rescaled;
//   * runs lag_body: the product of tile kt-1 and the scores of tile kt+1
//     beside tile kt's exponentials;
//   * waits for K_{kt+2} and V_kt, the loads issued in step kt-2, leaving the
//     four later tile loads in flight, and synchronises the workgroup.
// O receives the tiles' products in key order, each after the rescales of the
// tiles before it: the arithmetic and its order are those of taking each tile
// whole (the debug key loop below).
template <class T, int D, int BK, bool CAUSAL, bool KV8, bool F8, class KStg, class VStg>
__device__ __forceinline__ void lag_step(int kt, const char* kcur, const char* vprev, char* kload, char* vload,
                                         f32x16 (&s_cur)[BK / 32], f32x16 (&s_nxt)[BK / 32],
                                         u32x4 (&pcur)[BK / 16], const u32x4 (&pprev)[BK / 16], const KStg& ks,
                                         const VStg& vs, Acc<D>& st, const Offs<D, BK>& o, const Geo& g,
                                         bool wave_live, int w_last, int w_lo, int qrow, int h, float cexp) {
  static_assert(F8, "the lagged step serves the FP8 form");
  const int n = g.nkt;
  const int e[KStg::EPT] = {};  // contiguous tiles: no block table
  __builtin_amdgcn_sched_barrier(0);
  ks.load(kt + 4, g.Lk, kload, e);
  __builtin_amdgcn_sched_barrier(0);
  vs.load(kt + 2, g.Lk, vload, e);
  __builtin_amdgcn_sched_barrier(0);
  // causal: tiles entirely above this wavefront's part of the diagonal are
  // skipped (monotone in kt: work implies prev and work_next implies work)
  const bool work = wave_live && (!CAUSAL || kt * BK <= w_last);
  const bool prev = kt > 0 && wave_live && (!CAUSAL || (kt - 1) * BK <= w_last);
  const bool work_next = kt + 1 < n && wave_live && (!CAUSAL || (kt + 1) * BK <= w_last);
  if (work) {
    softmax_mask<D, BK, CAUSAL>(s_cur, g, kt * BK, qrow, w_lo, h);
    const float mx = tile_max<D, BK>(s_cur, cexp);
    bool pv_due = prev;
    if (__builtin_amdgcn_ballot_w64(max_grows<D, F8>(mx, st))) {
      if (prev) {
        tile_pv<T, D, BK, KV8, F8>(st, pprev, vprev, o);
        pv_due = false;
      }
      rescale<D, F8>(st, mx);
    }
    const float msub = max_to_subtract(st);
    if (pv_due && work_next)
      lag_body<T, D, BK, KV8, F8, true, true>(s_cur, s_nxt, pcur, pprev, kcur, vprev, st, o, msub, cexp);
    else if (pv_due)
      lag_body<T, D, BK, KV8, F8, true, false>(s_cur, s_nxt, pcur, pprev, kcur, vprev, st, o, msub, cexp);
    else if (work_next)
      lag_body<T, D, BK, KV8, F8, false, true>(s_cur, s_nxt, pcur, pprev, kcur, vprev, st, o, msub, cexp);
    else
      lag_body<T, D, BK, KV8, F8, false, false>(s_cur, s_nxt, pcur, pprev, kcur, vprev, st, o, msub, cexp);
  } else if (prev) {
    tile_pv<T, D, BK, KV8, F8>(st, pprev, vprev, o);
  }
  ring_barrier<4, KStg::CPT>();
}

// Debug form of the key loop (built with ATTN_SINGLE_BUFFER): one K and one V
// buffer, and for each tile the loads, a barrier, the tile's whole arithmetic
// (the same functions in the same order as the pipelined steps) and a second
// barrier before the buffers are reused. Nothing overlaps, so a result that
// differs from the pipelined kernel's, bit for bit, points at a staging race.
template <class T, int D, int BK, bool CAUSAL, bool KV8, bool F8, class KStg, class VStg>
__device__ __forceinline__ void single_buffer_loop(char* kbuf, char* vbuf, const KStg& ks, const VStg& vs,
                                                   Acc<D>& st, const Offs<D, BK>& o, const Geo& g, bool wave_live,
                                                   int w_last, int w_lo, int qrow, int h, float cexp) {
  using S = Shape<D, BK>;
  for (int kt = 0; kt < g.nkt; ++kt) {
    int e[KStg::EPT];
    ks.entries(kt, e);
    ks.load(kt, g.Lk, kbuf, e);
    vs.load(kt, g.Lk, vbuf, e);
    staged_barrier();
    if (wave_live && (!CAUSAL || kt * BK <= w_last)) {
      f32x16 s[S::KB];
      u32x4 pf[S::PS] = {};
      tile_qk_plain<T, D, BK, KV8, F8>(s, kbuf, o, st);
      softmax_mask<D, BK, CAUSAL>(s, g, kt * BK, qrow, w_lo, h);
      if constexpr (F8) {
        const float msub = softmax_max<T, D, BK, true>(s, st, cexp);
        softmax_exp<T, D, BK, true>(s, pf, st, msub, cexp);
        tile_pv<T, D, BK, KV8, true>(st, pf, vbuf, o);
      } else {
        const float l0 = st.l, lr0 = st.lr;
        const float ls = softmax_exp<T, D, BK>(s, pf, st, st.m, cexp);
        finish_tile<T, D, BK, KV8>(s, pf, st, o, vbuf, ls, l0, lr0, cexp);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 4 wavefronts x 32 rows, pipelined key steps over R-deep rings of K and V
// buffers (R = 2: double buffering; R = 4: the deep ring of the FP8 prefill).
template <class T, int D, int BQ, int BK, bool CAUSAL, bool PAGED, bool KV8, int R>
__global__ __launch_bounds__(BQ * 2, (2 * R * Shape<D, BK, KV8>::TILE > 80 * 1024 ? 1 : 2)) void prefill_kernel(
    PrefillArgs a) {
  // E4M3 tiles: from the paged cache (16-bit products), or, contiguous, the FP8 form
  constexpr bool F8 = KV8 && !PAGED;
  using S = Shape<D, BK, KV8>;
  constexpr int THREADS = (BQ / 32) * 64;
  static_assert(R == 2 || (R == 4 && F8), "ring depth");
  // K of tile t lives in kb[t % R], V of tile t in vb[t % R]; separate LDS
  // arrays, so the compiler never orders reads of one behind loads into another
  constexpr int XTRA = R > 2 ? S::TILE : 16;
  __shared__ __align__(16) char kb0[S::TILE];
  __shared__ __align__(16) char kb1[S::TILE];
  __shared__ __align__(16) char vb0[S::TILE];
  __shared__ __align__(16) char vb1[S::TILE];
  __shared__ __align__(16) char kb2[XTRA];
  __shared__ __align__(16) char kb3[XTRA];
  __shared__ __align__(16) char vb2[XTRA];
  __shared__ __align__(16) char vb3[XTRA];

  // paged form: the sequence's block-table row, read once into LDS
  __shared__ __align__(16) int tbl[PAGED ? kMaxPagedPrefillBlocks : 4];

  // w (and so w_lo, w_last, wave_live) is the same in every lane of a
  // wavefront; readfirstlane lets the compiler see that, so the 16-bit
  // forms' per-tile work / mask conditions become scalar branches instead of
  // exec masks. (The FP8 form's lagged step keeps the vector form: with
  // scalar branches the compiler's code for its four step variants spills.)
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = F8 ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const Geo g = make_geo<D, BQ, BK, CAUSAL, PAGED>(a);
  const int w_lo = g.q_lo + w * 32;
  const int qrow = w_lo + (lane & 31);
  Acc<D> st;
  load_q<T, D, KV8, F8>(st, g, qrow, h, PAGED ? a.rope : nullptr, a.max_pos,
                        static_cast<const uint8_t*>(a.q) + (size_t)(g.b * a.Hq + g.hq) * a.Tq * D);
  Offs<D, BK> o;
  make_offs<D, BK, KV8, F8>(o, lane);
  using KStg = Stager<D, BK, THREADS, PAGED, KV8, false>;
  using VStg = Stager<D, BK, THREADS, PAGED, KV8, true>;
  KStg ks;
  VStg vs;
  // E4M3 inputs: the scales multiply every score (q_scale k_scale) and every value (v_scale)
  const float cexp = KV8 ? a.c * a.k_scale * (F8 ? a.q_scale : 1.f) : a.c;
  if constexpr (PAGED) {
    // byte offsets: kv head kvh of physical block 0, and one physical block
    const size_t head = (size_t)g.kvh * 16 * S::RB, bstride = (size_t)a.Hkv * 16 * S::RB;
    ks.init(static_cast<const char*>(a.k) + head, tid, bstride, tbl);
    vs.init(static_cast<const char*>(a.v) + head, tid, bstride, tbl);
    const int nb = min((g.Lk + 15) / 16, kMaxPagedPrefillBlocks);
    const int* trow = a.table + (size_t)g.b * a.max_blocks;
    // an id outside [0, num_blocks) is an unmapped block: kept as -1, read as zeros
    for (int i = tid; i < nb; i += THREADS) {
      const int id = trow[i];
      tbl[i] = (unsigned)id < (unsigned)a.num_blocks ? id : -1;
    }
    __syncthreads();
  } else if constexpr (F8) {
    const size_t head = (size_t)(g.b * a.Hkv + g.kvh) * a.Tk * D;  // bytes: 1 per element
    ks.init(static_cast<const char*>(a.k) + head, tid);
    vs.init(static_cast<const char*>(a.v) + head, tid);
  } else {
    ks.init(reinterpret_cast<const char*>(g.Kg), tid);
    vs.init(reinterpret_cast<const char*>(g.Vg), tid);
  }

  const bool wave_live = w_lo < g.Lq;
  const int w_last = min(w_lo + 31, g.Lq - 1) + g.off;  // last key any row of this wavefront sees
#if defined(ATTN_SINGLE_BUFFER)
  (void)kb1;
  (void)vb1;
  (void)kb2;
  (void)kb3;
  (void)vb2;
  (void)vb3;
  q_modes<T, D, F8>(st, g, a.qmode, qrow);
  single_buffer_loop<T, D, BK, CAUSAL, KV8, F8>(kb0, vb0, ks, vs, st, o, g, wave_live, w_last, w_lo, qrow, h, cexp);
#else
  const int n = g.nkt;
  f32x16 s0[S::KB], s1[S::KB];
  if constexpr (!F8) {
    // 16-bit products: the double-buffered loop (K two tiles ahead, V one)
    static_assert(R == 2, "16-bit products: double buffering");
    (void)kb2;
    (void)kb3;
    (void)vb2;
    (void)vb3;
    int ecar[KStg::EPT] = {};  // physical blocks of the tile after the current one
    if (n > 0) {
      int e0[KStg::EPT];
      ks.entries(0, e0);
      ks.load(0, g.Lk, kb0, e0);
      vs.load(0, g.Lk, vb0, e0);
      if (n > 1) {
        ks.entries(1, ecar);
        ks.load(1, g.Lk, kb1, ecar);
      }
    }
    // K_0 has landed when at most the loads issued after it (V_0's, and K_1's
    // when there is a second tile) are in flight: the vector memory counter
    // drains in issue order, so the scores of tile 0 start while V_0 and K_1
    // still travel
    if (n > 1)
      ring_barrier<2, KStg::CPT>();
    else if (n == 1)
      ring_barrier<1, KStg::CPT>();
    else
      ring_barrier<0, KStg::CPT>();
    q_modes<T, D, F8>(st, g, a.qmode, qrow);
    if (n > 0 && wave_live && (!CAUSAL || 0 <= w_last)) tile_qk<T, D, BK, KV8, F8>(s0, kb0, o, st);
    // Step 0 reads V_0 and K_1, which must have landed, and loads K_2 into
    // kb0, which every wavefront has just read as K_0 (each wavefront stages
    // only its own rows of a tile but reads all of them): no wavefront may
    // start those loads before all have finished reading. Later steps reuse a
    // buffer only after the barrier ending the step that read it.
    if (n > 0) staged_barrier();
    for (int kt = 0; kt < n; kt += 2) {
      pipe_step<T, D, BK, CAUSAL, KV8>(kt, kb1, vb0, kb0, vb1, s0, s1, ks, vs, ecar, st, o, g, wave_live, w_last,
                                       w_lo, qrow, h, cexp);
      if (kt + 1 < n)
        pipe_step<T, D, BK, CAUSAL, KV8>(kt + 1, kb0, vb1, kb1, vb0, s1, s0, ks, vs, ecar, st, o, g, wave_live,
                                         w_last, w_lo, qrow, h, cexp);
    }
  } else {
    // FP8 form: the lagged loop over four-deep rings
    static_assert(R == 4, "FP8 form: the deep ring");
    u32x4 p0[S::PS] = {}, p1[S::PS] = {};  // P^T of the even / odd tiles
    // prologue: K0 K1 K2 V0 K3 V1, in this order (the waits count on it): the
    // loads steps -4 .. -1 would have issued
    const int e[KStg::EPT] = {};
    ks.load(0, g.Lk, kb0, e);
    __builtin_amdgcn_sched_barrier(0);
    ks.load(1, g.Lk, kb1, e);
    __builtin_amdgcn_sched_barrier(0);
    ks.load(2, g.Lk, kb2, e);
    __builtin_amdgcn_sched_barrier(0);
    vs.load(0, g.Lk, vb0, e);
    __builtin_amdgcn_sched_barrier(0);
    ks.load(3, g.Lk, kb3, e);
    __builtin_amdgcn_sched_barrier(0);
    vs.load(1, g.Lk, vb1, e);
    __builtin_amdgcn_sched_barrier(0);
    // K0 has landed when at most K1, K2, V0, K3, V1 are in flight
    ring_barrier<5, KStg::CPT>();
    q_modes<T, D, F8>(st, g, a.qmode, qrow);
    if (n > 0 && wave_live && (!CAUSAL || 0 <= w_last)) tile_qk<T, D, BK, KV8, F8>(s0, kb0, o, st);
    // K1 has landed when at most K2, V0, K3, V1 are in flight; the barrier also
    // keeps step 0's load of K4 into kb0 behind every wavefront's reads of K0
    ring_barrier<4, KStg::CPT>();
    for (int kt = 0; kt < n; kt += 4) {
      lag_step<T, D, BK, CAUSAL, KV8, F8>(kt, kb1, vb3, kb0, vb2, s0, s1, p0, p1, ks, vs, st, o, g, wave_live,
                                          w_last, w_lo, qrow, h, cexp);
      if (kt + 1 >= n) break;
      lag_step<T, D, BK, CAUSAL, KV8, F8>(kt + 1, kb2, vb0, kb1, vb3, s1, s0, p1, p0, ks, vs, st, o, g, wave_live,
                                          w_last, w_lo, qrow, h, cexp);
      if (kt + 2 >= n) break;
      lag_step<T, D, BK, CAUSAL, KV8, F8>(kt + 2, kb3, vb1, kb2, vb0, s0, s1, p0, p1, ks, vs, st, o, g, wave_live,
                                          w_last, w_lo, qrow, h, cexp);
      if (kt + 3 >= n) break;
      lag_step<T, D, BK, CAUSAL, KV8, F8>(kt + 3, kb0, vb2, kb3, vb1, s1, s0, p1, p0, ks, vs, st, o, g, wave_live,
                                          w_last, w_lo, qrow, h, cexp);
    }
    // the loads past the last tile are still writing (zeros) into LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the product of the last tile (its V landed before the last step's barrier)
    const int last = n - 1;
    if (n > 0 && wave_live && (!CAUSAL || last * BK <= w_last)) {
      const char* vlast = last % 4 == 0 ? vb0 : last % 4 == 1 ? vb1 : last % 4 == 2 ? vb2 : vb3;
      if (last & 1)
        tile_pv<T, D, BK, KV8, F8>(st, p1, vlast, o);
      else
        tile_pv<T, D, BK, KV8, F8>(st, p0, vlast, o);
    }
  }
#endif
  epilogue<T, D>(st, g, a.Tq, qrow, h, KV8 ? a.v_scale : 1.f, F8 ? kF8PScaleLog2 : 0.f);
}

// ---------------------------------------------------------------------------
template <class T, int D, int BK, bool CAUSAL, bool PAGED, bool KV8 = false>
static hipError_t launch_D(const PrefillArgs& a, hipStream_t stream) {
  PrefillArgs x = a;
  x.nqt = (a.Tq + 127) / 128;
  const long long blocks = (long long)x.nqt * a.Hq * a.B;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  x.xcd_remap = (blocks % (8LL * a.G) == 0) ? 1 : 0;
  // longest-first order of the chunked prefill's groups (a ranking loop over
  // B * nqt groups per lane, so only for batches of at most 64 sequences)
  x.lpt = (PAGED && a.B <= 64 && (long long)x.nqt * a.B <= 256) ? 1 : 0;
  // the FP8 form (contiguous E4M3 tiles) runs the lagged loop over four-deep
  // rings: 64 KiB of LDS at 8-bit tiles, two workgroups per CU as in 16 bits
  constexpr int R = (!PAGED && KV8) ? 4 : 2;
  hipLaunchKernelGGL((prefill_kernel<T, D, 128, BK, CAUSAL, PAGED, KV8, R>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, x);
  return hipGetLastError();
}

template <class T, bool PAGED, bool KV8 = false>
static hipError_t launch_t(const PrefillArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_D<T, 128, 64, true, PAGED, KV8>(a, stream)
                  : launch_D<T, 128, 64, false, PAGED, KV8>(a, stream);
  return causal ? launch_D<T, 64, 64, true, PAGED, KV8>(a, stream) : launch_D<T, 64, 64, false, PAGED, KV8>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream) {
  return bf16 ? launch_t<BF16, false>(a, D, causal, stream) : launch_t<F16, false>(a, D, causal, stream);
}

hipError_t launch_prefill_paged(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream) {
  return bf16 ? launch_t<BF16, true>(a, D, causal, stream) : launch_t<F16, true>(a, D, causal, stream);
}

hipError_t launch_prefill_paged_fp8(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream) {
  return bf16 ? launch_t<BF16, true, true>(a, D, causal, stream) : launch_t<F16, true, true>(a, D, causal, stream);
}

hipError_t launch_prefill_fp8(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream) {
  return bf16 ? launch_t<BF16, false, true>(a, D, causal, stream) : launch_t<F16, false, true>(a, D, causal, stream);
}

}  // namespace attn
