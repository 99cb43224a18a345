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
// Work decomposition. One workgroup of BQ/32 wavefronts owns BQ consecutive
// query rows of one (batch, query head); each wavefront owns 32 rows. The
// workgroup streams the key/value rows of its kv head in tiles of BK keys,
// double-buffered in LDS: while tile j is consumed, tile j+1 travels from HBM
// into registers and is written to the other buffer, one barrier per tile.
// K and V tiles are stored row-major with a 16-byte-chunk XOR swizzle that
// keeps every LDS access pattern below free of bank conflicts.
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
// unrounded probabilities. The max only moves when a tile's max
// exceeds it by more than kLazyRescale (in log2 units); otherwise p = 2^(x-m)
// is at most 2^kLazyRescale, which fp32 and the 16-bit P hold without loss of
// relative precision. O = O^T / l and lse = (m + log2 l) ln 2 are exact
// rearrangements of the same sums.
//
// Masking is a selection of -inf on the raw score (never an addition), and
// only on tiles that need it (the causal diagonal, the ragged / Tk tail).
// Value rows beyond the sequence are zero-filled in LDS so 0 * NaN cannot
// reach O. Causal tiles entirely above the diagonal are skipped; causal
// workgroups are issued heaviest (last query tile) first, and the G query
// heads that share a kv head are placed on one XCD (one L2) next to each other.
#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kLazyRescale = 8.0f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte chunk slot of (row, chunk c) inside an LDS row: c ^ f(row). The
// functions are chosen so that the K operand reads (16 rows, one chunk), the
// transposing V reads (4 rows x 2 chunks per 16 lanes) and the row-major tile
// writes all hit distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}

template <class T, int D, int BQ, int BK, bool CAUSAL>
__global__ __launch_bounds__(BQ * 2, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int WAVES = BQ / 32;
  constexpr int THREADS = WAVES * 64;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int KB = BK / 32;  // 32-key blocks of S^T
  constexpr int PS = BK / 16;  // k-steps of O^T += V^T P^T
  constexpr int RB = D * 2;    // bytes per tile row
  constexpr int C8 = D / 8;    // 16-byte chunks per row
  constexpr int CHUNKS = BK * C8;
  constexpr int CPT = CHUNKS / THREADS;  // chunks per thread per tile (K and V each)
  constexpr int TILE = BK * RB;          // bytes of one K or V tile
  static_assert(BQ % 32 == 0 && BK % 32 == 0 && D % 32 == 0 && CHUNKS % THREADS == 0, "tile shape");

  // [buffer][K | V][tile]
  __shared__ __align__(16) char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;   // half of the wavefront
  const int c32 = lane & 31;
  const int g16 = lane >> 4;  // 16-lane group
  const int i16 = lane & 15;

  // ---- which tile: heaviest-first for causal; G consecutive ids share a kv head
  int id = blockIdx.x;
  if (a.xcd_remap) {  // members of a kv-head group land on one XCD (dispatch is round-robin over 8)
    const int x = id & 7, slot = id >> 3;
    id = ((slot / a.G) * 8 + x) * a.G + slot % a.G;
  }
  const int per = a.Hq * a.B;
  const int qt = CAUSAL ? (a.nqt - 1 - id / per) : (id / per);
  const int rem = id % per;
  const int hq = rem % a.Hq;
  const int b = rem / a.Hq;
  const int kvh = hq / a.G;

  int Lq = a.Tq, Lk = a.Tk;
  if (a.seq_lens) {
    Lq = a.seq_lens[b];
    Lk = Lq;
  }
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q_lo = qt * BQ;

  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + (size_t)(b * a.Hq + hq) * a.Tq * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (size_t)(b * a.Hkv + kvh) * a.Tk * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (size_t)(b * a.Hkv + kvh) * a.Tk * D;
  uint16_t* Og = static_cast<uint16_t*>(a.o) + (size_t)(b * a.Hq + hq) * a.Tq * D;
  float* Lg = a.lse ? a.lse + (size_t)(b * a.Hq + hq) * a.Tq : nullptr;

  // exclusive key bound of the whole tile
  int kend = Lk;
  if (CAUSAL) kend = min(Lk, min(q_lo + BQ, Lq) + off);
  const int nkt = (q_lo < Lq && kend > 0) ? (kend + BK - 1) / BK : 0;

  const int qrow = q_lo + w * 32 + c32;  // this lane's query row
  const int w_lo = q_lo + w * 32;        // first row of this wavefront

  // ---- Q^T fragments (B operand): lane holds Q[qrow][16s + 8h .. +8)
  u32x4 qf[KS];
  {
    const bool live = qrow < Lq;
    const uint32_t flip = a.qmode == 1 ? 0x80008000u : 0u;
    const bool zero = a.qmode == 2 || !live;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qg + (size_t)(live ? qrow : 0) * D + 8 * h);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = src[2 * s];
      x ^= flip;
      qf[s] = zero ? u32x4{0, 0, 0, 0} : x;
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;   // sum of p in fp32 (for lse)
  float lr_run = 0.f;  // sum of p rounded to the 16-bit type (normalises O)

  // ---- tile staging: global -> registers -> LDS (row-major, swizzled)
  u32x4 kreg[CPT], vreg[CPT];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * THREADS;
      const int key = k0 + ch / C8;
      const int c = ch % C8;
      if (key < Lk) {
        kreg[i] = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + c * 8);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + c * 8);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lds_store = [&](int buf) {
    char* kt_ = smem + buf * 2 * TILE;
    char* vt_ = kt_ + TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * THREADS;
      const int r = ch / C8;
      const int c = ch % C8;
      const int o = r * RB + 16 * (c ^ swz<D>(r));
      *reinterpret_cast<u32x4*>(kt_ + o) = kreg[i];
      *reinterpret_cast<u32x4*>(vt_ + o) = vreg[i];
    }
  };

  if (nkt > 0) {
    gload(0);
    lds_store(0);
  }
  __syncthreads();

  const float cexp = a.c;  // scale * log2(e) > 0
  const bool wave_live = w_lo < Lq;

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const char* Ks = smem + buf * 2 * TILE;
    const char* Vs = Ks + TILE;

    // skip tiles entirely above this wavefront's part of the diagonal
    const bool wave_work = wave_live && (!CAUSAL || k0 <= min(w_lo + 31, Lq - 1) + off);
    if (wave_work) {
      // ---- S^T = K Q^T
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x16{};
        const int row = kb * 32 + c32;
        const char* krow = Ks + row * RB;
        const int sw = swz<D>(row);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 af = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * s + h) ^ sw));
          sacc[kb] = T::mfma32(af, qf[s], sacc[kb]);
        }
      }
      // ---- mask (selection) where the tile crosses the diagonal or the tail
      const bool need_mask = (k0 + BK > Lk) || (CAUSAL && k0 + BK - 1 > w_lo + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(Lk - 1, qrow + off) : (Lk - 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            sacc[kb][r] = key > lim ? -__builtin_inff() : sacc[kb][r];
          }
      }
      // ---- tile max (raw scores; cexp > 0)
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = half_swap_max(mx) * cexp;  // -inf stays -inf (cexp > 0)
      // ---- lazy rescale: move m only when the max grows by more than the margin
      const bool grow = mx > m_run + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;  // m_run=-inf -> 0
        m_run = m_new;
        l_run *= alpha;
        lr_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      }
      const float msub = m_run == -__builtin_inff() ? 0.f : m_run;
      // ---- p = 2^(s*c - m), row sums, pack to the P^T operand
      u32x4 pf[PS];
      float lsum = 0.f, lrsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(__builtin_fmaf(sacc[kb][8 * hf + e], cexp, -msub));
            lsum += p[e];
          }
          const u32x4 pk = {T::pack2(p[0], p[1]), T::pack2(p[2], p[3]), T::pack2(p[4], p[5]),
                            T::pack2(p[6], p[7])};
          // the normaliser adds the rounded probabilities the P.V product uses
#pragma unroll
          for (int e = 0; e < 4; ++e) lrsum = T::sum2(pk[e], lrsum);
          pf[kb * 2 + hf] = pk;
        }
      l_run += lsum;
      lr_run += lrsum;
      // ---- O^T += V^T P^T; the V^T operand comes from transposing LDS reads.
      // k-step s covers keys 16s + 8r + 4h + (0..3) for element group r = 0, 1;
      // lane i of 16-lane group g addresses row (those keys' base) + i/4 at
      // columns 32db + 16(g%2) + 4(i%4) and receives column 32db + 16(g%2) + i.
      const int vrow_l = 4 * h + (i16 >> 2);
      const int vcol_l = 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + vcol_l;
#pragma unroll
        for (int s = 0; s < PS; ++s) {
          i16x4 part[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int row = 16 * s + 8 * r + vrow_l;
            const int o = row * RB + 16 * ((col >> 3) ^ swz<D>(row)) + 2 * (col & 7);
            part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + o));
          }
          const u32x2 p0 = __builtin_bit_cast(u32x2, part[0]);
          const u32x2 p1 = __builtin_bit_cast(u32x2, part[1]);
          const u32x4 af = {p0[0], p0[1], p1[0], p1[1]};
          oacc[db] = T::mfma32(af, pf[s], oacc[db]);
        }
      }
    }
    if (kt + 1 < nkt) lds_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) ln 2; padding rows -> 0, -inf
  const float l_tot = half_swap_sum(l_run);
  const float lr_tot = half_swap_sum(lr_run);
  if (qrow >= a.Tq) return;
  const bool has = qrow < Lq && l_tot > 0.f;
  const float inv = has ? 1.f / lr_tot : 0.f;
  uint16_t* orow = Og + (size_t)qrow * D + 4 * h;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk = {T::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                  T::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g) = pk;
    }
  if (Lg && h == 0) Lg[qrow] = has ? (m_run + fast_log2(l_tot)) * kLn2 : -__builtin_inff();
}

template <class T, int D, int BQ, int BK, bool CAUSAL>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  PrefillArgs x = a;
  x.nqt = (a.Tq + BQ - 1) / BQ;
  const long long blocks = (long long)x.nqt * a.Hq * a.B;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  x.xcd_remap = (blocks % (8LL * a.G) == 0) ? 1 : 0;
  hipLaunchKernelGGL((prefill_kernel<T, D, BQ, BK, CAUSAL>), dim3((unsigned)blocks), dim3(BQ * 2), 0, stream,
                     x);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_t(const PrefillArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128) {
    return causal ? launch_one<T, 128, 128, 64, true>(a, stream) : launch_one<T, 128, 128, 64, false>(a, stream);
  }
  return causal ? launch_one<T, 64, 128, 128, true>(a, stream) : launch_one<T, 64, 128, 128, false>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream) {
  return bf16 ? launch_t<BF16>(a, D, causal, stream) : launch_t<F16>(a, D, causal, stream);
}

}  // namespace attn
