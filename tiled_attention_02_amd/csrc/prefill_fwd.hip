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
// workgroup streams the key/value rows of its kv head in tiles of BK keys:
//   * K tile   -> LDS, row-major (row stride D+8 elements),
//   * V tile   -> LDS, transposed to [D][BK] (row stride BK+8), keys permuted
//                 inside each 16-key group as [0-3, 8-11, 4-7, 12-15] so that
//                 every lane's operand of the P.V product is one 16-byte read.
// Scores are computed transposed, S^T = K Q^T (keys on MFMA rows, the 32
// queries of a wavefront on columns), so that a lane holds 16 keys of one
// query per 32-key block: the row max and row sum are in-lane reductions plus
// one exchange with lane l^32. The transposed scores are, after exp2 and
// rounding, exactly the B operand of O^T += V^T P^T, so P never leaves the
// registers. Q^T lives in registers for the whole key loop.
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
// workgroups are issued heaviest (last query tile) first.
#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kLazyRescale = 8.0f;

template <class T, int D, int BQ, int BK, bool CAUSAL>
__global__ __launch_bounds__(BQ * 2) void prefill_kernel(PrefillArgs a) {
  constexpr int WAVES = BQ / 32;
  constexpr int THREADS = WAVES * 64;
  constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int KB = BK / 32;  // 32-key blocks of S^T
  constexpr int PS = BK / 16;  // k-steps of O^T += V^T P^T
  constexpr int KLD = D + 8;   // K tile row stride (elements)
  constexpr int VLD = BK + 8;  // V^T tile row stride (elements)
  constexpr int C8 = D / 8;    // 16-byte chunks per row
  constexpr int TASKS = (BK / 4) * C8;  // a task = 4 consecutive rows x one chunk
  constexpr int TPT = (TASKS + THREADS - 1) / THREADS;
  static_assert(BQ % 32 == 0 && BK % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __align__(16) uint16_t Ks[BK * KLD];
  __shared__ __align__(16) uint16_t Vt[D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;   // half of the wavefront
  const int c32 = lane & 31;

  // ---- which tile: heaviest-first for causal; consecutive ids share a kv head
  const int per = a.Hq * a.B;
  const int id = blockIdx.x;
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

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[TPT][4], vreg[TPT][4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int task = tid + i * THREADS;
      if (TASKS % THREADS == 0 || task < TASKS) {
        const int c = task % C8;
        const int r0 = (task / C8) * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + r0 + r;
          if (key < Lk) {
            kreg[i][r] = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + c * 8);
            vreg[i][r] = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + c * 8);
          } else {
            kreg[i][r] = u32x4{0, 0, 0, 0};
            vreg[i][r] = u32x4{0, 0, 0, 0};
          }
        }
      }
    }
  };
  auto lds_store = [&]() {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int task = tid + i * THREADS;
      if (TASKS % THREADS == 0 || task < TASKS) {
        const int c = task % C8;
        const int r0 = (task / C8) * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<u32x4*>(&Ks[(r0 + r) * KLD + c * 8]) = kreg[i][r];
        // 4 rows x 8 columns -> 8 columns x 4 keys (transpose through v_perm)
        const int g4 = (r0 & 15) >> 2;
        const int pos = (r0 & ~15) + (((g4 & 1) << 3) | ((g4 >> 1) << 2));
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // dword e holds columns 2e, 2e+1
          const uint32_t x0 = vreg[i][0][e], x1 = vreg[i][1][e], x2 = vreg[i][2][e], x3 = vreg[i][3][e];
          u32x2 lo = {pack_lo16(x0, x1), pack_lo16(x2, x3)};  // column 2e, keys r0..r0+3
          u32x2 hi = {pack_hi16(x0, x1), pack_hi16(x2, x3)};  // column 2e+1
          *reinterpret_cast<u32x2*>(&Vt[(c * 8 + 2 * e) * VLD + pos]) = lo;
          *reinterpret_cast<u32x2*>(&Vt[(c * 8 + 2 * e + 1) * VLD + pos]) = hi;
        }
      }
    }
  };

  if (nkt > 0) {
    gload(0);
    lds_store();
  }
  __syncthreads();

  const float cexp = a.c;  // scale * log2(e) > 0
  const bool wave_live = w_lo < Lq;

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    if (kt + 1 < nkt) gload(kt + 1);

    // skip tiles entirely above this wavefront's part of the diagonal
    const bool wave_work = wave_live && (!CAUSAL || k0 <= min(w_lo + 31, Lq - 1) + off);
    if (wave_work) {
      // ---- S^T = K Q^T
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x16{};
        const uint16_t* krow = &Ks[(kb * 32 + c32) * KLD + 8 * h];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 af = *reinterpret_cast<const u32x4*>(krow + 16 * s);
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
      // ---- p = 2^(s*c - m), row sum, pack to the P^T operand
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
          // the row sum adds the rounded probabilities the P.V product uses
#pragma unroll
          for (int e = 0; e < 4; ++e) lrsum = T::sum2(pk[e], lrsum);
          pf[kb * 2 + hf] = pk;
        }
      l_run += lsum;
      lr_run += lrsum;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = &Vt[(db * 32 + c32) * VLD + 8 * h];
#pragma unroll
        for (int s = 0; s < PS; ++s) {
          const u32x4 af = *reinterpret_cast<const u32x4*>(vrow + 16 * s);
          oacc[db] = T::mfma32(af, pf[s], oacc[db]);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      lds_store();
      __syncthreads();
    }
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
