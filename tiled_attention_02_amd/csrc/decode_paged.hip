// One-token decode attention through a paged KV cache, gfx950.
//
// Method: the-ai.news, "Snelle attention-kernels en operatorfusie versnellen
// AI-modellen", section "FlashAttention-type aandacht en gepagineerde
// aandacht": the KV cache is split into fixed-size blocks (16 tokens in the
// vLLM example) and a block table maps logical positions to physical blocks;
// the attention kernel translates every position through that table. The KV
// cache holds the keys/values of earlier tokens so the new token attends to
// the cache instead of recomputing it ("讨论CUDA图形优化与推理加速", section
// on the KV cache). Long key ranges are split across workgroups and reduced
// in a second pass, the split-K decomposition of "天下苦英偉達久矣！PyTorch免CUDA
// 加速推理，Triton時代要來？", section "Triton SplitK GEMM 內核", applied to the
// key axis; the merge is the softmax-statistics update of blockwise attention.
//
// Decomposition: one workgroup (4 wavefronts) per (split of 256 tokens, kv
// head, sequence). Wavefront w takes cache blocks 4w .. 4w+3 of the split, two
// blocks (32 tokens) per step, and serves all G = Hq/Hkv query heads of the kv
// head from one read of each key/value block:
//   S^T = K Q^T       v_mfma_f32_16x16x32: rows = 16 tokens of a block,
//                     columns = query heads (G <= 16, the rest zero).
//   O  += P V         v_mfma_f32_16x16x32: rows = heads, columns = 16 of D,
//                     contraction = the 32 tokens of the two blocks.
// The transposed scores of the two blocks are already the A operand (P) of
// the second product. The V operand needs 8 tokens at one column per lane:
// lane (g = l/16, c = l%16) loads 16-byte rows of its 8 tokens at columns
// [8c, 8c+8) and transposes them in registers (v_perm), so output column
// n of product n is d = 8c + n (for D = 128).
// Every (block, kv head) of K and V is 16*D contiguous elements, read once.
// The 4 wavefronts merge through LDS and write one partial (O normalised, log2
// of its sum) per (sequence, query head, split); a second, light kernel merges
// the partials. A sequence with a single split writes its output directly.
#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kDecodeLazy = 8.0f;

template <class T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;   // k-steps of S^T (32 columns of D each)
  constexpr int VC = D / 16;   // columns of V per lane (= number of P.V products)
  constexpr int NPAIR = 2;     // block pairs per wavefront
  static_assert(D == 128 || D == 64, "head size");

  __shared__ float s_o[4][16][D];
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  __shared__ float s_lr[4][16];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar table loads
  const int g = lane >> 4;
  const int c = lane & 15;
  const int G = a.G;
  const int blk0 = split * kSplitBlocks + 4 * w;
  const int* trow = a.table + (size_t)b * a.max_blocks;

  // The block-table entries of this wavefront's 4 blocks are read together with
  // the context length (scalar loads, one round trip); entries at or beyond the
  // sequence's end are read only if they exist in the table and never used.
  int phys[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) phys[i] = trow[min(blk0 + i, a.max_blocks - 1)];
  // materialise the four entries here (one wait for all) rather than letting
  // the compiler sink each load into the branch that uses it
  asm volatile("" ::"s"(phys[0]), "s"(phys[1]), "s"(phys[2]), "s"(phys[3]));
  const int ctx = a.ctx[b];
  const int nblk = (ctx + kDecodeBlock - 1) / kDecodeBlock;
  const int nsp = (nblk + kSplitBlocks - 1) / kSplitBlocks;
  if (split >= nsp) return;  // uniform across the workgroup

  // ---- q^T operand: head c, columns 32s + 8g .. +8 (step s, lane group g)
  u32x4 qf[KS];
  {
    const bool live = c < G && a.qmode != 2;
    const uint32_t flip = a.qmode == 1 ? 0x80008000u : 0u;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + kvh * G + (live ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + 32 * s + 8 * g);
      x ^= flip;
      qf[s] = live ? x : u32x4{0, 0, 0, 0};
    }
  }

  const size_t head_stride = (size_t)kDecodeBlock * D;  // one (block, kv head)
  const size_t block_stride = (size_t)a.Hkv * head_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.kc) + kvh * head_stride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.vc) + kvh * head_stride;

  // ---- issue every load of this wavefront's blocks at once (blocks inside the
  // sequence only: a wave-uniform test). A K load instruction reads 64
  // contiguous bytes of each of 16 token rows, so each 128-byte line is
  // requested by two consecutive instructions: these loads keep the normal
  // cache policy so the second one hits. A V load instruction reads 4 whole
  // rows, so V is streamed with non-temporal loads. Slots at or beyond ctx in the last
  // block may hold anything (NaN included): they are loaded (the block exists)
  // and their V rows replaced by zeros, so p = 0 cannot meet 0 * NaN.
  u32x4 kreg[NPAIR][2][KS];
  typedef uint32_t vchunk __attribute__((ext_vector_type(VC / 2)));
  vchunk vreg[NPAIR][8];
#pragma unroll
  for (int p = 0; p < NPAIR; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = blk0 + 2 * p + j;
      if (blk < nblk) {
        const uint16_t* kb = kbase + (size_t)phys[2 * p + j] * block_stride;
        const uint16_t* vb = vbase + (size_t)phys[2 * p + j] * block_stride;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kreg[p][j][s] = *reinterpret_cast<const u32x4*>(kb + c * D + 32 * s + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vreg[p][4 * j + e] = __builtin_nontemporal_load(reinterpret_cast<const vchunk*>(vb + (4 * g + e) * D + VC * c));
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) kreg[p][j][s] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) vreg[p][4 * j + e] = vchunk{};
      }
    }
  if ((blk0 + 4) * kDecodeBlock > ctx) {  // this wavefront holds the sequence's tail
#pragma unroll
    for (int p = 0; p < NPAIR; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (blk0 + 2 * p + (e >> 2)) * kDecodeBlock + 4 * g + (e & 3);
        vreg[p][e] = t < ctx ? vreg[p][e] : vchunk{};
      }
  }

  f32x4 oacc[VC];
#pragma unroll
  for (int n = 0; n < VC; ++n) oacc[n] = f32x4{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;   // fp32 sum of p (lse)
  float lr_run = 0.f;  // sum of the rounded p (normalises O)
  const float cexp = a.c;

#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    const int t0 = (blk0 + 2 * p) * kDecodeBlock;  // first token of the pair
    if (t0 >= ctx) break;                         // uniform across the wavefront
    f32x4 sacc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sacc[j] = f32x4{};
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[j] = T::mfma16(kreg[p][j][s], qf[s], sacc[j]);
    }
    if (t0 + 32 > ctx) {  // tail: hide tokens at or beyond ctx
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sacc[j][r] = (t0 + 16 * j + 4 * g + r) >= ctx ? -__builtin_inff() : sacc[j][r];
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = half_swap_max(mx) * cexp;
    const bool grow = mx > m_run + kDecodeLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
      lr_run *= alpha;
      // output rows are heads 4g + r: fetch their factors from lane 4g + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
        for (int n = 0; n < VC; ++n) oacc[n][r] *= ar;
      }
    }
    const float msub = m_run == -__builtin_inff() ? 0.f : m_run;
    float pv[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[4 * j + r] = fast_exp2(__builtin_fmaf(sacc[j][r], cexp, -msub));
        l_run += pv[4 * j + r];
      }
    const u32x4 pf = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                      T::pack2(pv[6], pv[7])};
    // the running sum adds the rounded probabilities that the P.V product applies
#pragma unroll
    for (int e = 0; e < 4; ++e) lr_run = T::sum2(pf[e], lr_run);
    // V operand of product n: element e = V[token e][VC*c + n]
#pragma unroll
    for (int n = 0; n < VC; ++n) {
      const int dw = n >> 1;
      u32x4 vf;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x0 = vreg[p][2 * k][dw], x1 = vreg[p][2 * k + 1][dw];
        vf[k] = (n & 1) ? pack_hi16(x0, x1) : pack_lo16(x0, x1);
      }
      oacc[n] = T::mfma16(pf, vf, oacc[n]);
    }
  }

  // ---- wavefront totals per head, then merge the 4 wavefronts through LDS
  float l_head = l_run + __shfl_xor(l_run, 16);
  l_head = half_swap_sum(l_head);
  float lr_head = lr_run + __shfl_xor(lr_run, 16);
  lr_head = half_swap_sum(lr_head);
  if (g == 0) {
    s_m[w][c] = m_run;
    s_l[w][c] = l_head;
    s_lr[w][c] = lr_head;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int n = 0; n < VC; ++n) s_o[w][4 * g + r][VC * c + n] = oacc[n][r];
  __syncthreads();

  const bool single = nsp == 1;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -__builtin_inff();
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hh]);
    float L = 0.f, LR = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float wt = s_m[ww][hh] == -__builtin_inff() ? 0.f : fast_exp2(s_m[ww][hh] - M);
      L += s_l[ww][hh] * wt;
      LR += s_lr[ww][hh] * wt;
      acc += s_o[ww][hh][d] * wt;
    }
    const float val = acc / LR;  // LR > 0: the split holds at least one visible token
    const int hq = kvh * G + hh;
    if (single) {
      const size_t oi = ((size_t)b * a.Hq + hq) * D + d;
      uint16_t* op = static_cast<uint16_t*>(a.o);
      op[oi] = (uint16_t)(T::pack2(val, 0.f) & 0xffffu);
      if (d == 0 && a.lse) a.lse[(size_t)b * a.Hq + hq] = (M + fast_log2(L)) * kLn2;
    } else {
      float* wp = a.ws + (((size_t)b * a.Hq + hq) * a.nsplit + split) * (D + 2);
      wp[d] = val;
      if (d == 0) wp[D] = M + fast_log2(L);
    }
  }
}

// Second pass (the reduction of the split-K decomposition): merge the partials
// of a sequence's splits. One workgroup of D threads per (query head,
// sequence); thread d produces output column d. The partials are combined
// with a running maximum, 8 splits per step so that 16 loads are in flight.
template <class T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int ctx = a.ctx[b];
  const int nblk = (ctx + kDecodeBlock - 1) / kDecodeBlock;
  const int nsp = (nblk + kSplitBlocks - 1) / kSplitBlocks;
  if (nsp == 1) return;  // the first pass wrote this head's output
  const int d = threadIdx.x;
  const float* wp = a.ws + ((size_t)b * a.Hq + hq) * a.nsplit * (D + 2);
  float m = -__builtin_inff(), W = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += 8) {
    float ls[8], part[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = min(s0 + u, nsp - 1);  // valid address; weight 0 below
      ls[u] = wp[(size_t)sp * (D + 2) + D];
      part[u] = wp[(size_t)sp * (D + 2) + d];
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < 8; ++u) mc = s0 + u < nsp ? fmaxf(mc, ls[u]) : mc;
    const float r = fast_exp2(m - mc);  // 0 on the first step (m = -inf, W = acc = 0)
    W *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wt = s0 + u < nsp ? fast_exp2(ls[u] - mc) : 0.f;
      W += wt;
      acc += wt * part[u];
    }
    m = mc;
  }
  uint16_t* op = static_cast<uint16_t*>(a.o);
  op[((size_t)b * a.Hq + hq) * D + d] = (uint16_t)(T::pack2(acc / W, 0.f) & 0xffffu);
  if (d == 0 && a.lse) a.lse[(size_t)b * a.Hq + hq] = (m + fast_log2(W)) * kLn2;
}

template <class T, int D>
static hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(a.nsplit, a.Hkv, a.B), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.Hq, a.B), dim3(D), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (a.D == 128) return bf16 ? launch_d<BF16, 128>(a, stream) : launch_d<F16, 128>(a, stream);
  return bf16 ? launch_d<BF16, 64>(a, stream) : launch_d<F16, 64>(a, stream);
}

}  // namespace attn
