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
// Decomposition: one wavefront per (split of 256 tokens = 16 cache blocks,
// kv head, sequence). It streams its blocks through 16 KiB of LDS (16-bit
// cache: one block per step, in two 8 KiB step buffers; E4M3 cache: four
// blocks per step in one buffer) and serves all G = Hq/Hkv query heads of
// the kv head from one read of each block:
//   S^T = K Q^T       v_mfma_f32_16x16x32: rows = 16 tokens of a block,
//                     columns = query heads (G <= 16, the rest zero).
//   O  += P V         rows = heads, columns = 16 of D; 16-bit cache:
//                     v_mfma_f32_16x16x16 over one block's 16 tokens; E4M3
//                     cache: v_mfma_f32_16x16x32 over a block pair's 32.
// Every (block, kv head) of K and V is 16*D contiguous elements, read once,
// straight into LDS; the transposed scores of two blocks are already the
// A operand (P) of the second product, and V's operand comes from LDS through
// the transposing reads. The split's partial (O normalised, log2 of its sum)
// is written from registers; a second, light kernel merges the partials.
// When the whole batch fits in one split the first kernel writes the output.
//
// FP8 form: the caches hold E4M3 codes with one scale per cache (an entry
// means code value * scale). Blocks are half the bytes; the operands are
// converted to the 16-bit type right after their LDS reads (exact: E4M3 values
// are bf16 and fp16 values), and the two scales are folded out of the
// products: k_scale into the exponent factor of the scores, v_scale into the
// final normalisation. This is the fusion of dequantisation into the
// consuming product named on the-ai.news page's operator-fusion section.
#include <mutex>

#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kDecodeLazy = 8.0f;
constexpr int kDecodeDword3 = 0x00020000;  // raw (untyped) buffer descriptor, 32-bit data

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// LDS image of one half-step's cache blocks: K blocks 0 .. NB-1, then V blocks
// 0 .. NB-1, each 16 token rows of RB bytes, row-major with a 16-byte-chunk
// XOR swizzle: chunk c of row r sits in slot c ^ f(r). LDS serves 256 bytes
// per cycle (16 lanes of a 16-byte access, 32 lanes of an 8-byte one); f makes
// the K operand reads and the transposing V reads of each lane group hit
// distinct banks. A wavefront owns NBUF such buffers, 16 KiB together at
// D = 128, so ten wavefronts fit a CU either way.
template <int D, bool KV8>
struct StepLds {
  // 16-bit cache: steps of 1 block (16 tokens, 8 KiB of K and V) in two step
  // buffers (one in flight during the other's compute; measured 2.7 % faster
  // than one buffer of 2 blocks). E4M3 cache: steps of 4 blocks (64 tokens,
  // 16 KiB) in one buffer, loaded after the step's reads (measured 2.7 %
  // faster than two buffers of 2 blocks).
  static constexpr int NB = KV8 ? 4 : 1;
  static constexpr int NBUF = KV8 ? 1 : 2;
  static constexpr int EB = KV8 ? 1 : 2;     // bytes per cache element
  static constexpr int RB = EB * D;          // bytes per token row
  static constexpr int BLK = 16 * RB;        // one (block, kv head) of K or V
  static constexpr int BYTES = 2 * NB * BLK; // one step buffer
  static constexpr int RPI = 1024 / RB;      // rows filled by one wavefront load instruction
  static constexpr int NI = 16 / RPI;        // load instructions per block
  static constexpr int LOADS = 2 * NB * NI;  // load instructions per step
  static constexpr int C8 = RB / 16;         // 16-byte chunks per row
};

// 16-bit cache: one swizzle for K and V. K reads: 16 rows at one chunk per
// 16 lanes; V reads (ds_read_b64_tr_b16): 4 rows x 2 chunk halves per 16
// lanes, 8 rows per 32 lanes.
template <int D>
__device__ __forceinline__ int dswz(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
}
// E4M3 cache: rows of D bytes. K reads are 8 bytes per lane (rows 0..15 at
// two adjacent 8-byte chunks per 32 lanes): rows of equal parity (D = 128; of
// equal row % 4 at D = 64) must take distinct chunk swaps. V reads
// (ds_read_b64_tr_b8) take rows 0..7 of both V blocks at two adjacent 8-byte
// chunks per 32 lanes, so the V swizzle also depends on the block's parity.
template <int D>
__device__ __forceinline__ int kswz8(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int vswz8(int row, int blk) {
  if constexpr (D == 128) return ((row >> 1) & 3) | (blk << 2);
  else return ((row >> 2) & 1) | (blk << 1);
}
template <int D, bool KV8>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (KV8) return kswz8<D>(row);
  else return dswz<D>(row);
}
template <int D, bool KV8>
__device__ __forceinline__ int vswz(int row, int blk) {
  if constexpr (KV8) return vswz8<D>(row, blk);
  else return dswz<D>(row);
}

// Per-lane byte offsets, identical for every step.
template <int D, bool KV8>
struct DecOffs {
  int ldk[StepLds<D, KV8>::NI];     // chunk fetched by load instruction i of a K block
  int ldv[2][StepLds<D, KV8>::NI];  // ... of an even / odd V block
  int k[D / 32];                    // K operand of k-step s
  int v[D / 16];                    // V operand of product n (16-bit: first of two reads; E4M3: the read)
};

template <int D, bool KV8>
__device__ __forceinline__ void make_dec_offs(DecOffs<D, KV8>& o, int lane) {
  using L = StepLds<D, KV8>;
  const int g = lane >> 4, c = lane & 15;
  // load instruction i writes rows RPI*i .. (1 KiB of consecutive LDS, lane l
  // at 16 l): lane l fetches the logical chunk its slot holds
#pragma unroll
  for (int i = 0; i < L::NI; ++i) {
    const int row = L::RPI * i + lane / L::C8;
    const int slot = lane % L::C8;
    o.ldk[i] = row * L::RB + 16 * (slot ^ kswz<D, KV8>(row));
    o.ldv[0][i] = row * L::RB + 16 * (slot ^ vswz<D, KV8>(row, 0));
    o.ldv[1][i] = row * L::RB + 16 * (slot ^ vswz<D, KV8>(row, 1));
  }
  if constexpr (!KV8) {
    // K operand (A of S^T = K Q^T): lane (g, c) takes token c, columns
    // 32s + 8g .. +8, i.e. chunk 4s + g
#pragma unroll
    for (int s = 0; s < D / 32; ++s) o.k[s] = c * L::RB + 16 * ((4 * s + g) ^ dswz<D>(c));
    // V^T operand of product n (B of O += P V, columns 16n .. 16n + 15): in
    // each 16-lane group g, lane i = a + 4e addresses token row 4g + e at
    // columns 16n + 4a .. +4 and receives column 16n + i of those 4 rows
    const int i = lane & 15, a4 = i & 3, row = 4 * g + (i >> 2);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) o.v[n] = row * L::RB + 16 * ((2 * n + (a4 >> 1)) ^ dswz<D>(row)) + 8 * (a4 & 1);
  } else {
    // K operand: lane (g, c) takes token c, columns 32s + 8g .. +8: the 8-byte
    // half (g & 1) of 16-byte chunk 2s + (g >> 1)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) o.k[s] = c * L::RB + 16 * ((2 * s + (g >> 1)) ^ kswz8<D>(c)) + 8 * (g & 1);
    // V operand of product n via ds_read_b64_tr_b8: within each 16-lane group,
    // lane j receives byte (j & 7) of the 8 bytes read by lanes 2e + (j >> 3),
    // e = 0..7. So lane s addresses token e = s >> 1 of the group's 8 (block
    // e >> 2 of a block pair, row 4g + e % 4: P's contraction order) at
    // columns 16n + 8(s & 1) .. +8, and lane j receives column 16n + j of the
    // 8 tokens. Offsets of the step's first block pair; the next pair is 2 BLK on.
    const int e = c >> 1, bb = e >> 2, row = 4 * g + (e & 3);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
      o.v[n] = (L::NB + bb) * L::BLK + row * L::RB + 16 * (n ^ vswz8<D>(row, bb)) + 8 * (c & 1);
  }
}

// Starts the loads of one step's blocks (K and V of each) into an LDS step
// buffer: buffer loads that write LDS directly, each instruction 1 KiB of
// consecutive bytes of one block (whole rows). ph[j] is block j's physical
// block; a block past the sequence's last one carries the step's first block
// instead (a cache hit: every token there is masked or zeroed anyway). An id
// outside [0, num_blocks) is an unmapped block: its descriptor covers no bytes,
// so the hardware writes zeros to LDS and nothing outside the caches is read.
template <int D, bool KV8>
__device__ __forceinline__ void load_step(char* buf, const char* kbase, const char* vbase, size_t block_stride,
                                          const int (&ph)[StepLds<D, KV8>::NB], int num_blocks,
                                          const DecOffs<D, KV8>& o) {
  using L = StepLds<D, KV8>;
#pragma unroll
  for (int j = 0; j < L::NB; ++j) {
    const bool mapped = (unsigned)ph[j] < (unsigned)num_blocks;
    const size_t off = (size_t)(mapped ? ph[j] : 0) * block_stride;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint64_t p = reinterpret_cast<uint64_t>((kv ? vbase : kbase) + off);
      // uniform by construction; readfirstlane keeps the descriptor scalar
      const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(pu), (short)0, mapped ? L::BLK : 0, kDecodeDword3);
      char* dst = buf + (L::NB * kv + j) * L::BLK;
      // the host compilation pass of this file does not know this builtin (it
      // would drop the kernels' host stubs); the function only runs on the device
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int i = 0; i < L::NI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + i * 1024), 16,
                                                 kv ? o.ldv[j & 1][i] : o.ldk[i], 0, 0, /*non-temporal*/ 2);
#else
      (void)rsrc;
      (void)dst;
#endif
    }
  }
}

// Online-softmax state of one wavefront: per lane, head c's running max (log2
// units), the fp32 sum of p and the sum of the rounded p over the lane's
// tokens; the accumulator rows are heads 4g + r, product n covers columns
// 16n .. 16n + 15 (lane c: column 16n + c).
template <int D>
struct WaveState {
  f32x4 o[D / 16];
  float m, l, lr;
};

// One step: the 16 * NB tokens starting at t0, from an LDS step buffer. In
// the sequence's last step (TAIL) tokens >= ctx are masked, and their V rows
// are zeroed in LDS first, since unused cache slots may hold anything, NaN
// included.
template <class T, int D, bool KV8, bool TAIL>
__device__ __forceinline__ void step_compute(WaveState<D>& st, char* buf, const u32x4 (&qf)[D / 32],
                                             const DecOffs<D, KV8>& o, int t0, int ctx, float cexp, int lane) {
  using L = StepLds<D, KV8>;
  constexpr int NB = L::NB;
  constexpr int KS = D / 32;
  constexpr int VC = D / 16;
  const int g = lane >> 4;
  if constexpr (TAIL) {
    // whole rows: the swizzle only permutes chunks within a row
#pragma unroll
    for (int k = 0; k < 16 * NB * L::C8 / 64; ++k) {
      const int idx = lane + 64 * k;
      const int row = idx / L::C8;  // 0 .. 16 NB - 1 over the step's blocks
      if (t0 + row >= ctx)
        *reinterpret_cast<u32x4*>(buf + NB * L::BLK + (row >> 4) * L::BLK + (row & 15) * L::RB +
                                  16 * (idx % L::C8)) = u32x4{0, 0, 0, 0};
    }
  }
  f32x4 sacc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    sacc[j] = f32x4{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 kf;
      if constexpr (KV8)
        kf = e4m3x8<T>(*reinterpret_cast<const u32x2*>(buf + j * L::BLK + o.k[s]));
      else
        kf = *reinterpret_cast<const u32x4*>(buf + j * L::BLK + o.k[s]);
      sacc[j] = T::mfma16(kf, qf[s], sacc[j]);
    }
  }
  if constexpr (TAIL) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sacc[j][r] = (t0 + 16 * j + 4 * g + r) >= ctx ? -__builtin_inff() : sacc[j][r];
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < NB; ++j)
    mx = fmaxf(mx, fmaxf(fmaxf(sacc[j][0], sacc[j][1]), fmaxf(sacc[j][2], sacc[j][3])));
  mx = row_swap_max(mx);
  mx = half_swap_max(mx) * cexp;
  const bool grow = mx > st.m + kDecodeLazy;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float m_new = grow ? mx : st.m;
    const float alpha = grow ? fast_exp2(st.m - m_new) : 1.f;
    st.m = m_new;
    st.l *= alpha;
    st.lr *= alpha;
    // output rows are heads 4g + r: fetch their factors from lane 4g + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int n = 0; n < VC; ++n) st.o[n][r] *= ar;
    }
  }
  const float msub = st.m == -__builtin_inff() ? 0.f : st.m;
  float pv[4 * NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[4 * j + r] = fast_exp2(__builtin_fmaf(sacc[j][r], cexp, -msub));
      st.l += pv[4 * j + r];
    }
  if constexpr (NB == 1) {
    // one 16-bit block: P (heads x 16 tokens; lane group g holds tokens 4g ..
    // 4g + 3, the scores' own layout) times V (16 tokens x 16 columns, one
    // transposing read) on the 16x16x16 instruction
    const u32x2 pf = {T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3])};
    st.lr = T::sum2(pf[1], T::sum2(pf[0], st.lr));  // the rounded probabilities the product applies
#pragma unroll
    for (int n = 0; n < VC; ++n) {
      const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + L::BLK + o.v[n]));
      st.o[n] = T::mfma16k16(pf, __builtin_bit_cast(u32x2, v), st.o[n]);
    }
  } else {
    // P of each block pair h: in lane group g, tokens 4g .. 4g+3 of block 2h,
    // then of block 2h + 1; the transposing reads give V in the same order
    u32x4 pf[NB / 2];
#pragma unroll
    for (int h = 0; h < NB / 2; ++h) {
      const float* v = pv + 8 * h;
      pf[h] = u32x4{T::pack2(v[0], v[1]), T::pack2(v[2], v[3]), T::pack2(v[4], v[5]), T::pack2(v[6], v[7])};
      // the running sum adds the rounded probabilities that the P.V product applies
#pragma unroll
      for (int e = 0; e < 4; ++e) st.lr = T::sum2(pf[h][e], st.lr);
    }
#pragma unroll
    for (int n = 0; n < VC; ++n) {
      if constexpr (KV8) {
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
          const i32x2 v8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(buf + o.v[n] + 2 * h * L::BLK));
          st.o[n] = T::mfma16(pf[h], e4m3x8<T>(__builtin_bit_cast(u32x2, v8)), st.o[n]);
        }
      } else {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + NB * L::BLK + o.v[n]));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + (NB + 1) * L::BLK + o.v[n]));
        const u32x2 a0 = __builtin_bit_cast(u32x2, v0);
        const u32x2 a1 = __builtin_bit_cast(u32x2, v1);
        st.o[n] = T::mfma16(pf[0], u32x4{a0[0], a0[1], a1[0], a1[1]}, st.o[n]);
      }
    }
  }
}

// Step buffers per wavefront: 16 KiB together at D = 128. With two (16-bit
// cache), step p + 1's blocks travel into one while step p computes from the
// other, and step p + 2's loads start as soon as step p's reads have returned;
// with one (E4M3 cache), step p + 1's loads start once step p's reads have
// returned. Ten wavefronts per CU fit, so every workgroup of a typical batch
// starts at once. Ten per CU means three on some SIMDs: for the 16-bit cache
// the launch bound asks for at least three wavefronts per SIMD, which caps a
// wavefront at 170 registers. (With the bare bound the compiler may use all
// 512 of one wavefront, and does: the matrix instructions then accumulate in
// AGPRs and every step copies O between them and the VGPRs the rescale works
// in.) The E4M3 form keeps the bare bound and those copies: capped, its
// four-block steps measured 2-3 % slower per call (25.6-25.9 against
// 26.2-26.7 µs on the Qwen-shaped batch, three boxes).
template <class T, int D, bool KV8>
__global__ __launch_bounds__(64, KV8 ? 1 : 3) void decode_split_kernel(DecodeArgs a) {
  using L = StepLds<D, KV8>;
  constexpr int KS = D / 32;
  constexpr int VC = D / 16;
  constexpr int NB = L::NB;
  constexpr int NS = kSplitBlocks / NB;  // steps per split
  static_assert(D == 128 || D == 64, "head size");
  static_assert(L::NBUF == 1 || L::LOADS == 8 || L::LOADS == 4, "step load count (the partial wait below)");
  __shared__ __align__(16) char buf[L::NBUF * L::BYTES];

  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  // Workgroups reach the XCDs round-robin in launch order, so blockIdx.x
  // alone would pick the XCD (the grid's x extent is a multiple of 8 in
  // practice), and split 0 of every sequence, always live, would land on
  // one XCD while the late splits, live only for long contexts, share
  // another. Rotating the split by the (sequence, kv head) index spreads
  // each pair's live splits over consecutive XCDs from a rotating start.
  const int split = (int)(((unsigned)blockIdx.x + (unsigned)(kvh + a.Hkv * b)) % (unsigned)a.nsplit);
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int G = a.G;
  const int blk0 = split * kSplitBlocks;
  const int* trow = a.table + (size_t)b * a.max_blocks;

  // The split's block-table entries are read together with the context
  // length (scalar loads, one round trip); entries at or beyond the sequence's
  // end may be read (if they exist in the table) but are never used.
  int phys[kSplitBlocks];
#pragma unroll
  for (int i = 0; i < kSplitBlocks; ++i) phys[i] = trow[min(blk0 + i, a.max_blocks - 1)];
  // materialise the entries here (one wait for all) rather than letting the
  // compiler sink each load into the branch that uses it
  static_assert(kSplitBlocks % 8 == 0, "split length");
#pragma unroll
  for (int i = 0; i < kSplitBlocks; i += 8)
    asm volatile("" ::"s"(phys[i]), "s"(phys[i + 1]), "s"(phys[i + 2]), "s"(phys[i + 3]), "s"(phys[i + 4]),
                 "s"(phys[i + 5]), "s"(phys[i + 6]), "s"(phys[i + 7]));
  const int ctx = a.ctx[b];
  const int nblk = (ctx + kDecodeBlock - 1) / kDecodeBlock;
  const int nsp = (nblk + kSplitBlocks - 1) / kSplitBlocks;
  if (split >= nsp) {
    // a split past the sequence's end publishes an empty partial (log2-sum-exp
    // = -inf, weight 0) so that the merge needs no context length
    if (a.nsplit > 1 && lane < G)
      a.ws[(((size_t)b * a.Hq + kvh * G + lane) * a.nsplit + split) * (D + 4) + D] = -__builtin_inff();
    return;
  }
  const int nb = min(kSplitBlocks, nblk - blk0);  // blocks of this split, >= 1
  const int ns = (nb + NB - 1) / NB;  // live steps

  const size_t head_bytes = (size_t)L::BLK;  // one (block, kv head)
  const size_t block_stride = (size_t)a.Hkv * head_bytes;
  const char* kbase = static_cast<const char*>(a.kc) + kvh * head_bytes;
  const char* vbase = static_cast<const char*>(a.vc) + kvh * head_bytes;
  DecOffs<D, KV8> o;
  make_dec_offs<D, KV8>(o, lane);
  // E4M3 caches: k_scale multiplies every score, v_scale every value
  const float cexp = KV8 ? a.c * a.k_scale : a.c;

  // ---- q^T operand: head c, columns 32s + 8g .. +8 (step s, lane group g)
  u32x4 qf[KS];
  const bool q_live = c < G && a.qmode != 2;
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + kvh * G + (q_live ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 32 * s + 8 * g);
  }
  // rotary embedding (optional) at the query's position ctx - 1: fragment
  // s < KS/2 holds columns 32s + 8g .. +8 of the first half, s + KS/2 their
  // partners; the table values are loaded here and applied once the K/V loads
  // are under way
  f32x4 rcs[KS / 2][2], rsn[KS / 2][2];
  if (a.rope) {
    const float* tr = a.rope + (size_t)min(ctx - 1, a.max_pos - 1) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS / 2; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        rcs[s][u] = *reinterpret_cast<const f32x4*>(tr + 32 * s + 4 * u);
        rsn[s][u] = *reinterpret_cast<const f32x4*>(tr + D / 2 + 32 * s + 4 * u);
      }
  }

  // Step q's physical blocks (q < ns): a block past the split's last one
  // carries the step's first block (a cache hit; its tokens are masked), so
  // that every step issues the same loads. q is a compile-time index wherever
  // this is used (the step loop is unrolled); the selection is made between
  // values (readfirstlane), not between array elements, which the compiler
  // would turn into one dynamically indexed load and so keep phys[] in
  // scratch memory.
  auto step_blocks = [&](int q, int (&ph)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = NB * q + j;
      const int own = __builtin_amdgcn_readfirstlane(phys[i]);
      const int first = __builtin_amdgcn_readfirstlane(phys[NB * q]);
      ph[j] = i < nb ? own : first;
    }
  };
  {
    int ph[NB];
    step_blocks(0, ph);
    load_step<D, KV8>(buf, kbase, vbase, block_stride, ph, a.num_blocks, o);
    if (L::NBUF == 2 && ns > 1) {
      step_blocks(1, ph);
      load_step<D, KV8>(buf + L::BYTES, kbase, vbase, block_stride, ph, a.num_blocks, o);
    }
  }

  if (a.rope) {
#pragma unroll
    for (int s = 0; s < KS / 2; ++s) {
      const float cs[8] = {rcs[s][0][0], rcs[s][0][1], rcs[s][0][2], rcs[s][0][3],
                           rcs[s][1][0], rcs[s][1][1], rcs[s][1][2], rcs[s][1][3]};
      const float sn[8] = {rsn[s][0][0], rsn[s][0][1], rsn[s][0][2], rsn[s][0][3],
                           rsn[s][1][0], rsn[s][1][1], rsn[s][1][2], rsn[s][1][3]};
      rope8<T>(qf[s], qf[s + KS / 2], cs, sn);
    }
  }
  {
    const uint32_t flip = a.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = q_live ? (qf[s] ^ flip) : u32x4{0, 0, 0, 0};
  }

  WaveState<D> st;
#pragma unroll
  for (int n = 0; n < VC; ++n) st.o[n] = f32x4{};
  st.m = -__builtin_inff();
  st.l = 0.f;
  st.lr = 0.f;

  // (not unrolled: the loop has a data-dependent exit, and the buffer of
  // step p is addressed from p's parity)
  for (int p = 0; p < NS; ++p) {
    if (p >= ns) break;  // wave-uniform
    // step p has landed: with step p + 1's loads issued after it, at most
    // those LOADS instructions may still be outstanding (loads complete in
    // order for this count)
    if (L::NBUF == 2 && p + 1 < ns) {
      if constexpr (L::LOADS == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    char* cur = buf + (L::NBUF == 2 ? (p & 1) * L::BYTES : 0);
    const int t0 = (blk0 + NB * p) * kDecodeBlock;
    if (t0 + 16 * NB > ctx)
      step_compute<T, D, KV8, true>(st, cur, qf, o, t0, ctx, cexp, lane);
    else
      step_compute<T, D, KV8, false>(st, cur, qf, o, t0, ctx, cexp, lane);
    if (p + L::NBUF < NS && p + L::NBUF < ns) {
      // every read of this buffer has returned before a later step's data is written to it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int q = p + L::NBUF < NS ? p + L::NBUF : 0;  // in range also where the branch is dead
      int ph[NB];
      step_blocks(q, ph);
      load_step<D, KV8>(cur, kbase, vbase, block_stride, ph, a.num_blocks, o);
    }
  }

  // ---- per-head totals (lane c: head c), then the split's result per head
  float l_head = st.l + __shfl_xor(st.l, 16);
  l_head = half_swap_sum(l_head);
  float lr_head = st.lr + __shfl_xor(st.lr, 16);
  lr_head = half_swap_sum(lr_head);
  const bool single = a.nsplit == 1;  // the whole grid has one split: no merge pass
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    // > 0: the split holds a visible token
    const float inv = (KV8 ? a.v_scale : 1.f) / __shfl(lr_head, h);
    if (h < G) {
      const int hq = kvh * G + h;
      if (single) {
        uint16_t* op = static_cast<uint16_t*>(a.o) + ((size_t)b * a.Hq + hq) * D + c;
#pragma unroll
        for (int n = 0; n < VC; ++n) op[16 * n] = (uint16_t)(T::pack2(st.o[n][r] * inv, 0.f) & 0xffffu);
      } else {
        float* wp = a.ws + (((size_t)b * a.Hq + hq) * a.nsplit + split) * (D + 4) + c;
#pragma unroll
        for (int n = 0; n < VC; ++n) wp[16 * n] = st.o[n][r] * inv;
      }
    }
  }
  if (g == 0 && c < G) {  // lane c holds head c's statistics
    const int hq = kvh * G + c;
    const float lse2 = st.m + fast_log2(l_head);
    if (single) {
      if (a.lse) a.lse[(size_t)b * a.Hq + hq] = lse2 * kLn2;
    } else {
      a.ws[(((size_t)b * a.Hq + hq) * a.nsplit + split) * (D + 4) + D] = lse2;
    }
  }
}

// Second pass (the reduction of the split-K decomposition): merge the partials
// of a sequence's splits. One workgroup of D threads per (query head,
// sequence); thread d produces output column d. Every split slot holds a
// partial (splits past the sequence's end hold log2-sum-exp = -inf, and their
// values are never used), so the slots are read 16 at a time with no
// dependent load (one round for up to 16 splits).
template <class T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const float* wp = a.ws + ((size_t)b * a.Hq + hq) * a.nsplit * (D + 4);
  float m = -__builtin_inff(), W = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += 16) {
    float ls[16], part[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sp = min(s0 + u, a.nsplit - 1);  // valid address; weight 0 below
      ls[u] = wp[(size_t)sp * (D + 4) + D];
      part[u] = wp[(size_t)sp * (D + 4) + d];
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < 16; ++u) mc = s0 + u < a.nsplit ? fmaxf(mc, ls[u]) : mc;
    const float r = mc == -__builtin_inff() ? 0.f : fast_exp2(m - mc);  // 0 while nothing is merged
    W *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool live = s0 + u < a.nsplit && ls[u] != -__builtin_inff();
      const float wt = live ? fast_exp2(ls[u] - mc) : 0.f;
      W += wt;
      acc += live ? wt * part[u] : 0.f;  // an empty slot's values are never read into O
    }
    m = mc;
  }
  uint16_t* op = static_cast<uint16_t*>(a.o);
  op[((size_t)b * a.Hq + hq) * D + d] = (uint16_t)(T::pack2(acc / W, 0.f) & 0xffffu);
  if (d == 0 && a.lse) a.lse[(size_t)b * a.Hq + hq] = (m + fast_log2(W)) * kLn2;
}

template <class T, int D, bool KV8>
static hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D, KV8>), dim3(a.nsplit, a.Hkv, a.B), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.Hq, a.B), dim3(D), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (a.D == 128) return bf16 ? launch_d<BF16, 128, false>(a, stream) : launch_d<F16, 128, false>(a, stream);
  return bf16 ? launch_d<BF16, 64, false>(a, stream) : launch_d<F16, 64, false>(a, stream);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (a.D == 128) return bf16 ? launch_d<BF16, 128, true>(a, stream) : launch_d<F16, 128, true>(a, stream);
  return bf16 ? launch_d<BF16, 64, true>(a, stream) : launch_d<F16, 64, true>(a, stream);
}

// Split partials of the entry point that allocates nothing: a file-scope device
// array, one copy per GPU for the life of the process. In host code its name is
// a host-side stand-in, not a device address; the device address of each GPU's
// copy comes from hipGetSymbolAddress with that GPU current, once per device,
// and only that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace attn
