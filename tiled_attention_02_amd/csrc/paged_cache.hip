// Writing new keys/values into the paged KV cache (16-bit, or E4M3 codes).
//
// The paged cache keeps a sequence's keys and values in fixed-size blocks of
// 16 tokens, found through a per-sequence block table (the-ai.news, "Snelle
// attention-kernels en operatorfusie versnellen AI-modellen", section
// "FlashAttention-type aandacht en gepagineerde aandacht"). Token i of a new
// chunk becomes position start + i: physical block table[(start + i) / 16],
// slot (start + i) % 16. The copy is pure data movement, bound by HBM
// bandwidth: every 16-byte chunk of a new K/V row is read once and written
// once. Consecutive threads take consecutive chunks of a row, and consecutive
// rows of one block are contiguous in the cache, so reads and writes both
// coalesce into whole rows (256 bytes at D = 128).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "launch.h"

namespace attn {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A workgroup moves consecutive new rows of one (sequence, kv head): each
// thread one 16-byte chunk of the destination row of K and of V for each of
// RPT rows, STRIDE rows apart, so every wavefront instruction covers whole
// contiguous rows and a thread keeps 2 * RPT loads in flight. The loads of
// the new rows depend only on the sequence's chunk length, so they are issued
// together with the block-table entries that place them: one round trip for
// the two per-sequence scalars, then one for the data and the entries.
//
// MODE 0 copies 16-bit rows. MODE 1 / 2 (bf16 / fp16 input) writes E4M3
// codes of x / scale: float32 division (correctly rounded), magnitudes
// clamped to 448 (the conversion would give NaN above 464; values in
// (448, 464] round to 448 either way; NaN stays NaN), then the conversion's
// round to nearest even.
//
// The division is the kernel's main cost (a correctly rounded divide is about
// ten instructions), so for scales in [2^-100, 2^100] it is done as
// q0 = x * rcp, q1 = fma(fma(-scale, q0, x), rcp, q0) with rcp the correctly
// rounded 1 / scale: by Markstein's theorem (rcp within half an ulp of
// 1 / scale, q0 within one ulp of x / scale, the remainder exact in an FMA)
// q1 is the correctly rounded quotient when no step overflows or underflows,
// which holds for 16-bit x and such scales wherever the code depends on it
// (quotients of 2^-12 to 464; checked exactly, with rational arithmetic, for
// every bf16 and fp16 value and a set of scales). Quotients of 464 or more
// keep q0: they saturate to 448 either way, and an infinite q0 would turn the
// correction into NaN; the sign of zero comes from q0. Other scales take the
// division itself.
constexpr int kAppendRowsPerThread = 4;
// rows per thread of the quantizing modes (two source chunks per destination
// chunk, 32 rows per workgroup): measured on a 1024-row chunk of 4 sequences
// with 8 kv heads, 11.2 us at four rows, 8.7 at two, 7.8 at one (the copy is
// fastest at four: 7.4 us, 8.2 at two)
constexpr int kAppendRowsPerThread8 = 1;
template <int MODE>
constexpr int append_rows_per_thread() { return MODE ? kAppendRowsPerThread8 : kAppendRowsPerThread; }

template <int MODE>
__device__ __forceinline__ float elem_to_f32(uint32_t w, int half) {
  const uint32_t bits = half ? (w >> 16) : (w & 0xffffu);
  if constexpr (MODE == 1) return __builtin_bit_cast(float, bits << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ float clamp448(float y) { return y > 448.f ? 448.f : (y < -448.f ? -448.f : y); }

template <bool FAST>
__device__ __forceinline__ float e4m3_in_range(float x, float scale, float rcp) {
  if constexpr (FAST) {
    const float q0 = x * rcp;
    // the sign from q0: for x = -0 the correction computes (+0) + (-0) = +0
    const float q1 = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-scale, q0, x), rcp, q0), q0);
    return clamp448(__builtin_fabsf(q0) < 464.f ? q1 : q0);
  } else {
    (void)rcp;
    return clamp448(__fdiv_rn(x, scale));
  }
}

// scale range of the multiply-and-correct division
__device__ __forceinline__ bool fast_quotient(float scale) { return scale >= 0x1p-100f && scale <= 0x1p100f; }

// 16 source elements (two 16-byte chunks) -> 16 E4M3 codes, code e in byte e.
template <int MODE, bool FAST>
__device__ __forceinline__ u32x4_t quantize16_t(const u32x4_t (&x)[2], float scale, float rcp) {
  u32x4_t out;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w0 = x[d / 2][2 * (d % 2)], w1 = x[d / 2][2 * (d % 2) + 1];
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_in_range<FAST>(elem_to_f32<MODE>(w0, 0), scale, rcp),
                                            e4m3_in_range<FAST>(elem_to_f32<MODE>(w0, 1), scale, rcp), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_in_range<FAST>(elem_to_f32<MODE>(w1, 0), scale, rcp),
                                        e4m3_in_range<FAST>(elem_to_f32<MODE>(w1, 1), scale, rcp), r, true);
    out[d] = (uint32_t)r;
  }
  return out;
}

// rcp: the correctly rounded 1 / scale (used when fast_quotient(scale))
template <int MODE>
__device__ __forceinline__ u32x4_t quantize16(const u32x4_t (&x)[2], float scale, float rcp) {
  if (fast_quotient(scale)) return quantize16_t<MODE, true>(x, scale, rcp);  // uniform branch
  return quantize16_t<MODE, false>(x, scale, rcp);
}

template <int D, bool HAS_LENS, int MODE>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int NS = MODE ? 2 : 1;             // 16-byte source chunks per destination chunk
  constexpr int EPC = 8 * NS;                  // elements per destination chunk
  constexpr int CPR = D / EPC;                 // destination chunks per row
  constexpr int EB = MODE ? 1 : 2;             // destination bytes per element
  constexpr int RPT = append_rows_per_thread<MODE>();
  constexpr int STRIDE = 256 / CPR;            // rows covered by one pass of the workgroup
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % CPR;
  const int t0 = blockIdx.x * (STRIDE * RPT) + threadIdx.x / CPR;
  const int start = a.start[b];
  const int n = HAS_LENS ? min(a.new_lens[b], a.Tnew) : a.Tnew;
  asm volatile("" ::"s"(start), "s"(n));  // both scalars in one round trip
  if (t0 >= n) return;
  const size_t row0 = (size_t)(b * a.Hkv + kvh) * a.Tnew;
  const int* trow = a.table + (size_t)b * a.max_blocks;
  u32x4_t kx[RPT][NS], vx[RPT][NS];
  int phys[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    // rows past the chunk re-read the last valid row (in bounds) and are dropped below
    const int t = min(t0 + j * STRIDE, n - 1);
    const size_t src = (row0 + t) * D + EPC * c;
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      kx[j][h] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.k_new) + src + 8 * h));
      vx[j][h] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.v_new) + src + 8 * h));
    }
    phys[j] = trow[min(max((start + t) / kDecodeBlock, 0), a.max_blocks - 1)];
  }
  // keeps the data loads here, ahead of the checks on the entries (the
  // compiler would otherwise sink them into the stores' blocks)
#pragma unroll
  for (int j = 0; j < RPT; ++j)
#pragma unroll
    for (int h = 0; h < NS; ++h) asm volatile("" ::"v"(kx[j][h]), "v"(vx[j][h]));
  // correctly rounded reciprocals of the scales (E4M3 modes)
  const float k_rcp = MODE ? __fdiv_rn(1.f, a.k_scale) : 1.f;
  const float v_rcp = MODE ? __fdiv_rn(1.f, a.v_scale) : 1.f;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int t = t0 + j * STRIDE;
    const int pos = start + t;
    // past the chunk, outside the table or on an unmapped entry: nothing to write
    if (t >= n || pos < 0 || pos / kDecodeBlock >= a.max_blocks || phys[j] < 0 || phys[j] >= a.num_blocks) continue;
    const size_t dst = ((((size_t)phys[j] * a.Hkv + kvh) * kDecodeBlock + pos % kDecodeBlock) * D + EPC * c) * EB;
    u32x4_t ko, vo;
    if constexpr (MODE == 0) {
      ko = kx[j][0];
      vo = vx[j][0];
    } else {
      ko = quantize16<MODE>(kx[j], a.k_scale, k_rcp);
      vo = quantize16<MODE>(vx[j], a.v_scale, v_rcp);
    }
    *reinterpret_cast<u32x4_t*>(static_cast<char*>(a.kc) + dst) = ko;
    *reinterpret_cast<u32x4_t*>(static_cast<char*>(a.vc) + dst) = vo;
  }
}

template <int D, int MODE>
static void launch_dm(const AppendArgs& a, dim3 grid, hipStream_t stream) {
  if (a.new_lens)
    hipLaunchKernelGGL((append_kernel<D, true, MODE>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((append_kernel<D, false, MODE>), grid, dim3(256), 0, stream, a);
}

template <int MODE>
static hipError_t launch_mode(const AppendArgs& a, hipStream_t stream) {
  const long long epc = MODE ? 16 : 8;
  const long long rows_per_wg = (256 / (a.D / epc)) * append_rows_per_thread<MODE>();
  const long long gx = (a.Tnew + rows_per_wg - 1) / rows_per_wg;
  if (gx > 0x7fffffffLL || a.Hkv > 65535 || a.B > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 128)
    launch_dm<128, MODE>(a, grid, stream);
  else
    launch_dm<64, MODE>(a, grid, stream);
  return hipGetLastError();
}

// Rotary form: K rows are rotated at their positions (start + i) on the way
// into the cache, V rows copied. A thread owns the column pairs (i, i + D/2)
// of one 8-column chunk i = 8c of RPT rows: K chunks c and c + C8/2, the
// table's cosines and sines of those 8 frequencies, and the same two V chunks.
template <int D, bool HAS_LENS, class T>
__global__ __launch_bounds__(256) void append_rope_kernel(AppendArgs a) {
  constexpr int C8 = D / 8;        // 16-byte chunks per row
  constexpr int CPR = C8 / 2;      // threads per row
  constexpr int RPT = kAppendRowsPerThread;
  constexpr int STRIDE = 256 / CPR;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % CPR;
  const int t0 = blockIdx.x * (STRIDE * RPT) + threadIdx.x / CPR;
  const int start = a.start[b];
  const int n = HAS_LENS ? min(a.new_lens[b], a.Tnew) : a.Tnew;
  asm volatile("" ::"s"(start), "s"(n));  // both scalars in one round trip
  if (t0 >= n) return;
  const size_t row0 = (size_t)(b * a.Hkv + kvh) * a.Tnew;
  const int* trow = a.table + (size_t)b * a.max_blocks;
  u32x4_t kx[RPT][2], vx[RPT][2];
  f32x4 cs[RPT][2], sn[RPT][2];
  int phys[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int t = min(t0 + j * STRIDE, n - 1);  // rows past the chunk: in bounds, dropped below
    const size_t src = (row0 + t) * D + 8 * c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kx[j][h] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.k_new) + src + h * (D / 2)));
      vx[j][h] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.v_new) + src + h * (D / 2)));
    }
    const float* tr = a.rope + (size_t)min(max(start + t, 0), a.max_pos - 1) * D + 8 * c;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      cs[j][u] = *reinterpret_cast<const f32x4*>(tr + 4 * u);
      sn[j][u] = *reinterpret_cast<const f32x4*>(tr + D / 2 + 4 * u);
    }
    phys[j] = trow[min(max((start + t) / kDecodeBlock, 0), a.max_blocks - 1)];
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(kx[j][h]), "v"(vx[j][h]));
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int t = t0 + j * STRIDE;
    const int pos = start + t;
    if (t >= n || pos < 0 || pos / kDecodeBlock >= a.max_blocks || phys[j] < 0 || phys[j] >= a.num_blocks) continue;
    const float c8[8] = {cs[j][0][0], cs[j][0][1], cs[j][0][2], cs[j][0][3], cs[j][1][0], cs[j][1][1], cs[j][1][2],
                         cs[j][1][3]};
    const float s8[8] = {sn[j][0][0], sn[j][0][1], sn[j][0][2], sn[j][0][3], sn[j][1][0], sn[j][1][1], sn[j][1][2],
                         sn[j][1][3]};
    u32x4 k1 = kx[j][0], k2 = kx[j][1];
    rope8<T>(k1, k2, c8, s8);
    const size_t dst = (((size_t)phys[j] * a.Hkv + kvh) * kDecodeBlock + pos % kDecodeBlock) * D + 8 * c;
    uint16_t* kc = static_cast<uint16_t*>(a.kc) + dst;
    uint16_t* vc = static_cast<uint16_t*>(a.vc) + dst;
    *reinterpret_cast<u32x4*>(kc) = k1;
    *reinterpret_cast<u32x4*>(kc + D / 2) = k2;
    *reinterpret_cast<u32x4_t*>(vc) = vx[j][0];
    *reinterpret_cast<u32x4_t*>(vc + D / 2) = vx[j][1];
  }
}

template <int D, class T>
static void launch_rope_d(const AppendArgs& a, dim3 grid, hipStream_t stream) {
  if (a.new_lens)
    hipLaunchKernelGGL((append_rope_kernel<D, true, T>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((append_rope_kernel<D, false, T>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) { return launch_mode<0>(a, stream); }

hipError_t launch_append_rope(const AppendArgs& a, bool bf16, hipStream_t stream) {
  const long long rows_per_wg = (256 / (a.D / 16)) * kAppendRowsPerThread;
  const long long gx = (a.Tnew + rows_per_wg - 1) / rows_per_wg;
  if (gx > 0x7fffffffLL || a.Hkv > 65535 || a.B > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 128)
    bf16 ? launch_rope_d<128, BF16>(a, grid, stream) : launch_rope_d<128, F16>(a, grid, stream);
  else
    bf16 ? launch_rope_d<64, BF16>(a, grid, stream) : launch_rope_d<64, F16>(a, grid, stream);
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, bool bf16, hipStream_t stream) {
  return bf16 ? launch_mode<1>(a, stream) : launch_mode<2>(a, stream);
}

}  // namespace attn
