// Split-K matrix product for the linear layers of a decode step, gfx950.
//
// Method: comemg.com, "天下苦英偉達久矣！PyTorch免CUDA加速推理，Triton時代要來？",
// section "Triton SplitK GEMM 內核": the linear layers run as an FP16 GEMM
// whose reduction (K) dimension is split across workers and the pieces
// summed; section "GEMM 內核調優" tunes the kernel for each weight shape.
// Here y[m, n] = sum_k x[m, k] w[n, k] for activations x [M, K], weight w
// [N, K] and output y [M, N], all 16-bit, products and sums in fp32.
//
// At decode sizes (M = a few tokens) the product is a stream of the weight
// (N * K * 2 bytes, read once) with a few flops per byte: HBM-bound. The
// split of K is made inside a workgroup: its waves take consecutive K ranges
// of the same R weight rows and sum their partial tiles in LDS at the end.
// One launch, no workspace, and a fixed summation order (deterministic); the
// workgroups (N / R of them) are enough to fill the chip without splitting
// K across workgroups, which would need a second pass or a cross-workgroup
// merge.
//
// Per k-step of 32 a wave issues one v_mfma_f32_16x16x32 per (16 weight rows,
// 16 activation rows): the A operand is 16 bytes per lane of a weight row
// (row l % 16, k = 8 (l / 16) .. +8), loaded straight from HBM with a
// non-temporal buffer load; the B operand is the same 16 bytes of an
// activation row (cached: every workgroup reads x). Rows past N or M and k
// past the wave's range read as zero (out-of-range buffer offsets), so no
// branch guards the loads.
#include "attn_device.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kGemmDword3 = 0x00020000;  // raw (untyped) buffer descriptor, 32-bit data
constexpr int kOutOfRange = 0x7ffffff0;  // a buffer offset past any range: the load returns zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(pu), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane((int)bytes), kGemmDword3);
}

// AUX: the cache policy bits of the load (2: non-temporal)
template <int AUX>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
#else
  (void)r;
  (void)off;
  return u32x4{};
#endif
}

}  // namespace

// R weight rows per workgroup (R / 16 row tiles), MT tiles of 16 activation
// rows (M <= 16 MT), U k-steps of 32 per round of loads; blockDim.x = 64 * NW.
template <class T, int R, int MT, int U>
__global__ __launch_bounds__(1024) void gemm_splitk_kernel(GemmArgs a) {
  constexpr int RT = R / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * R;

  // this workgroup's weight rows; rows past N are past the descriptor's range
  const int rows = min(R, a.N - n0);
  const __amdgpu_buffer_rsrc_t wr =
      gemm_rsrc(static_cast<const uint16_t*>(a.w) + (size_t)n0 * a.K, (uint32_t)rows * a.K * 2u);
  const __amdgpu_buffer_rsrc_t xr = gemm_rsrc(a.x, (uint32_t)a.M * a.K * 2u);

  // the wave's K range: a.kslice elements (a multiple of 32), the last one cut at K
  const int k_lo = wave * a.kslice;
  const int k_hi = min(a.K, k_lo + a.kslice);
  // per-lane byte offsets of the first k-step; k advances by 64 bytes per step
  int woff[RT], xoff[MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) woff[rt] = ((16 * rt + c) * a.K + k_lo + 8 * g) * 2;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xoff[mt] = ((16 * mt + c) * a.K + k_lo + 8 * g) * 2;

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{};

  for (int k = k_lo; k < k_hi; k += 32 * U) {
    u32x4 af[U][RT], bf[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // this lane's 8 elements lie inside the wave's range (K and the range
      // ends are multiples of 8), or the load reads zero
      const bool live = k + 32 * u + 8 * g < k_hi;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        af[u][rt] = load16</*non-temporal*/ 2>(wr, live ? woff[rt] + 64 * u : kOutOfRange);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) bf[u][mt] = load16<0>(xr, live ? xoff[mt] + 64 * u : kOutOfRange);
    }
    // every load of the round is issued before the first product waits for one
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = T::mfma16(af[u][rt], bf[u][mt], acc[rt][mt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) woff[rt] += 64 * U;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xoff[mt] += 64 * U;
  }

  // ---- sum the waves' partial tiles (in wave order) and write y
  // red[wave][rt][mt][lane] holds the lane's 4 accumulator values: weight rows
  // 16 rt + 4 g + r, activation row 16 mt + c
  extern __shared__ __align__(16) f32x4 red[];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave * RT + rt) * MT + mt) * 64 + lane] = acc[rt][mt];
  __syncthreads();
  for (int e = threadIdx.x; e < RT * MT * 64; e += blockDim.x) {
    f32x4 s = red[e];
    for (int v = 1; v < nw; ++v) s += red[v * RT * MT * 64 + e];
    const int l = e & 63, mt = (e >> 6) % MT, rt = (e >> 6) / MT;
    const int m = 16 * mt + (l & 15);
    const int n = n0 + 16 * rt + 4 * (l >> 4);
    if (m >= a.M) continue;
    uint16_t* yp = static_cast<uint16_t*>(a.y) + (size_t)m * a.N + n;
    if (a.vec_store && n + 3 < a.N) {
      *reinterpret_cast<u32x2*>(yp) = u32x2{T::pack2(s[0], s[1]), T::pack2(s[2], s[3])};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < a.N) yp[r] = (uint16_t)(T::pack2(s[r], 0.f) & 0xffffu);
    }
  }
}

// The partial tiles of every wave sit in LDS for the reduction: up to
// 16 waves x 2 x 4 tiles x 1 KiB = 128 KiB, above the 64 KiB a launch gets
// without asking (gfx950 has 160 KiB per CU).
template <class K>
static hipError_t launch_k(K kernel, const GemmArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, stream, a);
  return hipGetLastError();
}

template <class T, int R, int MT>
static hipError_t launch_u(const GemmArgs& a, int waves, int unroll, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + R - 1) / R)), block((unsigned)(64 * waves));
  const size_t lds = (size_t)waves * (R / 16) * MT * 64 * sizeof(f32x4);
  switch (unroll) {
    case 1: return launch_k(gemm_splitk_kernel<T, R, MT, 1>, a, grid, block, lds, stream);
    case 2: return launch_k(gemm_splitk_kernel<T, R, MT, 2>, a, grid, block, lds, stream);
    case 4: return launch_k(gemm_splitk_kernel<T, R, MT, 4>, a, grid, block, lds, stream);
    default: return launch_k(gemm_splitk_kernel<T, R, MT, 8>, a, grid, block, lds, stream);
  }
}

template <class T, int R>
static hipError_t launch_r(const GemmArgs& a, const GemmConfig& cfg, hipStream_t stream) {
  switch ((a.M + 15) / 16) {  // tiles of 16 activation rows
    case 1: return launch_u<T, R, 1>(a, cfg.waves, cfg.unroll, stream);
    case 2: return launch_u<T, R, 2>(a, cfg.waves, cfg.unroll, stream);
    case 3: return launch_u<T, R, 3>(a, cfg.waves, cfg.unroll, stream);
    default: return launch_u<T, R, 4>(a, cfg.waves, cfg.unroll, stream);
  }
}

template <class T>
static hipError_t launch_t(const GemmArgs& a, const GemmConfig& cfg, hipStream_t stream) {
  return cfg.rows == 32 ? launch_r<T, 32>(a, cfg, stream) : launch_r<T, 16>(a, cfg, stream);
}

hipError_t launch_gemm(const GemmArgs& a, const GemmConfig& cfg, bool bf16, hipStream_t stream) {
  return bf16 ? launch_t<BF16>(a, cfg, stream) : launch_t<F16>(a, cfg, stream);
}

}  // namespace attn
