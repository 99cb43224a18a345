// Writing new keys/values into the paged KV cache.
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

#include "launch.h"

namespace attn {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int C8 = D / 8;  // 16-byte chunks per row
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int t = idx / C8, c = idx % C8;
  const int n = a.new_lens ? min(a.new_lens[b], a.Tnew) : a.Tnew;
  if (t >= n) return;
  const int pos = a.start[b] + t;
  const int lb = pos / kDecodeBlock;
  if (pos < 0 || lb >= a.max_blocks) return;  // outside the table: nothing to write
  const int phys = a.table[(size_t)b * a.max_blocks + lb];
  if (phys < 0 || phys >= a.num_blocks) return;  // unmapped block: nothing to write
  const size_t src = ((size_t)(b * a.Hkv + kvh) * a.Tnew + t) * D + 8 * c;
  const size_t dst = (((size_t)phys * a.Hkv + kvh) * kDecodeBlock + pos % kDecodeBlock) * D + 8 * c;
  const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.k_new) + src);
  const u32x4_t vx = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.v_new) + src);
  *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.kc) + dst) = kx;
  *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.vc) + dst) = vx;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const long long chunks = (long long)a.Tnew * (a.D / 8);
  const long long gx = (chunks + 255) / 256;
  if (gx > 0x7fffffffLL || a.Hkv > 65535 || a.B > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
