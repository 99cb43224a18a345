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

// A workgroup moves RPW consecutive new rows of one (sequence, kv head): each
// thread one 16-byte chunk of K and of V for each of RPT rows, RPW / RPT rows
// apart, so every wavefront instruction covers whole contiguous rows and a
// thread keeps 2 * RPT loads in flight. The loads of the new rows depend only
// on the sequence's chunk length, so they are issued together with the
// block-table entries that place them: one round trip for the two
// per-sequence scalars, then one for the data and the entries.
constexpr int kAppendRowsPerThread = 4;

template <int D, bool HAS_LENS>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int C8 = D / 8;                    // 16-byte chunks per row
  constexpr int RPT = kAppendRowsPerThread;
  constexpr int STRIDE = 256 / C8;             // rows covered by one pass of the workgroup
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % C8;
  const int t0 = blockIdx.x * (STRIDE * RPT) + threadIdx.x / C8;
  const int start = a.start[b];
  const int n = HAS_LENS ? min(a.new_lens[b], a.Tnew) : a.Tnew;
  asm volatile("" ::"s"(start), "s"(n));  // both scalars in one round trip
  if (t0 >= n) return;
  const size_t row0 = (size_t)(b * a.Hkv + kvh) * a.Tnew;
  const int* trow = a.table + (size_t)b * a.max_blocks;
  u32x4_t kx[RPT], vx[RPT];
  int phys[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    // rows past the chunk re-read the last valid row (in bounds) and are dropped below
    const int t = min(t0 + j * STRIDE, n - 1);
    const size_t src = (row0 + t) * D + 8 * c;
    kx[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.k_new) + src));
    vx[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.v_new) + src));
    phys[j] = trow[min(max((start + t) / kDecodeBlock, 0), a.max_blocks - 1)];
  }
  // keeps the data loads here, ahead of the checks on the entries (the
  // compiler would otherwise sink them into the stores' blocks)
#pragma unroll
  for (int j = 0; j < RPT; ++j) asm volatile("" ::"v"(kx[j]), "v"(vx[j]));
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int t = t0 + j * STRIDE;
    const int pos = start + t;
    // past the chunk, outside the table or on an unmapped entry: nothing to write
    if (t >= n || pos < 0 || pos / kDecodeBlock >= a.max_blocks || phys[j] < 0 || phys[j] >= a.num_blocks) continue;
    const size_t dst = (((size_t)phys[j] * a.Hkv + kvh) * kDecodeBlock + pos % kDecodeBlock) * D + 8 * c;
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.kc) + dst) = kx[j];
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.vc) + dst) = vx[j];
  }
}

template <int D>
static void launch_d(const AppendArgs& a, dim3 grid, hipStream_t stream) {
  if (a.new_lens)
    hipLaunchKernelGGL((append_kernel<D, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((append_kernel<D, false>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const long long rows_per_wg = (256 / (a.D / 8)) * kAppendRowsPerThread;
  const long long gx = (a.Tnew + rows_per_wg - 1) / rows_per_wg;
  if (gx > 0x7fffffffLL || a.Hkv > 65535 || a.B > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 128)
    launch_d<128>(a, grid, stream);
  else
    launch_d<64>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace attn
