// Internal interface between the C ABI (libattn.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

// qmode: how the kernels read q so that the exponent factor c is always > 0.
//   0: as stored (scale > 0), 1: sign flipped (scale < 0, exact in 16-bit),
//   2: zero (scale == 0: every score is exactly 0).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* seq_lens;
  int B, Hq, Hkv, Tq, Tk;
  int G;      // Hq / Hkv
  int nqt;    // number of query tiles (set by the launcher)
  float c;    // |scale| * log2(e), or 1 when scale == 0
  int qmode;
  int xcd_remap;  // set by the launcher: group kv-head siblings on one XCD
  int lpt;        // set by the launcher (paged form): query-tile groups in decreasing work
  // paged form (chunked prefill): k / v are the caches [num_blocks][Hkv][16][D]
  const int* table;     // [B][max_blocks]
  const int* ctx_lens;  // [B] keys per sequence
  const int* q_lens;    // [B] query rows per sequence, or null (all Tq)
  int max_blocks, num_blocks;
  // rotary embedding of the query rows (paged form), or null: table [max_pos][D]
  // fp32, cosines in columns 0 .. D/2-1, sines in D/2 .. D-1
  const float* rope;
  int max_pos;
  // E4M3 inputs (fp8 forms): an entry means code value * scale
  float k_scale, v_scale, q_scale;
};

struct AppendArgs {
  const void* k_new;  // [B][Hkv][Tnew][D]
  const void* v_new;
  void* kc;           // [num_blocks][Hkv][16][D]
  void* vc;
  const int* table;   // [B][max_blocks]
  const int* start;   // [B]
  const int* new_lens;  // [B] or null (all Tnew)
  int B, Hkv, Tnew, D, max_blocks, num_blocks;
  // fp8 form: the caches hold E4M3 codes of x / scale
  float k_scale, v_scale;
  // rope form: K rows rotated at their positions (table as in PrefillArgs)
  const float* rope;
  int max_pos;
};

constexpr int kMaxPagedPrefillBlocks = 2048;  // block-table entries a chunked prefill keeps in LDS

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int* table;
  const int* ctx;
  void* o;
  float* lse;
  float* ws;   // per-split partials: [B][Hq][nsplit][D + 4] fp32 (O, then log2-sum-exp, pad)
  int B, Hq, Hkv, G, D;
  int max_blocks;
  int num_blocks;  // physical blocks in the caches: ids outside [0, num_blocks) read as zeros
  int nsplit;  // maximum number of splits per sequence
  float c;
  int qmode;
  // E4M3 caches (fp8 form): an entry means code value * scale
  float k_scale, v_scale;
  // rotary embedding of the query at position ctx - 1, or null (table as in PrefillArgs)
  const float* rope;
  int max_pos;
};

constexpr int kDecodeBlock = 16;        // tokens per cache block
constexpr int kSplitBlocks = 16;        // cache blocks per split (256 tokens)

// Split-K linear-layer product y [M, N] = x [M, K] w [N, K]^T (16-bit).
struct GemmArgs {
  const void* x;
  const void* w;
  void* y;
  int M, N, K;   // M <= kGemmRowsPerLaunch per launch (the C ABI splits larger M)
  int kslice;    // K elements per wave: a multiple of 32, waves * kslice >= K
  int vec_store; // N % 4 == 0 and y 8-byte aligned: 4 outputs per store
};
// rows: weight rows per workgroup (16 or 32); waves: waves per workgroup
// (1 .. 16), each taking one K range; unroll: k-steps of 32 per round of loads
// (1, 2, 4 or 8)
struct GemmConfig {
  int rows, waves, unroll;
};
constexpr int kGemmRowsPerLaunch = 64;  // activation rows per launch: up to 4 tiles of 16

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream);
hipError_t launch_prefill_paged(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream);
hipError_t launch_prefill_paged_fp8(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream);
hipError_t launch_prefill_fp8(const PrefillArgs& a, bool bf16, int D, bool causal, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_append_fp8(const AppendArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_append_rope(const AppendArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, bool bf16, hipStream_t stream);

// The no-allocation decode's scratch: a static device array of this many bytes
// per GPU (the split partials of up to 16 Ki (sequence, query head) pairs with
// 16 splits of 256 tokens at D = 128). decode_scratch returns the current
// device's copy's address, looked up once per device with that device current.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_gemm(const GemmArgs& a, const GemmConfig& cfg, bool bf16, hipStream_t stream);

// Workspace: the per-split partials (Hkv is part of the signature so that a
// layout that depends on it stays a library-internal change).
inline size_t decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_blocks) {
  (void)Hkv;
  const size_t nsplit = (size_t)(max_blocks + kSplitBlocks - 1) / kSplitBlocks;
  return (size_t)B * Hq * nsplit * (size_t)(D + 4) * sizeof(float);
}

}  // namespace attn
