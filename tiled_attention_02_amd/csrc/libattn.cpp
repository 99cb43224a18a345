// C ABI of libattn: argument validation, kernel selection and launch on the
// caller's stream. Nothing here allocates device memory or synchronises.
#include "../../include/libattn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

attn_status ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr float kLog2e = 1.4426950408889634f;

// A rotary table (null = no rotation): [max_pos][D] fp32, 16-byte aligned.
attn_status check_rope(const char* fn, const float* rope, int max_pos, int D) {
  if (!rope) return ATTN_OK;
  if (max_pos < 1) return fail(ATTN_ERR_INVALID, "%s: max_pos must be >= 1", fn);
  if (!aligned16(rope)) return fail(ATTN_ERR_INVALID, "%s: the rotary table must be 16-byte aligned", fn);
  if ((double)max_pos * D >= 2147483648.0) return fail(ATTN_ERR_UNSUPPORTED, "%s: rotary table too large", fn);
  return ATTN_OK;
}

// |scale| * log2(e) and how q must be read so that the factor is positive.
void scale_mode(float scale, float* c, int* qmode) {
  if (scale == 0.0f) {
    *c = 1.0f;
    *qmode = 2;
  } else if (scale < 0.0f) {
    *c = -scale * kLog2e;
    *qmode = 1;
  } else {
    *c = scale * kLog2e;
    *qmode = 0;
  }
}

// Shared by the 16-bit and the E4M3 cache forms of the paged decode.
// use_scratch: the partials go to the library's static per-device scratch array
// (the no-allocation entry point) instead of the caller's workspace.
attn_status decode_impl(const char* fn, bool fp8, const void* q, const void* k_cache, const void* v_cache,
                        float k_scale, float v_scale, const float* rope, int max_pos, const int* block_table,
                        const int* ctx_lens, void* o, float* lse, int B, int Hq, int Hkv, int D, int block_size,
                        int max_blocks_per_seq, int num_blocks, float scale, attn_dtype dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, bool use_scratch = false) {
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !o)
    return fail(ATTN_ERR_INVALID, "%s: q, caches, block_table, ctx_lens and o must be non-null", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (block_size != attn::kDecodeBlock)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: block_size=%d (supported: 16)", fn, block_size);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: head size D=%d (supported: 64, 128)", fn, D);
  if (Hq / Hkv > 16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: group size Hq/Hkv=%d (supported: <= 16)", fn, Hq / Hkv);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite", fn);
  if (fp8 && !(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(ATTN_ERR_INVALID, "%s: k_scale and v_scale must be finite and > 0", fn);
  const double ncache = (double)num_blocks * Hkv * block_size * D;
  if (ncache >= 9.0e18 || (double)B * max_blocks_per_seq >= 2147483648.0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERR_INVALID, "%s: q, caches and o must be 16-byte aligned", fn);
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(ctx_lens) & 3u))
    return fail(ATTN_ERR_INVALID, "%s: lse, block_table and ctx_lens must be 4-byte aligned", fn);
  if (attn_status st = check_rope(fn, rope, max_pos, D); st != ATTN_OK) return st;
  const size_t need = attn::decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq);
  const int nsplit = (max_blocks_per_seq + attn::kSplitBlocks - 1) / attn::kSplitBlocks;
  if (use_scratch) {
    if (need > attn::kDecodeScratchBytes)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "%s: the split partials need %zu bytes, more than the %zu-byte scratch of this entry point "
                  "(use attn_decode_paged with a workspace)",
                  fn, need, attn::kDecodeScratchBytes);
  } else if (nsplit > 1) {
    if (!workspace) return fail(ATTN_ERR_INVALID, "%s: workspace is null (%zu bytes needed)", fn, need);
    if (workspace_bytes < need)
      return fail(ATTN_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(ATTN_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
  }
  if (nsplit > 65535 || Hkv > 65535 || B > 65535 || Hq > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: grid too large (splits=%d Hkv=%d Hq=%d B=%d)", fn, nsplit, Hkv, Hq, B);
  if (use_scratch) {
    // the current device's copy of the scratch array (looked up once per device)
    const hipError_t e = attn::decode_scratch(&workspace);
    if (e != hipSuccess || !workspace)
      return fail(ATTN_ERR_HIP, "%s: device address of the scratch array: %s", fn, hipGetErrorString(e));
  }

  attn::DecodeArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.table = block_table;
  a.ctx = ctx_lens;
  a.o = o;
  a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.D = D;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.nsplit = nsplit;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.rope = rope;
  a.max_pos = max_pos;
  scale_mode(scale, &a.c, &a.qmode);
  hipError_t e = fp8 ? attn::launch_decode_fp8(a, dtype == ATTN_BF16, stream)
                     : attn::launch_decode(a, dtype == ATTN_BF16, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// Shared by the 16-bit copy and the E4M3 quantizing forms of the append.
attn_status append_impl(const char* fn, bool fp8, const void* k_new, const void* v_new, void* k_cache,
                        void* v_cache, float k_scale, float v_scale, const float* rope, int max_pos,
                        const int* block_table, const int* start_pos, const int* new_lens, int B, int Hkv, int Tnew,
                        int D, int block_size, int max_blocks_per_seq, int num_blocks, attn_dtype dtype,
                        hipStream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !start_pos)
    return fail(ATTN_ERR_INVALID, "%s: k_new, v_new, caches, block_table and start_pos must be non-null", fn);
  if (B < 1 || Hkv < 1 || Tnew < 1 || D < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (block_size != attn::kDecodeBlock)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: block_size=%d (supported: 16)", fn, block_size);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: head size D=%d (supported: 64, 128)", fn, D);
  if (fp8 && !(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(ATTN_ERR_INVALID, "%s: k_scale and v_scale must be finite and > 0", fn);
  const double nnew = (double)B * Hkv * Tnew * D, ncache = (double)num_blocks * Hkv * block_size * D;
  if (nnew >= 2147483648.0 || ncache >= 9.0e18 || (double)B * max_blocks_per_seq >= 2147483648.0 || B > 65535 ||
      Hkv > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(ATTN_ERR_INVALID, "%s: k_new, v_new and the caches must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(start_pos) & 3u) ||
      (new_lens && (reinterpret_cast<uintptr_t>(new_lens) & 3u)))
    return fail(ATTN_ERR_INVALID, "%s: block_table, start_pos and new_lens must be 4-byte aligned", fn);
  if (attn_status st = check_rope(fn, rope, max_pos, D); st != ATTN_OK) return st;

  attn::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kc = k_cache;
  a.vc = v_cache;
  a.table = block_table;
  a.start = start_pos;
  a.new_lens = new_lens;
  a.B = B;
  a.Hkv = Hkv;
  a.Tnew = Tnew;
  a.D = D;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.rope = rope;
  a.max_pos = max_pos;
  hipError_t e = fp8    ? attn::launch_append_fp8(a, dtype == ATTN_BF16, stream)
                 : rope ? attn::launch_append_rope(a, dtype == ATTN_BF16, stream)
                        : attn::launch_append(a, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

attn_status fwd_paged_impl(const char* fn, bool fp8, const void* q, const void* k_cache, const void* v_cache,
                           float k_scale, float v_scale, const float* rope, int max_pos, const int* block_table, const int* ctx_lens,
                           const int* q_lens, void* o, float* lse, int B, int Hq, int Hkv, int Tq, int D,
                           int block_size, int max_blocks_per_seq, int num_blocks, float scale, int causal,
                           attn_dtype dtype, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !o)
    return fail(ATTN_ERR_INVALID, "%s: q, caches, block_table, ctx_lens and o must be non-null", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || D < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (block_size != attn::kDecodeBlock)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: block_size=%d (supported: 16)", fn, block_size);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: head size D=%d (supported: 64, 128)", fn, D);
  if (max_blocks_per_seq > attn::kMaxPagedPrefillBlocks)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: max_blocks_per_seq=%d (supported: <= %d)", fn, max_blocks_per_seq,
                attn::kMaxPagedPrefillBlocks);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite", fn);
  const double nq = (double)B * Hq * Tq * D, ncache = (double)num_blocks * Hkv * block_size * D;
  if (nq >= 2147483648.0 || ncache >= 9.0e18 || (double)B * max_blocks_per_seq >= 2147483648.0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERR_INVALID, "%s: q, caches and o must be 16-byte aligned", fn);
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) || (q_lens && (reinterpret_cast<uintptr_t>(q_lens) & 3u)))
    return fail(ATTN_ERR_INVALID, "%s: lse, block_table, ctx_lens and q_lens must be 4-byte aligned", fn);

  if (fp8 && !(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(ATTN_ERR_INVALID, "%s: k_scale and v_scale must be finite and > 0", fn);
  if (attn_status st = check_rope(fn, rope, max_pos, D); st != ATTN_OK) return st;

  attn::PrefillArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  a.seq_lens = nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.Tk = 0;
  a.G = Hq / Hkv;
  a.nqt = 0;
  a.xcd_remap = 0;
  a.table = block_table;
  a.ctx_lens = ctx_lens;
  a.q_lens = q_lens;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.rope = rope;
  a.max_pos = max_pos;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  scale_mode(scale, &a.c, &a.qmode);
  hipError_t e = fp8 ? attn::launch_prefill_paged_fp8(a, dtype == ATTN_BF16, D, causal != 0, stream)
                     : attn::launch_prefill_paged(a, dtype == ATTN_BF16, D, causal != 0, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// Linear-layer product: configurations tuned per weight shape. Each entry was
// the fastest of every (rows, waves, unroll) configuration for its shape on
// MI355X at M = 2 (an exhaustive sweep through attn_gemm_splitk_cfg, median of
// 7 calls each after a cache eviction); other shapes take kGemmDefault.
struct GemmTuned {
  int N, K;
  attn::GemmConfig cfg;
};
constexpr GemmTuned kGemmTuned[] = {
    {6144, 4096, {16, 4, 4}},    // fused q/k/v projection
    {4096, 4096, {16, 8, 4}},    // output projection
    {28672, 4096, {16, 8, 4}},   // fused gate/up projection
    {4096, 14336, {16, 12, 2}},  // down projection
};
constexpr attn::GemmConfig kGemmDefault = {16, 8, 4};

attn::GemmConfig gemm_config(int N, int K) {
  for (const GemmTuned& t : kGemmTuned)
    if (t.N == N && t.K == K) return t.cfg;
  return kGemmDefault;
}

attn_status gemm_impl(const char* fn, const void* x, const void* w, void* y, int M, int N, int K,
                      attn_dtype dtype, attn::GemmConfig cfg, hipStream_t stream) {
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (M < 0 || N < 0 || K < 0) return fail(ATTN_ERR_INVALID, "%s: negative size (M=%d N=%d K=%d)", fn, M, N, K);
  if (K % 8 != 0) return fail(ATTN_ERR_UNSUPPORTED, "%s: K = %d is not a multiple of 8", fn, K);
  if (K >= (1 << 24)) return fail(ATTN_ERR_UNSUPPORTED, "%s: K = %d too large", fn, K);
  if (cfg.rows != 16 && cfg.rows != 32)
    return fail(ATTN_ERR_INVALID, "%s: rows = %d (16 or 32)", fn, cfg.rows);
  if (cfg.waves < 1 || cfg.waves > 16) return fail(ATTN_ERR_INVALID, "%s: waves = %d (1 .. 16)", fn, cfg.waves);
  if (cfg.unroll != 1 && cfg.unroll != 2 && cfg.unroll != 4 && cfg.unroll != 8)
    return fail(ATTN_ERR_INVALID, "%s: unroll = %d (1, 2, 4 or 8)", fn, cfg.unroll);
  if (M == 0 || N == 0) return ok();
  if (!y || (K > 0 && (!x || !w)))
    return fail(ATTN_ERR_INVALID, "%s: y, and x and w unless K == 0, must be non-null", fn);
  if (!aligned16(x) || !aligned16(w)) return fail(ATTN_ERR_INVALID, "%s: x and w must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(y) & 1u) return fail(ATTN_ERR_INVALID, "%s: y must be 2-byte aligned", fn);
  attn::GemmArgs a;
  a.w = w;
  a.N = N;
  a.K = K;
  // each wave's K range: a multiple of 32, the waves together covering K
  const int per = (K + cfg.waves - 1) / cfg.waves;
  a.kslice = per < 32 ? 32 : (per + 31) / 32 * 32;
  a.vec_store = (N % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7u) == 0) ? 1 : 0;
  // one launch per kGemmRowsPerLaunch activation rows
  for (int m0 = 0; m0 < M; m0 += attn::kGemmRowsPerLaunch) {
    a.x = static_cast<const uint16_t*>(x) + (size_t)m0 * K;
    a.y = static_cast<uint16_t*>(y) + (size_t)m0 * N;
    a.M = M - m0 < attn::kGemmRowsPerLaunch ? M - m0 : attn::kGemmRowsPerLaunch;
    const hipError_t e = attn::launch_gemm(a, cfg, dtype == ATTN_BF16, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_STATUS_UNKNOWN";
}

const char* attn_last_error(void) { return g_err; }

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Tq, int Tk, int D, float scale, int causal, const int* seq_lens, attn_dtype dtype,
                     hipStream_t stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID, "attn_fwd: q, k, v and o must be non-null");
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || D < 1)
    return fail(ATTN_ERR_INVALID, "attn_fwd: sizes must be >= 1 (B=%d Hq=%d Hkv=%d Tq=%d Tk=%d D=%d)", B, Hq, Hkv,
                Tq, Tk, D);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "attn_fwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: unknown dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: head size D=%d (supported: 64, 128)", D);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID, "attn_fwd: scale must be finite");
  if (seq_lens && Tq != Tk)
    return fail(ATTN_ERR_INVALID, "attn_fwd: seq_lens requires Tq == Tk (got %d, %d)", Tq, Tk);
  const double nq = (double)B * Hq * Tq * D, nk = (double)B * Hkv * Tk * D;
  if (nq >= 2147483648.0 || nk >= 2147483648.0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: tensors must hold fewer than 2^31 elements");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID, "attn_fwd: q, k, v and o must be 16-byte aligned");
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)))
    return fail(ATTN_ERR_INVALID, "attn_fwd: lse / seq_lens must be 4-byte aligned");

  attn::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.seq_lens = seq_lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.Tk = Tk;
  a.G = Hq / Hkv;
  a.nqt = 0;
  a.xcd_remap = 0;
  a.table = nullptr;
  a.ctx_lens = nullptr;
  a.q_lens = nullptr;
  a.max_blocks = 0;
  a.num_blocks = 0;
  a.rope = nullptr;
  a.max_pos = 0;
  scale_mode(scale, &a.c, &a.qmode);
  hipError_t e = attn::launch_prefill(a, dtype == ATTN_BF16, D, causal != 0, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "attn_fwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale, float v_scale,
                         void* o, float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                         const int* seq_lens, attn_dtype dtype, hipStream_t stream) {
  const char* fn = "attn_fwd_fp8";
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID, "%s: q, k, v and o must be non-null", fn);
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || D < 1)
    return fail(ATTN_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dtype);
  if (D != 64 && D != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: head size D=%d (supported: 64, 128)", fn, D);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite", fn);
  if (!(isfinite(q_scale) && isfinite(k_scale) && isfinite(v_scale) && q_scale > 0.f && k_scale > 0.f &&
        v_scale > 0.f))
    return fail(ATTN_ERR_INVALID, "%s: q_scale, k_scale and v_scale must be finite and > 0", fn);
  if (seq_lens && Tq != Tk) return fail(ATTN_ERR_INVALID, "%s: seq_lens requires Tq == Tk (got %d, %d)", fn, Tq, Tk);
  const double nq = (double)B * Hq * Tq * D, nk = (double)B * Hkv * Tk * D;
  if (nq >= 2147483648.0 || nk >= 2147483648.0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: tensors must hold fewer than 2^31 elements", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID, "%s: q, k, v and o must be 16-byte aligned", fn);
  if ((lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)))
    return fail(ATTN_ERR_INVALID, "%s: lse / seq_lens must be 4-byte aligned", fn);

  attn::PrefillArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.seq_lens = seq_lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.Tk = Tk;
  a.G = Hq / Hkv;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  scale_mode(scale, &a.c, &a.qmode);
  hipError_t e = attn::launch_prefill_fp8(a, dtype == ATTN_BF16, D, causal != 0, stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

attn_status attn_gemm_splitk(const void* x, const void* w, void* y, int M, int N, int K, attn_dtype dtype,
                             hipStream_t stream) {
  return gemm_impl("attn_gemm_splitk", x, w, y, M, N, K, dtype, gemm_config(N, K), stream);
}

attn_status attn_gemm_splitk_cfg(const void* x, const void* w, void* y, int M, int N, int K, attn_dtype dtype,
                                 int rows, int waves, int unroll, hipStream_t stream) {
  return gemm_impl("attn_gemm_splitk_cfg", x, w, y, M, N, K, dtype, attn::GemmConfig{rows, waves, unroll}, stream);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_blocks_per_seq, int block_size) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1 || block_size != attn::kDecodeBlock ||
      (D != 64 && D != 128))
    return 0;
  return attn::decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq);
}

attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                              const int* ctx_lens, void* o, float* lse, int B, int Hq, int Hkv, int D,
                              int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                              attn_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("attn_decode_paged", false, q, k_cache, v_cache, 1.f, 1.f, nullptr, 0, block_table, ctx_lens, o, lse, B,
                     Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, scale, dtype, workspace,
                     workspace_bytes, stream);
}

attn_status attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                                      const int* ctx_lens, void* o, float* lse, int B, int Hq, int Hkv, int D,
                                      int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                                      attn_dtype dtype, hipStream_t stream) {
  return decode_impl("attn_decode_paged_noalloc", false, q, k_cache, v_cache, 1.f, 1.f, nullptr, 0, block_table,
                     ctx_lens, o, lse, B, Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                     nullptr, 0, stream, /*use_scratch=*/true);
}

attn_status attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                  float v_scale, const int* block_table, const int* ctx_lens, void* o, float* lse,
                                  int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                                  int num_blocks, float scale, attn_dtype dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("attn_decode_paged_fp8", true, q, k_cache, v_cache, k_scale, v_scale, nullptr, 0, block_table, ctx_lens,
                     o, lse, B, Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, scale, dtype, workspace,
                     workspace_bytes, stream);
}

attn_status attn_decode_paged_rope(const void* q, const void* k_cache, const void* v_cache, const float* rope,
                                   int max_pos, const int* block_table, const int* ctx_lens, void* o, float* lse,
                                   int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                                   int num_blocks, float scale, attn_dtype dtype, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (!rope) return fail(ATTN_ERR_INVALID, "attn_decode_paged_rope: the rotary table must be non-null");
  return decode_impl("attn_decode_paged_rope", false, q, k_cache, v_cache, 1.f, 1.f, rope, max_pos, block_table,
                     ctx_lens, o, lse, B, Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                     workspace, workspace_bytes, stream);
}

attn_status attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                           const int* ctx_lens, const int* q_lens, void* o, float* lse, int B, int Hq, int Hkv,
                           int Tq, int D, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           int causal, attn_dtype dtype, hipStream_t stream) {
  return fwd_paged_impl("attn_fwd_paged", false, q, k_cache, v_cache, 1.f, 1.f, nullptr, 0, block_table, ctx_lens, q_lens, o, lse, B,
                        Hq, Hkv, Tq, D, block_size, max_blocks_per_seq, num_blocks, scale, causal, dtype, stream);
}

attn_status attn_fwd_paged_rope(const void* q, const void* k_cache, const void* v_cache, const float* rope,
                                int max_pos, const int* block_table, const int* ctx_lens, const int* q_lens, void* o,
                                float* lse, int B, int Hq, int Hkv, int Tq, int D, int block_size,
                                int max_blocks_per_seq, int num_blocks, float scale, int causal, attn_dtype dtype,
                                hipStream_t stream) {
  if (!rope) return fail(ATTN_ERR_INVALID, "attn_fwd_paged_rope: the rotary table must be non-null");
  return fwd_paged_impl("attn_fwd_paged_rope", false, q, k_cache, v_cache, 1.f, 1.f, rope, max_pos, block_table, ctx_lens, q_lens, o,
                        lse, B, Hq, Hkv, Tq, D, block_size, max_blocks_per_seq, num_blocks, scale, causal, dtype,
                        stream);
}

attn_status attn_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                               float v_scale, const float* rope, int max_pos, const int* block_table,
                               const int* ctx_lens, const int* q_lens, void* o, float* lse, int B, int Hq, int Hkv,
                               int Tq, int D, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                               int causal, attn_dtype dtype, hipStream_t stream) {
  return fwd_paged_impl("attn_fwd_paged_fp8", true, q, k_cache, v_cache, k_scale, v_scale, rope, max_pos,
                        block_table, ctx_lens, q_lens, o, lse, B, Hq, Hkv, Tq, D, block_size, max_blocks_per_seq,
                        num_blocks, scale, causal, dtype, stream);
}

attn_status attn_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int* block_table, const int* start_pos, const int* new_lens, int B, int Hkv,
                              int Tnew, int D, int block_size, int max_blocks_per_seq, int num_blocks,
                              attn_dtype dtype, hipStream_t stream) {
  return append_impl("attn_cache_append", false, k_new, v_new, k_cache, v_cache, 1.f, 1.f, nullptr, 0, block_table,
                     start_pos, new_lens, B, Hkv, Tnew, D, block_size, max_blocks_per_seq, num_blocks, dtype, stream);
}

attn_status attn_cache_append_rope(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   const float* rope, int max_pos, const int* block_table, const int* start_pos,
                                   const int* new_lens, int B, int Hkv, int Tnew, int D, int block_size,
                                   int max_blocks_per_seq, int num_blocks, attn_dtype dtype, hipStream_t stream) {
  if (!rope) return fail(ATTN_ERR_INVALID, "attn_cache_append_rope: the rotary table must be non-null");
  return append_impl("attn_cache_append_rope", false, k_new, v_new, k_cache, v_cache, 1.f, 1.f, rope, max_pos,
                     block_table, start_pos, new_lens, B, Hkv, Tnew, D, block_size, max_blocks_per_seq, num_blocks,
                     dtype, stream);
}

attn_status attn_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache, float k_scale,
                                  float v_scale, const int* block_table, const int* start_pos, const int* new_lens,
                                  int B, int Hkv, int Tnew, int D, int block_size, int max_blocks_per_seq,
                                  int num_blocks, attn_dtype dtype, hipStream_t stream) {
  return append_impl("attn_cache_append_fp8", true, k_new, v_new, k_cache, v_cache, k_scale, v_scale, nullptr, 0,
                     block_table, start_pos, new_lens, B, Hkv, Tnew, D, block_size, max_blocks_per_seq, num_blocks,
                     dtype, stream);
}

}  // extern "C"
