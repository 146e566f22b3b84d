// Permute token activations into the per-instance dispatch buffer (UltraEP article,
// section "流式通信算子加速动态权重分发": dispatch follows the reroute plan once the
// replica weights are in place).
//
// HBM-bound: every source row is read once and written to its K destination rows
// with 16-byte vector loads and stores.  One wave per source token; a 256-thread
// workgroup moves 4 tokens.  The K destination rows are loaded by lanes 0..K-1 and
// broadcast with readlane, so store addresses stay uniform per row.  Rows are moved
// in slices of kVec 16-byte vectors per lane (1 KiB per wave per vector), all loads
// of a slice issued before its stores.
//
// Read and write phases.  One source row feeds eight destination rows, and HBM takes
// such a mixed stream markedly slower than a pure one (on MI355X a sequential
// 1:8 read/write stream ran about 11 % below a write-only one).  The source range is
// therefore moved in chunks of at most kChunkBytes of source rows, below the 256 MB
// last-level cache: a read-only pass (prefetch_kernel, plain loads, which fill that
// cache) pulls the chunk in, then the permute of the chunk reads it back with
// non-temporal loads and writes with streaming stores (nt sc1), which go to HBM
// without allocating in that cache and so leave the chunk in place.  HBM thus sees a short
// read-only phase, then a write-only phase, per chunk; the launch boundary between
// them keeps the phases apart (the same two phases in one launch, ordered by block
// id, overlapped and ran slower).  Measured on MI355X against one plain launch:
// 3.79 -> 3.65 ms on the Qwen3-235B layer (K = 8, 8 KiB rows), 6.95 -> 6.34 ms on the
// DeepSeek-V3 layout (K = 9, 14 KiB rows), unchanged at 21.5 ms on the LPLB layer.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block -> token map
// gives each XCD one contiguous token range, so rows that consecutive tokens write
// into the same instance block meet in one L2.
//
// The inverse map row_src is written by a second, separate launch: 4-byte scattered
// stores mixed into the row stream cost several times more than on their own
// (measured on MI355X: about 4 % of the whole-group permute inline, under 1 % apart).
#include <algorithm>

#include "common.h"

namespace uep {

constexpr int kPmThreads = 256;
constexpr int kPmTokPerBlock = kPmThreads / kWave;
constexpr int kVec = 8;   // 16-byte vectors per lane per slice (8 KiB per wave)
constexpr int64_t kChunkBytes = 224ll << 20;   // source bytes per read/write phase pair
constexpr int kPfVec = 4;                       // 16-byte loads per thread in the read pass

// Read-only pass over vectors [v0, v1) of x: pulls them into the last-level cache.
// The loaded values feed an empty asm statement, so the loads are kept.
__global__ __launch_bounds__(kPmThreads) void prefetch_kernel(const u32x4* __restrict__ x,
                                                              int64_t v0, int64_t v1) {
  const int64_t base = v0 + (int64_t)blockIdx.x * kPmThreads * kPfVec + threadIdx.x;
  u32x4 b[kPfVec];
#pragma unroll
  for (int k = 0; k < kPfVec; ++k) {
    const int64_t v = base + (int64_t)k * kPmThreads;
    b[k] = v < v1 ? x[v] : u32x4{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kPfVec; ++k) acc |= b[k].x | b[k].y | b[k].z | b[k].w;
  asm volatile("" ::"v"(acc));
}

__global__ __launch_bounds__(kPmThreads) void permute_kernel(const u32x4* __restrict__ x,
                                                             const int32_t* __restrict__ dest_row,
                                                             u32x4* __restrict__ out, int64_t out_rows,
                                                             int64_t g0, int64_t g1, int K, int nvec,
                                                             int32_t* err) {
  const int lane = threadIdx.x % kWave;
  const int64_t b = xcd_block(blockIdx.x, gridDim.x);
  // the wave's token, uniform (readfirstlane), so the row spans below live in SGPRs
  const int64_t g = g0 + b * kPmTokPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (g >= g1) return;
  const int d_mine = checked_row(lane < K ? dest_row[g * K + lane] : -1, out_rows, err);
  // source and destination rows as buffer spans: a vector past the row's end reads as
  // zero and is not written, so no lane needs a guard
  const span_t src = span_of(x + g * nvec, (int64_t)nvec * 16);
  for (int v0 = 0; v0 < nvec; v0 += kVec * kWave) {
    u32x4 buf[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) buf[u] = stream_load(src, (v0 + u * kWave + lane) * 16);
    for (int k = 0; k < K; ++k) {
      const int d = readlane(d_mine, k);
      if (d < 0) continue;
      const span_t dst = span_of(out + (int64_t)d * nvec, (int64_t)nvec * 16);
#pragma unroll
      for (int u = 0; u < kVec; ++u) stream_store(buf[u], dst, (v0 + u * kWave + lane) * 16);
    }
  }
}

// row_src[dest_row[j]] = j for the pairs j in [j0, j1), one thread per pair (rows
// outside the buffer were flagged by the permute and are skipped here).
__global__ __launch_bounds__(kPmThreads) void row_src_kernel(const int32_t* __restrict__ dest_row,
                                                             int32_t* __restrict__ row_src,
                                                             int64_t out_rows, int64_t j0,
                                                             int64_t j1, int swizzle) {
  const int64_t b = swizzle ? xcd_block(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t j = j0 + b * kPmThreads + threadIdx.x;
  if (j >= j1) return;
  const int32_t d = dest_row[j];
  if (d >= 0 && d < out_rows) row_src[d] = (int32_t)j;
}

}  // namespace uep

using namespace uep;

extern "C" uep_status uep_permute(const uint16_t* x, const int32_t* dest_row, int32_t R, int32_t T,
                                  int32_t K, int32_t H, int32_t r_begin, int32_t r_end,
                                  uint16_t* out, int64_t out_rows, int32_t* row_src, int32_t* err,
                                  void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || H <= 0 || out_rows < 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (K > 64 || H % 8 != 0 || H > (1 << 29) || (int64_t)R * T * K >= (1ll << 31))
    return UEP_EGEOM;
  const int64_t g0 = (int64_t)r_begin * T, g1 = (int64_t)r_end * T;
  if (g1 == g0) return UEP_OK;
  if (!x || !dest_row || !out) return UEP_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) % 16 != 0)
    return UEP_EGEOM;
  const int nvec = H / 8;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  hipStream_t s = uep_stream(stream);
  // tokens per phase pair: the range split into the fewest chunks of at most
  // kChunkBytes of source rows, equal up to a multiple of 64 tokens
  const int64_t cap = std::max<int64_t>(64, kChunkBytes / ((int64_t)H * 2) / 64 * 64);
  const int64_t n_chunks = (g1 - g0 + cap - 1) / cap;
  const int64_t chunk = ((g1 - g0 + n_chunks - 1) / n_chunks + 63) / 64 * 64;
  for (int64_t c0 = g0; c0 < g1; c0 += chunk) {
    const int64_t c1 = std::min(g1, c0 + chunk);
    const int64_t v0 = c0 * nvec, v1 = c1 * nvec;
    const int64_t pf_per = (int64_t)kPmThreads * kPfVec;
    const int64_t pf_blocks = (v1 - v0 + pf_per - 1) / pf_per;
    hipLaunchKernelGGL(prefetch_kernel, dim3((unsigned)pf_blocks), dim3(kPmThreads), 0, s, xv, v0,
                       v1);
    UEP_CHECK_LAUNCH();
    const int64_t blocks = (c1 - c0 + kPmTokPerBlock - 1) / kPmTokPerBlock;
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(kPmThreads), 0, s, xv, dest_row,
                       ov, out_rows, c0, c1, K, nvec, err);
    UEP_CHECK_LAUNCH();
  }
  if (row_src) {
    const int64_t j0 = g0 * K, j1 = g1 * K;
    const int64_t rblocks = (j1 - j0 + kPmThreads - 1) / kPmThreads;
    // The XCD map helps once the scatter spans many blocks (measured: whole
    // Qwen-layer group faster, one rank's share slower).
    const int swizzle = rblocks >= 4096;
    hipLaunchKernelGGL(row_src_kernel, dim3((unsigned)rblocks), dim3(kPmThreads), 0, s, dest_row, row_src,
                       out_rows, j0, j1, swizzle);
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
