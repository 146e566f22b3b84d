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
// Workgroups are dispatched round-robin over the 8 XCDs; the block -> token map
// gives each XCD one contiguous token range, so rows that consecutive tokens write
// into the same instance block meet in one L2.
//
// The inverse map row_src is written by a second, separate launch: 4-byte scattered
// stores mixed into the row stream cost several times more than on their own
// (measured on MI355X: about 4 % of the whole-group permute inline, under 1 % apart).
#include "common.h"

namespace uep {

constexpr int kPmThreads = 256;
constexpr int kPmTokPerBlock = kPmThreads / kWave;
constexpr int kVec = 8;   // 16-byte vectors per lane per slice (8 KiB per wave)

template <bool kNT>
__global__ __launch_bounds__(kPmThreads) void permute_kernel(const u32x4* __restrict__ x,
                                                             const int32_t* __restrict__ dest_row,
                                                             u32x4* __restrict__ out, int64_t out_rows,
                                                             int64_t g0, int64_t g1, int K, int nvec,
                                                             int32_t* err) {
  const int lane = threadIdx.x % kWave;
  const int64_t b = xcd_block(blockIdx.x, gridDim.x);
  const int64_t g = g0 + b * kPmTokPerBlock + threadIdx.x / kWave;
  if (g >= g1) return;
  const int d_mine = checked_row(lane < K ? dest_row[g * K + lane] : -1, out_rows, err);
  const u32x4* src = x + g * nvec;
  for (int v0 = 0; v0 < nvec; v0 += kVec * kWave) {
    u32x4 buf[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nvec) buf[u] = kNT ? __builtin_nontemporal_load(src + v) : src[v];
    }
    for (int k = 0; k < K; ++k) {
      const int d = readlane(d_mine, k);
      if (d < 0) continue;
      u32x4* dst = out + (int64_t)d * nvec;
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nvec) {
          if (kNT) __builtin_nontemporal_store(buf[u], dst + v);
          else dst[v] = buf[u];
        }
      }
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
  if (K > 64 || H % 8 != 0 || (int64_t)R * T * K >= (1ll << 31)) return UEP_EGEOM;
  const int64_t g0 = (int64_t)r_begin * T, g1 = (int64_t)r_end * T;
  if (g1 == g0) return UEP_OK;
  if (!x || !dest_row || !out) return UEP_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) % 16 != 0)
    return UEP_EGEOM;
  const int64_t blocks = (g1 - g0 + kPmTokPerBlock - 1) / kPmTokPerBlock;
  // Rows up to 8 KiB move fastest with plain loads and stores, longer rows with
  // non-temporal ones (measured on MI355X).
  const bool nt = H * 2 > 8192;
  const dim3 grid((unsigned)blocks), block(kPmThreads);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* ov = reinterpret_cast<u32x4*>(out);
  hipStream_t s = uep_stream(stream);
  if (nt)
    hipLaunchKernelGGL(permute_kernel<true>, grid, block, 0, s, xv, dest_row, ov, out_rows, g0, g1,
                       K, H / 8, err);
  else
    hipLaunchKernelGGL(permute_kernel<false>, grid, block, 0, s, xv, dest_row, ov, out_rows, g0, g1,
                       K, H / 8, err);
  UEP_CHECK_LAUNCH();
  if (row_src) {
    const int64_t j0 = g0 * K, j1 = g1 * K;
    const int64_t rblocks = (j1 - j0 + kPmThreads - 1) / kPmThreads;
    // The XCD map helps once the scatter spans many blocks (measured: whole
    // Qwen-layer group faster, one rank's share slower).
    const int swizzle = rblocks >= 4096;
    hipLaunchKernelGGL(row_src_kernel, dim3((unsigned)rblocks), block, 0, s, dest_row, row_src,
                       out_rows, j0, j1, swizzle);
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
