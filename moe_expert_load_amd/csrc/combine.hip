// Combine: expert outputs from the per-instance dispatch buffer back to token order
// (Waterfill/LPLB blog, section "背景知识与设计原则": DeepEP's combine brings a
// token's routed-expert outputs back; section "共享专家融合作为启用机制": with shared-
// expert fusion the shared slot is one more column of the same layout and combine).
// The weighted sum with the router weights as input is the standard MoE output:
//   y[g] = bf16( sum over k with dest_row[g][k] >= 0 of  w[g][k] * out[dest_row[g][k]] )
// with each product and each addition rounded in fp32, k ascending from +0.0, no
// fused multiply-add, then nearest-even rounding to bf16.
//
// HBM-bound, the permute in reverse: one wave per output token, 4 tokens per
// 256-thread workgroup on the XCD-aware block map; lanes 0..K-1 hold the token's
// rows and weights, broadcast by readlane.  A row is processed in slices of 4 x 16 B
// per lane (4 KiB per wave); the slices of 4 consecutive k are loaded together
// (non-temporal: every dispatch row is read once; +3 % measured) before they are
// accumulated in order.
#include "common.h"

namespace uep {

constexpr int kCbThreads = 256;
constexpr int kCbTokPerBlock = kCbThreads / kWave;
constexpr int kCbVec = 4;     // 16-byte vectors per lane per slice (8 bf16 each)
constexpr int kCbGroup = 4;   // rows loaded together

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// nearest-even fp32 -> bf16; a NaN becomes a quiet NaN with its sign
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kCbThreads) void combine_kernel(const u32x4* __restrict__ y_disp,
                                                             const int32_t* __restrict__ dest_row,
                                                             const float* __restrict__ gate_w,
                                                             u32x4* __restrict__ y,
                                                             int64_t out_rows, int64_t g0,
                                                             int64_t g1, int K, int nvec,
                                                             int32_t* err) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x % kWave;
  const int64_t b = xcd_block(blockIdx.x, gridDim.x);
  // the wave's token, uniform (readfirstlane), so the row spans below live in SGPRs
  const int64_t g = g0 + b * kCbTokPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (g >= g1) return;
  const int d_mine = checked_row(lane < K ? dest_row[g * K + lane] : -1, out_rows, err);
  const int w_mine = lane < K ? __float_as_int(gate_w[g * K + lane]) : 0;
  for (int v0 = 0; v0 < nvec; v0 += kCbVec * kWave) {
    float acc[kCbVec * 8];
#pragma unroll
    for (int i = 0; i < kCbVec * 8; ++i) acc[i] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kCbGroup) {
      int dq[kCbGroup];
      float wq[kCbGroup];
      u32x4 buf[kCbGroup][kCbVec];
#pragma unroll
      for (int q = 0; q < kCbGroup; ++q) {
        const int k = k0 + q;
        dq[q] = k < K ? readlane(d_mine, k) : -1;
        wq[q] = k < K ? __int_as_float(readlane(w_mine, k)) : 0.0f;
        if (dq[q] >= 0) {          // a span per row: vectors past its end read as zero
          const span_t src = span_of(y_disp + (int64_t)dq[q] * nvec, (int64_t)nvec * 16);
#pragma unroll
          for (int u = 0; u < kCbVec; ++u) buf[q][u] = stream_load(src, (v0 + u * kWave + lane) * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < kCbGroup; ++q) {
        if (dq[q] < 0) continue;
        const float w = wq[q];
#pragma unroll
        for (int u = 0; u < kCbVec; ++u) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float p0 = w * bf16_lo(buf[q][u][c]);
            const float p1 = w * bf16_hi(buf[q][u][c]);
            acc[u * 8 + 2 * c] = acc[u * 8 + 2 * c] + p0;
            acc[u * 8 + 2 * c + 1] = acc[u * 8 + 2 * c + 1] + p1;
          }
        }
      }
    }
    const span_t dst = span_of(y + g * nvec, (int64_t)nvec * 16);
#pragma unroll
    for (int u = 0; u < kCbVec; ++u) {           // past the row's end: not written
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[c] = f32_to_bf16(acc[u * 8 + 2 * c]) | (f32_to_bf16(acc[u * 8 + 2 * c + 1]) << 16);
      stream_store(o, dst, (v0 + u * kWave + lane) * 16);
    }
  }
}

}  // namespace uep

using namespace uep;

extern "C" uep_status uep_combine(const uint16_t* y_disp, int64_t out_rows,
                                  const int32_t* dest_row, const float* gate_w, int32_t R,
                                  int32_t T, int32_t K, int32_t H, int32_t r_begin, int32_t r_end,
                                  uint16_t* y, int32_t* err, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || H <= 0 || out_rows < 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (K > 64 || H % 8 != 0 || H > (1 << 29) || (int64_t)R * T * K >= (1ll << 31))
    return UEP_EGEOM;
  const int64_t g0 = (int64_t)r_begin * T, g1 = (int64_t)r_end * T;
  if (g1 == g0) return UEP_OK;
  if (!y_disp || !dest_row || !gate_w || !y) return UEP_EINVAL;
  if ((reinterpret_cast<uintptr_t>(y_disp) | reinterpret_cast<uintptr_t>(y)) % 16 != 0)
    return UEP_EGEOM;
  const int64_t blocks = (g1 - g0 + kCbTokPerBlock - 1) / kCbTokPerBlock;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCbThreads), 0,
                     uep_stream(stream), reinterpret_cast<const u32x4*>(y_disp), dest_row, gate_w,
                     reinterpret_cast<u32x4*>(y), out_rows, g0, g1, K, H / 8, err);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
