// Waterfill placement of every token's shared-expert slot (Waterfill/LPLB blog,
// section "Waterfill算法执行步骤": load score L_r, waterline
// H = ceil((sum_r L_r + N) / R), slack S_r = max(H - L_r, 0), per-token sampling in
// proportion to slack with a small local preference, zero-slack fallback to a
// clearly lighter candidate; section "通信权衡与模式选择": candidates are the ranks
// the token already visits plus its own, or every rank in the all-rank mode; section
// "共享专家融合作为启用机制": the top-k output gains one column for the shared expert).
//
// wf_prologue: one workgroup turns the load matrix into L_r, H and S_r.
// wf_sample: one thread per token.  The candidate set is a 64-bit mask of visited
//   ranks (R <= 64) minus the source rank, walked in ascending order after the
//   source; the draw is word 0 of Philox4x64-10 (Salmon et al., SC'11) at counter
//   (global token index, 0, 0, 0) and key (seed, layer), scaled to the total weight
//   with a 64x64->128-bit multiply, so the choice is exact integer arithmetic.
#include "common.h"
#include "philox.h"

namespace uep {

__global__ __launch_bounds__(256) void wf_prologue(const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ batch_size, int R,
                                                   int E, int T, int32_t* __restrict__ waterline,
                                                   int32_t* __restrict__ slack,
                                                   int32_t* __restrict__ rank_load) {
  extern __shared__ int32_t wf_lds[];   // [E] expert loads
  __shared__ int32_t s_L[64];
  __shared__ int32_t s_H;
  const int E_loc = E / R;
  for (int e = threadIdx.x; e < E; e += blockDim.x) wf_lds[e] = column_sum(counts, R, E, e);
  __syncthreads();
  if (threadIdx.x < R) {
    int L = 0;
    for (int j = 0; j < E_loc; ++j) L += wf_lds[threadIdx.x * E_loc + j];
    s_L[threadIdx.x] = L;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t tot = 0;
    for (int r = 0; r < R; ++r) {
      const int b = batch_size[r];
      tot += s_L[r] + (b < 0 ? 0 : (b > T ? T : b));
    }
    s_H = (int)((tot + R - 1) / R);
    waterline[0] = s_H;
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int L = s_L[threadIdx.x];
    rank_load[threadIdx.x] = L;
    slack[threadIdx.x] = max(s_H - L, 0);
  }
}

__global__ __launch_bounds__(256) void wf_sample(const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ batch_size,
                                                 const int32_t* __restrict__ slack,
                                                 const int32_t* __restrict__ rank_load, int R,
                                                 int T, int K, int E, uint64_t seed,
                                                 uint64_t layer, int shift, int all_ranks,
                                                 int32_t* __restrict__ shared_rank,
                                                 int32_t* __restrict__ ext) {
  __shared__ int32_t s_S[64], s_L[64], s_B[64];
  if (threadIdx.x < R) {
    s_S[threadIdx.x] = slack[threadIdx.x];
    s_L[threadIdx.x] = rank_load[threadIdx.x];
    s_B[threadIdx.x] = batch_size[threadIdx.x];
  }
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)R * T) return;
  const int r0 = (int)(g / T), t = (int)(g % T);
  const int E_loc = E / R;
  const int32_t* tok = ids + g * K;
  int choice = -1;
  uint64_t visited = 0;
  for (int k = 0; k < K; ++k) {
    const int e = tok[k];
    if (ext) ext[g * (K + 1) + k] = e;
    if (e >= 0 && e < E) visited |= 1ull << (e / E_loc);
  }
  if (t < s_B[r0]) {
    if (all_ranks) visited = R == 64 ? ~0ull : (1ull << R) - 1;
    visited &= ~(1ull << r0);
    const int64_t big = 1ll << shift;
    const int64_t w0 = (big + 1) * s_S[r0];
    int64_t W = w0;
    for (uint64_t m = visited; m; m &= m - 1) W += big * s_S[__ffsll((unsigned long long)m) - 1];
    if (W > 0) {
      const uint64_t u = philox4x64_10_w0((uint64_t)g, 0, 0, 0, seed, layer);
      const uint64_t v = __umul64hi(u, (uint64_t)W);
      uint64_t run = (uint64_t)w0;
      choice = r0;
      if (!(run > v)) {
        for (uint64_t m = visited; m; m &= m - 1) {
          const int c = __ffsll((unsigned long long)m) - 1;
          run += (uint64_t)(big * s_S[c]);
          if (run > v) { choice = c; break; }
        }
      }
    } else {
      choice = r0;
      int64_t bestL = -1;
      const int64_t lr0 = s_L[r0];
      for (uint64_t m = visited; m; m &= m - 1) {
        const int c = __ffsll((unsigned long long)m) - 1;
        const int64_t lc = s_L[c];
        if ((big + 1) * lc < big * lr0 && (bestL < 0 || lc < bestL)) {
          bestL = lc;
          choice = c;
        }
      }
    }
  }
  shared_rank[g] = choice;
  if (ext) ext[g * (K + 1) + K] = choice >= 0 ? E + choice : -1;
}

}  // namespace uep

using namespace uep;

extern "C" uep_status uep_waterfill(const int32_t* counts, const int32_t* topk_ids,
                                    const int32_t* batch_size, int32_t R, int32_t T, int32_t K,
                                    int32_t E, uint64_t seed, uint64_t layer,
                                    int32_t local_pref_shift, int32_t all_ranks,
                                    int32_t* shared_rank,
                                    int32_t* waterline, int32_t* slack, int32_t* rank_load,
                                    int32_t* ext_topk, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0) return UEP_EINVAL;
  if (R > 64 || E % R != 0 || E > 4096 || K > 64 || local_pref_shift < 0 ||
      local_pref_shift > 8 || (int64_t)R * T * (K + 1) >= (1ll << 31))
    return UEP_EGEOM;
  if (!counts || !batch_size || !waterline || !slack || !rank_load) return UEP_EINVAL;
  if (T > 0 && (!topk_ids || !shared_rank)) return UEP_EINVAL;
  hipStream_t s = uep_stream(stream);
  hipLaunchKernelGGL(wf_prologue, dim3(1), dim3(256), sizeof(int32_t) * E, s, counts, batch_size,
                     R, E, T, waterline, slack, rank_load);
  UEP_CHECK_LAUNCH();
  if (T > 0) {
    const int64_t n = (int64_t)R * T;
    hipLaunchKernelGGL(wf_sample, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, topk_ids,
                       batch_size, slack, rank_load, R, T, K, E, seed, layer, local_pref_shift,
                       all_ranks ? 1 : 0, shared_rank, ext_topk);
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
