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
//   source; in the all-rank mode the running weights are prefix sums of the slack,
//   searched by bisection.  The draw is word 0 of Philox4x64-10 (Salmon et al.,
//   SC'11) at counter (global token index, 0, 0, 0) and key (seed, layer), scaled to
//   the total weight with a 64x64->128-bit multiply, so the choice is exact integer
//   arithmetic.
#include "common.h"
#include "philox.h"

namespace uep {

__global__ __launch_bounds__(256) void wf_prologue(const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ batch_size, int R,
                                                   int E, int T, int32_t* __restrict__ waterline,
                                                   int32_t* __restrict__ slack,
                                                   int32_t* __restrict__ rank_load) {
  extern __shared__ int32_t wf_lds[];   // [E] expert loads
  __shared__ int32_t s_L[64], s_B[64];
  __shared__ int32_t s_H;
  const int E_loc = E / R;
  for (int e = threadIdx.x; e < E; e += blockDim.x) wf_lds[e] = column_sum(counts, R, E, e);
  if (threadIdx.x < R) {
    const int b = batch_size[threadIdx.x];
    s_B[threadIdx.x] = b < 0 ? 0 : (b > T ? T : b);
  }
  __syncthreads();
  if (threadIdx.x < R) {
    int L = 0;
    for (int j = 0; j < E_loc; ++j) L += wf_lds[threadIdx.x * E_loc + j];
    s_L[threadIdx.x] = L;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t tot = 0;
    for (int r = 0; r < R; ++r) tot += (int64_t)s_L[r] + s_B[r];
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

// One workgroup = up to 256 consecutive tokens of rank r0 = blockIdx.y, one thread
// per token.  The block's top-k rows are read coalesced into an LDS tile with K + 1
// columns; the thread's choice fills the extra column and the tile is written back
// coalesced as the fused top-(K+1) rows.  Home ranks come from an LDS table.
template <bool kStage>
__global__ __launch_bounds__(256) void wf_sample(const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ batch_size,
                                                 const int32_t* __restrict__ slack,
                                                 const int32_t* __restrict__ rank_load, int R,
                                                 int T, int K, int E, uint64_t seed,
                                                 uint64_t layer, int shift, int all_ranks,
                                                 int32_t* __restrict__ shared_rank,
                                                 int32_t* __restrict__ ext) {
  __shared__ int32_t s_S[64], s_L[64];
  __shared__ int64_t s_cum[65];           // prefix sums of slack (all-rank mode)
  __shared__ int32_t s_B;
  extern __shared__ int32_t wf_dyn[];     // home[E], then the [256][K+1] tile
  int32_t* home = wf_dyn;
  int32_t* tile = wf_dyn + E;
  const int r0 = blockIdx.y;
  const int t_base = blockIdx.x * 256;
  const int n_tok = min(256, T - t_base);
  const int E_loc = E / R;
  const int K1 = K + 1;
  const int64_t g_base = (int64_t)r0 * T + t_base;
  for (int e = threadIdx.x; e < E; e += 256) home[e] = e / E_loc;
  if (threadIdx.x < R) {
    s_S[threadIdx.x] = slack[threadIdx.x];
    s_L[threadIdx.x] = rank_load[threadIdx.x];
  }
  if (threadIdx.x == 0) s_B = batch_size[r0];
  if (kStage) {
    const int32_t* src = ids + g_base * K;
    for (int j = threadIdx.x; j < n_tok * K; j += 256) {
      const int tt = j / K;
      tile[tt * K1 + (j - tt * K)] = src[j];
    }
  }
  __syncthreads();
  if (all_ranks && threadIdx.x == 0) {
    int64_t c = 0;
    for (int r = 0; r < R; ++r) { s_cum[r] = c; c += s_S[r]; }
    s_cum[R] = c;
  }
  if (all_ranks) __syncthreads();
  const int t = t_base + threadIdx.x;
  if (threadIdx.x < n_tok) {
    const int64_t g = g_base + threadIdx.x;
    int choice = -1;
    uint64_t visited = 0;
    for (int k = 0; k < K; ++k) {
      const int e = kStage ? tile[threadIdx.x * K1 + k] : ids[g * K + k];
      if (!kStage && ext) ext[g * K1 + k] = e;
      if (e >= 0 && e < E) visited |= 1ull << home[e];
    }
    if (t < s_B) {
      const int64_t big = 1ll << shift;
      const int64_t w0 = (big + 1) * s_S[r0];
      if (all_ranks) {
        const int64_t tot = s_cum[R] - s_S[r0];
        const int64_t W = w0 + big * tot;
        if (W > 0) {
          const uint64_t u = philox4x64_10_w0((uint64_t)g, 0, 0, 0, seed, layer);
          const uint64_t v = __umul64hi(u, (uint64_t)W);
          if (v < (uint64_t)w0) {
            choice = r0;
          } else {
            // first c != r0 with big * (slack of ranks <= c, r0 excluded) > v - w0
            const uint64_t vr = v - (uint64_t)w0;
            int lo = 0, hi = R - 1;
            while (lo < hi) {
              const int mid = (lo + hi) / 2;
              const int64_t cm = s_cum[mid + 1] - (r0 <= mid ? s_S[r0] : 0);
              if ((uint64_t)(big * cm) > vr) hi = mid; else lo = mid + 1;
            }
            choice = lo;
          }
        } else {
          choice = r0;
          int64_t bestL = -1;
          const int64_t lr0 = s_L[r0];
          for (int c = 0; c < R; ++c) {
            const int64_t lc = s_L[c];
            if (c != r0 && (big + 1) * lc < big * lr0 && (bestL < 0 || lc < bestL)) {
              bestL = lc;
              choice = c;
            }
          }
        }
      } else {
        visited &= ~(1ull << r0);
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
    }
    shared_rank[g] = choice;
    const int col = choice >= 0 ? E + choice : -1;
    if (kStage) tile[threadIdx.x * K1 + K] = col;
    else if (ext) ext[g * K1 + K] = col;
  }
  if (kStage && ext) {
    __syncthreads();
    // streaming stores (nt sc1), 16-byte vectors when the rows and the tile allow: the
    // next launch reads the fused rows from memory, and the end of this one has no
    // dirty lines to write back
    int32_t* dst = ext + g_base * K1;
    const int n = n_tok * K1;
    const span_t sp = span_of(dst, (int64_t)n * 4);
    int j0 = 0;
    if (((reinterpret_cast<uintptr_t>(dst) | (uintptr_t)E * 4) & 15) == 0) {
      for (int i = threadIdx.x; i < n / 4; i += 256)
        stream_store(*reinterpret_cast<const u32x4*>(tile + 4 * i), sp, 16 * i);
      j0 = n / 4 * 4;
    }
    for (int j = j0 + threadIdx.x; j < n; j += 256) stream_store_b32((uint32_t)tile[j], sp, 4 * j);
  }
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
    const dim3 grid((unsigned)((T + 255) / 256), (unsigned)R);
    const size_t tile = sizeof(int32_t) * (size_t)(E + 256 * (K + 1));
    if (tile <= 48 * 1024)
      hipLaunchKernelGGL(wf_sample<true>, grid, dim3(256), tile, s, topk_ids, batch_size, slack,
                         rank_load, R, T, K, E, seed, layer, local_pref_shift, all_ranks ? 1 : 0,
                         shared_rank, ext_topk);
    else
      hipLaunchKernelGGL(wf_sample<false>, grid, dim3(256), sizeof(int32_t) * E, s, topk_ids,
                         batch_size, slack, rank_load, R, T, K, E, seed, layer, local_pref_shift,
                         all_ranks ? 1 : 0, shared_rank, ext_topk);
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
