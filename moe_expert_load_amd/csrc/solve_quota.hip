// Joint replica placement + quota solve (UltraEP article, section
// "Quota 同时决定专家副本与 token 分流"): the uep_solve_quota entry point, one
// 256-thread workgroup running solve_body (solve_quota.h, where the search and its
// rule are), and the identity quotas of a fixed placement.
#include "solve_quota.h"

namespace uep {

template <int kS>
__global__ __launch_bounds__(kSqThreads) void solve_quota_kernel(
    const int32_t* __restrict__ counts, int R, int E, int S, int q_min,
    int32_t* __restrict__ slot_expert, int32_t* __restrict__ inst_expert,
    int32_t* __restrict__ inst_quota, int32_t* __restrict__ rank_load,
    int32_t* __restrict__ stats) {
  extern __shared__ int32_t sq_lds[];       // [E] main quotas
  solve_body<kS>(counts, R, E, S, q_min, slot_expert, inst_expert, inst_quota, rank_load, stats,
                 sq_lds);
}

// Four lanes per instance (a quad), each summing every fourth rank with its (at most
// 16) loads in flight: one round trip for R <= 64; the quad adds with two DPP steps.
__global__ __launch_bounds__(256) void identity_quota_kernel(const int32_t* __restrict__ counts,
                                                             int R, int E, int n_inst,
                                                             const int32_t* __restrict__ inst_expert,
                                                             int32_t* __restrict__ inst_quota) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = t / 4, part = t % 4;
  const int e = i < n_inst ? inst_expert[i] : -1;
  const bool ok = e >= 0 && e < E;
  int v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)         // clamped address, no branch: every load issues
    v[u] = counts[(int64_t)min(part + 4 * u, R - 1) * E + (ok ? e : 0)];
  int acc = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) acc += ok && part + 4 * u < R ? v[u] : 0;
  // every lane takes part (the grid covers whole quads): quad_perm [1,0,3,2], [2,3,0,1]
  acc += __builtin_amdgcn_mov_dpp(acc, 0xB1, 0xF, 0xF, true);
  acc += __builtin_amdgcn_mov_dpp(acc, 0x4E, 0xF, 0xF, true);
  if (part == 0 && i < n_inst) inst_quota[i] = acc;
}

}  // namespace uep

using namespace uep;

extern "C" uep_status uep_solve_quota(const int32_t* counts, int32_t R, int32_t E, int32_t S,
                                      int32_t q_min, int32_t* slot_expert, int32_t* inst_expert,
                                      int32_t* inst_quota, int32_t* rank_load, int32_t* stats,
                                      void* stream) {
  if (R <= 0 || E <= 0 || S < 0 || q_min < 0) return UEP_EINVAL;
  if (R > 64 || E > 4096 || E % R != 0 || S > kSqMaxS || E / R > 64) return UEP_EGEOM;
  if (!counts || !inst_expert || !inst_quota || !rank_load || !stats || (S > 0 && !slot_expert))
    return UEP_EINVAL;
  const size_t lds = sizeof(int32_t) * E;
  hipStream_t st = uep_stream(stream);
#define UEP_SQ_LAUNCH(KS)                                                                     \
  hipLaunchKernelGGL(solve_quota_kernel<KS>, dim3(1), dim3(kSqThreads), lds, st, counts, R, E, \
                     S, q_min, slot_expert, inst_expert, inst_quota, rank_load, stats)
  if (S <= 1) UEP_SQ_LAUNCH(1);
  else if (S <= 2) UEP_SQ_LAUNCH(2);
  else if (S <= 4) UEP_SQ_LAUNCH(4);
  else UEP_SQ_LAUNCH(8);
#undef UEP_SQ_LAUNCH
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}

extern "C" uep_status uep_identity_quota(const int32_t* counts, int32_t R, int32_t E,
                                         int32_t n_inst, const int32_t* inst_expert,
                                         int32_t* inst_quota, void* stream) {
  if (R <= 0 || E <= 0 || n_inst < 0) return UEP_EINVAL;
  if (R > 64 || n_inst >= (1 << 28)) return UEP_EGEOM;
  if (n_inst == 0) return UEP_OK;
  if (!counts || !inst_expert || !inst_quota) return UEP_EINVAL;
  hipLaunchKernelGGL(identity_quota_kernel, dim3((4 * n_inst + 255) / 256), dim3(256), 0,
                     uep_stream(stream), counts, R, E, n_inst, inst_expert, inst_quota);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
