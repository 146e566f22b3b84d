// Joint replica placement + quota solve (UltraEP article, section
// "Quota 同时决定专家副本与 token 分流"; constraints of the same section: S slots per
// rank, no expert twice on a rank, minimum quota of a new replica; section
// "共享冗余 slot 管理动态专家副本": mains never move).
//
// Expert loads are summed by the whole workgroup (LDS integer atomics, exact in any
// order); the search is one wave64, lane r = rank r: L_r, free slots and the rank's
// slot table live in registers, per-expert main quotas in LDS.  Each step is a handful of wave
// DPP wave reductions + a ballot (argmax over ranks, argmin over receivers), so the whole
// solve is a strictly sequential loop of at most E + 2R steps with no barrier
// other than the wave itself.
//
// Step rule ("fill to the waterline", T* = ceil(sum_e c_e / R)): h = most loaded
// rank (lowest index on ties); stop if L_h <= T*.  Donors are h's mains with a
// non-zero quota, quota descending then id ascending.  For a donor e: top up the
// least loaded rank (< T*) already holding a replica of e, moving
// min(q_e, L_h - T*, T* - L_j); otherwise open a replica in the lowest free slot of
// the least loaded rank (< T*, free slot, no copy of e) if that move is >= q_min.
// The first donor that can move ends the step; none -> stop.
#include "common.h"

namespace uep {

constexpr int kSqMaxS = 8;
constexpr int kSqThreads = 256;
constexpr int kBig = 0x7fffffff;

__global__ __launch_bounds__(kSqThreads) void solve_quota_kernel(
    const int32_t* __restrict__ counts, int R, int E, int S, int q_min,
    int32_t* __restrict__ slot_expert, int32_t* __restrict__ inst_expert,
    int32_t* __restrict__ inst_quota, int32_t* __restrict__ rank_load,
    int32_t* __restrict__ stats) {
  extern __shared__ int32_t sq_lds[];       // [E] main quotas, starting at the expert loads
  const int tid = threadIdx.x;
  const int E_loc = E / R;
  for (int e = tid; e < E; e += kSqThreads) sq_lds[e] = 0;
  __syncthreads();
  {
    // per = threads per expert; each sums every per-th rank with loads in flight
    const int per = E >= kSqThreads ? 1 : kSqThreads / E;
    const int part = tid % per;
    for (int e = tid / per; e < E; e += kSqThreads / per) {
      int acc[4] = {0, 0, 0, 0};
      int r = part;
      for (; r + 3 * per < R; r += 4 * per) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += counts[(int64_t)(r + u * per) * E + e];
      }
      for (; r < R; r += per) acc[0] += counts[(int64_t)r * E + e];
      atomicAdd(&sq_lds[e], (acc[0] + acc[1]) + (acc[2] + acc[3]));
    }
  }
  __syncthreads();
  if (tid >= kWave) return;                 // the search itself is one wave

  // Only this wave touches the quotas from here on; its LDS accesses execute in
  // program order, so plain loads and stores are enough.
  int32_t* q_main = sq_lds;
  const int lane = tid;
  const bool active = lane < R;
  int L = 0;
  if (active)
    for (int j = 0; j < E_loc; ++j) L += q_main[lane * E_loc + j];
  int sl_e[kSqMaxS], sl_q[kSqMaxS];         // this rank's slots
#pragma unroll
  for (int s = 0; s < kSqMaxS; ++s) { sl_e[s] = -1; sl_q[s] = 0; }
  int free_slots = active ? S : 0;
  const int total = wave_sum(L);
  const int t_star = (total + R - 1) / R;

  int steps = 0, n_rep = 0, stuck = 0;
  for (;;) {
    const int Lh = wave_max(active ? L : INT32_MIN);
    if (Lh <= t_star) break;
    const int h = first_lane(active && L == Lh);
    const int over = Lh - t_star;
    const int qj = lane < E_loc ? q_main[h * E_loc + lane] : 0;
    bool tried = false, moved = false;
    for (;;) {
      // next donor: largest untried main quota on h, lowest expert id on ties
      const int dk = (lane < E_loc && qj > 0 && !tried) ? qj : -1;
      const int qd = wave_max(dk);
      if (qd <= 0) break;
      const int jd = first_lane(dk == qd);
      const int e = h * E_loc + jd;
      int has = -1;
#pragma unroll
      for (int s = 0; s < kSqMaxS; ++s)
        if (s < S && sl_e[s] == e) has = s;
      // top up an existing replica below the waterline
      const bool c1 = active && lane != h && has >= 0 && L < t_star;
      const int kj = wave_min(c1 ? L : kBig);
      if (kj != kBig) {
        const int j = first_lane(c1 && L == kj);
        const int delta = min(qd, min(over, t_star - kj));
        if (lane == j) {
#pragma unroll
          for (int s = 0; s < kSqMaxS; ++s)
            if (s == has) sl_q[s] += delta;
          L += delta;
        }
        if (lane == h) L -= delta;
        if (lane == 0) q_main[e] = qd - delta;
        moved = true;
        break;
      }
      // open a new replica on the least loaded eligible rank
      const bool c2 = active && lane != h && free_slots > 0 && has < 0 && L < t_star;
      const int kt = wave_min(c2 ? L : kBig);
      if (kt != kBig) {
        const int delta = min(qd, min(over, t_star - kt));
        if (delta >= q_min) {
          const int t = first_lane(c2 && L == kt);
          if (lane == t) {
            const int slot = S - free_slots;
#pragma unroll
            for (int s = 0; s < kSqMaxS; ++s)
              if (s == slot) { sl_e[s] = e; sl_q[s] = delta; }
            free_slots -= 1;
            L += delta;
          }
          if (lane == h) L -= delta;
          if (lane == 0) q_main[e] = qd - delta;
          ++n_rep;
          moved = true;
          break;
        }
      }
      if (lane == jd) tried = true;
    }
    if (!moved) { stuck = 1; break; }
    ++steps;
  }

  const int ipr = E_loc + S;
  for (int i = lane; i < R * E_loc; i += kWave) {
    const int r = i / E_loc, j = i % E_loc;
    inst_expert[r * ipr + j] = i;
    inst_quota[r * ipr + j] = q_main[i];
  }
  if (active) {
#pragma unroll
    for (int s = 0; s < kSqMaxS; ++s)
      if (s < S) {
        inst_expert[lane * ipr + E_loc + s] = sl_e[s];
        inst_quota[lane * ipr + E_loc + s] = sl_q[s];
        slot_expert[lane * S + s] = sl_e[s];
      }
    rank_load[lane] = L;
  }
  if (lane == 0) {
    stats[0] = n_rep;
    stats[1] = steps;
    stats[2] = t_star;
    stats[3] = stuck;
  }
}

__global__ void identity_quota_kernel(const int32_t* __restrict__ counts, int R, int E, int n_inst,
                                      const int32_t* __restrict__ inst_expert,
                                      int32_t* __restrict__ inst_quota) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_inst) return;
  const int e = inst_expert[i];
  inst_quota[i] = (e >= 0 && e < E) ? column_sum(counts, R, E, e) : 0;
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
  hipLaunchKernelGGL(solve_quota_kernel, dim3(1), dim3(kSqThreads), lds, uep_stream(stream), counts, R, E,
                     S, q_min, slot_expert, inst_expert, inst_quota, rank_load, stats);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}

extern "C" uep_status uep_identity_quota(const int32_t* counts, int32_t R, int32_t E,
                                         int32_t n_inst, const int32_t* inst_expert,
                                         int32_t* inst_quota, void* stream) {
  if (R <= 0 || E <= 0 || n_inst < 0) return UEP_EINVAL;
  if (n_inst == 0) return UEP_OK;
  if (!counts || !inst_expert || !inst_quota) return UEP_EINVAL;
  hipLaunchKernelGGL(identity_quota_kernel, dim3((n_inst + 255) / 256), dim3(256), 0,
                     uep_stream(stream), counts, R, E, n_inst, inst_expert, inst_quota);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
