// Joint replica placement + quota solve (UltraEP article, section
// "Quota 同时决定专家副本与 token 分流"; constraints of the same section: S slots per
// rank, no expert twice on a rank, minimum quota of a new replica; section
// "共享冗余 slot 管理动态专家副本": mains never move).
//
// One wave64, lane r = rank r.  L_r and free slots live in registers, per-expert
// main quotas and the slot table in LDS.  Each step is a handful of wave
// reductions (argmax over ranks, argmin over candidate receivers), so the whole
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
constexpr int kBig = 0x7fffffff;

__global__ __launch_bounds__(64) void solve_quota_kernel(const int32_t* __restrict__ counts, int R,
                                                         int E, int S, int q_min,
                                                         int32_t* __restrict__ slot_expert,
                                                         int32_t* __restrict__ inst_expert,
                                                         int32_t* __restrict__ inst_quota,
                                                         int32_t* __restrict__ rank_load,
                                                         int32_t* __restrict__ stats) {
  extern __shared__ int32_t sq_lds[];
  int32_t* q_main = sq_lds;                 // [E]
  int32_t* slot_e = q_main + E;             // [R][S]
  int32_t* slot_q = slot_e + R * kSqMaxS;   // [R][S]
  const int lane = threadIdx.x;
  const int E_loc = E / R;

  for (int e = lane; e < E; e += kWave) {
    int c = 0;
    for (int r = 0; r < R; ++r) c += counts[(int64_t)r * E + e];
    q_main[e] = c;
  }
  for (int i = lane; i < R * kSqMaxS; i += kWave) { slot_e[i] = -1; slot_q[i] = 0; }
  __syncthreads();

  const bool active = lane < R;
  int L = 0;
  if (active)
    for (int j = 0; j < E_loc; ++j) L += q_main[lane * E_loc + j];
  int free_slots = active ? S : 0;
  const int total = wave_sum(L);
  const int t_star = (total + R - 1) / R;

  int steps = 0, n_rep = 0, stuck = 0;
  for (;;) {
    int Lh = active ? L : -1, h = active ? lane : kBig;
    wave_argmax(Lh, h);
    if (Lh <= t_star) break;
    const int over = Lh - t_star;
    // donor order among h's mains: quota descending, expert id ascending
    int my_q = -1, my_e = -1, my_ord = kBig;
    if (lane < E_loc) {
      my_e = h * E_loc + lane;
      my_q = q_main[my_e];
    }
    if (lane < E_loc && my_q > 0) {
      int ord = 0;
      for (int j = 0; j < E_loc; ++j) {
        const int qj = q_main[h * E_loc + j];
        ord += (qj > my_q) || (qj == my_q && j < lane);
      }
      my_ord = ord;
    }
    const int n_donor = __popcll(ballot(lane < E_loc && my_q > 0));
    bool moved = false;
    for (int d = 0; d < n_donor && !moved; ++d) {
      const uint64_t who = ballot(my_ord == d);
      const int src = __ffsll((unsigned long long)who) - 1;
      const int e = readlane(my_e, src);
      const int qe = readlane(my_q, src);
      // does this rank hold a replica of e, and in which slot?
      int has = -1;
      if (active)
        for (int s = 0; s < S; ++s)
          if (slot_e[lane * kSqMaxS + s] == e) has = s;
      // top-up an existing replica below the waterline
      int kj = (active && lane != h && has >= 0 && L < t_star) ? L : kBig;
      int j = (kj == kBig) ? kBig : lane;
      wave_argmin(kj, j);
      if (j != kBig) {
        const int delta = min(qe, min(over, t_star - kj));
        if (lane == j) {
          slot_q[lane * kSqMaxS + has] += delta;
          L += delta;
        }
        if (lane == h) L -= delta;
        if (lane == 0) q_main[e] = qe - delta;
        moved = true;
        break;
      }
      // open a new replica on the least loaded eligible rank
      int kt = (active && lane != h && free_slots > 0 && has < 0 && L < t_star) ? L : kBig;
      int t = (kt == kBig) ? kBig : lane;
      wave_argmin(kt, t);
      if (t != kBig) {
        const int delta = min(qe, min(over, t_star - kt));
        if (delta >= q_min) {
          if (lane == t) {
            const int s = S - free_slots;
            slot_e[lane * kSqMaxS + s] = e;
            slot_q[lane * kSqMaxS + s] = delta;
            free_slots -= 1;
            L += delta;
          }
          if (lane == h) L -= delta;
          if (lane == 0) q_main[e] = qe - delta;
          ++n_rep;
          moved = true;
        }
      }
    }
    __syncthreads();
    if (!moved) { stuck = 1; break; }
    ++steps;
  }
  __syncthreads();

  const int ipr = E_loc + S;
  for (int i = lane; i < R * ipr; i += kWave) {
    const int r = i / ipr, j = i % ipr;
    if (j < E_loc) {
      inst_expert[i] = r * E_loc + j;
      inst_quota[i] = q_main[r * E_loc + j];
    } else {
      inst_expert[i] = slot_e[r * kSqMaxS + (j - E_loc)];
      inst_quota[i] = slot_q[r * kSqMaxS + (j - E_loc)];
    }
  }
  for (int i = lane; i < R * S; i += kWave) slot_expert[i] = slot_e[(i / S) * kSqMaxS + i % S];
  if (active) rank_load[lane] = L;
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
  int q = 0;
  if (e >= 0 && e < E)
    for (int r = 0; r < R; ++r) q += counts[(int64_t)r * E + e];
  inst_quota[i] = q;
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
  const size_t lds = sizeof(int32_t) * (E + 2 * R * kSqMaxS);
  hipLaunchKernelGGL(solve_quota_kernel, dim3(1), dim3(64), lds, uep_stream(stream), counts, R, E,
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
