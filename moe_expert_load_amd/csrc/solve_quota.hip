// Joint replica placement + quota solve (UltraEP article, section
// "Quota 同时决定专家副本与 token 分流"; constraints of the same section: S slots per
// rank, no expert twice on a rank, minimum quota of a new replica; section
// "共享冗余 slot 管理动态专家副本": mains never move).
//
// Expert loads are summed by the whole workgroup (LDS integer atomics, exact in any
// order); the search is one wave64, lane r = rank r: L_r, free slots and the rank's
// slot table live in registers, per-expert main quotas in LDS.  A step is a few DPP
// wave reductions (argmax over ranks, argmax over donors, argmin over receivers), so
// the whole solve is a strictly sequential loop, one replica per step (at most R*S
// steps), with no barrier other than the wave itself.
//
// Step rule ("fill to the waterline", T* = ceil(sum_e c_e / R)): h = most loaded
// rank (lowest index on ties); stop if L_h <= T*.  Donors are h's mains with a
// non-zero quota, quota descending then id ascending.  For a donor e: open a replica
// in the lowest free slot of the least loaded rank t (L_t < T*, a free slot, no copy
// of e), moving min(q_e, L_h - T*, T* - L_t) if that is >= q_min.  The first donor
// that can move ends the step.  None -> a relay (the article's other kind of step,
// an update of the quota distribution): for the donors of h in the same order, the
// first rank x != h (lowest index) with a free slot, no copy of e and L_x >= T* one of
// whose mains f (quota left) has a replica on a rank y with L_y < T*: d2 =
// min(q_f, T* - L_y) moves from x's main to y's replica, and e opens on x with
// d = min(q_e, L_h - T*, T* - (L_x - d2)) if d >= q_min.  No relay -> stop.  No rank
// ever rises above T*, and every step opens a replica (at most R*S steps).
//
// Relay lemma (proved by induction over the steps): a main with quota left has at
// most one replica holder below T*, and a rank that has such a main is at exactly
// T* and holds no replica.  A rank above T* has only ever donated; a replica stays
// below T* with quota left on its main only when the donor came down to exactly T*
// in that step, which happens once per rank; a relay uses that pair up.  So a
// qualifying relay rank has a single (f, y), and the order of its mains, the choice
// among holders of f and the load order among relay ranks decide nothing: the relay
// below takes the one pair it finds and the lowest qualifying index.
#include "common.h"

namespace uep {

constexpr int kSqMaxS = 8;
constexpr int kSqThreads = 256;
constexpr int kBig = 0x7fffffff;
constexpr int kPackBits = 25;               // loads below 2^25 fit a (load, lane) key

// Unsigned wave minimum (same DPP pattern and foldable form as wave_reduce_dpp).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}

// One rank's search state, held by lane r (kS >= S slots in registers).
template <int kS>
struct SqLane {
  int L;                 // current load of the rank
  int sl_e[kS], sl_q[kS];
  int free_slots;
};

template <int kS>
__device__ __forceinline__ int slot_of(const SqLane<kS>& st, int S, int e) {
  int has = -1;
#pragma unroll
  for (int s = 0; s < kS; ++s)
    if (s < S && st.sl_e[s] == e) has = s;
  return has;
}

template <int kS>
__device__ __forceinline__ void open_slot(SqLane<kS>& st, int S, int e, int delta) {
  const int slot = S - st.free_slots;
#pragma unroll
  for (int s = 0; s < kS; ++s)
    if (s == slot) { st.sl_e[s] = e; st.sl_q[s] = delta; }
  st.free_slots -= 1;
}

// Relay step for the stuck heaviest rank h (see the rule above).  by[] (E entries of
// LDS) receives, per expert, (load << 6 | rank) of a replica holder below T*: by the
// relay lemma a main with quota left has at most one, so the entries read below have
// a single writer (entries of emptied mains may have several and are never read).
// A rank x qualifies when it has that pair and the room it frees, T* - (L_x - d2), is
// at least q_min; given a donor whose quota and h's excess are both >= q_min, this
// does not depend on the donor, so every lane finds its pair once, and each donor
// costs one ballot over the candidate ranks.  It fails at once when h's excess is
// below q_min or no lane qualifies, since every donor would then fail.
template <int kS>
__device__ bool sq_relay(SqLane<kS>& st, int32_t* q_main, uint64_t* by, int lane, bool active,
                         int E, int E_loc, int S, int q_min, int t_star, int h, int Lh,
                         int& n_rep) {
  if (Lh - t_star < q_min) return false;
  for (int e = lane; e < E; e += kWave) by[e] = ~0ull;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (active && st.L < t_star) {
#pragma unroll
    for (int s = 0; s < kS; ++s)
      if (s < S && st.sl_e[s] >= 0) by[st.sl_e[s]] = ((uint64_t)st.L << 6) | (uint64_t)lane;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // this lane as the relay rank x: its main with quota left and a holder below T*
  int bf = -1, by_l = 0, bd2 = 0, room = 0;
  if (active && lane != h && st.free_slots > 0 && st.L >= t_star) {
    for (int j0 = 0; j0 < E_loc; j0 += 8) {
      int qf[8];
      uint64_t key[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {        // the batch's loads first, then the test
        const int f = lane * E_loc + min(j0 + u, E_loc - 1);
        qf[u] = q_main[f];
        key[u] = by[f];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= E_loc || qf[u] <= 0 || key[u] == ~0ull) continue;
        const int d2 = min(qf[u], t_star - (int)(key[u] >> 6));
        if (t_star - (st.L - d2) < q_min) continue;
        bf = lane * E_loc + j0 + u; by_l = (int)(key[u] & 63u); bd2 = d2;
        room = t_star - (st.L - d2);
      }
    }
  }
  if (ballot(bf >= 0) == 0) return false;
  const int qj = lane < E_loc ? q_main[h * E_loc + lane] : 0;
  bool tried = false;
  for (;;) {
    // donors of h in donor order: largest untried main quota, lowest expert id on ties;
    // the quotas only fall from here, so one below q_min ends the relay
    const int qd = wave_max((lane < E_loc && qj > 0 && !tried) ? qj : 0);
    if (qd <= 0 || qd < q_min) return false;
    const int jd = first_lane(lane < E_loc && qj == qd && !tried);
    const int e = h * E_loc + jd;
    const int x = first_lane(bf >= 0 && slot_of<kS>(st, S, e) < 0);
    if (x >= 0) {
      const int f = readlane(bf, x), y = readlane(by_l, x), d2 = readlane(bd2, x);
      const int d = min(qd, min(Lh - t_star, readlane(room, x)));
      if (lane == y) {
#pragma unroll
        for (int s = 0; s < kS; ++s)
          if (s < S && st.sl_e[s] == f) st.sl_q[s] += d2;
        st.L += d2;
      }
      if (lane == x) { open_slot<kS>(st, S, e, d); st.L += d - d2; }
      if (lane == h) st.L -= d;
      if (lane == 0) { q_main[e] -= d; q_main[f] -= d2; }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      ++n_rep;
      return true;
    }
    if (lane == jd) tried = true;
  }
}

// The search with packed keys (every load < 2^25): (load << 6 | lane) makes one
// reduction give value and lowest lane together.
template <int kS>
__device__ __forceinline__ void search_packed(SqLane<kS>& st, int32_t* q_main, uint64_t* by, int lane, bool active,
                                              int R, int E_loc, int S, int q_min, int t_star,
                                              int& steps, int& n_rep, int& stuck) {
  for (;;) {
    const int kh = wave_max(active ? (st.L << 6) | (63 - lane) : -1);
    const int Lh = kh >> 6;
    if (Lh <= t_star) break;
    const int h = 63 - (kh & 63);
    const int over = Lh - t_star;
    // every move, plain or relay, is at most the excess: below q_min nothing can move
    if (over < q_min) { stuck = 1; break; }
    const int qj = lane < E_loc ? q_main[h * E_loc + lane] : 0;
    bool tried = false, moved = false;
    // no rank below T* with a free slot: no donor can move directly, go to the relay
    const bool any_recv = ballot(active && lane != h && st.L < t_star && st.free_slots > 0) != 0;
    for (; any_recv;) {
      // next donor: largest untried main quota on h, lowest expert id on ties; the
      // quotas only fall from here, so one below q_min ends the scan
      const int kd = wave_max((lane < E_loc && qj > 0 && !tried) ? (qj << 6) | (63 - lane) : -1);
      if (kd < 0 || (kd >> 6) < q_min) break;
      const int qd = kd >> 6, jd = 63 - (kd & 63);
      const int e = h * E_loc + jd;
      const bool c2 = active && lane != h && st.L < t_star && st.free_slots > 0 &&
                      slot_of<kS>(st, S, e) < 0;
      const uint32_t km = wave_min_u32(c2 ? ((uint32_t)st.L << 6) | (uint32_t)lane : 0xFFFFFFFFu);
      if (km != 0xFFFFFFFFu) {
        const int tgt = (int)(km & 63u);
        const int Lt = (int)(km >> 6);
        const int delta = min(qd, min(over, t_star - Lt));
        if (delta >= q_min) {                         // open a new replica
          if (lane == tgt) { open_slot<kS>(st, S, e, delta); st.L += delta; }
          if (lane == h) st.L -= delta;
          if (lane == 0) q_main[e] = qd - delta;
          ++n_rep;
          moved = true;
          break;
        }
      }
      if (lane == jd) tried = true;
    }
    if (!moved)
      moved = sq_relay<kS>(st, q_main, by, lane, active, R * E_loc, E_loc, S, q_min, t_star,
                                 h, Lh, n_rep);
    if (!moved) { stuck = 1; break; }
    ++steps;
  }
}

// The same rule for any load below 2^31: value reductions, then ballots.
template <int kS>
__device__ __forceinline__ void search_wide(SqLane<kS>& st, int32_t* q_main, uint64_t* by, int lane, bool active,
                                            int R, int E_loc, int S, int q_min, int t_star,
                                            int& steps, int& n_rep, int& stuck) {
  for (;;) {
    const int Lh = wave_max(active ? st.L : INT32_MIN);
    if (Lh <= t_star) break;
    const int h = first_lane(active && st.L == Lh);
    const int over = Lh - t_star;
    if (over < q_min) { stuck = 1; break; }
    const int qj = lane < E_loc ? q_main[h * E_loc + lane] : 0;
    bool tried = false, moved = false;
    const bool any_recv = ballot(active && lane != h && st.L < t_star && st.free_slots > 0) != 0;
    for (; any_recv;) {
      const int dk = (lane < E_loc && qj > 0 && !tried) ? qj : -1;
      const int qd = wave_max(dk);
      if (qd <= 0 || qd < q_min) break;
      const int jd = first_lane(dk == qd);
      const int e = h * E_loc + jd;
      const bool c2 = active && lane != h && st.free_slots > 0 && st.L < t_star &&
                      slot_of<kS>(st, S, e) < 0;
      const int kt = wave_min(c2 ? st.L : kBig);
      if (kt != kBig) {
        const int delta = min(qd, min(over, t_star - kt));
        if (delta >= q_min) {
          const int t = first_lane(c2 && st.L == kt);
          if (lane == t) { open_slot<kS>(st, S, e, delta); st.L += delta; }
          if (lane == h) st.L -= delta;
          if (lane == 0) q_main[e] = qd - delta;
          ++n_rep;
          moved = true;
          break;
        }
      }
      if (lane == jd) tried = true;
    }
    if (!moved)
      moved = sq_relay<kS>(st, q_main, by, lane, active, R * E_loc, E_loc, S, q_min, t_star,
                                  h, Lh, n_rep);
    if (!moved) { stuck = 1; break; }
    ++steps;
  }
}

template <int kS>
__global__ __launch_bounds__(kSqThreads) void solve_quota_kernel(
    const int32_t* __restrict__ counts, int R, int E, int S, int q_min,
    int32_t* __restrict__ slot_expert, int32_t* __restrict__ inst_expert,
    int32_t* __restrict__ inst_quota, int32_t* __restrict__ rank_load,
    int32_t* __restrict__ stats) {
  extern __shared__ uint64_t sq_lds64[];    // [E] relay table, then [E] main quotas
  uint64_t* by = sq_lds64;
  int32_t* sq_lds = reinterpret_cast<int32_t*>(sq_lds64 + E);
  const int tid = threadIdx.x;
  const int E_loc = E / R;
  for (int e = tid; e < E; e += kSqThreads) sq_lds[e] = 0;
  __syncthreads();
  {
    // per = threads per expert; each sums every per-th rank, up to 16 predicated
    // loads in flight (one round whenever R <= 16 * per)
    const int per = E >= kSqThreads ? 1 : kSqThreads / E;
    const int part = tid % per;
    for (int e = tid / per; e < E; e += kSqThreads / per) {
      int acc = 0;
      for (int r0 = part; r0 < R; r0 += 16 * per) {
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)     // clamped address, no branch: every load issues
          v[u] = counts[(int64_t)min(r0 + u * per, R - 1) * E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += r0 + u * per < R ? v[u] : 0;
      }
      atomicAdd(&sq_lds[e], acc);
    }
  }
  __syncthreads();
  if (tid >= kWave) return;                 // the search itself is one wave

  // Only this wave touches the quotas from here on; its LDS accesses execute in
  // program order, so plain loads and stores are enough.
  int32_t* q_main = sq_lds;
  const int lane = tid;
  const bool active = lane < R;
  SqLane<kS> st;
  st.L = 0;
  if (active)
    for (int j = 0; j < E_loc; ++j) st.L += q_main[lane * E_loc + j];
#pragma unroll
  for (int s = 0; s < kS; ++s) { st.sl_e[s] = -1; st.sl_q[s] = 0; }
  st.free_slots = active ? S : 0;
  const int total = wave_sum(st.L);
  const int t_star = (total + R - 1) / R;

  int steps = 0, n_rep = 0, stuck = 0;
  if (total < (1 << kPackBits))
    search_packed<kS>(st, q_main, by, lane, active, R, E_loc, S, q_min, t_star, steps, n_rep, stuck);
  else
    search_wide<kS>(st, q_main, by, lane, active, R, E_loc, S, q_min, t_star, steps, n_rep, stuck);

  const int ipr = E_loc + S;
  for (int i = lane; i < R * E_loc; i += kWave) {
    const int r = i / E_loc, j = i % E_loc;
    inst_expert[r * ipr + j] = i;
    inst_quota[r * ipr + j] = q_main[i];
  }
  if (active) {
#pragma unroll
    for (int s = 0; s < kS; ++s)
      if (s < S) {
        inst_expert[lane * ipr + E_loc + s] = st.sl_e[s];
        inst_quota[lane * ipr + E_loc + s] = st.sl_q[s];
        slot_expert[lane * S + s] = st.sl_e[s];
      }
    rank_load[lane] = st.L;
  }
  if (lane == 0) {
    stats[0] = n_rep;
    stats[1] = steps;
    stats[2] = t_star;
    stats[3] = stuck;
  }
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
  const size_t lds = (sizeof(uint64_t) + sizeof(int32_t)) * E;
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
