// Device side of the joint replica placement and quota solve, shared by
// solve_quota.hip (uep_solve_quota) and load_matrix.hip (the fused plan call).
//
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
#pragma once

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
  int pf, py;            // the rank's live pair: its main pf has a replica on lane py
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

// Relay step for the stuck heaviest rank h (see the rule above).  By the relay lemma a
// qualifying relay rank x has exactly one (main f, holder y below T*) pair, the one it
// gained when it came down to T* as a donor, so each lane records that pair then
// (SqLane::pf / py) and the relay only checks it is still live (f's main has quota
// left, y is still below T*) instead of searching x's mains and f's holders.  A rank
// qualifies when it has that pair and the room it frees, T* - (L_x - d2), is at least
// q_min; given a donor whose quota and h's excess are both >= q_min, this does not
// depend on the donor (a relay rank holds no replica, so it never holds the donor), so
// every lane decides once, and each donor costs one ballot over the candidate ranks.
// It fails at once when h's excess is below q_min or no lane qualifies.
template <int kS>
__device__ bool sq_relay(SqLane<kS>& st, int32_t* q_main, int lane, bool active, int E_loc,
                         int S, int q_min, int t_star, int h, int Lh, int& n_rep) {
  if (Lh - t_star < q_min) return false;
  // this lane as the relay rank x: its recorded pair, if still live
  const int Ly = shfl(st.L, st.pf >= 0 ? st.py : lane);
  int bf = -1, by_l = 0, bd2 = 0, room = 0;
  if (active && lane != h && st.free_slots > 0 && st.L >= t_star && st.pf >= 0 && Ly < t_star) {
    const int qf = q_main[st.pf];
    const int d2 = min(qf, t_star - Ly);
    if (qf > 0 && t_star - (st.L - d2) >= q_min) {
      bf = st.pf; by_l = st.py; bd2 = d2;
      room = t_star - (st.L - d2);
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
      if (lane == x) { open_slot<kS>(st, S, e, d); st.L += d - d2; st.pf = -1; }
      if (lane == h) {
        st.L -= d;
        // h down to T* with x left below it and quota left on e: h's pair
        if (d == Lh - t_star && d < d2 && qd - d > 0) { st.pf = e; st.py = x; }
      }
      if (lane == 0) { q_main[e] -= d; q_main[f] -= d2; }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      ++n_rep;
      return true;
    }
    if (lane == jd) tried = true;
  }
}

// Donor key of main j with quota q: (q << 6 | 63 - j) when q > 0, else ~j.  The keys of
// one rank are distinct, order its mains by quota descending then index ascending, and
// 63 - (key & 63) gives j back in both forms; key >> 6 is q, or -1 when q is 0.  The
// fast search keeps each rank's keys sorted in that order, so the first donor is the
// first key.
__device__ __forceinline__ int donor_key(int q, int j) { return q > 0 ? (q << 6) | (63 - j) : ~j; }

__device__ __forceinline__ int key_main(int k) { return 63 - (k & 63); }

// Odd-even transposition sort, descending (kQ rounds sort kQ keys).
template <int kQ>
__device__ __forceinline__ void sort_keys(int (&k)[kQ]) {
#pragma unroll
  for (int r = 0; r < kQ; ++r)
#pragma unroll
    for (int j = r & 1; j + 1 < kQ; j += 2) {
      const int a = max(k[j], k[j + 1]), b = min(k[j], k[j + 1]);
      k[j] = a;
      k[j + 1] = b;
    }
}

// Sorted keys with the first one replaced by x <= k[0]: entry j of the merge of
// k[1..kQ-1] with x is the median of k[j], k[j + 1] and x (the last is min(k[kQ-1], x)).
// With x = k[0] the keys stay as they are, so every lane runs it.
__device__ __forceinline__ int med3_i32(int a, int b, int c) {
  int r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int kQ>
__device__ __forceinline__ void replace_first_key(int (&k)[kQ], int x) {
#pragma unroll
  for (int j = 0; j + 1 < kQ; ++j) k[j] = med3_i32(k[j], k[j + 1], x);
  k[kQ - 1] = min(k[kQ - 1], x);
}

// One pass of compare-exchanges down the keys: puts back in order a sorted set of keys
// in which one key has decreased.
template <int kQ>
__device__ __forceinline__ void sink_key(int (&k)[kQ]) {
#pragma unroll
  for (int j = 0; j + 1 < kQ; ++j) {
    const int a = max(k[j], k[j + 1]), b = min(k[j], k[j + 1]);
    k[j] = a;
    k[j + 1] = b;
  }
}

// Relay on the register keys of the fast search below (the rule of sq_relay; lanes as
// there).  kd is h's first donor key; the caller has checked h's excess against q_min.
// By the relay lemma a qualifying relay rank holds no replica, so it never holds h's
// first donor and the first donor always finds x; should no qualifying rank be free of
// that donor all the same, the general relay decides (returns -1).  Each lane reads the
// quota of its own pair main f from its keys, and every update is a select on the
// registers only (the caller writes the quotas to LDS when it needs them there).
// Returns 1 for a move, 0 for none.
template <int kS, int kQ>
__device__ __forceinline__ int sq_relay_keys(SqLane<kS>& st, int (&kq)[kQ], int lane,
                                             bool active, int E_loc, int S,
                                             int q_min, int t_star, int h, int Lh, int kd,
                                             int& n_rep) {
  // no donor of at least q_min on h: nothing can move
  if (kd < 0 || (kd >> 6) < q_min) return 0;
  const int qd = kd >> 6, jd = key_main(kd);
  const int e = h * E_loc + jd;
  // this lane as the relay rank x: its recorded pair, if still live
  const int Ly = shfl(st.L, st.pf >= 0 ? st.py : lane);
  const int jf = st.pf - lane * E_loc;      // the pair's main among the lane's own mains
  int kf = -1;
#pragma unroll
  for (int j = 0; j < kQ; ++j) kf = key_main(kq[j]) == jf ? kq[j] : kf;
  const int qf = kf >= 0 ? kf >> 6 : 0;
  const int d2 = min(qf, t_star - Ly);
  const bool cand = active && lane != h && st.free_slots > 0 && st.L >= t_star && st.pf >= 0 &&
                    Ly < t_star && qf > 0 && t_star - (st.L - d2) >= q_min;
  bool copy = false;
#pragma unroll
  for (int s = 0; s < kS; ++s) copy |= st.sl_e[s] == e;
  const uint64_t any = ballot(cand), free_of_e = ballot(cand && !copy);
  if (free_of_e == 0) return any ? -1 : 0;
  const int x = __ffsll((unsigned long long)free_of_e) - 1;
  const int f = readlane(st.pf, x), y = readlane(st.py, x), d2x = readlane(d2, x);
  const int Lx = readlane(st.L, x), Lyx = readlane(Ly, x);
  const int d = min(qd, min(Lh - t_star, t_star - (Lx - d2x)));
  const bool is_y = lane == y, is_x = lane == x, is_h = lane == h;
  if (kS == 1) {            // x's only slot is free
    st.sl_q[0] = is_x ? d : ((is_y && st.sl_e[0] == f) ? st.sl_q[0] + d2x : st.sl_q[0]);
    st.sl_e[0] = is_x ? e : st.sl_e[0];
  } else {
    const int slot = S - st.free_slots;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const bool here = is_x && s == slot;
      st.sl_q[s] += (is_y && s < S && st.sl_e[s] == f) ? d2x : 0;
      st.sl_e[s] = here ? e : st.sl_e[s];
      st.sl_q[s] = here ? d : st.sl_q[s];
    }
  }
  st.free_slots -= is_x ? 1 : 0;
  // the three new loads are uniform; one select each (the lanes differ)
  const int nLy = Lyx + d2x, nLx = Lx + d - d2x, nLh = Lh - d;
  int L = st.L;
  L = is_h ? nLh : L;
  L = is_x ? nLx : L;
  L = is_y ? nLy : L;
  st.L = L;
  // h down to T* with x left below it and quota left on e: h's pair; x's pair is used up
  const bool rec = is_h && d == Lh - t_star && d < d2x && qd - d > 0;
  st.pf = rec ? e : (is_x ? -1 : st.pf);
  st.py = rec ? x : st.py;
  // h's first donor and x's pair main lose quota: each lane changes at most one key,
  // which only falls, so one pass down puts the keys back in order
  const int ke = donor_key(qd - d, jd);                 // uniform
  const int kfn = donor_key(qf - d2, jf);               // this lane's, used on x
  int old = kf, knew = kf;                              // other lanes: no change
  old = is_h ? kq[0] : old;
  knew = is_h ? ke : knew;
  knew = is_x ? kfn : knew;
#pragma unroll
  for (int j = 0; j < kQ; ++j) kq[j] = kq[j] == old ? knew : kq[j];
  sink_key<kQ>(kq);
  ++n_rep;
  return 1;
}

// The two reductions of a search step at once, every lane active, results uniform:
// max of kh and unsigned min of kr.  DPP within each row of 16 lanes, then gfx950's row
// swaps (permlane16_swap pairs rows 0-1 and 2-3 of its operands, permlane32_swap the
// halves), so the last steps stay in VALU and one readfirstlane ends each; the two
// chains are interleaved so neither waits on its own DPP hazards.
// kHalf (R <= 32: lanes 32..63 hold no rank): the halves need no exchange, and lane 0
// already holds both results after the row swap.
template <bool kHalf>
__device__ __forceinline__ void wave_max_min_sw(int& kh, uint32_t& kr) {
  int a = kh;
  uint32_t b = kr;
  a = max(a, __builtin_amdgcn_mov_dpp(a, 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
  b = min(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, true));
  a = max(a, __builtin_amdgcn_mov_dpp(a, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
  b = min(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xF, 0xF, true));
  a = max(a, __builtin_amdgcn_mov_dpp(a, 0x124, 0xF, 0xF, true));   // row_ror:4
  b = min(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x124, 0xF, 0xF, true));
  a = max(a, __builtin_amdgcn_mov_dpp(a, 0x128, 0xF, 0xF, true));   // row_ror:8
  b = min(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x128, 0xF, 0xF, true));
  const auto a16 = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const auto b16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  a = max((int)a16[0], (int)a16[1]);
  b = min((uint32_t)b16[0], (uint32_t)b16[1]);
  if (kHalf) {
    kh = __builtin_amdgcn_readfirstlane(a);
    kr = (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
    return;
  }
  const auto a32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const auto b32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  kh = __builtin_amdgcn_readfirstlane(max((int)a32[0], (int)a32[1]));
  kr = (uint32_t)__builtin_amdgcn_readfirstlane((int)min((uint32_t)b32[0], (uint32_t)b32[1]));
}

// The search with packed keys (every load < 2^25): (load << 6 | lane) makes one
// reduction give value and lowest lane together.
//
// Fast steps (kQ > 0, E_loc <= kQ): lane r also holds, in registers, the donor keys of
// its mains (donor_key), sorted, so the first is the rank's first donor (largest quota,
// lowest index on ties) and h's first donor is one readlane; a step changes one key of
// h, its first, which only falls, and one median per key puts it back in order.  On
// R <= 32 ranks the reductions stay in the lower half of the wave.  The lightest possible receiver (L < T*, a free slot; such a rank is never
// h) depends neither on h nor on the donor, so its reduction runs beside h's.  A plain
// step is then decided without a scan: if that receiver holds no copy of the first
// donor, it is the rule's receiver for that donor, and it moves
// delta = min(q, L_h - T*, T* - L_t) if that is at least q_min (no first donor gives
// q = -1, no receiver a negative room: both fail that test).  Every per-lane update is a
// select: one wave runs the whole chain, and a taken branch costs it more than the work
// it would skip.  If the receiver's room or the first donor's quota is below q_min, no
// donor can move at all (every receiver has at most that room, every donor at most that
// quota) and the step is a relay, also on the keys.  Only when that receiver holds a
// copy of the first donor (or the lemma's premise failed) does the step take the donor
// scan or the general relay, on the quotas written back to LDS, and reload the keys
// after.  The quotas are written back to LDS at the end for the outputs.
template <int kS, int kQ, bool kHalf>
__device__ __forceinline__ void search_packed(SqLane<kS>& st, int32_t* q_main, int lane, bool active,
                                              int R, int E_loc, int S, int q_min, int t_star,
                                              int& steps, int& n_rep, int& stuck) {
  constexpr int kQn = kQ > 0 ? kQ : 1;
  int kq[kQn];                       // donor keys of the own mains, sorted (fast steps only);
                                     // kq[0] is the rank's first donor
  int nrep = 0;                      // replicas opened = steps taken (every step opens one)
  auto load_q = [&]() {              // clamped addresses: every read issues, no branch
    const int r = min(lane, R - 1);
#pragma unroll
    for (int j = 0; j < kQn; ++j) {
      const int v = q_main[r * E_loc + min(j, E_loc - 1)];
      kq[j] = donor_key(active && j < E_loc ? v : 0, j);
    }
    sort_keys<kQn>(kq);
  };
  auto store_q = [&]() {
    if (active) {
#pragma unroll
      for (int j = 0; j < kQn; ++j) {
        const int jj = key_main(kq[j]);
        if (jj < E_loc) q_main[lane * E_loc + jj] = kq[j] >= 0 ? kq[j] >> 6 : 0;
      }
    }
  };
  if (kQ > 0) load_q();
  for (;;) {
    int kh = active ? (st.L << 6) | (63 - lane) : -1;
    uint32_t kr = active && st.L < t_star && st.free_slots > 0
                      ? ((uint32_t)st.L << 6) | (uint32_t)lane : 0xFFFFFFFFu;
    wave_max_min_sw<kHalf>(kh, kr);
    const int Lh = kh >> 6;
    if (Lh <= t_star) break;
    const int h = 63 - (kh & 63);
    const int over = Lh - t_star;
    const int Lt = (int)(kr >> 6), tgt = (int)(kr & 63u);
    if (kQ > 0) {
      const int kd = readlane(kq[0], h);
      const int qd = kd >> 6, jd = 63 - (kd & 63);
      const int e = h * E_loc + jd;
      const int room = min(qd, t_star - Lt);
      const int delta = min(over, room);
      // does the receiver hold a copy of e?  Not with one slot per rank: its only slot is
      // free, and e's main is on h.  (Slots past S hold -1, never an expert.)
      bool held = false;
      if (kS > 1) {
        bool any = false;
#pragma unroll
        for (int s = 0; s < kS; ++s) any |= st.sl_e[s] == e;
        held = ((ballot(any) >> tgt) & 1ull) != 0;
      }
      if (__builtin_expect(delta >= q_min && !held, 1)) {
        const bool is_t = lane == tgt, is_h = lane == h;
        if (kS == 1) {          // the receiver's only slot is free
          st.sl_e[0] = is_t ? e : st.sl_e[0];
          st.sl_q[0] = is_t ? delta : st.sl_q[0];
        } else {
          const int slot = S - st.free_slots;
#pragma unroll
          for (int s = 0; s < kS; ++s) {
            const bool here = is_t && s == slot;
            st.sl_e[s] = here ? e : st.sl_e[s];
            st.sl_q[s] = here ? delta : st.sl_q[s];
          }
        }
        st.free_slots -= is_t ? 1 : 0;
        st.L = is_t ? Lt + delta : (is_h ? Lh - delta : st.L);
        // h down to T* (delta = over) with the receiver left below it and quota left on
        // e (delta below both the room and the quota): h's pair
        const bool rec = is_h && over < room;
        st.pf = rec ? e : st.pf;
        st.py = rec ? tgt : st.py;
        // h's first donor (its first key) gets the quota left, the other lanes keep theirs
        replace_first_key<kQn>(kq, is_h ? donor_key(qd - delta, jd) : kq[0]);
        ++nrep;
        continue;
      }
    }
    // every move, plain or relay, is at most the excess: below q_min nothing can move
    if (over < q_min) { stuck = 1; break; }
    // no rank below T* with a free slot: no donor can move directly, go to the relay
    bool plain = kr != 0xFFFFFFFFu;
    if (kQ > 0) {
      const int kd = readlane(kq[0], h);
      if (kd < 0 || (kd >> 6) < q_min || t_star - Lt < q_min) plain = false;
      if (!plain) {
        const int rk = sq_relay_keys<kS, kQn>(st, kq, lane, active, E_loc, S, q_min, t_star,
                                              h, Lh, kd, nrep);
        if (rk == 0) { stuck = 1; break; }
        if (rk > 0) continue;
      }
      store_q();
    }
    const int qj = plain && lane < E_loc ? q_main[h * E_loc + lane] : 0;
    bool tried = false, moved = false;
    for (; plain;) {
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
        const int tgt2 = (int)(km & 63u);
        const int Lt2 = (int)(km >> 6);
        const int delta = min(qd, min(over, t_star - Lt2));
        if (delta >= q_min) {                         // open a new replica
          if (lane == tgt2) { open_slot<kS>(st, S, e, delta); st.L += delta; }
          if (lane == h) {
            st.L -= delta;
            // h down to T* with the receiver left below it and quota left on e
            if (delta == over && Lt2 + delta < t_star && qd - delta > 0) { st.pf = e; st.py = tgt2; }
          }
          if (lane == 0) q_main[e] = qd - delta;
          ++nrep;
          moved = true;
          break;
        }
      }
      if (lane == jd) tried = true;
    }
    if (!moved)
      moved = sq_relay<kS>(st, q_main, lane, active, E_loc, S, q_min, t_star, h, Lh, nrep);
    if (!moved) { stuck = 1; break; }
    if (kQ > 0) load_q();
  }
  if (kQ > 0) store_q();
  n_rep += nrep;
  steps += nrep;
}

// The same rule for any load below 2^31: value reductions, then ballots.
template <int kS>
__device__ __forceinline__ void search_wide(SqLane<kS>& st, int32_t* q_main, int lane, bool active,
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
          if (lane == h) {
            st.L -= delta;
            if (delta == over && kt + delta < t_star && qd - delta > 0) { st.pf = e; st.py = t; }
          }
          if (lane == 0) q_main[e] = qd - delta;
          ++n_rep;
          moved = true;
          break;
        }
      }
      if (lane == jd) tried = true;
    }
    if (!moved)
      moved = sq_relay<kS>(st, q_main, lane, active, E_loc, S, q_min, t_star, h, Lh, n_rep);
    if (!moved) { stuck = 1; break; }
    ++steps;
  }
}

// The whole solve for one 256-thread workgroup: column sums by every thread, then the
// search by wave 0.  sq_lds holds E ints of LDS.  Shared by solve_quota_kernel and the
// fused plan kernel, which runs it in its block 0.
template <int kS>
__device__ __forceinline__ void solve_body(const int32_t* __restrict__ counts, int R, int E, int S,
                                           int q_min, int32_t* __restrict__ slot_expert,
                                           int32_t* __restrict__ inst_expert,
                                           int32_t* __restrict__ inst_quota,
                                           int32_t* __restrict__ rank_load,
                                           int32_t* __restrict__ stats, int32_t* sq_lds) {
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
  st.pf = -1;
  st.py = 0;
  const int total = wave_sum(st.L);
  const int t_star = (total + R - 1) / R;

  int steps = 0, n_rep = 0, stuck = 0;
#define UEP_SQ_PACKED(KQ, HALF) \
  search_packed<kS, KQ, HALF>(st, q_main, lane, active, R, E_loc, S, q_min, t_star, steps, n_rep, stuck)
  if (total < (1 << kPackBits) && E_loc <= 4 && R <= 32)
    UEP_SQ_PACKED(4, true);
  else if (total < (1 << kPackBits) && E_loc <= 4)
    UEP_SQ_PACKED(4, false);
  else if (total < (1 << kPackBits) && E_loc <= 8)
    UEP_SQ_PACKED(8, false);
  else if (total < (1 << kPackBits))
    UEP_SQ_PACKED(0, false);
#undef UEP_SQ_PACKED
  else
    search_wide<kS>(st, q_main, lane, active, R, E_loc, S, q_min, t_star, steps, n_rep, stuck);

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

}  // namespace uep
