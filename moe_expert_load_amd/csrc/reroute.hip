// Local-first reroute and per-token assignment (UltraEP article, section
// "Quota 同时决定专家副本与 token 分流": local instance first, the rest to remote
// instances by their remaining quota, then the aggregate quotas are realised per
// token).
//
// rr_expert: one wave per logical expert, lane r = source rank r.  An expert has at
//   most one instance per rank, and instance ids grow with the rank, so lane r also
//   owns "the instance of e on rank r".  The local pass is a min(); the remote pass
//   lays residual demands (ascending source) against remaining capacities
//   (ascending instance) with two wave scans, and every owner lane writes its
//   column of the transfer matrix X as interval overlaps.  Every source lane then
//   emits its segments {first bucket position, instance, row base, length}:
//   local first, then remote instances in ascending id.  Lanes exchange values only
//   by readlane (no LDS, no barrier).  Blocks beyond E zero the columns of unused
//   instances.
// rr_assign: a workgroup takes 2048 pairs of one rank, stages that rank's segments in
//   LDS, and gives every pair its instance and dispatch row by a short backwards scan
//   over its (rank, expert) segments.
#include "common.h"

namespace uep {

struct RrGeom {
  int R, T, K, E, ipr, I, seg_cap;
};

constexpr int kRrPre = 4;   // instance quotas per lane loaded up front (256 instances)

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) {
  return max(0, min(a1, b1) - max(a0, b0));
}

__global__ __launch_bounds__(64) void rr_expert(const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ inst_expert,
                                                const int32_t* __restrict__ inst_quota,
                                                int32_t* __restrict__ xfer,
                                                int32_t* __restrict__ inst_offset,
                                                int32_t* __restrict__ seg_base,
                                                int32_t* __restrict__ seg_cnt,
                                                int4* __restrict__ segs, int32_t* err, RrGeom g) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int R = g.R, I = g.I, E = g.E;

  if (e < I) {                              // column of an unused instance, checks of the table
    const int ie = inst_expert[e];
    if (ie < 0) {
      for (int s = lane; s < R; s += kWave) xfer[(int64_t)s * I + e] = 0;
      if (lane == 0 && inst_quota[e] != 0) set_err(err, UEP_ERR_BAD_QUOTA);
    }
    if (lane == 0 && (ie >= E || ie < -1)) set_err(err, UEP_ERR_BAD_QUOTA);
  }
  if (e >= E) return;

  const bool active = lane < R;
  // Every load is issued before any is used: the expert's column of the load matrix,
  // this lane's row of the instance table (its experts and quotas: the lane's own
  // instance of e and that instance's quota come from it), and the first kRrPre x 64
  // quotas for the row offsets.  The expert's work is then one memory round trip deep.
  const int C = active ? counts[(int64_t)lane * E + e] : 0;
  int qpre[kRrPre];
#pragma unroll
  for (int u = 0; u < kRrPre; ++u) {
    const int i = u * kWave + lane;
    qpre[u] = i < I ? inst_quota[i] : 0;
  }
  int my_i = -1, dup = 0, q = 0;
  if (active) {
#pragma unroll 8
    for (int j = 0; j < g.ipr; ++j) {
      const int ie = inst_expert[lane * g.ipr + j];
      const int iq = inst_quota[lane * g.ipr + j];
      if (ie == e) {
        if (my_i < 0) { my_i = lane * g.ipr + j; q = iq; } else dup = 1;
      }
    }
  }
  if (dup) set_err(err, UEP_ERR_INST_DUP);

  // exclusive prefix of all quotas: first row of my instance (expert 0 writes the array)
  int running = 0, my_off = 0, negq = 0;
  for (int base = 0, u = 0; base < I; base += kWave, ++u) {
    const int i = base + lane;
    int qi = 0;
#pragma unroll
    for (int w = 0; w < kRrPre; ++w) qi = w == u ? qpre[w] : qi;
    if (u >= kRrPre) qi = i < I ? inst_quota[i] : 0;
    negq |= qi < 0;
    const int incl = wave_incl_scan(qi);
    const int excl = incl - qi;
    if (e == 0 && i < I) inst_offset[i] = running + excl;
    const int src = min(max(my_i - base, 0), kWave - 1);
    const int v = shfl(excl, src);
    if (my_i >= base && my_i < base + kWave) my_off = running + v;
    running += readlane(incl, kWave - 1);
  }
  if (e == 0 && lane == 0) inst_offset[I] = running;
  if (e == 0 && negq) set_err(err, UEP_ERR_BAD_QUOTA);

  const int xl = min(C, q);                 // local pass
  const int D = C - xl, Q = q - xl;
  const int d_incl = wave_incl_scan(D), q_incl = wave_incl_scan(Q);
  const int d_lo = d_incl - D, q_lo = q_incl - Q;
  if (lane == 0 && readlane(d_incl, kWave - 1) != readlane(q_incl, kWave - 1))
    set_err(err, UEP_ERR_QUOTA_SUM);

  // Only ranks holding an instance of e matter (usually one or two).  For each such
  // owner o, in ascending rank, every source lane s computes the tokens it sends o:
  // the overlap of its demand interval [d_lo_s, d_lo_s + D_s) with o's capacity
  // interval [q_lo_o, q_lo_o + Q_o), plus o's local tokens when s == o, and writes
  // its entry of o's column of X.  Rows of an instance are ordered by source rank, so
  // source s starts in o's block after the overlap of [0, d_lo_s) with o's interval,
  // plus o's local tokens when o < s.  Segments of a source: its local instance first,
  // then the remote owners in ascending rank.
  const uint64_t owners = ballot(active && my_i >= 0);
  int n = active ? (xl > 0) : 0;
  for (uint64_t m = owners; m; m &= m - 1) {
    const int o = __ffsll((unsigned long long)m) - 1;
    const int oi = readlane(my_i, o), oql = readlane(q_lo, o), oqh = oql + readlane(Q, o);
    const int oxl = readlane(xl, o);
    if (active) {
      const int x = overlap(d_lo, d_lo + D, oql, oqh);
      xfer[(int64_t)lane * I + oi] = x + (lane == o ? oxl : 0);
      n += (lane != o && x > 0);
    }
  }
  const int n_incl = wave_incl_scan(n);
  const int n_tot = readlane(n_incl, kWave - 1);
  if (lane == 0 && n_tot > g.seg_cap) set_err(err, UEP_ERR_COVER);
  const bool fits = n_tot <= g.seg_cap;
  int k = e * g.seg_cap + (n_incl - n);
  if (active) {
    seg_base[(int64_t)lane * E + e] = k;
    seg_cnt[(int64_t)lane * E + e] = fits ? n : 0;
    if (fits && xl > 0) segs[k++] = make_int4(0, my_i, my_off + overlap(0, d_lo, q_lo, q_lo + Q), xl);
  }
  for (uint64_t m = owners; m; m &= m - 1) {
    const int o = __ffsll((unsigned long long)m) - 1;
    const int oi = readlane(my_i, o), oql = readlane(q_lo, o), oqh = oql + readlane(Q, o);
    const int ooff = readlane(my_off, o), oxl = readlane(xl, o);
    if (fits && active && o != lane) {
      const int lo = max(d_lo, oql), hi = min(d_lo + D, oqh);
      if (hi > lo) {
        const int b0 = xl + (lo - d_lo);
        const int before = overlap(0, d_lo, oql, oqh) + (o < lane ? oxl : 0);
        segs[k++] = make_int4(b0, oi, ooff + before - b0, hi - lo);
      }
    }
  }
}

// Fallback for geometries whose segment table does not fit in LDS: one thread per
// pair, the (rank, expert) list walked backwards in global memory.
__global__ __launch_bounds__(256) void rr_assign_flat(const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ bucket_pos,
                                                      const int32_t* __restrict__ seg_base,
                                                      const int32_t* __restrict__ seg_cnt,
                                                      const int4* __restrict__ segs,
                                                      int32_t* __restrict__ dest_inst,
                                                      int32_t* __restrict__ dest_row, int32_t* err,
                                                      int64_t j0, int64_t j1, RrGeom g) {
  const int64_t j = j0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= j1) return;
  const int e = ids[j], b = bucket_pos[j];
  const int r = (int)(j / ((int64_t)g.T * g.K));
  int di = -1, dr = -1;
  if (e >= 0 && e < g.E) {
    const int sb = seg_base[(int64_t)r * g.E + e];
    int k = seg_cnt[(int64_t)r * g.E + e] - 1;
    int4 sg = make_int4(0, -1, 0, 0);
    for (; k >= 0; --k) {
      sg = segs[sb + k];
      if (sg.x <= b) break;
    }
    if (k >= 0 && b < sg.x + sg.w) {
      di = sg.y;
      dr = sg.z + b;
    } else {
      set_err(err, UEP_ERR_COVER);
    }
  }
  dest_inst[j] = di;
  dest_row[j] = dr;
}

constexpr int kRaThreads = 256;
constexpr size_t kRaMaxLds = 60 * 1024;               // staged segment table limit
constexpr int kRaBase = 4;                            // list bases per thread held in registers

// One workgroup = 256 * kPer consecutive pairs of one source rank r.  The rank's
// segment lists (every expert's) are first copied into LDS, compacted by an
// exclusive scan of their lengths: each instance receives r's tokens of one expert
// only, so the rank has at most I segments.  The pairs' ids and bucket positions are
// loaded before that staging; each pair then walks its (r, expert) list backwards in
// LDS to the segment holding its bucket position.
template <bool kVec4, int kPer>
__global__ __launch_bounds__(kRaThreads) void rr_assign(const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ bucket_pos,
                                                        const int32_t* __restrict__ seg_base,
                                                        const int32_t* __restrict__ seg_cnt,
                                                        const int4* __restrict__ segs,
                                                        int32_t* __restrict__ dest_inst,
                                                        int32_t* __restrict__ dest_row, int32_t* err,
                                                        int r_begin, RrGeom g) {
  extern __shared__ int4 ra_lds[];
  int4* lsegs = ra_lds;                                          // [I]
  int32_t* loff = reinterpret_cast<int32_t*>(ra_lds + g.I);      // [E]
  int32_t* lcnt = loff + g.E;                                    // [E]
  __shared__ int32_t wave_tot[kRaThreads / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int r = r_begin + blockIdx.y;
  const int64_t n_pairs = (int64_t)g.T * g.K;
  const int64_t p0 = (int64_t)blockIdx.x * kRaThreads * kPer;
  const int64_t p1 = min(n_pairs, p0 + kRaThreads * kPer);
  const int64_t rbase = (int64_t)r * n_pairs;

  // 1. this thread's pairs (issued first; consumed after the staging)
  int e_[kPer], b_[kPer];
  if (kVec4) {
#pragma unroll
    for (int it = 0; it < kPer / 4; ++it) {
      const int64_t j = p0 + 4 * ((int64_t)it * kRaThreads + tid);
      int4 ev = make_int4(-1, -1, -1, -1), bv = make_int4(0, 0, 0, 0);
      if (j < p1) {
        ev = *reinterpret_cast<const int4*>(ids + rbase + j);
        bv = *reinterpret_cast<const int4*>(bucket_pos + rbase + j);
      }
      e_[4 * it] = ev.x; e_[4 * it + 1] = ev.y; e_[4 * it + 2] = ev.z; e_[4 * it + 3] = ev.w;
      b_[4 * it] = bv.x; b_[4 * it + 1] = bv.y; b_[4 * it + 2] = bv.z; b_[4 * it + 3] = bv.w;
    }
  } else {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int64_t j = p0 + (int64_t)it * kRaThreads + tid;
      e_[it] = j < p1 ? ids[rbase + j] : -1;
      b_[it] = j < p1 ? bucket_pos[rbase + j] : 0;
    }
  }

  // 2. segment counts and list bases of rank r, loaded together: thread t owns experts
  //    [t*m, t*m + m); the bases of its first kRaBase experts stay in registers
  const int m = (g.E + kRaThreads - 1) / kRaThreads;
  const int ea = min(g.E, tid * m), eb = min(g.E, ea + m);
  int base_[kRaBase];
#pragma unroll
  for (int u = 0; u < kRaBase; ++u) base_[u] = ea + u < eb ? seg_base[(int64_t)r * g.E + ea + u] : 0;
  int mine = 0;
  for (int e = ea; e < eb; ++e) {
    const int n = seg_cnt[(int64_t)r * g.E + e];
    lcnt[e] = n;
    mine += n;
  }
  const int incl = wave_incl_scan(mine);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int ww = 0; ww < w; ++ww) run += wave_tot[ww];
  // 3. copy the lists into LDS, compacted
  for (int e = ea; e < eb; ++e) {
    int n = lcnt[e];
    if (run + n > g.I) {                    // cannot happen for a consistent plan
      set_err(err, UEP_ERR_COVER);
      n = max(0, g.I - run);
      lcnt[e] = n;
    }
    loff[e] = run;
    int sb = 0;
#pragma unroll
    for (int u = 0; u < kRaBase; ++u) sb = e - ea == u ? base_[u] : sb;
    if (e - ea >= kRaBase) sb = seg_base[(int64_t)r * g.E + e];
    for (int k = 0; k < n; ++k) lsegs[run + k] = segs[sb + k];
    run += n;
  }
  __syncthreads();

  // 4. look the pairs up
  int di_[kPer], dr_[kPer];
  int bad = 0;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = e_[it], b = b_[it];
    di_[it] = -1;
    dr_[it] = -1;
    if (e < 0 || e >= g.E) continue;
    const int o = loff[e];
    int k = lcnt[e] - 1;
    int4 sg = make_int4(0, -1, 0, 0);
    for (; k >= 0; --k) {
      sg = lsegs[o + k];
      if (sg.x <= b) break;
    }
    if (k >= 0 && b < sg.x + sg.w) {
      di_[it] = sg.y;
      dr_[it] = sg.z + b;
    } else {
      bad = 1;
    }
  }
  if (bad) set_err(err, UEP_ERR_COVER);

  // 5. store
  if (kVec4) {
#pragma unroll
    for (int it = 0; it < kPer / 4; ++it) {
      const int64_t j = p0 + 4 * ((int64_t)it * kRaThreads + tid);
      if (j < p1) {
        *reinterpret_cast<int4*>(dest_inst + rbase + j) =
            make_int4(di_[4 * it], di_[4 * it + 1], di_[4 * it + 2], di_[4 * it + 3]);
        *reinterpret_cast<int4*>(dest_row + rbase + j) =
            make_int4(dr_[4 * it], dr_[4 * it + 1], dr_[4 * it + 2], dr_[4 * it + 3]);
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int64_t j = p0 + (int64_t)it * kRaThreads + tid;
      if (j < p1) {
        dest_inst[rbase + j] = di_[it];
        dest_row[rbase + j] = dr_[it];
      }
    }
  }
}

static void rr_ws_layout(int R, int E, size_t* off_cnt, size_t* off_segs, size_t* total,
                         int* seg_cap) {
  *seg_cap = 3 * R + 1;
  const size_t a = sizeof(int32_t) * (size_t)R * E;
  *off_cnt = a;
  *off_segs = (2 * a + 15) / 16 * 16;
  *total = *off_segs + sizeof(int4) * (size_t)E * (*seg_cap);
}

}  // namespace uep

using namespace uep;

extern "C" size_t uep_reroute_workspace_size(int32_t R, int32_t E, int32_t inst_per_rank) {
  if (R <= 0 || E <= 0 || inst_per_rank <= 0) return 0;
  size_t a, b, t;
  int cap;
  rr_ws_layout(R, E, &a, &b, &t, &cap);
  return t;
}

extern "C" uep_status uep_reroute_assign(const int32_t* counts, const int32_t* topk_ids,
                                         const int32_t* bucket_pos, int32_t R, int32_t T,
                                         int32_t K, int32_t E, int32_t inst_per_rank,
                                         const int32_t* inst_expert, const int32_t* inst_quota,
                                         int32_t r_begin, int32_t r_end, int32_t* xfer,
                                         int32_t* inst_offset, int32_t* dest_inst,
                                         int32_t* dest_row, int32_t* err, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0 || inst_per_rank <= 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (R > 64 || E > 4096 || K > 64 || (int64_t)R * T * K >= (1ll << 31) ||
      (int64_t)R * inst_per_rank > (1 << 20))
    return UEP_EGEOM;
  if (!counts || !inst_expert || !inst_quota || !xfer || !inst_offset) return UEP_EINVAL;
  const bool pairs = r_end > r_begin && T > 0;
  if (pairs && (!topk_ids || !bucket_pos || !dest_inst || !dest_row)) return UEP_EINVAL;
  size_t off_cnt, off_segs, total;
  int cap;
  rr_ws_layout(R, E, &off_cnt, &off_segs, &total, &cap);
  if (!ws || ws_bytes < total) return UEP_EWORKSPACE;
  RrGeom g{R, T, K, E, inst_per_rank, R * inst_per_rank, cap};
  char* w = static_cast<char*>(ws);
  int32_t* seg_base = reinterpret_cast<int32_t*>(w);
  int32_t* seg_cnt = reinterpret_cast<int32_t*>(w + off_cnt);
  int4* segs = reinterpret_cast<int4*>(w + off_segs);
  hipStream_t s = uep_stream(stream);
  const int blocks = E > g.I ? E : g.I;
  hipLaunchKernelGGL(rr_expert, dim3(blocks), dim3(64), 0, s, counts, inst_expert, inst_quota,
                     xfer, inst_offset, seg_base, seg_cnt, segs, err, g);
  UEP_CHECK_LAUNCH();
  if (pairs) {
    const bool vec = ((int64_t)T * K) % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(topk_ids) | reinterpret_cast<uintptr_t>(bucket_pos) |
                       reinterpret_cast<uintptr_t>(dest_inst) | reinterpret_cast<uintptr_t>(dest_row)) %
                      16) == 0;
    // 8 pairs per thread when that still gives >= 512 workgroups, else 4
    const int64_t pairs_all = (int64_t)T * K * (r_end - r_begin);
    const int per = pairs_all >= 512ll * kRaThreads * 8 ? 8 : 4;
    const int64_t chunks = ((int64_t)T * K + kRaThreads * per - 1) / (kRaThreads * per);
    const dim3 grid((unsigned)chunks, (unsigned)(r_end - r_begin));
    const size_t lds = sizeof(int4) * (size_t)g.I + 2 * sizeof(int32_t) * (size_t)E;
    if (lds > kRaMaxLds) {
      const int64_t j0 = (int64_t)r_begin * T * K, j1 = (int64_t)r_end * T * K;
      hipLaunchKernelGGL(rr_assign_flat, dim3((unsigned)((j1 - j0 + 255) / 256)), dim3(256), 0, s,
                         topk_ids, bucket_pos, seg_base, seg_cnt, segs, dest_inst, dest_row, err,
                         j0, j1, g);
    } else if (vec && per == 8) {
      hipLaunchKernelGGL((rr_assign<true, 8>), grid, dim3(kRaThreads), lds, s, topk_ids,
                         bucket_pos, seg_base, seg_cnt, segs, dest_inst, dest_row, err, r_begin, g);
    } else if (vec) {
      hipLaunchKernelGGL((rr_assign<true, 4>), grid, dim3(kRaThreads), lds, s, topk_ids,
                         bucket_pos, seg_base, seg_cnt, segs, dest_inst, dest_row, err, r_begin, g);
    } else if (per == 8) {
      hipLaunchKernelGGL((rr_assign<false, 8>), grid, dim3(kRaThreads), lds, s, topk_ids,
                         bucket_pos, seg_base, seg_cnt, segs, dest_inst, dest_row, err, r_begin, g);
    } else {
      hipLaunchKernelGGL((rr_assign<false, 4>), grid, dim3(kRaThreads), lds, s, topk_ids,
                         bucket_pos, seg_base, seg_cnt, segs, dest_inst, dest_row, err, r_begin, g);
    }
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
