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
// rr_assign: one thread per (token, expert) pair; a short backwards scan over the
//   pair's (rank, expert) segments gives instance and dispatch row.
#include "common.h"

namespace uep {

struct RrGeom {
  int R, T, K, E, ipr, I, seg_cap;
};

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
  int my_i = -1, dup = 0;
  if (active)
    for (int j = 0; j < g.ipr; ++j)
      if (inst_expert[lane * g.ipr + j] == e) {
        if (my_i < 0) my_i = lane * g.ipr + j; else dup = 1;
      }
  if (dup) set_err(err, UEP_ERR_INST_DUP);

  // exclusive prefix of all quotas: first row of my instance (expert 0 writes the array)
  int running = 0, my_off = 0, negq = 0;
  for (int base = 0; base < I; base += kWave) {
    const int i = base + lane;
    const int q = i < I ? inst_quota[i] : 0;
    negq |= q < 0;
    const int incl = wave_incl_scan(q);
    const int excl = incl - q;
    if (e == 0 && i < I) inst_offset[i] = running + excl;
    const int src = min(max(my_i - base, 0), kWave - 1);
    const int v = shfl(excl, src);
    if (my_i >= base && my_i < base + kWave) my_off = running + v;
    running += readlane(incl, kWave - 1);
  }
  if (e == 0 && lane == 0) inst_offset[I] = running;
  if (e == 0 && negq) set_err(err, UEP_ERR_BAD_QUOTA);

  const int C = active ? counts[(int64_t)lane * E + e] : 0;
  const int q = my_i >= 0 ? inst_quota[my_i] : 0;
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

__device__ __forceinline__ void assign_one(int e, int b, int r, const int32_t* __restrict__ seg_base,
                                           const int32_t* __restrict__ seg_cnt,
                                           const int4* __restrict__ segs, int32_t* err,
                                           const RrGeom& g, int& di, int& dr) {
  di = -1;
  dr = -1;
  if (e < 0 || e >= g.E) return;
  const int sb = seg_base[(int64_t)r * g.E + e];
  const int n = seg_cnt[(int64_t)r * g.E + e];
  int k = n - 1;
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

__global__ __launch_bounds__(256) void rr_assign(const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ bucket_pos,
                                                 const int32_t* __restrict__ seg_base,
                                                 const int32_t* __restrict__ seg_cnt,
                                                 const int4* __restrict__ segs,
                                                 int32_t* __restrict__ dest_inst,
                                                 int32_t* __restrict__ dest_row, int32_t* err,
                                                 int64_t j0, int64_t j1, RrGeom g) {
  const int64_t j = j0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= j1) return;
  int di, dr;
  assign_one(ids[j], bucket_pos[j], (int)(j / ((int64_t)g.T * g.K)), seg_base, seg_cnt, segs, err,
             g, di, dr);
  dest_inst[j] = di;
  dest_row[j] = dr;
}

// four consecutive pairs per thread (16-byte loads and stores); needs T*K % 4 == 0 so
// the four pairs share a rank and j0 is aligned
__global__ __launch_bounds__(256) void rr_assign4(const int4* __restrict__ ids,
                                                  const int4* __restrict__ bucket_pos,
                                                  const int32_t* __restrict__ seg_base,
                                                  const int32_t* __restrict__ seg_cnt,
                                                  const int4* __restrict__ segs,
                                                  int4* __restrict__ dest_inst,
                                                  int4* __restrict__ dest_row, int32_t* err,
                                                  int64_t q0, int64_t q1, RrGeom g) {
  const int64_t qd = q0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (qd >= q1) return;
  const int r = (int)(qd * 4 / ((int64_t)g.T * g.K));
  const int4 e = ids[qd], b = bucket_pos[qd];
  int4 di, dr;
  assign_one(e.x, b.x, r, seg_base, seg_cnt, segs, err, g, di.x, dr.x);
  assign_one(e.y, b.y, r, seg_base, seg_cnt, segs, err, g, di.y, dr.y);
  assign_one(e.z, b.z, r, seg_base, seg_cnt, segs, err, g, di.z, dr.z);
  assign_one(e.w, b.w, r, seg_base, seg_cnt, segs, err, g, di.w, dr.w);
  dest_inst[qd] = di;
  dest_row[qd] = dr;
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
    const int64_t j0 = (int64_t)r_begin * T * K, j1 = (int64_t)r_end * T * K;
    const bool vec = ((int64_t)T * K) % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(topk_ids) | reinterpret_cast<uintptr_t>(bucket_pos) |
                       reinterpret_cast<uintptr_t>(dest_inst) | reinterpret_cast<uintptr_t>(dest_row)) %
                      16) == 0;
    if (vec) {
      const int64_t q0 = j0 / 4, q1 = j1 / 4;
      const int64_t nb = (q1 - q0 + 255) / 256;
      hipLaunchKernelGGL(rr_assign4, dim3((unsigned)nb), dim3(256), 0, s,
                         reinterpret_cast<const int4*>(topk_ids),
                         reinterpret_cast<const int4*>(bucket_pos), seg_base, seg_cnt, segs,
                         reinterpret_cast<int4*>(dest_inst), reinterpret_cast<int4*>(dest_row), err,
                         q0, q1, g);
    } else {
      const int64_t nb = (j1 - j0 + 255) / 256;
      hipLaunchKernelGGL(rr_assign, dim3((unsigned)nb), dim3(256), 0, s, topk_ids, bucket_pos,
                         seg_base, seg_cnt, segs, dest_inst, dest_row, err, j0, j1, g);
    }
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
