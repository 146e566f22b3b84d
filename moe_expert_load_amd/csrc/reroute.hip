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
//   local first, then remote instances in ascending id.  Blocks beyond E zero the
//   columns of unused instances.
// rr_assign: one thread per (token, expert) pair; a short backwards scan over the
//   pair's (rank, expert) segments gives instance and dispatch row.
#include "common.h"

namespace uep {

struct RrGeom {
  int R, T, K, E, ipr, I, seg_cap;
};

__global__ __launch_bounds__(64) void rr_expert(const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ inst_expert,
                                                const int32_t* __restrict__ inst_quota,
                                                int32_t* __restrict__ xfer,
                                                int32_t* __restrict__ inst_offset,
                                                int32_t* __restrict__ seg_base,
                                                int32_t* __restrict__ seg_cnt,
                                                int4* __restrict__ segs, int32_t* err, RrGeom g) {
  __shared__ int32_t o_inst[kWave], o_qlo[kWave], o_qhi[kWave], o_off[kWave];
  __shared__ int32_t s_dlo[kWave], s_dhi[kWave];
  __shared__ int32_t so[kWave * kWave];   // so[src][owner] = rows of earlier sources in owner's instance
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
  o_inst[lane] = my_i;
  o_qlo[lane] = q_lo;
  o_qhi[lane] = q_lo + Q;
  o_off[lane] = my_off;
  s_dlo[lane] = d_lo;
  s_dhi[lane] = d_lo + D;
  __syncthreads();

  // owner lane: its column of X and the running row offset of every source in it
  if (active && my_i >= 0) {
    int run = 0;
    for (int s = 0; s < R; ++s) {
      int x = max(0, min(s_dhi[s], q_lo + Q) - max(s_dlo[s], q_lo));
      if (s == lane) x += xl;
      xfer[(int64_t)s * I + my_i] = x;
      so[s * kWave + lane] = run;
      run += x;
    }
  }
  __syncthreads();

  // segments of source lane: local, then remote owners in ascending rank
  int n = 0;
  if (active) {
    n = xl > 0;
    for (int o = 0; o < R; ++o) {
      if (o == lane || o_inst[o] < 0) continue;
      const int lo = max(d_lo, o_qlo[o]), hi = min(d_lo + D, o_qhi[o]);
      n += hi > lo;
    }
  }
  const int n_incl = wave_incl_scan(n);
  if (lane == 0 && readlane(n_incl, kWave - 1) > g.seg_cap) set_err(err, UEP_ERR_COVER);
  if (active && readlane(n_incl, kWave - 1) <= g.seg_cap) {
    int k = e * g.seg_cap + (n_incl - n);
    seg_base[(int64_t)lane * E + e] = k;
    seg_cnt[(int64_t)lane * E + e] = n;
    if (xl > 0) segs[k++] = make_int4(0, my_i, my_off + so[lane * kWave + lane], xl);
    for (int o = 0; o < R; ++o) {
      if (o == lane || o_inst[o] < 0) continue;
      const int lo = max(d_lo, o_qlo[o]), hi = min(d_lo + D, o_qhi[o]);
      if (hi > lo) {
        const int b0 = xl + (lo - d_lo);
        segs[k++] = make_int4(b0, o_inst[o], o_off[o] + so[lane * kWave + o] - b0, hi - lo);
      }
    }
  } else if (active) {
    seg_cnt[(int64_t)lane * E + e] = 0;
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
  const int e = ids[j];
  int di = -1, dr = -1;
  if (e >= 0 && e < g.E) {
    const int r = (int)(j / ((int64_t)g.T * g.K));
    const int b = bucket_pos[j];
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
  dest_inst[j] = di;
  dest_row[j] = dr;
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
    const int64_t nb = (j1 - j0 + 255) / 256;
    hipLaunchKernelGGL(rr_assign, dim3((unsigned)nb), dim3(256), 0, s, topk_ids, bucket_pos,
                       seg_base, seg_cnt, segs, dest_inst, dest_row, err, j0, j1, g);
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
