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
//   local first, then remote instances in ascending id, into the expert's list, and
//   the first two of them also into a dense (rank, expert) table.  Lanes exchange
//   values only by readlane (no LDS, no barrier).  Blocks beyond E zero the columns of
//   unused instances.
// rr_assign: one thread per 4 pairs of one rank; each pair reads its (rank,
//   expert) entry of the dense table (32 bytes) and finds its segment there, or, for
//   the rare pair past a (rank, expert)'s second segment, in the expert's list.
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
                                                int4* __restrict__ seg_inline,
                                                int4* __restrict__ segs, int32_t* err, RrGeom g) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int R = g.R, I = g.I, E = g.E;

  // block e also clears X's column e when instance e is unused, and checks its table
  // entry; an expert's block does this after its own work, whose loads go first
  auto unused_column = [&]() {
    if (e >= I) return;
    const int ie = inst_expert[e];
    if (ie < 0) {
      for (int s = lane; s < R; s += kWave) xfer[(int64_t)s * I + e] = 0;
      if (lane == 0 && inst_quota[e] != 0) set_err(err, UEP_ERR_BAD_QUOTA);
    }
    if (lane == 0 && (ie >= E || ie < -1)) set_err(err, UEP_ERR_BAD_QUOTA);
  };
  if (e >= E) {
    unused_column();
    return;
  }

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
  // A segment goes to the expert's list, and the lane's first two also to its entry of
  // the dense (rank, expert) table.  The first segment starts at bucket position 0, so
  // its table record holds the segment count in that field instead.
  int4* inl = seg_inline + ((int64_t)lane * E + e) * 2;
  int idx = 0;
  auto emit = [&](int4 sg) {
    segs[k++] = sg;
    if (idx == 0) inl[0] = make_int4(n, sg.y, sg.z, sg.w);
    else if (idx == 1) inl[1] = sg;
    ++idx;
  };
  if (active) {
    seg_base[(int64_t)lane * E + e] = k;
    if (!fits || n == 0) inl[0] = make_int4(0, -1, 0, 0);
    if (fits && xl > 0) emit(make_int4(0, my_i, my_off + overlap(0, d_lo, q_lo, q_lo + Q), xl));
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
        emit(make_int4(b0, oi, ooff + before - b0, hi - lo));
      }
    }
  }
  unused_column();
}

constexpr int kRaThreads = 256;
constexpr size_t kRaMaxLds = 32 * 1024;   // rank's table row staged in LDS up to this size

// A workgroup takes 256 * kPer consecutive pairs of one source rank r.  The pairs' ids
// and bucket positions are loaded (16-byte vectors when kVec4) together with rank r's
// row of the dense table, which kLds stages in LDS with one coalesced copy (E x 32
// bytes); without kLds each pair gathers its entry from global memory.  An entry holds
// the (r, expert)'s first two segments, with the segment count in the first.  A bucket
// position in neither is looked up backwards in the expert's list (only a (rank,
// expert) with more than two segments has one there).
template <bool kVec4, int kPer, bool kLds>
__global__ __launch_bounds__(kRaThreads) void rr_assign(const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ bucket_pos,
                                                        const int32_t* __restrict__ seg_base,
                                                        const int4* __restrict__ seg_inline,
                                                        const int4* __restrict__ segs,
                                                        int32_t* __restrict__ dest_inst,
                                                        int32_t* __restrict__ dest_row, int32_t* err,
                                                        int r_begin, RrGeom g) {
  extern __shared__ int4 ra_tab[];            // [E][2] when kLds
  const int tid = threadIdx.x;
  const int r = r_begin + blockIdx.y;
  const int64_t n_pairs = (int64_t)g.T * g.K;
  const int64_t p0 = (int64_t)blockIdx.x * kRaThreads * kPer;
  const int64_t p1 = min(n_pairs, p0 + kRaThreads * kPer);
  const int64_t rbase = (int64_t)r * n_pairs;

  // 1. this thread's pairs
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

  // 2. every pair's table entry: rank r's row staged in LDS, or gathered per pair
  const int4* row = seg_inline + (int64_t)r * g.E * 2;
  if (kLds) {
    for (int i = tid; i < 2 * g.E; i += kRaThreads) ra_tab[i] = row[i];
    __syncthreads();
  }
  int4 s0[kPer], s1[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = e_[it] >= 0 && e_[it] < g.E ? e_[it] : 0;
    const int4* t = kLds ? ra_tab + 2 * e : row + 2 * e;
    s0[it] = t[0];
    s1[it] = t[1];
  }

  // 3. resolve
  int di_[kPer], dr_[kPer];
  int bad = 0;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = e_[it], b = b_[it];
    di_[it] = -1;
    dr_[it] = -1;
    if (e < 0 || e >= g.E) continue;
    const int cnt = s0[it].x;
    if (cnt >= 1 && b >= 0 && b < s0[it].w) {
      di_[it] = s0[it].y;
      dr_[it] = s0[it].z + b;
    } else if (cnt >= 2 && b >= s1[it].x && b < s1[it].x + s1[it].w) {
      di_[it] = s1[it].y;
      dr_[it] = s1[it].z + b;
    } else if (cnt > 2) {
      const int sb = seg_base[(int64_t)r * g.E + e];
      for (int k = cnt - 1; k >= 2; --k) {
        const int4 sg = segs[sb + k];
        if (sg.x <= b) {
          if (b < sg.x + sg.w) {
            di_[it] = sg.y;
            dr_[it] = sg.z + b;
          }
          break;
        }
      }
    }
    if (di_[it] < 0) bad = 1;
  }
  if (bad) set_err(err, UEP_ERR_COVER);

  // 4. store, streaming (nt sc1): the outputs go to HBM without staying dirty in this
  // XCD's L2, so the end of the launch has nothing to write back before the next kernel
  // may start (measured on MI355X, the Qwen3-235B layer's 2 M pairs graph-replayed:
  // 6.9 -> 4.7 us).  The spans cover the workgroup's pairs: nothing past p1 is written.
  const span_t si = span_of(dest_inst + rbase + p0, (p1 - p0) * 4);
  const span_t sr = span_of(dest_row + rbase + p0, (p1 - p0) * 4);
  if (kVec4) {
#pragma unroll
    for (int it = 0; it < kPer / 4; ++it) {
      const int off = 16 * (it * kRaThreads + tid);
      stream_store(u32x4{(uint32_t)di_[4 * it], (uint32_t)di_[4 * it + 1],
                         (uint32_t)di_[4 * it + 2], (uint32_t)di_[4 * it + 3]}, si, off);
      stream_store(u32x4{(uint32_t)dr_[4 * it], (uint32_t)dr_[4 * it + 1],
                         (uint32_t)dr_[4 * it + 2], (uint32_t)dr_[4 * it + 3]}, sr, off);
    }
  } else {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int off = 4 * (it * kRaThreads + tid);
      stream_store_b32((uint32_t)di_[it], si, off);
      stream_store_b32((uint32_t)dr_[it], sr, off);
    }
  }
}

// Workspace: the list bases [R][E] (int32), the dense table [R][E][2] (int4), then each
// expert's segment list (seg_cap int4 entries).
static void rr_ws_layout(int R, int E, size_t* off_inline, size_t* off_segs, size_t* total,
                         int* seg_cap) {
  *seg_cap = 3 * R + 1;
  const size_t a = sizeof(int32_t) * (size_t)R * E;
  *off_inline = (a + 15) / 16 * 16;
  *off_segs = *off_inline + 2 * sizeof(int4) * (size_t)R * E;
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
  size_t off_inline, off_segs, total;
  int cap;
  rr_ws_layout(R, E, &off_inline, &off_segs, &total, &cap);
  if (!ws || ws_bytes < total) return UEP_EWORKSPACE;
  RrGeom g{R, T, K, E, inst_per_rank, R * inst_per_rank, cap};
  char* w = static_cast<char*>(ws);
  int32_t* seg_base = reinterpret_cast<int32_t*>(w);
  int4* seg_inline = reinterpret_cast<int4*>(w + off_inline);
  int4* segs = reinterpret_cast<int4*>(w + off_segs);
  hipStream_t s = uep_stream(stream);
  const int blocks = E > g.I ? E : g.I;
  hipLaunchKernelGGL(rr_expert, dim3(blocks), dim3(64), 0, s, counts, inst_expert, inst_quota,
                     xfer, inst_offset, seg_base, seg_inline, segs, err, g);
  UEP_CHECK_LAUNCH();
  if (pairs) {
    const bool vec = ((int64_t)T * K) % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(topk_ids) | reinterpret_cast<uintptr_t>(bucket_pos) |
                       reinterpret_cast<uintptr_t>(dest_inst) | reinterpret_cast<uintptr_t>(dest_row)) %
                      16) == 0;
    // 4 pairs per thread: more, smaller workgroups finish sooner (measured on MI355X,
    // the Qwen3-235B layer's 2 M pairs graph-replayed: 4 pairs 6.9 us, 8 pairs 7.5 us,
    // 16 pairs 8.5 us)
    const int per = 4;
    const int64_t chunks = ((int64_t)T * K + kRaThreads * per - 1) / (kRaThreads * per);
    const dim3 grid((unsigned)chunks, (unsigned)(r_end - r_begin));
    // rank r's table row in LDS when it is small enough for several workgroups per CU
    const size_t tab = 2 * sizeof(int4) * (size_t)E;
    const bool lds = tab <= kRaMaxLds;
#define UEP_RA(V, P, L)                                                                          \
  hipLaunchKernelGGL((rr_assign<V, P, L>), grid, dim3(kRaThreads), L ? tab : 0, s, topk_ids,     \
                     bucket_pos, (const int32_t*)seg_base, (const int4*)seg_inline,             \
                     (const int4*)segs, dest_inst, dest_row, err, r_begin, g)
#define UEP_RA_L(V, P)                   \
  do {                                   \
    if (lds) UEP_RA(V, P, true);         \
    else UEP_RA(V, P, false);            \
  } while (0)
    if (vec) UEP_RA_L(true, 4);
    else UEP_RA_L(false, 4);
#undef UEP_RA_L
#undef UEP_RA
    UEP_CHECK_LAUNCH();
  }
  return UEP_OK;
}
