// Load matrix + stable bucket positions (UltraEP article, section
// "在 Gate 之后获取当前层真实负载": the exact per-expert load of this layer,
// gathered for the whole EP group into one matrix).
//
// Main path (E <= 1024, K <= 16), two launches over chunks of a rank's tokens (three
// for long ranks):
//   lm_hist: per-chunk expert histogram with LDS integer atomics (order-free), the
//     chunk's ids read as one flat coalesced range.
//   lm_scan (long ranks only): each rank's chunk histograms become exclusive prefixes.
//   lm_rank: each of the 4 waves walks its quarter of the chunk 64 tokens at a time,
//     lane = token.  Every lane ORs its bit into a per-expert 64-bit lane mask in LDS
//     for each of its K experts; a pair's rank among the wave's 64 tokens is then the
//     popcount of its expert's mask below its lane, plus the wave's running count.
//     Waves are stitched with an LDS scan and earlier chunks' histograms are added,
//     giving the final positions.  Token order is kept by construction.
// Fallback (larger E or K): lm_chunk ranks pairs with one ballot per id bit
//   (match-any), lm_fix adds the earlier chunks' counts.
// Counts only (no bucket_pos): lm_hist, then lm_counts sums each rank's chunks.
// Pairs of one expert are ranked in token order: ids are distinct inside a token.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "load_matrix.h"
#include "solve_quota.h"

namespace uep {

// Per-chunk expert histogram.  A histogram has no token order, so the chunk's
// (t1 - t0) * K ids are read as one flat range: every load instruction of a wave
// covers 256 consecutive bytes, whatever K is, and the first 8 loads of each thread
// are issued before the LDS is cleared.
__global__ __launch_bounds__(256) void lm_hist(const int32_t* __restrict__ ids,
                                               int32_t* __restrict__ chunk_hist, int32_t* err,
                                               LmGeom g) {
  extern __shared__ int32_t lh_lds[];                 // [E]
  const int r = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x;
  const int t0 = c * g.tok_per_chunk, t1 = min(g.T, t0 + g.tok_per_chunk);
  const int32_t* p = ids + ((int64_t)r * g.T + t0) * g.K;
  const int n = (t1 - t0) * g.K;                      // >= K >= 1: launched only for T > 0
  int v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = p[min(u * 256 + tid, n - 1)];
  for (int e = tid; e < g.E; e += 256) lh_lds[e] = 0;
  __syncthreads();
  int bad = 0;
  for (int i0 = 0;;) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = v[u];
      if (i0 + u * 256 + tid < n) {
        if (e < -1 || e >= g.E) bad = 1;
        else if (e >= 0) atomicAdd(&lh_lds[e], 1);
      }
    }
    i0 += 8 * 256;
    if (i0 >= n) break;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[min(i0 + u * 256 + tid, n - 1)];
  }
  if (bad) set_err(err, UEP_ERR_ID_RANGE);
  __syncthreads();
  int32_t* ch = chunk_hist + ((int64_t)r * g.n_chunks + c) * g.E;
  for (int e = tid; e < g.E; e += 256) ch[e] = lh_lds[e];
}

// Counts only: counts[r][e] = sum of rank r's chunk histograms (one workgroup per rank).
// When E < 256, tpe adjacent threads share an expert, each over every tpe-th chunk
// (so all 256 threads load, up to 16 loads in flight each), and add their sums with
// lane exchanges.
__global__ __launch_bounds__(256) void lm_counts(const int32_t* __restrict__ chunk_hist,
                                                 int32_t* __restrict__ counts, LmGeom g) {
  const int r = blockIdx.x;
  const int32_t* ch = chunk_hist + (int64_t)r * g.n_chunks * g.E;
  const int tpe = g.E >= 256 ? 1 : g.E >= 128 ? 2 : g.E >= 64 ? 4 : g.E >= 32 ? 8 : 16;
  const int part = threadIdx.x % tpe;
  for (int e = threadIdx.x / tpe; e < g.E; e += 256 / tpe) {
    int s = 0;
    if (g.T > 0)
      for (int c0 = part; c0 < g.n_chunks; c0 += 16 * tpe) {
        int acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          acc[u] = ch[(int64_t)min(c0 + u * tpe, g.n_chunks - 1) * g.E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += c0 + u * tpe < g.n_chunks ? acc[u] : 0;
      }
    for (int o = 1; o < tpe; o <<= 1) s += __shfl_xor(s, o, kWave);
    if (part == 0) counts[(int64_t)r * g.E + e] = s;
  }
}

// Long ranks (more earlier chunks than one round of prefix loads covers): each rank's
// chunk histograms are turned into exclusive prefixes in place, so a ranking
// workgroup loads one row instead of summing every earlier chunk's (which reads the
// histograms about n_chunks / 2 times over).  Four threads per expert, each over a
// quarter of the chunks: sums, an LDS exchange of the four partial sums, then the
// prefixes written from the re-read (now cached) counts.  With counts non-null the
// last part's running sum, the rank's total, is also written there (the load matrix,
// so no separate counts launch is needed).
constexpr int kLmScanParts = 4;

__global__ __launch_bounds__(256) void lm_scan(int32_t* __restrict__ chunk_hist,
                                               int32_t* __restrict__ counts, LmGeom g) {
  __shared__ int32_t part_sum[256];
  const int r = blockIdx.y;
  const int e = blockIdx.x * (256 / kLmScanParts) + threadIdx.x / kLmScanParts;
  const int q = threadIdx.x % kLmScanParts;
  const int span = (g.n_chunks + kLmScanParts - 1) / kLmScanParts;
  const int c_lo = min(g.n_chunks, q * span), c_hi = min(g.n_chunks, c_lo + span);
  int32_t* ch = chunk_hist + (int64_t)r * g.n_chunks * g.E;
  int sum = 0;
  if (e < g.E) {
    for (int c0 = c_lo; c0 < c_hi; c0 += 16) {
      int acc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] = ch[(int64_t)min(c0 + u, c_hi - 1) * g.E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) sum += c0 + u < c_hi ? acc[u] : 0;
    }
  }
  part_sum[threadIdx.x] = sum;
  __syncthreads();
  int run = 0;
  for (int q2 = 0; q2 < q; ++q2) run += part_sum[threadIdx.x - q + q2];
  if (e < g.E) {
    for (int c0 = c_lo; c0 < c_hi; c0 += 16) {
      int acc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] = ch[(int64_t)min(c0 + u, c_hi - 1) * g.E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < c_hi) {
          ch[(int64_t)(c0 + u) * g.E + e] = run;
          run += acc[u];
        }
    }
    if (counts && q == kLmScanParts - 1) counts[(int64_t)r * g.E + e] = run;
  }
}

// kMaxK bounds K (8, 12 or 16): per-token arrays stay small (K <= 8: six waves per
// SIMD), so the 1024 workgroups of a 32-rank layer fit the chip in one round.
template <int kMaxK, bool kTile>
__global__ __launch_bounds__(256) void lm_rank(const int32_t* __restrict__ ids,
                                               int32_t* __restrict__ bucket_pos,
                                               const int32_t* __restrict__ chunk_hist,
                                               int32_t* __restrict__ counts, int32_t* err,
                                               LmGeom g, bool vec, bool scanned) {
  extern __shared__ uint64_t lr_lds[];
  lm_rank_body<kMaxK, kTile, false>(ids, bucket_pos, chunk_hist, counts, err, g, vec, scanned,
                             blockIdx.x, blockIdx.y, lr_lds);
}

// Fused plan launch: block 0 runs the quota solve on the load matrix that the launch
// before it finished (the solve needs the counts only), while blocks 1.. rank the
// chunks as lm_rank does.  The solve is one workgroup's dependent chain, several times
// longer than the ranking, so the ranking costs the plan no time of its own.
template <int kMaxK, bool kTile, int kS, bool kStream>
__global__ __launch_bounds__(256) void plan_rank_solve(
    const int32_t* __restrict__ ids, int32_t* __restrict__ bucket_pos,
    const int32_t* __restrict__ chunk_hist, int32_t* err, LmGeom g, bool vec, bool scanned,
    const int32_t* __restrict__ counts, int S, int q_min, int32_t* __restrict__ slot_expert,
    int32_t* __restrict__ inst_expert, int32_t* __restrict__ inst_quota,
    int32_t* __restrict__ rank_load, int32_t* __restrict__ stats) {
  extern __shared__ uint64_t pl_lds[];
  if (blockIdx.x == 0) {
    solve_body<kS>(counts, g.R, g.E, S, q_min, slot_expert, inst_expert, inst_quota, rank_load,
                   stats, reinterpret_cast<int32_t*>(pl_lds));
    return;
  }
  const int b = (int)blockIdx.x - 1;
  lm_rank_body<kMaxK, kTile, kStream>(ids, bucket_pos, chunk_hist, nullptr, err, g, vec, scanned,
                             b % g.n_chunks, b / g.n_chunks, pl_lds);
}

__global__ __launch_bounds__(kLmThreads) void lm_chunk(const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ bucket_pos,
                                                       int32_t* __restrict__ chunk_hist,
                                                       int32_t* err, LmGeom g) {
  extern __shared__ int32_t lm_lds[];                 // [kLmWaves][E] wave histograms
  const int r = blockIdx.y, c = blockIdx.x;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int i = threadIdx.x; i < kLmWaves * g.E; i += kLmThreads) lm_lds[i] = 0;
  __syncthreads();

  const int64_t rank_base = (int64_t)r * g.T * g.K;
  const int t0 = c * g.tok_per_chunk;
  const int t1 = min(g.T, t0 + g.tok_per_chunk);
  const int p0 = t0 * g.K, p1 = t1 * g.K;             // pair range of this chunk
  const int per_wave = kLmItems * kWave;
  const int wb = p0 + w * per_wave;

  int e_reg[kLmItems];
  int rank_reg[kLmItems];
  int bad = 0;
#pragma unroll
  for (int it = 0; it < kLmItems; ++it) {
    const int j = wb + it * kWave + lane;
    int e = -1;
    if (j < p1) {
      e = ids[rank_base + j];
      if (e < -1 || e >= g.E) { bad = 1; e = -1; }
    }
    // match-any over the id bits: lanes with the same non-negative id
    uint64_t m = ballot(e >= 0);
    for (int b = 0; b < g.id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = ballot(bit);
      m &= bit ? bb : ~bb;
    }
    int rk = 0;
    if (e >= 0) {
      const int before = __popcll(m & lanemask_lt());
      const int base = lm_lds[w * g.E + e];
      rk = base + before;
      const bool last = (m >> lane) == 1ull;          // highest lane of its group
      __builtin_amdgcn_wave_barrier();
      if (last) lm_lds[w * g.E + e] = base + __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    e_reg[it] = e;
    rank_reg[it] = rk;
  }
  if (bad) set_err(err, UEP_ERR_ID_RANGE);
  __syncthreads();
  int32_t* ch = chunk_hist + ((int64_t)r * g.n_chunks + c) * g.E;
  for (int e = threadIdx.x; e < g.E; e += kLmThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kLmWaves; ++ww) {
      const int v = lm_lds[ww * g.E + e];
      lm_lds[ww * g.E + e] = run;
      run += v;
    }
    ch[e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kLmItems; ++it) {
    const int j = wb + it * kWave + lane;
    if (j < p1) {
      const int e = e_reg[it];
      bucket_pos[rank_base + j] = e >= 0 ? lm_lds[w * g.E + e] + rank_reg[it] : -1;
    }
  }
}

__global__ __launch_bounds__(kLmThreads) void lm_fix(const int32_t* __restrict__ ids,
                                                     int32_t* __restrict__ bucket_pos,
                                                     const int32_t* __restrict__ chunk_hist,
                                                     int32_t* __restrict__ counts, int32_t* err,
                                                     LmGeom g) {
  extern __shared__ int32_t pre[];                    // [E] earlier chunks' counts
  const int r = blockIdx.y, c = blockIdx.x;
  const int32_t* ch = chunk_hist + (int64_t)r * g.n_chunks * g.E;
  for (int e = threadIdx.x; e < g.E; e += kLmThreads) {
    int s = 0;
    for (int cc = 0; cc < c; ++cc) s += ch[(int64_t)cc * g.E + e];
    pre[e] = s;
    if (c == g.n_chunks - 1)
      counts[(int64_t)r * g.E + e] = s + (g.T > 0 ? ch[(int64_t)c * g.E + e] : 0);
  }
  __syncthreads();
  const int t0 = c * g.tok_per_chunk;
  const int t1 = min(g.T, t0 + g.tok_per_chunk);
  const int64_t rank_base = (int64_t)r * g.T * g.K;
  int dup = 0;
  for (int t = t0 + threadIdx.x; t < t1; t += kLmThreads) {
    const int64_t base = rank_base + (int64_t)t * g.K;
    if (g.K <= kLmFastK) {
      // the token's ids and provisional positions in registers, all loads issued first
      int e[kLmFastK], b[kLmFastK];
#pragma unroll
      for (int k = 0; k < kLmFastK; ++k)
        if (k < g.K) { e[k] = ids[base + k]; b[k] = bucket_pos[base + k]; }
#pragma unroll
      for (int k = 0; k < kLmFastK; ++k) {
        if (k >= g.K) break;
        const bool valid = e[k] >= 0 && e[k] < g.E;
#pragma unroll
        for (int k2 = 0; k2 < kLmFastK; ++k2)
          if (k2 < k) dup |= valid && e[k2] == e[k];
        if (valid) bucket_pos[base + k] = b[k] + pre[e[k]];
      }
    } else {
      for (int k = 0; k < g.K; ++k) {
        const int e = ids[base + k];
        if (e < 0 || e >= g.E) continue;
        for (int k2 = 0; k2 < k; ++k2) dup |= (ids[base + k2] == e);
        bucket_pos[base + k] += pre[e];
      }
    }
  }
  if (dup) set_err(err, UEP_ERR_DUP_ID);
}

}  // namespace uep

using namespace uep;

extern "C" size_t uep_load_matrix_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E) {
  if (R <= 0 || T < 0 || K <= 0 || K > 64 || E <= 0) return 0;
  LmGeom g = lm_geom(R, T, K, E);
  return sizeof(int32_t) * (size_t)R * g.n_chunks * E;
}

extern "C" uep_status uep_load_matrix(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                                      int32_t E, int32_t* counts, int32_t* bucket_pos,
                                      int32_t* err, void* ws, size_t ws_bytes, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0) return UEP_EINVAL;
  if (R > 64 || K > 64 || E > kLmMaxE || (int64_t)R * T * K >= (1ll << 31)) return UEP_EGEOM;
  if (!counts || (T > 0 && !topk_ids)) return UEP_EINVAL;
  if (!ws || ws_bytes < uep_load_matrix_workspace_size(R, T, K, E)) return UEP_EWORKSPACE;
  LmGeom g = lm_geom(R, T, K, E);
  hipStream_t s = uep_stream(stream);
  dim3 grid(g.n_chunks, R);
  if (!bucket_pos) {          // counts only: flat histograms, then one sum per rank
    if (T > 0) {
      hipLaunchKernelGGL(lm_hist, grid, dim3(256), sizeof(int32_t) * E, s, topk_ids, (int32_t*)ws,
                         err, g);
      UEP_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(lm_counts, dim3(R), dim3(256), 0, s, (const int32_t*)ws, counts, g);
    UEP_CHECK_LAUNCH();
    return UEP_OK;
  }
  if (lm_bitmap(K, E)) {
    const bool vec = K % 4 == 0 && reinterpret_cast<uintptr_t>(topk_ids) % 16 == 0 &&
                     (T == 0 || reinterpret_cast<uintptr_t>(bucket_pos) % 16 == 0);
    if (T > 0) {
      hipLaunchKernelGGL(lm_hist, grid, dim3(256), sizeof(int32_t) * E, s, topk_ids, (int32_t*)ws,
                         err, g);
      UEP_CHECK_LAUNCH();
    }
    // long ranks: one in-place scan of the chunk histograms instead of every ranking
    // workgroup summing the earlier ones (more than one round of 16 loads per thread)
    const int per = E >= 256 ? 1 : 256 / E;
    const bool scanned = T > 0 && g.n_chunks > 16 * per;
    if (scanned) {
      hipLaunchKernelGGL(lm_scan, dim3((E + 63) / 64, R), dim3(256), 0, s, (int32_t*)ws,
                         (int32_t*)nullptr, g);
      UEP_CHECK_LAUNCH();
    }
    const size_t lds = sizeof(uint64_t) * 4 * E + sizeof(int32_t) * 5 * E;
    const size_t lds_tile = lds + sizeof(int32_t) * 2 * (size_t)g.tok_per_chunk * K;
    const bool tile = !vec && lds_tile <= kLmTileMaxLds;
    const size_t sh = tile ? lds_tile : lds;
    const int32_t* ch = (const int32_t*)ws;
#define UEP_LM_RANK(KM, TL) \
    hipLaunchKernelGGL((lm_rank<KM, TL>), grid, dim3(256), sh, s, topk_ids, bucket_pos, ch, counts, \
                       err, g, vec, scanned)
    if (K <= 8) {
      if (tile) UEP_LM_RANK(8, true); else UEP_LM_RANK(8, false);
    } else if (K <= 12) {
      if (tile) UEP_LM_RANK(12, true); else UEP_LM_RANK(12, false);
    } else {
      if (tile) UEP_LM_RANK(16, true); else UEP_LM_RANK(16, false);
    }
#undef UEP_LM_RANK
    UEP_CHECK_LAUNCH();
    return UEP_OK;
  }
  if (T > 0) {
    hipLaunchKernelGGL(lm_chunk, grid, dim3(kLmThreads), sizeof(int32_t) * kLmWaves * E, s,
                       topk_ids, bucket_pos, (int32_t*)ws, err, g);
    UEP_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(lm_fix, grid, dim3(kLmThreads), sizeof(int32_t) * E, s, topk_ids, bucket_pos,
                     (const int32_t*)ws, counts, err, g);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}

// ---------------------------------------------------------------------------------
// uep_plan: uep_load_matrix, uep_solve_quota and uep_reroute_assign in one call, with
// the solve overlapped with the ranking.  Launches: lm_hist, lm_counts (the load
// matrix; for long ranks lm_scan, which also writes it), plan_rank_solve (solve ||
// ranking), then the
// reroute and assignment of uep_reroute_assign.  Geometries off the ranking fast path
// (E > 1024 or K > 16) run the three calls one after the other instead.
static size_t plan_align(size_t b) { return (b + 255) / 256 * 256; }

extern "C" size_t uep_plan_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E, int32_t S) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0 || S < 0 || E % R != 0) return 0;
  return plan_align(uep_load_matrix_workspace_size(R, T, K, E)) +
         uep_reroute_workspace_size(R, E, E / R + S);
}

extern "C" uep_status uep_plan(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                               int32_t E, int32_t S, int32_t q_min, int32_t r_begin,
                               int32_t r_end, int32_t* counts, int32_t* bucket_pos,
                               int32_t* slot_expert, int32_t* inst_expert, int32_t* inst_quota,
                               int32_t* rank_load, int32_t* stats, int32_t* xfer,
                               int32_t* inst_offset, int32_t* dest_inst, int32_t* dest_row,
                               int32_t* err, void* ws, size_t ws_bytes, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0 || S < 0 || q_min < 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (R > 64 || K > 64 || E > 4096 || E % R != 0 || E / R > 64 || S > kSqMaxS ||
      (int64_t)R * T * K >= (1ll << 31))
    return UEP_EGEOM;
  // every check of the three calls, before anything is enqueued
  if (!counts || !inst_expert || !inst_quota || !rank_load || !stats || !xfer || !inst_offset ||
      (S > 0 && !slot_expert) || (T > 0 && (!topk_ids || !bucket_pos)) ||
      (T > 0 && r_end > r_begin && (!dest_inst || !dest_row)))
    return UEP_EINVAL;
  if ((int64_t)R * (E / R + S) > (1 << 20)) return UEP_EGEOM;
  if (!ws || ws_bytes < uep_plan_workspace_size(R, T, K, E, S)) return UEP_EWORKSPACE;
  const size_t lm_bytes = plan_align(uep_load_matrix_workspace_size(R, T, K, E));
  void* rr_ws = static_cast<char*>(ws) + lm_bytes;
  const size_t rr_bytes = ws_bytes - lm_bytes;
  const int ipr = E / R + S;
  if (!lm_bitmap(K, E) || T == 0) {
    uep_status st = uep_load_matrix(topk_ids, R, T, K, E, counts, bucket_pos, err, ws, lm_bytes,
                                    stream);
    if (st == UEP_OK)
      st = uep_solve_quota(counts, R, E, S, q_min, slot_expert, inst_expert, inst_quota,
                           rank_load, stats, stream);
    if (st == UEP_OK)
      st = uep_reroute_assign(counts, topk_ids, bucket_pos, R, T, K, E, ipr, inst_expert,
                              inst_quota, r_begin, r_end, xfer, inst_offset, dest_inst, dest_row,
                              err, rr_ws, rr_bytes, stream);
    return st;
  }
  LmGeom g = lm_geom(R, T, K, E);
  hipStream_t s = uep_stream(stream);
  int32_t* hist = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(lm_hist, dim3(g.n_chunks, R), dim3(256), sizeof(int32_t) * E, s, topk_ids,
                     hist, err, g);
  UEP_CHECK_LAUNCH();
  // long ranks: the scan also writes the load matrix (no counts launch)
  const int per = E >= 256 ? 1 : 256 / E;
  const bool scanned = g.n_chunks > 16 * per;
  if (scanned)
    hipLaunchKernelGGL(lm_scan, dim3((E + 63) / 64, R), dim3(256), 0, s, hist, counts, g);
  else
    hipLaunchKernelGGL(lm_counts, dim3(R), dim3(256), 0, s, (const int32_t*)hist, counts, g);
  UEP_CHECK_LAUNCH();
  const bool vec = K % 4 == 0 && reinterpret_cast<uintptr_t>(topk_ids) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(bucket_pos) % 16 == 0;
  const size_t lds = sizeof(uint64_t) * 4 * E + sizeof(int32_t) * 5 * E;
  const size_t lds_tile = lds + sizeof(int32_t) * 2 * (size_t)g.tok_per_chunk * K;
  const bool tile = !vec && lds_tile <= kLmTileMaxLds;
  // untiled, the positions leave through an LDS tile with streaming stores while the
  // LDS still fits (lm_rank_body, kStream)
  const size_t lds_pos = lds + sizeof(int32_t) * (size_t)g.tok_per_chunk * K;
  const bool stream_pos = !tile && lds_pos <= kLmTileMaxLds;
  const size_t sh = std::max(tile ? lds_tile : (stream_pos ? lds_pos : lds), sizeof(int32_t) * (size_t)E);
  const dim3 grid(1 + g.n_chunks * R);
#define UEP_PLAN_FUSED(KM, TL, KS, ST)                                                          \
  hipLaunchKernelGGL((plan_rank_solve<KM, TL, KS, ST>), grid, dim3(256), sh, s, topk_ids,        \
                     bucket_pos, (const int32_t*)hist, err, g, vec, scanned,                    \
                     (const int32_t*)counts, S, q_min, slot_expert, inst_expert, inst_quota,    \
                     rank_load, stats)
#define UEP_PLAN_S(KM, TL, ST)                        \
  do {                                                \
    if (S <= 1) UEP_PLAN_FUSED(KM, TL, 1, ST);        \
    else if (S <= 2) UEP_PLAN_FUSED(KM, TL, 2, ST);   \
    else if (S <= 4) UEP_PLAN_FUSED(KM, TL, 4, ST);   \
    else UEP_PLAN_FUSED(KM, TL, 8, ST);               \
  } while (0)
#define UEP_PLAN_K(KM)                                \
  do {                                                \
    if (tile) UEP_PLAN_S(KM, true, false);            \
    else if (stream_pos) UEP_PLAN_S(KM, false, true); \
    else UEP_PLAN_S(KM, false, false);                \
  } while (0)
  if (K <= 8) UEP_PLAN_K(8);
  else if (K <= 12) UEP_PLAN_K(12);
  else UEP_PLAN_K(16);
#undef UEP_PLAN_K
#undef UEP_PLAN_S
#undef UEP_PLAN_FUSED
  UEP_CHECK_LAUNCH();
  return uep_reroute_assign(counts, topk_ids, bucket_pos, R, T, K, E, ipr, inst_expert, inst_quota,
                            r_begin, r_end, xfer, inst_offset, dest_inst, dest_row, err, rr_ws,
                            rr_bytes, stream);
}

// ---------------------------------------------------------------------------------
// uep_load_matrix_noalloc: the same call with its chunk histograms in a library-owned
// device array instead of a caller workspace, for callers that cannot allocate.
//
// `scratch` is a file-scope device array: each GPU the library runs on holds its own
// copy until the process ends.  Its device address is looked up once per device, with
// that device current, on the first call there (hipGetSymbolAddress); the host-side
// name of the array is only a stand-in and is never handed to a kernel.  Every call on
// one GPU shares that GPU's array, so calls that overlap on one GPU (two streams, or
// two host threads) race on it.  The kernels write every histogram they read before
// reading it, so nothing needs clearing between calls.
namespace uep {
constexpr size_t kLmScratchBytes = 8u << 20;
constexpr int kLmMaxDevices = 64;
}  // namespace uep

static __device__ __align__(256) int32_t scratch[uep::kLmScratchBytes / sizeof(int32_t)];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[uep::kLmMaxDevices] = {};
}  // namespace

extern "C" uep_status uep_load_matrix_noalloc(const int32_t* topk_ids, int32_t R, int32_t T,
                                              int32_t K, int32_t E, int32_t* counts,
                                              int32_t* bucket_pos, int32_t* err, void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0) return UEP_EINVAL;
  const size_t need = uep_load_matrix_workspace_size(R, T, K, E);
  if (need > kLmScratchBytes) return UEP_EWORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kLmMaxDevices) return UEP_EHIP;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return UEP_EHIP;
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return uep_load_matrix(topk_ids, R, T, K, E, counts, bucket_pos, err, ptr, kLmScratchBytes,
                         stream);
}
