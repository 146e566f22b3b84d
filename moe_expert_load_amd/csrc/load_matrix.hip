// Load matrix + stable bucket positions (UltraEP article, section
// "在 Gate 之后获取当前层真实负载": the exact per-expert load of this layer,
// gathered for the whole EP group into one matrix).
//
// Two launches over chunks of one rank's (token, expert) pairs:
//   lm_chunk: every 256-thread workgroup takes 4096 consecutive pairs (whole
//     tokens).  Each wave walks its 1024 pairs 64 at a time; lanes holding the same
//     expert are found with one ballot per id bit (match-any), so a pair's rank
//     inside the wave is a popcount of lower matching lanes and the last matching
//     lane bumps the wave's LDS counter -- no atomics, order fixed by pair index.
//     The 4 wave histograms are scanned in LDS, giving chunk-relative positions and
//     the chunk histogram (to workspace).
//   lm_fix: one workgroup per chunk adds the exclusive sum of earlier chunks'
//     histograms, checks each token for repeated experts, and the last chunk of a
//     rank writes counts[r][:].
// Pairs are counted in pair order j = t*K + k; since ids are distinct within a
// token, pair order inside a bucket is token order.
#include "common.h"

namespace uep {

constexpr int kLmThreads = 256;
constexpr int kLmItems = 16;                          // pairs per lane
constexpr int kLmPairs = kLmThreads * kLmItems;       // 4096 pairs per chunk
constexpr int kLmWaves = kLmThreads / kWave;
constexpr int kLmMaxE = 4096;
constexpr int kLmFastK = 16;                         // register path of lm_fix

struct LmGeom {
  int R, T, K, E, tok_per_chunk, n_chunks, id_bits;
};

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

static LmGeom lm_geom(int R, int T, int K, int E) {
  LmGeom g;
  g.R = R; g.T = T; g.K = K; g.E = E;
  g.tok_per_chunk = kLmPairs / K;
  g.n_chunks = T > 0 ? (T + g.tok_per_chunk - 1) / g.tok_per_chunk : 1;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  g.id_bits = bits;
  return g;
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
  if (!counts || (T > 0 && (!topk_ids || !bucket_pos))) return UEP_EINVAL;
  if (!ws || ws_bytes < uep_load_matrix_workspace_size(R, T, K, E)) return UEP_EWORKSPACE;
  LmGeom g = lm_geom(R, T, K, E);
  hipStream_t s = uep_stream(stream);
  dim3 grid(g.n_chunks, R);
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
