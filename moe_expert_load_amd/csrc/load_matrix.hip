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

constexpr int kLmBitmapMaxE = 1024;
constexpr int kLmBitmapMaxK = 16;

// K ids of token (base) into registers; 16-byte loads when K % 4 == 0 and aligned
template <int kN>
__device__ __forceinline__ void load_token(const int32_t* __restrict__ p, int K, bool vec,
                                           int (&v)[kN]) {
  if (vec) {
#pragma unroll
    for (int k = 0; k < kN; k += 4)
      if (k < K) {
        const int4 q = *reinterpret_cast<const int4*>(p + k);
        v[k] = q.x; v[k + 1] = q.y; v[k + 2] = q.z; v[k + 3] = q.w;
      }
  } else {
#pragma unroll
    for (int k = 0; k < kN; ++k)
      if (k < K) v[k] = p[k];
  }
}

template <int kN>
__device__ __forceinline__ void store_token(int32_t* __restrict__ p, int K, bool vec,
                                            const int (&v)[kN]) {
  if (vec) {
#pragma unroll
    for (int k = 0; k < kN; k += 4)
      if (k < K) *reinterpret_cast<int4*>(p + k) = make_int4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < kN; ++k)
      if (k < K) p[k] = v[k];
  }
}

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

// Counts only: counts[r][e] = sum of rank r's chunk histograms (one workgroup per rank,
// up to 16 loads in flight per thread).
__global__ __launch_bounds__(256) void lm_counts(const int32_t* __restrict__ chunk_hist,
                                                 int32_t* __restrict__ counts, LmGeom g) {
  const int r = blockIdx.x;
  const int32_t* ch = chunk_hist + (int64_t)r * g.n_chunks * g.E;
  for (int e = threadIdx.x; e < g.E; e += 256) {
    int s = 0;
    if (g.T > 0)
      for (int c0 = 0; c0 < g.n_chunks; c0 += 16) {
        int acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = ch[(int64_t)min(c0 + u, g.n_chunks - 1) * g.E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += c0 + u < g.n_chunks ? acc[u] : 0;
      }
    counts[(int64_t)r * g.E + e] = s;
  }
}

// Long ranks (more earlier chunks than one round of prefix loads covers): each rank's
// chunk histograms are turned into exclusive prefixes in place, so a ranking
// workgroup loads one row instead of summing every earlier chunk's (which reads the
// histograms about n_chunks / 2 times over).  Four threads per expert, each over a
// quarter of the chunks: sums, an LDS exchange of the four partial sums, then the
// prefixes written from the re-read (now cached) counts.
constexpr int kLmScanParts = 4;

__global__ __launch_bounds__(256) void lm_scan(int32_t* __restrict__ chunk_hist, LmGeom g) {
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
  }
}

// kMaxK bounds K (8, 12 or 16): per-token arrays stay small (K <= 8: six waves per
// SIMD), so the 1024 workgroups of a 32-rank layer fit the chip in one round.
// kTile (for K % 4 != 0, where a token's ids are not 16-byte vectors): the chunk's ids
// come in through one flat coalesced read into an LDS tile, the lanes read their
// tokens' ids from it, and the final positions leave through a second tile and one
// flat coalesced write, instead of K strided 4-byte accesses per lane.
constexpr int kLmTileLd = 16;                          // flat loads per thread: 4096 ids
constexpr size_t kLmTileMaxLds = 64 * 1024;            // tiles only while the LDS fits 64 KiB

template <int kMaxK, bool kTile>
__global__ __launch_bounds__(256) void lm_rank(const int32_t* __restrict__ ids,
                                               int32_t* __restrict__ bucket_pos,
                                               const int32_t* __restrict__ chunk_hist,
                                               int32_t* __restrict__ counts, int32_t* err,
                                               LmGeom g, bool vec, bool scanned) {
  extern __shared__ uint64_t lr_lds[];
  uint64_t* mask = lr_lds;                                             // [4][E]
  int32_t* whist = reinterpret_cast<int32_t*>(lr_lds + 4 * g.E);       // [4][E]
  int32_t* pre = whist + 4 * g.E;                                      // [E]
  int32_t* idt = pre + g.E;                        // kTile: [tok_per_chunk * K] ids
  int32_t* pt = idt + g.tok_per_chunk * g.K;       // kTile: [tok_per_chunk * K] positions
  const int r = blockIdx.y, c = blockIdx.x;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int32_t* ch = chunk_hist + (int64_t)r * g.n_chunks * g.E;
  const int t0 = c * g.tok_per_chunk, t1 = min(g.T, t0 + g.tok_per_chunk);
  const int tpw = g.tok_per_chunk / 4;
  const int tw0 = t0 + w * tpw, tw1 = min(t1, tw0 + tpw);
  const int64_t chunk_base = ((int64_t)r * g.T + t0) * g.K;
  const int n = (t1 - t0) * g.K;
  // loads issued before anything else: the chunk's flat ids (kTile), or the wave's
  // first 64 tokens
  int v0[kMaxK], pos0[kMaxK];
  int tv[kTile ? kLmTileLd : 1];
  if (kTile) {
#pragma unroll
    for (int u = 0; u < kLmTileLd; ++u)
      if (u * 256 < n) tv[u] = ids[chunk_base + min(u * 256 + (int)threadIdx.x, n - 1)];
  } else if (tw0 + lane < tw1) {
    load_token(ids + ((int64_t)r * g.T + tw0 + lane) * g.K, g.K, vec, v0);
  }
  // scanned: chunk_hist already holds each chunk's exclusive prefix (E <= 1024 here)
  int pv[kLmBitmapMaxE / 256];
  if (scanned) {
#pragma unroll
    for (int u = 0; u < kLmBitmapMaxE / 256; ++u) {
      const int e = threadIdx.x + 256 * u;
      if (e < g.E) pv[u] = ch[(int64_t)c * g.E + e];
    }
  }
#pragma unroll
  for (int u = 0; u < kLmBitmapMaxE / 256; ++u) {
    const int e = threadIdx.x + 256 * u;
    if (e < g.E) {
      pre[e] = scanned ? pv[u] : 0;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) { mask[ww * g.E + e] = 0; whist[ww * g.E + e] = 0; }
    }
  }
  if (kTile) {
#pragma unroll
    for (int u = 0; u < kLmTileLd; ++u)
      if (u * 256 + (int)threadIdx.x < n) idt[u * 256 + threadIdx.x] = tv[u];
  }
  __syncthreads();
  if (kTile && tw0 + lane < tw1) {
#pragma unroll
    for (int k = 0; k < kMaxK; ++k)
      if (k < g.K) v0[k] = idt[(tw0 + lane - t0) * g.K + k];
  }
  // otherwise pre[e] = sum of the earlier chunks' histograms: `per` threads per
  // expert, each with up to 16 independent loads in flight, combined by LDS atomics
  if (!scanned) {
    const int per = g.E >= 256 ? 1 : 256 / g.E;
    const int part = threadIdx.x % per;
    for (int e = threadIdx.x / per; e < g.E; e += 256 / per) {
      int s = 0;
      for (int cc0 = part; cc0 < c; cc0 += 16 * per) {
        int acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int cc = cc0 + u * per;
          acc[u] = cc < c ? ch[(int64_t)cc * g.E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) s += acc[u];
      }
      if (s) atomicAdd(&pre[e], s);
    }
  }
  uint64_t* vmask = mask + w * g.E;       // this wave's masks and running counts
  int32_t* vhist = whist + w * g.E;
  const uint64_t below = lanemask_lt();
  // one batch of at most 64 tokens per wave: running counts stay 0 and the wave's
  // per-expert counts are read from its masks afterwards
  const bool one = tpw <= kWave;
  // pass 1: ranks among the wave's tokens (provisional, relative to the wave).  The
  // first 64 tokens of the wave stay in registers for pass 2; later ones (only when a
  // wave has more than 64 tokens) go through the position tile (kTile) or bucket_pos.
  for (int tb = tw0; tb < tw1; tb += kWave) {
    const int t = tb + lane;
    const bool live = t < tw1;
    int v[kMaxK];
    int32_t* bp = bucket_pos + ((int64_t)r * g.T + t) * g.K;
    if (tb == tw0) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) v[k] = v0[k];
    } else if (live) {
      if (kTile) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < g.K) v[k] = idt[(t - t0) * g.K + k];
      } else {
        load_token(ids + ((int64_t)r * g.T + t) * g.K, g.K, vec, v);
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= g.K) break;
      if (live && v[k] >= 0 && v[k] < g.E) atomicOr((unsigned long long*)&mask[w * g.E + v[k]], 1ull << lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int pos[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= g.K) break;
      pos[k] = -1;
      if (live && v[k] >= 0 && v[k] < g.E)
        pos[k] = (one ? 0 : vhist[v[k]]) + __popcll(vmask[v[k]] & below);
    }
    if (!one) {       // fold the batch into the running counts, clear the masks
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      for (int e = lane; e < g.E; e += kWave) {
        const uint64_t m = vmask[e];
        if (m) {
          vhist[e] = vhist[e] + __popcll(m);
          vmask[e] = 0;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    if (tb == tw0) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) { v0[k] = v[k]; pos0[k] = pos[k]; }
    } else if (live) {
      if (kTile) {
#pragma unroll
        for (int k = 0; k < kMaxK; ++k)
          if (k < g.K) pt[(t - t0) * g.K + k] = pos[k];
      } else {
        store_token(bp, g.K, vec, pos);
      }
    }
  }
  __syncthreads();
  // wave offsets: earlier chunks + earlier waves of this chunk; the last chunk also
  // writes the rank's row of the load matrix
  for (int e = threadIdx.x; e < g.E; e += 256) {
    int run = pre[e];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int x = one ? (int)__popcll(mask[ww * g.E + e]) : whist[ww * g.E + e];
      whist[ww * g.E + e] = run;
      run += x;
    }
    if (c == g.n_chunks - 1) counts[(int64_t)r * g.E + e] = run;
  }
  __syncthreads();
  // pass 2: final positions, and the check for an expert twice in one token
  int dup = 0;
  for (int tb = tw0; tb < tw1; tb += kWave) {
    const int t = tb + lane;
    if (t >= tw1) continue;
    int v[kMaxK], pos[kMaxK];
    const int64_t base = ((int64_t)r * g.T + t) * g.K;
    if (tb == tw0) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) { v[k] = v0[k]; pos[k] = pos0[k]; }
    } else if (kTile) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < g.K) { v[k] = idt[(t - t0) * g.K + k]; pos[k] = pt[(t - t0) * g.K + k]; }
    } else {
      load_token(ids + base, g.K, vec, v);
      load_token(bucket_pos + base, g.K, vec, pos);
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= g.K) break;
      const bool ok = v[k] >= 0 && v[k] < g.E;
#pragma unroll
      for (int k2 = 0; k2 < kMaxK; ++k2)
        if (k2 < k) dup |= ok && v[k2] == v[k];
      if (ok) pos[k] += whist[w * g.E + v[k]];
    }
    if (kTile) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < g.K) pt[(t - t0) * g.K + k] = pos[k];
    } else {
      store_token(bucket_pos + base, g.K, vec, pos);
    }
  }
  if (dup) set_err(err, UEP_ERR_DUP_ID);
  if (kTile) {          // the chunk's positions leave in one flat coalesced write
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) bucket_pos[chunk_base + i] = pt[i];
  }
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

static bool lm_bitmap(int K, int E) { return E <= kLmBitmapMaxE && K <= kLmBitmapMaxK; }

static LmGeom lm_geom(int R, int T, int K, int E) {
  LmGeom g;
  g.R = R; g.T = T; g.K = K; g.E = E;
  if (lm_bitmap(K, E)) {
    // whole waves of tokens: 256 * max(1, floor(8 / K)) tokens, at most 2048 per chunk
    g.tok_per_chunk = 256 * (K >= 8 ? 1 : 8 / K);
  } else {
    g.tok_per_chunk = kLmPairs / K;
  }
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
      hipLaunchKernelGGL(lm_scan, dim3((E + 63) / 64, R), dim3(256), 0, s, (int32_t*)ws, g);
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
