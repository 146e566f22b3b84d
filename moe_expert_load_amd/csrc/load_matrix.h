// Device side of the load matrix shared by load_matrix.hip (uep_load_matrix, uep_plan)
// and lplb.hip (the fused LPLB plan): the chunk geometry, the per-chunk ranking body and
// the declarations of the chunk-histogram kernels (UltraEP article, section
// "在 Gate 之后获取当前层真实负载").
#pragma once

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

// kTile (for K % 4 != 0, where a token's ids are not 16-byte vectors): the chunk's ids
// come in through one flat coalesced read into an LDS tile, the lanes read their
// tokens' ids from it, and the final positions leave through a second tile and one
// flat coalesced write, instead of K strided 4-byte accesses per lane.
constexpr int kLmTileLd = 16;                          // flat loads per thread: 4096 ids
constexpr size_t kLmTileMaxLds = 64 * 1024;            // tiles only while the LDS fits 64 KiB

// The ranking of chunk c of rank r by one 256-thread workgroup (lr_lds: the dynamic LDS
// the launch sizes); counts may be NULL when the load matrix is already written.
template <int kMaxK, bool kTile, bool kStream>
__device__ __forceinline__ void lm_rank_body(const int32_t* __restrict__ ids,
                                             int32_t* __restrict__ bucket_pos,
                                             const int32_t* __restrict__ chunk_hist,
                                             int32_t* __restrict__ counts, int32_t* err,
                                             const LmGeom& g, bool vec, bool scanned, int c,
                                             int r, uint64_t* lr_lds) {
  uint64_t* mask = lr_lds;                                             // [4][E]
  int32_t* whist = reinterpret_cast<int32_t*>(lr_lds + 4 * g.E);       // [4][E]
  int32_t* pre = whist + 4 * g.E;                                      // [E]
  int32_t* idt = pre + g.E;                        // kTile: [tok_per_chunk * K] ids
  // kTile or kStream: [tok_per_chunk * K] positions (after the ids, or in their place)
  int32_t* pt = kTile ? idt + g.tok_per_chunk * g.K : idt;
  constexpr bool kPt = kTile || kStream;
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
      if (kPt) {
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
    if (counts && c == g.n_chunks - 1) counts[(int64_t)r * g.E + e] = run;
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
    } else if (kStream) {
      load_token(ids + base, g.K, vec, v);
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < g.K) pos[k] = pt[(t - t0) * g.K + k];
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
    if (kPt) {
#pragma unroll
      for (int k = 0; k < kMaxK; ++k)
        if (k < g.K) pt[(t - t0) * g.K + k] = pos[k];
    } else {
      store_token(bucket_pos + base, g.K, vec, pos);
    }
  }
  if (dup) set_err(err, UEP_ERR_DUP_ID);
  if (kPt) {            // the chunk's positions leave in one flat coalesced write
    __syncthreads();
    if (kStream) {
      // streaming stores: nothing is left dirty in the L2 for the end of the launch to
      // write back; 16-byte vectors when the chunk and the tile are 16-byte aligned
      const span_t sp = span_of(bucket_pos + chunk_base, (int64_t)n * 4);
      if (vec && g.E % 4 == 0) {
        for (int i = threadIdx.x; 4 * i < n; i += 256)
          stream_store(*reinterpret_cast<const u32x4*>(pt + 4 * i), sp, 16 * i);
      } else {
        for (int i = threadIdx.x; i < n; i += 256) stream_store_b32((uint32_t)pt[i], sp, 4 * i);
      }
    } else {
      for (int i = threadIdx.x; i < n; i += 256) bucket_pos[chunk_base + i] = pt[i];
    }
  }
}

inline bool lm_bitmap(int K, int E) { return E <= kLmBitmapMaxE && K <= kLmBitmapMaxK; }

inline LmGeom lm_geom(int R, int T, int K, int E) {
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

// The chunk-histogram kernels (load_matrix.hip), also launched by the fused LPLB plan.
__global__ __launch_bounds__(256) void lm_hist(const int32_t* __restrict__ ids,
                                               int32_t* __restrict__ chunk_hist, int32_t* err,
                                               LmGeom g);
__global__ __launch_bounds__(256) void lm_counts(const int32_t* __restrict__ chunk_hist,
                                                 int32_t* __restrict__ counts, LmGeom g);
__global__ __launch_bounds__(256) void lm_scan(int32_t* __restrict__ chunk_hist,
                                               int32_t* __restrict__ counts, LmGeom g);

}  // namespace uep
