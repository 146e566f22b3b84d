// LPLB: min-max split of replicated experts' load over their copies (Waterfill/LPLB
// blog, sections "线性规划（LP）公式化构建" and "决策变量与矩阵规模优化": minimise the
// peak rank load M; per rank, copy allocation + fixed single-copy load + slack = M;
// per replicated expert, the split sums to its true count; the structural matrix is
// built offline from the placement, only the right-hand side changes per batch; a
// Big-M auxiliary column keeps the system feasible and is driven to zero.  Section
// "从全局计数到LP求解的工程实现": every rank solves the same LP on the GPU with an
// interior-point method into preallocated buffers.  Section "从LP解决方案到Token调度":
// the split decides how each replicated expert's tokens go to its copies).
//
// Standard form, loads scaled by sigma = max(1, mean rank load):
//   variables x_p (copies), s_r (rank slacks), M, a (Big-M column, cost 8), all >= 0
//   rank r  : M + a - s_r - sum_{p on r} x_p = F_r     group g : sum_{p in g} x_p = c_g
// Solver: Mehrotra predictor-corrector, fp32 iterates, one workgroup.  The normal
// equations A D A^T dy = rhs are reduced by eliminating the (diagonal) expert rows;
// the remaining R x R rank matrix P = (d_M + d_a) 11^T + diag(d_s) + sum over groups
// of a weighted Laplacian of the copies' ranks is assembled and factored as
// U diag(p) U^T (LDL^T, no square roots) in fp64 in LDS.  fp32 is not enough there:
// the dense M direction (d_M -> inf) swamps the differential entries of copies whose
// optimal share is a small fraction of the peak.  Diagonal entries are formed as sums
// of positive terms (no cancellation); a pivot that lost its precision is treated as
// infinite (1/p = 1e-64, Cholesky-infinity), which drops that direction.  Iterations stop once the duality gap is below 1e-4 of the
// objective M (or mu < 1e-9), at most `iters` of them.
// Output: x >= 0 normalised so each group sums exactly to its count, m = the max rank
// load of that split, and integer quotas by largest remainder on rint(x * 256).
#include <math.h>

#include <algorithm>
#include <vector>

#include "common.h"
#include "load_matrix.h"
#include "philox.h"

namespace uep {

constexpr int kLpThreads = 256;
constexpr int kLpMaxR = 64;
constexpr int kLpMaxG = 128;
constexpr int kLpMaxN = 256;
constexpr int kLpMaxE = 4096;
constexpr int kLpMaxI = 64 * 40;
constexpr int kLpMagic = 0x4C50424D;             // structure layout 2: with lane groups
constexpr int kLpLanes = 256;                     // lane slots of the block path (one workgroup)
constexpr float kBigM = 8.0f;
constexpr float kEta = 0.99f;
constexpr float kMuStop = 1e-9f;
constexpr double kGapRel = 1e-4;
constexpr int kLpPanel = 16;             // Cholesky panel width (divides 16)
constexpr double kPivTol = 1e-13;
constexpr int kLpMaxNV = kLpMaxN + kLpMaxR + 2;
constexpr int kLpMaxRows = kLpMaxR + kLpMaxG;

// device structure (int32 words):
// [0..7] magic, R, E, ipr, I, G, n, n_ent
// grp_expert[G] | grp_start[G+1] | copy_inst[n] | copy_rank[n] | copy_group[n] |
// rank_start[R+1] | rank_copy[n] | exp_inst[E] | inst_expert[I] | inst_copy[I] |
// ent_rr[n_ent] | ent_start[n_ent+1] | ent_p[n_pair] | ent_q[n_pair]
// ent_*: the off-diagonal entries (r > r') of the rank matrix that copies of one
// group touch: entry e = (ent_rr[e] / 64, ent_rr[e] % 64) sums the pairs
// (ent_p[k] on r, ent_q[k] on r') for k in [ent_start[e], ent_start[e+1]).
// exp_inst[e]: instance of a single-copy expert, -2 - g for replicated group g, -1 none
// inst_copy[i]: copy index of instance i, or -1
// then: blk | lane_rank[256] | rank_lane[R]
// blk (0, 8 or 16): the lane-group size of the block solve, 0 for the dense one.  The
// rank matrix couples two ranks only when a replicated expert has copies on both, so
// its off-diagonal part splits into connected components; with every component at
// most blk ranks, the components are packed into 256 / blk groups of blk lanes
// (first fit, largest first), lane_rank[l] is the rank of lane l (-1: padding) and
// rank_lane[r] its lane.
struct LpView {
  int R, E, ipr, I, G, n, n_ent, blk;
  const int32_t *grp_expert, *grp_start, *copy_inst, *copy_rank, *copy_group;
  const int32_t *rank_start, *rank_copy, *exp_inst, *inst_expert, *inst_copy;
  const int32_t *ent_rr, *ent_start, *ent_p, *ent_q, *lane_rank, *rank_lane;
};

__host__ __device__ inline size_t lp_words(int R, int E, int I, int G, int n, int n_ent,
                                           int n_pair) {
  return 8 + (size_t)G + (G + 1) + 3 * (size_t)n + (R + 1) + n + E + 2 * (size_t)I +
         (size_t)n_ent + (n_ent + 1) + 2 * (size_t)n_pair + 1 + kLpLanes + R;
}

__device__ inline LpView lp_view(const int32_t* w) {
  LpView v;
  v.R = w[1]; v.E = w[2]; v.ipr = w[3]; v.I = w[4]; v.G = w[5]; v.n = w[6]; v.n_ent = w[7];
  const int32_t* p = w + 8;
  v.grp_expert = p; p += v.G;
  v.grp_start = p; p += v.G + 1;
  v.copy_inst = p; p += v.n;
  v.copy_rank = p; p += v.n;
  v.copy_group = p; p += v.n;
  v.rank_start = p; p += v.R + 1;
  v.rank_copy = p; p += v.n;
  v.exp_inst = p; p += v.E;
  v.inst_expert = p; p += v.I;
  v.inst_copy = p; p += v.I;
  v.ent_rr = p; p += v.n_ent;
  v.ent_start = p; p += v.n_ent + 1;
  const int n_pair = v.ent_start[v.n_ent];
  v.ent_p = p; p += n_pair;
  v.ent_q = p; p += n_pair;
  v.blk = *p; p += 1;
  v.lane_rank = p; p += kLpLanes;
  v.rank_lane = p;
  return v;
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

struct LpShared {
  // structure (copied from global)
  int32_t grp_start[kLpMaxG + 1], copy_rank[kLpMaxN], copy_group[kLpMaxN];
  int32_t rank_start[kLpMaxR + 1], rank_copy[kLpMaxN];
  // problem data
  float f[kLpMaxR], hh[kLpMaxG];
  int32_t cnt_i[kLpMaxG];
  // iterates and work vectors (fp32)
  float v[kLpMaxNV], z[kLpMaxNV], dv[kLpMaxNV], dz[kLpMaxNV], rc[kLpMaxNV], tv[kLpMaxNV];
  float y[kLpMaxRows], dy[kLpMaxRows], rb[kLpMaxRows], rhs[kLpMaxRows];
  // normal equations (fp64)
  double d[kLpMaxNV], rbeta[kLpMaxG], cd[kLpMaxN], u64[kLpMaxR];
  double P[kLpMaxR][kLpMaxR + 1];
  double Dinv[kLpMaxR], d0[kLpMaxR];
  double colbuf[2][kLpMaxR];
  // reductions
  double red[kLpThreads / kWave];
  float redf[kLpThreads / kWave];
  double redn[4][kLpThreads / kWave];
  double ysum;                            // sum of the new rank duals (dense solve)
  int32_t Fi[kLpMaxR], hc[kLpMaxG];       // fixed load per rank, count per group
};

// Wave reductions by DPP (quad_perm xor 1, xor 2, row_ror 4 and 8 leave every row of
// 16 lanes holding its row's total; the four rows are combined from lanes 0/16/32/48),
// then across the 4 waves through LDS.  Every lane of the workgroup must take part.
// A block reduction has one barrier, between the waves' partials and their reads: the
// LP keeps at least one barrier between the reads of one reduction and the writes of
// the next (every pair of consecutive reductions in it has one), so the partials of
// the previous reduction are never overwritten while still being read.
// Every lane has a source lane in its own row under these patterns, so mov_dpp's
// bound_ctrl never applies; the form lets the compiler fold a move into its fp32 op.
__device__ __forceinline__ double dpp_d(double v, int ctrl_sel) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  switch (ctrl_sel) {
    case 0: lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, true);
            hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, true); break;
    case 1: lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, true);
            hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, true); break;
    case 2: lo = __builtin_amdgcn_mov_dpp(lo, 0x124, 0xF, 0xF, true);
            hi = __builtin_amdgcn_mov_dpp(hi, 0x124, 0xF, 0xF, true); break;
    default: lo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, true);
             hi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, true); break;
  }
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
  int b = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: b = __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true); break;
    case 1: b = __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true); break;
    case 2: b = __builtin_amdgcn_mov_dpp(b, 0x124, 0xF, 0xF, true); break;
    default: b = __builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true); break;
  }
  return __int_as_float(b);
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int c = 0; c < 4; ++c) x += dpp_d(x, c);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

__device__ __forceinline__ float wave_min_f(float x) {
#pragma unroll
  for (int c = 0; c < 4; ++c) x = fminf(x, dpp_f(x, c));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fminf(fminf(a, b), fminf(c, d));
}

__device__ __forceinline__ double blk_sum(double x, LpShared& S) {
  x = wave_sum_d(x);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) S.red[w] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kLpThreads / kWave; ++i) t += S.red[i];
  return t;
}

__device__ __forceinline__ float blk_min(float x, LpShared& S) {
  x = wave_min_f(x);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) S.redf[w] = x;
  __syncthreads();
  float t = S.redf[0];
#pragma unroll
  for (int i = 1; i < kLpThreads / kWave; ++i) t = fminf(t, S.redf[i]);
  return t;
}

// two minima in one pass (primal and dual step lengths)
__device__ __forceinline__ void blk_min2(float& x, float& y, LpShared& S) {
  x = wave_min_f(x);
  y = wave_min_f(y);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) { S.redf[w] = x; S.red[w] = y; }
  __syncthreads();
  float tx = S.redf[0], ty = (float)S.red[0];
#pragma unroll
  for (int i = 1; i < kLpThreads / kWave; ++i) {
    tx = fminf(tx, S.redf[i]);
    ty = fminf(ty, (float)S.red[i]);
  }
  x = tx;
  y = ty;
}

// kN block sums in one pass (each summed in the same order as blk_sum)
template <int kN>
__device__ __forceinline__ void blk_sum_n(double (&x)[kN], LpShared& S) {
#pragma unroll
  for (int j = 0; j < kN; ++j) x[j] = wave_sum_d(x[j]);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
#pragma unroll
    for (int j = 0; j < kN; ++j) S.redn[j][w] = x[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kN; ++j) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kLpThreads / kWave; ++i) t += S.redn[j][i];
    x[j] = t;
  }
}

// Row i of A (i < R + G) belongs to thread i, which holds the row's range for the whole
// solve: rank_copy[lo, hi) for a rank row, the copies [lo, hi) for a group row.
static_assert(kLpMaxR + kLpMaxG <= kLpThreads, "one row of A per thread");
struct LpRow {
  int lo, hi;
};

__device__ __forceinline__ LpRow lp_row(int R, int G, const LpShared& S) {
  const int i = threadIdx.x;
  if (i < R) return {S.rank_start[i], S.rank_start[i + 1]};
  if (i < R + G) return {S.grp_start[i - R], S.grp_start[i - R + 1]};
  return {0, 0};
}

// out[i] = fin(i, (A * vec)_i) for i < R + G, with vec(j) the j-th element (read from
// LDS or formed on the fly).  Thread i writes out[i] only: a caller that next touches
// out[i] in thread i needs no barrier in between.
template <class Vec, class Fin>
__device__ __forceinline__ void lp_Av(Vec vec, Fin fin, float* out, int n, int R, int G,
                                      const LpRow& W, LpShared& S) {
  const float Ma = vec(n + R) + vec(n + R + 1);
  const int i = threadIdx.x;
  if (i < R) {
    float acc = Ma - vec(n + i);
    for (int k = W.lo; k < W.hi; ++k) acc -= vec(S.rank_copy[k]);
    out[i] = fin(i, acc);
  } else if (i < R + G) {
    float acc = 0.0f;
    for (int p = W.lo; p < W.hi; ++p) acc += vec(p);
    out[i] = fin(i, acc);
  }
}

// (A^T y)_i, given ys = the sum of the rank duals (the M and a columns)
__device__ __forceinline__ float lp_ATy_at(int i, const float* yv, float ys, int n, int R,
                                           const LpShared& S) {
  if (i < n) return -yv[S.copy_rank[i]] + yv[R + S.copy_group[i]];
  if (i < n + R) return -yv[i - n];
  return ys;
}

// out[nv] = A^T * y
__device__ __forceinline__ void lp_ATy(const float* yv, float* out, int n, int R, int G, LpShared& S) {
  float part = 0.0f;
  for (int r = threadIdx.x; r < R; r += kLpThreads) part += yv[r];
  const float ys = (float)blk_sum((double)part, S);
  for (int i = threadIdx.x; i < n + R + 2; i += kLpThreads) out[i] = lp_ATy_at(i, yv, ys, n, R, S);
}

__device__ inline float lp_cost(int i, int n, int R) {
  return i == n + R ? 1.0f : (i == n + R + 1 ? kBigM : 0.0f);
}

// largest steps in [0, 1] keeping v + ap dv >= 0 and z + ad dz >= 0
__device__ __forceinline__ void lp_steps(int nv, LpShared& S, float& ap, float& ad) {
  float a = 1.0f, b = 1.0f;
  for (int i = threadIdx.x; i < nv; i += kLpThreads) {
    if (S.dv[i] < 0.0f) a = fminf(a, -S.v[i] / S.dv[i]);
    if (S.dz[i] < 0.0f) b = fminf(b, -S.z[i] / S.dz[i]);
  }
  blk_min2(a, b, S);
  ap = a;
  ad = b;
}

// The right-hand side of the rank system: rank r's row plus, for every copy p on r,
// d_p times its group's row divided by beta.
__device__ __forceinline__ void lp_rank_rhs(int R, const LpRow& W, LpShared& S) {
  const int r = threadIdx.x;
  if (r < R) {
    double acc = S.rhs[r];
    for (int k = W.lo; k < W.hi; ++k) {
      const int p = S.rank_copy[k], g = S.copy_group[p];
      acc += S.d[p] * ((double)S.rhs[R + g] * S.rbeta[g]);
    }
    S.u64[r] = acc;
  }
}

// dy from the solved rank part u64: dy_r = u_r, and for group row g,
// dy = (rhs_g + sum over its copies of d_p u_(rank of p)) / beta_g
__device__ __forceinline__ void lp_dy(int R, int G, const LpRow& W, LpShared& S) {
  const int i = threadIdx.x;
  if (i < R) {
    S.dy[i] = (float)S.u64[i];
  } else if (i < R + G) {
    double acc = S.rhs[i];
    for (int p = W.lo; p < W.hi; ++p) acc += S.d[p] * S.u64[S.copy_rank[p]];
    S.dy[i] = (float)(acc * S.rbeta[i - R]);
  }
}

// lp_steps, and in the same pass the sums that expand the affine complementarity
// sum_i (v_i + ap dv_i)(z_i + ad dz_i) = vz + ap dvz + ad vdz + ap ad dvdz (fp64 products)
__device__ __forceinline__ void lp_steps_aff(int nv, LpShared& S, float& ap, float& ad,
                                             double (&sums)[4]) {
  float a = 1.0f, b = 1.0f;
  double x[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < nv; i += kLpThreads) {
    const float v = S.v[i], z = S.z[i], dv = S.dv[i], dz = S.dz[i];
    if (dv < 0.0f) a = fminf(a, -v / dv);
    if (dz < 0.0f) b = fminf(b, -z / dz);
    x[0] += (double)v * (double)z;
    x[1] += (double)dv * (double)z;
    x[2] += (double)v * (double)dz;
    x[3] += (double)dv * (double)dz;
  }
  a = wave_min_f(a);
  b = wave_min_f(b);
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = wave_sum_d(x[j]);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    S.redf[w] = a;
    S.red[w] = b;
#pragma unroll
    for (int j = 0; j < 4; ++j) S.redn[j][w] = x[j];
  }
  __syncthreads();
  float ta = S.redf[0], tb = (float)S.red[0];
#pragma unroll
  for (int i = 1; i < kLpThreads / kWave; ++i) {
    ta = fminf(ta, S.redf[i]);
    tb = fminf(tb, (float)S.red[i]);
  }
  ap = ta;
  ad = tb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kLpThreads / kWave; ++i) t += S.redn[j][i];
    sums[j] = t;
  }
}

// dy = (A D A^T)^{-1} rhs with the factored rank matrix; returns the sum of dy's rank part
__device__ __forceinline__ double lp_solve(int n, int R, int G, const LpRow& W, LpShared& S) {
  lp_rank_rhs(R, W, S);
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    double b = l < R ? S.u64[l] : 0.0;       // padded rows solve to 0
    // L = U D^(1/2) with U unit lower triangular: U z = r1, w = D^-1 z, U^T u = w,
    // so every substitution step is one broadcast and one FMA.  P holds U's strictly
    // lower part and zeros elsewhere, so lanes outside the triangle add 0: no
    // branches, and each pass loads its 64 entries in one burst before the chain.
    const double dinv_l = S.Dinv[l];
    double u[kLpMaxR];
#pragma unroll
    for (int q = 0; q < kLpMaxR; ++q) u[q] = S.P[l][q];
#pragma unroll
    for (int q = 0; q < kLpMaxR; ++q) b = fma(-u[q], readlane_d(b, q), b);   // U z = r1
    b *= dinv_l;                                                            // w = D^-1 z
#pragma unroll
    for (int q = 0; q < kLpMaxR; ++q) u[q] = S.P[q][l];
#pragma unroll
    for (int q = kLpMaxR - 1; q >= 0; --q) b = fma(-u[q], readlane_d(b, q), b);  // U^T u = w
    if (l < R) S.u64[l] = b;
    const double ys = wave_sum_d(l < R ? b : 0.0);
    if (l == 0) S.ysum = ys;
  }
  __syncthreads();
  lp_dy(R, G, W, S);
  const double ys = S.ysum;
  __syncthreads();
  return ys;
}

// The hardware reciprocal estimate is good to about 2^-24 relative; one Newton step
// brings it to about 2^-47, far beyond what the fp32 iterates resolve.
__device__ __forceinline__ double rcp_d(double x) {
  const double y = __builtin_amdgcn_rcp(x);
  return fma(y, fma(-x, y, 1.0), y);
}

// d = v / z (the diagonal of the normal equations); for every group g, 1 / beta_g with
// beta_g the sum of its copies' d; for every copy p of g, cd_p = d_p * (the sum of the
// other copies' d) / beta_g, its share of its rank's diagonal (a sum of positive terms:
// no cancellation).  One thread per copy sums its group in index order, so every copy
// of a group forms the same beta.  Returns the dense coefficient delta = d_M + d_a of
// the rank matrix's 11^T term.
__device__ __forceinline__ double lp_scaling(int n, int R, int G, LpShared& S) {
  const int nv = n + R + 2;
  for (int i = threadIdx.x; i < nv; i += kLpThreads) S.d[i] = (double)S.v[i] / (double)S.z[i];
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += kLpThreads) {
    const int g = S.copy_group[p], q0 = S.grp_start[g], q1 = S.grp_start[g + 1];
    double b = 0.0, others = 0.0;
    for (int q = q0; q < q1; ++q) {
      const double dq = S.d[q];
      b += dq;
      if (q != p) others += dq;
    }
    const double rb = rcp_d(b);
    S.cd[p] = S.d[p] * (others * rb);
    if (p == q0) S.rbeta[g] = rb;
  }
  return S.d[n + R] + S.d[n + R + 1];
}

// rank r's diagonal entry of the rank matrix without the dense term: its slack's d plus
// cd of every copy on r
__device__ __forceinline__ double lp_rank_diag(int n, int r, const LpShared& S) {
  double diag = S.d[n + r];
  for (int k = S.rank_start[r]; k < S.rank_start[r + 1]; ++k) diag += S.cd[S.rank_copy[k]];
  return diag;
}

// One off-diagonal entry of the rank matrix (r > r') as the thread that forms it every
// iteration keeps it: its position, and the first of the pairs of copies of one group on
// r and r' that it sums, with that pair's group, held in registers (the structure is
// constant over the solve); further pairs are read from the structure.
struct LpEnt {
  int e;                 // entry index, -1: the thread has none
  int rr;                // r * 64 + r'
  int l1, l2;            // the lanes of r and r' in the block solve
  int p, q, gp;          // first pair and the group of p
  int k1, k_end;         // remaining pairs [k1, k_end)
};

__device__ __forceinline__ LpEnt lp_ent_load(int e, const LpView& L, const LpShared& S) {
  LpEnt c;
  c.e = e < L.n_ent ? e : -1;
  if (c.e < 0) return c;
  c.rr = L.ent_rr[e];
  c.l1 = L.rank_lane[c.rr / kLpMaxR];
  c.l2 = L.rank_lane[c.rr % kLpMaxR];
  const int k0 = L.ent_start[e];
  c.k_end = L.ent_start[e + 1];
  c.k1 = k0 + 1;
  c.p = L.ent_p[k0];
  c.q = L.ent_q[k0];
  c.gp = S.copy_group[c.p];
  return c;
}

// the entry is -off: sum over its pairs of d_p d_q / beta
__device__ __forceinline__ double lp_entry_off(const LpEnt& c, const LpView& L, const LpShared& S) {
  double off = S.d[c.p] * (S.d[c.q] * S.rbeta[c.gp]);
  for (int k = c.k1; k < c.k_end; ++k) {
    const int p = L.ent_p[k], q = L.ent_q[k];
    off += S.d[p] * (S.d[q] * S.rbeta[S.copy_group[p]]);
  }
  return off;
}

__device__ __forceinline__ void lp_factor(int n, int R, int G, const LpView& L, const LpEnt& C,
                                          LpShared& S) {
  const double delta = lp_scaling(n, R, G, S);
  // every entry starts at the dense M/a term; the matrix is padded to 64 x 64 with
  // identity rows and columns beyond R so the factorization has no bounds tests
  for (int idx = threadIdx.x; idx < kLpMaxR * kLpMaxR; idx += kLpThreads) {
    const int r = idx / kLpMaxR, c = idx % kLpMaxR;
    S.P[r][c] = (r < R && c < R) ? delta : (r == c ? 1.0 : 0.0);
  }
  for (int r = R + threadIdx.x; r < kLpMaxR; r += kLpThreads) S.d0[r] = 1.0;
  __syncthreads();
  // diagonal: slack term plus each copy's cd
  for (int r = threadIdx.x; r < R; r += kLpThreads) {
    const double diag = delta + lp_rank_diag(n, r, S);
    S.P[r][r] = diag;
    S.d0[r] = diag;
  }
  // off-diagonal entries touched by copies of one group on both ranks
  for (int e = threadIdx.x; e < L.n_ent; e += kLpThreads) {
    const LpEnt c = e == (int)threadIdx.x ? C : lp_ent_load(e, L, S);
    S.P[c.rr / kLpMaxR][c.rr % kLpMaxR] = delta - lp_entry_off(c, L, S);
  }
  __syncthreads();
  // Blocked right-looking LDL^T (Cholesky without square roots), panels of kLpPanel
  // columns.  Thread (ti, tk) keeps a 4x4 register tile of the trailing matrix: rows
  // i = ti + 16a, columns k = tk + 16b.  For each panel: the tiles of the panel's
  // columns are published to LDS; wave 0 factors the 64 x kLpPanel panel with one row
  // per lane and stores the unit lower factor U (U_ic = a_ic / p_c strictly below the
  // diagonal, zeros elsewhere), the pivots p_c and 1/p_c; then every thread subtracts
  // the panel's product from the trailing entries of its tile, U_ij (U_kj p_j).  In
  // the panel the unscaled column entries a_kc are broadcast (readlane) while the
  // pivot's reciprocal is still being formed, so a column's dependent chain is one
  // broadcast, the reciprocal, one multiply and one FMA.  The panel width trades wave
  // 0's serial broadcasts against barriers: 16 columns measured best on MI355X (4 and 8
  // slower by 6% and 1%).  A pivot that lost its
  // precision (p_c <= tol * original diagonal) drops its direction: its column of U
  // is 0 and 1/p_c is replaced by 1e-64.
  const int ti = threadIdx.x / 16, tk = threadIdx.x % 16;
  double* piv = S.colbuf[0];
  double A[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) A[a][b] = S.P[ti + 16 * a][tk + 16 * b];
  __syncthreads();
#pragma unroll
  for (int pb = 0; pb < kLpMaxR / kLpPanel; ++pb) {
    const int c0 = kLpPanel * pb, c1 = c0 + kLpPanel;
    const int bb = c0 / 16, k0 = c0 % 16;
    if (tk >= k0 && tk < k0 + kLpPanel) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (16 * a + 15 >= c0) S.P[ti + 16 * a][tk + 16 * bb] = A[a][bb];
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // the lane index is re-read per panel (empty asm, no instruction) so the 64
      // lane-vs-column compares stay inside the loop instead of being hoisted out of
      // the interior-point loop as 64 live masks
      int l = threadIdx.x;
      asm volatile("" : "+v"(l));
      double r[kLpPanel], thr[kLpPanel];
#pragma unroll
      for (int j = 0; j < kLpPanel; ++j) {
        r[j] = S.P[l][c0 + j];
        thr[j] = kPivTol * S.d0[c0 + j];
      }
      double my_piv = 0.0, my_dinv = 0.0;
#pragma unroll
      for (int j = 0; j < kLpPanel; ++j) {
        const int c = c0 + j;
        const double pj = readlane_d(r[j], c);
        double akc[kLpPanel];                                // a_kc of the panel's later rows
#pragma unroll
        for (int j2 = j + 1; j2 < kLpPanel; ++j2) akc[j2] = readlane_d(r[j], c0 + j2);
        const bool bad = !(pj > thr[j]);
        const double rc = bad ? 0.0 : rcp_d(pj);
        if (l == c) {
          my_piv = pj;
          my_dinv = bad ? 1e-64 : rc;
        }
        const double u = l > c ? r[j] * rc : 0.0;           // U_lc (0 on and above)
        S.P[l][c] = u;
#pragma unroll
        for (int j2 = j + 1; j2 < kLpPanel; ++j2) r[j2] = fma(-u, akc[j2], r[j2]);
      }
      if (l >= c0 && l < c1) {
        piv[l] = my_piv;
        S.Dinv[l] = my_dinv;
      }
    }
    __syncthreads();
    if (c1 < kLpMaxR) {
#pragma unroll
      for (int j = 0; j < kLpPanel; ++j) {
        const double pj = piv[c0 + j];
        double ui[4], uk[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) ui[a] = 16 * a + 15 >= c1 ? S.P[ti + 16 * a][c0 + j] : 0.0;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) uk[b2] = 16 * b2 + 15 >= c1 ? S.P[tk + 16 * b2][c0 + j] * pj : 0.0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b2 = 0; b2 < 4; ++b2)
            if (16 * a + 15 >= c1 && 16 * b2 + 15 >= c1 && ti + 16 * a >= c1 && tk + 16 * b2 >= c1)
              A[a][b2] = fma(-ui[a], uk[b2], A[a][b2]);
      }
    }
  }
}

// ---- block solve of the rank matrix P = B + delta 11^T ---------------------------
// B (P without its dense term) is block diagonal over the components of the rank
// coupling graph, packed into groups of kBlk lanes (lane_rank).  Every group factors
// its block as U diag(p) U^T in registers, one row per lane, the rows broadcast within
// the group by DPP moves; all groups at once.  A solve is then one forward and one
// backward substitution per group and the rank-one correction of Sherman-Morrison:
// P^-1 b = v - w (delta 1^T v) / (1 + delta 1^T w), v = B^-1 b, w = B^-1 1, both fp64.
// Pivots that lost their precision are dropped as in the dense factorization.

// Lane J of every aligned group of kBlk (8 or 16) lanes, to every lane of its group, by
// DPP moves (no trip through the LDS unit).  row_newbcast:N (DPP control 0x150 + N,
// gfx90a and later) gives every lane of a 16-lane row the row's lane N: one move for
// groups of 16; groups of 8 take lane J of the row, then, in banks 2 and 3 (the upper
// 8 lanes), lane 8 + J.
template <int kBlk, int J>
__device__ __forceinline__ int grp_bcast_i(int x) {
  static_assert(kBlk == 8 || kBlk == 16, "groups of 8 or 16 lanes");
  const int r = __builtin_amdgcn_mov_dpp(x, 0x150 + J, 0xF, 0xF, false);
  if constexpr (kBlk == 16) return r;
  return __builtin_amdgcn_update_dpp(r, x, 0x150 + 8 + J, 0xF, 0xC, false);
}

template <int kBlk, int J>
__device__ __forceinline__ double grp_bcast_j(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = grp_bcast_i<kBlk, J>((int)(uint32_t)u);
  const int hi = grp_bcast_i<kBlk, J>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// the same with j a loop index of a fully unrolled loop (the switch folds away)
template <int kBlk>
__device__ __forceinline__ double grp_bcast(double v, int j) {
  switch (j) {
    case 0: return grp_bcast_j<kBlk, 0>(v);
    case 1: return grp_bcast_j<kBlk, 1>(v);
    case 2: return grp_bcast_j<kBlk, 2>(v);
    case 3: return grp_bcast_j<kBlk, 3>(v);
    case 4: return grp_bcast_j<kBlk, 4>(v);
    case 5: return grp_bcast_j<kBlk, 5>(v);
    case 6: return grp_bcast_j<kBlk, 6>(v);
    case 7: return grp_bcast_j<kBlk, 7>(v);
  }
  if constexpr (kBlk == 16) {
    switch (j) {
      case 8: return grp_bcast_j<kBlk, 8>(v);
      case 9: return grp_bcast_j<kBlk, 9>(v);
      case 10: return grp_bcast_j<kBlk, 10>(v);
      case 11: return grp_bcast_j<kBlk, 11>(v);
      case 12: return grp_bcast_j<kBlk, 12>(v);
      case 13: return grp_bcast_j<kBlk, 13>(v);
      case 14: return grp_bcast_j<kBlk, 14>(v);
      default: return grp_bcast_j<kBlk, 15>(v);
    }
  }
  return v;
}

template <int kBlk>
struct LpBlk {
  double r[kBlk];        // the lane's row of its block; after factoring, U's strict lower part
  double dinv, w;        // 1 / pivot (1e-64 for a dropped pivot), and (B^-1 1) on this lane
  double s1, delta;      // sum of B^-1 1 over the ranks, and delta = d_M + d_a
  int a, base, rank;     // row in the group, the group's first lane, the rank (-1: padding)
};

// x = B_g^-1 b on the lane's group (U's columns read back from LDS for the backward pass)
template <int kBlk>
__device__ __forceinline__ double lpb_subst(const LpBlk<kBlk>& B, double b, const double* ust) {
  double z = b;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) {                      // U z = b
    const double zj = grp_bcast<kBlk>(z, j);
    if (B.a > j) z = fma(-B.r[j], zj, z);
  }
  z *= B.dinv;
  double uc[kBlk];
#pragma unroll
  for (int j = 0; j < kBlk; ++j) uc[j] = ust[(B.base + j) * kBlk + B.a];
#pragma unroll
  for (int j = kBlk - 1; j >= 0; --j) {                 // U^T x = D^-1 z
    const double xj = grp_bcast<kBlk>(z, j);
    if (B.a < j) z = fma(-uc[j], xj, z);
  }
  return z;
}

template <int kBlk>
__device__ __forceinline__ void lpb_factor(LpBlk<kBlk>& B, int n, int R, int G, const LpView& L,
                                           const LpEnt& C, LpShared& S) {
  double* ust = &S.P[0][0];                 // kLpLanes rows of kBlk entries
  const int t = threadIdx.x;
  // every lane clears its own row (the last solve's reads of U ended at a barrier)
#pragma unroll
  for (int b = 0; b < kBlk; ++b) ust[t * kBlk + b] = 0.0;
  B.delta = lp_scaling(n, R, G, S);
  __syncthreads();                          // cd, 1 / beta and the cleared rows complete
  if (B.rank >= 0) ust[t * kBlk + B.a] = lp_rank_diag(n, B.rank, S);
  else ust[t * kBlk + B.a] = 1.0;
  for (int e = t; e < L.n_ent; e += kLpThreads) {
    const LpEnt c = e == t ? C : lp_ent_load(e, L, S);
    const double off = -lp_entry_off(c, L, S);
    ust[c.l1 * kBlk + c.l2 % kBlk] = off;
    ust[c.l2 * kBlk + c.l1 % kBlk] = off;
  }
  __syncthreads();
  double d0 = 0.0;
#pragma unroll
  for (int b = 0; b < kBlk; ++b) {
    B.r[b] = ust[t * kBlk + b];
    if (b == B.a) d0 = B.r[b];
  }
  B.dinv = 0.0;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) {
    const double pj = grp_bcast<kBlk>(B.r[j], j);
    const double thr = kPivTol * grp_bcast<kBlk>(d0, j);
    double ajb[kBlk];
#pragma unroll
    for (int b = j + 1; b < kBlk; ++b) ajb[b] = grp_bcast<kBlk>(B.r[b], j);
    const bool bad = !(pj > thr);
    const double rc = bad ? 0.0 : rcp_d(pj);
    if (B.a == j) B.dinv = bad ? 1e-64 : rc;
    if (B.a > j) {
      const double u = B.r[j] * rc;
      B.r[j] = u;
#pragma unroll
      for (int b = j + 1; b < kBlk; ++b) B.r[b] = fma(-u, ajb[b], B.r[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < kBlk; ++b) ust[t * kBlk + b] = b < B.a ? B.r[b] : 0.0;
  __syncthreads();
  B.w = lpb_subst<kBlk>(B, B.rank >= 0 ? 1.0 : 0.0, ust);
  B.s1 = blk_sum(B.rank >= 0 ? B.w : 0.0, S);
}

// dy = (A D A^T)^{-1} rhs with the block factors (the group rows as in lp_solve); returns
// the sum of dy's rank part, sum(v) - sum(w) c by the same correction
template <int kBlk>
__device__ __forceinline__ double lpb_solve(const LpBlk<kBlk>& B, int n, int R, int G,
                                            const LpRow& W, LpShared& S) {
  lp_rank_rhs(R, W, S);
  __syncthreads();
  const double v = lpb_subst<kBlk>(B, B.rank >= 0 ? S.u64[B.rank] : 0.0, &S.P[0][0]);
  const double sv = blk_sum(B.rank >= 0 ? v : 0.0, S);
  const double c = B.delta * sv / (1.0 + B.delta * B.s1);
  const double y = v - B.w * c;
  if (B.rank >= 0) S.u64[B.rank] = y;
  __syncthreads();
  lp_dy(R, G, W, S);
  __syncthreads();
  return sv - B.s1 * c;
}

// The interior-point loop: Mehrotra predictor-corrector from the starting point in S,
// at most `iters` steps; kBlk = 0 factors the rank matrix densely, kBlk = 8 or 16 uses
// the block solve over lane groups of that size.  Returns the number of steps run.
template <int kBlk>
__device__ __forceinline__ int lp_ipm(int iters, int n, int R, int G, const LpView& L,
                                      LpShared& S) {
  const int nv = n + R + 2;
  const int tid = threadIdx.x;
  int run = 0;
  LpBlk<(kBlk > 0 ? kBlk : 1)> B;
  if constexpr (kBlk > 0) {
    B.a = tid % kBlk;
    B.base = tid - B.a;
    B.rank = L.lane_rank[tid];
  }
  // Barriers below separate only accesses across threads: a loop over i that reads
  // what the same thread wrote at index i in the step before needs none.
  const auto plus_rb = [&](int i, float a) { return a + S.rb[i]; };
  const LpEnt C = lp_ent_load(tid, L, S);
  const LpRow W = lp_row(R, G, S);
  for (int it = 0; it < iters; ++it) {
    // residuals and complementarity: rb = b - A v, rc = c - A^T y - z
    lp_Av([&](int j) { return S.v[j]; },
          [&](int i, float a) { return (i < R ? S.f[i] : S.hh[i - R]) - a; }, S.rb, n, R, G, W, S);
    // the duality gap and the sum of the rank duals in one reduction
    double gy[2] = {0.0, 0.0};
    for (int i = tid; i < nv; i += kLpThreads) gy[0] += (double)(S.v[i] * S.z[i]);
    {
      float part = 0.0f;
      for (int r = tid; r < R; r += kLpThreads) part += S.y[r];
      gy[1] = part;
    }
    blk_sum_n<2>(gy, S);
    const double gap = gy[0];
    const float ys = (float)gy[1];
    for (int i = tid; i < nv; i += kLpThreads)
      S.rc[i] = lp_cost(i, n, R) - lp_ATy_at(i, S.y, ys, n, R, S) - S.z[i];
    const float mu = (float)(gap / nv);
    // stop once the duality gap, which bounds the objective error of a feasible
    // iterate, is below kGapRel of the objective (fp32 iterates gain nothing beyond)
    if (!(mu >= kMuStop) || gap <= kGapRel * fmax(1.0, (double)S.v[n + R])) break;
    ++run;
    if constexpr (kBlk > 0) lpb_factor<kBlk>(B, n, R, G, L, C, S);
    else lp_factor(n, R, G, L, C, S);
    // predictor: rhs = rb + A (v + D rc), the vector formed inside the product
    lp_Av([&](int j) { return S.v[j] + (float)(S.d[j] * S.rc[j]); }, plus_rb, S.rhs, n, R, G, W, S);
    __syncthreads();
    double dys;
    if constexpr (kBlk > 0) dys = lpb_solve<kBlk>(B, n, R, G, W, S);
    else dys = lp_solve(n, R, G, W, S);
    for (int i = tid; i < nv; i += kLpThreads) {
      S.dz[i] = S.rc[i] - lp_ATy_at(i, S.dy, (float)dys, n, R, S);
      S.dv[i] = -S.v[i] - (float)(S.d[i] * S.dz[i]);
    }
    float ap, ad;
    double sums[4];
    lp_steps_aff(nv, S, ap, ad, sums);
    const double ca = sums[0] + (double)ap * sums[1] + (double)ad * sums[2] +
                      (double)ap * (double)ad * sums[3];
    const float mu_aff = (float)(fmax(ca, 0.0) / nv);
    const float ratio = mu_aff / mu;
    const float sg = ratio * ratio * ratio;
    // corrector: rmu = sg mu - v z - dv dz ; rhs = rb + A (D rc - rmu / z)
    for (int i = tid; i < nv; i += kLpThreads) {
      const float rmu = sg * mu - S.v[i] * S.z[i] - S.dv[i] * S.dz[i];
      S.dv[i] = rmu;                       // keep rmu in dv until the new direction
      S.tv[i] = (float)(S.d[i] * S.rc[i]) - rmu / S.z[i];
    }
    __syncthreads();
    lp_Av([&](int j) { return S.tv[j]; }, plus_rb, S.rhs, n, R, G, W, S);
    __syncthreads();
    if constexpr (kBlk > 0) dys = lpb_solve<kBlk>(B, n, R, G, W, S);
    else dys = lp_solve(n, R, G, W, S);
    for (int i = tid; i < nv; i += kLpThreads) {
      const float rmu = S.dv[i];
      S.dz[i] = S.rc[i] - lp_ATy_at(i, S.dy, (float)dys, n, R, S);
      S.dv[i] = rmu / S.z[i] - (float)(S.d[i] * S.dz[i]);
    }
    float ap2, ad2;
    lp_steps(nv, S, ap2, ad2);
    for (int i = tid; i < nv; i += kLpThreads) {
      S.v[i] += kEta * ap2 * S.dv[i];
      S.z[i] += kEta * ad2 * S.dz[i];
    }
    for (int i = tid; i < R + G; i += kLpThreads) S.y[i] += kEta * ad2 * S.dy[i];
    __syncthreads();
  }
  return run;
}

// The whole LP solve for one 256-thread workgroup whose LDS state is S (lplb_kernel's,
// or block 0's in the fused plan launch).
__device__ __forceinline__ void lplb_body(LpShared& S, const int32_t* __restrict__ counts,
                                          const int32_t* __restrict__ lpw, int iters,
                                          float* __restrict__ x_out, float* __restrict__ m_out,
                                          int32_t* __restrict__ inst_quota,
                                          int32_t* __restrict__ stats, int32_t* err) {
  // a buffer that is not a structure from uep_lplb_prepare (or sizes beyond the LDS
  // tables) is refused whole: nothing but the error word is written
  if (lpw[0] != kLpMagic || lpw[1] < 1 || lpw[1] > kLpMaxR || lpw[2] < 1 || lpw[2] > kLpMaxE ||
      lpw[3] < 1 || lpw[4] != lpw[1] * lpw[3] || lpw[4] > kLpMaxI || lpw[5] < 0 ||
      lpw[5] > kLpMaxG || lpw[6] < 0 || lpw[6] > kLpMaxN || lpw[7] < 0) {
    if (threadIdx.x == 0) set_err(err, UEP_ERR_LP);
    return;
  }
  const LpView L = lp_view(lpw);
  if (L.blk != 0 && L.blk != 8 && L.blk != 16) {
    if (threadIdx.x == 0) set_err(err, UEP_ERR_LP);
    return;
  }
  const int R = L.R, E = L.E, G = L.G, n = L.n, nv = n + R + 2;
  const int tid = threadIdx.x;

  for (int i = tid; i <= G; i += kLpThreads) S.grp_start[i] = L.grp_start[i];
  for (int i = tid; i < n; i += kLpThreads) {
    S.copy_rank[i] = L.copy_rank[i];
    S.copy_group[i] = L.copy_group[i];
    S.rank_copy[i] = L.rank_copy[i];
  }
  for (int i = tid; i <= R; i += kLpThreads) S.rank_start[i] = L.rank_start[i];
  for (int r = tid; r < R; r += kLpThreads) S.Fi[r] = 0;
  __syncthreads();
  // expert loads (column sums of the load matrix): fixed load per rank, count per group
  int bad = 0;
  for (int e = tid; e < E; e += kLpThreads) {
    const int c = column_sum(counts, R, E, e);
    const int i = L.exp_inst[e];
    if (c > 0 && i == -1) bad |= UEP_ERR_LP;
    if (c >= (1 << 27)) bad |= UEP_ERR_LP;
    if (i >= 0) atomicAdd(&S.Fi[i / L.ipr], c);       // integer: exact in any order
    else if (i <= -2) S.hc[-2 - i] = c;
  }
  if (bad) set_err(err, bad);
  __syncthreads();
  double part = 0.0;
  for (int r = tid; r < R; r += kLpThreads) part += S.Fi[r];
  for (int g = tid; g < G; g += kLpThreads) part += S.hc[g];
  const double total = blk_sum(part, S);
  const double sigma = fmax(1.0, total / R);
  for (int r = tid; r < R; r += kLpThreads) S.f[r] = (float)(S.Fi[r] / sigma);
  for (int g = tid; g < G; g += kLpThreads) {
    S.hh[g] = (float)(S.hc[g] / sigma);
    S.cnt_i[g] = S.grp_start[g + 1] - S.grp_start[g];
  }
  __syncthreads();

  int run = 0;
  if (G > 0) {
    // starting point: balanced split, slacks >= 1, a = 1; duals y_r = 0.5 / R
    for (int p = tid; p < n; p += kLpThreads) {
      const int g = S.copy_group[p];
      S.tv[p] = S.hh[g] / (float)S.cnt_i[g];
    }
    __syncthreads();
    float lmax = -1e30f;
    for (int r = tid; r < R; r += kLpThreads) {
      float ld = S.f[r];
      for (int k = S.rank_start[r]; k < S.rank_start[r + 1]; ++k) ld += S.tv[S.rank_copy[k]];
      S.rb[r] = ld;
      lmax = fmaxf(lmax, ld);
    }
    const float M0 = -blk_min(-lmax, S);
    for (int i = tid; i < nv; i += kLpThreads) {
      float val;
      if (i < n) val = S.tv[i] + 0.1f;
      else if (i < n + R) val = M0 - S.rb[i - n] + 1.0f;
      else if (i == n + R) val = M0;
      else val = 1.0f;
      S.v[i] = val;
    }
    for (int i = tid; i < R + G; i += kLpThreads) S.y[i] = i < R ? 0.5f / R : 0.0f;
    __syncthreads();
    lp_ATy(S.y, S.tv, n, R, G, S);
    __syncthreads();
    for (int i = tid; i < nv; i += kLpThreads) S.z[i] = fmaxf(lp_cost(i, n, R) - S.tv[i], 0.0f) + 1.0f;
    __syncthreads();

    if (L.blk == 8) run = lp_ipm<8>(iters, n, R, G, L, S);
    else if (L.blk == 16) run = lp_ipm<16>(iters, n, R, G, L, S);
    else run = lp_ipm<0>(iters, n, R, G, L, S);
  }

  // split: clip, scale back, normalise every group to its count
  for (int g = tid; g < G; g += kLpThreads) {
    const int p0 = S.grp_start[g], p1 = S.grp_start[g + 1];
    const int c = S.hc[g];
    double sum = 0.0;
    for (int p = p0; p < p1; ++p) sum += (double)(fmaxf(S.v[p], 0.0f) * (float)sigma);
    for (int p = p0; p < p1; ++p) {
      const double xp = (double)(fmaxf(S.v[p], 0.0f) * (float)sigma);
      S.tv[p] = sum > 0.0 ? (float)(xp * ((double)c / sum)) : (float)((double)c / (p1 - p0));
      x_out[p] = S.tv[p];
    }
  }
  __syncthreads();
  double mx = 0.0;
  for (int r = tid; r < R; r += kLpThreads) {
    double ld = S.Fi[r];
    for (int k = S.rank_start[r]; k < S.rank_start[r + 1]; ++k) ld += S.tv[S.rank_copy[k]];
    mx = fmax(mx, ld);
  }
  {
    float mxf = (float)mx;
    mxf = -blk_min(-mxf, S);
    if (tid == 0) m_out[0] = mxf;
  }
  // integer quotas: single-copy instances take the whole load, copies by largest remainder
  for (int i = tid; i < L.I; i += kLpThreads) {
    const int e = L.inst_expert[i];
    if (e < 0) { inst_quota[i] = 0; continue; }
    if (L.inst_copy[i] < 0) {
      inst_quota[i] = column_sum(counts, R, E, e);
      continue;
    }
    const int p = L.inst_copy[i], g = S.copy_group[p];
    const int p0 = S.grp_start[g], p1 = S.grp_start[g + 1];
    const int64_t c = S.hc[g];
    int64_t W = 0;
    for (int q = p0; q < p1; ++q) W += (int64_t)rint((double)fmaxf(S.tv[q], 0.0f) * 256.0);
    int64_t q_mine;
    if (W == 0) {
      const int k = p - p0, cnt = p1 - p0;
      q_mine = c / cnt + (k < c % cnt ? 1 : 0);
    } else {
      int64_t base_sum = 0;
      const int64_t wp = (int64_t)rint((double)fmaxf(S.tv[p], 0.0f) * 256.0);
      const int64_t rem_p = (c * wp) % W;
      int rank_of_p = 0;                    // copies ahead of p in (remainder desc, index asc)
      for (int q = p0; q < p1; ++q) {
        const int64_t wq = (int64_t)rint((double)fmaxf(S.tv[q], 0.0f) * 256.0);
        base_sum += (c * wq) / W;
        const int64_t rem_q = (c * wq) % W;
        rank_of_p += (rem_q > rem_p) || (rem_q == rem_p && q < p);
      }
      const int64_t left = c - base_sum;
      q_mine = (c * wp) / W + (rank_of_p < left ? 1 : 0);
    }
    inst_quota[i] = (int32_t)q_mine;
  }
  if (tid == 0 && stats) {
    stats[0] = G;
    stats[1] = n;
    stats[2] = run;
    stats[3] = L.blk;
  }
}

__global__ __launch_bounds__(kLpThreads) void lplb_kernel(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ lpw,
                                                          int iters, float* __restrict__ x_out,
                                                          float* __restrict__ m_out,
                                                          int32_t* __restrict__ inst_quota,
                                                          int32_t* __restrict__ stats,
                                                          int32_t* err) {
  __shared__ LpShared S;                    // static LDS: no dynamic-base lookups
  lplb_body(S, counts, lpw, iters, x_out, m_out, inst_quota, stats, err);
}

// Fused LPLB plan launch: block 0 solves the LP on the load matrix the launches before
// it wrote (the LP needs the counts only), while blocks 1.. rank the chunks as lm_rank
// does, in the same static LDS block (the ranking needs less than the LP's state).  The
// LP is one workgroup's chain of iterations, several times longer than the ranking, so
// the ranking costs the plan no time of its own.
template <int kMaxK, bool kTile>
__global__ __launch_bounds__(kLpThreads) void lplb_rank_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ bucket_pos,
    const int32_t* __restrict__ chunk_hist, int32_t* err, LmGeom g, bool vec, bool scanned,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ lpw, int iters,
    float* __restrict__ x_out, float* __restrict__ m_out, int32_t* __restrict__ inst_quota,
    int32_t* __restrict__ stats) {
  __shared__ LpShared S;
  if (blockIdx.x == 0) {
    lplb_body(S, counts, lpw, iters, x_out, m_out, inst_quota, stats, err);
    return;
  }
  const int b = (int)blockIdx.x - 1;
  lm_rank_body<kMaxK, kTile, false>(ids, bucket_pos, chunk_hist, nullptr, err, g, vec, scanned,
                                    b % g.n_chunks, b / g.n_chunks,
                                    reinterpret_cast<uint64_t*>(&S));
}

// LPLB's per-token copy draw (section "从LP解决方案到Token调度": the split,
// normalised per replicated expert, is a distribution over its physical copies from
// which every token routed to that expert draws one; a single-copy expert keeps its
// only instance).  Weights are the integers w_p = rint(max(x_p, 0) * 256) of the
// quota step; the draw for slot k of global token g is word k mod 4 of Philox4x64-10
// at counter (g, k div 4, 1, 0), key (seed, layer), scaled by a 64x64->128-bit
// product, so the choice is exact integer arithmetic and one block of the generator
// serves four slots.
//
// Each workgroup first stages the small tables in LDS (expert -> instance or group,
// the groups' running copy weights and the copies' instances), then walks quads of
// four consecutive slots of one token (one thread per quad, grid-stride): one Philox
// block per quad, every lookup after the id load an LDS read, and ids and results
// moved as 16-byte vectors when K % 4 == 0.
constexpr int kLsThreads = 256;
constexpr int kLsMaxBlocks = 2048;          // 8 workgroups per CU of a 256-CU device

__device__ __forceinline__ uint64_t copy_weight(float x) {
  return (uint64_t)rintf(fmaxf(x, 0.0f) * 256.0f);
}

struct LsShared {
  int32_t ei[kLpMaxE];                      // exp_inst: instance, -2 - group, or -1
  uint64_t cw[kLpMaxN];                     // running weight of copies within their group
  int32_t ci[kLpMaxN];                      // copy -> instance
  int32_t gs[kLpMaxG + 1];                  // group -> first copy
};

__global__ __launch_bounds__(kLsThreads) void lplb_sample_kernel(const int32_t* __restrict__ ids,
                                                                 int64_t n_tok, int K, int R,
                                                                 const int32_t* __restrict__ lpw,
                                                                 const float* __restrict__ x,
                                                                 uint64_t seed, uint64_t layer,
                                                                 int32_t* __restrict__ dest_inst,
                                                                 int32_t* err, bool vec) {
  __shared__ LsShared S;
  const int qpt = (K + 3) / 4;                           // quads per token
  const int64_t n_quad = n_tok * qpt;
  // a structure for other ranks, or sizes beyond the LDS tables, is refused whole
  if (lpw[0] != kLpMagic || lpw[1] != R || lpw[2] < 1 || lpw[2] > kLpMaxE || lpw[5] < 0 ||
      lpw[5] > kLpMaxG || lpw[6] < 0 || lpw[6] > kLpMaxN) {
    for (int64_t q = (int64_t)blockIdx.x * kLsThreads + threadIdx.x; q < n_quad;
         q += (int64_t)gridDim.x * kLsThreads) {
      const int64_t g = q / qpt;
      const int k0 = (int)(q % qpt) * 4;
      for (int k = k0; k < min(K, k0 + 4); ++k) dest_inst[g * K + k] = -1;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) set_err(err, UEP_ERR_LP);
    return;
  }
  const LpView L = lp_view(lpw);
  for (int e = threadIdx.x; e < L.E; e += kLsThreads) S.ei[e] = L.exp_inst[e];
  for (int c = threadIdx.x; c < L.n; c += kLsThreads) {
    S.cw[c] = copy_weight(x[c]);
    S.ci[c] = L.copy_inst[c];
  }
  for (int g = threadIdx.x; g <= L.G; g += kLsThreads) S.gs[g] = L.grp_start[g];
  __syncthreads();
  for (int g = threadIdx.x; g < L.G; g += kLsThreads) {
    uint64_t run = 0;
    for (int c = S.gs[g]; c < S.gs[g + 1]; ++c) {
      run += S.cw[c];
      S.cw[c] = run;
    }
  }
  __syncthreads();
  int bad = 0;
  for (int64_t q = (int64_t)blockIdx.x * kLsThreads + threadIdx.x; q < n_quad;
       q += (int64_t)gridDim.x * kLsThreads) {
    const int64_t g = q / qpt;
    const int k0 = (int)(q % qpt) * 4;
    const int64_t j0 = g * K + k0;
    int e[4], out[4];
    if (vec) {
      const int4 v = *reinterpret_cast<const int4*>(ids + j0);
      e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = k0 + u < K ? ids[j0 + u] : -1;
    }
    int grp[4];                                        // group of a slot that draws, or -1
    bool draw = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      out[u] = -1;
      grp[u] = -1;
      if (e[u] >= L.E || e[u] < -1) {
        bad |= UEP_ERR_ID_RANGE;
      } else if (e[u] >= 0) {
        const int ei = S.ei[e[u]];
        if (ei >= 0) out[u] = ei;
        else if (ei == -1) bad |= UEP_ERR_LP;
        else grp[u] = -2 - ei;
        draw |= grp[u] >= 0;
      }
    }
    if (draw) {
      uint64_t r[4];
      philox4x64_10((uint64_t)g, (uint64_t)(k0 / 4), 1, 0, seed, layer, r);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (grp[u] < 0) continue;
        const int c0 = S.gs[grp[u]], c1 = S.gs[grp[u] + 1];
        const uint64_t W = S.cw[c1 - 1];
        int pick = c0;
        if (W == 0) {
          pick = c0 + (int)__umul64hi(r[u], (uint64_t)(c1 - c0));
        } else {
          const uint64_t v = __umul64hi(r[u], W);
          while (pick < c1 - 1 && S.cw[pick] <= v) ++pick;
        }
        out[u] = S.ci[pick];
      }
    }
    if (vec) {
      *reinterpret_cast<int4*>(dest_inst + j0) = make_int4(out[0], out[1], out[2], out[3]);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k0 + u < K) dest_inst[j0 + u] = out[u];
    }
  }
  if (bad) set_err(err, bad);
}

}  // namespace uep

using namespace uep;

extern "C" size_t uep_lplb_struct_size(int32_t R, int32_t E, int32_t inst_per_rank) {
  if (R <= 0 || E <= 0 || inst_per_rank <= 0) return 0;
  const int I = R * inst_per_rank;
  // at most I copies; each copy pairs with at most one copy per other rank
  const int n_pair = I * (R - 1);
  return sizeof(int32_t) * lp_words(R, E, I, E, I, R * R, n_pair);
}

extern "C" uep_status uep_lplb_prepare(const int32_t* ie, int32_t R, int32_t E,
                                       int32_t inst_per_rank, void* lp, size_t lp_bytes,
                                       void* stream) {
  if (R <= 0 || E <= 0 || inst_per_rank <= 0 || !ie || !lp) return UEP_EINVAL;
  const int I = R * inst_per_rank;
  if (R > kLpMaxR || E > kLpMaxE || I > kLpMaxI) return UEP_EGEOM;
  if (lp_bytes < uep_lplb_struct_size(R, E, inst_per_rank)) return UEP_EWORKSPACE;
  std::vector<std::vector<int>> inst_of(E);
  for (int i = 0; i < I; ++i) {
    const int e = ie[i];
    if (e < -1 || e >= E) return UEP_EINVAL;
    if (e >= 0) inst_of[e].push_back(i);
  }
  std::vector<int> grp_expert, grp_start{0}, copy_inst, copy_rank, copy_group;
  std::vector<int> exp_inst(E, -1), inst_copy(I, -1);
  for (int e = 0; e < E; ++e) {
    const auto& v = inst_of[e];
    for (size_t a = 0; a < v.size(); ++a)
      for (size_t b = a + 1; b < v.size(); ++b)
        if (v[a] / inst_per_rank == v[b] / inst_per_rank) return UEP_EINVAL;
    if (v.size() == 1) exp_inst[e] = v[0];
    if (v.size() >= 2) {
      const int g = (int)grp_expert.size();
      exp_inst[e] = -2 - g;
      grp_expert.push_back(e);
      for (int i : v) {
        inst_copy[i] = (int)copy_inst.size();
        copy_inst.push_back(i);
        copy_rank.push_back(i / inst_per_rank);
        copy_group.push_back(g);
      }
      grp_start.push_back((int)copy_inst.size());
    }
  }
  const int G = (int)grp_expert.size(), n = (int)copy_inst.size();
  if (G > kLpMaxG || n > kLpMaxN) return UEP_EGEOM;
  // lower off-diagonal entries of the rank matrix and the copy pairs that form them
  std::vector<std::vector<std::pair<int, int>>> ent(R * kLpMaxR);
  for (int g = 0; g < G; ++g)
    for (int p = grp_start[g]; p < grp_start[g + 1]; ++p)
      for (int q = grp_start[g]; q < grp_start[g + 1]; ++q)
        if (copy_rank[p] > copy_rank[q]) ent[copy_rank[p] * kLpMaxR + copy_rank[q]].push_back({p, q});
  std::vector<int> ent_rr, ent_start{0}, ent_p, ent_q;
  for (int rr = 0; rr < R * kLpMaxR; ++rr) {
    if (ent[rr].empty()) continue;
    ent_rr.push_back(rr);
    for (auto& pq : ent[rr]) { ent_p.push_back(pq.first); ent_q.push_back(pq.second); }
    ent_start.push_back((int)ent_p.size());
  }
  const int n_ent = (int)ent_rr.size(), n_pair = (int)ent_p.size();
  std::vector<int> rank_start(R + 1, 0), rank_copy(n);
  for (int p = 0; p < n; ++p) rank_start[copy_rank[p] + 1]++;
  for (int r = 0; r < R; ++r) rank_start[r + 1] += rank_start[r];
  {
    std::vector<int> fill(rank_start.begin(), rank_start.end() - 1);
    for (int p = 0; p < n; ++p) rank_copy[fill[copy_rank[p]]++] = p;
  }
  // components of the rank coupling graph, packed into lane groups for the block solve
  std::vector<int> parent(R);
  for (int r = 0; r < R; ++r) parent[r] = r;
  auto find = [&](int a) {
    while (parent[a] != a) a = parent[a] = parent[parent[a]];
    return a;
  };
  for (int g = 0; g < G; ++g)
    for (int p = grp_start[g] + 1; p < grp_start[g + 1]; ++p)
      parent[find(copy_rank[p])] = find(copy_rank[grp_start[g]]);
  std::vector<std::vector<int>> comps;
  {
    std::vector<int> comp_of(R, -1);
    for (int r = 0; r < R; ++r) {
      const int root = find(r);
      if (comp_of[root] < 0) { comp_of[root] = (int)comps.size(); comps.emplace_back(); }
      comps[comp_of[root]].push_back(r);
    }
  }
  size_t biggest = 0;
  for (auto& c : comps) biggest = std::max(biggest, c.size());
  int blk = biggest <= 8 ? 8 : (biggest <= 16 ? 16 : 0);
  std::vector<int> lane_rank(kLpLanes, -1), rank_lane(R, -1);
  if (blk > 0) {
    std::vector<int> order(comps.size());
    for (size_t c = 0; c < comps.size(); ++c) order[c] = (int)c;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return comps[a].size() > comps[b].size(); });
    const int n_bins = kLpLanes / blk;
    std::vector<int> fill(n_bins, 0);
    for (int c : order) {
      int b = 0;
      while (b < n_bins && fill[b] + (int)comps[c].size() > blk) ++b;
      if (b == n_bins) { blk = 0; break; }
      for (int r : comps[c]) {
        const int l = b * blk + fill[b]++;
        lane_rank[l] = r;
        rank_lane[r] = l;
      }
    }
    if (blk == 0) std::fill(lane_rank.begin(), lane_rank.end(), -1);
  }
  const size_t words = lp_words(R, E, I, G, n, n_ent, n_pair);
  if (lp_bytes < words * sizeof(int32_t)) return UEP_EWORKSPACE;
  std::vector<int32_t> w(words, 0);
  w[0] = kLpMagic; w[1] = R; w[2] = E; w[3] = inst_per_rank; w[4] = I; w[5] = G; w[6] = n;
  w[7] = n_ent;
  size_t o = 8;
  auto put = [&](const std::vector<int>& a) { for (int x : a) w[o++] = x; };
  put(grp_expert); put(grp_start); put(copy_inst); put(copy_rank); put(copy_group);
  put(rank_start); put(rank_copy); put(exp_inst);
  for (int i = 0; i < I; ++i) w[o++] = ie[i];
  put(inst_copy);
  put(ent_rr); put(ent_start); put(ent_p); put(ent_q);
  w[o++] = blk;
  put(lane_rank); put(rank_lane);
  hipStream_t s = uep_stream(stream);
  if (hipMemcpyAsync(lp, w.data(), w.size() * sizeof(int32_t), hipMemcpyHostToDevice, s) !=
      hipSuccess)
    return UEP_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return UEP_EHIP;
  return UEP_OK;
}

extern "C" uep_status uep_lplb(const int32_t* counts, const void* lp, int32_t iters, float* x,
                               float* m, int32_t* inst_quota, int32_t* stats, int32_t* err,
                               void* stream) {
  if (!counts || !lp || !x || !m || !inst_quota || iters < 0 || iters > 200) return UEP_EINVAL;
  hipLaunchKernelGGL(lplb_kernel, dim3(1), dim3(kLpThreads), 0, uep_stream(stream),
                     counts, static_cast<const int32_t*>(lp), iters, x, m, inst_quota, stats, err);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}

// uep_lplb_plan: uep_load_matrix, uep_lplb and uep_reroute_assign in one call, with the
// LP solved concurrently with the bucket-position ranking (lplb_rank_kernel).  Launches:
// lm_hist, lm_counts (the load matrix; for long ranks lm_scan, which also writes it),
// lplb_rank_kernel, then the reroute and assignment of uep_reroute_assign.  Geometries
// off the ranking fast path, or whose ranking would not fit the LP's LDS block, run the
// three calls in sequence.
static size_t lp_plan_align(size_t b) { return (b + 255) / 256 * 256; }

extern "C" size_t uep_lplb_plan_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E,
                                               int32_t inst_per_rank) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0 || inst_per_rank <= 0) return 0;
  return lp_plan_align(uep_load_matrix_workspace_size(R, T, K, E)) +
         uep_reroute_workspace_size(R, E, inst_per_rank);
}

extern "C" uep_status uep_lplb_plan(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                                    int32_t E, const void* lp, int32_t inst_per_rank,
                                    const int32_t* inst_expert, int32_t iters, int32_t r_begin,
                                    int32_t r_end, int32_t* counts, int32_t* bucket_pos,
                                    float* x, float* m, int32_t* inst_quota, int32_t* stats,
                                    int32_t* xfer, int32_t* inst_offset, int32_t* dest_inst,
                                    int32_t* dest_row, int32_t* err, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (R <= 0 || T < 0 || K <= 0 || E <= 0 || inst_per_rank <= 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (R > kLpMaxR || K > 64 || E > kLmMaxE || (int64_t)R * T * K >= (1ll << 31) ||
      (int64_t)R * inst_per_rank > (1 << 20))
    return UEP_EGEOM;
  // every check of the three calls, before anything is enqueued
  if (!counts || !lp || !x || !m || !inst_quota || !inst_expert || !xfer || !inst_offset ||
      iters < 0 || iters > 200 || (T > 0 && (!topk_ids || !bucket_pos)) ||
      (T > 0 && r_end > r_begin && (!dest_inst || !dest_row)))
    return UEP_EINVAL;
  if (!ws || ws_bytes < uep_lplb_plan_workspace_size(R, T, K, E, inst_per_rank))
    return UEP_EWORKSPACE;
  const size_t lm_bytes = lp_plan_align(uep_load_matrix_workspace_size(R, T, K, E));
  void* rr_ws = static_cast<char*>(ws) + lm_bytes;
  const size_t rr_bytes = ws_bytes - lm_bytes;
  LmGeom g = lm_geom(R, T, K, E);
  const bool vec = K % 4 == 0 && reinterpret_cast<uintptr_t>(topk_ids) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(bucket_pos) % 16 == 0;
  const size_t lds = sizeof(uint64_t) * 4 * E + sizeof(int32_t) * 5 * E;
  const size_t lds_tile = lds + sizeof(int32_t) * 2 * (size_t)g.tok_per_chunk * K;
  const bool tile = !vec && lds_tile <= kLmTileMaxLds;
  if (!lm_bitmap(K, E) || T == 0 || (tile ? lds_tile : lds) > sizeof(LpShared)) {
    uep_status st = uep_load_matrix(topk_ids, R, T, K, E, counts, bucket_pos, err, ws, lm_bytes,
                                    stream);
    if (st == UEP_OK) st = uep_lplb(counts, lp, iters, x, m, inst_quota, stats, err, stream);
    if (st == UEP_OK)
      st = uep_reroute_assign(counts, topk_ids, bucket_pos, R, T, K, E, inst_per_rank,
                              inst_expert, inst_quota, r_begin, r_end, xfer, inst_offset,
                              dest_inst, dest_row, err, rr_ws, rr_bytes, stream);
    return st;
  }
  hipStream_t s = uep_stream(stream);
  int32_t* hist = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(lm_hist, dim3(g.n_chunks, R), dim3(256), sizeof(int32_t) * E, s, topk_ids,
                     hist, err, g);
  UEP_CHECK_LAUNCH();
  // long ranks: one scan of the chunk histograms, which also writes the load matrix,
  // instead of every ranking workgroup summing the earlier chunks (on a 64-chunk rank
  // that ranking outlasts the LP)
  const int per = E >= 256 ? 1 : 256 / E;
  const bool scanned = g.n_chunks > 16 * per;
  if (scanned)
    hipLaunchKernelGGL(lm_scan, dim3((E + 63) / 64, R), dim3(256), 0, s, hist, counts, g);
  else
    hipLaunchKernelGGL(lm_counts, dim3(R), dim3(256), 0, s, (const int32_t*)hist, counts, g);
  UEP_CHECK_LAUNCH();
  const dim3 grid(1 + g.n_chunks * R);
  const int32_t* lpw = static_cast<const int32_t*>(lp);
#define UEP_LP_FUSED(KM, TL)                                                                  \
  hipLaunchKernelGGL((lplb_rank_kernel<KM, TL>), grid, dim3(kLpThreads), 0, s, topk_ids,      \
                     bucket_pos, (const int32_t*)hist, err, g, vec, scanned,                  \
                     (const int32_t*)counts, lpw, iters, x, m, inst_quota, stats)
  if (K <= 8) {
    if (tile) UEP_LP_FUSED(8, true); else UEP_LP_FUSED(8, false);
  } else if (K <= 12) {
    if (tile) UEP_LP_FUSED(12, true); else UEP_LP_FUSED(12, false);
  } else {
    if (tile) UEP_LP_FUSED(16, true); else UEP_LP_FUSED(16, false);
  }
#undef UEP_LP_FUSED
  UEP_CHECK_LAUNCH();
  return uep_reroute_assign(counts, topk_ids, bucket_pos, R, T, K, E, inst_per_rank, inst_expert,
                            inst_quota, r_begin, r_end, xfer, inst_offset, dest_inst, dest_row,
                            err, rr_ws, rr_bytes, stream);
}

extern "C" uep_status uep_lplb_sample(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                                      const void* lp, const float* x, uint64_t seed,
                                      uint64_t layer, int32_t* dest_inst, int32_t* err,
                                      void* stream) {
  if (R <= 0 || T < 0 || K <= 0) return UEP_EINVAL;
  if (R > kLpMaxR || K > 64 || (int64_t)R * T * K >= (1ll << 31)) return UEP_EGEOM;
  const int64_t n_tok = (int64_t)R * T;
  if (n_tok == 0) return UEP_OK;
  if (!topk_ids || !lp || !x || !dest_inst) return UEP_EINVAL;
  const int64_t n_quad = n_tok * ((K + 3) / 4);
  const bool vec = K % 4 == 0 && reinterpret_cast<uintptr_t>(topk_ids) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dest_inst) % 16 == 0;
  const int64_t blocks = std::min<int64_t>((n_quad + kLsThreads - 1) / kLsThreads, kLsMaxBlocks);
  hipLaunchKernelGGL(lplb_sample_kernel, dim3((unsigned)blocks), dim3(kLsThreads), 0,
                     uep_stream(stream), topk_ids, n_tok, K, R, static_cast<const int32_t*>(lp), x,
                     seed, layer, dest_inst, err, vec);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
