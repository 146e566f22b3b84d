// Shared device helpers for libuep (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uep.h"

namespace uep {

constexpr int kWave = 64;

// 16-byte vector used for bit-exact row moves (native clang vector so that the
// non-temporal builtins accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ int shfl(int v, int src) { return __shfl(v, src, kWave); }

__device__ __forceinline__ int wave_incl_scan(int v);
// wave-wide sum, uniform result
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

// Inclusive prefix sum across the wave: Hillis-Steele inside each row of 16 lanes
// with DPP row_shr (lanes shifted in from outside the row read 0), then row_bcast:15
// and row_bcast:31 carry the row totals into the rows above.  All lanes active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// (value, index) reductions with the lowest index winning ties.  Inactive lanes
// pass index = INT32_MAX.
__device__ __forceinline__ void wave_argmax(int& v, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int v2 = __shfl_xor(v, o, kWave);
    int i2 = __shfl_xor(idx, o, kWave);
    if (v2 > v || (v2 == v && i2 < idx)) { v = v2; idx = i2; }
  }
}

__device__ __forceinline__ void wave_argmin(int& v, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int v2 = __shfl_xor(v, o, kWave);
    int i2 = __shfl_xor(idx, o, kWave);
    if (v2 < v || (v2 == v && i2 < idx)) { v = v2; idx = i2; }
  }
}

// Wave-wide max / min of an int, uniform result: DPP butterflies inside each row of
// 16 lanes (quad_perm xor 1, xor 2, then row_ror 4 and 8), then the four row results
// are combined with readlane.  Every lane of the wave must be active.  These four
// patterns give every lane a source lane in its own row, so bound_ctrl never applies;
// the mov_dpp form lets the compiler fold each move into its max/min, one
// v_max_i32_dpp (or v_min) per step instead of a copy, a DPP move and the max.
template <bool kMax>
__device__ __forceinline__ int wave_reduce_dpp(int v) {
  auto op = [](int a, int b) { return kMax ? max(a, b) : min(a, b); };
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));  // row_ror:4
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));  // row_ror:8
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ int wave_max(int v) { return wave_reduce_dpp<true>(v); }
__device__ __forceinline__ int wave_min(int v) { return wave_reduce_dpp<false>(v); }

// Lowest lane whose predicate holds (-1 if none).
__device__ __forceinline__ int first_lane(bool p) {
  const uint64_t b = __ballot(p);
  return b ? __ffsll((unsigned long long)b) - 1 : -1;
}

// sum_r counts[r][e] with up to 32 predicated loads in flight (two rounds for
// R <= 64): the matrix was just written by another kernel, so each round costs a
// full trip to the last-level cache
__device__ __forceinline__ int column_sum(const int32_t* __restrict__ counts, int R, int E, int e) {
  int s = 0;
  for (int r0 = 0; r0 < R; r0 += 32) {
    int v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u)       // clamped address, no branch: every load issues
      v[u] = counts[(int64_t)min(r0 + u, R - 1) * E + e];
#pragma unroll
    for (int u = 0; u < 32; ++u) s += r0 + u < R ? v[u] : 0;
  }
  return s;
}

// Bijection of [0, nb) for HBM-streaming grids: workgroup b runs on XCD b % 8; that
// XCD's workgroups take one contiguous range of logical block ids (the first nb % 8
// XCDs one more), so neighbouring blocks share an L2.
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb) {
  const int64_t q = nb / 8, rem = nb % 8, xcd = b % 8, idx = b / 8;
  return (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + idx;
}

// Streaming stores for data the kernel writes once and does not read back: 16-byte
// buffer stores with the cache-policy bits nt (non-temporal) and sc1 (device scope).
// A buffer resource covers one contiguous destination span (raw, untyped access;
// word 3 as gfx9 descriptors need: 32-bit data format); the hardware drops a store
// at or past `bytes`.  Measured on MI355X against non-temporal global stores (nt
// alone): the whole-group permute of the Qwen3-235B layer 3.65 -> 3.57-3.61 ms, the
// 26-slot staging 274 -> 264-267 us, a write-only stream unchanged (all eight
// combinations of sc0, nt, sc1 within 3 % of each other there), the combine's token
// rows 3.74 -> 3.61 ms.
typedef __amdgpu_buffer_rsrc_t span_t;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCpolStream = 2 | 16;   // nt | sc1

__device__ __forceinline__ span_t span_of(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes < INT32_MAX ? bytes : INT32_MAX), kRsrcWord3);
}

// 16 bytes at byte offset `off` of the span
__device__ __forceinline__ void stream_store(u32x4 v, span_t s, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, s, off, 0, kCpolStream);
}

// 4 bytes at byte offset `off` of the span, streaming like stream_store
__device__ __forceinline__ void stream_store_b32(uint32_t v, span_t s, int off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, s, off, 0, kCpolStream);
}

// Non-temporal 16-byte load at byte offset `off` of the span; zeros at or past its end.
// The span's bound replaces a per-lane guard, whose exec-mask branch around every load
// and store of a row cost the permute 1.3 % (3.61 -> 3.56 ms, same box).
__device__ __forceinline__ u32x4 stream_load(span_t s, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(s, off, 0, 2);   // nt
}

__device__ __forceinline__ void set_err(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// A dispatch row taken from device data: rows outside [-1, out_rows) become -1 (no
// row) and raise UEP_ERR_ROW_RANGE once per wave.  Every lane of the wave calls it.
__device__ __forceinline__ int checked_row(int d, int64_t out_rows, int32_t* err) {
  const bool bad = d < -1 || d >= out_rows;
  const uint64_t m = ballot(bad);
  if (m && (threadIdx.x % kWave) == (unsigned)(__ffsll((unsigned long long)m) - 1))
    set_err(err, UEP_ERR_ROW_RANGE);
  return bad ? -1 : d;
}

}  // namespace uep

// Host-side helpers.
#define UEP_CHECK_LAUNCH()                               \
  do {                                                   \
    if (hipGetLastError() != hipSuccess) return UEP_EHIP; \
  } while (0)

static inline hipStream_t uep_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
