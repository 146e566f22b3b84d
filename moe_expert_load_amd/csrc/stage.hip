// Redundant-slot weight staging and backward gradient reduction (UltraEP article:
// section "共享冗余 slot 管理动态专家副本" -- fixed slots per rank shared by all MoE
// layers, weights + gradient buffer, no optimizer state; section
// "复用前向方案，完成权重恢复与梯度归约" -- backward reuses the cached plan, re-stages
// the replica weights, reduces replica gradients into the main's gradient buffer
// and clears the redundant gradient buffer; section "流式通信算子加速动态权重分发" --
// persistent kernel pulling fixed-size tiles from a device-side task list).
//
// One persistent grid.  Each workgroup first turns the slot table into its task
// list in LDS (no host round trip: the plan stays on the device): the selected slots
// grouped by expert.  It then walks tasks = (expert group) x tile with a grid stride.  A tile is 256 threads x
// kStVec 16-byte vectors = 16 KiB of bf16 weights (or fp32 gradients); all loads of
// a tile are issued before its stores.  Tile size, grid (16 workgroups per CU) and the
// cache policy were picked by measurement on MI355X: the weight copy streams its slot
// stores (nt sc1); the gradient reduction keeps plain stores for the main gradient it
// has just read and non-temporal ones for the cleared replicas (streaming both ran
// 25 % slower).
//
// GRAD_REDUCE keeps the article's order fixed: for every element the main's
// gradient is added to the replicas' gradients one at a time in ascending rank
// (fp32, round to nearest even, no FMA), then each replica gradient is set to +0.
#include <atomic>

#include "common.h"

namespace uep {

constexpr int kStThreads = 256;
constexpr int kStVec = 4;                         // 16 KiB tiles (measured best on MI355X)
constexpr int kStTileVec = kStThreads * kStVec;   // 16-byte vectors per tile
constexpr int kStMaxSlots = 64 * 8;

// Slot groups, one per expert among the selected slots, members in slot order, built
// in LDS by the whole workgroup.  kByHome selects slots whose expert is homed in
// [r_begin, r_end) (gradients go to the main's rank), else slots of ranks in
// [r_begin, r_end) (weights go to the slot's rank).
struct StGroups {
  int32_t sel_e[kStMaxSlots];                 // selected slot's expert, else -1
  int32_t lead_cnt[kStMaxSlots];              // group size at its first slot, else 0
  int32_t lead_of[kStMaxSlots], pos_in[kStMaxSlots];   // first slot and rank of a member
  int32_t grp_of[kStMaxSlots];                // group index of a leading slot
  int32_t g_exp[kStMaxSlots], g_first[kStMaxSlots + 1], g_mem[kStMaxSlots];
  int32_t n_grp;
};

template <bool kByHome>
__device__ __forceinline__ bool st_selected(int i, int e, int S, int E_loc, int n_exp,
                                            int r_begin, int r_end) {
  if (e < 0 || e >= n_exp) return false;        // empty, or not an expert: skipped
  const int r = kByHome ? e / E_loc : i / S;
  return r >= r_begin && r < r_end;
}

// Every workgroup of the persistent grid builds the table at its start, so the build
// is kept short: one coalesced read of the slot table, LDS-only comparisons, and the
// leaders compacted in slot order by wave 0 with a ballot and a prefix sum (64 slots
// per round), three barriers in all.
template <bool kByHome>
__device__ __forceinline__ void st_build_groups(const int32_t* __restrict__ slot_expert, int n_slots,
                                                int S, int E_loc, int r_begin, int r_end,
                                                StGroups& G) {
  const int n_exp = n_slots / S * E_loc;           // R ranks x E_loc mains
  for (int i = threadIdx.x; i < n_slots; i += kStThreads) {
    const int e = slot_expert[i];
    G.sel_e[i] = st_selected<kByHome>(i, e, S, E_loc, n_exp, r_begin, r_end) ? e : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_slots; i += kStThreads) {
    const int e = G.sel_e[i];
    int cnt = 0, pos = 0, first = i;
    if (e >= 0)
      for (int i2 = 0; i2 < n_slots; ++i2) {
        const bool same = G.sel_e[i2] == e;
        cnt += same;
        if (i2 < i && same) {
          ++pos;
          first = min(first, i2);
        }
      }
    G.lead_cnt[i] = (e >= 0 && first == i) ? cnt : 0;
    G.lead_of[i] = first;
    G.pos_in[i] = pos;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    int ng = 0, nm = 0;
    for (int base = 0; base < n_slots; base += kWave) {
      const int i = base + threadIdx.x;
      const int cnt = i < n_slots ? G.lead_cnt[i] : 0;
      const uint64_t lead = ballot(cnt > 0);
      const int incl = wave_incl_scan(cnt);
      if (cnt > 0) {
        const int gi = ng + __popcll(lead & lanemask_lt());
        G.grp_of[i] = gi;
        G.g_exp[gi] = G.sel_e[i];
        G.g_first[gi] = nm + incl - cnt;
      }
      ng += __popcll(lead);
      nm += readlane(incl, kWave - 1);
    }
    if (threadIdx.x == 0) {
      G.g_first[ng] = nm;
      G.n_grp = ng;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_slots; i += kStThreads)     // members, in slot order
    if (G.sel_e[i] >= 0) G.g_mem[G.g_first[G.grp_of[G.lead_of[i]]] + G.pos_in[i]] = i;
  __syncthreads();
}

// Weights: each tile of an expert's main is read once and written to every slot of
// its group, so an expert replicated n times costs one read and n writes.
__global__ __launch_bounds__(kStThreads) void stage_weights_kernel(
    const int32_t* __restrict__ slot_expert, int R, int E, int S, int r_begin, int r_end,
    const u32x4* __restrict__ main_w, u32x4* __restrict__ slot_w, int64_t nvec) {
  __shared__ StGroups G;
  st_build_groups<false>(slot_expert, R * S, S, E / R, r_begin, r_end, G);
  const int64_t tiles = (nvec + kStTileVec - 1) / kStTileVec;
  const int64_t tasks = G.n_grp * tiles;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int gi = (int)(task / tiles);
    const int64_t v0 = (task % tiles) * kStTileVec;
    const u32x4* src = main_w + (int64_t)G.g_exp[gi] * nvec;
    u32x4 buf[kStVec];
#pragma unroll
    for (int k = 0; k < kStVec; ++k) {
      const int64_t v = v0 + k * kStThreads + threadIdx.x;
      if (v < nvec) buf[k] = src[v];
    }
    const int64_t span = min((int64_t)kStTileVec, nvec - v0) * 16;
    for (int m = G.g_first[gi]; m < G.g_first[gi + 1]; ++m) {
      const span_t dst = span_of(slot_w + (int64_t)G.g_mem[m] * nvec + v0, span);
#pragma unroll
      for (int k = 0; k < kStVec; ++k) {
        const int64_t v = v0 + k * kStThreads + threadIdx.x;
        if (v < nvec) stream_store(buf[k], dst, (k * kStThreads + threadIdx.x) * 16);
      }
    }
  }
}

__global__ __launch_bounds__(kStThreads) void stage_grad_kernel(
    const int32_t* __restrict__ slot_expert, int R, int E, int S, int r_begin, int r_end,
    f32x4* __restrict__ main_grad, f32x4* __restrict__ slot_grad, int64_t nvec) {
  // groups: one per replicated expert homed in [r_begin, r_end), members in slot order
  __shared__ StGroups G;
  st_build_groups<true>(slot_expert, R * S, S, E / R, r_begin, r_end, G);
  const int n_grp = G.n_grp;
  const int32_t* g_exp = G.g_exp;
  const int32_t* g_first = G.g_first;
  const int32_t* g_mem = G.g_mem;
  const int64_t tiles = (nvec + kStTileVec - 1) / kStTileVec;
  const int64_t tasks = n_grp * tiles;
  for (int64_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const int gi = (int)(task / tiles);
    const int64_t v0 = (task % tiles) * kStTileVec;
    f32x4* mg = main_grad + (int64_t)g_exp[gi] * nvec;
    const int m0 = g_first[gi], m1 = g_first[gi + 1];
    // the tile's main vectors, then each replica's vectors, all loads of one
    // operand in flight together; sums in slot order, one fp32 add at a time
    f32x4 acc[kStVec];
#pragma unroll
    for (int k = 0; k < kStVec; ++k) {
      const int64_t v = v0 + k * kStThreads + threadIdx.x;
      acc[k] = v < nvec ? mg[v] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int m = m0; m < m1; ++m) {
      f32x4* sg = slot_grad + (int64_t)g_mem[m] * nvec;
      f32x4 add[kStVec];
#pragma unroll
      for (int k = 0; k < kStVec; ++k) {
        const int64_t v = v0 + k * kStThreads + threadIdx.x;
        add[k] = v < nvec ? __builtin_nontemporal_load(sg + v) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int k = 0; k < kStVec; ++k) {
        const int64_t v = v0 + k * kStThreads + threadIdx.x;
        acc[k].x = acc[k].x + add[k].x;
        acc[k].y = acc[k].y + add[k].y;
        acc[k].z = acc[k].z + add[k].z;
        acc[k].w = acc[k].w + add[k].w;
        if (v < nvec) __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, sg + v);
      }
    }
#pragma unroll
    for (int k = 0; k < kStVec; ++k) {
      const int64_t v = v0 + k * kStThreads + threadIdx.x;
      if (v < nvec) mg[v] = acc[k];
    }
  }
}

// 16 workgroups per CU of the current device (the CU count is looked up once per device)
static int st_grid() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * 16;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    hipDeviceProp_t p;
    n = (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
            ? p.multiProcessorCount : 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n * 16;
}

}  // namespace uep

using namespace uep;

extern "C" uep_status uep_stage_replica_weights(int32_t mode, int32_t R, int32_t E, int32_t S,
                                                const int32_t* slot_expert, int32_t r_begin,
                                                int32_t r_end, const uint16_t* main_w,
                                                uint16_t* slot_w, float* main_grad,
                                                float* slot_grad, int64_t expert_elems,
                                                void* stream) {
  if (R <= 0 || E <= 0 || S < 0 || expert_elems < 0) return UEP_EINVAL;
  if (r_begin < 0 || r_end > R || r_begin > r_end) return UEP_EINVAL;
  if (R > 64 || S > 8 || E % R != 0 || expert_elems % 8 != 0) return UEP_EGEOM;
  if (S == 0 || expert_elems == 0 || r_begin == r_end) return UEP_OK;
  if (!slot_expert) return UEP_EINVAL;
  hipStream_t s = uep_stream(stream);
  if (mode == UEP_STAGE_WEIGHTS) {
    if (!main_w || !slot_w) return UEP_EINVAL;
    if ((reinterpret_cast<uintptr_t>(main_w) | reinterpret_cast<uintptr_t>(slot_w)) % 16)
      return UEP_EGEOM;
    hipLaunchKernelGGL(stage_weights_kernel, dim3(st_grid()), dim3(kStThreads), 0, s,
                       slot_expert, R, E, S, r_begin, r_end,
                       reinterpret_cast<const u32x4*>(main_w), reinterpret_cast<u32x4*>(slot_w),
                       expert_elems / 8);
  } else if (mode == UEP_STAGE_GRAD_REDUCE) {
    if (!main_grad || !slot_grad) return UEP_EINVAL;
    if ((reinterpret_cast<uintptr_t>(main_grad) | reinterpret_cast<uintptr_t>(slot_grad)) % 16)
      return UEP_EGEOM;
    hipLaunchKernelGGL(stage_grad_kernel, dim3(st_grid()), dim3(kStThreads), 0, s, slot_expert,
                       R, E, S, r_begin, r_end, reinterpret_cast<f32x4*>(main_grad),
                       reinterpret_cast<f32x4*>(slot_grad), expert_elems / 4);
  } else {
    return UEP_EINVAL;
  }
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
