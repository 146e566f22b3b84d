// placeholder until the LPLB kernel lands
#include "common.h"
extern "C" size_t uep_lplb_struct_size(int32_t R, int32_t E, int32_t inst_per_rank) { return 0; }
extern "C" uep_status uep_lplb_prepare(const int32_t* inst_expert_host, int32_t R, int32_t E,
                            int32_t inst_per_rank, void* lp, size_t lp_bytes, void* stream) { return UEP_EGEOM; }
extern "C" uep_status uep_lplb(const int32_t* counts, const void* lp, int32_t iters, float* x, float* m,
                    int32_t* inst_quota, int32_t* stats, int32_t* err, void* stream) { return UEP_EGEOM; }
