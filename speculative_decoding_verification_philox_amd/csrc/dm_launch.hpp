// dm_launch.hpp -- launch wrappers of the verify-step kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "dm_common.hpp"

namespace dmv {

hipError_t launch_prep(const Plan& P, const void* h, void* Hm, uint32_t* dbg_mask, hipStream_t st);
hipError_t launch_gemm(const Plan& P, const void* W, const void* Hm, float* logits, Stat* part, hipStream_t st);
hipError_t launch_combine(const Plan& P, const Stat* part, RowStat* rowstat, RowStat* centstat, int32_t* dbg_head_arg,
                          float* dbg_head_logz, int32_t* dbg_cent_arg, float* dbg_cent_logz, hipStream_t st);
hipError_t launch_js(const Plan& P, const float* logits, const float* q_hat, const RowStat* rowstat,
                     const RowStat* centstat, float* jspart, hipStream_t st);
hipError_t launch_decide(const Plan& P, const int32_t* draft, const float* q_hat, const float* logits,
                         const RowStat* rowstat, const RowStat* centstat, const float* jspart, int32_t* accept_len,
                         int32_t* out_token, unsigned long long* race_best, uint8_t* dbg_flags, float* dbg_js_heads,
                         float* dbg_js_draft, hipStream_t st);
hipError_t launch_race(const Plan& P, const float* q_hat, const float* logits, const RowStat* rowstat,
                       const int32_t* accept_len, unsigned long long* race_best, int32_t* out_token, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);

// Vocabulary strips (16 rows each) one workgroup of the skinny GEMM covers.
int skinny_strips_per_group();

}  // namespace dmv
