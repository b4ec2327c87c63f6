// dm_launch.hpp -- launch wrappers of the verify-step kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "dm_common.hpp"

namespace dmv {

hipError_t launch_prep(const Plan& P, const void* h, void* Hm, RowMeta* meta, uint32_t* dbg_mask, hipStream_t st);
hipError_t launch_pack_w(const void* W, void* Wp, int V, int nkb, size_t n16, hipStream_t st);
hipError_t launch_gemm(const Plan& P, const void* W, const void* Hm, const RowMeta* meta, float* logits, Stat* part,
                       hipStream_t st);
hipError_t launch_combine(const Plan& P, const Stat* part, RowStat* rowstat, RowStat* centstat,
                          unsigned long long* race_best, int32_t* dbg_head_arg, float* dbg_head_logz,
                          int32_t* dbg_cent_arg, float* dbg_cent_logz, hipStream_t st);
hipError_t launch_filter(const Plan& P, const float* logits, const RowStat* rowstat, FiltStat* filt,
                         int32_t* dbg_count, float* dbg_logz, hipStream_t st);
hipError_t launch_vocab(const Plan& P, const int32_t* draft, const float* q_hat, const int32_t* tree_parent,
                        const float* logits, const RowStat* rowstat, const RowStat* centstat, float* jspart,
                        unsigned long long* race_best, const FiltStat* filt, int32_t* accept_len, int32_t* out_token,
                        int32_t* accept_pos, uint32_t* data_status, uint8_t* dbg_flags, float* dbg_js_heads,
                        float* dbg_js_draft, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);

// Vocabulary strips (16 rows each) one workgroup of the skinny GEMM covers.
int skinny_strips_per_group();

}  // namespace dmv
