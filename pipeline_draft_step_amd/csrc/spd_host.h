// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spd_common.h"
#include "spd_gemm.h"

namespace spd {

// last HIP error seen by a launch on this thread
int& last_hip_error_ref();

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

inline int check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    last_hip_error_ref() = (int)e;
    return SPD_E_HIP;
  }
  return SPD_OK;
}

inline int check_config(const spd_config* c) {
  if (!c) return SPD_E_INVALID;
  if (c->n < 1 || c->n > SPD_MAX_STAGES || c->m < 1 || c->m > SPD_MAX_ANCHORS) return SPD_E_INVALID;
  if (c->L < 1 || c->d < 1 || c->Ls < 0 || c->V < 1) return SPD_E_INVALID;
  if (c->dtype != SPD_F32 && c->dtype != SPD_BF16) return SPD_E_INVALID;
  if (c->anchor_mode != SPD_ANCHOR_ZERO_MASK && c->anchor_mode != SPD_ANCHOR_CLAMP_MIN)
    return SPD_E_INVALID;
  if (!(c->rms_eps >= 0.f)) return SPD_E_INVALID;
  return SPD_OK;
}

template <typename WT, int NT, typename In, typename Epi, typename RM>
int launch_gemm(const GemmPlan& p, const GemmShape& g, const In& in, const Epi& epi, const RM& rm,
                hipStream_t st) {
  dim3 grid(p.nblocks * p.S, p.mtiles);
  if (p.MT == 1)
    hipLaunchKernelGGL((gemm_skinny_kernel<WT, 1, NT, In, Epi, RM>), grid, dim3(GEMM_THREADS),
                       p.lds_bytes, st, g, in, epi, rm);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<WT, 2, NT, In, Epi, RM>), grid, dim3(GEMM_THREADS),
                       p.lds_bytes, st, g, in, epi, rm);
  int rc = check_launch();
  if (rc || p.S == 1) return rc;
  dim3 fgrid(p.nblocks, p.mtiles);
  if (p.MT == 1)
    hipLaunchKernelGGL((gemm_finish_kernel<1, NT, Epi, RM>), fgrid, dim3(GEMM_THREADS), 0, st, g, epi,
                       rm);
  else
    hipLaunchKernelGGL((gemm_finish_kernel<2, NT, Epi, RM>), fgrid, dim3(GEMM_THREADS), 0, st, g, epi,
                       rm);
  return check_launch();
}

size_t fuse_workspace(const spd_config* cfg, int M);
size_t pdm_workspace(const spd_config* cfg, int M, int64_t T_cap);
size_t lm_head_workspace(const spd_config* cfg, int rows);
size_t verify_workspace(int B, int gamma, int V);

}  // namespace spd
