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
  if (c->feature_schedule < SPD_SCHEDULE_PRE_STEP || c->feature_schedule > SPD_SCHEDULE_FIRST_STAGE)
    return SPD_E_INVALID;
  if (c->top_k < 0 || c->top_k > SPD_TOP_K_MAX || !(c->top_p >= 0.f && c->top_p <= 1.f))
    return SPD_E_INVALID;
  if (c->head_workgroups < 0) return SPD_E_INVALID;
  return SPD_OK;
}

constexpr int CTR_FINAL = SPD_WS_COUNTER_BYTES / 4 - 16;  // counter of a second-level arrival
constexpr int CTR_HEAD = CTR_FINAL - 1024;  // vocabulary-head counters [CTR_HEAD, CTR_FINAL)

template <typename WT, int NT, typename In, typename Epi, typename RM>
int launch_gemm(const GemmPlan& p, const GemmShape& g, const In& in, const Epi& epi, const RM& rm,
                hipStream_t st) {
  if ((size_t)p.mtiles * p.nblocks >= (size_t)CTR_HEAD) return SPD_E_UNSUPPORTED;
  if ((size_t)p.S * g.M * g.N * 4 >= ((size_t)1 << 31)) return SPD_E_UNSUPPORTED;  // 32-bit offsets
  GemmShape gs = g;
  gs.x_bytes = p.x_bytes;
  gs.ytile_bytes = p.ytile_bytes;
  dim3 grid(p.nblocks * p.S, p.mtiles);
  if (p.MT == 1)
    hipLaunchKernelGGL((gemm_skinny_kernel<WT, 1, NT, In, Epi, RM>), grid, dim3(GEMM_THREADS),
                       p.lds_bytes, st, gs, in, epi, rm);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<WT, 2, NT, In, Epi, RM>), grid, dim3(GEMM_THREADS),
                       p.lds_bytes, st, gs, in, epi, rm);
  return check_launch();
}

size_t fuse_workspace(const spd_config* cfg, int M);
size_t pdm_workspace(const spd_config* cfg, int M, int64_t T_cap);
size_t lm_head_workspace(const spd_config* cfg, int rows);
size_t verify_workspace(int B, int gamma, int V);

}  // namespace spd
