// Row tile of the MFMA attention path, shared by the kernel and the plan.
#pragma once

#include "pa_internal.h"

namespace pa {

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 8
#endif
constexpr int kMfmaWaves = PA_PF_WAVES;          // waves per MFMA workgroup, 32 query rows each
constexpr int kMfmaRows = 32 * kMfmaWaves;
#ifndef PA_PF_BN
#define PA_PF_BN 64
#endif
constexpr int kMfmaBN = PA_PF_BN;   // keys per step of a row tile

}  // namespace pa
