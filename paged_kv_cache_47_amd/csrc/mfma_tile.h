// Row tile of the MFMA attention path, shared by the kernel and the plan.
#pragma once

#include "pa_internal.h"

namespace pa {

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 8
#endif
constexpr int kMfmaWaves = PA_PF_WAVES;          // waves per MFMA workgroup, 32 query rows each
constexpr int kMfmaRows = 32 * kMfmaWaves;
constexpr int kMfmaBN = 64;   // keys per step of a row tile       // query rows per MFMA workgroup

}  // namespace pa
