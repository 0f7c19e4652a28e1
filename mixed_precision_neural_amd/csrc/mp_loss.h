// The scaled MSE loss of mp_loss_mse (mp_aux.hip), shared by the entry points that differ only
// in where the per-block partials live. Internal to libmp; not part of the public ABI.
#pragma once

#include "mp_internal.h"

namespace mp {

// Checks the arguments every MSE entry point shares (sizes, null pointers).
mp_status loss_mse_args(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, const mp_scaler* scaler,
                        const float* loss, const uint16_t* dy);
// FP32 partials the loss kernels write for M x N elements (one per block, at most 1024).
size_t loss_mse_partials(int64_t M, int64_t N);
// Launches the loss with its partials in `partials` (loss_mse_partials(M, N) floats) on s.
mp_status loss_mse_into(const uint16_t* y, const uint16_t* t, int64_t M, int64_t N, float c,
                        const mp_scaler* scaler, float* loss, uint16_t* dy, float* partials, hipStream_t s);

}  // namespace mp
